"""Benchmark of the hot path on one MI355X.

One step = the whole path on one batch of the Llama-3-8B-shaped layer
(8 KV / 32 query heads, head_dim 128, 32768 tokens, 128-token fp16 window,
16 groups x 8 dims, 1 stage, C = 256):
  encode    K and V of the 32640 coded tokens (rotation, distance GEMM on
            MFMA, argmin, residual update, code store),
  reconstruct  every coded vector from its codes (sum of codewords, unrotated),
  decode    single-token attention for the 32 query heads over the codes and
            the fp16 window (q rotation, LUT, code streaming, split-K, LSE merge).
Inputs are resident in HBM before timing; a 512 MB write between the
producer kernels and the decode evicts the 256 MB Infinity Cache so the decode
reads its codes from HBM.

Prints ONE JSON line.  ``value`` is the decode effective bandwidth (code +
window + LUT bytes over the decode kernels' time); the encode throughput and
its fraction of the bf16 MFMA peak are reported beside it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6     # dense MFMA, 256 CU x 2.4 GHz x 4096 flop/clk/CU
VALU_LANE_OPS = 256 * 2.4e9 * 64  # non-packed 32-bit VALU lane-ops per second


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-flush", action="store_true")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_attention_fwht_amd as kvq
    import synth

    w = synth.workload(args.workload)
    if w.n_q_heads == 0:
        print("bench.py: the step needs a decode workload (with query heads)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_inputs(w)
    B, Hkv, Hq, D, T, W = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.tokens, w.window
    S, G, C, Tc = w.n_stages, w.n_groups, w.n_codewords, w.code_tokens
    if w.x_dtype == "bf16":
        x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp["x"]).to(dev)
    cb = torch.from_numpy(inp["cb"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    kw = torch.from_numpy(inp["k_win"]).to(dev) if W > 0 else None
    vw = torch.from_numpy(inp["v_win"]).to(dev) if W > 0 else None
    codes = torch.empty((2, B * Hkv, Tc, S, G), dtype=torch.uint8, device=dev)
    enc_ws = torch.empty(max(kvq.encode_workspace_size(D, G, S, C, 2), 16), dtype=torch.uint8,
                         device=dev)
    recon = torch.empty((2, B * Hkv, Tc, D), dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    att_ws = torch.empty(max(kvq.attend_workspace_size(B, Hq, Hkv, D, Tc, W, S, G, C), 16),
                         dtype=torch.uint8, device=dev)
    flush_buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    kc = codes[0].view(B, Hkv, Tc, S, G)
    vc = codes[1].view(B, Hkv, Tc, S, G)

    def flush(i):
        if not args.no_flush:
            flush_buf.fill_(float(i))

    evs = []

    def step(i, timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
        flush(i)
        if timed: e[0].record()
        kvq.encode(x, cb, n_rows=Tc, codes=codes, workspace=enc_ws)
        if timed: e[1].record()
        kvq.decode_reconstruct(codes, cb, unrotate=True, out=recon)
        if timed: e[2].record()
        flush(i + 1)
        if timed: e[3].record()
        kvq.attend_decode(q, kc, vc, cb[0], cb[1], kw, vw, out=out, workspace=att_ws)
        if timed:
            e[4].record()
            evs.append(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    rec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    att_ms = np.array([e[3].elapsed_time(e[4]) for e in evs])

    n_vec = 2 * B * Hkv * Tc
    enc_flops = 2.0 * D * C * S * n_vec
    code_b = 2 * B * Hkv * Tc * S * G
    win_b = 2 * B * Hkv * W * D * 2
    lut_b = B * Hq * S * G * C * 4
    eff_b = code_b + win_b + lut_b
    rec_b = n_vec * (S * G + 4 * D)

    att_s = float(np.median(att_ms)) * 1e-3
    enc_s = float(np.median(enc_ms)) * 1e-3
    rec_s = float(np.median(rec_ms)) * 1e-3
    dec_gbs = eff_b / att_s / 1e9
    enc_tflops = enc_flops / enc_s / 1e12
    cand_per_s = n_vec * S * G * C / enc_s
    times = {"encode": enc_s, "reconstruct": rec_s, "decode": att_s}
    dominant = max(times, key=times.get)
    if dominant == "encode":
        roof = {"kernel": "encode (kvq_encode: codebook pack + encode_mfma_kernel)", "bound": "mfma",
                "achieved": round(enc_tflops, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(enc_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None}
    elif dominant == "reconstruct":
        gbs = rec_b / rec_s / 1e9
        roof = {"kernel": "reconstruct_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": None}
    else:
        roof = {"kernel": "decode (attn_prep + attn_chunk + attn_merge)", "bound": "hbm",
                "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None}

    res = {
        "metric": "decode-attn effective HBM GB/s (% peak) + encode Mvec/s (% MFMA peak)",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} Hkv={Hkv} Hq={Hq} D={D} T={T} W={W} "
                               f"G={G}x{D // G} S={S} C={C}", "global_batch": B, "seq_len": T,
                   "parallelism": "none (1 GPU)"},
        "decode": {"value": round(dec_gbs, 2), "unit": "GB/s",
                   "pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 3),
                   "ms": round(att_s * 1e3, 5), "effective_bytes": eff_b,
                   "bytes": {"codes": code_b, "window": win_b, "lut": lut_b},
                   "cache_flushed": not args.no_flush},
        "encode": {"value": round(n_vec / enc_s / 1e6, 2), "unit": "Mvec/s",
                   "pct_bf16_mfma_peak": round(100 * enc_tflops / BF16_PEAK_TFLOPS, 3),
                   "ms": round(enc_s * 1e3, 5), "vectors": n_vec, "algorithmic_flops": enc_flops,
                   "candidates_per_s": cand_per_s,
                   "pct_valu_argmin_bound": round(100 * cand_per_s * 1.5 / VALU_LANE_OPS, 2)},
        "reconstruct": {"value": round(rec_b / rec_s / 1e9, 1), "unit": "GB/s",
                        "ms": round(rec_s * 1e3, 5)},
        "kernel_ms_p10_p90": {"encode": [round(float(np.percentile(enc_ms, p)), 5) for p in (10, 90)],
                              "reconstruct": [round(float(np.percentile(rec_ms, p)), 5) for p in (10, 90)],
                              "decode": [round(float(np.percentile(att_ms, p)), 5) for p in (10, 90)]},
        "roofline": roof,
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, codes, eff_b, dec_gbs)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, inp, codes, eff_b, dec_gbs):
    """The float64 oracle on a bounded sample of the same workload: decode
    attention for 2 of the KV heads (all their query heads, every coded token
    plus the window), and encode of 8192 vectors."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = os.cpu_count()
    B, Hkv, Hq, Tc, S, G = w.batch, w.n_kv_heads, w.n_q_heads, w.code_tokens, w.n_stages, w.n_groups
    rep = Hq // Hkv
    kvs = 2
    c = codes.cpu().numpy()
    kc = c[0].reshape(B, Hkv, Tc, S, G)[:1, :kvs]
    vc = c[1].reshape(B, Hkv, Tc, S, G)[:1, :kvs]
    t0 = time.perf_counter()
    oracle.attend(inp["q"][:1, :kvs * rep], kc, vc, inp["cb"][0], inp["cb"][1],
                  inp["k_win"][:1, :kvs] if w.window else None,
                  inp["v_win"][:1, :kvs] if w.window else None)
    t_dec = time.perf_counter() - t0
    frac = kvs / (B * Hkv)
    gbs = eff_b * frac / t_dec / 1e9
    xs = inp["x_f32"][0].reshape(-1, w.head_dim)[:8192].astype(np.float64)
    t0 = time.perf_counter()
    oracle.rvq_encode(xs, inp["cb"][0])
    t_enc = time.perf_counter() - t0
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(blas), "kind": "oracle",
            "sample": f"decode: {kvs} of {B * Hkv} (sequence, KV head) pairs with all {rep} query "
                      f"heads each, {Tc} coded + {w.window} window tokens ({t_dec:.1f} s); encode: "
                      f"8192 vectors ({t_enc:.1f} s). float64 NumPy; elementwise work on one core, "
                      f"matrix products on {blas} BLAS threads",
            "encode_mvec_per_s": round(8192 / t_enc / 1e6, 6),
            "gpu_over_cpu_decode": round(dec_gbs / gbs, 1)}


if __name__ == "__main__":
    main()
