"""Benchmark of the hot path on one MI355X.

One step = the whole path on one batch of the long-context layer (1 sequence
x 131072 tokens, 8 KV / 32 query heads, head_dim 128, Laplace K/V with
per-channel scales, 4 residual stages of 16 groups x 8 dims, C = 256, a
256-token fp16 window):
  encode       K and V of the 130816 coded tokens (rotation, distance GEMM on
               MFMA, argmin, residual update, code store),
  reconstruct  every coded vector from its codes (sum of codewords, unrotated),
  decode       single-token attention for the 32 query heads over the codes
               and the fp16 window (q rotation, LUT, code streaming, split-K,
               LSE merge).
Inputs are resident in HBM before timing.  The codebooks are packed into the
encode workspace once at set-up (they are constants of the layer, like
weights); each step's encode reads the packed copy, and the packing pass,
left out of the step, is timed on its own and reported beside the encode.
Before the encode and before the decode the caches are evicted clean: a
512 MB write replaces every line of the 256 MB Infinity Cache and the L2s,
then a 512 MB read of a second buffer writes those dirty lines back and
leaves clean ones, so each call reads its inputs from HBM and no write-back
of other data shares HBM with it.  The decode after the write alone (dirty
lines still cached) is reported beside it as ``dirty_eviction_us``.

Prints ONE JSON line.  ``value`` is the long-context decode's effective
bandwidth (code + window + LUT bytes over the decode call's time: LUT and
table pass, chunk kernel and LSE merge).  ``roofline`` is that decode call's
(HBM-bound); ``roofline_encode`` is the 32-layer bulk prefill encode's
(MFMA-bound: 2 D C S flops per vector over the mean kernel time).  The same
step on the Llama-shaped layer and the Qwen-shaped batch is reported under
``secondary``; the streaming calls (append, flush), the dual-transform calls
(factor calibration, smoothed key encode, decode with the factors folded into
the query), the K-means fitting of the key codebooks on a 65,536-vector
sample, the scalar residual variant (2 bits per stage) and the rotation alone
are timed on the Llama-shaped layer after the step.  Each roofline's HBM
``traffic`` comes from the rocprofv3 counter summary committed for its
kernels, and is null when one of their sources has changed since those
counters were taken.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6         # dense MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
VALU_LANE_OPS = 256 * 2.4e9 * 64  # non-packed 32-bit VALU lane-ops per second
CSRC = os.path.join(ROOT, "compressed_attention_fwht_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ("attend.hip", "attend_rc.hip", "attend_common.h", "kvq_device.h")
ENCODE_SOURCES = ("encode.hip", "kvq_device.h")
DECODE_TRAFFIC = "attend_decode_longctx_traffic.md"
ENCODE_TRAFFIC = "encode_mfma_kernel_prefill_traffic.md"
WORKLOAD_TAG = {2: "llama8b", 3: "qwen7b", 4: "longctx"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--secondary", default="2,3",
                   help="comma-separated decode workloads timed after the main step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the 32-layer bulk prefill encode measurement")
    p.add_argument("--no-flush", action="store_true")
    p.add_argument("--step-only", action="store_true",
                   help="time the main step only (no graph replays, dirty-eviction decode, "
                        "secondary workloads, prefill, streaming, "
                        "dual-transform, fitting, scalar or rotation legs), so a profiler sees "
                        "only the step's kernels")
    p.add_argument("--prefill-only", action="store_true",
                   help="time the 32-layer bulk prefill encode only")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a plain 256 MiB device copy 3x first (scale for HBM counters)")
    return p.parse_args()


def source_sha(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def profiled_traffic(fname, sources):
    """HBM bytes per launch from the committed counter summary
    profiles/<fname> (its JSON block), or None when there is none or one of
    ``sources`` changed since it was taken."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None, None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None, fname
    d = json.loads(m.group(1))
    shas = d.get("sources_sha256", {})
    if "traffic_bytes_per_launch" not in d or any(shas.get(s) != source_sha(s) for s in sources):
        return None, fname
    return d["traffic_bytes_per_launch"], fname


def cuda_events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


class Layer:
    """One decode workload's layer resident on the GPU: K|V inputs, codebooks,
    query, fp16 window, codes, reconstruction and workspaces; the codebooks are
    packed into the encode workspace at set-up."""

    def __init__(self, torch, kvq, synth, key, dev):
        w = synth.workload(key)
        if w.n_q_heads == 0:
            raise SystemExit("bench.py: the step needs a decode workload (with query heads)")
        self.w, self.key, self.kvq = w, key, kvq
        self.inp = inp = synth.make_inputs(w)
        B, Hkv, Hq, D, W = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window
        S, G, C, Tc = w.n_stages, w.n_groups, w.n_codewords, w.code_tokens
        if w.x_dtype == "bf16":
            self.x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            self.x = torch.from_numpy(inp["x"]).to(dev)
        self.cb = torch.from_numpy(inp["cb"]).to(dev)
        self.q = torch.from_numpy(inp["q"]).to(dev)
        self.kw = torch.from_numpy(inp["k_win"]).to(dev) if W > 0 else None
        self.vw = torch.from_numpy(inp["v_win"]).to(dev) if W > 0 else None
        self.codes = torch.empty((2, B * Hkv, Tc, S, G), dtype=torch.uint8, device=dev)
        self.enc_ws = torch.empty(max(kvq.encode_workspace_size(D, G, S, C, 2), 16),
                                  dtype=torch.uint8, device=dev)
        self.recon = torch.empty((2, B * Hkv, Tc, D), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.att_ws = torch.empty(max(kvq.attend_workspace_size(B, Hq, Hkv, D, Tc, W, S, G, C), 16),
                                  dtype=torch.uint8, device=dev)
        self.kc = self.codes[0].view(B, Hkv, Tc, S, G)
        self.vc = self.codes[1].view(B, Hkv, Tc, S, G)
        self.encode(packed=False)                 # set-up: pack the codebooks (layer constants)
        torch.cuda.synchronize()
        n_vec = 2 * B * Hkv * Tc
        self.n_vec = n_vec
        self.enc_flops = 2.0 * D * C * S * n_vec
        self.code_b = 2 * B * Hkv * Tc * S * G
        self.win_b = 2 * B * Hkv * W * D * 2
        self.lut_b = B * Hq * S * G * C * 4
        self.eff_b = self.code_b + self.win_b + self.lut_b
        self.rec_b = n_vec * (S * G + 4 * D)

    def name(self):
        w = self.w
        return (f"{w.name}: B={w.batch} Hkv={w.n_kv_heads} Hq={w.n_q_heads} D={w.head_dim} "
                f"T={w.tokens} W={w.window} G={w.n_groups}x{w.head_dim // w.n_groups} "
                f"S={w.n_stages} C={w.n_codewords}")

    def encode(self, packed=True):
        w = self.w
        self.kvq.encode(self.x, self.cb, n_rows=w.code_tokens, codes=self.codes,
                        workspace=self.enc_ws, packed=packed)

    def reconstruct(self):
        self.kvq.decode_reconstruct(self.codes, self.cb, unrotate=True, out=self.recon)

    def decode(self):
        self.kvq.attend_decode(self.q, self.kc, self.vc, self.cb[0], self.cb[1], self.kw, self.vw,
                               out=self.out, workspace=self.att_ws)


def time_steps(torch, L, steps, warmup, flush):
    """warmup untimed steps, then ``steps`` timed ones; per step HIP events
    on the current stream (the one every call launches on) around the encode,
    the reconstruction and the decode.  Returns per-call ms arrays and the
    wall time of the timed steps."""
    evs = []

    def step(i, timed):
        e = cuda_events(torch, 5) if timed else None
        flush(i)
        if timed: e[0].record()
        L.encode()
        if timed: e[1].record()
        L.reconstruct()
        if timed: e[2].record()
        flush(i + 1)
        if timed: e[3].record()
        L.decode()
        if timed:
            e[4].record()
            evs.append(e)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc = np.array([e[0].elapsed_time(e[1]) for e in evs])
    rec = np.array([e[1].elapsed_time(e[2]) for e in evs])
    att = np.array([e[3].elapsed_time(e[4]) for e in evs])
    return enc, rec, att, wall


def packing_us(torch, kvq, L, reps=20):
    """Codebook packing pass, left out of the step: a one-row-per-sequence
    encode that packs its codebooks minus the same encode reading the packed
    copy (median of each), so the encode itself is negligible in both."""
    w = L.w
    small = torch.empty((2, w.batch * w.n_kv_heads, 1, w.n_stages, w.n_groups),
                        dtype=torch.uint8, device=L.codes.device)
    ts = {True: [], False: []}
    for i in range(reps + 2):
        for packed in (True, False):
            e0, e1 = cuda_events(torch, 2)
            e0.record()
            kvq.encode(L.x, L.cb, n_rows=1, codes=small, workspace=L.enc_ws, packed=packed)
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts[packed].append(e0.elapsed_time(e1))
    return round((float(np.median(ts[False])) - float(np.median(ts[True]))) * 1e3, 2)


def graph_replay_us(torch, L, flush, reps):
    """The decode call replayed from a HIP graph (captured once), caches
    evicted before each replay: the launch gaps between its kernels leave the
    measured latency."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.decode()
    gts = []
    for i in range(reps + 3):
        flush(i)
        e0, e1 = cuda_events(torch, 2)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            gts.append(e0.elapsed_time(e1))
    del graph
    return round(float(np.median(gts)) * 1e3, 2)


def decode_after(torch, L, evict, reps):
    """Median decode call time (us) with ``evict`` run before each call."""
    ts = []
    for i in range(reps + 3):
        evict(i)
        e0, e1 = cuda_events(torch, 2)
        e0.record()
        L.decode()
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1))
    return round(float(np.median(ts)) * 1e3, 2)


def layer_report(torch, kvq, L, enc_ms, rec_ms, att_ms, flush, reps, graphs=True):
    w = L.w
    att_s = float(np.median(att_ms)) * 1e-3
    enc_s = float(np.median(enc_ms)) * 1e-3
    rec_s = float(np.median(rec_ms)) * 1e-3
    dec_gbs = L.eff_b / att_s / 1e9
    enc_tflops = L.enc_flops / enc_s / 1e12
    cand_per_s = L.n_vec * w.n_stages * w.n_groups * w.n_codewords / enc_s
    # the layer's cache as the library counts it (kvq_cache_bytes), and its
    # size against the same tokens held as dense fp16
    cache = kvq.cache_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.code_tokens,
                            w.window, w.n_stages, w.n_groups, w.n_codewords)
    cache["vs_dense_fp16"] = round(cache["dense"] / (cache["code"] + cache["window"]), 2)
    rep = {
        "workload": L.name(),
        "decode": {"value": round(dec_gbs, 2), "unit": "GB/s",
                   "pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 3),
                   "us": round(att_s * 1e6, 2), "effective_bytes": L.eff_b,
                   "bytes": {"codes": L.code_b, "window": L.win_b, "lut": L.lut_b},
                   "codes_window_gbs": round((L.code_b + L.win_b) / att_s / 1e9, 2),
                   "cache": cache},
        "encode": {"value": round(L.n_vec / enc_s / 1e6, 2), "unit": "Mvec/s",
                   "pct_bf16_mfma_peak": round(100 * enc_tflops / BF16_PEAK_TFLOPS, 3),
                   "us": round(enc_s * 1e6, 2), "vectors": L.n_vec,
                   "algorithmic_flops": L.enc_flops, "candidates_per_s": cand_per_s,
                   "pct_valu_argmin_bound": round(100 * cand_per_s * 1.5 / VALU_LANE_OPS, 2),
                   "codebook_packing_us": packing_us(torch, kvq, L),
                   "note": "codebooks packed once at set-up and read packed by every timed "
                           "encode; the packing pass (codebook_packing_us) is not in the step"},
        "reconstruct": {"value": round(L.rec_b / rec_s / 1e9, 1), "unit": "GB/s",
                        "us": round(rec_s * 1e6, 2)},
        "kernel_ms_p10_p90": {k: [round(float(np.percentile(v, p)), 5) for p in (10, 90)]
                              for k, v in (("encode", enc_ms), ("reconstruct", rec_ms),
                                           ("decode", att_ms))},
    }
    if graphs:
        rep["decode"]["graph_replay_us"] = graph_replay_us(torch, L, flush, reps)
    return rep


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_attention_fwht_amd as kvq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:                 # a copy kernel of known size for the counters
        src = torch.empty(256 * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.prefill_only:
        print(json.dumps({"encode_prefill": prefill_encode(torch, kvq, synth, dev)}), flush=True)
        return

    flush_buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    clean_buf = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def flush(i):
        if not args.no_flush:
            flush_buf.fill_(float(i))
            clean_buf.sum()

    def flush_dirty(i):
        if not args.no_flush:
            flush_buf.fill_(float(i))

    L = Layer(torch, kvq, synth, args.workload, dev)
    w = L.w
    enc_ms, rec_ms, att_ms, wall = time_steps(torch, L, args.steps, args.warmup, flush)

    # roofline of the decode call on its mean time (events on the stream it
    # launches on): code + window + LUT bytes per call
    mean_dec = float(np.mean(att_ms)) * 1e-3
    ach = L.eff_b / mean_dec / 1e9
    traffic, prof = profiled_traffic(DECODE_TRAFFIC, DECODE_SOURCES)
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "kvq_attend_decode: attn_rc_prep (LUT and V tables) + attn_rc "
                      "(chunks) + attn_merge (LSE)",
            "per_launch": {"bytes": L.eff_b, "mean_us": round(mean_dec * 1e6, 3),
                           "workload": L.name()},
            "counters": prof}

    main_rep = layer_report(torch, kvq, L, enc_ms, rec_ms, att_ms, flush, args.steps,
                            graphs=not args.step_only)
    if not args.step_only:
        main_rep["decode"]["dirty_eviction_us"] = decode_after(torch, L, flush_dirty, args.steps)
        main_rep["decode"]["layers_graph"] = decode_layers_graph(
            torch, kvq, L.q, L.kc, L.vc, L.cb, L.kw, L.vw, L.out, L.att_ws, flush, L.eff_b,
            args.steps)
    dec_gbs = main_rep["decode"]["value"]
    res = {
        "metric": "decode-attn effective HBM GB/s (% peak) + encode Mvec/s (% MFMA peak)",
        "value": dec_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtypes": {"k_v_in": w.x_dtype, "window": "f16", "query": "f32", "codebooks": "f32",
                   "codes": "u8", "encode_contraction": "bf16 MFMA (codebook hi + lo), f32 sums",
                   "decode": "f32 LUT and softmax, u64 fixed-point histograms"},
        "data": "synthetic",
        "config": {"workload": L.name(), "global_batch": w.batch, "seq_len": w.tokens,
                   "parallelism": "none (1 GPU)"},
        "decode": dict(main_rep["decode"], cache_flushed=not args.no_flush),
        "encode": main_rep["encode"],
        "reconstruct": main_rep["reconstruct"],
        "kernel_ms_p10_p90": main_rep["kernel_ms_p10_p90"],
        "roofline": roof,
    }
    inp_main, codes_main = L.inp, L.codes.cpu()
    eff_main = L.eff_b
    del L
    torch.cuda.empty_cache()

    if not args.step_only:
        sec = {}
        aux = None
        for key in [int(k) for k in args.secondary.split(",") if k.strip()]:
            S2 = Layer(torch, kvq, synth, key, dev)
            e2, r2, a2, _ = time_steps(torch, S2, args.steps, args.warmup, flush)
            sec[WORKLOAD_TAG.get(key, str(key))] = layer_report(torch, kvq, S2, e2, r2, a2, flush,
                                                                args.steps)
            if key == 2:
                aux = S2
            else:
                del S2
            torch.cuda.empty_cache()
        res["secondary"] = sec
        if aux is not None:
            A = aux
            tag = " (Llama-shaped layer)"
            res["smooth"] = smooth_calls(torch, kvq, A.x, A.cb, A.q, A.kc, A.vc, A.kw, A.vw, A.w,
                                         dev, flush)
            res["fit"] = fit_calls(torch, kvq, A.x, A.cb, A.w, dev)
            res["scalar"] = scalar_calls(torch, kvq, A.x, A.q, A.kw, A.vw, A.w, dev, flush)
            res["rotate"] = rotate_calls(torch, kvq, A.x, A.w, dev, flush)
            res["stream"] = stream_calls(torch, kvq, A.inp, A.w, dev)
            for k in ("smooth", "fit", "scalar", "rotate", "stream"):
                res[k]["layer"] = A.name() + tag
            del A, aux
        del flush_buf, clean_buf
        torch.cuda.empty_cache()
        if not args.no_prefill:
            pre = prefill_encode(torch, kvq, synth, dev)
            res["encode_prefill"] = pre
            res["roofline_encode"] = pre.pop("roofline")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp_main, codes_main, eff_main, dec_gbs)
    print(json.dumps(res), flush=True)


def prefill_encode(torch, kvq, synth, dev, reps=10):
    """Encode throughput of the 32-layer bulk prefill workload (32 layers x
    K|V x 8 KV heads x 32768 tokens, 16x8 groups, 2 stages): one kvq_encode
    call over all 64 books.  K/V are drawn on the GPU with the workload's law
    (N(0,1), rotate-half RoPE theta 5e5 on K, bf16); codebooks are the
    workload's own."""
    w = synth.workload(5)
    L, H, T, D = w.layers, w.n_kv_heads, w.tokens, w.head_dim
    S, G, C = w.n_stages, w.n_groups, w.n_codewords
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    x = torch.empty((2 * L, H, T, D), dtype=torch.bfloat16, device=dev)
    half = D // 2
    inv = w.rope_theta ** (-2.0 * torch.arange(half, dtype=torch.float64, device=dev) / D)
    ang = torch.arange(T, dtype=torch.float64, device=dev)[:, None] * inv[None, :]
    cs, sn = torch.cos(ang).float(), torch.sin(ang).float()
    for b in range(2 * L):
        v = torch.randn((H, T, D), generator=gen, device=dev, dtype=torch.float32)
        if b % 2 == 0:                                  # K carries RoPE
            x1, x2 = v[..., :half].clone(), v[..., half:].clone()
            v[..., :half] = x1 * cs - x2 * sn
            v[..., half:] = x2 * cs + x1 * sn
        x[b] = v.to(torch.bfloat16)
    cb = torch.from_numpy(synth.make_codebooks(w)).to(dev)
    codes = torch.empty((2 * L, H, T, S, G), dtype=torch.uint8, device=dev)
    ws = torch.empty(kvq.encode_workspace_size(D, G, S, C, 2 * L), dtype=torch.uint8, device=dev)
    kvq.encode(x, cb, codes=codes, workspace=ws)       # packs the codebooks, warms up
    torch.cuda.synchronize()
    ts = []
    for i in range(reps + 1):
        e0, e1 = cuda_events(torch, 2)
        e0.record()
        kvq.encode(x, cb, codes=codes, workspace=ws, packed=True)
        e1.record()
        torch.cuda.synchronize()
        if i >= 1:
            ts.append(e0.elapsed_time(e1))
    # the packing pass alone: a one-row-per-sequence encode that packs minus
    # one that reads the packed copy
    small = torch.empty((2 * L, H, 1, S, G), dtype=torch.uint8, device=dev)
    tq = {True: [], False: []}
    for i in range(reps + 2):
        for packed in (True, False):
            e0, e1 = cuda_events(torch, 2)
            e0.record()
            kvq.encode(x, cb, n_rows=1, codes=small, workspace=ws, packed=packed)
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                tq[packed].append(e0.elapsed_time(e1))
    n_vec = 2 * L * H * T
    t = float(np.median(ts)) * 1e-3
    t_mean = float(np.mean(ts)) * 1e-3
    flops = 2.0 * D * C * S * n_vec
    name = (f"{w.name}: {L} layers x K|V x Hkv={H} x T={T}, D={D}, "
            f"G={G}x{D // G} S={S} C={C}")
    ach = flops / t_mean / 1e12
    traffic, prof = profiled_traffic(ENCODE_TRAFFIC, ENCODE_SOURCES)
    roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": "encode_mfma_kernel (kvq_encode over the 64 books, codebooks packed)",
            "per_launch": {"flops": flops, "vectors": n_vec, "mean_us": round(t_mean * 1e6, 2),
                           "workload": name},
            "counters": prof}
    pack_us = (float(np.median(tq[False])) - float(np.median(tq[True]))) * 1e3
    del codes, ws, small
    # the scalar residual variant on the same 64 books, 2 bits per stage (levels
    # for the unit-variance source)
    bits = 2
    lv = scalar_levels(torch, kvq, [1.0] * (2 * L), bits, dev)
    sc = torch.empty((2 * L, H, T, 2, D * bits // 8), dtype=torch.uint8, device=dev)
    kvq.scalar_encode(x, lv, bits, codes=sc)
    torch.cuda.synchronize()
    ts2 = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.scalar_encode(x, lv, bits, codes=sc)
        e1.record()
        torch.cuda.synchronize()
        ts2.append(e0.elapsed_time(e1))
    t2 = float(np.median(ts2)) * 1e-3
    sb = n_vec * (2 * D + 2 * D * bits // 8)
    del x, sc
    torch.cuda.empty_cache()
    return {"workload": name,
            "value": round(n_vec / t / 1e6, 2), "unit": "Mvec/s", "ms": round(t * 1e3, 4),
            "vectors": n_vec, "pct_bf16_mfma_peak": round(100 * flops / t / 1e12 / BF16_PEAK_TFLOPS, 3),
            "reps": reps, "roofline": roof,
            "codebook_packing_us": round(pack_us, 2),
            "note": "codebooks of the 64 books packed once, read packed by every timed encode; "
                    "the packing pass (codebook_packing_us) is not in the timed encode",
            "scalar_2bit": {"ms": round(t2 * 1e3, 4), "bytes": sb,
                            "gbs": round(sb / t2 / 1e9, 1),
                            "pct_hbm_peak": round(100 * sb / t2 / 1e9 / HBM_PEAK_GBS, 2),
                            "note": "kvq_scalar_encode of the same bf16 books, 2 bits per stage: "
                                    "bf16 in + packed codes out"}}


def scalar_levels(torch, kvq, sigmas, bits, dev):
    """Levels [books][2][2^bits] of the scalar variant: stage 1 = sigma x the
    unit Gaussian Lloyd-Max levels, stage 2 = sigma x sqrt(stage-1 error) x the
    unit Laplacian ones (both from the library's kvq_lloyd_max)."""
    g, dg = kvq.lloyd_max("gaussian", bits)
    lap, _ = kvq.lloyd_max("laplacian", bits)
    rows = [[[v * s for v in g], [v * s * float(np.sqrt(dg)) for v in lap]] for s in sigmas]
    return torch.tensor(rows, dtype=torch.float32, device=dev)


def decode_layers_graph(torch, kvq, q, kc, vc, cb, kw, vw, out, ws, flush, eff_b, reps,
                        n_layers=32):
    """One decode token through n_layers layers: n_layers decode calls, each on
    a layer of its own (codes, codebooks, query and window of the layer's
    shape; codes drawn at random), captured in one HIP graph and replayed after
    a cache-evicting fill; reported per layer.  The launch gaps between calls
    are the graph's, as a decode loop over the layers would have them."""
    g = torch.Generator(device=kc.device).manual_seed(7)
    per = []
    for _ in range(n_layers):
        per.append((torch.randn(q.shape, generator=g, device=q.device),
                    torch.randint(0, 256, kc.shape, generator=g, device=kc.device,
                                  dtype=torch.uint8),
                    torch.randint(0, 256, vc.shape, generator=g, device=vc.device,
                                  dtype=torch.uint8),
                    cb * 1.0, kw.clone() if kw is not None else None,
                    vw.clone() if vw is not None else None))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for (ql, kl, vl, cbl, kwl, vwl) in per:
            kvq.attend_decode(ql, kl, vl, cbl[0], cbl[1], kwl, vwl, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (ql, kl, vl, cbl, kwl, vwl) in per:
            kvq.attend_decode(ql, kl, vl, cbl[0], cbl[1], kwl, vwl, out=out, workspace=ws)
    ts = []
    for i in range(reps + 3):
        flush(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1))
    del graph, per
    t = float(np.median(ts)) * 1e-3 / n_layers
    return {"layers": n_layers, "us_per_layer": round(t * 1e6, 2),
            "gbs": round(eff_b / t / 1e9, 1),
            "note": "decode of one token over n layers of the workload's shape (random codes, "
                    "layers of their own), one HIP graph, caches evicted before the token"}


def rotate_calls(torch, kvq, x, w, dev, flush, reps=20):
    """kvq_rotate alone: the layer's K and V rows (input dtype) -> float32
    rotated rows, flushed caches; HBM-bound (input bytes + 4 bytes per element
    out)."""
    rows = x.reshape(-1, w.head_dim)
    out = torch.empty(rows.shape, dtype=torch.float32, device=dev)
    ms = []
    for i in range(reps + 3):
        flush(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.rotate(rows, out=out)
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    t = float(np.median(ms)) * 1e-3
    nbytes = rows.numel() * (rows.element_size() + 4)
    return {"us": round(t * 1e6, 2), "rows": rows.shape[0], "bytes": nbytes,
            "gbs": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2),
            "note": "all of the layer's K and V rows, input dtype in, float32 out"}


def scalar_calls(torch, kvq, x, q, kw, vw, w, dev, flush, bits=2, reps=20):
    """The scalar residual variant on the same layer (2 bits per stage): encode
    of K and V, reconstruction (unrotated float32), and decode attention over
    the packed codes through the product codebook.  Levels from each book's
    per-element deviation (measured once at set-up)."""
    B, Hkv, Hq, D, W, Tc = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window, w.code_tokens
    sig = [float(torch.sqrt(torch.mean(x[b, :, :Tc].float() ** 2))) for b in range(2)]
    lv = scalar_levels(torch, kvq, sig, bits, dev)
    G = D * bits // 8
    codes = torch.empty((2, B * Hkv, Tc, 2, G), dtype=torch.uint8, device=dev)
    recon = torch.empty((2, B * Hkv, Tc, D), dtype=torch.float32, device=dev)
    kcb = kvq.scalar_product_codebook(lv[0], bits, D)
    vcb = kvq.scalar_product_codebook(lv[1], bits, D)
    kc = codes[0].view(B, Hkv, Tc, 2, G)
    vc = codes[1].view(B, Hkv, Tc, 2, G)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    att_ws = torch.empty(max(kvq.attend_workspace_size(B, Hq, Hkv, D, Tc, W, 2, G, 256), 16),
                         dtype=torch.uint8, device=dev)
    calls = {
        "encode": lambda: kvq.scalar_encode(x, lv, bits, n_rows=Tc, codes=codes),
        "reconstruct": lambda: kvq.scalar_decode_reconstruct(codes, lv, bits, unrotate=True,
                                                            out=recon),
        "decode": lambda: kvq.attend_decode(q, kc, vc, kcb, vcb, kw, vw, out=out,
                                            workspace=att_ws),
    }
    ms = {k: [] for k in calls}
    for i in range(reps + 3):
        for k, f in calls.items():
            flush(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                ms[k].append(e0.elapsed_time(e1))
    med = {k: float(np.median(v)) * 1e-3 for k, v in ms.items()}
    n_vec = 2 * B * Hkv * Tc
    sbytes = 2 * D * bits // 8
    enc_b = n_vec * (2 * D + sbytes)
    rec_b = n_vec * (sbytes + 4 * D)
    dec_b = n_vec * sbytes + 2 * B * Hkv * W * D * 2 + B * Hq * 2 * G * 256 * 4
    res = {"bits": bits, "code_bytes_per_vector": sbytes}
    for k, b in (("encode", enc_b), ("reconstruct", rec_b), ("decode", dec_b)):
        res[k] = {"us": round(med[k] * 1e6, 2), "bytes": b, "gbs": round(b / med[k] / 1e9, 1),
                  "pct_hbm_peak": round(100 * b / med[k] / 1e9 / HBM_PEAK_GBS, 2)}
    res["note"] = ("decode bytes = packed codes + fp16 window + LUT (2 x G x 256 floats per query "
                   "head); the product codebook makes the packed bytes ordinary decode codes")
    return res


def smooth_calls(torch, kvq, x, cb, q, kc, vc, kw, vw, w, dev, flush, reps=20):
    """The dual transform on the same layer: calibrating the key factors
    (one row per KV head) over the coded tokens, encoding the keys with and
    without the division, and decode with the factors folded into the query.
    Each timed call follows a cache-evicting write, like the step."""
    B, Hkv, Hq, D, W = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window
    S, G, C, Tc = w.n_stages, w.n_groups, w.n_codewords, w.code_tokens
    xk, cbk = x[:1], cb[:1]
    lam = torch.empty((1, Hkv, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kvq.encode_workspace_size(D, G, S, C, 1), 16), dtype=torch.uint8,
                     device=dev)
    codes = torch.empty((1, B * Hkv, Tc, S, G), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    att_ws = torch.empty(max(kvq.attend_workspace_size(B, Hq, Hkv, D, Tc, W, S, G, C), 16),
                         dtype=torch.uint8, device=dev)
    kvq.encode(xk, cbk, n_rows=Tc, codes=codes, workspace=ws)          # packs the K books
    calls = {
        "calibrate": lambda: kvq.smooth_calibrate(xk, Hkv, n_rows=Tc, out=lam),
        "encode_k_smooth": lambda: kvq.encode(xk, cbk, n_rows=Tc, codes=codes, workspace=ws,
                                              packed=True, smooth=lam),
        "encode_k_plain": lambda: kvq.encode(xk, cbk, n_rows=Tc, codes=codes, workspace=ws,
                                             packed=True),
        "decode_smooth": lambda: kvq.attend_decode(q, kc, vc, cb[0], cb[1], kw, vw, out=out,
                                                   workspace=att_ws, k_smooth=lam[0]),
    }
    ms = {k: [] for k in calls}
    for i in range(reps + 3):
        for k, f in calls.items():
            flush(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                ms[k].append(e0.elapsed_time(e1))
    med = {k: float(np.median(v)) for k, v in ms.items()}
    cal_bytes = B * Hkv * Tc * D * 2
    return {"calibrate_us": round(med["calibrate"] * 1e3, 2),
            "calibrate_gbs": round(cal_bytes / (med["calibrate"] * 1e-3) / 1e9, 1),
            "encode_k_smooth_us": round(med["encode_k_smooth"] * 1e3, 2),
            "encode_k_plain_us": round(med["encode_k_plain"] * 1e3, 2),
            "decode_smooth_us": round(med["decode_smooth"] * 1e3, 2),
            "note": f"keys of the layer ({B * Hkv * Tc} vectors), factors one row per KV head"}


def fit_calls(torch, kvq, x, cb, w, dev, sample=65536, n_iter=10, reps=5):
    """K-means fitting of the layer's key codebooks on a sample of ``sample``
    vectors: the first sample / (sequences x KV heads) tokens of every
    (sequence, KV head) (8,192 of each of the 8 KV heads for the Llama-shaped
    layer), ``n_iter`` Lloyd iterations from the layer's codebooks."""
    D, S, G, C = w.head_dim, w.n_stages, w.n_groups, w.n_codewords
    xk = x[0]                                           # [B*Hkv][T][D] keys, rows [0, rows) used
    H = xk.shape[0]
    rows = min(sample // H, xk.shape[1])
    ws = torch.empty(kvq.codebook_fit_workspace_size(D, G, S, C, H * rows), dtype=torch.uint8,
                     device=dev)
    cb0 = cb[0].clone()
    out = cb0.clone()
    ms = []
    for i in range(reps + 1):
        out.copy_(cb0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.codebook_fit(xk, out, n_iter, n_rows=rows, workspace=ws, inplace=True)
        e1.record()
        torch.cuda.synchronize()
        if i >= 1:
            ms.append(e0.elapsed_time(e1))
    t = float(np.median(ms))
    return {"ms": round(t, 4), "ms_per_iteration": round(t / n_iter, 4), "vectors": H * rows,
            "n_iter": n_iter, "stages": S,
            "note": "per iteration: assignment (codebook packing + encode of the sample) + "
                    "fixed-point centroid sums + update; the sample is L2/Infinity-Cache resident"}


def stream_calls(torch, kvq, inp, w, dev, reps=20, wcap=192, n_flush=64):
    """Latency of the streaming calls on the same layer: one window append
    (a token per KV head) and one flush of the oldest 64 window tokens of
    every KV head (K and V encoded into codes, the window compacted).  Each
    timed call starts from a full window of wcap tokens."""
    B, H, D = w.batch, w.n_kv_heads, w.head_dim
    S, G, C = w.n_stages, w.n_groups, w.n_codewords
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    kw = torch.randn((B, H, wcap, D), generator=g, device=dev).to(torch.float16)
    vw = torch.randn((B, H, wcap, D), generator=g, device=dev).to(torch.float16)
    kc = torch.zeros((B, H, w.tokens, S, G), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    kcb = torch.from_numpy(inp["cb"][0]).to(dev)
    vcb = torch.from_numpy(inp["cb"][1]).to(dev)
    ws = torch.empty(max(kvq.window_flush_workspace_size(D, G, S, C), 16), dtype=torch.uint8,
                     device=dev)
    kn = torch.randn((B, H, D), generator=g, device=dev).to(torch.float16)
    vn = torch.randn((B, H, D), generator=g, device=dev).to(torch.float16)
    tf, ta = [], []
    kvq.window_flush(kw, vw, wcap, n_flush, kc, vc, 0, kcb, vcb, workspace=ws)   # packs the books
    for i in range(reps + 3):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        kvq.window_flush(kw, vw, wcap, n_flush, kc, vc, (i % 8) * n_flush, kcb, vcb, workspace=ws,
                         packed=True)
        e[1].record()
        kvq.window_append(kn, vn, kw, vw, wcap - n_flush)
        e[2].record()
        torch.cuda.synchronize()
        if i >= 3:
            tf.append(e[0].elapsed_time(e[1]))
            ta.append(e[1].elapsed_time(e[2]))
    return {"flush_us": round(float(np.median(tf)) * 1e3, 2),
            "append_us": round(float(np.median(ta)) * 1e3, 2),
            "flush_vectors": 2 * B * H * n_flush, "window_cap": wcap,
            "note": "flush = K and V encode of the oldest tokens (codebooks packed once) + "
                    "window compaction"}


def cpu_baseline(w, inp, codes, eff_b, dec_gbs, budget_s=10.0, enc_budget_s=6.0):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: whole decode calls (all sequences, KV heads and query heads,
    every coded token plus the window) repeated until at least ``budget_s``
    seconds have passed (one call of the long-context layer takes longer),
    then encode of growing batches of the layer's key vectors until
    ``enc_budget_s`` seconds have passed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = os.cpu_count()
    B, Hkv, Tc, S, G = w.batch, w.n_kv_heads, w.code_tokens, w.n_stages, w.n_groups
    c = codes.cpu().numpy()
    kc = c[0].reshape(B, Hkv, Tc, S, G)
    vc = c[1].reshape(B, Hkv, Tc, S, G)
    reps, t_dec = 0, 0.0
    while t_dec < budget_s:
        t0 = time.perf_counter()
        oracle.attend(inp["q"], kc, vc, inp["cb"][0], inp["cb"][1],
                      inp["k_win"] if w.window else None, inp["v_win"] if w.window else None)
        t_dec += time.perf_counter() - t0
        reps += 1
    gbs = eff_b * reps / t_dec / 1e9
    xs_all = inp["x_f32"][0].reshape(-1, w.head_dim)
    n_enc, t_enc, n = 0, 0.0, 4096
    while t_enc < enc_budget_s and n_enc < xs_all.shape[0]:
        xs = xs_all[n_enc:n_enc + n].astype(np.float64)
        t0 = time.perf_counter()
        oracle.rvq_encode(xs, inp["cb"][0])
        t_enc += time.perf_counter() - t0
        n_enc += xs.shape[0]
        n *= 2
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(blas), "kind": "oracle",
            "sample": f"decode: {reps} whole decode calls of the workload ({B * Hkv} (sequence, "
                      f"KV head) pairs, {w.n_q_heads} query heads, {Tc} coded + {w.window} window "
                      f"tokens) in {t_dec:.1f} s; encode: the first {n_enc} K vectors in "
                      f"{t_enc:.1f} s. float64 NumPy; elementwise work on one core, matrix "
                      f"products on {blas} BLAS threads",
            "encode_mvec_per_s": round(n_enc / t_enc / 1e6, 6),
            "gpu_over_cpu_decode": round(dec_gbs / gbs, 1),
            "host": host_cpu()}


def host_cpu():
    """The host the oracle ran on: CPU model, logical CPUs, the CPUs this
    process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity": affinity}


if __name__ == "__main__":
    main()
