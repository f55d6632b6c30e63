"""Parity of the dual-transform calls (per-channel smoothing of the keys by
sqrt(max |K_i|) ahead of the rotation, folded into the query at decode) with
the float64 oracle, through the C ABI.

Bars: calibrated factors bit-exact (float32 of the oracle's float64 square
root of an exact maximum; the square root of a float32-exact value rounded
through float64 equals the correctly rounded float32 one); codes exact except
accepted near ties; reconstruction per channel within 1e-6 * |x_hat| after
dividing out the factor; attention 2e-3 max-abs and 1e-3 relative L2.  Factors
of 1 must reproduce the plain calls bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import compressed_attention_fwht_amd as kvq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_dev(inp_x, w):
    if w.x_dtype == "bf16":
        return torch.from_numpy(inp_x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(inp_x).cuda()


def key_setup(w, inp, n_scale):
    """Oracle factors of the coded keys (float32, as the calls take them) and
    K codebooks rescaled to the smoothed keys' per-coordinate RMS (a power of
    two, so the workload's codebook law keeps its shape)."""
    Tc = w.code_tokens
    k = inp["x_f32"][0][:, :Tc].astype(np.float64)
    lam = oracle.smooth_factors(k, n_scale).astype(np.float32)
    rows = oracle.smooth_rows(lam, np.arange(w.n_seq))[:, None, :]
    ratio = np.sqrt(np.mean((k / rows) ** 2) / np.mean(k ** 2))
    kcb = (inp["cb"][0] * np.float32(2.0 ** np.round(np.log2(ratio)))).astype(np.float32)
    return lam, kcb


# -------------------------------------------------------------- calibration
@pytest.mark.parametrize("key,over,n_scale,n_rows", [
    (2, dict(tokens=1300, window=128), 8, 1172),       # one row per KV head, bf16
    (2, dict(tokens=1300, window=128), 1, 1300),       # one row per book
    (2, dict(tokens=700, window=0), 3, 513),           # rows shared unevenly
    (3, dict(batch=3, tokens=600, window=64), 12, 600),  # one row per sequence
    (1, dict(), 1, 1024),                              # fp32 input, D = 64
])
def test_smooth_calibrate_bit_exact(key, over, n_scale, n_rows):
    say(f"smooth calibrate workload {key} {over} n_scale={n_scale} rows={n_rows}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    x = to_dev(inp["x"], w)
    got = kvq.smooth_calibrate(x, n_scale, n_rows=n_rows).cpu().numpy()
    for b in range(x.shape[0]):
        ref = oracle.smooth_factors(inp["x_f32"][b][:, :n_rows].astype(np.float64), n_scale)
        assert np.array_equal(got[b], ref.astype(np.float32)), (b, np.abs(got[b] - ref).max())


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_smooth_calibrate_every_instance(D, dt):
    """Every (head size, input dtype) instance of the channel-maximum kernel
    on random rows (two books, three sequences sharing two factor rows, a
    ragged row count): bit-exact against the oracle."""
    say(f"smooth calibrate instance D {D} {dt}")
    rng = np.random.default_rng(7100 + D + len(dt))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    x = torch.from_numpy((rng.standard_normal((2, 3, 203, D)) *
                          rng.uniform(0.1, 8.0, size=(1, 1, 1, D))).astype(np.float32)).to(tdt).cuda()
    got = kvq.smooth_calibrate(x, 2, n_rows=190).cpu().numpy()
    xf = x.double().cpu().numpy()
    for b in range(2):
        ref = oracle.smooth_factors(xf[b][:, :190], 2)
        assert np.array_equal(got[b], ref.astype(np.float32)), (b, np.abs(got[b] - ref).max())


def test_smooth_calibrate_special_inputs():
    say("smooth calibrate: f16 input, zero channels, empty rows, unmapped rows")
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((2, 5, 40, 128)) * np.exp(rng.uniform(-3, 3, 128))).astype(np.float16)
    x[:, :, :, 7] = 0                                   # an all-zero channel -> 1
    x[1, 2, :, 9] = -0.0
    xd = cuda(x)
    got = kvq.smooth_calibrate(xd, 7).cpu().numpy()     # rows 5, 6 have no sequence -> 1
    for b in range(2):
        ref = oracle.smooth_factors(x[b].astype(np.float64), 7).astype(np.float32)
        assert np.array_equal(got[b], ref)
    assert np.all(got[:, :, 7] == 1.0) and np.all(got[:, 5:] == 1.0)
    ones = kvq.smooth_calibrate(xd, 2, n_rows=0).cpu().numpy()
    assert np.all(ones == 1.0)
    # a second call into the same buffer starts from scratch
    out = torch.full((2, 3, 128), 1e30, dtype=torch.float32, device="cuda")
    again = kvq.smooth_calibrate(xd, 3, out=out).cpu().numpy()
    for b in range(2):
        assert np.array_equal(again[b], oracle.smooth_factors(x[b].astype(np.float64), 3)
                              .astype(np.float32))


# ------------------------------------------------------------------- encode
@pytest.mark.parametrize("key,over,n_scale", [
    (2, dict(tokens=1300, window=128), 8),             # S = 1, outlier channels
    (3, dict(batch=2, tokens=700, window=64), 4),      # S = 2, one row per KV head
    (4, dict(tokens=900, window=256), 1),              # S = 4, Laplace with channel scales
    (1, dict(), 1),                                    # D = 64, generic kernel
])
@pytest.mark.parametrize("generic", [False, True])
def test_encode_smooth_parity(key, over, n_scale, generic):
    say(f"encode smooth workload {key} {over} n_scale={n_scale} generic={generic}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    lam, kcb = key_setup(w, inp, n_scale)
    x = to_dev(inp["x"], w)[:1]                         # the keys
    codes = kvq.encode(x, cuda(kcb[None]), n_rows=Tc, generic=generic,
                       smooth=cuda(lam[None])).cpu().numpy()[0]
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(w.n_seq))[:, None, :]
    xs = oracle.smooth_keys(inp["x_f32"][0][:, :Tc].astype(np.float64), rows)
    res = oracle.check_codes(xs.reshape(-1, w.head_dim), kcb,
                             codes.reshape(-1, w.n_stages, w.n_groups))
    say("   ", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
    assert res["hard"] == 0 and res["exact"] >= 0.999 * res["total"]


@pytest.mark.parametrize("generic", [False, True])
def test_encode_smooth_unit_factors_equal_plain(generic):
    say(f"encode smooth with factors 1, generic={generic}")
    w = synth.workload(3, batch=1, tokens=1100, window=0)
    inp = synth.make_inputs(w)
    x, cb = to_dev(inp["x"], w), cuda(inp["cb"])
    ones = torch.ones((2, 3, 128), dtype=torch.float32, device="cuda")
    assert torch.equal(kvq.encode(x, cb, generic=generic, smooth=ones),
                       kvq.encode(x, cb, generic=generic))


# -------------------------------------------------------------- reconstruct
@pytest.mark.parametrize("key,over,n_scale", [
    (2, dict(tokens=1300, window=0), 8),
    (3, dict(batch=2, tokens=500, window=0), 3),
    (1, dict(), 1),
])
def test_reconstruct_smooth_parity(key, over, n_scale):
    say(f"reconstruct smooth workload {key} {over} n_scale={n_scale}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    lam, kcb = key_setup(w, inp, n_scale)
    rng = np.random.default_rng(key)
    codes = rng.integers(0, 256, size=(1, w.n_seq, w.tokens, w.n_stages, w.n_groups),
                         dtype=np.uint8)
    got = kvq.decode_reconstruct(cuda(codes), cuda(kcb[None]),
                                 smooth=cuda(lam[None])).cpu().numpy()[0].astype(np.float64)
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(w.n_seq))[:, None, :]
    plain = oracle.reconstruct(codes[0], kcb)
    ref = oracle.reconstruct_smooth(codes[0], kcb, rows)
    err = np.abs(got - ref) / rows                       # back to the unsmoothed scale
    bound = 1e-6 * np.linalg.norm(plain, axis=-1, keepdims=True)
    assert np.all(err <= bound), float(np.max(err / bound))


# ------------------------------------------------------------------- decode
def _decode_smooth(w, inp, ck, cv, lam, kcb, **kw):
    B, Hkv, Tc = w.batch, w.n_kv_heads, w.code_tokens
    ck = ck.reshape(B, Hkv, Tc, w.n_stages, w.n_groups)
    cv = cv.reshape(B, Hkv, Tc, w.n_stages, w.n_groups)
    W = w.window
    kwin = inp["k_win"] if W > 0 else None
    vwin = inp["v_win"] if W > 0 else None
    got = kvq.attend_decode(cuda(inp["q"]), cuda(ck), cuda(cv), cuda(kcb), cuda(inp["cb"][1]),
                            None if kwin is None else cuda(kwin),
                            None if vwin is None else cuda(vwin), k_smooth=cuda(lam),
                            **kw).cpu().numpy()
    ref = oracle.attend(inp["q"], ck, cv, kcb, inp["cb"][1], kwin, vwin,
                        k_smooth=lam.astype(np.float64))
    return oracle.check_attn(got, ref)


@pytest.mark.parametrize("key,over,n_scale", [
    (2, dict(tokens=3000, window=128), 8),             # window slices on the chunk blocks
    (3, dict(batch=3, tokens=2100, window=64), 4),     # GQA 7 (head splits)
    (3, dict(batch=2, tokens=1500, window=33), 6),     # one row per sequence
    (4, dict(tokens=5000, window=2300), 1),            # window blocks of their own
])
def test_decode_smooth_parity(key, over, n_scale):
    say(f"decode smooth workload {key} {over} n_scale={n_scale}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    lam, kcb = key_setup(w, inp, n_scale)
    Tc = w.code_tokens
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(w.n_seq))[:, None, :]
    ck = oracle.smooth_encode(inp["x_f32"][0][:, :Tc].astype(np.float64), rows, kcb)
    cv = oracle.rvq_encode(inp["x_f32"][1][:, :Tc].reshape(-1, w.head_dim), inp["cb"][1])
    res = _decode_smooth(w, inp, ck, cv, lam, kcb)
    say("   ", res)
    assert res["ok"], res


@pytest.mark.parametrize("key,over", [
    (4, dict(tokens=40000, window=256)),                 # rotated-code kernels' prep tables
    (2, dict(batch=3, tokens=7000, window=128, n_stages=3)),  # attn_lut_kernel's tables
])
def test_decode_smooth_table_pass(key, over):
    """Long caches whose tables come from a pass of their own, the factors
    folded into the query there: the rotated-code kernels' prep kernel (four
    stages) and attn_lut_kernel (three stages, where building the LUT in every
    chunk block would re-read more than 96 MB of codebook)."""
    say(f"decode smooth, tables from their own pass: workload {key} {over} (random codes)")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    lam, kcb = key_setup(w, inp, 8)
    rng = np.random.default_rng(9)
    shp = (w.batch * w.n_kv_heads * w.code_tokens, w.n_stages, w.n_groups)
    ck = rng.integers(0, 256, size=shp, dtype=np.uint8)
    cv = rng.integers(0, 256, size=shp, dtype=np.uint8)
    res = _decode_smooth(w, inp, ck, cv, lam, kcb)
    say("   ", res)
    assert res["ok"], res


def test_decode_smooth_unit_factors_equal_plain():
    say("decode smooth with factors 1")
    w = synth.workload(3, batch=2, tokens=1500, window=33)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(2)
    shp = (w.batch, w.n_kv_heads, w.code_tokens, w.n_stages, w.n_groups)
    ck = cuda(rng.integers(0, 256, size=shp, dtype=np.uint8))
    cv = cuda(rng.integers(0, 256, size=shp, dtype=np.uint8))
    args = (cuda(inp["q"]), ck, cv, cuda(inp["cb"][0]), cuda(inp["cb"][1]), cuda(inp["k_win"]),
            cuda(inp["v_win"]))
    ones = torch.ones((w.n_kv_heads, 128), dtype=torch.float32, device="cuda")
    assert torch.equal(kvq.attend_decode(*args, k_smooth=ones), kvq.attend_decode(*args))


# ---------------------------------------------------------------- streaming
@pytest.mark.parametrize("key,over,wcap,nflush", [
    (3, dict(batch=2, tokens=300, window=0), 96, 64),     # MFMA encode (small-batch blocks)
    (1, dict(tokens=150, window=0), 40, 24),              # generic encode, D = 64
])
def test_streaming_smooth_parity(key, over, wcap, nflush):
    """Appends and smoothing flushes: flushed key codes follow the smoothed
    keys, value codes the plain ones, and decode over the grown cache with the
    factors matches the oracle on the same codes."""
    say(f"streaming smooth workload {key} {over} cap {wcap} flush {nflush}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    B, H, T, D = w.batch, w.n_kv_heads, w.tokens, w.head_dim
    S, G = w.n_stages, w.n_groups
    tk = inp["x_f32"][0].reshape(B, H, T, D).astype(np.float16)
    tv = inp["x_f32"][1].reshape(B, H, T, D).astype(np.float16)
    lam = oracle.smooth_factors(tk.reshape(B * H, T, D).astype(np.float64), B * H)
    lam = lam.astype(np.float32)
    kcb, vcb = inp["cb"][0] * np.float32(0.25), inp["cb"][1]
    kw = torch.zeros((B, H, wcap, D), dtype=torch.float16, device="cuda")
    vw = torch.zeros_like(kw)
    kc = torch.zeros((B, H, T, S, G), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    kcb_d, vcb_d, lam_d = cuda(kcb), cuda(vcb), cuda(lam)
    tk_d, tv_d = cuda(tk), cuda(tv)
    ws = torch.empty(max(kvq.window_flush_workspace_size(D, G, S, w.n_codewords), 16),
                     dtype=torch.uint8, device="cuda")
    nw = nc = flushes = 0
    for t in range(T):
        if nw == wcap:
            kvq.window_flush(kw, vw, nw, nflush, kc, vc, nc, kcb_d, vcb_d, workspace=ws,
                             packed=flushes > 0, k_smooth=lam_d)
            flushes += 1
            nw, nc = nw - nflush, nc + nflush
        kvq.window_append(tk_d[:, :, t].contiguous(), tv_d[:, :, t].contiguous(), kw, vw, nw)
        nw += 1
    torch.cuda.synchronize()
    assert flushes >= 2
    assert np.array_equal(kw.cpu().numpy()[:, :, :nw], tk[:, :, nc:])
    kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(B * H)).reshape(B, H, 1, D)
    ks = oracle.smooth_keys(tk[:, :, :nc].astype(np.float64), rows)
    for codes, xs, cb in ((kcn, ks, kcb), (vcn, tv[:, :, :nc].astype(np.float64), vcb)):
        res = oracle.check_codes(xs.reshape(-1, D), cb, codes[:, :, :nc].reshape(-1, S, G))
        say("   codes", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
        assert res["hard"] == 0
    q = np.random.default_rng(6).standard_normal((B, w.n_q_heads, D)).astype(np.float32)
    got = kvq.attend_decode(cuda(q), kc, vc, kcb_d, vcb_d, kw, vw, n_code=nc, n_window=nw,
                            k_smooth=lam_d).cpu().numpy()
    ref = oracle.attend(q, kcn[:, :, :nc], vcn[:, :, :nc], kcb, vcb, tk[:, :, nc:], tv[:, :, nc:],
                        k_smooth=lam.astype(np.float64))
    res = oracle.check_attn(got, ref)
    say("   decode", res)
    assert res["ok"], res


# ----------------------------------------------------- full size (sampled)
def test_full_size_smooth_llama_layer():
    """The Llama-shaped layer at full size: calibrate the key factors on the
    GPU (bit-exact), encode the keys with them (sampled code check), decode
    with the folded query against the oracle on the same codes."""
    say("full-size Llama-shaped layer with the dual transform")
    w = synth.workload(2)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    x = to_dev(inp["x"], w)
    lam_d = kvq.smooth_calibrate(x[:1], w.n_kv_heads, n_rows=Tc)
    lam, kcb = key_setup(w, inp, w.n_kv_heads)
    assert np.array_equal(lam_d.cpu().numpy()[0], lam)
    kc = kvq.encode(x[:1], cuda(kcb[None]), n_rows=Tc, smooth=lam_d).cpu().numpy()[0]
    vc = kvq.encode(x[1:], cuda(inp["cb"][1:]), n_rows=Tc).cpu().numpy()[0]
    del x
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(w.n_seq))[:, None, :]
    xs = oracle.smooth_keys(inp["x_f32"][0][:, :Tc].astype(np.float64), rows).reshape(-1, 128)
    flat = kc.reshape(-1, 1, 16)
    idx = np.arange(0, flat.shape[0], 97)
    res = oracle.check_codes(xs[idx], kcb, flat[idx])
    say("   keys", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
    assert res["hard"] == 0
    res = _decode_smooth(w, inp, kc, vc, lam, kcb)
    say("   decode", res)
    assert res["ok"], res
