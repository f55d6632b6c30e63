"""Parity of the HIP library (through its C ABI) with the float64 oracle.

Tolerances (see oracle/check.py): codes exact except accepted near ties
(relative 1e-4), reconstruction 1e-6 absolute (and bit-exact to the rounded
float64 sum), attention 2e-3 max-abs and 1e-3 relative L2.  Inputs come from
the seeded workload generator; the reduced sizes keep the distributions of
the named workloads and span several tiles plus a ragged tail.
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


def to_dev(inp_x, w):
    if w.x_dtype == "bf16":
        return torch.from_numpy(inp_x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(inp_x).cuda()


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------ rotate
@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotate_identity_is_orthonormal(D):
    say(f"rotate identity D={D}")
    y = kvq.rotate(torch.eye(D, dtype=torch.float32, device="cuda")).double().cpu().numpy()
    assert np.max(np.abs(y @ y.T - np.eye(D))) <= 1e-6
    assert np.max(np.abs(y - oracle.hadamard_matrix(D))) <= 1e-7


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D,n", [(64, 1), (64, 1001), (128, 63), (128, 4097), (256, 333)])
def test_rotate_parity(dt, D, n):
    say(f"rotate parity dtype={dt} D={D} rows={n}")
    g = torch.Generator().manual_seed(D * 7 + n)
    x = (torch.randn(n, D, generator=g) * 3).to(dt)
    y = kvq.rotate(x.cuda()).cpu().double().numpy()
    xd = x.double().numpy()
    ref = oracle.fwht(xd)
    nrm = np.linalg.norm(xd, axis=1)
    assert np.max(np.abs(y - ref).max(axis=1) / nrm) <= 1e-6
    assert np.max(np.abs(np.linalg.norm(y, axis=1) - nrm) / nrm) <= 1e-6


def test_rotate_in_place_f32():
    say("rotate in place")
    x = torch.randn(777, 128, dtype=torch.float32)
    xd = x.cuda()
    kvq.rotate(xd, out=xd)
    assert np.max(np.abs(xd.cpu().double().numpy() - oracle.fwht(x.double().numpy()))) <= 1e-5


# ------------------------------------------------------------- reconstruct
@pytest.mark.parametrize("key", [1, 2, 3, 4])
def test_reconstruct_parity(key):
    say(f"reconstruct parity workload {key}")
    w = synth.workload(key)
    cb = synth.make_codebooks(w)[:2]                        # K and V books
    rng = np.random.default_rng(key)
    n = 2000 + 17
    codes = rng.integers(0, w.n_codewords, size=(2, n, w.n_stages, w.n_groups), dtype=np.uint8)
    got = kvq.decode_reconstruct(cuda(codes), cuda(cb)).cpu().numpy()
    for b in range(2):
        ref = oracle.reconstruct_rot(codes[b], cb[b])
        assert np.array_equal(got[b], ref.astype(np.float32))     # correctly rounded sum
        assert oracle.check_recon(got[b], ref)["ok"]
    got_u = kvq.decode_reconstruct(cuda(codes), cuda(cb), unrotate=True).cpu().numpy()
    for b in range(2):
        ref = oracle.reconstruct(codes[b], cb[b])
        nrm = np.linalg.norm(ref, axis=1, keepdims=True)
        assert np.max(np.abs(got_u[b] - ref) / nrm) <= 1e-6


def test_reconstruct_out_of_range_codes_clamp():
    say("reconstruct clamp")
    rng = np.random.default_rng(0)
    cb = rng.standard_normal((1, 2, 16, 100, 8)).astype(np.float32)
    codes = rng.integers(0, 256, size=(1, 300, 2, 16), dtype=np.uint8)
    got = kvq.decode_reconstruct(cuda(codes), cuda(cb)).cpu().numpy()
    ref = oracle.reconstruct_rot(np.minimum(codes[0], 99), cb[0]).astype(np.float32)
    assert np.array_equal(got[0], ref)


@pytest.mark.parametrize("D,G,C,n", [
    (128, 16, 256, 1),          # one vector: a single partial row group
    (128, 16, 256, 5),
    (128, 16, 100, 777),        # C < 256 with out-of-range codes (clamped)
    (64, 8, 256, 3001),         # 64 KiB of codebooks: two blocks per CU
    (256, 32, 64, 1234),        # D = 256 in LDS (C = 64)
])
@pytest.mark.parametrize("S", [1, 2, 4])
def test_reconstruct_lds_shapes(D, G, C, n, S):
    """Books whose per-stage codebooks fit the LDS kernel (stage 0 in LDS, later
    stages through the caches), at ragged and tiny sizes; rotated output
    bit-exact, unrotated within 1e-6 * |x_hat|."""
    say(f"reconstruct, LDS kernel: D {D} G {G} C {C} n {n} S {S}")
    rng = np.random.default_rng(D + C + n + S)
    dsub = D // G
    cb = rng.standard_normal((2, S, G, C, dsub)).astype(np.float32)
    codes = rng.integers(0, 256, size=(2, n, S, G), dtype=np.uint8)
    clamped = np.minimum(codes, C - 1)
    got = kvq.decode_reconstruct(cuda(codes), cuda(cb)).cpu().numpy()
    got_u = kvq.decode_reconstruct(cuda(codes), cuda(cb), unrotate=True).cpu().numpy()
    for b in range(2):
        ref = oracle.reconstruct_rot(clamped[b], cb[b])
        assert np.array_equal(got[b], ref.astype(np.float32))
        ref_u = oracle.reconstruct(clamped[b], cb[b])
        nrm = np.linalg.norm(ref_u, axis=1, keepdims=True)
        assert np.max(np.abs(got_u[b] - ref_u) / nrm) <= 1e-6


@pytest.mark.parametrize("G,n", [
    (16, 520192),               # the Qwen-shaped layer's K (or V) vectors per book
    (2, 100001),                # 4 code bytes per row: batches start off 16-byte boundaries
])
def test_reconstruct_two_stages_many_batches(G, n):
    """Two-stage books at sizes where every block of the half-table kernel
    codes several batches (the halves taken in alternating order, the code
    rows of each batch copied into LDS): rotated output bit-exact everywhere,
    unrotated within 1e-6 * |x_hat| on every 97th vector."""
    say(f"reconstruct, two stages: G {G} n {n} x 2 books")
    D, S, C = 128, 2, 256
    rng = np.random.default_rng(G + n)
    cb = rng.standard_normal((2, S, G, C, D // G)).astype(np.float32)
    codes = rng.integers(0, 256, size=(2, n, S, G), dtype=np.uint8)
    dc, dcb = cuda(codes), cuda(cb)
    got = kvq.decode_reconstruct(dc, dcb).cpu().numpy()
    got_u = kvq.decode_reconstruct(dc, dcb, unrotate=True).cpu().numpy()
    idx = np.arange(0, n, 97)
    for b in range(2):
        ref = oracle.reconstruct_rot(codes[b], cb[b])
        assert np.array_equal(got[b], ref.astype(np.float32))
        ref_u = oracle.reconstruct(codes[b][idx], cb[b])
        nrm = np.linalg.norm(ref_u, axis=1, keepdims=True)
        assert np.max(np.abs(got_u[b][idx] - ref_u) / nrm) <= 1e-6


def test_reconstruct_full_size_llama_layer_sampled():
    """The Llama-shaped layer's K and V books at full size (261,120 vectors each,
    the bench's launch), every 97th vector against the oracle."""
    say("reconstruct, full-size Llama-shaped layer, sampled")
    w = synth.workload(2)
    cb = synth.make_codebooks(w)[:2]
    rng = np.random.default_rng(11)
    n = w.n_kv_heads * w.code_tokens
    codes = rng.integers(0, 256, size=(2, n, 1, w.n_groups), dtype=np.uint8)
    got_u = kvq.decode_reconstruct(cuda(codes), cuda(cb), unrotate=True).cpu().numpy()
    idx = np.arange(0, n, 97)
    for b in range(2):
        ref = oracle.reconstruct(codes[b][idx], cb[b])
        nrm = np.linalg.norm(ref, axis=1, keepdims=True)
        assert np.max(np.abs(got_u[b][idx] - ref) / nrm) <= 1e-6


# ------------------------------------------------------------------ encode
SMALL_ENCODE = [
    (1, dict()),                                              # tiny, full size
    (2, dict(tokens=1300, window=128)),                       # n_rows 1172 < stride
    (3, dict(batch=2, tokens=700, window=64)),
    (4, dict(tokens=900, window=256)),
    (5, dict(layers=2, tokens=333)),
]


def _encode_case(key, over, generic=False, pre_rotated=False, f16=False):
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    x = to_dev(inp["x"], w)
    xf = inp["x_f32"].astype(np.float64)
    if f16:
        x = x.float().half()
        xf = x.float().cpu().numpy().astype(np.float64)
    if pre_rotated:
        xr = oracle.fwht(xf)
        x = torch.from_numpy(xr.astype(np.float32)).cuda()
        if w.x_dtype == "bf16":
            x = x.bfloat16()
        xf = x.double().cpu().numpy()
    n_rows = w.tokens - w.window
    codes = kvq.encode(x, cuda(inp["cb"]), n_rows=n_rows, generic=generic,
                       pre_rotated=pre_rotated).cpu().numpy()
    tot = {"total": 0, "exact": 0, "near_tie": 0, "hard": 0}
    for b in range(x.shape[0]):
        xb = xf[b][:, :n_rows].reshape(-1, w.head_dim)
        res = oracle.check_codes(xb, inp["cb"][b], codes[b].reshape(-1, w.n_stages, w.n_groups),
                                 rotate=not pre_rotated)
        for k in tot:
            tot[k] += res[k]
        assert res["hard"] == 0, (key, b, res)
    return tot


@pytest.mark.parametrize("key,over", SMALL_ENCODE)
@pytest.mark.parametrize("generic", [False, True])
def test_encode_parity(key, over, generic):
    say(f"encode parity workload {key} {over} generic={generic}")
    tot = _encode_case(key, over, generic=generic)
    say("   ", tot)
    assert tot["exact"] >= 0.999 * tot["total"]


def test_encode_pre_rotated_and_f16():
    say("encode pre-rotated bf16 / f16 input")
    for pre, f16 in ((True, False), (False, True)):
        tot = _encode_case(3, dict(batch=1, tokens=1100, window=64), pre_rotated=pre, f16=f16)
        assert tot["hard"] == 0 and tot["exact"] >= 0.999 * tot["total"]


def test_encode_packed_codebooks_reused():
    say("encode with codebooks packed by an earlier call")
    w = synth.workload(3, batch=1, tokens=1500, window=0)
    inp = synth.make_inputs(w)
    x = to_dev(inp["x"], w)
    cb = cuda(inp["cb"])
    ws = torch.empty(kvq.encode_workspace_size(128, 16, 2, 256, 2), dtype=torch.uint8,
                     device="cuda")
    first = kvq.encode(x, cb, workspace=ws)
    again = kvq.encode(x, cb, workspace=ws, packed=True)
    assert torch.equal(first, again)
    # the packed copy, not the float codebooks, is what the packed call reads
    garbage = torch.full_like(cb, float("nan"))
    assert torch.equal(kvq.encode(x, garbage, workspace=ws, packed=True), first)


def test_encode_deterministic():
    say("encode determinism")
    w = synth.workload(2, tokens=2000, window=0)
    inp = synth.make_inputs(w)
    x, cb = to_dev(inp["x"], w), cuda(inp["cb"])
    a = kvq.encode(x, cb)
    b = kvq.encode(x, cb)
    assert torch.equal(a, b)


def test_encode_codeword_inputs_return_own_index():
    """Pre-rotated inputs that are exactly codeword rows come back with their
    own indices, on both kernels."""
    say("encode codeword inputs")
    rng = np.random.default_rng(4)
    cb = (rng.standard_normal((1, 1, 16, 256, 8)) * 0.5).astype(np.float32)
    z = rng.integers(0, 256, size=(512, 16))
    x = np.stack([np.concatenate([cb[0, 0, g, z[n, g]] for g in range(16)]) for n in range(512)])
    xb = torch.from_numpy(x).cuda().bfloat16()                   # bf16-exact codewords needed
    xq = xb.double().cpu().numpy()
    cbq = np.empty_like(cb)
    for g in range(16):                                            # book holding the bf16 rows
        cbq[0, 0, g] = cb[0, 0, g]
        cbq[0, 0, g, z[:, g]] = xq[:, 8 * g:8 * g + 8]
    for generic in (False, True):
        codes = kvq.encode(xb.view(1, 1, 512, 128), cuda(cbq), pre_rotated=True,
                           generic=generic).cpu().numpy()
        assert np.array_equal(codes[0, 0, :, 0, :], z)


# ------------------------------------------------------------------ decode
SMALL_DECODE = [
    (1, dict()),
    (2, dict(tokens=3000, window=128)),
    (3, dict(batch=3, tokens=2100, window=64)),
    (4, dict(tokens=5000, window=256)),
]


def _decode_case(w, inp, codes_k, codes_v, **kw):
    B, Hkv, Tc = w.batch, w.n_kv_heads, w.code_tokens
    ck = codes_k.reshape(B, Hkv, Tc, w.n_stages, w.n_groups)
    cv = codes_v.reshape(B, Hkv, Tc, w.n_stages, w.n_groups)
    kwin = inp.get("k_win")
    vwin = inp.get("v_win")
    kw_t = cuda(kwin) if kwin is not None and w.window > 0 else None
    vw_t = cuda(vwin) if vwin is not None and w.window > 0 else None
    got = kvq.attend_decode(cuda(inp["q"]), cuda(ck), cuda(cv), cuda(inp["cb"][0]),
                            cuda(inp["cb"][1]), kw_t, vw_t, **kw).cpu().numpy()
    ref = oracle.attend(inp["q"], ck, cv, inp["cb"][0], inp["cb"][1],
                        kwin if w.window > 0 else None, vwin if w.window > 0 else None,
                        scale=kw.get("scale"))
    return oracle.check_attn(got, ref)


@pytest.mark.parametrize("key,over", SMALL_DECODE)
def test_decode_parity(key, over):
    say(f"decode parity workload {key} {over}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    codes = [oracle.rvq_encode(inp["x_f32"][b][:, :Tc].reshape(-1, w.head_dim), inp["cb"][b])
             for b in range(2)]
    res = _decode_case(w, inp, codes[0], codes[1])
    say("   ", res)
    assert res["ok"], res


@pytest.mark.parametrize("B,Hkv,R,Tc,W", [
    (3, 4, 4, 12000, 200),     # 264 chunk blocks, window slices on them
    (3, 1, 7, 23000, 2500),    # GQA 7 in head pairs (ragged last), window blocks of their own
])
def test_decode_general_lut_pass(B, Hkv, R, Tc, W):
    """Three-stage caches (outside the rotated-code kernels' shape), long
    enough that building each unit's LUT in every chunk block would re-read
    more than 96 MB of K codebook, so the plan stages it from attn_lut_kernel
    (264 chunk blocks of two heads, 99 MB of re-reads)."""
    say(f"decode through the separate LUT pass: B {B} Hkv {Hkv} GQA {R} Tc {Tc} W {W}")
    rng = np.random.default_rng(700 + R)
    S, D, G, C, dsub = 3, 128, 16, 256, 8
    Hq = Hkv * R
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    vcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    kc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    vc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    got = kvq.attend_decode(cuda(q), cuda(kc), cuda(vc), cuda(kcb), cuda(vcb), cuda(kw),
                            cuda(vw)).cpu().numpy()
    ref = oracle.attend(q, kc, vc, kcb, vcb, kw, vw)
    res = oracle.check_attn(got, ref)
    say("   ", {k: res[k] for k in ("ok", "max_abs", "rel_l2")})
    assert res["ok"], res


@pytest.mark.parametrize("B,Hq,Hkv,D,S,G,Tc,W", [
    (128, 32, 8, 128, 1, 16, 70, 16),   # one stage, GQA 4: 1,024 single-chunk blocks
    (64, 8, 8, 128, 2, 16, 70, 0),      # two stages, one query head per KV head
    (64, 8, 8, 128, 4, 16, 40, 24),     # four stages, one query head per KV head
    (64, 32, 8, 256, 1, 32, 50, 8),     # 256-dim heads, window in a block of its own
    (128, 16, 8, 64, 2, 8, 60, 20),     # 64-dim heads, GQA 2
])
def test_decode_large_batch_lut_pass(B, Hq, Hkv, D, S, G, Tc, W):
    """Many short sequences (a serving batch): one chunk per (sequence, KV
    head, head split), 512-1,024 blocks, whose in-block LUT builds would
    re-read 128-256 MB of K codebook, so the plan stages each unit's LUT from
    attn_lut_kernel; the heads-per-block, head-size and code-row variants of
    that path."""
    say(f"large-batch decode through the LUT pass: B {B} Hq {Hq} Hkv {Hkv} D {D} S {S} G {G} "
        f"Tc {Tc} W {W}")
    rng = np.random.default_rng(900 + B + D + S)
    C, dsub = 256, D // G
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    vcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    kc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    vc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    got = kvq.attend_decode(cuda(q), cuda(kc), cuda(vc), cuda(kcb), cuda(vcb),
                            None if kw is None else cuda(kw),
                            None if vw is None else cuda(vw)).cpu().numpy()
    ref = oracle.attend(q, kc, vc, kcb, vcb, kw, vw)
    res = oracle.check_attn(got, ref)
    say("   ", {k: res[k] for k in ("ok", "max_abs", "rel_l2")})
    assert res["ok"], res


@pytest.mark.parametrize("B,Hq,Hkv,D,S,G,C,Tc,W", [
    # window only: the chunk kernel's window blocks, per heads-per-block and code-row class
    (2, 4, 4, 128, 3, 16, 256, 0, 300),
    (2, 4, 4, 64, 1, 8, 256, 0, 300),
    (2, 4, 4, 128, 1, 16, 256, 0, 300),
    (2, 8, 4, 256, 1, 32, 256, 0, 300),
    (2, 8, 4, 128, 1, 16, 256, 0, 300),
    (2, 8, 4, 128, 2, 16, 256, 0, 300),
    (2, 8, 4, 128, 4, 16, 256, 0, 300),
    (2, 16, 4, 128, 3, 16, 256, 0, 300),
    (2, 16, 4, 128, 4, 16, 256, 0, 300),
    # 256-dim heads two per block, LUT built in the chunk blocks
    (2, 8, 4, 256, 1, 32, 256, 900, 40),
    # serving batches whose LUTs come from attn_lut_kernel: 1, 2 and 4 heads, 64/256 dims
    (64, 8, 8, 256, 1, 32, 256, 50, 0),
    (128, 8, 8, 64, 2, 8, 256, 50, 0),
    (64, 16, 8, 256, 1, 32, 256, 50, 0),
    (128, 32, 8, 64, 2, 8, 256, 50, 0),
    # 64-byte code rows, two heads per block, a book of 128 (outside the rotated-code shape)
    (2, 8, 4, 128, 2, 32, 128, 900, 40),
])
def test_decode_dispatch_variants(B, Hq, Hkv, D, S, G, C, Tc, W):
    """The remaining (heads per block, head size, code-row size, LUT mode)
    instances of the general decode kernel and of attn_lut_kernel: window-only
    calls, 256-dim heads in pairs, and large batches with staged LUTs."""
    say(f"decode variant: B {B} Hq {Hq} Hkv {Hkv} D {D} S {S} G {G} C {C} Tc {Tc} W {W}")
    rng = np.random.default_rng(6000 + B + Hq + D + S + Tc)
    dsub = D // G
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    vcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    kc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    vc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    got = kvq.attend_decode(cuda(q), cuda(kc), cuda(vc), cuda(kcb), cuda(vcb),
                            None if kw is None else cuda(kw),
                            None if vw is None else cuda(vw)).cpu().numpy()
    ref = oracle.attend(q, kc, vc, kcb, vcb, kw, vw)
    res = oracle.check_attn(got, ref)
    say("   ", {k: res[k] for k in ("ok", "max_abs", "rel_l2")})
    assert res["ok"], res


def test_decode_random_codes_and_scale():
    say("decode random codes, explicit scale, GQA 7")
    w = synth.workload(3, batch=2, tokens=1500, window=33)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(1)
    shp = (w.batch * w.n_kv_heads * w.code_tokens, w.n_stages, w.n_groups)
    ck = rng.integers(0, 256, size=shp, dtype=np.uint8)
    cv = rng.integers(0, 256, size=shp, dtype=np.uint8)
    res = _decode_case(w, inp, ck, cv, scale=0.05)
    assert res["ok"], res


def test_decode_window_only_equals_dense_softmax():
    say("decode window only")
    w = synth.workload(2, tokens=200, window=200)
    inp = synth.make_inputs(w)
    empty = np.zeros((0, w.n_stages, w.n_groups), dtype=np.uint8)
    res = _decode_case(w, inp, empty, empty)
    assert res["ok"], res


@pytest.mark.parametrize("key,over", [
    (2, dict(tokens=6000, window=4500)),                  # 3 window blocks, ragged last
    (3, dict(batch=2, tokens=2500, window=2500)),         # window only, 2 blocks, GQA 7
    (1, dict(tokens=3000, window=2049)),                  # D 64, one-token last block
])
def test_decode_long_window(key, over):
    say(f"decode long window workload {key} {over}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    if Tc:
        codes = [oracle.rvq_encode(inp["x_f32"][b][:, :Tc].reshape(-1, w.head_dim), inp["cb"][b])
                 for b in range(2)]
    else:
        codes = [np.zeros((0, w.n_stages, w.n_groups), dtype=np.uint8)] * 2
    res = _decode_case(w, inp, codes[0], codes[1])
    say("   ", res)
    assert res["ok"], res


def test_decode_reused_workspace_and_smaller_call():
    say("decode twice on one workspace, then a smaller batch on it")
    w = synth.workload(3, batch=2, tokens=2600, window=40)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    codes = [oracle.rvq_encode(inp["x_f32"][b][:, :Tc].reshape(-1, w.head_dim), inp["cb"][b])
             for b in range(2)]
    shp = (w.batch, w.n_kv_heads, Tc, w.n_stages, w.n_groups)
    args = (cuda(inp["q"]), cuda(codes[0].reshape(shp)), cuda(codes[1].reshape(shp)),
            cuda(inp["cb"][0]), cuda(inp["cb"][1]), cuda(inp["k_win"]), cuda(inp["v_win"]))
    sz = kvq.attend_workspace_size(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, Tc, w.window,
                                   w.n_stages, w.n_groups, w.n_codewords)
    ws = torch.full((sz,), 0xAB, dtype=torch.uint8, device="cuda")      # no zeroing needed
    first = kvq.attend_decode(*args, workspace=ws).cpu().numpy()
    second = kvq.attend_decode(*args, workspace=ws).cpu().numpy()
    assert np.array_equal(first, second)
    ref = oracle.attend(inp["q"], codes[0].reshape(shp), codes[1].reshape(shp), inp["cb"][0],
                        inp["cb"][1], inp["k_win"], inp["v_win"])
    res = oracle.check_attn(second, ref)
    assert res["ok"], res
    small = kvq.attend_decode(args[0][:1].contiguous(), args[1][:1].contiguous(),
                              args[2][:1].contiguous(), args[3], args[4],
                              args[5][:1].contiguous(), args[6][:1].contiguous(),
                              workspace=ws).cpu().numpy()
    res = oracle.check_attn(small, ref[:1])
    assert res["ok"], res


@pytest.mark.parametrize("key,over,wcap,nflush", [
    (3, dict(batch=2, tokens=300, window=0), 96, 64),     # MFMA encode, S = 2, GQA 7
    (1, dict(tokens=150, window=0), 40, 24),              # generic encode, D = 64
])
def test_streaming_window_parity(key, over, wcap, nflush):
    """Tokens appended one at a time, the oldest nflush flushed into codes
    whenever the window is full: window buffers bit-exact with the oracle's
    stream, codes within the near-tie rule, then decode over the grown cache
    (capacity strides) against the oracle on the same codes."""
    say(f"streaming window workload {key} {over} cap {wcap} flush {nflush}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    B, H, T, D = w.batch, w.n_kv_heads, w.tokens, w.head_dim
    S, G = w.n_stages, w.n_groups
    tk = inp["x_f32"][0].reshape(B, H, T, D).astype(np.float16)
    tv = inp["x_f32"][1].reshape(B, H, T, D).astype(np.float16)
    kcb, vcb = inp["cb"][0], inp["cb"][1]
    ccap = T
    kw = torch.zeros((B, H, wcap, D), dtype=torch.float16, device="cuda")
    vw = torch.zeros_like(kw)
    kc = torch.zeros((B, H, ccap, S, G), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    kcb_d, vcb_d = cuda(kcb), cuda(vcb)
    tk_d, tv_d = cuda(tk), cuda(tv)
    okw = np.zeros((B, H, wcap, D), np.float16); ovw = np.zeros_like(okw)
    nw = nc = 0
    flushed = []
    ws = torch.empty(max(kvq.window_flush_workspace_size(D, G, S, w.n_codewords), 16),
                     dtype=torch.uint8, device="cuda")
    for t in range(T):
        if nw == wcap:                                   # the first flush packs the books
            kvq.window_flush(kw, vw, nw, nflush, kc, vc, nc, kcb_d, vcb_d, workspace=ws,
                             packed=bool(flushed))
            okw[:, :, :nw - nflush] = okw[:, :, nflush:nw].copy()
            ovw[:, :, :nw - nflush] = ovw[:, :, nflush:nw].copy()
            flushed.append((nc, nflush))
            nw, nc = nw - nflush, nc + nflush
        kvq.window_append(tk_d[:, :, t].contiguous(), tv_d[:, :, t].contiguous(), kw, vw, nw)
        okw[:, :, nw] = tk[:, :, t]
        ovw[:, :, nw] = tv[:, :, t]
        nw += 1
    torch.cuda.synchronize()
    assert nc > 0 and len(flushed) >= 2
    assert np.array_equal(kw.cpu().numpy()[:, :, :nw], tk[:, :, nc:])
    assert np.array_equal(vw.cpu().numpy()[:, :, :nw], tv[:, :, nc:])
    assert np.array_equal(kw.cpu().numpy(), okw) and np.array_equal(vw.cpu().numpy(), ovw)
    kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()
    assert not kcn[:, :, nc:].any()                      # rows past the count untouched
    for codes, toks, cb in ((kcn, tk, kcb), (vcn, tv, vcb)):
        res = oracle.check_codes(toks[:, :, :nc].astype(np.float64).reshape(-1, D), cb,
                                 codes[:, :, :nc].reshape(-1, S, G))
        say("   codes", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
        assert res["hard"] == 0
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, w.n_q_heads, D)).astype(np.float32)
    got = kvq.attend_decode(cuda(q), kc, vc, kcb_d, vcb_d, kw, vw, n_code=nc,
                            n_window=nw).cpu().numpy()
    ref = oracle.attend(q, kcn[:, :, :nc], vcn[:, :, :nc], kcb, vcb, tk[:, :, nc:], tv[:, :, nc:])
    res = oracle.check_attn(got, ref)
    say("   decode", res)
    assert res["ok"], res


def test_decode_codes_only_short():
    say("decode codes only, short cache")
    w = synth.workload(4, tokens=37, window=0)
    inp = synth.make_inputs(w)
    codes = [oracle.rvq_encode(inp["x_f32"][b].reshape(-1, 128), inp["cb"][b]) for b in range(2)]
    res = _decode_case(w, inp, codes[0], codes[1])
    assert res["ok"], res



@pytest.mark.parametrize("key,delta,every", [(2, 15.5, 1024), (3, 14.0, 2048), (4, 14.0, 4096)])
def test_decode_attention_sink_chunks(key, delta, every):
    """Peaky softmax inside the split-K chunks, at the workload's full shape:
    every `every`-th coded token is a sink whose key scores `delta` nats
    above every other key (all other coded keys share one code row, the
    window keys equal their reconstruction), and the V rows differ by several
    units (V codebook x10, random V codes).  On the long-context shape each
    4088-token chunk holds one sink and 4087 weights of e^-14, 3.4e-3 of its
    mass: a fixed-point weight step taken from the chunk length alone (2^-19)
    rounds them all to zero, about 5e-2 off in the output (CPU emulation of
    that rule).  The Qwen-shaped batch (16 sequences, two stages, seven query
    heads per KV head split 4 + 3 over two blocks) has two sinks per chunk.  Query heads are equal so every head sees the same gap.  The
    fp32 log-sum-exp combine must still meet 2e-3 max-abs / 1e-3 relative L2
    ("Differential-KV" README, Flash-Style LSE Combine)."""
    w = synth.workload(key)
    B, Hkv, Hq, D, W = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window
    S, G, C, Tc = w.n_stages, w.n_groups, w.n_codewords, w.code_tokens
    say(f"decode attention-sink chunks, {w.name} shape: Tc={Tc} W={W} S={S}")
    cb = synth.make_codebooks(w)
    kcb = cb[0]
    vcb = np.ascontiguousarray(cb[1] * 10.0)
    rng = np.random.default_rng(20 + key)
    q0 = rng.standard_normal(D)
    q = np.broadcast_to(q0.astype(np.float32), (B, Hq, D)).copy()
    # sink code: per (stage, group) the entry with the largest q_rot . c
    # (greedy per stage); the other keys: one random code row
    qr = oracle.fwht(q0[None, :])[0]
    dsub = D // G
    sink = np.array([[int(np.argmax(kcb[s, g].astype(np.float64) @ qr[g * dsub:(g + 1) * dsub]))
                      for g in range(G)] for s in range(S)], dtype=np.uint8)
    other = rng.integers(0, C, size=(S, G), dtype=np.uint8)
    k_sink = oracle.reconstruct(sink[None], kcb)[0]
    k_other = oracle.reconstruct(other[None], kcb)[0]
    gap = float(q0 @ (k_sink - k_other)) / np.sqrt(D)
    assert gap > 0.5, gap
    scale = float(delta / (gap * np.sqrt(D)))          # softmax scale: sink - rest = delta
    ck = np.broadcast_to(other, (B, Hkv, Tc, S, G)).copy()
    ck[:, :, ::every] = sink
    cv = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kwin = np.broadcast_to(k_other.astype(np.float16), (B, Hkv, W, D)).copy()
    vwin = (rng.standard_normal((B, Hkv, W, D)) * 5).astype(np.float16)
    got = kvq.attend_decode(cuda(q), cuda(ck), cuda(cv), cuda(kcb), cuda(vcb), cuda(kwin),
                            cuda(vwin), scale=scale).cpu().numpy()
    ref = oracle.attend(q, ck, cv, kcb, vcb, kwin, vwin, scale=scale)
    # the construction is as described: delta nats between the sink and the rest
    kr = oracle.reconstruct(ck[0, 0, :every + 1].reshape(-1, S, G), kcb)
    sc = kr @ q0 * scale
    assert abs((sc[0] - sc[1]) - delta) < 1e-6 and abs(sc[every] - sc[0]) < 1e-9
    spread = np.abs(ref - ref.mean(axis=(0, 1), keepdims=True)).max()
    res = oracle.check_attn(got, ref)
    say("   ", res, "output spread", round(float(spread), 3))
    assert res["ok"], res

# ------------------------------------------------------------- full sizes
@pytest.mark.timeout(600)
@pytest.mark.parametrize("key", [2, 3, 4])
def test_full_size_encode_and_decode(key):
    """Full-size decode workloads: the K book's codes checked against the
    oracle for every coded vector of the layer (the check split over worker
    processes), the V book's on every 97th vector, then decode over the
    GPU's codes."""
    from parallel_check import check_codes_all
    say(f"full-size workload {key}: encode (K book every vector, V book every 97th) + decode")
    w = synth.workload(key)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    x = to_dev(inp["x"], w)
    codes = kvq.encode(x, cuda(inp["cb"]), n_rows=Tc)
    torch.cuda.synchronize()
    codes_np = codes.cpu().numpy()
    del x
    for b in range(2):
        flat = codes_np[b].reshape(-1, w.n_stages, w.n_groups)
        xs = inp["x_f32"][b][:, :Tc].reshape(-1, w.head_dim)
        if b == 0:
            res = check_codes_all(xs, inp["cb"][b], flat)
            assert res["total"] == xs.shape[0] * w.n_stages * w.n_groups
        else:
            idx = np.arange(0, flat.shape[0], 97)
            res = oracle.check_codes(xs[idx].astype(np.float64), inp["cb"][b], flat[idx])
        say("   book", b, {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
        assert res["hard"] == 0, res["hard_examples"]
    res = _decode_case(w, inp, codes_np[0], codes_np[1])
    say("   decode", res)
    assert res["ok"], res


def test_full_size_prefill_layers_sampled():
    say("prefill workload: 2 of 32 layers at full per-layer size, sampled check")
    w = synth.workload(5)
    inp = synth.make_inputs(w, layers=[0, 31])
    x = to_dev(inp["x"], w)
    codes = kvq.encode(x, cuda(inp["cb"])).cpu().numpy()
    for b in range(x.shape[0]):
        flat = codes[b].reshape(-1, 2, 16)
        xs = inp["x_f32"][b].reshape(-1, 128)
        idx = np.arange(0, flat.shape[0], 131)
        res = oracle.check_codes(xs[idx].astype(np.float64), inp["cb"][b], flat[idx])
        assert res["hard"] == 0, res


@pytest.mark.parametrize("first", [0, 8, 16, 24])
def test_prefill_every_layer_sampled(first):
    """The prefill workload's sample check: for every one of its 32 layers
    (8 per test), K and V of all 8 KV heads, every 64th token, coded at full
    per-layer size on the GPU and checked against the oracle."""
    w = synth.workload(5)
    for layer in range(first, first + 8):
        say(f"prefill layer {layer}: encode K and V (8 heads x 32768 tokens), check every 64th token")
        inp = synth.make_inputs(w, layers=[layer])
        x = to_dev(inp["x"], w)
        codes = kvq.encode(x, cuda(inp["cb"]))[:, :, ::64].cpu().numpy()
        del x
        for b in range(2):
            xs = inp["x_f32"][b][:, ::64].reshape(-1, 128).astype(np.float64)
            res = oracle.check_codes(xs, inp["cb"][b], codes[b].reshape(-1, 2, 16))
            assert res["hard"] == 0, (layer, b, res)
            assert res["exact"] >= 0.999 * res["total"], (layer, b, res)


def test_decode_independent_of_chunk_count():
    """Split-K invariance on the GPU: one sequence decoded alone (20 chunks of
    1000 tokens) and inside a batch of four copies (8 chunks of 2500 tokens, a
    different fixed-point scale and merge) agree to the fixed-point rounding;
    the batch rows, which share a plan, agree bit for bit."""
    say("decode: chunk-count invariance")
    w = synth.workload(2, tokens=20128, window=128)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    rng = np.random.default_rng(8)
    ck = rng.integers(0, 256, size=(1, 8, Tc, 1, 16), dtype=np.uint8)
    cv = rng.integers(0, 256, size=(1, 8, Tc, 1, 16), dtype=np.uint8)
    args = (cuda(inp["cb"][0]), cuda(inp["cb"][1]))
    one = kvq.attend_decode(cuda(inp["q"]), cuda(ck), cuda(cv), *args, cuda(inp["k_win"]),
                            cuda(inp["v_win"])).cpu().numpy()
    rep = lambda a: np.ascontiguousarray(np.repeat(a, 4, axis=0))
    four = kvq.attend_decode(cuda(rep(inp["q"])), cuda(rep(ck)), cuda(rep(cv)), *args,
                             cuda(rep(inp["k_win"])), cuda(rep(inp["v_win"]))).cpu().numpy()
    # plans differ: chunk length 1000 vs 2500 (8 vs 32 units over 256 blocks)
    for b in range(1, 4):
        assert np.array_equal(four[b], four[0])
    scale = np.abs(one).max()
    assert np.max(np.abs(four[0] - one[0])) <= 2e-5 * scale, np.max(np.abs(four[0] - one[0]))
    ref = oracle.attend(inp["q"], ck, cv, inp["cb"][0], inp["cb"][1], inp["k_win"], inp["v_win"])
    assert oracle.check_attn(one, ref)["ok"] and oracle.check_attn(four[:1], ref)["ok"]
