"""Seeded sweep of decode and reconstruction shapes against the float64 oracle,
through the C ABI: batch, KV heads, GQA ratio, head size, groups, stages,
codebook size, coded and window lengths drawn at random (small enough for the
oracle), so the plan's choices (heads per block, head splits, chunking, window
slices or window blocks, LUT built per block or in its own pass) and the
kernels' ragged edges meet many combinations.  Bars as elsewhere: attention
within 2e-3 max-abs and 1e-3 relative L2; rotated reconstruction bit-exact,
unrotated within 1e-6 * |x_hat|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
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


def _shape(rng):
    # redraw until one query head's tables fit the chunk kernel's LDS (the
    # library reports larger ones as unsupported)
    while True:
        D = int(rng.choice([64, 128, 256]))
        dsub = int(rng.choice([d for d in (4, 8, 16, 32) if D // d <= 64]))
        G = D // dsub
        S = int(rng.integers(1, 5))
        C = int(rng.choice([16, 100, 256]))
        if S * G * (C + 4) * 4 + 8 * D * 4 <= 140 * 1024:
            break
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4]))
    R = int(rng.choice([1, 2, 3, 4, 5, 7, 8]))
    Tc = int(rng.choice([0, int(rng.integers(1, 300)), int(rng.integers(300, 5000))]))
    W = int(rng.choice([0, int(rng.integers(1, 80)), int(rng.integers(80, 300))]))
    if Tc + W == 0:
        Tc = 17
    return dict(D=D, dsub=dsub, G=G, S=S, C=C, B=B, Hkv=Hkv, R=R, Tc=Tc, W=W)


CASES = list(range(40))


@pytest.mark.parametrize("case", CASES)
def test_decode_sweep(case):
    rng = np.random.default_rng(1000 + case)
    p = _shape(rng)
    D, G, S, C, B, Hkv, R, Tc, W = (p[k] for k in ("D", "G", "S", "C", "B", "Hkv", "R", "Tc", "W"))
    dsub = D // G
    say(f"decode sweep case {case}: {p}")
    Hq = Hkv * R
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


def _rotated_code_case(rng, G, stages):
    D, C, dsub = 128, 256, 128 // G
    S = int(rng.choice(stages))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4]))
    R = int(rng.choice([2, 3, 4, 5, 7, 8]))
    Tc = int(rng.choice([1, int(rng.integers(2, 1100)), int(rng.integers(1100, 9000))]))
    W = int(rng.choice([0, int(rng.integers(1, 64)), int(rng.integers(300, 1200))]))
    smooth = bool(rng.integers(0, 4) == 0)
    say(f"rotated-code decode: G {G} S {S} B {B} Hkv {Hkv} GQA {R} Tc {Tc} W {W} smooth {smooth}")
    Hq = Hkv * R
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    vcb = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
           * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    kc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    vc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    lam = rng.uniform(0.5, 2.0, size=(1, D)).astype(np.float32) if smooth else None
    got = kvq.attend_decode(cuda(q), cuda(kc), cuda(vc), cuda(kcb), cuda(vcb),
                            None if kw is None else cuda(kw), None if vw is None else cuda(vw),
                            k_smooth=None if lam is None else cuda(lam)).cpu().numpy()
    ref = oracle.attend(q, kc, vc, kcb, vcb, kw, vw,
                        k_smooth=None if lam is None else lam.astype(np.float64))
    res = oracle.check_attn(got, ref)
    say("   ", {k: res[k] for k in ("ok", "max_abs", "rel_l2")})
    assert res["ok"], res


@pytest.mark.parametrize("case", list(range(16)))
def test_rotated_code_decode_sweep(case):
    """The cache shape of the rotated-code kernels (128-dim heads, 16 groups of
    8, C = 256, two or four stages, at least two query heads per KV head):
    head groups of 1-4 heads (GQA 2-8, head splits with a ragged last one),
    coded lengths from a single token to several chunks with a ragged tail,
    no window, short windows riding on the chunk blocks and long ones in
    blocks of their own, the factors of the dual transform on some cases."""
    _rotated_code_case(np.random.default_rng(3000 + case), 16, [2, 4])


@pytest.mark.parametrize("case", list(range(12)))
def test_rotated_code_decode_sweep_32_groups(case):
    """The same sweep for the rotated-code kernels' other row shape: 32 groups
    of 4 dims (the product codebooks of 2-bit scalar codes), one or two
    stages."""
    _rotated_code_case(np.random.default_rng(3100 + case), 32, [1, 2])


@pytest.mark.parametrize("case", list(range(20)))
def test_reconstruct_sweep(case):
    rng = np.random.default_rng(2000 + case)
    D = int(rng.choice([64, 128, 256]))
    dsub = int(rng.choice([8, 16, 32]))
    G = D // dsub
    S = int(rng.integers(1, 6))
    C = int(rng.choice([16, 100, 256]))
    nb = int(rng.integers(1, 4))
    n = int(rng.choice([1, int(rng.integers(2, 200)), int(rng.integers(200, 3000))]))
    say(f"reconstruct sweep case {case}: D {D} G {G} S {S} C {C} books {nb} n {n}")
    cb = rng.standard_normal((nb, S, G, C, dsub)).astype(np.float32)
    codes = rng.integers(0, 256, size=(nb, n, S, G), dtype=np.uint8)
    clamped = np.minimum(codes, C - 1)
    got = kvq.decode_reconstruct(cuda(codes), cuda(cb)).cpu().numpy()
    got_u = kvq.decode_reconstruct(cuda(codes), cuda(cb), unrotate=True).cpu().numpy()
    for b in range(nb):
        ref = oracle.reconstruct_rot(clamped[b], cb[b])
        assert np.array_equal(got[b], ref.astype(np.float32))
        ref_u = oracle.reconstruct(clamped[b], cb[b])
        nrm = np.linalg.norm(ref_u, axis=1, keepdims=True)
        assert np.max(np.abs(got_u[b] - ref_u) / nrm) <= 1e-6


@pytest.mark.parametrize("D,dsub,S,C,nb,n", [
    (128, 8, 3, 256, 2, 3000),        # half tables, three stages
    (128, 128, 2, 256, 2, 2000),      # one group (odd): stage-0 book in LDS, rows staged
    (128, 128, 4, 256, 1, 2000),
    (64, 64, 4, 256, 2, 2000),
    (128, 8, 5, 256, 2, 2000),        # five stages: the cache kernel
    (64, 8, 5, 100, 2, 2000),
    (128, 8, 1, 256, 1, 600000),      # LDS kernels whose blocks' code rows no longer fit
    (64, 8, 1, 256, 1, 1100000),      # beside the book: rows read from global memory
    (256, 8, 1, 128, 1, 300000),
    (64, 64, 2, 256, 1, 4200000),
    (128, 128, 2, 256, 1, 4300000),
    (64, 64, 4, 256, 1, 2100000),
    (128, 128, 4, 256, 1, 2100000),
])
def test_reconstruct_dispatch_variants(D, dsub, S, C, nb, n):
    """Each reconstruction kernel variant the launcher can pick: half tables
    at three stages, the whole stage-0 book in LDS for a single group (two
    and four stages) with the blocks' code rows staged beside it or, for large
    calls, read from global memory, and the cache kernel for five stages.
    Rotated output bit-exact, unrotated within 1e-6 * |x_hat|; calls over
    10,000 vectors per book on every 97th vector and the last."""
    G = D // dsub
    say(f"reconstruct variant: D {D} G {G} S {S} C {C} books {nb} n {n}")
    rng = np.random.default_rng(4000 + D + dsub + S + nb)
    cb = rng.standard_normal((nb, S, G, C, dsub)).astype(np.float32)
    codes = rng.integers(0, 256, size=(nb, n, S, G), dtype=np.uint8)
    clamped = np.minimum(codes, C - 1)
    idx = np.arange(n) if n <= 10000 else np.r_[np.arange(0, n, 97), n - 1]
    idx_t = torch.from_numpy(idx).cuda()
    for unrot in (False, True):
        got = kvq.decode_reconstruct(cuda(codes), cuda(cb), unrotate=unrot)
        got = got[:, idx_t].cpu().numpy()
        for b in range(nb):
            if not unrot:
                ref = oracle.reconstruct_rot(clamped[b][idx], cb[b])
                assert np.array_equal(got[b], ref.astype(np.float32)), b
            else:
                ref = oracle.reconstruct(clamped[b][idx], cb[b])
                nrm = np.linalg.norm(ref, axis=1, keepdims=True)
                assert np.max(np.abs(got[b] - ref) / nrm) <= 1e-6, b
        del got
        torch.cuda.empty_cache()


@pytest.mark.parametrize("case", list(range(24)))
def test_encode_sweep(case):
    """Encode shapes: every other case is an MFMA-eligible one (D = 128,
    dsub = 8, C = 256, 2-byte input; 1-4 stages, small batches that split
    the groups over blocks), the rest random for the generic kernel (D, dsub,
    C, stages, dtype, rotation done by the caller or not).  Every code follows
    the oracle's rule (exact, or within the 1e-4 near-tie band)."""
    rng = np.random.default_rng(3000 + case)
    mfma = case % 2 == 0
    if mfma:
        D, dsub, C = 128, 8, 256
        dt = [torch.bfloat16, torch.float16][int(rng.integers(0, 2))]
    else:
        D = int(rng.choice([64, 128, 256]))
        dsub = int(rng.choice([d for d in (8, 16, 32, 64, 128) if d <= D]))
        C = int(rng.choice([16, 100, 256]))
        dt = [torch.float32, torch.bfloat16, torch.float16][int(rng.integers(0, 3))]
    G = D // dsub
    S = int(rng.integers(1, 5))
    nb = int(rng.integers(1, 3))
    n = int(rng.choice([1, int(rng.integers(2, 300)), int(rng.integers(300, 3000))]))
    pre = bool(rng.integers(0, 2)) and not mfma
    say(f"encode sweep case {case}: D {D} dsub {dsub} C {C} S {S} books {nb} n {n} {dt} "
        f"pre_rotated={pre}")
    cb = (rng.standard_normal((nb, S, G, C, dsub)) / np.sqrt(dsub)
          * (0.5 ** np.arange(S))[None, :, None, None, None]).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((nb, 1, n, D)).astype(np.float32)).to(dt).cuda()
    xf = x.double().cpu().numpy()
    codes = kvq.encode(x, cuda(cb), pre_rotated=pre).cpu().numpy()
    assert codes.shape == (nb, 1, n, S, G)
    for b in range(nb):
        res = oracle.check_codes(xf[b, 0], cb[b], codes[b, 0], rotate=not pre)
        assert res["hard"] == 0, (case, b, {k: res[k] for k in ("total", "exact", "near_tie",
                                                                  "hard")})


@pytest.mark.parametrize("D,dsub,S,C,dt,n", [
    # MFMA kernel, batches of at least 512 tiles (each block codes all 16 groups)
    (128, 8, 1, 256, "f16", 140000),
    (128, 8, 2, 256, "f16", 140000),
    (128, 8, 3, 256, "bf16", 270000),
    (128, 8, 3, 256, "f16", 270000),
    (128, 8, 4, 256, "f16", 270000),
    # generic kernel, the (D, dsub) pairs not drawn by the sweep above
    (128, 128, 2, 100, "f32", 700),
    (128, 32, 3, 256, "bf16", 700),
    (128, 64, 1, 16, "f16", 700),
    (256, 16, 2, 256, "f32", 700),
    (256, 64, 3, 100, "bf16", 700),
    (64, 32, 2, 256, "f16", 700),
    (64, 8, 4, 100, "f32", 700),
])
def test_encode_dispatch_variants(D, dsub, S, C, dt, n):
    """Encode kernel variants the sweep's shapes do not reach: the MFMA
    kernel's full-group instances for 2-byte inputs at 1-4 stages (checked on
    every 97th vector and the last), and generic-kernel head and group sizes.
    Every checked code follows the oracle's rule."""
    G = D // dsub
    say(f"encode variant: D {D} dsub {dsub} S {S} C {C} {dt} n {n}")
    rng = np.random.default_rng(5000 + D + dsub + S + n)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    cb = (rng.standard_normal((1, S, G, C, dsub)) / np.sqrt(dsub)
          * (0.5 ** np.arange(S))[None, :, None, None, None]).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((1, 1, n, D)).astype(np.float32)).to(tdt).cuda()
    codes = kvq.encode(x, cuda(cb))
    assert codes.shape == (1, 1, n, S, G)
    idx = np.arange(n) if n <= 10000 else np.r_[np.arange(0, n, 97), n - 1]
    idx_t = torch.from_numpy(idx).cuda()
    xf = x[0, 0, idx_t].double().cpu().numpy()
    got = codes[0, 0, idx_t].cpu().numpy()
    res = oracle.check_codes(xf, cb[0], got)
    say("   ", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
    assert res["hard"] == 0, {k: res[k] for k in ("total", "exact", "near_tie", "hard")}


@pytest.mark.parametrize("case", list(range(16)))
def test_scalar_sweep(case):
    """Scalar variant shapes: D 64-256, b = 1, 2, 4, 1-3 books, ragged row
    counts, f32/bf16/f16 input; encode under the threshold rule and the
    reconstruction bit-exact (rotated) / within 1e-6 * |x_hat| (unrotated)."""
    rng = np.random.default_rng(4000 + case)
    D = int(rng.choice([64, 128, 256]))
    bits = int(rng.choice([1, 2, 3, 4]))
    nb = int(rng.integers(1, 4))
    n = int(rng.choice([1, int(rng.integers(2, 300)), int(rng.integers(300, 3000))]))
    dt = [torch.float32, torch.bfloat16, torch.float16][int(rng.integers(0, 3))]
    say(f"scalar sweep case {case}: D {D} bits {bits} books {nb} n {n} {dt}")
    g = oracle.lloyd_max_levels("gaussian", bits)
    lap = oracle.lloyd_max_levels("laplacian", bits)
    dg = oracle.lloyd_max_distortion("gaussian", g)
    sd = rng.uniform(0.5, 2.0, size=nb)
    lv = np.stack([[g * s, lap * s * np.sqrt(dg)] for s in sd]).astype(np.float32)
    x = torch.from_numpy((rng.standard_normal((nb, 1, n, D)) * sd[:, None, None, None])
                         .astype(np.float32)).to(dt).cuda()
    codes = kvq.scalar_encode(x, cuda(lv), bits).cpu().numpy()
    nbytes = D * bits // 8
    assert codes.shape == (nb, 1, n, 2, nbytes)
    xf = x.double().cpu().numpy()
    rot = kvq.scalar_decode_reconstruct(cuda(codes), cuda(lv), bits).cpu().numpy()
    unr = kvq.scalar_decode_reconstruct(cuda(codes), cuda(lv), bits, unrotate=True).cpu().numpy()
    for b in range(nb):
        z = oracle.unpack_bits(codes[b, 0], bits)
        y = oracle.fwht(xf[b, 0])
        res = oracle.check_scalar_codes(y, lv[b, 0], lv[b, 1], z[:, 0], z[:, 1])
        assert res["hard"] == 0, (case, b, res)
        ref = oracle.scalar_reconstruct(z[:, 0], z[:, 1], lv[b, 0], lv[b, 1], unrotate=False)
        assert np.array_equal(rot[b, 0], ref.astype(np.float32))
        ref_u = oracle.fwht(ref)
        nrm = np.linalg.norm(ref, axis=1, keepdims=True)
        assert np.all(np.abs(unr[b, 0] - ref_u) <= 1e-6 * nrm)


@pytest.mark.parametrize("case", list(range(12)))
def test_smoothed_decode_sweep(case):
    """Dual transform on random shapes: factors from the GPU calibration equal
    the oracle's, the keys' codes follow the code rule on the smoothed, rotated
    keys, and decode with the factors folded into the query matches the
    oracle's attention over the smoothed reconstruction."""
    rng = np.random.default_rng(5000 + case)
    D = 128
    G, dsub, S, C = 16, 8, int(rng.integers(1, 3)), 256
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    R = int(rng.choice([1, 3, 4]))
    Tc = int(rng.integers(1, 1500))
    W = int(rng.choice([0, int(rng.integers(1, 100))]))
    say(f"smoothed decode sweep case {case}: S {S} B {B} Hkv {Hkv} R {R} Tc {Tc} W {W}")
    scale_ch = np.exp(rng.uniform(np.log(0.3), np.log(8.0), size=(B * Hkv, 1, D)))
    k = (rng.standard_normal((B * Hkv, Tc, D)) * scale_ch).astype(np.float32)
    kt = torch.from_numpy(k).cuda()[None]                       # [1][B*Hkv][Tc][D]
    lam = kvq.smooth_calibrate(kt, B * Hkv).cpu().numpy()[0]    # one row per (sequence, KV head)
    ref_lam = oracle.smooth_factors(k.astype(np.float64), B * Hkv)
    assert np.array_equal(lam, ref_lam.astype(np.float32))
    cb = (rng.standard_normal((2, S, G, C, dsub)) / np.sqrt(dsub) * 0.5
          * (0.5 ** np.arange(S))[None, :, None, None, None]).astype(np.float32)
    kc = kvq.encode(kt, cuda(cb[:1]), smooth=cuda(lam[None])).cpu().numpy()[0]
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(B * Hkv))
    ys = oracle.fwht(oracle.smooth_keys(k.astype(np.float64), rows[:, None, :]).reshape(-1, D))
    res = oracle.check_codes(ys, cb[0], kc.reshape(-1, S, G), rotate=False)
    assert res["hard"] == 0, res
    vc = rng.integers(0, C, size=(B, Hkv, Tc, S, G), dtype=np.uint8)
    kcs = kc.reshape(B, Hkv, Tc, S, G)
    q = rng.standard_normal((B, Hkv * R, D)).astype(np.float32)
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16) if W else None
    got = kvq.attend_decode(cuda(q), cuda(kcs), cuda(vc), cuda(cb[0]), cuda(cb[1]),
                            None if kw is None else cuda(kw), None if vw is None else cuda(vw),
                            k_smooth=cuda(lam)).cpu().numpy()
    ref = oracle.attend(q, kcs, vc, cb[0], cb[1], kw, vw, k_smooth=lam.astype(np.float64))
    r = oracle.check_attn(got, ref)
    assert r["ok"], r
