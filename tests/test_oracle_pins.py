"""Pins of the CPU oracle to facts outside itself (closed forms, library
routines, brute force, hand-worked fixtures, invariants).  CPU only.

Each group of tests is chosen so that a plausible slip in the oracle (a
dropped normalisation, a wrong sign or index, argmax for argmin, a transposed
operand, a wrong GQA mapping) fails at least one of them; the mutation tests
at the end plant such slips in local copies and show that they are caught.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.spatial.distance as ssd
import torch

import oracle
from oracle import (hadamard_matrix, fwht, nearest, rvq_encode, reconstruct_rot,
                    reconstruct, attend, attend_dense, lse_merge)
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = np.array([float(t) for t in v.split()])
    return out


# --------------------------------------------------------------------------- O1
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_closed_form_and_library(n):
    h = hadamard_matrix(n)
    i = np.arange(n)
    pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
    closed = np.where(pc % 2 == 0, 1.0, -1.0) / np.sqrt(n)
    assert np.array_equal(h, closed)
    assert np.array_equal(h, scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwht_invariants(d):
    h = fwht(np.eye(d))                      # rotate the identity: rows are H
    assert np.max(np.abs(h @ h.T - np.eye(d))) <= 1e-12
    assert np.array_equal(h, h.T)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, d))
    y = fwht(x)
    assert np.max(np.abs(np.linalg.norm(y, axis=1) - np.linalg.norm(x, axis=1))
                  / np.linalg.norm(x, axis=1)) <= 1e-12
    assert np.max(np.abs(fwht(y) - x)) <= 1e-12
    e0 = np.zeros(d); e0[0] = 1
    assert np.allclose(fwht(e0), np.full(d, 1 / np.sqrt(d)), atol=0, rtol=1e-15)
    ones = np.ones(d)
    expect = np.zeros(d); expect[0] = np.sqrt(d)
    assert np.max(np.abs(fwht(ones) - expect)) <= 1e-12


def test_fwht_golden_d4():
    g = _read_golden("fwht_d4.txt")
    assert np.allclose(fwht(g["x"]), g["y"], atol=1e-15, rtol=0)


def test_fwht_matches_torch_butterfly():
    """An independent recursive butterfly (library ops only) agrees with the
    dense product."""
    def butterfly(x):
        n = x.shape[-1]
        if n == 1:
            return x
        a, b = x[..., : n // 2], x[..., n // 2:]
        return torch.cat([butterfly(a + b), butterfly(a - b)], dim=-1)
    x = torch.randn(20, 128, dtype=torch.float64)
    ref = butterfly(x) / np.sqrt(128)
    assert torch.max(torch.abs(torch.from_numpy(fwht(x.numpy())) - ref)) <= 1e-12


# --------------------------------------------------------------------------- O2
def test_nearest_equals_exhaustive_cdist():
    rng = np.random.default_rng(1)
    r = rng.standard_normal((300, 8))
    cb = rng.standard_normal((256, 8)) * 0.4
    z, d = nearest(r, cb)
    ref_d = ssd.cdist(r, cb, "sqeuclidean")
    assert np.max(np.abs(d - ref_d)) <= 1e-12
    # second, independent formulation: |x|^2 + |c|^2 - 2 x.c
    alt = (r ** 2).sum(1)[:, None] + (cb ** 2).sum(1)[None] - 2 * r @ cb.T
    z_alt = np.argmin(alt, axis=1)
    srt = np.sort(ref_d, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > 1e-9
    assert np.array_equal(z[clear], z_alt[clear])
    assert np.array_equal(z, np.argmin(ref_d, axis=1))


def test_single_stage_full_dim_equals_exhaustive_search():
    """Tiny-workload stage 0 alone (one full 64-dim codebook of 256 entries)
    equals exhaustive nearest-neighbour search after an independently built
    rotation (scipy's Hadamard)."""
    w = synth.workload(1, tokens=200)
    inp = synth.make_inputs(w)
    x = inp["x_f32"][0, 0].astype(np.float64)
    cb = inp["cb"][0][:1]                      # [1][1][256][64]
    codes = rvq_encode(x, cb)
    y = x @ (scipy.linalg.hadamard(64) / 8.0)
    ref = np.argmin(ssd.cdist(y, cb[0, 0].astype(np.float64), "sqeuclidean"), axis=1)
    assert np.array_equal(codes[:, 0, 0], ref)


def test_codeword_inputs_return_own_index():
    rng = np.random.default_rng(3)
    cb = rng.standard_normal((1, 4, 256, 8)).astype(np.float32)
    x = np.concatenate([cb[0, g] for g in range(4)], axis=1).astype(np.float64)  # [256][32]
    codes, st = rvq_encode(x, cb, rotate=False, with_stats=True)
    for g in range(4):
        assert np.array_equal(codes[:, 0, g], np.arange(256))
    assert np.all(st["d1"] == 0)
    assert np.array_equal(reconstruct_rot(codes, cb), x)


def test_rvq_golden_2d():
    g = _read_golden("rvq_2d.txt")
    cb = np.stack([g["cb0"].reshape(4, 2), g["cb1"].reshape(4, 2)])[:, None]  # [2][1][4][2]
    codes, st = rvq_encode(g["x"][None], cb, rotate=False, with_stats=True)
    assert codes[0, :, 0].tolist() == g["codes"].astype(int).tolist()
    assert np.allclose(st["resid2"][0, :, 0], g["resid2"], atol=1e-15, rtol=1e-12)
    assert np.allclose(reconstruct_rot(codes, cb)[0], g["recon"], atol=1e-15)


def test_residual_chain_second_stage_is_nearest_to_residual():
    w = synth.workload(3, batch=1, tokens=300, window=0)
    inp = synth.make_inputs(w)
    x = inp["x_f32"][0, 0].astype(np.float64)
    cb = inp["cb"][0]
    codes = rvq_encode(x, cb)
    y = x @ (scipy.linalg.hadamard(128) / np.sqrt(128))
    cb64 = cb.astype(np.float64)
    for g in (0, 5, 15):
        r = y[:, 8 * g:8 * g + 8]
        z0 = np.argmin(ssd.cdist(r, cb64[0, g], "sqeuclidean"), axis=1)
        assert np.array_equal(codes[:, 0, g], z0)
        r1 = r - cb64[0, g][z0]
        z1 = np.argmin(ssd.cdist(r1, cb64[1, g], "sqeuclidean"), axis=1)
        assert np.array_equal(codes[:, 1, g], z1)


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_total_error_non_increasing_per_stage(key):
    w = synth.workload(key, batch=1, tokens=400, window=0, layers=1)
    inp = synth.make_inputs(w)
    x = inp["x_f32"][0].reshape(-1, w.head_dim)[:600]
    _, st = rvq_encode(x, inp["cb"][0], with_stats=True)
    tot = st["resid2"].sum(axis=(0, 2))
    y2 = (fwht(x) ** 2).sum()
    assert tot[0] <= y2
    assert np.all(np.diff(tot) <= 0)


def test_per_vector_error_non_increasing_with_zero_entry():
    rng = np.random.default_rng(5)
    cb = rng.standard_normal((4, 16, 256, 8)).astype(np.float32) * 0.5
    cb[:, :, 0, :] = 0.0                       # entry 0 is the zero vector
    x = rng.standard_normal((500, 128))
    _, st = rvq_encode(x, cb, with_stats=True)
    y = fwht(x)
    e0 = (y.reshape(500, 16, 8) ** 2).sum(-1)
    seq = np.concatenate([e0[:, None, :], st["resid2"]], axis=1)
    assert np.all(np.diff(seq, axis=1) <= 1e-12)


def test_greedy_is_stagewise_not_joint():
    """Exhaustive joint search over all C^S pairs is never worse than greedy,
    and greedy's first choice is the stage-0 nearest entry."""
    rng = np.random.default_rng(11)
    cb = rng.standard_normal((2, 1, 4, 3))
    x = rng.standard_normal((200, 3))
    codes, st = rvq_encode(x, cb, rotate=False, with_stats=True)
    strictly_better = 0
    for n in range(200):
        best = min(np.sum((x[n] - cb[0, 0, a] - cb[1, 0, b]) ** 2)
                   for a, b in itertools.product(range(4), range(4)))
        assert best <= st["resid2"][n, 1, 0] + 1e-12
        strictly_better += best < st["resid2"][n, 1, 0] - 1e-12
        assert codes[n, 0, 0] == np.argmin(((x[n] - cb[0, 0]) ** 2).sum(1))
    assert strictly_better > 0                  # greedy really differs from joint


# --------------------------------------------------------------------------- O3
def test_reconstruct_explicit_loop():
    rng = np.random.default_rng(2)
    cb = rng.standard_normal((3, 4, 16, 2))
    codes = rng.integers(0, 16, size=(7, 3, 4)).astype(np.uint8)
    out = reconstruct_rot(codes, cb)
    for n in range(7):
        for g in range(4):
            for j in range(2):
                ref = 0.0
                for s in range(3):
                    ref += cb[s, g, codes[n, s, g], j]
                assert out[n, 2 * g + j] == pytest.approx(ref, abs=1e-15)


def test_decode_of_encode_is_identity_on_codeword_sums():
    rng = np.random.default_rng(9)
    cb = (rng.standard_normal((2, 16, 256, 8)) * [[[[1.0]]], [[[0.1]]]]).astype(np.float32)
    cb[1, :, 0, :] = 0.0                 # stage 1 can add nothing
    z = rng.integers(0, 256, size=(64, 16))
    x_rot = np.stack([np.concatenate([cb[0, g, z[n, g]] for g in range(16)]) for n in range(64)])
    x = fwht(x_rot)                      # original-domain input whose rotation is a codeword row
    codes = rvq_encode(x, cb)
    assert np.array_equal(codes[:, 0, :], z)
    assert np.all(codes[:, 1, :] == 0)
    assert np.max(np.abs(reconstruct(codes, cb) - x)) <= 1e-12


# --------------------------------------------------------------------------- O4
def _sdpa(q, k, v, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(k), torch.from_numpy(v),
        scale=scale)[:, :, 0, :].numpy()


def test_window_only_equals_dense_softmax_library():
    rng = np.random.default_rng(4)
    B, Hkv, Hq, W, D = 2, 4, 8, 37, 128
    q = rng.standard_normal((B, Hq, D))
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    empty = np.zeros((B, Hkv, 0, 1, 16), dtype=np.uint8)
    got = attend(q, empty, empty, None, None, kw, vw)
    rep = Hq // Hkv
    kk = np.repeat(kw.astype(np.float64), rep, axis=1)   # head h reads kv h // rep
    vv = np.repeat(vw.astype(np.float64), rep, axis=1)
    ref = _sdpa(q, kk, vv, 1 / np.sqrt(D))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 16))
    k = np.repeat(rng.standard_normal((1, 1, 16)), 9, axis=1).repeat(3, axis=0)
    v = rng.standard_normal((3, 9, 16))
    out = attend_dense(q, k, v, 0.25)
    assert np.allclose(out, v.mean(axis=1), atol=1e-14)      # equal keys -> mean of values
    out1 = attend_dense(q, k[:, :1], v[:, :1], 0.25)
    assert np.allclose(out1, v[:, 0], atol=1e-15)            # one token -> its value


def test_lse_partition_invariance():
    rng = np.random.default_rng(8)
    T, D = 1000, 32
    q = rng.standard_normal(D)
    k = rng.standard_normal((T, D)) * 2
    v = rng.standard_normal((T, D))
    full = attend_dense(q[None], k[None], v[None], 0.3)[0]
    cuts = [0, 1, 150, 151, 600, 1000]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = 0.3 * (k[a:b] @ q)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ v[a:b]))
    assert np.max(np.abs(lse_merge(parts) - full)) <= 1e-12


def test_query_side_rotation_identity():
    rng = np.random.default_rng(10)
    q = rng.standard_normal(128)
    k_rot = rng.standard_normal((40, 128))
    assert np.allclose(fwht(k_rot) @ q, k_rot @ fwht(q), atol=1e-12)


def test_attend_coded_matches_library_on_reconstruction():
    w = synth.workload(3, batch=2, tokens=300, window=20)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    x = inp["x_f32"]
    codes = [rvq_encode(x[b].reshape(-1, 128)[:, :], inp["cb"][b]).reshape(w.batch, w.n_kv_heads, w.tokens, 2, 16)
             for b in range(2)]
    kc, vc = codes[0][:, :, :Tc], codes[1][:, :, :Tc]
    got = attend(inp["q"], kc, vc, inp["cb"][0], inp["cb"][1], inp["k_win"], inp["v_win"])
    kh = np.concatenate([reconstruct(kc, inp["cb"][0]), inp["k_win"].astype(np.float64)], axis=2)
    vh = np.concatenate([reconstruct(vc, inp["cb"][1]), inp["v_win"].astype(np.float64)], axis=2)
    rep = w.n_q_heads // w.n_kv_heads
    ref = _sdpa(inp["q"].astype(np.float64), np.repeat(kh, rep, 1), np.repeat(vh, rep, 1),
                1 / np.sqrt(128))
    assert np.max(np.abs(got - ref)) <= 1e-12


# ---------------------------------------------------------------- byte account
def test_compression_ratios_match_pages():
    """'VeloxQuant-MLX 0.5.1', v6 results: product VQ key compression 16x at
    1 bit/elem and 8x at 2 bits/elem, for head_dim 64 and 128 alike."""
    for d in (64, 128):
        assert oracle.compression_ratio_vs_fp16(d, 1, d // 8) == 16.0
        assert oracle.compression_ratio_vs_fp16(d, 2, d // 8) == 8.0
    assert oracle.compression_ratio_vs_fp16(128, 4, 16) == 4.0
    assert oracle.code_bytes_per_vector(2, 16) == 32


# --------------------------------------------------------------- synth inputs
def test_synth_deterministic_and_shaped():
    a = synth.make_inputs(synth.workload(2, tokens=512, window=128))
    b = synth.make_inputs(synth.workload(2, tokens=512, window=128))
    for k in ("x", "cb", "q", "k_win", "v_win"):
        assert np.array_equal(a[k], b[k])
    w = a["workload"]
    assert a["x"].shape == (2, 8, 512, 128) and a["x"].dtype == np.uint16
    assert a["cb"].shape == (2, 1, 16, 256, 8)
    assert a["k_win"].shape == (1, 8, 128, 128) and a["k_win"].dtype == np.float16
    # window = the last W tokens, cast from the bf16 values
    assert np.array_equal(a["k_win"][0, 3].astype(np.float32), a["x_f32"][0, 3, 384:])
    # 4 outlier channels per head (same on K and V), scaled x10: V column energy
    v = a["x_f32"][1].astype(np.float64)
    col = (v ** 2).mean(axis=1)                     # [seq][D]
    assert np.all((col > 30).sum(axis=1) == 4)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    back = synth.bf16_bits_to_f32(synth.bf16_bits(x))
    assert back[0] == 1.0 and back[1] == 1.0            # tie -> even
    assert back[2] == np.float32(1.0 + 4 * 2 ** -8)     # tie -> even (up)
    assert back[3] == -2.5
    assert torch.equal(torch.from_numpy(x).to(torch.bfloat16).float(), torch.from_numpy(back))


# -------------------------------------------------------- planted-slip checks
def test_pins_catch_planted_slips():
    """Local mutants of oracle steps fail the pins above."""
    d = 64
    # (a) missing 1/sqrt(D): H H^T != I
    h_bad = hadamard_matrix(d) * np.sqrt(d)
    assert np.max(np.abs(h_bad @ h_bad.T - np.eye(d))) > 1
    # (b) a sign slip in the Sylvester step: no longer matches scipy
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, -h], [h, h]])
    assert not np.array_equal(h / 8, scipy.linalg.hadamard(d) / 8)
    # (c) argmax instead of argmin breaks the codeword-returns-own-index pin
    rng = np.random.default_rng(3)
    cb = rng.standard_normal((256, 8))
    d2 = ssd.cdist(cb, cb, "sqeuclidean")
    assert not np.array_equal(np.argmax(d2, axis=1), np.arange(256))
    # (d) residual update with + instead of - breaks error monotonicity
    x = rng.standard_normal((500, 8))
    cbs = rng.standard_normal((2, 256, 8)) * [[[1.0]], [[0.5]]]
    r = x.copy()
    errs = [(r ** 2).sum()]
    for s in range(2):
        z = np.argmin(ssd.cdist(r, cbs[s], "sqeuclidean"), axis=1)
        r = r + cbs[s][z]
        errs.append((r ** 2).sum())
    assert np.any(np.diff(errs) > 0)
    # (e) GQA mapping h % Hkv instead of h // rep differs from the library pin
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((2, 5, 16))
    v = rng.standard_normal((2, 5, 16))
    good = attend_dense(q, k, v, 0.25)
    bad = np.stack([attend_dense(q[h:h + 1], k[h % 2:h % 2 + 1], v[h % 2:h % 2 + 1], 0.25)[0]
                    for h in range(8)])
    assert np.max(np.abs(good - bad)) > 1e-3


# ------------------------------------------------------------ streaming window
def _stream(oracle_mod, tokens_k, tokens_v, wcap, n_flush, k_cb, v_cb, code_cap):
    """Append tokens one at a time; flush the oldest n_flush when the window is
    full before an append (the cache protocol of the streaming calls)."""
    B, H, T, D = tokens_k.shape
    S, G = k_cb.shape[0], k_cb.shape[1]
    kw = np.zeros((B, H, wcap, D), np.float16); vw = np.zeros_like(kw)
    kc = np.zeros((B, H, code_cap, S, G), np.uint8); vc = np.zeros_like(kc)
    nw = nc = 0
    for t in range(T):
        if nw == wcap:
            kw, vw, kc, vc = oracle_mod.window_flush(kw, vw, nw, n_flush, kc, vc, nc, k_cb, v_cb)
            nw, nc = nw - n_flush, nc + n_flush
        kw, vw = oracle_mod.window_append(kw, vw, nw, tokens_k[:, :, t], tokens_v[:, :, t])
        nw += 1
    return kw, vw, kc, vc, nw, nc


def test_streaming_window_equals_one_shot_encode():
    """Encoding is per vector, so a cache built by appends and flushes holds
    exactly the one-shot codes of its oldest tokens and the newest tokens
    uncompressed, in order."""
    rng = np.random.default_rng(7)
    B, H, T, D, S, G = 2, 2, 70, 128, 2, 16
    tk = rng.standard_normal((B, H, T, D)).astype(np.float16)
    tv = rng.standard_normal((B, H, T, D)).astype(np.float16)
    k_cb = (rng.standard_normal((S, G, 256, 8)) / np.sqrt(8) * np.array([1, .5])[:, None, None, None])
    v_cb = (rng.standard_normal((S, G, 256, 8)) / np.sqrt(8) * np.array([1, .5])[:, None, None, None])
    kw, vw, kc, vc, nw, nc = _stream(oracle, tk, tv, 24, 16, k_cb, v_cb, 64)
    assert nc == 48 and nw == 22                      # 70 = 48 coded + 22 in the window
    assert np.array_equal(kw[:, :, :nw], tk[:, :, nc:]) and np.array_equal(vw[:, :, :nw], tv[:, :, nc:])
    k_once = oracle.rvq_encode(tk[:, :, :nc].astype(np.float64).reshape(-1, D), k_cb)
    v_once = oracle.rvq_encode(tv[:, :, :nc].astype(np.float64).reshape(-1, D), v_cb)
    assert np.array_equal(kc[:, :, :nc].reshape(-1, S, G), k_once)
    assert np.array_equal(vc[:, :, :nc].reshape(-1, S, G), v_once)
    # the streamed cache attends like the whole sequence with those codes
    q = rng.standard_normal((B, 4, D))
    a = oracle.attend(q, kc[:, :, :nc], vc[:, :, :nc], k_cb, v_cb, kw[:, :, :nw], vw[:, :, :nw])
    kk = np.concatenate([np.stack([oracle.reconstruct(kc[b, :, :nc].reshape(-1, S, G), k_cb)
                                   .reshape(H, nc, D) for b in range(B)]),
                         tk[:, :, nc:].astype(np.float64)], axis=2)
    vv = np.concatenate([np.stack([oracle.reconstruct(vc[b, :, :nc].reshape(-1, S, G), v_cb)
                                   .reshape(H, nc, D) for b in range(B)]),
                         tv[:, :, nc:].astype(np.float64)], axis=2)
    ref = np.stack([oracle.attend_dense(q[b], kk[b], vv[b], 1 / np.sqrt(D)) for b in range(B)])
    assert np.allclose(a, ref, rtol=0, atol=1e-12)


def test_window_flush_moves_rows_and_keeps_the_tail():
    rng = np.random.default_rng(3)
    kw = rng.standard_normal((1, 1, 10, 64)).astype(np.float16)
    vw = rng.standard_normal((1, 1, 10, 64)).astype(np.float16)
    cb = rng.standard_normal((1, 1, 256, 64)) / 8
    kc = np.zeros((1, 1, 8, 1, 1), np.uint8)
    k2, v2, kc2, vc2 = oracle.window_flush(kw, vw, 9, 3, kc, kc.copy(), 5, cb, cb)
    assert np.array_equal(k2[0, 0, :6], kw[0, 0, 3:9])       # moved to the front
    assert np.array_equal(k2[0, 0, 6:], kw[0, 0, 6:])        # rows past the count untouched
    assert np.array_equal(kc2[0, 0, :5], kc[0, 0, :5])       # earlier codes untouched
    assert np.array_equal(kc2[0, 0, 5:8, 0, 0],
                          oracle.rvq_encode(kw[0, 0, :3].astype(np.float64), cb)[:, 0, 0])
    with pytest.raises(ValueError):
        oracle.window_flush(kw, vw, 9, 3, kc, kc, 6, cb, cb)  # code buffer too small


# ------------------------------------------------------------- dual transform
# "VeloxQuant-MLX 0.5.1", VecInfer section: each key channel is divided by
# sqrt(max |K_i|) before the Walsh-Hadamard rotation, and the inverse is folded
# into the query, leaving the scores unchanged.
def test_smooth_factors_hand_values():
    """Channel maxima worked by hand: sequences 0 and 2 share row 0 at two
    rows, every sequence row 0 at one row, row 3 of four has no sequence."""
    k = np.array([[[-4.0, 0.0, 0.25], [1.0, 0.0, -9.0]],      # |max| 4, 0, 9
                  [[2.0, 0.0, 0.0], [0.0, 0.0, 0.0]],         # |max| 2, 0, 0
                  [[0.0, 1.0, 0.0], [0.0, -16.0, 0.0]]])      # |max| 0, 16, 0
    assert np.array_equal(oracle.smooth_factors(k, 1), [[2.0, 4.0, 3.0]])
    assert np.array_equal(oracle.smooth_factors(k, 2), [[2.0, 4.0, 3.0], [np.sqrt(2.0), 1.0, 1.0]])
    lam4 = oracle.smooth_factors(k, 4)
    assert np.array_equal(lam4[0], [2.0, 1.0, 3.0]) and np.array_equal(lam4[3], [1.0, 1.0, 1.0])
    assert np.array_equal(lam4[2], [1.0, 4.0, 1.0])
    assert np.array_equal(oracle.smooth_rows(lam4, [0, 5, 7]), lam4[[0, 1, 3]])


def test_smoothing_square_roots_the_channel_maxima():
    """After division by sqrt(max |K_i|) the largest magnitude of channel i
    is sqrt(max |K_i|): the spread between channels is square-rooted."""
    rng = np.random.default_rng(11)
    k = rng.standard_normal((3, 200, 64)) * np.exp(rng.uniform(-2, 3, size=64))
    lam = oracle.smooth_factors(k, 1)
    ks = oracle.smooth_keys(k, lam[0])
    mx, mxs = np.abs(k).max(axis=(0, 1)), np.abs(ks).max(axis=(0, 1))
    assert np.allclose(mxs, np.sqrt(mx), rtol=1e-14)
    assert np.isclose(mxs.max() / mxs.min(), np.sqrt(mx.max() / mx.min()), rtol=1e-12)


def test_smooth_absorption_leaves_scores_unchanged():
    """(H (lam * q)) . (H (k / lam)) = q . k for every key: H is orthonormal."""
    rng = np.random.default_rng(12)
    k = rng.standard_normal((1, 300, 128)) * np.r_[np.full(124, 1.0), np.full(4, 10.0)]
    q = rng.standard_normal((5, 128))
    lam = oracle.smooth_factors(k, 1)[0]
    lhs = fwht(oracle.smooth_query(q, lam)) @ fwht(oracle.smooth_keys(k[0], lam)).T
    assert np.allclose(lhs, q @ k[0].T, rtol=0, atol=1e-11 * np.abs(q @ k[0].T).max())
    # the wrong direction (dividing the query) does not cancel
    bad = fwht(q / lam) @ fwht(oracle.smooth_keys(k[0], lam)).T
    assert np.max(np.abs(bad - q @ k[0].T)) > 1e-2


def test_smooth_encode_special_cases():
    """Factors of 1 change nothing; with a uniform power-of-two factor c,
    |x/c - e|^2 = |x - c e|^2 / c^2 exactly, so coding x/c equals coding x
    with the codebooks multiplied by c (and differs from dividing them)."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((400, 128))
    cb = rng.standard_normal((2, 16, 256, 8)) / np.sqrt(8) * np.array([1, .5])[:, None, None, None]
    assert np.array_equal(oracle.smooth_encode(x, np.ones(128), cb), rvq_encode(x, cb))
    assert np.array_equal(oracle.smooth_encode(x, np.full(128, 4.0), cb), rvq_encode(x, cb * 4.0))
    assert not np.array_equal(oracle.smooth_encode(x, np.full(128, 4.0), cb), rvq_encode(x, cb / 4.0))


def test_smooth_attention_with_representable_codebooks_is_exact():
    """Codebooks whose entries are exactly the smoothed, rotated key groups
    (and the rotated value groups) reproduce every coded token, so smoothed
    decode attention equals textbook softmax attention over the original keys
    and values; the fp16 window keeps its original keys."""
    rng = np.random.default_rng(14)
    B, Hkv, Hq, T, W, D, G = 2, 2, 4, 150, 9, 64, 8
    dsub = D // G
    k = rng.standard_normal((B, Hkv, T, D)) * np.exp(rng.uniform(-1, 2, size=(1, Hkv, 1, D)))
    v = rng.standard_normal((B, Hkv, T, D))
    kw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    vw = rng.standard_normal((B, Hkv, W, D)).astype(np.float16)
    lam = oracle.smooth_factors(k.reshape(B * Hkv, T, D), Hkv)          # one row per KV head
    q = rng.standard_normal((B, Hq, D))
    kc = np.empty((B, Hkv, T, 1, G), np.uint8); vc = np.empty_like(kc)
    out = np.empty((B, Hq, D))
    for b in range(B):
        for h in range(Hkv):
            # one codebook set per (sequence, KV head): entry t = token t's group
            kt = fwht(oracle.smooth_keys(k[b, h], lam[h]))
            vt = fwht(v[b, h])
            far = 1e3 * (1 + np.arange(256 - T))[:, None]
            kcb = np.stack([np.concatenate([kt[:, g * dsub:(g + 1) * dsub], far + 0 * kt[:1, :dsub]])
                            for g in range(G)])[None]
            vcb = np.stack([np.concatenate([vt[:, g * dsub:(g + 1) * dsub], far + 0 * vt[:1, :dsub]])
                            for g in range(G)])[None]
            zk = oracle.smooth_encode(k[b, h], lam[h], kcb)
            assert np.array_equal(zk[:, 0, :], np.repeat(np.arange(T)[:, None], G, 1))
            one = oracle.attend(q[b:b + 1, 2 * h:2 * h + 2], zk[None, None], rvq_encode(v[b, h], vcb)[None, None],
                                kcb, vcb, kw[b:b + 1, h:h + 1], vw[b:b + 1, h:h + 1],
                                k_smooth=lam[h:h + 1])
            ref = attend_dense(q[b, 2 * h:2 * h + 2],
                               np.concatenate([k[b, h:h + 1], kw[b, h:h + 1].astype(np.float64)], 1),
                               np.concatenate([v[b, h:h + 1], vw[b, h:h + 1].astype(np.float64)], 1),
                               1 / np.sqrt(D))
            assert np.allclose(one[0], ref, rtol=0, atol=1e-10)
            # the factor row is chosen by (b * Hkv + kv) % n_scale
            two = oracle.attend(q[b:b + 1, 2 * h:2 * h + 2], zk[None, None], rvq_encode(v[b, h], vcb)[None, None],
                                kcb, vcb, kw[b:b + 1, h:h + 1], vw[b:b + 1, h:h + 1],
                                k_smooth=np.stack([lam[h]] * (b + 1)))
            assert np.allclose(two, one, rtol=0, atol=1e-12)


def test_streaming_with_smoothing_equals_one_shot_smooth_encode():
    """Flushed keys are smoothed with their (sequence, KV head) row; values
    are not smoothed."""
    rng = np.random.default_rng(15)
    B, H, T, D, S, G = 2, 3, 40, 64, 1, 8
    tk = (rng.standard_normal((B, H, T, D)) * np.exp(rng.uniform(-1, 2, size=D))).astype(np.float16)
    tv = rng.standard_normal((B, H, T, D)).astype(np.float16)
    cb = rng.standard_normal((S, G, 256, 8)) / np.sqrt(8)
    lam = oracle.smooth_factors(tk.reshape(B * H, T, D).astype(np.float64), H)
    kw = np.zeros((B, H, 16, D), np.float16); vw = np.zeros_like(kw)
    kc = np.zeros((B, H, 32, S, G), np.uint8); vc = np.zeros_like(kc)
    nw = nc = 0
    for t in range(T):
        if nw == 16:
            kw, vw, kc, vc = oracle.window_flush(kw, vw, nw, 8, kc, vc, nc, cb, cb, k_smooth=lam)
            nw, nc = nw - 8, nc + 8
        kw, vw = oracle.window_append(kw, vw, nw, tk[:, :, t], tv[:, :, t])
        nw += 1
    assert nc == 24
    xk = tk[:, :, :nc].astype(np.float64)
    lam_rows = oracle.smooth_rows(lam, np.arange(B * H)).reshape(B, H, 1, D)
    k_once = oracle.smooth_encode(xk, np.broadcast_to(lam_rows, xk.shape), cb)
    assert np.array_equal(kc[:, :, :nc].reshape(-1, S, G), k_once)
    v_once = rvq_encode(tv[:, :, :nc].astype(np.float64).reshape(-1, D), cb)
    assert np.array_equal(vc[:, :, :nc].reshape(-1, S, G), v_once)
    assert not np.array_equal(k_once, rvq_encode(xk.reshape(-1, D), cb))


# ---------------------------------------------------------- codebook fitting
# "VeloxQuant-MLX 0.5.1", VecInfer section: K-means codebooks trained before
# use; "VQKV" summary, 2. Methodology: trained stage codebooks.
def test_lloyd_update_hand_values():
    """Means worked by hand; an entry that attracts no vector keeps its value."""
    r = np.array([[0.0], [1.0], [10.0], [11.0]])
    new = oracle.lloyd_update(r, np.array([0, 0, 1, 1]), np.array([[0.0], [10.0], [100.0]]))
    assert np.array_equal(new, [[0.5], [10.5], [100.0]])


@pytest.mark.parametrize("rotate", [False, True])
def test_fit_single_stage_equals_scipy_kmeans2(rotate):
    """One stage, one group: Lloyd iterations from a given start equal
    scipy.cluster.vq.kmeans2 (minit='matrix'), including kept empty entries."""
    from scipy.cluster.vq import kmeans2
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1500, 8)) * np.array([1, 2, 3, 1, 1, .5, 1, 4])
    init = rng.standard_normal((1, 1, 24, 8))
    init[0, 0, 5] = 50.0                                   # never nearest: stays put
    fitted = oracle.fit_codebooks(x, init, 6, rotate=rotate)
    y = fwht(x) if rotate else x
    with np.errstate(all="ignore"), __import__("warnings").catch_warnings():
        __import__("warnings").simplefilter("ignore")
        ref, _ = kmeans2(y, init[0, 0].copy(), iter=6, minit="matrix", missing="warn")
    assert np.allclose(fitted[0, 0], ref, rtol=0, atol=1e-12)
    assert np.array_equal(fitted[0, 0, 5], init[0, 0, 5])


def test_fit_groups_independent_and_stages_on_residuals():
    """Groups fit on their own column slices; stage 1 fits the residuals the
    fitted stage 0 leaves (assignment with the final stage-0 entries)."""
    from scipy.cluster.vq import kmeans2, vq
    import warnings
    rng = np.random.default_rng(32)
    x = rng.standard_normal((900, 16))
    init = rng.standard_normal((2, 2, 12, 8)) * np.array([1.0, 0.5])[:, None, None, None]
    fitted = oracle.fit_codebooks(x, init, 4, rotate=False)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for g in range(2):
            y = x[:, 8 * g:8 * g + 8]
            c0, _ = kmeans2(y, init[0, g].copy(), iter=4, minit="matrix", missing="warn")
            z0, _ = vq(y, c0)
            c1, _ = kmeans2(y - c0[z0], init[1, g].copy(), iter=4, minit="matrix", missing="warn")
            assert np.allclose(fitted[0, g], c0, atol=1e-12)
            assert np.allclose(fitted[1, g], c1, atol=1e-12)


def test_fit_distortion_never_increases():
    """Lloyd's property: each assignment's distortion is at most the one
    before it, per (stage, group)."""
    rng = np.random.default_rng(33)
    x = rng.laplace(size=(2000, 32)) * np.exp(rng.uniform(-1, 1, 32))
    init = rng.standard_normal((2, 4, 32, 8))
    _, hist = oracle.fit_codebooks(x, init, 8, with_history=True)
    for s in range(2):
        for g in range(4):
            h = np.array(hist[s][g])
            assert len(h) == 9
            assert np.all(np.diff(h) <= 1e-9 * h[0]), h
            assert h[-1] < h[0]


# -------------------------------------------------- scalar residual variant
# "VeloxQuant-MLX 0.5.1": Architecture, TurboQuantRVQ pipeline (Gaussian then
# Laplacian Lloyd-Max stages on the rotated vector, decode by summing and
# unrotating); throughput journey (boundary-sum quantise, same indices as the
# argmin); module table (dsa.bit_pack sub-byte index packing).
# Lloyd-Max reference values: J. Max, "Quantizing for minimum distortion" (1960),
# unit-variance Gaussian; M. D. Paez and T. H. Glisson, "Minimum mean-squared-
# error quantization in speech PCM and DPCM systems" (1972), unit-variance
# Laplacian.  Positive half of each symmetric level set.
MAX_GAUSS = {1: [0.7979], 2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152],
             4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733]}
PG_LAPLACE = {1: [0.7071], 2: [0.4198, 1.834], 3: [0.2334, 0.8330, 1.6725, 3.0867]}


@pytest.mark.parametrize("kind,table", [("gaussian", MAX_GAUSS), ("laplacian", PG_LAPLACE)])
def test_lloyd_max_levels_match_published_tables(kind, table):
    for bits, half in table.items():
        lv = oracle.lloyd_max_levels(kind, bits)
        assert np.allclose(lv, -lv[::-1], atol=1e-12)                 # symmetric
        assert np.allclose(lv[len(lv) // 2:], half, rtol=0, atol=1.5e-3), (kind, bits, lv)
    one = oracle.lloyd_max_levels(kind, 1)[1]
    assert np.isclose(one, np.sqrt(2 / np.pi) if kind == "gaussian" else 1 / np.sqrt(2),
                      rtol=0, atol=1e-10)                            # E|X| in closed form


def test_lloyd_max_distortion_closed_form_and_table():
    g1 = oracle.lloyd_max_distortion("gaussian", oracle.lloyd_max_levels("gaussian", 1))
    assert np.isclose(g1, 1 - 2 / np.pi, rtol=0, atol=1e-9)
    for bits, mse in ((2, 0.1175), (3, 0.03454), (4, 0.009497)):      # Max (1960)
        d = oracle.lloyd_max_distortion("gaussian", oracle.lloyd_max_levels("gaussian", bits))
        assert np.isclose(d, mse, rtol=2e-3), (bits, d)


def test_boundary_sum_equals_nearest_level():
    """The pages report 100 % index match of boundary-sum against argmin."""
    rng = np.random.default_rng(41)
    for bits in (1, 2, 3, 4):
        for kind in ("gaussian", "laplacian"):
            lv = oracle.lloyd_max_levels(kind, bits) * rng.uniform(0.3, 3.0)
            y = rng.standard_normal(50000) * 2
            assert np.array_equal(oracle.boundary_sum(y, lv), oracle.scalar_nearest(y, lv))


def test_pack_bits_hand_fixture_and_roundtrip():
    assert oracle.pack_bits(np.array([[1, 0, 1, 1, 0, 0, 0, 1]]), 1)[0, 0] == 0x8D
    assert oracle.pack_bits(np.array([[3, 0, 1, 2]]), 2)[0, 0] == 0x93
    assert oracle.pack_bits(np.array([[0xA, 0x5]]), 4)[0, 0] == 0x5A
    # 3 bits: elements 5, 3, 6, 1, 7, 0, 2, 4 give the bit string (each element
    # least significant bit first) 101 110 011 100 111 000 010 001, i.e. the
    # bytes (first bit = bit 0) 10111001, 11001110, 00010001 = 0x9D, 0x73, 0x88;
    # the same as the little-endian bytes of sum z_i * 8^i = 0x88739D
    z3 = np.array([[5, 3, 6, 1, 7, 0, 2, 4]])
    assert sum(int(v) << (3 * i) for i, v in enumerate(z3[0])) == 0x88739D
    assert list(oracle.pack_bits(z3, 3)[0]) == [0x9D, 0x73, 0x88]
    assert np.array_equal(oracle.unpack_bits(np.array([[0x9D, 0x73, 0x88]], dtype=np.uint8), 3), z3)
    rng = np.random.default_rng(42)
    for bits in (1, 2, 3, 4):
        z = rng.integers(0, 2 ** bits, size=(7, 128))
        p = oracle.pack_bits(z, bits)
        assert p.shape == (7, 128 * bits // 8)
        assert np.array_equal(oracle.unpack_bits(p, bits), z)


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_product_codebook_decodes_packed_scalar_codes(bits):
    """A packed byte of stage s is an ordinary code of the product codebook:
    the VQ reconstruction of the packed codes equals the scalar one."""
    rng = np.random.default_rng(43)
    D = 64
    l1 = oracle.lloyd_max_levels("gaussian", bits) * 1.7
    l2 = oracle.lloyd_max_levels("laplacian", bits) * 0.4
    x = rng.standard_normal((300, D)) * 1.7
    z1, z2 = oracle.scalar_rvq_encode(x, l1, l2)
    codes = np.stack([oracle.pack_bits(z1, bits), oracle.pack_bits(z2, bits)], axis=1)
    cb = oracle.scalar_product_codebook(l1, l2, bits, D)
    assert cb.shape == (2, D * bits // 8, 256, 8 // bits)
    assert np.array_equal(reconstruct_rot(codes, cb),
                          oracle.scalar_reconstruct(z1, z2, l1, l2, unrotate=False))
    # and decode attention over either form agrees
    q = rng.standard_normal((1, 2, D))
    kc = codes.reshape(1, 1, 300, 2, -1)
    a = oracle.attend_scalar(q, kc, kc, (l1, l2), (l1, l2), bits)
    b = oracle.attend(q, kc, kc, cb, cb)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_scalar_rvq_stage_errors_follow_lloyd_max():
    """On Gaussian vectors (still Gaussian after the orthonormal rotation) the
    first stage's mean squared error per element is the Lloyd-Max distortion;
    the Laplacian second stage, scaled to the residual's deviation, lowers it."""
    rng = np.random.default_rng(44)
    x = rng.standard_normal((20000, 64)) * 2.0
    for bits in (1, 2):
        d1 = oracle.lloyd_max_distortion("gaussian", oracle.lloyd_max_levels("gaussian", bits))
        l1 = oracle.lloyd_max_levels("gaussian", bits) * 2.0
        l2 = oracle.lloyd_max_levels("laplacian", bits) * 2.0 * np.sqrt(d1)
        z1, z2 = oracle.scalar_rvq_encode(x, l1, l2)
        y = oracle.fwht(x)
        e1 = np.mean((y - l1[z1]) ** 2) / 4.0
        e2 = np.mean((y - oracle.scalar_reconstruct(z1, z2, l1, l2, unrotate=False)) ** 2) / 4.0
        assert abs(e1 - d1) < 0.02 * d1, (bits, e1, d1)
        assert e2 < 0.5 * e1
