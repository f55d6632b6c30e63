"""Parity of kvq_codebook_fit (K-means / Lloyd fitting of the residual product
codebooks on a sample) with the float64 oracle, through the C ABI.

K-means is iterative, so the element-wise check is one iteration at a time:
the GPU's assignment (the encode kernels, run with the same entries and the
earlier stages' fitted ones) follows the code rule against the oracle's
distances, and every fitted entry equals the oracle's mean of the residuals
(y minus the earlier-stage entries that same assignment chose, the chain
taken in float64) the GPU assigned to it within 1e-6 * the largest residual
component of its group (the fixed-point sums themselves are exact to 2^-30
of that bound), plus, at stage s > 0, s * 2^-23 * max|y| of the group: the
kernel forms its residuals in float32, one rounding per subtraction.  Entries
no vector chose must come back bit-identical.  Over several iterations the
checks are Lloyd's properties: the distortion of the fitted codebooks never
increases, and ends within 1 % of the oracle's own fit from the same start.
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


def sample(key, n_rows, **over):
    """Keys of a workload as the fitting sample: x [n_seq][T][D] on the GPU
    (bf16 or fp32), their float64 values, the K codebooks as start."""
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    if w.x_dtype == "bf16":
        x = torch.from_numpy(inp["x"][0].view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp["x"][0]).cuda()
    xf = inp["x_f32"][0][:, :n_rows].astype(np.float64)
    return w, x, xf, inp["cb"][0]


def residual(y, cb, codes, s):
    """The oracle's residual chain in float64: y minus the entries of stages
    0..s-1 that codes [n][>=s][G] chose (the GPU's codes, teacher-forced)."""
    G = cb.shape[1]
    r = np.asarray(y, dtype=np.float64).copy()
    for t in range(s):
        r -= np.concatenate([cb[t, g][codes[:, t, g]] for g in range(G)], axis=1).astype(np.float64)
    return r


def check_step(r, z, init, fitted, dsub, y=None, s=0):
    """One Lloyd update per group: the fitted entries against the oracle's
    float64 means of r over the GPU's assignment z; unchosen entries
    unchanged.  The kernel's residuals of stage s are float32 (the rotation
    rounded once, then s subtractions each rounded once), so beyond the
    1e-6 * max|r| bound of the sums a stage-s entry may differ from the
    float64 chain by s * 2^-23 * max|y| of its group."""
    G = init.shape[0]
    for g in range(G):
        rg = r[:, g * dsub:(g + 1) * dsub]
        ref = oracle.lloyd_update(rg, z[:, g], init[g])
        tol = 1e-6 * np.abs(rg).max()
        if s > 0:
            tol += s * 2.0 ** -23 * np.abs(y[:, g * dsub:(g + 1) * dsub]).max()
        err = np.abs(fitted[g].astype(np.float64) - ref)
        assert err.max() <= tol, (g, err.max(), tol)
        unused = np.setdiff1d(np.arange(init.shape[1]), z[:, g])
        assert np.array_equal(fitted[g][unused], init[g][unused])


@pytest.mark.parametrize("key,over,n_rows", [
    (2, dict(tokens=2100, window=0), 2000),     # S = 1, outlier channels, MFMA assignment
    (1, dict(), 1024),                          # D = 64, one 64-dim group, S = 2, generic kernel
])
def test_fit_one_iteration_parity(key, over, n_rows):
    say(f"codebook fit, one iteration, workload {key} {over} rows {n_rows}")
    w, x, xf, init = sample(key, n_rows, **over)
    S, G, C, dsub = init.shape
    fitted = kvq.codebook_fit(x, cuda(init), 1, n_rows=n_rows).cpu().numpy()
    y = oracle.fwht(xf.reshape(-1, w.head_dim))
    # stage 0: the GPU's assignment with the starting entries
    z0 = kvq.encode(x[None], cuda(init[None, :1]), n_rows=n_rows).cpu().numpy()
    z0 = z0.reshape(-1, 1, G)
    res = oracle.check_codes(y, init[:1], z0, rotate=False)
    say("   stage 0 assignment", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
    assert res["hard"] == 0
    check_step(y, z0[:, 0], init[0], fitted[0], dsub)
    if S > 1:
        # stage 1's assignment runs the fitted stage 0 and then stage 1; its
        # residuals are y minus the stage-0 entries that same call chose
        both = np.concatenate([fitted[:1], init[1:2]])
        zz = kvq.encode(x[None], cuda(both[None]), n_rows=n_rows).cpu().numpy().reshape(-1, 2, G)
        r1 = residual(y, fitted, zz, 1)
        z1 = zz[:, 1]
        res = oracle.check_codes(r1, init[1:2], z1[:, None, :], rotate=False)
        say("   stage 1 assignment", {k: res[k] for k in ("total", "exact", "near_tie", "hard")})
        assert res["hard"] == 0
        check_step(r1, z1, init[1], fitted[1], dsub, y, 1)


@pytest.mark.parametrize("D,dsub,S,C,dt", [
    (128, 16, 1, 64, "f32"),
    (128, 8, 2, 256, "f16"),
    (256, 8, 2, 100, "f32"),
    (256, 32, 1, 256, "bf16"),
    (256, 16, 1, 64, "f16"),
    (64, 16, 2, 64, "bf16"),
    (64, 8, 1, 100, "f16"),
])
def test_fit_kernel_instances(D, dsub, S, C, dt):
    """The fitting kernels' (head size, input dtype) preparation instances,
    accumulation slices of 8, 16 and 32 dims and the between-stage bound at
    each head size, on random samples (two sequences, a ragged row count):
    one Lloyd iteration per stage against the oracle's update over the GPU's
    assignment, as in the workload tests above."""
    G = D // dsub
    say(f"codebook fit instance D {D} dsub {dsub} S {S} C {C} {dt}")
    rng = np.random.default_rng(7200 + D + dsub + S + C)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    n_rows = 590
    x = torch.from_numpy(rng.standard_normal((2, 600, D)).astype(np.float32)).to(tdt).cuda()
    xf = x[:, :n_rows].double().cpu().numpy()
    init = (rng.standard_normal((S, G, C, dsub)) / np.sqrt(dsub)
            * (0.5 ** np.arange(S))[:, None, None, None]).astype(np.float32)
    fitted = kvq.codebook_fit(x, cuda(init), 1, n_rows=n_rows).cpu().numpy()
    y = oracle.fwht(xf.reshape(-1, D))
    z0 = kvq.encode(x[None], cuda(init[None, :1]), n_rows=n_rows).cpu().numpy().reshape(-1, 1, G)
    res = oracle.check_codes(y, init[:1], z0, rotate=False)
    assert res["hard"] == 0
    check_step(y, z0[:, 0], init[0], fitted[0], dsub)
    if S > 1:
        both = np.concatenate([fitted[:1], init[1:2]])
        zz = kvq.encode(x[None], cuda(both[None]), n_rows=n_rows).cpu().numpy().reshape(-1, 2, G)
        r1 = residual(y, fitted, zz, 1)
        res = oracle.check_codes(r1, init[1:2], zz[:, 1][:, None, :], rotate=False)
        assert res["hard"] == 0
        check_step(r1, zz[:, 1], init[1], fitted[1], dsub, y, 1)


def test_fit_one_iteration_two_stages_mfma():
    """Stage chaining on the MFMA assignment (Qwen-shaped keys, S = 2)."""
    say("codebook fit, one iteration, two stages, MFMA assignment")
    w, x, xf, init = sample(3, 1500, batch=1, tokens=1500, window=0)
    S, G, C, dsub = init.shape
    fitted = kvq.codebook_fit(x, cuda(init), 1).cpu().numpy()
    y = oracle.fwht(xf.reshape(-1, 128))
    z0 = kvq.encode(x[None], cuda(init[None, :1])).cpu().numpy().reshape(-1, G)
    check_step(y, z0, init[0], fitted[0], dsub)
    both = np.concatenate([fitted[:1], init[1:2]])
    zz = kvq.encode(x[None], cuda(both[None])).cpu().numpy().reshape(-1, 2, G)
    r1 = residual(y, fitted, zz, 1)
    z1 = zz[:, 1]
    res = oracle.check_codes(r1, init[1:2], z1[:, None, :], rotate=False)
    assert res["hard"] == 0
    check_step(r1, z1, init[1], fitted[1], dsub, y, 1)


def test_fit_smoothed_keys_one_iteration():
    say("codebook fit on smoothed keys, one iteration")
    w, x, xf, init = sample(2, 1500, tokens=1500, window=0)
    G, dsub = init.shape[1], init.shape[3]
    lam = oracle.smooth_factors(xf, w.n_kv_heads).astype(np.float32)
    init = (init * np.float32(0.25)).astype(np.float32)
    fitted = kvq.codebook_fit(x, cuda(init), 1, smooth=cuda(lam)).cpu().numpy()
    rows = oracle.smooth_rows(lam.astype(np.float64), np.arange(w.n_seq))[:, None, :]
    y = oracle.fwht(oracle.smooth_keys(xf, rows).reshape(-1, 128))
    z0 = kvq.encode(x[None], cuda(init[None]), smooth=cuda(lam[None])).cpu().numpy()
    z0 = z0.reshape(-1, G)
    res = oracle.check_codes(y, init, z0[:, None, :], rotate=False)
    assert res["hard"] == 0
    check_step(y, z0, init[0], fitted[0], dsub)


def test_fit_deterministic_and_zero_iterations():
    say("codebook fit: repeatable, n_iter = 0 leaves the entries")
    w, x, xf, init = sample(3, 1000, batch=1, tokens=1000, window=0)
    cb = cuda(init)
    a = kvq.codebook_fit(x, cb, 3)
    b = kvq.codebook_fit(x, cb, 3)
    assert torch.equal(a, b)
    assert not torch.equal(a, cb)
    assert torch.equal(kvq.codebook_fit(x, cb, 0), cb)
    ws = torch.empty(kvq.codebook_fit_workspace_size(128, 16, 2, 256, 4 * 1000), dtype=torch.uint8,
                     device="cuda")
    c = kvq.codebook_fit(x, cb, 3, workspace=ws)         # a workspace passed in, then reused
    d = kvq.codebook_fit(x, cb, 3, workspace=ws)
    assert torch.equal(a, c) and torch.equal(c, d)


def test_fit_distortion_never_increases_and_matches_oracle_fit():
    """Lloyd's property on the GPU fits with 0, 1, 2, 4, 8 iterations (the
    oracle measures each fitted codebook's distortion exactly), and the
    8-iteration distortion is within 1 % of the oracle's own 8-iteration fit
    from the same start."""
    say("codebook fit: distortion over iterations")
    w, x, xf, init = sample(2, 512, tokens=512, window=0)
    G, dsub = init.shape[1], init.shape[3]
    y = oracle.fwht(xf.reshape(-1, 128))

    def distortion(cb):
        tot = 0.0
        for g in range(G):
            z, d = oracle.nearest(y[:, g * dsub:(g + 1) * dsub], cb[0, g])
            tot += d[np.arange(len(z)), z].sum()
        return tot

    cb0 = cuda(init)
    ds = [distortion(kvq.codebook_fit(x, cb0, k).cpu().numpy().astype(np.float64))
          for k in (0, 1, 2, 4, 8)]
    say("   distortion", [f"{d:.6g}" for d in ds])
    assert all(b <= a * (1 + 1e-6) for a, b in zip(ds, ds[1:])), ds
    assert ds[-1] < 0.9 * ds[0]
    ref = distortion(oracle.fit_codebooks(xf.reshape(-1, 128), init, 8))
    say("   oracle fit", f"{ref:.6g}")
    assert abs(ds[-1] - ref) <= 0.01 * ref


def test_fit_five_stages_mfma_then_generic():
    """Five stages: the assignments of stages 0-3 run on the MFMA path (packed
    codebooks in the workspace), stage 4's on the generic kernel.  Stage 0 and
    stage 4 each follow one Lloyd update of the GPU's own assignment."""
    say("codebook fit, five stages")
    w, x, xf, init3 = sample(3, 1200, batch=1, tokens=1200, window=0)
    rng = np.random.default_rng(51)
    G, C, dsub = 16, 256, 8
    init = (rng.standard_normal((5, G, C, dsub)) / np.sqrt(8)
            * (0.5 ** np.arange(5))[:, None, None, None]).astype(np.float32)
    fitted = kvq.codebook_fit(x, cuda(init), 1).cpu().numpy()
    assert np.all(np.isfinite(fitted))
    y = oracle.fwht(xf.reshape(-1, 128))
    z0 = kvq.encode(x[None], cuda(init[None, :1])).cpu().numpy().reshape(-1, G)
    check_step(y, z0, init[0], fitted[0], dsub)
    # stage 4's assignment (generic kernel) runs the four fitted stages itself;
    # its residuals follow that call's own stage 0-3 codes
    both = np.concatenate([fitted[:4], init[4:5]])
    zz = kvq.encode(x[None], cuda(both[None])).cpu().numpy().reshape(-1, 5, G)
    r4 = residual(y, fitted, zz, 4)
    z4 = zz[:, 4]
    res = oracle.check_codes(r4, init[4:5], z4[:, None, :], rotate=False)
    assert res["hard"] == 0
    check_step(r4, z4, init[4], fitted[4], dsub, y, 4)
    assert torch.equal(kvq.codebook_fit(x, cuda(init), 1), cuda(fitted))
