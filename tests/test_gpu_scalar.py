"""Parity of the scalar residual variant (two Lloyd-Max stages on the rotated
vector, boundary-sum indices, sub-byte packing) with the float64 oracle,
through the C ABI.

Bars: indices equal the oracle's nearest levels except where the candidate's
squared distance is within a relative 1e-4 of the best level's, the code rule
of the vector quantiser (oracle.check_scalar_codes); reconstruction in the rotated
domain within one float32 rounding of the level sum, unrotated within 1e-6 *
|x_hat|; the product codebook bit-exact; decode attention through it within
2e-3 max-abs and 1e-3 relative L2 of the oracle's attention over the scalar
reconstruction.  Levels: the oracle's Lloyd-Max levels, stage 1 scaled by the
sample's per-element deviation, stage 2 by that times the square root of the
stage-1 distortion (the residual's deviation for a Gaussian source).
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


_LEVELS = {}


def unit_levels(bits):
    if bits not in _LEVELS:
        g = oracle.lloyd_max_levels("gaussian", bits)
        _LEVELS[bits] = (g, oracle.lloyd_max_levels("laplacian", bits),
                         oracle.lloyd_max_distortion("gaussian", g))
    return _LEVELS[bits]


def book_levels(xf, bits):
    """[n_books][2][2^bits] float32 levels for the books of xf [nb][...][D]."""
    g, lap, dg = unit_levels(bits)
    out = []
    for b in range(xf.shape[0]):
        sd = float(np.sqrt(np.mean(np.asarray(xf[b], dtype=np.float64) ** 2)))
        out.append([g * sd, lap * sd * np.sqrt(dg)])
    return np.asarray(out, dtype=np.float32)


@pytest.mark.parametrize("key,over", [
    (2, dict(tokens=1300, window=128)),        # bf16 with outlier channels, rows < stride
    (3, dict(batch=2, tokens=700, window=64)),
    (1, dict()),                                # fp32, D = 64
])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_scalar_encode_parity(key, over, bits):
    say(f"scalar encode workload {key} {over} bits {bits}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    x = to_dev(inp["x"], w)
    xf = inp["x_f32"][:, :, :Tc]
    lv = book_levels(xf, bits)
    codes = kvq.scalar_encode(x, cuda(lv), bits, n_rows=Tc).cpu().numpy()
    assert codes.shape == (x.shape[0], w.n_seq, Tc, 2, w.head_dim * bits // 8)
    tot = {"total": 0, "exact": 0, "near_tie": 0, "hard": 0}
    for b in range(x.shape[0]):
        z = oracle.unpack_bits(codes[b].reshape(-1, 2, codes.shape[-1]), bits)
        y = oracle.fwht(xf[b].reshape(-1, w.head_dim).astype(np.float64))
        res = oracle.check_scalar_codes(y, lv[b, 0], lv[b, 1], z[:, 0], z[:, 1])
        for k in tot:
            tot[k] += res[k]
    say("   ", tot)
    assert tot["hard"] == 0 and tot["exact"] >= 0.9999 * tot["total"]


def test_scalar_encode_pre_rotated_and_f16():
    say("scalar encode, pre-rotated f32 and f16 inputs")
    w = synth.workload(3, batch=1, tokens=900, window=0)
    inp = synth.make_inputs(w)
    xf = inp["x_f32"].astype(np.float64)
    lv = book_levels(xf, 2)
    y = oracle.fwht(xf)
    codes = kvq.scalar_encode(cuda(y.astype(np.float32)), cuda(lv), 2, pre_rotated=True)
    xh = torch.from_numpy(inp["x_f32"]).half().cuda()
    codes_h = kvq.scalar_encode(xh, cuda(lv), 2)
    yh = oracle.fwht(xh.double().cpu().numpy())
    for c, yy in ((codes, y), (codes_h, yh)):
        c = c.cpu().numpy()
        for b in range(2):
            z = oracle.unpack_bits(c[b].reshape(-1, 2, 32), 2)
            res = oracle.check_scalar_codes(yy[b].reshape(-1, 128), lv[b, 0], lv[b, 1],
                                            z[:, 0], z[:, 1])
            assert res["hard"] == 0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_scalar_encode_every_instance(D, dt, bits):
    """Every (head size, input dtype, bits) instance of the scalar encode
    kernel on random rows (two books, one ragged row count): the oracle's
    code rule on every code."""
    say(f"scalar encode instance D {D} {dt} bits {bits}")
    rng = np.random.default_rng(7000 + D + bits + len(dt))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    x = torch.from_numpy(rng.standard_normal((2, 1, 301, D)).astype(np.float32)).to(tdt).cuda()
    xf = x.double().cpu().numpy()
    lv = book_levels(xf, bits)
    codes = kvq.scalar_encode(x, cuda(lv), bits).cpu().numpy()
    assert codes.shape == (2, 1, 301, 2, D * bits // 8)
    for b in range(2):
        z = oracle.unpack_bits(codes[b].reshape(-1, 2, codes.shape[-1]), bits)
        y = oracle.fwht(xf[b].reshape(-1, D))
        res = oracle.check_scalar_codes(y, lv[b, 0], lv[b, 1], z[:, 0], z[:, 1])
        assert res["hard"] == 0, (b, {k: res[k] for k in ("total", "exact", "near_tie", "hard")})


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_scalar_reconstruct_parity(bits, D):
    say(f"scalar reconstruct D {D} bits {bits}")
    rng = np.random.default_rng(D + bits)
    g, lap, dg = unit_levels(bits)
    lv = np.asarray([[g * 1.3, lap * 1.3 * np.sqrt(dg)], [g * 0.7, lap * 0.7 * np.sqrt(dg)]],
                    dtype=np.float32)
    codes = rng.integers(0, 256, size=(2, 777, 2, D * bits // 8), dtype=np.uint8)
    rot = kvq.scalar_decode_reconstruct(cuda(codes), cuda(lv), bits).cpu().numpy()
    unr = kvq.scalar_decode_reconstruct(cuda(codes), cuda(lv), bits, unrotate=True).cpu().numpy()
    for b in range(2):
        z = oracle.unpack_bits(codes[b], bits)
        ref = oracle.scalar_reconstruct(z[:, 0], z[:, 1], lv[b, 0], lv[b, 1], unrotate=False)
        assert np.array_equal(rot[b], ref.astype(np.float32))   # one rounding of the level sum
        ref_u = oracle.fwht(ref)
        assert np.all(np.abs(unr[b] - ref_u) <= 1e-6 * np.linalg.norm(ref, axis=1, keepdims=True))


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_scalar_product_codebook_exact(bits):
    say(f"scalar product codebook bits {bits}")
    g, lap, dg = unit_levels(bits)
    lv = np.asarray([g * 2.0, lap * 0.5], dtype=np.float32)
    cb = kvq.scalar_product_codebook(cuda(lv), bits, 128).cpu().numpy()
    ref = oracle.scalar_product_codebook(lv[0], lv[1], bits, 128).astype(np.float32)
    assert np.array_equal(cb, ref)


@pytest.mark.parametrize("key,over,bits", [
    (2, dict(tokens=3000, window=128), 1),      # 16 groups of 8 dims: rotated-code kernels
    (2, dict(tokens=3000, window=128), 2),      # 32 groups of 4 dims: rotated-code kernels
    (3, dict(batch=3, tokens=2100, window=64), 2),
    (1, dict(tokens=1500, window=0), 1),        # D = 64
    (2, dict(tokens=3000, window=128), 4),      # 64 groups of 2 dims: general kernel
    (3, dict(batch=2, tokens=1800, window=64), 4),
    (1, dict(tokens=1500, window=0), 4),        # D = 64, 32 groups of 2 dims
])
def test_scalar_decode_through_product_codebook(key, over, bits):
    say(f"scalar decode workload {key} {over} bits {bits}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc, D = w.code_tokens, w.head_dim
    x = to_dev(inp["x"], w)
    xf = inp["x_f32"][:, :, :Tc]
    lv = book_levels(xf, bits)
    codes = kvq.scalar_encode(x, cuda(lv), bits, n_rows=Tc)
    G = D * bits // 8
    kc = codes[0].reshape(w.batch, w.n_kv_heads, Tc, 2, G)
    vc = codes[1].reshape(w.batch, w.n_kv_heads, Tc, 2, G)
    kcb = kvq.scalar_product_codebook(cuda(lv[0]), bits, D)
    vcb = kvq.scalar_product_codebook(cuda(lv[1]), bits, D)
    W = w.window
    kwin = inp["k_win"] if W > 0 else None
    vwin = inp["v_win"] if W > 0 else None
    q = inp["q"] if w.n_q_heads > 0 else np.random.default_rng(3).standard_normal(
        (w.batch, 4, D)).astype(np.float32)
    got = kvq.attend_decode(cuda(q), kc.contiguous(), vc.contiguous(), kcb, vcb,
                            None if kwin is None else cuda(kwin),
                            None if vwin is None else cuda(vwin)).cpu().numpy()
    ref = oracle.attend_scalar(q, kc.cpu().numpy(), vc.cpu().numpy(), (lv[0, 0], lv[0, 1]),
                               (lv[1, 0], lv[1, 1]), bits, kwin, vwin)
    res = oracle.check_attn(got, ref)
    say("   ", res)
    assert res["ok"], res


def test_full_size_scalar_llama_layer():
    """The Llama-shaped layer at full size, 2 bits per stage: encode (sampled
    index check), decode through the product codebook against the oracle."""
    say("full-size Llama-shaped layer, scalar variant, 2 bits")
    w = synth.workload(2)
    inp = synth.make_inputs(w)
    Tc, D, bits = w.code_tokens, 128, 2
    x = to_dev(inp["x"], w)
    lv = book_levels(inp["x_f32"][:, :, :Tc], bits)
    codes = kvq.scalar_encode(x, cuda(lv), bits, n_rows=Tc)
    cn = codes.cpu().numpy()
    del x
    for b in range(2):
        flat = cn[b].reshape(-1, 2, 32)
        idx = np.arange(0, flat.shape[0], 97)
        z = oracle.unpack_bits(flat[idx], bits)
        y = oracle.fwht(inp["x_f32"][b][:, :Tc].reshape(-1, D)[idx].astype(np.float64))
        res = oracle.check_scalar_codes(y, lv[b, 0], lv[b, 1], z[:, 0], z[:, 1])
        say("   book", b, res)
        assert res["hard"] == 0
    kc = codes[0].reshape(1, 8, Tc, 2, 32)
    vc = codes[1].reshape(1, 8, Tc, 2, 32)
    got = kvq.attend_decode(cuda(inp["q"]), kc.contiguous(), vc.contiguous(),
                            kvq.scalar_product_codebook(cuda(lv[0]), bits, D),
                            kvq.scalar_product_codebook(cuda(lv[1]), bits, D),
                            cuda(inp["k_win"]), cuda(inp["v_win"])).cpu().numpy()
    ref = oracle.attend_scalar(inp["q"], cn[0].reshape(1, 8, Tc, 2, 32),
                               cn[1].reshape(1, 8, Tc, 2, 32), (lv[0, 0], lv[0, 1]),
                               (lv[1, 0], lv[1, 1]), bits, inp["k_win"], inp["v_win"])
    res = oracle.check_attn(got, ref)
    say("   decode", res)
    assert res["ok"], res
