"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments before touching the GPU.  CPU only: no call here reaches
a HIP API (every call below fails validation first, or is a pure host size
query)."""
import ctypes
import os
import re
import subprocess

import pytest

import compressed_attention_fwht_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, DTYPE = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"KVQ_API\s+[\w\s\*]+?\b(kvq_\w+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("kvq_rotate", "kvq_encode", "kvq_decode_reconstruct", "kvq_attend_decode"):
        assert n in names
    assert set(names) == set(kvq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = kvq.lib
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in _declared():
        assert n in exported, n
    # nothing else of ours leaks out of the shared object
    assert not [s for s in exported if "kvq" in s and not s.startswith("kvq_")]


def test_status_strings():
    for st in range(8):
        assert kvq.status_string(st)
    assert kvq.lib.kvq_last_hip_error() == 0


def _vq(D=128, G=16, S=2, C=256):
    return kvq.VqDesc(D, G, S, C)


def _enc(x=FAKE, xt=1, vq=None, nb=1, ns=1, stride=64, rows=64, cb=FAKE, codes=FAKE, flags=0,
         ws=FAKE, wsb=1 << 30):
    vq = _vq() if vq is None else vq
    return kvq.lib.kvq_encode(x, xt, ctypes.byref(vq), nb, ns, stride, rows, cb, codes, flags, ws,
                              wsb, None)


def test_encode_argument_errors():
    assert _enc(xt=9) == DTYPE
    assert _enc(x=0) == NULL
    assert _enc(codes=0) == NULL
    assert _enc(cb=0) == NULL
    assert _enc(x=FAKE + 4) == ALIGN
    assert _enc(codes=FAKE + 8) == ALIGN
    assert _enc(rows=65) == SHAPE                        # rows beyond the sequence stride
    assert _enc(nb=-1) == SHAPE
    assert _enc(flags=0x80) == SHAPE
    assert _enc(flags=0x10) == SHAPE
    assert _enc(flags=0x8, x=0) == NULL                   # KVQ_CODEBOOKS_PACKED is a known flag
    assert _enc(vq=_vq(D=96, G=12)) == SHAPE             # head_dim not 64/128/256
    assert _enc(vq=_vq(G=15)) == SHAPE                   # G does not divide D
    assert _enc(vq=_vq(G=32)) == SHAPE                   # dsub 4 < 8
    assert _enc(vq=_vq(S=0)) == SHAPE
    assert _enc(vq=_vq(S=9)) == SHAPE
    assert _enc(vq=_vq(C=257)) == SHAPE
    assert _enc(vq=_vq(C=0)) == SHAPE
    assert _enc(ws=0, wsb=0) == WS                       # MFMA path needs the packed books
    assert _enc(wsb=100) == WS
    assert _enc(ws=FAKE + 4) == ALIGN
    # zero-size work is a no-op that returns before any HIP call
    assert _enc(nb=0) == OK and _enc(ns=0) == OK and _enc(rows=0, x=0, cb=0, codes=0) == OK
    assert kvq.lib.kvq_encode(FAKE, 1, None, 1, 1, 1, 1, FAKE, FAKE, 0, FAKE, 1, None) == NULL


def test_encode_workspace_sizes():
    assert kvq.encode_workspace_size(128, 16, 2, 256, 64) == 64 * 16 * 2 * 20480
    assert kvq.encode_workspace_size(128, 16, 1, 256, 2) == 2 * 16 * 20480
    assert kvq.encode_workspace_size(64, 1, 2, 256, 2) == 0      # generic path, no workspace
    with pytest.raises(kvq.KvqError):
        kvq.encode_workspace_size(100, 4, 2, 256, 1)


def test_rotate_argument_errors():
    L = kvq.lib
    assert L.kvq_rotate(FAKE, 5, FAKE, 10, 128, None) == DTYPE
    assert L.kvq_rotate(FAKE, 1, FAKE, 10, 100, None) == SHAPE
    assert L.kvq_rotate(FAKE, 1, FAKE, -1, 128, None) == SHAPE
    assert L.kvq_rotate(0, 1, FAKE, 10, 128, None) == NULL
    assert L.kvq_rotate(FAKE, 1, FAKE + 2, 10, 128, None) == ALIGN
    assert L.kvq_rotate(FAKE, 1, FAKE, 10, 128, None) == SHAPE   # bf16 in place: overlap
    assert L.kvq_rotate(FAKE, 0, FAKE + 16, 10, 128, None) == SHAPE  # partial f32 overlap
    assert L.kvq_rotate(0, 1, 0, 0, 128, None) == OK               # no rows: no-op


def test_reconstruct_argument_errors():
    L = kvq.lib
    vq = _vq()
    assert L.kvq_decode_reconstruct(0, ctypes.byref(vq), 1, 10, FAKE, FAKE, 0, None) == NULL
    assert L.kvq_decode_reconstruct(FAKE, ctypes.byref(vq), 1, 10, FAKE, FAKE, 8, None) == SHAPE
    assert L.kvq_decode_reconstruct(FAKE + 1, ctypes.byref(vq), 1, 10, FAKE, FAKE, 0, None) == ALIGN
    assert L.kvq_decode_reconstruct(FAKE, ctypes.byref(_vq(S=0)), 1, 10, FAKE, FAKE, 0, None) == SHAPE
    assert L.kvq_decode_reconstruct(0, ctypes.byref(vq), 1, 0, 0, 0, 0, None) == OK


def _attn(B=1, Hq=32, Hkv=8, Tc=1000, W=16, S=1, G=16, C=256, D=128, scale=0.0):
    return kvq.AttnDesc(B, Hq, Hkv, Tc, W, kvq.VqDesc(D, G, S, C), scale)


def _att(a, q=FAKE, kc=FAKE, vc=FAKE, kcb=FAKE, vcb=FAKE, kw=FAKE, vw=FAKE, out=FAKE, ws=FAKE,
         wsb=1 << 34):
    return kvq.lib.kvq_attend_decode(ctypes.byref(a), q, kc, vc, kcb, vcb, kw, vw, out, ws, wsb, None)


def test_attend_argument_errors():
    assert _att(_attn(Hq=30)) == SHAPE                 # Hq not a multiple of Hkv
    assert _att(_attn(Tc=0, W=0)) == SHAPE
    assert _att(_attn(Tc=-1)) == SHAPE
    assert _att(_attn(B=0)) == SHAPE
    assert _att(_attn(scale=float("nan"))) == SHAPE
    assert _att(_attn(), q=0) == NULL
    assert _att(_attn(), kc=0) == NULL
    assert _att(_attn(), kw=0) == NULL
    assert _att(_attn(W=0), kw=0, vw=0, ws=0) == NULL
    assert _att(_attn(), out=FAKE + 4) == ALIGN
    assert _att(_attn(), wsb=10) == WS
    assert _att(_attn(D=256, S=8, G=32)) == UNSUP       # tables exceed LDS
    assert kvq.lib.kvq_attend_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                     None) == NULL


def test_attend_noalloc_argument_errors():
    """The no-allocation entry point runs the same checks as kvq_attend_decode
    and refuses a shape whose workspace exceeds its device array, all before any
    HIP call."""
    L = kvq.lib

    def na(a, q=FAKE, out=FAKE, kw=FAKE):
        return L.kvq_attend_decode_noalloc(ctypes.byref(a), q, FAKE, FAKE, FAKE, FAKE, kw, FAKE,
                                           out, None)
    assert L.kvq_attend_decode_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == NULL
    assert na(_attn(Hq=30)) == SHAPE
    assert na(_attn(), q=0) == NULL
    assert na(_attn(), kw=0) == NULL
    assert na(_attn(), out=FAKE + 4) == ALIGN
    assert na(_attn(D=256, S=8, G=32)) == UNSUP
    big = _attn(B=64, Hq=28, Hkv=4, Tc=8128, W=64, S=2)
    need = kvq.attend_workspace_size(64, 28, 4, 128, 8128, 64, 2, 16, 256)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    assert na(big) == WS
    # the decode workloads' shapes fit the array
    for (B, Hq, Hkv, Tc, W, S) in [(1, 32, 8, 32640, 128, 1), (16, 28, 4, 8128, 64, 2),
                                   (1, 32, 8, 130816, 256, 4)]:
        assert kvq.attend_workspace_size(B, Hq, Hkv, 128, Tc, W, S, 16, 256) \
            <= kvq.NOALLOC_SCRATCH_BYTES


def test_attend_workspace_sizes():
    # [LUT of B*Hq*S*G*C floats, when a separate pass builds it], then per
    # (b, h) one record of D + 4 floats per chunk and per window block
    sz = kvq.attend_workspace_size(1, 32, 8, 128, 32640, 128, 1, 16, 256)
    assert sz % (32 * 132 * 4) == 0 and 8 <= sz // (32 * 132 * 4) <= 64   # LUT built in blocks
    big = kvq.attend_workspace_size(1, 32, 8, 128, 130816, 256, 4, 16, 256)
    # long context: per (sequence, KV head, four query heads) a table of 4 stages
    # x 16 groups x 256 codewords x 4 heads of floats, then the V codebook in the
    # contraction's order, then 32 chunk records per head (the window rides on
    # the chunk blocks)
    lut = 8 * 64 * 256 * 4 * 4 + 4 * 16 * 256 * 8 * 4
    assert big == lut + 32 * 32 * 132 * 4
    sz_w = kvq.attend_workspace_size(2, 4, 2, 64, 0, 50, 2, 1, 256)   # window only
    assert sz_w == 2 * 4 * 1 * 68 * 4                                  # no LUT, one window block


def test_cache_bytes_match_the_closed_form_and_the_workload_tables():
    """kvq_cache_bytes: codes = tokens x the oracle's code bytes per vector
    (pinned there to the pages' 16x / 8x ratios), the window and codebooks in
    fp16 / float32, and the code and window byte counts of the decode workloads'
    table (Llama-, Qwen-shaped and long-context caches)."""
    import oracle
    for (B, Hq, Hkv, T, W, S, code, win) in [
            (1, 32, 8, 32768, 128, 1, 8_355_840, 524_288),
            (16, 28, 4, 8192, 64, 2, 33_292_288, 2_097_152),
            (1, 32, 8, 131072, 256, 4, 133_955_584, 1_048_576)]:
        r = kvq.cache_bytes(B, Hq, Hkv, 128, T - W, W, S, 16, 256)
        assert r["code"] == code and r["window"] == win
        assert r["code"] == 2 * B * Hkv * (T - W) * oracle.code_bytes_per_vector(S, 16)
        assert r["codebooks"] == 2 * S * 16 * 256 * 8 * 4
        assert r["dense"] == 2 * B * Hkv * T * 128 * 2
        # codes alone against the same tokens in fp16: the oracle's ratio
        assert r["dense"] * (T - W) / T / r["code"] == pytest.approx(
            oracle.compression_ratio_vs_fp16(128, S, 16))
    tiny = kvq.cache_bytes(1, 1, 1, 64, 1024, 0, 2, 1, 256)
    assert tiny == {"code": 4096, "window": 0, "codebooks": 2 * 2 * 256 * 64 * 4,
                    "dense": 2 * 1024 * 64 * 2}
    assert kvq.cache_bytes(2, 4, 2, 64, 0, 0, 1, 8, 256)["dense"] == 0   # empty cache


def test_cache_bytes_argument_errors():
    u = [ctypes.c_uint64(7) for _ in range(4)]
    refs = [ctypes.byref(x) for x in u]

    def call(a, *ptrs):
        return kvq.lib.kvq_cache_bytes(ctypes.byref(a), *(ptrs or refs))
    assert call(_attn(Hq=30)) == SHAPE
    assert call(_attn(Tc=-1)) == SHAPE
    assert call(_attn(B=0)) == SHAPE
    assert call(_attn(G=3)) == SHAPE
    assert call(_attn(B=1 << 30, Hkv=1 << 30, Hq=1 << 30, Tc=1 << 30)) == SHAPE   # past 2^63
    assert call(_attn(), refs[0], None, refs[2], refs[3]) == NULL
    assert kvq.lib.kvq_cache_bytes(None, *refs) == NULL
    assert [x.value for x in u] == [7, 7, 7, 7]          # nothing written on error
    with pytest.raises(kvq.KvqError):
        kvq.cache_bytes(1, 30, 8, 128, 10, 0, 1, 16, 256)


def test_window_append_argument_errors():
    L = kvq.lib
    assert L.kvq_window_append(1, 2, 100, 8, 0, FAKE, FAKE, FAKE, FAKE, None) == SHAPE   # head_dim
    assert L.kvq_window_append(1, 2, 128, 8, 8, FAKE, FAKE, FAKE, FAKE, None) == SHAPE   # full
    assert L.kvq_window_append(1, 2, 128, 8, -1, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.kvq_window_append(0, 2, 128, 8, 0, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.kvq_window_append(1, 2, 128, 8, 0, 0, FAKE, FAKE, FAKE, None) == NULL
    assert L.kvq_window_append(1, 2, 128, 8, 0, FAKE, FAKE, FAKE + 8, FAKE, None) == ALIGN


def _flush(vq=None, B=1, H=2, wcap=32, nw=32, nf=16, ccap=100, nc=0, kw=FAKE, ws=FAKE,
           wsb=1 << 30, flags=0):
    vq = _vq() if vq is None else vq
    return kvq.lib.kvq_window_flush(ctypes.byref(vq), B, H, wcap, nw, nf, kw, FAKE, ccap, nc, FAKE,
                                    FAKE, FAKE, FAKE, flags, ws, wsb, None)


def test_window_flush_argument_errors():
    assert _flush(nf=33) == SHAPE                       # more than the window holds
    assert _flush(nw=33) == SHAPE                       # more than its capacity
    assert _flush(nc=90) == SHAPE                       # codes past their capacity
    assert _flush(vq=_vq(D=96, G=12)) == SHAPE
    assert _flush(B=0) == SHAPE
    assert _flush(kw=0) == NULL
    assert _flush(kw=FAKE + 2) == ALIGN
    assert _flush(ws=0, wsb=0) == WS                    # MFMA path needs packed books
    assert _flush(nf=0, kw=0, ws=0, wsb=0) == OK        # nothing to flush: no-op
    assert _flush(flags=0x1) == SHAPE                   # only KVQ_CODEBOOKS_PACKED is known
    assert _flush(flags=0x8, kw=0) == NULL
    assert kvq.window_flush_workspace_size(128, 16, 2, 256) == 2 * 16 * 2 * 20480
    assert kvq.window_flush_workspace_size(64, 1, 2, 256) == 0   # generic kernel


def _sd(f=FAKE, n=8):
    return kvq.SmoothDesc(f, n)


def test_smooth_calibrate_argument_errors():
    L = kvq.lib
    cal = lambda x=FAKE, xt=1, D=128, nb=1, ns=8, st=64, nr=64, nsc=8, f=FAKE: \
        L.kvq_smooth_calibrate(x, xt, D, nb, ns, st, nr, nsc, f, None)
    assert cal(xt=7) == DTYPE
    assert cal(D=96) == SHAPE
    assert cal(nsc=0) == SHAPE
    assert cal(nr=65) == SHAPE                           # rows beyond the stride
    assert cal(nb=-1) == SHAPE
    assert cal(nb=0, f=0) == OK                          # nothing to write
    assert cal(f=0) == NULL
    assert cal(x=0) == NULL
    assert cal(f=FAKE + 4) == ALIGN
    assert cal(x=FAKE + 2) == ALIGN
    assert cal(f=FAKE + 64 * 128) == SHAPE               # output inside the input


def test_encode_smooth_argument_errors():
    L = kvq.lib
    vq = _vq()
    enc = lambda sd, flags=0, x=FAKE: L.kvq_encode_smooth(x, 1, ctypes.byref(vq), 1, 1, 64, 64, sd,
                                                          FAKE, FAKE, flags, FAKE, 1 << 30, None)
    assert enc(None) == NULL
    assert enc(ctypes.byref(_sd(f=0))) == NULL
    assert enc(ctypes.byref(_sd(n=0))) == SHAPE
    assert enc(ctypes.byref(_sd(f=FAKE + 4))) == ALIGN
    assert enc(ctypes.byref(_sd()), flags=0x1) == UNSUP   # division needs the original channels
    assert enc(ctypes.byref(_sd()), x=0) == NULL


def test_reconstruct_attend_flush_smooth_argument_errors():
    L = kvq.lib
    vq = _vq()
    rec = lambda sd, nr=64, out=FAKE: L.kvq_decode_reconstruct_smooth(
        FAKE, ctypes.byref(vq), 1, 2, nr, FAKE, sd, out, None)
    assert rec(None) == NULL
    assert rec(ctypes.byref(_sd(n=-1))) == SHAPE
    assert rec(ctypes.byref(_sd()), nr=-1) == SHAPE
    assert rec(ctypes.byref(_sd()), out=0) == NULL
    assert rec(ctypes.byref(_sd()), nr=0, out=0) == OK      # empty: no-op
    a = kvq.AttnDesc(1, 32, 8, 1024, 16, _vq(), 0.0, 0, 0)
    att = lambda sd: L.kvq_attend_decode_smooth(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, sd,
                                                FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert att(None) == NULL
    assert att(ctypes.byref(_sd(f=FAKE + 8))) == ALIGN
    fl = lambda sd: L.kvq_window_flush_smooth(ctypes.byref(vq), 1, 2, 32, 32, 16, FAKE, FAKE, 100,
                                              0, FAKE, FAKE, FAKE, FAKE, sd, 0, FAKE, 1 << 30, None)
    assert fl(None) == NULL
    assert fl(ctypes.byref(_sd(n=0))) == SHAPE


def test_codebook_fit_argument_errors():
    L = kvq.lib
    vq = _vq()
    sz = ctypes.c_size_t(0)
    assert L.kvq_codebook_fit_workspace_size(ctypes.byref(vq), 1 << 25, ctypes.byref(sz)) == SHAPE
    assert L.kvq_codebook_fit_workspace_size(ctypes.byref(vq), 1000, None) == NULL
    assert L.kvq_codebook_fit_workspace_size(ctypes.byref(vq), 1000, ctypes.byref(sz)) == OK
    assert sz.value >= 1000 * (4 * 128 + 2 * 16)
    fit = lambda x=FAKE, xt=1, ns=4, st=64, nr=64, sd=None, it=3, cb=FAKE, ws=FAKE, wsb=1 << 30: \
        L.kvq_codebook_fit(x, xt, ctypes.byref(vq), ns, st, nr, sd, it, cb, ws, wsb, None)
    assert fit(xt=5) == DTYPE
    assert fit(nr=65) == SHAPE
    assert fit(it=-1) == SHAPE
    assert fit(ns=1 << 20, nr=64) == SHAPE               # more than 2^24 vectors
    assert fit(cb=0) == NULL
    assert fit(ws=0) == NULL
    assert fit(x=FAKE + 2) == ALIGN
    assert fit(wsb=1000) == WS
    assert fit(sd=ctypes.byref(_sd(n=0))) == SHAPE
    assert fit(ns=0, x=0, cb=0, ws=0) == OK               # empty sample: no-op


def test_lloyd_max_host_call_matches_the_oracle():
    """kvq_lloyd_max runs on the host (no GPU): its closed-form moments agree
    with the oracle's quadrature."""
    import oracle
    for kind in ("gaussian", "laplacian"):
        for bits in (1, 2, 3, 4):
            lv, d = kvq.lloyd_max(kind, bits)
            ref = oracle.lloyd_max_levels(kind, bits)
            assert max(abs(a - b) for a, b in zip(lv, ref)) < 1e-9, (kind, bits)
            assert abs(d - oracle.lloyd_max_distortion(kind, ref)) < 1e-9
    L = kvq.lib
    buf = (ctypes.c_double * 16)()
    assert L.kvq_lloyd_max(2, 2, buf, None) == SHAPE
    assert L.kvq_lloyd_max(0, 5, buf, None) == SHAPE
    assert L.kvq_lloyd_max(0, 2, None, None) == NULL


def test_scalar_argument_errors():
    L = kvq.lib
    enc = lambda x=FAKE, xt=1, D=128, b=2, nb=1, ns=2, st=64, nr=64, lv=FAKE, c=FAKE, fl=0: \
        L.kvq_scalar_encode(x, xt, D, b, nb, ns, st, nr, lv, c, fl, None)
    assert enc(xt=4) == DTYPE
    assert enc(D=96) == SHAPE
    assert enc(b=5) == SHAPE                           # packing covers 1..4 bits
    assert enc(b=0) == SHAPE
    assert enc(nr=65) == SHAPE
    assert enc(fl=0x2) == SHAPE
    assert enc(lv=0) == NULL
    assert enc(c=FAKE + 1) == ALIGN
    assert enc(ns=0, x=0, lv=0, c=0) == OK
    rec = lambda b=2, nb=1, n=10, lv=FAKE, o=FAKE, fl=0: \
        L.kvq_scalar_decode_reconstruct(FAKE, 128, b, nb, n, lv, o, fl, None)
    assert rec(b=8) == SHAPE
    assert rec(fl=0x1) == SHAPE
    assert rec(o=0) == NULL
    assert rec(n=0, o=0) == OK
    assert L.kvq_scalar_product_codebook(128, 3, FAKE, FAKE, None) == SHAPE
    assert L.kvq_scalar_product_codebook(128, 2, FAKE, 0, None) == NULL
    # decode attention accepts 4-dim groups (2-bit scalar codes) and 2-dim ones
    # (4-bit codes: one head per block, the 128-group table fills the LDS), not 1-dim
    sz = ctypes.c_size_t(0)
    a4 = kvq.AttnDesc(1, 4, 1, 100, 0, kvq.VqDesc(128, 32, 2, 256), 0.0, 0, 0)
    assert L.kvq_attend_workspace_size(ctypes.byref(a4), ctypes.byref(sz)) == OK
    a2 = kvq.AttnDesc(1, 4, 1, 100, 0, kvq.VqDesc(128, 64, 2, 256), 0.0, 0, 0)
    assert L.kvq_attend_workspace_size(ctypes.byref(a2), ctypes.byref(sz)) == OK
    a1 = kvq.AttnDesc(1, 4, 1, 100, 0, kvq.VqDesc(128, 128, 2, 256), 0.0, 0, 0)
    assert L.kvq_attend_workspace_size(ctypes.byref(a1), ctypes.byref(sz)) == SHAPE
    # 2-dim groups of a 256-dim head need a 256 KiB table: no kernel
    a3 = kvq.AttnDesc(1, 4, 1, 100, 0, kvq.VqDesc(256, 128, 2, 256), 0.0, 0, 0)
    assert L.kvq_attend_workspace_size(ctypes.byref(a3), ctypes.byref(sz)) == UNSUP
    # the encode still needs 8 dims per group
    vq4 = kvq.VqDesc(128, 32, 2, 256)
    assert L.kvq_encode(FAKE, 1, ctypes.byref(vq4), 1, 1, 64, 64, FAKE, FAKE, 0, FAKE, 1 << 30,
                        None) == SHAPE
