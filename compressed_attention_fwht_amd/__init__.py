"""kvq -- rotated residual/product VQ of the KV cache and LUT decode attention
on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libkvq.so`` (C ABI in ``include/kvq.h``).  Every
step of the path runs in the library's HIP kernels; this module only turns
torch device tensors into pointers, sizes and the current HIP stream, and
raises :class:`KvqError` when the library reports a non-OK status.  The
library is loaded on first use (``lib``); if it has not been built that use
raises ImportError: there is no fallback path.

Calls (same names as the C ABI):
  rotate(x)                                  y = H_D x            [..., D] -> f32
  encode(x, codebooks, n_rows=...)           codes uint8 [books][seq][rows][S][G]
  decode_reconstruct(codes, codebooks)       sum of codewords     -> f32 [..., D]
  attend_decode(q, k_codes, v_codes, k_cb, v_cb, k_win, v_win) -> f32 [B][Hq][D]
  cache_bytes(B, Hq, Hkv, D, Tc, W, S, G, C) bytes a layer's compressed cache holds
  window_append / window_flush               streaming fp16 window -> codes
  smooth_calibrate(k, n_scale)               dual-transform factors f32 [books][n_scale][D]
  codebook_fit(x, init, n_iter)              K-means codebooks [S][G][C][dsub] f32 on a sample
  lloyd_max / scalar_encode / scalar_decode_reconstruct / scalar_product_codebook
                                             two-pass scalar residual variant, packed codes
  (encode, decode_reconstruct, attend_decode and window_flush take the factors
  as ``smooth=`` / ``k_smooth=`` and then call the *_smooth entry points)
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["KvqError", "LIB_PATH", "lib", "rotate", "encode", "encode_workspace_size",
           "decode_reconstruct", "attend_decode", "attend_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
           "attend_workspace_size", "cache_bytes",
           "window_append",
           "window_flush", "window_flush_workspace_size", "smooth_calibrate", "codebook_fit",
           "codebook_fit_workspace_size", "lloyd_max", "scalar_encode",
           "scalar_decode_reconstruct", "scalar_product_codebook", "EXPORTS",
           "KVQ_INPUT_PRE_ROTATED", "SmoothDesc",
           "KVQ_UNROTATE", "KVQ_ENCODE_GENERIC", "KVQ_CODEBOOKS_PACKED", "VqDesc", "AttnDesc",
           "status_string"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_INPUT_PRE_ROTATED = 0x1
KVQ_UNROTATE = 0x2
KVQ_ENCODE_GENERIC = 0x4
KVQ_CODEBOOKS_PACKED = 0x8
F32, BF16, F16 = 0, 1, 2

EXPORTS = ("kvq_rotate", "kvq_encode_workspace_size", "kvq_encode", "kvq_decode_reconstruct",
           "kvq_attend_workspace_size", "kvq_attend_decode", "kvq_attend_decode_noalloc",
           "kvq_cache_bytes",
           "kvq_window_append",
           "kvq_window_flush_workspace_size", "kvq_window_flush", "kvq_smooth_calibrate",
           "kvq_encode_smooth", "kvq_decode_reconstruct_smooth", "kvq_attend_decode_smooth",
           "kvq_window_flush_smooth", "kvq_codebook_fit_workspace_size", "kvq_codebook_fit",
           "kvq_lloyd_max", "kvq_scalar_encode", "kvq_scalar_decode_reconstruct",
           "kvq_scalar_product_codebook",
           "kvq_status_string", "kvq_last_hip_error")


class VqDesc(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("n_stages", ctypes.c_int32), ("n_codewords", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("n_code_tokens", ctypes.c_int32),
                ("n_window", ctypes.c_int32), ("vq", VqDesc), ("softmax_scale", ctypes.c_float),
                ("code_stride", ctypes.c_int32), ("window_stride", ctypes.c_int32)]


class SmoothDesc(ctypes.Structure):
    _fields_ = [("factors", ctypes.c_void_p), ("n_scale", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m compressed_attention_fwht_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    L.kvq_rotate.argtypes = [P, I32, P, I64, I32, P]
    L.kvq_encode_workspace_size.argtypes = [ctypes.POINTER(VqDesc), I64, ctypes.POINTER(SZ)]
    L.kvq_encode.argtypes = [P, I32, ctypes.POINTER(VqDesc), I64, I64, I64, I64, P, P, U32, P, SZ, P]
    L.kvq_decode_reconstruct.argtypes = [P, ctypes.POINTER(VqDesc), I64, I64, P, P, U32, P]
    L.kvq_attend_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)]
    L.kvq_attend_decode.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, SZ, P]
    L.kvq_attend_decode_noalloc.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P]
    U64P = ctypes.POINTER(ctypes.c_uint64)
    L.kvq_cache_bytes.argtypes = [ctypes.POINTER(AttnDesc), U64P, U64P, U64P, U64P]
    L.kvq_window_append.argtypes = [I32, I32, I32, I32, I32, P, P, P, P, P]
    L.kvq_window_flush_workspace_size.argtypes = [ctypes.POINTER(VqDesc), ctypes.POINTER(SZ)]
    L.kvq_window_flush.argtypes = [ctypes.POINTER(VqDesc), I32, I32, I32, I32, I32, P, P, I32, I32,
                                   P, P, P, P, U32, P, SZ, P]
    SD = ctypes.POINTER(SmoothDesc)
    L.kvq_smooth_calibrate.argtypes = [P, I32, I32, I64, I64, I64, I64, I32, P, P]
    L.kvq_encode_smooth.argtypes = [P, I32, ctypes.POINTER(VqDesc), I64, I64, I64, I64, SD, P, P,
                                    U32, P, SZ, P]
    L.kvq_decode_reconstruct_smooth.argtypes = [P, ctypes.POINTER(VqDesc), I64, I64, I64, P, SD,
                                                P, P]
    L.kvq_attend_decode_smooth.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, SD, P, P, P,
                                           P, SZ, P]
    L.kvq_window_flush_smooth.argtypes = [ctypes.POINTER(VqDesc), I32, I32, I32, I32, I32, P, P,
                                          I32, I32, P, P, P, P, SD, U32, P, SZ, P]
    L.kvq_codebook_fit_workspace_size.argtypes = [ctypes.POINTER(VqDesc), I64, ctypes.POINTER(SZ)]
    L.kvq_codebook_fit.argtypes = [P, I32, ctypes.POINTER(VqDesc), I64, I64, I64, SD, I32, P, P,
                                   SZ, P]
    DP = ctypes.POINTER(ctypes.c_double)
    L.kvq_lloyd_max.argtypes = [I32, I32, DP, DP]
    L.kvq_scalar_encode.argtypes = [P, I32, I32, I32, I64, I64, I64, I64, P, P, U32, P]
    L.kvq_scalar_decode_reconstruct.argtypes = [P, I32, I32, I64, I64, P, P, U32, P]
    L.kvq_scalar_product_codebook.argtypes = [I32, I32, P, P, P]
    L.kvq_status_string.argtypes = [I32]
    L.kvq_status_string.restype = ctypes.c_char_p
    L.kvq_last_hip_error.argtypes = []
    for name in EXPORTS:
        if name not in ("kvq_status_string",):
            getattr(L, name).restype = ctypes.c_int32 if name != "kvq_last_hip_error" else ctypes.c_int
    return L


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):          # module attribute ``lib`` loads the library
    if name == "lib":
        return _lib()
    raise AttributeError(name)


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib().kvq_status_string(status).decode()
        if status == 7:
            msg += f" (hipError {_lib().kvq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def status_string(status: int) -> str:
    return _lib().kvq_status_string(status).decode()


def _check(st: int, where: str):
    if st != 0:
        raise KvqError(st, where)


# --------------------------------------------------------------- torch glue
# The C ABI sees only pointers and the sizes in its descriptors, so every
# wrapper checks each tensor's dtype, shape, layout and device against those
# sizes before the call: a mismatch raises TypeError (dtype) or ValueError
# (shape, layout, device) and nothing is launched.
def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _need_contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, name, dtypes, shape=None, ndim=None):
    """t has one of ``dtypes`` (a torch dtype or a tuple of them), the given
    shape (None entries match anything) or number of dimensions, and is
    contiguous."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None:
        shape = tuple(shape)
        if t.dim() != len(shape) or any(e is not None and int(a) != int(e)
                                         for a, e in zip(t.shape, shape)):
            want = "[" + "][".join("*" if e is None else str(e) for e in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(ref, **ts):
    """Every tensor of ts (None skipped) is a GPU tensor on ref's device."""
    for name, t in ts.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {ref.device}")


def _workspace(ws, name="workspace"):
    if ws is not None:
        _expect(ws, name, _torch().uint8, ndim=1)


def _smooth_desc(factors, n_books, D):
    """SmoothDesc of a float32 factor tensor [n_books][n_scale][D] (or
    [n_scale][D] when n_books == 1)."""
    _need_contig(factors)
    if factors.dtype != _torch().float32:
        raise TypeError("smoothing factors must be float32")
    if factors.dim() == 2:
        factors = factors.unsqueeze(0)
    if factors.dim() != 3 or factors.shape[0] != n_books or factors.shape[2] != D:
        raise ValueError(f"smoothing factors must be [{n_books}][n_scale][{D}], got "
                         f"{tuple(factors.shape)}")
    return SmoothDesc(_ptr(factors), factors.shape[1])


def _dims(x, name, n):
    if x.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(x.shape)}")
    return x.shape


def smooth_calibrate(x, n_scale=1, *, n_rows=None, out=None):
    """Dual-transform factors of x [n_books][n_seq][seq_stride][D]
    (f32/bf16/f16): f[b][j][i] = sqrt(max |x[b][n][t][i]|) over sequences n
    with n % n_scale == j and rows t < n_rows (1 where the maximum is 0).
    Returns f32 [n_books][n_scale][D]."""
    torch = _torch()
    _dtype_code(x)
    _need_contig(x)
    nb, ns, stride, D = _dims(x, "x", 4)
    n_rows = stride if n_rows is None else n_rows
    if out is None:
        out = torch.empty((nb, n_scale, D), dtype=torch.float32, device=x.device)
    _expect(out, "out", torch.float32, (nb, n_scale, D))
    _same_device(x, x=x, out=out)
    _check(_lib().kvq_smooth_calibrate(_ptr(x), _dtype_code(x), D, nb, ns, stride, n_rows,
                                       int(n_scale), _ptr(out), _stream(x)),
           "kvq_smooth_calibrate")
    return out


def codebook_fit_workspace_size(head_dim, n_groups, n_stages, n_codewords, n_vectors) -> int:
    vq = VqDesc(head_dim, n_groups, n_stages, n_codewords)
    sz = ctypes.c_size_t(0)
    _check(_lib().kvq_codebook_fit_workspace_size(ctypes.byref(vq), n_vectors, ctypes.byref(sz)),
           "kvq_codebook_fit_workspace_size")
    return sz.value


def codebook_fit(x, init, n_iter, *, n_rows=None, smooth=None, workspace=None, inplace=False):
    """K-means (Lloyd) codebooks fitted on the sample x ([N][D] or
    [n_seq][seq_stride][D], f32/bf16/f16, rows [0, n_rows) of each sequence),
    stage by stage on the residuals, starting from init [S][G][C][dsub] f32.
    ``smooth``: f32 [n_scale][D] dual-transform factors (sequence n uses row
    n % n_scale).  Returns the fitted codebooks (init itself when
    ``inplace``)."""
    torch = _torch()
    _dtype_code(x)
    _need_contig(x)
    if x.dim() == 2:
        x = x.unsqueeze(0)
    ns, stride, D = _dims(x, "x", 3)
    n_rows = stride if n_rows is None else n_rows
    _expect(init, "init", torch.float32, ndim=4)
    S, G, C, dsub = init.shape
    if G * dsub != D:
        raise ValueError(f"init [S][G][C][dsub] must have G * dsub = D = {D}, got "
                         f"{tuple(init.shape)}")
    _workspace(workspace)
    _same_device(x, x=x, init=init, smooth=smooth, workspace=workspace)
    cb = init if inplace else init.clone()
    vq = VqDesc(D, G, S, C)
    need = codebook_fit_workspace_size(D, G, S, C, ns * n_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    sd = None if smooth is None else ctypes.byref(_smooth_desc(smooth, 1, D))
    _check(_lib().kvq_codebook_fit(_ptr(x), _dtype_code(x), ctypes.byref(vq), ns, stride, n_rows,
                                   sd, int(n_iter), _ptr(cb), _ptr(workspace), workspace.numel(),
                                   _stream(x)), "kvq_codebook_fit")
    return cb


KVQ_LEVELS_GAUSSIAN, KVQ_LEVELS_LAPLACIAN = 0, 1


def lloyd_max(kind, bits):
    """Levels (ascending, float64 list) and mean squared error of the
    Lloyd-Max quantiser with 2^bits levels for the unit-variance density
    ``kind`` ("gaussian" or "laplacian"); computed by the library on the host."""
    k = {"gaussian": KVQ_LEVELS_GAUSSIAN, "laplacian": KVQ_LEVELS_LAPLACIAN}[kind]
    lv = (ctypes.c_double * (1 << bits))()
    d = ctypes.c_double(0.0)
    _check(_lib().kvq_lloyd_max(k, bits, lv, ctypes.byref(d)), "kvq_lloyd_max")
    return list(lv), d.value


def _scalar_bits(bits, product=False):
    ok = (1, 2, 4) if product else (1, 2, 3, 4)
    if bits not in ok:
        raise ValueError(f"bits must be one of {ok}, got {bits}")


def scalar_encode(x, levels, bits, *, n_rows=None, pre_rotated=False, codes=None):
    """Two-pass scalar codes of rows [0, n_rows) of every sequence of x
    [n_books][n_seq][seq_stride][D] (f32/bf16/f16); levels f32
    [n_books][2][2^bits].  Returns u8 [n_books][n_seq][n_rows][2][D*bits/8]."""
    torch = _torch()
    _scalar_bits(bits)
    _dtype_code(x)
    _need_contig(x)
    nb, ns, stride, D = _dims(x, "x", 4)
    n_rows = stride if n_rows is None else n_rows
    _expect(levels, "levels", torch.float32, (nb, 2, 1 << bits))
    if codes is None:
        codes = torch.empty((nb, ns, n_rows, 2, D * bits // 8), dtype=torch.uint8,
                            device=x.device)
    _expect(codes, "codes", torch.uint8, (nb, ns, n_rows, 2, D * bits // 8))
    _same_device(x, x=x, levels=levels, codes=codes)
    _check(_lib().kvq_scalar_encode(_ptr(x), _dtype_code(x), D, bits, nb, ns, stride, n_rows,
                                    _ptr(levels), _ptr(codes),
                                    KVQ_INPUT_PRE_ROTATED if pre_rotated else 0, _stream(x)),
           "kvq_scalar_encode")
    return codes


def scalar_decode_reconstruct(codes, levels, bits, *, unrotate=False, out=None):
    """codes u8 [n_books][...][2][D*bits/8], levels f32 [n_books][2][2^bits] ->
    f32 [n_books][...][D]: levels1[z1] + levels2[z2] (then H_D if unrotate)."""
    torch = _torch()
    _scalar_bits(bits)
    _expect(codes, "codes", torch.uint8)
    if codes.dim() < 3 or codes.shape[-2] != 2:
        raise ValueError(f"codes must be [n_books][...][2][D*bits/8], got {tuple(codes.shape)}")
    nb = codes.shape[0]
    _expect(levels, "levels", torch.float32, (nb, 2, 1 << bits))
    D = codes.shape[-1] * 8 // bits
    per_book = codes.numel() // (nb * 2 * codes.shape[-1]) if codes.numel() else 0
    if out is None:
        out = torch.empty(codes.shape[:-2] + (D,), dtype=torch.float32, device=codes.device)
    _expect(out, "out", torch.float32, tuple(codes.shape[:-2]) + (D,))
    _same_device(codes, codes=codes, levels=levels, out=out)
    _check(_lib().kvq_scalar_decode_reconstruct(_ptr(codes), D, bits, nb, per_book, _ptr(levels),
                                                _ptr(out), KVQ_UNROTATE if unrotate else 0,
                                                _stream(codes)),
           "kvq_scalar_decode_reconstruct")
    return out


def scalar_product_codebook(levels, bits, head_dim, out=None):
    """The product codebook f32 [2][D*bits/8][256][8/bits] of one book's levels
    [2][2^bits]; with it kvq_attend_decode reads packed scalar codes."""
    torch = _torch()
    _scalar_bits(bits, product=True)
    _expect(levels, "levels", torch.float32, (2, 1 << bits))
    G, k = head_dim * bits // 8, 8 // bits
    if out is None:
        out = torch.empty((2, G, 256, k), dtype=torch.float32, device=levels.device)
    _expect(out, "out", torch.float32, (2, G, 256, k))
    _same_device(levels, levels=levels, out=out)
    _check(_lib().kvq_scalar_product_codebook(head_dim, bits, _ptr(levels), _ptr(out),
                                              _stream(levels)), "kvq_scalar_product_codebook")
    return out


def rotate(x, out=None):
    """y = H_D x over the last axis.  x: cuda tensor f32/bf16/f16 [..., D]."""
    torch = _torch()
    _dtype_code(x)
    _need_contig(x)
    if x.dim() < 1:
        raise ValueError("x must have a last (head) axis")
    D = x.shape[-1]
    n = x.numel() // D if D else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _expect(out, "out", torch.float32, tuple(x.shape))
    _same_device(x, x=x, out=out)
    _check(_lib().kvq_rotate(_ptr(x), _dtype_code(x), _ptr(out), n, D, _stream(x)), "kvq_rotate")
    return out


def encode_workspace_size(head_dim, n_groups, n_stages, n_codewords, n_books) -> int:
    vq = VqDesc(head_dim, n_groups, n_stages, n_codewords)
    sz = ctypes.c_size_t(0)
    _check(_lib().kvq_encode_workspace_size(ctypes.byref(vq), n_books, ctypes.byref(sz)),
           "kvq_encode_workspace_size")
    return sz.value


def encode(x, codebooks, *, n_rows=None, pre_rotated=False, generic=False, codes=None,
           workspace=None, packed=False, smooth=None):
    """Encode rows [0, n_rows) of every sequence.

    x: [n_books][n_seq][seq_stride][D] (f32/bf16/f16); codebooks:
    [n_books][S][G][C][dsub] f32.  Returns codes [n_books][n_seq][n_rows][S][G] u8.
    ``packed``: ``workspace`` already holds these codebooks packed by an
    earlier call (KVQ_CODEBOOKS_PACKED).  ``smooth``: dual-transform factors
    f32 [n_books][n_scale][D]; x is divided by them before the rotation
    (kvq_encode_smooth)."""
    torch = _torch()
    _dtype_code(x)
    _need_contig(x)
    nb, ns, stride, D = _dims(x, "x", 4)
    _expect(codebooks, "codebooks", torch.float32, ndim=5)
    _, S, G, C, dsub = codebooks.shape
    _expect(codebooks, "codebooks", torch.float32, (nb, S, G, C, D // G if G else 0))
    if G * dsub != D:
        raise ValueError(f"codebooks [n_books][S][G][C][dsub] must have G * dsub = D = {D}")
    n_rows = stride if n_rows is None else n_rows
    vq = VqDesc(D, G, S, C)
    if codes is None:
        codes = torch.empty((nb, ns, n_rows, S, G), dtype=torch.uint8, device=x.device)
    _expect(codes, "codes", torch.uint8, (nb, ns, n_rows, S, G))
    _workspace(workspace)
    _same_device(x, x=x, codebooks=codebooks, codes=codes, workspace=workspace, smooth=smooth)
    need = encode_workspace_size(D, G, S, C, nb)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if packed and workspace is None:
        raise ValueError("packed=True needs the workspace holding the packed codebooks")
    flags = ((KVQ_INPUT_PRE_ROTATED if pre_rotated else 0) | (KVQ_ENCODE_GENERIC if generic else 0)
             | (KVQ_CODEBOOKS_PACKED if packed else 0))
    ws_bytes = workspace.numel() if workspace is not None else 0
    if smooth is not None:
        sd = _smooth_desc(smooth, nb, D)
        _check(_lib().kvq_encode_smooth(_ptr(x), _dtype_code(x), ctypes.byref(vq), nb, ns, stride,
                                        n_rows, ctypes.byref(sd), _ptr(codebooks), _ptr(codes),
                                        flags, _ptr(workspace), ws_bytes, _stream(x)),
               "kvq_encode_smooth")
        return codes
    _check(_lib().kvq_encode(_ptr(x), _dtype_code(x), ctypes.byref(vq), nb, ns, stride, n_rows,
                          _ptr(codebooks), _ptr(codes), flags, _ptr(workspace), ws_bytes,
                          _stream(x)), "kvq_encode")
    return codes


def decode_reconstruct(codes, codebooks, *, unrotate=False, out=None, smooth=None):
    """codes [n_books][...][S][G] u8, codebooks [n_books][S][G][C][dsub] f32 ->
    f32 [n_books][...][D] (rotated domain unless ``unrotate``).  ``smooth``:
    the factors the codes' vectors were divided by (codes then
    [n_books][n_seq][n_rows][S][G]); the output is the original domain,
    factors times the unrotated sum (kvq_decode_reconstruct_smooth)."""
    torch = _torch()
    _expect(codebooks, "codebooks", torch.float32, ndim=5)
    nb, S, G, C, dsub = codebooks.shape
    D = G * dsub
    _expect(codes, "codes", torch.uint8)
    if codes.dim() < 3 or codes.shape[0] != nb or tuple(codes.shape[-2:]) != (S, G):
        raise ValueError(f"codes must be [{nb}][...][{S}][{G}], got {tuple(codes.shape)}")
    if smooth is not None:
        if codes.dim() != 5:
            raise ValueError("smooth=: codes must be [n_books][n_seq][n_rows][S][G]")
        _, ns, nr = codes.shape[:3]
        if out is None:
            out = torch.empty((nb, ns, nr, D), dtype=torch.float32, device=codes.device)
        _expect(out, "out", torch.float32, (nb, ns, nr, D))
        _same_device(codes, codes=codes, codebooks=codebooks, out=out, smooth=smooth)
        sd = _smooth_desc(smooth, nb, D)
        vq = VqDesc(D, G, S, C)
        _check(_lib().kvq_decode_reconstruct_smooth(_ptr(codes), ctypes.byref(vq), nb, ns, nr,
                                                    _ptr(codebooks), ctypes.byref(sd), _ptr(out),
                                                    _stream(codes)),
               "kvq_decode_reconstruct_smooth")
        return out
    per_book = codes.numel() // (nb * S * G) if codes.numel() else 0
    if out is None:
        out = torch.empty(codes.shape[:-2] + (D,), dtype=torch.float32, device=codes.device)
    _expect(out, "out", torch.float32, tuple(codes.shape[:-2]) + (D,))
    _same_device(codes, codes=codes, codebooks=codebooks, out=out)
    vq = VqDesc(D, G, S, C)
    _check(_lib().kvq_decode_reconstruct(_ptr(codes), ctypes.byref(vq), nb, per_book,
                                      _ptr(codebooks), _ptr(out),
                                      KVQ_UNROTATE if unrotate else 0, _stream(codes)),
           "kvq_decode_reconstruct")
    return out


def _attn_desc(B, Hq, Hkv, D, Tc, W, S, G, C, scale, code_stride=0, window_stride=0):
    return AttnDesc(B, Hq, Hkv, Tc, W, VqDesc(D, G, S, C), 0.0 if scale is None else float(scale),
                    code_stride, window_stride)


def attend_workspace_size(B, Hq, Hkv, D, Tc, W, S, G, C, scale=None) -> int:
    a = _attn_desc(B, Hq, Hkv, D, Tc, W, S, G, C, scale)
    sz = ctypes.c_size_t(0)
    _check(_lib().kvq_attend_workspace_size(ctypes.byref(a), ctypes.byref(sz)),
           "kvq_attend_workspace_size")
    return sz.value


def cache_bytes(B, Hq, Hkv, D, Tc, W, S, G, C) -> dict:
    """Bytes one layer's compressed cache holds (K and V): ``code``, ``window``
    (fp16), ``codebooks`` (float32) and ``dense`` (the same tokens as a dense
    fp16 cache), from kvq_cache_bytes (host arithmetic, no GPU)."""
    a = _attn_desc(B, Hq, Hkv, D, Tc, W, S, G, C, None)
    v = [ctypes.c_uint64(0) for _ in range(4)]
    _check(_lib().kvq_cache_bytes(ctypes.byref(a), *[ctypes.byref(x) for x in v]),
           "kvq_cache_bytes")
    return {"code": v[0].value, "window": v[1].value, "codebooks": v[2].value,
            "dense": v[3].value}


def _attend_args(q, k_codes, v_codes, k_cb, v_cb, k_win, v_win, out, scale, n_code, n_window):
    """Checks the decode call's tensors against each other and returns its
    descriptor: q [B][Hq][D] f32, k/v_codes [B][Hkv][Tcap][S][G] u8, k/v_cb
    [S][G][C][D/G] f32, k/v_win [B][Hkv][Wcap][D] f16 (both or neither),
    out [B][Hq][D] f32 (None: the caller allocates it)."""
    torch = _torch()
    _expect(q, "q", torch.float32, ndim=3)
    B, Hq, D = q.shape
    _expect(k_codes, "k_codes", torch.uint8, ndim=5)
    _, Hkv, Tcap, S, G = k_codes.shape
    _expect(k_codes, "k_codes", torch.uint8, (B, Hkv, Tcap, S, G))
    _expect(v_codes, "v_codes", torch.uint8, (B, Hkv, Tcap, S, G))
    if G <= 0 or D % G:
        raise ValueError(f"the code groups G = {G} must divide the head dimension D = {D}")
    _expect(k_cb, "k_cb", torch.float32, ndim=4)
    C = k_cb.shape[2]
    _expect(k_cb, "k_cb", torch.float32, (S, G, C, D // G))
    _expect(v_cb, "v_cb", torch.float32, (S, G, C, D // G))
    if (k_win is None) != (v_win is None):
        raise ValueError("k_win and v_win go together")
    Wcap = 0
    if k_win is not None:
        _expect(k_win, "k_win", torch.float16, ndim=4)
        Wcap = k_win.shape[2]
        _expect(k_win, "k_win", torch.float16, (B, Hkv, Wcap, D))
        _expect(v_win, "v_win", torch.float16, (B, Hkv, Wcap, D))
    if out is not None:
        _expect(out, "out", torch.float32, (B, Hq, D))
    _same_device(q, q=q, k_codes=k_codes, v_codes=v_codes, k_cb=k_cb, v_cb=v_cb, k_win=k_win,
                 v_win=v_win, out=out)
    Tc = Tcap if n_code is None else int(n_code)
    W = Wcap if n_window is None else int(n_window)
    return _attn_desc(B, Hq, Hkv, D, Tc, W, S, G, C, scale, Tcap, Wcap)


def attend_decode(q, k_codes, v_codes, k_cb, v_cb, k_win=None, v_win=None, *, scale=None,
                  out=None, workspace=None, n_code=None, n_window=None, k_smooth=None):
    """q [B][Hq][D] f32; k/v_codes [B][Hkv][Tcap][S][G] u8; k/v_cb [S][G][C][dsub]
    f32; k/v_win [B][Hkv][Wcap][D] f16 (or None).  Rows [0, n_code) of the
    codes and [0, n_window) of the window are attended (default: all rows).
    ``k_smooth``: f32 [n_scale][D] factors the coded keys were divided by
    (kvq_attend_decode_smooth).  Returns f32 [B][Hq][D]."""
    torch = _torch()
    _workspace(workspace)
    a = _attend_args(q, k_codes, v_codes, k_cb, v_cb, k_win, v_win, out, scale, n_code, n_window)
    _same_device(q, workspace=workspace, k_smooth=k_smooth)
    B, Hq, D = q.shape
    sz = ctypes.c_size_t(0)
    _check(_lib().kvq_attend_workspace_size(ctypes.byref(a), ctypes.byref(sz)),
           "kvq_attend_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(sz.value, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if k_smooth is not None:
        sd = _smooth_desc(k_smooth, 1, D)
        _check(_lib().kvq_attend_decode_smooth(ctypes.byref(a), _ptr(q), _ptr(k_codes),
                                               _ptr(v_codes), _ptr(k_cb), _ptr(v_cb),
                                               ctypes.byref(sd), _ptr(k_win), _ptr(v_win),
                                               _ptr(out), _ptr(workspace), workspace.numel(),
                                               _stream(q)),
               "kvq_attend_decode_smooth")
        return out
    _check(_lib().kvq_attend_decode(ctypes.byref(a), _ptr(q), _ptr(k_codes), _ptr(v_codes),
                                 _ptr(k_cb), _ptr(v_cb), _ptr(k_win), _ptr(v_win), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(q)),
           "kvq_attend_decode")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20      # KVQ_NOALLOC_SCRATCH_BYTES


def attend_decode_noalloc(q, k_codes, v_codes, k_cb, v_cb, k_win=None, v_win=None, *, out,
                          scale=None, n_code=None, n_window=None):
    """kvq_attend_decode_noalloc: attend_decode without a workspace (the
    library's per-GPU array of NOALLOC_SCRATCH_BYTES).  ``out`` [B][Hq][D] f32
    is required, so this call allocates nothing."""
    if out is None:
        raise ValueError("out is required")
    a = _attend_args(q, k_codes, v_codes, k_cb, v_cb, k_win, v_win, out, scale, n_code, n_window)
    _check(_lib().kvq_attend_decode_noalloc(ctypes.byref(a), _ptr(q), _ptr(k_codes),
                                            _ptr(v_codes), _ptr(k_cb), _ptr(v_cb), _ptr(k_win),
                                            _ptr(v_win), _ptr(out), _stream(q)),
           "kvq_attend_decode_noalloc")
    return out


def window_append(k_new, v_new, k_win, v_win, n_window):
    """Write one token per (sequence, KV head), k/v_new [B][Hkv][D] f16, into
    row n_window of the window buffers k/v_win [B][Hkv][Wcap][D] f16."""
    torch = _torch()
    _expect(k_win, "k_win", torch.float16, ndim=4)
    B, Hkv, Wcap, D = k_win.shape
    _expect(v_win, "v_win", torch.float16, (B, Hkv, Wcap, D))
    _expect(k_new, "k_new", torch.float16, (B, Hkv, D))
    _expect(v_new, "v_new", torch.float16, (B, Hkv, D))
    _same_device(k_win, k_new=k_new, v_new=v_new, k_win=k_win, v_win=v_win)
    _check(_lib().kvq_window_append(B, Hkv, D, Wcap, int(n_window), _ptr(k_new), _ptr(v_new),
                                    _ptr(k_win), _ptr(v_win), _stream(k_win)),
           "kvq_window_append")


def window_flush_workspace_size(head_dim, n_groups, n_stages, n_codewords) -> int:
    vq = VqDesc(head_dim, n_groups, n_stages, n_codewords)
    sz = ctypes.c_size_t(0)
    _check(_lib().kvq_window_flush_workspace_size(ctypes.byref(vq), ctypes.byref(sz)),
           "kvq_window_flush_workspace_size")
    return sz.value


def window_flush(k_win, v_win, n_window, n_flush, k_codes, v_codes, n_code, k_cb, v_cb, *,
                 workspace=None, packed=False, k_smooth=None):
    """Encode window rows [0, n_flush) into code rows [n_code, n_code + n_flush)
    (K with k_cb, V with v_cb), then move window rows [n_flush, n_window) to
    the front.  k/v_win [B][Hkv][Wcap][D] f16; k/v_codes [B][Hkv][Tcap][S][G] u8;
    k/v_cb [S][G][C][dsub] f32.  ``packed``: ``workspace`` still holds these
    codebooks packed by an earlier flush (KVQ_CODEBOOKS_PACKED).  ``k_smooth``:
    f32 [n_scale][D] factors the flushed keys are divided by
    (kvq_window_flush_smooth)."""
    torch = _torch()
    _expect(k_win, "k_win", torch.float16, ndim=4)
    B, Hkv, Wcap, D = k_win.shape
    _expect(v_win, "v_win", torch.float16, (B, Hkv, Wcap, D))
    _expect(k_codes, "k_codes", torch.uint8, ndim=5)
    Tcap, S, G = k_codes.shape[2:]
    _expect(k_codes, "k_codes", torch.uint8, (B, Hkv, Tcap, S, G))
    _expect(v_codes, "v_codes", torch.uint8, (B, Hkv, Tcap, S, G))
    if G <= 0 or D % G:
        raise ValueError(f"the code groups G = {G} must divide the head dimension D = {D}")
    _expect(k_cb, "k_cb", torch.float32, ndim=4)
    C = k_cb.shape[2]
    _expect(k_cb, "k_cb", torch.float32, (S, G, C, D // G))
    _expect(v_cb, "v_cb", torch.float32, (S, G, C, D // G))
    _workspace(workspace)
    _same_device(k_win, k_win=k_win, v_win=v_win, k_codes=k_codes, v_codes=v_codes, k_cb=k_cb,
                 v_cb=v_cb, workspace=workspace, k_smooth=k_smooth)
    vq = VqDesc(D, G, S, C)
    need = window_flush_workspace_size(D, G, S, C)
    if packed and workspace is None:
        raise ValueError("packed=True needs the workspace holding the packed codebooks")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_win.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    flags = KVQ_CODEBOOKS_PACKED if packed else 0
    if k_smooth is not None:
        sd = _smooth_desc(k_smooth, 1, D)
        _check(_lib().kvq_window_flush_smooth(ctypes.byref(vq), B, Hkv, Wcap, int(n_window),
                                              int(n_flush), _ptr(k_win), _ptr(v_win), Tcap,
                                              int(n_code), _ptr(k_codes), _ptr(v_codes),
                                              _ptr(k_cb), _ptr(v_cb), ctypes.byref(sd), flags,
                                              _ptr(workspace), ws_bytes, _stream(k_win)),
               "kvq_window_flush_smooth")
        return
    _check(_lib().kvq_window_flush(ctypes.byref(vq), B, Hkv, Wcap, int(n_window), int(n_flush),
                                   _ptr(k_win), _ptr(v_win), Tcap, int(n_code), _ptr(k_codes),
                                   _ptr(v_codes), _ptr(k_cb), _ptr(v_cb), flags, _ptr(workspace),
                                   ws_bytes, _stream(k_win)),
           "kvq_window_flush")
