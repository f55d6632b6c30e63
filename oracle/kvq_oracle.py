"""CPU oracle for rotated residual/product VQ of the KV cache and LUT decode
attention -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import, call or execute anything in this package.  It shares no code
with the HIP library: it imports NumPy and nothing else from this
repository.

Everything here is float64 NumPy written as the plain definition of each step,
in the order the pages give, with no blocking or fusion beyond what the
definition states.  A block loop over vectors is used only to bound memory.

Sources (page title -- section):
  [ZK]   "ZeroKV-Neo 4.0.0" (PyPI project page) -- Architecture: the FWHT
         "energy spreading" step before quantisation; the FP16 hot tier.
  [VQKV] "VQKV: High-Fidelity and High-Ratio Cache Compression via
         Vector-Quantization" (gist.science summary) -- 2. Methodology,
         Residual Simple Vector Quantization (RSimVQ): nearest entry in the
         first codebook, residual, next codebook, N stages; reconstruction as
         the sum of retrieved entries; 3. Inference Integration: codes stored
         at prefill, local sliding window of recent tokens kept uncompressed.
  [VI]   "VeloxQuant-MLX 0.5.1" (PyPI project page) -- VecInfer section:
         product VQ after a Walsh-Hadamard rotation with one codebook per
         sub-vector, inverse transform absorbed into the query; Architecture:
         the residual pipeline decodes by summing stage outputs then
         unrotating.
  [DKV]  "Differential-KV" README -- Decode & Prefill Innovations: scoring the
         query in the compressed domain without materialising K; merging with
         the dense recency window by an fp32 log-sum-exp combine.
  Streaming window: [VI] Quick start (a cache grown one token at a time by
         append, read by attend); [ZK] profiling output (periodic
         flush_quantize calls); [VQKV] 3. Inference Integration (recent tokens
         uncompressed in a local window, older ones compressed).
  Dual transform: [VI] VecInfer section (each key channel divided by the
         square root of its largest magnitude before the Walsh-Hadamard
         rotation; the inverse folded into the query so the scores are
         unchanged).
  Codebook fitting: [VI] VecInfer section (codebooks are K-means codebooks
         trained beforehand; the allocator list names train_codebook);
         [VQKV] 2. Methodology (the residual codebooks are trained).
  Scalar residual variant: [VI] Architecture, TurboQuantRVQ pipeline (rotate,
         stage-1 Gaussian Lloyd-Max scalar quantiser, residual, stage-2
         Laplacian Lloyd-Max, indices only, decode by summing then
         unrotating); module table (turboquant_rvq, Lloyd-Max codebooks,
         dsa.bit_pack sub-byte index packing); throughput journey
         (boundary-sum quantise in place of the argmin, same indices).

Parity status of each function is stated in its docstring; every function is
pinned by ``tests/test_oracle_pins.py`` against closed forms, library routines
or brute force.
"""
from __future__ import annotations

import numpy as np

__all__ = ["hadamard_matrix", "fwht", "nearest", "rvq_encode", "reconstruct_rot",
           "reconstruct", "attend", "attend_dense", "lse_merge", "window_append",
           "window_flush", "smooth_factors", "smooth_keys", "smooth_query", "smooth_encode",
           "reconstruct_smooth", "smooth_rows", "lloyd_update", "fit_codebooks",
           "lloyd_max_levels", "lloyd_max_distortion", "scalar_nearest", "boundary_sum",
           "scalar_rvq_encode", "pack_bits", "unpack_bits", "scalar_reconstruct",
           "scalar_product_codebook", "attend_scalar",
           "code_bytes_per_vector",
           "compression_ratio_vs_fp16"]


# ----------------------------------------------------------------------------
# O1 -- Walsh-Hadamard rotation  [ZK Architecture "FWHT (energy spreading)"],
#       [VI VecInfer "Walsh-Hadamard rotation"]
# ----------------------------------------------------------------------------
def hadamard_matrix(n: int) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order n (a power of two),
    natural order: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]], divided by
    sqrt(n).  No random sign flips (none is stated for this path)."""
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Hadamard order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(float(n))


def fwht(x: np.ndarray) -> np.ndarray:
    """y = H_D x for every row (last axis), as a dense product with the
    matrix above (deliberately not a butterfly, so it is checkable by eye).
    H is symmetric and orthonormal, hence self-inverse."""
    x = np.asarray(x, dtype=np.float64)
    return x @ hadamard_matrix(x.shape[-1])


# ----------------------------------------------------------------------------
# O2 -- greedy residual VQ per group  [VQKV 2. Methodology, RSimVQ steps 1-4],
#       product split into groups with one codebook each  [VI VecInfer]
# ----------------------------------------------------------------------------
def nearest(r: np.ndarray, cb: np.ndarray):
    """Nearest codeword by squared Euclidean distance, all candidates.

    r: [N][dsub], cb: [C][dsub].  Returns (z, d) with d[n][c] = sum_j
    (r[n][j] - cb[c][j])^2 in float64 and z = first index of the minimum
    (exact ties go to the lowest index)."""
    r = np.asarray(r, dtype=np.float64)
    cb = np.asarray(cb, dtype=np.float64)
    diff = r[:, None, :] - cb[None, :, :]
    d = np.einsum("ncj,ncj->nc", diff, diff)
    return np.argmin(d, axis=1), d


def rvq_encode(x: np.ndarray, codebooks: np.ndarray, *, rotate: bool = True,
               block: int = 4096, with_stats: bool = False):
    """Encode vectors into uint8 codes.

    x: [N][D]; codebooks: [S][G][C][dsub] with G*dsub = D, C <= 256.
    Steps for each vector [VQKV RSimVQ]:
      y = H_D x (unless ``rotate`` is False: input already rotated);
      for each group g independently, r = y[g*dsub:(g+1)*dsub];
      for s = 0..S-1: z_s = nearest entry of codebook (s, g) to r;
                      r <- r - codebook(s, g)[z_s].
    Returns codes [N][S][G] uint8 and, with ``with_stats``, a dict with the
    best distance d1, the second-best d2 and the residual energy |r|^2 after
    each stage, all [N][S][G] float64.
    """
    S, G, C, dsub = codebooks.shape
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape
    if G * dsub != D or C > 256:
        raise ValueError("codebook shape does not match the vectors")
    codes = np.empty((N, S, G), dtype=np.uint8)
    d1 = np.empty((N, S, G)); d2 = np.empty((N, S, G)); res = np.empty((N, S, G))
    cb = np.asarray(codebooks, dtype=np.float64)
    for lo in range(0, N, block):
        hi = min(N, lo + block)
        y = fwht(x[lo:hi]) if rotate else x[lo:hi]
        for g in range(G):
            r = y[:, g * dsub:(g + 1) * dsub].copy()
            for s in range(S):
                z, d = nearest(r, cb[s, g])
                codes[lo:hi, s, g] = z
                if with_stats:
                    part = np.partition(d, 1, axis=1) if C > 1 else np.concatenate([d, d], 1)
                    d1[lo:hi, s, g] = part[:, 0]
                    d2[lo:hi, s, g] = part[:, 1]
                r = r - cb[s, g][z]
                if with_stats:
                    res[lo:hi, s, g] = np.einsum("nj,nj->n", r, r)
    if with_stats:
        return codes, {"d1": d1, "d2": d2, "resid2": res}
    return codes


# ----------------------------------------------------------------------------
# O3 -- reconstruction as the sum of retrieved entries  [VQKV RSimVQ
#       "Reconstruction"], decode then unrotate  [VI Architecture, residual
#       pipeline decode]
# ----------------------------------------------------------------------------
def reconstruct_rot(codes: np.ndarray, codebooks: np.ndarray) -> np.ndarray:
    """x_hat_rot[g*dsub:(g+1)*dsub] = sum_s codebook(s, g)[z_s], float64,
    in the rotated domain.  codes [..., S, G] -> [..., D]."""
    S, G, C, dsub = codebooks.shape
    codes = np.asarray(codes)
    cb = np.asarray(codebooks, dtype=np.float64)
    out = np.zeros(codes.shape[:-2] + (G * dsub,), dtype=np.float64)
    for g in range(G):
        for s in range(S):
            out[..., g * dsub:(g + 1) * dsub] += cb[s, g][codes[..., s, g]]
    return out


def reconstruct(codes: np.ndarray, codebooks: np.ndarray) -> np.ndarray:
    """Reconstruction in the original domain: H_D applied to the rotated sum
    (H is its own inverse)."""
    return fwht(reconstruct_rot(codes, codebooks))


# ----------------------------------------------------------------------------
# O4 -- single-token decode attention over the coded cache plus the fp16
#       recency window  [VQKV 3. Inference Integration (decode; local window)],
#       [DKV Decode & Prefill Innovations], [VI VecInfer: q~ . K~^T = q . K^T]
# ----------------------------------------------------------------------------
def attend_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Textbook softmax attention of one query row per head.

    q: [Hq][D]; k, v: [Hkv][T][D]; query head h reads KV head h // (Hq/Hkv).
    o[h] = softmax(scale * K q[h]) V, in float64."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    Hkv = k.shape[0]
    rep = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kk = np.asarray(k[h // rep], dtype=np.float64)
        vv = np.asarray(v[h // rep], dtype=np.float64)
        s = (kk @ q[h]) * scale
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ vv
    return out


def attend(q, k_codes, v_codes, k_cb, v_cb, k_win=None, v_win=None, scale=None,
           k_smooth=None):
    """Decode attention for a batch.

    q: [B][Hq][D] (original domain); k_codes, v_codes: [B][Hkv][Tc][S][G];
    k_cb, v_cb: [S][G][C][dsub]; k_win, v_win: fp16 [B][Hkv][W][D] or None.
    Keys/values of the coded part are the reconstructions H (sum of entries);
    the window tokens follow them on the same axis.  scale defaults to
    1/sqrt(D).  k_smooth: smoothing factors [n_scale][D] the coded keys were
    divided by before encoding (dual transform); the coded keys are then
    reconstruct_smooth of their codes, KV head kv of sequence b using row
    (b * Hkv + kv) % n_scale.  The window keeps the original keys.  Returns
    float64 [B][Hq][D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        parts_k, parts_v = [], []
        if k_codes is not None and k_codes.shape[2] > 0:
            kk = reconstruct(k_codes[b], k_cb)
            if k_smooth is not None:
                Hkv = kk.shape[0]
                kk = kk * smooth_rows(k_smooth, b * Hkv + np.arange(Hkv))[:, None, :]
            parts_k.append(kk)
            parts_v.append(reconstruct(v_codes[b], v_cb))
        if k_win is not None and k_win.shape[2] > 0:
            parts_k.append(np.asarray(k_win[b], dtype=np.float64))
            parts_v.append(np.asarray(v_win[b], dtype=np.float64))
        k = np.concatenate(parts_k, axis=1)
        v = np.concatenate(parts_v, axis=1)
        out[b] = attend_dense(q[b], k, v, scale)
    return out


# ----------------------------------------------------------------------------
# Streaming window  [VI Quick start append/attend], [ZK flush_quantize],
#                   [VQKV 3. local window]
# ----------------------------------------------------------------------------
def window_append(k_win, v_win, n_window, k_new, v_new):
    """Returns copies of the window buffers [B][Hkv][Wcap][D] fp16 with the
    tokens k_new, v_new [B][Hkv][D] written at row n_window (n_window < Wcap).
    """
    k_win = np.array(k_win, copy=True)
    v_win = np.array(v_win, copy=True)
    if not 0 <= n_window < k_win.shape[2]:
        raise ValueError("window is full")
    k_win[:, :, n_window] = k_new
    v_win[:, :, n_window] = v_new
    return k_win, v_win


def window_flush(k_win, v_win, n_window, n_flush, k_codes, v_codes, n_code, k_cb, v_cb,
                 k_smooth=None):
    """The oldest n_flush window tokens (rows [0, n_flush) of every
    (sequence, KV head)) become codes at rows [n_code, n_code + n_flush) --
    rvq_encode of the fp16 values, K with k_cb, V with v_cb; with k_smooth
    ([n_scale][D]) the keys of (sequence b, KV head kv) are smooth_encode'd
    with row (b * Hkv + kv) % n_scale -- and the rows [n_flush, n_window)
    that stay uncompressed move to the front.  Buffers: windows
    [B][Hkv][Wcap][D] fp16, codes [B][Hkv][Tcap][S][G] uint8.  Returns new
    (k_win, v_win, k_codes, v_codes); rows past the new counts keep what they
    held."""
    if not 0 <= n_flush <= n_window <= k_win.shape[2]:
        raise ValueError("bad window counts")
    if n_code + n_flush > k_codes.shape[2]:
        raise ValueError("code buffer too small")
    k_win, v_win = np.array(k_win, copy=True), np.array(v_win, copy=True)
    k_codes, v_codes = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    B, H, _, D = k_win.shape
    S, G = k_codes.shape[3], k_codes.shape[4]
    for win, codes, cb, sm in ((k_win, k_codes, k_cb, k_smooth), (v_win, v_codes, v_cb, None)):
        x = win[:, :, :n_flush].astype(np.float64)
        if sm is None:
            z = rvq_encode(x.reshape(-1, D), cb)
        else:
            lam = smooth_rows(sm, np.arange(B * H)).reshape(B, H, 1, D)
            z = smooth_encode(x, np.broadcast_to(lam, x.shape), cb)
        codes[:, :, n_code:n_code + n_flush] = z.reshape(B, H, n_flush, S, G)
        keep = win[:, :, n_flush:n_window].copy()
        win[:, :, :n_window - n_flush] = keep
    return k_win, v_win, k_codes, v_codes


# ----------------------------------------------------------------------------
# Dual transform  [VI VecInfer: per-channel smooth scaling lambda_i =
#       sqrt(max |K_i|) followed by the Walsh-Hadamard rotation; the inverse
#       transform is absorbed into the queries]
# ----------------------------------------------------------------------------
def smooth_factors(k, n_scale: int = 1) -> np.ndarray:
    """Smoothing factors of keys k [n_seq][T][D] (original domain).

    lam[j][i] = sqrt(max |k[n][t][i]|) over every token t of every sequence n
    with n % n_scale == j.  A channel whose maximum is 0 -- or a row j that no
    sequence maps to -- gets 1: any positive factor leaves an all-zero channel
    at zero, and 1 leaves the query untouched too.  Returns float64
    [n_scale][D]."""
    k = np.abs(np.asarray(k, dtype=np.float64))
    n_seq, _, D = k.shape
    lam = np.ones((n_scale, D), dtype=np.float64)
    for j in range(n_scale):
        rows = k[j::n_scale].reshape(-1, D)
        if rows.shape[0] == 0:
            continue
        m = rows.max(axis=0)
        lam[j] = np.where(m > 0.0, np.sqrt(m), 1.0)
    return lam


def smooth_rows(lam, seq_index) -> np.ndarray:
    """The factor rows that sequences seq_index use: lam[n % n_scale]."""
    lam = np.asarray(lam, dtype=np.float64)
    return lam[np.asarray(seq_index) % lam.shape[0]]


def smooth_keys(k, lam) -> np.ndarray:
    """Keys with every channel divided by its factor (lam broadcasts over
    the leading axes of k)."""
    return np.asarray(k, dtype=np.float64) / np.asarray(lam, dtype=np.float64)


def smooth_query(q, lam) -> np.ndarray:
    """The query with the inverse of the key smoothing folded in: channel i
    multiplied by lam_i, so smooth_query(q) . smooth_keys(k) = q . k."""
    return np.asarray(q, dtype=np.float64) * np.asarray(lam, dtype=np.float64)


def smooth_encode(x, lam, codebooks, **kw):
    """Codes of the smoothed vectors: rvq_encode(x / lam) (rotation
    included).  x: [..., D]; lam broadcasts to x.  Returns [N][S][G] for the
    rows of x flattened."""
    y = smooth_keys(x, lam)
    return rvq_encode(y.reshape(-1, y.shape[-1]), codebooks, **kw)


def reconstruct_smooth(codes, codebooks, lam) -> np.ndarray:
    """Original-domain keys from codes of smoothed keys: the factors times
    the unrotated reconstruction (the rotation is undone first, then the
    division).  lam broadcasts to the output [..., D]."""
    return reconstruct(codes, codebooks) * np.asarray(lam, dtype=np.float64)


# ----------------------------------------------------------------------------
# Codebook fitting  [VI VecInfer: K-means codebooks per sub-vector, trained
#       before use ("train_codebook")], [VQKV 2. Methodology: the stage
#       codebooks are trained]
# ----------------------------------------------------------------------------
def lloyd_update(r, z, cb):
    """One K-means centroid update: entry c becomes the mean of the vectors
    r [N][dsub] assigned to it (z [N]); an entry with no vector keeps its
    value.  cb [C][dsub] is not modified; returns the new float64 entries."""
    r = np.asarray(r, dtype=np.float64)
    new = np.array(cb, dtype=np.float64, copy=True)
    for c in range(new.shape[0]):
        members = r[np.asarray(z) == c]
        if members.shape[0] > 0:
            new[c] = members.mean(axis=0)
    return new


def fit_codebooks(x, init, n_iter: int, *, rotate: bool = True, with_history: bool = False):
    """Fit residual product codebooks by K-means (Lloyd), stage by stage.

    x: [N][D] sample vectors (original domain, or rotated when ``rotate`` is
    False); init: [S][G][C][dsub] starting entries.  For each stage s and each
    group g, on the residuals r that the earlier (already fitted) stages
    leave: n_iter times {assign every vector to its nearest entry (squared
    distance, lowest index on ties); replace every entry by the mean of its
    vectors (entries with none keep theirs)}; then assign once more with the
    fitted entries and subtract them, giving the next stage's residuals.
    Returns the fitted float64 codebooks (and, with ``with_history``, the
    per-iteration distortion sum over vectors of |r - C[z]|^2 per (s, g)
    measured at each assignment, a list [S][G][n_iter + 1])."""
    cb = np.array(init, dtype=np.float64, copy=True)
    S, G, C, dsub = cb.shape
    y = fwht(x) if rotate else np.asarray(x, dtype=np.float64)
    hist = [[[] for _ in range(G)] for _ in range(S)]
    for g in range(G):
        r = y[:, g * dsub:(g + 1) * dsub].copy()
        for s in range(S):
            for _ in range(n_iter):
                z, d = nearest(r, cb[s, g])
                hist[s][g].append(float(d[np.arange(len(z)), z].sum()))
                cb[s, g] = lloyd_update(r, z, cb[s, g])
            z, d = nearest(r, cb[s, g])
            hist[s][g].append(float(d[np.arange(len(z)), z].sum()))
            r = r - cb[s, g][z]
    return (cb, hist) if with_history else cb


# ----------------------------------------------------------------------------
# Scalar residual variant  [VI Architecture: TurboQuantRVQ pipeline; module
#       table: turboquant_rvq, Lloyd-Max codebooks, dsa.bit_pack; throughput
#       journey: boundary-sum quantise]
# ----------------------------------------------------------------------------
def _unit_pdf(kind: str):
    if kind == "gaussian":
        return lambda t: np.exp(-0.5 * t * t) / np.sqrt(2.0 * np.pi)
    if kind == "laplacian":
        s = 1.0 / np.sqrt(2.0)                      # unit variance: scale 1/sqrt(2)
        return lambda t: np.exp(-np.abs(t) / s) / (2.0 * s)
    raise ValueError(kind)


def lloyd_max_levels(kind: str, bits: int, tol: float = 1e-13, max_iter: int = 10000):
    """Lloyd-Max quantiser of 2^bits levels for the unit-variance density
    ``kind`` ("gaussian" or "laplacian"): alternate {thresholds = midpoints of
    neighbouring levels; level = centroid of the density over its cell}, each
    integral by adaptive quadrature, until the levels move less than tol.
    Returns the sorted float64 levels."""
    from scipy import integrate
    pdf = _unit_pdf(kind)
    n = 2 ** bits
    lv = np.linspace(-2.0, 2.0, n)
    for _ in range(max_iter):
        t = (lv[1:] + lv[:-1]) / 2.0
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        new = np.empty(n)
        for k in range(n):
            a, b = edges[k], edges[k + 1]
            mass = integrate.quad(pdf, a, b, limit=200)[0]
            first = integrate.quad(lambda u: u * pdf(u), a, b, limit=200)[0]
            new[k] = first / mass
        done = np.max(np.abs(new - lv)) < tol
        lv = new
        if done:
            break
    return lv


def lloyd_max_distortion(kind: str, levels) -> float:
    """Mean squared error of nearest-level quantisation of the unit-variance
    density by these levels (by quadrature)."""
    from scipy import integrate
    pdf = _unit_pdf(kind)
    lv = np.asarray(levels, dtype=np.float64)
    t = (lv[1:] + lv[:-1]) / 2.0
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    return float(sum(integrate.quad(lambda u, c=c: (u - c) ** 2 * pdf(u), a, b, limit=200)[0]
                     for a, b, c in zip(edges[:-1], edges[1:], lv)))


def scalar_nearest(y, levels):
    """Index of the nearest level for every element (lowest index on exact
    ties), the plain definition."""
    y = np.asarray(y, dtype=np.float64)
    lv = np.asarray(levels, dtype=np.float64)
    return np.argmin((y[..., None] - lv) ** 2, axis=-1).astype(np.uint8)


def boundary_sum(y, levels):
    """The index as the number of decision thresholds (midpoints of sorted
    neighbouring levels) strictly below the element."""
    y = np.asarray(y, dtype=np.float64)
    lv = np.asarray(levels, dtype=np.float64)
    t = (lv[1:] + lv[:-1]) / 2.0
    return (y[..., None] > t).sum(axis=-1).astype(np.uint8)


def scalar_rvq_encode(x, levels1, levels2, *, rotate: bool = True):
    """Two-pass scalar residual quantisation of every element of the rotated
    vectors: z1 = nearest of levels1 to y, r = y - levels1[z1], z2 = nearest
    of levels2 to r.  x: [N][D].  Returns (z1, z2), uint8 [N][D] each."""
    y = fwht(x) if rotate else np.asarray(x, dtype=np.float64)
    l1 = np.asarray(levels1, dtype=np.float64)
    l2 = np.asarray(levels2, dtype=np.float64)
    z1 = scalar_nearest(y, l1)
    z2 = scalar_nearest(y - l1[z1], l2)
    return z1, z2


def pack_bits(z, bits: int):
    """Sub-byte packing of indices z [..., D] (values < 2^bits, bits 1..4,
    D * bits a multiple of 8) as one least-significant-first bit string per
    row: bit t of element i is bit 8 * j + k of the row's bytes, where
    i * bits + t = 8 * j + k.  For bits 1, 2 and 4 element i fills bits
    [(i mod k) * bits, ...) of byte i // k (k = 8 / bits); for 3 bits an
    element can straddle two bytes.  Returns uint8 [..., D*bits/8]."""
    z = np.asarray(z, dtype=np.uint8)
    D = z.shape[-1]
    if (D * bits) % 8:
        raise ValueError("D * bits must fill whole bytes")
    t = np.arange(bits, dtype=np.uint8)
    stream = (z[..., :, None] >> t) & 1                      # [..., D, bits]: bit t of z_i
    stream = stream.reshape(z.shape[:-1] + (D * bits // 8, 8))
    weights = (1 << np.arange(8)).astype(np.uint32)
    return (stream.astype(np.uint32) * weights).sum(axis=-1).astype(np.uint8)


def unpack_bits(codes, bits: int):
    """Inverse of pack_bits: uint8 [..., B] -> indices [..., B*8/bits]."""
    c = np.asarray(codes, dtype=np.uint8)
    nbytes = c.shape[-1]
    stream = (c[..., :, None] >> np.arange(8, dtype=np.uint8)) & 1     # [..., B, 8]
    stream = stream.reshape(c.shape[:-1] + (nbytes * 8 // bits, bits))
    weights = (1 << np.arange(bits)).astype(np.uint32)
    return (stream.astype(np.uint32) * weights).sum(axis=-1).astype(np.uint8)


def scalar_reconstruct(z1, z2, levels1, levels2, *, unrotate: bool = True):
    """y_hat = levels1[z1] + levels2[z2] per element, then H (the decode)."""
    l1 = np.asarray(levels1, dtype=np.float64)
    l2 = np.asarray(levels2, dtype=np.float64)
    y = l1[np.asarray(z1)] + l2[np.asarray(z2)]
    return fwht(y) if unrotate else y


def scalar_product_codebook(levels1, levels2, bits: int, head_dim: int):
    """The product codebook [2][G][256][k] (k = 8/bits, G = head_dim / k)
    under which a packed byte of stage s is an ordinary code: entry c holds
    levels_s[(c >> (j*bits)) & (2^bits - 1)] for j < k, the same for every
    group.  With it the packed scalar codes decode by reconstruct_rot."""
    k = 8 // bits
    G = head_dim // k
    c = np.arange(256)[:, None]
    idx = (c >> (np.arange(k)[None, :] * bits)) & ((1 << bits) - 1)
    out = np.empty((2, G, 256, k))
    for s, lv in enumerate((levels1, levels2)):
        out[s] = np.asarray(lv, dtype=np.float64)[idx][None]
    return out


def attend_scalar(q, k_codes, v_codes, k_levels, v_levels, bits, k_win=None, v_win=None,
                  scale=None):
    """Decode attention over packed scalar codes: k_codes, v_codes
    [B][Hkv][Tc][2][D*bits/8] uint8 (stage-1 bytes, then stage-2 bytes);
    k_levels, v_levels: (levels1, levels2) pairs.  Keys and values of the
    coded part are scalar_reconstruct of the unpacked indices; the rest as
    attend."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((B, Hq, D))
    for b in range(B):
        parts_k, parts_v = [], []
        if k_codes is not None and k_codes.shape[2] > 0:
            for codes, lv, parts in ((k_codes, k_levels, parts_k), (v_codes, v_levels, parts_v)):
                z = unpack_bits(codes[b], bits)                 # [Hkv][Tc][2][D]
                parts.append(scalar_reconstruct(z[:, :, 0], z[:, :, 1], lv[0], lv[1]))
        if k_win is not None and k_win.shape[2] > 0:
            parts_k.append(np.asarray(k_win[b], dtype=np.float64))
            parts_v.append(np.asarray(v_win[b], dtype=np.float64))
        out[b] = attend_dense(q[b], np.concatenate(parts_k, axis=1),
                              np.concatenate(parts_v, axis=1), scale)
    return out


def lse_merge(parts):
    """Log-sum-exp merge of partial softmax results [DKV "Flash-Style LSE
    Combine"].  parts: iterable of (m, l, o) with m the partial max logit,
    l = sum exp(s - m) and o = sum exp(s - m) v (unnormalised).  Returns the
    normalised output sum_i e^(m_i - m*) o_i / sum_i e^(m_i - m*) l_i."""
    parts = list(parts)
    m_star = max(p[0] for p in parts)
    num = sum(np.exp(m - m_star) * np.asarray(o, dtype=np.float64) for m, _, o in parts)
    den = sum(np.exp(m - m_star) * l for m, l, _ in parts)
    return num / den


# ----------------------------------------------------------------------------
# Byte accounting  [VI v6 results: key compression 16x at 1 bit/elem, 8x at
# 2 bits/elem; VI "dsa.bit_pack" sub-byte index packing]
# ----------------------------------------------------------------------------
def code_bytes_per_vector(n_stages: int, n_groups: int, n_codewords: int = 256) -> float:
    """Code bits per vector / 8: S*G codes of ceil(log2 C) bits each."""
    bits = int(np.ceil(np.log2(n_codewords)))
    return n_stages * n_groups * bits / 8.0


def compression_ratio_vs_fp16(head_dim: int, n_stages: int, n_groups: int,
                              n_codewords: int = 256) -> float:
    """fp16 bytes of one vector over its code bytes (codebooks excluded)."""
    return 2.0 * head_dim / code_bytes_per_vector(n_stages, n_groups, n_codewords)
