// C ABI of libkvq: argument validation (before any HIP call), workspace
// sizing and kernel dispatch.  See include/kvq.h for the contract.
#include <math.h>

#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

// Workspace of kvq_attend_decode_noalloc: one copy per GPU, held until the
// process ends.  In host code this name is a host-side stand-in, not a device
// address; the device address comes from hipGetSymbolAddress (scratch_base).
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// min_dsub: 8 for the encode, reconstruction and fitting kernels, 4 for decode
// attention (its V contraction works on 4 dims at a time).
kvq_status check_vq(const kvq_vq_desc* vq, int min_dsub = 8) {
  if (!vq) return KVQ_ERR_NULL;
  const int D = vq->head_dim, G = vq->n_groups, S = vq->n_stages, C = vq->n_codewords;
  if (D != 64 && D != 128 && D != 256) return KVQ_ERR_SHAPE;
  if (G < 1 || G > D || D % G != 0) return KVQ_ERR_SHAPE;
  const int dsub = D / G;
  if (!pow2(dsub) || dsub < min_dsub || dsub > 128) return KVQ_ERR_SHAPE;
  if (S < 1 || S > 8) return KVQ_ERR_SHAPE;
  if (C < 1 || C > 256) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

inline bool valid_dtype(kvq_dtype t) { return t == KVQ_F32 || t == KVQ_BF16 || t == KVQ_F16; }

kvq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  g_last_hip_error = (int)e;
  return KVQ_ERR_HIP;
}

kvq_status check_attn(const kvq_attn_desc* a, kvq::AttnPlan* plan) {
  if (!a) return KVQ_ERR_NULL;
  kvq_status st = check_vq(&a->vq, 2);      // 2-dim groups: 4-bit scalar codes
  if (st != KVQ_OK) return st;
  if (a->batch < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1) return KVQ_ERR_SHAPE;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (a->n_code_tokens < 0 || a->n_window < 0) return KVQ_ERR_SHAPE;
  if ((int64_t)a->n_code_tokens + a->n_window == 0) return KVQ_ERR_SHAPE;
  if (a->code_stride != 0 && a->code_stride < a->n_code_tokens) return KVQ_ERR_SHAPE;
  if (a->window_stride != 0 && a->window_stride < a->n_window) return KVQ_ERR_SHAPE;
  if ((int64_t)a->batch * a->n_q_heads > 0x7fffffff) return KVQ_ERR_SHAPE;
  if (a->batch > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!(a->softmax_scale == a->softmax_scale)) return KVQ_ERR_SHAPE;   // NaN
  const kvq_vq_desc& v = a->vq;
  *plan = kvq::attn_plan(a->batch, a->n_q_heads, a->n_kv_heads, v.head_dim, v.n_stages,
                         v.n_groups, v.n_codewords, a->n_code_tokens, a->n_window);
  if (a->n_code_tokens > 0) {
    if (plan->rp == 0) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)a->n_kv_heads * plan->n_hsplit > 65535) return KVQ_ERR_UNSUPPORTED;
  }
  return KVQ_OK;
}

kvq_status check_smooth(const kvq_smooth_desc* sm) {
  if (!sm || !sm->factors) return KVQ_ERR_NULL;
  if (sm->n_scale < 1) return KVQ_ERR_SHAPE;
  if (!aligned16(sm->factors)) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

kvq::Smooth to_smooth(const kvq_smooth_desc* sm) {
  kvq::Smooth r;
  if (sm) {
    r.f = sm->factors;
    r.n_scale = sm->n_scale;
  }
  return r;
}

// kvq_encode and kvq_encode_smooth (smooth == nullptr: no division)
kvq_status encode_common(const void* x, kvq_dtype xt, const kvq_vq_desc* vq, int64_t n_books,
                         int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                         const kvq_smooth_desc* smooth, const float* codebooks, uint8_t* codes,
                         uint32_t flags, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(xt)) return KVQ_ERR_DTYPE;
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (flags & ~(KVQ_INPUT_PRE_ROTATED | KVQ_ENCODE_GENERIC | KVQ_CODEBOOKS_PACKED))
    return KVQ_ERR_SHAPE;
  if (smooth && (flags & KVQ_INPUT_PRE_ROTATED)) return KVQ_ERR_UNSUPPORTED;
  if (n_books < 0 || n_seq < 0 || seq_stride < 0 || n_rows < 0) return KVQ_ERR_SHAPE;
  if (n_rows > seq_stride) return KVQ_ERR_SHAPE;
  if (smooth) {
    st = check_smooth(smooth);
    if (st != KVQ_OK) return st;
  }
  if (n_books == 0 || n_seq == 0 || n_rows == 0) return KVQ_OK;
  if (!x || !codebooks || !codes) return KVQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codebooks) || !aligned16(codes)) return KVQ_ERR_ALIGN;
  const int D = vq->head_dim, G = vq->n_groups, S = vq->n_stages, C = vq->n_codewords;
  const int64_t n_per_book = n_seq * n_rows;
  if (n_seq > ((int64_t)1 << 40) / n_rows) return KVQ_ERR_SHAPE;
  const int64_t tile = 64;   // smallest tile of either kernel
  if (n_books * ((n_per_book + tile - 1) / tile) > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
  const bool generic = (flags & KVQ_ENCODE_GENERIC) != 0 ||
                       !kvq::encode_mfma_eligible(D, G, S, C, (int)xt);
  if (!generic) {
    const size_t need = kvq::encode_workspace_bytes(D, G, S, C, n_books);
    if (ws_bytes < need || (need > 0 && !workspace)) return KVQ_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return KVQ_ERR_ALIGN;
  }
  return hip_status(kvq::launch_encode(x, (int)xt, D, G, S, C, n_books, n_seq, seq_stride, n_rows,
                                       codebooks, codes, n_rows, 0,
                                       (flags & KVQ_INPUT_PRE_ROTATED) ? 1 : 0,
                                       generic ? 1 : 0, (flags & KVQ_CODEBOOKS_PACKED) ? 1 : 0,
                                       workspace, to_smooth(smooth), stream));
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case KVQ_ERR_UNSUPPORTED: return "valid request the library has no kernel for";
    case KVQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_DTYPE: return "unknown element type";
    case KVQ_ERR_HIP: return "a HIP call failed (see kvq_last_hip_error)";
  }
  return "unknown status";
}

int kvq_last_hip_error(void) { return g_last_hip_error; }

kvq_status kvq_rotate(const void* x, kvq_dtype xt, float* y, int64_t n_rows, int32_t dim,
                      hipStream_t stream) {
  if (!valid_dtype(xt)) return KVQ_ERR_DTYPE;
  if (dim != 64 && dim != 128 && dim != 256) return KVQ_ERR_SHAPE;
  if (n_rows < 0) return KVQ_ERR_SHAPE;
  if (n_rows == 0) return KVQ_OK;
  if (!x || !y) return KVQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return KVQ_ERR_ALIGN;
  if (n_rows > ((int64_t)1 << 40) / dim) return KVQ_ERR_SHAPE;
  if (xt != KVQ_F32) {  // a half-width input may not overlap the float output
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    const uintptr_t xe = xa + (uintptr_t)(n_rows * dim * 2), ye = ya + (uintptr_t)(n_rows * dim * 4);
    if (xa < ye && ya < xe) return KVQ_ERR_SHAPE;
  } else if (x != y) {
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y, n = (uintptr_t)(n_rows * dim * 4);
    if (xa < ya + n && ya < xa + n) return KVQ_ERR_SHAPE;   // partial overlap
  }
  return hip_status(kvq::launch_rotate(x, (int)xt, y, n_rows, dim, stream));
}

kvq_status kvq_encode_workspace_size(const kvq_vq_desc* vq, int64_t n_books, size_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (n_books < 0) return KVQ_ERR_SHAPE;
  *bytes = kvq::encode_workspace_bytes(vq->head_dim, vq->n_groups, vq->n_stages,
                                       vq->n_codewords, n_books);
  return KVQ_OK;
}

kvq_status kvq_encode(const void* x, kvq_dtype xt, const kvq_vq_desc* vq, int64_t n_books,
                      int64_t n_seq, int64_t seq_stride, int64_t n_rows, const float* codebooks,
                      uint8_t* codes, uint32_t flags, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  return encode_common(x, xt, vq, n_books, n_seq, seq_stride, n_rows, nullptr, codebooks, codes,
                       flags, workspace, ws_bytes, stream);
}

kvq_status kvq_encode_smooth(const void* x, kvq_dtype xt, const kvq_vq_desc* vq, int64_t n_books,
                             int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                             const kvq_smooth_desc* smooth, const float* codebooks,
                             uint8_t* codes, uint32_t flags, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  if (!smooth) return KVQ_ERR_NULL;
  return encode_common(x, xt, vq, n_books, n_seq, seq_stride, n_rows, smooth, codebooks, codes,
                       flags, workspace, ws_bytes, stream);
}

kvq_status kvq_smooth_calibrate(const void* x, kvq_dtype xt, int32_t head_dim, int64_t n_books,
                                int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                                int32_t n_scale, float* factors, hipStream_t stream) {
  if (!valid_dtype(xt)) return KVQ_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_SHAPE;
  if (n_books < 0 || n_seq < 0 || seq_stride < 0 || n_rows < 0 || n_scale < 1)
    return KVQ_ERR_SHAPE;
  if (n_rows > seq_stride) return KVQ_ERR_SHAPE;
  if (n_books == 0) return KVQ_OK;
  if (!factors) return KVQ_ERR_NULL;
  if (!aligned16(factors)) return KVQ_ERR_ALIGN;
  if (n_books > ((int64_t)1 << 40) / ((int64_t)n_scale * head_dim)) return KVQ_ERR_SHAPE;
  const bool reads = n_seq > 0 && n_rows > 0;
  if (reads) {
    if (!x) return KVQ_ERR_NULL;
    if (!aligned16(x)) return KVQ_ERR_ALIGN;
    if (n_seq > ((int64_t)1 << 40) / seq_stride / n_books / head_dim) return KVQ_ERR_SHAPE;
    const int64_t row_blocks = (n_rows + 63) / 64;     // the smallest block covers 64 rows
    if (n_books * n_seq > 0x7fffffffLL / row_blocks) return KVQ_ERR_UNSUPPORTED;
    const int esz = xt == KVQ_F32 ? 4 : 2;
    const uintptr_t xa = (uintptr_t)x, fa = (uintptr_t)factors;
    const uintptr_t xe = xa + (uintptr_t)(n_books * n_seq * seq_stride * head_dim * esz);
    const uintptr_t fe = fa + (uintptr_t)((int64_t)n_books * n_scale * head_dim * 4);
    if (xa < fe && fa < xe) return KVQ_ERR_SHAPE;       // output may not overlap the input
  }
  return hip_status(kvq::launch_smooth_calibrate(x, (int)xt, head_dim, n_books, n_seq, seq_stride,
                                                 n_rows, n_scale, factors, stream));
}

kvq_status kvq_codebook_fit_workspace_size(const kvq_vq_desc* vq, int64_t n_vectors,
                                          size_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (n_vectors < 0 || n_vectors > KVQ_FIT_MAX_VECTORS) return KVQ_ERR_SHAPE;
  *bytes = kvq::fit_layout(vq->head_dim, vq->n_groups, vq->n_stages, vq->n_codewords, n_vectors)
               .total;
  return KVQ_OK;
}

kvq_status kvq_codebook_fit(const void* x, kvq_dtype xt, const kvq_vq_desc* vq, int64_t n_seq,
                            int64_t seq_stride, int64_t n_rows, const kvq_smooth_desc* smooth,
                            int32_t n_iter, float* codebooks, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  if (!valid_dtype(xt)) return KVQ_ERR_DTYPE;
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (n_seq < 0 || seq_stride < 0 || n_rows < 0 || n_rows > seq_stride) return KVQ_ERR_SHAPE;
  if (n_iter < 0 || n_iter > 100000) return KVQ_ERR_SHAPE;
  if (smooth) {
    st = check_smooth(smooth);
    if (st != KVQ_OK) return st;
  }
  if (n_seq == 0 || n_rows == 0) return KVQ_OK;
  if (n_seq > KVQ_FIT_MAX_VECTORS / n_rows) return KVQ_ERR_SHAPE;
  const int64_t n = n_seq * n_rows;
  if (!x || !codebooks || !workspace) return KVQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codebooks) || !aligned16(workspace)) return KVQ_ERR_ALIGN;
  const int D = vq->head_dim, G = vq->n_groups, S = vq->n_stages, C = vq->n_codewords;
  if (ws_bytes < kvq::fit_layout(D, G, S, C, n).total) return KVQ_ERR_WORKSPACE;
  return hip_status(kvq::launch_codebook_fit(x, (int)xt, D, G, S, C, n_seq, seq_stride, n_rows,
                                             to_smooth(smooth), n_iter, codebooks, workspace,
                                             stream));
}

kvq_status kvq_lloyd_max(kvq_levels_kind kind, int32_t bits, double* levels,
                         double* distortion) {
  if (kind != KVQ_LEVELS_GAUSSIAN && kind != KVQ_LEVELS_LAPLACIAN) return KVQ_ERR_SHAPE;
  if (bits < 1 || bits > 4) return KVQ_ERR_SHAPE;
  if (!levels) return KVQ_ERR_NULL;
  kvq::lloyd_max((int)kind, bits, levels, distortion);
  return KVQ_OK;
}

// codes of 1..4 bits; the product codebook needs whole elements per byte
static bool scalar_bits_ok(int bits) { return bits >= 1 && bits <= 4; }
static bool product_bits_ok(int bits) { return bits == 1 || bits == 2 || bits == 4; }

kvq_status kvq_scalar_encode(const void* x, kvq_dtype xt, int32_t head_dim, int32_t bits,
                             int64_t n_books, int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                             const float* levels, uint8_t* codes, uint32_t flags,
                             hipStream_t stream) {
  if (!valid_dtype(xt)) return KVQ_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_SHAPE;
  if (!scalar_bits_ok(bits)) return KVQ_ERR_SHAPE;
  if (flags & ~KVQ_INPUT_PRE_ROTATED) return KVQ_ERR_SHAPE;
  if (n_books < 0 || n_seq < 0 || seq_stride < 0 || n_rows < 0 || n_rows > seq_stride)
    return KVQ_ERR_SHAPE;
  if (n_books == 0 || n_seq == 0 || n_rows == 0) return KVQ_OK;
  if (n_books > 65535) return KVQ_ERR_UNSUPPORTED;
  if (n_seq > ((int64_t)1 << 40) / n_rows) return KVQ_ERR_SHAPE;
  if (!x || !levels || !codes) return KVQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(levels) || !aligned16(codes)) return KVQ_ERR_ALIGN;
  return hip_status(kvq::launch_scalar_encode(x, (int)xt, head_dim, bits, n_books, n_seq,
                                              seq_stride, n_rows, levels, codes,
                                              (flags & KVQ_INPUT_PRE_ROTATED) ? 1 : 0, stream));
}

kvq_status kvq_scalar_decode_reconstruct(const uint8_t* codes, int32_t head_dim, int32_t bits,
                                         int64_t n_books, int64_t n_per_book,
                                         const float* levels, float* out, uint32_t flags,
                                         hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_SHAPE;
  if (!scalar_bits_ok(bits)) return KVQ_ERR_SHAPE;
  if (flags & ~KVQ_UNROTATE) return KVQ_ERR_SHAPE;
  if (n_books < 0 || n_per_book < 0) return KVQ_ERR_SHAPE;
  if (n_books == 0 || n_per_book == 0) return KVQ_OK;
  if (n_books > 65535) return KVQ_ERR_UNSUPPORTED;
  if (n_per_book > ((int64_t)1 << 40) / n_books) return KVQ_ERR_SHAPE;
  if (!codes || !levels || !out) return KVQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(levels) || !aligned16(out)) return KVQ_ERR_ALIGN;
  return hip_status(kvq::launch_scalar_reconstruct(codes, head_dim, bits, n_books, n_per_book,
                                                   levels, out,
                                                   (flags & KVQ_UNROTATE) ? 1 : 0, stream));
}

kvq_status kvq_scalar_product_codebook(int32_t head_dim, int32_t bits, const float* levels,
                                       float* codebooks, hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_SHAPE;
  if (!product_bits_ok(bits)) return KVQ_ERR_SHAPE;
  if (!levels || !codebooks) return KVQ_ERR_NULL;
  if (!aligned16(levels) || !aligned16(codebooks)) return KVQ_ERR_ALIGN;
  return hip_status(kvq::launch_scalar_product_cb(levels, head_dim, bits, codebooks, stream));
}

kvq_status kvq_decode_reconstruct(const uint8_t* codes, const kvq_vq_desc* vq, int64_t n_books,
                                  int64_t n_per_book, const float* codebooks, float* out,
                                  uint32_t flags, hipStream_t stream) {
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (flags & ~KVQ_UNROTATE) return KVQ_ERR_SHAPE;
  if (n_books < 0 || n_per_book < 0) return KVQ_ERR_SHAPE;
  if (n_books == 0 || n_per_book == 0) return KVQ_OK;
  if (!codes || !codebooks || !out) return KVQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(codebooks) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (n_per_book > ((int64_t)1 << 40) / n_books) return KVQ_ERR_SHAPE;
  return hip_status(kvq::launch_reconstruct(codes, codebooks, out, n_books, n_per_book,
                                            vq->head_dim, vq->n_groups, vq->n_stages,
                                            vq->n_codewords, (flags & KVQ_UNROTATE) ? 1 : 0,
                                            n_per_book, kvq::Smooth{}, stream));
}

kvq_status kvq_decode_reconstruct_smooth(const uint8_t* codes, const kvq_vq_desc* vq,
                                         int64_t n_books, int64_t n_seq, int64_t n_rows,
                                         const float* codebooks, const kvq_smooth_desc* smooth,
                                         float* out, hipStream_t stream) {
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  st = check_smooth(smooth);
  if (st != KVQ_OK) return st;
  if (n_books < 0 || n_seq < 0 || n_rows < 0) return KVQ_ERR_SHAPE;
  if (n_books == 0 || n_seq == 0 || n_rows == 0) return KVQ_OK;
  if (!codes || !codebooks || !out) return KVQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(codebooks) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (n_seq > ((int64_t)1 << 40) / n_rows) return KVQ_ERR_SHAPE;
  const int64_t n_per_book = n_seq * n_rows;
  if (n_per_book > ((int64_t)1 << 40) / n_books) return KVQ_ERR_SHAPE;
  return hip_status(kvq::launch_reconstruct(codes, codebooks, out, n_books, n_per_book,
                                            vq->head_dim, vq->n_groups, vq->n_stages,
                                            vq->n_codewords, 1, n_rows, to_smooth(smooth),
                                            stream));
}

kvq_status kvq_window_append(int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                             int32_t window_cap, int32_t n_window, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* k_win, uint16_t* v_win,
                             hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_SHAPE;
  if (batch < 1 || n_kv_heads < 1 || window_cap < 1) return KVQ_ERR_SHAPE;
  if (n_window < 0 || n_window >= window_cap) return KVQ_ERR_SHAPE;
  if ((int64_t)batch * n_kv_heads > 0x7fffffff) return KVQ_ERR_SHAPE;
  if (!k_new || !v_new || !k_win || !v_win) return KVQ_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_win) || !aligned16(v_win))
    return KVQ_ERR_ALIGN;
  return hip_status(kvq::launch_window_append(k_new, v_new, k_win, v_win,
                                              (int64_t)batch * n_kv_heads, head_dim, window_cap,
                                              n_window, stream));
}

kvq_status kvq_window_flush_workspace_size(const kvq_vq_desc* vq, size_t* bytes) {
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_ERR_NULL;
  const size_t one = kvq::encode_workspace_bytes(vq->head_dim, vq->n_groups, vq->n_stages,
                                                 vq->n_codewords, 1);
  *bytes = 2 * ((one + 255) & ~(size_t)255);            // K books, then V books
  return KVQ_OK;
}

static kvq_status window_flush_common(const kvq_vq_desc* vq, int32_t batch, int32_t n_kv_heads,
                                      int32_t window_cap, int32_t n_window, int32_t n_flush,
                                      uint16_t* k_win, uint16_t* v_win, int32_t code_cap,
                                      int32_t n_code, uint8_t* k_codes, uint8_t* v_codes,
                                      const float* k_cb, const float* v_cb,
                                      const kvq_smooth_desc* k_smooth, uint32_t flags,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  kvq_status st = check_vq(vq);
  if (st != KVQ_OK) return st;
  if (k_smooth) {
    st = check_smooth(k_smooth);
    if (st != KVQ_OK) return st;
  }
  if (flags & ~KVQ_CODEBOOKS_PACKED) return KVQ_ERR_SHAPE;
  if (batch < 1 || n_kv_heads < 1 || window_cap < 1 || code_cap < 0) return KVQ_ERR_SHAPE;
  if (n_window < 0 || n_window > window_cap) return KVQ_ERR_SHAPE;
  if (n_flush < 0 || n_flush > n_window) return KVQ_ERR_SHAPE;
  if (n_code < 0 || (int64_t)n_code + n_flush > code_cap) return KVQ_ERR_SHAPE;
  if ((int64_t)batch * n_kv_heads > 0x7fffffff) return KVQ_ERR_SHAPE;
  if (n_flush == 0) return KVQ_OK;
  if (!k_win || !v_win || !k_codes || !v_codes || !k_cb || !v_cb) return KVQ_ERR_NULL;
  if (!aligned16(k_win) || !aligned16(v_win) || !aligned16(k_codes) || !aligned16(v_codes) ||
      !aligned16(k_cb) || !aligned16(v_cb))
    return KVQ_ERR_ALIGN;
  const int D = vq->head_dim, G = vq->n_groups, S = vq->n_stages, C = vq->n_codewords;
  const int64_t units = (int64_t)batch * n_kv_heads;
  if (((int64_t)n_flush * units + 63) / 64 > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
  size_t need = 0;
  kvq_window_flush_workspace_size(vq, &need);
  const size_t half = need / 2;
  const bool mfma = kvq::encode_mfma_eligible(D, G, S, C, (int)KVQ_F16);
  if (mfma) {
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const int packed = (flags & KVQ_CODEBOOKS_PACKED) ? 1 : 0;
  hipError_t e = kvq::launch_encode(k_win, (int)KVQ_F16, D, G, S, C, 1, units, window_cap, n_flush,
                                    k_cb, k_codes, code_cap, n_code, 0, 0, packed, ws,
                                    to_smooth(k_smooth), stream);
  if (e == hipSuccess)
    e = kvq::launch_encode(v_win, (int)KVQ_F16, D, G, S, C, 1, units, window_cap, n_flush, v_cb,
                           v_codes, code_cap, n_code, 0, 0, packed, mfma ? ws + half : nullptr,
                           kvq::Smooth{}, stream);
  if (e == hipSuccess)
    e = kvq::launch_window_compact(k_win, v_win, units, D, window_cap, n_window, n_flush, stream);
  return hip_status(e);
}

kvq_status kvq_window_flush(const kvq_vq_desc* vq, int32_t batch, int32_t n_kv_heads,
                            int32_t window_cap, int32_t n_window, int32_t n_flush,
                            uint16_t* k_win, uint16_t* v_win, int32_t code_cap, int32_t n_code,
                            uint8_t* k_codes, uint8_t* v_codes, const float* k_cb,
                            const float* v_cb, uint32_t flags, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  return window_flush_common(vq, batch, n_kv_heads, window_cap, n_window, n_flush, k_win, v_win,
                             code_cap, n_code, k_codes, v_codes, k_cb, v_cb, nullptr, flags,
                             workspace, ws_bytes, stream);
}

kvq_status kvq_window_flush_smooth(const kvq_vq_desc* vq, int32_t batch, int32_t n_kv_heads,
                                   int32_t window_cap, int32_t n_window, int32_t n_flush,
                                   uint16_t* k_win, uint16_t* v_win, int32_t code_cap,
                                   int32_t n_code, uint8_t* k_codes, uint8_t* v_codes,
                                   const float* k_cb, const float* v_cb,
                                   const kvq_smooth_desc* k_smooth, uint32_t flags,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!k_smooth) return KVQ_ERR_NULL;
  return window_flush_common(vq, batch, n_kv_heads, window_cap, n_window, n_flush, k_win, v_win,
                             code_cap, n_code, k_codes, v_codes, k_cb, v_cb, k_smooth, flags,
                             workspace, ws_bytes, stream);
}

kvq_status kvq_cache_bytes(const kvq_attn_desc* a, uint64_t* code_bytes, uint64_t* window_bytes,
                           uint64_t* codebook_bytes, uint64_t* dense_bytes) {
  if (!a || !code_bytes || !window_bytes || !codebook_bytes || !dense_bytes) return KVQ_ERR_NULL;
  const kvq_status st = check_vq(&a->vq, 4);
  if (st != KVQ_OK) return st;
  if (a->batch < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1) return KVQ_ERR_SHAPE;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (a->n_code_tokens < 0 || a->n_window < 0) return KVQ_ERR_SHAPE;
  const kvq_vq_desc& v = a->vq;
  using u128 = unsigned __int128;
  const u128 heads = (u128)2 * (u128)a->batch * (u128)a->n_kv_heads;   // K and V rows
  const u128 code = heads * (u128)a->n_code_tokens * (u128)(v.n_stages * v.n_groups);
  const u128 win = heads * (u128)a->n_window * (u128)v.head_dim * 2;
  const u128 books = (u128)2 * v.n_stages * v.n_groups * v.n_codewords * (v.head_dim / v.n_groups) * 4;
  const u128 dense = heads * ((u128)a->n_code_tokens + (u128)a->n_window) * (u128)v.head_dim * 2;
  const u128 lim = (u128)1 << 63;
  if (code > lim || win > lim || dense > lim) return KVQ_ERR_SHAPE;
  *code_bytes = (uint64_t)code;
  *window_bytes = (uint64_t)win;
  *codebook_bytes = (uint64_t)books;
  *dense_bytes = (uint64_t)dense;
  return KVQ_OK;
}

kvq_status kvq_attend_workspace_size(const kvq_attn_desc* a, size_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  kvq::AttnPlan plan;
  kvq_status st = check_attn(a, &plan);
  if (st != KVQ_OK) return st;
  *bytes = plan.ws_bytes;
  return KVQ_OK;
}

// Every check of a decode call except the workspace's, before any HIP call.
static kvq_status attend_check(const kvq_attn_desc* a, const float* q, const uint8_t* k_codes,
                               const uint8_t* v_codes, const float* k_cb, const float* v_cb,
                               const kvq_smooth_desc* k_smooth, const uint16_t* k_win,
                               const uint16_t* v_win, const float* out, kvq::AttnPlan* plan) {
  kvq_status st = check_attn(a, plan);
  if (st != KVQ_OK) return st;
  if (k_smooth) {
    st = check_smooth(k_smooth);
    if (st != KVQ_OK) return st;
  }
  if (!q || !out) return KVQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (a->n_code_tokens > 0) {
    if (!k_codes || !v_codes || !k_cb || !v_cb) return KVQ_ERR_NULL;
    if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_cb) || !aligned16(v_cb))
      return KVQ_ERR_ALIGN;
  }
  if (a->n_window > 0) {
    if (!k_win || !v_win) return KVQ_ERR_NULL;
    if (!aligned16(k_win) || !aligned16(v_win)) return KVQ_ERR_ALIGN;
  }
  return KVQ_OK;
}

static kvq_status attend_common(const kvq_attn_desc* a, const float* q, const uint8_t* k_codes,
                                const uint8_t* v_codes, const float* k_cb, const float* v_cb,
                                const kvq_smooth_desc* k_smooth, const uint16_t* k_win,
                                const uint16_t* v_win, float* out, void* workspace,
                                size_t ws_bytes, hipStream_t stream) {
  kvq::AttnPlan plan;
  kvq_status st = attend_check(a, q, k_codes, v_codes, k_cb, v_cb, k_smooth, k_win, v_win, out,
                               &plan);
  if (st != KVQ_OK) return st;
  if (!workspace) return KVQ_ERR_NULL;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (ws_bytes < plan.ws_bytes) return KVQ_ERR_WORKSPACE;
  const kvq_vq_desc& v = a->vq;
  const float scale = a->softmax_scale > 0.0f ? a->softmax_scale
                                              : (float)(1.0 / sqrt((double)v.head_dim));
  return hip_status(kvq::launch_attend(plan, a->batch, a->n_q_heads, a->n_kv_heads, v.head_dim,
                                       v.n_stages, v.n_groups, v.n_codewords, a->n_code_tokens,
                                       a->n_window,
                                       a->code_stride ? a->code_stride : a->n_code_tokens,
                                       a->window_stride ? a->window_stride : a->n_window,
                                       scale, q, k_codes, v_codes, k_cb, v_cb, k_win,
                                       v_win, out, workspace, to_smooth(k_smooth), stream));
}

kvq_status kvq_attend_decode(const kvq_attn_desc* a, const float* q, const uint8_t* k_codes,
                             const uint8_t* v_codes, const float* k_cb, const float* v_cb,
                             const uint16_t* k_win, const uint16_t* v_win, float* out,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  return attend_common(a, q, k_codes, v_codes, k_cb, v_cb, nullptr, k_win, v_win, out, workspace,
                       ws_bytes, stream);
}

// Device address of `scratch` on the current device: looked up with that
// device current the first time a call runs on it, then kept (one address per
// device; the lookup is guarded for calls from several host threads).  A
// stream of another device is refused: its kernels would reach this device's
// copy.
static kvq_status scratch_base(hipStream_t stream, void** base) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    if (sdev != dev) return KVQ_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    addr[dev] = p;
  }
  *base = addr[dev];
  return KVQ_OK;
}

kvq_status kvq_attend_decode_noalloc(const kvq_attn_desc* a, const float* q,
                                     const uint8_t* k_codes, const uint8_t* v_codes,
                                     const float* k_cb, const float* v_cb,
                                     const uint16_t* k_win, const uint16_t* v_win, float* out,
                                     hipStream_t stream) {
  kvq::AttnPlan plan;
  kvq_status st = attend_check(a, q, k_codes, v_codes, k_cb, v_cb, nullptr, k_win, v_win, out,
                               &plan);
  if (st != KVQ_OK) return st;
  if (plan.ws_bytes > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_base(stream, &ws);
  if (st != KVQ_OK) return st;
  return attend_common(a, q, k_codes, v_codes, k_cb, v_cb, nullptr, k_win, v_win, out, ws,
                       (size_t)KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

kvq_status kvq_attend_decode_smooth(const kvq_attn_desc* a, const float* q,
                                    const uint8_t* k_codes, const uint8_t* v_codes,
                                    const float* k_cb, const float* v_cb,
                                    const kvq_smooth_desc* k_smooth, const uint16_t* k_win,
                                    const uint16_t* v_win, float* out, void* workspace,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!k_smooth) return KVQ_ERR_NULL;
  return attend_common(a, q, k_codes, v_codes, k_cb, v_cb, k_smooth, k_win, v_win, out,
                       workspace, ws_bytes, stream);
}

}  // extern "C"
