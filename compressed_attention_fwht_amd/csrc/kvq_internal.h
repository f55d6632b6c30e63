// Internal launch interface between the C ABI (kvq_abi.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq_device.h"

namespace kvq {

// Decode-attention tables (LUT + V histogram) must fit this many LDS bytes.
constexpr size_t ATTN_LDS_TABLES = 150 * 1024;
constexpr int ATTN_MAX_CHUNK = 4096;   // tokens per split-K chunk, upper bound
constexpr int ATTN_MIN_CHUNK = 1024;   // preferred lower bound on chunk length
constexpr int ATTN_WIN_BLOCK = 2048;   // fp16 window tokens per window block
constexpr int RC_MAX_CHUNK = 4096;     // tokens per chunk of the rotated-code decode kernel

struct AttnPlan {
  int rc;          // 1: rotated-code kernels (attend_rc.hip), else the general ones
  int rp;          // query heads per chunk block (0: tables do not fit LDS)
  int n_hsplit;    // blocks per KV head along the query heads of its group
  int n_chunks;    // split-K chunks along the coded tokens
  int chunk;       // tokens per chunk
  int cparts;      // codeword ranges per (stage, dims) item in the V contraction
  int wslice;      // window tokens joining each chunk block (0: window blocks)
  int n_wblocks;   // window blocks of ATTN_WIN_BLOCK tokens, records after the chunks' ones
  int fuse_lut;    // 1: chunk blocks build their LUT (no attn_lut pass, no LUT bytes)
  int pstride;     // floats per partial record (m, l, pad, pad, o[D])
  size_t lut_slice;  // bytes of one (sequence, KV head, head split) LUT slice
  size_t lut_bytes, part_bytes, ws_bytes;
};

// Dual-transform smoothing factors [n_books][n_scale][D] (f == nullptr: none);
// sequence n of a book uses row n % n_scale.
struct Smooth {
  const float* f = nullptr;
  int64_t n_scale = 1;
};

AttnPlan attn_plan(int B, int Hq, int Hkv, int D, int S, int G, int C, int Tc, int W);

hipError_t launch_rotate(const void* x, int xt, float* y, int64_t n_rows, int dim, hipStream_t s);

size_t encode_workspace_bytes(int D, int G, int S, int C, int64_t n_books);
bool encode_mfma_eligible(int D, int G, int S, int C, int xt);
hipError_t launch_encode(const void* x, int xt, int D, int G, int S, int C, int64_t n_books,
                         int64_t n_seq, int64_t seq_stride, int64_t n_rows, const float* cb,
                         uint8_t* codes, int64_t code_stride, int64_t code_row0, int pre_rotated,
                         int force_generic, int packed, void* ws, Smooth sm, hipStream_t st);

// With sm.f the output is unrotated and multiplied by the factor row of each
// vector's sequence (n_rows vectors per sequence).
hipError_t launch_reconstruct(const uint8_t* codes, const float* cb, float* out, int64_t n_books,
                              int64_t n_per_book, int D, int G, int S, int C, int unrotate,
                              int64_t n_rows, Smooth sm, hipStream_t s);

// Rotated-code decode (head_dim 128, 16 x 8-dim groups, C = 256, 1/2/4 stages,
// GQA >= 2): eligibility, LUT bytes per unit, and the launch of its LUT /
// window kernel and chunk kernel (records only; the merge follows).
bool attn_rc_eligible(int D, int G, int S, int C, int Hq, int Hkv, int Tc);
size_t attn_rc_table_bytes(int S, int G);
int attn_rc_window_blocks(int W);
int attn_rc_window_slice(int W, int n_chunks);
hipError_t launch_attend_rc(const AttnPlan& p, int B, int Hq, int Hkv, int S, int G, int Tc,
                            int W, int cstride, int wstride, float scale, const float* q,
                            const uint8_t* kc, const uint8_t* vc, const float* kcb,
                            const float* vcb, const uint16_t* kw, const uint16_t* vw,
                            uint8_t* lut, float* part, Smooth ksm, hipStream_t st);

hipError_t launch_attend(const AttnPlan& p, int B, int Hq, int Hkv, int D, int S, int G, int C,
                         int Tc, int W, int cstride, int wstride, float scale, const float* q,
                         const uint8_t* kc,
                         const uint8_t* vc, const float* kcb, const float* vcb,
                         const uint16_t* kw, const uint16_t* vw, float* out, void* ws,
                         Smooth ksm, hipStream_t st);

hipError_t launch_smooth_calibrate(const void* x, int xt, int D, int64_t n_books, int64_t n_seq,
                                   int64_t seq_stride, int64_t n_rows, int64_t n_scale, float* f,
                                   hipStream_t st);

// Codebook fitting workspace: residuals f32 [N][D], codes [N][S][G], packed
// codebooks for the assignment, 64-bit partial sums [chunks][G][dsub][C],
// partial counts [chunks][G][C], per-stage bounds [S+1][copies][G]; byte
// offsets, each 256-aligned.
struct FitLayout {
  size_t resid, codes, pack, acc, cnt, bound, total;
};
FitLayout fit_layout(int D, int G, int S, int C, int64_t n);
hipError_t launch_codebook_fit(const void* x, int xt, int D, int G, int S, int C, int64_t n_seq,
                               int64_t seq_stride, int64_t n_rows, Smooth sm, int n_iter,
                               float* cb, void* ws, hipStream_t st);

// Scalar residual variant (bits in {1, 2, 4}); lloyd_max runs on the host.
int lloyd_max(int kind, int bits, double* levels, double* distortion);
hipError_t launch_scalar_encode(const void* x, int xt, int D, int bits, int64_t n_books,
                                int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                                const float* levels, uint8_t* codes, int pre_rotated,
                                hipStream_t st);
hipError_t launch_scalar_reconstruct(const uint8_t* codes, int D, int bits, int64_t n_books,
                                     int64_t n, const float* levels, float* out, int unrotate,
                                     hipStream_t st);
hipError_t launch_scalar_product_cb(const float* levels, int D, int bits, float* cb,
                                    hipStream_t st);

hipError_t launch_window_append(const uint16_t* kn, const uint16_t* vn, uint16_t* kw,
                                uint16_t* vw, int64_t units, int D, int wcap, int row,
                                hipStream_t st);
hipError_t launch_window_compact(uint16_t* kw, uint16_t* vw, int64_t units, int D, int wcap, int n,
                                 int shift, hipStream_t st);

}  // namespace kvq
