// Calibration of the dual transform's smoothing factors.
//
// "VeloxQuant-MLX 0.5.1", VecInfer section: each key channel i is scaled by
// lambda_i = sqrt(max |K_i|) before the Walsh-Hadamard rotation.  Here the
// maximum runs over the rows [0, n_rows) of every sequence that maps to a
// factor row (sequence n -> row n % n_scale).
//
// Three kernels on the caller's stream, all writing the output array only:
//   1. smooth_clear_kernel  -- the output, read as uint32, set to 0;
//   2. smooth_max_kernel    -- per block, the channel maxima of |x| over a
//      range of rows of one sequence (8 rows per thread, loaded together),
//      folded into the output with 32-bit atomic max on the float bit
//      patterns (|x| >= 0 orders like its bits; a NaN's bits exceed every
//      finite value's and +inf's, so NaN wins);
//   3. smooth_finish_kernel -- bits -> sqrt (correctly rounded float32), or 1
//      where the maximum is 0.
// HBM-bound: one read of the 2- or 4-byte input.
#include "kvq_internal.h"

namespace kvq {

// rows per thread, loaded together (their loads are all in flight at once)
constexpr int SM_RPT = 8;

__global__ __launch_bounds__(256) void smooth_clear_kernel(uint32_t* __restrict__ f, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    f[i] = 0u;
}

// 1-D grid: block = (book, sequence, range of 256/L * SM_RPT rows).  L = D/8
// lanes per row, 8 channels per lane; a thread takes SM_RPT rows 256/L apart.
template <int D, int XT>
__global__ __launch_bounds__(256) void smooth_max_kernel(const void* __restrict__ x,
                                                         uint32_t* __restrict__ f, int64_t n_seq,
                                                         int64_t seq_stride, int64_t n_rows,
                                                         int64_t n_scale, int64_t row_blocks) {
  constexpr int L = D / 8;
  constexpr int RPP = 256 / L;                          // rows per pass of the block
  constexpr int ESZ = XT == 0 ? 4 : 2;
  __shared__ uint32_t red[RPP][D];
  const int tid = threadIdx.x;
  const int col = tid % L, rsub = tid / L;
  const int64_t rb = blockIdx.x % row_blocks;
  const int64_t bs = blockIdx.x / row_blocks;           // book * n_seq + seq
  const int64_t seq = bs % n_seq, book = bs / n_seq;
  const int64_t r0 = rb * (RPP * SM_RPT) + rsub;
  const char* base = reinterpret_cast<const char*>(x) + (bs * seq_stride * D + col * 8) * ESZ;
  uint32_t m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0u;
  // rows past the end repeat the last row (no branch around the loads, so
  // all of them are in flight together; a repeated row leaves the maximum)
  float v[SM_RPT][8];
#pragma unroll
  for (int k = 0; k < SM_RPT; ++k) {
    const int64_t r = r0 + (int64_t)k * RPP;
    load8<XT>(base + (r < n_rows ? r : n_rows - 1) * D * ESZ, v[k]);
  }
  __builtin_amdgcn_sched_barrier(0);                    // every load issued before any use
#pragma unroll
  for (int k = 0; k < SM_RPT; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = __float_as_uint(v[k][e]) & 0x7fffffffu;
      m[e] = a > m[e] ? a : m[e];
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub][col * 8 + e] = m[e];
  __syncthreads();
  if (tid < D) {
    uint32_t a = red[0][tid];
    for (int i = 1; i < RPP; ++i) a = red[i][tid] > a ? red[i][tid] : a;
    if (a != 0u) atomicMax(f + (book * n_scale + seq % n_scale) * D + tid, a);
  }
}

__global__ __launch_bounds__(256) void smooth_finish_kernel(float* __restrict__ f, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint32_t b = reinterpret_cast<const uint32_t*>(f)[i];
    f[i] = b == 0u ? 1.0f : sqrtf(__uint_as_float(b));
  }
}

template <int D, int XT>
static void launch_smooth_max(const void* x, uint32_t* f, int64_t blocks, int64_t n_seq,
                              int64_t seq_stride, int64_t n_rows, int64_t n_scale,
                              int64_t row_blocks, hipStream_t st) {
  smooth_max_kernel<D, XT><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
      x, f, n_seq, seq_stride, n_rows, n_scale, row_blocks);
}

hipError_t launch_smooth_calibrate(const void* x, int xt, int D, int64_t n_books, int64_t n_seq,
                                   int64_t seq_stride, int64_t n_rows, int64_t n_scale,
                                   float* f, hipStream_t st) {
  const int64_t n_out = n_books * n_scale * D;
  if (n_out == 0) return hipSuccess;
  int64_t cblocks = (n_out + 255) / 256;
  if (cblocks > 4096) cblocks = 4096;
  uint32_t* fu = reinterpret_cast<uint32_t*>(f);
  smooth_clear_kernel<<<dim3((unsigned)cblocks), dim3(256), 0, st>>>(fu, n_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_seq > 0 && n_rows > 0) {
    const int64_t rows_per_block = (int64_t)(256 / (D / 8)) * SM_RPT;
    const int64_t row_blocks = (n_rows + rows_per_block - 1) / rows_per_block;
    const int64_t blocks = n_books * n_seq * row_blocks;
#define KVQ_SM(DD)                                                                             \
  if (D == DD) {                                                                              \
    if (xt == 0) launch_smooth_max<DD, 0>(x, fu, blocks, n_seq, seq_stride, n_rows, n_scale,  \
                                          row_blocks, st);                                    \
    else if (xt == 1) launch_smooth_max<DD, 1>(x, fu, blocks, n_seq, seq_stride, n_rows,      \
                                               n_scale, row_blocks, st);                      \
    else launch_smooth_max<DD, 2>(x, fu, blocks, n_seq, seq_stride, n_rows, n_scale,          \
                                  row_blocks, st);                                            \
  }
    KVQ_SM(64) KVQ_SM(128) KVQ_SM(256)
#undef KVQ_SM
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  smooth_finish_kernel<<<dim3((unsigned)cblocks), dim3(256), 0, st>>>(f, n_out);
  return hipGetLastError();
}

}  // namespace kvq
