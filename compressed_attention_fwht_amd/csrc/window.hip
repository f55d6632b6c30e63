// Streaming window maintenance around the coded cache: new decode tokens are
// appended to the fp16 window, and the window's oldest tokens are flushed --
// encoded into codes appended after the coded tokens -- when it fills
// ("VeloxQuant-MLX 0.5.1", Quick start: a cache grown by append and read by
// attend; "ZeroKV-Neo 4.0.0", profiling output: periodic flush_quantize
// calls; "VQKV" summary, 3. Inference Integration: recent tokens kept
// uncompressed in a local window, the rest compressed).
//
// The flush's encode is the encode kernel with its code rows placed at
// [n_code, n_code + n_flush) of each (sequence, KV head); what is left in the
// window then moves to its front (window_compact_kernel).
#include "kvq_internal.h"

namespace kvq {

// grid (B*Hkv), block 64: one 16-byte piece of the new row per lane.
__global__ void window_append_kernel(const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                                     uint16_t* __restrict__ kw, uint16_t* __restrict__ vw, int D,
                                     int wcap, int row) {
  const int64_t u = blockIdx.x;
  for (int p = threadIdx.x; p < D / 8; p += blockDim.x) {
    const uint4 a = reinterpret_cast<const uint4*>(kn + u * D)[p];
    const uint4 b = reinterpret_cast<const uint4*>(vn + u * D)[p];
    reinterpret_cast<uint4*>(kw + (u * wcap + row) * D)[p] = a;
    reinterpret_cast<uint4*>(vw + (u * wcap + row) * D)[p] = b;
  }
}

// grid (B*Hkv, 2: K / V), block 256.  Moves rows [shift, n) of one window to
// [0, n - shift).  Destination rows lie below their sources, so moving chunks
// of at most `shift` rows in increasing order, each read completely before it
// is written, never overwrites a row that is still to be read.
__global__ __launch_bounds__(256) void window_compact_kernel(uint16_t* __restrict__ kw,
                                                             uint16_t* __restrict__ vw, int D,
                                                             int wcap, int n, int shift) {
  uint16_t* w = (blockIdx.y == 0 ? kw : vw) + (int64_t)blockIdx.x * wcap * D;
  const int P = D / 8;                                  // 16-byte pieces per row
  const int rows_per = (256 / P) < shift ? (256 / P) : shift;
  const int m = n - shift;                              // rows to move
  for (int r0 = 0; r0 < m; r0 += rows_per) {
    const int nr = (m - r0) < rows_per ? (m - r0) : rows_per;
    const int pid = threadIdx.x;
    const bool act = pid < nr * P;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (act) v = reinterpret_cast<const uint4*>(w + (int64_t)(shift + r0) * D)[pid];
    __syncthreads();
    if (act) reinterpret_cast<uint4*>(w + (int64_t)r0 * D)[pid] = v;
    __syncthreads();
  }
}

hipError_t launch_window_append(const uint16_t* kn, const uint16_t* vn, uint16_t* kw,
                                uint16_t* vw, int64_t units, int D, int wcap, int row,
                                hipStream_t st) {
  window_append_kernel<<<dim3((unsigned)units), 64, 0, st>>>(kn, vn, kw, vw, D, wcap, row);
  return hipGetLastError();
}

hipError_t launch_window_compact(uint16_t* kw, uint16_t* vw, int64_t units, int D, int wcap, int n,
                                 int shift, hipStream_t st) {
  if (n - shift <= 0) return hipSuccess;
  window_compact_kernel<<<dim3((unsigned)units, 2), 256, 0, st>>>(kw, vw, D, wcap, n, shift);
  return hipGetLastError();
}

}  // namespace kvq
