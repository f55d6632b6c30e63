// K3 -- reconstruction from codes: x_rot[g*dsub + j] = sum_s C_sg[z_sg][j],
// optionally followed by the inverse rotation x = H_D x_rot.
//
// "VQKV" summary, 2. Methodology (RSimVQ reconstruction as the sum of the
// retrieved entries); "VeloxQuant-MLX 0.5.1", Architecture (decode by summing
// stage outputs, then unrotate).
//
// The stage sum is accumulated in float64 and rounded once to float32, so the
// result is the correctly rounded sum whatever the stage order.  Layout as in
// K1: L = D/8 lanes per row, 8 output dims per lane (coalesced 32-byte
// stores), which is also the layout the optional unrotation needs.
// HBM-bound by the 4*D-byte float32 output per vector.
#include "kvq_internal.h"

namespace kvq {

// Each lane handles UNR independent vectors per iteration, stage-outer so
// that the code bytes and codeword rows of all UNR vectors are in flight
// together (memory-level parallelism).  dsub >= 8: a lane's 8 output dims lie
// in one group.
template <int D>
__global__ __launch_bounds__(256) void reconstruct_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ cb, float* __restrict__ out,
    int64_t n_books, int64_t n_per_book, int G, int S, int C, int dsub, int unrotate,
    const float* __restrict__ smooth, int64_t n_scale, int64_t n_rows) {
  constexpr int L = D / 8;
  constexpr int ROWS_PER_WAVE = 64 / L;
  constexpr int UNR = 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n_total = n_books * n_per_book;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int sub = lane / L;
  const int col = lane % L;
  const int SG = S * G;
  const int64_t book_stride = (int64_t)S * G * C * dsub;   // floats per book
  const int64_t step = waves_total * ROWS_PER_WAVE;
  const int d0 = col * 8;
  const int g = d0 / dsub, j0 = d0 % dsub;
  for (int64_t base = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * ROWS_PER_WAVE;
       base < n_total; base += step * UNR) {
    const uint8_t* crow[UNR];
    const float* bk[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      int64_t vec = base + u * step + sub;
      if (vec >= n_total) vec = n_total - 1;              // keep every lane in the butterfly
      crow[u] = codes + vec * SG + g;
      bk[u] = cb + (vec / n_per_book) * book_stride + (int64_t)g * C * dsub + j0;
    }
    double acc[UNR][8];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0;
    for (int s = 0; s < S; ++s) {
      int z[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        z[u] = crow[u][s * G];
        z[u] = z[u] < C ? z[u] : C - 1;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float4* p = reinterpret_cast<const float4*>(bk[u] + ((int64_t)s * G * C + z[u]) * dsub);
        const float4 a = p[0], c = p[1];
        acc[u][0] += a.x; acc[u][1] += a.y; acc[u][2] += a.z; acc[u][3] += a.w;
        acc[u][4] += c.x; acc[u][5] += c.y; acc[u][6] += c.z; acc[u][7] += c.w;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t vec = base + u * step + sub;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)acc[u][e];
      if (unrotate) {                       // uniform branch: all lanes take it
        hadamard_row<8, L>(v, lane);
        constexpr float sc = rsqrt_pow2(D);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= sc;
      }
      if (smooth != nullptr && vec < n_total) {   // dual transform undone: times the factors
        const int64_t book = vec / n_per_book;
        const int64_t seq = (vec - book * n_per_book) / n_rows;
        const float4* lp = reinterpret_cast<const float4*>(
            smooth + (book * n_scale + seq % n_scale) * D + col * 8);
        const float4 a = lp[0], c = lp[1];
        v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
        v[4] *= c.x; v[5] *= c.y; v[6] *= c.z; v[7] *= c.w;
      }
      if (vec < n_total) {
        float4* o = reinterpret_cast<float4*>(out + vec * D + col * 8);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

hipError_t launch_reconstruct(const uint8_t* codes, const float* cb, float* out, int64_t n_books,
                              int64_t n_per_book, int D, int G, int S, int C, int unrotate,
                              int64_t n_rows, Smooth sm, hipStream_t s) {
  const int64_t n = n_books * n_per_book;
  if (n == 0) return hipSuccess;
  const int dsub = D / G;
  const int rows_per_block = 4 * (64 / (D / 8)) * 4;      // 4 waves, 4 vectors per lane
  int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  if (blocks > 16384) blocks = 16384;
  auto kern = D == 64 ? reconstruct_kernel<64> : D == 128 ? reconstruct_kernel<128>
                                                          : reconstruct_kernel<256>;
  kern<<<dim3((unsigned)blocks), 256, 0, s>>>(codes, cb, out, n_books, n_per_book, G, S, C, dsub,
                                              unrotate, sm.f, sm.n_scale, n_rows);
  return hipGetLastError();
}

}  // namespace kvq
