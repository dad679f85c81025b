// Step 1: landmark queries by adaptive average pooling of Q (landmark
// construction in the method sections of the MiTA summaries: Q is down-sampled
// by average pooling into m landmark queries).
//
// One workgroup per (landmark, slice). Threads read the window's rows of Q in
// 16-byte pieces (d contiguous, so a row is read by d/8 neighbouring threads) and
// accumulate in fp64, which is exact for bf16 inputs. The mean is then written as
// fp64, as the MFMA operand (two bf16 parts hi + lo for bf16 inputs, fp32 for
// fp32 inputs) and as an upper bound of its 2-norm.
#include "common.h"
#include "plan.h"

namespace mita {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q, double* __restrict__ qt64,
                                                   void* __restrict__ qtop, float* __restrict__ qtnorm, int N,
                                                   int m, int grid_h, int grid_w, int pool_h, int pool_w) {
  constexpr int TPR = D / 8;          // threads per row, 8 elements each
  constexpr int RPI = 256 / TPR;      // rows per iteration
  const int i = blockIdx.x, z = blockIdx.y, t = threadIdx.x;
  const int a = i / pool_w, b = i % pool_w;
  const int r0 = (int)(((int64_t)a * grid_h) / pool_h);
  const int r1 = (int)(((int64_t)(a + 1) * grid_h + pool_h - 1) / pool_h);
  const int c0 = (int)(((int64_t)b * grid_w) / pool_w);
  const int c1 = (int)(((int64_t)(b + 1) * grid_w + pool_w - 1) / pool_w);
  const int wc = c1 - c0, cnt = (r1 - r0) * wc;
  const int col = (t % TPR) * 8, rsub = t / TPR;
  const T* base = Q + (size_t)z * N * D;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int w = rsub; w < cnt; w += RPI) {
    const int n = (r0 + w / wc) * grid_w + c0 + w % wc;
    const T* row = base + (size_t)n * D + col;
    if constexpr (sizeof(T) == 2) {
      uint4 v = *(const uint4*)row;
      const uint16_t* h = (const uint16_t*)&v;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (double)bf16_to_f32(h[e]);
    } else {
      float4 v0 = *(const float4*)row, v1 = *(const float4*)(row + 4);
      acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
      acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
    }
  }
  __shared__ double red[RPI][D];
  __shared__ double nrm[256 / WAVE];
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub][col + e] = acc[e];
  __syncthreads();
  double sq = 0.0;
  if (t < D) {
    double sum = 0.0;
    for (int r = 0; r < RPI; ++r) sum += red[r][t];
    const double q = sum / (double)cnt;
    const size_t o = ((size_t)z * m + i) * D + t;
    qt64[o] = q;
    if constexpr (sizeof(T) == 2) {
      const uint16_t hi = f64_to_bf16(q);
      const uint16_t lo = f64_to_bf16(q - (double)bf16_to_f32(hi));
      uint16_t* op = (uint16_t*)qtop;
      op[((size_t)z * 2 * m + i) * D + t] = hi;
      op[((size_t)z * 2 * m + m + i) * D + t] = lo;
    } else {
      ((float*)qtop)[o] = (float)q;
    }
    sq = q * q;
  }
  sq = wave_sum_f64(sq);
  if ((t % WAVE) == 0) nrm[t / WAVE] = sq;
  __syncthreads();
  if (t == 0) {
    double tot = 0.0;
    for (int w = 0; w < 256 / WAVE; ++w) tot += nrm[w];
    qtnorm[(size_t)z * m + i] = (float)(sqrt(tot) * (1.0 + 1e-6));
  }
}

template <typename T, int D>
static hipError_t pool_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  dim3 grid(p.m, p.BH);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, (const T*)Q, (double*)(ws + p.ws.qt64),
                     (void*)(ws + p.ws.qtop), (float*)(ws + p.ws.qtnorm), p.N, p.m, p.grid_h, p.grid_w, p.pool_h,
                     p.pool_w);
  return hipGetLastError();
}

hipError_t launch_pool(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? pool_launch<uint16_t, 64>(p, Q, ws, st) : pool_launch<uint16_t, 128>(p, Q, ws, st);
  return p.d == 64 ? pool_launch<float, 64>(p, Q, ws, st) : pool_launch<float, 128>(p, Q, ws, st);
}

}  // namespace mita
