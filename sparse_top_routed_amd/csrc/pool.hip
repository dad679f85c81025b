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

// One wave per landmark (four per workgroup): lanes read the window's rows in
// 16-byte pieces (a row is d/8 neighbouring lanes), four rows per lane in
// flight, and the row groups are summed with shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q, double* __restrict__ qt64,
                                                   void* __restrict__ qtop, float* __restrict__ qtnorm,
                                                   int N, int m,
                                                   int grid_h, int grid_w, int pool_h, int pool_w) {
  constexpr int TPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPW = WAVE / TPR;     // rows per wave step
  // the landmark index is wave-uniform: keep the window arithmetic scalar
  const int i = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), z = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (i >= m) return;
  const int a = i / pool_w, b = i % pool_w;
  // window bounds floor(a L / M) and ceil((a + 1) L / M): the products are
  // integers below 2^53 and a non-integer quotient is at least 1/M away from an
  // integer, so the rounded fp64 quotient gives the exact floor and ceil
  const int r0 = (int)floor((double)a * grid_h / pool_h);
  const int r1 = (int)ceil((double)(a + 1) * grid_h / pool_h);
  const int c0 = (int)floor((double)b * grid_w / pool_w);
  const int c1 = (int)ceil((double)(b + 1) * grid_w / pool_w);
  const int wc = c1 - c0, cnt = (r1 - r0) * wc;
  const int col = (lane % TPR) * 8, rsub = lane / TPR;
  const T* base = Q + (size_t)z * N * D;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int w0 = rsub; w0 < cnt; w0 += 4 * RPW) {
    uint4 v[4][sizeof(T) == 2 ? 1 : 2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int w = w0 + u * RPW, wl = min(w, cnt - 1);   // unconditional load, zeroed after
      const int n = (r0 + wl / wc) * grid_w + c0 + wl % wc;
      const T* row = base + (size_t)n * D + col;
#pragma unroll
      for (int h = 0; h < (sizeof(T) == 2 ? 1 : 2); ++h) {
        const uint4 x = *(const uint4*)(row + h * 4);
        v[u][h] = w < cnt ? x : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (sizeof(T) == 2) {
        const uint16_t* h = (const uint16_t*)&v[u][0];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)bf16_to_f32(h[e]);
      } else {
        const float* f = (const float*)&v[u][0];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
      }
    }
  }
  // sum the row groups (lanes that share a column differ by multiples of TPR)
#pragma unroll
  for (int o = TPR; o < WAVE; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, WAVE);
  double q[8], sq = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    q[e] = acc[e] / (double)cnt;
    sq += q[e] * q[e];
  }
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) sq += __shfl_xor(sq, o, WAVE);
  if (lane < TPR) {
    const size_t o = ((size_t)z * m + i) * D + col;
#pragma unroll
    for (int e = 0; e < 8; e += 2) *(double2*)(qt64 + o + e) = make_double2(q[e], q[e + 1]);
    if constexpr (sizeof(T) == 2) {
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f64_to_bf16(q[e]);
        lo[e] = f64_to_bf16(q[e] - (double)bf16_to_f32(hi[e]));
      }
      uint16_t* op = (uint16_t*)qtop;
      *(uint4*)(op + ((size_t)z * 2 * m + i) * D + col) = *(const uint4*)hi;
      *(uint4*)(op + ((size_t)z * 2 * m + m + i) * D + col) = *(const uint4*)lo;
    } else {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (float)q[e];
      *(float4*)((float*)qtop + o) = make_float4(f[0], f[1], f[2], f[3]);
      *(float4*)((float*)qtop + o + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    if (lane == 0) qtnorm[(size_t)z * m + i] = (float)(sqrt(sq) * (1.0 + 1e-6));
  }
}

template <typename T, int D>
static hipError_t pool_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  dim3 grid((p.m + 3) / 4, p.BH);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, (const T*)Q, (double*)(ws + p.ws.qt64),
                     (void*)(ws + p.ws.qtop), (float*)(ws + p.ws.qtnorm), p.N, p.m, p.grid_h, p.grid_w, p.pool_h, p.pool_w);
  return hipGetLastError();
}

hipError_t launch_pool(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? pool_launch<uint16_t, 64>(p, Q, ws, st) : pool_launch<uint16_t, 128>(p, Q, ws, st);
  return p.d == 64 ? pool_launch<float, 64>(p, Q, ws, st) : pool_launch<float, 128>(p, Q, ws, st);
}

}  // namespace mita
