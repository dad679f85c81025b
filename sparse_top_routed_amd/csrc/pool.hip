// Step 1: landmark queries by adaptive average pooling of Q (landmark
// construction in the method sections of the MiTA summaries: Q is down-sampled
// by average pooling into m landmark queries).
//
// Two forms. For 2D token grids, a workgroup streams one band of Q (the rows of
// a row of pooling windows, contiguous runs of tokens) and sums columns first;
// otherwise (1D sequences, very wide rows) a wave reads one landmark's window.
// Both accumulate in fp64, which is exact for bf16 inputs. The mean is written as
// fp64, as the MFMA operand (two bf16 parts hi + lo for bf16 inputs, fp32 for
// fp32 inputs) and as an upper bound of its 2-norm.
#include "common.h"
#include "plan.h"

#include <algorithm>

namespace mita {

constexpr size_t kPoolBandLds = 32 * 1024;   // fp64 column sums of one band's column group

// Adds the 8 elements of a 16-byte piece (bf16) or two pieces (fp32) to acc in fp64.
template <typename T>
__device__ __forceinline__ void acc_piece(const u32x4 (&v)[sizeof(T) == 2 ? 1 : 2], double (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x;
    if constexpr (sizeof(T) == 2) {
      const uint32_t wv = v[0][e >> 1];
      x = __uint_as_float((e & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
    } else {
      x = __uint_as_float(v[e >> 2][e & 3]);
    }
    acc[e] += (double)x;
  }
}

// Writes landmark i of slice z: fp64, the MFMA operand (bf16 hi + lo parts, or
// fp32) and an upper bound of its 2-norm (sq = its squared norm, any lane).
template <typename T>
__device__ __forceinline__ void put_landmark(double* qt64, void* qtop, int z, int m, int D, int i, int d,
                                             double q) {
  const size_t o = ((size_t)z * m + i) * D + d;
  qt64[o] = q;
  if constexpr (sizeof(T) == 2) {
    const uint16_t hi = f64_to_bf16(q);
    const uint16_t lo = f64_to_bf16(q - (double)bf16_to_f32(hi));
    uint16_t* op = (uint16_t*)qtop;
    op[((size_t)z * 2 * m + i) * D + d] = hi;
    op[((size_t)z * 2 * m + m + i) * D + d] = lo;
  } else {
    ((float*)qtop)[o] = (float)q;
  }
}

// One wave per landmark (four per workgroup), for windows of any shape: the
// window is read row by row, lanes taking consecutive tokens of a row in 16-byte
// pieces (a token is d/8 neighbouring lanes), eight pieces per lane in flight;
// the lane groups are summed with shuffles at the end.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q, double* __restrict__ qt64,
                                                   void* __restrict__ qtop, float* __restrict__ qtnorm,
                                                   int N, int m,
                                                   int grid_h, int grid_w, int pool_h, int pool_w) {
  constexpr int TPR = D / 8;          // lanes per token, 8 elements each
  constexpr int RPW = WAVE / TPR;     // tokens per wave step
  constexpr int PU = 8;               // wave steps in flight
  constexpr int H = sizeof(T) == 2 ? 1 : 2;
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
  const int col = (lane % TPR) * 8, tsub = lane / TPR;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = r0; r < r1; ++r) {
    const T* row = Q + ((size_t)z * N + (size_t)r * grid_w + c0) * D;   // wave-uniform
    for (int t0 = 0; t0 < wc; t0 += PU * RPW) {
      u32x4 v[PU][H];
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const int t = t0 + u * RPW + tsub, tl = min(t, wc - 1);   // unconditional load, zeroed after
#pragma unroll
        for (int h = 0; h < H; ++h) {
          const u32x4 x = *(const u32x4*)(row + (uint32_t)(tl * D + col + 4 * h));
          v[u][h] = t < wc ? x : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < PU; ++u) acc_piece<T>(v[u], acc);
    }
  }
  // sum the token groups (lanes that share a column differ by multiples of TPR)
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
#pragma unroll
    for (int e = 0; e < 8; ++e) put_landmark<T>(qt64, qtop, z, m, D, i, col + e, q[e]);
    if (lane == 0) qtnorm[(size_t)z * m + i] = (float)(sqrt(sq) * (1.0 + 1e-6));
  }
}

// Row-band form for 2D grids: one workgroup per (row of landmarks, group of lb
// neighbouring landmarks in it) streams the band's tokens once (pooling window
// rows [r0, r1) by the group's columns, contiguous runs of tokens), forms the
// column sums in fp64 in LDS, and then sums each landmark's columns. Same fp64
// arithmetic (exact for bf16 inputs), rows summed first and columns second.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_band_kernel(const T* __restrict__ Q, double* __restrict__ qt64,
                                                        void* __restrict__ qtop, float* __restrict__ qtnorm,
                                                        int N, int m, int grid_h, int grid_w, int pool_h,
                                                        int pool_w, int lb, int ngroups) {
  extern __shared__ double colsum[];   // [columns of the group][D]
  constexpr int TPR = D / 8;           // threads per token, 8 elements each
  constexpr int H = sizeof(T) == 2 ? 1 : 2;
  constexpr int PU = 8;                // rows in flight per thread
  const int a = blockIdx.x / ngroups, g = blockIdx.x % ngroups, z = blockIdx.y, tid = threadIdx.x;
  const int b0 = g * lb, b1 = min(b0 + lb, pool_w);
  const int r0 = (int)floor((double)a * grid_h / pool_h);
  const int r1 = (int)ceil((double)(a + 1) * grid_h / pool_h);
  const int cs0 = (int)floor((double)b0 * grid_w / pool_w);
  const int cs1 = (int)ceil((double)b1 * grid_w / pool_w);
  const int R = r1 - r0, ncol = cs1 - cs0;
  const T* base = Q + ((size_t)z * N + (size_t)r0 * grid_w + cs0) * D;   // wave-uniform
  const uint32_t rstride = (uint32_t)grid_w * D;
  // two items (token column x 8-element piece) per thread in flight at once
  for (int it0 = tid; it0 < ncol * TPR; it0 += 512) {
    const int it1 = min(it0 + 256, ncol * TPR - 1);   // a repeat of the last item is not stored
    const uint32_t off0 = (uint32_t)((it0 / TPR) * D + (it0 % TPR) * 8);
    const uint32_t off1 = (uint32_t)((it1 / TPR) * D + (it1 % TPR) * 8);
    double acc0[8], acc1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.0;
    for (int rb = 0; rb < R; rb += PU) {
      u32x4 v0[PU][H], v1[PU][H];
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const uint32_t r = (uint32_t)min(rb + u, R - 1);   // unconditional load; rows past R skipped below
#pragma unroll
        for (int h = 0; h < H; ++h) {
          v0[u][h] = *(const u32x4*)(base + (off0 + r * rstride + 4 * h));
          v1[u][h] = *(const u32x4*)(base + (off1 + r * rstride + 4 * h));
        }
      }
#pragma unroll
      for (int u = 0; u < PU; ++u)
        if (rb + u < R) {   // uniform condition
          acc_piece<T>(v0[u], acc0);
          acc_piece<T>(v1[u], acc1);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) *(double2*)(colsum + off0 + e) = make_double2(acc0[e], acc0[e + 1]);
    if (it0 + 256 < ncol * TPR)
#pragma unroll
      for (int e = 0; e < 8; e += 2) *(double2*)(colsum + off1 + e) = make_double2(acc1[e], acc1[e + 1]);
  }
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  for (int b = b0 + w; b < b1; b += 4) {
    const int c0 = (int)floor((double)b * grid_w / pool_w) - cs0;
    const int c1 = (int)ceil((double)(b + 1) * grid_w / pool_w) - cs0;
    const int cnt = R * (c1 - c0);
    const int i = a * pool_w + b;
    double q[D / 64], sq = 0.0;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      double s = 0.0;
      for (int c = c0; c < c1; ++c) s += colsum[c * D + lane + 64 * e];
      q[e] = s / (double)cnt;
      sq += q[e] * q[e];
    }
    sq = wave_sum_f64(sq);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) put_landmark<T>(qt64, qtop, z, m, D, i, lane + 64 * e, q[e]);
    if (lane == 0) qtnorm[(size_t)z * m + i] = (float)(sqrt(sq) * (1.0 + 1e-6));
  }
}

// Columns spanned by landmarks [b0, b1) of a row of pool_w over grid_w columns.
static int64_t band_span(int64_t b0, int64_t b1, int64_t grid_w, int64_t pool_w) {
  const int64_t lo = b0 * grid_w / pool_w, hi = (b1 * grid_w + pool_w - 1) / pool_w;
  return hi - lo;
}

// Landmarks per band group such that every group's column sums fit kPoolBandLds;
// 0 if not even one landmark's window fits.
static int band_group(int grid_w, int pool_w, int D) {
  const int64_t cap = (int64_t)(kPoolBandLds / (D * sizeof(double)));   // columns
  auto fits = [&](int64_t lb) {
    for (int64_t b0 = 0; b0 < pool_w; b0 += lb)
      if (band_span(b0, std::min<int64_t>(b0 + lb, pool_w), grid_w, pool_w) > cap) return false;
    return true;
  };
  // a group of lb landmarks spans at most lb grid_w / pool_w + 2 columns
  int64_t lb = std::max<int64_t>(0, (cap - 2) * pool_w / grid_w);
  lb = std::min<int64_t>(lb, pool_w);
  if (lb == 0) return fits(1) ? 1 : 0;
  while (lb < pool_w && fits(lb + 1)) ++lb;
  // spread the landmarks evenly over the groups
  const int64_t ng = (pool_w + lb - 1) / lb;
  return (int)((pool_w + ng - 1) / ng);
}

template <typename T, int D>
static hipError_t pool_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  const int lb = p.grid_h > 1 ? band_group(p.grid_w, p.pool_w, D) : 0;
  if (lb > 0) {
    const int ng = (p.pool_w + lb - 1) / lb;
    int64_t span = 0;
    for (int b0 = 0; b0 < p.pool_w; b0 += lb)
      span = std::max<int64_t>(span, band_span(b0, std::min(b0 + lb, p.pool_w), p.grid_w, p.pool_w));
    hipLaunchKernelGGL((pool_band_kernel<T, D>), dim3(p.pool_h * ng, p.BH), dim3(256),
                       (size_t)span * D * sizeof(double), st, (const T*)Q, (double*)(ws + p.ws.qt64),
                       (void*)(ws + p.ws.qtop), (float*)(ws + p.ws.qtnorm), p.N, p.m, p.grid_h, p.grid_w,
                       p.pool_h, p.pool_w, lb, ng);
    return hipGetLastError();
  }
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
