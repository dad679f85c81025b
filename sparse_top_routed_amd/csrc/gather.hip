// Step 5: output. For query q with routed experts e_1..e_s, softmax attention
// over K* = [Q~, K_{I_e1}, ..., K_{I_es}] and V* = [V~, V_{I_e1}, ..., V_{I_es}]
// with scale 1/sqrt(d) (the Dutch MiTA summary's formula; a token in two of the
// query's experts is counted twice, as the concatenation says).
//
// The (query, slot) pairs are bucketed by expert with a counting sort (histogram,
// scan, scatter). The gather kernel then runs one workgroup per tile of up to 64
// queries of one bucket: the expert's k token rows are gathered into LDS 64 at a
// time and every query of the tile attends them on MFMA, so each gathered row is
// read once per tile rather than once per query. With s = 1 the same workgroup
// also attends the m landmark pairs and writes the output; with s > 1 it writes
// an unnormalised partial per (query, slot) and the combine kernel attends the
// landmark pairs and merges the s + 1 partial softmaxes.
#include "attn_core.h"

namespace mita {

__global__ __launch_bounds__(256) void clear_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void bucket_hist_kernel(const int32_t* __restrict__ E, uint32_t* __restrict__ bcount,
                                                          int Ns, int m) {
  extern __shared__ uint32_t h[];
  const int z = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  const int start = blockIdx.x * 4096, end = min(Ns, start + 4096);
  for (int e = start + tid; e < end; e += 256) {
    const int x = Ez[e];
    if ((unsigned)x < (unsigned)m) atomicAdd(&h[x], 1u);
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256)
    if (h[i]) atomicAdd(&bcount[(size_t)z * m + i], h[i]);
}

// Exclusive scans of the bucket sizes and of their query-tile counts, per slice.
__global__ __launch_bounds__(256) void bucket_scan_kernel(const uint32_t* __restrict__ bcount, uint32_t* __restrict__ boff,
                                                          uint32_t* __restrict__ toff, int m) {
  __shared__ uint32_t wtot[4];
  const int z = blockIdx.x, tid = threadIdx.x;
  const int per = (m + 255) / 256, i0 = min(m, tid * per), i1 = min(m, i0 + per);
  const uint32_t* c = bcount + (size_t)z * m;
  uint32_t sc = 0, st = 0;
  for (int i = i0; i < i1; ++i) { sc += c[i]; st += (c[i] + kQueryTile - 1) / kQueryTile; }
  uint32_t totc, tott;
  uint32_t oc = block_incl_scan(sc, wtot, totc) - sc;
  uint32_t ot = block_incl_scan(st, wtot, tott) - st;
  uint32_t* bo = boff + (size_t)z * (m + 1);
  uint32_t* to = toff + (size_t)z * (m + 1);
  for (int i = i0; i < i1; ++i) {
    bo[i] = oc;
    to[i] = ot;
    oc += c[i];
    ot += (c[i] + kQueryTile - 1) / kQueryTile;
  }
  if (tid == 0) { bo[m] = totc; to[m] = tott; }
}

// Scatter (query * s + slot) into its bucket; ranges are reserved per workgroup.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ E,
                                                             const uint32_t* __restrict__ boff,
                                                             uint32_t* __restrict__ bcursor, int32_t* __restrict__ perm,
                                                             int Ns, int m) {
  extern __shared__ uint32_t h[];  // [0, m): local counts, [m, 2m): global bases
  const int z = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  const int start = blockIdx.x * 4096;
  uint32_t rank[16];
  int ex[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = start + tid + 256 * u;
    ex[u] = e < Ns ? Ez[e] : -1;
    if ((unsigned)ex[u] >= (unsigned)m) ex[u] = -1;
    rank[u] = ex[u] >= 0 ? atomicAdd(&h[ex[u]], 1u) : 0u;
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256)
    if (h[i]) h[m + i] = boff[(size_t)z * (m + 1) + i] + atomicAdd(&bcursor[(size_t)z * m + i], h[i]);
  __syncthreads();
  int32_t* pz = perm + (size_t)z * Ns;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (ex[u] >= 0) pz[h[m + ex[u]] + rank[u]] = start + tid + 256 * u;
}

// Query fragments of one query row (zeros when the row is absent).
template <typename T, int D>
struct QFrag {
  uint4 b[1][D / 32];
  float f[D / 4];
  __device__ __forceinline__ void load(const T* qrow, bool ok, int g) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) b[0][ks] = ok ? *(const uint4*)(qrow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) f[ks] = ok ? qrow[4 * ks + g] : 0.f;
    }
  }
};

template <typename T, int D>
struct AttnLds {
  using TL = Tiles<T, D>;
  __align__(16) T k0[TL::KTILE];
  __align__(16) T k1[sizeof(T) == 2 ? TL::KTILE : 8];
  __align__(16) T v[TL::VTILE];
};

// One 64-key block of attention for the wave's 16 queries, keys already staged.
template <typename T, int D, int KP>
__device__ __forceinline__ void attend_block(AttnLds<T, D>& sm, const QFrag<T, D>& qf, int live, float sl2e,
                                             float& mrun, float& lrun, f32x4 (&o)[D / 16], int lane) {
  const int g = lane >> 4;
  f32x4 acc[4];
  if constexpr (sizeof(T) == 2)
    qk_bf16<D, KP, 1>((const uint16_t*)sm.k0, (const uint16_t*)sm.k1, qf.b, acc, lane);
  else
    qk_f32<D>((const float*)sm.k0, qf.f, acc, lane);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[kt][j] = (16 * kt + 4 * g + j < live) ? acc[kt][j] * sl2e : -INFINITY;
  const float alpha = online_softmax(acc, mrun, lrun);
  rescale<D>(o, alpha);
  if constexpr (sizeof(T) == 2)
    pv_bf16<D>((const uint16_t*)sm.v, acc, o, lane);
  else
    pv_f32<D>((const float*)sm.v, acc, o, lane);
}

// Attention over the m landmark pairs (keys Q~, values V~). Block-uniform call.
template <typename T, int D>
__device__ __forceinline__ void attend_landmarks(AttnLds<T, D>& sm, const QFrag<T, D>& qf, const void* qtop,
                                                 const void* vtop, int z, int m, float sl2e, float& mrun, float& lrun,
                                                 f32x4 (&o)[D / 16], int tid) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  const int lane = tid & 63;
  const T* p0 = BF ? (const T*)((const uint16_t*)qtop + (size_t)z * 2 * m * D) : (const T*)((const float*)qtop + (size_t)z * m * D);
  const T* p1 = p0 + (size_t)m * D;
  const T* vz = BF ? (const T*)((const uint16_t*)vtop + (size_t)z * m * D) : (const T*)((const float*)vtop + (size_t)z * m * D);
  for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {
    const int live = min(kKeyBlock, m - lb0);
    stage_rows<T, D>(sm.k0, TL::KSTR, [&](int rr) { return p0 + (size_t)(lb0 + rr) * D; }, live, tid);
    if constexpr (BF) {
      stage_rows<T, D>(sm.k1, TL::KSTR, [&](int rr) { return p1 + (size_t)(lb0 + rr) * D; }, live, tid);
      stage_vt_bf16<D>((uint16_t*)sm.v, [&](int rr) { return (const uint16_t*)vz + (size_t)(lb0 + rr) * D; }, live, tid);
    } else {
      stage_rows<T, D>(sm.v, TL::VSTR, [&](int rr) { return vz + (size_t)(lb0 + rr) * D; }, live, tid);
    }
    __syncthreads();
    attend_block<T, D, BF ? 2 : 1>(sm, qf, live, sl2e, mrun, lrun, o, lane);
    __syncthreads();
  }
}

// Write 4 consecutive outputs d0..d0+3 of one row.
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    *(uint2*)dst = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  } else {
    *(float4*)dst = make_float4(a, b, c, d);
  }
}

template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, const int32_t* __restrict__ I,
                                                     const uint32_t* __restrict__ boff, const uint32_t* __restrict__ toff,
                                                     const int32_t* __restrict__ perm, const void* __restrict__ qtop,
                                                     const void* __restrict__ vtop, T* __restrict__ out,
                                                     float* __restrict__ pacc, float* __restrict__ pml, int N, int m,
                                                     int k, int s, float sl2e) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  __shared__ AttnLds<T, D> sm;
  __shared__ int s_e, s_start, s_cnt;
  const int t = blockIdx.x, z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15,
            g = lane >> 4;
  const uint32_t* tz = toff + (size_t)z * (m + 1);
  const uint32_t* bz = boff + (size_t)z * (m + 1);
  if (tid == 0) {
    if ((uint32_t)t >= tz[m]) {
      s_e = -1;
    } else {
      int lo = 0, hi = m - 1;  // last e with tz[e] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tz[mid] <= (uint32_t)t) lo = mid; else hi = mid - 1;
      }
      s_e = lo;
      s_start = (int)(t - tz[lo]) * kQueryTile;
      s_cnt = min(kQueryTile, (int)(bz[lo + 1] - bz[lo]) - s_start);
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int rowi = 16 * w + r;
  const bool ok = rowi < s_cnt;
  const int entry = ok ? perm[(size_t)z * N * s + bz[e] + s_start + rowi] : 0;
  const int q = entry / s, slot = entry % s;
  QFrag<T, D> qf;
  qf.load(Q + ((size_t)z * N + q) * D, ok, g);

  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (FUSED) attend_landmarks<T, D>(sm, qf, qtop, vtop, z, m, sl2e, mrun, lrun, o, tid);

  const int32_t* Ie = I + ((size_t)z * m + e) * k;
  const T* Kz = K + (size_t)z * N * D;
  const T* Vz = V + (size_t)z * N * D;
  for (int kb = 0; kb < k; kb += kKeyBlock) {
    const int live = min(kKeyBlock, k - kb);
    stage_rows<T, D>(sm.k0, TL::KSTR, [&](int rr) { return Kz + (size_t)Ie[kb + rr] * D; }, live, tid);
    if constexpr (BF)
      stage_vt_bf16<D>((uint16_t*)sm.v, [&](int rr) { return (const uint16_t*)Vz + (size_t)Ie[kb + rr] * D; }, live, tid);
    else
      stage_rows<T, D>(sm.v, TL::VSTR, [&](int rr) { return Vz + (size_t)Ie[kb + rr] * D; }, live, tid);
    __syncthreads();
    attend_block<T, D, 1>(sm, qf, live, sl2e, mrun, lrun, o, lane);
    __syncthreads();
  }

  const float l = quad_sum(lrun);
  if (!ok) return;
  if constexpr (FUSED) {
    T* orow = out + ((size_t)z * N + q) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      store4<T>(orow + 16 * dt + 4 * g, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
  } else {
    const size_t ps = ((size_t)z * N + q) * s + slot;
    float* prow = pacc + ps * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *(float4*)(prow + 16 * dt + 4 * g) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) *(float2*)(pml + ps * 2) = make_float2(mrun, l);
  }
}

// s > 1: landmark part for 64 consecutive queries, merged with their s partials.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ Q, const void* __restrict__ qtop,
                                                      const void* __restrict__ vtop, const float* __restrict__ pacc,
                                                      const float* __restrict__ pml, T* __restrict__ out, int N, int m,
                                                      int s, float sl2e) {
  __shared__ AttnLds<T, D> sm;
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int q = blockIdx.x * kQueryTile + 16 * w + r;
  const bool ok = q < N;
  QFrag<T, D> qf;
  qf.load(Q + ((size_t)z * N + (ok ? q : 0)) * D, ok, g);
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  attend_landmarks<T, D>(sm, qf, qtop, vtop, z, m, sl2e, mrun, lrun, o, tid);
  const float l = quad_sum(lrun);
  if (!ok) return;
  const size_t p0 = ((size_t)z * N + q) * s;
  float M = mrun;
  for (int sl = 0; sl < s; ++sl) M = fmaxf(M, pml[(p0 + sl) * 2]);
  const float fl = exp2f(mrun - M);
  float L = l * fl;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[dt][j] *= fl;
  for (int sl = 0; sl < s; ++sl) {
    const float2 ml = *(const float2*)(pml + (p0 + sl) * 2);
    const float f = exp2f(ml.x - M);
    L += f * ml.y;
    const float* prow = pacc + (p0 + sl) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const float4 a = *(const float4*)(prow + 16 * dt + 4 * g);
      o[dt][0] += f * a.x;
      o[dt][1] += f * a.y;
      o[dt][2] += f * a.z;
      o[dt][3] += f * a.w;
    }
  }
  const float inv = 1.f / L;
  T* orow = out + ((size_t)z * N + q) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    store4<T>(orow + 16 * dt + 4 * g, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
}

template <typename T, int D>
static hipError_t gather_launch(const Plan& p, const void* Q, const void* K, const void* V, void* out, char* ws,
                                hipStream_t st) {
  const int Ns = p.N * p.s;
  const int nclear = (int)((p.ws.bcursor + (size_t)p.BH * p.m * 4 - p.ws.bcount) / 4);
  hipLaunchKernelGGL(clear_kernel, dim3(std::min(1024, (nclear + 255) / 256)), dim3(256), 0, st,
                     (uint32_t*)(ws + p.ws.bcount), nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 bgrid((Ns + 4095) / 4096, p.BH);
  hipLaunchKernelGGL(bucket_hist_kernel, bgrid, dim3(256), (size_t)p.m * 4, st, (const int32_t*)(ws + p.ws.E),
                     (uint32_t*)(ws + p.ws.bcount), Ns, p.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(p.BH), dim3(256), 0, st, (const uint32_t*)(ws + p.ws.bcount),
                     (uint32_t*)(ws + p.ws.boff), (uint32_t*)(ws + p.ws.toff), p.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_scatter_kernel, bgrid, dim3(256), (size_t)p.m * 8, st, (const int32_t*)(ws + p.ws.E),
                     (const uint32_t*)(ws + p.ws.boff), (uint32_t*)(ws + p.ws.bcursor), (int32_t*)(ws + p.ws.perm), Ns,
                     p.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const void* vtop = p.dtype == MITA_BF16 ? (const void*)(ws + p.ws.vt16) : (const void*)(ws + p.ws.vt32);
  const dim3 ggrid(p.max_tiles, p.BH);
  if (p.s == 1) {
    hipLaunchKernelGGL((gather_kernel<T, D, true>), ggrid, dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const int32_t*)(ws + p.ws.I), (const uint32_t*)(ws + p.ws.boff),
                       (const uint32_t*)(ws + p.ws.toff), (const int32_t*)(ws + p.ws.perm),
                       (const void*)(ws + p.ws.qtop), vtop, (T*)out, (float*)nullptr, (float*)nullptr, p.N, p.m, p.k,
                       p.s, sl2e);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gather_kernel<T, D, false>), ggrid, dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                     (const int32_t*)(ws + p.ws.I), (const uint32_t*)(ws + p.ws.boff), (const uint32_t*)(ws + p.ws.toff),
                     (const int32_t*)(ws + p.ws.perm), (const void*)(ws + p.ws.qtop), vtop, (T*)out,
                     (float*)(ws + p.ws.pacc), (float*)(ws + p.ws.pml), p.N, p.m, p.k, p.s, sl2e);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(p.qtiles, p.BH), dim3(256), 0, st, (const T*)Q,
                     (const void*)(ws + p.ws.qtop), vtop, (const float*)(ws + p.ws.pacc), (const float*)(ws + p.ws.pml),
                     (T*)out, p.N, p.m, p.s, sl2e);
  return hipGetLastError();
}

hipError_t launch_gather(const Plan& p, const void* Q, const void* K, const void* V, void* out, char* ws,
                         hipStream_t st) {
  if (p.dtype == MITA_BF16)
    return p.d == 64 ? gather_launch<uint16_t, 64>(p, Q, K, V, out, ws, st) : gather_launch<uint16_t, 128>(p, Q, K, V, out, ws, st);
  return p.d == 64 ? gather_launch<float, 64>(p, Q, K, V, out, ws, st) : gather_launch<float, 128>(p, Q, K, V, out, ws, st);
}

// Route-step counter block (queued-query count) is cleared before routing.
hipError_t launch_clear(const Plan& p, char* ws, hipStream_t st) {
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(256), 0, st, (uint32_t*)(ws + p.ws.counters), 64);
  return hipGetLastError();
}

}  // namespace mita
