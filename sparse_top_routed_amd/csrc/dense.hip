// Full softmax attention, O = softmax(Q K^T / sqrt d) V over all N keys of a
// (batch, head) slice: the quadratic standard attention whose cost MiTA avoids
// (MiTA pages: the introduction and problem statement on standard attention's
// O(N^2) cost; every speed figure the pages give is relative to it). Not a step
// of MiTA: a comparator on the same inputs, for measuring the speed-up.
//
// Flash-style: a workgroup takes consecutive queries of one slice and streams
// the slice's keys and values through LDS 64 at a time with an online softmax;
// scores and probabilities stay in registers. fp32 (dense_kernel): 64 queries,
// 16 per wave, the next block fetched into registers while the current one
// computes. bf16 (densed_kernel): the routed-expert kernel's inner loop, below.
// Each XCD takes a contiguous run of the (slice, query tile) items, so the
// workgroups reading one slice's keys and values share that XCD's L2
// (workgroups are dealt round-robin over the 8 XCDs).
#include "attn_core.h"

namespace mita {

template <typename T, int D>
__global__ __launch_bounds__(256) void dense_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, T* __restrict__ out, int N, int qtiles,
                                                    int BH, float sl2e) {
  __shared__ AttnLds<T, D> sm;
  // workgroup b runs on XCD b % 8; the 8 XCDs each take a contiguous run of the
  // (slice, query tile) items, so the workgroups of one slice meet in one L2
  const long items = (long)qtiles * BH, per = (items + 7) / 8;
  const long it = (long)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (it >= items) return;   // workgroup-uniform
  const int z = (int)(it / qtiles), qt = (int)(it % qtiles);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int q = 64 * qt + 16 * w + r;
  const bool wave_live = 64 * qt + 16 * w < N;
  const T* Kz = K + (size_t)z * N * D;
  const T* Vz = V + (size_t)z * N * D;
  QFrag<T, D> qf;
  qf.load(Q + ((size_t)z * N + min(q, N - 1)) * D, g);
  KVRegs<T, D, 1> R;
  auto fetch = [&](int kb) {   // block-uniform
    const int live = min(kKeyBlock, N - kb);
    R.k[0].load([&](int rr) { return Kz + (size_t)(kb + rr) * D; }, live, tid);
    R.v.load([&](int rr) { return Vz + (size_t)(kb + rr) * D; }, live, tid);
  };
  fetch(0);
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < N; kb += kKeyBlock) {
    R.store(sm, tid);
    __syncthreads();
    if (kb + kKeyBlock < N) fetch(kb + kKeyBlock);
    attend_block<T, D, 1>(sm, qf, min(kKeyBlock, N - kb), sl2e, mrun, lrun, o, lane, wave_live);
    __syncthreads();
  }
  const float inv = 1.f / quad_sum(lrun);
  if (q < N) {
    T* orow = out + ((size_t)z * N + q) * D;
    store_row<T, D>(orow, o, inv, g);
  }
}

// bf16: 128 queries per workgroup, four waves of two 16-query column tiles (so
// every staged key or value fragment feeds two MFMAs); key/value blocks of 64
// rows by direct global-to-LDS loads into tiles swizzled for the score reads and
// the transposed value reads, double-buffered (the next block is requested while
// one computes); the lazily raised softmax reference of the routed-expert kernel.
// Same XCD mapping as dense_kernel.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void densed_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ out, int N, int qtiles, int BH, float sl2e) {
  constexpr int QT = 2;
  using Sw = SwzTile<D>;
  // one shared object: with separate ones the compiler's LDS scopes would make the
  // next block's loads look like writes to the block being read
  __shared__ __align__(16) struct {
    uint16_t rk[2][Sw::TILE];
    uint16_t rv[2][Sw::TILE];
  } sm;
  const long items = (long)qtiles * BH, per = (items + 7) / 8;
  const long it = (long)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (it >= items) return;   // workgroup-uniform
  const int z = (int)(it / qtiles), qtile = (int)(it % qtiles);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const uint16_t* Kz = K + (size_t)z * N * D;
  const uint16_t* Vz = V + (size_t)z * N * D;
  // keys of this lane's rows of the block at kb (rows past N repeat the last key)
  auto rows = [&](int kb, int (&id)[Sw::NI]) {
#pragma unroll
    for (int u = 0; u < Sw::NI; ++u) id[u] = min(kb + 16 * w + u * Sw::RPI + lane / Sw::CPR, N - 1);
  };
  {
    int id0[Sw::NI];
    rows(0, id0);
    dma_rows<D>(sm.rk[0], sm.rv[0], Kz, Vz, id0, w, lane);
  }
  const int q0 = 128 * qtile + 32 * w;   // query of column tile qt: q0 + 16 qt + r
  uint4 qf[QT][D / 32];
  float mrun[QT], lrun[QT];
  f32x4 o[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const uint16_t* qrow = Q + ((size_t)z * N + min(q0 + 16 * qt + r, N - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[qt][ks] = ld16(qrow + 32 * ks + 8 * g);
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nblk = (N + kKeyBlock - 1) / kKeyBlock;
  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kKeyBlock;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // block j staged; every wave done with block j - 1
    // the next block's loads and this block's reads go through distinct __restrict__
    // parameters, so the compiler does not wait for the loads before the reads
    auto step = [&](uint16_t* __restrict__ nk, uint16_t* __restrict__ nv, const uint16_t* __restrict__ ck,
                    const uint16_t* __restrict__ cv) __attribute__((always_inline)) {
      if (j + 1 < nblk) {   // block-uniform
        int idn[Sw::NI];
        rows(kb + kKeyBlock, idn);
        dma_rows<D>(nk, nv, Kz, Vz, idn, w, lane);
      }
      f32x4 acc[QT][4];
      __builtin_amdgcn_s_setprio(1);
      qk_bf16_swz<D, QT>(ck, qf, acc, lane);
      lazy_softmax<D, QT>(acc, min(kKeyBlock, N - kb), sl2e, mrun, lrun, o, lane);
      pv_bf16_swz<D, QT>(cv, acc, o, lrun, lane);
      __builtin_amdgcn_s_setprio(0);
    };
    step(sm.rk[(j + 1) & 1], sm.rv[(j + 1) & 1], sm.rk[j & 1], sm.rv[j & 1]);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 16 * qt + r;
    const float inv = 1.f / quad_sum(lrun[qt]);
    if (q < N) store_row<uint16_t, D>(out + ((size_t)z * N + q) * D, o[qt], inv, g);
  }
}

template <typename T, int D>
static hipError_t dense_launch(const void* Q, const void* K, const void* V, void* out, int BH, int N,
                               hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  if constexpr (sizeof(T) == 2) {
    const int qtiles = (N + 127) / 128;
    const long grid = 8 * (((long)qtiles * BH + 7) / 8);
    hipLaunchKernelGGL((densed_kernel<D>), dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)Q,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)out, N, qtiles, BH, sl2e);
  } else {
    const int qtiles = (N + 63) / 64;
    const long grid = 8 * (((long)qtiles * BH + 7) / 8);
    hipLaunchKernelGGL((dense_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)Q, (const T*)K,
                       (const T*)V, (T*)out, N, qtiles, BH, sl2e);
  }
  return hipGetLastError();
}

hipError_t launch_dense(int dtype, int d, int BH, int N, const void* Q, const void* K, const void* V, void* out,
                        hipStream_t st) {
  if (dtype == MITA_BF16)
    return d == 64 ? dense_launch<uint16_t, 64>(Q, K, V, out, BH, N, st)
                   : dense_launch<uint16_t, 128>(Q, K, V, out, BH, N, st);
  return d == 64 ? dense_launch<float, 64>(Q, K, V, out, BH, N, st) : dense_launch<float, 128>(Q, K, V, out, BH, N, st);
}

}  // namespace mita
