// Full softmax attention, O = softmax(Q K^T / sqrt d) V over all N keys of a
// (batch, head) slice: the quadratic standard attention whose cost MiTA avoids
// (MiTA pages: the introduction and problem statement on standard attention's
// O(N^2) cost; every speed figure the pages give is relative to it). Not a step
// of MiTA: a comparator on the same inputs, for measuring the speed-up.
//
// Flash-style: a workgroup takes 64 consecutive queries of one slice (16 per
// wave) and streams the slice's keys and values through LDS 64 at a time (the
// next block is fetched into registers while the current one computes) with
// an online softmax; scores and probabilities stay in registers. Same MFMA
// tiles as the output step. Each XCD takes a contiguous run of the (slice,
// query tile) items, so the workgroups reading one slice's keys and values
// share that XCD's L2 (workgroups are dealt round-robin over the 8 XCDs).
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

template <typename T, int D>
static hipError_t dense_launch(const void* Q, const void* K, const void* V, void* out, int BH, int N,
                               hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const int qtiles = (N + 63) / 64;
  const long items = (long)qtiles * BH;
  const long grid = 8 * ((items + 7) / 8);
  hipLaunchKernelGGL((dense_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)Q, (const T*)K,
                     (const T*)V, (T*)out, N, qtiles, BH, sl2e);
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
