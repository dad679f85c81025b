// Step 2: the shared expert V~ = softmax(Q~ K^T / sqrt d) V and the score rows
// q~_i . K_n that step 3 ranks (compression step of the MiTA summaries: the
// landmark queries attend over all keys and values; the same activations pick
// the deformable experts, so one pass produces both).
//
// Flash-style: a workgroup takes 64 landmarks (16 per wave) and one chunk of
// keys (the workgroups sharing a chunk are placed on one XCD), streams the chunk through LDS 64 keys at a time (the next block is
// fetched into registers while the current one computes) and keeps an online
// softmax. A second kernel merges the chunks' partial softmaxes into V~ (and,
// from the group maxima below, sets step 3's candidate thresholds). The
// scores themselves do not go to memory: only maxima of groups of 16 (one
// lane's share of a block) or 64 (a block) per landmark, from which step 3 sets
// a threshold that its candidates must reach (written out in full only on
// request, for checking).
// bf16 inputs: Q~ enters the MFMA as two bf16 parts (hi + lo) so the scores
// carry ~16 more bits than a bf16 Q~ would; fp32 inputs use the fp32 MFMA.
// The workgroups of landmark tile 0 also record max_n |K_n|_2 per chunk, which
// bounds the score error for the exact top-k of step 3.
#include "sweep.h"

namespace mita {

template <typename T, int D>
__global__ __launch_bounds__(256) void landmark_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                       const void* __restrict__ qtop, float* __restrict__ S,
                                                       float* __restrict__ lpart, float* __restrict__ kmax,
                                                       float* __restrict__ bmax, int N, int m, int lchunk, int nsplit,
                                                       int gq, int nbg, int lm_tiles, int BH, float sl2e) {
  using TL = Tiles<T, D>;
  __shared__ __align__(16) T Ks[TL::KTILE];
  __shared__ __align__(16) T Vs[TL::VTILE];
  __shared__ float kred[4];
  int lt, c, z;
  if (!chunk_item(lm_tiles, nsplit, BH, lt, c, z)) return;   // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int lm = lt * kLandmarkTile + 16 * w + r;
  const bool lm_ok = lm < m;
  const int lmc = lm_ok ? lm : m - 1;   // padding lanes compute on a real landmark, never write
  const int k0 = c * lchunk, k1 = min(N, k0 + lchunk);

  LmFrag<T, D> qfr;
  qfr.load(qtop, z, m, lmc, g);
  LmState<D> st;
  st.init();
  float kmx = 0.f;
  float* Srow = S ? S + ((size_t)z * m + lmc) * N : nullptr;
  float* Brow = bmax + ((size_t)z * m + lmc) * nbg;
  shared_expert_sweep<T, D>(K + (size_t)z * N * D, V + (size_t)z * N * D, k0, k1, qfr, Ks, Vs, lt == 0, kmx, Brow,
                            gq, Srow, (N & 3) == 0, lm_ok, sl2e, st, tid);

  if (lt == 0) {
    kmx = wave_max(kmx);
    if (lane == 0) kred[w] = kmx;
    __syncthreads();
    if (tid == 0) {
      const float mx = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
      kmax[(size_t)z * nsplit + c] = sqrtf(mx) * 1.0001f + 1e-30f;
    }
  }
  // partial softmax of this chunk: [max, sum, pad, pad, acc[D]] per landmark
  const float lrun = quad_sum(st.lrun);
  if (lm_ok) {
    float* P = lpart + (((size_t)z * m + lm) * nsplit + c) * (D + 4);
    if (g == 0) *(float2*)P = make_float2(st.mrun, lrun);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *(float4*)(P + 4 + 16 * dt + 4 * g) = make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
  }
}

template <typename T, int D>
static hipError_t landmark_launch(const Plan& p, const void* K, const void* V, char* ws, float* S_out,
                                  hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const int grid = 8 * ((p.nsplit * p.BH + 7) / 8) * p.lm_tiles;   // see chunk_item
  hipLaunchKernelGGL((landmark_kernel<T, D>), dim3(grid), dim3(256), 0, st, (const T*)K, (const T*)V,
                     (const void*)(ws + p.ws.qtop), S_out, (float*)(ws + p.ws.lpart), (float*)(ws + p.ws.kmax),
                     (float*)(ws + p.ws.bmax), p.N, p.m, p.lchunk, p.nsplit, p.gq, p.nbg, p.lm_tiles, p.BH, sl2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the chunks' partial softmaxes merged into V~, and the candidate thresholds of
  // step 3 from the group maxima (merge_thresh_kernel, with the top-k kernels)
  return launch_merge_thresh(p, ws, st);
}

hipError_t launch_landmark(const Plan& p, const void* K, const void* V, char* ws, float* S_out, hipStream_t st) {
  if (p.dtype == MITA_BF16)
    return p.d == 64 ? landmark_launch<uint16_t, 64>(p, K, V, ws, S_out, st)
                     : landmark_launch<uint16_t, 128>(p, K, V, ws, S_out, st);
  return p.d == 64 ? landmark_launch<float, 64>(p, K, V, ws, S_out, st) : landmark_launch<float, 128>(p, K, V, ws, S_out, st);
}

}  // namespace mita
