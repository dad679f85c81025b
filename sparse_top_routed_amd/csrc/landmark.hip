// Step 2: the shared expert V~ = softmax(Q~ K^T / sqrt d) V and the score rows
// q~_i . K_n that step 3 ranks (compression step of the MiTA summaries: the
// landmark queries attend over all keys and values; the same activations pick
// the deformable experts, so one pass produces both).
//
// Flash-style: a workgroup takes 64 landmarks (16 per wave) and one chunk of
// keys, streams the chunk through LDS 64 keys at a time, writes the unscaled
// scores, and keeps an online softmax. Chunks are merged by a second kernel.
// bf16 inputs: Q~ enters the MFMA as two bf16 parts (hi + lo) so the scores
// carry ~16 more bits than a bf16 Q~ would; fp32 inputs use the fp32 MFMA.
// The workgroups of landmark tile 0 also record max_n |K_n|_2 per chunk, which
// bounds the score error for the exact top-k of step 3.
#include "attn_core.h"

namespace mita {

template <typename T, int D>
__global__ __launch_bounds__(256) void landmark_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                       const void* __restrict__ qtop, float* __restrict__ S,
                                                       float* __restrict__ lpart, float* __restrict__ kmax, int N,
                                                       int m, int lchunk, int nsplit, float sl2e) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  __shared__ __align__(16) T Ks[TL::KTILE];
  __shared__ __align__(16) T Vs[TL::VTILE];
  __shared__ float kred[4];
  const int lt = blockIdx.x, c = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int lm = lt * kLandmarkTile + 16 * w + r;
  const bool lm_ok = lm < m;
  const int lmc = lm_ok ? lm : m - 1;   // padding lanes compute on a real landmark, never write
  const int k0 = c * lchunk, k1 = min(N, k0 + lchunk);
  const T* Kz = K + (size_t)z * N * D;
  const T* Vz = V + (size_t)z * N * D;

  uint4 qb[2][D / 32];
  float qf[D / 4];
  if constexpr (BF) {
    const uint16_t* qt = (const uint16_t*)qtop;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qb[p][ks] = *(const uint4*)(qt + ((size_t)(z * 2 + p) * m + lmc) * D + 32 * ks + 8 * g);
  } else {
    const float* qt = (const float*)qtop;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) qf[ks] = qt[((size_t)z * m + lmc) * D + 4 * ks + g];
  }

  float mrun = -INFINITY, lrun = 0.f, kmx = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* Srow = S + ((size_t)z * m + (lm_ok ? lm : 0)) * N;
  const bool vec_store = (N & 3) == 0;

  for (int kb = k0; kb < k1; kb += kKeyBlock) {
    const int nvalid = min(kKeyBlock, k1 - kb);
    auto krow = [&](int rr) { return Kz + (size_t)(kb + rr) * D; };
    auto vrow = [&](int rr) { return Vz + (size_t)(kb + rr) * D; };
    stage_rows<T, D>(Ks, TL::KSTR, krow, nvalid, tid);
    if constexpr (BF)
      stage_vt_bf16<D>((uint16_t*)Vs, vrow, nvalid, tid);
    else
      stage_rows<T, D>(Vs, TL::VSTR, vrow, nvalid, tid);
    __syncthreads();

    if (lt == 0) {  // squared norms of the staged keys: 4 threads per row
      const int row = tid >> 2, part = tid & 3;
      const T* kr = Ks + row * TL::KSTR + part * (D / 4);
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < D / 4; ++e) {
        float x;
        if constexpr (BF) x = bf16_to_f32(kr[e]); else x = kr[e];
        sq = fmaf(x, x, sq);
      }
      sq += __shfl_xor(sq, 1, WAVE);
      sq += __shfl_xor(sq, 2, WAVE);
      kmx = fmaxf(kmx, sq);
    }

    f32x4 acc[4];
    if constexpr (BF)
      qk_bf16<D, 1, 2>((const uint16_t*)Ks, nullptr, qb, acc, lane);
    else
      qk_f32<D>((const float*)Ks, qf, acc, lane);

    if (lm_ok) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int key = kb + 16 * kt + 4 * g;
        if (vec_store && key + 3 < k1) {
          *(float4*)(Srow + key) = make_float4(acc[kt][0], acc[kt][1], acc[kt][2], acc[kt][3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key + j < k1) Srow[key + j] = acc[kt][j];
        }
      }
    }
    const float alpha = online_softmax(acc, nvalid, sl2e, mrun, lrun, lane);
    rescale<D>(o, alpha);
    if constexpr (BF)
      pv_bf16<D>((const uint16_t*)Vs, acc, o, lane);
    else
      pv_f32<D>((const float*)Vs, acc, o, lane);
    __syncthreads();
  }

  if (lt == 0) {
    kmx = wave_max(kmx);
    if (lane == 0) kred[w] = kmx;
    __syncthreads();
    if (tid == 0) {
      const float mx = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
      kmax[(size_t)z * nsplit + c] = sqrtf(mx) * 1.0001f + 1e-30f;
    }
  }
  lrun = quad_sum(lrun);
  if (lm_ok) {
    float* P = lpart + (((size_t)z * m + lm) * nsplit + c) * (D + 2);
    if (g == 0) {
      P[0] = mrun;
      P[1] = lrun;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) P[2 + 16 * dt + 4 * g + j] = o[dt][j];
  }
}

// Merge the per-chunk partial softmaxes of each landmark: one wave per row.
template <int D>
__global__ __launch_bounds__(256) void landmark_merge_kernel(const float* __restrict__ lpart, float* __restrict__ vt32,
                                                             uint16_t* __restrict__ vt16, int rows, int nsplit) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* P = lpart + (size_t)row * nsplit * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < nsplit; ++c) M = fmaxf(M, P[(size_t)c * (D + 2)]);
  float L = 0.f, acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int c = 0; c < nsplit; ++c) {
    const float* Pc = P + (size_t)c * (D + 2);
    const float f = exp2f(Pc[0] - M);
    L += f * Pc[1];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] += f * Pc[2 + lane + 64 * e];
  }
#pragma unroll
  for (int e = 0; e < D / 64; ++e) {
    const float v = acc[e] / L;
    vt32[(size_t)row * D + lane + 64 * e] = v;
    vt16[(size_t)row * D + lane + 64 * e] = f32_to_bf16(v);
  }
}

template <typename T, int D>
static hipError_t landmark_launch(const Plan& p, const void* K, const void* V, char* ws, hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  dim3 grid(p.lm_tiles, p.nsplit, p.BH);
  hipLaunchKernelGGL((landmark_kernel<T, D>), grid, dim3(256), 0, st, (const T*)K, (const T*)V,
                     (const void*)(ws + p.ws.qtop), (float*)(ws + p.ws.S), (float*)(ws + p.ws.lpart),
                     (float*)(ws + p.ws.kmax), p.N, p.m, p.lchunk, p.nsplit, sl2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.BH * p.m;
  hipLaunchKernelGGL((landmark_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, st,
                     (const float*)(ws + p.ws.lpart), (float*)(ws + p.ws.vt32), (uint16_t*)(ws + p.ws.vt16), rows,
                     p.nsplit);
  return hipGetLastError();
}

hipError_t launch_landmark(const Plan& p, const void* K, const void* V, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16)
    return p.d == 64 ? landmark_launch<uint16_t, 64>(p, K, V, ws, st) : landmark_launch<uint16_t, 128>(p, K, V, ws, st);
  return p.d == 64 ? landmark_launch<float, 64>(p, K, V, ws, st) : landmark_launch<float, 128>(p, K, V, ws, st);
}

}  // namespace mita
