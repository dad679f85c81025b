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

// bf16 with m > 64: 128 landmarks per workgroup, two 16-landmark column tiles per
// wave, so every staged key fragment feeds two MFMAs per Q~ plane and every value
// fragment two. Key/value blocks are staged by direct global-to-LDS loads into
// tiles swizzled for the score reads and the transposed value reads, double-
// buffered (a block's rows are requested while the previous block computes);
// the softmax keeps a lazily raised reference. Per landmark the MFMA sequence of
// the scores is that of landmark_kernel and of the candidate kernel, so the group
// maxima are the bits the candidates see.
constexpr int kLandmarkTileD = 128;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void landmarkd_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, const uint16_t* __restrict__ qtop,
    float* __restrict__ S, float* __restrict__ lpart, float* __restrict__ kmax, float* __restrict__ bmax, int N, int m,
    int lchunk, int nsplit, int gq, int nbg, int lm_tiles, int BH, float sl2e) {
  constexpr int QT = 2;
  using Sw = SwzTile<D>;
  // one shared object: with separate ones the compiler's LDS scopes would make the
  // next block's loads look like writes to the block being read
  __shared__ __align__(16) struct {
    uint16_t rk[2][Sw::TILE];
    uint16_t rv[2][Sw::TILE];
    float gmx[kLandmarkTileD][16];   // maxima of groups of 64: 16 blocks per landmark row
    float kred[4];
  } sm;
  int lt, c, z;
  if (!chunk_item(lm_tiles, nsplit, BH, lt, c, z)) return;   // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int k0 = c * lchunk, k1 = min(N, k0 + lchunk);
  const uint16_t* Kz = K + (size_t)z * N * D;
  const uint16_t* Vz = V + (size_t)z * N * D;
  // keys of this lane's rows of the block at kb (rows past the chunk's end repeat its last key)
  auto rows = [&](int kb, int (&id)[Sw::NI]) {
#pragma unroll
    for (int u = 0; u < Sw::NI; ++u) id[u] = min(kb + 16 * w + u * Sw::RPI + lane / Sw::CPR, k1 - 1);
  };
  {
    int id0[Sw::NI];
    rows(k0, id0);
    dma_rows<D>(sm.rk[0], sm.rv[0], Kz, Vz, id0, w, lane);
  }
  int lmc[QT];
  bool lm_ok[QT];
  uint4 qb[QT][2][D / 32];
  float mrun[QT], lrun[QT];
  f32x4 o[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int lm = lt * kLandmarkTileD + 32 * w + 16 * qt + r;
    lm_ok[qt] = lm < m;
    lmc[qt] = lm_ok[qt] ? lm : m - 1;   // padding lanes compute on a real landmark, never write
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qb[qt][p][ks] = ld16(qtop + ((size_t)(z * 2 + p) * m + lmc[qt]) * D + 32 * ks + 8 * g);
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float kmx = 0.f;
  const int nblk = (k1 - k0 + kKeyBlock - 1) / kKeyBlock;
  // Maxima of groups of 64 (one per block and landmark): a store per block would
  // put 4 bytes into a different row from each of 16 lanes, and lines would be
  // written back partly filled. Instead each wave keeps its rows' maxima of 16
  // blocks in LDS (rows 32 w .. 32 w + 31: no other wave touches them) and stores
  // them as 64 contiguous bytes per row (rows and groups 16-byte aligned).
  const bool gpack = gq == 64 && nbg % 4 == 0 && (k0 / kKeyBlock) % 16 == 0;
  auto gflush = [&](int blk_first, int nb16) {   // blocks blk_first .. + nb16 - 1 of the wave's 32 rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = 32 * w + 16 * h + (lane >> 2), q4 = lane & 3;   // row of the tile, its quarter
      const int lm = lt * kLandmarkTileD + rl;
      if (lm < m) {
        float* dst = bmax + ((size_t)z * m + lm) * nbg + blk_first + 4 * q4;
        const float* src = &sm.gmx[rl][4 * q4];
        if (nb16 == 16) {
          *(float4*)dst = *(const float4*)src;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (4 * q4 + u < nb16) dst[u] = src[u];
        }
      }
    }
  };
  for (int j = 0; j < nblk; ++j) {
    const int kb = k0 + j * kKeyBlock;
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
      if (D != 64 && lt == 0) {   // workgroup-uniform
        // squared key norms beside the scores: wave w re-reads the rows of its
        // key tile kt = w at the addresses the score reads use (no bank
        // conflicts), the four lanes of a row each a quarter of it
        float nsq = 0.f;
        qk2_bf16_swz<D, QT>(ck, qb, acc, lane, w, &nsq);
        nsq += __shfl_xor(nsq, 16, WAVE);
        nsq += __shfl_xor(nsq, 32, WAVE);
        kmx = fmaxf(kmx, nsq);
      } else {
        qk2_bf16_swz<D, QT>(ck, qb, acc, lane);
      }
      const int blk = kb / kKeyBlock;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {   // group maxima (and the scores when asked for) as the sweep writes them
        float* Brow = bmax + ((size_t)z * m + lmc[qt]) * nbg;
        float gk[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          gk[kt] = -INFINITY;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            gk[kt] = fmaxf(gk[kt], kb + 16 * kt + 4 * g + jj < k1 ? acc[qt][kt][jj] : -INFINITY);
        }
        if (gq == 4) {
          if (lm_ok[qt]) *(float4*)(Brow + 16 * blk + 4 * g) = make_float4(gk[0], gk[1], gk[2], gk[3]);
        } else {
          float gm = fmaxf(fmaxf(gk[0], gk[1]), fmaxf(gk[2], gk[3]));
          if (gq == 64) gm = quad_max(gm);
          if (gpack) {   // block-uniform
            if (g == 0) sm.gmx[32 * w + 16 * qt + r][j & 15] = gm;
          } else if (lm_ok[qt] && (gq == 16 || g == 0)) {
            Brow[gq == 16 ? 4 * blk + g : blk] = gm;
          }
        }
        if (S && lm_ok[qt]) {
          float* Srow = S + ((size_t)z * m + lmc[qt]) * N;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int key = kb + 16 * kt + 4 * g + jj;
              if (key < k1) Srow[key] = acc[qt][kt][jj];
            }
        }
      }
      lazy_softmax<D, QT>(acc, min(kKeyBlock, k1 - kb), sl2e, mrun, lrun, o, lane);
      pv_bf16_swz<D, QT>(cv, acc, o, lrun, lane);
      __builtin_amdgcn_s_setprio(0);
      if (D == 64 && lt == 0) {   // squared key norms (a row's 16-byte pieces in any order)
        // CH lanes read the CH pieces of a row (a half-wave reads contiguous rows:
        // no bank conflicts), NR rows per lane; the sums over the CH lanes first
        // trade half of a lane's rows with the partner lane, then add plainly.
        // Measured with d = 64: 6 % off the kernel against 4 threads per row, and
        // 10 % faster than the rows read beside the score products (the d = 128 form)
        constexpr int CH = D / 8, NR = D / 32, RS = 256 / CH;
        float sq[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const uint4 v = *(const uint4*)(ck + (tid / CH + RS * i) * D + 8 * (tid % CH));
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(wv[e] << 16), hi = __uint_as_float(wv[e] & 0xffff0000u);
            a = fmaf(lo, lo, a);
            a = fmaf(hi, hi, a);
          }
          sq[i] = a;
        }
        int b = CH / 2;
#pragma unroll
        for (int h = NR / 2; h >= 1; h >>= 1, b >>= 1) {
          const bool up = lane & b;
#pragma unroll
          for (int i = 0; i < h; ++i) {
            const float send = up ? sq[i] : sq[i + h], keep = up ? sq[i + h] : sq[i];
            sq[i] = keep + __shfl_xor(send, b, WAVE);
          }
        }
#pragma unroll
        for (; b >= 1; b >>= 1) sq[0] += __shfl_xor(sq[0], b, WAVE);
        kmx = fmaxf(kmx, sq[0]);
      }
    };
    step(sm.rk[(j + 1) & 1], sm.rv[(j + 1) & 1], sm.rk[j & 1], sm.rv[j & 1]);
    if (gpack && ((j & 15) == 15 || j == nblk - 1))   // block-uniform: a group of 16 blocks, or the chunk, ends
      gflush(k0 / kKeyBlock + (j & ~15), (j & 15) + 1);
  }
  if (lt == 0) {
    kmx = wave_max(kmx);
    if (lane == 0) sm.kred[w] = kmx;
    __syncthreads();
    if (tid == 0) {
      const float mx = fmaxf(fmaxf(sm.kred[0], sm.kred[1]), fmaxf(sm.kred[2], sm.kred[3]));
      kmax[(size_t)z * nsplit + c] = sqrtf(mx) * 1.0001f + 1e-30f;
    }
  }
  // partial softmax of this chunk: [reference, sum, pad, pad, acc[D]] per landmark
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = quad_sum(lrun[qt]);
    if (lm_ok[qt]) {
      float* P = lpart + (((size_t)z * m + lmc[qt]) * nsplit + c) * (D + 4);
      if (g == 0) *(float2*)P = make_float2(mrun[qt], l);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *(float4*)(P + 4 + 16 * dt + 4 * g) = make_float4(o[qt][dt][0], o[qt][dt][1], o[qt][dt][2], o[qt][dt][3]);
    }
  }
}

template <typename T, int D>
static hipError_t landmark_launch(const Plan& p, const void* K, const void* V, char* ws, float* S_out,
                                  hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  if (sizeof(T) == 2 && p.m > kLandmarkTile) {   // bf16, several landmark tiles: the direct-load kernel
    const int tiles = (p.m + kLandmarkTileD - 1) / kLandmarkTileD;
    const int grid = 8 * ((p.nsplit * p.BH + 7) / 8) * tiles;   // see chunk_item
    hipLaunchKernelGGL((landmarkd_kernel<D>), dim3(grid), dim3(256), 0, st, (const uint16_t*)K, (const uint16_t*)V,
                       (const uint16_t*)(ws + p.ws.qtop), S_out, (float*)(ws + p.ws.lpart), (float*)(ws + p.ws.kmax),
                       (float*)(ws + p.ws.bmax), p.N, p.m, p.lchunk, p.nsplit, p.gq, p.nbg, tiles, p.BH, sl2e);
  } else {
    const int grid = 8 * ((p.nsplit * p.BH + 7) / 8) * p.lm_tiles;   // see chunk_item
    hipLaunchKernelGGL((landmark_kernel<T, D>), dim3(grid), dim3(256), 0, st, (const T*)K, (const T*)V,
                       (const void*)(ws + p.ws.qtop), S_out, (float*)(ws + p.ws.lpart), (float*)(ws + p.ws.kmax),
                       (float*)(ws + p.ws.bmax), p.N, p.m, p.lchunk, p.nsplit, p.gq, p.nbg, p.lm_tiles, p.BH, sl2e);
  }
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
