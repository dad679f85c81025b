// Step 3: deformable experts. I_i = the k tokens with the largest q~_i . K_n
// (deformable experts of the MiTA summaries: top-k activations of K^T q~_i over
// the whole sequence, ties to the lower index here, ids listed ascending).
//
// The score rows never go to memory. Step 2 leaves, per row, the maxima of
// groups of 16 or 64 approximate scores; every group maximum is itself a score,
// so the k-th largest of them, tau, is a lower bound of the row's k-th largest
// approximate score T. Then:
//   1. threshold (at the end of step 2, with the shared-expert merge): tau per
//      row by a bit search over the group maxima; the candidate threshold is
//      tau - 2E (E_i = gamma |q~_i| max|K|, the proven bound on an approximate
//      score's error), rounded down;
//   2. candidate kernel: recomputes the approximate scores exactly as step 2 did
//      (same MFMA sequence on the same operands, so the same bits) and writes
//      every score at or above the threshold, with its token id, in index
//      order, to a list per (row, key chunk);
//   3. select kernel, one wave per row: T is the k-th largest candidate score;
//      scores above T + 2E are in, below T - 2E out, and the band between is
//      re-scored in fp64 from Q~ (fp64) and K and cut by (fp64 score, lower id);
//   4. rows whose lists overflow (massive ties) take an exact fallback: fp64
//      scores of the whole row and an 8-bit radix select on their order keys.
// Every token that could be in the exact top-k is a candidate: anything within
// 2E of T is at least tau - 2E.
#include "sweep.h"

namespace mita {

constexpr int kCandListMax = 1024;   // blocks of a key chunk the candidate kernel lists (more: no skipping)
constexpr int kBandMax = 128;   // band members the select kernel re-scores in LDS (more: fallback; a band
                                 // normally holds a few members, and LDS per wave sets the occupancy)

__device__ __forceinline__ float round_down_f32(double x) {
  float f = (float)x;
  if ((double)f > x) f = nextafterf(f, -INFINITY);
  return f;
}
__device__ __forceinline__ float round_up_f32(double x) {
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, INFINITY);
  return f;
}

__device__ __forceinline__ uint32_t ballot_count(bool p) { return (uint32_t)__popcll(__ballot(p)); }
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Error bound of row `row`'s approximate scores (all lanes active).
__device__ __forceinline__ double row_bound(const float* qtnorm, const float* kmax, int nsplit, int row, int z,
                                            double gamma, int lane) {
  float kmx = 0.f;
  for (int c = lane; c < nsplit; c += 64) kmx = fmaxf(kmx, kmax[(size_t)z * nsplit + c]);
  return gamma * (double)qtnorm[row] * (double)wave_max(kmx);
}

// fp64 dot product of a landmark query (fp64) with one key row, by one lane; the
// key row is fetched in 16-byte pieces that are all in flight together.
template <typename T, int D>
__device__ __forceinline__ double dot64_row(const double* __restrict__ q, const T* __restrict__ kr) {
  constexpr int EPC = 16 / sizeof(T);
  uint4 kc[D / EPC];
#pragma unroll
  for (int c = 0; c < D / EPC; ++c) kc[c] = ld16(kr + c * EPC);
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < D / EPC; ++c) {
    if constexpr (sizeof(T) == 2) {
      const uint16_t* h = (const uint16_t*)&kc[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fma(q[8 * c + e], (double)bf16_to_f32(h[e]), s);
    } else {
      const float* f = (const float*)&kc[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fma(q[4 * c + e], (double)f[e], s);
    }
  }
  return s;
}

__device__ __forceinline__ void band_keys(double Tf, double E, uint32_t& hiKey, uint32_t& loKey) {
  hiKey = (Tf + 2.0 * E < INFINITY) ? f32_key(round_up_f32(Tf + 2.0 * E)) : 0xFFFFFFFFu;
  loKey = (Tf - 2.0 * E > -INFINITY) ? max(1u, f32_key(round_down_f32(Tf - 2.0 * E))) : 1u;
}

// The k-th largest of a wave's order keys (lane's keys in v[0..ns), 0 = absent;
// at least k present), by a bit search from the top: the largest P with at
// least k keys >= P. Every present key lies between the wave's smallest and
// largest, so the bits those two share are settled at once. With lowbit > 0
// the bits below lowbit stay 0: the result is then a lower bound of the k-th
// largest key that differs from it only in those bits.
template <int PV>
__device__ __forceinline__ uint32_t kth_largest_key(const uint32_t (&v)[PV], int ns, uint32_t k, int lowbit) {
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int p = 0; p < PV; ++p)
    if (p < ns) {
      hi = max(hi, v[p]);
      lo = min(lo, v[p] ? v[p] : 0xFFFFFFFFu);
    }
  hi = wave_max_uniform(hi);
  lo = wave_min_uniform(lo);
  const uint32_t low_mask = (1u << lowbit) - 1u;
  if (hi == lo) return hi & ~low_mask;
  const int top = 31 - __builtin_clz(hi ^ lo);   // highest bit where the keys can differ
  uint32_t pfx = top == 31 ? 0u : hi & ~((2u << top) - 1u);
  for (int b = top; b >= lowbit; --b) {
    const uint32_t cand = pfx | (1u << b);
    uint32_t c = 0;
#pragma unroll
    for (int p = 0; p < PV; ++p)
      if (p < ns) c += ballot_count(v[p] >= cand);
    if (c >= k) pfx = cand;
  }
  return pfx;
}

// ---------------------------------------------------------------- 1. threshold
// Candidate threshold of one row (as an order key; 0: none, every score is a
// candidate) from its nbg group maxima, lane l holding maxima l, 64 + l, ...
// (order keys, 0 past nbg): tau = the k-th largest maximum by a bit search
// (ballots: one compare per register, the counting on the scalar unit) that
// leaves the 12 lowest key bits at 0 (a lower bound of it, within 2^-11 of it
// relative: the threshold only has to be low enough), then tau - 2E rounded
// down.
template <int PV>
__device__ __forceinline__ uint32_t thresh_key(const uint32_t (&v)[PV], int nbg, int k, double E) {
  uint32_t key = 0u;
  if (nbg >= k) {
    const uint32_t pfx = kth_largest_key<PV>(v, PV, (uint32_t)k, 12);
    const float tau = key_f32(pfx);
    if (tau > -INFINITY && tau < INFINITY) {
      const double t = (double)tau - 2.0 * E;
      key = t > -INFINITY ? max(1u, f32_key(round_down_f32(t))) : 0u;
    }
  }
  return key;
}

// Loads a row's group maxima as order keys (lane l: maxima l, 64 + l, ...).
template <int PV>
__device__ __forceinline__ void load_group_keys(const float* br, int nbg, int lane, uint32_t (&v)[PV]) {
#pragma unroll
  for (int p = 0; p < PV; ++p) {
    const int i = 64 * p + lane;
    const float x = br[max(0, min(i, nbg - 1))];   // nbg = 0: no threshold, the load stays in bounds
    v[p] = i < nbg ? f32_key(x) : 0u;
  }
}

// End of step 2 and start of step 3, one wave per score row (four rows per
// workgroup): the chunks' partial softmaxes of landmark i are merged into V~_i
// (lane l: columns l, l + 64, ...), and the row's candidate threshold is set
// from its group maxima (at most 64 PV, in registers). Merging here, where each
// row's maxima are read anyway, saves a launch between the two steps. CB chunks'
// partials are loaded at once: 8, or 4 when there are at most 4 chunks (fewer
// clamped duplicate loads when nsplit < 8, none when nsplit = 4; 4 us less on the
// ViT-B-like forward, which has 3 chunks).
template <int D, int PV, int CB>
__global__ __launch_bounds__(256) void merge_thresh_kernel(const float* __restrict__ lpart,
                                                           float* __restrict__ vt32, uint16_t* __restrict__ vt16,
                                                           const float* __restrict__ bmax,
                                                           const float* __restrict__ qtnorm,
                                                           const float* __restrict__ kmax, int nsplit,
                                                           uint32_t* __restrict__ thr, int nbg, int m, int k,
                                                           double gamma, int rows, float* __restrict__ lse_se) {
  constexpr int CW = D / 64;
  const int tid = threadIdx.x, lane = tid & 63, row = blockIdx.x * 4 + (tid >> 6);
  if (row >= rows) return;   // wave-uniform
  const int z = row / m;
  // every independent load first: the group maxima, the error-bound inputs and
  // the first chunks' partials [max, sum, pad, pad, acc[D]]
  uint32_t v[PV];
  load_group_keys<PV>(bmax + (size_t)row * nbg, nbg, lane, v);
  float kmx = 0.f;
  for (int c = lane; c < nsplit; c += 64) kmx = fmaxf(kmx, kmax[(size_t)z * nsplit + c]);
  const float qn = qtnorm[row];
  const float* Pr = lpart + (size_t)row * nsplit * (D + 4);
  float2 ml[CB];
  float a[CB][CW];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float* Pc = Pr + (size_t)min(c0 + u, nsplit - 1) * (D + 4);
      ml[u] = *(const float2*)Pc;
#pragma unroll
      for (int e = 0; e < CW; ++e) a[u][e] = Pc[4 + lane + 64 * e];
    }
  };
  fetch(0);
  float M = -INFINITY;
  for (int c = lane; c < nsplit; c += 64) M = fmaxf(M, Pr[(size_t)c * (D + 4)]);
  M = wave_max(M);
  float L = 0.f, acc[CW];
#pragma unroll
  for (int e = 0; e < CW; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += CB) {
    if (c0 > 0) fetch(c0);
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (c0 + u < nsplit) {
        const float f = __builtin_amdgcn_exp2f(ml[u].x - M);
        L = fmaf(f, ml[u].y, L);
#pragma unroll
        for (int e = 0; e < CW; ++e) acc[e] = fmaf(f, a[u][e], acc[e]);
      }
    }
  }
  const float inv = 1.f / L;
  if (lane == 0) lse_se[row] = M + log2f(L);
#pragma unroll
  for (int e = 0; e < CW; ++e) {
    const float x = acc[e] * inv;
    vt32[(size_t)row * D + lane + 64 * e] = x;
    vt16[(size_t)row * D + lane + 64 * e] = f32_to_bf16(x);
  }

  const double E = gamma * (double)qn * (double)wave_max(kmx);
  const uint32_t key = thresh_key<PV>(v, nbg, k, E);
  if (lane == 0) thr[row] = key;
}

// ---------------------------------------------------------------- 2. candidates
// Same workgroup shape and MFMA sequence as the shared-expert kernel (64
// landmarks x one key chunk, 16 landmarks per wave), K only.
template <typename T, int D>
__global__ __launch_bounds__(256) void topk_cand_kernel(const T* __restrict__ K, const void* __restrict__ qtop,
                                                        const uint32_t* __restrict__ thr, uint2* __restrict__ cand,
                                                        uint32_t* __restrict__ ccnt, uint32_t* __restrict__ glist,
                                                        int N, int m, int lchunk, int nsplit, int capc, int lm_tiles,
                                                        int BH) {
  using TL = Tiles<T, D>;
  __shared__ __align__(16) T Ks[TL::KTILE];
  if (blockIdx.x == 0 && threadIdx.x == 0) glist[0] = 0u;   // no fallback rows yet (the select kernel adds them)
  int lt, c, z;
  if (!chunk_item(lm_tiles, nsplit, BH, lt, c, z)) return;   // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int lm = lt * kLandmarkTile + 16 * w + r;
  const bool lm_ok = lm < m;
  const int lmc = lm_ok ? lm : m - 1;
  const int k0 = c * lchunk, k1 = min(N, k0 + lchunk);
  const size_t row = (size_t)z * m + lmc;
  LmFrag<T, D> qfr;
  qfr.load(qtop, z, m, lmc, g);
  const uint32_t tk = thr[row];
  const float tf = tk ? key_f32(tk) : -INFINITY;   // compare the scores themselves (same order)
  uint32_t base = 0;
  candidate_sweep<T, D>(K + (size_t)z * N * D, k0, k1, qfr, Ks, tf, cand + (row * nsplit + c) * (size_t)capc, capc,
                        lm_ok, base, tid);
  if (lm_ok && g == 0) ccnt[row * nsplit + c] = min(base, (uint32_t)capc + 1u);
}

// bf16 with m > 64: 128 landmarks per workgroup (two column tiles per wave),
// key blocks staged by direct loads into swizzled double-buffered tiles; the
// scores by the shared-expert kernel's MFMA sequence (qk2_bf16_swz: k-slices in
// order, hi then lo plane), so a score here has the bits the group maxima came
// from. Candidates as in candidate_sweep, per column tile.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void topk_candd_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ qtop, const uint32_t* __restrict__ thr,
    const float* __restrict__ bmax, uint2* __restrict__ cand, uint32_t* __restrict__ ccnt,
    uint32_t* __restrict__ glist, int N, int m, int lchunk, int nsplit, int capc, int lm_tiles, int BH, int nbg,
    int gq) {
  constexpr int QT = 2;
  using Sw = SwzTile<D>;
  __shared__ __align__(16) struct {
    uint16_t rk[2][Sw::TILE];
    uint16_t blist[kCandListMax];   // the chunk's blocks that hold a candidate, in key order
    uint32_t need[kCandListMax / 32];   // the same as a bitmap
    uint32_t wtot[4];
  } sm;
  if (blockIdx.x == 0 && threadIdx.x == 0) glist[0] = 0u;   // no fallback rows yet (the select kernel adds them)
  int lt, c, z;
  if (!chunk_item(lm_tiles, nsplit, BH, lt, c, z)) return;   // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int k0 = c * lchunk, k1 = min(N, k0 + lchunk);
  const uint16_t* Kz = K + (size_t)z * N * D;
  const int nblk_all = (k1 - k0 + kKeyBlock - 1) / kKeyBlock;
  // Blocks to score: a block whose scores stay below every row's threshold holds
  // no candidate, and with groups of 64 the shared-expert kernel left each row's
  // block maximum (the same score bits as here). Block b is kept when some
  // landmark row of the tile has its maximum at or above the row's threshold; the
  // kept blocks are listed in key order, so the candidate lists are those of a full
  // sweep. Smaller groups (k large against N / 64: candidates in most blocks) or
  // more blocks than the list holds: every block is scored.
  int nblk;
  if (gq == kKeyBlock && nblk_all <= kCandListMax) {   // one group maximum per block (candidates sparse per block)
    const int blk0 = k0 / kKeyBlock, nwd = (nblk_all + 31) / 32;
    for (int i = tid; i < nwd; i += 256) sm.need[i] = 0u;
    __syncthreads();
    // two threads per landmark row, each a half of the chunk's bitmap words: a
    // word's 32 blocks compared in registers, then one LDS OR per word
    const int rr = tid >> 1, lm = lt * 128 + rr;
    if (lm < m) {
      const uint32_t tk = thr[(size_t)z * m + lm];
      const float t = tk ? key_f32(tk) : -INFINITY;
      const float* gm = bmax + ((size_t)z * m + lm) * nbg + blk0;
      const int wh = (nwd + 1) / 2, wd0 = (tid & 1) * wh, wd1 = min(nwd, wd0 + wh);
      for (int wd = wd0; wd < wd1; ++wd) {
        float bm[32];   // all 32 loads issued before the compares (indices clamped into the chunk)
#pragma unroll
        for (int bb = 0; bb < 32; ++bb) bm[bb] = gm[min(32 * wd + bb, nblk_all - 1)];
        uint32_t bits = 0;
#pragma unroll
        for (int bb = 0; bb < 32; ++bb) bits |= (32 * wd + bb < nblk_all && bm[bb] >= t) ? 1u << bb : 0u;
        if (bits) atomicOr(&sm.need[wd], bits);
      }
    }
    __syncthreads();
    nblk = 0;
    for (int b0 = 0; b0 < nblk_all; b0 += 256) {   // workgroup-uniform
      const int b = b0 + tid;
      const uint32_t keep = b < nblk_all ? (sm.need[b >> 5] >> (b & 31)) & 1u : 0u;
      uint32_t tot;
      const uint32_t pos = block_incl_scan(keep, sm.wtot, tot) - keep;
      if (keep) sm.blist[nblk + pos] = (uint16_t)b;
      nblk += (int)tot;
    }
    __syncthreads();
  } else {
    nblk = nblk_all;
  }
  auto blk_key = [&](int i) {
    return k0 + kKeyBlock * (gq == kKeyBlock && nblk_all <= kCandListMax ? (int)sm.blist[i] : i);
  };
  auto rows = [&](int kb, int (&id)[Sw::NI]) {
#pragma unroll
    for (int u = 0; u < Sw::NI; ++u) id[u] = min(kb + 16 * w + u * Sw::RPI + lane / Sw::CPR, k1 - 1);
  };
  if (nblk > 0) {
    int id0[Sw::NI];
    rows(blk_key(0), id0);
    dma_rows_k<D>(sm.rk[0], Kz, id0, w, lane);
  }
  bool lm_ok[QT];
  size_t rowi[QT];
  float tf[QT];
  uint32_t base[QT];
  uint4 qb[QT][2][D / 32];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int lm = lt * 128 + 32 * w + 16 * qt + r;
    lm_ok[qt] = lm < m;
    const int lmc = lm_ok[qt] ? lm : m - 1;
    rowi[qt] = (size_t)z * m + lmc;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qb[qt][p][ks] = ld16(qtop + ((size_t)(z * 2 + p) * m + lmc) * D + 32 * ks + 8 * g);
    const uint32_t tk = thr[rowi[qt]];
    tf[qt] = tk ? key_f32(tk) : -INFINITY;   // compare the scores themselves (same order)
    base[qt] = 0;
  }
  for (int j = 0; j < nblk; ++j) {
    const int kb = blk_key(j);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // block j staged; every wave done with block j - 1
    auto step = [&](uint16_t* __restrict__ nk, const uint16_t* __restrict__ ck) __attribute__((always_inline)) {
      if (j + 1 < nblk) {   // block-uniform
        int idn[Sw::NI];
        rows(blk_key(j + 1), idn);
        dma_rows_k<D>(nk, Kz, idn, w, lane);
      }
      f32x4 acc[QT][4];
      qk2_bf16_swz<D, QT>(ck, qb, acc, lane);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // per kt: this lane's candidate count in a byte of one word
        uint32_t flags = 0, packed = 0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const bool pr = (kb + 16 * kt + 4 * g + jj < k1) & (acc[qt][kt][jj] >= tf[qt]);
            flags |= pr ? 1u << (4 * kt + jj) : 0u;
            packed += pr ? 1u << (8 * kt) : 0u;
          }
        const uint32_t p0 = __shfl(packed, r, WAVE), p1 = __shfl(packed, r + 16, WAVE);
        const uint32_t p2 = __shfl(packed, r + 32, WAVE), p3 = __shfl(packed, r + 48, WAVE);
        const uint32_t tot = p0 + p1 + p2 + p3;   // no byte exceeds 16: no carries
        const uint32_t ex = (g > 0 ? p0 : 0u) + (g > 1 ? p1 : 0u) + (g > 2 ? p2 : 0u);
        // slot of the lane's first candidate of each kt: the landmark's candidates
        // of earlier kt, then those of lanes with smaller g
        const uint32_t first = ex + (tot << 8) + (tot << 16) + (tot << 24);
        uint2* seg = cand + (rowi[qt] * nsplit + c) * (size_t)capc;
        uint32_t fl = lm_ok[qt] ? flags : 0u;
        while (fl) {   // one pass per candidate of the lane, in key order
          const int bit = __builtin_ctz(fl);
          fl &= fl - 1u;
          const int kt = bit >> 2;
          const uint32_t pos = base[qt] + ((first >> (8 * kt)) & 255u) +
                               (uint32_t)__builtin_popcount(flags & ((1u << bit) - 1u) & (0xFu << (4 * kt)));
          float x = acc[qt][0][0];
#pragma unroll
          for (int b = 1; b < 16; ++b) x = bit == b ? acc[qt][b >> 2][b & 3] : x;
          if (pos < (uint32_t)capc) seg[pos] = make_uint2(f32_key(x), (uint32_t)(kb + 16 * kt + 4 * g + (bit & 3)));
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) base[qt] += (tot >> (8 * kt)) & 255u;
      }
    };
    step(sm.rk[(j + 1) & 1], sm.rk[j & 1]);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    if (lm_ok[qt] && g == 0) ccnt[rowi[qt] * nsplit + c] = min(base[qt], (uint32_t)capc + 1u);
}

// ---------------------------------------------------------------- 3. select
// One wave per row (WPB rows per workgroup). The row's candidate lists (index
// order, chunk after chunk) go to LDS; candidate j is slot j / 64 of lane j % 64
// in registers.
template <typename T, int D, int CAP, int WPB>
__global__ __launch_bounds__(64 * WPB) void topk_select_kernel(const uint2* __restrict__ cand,
                                                               const uint32_t* __restrict__ ccnt,
                                                               const float* __restrict__ qtnorm,
                                                               const float* __restrict__ kmax, int nsplit,
                                                               const double* __restrict__ qt64,
                                                               const T* __restrict__ K, int32_t* __restrict__ I,
                                                               uint32_t* __restrict__ glist, int N, int m, int k,
                                                               int capc, double gamma, int rows) {
  constexpr int SL = CAP / 64;
  constexpr int BAND = CAP < kBandMax ? CAP : kBandMax;
  __shared__ uint2 cs_s[WPB][CAP];
  __shared__ uint32_t blist_s[WPB][BAND];
  __shared__ double bsc_s[WPB][BAND];
  __shared__ uint8_t bkeep_s[WPB][BAND];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, row = blockIdx.x * WPB + w, z = row / m;
  if (row >= rows) return;   // wave-uniform; the waves of a workgroup never synchronise
  uint2* cs = cs_s[w];
  uint32_t* blist = blist_s[w];
  double* bsc = bsc_s[w];
  uint8_t* bkeep = bkeep_s[w];
  const uint32_t* cnt = ccnt + (size_t)row * nsplit;
  const uint2* segs = cand + (size_t)row * nsplit * capc;
  auto fallback = [&]() {
    if (lane == 0) glist[1 + atomicAdd(&glist[0], 1u)] = (uint32_t)row;
  };

  // gather the lists; any overflow, or more than CAP in all, goes to the fallback;
  // chunk offsets: exclusive sums of the counts
  uint32_t total = 0;
  if (nsplit <= 64) {   // one chunk per lane; offsets stay in registers
    const uint32_t n = lane < nsplit ? cnt[lane] : 0u;
    const uint32_t off = wave_excl_scan(n, total);
    total = __builtin_amdgcn_readfirstlane(total);   // wave-uniform: keep the loops below scalar
    if (__any(n > (uint32_t)capc) || total > (uint32_t)CAP || total < (uint32_t)k) {
      fallback();
      return;
    }
    // candidate j: chunk c with off_c <= j < off_{c+1} (offsets ascend)
    for (uint32_t j = lane; j < total; j += 64) {
      int c = 0;
      uint32_t oc = 0;
      for (int i = 1; i < nsplit; ++i) {
        const uint32_t oi = __builtin_amdgcn_readlane(off, i);
        c = oi <= j ? i : c;
        oc = oi <= j ? oi : oc;
      }
      cs[j] = segs[(size_t)c * capc + (j - oc)];
    }
  } else {   // many chunks: offsets in LDS (the band list's space, free until later)
    bool over = false;
    for (int c0 = 0; c0 < nsplit; c0 += 64) {
      const int c = c0 + lane;
      const uint32_t n = c < nsplit ? cnt[c] : 0u;
      over |= n > (uint32_t)capc;
      uint32_t tot;
      const uint32_t ex = wave_excl_scan(n, tot);
      if (c < nsplit && c < BAND) blist[c] = total + ex;
      total += tot;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    if (__any(over) || total > (uint32_t)CAP || total < (uint32_t)k || nsplit > BAND) {
      fallback();
      return;
    }
    wave_sync();
    for (uint32_t j = lane; j < total; j += 64) {
      int c = 0;
      while (c + 1 < nsplit && blist[c + 1] <= j) ++c;
      cs[j] = segs[(size_t)c * capc + (j - blist[c])];
    }
  }
  wave_sync();
  const double E = row_bound(qtnorm, kmax, nsplit, row, z, gamma, lane);
  const int ns = __builtin_amdgcn_readfirstlane((int)((total + 63) / 64));
  uint32_t ck[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    const uint32_t j = sl * 64 + lane;
    ck[sl] = (sl < ns && j < total) ? cs[j].x : 0u;
  }
  // exact k-th largest candidate key
  const uint32_t that = kth_largest_key<SL>(ck, ns, (uint32_t)k, 0);
  uint32_t hiKey, loKey;
  band_keys((double)key_f32(that), E, hiKey, loKey);
  uint32_t cin = 0, nb = 0;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    if (sl < ns) {
      cin += ballot_count(ck[sl] > hiKey);
      const bool inb = ck[sl] >= loKey && ck[sl] <= hiKey;
      const uint64_t msk = __ballot(inb);
      if (inb) {
        const uint32_t bp = nb + lanes_below(msk);
        if (bp < (uint32_t)BAND) blist[bp] = sl * 64 + lane;
      }
      nb += (uint32_t)__popcll(msk);
    }
  }
  nb = __builtin_amdgcn_readfirstlane(nb);
  cin = __builtin_amdgcn_readfirstlane(cin);
  if (nb > (uint32_t)BAND) {
    fallback();
    return;
  }
  const uint32_t need = (uint32_t)k - cin;
  // band members that make the cut; when the band holds exactly as many members
  // as places left, no re-scoring is needed (the usual case)
  bool keep[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) keep[sl] = nb == need;
  if (nb != need) {
    wave_sync();
    const double* qrow = qt64 + (size_t)row * D;
    const T* Kz = K + (size_t)z * N * D;
    for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
      const uint32_t bi = b0 + lane;
      if (bi < nb) bsc[bi] = dot64_row<T, D>(qrow, Kz + (size_t)cs[blist[bi]].y * D);
    }
    wave_sync();
    for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
      const uint32_t bi = b0 + lane;
      if (bi < nb) {
        const double sj = bsc[bi];
        const uint32_t ij = cs[blist[bi]].y;
        uint32_t rank = 0;
        for (uint32_t f = 0; f < nb; ++f) {
          const double si = bsc[f];
          rank += ((si > sj) | ((si == sj) & (cs[blist[f]].y < ij))) ? 1u : 0u;
        }
        bkeep[bi] = rank < need ? 1 : 0;
      }
    }
    wave_sync();
    // back to candidate order: band position of each band member by a second ballot pass
    uint32_t bp = 0;
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      keep[sl] = false;
      if (sl < ns) {
        const bool inb = ck[sl] >= loKey && ck[sl] <= hiKey;
        const uint64_t msk = __ballot(inb);
        if (inb) keep[sl] = bkeep[bp + lanes_below(msk)] != 0;
        bp += (uint32_t)__popcll(msk);
      }
    }
  }
  // output in index order: members above the band and the band members kept
  int32_t* Irow = I + (size_t)row * k;
  uint32_t outpos = 0;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    if (sl < ns) {
      const uint32_t j = sl * 64 + lane;
      const bool sel = j < total && (ck[sl] > hiKey || (ck[sl] >= loKey && keep[sl]));
      const uint64_t msk = __ballot(sel);
      if (sel) {
        const uint32_t op = outpos + lanes_below(msk);
        if (op < (uint32_t)k) Irow[op] = (int32_t)cs[j].y;
      }
      outpos += (uint32_t)__popcll(msk);
    }
  }
}

// ---------------------------------------------------------------- 4. fallback
// Exact selection straight from the definition, for rows the select kernel
// handed over: fp64 scores of the whole row (scratch row per workgroup), the
// k-th largest fp64 order key by an 8-bit radix select over an LDS histogram,
// then the row in index order: keys above it, and as many equal to it as places
// remain (lower ids first).
template <typename T, int D>
__global__ __launch_bounds__(64) void topk_general_kernel(const double* __restrict__ qt64, const T* __restrict__ K,
                                                          int32_t* __restrict__ I, const uint32_t* __restrict__ glist,
                                                          double* __restrict__ gscr, int N, int m, int k) {
  __shared__ uint32_t hist[256];
  const int lane = threadIdx.x;
  const uint32_t total = glist[0];
  double* sc = gscr + (size_t)blockIdx.x * N;
  for (uint32_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int row = (int)glist[1 + t], z = row / m;
    const double* qrow = qt64 + (size_t)row * D;
    const T* Kz = K + (size_t)z * N * D;
    for (int n = lane; n < N; n += 64) sc[n] = dot64_row<T, D>(qrow, Kz + (size_t)n * D);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    uint64_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)k;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
      wave_sync();
      for (int n = lane; n < N; n += 64) {
        const uint64_t key = f64_key(sc[n]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
      }
      wave_sync();
      // the bin holding the need-th largest key: suffix sums over 4 bins per lane
      uint32_t h[4], ls = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) { h[b] = hist[4 * lane + b]; ls += h[b]; }
      uint32_t suf = ls;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_down(suf, o, WAVE);
        if (lane + o < 64) suf += x;
      }
      const uint32_t ab = suf - ls;
      const bool cross = ab < need && suf >= need;
      uint32_t mybin = 0, myab = 0;
      if (cross) {
        uint32_t run = ab;
        for (int b = 3; b >= 0; --b) {
          if (run + h[b] >= need) { mybin = 4 * lane + b; myab = run; break; }
          run += h[b];
        }
      }
      const uint64_t cm = __ballot(cross);
      const int src = cm ? __ffsll((unsigned long long)cm) - 1 : 0;
      prefix |= (uint64_t)__shfl(mybin, src, WAVE) << shift;
      pmask |= 255ull << shift;
      need -= __shfl(myab, src, WAVE);
      wave_sync();
    }
    int32_t* Irow = I + (size_t)row * k;
    uint32_t outpos = 0, ties = 0;
    for (int c0 = 0; c0 < N; c0 += 64) {
      const int n = c0 + lane;
      const uint64_t key = n < N ? f64_key(sc[n]) : 0ull;
      const bool tie = n < N && key == prefix;
      const uint64_t tm = __ballot(tie);
      const bool sel = (n < N && key > prefix) || (tie && ties + lanes_below(tm) < need);
      ties += (uint32_t)__popcll(tm);
      const uint64_t sm = __ballot(sel);
      if (sel) {
        const uint32_t op = outpos + lanes_below(sm);
        if (op < (uint32_t)k) Irow[op] = n;
      }
      outpos += (uint32_t)__popcll(sm);
    }
    wave_sync();
  }
}

// Every row to the fallback (k too large for the select kernel).
__global__ __launch_bounds__(256) void topk_all_rows_kernel(uint32_t* __restrict__ glist, int rows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) glist[0] = (uint32_t)rows;
  if (i < rows) glist[1 + i] = (uint32_t)i;
}

template <typename T, int D>
static hipError_t topk_launch(const Plan& p, const void* K, char* ws, hipStream_t st) {
  const int rows = p.BH * p.m;
  uint32_t* glist = (uint32_t*)(ws + p.ws.glist);
  hipError_t e = hipSuccess;
  if (p.cap > 0) {
    // candidates against the thresholds the landmark step set (merge_thresh_kernel)
    if (sizeof(T) == 2 && p.m > kLandmarkTile) {   // bf16, several landmark tiles: the direct-load kernel
      const int tiles = (p.m + 127) / 128;
      const int cgrid = 8 * ((p.nsplit * p.BH + 7) / 8) * tiles;   // see chunk_item
      hipLaunchKernelGGL((topk_candd_kernel<D>), dim3(cgrid), dim3(256), 0, st, (const uint16_t*)K,
                         (const uint16_t*)(ws + p.ws.qtop), (const uint32_t*)(ws + p.ws.thr),
                         (const float*)(ws + p.ws.bmax), (uint2*)(ws + p.ws.cand), (uint32_t*)(ws + p.ws.ccnt), glist,
                         p.N, p.m, p.lchunk, p.nsplit, p.capc, tiles, p.BH, p.nbg, p.gq);
    } else {
      const int cgrid = 8 * ((p.nsplit * p.BH + 7) / 8) * p.lm_tiles;   // see chunk_item
      hipLaunchKernelGGL((topk_cand_kernel<T, D>), dim3(cgrid), dim3(256), 0, st, (const T*)K,
                         (const void*)(ws + p.ws.qtop), (const uint32_t*)(ws + p.ws.thr), (uint2*)(ws + p.ws.cand),
                         (uint32_t*)(ws + p.ws.ccnt), glist, p.N, p.m, p.lchunk, p.nsplit, p.capc, p.lm_tiles, p.BH);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto sel = [&](auto kern, int wpb) {
      hipLaunchKernelGGL(kern, dim3((rows + wpb - 1) / wpb), dim3(64 * wpb), 0, st, (const uint2*)(ws + p.ws.cand),
                         (const uint32_t*)(ws + p.ws.ccnt), (const float*)(ws + p.ws.qtnorm),
                         (const float*)(ws + p.ws.kmax), p.nsplit, (const double*)(ws + p.ws.qt64), (const T*)K,
                         (int32_t*)(ws + p.ws.I), glist, p.N, p.m, p.k, p.capc, p.gamma_qk, rows);
    };
    switch (p.cap) {   // LDS per wave grows with the capacity: fewer rows per workgroup
      case 256: sel(topk_select_kernel<T, D, 256, 4>, 4); break;
      case 512: sel(topk_select_kernel<T, D, 512, 4>, 4); break;
      case 1024: sel(topk_select_kernel<T, D, 1024, 2>, 2); break;
      case 2048: sel(topk_select_kernel<T, D, 2048, 1>, 1); break;
      default: sel(topk_select_kernel<T, D, 4096, 1>, 1); break;
    }
  } else {
    hipLaunchKernelGGL(topk_all_rows_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, glist, rows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((topk_general_kernel<T, D>), dim3(p.gwaves), dim3(64), 0, st,
                     (const double*)(ws + p.ws.qt64), (const T*)K, (int32_t*)(ws + p.ws.I), (const uint32_t*)glist,
                     (double*)(ws + p.ws.gscr), p.N, p.m, p.k);
  return hipGetLastError();
}

template <int D>
static hipError_t merge_thresh_launch(const Plan& p, char* ws, hipStream_t st) {
  const int rows = p.BH * p.m;
  // rows of more than kTopkMaxGroups group maxima, or k beyond the select kernel:
  // no threshold (every score a candidate, or every row to the fallback)
  const int nbg = (p.cap > 0 && p.nbg <= kTopkMaxGroups) ? p.nbg : 0;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((rows + 3) / 4), dim3(256), 0, st, (const float*)(ws + p.ws.lpart),
                       (float*)(ws + p.ws.vt32), (uint16_t*)(ws + p.ws.vt16), (const float*)(ws + p.ws.bmax),
                       (const float*)(ws + p.ws.qtnorm), (const float*)(ws + p.ws.kmax), p.nsplit,
                       (uint32_t*)(ws + p.ws.thr), nbg, p.m, p.k, p.gamma_qk, rows, (float*)(ws + p.ws.lse_se));
  };
  if (p.nsplit <= 4) {
    if (nbg <= 256) go(merge_thresh_kernel<D, 4, 4>);
    else if (nbg <= 1024) go(merge_thresh_kernel<D, 16, 4>);
    else go(merge_thresh_kernel<D, 64, 4>);
  } else {
    if (nbg <= 256) go(merge_thresh_kernel<D, 4, 8>);
    else if (nbg <= 1024) go(merge_thresh_kernel<D, 16, 8>);
    else go(merge_thresh_kernel<D, 64, 8>);
  }
  return hipGetLastError();
}

hipError_t launch_merge_thresh(const Plan& p, char* ws, hipStream_t st) {
  return p.d == 64 ? merge_thresh_launch<64>(p, ws, st) : merge_thresh_launch<128>(p, ws, st);
}

hipError_t launch_topk(const Plan& p, const void* K, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? topk_launch<uint16_t, 64>(p, K, ws, st) : topk_launch<uint16_t, 128>(p, K, ws, st);
  return p.d == 64 ? topk_launch<float, 64>(p, K, ws, st) : topk_launch<float, 128>(p, K, ws, st);
}

}  // namespace mita
