// Step 3: deformable experts. I_i = the k tokens with the largest q~_i . K_n
// (deformable experts of the MiTA summaries: top-k activations of K^T q~_i over
// the whole sequence, ties to the lower index here, ids listed ascending).
//
// The m x N score rows from step 2 carry a bounded error E_i = gamma |q~_i| max|K|.
// Selection is exact anyway:
//   1. segment kernel: each workgroup loads <= 8192 scores of one row into LDS once
//      (as order-preserving uint32 keys), builds a 4096-bin histogram of the top
//      12 key bits, finds the bin holding its local k-th largest score and keeps
//      every score >= (that bin's lower edge) - 2 E_i, in index order;
//   2. row kernel: radix-selects the k-th largest approximate score T among the
//      candidates; scores above T + 2E are in, scores below T - 2E are out, and
//      the band between is re-scored in fp64 from Q~ (fp64) and K, which decides
//      the remaining places by (fp64 score, lower index).
// Every token of the true top-k is a candidate: a segment's share of the global
// top-k lies within its own top-k, and the band covers any score whose fp32
// rank could differ from its fp64 rank.
#include "attn_core.h"

namespace mita {

constexpr int kBandLds = 1024;   // band entries cached in LDS by the row kernel

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

__device__ __forceinline__ float slice_kmax(const float* kmax, int z, int nsplit) {
  float mx = 0.f;
  for (int c = 0; c < nsplit; ++c) mx = fmaxf(mx, kmax[(size_t)z * nsplit + c]);
  return mx;
}

__global__ __launch_bounds__(256) void topk_segment_kernel(const float* __restrict__ S, const float* __restrict__ qtnorm,
                                                           const float* __restrict__ kmax, int nsplit,
                                                           uint32_t* __restrict__ cand_key,
                                                           uint32_t* __restrict__ cand_idx,
                                                           uint32_t* __restrict__ cand_cnt, int N, int m, int seg,
                                                           int G, int k, double gamma) {
  __shared__ __align__(16) uint32_t keys[kTopkSegMax];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t s_bin;
  const int g = blockIdx.x, row = blockIdx.y, z = row / m, tid = threadIdx.x;
  const int n0 = g * seg, n1 = min(N, n0 + seg), L = n1 - n0;
  const float* Srow = S + (size_t)row * N + n0;

  for (int i = tid; i < 4096; i += 256) hist[i] = 0;
  if (tid == 0) s_bin = 0;
  __syncthreads();
  if ((N & 3) == 0) {
    for (int i = tid * 4; i < L; i += 1024) {
      if (i + 3 < L) {
        const float4 v = *(const float4*)(Srow + i);
        const uint4 kk = make_uint4(f32_key(v.x), f32_key(v.y), f32_key(v.z), f32_key(v.w));
        *(uint4*)(keys + i) = kk;
        atomicAdd(&hist[kk.x >> 20], 1u);
        atomicAdd(&hist[kk.y >> 20], 1u);
        atomicAdd(&hist[kk.z >> 20], 1u);
        atomicAdd(&hist[kk.w >> 20], 1u);
      } else {
        for (int u = i; u < L; ++u) {
          const uint32_t kk = f32_key(Srow[u]);
          keys[u] = kk;
          atomicAdd(&hist[kk >> 20], 1u);
        }
      }
    }
  } else {
    for (int i = tid; i < L; i += 256) {
      const uint32_t kk = f32_key(Srow[i]);
      keys[i] = kk;
      atomicAdd(&hist[kk >> 20], 1u);
    }
  }
  __syncthreads();

  // bin holding the local k-th largest: thread t owns bins [16t, 16t + 16)
  const uint32_t kl = (uint32_t)min(k, L);
  uint32_t loc = 0;
#pragma unroll
  for (int b = 0; b < 16; ++b) loc += hist[16 * tid + b];
  uint32_t total;
  const uint32_t pre = block_incl_scan(loc, wtot, total);
  const uint32_t suffix = total - pre + loc;  // bins >= 16 t
  const uint32_t above = suffix - loc;        // bins >= 16 (t + 1)
  if (above < kl && suffix >= kl) {
    uint32_t run = above;
    for (int b = 15; b >= 0; --b) {
      run += hist[16 * tid + b];
      if (run >= kl) { s_bin = 16 * tid + b; break; }
    }
  }
  __syncthreads();
  const uint32_t bin = s_bin;
  uint32_t kt = 0;
  if (bin > 8) {  // bins 0..8 hold only NaN and -inf patterns: keep everything
    const double E = gamma * (double)qtnorm[row] * (double)slice_kmax(kmax, z, nsplit);
    const double t = (double)key_f32(bin << 20) - 2.0 * E;
    kt = (t > -INFINITY) ? f32_key(round_down_f32(t)) : 0u;
  }

  // ordered compaction of keys >= kt
  uint32_t* ck = cand_key + (size_t)row * N + n0;
  uint32_t* ci = cand_idx + (size_t)row * N + n0;
  uint32_t base = 0;
  for (int c0 = 0; c0 < L; c0 += 1024) {
    const int i = c0 + tid * 4;
    uint4 kk = make_uint4(0, 0, 0, 0);
    if (i + 3 < L) {
      kk = *(const uint4*)(keys + i);
    } else {
      if (i < L) kk.x = keys[i];
      if (i + 1 < L) kk.y = keys[i + 1];
      if (i + 2 < L) kk.z = keys[i + 2];
    }
    const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
    uint32_t f = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) f += (i + u < L && kv[u] >= kt) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = base + block_incl_scan(f, wtot, tot) - f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u < L && kv[u] >= kt) {
        ck[pos] = kv[u];
        ci[pos] = (uint32_t)(n0 + i + u);
        ++pos;
      }
    base += tot;
  }
  if (tid == 0) cand_cnt[(size_t)row * G + g] = base;
}

// fp64 score q~_i . K_n (inputs widened exactly), one thread.
template <typename T, int D>
__device__ __forceinline__ double score64_thread(const double* qrow, const T* krow) {
  double s = 0.0;
  for (int j = 0; j < D; ++j) {
    double x;
    if constexpr (sizeof(T) == 2) x = (double)bf16_to_f32(krow[j]); else x = (double)krow[j];
    s = fma(qrow[j], x, s);
  }
  return s;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void topk_row_kernel(const uint32_t* __restrict__ cand_key,
                                                       const uint32_t* __restrict__ cand_idx,
                                                       const uint32_t* __restrict__ cand_cnt,
                                                       const float* __restrict__ qtnorm, const float* __restrict__ kmax,
                                                       int nsplit, const double* __restrict__ qt64,
                                                       const T* __restrict__ K, int32_t* __restrict__ I, int N, int m,
                                                       int seg, int G, int k, double gamma) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t s_digit, s_above;
  __shared__ uint32_t bidx[kBandLds];
  __shared__ double bsc[kBandLds];
  __shared__ uint8_t bsel[kBandLds];
  const int row = blockIdx.x, z = row / m, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t* ckr = cand_key + (size_t)row * N;
  const uint32_t* cir = cand_idx + (size_t)row * N;
  const uint32_t* cnt = cand_cnt + (size_t)row * G;
  const double* qrow = qt64 + (size_t)row * D;
  const T* Kz = K + (size_t)z * N * D;

  // 1. radix select of the k-th largest candidate key (8 bits per pass)
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int g = 0; g < G; ++g) {
      const uint32_t n = cnt[g];
      const uint32_t* ck = ckr + (size_t)g * seg;
      for (uint32_t e = tid; e < n; e += 256) {
        const uint32_t key = ck[e];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    const uint32_t v = hist[tid];
    uint32_t total;
    const uint32_t pre = block_incl_scan(v, wtot, total);
    const uint32_t suffix = total - pre + v, above = suffix - v;
    if (above < krem && suffix >= krem) { s_digit = tid; s_above = above; }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    krem -= s_above;
    __syncthreads();
  }

  // 2. certainty band around the approximate k-th score
  const double E = gamma * (double)qtnorm[row] * (double)slice_kmax(kmax, z, nsplit);
  const double That = (double)key_f32(prefix);
  const double hi = That + 2.0 * E, lo = That - 2.0 * E;
  const uint32_t hiKey = (hi < INFINITY) ? f32_key(round_up_f32(hi)) : 0xFFFFFFFFu;
  const uint32_t loKey = (lo > -INFINITY) ? f32_key(round_down_f32(lo)) : 0u;

  uint32_t c_in = 0, c_band = 0;
  for (int g = 0; g < G; ++g) {
    const uint32_t n = cnt[g];
    const uint32_t* ck = ckr + (size_t)g * seg;
    for (uint32_t e = tid; e < n; e += 256) {
      const uint32_t key = ck[e];
      c_in += key > hiKey;
      c_band += (key >= loKey && key <= hiKey);
    }
  }
  uint32_t tin, tband;
  block_incl_scan(c_in, wtot, tin);
  block_incl_scan(c_band, wtot, tband);
  const uint32_t need = (uint32_t)k - tin;   // places decided by the fp64 scores (>= 1)
  const bool cached = tband <= (uint32_t)kBandLds;

  // 3a. small band: gather it (index order), score in fp64 one wave per entry, rank
  uint64_t vstar = 0;
  uint32_t ties_needed = 0;
  if (cached) {
    uint32_t base = 0;
    for (int g = 0; g < G; ++g) {
      const uint32_t n = cnt[g];
      const uint32_t* ck = ckr + (size_t)g * seg;
      const uint32_t* ci = cir + (size_t)g * seg;
      for (uint32_t c0 = 0; c0 < n; c0 += 256) {
        const uint32_t e = c0 + tid;
        uint32_t key = 0;
        if (e < n) key = ck[e];
        const uint32_t f = (e < n && key >= loKey && key <= hiKey) ? 1u : 0u;
        uint32_t tot;
        const uint32_t pos = base + block_incl_scan(f, wtot, tot) - f;
        if (f) bidx[pos] = ci[e];
        base += tot;
      }
    }
    __syncthreads();
    for (uint32_t e = w; e < tband; e += 4) {
      const T* kr = Kz + (size_t)bidx[e] * D;
      double part = 0.0;
      for (int j = lane; j < D; j += 64) {
        double x;
        if constexpr (sizeof(T) == 2) x = (double)bf16_to_f32(kr[j]); else x = (double)kr[j];
        part = fma(qrow[j], x, part);
      }
      part = wave_sum_f64(part);
      if (lane == 0) bsc[e] = part;
    }
    __syncthreads();
    for (uint32_t e = tid; e < tband; e += 256) {
      const double se = bsc[e];
      const uint32_t ie = bidx[e];
      uint32_t rank = 0;
      for (uint32_t f = 0; f < tband; ++f) {
        const double sf = bsc[f];
        rank += (sf > se || (sf == se && bidx[f] < ie)) ? 1u : 0u;
      }
      bsel[e] = rank < need;
    }
    __syncthreads();
  } else {
    // 3b. large band (degenerate inputs): radix select over fp64 order keys,
    // re-scoring band members on the fly in every pass.
    uint64_t pfx = 0, pm = 0;
    uint32_t rem = need;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int g = 0; g < G; ++g) {
        const uint32_t n = cnt[g];
        const uint32_t* ck = ckr + (size_t)g * seg;
        const uint32_t* ci = cir + (size_t)g * seg;
        for (uint32_t e = tid; e < n; e += 256) {
          const uint32_t key = ck[e];
          if (key < loKey || key > hiKey) continue;
          const uint64_t k64 = f64_key(score64_thread<T, D>(qrow, Kz + (size_t)ci[e] * D));
          if ((k64 & pm) == pfx) atomicAdd(&hist[(uint32_t)(k64 >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      const uint32_t v = hist[tid];
      uint32_t total;
      const uint32_t pre = block_incl_scan(v, wtot, total);
      const uint32_t suffix = total - pre + v, above = suffix - v;
      if (above < rem && suffix >= rem) { s_digit = tid; s_above = above; }
      __syncthreads();
      pfx |= (uint64_t)s_digit << shift;
      pm |= (uint64_t)255 << shift;
      rem -= s_above;
      __syncthreads();
    }
    vstar = pfx;
    ties_needed = rem;   // entries equal to vstar taken in index order
  }

  // 4. output in index order: definite members, then band picks
  int32_t* Irow = I + (size_t)row * k;
  uint32_t outpos = 0, ties_seen = 0;
  uint32_t bslot = 0;
  for (int g = 0; g < G; ++g) {
    const uint32_t n = cnt[g];
    const uint32_t* ck = ckr + (size_t)g * seg;
    const uint32_t* ci = cir + (size_t)g * seg;
    for (uint32_t c0 = 0; c0 < n; c0 += 256) {
      const uint32_t e = c0 + tid;
      uint32_t key = 0, idx = 0;
      if (e < n) { key = ck[e]; idx = ci[e]; }
      const bool inb = e < n && key >= loKey && key <= hiKey;
      uint32_t sel = (e < n && key > hiKey) ? 1u : 0u;
      if (cached) {
        uint32_t tot;
        const uint32_t slot = bslot + block_incl_scan(inb ? 1u : 0u, wtot, tot) - (inb ? 1u : 0u);
        if (inb && bsel[slot]) sel = 1u;
        bslot += tot;
      } else {
        uint64_t k64 = 0;
        if (inb) k64 = f64_key(score64_thread<T, D>(qrow, Kz + (size_t)idx * D));
        if (inb && k64 > vstar) sel = 1u;
        const uint32_t tie = (inb && k64 == vstar) ? 1u : 0u;
        uint32_t tot;
        const uint32_t trank = ties_seen + block_incl_scan(tie, wtot, tot) - tie;
        if (tie && trank < ties_needed) sel = 1u;
        ties_seen += tot;
      }
      uint32_t tot;
      const uint32_t pos = outpos + block_incl_scan(sel, wtot, tot) - sel;
      if (sel && pos < (uint32_t)k) Irow[pos] = (int32_t)idx;
      outpos += tot;
    }
  }
}

// ---------------------------------------------------------------- rows of up to 4096 scores
// One wave owns a whole row in registers (lane l holds scores 64 i + l, so every
// register index is one coalesced 256-byte load and, in index order, a run of 64).
// Counting is done with ballots (the popcounts run on the scalar unit, leaving
// one vector compare per element). Steps:
//   1. the top 4 key bits of the k-th largest score by a bit search (they hold
//      sign and high exponent bits, which take few values);
//   2. the next 8 bits by an LDS histogram over the scores sharing those 4 bits;
//   3. every score >= (that 12-bit bucket's lower edge - 2E) goes, in index
//      order, to an LDS list (typically k plus a few dozen);
//   4. on the list: the exact k-th largest by a bit search, the band within 2E
//      of it re-scored in fp64 (one lane per member), output in index order.
// Rows whose list would overflow (massive ties) take a slower general path.
// No block barriers: the four waves of a workgroup work on four rows.
constexpr int kWaveCap = 512;

__device__ __forceinline__ uint32_t ballot_count(bool p) { return (uint32_t)__popcll(__ballot(p)); }
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ void wave_bucket(const uint32_t* hist, uint32_t need, int lane, uint32_t& bin,
                                            uint32_t& above) {
  uint32_t h[4], ls = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) { h[b] = hist[4 * lane + b]; ls += h[b]; }
  uint32_t suf = ls;  // bins of lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_down(suf, o, WAVE);
    if (lane + o < 64) suf += t;
  }
  const uint32_t ab = suf - ls;
  const bool cross = ab < need && suf >= need;
  uint32_t mybin = 0, myab = 0;
  if (cross) {
    uint32_t run = ab;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (run + h[b] >= need) { mybin = 4 * lane + b; myab = run; break; }
      run += h[b];
    }
  }
  const uint64_t msk = __ballot(cross);
  const int src = msk ? __ffsll((unsigned long long)msk) - 1 : 0;
  bin = __shfl(mybin, src, WAVE);
  above = __shfl(myab, src, WAVE);
}

template <typename T>
__device__ __forceinline__ double kval64(const T* kr, int c) {
  if constexpr (sizeof(T) == 2) return (double)bf16_to_f32(((const uint16_t*)kr)[c]);
  else return (double)kr[c];
}

// fp64 dot product of a landmark query (fp64) with one key row, by one lane; the
// key row is fetched in 16-byte pieces that are all in flight together.
template <typename T, int D>
__device__ __forceinline__ double dot64_row(const double* __restrict__ q, const T* __restrict__ kr) {
  constexpr int EPC = 16 / sizeof(T);
  uint4 kc[D / EPC];
#pragma unroll
  for (int c = 0; c < D / EPC; ++c) kc[c] = *(const uint4*)(kr + c * EPC);
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

template <typename T, int D, int PL>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ S, const float* __restrict__ qtnorm,
                                                        const float* __restrict__ kmax, int nsplit,
                                                        const double* __restrict__ qt64, const T* __restrict__ K,
                                                        int32_t* __restrict__ I, uint32_t* __restrict__ gen_list,
                                                        uint32_t* __restrict__ gen_count, int N, int m, int k,
                                                        double gamma, int rows) {
  __shared__ uint32_t hist_s[4][256 + 64];   // 256 bins + one trash bin per lane
  __shared__ uint2 cand_s[4][kWaveCap + 64];   // (order key, token id), then trash slots
  __shared__ double csc_s[4][kWaveCap];
  __shared__ uint8_t kflag_s[4][kWaveCap];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x * 4 + w;
  if (row >= rows) return;
  uint32_t* hist = hist_s[w];
  uint2* cand = cand_s[w];
  double* csc = csc_s[w];
  uint8_t* kflag = kflag_s[w];
  const int z = row / m;
  const float* Srow = S + (size_t)row * N;
  const T* Kz = K + (size_t)z * N * D;
  const double* qrow = qt64 + (size_t)row * D;

  // small loads first, so waiting for them does not wait for the row
  float kmx = 0.f;
  for (int c = lane; c < nsplit; c += 64) kmx = fmaxf(kmx, kmax[(size_t)z * nsplit + c]);
  const float qtn = qtnorm[row];
  // coalesced: register group j holds scores 4 (64 j + lane) + c, c < 4, so each
  // load instruction reads 1 KiB contiguously; index order is (group, lane, c)
  constexpr int PG = PL / 4;
  uint32_t kv[PL];
  if ((N & 3) == 0) {
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int n = (64 * j + lane) * 4;
      const float4 x = *(const float4*)(Srow + min(n, N - 4));   // unconditional (no branch, no wait)
      kv[4 * j + 0] = n < N ? f32_key(x.x) : 0u;                  // 0: absent (no finite score maps to 0)
      kv[4 * j + 1] = n < N ? f32_key(x.y) : 0u;
      kv[4 * j + 2] = n < N ? f32_key(x.z) : 0u;
      kv[4 * j + 3] = n < N ? f32_key(x.w) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PG; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = (64 * j + lane) * 4 + c;
        const float x = Srow[min(n, N - 1)];
        kv[4 * j + c] = n < N ? f32_key(x) : 0u;
      }
  }
  for (int b = lane; b < 256 + 64; b += 64) hist[b] = 0;
  const double E = gamma * (double)qtn * (double)wave_max(kmx);

  // 1. top key byte of the k-th largest: walk the distinct top bytes downwards
  //    from the maximum (they are few: sign and high exponent bits)
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) lmax = max(lmax, kv[i]);
  uint32_t b8 = wave_max_uniform(lmax) >> 24, above8 = 0;
  for (;;) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) c += (kv[i] >> 24) == b8 ? 1u : 0u;
    c = wave_sum_uniform(c);
    if (above8 + c >= (uint32_t)k || b8 == 0) break;
    above8 += c;
    uint32_t nm = 0;   // largest key under the current top byte
#pragma unroll
    for (int i = 0; i < PL; ++i) nm = ((kv[i] >> 24) < b8) ? max(nm, kv[i]) : nm;
    b8 = wave_max_uniform(nm) >> 24;
  }
  // 2. next byte by an LDS histogram over the scores under that top byte (the
  //    others count into per-lane trash bins: no branches, no conflicts)
  wave_sync();
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint32_t bin = ((kv[i] >> 24) == b8 && kv[i]) ? ((kv[i] >> 16) & 255u) : 256u + lane;
    atomicAdd(&hist[bin], 1u);
  }
  wave_sync();
  uint32_t b16, above16;
  wave_bucket(hist, (uint32_t)k - above8, lane, b16, above16);
  const uint32_t edge = (b8 << 24) | (b16 << 16);
  uint32_t kt = 1u;
  if (edge >= 0x00800000u) {
    const double t = (double)key_f32(edge) - 2.0 * E;
    if (t > -INFINITY) kt = max(1u, f32_key(round_down_f32(t)));
  }
  // 3. candidates (>= kt) in index order: per-group counts, three groups per
  //    word (10-bit fields), one prefix scan per word
  constexpr int PW = (PG + 2) / 3;
  uint32_t gofs[PG];
  uint32_t cnt = 0;
#pragma unroll
  for (int wdx = 0; wdx < PW; ++wdx) {
    uint32_t packed = 0;
#pragma unroll
    for (int f = 0; f < 3; ++f) {
      const int j = 3 * wdx + f;
      if (j < PG) {
        uint32_t c = 0;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) c += kv[4 * j + cc] >= kt ? 1u : 0u;
        packed |= c << (10 * f);
      }
    }
    uint32_t tot;
    const uint32_t ex = wave_excl_scan(packed, tot);
#pragma unroll
    for (int f = 0; f < 3; ++f) {
      const int j = 3 * wdx + f;
      if (j < PG) {
        gofs[j] = cnt + ((ex >> (10 * f)) & 1023u);
        cnt += (tot >> (10 * f)) & 1023u;
      }
    }
  }
  if (cnt > (uint32_t)kWaveCap) {   // massive ties: the general kernel takes the row
    if (lane == 0) gen_list[atomicAdd(gen_count, 1u)] = (uint32_t)row;
    return;
  }
#pragma unroll
  for (int j = 0; j < PG; ++j) {
    uint32_t pos = gofs[j];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint32_t x = kv[4 * j + cc];
      const bool p = x >= kt;
      const uint32_t dst = p ? pos : (uint32_t)(kWaveCap + lane);   // trash slot: no branch
      cand[dst] = make_uint2(x, (uint32_t)((64 * j + lane) * 4 + cc));
      pos += p ? 1u : 0u;
    }
  }
  wave_sync();

  // 4. exact k-th largest: it lies in the 16-bit bucket [edge, edge + 2^16) and is
  //    the r-th largest there, r = k - (scores above the bucket); search the low
  //    16 bits among the bucket's candidates (candidate j: slot j / 64 of lane j % 64)
  constexpr int SL = kWaveCap / 64;
  const int ns = (int)((cnt + 63) / 64);
  uint32_t ck[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    const uint32_t j = sl * 64 + lane;
    ck[sl] = (sl < ns && j < cnt) ? cand[j].x : 0u;
  }
  const uint32_t r = (uint32_t)k - above8 - above16;
  uint32_t that = edge;
  for (int b = 15; b >= 0; --b) {
    const uint32_t tst = that | (1u << b);
    uint32_t c = 0;
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
      if (sl < ns) c += ballot_count(ck[sl] >= tst && ck[sl] < edge + 0x10000u);
    if (c >= r) that = tst;
  }
  uint32_t hiKey, loKey;
  band_keys((double)key_f32(that), E, hiKey, loKey);
  uint32_t cin = 0, nb = 0;
  // band members: their list slots go to the (now free) histogram array
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    if (sl < ns) {
      cin += ballot_count(ck[sl] > hiKey);
      const bool inb = ck[sl] >= loKey && ck[sl] <= hiKey;
      const uint64_t msk = __ballot(inb);
      if (inb) {
        const uint32_t bp = nb + lanes_below(msk);
        if (bp < 256u) hist[bp] = sl * 64 + lane;
      }
      nb += (uint32_t)__popcll(msk);
    }
  }
  const uint32_t need = (uint32_t)k - cin;
  // keep[sl]: band members that make the cut. When the band holds exactly as many
  // members as places left, no re-scoring is needed (the usual case: the band
  // is the k-th score alone).
  bool keep[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) keep[sl] = nb == need;
  if (nb != need) {
    wave_sync();
    if (nb <= 256u) {
      // fp64 scores, one lane per member, then ranks by (score desc, index asc)
      for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
        const uint32_t bi = b0 + lane;
        if (bi < nb) {
          const uint32_t slot = hist[bi];
          csc[slot] = dot64_row<T, D>(qrow, Kz + (size_t)cand[slot].y * D);
        }
      }
      wave_sync();
      for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
        const uint32_t bi = b0 + lane;
        if (bi < nb) {
          const uint32_t slot = hist[bi];
          const double sj = csc[slot];
          const uint32_t ij = cand[slot].y;
          uint32_t rank = 0;
          for (uint32_t f = 0; f < nb; ++f) {
            const uint32_t sf = hist[f];
            const double si = csc[sf];
            rank += (si > sj || (si == sj && cand[sf].y < ij)) ? 1u : 0u;
          }
          kflag[slot] = rank < need ? 1 : 0;
        }
      }
    } else {
      for (uint32_t j = lane; j < cnt; j += 64) {
        const uint32_t kj = cand[j].x;
        if (kj >= loKey && kj <= hiKey) csc[j] = dot64_row<T, D>(qrow, Kz + (size_t)cand[j].y * D);
      }
      wave_sync();
      for (uint32_t j = lane; j < cnt; j += 64) {
        const uint32_t kj = cand[j].x;
        if (kj < loKey || kj > hiKey) continue;
        const double sj = csc[j];
        const uint32_t ij = cand[j].y;
        uint32_t rank = 0;
        for (uint32_t i2 = 0; i2 < cnt; ++i2) {
          const uint32_t ki = cand[i2].x;
          if (ki >= loKey && ki <= hiKey) {
            const double si = csc[i2];
            rank += (si > sj || (si == sj && cand[i2].y < ij)) ? 1u : 0u;
          }
        }
        kflag[j] = rank < need ? 1 : 0;
      }
    }
    wave_sync();
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      const uint32_t j = sl * 64 + lane;
      keep[sl] = (sl < ns && j < cnt && ck[sl] >= loKey && ck[sl] <= hiKey) ? kflag[j] != 0 : false;
    }
  }
  // output in index order: members above the band and the band members kept
  int32_t* Irow = I + (size_t)row * k;
  uint32_t outpos = 0;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    if (sl < ns) {
      const uint32_t j = sl * 64 + lane;
      const bool sel = j < cnt && (ck[sl] > hiKey || (ck[sl] >= loKey && keep[sl]));
      const uint64_t msk = __ballot(sel);
      if (sel) {
        const uint32_t op = outpos + lanes_below(msk);
        if (op < (uint32_t)k) Irow[op] = (int32_t)cand[j].y;
      }
      outpos += (uint32_t)__popcll(msk);
    }
  }
}

// Rows the wave kernel could not list (massive ties): one wave per row, straight
// from the score row in global memory. Exact k-th largest by a bit search over
// the order keys; the band around it decided by fp64 scores (recomputed on the
// fly) with a bit search over fp64 order keys; ties to the lower index.
template <typename T, int D>
__global__ __launch_bounds__(64) void topk_general_kernel(const float* __restrict__ S, const float* __restrict__ qtnorm,
                                                          const float* __restrict__ kmax, int nsplit,
                                                          const double* __restrict__ qt64, const T* __restrict__ K,
                                                          int32_t* __restrict__ I, const uint32_t* __restrict__ gen_list,
                                                          const uint32_t* __restrict__ gen_count, int N, int m, int k,
                                                          double gamma) {
  const int lane = threadIdx.x;
  const uint32_t total = *gen_count;
  for (uint32_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int row = (int)gen_list[t], z = row / m;
    const float* Srow = S + (size_t)row * N;
    const T* Kz = K + (size_t)z * N * D;
    const double* qrow = qt64 + (size_t)row * D;
    float kmx = 0.f;
    for (int c = lane; c < nsplit; c += 64) kmx = fmaxf(kmx, kmax[(size_t)z * nsplit + c]);
    const double E = gamma * (double)qtnorm[row] * (double)wave_max(kmx);
    uint32_t pfx = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = pfx | (1u << b);
      uint32_t c = 0;
      for (int n = lane; n < N; n += 64) c += f32_key(Srow[n]) >= cand ? 1u : 0u;
      if (wave_sum_uniform(c) >= (uint32_t)k) pfx = cand;
    }
    uint32_t hiKey, loKey;
    band_keys((double)key_f32(pfx), E, hiKey, loKey);
    uint32_t cin = 0;
    for (int n = lane; n < N; n += 64) cin += f32_key(Srow[n]) > hiKey ? 1u : 0u;
    const uint32_t need = (uint32_t)k - wave_sum_uniform(cin);
    auto score = [&](int n) {
      const T* kr = Kz + (size_t)n * D;
      double sc = 0.0;
      for (int c = 0; c < D; ++c) sc = fma(qrow[c], kval64<T>(kr, c), sc);
      return sc;
    };
    uint64_t p64 = 0;
    for (int b = 63; b >= 0; --b) {
      const uint64_t cand = p64 | (1ull << b);
      uint32_t c = 0;
      for (int n = lane; n < N; n += 64) {
        const uint32_t x = f32_key(Srow[n]);
        if (x >= loKey && x <= hiKey) c += f64_key(score(n)) >= cand ? 1u : 0u;
      }
      if (wave_sum_uniform(c) >= need) p64 = cand;
    }
    uint32_t gtl = 0;
    for (int n = lane; n < N; n += 64) {
      const uint32_t x = f32_key(Srow[n]);
      if (x >= loKey && x <= hiKey) gtl += f64_key(score(n)) > p64 ? 1u : 0u;
    }
    const uint32_t ties_needed = need - wave_sum_uniform(gtl);
    int32_t* Irow = I + (size_t)row * k;
    uint32_t outpos = 0, ties_seen = 0;
    for (int c0 = 0; c0 < N; c0 += 64) {
      const int n = c0 + lane;
      bool sel = false, tie = false;
      if (n < N) {
        const uint32_t x = f32_key(Srow[n]);
        if (x > hiKey) {
          sel = true;
        } else if (x >= loKey) {
          const uint64_t k64 = f64_key(score(n));
          sel = k64 > p64;
          tie = k64 == p64;
        }
      }
      const uint64_t tm = __ballot(tie);
      if (tie && ties_seen + lanes_below(tm) < ties_needed) sel = true;
      ties_seen += (uint32_t)__popcll(tm);
      const uint64_t sm = __ballot(sel);
      if (sel) {
        const uint32_t op = outpos + lanes_below(sm);
        if (op < (uint32_t)k) Irow[op] = n;
      }
      outpos += (uint32_t)__popcll(sm);
    }
  }
}

__global__ void topk_zero_kernel(uint32_t* __restrict__ p) { *p = 0u; }

template <typename T, int D>
static hipError_t topk_launch(const Plan& p, const void* K, char* ws, hipStream_t st) {
  const int rows = p.BH * p.m;
  if (p.N <= kTopkWaveMax) {
    uint32_t* gen_count = (uint32_t*)(ws + p.ws.counters) + 32;   // counter of rows for the general kernel
    uint32_t* gen_list = (uint32_t*)(ws + p.ws.cand_idx);
    hipLaunchKernelGGL(topk_zero_kernel, dim3(1), dim3(1), 0, st, gen_count);
    const dim3 grid((rows + 3) / 4);
    auto args = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const float*)(ws + p.ws.S), (const float*)(ws + p.ws.qtnorm),
                         (const float*)(ws + p.ws.kmax), p.nsplit, (const double*)(ws + p.ws.qt64), (const T*)K,
                         (int32_t*)(ws + p.ws.I), gen_list, gen_count, p.N, p.m, p.k, p.gamma_qk, rows);
    };
    if (p.N <= 1024) args(topk_wave_kernel<T, D, 16>);
    else if (p.N <= 2048) args(topk_wave_kernel<T, D, 32>);
    else if (p.N <= 3328) args(topk_wave_kernel<T, D, 52>);
    else args(topk_wave_kernel<T, D, 64>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_general_kernel<T, D>), dim3(256), dim3(64), 0, st, (const float*)(ws + p.ws.S),
                       (const float*)(ws + p.ws.qtnorm), (const float*)(ws + p.ws.kmax), p.nsplit,
                       (const double*)(ws + p.ws.qt64), (const T*)K, (int32_t*)(ws + p.ws.I),
                       (const uint32_t*)gen_list, (const uint32_t*)gen_count, p.N, p.m, p.k, p.gamma_qk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_segment_kernel, dim3(p.G, rows), dim3(256), 0, st, (const float*)(ws + p.ws.S),
                     (const float*)(ws + p.ws.qtnorm), (const float*)(ws + p.ws.kmax), p.nsplit,
                     (uint32_t*)(ws + p.ws.cand_key), (uint32_t*)(ws + p.ws.cand_idx), (uint32_t*)(ws + p.ws.cand_cnt),
                     p.N, p.m, p.seg, p.G, p.k, p.gamma_qk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_row_kernel<T, D>), dim3(rows), dim3(256), 0, st, (const uint32_t*)(ws + p.ws.cand_key),
                     (const uint32_t*)(ws + p.ws.cand_idx), (const uint32_t*)(ws + p.ws.cand_cnt),
                     (const float*)(ws + p.ws.qtnorm), (const float*)(ws + p.ws.kmax), p.nsplit,
                     (const double*)(ws + p.ws.qt64), (const T*)K, (int32_t*)(ws + p.ws.I), p.N, p.m, p.seg, p.G, p.k,
                     p.gamma_qk);
  return hipGetLastError();
}

hipError_t launch_topk(const Plan& p, const void* K, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? topk_launch<uint16_t, 64>(p, K, ws, st) : topk_launch<uint16_t, 128>(p, K, ws, st);
  return p.d == 64 ? topk_launch<float, 64>(p, K, ws, st) : topk_launch<float, 128>(p, K, ws, st);
}

}  // namespace mita
