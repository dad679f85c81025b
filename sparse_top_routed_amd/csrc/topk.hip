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

template <typename T, int D>
static hipError_t topk_launch(const Plan& p, const void* K, char* ws, hipStream_t st) {
  const int rows = p.BH * p.m;
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
