// Step 4: routing. Each query q goes to the s landmarks with the largest
// q . q~_i, ties to the lower landmark id (the MiTA summaries route a query to a
// subset of the deformable experts without giving the rule; this dot-product
// top-s is the reading taken).
//
// Fast kernel (s <= 6): a workgroup takes 64 queries (16 per wave); landmark
// blocks of 64 are staged in LDS and multiplied on MFMA (bf16: Q~ as hi + lo
// parts, so the scores have a proven error E_q = gamma |q| max|q~|). Each lane
// keeps a sorted top list of its landmarks; the four lanes of a query merge
// theirs. If the s-th and (s+1)-th scores are more than 2E_q apart the set is
// certain; otherwise the entries within 2E_q of the s-th score are re-scored in
// fp64 (when the list provably holds all of them), or the query is queued for
// the exact kernel, which scores all m landmarks in fp64 and ranks them. For
// s > 6 every query goes through the exact kernel.
#include "attn_core.h"

namespace mita {

// Insert into a descending top list. Within a lane the landmarks arrive in
// increasing id, so an equal later value must stay below: strict comparison.
template <int TM>
__device__ __forceinline__ void list_insert_ordered(float (&tv)[TM], int (&ti)[TM], float v, int i) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const bool better = v > tv[j];
    const float ov = tv[j];
    const int oi = ti[j];
    tv[j] = better ? v : ov;
    ti[j] = better ? i : oi;
    v = better ? ov : v;
    i = better ? oi : i;
  }
}

// Same with ties broken by the lower id (merging lists of different lanes).
template <int TM>
__device__ __forceinline__ void list_insert(float (&tv)[TM], int (&ti)[TM], float v, int i) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const bool better = v > tv[j] || (v == tv[j] && i < ti[j]);
    const float ov = tv[j];
    const int oi = ti[j];
    tv[j] = better ? v : ov;
    ti[j] = better ? i : oi;
    v = better ? ov : v;
    i = better ? oi : i;
  }
}

template <typename T>
__device__ __forceinline__ double load_f64(const T* p, int c) {
  if constexpr (sizeof(T) == 2) return (double)bf16_to_f32(((const uint16_t*)p)[c]);
  else return (double)p[c];
}

template <typename T, int D, int TM>
__global__ __launch_bounds__(256) void route_fast_kernel(const T* __restrict__ Q, const void* __restrict__ qtop,
                                                         const double* __restrict__ qt64,
                                                         const float* __restrict__ qtnorm, int32_t* __restrict__ E,
                                                         uint32_t* __restrict__ counters, uint32_t* __restrict__ rflag,
                                                         int N, int m, int s, double gamma) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  __shared__ __align__(16) T Ks0[TL::KTILE];
  __shared__ __align__(16) T Ks1[BF ? TL::KTILE : 8];
  __shared__ float s_red[4];
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int q = blockIdx.x * kQueryTile + 16 * w + r;
  const bool q_ok = q < N;
  const T* qrow = Q + ((size_t)z * N + (q_ok ? q : N - 1)) * D;   // padding rows reuse a real row

  // issue every independent load before the first wait: the query fragments,
  // the landmark norms and (inside the loop) the first landmark block
  uint4 qb[1][D / 32];
  float qf[D / 4];
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qb[0][ks] = *(const uint4*)(qrow + 32 * ks + 8 * g);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) qf[ks] = qrow[4 * ks + g];
  }
  float qtm = 0.f;
  for (int i = tid; i < m; i += 256) qtm = fmaxf(qtm, qtnorm[(size_t)z * m + i]);

  float tv[TM];
  int ti[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) { tv[j] = -INFINITY; ti[j] = 0x7FFFFFFF; }

  const T* plane0 = BF ? (const T*)((const uint16_t*)qtop + (size_t)z * 2 * m * D) : (const T*)((const float*)qtop + (size_t)z * m * D);
  const T* plane1 = BF ? plane0 + (size_t)m * D : plane0;
  for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {
    const int nvalid = min(kKeyBlock, m - lb0);
    stage_rows<T, D>(Ks0, TL::KSTR, [&](int rr) { return plane0 + (size_t)(lb0 + rr) * D; }, nvalid, tid);
    if constexpr (BF)
      stage_rows<T, D>(Ks1, TL::KSTR, [&](int rr) { return plane1 + (size_t)(lb0 + rr) * D; }, nvalid, tid);
    __syncthreads();
    f32x4 acc[4];
    if constexpr (BF)
      qk_bf16<D, 2, 1>((const uint16_t*)Ks0, (const uint16_t*)Ks1, qb, acc, lane);
    else
      qk_f32<D>((const float*)Ks0, qf, acc, lane);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int li = lb0 + 16 * kt + 4 * g + j;
        if (li < m) list_insert_ordered<TM>(tv, ti, acc[kt][j], li);
      }
  }
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
    float ov[TM];
    int oi[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) { ov[j] = __shfl_xor(tv[j], sh, WAVE); oi[j] = __shfl_xor(ti[j], sh, WAVE); }
#pragma unroll
    for (int j = 0; j < TM; ++j) list_insert<TM>(tv, ti, ov[j], oi[j]);
  }

  float sq = 0.f;
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const uint16_t* h = (const uint16_t*)&qb[0][ks];
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float x = bf16_to_f32(h[e]); sq = fmaf(x, x, sq); }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks) sq = fmaf(qf[ks], qf[ks], sq);
  }
  const float qn = sqrtf(quad_sum(sq)) * 1.0001f;
  qtm = wave_max(qtm);
  if (lane == 0) s_red[w] = qtm;
  __syncthreads();
  const double qtmax = (double)fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const double Eq = gamma * (double)qn * qtmax;
  // s-th and (s+1)-th entries without dynamic register indexing
  float v_s = -INFINITY, v_s1 = -INFINITY;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    if (j == s - 1) v_s = tv[j];
    if (j == s) v_s1 = tv[j];
  }
  const double That = (double)v_s;
  bool certain = s >= m, refine = false, queue = false;
  if (!certain) {
    certain = (double)v_s - (double)v_s1 > 2.0 * Eq;
    if (!certain) {
      if (m <= TM || (double)tv[TM - 1] < That - 2.0 * Eq) refine = true; else queue = true;
    }
  }
  refine = refine && q_ok;
  int32_t* Eq_out = E + ((size_t)z * N + q) * s;
  if (q_ok && g == 0) {
    if (certain) {
#pragma unroll
      for (int j = 0; j < TM; ++j)
        if (j < s) Eq_out[j] = ti[j];
    } else if (queue) {
      const uint32_t pos = atomicAdd(&counters[0], 1u);
      rflag[pos] = (uint32_t)(z * N + q);
    }
  }
  if (__any(refine)) {
    // fp64 scores of the band entries: the four lanes of a query split d
    double s64[TM];
    bool band[TM];
    int c_in = 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const double v = (double)tv[j];
      band[j] = refine && ti[j] < m && v >= That - 2.0 * Eq && v <= That + 2.0 * Eq;
      c_in += (refine && ti[j] < m && v > That + 2.0 * Eq) ? 1 : 0;
      double part = 0.0;
      if (band[j]) {
        const double* qr = qt64 + ((size_t)z * m + ti[j]) * D;
        for (int e = 0; e < D / 4; ++e) {
          const int c = g * (D / 4) + e;
          part = fma(qr[c], load_f64<T>(qrow, c), part);
        }
      }
      part += __shfl_xor(part, 16, WAVE);
      part += __shfl_xor(part, 32, WAVE);
      s64[j] = part;
    }
    if (refine && g == 0) {
      const int need = s - c_in;
#pragma unroll
      for (int j = 0; j < TM; ++j)
        if (j < c_in) Eq_out[j] = ti[j];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        if (!band[j]) continue;
        int rank = 0;
#pragma unroll
        for (int f = 0; f < TM; ++f)
          rank += (band[f] && (s64[f] > s64[j] || (s64[f] == s64[j] && ti[f] < ti[j]))) ? 1 : 0;
        if (rank < need) Eq_out[c_in + rank] = ti[j];
      }
    }
  }
}

// Exact routing: one wave per query, all m scores in fp64 (kept in LDS), the
// s-th largest found by a bit-serial search over order keys, then the selected
// entries ranked by (score desc, id asc). Processes the queued queries, or all
// queries when `list` is NULL.
template <typename T, int D>
__global__ __launch_bounds__(64) void route_exact_kernel(const T* __restrict__ Q, const double* __restrict__ qt64,
                                                         int32_t* __restrict__ E, const uint32_t* __restrict__ counters,
                                                         const uint32_t* __restrict__ list, int N, int m, int s,
                                                         int total) {
  extern __shared__ double r64[];
  const int lane = threadIdx.x;
  const int count = list ? (int)counters[0] : total;
  for (int t = blockIdx.x; t < count; t += gridDim.x) {
    const int qid = list ? (int)list[t] : t;
    const int z = qid / N;
    const T* qrow = Q + (size_t)qid * D;
    for (int i = lane; i < m; i += 64) {
      const double* qr = qt64 + ((size_t)z * m + i) * D;
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc = fma(qr[c], load_f64<T>(qrow, c), acc);
      r64[i] = acc;
    }
    __syncthreads();
    uint64_t pfx = 0;
    for (int b = 63; b >= 0; --b) {
      const uint64_t cand = pfx | (1ull << b);
      int c = 0;
      for (int i = lane; i < m; i += 64) c += f64_key(r64[i]) >= cand ? 1 : 0;
      if (wave_sum_i(c) >= s) pfx = cand;
    }
    int32_t* Eo = E + (size_t)qid * s;
    for (int i = lane; i < m; i += 64) {
      const uint64_t ki = f64_key(r64[i]);
      if (ki < pfx) continue;
      int rank = 0;
      for (int f = 0; f < m; ++f) {
        const uint64_t kf = f64_key(r64[f]);
        rank += (kf > ki || (kf == ki && f < i)) ? 1 : 0;
      }
      if (rank < s) Eo[rank] = i;
    }
    __syncthreads();
  }
}

template <typename T, int D, int TM>
static hipError_t route_fast_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  hipLaunchKernelGGL((route_fast_kernel<T, D, TM>), dim3(p.qtiles, p.BH), dim3(256), 0, st, (const T*)Q,
                     (const void*)(ws + p.ws.qtop), (const double*)(ws + p.ws.qt64), (const float*)(ws + p.ws.qtnorm),
                     (int32_t*)(ws + p.ws.E), (uint32_t*)(ws + p.ws.counters), (uint32_t*)(ws + p.ws.rflag), p.N, p.m,
                     p.s, p.gamma_qk);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t route_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  hipError_t e = hipSuccess;
  const bool fast = p.s <= kRouteFastMaxS;
  if (fast) {
    if (p.s == 1) e = route_fast_launch<T, D, 3>(p, Q, ws, st);
    else if (p.s == 2) e = route_fast_launch<T, D, 4>(p, Q, ws, st);
    else if (p.s <= 4) e = route_fast_launch<T, D, 6>(p, Q, ws, st);
    else e = route_fast_launch<T, D, 8>(p, Q, ws, st);
    if (e != hipSuccess) return e;
  }
  const int total = p.BH * p.N;
  const int blocks = fast ? 2048 : std::min(total, 65536);
  hipLaunchKernelGGL((route_exact_kernel<T, D>), dim3(blocks), dim3(64), (size_t)p.m * 8, st, (const T*)Q,
                     (const double*)(ws + p.ws.qt64), (int32_t*)(ws + p.ws.E), (const uint32_t*)(ws + p.ws.counters),
                     fast ? (const uint32_t*)(ws + p.ws.rflag) : nullptr, p.N, p.m, p.s, total);
  return hipGetLastError();
}

hipError_t launch_route(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? route_launch<uint16_t, 64>(p, Q, ws, st) : route_launch<uint16_t, 128>(p, Q, ws, st);
  return p.d == 64 ? route_launch<float, 64>(p, Q, ws, st) : route_launch<float, 128>(p, Q, ws, st);
}

}  // namespace mita
