// Step 4: routing. Each query q goes to the s landmarks with the largest
// q . q~_i, ties to the lower landmark id (the MiTA summaries route a query to a
// subset of the deformable experts without giving the rule; this dot-product
// top-s is the reading taken).
//
// Fast kernels (s <= 6): 16 queries per wave; landmark blocks of 64 are staged
// in LDS and multiplied on MFMA (bf16: Q~ as hi + lo parts, so the scores have a
// proven error E_q = gamma |q| max|q~|). Each lane keeps a sorted top list of its
// landmarks' scores (m <= 64: the scores alone, which stay in registers; m > 64:
// float keys that carry the landmark id in their low mantissa bits); the four
// lanes of a query merge theirs. If
// the s-th and (s+1)-th scores are more than 2E_q apart the set is certain;
// otherwise the entries within 2E_q of the s-th score are re-scored in fp64, or
// (m > 64, band longer than the list) the query is queued for the exact kernel,
// which scores all m landmarks in fp64 and ranks them. For s > 6 every query
// goes through the exact kernel. The order of the s ids within a query's list
// is not specified.
#include "attn_core.h"

namespace mita {

// Descending top lists kept with three-input medians: inserting x into
// t[0] >= t[1] >= ... makes the new t[j] the median of the old t[j - 1], t[j]
// and x (t[0]: the maximum), one instruction per entry, all independent.
template <int TM>
__device__ __forceinline__ void top_insert(float (&t)[TM], float x) {
#pragma unroll
  for (int j = TM - 1; j >= 1; --j) t[j] = __builtin_amdgcn_fmed3f(t[j - 1], t[j], x);
  t[0] = fmaxf(t[0], x);
}
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}
template <int TM>
__device__ __forceinline__ void top_insert(uint32_t (&t)[TM], uint32_t x) {
#pragma unroll
  for (int j = TM - 1; j >= 1; --j) t[j] = med3_u32(t[j - 1], t[j], x);
  t[0] = max(t[0], x);
}

// Landmark score as a float key that carries its landmark id: the score with its
// low ib mantissa bits replaced by imask - id (imask = 2^ib - 1 >= m - 1). Keys of
// one query are distinct floats (finite: the exponent is untouched; scores near
// zero become denormals, which the kernels keep), ordered by value with three-input
// medians, one instruction per list entry; the empty entry is -inf. A key bounds its
// score from both sides: the score has the key's bits above the low ib, so it lies
// between the key with those bits cleared and with them set.
struct RouteKey {
  uint32_t imask;
  // idb: the id bits imask - id; nmask: ~imask
  __device__ __forceinline__ float make(float v, uint32_t idb, uint32_t nmask) const {
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, v) & nmask) | idb);
  }
  __device__ __forceinline__ int id(float k) const { return (int)(imask - (__builtin_bit_cast(uint32_t, k) & imask)); }
  __device__ __forceinline__ double lo(float k) const {
    const uint32_t u = __builtin_bit_cast(uint32_t, k);
    return (double)fminf(__builtin_bit_cast(float, u & ~imask), __builtin_bit_cast(float, u | imask));
  }
  __device__ __forceinline__ double hi(float k) const {
    const uint32_t u = __builtin_bit_cast(uint32_t, k);
    return (double)fmaxf(__builtin_bit_cast(float, u & ~imask), __builtin_bit_cast(float, u | imask));
  }
};
// Insert a key into a descending list of keys; the new maximum is the median of
// the old one, x and pinf = +inf. pinf comes from a run-time value: with a literal
// +inf the compiler turns the median into a maximum, which then quiets both
// operands first (three instructions instead of one).
template <int TM>
__device__ __forceinline__ void key_insert(float (&t)[TM], float x, float pinf) {
#pragma unroll
  for (int j = TM - 1; j >= 1; --j) t[j] = __builtin_amdgcn_fmed3f(t[j - 1], t[j], x);
  t[0] = __builtin_amdgcn_fmed3f(t[0], x, pinf);
}

template <typename T>
__device__ __forceinline__ double load_f64(const T* p, int c) {
  if constexpr (sizeof(T) == 2) return (double)bf16_to_f32(((const uint16_t*)p)[c]);
  else return (double)p[c];
}

// Exact top-s of one query by one wave: every landmark is scored in fp64 against
// the fp64 Q~ rows into r64 (m doubles of LDS), then for s <= 16 the winners are
// taken one at a time by a wave arg-max over (score desc, id asc); for larger s
// the s-th largest order key is found by a bit-serial search and the entries at
// or above it are ranked. Scoring: 8 lanes per landmark row, lane k of the eight
// taking 16 bytes of every 128-byte piece of it, so a load instruction reads 8
// rows of whole cache lines (a row per lane would touch 64 lines per instruction
// and leave the wave waiting on the address unit); the lane's query elements stay
// in registers, and the eight partial sums meet in three lane exchanges. RPP
// groups of 8 rows are in flight per pass.
template <typename T, int D, int RPP>
__device__ __forceinline__ void exact_route_wave(const T* qrow, const double* qt64z, int m, int s,
                                                 int32_t* Eo, double* r64, int lane) {
  constexpr int NC = D / 16;   // 128-byte pieces per row
  const int rg = lane >> 3, k = lane & 7;
  double qv[2 * NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qv[2 * c] = load_f64<T>(qrow, 16 * c + 2 * k);
    qv[2 * c + 1] = load_f64<T>(qrow, 16 * c + 2 * k + 1);
  }
  for (int i0 = 0; i0 < m; i0 += 8 * RPP) {
    double2 x[RPP][NC];
#pragma unroll
    for (int h = 0; h < RPP; ++h) {
      const double2* qr = (const double2*)(qt64z + (size_t)min(i0 + 8 * h + rg, m - 1) * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) x[h][c] = qr[8 * c + k];
    }
#pragma unroll
    for (int h = 0; h < RPP; ++h) {
      double a = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        a = fma(x[h][c].x, qv[2 * c], a);
        a = fma(x[h][c].y, qv[2 * c + 1], a);
      }
      a += __shfl_xor(a, 1, WAVE);
      a += __shfl_xor(a, 2, WAVE);
      a += __shfl_xor(a, 4, WAVE);
      if (k == 0 && i0 + 8 * h + rg < m) r64[i0 + 8 * h + rg] = a;
    }
  }
  wave_sync();
  if (s <= 16) {
    for (int rnd = 0; rnd < s; ++rnd) {
      double bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int i = lane; i < m; i += 64) {   // ids ascend within a lane: strict > keeps the lower id
        const double v = r64[i];
        if (v > bv) { bv = v; bi = i; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const double ov = __shfl_xor(bv, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
        bv = take ? ov : bv;
        bi = take ? oi : bi;
      }
      if (lane == 0) {
        Eo[rnd] = bi;
        r64[bi] = -INFINITY;   // scores are finite, so a taken entry never wins again
      }
      wave_sync();
    }
  } else {
    uint64_t pfx = 0;
    for (int b = 63; b >= 0; --b) {
      const uint64_t cand = pfx | (1ull << b);
      int c = 0;
      for (int i = lane; i < m; i += 64) c += f64_key(r64[i]) >= cand ? 1 : 0;
      if (wave_sum_i(c) >= s) pfx = cand;
    }
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
  }
  wave_sync();
}

// Fast router for m <= 64: the landmark block is staged once for all the
// workgroup's query tiles, and each query's m scores are still in registers
// when its set is decided: band members are re-scored in fp64 right there.
template <typename T, int D, int TM>
__global__ __launch_bounds__(256) void route_fast_kernel(const T* __restrict__ Q, const void* __restrict__ qtop,
                                                         const double* __restrict__ qt64,
                                                         const float* __restrict__ qtnorm, int32_t* __restrict__ E,
                                                         uint32_t* __restrict__ counters, uint32_t* __restrict__ rflag,
                                                         int N, int m, int s, double gamma, int qtiles, int tpw) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  __shared__ __align__(16) T Ks0[TL::KTILE];
  __shared__ __align__(16) T Ks1[BF ? TL::KTILE : 8];
  __shared__ float s_red[4];
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * tpw, t1 = min(qtiles, t0 + tpw);
  const T* plane0 = BF ? (const T*)((const uint16_t*)qtop + (size_t)z * 2 * m * D) : (const T*)((const float*)qtop + (size_t)z * m * D);
  const T* plane1 = BF ? plane0 + (size_t)m * D : plane0;
  const double* qt64z = qt64 + (size_t)z * m * D;
  auto stage = [&](int lb0) {
    const int nvalid = min(kKeyBlock, m - lb0);
    stage_rows<T, D>(Ks0, TL::KSTR, [&](int rr) { return plane0 + (size_t)(lb0 + rr) * D; }, nvalid, tid);
    if constexpr (BF)
      stage_rows<T, D>(Ks1, TL::KSTR, [&](int rr) { return plane1 + (size_t)(lb0 + rr) * D; }, nvalid, tid);
  };
  auto qrow_of = [&](int t) {   // this thread's query row of tile t (padding rows reuse a real row)
    const int q = min(t * kQueryTile + 16 * w + r, N - 1);
    return Q + ((size_t)z * N + q) * D;
  };
  auto load_q = [&](uint4 (&qb)[1][D / 32], float (&qf)[D / 4], const T* qrow) {
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qb[0][ks] = ld16(qrow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) qf[ks] = qrow[4 * ks + g];
    }
  };

  // independent loads first: the first query tile, the landmark norms, the landmark block
  uint4 qb[1][D / 32], qb_n[1][D / 32];
  float qf[D / 4], qf_n[D / 4];
  load_q(qb_n, qf_n, qrow_of(t0));
  float qtm = 0.f;
  for (int i = tid; i < m; i += 256) qtm = fmaxf(qtm, qtnorm[(size_t)z * m + i]);
  stage(0);
  qtm = wave_max(qtm);
  if (lane == 0) s_red[w] = qtm;
  __syncthreads();
  const double qtmax = (double)fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  for (int t = t0; t < t1; ++t) {
    const int q = t * kQueryTile + 16 * w + r;
    const bool q_ok = q < N;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qb[0][ks] = qb_n[0][ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) qf[ks] = qf_n[ks];
    }
    load_q(qb_n, qf_n, qrow_of(min(t + 1, t1 - 1)));   // next tile's rows in flight

    float tv[TM];   // the TM largest scores of the lane, then of the query
#pragma unroll
    for (int j = 0; j < TM; ++j) tv[j] = -INFINITY;
    f32x4 acc[4];
    for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {   // one block (m <= 64)
      if constexpr (BF)
        qk_bf16<D, 2, 1>((const uint16_t*)Ks0, (const uint16_t*)Ks1, qb, acc, lane);
      else
        qk_f32<D>((const float*)Ks0, qf, acc, lane);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int li = lb0 + 16 * kt + 4 * g + j;   // past m: -inf
          if (li >= m) acc[kt][j] = -INFINITY;
          top_insert<TM>(tv, acc[kt][j]);
        }
    }
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      float ov[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) ov[j] = __shfl_xor(tv[j], sh, WAVE);
#pragma unroll
      for (int j = 0; j < TM; ++j) top_insert<TM>(tv, ov[j]);
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
    const double Eq = gamma * (double)qn * qtmax;
    // s-th and (s+1)-th scores without dynamic register indexing
    float v_s = -INFINITY, v_s1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j == s - 1) v_s = tv[j];
      if (j == s) v_s1 = tv[j];
    }
    const double That = (double)v_s, lo = That - 2.0 * Eq, hi = That + 2.0 * Eq;
    const bool certain = s >= m || (double)v_s - (double)v_s1 > 2.0 * Eq;
    const bool unc = q_ok && !certain;
    int32_t* Eq_out = E + ((size_t)z * N + min(q, N - 1)) * s;
    // Landmarks of the query in a mask over its quad (bit 16 g' + 4 kt + j: lane
    // g' of the quad, score acc[kt][j]) and written to Eq_out[base ..] by one
    // lane per member. Certain: the s scores >= v_s (more than 2 E_q above the
    // rest, so no tie at the boundary). Uncertain: those above the band are in,
    // the band is re-scored in fp64.
    auto quad_mask = [&](auto pred) {   // the query's scores that satisfy pred
      uint32_t mk = 0;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mk |= pred(acc[kt][j]) ? 1u << (4 * kt + j) : 0u;
      uint64_t qm = 0;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) qm |= (uint64_t)__shfl(mk, r + 16 * gg, WAVE) << (16 * gg);
      return qm;
    };
    auto landmark_of = [](int bit) { const int b = bit & 15; return 16 * (b >> 2) + 4 * (bit >> 4) + (b & 3); };
    auto write_mask = [&](uint64_t qm, int base) {   // same trip count on the four lanes of a query
      int pos = base;
      while (qm) {
        const int bit = __builtin_ctzll(qm);
        qm &= qm - 1;
        if (g == 0) Eq_out[pos] = landmark_of(bit);
        ++pos;
      }
      return pos;
    };
    {
      const bool take = q_ok && certain;
      const uint64_t qm = quad_mask([&](float v) { return take && v >= v_s; });
      write_mask(qm, 0);
    }
    if (!__any(unc)) continue;

    // entries above the band are in for sure; the band is ranked in fp64
    const uint64_t in_m = quad_mask([&](float v) { return unc && (double)v > hi; });
    const int c_in = write_mask(in_m, 0);
    const int need = s - c_in;
    // fp64 partial dot of this lane's share of the query with landmark li
    auto part64 = [&](int li) {
      const double* qr = qt64z + (size_t)li * D;
      double part = 0.0;
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const uint16_t* h = (const uint16_t*)&qb[0][ks];
#pragma unroll
          for (int e = 0; e < 8; ++e) part = fma(qr[32 * ks + 8 * g + e], (double)bf16_to_f32(h[e]), part);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 4; ++ks) part = fma(qr[4 * ks + g], (double)qf[ks], part);
      }
      part += __shfl_xor(part, 16, WAVE);
      return part + __shfl_xor(part, 32, WAVE);
    };
    // every score of the query is in acc (lanes of the quad hold 16 each):
    // the band members are re-scored one by one, quad-uniformly
    uint64_t qm = quad_mask([&](float v) { return unc && (double)v >= lo && (double)v <= hi; });
    double bv[TM];
    int bi[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) { bv[j] = -INFINITY; bi[j] = 0x7FFFFFFF; }
    while (qm) {   // same trip count on the four lanes of a query
      const int bit = __builtin_ctzll(qm);
      qm &= qm - 1;
      double v = part64(landmark_of(bit));
      int i = landmark_of(bit);
#pragma unroll
      for (int j = 0; j < TM; ++j) {   // insert by (score desc, id asc)
        const bool better = (v > bv[j]) | ((v == bv[j]) & (i < bi[j]));
        const double ov = bv[j];
        const int oi = bi[j];
        bv[j] = better ? v : ov;
        bi[j] = better ? i : oi;
        v = better ? ov : v;
        i = better ? oi : i;
      }
    }
    if (unc && g == 0) {
#pragma unroll
      for (int j = 0; j < TM; ++j)
        if (j < need) Eq_out[c_in + j] = bi[j];
    }
  }
}

// Fast router for m > 64: a workgroup takes TPW query tiles at once (their query
// fragments and top lists stay in registers) and streams the landmark blocks
// through LDS once for all of them, so each block is staged once per TPW tiles.
// At least three waves per SIMD (the gathers of Q rows need the occupancy); the
// d = 128 forms fit in 120 VGPRs and run four.
// A query is certain, or its band is re-scored in fp64 when the list holds it,
// or it is queued for the exact kernel.
template <typename T, int D, int TM, int TPW, bool MFULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void route_multi_kernel(const T* __restrict__ Q, const void* __restrict__ qtop,
                                                          const double* __restrict__ qt64,
                                                          const float* __restrict__ qtnorm, int32_t* __restrict__ E,
                                                          uint32_t* __restrict__ counters,
                                                          uint32_t* __restrict__ rflag, int N, int m, int s,
                                                          double gamma, int qtiles) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  __shared__ __align__(16) T Ks0[BF ? 8 : TL::KTILE];   // fp32 key tile (bf16 tiles: below)
  __shared__ float s_red[4];
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * TPW;
  const T* plane0 = BF ? (const T*)((const uint16_t*)qtop + (size_t)z * 2 * m * D) : (const T*)((const float*)qtop + (size_t)z * m * D);
  const T* plane1 = BF ? plane0 + (size_t)m * D : plane0;
  const double* qt64z = qt64 + (size_t)z * m * D;

  // query fragments of the TPW tiles (tiles past the end repeat the last row)
  uint4 qb[TPW][D / 32];
  float qf[TPW][D / 4];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int q = min((t0 + tt) * kQueryTile + 16 * w + r, N - 1);
    const T* qrow = Q + ((size_t)z * N + q) * D;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qb[tt][ks] = ld16(qrow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) qf[tt][ks] = qrow[4 * ks + g];
    }
  }
  float qtm = 0.f;
  for (int i = tid; i < m; i += 256) qtm = fmaxf(qtm, qtnorm[(size_t)z * m + i]);
  qtm = wave_max(qtm);
  if (lane == 0) s_red[w] = qtm;

  const RouteKey rk{(2u << (31 - __builtin_clz((uint32_t)(m - 1)))) - 1u};   // m > 64: imask >= m - 1
  const float pinf = __builtin_bit_cast(float, 0x7F800000u | ((uint32_t)m >> 31));   // +inf (m > 0)
  float tk[TPW][TM];   // the TM largest keys of the lane, then of the query
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int j = 0; j < TM; ++j) tk[tt][j] = -INFINITY;
  // In the block loop a key's id bits leave out the lane's 4 g: imask - (lb0 + 16 kt
  // + j) = (imask - lb0) ^ (16 kt + j) (the low 6 bits of imask - lb0 are ones) is
  // the same for every lane, a scalar, so a key costs one instruction. A lane's
  // ids are still distinct; 4 g is put in after the loop (bits 2-3 of every such
  // id are ones, so XOR 4 g subtracts it and keeps the lane's order).
  // ~imask in a vector register (the result of a lane exchange counts as
  // per-lane), so that with the scalar id bits a key is one v_and_or_b32 (a vector
  // instruction reads at most one scalar register)
  const uint32_t nmask = (uint32_t)__shfl((int)~rk.imask, lane, WAVE);
  auto take = [&](const f32x4 (&acct)[TPW][4], int lb0) {
    const uint32_t cb = rk.imask - (uint32_t)lb0;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int li = lb0 + 16 * kt + 4 * g + j;
          const float key = rk.make(acct[tt][kt][j], cb ^ (uint32_t)(16 * kt + j), nmask);
          // past m: -inf, which never enters the list (a bit select: a conditional
          // here compiled to a branch per score); none when m is a multiple of the block
          const uint32_t keep = (uint32_t)((li - m) >> 31);
          key_insert<TM>(tk[tt],
                         MFULL ? key
                               : __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, key) & keep) | (0xFF800000u & ~keep)),
                         pinf);
        }
  };
  if constexpr (BF) {
    // Landmark blocks (hi and lo planes of Q~) by direct loads into swizzled
    // tiles, one buffer: once every wave has read a block, the next block's loads
    // are issued and fly while the top lists take this block's scores. The loads
    // go through one buffer resource over both planes: a lane's offset within a
    // block is fixed, the block's offset a scalar. Rows past m read the lo plane
    // or, past its end, zeros: finite scores, masked by index.
    __shared__ __align__(16) uint16_t Th[UTile<D>::TILE];
    __shared__ __align__(16) uint16_t Tl[UTile<D>::TILE];
    using U = UTile<D>;
    constexpr int NI = kKeyBlock / 4 / U::RPI;   // load instructions per wave per tile
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(plane0, 2u * (uint32_t)m * D * 2);
    uint32_t voff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int row = 16 * w + u * U::RPI + lane / U::CPR;
      voff[u] = (uint32_t)row * (D * 2) + 16 * ((lane % U::CPR) ^ U::swz_k(row));
    }
    const int ws = __builtin_amdgcn_readfirstlane(w);   // LDS bases in scalar registers
    auto stage = [&](int lb0) {
      const uint32_t sh = (uint32_t)lb0 * (D * 2), sl = sh + (uint32_t)m * (D * 2);
#pragma unroll
      for (int u = 0; u < NI; ++u) lds_dma16_buf(rs, voff[u], sh, Th + (16 * ws + u * U::RPI) * D);
#pragma unroll
      for (int u = 0; u < NI; ++u) lds_dma16_buf(rs, voff[u], sl, Tl + (16 * ws + u * U::RPI) * D);
    };
    stage(0);
    for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();   // the block is in LDS (every wave's share)
      // per score the MFMA sequence of the padded-tile form: k-slices in order,
      // hi then lo plane
      f32x4 acct[TPW][4];
      uqk<D, TPW, 2>(Th, Tl, qb, acct, lane);
      __syncthreads();   // every wave has read the block
      if (lb0 + kKeyBlock < m) stage(lb0 + kKeyBlock);   // block-uniform
      take(acct, lb0);
    }
  } else {
    for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {
      __syncthreads();   // readers of the previous block are done
      const int nvalid = min(kKeyBlock, m - lb0);
      stage_rows<T, D>(Ks0, TL::KSTR, [&](int rr) { return plane0 + (size_t)(lb0 + rr) * D; }, nvalid, tid);
      __syncthreads();
      f32x4 acct[TPW][4];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acct[tt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      constexpr int KSTR = TL::KSTR;
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const float a = ((const float*)Ks0)[(16 * kt + r) * KSTR + 4 * ks + g];
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) acct[tt][kt] = mma_f32(a, qf[tt][ks], acct[tt][kt]);
        }
      take(acct, lb0);
    }
  }
  __syncthreads();   // s_red (written before the loop) for every wave
  const double qtmax = (double)fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int q = (t0 + tt) * kQueryTile + 16 * w + r;
    const bool q_ok = (t0 + tt) < qtiles && q < N;
    const T* qrow = Q + ((size_t)z * N + min(q, N - 1)) * D;
#pragma unroll
    for (int j = 0; j < TM; ++j)   // the lane's 4 g into the id bits (-inf: an empty entry)
      if (tk[tt][j] != -INFINITY) tk[tt][j] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, tk[tt][j]) ^ (4u * g));
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      float ok[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) ok[j] = __shfl_xor(tk[tt][j], sh, WAVE);
#pragma unroll
      for (int j = 0; j < TM; ++j) key_insert<TM>(tk[tt], ok[j], pinf);
    }
    float sq = 0.f;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const uint16_t* h = (const uint16_t*)&qb[tt][ks];
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float x = bf16_to_f32(h[e]); sq = fmaf(x, x, sq); }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) sq = fmaf(qf[tt][ks], qf[tt][ks], sq);
    }
    const float qn = sqrtf(quad_sum(sq)) * 1.0001f;
    const double Eq = gamma * (double)qn * qtmax;
    // s-th and (s+1)-th keys without dynamic register indexing; each key bounds
    // its score from both sides, so the s-th score lies in [lo(k_s), hi(k_s)]
    float k_s = -INFINITY, k_s1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j == s - 1) k_s = tk[tt][j];
      if (j == s) k_s1 = tk[tt][j];
    }
    const double lo = rk.lo(k_s) - 2.0 * Eq, hi = rk.hi(k_s) + 2.0 * Eq;
    const bool certain = s >= m || rk.lo(k_s) - rk.hi(k_s1) > 2.0 * Eq;
    int32_t* Eq_out = E + ((size_t)z * N + min(q, N - 1)) * s;
    if (q_ok && g == 0 && certain) {
#pragma unroll
      for (int j = 0; j < TM; ++j)
        if (j < s) Eq_out[j] = rk.id(tk[tt][j]);
    }
    const bool unc = q_ok && !certain;
    if (!__any(unc)) continue;
    // in for sure: keys whose lowest possible score is above the band (they lead the list)
    int c_in = 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) c_in += (j < s && rk.lo(tk[tt][j]) > hi) ? 1 : 0;
    if (unc && g == 0) {
#pragma unroll
      for (int j = 0; j < TM; ++j)
        if (j < c_in) Eq_out[j] = rk.id(tk[tt][j]);
    }
    // the list holds the whole band when its last key's highest possible score is below it
    const bool refine = unc && rk.hi(tk[tt][TM - 1]) < lo;
    if (unc && !refine && g == 0) {
      const uint32_t pos = atomicAdd(&counters[0], 1u);
      rflag[pos] = (uint32_t)(z * N + q);
    }
    // Band re-scoring in fp64, compacted: the wave takes its queries to refine two
    // at a time (lanes 32 slot .. + 31 for one query, 4 lanes per list entry, each
    // a quarter of the row), so a tile with one uncertain query pays for that one.
    uint64_t rq = __ballot(refine && g == 0);   // bit r: query r of the tile (lane r is its g = 0 lane)
    while (rq) {   // wave-uniform
      const int s0 = __builtin_ctzll(rq);
      rq &= rq - 1;
      const int s1 = rq ? __builtin_ctzll(rq) : -1;
      if (rq) rq &= rq - 1;
      const int slot = lane >> 5, j = (lane & 31) >> 2, part = lane & 3;
      const int src = slot ? s1 : s0;
      const int srcl = max(src, 0);
      const bool act = src >= 0 && j < TM;
      // the query's list, band and count above it, from its lane
      float kk[TM];
#pragma unroll
      for (int f = 0; f < TM; ++f) kk[f] = __shfl(tk[tt][f], srcl, WAVE);
      const double blo = __shfl(lo, srcl, WAVE);
      const int cin = __shfl(c_in, srcl, WAVE);
      float myk = kk[0];
#pragma unroll
      for (int f = 1; f < TM; ++f) myk = f == j ? kk[f] : myk;
      const int myid = rk.id(myk);
      const int qs = (t0 + tt) * kQueryTile + 16 * w + srcl;
      double acc = 0.0;
      if (act) {
        constexpr int QD = D / 4;   // elements per lane
        const double2* qr = (const double2*)(qt64z + (size_t)myid * D + QD * part);
        const T* qrow = Q + ((size_t)z * N + qs) * D + QD * part;
        if constexpr (BF) {
#pragma unroll
          for (int c = 0; c < QD / 8; ++c) {
            const uint4 u = ((const uint4*)qrow)[c];
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double2 t = qr[4 * c + e];
              acc = fma(t.x, (double)__builtin_bit_cast(float, uw[e] << 16), acc);
              acc = fma(t.y, (double)__builtin_bit_cast(float, uw[e] & 0xFFFF0000u), acc);
            }
          }
        } else {
#pragma unroll
          for (int c = 0; c < QD / 4; ++c) {
            const float4 x = ((const float4*)qrow)[c];
            const double2 t0v = qr[2 * c], t1v = qr[2 * c + 1];
            acc = fma(t0v.x, (double)x.x, acc);
            acc = fma(t0v.y, (double)x.y, acc);
            acc = fma(t1v.x, (double)x.z, acc);
            acc = fma(t1v.y, (double)x.w, acc);
          }
        }
      }
      acc += __shfl_xor(acc, 1, WAVE);
      acc += __shfl_xor(acc, 2, WAVE);
      double sv[TM];
#pragma unroll
      for (int f = 0; f < TM; ++f) sv[f] = __shfl(acc, 32 * slot + 4 * f, WAVE);
      if (act && part == 0) {
        bool band[TM];
        double mysv = sv[0];
        bool myband = false;
#pragma unroll
        for (int f = 0; f < TM; ++f) {
          band[f] = f >= cin && kk[f] != -INFINITY && rk.hi(kk[f]) >= blo;
          if (f == j) {
            mysv = sv[f];
            myband = band[f];
          }
        }
        if (myband) {
          int rank = 0;   // by (fp64 score desc, id asc) among the band
#pragma unroll
          for (int f = 0; f < TM; ++f) {
            const int idf = rk.id(kk[f]);
            rank += (band[f] && ((sv[f] > mysv) | ((sv[f] == mysv) & (idf < myid)))) ? 1 : 0;
          }
          if (rank < s - cin) E[((size_t)z * N + qs) * s + cin + rank] = myid;
        }
      }
    }
  }
}

// Exact routing kernel: one wave per query (up to four per workgroup), for the
// queries the fast kernel queued or for all queries when `list` is NULL (s > 6).
template <typename T, int D>
__global__ __launch_bounds__(256) void route_exact_kernel(const T* __restrict__ Q, const double* __restrict__ qt64,
                                                          int32_t* __restrict__ E, const uint32_t* __restrict__ counters,
                                                          const uint32_t* __restrict__ list, int N, int m, int s,
                                                          int total) {
  extern __shared__ double x64[];   // per wave: [m] scores (and D doubles not used)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double* r64 = x64 + (size_t)w * (m + D);
  const int count = list ? (int)counters[0] : total;
  const int nw = blockDim.x >> 6;
  for (int t = blockIdx.x * nw + w; t < count; t += gridDim.x * nw) {
    const int qid = list ? (int)list[t] : t;
    const int z = qid / N;
    exact_route_wave<T, D, 2>(Q + (size_t)qid * D, qt64 + (size_t)z * m * D, m, s, E + (size_t)qid * s, r64, lane);
  }
}

// m <= 64: every query is settled in route_fast_kernel (all its scores at hand).
// Larger m: route_multi_kernel, with the queries its lists cannot settle queued
// for the exact kernel.
template <typename T, int D, int TM, bool RES>
static hipError_t route_fast_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  if constexpr (RES) {
    // several query tiles per workgroup (the landmarks stay staged), as many as
    // make the grid one round of resident workgroups
    static PerDevice occ;
    const int slots = device_cu_count() * resident_per_cu(occ, route_fast_kernel<T, D, TM>, 256);
    const int per_slice = std::max(1, slots / p.BH);
    const int tpw = (p.qtiles + per_slice - 1) / per_slice;
    hipLaunchKernelGGL((route_fast_kernel<T, D, TM>), dim3((p.qtiles + tpw - 1) / tpw, p.BH), dim3(256), 0,
                       st, (const T*)Q, (const void*)(ws + p.ws.qtop), (const double*)(ws + p.ws.qt64),
                       (const float*)(ws + p.ws.qtnorm), (int32_t*)(ws + p.ws.E), (uint32_t*)(ws + p.ws.counters),
                       (uint32_t*)(ws + p.ws.rflag), p.N, p.m, p.s, p.gamma_qk, p.qtiles, tpw);
  } else {
    // landmark blocks streamed once per TPW query tiles (fewer when the query
    // fragments of all TPW tiles would crowd the registers)
    constexpr int TPW = (sizeof(T) == 2 && D == 64) ? 4 : 2;
    // the rare queries the lists cannot settle go to the exact kernel (an in-kernel
    // exact pass would cost every workgroup its registers)
    auto kern = p.m % kKeyBlock == 0 ? route_multi_kernel<T, D, TM, TPW, true> : route_multi_kernel<T, D, TM, TPW, false>;
    hipLaunchKernelGGL(kern, dim3((p.qtiles + TPW - 1) / TPW, p.BH), dim3(256), 0, st, (const T*)Q,
                       (const void*)(ws + p.ws.qtop), (const double*)(ws + p.ws.qt64), (const float*)(ws + p.ws.qtnorm),
                       (int32_t*)(ws + p.ws.E), (uint32_t*)(ws + p.ws.counters), (uint32_t*)(ws + p.ws.rflag), p.N,
                       p.m, p.s, p.gamma_qk, p.qtiles);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t route_launch(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  hipError_t e = hipSuccess;
  const bool fast = p.s <= kRouteFastMaxS;
  if (fast) {
    // m <= 64: lists of s + 1 entries certify the set, and the band is re-scored
    // from the scores in registers. Larger m: lists of s + 2, so that the band
    // of an uncertain query usually ends inside the list and is re-scored
    // there; the rest is queued.
    if (p.m <= kKeyBlock) {
      if (p.s == 1) e = route_fast_launch<T, D, 2, true>(p, Q, ws, st);
      else if (p.s == 2) e = route_fast_launch<T, D, 3, true>(p, Q, ws, st);
      else if (p.s <= 4) e = route_fast_launch<T, D, 5, true>(p, Q, ws, st);
      else e = route_fast_launch<T, D, 7, true>(p, Q, ws, st);
    } else {
      if (p.s == 1) e = route_fast_launch<T, D, 3, false>(p, Q, ws, st);
      else if (p.s == 2) e = route_fast_launch<T, D, 4, false>(p, Q, ws, st);
      else if (p.s <= 4) e = route_fast_launch<T, D, 6, false>(p, Q, ws, st);
      else e = route_fast_launch<T, D, 8, false>(p, Q, ws, st);
    }
    if (e != hipSuccess) return e;
    if (p.m <= kKeyBlock) return hipSuccess;   // settled in the fast kernel
  }
  const int total = p.BH * p.N;
  const int nw = (size_t)4 * (p.m + p.d) * 8 <= 65536 ? 4 : 1;   // LDS: m scores + the query row per wave
  const int blocks = fast ? 4096 / nw : std::min((total + nw - 1) / nw, 65536);
  hipLaunchKernelGGL((route_exact_kernel<T, D>), dim3(blocks), dim3(64 * nw), (size_t)nw * (p.m + p.d) * 8, st,
                     (const T*)Q, (const double*)(ws + p.ws.qt64), (int32_t*)(ws + p.ws.E),
                     (const uint32_t*)(ws + p.ws.counters), fast ? (const uint32_t*)(ws + p.ws.rflag) : nullptr, p.N,
                     p.m, p.s, total);
  return hipGetLastError();
}

// Routing beside steps 2-3 (on a second stream) pays while its grid is short, at
// most two rounds of resident workgroups (taken as four per CU, the fast router's
// occupancy), or for d = 64, whose shared-expert and top-k kernels leave more of
// the CUs' issue slots idle. A longer d = 128 routing grid only competes with those
// kernels for the same CUs, and the forward runs better with routing first on the
// caller's stream (measured: very long 6.75 -> 6.59 ms, long 2.99 -> 2.89 ms in
// line; seg-like, d = 64 and 6144 routing workgroups: 1.43 ms beside, 1.49 ms in
// line).
bool route_alongside(const Plan& p) {
  if (p.m <= kKeyBlock && p.s <= kRouteFastMaxS) return true;   // one round by construction
  if (p.d == 64) return true;
  const int64_t wgs = p.s <= kRouteFastMaxS ? (int64_t)((p.qtiles + 1) / 2) * p.BH   // two query tiles per workgroup
                                            : ((int64_t)p.BH * p.N + 3) / 4;        // exact kernel: four queries
  return wgs <= 2LL * 4 * device_cu_count();
}

hipError_t launch_route(const Plan& p, const void* Q, char* ws, hipStream_t st) {
  if (p.dtype == MITA_BF16) return p.d == 64 ? route_launch<uint16_t, 64>(p, Q, ws, st) : route_launch<uint16_t, 128>(p, Q, ws, st);
  return p.d == 64 ? route_launch<float, 64>(p, Q, ws, st) : route_launch<float, 128>(p, Q, ws, st);
}

}  // namespace mita
