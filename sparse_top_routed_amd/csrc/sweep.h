// Key sweeps of a workgroup of 64 landmarks (16 per wave) over a range of keys,
// shared by the shared-expert kernel (step 2) and the candidate kernel (step 3).
//
// Both sweeps stream the keys through LDS 64 at a time (the next blocks are
// fetched into registers while the current one computes) and compute the same
// approximate scores q~_i . K_n with the same MFMA sequence on the same operands,
// so a score seen by the candidate sweep has the bits the shared-expert sweep
// saw (the exactness argument of step 3 depends on it).
#pragma once
#include <type_traits>

#include "attn_core.h"

namespace mita {

// The wave's 16 landmark rows as MFMA operands: bf16 inputs take Q~ as two bf16
// parts (hi + lo, ~16 more bits than a bf16 Q~), fp32 inputs take Q~ in fp32.
template <typename T, int D>
struct LmFrag {
  static constexpr bool BF = sizeof(T) == 2;
  uint4 qb[2][D / 32];
  float qf[D / 4];
  __device__ __forceinline__ void load(const void* qtop, int z, int m, int lmc, int g) {
    if constexpr (BF) {
      const uint16_t* qt = (const uint16_t*)qtop;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          qb[p][ks] = ld16(qt + ((size_t)(z * 2 + p) * m + lmc) * D + 32 * ks + 8 * g);
    } else {
      const float* qt = (const float*)qtop;
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) qf[ks] = qt[((size_t)z * m + lmc) * D + 4 * ks + g];
    }
  }
  // S^T tile of the staged 64-key block: lane holds keys 16 kt + 4 (lane / 16) + j
  // of landmark lane % 16.
  __device__ __forceinline__ void scores(const T* Ks, f32x4 (&acc)[4], int lane) const {
    if constexpr (BF)
      qk_bf16<D, 1, 2>((const uint16_t*)Ks, nullptr, qb, acc, lane);
    else
      qk_f32<D>((const float*)Ks, qf, acc, lane);
  }
};

// Online-softmax state of the shared expert for the lane's landmark.
template <int D>
struct LmState {
  float mrun, lrun;
  f32x4 o[D / 16];
  __device__ __forceinline__ void init() {
    mrun = -INFINITY;
    lrun = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Shared-expert sweep over keys [k0, k1) (k1 > k0): online softmax of the
// scores against V, the maxima of groups of gq (4: a lane's share of one 16-key
// tile; 16: its share of a block; 64: a block) scores into Brow[group] (the
// global group index), the
// scores into Srow when it is not null, and, when `norms`, the largest squared
// key norm seen into kmx (per thread; reduce over the workgroup).
template <typename T, int D>
__device__ __forceinline__ void shared_expert_sweep(const T* Kz, const T* Vz, int k0, int k1, const LmFrag<T, D>& qfr,
                                                    T* Ks, T* Vs, bool norms, float& kmx, float* Brow, int gq,
                                                    float* Srow, bool vec_store, bool lm_ok, float sl2e,
                                                    LmState<D>& st, int tid) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  const int lane = tid & 63, g = lane >> 4;
  const int last_kb = k0 + ((k1 - k0 - 1) / kKeyBlock) * kKeyBlock;
  RowRegs<T, D> KR;
  std::conditional_t<BF, VtRegs<D>, RowRegs<T, D>> VR;
  auto fetch = [&](int kb) {   // blocks past the end repeat the last block: no branch
    const int nb = min(kb, last_kb);
    const int nv = min(kKeyBlock, k1 - nb);
    KR.load([&](int rr) { return Kz + (size_t)(nb + rr) * D; }, nv, tid);
    VR.load([&](int rr) { return Vz + (size_t)(nb + rr) * D; }, nv, tid);
  };
  fetch(k0);

  for (int kb = k0; kb < k1; kb += kKeyBlock) {
    const int nvalid = min(kKeyBlock, k1 - kb);
    KR.store(Ks, TL::KSTR, tid);
    if constexpr (BF) VR.store((uint16_t*)Vs, tid); else VR.store(Vs, TL::VSTR, tid);
    __syncthreads();
    fetch(kb + kKeyBlock);   // the next block, while this one computes

    if (BF && norms) {   // squared norms of the staged keys: wave w the rows of key tile w,
      // read where the score products read them, the four lanes of a row a quarter each
      const uint16_t* kr = (const uint16_t*)Ks + (16 * (tid >> 6) + (lane & 15)) * TL::KSTR + 8 * g;
      float sq = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const uint4 a = *(const uint4*)(kr + 32 * ks);
        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, a.x), sq, false);
        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, a.y), sq, false);
        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, a.z), sq, false);
        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, a.w), sq, false);
      }
      sq += __shfl_xor(sq, 16, WAVE);
      sq += __shfl_xor(sq, 32, WAVE);
      kmx = fmaxf(kmx, sq);
    } else if (norms) {   // squared norms of the staged keys: 4 threads per row
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
    qfr.scores(Ks, acc, lane);

    {   // group maxima for the top-k threshold: one lane's 4 scores of one kt (gq = 4),
        // its 16 scores (gq = 16), or the block's 64
      float gk[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        gk[kt] = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) gk[kt] = fmaxf(gk[kt], kb + 16 * kt + 4 * g + j < k1 ? acc[kt][j] : -INFINITY);
      }
      const int blk = kb / kKeyBlock;
      if (gq == 4) {
        if (lm_ok) *(float4*)(Brow + 16 * blk + 4 * g) = make_float4(gk[0], gk[1], gk[2], gk[3]);
      } else {
        float gm = fmaxf(fmaxf(gk[0], gk[1]), fmaxf(gk[2], gk[3]));
        if (gq == 64) gm = quad_max(gm);
        if (lm_ok && (gq == 16 || g == 0)) Brow[gq == 16 ? 4 * blk + g : blk] = gm;
      }
    }
    if (Srow && lm_ok) {   // the scores themselves only when asked for
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
    const float alpha = online_softmax(acc, nvalid, sl2e, st.mrun, st.lrun, lane);
    rescale<D>(st.o, alpha);
    if constexpr (BF)
      pv_bf16<D>((const uint16_t*)Vs, acc, st.o, lane);
    else
      pv_f32<D>((const float*)Vs, acc, st.o, lane);
    __syncthreads();
  }
}

// Candidate sweep over keys [k0, k1): every score >= tf goes to seg (slots
// [0, capc), index order) with its token id, as (order key, id); `base` counts
// the lane's landmark's candidates (also those past capc). Per kt, the four
// lanes of a landmark take consecutive slots by an exclusive count over g.
template <typename T, int D>
__device__ __forceinline__ void candidate_sweep(const T* Kz, int k0, int k1, const LmFrag<T, D>& qfr, T* Ks,
                                                float tf, uint2* seg, int capc, bool lm_ok, uint32_t& base, int tid) {
  using TL = Tiles<T, D>;
  const int lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int last_kb = k0 + ((k1 - k0 - 1) / kKeyBlock) * kKeyBlock;
  RowRegs<T, D> KR;
  auto fetch = [&](int kb) {
    const int nb = min(kb, last_kb);
    KR.load([&](int rr) { return Kz + (size_t)(nb + rr) * D; }, min(kKeyBlock, k1 - nb), tid);
  };
  fetch(k0);

  for (int kb = k0; kb < k1; kb += kKeyBlock) {
    KR.store(Ks, TL::KSTR, tid);
    __syncthreads();
    fetch(kb + kKeyBlock);
    f32x4 acc[4];
    qfr.scores(Ks, acc, lane);
    // per kt: this lane's candidate count in a byte of one word
    uint32_t flags = 0, packed = 0;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool p = (kb + 16 * kt + 4 * g + j < k1) & (acc[kt][j] >= tf);
        flags |= p ? 1u << (4 * kt + j) : 0u;
        packed += p ? 1u << (8 * kt) : 0u;
      }
    const uint32_t p0 = __shfl(packed, r, WAVE), p1 = __shfl(packed, r + 16, WAVE);
    const uint32_t p2 = __shfl(packed, r + 32, WAVE), p3 = __shfl(packed, r + 48, WAVE);
    const uint32_t tot = p0 + p1 + p2 + p3;   // no byte exceeds 16: no carries
    const uint32_t ex = (g > 0 ? p0 : 0u) + (g > 1 ? p1 : 0u) + (g > 2 ? p2 : 0u);
    // slot of the lane's first candidate of each kt (one byte per kt): the
    // landmark's candidates of earlier kt, then those of lanes with smaller g;
    // the byte sums stay below 256
    const uint32_t first = ex + (tot << 8) + (tot << 16) + (tot << 24);
    // one pass per candidate of the lane (few: most scores are below the
    // threshold), in (kt, j) order, i.e. in key order
    uint32_t fl = lm_ok ? flags : 0u;
    while (fl) {
      const int bit = __builtin_ctz(fl);
      fl &= fl - 1u;
      const int kt = bit >> 2;
      const uint32_t pos = base + ((first >> (8 * kt)) & 255u) +
                           (uint32_t)__builtin_popcount(flags & ((1u << bit) - 1u) & (0xFu << (4 * kt)));
      float x = acc[0][0];
#pragma unroll
      for (int b = 1; b < 16; ++b) x = bit == b ? acc[b >> 2][b & 3] : x;
      if (pos < (uint32_t)capc)
        seg[pos] = make_uint2(f32_key(x), (uint32_t)(kb + 16 * kt + 4 * g + (bit & 3)));
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) base += (tot >> (8 * kt)) & 255u;
    __syncthreads();
  }
}

}  // namespace mita
