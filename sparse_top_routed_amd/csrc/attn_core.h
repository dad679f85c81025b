// Wave-level pieces of flash-style attention on gfx950 MFMA, shared by the
// shared-expert, gather, combine and full-attention kernels.
//
// A workgroup is 4 waves; each wave owns 16 queries. Keys arrive in blocks of
// 64 staged in LDS. Scores are computed transposed, S^T = K Q^T, with the
// 16x16 MFMA tiles, so lane l holds the scores of query l%16 against keys
// 4*(l/16) + j (+16 per tile). Those four consecutive keys are exactly what the
// lane must feed as the B operand of the P.V product when V^T is the A operand,
// so the probabilities never leave registers: bf16 needs V^T in LDS (written
// transposed while staging), fp32 reads V rows directly.
#pragma once
#include <type_traits>

#include "common.h"
#include "plan.h"

namespace mita {

template <typename T, int D>
struct Tiles {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int KSTR = D + (BF ? 8 : 4);                 // key tile row stride (elements)
  static constexpr int VSTR = BF ? (kKeyBlock + 8) : (D + 4);   // bf16: V^T rows of 64 keys; fp32: V rows
  static constexpr int KTILE = kKeyBlock * KSTR;                // elements per key tile
  static constexpr int VTILE = BF ? D * VSTR : kKeyBlock * VSTR;
  static constexpr int EPC = 16 / sizeof(T);                    // elements per 16-byte chunk
};

// A thread's share of one 64-row block, held in registers so the loads can be
// issued early (prefetch) and written to LDS later. Rows r >= nvalid repeat row
// nvalid - 1 (a real row, so finite): every consumer masks those keys out of
// the softmax. Zeroing them with a select after the load would let the compiler
// turn the load into a branch that waits for it, which defeats the prefetch.
template <typename T, int D>
struct RowRegs {
  static constexpr int EPC = 16 / sizeof(T), CPR = D / EPC, PER = kKeyBlock * CPR / 256;
  uint4 v[PER];
  template <typename RowFn>
  __device__ __forceinline__ void load(RowFn rowptr, int nvalid, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u, r = c / CPR, cc = (c % CPR) * EPC;
      v[u] = ld16(rowptr(min(r, nvalid - 1)) + cc);
    }
  }
  __device__ __forceinline__ void store(T* dst, int stride, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u, r = c / CPR, cc = (c % CPR) * EPC;
      *(uint4*)(dst + r * stride + cc) = v[u];
    }
  }
};

// Copy 64 rows into a key tile: row r comes from rowptr(r) (D contiguous
// elements, 16-byte aligned); rows r >= nvalid repeat row nvalid - 1, so their
// scores are finite and the caller excludes them by index. Every load is issued
// before the first store (one wait for all of them).
template <typename T, int D, typename RowFn>
__device__ __forceinline__ void stage_rows(T* dst, int stride, RowFn rowptr, int nvalid, int tid) {
  RowRegs<T, D> rr;
  rr.load(rowptr, nvalid, tid);
  rr.store(dst, stride, tid);
}

// Slot of key quad qd (keys 4 qd .. 4 qd + 3) in row d of a bf16 V^T tile.
// The XOR swizzle spreads both access patterns over distinct LDS banks: the
// transposed writes (a wave covers d rows 8 apart) and the MFMA operand reads
// (16 consecutive rows, one quad each).
template <int D>
__device__ __forceinline__ int vt_quad(int d, int qd) {
  const int c = (d >> 3) & (D / 8 - 1);
  return qd ^ (D == 64 ? ((c << 1) | (c & 1)) : c);
}

// Same for a bf16 V block that is written transposed (V^T [D][64 + pad], key
// quads placed by vt_quad). Each thread holds RPT consecutive rows of one
// 8-element column chunk, so the transposed writes are RPT keys wide.
template <int D>
struct VtRegs {
  static constexpr int CPR = D / 8, RPT = kKeyBlock * CPR / 256;   // 2 rows (d = 64) or 4 rows (d = 128)
  uint4 v[RPT];
  template <typename RowFn>
  __device__ __forceinline__ void load(RowFn rowptr, int nvalid, int tid) {
    const int kg = tid / CPR, cc = (tid % CPR) * 8;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int r = kg * RPT + u;
      v[u] = ld16(rowptr(min(r, nvalid - 1)) + cc);
    }
  }
  __device__ __forceinline__ void store(uint16_t* Vt, int tid) const {
    constexpr int VSTR = Tiles<uint16_t, D>::VSTR;
    const int kg = tid / CPR, cc = (tid % CPR) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e of each row: low halves (e even) or high halves (e odd) of word e / 2
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int q = e >> 1, d = cc + e;
      const uint32_t w01 = __builtin_amdgcn_perm(((const uint32_t*)&v[1])[q], ((const uint32_t*)&v[0])[q], sel);
      if constexpr (RPT == 4) {
        const uint32_t w23 = __builtin_amdgcn_perm(((const uint32_t*)&v[3])[q], ((const uint32_t*)&v[2])[q], sel);
        *(uint2*)(Vt + d * VSTR + 4 * vt_quad<D>(d, kg)) = make_uint2(w01, w23);
      } else {
        *(uint32_t*)(Vt + d * VSTR + 4 * vt_quad<D>(d, kg >> 1) + 2 * (kg & 1)) = w01;
      }
    }
  }
};

// S^T block (64 keys x 16 queries) for bf16. Query side: QP parts in registers
// (qf[p][ks] is lane's 8 elements 32*ks + 8*(lane/16) of query lane%16). Key
// side: one tile, or two (hi, lo) when KP == 2.
template <int D, int KP, int QP>
__device__ __forceinline__ void qk_bf16(const uint16_t* Ks0, const uint16_t* Ks1, const uint4 (&qf)[QP][D / 32],
                                        f32x4 (&acc)[4], int lane) {
  constexpr int KSTR = Tiles<uint16_t, D>::KSTR;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int off = (16 * kt + r) * KSTR + 32 * ks + 8 * g;
      const uint4 a0 = *(const uint4*)(Ks0 + off);
#pragma unroll
      for (int p = 0; p < QP; ++p) acc[kt] = mma_bf16(a0, qf[p][ks], acc[kt]);
      if constexpr (KP == 2) {
        const uint4 a1 = *(const uint4*)(Ks1 + off);
        acc[kt] = mma_bf16(a1, qf[0][ks], acc[kt]);
      }
    }
  }
}

// S^T block for fp32 (qf[ks] is element 4*ks + lane/16 of query lane%16).
template <int D>
__device__ __forceinline__ void qk_f32(const float* Ks, const float (&qf)[D / 4], f32x4 (&acc)[4], int lane) {
  constexpr int KSTR = Tiles<float, D>::KSTR;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[kt] = mma_f32(Ks[(16 * kt + r) * KSTR + 4 * ks + g], qf[ks], acc[kt]);
  }
}

// Online softmax over one block of raw scores (lane's keys 16 kt + 4 (lane/16) + j;
// keys at or beyond `live` are masked). Works in the log2 domain: with
// c = log2(e) / sqrt(d), p = 2^(c s - m). On return x holds the unnormalised
// probabilities; the returned factor rescales earlier sums.
__device__ __forceinline__ float online_softmax(f32x4 (&x)[4], int live, float c, float& mrun, float& lrun,
                                                int lane) {
  if (live < kKeyBlock) {
    const int g = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (16 * kt + 4 * g + j >= live) x[kt][j] = -INFINITY;
  }
  float bm = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) bm = fmaxf(bm, x[kt][j]);
  bm = quad_max(bm);
  const float mnew = fmaxf(mrun, bm * c);
  // raw v_exp_f32 (no denormal range fix-up: probabilities below 2^-126 flush to 0)
  const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(x[kt][j], c, -mnew));
      x[kt][j] = p;
      sum += p;
    }
  lrun = lrun * alpha + sum;
  mrun = mnew;
  return alpha;
}

template <int D>
__device__ __forceinline__ void rescale(f32x4 (&o)[D / 16], float alpha) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[dt][j] *= alpha;
}

// Softmax of one block for QT column tiles against a lazily raised reference
// (log2 domain, p = 2^(c s - mrun)): a row's reference moves up to its block
// maximum only when that maximum exceeds it by more than kLazyLog2, and only then
// are the row's output and sum rescaled (one wave-uniform branch for all tiles).
// Numerator and denominator share the reference, so the softmax is unchanged;
// the probabilities stay below 2^kLazyLog2. Row sums are left to the caller.
// A row's maximum is the largest of its four lanes' maxima, so the test runs on
// each lane's own maximum (c > 0 keeps the order) and the row maxima, which need
// lanes of other lane groups, are formed only in the rare branch that moves a
// reference.
constexpr float kLazyLog2 = 8.f;

template <int D, int QT>
__device__ __forceinline__ void lazy_softmax(f32x4 (&x)[QT][4], int live, float c, float (&mrun)[QT],
                                             float (&lrun)[QT], f32x4 (&o)[QT][D / 16], int lane) {
  float lm[QT];
  bool any = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (live < kKeyBlock) {   // block-uniform; key 16 kt + 4 g + j is masked when 16 kt + j >= live - 4 g
      const int lim = live - 4 * (lane >> 4);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (16 * kt + j >= lim) x[qt][kt][j] = -INFINITY;
    }
    float v = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) v = fmaxf(v, x[qt][kt][j]);
    lm[qt] = v;
    any |= v * c > mrun[qt] + kLazyLog2;
  }
  if (__builtin_amdgcn_ballot_w64(any) != 0) {   // wave-uniform
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma clang fp contract(off)   // bm rounded: alpha takes the new reference itself
      const float bm = quad_max(lm[qt]) * c;
      const bool up = bm > mrun[qt] + kLazyLog2;
      // raw v_exp_f32; 2^(-inf) = 0 clears the empty state of the first block
      const float alpha = up ? __builtin_amdgcn_exp2f(mrun[qt] - bm) : 1.f;
      mrun[qt] = up ? bm : mrun[qt];
      lrun[qt] *= alpha;
      rescale<D>(o[qt], alpha);
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[qt][kt][j] = __builtin_amdgcn_exp2f(fmaf(x[qt][kt][j], c, -mrun[qt]));
}

// Sum of the two bf16 halves of w added to acc (one v_dot2 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}

// O^T += V^T P^T for bf16: o[dt] holds O^T[16*dt + 4*(lane/16) + j][lane%16].
template <int D>
__device__ __forceinline__ void pv_bf16(const uint16_t* Vt, const f32x4 (&p)[4], f32x4 (&o)[D / 16], int lane) {
  constexpr int VSTR = Tiles<uint16_t, D>::VSTR;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 b;
    b.x = pack_bf16x2(p[2 * h][0], p[2 * h][1]);
    b.y = pack_bf16x2(p[2 * h][2], p[2 * h][3]);
    b.z = pack_bf16x2(p[2 * h + 1][0], p[2 * h + 1][1]);
    b.w = pack_bf16x2(p[2 * h + 1][2], p[2 * h + 1][3]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int d = 16 * dt + r;
      const uint16_t* row = Vt + d * VSTR;
      const uint2 lo = *(const uint2*)(row + 4 * vt_quad<D>(d, 8 * h + g));
      const uint2 hi = *(const uint2*)(row + 4 * vt_quad<D>(d, 8 * h + 4 + g));
      o[dt] = mma_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), b, o[dt]);
    }
  }
}

// Same for fp32, V rows read directly from the row-major V tile.
template <int D>
__device__ __forceinline__ void pv_f32(const float* Vs, const f32x4 (&p)[4], f32x4 (&o)[D / 16], int lane) {
  constexpr int VSTR = Tiles<float, D>::VSTR;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* row = Vs + (16 * kt + 4 * g + j) * VSTR + r;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] = mma_f32(row[16 * dt], p[kt][j], o[dt]);
    }
}

// Query fragments of one query row (zeros when the row is absent).
template <typename T, int D>
struct QFrag {
  uint4 b[1][D / 32];
  float f[D / 4];
  // qrow must be a valid row; absent rows (padding) load a real row and their
  // results are never written, since every row of the tile is independent.
  __device__ __forceinline__ void load(const T* qrow, int g) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) b[0][ks] = ld16(qrow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) f[ks] = qrow[4 * ks + g];
    }
  }
};

template <typename T, int D>
struct AttnLds {
  using TL = Tiles<T, D>;
  __align__(16) T k0[TL::KTILE];
  __align__(16) T k1[sizeof(T) == 2 ? TL::KTILE : 8];
  __align__(16) T v[TL::VTILE];
};

// One 64-key block of attention for the wave's 16 queries, keys already staged.
template <typename T, int D, int KP>
__device__ __forceinline__ void attend_block(AttnLds<T, D>& sm, const QFrag<T, D>& qf, int live, float sl2e,
                                             float& mrun, float& lrun, f32x4 (&o)[D / 16], int lane,
                                             bool wave_live = true) {
  if (!wave_live) return;   // all 16 rows of this wave are padding (wave-uniform)
  f32x4 acc[4];
  if constexpr (sizeof(T) == 2)
    qk_bf16<D, KP, 1>((const uint16_t*)sm.k0, (const uint16_t*)sm.k1, qf.b, acc, lane);
  else
    qk_f32<D>((const float*)sm.k0, qf.f, acc, lane);
  const float alpha = online_softmax(acc, live, sl2e, mrun, lrun, lane);
  rescale<D>(o, alpha);
  if constexpr (sizeof(T) == 2)
    pv_bf16<D>((const uint16_t*)sm.v, acc, o, lane);
  else
    pv_f32<D>((const float*)sm.v, acc, o, lane);
}

// Register copies of one key block and its value block (bf16 values transposed).
template <typename T, int D, int KP>
struct KVRegs {
  RowRegs<T, D> k[KP];
  std::conditional_t<sizeof(T) == 2, VtRegs<D>, RowRegs<T, D>> v;
  __device__ __forceinline__ void store(AttnLds<T, D>& sm, int tid) const {
    using TL = Tiles<T, D>;
    k[0].store(sm.k0, TL::KSTR, tid);
    if constexpr (KP == 2) k[1].store(sm.k1, TL::KSTR, tid);
    if constexpr (sizeof(T) == 2) v.store((uint16_t*)sm.v, tid); else v.store(sm.v, TL::VSTR, tid);
  }
};

// gfx950 transpose read ds_read_b64_tr_b16: within each 16-lane group, lane i
// supplies the address of 4 consecutive 16-bit elements (row i / 4 of a 4 x 16
// patch, columns 4 (i % 4) ..) and receives column i of the patch, one element
// per row (lane layout checked on the GPU).
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// ---------------------------------------------------------------- swizzled tiles, direct loads
// 64-row bf16 tiles without padding, filled by direct global-to-LDS loads
// (global_load_lds_dwordx4: lane i of a wave's instruction writes 16 bytes at the
// instruction's LDS base + 16 i, so each instruction fills 1 KB of whole rows).
// Bank conflicts are avoided by placing 16-byte chunk c of row r at chunk
// c ^ swz(r) of the row instead of padding:
//   K (read as QK fragments, 16 consecutive rows at one chunk): the 16 rows must
//     land on 16 distinct chunks (D = 128: r & 15; D = 64, two rows per 64 banks:
//     (r >> 1) & 7);
//   V (read transposed, a half-wave takes 8 consecutive rows x 2 neighbouring
//     chunks): the 8 rows' chunk pairs must be disjoint (D = 128: 2 (r & 7);
//     D = 64: 2 ((r >> 1) & 3)).
template <int D>
struct SwzTile {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = kKeyBlock * D;     // elements
  static constexpr int RPI = 512 / D;            // rows per 1 KB load instruction
  static constexpr int NI = kKeyBlock / RPI / 4; // load instructions per wave per tile
  __device__ static __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// A wave's share of one 64-row block (rows 16 w .. 16 w + 15) by direct loads:
// row ids from `ids` (the token of each of the lane's NI rows), K and V tiles.
template <int D>
__device__ __forceinline__ void dma_rows(uint16_t* Kt, uint16_t* Vt, const uint16_t* Kz, const uint16_t* Vz,
                                         const int (&ids)[SwzTile<D>::NI], int w, int lane) {
  using S = SwzTile<D>;
  const int p = lane % S::CPR;
#pragma unroll
  for (int u = 0; u < S::NI; ++u) {
    const int row = 16 * w + u * S::RPI + lane / S::CPR;
    const size_t src = (size_t)ids[u] * D;
    const int lds_row0 = 16 * w + u * S::RPI;
    lds_dma16(Kz + src + 8 * (p ^ S::swz_k(row)), Kt + lds_row0 * D);
    lds_dma16(Vz + src + 8 * (p ^ S::swz_v(row)), Vt + lds_row0 * D);
  }
}

// dma_rows through raw buffer resources (base of the slice's K or V, records =
// its byte size; dword 3 = 0x00020000 for gfx9 raw buffers): the row offsets are
// 32-bit (ids < N, N d 2 < 2^31 bytes), so each load costs one address add.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)l, 16, off, 0, 0, 0);
}
// The same with a wave-uniform byte offset added (a scalar register).
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)l, 16, off, soff, 0, 0);
}
template <int D>
__device__ __forceinline__ void dma_rows_buf(uint16_t* Kt, uint16_t* Vt, __amdgpu_buffer_rsrc_t rsK,
                                             __amdgpu_buffer_rsrc_t rsV, const int (&ids)[SwzTile<D>::NI], int w,
                                             int lane) {
  using S = SwzTile<D>;
  const int p = lane % S::CPR;
#pragma unroll
  for (int u = 0; u < S::NI; ++u) {
    const int row = 16 * w + u * S::RPI + lane / S::CPR;
    const uint32_t src = (uint32_t)ids[u] * (D * 2);
    const int lds_row0 = 16 * w + u * S::RPI;
    lds_dma16_buf(rsK, src + 16 * (p ^ S::swz_k(row)), Kt + lds_row0 * D);
    lds_dma16_buf(rsV, src + 16 * (p ^ S::swz_v(row)), Vt + lds_row0 * D);
  }
}

// The key tile of dma_rows alone (swizzled for score reads).
template <int D>
__device__ __forceinline__ void dma_rows_k(uint16_t* Kt, const uint16_t* Kz, const int (&ids)[SwzTile<D>::NI], int w,
                                           int lane) {
  using S = SwzTile<D>;
  const int p = lane % S::CPR;
#pragma unroll
  for (int u = 0; u < S::NI; ++u) {
    const int row = 16 * w + u * S::RPI + lane / S::CPR;
    lds_dma16(Kz + (size_t)ids[u] * D + 8 * (p ^ S::swz_k(row)), Kt + (16 * w + u * S::RPI) * D);
  }
}

// QT column tiles of scores from a swizzled K tile.
template <int D, int QT>
__device__ __forceinline__ void qk_bf16_swz(const uint16_t* Ks, const uint4 (&qf)[QT][D / 32], f32x4 (&acc)[QT][4],
                                            int lane) {
  using S = SwzTile<D>;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    // row 16 kt + r has the swizzle of r (16 kt changes neither r & 15 nor (r >> 1) & 7)
    const uint16_t* col = Ks + r * D + 8 * ((4 * ks + g) ^ S::swz_k(r));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint4 a0 = *(const uint4*)(col + 16 * kt * D);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) acc[qt][kt] = mma_bf16(a0, qf[qt][ks], acc[qt][kt]);
    }
  }
}

// QT column tiles of scores from a swizzled K tile against two query planes
// (hi, lo): per accumulator the MFMA sequence of qk_bf16<D, 1, 2> (k-slices in
// order, hi then lo), so the scores are the same bits.
template <int D, int QT>
__device__ __forceinline__ void qk2_bf16_swz(const uint16_t* Ks, const uint4 (&qb)[QT][2][D / 32],
                                             f32x4 (&acc)[QT][4], int lane, int ktn = -1, float* nsq = nullptr) {
  using S = SwzTile<D>;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const uint16_t* col = Ks + r * D + 8 * ((4 * ks + g) ^ S::swz_k(r));
    if (nsq) {   // squared norm of row 16 ktn + r over this lane's pieces (same addresses as the reads below)
      const uint4 an = *(const uint4*)(col + 16 * ktn * D);
      *nsq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, an.x), __builtin_bit_cast(bf16x2, an.x), *nsq, false);
      *nsq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, an.y), __builtin_bit_cast(bf16x2, an.y), *nsq, false);
      *nsq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, an.z), __builtin_bit_cast(bf16x2, an.z), *nsq, false);
      *nsq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, an.w), __builtin_bit_cast(bf16x2, an.w), *nsq, false);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint4 a0 = *(const uint4*)(col + 16 * kt * D);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        acc[qt][kt] = mma_bf16(a0, qb[qt][0][ks], acc[qt][kt]);
        acc[qt][kt] = mma_bf16(a0, qb[qt][1][ks], acc[qt][kt]);
      }
    }
  }
}

// P V from a swizzled row-major V tile: V^T fragments by transposed reads; the
// lane's probabilities (bf16, as multiplied) are added to lsum. Lane (r,
// g) needs rows (keys) 4 q .. 4 q + 3 of column (d) 16 dt + r with q = 8 h + g (low
// half) or 8 h + 4 + g (high half): the 4 x 16 patch of rows 4 q .. and columns 16 dt ..
template <int D, int QT>
__device__ __forceinline__ void pv_bf16_swz(const uint16_t* Vs, const f32x4 (&p)[QT][4], f32x4 (&o)[QT][D / 16],
                                            float (&lsum)[QT], int lane) {
  using S = SwzTile<D>;
  const int g = lane >> 4, i = lane & 15;
  const int row = 4 * g + (i >> 2);           // + 32 h + 16 hi: multiples of 8, same swizzle
  const int sw = S::swz_v(row), b = (i & 3) >> 1, half = i & 1;
  const uint16_t* rb = Vs + row * D + 4 * half;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 bb[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      bb[qt].x = pack_bf16x2(p[qt][2 * h][0], p[qt][2 * h][1]);
      bb[qt].y = pack_bf16x2(p[qt][2 * h][2], p[qt][2 * h][3]);
      bb[qt].z = pack_bf16x2(p[qt][2 * h + 1][0], p[qt][2 * h + 1][1]);
      bb[qt].w = pack_bf16x2(p[qt][2 * h + 1][2], p[qt][2 * h + 1][3]);
      // the row sum adds the probabilities as rounded for the product
      lsum[qt] = add_bf16x2(bb[qt].w, add_bf16x2(bb[qt].z, add_bf16x2(bb[qt].y, add_bf16x2(bb[qt].x, lsum[qt]))));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int ch = 8 * ((2 * dt + b) ^ sw);
      const uint2 lo = lds_read_tr16(rb + (32 * h) * D + ch);
      const uint2 hi = lds_read_tr16(rb + (32 * h + 16) * D + ch);
      const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) o[qt][dt] = mma_bf16(a, bb[qt], o[qt][dt]);
    }
  }
}

// ---------------------------------------------------------------- tiles of NW-wave workgroups
// 64-row bf16 tiles filled by direct loads from NW waves (rows w 64 / NW .. of
// the tile per wave), swizzled as SwzTile: chunk c of row r at c ^ swz_k(r) in a
// tile read as QK operands, at c ^ swz_v(r) in one read transposed. (A single
// swizzle for both reads, 2 (r & 7) | (r >> 3 & 1), measured one LDS bank-conflict
// cycle per MFMA on the QK reads; swz_k and swz_v measure none.)
template <int D>
struct UTile {
  static constexpr int CPR = D / 8, TILE = kKeyBlock * D, RPI = 512 / D;
  __device__ static __forceinline__ int swz_k(int r) { return SwzTile<D>::swz_k(r); }
  __device__ static __forceinline__ int swz_v(int r) { return SwzTile<D>::swz_v(r); }
};

// VT: the tile is read transposed (swz_v), else as QK operands (swz_k).
template <int D, int NW, bool VT, typename RowFn>
__device__ __forceinline__ void udma(uint16_t* tile, RowFn rowp, int w, int lane) {
  using U = UTile<D>;
  constexpr int RPW = kKeyBlock / NW, NI = RPW / U::RPI;
  static_assert(NI >= 1, "rows per wave below one load instruction");
  const int p = lane % U::CPR;
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int r0 = w * RPW + u * U::RPI, row = r0 + lane / U::CPR;
    lds_dma16(rowp(row) + 8 * (p ^ (VT ? U::swz_v(row) : U::swz_k(row))), tile + r0 * D);
  }
}

// Scores of the 64 tile rows against the wave's QT x 16 register rows; with KP =
// 2 the second tile (the lo plane of Q~) is added after the first at every step,
// the order qk_bf16<D, 2, 1> uses.
template <int D, int QT, int KP>
__device__ __forceinline__ void uqk(const uint16_t* T0, const uint16_t* T1, const uint4 (&qf)[QT][D / 32],
                                    f32x4 (&acc)[QT][4], int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const int off = r * D + 8 * ((4 * ks + g) ^ UTile<D>::swz_k(r));   // 16 kt keeps the swizzle
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint4 a0 = *(const uint4*)(T0 + off + 16 * kt * D);
      uint4 a1;
      if constexpr (KP == 2) a1 = *(const uint4*)(T1 + off + 16 * kt * D);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        acc[qt][kt] = mma_bf16(a0, qf[qt][ks], acc[qt][kt]);
        if constexpr (KP == 2) acc[qt][kt] = mma_bf16(a1, qf[qt][ks], acc[qt][kt]);
      }
    }
  }
}

// o[qt][dt] += T^T p[qt] (transposed reads of the tile), the order pv_bf16 uses.
template <int D, int QT>
__device__ __forceinline__ void upv(const uint16_t* T, const f32x4 (&p)[QT][4], f32x4 (&o)[QT][D / 16],
                                    float (&lsum)[QT], int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int row = 4 * g + (i >> 2);   // + 32 h + 16 hi: bits the swizzle does not use
  const int sw = UTile<D>::swz_v(row), b = (i & 3) >> 1;
  const uint16_t* rb = T + row * D + 4 * (i & 1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 bb[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      bb[qt].x = pack_bf16x2(p[qt][2 * h][0], p[qt][2 * h][1]);
      bb[qt].y = pack_bf16x2(p[qt][2 * h][2], p[qt][2 * h][3]);
      bb[qt].z = pack_bf16x2(p[qt][2 * h + 1][0], p[qt][2 * h + 1][1]);
      bb[qt].w = pack_bf16x2(p[qt][2 * h + 1][2], p[qt][2 * h + 1][3]);
      // the row sum adds the probabilities as rounded for the product
      lsum[qt] = add_bf16x2(bb[qt].w, add_bf16x2(bb[qt].z, add_bf16x2(bb[qt].y, add_bf16x2(bb[qt].x, lsum[qt]))));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int ch = 8 * ((2 * dt + b) ^ sw);
      const uint2 lo = lds_read_tr16(rb + (32 * h) * D + ch);
      const uint2 hi = lds_read_tr16(rb + (32 * h + 16) * D + ch);
      const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) o[qt][dt] = mma_bf16(a, bb[qt], o[qt][dt]);
    }
  }
}

// A row's D outputs in the S^T layout sit on its four lanes (lane group g holds
// columns 16 dt + 4 g .. + 3 of every 16-column block dt), 8 bytes per block for
// 16-bit values. Row stores and loads go in 16-byte pieces instead: over a pair of
// blocks (dt, dt + 1) the lanes of groups g and g ^ 1 trade half their values
// with v_permlane16_swap, after which even g holds columns 16 dt + 4 g .. + 7 and
// odd g columns 16 (dt + 1) + 4 (g - 1) .. + 7, at this offset (in elements) from
// the row's start. The trade is its own inverse: applied to such a piece after a
// load it gives back the two 8-byte values of the lane's own columns.
__device__ __forceinline__ int pair_col(int dt, int g) { return 16 * dt + 16 * (g & 1) + 4 * (g & 2); }
// lane values a (block dt), b (block dt + 1), two 32-bit words each -> the piece
__device__ __forceinline__ uint4 pair_trade(uint2 a, uint2 b) {
  const auto x = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  return make_uint4(x[0], y[0], x[1], y[1]);
}
// the piece -> the lane values of blocks dt (first) and dt + 1 (second)
__device__ __forceinline__ void pair_untrade(uint4 c, uint2& a, uint2& b) {
  const auto x = __builtin_amdgcn_permlane16_swap(c.x, c.z, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(c.y, c.w, false, false);
  a = make_uint2(x[0], y[0]);
  b = make_uint2(x[1], y[1]);
}

// One row's D outputs o[dt] * inv from its four lanes (every lane of the row
// calls it): 16-byte pieces for bf16, the lane's 16 bytes per block for fp32.
template <typename T, int D>
__device__ __forceinline__ void store_row(T* orow, const f32x4 (&o)[D / 16], float inv, int g) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int dt = 0; dt < D / 16; dt += 2)
      *(uint4*)(orow + pair_col(dt, g)) =
          pair_trade(make_uint2(pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)),
                     make_uint2(pack_bf16x2(o[dt + 1][0] * inv, o[dt + 1][1] * inv),
                                pack_bf16x2(o[dt + 1][2] * inv, o[dt + 1][3] * inv)));
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *(float4*)(orow + 16 * dt + 4 * g) = make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
  }
}

}  // namespace mita
