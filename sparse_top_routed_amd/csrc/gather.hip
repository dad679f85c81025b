// Step 5: output. For query q with routed experts e_1..e_s, softmax attention
// over K* = [Q~, K_{I_e1}, ..., K_{I_es}] and V* = [V~, V_{I_e1}, ..., V_{I_es}]
// with scale 1/sqrt(d) (the Dutch MiTA summary's formula; a token in two of the
// query's experts is counted twice, as the concatenation says).
//
// The (query, slot) pairs are bucketed by expert with a counting sort (histogram,
// scan, scatter). The gather kernel then runs one workgroup per tile of up to 64
// queries of one bucket: the expert's k token rows are gathered into LDS 64 at a
// time and every query of the tile attends them on MFMA, so each gathered row is
// read once per tile rather than once per query. With s = 1 and m <= 64 the
// same workgroup also attends the m landmark pairs (one block, resident in LDS)
// and writes the output; otherwise it writes a partial per (query, slot): its
// softmax max and sum, and its output o / sum divided by its largest magnitude
// (fp16 for bf16 inputs, fp32 otherwise), and the combine kernel attends the
// landmark pairs (once per 64 consecutive queries) and merges the s + 1 partial
// softmaxes.
#include <type_traits>

#include "attn_core.h"

namespace mita {

// Wave priority of the partial-path kernel while a block's MFMA work is in flight.
constexpr int kGatherPrio = 1;

__global__ __launch_bounds__(256) void clear_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void bucket_hist_kernel(const int32_t* __restrict__ E, uint32_t* __restrict__ bcount,
                                                          int Ns, int m) {
  extern __shared__ uint32_t h[];
  const int z = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  const int start = blockIdx.x * 4096, end = min(Ns, start + 4096);
  for (int e = start + tid; e < end; e += 256) {
    const int x = Ez[e];
    if ((unsigned)x < (unsigned)m) atomicAdd(&h[x], 1u);
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256)
    if (h[i]) atomicAdd(&bcount[(size_t)z * m + i], h[i]);
}

// Exclusive scan of the bucket sizes, then the table of query tiles (at most
// trows rows of one bucket each) that the gather kernel walks; unused
// entries are marked with expert -1.
__global__ __launch_bounds__(256) void bucket_scan_kernel(const uint32_t* __restrict__ bcount, uint32_t* __restrict__ boff,
                                                          int4* __restrict__ tiles, int m, int max_tiles, int trows) {
  __shared__ uint32_t wtot[4];
  const int z = blockIdx.x, tid = threadIdx.x;
  const int per = (m + 255) / 256, i0 = min(m, tid * per), i1 = min(m, i0 + per);
  const uint32_t* c = bcount + (size_t)z * m;
  uint32_t sc = 0, st = 0;
  for (int i = i0; i < i1; ++i) { sc += c[i]; st += (c[i] + trows - 1) / trows; }
  uint32_t totc, tott;
  uint32_t oc = block_incl_scan(sc, wtot, totc) - sc;
  uint32_t ot = block_incl_scan(st, wtot, tott) - st;
  uint32_t* bo = boff + (size_t)z * (m + 1);
  int4* tz = tiles + (size_t)z * max_tiles;
  for (int i = i0; i < i1; ++i) {
    bo[i] = oc;
    for (uint32_t r = 0; r < c[i]; r += trows, ++ot)
      tz[ot] = make_int4(i, (int)r, (int)min((uint32_t)trows, c[i] - r), (int)(oc + r));
    oc += c[i];
  }
  if (tid == 0) bo[m] = totc;
  for (int t = (int)tott + tid; t < max_tiles; t += 256) tz[t] = make_int4(-1, 0, 0, 0);
}

// Scatter (query * s + slot) into its bucket; ranges are reserved per workgroup.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ E,
                                                             const uint32_t* __restrict__ boff,
                                                             uint32_t* __restrict__ bcursor, int32_t* __restrict__ perm,
                                                             int Ns, int m) {
  extern __shared__ uint32_t h[];  // [0, m): local counts, [m, 2m): global bases
  const int z = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  const int start = blockIdx.x * 4096;
  uint32_t rank[16];
  int ex[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = start + tid + 256 * u;
    ex[u] = e < Ns ? Ez[e] : -1;
    if ((unsigned)ex[u] >= (unsigned)m) ex[u] = -1;
    rank[u] = ex[u] >= 0 ? atomicAdd(&h[ex[u]], 1u) : 0u;
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256)
    if (h[i]) h[m + i] = boff[(size_t)z * (m + 1) + i] + atomicAdd(&bcursor[(size_t)z * m + i], h[i]);
  __syncthreads();
  int32_t* pz = perm + (size_t)z * Ns;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (ex[u] >= 0) pz[h[m + ex[u]] + rank[u]] = start + tid + 256 * u;
}

// The whole counting sort of one slice in one workgroup, for slices of at most
// 256 PER (query, slot) pairs: bucket sizes by LDS atomics (each pair keeps the
// rank its atomic returned), their exclusive scan, the tile table and the
// scatter. Ranks within a bucket follow the atomics' order; every query of a
// tile is computed on its own, so the output does not depend on it.
template <int PER>
__global__ __launch_bounds__(256) void bucket_slice_kernel(const int32_t* __restrict__ E, uint32_t* __restrict__ boff,
                                                           int4* __restrict__ tiles, int32_t* __restrict__ perm,
                                                           int Ns, int m, int max_tiles, int trows) {
  extern __shared__ uint32_t h[];   // [0, m): bucket sizes, [m, 2m): bucket offsets
  __shared__ uint32_t wtot[4];
  const int z = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  int ex[PER];
  uint32_t rank[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + 256 * u;
    ex[u] = e < Ns ? Ez[e] : -1;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if ((unsigned)ex[u] >= (unsigned)m) ex[u] = -1;
    rank[u] = ex[u] >= 0 ? atomicAdd(&h[ex[u]], 1u) : 0u;
  }
  __syncthreads();
  const int per = (m + 255) / 256, i0 = min(m, tid * per), i1 = min(m, i0 + per);
  uint32_t sc = 0, st = 0;
  for (int i = i0; i < i1; ++i) { sc += h[i]; st += (h[i] + trows - 1) / trows; }
  uint32_t totc, tott;
  uint32_t oc = block_incl_scan(sc, wtot, totc) - sc;
  uint32_t ot = block_incl_scan(st, wtot, tott) - st;
  uint32_t* bo = boff + (size_t)z * (m + 1);
  int4* tz = tiles + (size_t)z * max_tiles;
  for (int i = i0; i < i1; ++i) {
    const uint32_t c = h[i];
    bo[i] = oc;
    h[m + i] = oc;
    for (uint32_t r = 0; r < c; r += trows, ++ot)
      tz[ot] = make_int4(i, (int)r, (int)min((uint32_t)trows, c - r), (int)(oc + r));
    oc += c;
  }
  if (tid == 0) bo[m] = totc;
  for (int t = (int)tott + tid; t < max_tiles; t += 256) tz[t] = make_int4(-1, 0, 0, 0);
  __syncthreads();
  int32_t* pz = perm + (size_t)z * Ns;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (ex[u] >= 0) pz[h[m + ex[u]] + rank[u]] = tid + 256 * u;
}

// Landmark block lb0 of slice z: keys Q~ (hi and lo planes for bf16), values V~.
template <typename T, int D>
__device__ __forceinline__ void load_landmarks(KVRegs<T, D, sizeof(T) == 2 ? 2 : 1>& R, const void* qtop,
                                               const void* vtop, int z, int m, int lb0, int tid) {
  constexpr bool BF = sizeof(T) == 2;
  const T* p0 = BF ? (const T*)((const uint16_t*)qtop + (size_t)z * 2 * m * D) : (const T*)((const float*)qtop + (size_t)z * m * D);
  const T* vz = BF ? (const T*)((const uint16_t*)vtop + (size_t)z * m * D) : (const T*)((const float*)vtop + (size_t)z * m * D);
  const int live = min(kKeyBlock, m - lb0);
  R.k[0].load([&](int rr) { return p0 + (size_t)(lb0 + rr) * D; }, live, tid);
  if constexpr (BF) R.k[1].load([&](int rr) { return p0 + (size_t)(m + lb0 + rr) * D; }, live, tid);
  R.v.load([&](int rr) { return vz + (size_t)(lb0 + rr) * D; }, live, tid);
}

// Attention over the m landmark pairs (keys Q~, values V~), block 0 already in
// registers (R). The next block is fetched into R while the current one
// computes. Block-uniform call; ends with the LDS tiles free again.
template <typename T, int D>
__device__ __forceinline__ void attend_landmarks(AttnLds<T, D>& sm, KVRegs<T, D, sizeof(T) == 2 ? 2 : 1>& R,
                                                 const QFrag<T, D>& qf, const void* qtop, const void* vtop, int z,
                                                 int m, float sl2e, float& mrun, float& lrun, f32x4 (&o)[D / 16],
                                                 int tid, bool wave_live = true) {
  constexpr int KP = sizeof(T) == 2 ? 2 : 1;
  const int lane = tid & 63;
  for (int lb0 = 0; lb0 < m; lb0 += kKeyBlock) {
    R.store(sm, tid);
    __syncthreads();
    if (lb0 + kKeyBlock < m) load_landmarks<T, D>(R, qtop, vtop, z, m, lb0 + kKeyBlock, tid);   // block-uniform
    attend_block<T, D, KP>(sm, qf, min(kKeyBlock, m - lb0), sl2e, mrun, lrun, o, lane, wave_live);
    __syncthreads();
  }
}

// LDS of the persistent gather kernel: the routed key/value block, the slice's
// landmark block (kept resident while consecutive tiles share a slice; also the
// staging area when m > 64) and the workgroup's list of tiles.
template <typename T, int D, bool FUSED>
struct GatherLds {
  using TL = Tiles<T, D>;
  __align__(16) T rk[TL::KTILE];
  __align__(16) T rv[TL::VTILE];
  AttnLds<T, D> lm;      // landmark block (used only when the landmark part is fused)
  int4 tile[256];
  int tz[256];
  uint32_t wtot[4];
};
template <typename T, int D>
struct GatherLds<T, D, false> {
  using TL = Tiles<T, D>;
  __align__(16) T rk[TL::KTILE];
  __align__(16) T rv[TL::VTILE];
  int4 tile[256];
  int tz[256];
  uint32_t wtot[4];
};

// LDS of the one-pass kernel: two routed key/value blocks (tile t computes from
// one while tile t + 1 is written to the other), the slice's landmark block and
// the workgroup's list of tiles.
template <typename T, int D>
struct Gather1Lds {
  using TL = Tiles<T, D>;
  __align__(16) T rk[2][TL::KTILE];
  __align__(16) T rv[2][TL::VTILE];
  AttnLds<T, D> lm;
  int4 tile[256];
  int tz[256];
  uint32_t wtot[4];
};

template <typename T, int D, int KP>
__device__ __forceinline__ void attend_tiles(const T* kt0, const T* kt1, const T* vt, const QFrag<T, D>& qf,
                                             int live, float sl2e, float& mrun, float& lrun, f32x4 (&o)[D / 16],
                                             int lane) {
  f32x4 acc[4];
  if constexpr (sizeof(T) == 2)
    qk_bf16<D, KP, 1>((const uint16_t*)kt0, (const uint16_t*)kt1, qf.b, acc, lane);
  else
    qk_f32<D>((const float*)kt0, qf.f, acc, lane);
  const float alpha = online_softmax(acc, live, sl2e, mrun, lrun, lane);
  rescale<D>(o, alpha);
  if constexpr (sizeof(T) == 2)
    pv_bf16<D>((const uint16_t*)vt, acc, o, lane);
  else
    pv_f32<D>((const float*)vt, acc, o, lane);
}

// Row indices (token ids) of a thread's share of one 64-row routed block,
// fetched ahead of the rows themselves.
template <typename T, int D>
struct RowIdx {
  static constexpr int PK = RowRegs<T, D>::PER;
  static constexpr int PV = sizeof(T) == 2 ? VtRegs<D>::RPT : RowRegs<T, D>::PER;
  int ik[PK], iv[PV];
  __device__ __forceinline__ void load(const int32_t* Ie, int k, int kb, int tid) {
    constexpr int CPR = RowRegs<T, D>::CPR;
#pragma unroll
    for (int u = 0; u < PK; ++u) ik[u] = Ie[min(kb + (tid + 256 * u) / CPR, k - 1)];
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      const int r = sizeof(T) == 2 ? (tid / VtRegs<D>::CPR) * VtRegs<D>::RPT + u : (tid + 256 * u) / CPR;
      iv[u] = Ie[min(kb + r, k - 1)];
    }
  }
};

// Rows of a routed block from already-fetched indices. The indices are clamped
// to the expert's last token, so rows past the block's end repeat a real row;
// the softmax masks those keys. (No select after the load: the compiler would
// turn it into a branch, and the registers it leaves pending force a full wait
// further on.)
template <typename T, int D>
__device__ __forceinline__ void load_rows(KVRegs<T, D, 1>& R, const RowIdx<T, D>& ix, const T* Kz, const T* Vz,
                                          int tid) {
  using RK = RowRegs<T, D>;
#pragma unroll
  for (int u = 0; u < RK::PER; ++u) {
    const int c = tid + 256 * u, cc = (c % RK::CPR) * RK::EPC;
    R.k[0].v[u] = ld16(Kz + (size_t)ix.ik[u] * D + cc);
  }
  if constexpr (sizeof(T) == 2) {
    using VR = VtRegs<D>;
    const int cc = (tid % VR::CPR) * 8;
#pragma unroll
    for (int u = 0; u < VR::RPT; ++u) R.v.v[u] = ld16(Vz + (size_t)ix.iv[u] * D + cc);
  } else {
#pragma unroll
    for (int u = 0; u < RK::PER; ++u) {
      const int c = tid + 256 * u, cc = (c % RK::CPR) * RK::EPC;
      R.v.v[u] = ld16(Vz + (size_t)ix.iv[u] * D + cc);
    }
  }
}

// Persistent expert-grouped attention. The tile table (slice-major, the tiles
// of one expert adjacent) is cut into one contiguous run per group of gs
// workgroups; the gs members of a group sit on one XCD (workgroups go
// round-robin to the 8 XCDs) and each takes every gs-th entry of the run, so
// they work on neighbouring tiles of the same expert at the same time and that
// expert's gathered rows come from the XCD's L2 after the first read. Each
// workgroup lists its real tiles in LDS and streams their 64-key routed blocks
// (block j = tile j / B, keys 64 (j % B), B = ceil(k / 64)). While block j
// computes, the rows of block j + 1 (their indices already in registers) and the
// indices of block j + 2 are in flight, so no prefetch waits on a dependent
// load; during a tile's last block, so are the next tile's query rows. FUSED (s = 1, m <= 64): each tile also attends the slice's landmark
// pairs, kept resident in LDS while the slice does not change.
// The bf16 d = 64 forms need only a few registers more than three waves per
// SIMD allow: held to three.
template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && D == 64 ? 3 : 1)))
void gather_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, const int32_t* __restrict__ I,
                                                     const int4* __restrict__ tiles, const int32_t* __restrict__ perm,
                                                     const void* __restrict__ qtop, const void* __restrict__ vtop,
                                                     T* __restrict__ out, void* __restrict__ pacc,
                                                     float* __restrict__ pml, int N, int m, int k, int s,
                                                     int max_tiles, long total, long gchunk, int gs, float sl2e,
                                                     float* __restrict__ lse) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  constexpr int KP = BF ? 2 : 1;
  __shared__ GatherLds<T, D, FUSED> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int rowi = 16 * w + r;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3, gpx = (int)(gridDim.x >> 3) / gs;
  if (jx >= gpx * gs) return;   // workgroup-uniform
  const int grp = xcd * gpx + jx / gs, jj = jx % gs;
  // this workgroup's entries: g0 + jj + gs e, e = 0 .. nent - 1
  const long g0 = (long)grp * gchunk, g1 = min(total, g0 + gchunk);
  const long nent = g1 - g0 > jj ? (g1 - g0 - jj + gs - 1) / gs : 0;
  // FUSED (s = 1, m <= 64): the slice's landmark block stays resident in LDS
  const bool resident = FUSED;
  const int B = (k + kKeyBlock - 1) / kKeyBlock;

  for (long base = 0; base < nent; base += 256) {
    // list the real tiles of this batch of entries
    const long e = base + tid, ent = g0 + jj + gs * e;
    const int4 te = e < nent ? tiles[ent] : make_int4(-1, 0, 0, 0);
    const uint32_t f = te.x >= 0 ? 1u : 0u;
    uint32_t nt;
    const uint32_t pos = block_incl_scan(f, sm.wtot, nt) - f;
    if (f) {
      sm.tile[pos] = te;
      sm.tz[pos] = (int)(ent / max_tiles);
    }
    __syncthreads();
    if (nt == 0) continue;
    const int nblk = (int)nt * B;
    // block j -> (slice, expert index list, key offset); past the end: the last block
    auto blk = [&](int j, int& zb, const int32_t*& Ieb, int& kbb) {
      j = min(j, nblk - 1);
      const int ti = j / B;
      zb = sm.tz[ti];
      Ieb = I + ((size_t)zb * m + sm.tile[ti].x) * k;
      kbb = (j % B) * kKeyBlock;
    };

    // prologue: rows of block 0, indices of block 1, query ids and rows of tile 0
    RowIdx<T, D> ix;
    KVRegs<T, D, 1> RR;
    {
      int zb, kbb;
      const int32_t* Ieb;
      blk(0, zb, Ieb, kbb);
      ix.load(Ieb, k, kbb, tid);
      load_rows<T, D>(RR, ix, K + (size_t)zb * N * D, V + (size_t)zb * N * D, tid);
      blk(1, zb, Ieb, kbb);
      ix.load(Ieb, k, kbb, tid);
    }
    // query ids: tile 0 and 1 now, tile t + 2 while tile t runs; query rows of
    // tile t + 1 while tile t runs (their ids arrived a tile earlier)
    auto qid = [&](int t) {
      t = min(t, (int)nt - 1);
      const int4 te = sm.tile[t];
      return perm[(size_t)sm.tz[t] * N * s + te.w + min(rowi, te.z - 1)];
    };
    int4 cur = sm.tile[0];
    int zc = sm.tz[0], zl = -1;
    int entry = qid(0), entry_n = qid(1), entry_nn = entry_n;
    QFrag<T, D> qf;
    qf.load(Q + ((size_t)zc * N + entry / s) * D, g);
    QFrag<T, D> qf_n = qf;
    float mrun = -INFINITY, lrun = 0.f;
    f32x4 o[D / 16];

    for (int j = 0; j < nblk; ++j) {
      const int ti = j / B, kb = (j % B) * kKeyBlock;
      const bool newtile = kb == 0;   // block-uniform
      if (newtile) {
        if (j > 0) {
          cur = sm.tile[ti];
          zc = sm.tz[ti];
          entry = entry_n;
          entry_n = entry_nn;
          qf = qf_n;
        }
        entry_nn = qid(ti + 2);
        mrun = -INFINITY;
        lrun = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();   // earlier readers of the routed (and landmark) tiles are done
      RR.k[0].store(sm.rk, TL::KSTR, tid);
      if constexpr (BF) RR.v.store((uint16_t*)sm.rv, tid); else RR.v.store(sm.rv, TL::VSTR, tid);
      if constexpr (FUSED) {
        if (resident && newtile && zc != zl) {   // the slice's landmark block, staged once per slice
          KVRegs<T, D, KP> LR;
          load_landmarks<T, D>(LR, qtop, vtop, zc, m, 0, tid);
          LR.store(sm.lm, tid);
          zl = zc;
        }
      }
      __syncthreads();
      {   // rows of block j + 1 (indices in hand), indices of block j + 2, query rows of the next tile
        int zb, kbb;
        const int32_t* Ieb;
        blk(j + 1, zb, Ieb, kbb);
        load_rows<T, D>(RR, ix, K + (size_t)zb * N * D, V + (size_t)zb * N * D, tid);
        blk(j + 2, zb, Ieb, kbb);
        ix.load(Ieb, k, kbb, tid);
        if (kb + kKeyBlock >= k) {   // the tile's last block: the next tile's query rows (block-uniform)
          const int tn = min(ti + 1, (int)nt - 1);
          qf_n.load(Q + ((size_t)sm.tz[tn] * N + entry_n / s) * D, g);
        }
      }
      const bool wave_live = 16 * w < cur.z;
      if constexpr (FUSED) {   // the landmark part, first block of each tile
        if (newtile && wave_live)
          attend_tiles<T, D, KP>(sm.lm.k0, sm.lm.k1, sm.lm.v, qf, m, sl2e, mrun, lrun, o, lane);
      }
      if (wave_live) attend_tiles<T, D, 1>(sm.rk, nullptr, sm.rv, qf, min(kKeyBlock, k - kb), sl2e, mrun, lrun, o, lane);

      if (kb + kKeyBlock >= k) {   // last block of the tile: write it out
        const float l = quad_sum(lrun);
        const int q = entry / s, slot = entry % s;
        if (rowi < cur.z) {
          if constexpr (FUSED) {
            T* orow = out + ((size_t)zc * N + q) * D;
            const float inv = 1.f / l;
            if (g == 0) lse[(size_t)zc * N + q] = mrun + log2f(l);
            store_row<T, D>(orow, o, inv, g);
          } else {   // the slot's output o / l, divided by its largest magnitude (the quad holds the row)
            const size_t ps = ((size_t)zc * N + q) * s + slot;
            const float inv = 1.f / l;
            float amax = 0.f;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
              for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(o[dt][j]));
            amax = quad_max(amax) * inv;
            const float sc = amax > 0.f ? amax : 1.f, wv = inv / sc;
            if constexpr (BF) {   // fp16 in [-1, 1]: 2^-11 relative to the slot's largest value
              uint16_t* prow = (uint16_t*)pacc + ps * D;   // 16-byte pieces (pair_trade)
#pragma unroll
              for (int dt = 0; dt < D / 16; dt += 2)
                *(uint4*)(prow + pair_col(dt, g)) =
                    pair_trade(make_uint2(pack_f16x2(o[dt][0] * wv, o[dt][1] * wv), pack_f16x2(o[dt][2] * wv, o[dt][3] * wv)),
                               make_uint2(pack_f16x2(o[dt + 1][0] * wv, o[dt + 1][1] * wv),
                                          pack_f16x2(o[dt + 1][2] * wv, o[dt + 1][3] * wv)));
            } else {
              float* prow = (float*)pacc + ps * D;
#pragma unroll
              for (int dt = 0; dt < D / 16; ++dt)
                *(float4*)(prow + 16 * dt + 4 * g) =
                    make_float4(o[dt][0] * wv, o[dt][1] * wv, o[dt][2] * wv, o[dt][3] * wv);
            }
            if (g == 0) *(float4*)(pml + ps * 4) = make_float4(mrun, l, sc, 0.f);
          }
        }
      }
    }
    __syncthreads();   // the tile list is rewritten by the next batch
  }
}

// Routed part of the output for bf16 inputs when each (query, slot) pair leaves a
// partial softmax (s > 1 or m > 64). Tiles of 64 QT queries of one bucket: each
// wave owns QT column tiles of 16 queries, so every K and V fragment it reads
// from LDS feeds QT MFMAs. Same persistent walk as gather_kernel (groups of gs
// workgroups on one XCD, interleaved over a contiguous run of the tile table, so
// an expert's gathered rows are shared through that XCD's L2). The routed blocks
// are staged by direct global-to-LDS loads into swizzled tiles (no staging
// registers: that room goes to the second column tile) and double-buffered: a
// block's rows are requested one block ahead (they land while the previous block
// computes), its token ids two blocks ahead, and during a tile's last block the
// next tile's query rows load into the registers of the current ones once its
// last scores are taken. V stays row-major and is read transposed. While a wave's
// MFMA work is in flight its priority is raised, so the other wave of the SIMD
// does its softmax meanwhile. Held to two waves per SIMD. The softmax keeps a
// lazily raised reference and sums the probabilities as rounded for P V
// (lazy_softmax).
// Landmark merge (bf16): waves per workgroup and landmark buffers. Four-wave
// workgroups, two per CU, so while one waits for its partials the other computes
// (eight waves in one workgroup run in lockstep: very long merge 1.41 ms against
// 1.24 ms). With Q~ staged as one bf16 tile, two buffers take 64 KB of LDS for
// d = 128 and two workgroups still fit a CU; the next block then loads while this
// one computes: very long merge 1.16 -> 1.07 ms, long 0.62 -> 0.58 ms against one
// buffer.
constexpr int kCombineWaves = 4, kCombineBuffers = 2;

template <int D>
struct GatherDLds {
  __align__(16) uint16_t rk[2][SwzTile<D>::TILE];
  __align__(16) uint16_t rv[2][SwzTile<D>::TILE];
  int4 tile[256];
  int tz[256];
  uint32_t wtot[4];
};

// KFULL: k is a multiple of the key block (no block of an expert is partial, and
// the kernel carries no masking code).
template <int D, int QT, bool KFULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gatherd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ I, const int4* __restrict__ tiles, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ pacc, float* __restrict__ pml, int N, int m, int k, int s, int max_tiles, long total,
    long gchunk, int gs, float sl2e) {
  using T = uint16_t;
  using S = SwzTile<D>;
  __shared__ GatherDLds<D> sm;
  // Two column tiles per wave: wave-uniform values in scalar registers (scalar
  // row offsets and LDS targets, a scalar branch for idle waves) and buffer
  // loads for the staged rows cut a fifth of the vector instructions per block
  // and measured faster; with one column tile (64-row tiles, more idle waves)
  // the same changes measured slower, so that form keeps vector values.
  constexpr bool kScalar = QT == 2;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
  const int w = kScalar ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int row0 = QT * 16 * w + (lane & 15);   // row of the wave's column tile qt: row0 + 16 qt
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3, gpx = (int)(gridDim.x >> 3) / gs;
  if (jx >= gpx * gs) return;   // workgroup-uniform
  const int grp = xcd * gpx + jx / gs, jj = jx % gs;
  const long g0 = (long)grp * gchunk, g1 = min(total, g0 + gchunk);
  const long nent = g1 - g0 > jj ? (g1 - g0 - jj + gs - 1) / gs : 0;
  const int B = (k + kKeyBlock - 1) / kKeyBlock;

  for (long base = 0; base < nent; base += 256) {
    const long e = base + tid, ent = g0 + jj + gs * e;
    const int4 te = e < nent ? tiles[ent] : make_int4(-1, 0, 0, 0);
    const uint32_t f = te.x >= 0 ? 1u : 0u;
    uint32_t nt;
    const uint32_t pos = block_incl_scan(f, sm.wtot, nt) - f;
    if (f) {
      sm.tile[pos] = te;
      sm.tz[pos] = (int)(ent / max_tiles);
    }
    __syncthreads();
    if (nt == 0) continue;
    const int nblk = (int)nt * B;
    // Cursor of the token ids being fetched (two blocks ahead of the block that
    // computes): tile it2, block bi2 of it, and that tile's slice and expert list,
    // read from the tile table only when the cursor enters a tile (past the last
    // tile it stays on the last one: those ids are fetched, never staged).
    int it2 = 0, bi2 = 0, zI = 0;
    const int32_t* IeI = I;
    auto enter = [&](int t) {
      t = min(t, (int)nt - 1);
      zI = kScalar ? __builtin_amdgcn_readfirstlane(sm.tz[t]) : sm.tz[t];
      const int ex = kScalar ? __builtin_amdgcn_readfirstlane(sm.tile[t].x) : sm.tile[t].x;
      IeI = I + ((size_t)zI * m + ex) * k;
    };
    enter(0);
    // the slice's K and V as raw buffers: each staged row is a 32-bit offset
    auto rsK = [&](int zb) { return raw_rsrc(K + (size_t)zb * N * D, (uint32_t)N * D * 2); };
    auto rsV = [&](int zb) { return raw_rsrc(V + (size_t)zb * N * D, (uint32_t)N * D * 2); };
    // token ids of this lane's rows of the cursor's block (rows past the expert's
    // end repeat its last token), then the cursor moves one block on
    auto ids = [&](int (&id)[S::NI], int& zb) {
      zb = zI;
      const int kbb = bi2 * kKeyBlock;
#pragma unroll
      for (int u = 0; u < S::NI; ++u) id[u] = IeI[min(kbb + 16 * w + u * S::RPI + lane / S::CPR, k - 1)];
      if (++bi2 == B) {
        bi2 = 0;
        enter(++it2);
      }
    };
    auto qids = [&](int t, int (&ent_)[QT]) {
      t = min(t, (int)nt - 1);
      const int4 tt = sm.tile[t];
      const size_t pb = (size_t)sm.tz[t] * N * s + tt.w;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) ent_[qt] = perm[pb + min(row0 + 16 * qt, tt.z - 1)];
    };
    auto qload = [&](int t, const int (&ent_)[QT], uint4 (&qf_)[QT][D / 32]) {
      const T* Qz = Q + (size_t)sm.tz[min(t, (int)nt - 1)] * N * D;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const T* qrow = Qz + (size_t)(ent_[qt] / s) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) qf_[qt][ks] = ld16(qrow + 32 * ks + 8 * g);
      }
    };

    // prologue: block 0 requested into buffer 0, ids of block 1 in flight
    int id_n[S::NI], z_n;
    {
      int id0[S::NI], z0;
      ids(id0, z0);
      if constexpr (kScalar)
        dma_rows_buf<D>(sm.rk[0], sm.rv[0], rsK(z0), rsV(z0), id0, w, lane);
      else
        dma_rows<D>(sm.rk[0], sm.rv[0], K + (size_t)z0 * N * D, V + (size_t)z0 * N * D, id0, w, lane);
      ids(id_n, z_n);
    }
    int qe[QT], qe_n[QT], qe_nn[QT];
    qids(0, qe);
    qids(1, qe_n);
    uint4 qf[QT][D / 32];
    qload(0, qe, qf);
    float mrun[QT], lrun[QT];
    f32x4 o[QT][D / 16];
    int4 cur = sm.tile[0];
    int zc = sm.tz[0];

    for (int j = 0, ti = 0, bi = 0; j < nblk; ++j) {   // block bi of tile ti
      const int kb = bi * kKeyBlock;
      const bool newtile = kb == 0;   // block-uniform
      const bool lastblk = kb + kKeyBlock >= k;
      if (newtile) {
        if (j > 0) {
          cur = sm.tile[ti];
          zc = sm.tz[ti];
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            qe[qt] = qe_n[qt];
            qe_n[qt] = qe_nn[qt];
          }
        }
        qids(ti + 2, qe_nn);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          mrun[qt] = -INFINITY;
          lrun[qt] = 0.f;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // this wave's loads of block j have landed; after the barrier every wave's
      // have, and every wave is done with block j - 1 (buffer (j + 1) & 1 is free)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // The next block's loads and this block's reads go through distinct
      // __restrict__ parameters of one inlined function, so the compiler knows
      // they cannot overlap and does not wait for the loads before the reads.
      auto step = [&](uint16_t* __restrict__ nk, uint16_t* __restrict__ nv, const uint16_t* __restrict__ ck,
                      const uint16_t* __restrict__ cv) __attribute__((always_inline)) {
        if (j + 1 < nblk) {   // block-uniform
          if constexpr (kScalar)
            dma_rows_buf<D>(nk, nv, rsK(z_n), rsV(z_n), id_n, w, lane);
          else
            dma_rows<D>(nk, nv, K + (size_t)z_n * N * D, V + (size_t)z_n * N * D, id_n, w, lane);
        }
        ids(id_n, z_n);
        // The wave has live rows (with kScalar a scalar condition, so the two paths
        // stay apart). The scores live inside the busy path (merging them with the
        // idle path would cost a register fill per block); the next tile's query
        // rows (block-uniform) load once the scores no longer need qf.
        const bool live = QT * 16 * w < (kScalar ? __builtin_amdgcn_readfirstlane(cur.z) : cur.z);
        if (live) {
          f32x4 acc[QT][4];
          __builtin_amdgcn_s_setprio(kGatherPrio);
          qk_bf16_swz<D, QT>(ck, qf, acc, lane);
          if (lastblk) qload(ti + 1, qe_n, qf);
          lazy_softmax<D, QT>(acc, KFULL ? kKeyBlock : min(kKeyBlock, k - kb), sl2e, mrun, lrun, o, lane);
          pv_bf16_swz<D, QT>(cv, acc, o, lrun, lane);
          __builtin_amdgcn_s_setprio(0);
        } else if (lastblk) {
          // an idle wave waits for its loads here: the compiler may lay this path
          // out ahead of the busy one, and loads left in flight would then make the
          // busy path's key reads wait for them
          qload(ti + 1, qe_n, qf);
          if constexpr (kScalar) __builtin_amdgcn_s_waitcnt(0);
        }
      };
      step(sm.rk[(j + 1) & 1], sm.rv[(j + 1) & 1], sm.rk[j & 1], sm.rv[j & 1]);
      if (lastblk) {   // the tile's partials: o / l divided by its largest magnitude, as fp16
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float l = quad_sum(lrun[qt]);
          if (row0 + 16 * qt < cur.z) {
            const int q = qe[qt] / s, slot = qe[qt] % s;
            const size_t ps = ((size_t)zc * N + q) * s + slot;
            const float inv = 1.f / l;
            float amax = 0.f;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
              for (int jj2 = 0; jj2 < 4; ++jj2) amax = fmaxf(amax, fabsf(o[qt][dt][jj2]));
            amax = quad_max(amax) * inv;
            const float sc = amax > 0.f ? amax : 1.f, wv = inv / sc;
            uint16_t* prow = pacc + ps * D;
            // 16-byte pieces (pair_trade): the row's four lanes store 64 contiguous bytes
#pragma unroll
            for (int dt = 0; dt < D / 16; dt += 2)
              *(uint4*)(prow + pair_col(dt, g)) =
                  pair_trade(make_uint2(pack_f16x2(o[qt][dt][0] * wv, o[qt][dt][1] * wv),
                                        pack_f16x2(o[qt][dt][2] * wv, o[qt][dt][3] * wv)),
                             make_uint2(pack_f16x2(o[qt][dt + 1][0] * wv, o[qt][dt + 1][1] * wv),
                                        pack_f16x2(o[qt][dt + 1][2] * wv, o[qt][dt + 1][3] * wv)));
            if (g == 0) *(float4*)(pml + ps * 4) = make_float4(mrun[qt], l, sc, 0.f);
          }
        }
      }
      if (++bi == B) {
        bi = 0;
        ++ti;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // the tile list and the buffers are rewritten by the next batch
  }
}

// Scores of one staged 64-key block against the wave's 16 queries (S^T tile),
// keys past `live` set to -inf.
template <typename T, int D, int KP>
__device__ __forceinline__ void block_scores(const T* k0, const T* k1, const QFrag<T, D>& qf, int live,
                                             f32x4 (&x)[4], int lane) {
  if constexpr (sizeof(T) == 2)
    qk_bf16<D, KP, 1>((const uint16_t*)k0, (const uint16_t*)k1, qf.b, x, lane);
  else
    qk_f32<D>((const float*)k0, qf.f, x, lane);
  if (live < kKeyBlock) {
    const int g = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (16 * kt + 4 * g + j >= live) x[kt][j] = -INFINITY;
  }
}

// s = 1 with k <= 64 and m <= 64: every tile is one routed block plus the
// slice's landmark block, so the softmax over the m + k keys is taken in one
// pass (no running rescale). Same persistent walk as gather_kernel; the routed
// blocks are double-buffered in LDS, so each tile needs one barrier. While tile
// t computes, the rows of tiles t + 2 and t + 3 (two register sets), the expert
// indices of tile t + 4, the query rows of tiles t + 1 and t + 2 and the query
// ids of tile t + 3 are in flight: three workgroups' LDS would not fit in a CU,
// so the two resident ones hide the gathers' latency with depth instead.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather1_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const T* __restrict__ V, const int32_t* __restrict__ I,
                                                      const int4* __restrict__ tiles, const int32_t* __restrict__ perm,
                                                      const void* __restrict__ qtop, const void* __restrict__ vtop,
                                                      T* __restrict__ out, int N, int m, int k, int max_tiles,
                                                      int BH, int gs, float sl2e, float* __restrict__ lse) {
  using TL = Tiles<T, D>;
  constexpr bool BF = TL::BF;
  constexpr int KP = BF ? 2 : 1;
  __shared__ Gather1Lds<T, D> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int rowi = 16 * w + r;
  // Workgroups go round-robin to the 8 XCDs. The gs workgroups of a group (all
  // on one XCD) share one slice at a time, each taking every gs-th entry of its
  // tile table, so the slice's gathered rows, which recur across experts, are
  // served from that XCD's L2.
  const int xcd = blockIdx.x % 8, jx = blockIdx.x / 8, gpx = (int)(gridDim.x / 8) / gs;
  if (jx >= gpx * gs) return;   // workgroup-uniform
  const int grp = xcd * gpx + jx / gs, jj = jx % gs, ngroups = 8 * gpx;
  const int per = (max_tiles + gs - 1) / gs;
  // this workgroup's entries, slice after slice: entry e is table entry
  // jj + gs (e % per) of slice grp + (e / per) ngroups (interleaved, because the
  // real tiles sit at the front of each slice's table)
  const long nent = (long)((BH - grp + ngroups - 1) / ngroups) * per;

  for (long base = 0; base < nent; base += 256) {
    const long e = base + tid;
    const int zs = grp + (int)(e / per) * ngroups, off = jj + gs * (int)(e % per);
    const bool in = e < nent && zs < BH && off < max_tiles;
    const long ent = in ? (long)zs * max_tiles + off : 0;
    const int4 te = in ? tiles[ent] : make_int4(-1, 0, 0, 0);
    const uint32_t f = te.x >= 0 ? 1u : 0u;
    uint32_t nt;
    const uint32_t pos = block_incl_scan(f, sm.wtot, nt) - f;
    if (f) {
      sm.tile[pos] = te;
      sm.tz[pos] = (int)(ent / max_tiles);
    }
    __syncthreads();
    if (nt == 0) continue;
    const int last = (int)nt - 1;
    auto expert = [&](int t) {   // index list of tile t's expert (past the end: the last tile)
      t = min(t, last);
      return I + ((size_t)sm.tz[t] * m + sm.tile[t].x) * k;
    };
    auto qid = [&](int t) {      // query id of this thread's row of tile t
      t = min(t, last);
      const int4 e = sm.tile[t];
      return perm[(size_t)sm.tz[t] * N + e.w + min(rowi, e.z - 1)];
    };
    auto slice_kv = [&](int t, const T*& Kb, const T*& Vb) {
      const size_t o = (size_t)sm.tz[min(t, last)] * N * D;
      Kb = K + o;
      Vb = V + o;
    };
    auto store_rows = [&](const KVRegs<T, D, 1>& R, int b) {
      R.k[0].store(sm.rk[b], TL::KSTR, tid);
      if constexpr (BF) R.v.store((uint16_t*)sm.rv[b], tid); else R.v.store(sm.rv[b], TL::VSTR, tid);
    };

    // prologue: tile 0's rows straight to buffer 0, tile 1's rows in RA, tile
    // 2's in RB, tile 3's indices in flight; query rows of tiles 0 and 1
    RowIdx<T, D> ix;
    KVRegs<T, D, 1> RA, RB;
    {
      const T *Kb, *Vb;
      ix.load(expert(0), k, 0, tid);
      slice_kv(0, Kb, Vb);
      load_rows<T, D>(RA, ix, Kb, Vb, tid);
      ix.load(expert(1), k, 0, tid);
      store_rows(RA, 0);
      slice_kv(1, Kb, Vb);
      load_rows<T, D>(RA, ix, Kb, Vb, tid);
      ix.load(expert(2), k, 0, tid);
      slice_kv(2, Kb, Vb);
      load_rows<T, D>(RB, ix, Kb, Vb, tid);
      ix.load(expert(3), k, 0, tid);
    }
    int q = qid(0), q_n = qid(1), q_nn = qid(2), q_n3 = q_nn;
    QFrag<T, D> qf, qf_n;
    qf.load(Q + ((size_t)sm.tz[0] * N + q) * D, g);
    qf_n.load(Q + ((size_t)sm.tz[min(1, last)] * N + q_n) * D, g);
    QFrag<T, D> qf_nn = qf_n;
    int zl = -1;   // slice in the landmark buffer

    // one barrier per tile: at iteration t the rows of tile t + 1 (in Rc) go to
    // the other buffer, whose last readers (tile t - 1) finished before the
    // barrier; Rc then takes the rows of tile t + 3, while Rn holds tile t + 2's
    auto tile_step = [&](int t, KVRegs<T, D, 1>& Rc) {
      const int4 cur = sm.tile[t];
      const int zc = sm.tz[t];
      if (t > 0) {
        q = q_n;
        q_n = q_nn;
        q_nn = q_n3;
        qf = qf_n;
        qf_n = qf_nn;
      }
      q_n3 = qid(t + 3);
      __syncthreads();
      store_rows(Rc, (t + 1) & 1);
      if (zc != zl) {   // a new slice: its landmark block (uniform branch)
        KVRegs<T, D, KP> LR;
        load_landmarks<T, D>(LR, qtop, vtop, zc, m, 0, tid);
        LR.store(sm.lm, tid);
        zl = zc;
        __syncthreads();
      }
      {   // rows of tile t + 3 (indices in hand), indices of tile t + 4, query rows of tile t + 2
        const T *Kb, *Vb;
        slice_kv(t + 3, Kb, Vb);
        load_rows<T, D>(Rc, ix, Kb, Vb, tid);
        ix.load(expert(t + 4), k, 0, tid);
        qf_nn.load(Q + ((size_t)sm.tz[min(t + 2, last)] * N + q_nn) * D, g);
      }
      if (16 * w < cur.z) {   // wave has live rows (uniform)
        const int b = t & 1;
        f32x4 xl[4], xr[4];
        block_scores<T, D, KP>(sm.lm.k0, sm.lm.k1, qf, m, xl, lane);
        block_scores<T, D, 1>(sm.rk[b], nullptr, qf, k, xr, lane);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(xl[kt][j], xr[kt][j]));
        mx = quad_max(mx) * sl2e;
        float l = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xl[kt][j] = __builtin_amdgcn_exp2f(fmaf(xl[kt][j], sl2e, -mx));
            xr[kt][j] = __builtin_amdgcn_exp2f(fmaf(xr[kt][j], sl2e, -mx));
            l += xl[kt][j] + xr[kt][j];
          }
        f32x4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
          pv_bf16<D>((const uint16_t*)sm.lm.v, xl, o, lane);
          pv_bf16<D>((const uint16_t*)sm.rv[b], xr, o, lane);
        } else {
          pv_f32<D>((const float*)sm.lm.v, xl, o, lane);
          pv_f32<D>((const float*)sm.rv[b], xr, o, lane);
        }
        const float lt = quad_sum(l), inv = 1.f / lt;
        if (rowi < cur.z) {
          if (g == 0) lse[(size_t)zc * N + q] = mx + log2f(lt);
          T* orow = out + ((size_t)zc * N + q) * D;
          store_row<T, D>(orow, o, inv, g);
        }
      }
    };
    for (int t = 0; t < (int)nt; t += 2) {   // two steps per trip: the register sets swap roles
      tile_step(t, RA);
      if (t + 1 < (int)nt) tile_step(t + 1, RB);
    }
    __syncthreads();   // the tile list is rewritten by the next batch
  }
}

// s > 1: landmark part for 64 consecutive queries, merged with their s partials.
// The partial softmaxes seed the online-softmax state (reference max, sum and
// unnormalised output), so their loads overlap those of the query rows and the
// first landmark block; the landmark blocks then continue the same softmax.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ Q, const void* __restrict__ qtop,
                                                      const void* __restrict__ vtop, const void* __restrict__ pacc,
                                                      const float* __restrict__ pml, T* __restrict__ out, int N, int m,
                                                      int s, float sl2e, float* __restrict__ lse) {
  __shared__ AttnLds<T, D> sm;
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int q = blockIdx.x * kQueryTile + 16 * w + r;
  const bool ok = q < N;
  const int qc = ok ? q : N - 1;
  QFrag<T, D> qf;
  qf.load(Q + ((size_t)z * N + qc) * D, g);
  KVRegs<T, D, sizeof(T) == 2 ? 2 : 1> LR;
  load_landmarks<T, D>(LR, qtop, vtop, z, m, 0, tid);
  // seed: M = the largest partial reference; o, l = the partials rescaled to it
  // (l on one lane of the quad: the lanes' sums are added at the end)
  const size_t p0 = ((size_t)z * N + qc) * s;
  float M = -INFINITY;
  for (int sl = 0; sl < s; ++sl) M = fmaxf(M, pml[(p0 + sl) * 4]);
  float lrun = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < s; ++sl) {   // slot partial: (max, sum, scale) and its output / (sum * scale)
    const float4 ml = *(const float4*)(pml + (p0 + sl) * 4);
    const float f = exp2f(ml.x - M);
    lrun += f * ml.y;
    const float wv = f * ml.y * ml.z;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float4 a;
      if constexpr (sizeof(T) == 2) {   // 16-byte pieces (pair_untrade)
        if (dt % 2) continue;
        uint2 u0, u1;
        pair_untrade(*(const uint4*)((const uint16_t*)pacc + (p0 + sl) * D + pair_col(dt, g)), u0, u1);
        o[dt + 1][0] += wv * f16_lo(u1.x);
        o[dt + 1][1] += wv * f16_hi(u1.x);
        o[dt + 1][2] += wv * f16_lo(u1.y);
        o[dt + 1][3] += wv * f16_hi(u1.y);
        a = make_float4(f16_lo(u0.x), f16_hi(u0.x), f16_lo(u0.y), f16_hi(u0.y));
      } else {
        a = *(const float4*)((const float*)pacc + (p0 + sl) * D + 16 * dt + 4 * g);
      }
      o[dt][0] += wv * a.x;
      o[dt][1] += wv * a.y;
      o[dt][2] += wv * a.z;
      o[dt][3] += wv * a.w;
    }
  }
  if (g != 0) lrun = 0.f;
  float mrun = M;
  attend_landmarks<T, D>(sm, LR, qf, qtop, vtop, z, m, sl2e, mrun, lrun, o, tid);
  if (!ok) return;
  const float lt = quad_sum(lrun), inv = 1.f / lt;
  if (g == 0) lse[(size_t)z * N + q] = mrun + log2f(lt);
  T* orow = out + ((size_t)z * N + q) * D;
  store_row<T, D>(orow, o, inv, g);
}

// The same for bf16 inputs with NW waves of QT column tiles (16 QT NW consecutive
// queries per workgroup): the landmark blocks (Q~ as bf16, V~) are staged by
// direct loads into tiles that every wave reads (V~ transposed), so each block is
// fetched once per 16 QT NW queries and each fragment read feeds QT MFMAs. These
// scores only weight the output (no selection rests on them), so Q~ takes the
// precision of the other bf16 operands: its hi plane, the bf16 rounding of the
// fp64 landmark (routing and the expert sets use both planes). The softmax keeps
// a lazily raised reference and sums the probabilities as rounded for the product
// (see lazy_softmax).
// MFULL: m is a multiple of the key block (no masking code). SU: partial slots
// loaded together in the seed (1, 2 or 4). NB: landmark buffers (2: the next
// block loads while one computes; 1: less LDS, so more workgroups per CU).
template <int D, int QT, int NW, bool MFULL, int SU, int NB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void combined_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ qtop, const uint16_t* __restrict__ vt16,
    const uint16_t* __restrict__ pacc, const float* __restrict__ pml, uint16_t* __restrict__ out, int N, int m, int s,
    float sl2e, float* __restrict__ lse) {
  using U = UTile<D>;
  // one shared object: with separate ones the compiler's LDS scopes would make the
  // next block's loads look like writes to the block being read
  __shared__ __align__(16) struct {
    uint16_t kk[NB][U::TILE];   // Q~ (hi plane)
    uint16_t vv[NB][U::TILE];
  } sm;
  const int z = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int qw = blockIdx.x * (16 * QT * NW) + QT * 16 * w + r;   // query of column tile qt: qw + 16 qt
  const uint16_t* hz = qtop + (size_t)z * 2 * m * D;
  const uint16_t* vz = vt16 + (size_t)z * m * D;
  auto stage = [&](int lb, uint16_t* tk, uint16_t* tv) __attribute__((always_inline)) {
    udma<D, NW, false>(tk, [&](int row) __attribute__((always_inline)) { return hz + (size_t)min(lb + row, m - 1) * D; }, w, lane);
    udma<D, NW, true>(tv, [&](int row) __attribute__((always_inline)) { return vz + (size_t)min(lb + row, m - 1) * D; }, w, lane);
  };
  stage(0, sm.kk[0], sm.vv[0]);
  // seed: per query, M = the largest partial reference; o, l = the partials rescaled to it
  // (l on one lane of the quad: the lanes' sums are added at the end). The first SU
  // slots' loads are all issued before any is used (slots past s repeat slot s - 1
  // with weight 0); slots past SU follow one at a time.
  uint4 qf[QT][D / 32];
  float mrun[QT], lrun[QT];
  f32x4 o[QT][D / 16];
  size_t p0[QT];
  float4 ml[QT][SU];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qc = min(qw + 16 * qt, N - 1);
    const uint16_t* qrow = Q + ((size_t)z * N + qc) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[qt][ks] = ld16(qrow + 32 * ks + 8 * g);
    p0[qt] = ((size_t)z * N + qc) * s;
#pragma unroll
    for (int sl = 0; sl < SU; ++sl) ml[qt][sl] = *(const float4*)(pml + (p0[qt] + min(sl, s - 1)) * 4);
  }
  // partial rows in the 16-byte pieces the routed kernel stores (pair_untrade below)
  uint4 u[QT][SU][D / 32];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int sl = 0; sl < SU; ++sl)
#pragma unroll
      for (int dp = 0; dp < D / 32; ++dp)
        u[qt][sl][dp] = *(const uint4*)(pacc + (p0[qt] + min(sl, s - 1)) * D + pair_col(2 * dp, g));
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float M = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < SU; ++sl) M = fmaxf(M, ml[qt][sl].x);
    for (int sl = SU; sl < s; ++sl) M = fmaxf(M, pml[(p0[qt] + sl) * 4]);
    float l = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto add = [&](const float4& m4, const uint4 (&uc)[D / 32], bool use) __attribute__((always_inline)) {
      const float f = use ? exp2f(m4.x - M) : 0.f;
      l += f * m4.y;
      const float wv = f * m4.y * m4.z;
#pragma unroll
      for (int dp = 0; dp < D / 32; ++dp) {
        uint2 uu[2];
        pair_untrade(uc[dp], uu[0], uu[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int dt = 2 * dp + h;
          o[qt][dt][0] += wv * f16_lo(uu[h].x);
          o[qt][dt][1] += wv * f16_hi(uu[h].x);
          o[qt][dt][2] += wv * f16_lo(uu[h].y);
          o[qt][dt][3] += wv * f16_hi(uu[h].y);
        }
      }
    };
#pragma unroll
    for (int sl = 0; sl < SU; ++sl) add(ml[qt][sl], u[qt][sl], sl < s);
    for (int sl = SU; sl < s; ++sl) {
      uint4 ut[D / 32];
#pragma unroll
      for (int dp = 0; dp < D / 32; ++dp) ut[dp] = *(const uint4*)(pacc + (p0[qt] + sl) * D + pair_col(2 * dp, g));
      add(*(const float4*)(pml + (p0[qt] + sl) * 4), ut, true);
    }
    mrun[qt] = M;
    lrun[qt] = g != 0 ? 0.f : l;
  }
  const int nb = (m + kKeyBlock - 1) / kKeyBlock;
  auto attend = [&](int j, const uint16_t* ck, const uint16_t* cv) __attribute__((always_inline)) {
    f32x4 acc[QT][4];
    __builtin_amdgcn_s_setprio(1);
    uqk<D, QT, 1>(ck, nullptr, qf, acc, lane);
    lazy_softmax<D, QT>(acc, MFULL ? kKeyBlock : min(kKeyBlock, m - j * kKeyBlock), sl2e, mrun, lrun, o, lane);
    upv<D, QT>(cv, acc, o, lrun, lane);
    __builtin_amdgcn_s_setprio(0);
  };
  for (int j = 0; j < nb; ++j) {
    if constexpr (NB == 1) {
      if (j > 0) {
        __syncthreads();   // every wave done with block j - 1
        stage(j * kKeyBlock, sm.kk[0], sm.vv[0]);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();   // block j staged
      attend(j, sm.kk[0], sm.vv[0]);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();   // block j staged; every wave done with block j - 1
      // the next block's loads and this block's reads go through distinct __restrict__
      // parameters, so the compiler does not wait for the loads before the reads
      auto step = [&](uint16_t* __restrict__ nk, uint16_t* __restrict__ nv, const uint16_t* __restrict__ ck,
                      const uint16_t* __restrict__ cv) __attribute__((always_inline)) {
        // unconditional (rows clamp to the last landmark): a branch around the loads
        // would merge two states here and the compiler would then wait for them
        stage((j + 1) * kKeyBlock, nk, nv);
        attend(j, ck, cv);
      };
      const int b = j & 1, nbuf = (j + 1) & 1;
      step(sm.kk[nbuf], sm.vv[nbuf], sm.kk[b], sm.vv[b]);
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = qw + 16 * qt;
    const float lt = quad_sum(lrun[qt]), inv = 1.f / lt;
    uint4 pc[D / 32];   // the row in 16-byte pieces (pair_trade), formed by all lanes
#pragma unroll
    for (int dp = 0; dp < D / 32; ++dp) {
      const f32x4 &a = o[qt][2 * dp], &b = o[qt][2 * dp + 1];
      pc[dp] = pair_trade(make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)),
                          make_uint2(pack_bf16x2(b[0] * inv, b[1] * inv), pack_bf16x2(b[2] * inv, b[3] * inv)));
    }
    if (q >= N) continue;
    if (g == 0) lse[(size_t)z * N + q] = mrun[qt] + log2f(lt);
    uint16_t* orow = out + ((size_t)z * N + q) * D;
#pragma unroll
    for (int dp = 0; dp < D / 32; ++dp) *(uint4*)(orow + pair_col(2 * dp, g)) = pc[dp];
  }
}

// Counting sort of the (query, slot) pairs by expert and the tile table.
hipError_t launch_bucket(const Plan& p, char* ws, hipStream_t st) {
  const int Ns = p.N * p.s;
  if (Ns <= 256 * kBucketSlicePer && (size_t)p.m * 8 <= 64 * 1024) {   // one workgroup per slice
    hipLaunchKernelGGL(bucket_slice_kernel<kBucketSlicePer>, dim3(p.BH), dim3(256), (size_t)p.m * 8, st,
                       (const int32_t*)(ws + p.ws.E), (uint32_t*)(ws + p.ws.boff), (int4*)(ws + p.ws.tiles),
                       (int32_t*)(ws + p.ws.perm), Ns, p.m, p.max_tiles, p.trows);
    return hipGetLastError();
  }
  const int nclear = (int)((p.ws.bcursor + (size_t)p.BH * p.m * 4 - p.ws.bcount) / 4);
  hipLaunchKernelGGL(clear_kernel, dim3(std::min(1024, (nclear + 255) / 256)), dim3(256), 0, st,
                     (uint32_t*)(ws + p.ws.bcount), nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 bgrid((Ns + 4095) / 4096, p.BH);
  hipLaunchKernelGGL(bucket_hist_kernel, bgrid, dim3(256), (size_t)p.m * 4, st, (const int32_t*)(ws + p.ws.E),
                     (uint32_t*)(ws + p.ws.bcount), Ns, p.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(p.BH), dim3(256), 0, st, (const uint32_t*)(ws + p.ws.bcount),
                     (uint32_t*)(ws + p.ws.boff), (int4*)(ws + p.ws.tiles), p.m, p.max_tiles, p.trows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bucket_scatter_kernel, bgrid, dim3(256), (size_t)p.m * 8, st, (const int32_t*)(ws + p.ws.E),
                     (const uint32_t*)(ws + p.ws.boff), (uint32_t*)(ws + p.ws.bcursor), (int32_t*)(ws + p.ws.perm), Ns,
                     p.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return hipSuccess;
}

template <typename T, int D>
static hipError_t gather_launch(const Plan& p, const void* Q, const void* K, const void* V, void* out, char* ws,
                                hipStream_t st) {
  hipError_t e = hipSuccess;
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const void* vtop = p.dtype == MITA_BF16 ? (const void*)(ws + p.ws.vt16) : (const void*)(ws + p.ws.vt32);
  static PerDevice c_f, c_p, c_1;
  const int n_cu = device_cu_count();
  // persistent grid: one resident workgroup per slot, in groups of gs on one XCD,
  // each group walking a contiguous run of the tile table
  const long total = (long)p.max_tiles * p.BH;
  const int slots = n_cu * (p.s == 1 ? resident_per_cu(c_f, gather_kernel<T, D, true>, 256)
                                     : resident_per_cu(c_p, gather_kernel<T, D, false>, 256));
  const int gsz = std::max(1, std::min(8, slots / 8));
  const int grid = std::max(8 * gsz, slots / (8 * gsz) * 8 * gsz);
  const long gchunk = (total + grid / gsz - 1) / (grid / gsz);
  // the one-pass kernel where its double-buffered LDS fits a workgroup
  constexpr bool one_pass_fits = sizeof(Gather1Lds<T, D>) <= 160 * 1024;
  if constexpr (one_pass_fits) if (p.s == 1 && p.k <= kKeyBlock && p.m <= kKeyBlock) {
    // resident workgroups in groups of up to 16 per XCD-slice (a multiple of 8 x gs)
    const int slots = n_cu * resident_per_cu(c_1, gather1_kernel<T, D>, 256);
    const int gs = std::max(1, std::min(8, slots / 8));
    const int g1 = std::max(8 * gs, slots / (8 * gs) * 8 * gs);
    hipLaunchKernelGGL((gather1_kernel<T, D>), dim3(g1), dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const int32_t*)(ws + p.ws.I), (const int4*)(ws + p.ws.tiles), (const int32_t*)(ws + p.ws.perm),
                       (const void*)(ws + p.ws.qtop), vtop, (T*)out, p.N, p.m, p.k, p.max_tiles, p.BH, gs, sl2e,
                       (float*)(ws + p.ws.lse));
    return hipGetLastError();
  }
  if (p.s == 1 && p.m <= kKeyBlock) {
    hipLaunchKernelGGL((gather_kernel<T, D, true>), dim3(grid), dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                       (const int32_t*)(ws + p.ws.I), (const int4*)(ws + p.ws.tiles), (const int32_t*)(ws + p.ws.perm),
                       (const void*)(ws + p.ws.qtop), vtop, (T*)out, (float*)nullptr, (float*)nullptr, p.N, p.m, p.k,
                       p.s, p.max_tiles, total, gchunk, gsz, sl2e, (float*)(ws + p.ws.lse));
    return hipGetLastError();
  }
  // bf16 partials: the direct-load kernel, 1 or 2 column tiles per wave (its buffer
  // offsets within a slice's K / V are 32-bit)
  if (sizeof(T) == 2 && (int64_t)p.N * D * 2 < ((int64_t)1 << 31)) {
    static PerDevice c_q1, c_q2, c_q1f, c_q2f;
    auto go = [&](auto kern, PerDevice& cache) {
      const int sl = n_cu * resident_per_cu(cache, kern, 256);
      const int gq = std::max(1, std::min(8, sl / 8));
      const int gr = std::max(8 * gq, sl / (8 * gq) * 8 * gq);
      const long gc = (total + gr / gq - 1) / (gr / gq);
      hipLaunchKernelGGL(kern, dim3(gr), dim3(256), 0, st, (const uint16_t*)Q, (const uint16_t*)K,
                         (const uint16_t*)V, (const int32_t*)(ws + p.ws.I), (const int4*)(ws + p.ws.tiles),
                         (const int32_t*)(ws + p.ws.perm), (uint16_t*)(ws + p.ws.pacc), (float*)(ws + p.ws.pml), p.N,
                         p.m, p.k, p.s, p.max_tiles, total, gc, gq, sl2e);
    };
    const bool kfull = p.k % kKeyBlock == 0;
    if (p.gqt == 2) {
      if (kfull) go(gatherd_kernel<D, 2, true>, c_q2f); else go(gatherd_kernel<D, 2, false>, c_q2);
    } else {
      if (kfull) go(gatherd_kernel<D, 1, true>, c_q1f); else go(gatherd_kernel<D, 1, false>, c_q1);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gather_kernel<T, D, false>), dim3(grid), dim3(256), 0, st, (const T*)Q, (const T*)K, (const T*)V,
                     (const int32_t*)(ws + p.ws.I), (const int4*)(ws + p.ws.tiles), (const int32_t*)(ws + p.ws.perm),
                     (const void*)(ws + p.ws.qtop), vtop, (T*)out, (void*)(ws + p.ws.pacc), (float*)(ws + p.ws.pml),
                     p.N, p.m, p.k, p.s, p.max_tiles, total, gchunk, gsz, sl2e, (float*)nullptr);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t combine_launch(const Plan& p, const void* Q, void* out, char* ws, hipStream_t st) {
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const void* vtop = p.dtype == MITA_BF16 ? (const void*)(ws + p.ws.vt16) : (const void*)(ws + p.ws.vt32);
  if constexpr (sizeof(T) == 2) {   // bf16: waves of 2 column tiles
    // d = 64: eight waves per workgroup (each landmark block staged once per 256
    // queries; measured 7 % faster on the seg-like inputs, 15-20 % slower for d = 128)
    constexpr int QT = 2, NW = D == 64 ? 8 : kCombineWaves, NB = kCombineBuffers, QPW = 16 * QT * NW;
    const bool mfull = p.m % kKeyBlock == 0;
    auto pick = [&](auto su) {
      constexpr int SU = decltype(su)::value;
      return mfull ? combined_kernel<D, QT, NW, true, SU, NB> : combined_kernel<D, QT, NW, false, SU, NB>;
    };
    auto kern = p.s == 1 ? pick(std::integral_constant<int, 1>{})
              : p.s == 2 ? pick(std::integral_constant<int, 2>{}) : pick(std::integral_constant<int, 4>{});
    hipLaunchKernelGGL(kern, dim3((p.N + QPW - 1) / QPW, p.BH), dim3(64 * NW), 0, st, (const uint16_t*)Q,
                       (const uint16_t*)(ws + p.ws.qtop), (const uint16_t*)vtop, (const uint16_t*)(ws + p.ws.pacc),
                       (const float*)(ws + p.ws.pml), (uint16_t*)out, p.N, p.m, p.s, sl2e, (float*)(ws + p.ws.lse));
    return hipGetLastError();
  }
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(p.qtiles, p.BH), dim3(256), 0, st, (const T*)Q,
                     (const void*)(ws + p.ws.qtop), vtop, (const void*)(ws + p.ws.pacc), (const float*)(ws + p.ws.pml),
                     (T*)out, p.N, p.m, p.s, sl2e, (float*)(ws + p.ws.lse));
  return hipGetLastError();
}

hipError_t launch_gather(const Plan& p, const void* Q, const void* K, const void* V, void* out, char* ws,
                         hipStream_t st) {
  if (p.dtype == MITA_BF16)
    return p.d == 64 ? gather_launch<uint16_t, 64>(p, Q, K, V, out, ws, st) : gather_launch<uint16_t, 128>(p, Q, K, V, out, ws, st);
  return p.d == 64 ? gather_launch<float, 64>(p, Q, K, V, out, ws, st) : gather_launch<float, 128>(p, Q, K, V, out, ws, st);
}

bool has_combine(const Plan& p) { return p.s > 1 || p.m > kKeyBlock; }

hipError_t launch_combine(const Plan& p, const void* Q, void* out, char* ws, hipStream_t st) {
  if (!has_combine(p)) return hipSuccess;   // the gather kernels wrote the output
  if (p.dtype == MITA_BF16)
    return p.d == 64 ? combine_launch<uint16_t, 64>(p, Q, out, ws, st) : combine_launch<uint16_t, 128>(p, Q, out, ws, st);
  return p.d == 64 ? combine_launch<float, 64>(p, Q, out, ws, st) : combine_launch<float, 128>(p, Q, out, ws, st);
}

// Route-step counter block (queued-query count) is cleared before routing; only
// the fast router for m > 64 queues queries.
hipError_t launch_clear(const Plan& p, char* ws, hipStream_t st) {
  if (!(p.s <= kRouteFastMaxS && p.m > kKeyBlock)) return hipSuccess;
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(256), 0, st, (uint32_t*)(ws + p.ws.counters), 64);
  return hipGetLastError();
}

}  // namespace mita
