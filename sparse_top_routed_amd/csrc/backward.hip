// Backward of the MiTA attention forward pass (bf16 inputs): dQ, dK, dV of
// sum(dO * O) with the expert sets I and the routing E held fixed (selections are
// not differentiable). The MiTA pages report training through the operator (Long
// Range Arena training wall-clock: Arabic/Hindi section 4, Dutch "Resultaten")
// but give no backward; this is the chain rule through the forward as defined.
//
// Every part of the forward is softmax attention between a set of queries and a
// set of keys whose normalisers the forward recorded (log2-sum-exp lse, so a
// weight is 2^(c s - lse) with c = log2(e) / sqrt d):
//   routed:   for each expert e, the queries routed to it (its bucket) over the
//             keys/values K[I_e], V[I_e];
//   landmark: every query over the m landmark keys Q~ and values V~ (the shared
//             expert's slots of the final attention);
//   shared:   the m landmarks as queries over all N keys/values (V~ itself), whose
//             output gradient is dV~ (gathered from the landmark part).
// With P the weights, dP = dO V^T, D = rowsum(dO * O) and dS = P (dP - D): dq =
// dS K / sqrt d, dk = dS^T q / sqrt d, dv = P^T dO. Two kernels do this for any
// of the three parts: key-outer (a workgroup owns 64 keys and walks all their
// queries: dK, dV) and query-outer (a workgroup owns a tile of queries and walks
// all their keys: dQ). Then Q~ passes its gradient back through the pooling.
//
// Determinism: no float atomics. Partial sums go to per-part buffers reduced in
// a fixed order; each expert's queries are taken in ascending (query, slot) order
// (a stable re-sort of the routing); a token's routed dK/dV rows are summed over
// the experts that hold it in expert order (an inverse list placed by per-token
// expert bitmaps).
//
// Tiles (64 rows of D bf16) are read two ways: as QK operands (16-byte reads:
// lanes r = 0..15 of 16 consecutive rows, two 16-byte chunks per row per half-wave)
// and transposed (8-byte reads: 8 consecutive rows x 2 neighbouring chunks per
// half-wave). Chunk c of row r sits at chunk c ^ f(r), f(r) = 2 h(r), where h
// is chosen so that neither read meets a bank conflict when a half-wave's 16-byte
// reads are served over 128 four-byte banks (512 bytes) and its 8-byte reads over
// 64 or 128 banks (a single swizzle that is conflict-free over 64 banks,
// 2 (r & 7) | (r >> 3 & 1), measured one conflict cycle per MFMA on the QK reads):
//   D = 128 (a row is 64 banks): h(r) = (r & 7) ^ (r >> 3 & 1), a permutation of
//     0..7 over the even and over the odd rows of 16 (QK) and over 8 aligned rows
//     (transposed);
//   D = 64 (a row is 32 banks): h(r) = ((r >> 2) ^ (r & 2)) & 3, distinct over the
//     four rows r & 3 = c of 16 (QK) and over the four rows of either parity of 8
//     aligned rows (transposed).
#include "attn_core.h"

namespace mita {

template <int D>
struct BT {
  static constexpr int CPR = D / 8, TILE = kKeyBlock * D, RPI = 512 / D;
  __device__ static __forceinline__ int swz(int r) {
    return D == 128 ? 2 * ((r & 7) ^ ((r >> 3) & 1)) : 2 * (((r >> 2) ^ (r & 2)) & 3);
  }
};

// A wave's share (rows w RPW .. + RPW) of a 64-row tile by direct global-to-LDS
// loads; rowp(row) gives the row's source (D contiguous bf16).
template <int D, int NW, typename RowFn>
__device__ __forceinline__ void bdma(uint16_t* tile, RowFn rowp, int w, int lane) {
  using B = BT<D>;
  constexpr int RPW = kKeyBlock / NW, NI = RPW / B::RPI;
  static_assert(NI >= 1, "rows per wave below one load instruction");
  const int p = lane % B::CPR;
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int r0 = w * RPW + u * B::RPI, row = r0 + lane / B::CPR;
    lds_dma16(rowp(row) + 8 * (p ^ B::swz(row)), tile + r0 * D);
  }
}

// Scores of the 64 tile rows (A operand) against 16 register rows (B operand,
// bf[ks] = a row's elements 32 ks + 8 (lane / 16) ..): lane (r, g) gets
// C[tile row 16 kt + 4 g + j][register row r].
template <int D>
__device__ __forceinline__ void bqk(const uint16_t* T, const uint4 (&bf)[D / 32], f32x4 (&acc)[4], int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const uint16_t* col = T + r * D + 8 * ((4 * ks + g) ^ BT<D>::swz(r));   // 16 kt keeps the swizzle
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[kt] = mma_bf16(*(const uint4*)(col + 16 * kt * D), bf[ks], acc[kt]);
  }
}

// o[dt] += T^T p: A operand = the tile transposed (transposed reads), B operand =
// p in the layout bqk leaves (lane (r, g): rows 16 kt + 4 g + j of column r);
// lane (r, g) gets o[column 16 dt + 4 g + j][register row r].
template <int D>
__device__ __forceinline__ void bpt(const uint16_t* T, const f32x4 (&p)[4], f32x4 (&o)[D / 16], int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int row = 4 * g + (i >> 2);   // + 32 h + 16 hi: bits the swizzle does not use
  const int sw = BT<D>::swz(row), b = (i & 3) >> 1;
  const uint16_t* rb = T + row * D + 4 * (i & 1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 bb;
    bb.x = pack_bf16x2(p[2 * h][0], p[2 * h][1]);
    bb.y = pack_bf16x2(p[2 * h][2], p[2 * h][3]);
    bb.z = pack_bf16x2(p[2 * h + 1][0], p[2 * h + 1][1]);
    bb.w = pack_bf16x2(p[2 * h + 1][2], p[2 * h + 1][3]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int ch = 8 * ((2 * dt + b) ^ sw);
      const uint2 lo = lds_read_tr16(rb + (32 * h) * D + ch);
      const uint2 hi = lds_read_tr16(rb + (32 * h + 16) * D + ch);
      o[dt] = mma_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), bb, o[dt]);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_bfrag(uint4 (&f)[D / 32], const uint16_t* row, int g) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) f[ks] = ld16(row + 32 * ks + 8 * g);
}

enum BwdPart { kRouted = 0, kLandmark = 1, kShared = 2 };

struct BwdArgs {
  const uint16_t *Q, *K, *V, *dO;   // [BH, N, D]
  const uint16_t* qt16;             // Q~ planes [BH, 2, m, D] (the hi plane is used)
  const uint16_t* vt16;             // V~ [BH, m, D] bf16
  const uint16_t* dvt16;            // dV~ [BH, m, D] bf16 (from the landmark part)
  const int32_t *I, *perm;
  const int4* tiles;
  const uint32_t* boff;
  const float *lse, *lse_se, *Dq, *Di;
  float *dKe, *dVe;                 // routed: [BH, m, k, D]
  float *lm_dqt, *lm_dvt;           // landmark key-outer parts: [qparts, BH, m, D]
  float *dKs, *dVs;                 // shared: [BH, N, D]
  float* dQp;                       // routed query-outer: [BH, N, s, D]
  float* dQl;                       // landmark query-outer: [BH, N, D]
  float* se_dqt;                    // shared query-outer parts: [kparts, BH, m, D]
  int BH, N, m, k, s, max_tiles, qparts, kparts;
  float c, rsd;                     // log2(e) / sqrt d, 1 / sqrt d
};

__device__ __forceinline__ int part_lo(int n, int parts, int i) { return (int)((long)n * i / parts); }

// ---------------------------------------------------------------- key-outer
// Workgroup = 64 keys (16 per wave, held as B fragments) of one (slice, key
// set); it walks the key set's queries 64 at a time, staged in LDS (rows of Q
// and dO, and their lse and D, all by direct loads; double-buffered), and
// accumulates dK^T += Q^T dS, dV^T += dO^T P for its keys. The source rows of a
// chunk (through the bucket permutation for the routed part) are read one chunk
// ahead, so no load waits inside a chunk; rows past the set's end repeat its last
// query and are masked out of P.
template <int D>
struct KvLds {
  uint16_t qs[2][BT<D>::TILE];
  uint16_t os[2][BT<D>::TILE];
  float ls[2][kKeyBlock], ds[2][kKeyBlock];
};

__device__ __forceinline__ void lds_dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

template <int D, int PART>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_kernel(BwdArgs a) {
  using B = BT<D>;
  constexpr int NI = (kKeyBlock / 4) / B::RPI;   // rows a lane stages per tile
  // one shared object: with separate ones the compiler's LDS scopes would make the
  // next chunk's loads look like writes to the chunk being read
  __shared__ __align__(16) KvLds<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int N = a.N, m = a.m, k = a.k, s = a.s;
  int z, e = 0, kb, nkeys, q0 = 0, nq;
  if constexpr (PART == kRouted) {
    const int kbn = (k + kKeyBlock - 1) / kKeyBlock;
    const int pe = blockIdx.x / kbn;
    z = pe / m;
    e = pe % m;
    kb = (blockIdx.x % kbn) * kKeyBlock;
    nkeys = k;
    const uint32_t* bo = a.boff + (size_t)z * (m + 1);
    q0 = (int)bo[e];
    nq = (int)bo[e + 1] - q0;
  } else if constexpr (PART == kLandmark) {
    const int kbn = (m + kKeyBlock - 1) / kKeyBlock;
    const int qp = blockIdx.x % a.qparts, zk = blockIdx.x / a.qparts;
    z = zk / kbn;
    kb = (zk % kbn) * kKeyBlock;
    nkeys = m;
    q0 = part_lo(N, a.qparts, qp);
    nq = part_lo(N, a.qparts, qp + 1) - q0;
  } else {
    const int kbn = (N + kKeyBlock - 1) / kKeyBlock;
    z = blockIdx.x / kbn;
    kb = (blockIdx.x % kbn) * kKeyBlock;
    nkeys = N;
    nq = m;
  }
  // this lane's key (register row r of the wave) and its K, V rows
  const int key = kb + 16 * w + r, keyc = min(key, nkeys - 1);
  const uint16_t *krow, *vrow;
  if constexpr (PART == kRouted) {
    const int t = a.I[((size_t)z * m + e) * k + keyc];
    krow = a.K + ((size_t)z * N + t) * D;
    vrow = a.V + ((size_t)z * N + t) * D;
  } else if constexpr (PART == kLandmark) {
    krow = a.qt16 + ((size_t)z * 2 * m + keyc) * D;
    vrow = a.vt16 + ((size_t)z * m + keyc) * D;
  } else {
    krow = a.K + ((size_t)z * N + keyc) * D;
    vrow = a.V + ((size_t)z * N + keyc) * D;
  }
  uint4 kf[D / 32], vf[D / 32];
  load_bfrag<D>(kf, krow, g);
  load_bfrag<D>(vf, vrow, g);
  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // row of query t of the set, as read ahead (the bucket entry for the routed
  // part: the division waits for the load, so it is left to the use), and as used
  auto qsrc = [&](int t) {
    const int tc = min(t, max(nq - 1, 0));
    if constexpr (PART == kShared) return tc;
    if constexpr (PART == kRouted) return a.perm[(size_t)z * N * s + q0 + tc];
    return q0 + tc;
  };
  auto qfin = [&](int x) {
    if constexpr (PART == kRouted) return x / s;
    return x;
  };
  // the rows this lane stages of the chunk at c (NI of a tile), and the row whose
  // lse and D it loads (wave 0)
  auto chunk_rows = [&](int c, int (&qi)[NI], int& ql) {
#pragma unroll
    for (int u = 0; u < NI; ++u) qi[u] = qsrc(c + 16 * w + u * B::RPI + lane / B::CPR);
    ql = qsrc(c + lane);
  };
  auto qsrc_row = [&](int x, bool grad) {
    const int q = qfin(x);
    if constexpr (PART == kShared)
      return grad ? a.dvt16 + ((size_t)z * m + q) * D : a.qt16 + ((size_t)z * 2 * m + q) * D;
    else
      return (grad ? a.dO : a.Q) + ((size_t)z * N + q) * D;
  };
  auto stage = [&](const int (&qi)[NI], int ql, uint16_t* qt, uint16_t* ot, float* lsb, float* dsb) {
    const int p = lane % B::CPR;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int r0 = 16 * w + u * B::RPI, row = r0 + lane / B::CPR;
      lds_dma16(qsrc_row(qi[u], false) + 8 * (p ^ B::swz(row)), qt + r0 * D);
      lds_dma16(qsrc_row(qi[u], true) + 8 * (p ^ B::swz(row)), ot + r0 * D);
    }
    if (w == 0) {
      const int q = qfin(ql);
      if constexpr (PART == kShared) {
        lds_dma4(a.lse_se + (size_t)z * m + q, lsb);
        lds_dma4(a.Di + (size_t)z * m + q, dsb);
      } else {
        lds_dma4(a.lse + (size_t)z * N + q, lsb);
        lds_dma4(a.Dq + (size_t)z * N + q, dsb);
      }
    }
  };
  const int nch = (nq + kKeyBlock - 1) / kKeyBlock;
  int qi_n[NI], ql_n;
  if (nch > 0) {
    int qi0[NI], ql0;
    chunk_rows(0, qi0, ql0);
    stage(qi0, ql0, sm.qs[0], sm.os[0], sm.ls[0], sm.ds[0]);
    chunk_rows(kKeyBlock, qi_n, ql_n);
  }
  for (int ci = 0; ci < nch; ++ci) {
    const int c = ci * kKeyBlock;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // chunk ci staged; every wave done with chunk ci - 1
    auto step = [&](uint16_t* __restrict__ nq_t, uint16_t* __restrict__ no_t, float* __restrict__ nls,
                    float* __restrict__ nds, const uint16_t* __restrict__ cq, const uint16_t* __restrict__ co,
                    const float* __restrict__ cls, const float* __restrict__ cds) __attribute__((always_inline)) {
      if (ci + 1 < nch) {   // block-uniform
        stage(qi_n, ql_n, nq_t, no_t, nls, nds);
        chunk_rows(c + 2 * kKeyBlock, qi_n, ql_n);
      }
      f32x4 sc[4], dp[4];
      bqk<D>(cq, kf, sc, lane);   // S[query 16 kt + 4 g + j][key r]
      bqk<D>(co, vf, dp, lane);   // dP[query][key]
      const int lim = nq - c - 4 * g;   // query 16 kt + 4 g + j of the chunk is past the set when 16 kt + j >= lim
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float4 l4 = *(const float4*)(cls + 16 * kt + 4 * g), d4 = *(const float4*)(cds + 16 * kt + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pv = __builtin_amdgcn_exp2f(fmaf(sc[kt][j], a.c, -lv[j]));
          pv = 16 * kt + j < lim ? pv : 0.f;
          sc[kt][j] = pv;
          dp[kt][j] = pv * (dp[kt][j] - dvv[j]);
        }
      }
      bpt<D>(co, sc, dv, lane);   // dV^T += dO^T P
      bpt<D>(cq, dp, dk, lane);   // dK^T += Q^T dS
    };
    const int b = ci & 1, nb = (ci + 1) & 1;
    step(sm.qs[nb], sm.os[nb], sm.ls[nb], sm.ds[nb], sm.qs[b], sm.os[b], sm.ls[b], sm.ds[b]);
  }
  if (key >= nkeys) return;
  float *kd, *vd;
  if constexpr (PART == kRouted) {
    const size_t o = (((size_t)z * m + e) * k + key) * D;
    kd = a.dKe + o;
    vd = a.dVe + o;
  } else if constexpr (PART == kLandmark) {
    const size_t o = (((size_t)(blockIdx.x % a.qparts) * a.BH + z) * m + key) * D;
    kd = a.lm_dqt + o;
    vd = a.lm_dvt + o;
  } else {
    const size_t o = ((size_t)z * N + key) * D;
    kd = a.dKs + o;
    vd = a.dVs + o;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    *(float4*)(kd + 16 * dt + 4 * g) =
        make_float4(dk[dt][0] * a.rsd, dk[dt][1] * a.rsd, dk[dt][2] * a.rsd, dk[dt][3] * a.rsd);
    *(float4*)(vd + 16 * dt + 4 * g) = make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  }
}

// ---------------------------------------------------------------- query-outer
// Workgroup = NW waves of 16 queries (Q and dO rows as B fragments, lse and D per
// lane); it walks the queries' keys 64 at a time (K and V rows staged by direct
// loads, double-buffered; the routed part's token ids read a block ahead) and
// accumulates dQ^T += K^T dS^T.
template <int D>
struct QLds {
  uint16_t kst[2][BT<D>::TILE];
  uint16_t vst[2][BT<D>::TILE];
};

template <int D, int PART, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_q_kernel(BwdArgs a) {
  // one shared object (see bwd_kv_kernel)
  __shared__ __align__(16) QLds<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int N = a.N, m = a.m, k = a.k, s = a.s;
  int z, e = 0, nrows, k0 = 0, nkeys, row0 = 0;
  int4 te = make_int4(0, 0, 0, 0);
  if constexpr (PART == kRouted) {
    z = blockIdx.x / a.max_tiles;
    te = a.tiles[blockIdx.x];
    if (te.x < 0) return;   // workgroup-uniform: an unused table entry
    e = te.x;
    nrows = te.z;
    nkeys = k;
  } else if constexpr (PART == kLandmark) {
    const int qtn = (N + 16 * NW - 1) / (16 * NW);
    z = blockIdx.x / qtn;
    row0 = (blockIdx.x % qtn) * 16 * NW;
    nrows = min(16 * NW, N - row0);
    nkeys = m;
  } else {
    const int ltn = (m + 16 * NW - 1) / (16 * NW);
    const int kp = blockIdx.x % a.kparts, zl = blockIdx.x / a.kparts;
    z = zl / ltn;
    row0 = (zl % ltn) * 16 * NW;
    nrows = min(16 * NW, m - row0);
    k0 = part_lo(N, a.kparts, kp);
    nkeys = part_lo(N, a.kparts, kp + 1) - k0;
  }
  // this lane's query (register row r of the wave)
  const int rw = 16 * w + r, rc = min(rw, nrows - 1);
  int q = 0, slot = 0;
  const uint16_t *qrow, *orow;
  float lq, dq_;
  if constexpr (PART == kShared) {
    q = row0 + rc;   // a landmark
    qrow = a.qt16 + ((size_t)z * 2 * m + q) * D;
    orow = a.dvt16 + ((size_t)z * m + q) * D;
    lq = a.lse_se[(size_t)z * m + q];
    dq_ = a.Di[(size_t)z * m + q];
  } else {
    if constexpr (PART == kRouted) {
      const int ent = a.perm[(size_t)z * N * s + te.w + rc];
      q = ent / s;
      slot = ent % s;
    } else {
      q = row0 + rc;
    }
    qrow = a.Q + ((size_t)z * N + q) * D;
    orow = a.dO + ((size_t)z * N + q) * D;
    lq = a.lse[(size_t)z * N + q];
    dq_ = a.Dq[(size_t)z * N + q];
  }
  uint4 qf[D / 32], of[D / 32];
  load_bfrag<D>(qf, qrow, g);
  load_bfrag<D>(of, orow, g);
  f32x4 dq[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // key t of the set (clamped to the last), as read ahead (a token id for the
  // routed part), and the K or V row it names
  using B = BT<D>;
  constexpr int RPW = kKeyBlock / NW, NI = RPW / B::RPI;   // rows a wave, and a lane, stage per tile
  auto ksrc = [&](int t) {
    const int tc = min(t, nkeys - 1);
    if constexpr (PART == kRouted) return (int)a.I[((size_t)z * m + e) * k + tc];
    else if constexpr (PART == kLandmark) return tc;
    else return k0 + tc;
  };
  auto krow = [&](int x, bool val) {
    if constexpr (PART == kLandmark)
      return val ? a.vt16 + ((size_t)z * m + x) * D : a.qt16 + ((size_t)z * 2 * m + x) * D;
    else
      return (val ? a.V : a.K) + ((size_t)z * N + x) * D;
  };
  auto block_rows = [&](int kb, int (&ti)[NI]) {
#pragma unroll
    for (int u = 0; u < NI; ++u) ti[u] = ksrc(kb + w * RPW + u * B::RPI + lane / B::CPR);
  };
  auto stage = [&](const int (&ti)[NI], uint16_t* kt_, uint16_t* vt_) {
    const int p = lane % B::CPR;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int r0 = w * RPW + u * B::RPI, row = r0 + lane / B::CPR;
      lds_dma16(krow(ti[u], false) + 8 * (p ^ B::swz(row)), kt_ + r0 * D);
      lds_dma16(krow(ti[u], true) + 8 * (p ^ B::swz(row)), vt_ + r0 * D);
    }
  };
  const int nb = (nkeys + kKeyBlock - 1) / kKeyBlock;
  const bool live = 16 * w < nrows;   // wave-uniform
  int ti_n[NI];
  {
    int ti0[NI];
    block_rows(0, ti0);
    stage(ti0, sm.kst[0], sm.vst[0]);
    block_rows(kKeyBlock, ti_n);
  }
  for (int bi = 0; bi < nb; ++bi) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&](uint16_t* __restrict__ nk, uint16_t* __restrict__ nv, const uint16_t* __restrict__ ck,
                    const uint16_t* __restrict__ cv) __attribute__((always_inline)) {
      if (bi + 1 < nb) {   // block-uniform: the next block's rows, the one after's ids
        stage(ti_n, nk, nv);
        block_rows((bi + 2) * kKeyBlock, ti_n);
      }
      if (!live) return;
      f32x4 sc[4], dp[4];
      bqk<D>(ck, qf, sc, lane);   // S^T[key 16 kt + 4 g + j][query r]
      bqk<D>(cv, of, dp, lane);   // dP^T
      const int livek = nkeys - bi * kKeyBlock;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = 16 * kt + 4 * g + j < livek ? __builtin_amdgcn_exp2f(fmaf(sc[kt][j], a.c, -lq)) : 0.f;
          dp[kt][j] = p * (dp[kt][j] - dq_);
        }
      bpt<D>(ck, dp, dq, lane);   // dQ^T += K^T dS^T
    };
    step(sm.kst[(bi + 1) & 1], sm.vst[(bi + 1) & 1], sm.kst[bi & 1], sm.vst[bi & 1]);
  }
  if (rw >= nrows) return;
  float* dst;
  if constexpr (PART == kRouted) dst = a.dQp + (((size_t)z * N + q) * s + slot) * D;
  else if constexpr (PART == kLandmark) dst = a.dQl + ((size_t)z * N + q) * D;
  else dst = a.se_dqt + (((size_t)(blockIdx.x % a.kparts) * a.BH + z) * m + q) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *(float4*)(dst + 16 * dt + 4 * g) =
        make_float4(dq[dt][0] * a.rsd, dq[dt][1] * a.rsd, dq[dt][2] * a.rsd, dq[dt][3] * a.rsd);
}

// ---------------------------------------------------------------- small kernels
__global__ __launch_bounds__(256) void bwd_clear_kernel(uint32_t* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0u;
}

// out[row] = sum_d x[row][d] y[row][d] (16 lanes per row, fp32 sums in a fixed order).
template <int D, typename TX, typename TY>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const TX* __restrict__ x, const TY* __restrict__ y,
                                                         float* __restrict__ out, long rows) {
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      const int d = c * (D / 16) + e;
      float xv, yv;
      if constexpr (sizeof(TX) == 2) xv = bf16_to_f32(x[row * D + d]); else xv = x[row * D + d];
      if constexpr (sizeof(TY) == 2) yv = bf16_to_f32(y[row * D + d]); else yv = y[row * D + d];
      acc = fmaf(xv, yv, acc);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
  if (row < rows && c == 0) out[row] = acc;
}

// Landmark part reduced over its query parts: dQ~ (into dqt), dV~ (fp32 and bf16).
__global__ __launch_bounds__(256) void bwd_lm_reduce_kernel(const float* __restrict__ lm_dqt,
                                                            const float* __restrict__ lm_dvt, int parts, long n,
                                                            float* __restrict__ dqt, float* __restrict__ dvt,
                                                            uint16_t* __restrict__ dvt16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float a = 0.f, b = 0.f;
    for (int p = 0; p < parts; ++p) {
      a += lm_dqt[(size_t)p * n + i];
      b += lm_dvt[(size_t)p * n + i];
    }
    dqt[i] = a;
    dvt[i] = b;
    dvt16[i] = f32_to_bf16(b);
  }
}

// dqt += the shared part's query-outer parts, in part order.
__global__ __launch_bounds__(256) void bwd_se_reduce_kernel(const float* __restrict__ se_dqt, int parts, long n,
                                                            float* __restrict__ dqt) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float a = 0.f;
    for (int p = 0; p < parts; ++p) a += se_dqt[(size_t)p * n + i];
    dqt[i] += a;
  }
}

// The routed key-outer kernel sums each expert's queries in bucket order, and
// the forward fills its buckets with atomics (any order: it computes every query
// on its own). For sums in a fixed order the backward re-sorts the routing with a
// stable counting sort: within each bucket, (query * s + slot) ascending, at the
// forward's bucket offsets. Chunks of kPermChunk entries, a quarter per wave.
constexpr int kPermChunk = 4096;

// Entries of each expert per chunk (integer counts: order-free).
__global__ __launch_bounds__(256) void bwd_perm_count_kernel(const int32_t* __restrict__ E, uint32_t* __restrict__ cb,
                                                             int Ns, int m, int nch) {
  extern __shared__ uint32_t h[];   // [m]
  const int c = blockIdx.x, z = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < m; i += 256) h[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  for (int j = tid; j < kPermChunk; j += 256) {
    const int e = c * kPermChunk + j;
    const int x = e < Ns ? Ez[e] : -1;
    if ((unsigned)x < (unsigned)m) atomicAdd(&h[x], 1u);
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256) cb[((size_t)z * nch + c) * m + i] = h[i];
}

// Per (slice, expert): the chunk counts become the chunk's first position in the
// bucket (the bucket offset plus the counts of the chunks before it).
__global__ __launch_bounds__(256) void bwd_perm_scan_kernel(const uint32_t* __restrict__ boff,
                                                            uint32_t* __restrict__ cb, int m, int nch, long n) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const long z = t / m;
  const int e = (int)(t - z * m);
  uint32_t run = boff[z * (m + 1) + e];
  uint32_t* col = cb + (size_t)z * nch * m + e;
  for (int c0 = 0; c0 < nch; c0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + u < nch ? col[(size_t)(c0 + u) * m] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < nch) {
        col[(size_t)(c0 + u) * m] = run;
        run += v[u];
      }
  }
}

// Scatter in entry order: each wave takes its quarter of the chunk 64 entries at
// a time; lanes with the same expert get consecutive positions in lane order
// (one ballot per distinct expert), after every earlier entry of that expert.
__global__ __launch_bounds__(256) void bwd_perm_fill_kernel(const int32_t* __restrict__ E,
                                                            const uint32_t* __restrict__ cb,
                                                            int32_t* __restrict__ perm, int Ns, int m, int nch) {
  extern __shared__ uint32_t cw[];   // [4][m]: per-wave counts, then per-wave cursors
  const int c = blockIdx.x, z = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  constexpr int kSteps = kPermChunk / 256;
  for (int i = tid; i < 4 * m; i += 256) cw[i] = 0;
  __syncthreads();
  const int32_t* Ez = E + (size_t)z * Ns;
  const int w0 = c * kPermChunk + w * (kPermChunk / 4);
  int ex[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int e = w0 + 64 * u + lane;
    ex[u] = e < Ns ? Ez[e] : -1;
    if ((unsigned)ex[u] >= (unsigned)m) ex[u] = -1;
    if (ex[u] >= 0) atomicAdd(&cw[w * m + ex[u]], 1u);
  }
  __syncthreads();
  for (int i = tid; i < m; i += 256) {
    uint32_t run = cb[((size_t)z * nch + c) * m + i];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t t = cw[v * m + i];
      cw[v * m + i] = run;
      run += t;
    }
  }
  __syncthreads();
  int32_t* pz = perm + (size_t)z * Ns;
  uint32_t* cur = cw + w * m;
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int x = ex[u];
    uint64_t todo = __ballot(x >= 0);
    while (todo) {
      const int key = __builtin_amdgcn_readlane(x, __builtin_ctzll(todo));
      const uint64_t same = __ballot(x == key);
      const uint32_t b = cur[key];
      if (x == key) {
        const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
        pz[b + r] = w0 + 64 * u + lane;
      }
      if (lane == 0) cur[key] = b + (uint32_t)__popcll(same);
      todo &= ~same;
    }
  }
}

// Inverse lists of the expert sets: per token, the (expert, slot) entries of the
// experts that hold it, in expert order. Each token gets a bitmap of the experts
// holding it (atomic OR: order-free); its count is the bitmap's popcount, its list
// offset an exclusive scan of the counts (per block of kInvBlock tokens, then over
// the blocks of a slice), and an entry's place in the list the popcount of the
// token's bits below its expert: every step is parallel and the order is fixed.
constexpr int kInvBlock = 1024;   // tokens per scan block (256 threads x 4)

__global__ __launch_bounds__(256) void bwd_inv_mark_kernel(const int32_t* __restrict__ I,
                                                           uint32_t* __restrict__ bits, int N, int m, int k, int W,
                                                           long total) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long z = i / ((long)m * k);
    const int e = (int)((i / k) % m);
    atomicOr(&bits[((size_t)z * N + I[i]) * W + (e >> 5)], 1u << (e & 31));   // integer OR: order-free
  }
}

// Counts, and their exclusive scan within each block of kInvBlock tokens (off);
// the block totals go to bsum [BH, nb].
__global__ __launch_bounds__(256) void bwd_inv_count_kernel(const uint32_t* __restrict__ bits,
                                                            uint32_t* __restrict__ cnt, uint32_t* __restrict__ off,
                                                            uint32_t* __restrict__ bsum, int N, int W, int nb) {
  __shared__ uint32_t wtot[4];
  const int b = blockIdx.x, z = blockIdx.y, tid = threadIdx.x;
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = b * kInvBlock + 4 * tid + u;
    c[u] = 0;
    if (t < N) {
      const uint32_t* bt = bits + ((size_t)z * N + t) * W;
      for (int w = 0; w < W; ++w) c[u] += __popc(bt[w]);
    }
    sum += c[u];
  }
  uint32_t tot;
  uint32_t run = block_incl_scan(sum, wtot, tot) - sum;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = b * kInvBlock + 4 * tid + u;
    if (t < N) {
      cnt[(size_t)z * N + t] = c[u];
      off[(size_t)z * N + t] = run;
    }
    run += c[u];
  }
  if (tid == 0) bsum[(size_t)z * nb + b] = tot;
}

// Exclusive scan of each slice's block totals (one workgroup per slice), then
// added to the offsets of the block's tokens by bwd_inv_offset_kernel.
__global__ __launch_bounds__(256) void bwd_inv_bscan_kernel(uint32_t* __restrict__ bsum, int nb) {
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t carry;
  const int z = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < nb; b0 += 256) {
    const int b = b0 + tid;
    const uint32_t v = b < nb ? bsum[(size_t)z * nb + b] : 0u;
    uint32_t tot;
    const uint32_t ex = block_incl_scan(v, wtot, tot) - v + carry;
    if (b < nb) bsum[(size_t)z * nb + b] = ex;
    __syncthreads();
    if (tid == 0) carry += tot;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void bwd_inv_offset_kernel(uint32_t* __restrict__ off,
                                                             const uint32_t* __restrict__ bsum, int N, int nb,
                                                             long total) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long z = i / N;
    off[i] += bsum[z * nb + (i - z * N) / kInvBlock];
  }
}

// Each (expert, slot) entry written at its token's offset plus the number of
// experts below it that hold the token.
__global__ __launch_bounds__(256) void bwd_inv_fill_kernel(const int32_t* __restrict__ I,
                                                           const uint32_t* __restrict__ bits,
                                                           const uint32_t* __restrict__ off,
                                                           uint32_t* __restrict__ list, int N, int m, int k, int W,
                                                           long total) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long z = i / ((long)m * k);
    const int ej = (int)(i - z * (long)m * k), e = ej / k;
    const int t = I[i];
    const uint32_t* bt = bits + ((size_t)z * N + t) * W;
    uint32_t r = __popc(bt[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int w = 0; w < (e >> 5); ++w) r += __popc(bt[w]);
    list[(size_t)z * m * k + off[(size_t)z * N + t] + r] = (uint32_t)ej;
  }
}

// dK, dV of each token: the shared part's rows plus the routed rows of every
// expert holding it, in expert order (16 lanes per token).
template <int D>
__global__ __launch_bounds__(256) void bwd_final_kv_kernel(const float* __restrict__ dKs, const float* __restrict__ dVs,
                                                           const float* __restrict__ dKe, const float* __restrict__ dVe,
                                                           const uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ off,
                                                           const uint32_t* __restrict__ list, float* __restrict__ dK,
                                                           float* __restrict__ dV, int N, int mk, long rows) {
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int c = threadIdx.x & 15;
  constexpr int E = D / 16;   // elements per lane
  const long z = row / N;
  float ak[E], av[E];
#pragma unroll
  for (int u = 0; u < E; ++u) {
    ak[u] = dKs[row * D + c * E + u];
    av[u] = dVs[row * D + c * E + u];
  }
  const uint32_t n = cnt[row], o = off[row];
  const uint32_t* lz = list + (size_t)z * mk;
  for (uint32_t t = 0; t < n; ++t) {
    const size_t src = ((size_t)z * mk + min(lz[o + t], (uint32_t)mk - 1u)) * D + c * E;   // entries < m k
#pragma unroll
    for (int u = 0; u < E; ++u) {
      ak[u] += dKe[src + u];
      av[u] += dVe[src + u];
    }
  }
#pragma unroll
  for (int u = 0; u < E; ++u) {
    dK[row * D + c * E + u] = ak[u];
    dV[row * D + c * E + u] = av[u];
  }
}

// dQ of each token: its routed slots in slot order, its landmark part, then dQ~
// of every pooling window holding it divided by the window size (windows
// [floor(i L / M), ceil((i + 1) L / M)) per axis, taken in ascending order).
template <int D>
__global__ __launch_bounds__(256) void bwd_final_q_kernel(const float* __restrict__ dQp, const float* __restrict__ dQl,
                                                          const float* __restrict__ dqt, float* __restrict__ dQ, int N,
                                                          int s, int m, int gh, int gw, int ph, int pw, long rows) {
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int c = threadIdx.x & 15;
  constexpr int E = D / 16;
  const long z = row / N;
  const int n = (int)(row % N), ar = n / gw, ac = n % gw;
  float acc[E];
#pragma unroll
  for (int u = 0; u < E; ++u) acc[u] = 0.f;
  for (int sl = 0; sl < s; ++sl)
#pragma unroll
    for (int u = 0; u < E; ++u) acc[u] += dQp[((size_t)row * s + sl) * D + c * E + u];
#pragma unroll
  for (int u = 0; u < E; ++u) acc[u] += dQl[(size_t)row * D + c * E + u];
  // candidate windows along each axis: the one at floor(p M / L) and its neighbours
  auto win = [](long i, long L, long M, long& lo, long& hi) {
    lo = (i * L) / M;
    hi = ((i + 1) * L + M - 1) / M;
  };
  const long ir = (long)ar * ph / gh, ic = (long)ac * pw / gw;
  for (long i = max(0L, ir - 1); i <= min((long)ph - 1, ir + 1); ++i) {
    long r0, r1;
    win(i, gh, ph, r0, r1);
    if (ar < r0 || ar >= r1) continue;
    for (long j = max(0L, ic - 1); j <= min((long)pw - 1, ic + 1); ++j) {
      long c0, c1;
      win(j, gw, pw, c0, c1);
      if (ac < c0 || ac >= c1) continue;
      const float inv = 1.f / (float)((r1 - r0) * (c1 - c0));
      const float* src = dqt + ((size_t)z * m + i * pw + j) * D + c * E;
#pragma unroll
      for (int u = 0; u < E; ++u) acc[u] += src[u] * inv;
    }
  }
#pragma unroll
  for (int u = 0; u < E; ++u) dQ[(size_t)row * D + c * E + u] = acc[u];
}

// ---------------------------------------------------------------- host side
static int parts_for(long base, long target, long cap) {
  long p = (target + base - 1) / base;
  return (int)std::max(1L, std::min(p, cap));
}

void backward_plan(const Plan& p, BwdLayout* L) {
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = (off + bytes + 255) & ~(size_t)255; return o; };
  const size_t bh = p.BH, N = p.N, m = p.m, k = p.k, s = p.s, d = p.d;
  L->qparts = parts_for((long)p.BH * ((p.m + kKeyBlock - 1) / kKeyBlock), 1024, (p.N + kKeyBlock - 1) / kKeyBlock);
  L->kparts = parts_for((long)p.BH * ((p.m + kKeyBlock - 1) / kKeyBlock), 1024, (p.N + kKeyBlock - 1) / kKeyBlock);
  L->Dq = take(bh * N * 4);
  L->Di = take(bh * m * 4);
  L->dvt = take(bh * m * d * 4);
  L->dvt16 = take(bh * m * d * 2);
  L->dqt = take(bh * m * d * 4);
  L->lm_dqt = take((size_t)L->qparts * bh * m * d * 4);
  L->lm_dvt = take((size_t)L->qparts * bh * m * d * 4);
  L->se_dqt = take((size_t)L->kparts * bh * m * d * 4);
  L->dQp = take(bh * N * s * d * 4);
  L->dQl = take(bh * N * d * 4);
  L->dKe = take(bh * m * k * d * 4);
  L->dVe = take(bh * m * k * d * 4);
  L->dKs = take(bh * N * d * 4);
  L->dVs = take(bh * N * d * 4);
  L->iw = (p.m + 31) / 32;
  L->inb = (int)((N + kInvBlock - 1) / kInvBlock);
  L->icnt = take(bh * N * 4);
  L->ibits = take(bh * N * (size_t)L->iw * 4);
  L->ioff = take(bh * N * 4);
  L->ibsum = take(bh * (size_t)L->inb * 4);
  L->ilist = take(bh * m * k * 4);
  L->pnch = (int)((N * s + kPermChunk - 1) / kPermChunk);
  L->psort = take(bh * N * s * 4);
  L->pbase = take(bh * (size_t)L->pnch * m * 4);
  L->total = off;
}

template <int D>
static hipError_t backward_launch(const Plan& p, const BwdLayout& L, const void* Q, const void* K, const void* V,
                                  const void* O, const void* dO, float* dQ, float* dK, float* dV, const char* fws,
                                  char* bws, hipStream_t st) {
  BwdArgs a{};
  a.Q = (const uint16_t*)Q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.dO = (const uint16_t*)dO;
  a.qt16 = (const uint16_t*)(fws + p.ws.qtop);
  a.vt16 = (const uint16_t*)(fws + p.ws.vt16);
  a.dvt16 = (const uint16_t*)(bws + L.dvt16);
  a.I = (const int32_t*)(fws + p.ws.I);
  a.perm = (const int32_t*)(bws + L.psort);
  a.tiles = (const int4*)(fws + p.ws.tiles);
  a.boff = (const uint32_t*)(fws + p.ws.boff);
  a.lse = (const float*)(fws + p.ws.lse);
  a.lse_se = (const float*)(fws + p.ws.lse_se);
  a.Dq = (const float*)(bws + L.Dq);
  a.Di = (const float*)(bws + L.Di);
  a.dKe = (float*)(bws + L.dKe);
  a.dVe = (float*)(bws + L.dVe);
  a.lm_dqt = (float*)(bws + L.lm_dqt);
  a.lm_dvt = (float*)(bws + L.lm_dvt);
  a.dKs = (float*)(bws + L.dKs);
  a.dVs = (float*)(bws + L.dVs);
  a.dQp = (float*)(bws + L.dQp);
  a.dQl = (float*)(bws + L.dQl);
  a.se_dqt = (float*)(bws + L.se_dqt);
  a.BH = p.BH; a.N = p.N; a.m = p.m; a.k = p.k; a.s = p.s; a.max_tiles = p.max_tiles;
  a.qparts = L.qparts; a.kparts = L.kparts;
  a.c = (float)(1.4426950408889634 / sqrt((double)D));
  a.rsd = (float)(1.0 / sqrt((double)D));
  const long BH = p.BH, N = p.N, m = p.m, k = p.k;
  hipError_t e;
#define MITA_CHECK_LAUNCH() do { if ((e = hipGetLastError()) != hipSuccess) return e; } while (0)
  // D_q = dO . O
  hipLaunchKernelGGL((bwd_rowdot_kernel<D, uint16_t, uint16_t>), dim3((unsigned)((BH * N + 15) / 16)), dim3(256), 0,
                     st, (const uint16_t*)dO, (const uint16_t*)O, (float*)(bws + L.Dq), BH * N);
  MITA_CHECK_LAUNCH();
  // the routing re-sorted in a fixed order
  {
    const dim3 grid((unsigned)L.pnch, (unsigned)BH);
    const int Ns = p.N * p.s;
    hipLaunchKernelGGL(bwd_perm_count_kernel, grid, dim3(256), (size_t)p.m * 4, st, (const int32_t*)(fws + p.ws.E),
                       (uint32_t*)(bws + L.pbase), Ns, p.m, L.pnch);
    MITA_CHECK_LAUNCH();
    hipLaunchKernelGGL(bwd_perm_scan_kernel, dim3((unsigned)((BH * m + 255) / 256)), dim3(256), 0, st,
                       (const uint32_t*)(fws + p.ws.boff), (uint32_t*)(bws + L.pbase), p.m, L.pnch, BH * m);
    MITA_CHECK_LAUNCH();
    hipLaunchKernelGGL(bwd_perm_fill_kernel, grid, dim3(256), (size_t)p.m * 16, st, (const int32_t*)(fws + p.ws.E),
                       (const uint32_t*)(bws + L.pbase), (int32_t*)(bws + L.psort), Ns, p.m, L.pnch);
    MITA_CHECK_LAUNCH();
  }
  // routed part: dQ per (query, slot); dK, dV per (expert, slot of its list)
  if (p.trows == 128)
    hipLaunchKernelGGL((bwd_q_kernel<D, kRouted, 8>), dim3((unsigned)(BH * p.max_tiles)), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_q_kernel<D, kRouted, 4>), dim3((unsigned)(BH * p.max_tiles)), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  const long kbn = (k + kKeyBlock - 1) / kKeyBlock, mbn = (m + kKeyBlock - 1) / kKeyBlock;
  hipLaunchKernelGGL((bwd_kv_kernel<D, kRouted>), dim3((unsigned)(BH * m * kbn)), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  // landmark part of the final attention: dQ per query; dQ~, dV~ per landmark (query parts, then reduced)
  hipLaunchKernelGGL((bwd_q_kernel<D, kLandmark, 4>), dim3((unsigned)(BH * ((N + 63) / 64))), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL((bwd_kv_kernel<D, kLandmark>), dim3((unsigned)(BH * mbn * L.qparts)), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  const long nmd = BH * m * D;
  hipLaunchKernelGGL(bwd_lm_reduce_kernel, dim3((unsigned)std::min<long>(4096, (nmd + 255) / 256)), dim3(256), 0, st,
                     (const float*)(bws + L.lm_dqt), (const float*)(bws + L.lm_dvt), L.qparts, nmd,
                     (float*)(bws + L.dqt), (float*)(bws + L.dvt), (uint16_t*)(bws + L.dvt16));
  MITA_CHECK_LAUNCH();
  // D_i = dV~ . V~
  hipLaunchKernelGGL((bwd_rowdot_kernel<D, float, float>), dim3((unsigned)((BH * m + 15) / 16)), dim3(256), 0, st,
                     (const float*)(bws + L.dvt), (const float*)(fws + p.ws.vt32), (float*)(bws + L.Di), BH * m);
  MITA_CHECK_LAUNCH();
  // shared expert: dK, dV per token; dQ~ per landmark (key parts, then added to dQ~)
  hipLaunchKernelGGL((bwd_kv_kernel<D, kShared>), dim3((unsigned)(BH * ((N + 63) / 64))), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL((bwd_q_kernel<D, kShared, 4>), dim3((unsigned)(BH * mbn * L.kparts)), dim3(256), 0, st, a);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_se_reduce_kernel, dim3((unsigned)std::min<long>(4096, (nmd + 255) / 256)), dim3(256), 0, st,
                     (const float*)(bws + L.se_dqt), L.kparts, nmd, (float*)(bws + L.dqt));
  MITA_CHECK_LAUNCH();
  // inverse lists of the expert sets, then dK, dV and dQ assembled
  const long nN = BH * N, nmk = BH * m * k, nbits = nN * L.iw;
  hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)std::min<long>(4096, (nbits + 255) / 256)), dim3(256), 0, st,
                     (uint32_t*)(bws + L.ibits), nbits);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_inv_mark_kernel, dim3((unsigned)std::min<long>(8192, (nmk + 255) / 256)), dim3(256), 0, st,
                     (const int32_t*)(fws + p.ws.I), (uint32_t*)(bws + L.ibits), p.N, p.m, p.k, L.iw, nmk);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_inv_count_kernel, dim3((unsigned)L.inb, (unsigned)BH), dim3(256), 0, st,
                     (const uint32_t*)(bws + L.ibits), (uint32_t*)(bws + L.icnt), (uint32_t*)(bws + L.ioff),
                     (uint32_t*)(bws + L.ibsum), p.N, L.iw, L.inb);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_inv_bscan_kernel, dim3((unsigned)BH), dim3(256), 0, st, (uint32_t*)(bws + L.ibsum), L.inb);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_inv_offset_kernel, dim3((unsigned)std::min<long>(4096, (nN + 255) / 256)), dim3(256), 0, st,
                     (uint32_t*)(bws + L.ioff), (const uint32_t*)(bws + L.ibsum), p.N, L.inb, nN);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_inv_fill_kernel, dim3((unsigned)std::min<long>(8192, (nmk + 255) / 256)), dim3(256), 0, st,
                     (const int32_t*)(fws + p.ws.I), (const uint32_t*)(bws + L.ibits), (const uint32_t*)(bws + L.ioff),
                     (uint32_t*)(bws + L.ilist), p.N, p.m, p.k, L.iw, nmk);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL((bwd_final_kv_kernel<D>), dim3((unsigned)((nN + 15) / 16)), dim3(256), 0, st,
                     (const float*)(bws + L.dKs), (const float*)(bws + L.dVs), (const float*)(bws + L.dKe),
                     (const float*)(bws + L.dVe), (const uint32_t*)(bws + L.icnt), (const uint32_t*)(bws + L.ioff),
                     (const uint32_t*)(bws + L.ilist), dK, dV, p.N, p.m * p.k, nN);
  MITA_CHECK_LAUNCH();
  hipLaunchKernelGGL((bwd_final_q_kernel<D>), dim3((unsigned)((nN + 15) / 16)), dim3(256), 0, st,
                     (const float*)(bws + L.dQp), (const float*)(bws + L.dQl), (const float*)(bws + L.dqt), dQ, p.N,
                     p.s, p.m, p.grid_h, p.grid_w, p.pool_h, p.pool_w, nN);
  MITA_CHECK_LAUNCH();
#undef MITA_CHECK_LAUNCH
  return hipSuccess;
}

hipError_t launch_backward(const Plan& p, const BwdLayout& L, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, float* dQ, float* dK, float* dV, const char* fws, char* bws,
                           hipStream_t st) {
  return p.d == 64 ? backward_launch<64>(p, L, Q, K, V, O, dO, dQ, dK, dV, fws, bws, st)
                   : backward_launch<128>(p, L, Q, K, V, O, dO, dQ, dK, dV, fws, bws, st);
}

}  // namespace mita
