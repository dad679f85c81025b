// Host-side plan of one MiTA forward call: validated sizes, launch shapes and the
// carving of the caller's workspace into the intermediates of the five steps.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mita.h"

namespace mita {

constexpr int kMaxLandmarks = 4096;
constexpr int kLandmarkTile = 64;     // landmarks per workgroup in the shared-expert kernel
constexpr int kKeyBlock = 64;         // keys per LDS block in the attention kernels
constexpr int kQueryTile = 64;        // queries per workgroup in the router, gather and combine kernels
constexpr int kTopkMaxGroups = 4096;  // group maxima per score row that the threshold kernel ranks
constexpr int kTopkMaxCap = 4096;     // candidates per row the select kernel holds (larger k: exact fallback)
constexpr int kTopkGeneralWaves = 64; // fewest waves (each with an fp64 score row of scratch) of the fallback kernel
constexpr int kTopkGeneralWavesMax = 4096;
constexpr int kBucketSlicePer = 16;   // pairs per thread of the one-workgroup counting sort (slices of <= 4096 pairs)
constexpr int kRouteFastMaxS = 6;     // the router keeps per-lane top lists up to this s

// Workspace offsets (bytes) of every intermediate buffer.
struct Layout {
  size_t qt64;      // f64 [BH, m, d]     landmark queries
  size_t qtop;      // bf16 [BH, 2, m, d] hi/lo split of Q~ (bf16 path) or f32 [BH, m, d]
  size_t qtnorm;    // f32 [BH, m]        upper bound of |q~_i|_2
  size_t lpart;     // f32 [BH, m, nsplit, d + 4]  per-chunk (max, sum, pad, pad, acc) of the shared expert
  size_t kmax;      // f32 [BH, nsplit]   upper bound of max_n |K_n|_2 per key chunk
  size_t vt32;      // f32 [BH, m, d]     shared expert V~
  size_t vt16;      // bf16 [BH, m, d]    V~ rounded to bf16 (MFMA operand)
  size_t bmax;      // f32 [BH * m, nbg]  maxima of groups of 4, 16 or 64 approximate scores q~_i . K_n
  size_t thr;       // u32 [BH * m]       order key of the candidate threshold of each score row
  size_t cand;      // u32x2 [BH * m, nsplit, capc] candidates (order key, token id) per key chunk
  size_t ccnt;      // u32 [BH * m, nsplit] candidates per chunk (capc + 1: overflow)
  size_t glist;     // u32 [BH * m + 1]   rows for the exact fallback, count first
  size_t gscr;      // f64 [gwaves, N] fp64 score rows of the fallback
  size_t I;         // i32 [BH, m, k]     expert token sets, ascending
  size_t E;         // i32 [BH, N, s]     routed experts per query
  size_t counters;  // u32 block cleared at the start of routing (below)
  size_t rflag;     // u32 [BH * N]       queries whose routing needs the exact fp64 pass
  size_t bcount;    // u32 [BH, m]        queries routed to each expert
  size_t bcursor;   // u32 [BH, m]        scatter cursors
  size_t boff;      // u32 [BH, m + 1]    bucket offsets
  size_t tiles;     // int4 [BH, max_tiles] query tiles: (expert, first row, rows, perm offset) or -1
  size_t perm;      // i32 [BH, N * s]    (query * s + slot) grouped by expert
  size_t pacc;      // [BH, N, s, d] per-slot outputs o / (sum * scale): fp16 (bf16 inputs) or f32
  size_t pml;       // f32 [BH, N, s, 4] per-slot (max, sum, scale, pad)
  size_t lse;       // f32 [BH, N]        log2-sum-exp of each query's final softmax (for the backward)
  size_t lse_se;    // f32 [BH, m]        log2-sum-exp of each landmark's shared-expert softmax
  size_t total;
  size_t counters_bytes;
};

struct Plan {
  int B, H, N, d, m, k, s;
  int grid_h, grid_w, pool_h, pool_w;
  int dtype;        // mita_dtype
  int esize;        // bytes per input element
  int BH;
  // shared-expert kernel
  int lm_tiles;     // ceil(m / kLandmarkTile)
  int lchunk;       // keys per workgroup (multiple of kKeyBlock)
  int nsplit;       // ceil(N / lchunk)
  // top-k select
  int gq;           // scores per group maximum: 4 (a lane's share of one 16-key tile), 16 (its share of a key block) or 64 (a block)
  int nbg;          // group maxima per row: ceil(N / 64) * 64 / gq
  int cap;          // candidates per row the select kernel holds (multiple of 64, or 0: fallback for all rows)
  int gwaves;       // waves of the fallback kernel (64 .. 4096, ~64 MiB of score rows)
  int capc;         // candidate slots per (row, key chunk): min(lchunk, cap)
  // router and output
  int qtiles;       // ceil(N / kQueryTile)
  int gqt;          // 16-query column tiles per wave of the routed-expert kernel (1 or 2)
  int trows;        // rows (queries) per tile of the bucket tile table: 64 gqt
  int max_tiles;    // upper bound of query tiles over all buckets of one slice
  double gamma_qk;  // relative error bound of an approximate score, in units of |q~| |k|
  Layout ws;
};

// Backward workspace: offsets (bytes) of its buffers, and the parts that split
// the landmark part's queries and the shared part's keys for parallelism.
struct BwdLayout {
  int qparts, kparts;
  int pnch;         // chunks of the routing re-sort: ceil(N s / 4096)
  size_t Dq;        // f32 [BH, N]          rowsum(dO * O)
  size_t Di;        // f32 [BH, m]          rowsum(dV~ * V~)
  size_t dvt;       // f32 [BH, m, d]       dV~
  size_t dvt16;     // bf16 [BH, m, d]      dV~ (MFMA operand)
  size_t dqt;       // f32 [BH, m, d]       dQ~ (landmark and shared parts)
  size_t lm_dqt;    // f32 [qparts, BH, m, d]
  size_t lm_dvt;    // f32 [qparts, BH, m, d]
  size_t se_dqt;    // f32 [kparts, BH, m, d]
  size_t dQp;       // f32 [BH, N, s, d]    routed dQ per (query, slot)
  size_t dQl;       // f32 [BH, N, d]       landmark-part dQ
  size_t dKe;       // f32 [BH, m, k, d]    routed dK per (expert, list slot)
  size_t dVe;       // f32 [BH, m, k, d]
  size_t dKs;       // f32 [BH, N, d]       shared-part dK
  size_t dVs;       // f32 [BH, N, d]
  int iw;           // words of a token's expert bitmap: ceil(m / 32)
  int inb;          // scan blocks of the inverse-list offsets per slice
  size_t icnt;      // u32 [BH, N]          experts holding each token
  size_t ibits;     // u32 [BH, N, iw]      the experts holding each token, as bits
  size_t ioff;      // u32 [BH, N]          list offsets
  size_t ibsum;     // u32 [BH, inb]        per scan block: token total, then its offset
  size_t ilist;     // u32 [BH, m k]        (expert, slot) entries per token, in expert order
  size_t psort;     // i32 [BH, N s]        the routing grouped by expert, (query * s + slot) ascending per bucket
  size_t pbase;     // u32 [BH, pnch, m]    per chunk: entries of each expert, then their first position
  size_t total;
};
void backward_plan(const Plan& p, BwdLayout* L);
// The backward on `stream`: reads the forward's workspace fws, writes fp32 dQ, dK, dV.
hipError_t launch_backward(const Plan& p, const BwdLayout& L, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, float* dQ, float* dK, float* dV, const char* fws, char* bws,
                           hipStream_t st);

// A value per device, computed once on first use with that device current;
// safe when several host threads launch at once.
struct PerDevice {
  static constexpr int kMax = 64;
  std::once_flag once[kMax];
  int val[kMax] = {};
  template <class F>
  int get(F&& f) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMax) return f();
    std::call_once(once[dev], [&] { val[dev] = f(); });
    return val[dev];
  }
};

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

// Workgroups of `threads` threads (no dynamic LDS) of `kern` resident per CU on the
// current device, at least 1; `cache` holds the answer per device.
template <typename Kern>
int resident_per_cu(PerDevice& cache, Kern kern, int threads) {
  return cache.get([&] {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess || occ < 1) occ = 1;
    return occ;
  });
}

// Validate arguments and build the plan. Returns MITA_OK or a negative status and
// fills `err` (static storage) with the reason.
// `compact`: the exact top-k fallback gets its fewest waves (kTopkGeneralWaves), so
// the workspace is as small as it can be (the fixed-scratch entry point uses it).
mita_status make_plan(const mita_shape* shape, int m, int k, int s, Plan* p, const char** err,
                      bool compact = false);

// Kernel launchers (one per step; each returns the first HIP error it meets).
hipError_t launch_clear(const Plan& p, char* ws, hipStream_t st);
hipError_t launch_pool(const Plan& p, const void* Q, char* ws, hipStream_t st);
hipError_t launch_landmark(const Plan& p, const void* K, const void* V, char* ws, float* S_out, hipStream_t st);
hipError_t launch_topk(const Plan& p, const void* K, char* ws, hipStream_t st);
// Shared-expert merge into V~ and the top-k candidate thresholds (end of step 2).
hipError_t launch_merge_thresh(const Plan& p, char* ws, hipStream_t st);
// Full softmax attention over all N keys of each slice (the comparator; no workspace).
hipError_t launch_dense(int dtype, int d, int BH, int N, const void* Q, const void* K, const void* V, void* out,
                        hipStream_t st);
hipError_t launch_route(const Plan& p, const void* Q, char* ws, hipStream_t st);
bool route_alongside(const Plan& p);   // routing on a second stream beside steps 2-3
hipError_t launch_bucket(const Plan& p, char* ws, hipStream_t st);
// Step 5, routed part: each expert's bucket of queries over its gathered keys. Writes
// the output itself when the landmark part is fused (s = 1, m <= 64), else partials.
hipError_t launch_gather(const Plan& p, const void* Q, const void* K, const void* V, void* out, char* ws,
                         hipStream_t st);
// Step 5, landmark part and merge (no launch when launch_gather wrote the output).
bool has_combine(const Plan& p);
hipError_t launch_combine(const Plan& p, const void* Q, void* out, char* ws, hipStream_t st);

}  // namespace mita
