// Device helpers shared by the gfx950 kernels of the MiTA forward pass.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load as one vector value (a uint4 aggregate copy can end up
// as a memcpy into a stack slot).
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 x = *(const u32x4*)p;
  return make_uint4(x[0], x[1], x[2], x[3]);
}

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// double -> bf16 bits, round to nearest even, without a detour through float
// (a double rounding could move the value by more than half a bf16 ulp).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  // Round the double to 8 significant bits: split with a power-of-two shifter.
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48);
  int e;
  frexp(x, &e);                       // |x| in [2^(e-1), 2^e)
  double sh = ldexp(1.0, e - 8 + 52); // adding and removing sh keeps 8 significant bits (RNE)
  double r = (x > 0) ? ((x + sh) - sh) : ((x - sh) + sh);
  float f = (float)r;                 // exact: r has 8 significant bits
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// ---------------------------------------------------------------- XCD placement
// Workgroups of a 1D grid go round-robin to the 8 XCDs (each with its own L2).
// Work item (lt, c, z) of this workgroup for a landmark-tile x key-chunk x slice
// problem such that the lm_tiles workgroups sharing one key chunk run on one
// XCD and read the chunk through its L2 once. Grid: 8 ceil(nsplit BH / 8)
// lm_tiles workgroups; returns false for the padding ones.
__device__ __forceinline__ bool chunk_item(int lm_tiles, int nsplit, int BH, int& lt, int& c, int& z) {
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  lt = j % lm_tiles;
  const int G = (j / lm_tiles) * 8 + xcd;
  if (G >= nsplit * BH) return false;
  c = G % nsplit;
  z = G / nsplit;
  return true;
}

// ---------------------------------------------------------------- order keys
// Monotone map of float32 onto uint32: a < b (as floats) iff key(a) < key(b).
__device__ __forceinline__ uint32_t f32_key(float x) {
  // negative: all bits flipped; otherwise the sign bit set (no branch or select)
  const uint32_t u = __float_as_uint(x);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Same map for float64 onto uint64.
__device__ __forceinline__ uint64_t f64_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
// Reduce over the four lanes l, l^16, l^32, l^48 (one column of an MFMA 16x16 tile)
// with the gfx950 lane swaps (VALU; no LDS round trip). v_permlane16_swap with both
// operands v leaves v[l] in one result and v[l ^ 16] in the other (likewise 32),
// so every lane combines the same pairs as an xor-shuffle reduction would.
__device__ __forceinline__ float xor16_max(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float quad_max(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float quad_sum(float v) { return xor32_sum(xor16_sum(v)); }

// Orders LDS traffic between the lanes of one wave (waves execute their LDS
// operations in order; this stops the compiler from moving them across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Exclusive prefix sum across the lanes of a wave; `total` gets the wave sum.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(x, o, WAVE);
    if (lane >= o) x += t;
  }
  total = __shfl(x, 63, WAVE);
  return x - v;
}

// DPP-based reductions (no LDS round trip): within each row of 16 lanes, then
// across the four rows with readlane; the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_uniform(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));
  x = max(x, dpp_u32<0x4E>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));
  return max(max((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ uint32_t wave_min_uniform(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));
  x = min(x, dpp_u32<0x4E>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  return min(min((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
             min((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

// Inclusive prefix sum over the 256 threads of a block, in thread order.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, WAVE);
    if (lane >= o) v += t;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) off += (i < w) ? wtot[i] : 0u;
  total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();
  return v + off;
}

// ---------------------------------------------------------------- MFMA wrappers
// 16x16 output tiles: lane l holds C[4*(l/16) + j][l%16], j = 0..3.
// bf16, K = 32: lane l supplies A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16].
__device__ __forceinline__ f32x4 mma_bf16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
// f32, K = 4: lane l supplies A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two floats as fp16 bits (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace mita
