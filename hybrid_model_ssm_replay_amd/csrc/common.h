// Shared device helpers for the replay decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "replayssm.h"

namespace rssm {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxL = REPLAY_MAX_WINDOW;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Workgroups are dispatched round-robin over the XCDs (workgroup i runs on XCD
// i % 8).  Renumber them so that each XCD receives one contiguous range of
// logical tiles: tiles that share data (the heads of one sequence or of one
// B/C group) then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks % kXcds) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

__device__ __forceinline__ floatx4 mfma_16x16x4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float f4get(float4 v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Workgroup barrier for LDS hand-off only: waits for this wave's LDS traffic,
// not for its outstanding global loads, so checkpoint loads issued before the
// barrier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Sum over the 16 lanes l, l^1, ..., l^15 (one row of 16 lanes).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 8, kWave);
  v += __shfl_xor(v, 4, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 1, kWave);
  return v;
}
// ---- record element types ---------------------------------------------------
// Record vector fields are float32, or bf16 (REPLAY_FLAG_BF16_RECORDS) stored
// as the upper half of a float32 bit pattern: widening is an exact shift, and
// a value read from a bf16 field is stored back exactly by truncation.
typedef uint16_t bf16_t;

template <typename R>
__device__ __forceinline__ float ldr(const R *p);
template <>
__device__ __forceinline__ float ldr<float>(const float *p) {
  return *p;
}
template <>
__device__ __forceinline__ float ldr<bf16_t>(const bf16_t *p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// Four consecutive elements (16-byte aligned for float32, 8-byte for bf16).
template <typename R>
__device__ __forceinline__ float4 ldr4(const R *p);
template <>
__device__ __forceinline__ float4 ldr4<float>(const float *p) {
  return ld4(p);
}
template <>
__device__ __forceinline__ float4 ldr4<bf16_t>(const bf16_t *p) {
  const uint2 w = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}

// Stores of values the field holds exactly (values read from such a field).
template <typename R>
__device__ __forceinline__ void str(R *p, float v);
template <>
__device__ __forceinline__ void str<float>(float *p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void str<bf16_t>(bf16_t *p, float v) {
  *p = (bf16_t)(__float_as_uint(v) >> 16);
}
template <typename R>
__device__ __forceinline__ void str4(R *p, float4 v);
template <>
__device__ __forceinline__ void str4<float>(float *p, float4 v) {
  st4(p, v);
}
template <>
__device__ __forceinline__ void str4<bf16_t>(bf16_t *p, float4 v) {
  *reinterpret_cast<uint2 *>(p) = make_uint2((__float_as_uint(v.x) >> 16) | (__float_as_uint(v.y) & 0xFFFF0000u),
                                             (__float_as_uint(v.z) >> 16) | (__float_as_uint(v.w) & 0xFFFF0000u));
}

// Maximum over the 16 lanes of a row, by DPP within the row: the quad swaps
// [1,0,3,2] and [2,3,0,1], then the half-row mirror (quads 0 <-> 1, 2 <-> 3)
// and the row mirror (halves 0 <-> 1).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

// One 16-byte global-to-LDS load per lane (global_load_lds_dwordx4): lane l's
// 16 bytes from src go to lds[l]; lds must be the same for the whole wave.
// Completion is counted by vmcnt like any load.
__device__ __forceinline__ void dma16(const float *src, float4 *lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), (lds_void *)(lds), 16, 0, 0);
}

// One record vector (N elements of type R) into LDS at dst, which is the same
// for the whole wave, by direct global-to-LDS loads: lane l < N sizeof(R) / 16
// moves bytes 16 l .. 16 l + 15.  The data is there once vmcnt reaches zero.
template <int N, typename R>
__device__ __forceinline__ void dma_vec(const R *src, void *dst, int lane) {
  constexpr int kLanes = N * (int)sizeof(R) / 16;
  static_assert(kLanes >= 1 && kLanes <= kWave, "record vector must be 16 .. 1024 bytes");
  if (lane < kLanes)
    dma16(reinterpret_cast<const float *>(reinterpret_cast<const char *>(src) + 16 * lane),
          reinterpret_cast<float4 *>(dst));
}

// Four elements per lane into LDS as float32, lane l's at lds[l] (lds the same
// for the whole wave): a direct global-to-LDS load for float32 fields, a load,
// exact widening and LDS store for bf16 fields.  Either way the data is in
// place after s_waitcnt(0) and a barrier.
template <typename R>
__device__ __forceinline__ void stage4(const R *src, float4 *lds, int lane);
template <>
__device__ __forceinline__ void stage4<float>(const float *src, float4 *lds, int) {
  dma16(src, lds);
}
template <>
__device__ __forceinline__ void stage4<bf16_t>(const bf16_t *src, float4 *lds, int lane) {
  lds[lane] = ldr4<bf16_t>(src);
}

// Program-order fence for LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the four lanes l, l^16, l^32, l^48 (the four k-quarters of an MFMA
// row), by the gfx950 row-swap instructions instead of LDS permutes: with both
// operands v, v_permlane16_swap leaves row r of v in one result and row r ^ 1 in
// the other (rows of 16 lanes), and v_permlane32_swap does the same for the two
// halves of the wave.  Every lane adds the same two values (in either order),
// so all four lanes get the same sum.  All 64 lanes must be active.
__device__ __forceinline__ float sum_quarters(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Double-buffered pointer words: half p holds pos[batch] then ckpt_pos[batch].
// A launch reads half `cur` and writes half `cur ^ 1`, so no tile of a launch
// can observe another tile's update of the same sequence.
struct PtrHalves {
  const int32_t *pos_in;
  const int32_t *ckpt_in;
  int32_t *pos_out;
  int32_t *ckpt_out;
};

}  // namespace rssm

namespace rssm {

// Division by a divisor fixed for the whole launch, as a multiply-high and a
// shift (round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994): with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (umulhi(n, m) + n) >> s for
// 0 <= n < 2^31.  The host fills it; kernels divide tile indices and token
// positions with it instead of a ~20-instruction integer division.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ int fdiv(int n, const FastDiv &f) {
  const uint32_t t = __umulhi((uint32_t)n, f.m);
  return (int)((t + (uint32_t)n) >> f.s);
}
__device__ __forceinline__ int fmod_(int n, const FastDiv &f) { return n - fdiv(n, f) * (int)f.d; }

// Decay skip (REPLAY_FLAG_DECAY_SKIP): a head whose window log-decay is below
// ln 2^-24 drops its checkpoint term [P3, Perspective, paragraph 1].
constexpr float kDecaySkipLog = -16.635532333438686f;  // ln 2^-24

// A pointer pair the kernels act on: 0 <= ckpt_pos <= pos <= ckpt_pos + L.
// Any other pair (corrupted, or negative) flags its sequence, which is then
// skipped: ring slots are only ever computed from non-negative positions, the
// domain of fdiv / fmod_ above.
__device__ __forceinline__ bool pointers_ok(int pos, int ck, int L) {
  return (uint32_t)(pos - ck) <= (uint32_t)L && ck >= 0;  // one unsigned compare for 0 <= count <= L
}

// (s0 + j) mod d for 0 <= s0 < d and 0 <= j < d: one compare, no division.
__device__ __forceinline__ int wrap(int s0, int j, int d) {
  const int v = s0 + j;
  return v >= d ? v - d : v;
}

}  // namespace rssm
