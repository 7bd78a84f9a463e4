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

// Streaming loads of data touched exactly once per launch (the checkpoint):
// non-temporal, so they do not evict the ring records and parameters that the
// other tiles of the same sequence re-read.
__device__ __forceinline__ float4 ld4_stream(const float *p) {
  float4 v;
  v.x = __builtin_nontemporal_load(p + 0);
  v.y = __builtin_nontemporal_load(p + 1);
  v.z = __builtin_nontemporal_load(p + 2);
  v.w = __builtin_nontemporal_load(p + 3);
  return v;
}
__device__ __forceinline__ void st4_stream(float *p, float4 v) {
  __builtin_nontemporal_store(v.x, p + 0);
  __builtin_nontemporal_store(v.y, p + 1);
  __builtin_nontemporal_store(v.z, p + 2);
  __builtin_nontemporal_store(v.w, p + 3);
}

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
// Sum over the four lanes l, l^16, l^32, l^48 (the four k-quarters of an MFMA row).
__device__ __forceinline__ float sum_quarters(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
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
