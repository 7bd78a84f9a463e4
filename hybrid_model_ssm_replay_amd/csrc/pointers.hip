// Pointer kernels (init, commit) and the HBM probe used by the measurements.
#include "internal.h"

namespace rssm {
namespace {

__global__ void init_pointers_k(int32_t *words, int nwords, int32_t *status) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nwords) words[i] = 0;
  if (i == 0) *status = 0;
}

// Accept the first accepted[b] drafts: a pointer move [P1, Interpretation 3;
// P3, Interpretation 3].  Out-of-range counts are clamped to 0..T and flagged.
__global__ void commit_k(PtrHalves p, int B, const int32_t *accepted, int T, int32_t *status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = accepted[b];
  const int adv = a < 0 ? 0 : (a > T ? T : a);
  if (adv != a) atomicOr(status, REPLAY_STATUS_ACCEPT_CLAMPED);
  p.pos_out[b] = p.pos_in[b] + adv;
  p.ckpt_out[b] = p.ckpt_in[b];
}

// Ring slot of each sequence's next record: pos mod the slot count.  A
// negative pos (never produced by the library) maps to slot 0.
__global__ void record_slots_k(const int32_t *pos, int B, int slots, int32_t *out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int p = pos[b];
  out[b] = p < 0 ? 0 : p % slots;
}

__global__ void snapshot_commit_k(int32_t *cur, const int32_t *accepted, int B, int T, int nslots) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = accepted[b];
  const int adv = a < 0 ? 0 : (a > T ? T : a);
  cur[b] = (cur[b] + adv) % nslots;
}

// Plain 16-byte streams: one float4 per thread, grid covering the buffer.
__global__ void probe_read_k(const float4 *__restrict__ src, float4 *__restrict__ dst, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = src[i];
  if (v.x == 1.2345e-30f && v.y == -7.0e29f) dst[0] = v;  // keeps the load; never true for probe data
}
__global__ void probe_copy_k(const float4 *__restrict__ src, float4 *__restrict__ dst, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) dst[i] = src[i];
}

}  // namespace

int launch_init_pointers(int32_t *words, int nwords, int32_t *status, hipStream_t st) {
  const int n = nwords > 1 ? nwords : 1;
  hipLaunchKernelGGL(init_pointers_k, dim3((n + 255) / 256), dim3(256), 0, st, words, nwords, status);
  return (int)hipGetLastError();
}

int launch_commit(PtrHalves p, int B, const int32_t *accepted, int T, int32_t *status, hipStream_t st) {
  hipLaunchKernelGGL(commit_k, dim3((B + 255) / 256), dim3(256), 0, st, p, B, accepted, T, status);
  return (int)hipGetLastError();
}

int launch_record_slots(const int32_t *pos, int batch, int slots, int32_t *out, hipStream_t st) {
  hipLaunchKernelGGL(record_slots_k, dim3((batch + 255) / 256), dim3(256), 0, st, pos, batch, slots, out);
  return (int)hipGetLastError();
}

int launch_snapshot_commit(int32_t *cur, const int32_t *accepted, int B, int T, int nslots, hipStream_t st) {
  hipLaunchKernelGGL(snapshot_commit_k, dim3((B + 255) / 256), dim3(256), 0, st, cur, accepted, B, T, nslots);
  return (int)hipGetLastError();
}

int launch_probe(const void *src, void *dst, size_t bytes, int mode, hipStream_t st) {
  const size_t n4 = bytes / 16;
  const size_t blocks = (n4 + 255) / 256;
  if (blocks == 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  if (mode == 0)
    hipLaunchKernelGGL(probe_read_k, dim3((unsigned)blocks), dim3(256), 0, st, (const float4 *)src, (float4 *)dst, n4);
  else
    hipLaunchKernelGGL(probe_copy_k, dim3((unsigned)blocks), dim3(256), 0, st, (const float4 *)src, (float4 *)dst, n4);
  return (int)hipGetLastError();
}

}  // namespace rssm
