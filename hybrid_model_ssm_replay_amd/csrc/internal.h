// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace rssm {

constexpr uint32_t kCtxMagic = 0x52535331u;  // "RSS1"

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Ring layout.  Every field is indexed by ring slot: the record at token
// position t lives in slot t % Ls, with Ls = L, or 2L when the caller writes
// the records into the ring (REPLAY_FLAG_RECORDS_IN_RING); the L below stands
// for Ls.  The exception is the Mamba-2 B field, shared by the heads of a
// group, which always has 2L slots: a tile that appends a record may then never
// overwrite a B record that another tile of the same group is still folding or
// reading in the same launch (the window plus the drafts of one call span at
// most 2L positions).  Fields are float32, except the record vector fields
// (Mamba-2 x and B, GDN k and v), which are bf16 with REPLAY_FLAG_BF16_RECORDS.
struct RingLayout {
  // Mamba-2: f0 = x [L][B][H][P] (slot-major: one step's appends form one
  //          contiguous block), f1 = B [B][G][2L][N], f2 = dt [B][H][L].
  // GDN:     f0 = k [L][B][H][dk], f1 = u [L][B][H][dv] (pseudo-values,
  //          slot-major), f2 = alpha [B][H][L], f3 = beta [B][H][L], and with
  //          a separate read copy (ckpt_fmt != read_fmt) f4 = v [L][B][H][dv]:
  //          the fold then re-solves the pseudo-values from the checkpoint.
  size_t off[5];
  size_t bytes;
};

// Whether a GDN fold re-solves the window from the checkpoint and the values v
// (a separate read copy: the cached pseudo-values were computed from the read
// copy and must not enter the recurrence), or folds the cached pseudo-values.
inline bool gdn_refold(const replay_config &c) { return c.ckpt_fmt != c.read_fmt; }

inline bool bf16_records(const replay_config &c) { return (c.flags & REPLAY_FLAG_BF16_RECORDS) != 0; }
inline bool records_in_ring(const replay_config &c) { return (c.flags & REPLAY_FLAG_RECORDS_IN_RING) != 0; }
// Slots of the ring fields indexed by position mod Ls (all but the Mamba-2 B field).
inline int ring_slots(const replay_config &c) { return records_in_ring(c) ? 2 * c.window : c.window; }

inline RingLayout ring_layout(const replay_config &c) {
  RingLayout r{};
  const size_t re = bf16_records(c) ? 2 : 4;  // bytes per record vector element
  const size_t Ls = ring_slots(c);
  const size_t B = c.batch, H = c.heads, G = c.groups, L = c.window, P = c.head_dim, N = c.state_dim;
  size_t sz[5] = {0, 0, 0, 0, 0};  // bytes
  if (c.kind == REPLAY_KIND_MAMBA2) {
    sz[0] = B * H * Ls * P * re;
    sz[1] = B * G * 2 * L * N * re;
    sz[2] = B * H * Ls * 4;
  } else {
    sz[0] = B * H * Ls * N * re;
    sz[1] = B * H * Ls * P * 4;
    sz[2] = B * H * Ls * 4;
    sz[3] = B * H * Ls * 4;
    sz[4] = gdn_refold(c) ? B * H * Ls * P * re : 0;
  }
  size_t o = 0;
  for (int i = 0; i < 5; ++i) {
    r.off[i] = o;
    o += align256(sz[i]);
  }
  r.bytes = o;
  return r;
}

// Shape of one launch, as the kernels see it, with the launch-invariant
// divisors the kernels need (heads, heads per group, L, 2 L).
// Ls is the slot count of the slot-indexed ring fields other than the Mamba-2
// B field (which always has 2L): L, or 2L when the caller writes the records
// into the ring (REPLAY_FLAG_RECORDS_IN_RING).
struct Shape {
  int B, H, G, P, N, L, Ls;
  FastDiv fH, fHpg, fL, f2L, fLs;
};

inline Shape make_shape(int B, int H, int G, int P, int N, int L, int Ls) {
  return Shape{B, H, G, P, N, L, Ls, make_fastdiv((uint32_t)H), make_fastdiv((uint32_t)(H / G)),
               make_fastdiv((uint32_t)L), make_fastdiv((uint32_t)(2 * L)), make_fastdiv((uint32_t)Ls)};
}

// Mamba-2 ---------------------------------------------------------------
// Record vector fields (x, B, C here; q, k, v for GDN) and their ring copies
// are float32, or bf16 when `bf16` is set (REPLAY_FLAG_BF16_RECORDS); the
// kernels take the element type as a template parameter.
struct M2Ring {
  void *x;    // [L][B][H][P]
  void *Bm;   // [B][G][2L][N]
  float *dt;  // [B][H][L]
};

struct M2StepArgs {
  Shape s;
  int decay_skip;  // REPLAY_FLAG_DECAY_SKIP set
  float *ckpt;
  M2Ring ring;
  PtrHalves ptr;
  int32_t *status;
  const float *A, *D;
  const void *x, *Bm, *Cm;  // this token: [B][H][P], [B][G][N], [B][G][N]
  const float *dt;           // [B][H]
  int bf16;
  int in_ring;               // x, B, dt are already in their ring slots (x, Bm, dt unused)
  float *y;                  // [B][H][P]
};

struct M2VerifyArgs {
  Shape s;
  int decay_skip;
  int T;
  float *ckpt;
  M2Ring ring;
  PtrHalves ptr;
  int32_t *status;
  const float *A, *D;
  const void *x, *Bm, *Cm;  // drafts: [B][T][H][P], [B][T][G][N], [B][T][G][N]
  const float *dt;           // [B][T][H]
  int bf16;
  int in_ring;               // the drafts' x, B, dt are already in their ring slots
  float *y;                  // [B][T][H][P]
};

struct M2FlushArgs {
  Shape s;
  int decay_skip;
  float *ckpt;
  M2Ring ring;
  PtrHalves ptr;
  int32_t *status;
  const float *A;
  const uint8_t *mask;  // [B] or NULL
  int bf16;
};

struct M2ConvArgs {
  Shape s;
  float *state;  // [B][H][P][N]
  const float *A, *D;
  const void *x, *Bm, *Cm;
  const float *dt;
  int bf16;
  float *y;
};

struct M2SnapArgs {
  Shape s;
  int T, nslots;
  float *slots;  // [B][nslots][H][P][N]
  const int32_t *cur;
  const float *A, *D;
  const void *x, *Bm, *Cm;  // drafts, as M2VerifyArgs
  const float *dt;
  int bf16;
  float *y;
};

// Gated DeltaNet ---------------------------------------------------------
struct GdnRing {
  void *k;       // [L][B][H][dk] (slot-major)
  float *u;      // [L][B][H][dv] (slot-major): pseudo-values
  float *alpha;  // [B][H][L]
  float *beta;   // [B][H][L]
  void *v;       // [L][B][H][dv] (slot-major), separate read copy only; else NULL
};

struct GdnStepArgs {
  Shape s;  // P = d_v, N = d_k
  int decay_skip;  // REPLAY_FLAG_DECAY_SKIP set (float32 copies only)
  GdnRing ring;
  PtrHalves ptr;
  int32_t *status;
  const void *q, *k, *v;        // this token: [B][H][dk], [B][H][dk], [B][H][dv]
  const float *alpha, *beta;    // [B][H]
  int bf16;
  int in_ring;                  // k, alpha, beta are already in their ring slots
  float *y;                     // [B][H][dv]
};

struct GdnVerifyArgs {
  Shape s;
  int decay_skip;  // REPLAY_FLAG_DECAY_SKIP set (float32 copies only)
  int T;
  GdnRing ring;
  PtrHalves ptr;
  int32_t *status;
  const void *q, *k, *v;  // drafts: [B][T][H][...]
  const float *alpha, *beta;
  int bf16;
  int in_ring;            // the drafts' k, alpha, beta are already in their ring slots
  float *y;               // [B][T][H][dv]
};

struct GdnFlushArgs {
  Shape s;
  int decay_skip;  // REPLAY_FLAG_DECAY_SKIP set (float32 copies only)
  GdnRing ring;
  PtrHalves ptr;
  int32_t *status;
  const uint8_t *mask;
  int bf16;
};

struct GdnConvArgs {
  Shape s;
  float *state;  // [B][H][dv][dk]
  const void *q, *k, *v;
  const float *alpha, *beta;
  int bf16;
  float *y;
};

struct GdnSnapArgs {
  Shape s;
  int T, nslots;
  float *slots;  // [B][nslots][H][dv][dk]
  const int32_t *cur;
  const void *q, *k, *v;  // drafts
  const float *alpha, *beta;
  int bf16;
  float *y;
};

// Stored copies of a layer's state: the checkpoint that carries the recurrence
// (ckpt_fmt) and the copy non-fold steps read (read_fmt; the same storage when
// the formats are equal).  e2m1 copies keep their scales after the codes.
struct FormatBufs {
  int ckpt_fmt, read_fmt;
  void *ckpt;
  uint8_t *ckpt_scales;
  void *read;
  uint8_t *read_scales;
  int8_t *read_cols;  // two-axis e2m1 read copy: column exponents [B][H][dk]
  uint64_t seed;
};

struct EncodeArgs {
  Shape s;
  const float *src;         // [B][H][P][N] float32 state (GDN: P = d_v, N = d_k)
  const int32_t *ckpt_pos;  // current ckpt_pos[B] (stochastic-rounding counter)
  int write_ckpt;           // 0: write only the read copy
};

// Bytes of one stored copy of n elements with ncols state columns in all
// (batch x heads x state_dim), where an e2m1 copy's block scales start, and
// where a two-axis copy's column exponents start.
inline size_t e2m1_scale_offset(size_t n) { return align256(n / 2); }
inline size_t e2m1_cols_offset(size_t n) { return align256(e2m1_scale_offset(n) + n / 16); }
inline size_t state_bytes(int fmt, size_t n, size_t ncols) {
  switch (fmt) {
    case REPLAY_FMT_F32: return 4 * n;
    case REPLAY_FMT_F16_SR: return 2 * n;
    case REPLAY_FMT_F8E4M3: return n;
    case REPLAY_FMT_F4E2M1_CS: return e2m1_cols_offset(n) + ncols;
    default: return e2m1_scale_offset(n) + n / 16;
  }
}

// Launchers (return a hipError_t value).
int launch_gdn_step(const GdnStepArgs &a, const FormatBufs &f, hipStream_t st);
int launch_gdn_verify(const GdnVerifyArgs &a, const FormatBufs &f, hipStream_t st);
int launch_gdn_flush(const GdnFlushArgs &a, const FormatBufs &f, hipStream_t st);
int launch_encode_state(const EncodeArgs &a, const FormatBufs &f, hipStream_t st);
int launch_gdn_conv(const GdnConvArgs &a, hipStream_t st);
int launch_gdn_snapshot(const GdnSnapArgs &a, hipStream_t st);
int launch_record_slots(const int32_t *pos, int batch, int slots, int32_t *out, hipStream_t st);
int launch_m2_step(const M2StepArgs &a, const FormatBufs &f, hipStream_t st);
int launch_m2_verify(const M2VerifyArgs &a, const FormatBufs &f, hipStream_t st);
int launch_m2_flush(const M2FlushArgs &a, const FormatBufs &f, hipStream_t st);
int launch_m2_conv(const M2ConvArgs &a, hipStream_t st);
int launch_m2_snapshot(const M2SnapArgs &a, hipStream_t st);

// Pointer kernels -------------------------------------------------------
int launch_init_pointers(int32_t *words, int nwords, int32_t *status, hipStream_t st);
int launch_commit(PtrHalves p, int B, const int32_t *accepted, int T, int32_t *status, hipStream_t st);
int launch_snapshot_commit(int32_t *cur, const int32_t *accepted, int B, int T, int nslots, hipStream_t st);
int launch_probe(const void *src, void *dst, size_t bytes, int mode, hipStream_t st);

// Launch geometry of the per-head kernels: one workgroup per (sequence, head).
// wave_per_head kernels (step, conventional, snapshot): RBW row blocks of 16
// rows per wave, RBW = 2 when the number of row blocks is even, else 1.
// Workgroup kernels (flush, verify): one wave per row block, at most 4 waves,
// RBW = 2 at P = 128.  Supported P: 16, 32, 48, 64, 128.
inline bool tile_geometry(int P, bool wave_per_head, int *waves, int *rbw) {
  if (P % 16 || P < 16) return false;
  const int rb = P / 16;
  if (rb > 4 && rb != 8) return false;
  if (wave_per_head) {
    *rbw = (rb % 2 == 0) ? 2 : 1;
    *waves = rb / *rbw;
    return true;
  }
  *waves = rb <= 4 ? rb : 4;
  *rbw = rb / *waves;
  return true;
}

}  // namespace rssm
