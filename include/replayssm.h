/*
 * replayssm.h -- C ABI of the ReplaySSM decode library for AMD Instinct MI355X (gfx950).
 *
 * The library computes one state-space layer's decode step with the state held
 * as a checkpoint plus a ring buffer of the last L <= 16 input records, instead
 * of a state that is read and written back at every token.  Pages cited:
 *   [P1] "Hybrid-model decoding has a new bottleneck: stop writing the SSM state
 *        every step, and speculative throughput reaches 2.10x"
 *   [P2] "NVIDIA and Dao AI Lab speed up hybrid-model decoding"
 *   [P3] "SSM decoding stops writing state every step: caching recent inputs
 *        halves state traffic and matches vLLM speculation"
 * The layer recurrences are the published Mamba-2 (SSD) and Gated DeltaNet
 * decode updates:
 *   Mamba-2, per head h with B/C group g = h / (heads / groups):
 *       S_h <- exp(dt_h A_h) S_h + dt_h x_h B_g^T,   y_h = S_h C_g + D_h x_h
 *   Gated DeltaNet, per head:
 *       S <- alpha S (I - beta k k^T) + beta v k^T,  o = S q
 * In both, the output is read from the state after the token's update.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers unless stated otherwise; the
 *     library never allocates, frees or copies to the host.  The caller owns
 *     every buffer and keeps it alive until the work queued on the stream ends.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; none synchronises the host.
 *   - Return value: REPLAY_OK, or a negative code.  REPLAY_EINVAL (bad shape,
 *     NULL pointer, misaligned pointer, unsupported pair of formats) is returned
 *     before anything is enqueued; REPLAY_EHIP reports a failed kernel launch.
 *   - Floating-point arrays are float32 (the record vector fields are bf16 with
 *     REPLAY_FLAG_BF16_RECORDS), C-contiguous, 16-byte aligned.
 *   - Calls on one context must be issued on one stream (or be ordered by the
 *     caller): they read pointer words written by the previous call.
 *   - Anomalies found on the device (a clamped accept count, a corrupted
 *     pointer pair) set sticky bits in `status`; the affected sequence is
 *     clamped or skipped, never read out of bounds.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REPLAY_MAX_WINDOW 16

/* Layer families. */
#define REPLAY_KIND_MAMBA2 0
#define REPLAY_KIND_GDN 1

/* Storage formats of the checkpoint (recurrence copy) and of the read copy. */
#define REPLAY_FMT_F32 0
#define REPLAY_FMT_F16_SR 1     /* IEEE binary16, written with stochastic rounding */
#define REPLAY_FMT_F8E4M3 2     /* OCP FP8 e4m3fn, round to nearest even, saturating */
#define REPLAY_FMT_F4E2M1_B16 3 /* 4-bit e2m1 values, one e4m3 scale per 16 */
#define REPLAY_FMT_F4E2M1_CS 4  /* F4E2M1_B16 plus a power-of-two scale per state column (read copy only) */

/* Option flags (replay_config.flags). */
#define REPLAY_FLAG_DECAY_SKIP 0x1u   /* Mamba-2: drop the checkpoint term of heads whose decay is below 2^-24 */
#define REPLAY_FLAG_BF16_RECORDS 0x2u /* record vector fields (Mamba-2 x, B, C; GDN q, k, v) are bf16 */
#define REPLAY_FLAG_RECORDS_IN_RING 0x4u /* the caller writes the stored record fields into the ring */

/* Return codes. */
#define REPLAY_OK 0
#define REPLAY_EINVAL (-1)
#define REPLAY_EHIP (-2)
#define REPLAY_ENOTSUP (-3)

/* Sticky bits of the device status word. */
#define REPLAY_STATUS_ACCEPT_CLAMPED 0x1 /* commit got accepted < 0 or > drafts pending */
#define REPLAY_STATUS_BAD_POINTERS 0x2   /* ckpt_pos < 0 or pos - ckpt_pos outside 0..L: sequence skipped */

/*
 * Every output is read from the state that includes its own token [P3,
 * Interpretation 1].  Outputs of a step or verify that folds first come from
 * the fold result (float32); all other outputs read the read copy plus the
 * buffered records, so only they carry the read copy's rounding [P3,
 * Perspective, paragraph 2].
 *
 * Layer shape and options.
 *   kind        REPLAY_KIND_MAMBA2 or REPLAY_KIND_GDN.
 *   batch       sequences, >= 1.
 *   heads       heads per sequence, >= 1.
 *   groups      Mamba-2: B/C groups, heads % groups == 0 (contiguous blocks of
 *               heads / groups heads share a group).  GDN: must equal heads.
 *   head_dim    Mamba-2: P.  GDN: d_v.  Multiple of 16, at most 128.
 *   state_dim   Mamba-2: N.  GDN: d_k.  One of 16, 32, 64, 128.
 *   window      L, the ring length, 1..16.  A window folds into the checkpoint
 *               only once it is full [P2, paragraph 3; P3, Interpretation 2].
 *   max_draft   largest T a verify call will use, 0..L (sizes the ring).
 *   ckpt_fmt    format of the checkpoint that carries the recurrence.
 *   read_fmt    format of the copy the outputs read; equal to ckpt_fmt
 *               means a single copy [P1, Interpretation 4; P3, Interpretation 3].
 *               Outputs of calls that do not fold read the read copy plus the
 *               buffered records in float32; a fold starts from the
 *               checkpoint, so the read copy's rounding never enters the
 *               recurrence.
 *   seed        key of the stochastic-rounding generator (Philox-4x32-10; the
 *               fold that sets ckpt_pos of sequence b draws element e of head h
 *               from word e % 4 of Philox(counter (e / 4, h, b, ckpt_pos),
 *               key (seed low 32 bits, seed high 32 bits)), top 24 bits).
 *   flags       an OR of REPLAY_FLAG_DECAY_SKIP, REPLAY_FLAG_BF16_RECORDS and
 *               REPLAY_FLAG_RECORDS_IN_RING.
 *               REPLAY_FLAG_DECAY_SKIP (Mamba-2 only, else REPLAY_ENOTSUP):
 *               a head whose window decay exp(A s) (s = the dt summed over the
 *               window records a computation uses) is below 2^-24 drops the
 *               checkpoint term: a step then does not read that head's
 *               checkpoint, and its fold is a pure write of the folded records
 *               [P3, Perspective, paragraph 1].  An approximation: each output
 *               moves by at most 2^-24 |S0 C|.  Verify applies the same rule to
 *               its outputs and fold-first but always reads the checkpoint.
 *               REPLAY_FLAG_BF16_RECORDS: the record vector fields (Mamba-2
 *               x, B, C; GDN q, k, v) of every call, and their copies in the
 *               ring, are bf16, which halves the record traffic the pages
 *               count next to the state [P1, Synopsis]; values are widened
 *               exactly, so the arithmetic (float32) and the state, pseudo-
 *               values and outputs (float32) are unchanged.
 *               REPLAY_FLAG_RECORDS_IN_RING (zero-copy append): the producer of
 *               the records writes the fields the ring keeps (Mamba-2 x, B,
 *               dt; GDN k, alpha, beta) straight into their ring slots before
 *               each step or verify (replay_record_slots, replay_ring_view),
 *               and those calls take only the other fields from their record
 *               argument (Mamba-2 C; GDN q, v), so no call copies a record into
 *               the ring.  The ring then has 2L slots per field: the slot of a
 *               step's new record, or of T <= L drafts, is never one the
 *               window still holds.
 *   reserved    must be 0.
 * Supported format pairs (ckpt_fmt, read_fmt): (F32, F32) for both families;
 * for Gated DeltaNet with state_dim = 128 also (F32 | F16_SR | F8E4M3, F4E2M1_B16)
 * (split precision), (F32 | F16_SR | F8E4M3, F4E2M1_CS) (split precision with
 * the two-axis read copy) and (F16_SR, F16_SR), (F8E4M3, F8E4M3), (F4E2M1_B16,
 * F4E2M1_B16) (one shared low-precision copy).  Other pairs: REPLAY_ENOTSUP.
 *
 * Storage formats, per element of [batch][heads][head_dim][state_dim]:
 *   F32         float32.
 *   F16_SR      IEEE binary16, written with stochastic rounding
 *               RTZ16(x + sign(x) (r / 2^24) ulp16(|x|)), saturating at +-65504.
 *   F8E4M3      OCP e4m3fn, round to nearest even, saturating at +-448.
 *   F4E2M1_B16  4-bit e2m1 codes (two per byte, the even element in the low
 *               nibble) followed, at the next 256-byte boundary, by one e4m3
 *               scale byte per 16 consecutive state_dim elements:
 *               s = e4m3(amax / 6); element codes round x / s to
 *               {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code, clamped).
 *   F4E2M1_CS   scales along both axes of each head's [head_dim][state_dim]
 *               state (the pages suggest separate state and channel scales for
 *               the read copy [P1, Perspective, paragraph 2]): the F4E2M1_B16
 *               codes and block scales (blocks along state_dim, inside one
 *               head_dim channel) of x / 2^e[n], followed, at the next 256-byte
 *               boundary after the block scales, by one signed byte e[n] per
 *               state column [batch][heads][state_dim]:
 *               e[n] = max(floor(log2 amax_n) - 5, -126), amax_n the largest
 *               |x| of column n over the head's channels (-126 when zero), so
 *               that amax_n / 2^e[n] lies in [32, 64).  Decoded value:
 *               e2m1 x block scale x 2^e[n].
 * An all-zero buffer is the zero state in every format.
 */
typedef struct replay_config {
  int32_t kind;
  int32_t batch;
  int32_t heads;
  int32_t groups;
  int32_t head_dim;
  int32_t state_dim;
  int32_t window;
  int32_t max_draft;
  int32_t ckpt_fmt;
  int32_t read_fmt;
  uint64_t seed;
  uint32_t flags;
  uint32_t reserved;
} replay_config;

/*
 * Device buffers of one layer, all allocated by the caller.
 *   ckpt       replay_ckpt_bytes(cfg) bytes, layout [batch][heads][head_dim][state_dim]
 *              (state_dim contiguous) in ckpt_fmt; 256-byte aligned unless F32.
 *              It changes only at a fold (and replay_set_state).
 *   read_copy  replay_read_copy_bytes(cfg) bytes (256-byte aligned), or NULL
 *              when that is 0 (read_fmt == ckpt_fmt).
 *   ring       replay_ring_bytes(cfg) bytes; layout private to the library.
 *   pointers   replay_pointer_words(cfg) int32 words: two halves, each
 *              {pos[batch], ckpt_pos[batch]}; see replay_current_pointers().
 *   status     one int32, sticky anomaly bits (cleared by replay_init).
 *   A, D       Mamba-2 per-head decay rate A[heads] (negative) and skip weight
 *              D[heads]; NULL for GDN.
 */
typedef struct replay_buffers {
  void *ckpt;
  void *read_copy;
  void *ring;
  int32_t *pointers;
  int32_t *status;
  const float *A;
  const float *D;
} replay_buffers;

/*
 * One record per sequence (step) or T records per sequence (verify).  The
 * vector fields f0, f1, f2 are float32, or bf16 (IEEE binary32 with the low 16
 * bits dropped) when the configuration sets REPLAY_FLAG_BF16_RECORDS; the
 * per-head scalars f3, f4 are always float32:
 *   Mamba-2: f0 = x [batch][heads][P], f1 = B [batch][groups][N],
 *            f2 = C [batch][groups][N], f3 = dt [batch][heads] (already
 *            positive, i.e. after any softplus), f4 unused.
 *   GDN:     f0 = q [batch][heads][d_k], f1 = k [batch][heads][d_k],
 *            f2 = v [batch][heads][d_v], f3 = alpha [batch][heads] in (0, 1],
 *            f4 = beta [batch][heads].
 * For verify every field has a draft axis after batch: x [batch][T][heads][P] etc.
 */
/* With REPLAY_FLAG_RECORDS_IN_RING the fields kept in the ring (Mamba-2 f0, f1,
 * f3; GDN f1, f3, f4) are not read and may be NULL. */
typedef struct replay_record {
  const void *f0;
  const void *f1;
  const void *f2;
  const float *f3;
  const float *f4;
} replay_record;

/* Caller-owned context (plain data, no destroy call).  Fields are managed by the
 * library; callers read them only through the functions below. */
typedef struct replay_ctx {
  replay_config cfg;
  replay_buffers buf;
  int32_t parity;    /* which half of buf.pointers holds the current pointers */
  int32_t t_pending; /* drafts staged by the last verify and not yet committed */
  uint32_t magic;
  int32_t reserved;
} replay_ctx;

/* ---- sizes and checks (host only, no device work) ---------------------- */

/* REPLAY_OK if the configuration is supported, REPLAY_EINVAL / REPLAY_ENOTSUP otherwise. */
int replay_validate_config(const replay_config *cfg);
/* Bytes of each device buffer; 0 for an invalid configuration. */
size_t replay_ckpt_bytes(const replay_config *cfg);
size_t replay_read_copy_bytes(const replay_config *cfg);
size_t replay_ring_bytes(const replay_config *cfg);
size_t replay_pointer_words(const replay_config *cfg);
/* Static text for a return code. */
const char *replay_strerror(int code);
/* sizeof of the ABI structs, for bindings: 0 replay_config, 1 replay_buffers,
 * 2 replay_record, 3 replay_ctx, 4 replay_ring_view. */
size_t replay_abi_sizeof(int which);

/* ---- the decode calls -------------------------------------------------- */

/* Set up one layer's state as the method holds it: a checkpoint plus a buffer
 * of the inputs since it [P1, Synopsis; P2, paragraph 3], here with an empty
 * buffer.  Fills *ctx from cfg and buf (both copied; buf's device buffers stay
 * owned by the caller) and enqueues pos = ckpt_pos = 0 for every sequence and
 * status = 0.  The checkpoint buffer already holds the initial state in
 * ckpt_fmt; with an F32 checkpoint and a separate read copy (the split
 * precision of [P1, Interpretation 4; P3, Interpretation 3]) the read copy is
 * written from it here.  (For other formats load the state with
 * replay_set_state, or start from all-zero buffers.)  REPLAY_EINVAL for a NULL
 * or misaligned buffer, REPLAY_EINVAL / REPLAY_ENOTSUP for the configuration;
 * *ctx is then left unusable. */
int replay_init(replay_ctx *ctx, const replay_config *cfg, const replay_buffers *buf, void *stream);

/* Replace the state of every sequence with the float32 `state`
 * ([batch][heads][head_dim][state_dim], device), encoding it into the
 * checkpoint and the read copy in their formats.  Pointers are unchanged: the
 * state becomes the checkpoint at each sequence's ckpt_pos (call it with empty
 * windows, e.g. right after replay_init or a full replay_flush). */
int replay_set_state(replay_ctx *ctx, const float *state, void *stream);

/* One decode token for every sequence [P1, Interpretation 2; P3, Interpretation 2]:
 * if a sequence's window is full (L records) it is first folded into the
 * checkpoint; then the record is appended and y is computed from one read of
 * the checkpoint plus the buffered records, with no state write-back.
 * y: Mamba-2 [batch][heads][P], GDN [batch][heads][d_v].  Discards drafts still
 * pending from a verify (the same as commit of 0). */
int replay_step(replay_ctx *ctx, const replay_record *rec, float *y, void *stream);

/* Fold every committed record of the sequences with seq_mask[b] != 0 (device
 * uint8 [batch]; NULL = all) into the checkpoint -- the fold a full buffer
 * triggers [P2, paragraph 3; P3, Interpretation 2], here on demand: the call
 * for a caller that needs the state in the checkpoint alone before the window
 * has filled (e.g. to save it; copying the stored copies and the current
 * pointers then saves the whole state).  Sequences with an empty window are left unchanged.
 * Drafts still pending from a verify are discarded, as by a step (the same as
 * commit of 0): a later commit finds none and clamps its counts to 0. */
int replay_flush(replay_ctx *ctx, const uint8_t *seq_mask, void *stream);

/* Speculative verification of T drafts per sequence, 1 <= T <= max_draft
 * [P1, Interpretation 3; P3, Interpretation 3]: sequences whose window cannot
 * hold T more records are folded first; the drafts are staged in the ring and
 * y receives the T outputs each draft would produce, [batch][T][heads][head_dim],
 * without writing any intermediate state. */
int replay_verify(replay_ctx *ctx, int32_t T, const replay_record *drafts, float *y, void *stream);

/* Accept the first accepted[b] drafts of each sequence (device int32 [batch],
 * read on the device: no host round trip): a pointer move only, since rolling
 * back to the accepted prefix needs no state restore [P1, Interpretation 3;
 * P3, Interpretation 3].  pos[b] += accepted[b]; values outside 0..T_pending
 * (T_pending = the T of the last verify, 0 after any other call) are clamped
 * and set REPLAY_STATUS_ACCEPT_CLAMPED.  Rejected drafts are simply left behind
 * in the ring, to be overwritten. */
int replay_commit(replay_ctx *ctx, const int32_t *accepted, void *stream);

/* Device addresses of the current pos[batch] and ckpt_pos[batch] arrays (valid
 * until the next call that enqueues work on ctx). */
int replay_current_pointers(const replay_ctx *ctx, const int32_t **pos, const int32_t **ckpt_pos);

/* ---- zero-copy append (REPLAY_FLAG_RECORDS_IN_RING) ------------------------ */

/* Where a producer writes the stored record fields (device addresses inside the
 * ring buffer; f[i] matches record field fi, NULL for fields not kept):
 *   Mamba-2: f[0] = x  [slots][batch][heads][P]   (slot-major),
 *            f[1] = B  [batch][groups][slots][N],
 *            f[3] = dt [batch][heads][slots]      (float32);
 *   GDN:     f[1] = k  [slots][batch][heads][d_k] (slot-major),
 *            f[3] = alpha, f[4] = beta [batch][heads][slots] (float32).
 * slots = 2 window; vector fields are bf16 with REPLAY_FLAG_BF16_RECORDS.
 * REPLAY_EINVAL unless the context was configured with RECORDS_IN_RING. */
typedef struct replay_ring_view {
  void *f[5];
  int32_t slots;
  int32_t reserved;
} replay_ring_view;
int replay_ring_fields(const replay_ctx *ctx, replay_ring_view *view);

/* Enqueue slot[b] = pos[b] mod slots (device int32 [batch]): the ring slot of
 * sequence b's next record; draft i of a verify goes to (slot[b] + i) mod slots.
 * The slots stay valid until the next step, verify, commit or flush of ctx, so
 * the producer writes between this call and the step or verify it feeds, on
 * the same stream (or ordered after it).  REPLAY_EINVAL unless RECORDS_IN_RING. */
int replay_record_slots(const replay_ctx *ctx, int32_t *slots, void *stream);

/* ---- in-run baselines (for measurement, not part of the replay method) ---- */

/* Conventional decode step: load the F32 state [batch][heads][head_dim][state_dim],
 * update it, compute y from the updated state, store it back -- L reads and L
 * writes per window [P1, Interpretation 2; P3, Interpretation 1].  cfg->window,
 * max_draft and formats are ignored.  A, D: Mamba-2 parameters, NULL for GDN. */
int replay_conv_step(const replay_config *cfg, float *state, const float *A, const float *D,
                     const replay_record *rec, float *y, void *stream);

/* Snapshot-per-draft verification, the scheme the method replaces
 * [P1, Interpretation 3; P3, Interpretation 3]: slots holds cfg->max_draft + 1
 * F32 states per sequence, [batch][max_draft + 1][heads][head_dim][state_dim];
 * cur[b] names the current slot.  Reads slot cur[b] once, and after each draft
 * i (0-based) writes the state to slot (cur[b] + 1 + i) mod (max_draft + 1):
 * one read and T writes.  y as for replay_verify. */
int replay_snapshot_verify(const replay_config *cfg, float *slots, const int32_t *cur, int32_t T,
                           const float *A, const float *D, const replay_record *drafts, float *y,
                           void *stream);
/* cur[b] <- (cur[b] + clamp(accepted[b], 0, T)) mod (max_draft + 1). */
int replay_snapshot_commit(const replay_config *cfg, int32_t *cur, const int32_t *accepted, int32_t T,
                           void *stream);

/* HBM ceiling probe: mode 0 reads `bytes` from src (dst receives at most 16
 * bytes, written only if a never-occurring value is read); mode 1 copies
 * src to dst.  bytes must be a multiple of 16. */
int replay_hbm_probe(const void *src, void *dst, size_t bytes, int mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
