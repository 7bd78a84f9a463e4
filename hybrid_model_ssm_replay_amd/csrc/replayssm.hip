// Host side of the C ABI declared in include/replayssm.h: argument checks,
// buffer sizing, pointer-half bookkeeping and kernel launches.  Nothing here
// allocates device memory or synchronises the host.
#include <string.h>

#include "internal.h"

using namespace rssm;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t state_elems(const replay_config &c) { return (size_t)c.batch * c.heads * c.head_dim * c.state_dim; }
size_t state_cols(const replay_config &c) { return (size_t)c.batch * c.heads * c.state_dim; }

int check_cfg(const replay_config *c) {
  if (!c) return REPLAY_EINVAL;
  if (c->kind != REPLAY_KIND_MAMBA2 && c->kind != REPLAY_KIND_GDN) return REPLAY_EINVAL;
  if (c->batch < 1 || c->heads < 1 || c->groups < 1) return REPLAY_EINVAL;
  if (c->heads % c->groups) return REPLAY_EINVAL;
  if (c->kind == REPLAY_KIND_GDN && c->groups != c->heads) return REPLAY_EINVAL;
  int waves, rbw;
  if (!tile_geometry(c->head_dim, true, &waves, &rbw)) return REPLAY_EINVAL;
  if (c->state_dim != 16 && c->state_dim != 32 && c->state_dim != 64 && c->state_dim != 128) return REPLAY_EINVAL;
  if (c->window < 1 || c->window > REPLAY_MAX_WINDOW) return REPLAY_EINVAL;
  if (c->max_draft < 0 || c->max_draft > c->window) return REPLAY_EINVAL;
  if ((int64_t)c->batch * c->heads > 0x7fffffffLL) return REPLAY_EINVAL;
  if (c->kind == REPLAY_KIND_GDN) {
    // Four waves of 16 d_v rows x RBW per head; keys at least 32 wide.
    if (c->head_dim != 64 && c->head_dim != 128) return REPLAY_EINVAL;
    if (c->state_dim < 32) return REPLAY_EINVAL;
  }
  if ((c->flags & ~(REPLAY_FLAG_DECAY_SKIP | REPLAY_FLAG_BF16_RECORDS | REPLAY_FLAG_RECORDS_IN_RING)) || c->reserved)
    return REPLAY_EINVAL;
  // The decay skip is float32-only for both families.
  if ((c->flags & REPLAY_FLAG_DECAY_SKIP) && (c->ckpt_fmt != REPLAY_FMT_F32 || c->read_fmt != REPLAY_FMT_F32))
    return REPLAY_ENOTSUP;
  if (c->ckpt_fmt < REPLAY_FMT_F32 || c->ckpt_fmt > REPLAY_FMT_F4E2M1_CS) return REPLAY_EINVAL;
  if (c->read_fmt < REPLAY_FMT_F32 || c->read_fmt > REPLAY_FMT_F4E2M1_CS) return REPLAY_EINVAL;
  if (c->ckpt_fmt == REPLAY_FMT_F32 && c->read_fmt == REPLAY_FMT_F32) return REPLAY_OK;
  // Low-precision copies: state_dim 128 (Mamba-2 also head_dim 64 or 128); the
  // read copy is e2m1 (split precision) or the checkpoint itself (one shared
  // copy); an f32 read copy next to a lower-precision checkpoint is not a
  // supported pair.
  if (c->state_dim != 128) return REPLAY_ENOTSUP;
  if (c->read_fmt != c->ckpt_fmt && c->read_fmt != REPLAY_FMT_F4E2M1_B16 && c->read_fmt != REPLAY_FMT_F4E2M1_CS)
    return REPLAY_ENOTSUP;
  // The two-axis copy is a read copy only: it never carries the recurrence.
  if (c->ckpt_fmt == REPLAY_FMT_F4E2M1_CS) return REPLAY_ENOTSUP;
  if (c->kind == REPLAY_KIND_MAMBA2) {
    // Mamba-2: block-scaled e2m1 read copy only (the two-axis encoder is the
    // GDN tile's), and no decay skip or zero-copy append with low precision.
    if (c->head_dim != 64 && c->head_dim != 128) return REPLAY_ENOTSUP;
    if (c->read_fmt == REPLAY_FMT_F4E2M1_CS) return REPLAY_ENOTSUP;
    if (c->flags & (REPLAY_FLAG_DECAY_SKIP | REPLAY_FLAG_RECORDS_IN_RING)) return REPLAY_ENOTSUP;
  }
  return REPLAY_OK;
}

int check_ctx(const replay_ctx *ctx) {
  if (!ctx || ctx->magic != kCtxMagic) return REPLAY_EINVAL;
  return REPLAY_OK;
}

Shape shape_of(const replay_config &c) {
  return make_shape(c.batch, c.heads, c.groups, c.head_dim, c.state_dim, c.window, ring_slots(c));
}

PtrHalves halves(const replay_ctx &ctx) {
  const int B = ctx.cfg.batch;
  int32_t *cur = ctx.buf.pointers + (size_t)(ctx.parity & 1) * 2 * B;
  int32_t *nxt = ctx.buf.pointers + (size_t)((ctx.parity & 1) ^ 1) * 2 * B;
  return PtrHalves{cur, cur + B, nxt, nxt + B};
}

M2Ring m2_ring(const replay_ctx &ctx) {
  const RingLayout lay = ring_layout(ctx.cfg);
  char *base = (char *)ctx.buf.ring;
  return M2Ring{(float *)(base + lay.off[0]), (float *)(base + lay.off[1]), (float *)(base + lay.off[2])};
}

GdnRing gdn_ring(const replay_ctx &ctx) {
  const RingLayout lay = ring_layout(ctx.cfg);
  char *base = (char *)ctx.buf.ring;
  return GdnRing{(float *)(base + lay.off[0]), (float *)(base + lay.off[1]), (float *)(base + lay.off[2]),
                 (float *)(base + lay.off[3]), gdn_refold(ctx.cfg) ? (float *)(base + lay.off[4]) : nullptr};
}

FormatBufs formats(const replay_ctx &ctx) {
  const replay_config &c = ctx.cfg;
  const size_t n = state_elems(c);
  FormatBufs f{};
  f.ckpt_fmt = c.ckpt_fmt;
  f.read_fmt = c.read_fmt;
  f.seed = c.seed;
  f.ckpt = ctx.buf.ckpt;
  f.ckpt_scales = c.ckpt_fmt == REPLAY_FMT_F4E2M1_B16 ? (uint8_t *)ctx.buf.ckpt + e2m1_scale_offset(n) : nullptr;
  if (c.read_fmt == c.ckpt_fmt) {
    f.read = f.ckpt;
    f.read_scales = f.ckpt_scales;
  } else {
    f.read = ctx.buf.read_copy;
    const bool e2m1 = c.read_fmt == REPLAY_FMT_F4E2M1_B16 || c.read_fmt == REPLAY_FMT_F4E2M1_CS;
    f.read_scales = e2m1 ? (uint8_t *)ctx.buf.read_copy + e2m1_scale_offset(n) : nullptr;
    f.read_cols = c.read_fmt == REPLAY_FMT_F4E2M1_CS ? (int8_t *)ctx.buf.read_copy + e2m1_cols_offset(n) : nullptr;
  }
  return f;
}

int hip_status(int e) { return e == 0 ? REPLAY_OK : REPLAY_EHIP; }

// The fields a call reads from its record argument are present and aligned;
// with the records in the ring only Mamba-2 C and GDN q, v are read.
bool rec_ok(const replay_record *r, int kind, bool in_ring = false) {
  if (!r) return false;
  if (in_ring) {
    if (kind == REPLAY_KIND_MAMBA2) return r->f2 && aligned16(r->f2);
    return r->f0 && r->f2 && aligned16(r->f0) && aligned16(r->f2);
  }
  if (!r->f0 || !r->f1 || !r->f2 || !r->f3) return false;
  if (kind == REPLAY_KIND_GDN && !r->f4) return false;
  return aligned16(r->f0) && aligned16(r->f1) && aligned16(r->f2);
}

}  // namespace

extern "C" {

int replay_validate_config(const replay_config *cfg) { return check_cfg(cfg); }

size_t replay_ckpt_bytes(const replay_config *c) {
  if (check_cfg(c) != REPLAY_OK) return 0;
  return state_bytes(c->ckpt_fmt, state_elems(*c), state_cols(*c));
}

size_t replay_read_copy_bytes(const replay_config *c) {
  if (check_cfg(c) != REPLAY_OK) return 0;
  return c->read_fmt == c->ckpt_fmt ? 0 : state_bytes(c->read_fmt, state_elems(*c), state_cols(*c));
}

size_t replay_ring_bytes(const replay_config *c) {
  if (check_cfg(c) != REPLAY_OK) return 0;
  return ring_layout(*c).bytes;
}

size_t replay_pointer_words(const replay_config *c) {
  if (check_cfg(c) != REPLAY_OK) return 0;
  return (size_t)4 * c->batch;
}

const char *replay_strerror(int code) {
  switch (code) {
    case REPLAY_OK: return "ok";
    case REPLAY_EINVAL: return "invalid argument";
    case REPLAY_EHIP: return "HIP launch failed";
    case REPLAY_ENOTSUP: return "unsupported configuration";
    default: return "unknown error";
  }
}

size_t replay_abi_sizeof(int which) {
  switch (which) {
    case 0: return sizeof(replay_config);
    case 1: return sizeof(replay_buffers);
    case 2: return sizeof(replay_record);
    case 3: return sizeof(replay_ctx);
    case 4: return sizeof(replay_ring_view);
    default: return 0;
  }
}

int replay_init(replay_ctx *ctx, const replay_config *cfg, const replay_buffers *buf, void *stream) {
  if (!ctx || !buf) return REPLAY_EINVAL;
  const int rc = check_cfg(cfg);
  if (rc != REPLAY_OK) return rc;
  if (!buf->ckpt || !buf->ring || !buf->pointers || !buf->status) return REPLAY_EINVAL;
  if (!aligned16(buf->ckpt) || !aligned16(buf->ring) || ((uintptr_t)buf->ring & 255u)) return REPLAY_EINVAL;
  if (!aligned16(buf->pointers)) return REPLAY_EINVAL;
  if (cfg->kind == REPLAY_KIND_MAMBA2 && (!buf->A || !buf->D)) return REPLAY_EINVAL;
  if (cfg->read_fmt != cfg->ckpt_fmt && (!buf->read_copy || ((uintptr_t)buf->read_copy & 255u))) return REPLAY_EINVAL;
  if (((uintptr_t)buf->ckpt & 255u) && cfg->ckpt_fmt != REPLAY_FMT_F32) return REPLAY_EINVAL;
  memset(ctx, 0, sizeof(*ctx));
  ctx->cfg = *cfg;
  ctx->buf = *buf;
  ctx->parity = 0;
  ctx->t_pending = 0;
  int e = launch_init_pointers(buf->pointers, (int)replay_pointer_words(cfg), buf->status, (hipStream_t)stream);
  if (e) return REPLAY_EHIP;
  if (cfg->ckpt_fmt == REPLAY_FMT_F32 && cfg->read_fmt != REPLAY_FMT_F32) {
    // The read copy starts as the encoding of the initial float32 checkpoint.
    EncodeArgs a{};
    a.s = shape_of(*cfg);
    a.src = (const float *)buf->ckpt;
    a.ckpt_pos = buf->pointers;  // half 0: all zero after the init kernel
    a.write_ckpt = 0;
    e = launch_encode_state(a, formats(*ctx), (hipStream_t)stream);
    if (e) return REPLAY_EHIP;
  }
  ctx->magic = kCtxMagic;
  return REPLAY_OK;
}

int replay_set_state(replay_ctx *ctx, const float *state, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK || !state || !aligned16(state)) return REPLAY_EINVAL;
  const replay_config &c = ctx->cfg;
  if (c.kind == REPLAY_KIND_MAMBA2 && c.ckpt_fmt == REPLAY_FMT_F32 && c.read_fmt == REPLAY_FMT_F32) {
    const hipError_t e = hipMemcpyAsync(ctx->buf.ckpt, state, state_elems(c) * sizeof(float),
                                        hipMemcpyDeviceToDevice, (hipStream_t)stream);
    return e == hipSuccess ? REPLAY_OK : REPLAY_EHIP;
  }
  EncodeArgs a{};
  a.s = shape_of(c);
  a.src = state;
  a.ckpt_pos = halves(*ctx).ckpt_in;
  a.write_ckpt = 1;
  return hip_status(launch_encode_state(a, formats(*ctx), (hipStream_t)stream));
}

int replay_ring_fields(const replay_ctx *ctx, replay_ring_view *view) {
  if (check_ctx(ctx) != REPLAY_OK || !view || !records_in_ring(ctx->cfg)) return REPLAY_EINVAL;
  const RingLayout lay = ring_layout(ctx->cfg);
  char *base = (char *)ctx->buf.ring;
  *view = replay_ring_view{};
  view->slots = ring_slots(ctx->cfg);
  if (ctx->cfg.kind == REPLAY_KIND_MAMBA2) {
    view->f[0] = base + lay.off[0];
    view->f[1] = base + lay.off[1];
    view->f[3] = base + lay.off[2];
  } else {
    view->f[1] = base + lay.off[0];
    view->f[3] = base + lay.off[2];
    view->f[4] = base + lay.off[3];
  }
  return REPLAY_OK;
}

int replay_record_slots(const replay_ctx *ctx, int32_t *slots, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK || !slots || !records_in_ring(ctx->cfg)) return REPLAY_EINVAL;
  return hip_status(launch_record_slots(halves(*ctx).pos_in, ctx->cfg.batch, ring_slots(ctx->cfg), slots,
                                        (hipStream_t)stream));
}

int replay_current_pointers(const replay_ctx *ctx, const int32_t **pos, const int32_t **ckpt_pos) {
  if (check_ctx(ctx) != REPLAY_OK || !pos || !ckpt_pos) return REPLAY_EINVAL;
  const PtrHalves p = halves(*ctx);
  *pos = p.pos_in;
  *ckpt_pos = p.ckpt_in;
  return REPLAY_OK;
}

int replay_step(replay_ctx *ctx, const replay_record *rec, float *y, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK) return REPLAY_EINVAL;
  const replay_config &c = ctx->cfg;
  if (!rec_ok(rec, c.kind, records_in_ring(c)) || !y || !aligned16(y)) return REPLAY_EINVAL;
  int e;
  if (c.kind == REPLAY_KIND_MAMBA2) {
    M2StepArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.ckpt = (float *)ctx->buf.ckpt;
    a.ring = m2_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.A = ctx->buf.A;
    a.D = ctx->buf.D;
    a.x = rec->f0;
    a.Bm = rec->f1;
    a.Cm = rec->f2;
    a.dt = rec->f3;
    a.bf16 = bf16_records(c);
    a.in_ring = records_in_ring(c) ? 1 : 0;
    a.y = y;
    e = launch_m2_step(a, formats(*ctx), (hipStream_t)stream);
  } else {
    GdnStepArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.ring = gdn_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.q = rec->f0;
    a.k = rec->f1;
    a.v = rec->f2;
    a.alpha = rec->f3;
    a.beta = rec->f4;
    a.bf16 = bf16_records(c);
    a.in_ring = records_in_ring(c) ? 1 : 0;
    a.y = y;
    e = launch_gdn_step(a, formats(*ctx), (hipStream_t)stream);
  }
  if (e) return REPLAY_EHIP;
  ctx->parity ^= 1;
  ctx->t_pending = 0;
  return REPLAY_OK;
}

int replay_flush(replay_ctx *ctx, const uint8_t *seq_mask, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK) return REPLAY_EINVAL;
  const replay_config &c = ctx->cfg;
  int e;
  if (c.kind == REPLAY_KIND_MAMBA2) {
    M2FlushArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.ckpt = (float *)ctx->buf.ckpt;
    a.ring = m2_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.A = ctx->buf.A;
    a.mask = seq_mask;
    a.bf16 = bf16_records(c);
    e = launch_m2_flush(a, formats(*ctx), (hipStream_t)stream);
  } else {
    GdnFlushArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.ring = gdn_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.mask = seq_mask;
    a.bf16 = bf16_records(c);
    e = launch_gdn_flush(a, formats(*ctx), (hipStream_t)stream);
  }
  if (e) return REPLAY_EHIP;
  ctx->parity ^= 1;
  ctx->t_pending = 0;  // a flush discards pending drafts, like a step or a verify
  return REPLAY_OK;
}

int replay_verify(replay_ctx *ctx, int32_t T, const replay_record *drafts, float *y, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK) return REPLAY_EINVAL;
  const replay_config &c = ctx->cfg;
  if (T < 1 || T > c.max_draft || T > c.window) return REPLAY_EINVAL;
  if (!rec_ok(drafts, c.kind, records_in_ring(c)) || !y || !aligned16(y)) return REPLAY_EINVAL;
  int e;
  if (c.kind == REPLAY_KIND_MAMBA2) {
    M2VerifyArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.T = T;
    a.ckpt = (float *)ctx->buf.ckpt;
    a.ring = m2_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.A = ctx->buf.A;
    a.D = ctx->buf.D;
    a.x = drafts->f0;
    a.Bm = drafts->f1;
    a.Cm = drafts->f2;
    a.dt = drafts->f3;
    a.bf16 = bf16_records(c);
    a.in_ring = records_in_ring(c) ? 1 : 0;
    a.y = y;
    e = launch_m2_verify(a, formats(*ctx), (hipStream_t)stream);
  } else {
    GdnVerifyArgs a{};
    a.s = shape_of(c);
    a.decay_skip = (c.flags & REPLAY_FLAG_DECAY_SKIP) ? 1 : 0;
    a.T = T;
    a.ring = gdn_ring(*ctx);
    a.ptr = halves(*ctx);
    a.status = ctx->buf.status;
    a.q = drafts->f0;
    a.k = drafts->f1;
    a.v = drafts->f2;
    a.alpha = drafts->f3;
    a.beta = drafts->f4;
    a.bf16 = bf16_records(c);
    a.in_ring = records_in_ring(c) ? 1 : 0;
    a.y = y;
    e = launch_gdn_verify(a, formats(*ctx), (hipStream_t)stream);
  }
  if (e) return REPLAY_EHIP;
  ctx->parity ^= 1;
  ctx->t_pending = T;
  return REPLAY_OK;
}

int replay_commit(replay_ctx *ctx, const int32_t *accepted, void *stream) {
  if (check_ctx(ctx) != REPLAY_OK || !accepted) return REPLAY_EINVAL;
  const int e = launch_commit(halves(*ctx), ctx->cfg.batch, accepted, ctx->t_pending, ctx->buf.status,
                              (hipStream_t)stream);
  if (e) return REPLAY_EHIP;
  ctx->parity ^= 1;
  ctx->t_pending = 0;
  return REPLAY_OK;
}

int replay_conv_step(const replay_config *cfg, float *state, const float *A, const float *D,
                     const replay_record *rec, float *y, void *stream) {
  const int rc = check_cfg(cfg);
  if (rc != REPLAY_OK) return rc;
  if (!state || !aligned16(state) || !rec_ok(rec, cfg->kind) || !y || !aligned16(y)) return REPLAY_EINVAL;
  if (cfg->kind == REPLAY_KIND_MAMBA2) {
    if (!A || !D) return REPLAY_EINVAL;
    M2ConvArgs a{};
    a.s = shape_of(*cfg);
    a.state = state;
    a.A = A;
    a.D = D;
    a.x = rec->f0;
    a.Bm = rec->f1;
    a.Cm = rec->f2;
    a.dt = rec->f3;
    a.bf16 = bf16_records(*cfg);
    a.y = y;
    return hip_status(launch_m2_conv(a, (hipStream_t)stream));
  }
  GdnConvArgs a{};
  a.s = shape_of(*cfg);
  a.state = state;
  a.q = rec->f0;
  a.k = rec->f1;
  a.v = rec->f2;
  a.alpha = rec->f3;
  a.beta = rec->f4;
  a.bf16 = bf16_records(*cfg);
  a.y = y;
  return hip_status(launch_gdn_conv(a, (hipStream_t)stream));
}

int replay_snapshot_verify(const replay_config *cfg, float *slots, const int32_t *cur, int32_t T,
                           const float *A, const float *D, const replay_record *drafts, float *y,
                           void *stream) {
  const int rc = check_cfg(cfg);
  if (rc != REPLAY_OK) return rc;
  if (T < 1 || T > cfg->max_draft) return REPLAY_EINVAL;
  if (!slots || !aligned16(slots) || !cur || !rec_ok(drafts, cfg->kind) || !y || !aligned16(y)) return REPLAY_EINVAL;
  if (cfg->kind == REPLAY_KIND_MAMBA2) {
    if (!A || !D) return REPLAY_EINVAL;
    M2SnapArgs a{};
    a.s = shape_of(*cfg);
    a.T = T;
    a.nslots = cfg->max_draft + 1;
    a.slots = slots;
    a.cur = cur;
    a.A = A;
    a.D = D;
    a.x = drafts->f0;
    a.Bm = drafts->f1;
    a.Cm = drafts->f2;
    a.dt = drafts->f3;
    a.bf16 = bf16_records(*cfg);
    a.y = y;
    return hip_status(launch_m2_snapshot(a, (hipStream_t)stream));
  }
  GdnSnapArgs a{};
  a.s = shape_of(*cfg);
  a.T = T;
  a.nslots = cfg->max_draft + 1;
  a.slots = slots;
  a.cur = cur;
  a.q = drafts->f0;
  a.k = drafts->f1;
  a.v = drafts->f2;
  a.alpha = drafts->f3;
  a.beta = drafts->f4;
  a.bf16 = bf16_records(*cfg);
  a.y = y;
  return hip_status(launch_gdn_snapshot(a, (hipStream_t)stream));
}

int replay_snapshot_commit(const replay_config *cfg, int32_t *cur, const int32_t *accepted, int32_t T,
                           void *stream) {
  const int rc = check_cfg(cfg);
  if (rc != REPLAY_OK) return rc;
  if (!cur || !accepted || T < 0 || T > cfg->max_draft) return REPLAY_EINVAL;
  return hip_status(launch_snapshot_commit(cur, accepted, cfg->batch, T, cfg->max_draft + 1, (hipStream_t)stream));
}

int replay_hbm_probe(const void *src, void *dst, size_t bytes, int mode, void *stream) {
  if (!src || !dst || (bytes & 15) || (mode != 0 && mode != 1)) return REPLAY_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return REPLAY_EINVAL;
  return hip_status(launch_probe(src, dst, bytes, mode, (hipStream_t)stream));
}

}  // extern "C"
