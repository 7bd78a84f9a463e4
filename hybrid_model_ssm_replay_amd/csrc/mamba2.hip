// Mamba-2 replay decode kernels for gfx950.
//
// Tile = one (sequence, head): the head's P x N float32 checkpoint.  Each wave
// owns RBW blocks of 16 rows.  Register layout of the checkpoint, shared by
// every kernel here: lane l holds, for row block k and column chunk c,
//     s[k][c] = S[16 * rb + (l % 16)][16 * c + 4 * (l / 16) + 0..3]
// (one 16-byte load per lane; rb = wave * RBW + k).  The same layout is
//   - the A operand of v_mfma_f32_16x16x4f32 with K running over the four
//     elements of the float4 (used by verify's S0 . [C_1 .. C_T]), and
//   - the accumulator layout of that MFMA for the transposed fold
//     S^T = e^{...} S0^T + B^T X~^T (M = state column, N = row, K = record),
// so the fold result never leaves registers before it is stored.
//
// Replay identities (derived from the Mamba-2 decode recurrence
// S <- exp(dt A) S + dt x B^T, y = S C + D x by unrolling the window; the
// method keeps a checkpoint plus the recent inputs [P1, Synopsis; P2,
// paragraph 3; P3, Interpretation 2]):
//   y_m   = exp(A s_{1..m}) S0 C_m + sum_j exp(A s_{j+1..m}) dt_j (B_j . C_m) x_j + D x_m
//   S_new = exp(A s_{1..L}) S0 + sum_j exp(A s_{j+1..L}) dt_j x_j B_j^T
// where s_{a..b} is the sum of dt over records a..b.  Decays are formed from
// these segment sums directly (never as ratios of cumulative decays, which
// underflow for fast-decaying heads).
#include "internal.h"

namespace rssm {
namespace {

template <int NCH>
struct M2Smem {
  float Bs[kMaxL][16 * NCH + 16];  // fold: B records (rows padded: conflict-free MFMA operand reads)
  float dot[kMaxL];                // step: B_r . C
  float dt[kMaxL];                 // verify: dt of window records
  float dots[kMaxL][kMaxL];        // verify: [record][draft] B_r . C_draft
  float coef[kMaxL][kMaxL];        // verify: [draft][record] output weight
  float scale[kMaxL];              // verify: [draft] weight of S0 . C
};

struct TileCtx {
  int tid, lane, wave, nthreads, q, r16;
};

__device__ __forceinline__ TileCtx tile_ctx() {
  TileCtx t;
  t.tid = threadIdx.x;
  t.lane = t.tid & 63;
  t.wave = t.tid >> 6;
  t.nthreads = blockDim.x;
  t.q = t.lane >> 4;
  t.r16 = t.lane & 15;
  return t;
}

template <int NCH, int RBW>
__device__ __forceinline__ void load_tile(float4 (&s)[RBW][NCH], const float *S, const TileCtx &t) {
  constexpr int N = 16 * NCH;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (t.wave * RBW + k) * 16 + t.r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s[k][c] = ld4(S + (size_t)row * N + 16 * c + 4 * t.q);
  }
}

template <int NCH, int RBW>
__device__ __forceinline__ void store_tile(const float4 (&s)[RBW][NCH], float *S, const TileCtx &t) {
  constexpr int N = 16 * NCH;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (t.wave * RBW + k) * 16 + t.r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) st4(S + (size_t)row * N + 16 * c + 4 * t.q, s[k][c]);
  }
}

// Exclusive suffix sum over lanes 0..15 of a wave: returns sum_{i > lane} v_i
// (lanes 0..15), and the total in *total (every lane).  Lanes >= 16 must pass 0.
__device__ __forceinline__ float suffix_sum16(float v, int lane, float *total) {
  float t = v;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const float u = __shfl_down(t, off, kWave);
    if (lane + off < 16) t += u;
  }
  *total = __shfl(t, 0, kWave);
  const float nxt = __shfl_down(t, 1, kWave);
  return lane < 15 ? nxt : 0.f;
}

// Fold the cnt (1..L) committed records at positions base .. base+cnt-1 into
// the register tile: s <- exp(A s_{1..cnt}) s + sum_r exp(A s_{r+1..cnt}) dt_r x_r B_r^T.
// Ends with a barrier; sm.Bs is free again afterwards.
template <int NCH, int RBW>
__device__ __forceinline__ void fold_tile(float4 (&s)[RBW][NCH], M2Smem<NCH> &sm, int cnt, int base,
                                          float Ah, const float *rx, const float *rdt, const float *rB,
                                          int L, int P, const TileCtx &t) {
  constexpr int N = 16 * NCH;
  // Stage B_r (cnt x N) in LDS; zero the rows up to the next multiple of 4.
  const int rows4 = (cnt + 3) & ~3;
  for (int e = 4 * t.tid; e < rows4 * N; e += 4 * t.nthreads) {
    const int r = e / N, n = e - r * N;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < cnt) v = ld4(rB + (size_t)((base + r) % (2 * L)) * N + n);
    *reinterpret_cast<float4 *>(&sm.Bs[r][n]) = v;
  }
  // Decay weights, per wave, record r in lane r.
  const float dtv = t.lane < cnt ? rdt[(base + t.lane) % L] : 0.f;
  float total;
  const float seg = suffix_sum16(dtv, t.lane, &total);
  const float f = __expf(Ah * seg) * dtv;
  const float scale = __expf(Ah * total);
  lds_barrier();
  const int nsteps = rows4 >> 2;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (t.wave * RBW + k) * 16 + t.r16;
    float xb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r = 4 * st + t.q;
      const float fr = __shfl(f, r, kWave);
      xb[st] = (r < cnt) ? fr * rx[(size_t)((base + r) % L) * P + row] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 acc = {s[k][c].x * scale, s[k][c].y * scale, s[k][c].z * scale, s[k][c].w * scale};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < nsteps) acc = mfma_16x16x4(sm.Bs[4 * st + t.q][16 * c + t.r16], xb[st], acc);
      }
      s[k][c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
  __syncthreads();
}

// ---- replay step ----------------------------------------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void m2_replay_step(M2StepArgs a) {
  constexpr int N = 16 * NCH;
  __shared__ M2Smem<NCH> sm;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / sh.H, h = tile - b * sh.H;
  const int hpg = sh.H / sh.G, g = h / hpg;
  const int P = sh.P, L = sh.L;

  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  if (count < 0 || count > L) {
    if (h == 0 && t.tid == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  const bool fold = count == L;
  float *S = a.ckpt + ((size_t)b * sh.H + h) * P * N;
  float4 s[RBW][NCH];
  load_tile<NCH, RBW>(s, S, t);

  const float Ah = a.A[h];
  float *rx = a.ring.x + ((size_t)b * sh.H + h) * L * P;
  float *rdt = a.ring.dt + ((size_t)b * sh.H + h) * L;
  float *rB = a.ring.Bm + ((size_t)b * sh.G + g) * 2 * L * N;
  const float *xin = a.x + ((size_t)b * sh.H + h) * P;
  const float *Bin = a.Bm + ((size_t)b * sh.G + g) * N;
  const float *Cin = a.Cm + ((size_t)b * sh.G + g) * N;
  const float dt_in = a.dt[(size_t)b * sh.H + h];

  int base = ck;
  if (fold) {
    fold_tile<NCH, RBW>(s, sm, L, ck, Ah, rx, rdt, rB, L, P, t);
    store_tile<NCH, RBW>(s, S, t);
    base = pos;
  }
  const int m = pos - base + 1;  // window records including this token (1..L)

  // dt of the window, record r in lane r; segment sums for the decays.
  const float dtv = t.lane < m - 1 ? rdt[(base + t.lane) % L] : (t.lane == m - 1 ? dt_in : 0.f);
  float total;
  const float seg = suffix_sum16(dtv, t.lane, &total);

  // B_r . C for every window record: 16 lanes per record, 4 records per wave pass.
  for (int r0 = 4 * t.wave; r0 < m; r0 += 4 * (t.nthreads >> 6)) {
    const int r = r0 + t.q;
    float part = 0.f;
    if (r < m) {
      const float *Br = (r == m - 1) ? Bin : rB + (size_t)((base + r) % (2 * L)) * N;
#pragma unroll
      for (int i = 0; i < NCH; ++i) part += Br[t.r16 + 16 * i] * Cin[t.r16 + 16 * i];
    }
    part = sum16(part);
    if (t.r16 == 0 && r < m) sm.dot[r] = part;
  }
  lds_barrier();
  const float w = t.lane < m ? __expf(Ah * seg) * dtv * sm.dot[t.lane] : 0.f;
  const float scale = __expf(Ah * total);
  const float Dh = a.D[h];

  float4 cv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) cv[c] = ld4(Cin + 16 * c + 4 * t.q);
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (t.wave * RBW + k) * 16 + t.r16;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc += dot4(s[k][c], cv[c]);
    acc *= scale;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r = 4 * st + t.q;
      const float wr = __shfl(w, r, kWave);
      if (r < m) {
        const float xv = (r == m - 1) ? xin[row] : rx[(size_t)((base + r) % L) * P + row];
        acc += wr * xv;
      }
    }
    acc = sum_quarters(acc);
    if (t.q == 0) a.y[((size_t)b * sh.H + h) * P + row] = acc + Dh * xin[row];
  }

  // Append this token's record.  After a fold the slot of x / dt being written
  // held the oldest folded record: wait until every wave has consumed it.
  if (fold) __syncthreads();
  const int slot = pos % L;
  for (int i = t.tid; i < P; i += t.nthreads) rx[(size_t)slot * P + i] = xin[i];
  if (t.tid == 0) rdt[slot] = dt_in;
  if (h % hpg == 0)
    for (int i = t.tid; i < N; i += t.nthreads) rB[(size_t)(pos % (2 * L)) * N + i] = Bin[i];
  if (h == 0 && t.tid == 0) {
    a.ptr.pos_out[b] = pos + 1;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- explicit flush ---------------------------------------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void m2_flush(M2FlushArgs a) {
  constexpr int N = 16 * NCH;
  __shared__ M2Smem<NCH> sm;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / sh.H, h = tile - b * sh.H;
  const int g = h / (sh.H / sh.G);
  const int P = sh.P, L = sh.L;
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  const bool bad = count < 0 || count > L;
  const bool fold = !bad && count > 0 && (a.mask == nullptr || a.mask[b] != 0);
  if (h == 0 && t.tid == 0) {
    if (bad) atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = fold ? pos : ck;
  }
  if (!fold) return;
  float *S = a.ckpt + ((size_t)b * sh.H + h) * P * N;
  float4 s[RBW][NCH];
  load_tile<NCH, RBW>(s, S, t);
  const float *rx = a.ring.x + ((size_t)b * sh.H + h) * L * P;
  const float *rdt = a.ring.dt + ((size_t)b * sh.H + h) * L;
  const float *rB = a.ring.Bm + ((size_t)b * sh.G + g) * 2 * L * N;
  fold_tile<NCH, RBW>(s, sm, count, ck, a.A[h], rx, rdt, rB, L, P, t);
  store_tile<NCH, RBW>(s, S, t);
}

// ---- speculative verify -------------------------------------------------
// T drafts follow the c committed window records.  Outputs for draft i
// (window record c + i):
//   y_i = exp(A s_{1..c+i}) S0 C_i + sum_{r <= c+i} exp(A s_{r+1..c+i}) dt_r (B_r . C_i) x_r + D x_{c+i}
// S0 . [C_0 .. C_{T-1}] and the B_r . C_i table are MFMA products; no state
// is written except by a fold-first when c + T > L.
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void m2_replay_verify(M2VerifyArgs a) {
  constexpr int N = 16 * NCH;
  __shared__ M2Smem<NCH> sm;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int T = a.T;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / sh.H, h = tile - b * sh.H;
  const int hpg = sh.H / sh.G, g = h / hpg;
  const int P = sh.P, L = sh.L, H = sh.H, G = sh.G;

  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  if (count < 0 || count > L) {
    if (h == 0 && t.tid == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  const bool fold = count + T > L;  // implies count >= 1 because T <= L
  float *S = a.ckpt + ((size_t)b * H + h) * P * N;
  float4 s[RBW][NCH];
  load_tile<NCH, RBW>(s, S, t);
  const float Ah = a.A[h];
  float *rx = a.ring.x + ((size_t)b * H + h) * L * P;
  float *rdt = a.ring.dt + ((size_t)b * H + h) * L;
  float *rB = a.ring.Bm + ((size_t)b * G + g) * 2 * L * N;
  int base = ck;
  if (fold) {
    fold_tile<NCH, RBW>(s, sm, count, ck, Ah, rx, rdt, rB, L, P, t);
    store_tile<NCH, RBW>(s, S, t);
    base = pos;
  }
  const int c = pos - base;  // committed records in the window
  const int nrec = c + T;    // <= L

  auto draft_x = [&](int i) { return a.x + (((size_t)b * T + i) * H + h) * P; };
  auto draft_B = [&](int i) { return a.Bm + (((size_t)b * T + i) * G + g) * N; };
  auto draft_C = [&](int i) { return a.Cm + (((size_t)b * T + i) * G + g) * N; };
  auto rec_B = [&](int r) -> const float * {
    return r < c ? rB + (size_t)((base + r) % (2 * L)) * N : draft_B(r - c);
  };

  // C of draft r16 at this lane's columns (zero for lanes without a draft).
  float4 cd[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc)
    cd[cc] = t.r16 < T ? ld4(draft_C(t.r16) + 16 * cc + 4 * t.q) : make_float4(0.f, 0.f, 0.f, 0.f);

  if (t.wave == 0) {
    // dt of the window records.
    if (t.lane < nrec)
      sm.dt[t.lane] = t.lane < c ? rdt[(base + t.lane) % L] : a.dt[((size_t)b * T + (t.lane - c)) * H + h];
    // dots[r][i] = B_r . C_i: M = record, N = draft, K = state column.
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const float *Br = t.r16 < nrec ? rec_B(t.r16) : nullptr;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const float4 bv = Br ? ld4(Br + 16 * cc + 4 * t.q) : make_float4(0.f, 0.f, 0.f, 0.f);
      acc = mfma_16x16x4(bv.x, cd[cc].x, acc);
      acc = mfma_16x16x4(bv.y, cd[cc].y, acc);
      acc = mfma_16x16x4(bv.z, cd[cc].z, acc);
      acc = mfma_16x16x4(bv.w, cd[cc].w, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.dots[4 * t.q + i][t.r16] = acc[i];
  }
  lds_barrier();
  {
    // coef[i][r] for draft i = tid / 16, record r = tid % 16.
    const int i = t.tid >> 4, r = t.tid & 15;
    if (i < T) {
      const int last = c + i;
      float cf = 0.f;
      if (r <= last) {
        float sg = 0.f;
        for (int j = r + 1; j <= last; ++j) sg += sm.dt[j];
        cf = __expf(Ah * sg) * sm.dt[r] * sm.dots[r][i];
      }
      sm.coef[i][r] = cf;
      if (r == 0) {
        float tot = 0.f;
        for (int j = 0; j <= last; ++j) tot += sm.dt[j];
        sm.scale[i] = __expf(Ah * tot);
      }
    }
  }
  lds_barrier();

  const float Dh = a.D[h];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int rb = t.wave * RBW + k;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      acc = mfma_16x16x4(s[k][cc].x, cd[cc].x, acc);
      acc = mfma_16x16x4(s[k][cc].y, cd[cc].y, acc);
      acc = mfma_16x16x4(s[k][cc].z, cd[cc].z, acc);
      acc = mfma_16x16x4(s[k][cc].w, cd[cc].w, acc);
    }
    // Lane holds rows p0 .. p0+3 of draft i.
    const int i = t.r16;
    if (i < T) {
      const int p0 = rb * 16 + 4 * t.q;
      const float sc = sm.scale[i];
      float4 o = make_float4(sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
      for (int r = 0; r <= c + i; ++r) {
        const float cf = sm.coef[i][r];
        const float4 xv = ld4(r < c ? rx + (size_t)((base + r) % L) * P + p0 : draft_x(r - c) + p0);
        o.x += cf * xv.x;
        o.y += cf * xv.y;
        o.z += cf * xv.z;
        o.w += cf * xv.w;
      }
      const float4 xl = ld4(draft_x(i) + p0);
      o.x += Dh * xl.x;
      o.y += Dh * xl.y;
      o.z += Dh * xl.z;
      o.w += Dh * xl.w;
      st4(a.y + (((size_t)b * T + i) * H + h) * P + p0, o);
    }
  }

  // Stage the drafts in the ring (after every wave is done with the folded slots).
  __syncthreads();
  for (int e = t.tid; e < T * P; e += t.nthreads) {
    const int i = e / P, p = e - i * P;
    rx[(size_t)((pos + i) % L) * P + p] = draft_x(i)[p];
  }
  if (t.tid < T) rdt[(pos + t.tid) % L] = a.dt[((size_t)b * T + t.tid) * H + h];
  if (h % hpg == 0)
    for (int e = t.tid; e < T * N; e += t.nthreads) {
      const int i = e / N, n = e - i * N;
      rB[(size_t)((pos + i) % (2 * L)) * N + n] = draft_B(i)[n];
    }
  if (h == 0 && t.tid == 0) {
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- baseline: conventional load-update-store step -------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void m2_conv_step(M2ConvArgs a) {
  constexpr int N = 16 * NCH;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / sh.H, h = tile - b * sh.H;
  const int g = h / (sh.H / sh.G);
  const int P = sh.P;
  float *S = a.state + ((size_t)b * sh.H + h) * P * N;
  float4 s[RBW][NCH];
  load_tile<NCH, RBW>(s, S, t);
  const float dt = a.dt[(size_t)b * sh.H + h];
  const float decay = __expf(dt * a.A[h]);
  const float Dh = a.D[h];
  const float *xin = a.x + ((size_t)b * sh.H + h) * P;
  const float *Bin = a.Bm + ((size_t)b * sh.G + g) * N;
  const float *Cin = a.Cm + ((size_t)b * sh.G + g) * N;
  float4 bv[NCH], cv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    bv[c] = ld4(Bin + 16 * c + 4 * t.q);
    cv[c] = ld4(Cin + 16 * c + 4 * t.q);
  }
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (t.wave * RBW + k) * 16 + t.r16;
    const float xv = xin[row];
    const float dx = dt * xv;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float4 &v = s[k][c];
      v.x = decay * v.x + dx * bv[c].x;
      v.y = decay * v.y + dx * bv[c].y;
      v.z = decay * v.z + dx * bv[c].z;
      v.w = decay * v.w + dx * bv[c].w;
      acc += dot4(v, cv[c]);
    }
    acc = sum_quarters(acc);
    if (t.q == 0) a.y[((size_t)b * sh.H + h) * P + row] = acc + Dh * xv;
  }
  store_tile<NCH, RBW>(s, S, t);
}

// ---- baseline: snapshot-per-draft verify -----------------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void m2_snapshot_verify(M2SnapArgs a) {
  constexpr int N = 16 * NCH;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int T = a.T, H = sh.H, G = sh.G, P = sh.P;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / H, h = tile - b * H;
  const int g = h / (H / G);
  const int cur = a.cur[b];
  if (cur < 0 || cur >= a.nslots) return;  // never index outside the slot array
  const size_t head_elems = (size_t)P * N;
  auto slot_ptr = [&](int sl) { return a.slots + (((size_t)b * a.nslots + sl) * H + h) * head_elems; };
  float4 s[RBW][NCH];
  load_tile<NCH, RBW>(s, slot_ptr(cur), t);
  const float Ah = a.A[h], Dh = a.D[h];
  for (int i = 0; i < T; ++i) {
    const float dt = a.dt[((size_t)b * T + i) * H + h];
    const float decay = __expf(dt * Ah);
    const float *xin = a.x + (((size_t)b * T + i) * H + h) * P;
    const float *Bin = a.Bm + (((size_t)b * T + i) * G + g) * N;
    const float *Cin = a.Cm + (((size_t)b * T + i) * G + g) * N;
    float4 bv[NCH], cv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      bv[c] = ld4(Bin + 16 * c + 4 * t.q);
      cv[c] = ld4(Cin + 16 * c + 4 * t.q);
    }
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (t.wave * RBW + k) * 16 + t.r16;
      const float xv = xin[row];
      const float dx = dt * xv;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float4 &v = s[k][c];
        v.x = decay * v.x + dx * bv[c].x;
        v.y = decay * v.y + dx * bv[c].y;
        v.z = decay * v.z + dx * bv[c].z;
        v.w = decay * v.w + dx * bv[c].w;
        acc += dot4(v, cv[c]);
      }
      acc = sum_quarters(acc);
      if (t.q == 0) a.y[(((size_t)b * T + i) * H + h) * P + row] = acc + Dh * xv;
    }
    store_tile<NCH, RBW>(s, slot_ptr((cur + 1 + i) % a.nslots), t);
  }
}

// ---- dispatch ---------------------------------------------------------------
template <template <int, int> class K, typename Args>
int dispatch(const Args &a, int N, int P, int B, int H, hipStream_t st) {
  int waves, rbw;
  if (!tile_geometry(P, &waves, &rbw)) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)B * H)), block(64 * waves);
#define RSSM_CASE(NCH_, RBW_)                                   \
  if (N == 16 * NCH_ && rbw == RBW_) {                          \
    hipLaunchKernelGGL((K<NCH_, RBW_>::fn), grid, block, 0, st, a); \
    return (int)hipGetLastError();                              \
  }
  RSSM_CASE(1, 1) RSSM_CASE(2, 1) RSSM_CASE(4, 1) RSSM_CASE(8, 1)
  RSSM_CASE(1, 2) RSSM_CASE(2, 2) RSSM_CASE(4, 2) RSSM_CASE(8, 2)
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}

#define RSSM_WRAP(name, kern)                          \
  template <int NCH, int RBW>                          \
  struct name {                                        \
    static constexpr auto fn = kern<NCH, RBW>;         \
  };
RSSM_WRAP(StepK, m2_replay_step)
RSSM_WRAP(FlushK, m2_flush)
RSSM_WRAP(VerifyK, m2_replay_verify)
RSSM_WRAP(ConvK, m2_conv_step)
RSSM_WRAP(SnapK, m2_snapshot_verify)
#undef RSSM_WRAP

}  // namespace

int launch_m2_step(const M2StepArgs &a, hipStream_t st) {
  return dispatch<StepK>(a, a.s.N, a.s.P, a.s.B, a.s.H, st);
}
int launch_m2_flush(const M2FlushArgs &a, hipStream_t st) {
  return dispatch<FlushK>(a, a.s.N, a.s.P, a.s.B, a.s.H, st);
}
int launch_m2_verify(const M2VerifyArgs &a, hipStream_t st) {
  return dispatch<VerifyK>(a, a.s.N, a.s.P, a.s.B, a.s.H, st);
}
int launch_m2_conv(const M2ConvArgs &a, hipStream_t st) {
  return dispatch<ConvK>(a, a.s.N, a.s.P, a.s.B, a.s.H, st);
}
int launch_m2_snapshot(const M2SnapArgs &a, hipStream_t st) {
  return dispatch<SnapK>(a, a.s.N, a.s.P, a.s.B, a.s.H, st);
}

}  // namespace rssm
