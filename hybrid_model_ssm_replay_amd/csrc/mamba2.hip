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
// Kernel template parameters besides the tile shape: R, the element type of the
// record vector fields and their ring copies (float, or bf16_t with bf16
// records), SKIP (the decay skip below), for the step ZC (zero-copy append: the
// caller wrote this token's x, B, dt into their ring slots, and the ring fields
// have 2L slots), and CF, RF, the formats of the checkpoint and of the read
// copy (state_io.h; float32 both by default).  With a low-precision read copy
// the column map of the register tile is contiguous per lane (colq), and the
// MFMA row index M of chunk c stands for column mcol(c, M).
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
#include "state_io.h"

namespace rssm {
namespace {

// Decay skip (REPLAY_FLAG_DECAY_SKIP): a head whose window decay exp(A s) is
// below 2^-24 drops the checkpoint term, in outputs and folds alike, and a step
// does not read its checkpoint; its fold is then a pure write of the folded
// records [P3, Perspective, paragraph 1].  The comparison is A s < ln 2^-24 in
// float32, with s the dt summed over the window records the computation uses.

// exp(A s), or 0 when the decay skip drops it.
template <bool SKIP>
__device__ __forceinline__ float s0_weight(float As) {
  return (SKIP && As < kDecaySkipLog) ? 0.f : __expf(As);
}

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

// Inclusive suffix sum within each row of 16 lanes: lane (row, i) gets
// sum_{j >= i} v_(row, j).
__device__ __forceinline__ float row_suffix_sum16(float v, int lane) {
  float t = v;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const float u = __shfl_down(t, off, kWave);
    if ((lane & 15) + off < 16) t += u;
  }
  return t;
}

// Fold the cnt (1..L) committed records at positions base .. base+cnt-1 into
// the register tile: s <- exp(A s_{1..cnt}) s + sum_r exp(A s_{r+1..cnt}) dt_r x_r B_r^T.
// Ends with a barrier; sm.Bs is free again afterwards.
template <int NCH, int RBW, bool SKIP, typename R, int CM = kColIlv>
__device__ __forceinline__ void fold_tile(float4 (&s)[RBW][NCH], M2Smem<NCH> &sm, int cnt, int base,
                                          float Ah, const R *rx, const float *rdt, const R *rB,
                                          int L, int Ls, size_t xs, const TileCtx &t) {
  constexpr int N = 16 * NCH;
  // Stage B_r (cnt x N) in LDS; zero the rows up to the next multiple of 4.
  const int rows4 = (cnt + 3) & ~3;
  for (int e = 4 * t.tid; e < rows4 * N; e += 4 * t.nthreads) {
    const int r = e / N, n = e - r * N;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < cnt) v = ldr4<R>(rB + (size_t)((base + r) % (2 * L)) * N + n);
    *reinterpret_cast<float4 *>(&sm.Bs[r][n]) = v;
  }
  // Decay weights, per wave, record r in lane r.
  const float dtv = t.lane < cnt ? rdt[(base + t.lane) % Ls] : 0.f;
  float total;
  const float seg = suffix_sum16(dtv, t.lane, &total);
  const float f = __expf(Ah * seg) * dtv;
  const float scale = s0_weight<SKIP>(Ah * total);
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
      xb[st] = (r < cnt) ? fr * ldr<R>(rx + (size_t)((base + r) % Ls) * xs + row) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 acc = {s[k][c].x * scale, s[k][c].y * scale, s[k][c].z * scale, s[k][c].w * scale};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < nsteps) acc = mfma_16x16x4(sm.Bs[4 * st + t.q][mcol<NCH, CM>(c, t.r16)], xb[st], acc);
      }
      s[k][c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
  __syncthreads();
}

// ---- replay step ---------------------------------------------------------------
// The head's checkpoint lives in registers: each wave holds RBW row blocks of
// 16 rows, and a head takes P / (16 RBW) waves (two at P = 64).  Every load
// that does not depend on the pointers is issued first, so the checkpoint
// stream is in flight while the pointers, then the ring records, arrive.  No
// workgroup barrier on the non-fold path (a barrier there costs more than any
// LDS sharing it would allow): each wave stages what it reads of C and B in
// its own LDS region.
//
// Lane (r16, q) roles:  checkpoint rows 16 rb + r16, columns 16 c + 4 q + 0..3;
// for the B_j . C dots lane r16 stands for window record j = r16 and sums over
// the same columns as its checkpoint slice, reading the same C chunks from LDS
// for both products.

// Fold the cnt committed records at positions base.. into the register tile,
// wave-locally: s <- exp(A s_{1..cnt}) s + sum_r exp(A s_{r+1..cnt}) dt_r x_r B_r^T.
// Split in two so that callers can issue the record loads before the
// checkpoint stream: fold_load reads the records, fold_apply does the MFMAs.
template <int NCH, int RBW>
struct FoldIn {
  float f;             // lanes 0..15: exp(A s_{r+1..cnt}) dt_r for record r = lane
  float scale;         // exp(A s_{1..cnt})
  float aB[NCH][4];    // MFMA A operand: B_{4 st + q}[mcol(c, r16)]
  float xraw[4][RBW];  // x_{4 st + q}[row of block k]
  int nsteps;          // ceil(cnt / 4)
};

template <int NCH, int RBW, typename R, int CM = kColIlv>
__device__ __forceinline__ void fold_load(FoldIn<NCH, RBW> &fi, int cnt, int s0, int s0b, const R *rx,
                                          const float *rdt, const R *rB, int L, int Ls, size_t xs, int rb0,
                                          int lane) {
  // s0 = (position of record 0) mod Ls (x and dt slots), s0b = the same mod 2 L (B slots);
  // xs = x-ring slot stride.
  const int q = lane >> 4, r16 = lane & 15;
  const float dtl = rdt[wrap(s0, r16 < cnt ? r16 : cnt - 1, Ls)];
  fi.f = lane < cnt ? dtl : 0.f;  // dt for now; fold_apply turns it into the weight
  fi.nsteps = (cnt + 3) >> 2;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int r = 4 * st + q;
    const int rc = r < cnt ? r : cnt - 1;
    const R *Br = rB + wrap(s0b, rc, 2 * L) * (16 * NCH);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float v = ldr<R>(Br + mcol<NCH, CM>(c, r16));
      fi.aB[c][st] = r < cnt ? v : 0.f;
    }
    const R *xr = rx + wrap(s0, rc, Ls) * xs;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const float v = ldr<R>(xr + (rb0 + k) * 16 + r16);
      fi.xraw[st][k] = r < cnt ? v : 0.f;
    }
  }
}

template <int NCH, int RBW, bool SKIP>
__device__ __forceinline__ void fold_apply(float4 (&s)[RBW][NCH], FoldIn<NCH, RBW> &fi, float Ah, int lane) {
  const int q = lane >> 4;
  const float dtv = fi.f;
  float total;
  const float seg = suffix_sum16(dtv, lane, &total);
  const float f = __expf(Ah * seg) * dtv;
  const float scale = s0_weight<SKIP>(Ah * total);
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    float xb[4];  // MFMA B operand: f_r x_r[row], r = 4 st + q  (K = record, N = row)
#pragma unroll
    for (int st = 0; st < 4; ++st) xb[st] = __shfl(f, 4 * st + q, kWave) * fi.xraw[st][k];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 acc = {s[k][c].x * scale, s[k][c].y * scale, s[k][c].z * scale, s[k][c].w * scale};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if (st < fi.nsteps) acc = mfma_16x16x4(fi.aB[c][st], xb[st], acc);
      s[k][c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

template <int NCH, int RBW>
__device__ __forceinline__ void load_rows(float4 (&s)[RBW][NCH], const float *S, int rb0, int lane) {
  constexpr int N = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s[k][c] = ld4(S + (size_t)row * N + 16 * c + 4 * q);
  }
}

template <int NCH, int RBW>
__device__ __forceinline__ void store_rows(const float4 (&s)[RBW][NCH], float *S, int rb0, int lane) {
  constexpr int N = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) st4(S + (size_t)row * N + 16 * c + 4 * q, s[k][c]);
  }
}

// Value of acc[k] for k = sel (a per-lane index) without dynamic register indexing.
template <int RBW>
__device__ __forceinline__ float pick(const float (&acc)[RBW], int sel) {
  float v = acc[0];
#pragma unroll
  for (int k = 1; k < RBW; ++k) v = (sel == k) ? acc[k] : v;
  return v;
}

// Output of the newest of m window records from the checkpoint rows in s.
// Inputs are the already-loaded pieces: Cs (this token's C, in the wave's LDS
// region), bdot (the lane's partial B_{r16} . C), dtv (dt of record `lane`,
// lanes 0..15), xr[st][k] (x of record 4 st + q at row block k).  Returns the
// finished output of row 16 (rb0 + q) + r16 (lanes with q < RBW).
template <int NCH, int RBW, bool SKIP, typename R, int CM = kColIlv>
__device__ __forceinline__ float replay_output(const float4 (&s)[RBW][NCH], const R *Cs, float bdot, float dtv,
                                               const float (&xr)[4][RBW], int m, float Ah, int lane) {
  const int q = lane >> 4;
  const float dot = sum_quarters(bdot);
  float total;
  const float seg = suffix_sum16(dtv, lane, &total);
  const float w = lane < m ? __expf(Ah * seg) * dtv * dot : 0.f;
  const float scale = s0_weight<SKIP>(Ah * total);
  float acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) v += dot4(s[k][c], ldr4<R>(Cs + colq<NCH, CM>(c, q)));
    v *= scale;
#pragma unroll
    for (int st = 0; st < 4; ++st) v += __shfl(w, 4 * st + q, kWave) * xr[st][k];
    acc[k] = sum_quarters(v);
  }
  return pick<RBW>(acc, q);
}

// Bytes of one LDS row of the step kernel (a record vector plus 16 bytes, so
// that the rows of consecutive records start on different banks), and of one
// wave's region: this token's C, then the B of up to kMaxL window records.
template <int NCH, typename R>
constexpr int step_lds_row() { return 16 * NCH * (int)sizeof(R) + 16; }
template <int NCH, typename R>
constexpr int step_lds_wave() { return step_lds_row<NCH, R>() * (kMaxL + 1); }

// ZC: the token's x, B, dt are already in their ring slots (zero-copy append); a
// compile-time choice, because a run-time one costs the standard path 58 VGPRs.
//
// LDS: each wave has a private region (step_lds_wave bytes, dynamic shared
// memory) holding this token's C and the B of the window records it reads.
// Both arrive by direct global-to-LDS loads issued behind the checkpoint
// stream, so no VGPR holds them while the stream is in flight and the wave
// waits only for its own loads: there is no workgroup barrier on the
// non-fold path.
// Occupancy target: four waves per SIMD (at most 128 VGPRs) for the copying
// step.  The zero-copy variants get no target: their ring-slot addressing
// would then spill to scratch.
// Low-precision copies: no target either (their codecs need the registers).
template <bool ZC, int CF = REPLAY_FMT_F32, int RF = REPLAY_FMT_F32>
constexpr int step_waves_per_eu() { return (ZC || CF != REPLAY_FMT_F32 || RF != REPLAY_FMT_F32) ? 1 : 4; }

// With low-precision copies (CF, RF not both F32) the step reads the read copy
// and decodes it in registers; a fold decodes the checkpoint, folds in float32,
// stores both copies and outputs from the float32 fold result (only the steps
// that do not fold read the approximate copy [P3, Perspective, paragraph 2]).
template <int NCH, int RBW, bool SKIP, typename R, bool ZC, int CF = REPLAY_FMT_F32, int RF = REPLAY_FMT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(step_waves_per_eu<ZC, CF, RF>())))
void m2_replay_step(M2StepArgs a, StateBufs sb) {
  constexpr int N = 16 * NCH;
  constexpr int kRow = step_lds_row<NCH, R>();
  constexpr bool kF32 = CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32;
  constexpr int CM = col_map(CF, RF);
  static_assert(kF32 || (!SKIP && !ZC), "low-precision copies: no decay skip, no zero-copy append");
  extern __shared__ __align__(16) unsigned char m2_step_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int g = fdiv(h, sh.fHpg);
  const int P = sh.P, L = sh.L, Ls = sh.Ls;
  const int rb0 = wave * RBW;
  constexpr bool zc = ZC;
  unsigned char *wl = m2_step_lds + wave * step_lds_wave<NCH, R>();
  R *Cs = reinterpret_cast<R *>(wl);                             // this token's C
  unsigned char *Bs = wl + kRow;                                 // row j: B of window record j
  auto Brow = [&](int j) { return reinterpret_cast<R *>(Bs + j * kRow); };
  const size_t head = ((size_t)b * sh.H + h) * P * N;  // element offset of the head's state
  float *S = a.ckpt + head;
  const size_t xs = (size_t)sh.B * sh.H * P;  // x-ring slot stride (slot-major ring)
  R *rx = static_cast<R *>(a.ring.x) + ((size_t)b * sh.H + h) * P;
  float *rdt = a.ring.dt + ((size_t)b * sh.H + h) * Ls;
  R *rB = static_cast<R *>(a.ring.Bm) + ((size_t)b * sh.G + g) * 2 * L * N;
  const R *xin = zc ? nullptr : static_cast<const R *>(a.x) + ((size_t)b * sh.H + h) * P;
  const R *Bin = zc ? nullptr : static_cast<const R *>(a.Bm) + ((size_t)b * sh.G + g) * N;
  const R *Cin = static_cast<const R *>(a.Cm) + ((size_t)b * sh.G + g) * N;

  // 1. Everything whose address needs no pointer, checkpoint first: its loads
  //    are then in flight while the pointers arrive.  (Loads complete in issue
  //    order, so nothing issued later can delay it.)  The pointer words and the
  //    per-head scalars are read before the first global-to-LDS load, after
  //    which the compiler would no longer use scalar loads.
  //    With the decay skip the checkpoint stream waits for the decision, which
  //    needs the pointers and the head's dt ring row.
  float4 s[RBW][NCH];
  typename SIO<RF, NCH, RBW, CM>::Raw raw;  // low-precision copies: the read copy's stored bits
  if constexpr (!kF32) SIO<RF, NCH, RBW, CM>::load(raw, sb.rd, head, rb0, lane);
  else if constexpr (!SKIP) load_rows<NCH, RBW>(s, S, rb0, lane);
  const int pos_raw = a.ptr.pos_in[b], ck_raw = a.ptr.ckpt_in[b];
  float dt_in = zc ? 0.f : a.dt[(size_t)b * sh.H + h];
  const float Ah = a.A[h], Dh = a.D[h];
  const float dtrow = rdt[lane < Ls ? lane : 0];  // the head's whole dt ring, slot = lane
  dma_vec<N, R>(Cin, Cs, lane);

  // 2. Pointers.  A corrupted pair (count outside [0, L], or ckpt_pos < 0) is flagged and the
  //    sequence skipped: it computes on pointers (0, 0), so every ring index
  //    stays in range, and stores nothing.  No early return here: the compiler
  //    would sink the checkpoint loads below the branch, and every tile would
  //    then wait for the pointers before starting its stream.
  const bool bad = !pointers_ok(pos_raw, ck_raw, L);
  const int pos = bad ? 0 : pos_raw, ck = bad ? 0 : ck_raw;
  const int count = pos - ck;
  const bool fold = count == L;
  const int s0 = fmod_(ck, sh.fLs), s0b = fmod_(ck, sh.f2L);  // slots of window record 0
  const int slot = wrap(s0, count, Ls), slotb = wrap(s0b, count, 2 * L);  // slots of this token
  if (zc) {
    xin = rx + (size_t)slot * xs;
    Bin = rB + (size_t)slotb * N;
    dt_in = __shfl(dtrow, slot, kWave);
  }
  if constexpr (SKIP) {
    // The checkpoint term this call uses: the fold's (L records) or this
    // token's output (count + 1 records).  Read the checkpoint only if it stays.
    const int n = fold ? L : count + 1;
    const int j = r16 < n ? r16 : 0;
    const float d = __shfl(dtrow, wrap(s0, j < count ? j : 0, Ls), kWave);
    const float tot = sum16(r16 < n ? ((!fold && r16 == count) ? dt_in : d) : 0.f);
    if (Ah * tot < kDecaySkipLog) {
#pragma unroll
      for (int k = 0; k < RBW; ++k)
#pragma unroll
        for (int c = 0; c < NCH; ++c) s[k][c] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      load_rows<NCH, RBW>(s, S, rb0, lane);
    }
  }

  float bdot = 0.f, dtv;
  float xr[4][RBW];
  int base;
  if (!fold) {
    // 3. Window records (ring slots known now): B of records 0 .. m-1 into the
    //    wave's LDS rows, x of record 4 st + q at the lane's rows.  The x loads
    //    are unconditional on a clamped record index, masked afterwards.
    base = ck;
    const int m = count + 1;
    for (int j = 0; j < m; ++j) dma_vec<N, R>((j == m - 1) ? Bin : rB + wrap(s0b, j, 2 * L) * N, Brow(j), lane);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int j = 4 * st + q;
      const int jc = j < m ? j : m - 1;
      const R *xj = (jc == m - 1) ? xin : rx + wrap(s0, jc, Ls) * xs;
#pragma unroll
      for (int k = 0; k < RBW; ++k) {
        const float v = ldr<R>(xj + (rb0 + k) * 16 + r16);
        xr[st][k] = j < m ? v : 0.f;
      }
    }
    {
      // dt of record `lane`, permuted out of the ring row loaded up front.
      const float d = __shfl(dtrow, wrap(s0, r16 < m - 1 ? r16 : 0, Ls), kWave);
      dtv = lane < m - 1 ? d : (lane == m - 1 ? dt_in : 0.f);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's global-to-LDS loads have landed
    wave_lds_sync();
    {
      const R *Bj = Brow(r16 < m ? r16 : m - 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) bdot += dot4(ldr4<R>(Bj + 16 * c + 4 * q), ldr4<R>(Cs + 16 * c + 4 * q));
    }
    bdot = r16 < m ? bdot : 0.f;
    if constexpr (!kF32) SIO<RF, NCH, RBW, CM>::decode(s, raw);
  } else {
    // Fold the full window into the checkpoint, store it, and start the next
    // window with this token as its only record.
    FoldIn<NCH, RBW> fi;
    fold_load<NCH, RBW, R, CM>(fi, L, s0, s0b, rx, rdt, rB, L, Ls, xs, rb0, lane);
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const float v = ldr<R>(xin + (rb0 + k) * 16 + r16);
#pragma unroll
      for (int st = 0; st < 4; ++st) xr[st][k] = (st == 0 && q == 0) ? v : 0.f;
    }
    dtv = lane == 0 ? dt_in : 0.f;
    if constexpr (!kF32) {
      if constexpr (CF == RF) {
        SIO<RF, NCH, RBW, CM>::decode(s, raw);
      } else {
        typename SIO<CF, NCH, RBW, CM>::Raw rc;
        SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
        SIO<CF, NCH, RBW, CM>::decode(s, rc);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this token's C (global-to-LDS) has landed
    wave_lds_sync();
    fold_apply<NCH, RBW, SKIP>(s, fi, Ah, lane);
    if constexpr (kF32) store_rows<NCH, RBW>(s, S, rb0, lane);
    else store_copies<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
    base = pos;
    // This token's B . C after the fold: computing it earlier keeps more
    // registers live across the fold.
#pragma unroll
    for (int c = 0; c < NCH; ++c) bdot += dot4(ldr4<R>(Bin + 16 * c + 4 * q), ldr4<R>(Cs + 16 * c + 4 * q));
    bdot = r16 == 0 ? bdot : 0.f;
  }
  const int m = pos - base + 1;
  const float out = replay_output<NCH, RBW, SKIP, R, CM>(s, Cs, bdot, dtv, xr, m, Ah, lane);

  // 4. Append this token's record (unless the producer wrote it into the ring).
  //    After a fold the dt slot being written held a record that the other
  //    waves of a multi-wave head also read.
  if (fold && nwaves > 1 && !zc) __syncthreads();
  if (bad) {
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos_raw;
      a.ptr.ckpt_out[b] = ck_raw;
    }
    return;
  }
  if (q < RBW) {
    const int row = (rb0 + q) * 16 + r16;
    const float xv = ldr<R>(xin + row);
    a.y[((size_t)b * sh.H + h) * P + row] = out + Dh * xv;
    if (!zc) str<R>(rx + slot * xs + row, xv);
  }
  if (!zc) {
    if (threadIdx.x == 0) rdt[slot] = dt_in;
    if (h - g * (sh.H / sh.G) == 0 && wave == 0)
      for (int i = lane; i < N; i += kWave) rB[slotb * N + i] = Bin[i];
  }
  if (h == 0 && threadIdx.x == 0) {
    a.ptr.pos_out[b] = pos + 1;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- explicit flush ---------------------------------------------------------
template <int NCH, int RBW, bool SKIP, typename R, int CF = REPLAY_FMT_F32, int RF = REPLAY_FMT_F32>
__global__ __launch_bounds__(256) void m2_flush(M2FlushArgs a, StateBufs sb) {
  constexpr int N = 16 * NCH;
  constexpr bool kF32 = CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32;
  constexpr int CM = col_map(CF, RF);
  static_assert(kF32 || !SKIP, "low-precision copies: no decay skip");
  __shared__ M2Smem<NCH> sm;
  const TileCtx t = tile_ctx();
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = tile / sh.H, h = tile - b * sh.H;
  const int g = h / (sh.H / sh.G);
  const int P = sh.P, L = sh.L;
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  const bool bad = !pointers_ok(pos, ck, L);
  const bool fold = !bad && count > 0 && (a.mask == nullptr || a.mask[b] != 0);
  if (h == 0 && t.tid == 0) {
    if (bad) atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = fold ? pos : ck;
  }
  if (!fold) return;
  const size_t head = ((size_t)b * sh.H + h) * P * N;
  float *S = a.ckpt + head;
  const size_t xs = (size_t)sh.B * sh.H * P;
  const R *rx = static_cast<const R *>(a.ring.x) + ((size_t)b * sh.H + h) * P;
  const float *rdt = a.ring.dt + ((size_t)b * sh.H + h) * sh.Ls;
  const R *rB = static_cast<const R *>(a.ring.Bm) + ((size_t)b * sh.G + g) * 2 * L * N;
  float4 s[RBW][NCH];
  bool keep = true;  // the checkpoint term survives the decay skip
  if constexpr (SKIP) {
    const float d = rdt[(ck + (t.r16 < count ? t.r16 : 0)) % sh.Ls];
    keep = !(a.A[h] * sum16(t.r16 < count ? d : 0.f) < kDecaySkipLog);
  }
  if constexpr (!kF32) {
    typename SIO<CF, NCH, RBW, CM>::Raw rc;
    SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, t.wave * RBW, t.lane);
    SIO<CF, NCH, RBW, CM>::decode(s, rc);
  } else if (keep) {
    load_tile<NCH, RBW>(s, S, t);
  } else {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) s[k][c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  fold_tile<NCH, RBW, SKIP, R, CM>(s, sm, count, ck, a.A[h], rx, rdt, rB, L, sh.Ls, xs, t);
  if constexpr (kF32) store_tile<NCH, RBW>(s, S, t);
  else store_copies<CF, RF, NCH, RBW>(s, sb, head, t.wave * RBW, t.lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
}

// ---- speculative verify -------------------------------------------------
// T drafts follow the c committed window records.  Outputs for draft i
// (window record c + i):
//   y_i = exp(A s_{1..c+i}) S0 C_i + sum_{r <= c+i} exp(A s_{r+1..c+i}) dt_r (B_r . C_i) x_r + D x_{c+i}
// Geometry as the step: each wave owns RBW row blocks of the head.  Drafts go
// in passes of four through v_mfma_f32_4x4x1_16b_f32 (16 blocks of 4 x 4 x 1;
// lane l feeds block l / 4, row / column l % 4, and gets rows 0..3 of column
// l % 4 of its block), so no MFMA work is spent on absent drafts.  With lane
// l = r + 16 q, g = r / 4, m = r % 4, draft n = 4 p + m in pass p:
//   * S0 . C_n: block (g, q) takes rows 16 rb + 4 g + 0..3 over the columns of
//     quarter q of the register tile; a sum over q completes the products;
//   * B_r . C_n the same way, with record r in place of the row; a per-wave
//     LDS transpose then gives lane (r, q) the records 4 st + q it feeds;
//   * the record sum X~ . Coef^T (K = record 4 st + q) is accumulated onto the
//     scaled partial products before the sum over q.
// The drafts' C and the records' B reach LDS by direct global-to-LDS loads
// (global_load_lds_dwordx4: lane l of a load writes 16 bytes at base + 16 l),
// laid out so that every read is linear in the lane (no bank conflicts) and
// no VGPR holds them while the checkpoint stream is in flight (bf16 records:
// a load, exact widening and LDS store in the same layout).  Loads that
// need no pointer (checkpoint, drafts' C and x) are issued first; the drafts
// are staged in the ring from registers and LDS; no state is written except
// by a fold-first when c + T > L.
__device__ __forceinline__ floatx4 mfma_4x4x1(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

template <int NCH, int RBW, bool SKIP, typename R, int CF = REPLAY_FMT_F32, int RF = REPLAY_FMT_F32>
__global__ __launch_bounds__(256) void m2_replay_verify(M2VerifyArgs a, StateBufs stb) {
  constexpr int N = 16 * NCH;
  constexpr int kPass = kMaxL / 4;
  constexpr bool kF32 = CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32;
  constexpr int CM = col_map(CF, RF);
  static_assert(kF32 || !SKIP, "low-precision copies: no decay skip");
  __shared__ float4 ldsB[NCH][64];          // [chunk cc][r + 16 q]: B_r[colq(cc, q) .. + 3]
  __shared__ float4 ldsC[kPass * NCH * 16];  // [(p NCH + cc) 16 + 4 m + q]: C_{4 p + m}[colq(cc, q) .. + 3]
  __shared__ float dots_all[4][kMaxL][4];    // per wave: [record][draft of the pass] B_r . C_n
  // Per wave: x of draft i at the wave's rows (16 RBW elements of type R), for
  // the D x term; from LDS, the passes issue no global load, which would wait
  // for the previous pass's output stores.
  __shared__ __align__(16) unsigned char ldsX[4][kMaxL][16 * RBW * sizeof(R)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15, gq = r16 >> 2, m4 = r16 & 3;
  const Shape &sh = a.s;
  const int T = a.T;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int g = fdiv(h, sh.fHpg);
  const int P = sh.P, L = sh.L, H = sh.H, G = sh.G, Ls = sh.Ls;
  const int rb0 = wave * RBW;
  const bool zc = a.in_ring;  // the drafts' x, B, dt are already in their ring slots
  const size_t head = ((size_t)b * H + h) * P * N;
  float *S = a.ckpt + head;
  const size_t xs = (size_t)sh.B * H * P;
  R *rx = static_cast<R *>(a.ring.x) + ((size_t)b * H + h) * P;
  float *rdt = a.ring.dt + ((size_t)b * H + h) * Ls;
  R *rB = static_cast<R *>(a.ring.Bm) + ((size_t)b * G + g) * 2 * L * N;
  const R *dx = static_cast<const R *>(a.x), *dB = static_cast<const R *>(a.Bm), *dC = static_cast<const R *>(a.Cm);
  int sb = 0, sbb = 0, c = 0;  // window slots of record 0 (mod Ls, mod 2 L), committed records
  // Draft i is window record c + i; with zc its x and B are in the ring.
  auto draft_x = [&](int i) { return zc ? rx + (size_t)wrap(sb, c + i, Ls) * xs : dx + (((size_t)b * T + i) * H + h) * P; };
  auto draft_B = [&](int i) { return zc ? rB + (size_t)wrap(sbb, c + i, 2 * L) * N : dB + (((size_t)b * T + i) * G + g) * N; };
  auto draft_C = [&](int i) { return dC + (((size_t)b * T + i) * G + g) * N; };
  const int npass = (T + 3) >> 2;

  // 1. The checkpoint stream, the pointers, then the drafts' C into LDS (load
  //    j of the tile by wave j % nwaves).
  //    The pointer words are read before any global-to-LDS load: the compiler
  //    keeps loads that follow such a load off the scalar unit.
  float4 s[RBW][NCH];
  typename SIO<RF, NCH, RBW, CM>::Raw raw;  // low-precision copies: the read copy's stored bits
  if constexpr (kF32) load_rows<NCH, RBW>(s, S, rb0, lane);
  else SIO<RF, NCH, RBW, CM>::load(raw, stb.rd, head, rb0, lane);
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const float Ah = a.A[h], Dh = a.D[h];
  {
    const int nload = (npass * NCH * 16 + 63) >> 6;
    for (int j = wave; j < nload; j += nwaves) {
      const int slot = 64 * j + lane;
      const int q2 = slot & 3, m2 = (slot >> 2) & 3, pc = slot >> 4;  // pc = p NCH + cc
      const int p2 = pc / NCH, cc = pc - p2 * NCH;
      const int n = 4 * p2 + m2;
      stage4<R>(draft_C(n < T ? n : T - 1) + colq<NCH, CM>(cc, q2), &ldsC[64 * j], lane);
    }
  }

  // 2. Pointers; fold-first when the window cannot take T more records.
  const int count = pos - ck;
  if (!pointers_ok(pos, ck, L)) {
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    __builtin_amdgcn_s_waitcnt(0);  // no global-to-LDS load outlives the workgroup
    return;
  }
  const bool fold = count + T > L;  // implies count >= 1 because T <= L
  int base = ck;
  if (fold) {
    FoldIn<NCH, RBW> fi;
    fold_load<NCH, RBW, R, CM>(fi, count, fmod_(ck, sh.fLs), fmod_(ck, sh.f2L), rx, rdt, rB, L, Ls, xs, rb0, lane);
    if constexpr (!kF32) {  // the drafts' outputs then come from the float32 fold result
      if constexpr (CF == RF) {
        SIO<RF, NCH, RBW, CM>::decode(s, raw);
      } else {
        typename SIO<CF, NCH, RBW, CM>::Raw rc;
        SIO<CF, NCH, RBW, CM>::load(rc, stb.ck, head, rb0, lane);
        SIO<CF, NCH, RBW, CM>::decode(s, rc);
      }
    }
    fold_apply<NCH, RBW, SKIP>(s, fi, Ah, lane);  // stored after the wait in 3
    base = pos;
  } else if constexpr (!kF32) {
    SIO<RF, NCH, RBW, CM>::decode(s, raw);
  }
  c = pos - base;          // committed records in the window
  const int nrec = c + T;  // <= L
  sb = fmod_(base, sh.fLs);
  sbb = fmod_(base, sh.f2L);

  // 3. Window records.  B of record r16 at the tile columns into LDS (chunk cc
  //    by wave cc % nwaves); x of record 4 st + q at this lane's rows
  //    (record-sum A operand); dt of record r16.
  {
    const int rc = r16 < nrec ? r16 : nrec - 1;
    const R *Br = rc < c ? rB + (size_t)wrap(sbb, rc, 2 * L) * N : draft_B(rc - c);
    for (int cc = wave; cc < NCH; cc += nwaves) stage4<R>(Br + colq<NCH, CM>(cc, q), &ldsB[cc][0], lane);
  }
  float xa[RBW][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int r = 4 * st + q;
    const int rc = r < nrec ? r : nrec - 1;
    const R *xr = rc < c ? rx + (size_t)wrap(sb, rc, Ls) * xs : draft_x(rc - c);
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const float v = ldr<R>(xr + (rb0 + k) * 16 + r16);
      xa[k][st] = r < nrec ? v : 0.f;
    }
  }
  float dtl;
  {
    const int rc = r16 < nrec ? r16 : nrec - 1;
    const float v = (rc < c || zc) ? rdt[wrap(sb, rc, Ls)] : a.dt[((size_t)b * T + (rc - c)) * H + h];
    dtl = r16 < nrec ? v : 0.f;
  }
  for (int i = 0; i < T; ++i) dma_vec<16 * RBW, R>(draft_x(i) + rb0 * 16, ldsX[wave][i], lane);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's global-to-LDS loads have landed
  __syncthreads();                // and every other wave's
  // A fold-first's checkpoint stores go out only now: loads and stores share
  // one counter, so stores issued before the wait above would hold it until
  // they completed (and the window loads behind them).  They drain during
  // the passes.
  if (fold) {
    if constexpr (kF32) store_rows<NCH, RBW>(s, S, rb0, lane);
    else store_copies<CF, RF, NCH, RBW>(s, stb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
  }

  // 4. Passes of four drafts.
  const int nsteps = (nrec + 3) >> 2;
  for (int p = 0; p < npass; ++p) {
    const int n = 4 * p + m4;  // this lane's draft
    const int nc = n < T ? n : T - 1;
    float4 xl[RBW];  // x_n at rows 16 rb + 4 g + 0..3 (the D x term)
#pragma unroll
    for (int k = 0; k < RBW; ++k) xl[k] = ldr4<R>(reinterpret_cast<const R *>(ldsX[wave][nc]) + k * 16 + 4 * gq);
    const float4 *cdp = &ldsC[(p * NCH * 4 + m4) * 4 + q];  // C_n at tile chunk cc: cdp[16 cc]

    // dots[4 g + v][n] (register v, summed over q), transposed through LDS.
    {
      floatx4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const float4 bq = ldsB[cc][lane], cv = cdp[16 * cc];
        dacc = mfma_4x4x1(bq.x, cv.x, dacc);
        dacc = mfma_4x4x1(bq.y, cv.y, dacc);
        dacc = mfma_4x4x1(bq.z, cv.z, dacc);
        dacc = mfma_4x4x1(bq.w, cv.w, dacc);
      }
      float dsum[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) dsum[v] = sum_quarters(dacc[v]);  // every lane takes part
      if (p) wave_lds_sync();  // the previous pass has read the table
      if (q == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) dots_all[wave][4 * gq + v][m4] = dsum[v];
      }
      wave_lds_sync();
    }
    // Record-sum operand: coef[n][r], r = 4 st + q, and the S0 weight, from
    // segment sums of dt over records r+1 .. last (summed as they are, not as
    // differences of prefix sums).  Row q of the wave scans draft 4 p + q
    // (every row holds dt of record j in lane j); lane (q, r16) reads the sums
    // of its own draft m4 from row m4.
    const int last = n < T ? c + n : -1;
    float seg[4];
    float tot;
    {
      const int nq = 4 * p + q;
      const int lastq = nq < T ? c + nq : -1;
      const float sfx = row_suffix_sum16(r16 <= lastq ? dtl : 0.f, lane);  // records r16 .. lastq
      tot = __shfl(sfx, 16 * m4, kWave);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int r1 = 4 * st + q + 1;  // first record after r
        const float v = __shfl(sfx, 16 * m4 + (r1 < 16 ? r1 : 0), kWave);
        seg[st] = r1 < 16 ? v : 0.f;
      }
    }
    const float sc = s0_weight<SKIP>(Ah * tot);
    float cb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r = 4 * st + q;
      const float dtr = __shfl(dtl, r, kWave);
      cb[st] = r <= last ? __expf(Ah * seg[st]) * dtr * dots_all[wave][r][m4] : 0.f;
    }

#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const float4 cv = cdp[16 * cc];
        acc = mfma_4x4x1(s[k][cc].x, cv.x, acc);
        acc = mfma_4x4x1(s[k][cc].y, cv.y, acc);
        acc = mfma_4x4x1(s[k][cc].z, cv.z, acc);
        acc = mfma_4x4x1(s[k][cc].w, cv.w, acc);
      }
      acc = floatx4{sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if (st < nsteps) acc = mfma_4x4x1(xa[k][st], cb[st], acc);
      float4 o = make_float4(sum_quarters(acc[0]), sum_quarters(acc[1]), sum_quarters(acc[2]),
                             sum_quarters(acc[3]));
      o.x += Dh * xl[k].x;
      o.y += Dh * xl[k].y;
      o.z += Dh * xl[k].z;
      o.w += Dh * xl[k].w;
      if (q == 0 && n < T) st4(a.y + (((size_t)b * T + n) * H + h) * P + (rb0 + k) * 16 + 4 * gq, o);
    }
  }

  // 5. Stage the drafts (records c .. nrec-1) in the ring, unless the producer
  //    put them there.  The workgroup barrier above already ordered every
  //    wave's fold reads before this.
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int r = 4 * st + q;
    if (!zc && r >= c && r < nrec) {
#pragma unroll
      for (int k = 0; k < RBW; ++k) str<R>(rx + (size_t)wrap(sb, r, Ls) * xs + (rb0 + k) * 16 + r16, xa[k][st]);
    }
  }
  if (wave == 0 && !zc) {
    if (lane >= c && lane < nrec) rdt[wrap(sb, lane, Ls)] = dtl;
    if (h - g * (H / G) == 0 && r16 >= c && r16 < nrec) {
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) str4<R>(rB + (size_t)wrap(sbb, r16, 2 * L) * N + colq<NCH, CM>(cc, q), ldsB[cc][lane]);
    }
  }
  if (h == 0 && threadIdx.x == 0) {
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- baseline: conventional load-update-store step -------------------------
// Same geometry and load order as the replay step: one wave per head, every
// load issued before any arithmetic.
template <int NCH, int RBW, typename R>
__global__ __launch_bounds__(256) void m2_conv_step(M2ConvArgs a) {
  constexpr int N = 16 * NCH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int g = fdiv(h, sh.fHpg);
  const int P = sh.P, rb0 = wave * RBW;
  float *S = a.state + ((size_t)b * sh.H + h) * P * N;
  float4 s[RBW][NCH];
  load_rows<NCH, RBW>(s, S, rb0, lane);
  const R *Bin = static_cast<const R *>(a.Bm) + ((size_t)b * sh.G + g) * N;
  const R *Cin = static_cast<const R *>(a.Cm) + ((size_t)b * sh.G + g) * N;
  float4 bv[NCH], cv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    bv[c] = ldr4<R>(Bin + 16 * c + 4 * q);
    cv[c] = ldr4<R>(Cin + 16 * c + 4 * q);
  }
  const R *xin = static_cast<const R *>(a.x) + ((size_t)b * sh.H + h) * P;
  float xr[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) xr[k] = ldr<R>(xin + (rb0 + k) * 16 + r16);
  const float dt = a.dt[(size_t)b * sh.H + h];
  const float decay = __expf(dt * a.A[h]);
  const float Dh = a.D[h];
  float acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const float dx = dt * xr[k];
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float4 &e = s[k][c];
      e.x = decay * e.x + dx * bv[c].x;
      e.y = decay * e.y + dx * bv[c].y;
      e.z = decay * e.z + dx * bv[c].z;
      e.w = decay * e.w + dx * bv[c].w;
      v += dot4(e, cv[c]);
    }
    acc[k] = sum_quarters(v);
  }
  store_rows<NCH, RBW>(s, S, rb0, lane);
  if (q < RBW) {
    const int row = (rb0 + q) * 16 + r16;
    a.y[((size_t)b * sh.H + h) * P + row] = pick<RBW>(acc, q) + Dh * ldr<R>(xin + row);
  }
}

// ---- baseline: snapshot-per-draft verify -----------------------------------
// Bytes one draft takes in a wave's LDS region of the snapshot baseline: its B
// and C, and x at the wave's rows.
template <int NCH, int RBW, typename R>
constexpr int snap_lds_draft() { return 2 * 16 * NCH * (int)sizeof(R) + 16 * RBW * (int)sizeof(R); }

// Every draft's B, C and x (at the wave's rows) are staged into the wave's LDS
// region by direct global-to-LDS loads before the first snapshot store, so the
// draft loop issues no global load: a load issued after stores waits for them
// to complete, which would serialise the T snapshot writes.
template <int NCH, int RBW, typename R>
__global__ __launch_bounds__(256) void m2_snapshot_verify(M2SnapArgs a) {
  constexpr int N = 16 * NCH;
  constexpr int kVec = N * (int)sizeof(R), kDraft = snap_lds_draft<NCH, RBW, R>();
  extern __shared__ __align__(16) unsigned char m2_snap_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const Shape &sh = a.s;
  const int T = a.T, H = sh.H, G = sh.G, P = sh.P, rb0 = wave * RBW;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * H;
  const int g = fdiv(h, sh.fHpg);
  const int cur = a.cur[b];
  if (cur < 0 || cur >= a.nslots) return;  // never index outside the slot array
  const size_t head_elems = (size_t)P * N;
  auto slot_ptr = [&](int sl) { return a.slots + (((size_t)b * a.nslots + sl) * H + h) * head_elems; };
  unsigned char *wl = m2_snap_lds + (size_t)wave * T * kDraft;
  float4 s[RBW][NCH];
  load_rows<NCH, RBW>(s, slot_ptr(cur), rb0, lane);
  const float Ah = a.A[h], Dh = a.D[h];
  for (int i = 0; i < T; ++i) {
    const R *xin = static_cast<const R *>(a.x) + (((size_t)b * T + i) * H + h) * P;
    dma_vec<N, R>(static_cast<const R *>(a.Bm) + (((size_t)b * T + i) * G + g) * N,
                  reinterpret_cast<R *>(wl + i * kDraft), lane);
    dma_vec<N, R>(static_cast<const R *>(a.Cm) + (((size_t)b * T + i) * G + g) * N,
                  reinterpret_cast<R *>(wl + i * kDraft + kVec), lane);
    dma_vec<16 * RBW, R>(xin + rb0 * 16, reinterpret_cast<R *>(wl + i * kDraft + 2 * kVec), lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's global-to-LDS loads have landed
  wave_lds_sync();
  for (int i = 0; i < T; ++i) {
    const float dt = a.dt[((size_t)b * T + i) * H + h];
    const float decay = __expf(dt * Ah);
    const R *Bl = reinterpret_cast<const R *>(wl + i * kDraft);
    const R *Cl = reinterpret_cast<const R *>(wl + i * kDraft + kVec);
    const R *xl = reinterpret_cast<const R *>(wl + i * kDraft + 2 * kVec);  // x at rows rb0 16 ..
    float dx[RBW], v[RBW];
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      dx[k] = dt * ldr<R>(xl + k * 16 + r16);
      v[k] = 0.f;
    }
    // Column chunk outermost (each chunk of B and C read from LDS once); every
    // row's sum still runs over the chunks in order.
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float4 bv = ldr4<R>(Bl + 16 * c + 4 * q), cv = ldr4<R>(Cl + 16 * c + 4 * q);
#pragma unroll
      for (int k = 0; k < RBW; ++k) {
        float4 &e = s[k][c];
        e.x = decay * e.x + dx[k] * bv.x;
        e.y = decay * e.y + dx[k] * bv.y;
        e.z = decay * e.z + dx[k] * bv.z;
        e.w = decay * e.w + dx[k] * bv.w;
        v[k] += dot4(e, cv);
      }
    }
    float acc[RBW];
#pragma unroll
    for (int k = 0; k < RBW; ++k) acc[k] = sum_quarters(v[k]);
    if (q < RBW) {
      const int row = (rb0 + q) * 16 + r16;
      a.y[(((size_t)b * T + i) * H + h) * P + row] = pick<RBW>(acc, q) + Dh * ldr<R>(xl + q * 16 + r16);
    }
    store_rows<NCH, RBW>(s, slot_ptr((cur + 1 + i) % a.nslots), rb0, lane);
  }
}

// ---- dispatch ---------------------------------------------------------------
// Wave-per-head kernels: RBW = min(P / 16, 4) row blocks per wave, P / (16 RBW)
// waves per head.  Workgroup kernels (flush, verify): one wave per row block, up
// to 4 waves, RBW = 2 at P = 128.
template <template <int, int> class K, typename Args>
int dispatch(const Args &a, int N, int P, int B, int H, bool wave_per_head, hipStream_t st) {
  int waves, rbw;
  if (!tile_geometry(P, wave_per_head, &waves, &rbw)) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)B * H)), block(64 * waves);
#define RSSM_CASE(NCH_, RBW_)                                       \
  if (N == 16 * NCH_ && rbw == RBW_) {                              \
    hipLaunchKernelGGL((K<NCH_, RBW_>::fn), grid, block, 0, st, a); \
    return (int)hipGetLastError();                                  \
  }
#define RSSM_NCH(RBW_) RSSM_CASE(1, RBW_) RSSM_CASE(2, RBW_) RSSM_CASE(4, RBW_) RSSM_CASE(8, RBW_)
  RSSM_NCH(1) RSSM_NCH(2)
#undef RSSM_NCH
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}

// Format pairs (checkpoint, read copy) with low-precision copies: N = 128 only.
#define RSSM_M2_FMT_PAIRS(X)                      \
  X(REPLAY_FMT_F32, REPLAY_FMT_F4E2M1_B16)        \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F4E2M1_B16)     \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F4E2M1_B16)     \
  X(REPLAY_FMT_F4E2M1_B16, REPLAY_FMT_F4E2M1_B16) \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F16_SR)         \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F8E4M3)

// Kernels that take the stored copies: K<CF, RF, NCH, RBW>::fn with
// K<...>::lds(waves) bytes of dynamic LDS.  LP: the low-precision pairs are
// instantiated too (the decay skip and zero-copy append are float32-only).
template <template <int, int, int, int> class K, bool LP, typename Args>
int dispatch_fmt(const Args &a, const StateBufs &sb, int cf, int rf, bool wave_per_head, hipStream_t st) {
  int waves, rbw;
  if (!tile_geometry(a.s.P, wave_per_head, &waves, &rbw)) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)a.s.B * a.s.H)), block(64 * waves);
  const int N = a.s.N;
#define RSSM_CASE(CF_, RF_, NCH_, RBW_)                                                                  \
  if (cf == CF_ && rf == RF_ && N == 16 * NCH_ && rbw == RBW_) {                                        \
    const size_t lds = K<CF_, RF_, NCH_, RBW_>::lds(waves);                                             \
    hipLaunchKernelGGL((K<CF_, RF_, NCH_, RBW_>::fn), grid, block, lds, st, a, sb);                     \
    return (int)hipGetLastError();                                                                      \
  }
#define RSSM_NCH(RBW_)                               \
  RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, 1, RBW_) \
  RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, 2, RBW_) \
  RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, 4, RBW_) \
  RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, 8, RBW_)
  RSSM_NCH(1) RSSM_NCH(2)
  if constexpr (LP) {
#define RSSM_Q(CF_, RF_) RSSM_CASE(CF_, RF_, 8, 1) RSSM_CASE(CF_, RF_, 8, 2)
    RSSM_M2_FMT_PAIRS(RSSM_Q)
#undef RSSM_Q
  }
#undef RSSM_NCH
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}

// Kernel wrappers.  The step kernel takes step_lds_wave bytes of dynamic LDS per wave.
template <bool SKIP, typename R, bool ZC>
struct StepK {
  template <int CF, int RF, int NCH, int RBW>
  struct K {
    static constexpr auto fn = m2_replay_step<NCH, RBW, SKIP, R, ZC, CF, RF>;
    static size_t lds(int waves) { return (size_t)waves * step_lds_wave<NCH, R>(); }
  };
};
template <bool SKIP, typename R>
struct FlushK {
  template <int CF, int RF, int NCH, int RBW>
  struct K {
    static constexpr auto fn = m2_flush<NCH, RBW, SKIP, R, CF, RF>;
    static size_t lds(int) { return 0; }
  };
};
template <bool SKIP, typename R>
struct VerifyK {
  template <int CF, int RF, int NCH, int RBW>
  struct K {
    static constexpr auto fn = m2_replay_verify<NCH, RBW, SKIP, R, CF, RF>;
    static size_t lds(int) { return 0; }
  };
};
#define RSSM_WRAP(name, kern)                       \
  template <typename R>                             \
  struct name {                                     \
    template <int NCH, int RBW>                     \
    struct K {                                      \
      static constexpr auto fn = kern<NCH, RBW, R>; \
    };                                              \
  };
RSSM_WRAP(ConvK, m2_conv_step)
#undef RSSM_WRAP

// The step by the record element type, the decay skip and zero-copy append.
template <bool SKIP, bool ZC, typename Args>
int launch_step_sz(const Args &a, const StateBufs &sb, int cf, int rf, hipStream_t st) {
  constexpr bool LP = !SKIP && !ZC;
  return a.bf16 ? dispatch_fmt<StepK<SKIP, bf16_t, ZC>::template K, LP>(a, sb, cf, rf, true, st)
                : dispatch_fmt<StepK<SKIP, float, ZC>::template K, LP>(a, sb, cf, rf, true, st);
}
// Flush or verify (W) by the record element type and the decay skip.
template <template <bool, typename> class W, bool SKIP, typename Args>
int launch_fmt(const Args &a, const StateBufs &sb, int cf, int rf, bool wave_per_head, hipStream_t st) {
  return a.bf16 ? dispatch_fmt<W<SKIP, bf16_t>::template K, !SKIP>(a, sb, cf, rf, wave_per_head, st)
                : dispatch_fmt<W<SKIP, float>::template K, !SKIP>(a, sb, cf, rf, wave_per_head, st);
}

// Launch W<float>::K or W<bf16_t>::K by the record element type.
template <template <typename> class W, typename Args>
int dispatch_rec(const Args &a, bool wave_per_head, hipStream_t st) {
  return a.bf16 ? dispatch<W<bf16_t>::template K>(a, a.s.N, a.s.P, a.s.B, a.s.H, wave_per_head, st)
                : dispatch<W<float>::template K>(a, a.s.N, a.s.P, a.s.B, a.s.H, wave_per_head, st);
}

}  // namespace

int launch_m2_step(const M2StepArgs &a, const FormatBufs &f, hipStream_t st) {
  const StateBufs sb = state_bufs(f);
  if (a.decay_skip)
    return a.in_ring ? launch_step_sz<true, true>(a, sb, f.ckpt_fmt, f.read_fmt, st)
                     : launch_step_sz<true, false>(a, sb, f.ckpt_fmt, f.read_fmt, st);
  return a.in_ring ? launch_step_sz<false, true>(a, sb, f.ckpt_fmt, f.read_fmt, st)
                   : launch_step_sz<false, false>(a, sb, f.ckpt_fmt, f.read_fmt, st);
}
int launch_m2_flush(const M2FlushArgs &a, const FormatBufs &f, hipStream_t st) {
  const StateBufs sb = state_bufs(f);
  return a.decay_skip ? launch_fmt<FlushK, true>(a, sb, f.ckpt_fmt, f.read_fmt, false, st)
                      : launch_fmt<FlushK, false>(a, sb, f.ckpt_fmt, f.read_fmt, false, st);
}
int launch_m2_verify(const M2VerifyArgs &a, const FormatBufs &f, hipStream_t st) {
  const StateBufs sb = state_bufs(f);
  return a.decay_skip ? launch_fmt<VerifyK, true>(a, sb, f.ckpt_fmt, f.read_fmt, true, st)
                      : launch_fmt<VerifyK, false>(a, sb, f.ckpt_fmt, f.read_fmt, true, st);
}
int launch_m2_conv(const M2ConvArgs &a, hipStream_t st) { return dispatch_rec<ConvK>(a, true, st); }
// The snapshot baseline takes T snap_lds_draft bytes of dynamic LDS per wave.
template <typename R>
int launch_snapshot_r(const M2SnapArgs &a, hipStream_t st) {
  int waves, rbw;
  if (!tile_geometry(a.s.P, true, &waves, &rbw)) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)a.s.B * a.s.H)), block(64 * waves);
#define RSSM_CASE(NCH_, RBW_)                                                               \
  if (a.s.N == 16 * NCH_ && rbw == RBW_) {                                                  \
    const size_t lds = (size_t)waves * a.T * snap_lds_draft<NCH_, RBW_, R>();              \
    if (lds > 65536) {                                                                      \
      const hipError_t e = hipFuncSetAttribute((const void *)m2_snapshot_verify<NCH_, RBW_, R>, \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,  \
                                               (int)lds);                                   \
      if (e != hipSuccess) return (int)e;                                                   \
    }                                                                                       \
    hipLaunchKernelGGL((m2_snapshot_verify<NCH_, RBW_, R>), grid, block, lds, st, a);       \
    return (int)hipGetLastError();                                                          \
  }
#define RSSM_NCH(RBW_) RSSM_CASE(1, RBW_) RSSM_CASE(2, RBW_) RSSM_CASE(4, RBW_) RSSM_CASE(8, RBW_)
  RSSM_NCH(1) RSSM_NCH(2)
#undef RSSM_NCH
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}
int launch_m2_snapshot(const M2SnapArgs &a, hipStream_t st) {
  return a.bf16 ? launch_snapshot_r<bf16_t>(a, st) : launch_snapshot_r<float>(a, st);
}

}  // namespace rssm
