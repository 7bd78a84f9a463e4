// Gated DeltaNet replay decode kernels for gfx950.
//
// Recurrence (per head; S is d_v x d_k and multiplies keys from the right):
//     S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q
// equivalently S <- alpha S + u k^T with the pseudo-value u = beta (v - alpha S k).
// With a checkpoint S0 and window records 1..m, g_j = sum_{i<=j} log alpha_i,
// the pseudo-values solve the unit-lower-triangular system
//     u_t + beta_t sum_{j<t} e^{g_t - g_j} (k_t . k_j) u_j = beta_t (v_t - e^{g_t} S0 k_t)
// and the newest output and the fold are
//     o_m   = e^{g_m} S0 q_m + sum_{j<=m} e^{g_m - g_j} (k_j . q_m) u_j
//     S_new = e^{g_m} S0 + sum_j e^{g_m - g_j} u_j k_j^T.
// One read of S0 serves the whole window; the checkpoint is written only by a
// fold [P1, Synopsis; P2, paragraph 3; P3, Interpretation 2].
//
// The system is triangular, so u_t never changes once record t is appended:
// the ring keeps u_t (next to k_t, alpha_t, beta_t) and a step solves one new
// row.  A non-fold step is then a streaming pass over S0 for S0 k_m and S0 q_m
// on the VALU.  A fold is the MFMA rank-m update S^T += K^T U~^T.  With a
// separate read copy the cached u_t come from the read copy, so a fold
// re-solves them from the checkpoint and the buffered values v_t (kept in the
// ring for that purpose) with the full-window solve below.
//
// Tile = one (sequence, head); four waves, each holding 16 RBW rows (d_v
// indices) of S0 in registers:
//     s[k][c] = S[16 (rb0 + k) + (l % 16)][col(c, q) + 0..3],  q = l / 16.
// The column map col is a compile-time choice (colq below): interleaved
// (16 c + 4 q) when the copies are float32, contiguous per lane (4 NCH q + 4 c)
// when a low-precision copy is read, so that its bytes load wide and every
// 16-column e2m1 scale block lies inside one lane.  Keys and queries use the
// same map, so every contraction over d_k is unchanged.
// The full-window solve (verify, re-solving folds), per wave, with X = the
// window's keys in MFMA operand layout (lane (j, q) holds k_j[col(c, q) + 0..3],
// j = l % 16):
//   * W = S0 X^T (one v_mfma_f32_16x16x4f32 pass: M = row, N = record, K = d_k),
//   * the Gram matrix X X^T from the same operand registers,
//   * W goes through per-wave LDS so that each lane owns one row and runs the
//     m x m forward substitution for it with no cross-lane traffic,
//   * the fold's MFMA output layout equals the register layout of S0.
// Kernels are templated on the stored formats (CF, RF), the tile shape and R,
// the element type of the record vector fields and their ring copies (float,
// or bf16_t with bf16 records).  With zero-copy append (a.in_ring) the caller
// writes k, alpha, beta into their ring slots (2L slots per field) and the
// kernels read them there instead of copying them.
#include "state_io.h"

namespace rssm {
namespace {

template <int RBW>
struct GdnLds {
  float W[16 * RBW][17];      // [row][record]: S0 k_j
  float gram[16][17];         // k_t . k_j
  float A[16][17];            // beta_t e^{g_t - g_j} (k_t . k_j) for j < t, else 0
  float c1[16], c2[16];       // beta_t, beta_t e^{g_t}
  float us[16];               // e^{g_m - g_j}: pseudo-value weight in a fold
  float g[16], beta[16];
  float U[16][16 * RBW + 4];  // pseudo-values u_t [record][row]
};

// Inclusive prefix sum over lanes 0..15 (lanes >= 16 must pass 0).
__device__ __forceinline__ float prefix_sum16(float v, int lane) {
  float t = v;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const float u = __shfl_up(t, off, kWave);
    if ((lane & 15) >= off) t += u;
  }
  return t;
}

// The window of one wave: records 0..m-1 (keys in X, lane j's alpha_j, beta_j
// in al/be).  For t < known, vr[t] is this lane's row of the already known
// pseudo-value u_t; for known <= t < m it is the row of v_t (lanes < 16 RBW).
// Solves for the remaining pseudo-values and leaves every u_t in sm.U[t][row],
// the decay prefix g in sm.g and the fold weights e^{g_{m-1} - g_t} in sm.us.
template <int NCH, int RBW>
__device__ __forceinline__ void gdn_window(const float4 (&s)[RBW][NCH], const float4 (&X)[NCH], int m, int known,
                                           float al, float be, const float (&vr)[16], GdnLds<RBW> &sm, int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  // W = S0 X^T and the Gram matrix X X^T on the MFMA.
  floatx4 acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      acc[k] = mfma_16x16x4(s[k][c].x, X[c].x, acc[k]);
      acc[k] = mfma_16x16x4(s[k][c].y, X[c].y, acc[k]);
      acc[k] = mfma_16x16x4(s[k][c].z, X[c].z, acc[k]);
      acc[k] = mfma_16x16x4(s[k][c].w, X[c].w, acc[k]);
    }
  }
  floatx4 gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    gacc = mfma_16x16x4(X[c].x, X[c].x, gacc);
    gacc = mfma_16x16x4(X[c].y, X[c].y, gacc);
    gacc = mfma_16x16x4(X[c].z, X[c].z, gacc);
    gacc = mfma_16x16x4(X[c].w, X[c].w, gacc);
  }
#pragma unroll
  for (int k = 0; k < RBW; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.W[16 * k + 4 * q + i][r16] = acc[k][i];
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.gram[4 * q + i][r16] = gacc[i];
  // Per-record scalars, record j in lane j (lanes 0..15).
  const float la = lane < m ? __logf(al) : 0.f;
  const float g = prefix_sum16(la, lane);
  const float gm = __shfl(g, m - 1, kWave);
  if (lane < 16) {
    sm.g[lane] = g;
    sm.beta[lane] = lane < m ? be : 0.f;
    sm.c1[lane] = lane < m ? be : 0.f;
    sm.c2[lane] = lane < m ? be * __expf(g) : 0.f;
    sm.us[lane] = lane < m ? __expf(gm - g) : 0.f;
  }
  wave_lds_sync();
  // Coupling matrix A[t][j] = beta_t e^{g_t - g_j} (k_t . k_j), j < t.
#pragma unroll
  for (int e0 = 0; e0 < 256; e0 += 64) {
    const int e = e0 + lane, t = e >> 4, j = e & 15;
    sm.A[t][j] = (j < t && t < m) ? sm.beta[t] * __expf(sm.g[t] - sm.g[j]) * sm.gram[t][j] : 0.f;
  }
  wave_lds_sync();
  if (lane < 16 * RBW) {
    // Forward substitution for this lane's row; u[t] kept in registers.
    float u[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = 0.f;
      if (t < known) {
        v = vr[t];
      } else if (t < m) {
        v = sm.c1[t] * vr[t] - sm.c2[t] * sm.W[lane][t];
#pragma unroll
        for (int j = 0; j < t; ++j) v -= sm.A[t][j] * u[j];
      }
      u[t] = v;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sm.U[t][lane] = u[t];
  }
  wave_lds_sync();
}

// s <- escale s + K^T Ub: the MFMA rank-cnt update of a fold, with the A
// operand (M = column of chunk c, K = record) read from the key ring (cache
// resident) and the B operand ub[k][st] = weight x u of record 4 st + q at row
// 16 (rb0 + k) + (lane % 16), supplied by the caller.  The tile accumulates in
// place, four records at a time, so that only one group of keys is live.
template <int NCH, int RBW, int CM, typename R>
__device__ __forceinline__ void fold_rank(float4 (&s)[RBW][NCH], int cnt, int s0, const R *rk, size_t ks, int L,
                                          float escale, const float (&ub)[RBW][4], int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int nsteps = (cnt + 3) >> 2;
#pragma unroll
  for (int k = 0; k < RBW; ++k)
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      s[k][c] = make_float4(s[k][c].x * escale, s[k][c].y * escale, s[k][c].z * escale, s[k][c].w * escale);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st < nsteps) {
      const int r = 4 * st + q;
      const R *kr = rk + (size_t)wrap(s0, r < cnt ? r : cnt - 1, L) * ks;
      float aK[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float v = ldr<R>(kr + colq<NCH, CM>(c, r16 >> 2) + (r16 & 3));  // M = r16 in chunk c
        aK[c] = r < cnt ? v : 0.f;
      }
#pragma unroll
      for (int k = 0; k < RBW; ++k)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const floatx4 acc = mfma_16x16x4(aK[c], ub[k][st], floatx4{s[k][c].x, s[k][c].y, s[k][c].z, s[k][c].w});
          s[k][c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
  }
}

// Head bases of the ring fields: k, u, v slot-major (v: re-solving folds only;
// k and v hold record elements of type R), alpha and beta rows.
template <typename R>
struct GdnRingPtrs {
  R *rk;
  float *ru;
  R *rv;
  float *ral, *rbe;
  size_t ks, vs;  // slot strides of the k ring and of the u and v rings
};

template <typename R>
__device__ __forceinline__ GdnRingPtrs<R> gdn_ring_ptrs(const GdnRing &r, const Shape &sh, int b, int h) {
  GdnRingPtrs<R> p;
  const size_t bh = (size_t)b * sh.H + h;
  p.ks = (size_t)sh.B * sh.H * sh.N;
  p.vs = (size_t)sh.B * sh.H * sh.P;
  p.rk = static_cast<R *>(r.k) + bh * sh.N;
  p.ru = r.u + bh * sh.P;
  p.rv = r.v ? static_cast<R *>(r.v) + bh * sh.P : nullptr;
  p.ral = r.alpha + bh * sh.Ls;
  p.rbe = r.beta + bh * sh.Ls;
  return p;
}

// Keys of window records 0..cnt-1 at ring positions starting at slot s0, in
// operand layout (zeros beyond cnt).
template <int NCH, int CM, typename R>
__device__ __forceinline__ void load_keys(float4 (&X)[NCH], int cnt, const GdnRingPtrs<R> &rp, int s0, int L,
                                          int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int j = r16 < cnt ? r16 : cnt - 1;
  const R *kj = rp.rk + (size_t)wrap(s0, j, L) * rp.ks;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float4 v = ldr4<R>(kj + colq<NCH, CM>(c, q));
    X[c] = r16 < cnt ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Row `row` of ring field f (u or v) for window records 0..cnt-1 from slot s0.
template <typename E>
__device__ __forceinline__ void load_ring_rows(float (&vr)[16], int cnt, const E *f, size_t vs, int s0, int L,
                                               int row) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int tc = t < cnt ? t : (cnt > 0 ? cnt - 1 : 0);
    const float v = ldr<E>(f + (size_t)wrap(s0, tc, L) * vs + row);
    vr[t] = t < cnt ? v : 0.f;
  }
}

// Fold the cnt (>= 1) committed records that start at slot s0 into the tile s,
// which holds the decoded checkpoint:
//     S <- e^{g_cnt} S + sum_t e^{g_cnt - g_t} u_t k_t^T.
// With one stored copy (CF == RF) the cached pseudo-values are those of this
// checkpoint and are folded as they are.  With a separate read copy they were
// computed from the read copy, so the fold re-solves them from the checkpoint
// and the values v (a full-window solve through sm), and the read copy's
// rounding never enters the recurrence.
template <int CF, int RF, int NCH, int RBW, typename R, bool SKIP = false>
__device__ __forceinline__ void gdn_fold(float4 (&s)[RBW][NCH], int cnt, int s0, const GdnRingPtrs<R> &rp, int Ls,
                                         int rb0, int lane, GdnLds<RBW> *sm) {
  static_assert(!SKIP || CF == RF, "the decay skip folds the cached pseudo-values");
  constexpr int CM = col_map(CF, RF);
  const int q = lane >> 4, r16 = lane & 15;
  const int j = r16 < cnt ? r16 : cnt - 1;
  const float al = rp.ral[wrap(s0, j, Ls)];
  float ub[RBW][4];
  float escale;
  if constexpr (CF != RF) {
    float4 X[NCH];
    float vr[16];
    load_keys<NCH, CM, R>(X, cnt, rp, s0, Ls, lane);
    load_ring_rows(vr, cnt, rp.rv, rp.vs, s0, Ls, rb0 * 16 + (lane < 16 * RBW ? lane : 0));
    const float be = rp.rbe[wrap(s0, j, Ls)];
    gdn_window<NCH, RBW>(s, X, cnt, 0, al, be, vr, *sm, lane);
    escale = __expf(sm->g[cnt - 1]);
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int st = 0; st < 4; ++st) ub[k][st] = sm->us[4 * st + q] * sm->U[4 * st + q][16 * k + r16];
  } else {
    const float la = lane < cnt ? __logf(al) : 0.f;
    const float g = prefix_sum16(la, lane);
    const float gl = __shfl(g, cnt - 1, kWave);
    const float us = lane < cnt ? __expf(gl - g) : 0.f;  // lane t: weight of record t
    escale = (SKIP && gl < kDecaySkipLog) ? 0.f : __expf(gl);  // decay skip: a pure write of the records
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r = 4 * st + q;
      const float w = __shfl(us, r, kWave);
      const float *ur = rp.ru + (size_t)wrap(s0, r < cnt ? r : cnt - 1, Ls) * rp.vs;
#pragma unroll
      for (int k = 0; k < RBW; ++k) ub[k][st] = w * ur[(rb0 + k) * 16 + r16];
    }
  }
  fold_rank<NCH, RBW, CM, R>(s, cnt, s0, rp.rk, rp.ks, Ls, escale, ub, lane);
}

// ---- replay step ------------------------------------------------------------
// The ring caches each record's pseudo-value u_t, computed when the record was
// appended from the S0 every output of the window reads (the decoded read
// copy).  A step that appends record m of its window then needs one read of S0
// for S0 k_m and S0 q_m, plus the older records' keys and pseudo-values:
//     u_m = beta_m (v_m - e^{g_m} S0 k_m - sum_{j<m} e^{g_m - g_j} (k_j . k_m) u_j)
//     o_m = e^{g_m} S0 q_m + sum_{j<=m} e^{g_m - g_j} (k_j . q_m) u_j.
// Lane (r, q) of a wave: S0 rows 16 (rb0 + k) + r, columns colq(c, q); the
// per-row recurrence runs in the lanes with q < RBW for row 16 (rb0 + q) + r.
// The key dot products are spread over the tile: thread group j (16 threads)
// takes k_j . k_m and k_j . q_m over NCH columns each (group 15: k_m . q_m),
// and k_m, q_m reach every wave through LDS, so no lane holds them whole.
// A step that finds the window full folds it first and stores both copies.
// Its own output comes from the float32 fold result it holds in registers
// (the outputs of steps that do not fold are the ones that read the
// approximate copy [P3, Perspective, paragraph 2]); the pseudo-value it caches
// for the next steps of the window is that of the read copy, which they read.
template <int NCH, typename R>
__device__ __forceinline__ void load_cols(float (&v)[NCH], const R *p) {
  if constexpr (NCH % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NCH / 4; ++i) {
      const float4 t = ldr4<R>(p + 4 * i);
      v[4 * i] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
  } else {
    static_assert(NCH == 2, "NCH is 2, 4 or 8");
    v[0] = ldr<R>(p);
    v[1] = ldr<R>(p + 1);
  }
}

// Float32 copies: held to 128 VGPRs (four waves per SIMD), which fits without
// spills; with the decay skip to 168 (three), where the decision's registers
// fit without spills.
// SKIP (decay skip, float32 copies): a head whose window log-decay (over the
// records the step's output or fold uses) is below ln 2^-24 does not read its
// checkpoint; its fold is a pure write of the folded records.
template <int CF, int RF, int NCH, int RBW, typename R, bool SKIP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32 ? (SKIP ? 3 : 4) : 1))) void gdn_replay_step(GdnStepArgs a, StateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  constexpr bool kLossy = RF != REPLAY_FMT_F32;  // the read copy is not the float32 fold result
  static_assert(!SKIP || (CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32), "decay skip: float32 copies only");
  constexpr int kMaxOld = 15;            // older records of a window (L <= 16)
  __shared__ float4 kq_s[2][DK / 4];     // k_m, q_m in natural column order
  __shared__ float dot_s[2][16];         // [0][j] = k_j . k_m, [1][j] = k_j . q_m; [1][15] = k_m . q_m
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int grp = threadIdx.x >> 4;      // record of this thread's key dot products
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, Ls = sh.Ls, rb0 = wave * RBW;
  const bool zc = a.in_ring;  // this token's k, alpha, beta are already in their ring slots
  const size_t bh = (size_t)b * sh.H + h;
  const size_t head = bh * DV * DK;
  const GdnRingPtrs<R> rp = gdn_ring_ptrs<R>(a.ring, sh, b, h);
  const R *qin = static_cast<const R *>(a.q) + bh * DK;
  const R *kin = zc ? nullptr : static_cast<const R *>(a.k) + bh * DK;
  const R *vin = static_cast<const R *>(a.v) + bh * DV;
  const int orow = (rb0 + (q < RBW ? q : 0)) * 16 + r16;  // this lane's output row (q < RBW)

  // 1. The read copy first (a non-fold step reads only it), then what needs no
  //    pointer.  With the decay skip the read waits for the decision (below).
  // Float32 copies load straight into the tile s (decay skip: once decided);
  // other formats keep the stored bits in raw until they are decoded.
  constexpr bool kF32 = CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32;
  typename SIO<RF, NCH, RBW, CM>::Raw raw;
  float4 s[RBW][NCH];
  if constexpr (kF32 && !SKIP) load_rows_g<NCH, RBW, CM>(s, static_cast<const float *>(sb.rd.data) + head, rb0, lane);
  else if constexpr (!SKIP) SIO<RF, NCH, RBW, CM>::load(raw, sb.rd, head, rb0, lane);
  float km[NCH], qm[NCH];  // columns NCH r16 .. of k_m and q_m
  if (!zc) load_cols<NCH, R>(km, kin + NCH * r16);
  load_cols<NCH, R>(qm, qin + NCH * r16);
  const float al_row = rp.ral[lane < Ls ? lane : 0];  // the head's alpha ring, slot = lane
  float al_in = zc ? 0.f : a.alpha[bh], be_in = zc ? 0.f : a.beta[bh];
  const float v_in = ldr<R>(vin + orow);

  // 2. Pointers.
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  if (count < 0 || count > L || ck < 0) {  // a flagged pair: no ring slot is computed from it
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  const bool fold = count == L;
  const int s0 = fmod_(ck, sh.fLs);
  const int slot = wrap(s0, count, Ls);  // this token's slot
  if (zc) {
    kin = rp.rk + (size_t)slot * rp.ks;
    load_cols<NCH, R>(km, kin + NCH * r16);
    al_in = __shfl(al_row, slot, kWave);
    be_in = rp.rbe[slot];
  }
  if constexpr (SKIP) {
    // The records whose decay multiplies the checkpoint term: the fold's L, or
    // this output's count + 1.  Read the checkpoint only if the term stays.
    const int n = fold ? L : count + 1;
    const int j = r16 < n ? r16 : 0;
    const float aj = __shfl(al_row, wrap(s0, j < count ? j : 0, Ls), kWave);
    const float ak = (!fold && r16 == count) ? al_in : aj;
    // Every 16-lane row computes the same sum: take lane 0's, so every lane
    // takes the same decision.  A dropped head's loads see an empty range and
    // return zeros without reading memory.
    const float tot = sum16(r16 < n ? __logf(ak) : 0.f);
    const bool drop = __builtin_amdgcn_readfirstlane(tot < kDecaySkipLog ? 1 : 0);
    load_rows_masked<NCH, RBW, CM>(s, static_cast<const float *>(sb.rd.data) + head,
                                   drop ? 0u : (uint32_t)(DV * DK * sizeof(float)), rb0, lane);
  }
  int base = ck, sb0 = s0;
  float kj[NCH];         // this thread's slice of key grp (an older record)
  float uo[kMaxOld];     // older pseudo-values of this lane's row
  float sk_fold = 0.f, sq_fold = 0.f;  // low-precision read copy: S k_m, S q_m of the fold result
  if (fold) {
    if constexpr (RF == CF) {
      // (e2m1: decoded apart from the non-fold branch's decode; 190 -> 155 VGPRs)
      if constexpr (RF == REPLAY_FMT_F4E2M1_B16) opaque_words(raw);
      if constexpr (!SKIP && !kF32) SIO<RF, NCH, RBW, CM>::decode(s, raw);
      gdn_fold<CF, RF, NCH, RBW, R, SKIP>(s, L, s0, rp, Ls, rb0, lane, nullptr);
    } else {
      __shared__ GdnLds<RBW> lds_all[4];
      typename SIO<CF, NCH, RBW, CM>::Raw rc;
      SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
      SIO<CF, NCH, RBW, CM>::decode(s, rc);
      gdn_fold<CF, RF, NCH, RBW, R>(s, L, s0, rp, Ls, rb0, lane, &lds_all[wave]);
    }
    if constexpr (kLossy) {
      // This token's output comes from the float32 fold result: its products
      // S k_m and S q_m first (k_m, q_m reach every wave through LDS), then
      // both copies are stored and s becomes what the read copy holds, the S0
      // of the window's later steps (and of the pseudo-value cached here).
      if (grp == 0) {
        float *kd = reinterpret_cast<float *>(kq_s[0]), *qd = reinterpret_cast<float *>(kq_s[1]);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          kd[NCH * r16 + i] = km[i];
          qd[NCH * r16 + i] = qm[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < RBW; ++k) {
        float ak = 0.f, aq = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int c4 = colq<NCH, CM>(c, q) >> 2;
          ak += dot4(s[k][c], kq_s[0][c4]);
          aq += dot4(s[k][c], kq_s[1][c4]);
          __builtin_amdgcn_sched_barrier(0);  // one chunk of k_m, q_m live at a time
        }
        ak = sum_quarters(ak);
        aq = sum_quarters(aq);
        if (q == k) {
          sk_fold = ak;
          sq_fold = aq;
        }
      }
    }
    // s becomes what the read copy now holds (float32 copies: the fold result itself).
    store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
    base = pos;
    sb0 = slot;
#pragma unroll
    for (int i = 0; i < NCH; ++i) kj[i] = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxOld; ++t) uo[t] = 0.f;
  } else {
    // The count older records, then the read copy (after the ring loads in program order).
    const int j = grp < count ? grp : 0;
    load_cols<NCH, R>(kj, rp.rk + (size_t)wrap(s0, j, Ls) * rp.ks + NCH * r16);
#pragma unroll
    for (int t = 0; t < kMaxOld; ++t) {
      const int tc = t < count ? t : 0;
      const float v = rp.ru[(size_t)wrap(s0, tc, Ls) * rp.vs + orow];
      uo[t] = t < count ? v : 0.f;
    }
    if constexpr (!SKIP && !kF32) SIO<RF, NCH, RBW, CM>::decode(s, raw);
  }
  const int nold = pos - base;  // older records in this window

  // Key dot products (group grp), and k_m, q_m into LDS (group 0).
  {
    float dk = 0.f, dq = 0.f;
    if (grp == 15) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) dq += km[i] * qm[i];
    } else if (grp < nold) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        dk += kj[i] * km[i];
        dq += kj[i] * qm[i];
      }
    }
    dk = sum16(dk);
    dq = sum16(dq);
    if (r16 == 0) {
      dot_s[0][grp] = dk;
      dot_s[1][grp] = dq;
    }
    if (grp == 0 && !(kLossy && fold)) {  // (a lossy fold step has written them already)
      float *kd = reinterpret_cast<float *>(kq_s[0]), *qd = reinterpret_cast<float *>(kq_s[1]);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        kd[NCH * r16 + i] = km[i];
        qd[NCH * r16 + i] = qm[i];
      }
    }
  }
  // Also orders every wave's fold reads of the ring before the append below.
  __syncthreads();

  // Per-record decay prefix, record j in lane j: older records from the ring, then this token.
  float al;
  {
    const int j = r16 < nold ? r16 : 0;
    const float a1 = __shfl(al_row, wrap(sb0, j, Ls), kWave);
    al = r16 < nold ? a1 : (r16 == nold ? al_in : 1.f);
  }
  const float g = prefix_sum16(lane < 16 ? __logf(al) : 0.f, lane);
  const float gm = __shfl(g, nold, kWave);
  // Weight of the checkpoint terms (0 for a head the decay skip drops).
  const float egm = (SKIP && gm < kDecaySkipLog) ? 0.f : __expf(gm);
  const float dec = __expf(gm - g);
  const float wk = r16 < nold ? dec * dot_s[0][r16] : 0.f;
  const float wq = r16 < nold ? dec * dot_s[1][r16] : 0.f;
  const float kmq = dot_s[1][15];
  // S0 k_m and S0 q_m for the rows of this lane, then this lane's output row.
  float skr = 0.f, sqr = 0.f;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    float ak = 0.f, aq = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int c4 = colq<NCH, CM>(c, q) >> 2;
      ak += dot4(s[k][c], kq_s[0][c4]);
      aq += dot4(s[k][c], kq_s[1][c4]);
    }
    ak = sum_quarters(ak);
    aq = sum_quarters(aq);
    if (q == k) {
      skr = ak;
      sqr = aq;
    }
  }
  // After a fold of a low-precision read copy the output takes the fold
  // result's products; the cached pseudo-value, those of the read copy (skr).
  const bool from_fold = kLossy && fold;
  const float sk_out = from_fold ? sk_fold : skr, sq_out = from_fold ? sq_fold : sqr;
  float acc_k = 0.f, acc_q = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxOld; ++t) {
    acc_k += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), t)) * uo[t];
    acc_q += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), t)) * uo[t];
  }
  const float uc = be_in * (v_in - egm * skr - acc_k);  // this token's pseudo-value from the window's S0
  const float um = kLossy ? be_in * (v_in - egm * sk_out - acc_k) : uc;  // ... and for its output
  const float o = egm * sq_out + acc_q + kmq * um;

  // 3. Output and append.
  if (q < RBW) {
    a.y[bh * DV + orow] = o;
    rp.ru[(size_t)slot * rp.vs + orow] = uc;
    if constexpr (RF != CF) str<R>(rp.rv + (size_t)slot * rp.vs + orow, v_in);
  }
  if (!zc)
    for (int i = threadIdx.x; i < DK; i += 64 * nwaves) rp.rk[(size_t)slot * rp.ks + i] = kin[i];
  if (threadIdx.x == 0) {
    if (!zc) {
      rp.ral[slot] = al_in;
      rp.rbe[slot] = be_in;
    }
    if (h == 0) {
      a.ptr.pos_out[b] = pos + 1;
      a.ptr.ckpt_out[b] = base;
    }
  }
}

// ---- explicit flush -------------------------------------------------------------
template <int CF, int RF, int NCH, int RBW, typename R, bool SKIP = false>
__global__ __launch_bounds__(256) void gdn_flush(GdnFlushArgs a, StateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  static_assert(!SKIP || (CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32), "decay skip: float32 copies only");
  __shared__ GdnLds<RBW> lds_all[RF != CF ? 4 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  const size_t head = bh * DV * DK;
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  const bool bad = !pointers_ok(pos, ck, L);
  const bool fold = !bad && count > 0 && (a.mask == nullptr || a.mask[b] != 0);
  if (h == 0 && threadIdx.x == 0) {
    if (bad) atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = fold ? pos : ck;
  }
  if (!fold) return;
  const GdnRingPtrs<R> rp = gdn_ring_ptrs<R>(a.ring, sh, b, h);
  const int s0 = fmod_(ck, sh.fLs);
  bool keep = true;  // the checkpoint term survives the decay skip
  if constexpr (SKIP) {
    const int r16 = lane & 15;
    const float aj = rp.ral[wrap(s0, r16 < count ? r16 : 0, sh.Ls)];
    keep = !(sum16(r16 < count ? __logf(aj) : 0.f) < kDecaySkipLog);
  }
  float4 s[RBW][NCH];
  if (keep) {
    typename SIO<CF, NCH, RBW, CM>::Raw rc;
    SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
    SIO<CF, NCH, RBW, CM>::decode(s, rc);
  } else {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) s[k][c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  gdn_fold<CF, RF, NCH, RBW, R, SKIP>(s, count, s0, rp, sh.Ls, rb0, lane, &lds_all[RF != CF ? wave : 0]);
  store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
}

__device__ __forceinline__ floatx4 mfma_4x4x1(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// ---- speculative verify ---------------------------------------------------------
// c committed records (pseudo-values cached in the ring) then T drafts
// (c + T <= L after a fold-first).  Draft d is window record t = c + d:
//   u_t = beta_t v_t - beta_t e^{g_t} S0 k_t - sum_{j<t} beta_t e^{g_t - g_j} (k_j . k_t) u_j
//   o_d = e^{g_t} S0 q_d + sum_{j<=t} e^{g_t - g_j} (k_j . q_d) u_j.
// Up to four drafts, the products run in one pass on
// v_mfma_f32_4x4x1_16b_f32 (16 blocks of 4 x 4 x 1; lane l feeds row / column
// l % 4 of block l / 4 and gets rows 0..3 of column l % 4): with lane
// l = r + 16 q of the register tile, g = r / 4, m = r % 4, block (g, q) takes
// rows 16 rb + 4 g + 0..3 (S0 k_d, S0 q_d) or records 4 g + 0..3 (k_j . k_d,
// k_j . q_d) over the columns of quarter q, and a sum over the quarters
// completes them, so absent drafts cost no MFMA work.  More drafts take one
// v_mfma_f32_16x16x4f32 sweep per eight (section 4).  The drafts' keys and queries and the window's keys
// reach LDS by direct global-to-LDS loads in the lane-linear operand layout
// (bf16 records: a load, exact widening and LDS store in the same layout).
// The draft rows of the triangular system are then solved per state row (one
// lane per row) with the committed rows known.  The drafts' keys, pseudo-
// values and scalars are staged in the ring, so that a commit is only a
// pointer move.
// Per wave; ND = 4 NP drafts at most.
template <int RBW, bool DUAL, int ND = kMaxL>
struct GdnVerifyLds {
  float W[16 * RBW][ND + 1];   // [row][draft]: S0 k_d
  float SQ[16 * RBW][ND + 1];  // [row][draft]: S0 q_d
  float g[16], beta[16];       // record j: decay prefix, beta
  // [record][row of the wave]: the committed records' pseudo-values, then the
  // drafts' values (c + T <= 16), staged by direct global-to-LDS loads issued
  // with the window's keys, so the solve finds them in LDS.
  float wst[16][16 * RBW];
  float WQ[DUAL ? 16 * RBW : 1][ND + 1];  // after a fold-first: Q k_d for the read copy Q (cached pseudo-values)
};

// The fold part only for a re-solving fold-first (a separate read copy).
template <int RBW, bool DUAL, int ND, bool REFOLD>
union GdnWaveLds {
  GdnLds<REFOLD ? RBW : 1> fold;       // a re-solving fold-first
  GdnVerifyLds<RBW, DUAL, ND> verify;  // the drafts (after the fold)
};

// Occupancy target for the float32 copies: three waves per SIMD (at most 168
// VGPRs; the LDS of three workgroups fits a CU).
template <int CF, int RF>
constexpr int verify_waves_per_eu() { return (CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32) ? 4 : 1; }

// SKIP (decay skip, float32 copies): the rule applies to the fold-first and to
// each draft's output, but the checkpoint is always read.
// NP: the most passes of four drafts the launch needs (T <= 4 NP); it sizes the
// drafts' LDS staging, so that short verifies leave LDS for more workgroups.
template <int CF, int RF, int NCH, int RBW, typename R, bool SKIP = false, int NP = kMaxL / 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(verify_waves_per_eu<CF, RF>())))
void gdn_replay_verify(GdnVerifyArgs a, StateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  constexpr int kPass = NP;
  constexpr int RW = 16 * RBW;                     // state rows of one wave
  constexpr bool kStage = sizeof(R) == 4;          // float32 records: staged by 4-byte direct loads
  constexpr bool kLossy = RF != REPLAY_FMT_F32;  // the read copy is not the float32 fold result
  static_assert(!SKIP || (CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32), "decay skip: float32 copies only");
  __shared__ float4 ldsK[NCH][64];                 // [chunk cc][record j + 16 q]: k_j at colq(cc, q)
  __shared__ float4 ldsD[kPass * 2 * NCH * 16];    // [((p 2 + w) NCH + cc) 16 + 4 m + q]: w = 0: k, 1: q of draft 4 p + m
  __shared__ GdnWaveLds<RBW, kLossy, 4 * NP, (CF != RF)> lds_all[4];
  // The draft-record coefficients, the same for every wave: written by wave 0.
  //   cA[d][j] = beta_t e^{g_t - g_j} (k_j . k_t) for j < t, else 0;
  //   cB[d][j] = e^{g_t - g_j} (k_j . q_d) for j <= t, else 0  (t = c + d).
  __shared__ __align__(16) float cA[4 * NP][16], cB[4 * NP][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15, gq = r16 >> 2, m4 = r16 & 3;
  GdnVerifyLds<RBW, kLossy, 4 * NP> &sv = lds_all[wave].verify;
  const Shape &sh = a.s;
  const int T = a.T;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, Ls = sh.Ls, rb0 = wave * RBW, H = sh.H;
  const bool zc = a.in_ring;  // the drafts' k, alpha, beta are already in their ring slots
  const size_t bh = (size_t)b * H + h;
  const size_t head = bh * DV * DK;
  const GdnRingPtrs<R> rp = gdn_ring_ptrs<R>(a.ring, sh, b, h);
  const int row = rb0 * 16 + (lane < 16 * RBW ? lane : 0);  // this lane's row in the solve
  const R *gq_ = static_cast<const R *>(a.q), *gk_ = static_cast<const R *>(a.k), *gv_ = static_cast<const R *>(a.v);
  int sp = 0;  // slot of position pos: draft i lives in slot (pos + i) mod Ls
  auto dq_ = [&](int i) { return gq_ + (((size_t)b * T + i) * H + h) * DK; };
  auto dk_ = [&](int i) { return zc ? rp.rk + (size_t)wrap(sp, i, Ls) * rp.ks : gk_ + (((size_t)b * T + i) * H + h) * DK; };
  auto dv_ = [&](int i) { return gv_ + (((size_t)b * T + i) * H + h) * DV; };
  auto dsc = [&](const float *f, int i) { return f[((size_t)b * T + i) * H + h]; };
  const int npass = min((T + 3) >> 2, kPass);

  // 1. The pointer words first (scalar loads issued ahead of the checkpoint
  //    stream), then, with one stored copy, the window's ring records, so
  //    that their loads do not queue behind the checkpoint's.
  constexpr bool kF32 = CF == REPLAY_FMT_F32 && RF == REPLAY_FMT_F32;
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  __builtin_amdgcn_sched_barrier(0);
  const int count = pos - ck;
  if (count < 0 || count > L || ck < 0) {
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  sp = fmod_(pos, sh.fLs);
  const bool fold = count + T > L;  // implies count >= 1 because T <= L
  const int s0 = fmod_(ck, sh.fLs);
  const int base = fold ? pos : ck, sb0 = fold ? wrap(s0, count, Ls) : s0;
  const int c = pos - base, nrec = c + T;

  // Window records: every key into LDS (committed from the ring, drafts from
  // the input; chunk cc by wave cc % nwaves), and alpha, beta of record r16.
  // The rows of this wave of the committed pseudo-values and of the drafts'
  // values go to the wave's LDS (64 / RW records per load).  With a separate
  // read copy the fold-first uses the same LDS, so these loads follow it.
  auto stage_window = [&]() {
    {
      const int j = r16 < nrec ? r16 : nrec - 1;
      const R *kj = j < c ? rp.rk + (size_t)wrap(sb0, j, Ls) * rp.ks : dk_(j - c);
      for (int cc = wave; cc < NCH; cc += nwaves) stage4<R>(kj + colq<NCH, CM>(cc, q), &ldsK[cc][0], lane);
    }
    if constexpr (kStage) {
      constexpr int kPer = 64 / RW;  // records per load instruction
      typedef __attribute__((address_space(3))) void lds_void;
      const int r = rb0 * 16 + lane % RW;
      const float *ru = rp.ru + r, *vd = reinterpret_cast<const float *>(dv_(0)) + r;
      const size_t vstride = (size_t)H * DV;  // draft to draft in the values input
#pragma unroll
      for (int j0 = 0; j0 < kMaxL; j0 += kPer) {
        if (j0 < nrec) {
          const int j = min(j0 + lane / RW, nrec - 1);
          const float *src = j < c ? ru + (size_t)wrap(sb0, j, Ls) * rp.vs : vd + (size_t)(j - c) * vstride;
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), (lds_void *)&sv.wst[j0][0], 4, 0, 0);
        }
      }
    }
  };
  float al, be;
  {
    const int j = r16 < nrec ? r16 : nrec - 1;
    const float a1 = (j < c || zc) ? rp.ral[wrap(sb0, j, Ls)] : dsc(a.alpha, j - c);
    const float b1 = (j < c || zc) ? rp.rbe[wrap(sb0, j, Ls)] : dsc(a.beta, j - c);
    al = r16 < nrec ? a1 : 1.f;
    be = r16 < nrec ? b1 : 0.f;
  }
  if constexpr (CF == RF) stage_window();

  // 2. The read copy, then the drafts' keys and queries into LDS (load j of
  //    the tile by wave j % nwaves).  Float32 copies load straight into the
  //    tile s; other formats keep the stored bits in raw until decoded.
  float4 s[RBW][NCH];
  typename SIO<RF, NCH, RBW, CM>::Raw raw;
  if constexpr (kF32) load_rows_g<NCH, RBW, CM>(s, static_cast<const float *>(sb.rd.data) + head, rb0, lane);
  else SIO<RF, NCH, RBW, CM>::load(raw, sb.rd, head, rb0, lane);
  {
    const int nload = (npass * 2 * NCH * 16) >> 6;
    for (int j = wave; j < nload; j += nwaves) {
      const int slot = 64 * j + lane;
      const int q2 = slot & 3, m2 = (slot >> 2) & 3, pwc = slot >> 4;  // pwc = (p 2 + w) NCH + cc
      const int cc = pwc % NCH, pw = pwc / NCH;
      const int n = 4 * (pw >> 1) + m2;
      const R *src = (pw & 1) ? dq_(n < T ? n : T - 1) : dk_(n < T ? n : T - 1);
      stage4<R>(src + colq<NCH, CM>(cc, q2), &ldsD[64 * j], lane);
    }
  }
  // 3. Fold-first when the window cannot take T more records.
  if (fold) {
    if constexpr (RF == CF) {
      if constexpr (!kF32) SIO<RF, NCH, RBW, CM>::decode(s, raw);
    } else {
      typename SIO<CF, NCH, RBW, CM>::Raw rc;
      SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
      SIO<CF, NCH, RBW, CM>::decode(s, rc);
    }
    if constexpr (CF != RF) gdn_fold<CF, RF, NCH, RBW, R, SKIP>(s, count, s0, rp, Ls, rb0, lane, &lds_all[wave].fold);
    else gdn_fold<CF, RF, NCH, RBW, R, SKIP>(s, count, s0, rp, Ls, rb0, lane, nullptr);
    // Float32 copies: s already is what the copy holds, stored after the
    // wait below.  Otherwise the drafts' outputs come from the fold result s,
    // and the copies are stored after the passes (4b).
  }
  if constexpr (CF != RF) {
    __syncthreads();  // every wave's fold is done with the LDS the window now takes
    stage_window();
  }
  if constexpr (!kF32)
    if (!fold) SIO<RF, NCH, RBW, CM>::decode(s, raw);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's global-to-LDS loads have landed
  __syncthreads();                // and every other wave's; all ring reads are done
  // A float32 fold-first's checkpoint stores go out only now: loads and stores
  // share one counter, so stores issued before the wait above would hold it
  // until they completed.  They drain during the passes.
  if constexpr (!kLossy)
    if (fold) store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);

  // 4. Record scalars (record j in lane j), then the passes.
  {
    const float gj = prefix_sum16(lane < 16 ? __logf(al) : 0.f, lane);
    if (lane < 16) {
      sv.g[lane] = gj;
      sv.beta[lane] = be;
    }
  }
  wave_lds_sync();
  if constexpr (NP >= 2) {
    // More than four drafts: sweeps over the column chunks on
    // v_mfma_f32_16x16x4f32, eight drafts per sweep, whose 16 output columns
    // n = lane % 16 are k and q of the sweep's drafts (n < 8: k, n >= 8: q).
    // The K index of an MFMA is the lane quarter q, which holds column
    // colq(cc, q) + e of its row in the tile (and of its record in ldsK), so
    // the products need no sum over the quarters: lane (r, q) gets rows
    // 4 q + 0..3 of column n, ready for LDS.
#pragma unroll
    for (int sw = 0; sw < NP / 2; ++sw) {
      const int dn = 8 * sw + (r16 & 7), wn = r16 >> 3;  // draft and vector (0: k, 1: q) of column n
      const float4 *bop = &ldsD[(((dn >> 2) * 2 + wn) * NCH) * 16 + 4 * (dn & 3) + q];  // chunk cc: bop[16 cc]
      floatx4 dd = {0.f, 0.f, 0.f, 0.f}, ws[RBW];
#pragma unroll
      for (int k = 0; k < RBW; ++k) ws[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const float4 bv = bop[16 * cc];
        if (wave == 0) {  // only wave 0's key dots are kept
          const float4 kj = ldsK[cc][lane];
          dd = mfma_16x16x4(kj.x, bv.x, dd);
          dd = mfma_16x16x4(kj.y, bv.y, dd);
          dd = mfma_16x16x4(kj.z, bv.z, dd);
          dd = mfma_16x16x4(kj.w, bv.w, dd);
        }
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
          ws[k] = mfma_16x16x4(s[k][cc].x, bv.x, ws[k]);
          ws[k] = mfma_16x16x4(s[k][cc].y, bv.y, ws[k]);
          ws[k] = mfma_16x16x4(s[k][cc].z, bv.z, ws[k]);
          ws[k] = mfma_16x16x4(s[k][cc].w, bv.w, ws[k]);
        }
      }
      {
        const int t = c + dn;
        const float gt = sv.g[t < kMaxL ? t : kMaxL - 1], bt = sv.beta[t < kMaxL ? t : kMaxL - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * q + i;  // record
          const float e = __expf(gt - sv.g[j]);
          if (wave == 0) {
            if (wn == 0) cA[dn][j] = (dn < T && j < t) ? bt * e * dd[i] : 0.f;
            else cB[dn][j] = (dn < T && j <= t) ? e * dd[i] : 0.f;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < RBW; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (wn == 0) sv.W[16 * k + 4 * q + i][dn] = ws[k][i];
          else sv.SQ[16 * k + 4 * q + i][dn] = ws[k][i];
        }
    }
  } else {
    for (int p = 0; p < npass; ++p) {
      const int d = 4 * p + m4;  // this lane's draft
      const float4 *kd = &ldsD[(p * 2 * NCH) * 16 + 4 * m4 + q];        // k_d at chunk cc: kd[16 cc]
      const float4 *qd = &ldsD[((p * 2 + 1) * NCH) * 16 + 4 * m4 + q];  // q_d at chunk cc: qd[16 cc]
      // One sweep over the column chunks feeds all six accumulation chains, so
      // each chunk of k_d, q_d is read from LDS once and dies at once.
      floatx4 dk = {0.f, 0.f, 0.f, 0.f}, dqq = {0.f, 0.f, 0.f, 0.f}, w[RBW], sq[RBW];
#pragma unroll
      for (int k = 0; k < RBW; ++k) w[k] = sq[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const float4 kv = kd[16 * cc], qv = qd[16 * cc];
        if (wave == 0) {  // only wave 0's key dots are kept
          const float4 kj = ldsK[cc][lane];
          dk = mfma_4x4x1(kj.x, kv.x, dk);
          dqq = mfma_4x4x1(kj.x, qv.x, dqq);
          dk = mfma_4x4x1(kj.y, kv.y, dk);
          dqq = mfma_4x4x1(kj.y, qv.y, dqq);
          dk = mfma_4x4x1(kj.z, kv.z, dk);
          dqq = mfma_4x4x1(kj.z, qv.z, dqq);
          dk = mfma_4x4x1(kj.w, kv.w, dk);
          dqq = mfma_4x4x1(kj.w, qv.w, dqq);
        }
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
          w[k] = mfma_4x4x1(s[k][cc].x, kv.x, w[k]);
          sq[k] = mfma_4x4x1(s[k][cc].x, qv.x, sq[k]);
          w[k] = mfma_4x4x1(s[k][cc].y, kv.y, w[k]);
          sq[k] = mfma_4x4x1(s[k][cc].y, qv.y, sq[k]);
          w[k] = mfma_4x4x1(s[k][cc].z, kv.z, w[k]);
          sq[k] = mfma_4x4x1(s[k][cc].z, qv.z, sq[k]);
          w[k] = mfma_4x4x1(s[k][cc].w, kv.w, w[k]);
          sq[k] = mfma_4x4x1(s[k][cc].w, qv.w, sq[k]);
        }
        if constexpr (NP != 1) __builtin_amdgcn_sched_barrier(0);  // keep each chunk's LDS reads with its MFMAs (register pressure)
      }
      if (wave == 0) {
        float kk[4], kq[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kk[v] = sum_quarters(dk[v]);
          kq[v] = sum_quarters(dqq[v]);
        }
        if (q == 0) {
          const int t = c + d;
          const float gt = sv.g[t < kMaxL ? t : kMaxL - 1], bt = sv.beta[t < kMaxL ? t : kMaxL - 1];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = 4 * gq + v;  // record
            const float e = __expf(gt - sv.g[j]);
            cA[d][j] = (d < T && j < t) ? bt * e * kk[v] : 0.f;
            cB[d][j] = (d < T && j <= t) ? e * kq[v] : 0.f;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < RBW; ++k) {
        float wv[4], sqv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          wv[v] = sum_quarters(w[k][v]);
          sqv[v] = sum_quarters(sq[k][v]);
        }
        if (q == 0) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            sv.W[16 * k + 4 * gq + v][d] = wv[v];
            sv.SQ[16 * k + 4 * gq + v][d] = sqv[v];
          }
        }
      }
    }
  }
  __syncthreads();  // wave 0's coefficients and each wave's own tables are in LDS

  // 4b. After a fold-first of a low-precision read copy: store both copies,
  //     then Q k_d from the read copy Q they now hold, for the pseudo-values
  //     the ring caches (the window's next steps read Q).
  if constexpr (kLossy) {
    if (fold) {
      store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
      for (int p = 0; p < npass; ++p) {
        const int d = 4 * p + m4;
        const float4 *kd = &ldsD[(p * 2 * NCH) * 16 + 4 * m4 + q];
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
          floatx4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc) {
            const float4 kv = kd[16 * cc];
            w = mfma_4x4x1(s[k][cc].x, kv.x, w);
            w = mfma_4x4x1(s[k][cc].y, kv.y, w);
            w = mfma_4x4x1(s[k][cc].z, kv.z, w);
            w = mfma_4x4x1(s[k][cc].w, kv.w, w);
          }
          float wv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) wv[v] = sum_quarters(w[v]);
          if (q == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) sv.WQ[16 * k + 4 * gq + v][d] = wv[v];
          }
        }
      }
      wave_lds_sync();
    }
  }

  // 5. The drafts' rows of the system and their outputs, one lane per state row.
  //    This row of the committed pseudo-values and of the drafts' values is
  //    loaded only now: held through the passes above it would cost a wave per
  //    SIMD.
  if (lane < 16 * RBW) {
    // u[t]: this row of pseudo-value t (committed, then solved); vrow[d] (bf16
    // records only): this row of draft d's value.  Float32 records come from
    // the wave's LDS (staged in section 3): wst[t] is committed u_t for t < c
    // and the value of draft t - c after.
    float u[kMaxL], vrow[kStage ? 1 : kMaxL];
    if constexpr (kStage) {
#pragma unroll
      for (int j = 0; j < kMaxL; ++j) u[j] = j < c ? sv.wst[j][lane] : 0.f;
    } else {
#pragma unroll
      for (int j = 0; j < kMaxL; ++j) {
        const int jc = j < c ? j : 0;
        const float v = rp.ru[(size_t)wrap(sb0, jc, Ls) * rp.vs + row];
        u[j] = j < c ? v : 0.f;
      }
#pragma unroll
      for (int d = 0; d < kMaxL; ++d) vrow[d] = ldr<R>(dv_(d < T ? d : T - 1) + row);
    }
    auto vval = [&](int t) { return kStage ? sv.wst[t][lane] : vrow[t - c]; };  // value of window record t
    const bool dual = kLossy && fold;  // outputs from the fold result, cached values from the read copy
#pragma unroll
    for (int t = 0; t < kMaxL; ++t) {
      if (t >= c && t < nrec) {
        const int d = t - c;
        const float bt = sv.beta[t];
        const float et = (SKIP && sv.g[t] < kDecaySkipLog) ? 0.f : __expf(sv.g[t]);  // checkpoint-term weight
        float v = bt * vval(t) - bt * et * sv.W[lane][d];
#pragma unroll
        for (int j = 0; j < t; ++j) v -= cA[d][j] * u[j];
        u[t] = v;
        float o = et * sv.SQ[lane][d];
#pragma unroll
        for (int j = 0; j <= t; ++j) o += cB[d][j] * u[j];
        a.y[(((size_t)b * T + d) * H + h) * DV + row] = o;
        if (!dual) rp.ru[(size_t)wrap(sb0, t, Ls) * rp.vs + row] = v;  // stage the pseudo-value
        if constexpr (RF != CF) str<R>(rp.rv + (size_t)wrap(sb0, t, Ls) * rp.vs + row, vval(t));
      }
    }
    if constexpr (kLossy) {
      if (dual) {  // c = 0 after a fold-first: the drafts are the whole window
#pragma unroll
        for (int t = 0; t < kMaxL; ++t) {
          if (t < nrec) {
            const float bt = sv.beta[t], et = __expf(sv.g[t]);
            float v = bt * vval(t) - bt * et * sv.WQ[lane][t];
#pragma unroll
            for (int j = 0; j < t; ++j) v -= cA[t][j] * u[j];
            u[t] = v;
            rp.ru[(size_t)wrap(sb0, t, Ls) * rp.vs + row] = v;
          }
        }
      }
    }
  }
  // 6. Stage the drafts' keys and scalars (unless the producer put them in the
  //    ring) from what the workgroup already holds, so that no store waits for
  //    a load: the keys from the passes' LDS operand (one 16-byte piece per
  //    thread), alpha and beta from the lanes of wave 0 that hold record r16.
  //    The workgroup barrier above already ordered every wave's reads of the
  //    folded slots before these writes.
  if (!zc) {
    constexpr int kPieces = NCH * 4;  // 16-byte pieces of a key
    for (int e = threadIdx.x; e < T * kPieces; e += 64 * nwaves) {
      const int d = e / kPieces, rem = e - d * kPieces, cc = rem >> 2, q2 = rem & 3;
      const float4 kv = ldsD[((d >> 2) * 2 * NCH + cc) * 16 + 4 * (d & 3) + q2];
      str4<R>(rp.rk + (size_t)wrap(sb0, c + d, Ls) * rp.ks + colq<NCH, CM>(cc, q2), kv);
    }
    if (wave == 0 && q == 0 && r16 >= c && r16 < nrec) {
      const int sl = wrap(sb0, r16, Ls);
      rp.ral[sl] = al;
      rp.rbe[sl] = be;
    }
  }
  if (h == 0 && threadIdx.x == 0) {
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- state encode: a float32 state into both stored copies -------------------------
// The stochastic-rounding counter uses each sequence's current ckpt_pos.
template <int CF, int RF, int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_encode_state(EncodeArgs a, StateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, rb0 = wave * RBW;
  const size_t head = ((size_t)b * sh.H + h) * DV * DK;
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW, CM>(s, a.src + head, rb0, lane);
  const SRKey key{sb.seed_lo, sb.seed_hi, (uint32_t)h, (uint32_t)b, (uint32_t)a.ckpt_pos[b]};
  if (a.write_ckpt) {
    typename SIO<CF, NCH, RBW, CM>::Raw rc;
    SIO<CF, NCH, RBW, CM>::encode(rc, s, rb0, lane, key);
    SIO<CF, NCH, RBW, CM>::write(rc, sb.ck, head, rb0, lane);
  }
  if constexpr (RF != CF) {
    typename SIO<RF, NCH, RBW, CM>::Raw rr;
    if constexpr (RF == REPLAY_FMT_F4E2M1_CS) SIO<RF, NCH, RBW, CM>::prepare(rr, s, lane, wave);
    SIO<RF, NCH, RBW, CM>::encode(rr, s, rb0, lane, key);
    SIO<RF, NCH, RBW, CM>::write(rr, sb.rd, head, rb0, lane);
  }
}

// ---- baselines: conventional step and snapshot-per-draft verify ----------------
// One token of the stepwise recurrence on the register tile:
//   Sk = S k;  S <- alpha S + (beta v - alpha beta Sk) k^T;  o = S q.
template <int NCH, int RBW, typename R>
__device__ __forceinline__ void gdn_update_rows(float4 (&s)[RBW][NCH], const R *qin, const R *kin, const R *vin,
                                                float alpha, float beta, int rb0, int lane,
                                                float *o_rows /* nullptr: no store */, int vrow0 = 0) {
  constexpr int CM = kColIlv;
  const int q = lane >> 4, r16 = lane & 15;
  float4 kv[NCH], qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    kv[c] = ldr4<R>(kin + colq<NCH, CM>(c, q));
    qv[c] = ldr4<R>(qin + colq<NCH, CM>(c, q));
  }
  float acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
    float sk = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) sk += dot4(s[k][c], kv[c]);
    sk = sum_quarters(sk);
    const float coef = beta * ldr<R>(vin + (row - vrow0)) - alpha * beta * sk;  // vin holds rows vrow0 ..
    float so = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float4 &e = s[k][c];
      e.x = alpha * e.x + coef * kv[c].x;
      e.y = alpha * e.y + coef * kv[c].y;
      e.z = alpha * e.z + coef * kv[c].z;
      e.w = alpha * e.w + coef * kv[c].w;
      so += dot4(e, qv[c]);
    }
    acc[k] = sum_quarters(so);
  }
  if (o_rows && q < RBW) {
    float v = acc[0];
#pragma unroll
    for (int k = 1; k < RBW; ++k) v = (q == k) ? acc[k] : v;
    o_rows[(rb0 + q) * 16 + r16] = v;
  }
}

template <int NCH, int RBW, typename R>
__global__ __launch_bounds__(256) void gdn_conv_step(GdnConvArgs a) {
  constexpr int DK = 16 * NCH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  float *S = a.state + bh * DV * DK;
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW, kColIlv>(s, S, rb0, lane);
  gdn_update_rows<NCH, RBW, R>(s, static_cast<const R *>(a.q) + bh * DK, static_cast<const R *>(a.k) + bh * DK,
                               static_cast<const R *>(a.v) + bh * DV, a.alpha[bh], a.beta[bh], rb0, lane,
                               a.y + bh * DV);
  store_rows_g<NCH, RBW, kColIlv>(s, S, rb0, lane);
}

// Bytes one draft takes in a wave's LDS region of the snapshot baseline: its q
// and k, and v at the wave's rows.
template <int NCH, int RBW, typename R>
constexpr int gsnap_lds_draft() { return 2 * 16 * NCH * (int)sizeof(R) + 16 * RBW * (int)sizeof(R); }

// Every draft's q, k and v (at the wave's rows) are staged into the wave's LDS
// region by direct global-to-LDS loads before the first snapshot store, so the
// draft loop issues no global load: a load issued after stores waits for them
// to complete, which would serialise the T snapshot writes.
template <int NCH, int RBW, typename R>
__global__ __launch_bounds__(256) void gdn_snapshot_verify(GdnSnapArgs a) {
  constexpr int DK = 16 * NCH;
  constexpr int kVec = DK * (int)sizeof(R), kDraft = gsnap_lds_draft<NCH, RBW, R>();
  extern __shared__ __align__(16) unsigned char gdn_snap_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Shape &sh = a.s;
  const int T = a.T, H = sh.H, DV = sh.P, rb0 = wave * RBW;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * H;
  const int cur = a.cur[b];
  if (cur < 0 || cur >= a.nslots) return;  // never index outside the slot array
  auto slot_ptr = [&](int sl) { return a.slots + (((size_t)b * a.nslots + sl) * H + h) * (size_t)DV * DK; };
  unsigned char *wl = gdn_snap_lds + (size_t)wave * T * kDraft;
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW, kColIlv>(s, slot_ptr(cur), rb0, lane);
  for (int i = 0; i < T; ++i) {
    const size_t d = ((size_t)b * T + i) * H + h;
    dma_vec<DK, R>(static_cast<const R *>(a.q) + d * DK, wl + i * kDraft, lane);
    dma_vec<DK, R>(static_cast<const R *>(a.k) + d * DK, wl + i * kDraft + kVec, lane);
    dma_vec<16 * RBW, R>(static_cast<const R *>(a.v) + d * DV + rb0 * 16, wl + i * kDraft + 2 * kVec, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's global-to-LDS loads have landed
  wave_lds_sync();
  for (int i = 0; i < T; ++i) {
    const size_t d = ((size_t)b * T + i) * H + h;
    gdn_update_rows<NCH, RBW, R>(s, reinterpret_cast<const R *>(wl + i * kDraft),
                                 reinterpret_cast<const R *>(wl + i * kDraft + kVec),
                                 reinterpret_cast<const R *>(wl + i * kDraft + 2 * kVec), a.alpha[d], a.beta[d], rb0,
                                 lane, a.y + d * DV, rb0 * 16);
    store_rows_g<NCH, RBW, kColIlv>(s, slot_ptr((cur + 1 + i) % a.nslots), rb0, lane);
  }
}

// ---- dispatch -----------------------------------------------------------------
// Four waves per head, RBW = d_v / 64 row blocks per wave (d_v in {64, 128}).
// Format pairs (checkpoint, read copy): (f32, f32) for every d_k in {32, 64,
// 128}; the low-precision pairs at d_k = 128.
#define RSSM_FMT_PAIRS(X)                                                                           \
  X(REPLAY_FMT_F32, REPLAY_FMT_F4E2M1_B16)                                                          \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F4E2M1_B16)                                                       \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F4E2M1_B16)                                                       \
  X(REPLAY_FMT_F32, REPLAY_FMT_F4E2M1_CS)                                                           \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F4E2M1_CS)                                                        \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F4E2M1_CS)                                                        \
  X(REPLAY_FMT_F4E2M1_B16, REPLAY_FMT_F4E2M1_B16)                                                   \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F16_SR)                                                           \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F8E4M3)

// LP: the low-precision format pairs are instantiated too (not with the decay skip).
template <template <int, int, int, int> class K, bool LP = true, typename Args>
int gdn_dispatch(const Args &a, const StateBufs &sb, int cf, int rf, hipStream_t st) {
  const int DK = a.s.N, DV = a.s.P;
  if (DV != 64 && DV != 128) return (int)hipErrorInvalidValue;
  const int rbw = DV / 64;
  const dim3 grid((unsigned)((size_t)a.s.B * a.s.H)), block(256);
#define RSSM_CASE(CF_, RF_, NCH_, RBW_)                                             \
  if (cf == CF_ && rf == RF_ && DK == 16 * NCH_ && rbw == RBW_) {                   \
    hipLaunchKernelGGL((K<CF_, RF_, NCH_, RBW_>::fn), grid, block, 0, st, a, sb); \
    return (int)hipGetLastError();                                                  \
  }
#define RSSM_F32(NCH_) RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, NCH_, 1) RSSM_CASE(REPLAY_FMT_F32, REPLAY_FMT_F32, NCH_, 2)
  RSSM_F32(2) RSSM_F32(4) RSSM_F32(8)
  if constexpr (LP) {
#define RSSM_Q(CF_, RF_) RSSM_CASE(CF_, RF_, 8, 1) RSSM_CASE(CF_, RF_, 8, 2)
    RSSM_FMT_PAIRS(RSSM_Q)
#undef RSSM_Q
  }
#undef RSSM_F32
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}

template <template <int, int> class K, typename Args>
int gdn_dispatch_f32(const Args &a, hipStream_t st) {
  const int DK = a.s.N, DV = a.s.P;
  if (DV != 64 && DV != 128) return (int)hipErrorInvalidValue;
  const int rbw = DV / 64;
  const dim3 grid((unsigned)((size_t)a.s.B * a.s.H)), block(256);
#define RSSM_CASE(NCH_, RBW_)                                       \
  if (DK == 16 * NCH_ && rbw == RBW_) {                             \
    hipLaunchKernelGGL((K<NCH_, RBW_>::fn), grid, block, 0, st, a); \
    return (int)hipGetLastError();                                  \
  }
  RSSM_CASE(2, 1) RSSM_CASE(4, 1) RSSM_CASE(8, 1) RSSM_CASE(2, 2) RSSM_CASE(4, 2) RSSM_CASE(8, 2)
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}

// Kernel wrappers over the record element type (float32, or bf16 records).
#define RSSM_WRAP4(name, kern)                                    \
  template <typename R, bool SKIP = false>                        \
  struct name {                                                   \
    template <int CF, int RF, int NCH, int RBW>                   \
    struct K {                                                    \
      static constexpr auto fn = kern<CF, RF, NCH, RBW, R, SKIP>; \
    };                                                            \
  };
RSSM_WRAP4(GStepK, gdn_replay_step)
RSSM_WRAP4(GFlushK, gdn_flush)
#undef RSSM_WRAP4
// The verify by its largest pass count NP (T <= 4 NP).
#define RSSM_WRAPV(name, NP_)                                                        \
  template <typename R, bool SKIP = false>                                           \
  struct name {                                                                      \
    template <int CF, int RF, int NCH, int RBW>                                      \
    struct K {                                                                       \
      static constexpr auto fn = gdn_replay_verify<CF, RF, NCH, RBW, R, SKIP, NP_>; \
    };                                                                               \
  };
RSSM_WRAPV(GVerifyK1, 1)
RSSM_WRAPV(GVerifyK2, 2)
RSSM_WRAPV(GVerifyK4, 4)
#undef RSSM_WRAPV
template <int CF, int RF, int NCH, int RBW>
struct GEncodeK {
  static constexpr auto fn = gdn_encode_state<CF, RF, NCH, RBW>;
};
#define RSSM_WRAP(name, kern)                       \
  template <typename R>                             \
  struct name {                                     \
    template <int NCH, int RBW>                     \
    struct K {                                      \
      static constexpr auto fn = kern<NCH, RBW, R>; \
    };                                              \
  };
RSSM_WRAP(GConvK, gdn_conv_step)
#undef RSSM_WRAP

// By the record element type and the decay skip (float32 copies only).
template <template <typename, bool> class W, typename Args>
int launch_gdn(const Args &a, const FormatBufs &f, hipStream_t st) {
  const StateBufs sb = state_bufs(f);
  if (a.decay_skip)
    return a.bf16 ? gdn_dispatch<W<bf16_t, true>::template K, false>(a, sb, f.ckpt_fmt, f.read_fmt, st)
                  : gdn_dispatch<W<float, true>::template K, false>(a, sb, f.ckpt_fmt, f.read_fmt, st);
  return a.bf16 ? gdn_dispatch<W<bf16_t, false>::template K>(a, sb, f.ckpt_fmt, f.read_fmt, st)
                : gdn_dispatch<W<float, false>::template K>(a, sb, f.ckpt_fmt, f.read_fmt, st);
}

}  // namespace

int launch_gdn_step(const GdnStepArgs &a, const FormatBufs &f, hipStream_t st) { return launch_gdn<GStepK>(a, f, st); }
int launch_gdn_flush(const GdnFlushArgs &a, const FormatBufs &f, hipStream_t st) { return launch_gdn<GFlushK>(a, f, st); }
int launch_gdn_verify(const GdnVerifyArgs &a, const FormatBufs &f, hipStream_t st) {
  if (a.T <= 4) return launch_gdn<GVerifyK1>(a, f, st);
  if (a.T <= 8) return launch_gdn<GVerifyK2>(a, f, st);
  return launch_gdn<GVerifyK4>(a, f, st);
}
int launch_encode_state(const EncodeArgs &a, const FormatBufs &f, hipStream_t st) {
  return gdn_dispatch<GEncodeK>(a, state_bufs(f), f.ckpt_fmt, f.read_fmt, st);
}
int launch_gdn_conv(const GdnConvArgs &a, hipStream_t st) {
  return a.bf16 ? gdn_dispatch_f32<GConvK<bf16_t>::template K>(a, st) : gdn_dispatch_f32<GConvK<float>::template K>(a, st);
}
// The snapshot baseline takes T gsnap_lds_draft bytes of dynamic LDS per wave.
template <typename R>
int launch_gsnap_r(const GdnSnapArgs &a, hipStream_t st) {
  const int DK = a.s.N, DV = a.s.P;
  if (DV != 64 && DV != 128) return (int)hipErrorInvalidValue;
  const int rbw = DV / 64;
  const dim3 grid((unsigned)((size_t)a.s.B * a.s.H)), block(256);
#define RSSM_CASE(NCH_, RBW_)                                                                  \
  if (DK == 16 * NCH_ && rbw == RBW_) {                                                        \
    const size_t lds = (size_t)4 * a.T * gsnap_lds_draft<NCH_, RBW_, R>();                    \
    if (lds > 65536) {                                                                         \
      const hipError_t e = hipFuncSetAttribute((const void *)gdn_snapshot_verify<NCH_, RBW_, R>, \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                               (int)lds);                                      \
      if (e != hipSuccess) return (int)e;                                                      \
    }                                                                                          \
    hipLaunchKernelGGL((gdn_snapshot_verify<NCH_, RBW_, R>), grid, block, lds, st, a);         \
    return (int)hipGetLastError();                                                             \
  }
  RSSM_CASE(2, 1) RSSM_CASE(4, 1) RSSM_CASE(8, 1) RSSM_CASE(2, 2) RSSM_CASE(4, 2) RSSM_CASE(8, 2)
#undef RSSM_CASE
  return (int)hipErrorInvalidValue;
}
int launch_gdn_snapshot(const GdnSnapArgs &a, hipStream_t st) {
  return a.bf16 ? launch_gsnap_r<bf16_t>(a, st) : launch_gsnap_r<float>(a, st);
}

}  // namespace rssm
