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
// Tile = one (sequence, head); four waves, each holding 16 RBW rows (d_v
// indices) of S0 in registers in the layout shared with the Mamba-2 kernels:
//     s[k][c] = S[16 (rb0 + k) + (l % 16)][16 c + 4 (l / 16) + 0..3].
// Per wave, with X = the window's keys in MFMA operand layout (lane (j, q)
// holds k_j[16 c + 4 q + 0..3], j = l % 16):
//   * W = S0 X^T (one v_mfma_f32_16x16x4f32 pass: M = row, N = record, K = d_k),
//   * the Gram matrix X X^T from the same operand registers,
//   * S0 q and k_j . q on the VALU (q has its own registers),
//   * W goes through per-wave LDS so that each lane owns one row and runs the
//     m x m forward substitution for it with no cross-lane traffic,
//   * a fold is the transposed MFMA rank-m update S^T += K^T U~^T whose output
//     layout equals the register layout of S0.
#include "internal.h"

namespace rssm {
namespace {

template <int RBW>
struct GdnLds {
  float W[16 * RBW][20];      // [row][record]: S0 k_j; column 16: S0 q
  float gram[16][17];         // k_t . k_j
  float A[16][17];            // beta_t e^{g_t - g_j} (k_t . k_j) for j < t, else 0
  float c1[16], c2[16];       // beta_t, beta_t e^{g_t}
  float dq[16];               // e^{g_m - g_j} (k_j . q)
  float us[16];               // e^{g_m - g_j}: pseudo-value weight in a fold
  float kq[16];               // k_j . q
  float g[16], beta[16];
  float U[16][16 * RBW + 4];  // pseudo-values u_t [record][row] (want_u)
};

// Program-order fence for LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

template <int NCH, int RBW>
__device__ __forceinline__ void load_rows_g(float4 (&s)[RBW][NCH], const float *S, int rb0, int lane) {
  constexpr int DK = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s[k][c] = ld4(S + (size_t)row * DK + 16 * c + 4 * q);
  }
}

template <int NCH, int RBW>
__device__ __forceinline__ void store_rows_g(const float4 (&s)[RBW][NCH], float *S, int rb0, int lane) {
  constexpr int DK = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) st4(S + (size_t)row * DK + 16 * c + 4 * q, s[k][c]);
  }
}

// The window of one wave: records 0..m-1 (keys in X, lane j's alpha_j, beta_j
// in al/be, this lane's row of v_t in vr[t] for lanes < 16 RBW).
// Computes the pseudo-values of every record for the wave's rows, and
//   want_o: the newest output o_{m-1} for row `lane` (lanes < 16 RBW), using q (qv);
//   want_u: the pseudo-values u_t in sm.U[t][row] (their fold weights in sm.us).
// Returns the output (or 0).
template <int NCH, int RBW>
__device__ __forceinline__ float gdn_window(const float4 (&s)[RBW][NCH], const float4 (&X)[NCH],
                                            const float4 (&qv)[NCH], int m, float al, float be,
                                            const float (&vr)[16], bool want_o, bool want_u, GdnLds<RBW> &sm,
                                            int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  // W = S0 X^T and the Gram matrix, both MFMA; S0 q and k . q on the VALU.
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
  float kq = 0.f;
  if (want_o) {
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      float v = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) v += dot4(s[k][c], qv[c]);
      v = sum_quarters(v);
      if (q == 0) sm.W[16 * k + r16][16] = v;
    }
    float p = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) p += dot4(X[c], qv[c]);
    kq = sum_quarters(p);  // lane (j, .): k_j . q
  }
  // Per-record scalars, record j in lane j (lanes 0..15).
  const float la = lane < m ? __logf(al) : 0.f;
  const float g = prefix_sum16(la, lane);
  const float gm = __shfl(g, m - 1, kWave);
  if (lane < 16) {
    sm.g[lane] = g;
    sm.beta[lane] = lane < m ? be : 0.f;
    sm.c1[lane] = lane < m ? be : 0.f;
    sm.c2[lane] = lane < m ? be * __expf(g) : 0.f;
    sm.dq[lane] = lane < m ? __expf(gm - g) * kq : 0.f;
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
  float o = 0.f;
  if (lane < 16 * RBW) {
    // Forward substitution for this lane's row; u[t] kept in registers.
    float u[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = 0.f;
      if (t < m) {
        v = sm.c1[t] * vr[t] - sm.c2[t] * sm.W[lane][t];
#pragma unroll
        for (int j = 0; j < t; ++j) v -= sm.A[t][j] * u[j];
      }
      u[t] = v;
    }
    if (want_o) {
      o = __expf(gm) * sm.W[lane][16];
#pragma unroll
      for (int j = 0; j < 16; ++j) o += sm.dq[j] * u[j];
    }
    if (want_u) {
#pragma unroll
      for (int t = 0; t < 16; ++t) sm.U[t][lane] = u[t];
    }
  }
  wave_lds_sync();
  return o;
}

// s <- e^{g_{cnt-1}} s + sum_t e^{g_{cnt-1} - g_t} u_t k_t^T for the cnt window
// records, with u_t and the weights already in sm.U and sm.us (gdn_window with
// want_u).  The MFMA A operand k_{4 st + q}[16 c + r16] is read from the ring
// (cache-resident).
template <int NCH, int RBW>
__device__ __forceinline__ void gdn_fold_apply(float4 (&s)[RBW][NCH], int cnt, int s0, const float *rk, size_t ks,
                                               int L, float escale, GdnLds<RBW> &sm, int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int nsteps = (cnt + 3) >> 2;
  float aK[NCH][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int r = 4 * st + q;
    const float *kr = rk + (size_t)wrap(s0, r < cnt ? r : cnt - 1, L) * ks;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float v = kr[16 * c + r16];
      aK[c][st] = r < cnt ? v : 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    float ub[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) ub[st] = sm.us[4 * st + q] * sm.U[4 * st + q][16 * k + r16];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 acc = {s[k][c].x * escale, s[k][c].y * escale, s[k][c].z * escale, s[k][c].w * escale};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if (st < nsteps) acc = mfma_16x16x4(aK[c][st], ub[st], acc);
      s[k][c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

struct GdnRingPtrs {
  float *rk, *rv, *ral, *rbe;  // head bases: k, v slot-major; alpha, beta per head row
  size_t ks, vs;               // slot strides of the k and v rings
};

__device__ __forceinline__ GdnRingPtrs gdn_ring_ptrs(const GdnRing &r, const Shape &sh, int b, int h) {
  GdnRingPtrs p;
  const size_t bh = (size_t)b * sh.H + h;
  p.ks = (size_t)sh.B * sh.H * sh.N;
  p.vs = (size_t)sh.B * sh.H * sh.P;
  p.rk = r.k + bh * sh.N;
  p.rv = r.v + bh * sh.P;
  p.ral = r.alpha + bh * sh.L;
  p.rbe = r.beta + bh * sh.L;
  return p;
}

// Keys of window records 0..cnt-1 at ring positions starting at slot s0, in
// operand layout (zeros beyond cnt); the record at index `last` (if >= 0) is
// taken from kin instead of the ring.
template <int NCH>
__device__ __forceinline__ void load_keys(float4 (&X)[NCH], int cnt, int last, const float *kin, const GdnRingPtrs &rp,
                                          int s0, int L, int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int j = r16 < cnt ? r16 : cnt - 1;
  const float *kj = (j == last) ? kin : rp.rk + (size_t)wrap(s0, j, L) * rp.ks;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float4 v = ld4(kj + 16 * c + 4 * q);
    X[c] = r16 < cnt ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// This lane's row of v_t for t < cnt (lanes < 16 RBW), record `last` from vin.
template <int RBW>
__device__ __forceinline__ void load_vrows(float (&vr)[16], int cnt, int last, const float *vin, const GdnRingPtrs &rp,
                                           int s0, int L, int rb0, int lane) {
  const int row = rb0 * 16 + (lane < 16 * RBW ? lane : 0);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int tc = t < cnt ? t : cnt - 1;
    const float *vt = (tc == last) ? vin : rp.rv + (size_t)wrap(s0, tc, L) * rp.vs;
    const float v = vt[row];
    vr[t] = t < cnt ? v : 0.f;
  }
}

// ---- replay step ------------------------------------------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_replay_step(GdnStepArgs a) {
  constexpr int DK = 16 * NCH;
  __shared__ GdnLds<RBW> lds_all[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  GdnLds<RBW> &sm = lds_all[wave];
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  float *S = a.ckpt + bh * DV * DK;
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  const float *qin = a.q + bh * DK, *kin = a.k + bh * DK, *vin = a.v + bh * DV;

  // 1. Checkpoint rows first, then what needs no pointer.
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW>(s, S, rb0, lane);
  float4 qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) qv[c] = ld4(qin + 16 * c + 4 * q);
  const float al_row = rp.ral[r16 < L ? r16 : 0], be_row = rp.rbe[r16 < L ? r16 : 0];
  const float al_in = a.alpha[bh], be_in = a.beta[bh];

  // 2. Pointers.
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  if (count < 0 || count > L) {
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  const bool fold = count == L;
  const int s0 = fmod_(ck, sh.fL);
  const int slot = wrap(s0, count, L);  // this token's slot
  int base = ck, sb = s0;
  float4 X[NCH];
  float vr[16];
  if (fold) {
    // Fold the full window (all records in the ring), store, restart the window.
    load_keys<NCH>(X, L, -1, kin, rp, s0, L, lane);
    load_vrows<RBW>(vr, L, -1, vin, rp, s0, L, rb0, lane);
    const float al = __shfl(al_row, wrap(s0, r16, L), kWave), be = __shfl(be_row, wrap(s0, r16, L), kWave);
    gdn_window<NCH, RBW>(s, X, qv, L, al, be, vr, false, true, sm, lane);
    float gl = sm.g[L - 1];
    gdn_fold_apply<NCH, RBW>(s, L, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
    store_rows_g<NCH, RBW>(s, S, rb0, lane);
    base = pos;
    sb = slot;
  }
  const int m = pos - base + 1;
  load_keys<NCH>(X, m, m - 1, kin, rp, sb, L, lane);
  load_vrows<RBW>(vr, m, m - 1, vin, rp, sb, L, rb0, lane);
  float al, be;
  {
    const int j = r16 < m - 1 ? r16 : 0;
    const float a1 = __shfl(al_row, wrap(sb, j, L), kWave), b1 = __shfl(be_row, wrap(sb, j, L), kWave);
    al = r16 < m - 1 ? a1 : (r16 == m - 1 ? al_in : 1.f);
    be = r16 < m - 1 ? b1 : (r16 == m - 1 ? be_in : 0.f);
  }
  const float o = gdn_window<NCH, RBW>(s, X, qv, m, al, be, vr, true, false, sm, lane);

  // 3. Output and append.  After a fold the slot being written held the
  //    oldest folded record, which every wave of the tile read.
  if (fold) __syncthreads();
  if (lane < 16 * RBW) {
    const int row = rb0 * 16 + lane;
    a.y[bh * DV + row] = o;
    rp.rv[(size_t)slot * rp.vs + row] = vin[row];
  }
  for (int i = threadIdx.x; i < DK; i += 64 * nwaves) rp.rk[(size_t)slot * rp.ks + i] = kin[i];
  if (threadIdx.x == 0) {
    rp.ral[slot] = al_in;
    rp.rbe[slot] = be_in;
    if (h == 0) {
      a.ptr.pos_out[b] = pos + 1;
      a.ptr.ckpt_out[b] = base;
    }
  }
}

// ---- explicit flush -------------------------------------------------------------
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_flush(GdnFlushArgs a) {
  constexpr int DK = 16 * NCH;
  __shared__ GdnLds<RBW> lds_all[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  GdnLds<RBW> &sm = lds_all[wave];
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  const bool bad = count < 0 || count > L;
  const bool fold = !bad && count > 0 && (a.mask == nullptr || a.mask[b] != 0);
  if (h == 0 && threadIdx.x == 0) {
    if (bad) atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = fold ? pos : ck;
  }
  if (!fold) return;
  float *S = a.ckpt + bh * DV * DK;
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW>(s, S, rb0, lane);
  const int s0 = fmod_(ck, sh.fL);
  float4 X[NCH], qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) qv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  float vr[16];
  load_keys<NCH>(X, count, -1, nullptr, rp, s0, L, lane);
  load_vrows<RBW>(vr, count, -1, nullptr, rp, s0, L, rb0, lane);
  const int j = r16 < count ? r16 : 0;
  const float al = rp.ral[wrap(s0, j, L)], be = rp.rbe[wrap(s0, j, L)];
  gdn_window<NCH, RBW>(s, X, qv, count, al, be, vr, false, true, sm, lane);
  const float gl = sm.g[count - 1];
  gdn_fold_apply<NCH, RBW>(s, count, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
  store_rows_g<NCH, RBW>(s, S, rb0, lane);
}

// ---- speculative verify ---------------------------------------------------------
// c committed records then T drafts (c + T <= L after a fold-first).  One
// forward substitution over all c + T records; draft i's output is
//   o_i = e^{g_{c+i}} S0 q_i + sum_{j <= c+i} e^{g_{c+i} - g_j} (k_j . q_i) u_j.
// S0 q_i is a second MFMA pass over the queries, k_j . q_i an MFMA of the key
// and query operand registers.
template <int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_replay_verify(GdnVerifyArgs a) {
  constexpr int DK = 16 * NCH;
  __shared__ GdnLds<RBW> lds_all[4];
  __shared__ float SQ_all[4][16 * RBW][17];  // [row][draft]: S0 q_i
  __shared__ float KQ_all[4][16][17];        // [record][draft]: k_j . q_i
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  GdnLds<RBW> &sm = lds_all[wave];
  float(&SQ)[16 * RBW][17] = SQ_all[wave];
  float(&KQ)[16][17] = KQ_all[wave];
  const Shape &sh = a.s;
  const int T = a.T;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW, H = sh.H;
  const size_t bh = (size_t)b * H + h;
  float *S = a.ckpt + bh * DV * DK;
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  auto dq_ = [&](int i) { return a.q + (((size_t)b * T + i) * H + h) * DK; };
  auto dk_ = [&](int i) { return a.k + (((size_t)b * T + i) * H + h) * DK; };
  auto dv_ = [&](int i) { return a.v + (((size_t)b * T + i) * H + h) * DV; };
  auto dsc = [&](const float *f, int i) { return f[((size_t)b * T + i) * H + h]; };

  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW>(s, S, rb0, lane);
  const int pos = a.ptr.pos_in[b], ck = a.ptr.ckpt_in[b];
  const int count = pos - ck;
  if (count < 0 || count > L) {
    if (h == 0 && threadIdx.x == 0) {
      atomicOr(a.status, REPLAY_STATUS_BAD_POINTERS);
      a.ptr.pos_out[b] = pos;
      a.ptr.ckpt_out[b] = ck;
    }
    return;
  }
  const bool fold = count + T > L;  // implies count >= 1 because T <= L
  const int s0 = fmod_(ck, sh.fL);
  int base = ck, sb = s0;
  float4 X[NCH], Q[NCH];
  float vr[16];
#pragma unroll
  for (int c = 0; c < NCH; ++c) Q[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (fold) {
    load_keys<NCH>(X, count, -1, nullptr, rp, s0, L, lane);
    load_vrows<RBW>(vr, count, -1, nullptr, rp, s0, L, rb0, lane);
    const int j = r16 < count ? r16 : 0;
    const float al = rp.ral[wrap(s0, j, L)], be = rp.rbe[wrap(s0, j, L)];
    gdn_window<NCH, RBW>(s, X, Q, count, al, be, vr, false, true, sm, lane);
    const float gl = sm.g[count - 1];
    gdn_fold_apply<NCH, RBW>(s, count, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
    store_rows_g<NCH, RBW>(s, S, rb0, lane);
    base = pos;
    sb = wrap(s0, count, L);
  }
  const int c = pos - base, nrec = c + T;
  // Keys: committed records from the ring, drafts from the input.
  {
    const int j = r16 < nrec ? r16 : nrec - 1;
    const float *kj = j < c ? rp.rk + (size_t)wrap(sb, j, L) * rp.ks : dk_(j - c);
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const float4 v = ld4(kj + 16 * cc + 4 * q);
      X[cc] = r16 < nrec ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int i = r16 < T ? r16 : T - 1;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const float4 v = ld4(dq_(i) + 16 * cc + 4 * q);
      Q[cc] = r16 < T ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  {
    const int row = rb0 * 16 + (lane < 16 * RBW ? lane : 0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tc = t < nrec ? t : nrec - 1;
      const float v = tc < c ? rp.rv[(size_t)wrap(sb, tc, L) * rp.vs + row] : dv_(tc - c)[row];
      vr[t] = t < nrec ? v : 0.f;
    }
  }
  float al, be;
  {
    const int j = r16 < nrec ? r16 : nrec - 1;
    const float a1 = j < c ? rp.ral[wrap(sb, j, L)] : dsc(a.alpha, j - c);
    const float b1 = j < c ? rp.rbe[wrap(sb, j, L)] : dsc(a.beta, j - c);
    al = r16 < nrec ? a1 : 1.f;
    be = r16 < nrec ? b1 : 0.f;
  }
  // S0 Q^T and K Q^T on the MFMA, into per-wave LDS.
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      acc = mfma_16x16x4(s[k][cc].x, Q[cc].x, acc);
      acc = mfma_16x16x4(s[k][cc].y, Q[cc].y, acc);
      acc = mfma_16x16x4(s[k][cc].z, Q[cc].z, acc);
      acc = mfma_16x16x4(s[k][cc].w, Q[cc].w, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) SQ[16 * k + 4 * q + i][r16] = acc[i];
  }
  {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      acc = mfma_16x16x4(X[cc].x, Q[cc].x, acc);
      acc = mfma_16x16x4(X[cc].y, Q[cc].y, acc);
      acc = mfma_16x16x4(X[cc].z, Q[cc].z, acc);
      acc = mfma_16x16x4(X[cc].w, Q[cc].w, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) KQ[4 * q + i][r16] = acc[i];
  }
  // Pseudo-values of all nrec records.
  gdn_window<NCH, RBW>(s, X, Q, nrec, al, be, vr, false, true, sm, lane);
  if (lane < 16 * RBW) {
    const int row = rb0 * 16 + lane;
    float u[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) u[t] = t < nrec ? sm.U[t][lane] : 0.f;
    for (int i = 0; i < T; ++i) {
      const int last = c + i;
      const float gi = sm.g[last];
      float o = __expf(gi) * SQ[lane][i];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j <= last) o += __expf(gi - sm.g[j]) * KQ[j][i] * u[j];
      a.y[(((size_t)b * T + i) * H + h) * DV + row] = o;
    }
  }
  // Stage the drafts in the ring after every wave is done with folded slots.
  __syncthreads();
  for (int i = 0; i < T; ++i) {
    const int sl = wrap(sb, c + i, L);
    if (lane < 16 * RBW) rp.rv[(size_t)sl * rp.vs + rb0 * 16 + lane] = dv_(i)[rb0 * 16 + lane];
    for (int e = threadIdx.x; e < DK; e += 256) rp.rk[(size_t)sl * rp.ks + e] = dk_(i)[e];
  }
  if (threadIdx.x < T) {
    const int sl = wrap(sb, c + threadIdx.x, L);
    rp.ral[sl] = dsc(a.alpha, threadIdx.x);
    rp.rbe[sl] = dsc(a.beta, threadIdx.x);
  }
  if (h == 0 && threadIdx.x == 0) {
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- baselines: conventional step and snapshot-per-draft verify ----------------
// One token of the stepwise recurrence on the register tile:
//   Sk = S k;  S <- alpha S + (beta v - alpha beta Sk) k^T;  o = S q.
template <int NCH, int RBW>
__device__ __forceinline__ void gdn_update_rows(float4 (&s)[RBW][NCH], const float *qin, const float *kin,
                                                const float *vin, float alpha, float beta, int rb0, int lane,
                                                float *o_rows /* nullptr: no store */) {
  const int q = lane >> 4, r16 = lane & 15;
  float4 kv[NCH], qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    kv[c] = ld4(kin + 16 * c + 4 * q);
    qv[c] = ld4(qin + 16 * c + 4 * q);
  }
  float acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
    float sk = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) sk += dot4(s[k][c], kv[c]);
    sk = sum_quarters(sk);
    const float coef = beta * vin[row] - alpha * beta * sk;
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

template <int NCH, int RBW>
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
  load_rows_g<NCH, RBW>(s, S, rb0, lane);
  gdn_update_rows<NCH, RBW>(s, a.q + bh * DK, a.k + bh * DK, a.v + bh * DV, a.alpha[bh], a.beta[bh], rb0, lane,
                            a.y + bh * DV);
  store_rows_g<NCH, RBW>(s, S, rb0, lane);
}

template <int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_snapshot_verify(GdnSnapArgs a) {
  constexpr int DK = 16 * NCH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Shape &sh = a.s;
  const int T = a.T, H = sh.H, DV = sh.P, rb0 = wave * RBW;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * H;
  const int cur = a.cur[b];
  if (cur < 0 || cur >= a.nslots) return;  // never index outside the slot array
  auto slot_ptr = [&](int sl) { return a.slots + (((size_t)b * a.nslots + sl) * H + h) * (size_t)DV * DK; };
  float4 s[RBW][NCH];
  load_rows_g<NCH, RBW>(s, slot_ptr(cur), rb0, lane);
  for (int i = 0; i < T; ++i) {
    const size_t d = ((size_t)b * T + i) * H + h;
    gdn_update_rows<NCH, RBW>(s, a.q + d * DK, a.k + d * DK, a.v + d * DV, a.alpha[d], a.beta[d], rb0, lane,
                              a.y + d * DV);
    store_rows_g<NCH, RBW>(s, slot_ptr((cur + 1 + i) % a.nslots), rb0, lane);
  }
}

// ---- dispatch -----------------------------------------------------------------
// All GDN kernels use the wave-per-row-block geometry with four waves per head:
// RBW = d_v / 64 row blocks per wave (d_v in {64, 128}).
template <template <int, int> class K, typename Args>
int gdn_dispatch(const Args &a, hipStream_t st) {
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

#define RSSM_WRAP(name, kern)                  \
  template <int NCH, int RBW>                  \
  struct name {                                \
    static constexpr auto fn = kern<NCH, RBW>; \
  };
RSSM_WRAP(GStepK, gdn_replay_step)
RSSM_WRAP(GFlushK, gdn_flush)
RSSM_WRAP(GVerifyK, gdn_replay_verify)
RSSM_WRAP(GConvK, gdn_conv_step)
RSSM_WRAP(GSnapK, gdn_snapshot_verify)
#undef RSSM_WRAP

}  // namespace

int launch_gdn_step(const GdnStepArgs &a, hipStream_t st) { return gdn_dispatch<GStepK>(a, st); }
int launch_gdn_flush(const GdnFlushArgs &a, hipStream_t st) { return gdn_dispatch<GFlushK>(a, st); }
int launch_gdn_verify(const GdnVerifyArgs &a, hipStream_t st) { return gdn_dispatch<GVerifyK>(a, st); }
int launch_gdn_conv(const GdnConvArgs &a, hipStream_t st) { return gdn_dispatch<GConvK>(a, st); }
int launch_gdn_snapshot(const GdnSnapArgs &a, hipStream_t st) { return gdn_dispatch<GSnapK>(a, st); }

}  // namespace rssm
