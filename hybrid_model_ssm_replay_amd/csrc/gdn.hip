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
// indices) of S0 in registers:
//     s[k][c] = S[16 (rb0 + k) + (l % 16)][col(c, q) + 0..3],  q = l / 16.
// The column map col is a compile-time choice (colq below): interleaved
// (16 c + 4 q) when the copies are float32, contiguous per lane (4 NCH q + 4 c)
// when a low-precision copy is read, so that its bytes load wide and every
// 16-column e2m1 scale block lies inside one lane.  Keys and queries use the
// same map, so every contraction over d_k is unchanged.
// Per wave, with X = the window's keys in MFMA operand layout (lane (j, q)
// holds k_j[col(c, q) + 0..3], j = l % 16):
//   * W = S0 X^T (one v_mfma_f32_16x16x4f32 pass: M = row, N = record, K = d_k),
//   * the Gram matrix X X^T from the same operand registers,
//   * S0 q and k_j . q on the VALU (q has its own registers),
//   * W goes through per-wave LDS so that each lane owns one row and runs the
//     m x m forward substitution for it with no cross-lane traffic,
//   * a fold is the transposed MFMA rank-m update S^T += K^T U~^T whose output
//     layout equals the register layout of S0.
#include "codecs.h"
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

// Column maps: which d_k columns lane quarter q holds in chunk c.
//   kColIlv:    16 c + 4 q     (a chunk is 16 contiguous columns across the
//                               quarters: each float32 load instruction covers
//                               16 rows x 64 contiguous bytes);
//   kColContig: 4 NCH q + 4 c  (a lane owns 4 NCH contiguous columns, so that
//                               low-precision copies load as wide contiguous
//                               bytes and e2m1 blocks of 16 lie inside a lane).
constexpr int kColIlv = 0, kColContig = 1;

// Interleaved when both stored copies are float32, contiguous otherwise.
constexpr int col_map(int cf, int rf) {
  return (cf == REPLAY_FMT_F32 && rf == REPLAY_FMT_F32) ? kColIlv : kColContig;
}

// First column of chunk c held by lane quarter q.
template <int NCH, int CM>
__device__ __forceinline__ int colq(int c, int q) {
  return CM == kColContig ? 4 * NCH * q + 4 * c : 16 * c + 4 * q;
}

template <int NCH, int RBW, int CM>
__device__ __forceinline__ void load_rows_g(float4 (&s)[RBW][NCH], const float *S, int rb0, int lane) {
  constexpr int DK = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s[k][c] = ld4(S + (size_t)row * DK + colq<NCH, CM>(c, q));
  }
}

template <int NCH, int RBW, int CM>
__device__ __forceinline__ void store_rows_g(const float4 (&s)[RBW][NCH], float *S, int rb0, int lane) {
  constexpr int DK = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) st4(S + (size_t)row * DK + colq<NCH, CM>(c, q), s[k][c]);
  }
}

// A vector (key or query) in the lane's column order.
template <int NCH, int CM>
__device__ __forceinline__ void load_vec(float4 (&v)[NCH], const float *p, int lane) {
  const int q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NCH; ++c) v[c] = ld4(p + colq<NCH, CM>(c, q));
}

// ---- state storage formats ------------------------------------------------------
// Where one head's state lives: element offset `head` of the head tile, the
// data array and, for e2m1, the scale array (one byte per 16 elements).
struct StateBuf {
  void *data;
  uint8_t *scales;
};

// Counter and key of the stochastic-rounding bits of one fold: element e of
// the head takes word e % 4 of Philox(e / 4, h, b, ckpt_pos) under the seed.
struct SRKey {
  uint32_t k0, k1, h, b, ckpt;
};

template <int FMT, int NCH, int RBW, int CM>
struct SIO;

template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F32, NCH, RBW, CM> {
  struct Raw {
    float4 v[RBW][NCH];
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    load_rows_g<NCH, RBW, CM>(r.v, (const float *)b.data + head, rb0, lane);
  }
  static __device__ __forceinline__ void decode(float4 (&s)[RBW][NCH], const Raw &r) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) s[k][c] = r.v[k][c];
  }
  static __device__ __forceinline__ void store(const float4 (&s)[RBW][NCH], const StateBuf &b, size_t head, int rb0,
                                               int lane, const SRKey &) {
    store_rows_g<NCH, RBW, CM>(s, (float *)b.data + head, rb0, lane);
  }
};

template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F16_SR, NCH, RBW, CM> {
  static constexpr int DK = 16 * NCH;
  struct Raw {
    uint2 v[RBW][NCH];  // four halves per chunk
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const __half *S = (const __half *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (CM == kColContig && NCH % 2 == 0) {  // 8 NCH contiguous bytes: 16-byte loads
        const uint4 *src = reinterpret_cast<const uint4 *>(S + (size_t)row * DK + colq<NCH, CM>(0, q));
#pragma unroll
        for (int p = 0; p < NCH / 2; ++p) {
          const uint4 w = src[p];
          r.v[k][2 * p] = make_uint2(w.x, w.y);
          r.v[k][2 * p + 1] = make_uint2(w.z, w.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          r.v[k][c] = *reinterpret_cast<const uint2 *>(S + (size_t)row * DK + colq<NCH, CM>(c, q));
      }
    }
  }
  static __device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)bits16));
  }
  static __device__ __forceinline__ void decode(float4 (&s)[RBW][NCH], const Raw &r) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint2 w = r.v[k][c];
        s[k][c] = make_float4(h2f(w.x & 0xFFFF), h2f(w.x >> 16), h2f(w.y & 0xFFFF), h2f(w.y >> 16));
      }
  }
  static __device__ __forceinline__ void store(const float4 (&s)[RBW][NCH], const StateBuf &b, size_t head, int rb0,
                                               int lane, const SRKey &key) {
    __half *S = (__half *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t e4 = (uint32_t)((row * DK + colq<NCH, CM>(c, q)) >> 2);
        const Philox4 r = philox4x32_10(e4, key.h, key.b, key.ckpt, key.k0, key.k1);
        const float4 v = s[k][c];
        const uint32_t h0 = __half_as_ushort(__float2half(f16_sr(v.x, r.x >> 8)));
        const uint32_t h1 = __half_as_ushort(__float2half(f16_sr(v.y, r.y >> 8)));
        const uint32_t h2 = __half_as_ushort(__float2half(f16_sr(v.z, r.z >> 8)));
        const uint32_t h3 = __half_as_ushort(__float2half(f16_sr(v.w, r.w >> 8)));
        *reinterpret_cast<uint2 *>(S + (size_t)row * DK + colq<NCH, CM>(c, q)) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      }
    }
  }
};

template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F8E4M3, NCH, RBW, CM> {
  static constexpr int DK = 16 * NCH;
  struct Raw {
    uint32_t v[RBW][NCH];  // four codes per chunk
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const uint8_t *S = (const uint8_t *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (CM == kColContig && NCH % 4 == 0) {  // 4 NCH contiguous bytes: 16-byte loads
        const uint4 *src = reinterpret_cast<const uint4 *>(S + (size_t)row * DK + colq<NCH, CM>(0, q));
#pragma unroll
        for (int p = 0; p < NCH / 4; ++p) {
          const uint4 w = src[p];
          r.v[k][4 * p] = w.x;
          r.v[k][4 * p + 1] = w.y;
          r.v[k][4 * p + 2] = w.z;
          r.v[k][4 * p + 3] = w.w;
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          r.v[k][c] = *reinterpret_cast<const uint32_t *>(S + (size_t)row * DK + colq<NCH, CM>(c, q));
      }
    }
  }
  static __device__ __forceinline__ void decode(float4 (&s)[RBW][NCH], const Raw &r) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(r.v[k][c], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(r.v[k][c], true);
        s[k][c] = make_float4(lo[0], lo[1], hi[0], hi[1]);
      }
  }
  static __device__ __forceinline__ void store(const float4 (&s)[RBW][NCH], const StateBuf &b, size_t head, int rb0,
                                               int lane, const SRKey &) {
    uint8_t *S = (uint8_t *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float4 v = s[k][c];
        const uint32_t w = e4m3_encode(v.x) | (e4m3_encode(v.y) << 8) | (e4m3_encode(v.z) << 16) |
                           (e4m3_encode(v.w) << 24);
        *reinterpret_cast<uint32_t *>(S + (size_t)row * DK + colq<NCH, CM>(c, q)) = w;
      }
    }
  }
};

// e2m1 + e4m3 scale per 16: a lane's 4 NCH columns of a row are NCH / 4 whole
// blocks (NCH = 4 or 8); codes are 2 NCH contiguous bytes, scales NCH / 4.
template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F4E2M1_B16, NCH, RBW, CM> {
  static_assert(NCH == 4 || NCH == 8, "e2m1 blocks must not straddle lanes");
  static_assert(CM == kColContig, "e2m1 needs the contiguous column map");
  static constexpr int DK = 16 * NCH;
  struct Raw {
    uint32_t codes[RBW][NCH / 2];  // 8 codes per word
    uint32_t scales[RBW];          // NCH / 4 scale bytes
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const uint8_t *C = (const uint8_t *)b.data + head / 2;
    const uint8_t *SC = b.scales + head / 16;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      const uint8_t *rowc = C + ((size_t)row * DK + colq<NCH, CM>(0, q)) / 2;
      if constexpr (NCH == 8) {  // 16 contiguous bytes of codes
        const uint4 w = *reinterpret_cast<const uint4 *>(rowc);
        r.codes[k][0] = w.x;
        r.codes[k][1] = w.y;
        r.codes[k][2] = w.z;
        r.codes[k][3] = w.w;
      } else {
        const uint2 w = *reinterpret_cast<const uint2 *>(rowc);
        r.codes[k][0] = w.x;
        r.codes[k][1] = w.y;
      }
      const uint8_t *rows = SC + ((size_t)row * DK + colq<NCH, CM>(0, q)) / 16;
      if constexpr (NCH == 8)
        r.scales[k] = *reinterpret_cast<const uint16_t *>(rows);
      else
        r.scales[k] = *rows;
    }
  }
  static __device__ __forceinline__ void decode(float4 (&s)[RBW][NCH], const Raw &r) {
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
#pragma unroll
      for (int p = 0; p < NCH / 2; ++p) {
        const float sc = e4m3_decode((r.scales[k] >> (8 * ((2 * p) / 4))) & 0xFF);
        const float2 a = e2m1_pair<0>(r.codes[k][p]), bb = e2m1_pair<1>(r.codes[k][p]);
        const float2 c2 = e2m1_pair<2>(r.codes[k][p]), d = e2m1_pair<3>(r.codes[k][p]);
        s[k][2 * p] = make_float4(a.x * sc, a.y * sc, bb.x * sc, bb.y * sc);
        s[k][2 * p + 1] = make_float4(c2.x * sc, c2.y * sc, d.x * sc, d.y * sc);
      }
    }
  }
  static __device__ __forceinline__ void store(const float4 (&s)[RBW][NCH], const StateBuf &b, size_t head, int rb0,
                                               int lane, const SRKey &) {
    uint8_t *C = (uint8_t *)b.data + head / 2;
    uint8_t *SC = b.scales + head / 16;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      uint8_t *rowc = C + ((size_t)row * DK + colq<NCH, CM>(0, q)) / 2;
      uint32_t scw = 0;
#pragma unroll
      for (int blk = 0; blk < NCH / 4; ++blk) {
        float amax = 0.f;
#pragma unroll
        for (int c = 4 * blk; c < 4 * blk + 4; ++c)
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(s[k][c].x), fabsf(s[k][c].y)), fmaxf(fabsf(s[k][c].z), fabsf(s[k][c].w))));
        const uint32_t scode = e4m3_encode(__fdiv_rn(amax, 6.f));
        const float sc = e4m3_decode(scode);
        scw |= scode << (8 * blk);
#pragma unroll
        for (int p = 2 * blk; p < 2 * blk + 2; ++p) {
          uint32_t w = 0;
          if (sc > 0.f) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float4 v = s[k][2 * p + h2];
              w |= (e2m1_code(v.x, sc) | (e2m1_code(v.y, sc) << 4) | (e2m1_code(v.z, sc) << 8) |
                    (e2m1_code(v.w, sc) << 12))
                   << (16 * h2);
            }
          }
          *reinterpret_cast<uint32_t *>(rowc + 4 * p) = w;
        }
      }
      uint8_t *rows = SC + ((size_t)row * DK + colq<NCH, CM>(0, q)) / 16;
      if constexpr (NCH == 8)
        *reinterpret_cast<uint16_t *>(rows) = (uint16_t)scw;
      else
        *rows = (uint8_t)scw;
    }
  }
};

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
// want_u).  The MFMA A operand (M = column of chunk c, K = record) is read from
// the ring (cache-resident).
template <int NCH, int RBW, int CM>
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
      const float v = kr[colq<NCH, CM>(c, r16 >> 2) + (r16 & 3)];  // M = r16 in chunk c
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
template <int NCH, int CM>
__device__ __forceinline__ void load_keys(float4 (&X)[NCH], int cnt, int last, const float *kin, const GdnRingPtrs &rp,
                                          int s0, int L, int lane) {
  const int q = lane >> 4, r16 = lane & 15;
  const int j = r16 < cnt ? r16 : cnt - 1;
  const float *kj = (j == last) ? kin : rp.rk + (size_t)wrap(s0, j, L) * rp.ks;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float4 v = ld4(kj + colq<NCH, CM>(c, q));
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

// State buffers of one launch: the checkpoint (format CF) and the read copy
// (format RF; the same buffer when RF == CF).
struct GdnStateBufs {
  StateBuf ck, rd;
  uint32_t seed_lo, seed_hi;
};

template <int CF, int RF, int NCH, int RBW>
__device__ __forceinline__ void store_both(const float4 (&s)[RBW][NCH], const GdnStateBufs &sb, size_t head, int rb0,
                                           int lane, uint32_t h, uint32_t b, uint32_t ckpt) {
  constexpr int CM = col_map(CF, RF);
  const SRKey key{sb.seed_lo, sb.seed_hi, h, b, ckpt};
  SIO<CF, NCH, RBW, CM>::store(s, sb.ck, head, rb0, lane, key);
  if constexpr (RF != CF) SIO<RF, NCH, RBW, CM>::store(s, sb.rd, head, rb0, lane, key);
}

// ---- replay step ------------------------------------------------------------
template <int CF, int RF, int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_replay_step(GdnStepArgs a, GdnStateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  __shared__ GdnLds<RBW> lds_all[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int r16 = lane & 15;
  GdnLds<RBW> &sm = lds_all[wave];
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  const size_t head = bh * DV * DK;
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  const float *qin = a.q + bh * DK, *kin = a.k + bh * DK, *vin = a.v + bh * DV;

  // 1. The read copy first (a non-fold step reads only it), then what needs no pointer.
  typename SIO<RF, NCH, RBW, CM>::Raw raw;
  SIO<RF, NCH, RBW, CM>::load(raw, sb.rd, head, rb0, lane);
  float4 qv[NCH];
  load_vec<NCH, CM>(qv, qin, lane);
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
  int base = ck, sb0 = s0;
  float4 s[RBW][NCH];
  float4 X[NCH];
  float vr[16];
  if (fold) {
    // Fold the full window from the recurrence checkpoint, store both copies,
    // and restart the window; this step's output comes from the fresh fp32 fold.
    if constexpr (RF == CF) {
      SIO<RF, NCH, RBW, CM>::decode(s, raw);
    } else {
      typename SIO<CF, NCH, RBW, CM>::Raw rc;
      SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
      SIO<CF, NCH, RBW, CM>::decode(s, rc);
    }
    load_keys<NCH, CM>(X, L, -1, kin, rp, s0, L, lane);
    load_vrows<RBW>(vr, L, -1, vin, rp, s0, L, rb0, lane);
    const float al = __shfl(al_row, wrap(s0, r16, L), kWave), be = __shfl(be_row, wrap(s0, r16, L), kWave);
    gdn_window<NCH, RBW>(s, X, qv, L, al, be, vr, false, true, sm, lane);
    const float gl = sm.g[L - 1];
    gdn_fold_apply<NCH, RBW, CM>(s, L, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
    store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
    base = pos;
    sb0 = slot;
  }
  const int m = pos - base + 1;
  load_keys<NCH, CM>(X, m, m - 1, kin, rp, sb0, L, lane);
  load_vrows<RBW>(vr, m, m - 1, vin, rp, sb0, L, rb0, lane);
  if (!fold) SIO<RF, NCH, RBW, CM>::decode(s, raw);  // after the ring loads in program order
  float al, be;
  {
    const int j = r16 < m - 1 ? r16 : 0;
    const float a1 = __shfl(al_row, wrap(sb0, j, L), kWave), b1 = __shfl(be_row, wrap(sb0, j, L), kWave);
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
template <int CF, int RF, int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_flush(GdnFlushArgs a, GdnStateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
  __shared__ GdnLds<RBW> lds_all[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  GdnLds<RBW> &sm = lds_all[wave];
  const Shape &sh = a.s;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int b = fdiv(tile, sh.fH), h = tile - b * sh.H;
  const int DV = sh.P, L = sh.L, rb0 = wave * RBW;
  const size_t bh = (size_t)b * sh.H + h;
  const size_t head = bh * DV * DK;
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
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  float4 s[RBW][NCH];
  {
    typename SIO<CF, NCH, RBW, CM>::Raw rc;
    SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
    SIO<CF, NCH, RBW, CM>::decode(s, rc);
  }
  const int s0 = fmod_(ck, sh.fL);
  float4 X[NCH], qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) qv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  float vr[16];
  load_keys<NCH, CM>(X, count, -1, nullptr, rp, s0, L, lane);
  load_vrows<RBW>(vr, count, -1, nullptr, rp, s0, L, rb0, lane);
  const int j = r16 < count ? r16 : 0;
  const float al = rp.ral[wrap(s0, j, L)], be = rp.rbe[wrap(s0, j, L)];
  gdn_window<NCH, RBW>(s, X, qv, count, al, be, vr, false, true, sm, lane);
  const float gl = sm.g[count - 1];
  gdn_fold_apply<NCH, RBW, CM>(s, count, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
  store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
}

// ---- speculative verify ---------------------------------------------------------
// c committed records then T drafts (c + T <= L after a fold-first).  One
// forward substitution over all c + T records; draft i's output is
//   o_i = e^{g_{c+i}} S0 q_i + sum_{j <= c+i} e^{g_{c+i} - g_j} (k_j . q_i) u_j.
// S0 q_i is a second MFMA pass over the queries, k_j . q_i an MFMA of the key
// and query operand registers.  Without a fold-first, S0 is the read copy.
template <int CF, int RF, int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_replay_verify(GdnVerifyArgs a, GdnStateBufs sb) {
  constexpr int DK = 16 * NCH;
  constexpr int CM = col_map(CF, RF);
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
  const size_t head = bh * DV * DK;
  const GdnRingPtrs rp = gdn_ring_ptrs(a.ring, sh, b, h);
  auto dq_ = [&](int i) { return a.q + (((size_t)b * T + i) * H + h) * DK; };
  auto dk_ = [&](int i) { return a.k + (((size_t)b * T + i) * H + h) * DK; };
  auto dv_ = [&](int i) { return a.v + (((size_t)b * T + i) * H + h) * DV; };
  auto dsc = [&](const float *f, int i) { return f[((size_t)b * T + i) * H + h]; };

  typename SIO<RF, NCH, RBW, CM>::Raw raw;
  SIO<RF, NCH, RBW, CM>::load(raw, sb.rd, head, rb0, lane);
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
  int base = ck, sb0 = s0;
  float4 s[RBW][NCH];
  float4 X[NCH], Q[NCH];
  float vr[16];
#pragma unroll
  for (int c = 0; c < NCH; ++c) Q[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (fold) {
    if constexpr (RF == CF) {
      SIO<RF, NCH, RBW, CM>::decode(s, raw);
    } else {
      typename SIO<CF, NCH, RBW, CM>::Raw rc;
      SIO<CF, NCH, RBW, CM>::load(rc, sb.ck, head, rb0, lane);
      SIO<CF, NCH, RBW, CM>::decode(s, rc);
    }
    load_keys<NCH, CM>(X, count, -1, nullptr, rp, s0, L, lane);
    load_vrows<RBW>(vr, count, -1, nullptr, rp, s0, L, rb0, lane);
    const int j = r16 < count ? r16 : 0;
    const float al = rp.ral[wrap(s0, j, L)], be = rp.rbe[wrap(s0, j, L)];
    gdn_window<NCH, RBW>(s, X, Q, count, al, be, vr, false, true, sm, lane);
    const float gl = sm.g[count - 1];
    gdn_fold_apply<NCH, RBW, CM>(s, count, s0, rp.rk, rp.ks, L, __expf(gl), sm, lane);
    store_both<CF, RF, NCH, RBW>(s, sb, head, rb0, lane, (uint32_t)h, (uint32_t)b, (uint32_t)pos);
    base = pos;
    sb0 = wrap(s0, count, L);
  }
  const int c = pos - base, nrec = c + T;
  // Keys: committed records from the ring, drafts from the input.
  {
    const int j = r16 < nrec ? r16 : nrec - 1;
    const float *kj = j < c ? rp.rk + (size_t)wrap(sb0, j, L) * rp.ks : dk_(j - c);
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const float4 v = ld4(kj + colq<NCH, CM>(cc, q));
      X[cc] = r16 < nrec ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int i = r16 < T ? r16 : T - 1;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const float4 v = ld4(dq_(i) + colq<NCH, CM>(cc, q));
      Q[cc] = r16 < T ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  {
    const int row = rb0 * 16 + (lane < 16 * RBW ? lane : 0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tc = t < nrec ? t : nrec - 1;
      const float v = tc < c ? rp.rv[(size_t)wrap(sb0, tc, L) * rp.vs + row] : dv_(tc - c)[row];
      vr[t] = t < nrec ? v : 0.f;
    }
  }
  float al, be;
  {
    const int j = r16 < nrec ? r16 : nrec - 1;
    const float a1 = j < c ? rp.ral[wrap(sb0, j, L)] : dsc(a.alpha, j - c);
    const float b1 = j < c ? rp.rbe[wrap(sb0, j, L)] : dsc(a.beta, j - c);
    al = r16 < nrec ? a1 : 1.f;
    be = r16 < nrec ? b1 : 0.f;
  }
  if (!fold) SIO<RF, NCH, RBW, CM>::decode(s, raw);
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
    const int sl = wrap(sb0, c + i, L);
    if (lane < 16 * RBW) rp.rv[(size_t)sl * rp.vs + rb0 * 16 + lane] = dv_(i)[rb0 * 16 + lane];
    for (int e = threadIdx.x; e < DK; e += 256) rp.rk[(size_t)sl * rp.ks + e] = dk_(i)[e];
  }
  if (threadIdx.x < T) {
    const int sl = wrap(sb0, c + threadIdx.x, L);
    rp.ral[sl] = dsc(a.alpha, threadIdx.x);
    rp.rbe[sl] = dsc(a.beta, threadIdx.x);
  }
  if (h == 0 && threadIdx.x == 0) {
    a.ptr.pos_out[b] = pos;
    a.ptr.ckpt_out[b] = base;
  }
}

// ---- state encode: a float32 state into both stored copies -------------------------
// The stochastic-rounding counter uses each sequence's current ckpt_pos.
template <int CF, int RF, int NCH, int RBW>
__global__ __launch_bounds__(256) void gdn_encode_state(GdnEncodeArgs a, GdnStateBufs sb) {
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
  const uint32_t ckpt = (uint32_t)a.ckpt_pos[b];
  const SRKey key{sb.seed_lo, sb.seed_hi, (uint32_t)h, (uint32_t)b, ckpt};
  if (a.write_ckpt) SIO<CF, NCH, RBW, CM>::store(s, sb.ck, head, rb0, lane, key);
  if constexpr (RF != CF) SIO<RF, NCH, RBW, CM>::store(s, sb.rd, head, rb0, lane, key);
}

// ---- baselines: conventional step and snapshot-per-draft verify ----------------
// One token of the stepwise recurrence on the register tile:
//   Sk = S k;  S <- alpha S + (beta v - alpha beta Sk) k^T;  o = S q.
template <int NCH, int RBW>
__device__ __forceinline__ void gdn_update_rows(float4 (&s)[RBW][NCH], const float *qin, const float *kin,
                                                const float *vin, float alpha, float beta, int rb0, int lane,
                                                float *o_rows /* nullptr: no store */) {
  constexpr int CM = kColIlv;
  const int q = lane >> 4, r16 = lane & 15;
  float4 kv[NCH], qv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    kv[c] = ld4(kin + colq<NCH, CM>(c, q));
    qv[c] = ld4(qin + colq<NCH, CM>(c, q));
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
  load_rows_g<NCH, RBW, kColIlv>(s, S, rb0, lane);
  gdn_update_rows<NCH, RBW>(s, a.q + bh * DK, a.k + bh * DK, a.v + bh * DV, a.alpha[bh], a.beta[bh], rb0, lane,
                            a.y + bh * DV);
  store_rows_g<NCH, RBW, kColIlv>(s, S, rb0, lane);
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
  load_rows_g<NCH, RBW, kColIlv>(s, slot_ptr(cur), rb0, lane);
  for (int i = 0; i < T; ++i) {
    const size_t d = ((size_t)b * T + i) * H + h;
    gdn_update_rows<NCH, RBW>(s, a.q + d * DK, a.k + d * DK, a.v + d * DV, a.alpha[d], a.beta[d], rb0, lane,
                              a.y + d * DV);
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
  X(REPLAY_FMT_F4E2M1_B16, REPLAY_FMT_F4E2M1_B16)                                                   \
  X(REPLAY_FMT_F16_SR, REPLAY_FMT_F16_SR)                                                           \
  X(REPLAY_FMT_F8E4M3, REPLAY_FMT_F8E4M3)

template <template <int, int, int, int> class K, typename Args>
int gdn_dispatch(const Args &a, const GdnStateBufs &sb, int cf, int rf, hipStream_t st) {
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
#define RSSM_Q(CF_, RF_) RSSM_CASE(CF_, RF_, 8, 1) RSSM_CASE(CF_, RF_, 8, 2)
  RSSM_FMT_PAIRS(RSSM_Q)
#undef RSSM_Q
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

#define RSSM_WRAP4(name, kern)                           \
  template <int CF, int RF, int NCH, int RBW>            \
  struct name {                                          \
    static constexpr auto fn = kern<CF, RF, NCH, RBW>;   \
  };
RSSM_WRAP4(GStepK, gdn_replay_step)
RSSM_WRAP4(GFlushK, gdn_flush)
RSSM_WRAP4(GVerifyK, gdn_replay_verify)
RSSM_WRAP4(GEncodeK, gdn_encode_state)
#undef RSSM_WRAP4
#define RSSM_WRAP(name, kern)                  \
  template <int NCH, int RBW>                  \
  struct name {                                \
    static constexpr auto fn = kern<NCH, RBW>; \
  };
RSSM_WRAP(GConvK, gdn_conv_step)
RSSM_WRAP(GSnapK, gdn_snapshot_verify)
#undef RSSM_WRAP

GdnStateBufs state_bufs(const GdnFormatBufs &f) {
  GdnStateBufs sb;
  sb.ck = StateBuf{f.ckpt, f.ckpt_scales};
  sb.rd = StateBuf{f.read, f.read_scales};
  sb.seed_lo = (uint32_t)(f.seed & 0xFFFFFFFFu);
  sb.seed_hi = (uint32_t)(f.seed >> 32);
  return sb;
}

}  // namespace

int launch_gdn_step(const GdnStepArgs &a, const GdnFormatBufs &f, hipStream_t st) {
  return gdn_dispatch<GStepK>(a, state_bufs(f), f.ckpt_fmt, f.read_fmt, st);
}
int launch_gdn_flush(const GdnFlushArgs &a, const GdnFormatBufs &f, hipStream_t st) {
  return gdn_dispatch<GFlushK>(a, state_bufs(f), f.ckpt_fmt, f.read_fmt, st);
}
int launch_gdn_verify(const GdnVerifyArgs &a, const GdnFormatBufs &f, hipStream_t st) {
  return gdn_dispatch<GVerifyK>(a, state_bufs(f), f.ckpt_fmt, f.read_fmt, st);
}
int launch_gdn_encode(const GdnEncodeArgs &a, const GdnFormatBufs &f, hipStream_t st) {
  return gdn_dispatch<GEncodeK>(a, state_bufs(f), f.ckpt_fmt, f.read_fmt, st);
}
int launch_gdn_conv(const GdnConvArgs &a, hipStream_t st) { return gdn_dispatch_f32<GConvK>(a, st); }
int launch_gdn_snapshot(const GdnSnapArgs &a, hipStream_t st) { return gdn_dispatch_f32<GSnapK>(a, st); }

}  // namespace rssm
