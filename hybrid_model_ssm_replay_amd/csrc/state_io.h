// Stored copies of a layer's state in registers and in HBM, shared by the
// Mamba-2 and Gated DeltaNet kernels.
//
// One wave holds RBW blocks of 16 state rows (Mamba-2 P, GDN d_v indices) of a
// head in registers: s[k][c] = S[16 (rb0 + k) + (l % 16)][colq(c, l / 16) + 0..3].
// The column map colq is a compile-time choice: interleaved (16 c + 4 q) when
// both copies are float32 (each float32 load instruction then covers 16 rows x
// 64 contiguous bytes), contiguous per lane (4 NCH q + 4 c) when a
// low-precision copy is read (its bytes load as wide contiguous words and every
// 16-element e2m1 scale block lies inside one lane).  Every contraction over the
// state columns pairs s with the same map, so results do not depend on it.
//
// SIO<FMT, ...> moves one wave's rows between registers and a storage format
// (codecs.h): load / write the stored bits, decode them exactly to float32,
// encode float32 with the format's rounding.  The checkpoint carries the
// recurrence and the read copy serves the outputs; the two are one buffer when
// their formats are equal [P1, Interpretation 4; P3, Interpretation 3].
#pragma once

#include "codecs.h"
#include "internal.h"

namespace rssm {
namespace {

// Column maps: which state columns (Mamba-2 N, GDN d_k) lane quarter q holds in chunk c.
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

// load_rows_g through a buffer resource that covers nbytes of the head from
// S: loads past nbytes return zeros without a memory access, so a head that
// reads nothing (nbytes = 0) runs the same code, with the same registers, as
// one that reads its rows (no branch around the loads).
template <int NCH, int RBW, int CM>
__device__ __forceinline__ void load_rows_masked(float4 (&s)[RBW][NCH], const float *S, uint32_t nbytes, int rb0,
                                                 int lane) {
  constexpr int DK = 16 * NCH;
  const int q = lane >> 4, r16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(S), (short)0, (int)nbytes,
                                                                      0x00020000);
#pragma unroll
  for (int k = 0; k < RBW; ++k) {
    const int row = (rb0 + k) * 16 + r16;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      s[k][c] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs, (row * DK + colq<NCH, CM>(c, q)) * 4, 0, 0));
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

// ---- state storage formats ------------------------------------------------------
// Where one head's state lives: element offset `head` of the head tile, the
// data array and, for e2m1, the scale array (one byte per 16 elements).
struct StateBuf {
  void *data;
  uint8_t *scales;
  int8_t *cols;  // two-axis e2m1: column exponents [B][H][d_k]
};

// Counter and key of the stochastic-rounding bits of one fold: element e of
// the head takes word e % 4 of Philox(e / 4, h, b, ckpt_pos) under the seed.
struct SRKey {
  uint32_t k0, k1, h, b, ckpt;
};

// SIO<FMT, ...>: one wave's rows of one head in a storage format.
//   Raw          the stored bits of the wave's rows, in registers;
//   load/write   Raw <-> memory;
//   decode       Raw -> float32 register tile (exact);
//   encode       float32 register tile -> Raw (the format's rounding).
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
  static __device__ __forceinline__ void encode(Raw &r, const float4 (&s)[RBW][NCH], int, int, const SRKey &) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) r.v[k][c] = s[k][c];
  }
  static __device__ __forceinline__ void write(const Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    store_rows_g<NCH, RBW, CM>(r.v, (float *)b.data + head, rb0, lane);
  }
};

template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F16_SR, NCH, RBW, CM> {
  static constexpr int DK = 16 * NCH;
  static constexpr bool kWide = CM == kColContig && NCH % 2 == 0;  // 8 NCH contiguous bytes: 16-byte accesses
  struct Raw {
    uint2 v[RBW][NCH];  // four halves per chunk
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const __half *S = (const __half *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (kWide) {
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
  static __device__ __forceinline__ void encode(Raw &r, const float4 (&s)[RBW][NCH], int rb0, int lane,
                                                const SRKey &key) {
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t e4 = (uint32_t)((row * DK + colq<NCH, CM>(c, q)) >> 2);
        const Philox4 rr = philox4x32_10(e4, key.h, key.b, key.ckpt, key.k0, key.k1);
        const float4 v = s[k][c];
        const uint32_t h0 = __half_as_ushort(__float2half(f16_sr(v.x, rr.x >> 8)));
        const uint32_t h1 = __half_as_ushort(__float2half(f16_sr(v.y, rr.y >> 8)));
        const uint32_t h2 = __half_as_ushort(__float2half(f16_sr(v.z, rr.z >> 8)));
        const uint32_t h3 = __half_as_ushort(__float2half(f16_sr(v.w, rr.w >> 8)));
        r.v[k][c] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      }
    }
  }
  static __device__ __forceinline__ void write(const Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    __half *S = (__half *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (kWide) {
        uint4 *dst = reinterpret_cast<uint4 *>(S + (size_t)row * DK + colq<NCH, CM>(0, q));
#pragma unroll
        for (int p = 0; p < NCH / 2; ++p)
          dst[p] = make_uint4(r.v[k][2 * p].x, r.v[k][2 * p].y, r.v[k][2 * p + 1].x, r.v[k][2 * p + 1].y);
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) *reinterpret_cast<uint2 *>(S + (size_t)row * DK + colq<NCH, CM>(c, q)) = r.v[k][c];
      }
    }
  }
};

template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F8E4M3, NCH, RBW, CM> {
  static constexpr int DK = 16 * NCH;
  static constexpr bool kWide = CM == kColContig && NCH % 4 == 0;  // 4 NCH contiguous bytes: 16-byte accesses
  struct Raw {
    uint32_t v[RBW][NCH];  // four codes per chunk
  };
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const uint8_t *S = (const uint8_t *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (kWide) {
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
  static __device__ __forceinline__ void encode(Raw &r, const float4 (&s)[RBW][NCH], int, int, const SRKey &) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float4 v = s[k][c];
        r.v[k][c] = e4m3_encode4(v.x, v.y, v.z, v.w);
      }
  }
  static __device__ __forceinline__ void write(const Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    uint8_t *S = (uint8_t *)b.data + head;
    const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const int row = (rb0 + k) * 16 + r16;
      if constexpr (kWide) {
        uint4 *dst = reinterpret_cast<uint4 *>(S + (size_t)row * DK + colq<NCH, CM>(0, q));
#pragma unroll
        for (int p = 0; p < NCH / 4; ++p)
          dst[p] = make_uint4(r.v[k][4 * p], r.v[k][4 * p + 1], r.v[k][4 * p + 2], r.v[k][4 * p + 3]);
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) *reinterpret_cast<uint32_t *>(S + (size_t)row * DK + colq<NCH, CM>(c, q)) = r.v[k][c];
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
  static __device__ __forceinline__ size_t row_elem(int rb0, int k, int lane) {
    return (size_t)((rb0 + k) * 16 + (lane & 15)) * DK + colq<NCH, CM>(0, lane >> 4);
  }
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    const uint8_t *C = (const uint8_t *)b.data + head / 2;
    const uint8_t *SC = b.scales + head / 16;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const size_t e = row_elem(rb0, k, lane);
      if constexpr (NCH == 8) {  // 16 contiguous bytes of codes
        const uint4 w = *reinterpret_cast<const uint4 *>(C + e / 2);
        r.codes[k][0] = w.x;
        r.codes[k][1] = w.y;
        r.codes[k][2] = w.z;
        r.codes[k][3] = w.w;
        r.scales[k] = *reinterpret_cast<const uint16_t *>(SC + e / 16);
      } else {
        const uint2 w = *reinterpret_cast<const uint2 *>(C + e / 2);
        r.codes[k][0] = w.x;
        r.codes[k][1] = w.y;
        r.scales[k] = SC[e / 16];
      }
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
  static __device__ __forceinline__ void encode(Raw &r, const float4 (&s)[RBW][NCH], int, int, const SRKey &) {
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      uint32_t scw = 0;
#pragma unroll
      for (int blk = 0; blk < NCH / 4; ++blk) {
        float amax = 0.f;
#pragma unroll
        for (int c = 4 * blk; c < 4 * blk + 4; ++c)
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(s[k][c].x), fabsf(s[k][c].y)), fmaxf(fabsf(s[k][c].z), fabsf(s[k][c].w))));
        const uint32_t scode = e4m3_encode(__fdiv_rn(amax, 6.f));
        const float sc = e4m3_decode(scode);
        const E2m1Thr th = e2m1_thresholds(sc);
        scw |= scode << (8 * blk);
#pragma unroll
        for (int p = 2 * blk; p < 2 * blk + 2; ++p) {
          uint32_t w = 0;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const float4 v = s[k][2 * p + h2];
            w |= (e2m1_code(v.x, th) | (e2m1_code(v.y, th) << 4) | (e2m1_code(v.z, th) << 8) |
                  (e2m1_code(v.w, th) << 12))
                 << (16 * h2);
          }
          r.codes[k][p] = sc > 0.f ? w : 0u;  // a zero scale makes the block zero
        }
      }
      r.scales[k] = scw;
    }
  }
  static __device__ __forceinline__ void write(const Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    uint8_t *C = (uint8_t *)b.data + head / 2;
    uint8_t *SC = b.scales + head / 16;
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
      const size_t e = row_elem(rb0, k, lane);
      if constexpr (NCH == 8) {
        *reinterpret_cast<uint4 *>(C + e / 2) = make_uint4(r.codes[k][0], r.codes[k][1], r.codes[k][2], r.codes[k][3]);
        *reinterpret_cast<uint16_t *>(SC + e / 16) = (uint16_t)r.scales[k];
      } else {
        *reinterpret_cast<uint2 *>(C + e / 2) = make_uint2(r.codes[k][0], r.codes[k][1]);
        SC[e / 16] = (uint8_t)r.scales[k];
      }
    }
  }
};

// Two-axis e2m1 (read copy only): the block format above of x / 2^e[n], with
// one signed exponent byte e[n] per d_k column of the head,
//     e[n] = max(floor(log2 amax_n) - 5, -126)   (amax_n over the head's rows),
// read from the biased exponent field of amax_n.  A lane's 4 NCH columns are
// contiguous, so their exponents are NCH words (word c: chunk c).  prepare()
// finds the column maxima over the four waves (DPP within a wave, LDS across
// waves: it contains a workgroup barrier, so every wave of the workgroup must
// call it) and divides the tile by 2^e in place; encode() is then the block
// encoder; decode() multiplies by 2^e again.  Division and multiplication by
// 2^e are exact (ldexp) unless a quotient is subnormal, which only happens for
// values that quantise to zero.
template <int NCH, int RBW, int CM>
struct SIO<REPLAY_FMT_F4E2M1_CS, NCH, RBW, CM> {
  using Base = SIO<REPLAY_FMT_F4E2M1_B16, NCH, RBW, CM>;
  static_assert(NCH % 4 == 0, "the exponent words load as 16-byte vectors");
  static constexpr int DK = 16 * NCH, DV = 64 * RBW;
  struct Raw {
    typename Base::Raw base;
    uint32_t ex[NCH];  // byte i of word c: exponent of column colq(c, q) + i
  };
  // This lane's exponents: column offset of the head (head / DV = (b H + h) d_k) plus its first column.
  static __device__ __forceinline__ int8_t *col_ptr(const StateBuf &b, size_t head, int lane) {
    return b.cols + head / DV + colq<NCH, CM>(0, lane >> 4);
  }
  static __device__ __forceinline__ int exp_of(uint32_t w, int i) { return (int)(int8_t)((w >> (8 * i)) & 0xFF); }
  static __device__ __forceinline__ void scale(float4 (&s)[RBW][NCH], const uint32_t (&ex)[NCH], int sign) {
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t w = ex[c];
        float4 &v = s[k][c];
        v = make_float4(__builtin_amdgcn_ldexpf(v.x, sign * exp_of(w, 0)), __builtin_amdgcn_ldexpf(v.y, sign * exp_of(w, 1)),
                        __builtin_amdgcn_ldexpf(v.z, sign * exp_of(w, 2)), __builtin_amdgcn_ldexpf(v.w, sign * exp_of(w, 3)));
      }
  }
  static __device__ __forceinline__ void load(Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    Base::load(r.base, b, head, rb0, lane);
    const uint4 *src = reinterpret_cast<const uint4 *>(col_ptr(b, head, lane));
#pragma unroll
    for (int p = 0; p < NCH / 4; ++p) {
      const uint4 w = src[p];
      r.ex[4 * p] = w.x;
      r.ex[4 * p + 1] = w.y;
      r.ex[4 * p + 2] = w.z;
      r.ex[4 * p + 3] = w.w;
    }
  }
  static __device__ __forceinline__ void decode(float4 (&s)[RBW][NCH], const Raw &r) {
    Base::decode(s, r.base);
    scale(s, r.ex, 1);
  }
  static __device__ __forceinline__ void prepare(Raw &r, float4 (&s)[RBW][NCH], int lane, int wave) {
    __shared__ float4 cmax[4][DK / 4];  // per wave: the maxima of its rows, natural column order
    const int q = lane >> 4;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float4 m = make_float4(fabsf(s[0][c].x), fabsf(s[0][c].y), fabsf(s[0][c].z), fabsf(s[0][c].w));
#pragma unroll
      for (int k = 1; k < RBW; ++k)
        m = make_float4(fmaxf(m.x, fabsf(s[k][c].x)), fmaxf(m.y, fabsf(s[k][c].y)), fmaxf(m.z, fabsf(s[k][c].z)),
                        fmaxf(m.w, fabsf(s[k][c].w)));
      m = make_float4(max16(m.x), max16(m.y), max16(m.z), max16(m.w));
      if ((lane & 15) == 0) cmax[wave][(colq<NCH, CM>(c, q)) >> 2] = m;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int c4 = colq<NCH, CM>(c, q) >> 2;
      float4 m = cmax[0][c4];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 t = cmax[w][c4];
        m = make_float4(fmaxf(m.x, t.x), fmaxf(m.y, t.y), fmaxf(m.z, t.z), fmaxf(m.w, t.w));
      }
      // e = max(biased exponent - 132, -126): floor(log2 amax) - 5, and -126 for zero or subnormal maxima.
      auto ex = [](float a) { return (uint32_t)max((int)(__float_as_uint(a) >> 23) - 132, -126) & 0xFFu; };
      r.ex[c] = ex(m.x) | (ex(m.y) << 8) | (ex(m.z) << 16) | (ex(m.w) << 24);
    }
    scale(s, r.ex, -1);
  }
  static __device__ __forceinline__ void encode(Raw &r, const float4 (&s)[RBW][NCH], int rb0, int lane,
                                                const SRKey &key) {
    Base::encode(r.base, s, rb0, lane, key);  // s was divided by 2^e in prepare()
  }
  static __device__ __forceinline__ void write(const Raw &r, const StateBuf &b, size_t head, int rb0, int lane) {
    Base::write(r.base, b, head, rb0, lane);
    if (rb0 == 0 && (lane & 15) == 0) {  // every wave holds the same exponents: wave 0 writes them
      uint4 *dst = reinterpret_cast<uint4 *>(col_ptr(b, head, lane));
#pragma unroll
      for (int p = 0; p < NCH / 4; ++p) dst[p] = make_uint4(r.ex[4 * p], r.ex[4 * p + 1], r.ex[4 * p + 2], r.ex[4 * p + 3]);
    }
  }
};

// State buffers of one launch: the checkpoint (format CF) and the read copy
// (format RF; the same buffer when RF == CF).
struct StateBufs {
  StateBuf ck, rd;
  uint32_t seed_lo, seed_hi;
};

// Encode the tile s into the checkpoint and (if separate) the read copy, and
// leave in s what the read copy now holds, decoded: the S0 of the window that
// starts here.  A two-axis read copy makes this a workgroup-wide step (column
// maxima over all rows): the callers decide per sequence, and a workgroup is
// one (sequence, head), so all four waves arrive together.
template <int CF, int RF, int NCH, int RBW>
__device__ __forceinline__ void store_both(float4 (&s)[RBW][NCH], const StateBufs &sb, size_t head, int rb0,
                                           int lane, uint32_t h, uint32_t b, uint32_t ckpt) {
  constexpr int CM = col_map(CF, RF);
  const SRKey key{sb.seed_lo, sb.seed_hi, h, b, ckpt};
  typename SIO<CF, NCH, RBW, CM>::Raw rc;
  SIO<CF, NCH, RBW, CM>::encode(rc, s, rb0, lane, key);
  SIO<CF, NCH, RBW, CM>::write(rc, sb.ck, head, rb0, lane);
  if constexpr (RF != CF) {
    typename SIO<RF, NCH, RBW, CM>::Raw rr;
    if constexpr (RF == REPLAY_FMT_F4E2M1_CS) SIO<RF, NCH, RBW, CM>::prepare(rr, s, lane, rb0 / RBW);
    SIO<RF, NCH, RBW, CM>::encode(rr, s, rb0, lane, key);
    SIO<RF, NCH, RBW, CM>::write(rr, sb.rd, head, rb0, lane);
    SIO<RF, NCH, RBW, CM>::decode(s, rr);
  } else if constexpr (CF != REPLAY_FMT_F32) {
    SIO<CF, NCH, RBW, CM>::decode(s, rc);
  }
}


// Encode the tile s into the checkpoint and (if separate) the read copy and
// leave s as it is (the float32 fold result).  For layers whose outputs need no
// decoded copy of the new checkpoint (Mamba-2); no two-axis read copy here.
template <int CF, int RF, int NCH, int RBW>
__device__ __forceinline__ void store_copies(const float4 (&s)[RBW][NCH], const StateBufs &sb, size_t head, int rb0,
                                             int lane, uint32_t h, uint32_t b, uint32_t ckpt) {
  static_assert(RF != REPLAY_FMT_F4E2M1_CS, "the two-axis copy needs the workgroup-wide encoder (store_both)");
  constexpr int CM = col_map(CF, RF);
  const SRKey key{sb.seed_lo, sb.seed_hi, h, b, ckpt};
  {
    typename SIO<CF, NCH, RBW, CM>::Raw rc;
    SIO<CF, NCH, RBW, CM>::encode(rc, s, rb0, lane, key);
    SIO<CF, NCH, RBW, CM>::write(rc, sb.ck, head, rb0, lane);
  }
  if constexpr (RF != CF) {
    typename SIO<RF, NCH, RBW, CM>::Raw rr;
    SIO<RF, NCH, RBW, CM>::encode(rr, s, rb0, lane, key);
    SIO<RF, NCH, RBW, CM>::write(rr, sb.rd, head, rb0, lane);
  }
}

// MFMA row index M (0..15) of column chunk c -> state column, for the rank-m
// update S^T += B^T X^T whose output lands in the register layout: output
// register i of lane quarter q is row M = 4 q + i, which holds column
// colq(c, q) + i.
template <int NCH, int CM>
__device__ __forceinline__ int mcol(int c, int M) {
  return colq<NCH, CM>(c, M >> 2) + (M & 3);
}

// An empty register constraint on every word of x: the compiler can no longer
// treat x as the same value on both sides, so code that decodes it in two
// branches is not hoisted above them (which would keep the decoded tile live
// across the branch).
template <typename T>
__device__ __forceinline__ void opaque_words(T &x) {
  static_assert(sizeof(T) % 4 == 0, "whole words");
  uint32_t *w = reinterpret_cast<uint32_t *>(&x);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" : "+v"(w[i]));
}

// Views of one launch's stored copies from the host-side description.
inline StateBufs state_bufs(const FormatBufs &f) {
  StateBufs sb;
  sb.ck = StateBuf{f.ckpt, f.ckpt_scales, nullptr};
  sb.rd = StateBuf{f.read, f.read_scales, f.read_cols};
  sb.seed_lo = (uint32_t)(f.seed & 0xFFFFFFFFu);
  sb.seed_hi = (uint32_t)(f.seed >> 32);
  return sb;
}

}  // namespace
}  // namespace rssm
