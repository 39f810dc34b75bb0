// Device-side constants and bit-layout helpers shared by the libtqattn kernels.
// Layouts are described in include/tqattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <type_traits>

namespace tq {

constexpr int kDim = 128;
constexpr int kTileTokens = 32;
constexpr int kMaxGroup = 16;
constexpr int kFmtF16 = 0;
constexpr int kFmtTurbo3 = 3;
constexpr int kFmtTurbo4 = 4;

__host__ __device__ constexpr int k_record_bytes(int fmt) { return fmt == kFmtTurbo3 ? 48 : 64; }
__host__ __device__ constexpr int v_chunk_bytes(int fmt) { return fmt == kFmtTurbo3 ? 24 : fmt == kFmtF16 ? 128 : 32; }
__host__ __device__ constexpr int v_tile_bytes(int fmt) { return 64 * v_chunk_bytes(fmt); }
__host__ __device__ constexpr int levels(int fmt) { return fmt == kFmtTurbo3 ? 8 : 16; }

// Byte order in memory.  Quantised records and chunks are stored in pieces (turbo4:
// 16 bytes, turbo3: 12 bytes, one sub-block) so that the lanes reading the same piece
// of neighbouring records / chunks read whole contiguous cache lines:
//  * turbo4 K, blocks of 16 tokens: piece p (record bytes 16p..16p+15) of token
//    16b + i at byte 1024 b + 256 p + 16 i;
//  * turbo3 K, blocks of 16 tokens: piece u (record bytes 12u..12u+11) of token
//    16b + i at byte 768 b + 384 (u % 2) + 192 (u / 2) + 12 i, so pieces {0, 2} and
//    {1, 3} each fill 384 contiguous bytes;
//  * V chunk c's piece p at tile byte 1024 p + 16 c (turbo4) or 768 p + 12 c (turbo3);
//  * fp16 K rows (256 bytes) and fp16 V chunks follow each other.
__host__ __device__ inline size_t k_byte_offset(int fmt, size_t t, int byte) {
  if (fmt == kFmtTurbo4) return (t >> 4) * 1024 + size_t(byte >> 4) * 256 + (t & 15) * 16 + (byte & 15);
  if (fmt == kFmtTurbo3) {
    const int u = byte / 12;
    return (t >> 4) * 768 + size_t(384 * (u & 1) + 192 * (u >> 1)) + (t & 15) * 12 + byte % 12;
  }
  return t * 256 + byte;
}
__host__ __device__ inline int v_chunk_byte_offset(int fmt, int chunk, int byte) {
  if (fmt == kFmtTurbo4) return (byte >> 4) * 1024 + chunk * 16 + (byte & 15);
  if (fmt == kFmtTurbo3) return (byte / 12) * 768 + chunk * 12 + byte % 12;
  return chunk * v_chunk_bytes(fmt) + byte;
}

// V tile: token slot r (0..31) <-> (slot group g = 0..3, element-token i = 0..7),
// r = 16*(i/4) + 4*g + (i%4).
__host__ __device__ inline int slot_group(int r) { return (r & 15) >> 2; }
__host__ __device__ inline int slot_elem(int r) { return ((r >> 4) << 2) | (r & 3); }
__host__ __device__ inline int slot_of(int g, int i) { return ((i >> 2) << 4) | (g << 2) | (i & 3); }

// ---- turbo3 sub-block: 32 three-bit codes in words w[0..2] (A, B, C).
__host__ __device__ inline uint32_t sub3_get(const uint32_t* w, int e) {
  const int j = e & 3;
  if (e < 24) return (w[e >> 3] >> (8 * j + ((e >> 2) & 1) * 3)) & 7u;
  const int word = e >= 28 ? 1 : 0;
  const uint32_t lo = (w[word] >> (8 * j + 6)) & 3u;
  const uint32_t hi = (w[2] >> (8 * j + 6 + word)) & 1u;
  return lo | (hi << 2);
}

__host__ __device__ inline void sub3_pack(const uint8_t* c, uint32_t* w) {
  uint32_t a = 0, b = 0, cc = 0;
  for (int j = 0; j < 4; ++j) {
    a |= (uint32_t(c[j]) & 7u) << (8 * j);
    a |= (uint32_t(c[4 + j]) & 7u) << (8 * j + 3);
    a |= (uint32_t(c[24 + j]) & 3u) << (8 * j + 6);
    b |= (uint32_t(c[8 + j]) & 7u) << (8 * j);
    b |= (uint32_t(c[12 + j]) & 7u) << (8 * j + 3);
    b |= (uint32_t(c[28 + j]) & 3u) << (8 * j + 6);
    cc |= (uint32_t(c[16 + j]) & 7u) << (8 * j);
    cc |= (uint32_t(c[20 + j]) & 7u) << (8 * j + 3);
    cc |= ((uint32_t(c[24 + j]) >> 2) & 1u) << (8 * j + 6);
    cc |= ((uint32_t(c[28 + j]) >> 2) & 1u) << (8 * j + 7);
  }
  w[0] = a;
  w[1] = b;
  w[2] = cc;
}

// ---- turbo4 octet word: 8 sign-magnitude nibbles.
__host__ __device__ inline int oct4_bit(int e) { return e < 4 ? 8 * e : 8 * (e - 4) + 4; }
__host__ __device__ inline uint32_t oct4_get_nibble(uint32_t w, int e) { return (w >> oct4_bit(e)) & 15u; }
__host__ __device__ inline uint32_t t4_index_of_nibble(uint32_t nib) {
  return (nib & 8u) ? 7u - (nib & 7u) : 8u + (nib & 7u);
}
__host__ __device__ inline uint32_t t4_nibble_of_index(uint32_t k) { return k >= 8u ? k - 8u : (8u | (7u - k)); }

__host__ __device__ inline uint32_t oct4_pack(const uint8_t* idx) {
  uint32_t w = 0;
  for (int e = 0; e < 8; ++e) w |= t4_nibble_of_index(idx[e]) << oct4_bit(e);
  return w;
}

__device__ inline float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// Value of lane (lane ^ M) within the same aligned 16-lane row, M in {1, 2, 4, 8},
// through DPP moves (VALU data paths, no LDS round trip): quad_perm covers xor 1
// and 2; xor 4 = half-row mirror (i ^ 7) then quad reversal (i ^ 3); xor 8 = the
// row rotated by 8 lanes ((i + 8) mod 16 = i ^ 8).  All 16 lanes of the row must
// be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xf, 0xf, false));
}
template <int M>
__device__ __forceinline__ uint32_t xor_lane16(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "xor distance within a 16-lane row");
  if constexpr (M == 1) return dpp_u32<0xb1>(v);                 // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_u32<0x4e>(v);            // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_u32<0x1b>(dpp_u32<0x141>(v));  // half mirror, quad_perm [3,2,1,0]
  else return dpp_u32<0x128>(v);                                // row_ror:8
}
template <int M>
__device__ __forceinline__ float xor_lane16(float v) {
  return __uint_as_float(xor_lane16<M>(__float_as_uint(v)));
}
template <int M>
__device__ __forceinline__ uint64_t xor_lane16(uint64_t v) {
  return uint64_t(xor_lane16<M>(uint32_t(v))) | (uint64_t(xor_lane16<M>(uint32_t(v >> 32))) << 32);
}
template <int M>
__device__ __forceinline__ double xor_lane16(double v) {
  return __longlong_as_double(int64_t(xor_lane16<M>(uint64_t(__double_as_longlong(v)))));
}

// Exchanges across any lane bit B = 0..5 of the wave, for values spread over all 64
// lanes: bits 0-3 through the DPP moves above, bits 4 and 5 through the gfx950 row
// swaps (permlane16_swap(v, v) hands each lane the values of lanes i & ~16 and
// i | 16; permlane32_swap the same for bit 5).  wave_sum gives both lanes of a pair
// the same sum; wave_butterfly gives the lower lane lo + hi and the upper lo - hi.
// Every lane of the wave must execute them together.
template <int B>
__device__ __forceinline__ void wave_pair_u32(uint32_t v, int lane, uint32_t& lo, uint32_t& hi) {
  static_assert(B >= 0 && B <= 5, "lane bit of a 64-lane wave");
  if constexpr (B == 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  } else if constexpr (B == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    const uint32_t o = xor_lane16<(1 << B)>(v);
    const bool upper = (lane >> B) & 1;
    lo = upper ? o : v;
    hi = upper ? v : o;
  }
}
template <int B>
__device__ __forceinline__ uint64_t wave_sum(uint64_t v, int lane) {
  if constexpr (B < 4) {
    return v + xor_lane16<(1 << B)>(v);
  } else {
    uint32_t l0, h0, l1, h1;
    wave_pair_u32<B>(uint32_t(v), lane, l0, h0);
    wave_pair_u32<B>(uint32_t(v >> 32), lane, l1, h1);
    return (uint64_t(l0) | (uint64_t(l1) << 32)) + (uint64_t(h0) | (uint64_t(h1) << 32));
  }
}
template <int B>
__device__ __forceinline__ double wave_sum(double v, int lane) {
  if constexpr (B < 4) {
    return v + xor_lane16<(1 << B)>(v);
  } else {
    uint32_t l0, h0, l1, h1;
    const uint64_t u = uint64_t(__double_as_longlong(v));
    wave_pair_u32<B>(uint32_t(u), lane, l0, h0);
    wave_pair_u32<B>(uint32_t(u >> 32), lane, l1, h1);
    return __longlong_as_double(int64_t(uint64_t(l0) | (uint64_t(l1) << 32))) +
           __longlong_as_double(int64_t(uint64_t(h0) | (uint64_t(h1) << 32)));
  }
}
template <int B>
__device__ __forceinline__ double wave_butterfly(double v, int lane) {
  const double sgn = ((lane >> B) & 1) ? -1.0 : 1.0;
  if constexpr (B < 4) {
    return fma(v, sgn, xor_lane16<(1 << B)>(v));   // o - v or v + o, one rounding
  } else {
    uint32_t l0, h0, l1, h1;
    const uint64_t u = uint64_t(__double_as_longlong(v));
    wave_pair_u32<B>(uint32_t(u), lane, l0, h0);
    wave_pair_u32<B>(uint32_t(u >> 32), lane, l1, h1);
    return fma(__longlong_as_double(int64_t(uint64_t(h0) | (uint64_t(h1) << 32))), sgn,
               __longlong_as_double(int64_t(uint64_t(l0) | (uint64_t(l1) << 32))));
  }
}
template <int B>
__device__ __forceinline__ float wave_butterfly(float v, int lane) {
  const float sgn = ((lane >> B) & 1) ? -1.f : 1.f;
  if constexpr (B < 4) {
    return __builtin_fmaf(v, sgn, xor_lane16<(1 << B)>(v));
  } else {
    uint32_t lo, hi;
    wave_pair_u32<B>(__float_as_uint(v), lane, lo, hi);
    return __builtin_fmaf(__uint_as_float(hi), sgn, __uint_as_float(lo));
  }
}

// Unnormalised 128-point Walsh-Hadamard transform of one row held by 16 lanes,
// 8 elements per lane (element 8*j + i in lane j = lane16, slot i).  Stages over
// element bits 0..2 are in-lane butterflies; stages over bits 3..6 exchange with
// lane j ^ 1, 2, 4, 8 of the same aligned 16-lane segment (DPP moves), so all 16
// lanes of a segment must execute it together.  Natural (Sylvester) order in and out.  Every
// kernel that rotates uses this one routine, so rotations done inside different
// kernels round identically.
__device__ inline void fwht128_row(float v[8], int lane16) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  auto stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float o = xor_lane16<M>(v[i]);
      v[i] = (lane16 & M) ? (o - v[i]) : (v[i] + o);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
}

// The 8 elements 8*lane16 .. 8*lane16+7 of a row of fp32 or fp16-bit values.
__device__ inline void load_row8(const void* base, bool fp32, size_t off, float v[8]) {
  if (fp32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = half_bits_to_float(uint16_t(w[i] & 0xffffu));
      v[2 * i + 1] = half_bits_to_float(uint16_t(w[i] >> 16));
    }
  }
}

// q into K's codec basis: v = H (s * v) / sqrt(128), in place (16-lane row layout);
// s8 = this lane's 8 signs s[8*lane16 .. 8*lane16+7].
__device__ inline void rotate_row_forward8(float v[8], const float s8[8], int lane16) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= s8[i];
  fwht128_row(v, lane16);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= kInvSqrtD;
}

__device__ inline void rotate_row_forward(float v[8], const float* signs, int lane16) {
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = signs[8 * lane16 + i];
  rotate_row_forward8(v, s8, lane16);
}

// Out of V's codec basis and into fp16: s * H (v) / sqrt(128), nearest-even fp16
// bits packed in pairs (element 8*lane16 + 2i in the low half of w[i]).
// 8 fp32 values rounded to nearest-even fp16, packed in pairs.
__device__ inline void round_row_f16(const float v[8], uint32_t w[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = uint32_t(__half_as_ushort(__float2half_rn(v[2 * i]))) |
           (uint32_t(__half_as_ushort(__float2half_rn(v[2 * i + 1]))) << 16);
}

// s8: the sign flips of this lane's elements 8*lane16 .. 8*lane16+7, already in registers
__device__ inline void rotate_row_inverse_f16_s8(float v[8], const float (&s8)[8], int lane16, uint32_t w[4]) {
  fwht128_row(v, lane16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = v[2 * i] * kInvSqrtD * s8[2 * i];
    const float x1 = v[2 * i + 1] * kInvSqrtD * s8[2 * i + 1];
    w[i] = uint32_t(__half_as_ushort(__float2half_rn(x0))) | (uint32_t(__half_as_ushort(__float2half_rn(x1))) << 16);
  }
}

__device__ inline void rotate_row_inverse_f16(float v[8], const float* signs, int lane16, uint32_t w[4]) {
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = signs[8 * lane16 + i];
  rotate_row_inverse_f16_s8(v, s8, lane16, w);
}

}  // namespace tq
