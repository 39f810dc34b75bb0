// MFMA split-K decode attention for gfx950 (the default decode kernel, variant 0).
//
// One wave per work item (split s of KV head h of sequence b); on latency-bound
// calls four waves per split, each taking a quarter of its tokens.  Both
// contractions run on v_mfma_f32_16x16x32_f16 with fp32 accumulation; the VALU
// only dequantises codes into MFMA operands and runs the online softmax.
//
// Column packing.  The G query heads of a KV head are padded to Gp = 4, 8 or
// 16 and the 16 MFMA columns carry NS = 16/Gp "sets" of them: column n is
// head n % Gp of set n / Gp, and set sigma works on its own 32-token V tile.
// An iteration therefore consumes NS tiles (32*NS tokens) and no softmax lane
// is spent on padding when G divides 16.
//
//   scores   S^T[token][col] = sum_k K[token][k] * Qhat[k][col]     (A = K, B = q)
//            The B operand of lane group g is zero unless g belongs to the
//            column's set, so each set only sees its own tokens; lane (g, n)
//            ends with the 8 scores of tile slots r = 16*rb + 4*g + j of its
//            column's tile -- the slots of V-tile chunk group g, element 4rb+j.
//   softmax  log2-domain online max/sum (the scale * log2(e) factor is folded
//            into q); the max is shared by the 4 lanes of a column.
//   values   O^T[dim][col] += sum_t V^T[dim][t] * Pn[t][col]    (A = V, B = P*n_V)
//            with one MFMA group per set, whose B operand is zero outside the set.
//
// Dequant (no LDS, no barrier; interleaved with the MFMA issue, which
// turboquant_plus "SMEM Pre-Dequant Experiment", "Why It Failed", found to be
// the point): fp16 codebook values come from byte tables held in registers via
// v_perm_b32 -- one lookup per 4 codes for the low bytes, one for the high
// bytes, two more to interleave them into fp16 pairs.  turbo3 looks up the full
// signed 8-entry table; turbo4 looks up 8 magnitudes and ORs the sign bit.
// The per-token norms multiply the fp32 scores (K) and the fp16 probabilities
// (V), never the operands.
#include <math.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_encode.h"
#include "tq_launch.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Build-time tuning knobs (the defaults are the measured best).
#ifndef TQ_MFMA_NS_SMALL_GROUP
#define TQ_MFMA_NS_SMALL_GROUP 4   // token sets per MFMA for group sizes <= 4 (4 or 2)
#endif
#ifndef TQ_MFMA_LAZY_RESCALE
#define TQ_MFMA_LAZY_RESCALE 1
#endif

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline half8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

// Byte tables of 8 fp16 values: lo/hi byte of entries 0..3 (x0) and 4..7 (x1).
struct ByteTable {
  uint32_t lo0, lo1, hi0, hi1;
};

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) { return __builtin_amdgcn_perm(hi, lo, sel); }

// The byte tables of 8 fp16 entries held as four words (entry 2i in the low half of
// w[i]): the low bytes of entries 0-3 are bytes 0, 2 of w[0], w[1], their high bytes
// bytes 1, 3; entries 4-7 likewise from w[2], w[3].  One byte gather each.
__device__ inline ByteTable make_table(const uint32_t (&w)[4]) {
  ByteTable t;
  t.lo0 = perm(w[1], w[0], 0x06040200u);
  t.hi0 = perm(w[1], w[0], 0x07050301u);
  t.lo1 = perm(w[3], w[2], 0x06040200u);
  t.hi1 = perm(w[3], w[2], 0x07050301u);
  return t;
}

// four table lookups (selector bytes 0..7) -> two dwords of fp16 pairs
__device__ inline void lookup4(const ByteTable& t, uint32_t sel, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = perm(t.lo1, t.lo0, sel);
  const uint32_t hi = perm(t.hi1, t.hi0, sel);
  d0 = perm(hi, lo, 0x05010400u);
  d1 = perm(hi, lo, 0x07030602u);
}

// turbo3: codes 8c..8c+7 of a sub-block (words A, B, C) as 8 fp16 codebook values.
template <int C>
__device__ inline half8 dq_turbo3(uint32_t A, uint32_t B, uint32_t Cw, const ByteTable& t) {
  uint32_t s0, s1;
  if (C == 0) {
    s0 = A & 0x07070707u;
    s1 = (A >> 3) & 0x07070707u;
  } else if (C == 1) {
    s0 = B & 0x07070707u;
    s1 = (B >> 3) & 0x07070707u;
  } else if (C == 2) {
    s0 = Cw & 0x07070707u;
    s1 = (Cw >> 3) & 0x07070707u;
  } else {
    s0 = ((A >> 6) & 0x03030303u) | ((Cw >> 4) & 0x04040404u);
    s1 = ((B >> 6) & 0x03030303u) | ((Cw >> 5) & 0x04040404u);
  }
  uint32_t d0, d1, d2, d3;
  lookup4(t, s0, d0, d1);
  lookup4(t, s1, d2, d3);
  return pack8(d0, d1, d2, d3);
}

// turbo4: the 8 sign-magnitude nibbles of an octet word as 8 fp16 codebook values.
__device__ inline half8 dq_turbo4(uint32_t w, const ByteTable& mag) {
  const uint32_t mA = w & 0x07070707u, mB = (w >> 4) & 0x07070707u;
  const uint32_t loA = perm(mag.lo1, mag.lo0, mA);
  const uint32_t hiA = perm(mag.hi1, mag.hi0, mA) | ((w << 4) & 0x80808080u);
  const uint32_t loB = perm(mag.lo1, mag.lo0, mB);
  const uint32_t hiB = perm(mag.hi1, mag.hi0, mB) | (w & 0x80808080u);
  return pack8(perm(hiA, loA, 0x05010400u), perm(hiA, loA, 0x07030602u), perm(hiB, loB, 0x05010400u),
               perm(hiB, loB, 0x07030602u));
}

// Norm scaling in one instruction instead of a convert and a multiply: an fma with a
// +0 addend, which the compiler emits as a mixed-precision v_fma_mix* reading the
// fp16 half of w directly (the product is rounded once; a -0 product becomes +0).
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
// x times the fp16 half HI of w
template <int HI>
__device__ inline float mul_half(float x, uint32_t w) {
  const half2v h = __builtin_bit_cast(half2v, w);
  return __builtin_fmaf(x, float(HI ? h.y : h.x), 0.f);
}
// the fp16 pair (lo * half 0 of w, hi * half 1 of w)
__device__ inline uint32_t mul_halves_pack(float lo, float hi, uint32_t w) {
  const half2v h = __builtin_bit_cast(half2v, w);
  half2v r;
  r.x = _Float16(__builtin_fmaf(lo, float(h.x), 0.f));
  r.y = _Float16(__builtin_fmaf(hi, float(h.y), 0.f));
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Reductions over the 4 lanes i, i^16, i^32, i^48 of an MFMA column, with the
// gfx950 row-swap permutes (no LDS round trip).  permlane16_swap(x, x) hands each
// lane the value of lane i & ~16 and of lane i | 16; permlane32_swap does the
// same for bit 5.  Every lane of the wave must be active.
__device__ inline float xmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float xsum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int N>
__device__ inline void load_words(uint32_t (&w)[N], const uint8_t* p) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// Quantised K/V words are read through a buffer resource over the (sequence, KV head)
// row -- its base in SGPRs, a 32-bit byte offset per lane (capacity is capped so a
// row's bytes stay under 2^31) -- which keeps 64-bit address arithmetic out of the
// loop.  Reads past the resource's size would return zeros; the kernel's never do.
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
constexpr int kNonTemporal = 2;   // buffer-load cache-policy bits: nt (each byte is read once)

// NP 16-byte pieces at off, off + stride, ... (turbo4 K records and V chunks): every
// piece load of the wave reads whole contiguous cache lines.
template <int NP, int N>
__device__ inline void load_pieces16(uint32_t (&w)[N], __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t stride) {
  static_assert(N == 4 * NP, "four words per piece");
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + i * stride, 0, kNonTemporal);
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// turbo3: the NP 12-byte pieces (sub-blocks) u0, u0 + 1, ... of this lane's token in
// a 16-token K block at off (piece u at off + 384 (u % 2) + 192 (u / 2)), and the two
// pieces of this lane's V chunk at off and off + 768.  Each load of the wave reads
// whole cache lines.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
template <int NP, int N>
__device__ inline void load_k3_pieces(uint32_t (&w)[N], __amdgpu_buffer_rsrc_t r, uint32_t off, int u0) {
  static_assert(N == 3 * NP, "three words per piece");
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int u = u0 + i;
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 384 * (u & 1) + 192 * (u >> 1), 0, kNonTemporal);
    w[3 * i] = v.x;
    w[3 * i + 1] = v.y;
    w[3 * i + 2] = v.z;
  }
}
template <int N>
__device__ inline void load_v3_pieces(uint32_t (&w)[N], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(N == 6, "two pieces of three words");
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 768 * i, 0, kNonTemporal);
    w[3 * i] = v.x;
    w[3 * i + 1] = v.y;
    w[3 * i + 2] = v.z;
  }
}
// four fp16 norms at byte offset off
__device__ inline uint2 load_norms4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

template <int N>
__device__ inline void zero_words(uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = 0;
}

// Decode step, two extra work groups of (sequence b, KV head h), at grid columns
// 0 (K) and 1 (V): one wave encodes the new token's K or V row (a quantised row over
// all 64 lanes, two elements each; an fp16 row on lanes 0-15) at slot L straight
// into the cache, then writes that side of the token's own
// partial for the G query heads -- K: score z_g = scale * q_g . k_hat (k_hat =
// n_K * c_K[idx] in K's basis, or the fp16 row) as m, and l = 1; V: o = v_hat =
// n_V * c_V[idx] in V's basis.  The regular splits cover the L earlier tokens and
// never read slot L, so all of them run side by side; the merge kernel folds this
// partial in like any other split.
template <int KFMT, int VFMT>
__device__ __forceinline__ void append_v_partial(const DecodeArgs& a, size_t row, int L, int lane) {
  const size_t p0 = partial_index(a, row, a.plan.max_splits, 0);
  if constexpr (VFMT == kFmtF16) {  // stored as it comes; the partial is the row itself
    const int j = lane & 15;
    if (lane >= 16) return;  // one 16-lane group
    float x[8];
    const uint4 v = *reinterpret_cast<const uint4*>(a.app.v_new + row * kDim + 8 * j);
    store_f16_v_row(a.app, row, L, v, j);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = half_bits_to_float(uint16_t(w[e >> 1] >> (16 * (e & 1))));
    for (int g = 0; g < a.group; ++g) {
      float4* o = reinterpret_cast<float4*>(a.part_o + (p0 + g) * kDim + 8 * j);
      o[0] = make_float4(x[0], x[1], x[2], x[3]);
      o[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  } else {  // the whole wave, two dims per lane
    WaveVInputs<VFMT> in;
    load_wave_v_inputs<VFMT>(a.app, row, L, a.app.v_new + row * kDim, lane, in);
    uint32_t code[2];
    const float nv = half_bits_to_float(append_v_row_wave<VFMT>(a.app, row, L, in, lane, code));
    const float x0 = nv * codebook_at<VFMT>(in.row.tab, code[0]), x1 = nv * codebook_at<VFMT>(in.row.tab, code[1]);
    const int e0 = wave_row_elem(lane);
    for (int g = 0; g < a.group; ++g) {
      float* o = a.part_o + (p0 + g) * kDim + e0;
      o[0] = x0;
      o[4] = x1;
    }
  }
}

// K side, F16 K: lanes 0-15 copy the row (requested before the q staging, so its
// memory round trip overlaps it) and score it against the unrotated q rows in qs.
__device__ __forceinline__ void append_k_partial_f16(const DecodeArgs& a, const float (*qs)[kDim], size_t row, int L,
                                                     int lane, const uint4& kraw) {
  const int j = lane & 15;
  if (lane >= 16) return;  // one 16-lane group
  float x[8];
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.app.k_data) + (row * a.cap + L) * kDim + 8 * j) = kraw;
  const uint32_t w[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = half_bits_to_float(uint16_t(w[e >> 1] >> (16 * (e & 1))));
  // this lane's share of every head's dot product, then one 16-lane reduction for all
  const int G = a.group;
  float d[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    float t = 0.f;
    if (g < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) t += qs[g][8 * j + e] * x[e];
    }
    d[g] = t;
  }
  auto sum_stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) d[g] += xor_lane16<M>(d[g]);
  };
  sum_stage(std::integral_constant<int, 1>{});
  sum_stage(std::integral_constant<int, 2>{});
  sum_stage(std::integral_constant<int, 4>{});
  sum_stage(std::integral_constant<int, 8>{});
  const size_t p0 = partial_index(a, row, a.plan.max_splits, 0);
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < G && j == g) {  // lane g stores head g
      a.part_ml[(p0 + g) * 2] = a.scale * kLog2e * d[g];  // log2 units, like the splits' m
      a.part_ml[(p0 + g) * 2 + 1] = 1.f;
    }
  }
}

// The G scores z_g = scale * q_g . k of the token's own partial, from this lane's two
// K elements x0, x1 (e0, e0 + 4 of the whole-wave layout): the sums over the wave run
// by halving -- the row swap over lane bit 5 sums head k with itself across the bit
// in lanes without it and head k + NV/2 in lanes with it, the swap over bit 4 halves
// again, and DPP sums over lane bits 0-3 finish NV/4 heads per 16-lane row: row r
// ends with heads NV/4 * r .. NV/4 * r + NV/4 - 1 (NV = G rounded up to 4, 8 or 16).
template <int NV>
__device__ __forceinline__ void store_head_scores_wave(const DecodeArgs& a, const float (*qs)[kDim], size_t row,
                                                       int lane, int e0, float x0, float x1) {
  const int G = a.group;
  float d[NV];
#pragma unroll
  for (int g = 0; g < NV; ++g) d[g] = g < G ? qs[g][e0] * x0 + qs[g][e0 + 4] * x1 : 0.f;
  float e[NV / 2];
#pragma unroll
  for (int k = 0; k < NV / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[k]), __float_as_uint(d[k + NV / 2]), false, false);
    e[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float f[NV / 4];
#pragma unroll
  for (int k = 0; k < NV / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(e[k]), __float_as_uint(e[k + NV / 4]), false, false);
    f[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  auto sum_stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
#pragma unroll
    for (int k = 0; k < NV / 4; ++k) f[k] += xor_lane16<M>(f[k]);
  };
  sum_stage(std::integral_constant<int, 1>{});
  sum_stage(std::integral_constant<int, 2>{});
  sum_stage(std::integral_constant<int, 4>{});
  sum_stage(std::integral_constant<int, 8>{});
  const int k = lane & 15, g = (NV / 4) * (lane >> 4) + k;
  if (k < NV / 4 && g < G) {
    float z = f[0];
#pragma unroll
    for (int i = 1; i < NV / 4; ++i) z = k == i ? f[i] : z;
    const size_t pidx = partial_index(a, row, a.plan.max_splits, g);
    a.part_ml[pidx * 2] = a.scale * kLog2e * z;  // log2 units, like the splits' m
    a.part_ml[pidx * 2 + 1] = 1.f;
  }
}

// K side, quantised K, over the whole wave: encode and store the row and rebuild
// k = s_K * H(n_K * c_K[idx]) / sqrt(128), two elements per lane (x0, x1: elements e0,
// e0 + 4); q stays unrotated, since q_rot . k_hat = q . k (the rotation is orthonormal).
template <int KFMT>
__device__ __forceinline__ void append_k_rebuild_wave(const DecodeArgs& a, size_t row, int L, int lane,
                                                      const WaveRowInputs<KFMT>& kin, float& x0, float& x1) {
  uint32_t code[2];
  const float nk = half_bits_to_float(append_k_row_wave<KFMT>(a.app, row, L, kin, lane, code));
  x0 = nk * codebook_at<KFMT>(kin.tab, code[0]);
  x1 = nk * codebook_at<KFMT>(kin.tab, code[1]);
  {
    const float u = x0, v = x1;   // element bit 2, in-lane
    x0 = u + v;
    x1 = u - v;
  }
  auto stage = [&](auto b_c) {
    constexpr int B = decltype(b_c)::value;
    x0 = wave_butterfly<B>(x0, lane);
    x1 = wave_butterfly<B>(x1, lane);
  };
  stage(std::integral_constant<int, 0>{});
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 3>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 5>{});
  x0 = x0 * kInvSqrtD * kin.sg[0];
  x1 = x1 * kInvSqrtD * kin.sg[1];
}

__device__ __forceinline__ void append_k_scores_wave(const DecodeArgs& a, const float (*qs)[kDim], size_t row,
                                                     int lane, float x0, float x1) {
  const int e0 = wave_row_elem(lane);
  if (a.group <= 4) store_head_scores_wave<4>(a, qs, row, lane, e0, x0, x1);
  else if (a.group <= 8) store_head_scores_wave<8>(a, qs, row, lane, e0, x0, x1);
  else store_head_scores_wave<16>(a, qs, row, lane, e0, x0, x1);
}

// The G query rows of KV head row `row` into LDS qs, in two phases so the rows'
// memory round trip overlaps other requests: q_request issues every load (rows
// r = 4k + lane/16, k < 4 covers G <= 16; rows past G re-read row G-1 and are
// never stored; no branch around a load, so the compiler never has to drain the
// queue early), q_pin marks the loaded words as used where it is called (so the
// compiler cannot sink the loads into the conditional blocks that use them, behind
// later requests), q_finish converts, rotates (the same 16-lane Walsh-Hadamard
// routine the stand-alone rotation uses, so both routes give identical bits) and
// stores rows 0..G-1.  q is either the caller's unrotated rows (fp16 or fp32) or fp32 rows
// already in K's basis (q_rotate = 0).  All 64 lanes; the caller synchronises.
struct QRaw {
  uint4 lo[4], hi[4];
  float4 s0, s1;  // this lane's K sign flips (elements 8j..8j+7)
};

template <bool SIGNS>
__device__ __forceinline__ void q_request(const DecodeArgs& a, size_t row, int lane, QRaw& q) {
  const int G = a.group, j = lane & 15, r0 = lane >> 4;
  const bool f32 = a.q_fp32 != 0;
  const size_t esz = f32 ? 4 : 2;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint8_t* rowp = static_cast<const uint8_t*>(a.q_in) + (row * G + min(4 * k + r0, G - 1)) * kDim * esz;
    const uint8_t* p = rowp + 8 * j * esz;  // elements 8j..8j+7: 32 bytes (fp32) or 16 (fp16)
    q.lo[k] = *reinterpret_cast<const uint4*>(p);
    q.hi[k] = *reinterpret_cast<const uint4*>(p + (f32 ? 16 : 0));
  }
  if constexpr (SIGNS) {  // K's sign flips (a quantised K format): q rotates into its basis
    q.s0 = reinterpret_cast<const float4*>(a.k_signs + 8 * j)[0];
    q.s1 = reinterpret_cast<const float4*>(a.k_signs + 8 * j)[1];
  } else {
    q.s0 = q.s1 = make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

__device__ __forceinline__ void pin4(uint4& v) {
  uint32_t x = v.x, y = v.y, z = v.z, w = v.w;
  asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
  v = make_uint4(x, y, z, w);
}
__device__ __forceinline__ void pin4(float4& v) {
  float x = v.x, y = v.y, z = v.z, w = v.w;
  asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
  v = make_float4(x, y, z, w);
}
__device__ __forceinline__ void q_pin(QRaw& q) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pin4(q.lo[k]);
    pin4(q.hi[k]);
  }
  pin4(q.s0);
  pin4(q.s1);
}

__device__ __forceinline__ void q_finish(const DecodeArgs& a, float (*qs)[kDim], int lane, const QRaw& q,
                                         bool rotate) {
  const int G = a.group, j = lane & 15, r0 = lane >> 4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (4 * k + r0 < G) {  // whole 16-lane segments
      float v[8];
      const uint32_t w[8] = {q.lo[k].x, q.lo[k].y, q.lo[k].z, q.lo[k].w, q.hi[k].x, q.hi[k].y, q.hi[k].z, q.hi[k].w};
      if (a.q_fp32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = half_bits_to_float(uint16_t(w[i >> 1] >> (16 * (i & 1))));
      }
      if (rotate) {
        const float s8[8] = {q.s0.x, q.s0.y, q.s0.z, q.s0.w, q.s1.x, q.s1.y, q.s1.z, q.s1.w};
        rotate_row_forward8(v, s8, j);
      }
      float4* d = reinterpret_cast<float4*>(&qs[4 * k + r0][8 * j]);
      d[0] = make_float4(v[0], v[1], v[2], v[3]);
      d[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// Four waves sharing a split stage its q rows two at a time: wave w takes rows
// 2w + lane / 32 (and 8 more for G > 8), each over 32 lanes of four elements
// (4 (lane % 32) .. + 3).  The rotation runs fwht128_row's butterflies in its order
// -- element bits 0-1 in-lane, bits 2-5 across lanes xor 1, 2, 4, 8, bit 6 across the
// row swap -- each the same single add or subtract, so q comes out with the same bits
// as from the 16-lane routine, on half its chain.  Rows past G re-read row G - 1 and
// are rotated but never stored (no lane of the wave is left out of an exchange).
struct QRawW {
  uint4 w[2];    // fp32 q: four floats; fp16 q: four halves in .x, .y
  float4 s;      // this lane's K sign flips (elements 4 (lane % 32) .. + 3)
};

template <bool SIGNS>
__device__ __forceinline__ void q_request_w(const DecodeArgs& a, size_t row, int lane, int wave, QRawW& q) {
  const int G = a.group, j = lane & 31;
  const bool f32 = a.q_fp32 != 0;
  const size_t esz = f32 ? 4 : 2;
#pragma unroll
  for (int k = 0; k < 2; ++k) {   // 16 bytes (fp32) or 8 (fp16, read twice): no branch around a load
    const size_t r = row * G + min(8 * k + 2 * wave + (lane >> 5), G - 1);
    const uint8_t* p = static_cast<const uint8_t*>(a.q_in) + (r * kDim + 4 * j) * esz;
    const uint2 lo = *reinterpret_cast<const uint2*>(p);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + (f32 ? 8 : 0));
    q.w[k] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  q.s = SIGNS ? reinterpret_cast<const float4*>(a.k_signs)[j] : make_float4(1.f, 1.f, 1.f, 1.f);
}

__device__ __forceinline__ void q_pin_w(QRawW& q) {
  pin4(q.w[0]);
  pin4(q.w[1]);
  pin4(q.s);
}

__device__ __forceinline__ void q_finish_w(const DecodeArgs& a, float (*qs)[kDim], int lane, int wave, const QRawW& q,
                                           bool rotate) {
  const int G = a.group, j = lane & 31;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (8 * k >= G) break;   // (uniform)
    float v[4];
    if (a.q_fp32) {
      v[0] = __uint_as_float(q.w[k].x);
      v[1] = __uint_as_float(q.w[k].y);
      v[2] = __uint_as_float(q.w[k].z);
      v[3] = __uint_as_float(q.w[k].w);
    } else {
      v[0] = half_bits_to_float(uint16_t(q.w[k].x));
      v[1] = half_bits_to_float(uint16_t(q.w[k].x >> 16));
      v[2] = half_bits_to_float(uint16_t(q.w[k].y));
      v[3] = half_bits_to_float(uint16_t(q.w[k].y >> 16));
    }
    if (rotate) {
      v[0] *= q.s.x;
      v[1] *= q.s.y;
      v[2] *= q.s.z;
      v[3] *= q.s.w;
#pragma unroll
      for (int h = 1; h < 4; h <<= 1) {   // element bits 0, 1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!(i & h)) {
            const float x = v[i], y = v[i + h];
            v[i] = x + y;
            v[i + h] = x - y;
          }
        }
      }
      auto stage = [&](auto m_c) {        // element bits 2..5: lanes xor 1, 2, 4, 8
        constexpr int M = decltype(m_c)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o = xor_lane16<M>(v[i]);
          v[i] = (lane & M) ? (o - v[i]) : (v[i] + o);
        }
      };
      stage(std::integral_constant<int, 1>{});
      stage(std::integral_constant<int, 2>{});
      stage(std::integral_constant<int, 4>{});
      stage(std::integral_constant<int, 8>{});
#pragma unroll
      for (int i = 0; i < 4; ++i) {         // element bit 6: lanes xor 16 (row swap)
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i]), false, false);
        const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
        v[i] = (lane & 16) ? (lo - hi) : (lo + hi);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] *= kInvSqrtD;
    }
    const int r = 8 * k + 2 * wave + (lane >> 5);
    if (r < G) reinterpret_cast<float4*>(&qs[r][4 * j])[0] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Decode step, K side as a whole: request the row and thresholds, encode, store and
// rebuild the row, then score it against the unrotated q rows in qs after the work
// group's one barrier.  STAGE_Q: this wave also stages q (requested first, so its
// round trip overlaps the row's); otherwise another wave of the work group does
// (append_stage_q), off this wave's chain.
template <int KFMT, bool STAGE_Q>
__device__ __forceinline__ void append_k_work(const DecodeArgs& a, float (*qs)[kDim], size_t row, int L, int lane) {
  QRaw q;
  if constexpr (STAGE_Q) q_request<false>(a, row, lane, q);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (KFMT == kFmtF16) {
    uint4 kraw = make_uint4(0, 0, 0, 0);
    if (lane < 16) kraw = *reinterpret_cast<const uint4*>(a.app.k_new + row * kDim + 8 * lane);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STAGE_Q) {
      q_pin(q);
      q_finish(a, qs, lane, q, false);
    }
    __syncthreads();
    append_k_partial_f16(a, qs, row, L, lane, kraw);
  } else {
    WaveRowInputs<KFMT> kin;
    load_wave_row_inputs<KFMT>(a.app.k_new + row * kDim, a.app.k_signs, a.app.k_cb, lane, kin);
    __builtin_amdgcn_sched_barrier(0);
    float x0, x1;
    append_k_rebuild_wave<KFMT>(a, row, L, lane, kin, x0, x1);
    if constexpr (STAGE_Q) {
      q_pin(q);
      q_finish(a, qs, lane, q, false);
    }
    __syncthreads();
    append_k_scores_wave(a, qs, row, lane, x0, x1);
  }
}

// The q staging of append_k_work<KFMT, false>, on another wave of its work group.
__device__ __forceinline__ void append_stage_q(const DecodeArgs& a, float (*qs)[kDim], size_t row, int lane) {
  QRaw q;
  q_request<false>(a, row, lane, q);
  q_pin(q);
  q_finish(a, qs, lane, q, false);
  __syncthreads();
}


// SPARSE: the sparse-V and sparse-K skips are compiled in (their branches cost the
// exact route a few percent of scheduling freedom, so that route goes without them).
// TS: waves per split.  With TS = 4 (latency-bound calls, where most SIMDs would have
// no wave) the split's tokens are shared: each wave streams a quarter of them in
// whole iterations with its own softmax state, the four share the staging of q, and
// they merge their states in LDS at the end, each wave storing a quarter of the
// split's partial -- one partial per split, as with one wave.
template <int KFMT, int VFMT, int NS, bool SPARSE, int TS = 1>
__global__ __launch_bounds__(64 * TS) void decode_mfma_kernel(DecodeArgs a, SeqLens lens) {
  constexpr int P = 4 / NS;                  // lane groups per set in the score MFMA
  constexpr int Gp = 16 / NS;                // columns (padded heads) per set
  constexpr int TOK = 32 * NS;               // tokens per iteration
  constexpr int REC = KFMT == kFmtF16 ? 256 : k_record_bytes(KFMT);
  constexpr int KW = REC / 4 / P;            // K words per lane per token
  constexpr int NKK = 4 * NS;                // score MFMAs per 16-token row block
  constexpr int VW = v_chunk_bytes(VFMT) / 4;  // V words per lane per tile
  constexpr int NACC = 8;                    // value MFMA blocks
  static_assert(TS == 1 || TS == 4, "one wave per split, or four sharing its tokens");

  // Work group -> (row, column): column c < col0 appends the new token (K, V) and
  // attends to it alone, the others are the splits.  When the decode step's grid has
  // more work groups than the chip has compute units (appends_last), it is taken in
  // dispatch order as every row's splits, then every row's two append work groups, so
  // the work groups that must share a unit are the append ones (one busy wave each),
  // not splits.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (a.appends_last) {
    const int ms = int(gridDim.x) - 2, rows = int(gridDim.y * gridDim.z);
    const int lin = int(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    int r, c;
    if (lin < rows * ms) {
      r = lin / ms;
      c = 2 + lin % ms;
    } else {
      r = (lin - rows * ms) >> 1;
      c = (lin - rows * ms) & 1;
    }
    bx = c;
    by = r % int(gridDim.y);
    bz = r / int(gridDim.y);
  }
  const int s = bx - a.col0;
  const int h = by, b = a.b0 + bz;
  const int G = a.group;
  const int L = min(lens.len[bz], a.cap);  // decode step: the length before the append
  const int chunk = a.plan.chunk;
  const int nsplit = min((L + chunk - 1) / chunk, a.plan.max_splits);
  const bool append_wg = s < 0;
  if (s >= nsplit && !(a.split_append && s < 2)) return;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wv = int(threadIdx.x >> 6);
  // This wave's tokens [t0, t1): the split's, or with TS waves per split its TS-th
  // share in whole iterations (a wave left without tokens gets t0 = t1 = the split's end).
  int t0 = s * chunk;
  int t1 = (s == nsplit - 1) ? L : t0 + chunk;
  if constexpr (TS > 1) {
    const int per = ((t1 - t0 + TOK - 1) / TOK + TS - 1) / TS * TOK;
    const int end = t1;
    t0 = min(t0 + wv * per, end);
    t1 = min(t0 + per, end);
  }

  const int sig = g / P, part = g % P;       // score-MFMA set and part of this lane
  const int sn = n / Gp, hn = n % Gp;        // this lane's column: set and head
  const size_t row = size_t(b) * a.hkv + h;
  // Chunk of q_len query positions (column hn is query position hn % q_len of its
  // head): the sequence's last q_len tokens are causal among themselves, so column
  // hn sees tokens < L - (q_len - 1 - hn % q_len) (in whichever splits they fall);
  // every column sees the tokens before t_all.
  const int t_all = min(t1, L - (a.q_len - 1));
  const int t_col = min(t1, L - (a.q_len - 1 - hn % a.q_len));
  // The row's K records and V tiles: fp16 K/V by pointer (this lane's contiguous share);
  // quantised K/V and norms through buffer resources over the row, with this lane's
  // offsets (K: 32-dim pieces kp0 .. kp0 + KPC - 1 of token n of each 16-token block;
  // V: pieces 0 and 1 of chunk `lane` of each tile)
  const uint8_t* krow = a.k_data + row * size_t(a.cap) * REC;
  const uint8_t* vrow = a.v_data + row * size_t(a.cap / kTileTokens) * v_tile_bytes(VFMT);
  const uint8_t* kbase = krow + part * (REC / P);
  const uint8_t* vbase = vrow + lane * (VW * 4);
  const __amdgpu_buffer_rsrc_t krs = row_rsrc(krow, uint32_t(a.cap) * REC);
  const __amdgpu_buffer_rsrc_t vrs = row_rsrc(vrow, uint32_t(a.cap / kTileTokens) * v_tile_bytes(VFMT));
  const __amdgpu_buffer_rsrc_t knrs = row_rsrc(KFMT == kFmtF16 ? nullptr : a.k_norms + row * size_t(a.cap), uint32_t(a.cap) * 2);
  const __amdgpu_buffer_rsrc_t vnrs = row_rsrc(VFMT == kFmtF16 ? nullptr : a.v_norms + row * size_t(a.cap), uint32_t(a.cap) * 2);
  constexpr int KPC = 4 / P;                 // 32-dim K pieces per lane
  const int kp0 = part * KPC;                // this lane's first K piece
  const uint32_t k_lane = KFMT == kFmtTurbo4 ? n * 16 + kp0 * 256 : n * 12;
  const uint32_t v_lane = VFMT == kFmtTurbo4 ? lane * 16 : lane * 12;
  __shared__ float qs[kMaxGroup][kDim];
  if (append_wg) {
    // The append is one long dependent chain (binary64 butterflies, exact norm,
    // thresholds) sharing its SIMD with streaming decode waves: let it issue first.
    // Wave 0 encodes; on the K side of a four-wave work group wave 1 stages q
    // meanwhile and the others only meet the one barrier.
    if (s == -1) {                         // the V side needs no q
      if (wv == 0) {
        __builtin_amdgcn_s_setprio(3);
        append_v_partial<KFMT, VFMT>(a, row, L, lane);
      }
      return;
    }
    if constexpr (TS == 1) {
      __builtin_amdgcn_s_setprio(3);
      append_k_work<KFMT, true>(a, qs, row, L, lane);
    } else if (wv == 0) {
      __builtin_amdgcn_s_setprio(3);
      append_k_work<KFMT, false>(a, qs, row, L, lane);
    } else if (wv == 1) {
      __builtin_amdgcn_s_setprio(3);
      append_stage_q(a, qs, row, lane);
    } else {
      __syncthreads();
    }
    return;
  }
  if (TS == 1 && a.split_append && s < 2) {
    // Bandwidth-bound step: two extra work groups would not fit in the one round of
    // splits, so the first two splits of the row append the token before their own
    // tokens (the kernel's other waves keep streaming meanwhile).
    __builtin_amdgcn_s_setprio(3);
    if (s == 0) append_k_work<KFMT, true>(a, qs, row, L, lane);
    if (s == 1 || a.plan.max_splits == 1) append_v_partial<KFMT, VFMT>(a, row, L, lane);
    __builtin_amdgcn_s_setprio(0);
    if (s >= nsplit) return;
    __syncthreads();  // the K side's reads of qs come before the rows staged below
  }

  // Register double-buffering by rotation: the K words of iteration i+1 are
  // requested as soon as iteration i's K has been turned into MFMA operands, and
  // the V words and norms of i+1 as soon as i's values are accumulated, so every
  // load has about half an iteration of this wave's own math to hide behind.
  uint32_t kw[2][KW];
  uint32_t vw[NS][VW];
  uint2 nk[2], nv[2];
  // Tiles past the split's last visible token are read from the last visible tile
  // instead (always in bounds); their scores are masked and their probabilities are 0.
  const int last_tile = (t1 - 1) >> 5;
  auto load_k = [&](int base) {
    const int tk = min((base >> 5) + sig, last_tile) << 5;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if constexpr (KFMT == kFmtTurbo4) load_pieces16<KW / 4>(kw[rb], krs, k_lane + uint32_t((tk >> 4) + rb) * 1024, 256);
      else if constexpr (KFMT == kFmtTurbo3)
        load_k3_pieces<KW / 3>(kw[rb], krs, k_lane + uint32_t((tk >> 4) + rb) * 768, kp0);
      else load_words(kw[rb], kbase + size_t(tk + 16 * rb + n) * REC);
    }
    if (KFMT != kFmtF16) {
      const int tn = min((base >> 5) + sn, last_tile) << 5;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) nk[rb] = load_norms4(knrs, uint32_t(tn + 16 * rb + 4 * g) * 2);
    }
  };
  auto load_v = [&](int base) {
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      const int tile = min((base >> 5) + sg, last_tile);
      const uint32_t voff = v_lane + uint32_t(tile) * v_tile_bytes(VFMT);
      if constexpr (VFMT == kFmtTurbo4) load_pieces16<2>(vw[sg], vrs, voff, 1024);
      else if constexpr (VFMT == kFmtTurbo3) load_v3_pieces(vw[sg], vrs, voff);
      else load_words(vw[sg], vbase + size_t(tile) * v_tile_bytes(VFMT));
    }
    const int tn = min((base >> 5) + sn, last_tile) << 5;
    if (VFMT != kFmtF16) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) nv[rb] = load_norms4(vnrs, uint32_t(tn + 16 * rb + 4 * g) * 2);
    }
  };
  // q rows first, then the first iteration's words: waiting for q (the oldest
  // requests) leaves the K/V words in flight while q is rotated and staged.
  QRaw qraw;
  QRawW qrw;
  if constexpr (TS > 1) q_request_w<KFMT != kFmtF16>(a, row, lane, wv, qrw);
  else q_request<KFMT != kFmtF16>(a, row, lane, qraw);
  // the 8 fp16 codebook entries each side's byte table needs (turbo4: the 8
  // magnitudes, entries 8..15); none for an fp16 side
  uint4 cbraw[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if constexpr (KFMT != kFmtF16) cbraw[0] = *reinterpret_cast<const uint4*>(a.k_cb + (KFMT == kFmtTurbo4 ? 8 : 0));
  if constexpr (VFMT != kFmtF16) cbraw[1] = *reinterpret_cast<const uint4*>(a.v_cb + (VFMT == kFmtTurbo4 ? 8 : 0));
  __builtin_amdgcn_sched_barrier(0);  // keep every q request ahead of the K/V requests
  load_k(t0);
  load_v(t0);
  __builtin_amdgcn_sched_barrier(0);  // ... and every K/V request ahead of the wait for q
  if constexpr (TS > 1) q_pin_w(qrw);
  else q_pin(qraw);
  pin4(cbraw[0]);
  pin4(cbraw[1]);

  // codebook byte tables from the words requested with q
  ByteTable ktab, vtab;
  {
    const uint32_t kc[4] = {cbraw[0].x, cbraw[0].y, cbraw[0].z, cbraw[0].w};
    const uint32_t vc[4] = {cbraw[1].x, cbraw[1].y, cbraw[1].z, cbraw[1].w};
    if (KFMT != kFmtF16) ktab = make_table(kc);
    vtab = make_table(vc);
  }

  if constexpr (TS > 1) q_finish_w(a, qs, lane, wv, qrw, a.q_rotate != 0);
  else q_finish(a, qs, lane, qraw, a.q_rotate != 0);
  __syncthreads();

  // Sparse K: kbound * n is an upper bound on this lane's column's score (log2
  // units) against any token of stored K norm n, whatever its codes -- by
  // Cauchy-Schwarz, |q| * n * sqrt(128) * max|c| (the rotation keeps |q|), widened by
  // 2^-8 for the fp16 rounding of q and the fp32 sums of the score MFMAs.
  float kbound = 0.f;
  if constexpr (SPARSE && KFMT != kFmtF16) {
    const float* qrow = &qs[min(hn, G - 1)][32 * g];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ss += qrow[i] * qrow[i];
    ss = xsum4(ss);
    const uint32_t kc[4] = {cbraw[0].x, cbraw[0].y, cbraw[0].z, cbraw[0].w};
    float cmax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) cmax = fmaxf(cmax, fabsf(half_bits_to_float(uint16_t(kc[i >> 1] >> (16 * (i & 1))))));
    kbound = a.scale * kLog2e * sqrtf(ss) * sqrtf(float(kDim)) * cmax * (1.f + 0x1p-8f);
  }

  // q in this lane's score-MFMA B slots: q[hn][32 kp0 + 8kk + t] * scale*log2(e),
  // zero unless the lane's k-slots belong to its column's set.
  // Kept in VGPRs: reading these operands from LDS inside the loop measured slower.
  half8 qb[NKK];
  {
    const bool use = hn < G && sig == sn;
    const float* qrow = &qs[min(hn, G - 1)][32 * kp0];
    const float f = use ? a.scale * kLog2e : 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const float4 x0 = reinterpret_cast<const float4*>(qrow + 8 * kk)[0];
      const float4 x1 = reinterpret_cast<const float4*>(qrow + 8 * kk)[1];
      qb[kk] = half8{_Float16(x0.x * f), _Float16(x0.y * f), _Float16(x0.z * f), _Float16(x0.w * f),
                     _Float16(x1.x * f), _Float16(x1.y * f), _Float16(x1.z * f), _Float16(x1.w * f)};
    }
  }
  floatx4 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Scores of the TOK tokens from `base` (log2 units, K norms applied, not yet
  // masked) into S; the next iteration's K words and norms are requested as soon
  // as this one's are turned into MFMA operands and the norms applied (the norms
  // are read straight from their fp16 words, whose registers the request reuses).
  auto score_phase = [&](int base, floatx4 (&S)[2]) {
    // ---- scores (dequant of each operand right before its MFMA)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      S[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        half8 A;
        if (KFMT == kFmtF16) {
          A = pack8(kw[rb][4 * kk], kw[rb][4 * kk + 1], kw[rb][4 * kk + 2], kw[rb][4 * kk + 3]);
        } else if (KFMT == kFmtTurbo4) {
          A = dq_turbo4(kw[rb][kk], ktab);
        } else {
          const int sb = 3 * (kk >> 2);
          const uint32_t wa = kw[rb][sb], wb = kw[rb][sb + 1], wc = kw[rb][sb + 2];
          switch (kk & 3) {
            case 0: A = dq_turbo3<0>(wa, wb, wc, ktab); break;
            case 1: A = dq_turbo3<1>(wa, wb, wc, ktab); break;
            case 2: A = dq_turbo3<2>(wa, wb, wc, ktab); break;
            default: A = dq_turbo3<3>(wa, wb, wc, ktab); break;
          }
        }
        const half8 qk = qb[kk];
        S[rb] = mfma(A, qk, S[rb]);
      }
    }
    if constexpr (KFMT != kFmtF16) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        S[rb][0] = mul_half<0>(S[rb][0], nk[rb].x);
        S[rb][1] = mul_half<1>(S[rb][1], nk[rb].x);
        S[rb][2] = mul_half<0>(S[rb][2], nk[rb].y);
        S[rb][3] = mul_half<1>(S[rb][3], nk[rb].y);
      }
    }
    load_k(base + TOK);     // next iteration's K words and K norms
  };

  // Softmax and values of the TOK tokens from `base` whose scores are in S.  TAIL:
  // the iteration reaches past t1 and the scores of slots >= t1 are masked (only
  // the last one can).
  auto value_phase = [&](int base, const floatx4 (&S)[2], auto tail_c) {
    constexpr bool TAIL = decltype(tail_c)::value;
    const int tn = ((base >> 5) + sn) << 5;      // first token of this lane's column tile
    float z[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = S[rb][j];
        if (TAIL && tn + 16 * rb + 4 * g + j >= t_col) v = -INFINITY;
        z[4 * rb + j] = v;
      }
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = xmax4(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // rescale only when a running max grew, and not from -inf: while a column's max is
    // -inf its l and o are still exactly 0 (every weight so far was 2^-inf = 0)
    if (!TQ_MFMA_LAZY_RESCALE || __any(m_new > m_run && m_run > -INFINITY)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[i] *= alpha;
    }
    m_run = m_new;
    // p = 2^(z - m); a masked slot has z = -inf and p = +0 exactly, and so does
    // p * n_V (norms are finite), so no select is needed.
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(z[i] - m_use);
    float psum = pr[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) psum += pr[i];
    half8 pb;
    if constexpr (VFMT == kFmtF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = _Float16(pr[i]);
    } else {
      const uint32_t pw[4] = {mul_halves_pack(pr[0], pr[1], nv[0].x), mul_halves_pack(pr[2], pr[3], nv[0].y),
                              mul_halves_pack(pr[4], pr[5], nv[1].x), mul_halves_pack(pr[6], pr[7], nv[1].y)};
      pb = pack8(pw[0], pw[1], pw[2], pw[3]);
    }
    l_run += psum;

    // ---- values: one MFMA group per set; B is zero outside the set.  Sparse V: a
    // set whose real heads all have every weight of its tile below the threshold
    // (relative to the running max) skips its tile (wave-uniform branch).
    const uint64_t keep = SPARSE ? __ballot(hn < G && mt - m_use >= a.v_skip_log2) : ~0ull;
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      constexpr uint64_t kRow = (1ull << Gp) - 1;
      const uint64_t set_lanes = (kRow << (sg * Gp)) * 0x0001000100010001ull;  // columns of set sg, all 4 rows
      if (SPARSE && (keep & set_lanes) == 0) continue;
      const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
      const half8 bsg = (sn == sg) ? pb : zero8;
#pragma unroll
      for (int nb = 0; nb < NACC; ++nb) {
        half8 A;
        if constexpr (VFMT == kFmtF16) {
          A = pack8(vw[sg][4 * nb], vw[sg][4 * nb + 1], vw[sg][4 * nb + 2], vw[sg][4 * nb + 3]);
        } else if constexpr (VFMT == kFmtTurbo4) {
          A = dq_turbo4(vw[sg][nb], vtab);
        } else {
          const int sb = 3 * (nb >> 2);
          const uint32_t wa = vw[sg][sb], wb = vw[sg][sb + 1], wc = vw[sg][sb + 2];
          switch (nb & 3) {
            case 0: A = dq_turbo3<0>(wa, wb, wc, vtab); break;
            case 1: A = dq_turbo3<1>(wa, wb, wc, vtab); break;
            case 2: A = dq_turbo3<2>(wa, wb, wc, vtab); break;
            default: A = dq_turbo3<3>(wa, wb, wc, vtab); break;
          }
        }
        acc[nb] = mfma(A, bsg, acc[nb]);
      }
    }
    load_v(base + TOK);     // next iteration's V words and V norms
  };

  // Sparse K (compiled in with sparse V): an iteration is skipped whole -- no K
  // dequant, no scores, no softmax update, no values -- when for every real column
  // the norm-only upper bound of its tile's scores, kbound * (largest K norm of the
  // tile), is below the column's running max + log2 tau_K, so every skipped token's
  // weight is below tau_K relative to a maximum already seen.  The iteration's words
  // were requested anyway; the next ones are requested as usual.
  auto k_skip = [&]() -> bool {
    if (!SPARSE || !(a.k_skip_log2 > -INFINITY)) return false;
    // norms are non-negative fp16, which order like their bit patterns: the largest
    // of the lane's 8 with packed 16-bit integer maxima, then of the column's 4 lanes
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 m2 = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, nk[0].x), __builtin_bit_cast(u16x2, nk[0].y)),
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, nk[1].x), __builtin_bit_cast(u16x2, nk[1].y)));
    const float nmax = xmax4(half_bits_to_float(m2.x > m2.y ? m2.x : m2.y));   // the column's 32-token tile
    return !__any(hn < G && kbound * nmax >= m_run + a.k_skip_log2);
  };

  int base = t0;
  floatx4 S[2];
  for (; base + TOK <= t_all; base += TOK) {
    if (k_skip()) {
      load_k(base + TOK);
      load_v(base + TOK);
      continue;
    }
    score_phase(base, S);
    value_phase(base, S, std::false_type{});
  }
  for (; base < t1; base += TOK) {  // at most two: t1 - t_all < 16 <= TOK
    if (k_skip()) {
      load_k(base + TOK);
      load_v(base + TOK);
      continue;
    }
    score_phase(base, S);
    value_phase(base, S, std::true_type{});
  }

  // ---- finish: sum l over the column's 4 lanes, merge the NS sets of each head
  float l_tot = xsum4(l_run);
  float m_fin = m_run;
  auto merge_sets = [&](auto dist) {  // merge with the set `dist` columns away (DPP, within the row)
    constexpr int STP = decltype(dist)::value;
    const float m_o = xor_lane16<STP>(m_fin);
    const float l_o = xor_lane16<STP>(l_tot);
    const float M = fmaxf(m_fin, m_o);
    const float fs = m_fin == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_fin - M);
    const float fo = m_o == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_o - M);
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o = xor_lane16<STP>(acc[i][j]);
        acc[i][j] = acc[i][j] * fs + o * fo;
      }
    }
    l_tot = l_tot * fs + l_o * fo;
    m_fin = M;
  };
  if constexpr (Gp <= 4) merge_sets(std::integral_constant<int, 4>{});
  if constexpr (Gp <= 8) merge_sets(std::integral_constant<int, 8>{});
  if constexpr (TS > 1) {
    // The split's waves meet in LDS: every wave leaves (m, l) and its o there, then
    // wave w merges and stores the quarter of each column's o in its j = w value
    // blocks (dims 8(4g + w) + nb), weighing every wave's state by 2^(m_v - M), M the
    // largest m (an empty state weighs 0).
    static_assert(TS == 4 && NACC == 8, "four waves, one value-block quarter each");
    __shared__ float2 stml[TS][64];
    __shared__ float4 sto[TS][4][2][64];
    stml[wv][lane] = make_float2(m_fin, l_tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sto[wv][j][0][lane] = make_float4(acc[0][j], acc[1][j], acc[2][j], acc[3][j]);
      sto[wv][j][1][lane] = make_float4(acc[4][j], acc[5][j], acc[6][j], acc[7][j]);
    }
    __syncthreads();
    float2 ml[TS];
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < TS; ++v) {
      ml[v] = stml[v][lane];
      M = fmaxf(M, ml[v].x);
    }
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < TS; ++v) {
      const float f = ml[v].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[v].x - M);
      const float4 lo = sto[v][wv][0][lane], hi = sto[v][wv][1][lane];
      l += ml[v].y * f;
      o[0] += lo.x * f;
      o[1] += lo.y * f;
      o[2] += lo.z * f;
      o[3] += lo.w * f;
      o[4] += hi.x * f;
      o[5] += hi.y * f;
      o[6] += hi.z * f;
      o[7] += hi.w * f;
    }
    if (n < Gp && hn < G) {
      const size_t pidx = partial_index(a, row, s, hn);
      float4* dst = reinterpret_cast<float4*>(a.part_o + pidx * kDim + 8 * (4 * g + wv));
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (g == 0 && wv == 0) {
        a.part_ml[pidx * 2] = M;  // log2 units
        a.part_ml[pidx * 2 + 1] = l;
      }
    }
    return;
  }
  // Partial of this split (unnormalised o, log2-domain m, l); the splits are merged
  // by a separate kernel: a release/acquire hand-off between waves of this kernel
  // would need an L2 write-back per wave, which measured far slower.
  if (n < Gp && hn < G) {
    const size_t pidx = partial_index(a, row, s, hn);
    float* o = a.part_o + pidx * kDim;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 8 * (4 * g + j);   // value block nb holds dims d0 + nb
      reinterpret_cast<float4*>(o + d0)[0] = make_float4(acc[0][j], acc[1][j], acc[2][j], acc[3][j]);
      reinterpret_cast<float4*>(o + d0)[1] = make_float4(acc[4][j], acc[5][j], acc[6][j], acc[7][j]);
    }
    if (g == 0) {
      a.part_ml[pidx * 2] = m_fin;  // log2 units
      a.part_ml[pidx * 2 + 1] = l_tot;
    }
  }
}

template <int KF, int VF, bool SPARSE>
void launch_sets(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  // decode step: the appended token's two work groups (if any) come first
  const dim3 grid(a.col0 + a.plan.max_splits, a.hkv, batch), block(64);
  // latency-bound calls (most SIMDs would be idle): four waves per split share its tokens
  if (a.plan.latency && !a.split_append) {
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, 1, SPARSE, 4>), grid, dim3(256), 0, stream, a, lens);
    return;
  }
  if constexpr (VF == kFmtF16)  // 128-byte V chunks: one token set keeps the registers in bounds
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, 1, SPARSE>), grid, block, 0, stream, a, lens);
  else if (a.group <= 16 / TQ_MFMA_NS_SMALL_GROUP)
    hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, TQ_MFMA_NS_SMALL_GROUP, SPARSE>), grid, block, 0, stream, a, lens);
  else if (a.group <= 8) hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, 2, SPARSE>), grid, block, 0, stream, a, lens);
  else hipLaunchKernelGGL((decode_mfma_kernel<KF, VF, 1, SPARSE>), grid, block, 0, stream, a, lens);
}

template <int KF, int VF>
hipError_t launch_fmt(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  if (a.v_skip_log2 > -INFINITY || a.k_skip_log2 > -INFINITY) launch_sets<KF, VF, true>(a, lens, batch, stream);
  else launch_sets<KF, VF, false>(a, lens, batch, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo3) return launch_fmt<kFmtTurbo3, kFmtTurbo3>(a, lens, batch, stream);
  if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo4) return launch_fmt<kFmtTurbo3, kFmtTurbo4>(a, lens, batch, stream);
  if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo3) return launch_fmt<kFmtTurbo4, kFmtTurbo3>(a, lens, batch, stream);
  if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo4) return launch_fmt<kFmtTurbo4, kFmtTurbo4>(a, lens, batch, stream);
  if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo3) return launch_fmt<kFmtF16, kFmtTurbo3>(a, lens, batch, stream);
  if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo4) return launch_fmt<kFmtF16, kFmtTurbo4>(a, lens, batch, stream);
  if (a.kfmt == kFmtF16 && a.vfmt == kFmtF16) return launch_fmt<kFmtF16, kFmtF16>(a, lens, batch, stream);
  return hipErrorInvalidValue;
}

}  // namespace tq
