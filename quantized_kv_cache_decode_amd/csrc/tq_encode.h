// Device-side encoder of the rotated scalar codec, shared by the append kernels
// and the decode step's in-kernel append (mlxcel PR #369, "Change": the append is
// the only cache mutation; turboquant_plus "SMEM Pre-Dequant Experiment", "What
// Would Actually Work", item 1: a value is the codebook entry at its index times
// the group norm).
//
// Per 128-element row x (fp16), held by a 16-lane group (lane j: elements 8j..8j+7)
// in the bulk encoder, or by a whole wave, two elements per lane, in the single-row
// appends (see the wave-wide section below):
//   norm  n = RNE_fp16(sqrt(sum x_i^2)), bit-exact: the sum of squares is taken in
//         binary64 (every square is exact; 11 roundings at most along any path of
//         the 16-lane sum), so sqrt is known to a relative 2^-49; the fp16 rounding
//         is decided from it unless it lies within 2^-45 of a rounding midpoint, in
//         which case (ties included) the exact integer method decides: each
//         |x_i| * 2^24 is an integer below 2^40, its square split in 20-bit halves
//         whose sums fit in u64, recombined in a u128, and the rounding decision is
//         an integer comparison (4 S vs q^2 (2k+1)^2).
//   yhat  = H (s * x): butterflies in binary64, exact (fp16 terms are multiples of
//         2^-24 below 2^16).
//   idx_i = #{j : y_i > n * beta_j} with y_i = yhat_i / sqrt(128) and beta_j the
//         midpoints of adjacent fp16 codebook entries, decided as yhat_i against
//         the thresholds n * beta_j * sqrt(128) in binary64, and, since the codebook
//         is symmetric (c[K-1-i] = -c[i], so beta is too, with 0 in the middle), as
//         |yhat_i| against the positive half of them.  This differs from dividing
//         first only where y_i is within a few ulps of a threshold -- inside the
//         1e-5 boundary margin the parity checks excuse.
#pragma once

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

constexpr double kSqrtD = 11.313708498984761;  // binary64 value of sqrt(128)

__device__ inline int bitlen_u128(unsigned __int128 v) {
  const uint64_t hi = uint64_t(v >> 64), lo = uint64_t(v);
  if (hi) return 128 - __builtin_clzll(hi);
  return lo ? 64 - __builtin_clzll(lo) : 0;
}

// fp16 bits of RNE(sqrt(S) * 2^-24), S = A*2^40 + Bsum*2^21 + C, saturating at 65504.
__device__ __forceinline__ uint16_t exact_norm_fp16(uint64_t A, uint64_t Bsum, uint64_t C) {
  const unsigned __int128 S = ((unsigned __int128)A << 40) + ((unsigned __int128)Bsum << 21) + C;
  if (S == 0) return 0;
  const int E = (bitlen_u128(S) - 1) >> 1;      // floor(log2 sqrt(S))
  const int eq = E <= 10 ? 0 : E - 10;          // fp16 spacing q = 2^eq (units of 2^-24)
  const uint64_t Sq = uint64_t(S >> (2 * eq));  // floor(S / q^2) < 2^22
  uint64_t k = uint64_t(sqrt(double(Sq)));
  while (k * k > Sq) --k;
  while ((k + 1) * (k + 1) <= Sq) ++k;
  const unsigned __int128 lhs = S << 2;
  const unsigned __int128 rhs = (unsigned __int128)((2 * k + 1) * (2 * k + 1)) << (2 * eq);
  if (lhs > rhs || (lhs == rhs && (k & 1))) ++k;
  const double v = ldexp(double(k), eq - 24);
  if (v > 65504.0) return 0x7bff;
  return __half_as_ushort(__float2half_rn(float(v)));  // v is an fp16 value: exact
}

// Decision thresholds beta_i = (c_i + c_{i+1}) / 2 of an ascending fp16 codebook,
// in binary64 (exact: a sum of two fp16 values, halved), held in registers.
template <int FMT>
__device__ __forceinline__ void load_thresholds(const uint16_t* cb, double (&beta)[levels(FMT) - 1]) {
  constexpr int K = levels(FMT);
  float c[K];
#pragma unroll
  for (int i = 0; i < K; ++i) c[i] = half_bits_to_float(cb[i]);
#pragma unroll
  for (int i = 0; i < K - 1; ++i) beta[i] = 0.5 * (double(c[i]) + double(c[i + 1]));
}

// fp16 bits of RNE(sqrt(ss)), ss a binary64 sum of squares whose square root is
// within a relative 2^-49 of the exact norm; 0xffff when that cannot decide the
// rounding (within 2^-45 of a rounding midpoint, ties included).  Saturates at 65504.
__device__ __forceinline__ uint32_t fast_norm_fp16(double ss) {
  if (ss == 0.0) return 0;
  const double r = sqrt(ss);
  if (r >= 65504.0) return 0x7bff;                // everything from 65504 up gives 65504
  const int e = ilogb(r);
  const int qe = (e < -14 ? -14 : e) - 10;        // fp16 spacing 2^qe at r (2^-24 below 2^-14)
  const double k = ldexp(r, -qe);                 // r in units of the spacing (exact)
  const double fk = floor(k);
  const double frac = k - fk;                     // exact
  if (fabs(frac - 0.5) <= k * 0x1p-45) return 0xffff;
  const double kr = frac > 0.5 ? fk + 1.0 : fk;
  return __half_as_ushort(__float2half_rn(float(ldexp(kr, qe))));  // an fp16 value: exact
}

// The exact norm (integer method) of a row held by a 16-lane group; every lane of
// the group must execute it.
__device__ __forceinline__ uint16_t exact_row_norm_fp16(const uint32_t (&w4)[4]) {
  uint64_t sA = 0, sB = 0, sC = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double xv = double(half_bits_to_float(uint16_t(w4[e >> 1] >> (16 * (e & 1)))));
    const uint64_t m = uint64_t(fabs(xv) * 16777216.0);  // exact integer < 2^40
    const uint64_t mh = m >> 20, ml = m & 0xfffffull;
    sA += mh * mh;
    sB += mh * ml;
    sC += ml * ml;
  }
  auto sum_stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
    sA += xor_lane16<M>(sA);
    sB += xor_lane16<M>(sB);
    sC += xor_lane16<M>(sC);
  };
  sum_stage(std::integral_constant<int, 1>{});
  sum_stage(std::integral_constant<int, 2>{});
  sum_stage(std::integral_constant<int, 4>{});
  sum_stage(std::integral_constant<int, 8>{});
  return exact_norm_fp16(sA, sB, sC);
}

// Value of lane (lane ^ M) of the 16-lane row for a binary64 value.  LDS_EXCHANGE: xor 4
// and 8 through ds_swizzle (one LDS-pipe instruction per 32-bit half, no VALU slot)
// instead of two DPP moves per half -- for throughput-bound callers whose many
// independent exchanges hide the LDS pipe's latency; xor 1 and 2 stay single DPP moves.
template <int M, bool LDS_EXCHANGE>
__device__ __forceinline__ double exchange_lane16(double v) {
  if constexpr (LDS_EXCHANGE && (M == 4 || M == 8)) {
    constexpr int kPattern = 0x1f | (M << 10);   // bit mode: lane ^ M within each group of 32
    const uint64_t u = uint64_t(__double_as_longlong(v));
    const uint32_t lo = uint32_t(__builtin_amdgcn_ds_swizzle(int(uint32_t(u)), kPattern));
    const uint32_t hi = uint32_t(__builtin_amdgcn_ds_swizzle(int(uint32_t(u >> 32)), kPattern));
    return __longlong_as_double(int64_t(uint64_t(lo) | (uint64_t(hi) << 32)));
  } else {
    return xor_lane16<M>(v);
  }
}

// Encode one 128-element row held by a 16-lane group (lane j: elements 8j..8j+7,
// fp16 bits in w4, sign flips in sg).  Returns the fp16 norm bits (the same in all
// 16 lanes) and this lane's 8 codes.  All 16 lanes of the group execute it together.
template <int FMT, bool LDS_EXCHANGE = false>
__device__ __forceinline__ uint16_t encode_row(const uint32_t (&w4)[4], const float (&sg)[8],
                                      const double (&beta)[levels(FMT) - 1], int j, uint8_t (&code)[8]) {
  double x[8];
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double xv = double(half_bits_to_float(uint16_t(w4[e >> 1] >> (16 * (e & 1)))));
    ss = fma(xv, xv, ss);  // the square is exact: one rounding per term
    x[e] = xv * double(sg[e]);
  }
  auto sum_stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
    ss += exchange_lane16<M, LDS_EXCHANGE>(ss);   // both lanes of a pair add the same two values: identical sums
  };
  sum_stage(std::integral_constant<int, 1>{});
  sum_stage(std::integral_constant<int, 2>{});
  sum_stage(std::integral_constant<int, 4>{});
  sum_stage(std::integral_constant<int, 8>{});
  // Walsh-Hadamard in binary64: element bits 0..2 in-lane, bits 3..6 across lanes j ^ 1..8
#pragma unroll
  for (int hh = 1; hh < 8; hh <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & hh)) {
        const double u = x[e], v = x[e + hh];
        x[e] = u + v;
        x[e + hh] = u - v;
      }
    }
  }
  auto fwht_stage = [&](auto m_c) {
    constexpr int M = decltype(m_c)::value;
    const double sgn = (j & M) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double o = exchange_lane16<M, LDS_EXCHANGE>(x[e]);
      x[e] = fma(x[e], sgn, o);  // o - x or x + o, exactly
    }
  };
  fwht_stage(std::integral_constant<int, 1>{});
  fwht_stage(std::integral_constant<int, 2>{});
  fwht_stage(std::integral_constant<int, 4>{});
  fwht_stage(std::integral_constant<int, 8>{});
  uint32_t nb = fast_norm_fp16(ss);
  if (nb == 0xffffu) nb = exact_row_norm_fp16(w4);  // the same for all 16 lanes of the row
  const uint16_t nbits = uint16_t(nb);
  const double nd = double(half_bits_to_float(nbits));
  constexpr int K = levels(FMT), Hf = K / 2;
  double U[Hf - 1];  // the positive thresholds, scaled by sqrt(128): n * beta_(Hf-1+k) * sqrt(128)
#pragma unroll
  for (int k = 1; k < Hf; ++k) U[k - 1] = (nd * beta[Hf - 1 + k]) * kSqrtD;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double a = fabs(x[e]);
    int cnt = 0;  // positive thresholds below |yhat|
#pragma unroll
    for (int k = 0; k < Hf - 1; ++k) cnt += a > U[k] ? 1 : 0;
    // y > 0: the Hf thresholds <= 0 and cnt positive ones lie below it; y <= 0: of the
    // Hf - 1 negative thresholds -U, those above -|y| (|y| < U) lie below it.  An all-zero
    // row (n = 0) encodes to index 0 everywhere.
    const int c = x[e] > 0.0 ? Hf + cnt : Hf - 1 - cnt;
    code[e] = uint8_t(nd == 0.0 ? 0 : c);
  }
  return nbits;
}

// Load the 8 fp16 elements 8j..8j+7 of a row and the matching sign flips.
__device__ __forceinline__ void load_row_and_signs(const uint16_t* src, const float* signs, int j, uint32_t (&w4)[4],
                                          float (&sg)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  w4[0] = raw.x;
  w4[1] = raw.y;
  w4[2] = raw.z;
  w4[3] = raw.w;
  const float4 s0 = reinterpret_cast<const float4*>(signs + 8 * j)[0];
  const float4 s1 = reinterpret_cast<const float4*>(signs + 8 * j)[1];
  sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
  sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
}

// Write the K record of token t of a row (row_k: the row's K bytes) from a 16-lane
// group's codes (lane j: dims 8j..8j+7).
template <int KFMT>
__device__ __forceinline__ void store_k_record(uint8_t* row_k, int t, const uint8_t (&code)[8], int j) {
  if (KFMT == kFmtTurbo4) {
    *reinterpret_cast<uint32_t*>(row_k + k_byte_offset(kFmtTurbo4, t, 4 * j)) = oct4_pack(code);
  } else {
    // Lanes 4q..4q+3 hold elements 8c..8c+7 (c = j % 4) of sub-block q.  Lanes with
    // c < 3 own word c outright (element 8c+i: byte i%4, bits 3*(i/4)); lane c = 3
    // holds elements 24..31, whose low two bits go to bits 6-7 of words A (24..27)
    // and B (28..31) and whose top bits go to bits 6 and 7 of word C.  Each lane
    // builds its share with constant shifts and the 4 lanes OR them together.
    const int c = j & 3;
    uint32_t own = 0, t0 = 0, t1 = 0, t2 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) own |= (uint32_t(code[i]) & 7u) << (8 * (i & 3) + 3 * (i >> 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t0 |= (uint32_t(code[i]) & 3u) << (8 * i + 6);
      t1 |= (uint32_t(code[4 + i]) & 3u) << (8 * i + 6);
      t2 |= ((uint32_t(code[i]) >> 2) & 1u) << (8 * i + 6);
      t2 |= ((uint32_t(code[4 + i]) >> 2) & 1u) << (8 * i + 7);
    }
    uint32_t w[3];
    w[0] = c == 0 ? own : (c == 3 ? t0 : 0u);
    w[1] = c == 1 ? own : (c == 3 ? t1 : 0u);
    w[2] = c == 2 ? own : (c == 3 ? t2 : 0u);
    w[0] |= xor_lane16<1>(w[0]);
    w[1] |= xor_lane16<1>(w[1]);
    w[2] |= xor_lane16<1>(w[2]);
    w[0] |= xor_lane16<2>(w[0]);
    w[1] |= xor_lane16<2>(w[1]);
    w[2] |= xor_lane16<2>(w[2]);
    if ((j & 3) == 0) {  // sub-block j / 4 is piece j / 4 of the record
      uint32_t* dst = reinterpret_cast<uint32_t*>(row_k + k_byte_offset(kFmtTurbo3, t, 12 * (j >> 2)));
      dst[0] = w[0];
      dst[1] = w[1];
      dst[2] = w[2];
    }
  }
}

// Decision thresholds (binary64) and v_perm byte tables of an fp16 codebook.
template <int FMT>
__device__ __forceinline__ void load_codebook(const uint16_t* cb, double (&beta)[levels(FMT) - 1],
                                              uint32_t (&tab)[levels(FMT) / 2]) {
  uint32_t c[levels(FMT)];
#pragma unroll
  for (int i = 0; i < levels(FMT); ++i) c[i] = cb[i];
#pragma unroll
  for (int i = 0; i < levels(FMT) - 1; ++i)
    beta[i] = 0.5 * (double(half_bits_to_float(uint16_t(c[i]))) + double(half_bits_to_float(uint16_t(c[i + 1]))));
#pragma unroll
  for (int h = 0; h < levels(FMT) / 8; ++h) {
    uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo0 |= (c[8 * h + i] & 0xffu) << (8 * i);
      lo1 |= (c[8 * h + 4 + i] & 0xffu) << (8 * i);
      hi0 |= (c[8 * h + i] >> 8) << (8 * i);
      hi1 |= (c[8 * h + 4 + i] >> 8) << (8 * i);
    }
    tab[4 * h] = lo0;
    tab[4 * h + 1] = lo1;
    tab[4 * h + 2] = hi0;
    tab[4 * h + 3] = hi1;
  }
}

// Codebook entry at a 3- or 4-bit index, as fp32, from the byte tables.
template <int FMT>
__device__ __forceinline__ float codebook_at(const uint32_t (&tab)[levels(FMT) / 2], uint32_t idx) {
  const uint32_t sel = idx & 7u;
  uint32_t lo = __builtin_amdgcn_perm(tab[1], tab[0], sel), hi = __builtin_amdgcn_perm(tab[3], tab[2], sel);
  if constexpr (levels(FMT) == 16) {
    const uint32_t lo8 = __builtin_amdgcn_perm(tab[5], tab[4], sel), hi8 = __builtin_amdgcn_perm(tab[7], tab[6], sel);
    lo = (idx & 8u) ? lo8 : lo;
    hi = (idx & 8u) ? hi8 : hi;
  }
  return half_bits_to_float(uint16_t((lo & 0xffu) | ((hi & 0xffu) << 8)));
}

// Copy an F16 K row (lane j: elements 8j..8j+7).
__device__ __forceinline__ void append_f16_k_row(const EncodeArgs& a, size_t row, int t, const uint16_t* src, int j) {
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_data) + (row * a.cap + t) * kDim + 8 * j) =
      *reinterpret_cast<const uint4*>(src + 8 * j);
}

// Store an F16 V row (lane j: dims 8j..8j+7) into its tile: chunk 16g + j, element
// 8*nb + i (i the token's element index in slot group g) is dim 8j + nb.
__device__ __forceinline__ void store_f16_v_row(const EncodeArgs& a, size_t row, int t, uint4 v, int j) {
  const int r = t % kTileTokens;
  uint16_t* chunk = reinterpret_cast<uint16_t*>(a.v_data + (row * (a.cap / kTileTokens) + t / kTileTokens) *
                                                              v_tile_bytes(kFmtF16)) +
                    (16 * slot_group(r) + j) * (v_chunk_bytes(kFmtF16) / 2) + slot_elem(r);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) chunk[8 * nb] = uint16_t(w[nb >> 1] >> (16 * (nb & 1)));
}

// ---- One row over a whole wave (the single-row appends: the decode step's and the
// one-row append kernel's).  Lane l = 16q + 4c + b holds elements e0 = 32q + 8c + b
// and e0 + 4: element bits 0-1 are lane bits 0-1, bit 2 is the lane's pair, bits 3-4
// are lane bits 2-3 and bits 5-6 lane bits 4-5.  The arithmetic is encode_row's (the same exact binary64
// transform, the same norm decision, the same thresholds), so codes and norms are
// bit-identical to it; each stage handles two values per lane instead of eight.
// All 64 lanes of the wave execute these routines together.
__device__ __forceinline__ int wave_row_elem(int lane) {
  return ((lane >> 4) << 5) | (((lane >> 2) & 3) << 3) | (lane & 3);
}

template <int FMT>
struct WaveRowInputs {
  uint32_t h01;          // fp16 bits of elements e0 (low half) and e0 + 4 (high half)
  float sg[2];           // their sign flips
  double beta[levels(FMT) - 1];
  uint32_t tab[levels(FMT) / 2];
};

template <int FMT>
__device__ __forceinline__ void load_wave_row_inputs(const uint16_t* src, const float* signs, const uint16_t* cb,
                                                     int lane, WaveRowInputs<FMT>& in) {
  const int e0 = wave_row_elem(lane);
  in.h01 = uint32_t(src[e0]) | (uint32_t(src[e0 + 4]) << 16);
  in.sg[0] = signs[e0];
  in.sg[1] = signs[e0 + 4];
  load_codebook<FMT>(cb, in.beta, in.tab);
}

// The exact norm (integer method) of a row spread over the wave.
__device__ __forceinline__ uint16_t exact_wave_row_norm_fp16(uint32_t h01, int lane) {
  uint64_t sA = 0, sB = 0, sC = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const double xv = double(half_bits_to_float(uint16_t(h01 >> (16 * e))));
    const uint64_t m = uint64_t(fabs(xv) * 16777216.0);  // exact integer < 2^40
    const uint64_t mh = m >> 20, ml = m & 0xfffffull;
    sA += mh * mh;
    sB += mh * ml;
    sC += ml * ml;
  }
  auto stage = [&](auto b_c) {
    constexpr int B = decltype(b_c)::value;
    sA = wave_sum<B>(sA, lane);
    sB = wave_sum<B>(sB, lane);
    sC = wave_sum<B>(sC, lane);
  };
  stage(std::integral_constant<int, 0>{});
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 3>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 5>{});
  return exact_norm_fp16(sA, sB, sC);
}

// Codes of elements e0 and e0 + 4 and the row's fp16 norm bits (the same in every
// lane).  The sum of squares takes 7 roundings at most along any path (one in-lane
// add, six exchange stages), within the 11 the norm decision allows for.
template <int FMT>
__device__ __forceinline__ uint16_t encode_wave_row(const WaveRowInputs<FMT>& in, int lane, uint32_t (&code)[2]) {
  const double x0 = double(half_bits_to_float(uint16_t(in.h01))), x1 = double(half_bits_to_float(uint16_t(in.h01 >> 16)));
  double ss = fma(x1, x1, x0 * x0);   // x0 * x0 is exact
  double x[2] = {x0 * double(in.sg[0]), x1 * double(in.sg[1])};
  {
    const double u = x[0], v = x[1];   // element bit 2, in-lane
    x[0] = u + v;
    x[1] = u - v;
  }
  auto stage = [&](auto b_c) {
    constexpr int B = decltype(b_c)::value;
    ss = wave_sum<B>(ss, lane);
    x[0] = wave_butterfly<B>(x[0], lane);
    x[1] = wave_butterfly<B>(x[1], lane);
  };
  stage(std::integral_constant<int, 0>{});
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 3>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 5>{});
  uint32_t nb = fast_norm_fp16(ss);
  if (nb == 0xffffu) nb = exact_wave_row_norm_fp16(in.h01, lane);   // uniform over the wave
  const uint16_t nbits = uint16_t(nb);
  const double nd = double(half_bits_to_float(nbits));
  constexpr int K = levels(FMT), Hf = K / 2;
  double U[Hf - 1];
#pragma unroll
  for (int k = 1; k < Hf; ++k) U[k - 1] = (nd * in.beta[Hf - 1 + k]) * kSqrtD;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const double a = fabs(x[e]);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < Hf - 1; ++k) cnt += a > U[k] ? 1 : 0;
    const int c = x[e] > 0.0 ? Hf + cnt : Hf - 1 - cnt;
    code[e] = uint32_t(nd == 0.0 ? 0 : c);
  }
  return nbits;
}

// Write token t's K record from the wave's codes.  turbo4: elements e0 and e0 + 4 are
// nibbles b and 4 + b of octet word 4q + c, i.e. record byte l.  turbo3: lane 12 + b
// of each sub-block's 16 lanes (elements 24 + b and 28 + b) owns bits 6-7 of byte b
// of words A, B and C; the other lanes own bits 0-5 of byte b of word c and fetch
// their bits 6-7 from it (ds_swizzle: lane l | 12 within each 32).
template <int KFMT>
__device__ __forceinline__ void store_k_record_wave(uint8_t* row_k, int t, const uint32_t (&code)[2], int lane) {
  if constexpr (KFMT == kFmtTurbo4) {
    const uint32_t byte = t4_nibble_of_index(code[0]) | (t4_nibble_of_index(code[1]) << 4);
    row_k[k_byte_offset(kFmtTurbo4, t, lane)] = uint8_t(byte);
  } else {
    const int c = (lane >> 2) & 3, b = lane & 3;
    const uint32_t top = ((code[0] & 3u) << 6) | ((code[1] & 3u) << 14) | (((code[0] >> 2) & 1u) << 22) |
                         (((code[1] >> 2) & 1u) << 23);
    constexpr int kFromLane12 = 0x1f | (0x0c << 5);   // bit mode: and 0x1f, or 12, xor 0
    const uint32_t from = uint32_t(__builtin_amdgcn_ds_swizzle(int(top), kFromLane12));
    if (c < 3) {
      const uint32_t byte = (code[0] & 7u) | ((code[1] & 7u) << 3) | ((from >> (8 * c)) & 0xc0u);
      row_k[k_byte_offset(kFmtTurbo3, t, 12 * (lane >> 4) + 4 * c + b)] = uint8_t(byte);
    }
  }
}

// Encode token t's K row over the whole wave and write its norm and record.
template <int KFMT>
__device__ __forceinline__ uint16_t append_k_row_wave(const EncodeArgs& a, size_t row, int t,
                                                      const WaveRowInputs<KFMT>& in, int lane, uint32_t (&code)[2]) {
  const uint16_t nbits = encode_wave_row<KFMT>(in, lane, code);
  if (lane == 0) a.k_norms[row * a.cap + t] = nbits;
  store_k_record_wave<KFMT>(a.k_data + row * a.cap * k_record_bytes(KFMT), t, code, lane);
  return nbits;
}

// The V side over the whole wave: this lane's two dims 8j + b and 8j + 4 + b (j = 4q + c)
// sit in chunk 16 g + j of the token's tile (g its slot group), in chunk words b and
// 4 + b (turbo4: a dim's word holds its 8 slots' nibbles) or word b of the chunk's two
// sub-blocks (turbo3: the token's field for dim d is element 8 (d % 4) + ei of d's
// sub-block, ei the slot's element index).  turbo3: the fields of dims 8j + 3 and
// 8j + 7 (sub-block elements 24 + ei) are split over words 0-2, so lane 3 of each
// quad writes nothing and lanes 0-2 take its codes (a quad broadcast) into the words
// they rewrite.  Every other slot's fields are kept.
template <int VFMT>
struct WaveVInputs {
  WaveRowInputs<VFMT> row;
  uint32_t cw[2];            // the two chunk words this lane rewrites
  uint32_t off[2];           // their byte offsets in the tile
  uint8_t* tile;
  int ei;                    // chunk element of the token's slot
};

template <int VFMT>
__device__ __forceinline__ void load_wave_v_inputs(const EncodeArgs& a, size_t row, int t, const uint16_t* src, int lane,
                                                   WaveVInputs<VFMT>& in) {
  const int r = t % kTileTokens, g = slot_group(r);
  in.ei = slot_elem(r);
  in.tile = a.v_data + (row * (a.cap / kTileTokens) + t / kTileTokens) * v_tile_bytes(VFMT);
  const int chunk = 16 * g + (wave_row_elem(lane) >> 3);
  if constexpr (VFMT == kFmtTurbo4) {
    in.off[0] = v_chunk_byte_offset(VFMT, chunk, 4 * (lane & 3));
    in.off[1] = v_chunk_byte_offset(VFMT, chunk, 16 + 4 * (lane & 3));
  } else {
    const int w = min(lane & 3, 2);  // lane 3 of a quad rewrites nothing (its words are lane 0-2's)
    in.off[0] = v_chunk_byte_offset(VFMT, chunk, 4 * w);
    in.off[1] = v_chunk_byte_offset(VFMT, chunk, 12 + 4 * w);
  }
  // a token in slot 0 starts the tile: the other slots hold nothing visible yet
#pragma unroll
  for (int i = 0; i < 2; ++i) in.cw[i] = r == 0 ? 0u : *reinterpret_cast<const uint32_t*>(in.tile + in.off[i]);
  load_wave_row_inputs<VFMT>(src, a.v_signs, a.v_cb, lane, in.row);
}

template <int VFMT>
__device__ __forceinline__ uint16_t append_v_row_wave(const EncodeArgs& a, size_t row, int t, WaveVInputs<VFMT>& in,
                                                      int lane, uint32_t (&code)[2]) {
  const uint16_t nbits = encode_wave_row<VFMT>(in.row, lane, code);
  const int b = lane & 3;
  if constexpr (VFMT == kFmtTurbo4) {
    const int sh = oct4_bit(in.ei);
#pragma unroll
    for (int i = 0; i < 2; ++i) in.cw[i] = (in.cw[i] & ~(15u << sh)) | (t4_nibble_of_index(code[i]) << sh);
  } else {
    const uint32_t c3 = dpp_u32<0xff>(code[0] | (code[1] << 8));   // quad_perm [3,3,3,3]
    const int jj = in.ei & 3, up = in.ei >> 2;
    const int sh = 8 * jj + 3 * up;      // own field (sub-block element 8b + ei, b < 3)
    const int s2 = 8 * jj + 6;           // low two bits of element 24 + ei, in word `up`
    const int s1 = 8 * jj + 6 + up;      // its top bit, in word 2
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t c = code[i], d = (c3 >> (8 * i)) & 0xffu;
      uint32_t m = 7u << sh, v = (c & 7u) << sh;
      if (b == up) {
        m |= 3u << s2;
        v |= (d & 3u) << s2;
      }
      if (b == 2) {
        m |= 1u << s1;
        v |= ((d >> 2) & 1u) << s1;
      }
      in.cw[i] = (in.cw[i] & ~m) | v;
    }
  }
  if (VFMT == kFmtTurbo4 || b < 3) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint32_t*>(in.tile + in.off[i]) = in.cw[i];
  }
  if (lane == 0) a.v_norms[row * a.cap + t] = nbits;
  return nbits;
}

}  // namespace tq
