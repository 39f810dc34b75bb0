// Encode + append of new K/V tokens (the cache update; mlxcel PR #369,
// "Change": the append is the only cache mutation).
//
// One workgroup per (32-token V tile touched by the append, KV head,
// sequence).  256 threads = 16 groups of 16 lanes; each group encodes one K or
// V row of a new token of the tile (lane j holds dims 8j..8j+7), so a
// one-token append keeps its dependency chains short.
//
// Per group x (fp16 [128]):
//   norm  n = RNE_fp16(sqrt(sum x_i^2)) computed exactly: each |x_i| * 2^24 is
//         an integer below 2^40; its square is split in 20-bit halves whose sums
//         fit in u64, recombined in a u128, and the fp16 rounding decision is an
//         integer comparison (4 S vs q^2 (2k+1)^2).
//   y     = H (s * x) / sqrt(128): butterflies in binary64 (exact: fp16 terms
//         are multiples of 2^-24 below 2^16), then one IEEE division.
//   idx_i = #{j : y_i > n * beta_j}, beta_j = midpoints of adjacent fp16 codebook
//         entries (n * beta_j is exact in binary64), found by binary search.
// K rows are written as token-major records; V codes are staged in LDS and
// written as whole V-tile chunk words by one thread per chunk, merging with the
// words of tokens already in the tile.  F16 K rows are copied unchanged.
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr double kSqrtD = 11.313708498984761;  // binary64 value of sqrt(128)

__device__ inline int bitlen_u128(unsigned __int128 v) {
  const uint64_t hi = uint64_t(v >> 64), lo = uint64_t(v);
  if (hi) return 128 - __builtin_clzll(hi);
  return lo ? 64 - __builtin_clzll(lo) : 0;
}

// fp16 bits of RNE(sqrt(S) * 2^-24), S = A*2^40 + Bsum*2^21 + C, saturating at 65504.
__device__ uint16_t exact_norm_fp16(uint64_t A, uint64_t Bsum, uint64_t C) {
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
__device__ inline void load_thresholds(const uint16_t* cb, double (&beta)[levels(FMT) - 1]) {
  constexpr int K = levels(FMT);
  float c[K];
#pragma unroll
  for (int i = 0; i < K; ++i) c[i] = half_bits_to_float(cb[i]);
#pragma unroll
  for (int i = 0; i < K - 1; ++i) beta[i] = 0.5 * (double(c[i]) + double(c[i + 1]));
}

// Encode one 128-element row held by a 16-lane group (lane j: elements 8j..8j+7,
// fp16 bits in w4, sign flips in sg).  Returns the fp16 norm bits (the same in all
// 16 lanes) and this lane's 8 codes.  All 16 lanes of the group execute it together.
template <int FMT>
__device__ inline uint16_t encode_row(const uint32_t (&w4)[4], const float (&sg)[8],
                                      const double (&beta)[levels(FMT) - 1], int j, uint8_t (&code)[8]) {
  double x[8];
  uint64_t sA = 0, sB = 0, sC = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double xv = double(half_bits_to_float(uint16_t(w4[e >> 1] >> (16 * (e & 1)))));
    const uint64_t m = uint64_t(fabs(xv) * 16777216.0);  // exact integer < 2^40
    const uint64_t mh = m >> 20, ml = m & 0xfffffull;
    sA += mh * mh;
    sB += mh * ml;
    sC += ml * ml;
    x[e] = xv * double(sg[e]);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    sA += __shfl_xor(sA, m, 16);
    sB += __shfl_xor(sB, m, 16);
    sC += __shfl_xor(sC, m, 16);
  }
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
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double o = __shfl_xor(x[e], m, 16);
      x[e] = (j & m) ? (o - x[e]) : (x[e] + o);
    }
  }
  const uint16_t nbits = exact_norm_fp16(sA, sB, sC);
  const double nd = double(half_bits_to_float(nbits));
  constexpr int K = levels(FMT);
  double T[K - 1];
#pragma unroll
  for (int i = 0; i < K - 1; ++i) T[i] = nd * beta[i];  // exact in binary64
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double y = x[e] / kSqrtD;
    int c = 0;  // the number of thresholds below y
#pragma unroll
    for (int i = 0; i < K - 1; ++i) c += y > T[i] ? 1 : 0;
    code[e] = uint8_t(c);
  }
  return nbits;
}

// Load the 8 fp16 elements 8j..8j+7 of a row and the matching sign flips.
__device__ inline void load_row_and_signs(const uint16_t* src, const float* signs, int j, uint32_t (&w4)[4],
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

// Write the K record of one token from a 16-lane group's codes (lane j: dims 8j..8j+7).
template <int KFMT>
__device__ inline void store_k_record(uint8_t* rec, const uint8_t (&code)[8], int j) {
  if (KFMT == kFmtTurbo4) {
    *reinterpret_cast<uint32_t*>(rec + 4 * j) = oct4_pack(code);
  } else {
    // lanes 4q..4q+3 hold elements 8c..8c+7 (c = j % 4) of sub-block q; OR their fields
    uint8_t c32[32] = {};
    const int c0 = 8 * (j & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) c32[c0 + e] = code[e];
    uint32_t w[3];
    sub3_pack(c32, w);
#pragma unroll
    for (int m = 1; m < 4; m <<= 1) {
      w[0] |= __shfl_xor(w[0], m, 16);
      w[1] |= __shfl_xor(w[1], m, 16);
      w[2] |= __shfl_xor(w[2], m, 16);
    }
    if ((j & 3) == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(rec + 12 * (j >> 2));
      dst[0] = w[0];
      dst[1] = w[1];
      dst[2] = w[2];
    }
  }
}

template <int KFMT, int VFMT>
__global__ __launch_bounds__(256) void encode_append_kernel(EncodeArgs a, AppendStarts starts) {
  const int b = a.b0 + blockIdx.z;
  const int h = blockIdx.y;
  const int start = starts.start[blockIdx.z];
  const int end = start + starts.count[blockIdx.z];
  const int tile = start / kTileTokens + blockIdx.x;
  const int lo = max(tile * kTileTokens, start);
  const int hi = min(tile * kTileTokens + kTileTokens, end);
  if (lo >= hi) return;  // uniform over the block

  __shared__ uint8_t vcodes[kTileTokens][kDim];
  const int tid = threadIdx.x;
  const size_t row = size_t(b) * a.hkv + h;  // (sequence, KV head) row
  // Threads 0..63 own V-tile chunk tid.  When the tile already holds other tokens,
  // its old words are requested now so the read overlaps the encode below.
  const bool whole = lo == tile * kTileTokens && hi == tile * kTileTokens + kTileTokens;
  uint8_t* chunk = a.v_data + (row * (a.cap / kTileTokens) + tile) * v_tile_bytes(VFMT) + (tid & 63) * v_chunk_bytes(VFMT);
  constexpr int kChunkWords = v_chunk_bytes(VFMT) / 4;
  uint32_t old[kChunkWords];
#pragma unroll
  for (int i = 0; i < kChunkWords; ++i) old[i] = 0;
  if (tid < 64 && !whole) {
#pragma unroll
    for (int i = 0; i < kChunkWords; ++i) old[i] = reinterpret_cast<const uint32_t*>(chunk)[i];
  }

  // Active rows: n_tok new tokens of this tile, each with a K row and a V row.
  // Group gi (16 lanes) encodes K of token lo + gi for gi < n_tok, else V of token lo + gi - n_tok.
  const int n_tok = hi - lo;
  const int j = tid & 15;                 // lane within the group: dims 8j..8j+7
  for (int gi = tid >> 4; gi < 2 * n_tok; gi += 16) {
    const bool is_v = gi >= n_tok;
    const int t = lo + (is_v ? gi - n_tok : gi);
    const int r = t - tile * kTileTokens;
    const size_t src_off = (row * a.t_new + size_t(t - start)) * kDim + 8 * j;
    const size_t slot = row * a.cap + t;
    uint32_t w4[4];
    float sg[8];
    uint8_t code[8];
    if (is_v) {
      double beta[levels(VFMT) - 1];
      load_row_and_signs(a.v_new + src_off, a.v_signs, j, w4, sg);
      load_thresholds<VFMT>(a.v_cb, beta);
      const uint16_t nbits = encode_row<VFMT>(w4, sg, beta, j, code);
      *reinterpret_cast<uint2*>(&vcodes[r][8 * j]) =
          make_uint2(uint32_t(code[0]) | uint32_t(code[1]) << 8 | uint32_t(code[2]) << 16 | uint32_t(code[3]) << 24,
                     uint32_t(code[4]) | uint32_t(code[5]) << 8 | uint32_t(code[6]) << 16 | uint32_t(code[7]) << 24);
      if (j == 0) a.v_norms[slot] = nbits;
    } else if (KFMT == kFmtF16) {
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_data) + slot * kDim + 8 * j) =
          *reinterpret_cast<const uint4*>(a.k_new + src_off);
    } else {
      constexpr int KQ = KFMT == kFmtF16 ? kFmtTurbo3 : KFMT;  // (F16 K never gets here)
      double beta[levels(KQ) - 1];
      load_row_and_signs(a.k_new + src_off, a.k_signs, j, w4, sg);
      load_thresholds<KQ>(a.k_cb, beta);
      const uint16_t nbits = encode_row<KQ>(w4, sg, beta, j, code);
      if (j == 0) a.k_norms[slot] = nbits;
      store_k_record<KQ>(a.k_data + slot * k_record_bytes(KQ), code, j);
    }
  }
  __syncthreads();

  // V tile chunks: one thread per chunk c = 16 g + n (dims 8n..8n+7, slots r(g, i)).
  if (tid < 64) {
    const int g = tid >> 4, n = tid & 15;
    uint8_t el[64];
    if (!whole) {
      if constexpr (VFMT == kFmtTurbo3) {
        const uint32_t w0[3] = {old[0], old[1], old[2]}, w1[3] = {old[3], old[4], old[5]};
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          el[e] = uint8_t(sub3_get(w0, e));
          el[32 + e] = uint8_t(sub3_get(w1, e));
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const uint32_t word = old[nb];
#pragma unroll
          for (int i = 0; i < 8; ++i) el[8 * nb + i] = uint8_t(t4_index_of_nibble(oct4_get_nibble(word, i)));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = slot_of(g, i);
      const int tt = tile * kTileTokens + rr;
      const bool fresh = tt >= lo && tt < hi;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (fresh) el[8 * nb + i] = vcodes[rr][8 * n + nb];
    }
    if constexpr (VFMT == kFmtTurbo3) {
      uint32_t w[6];
      sub3_pack(el, w);
      sub3_pack(el + 32, w + 3);
      uint32_t* dst = reinterpret_cast<uint32_t*>(chunk);
#pragma unroll
      for (int i = 0; i < 6; ++i) dst[i] = w[i];
    } else {
      uint32_t w[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) w[nb] = oct4_pack(el + 8 * nb);
      uint4* dst = reinterpret_cast<uint4*>(chunk);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
  if (blockIdx.x == 0 && h == 0 && tid == 0) a.seq_lens[b] = end;
}

// Replace code e (0..31) of a turbo3 sub-block (words w0, w1, w2 = A, B, C) with c.
// `e` may differ per call but the word each field lands in is chosen by selects,
// never by a run-time register index.
__device__ inline void sub3_set(uint32_t& w0, uint32_t& w1, uint32_t& w2, int e, uint32_t c) {
  const int jj = e & 3;
  if (e < 24) {
    const int sh = 8 * jj + ((e >> 2) & 1) * 3;
    const uint32_t m = 7u << sh, v = (c & 7u) << sh;
    const int word = e >> 3;
    if (word == 0) w0 = (w0 & ~m) | v;
    else if (word == 1) w1 = (w1 & ~m) | v;
    else w2 = (w2 & ~m) | v;
  } else {
    const int upper = e >= 28 ? 1 : 0;
    const int sh = 8 * jj + 6;
    const uint32_t m = 3u << sh, v = (c & 3u) << sh;
    if (upper) w1 = (w1 & ~m) | v;
    else w0 = (w0 & ~m) | v;
    const int hb = sh + upper;
    w2 = (w2 & ~(1u << hb)) | (((c >> 2) & 1u) << hb);
  }
}

// The decode step's append: one new token in every listed sequence (count 0 or 1).
// One 16-lane group per row; waves 0-1 of a block encode the K rows of 8 (sequence,
// KV head) pairs and waves 2-3 their V rows, so no wave mixes the two paths.  The V
// row's codes go straight into the 64 V-tile chunks of its tile: lane j rewrites the
// 8 fields of its chunk 16*g + j that belong to the token's slot (group g, element
// i), keeping the words of the other slots.  Every load is issued up front: one
// memory round trip, no barrier.
template <int KFMT, int VFMT>
__global__ __launch_bounds__(256) void append_one_kernel(EncodeArgs a, AppendStarts starts, int nb) {
  const int j = threadIdx.x & 15;
  const int pair = blockIdx.x * 8 + ((threadIdx.x >> 4) & 7);
  const bool is_v = threadIdx.x >= 128;
  const int i = pair / a.hkv, h = pair % a.hkv;
  if (i >= nb || starts.count[i] == 0) return;  // whole 16-lane groups
  const int b = a.b0 + i;
  const int t = starts.start[i];
  const size_t row = size_t(b) * a.hkv + h;
  const size_t slot = row * a.cap + t;
  const size_t src_off = row * a.t_new * kDim + 8 * j;  // token 0 of the new rows
  uint32_t w4[4];
  float sg[8];
  uint8_t code[8];
  if (is_v) {
    const int r = t % kTileTokens, g = slot_group(r), ei = slot_elem(r);
    uint8_t* chunk = a.v_data + (row * (a.cap / kTileTokens) + t / kTileTokens) * v_tile_bytes(VFMT) +
                     (16 * g + j) * v_chunk_bytes(VFMT);
    constexpr int kChunkWords = v_chunk_bytes(VFMT) / 4;
    uint32_t cw[kChunkWords];
    // a token in slot 0 starts the tile: the other slots hold nothing visible yet
#pragma unroll
    for (int k = 0; k < kChunkWords; ++k) cw[k] = r == 0 ? 0u : reinterpret_cast<const uint32_t*>(chunk)[k];
    double beta[levels(VFMT) - 1];
    load_row_and_signs(a.v_new + src_off, a.v_signs, j, w4, sg);
    load_thresholds<VFMT>(a.v_cb, beta);
    const uint16_t nbits = encode_row<VFMT>(w4, sg, beta, j, code);
    // chunk element 8*n8 + ei is dim 8j + n8 of this token
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8) {
      if (VFMT == kFmtTurbo4) {
        const int sh = oct4_bit(ei);
        cw[n8] = (cw[n8] & ~(15u << sh)) | (t4_nibble_of_index(code[n8]) << sh);
      } else {
        const int sb = n8 >> 2;  // sub-block of element 8*n8 + ei
        sub3_set(cw[3 * sb], cw[3 * sb + 1], cw[3 * sb + 2], 8 * (n8 & 3) + ei, code[n8]);
      }
    }
    if (VFMT == kFmtTurbo4) {
      uint4* dst = reinterpret_cast<uint4*>(chunk);
      dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(chunk);
#pragma unroll
      for (int k = 0; k < kChunkWords; ++k) dst[k] = cw[k];
    }
    if (j == 0) a.v_norms[slot] = nbits;
  } else {
    if (KFMT == kFmtF16) {
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_data) + slot * kDim + 8 * j) =
          *reinterpret_cast<const uint4*>(a.k_new + src_off);
    } else {
      constexpr int KQ = KFMT == kFmtF16 ? kFmtTurbo3 : KFMT;  // (F16 K never gets here)
      double beta[levels(KQ) - 1];
      load_row_and_signs(a.k_new + src_off, a.k_signs, j, w4, sg);
      load_thresholds<KQ>(a.k_cb, beta);
      const uint16_t nbits = encode_row<KQ>(w4, sg, beta, j, code);
      if (j == 0) a.k_norms[slot] = nbits;
      store_k_record<KQ>(a.k_data + slot * k_record_bytes(KQ), code, j);
    }
    if (h == 0 && j == 0) a.seq_lens[b] = t + 1;
  }
}

template <int KF, int VF>
void launch_one(const EncodeArgs& a, const AppendStarts& s, int nb, int max_tiles, bool single,
                hipStream_t stream) {
  if (single)
    hipLaunchKernelGGL((append_one_kernel<KF, VF>), dim3((nb * a.hkv + 7) / 8), dim3(256), 0, stream, a, s, nb);
  else
    hipLaunchKernelGGL((encode_append_kernel<KF, VF>), dim3(max_tiles, a.hkv, nb), dim3(256), 0, stream, a, s);
}

}  // namespace

hipError_t launch_encode_append(const EncodeArgs& a, const AppendStarts& starts, int nb, int max_tiles,
                                hipStream_t stream) {
  // one token per sequence at most (the decode step): the one-pass kernel
  bool single = a.t_new == 1;
  for (int i = 0; i < nb && single; ++i) single = starts.count[i] <= 1;
  const int k = a.kfmt, v = a.vfmt;
  if (k == kFmtTurbo3 && v == kFmtTurbo3) launch_one<kFmtTurbo3, kFmtTurbo3>(a, starts, nb, max_tiles, single, stream);
  else if (k == kFmtTurbo3 && v == kFmtTurbo4) launch_one<kFmtTurbo3, kFmtTurbo4>(a, starts, nb, max_tiles, single, stream);
  else if (k == kFmtTurbo4 && v == kFmtTurbo3) launch_one<kFmtTurbo4, kFmtTurbo3>(a, starts, nb, max_tiles, single, stream);
  else if (k == kFmtTurbo4 && v == kFmtTurbo4) launch_one<kFmtTurbo4, kFmtTurbo4>(a, starts, nb, max_tiles, single, stream);
  else if (k == kFmtF16 && v == kFmtTurbo3) launch_one<kFmtF16, kFmtTurbo3>(a, starts, nb, max_tiles, single, stream);
  else if (k == kFmtF16 && v == kFmtTurbo4) launch_one<kFmtF16, kFmtTurbo4>(a, starts, nb, max_tiles, single, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq
