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
  __shared__ double beta_k[15], beta_v[15];
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
  if (tid < levels(VFMT) - 1)
    beta_v[tid] = 0.5 * (double(half_bits_to_float(a.v_cb[tid])) + double(half_bits_to_float(a.v_cb[tid + 1])));
  if (KFMT != kFmtF16 && tid >= 32 && tid - 32 < levels(KFMT) - 1)
    beta_k[tid - 32] =
        0.5 * (double(half_bits_to_float(a.k_cb[tid - 32])) + double(half_bits_to_float(a.k_cb[tid - 31])));
  __syncthreads();

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
    if (!is_v && KFMT == kFmtF16) {
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_data) + slot * kDim + 8 * j) =
          *reinterpret_cast<const uint4*>(a.k_new + src_off);
      continue;
    }
    const uint4 raw = *reinterpret_cast<const uint4*>((is_v ? a.v_new : a.k_new) + src_off);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
    const float* sg = (is_v ? a.v_signs : a.k_signs) + 8 * j;
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
    const double* beta = is_v ? beta_v : beta_k;
    const int K = is_v ? levels(VFMT) : levels(KFMT);
    uint8_t code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double y = x[e] / kSqrtD;
      // count of thresholds n*beta below y, by binary search over the ascending thresholds
      int c = 0;
      for (int st = K >> 1; st >= 1; st >>= 1)
        if (y > nd * beta[c + st - 1]) c += st;
      code[e] = uint8_t(c);
    }
    if (is_v) {
      *reinterpret_cast<uint2*>(&vcodes[r][8 * j]) =
          make_uint2(uint32_t(code[0]) | uint32_t(code[1]) << 8 | uint32_t(code[2]) << 16 | uint32_t(code[3]) << 24,
                     uint32_t(code[4]) | uint32_t(code[5]) << 8 | uint32_t(code[6]) << 16 | uint32_t(code[7]) << 24);
      if (j == 0) a.v_norms[slot] = nbits;
    } else {
      if (j == 0) a.k_norms[slot] = nbits;
      uint8_t* rec = a.k_data + slot * k_record_bytes(KFMT);
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

template <int KF, int VF>
void launch_one(const EncodeArgs& a, const AppendStarts& s, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((encode_append_kernel<KF, VF>), grid, dim3(256), 0, stream, a, s);
}

}  // namespace

hipError_t launch_encode_append(const EncodeArgs& a, const AppendStarts& starts, int nb, int max_tiles,
                                hipStream_t stream) {
  const dim3 grid(max_tiles, a.hkv, nb);
  if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo3) launch_one<kFmtTurbo3, kFmtTurbo3>(a, starts, grid, stream);
  else if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo4) launch_one<kFmtTurbo3, kFmtTurbo4>(a, starts, grid, stream);
  else if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo3) launch_one<kFmtTurbo4, kFmtTurbo3>(a, starts, grid, stream);
  else if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo4) launch_one<kFmtTurbo4, kFmtTurbo4>(a, starts, grid, stream);
  else if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo3) launch_one<kFmtF16, kFmtTurbo3>(a, starts, grid, stream);
  else if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo4) launch_one<kFmtF16, kFmtTurbo4>(a, starts, grid, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq
