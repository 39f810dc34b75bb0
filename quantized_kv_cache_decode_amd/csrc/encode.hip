// Encode + append of new K/V tokens (the cache update; mlxcel PR #369,
// "Change": the append is the only cache mutation).
//
// One workgroup per (32-token V tile touched by the append, KV head,
// sequence).  256 threads = 64 four-lane groups: groups 0..31 encode the K row
// of tile slot r = group, groups 32..63 the V row of slot r = group - 32.  A
// lane holds 32 consecutive dims (lane q: dims 32q..32q+31).
//
// Per group x (fp16 [128]):
//   norm  n = RNE_fp16(sqrt(sum x_i^2)) computed exactly: each |x_i| * 2^24 is
//         an integer below 2^40; its square is split in 20-bit halves whose sums
//         fit in u64, recombined in a u128, and the fp16 rounding decision is an
//         integer comparison (4 S vs q^2 (2k+1)^2).
//   y     = H (s * x) / sqrt(128): butterflies in binary64 (exact: fp16 terms
//         are multiples of 2^-24 below 2^16), then one IEEE division.
//   idx_i = #{j : y_i > n * beta_j}, beta_j = midpoints of adjacent fp16 codebook
//         entries (n * beta_j is exact in binary64).
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
  if (tid < levels(VFMT) - 1)
    beta_v[tid] = 0.5 * (double(half_bits_to_float(a.v_cb[tid])) + double(half_bits_to_float(a.v_cb[tid + 1])));
  if (KFMT != kFmtF16 && tid >= 32 && tid - 32 < levels(KFMT) - 1)
    beta_k[tid - 32] =
        0.5 * (double(half_bits_to_float(a.k_cb[tid - 32])) + double(half_bits_to_float(a.k_cb[tid - 31])));
  __syncthreads();

  const int grp = tid >> 2, q = tid & 3;
  const bool is_v = grp >= 32;
  const int r = grp & 31;
  const int t = tile * kTileTokens + r;
  const bool active = t >= lo && t < hi;
  const size_t row = size_t(b) * a.hkv + h;  // (sequence, KV head) row
  const size_t src_off = (row * a.t_new + size_t(t - start)) * kDim + 32 * q;
  const size_t slot = row * a.cap + t;

  if (active) {
    if (!is_v && KFMT == kFmtF16) {
      const uint4* src = reinterpret_cast<const uint4*>(a.k_new + src_off);
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_data) + slot * kDim + 32 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = src[i];
    } else {
      const uint16_t* src = (is_v ? a.v_new : a.k_new) + src_off;
      const float* sg = (is_v ? a.v_signs : a.k_signs) + 32 * q;
      double x[32];
      uint64_t sA = 0, sB = 0, sC = 0;
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 raw = s4[i];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int e = 8 * i + 2 * k2 + half;
            const double xv = double(half_bits_to_float(uint16_t(w[k2] >> (16 * half))));
            const uint64_t m = uint64_t(fabs(xv) * 16777216.0);  // exact integer < 2^40
            const uint64_t mh = m >> 20, ml = m & 0xfffffull;
            sA += mh * mh;
            sB += mh * ml;
            sC += ml * ml;
            x[e] = xv * double(sg[e]);
          }
        }
      }
      // fold the four lanes' partial sums
#pragma unroll
      for (int m = 1; m < 4; m <<= 1) {
        sA += __shfl_xor(sA, m, 4);
        sB += __shfl_xor(sB, m, 4);
        sC += __shfl_xor(sC, m, 4);
      }
      // Walsh-Hadamard in binary64: in-lane bits 0..4, cross-lane bits 5..6
#pragma unroll
      for (int hh = 1; hh < 32; hh <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          if (!(e & hh)) {
            const double u = x[e], v = x[e + hh];
            x[e] = u + v;
            x[e + hh] = u - v;
          }
        }
      }
#pragma unroll
      for (int m = 1; m < 4; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const double o = __shfl_xor(x[e], m, 4);
          x[e] = (q & m) ? (o - x[e]) : (x[e] + o);
        }
      }
      const uint16_t nbits = exact_norm_fp16(sA, sB, sC);
      const double nd = double(half_bits_to_float(nbits));
      const double* beta = is_v ? beta_v : beta_k;
      const int nthr = (is_v ? levels(VFMT) : levels(KFMT)) - 1;
      uint8_t code[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const double y = x[e] / kSqrtD;
        int c = 0;
        for (int j = 0; j < nthr; ++j) c += (y > nd * beta[j]) ? 1 : 0;
        code[e] = uint8_t(c);
      }
      if (is_v) {
#pragma unroll
        for (int e = 0; e < 32; ++e) vcodes[r][32 * q + e] = code[e];
        if (q == 0) a.v_norms[slot] = nbits;
      } else {
        if (q == 0) a.k_norms[slot] = nbits;
        uint8_t* rec = a.k_data + slot * k_record_bytes(KFMT);
        if (KFMT == kFmtTurbo3) {
          uint32_t w[3];
          sub3_pack(code, w);
          uint32_t* dst = reinterpret_cast<uint32_t*>(rec + 12 * q);
          dst[0] = w[0];
          dst[1] = w[1];
          dst[2] = w[2];
        } else {
          uint4 w;
          w.x = oct4_pack(code);
          w.y = oct4_pack(code + 8);
          w.z = oct4_pack(code + 16);
          w.w = oct4_pack(code + 24);
          *reinterpret_cast<uint4*>(rec + 16 * q) = w;
        }
      }
    }
  }
  __syncthreads();

  // V tile chunks: one thread per chunk c = 16 g + n (dims 8n..8n+7, slots r(g, i)).
  if (tid < 64) {
    const int g = tid >> 4, n = tid & 15;
    uint8_t* chunk = a.v_data + (row * (a.cap / kTileTokens) + tile) * v_tile_bytes(VFMT) + tid * v_chunk_bytes(VFMT);
    uint8_t el[64];
    const bool whole = lo == tile * kTileTokens && hi == tile * kTileTokens + kTileTokens;
    if (!whole) {
      if (VFMT == kFmtTurbo3) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(chunk);
        uint32_t w0[3] = {w[0], w[1], w[2]}, w1[3] = {w[3], w[4], w[5]};
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          el[e] = uint8_t(sub3_get(w0, e));
          el[32 + e] = uint8_t(sub3_get(w1, e));
        }
      } else {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(chunk);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const uint32_t word = w[nb];
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
    if (VFMT == kFmtTurbo3) {
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
