// Encode + append of new K/V tokens (the cache update; mlxcel PR #369,
// "Change": the append is the only cache mutation).  The codec arithmetic is in
// tq_encode.h.
//
// encode_append_kernel (any number of rows): one workgroup per (32-token V tile
// touched by the append, KV head, sequence).  256 threads = 16 groups of 16
// lanes; each group encodes one K or V row of a new token of the tile (lane j
// holds dims 8j..8j+7).  K records are written piece by piece into their 16-token
// blocks; V codes are staged in LDS and written as whole V-tile chunk pieces by one
// thread per chunk, merging with the words of tokens already in the tile.  F16 K
// rows are copied unchanged.
//
// append_one_kernel (one new row per sequence at most): a work group of two waves per
// (sequence, KV head), wave 0 the K row and wave 1 the V row, each a quantised row
// over all 64 lanes (two elements per lane, the wave-wide encoder; fp16 rows are
// copied by 16 lanes); every load is issued up front (one memory round trip, no
// barrier).
#include "tq_encode.h"

namespace tq {
namespace {

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
  uint8_t* vtile = a.v_data + (row * (a.cap / kTileTokens) + tile) * v_tile_bytes(VFMT);
  constexpr int kChunkWords = VFMT == kFmtF16 ? 1 : v_chunk_bytes(VFMT) / 4;  // (F16 V: rows stored directly)
  uint32_t old[kChunkWords];
#pragma unroll
  for (int i = 0; i < kChunkWords; ++i) old[i] = 0;
  if (VFMT != kFmtF16 && tid < 64 && !whole) {
#pragma unroll
    for (int i = 0; i < kChunkWords; ++i)
      old[i] = *reinterpret_cast<const uint32_t*>(vtile + v_chunk_byte_offset(VFMT, tid & 63, 4 * i));
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
    if (is_v && VFMT == kFmtF16) {
      store_f16_v_row(a, row, t, *reinterpret_cast<const uint4*>(a.v_new + src_off), j);
    } else if (is_v) {
      constexpr int VQ = VFMT == kFmtF16 ? kFmtTurbo3 : VFMT;  // (F16 V handled above)
      double beta[levels(VQ) - 1];
      load_row_and_signs(a.v_new + src_off, a.v_signs, j, w4, sg);
      load_thresholds<VQ>(a.v_cb, beta);
      const uint16_t nbits = encode_row<VQ, true>(w4, sg, beta, j, code);
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
      const uint16_t nbits = encode_row<KQ, true>(w4, sg, beta, j, code);
      if (j == 0) a.k_norms[slot] = nbits;
      store_k_record<KQ>(a.k_data + row * a.cap * k_record_bytes(KQ), t, code, j);
    }
  }
  __syncthreads();

  // V tile chunks: one thread per chunk c = 16 g + n (dims 8n..8n+7, slots r(g, i)).
  if constexpr (VFMT != kFmtF16) if (tid < 64) {
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
      if (tt >= lo && tt < hi) {  // a new token: its 8 codes of dims 8n..8n+7 in one LDS read
        const uint2 c8 = *reinterpret_cast<const uint2*>(&vcodes[rr][8 * n]);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) el[8 * nb + i] = uint8_t((nb < 4 ? c8.x : c8.y) >> (8 * (nb & 3)));
      }
    }
    if constexpr (VFMT == kFmtTurbo3) {
      uint32_t w[6];
      sub3_pack(el, w);
      sub3_pack(el + 32, w + 3);
#pragma unroll
      for (int p = 0; p < 2; ++p) {  // two 12-byte pieces (one sub-block each)
        uint32_t* dst = reinterpret_cast<uint32_t*>(vtile + v_chunk_byte_offset(VFMT, tid, 12 * p));
        dst[0] = w[3 * p];
        dst[1] = w[3 * p + 1];
        dst[2] = w[3 * p + 2];
      }
    } else {
      uint32_t w[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) w[nb] = oct4_pack(el + 8 * nb);
      *reinterpret_cast<uint4*>(vtile + v_chunk_byte_offset(VFMT, tid, 0)) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(vtile + v_chunk_byte_offset(VFMT, tid, 16)) = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
  if (blockIdx.x == 0 && h == 0 && tid == 0) a.seq_lens[b] = end;
}

template <int KFMT, int VFMT>
__global__ __launch_bounds__(128) void append_one_kernel(EncodeArgs a, AppendStarts starts) {
  const int lane = threadIdx.x & 63;
  const bool is_v = threadIdx.x >= 64;
  const int i = blockIdx.x / a.hkv, h = blockIdx.x % a.hkv;
  if (starts.count[i] == 0) return;  // the whole work group
  const int b = a.b0 + i;
  const int t = starts.start[i];
  const size_t row = size_t(b) * a.hkv + h;
  const uint16_t* src = (is_v ? a.v_new : a.k_new) + row * a.t_new * kDim;  // token 0 of the new rows
  if (is_v) {
    if constexpr (VFMT == kFmtF16) {
      if (lane < 16) store_f16_v_row(a, row, t, *reinterpret_cast<const uint4*>(src + 8 * lane), lane);
    } else {
      WaveVInputs<VFMT> in;
      load_wave_v_inputs<VFMT>(a, row, t, src, lane, in);
      uint32_t code[2];
      append_v_row_wave<VFMT>(a, row, t, in, lane, code);
    }
  } else {
    if constexpr (KFMT == kFmtF16) {
      if (lane < 16) append_f16_k_row(a, row, t, src, lane);
    } else {
      WaveRowInputs<KFMT> in;
      load_wave_row_inputs<KFMT>(src, a.k_signs, a.k_cb, lane, in);
      uint32_t code[2];
      append_k_row_wave<KFMT>(a, row, t, in, lane, code);
    }
    if (h == 0 && lane == 0) a.seq_lens[b] = t + 1;
  }
}

template <int KF, int VF>
void launch_one(const EncodeArgs& a, const AppendStarts& s, int nb, int max_tiles, bool single,
                hipStream_t stream) {
  if (single)
    hipLaunchKernelGGL((append_one_kernel<KF, VF>), dim3(nb * a.hkv), dim3(128), 0, stream, a, s);
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
  else if (k == kFmtF16 && v == kFmtF16) launch_one<kFmtF16, kFmtF16>(a, starts, nb, max_tiles, single, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq
