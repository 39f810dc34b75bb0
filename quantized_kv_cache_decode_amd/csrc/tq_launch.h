// Host-side launchers of the libtqattn kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// ---- encode / append
constexpr int kAppendChunk = 256;  // sequences per encode launch (start offsets travel as kernel arguments)

struct EncodeArgs {
  int hkv, cap, kfmt, vfmt, t_new, b0;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_data;
  uint16_t* k_norms;
  uint8_t* v_data;
  uint16_t* v_norms;
  int32_t* seq_lens;
  const float* k_signs;
  const float* v_signs;
  const uint16_t* k_cb;
  const uint16_t* v_cb;
};

// Host lengths of the sequences of one launch (at most kAppendChunk of them; the
// host splits larger batches into several launches).
struct SeqLens {
  int32_t len[kAppendChunk];
};

struct AppendStarts {
  int32_t start[kAppendChunk];  // first slot written, per sequence of the launch
  int32_t count[kAppendChunk];  // rows appended, per sequence of the launch
};

hipError_t launch_encode_append(const EncodeArgs& a, const AppendStarts& starts, int nb, int max_tiles,
                                hipStream_t stream);

// ---- rotations
hipError_t launch_rotate_q(const void* q, bool q_fp32, bool rotate, const float* signs, float* q_rot, int rows,
                           hipStream_t stream);
hipError_t launch_inverse_rotate(const float* o_rot, bool rotate, const float* signs, uint16_t* out, int rows,
                                 hipStream_t stream);

// ---- decode
// Split plan: sequence b is cut into ceil(L_b / chunk) splits of `chunk` tokens
// (at most max_splits; the last split takes the remainder).  Each (b, kv head h)
// row owns `slots` = max_splits + 1 partial slots: slot s < max_splits holds split
// s, the last one the appended token's own partial in the decode step (where the
// token is appended and attended in one call).
struct DecodePlan {
  int chunk;
  int max_splits;
  int slots;
  int bandwidth_bound;  // >= 4M token-heads: long enough that HBM, not latency, sets the time
  int latency;          // a small call (the latency plan: about one split per compute unit)
};

struct DecodeArgs {
  int hkv, cap, kfmt, vfmt, group;
  float scale;
  DecodePlan plan;
  const uint8_t* k_data;
  const uint16_t* k_norms;
  const uint8_t* v_data;
  const uint16_t* v_norms;
  int b0;                   // first sequence of the launch (blockIdx z / y counts from it)
  int col0;                 // decode kernel grid: columns 0..col0-1 append the step's token (0 or 2)
  int appends_last;         // col0 = 2 and more work groups than compute units: the MFMA kernel
                            // takes its grid as every row's splits first, the append work groups last
  int split_append;         // decode step with col0 = 0: split 0 appends K and split 1 (split 0 when
                            // max_splits = 1) appends V, each before its own split
  const uint16_t* k_cb;
  const uint16_t* v_cb;
  const float* q_rot;       // [B][Hq][128] fp32 in K's basis (the reference kernel's input)
  const void* q_in;         // [B][Hq][128] q as the MFMA kernel reads it (fp32 or fp16 bits)
  int q_fp32;               // q_in is fp32 (else fp16 bits)
  int q_rotate;             // q_in goes through H(s_K * q)/sqrt(128) in-kernel (else it is in K's basis)
  float v_skip_log2;        // sparse V: log2 of the weight threshold, -inf when off
  float k_skip_log2;        // sparse K: log2 of the weight threshold, -inf when off (always off for F16 K)
  int v_rotated;            // V is stored in its rotated basis (the output is taken back); 0 for fp16 V
  int q_len;                // query positions per head (>= 1): a causal chunk of the last q_len tokens;
                            // `group` then counts (head, position) columns, head-major
  const float* k_signs;
  const float* v_signs;
  float* part_o;            // [B*Hkv*slots][group][128]   unnormalised sum_t 2^(z_t - m) v_t
  float* part_ml;           // [B*Hkv*slots][group][2]     m (log2 units: z = scale*log2(e)*q.k), l
  float* out_rot;           // [B][Hq][128] fp32 in V's basis, or NULL when `out` is written
  uint16_t* out;            // [B][Hq][128] fp16 bits in the original basis, or NULL
  int step;                 // decode step: the appended token has its own partial slot (app is set)
  EncodeArgs app;           // decode step: the one-token append (app.k_new == NULL otherwise)
};

inline __host__ __device__ size_t partial_index(const DecodeArgs& a, size_t row, int slot, int g) {
  return (row * a.plan.slots + slot) * a.group + g;
}

// Each launch covers sequences a.b0 .. a.b0 + nb - 1 (nb <= kAppendChunk) with
// their visible lengths in `lens` (the decode step: the lengths before the append).
hipError_t launch_decode_reference(const DecodeArgs& a, const SeqLens& lens, int nb, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, const SeqLens& lens, int nb, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs& a, const SeqLens& lens, int nb, hipStream_t stream);

// ---- measurement aid: plain streaming read (one XOR checksum word per work group)
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sums, int blocks, hipStream_t stream);

}  // namespace tq
