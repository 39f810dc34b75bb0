/*
 * libtqattn — single-token decode attention over a KV cache compressed with a
 * rotated scalar codec, for AMD Instinct MI355X (gfx950).
 *
 * Codec (per 128-element head-dim group of one token and one KV head):
 *   n   = fp16 L2 norm of the group (round to nearest even, saturating at 65504);
 *   y   = H (s * x) / sqrt(128): Rademacher sign flip s, then orthonormal
 *         Walsh-Hadamard H (natural Sylvester order);
 *   idx = nearest fp16 codebook entry to y / n: 8 entries ("turbo3", 3 bits)
 *         or 16 entries ("turbo4", 4 bits);
 *   reconstruction x_hat = s * H (n * c[idx]) / sqrt(128).
 * The pages this follows: turboquant_plus "SMEM Pre-Dequant Experiment"
 * (section "What Would Actually Work", item 1: dequant is a table entry at the
 * index times the group norm) and mlxcel PR #369 "route Turbo4Asym decode
 * through dequant-SDPA" (section "Change": codes live in the WHT-rotated basis;
 * fp16 K + 4-bit V is the asymmetric mode; attention runs in V's rotated basis
 * and only the [B, Hq, D] output is inverse-rotated, by
 * rotate(SDPA(q,k,v)) == SDPA(q,k,rotate(v))).
 *
 * Conventions shared by every call:
 *   - Every data pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state between calls (apart from the
 *     thread-local error string).
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     enqueued on it; nothing synchronises.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-OK status means nothing was launched.  TQ_EHIP means a launch
 *     failed; tq_last_error() describes the last non-OK status of the calling
 *     thread.
 *   - Query head h attends KV head h / (num_q_heads / num_kv_heads)
 *     (contiguous GQA groups).  Group sizes 1..16 are supported.
 *   - Only tq_encode_append and tq_decode_step write the cache; the other
 *     calls read it.
 *
 * Byte layouts (this library's own; the pages print none):
 *   turbo4 octet word: 8 codes in one little-endian u32; code e (0..3) in bits
 *     8e..8e+3, code e (4..7) in bits 8(e-4)+4..8(e-4)+7; each field is
 *     sign-magnitude (bit 3 set for the 8 negative centroids, bits 0..2 the
 *     magnitude rank, 0 = smallest |c|).
 *   turbo3 sub-block: 32 three-bit ascending indices c[0..31] in 3 u32 words
 *     A, B, C; for j = 0..3:
 *       A[8j..8j+2]=c[j]    A[8j+3..8j+5]=c[4+j]  A[8j+6..8j+7]=c[24+j]&3
 *       B[8j..8j+2]=c[8+j]  B[8j+3..8j+5]=c[12+j] B[8j+6..8j+7]=c[28+j]&3
 *       C[8j..8j+2]=c[16+j] C[8j+3..8j+5]=c[20+j] C[8j+6]=c[24+j]>>2
 *       C[8j+7]=c[28+j]>>2
 *   K record: turbo3 48 bytes = 4 sub-blocks (dims 32q..32q+31); turbo4 64
 *     bytes = 16 octet words (dims 8w..8w+7).  Both are stored in blocks of 16
 *     tokens, as pieces, so that the lanes reading the same piece of a block's
 *     tokens read contiguous bytes: turbo4 piece p (words 4p..4p+3) of token
 *     16b + i at byte 1024 b + 256 p + 16 i of its row; turbo3 piece q (sub-block
 *     q, 12 bytes) of token 16b + i at byte 768 b + 384 (q % 2) + 192 (q / 2) +
 *     12 i (pieces 0 and 2 of the block's 16 tokens fill bytes 0..383 of the
 *     block, pieces 1 and 3 bytes 384..767).
 *   V tile (32 tokens, token-tiled): 64 chunks; chunk 16g+n holds dims
 *     8n..8n+7 of the 8 tokens in tile slots r = 16(i/4) + 4g + (i%4),
 *     i = 0..7; chunk element 8*nb + i is dim 8n+nb of token slot r(g, i).
 *     turbo3 chunk = 2 sub-blocks (24 bytes), sub-block p of chunk c at tile
 *     byte 768 p + 12 c; turbo4 chunk =
 *     8 octet words, word nb = elements 8nb..8nb+7 (32 bytes), as two 16-byte
 *     pieces: piece p (words 4p..4p+3) of chunk c at tile byte 1024 p + 16 c;
 *     F16 chunk = the 64 elements as fp16 values (128 bytes) at tile byte
 *     128 c.  Tile: 1536 / 2048 / 8192 bytes.
 */
#ifndef TQATTN_H
#define TQATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* bad pointer, shape or value */
  TQ_EUNSUPPORTED = 2,  /* head_dim != 128, group size > 16, unknown format */
  TQ_ECAPACITY = 3,     /* an append would pass `capacity`, or a length exceeds it */
  TQ_EWORKSPACE = 4,    /* workspace smaller than tq_decode_workspace_size() */
  TQ_EHIP = 5           /* a HIP launch failed */
} tq_status;

typedef enum {
  TQ_FMT_F16 = 0,       /* raw half precision: K (asymmetric mode), or K and V together
                           (the uncompressed cache the pages compare every mode against) */
  TQ_FMT_TURBO3 = 3,    /* 3-bit codes + fp16 norm, 50 bytes per 128-group */
  TQ_FMT_TURBO4 = 4     /* 4-bit codes + fp16 norm, 66 bytes per 128-group */
} tq_format;

/* The cache of one attention layer.  All pointers are device memory.
 *   k_data   TURBO3/TURBO4: u8 [B][Hkv][capacity][48 | 64] K records;
 *            F16: fp16 [B][Hkv][capacity][128].
 *   k_norms  fp16 bits [B][Hkv][capacity]; NULL when k_format == TQ_FMT_F16.
 *   v_data   u8 [B][Hkv][capacity/32][1536 | 2048] V tiles.
 *   v_norms  fp16 bits [B][Hkv][capacity]; NULL when v_format == TQ_FMT_F16
 *            (allowed only with k_format == TQ_FMT_F16; V is then stored
 *            unrotated and v_signs / v_codebook are unused).
 *   seq_lens int32 [B]: visible tokens per sequence (the cache "offset"),
 *            kept up to date by tq_encode_append and tq_decode_step for callers
 *            that read it on the device; the decode calls take the lengths from
 *            the host.
 *   k_signs, v_signs   float [128] of +1/-1 (k_signs unused for F16 K).
 *   k_codebook, v_codebook   fp16 bits, ascending, 8 (turbo3) or 16 (turbo4)
 *            entries, symmetric (c[i] = -c[n-1-i]); k_codebook unused for F16 K.
 *   v_skip_threshold   sparse V, in [0, 1]; 0 turns it off.  The MFMA decode
 *            kernel skips the V dequant and the p.v products of a 32-token V
 *            tile for the query heads of a KV head when every weight of the tile,
 *            relative to the running maximum (so also relative to the final one),
 *            is below the threshold.  The score pass and the softmax sum still
 *            see every token: the result differs from exact attention by at most
 *            the skipped weights times |v|.  At 1e-6 the skipped weights sit below
 *            fp16 round-off (mlxcel PR #369, commit "docs(cache): add ADR 0002 on
 *            Turbo KV split-dequant vs fused (sparse-V study)"; turboquant_plus
 *            "SMEM Pre-Dequant Experiment", idea 2 "Sparse K attention", names the
 *            V-side skip).  The VALU reference variant (tq_decode_attention_variant
 *            1) ignores it and is exact.
 *   k_skip_threshold   sparse K, in [0, 1]; 0 turns it off (turboquant_plus
 *            "SMEM Pre-Dequant Experiment", idea 2 "Sparse K attention": skip the
 *            K work of positions whose contribution is negligible, judged from the
 *            norm alone).  The MFMA decode kernel skips a whole iteration (32 to 128
 *            tokens: K dequant, scores, softmax and values) when, for every query
 *            head of the KV head, the Cauchy-Schwarz bound
 *            scale * |q| * n * sqrt(128) * max|c| on the scores of the iteration's
 *            tokens (n their largest stored K norm) is below that head's running
 *            maximum score + ln(threshold): every skipped token's weight is below
 *            the threshold relative to a maximum already seen.  Unlike sparse V the
 *            skipped tokens also leave the softmax sum, so the result differs from
 *            exact attention by at most (D |o| + sum of the skipped weights times
 *            |v|) / (1 - D), D the skipped weight.  The words of a skipped iteration
 *            are still read (bandwidth is not saved, VALU and MFMA work is).  It has
 *            no effect with F16 K (no stored norms) or in the VALU reference
 *            variant; the first iteration of every split is never skipped.
 * capacity must be a positive multiple of 32 and at most TQ_MAX_CAPACITY (2^24
 * tokens: the decode kernel addresses one (sequence, KV head) row of quantised
 * K records, V tiles and norms with 32-bit byte offsets); head_dim must be 128.
 * The decode kernels read whole 32-token tiles and mask the slots at or past a
 * sequence's length, whose V norms are multiplied by an exact zero weight: they
 * must hold finite fp16 values (zero-fill the arrays when allocating them). */
#define TQ_MAX_CAPACITY (1 << 24)

typedef struct tq_cache {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t k_format;
  int32_t v_format;
  void* k_data;
  uint16_t* k_norms;
  void* v_data;
  uint16_t* v_norms;
  int32_t* seq_lens;
  const float* k_signs;
  const float* v_signs;
  const uint16_t* k_codebook;
  const uint16_t* v_codebook;
  float v_skip_threshold;
  float k_skip_threshold;
} tq_cache;

/* Encode new tokens and append them to each sequence
 * (mlxcel PR #369, "Change": the cache update is the only mutation).
 *   seq_lens_host  HOST int32 [B]: current visible length of each sequence.
 *   k_new, v_new   device fp16 [B][Hkv][t_new][128] (token rows before encoding).
 *   counts_host    HOST int32 [B] or NULL: sequence b appends its first
 *                  n_b = counts_host[b] rows (0 <= n_b <= t_new); NULL means
 *                  n_b = t_new for every sequence (the decode step's append).
 * Rows go to slots seq_lens_host[b] .. +n_b-1 and the kernel sets
 * cache->seq_lens[b] = seq_lens_host[b] + n_b.
 * Symmetric K and every V: rotate, take the fp16 norm, pick the nearest
 * centroid, pack (layouts above); F16 K rows are copied unchanged.  Norm and
 * decisions are computed exactly (integer sum of squares, binary64 rotation).
 * Sequences with n_b == 0 are left untouched.  Errors: TQ_ECAPACITY if
 * seq_lens_host[b] + n_b > capacity for some b; TQ_EINVAL for NULL pointers,
 * negative lengths or a count outside [0, t_new]. */
tq_status tq_encode_append(const tq_cache* cache, const int32_t* seq_lens_host,
                           const void* k_new, const void* v_new, int32_t t_new,
                           const int32_t* counts_host, void* stream);

/* Rotate queries into K's codec basis: q_rot = H (s_K * q) / sqrt(128)
 * (mlxcel PR #369, "Change": symmetric modes rotate Q because K is stored
 * rotated; the asymmetric fp16-K mode needs no Q rotation, and then q_rot = q).
 *   q      device [B][num_q_heads][128], fp32 if q_is_fp32 else fp16 bits.
 *   q_rot  device fp32 [B][num_q_heads][128]. */
tq_status tq_rotate_q(const tq_cache* cache, const void* q, int32_t q_is_fp32,
                      int32_t num_q_heads, float* q_rot, void* stream);

/* Bytes of device workspace the decode calls need for these lengths: split-K
 * partials (fp32 o, m, l per split and query head, plus one slot per (sequence,
 * KV head) for tq_decode_step's new token).
 * seq_lens_host: HOST int32 [B].  Returns 0 on invalid arguments (see
 * tq_last_error). */
size_t tq_decode_workspace_size(const tq_cache* cache, int32_t num_q_heads,
                                const int32_t* seq_lens_host);

/* Decode attention of one new query token per sequence against every visible
 * token, in V's rotated basis (mlxcel PR #369, "Change"; output of the full
 * dequant-then-attend reference up to rounding, "Result"):
 *   out_rot[b,h] = sum_t softmax_t(scale * q_rot[b,h] . k_t) * (n_V,t * c_V[idx_V,t])
 * with k_t = n_K,t * c_K[idx_K,t] (symmetric) or the fp16 K row (F16).
 * Split-K over the context with a per-sequence split count, then a
 * log-sum-exp merge of the splits.
 *   seq_lens_host  HOST int32 [B]: the visible lengths to attend over (normally
 *                  the lengths cache->seq_lens holds).  They size the launch and
 *                  travel as kernel arguments; the decode calls never read
 *                  cache->seq_lens.
 *   q_rot          device fp32 [B][num_q_heads][128] (from tq_rotate_q).
 *   out_rot        device fp32 [B][num_q_heads][128]; a sequence of length 0
 *                  gives zeros.
 *   workspace      device, >= tq_decode_workspace_size() bytes; no initial
 *                  contents needed; reusable by later calls (not by two calls
 *                  in flight at the same time).
 * The cache is not modified. */
tq_status tq_decode_attention(const tq_cache* cache, const int32_t* seq_lens_host,
                              const float* q_rot, int32_t num_q_heads, float scale,
                              float* out_rot, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Same as tq_decode_attention with an explicit kernel variant, for A/B
 * comparison of kernel designs: 0 = the MFMA kernel (what every other decode
 * call runs), 1 = the plain VALU reference kernel (quantised V formats only,
 * else TQ_EUNSUPPORTED).  Other values give TQ_EINVAL. */
tq_status tq_decode_attention_variant(const tq_cache* cache, const int32_t* seq_lens_host,
                                      const float* q_rot, int32_t num_q_heads, float scale,
                                      float* out_rot, void* workspace, size_t workspace_bytes,
                                      int32_t variant, void* stream);

/* The three decode calls in one: tq_rotate_q, tq_decode_attention and
 * tq_inverse_rotate_out, with the query rotation done inside the decode kernel
 * and the inverse rotation inside the split merge (two kernels, no q_rot or
 * out_rot buffers; mlxcel PR #369, "Change": only the [B, Hq, D] output leaves
 * V's rotated basis).  The result has the same bits as the three separate calls.
 *   q    device [B][num_q_heads][128], fp32 if q_is_fp32 else fp16 bits,
 *        unrotated (rotated into K's basis here unless k_format is F16).
 *   out  device fp16 bits [B][num_q_heads][128], original basis; a sequence of
 *        length 0 gives (signed) zeros.
 * seq_lens_host, scale, workspace and the errors are as for tq_decode_attention
 * (same workspace size).  Always the MFMA kernel. */
tq_status tq_decode_attention_fused(const tq_cache* cache, const int32_t* seq_lens_host,
                                    const void* q, int32_t q_is_fp32, int32_t num_q_heads,
                                    float scale, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Decode attention of a chunk of q_len query positions per sequence (speculative
 * verification, chunked decode): the chunk's tokens are the last q_len of each
 * sequence, already appended with tq_encode_append, and are causal among
 * themselves -- position tau (0 <= tau < q_len) attends to the first
 * seq_lens_host[b] - q_len + 1 + tau tokens.  The pages' decode output is
 * [B, Hq, Tq, D] (mlxcel PR #369, "Change"); q_len = 1 is
 * tq_decode_attention_fused.  Each (query head, position) pair is one column of
 * its KV head's decode, so group * q_len must be <= 16 (TQ_EUNSUPPORTED
 * otherwise); rotations as in tq_decode_attention_fused.
 *   seq_lens_host  HOST int32 [B]: lengths including the chunk; each >= q_len.
 *   q     device [B][num_q_heads][q_len][128], fp32 if q_is_fp32 else fp16 bits.
 *   out   device fp16 bits [B][num_q_heads][q_len][128], original basis.
 *   workspace  >= tq_decode_workspace_size(cache, num_q_heads * q_len,
 *                  seq_lens_host) bytes.
 * Other errors as for tq_decode_attention.  Always the MFMA kernel. */
tq_status tq_decode_chunk_fused(const tq_cache* cache, const int32_t* seq_lens_host,
                                const void* q, int32_t q_is_fp32, int32_t num_q_heads,
                                int32_t q_len, float scale, uint16_t* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* One whole decode step: append one new token to every sequence and attend to
 * all visible tokens, the new one included -- tq_encode_append (t_new = 1)
 * followed by tq_decode_attention_fused on the grown cache, in two kernels.
 * The new token is encoded and written by two extra work groups per
 * (sequence, KV head) of the decode kernel (on bandwidth-bound calls, >= 4M
 * visible token-heads, by the row's first two splits before their own tokens,
 * so that the splits still fill the chip in one round), which also take the
 * token's own softmax partial (its score against every query head of the
 * group, weight 1, value its reconstructed V row); the regular splits cover
 * the older tokens in parallel and the split merge folds the extra partial in (mlxcel PR #369,
 * "Change": the append is the only cache mutation and the rotated-basis route
 * attends right after it).  Codes, norms and cache->seq_lens end up exactly as
 * after tq_encode_append; the output agrees with the two-call route up to
 * rounding (the new token's score is taken in fp32 rather than on the matrix
 * cores).
 *   seq_lens_host  HOST int32 [B]: lengths BEFORE the append (= cache->seq_lens);
 *                  each must be < capacity.
 *   k_new, v_new   device fp16 [B][Hkv][1][128], the new token's rows.
 *   q, q_is_fp32, out   as for tq_decode_attention_fused.
 *   workspace      >= tq_decode_workspace_size(cache, num_q_heads, seq_lens_host)
 *                  with the lengths before the append.
 * Errors as for tq_encode_append and tq_decode_attention.  Always the MFMA kernel. */
tq_status tq_decode_step(const tq_cache* cache, const int32_t* seq_lens_host,
                         const void* k_new, const void* v_new, const void* q,
                         int32_t q_is_fp32, int32_t num_q_heads, float scale,
                         uint16_t* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc -- and so
 * cannot hand in a workspace: tq_decode_step with the split partials kept in
 * a device array of the library's own, TQ_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * GPU, held from the first call on that GPU until the process ends.  Same
 * kernels, same plan, same output and cache contents as tq_decode_step.
 *   Arguments as for tq_decode_step, without the workspace.  `stream` must
 *   belong to the calling thread's current device.
 *   Calls whose partials need more than TQ_NOALLOC_SCRATCH_BYTES (what
 *   tq_decode_workspace_size returns) give TQ_EWORKSPACE before anything is
 *   enqueued.  No hipMalloc or hipFree is made; the first call on a device
 *   resolves the array's device address once (hipGetSymbolAddress), and a
 *   failure there gives TQ_EHIP.
 *   Every call on one GPU shares that GPU's array and leaves its partials
 *   there; nothing in it needs initial contents.  Calls that overlap on one
 *   GPU (several streams or threads at once) race on it: serialise them. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tq_status tq_decode_step_noalloc(const tq_cache* cache, const int32_t* seq_lens_host,
                                 const void* k_new, const void* v_new, const void* q,
                                 int32_t q_is_fp32, int32_t num_q_heads, float scale,
                                 uint16_t* out, void* stream);

/* Back to the original basis: out = s_V * H (out_rot) / sqrt(128), rounded to
 * nearest-even fp16 (mlxcel PR #369, "Change": only the small [B, Hq, D]
 * output is inverse-rotated).
 *   out_rot  device fp32 [B][num_q_heads][128];  out  device fp16 bits, same shape. */
tq_status tq_inverse_rotate_out(const tq_cache* cache, const float* out_rot,
                                int32_t num_q_heads, uint16_t* out, void* stream);

/* Measurement aid, not a step of the method: a plain streaming read of `bytes`
 * bytes of device memory at `src` (16-byte aligned; bytes a positive multiple
 * of 16), the practical HBM read ceiling that the decode kernel's achieved
 * bandwidth is compared with.  `blocks` work groups of 256 lanes (1..2^20) read
 * 16-byte words in a grid-stride loop; work group i writes the XOR of the words
 * it read to sums[i] (device uint32 [blocks]), so the XOR of all of sums is the
 * XOR of the buffer's 32-bit words.  Invalid arguments give TQ_EINVAL. */
tq_status tq_stream_read(const void* src, size_t bytes, uint32_t* sums, int32_t blocks, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* tq_last_error(void);

/* Library version string. */
const char* tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQATTN_H */
