// C ABI of libtqattn: argument validation, split planning and kernel launches.
// Everything is validated on the host before the first launch; see include/tqattn.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/tqattn.h"
#include "tq_device.h"
#include "tq_launch.h"

namespace {

thread_local char g_err[512] = "";

tq_status fail(tq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

tq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_turbo(int f) { return f == TQ_FMT_TURBO3 || f == TQ_FMT_TURBO4; }

tq_status check_cache(const tq_cache* c) {
  if (!c) return fail(TQ_EINVAL, "cache is NULL");
  if (c->head_dim != 128) return fail(TQ_EUNSUPPORTED, "head_dim %d: only 128 is supported", c->head_dim);
  if (c->batch <= 0 || c->num_kv_heads <= 0) return fail(TQ_EINVAL, "batch and num_kv_heads must be positive");
  if (c->capacity <= 0 || c->capacity % 32) return fail(TQ_EINVAL, "capacity %d must be a positive multiple of 32", c->capacity);
  if (c->capacity > TQ_MAX_CAPACITY)
    return fail(TQ_EINVAL, "capacity %d exceeds %d (a row's quantised K and V bytes must stay under 2^31)", c->capacity,
                TQ_MAX_CAPACITY);
  if (!is_turbo(c->k_format) && c->k_format != TQ_FMT_F16)
    return fail(TQ_EUNSUPPORTED, "k_format %d: must be F16, TURBO3 or TURBO4", c->k_format);
  if (!is_turbo(c->v_format) && !(c->v_format == TQ_FMT_F16 && c->k_format == TQ_FMT_F16))
    return fail(TQ_EUNSUPPORTED, "v_format %d: must be TURBO3 or TURBO4 (F16 only with F16 K)", c->v_format);
  if (!c->k_data || !c->v_data || !c->seq_lens) return fail(TQ_EINVAL, "NULL cache pointer");
  if (is_turbo(c->v_format) && (!c->v_norms || !c->v_signs || !c->v_codebook))
    return fail(TQ_EINVAL, "NULL V norm/sign/codebook pointer for a quantised V format");
  if (is_turbo(c->k_format) && (!c->k_norms || !c->k_signs || !c->k_codebook))
    return fail(TQ_EINVAL, "NULL K norm/sign/codebook pointer for a quantised K format");
  if (!(c->v_skip_threshold >= 0.f && c->v_skip_threshold <= 1.f))
    return fail(TQ_EINVAL, "v_skip_threshold %g outside [0, 1]", (double)c->v_skip_threshold);
  if (!(c->k_skip_threshold >= 0.f && c->k_skip_threshold <= 1.f))
    return fail(TQ_EINVAL, "k_skip_threshold %g outside [0, 1]", (double)c->k_skip_threshold);
  const long long slots = (long long)c->batch * c->num_kv_heads * c->capacity;
  if (slots * 128 > (1LL << 46)) return fail(TQ_EINVAL, "cache too large");
  return TQ_OK;
}

tq_status check_heads(const tq_cache* c, int32_t num_q_heads) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads)
    return fail(TQ_EINVAL, "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                c->num_kv_heads);
  if (num_q_heads / c->num_kv_heads > tq::kMaxGroup)
    return fail(TQ_EUNSUPPORTED, "group size %d > %d", num_q_heads / c->num_kv_heads, tq::kMaxGroup);
  return TQ_OK;
}

tq_status check_lengths(const tq_cache* c, const int32_t* lens, int32_t extra) {
  if (!lens) return fail(TQ_EINVAL, "seq_lens_host is NULL");
  for (int b = 0; b < c->batch; ++b) {
    if (lens[b] < 0) return fail(TQ_EINVAL, "seq_lens_host[%d] = %d is negative", b, lens[b]);
    if ((long long)lens[b] + extra > c->capacity)
      return fail(TQ_ECAPACITY, "sequence %d: %d + %d tokens exceed capacity %d", b, lens[b], extra, c->capacity);
  }
  return TQ_OK;
}

#ifndef TQ_PLAN_MIN_CHUNK
#define TQ_PLAN_MIN_CHUNK 128   // shortest split, tokens (a multiple of 64)
#endif
#ifndef TQ_PLAN_ITEMS_SMALL_GROUP
#define TQ_PLAN_ITEMS_SMALL_GROUP 2048   // work items aimed for, group size <= 4
#endif
#ifndef TQ_PLAN_ITEMS
#define TQ_PLAN_ITEMS 4096               // work items aimed for, group size > 4
#endif
#ifndef TQ_PLAN_LATENCY_ITEMS
#define TQ_PLAN_LATENCY_ITEMS 256            // small calls: work items aimed for (one per compute unit)
#endif
#ifndef TQ_PLAN_LATENCY_BYTES
#define TQ_PLAN_LATENCY_BYTES (32LL << 20)   // small calls: packed K + V bytes up to this
#endif
#ifndef TQ_PLAN_FLOOR
#define TQ_PLAN_FLOOR 200   // bandwidth-bound calls: chunk >= TQ_PLAN_FLOOR * group tokens
#endif
#ifndef TQ_PLAN_SHARE_BYTES
#define TQ_PLAN_SHARE_BYTES (32LL << 10)     // small calls: a split streaming more than this keeps a unit to itself
#endif

// packed bytes per (token, KV head) of one side
long long token_bytes(int fmt) { return fmt == TQ_FMT_TURBO3 ? 50 : fmt == TQ_FMT_TURBO4 ? 66 : 256; }

// Split plan shared by the workspace query and the launch.  A fixed number of
// work items over the chip, each a multiple of 64 tokens: 2048 (2 waves per SIMD,
// all the decode kernel's register budget allows for group sizes <= 4) or 4096
// (its leaner variants for larger groups fit 3-4 waves per SIMD, and smaller items
// also even out ragged lengths).  Once the call is bandwidth-bound (>= 4M
// token-heads) the chunk is also kept long enough that the partials (G x 130
// floats, written then read) stay under ~4% of the packed bytes of the chunk.
// Small calls (up to 32 MB of packed K and V) aim at one split per compute unit; when a
// split streams more than 32 KB (fp16 K), the decode step's two append work groups per row
// are counted in, so that no two splits share a compute unit (two streaming waves on one
// unit share its load pipe and both finish late: the fp16-K 16K step's slowest splits, on
// its 257th-264th work groups and the units they share, ended 2 us after the median one).
tq::DecodePlan make_plan(const tq_cache* c, const int32_t* lens, int group) {
  long long total = 0;
  int lmax = 0;
  for (int b = 0; b < c->batch; ++b) {
    total += (long long)lens[b] * c->num_kv_heads;
    lmax = std::max(lmax, (int)lens[b]);
  }
  const long long items = group <= 4 ? TQ_PLAN_ITEMS_SMALL_GROUP : TQ_PLAN_ITEMS;
  long long chunk = (total + items - 1) / items;
  const bool bandwidth_bound = total >= (4LL << 20);
  if (bandwidth_bound) chunk = std::max(chunk, (long long)TQ_PLAN_FLOOR * group);
  // small calls (a few tens of MB): about one work group per compute unit -- more
  // splits only add waves that compete for the same units' load pipes
  const long long bytes = total * (token_bytes(c->k_format) + token_bytes(c->v_format));
  const long long tok_bytes = token_bytes(c->k_format) + token_bytes(c->v_format);
  auto round_chunk = [](long long ch) { return std::max((long long)TQ_PLAN_MIN_CHUNK, (ch + 63) / 64 * 64); };
  const bool latency = !bandwidth_bound && bytes <= TQ_PLAN_LATENCY_BYTES;
  if (latency) {
    chunk = std::max(chunk, (total + TQ_PLAN_LATENCY_ITEMS - 1) / TQ_PLAN_LATENCY_ITEMS);
    const long long rows = (long long)c->batch * c->num_kv_heads;
    const long long items = TQ_PLAN_LATENCY_ITEMS - 2 * rows;
    if (round_chunk(chunk) * tok_bytes > TQ_PLAN_SHARE_BYTES && items >= TQ_PLAN_LATENCY_ITEMS / 2)
      chunk = std::max(chunk, (total + items - 1) / items);
  }
  chunk = round_chunk(chunk);
  tq::DecodePlan p;
  p.chunk = (int)chunk;
  p.max_splits = std::max(1, (int)((lmax + chunk - 1) / chunk));
  p.slots = p.max_splits + 1;
  p.bandwidth_bound = bandwidth_bound;
  p.latency = latency;
  return p;
}

// Workspace: split partials o [items][G][128] and (m, l) [items][G][2] (fp32),
// items = B * Hkv * slots.
size_t partial_floats(const tq_cache* c, int32_t num_q_heads, const tq::DecodePlan& p) {
  return (size_t)c->batch * c->num_kv_heads * p.slots * (num_q_heads / c->num_kv_heads);
}

size_t workspace_bytes(const tq_cache* c, int32_t num_q_heads, const tq::DecodePlan& p) {
  return partial_floats(c, num_q_heads, p) * (128 + 2) * sizeof(float);
}

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_err; }

const char* tq_version(void) { return "libtqattn 0.1 (gfx950)"; }

tq_status tq_encode_append(const tq_cache* cache, const int32_t* seq_lens_host, const void* k_new,
                           const void* v_new, int32_t t_new, const int32_t* counts_host, void* stream) {
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if (t_new < 0) return fail(TQ_EINVAL, "t_new %d is negative", t_new);
  if ((st = check_lengths(cache, seq_lens_host, 0)) != TQ_OK) return st;
  for (int b = 0; b < cache->batch; ++b) {
    const int n = counts_host ? counts_host[b] : t_new;
    if (n < 0 || n > t_new) return fail(TQ_EINVAL, "counts_host[%d] = %d outside [0, %d]", b, n, t_new);
    if ((long long)seq_lens_host[b] + n > cache->capacity)
      return fail(TQ_ECAPACITY, "sequence %d: %d + %d tokens exceed capacity %d", b, seq_lens_host[b], n,
                  cache->capacity);
  }
  if (t_new == 0) return TQ_OK;
  if (!k_new || !v_new) return fail(TQ_EINVAL, "k_new / v_new is NULL");
  tq::EncodeArgs a;
  a.hkv = cache->num_kv_heads;
  a.cap = cache->capacity;
  a.kfmt = cache->k_format;
  a.vfmt = cache->v_format;
  a.t_new = t_new;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_data = static_cast<uint8_t*>(cache->k_data);
  a.k_norms = cache->k_norms;
  a.v_data = static_cast<uint8_t*>(cache->v_data);
  a.v_norms = cache->v_norms;
  a.seq_lens = cache->seq_lens;
  a.k_signs = cache->k_signs;
  a.v_signs = cache->v_signs;
  a.k_cb = cache->k_codebook;
  a.v_cb = cache->v_codebook;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < cache->batch; b0 += tq::kAppendChunk) {
    const int nb = std::min(tq::kAppendChunk, cache->batch - b0);
    tq::AppendStarts starts;
    memset(&starts, 0, sizeof(starts));
    int max_tiles = 0;
    for (int i = 0; i < nb; ++i) {
      const int st0 = seq_lens_host[b0 + i];
      const int n = counts_host ? counts_host[b0 + i] : t_new;
      starts.start[i] = st0;
      starts.count[i] = n;
      if (n > 0) max_tiles = std::max(max_tiles, (st0 + n - 1) / 32 - st0 / 32 + 1);
    }
    if (max_tiles == 0) continue;
    a.b0 = b0;
    st = hip_status(tq::launch_encode_append(a, starts, nb, max_tiles, s), "encode_append launch");
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

tq_status tq_rotate_q(const tq_cache* cache, const void* q, int32_t q_is_fp32, int32_t num_q_heads,
                      float* q_rot, void* stream) {
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != TQ_OK) return st;
  if (!q || !q_rot) return fail(TQ_EINVAL, "q / q_rot is NULL");
  const bool rotate = cache->k_format != TQ_FMT_F16;
  return hip_status(tq::launch_rotate_q(q, q_is_fp32 != 0, rotate, cache->k_signs, q_rot,
                                        cache->batch * num_q_heads, static_cast<hipStream_t>(stream)),
                    "rotate_q launch");
}

size_t tq_decode_workspace_size(const tq_cache* cache, int32_t num_q_heads, const int32_t* seq_lens_host) {
  if (check_cache(cache) != TQ_OK || check_heads(cache, num_q_heads) != TQ_OK ||
      check_lengths(cache, seq_lens_host, 0) != TQ_OK)
    return 0;
  return workspace_bytes(cache, num_q_heads, make_plan(cache, seq_lens_host, num_q_heads / cache->num_kv_heads));
}

namespace {

// Validation and argument set-up shared by the decode entry points.
tq_status decode_setup(const tq_cache* cache, const int32_t* seq_lens_host, int32_t num_q_heads, float scale,
                       void* workspace, size_t ws_bytes, tq::DecodeArgs& a) {
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != TQ_OK) return st;
  if ((st = check_lengths(cache, seq_lens_host, 0)) != TQ_OK) return st;
  const tq::DecodePlan plan = make_plan(cache, seq_lens_host, num_q_heads / cache->num_kv_heads);
  const size_t need = workspace_bytes(cache, num_q_heads, plan);
  if (!workspace || ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  memset(&a, 0, sizeof(a));
  a.hkv = cache->num_kv_heads;
  a.cap = cache->capacity;
  a.kfmt = cache->k_format;
  a.vfmt = cache->v_format;
  a.group = num_q_heads / cache->num_kv_heads;
  a.scale = scale;
  a.plan = plan;
  a.k_data = static_cast<const uint8_t*>(cache->k_data);
  a.k_norms = cache->k_norms;
  a.v_data = static_cast<const uint8_t*>(cache->v_data);
  a.v_norms = cache->v_norms;
  a.k_cb = cache->k_codebook;
  a.v_cb = cache->v_codebook;
  a.k_signs = cache->k_signs;  // read only for a quantised K format
  a.v_signs = cache->v_signs;  // read only for a quantised V format
  a.v_rotated = cache->v_format != TQ_FMT_F16;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + partial_floats(cache, num_q_heads, plan) * 128;
  a.col0 = 0;
  a.appends_last = 0;
  a.split_append = 0;
  a.v_skip_log2 = cache->v_skip_threshold > 0.f ? std::log2(cache->v_skip_threshold) : -INFINITY;
  // the K-side bound needs the stored norms of a quantised K format
  a.k_skip_log2 = cache->k_skip_threshold > 0.f && is_turbo(cache->k_format) ? std::log2(cache->k_skip_threshold)
                                                                            : -INFINITY;
  a.q_len = 1;
  return TQ_OK;
}

// Compute units of the current device (cached per device).
int compute_units() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Launch the decode kernel (variant 1: the VALU reference) and the split merge for
// every group of up to kAppendChunk sequences, with their host lengths as kernel
// arguments (the kernels never wait on a length read from memory).
tq_status launch_decode_and_merge(const tq_cache* cache, const int32_t* seq_lens_host, tq::DecodeArgs& a,
                                  int variant, hipStream_t s) {
  for (int b0 = 0; b0 < cache->batch; b0 += tq::kAppendChunk) {
    const int nb = std::min(tq::kAppendChunk, cache->batch - b0);
    tq::SeqLens lens;
    memset(&lens, 0, sizeof(lens));
    for (int i = 0; i < nb; ++i) lens.len[i] = seq_lens_host[b0 + i];
    a.b0 = b0;
    a.app.b0 = b0;
    tq_status st;
    // Decode step: on latency-bound calls the token gets two work groups of its own
    // (grid columns 0 and 1), which run beside the splits; on bandwidth-bound calls
    // the splits fill the chip in one round and the row's first two splits append it.
    const bool step = a.app.k_new != nullptr;
    a.step = step;
    a.col0 = step && !a.plan.bandwidth_bound ? 2 : 0;
    a.split_append = step && a.plan.bandwidth_bound;
    a.appends_last = variant != 1 && a.col0 == 2 &&
                     (long long)nb * cache->num_kv_heads * (a.col0 + a.plan.max_splits) > compute_units();
    const hipError_t e = variant == 1 ? tq::launch_decode_reference(a, lens, nb, s)
                                      : tq::launch_decode_mfma(a, lens, nb, s);
    if ((st = hip_status(e, "decode launch")) != TQ_OK) return st;
    if ((st = hip_status(tq::launch_combine(a, lens, nb, s), "combine launch")) != TQ_OK) return st;
  }
  return TQ_OK;
}

}  // namespace

tq_status tq_decode_attention_variant(const tq_cache* cache, const int32_t* seq_lens_host, const float* q_rot,
                                      int32_t num_q_heads, float scale, float* out_rot, void* workspace,
                                      size_t ws_bytes, int32_t variant, void* stream) {
  tq::DecodeArgs a;
  tq_status st = decode_setup(cache, seq_lens_host, num_q_heads, scale, workspace, ws_bytes, a);
  if (st != TQ_OK) return st;
  if (!q_rot || !out_rot) return fail(TQ_EINVAL, "q_rot / out_rot is NULL");
  if (variant < 0 || variant > 1) return fail(TQ_EINVAL, "unknown decode variant %d", variant);
  if (variant == 1 && cache->v_format == TQ_FMT_F16)
    return fail(TQ_EUNSUPPORTED, "the VALU reference variant reads quantised V only");
  a.q_rot = q_rot;  // (the reference kernel reads it; the MFMA kernel stages it as fp32 q, unrotated)
  a.q_in = q_rot;
  a.q_fp32 = 1;
  a.q_rotate = 0;
  a.out_rot = out_rot;
  // variant 0 (default) is the MFMA kernel, 1 the plain VALU reference kernel;
  // both are followed by the log-sum-exp merge of their splits
  return launch_decode_and_merge(cache, seq_lens_host, a, variant, static_cast<hipStream_t>(stream));
}

tq_status tq_decode_attention_fused(const tq_cache* cache, const int32_t* seq_lens_host, const void* q,
                                    int32_t q_is_fp32, int32_t num_q_heads, float scale, uint16_t* out,
                                    void* workspace, size_t ws_bytes, void* stream) {
  tq::DecodeArgs a;
  tq_status st = decode_setup(cache, seq_lens_host, num_q_heads, scale, workspace, ws_bytes, a);
  if (st != TQ_OK) return st;
  if (!q || !out) return fail(TQ_EINVAL, "q / out is NULL");
  a.q_in = q;
  a.q_fp32 = q_is_fp32 != 0;
  a.q_rotate = cache->k_format != TQ_FMT_F16;
  a.out = out;
  return launch_decode_and_merge(cache, seq_lens_host, a, 0, static_cast<hipStream_t>(stream));
}

tq_status tq_decode_chunk_fused(const tq_cache* cache, const int32_t* seq_lens_host, const void* q,
                                int32_t q_is_fp32, int32_t num_q_heads, int32_t q_len, float scale, uint16_t* out,
                                void* workspace, size_t ws_bytes, void* stream) {
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if (q_len < 1) return fail(TQ_EINVAL, "q_len %d must be positive", q_len);
  if ((st = check_heads(cache, num_q_heads)) != TQ_OK) return st;
  const int group = num_q_heads / cache->num_kv_heads;
  if ((long long)group * q_len > tq::kMaxGroup)
    return fail(TQ_EUNSUPPORTED, "group size %d x q_len %d exceeds %d columns", group, q_len, tq::kMaxGroup);
  if ((st = check_lengths(cache, seq_lens_host, 0)) != TQ_OK) return st;
  for (int b = 0; b < cache->batch; ++b)
    if (seq_lens_host[b] < q_len)
      return fail(TQ_EINVAL, "sequence %d holds %d tokens, fewer than the chunk's %d", b, seq_lens_host[b], q_len);
  // every (head, position) pair is a column of its KV head: q [B][Hq][q_len][128] is
  // [B][Hkv][group * q_len][128], and so is out
  tq::DecodeArgs a;
  if ((st = decode_setup(cache, seq_lens_host, num_q_heads * q_len, scale, workspace, ws_bytes, a)) != TQ_OK)
    return st;
  if (!q || !out) return fail(TQ_EINVAL, "q / out is NULL");
  a.q_len = q_len;
  a.q_in = q;
  a.q_fp32 = q_is_fp32 != 0;
  a.q_rotate = cache->k_format != TQ_FMT_F16;
  a.out = out;
  return launch_decode_and_merge(cache, seq_lens_host, a, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// Split partials of tq_decode_step_noalloc: one copy per GPU (each device that loads
// this code object holds its own), resolved to a device address once per device.
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.  Host code uses only this address: the
// array's name is a host-side stand-in, not a device address.
tq_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TQ_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}

// tq_decode_step's body after the workspace is known (validated by decode_setup).
tq_status decode_step_launch(const tq_cache* cache, const int32_t* seq_lens_host, const void* k_new,
                             const void* v_new, const void* q, int32_t q_is_fp32, tq::DecodeArgs& a, uint16_t* out,
                             void* stream);

}  // namespace

extern "C" {

tq_status tq_decode_step_noalloc(const tq_cache* cache, const int32_t* seq_lens_host, const void* k_new,
                                 const void* v_new, const void* q, int32_t q_is_fp32, int32_t num_q_heads,
                                 float scale, uint16_t* out, void* stream) {
  // Everything is checked on the host before the device is touched, the size against the
  // array included (a non-NULL stand-in passes decode_setup's workspace check).
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != TQ_OK) return st;
  if ((st = check_lengths(cache, seq_lens_host, 1)) != TQ_OK) return st;
  const size_t need = workspace_bytes(cache, num_q_heads,
                                      make_plan(cache, seq_lens_host, num_q_heads / cache->num_kv_heads));
  if (need > TQ_NOALLOC_SCRATCH_BYTES)
    return fail(TQ_EWORKSPACE, "the call's partials need %zu bytes, more than the %zu bytes of the no-allocation "
                "scratch array", need, (size_t)TQ_NOALLOC_SCRATCH_BYTES);
  if (!k_new || !v_new || !q || !out) return fail(TQ_EINVAL, "k_new / v_new / q / out is NULL");
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != TQ_OK) return st;
  tq::DecodeArgs a;
  if ((st = decode_setup(cache, seq_lens_host, num_q_heads, scale, ws, TQ_NOALLOC_SCRATCH_BYTES, a)) != TQ_OK)
    return st;
  return decode_step_launch(cache, seq_lens_host, k_new, v_new, q, q_is_fp32, a, out, stream);
}

tq_status tq_decode_step(const tq_cache* cache, const int32_t* seq_lens_host, const void* k_new, const void* v_new,
                         const void* q, int32_t q_is_fp32, int32_t num_q_heads, float scale, uint16_t* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  tq::DecodeArgs a;
  tq_status st = decode_setup(cache, seq_lens_host, num_q_heads, scale, workspace, ws_bytes, a);
  if (st != TQ_OK) return st;
  if ((st = check_lengths(cache, seq_lens_host, 1)) != TQ_OK) return st;  // room for the new token
  if (!k_new || !v_new || !q || !out) return fail(TQ_EINVAL, "k_new / v_new / q / out is NULL");
  return decode_step_launch(cache, seq_lens_host, k_new, v_new, q, q_is_fp32, a, out, stream);
}

}  // extern "C"

namespace {

tq_status decode_step_launch(const tq_cache* cache, const int32_t* seq_lens_host, const void* k_new,
                             const void* v_new, const void* q, int32_t q_is_fp32, tq::DecodeArgs& a, uint16_t* out,
                             void* stream) {
  a.q_in = q;
  a.q_fp32 = q_is_fp32 != 0;
  a.q_rotate = cache->k_format != TQ_FMT_F16;
  a.out = out;
  tq::EncodeArgs& e = a.app;
  e.hkv = cache->num_kv_heads;
  e.cap = cache->capacity;
  e.kfmt = cache->k_format;
  e.vfmt = cache->v_format;
  e.t_new = 1;
  e.b0 = 0;
  e.k_new = static_cast<const uint16_t*>(k_new);
  e.v_new = static_cast<const uint16_t*>(v_new);
  e.k_data = static_cast<uint8_t*>(cache->k_data);
  e.k_norms = cache->k_norms;
  e.v_data = static_cast<uint8_t*>(cache->v_data);
  e.v_norms = cache->v_norms;
  e.seq_lens = cache->seq_lens;
  e.k_signs = cache->k_signs;
  e.v_signs = cache->v_signs;
  e.k_cb = cache->k_codebook;
  e.v_cb = cache->v_codebook;
  return launch_decode_and_merge(cache, seq_lens_host, a, 0, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

tq_status tq_decode_attention(const tq_cache* cache, const int32_t* seq_lens_host, const float* q_rot,
                              int32_t num_q_heads, float scale, float* out_rot, void* workspace, size_t ws_bytes,
                              void* stream) {
  return tq_decode_attention_variant(cache, seq_lens_host, q_rot, num_q_heads, scale, out_rot, workspace, ws_bytes,
                                     0, stream);
}

tq_status tq_stream_read(const void* src, size_t bytes, uint32_t* sums, int32_t blocks, void* stream) {
  if (!src || !sums) return fail(TQ_EINVAL, "src / sums is NULL");
  if (bytes == 0 || bytes % 16) return fail(TQ_EINVAL, "bytes %zu must be a positive multiple of 16", bytes);
  if (blocks < 1 || blocks > (1 << 20)) return fail(TQ_EINVAL, "blocks %d outside [1, 2^20]", blocks);
  return hip_status(tq::launch_stream_read(src, bytes, sums, blocks, static_cast<hipStream_t>(stream)),
                    "stream_read launch");
}

tq_status tq_inverse_rotate_out(const tq_cache* cache, const float* out_rot, int32_t num_q_heads, uint16_t* out,
                                void* stream) {
  tq_status st = check_cache(cache);
  if (st != TQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != TQ_OK) return st;
  if (!out_rot || !out) return fail(TQ_EINVAL, "out_rot / out is NULL");
  return hip_status(tq::launch_inverse_rotate(out_rot, cache->v_format != TQ_FMT_F16, cache->v_signs, out,
                                              cache->batch * num_q_heads, static_cast<hipStream_t>(stream)),
                    "inverse_rotate launch");
}

}  // extern "C"
