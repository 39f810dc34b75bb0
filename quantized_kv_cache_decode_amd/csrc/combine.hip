// Log-sum-exp merge of the split-K partials of one (sequence, query head), and
// optionally the inverse rotation of the merged output (mlxcel PR #369,
// "Change": attention runs in V's rotated basis and only the [B, Hq, D] output
// is taken back to the original basis).
//
// Split s left (o_s, m_s, l_s): o_s = sum_t 2^(z_t - m_s) v_t, l_s = sum_t
// 2^(z_t - m_s), m_s its running max, with z = scale * log2(e) * q.k (log2 units,
// so every weight is one hardware exp2).  The merged output is
// sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s for any M; M = max_s m_s.
//
// One wave per (sequence, query head): lane j = lane % 16 owns dims 8j..8j+7 and
// lane group sg = lane / 16 takes splits sg, sg + 4, ...  Every load of a round
// is independent (one memory round trip for up to 4 * kBatch splits); each group
// keeps a running (m, l, o), and the four groups are merged with the gfx950 row
// swaps (lane bit 4, then bit 5) -- no LDS, no barrier.  Every group then holds
// the merged row; the inverse rotation spreads it over the wave.  When the call has
// few (sequence, head) rows (latency-bound calls: a few dozen waves on a 256-CU
// chip), a row gets WAVES waves: lane group sg of wave w takes splits 4w + sg,
// 4w + sg + 4 WAVES, ..., every group leaves its state in LDS, and wave 0 merges all
// 4 WAVES of them against their common maximum in one step.
#include <math.h>

#include <algorithm>

#include "tq_device.h"
#include "tq_launch.h"

#ifndef TQ_MERGE_FEW_ROWS
#define TQ_MERGE_FEW_ROWS 256
#endif
#ifndef TQ_MERGE_ROW_WAVES
#define TQ_MERGE_ROW_WAVES 4
#endif

namespace tq {
namespace {

constexpr int kGroups = 4;     // lane groups of 16 per wave
constexpr int kMaxBatch = 17;  // splits per lane group per round (68 per round)
constexpr int kFewRows = TQ_MERGE_FEW_ROWS;  // rows up to which a row gets kRowWaves waves
constexpr int kRowWaves = TQ_MERGE_ROW_WAVES;

__device__ inline float weight(float m, float M) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M); }

// Running state of a lane: the merge of the splits it has seen.
struct Acc {
  float m, l, o[8];
};

// Two states in a fixed order (x from the lower lane), so both lanes of a swapped
// pair compute the same bits.
__device__ inline Acc merge(const Acc& x, const Acc& y) {
  const float M = fmaxf(x.m, y.m);
  Acc r;
  r.m = M;
  if (M == -INFINITY) {
    r.l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.o[i] = 0.f;
    return r;
  }
  const float wx = weight(x.m, M), wy = weight(y.m, M);
  r.l = x.l * wx + y.l * wy;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.o[i] = x.o[i] * wx + y.o[i] * wy;
  return r;
}

// permlane16_swap(v, v) gives lane i the values of lanes i & ~16 and i | 16;
// permlane32_swap the same for bit 5.  All 64 lanes must be active.
template <bool BIT5>
__device__ inline void swap_pair(float v, float& lo, float& hi) {
  const uint32_t u = __float_as_uint(v);
  const auto r = BIT5 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <bool BIT5>
__device__ inline Acc merge_across(const Acc& a) {
  Acc lo, hi;
  swap_pair<BIT5>(a.m, lo.m, hi.m);
  swap_pair<BIT5>(a.l, lo.l, hi.l);
#pragma unroll
  for (int i = 0; i < 8; ++i) swap_pair<BIT5>(a.o[i], lo.o[i], hi.o[i]);
  return merge(lo, hi);
}

// The inverse rotation of the merged row spread over the whole wave, two elements per
// lane: lane (j, sg) takes elements 8j + 2sg and 8j + 2sg + 1 (every lane group holds the
// whole row on entry).  The butterflies and their order (element bits 0..6) are
// fwht128_row's, so the result has the bits of the stand-alone inverse rotation, on a
// shorter chain: one in-lane stage, two lane-group swaps and four DPP stages of two
// values instead of three in-lane stages and four DPP stages of eight.
__device__ inline uint32_t inverse_rotate_pair_f16(float x, float y, float s0, float s1, int lane) {
  {
    const float a = x, b = y;   // element bit 0
    x = a + b;
    y = a - b;
  }
  auto swap_stage = [&](auto bit5_c) {   // element bits 1 and 2: lane bits 4 and 5
    constexpr bool B5 = decltype(bit5_c)::value;
    const bool upper = (lane & (B5 ? 32 : 16)) != 0;
    float lo, hi;
    swap_pair<B5>(x, lo, hi);
    x = upper ? lo - hi : lo + hi;
    swap_pair<B5>(y, lo, hi);
    y = upper ? lo - hi : lo + hi;
  };
  swap_stage(std::false_type{});
  swap_stage(std::true_type{});
  auto dpp_stage = [&](auto m_c) {       // element bits 3..6: lane bits 0..3
    constexpr int M = decltype(m_c)::value;
    const float ox = xor_lane16<M>(x), oy = xor_lane16<M>(y);
    x = (lane & M) ? (ox - x) : (x + ox);
    y = (lane & M) ? (oy - y) : (y + oy);
  };
  dpp_stage(std::integral_constant<int, 1>{});
  dpp_stage(std::integral_constant<int, 2>{});
  dpp_stage(std::integral_constant<int, 4>{});
  dpp_stage(std::integral_constant<int, 8>{});
  const float x0 = x * kInvSqrtD * s0;
  const float x1 = y * kInvSqrtD * s1;
  return uint32_t(__half_as_ushort(__float2half_rn(x0))) | (uint32_t(__half_as_ushort(__float2half_rn(x1))) << 16);
}

// kBatch: splits per lane group per round, sized at launch to the call's longest
// sequence so that short calls do not issue loads they then mask.
template <bool INVERSE, int kBatch, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void combine_kernel(DecodeArgs a, SeqLens lens) {
  // No multiply-add contraction here: the normalised output must round the same
  // whether it goes to memory (then to the stand-alone inverse rotation) or
  // straight into the in-register rotation below.
#pragma clang fp contract(off)
  const int hq = blockIdx.x, b = a.b0 + blockIdx.y;
  const int G = a.group;
  const int h = hq / G, g = hq % G;
  // Decode step: the splits cover the tokens before the append and the appended
  // token has its own slot.
  const bool step = a.step != 0;
  const int L = min(lens.len[blockIdx.y], a.cap);
  const int nsplit = min((L + a.plan.chunk - 1) / a.plan.chunk, a.plan.max_splits);
  const int nparts = nsplit + (step ? 1 : 0);  // partial v lives in slot v, the step's last in slot max_splits
  const size_t p0 = partial_index(a, size_t(b) * a.hkv + h, 0, g);  // slot s: p0 + s*G
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, sg = lane >> 4;
  constexpr int kStride = kGroups * WAVES;  // lane groups of the work group

  // The V sign flips of this lane's 8 dims are requested first: the inverse rotation
  // at the end then waits for no memory round trip of its own.
  // (Requested unconditionally, so no branch makes the compiler wait for them early;
  // without a rotation they come from the workspace and are not used.)
  float4 sgn0 = make_float4(1.f, 1.f, 1.f, 1.f), sgn1 = sgn0;
  if constexpr (INVERSE) {
    const float* sp = a.v_rotated ? a.v_signs : a.part_o;   // (>= 128 floats either way)
    sgn0 = reinterpret_cast<const float4*>(sp + 8 * j)[0];
    sgn1 = reinterpret_cast<const float4*>(sp + 8 * j)[1];
  }
  // Slot v of this (row, head): partials at o_row + v * G * 128 and ml_row + v * G * 2
  // (the row's base is the same for every lane; the per-slot offsets fit in 32 bits).
  const float* o_row = a.part_o + p0 * kDim + 8 * j;
  const float* ml_row = a.part_ml + 2 * p0;

  Acc acc;
  acc.m = -INFINITY;
  acc.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc.o[i] = 0.f;
  for (int s0 = kGroups * wave + sg; s0 < nparts; s0 += kStride * kBatch) {
    float ms[kBatch], ls[kBatch];
    float4 oa[kBatch], ob[kBatch];
    // Every load of the round is issued unconditionally (a partial past the end
    // reads the step's slot, always in bounds) and masked afterwards, so the round
    // costs one memory round trip instead of one per partial.
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int v = s0 + kStride * k;
      const int slot = (v < nsplit ? v : a.plan.max_splits) * G;
      const float2 ml = *reinterpret_cast<const float2*>(ml_row + 2 * slot);
      const float4* src = reinterpret_cast<const float4*>(o_row + slot * kDim);
      ms[k] = ml.x;
      ls[k] = ml.y;
      oa[k] = src[0];
      ob[k] = src[1];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {   // (branches the whole wave skips when every lane is in)
      if (s0 + kStride * k >= nparts) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        oa[k] = ob[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mn = acc.m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mn = fmaxf(mn, ms[k]);
    if (mn == -INFINITY) continue;  // nothing seen yet (every l is 0 too)
    const float c = weight(acc.m, mn);
    acc.l *= c;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.o[i] *= c;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = weight(ms[k], mn);
      acc.l += w * ls[k];
      acc.o[0] += w * oa[k].x; acc.o[1] += w * oa[k].y; acc.o[2] += w * oa[k].z; acc.o[3] += w * oa[k].w;
      acc.o[4] += w * ob[k].x; acc.o[5] += w * ob[k].y; acc.o[6] += w * ob[k].z; acc.o[7] += w * ob[k].w;
    }
    acc.m = mn;
  }

  // the step's length update, once every reader of the old length has finished
  if (step && hq == 0 && threadIdx.x == 0) a.app.seq_lens[b] = L + 1;
  const size_t row = size_t(b) * a.hkv * G + hq;
  if constexpr (WAVES == 1) {
    acc = merge_across<false>(acc);  // groups {0,1} and {2,3}
    acc = merge_across<true>(acc);   // then the two halves: every lane holds the merged row
    float v[8];
    const float inv = nparts > 0 ? 1.f / acc.l : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = nparts > 0 ? acc.o[i] * inv : 0.f;
    if (INVERSE && a.v_rotated) {
      // lane (j, sg) rotates and stores elements 8j + 2sg and 8j + 2sg + 1
      const float s8[8] = {sgn0.x, sgn0.y, sgn0.z, sgn0.w, sgn1.x, sgn1.y, sgn1.z, sgn1.w};
      const float x = sg == 0 ? v[0] : sg == 1 ? v[2] : sg == 2 ? v[4] : v[6];
      const float y = sg == 0 ? v[1] : sg == 1 ? v[3] : sg == 2 ? v[5] : v[7];
      const float s0 = sg == 0 ? s8[0] : sg == 1 ? s8[2] : sg == 2 ? s8[4] : s8[6];
      const float s1 = sg == 0 ? s8[1] : sg == 1 ? s8[3] : sg == 2 ? s8[5] : s8[7];
      const uint32_t wv = inverse_rotate_pair_f16(x, y, s0, s1, lane);
      *reinterpret_cast<uint32_t*>(a.out + row * kDim + 8 * j + 2 * sg) = wv;
    } else if (INVERSE) {   // fp16 V: already the original basis
      uint32_t w[4];
      round_row_f16(v, w);
      if (sg == 0) *reinterpret_cast<uint4*>(a.out + row * kDim + 8 * j) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (sg == 0) {
      float4* dst = reinterpret_cast<float4*>(a.out_rot + row * kDim + 8 * j);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  } else {
    // Few rows: every lane group's state goes to LDS, and wave 0 merges all of them
    // against their common maximum in one step (every dim with the same weights),
    // lane (j, sg) taking dims 8j + 2sg and 8j + 2sg + 1 -- the layout the wave-wide
    // inverse rotation takes.
    constexpr int NG = kGroups * WAVES;
    static_assert((NG & (NG - 1)) == 0, "pairwise trees over a power of two of states");
    __shared__ float st_o[NG][kDim];
    __shared__ float2 st_ml[NG];
    const int gi = kGroups * wave + sg;
    float4* d = reinterpret_cast<float4*>(&st_o[gi][8 * j]);
    d[0] = make_float4(acc.o[0], acc.o[1], acc.o[2], acc.o[3]);
    d[1] = make_float4(acc.o[4], acc.o[5], acc.o[6], acc.o[7]);
    if (j == 0) st_ml[gi] = make_float2(acc.m, acc.l);
    __syncthreads();
    if (wave != 0) return;
    const int d0 = 8 * j + 2 * sg;
    float2 ml[NG];
    float mx[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      ml[i] = st_ml[i];
      mx[i] = ml[i].x;
    }
    // the maximum and the three sums as fixed pairwise trees (log2 NG levels instead
    // of NG - 1 dependent steps; the same order in every lane and on every call)
#pragma unroll
    for (int w = 1; w < NG; w *= 2)
#pragma unroll
      for (int i = 0; i < NG; i += 2 * w) mx[i] = fmaxf(mx[i], mx[i + w]);
    const float M = mx[0];
    float pl[NG], px[NG], py[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float c = weight(ml[i].x, M);   // (0 for an empty state)
      const float2 o = *reinterpret_cast<const float2*>(&st_o[i][d0]);
      pl[i] = c * ml[i].y;
      px[i] = c * o.x;
      py[i] = c * o.y;
    }
#pragma unroll
    for (int w = 1; w < NG; w *= 2) {
#pragma unroll
      for (int i = 0; i < NG; i += 2 * w) {
        pl[i] += pl[i + w];
        px[i] += px[i + w];
        py[i] += py[i + w];
      }
    }
    const float l = pl[0];
    float x = px[0], y = py[0];
    const float inv = nparts > 0 ? 1.f / l : 0.f;
    x = nparts > 0 ? x * inv : 0.f;
    y = nparts > 0 ? y * inv : 0.f;
    if (INVERSE && a.v_rotated) {
      const float s8[8] = {sgn0.x, sgn0.y, sgn0.z, sgn0.w, sgn1.x, sgn1.y, sgn1.z, sgn1.w};
      const float s0 = sg == 0 ? s8[0] : sg == 1 ? s8[2] : sg == 2 ? s8[4] : s8[6];
      const float s1 = sg == 0 ? s8[1] : sg == 1 ? s8[3] : sg == 2 ? s8[5] : s8[7];
      *reinterpret_cast<uint32_t*>(a.out + row * kDim + d0) = inverse_rotate_pair_f16(x, y, s0, s1, lane);
    } else if (INVERSE) {   // fp16 V: already the original basis
      *reinterpret_cast<uint32_t*>(a.out + row * kDim + d0) =
          uint32_t(__half_as_ushort(__float2half_rn(x))) | (uint32_t(__half_as_ushort(__float2half_rn(y))) << 16);
    } else {
      *reinterpret_cast<float2*>(a.out_rot + row * kDim + d0) = make_float2(x, y);
    }
  }
}

template <bool INVERSE, int WAVES>
void launch_batch(const DecodeArgs& a, const SeqLens& lens, int nb, int rounds, hipStream_t stream) {
  const dim3 grid(a.hkv * a.group, nb), block(64 * WAVES);
  if (rounds <= 1) hipLaunchKernelGGL((combine_kernel<INVERSE, 1, WAVES>), grid, block, 0, stream, a, lens);
  else if (rounds <= 2) hipLaunchKernelGGL((combine_kernel<INVERSE, 2, WAVES>), grid, block, 0, stream, a, lens);
  else if (rounds <= 3) hipLaunchKernelGGL((combine_kernel<INVERSE, 3, WAVES>), grid, block, 0, stream, a, lens);
  else if (rounds <= 5) hipLaunchKernelGGL((combine_kernel<INVERSE, 5, WAVES>), grid, block, 0, stream, a, lens);
  else if (rounds <= 9) hipLaunchKernelGGL((combine_kernel<INVERSE, 9, WAVES>), grid, block, 0, stream, a, lens);
  else hipLaunchKernelGGL((combine_kernel<INVERSE, kMaxBatch, WAVES>), grid, block, 0, stream, a, lens);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  // partials of the longest sequence of the launch (the step's own slot included)
  int most = 0;
  for (int i = 0; i < batch; ++i) {
    const int L = std::min(lens.len[i], a.cap);
    most = std::max(most, std::min((L + a.plan.chunk - 1) / a.plan.chunk, a.plan.max_splits));
  }
  most += a.app.k_new != nullptr ? 1 : 0;
  // Few rows (at most kFewRows): kRowWaves waves per row share its splits.
  const bool few = (long long)a.hkv * a.group * batch <= kFewRows;
  const int groups = kGroups * (few ? kRowWaves : 1);
  const int rounds = (most + groups - 1) / groups;
  if (a.out) {
    if (few) launch_batch<true, kRowWaves>(a, lens, batch, rounds, stream);
    else launch_batch<true, 1>(a, lens, batch, rounds, stream);
  } else {
    if (few) launch_batch<false, kRowWaves>(a, lens, batch, rounds, stream);
    else launch_batch<false, 1>(a, lens, batch, rounds, stream);
  }
  return hipGetLastError();
}

}  // namespace tq
