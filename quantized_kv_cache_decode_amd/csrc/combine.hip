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
// 256 threads: lane j = tid % 16 owns dims 8j..8j+7 and split group sg = tid / 16
// takes splits sg, sg + 16, ...  Every load of a batch is independent (one
// memory round trip for up to 64 splits); each group keeps a running (m, l, o),
// and the 16 groups are merged through LDS by the 16 threads of group 0, which
// hold exactly the 16-lane row layout the in-register Walsh-Hadamard transform
// wants.
#include <math.h>

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr int kSplitGroups = 16;
constexpr int kBatch = 5;  // splits per thread per round of loads (80 per round)

__device__ inline float weight(float m, float M) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M); }

template <bool INVERSE>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, SeqLens lens) {
  // No multiply-add contraction here: the normalised output must round the same
  // whether it goes to memory (then to the stand-alone inverse rotation) or
  // straight into the in-register rotation below.
#pragma clang fp contract(off)
  const int hq = blockIdx.x, b = a.b0 + blockIdx.y;
  const int G = a.group;
  const int h = hq / G, g = hq % G;
  // Decode step: the splits cover the tokens before the append and the appended
  // token has its own slot.
  const bool step = a.app.k_new != nullptr;
  const int L = min(lens.len[blockIdx.y], a.cap);
  const int nsplit = min((L + a.plan.chunk - 1) / a.plan.chunk, a.plan.max_splits);
  const int nparts = nsplit + (step ? 1 : 0);  // partial v lives in slot v, the step's last in slot max_splits
  const size_t p0 = partial_index(a, size_t(b) * a.hkv + h, 0, g);  // slot s: p0 + s*G
  const int j = threadIdx.x & 15, sg = threadIdx.x >> 4;

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int s0 = sg; s0 < nparts; s0 += kSplitGroups * kBatch) {
    float ms[kBatch], ls[kBatch];
    float4 oa[kBatch], ob[kBatch];
    // Every load of the round is issued unconditionally (a partial past the end
    // reads slot 0, always in bounds) and masked afterwards, so the round costs one
    // memory round trip instead of one per partial.
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int v = s0 + kSplitGroups * k;
      const size_t p = p0 + size_t(v < nsplit ? v : (v < nparts ? a.plan.max_splits : 0)) * G;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * p);
      const float4* src = reinterpret_cast<const float4*>(a.part_o + p * kDim + 8 * j);
      ms[k] = ml.x;
      ls[k] = ml.y;
      oa[k] = src[0];
      ob[k] = src[1];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (s0 + kSplitGroups * k >= nparts) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        oa[k] = ob[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mn = m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mn = fmaxf(mn, ms[k]);
    if (mn == -INFINITY) continue;  // nothing seen yet (every l is 0 too)
    const float c = weight(m, mn);
    l *= c;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= c;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = weight(ms[k], mn);
      l += w * ls[k];
      o[0] += w * oa[k].x; o[1] += w * oa[k].y; o[2] += w * oa[k].z; o[3] += w * oa[k].w;
      o[4] += w * ob[k].x; o[5] += w * ob[k].y; o[6] += w * ob[k].z; o[7] += w * ob[k].w;
    }
    m = mn;
  }

  __shared__ float sm[kSplitGroups], sl[kSplitGroups];
  __shared__ float4 so[kSplitGroups][32];
  so[sg][2 * j] = make_float4(o[0], o[1], o[2], o[3]);
  so[sg][2 * j + 1] = make_float4(o[4], o[5], o[6], o[7]);
  if (j == 0) {
    sm[sg] = m;
    sl[sg] = l;
  }
  __syncthreads();
  if (threadIdx.x >= 16) return;  // group 0 finishes (lanes 0..15 of wave 0)

  float M = sm[0];
#pragma unroll
  for (int k = 1; k < kSplitGroups; ++k) M = fmaxf(M, sm[k]);
  float lt = 0.f, v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
#pragma unroll
  for (int k = 0; k < kSplitGroups; ++k) {
    const float w = weight(sm[k], M);
    const float4 x = so[k][2 * j], y = so[k][2 * j + 1];
    lt += w * sl[k];
    v[0] += w * x.x; v[1] += w * x.y; v[2] += w * x.z; v[3] += w * x.w;
    v[4] += w * y.x; v[5] += w * y.y; v[6] += w * y.z; v[7] += w * y.w;
  }
  const float inv = nparts > 0 ? 1.f / lt : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = nparts > 0 ? v[i] * inv : 0.f;
  // the step's length update, once every reader of the old length has finished
  if (step && hq == 0 && j == 0) a.app.seq_lens[b] = L + 1;
  const size_t row = size_t(b) * a.hkv * G + hq;
  if (INVERSE) {
    uint32_t w[4];
    rotate_row_inverse_f16(v, a.v_signs, j, w);
    *reinterpret_cast<uint4*>(a.out + row * kDim + 8 * j) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* dst = reinterpret_cast<float4*>(a.out_rot + row * kDim + 8 * j);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  const dim3 grid(a.hkv * a.group, batch), block(256);
  if (a.out) hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, a, lens);
  else hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, a, lens);
  return hipGetLastError();
}

}  // namespace tq
