// Plain VALU split-K decode attention (the A/B reference variant) and the
// log-sum-exp split merge.
//
// Work item = (split s, KV head h, sequence b), 256 threads = 4 waves.  Each
// pass covers 256 tokens, 64 per wave:
//   scores   lane = token: the lane unpacks its token's K record and forms
//            z_g = scale * n_K * sum_d q_rot[g,d] * c_K[idx_d] for the G query
//            heads of this KV head (rotated basis; mlxcel PR #369, "Change");
//   softmax  running max / sum per head and wave (flash-decode style);
//   values   lane = dim pair: accumulates p_g,t * n_V,t * c_V[idx] over the
//            wave's 64 tokens, still in V's rotated basis.
// The 4 waves' (m, l, o) are merged in LDS and written as the split's partial.
// Dequant stays interleaved with the multiply-adds of the token that needs it
// (turboquant_plus "SMEM Pre-Dequant Experiment", "Why It Failed": separating
// a dequant phase from the math phase cost 2x there).
#include <math.h>

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

template <int FMT>
__device__ inline uint32_t k_code(const uint32_t* rec, int d) {
  if (FMT == kFmtTurbo3) return sub3_get(rec + 3 * (d >> 5), d & 31);
  return t4_index_of_nibble(oct4_get_nibble(rec[d >> 3], d & 7));
}

// Codes of dims d and d+1 (d even) of token t in V tile layout.
template <int FMT>
__device__ inline void v_code_pair(const uint8_t* v_row, int t, int d, uint32_t& c0, uint32_t& c1) {
  const int tile = t >> 5, r = t & 31;
  const int g = slot_group(r), i = slot_elem(r);
  const int n = d >> 3, nb = d & 7;
  const uint8_t* vt = v_row + size_t(tile) * v_tile_bytes(FMT);
  const int c = 16 * g + n;
  if (FMT == kFmtTurbo3) {
    const int e0 = 8 * nb + i, e1 = e0 + 8;   // sub-block e / 32 is piece e / 32 of the chunk
    c0 = sub3_get(reinterpret_cast<const uint32_t*>(vt + v_chunk_byte_offset(FMT, c, 12 * (e0 >> 5))), e0 & 31);
    c1 = sub3_get(reinterpret_cast<const uint32_t*>(vt + v_chunk_byte_offset(FMT, c, 12 * (e1 >> 5))), e1 & 31);
  } else {
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(vt + v_chunk_byte_offset(FMT, c, 4 * nb));
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(vt + v_chunk_byte_offset(FMT, c, 4 * nb + 4));
    c0 = t4_index_of_nibble(oct4_get_nibble(w0, i));
    c1 = t4_index_of_nibble(oct4_get_nibble(w1, i));
  }
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int KFMT, int VFMT>
__global__ __launch_bounds__(256) void decode_ref_kernel(DecodeArgs a, SeqLens lens) {
  const int s = blockIdx.x, h = blockIdx.y, b = a.b0 + blockIdx.z;
  const int G = a.group;
  const int L = min(lens.len[blockIdx.z], a.cap);
  const int chunk = a.plan.chunk;
  const int nsplit = min((L + chunk - 1) / chunk, a.plan.max_splits);
  if (s >= nsplit) return;
  const int t0 = s * chunk;
  const int t1 = (s == nsplit - 1) ? L : t0 + chunk;

  __shared__ float qs[kMaxGroup][kDim];
  __shared__ float ps[4][kMaxGroup][64];
  __shared__ float kcb[16], vcb[16];
  __shared__ float wm[4][kMaxGroup], wl[4][kMaxGroup];
  __shared__ float wo[4][kMaxGroup][kDim];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hq0 = h * G;
  const int Hq = a.hkv * G;
  for (int i = tid; i < G * kDim; i += 256) qs[i / kDim][i % kDim] = a.q_rot[(size_t(b) * Hq + hq0) * kDim + i];
  if (tid < 16) {
    kcb[tid] = (KFMT != kFmtF16 && tid < levels(KFMT)) ? half_bits_to_float(a.k_cb[tid]) : 0.f;
    vcb[tid] = tid < levels(VFMT) ? half_bits_to_float(a.v_cb[tid]) : 0.f;
  }
  __syncthreads();

  float m_run[kMaxGroup], l_run[kMaxGroup], acc0[kMaxGroup], acc1[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
  }

  const size_t row = size_t(b) * a.hkv + h;
  const uint8_t* v_row = a.v_data + row * size_t(a.cap / kTileTokens) * v_tile_bytes(VFMT);
  const int n_iter = (t1 - t0 + 255) / 256;
  for (int it = 0; it < n_iter; ++it) {
    const int base = t0 + it * 256 + w * 64;
    const int t = base + lane;
    const bool valid = t < t1;
    float z[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) z[g] = 0.f;
    if (valid) {
      if (KFMT == kFmtF16) {
        const uint16_t* kr = reinterpret_cast<const uint16_t*>(a.k_data) + (row * a.cap + t) * kDim;
        for (int d = 0; d < kDim; ++d) {
          const float kv = half_bits_to_float(kr[d]);
#pragma unroll
          for (int g = 0; g < kMaxGroup; ++g)
            if (g < G) z[g] += qs[g][d] * kv;
        }
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) z[g] *= a.scale;
      } else {
        constexpr int kWords = k_record_bytes(KFMT) / 4;
        uint32_t rec[kWords];
        const uint8_t* row_k = a.k_data + row * a.cap * k_record_bytes(KFMT);
#pragma unroll
        for (int i = 0; i < kWords; ++i) rec[i] = *reinterpret_cast<const uint32_t*>(row_k + k_byte_offset(KFMT, t, 4 * i));
#pragma unroll
        for (int d = 0; d < kDim; ++d) {
          const float kv = kcb[k_code<KFMT>(rec, d)];
#pragma unroll
          for (int g = 0; g < kMaxGroup; ++g)
            if (g < G) z[g] += qs[g][d] * kv;
        }
        const float f = a.scale * half_bits_to_float(a.k_norms[row * a.cap + t]);
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) z[g] *= f;
      }
    }
    const float nv = valid ? half_bits_to_float(a.v_norms[row * a.cap + t]) : 0.f;
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g < G) {
        const float mt = wave_max(valid ? z[g] : -INFINITY);
        const float m_new = fmaxf(m_run[g], mt);
        const float alpha = (m_run[g] == -INFINITY) ? 0.f : expf(m_run[g] - m_new);
        const float p = valid ? expf(z[g] - m_new) : 0.f;
        l_run[g] = l_run[g] * alpha + wave_sum(p);
        acc0[g] *= alpha;
        acc1[g] *= alpha;
        m_run[g] = m_new;
        ps[w][g][lane] = valid ? p * nv : 0.f;
      }
    }
    __syncthreads();
    const int d = 2 * lane;
    for (int tt = 0; tt < 64; ++tt) {
      const int t2 = base + tt;
      if (t2 >= t1) break;
      uint32_t c0, c1;
      v_code_pair<VFMT>(v_row, t2, d, c0, c1);
      const float v0 = vcb[c0], v1 = vcb[c1];
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) {
        if (g < G) {
          const float pw = ps[w][g][tt];
          acc0[g] += pw * v0;
          acc1[g] += pw * v1;
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g < G) {
      if (lane == 0) {
        wm[w][g] = m_run[g];
        wl[w][g] = l_run[g];
      }
      wo[w][g][2 * lane] = acc0[g];
      wo[w][g][2 * lane + 1] = acc1[g];
    }
  }
  __syncthreads();
  const size_t pidx = partial_index(a, row, s, 0);
  for (int i = tid; i < G * kDim; i += 256) {
    const int g = i / kDim, d = i % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, wm[ww][g]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = (wm[ww][g] == -INFINITY) ? 0.f : expf(wm[ww][g] - M);
      o += f * wo[ww][g][d];
      l += f * wl[ww][g];
    }
    a.part_o[(pidx + g) * kDim + d] = o;
    if (d == 0) {
      a.part_ml[(pidx + g) * 2] = M * 1.4426950408889634f;  // partials keep m in log2 units
      a.part_ml[(pidx + g) * 2 + 1] = l;
    }
  }
}

template <int KF, int VF>
void launch_ref(const DecodeArgs& a, const SeqLens& lens, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_ref_kernel<KF, VF>), grid, dim3(256), 0, stream, a, lens);
}

}  // namespace

hipError_t launch_decode_reference(const DecodeArgs& a, const SeqLens& lens, int batch, hipStream_t stream) {
  const dim3 grid(a.plan.max_splits, a.hkv, batch);
  if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo3) launch_ref<kFmtTurbo3, kFmtTurbo3>(a, lens, grid, stream);
  else if (a.kfmt == kFmtTurbo3 && a.vfmt == kFmtTurbo4) launch_ref<kFmtTurbo3, kFmtTurbo4>(a, lens, grid, stream);
  else if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo3) launch_ref<kFmtTurbo4, kFmtTurbo3>(a, lens, grid, stream);
  else if (a.kfmt == kFmtTurbo4 && a.vfmt == kFmtTurbo4) launch_ref<kFmtTurbo4, kFmtTurbo4>(a, lens, grid, stream);
  else if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo3) launch_ref<kFmtF16, kFmtTurbo3>(a, lens, grid, stream);
  else if (a.kfmt == kFmtF16 && a.vfmt == kFmtTurbo4) launch_ref<kFmtF16, kFmtTurbo4>(a, lens, grid, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq
