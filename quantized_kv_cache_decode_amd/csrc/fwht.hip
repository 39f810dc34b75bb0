// 128-point Walsh-Hadamard rotations of rows, in registers: one row per 16
// lanes, 8 elements per lane (fwht128_row); normalised by 1/sqrt(128).
//
// tq_rotate_q:          q_rot = H (s_K * q) / sqrt(128)   (fp16 or fp32 in, fp32 out)
// tq_inverse_rotate_out: out  = s_V * H (o) / sqrt(128)   (fp32 in, fp16 RNE out)
// (mlxcel PR #369, "Change": symmetric modes rotate Q into K's basis; only the
// small attention output is inverse-rotated out of V's basis.)
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

template <bool IN_FP32, bool ROTATE>
__global__ __launch_bounds__(256) void rotate_q_kernel(const void* __restrict__ q, const float* __restrict__ signs,
                                                       float* __restrict__ q_rot, int rows) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lane16 = threadIdx.x & 15;
  if (row >= rows) return;  // whole 16-lane segments leave together
  float v[8];
  const size_t base = size_t(row) * kDim + 8 * lane16;
  load_row8(q, IN_FP32, base, v);
  if (ROTATE) rotate_row_forward(v, signs, lane16);
  float4* o = reinterpret_cast<float4*>(q_rot + base);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ROTATE = false (fp16 V, stored unrotated): the fp16 rounding alone.
template <bool ROTATE>
__global__ __launch_bounds__(256) void inverse_rotate_kernel(const float* __restrict__ o_rot,
                                                             const float* __restrict__ signs,
                                                             uint16_t* __restrict__ out, int rows) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lane16 = threadIdx.x & 15;
  if (row >= rows) return;
  const size_t base = size_t(row) * kDim + 8 * lane16;
  const float4* p = reinterpret_cast<const float4*>(o_rot + base);
  const float4 a = p[0], b = p[1];
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t w[4];
  if (ROTATE) rotate_row_inverse_f16(v, signs, lane16, w);
  else round_row_f16(v, w);
  *reinterpret_cast<uint4*>(out + base) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

hipError_t launch_rotate_q(const void* q, bool q_fp32, bool rotate, const float* signs, float* q_rot, int rows,
                           hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 15) / 16), block(256);
  if (q_fp32) {
    if (rotate) hipLaunchKernelGGL((rotate_q_kernel<true, true>), grid, block, 0, stream, q, signs, q_rot, rows);
    else hipLaunchKernelGGL((rotate_q_kernel<true, false>), grid, block, 0, stream, q, signs, q_rot, rows);
  } else {
    if (rotate) hipLaunchKernelGGL((rotate_q_kernel<false, true>), grid, block, 0, stream, q, signs, q_rot, rows);
    else hipLaunchKernelGGL((rotate_q_kernel<false, false>), grid, block, 0, stream, q, signs, q_rot, rows);
  }
  return hipGetLastError();
}

hipError_t launch_inverse_rotate(const float* o_rot, bool rotate, const float* signs, uint16_t* out, int rows,
                                 hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 15) / 16), block(256);
  if (rotate) hipLaunchKernelGGL((inverse_rotate_kernel<true>), grid, block, 0, stream, o_rot, signs, out, rows);
  else hipLaunchKernelGGL((inverse_rotate_kernel<false>), grid, block, 0, stream, o_rot, signs, out, rows);
  return hipGetLastError();
}

}  // namespace tq
