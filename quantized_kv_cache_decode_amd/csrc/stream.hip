// Measurement aid, not a step of the decode path: a plain streaming read of a
// device buffer, the practical HBM read ceiling the decode kernel's achieved
// bandwidth is set against.  Every lane reads 16-byte words in a grid-stride
// loop (four independent non-temporal loads in flight per lane per round: each
// byte is read once, and on this chip that reads faster than cached loads at
// the same occupancy) and folds them into an XOR checksum; each work group
// writes one checksum word, so the loads cannot be dropped and the writes are
// negligible.
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ sums) {
  const size_t stride = size_t(gridDim.x) * kStreamThreads;
  size_t i = size_t(blockIdx.x) * kStreamThreads + threadIdx.x;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(s4 + i), b = __builtin_nontemporal_load(s4 + i + stride),
                c = __builtin_nontemporal_load(s4 + i + 2 * stride), d = __builtin_nontemporal_load(s4 + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // XOR over the work group: within each wave by lane exchanges, then across the
  // four waves through LDS
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), m, 64));
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sums[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sums, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sums);
  return hipGetLastError();
}

}  // namespace tq
