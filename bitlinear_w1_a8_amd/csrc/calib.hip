// Measurement helpers, not part of the forward: the ceilings that the
// forward's kernels are compared with, measured on the device at hand
// rather than taken from the data sheet.
//
//  - an empty kernel: the launch floor a short kernel cannot go below;
//  - a read of a large buffer at full width (16-byte loads, eight in flight
//    per lane, a grid-stride loop over every CU): the HBM read stream that a
//    weight-streaming kernel can hope for;
//  - back-to-back v_mfma_i32_32x32x32_i8, the tiled kernel's instruction, on
//    register operands: the int8 matrix-core rate at the clock the device
//    holds under that load.
// Every kernel leaves a checkable result, so that no work can be dropped.
#include "bl_internal.h"

namespace bl {
namespace {

__global__ void k_calib_empty() {}

// Each block leaves the XOR of all 32-bit words it read in sink[blockIdx.x].
__global__ __launch_bounds__(256) void k_calib_read(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 t = p[i];
    acc ^= t.x ^ t.y ^ t.z ^ t.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Every element of A and B is the int8 `byte` (a run-time value); four independent
// accumulators per wave hide the instruction's latency.  Each MFMA adds
// 32 * byte^2 to every element, so lane 0 of wave w leaves
// 4 * iters * 32 * byte^2 (mod 2^32) in sink[w].
__global__ __launch_bounds__(256) void k_calib_mfma(int iters, int byte, int32_t* __restrict__ sink) {
  const int b = byte & 0xff;
  const int w = b | (b << 8) | (b << 16) | (b << 24);
  const v4i a = {w, w, w, w};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c3, 0, 0, 0);
  }
  if ((threadIdx.x & 63) == 0)
    sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = c0[0] + c1[0] + c2[0] + c3[0];
}

}  // namespace

constexpr int kCalibMfmaBlocks = kCalibMfmaWaves / 4;   // four waves per SIMD on 256 CUs
static_assert(kCalibReadBlocks <= kCalibSinkLen && kCalibMfmaWaves <= kCalibSinkLen, "sink length");

hipError_t launch_calib_empty(hipStream_t stream) {
  k_calib_empty<<<1, 64, 0, stream>>>();
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  k_calib_read<<<kCalibReadBlocks, 256, 0, stream>>>(static_cast<const uint4*>(buf), bytes / 16,
                                                     sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, int byte, int32_t* sink, hipStream_t stream) {
  k_calib_mfma<<<kCalibMfmaBlocks, 256, 0, stream>>>(iters, byte, sink);
  return hipGetLastError();
}

}  // namespace bl
