// Measurement helpers, not part of the forward: the ceilings that the
// forward's kernels are compared with, measured on the device at hand
// rather than taken from the data sheet.
//
//  - an empty kernel: the launch floor a short kernel cannot go below;
//  - a read of a large buffer at full width (16-byte loads, eight in flight
//    per lane, over every CU) in two layouts: the HBM read stream that a
//    weight-streaming kernel can hope for is the better of the two;
//  - back-to-back v_mfma_i32_32x32x32_i8, the tiled kernel's instruction, on
//    register operands: the int8 matrix-core rate at the clock the device
//    holds under that load.
// Every kernel leaves a checkable result, so that no work can be dropped.
#include "bl_internal.h"

namespace bl {
namespace {

__global__ void k_calib_empty() {}

// Each wave leaves the XOR of all 32-bit words it read in
// sink[4 * blockIdx.x + wave].  Each lane keeps eight 16-byte loads in
// flight, in one of two layouts:
//  kReadChunks  - blocks take contiguous 32 KiB chunks (chunk c goes to block
//                 c % gridDim.x); a lane's loads are 4 KiB apart;
//  kReadStride  - a grid-stride loop; a lane's loads are a whole grid apart
//                 (4 MiB with 1024 blocks of 256 lanes).
// On MI355X the power-of-two distance of the second layout costs 10-20% on
// buffers of 64 MiB and more (4.65 against 5.65 TB/s at 64 MiB, rotated over
// 20 buffers); the caller measures both.  Eight loads in flight over 1024
// blocks read a 56 MiB buffer about 4% faster than four over 2048.  The
// result is reduced per wave (DPP, no LDS and no barrier): the reduction and
// the store at the end of the kernel cost about 0.5 us of a 10 us read.
template <int LAYOUT>
__global__ __launch_bounds__(256) void k_calib_read(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  constexpr int kU = 8;
  uint32_t acc = 0;
  int64_t tail;                                     // first vector of the part left over
  if constexpr (LAYOUT == kReadChunks) {
    constexpr int64_t kChunk = 256 * kU;            // 16-byte vectors per chunk
    const int64_t nch = n16 / kChunk;
    for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
      const uint4* q = p + c * kChunk + threadIdx.x;
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = q[u * 256];
#pragma unroll
      for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    tail = nch * kChunk;
  } else {
    const int64_t stride = (int64_t)gridDim.x * 256, round = kU * stride;
    const int64_t whole = n16 / round * round;      // vectors covered by whole rounds
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < whole; i += round) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = p[i + u * stride];
#pragma unroll
      for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    tail = whole;
  }
  // the rest, vector by vector over the whole grid
  for (int64_t i = tail + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256) {
    const uint4 t = p[i];
    acc ^= t.x ^ t.y ^ t.z ^ t.w;
  }
  acc = wave_xor_u(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
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
static_assert(4 * kCalibReadBlocks <= kCalibSinkLen && kCalibMfmaWaves <= kCalibSinkLen,
              "sink length");

hipError_t launch_calib_empty(hipStream_t stream) {
  k_calib_empty<<<1, 64, 0, stream>>>();
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* buf, int64_t bytes, int layout, uint32_t* sink,
                             hipStream_t stream) {
  const uint4* p = static_cast<const uint4*>(buf);
  if (layout == kReadChunks)
    k_calib_read<kReadChunks><<<kCalibReadBlocks, 256, 0, stream>>>(p, bytes / 16, sink);
  else if (layout == kReadStride)
    k_calib_read<kReadStride><<<kCalibReadBlocks, 256, 0, stream>>>(p, bytes / 16, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, int byte, int32_t* sink, hipStream_t stream) {
  k_calib_mfma<<<kCalibMfmaBlocks, 256, 0, stream>>>(iters, byte, sink);
  return hipGetLastError();
}

}  // namespace bl
