// mxs_stream_read: a plain read of a device buffer, the measured ceiling of the weight stream.
//
// A verification step that streams every weight once is bounded by Q <= BW / W ("Module 11.
// Speculative Decoding and Quantization", §1): the verify GEMM's achieved bandwidth is measured
// against BW. This kernel measures the BW a single kernel can draw from HBM on this device with
// nothing else to do: every lane issues 8 independent 16-byte non-temporal loads per step (the
// data is read once, so it is not kept in the caches), folds them into an XOR, and writes the
// result only if it equals a fixed constant, so no load can be dropped and almost nothing is
// written. Grid: two 256-thread workgroups per compute unit, each walking the buffer with the
// grid stride (the best of the unroll depths, workgroup sizes and grid sizes measured).
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                    uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (size_t)(kStreamUnroll - 1) * stride < n16; i += (size_t)kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + (size_t)u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) atomicOr(sink, 1u);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  stream_read_kernel<<<dim3((unsigned)(2 * device_cus())), dim3(kStreamThreads), 0, stream>>>(
      static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace mxs
