// Streaming read of a device buffer: the rate a plain read-only kernel reaches on this GPU's
// HBM, the practical ceiling to set beside the published 8 TB/s for the HBM-bound kernels
// (decode's split phase and kv_scatter).  Each lane reads 16 bytes at a time, four loads in
// flight per iteration, grid-strided over the buffer; the words are folded with XOR and one
// word per wave is written so the loads stay live.

#include "device.h"

namespace pkv {
namespace {

constexpr int kProbeBlocks = 4096;

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, int64_t n16, uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_stream_read_words(void) { return kProbeBlocks * 4; }

extern "C" int pkv_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16) return fail(PKV_ERR_INVAL, "stream_read: bad arguments");
  hipLaunchKernelGGL(stream_read, dim3(kProbeBlocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16,
                     out);
  return hip_check(hipGetLastError(), "stream_read launch");
}
