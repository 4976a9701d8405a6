// kv_scatter: write the new tokens' K and V rows into their KV pool slots.
//
// The pool is token-granular: one slot per token, each slot holding [hkv, d] values
// for K and for V (the radix-cache page stores one KV index per token in a node's
// value).  New tokens are the unmatched suffix of each request plus decoded tokens;
// their K/V rows arrive contiguous, in q-row order, and go to the slots the allocator
// handed out.
//
// One thread moves 16 source bytes.  Copies keep the dtype; the bf16 -> fp8 path
// quantises with the per-head inverse scale (OCP E4M3, round to nearest even,
// saturating), writing 8 bytes per thread.  HBM-bound: per token it reads
// 2*hkv*d*src_bytes and writes 2*hkv*d*pool_bytes.
//
// A slot outside [0, num_slots) is skipped (its token is not written), so a bad slot list
// cannot write past the pools.  Builds with PKV_DEBUG also copy the slot list to the host
// before the launch and reject out-of-range or repeated slots with PKV_ERR_SLOT.

#include <vector>

#include "device.h"

namespace pkv {
namespace {

// Copy: each thread moves one 16-byte chunk of K and the same chunk of V.
__global__ __launch_bounds__(256) void scatter_copy(const uint4* __restrict__ ksrc, const uint4* __restrict__ vsrc,
                                                    const int32_t* __restrict__ slots, int64_t n, int chunks_per_row,
                                                    uint32_t num_slots, uint4* __restrict__ kpool,
                                                    uint4* __restrict__ vpool) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * chunks_per_row) return;
  const int64_t tok = i / chunks_per_row;
  const int c = (int)(i - tok * chunks_per_row);
  const uint32_t slot = (uint32_t)slots[tok];
  if (slot >= num_slots) return;
  const int64_t dst = (int64_t)slot * chunks_per_row + c;
  const uint4 k = ksrc[i];
  const uint4 v = vsrc[i];
  kpool[dst] = k;
  vpool[dst] = v;
}

__device__ __forceinline__ uint32_t pack4_e4m3(uint32_t w0, uint32_t w1, float s) {
  return f32_to_e4m3(bf16_lo(w0) * s) | (f32_to_e4m3(bf16_hi(w0) * s) << 8) | (f32_to_e4m3(bf16_lo(w1) * s) << 16) |
         (f32_to_e4m3(bf16_hi(w1) * s) << 24);
}

// bf16 -> fp8: each thread reads 8 bf16 (16 B) of K and of V and writes 8 codes (8 B) each.
__global__ __launch_bounds__(256) void scatter_fp8(const uint4* __restrict__ ksrc, const uint4* __restrict__ vsrc,
                                                   const int32_t* __restrict__ slots, int64_t n, int chunks_per_row,
                                                   int chunks_per_head, uint32_t num_slots,
                                                   const float* __restrict__ kinv, const float* __restrict__ vinv,
                                                   uint2* __restrict__ kpool, uint2* __restrict__ vpool) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * chunks_per_row) return;
  const int64_t tok = i / chunks_per_row;
  const int c = (int)(i - tok * chunks_per_row);
  const int h = c / chunks_per_head;
  const uint32_t slot = (uint32_t)slots[tok];
  if (slot >= num_slots) return;
  const int64_t dst = (int64_t)slot * chunks_per_row + c;
  const uint4 k = ksrc[i];
  const uint4 v = vsrc[i];
  const float ks = kinv[h], vs = vinv[h];
  kpool[dst] = make_uint2(pack4_e4m3(k.x, k.y, ks), pack4_e4m3(k.z, k.w, ks));
  vpool[dst] = make_uint2(pack4_e4m3(v.x, v.y, vs), pack4_e4m3(v.z, v.w, vs));
}

// Device copy of the table emit of one decode step: req_to_token[b, seq_lens[b] - 1] = slots[b].
__global__ __launch_bounds__(256) void append_slots(int32_t* __restrict__ r2t, int64_t stride,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ slots, int32_t batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int pos = seq_lens[b] - 1;
  if (pos >= 0 && pos < stride) r2t[(int64_t)b * stride + pos] = slots[b];
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_append_slots(int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, const int32_t* slots,
                                int32_t batch, void* stream) {
  if (batch < 0 || stride <= 0) return fail(PKV_ERR_INVAL, "append_slots: bad sizes");
  if (batch == 0) return PKV_OK;
  if (!req_to_token || !seq_lens || !slots) return fail(PKV_ERR_INVAL, "append_slots: null pointer");
  hipLaunchKernelGGL(append_slots, dim3((batch + 255) / 256), dim3(256), 0, (hipStream_t)stream, req_to_token, stride,
                     seq_lens, slots, batch);
  return hip_check(hipGetLastError(), "append_slots launch");
}

extern "C" int pkv_kv_scatter(const void* k_src, const void* v_src, int32_t src_dtype, const int32_t* slots, int64_t n,
                              void* k_pool, void* v_pool, int32_t pool_dtype, int64_t num_slots, int32_t hkv,
                              int32_t d, const float* k_inv_scale, const float* v_inv_scale, void* stream) {
  if (n < 0 || hkv <= 0 || num_slots <= 0) return fail(PKV_ERR_INVAL, "kv_scatter: bad sizes");
  if (n == 0) return PKV_OK;
  if (!k_src || !v_src || !slots || !k_pool || !v_pool) return fail(PKV_ERR_INVAL, "kv_scatter: null pointer");
  if (d != 64 && d != 128) return fail(PKV_ERR_UNSUPPORTED, "kv_scatter: d=%d", d);
  if (num_slots > (int64_t)INT32_MAX) return fail(PKV_ERR_INVAL, "kv_scatter: num_slots beyond int32");
  hipStream_t st = (hipStream_t)stream;
#ifdef PKV_DEBUG
  {
    // debug builds: every slot in range and none twice (a repeated slot would race)
    std::vector<int32_t> h((size_t)n);
    if (int rc = hip_check(hipMemcpyAsync(h.data(), slots, (size_t)n * 4, hipMemcpyDeviceToHost, st), "kv_scatter slots"))
      return rc;
    if (int rc = hip_check(hipStreamSynchronize(st), "kv_scatter slots")) return rc;
    std::vector<uint8_t> seen((size_t)num_slots, 0);
    for (int64_t i = 0; i < n; ++i) {
      if (h[i] < 0 || h[i] >= num_slots) return fail(PKV_ERR_SLOT, "kv_scatter: slot %d of token %lld out of range", h[i], (long long)i);
      if (seen[h[i]]++) return fail(PKV_ERR_SLOT, "kv_scatter: slot %d written twice", h[i]);
    }
  }
#endif
  const int threads = 256;
  if ((src_dtype == PKV_F32 && pool_dtype == PKV_F32) || (src_dtype == PKV_BF16 && pool_dtype == PKV_BF16)) {
    const int esz = src_dtype == PKV_F32 ? 4 : 2;
    const int chunks = hkv * d * esz / 16;
    const int64_t total = n * chunks;
    hipLaunchKernelGGL(scatter_copy, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, st,
                       (const uint4*)k_src, (const uint4*)v_src, slots, n, chunks, (uint32_t)num_slots, (uint4*)k_pool,
                       (uint4*)v_pool);
  } else if (src_dtype == PKV_BF16 && pool_dtype == PKV_FP8_E4M3) {
    if (!k_inv_scale || !v_inv_scale) return fail(PKV_ERR_INVAL, "kv_scatter: fp8 pool needs inverse scales");
    const int chunks = hkv * d / 8;
    const int64_t total = n * chunks;
    hipLaunchKernelGGL(scatter_fp8, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, st,
                       (const uint4*)k_src, (const uint4*)v_src, slots, n, chunks, d / 8, (uint32_t)num_slots,
                       k_inv_scale, v_inv_scale, (uint2*)k_pool, (uint2*)v_pool);
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "kv_scatter: src dtype %d -> pool dtype %d", src_dtype, pool_dtype);
  }
  return hip_check(hipGetLastError(), "kv_scatter launch");
}
