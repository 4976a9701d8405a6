// Device helpers shared by the gfx950 kernels: vector types, bf16 / OCP E4M3 conversions,
// DPP reductions inside 16-lane rows, and the launch-argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace pkv {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP FP8 E4M3 ("fn"): bias 7, no infinities, 0x7F/0xFF NaN, max finite 448.
// Quantise a finite float: round to nearest even on the E4M3 grid, saturate to +-448,
// keep the sign (so tiny negatives give 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {               // |x| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {         // |x| < 2^-6: subnormal grid, step 2^-9
    // |x| * 512 is exact; rint rounds half to even; result 0..8 (8 = smallest normal)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 127u + 7u;      // E4M3 exponent field, 1..15
    const uint32_t keep = (a >> 20) & 7u;          // top 3 mantissa bits
    const uint32_t rem = a & 0xFFFFFu;             // dropped 20 bits
    code = (e << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) code += 1u;   // carry may bump e
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// E4M3 code -> bf16 bits of the code's value (exact: E4M3 values are bf16 values).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  uint32_t mag;
  if (e != 0) {
    mag = ((e + 120u) << 7) | (m << 4);
  } else {
    mag = __float_as_uint((float)m * 0.001953125f) >> 16;   // m * 2^-9, exact in bf16
  }
  return s | mag;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Two E4M3 codes (bytes 0 and 1 of `w`, or bytes 2 and 3 when hi) -> two floats, exactly.
// gfx950's conversion instruction decodes the OCP E4M3 format (checked against the
// format's definition for all 256 codes).
template <bool HI>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return make_float2(v[0], v[1]);
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same bits
// (each step adds a lane's value to its partner's, and addition commutes).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

inline int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

// Shared-prefix decode items (extend_attention.hip): for each item (first member, member
// count, first chunk s, span) of the host plan, the split partial of chunks s .. s + span - 1
// for every member, written at chunk s of the split phase's workspace layout (the other
// chunks of the span marked empty).  bf16 q with a bf16 or fp8 E4M3 pool, d = 128,
// group size 1, 2, 4 or 8.
int launch_decode_shared(const void* q, int32_t pool_dtype, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int64_t num_slots, const int32_t* r2t,
                         int64_t stride, int32_t batch, const int32_t* seq_lens, const int32_t* members,
                         const int32_t* items, int64_t n_items,
                         int chunk, int max_splits, int hq, int hkv, float sc_log2, float* ws_ml, float* ws_acc,
                         hipStream_t st);

}  // namespace pkv
