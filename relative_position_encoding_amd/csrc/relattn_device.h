// Device helpers shared by the gfx950 kernels of librelattn (the forward in
// relattn_kernels.hip, incremental decoding in relattn_decode.hip): vector
// types, address spaces, the hardware exponential and the integer index
// functions of the clip section and the T5 section.  Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include "relattn_internal.h"

namespace relattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define RELATTN_LDS __attribute__((address_space(3)))
#define RELATTN_GLOBAL __attribute__((address_space(1)))
#define RELATTN_CONST __attribute__((address_space(4)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 2^x with the hardware exponential (about 1 ulp; results below 2^-126,
// which cannot change a softmax sum at fp32 precision, flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Integer index functions.  The attention kernels and relattn_debug_indices
// both call these, so the dumped indices are the ones the kernels use.
// ---------------------------------------------------------------------------

// Table row of offset delta = j - i: clip(delta, c) + c (clip section).
__device__ __forceinline__ int clip_label(int delta, int c) {
  return min(max(delta, -c), c) + c;
}

// Bucket beta(delta) of the T5 section.
__device__ __forceinline__ int t5_bucket(int delta, const T5Buckets& t) {
  int base = 0;
  int a;
  if (t.bidir) {
    base = delta > 0 ? t.half : 0;
    a = delta < 0 ? -delta : delta;
  } else {
    a = delta < 0 ? -delta : 0;
  }
  if (a < t.exact) return base + a;
  int s = 0;
  for (int x = 0; x < t.nlog - 1; ++x) s += (a >= t.thr[x]) ? 1 : 0;
  return base + t.exact + s;
}

}  // namespace relattn
