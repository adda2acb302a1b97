// Device-side helpers shared by the linattn kernels: element conversion for
// the three storage types and the elu+1 feature map.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "linattn.h"

namespace la {

// Storage types of q, k, v and out.  bf16 is carried as raw 16-bit words.
using bf16_t = uint16_t;
using f16_t = _Float16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ float to_f32(f16_t x) { return float(x); }

// Round-to-nearest-even conversions (gfx950 v_cvt_pk_bf16_f32 / v_cvt_f16_f32).
__device__ __forceinline__ void store_f32(float x, float* d) { *d = x; }
__device__ __forceinline__ void store_f32(float x, bf16_t* d) {
  *d = __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ void store_f32(float x, f16_t* d) { *d = static_cast<f16_t>(x); }

// phi(x) = elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise
// (llm-arch-kb "Linear Attention", section 2, symbol legend).
__device__ __forceinline__ float elu1_accurate(float x) { return x > 0.f ? x + 1.f : expf(x); }
// The same function as max(x + 1, e^{-|x|}): for x <= 0, e^x >= 1 + x; for
// x > 0, e^{-x} < 1 < x + 1.  Four VALU operations (the multiply by log2 e
// takes -|x| as an input modifier; no compare and select).
__device__ __forceinline__ float elu1_fast(float x) { return fmaxf(x + 1.f, __expf(-fabsf(x))); }

// log f of an mLSTM forget gate from its pre-activation x (wikillm "Linear
// attention", Variants / mLSTM: a sigmoid forget gate, or an exponential
// one): log sigmoid(x) = min(x, 0) - log(1 + e^{-|x|}), or x itself.  The
// hardware exp2/log2 instructions serve: log(1 + y) for y = e^{-|x|} in
// (0, 1] comes within about 1e-7 absolute of log1p(y) (where 1 + y rounds to
// 1, y itself is below 6e-8), in a few instructions where the library's
// accurate exp and log1p take long range-reduction sequences.
__device__ __forceinline__ float log_forget(float x, int exp_form) {
  return exp_form ? x : fminf(x, 0.f) - __logf(1.f + __expf(-fabsf(x)));
}

// Reciprocal-like read-out factor for the three read-out forms, of a state
// held scaled by e^{-m} (m = 0 unless the mLSTM stabiliser is on); the
// output is the numerator times this factor:
//   LA_NORM_SUM  1 / (den + eps e^{-m})   = true num / (true den + eps)
//   LA_NORM_NONE e^{m}                    = true num
//   LA_NORM_MAX1 1 / max(|den|, e^{-m})   = true num / max(|true den|, 1)
__device__ __forceinline__ float readout_factor(int norm, float den, float eps, float m) {
  if (norm == LA_NORM_NONE) return expf(m);
  const float floor = expf(-m);
  if (norm == LA_NORM_MAX1) return 1.f / fmaxf(fabsf(den), floor);
  return 1.f / (den + eps * floor);
}

// Stand-in log weight of a token outside the chunk or the sequence: its
// exponential is 0 and it never raises a running maximum.
constexpr float kNoToken = -1e30f;

}  // namespace la
