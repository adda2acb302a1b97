// Machine-peak probes used by the benchmark to put measured denominators
// beside the published ones: a dense loop of back-to-back bf16 MFMAs.  Not
// part of the linattn ABI (built into libla_probe.so).
//
// Every wave runs CH independent accumulator chains of one MFMA shape,
// `iters` MFMAs per chain, on operands held in registers, so the matrix
// cores never wait for memory or for a dependent result; the accumulators
// are summed and stored at the end so nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int CH>
__global__ __launch_bounds__(256) void mfma_32x32x16_loop(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(float((threadIdx.x + i) & 7) * 0.125f);
    b[i] = static_cast<__bf16>(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  f32x16 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(256) void mfma_16x16x32_loop(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(float((threadIdx.x + i) & 7) * 0.125f);
    b[i] = static_cast<__bf16>(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  f32x4 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Enqueue `nblocks` workgroups of 256 threads (4 waves), each wave issuing
// CH independent chains of `iters` MFMAs: shape 0 v_mfma_f32_32x32x16_bf16
// (CH = 4), 1 v_mfma_f32_16x16x32_bf16 (CH = 8), 2 the 32x32x16 with CH = 2,
// 3 the 16x16x32 with CH = 16; `sink` holds nblocks * 256 floats.  FLOPs:
// nblocks * 4 * CH * iters * (32768 or 16384).  Returns a hipError_t.
int la_probe_mfma(int shape, int nblocks, int iters, float* sink, void* stream) {
  if (nblocks < 1 || iters < 1 || !sink) return int(hipErrorInvalidValue);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape == 0)
    mfma_32x32x16_loop<4><<<dim3(unsigned(nblocks)), dim3(256), 0, st>>>(iters, sink);
  else if (shape == 1)
    mfma_16x16x32_loop<8><<<dim3(unsigned(nblocks)), dim3(256), 0, st>>>(iters, sink);
  else if (shape == 2)   // 32x32x16 with 2 chains per wave, 8 * 32768 FLOPs per wave-iteration
    mfma_32x32x16_loop<2><<<dim3(unsigned(nblocks)), dim3(256), 0, st>>>(iters, sink);
  else if (shape == 3)   // 16x16x32 with 16 chains per wave
    mfma_16x16x32_loop<16><<<dim3(unsigned(nblocks)), dim3(256), 0, st>>>(iters, sink);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // extern "C"
