// Machine-peak probes used by the benchmark to put measured denominators
// beside the published ones: a dense loop of back-to-back bf16 MFMAs, and a
// probe of how VALU and MFMA work of two waves sharing a SIMD overlap.  Not
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

// Issue-overlap probe: one workgroup of 8 waves per compute unit (the 96 KB
// of LDS it holds keeps a second one off), so waves w and w + 4 share a SIMD.
// Waves 0-3 may run an MFMA loop (2 independent 32x32x16 chains, `mf_iters`
// MFMAs each), waves 4-7 (or all 8) a VALU loop (32 independent fp32 FMA
// chains, `va_iters` FMAs each): mode 0 MFMA waves alone, 1 one VALU wave per
// SIMD, 2 two VALU waves per SIMD, 3 one MFMA and one VALU wave per SIMD.
__global__ __launch_bounds__(512) void issue_probe(int mode, int mf_iters, int va_iters,
                                                   float* sink) {
  __shared__ float pad[24 * 1024];
  const int w = threadIdx.x >> 6;
  const bool mf = (mode == 0 || mode == 3) && w < 4;
  const bool va = (mode == 1 && w >= 4) || mode == 2 || (mode == 3 && w >= 4);
  float s = 0.f;
  if (mf) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(float((threadIdx.x + i) & 7) * 0.125f);
      b[i] = static_cast<__bf16>(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
    }
    f32x16 c0, c1;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = 0.f;
    for (int it = 0; it < mf_iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r];
  }
  if (va) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = float(threadIdx.x) * 1e-3f + float(i);
    for (int it = 0; it < va_iters; ++it) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = fmaf(x[i], 0.999f, 1e-3f);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) s += x[i];
  }
  pad[threadIdx.x] = s;
  __syncthreads();
  sink[blockIdx.x * 512 + threadIdx.x] = pad[(threadIdx.x + 1) & 511];
}

}  // namespace

extern "C" {

// The issue-overlap probe above: `nblocks` workgroups of 512 threads, `sink`
// holding nblocks * 512 floats; va_iters counts 32-FMA iterations.  Returns a
// hipError_t.
int la_probe_issue(int mode, int nblocks, int mf_iters, int va_iters, float* sink, void* stream) {
  if (mode < 0 || mode > 3 || nblocks < 1 || mf_iters < 1 || va_iters < 1 || !sink)
    return int(hipErrorInvalidValue);
  issue_probe<<<dim3(unsigned(nblocks)), dim3(512), 0, static_cast<hipStream_t>(stream)>>>(
      mode, mf_iters, va_iters, sink);
  return int(hipGetLastError());
}

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
