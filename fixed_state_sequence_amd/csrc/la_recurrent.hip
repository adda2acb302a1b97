// Per-token recurrent kernel: one workgroup per (b, h) state walks T tokens
// with its slice of S held in registers.  T = 1 is the decode step; T > 1 is
// the general prefill path (fp32 inputs, RFF features, widths the chunked
// MFMA kernel does not cover).
//
// Per token (llm-arch-kb "Linear Attention", section 2, causal recurrence;
// wikillm "Linear attention", Implementation sketch and Variants / RFA):
//   S <- alpha S + beta phi(k) v^T,  z <- alpha z + beta phi(k),
//   o  = phi(q)^T S / (phi(q)^T z + eps).
// With the mLSTM gates (wikillm "Linear attention", Variants / mLSTM) alpha
// is the forget gate and beta the exponential input gate; the state is held
// scaled by e^{-m}, m the log-domain running maximum
// m_t = max(log f_t + m_{t-1}, itilde_t), so the factors applied are
// e^{log f_t + m_{t-1} - m_t} and e^{itilde_t - m_t}, both <= 1.
//
// Layout of the work: the state S [d', d_v] (fp32, row-major) is cut into
// float4 column groups; thread t owns column group t % (d_v/4) of rows
// t / (d_v/4) + i * (256 / (d_v/4)).  A wave therefore reads whole rows,
// 16-byte loads, fully coalesced.  The read-out sums each thread's partial
// phi(q).S column sums with cross-lane shuffles, then across the 4 waves
// through LDS.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 256;

struct RecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* S;
  float* z;
  const float* W;
  const float* decay;
  const float* igate;   // mLSTM input-gate pre-activations
  float* stab;          // mLSTM stabiliser [B, H]
  int H, T, dh, dv, dp, D;
  int phi, decay_kind;
  int fgate_exp;        // mLSTM forget gate: sigmoid (0) or exp (1)
  int out_f32;  // out is fp32 (else the input type)
  int norm;     // read-out form (LA_NORM_*)
  int mode;     // 0 causal: update, then read out; 1 update only; 2 read-out only
  float eps;
};

template <typename DT, int NF4>
__global__ __launch_bounds__(NT) void recurrent_kernel(const RecArgs a) {
  const int64_t bh = blockIdx.x;
  const int h = int(bh % a.H);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ncg = a.dv >> 2;      // float4 column groups (a power of two <= 64)
  const int rpp = NT / ncg;       // state rows covered by one pass of the block
  const int cg = tid % ncg;
  const int r0 = tid / ncg;

  __shared__ __align__(16) float s_q[256], s_k[256], s_v[256];
  __shared__ __align__(16) float s_fq[256], s_fk[256];
  __shared__ __align__(16) float s_red[NT / 64][260];

  float* Sg = a.S + bh * a.dp * a.dv;
  float* zg = a.z + bh * a.dp;

  float4 st[NF4];
#pragma unroll
  for (int i = 0; i < NF4; ++i) {
    const int f = r0 + i * rpp;
    st[i] = f < a.dp ? *reinterpret_cast<const float4*>(Sg + int64_t(f) * a.dv + 4 * cg)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float zr = tid < a.dp ? zg[tid] : 0.f;

  const DT* qg = static_cast<const DT*>(a.q) + bh * int64_t(a.T) * a.dh;
  const DT* kg = static_cast<const DT*>(a.k) + bh * int64_t(a.T) * a.dh;
  const DT* vg = static_cast<const DT*>(a.v) + bh * int64_t(a.T) * a.dv;
  DT* og = static_cast<DT*>(a.out) + bh * int64_t(a.T) * a.dv;
  float* ogf = static_cast<float*>(a.out) + bh * int64_t(a.T) * a.dv;
  const float* dg = a.decay ? a.decay + bh * int64_t(a.T) : nullptr;
  const float* ig = a.igate ? a.igate + bh * int64_t(a.T) : nullptr;
  const float rsD = a.D > 0 ? 1.0f / sqrtf(float(a.D)) : 0.f;
  const bool mlstm = a.decay_kind == LA_GATE_MLSTM;
  float m = mlstm ? a.stab[bh] : 0.f;   // stabiliser (0: the state is unscaled)

  for (int t = 0; t < a.T; ++t) {
    if (tid < a.dh) {
      s_q[tid] = to_f32(qg[int64_t(t) * a.dh + tid]);
      s_k[tid] = to_f32(kg[int64_t(t) * a.dh + tid]);
    }
    if (tid < a.dv) s_v[tid] = to_f32(vg[int64_t(t) * a.dv + tid]);
    float alpha = 1.f, beta = 1.f;
    if (a.decay_kind == LA_DECAY_SSD) {
      alpha = dg[t];
    } else if (a.decay_kind == LA_GATE_RFA) {
      alpha = dg[t];
      beta = 1.f - alpha;
    } else if (mlstm) {
      const float lf = log_forget(dg[t], a.fgate_exp), it = ig[t];
      const float mn = fmaxf(lf + m, it);
      alpha = expf(lf + m - mn);
      beta = expf(it - mn);
      m = mn;
    }
    __syncthreads();

    if (a.phi == LA_PHI_ELU1) {
      if (tid < a.dp) {
        s_fq[tid] = elu1_accurate(s_q[tid]);
        s_fk[tid] = elu1_accurate(s_k[tid]);
      }
    } else if (a.phi == LA_PHI_IDENTITY) {
      if (tid < a.dp) {
        s_fq[tid] = s_q[tid];
        s_fk[tid] = s_k[tid];
      }
    } else {
      // phi(x) = D^{-1/2} [sin(W_h x); cos(W_h x)]: thread j < D projects q,
      // thread D <= j < 2D projects k.
      for (int j = tid; j < 2 * a.D; j += NT) {
        const int jj = j < a.D ? j : j - a.D;
        const float* x = j < a.D ? s_q : s_k;
        const float* w = a.W + (int64_t(h) * a.D + jj) * a.dh;
        float acc = 0.f;
        for (int i = 0; i < a.dh; ++i) acc = fmaf(w[i], x[i], acc);
        float sn, cs;
        sincosf(acc, &sn, &cs);
        float* dst = j < a.D ? s_fq : s_fk;
        dst[jj] = sn * rsD;
        dst[a.D + jj] = cs * rsD;
      }
    }
    __syncthreads();

    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + 4 * cg);
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      const int f = r0 + i * rpp;
      if (f < a.dp) {
        if (a.mode != 2) {
          const float kb = beta * s_fk[f];
          st[i].x = alpha * st[i].x + kb * v4.x;
          st[i].y = alpha * st[i].y + kb * v4.y;
          st[i].z = alpha * st[i].z + kb * v4.z;
          st[i].w = alpha * st[i].w + kb * v4.w;
        }
        const float qf = s_fq[f];
        num.x += qf * st[i].x;
        num.y += qf * st[i].y;
        num.z += qf * st[i].z;
        num.w += qf * st[i].w;
      }
    }
    float dpart = 0.f;
    if (tid < a.dp) {
      if (a.mode != 2) zr = alpha * zr + beta * s_fk[tid];
      dpart = s_fq[tid] * zr;
    }
    for (int off = ncg; off < 64; off <<= 1) {
      num.x += __shfl_xor(num.x, off);
      num.y += __shfl_xor(num.y, off);
      num.z += __shfl_xor(num.z, off);
      num.w += __shfl_xor(num.w, off);
    }
    for (int off = 32; off >= 1; off >>= 1) dpart += __shfl_xor(dpart, off);
    if (lane < ncg) *reinterpret_cast<float4*>(&s_red[wave][4 * cg]) = num;
    if (lane == 0) s_red[wave][256] = dpart;
    __syncthreads();
    if (tid < a.dv && a.mode != 1) {
      float n = 0.f, d = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) {
        n += s_red[w][tid];
        d += s_red[w][256];
      }
      const float o = a.norm == LA_NORM_SUM && !mlstm ? n / (d + a.eps)
                                                      : n * readout_factor(a.norm, d, a.eps, m);
      if (a.out_f32) ogf[int64_t(t) * a.dv + tid] = o;
      else store_f32(o, og + int64_t(t) * a.dv + tid);
    }
  }

#pragma unroll
  for (int i = 0; i < NF4; ++i) {
    const int f = r0 + i * rpp;
    if (f < a.dp) *reinterpret_cast<float4*>(Sg + int64_t(f) * a.dv + 4 * cg) = st[i];
  }
  if (tid < a.dp) zg[tid] = zr;
  if (mlstm && tid == 0) a.stab[bh] = m;
}

int passes(int dp, int dv) {
  const int ncg = dv / 4;
  const int rpp = NT / ncg;
  return (dp + rpp - 1) / rpp;
}

template <typename DT>
hipError_t launch_dt(const RecArgs& a, int64_t nbh, hipStream_t st) {
  const int np = passes(a.dp, a.dv);
  const dim3 grid{unsigned(nbh)}, block{unsigned(NT)};
  if (np <= 1) recurrent_kernel<DT, 1><<<grid, block, 0, st>>>(a);
  else if (np <= 2) recurrent_kernel<DT, 2><<<grid, block, 0, st>>>(a);
  else if (np <= 4) recurrent_kernel<DT, 4><<<grid, block, 0, st>>>(a);
  else if (np <= 8) recurrent_kernel<DT, 8><<<grid, block, 0, st>>>(a);
  else if (np <= 16) recurrent_kernel<DT, 16><<<grid, block, 0, st>>>(a);
  else recurrent_kernel<DT, 32><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool recurrent_supported(int dh, int dp, int dv) {
  if (dh < 1 || dh > 256 || dp < 1 || dp > 256 || dv < 4 || dv > 256 || dv % 4) return false;
  const int ncg = dv / 4;
  if (ncg & (ncg - 1)) return false;
  return passes(dp, dv) <= 32;
}

hipError_t launch_recurrent(const Problem& p, const void* q, const void* k, const void* v,
                            float* S, float* z, void* out, hipStream_t stream) {
  RecArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.S = S; a.z = z;
  a.W = p.W; a.decay = p.decay; a.igate = p.igate; a.stab = p.stab;
  a.H = p.H; a.T = p.T; a.dh = p.dh; a.dv = p.dv; a.dp = p.dp; a.D = p.D;
  a.phi = int(p.phi); a.decay_kind = int(p.decay_kind); a.eps = p.eps;
  a.fgate_exp = p.fgate_exp;
  a.norm = p.norm;
  a.out_f32 = p.out_dtype == LA_F32 ? 1 : 0;
  // non-causal: the whole sequence into the state first, then every token
  // reads it out ([kb] section 3, non-causal sketch)
  const int modes[2][2] = {{0, -1}, {1, 2}};
  for (int m : modes[p.noncausal ? 1 : 0]) {
    if (m < 0) break;
    a.mode = m;
    hipError_t e = hipErrorInvalidValue;
    switch (p.dtype) {
      case LA_F32: e = launch_dt<float>(a, p.BH(), stream); break;
      case LA_BF16: e = launch_dt<bf16_t>(a, p.BH(), stream); break;
      case LA_F16: e = launch_dt<f16_t>(a, p.BH(), stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- state init

namespace {
// Zero n floats at p: 16-byte stores over the 16-byte-aligned body, scalar
// stores for the tail (p itself is 4-byte aligned at least).
__device__ __forceinline__ void zero_range(float* p, int64_t n, int64_t i0, int64_t stride) {
  const int64_t head = p ? min(int64_t((16 - (reinterpret_cast<uintptr_t>(p) & 15)) & 15) / 4, n) : 0;
  const int64_t n4 = (n - head) / 4;
  float4* q = reinterpret_cast<float4*>(p + head);
  for (int64_t i = i0; i < n4; i += stride) q[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = i0; i < head; i += stride) p[i] = 0.f;
  for (int64_t i = head + 4 * n4 + i0; i < n; i += stride) p[i] = 0.f;
}

__global__ void fill_zero_kernel(float* S, int64_t nS, float* z, int64_t nz, float* m,
                                 int64_t nm) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  zero_range(S, nS, i0, stride);
  zero_range(z, nz, i0, stride);
  zero_range(m, nm, i0, stride);
}
}  // namespace

hipError_t launch_state_init(float* S, int64_t nS, float* z, int64_t nz, float* m, int64_t nm,
                             hipStream_t stream) {
  int64_t blocks = (nS / 4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  fill_zero_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(S, nS, z, nz, m, nm);
  return hipGetLastError();
}

}  // namespace la
