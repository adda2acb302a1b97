// Gradients of the causal prefill, one workgroup per (b, h) sequence with the
// state slice held in registers (the layout of the per-token forward kernel).
//
// With L = sum_t <dout_t, o_t> and the read-out o_t = num_t / D_t
// (num_t = S_t^T phi(q_t), D_t = phi(q_t).z_t + eps; or num_t alone; or
// num_t / max(|phi(q_t).z_t|, 1)), the recurrence S_t = alpha_t S_{t-1} +
// beta_t phi(k_t) v_t^T (llm-arch-kb "Linear Attention", section 2; wikillm
// "Linear attention", Implementation sketch, SSD and RFA) gives, in reverse
// mode:
//   g_num_t = dout_t / D_t,  g_den_t = -(dout_t . o_t) / D_t   (read-out)
//   dphi(q_t) = S_t g_num_t + z_t g_den_t
//   G_t = alpha_{t+1} G_{t+1} + phi(q_t) g_num_t^T,  g_t likewise with g_den
//   dphi(k_t) = beta_t (G_t v_t + g_t),  dv_t = beta_t G_t^T phi(k_t)
//   dS0 = alpha_0 G_0,  dz0 = alpha_0 g_0.
// The decay enters through the log-prefix l_t = sum_{r<=t} log alpha_r:
// every weight is e^{l_t - l_s} beta_s, so dL/dl_t = <phi(q_t), dphi(q_t)> -
// <phi(k_t), dphi(k_t)> and dL/dlog alpha_r = sum_{t>=r} dL/dl_t, a suffix sum
// kept during the reverse pass; beta's own gradient is phi(k_t).(G_t v_t + g_t).
// dL/dalpha_r is that sum over alpha_r, except for decays below kDecayExact,
// whose gradient decay_exact_kernel forms as <G_r, S_{r-1}> + <g_r, z_{r-1}>.
//
// mLSTM gates (wikillm "Linear attention", Variants / mLSTM): the state is
// held scaled by e^{-m_t} as in the forward, S'_t = alpha'_t S'_{t-1} +
// beta'_t k_t v_t^T with alpha'_t = e^{log f_t + m_{t-1} - m_t} and beta'_t =
// e^{itilde_t - m_t}, and the read-out of the scaled state (readout_factor)
// gives g'_num = e^{m_t} g_num, so the gradient state carried back is
// G'_t = e^{m_t} G_t: the same two passes with (alpha', beta') and bounded
// numbers throughout.  L depends on the gates through the true alpha_t =
// f_t and beta_t = e^{itilde_t}: dL/dlog f_r is the suffix sum above
// (times 1 - f_r for the sigmoid gate's pre-activation, 1 for the
// exponential one) and dL/ditilde_t = beta'_t k_t . (G'_t v_t + g'_t).
//
// Pass A walks t forward: it rebuilds S_t and z_t, the read-out, g_num,
// g_den and dq, and leaves g_num_t, g_den_t and <phi(q_t), dphi(q_t)> in the
// workspace (with the mLSTM gates also alpha'_t and beta'_t).  Pass B walks t backward carrying G, g.  The efficient-attention
// lesson ("Implementation reality") trains with the chunked form; this
// token-serial kernel is the exact reference-grade path for every supported
// configuration.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 256;

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* S0;   // initial state or null (zero)
  const float* z0;
  const float* decay;
  float* dq;
  float* dk;
  float* dv;
  float* ddecay;     // [BH, T] or null (mLSTM: dL/dfgate)
  const float* igate;   // mLSTM input-gate pre-activations [BH, T]
  const float* stab;    // mLSTM stabiliser of the start state [BH] (read with S0)
  float* digate;        // mLSTM dL/digate [BH, T]
  int fgate_exp;
  float* dS0;        // [BH, dp, dv] or null
  float* dz0;
  float* ws;         // [BH, T, dv + 2]
  int H, T, dh, dv_, dp;
  int phi, decay_kind, norm;
  int dout_f32;      // dout is fp32 (else the input type)
  float eps;
};

__device__ __forceinline__ float phi_of(float x, int phi) {
  return phi == LA_PHI_IDENTITY ? x : elu1_accurate(x);
}
// derivative: elu+1 has slope 1 above 0 and e^x below; the identity 1
__device__ __forceinline__ float dphi_of(float x, int phi) {
  return phi == LA_PHI_IDENTITY ? 1.f : (x > 0.f ? 1.f : expf(x));
}

template <typename DT>
__device__ __forceinline__ float load_dout(const BwdArgs& a, int64_t i) {
  return a.dout_f32 ? static_cast<const float*>(a.dout)[i] : to_f32(static_cast<const DT*>(a.dout)[i]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename DT, int NF4>
__global__ __launch_bounds__(NT) void backward_kernel(const BwdArgs a) {
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ncg = a.dv_ >> 2;     // float4 column groups (a power of two <= 64)
  const int rpp = NT / ncg;       // state rows covered by one pass of the block
  const int cg = tid % ncg;
  const int r0 = tid / ncg;

  __shared__ __align__(16) float s_q[256], s_k[256], s_v[256], s_do[256];
  __shared__ __align__(16) float s_fq[256], s_fk[256], s_gn[256], s_part[256];
  __shared__ __align__(16) float s_red[NT / 64][260];
  __shared__ float s_sc[NT / 64][4];

  const int64_t T = a.T;
  const DT* qg = static_cast<const DT*>(a.q) + bh * T * a.dh;
  const DT* kg = static_cast<const DT*>(a.k) + bh * T * a.dh;
  const DT* vg = static_cast<const DT*>(a.v) + bh * T * a.dv_;
  const int64_t do0 = bh * T * a.dv_;
  const float* dg = a.decay ? a.decay + bh * T : nullptr;
  const bool ml = a.decay_kind == LA_GATE_MLSTM;
  const float* ig = ml ? a.igate + bh * T : nullptr;
  // per token: g_num (d_v), g_den, <phi(q), dphi(q)>; mLSTM also alpha', beta'
  const int wst = a.dv_ + (ml ? 4 : 2);
  float* wsg = a.ws + bh * T * wst;

  auto coeffs = [&](int64_t t, float& al, float& be) {
    al = 1.f;
    be = 1.f;
    if (a.decay_kind == LA_DECAY_SSD) {
      al = dg[t];
    } else if (a.decay_kind == LA_GATE_RFA) {
      al = dg[t];
      be = 1.f - al;
    }
  };

  // ------------------------------------------------------------- pass A
  float4 st[NF4];
#pragma unroll
  for (int i = 0; i < NF4; ++i) {
    const int f = r0 + i * rpp;
    st[i] = (a.S0 && f < a.dp) ? *reinterpret_cast<const float4*>(a.S0 + (bh * a.dp + f) * a.dv_ + 4 * cg)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float zr = (a.z0 && tid < a.dp) ? a.z0[bh * a.dp + tid] : 0.f;
  float m = (ml && a.S0) ? a.stab[bh] : 0.f;   // mLSTM stabiliser (a zero start state has m = 0)

  for (int64_t t = 0; t < T; ++t) {
    if (tid < a.dh) {
      s_q[tid] = to_f32(qg[t * a.dh + tid]);
      s_k[tid] = to_f32(kg[t * a.dh + tid]);
    }
    if (tid < a.dv_) {
      s_v[tid] = to_f32(vg[t * a.dv_ + tid]);
      s_do[tid] = load_dout<DT>(a, do0 + t * a.dv_ + tid);
    }
    float alpha, beta;
    if (ml) {
      const float lf = log_forget(dg[t], a.fgate_exp), it = ig[t];
      const float mn = fmaxf(lf + m, it);
      alpha = expf(lf + m - mn);
      beta = expf(it - mn);
      m = mn;
    } else {
      coeffs(t, alpha, beta);
    }
    __syncthreads();
    if (tid < a.dp) {
      s_fq[tid] = phi_of(s_q[tid], a.phi);
      s_fk[tid] = phi_of(s_k[tid], a.phi);
    }
    __syncthreads();
    // update and numerator partials
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + 4 * cg);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      const int f = r0 + i * rpp;
      if (f < a.dp) {
        const float kb = beta * s_fk[f];
        st[i].x = alpha * st[i].x + kb * v4.x;
        st[i].y = alpha * st[i].y + kb * v4.y;
        st[i].z = alpha * st[i].z + kb * v4.z;
        st[i].w = alpha * st[i].w + kb * v4.w;
        const float qf = s_fq[f];
        num.x += qf * st[i].x;
        num.y += qf * st[i].y;
        num.z += qf * st[i].z;
        num.w += qf * st[i].w;
      }
    }
    float dpart = 0.f;
    if (tid < a.dp) {
      zr = alpha * zr + beta * s_fk[tid];
      dpart = s_fq[tid] * zr;
    }
    for (int off = ncg; off < 64; off <<= 1) {
      num.x += __shfl_xor(num.x, off);
      num.y += __shfl_xor(num.y, off);
      num.z += __shfl_xor(num.z, off);
      num.w += __shfl_xor(num.w, off);
    }
    dpart = wave_sum(dpart);
    if (lane < ncg) *reinterpret_cast<float4*>(&s_red[wave][4 * cg]) = num;
    if (lane == 0) s_red[wave][256] = dpart;
    __syncthreads();
    // read-out: divisor, output, g_num and the dot product dout . o
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) den += s_red[w][256];
    // o = num * scale, g_num = dout * scale (of the scaled state with the
    // mLSTM gates: e^{m} times the true g_num)
    const float scale = readout_factor(a.norm, den, a.eps, m);
    const float floor_ = ml ? expf(-m) : 1.f;   // the max1 read-out's floor in the state's scale
    float pv = 0.f;
    if (tid < a.dv_) {
      float n = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) n += s_red[w][tid];
      const float o = n * scale;
      s_gn[tid] = s_do[tid] * scale;
      pv = s_do[tid] * o;
    }
    pv = wave_sum(pv);
    if (lane == 0) s_sc[wave][0] = pv;
    __syncthreads();
    float dot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) dot += s_sc[w][0];
    float gden;
    if (a.norm == LA_NORM_NONE) gden = 0.f;
    else if (a.norm == LA_NORM_MAX1) gden = fabsf(den) > floor_ ? -copysignf(1.f, den) * dot * scale : 0.f;
    else gden = -dot * scale;
    // dphi(q_t) = S_t g_num + z_t g_den: the S part summed over the column groups
    const float4 gn4 = *reinterpret_cast<const float4*>(s_gn + 4 * cg);
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      float p = st[i].x * gn4.x + st[i].y * gn4.y + st[i].z * gn4.z + st[i].w * gn4.w;
      for (int off = 1; off < ncg; off <<= 1) p += __shfl_xor(p, off);
      const int f = r0 + i * rpp;
      if (cg == 0 && f < a.dp) s_part[f] = p;
    }
    __syncthreads();
    float qd = 0.f;
    if (tid < a.dp) {
      const float dfq = s_part[tid] + zr * gden;
      a.dq[(bh * T + t) * a.dh + tid] = dfq * dphi_of(s_q[tid], a.phi);
      qd = s_fq[tid] * dfq;
    }
    if (tid < a.dv_) wsg[t * wst + tid] = s_gn[tid];
    qd = wave_sum(qd);
    if (lane == 0) s_sc[wave][1] = qd;
    __syncthreads();
    if (tid == 0) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) s += s_sc[w][1];
      wsg[t * wst + a.dv_] = gden;
      wsg[t * wst + a.dv_ + 1] = s;
      if (ml) {
        wsg[t * wst + a.dv_ + 2] = alpha;
        wsg[t * wst + a.dv_ + 3] = beta;
      }
    }
  }
  __syncthreads();   // pass A's workspace rows visible to every thread

  // ------------------------------------------------------------- pass B
#pragma unroll
  for (int i = 0; i < NF4; ++i) st[i] = make_float4(0.f, 0.f, 0.f, 0.f);   // G
  float gr = 0.f;                                                          // g
  float R = 0.f;    // suffix sum of dL/dl_t
  float alpha_next = 0.f;
  for (int64_t t = T - 1; t >= 0; --t) {
    if (tid < a.dh) {
      s_q[tid] = to_f32(qg[t * a.dh + tid]);
      s_k[tid] = to_f32(kg[t * a.dh + tid]);
    }
    if (tid < a.dv_) {
      s_v[tid] = to_f32(vg[t * a.dv_ + tid]);
      s_gn[tid] = wsg[t * wst + tid];
    }
    const float gden = wsg[t * wst + a.dv_];
    const float qdq = wsg[t * wst + a.dv_ + 1];
    float alpha, beta;
    if (ml) {
      alpha = wsg[t * wst + a.dv_ + 2];
      beta = wsg[t * wst + a.dv_ + 3];
    } else {
      coeffs(t, alpha, beta);
    }
    __syncthreads();
    if (tid < a.dp) {
      s_fq[tid] = phi_of(s_q[tid], a.phi);
      s_fk[tid] = phi_of(s_k[tid], a.phi);
    }
    __syncthreads();
    // G_t = alpha_{t+1} G_{t+1} + phi(q_t) g_num_t^T; then G_t v_t (per row)
    // and G_t^T phi(k_t) (per column) partials
    const float4 gn4 = *reinterpret_cast<const float4*>(s_gn + 4 * cg);
    const float4 v4 = *reinterpret_cast<const float4*>(s_v + 4 * cg);
    float4 dvp = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      const int f = r0 + i * rpp;
      const float qf = f < a.dp ? s_fq[f] : 0.f;
      const float kf = f < a.dp ? s_fk[f] : 0.f;
      st[i].x = alpha_next * st[i].x + qf * gn4.x;
      st[i].y = alpha_next * st[i].y + qf * gn4.y;
      st[i].z = alpha_next * st[i].z + qf * gn4.z;
      st[i].w = alpha_next * st[i].w + qf * gn4.w;
      float p = st[i].x * v4.x + st[i].y * v4.y + st[i].z * v4.z + st[i].w * v4.w;
      for (int off = 1; off < ncg; off <<= 1) p += __shfl_xor(p, off);
      if (cg == 0 && f < a.dp) s_part[f] = p;
      dvp.x += kf * st[i].x;
      dvp.y += kf * st[i].y;
      dvp.z += kf * st[i].z;
      dvp.w += kf * st[i].w;
    }
    if (tid < a.dp) gr = alpha_next * gr + s_fq[tid] * gden;
    for (int off = ncg; off < 64; off <<= 1) {
      dvp.x += __shfl_xor(dvp.x, off);
      dvp.y += __shfl_xor(dvp.y, off);
      dvp.z += __shfl_xor(dvp.z, off);
      dvp.w += __shfl_xor(dvp.w, off);
    }
    if (lane < ncg) *reinterpret_cast<float4*>(&s_red[wave][4 * cg]) = dvp;
    __syncthreads();
    float kd = 0.f;
    if (tid < a.dp) {
      const float raw = s_part[tid] + gr;       // G_t v_t + g_t
      a.dk[(bh * T + t) * a.dh + tid] = beta * raw * dphi_of(s_k[tid], a.phi);
      kd = s_fk[tid] * raw;
    }
    if (tid < a.dv_) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) s += s_red[w][tid];
      a.dv[(bh * T + t) * a.dv_ + tid] = beta * s;
    }
    kd = wave_sum(kd);
    if (lane == 0) s_sc[wave][2] = kd;
    __syncthreads();
    float kdk = 0.f;   // phi(k_t) . (G_t v_t + g_t), the gradient of beta_t
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) kdk += s_sc[w][2];
    R += qdq - beta * kdk;
    if (tid == 0 && a.ddecay) {
      if (ml) {
        // R = dL/dlog f_t; 1 - sigmoid(x) = 1 / (1 + e^x)
        a.ddecay[bh * T + t] = a.fgate_exp ? R : R / (1.f + expf(dg[t]));
        a.digate[bh * T + t] = beta * kdk;
      } else {
        // near-zero decays: the exact term is added by decay_exact_kernel
        const float da = alpha < kDecayExact ? 0.f : R / alpha;
        if (a.decay_kind == LA_DECAY_SSD) a.ddecay[bh * T + t] = da;
        else if (a.decay_kind == LA_GATE_RFA) a.ddecay[bh * T + t] = da - kdk;
      }
    }
    alpha_next = alpha;
  }
  // the start state enters S_0 as alpha_0 S0
  if (a.dS0) {
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      const int f = r0 + i * rpp;
      if (f < a.dp) {
        float4 x = st[i];
        x.x *= alpha_next; x.y *= alpha_next; x.z *= alpha_next; x.w *= alpha_next;
        *reinterpret_cast<float4*>(a.dS0 + (bh * a.dp + f) * a.dv_ + 4 * cg) = x;
      }
    }
    if (tid < a.dp) a.dz0[bh * a.dp + tid] = alpha_next * gr;
  }
}

// ------------------------------------------------ exact decay gradient

// dL/dalpha_r = <G_r, S_{r-1}> + <gz_r, z_{r-1}> for every token r whose
// decay (or gate) is below kDecayExact: the state before r multiplies
// alpha_r in S_r = alpha_r S_{r-1} + beta_r phi(k_r) v_r^T (wikillm "Linear
// attention", Implementation sketch), and G_r is the gradient of S_r.
// Written out,
//   <G_r, S_{r-1}> = sum_{t >= r} w_t phi(q_t)^T S_{r-1} g_t,
//   w_t = prod_{r' = r+1..t} alpha_r',
// so one workgroup walks the segment forward: it builds S_{r-1} by the
// recurrence from the segment's start state (or from the last exact reset
// before r, where the state restarts from zero), then reads it out against
// every later query of the segment with weight w_t (up to the next exact
// reset, where w drops to 0), and adds w at the segment's end times the
// state product with the gradient state carried in from later segments.
// One workgroup per (b, h) and tile of 256 tokens; a tile with no such token
// returns at once.  The result is added to dd[r], which holds the gate's
// beta term (or 0).
constexpr int XT = 32;    // tokens staged in LDS at a time

int passes(int dp, int dv);

template <typename DT, int NF4>
__global__ __launch_bounds__(NT) void decay_exact_kernel(const DecayExactArgs a, int ntile) {
  const int64_t bh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const int tid = threadIdx.x;
  const int ncg = a.dv >> 2;
  const int rpp = NT / ncg;
  const int cg = tid % ncg;
  const int r0 = tid / ncg;
  const int64_t T = a.T;
  const float* al = a.decay + bh * T;

  __shared__ int s_list[NT];
  __shared__ int s_n;
  __shared__ __align__(16) float s_x[XT][256];   // phi(k) or phi(q)
  __shared__ __align__(16) float s_y[XT][256];   // v or g
  __shared__ float s_al[XT], s_be[XT], s_h[XT];
  __shared__ float s_red[NT / 64];
  __shared__ int s_ired[NT / 64];

  if (tid == 0) s_n = 0;
  __syncthreads();
  {
    const int64_t t = int64_t(tile) * NT + tid;
    if (t < T && al[t] < kDecayExact) s_list[atomicAdd(&s_n, 1)] = int(t);
  }
  __syncthreads();
  const int nflag = s_n;

  const DT* qg = static_cast<const DT*>(a.q) + bh * T * a.dh;
  const DT* kg = static_cast<const DT*>(a.k) + bh * T * a.dh;
  const DT* vg = static_cast<const DT*>(a.v) + bh * T * a.dv;
  auto phi = [&](float x) { return a.phi == LA_PHI_IDENTITY ? x : elu1_accurate(x); };
  auto beta_of = [&](float x) { return a.decay_kind == LA_GATE_RFA ? 1.f - x : 1.f; };
  // block-wide max of an int (every thread gets it)
  auto block_max = [&](int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
    __syncthreads();
    if ((tid & 63) == 0) s_ired[tid >> 6] = x;
    __syncthreads();
    int m = s_ired[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = max(m, s_ired[w]);
    return m;
  };

  for (int fi = 0; fi < nflag; ++fi) {
    const int r = s_list[fi];
    const int seg = r / a.seg_len;
    const int seg0 = seg * a.seg_len;
    const int seg1 = min(seg0 + a.seg_len, a.T) - 1;
    // the last exact reset before r within the segment (the state restarts there)
    int s_begin = -1;
    for (int base = r - 1; base >= seg0 && s_begin < 0; base -= NT) {
      const int t = base - tid;
      s_begin = block_max(t >= seg0 && al[t] == 0.f ? t : -1);
    }
    // the first exact reset after r (later queries get weight 0)
    int t_end = seg1;
    for (int base = r + 1; base <= seg1; base += NT) {
      const int t = base + tid;
      const int z = block_max(t <= seg1 && al[t] == 0.f ? -t : -(1 << 30));
      if (z > -(1 << 30)) {
        t_end = -z - 1;
        break;
      }
    }
    // the state before s_begin: zero after a reset, else the segment's start
    float4 st[NF4];
    float zr = 0.f;
    const bool from_start = s_begin < 0;
    if (from_start) s_begin = seg0;
#pragma unroll
    for (int i = 0; i < NF4; ++i) {
      const int f = r0 + i * rpp;
      st[i] = (from_start && a.S0 && f < a.dp)
                  ? *reinterpret_cast<const float4*>(a.S0 + bh * a.s_bh + seg * a.s_seg +
                                                     int64_t(f) * a.dv + 4 * cg)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (from_start && a.z0 && tid < a.dp) zr = a.z0[bh * a.z_bh + seg * a.s_seg + tid];

    // stage tokens [t0, t0 + n): x = phi(k) (update) or phi(q) (read-out);
    // y = v or g; alpha, beta and h
    auto stage = [&](int t0, int n, bool update) {
      __syncthreads();   // the previous block's reads done
      const DT* xg = update ? kg : qg;
      for (int i = tid; i < n * a.dh; i += NT) {
        const int j = i / a.dh, f = i % a.dh;
        s_x[j][f] = phi(to_f32(xg[int64_t(t0 + j) * a.dh + f]));
      }
      for (int i = tid; i < n * a.dv; i += NT) {
        const int j = i / a.dv, c = i % a.dv;
        const int64_t row = bh * T + t0 + j;
        float y;
        if (update) {
          y = to_f32(vg[int64_t(t0 + j) * a.dv + c]);
        } else if (a.mode == 0) {
          const float dv = a.dout_f32 ? static_cast<const float*>(a.dout)[row * a.dv + c]
                                      : to_f32(static_cast<const DT*>(a.dout)[row * a.dv + c]);
          y = a.tok[2 * row] * dv;
        } else {
          y = a.ws[row * (a.dv + 2) + c];
        }
        s_y[j][c] = y;
      }
      if (tid < n) {
        const int64_t row = bh * T + t0 + tid;
        s_al[tid] = al[t0 + tid];
        s_be[tid] = beta_of(al[t0 + tid]);
        if (!update) s_h[tid] = a.mode == 0 ? a.tok[2 * row + 1] : a.ws[row * (a.dv + 2) + a.dv];
      }
      __syncthreads();
    };

    // S_{r-1}, z_{r-1}: the recurrence over [s_begin, r)
    for (int t0 = s_begin; t0 < r; t0 += XT) {
      const int n = min(XT, r - t0);
      stage(t0, n, true);
      for (int j = 0; j < n; ++j) {
        const float alpha = s_al[j], beta = s_be[j];
        const float4 v4 = *reinterpret_cast<const float4*>(&s_y[j][4 * cg]);
#pragma unroll
        for (int i = 0; i < NF4; ++i) {
          const int f = r0 + i * rpp;
          if (f < a.dp) {
            const float kb = beta * s_x[j][f];
            st[i].x = fmaf(alpha, st[i].x, kb * v4.x);
            st[i].y = fmaf(alpha, st[i].y, kb * v4.y);
            st[i].z = fmaf(alpha, st[i].z, kb * v4.z);
            st[i].w = fmaf(alpha, st[i].w, kb * v4.w);
          }
        }
        if (tid < a.dp) zr = fmaf(alpha, zr, beta * s_x[j][tid]);
      }
    }
    // sum_{t = r..t_end} w_t (phi(q_t)^T S_{r-1} g_t + phi(q_t) . z_{r-1} h_t)
    float acc = 0.f, w = 1.f;
    for (int t0 = r; t0 <= t_end; t0 += XT) {
      const int n = min(XT, t_end + 1 - t0);
      stage(t0, n, false);
      for (int j = 0; j < n; ++j) {
        if (t0 + j > r) w *= s_al[j];
        const float4 g4 = *reinterpret_cast<const float4*>(&s_y[j][4 * cg]);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < NF4; ++i) {
          const int f = r0 + i * rpp;
          if (f < a.dp) {
            const float sg = st[i].x * g4.x + st[i].y * g4.y + st[i].z * g4.z + st[i].w * g4.w;
            p = fmaf(s_x[j][f], sg, p);
          }
        }
        if (tid < a.dp) p = fmaf(s_x[j][tid] * zr, s_h[j], p);
        acc = fmaf(w, p, acc);
      }
    }
    // the gradient state carried in from beyond the segment's end
    if (t_end == seg1 && a.gafter) {
      const float* G = a.gafter + (bh * a.nseg + seg) * (int64_t(a.dp) * a.dv + a.dp);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < NF4; ++i) {
        const int f = r0 + i * rpp;
        if (f < a.dp) {
          const float4 g4 = *reinterpret_cast<const float4*>(G + int64_t(f) * a.dv + 4 * cg);
          p += st[i].x * g4.x + st[i].y * g4.y + st[i].z * g4.z + st[i].w * g4.w;
        }
      }
      if (tid < a.dp) p = fmaf(G[int64_t(a.dp) * a.dv + tid], zr, p);
      acc = fmaf(w, p, acc);
    }
    acc = wave_sum(acc);
    __syncthreads();
    if ((tid & 63) == 0) s_red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < NT / 64; ++ww) x += s_red[ww];
      a.dd[bh * T + r] += x;
    }
  }
}

template <typename DT>
hipError_t launch_exact_dt(const DecayExactArgs& a, int64_t BH, hipStream_t st) {
  const int np = passes(a.dp, a.dv);
  const int ntile = (a.T + NT - 1) / NT;
  const dim3 grid{unsigned(BH * ntile)}, block{unsigned(NT)};
  if (np <= 1) decay_exact_kernel<DT, 1><<<grid, block, 0, st>>>(a, ntile);
  else if (np <= 2) decay_exact_kernel<DT, 2><<<grid, block, 0, st>>>(a, ntile);
  else if (np <= 4) decay_exact_kernel<DT, 4><<<grid, block, 0, st>>>(a, ntile);
  else if (np <= 8) decay_exact_kernel<DT, 8><<<grid, block, 0, st>>>(a, ntile);
  else if (np <= 16) decay_exact_kernel<DT, 16><<<grid, block, 0, st>>>(a, ntile);
  else decay_exact_kernel<DT, 32><<<grid, block, 0, st>>>(a, ntile);
  return hipGetLastError();
}

int passes(int dp, int dv) {
  const int ncg = dv / 4;
  const int rpp = NT / ncg;
  return (dp + rpp - 1) / rpp;
}

template <typename DT>
hipError_t launch_dt(const BwdArgs& a, int64_t nbh, hipStream_t st) {
  const int np = passes(a.dp, a.dv_);
  const dim3 grid{unsigned(nbh)}, block{unsigned(NT)};
  if (np <= 1) backward_kernel<DT, 1><<<grid, block, 0, st>>>(a);
  else if (np <= 2) backward_kernel<DT, 2><<<grid, block, 0, st>>>(a);
  else if (np <= 4) backward_kernel<DT, 4><<<grid, block, 0, st>>>(a);
  else if (np <= 8) backward_kernel<DT, 8><<<grid, block, 0, st>>>(a);
  else if (np <= 16) backward_kernel<DT, 16><<<grid, block, 0, st>>>(a);
  else backward_kernel<DT, 32><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decay_exact(const DecayExactArgs& a, la_dtype dtype, int64_t BH,
                              hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  switch (dtype) {
    case LA_F32: return launch_exact_dt<float>(a, BH, stream);
    case LA_BF16: return launch_exact_dt<bf16_t>(a, BH, stream);
    case LA_F16: return launch_exact_dt<f16_t>(a, BH, stream);
  }
  return hipErrorInvalidValue;
}

bool backward_supported(const Problem& p) {
  return (p.phi == LA_PHI_ELU1 || p.phi == LA_PHI_IDENTITY) && p.dp == p.dh &&
         !p.noncausal && recurrent_supported(p.dh, p.dp, p.dv);
}

size_t backward_workspace_bytes(const Problem& p) {
  if (backward_chunked(p)) return backward_chunked_workspace_bytes(p);
  const int per_token = p.dv + (p.decay_kind == LA_GATE_MLSTM ? 4 : 2);
  return size_t(p.BH()) * size_t(p.T) * size_t(per_token) * sizeof(float);
}

hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v,
                           const float* S0, const float* z0, const void* dout, float* dq,
                           float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                           void* ws, hipStream_t stream) {
  if (backward_chunked(p))
    return launch_backward_chunked(p, q, k, v, S0, z0, dout, dq, dk, dv, ddecay, dS0, dz0, ws,
                                   stream);
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.S0 = S0; a.z0 = z0; a.decay = p.decay;
  a.dq = dq; a.dk = dk; a.dv = dv; a.ddecay = ddecay; a.dS0 = dS0; a.dz0 = dz0;
  const bool ml = p.decay_kind == LA_GATE_MLSTM;
  a.igate = ml ? p.igate : nullptr;
  a.stab = ml ? p.stab : nullptr;
  a.digate = ml ? ddecay + p.BH() * p.T : nullptr;   // the second half of ddecay
  a.fgate_exp = ml ? p.fgate_exp : 0;
  a.ws = static_cast<float*>(ws);
  a.H = p.H; a.T = p.T; a.dh = p.dh; a.dv_ = p.dv; a.dp = p.dp;
  a.phi = int(p.phi); a.decay_kind = int(p.decay_kind); a.norm = p.norm;
  a.dout_f32 = p.out_dtype == LA_F32 ? 1 : 0;
  a.eps = p.eps;
  hipError_t e = hipErrorInvalidValue;
  switch (p.dtype) {
    case LA_F32: e = launch_dt<float>(a, p.BH(), stream); break;
    case LA_BF16: e = launch_dt<bf16_t>(a, p.BH(), stream); break;
    case LA_F16: e = launch_dt<f16_t>(a, p.BH(), stream); break;
  }
  if (e != hipSuccess || !ddecay || ml) return e;
  // near-zero decays: the exact gradient, over the whole sequence (one
  // segment from the initial state, nothing carried in after its end)
  DecayExactArgs x;
  x.q = q; x.k = k; x.v = v; x.decay = p.decay; x.decay_kind = int(p.decay_kind);
  x.phi = int(p.phi); x.mode = 1; x.tok = nullptr; x.dout = nullptr; x.dout_f32 = 0;
  x.ws = a.ws; x.S0 = S0; x.z0 = z0; x.s_bh = int64_t(p.dp) * p.dv; x.z_bh = p.dp; x.s_seg = 0;
  x.gafter = nullptr; x.nseg = 1; x.seg_len = p.T; x.dd = ddecay;
  x.T = p.T; x.dh = p.dh; x.dv = p.dv; x.dp = p.dp;
  return launch_decay_exact(x, p.dtype, p.BH(), stream);
}

}  // namespace la
