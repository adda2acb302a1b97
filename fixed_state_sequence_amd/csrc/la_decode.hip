// Decode step: one token for every (sequence, head) state.
//
// Per state (llm-arch-kb "Linear Attention", section 2, causal recurrence;
// wikillm "Linear attention", Implementation sketch and Variants / RFA):
//   S <- alpha S + beta phi(k) v^T,  z <- alpha z + beta phi(k),
//   o  = phi(q)^T S / (phi(q)^T z + eps).
// mLSTM gates (wikillm "Linear attention", Variants / mLSTM): alpha, beta are
// the forget gate and the exponential input gate, applied to a state held
// scaled by e^{-m} as e^{log f + m - m'} and e^{itilde - m'}, with the
// stabiliser m' = max(log f + m, itilde) stored back per state.
// The step reads and writes the whole state once and does O(d' d_v) work on
// it, so it is bound by HBM bandwidth (wikillm "When to use which": decoding
// with a fixed-size state is memory-bound).
//
// Work split.  One wave (WPS waves for states of 32 KB and more) owns one
// state; a 512-thread workgroup holds 8 / WPS states of the same
// head, so the RFF projection W_h is staged once in LDS and shared.  Within a
// wave, lane l owns float4 column group l % CG of a contiguous run of NI rows;
// one load instruction of the wave covers RPI = 64 / CG whole rows, so every
// row (256 B for d_v = 64) is read and written as full cache lines.  Every
// state load is issued before the feature map is computed, so the whole state
// is in flight while phi(q), phi(k) are formed.  The read-out phi(q)^T S is
// reduced across the lanes of a column group with cross-lane shuffles (and
// across the WPS waves through LDS).
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 512;

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* S;
  float* z;
  const float* W;       // [H, D, dh] (RFF)
  const float* decay;   // [N, H] (SSD a, RFA g or the mLSTM forget pre-activation)
  const float* igate;   // [N, H] mLSTM input-gate pre-activation
  float* stab;          // [N, H] mLSTM stabiliser
  int N, H, dh;
  int dhp;              // padded LDS row of W (floats)
  int out_f32;
  int norm;             // read-out form (LA_NORM_*)
  int ident;            // identity feature map (else elu+1), when not RFF
  int fgate_exp;        // mLSTM forget gate: sigmoid (0) or exp (1)
  float eps;
};

template <int DV, int DP, bool WIDE = false>
struct DecCfg {
  // waves per state: a 32 KB state is split over two waves (16 rows of
  // float4 per lane), so that four waves fit per SIMD; larger states take
  // one wave per 32 KB.  WIDE: a 32 KB state over four waves (8 rows per
  // lane), for state sets larger than the last-level cache (measured with
  // streamed accesses, 1024 x 16 states of 128 x 64: 200 -> 191 us per step;
  // 256 x 16, which the cache holds: 49.2 -> 52.5 us, so the two-wave split
  // stays there)
  static constexpr int WPS = DP * DV > 8192 ? DP * DV / 8192 : (DP * DV == 8192 ? (WIDE ? 4 : 2) : 1);
  static constexpr int SPW = (NT / 64) / WPS;                      // states per workgroup
  static constexpr int CG = DV / 4;                                // float4 column groups
  static constexpr int RPI = 64 / CG;                              // rows per wave instruction
  static constexpr int NI = DP / (RPI * WPS);                      // rows per lane
  static constexpr int ZPL = (DP + 64 * WPS - 1) / (64 * WPS);     // z entries per lane
  static_assert(NI * RPI * WPS == DP, "row split");
  static_assert(NI % 4 == 0 && NI <= 32, "rows per lane");
  static_assert(SPW * WPS == NT / 64, "waves");
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// The state is read and written exactly once per step.  A state set larger
// than the last-level cache is streamed past the caches (nontemporal loads
// and stores); a smaller one is loaded and stored normally, so that it stays
// in that cache from one step to the next.  Measured on 128 x 64 fp32
// states, 16 heads: up to 480 sequences (256 MB) normal accesses run at
// 0.75-0.79 of 8 TB/s against 0.68-0.72 streamed; at 640 sequences (341 MB)
// streaming wins (0.72 against 0.68), at 1024 (545 MB) 0.72 against 0.65.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld4_stream(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4_stream(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void st4(float* p, const float4& v) { *reinterpret_cast<float4*>(p) = v; }

// DHMAX bounds the q, k width held in LDS (d_h <= 128 for RFF, d' for elu+1).
// BIG: the call's state set exceeds the last-level cache (streamed state
// accesses; 32 KB states over four waves).
template <typename DT, int DV, int DP, bool RFF, int DECAY, bool BIG>
__global__ __launch_bounds__(NT) void decode_kernel(const DecArgs a) {
  using G = DecCfg<DV, DP, BIG>;
  constexpr int DHMAX = RFF ? 128 : DP;       // q, k width held in LDS
  extern __shared__ __align__(16) float s_W[];  // RFF projection, [D][dhp]
  __shared__ __align__(16) float s_x[G::SPW][2][DHMAX];
  __shared__ __align__(16) float s_v[G::SPW][DV];
  __shared__ __align__(16) float s_phi[G::SPW][2][DP];
  __shared__ __align__(16) float s_red[G::WPS > 1 ? NT / 64 : 1][DV + 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sidx = wave / G::WPS, wsub = wave % G::WPS;
  const int h = int(blockIdx.x % unsigned(a.H));
  const int n = int(blockIdx.x / unsigned(a.H)) * G::SPW + sidx;
  const bool valid = n < a.N;
  const int64_t st = int64_t(valid ? n : 0) * a.H + h;
  const int cg = lane % G::CG, rsub = lane / G::CG;
  const int row0 = (wsub * G::RPI + rsub) * G::NI;

  // ---- state loads first: NI float4 per lane, whole rows per instruction
  float* Sg = a.S + st * (DP * DV);
  float4 s[G::NI];
#pragma unroll
  for (int i = 0; i < G::NI; ++i)
    s[i] = BIG ? ld4_stream(Sg + (row0 + i) * DV + 4 * cg)   // st points at a real state even if !valid
               : ld4(Sg + (row0 + i) * DV + 4 * cg);
  float* zg = a.z + st * DP;
  float zr[G::ZPL];
#pragma unroll
  for (int j = 0; j < G::ZPL; ++j) {
    const int f = (j * G::WPS + wsub) * 64 + lane;
    zr[j] = (valid && f < DP) ? zg[f] : 0.f;
  }
  float alpha = 1.f, beta = 1.f, m = 0.f;
  if constexpr (DECAY == 3) {
    // stabilised mLSTM gates: m = max(log f + m_old, itilde)
    const float lf = valid ? log_forget(a.decay[st], a.fgate_exp) : 0.f;
    const float it = valid ? a.igate[st] : 0.f;
    const float mo = valid ? a.stab[st] : 0.f;
    m = fmaxf(lf + mo, it);
    alpha = expf(lf + mo - m);
    beta = expf(it - m);
  } else if constexpr (DECAY != 0) {
    alpha = valid ? a.decay[st] : 0.f;
    if constexpr (DECAY == 2) beta = 1.f - alpha;
  }

  // ---- stage q, k, v (and W) in LDS
  const int xw = RFF ? a.dh : DP;
  if (wsub == 0 && valid) {
    const DT* qg = static_cast<const DT*>(a.q) + st * xw;
    const DT* kg = static_cast<const DT*>(a.k) + st * xw;
    const DT* vg = static_cast<const DT*>(a.v) + st * DV;
    for (int i = lane; i < xw; i += 64) {
      s_x[sidx][0][i] = to_f32(qg[i]);
      s_x[sidx][1][i] = to_f32(kg[i]);
    }
    for (int i = lane; i < DV; i += 64) s_v[sidx][i] = to_f32(vg[i]);
  }
  if constexpr (RFF) {
    constexpr int D = DP / 2;
    const float* Wh = a.W + int64_t(h) * D * a.dh;
    if ((a.dh & 3) == 0 && (reinterpret_cast<uintptr_t>(a.W) & 15) == 0) {
      // float4 pieces (W 16-byte aligned): each group of q4 lanes takes one
      // row, no division
      const int q4 = a.dh >> 2;                 // float4 per row, <= 32
      const int rpg = 64 / q4 > 0 ? 64 / q4 : 1;   // rows per wave and pass
      const int sub = lane / q4, col = 4 * (lane - sub * q4);
      if (sub < rpg) {
        for (int j = wave * rpg + sub; j < D; j += (NT / 64) * rpg)
          *reinterpret_cast<float4*>(s_W + j * a.dhp + col) =
              *reinterpret_cast<const float4*>(Wh + j * a.dh + col);
      }
    } else {
      for (int j = wave; j < D; j += NT / 64)
        for (int i = lane; i < a.dh; i += 64) s_W[j * a.dhp + i] = Wh[j * a.dh + i];
    }
  }
  __syncthreads();

  // ---- feature maps: with one wave per state it forms phi(q) and phi(k);
  // with two or more, the first forms phi(q) and the second phi(k)
  if constexpr (RFF) {
    if (wsub < (G::WPS > 1 ? 2 : 1)) {
      // phi(x) = D^{-1/2} [sin(W_h x); cos(W_h x)] (wikillm, Variants / RFA)
      constexpr int D = DP / 2;
      const float rs = 1.0f / sqrtf(float(D));
      auto project = [&](int which) {
        const float* x = s_x[sidx][which];
        float* f = s_phi[sidx][which];
#pragma unroll
        for (int jj = 0; jj < (D + 63) / 64; ++jj) {
          const int j = lane + 64 * jj;
          if (j < D) {
            const float* w = s_W + j * a.dhp;
            float p = 0.f;
            int i = 0;
            for (; i + 4 <= a.dh; i += 4) {
              const float4 w4 = ld4(w + i), x4 = ld4(x + i);
              p = fmaf(w4.x, x4.x, p); p = fmaf(w4.y, x4.y, p);
              p = fmaf(w4.z, x4.z, p); p = fmaf(w4.w, x4.w, p);
            }
            for (; i < a.dh; ++i) p = fmaf(w[i], x[i], p);
            float sn, cs;
            sincosf(p, &sn, &cs);
            f[j] = sn * rs;
            f[D + j] = cs * rs;
          }
        }
      };
      if constexpr (G::WPS > 1) {
        project(wsub);
      } else {
        project(0);
        project(1);
      }
    }
  } else if (wsub == 0) {
    float* fq = s_phi[sidx][0];
    float* fk = s_phi[sidx][1];
    for (int f = lane; f < DP; f += 64) {
      const float x = s_x[sidx][0][f], y = s_x[sidx][1][f];
      fq[f] = a.ident ? x : elu1_accurate(x);
      fk[f] = a.ident ? y : elu1_accurate(y);
    }
  }
  __syncthreads();

  // ---- rank-1 update, read-out partials, state stores
  const float4 v4 = ld4(&s_v[sidx][4 * cg]);
  const float* fq = s_phi[sidx][0];
  const float* fk = s_phi[sidx][1];
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i4 = 0; i4 < G::NI; i4 += 4) {
    const float4 q4 = ld4(fq + row0 + i4), k4 = ld4(fk + row0 + i4);
    const float qs[4] = {q4.x, q4.y, q4.z, q4.w};
    const float ks[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float4& x = s[i4 + u];
      const float kb = beta * ks[u];
      x.x = fmaf(alpha, x.x, kb * v4.x);
      x.y = fmaf(alpha, x.y, kb * v4.y);
      x.z = fmaf(alpha, x.z, kb * v4.z);
      x.w = fmaf(alpha, x.w, kb * v4.w);
      num.x = fmaf(qs[u], x.x, num.x);
      num.y = fmaf(qs[u], x.y, num.y);
      num.z = fmaf(qs[u], x.z, num.z);
      num.w = fmaf(qs[u], x.w, num.w);
    }
  }
  if (valid) {
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      if constexpr (BIG) st4_stream(Sg + (row0 + i) * DV + 4 * cg, s[i]);
      else st4(Sg + (row0 + i) * DV + 4 * cg, s[i]);
    }
  }
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < G::ZPL; ++j) {
    const int f = (j * G::WPS + wsub) * 64 + lane;
    if (f < DP) {
      const float zn = fmaf(alpha, zr[j], beta * fk[f]);
      den = fmaf(fq[f], zn, den);
      if (valid) zg[f] = zn;
    }
  }
#pragma unroll
  for (int off = G::CG; off < 64; off <<= 1) {
    num.x += __shfl_xor(num.x, off);
    num.y += __shfl_xor(num.y, off);
    num.z += __shfl_xor(num.z, off);
    num.w += __shfl_xor(num.w, off);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if constexpr (G::WPS > 1) {
    if (lane < G::CG) *reinterpret_cast<float4*>(&s_red[wave][4 * cg]) = num;
    if (lane == 0) s_red[wave][DV] = den;
    __syncthreads();
    if (wsub == 0 && lane < G::CG) {
      num = make_float4(0.f, 0.f, 0.f, 0.f);
      den = 0.f;
#pragma unroll
      for (int w = 0; w < G::WPS; ++w) {
        const float4 p = ld4(&s_red[sidx * G::WPS + w][4 * cg]);
        num.x += p.x; num.y += p.y; num.z += p.z; num.w += p.w;
        den += s_red[sidx * G::WPS + w][DV];
      }
    }
  }
  if constexpr (DECAY == 3) {
    if (valid && wsub == 0 && lane == 0) a.stab[st] = m;
  }
  if (valid && wsub == 0 && lane < G::CG) {
    const float inv = a.norm == LA_NORM_SUM && DECAY != 3 ? 1.0f / (den + a.eps)
                                                          : readout_factor(a.norm, den, a.eps, m);
    const int64_t o0 = st * DV + 4 * cg;
    if (a.out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o0) =
          make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    } else {
      DT* og = static_cast<DT*>(a.out) + o0;
      store_f32(num.x * inv, og + 0);
      store_f32(num.y * inv, og + 1);
      store_f32(num.z * inv, og + 2);
      store_f32(num.w * inv, og + 3);
    }
  }
}

template <typename DT, int DV, int DP, bool RFF, bool BIG>
hipError_t launch_cfg(const DecArgs& a, la_decay kind, hipStream_t st) {
  using G = DecCfg<DV, DP, BIG>;
  const unsigned groups = unsigned((a.N + G::SPW - 1) / G::SPW);
  const dim3 grid{groups * unsigned(a.H)}, block{unsigned(NT)};
  const size_t lds = RFF ? size_t(DP / 2) * a.dhp * sizeof(float) : 0;
  switch (kind) {
    case LA_DECAY_NONE: decode_kernel<DT, DV, DP, RFF, 0, BIG><<<grid, block, lds, st>>>(a); break;
    case LA_DECAY_SSD: decode_kernel<DT, DV, DP, RFF, 1, BIG><<<grid, block, lds, st>>>(a); break;
    case LA_GATE_RFA: decode_kernel<DT, DV, DP, RFF, 2, BIG><<<grid, block, lds, st>>>(a); break;
    case LA_GATE_MLSTM: decode_kernel<DT, DV, DP, RFF, 3, BIG><<<grid, block, lds, st>>>(a); break;
  }
  return hipGetLastError();
}

// State sets beyond this many bytes stream from HBM rather than the 256 MB
// last-level cache: streamed accesses, and 32 KB states take the four-wave
// split.
constexpr int64_t kLlcBytes = int64_t(256) << 20;

template <typename DT, int DV, int DP, bool RFF>
hipError_t launch_decay(const DecArgs& a, la_decay kind, hipStream_t st) {
  if (int64_t(a.N) * a.H * (DP * DV + DP) * 4 > kLlcBytes)
    return launch_cfg<DT, DV, DP, RFF, true>(a, kind, st);
  return launch_cfg<DT, DV, DP, RFF, false>(a, kind, st);
}

template <typename DT, int DV, int DP>
hipError_t launch_phi(const DecArgs& a, la_phi phi, la_decay kind, hipStream_t st) {
  return phi == LA_PHI_RFF ? launch_decay<DT, DV, DP, true>(a, kind, st)
                           : launch_decay<DT, DV, DP, false>(a, kind, st);
}

template <typename DT, int DV>
hipError_t launch_dp(const DecArgs& a, int dp, la_phi phi, la_decay kind, hipStream_t st) {
  switch (dp) {
    case 64: return launch_phi<DT, DV, 64>(a, phi, kind, st);
    case 128: return launch_phi<DT, DV, 128>(a, phi, kind, st);
    case 256: return launch_phi<DT, DV, 256>(a, phi, kind, st);
  }
  return hipErrorInvalidValue;
}

template <typename DT>
hipError_t launch_dt(const DecArgs& a, int dp, int dv, la_phi phi, la_decay kind, hipStream_t st) {
  return dv == 64 ? launch_dp<DT, 64>(a, dp, phi, kind, st) : launch_dp<DT, 128>(a, dp, phi, kind, st);
}

}  // namespace

bool decode_supported(const Problem& p) {
  if (p.dv != 64 && p.dv != 128) return false;
  if (p.dp != 64 && p.dp != 128 && p.dp != 256) return false;
  if (p.phi == LA_PHI_RFF) {
    // W_h staged in LDS as D rows of dhp floats, within the 64 KB dynamic limit
    const size_t dhp = size_t((p.dh + 3) / 4) * 4 + 4;
    return p.dh >= 1 && p.dh <= 128 && size_t(p.D) * dhp * sizeof(float) <= 65536;
  }
  return p.dh == p.dp;
}

hipError_t launch_decode(const Problem& p, const void* q, const void* k, const void* v, float* S,
                         float* z, void* out, hipStream_t stream) {
  DecArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.S = S; a.z = z;
  a.W = p.W; a.decay = p.decay; a.igate = p.igate; a.stab = p.stab;
  a.N = p.B; a.H = p.H; a.dh = p.dh;
  a.dhp = ((p.dh + 3) / 4) * 4 + 4;
  a.out_f32 = p.out_dtype == LA_F32 ? 1 : 0;
  a.eps = p.eps;
  a.norm = p.norm;
  a.ident = p.phi == LA_PHI_IDENTITY ? 1 : 0;
  a.fgate_exp = p.fgate_exp;
  switch (p.dtype) {
    case LA_F32: return launch_dt<float>(a, p.dp, p.dv, p.phi, p.decay_kind, stream);
    case LA_BF16: return launch_dt<bf16_t>(a, p.dp, p.dv, p.phi, p.decay_kind, stream);
    case LA_F16: return launch_dt<f16_t>(a, p.dp, p.dv, p.phi, p.decay_kind, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
