// Chunked causal linear attention prefill on CDNA4 MFMA (gfx950).
//
// The recurrence S_t = alpha_t S_{t-1} + beta_t phi(k_t) v_t^T,
// o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps) is re-bracketed over chunks of
// C tokens: quadratic (masked) attention inside a chunk and the fp32 state
// carried between chunks (efficient-attention lesson "Linear attention",
// Researcher level, "Implementation reality"; wikillm "Linear attention",
// Decaying linear attention with a scalar state (SSD): quadratic blocks
// inside chunks and a short recurrence between them).  Inside chunk c with
// start state (S, z) and lc_t = sum_{r <= t, r in chunk} log alpha_r:
//   o_t = [ e^{lc_t} phi(q_t)^T S + sum_{s <= t} P_ts v_s ]
//       / [ e^{lc_t} phi(q_t)^T z + sum_{s <= t} P_ts + eps ],
//   P_ts = phi(q_t).phi(k_s) e^{lc_t - lc_s} beta_s,
//   S' = e^{lc_last} S + sum_s w_s phi(k_s) v_s^T,  w_s = beta_s e^{lc_last - lc_s},
// and z' likewise.  No decay: all exponentials are 1 and only the causal mask
// remains.
//
// Parallel schedule.  Each (b, h) sequence is cut into `segments` runs of
// whole chunks.  Stage 1: one workgroup per segment (except the last) folds
// its chunks into a segment state (S_seg, z_seg, log Gamma_seg).  Stage 2:
// per element of the state, an exclusive scan over segments turns those into
// each segment's start state, folding in the caller's initial state.  Stage 3:
// one workgroup per segment walks its chunks again from its start state and
// writes the outputs; the last segment writes the final state.
//
// Work split inside a workgroup (D = d' = d_v, NW = D / 32 waves): wave w owns
// value columns [32 w, 32 w + 32) of the state.  All MFMAs are
// v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulate).  With
// g = lane / 32 and n = lane % 32, operand registers hold 8 consecutive
// k-values "8 g .. 8 g + 7" of row/column n, and the accumulator holds column
// n, rows 8 j + 4 g + i (j, i = 0..3).  The state S (features x values) lives
// in accumulator registers for the whole walk; because an accumulator's
// column-n/row-set layout is exactly the operand layout for row n when the
// k-axis is permuted as [0-3, 8-11 | 4-7, 12-15] within every 16, the state
// feeds the read-out MFMA straight from registers, and the intra-chunk score
// tile feeds the P V product the same way.  Every LDS tile is stored in that
// permuted k-order so all operands agree.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Floor on log(alpha) so that alpha = 0 (a full reset) stays finite in the
// within-chunk log-prefix; e^-80 ~ 1.8e-35 is the smallest decay applied.
constexpr float kLogFloor = -80.0f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split a pair into bf16 high parts and bf16 low parts (x - high), so that
// high + low carries x to about 2^-16 relative.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 consecutive elements of storage type DT, as fp32.
__device__ __forceinline__ void unpack8(const u32x4& w, float* x, bf16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const u32x4& w, float* x, f16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = float(__builtin_bit_cast(f16_t, uint16_t(w[i] & 0xffffu)));
    x[2 * i + 1] = float(__builtin_bit_cast(f16_t, uint16_t(w[i] >> 16)));
  }
}

// Position of k-index k inside the permuted order: within each 16, quads 1
// and 2 are swapped ([0-3, 8-11, 4-7, 12-15] at positions 0..15).
__device__ __forceinline__ constexpr int perm_pos(int k) {
  const int q = (k >> 2) & 3;
  const int pq = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (k & ~15) | (pq << 2) | (k & 3);
}

template <int D, int C, bool VS>
struct Cfg {
  static constexpr int NW = D / 32;          // waves, 32 value columns each
  static constexpr int NT = 64 * NW;         // threads per workgroup (= 2 D)
  static constexpr int FB = D / 8;           // 16-byte feature blocks per row
  static constexpr int RPT = C * FB / NT;    // token rows per thread when loading (= C / 16)
  static constexpr int TB = C / 32;          // 32-token blocks of a chunk
  static constexpr int KS = D / 16;          // 16-feature k-steps
  static constexpr int KT = C / 16;          // 16-token k-steps
  static constexpr int MT = D / 32;          // 32-feature tiles of the state
  static constexpr int ROW_B = 2 * D + 16;   // token-major rows: bf16, padded 16 B
  static constexpr int TR_B = 2 * C;         // feature-major rows: bf16, XOR-swizzled
  static constexpr int TR = D * TR_B;        // one feature-major tile
  // stage 3: phi(q), phi(k) token-major; w phi(k) high/low and v (high/low
  // when VS) feature-major; then small fp32 arrays
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * ROW_B;
  static constexpr int OFF_KH = OFF_K + C * ROW_B;
  static constexpr int OFF_KL = OFF_KH + TR;
  static constexpr int OFF_VH = OFF_KL + TR;
  static constexpr int OFF_VL = OFF_VH + TR;
  static constexpr int OFF_L = OFF_VL + (VS ? TR : 0);  // lc_t, fp32 [C]
  static constexpr int OFF_B = OFF_L + 4 * C;           // beta_t, fp32 [C]
  static constexpr int OFF_DEN = OFF_B + 4 * C;         // inter-chunk denominators, fp32 [C]
  static constexpr int OFF_Z = OFF_DEN + 4 * C;         // z, fp32 [D]
  static constexpr int OFF_DZ = OFF_Z + 4 * D;          // per-wave z increments, fp32 [NW][D]
  static constexpr int LDS = OFF_DZ + 4 * NW * D;
  // stage 1: the feature-major tiles and the small arrays
  static constexpr int S1_KH = 0;
  static constexpr int S1_KL = S1_KH + TR;
  static constexpr int S1_VH = S1_KL + TR;
  static constexpr int S1_VL = S1_VH + TR;
  static constexpr int S1_Z = S1_VL + (VS ? TR : 0);
  static constexpr int S1_DZ = S1_Z + 4 * D;
  static constexpr int S1_LDS = S1_DZ + 4 * NW * D;
  static_assert(RPT == C / 16, "row split");
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "width");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// XOR swizzle (in 16-byte blocks) of feature-major rows, chosen so that the
// 16 lanes of an operand read (16 consecutive rows, one logical block) and
// the transposing writes (rows 8 apart) spread over the LDS banks.
template <int C>
__device__ __forceinline__ int swz(int m) {
  if constexpr (C == 128) return (m ^ (m >> 3)) & 15;
  else if constexpr (C == 64) return ((m >> 1) ^ (m >> 4)) & 7;
  else return ((m >> 2) ^ (m >> 4)) & 3;
}

// Byte offset of (row m, permuted token position pos) in a feature-major tile.
template <int C>
__device__ __forceinline__ int tr_off(int m, int pos) {
  const int blk = pos >> 3;
  return m * (2 * C) + ((blk ^ swz<C>(m)) << 4) + ((pos & 7) << 1);
}

// Write RPT consecutive tokens (first = tok, a multiple of RPT) of one
// feature-major row m as bf16 high parts, and (when lo != nullptr) the bf16
// low parts x - high into a second tile.
template <int C, int RPT>
__device__ __forceinline__ void tr_write(char* hi, char* lo, int m, int tok, const float* vals) {
  if constexpr (RPT == 2) {
    uint32_t h, l;
    split_bf16(vals[0], vals[1], h, l);
    const int off = tr_off<C>(m, perm_pos(tok));
    *reinterpret_cast<uint32_t*>(hi + off) = h;
    if (lo) *reinterpret_cast<uint32_t*>(lo + off) = l;
  } else {
#pragma unroll
    for (int qd = 0; qd < RPT / 4; ++qd) {
      uint32_t h0, l0, h1, l1;
      split_bf16(vals[4 * qd], vals[4 * qd + 1], h0, l0);
      split_bf16(vals[4 * qd + 2], vals[4 * qd + 3], h1, l1);
      const int off = tr_off<C>(m, perm_pos(tok + 4 * qd));
      *reinterpret_cast<u32x2*>(hi + off) = u32x2{h0, h1};
      if (lo) *reinterpret_cast<u32x2*>(lo + off) = u32x2{l0, l1};
    }
  }
}

// Write 8 features (first = 8 fb) of token-major row r, permuted order.
template <int ROW_B>
__device__ __forceinline__ void row_write(char* base, int r, int fb, const float* x) {
  const int f0 = 8 * fb;
  u32x2 a = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
  u32x2 b = {pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
  *reinterpret_cast<u32x2*>(base + r * ROW_B + 2 * perm_pos(f0)) = a;
  *reinterpret_cast<u32x2*>(base + r * ROW_B + 2 * perm_pos(f0 + 4)) = b;
}

struct PfArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* S;          // caller's state [BH, D, D] (initial in, final out)
  float* z;          // caller's normaliser [BH, D]
  const float* decay;  // [BH, T] or null
  float* ws_state;   // [BH, nseg, D*D + D]
  float* ws_logg;    // [BH, nseg]
  int T;
  int nseg;
  int cps;           // chunks per segment
  int out_f32;       // out is fp32 (else the input type)
  float eps;
};

// Within-chunk inclusive log-prefix of the decay, one wave: every wave of the
// workgroup computes it redundantly (no barrier needed).  Returns lc for
// token `lane` (and `lane + 64` in hi for C = 128) and the chunk total.
template <int C, int DECAY>
__device__ __forceinline__ void chunk_logprefix(const float* dg, int tok0, int T, int lane,
                                                float& lo, float& hi, float& total) {
  auto logdecay = [&](int r) -> float {
    const int t = tok0 + r;
    if (r >= C || t >= T) return 0.f;
    return fmaxf(__logf(dg[t]), kLogFloor);
  };
  lo = logdecay(lane);
  hi = C > 64 ? logdecay(lane + 64) : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float a = __shfl_up(lo, off);
    const float b = __shfl_up(hi, off);
    if (lane >= off) {
      lo += a;
      hi += b;
    }
  }
  if constexpr (C > 64) {
    hi += __shfl(lo, 63);
    total = __shfl(hi, 63);
  } else {
    total = __shfl(lo, C - 1);
  }
}

template <int C>
__device__ __forceinline__ float lc_of(float lo, float hi, int r) {
  const float a = __shfl(lo, r & 63);
  if constexpr (C > 64) {
    const float b = __shfl(hi, r & 63);
    return r >= 64 ? b : a;
  } else {
    return a;
  }
}

// ---------------------------------------------------------------- stage 1

template <int D, int C, int DECAY, typename DT>
__global__ __launch_bounds__(2 * D) void segment_state_kernel(const PfArgs a) {
  constexpr bool VS = __is_same(DT, f16_t);   // fp16 v needs a bf16 low part too
  using G = Cfg<D, C, VS>;
  __shared__ __align__(16) char smem[G::S1_LDS];
  const int nseg = a.nseg;
  const int bh = blockIdx.x / (nseg - 1);
  const int seg = blockIdx.x % (nseg - 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int fb = tid % G::FB, rg = tid / G::FB;
  const int nchunks = (a.T + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(c0 + a.cps, nchunks);

  const DT* kg = static_cast<const DT*>(a.k) + int64_t(bh) * a.T * D;
  const DT* vg = static_cast<const DT*>(a.v) + int64_t(bh) * a.T * D;
  const float* dg = DECAY ? a.decay + int64_t(bh) * a.T : nullptr;
  float* zl = reinterpret_cast<float*>(smem + G::S1_Z);
  float* dzl = reinterpret_cast<float*>(smem + G::S1_DZ);

  f32x16 acc[G::MT];
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) acc[mt] = f32x16{};
  if (tid < D) zl[tid] = 0.f;
  float logg = 0.f;

  for (int c = c0; c < c1; ++c) {
    const int tok0 = c * C;
    float lo = 0.f, hi = 0.f, ltot = 0.f;
    if constexpr (DECAY != 0) chunk_logprefix<C, DECAY>(dg, tok0, a.T, lane, lo, hi, ltot);
    logg += ltot;
    // ---- [A] load k, v rows; write w * phi(k) and v feature-major; z partials
    float kx[G::RPT][8], vx[G::RPT][8];
    float dz[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < G::RPT; ++i) {
      const int r = G::RPT * rg + i;
      const int t = tok0 + r;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (t < a.T) {
        kw = *reinterpret_cast<const u32x4*>(kg + int64_t(t) * D + 8 * fb);
        vw = *reinterpret_cast<const u32x4*>(vg + int64_t(t) * D + 8 * fb);
      }
      unpack8(kw, kx[i], DT{});
      unpack8(vw, vx[i], DT{});
      float w = t < a.T ? 1.f : 0.f;
      if constexpr (DECAY != 0) {
        const float lct = lc_of<C>(lo, hi, r);
        w *= __expf(ltot - lct);
        if constexpr (DECAY == 2) w *= (t < a.T ? 1.f - dg[t] : 0.f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kx[i][e] = w * elu1_fast(kx[i][e]);
        dz[e] += kx[i][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float col_k[G::RPT], col_v[G::RPT];
#pragma unroll
      for (int i = 0; i < G::RPT; ++i) {
        col_k[i] = kx[i][e];
        col_v[i] = vx[i][e];
      }
      tr_write<C, G::RPT>(smem + G::S1_KH, smem + G::S1_KL, 8 * fb + e, G::RPT * rg, col_k);
      tr_write<C, G::RPT>(smem + G::S1_VH, VS ? smem + G::S1_VL : nullptr, 8 * fb + e, G::RPT * rg,
                          col_v);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int off = G::FB; off < 64; off <<= 1) dz[e] += __shfl_xor(dz[e], off);
    if (lane < G::FB) {
      float* d = dzl + wave * D + 8 * fb;
      *reinterpret_cast<f32x4*>(d) = f32x4{dz[0], dz[1], dz[2], dz[3]};
      *reinterpret_cast<f32x4*>(d + 4) = f32x4{dz[4], dz[5], dz[6], dz[7]};
    }
    __syncthreads();
    // ---- [B] z and S updates
    const float gam = DECAY ? __expf(ltot) : 1.f;
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < G::NW; ++w) s += dzl[w * D + tid];
      zl[tid] = gam * zl[tid] + s;
    }
    u32x4 vh[G::KT], vl[G::KT];
#pragma unroll
    for (int kk = 0; kk < G::KT; ++kk) {
      const int off = tr_off<C>(32 * wave + n, 16 * kk + 8 * g);
      vh[kk] = *reinterpret_cast<const u32x4*>(smem + G::S1_VH + off);
      if constexpr (VS) vl[kk] = *reinterpret_cast<const u32x4*>(smem + G::S1_VL + off);
    }
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      if constexpr (DECAY != 0) acc[mt] *= gam;
#pragma unroll
      for (int kk = 0; kk < G::KT; ++kk) {
        const int off = tr_off<C>(32 * mt + n, 16 * kk + 8 * g);
        const u32x4 kh = *reinterpret_cast<const u32x4*>(smem + G::S1_KH + off);
        const u32x4 kl = *reinterpret_cast<const u32x4*>(smem + G::S1_KL + off);
        acc[mt] = mfma(kh, vh[kk], acc[mt]);
        acc[mt] = mfma(kl, vh[kk], acc[mt]);
        if constexpr (VS) acc[mt] = mfma(kh, vl[kk], acc[mt]);
      }
    }
    __syncthreads();
  }

  // write the segment state: S row-major [f][v], then z, then log Gamma
  float* dst = a.ws_state + (int64_t(bh) * nseg + seg) * (D * D + D);
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
      dst[f * D + 32 * wave + n] = acc[mt][r];
    }
  if (tid < D) dst[D * D + tid] = zl[tid];
  if (tid == 0) a.ws_logg[int64_t(bh) * nseg + seg] = logg;
}

// ---------------------------------------------------------------- stage 2

template <int D>
__global__ __launch_bounds__(256) void segment_scan_kernel(const PfArgs a) {
  constexpr int E = D * D + D;
  const int per_bh = (E + 255) / 256;
  const int bh = blockIdx.x / per_bh;
  const int e = (blockIdx.x % per_bh) * 256 + threadIdx.x;
  if (e >= E) return;
  float carry = e < D * D ? a.S[int64_t(bh) * D * D + e] : a.z[int64_t(bh) * D + (e - D * D)];
  float* base = a.ws_state + int64_t(bh) * a.nseg * E + e;
  const float* lg = a.ws_logg + int64_t(bh) * a.nseg;
  for (int s = 0; s < a.nseg; ++s) {
    const float x = base[int64_t(s) * E];
    base[int64_t(s) * E] = carry;
    if (s + 1 < a.nseg) carry = __expf(lg[s]) * carry + x;
  }
}

// ---------------------------------------------------------------- stage 3

template <int D, int C, int DECAY, typename DT>
__global__ __launch_bounds__(2 * D) void output_kernel(const PfArgs a) {
  constexpr bool VS = __is_same(DT, f16_t);   // fp16 v needs a bf16 low part too
  using G = Cfg<D, C, VS>;
  __shared__ __align__(16) char smem[G::LDS];
  const int nseg = a.nseg;
  const int bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int fb = tid % G::FB, rg = tid / G::FB;
  const int nchunks = (a.T + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(c0 + a.cps, nchunks);

  const DT* qg = static_cast<const DT*>(a.q) + int64_t(bh) * a.T * D;
  const DT* kg = static_cast<const DT*>(a.k) + int64_t(bh) * a.T * D;
  const DT* vg = static_cast<const DT*>(a.v) + int64_t(bh) * a.T * D;
  DT* og = static_cast<DT*>(a.out) + int64_t(bh) * a.T * D;
  const float* dg = DECAY ? a.decay + int64_t(bh) * a.T : nullptr;
  float* Ll = reinterpret_cast<float*>(smem + G::OFF_L);
  float* Bl = reinterpret_cast<float*>(smem + G::OFF_B);
  float* denl = reinterpret_cast<float*>(smem + G::OFF_DEN);
  float* zl = reinterpret_cast<float*>(smem + G::OFF_Z);
  float* dzl = reinterpret_cast<float*>(smem + G::OFF_DZ);

  // start state of this segment
  const float* S0 = a.S + int64_t(bh) * D * D;
  const float* z0 = a.z + int64_t(bh) * D;
  if (nseg > 1) {
    S0 = a.ws_state + (int64_t(bh) * nseg + seg) * (D * D + D);
    z0 = S0 + D * D;
  }
  f32x16 acc[G::MT];
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
      acc[mt][r] = S0[f * D + 32 * wave + n];
    }
  if (tid < D) zl[tid] = z0[tid];
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int tok0 = c * C;
    float lo = 0.f, hi = 0.f, ltot = 0.f;
    if constexpr (DECAY != 0) chunk_logprefix<C, DECAY>(dg, tok0, a.T, lane, lo, hi, ltot);

    // ---- [A] cooperative load: phi(q), phi(k) token-major; w phi(k), v
    //      feature-major; inter-chunk denominators; z increments.
    {
      float zf[8];
      *reinterpret_cast<f32x4*>(zf) = *reinterpret_cast<const f32x4*>(zl + 8 * fb);
      *reinterpret_cast<f32x4*>(zf + 4) = *reinterpret_cast<const f32x4*>(zl + 8 * fb + 4);
      float kw_[G::RPT][8], vx[G::RPT][8];
      float dz[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < G::RPT; ++i) {
        const int r = G::RPT * rg + i;
        const int t = tok0 + r;
        const bool valid = t < a.T;
        u32x4 qw = {0u, 0u, 0u, 0u}, kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
        if (valid) {
          qw = *reinterpret_cast<const u32x4*>(qg + int64_t(t) * D + 8 * fb);
          kw = *reinterpret_cast<const u32x4*>(kg + int64_t(t) * D + 8 * fb);
          vw = *reinterpret_cast<const u32x4*>(vg + int64_t(t) * D + 8 * fb);
        }
        float qx[8], kx[8];
        unpack8(qw, qx, DT{});
        unpack8(kw, kx, DT{});
        unpack8(vw, vx[i], DT{});
        float lct = 0.f, w = valid ? 1.f : 0.f, beta = 1.f;
        if constexpr (DECAY != 0) {
          lct = lc_of<C>(lo, hi, r);
          if constexpr (DECAY == 2) beta = valid ? 1.f - dg[t] : 0.f;
          w *= beta * __expf(ltot - lct);
        }
        float den = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qx[e] = valid ? elu1_fast(qx[e]) : 0.f;
          kx[e] = valid ? elu1_fast(kx[e]) : 0.f;
          den += qx[e] * zf[e];
          kw_[i][e] = w * kx[e];
          dz[e] += kw_[i][e];
        }
        row_write<G::ROW_B>(smem + G::OFF_Q, r, fb, qx);
        row_write<G::ROW_B>(smem + G::OFF_K, r, fb, kx);
#pragma unroll
        for (int off = 1; off < G::FB; off <<= 1) den += __shfl_xor(den, off);
        if (fb == 0) {
          if constexpr (DECAY != 0) den *= __expf(lct);
          denl[r] = den;
          Ll[r] = lct;
          Bl[r] = beta;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float col_k[G::RPT], col_v[G::RPT];
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) {
          col_k[i] = kw_[i][e];
          col_v[i] = vx[i][e];
        }
        tr_write<C, G::RPT>(smem + G::OFF_KH, smem + G::OFF_KL, 8 * fb + e, G::RPT * rg, col_k);
        tr_write<C, G::RPT>(smem + G::OFF_VH, VS ? smem + G::OFF_VL : nullptr, 8 * fb + e,
                            G::RPT * rg, col_v);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        for (int off = G::FB; off < 64; off <<= 1) dz[e] += __shfl_xor(dz[e], off);
      if (lane < G::FB) {
        float* d = dzl + wave * D + 8 * fb;
        *reinterpret_cast<f32x4*>(d) = f32x4{dz[0], dz[1], dz[2], dz[3]};
        *reinterpret_cast<f32x4*>(d + 4) = f32x4{dz[4], dz[5], dz[6], dz[7]};
      }
    }
    __syncthreads();

    // ---- [B] per wave: read-out of the carried state, masked intra-chunk
    //      attention, normalise and store, then fold the chunk into S and z.
    const float gam = DECAY ? __expf(ltot) : 1.f;
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < G::NW; ++w) s += dzl[w * D + tid];
      zl[tid] = gam * zl[tid] + s;   // z of the next chunk; read again after the barrier
    }
    // state as bf16 operands (k = features), from the accumulators
    u32x4 sf[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const int mt = ks >> 1, j0 = 2 * (ks & 1);
      const f32x16& s = acc[mt];
      sf[ks] = u32x4{pack_bf16(s[4 * j0 + 0], s[4 * j0 + 1]), pack_bf16(s[4 * j0 + 2], s[4 * j0 + 3]),
                     pack_bf16(s[4 * j0 + 4], s[4 * j0 + 5]), pack_bf16(s[4 * j0 + 6], s[4 * j0 + 7])};
    }
    u32x4 vh[G::KT], vl[G::KT];
#pragma unroll
    for (int kk = 0; kk < G::KT; ++kk) {
      const int off = tr_off<C>(32 * wave + n, 16 * kk + 8 * g);
      vh[kk] = *reinterpret_cast<const u32x4*>(smem + G::OFF_VH + off);
      if constexpr (VS) vl[kk] = *reinterpret_cast<const u32x4*>(smem + G::OFF_VL + off);
    }

#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb) {
      const int tl = 32 * tb + n;   // this lane's query token within the chunk
      u32x4 qf[G::KS];
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        qf[ks] = *reinterpret_cast<const u32x4*>(smem + G::OFF_Q + tl * G::ROW_B + 32 * ks + 16 * g);
      f32x16 o = f32x16{};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) o = mfma(sf[ks], qf[ks], o);
      float lct = 0.f;
      if constexpr (DECAY != 0) {
        lct = Ll[tl];
        o *= __expf(lct);
      }
      float dsum = 0.f;
#pragma unroll
      for (int sb = 0; sb <= tb; ++sb) {
        f32x16 p = f32x16{};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(smem + G::OFF_K + (32 * sb + n) * G::ROW_B + 32 * ks + 16 * g);
          p = mfma(kf, qf[ks], p);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int sl = 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
          float x = p[r];
          if constexpr (DECAY != 0) x *= __expf(lct - Ll[sl]) * Bl[sl];
          if (sb == tb && sl > tl) x = 0.f;
          p[r] = x;
          dsum += x;
        }
        // P = P_hi + P_lo (bf16 each): the P V product then carries the
        // fp32 scores the denominator sums, to ~2^-16.
        u32x4 ph0, pl0, ph1, pl1;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t a0, b0, a1, b1;
          split_bf16(p[2 * h], p[2 * h + 1], a0, b0);
          split_bf16(p[8 + 2 * h], p[8 + 2 * h + 1], a1, b1);
          ph0[h] = a0; pl0[h] = b0; ph1[h] = a1; pl1[h] = b1;
        }
        o = mfma(vh[2 * sb], ph0, o);
        o = mfma(vh[2 * sb], pl0, o);
        o = mfma(vh[2 * sb + 1], ph1, o);
        o = mfma(vh[2 * sb + 1], pl1, o);
        if constexpr (VS) {
          o = mfma(vl[2 * sb], ph0, o);
          o = mfma(vl[2 * sb + 1], ph1, o);
        }
      }
      dsum += __shfl_xor(dsum, 32);
      const float inv = 1.0f / (denl[tl] + dsum + a.eps);
      const int t = tok0 + tl;
      if (t < a.T) {
        if (a.out_f32) {
          float* orow = static_cast<float*>(a.out) + (int64_t(bh) * a.T + t) * D + 32 * wave + 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(orow + 8 * j) =
                f32x4{o[4 * j] * inv, o[4 * j + 1] * inv, o[4 * j + 2] * inv, o[4 * j + 3] * inv};
        } else {
          DT* orow = og + int64_t(t) * D + 32 * wave + 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float y0 = o[4 * j] * inv, y1 = o[4 * j + 1] * inv;
            const float y2 = o[4 * j + 2] * inv, y3 = o[4 * j + 3] * inv;
            u32x2 w;
            if constexpr (__is_same(DT, bf16_t)) {
              w = u32x2{pack_bf16(y0, y1), pack_bf16(y2, y3)};
            } else {
              typedef _Float16 h2 __attribute__((ext_vector_type(2)));
              w = u32x2{__builtin_bit_cast(uint32_t, h2{(f16_t)y0, (f16_t)y1}),
                        __builtin_bit_cast(uint32_t, h2{(f16_t)y2, (f16_t)y3})};
            }
            *reinterpret_cast<u32x2*>(orow + 8 * j) = w;
          }
        }
      }
    }

    // fold this chunk into the carried state: w phi(k) as high + low parts
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      if constexpr (DECAY != 0) acc[mt] *= gam;
#pragma unroll
      for (int kk = 0; kk < G::KT; ++kk) {
        const int off = tr_off<C>(32 * mt + n, 16 * kk + 8 * g);
        const u32x4 kh = *reinterpret_cast<const u32x4*>(smem + G::OFF_KH + off);
        const u32x4 kl = *reinterpret_cast<const u32x4*>(smem + G::OFF_KL + off);
        acc[mt] = mfma(kh, vh[kk], acc[mt]);
        acc[mt] = mfma(kl, vh[kk], acc[mt]);
        if constexpr (VS) acc[mt] = mfma(kh, vl[kk], acc[mt]);
      }
    }
    __syncthreads();
  }

  if (seg == nseg - 1) {
    float* Sd = a.S + int64_t(bh) * D * D;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        Sd[f * D + 32 * wave + n] = acc[mt][r];
      }
    if (tid < D) a.z[int64_t(bh) * D + tid] = zl[tid];
  }
}

// ---------------------------------------------------------------- dispatch

template <int D, int C, int DECAY, typename DT>
hipError_t launch3(const PfArgs& a, int64_t BH, int stage, hipStream_t st) {
  using G = Cfg<D, C, __is_same(DT, f16_t)>;
  if (stage == 1) {
    if (a.nseg <= 1) return hipSuccess;
    segment_state_kernel<D, C, DECAY, DT><<<dim3(unsigned(BH * (a.nseg - 1))), dim3(G::NT), 0, st>>>(a);
  } else if (stage == 2) {
    if (a.nseg <= 1) return hipSuccess;
    const int per_bh = (D * D + D + 255) / 256;
    segment_scan_kernel<D><<<dim3(unsigned(BH * per_bh)), dim3(256), 0, st>>>(a);
  } else {
    output_kernel<D, C, DECAY, DT><<<dim3(unsigned(BH * a.nseg)), dim3(G::NT), 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int D, int C, typename DT>
hipError_t launch_decay(const PfArgs& a, int64_t BH, la_decay kind, int stage, hipStream_t st) {
  switch (kind) {
    case LA_DECAY_NONE: return launch3<D, C, 0, DT>(a, BH, stage, st);
    case LA_DECAY_SSD: return launch3<D, C, 1, DT>(a, BH, stage, st);
    case LA_GATE_RFA: return launch3<D, C, 2, DT>(a, BH, stage, st);
  }
  return hipErrorInvalidValue;
}

template <int D, typename DT>
hipError_t launch_chunk(const PfArgs& a, int64_t BH, int chunk, la_decay kind, int stage,
                        hipStream_t st) {
  switch (chunk) {
    case 32: return launch_decay<D, 32, DT>(a, BH, kind, stage, st);
    case 64: return launch_decay<D, 64, DT>(a, BH, kind, stage, st);
    case 128:
      if constexpr (D <= 64) return launch_decay<D, 128, DT>(a, BH, kind, stage, st);
      break;
  }
  return hipErrorInvalidValue;
}

int chunks_per_segment(const Problem& p) {
  const int nchunks = (p.T + p.chunk - 1) / p.chunk;
  return (nchunks + p.segments - 1) / p.segments;
}

}  // namespace

bool mfma_supported(const Problem& p) {
  return (p.dtype == LA_BF16 || p.dtype == LA_F16) && p.phi == LA_PHI_ELU1 && p.dp == p.dv &&
         (p.dv == 64 || p.dv == 128);
}

// Chunks whose stage-3 tiles fit in the 160 KB of LDS of one compute unit.
bool mfma_chunk_fits(int d, int chunk) { return chunk <= 64 || d <= 64; }

// Aim for about two workgroups per compute unit on a 256-CU part, with at
// least two chunks per segment.
int mfma_default_segments(const Problem& p) {
  const int64_t target_wg = 512;
  const int64_t BH = p.BH();
  const int nchunks = (p.T + p.chunk - 1) / p.chunk;
  int64_t seg = (target_wg + BH - 1) / BH;
  const int64_t max_seg = nchunks >= 2 ? nchunks / 2 : 1;
  if (seg > max_seg) seg = max_seg;
  if (seg < 1) seg = 1;
  // no empty segments: the effective count is ceil(nchunks / cps)
  const int64_t cps = (nchunks + seg - 1) / seg;
  return int(cps > 0 ? (nchunks + cps - 1) / cps : 1);
}

size_t mfma_workspace_bytes(const Problem& p) {
  if (p.path != 1 || p.segments <= 1) return 0;
  const size_t E = size_t(p.dv) * p.dv + p.dv;
  const size_t n = size_t(p.BH()) * p.segments;
  return n * E * sizeof(float) + ((n * sizeof(float) + 255) / 256) * 256;
}

hipError_t launch_mfma_stage(const Problem& p, int stage, const void* q, const void* k,
                             const void* v, float* S, float* z, void* out, void* ws,
                             hipStream_t stream) {
  PfArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.S = S; a.z = z; a.decay = p.decay;
  a.T = p.T;
  a.cps = chunks_per_segment(p);
  const int nchunks = (p.T + p.chunk - 1) / p.chunk;
  a.nseg = (nchunks + a.cps - 1) / a.cps;
  a.eps = p.eps;
  a.out_f32 = p.out_dtype == LA_F32 ? 1 : 0;
  a.ws_logg = nullptr;
  a.ws_state = nullptr;
  if (a.nseg > 1) {
    const size_t E = size_t(p.dv) * p.dv + p.dv;
    a.ws_state = static_cast<float*>(ws);
    a.ws_logg = a.ws_state + size_t(p.BH()) * a.nseg * E;
  }
  if (p.dv == 128) {
    return p.dtype == LA_BF16 ? launch_chunk<128, bf16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream)
                              : launch_chunk<128, f16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream);
  }
  return p.dtype == LA_BF16 ? launch_chunk<64, bf16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream)
                            : launch_chunk<64, f16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream);
}

}  // namespace la
