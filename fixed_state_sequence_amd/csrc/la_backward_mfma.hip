// Gradients of the causal prefill by chunks on CDNA4 MFMA (gfx950), for
// bf16 inputs, d' = d_v = D in {64, 128}: elu+1 features with no decay, the
// SSD decay or the RFA gate, or identity features with the mLSTM gates.
//
// With L = sum_t <dout_t, o_t>, o_t = num_t r_t (r_t = 1 / (den_t + eps), or
// 1 / max(|den_t|, 1), or 1), the recurrence S_t = alpha_t S_{t-1} +
// beta_t phi(k_t) v_t^T (llm-arch-kb "Linear Attention", section 2; wikillm
// "Linear attention", Implementation sketch, SSD and RFA: (alpha, beta) =
// (1, 1), (a_t, 1) or (g_t, 1 - g_t)) gives, with the weights
// w_ts = beta_s prod_{r=s+1..t} alpha_r, g_t = r_t dout_t and h_t the
// gradient of the divisor (-r_t dout_t . o_t for the sum read-out):
//   dphi(q_t) = sum_{s<=t} w_ts (g_t . v_s + h_t) phi(k_s)   (= S_t g_t + z_t h_t)
//   dphi(k_s) = sum_{t>=s} w_ts (g_t . v_s + h_t) phi(q_t)   (= beta_s (G_s v_s + gz_s))
//   dv_s      = sum_{t>=s} w_ts (phi(q_t) . phi(k_s)) g_t    (= beta_s G_s^T phi(k_s))
// with the gradient state G_s = sum_{t>=s} (prod_{r=s+1..t} alpha_r)
// phi(q_t) g_t^T, gz_s likewise with h_t.  Both sums have the
// masked-quadratic form of the forward pass, so they take its chunked
// bracketing (efficient-attention lesson "Linear attention", "Implementation
// reality": chunks, quadratic inside, a scan across): inside a chunk the
// C x C score tiles, across chunks the states.  The decay enters through the
// within-chunk log-prefix l_t = sum_{r<=t in the chunk} log alpha_r: the
// weight of (t, s) inside a chunk is beta_s e^{l_t - l_s}, a state carried
// into the chunk reaches token t with e^{l_t}, and key s reaches the chunk's
// end with e^{l_last - l_s}, every factor at most 1.  The decay values'
// gradient goes through log alpha: dL/dl_t = <phi(q_t), dphi(q_t)> -
// <phi(k_t), dphi(k_t)>, and dL/dlog alpha_r is its suffix sum over t >= r;
// beta's own gradient is <phi(k_s), dphi(k_s)> / beta_s.
//
// mLSTM gates (wikillm "Linear attention", Variants / mLSTM): the state is
// carried scaled by the forward's stabiliser m_t = max(log f_t + m_{t-1},
// itilde_t), so the recurrence is the one above with alpha'_t = e^{log f_t
// + m_{t-1} - m_t} and beta'_t = e^{itilde_t - m_t}, both at most 1, and
// the read-out of the scaled state has its max1 floor at e^{-m_t}.  Pass A
// rebuilds m_t per chunk from each segment's start stabiliser (the
// prefill's scan) and leaves log alpha'_t, beta'_t for pass B.  L depends
// on the gates through the true alpha = f, beta = e^{itilde}: dL/dlog f_r
// is the suffix sum above, and dL/ditilde_r = beta'_r kd_r with kd_r =
// <phi(k_r), dphi(k_r)> / beta'_r as pass B leaves it; no gate gradient
// divides by a decay.
//
// Schedule (one workgroup per segment of whole 32-token chunks):
//   forward stages 1 and 2 of the prefill: the start state of every segment;
//   pass A (chunks in order): the forward read-out again (r_t, h_t, g_t),
//     dq, <phi(q_t), dphi(q_t)>, and the segment's share of the gradient
//     state, G_seg = sum over its tokens of (decay from the segment's start)
//     phi(q_t) g_t^T (and gz_seg), with the segment's total log-decay; the
//     state is held twice in registers (S and S^T, one per kind of wave;
//     see bwd_pass_a2);
//   reverse scan over the segments: G at every segment's end, and
//     dS0 = G before the first token, dz0 likewise;
//   pass B (chunks in reverse): dk, dv and <phi(k_s), dphi(k_s)> / beta_s
//     from the carried G, held twice in registers (G and G^T, one per kind
//     of wave; see bwd_pass_b2);
//   with a decay, a suffix sum per sequence turns the per-token terms into
//   the decay or gate gradient.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, g = lane / 32, n = lane % 32): an
// operand register holds k-values 8 g .. 8 g + 7 of row n; the accumulator
// holds column n, rows 8 (i / 4) + 4 g + i % 4.  Score tiles are computed
// with the token that is summed over on the accumulator's row axis, so that
// the accumulator, packed to bf16, is the next product's operand when the
// other operand's token axis is read in the permuted order perm_pos (every
// token tile is stored with its rows at perm_pos(token)).
//
// Precision.  Every product takes both operands as bf16 high + low parts
// (three MFMAs: hi hi, lo hi, hi lo), so each carries about 2^-16 relative
// error; v, and the identity features of bf16 inputs (the mLSTM gates), are
// exact in bf16, so the products with them take two MFMAs, or one.  Plain bf16 operands do not suffice here:
// the read-out's error reaches h = -g.o, and the terms S g + z h (and
// G v + gz) cancel down to sum_s phi(k_s) g.(v_s - o_t), amplifying it; the
// states and the score sums are random-sign sums whose rounding error stays
// near 2^-9 of their size instead of averaging out; and without decay the
// gradients of the first tokens are the largest (about 1/sqrt(t)), so an
// error measured against the rms of a long sequence is magnified (about
// 90x at 102400 tokens).
#include "la_internal.h"
#include "la_mfma_common.h"

#include <type_traits>

namespace la {
namespace {

constexpr int BCH = 32;                // chunk length
constexpr float kLogFloorB = -80.0f;   // log alpha floor: alpha = 0 stays finite

struct BwArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const void* dout;
  const float* decay;   // [BH, T] alpha (SSD), the gate g (RFA) or the mLSTM forget
                        // pre-activation; null without decay
  const float* igate;   // mLSTM: [BH, T] input-gate pre-activations
  // mLSTM: the stabiliser of each segment's start state at m0 + bh * m0_bh
  // + s (null: 0, the zero start state's)
  const float* m0;
  int64_t m0_bh;
  int fgate_exp;        // mLSTM: the forget pre-activation is log f itself
  int dout_f32;
  // start state of (b, h) and segment s at S0 + bh * s_bh + s * s_seg (z at
  // z0 + bh * z_bh + s * s_seg); null: zero
  const float* S0;
  const float* z0;
  int64_t s_bh, z_bh, s_seg;
  float* dq;
  float* dk;
  float* dv;
  float* gslot;  // [BH, nseg, D*D + D]: G_seg (pass A), then G at the segment's end (reverse scan)
  float* lgam;   // [BH, nseg]: the segment's total log-decay (pass A, with a decay)
  float* tok;    // [BH, T, 2]: r_t and h_t
  float* qd;     // [BH, T]: <phi(q_t), dphi(q_t)> (pass A, with a decay)
  float* kd;     // [BH, T]: <phi(k_t), dphi(k_t)> / beta_t (pass B, with a decay)
  float* dpart;  // [BH, ceil(T / DG_TILE)]: per-tile totals of the decay gradient's terms
  float* ab;     // mLSTM: [BH, T, 2]: log alpha'_t and beta'_t (pass A, for pass B)
  float* digate; // mLSTM: [BH, T]: dL/d input-gate pre-activation
  int T, cps, nseg, norm;
  float eps;
};

// This lane's index within its wave (0..63), formed anew where it is used:
// a value the compiler cannot move out of a loop, so the addresses derived
// from it are not held (and spilled) across the loop.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 x;
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.f;
  return x;
}

// The accumulator rows 8 (i / 4) + 4 g + i % 4, as bf16 high and low parts:
// the two k-steps of the next product.
__device__ __forceinline__ void split_acc(const f32x16& x, u32x4 (&hi)[2], u32x4 (&lo)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, l;
      split_bf16(x[8 * ks + 2 * e], x[8 * ks + 2 * e + 1], h, l);
      hi[ks][e] = h;
      lo[ks][e] = l;
    }
}

// Four features at byte offset `off` of a token row of a high/low tile pair,
// as fp32 (high + low carry phi to about 2^-16).  EX: the high parts are
// exact (bf16 inputs under identity features), the low tile is not read.
template <bool EX = false>
__device__ __forceinline__ f32x4 hilo4(const char* hi, const char* lo, int off) {
  const u32x2 h = *reinterpret_cast<const u32x2*>(hi + off);
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    r[2 * e] = __uint_as_float(h[e] << 16);
    r[2 * e + 1] = __uint_as_float(h[e] & 0xffff0000u);
  }
  if constexpr (!EX) {
    const u32x2 l = *reinterpret_cast<const u32x2*>(lo + off);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      r[2 * e] += __uint_as_float(l[e] << 16);
      r[2 * e + 1] += __uint_as_float(l[e] & 0xffff0000u);
    }
  }
  return r;
}

// Features 8 b .. 8 b + 7 of tile row `row` (already permuted) of a
// high/low tile pair, as fp32 (EX as in hilo4).
template <int D, bool EX = false>
__device__ __forceinline__ void hilo8(const char* hi, const char* lo, int row, int b, float (&x)[8]) {
  const int off = tile_off<D>(row, b);
  unpack8(*reinterpret_cast<const u32x4*>(hi + off), x, bf16_t{});
  if constexpr (!EX) {
    float l[8];
    unpack8(*reinterpret_cast<const u32x4*>(lo + off), l, bf16_t{});
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += l[e];
  }
}

// NK k-steps of a transposed operand (16 rows each) at columns col0 ..
// col0 + 31, read together before their MFMAs are issued.
template <int D, int NK>
__device__ __forceinline__ void tr_ops(const char* tile, int col0, int lane, u32x4 (&o)[NK]) {
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) o[ks] = tr_operand<D>(tile, 16 * ks, col0, lane);
}

// Sum of v[e] over the lanes of this wave that share lane % BPR (the rows
// the wave stages), written by the first row's lanes to dst[8 b + e].
template <int BPR>
__device__ __forceinline__ void wave_rows_sum8(float (&v)[8], int lane, float* dst) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = group_sum<BPR>(v[e]);
  if (lane < BPR) {
    *reinterpret_cast<f32x4*>(dst + 8 * lane) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(dst + 8 * lane + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// Decay of one chunk, computed by every wave (no barrier needed): lane l
// gets the inclusive log-prefix of token l % 32 in lam and its beta in bet,
// the chunk total in tot.  Tokens past the end have alpha = 1, beta = 0.
template <int DECAY>
__device__ __forceinline__ void chunk_decay(float alpha, int t0, int T, int lane, float& lam,
                                            float& bet, float& tot) {
  const bool valid = t0 + (lane & 31) < T;
  float la = 0.f;
  bet = 0.f;
  if (valid) {
    la = fmaxf(__logf(alpha), kLogFloorB);
    bet = DECAY == 2 ? 1.f - alpha : 1.f;
  }
  lam = wave_scan<32>(la, 0.f, ScanAdd{});
  tot = lane_bcast(lam, 31);
}

// One step of a prefix over the maps x -> max(x + A, B): the map of the lane
// that the DPP control CTRL reaches (the identity (0, -1e30) where none) is
// composed before this lane's.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void maxplus_step(float& A, float& B) {
  const float Ap = dpp_or<CTRL, ROWS>(A, 0.f), Bp = dpp_or<CTRL, ROWS>(B, -1e30f);
  B = fmaxf(Bp + A, B);
  A = Ap + A;
}

// The mLSTM gates of one chunk in the stabilised frame, computed by every
// wave (no barrier needed): from the stabiliser m before the chunk (mst, in
// every lane; replaced by the one after it), lane l gets for token l % 32
// the stabiliser m_t = max(log f_t + m_{t-1}, itilde_t) in mt, the
// inclusive log-prefix of alpha'_t = e^{log f_t + m_{t-1} - m_t} in lam and
// beta'_t = e^{itilde_t - m_t} in bet (la: log alpha'_t itself), the chunk
// total in tot.  m_t is a prefix over the maps x -> max(x + log f_t,
// itilde_t), which compose as (A1, B1) then (A2, B2) = (A1 + A2, max(B1 +
// A2, B2)).  Tokens past the end are the identity map (alpha' = 1, beta' = 0).
__device__ __forceinline__ void chunk_decay_ml(float fpre, float ipre, int fexp, int t0, int T,
                                               int lane, float& mst, float& mt, float& la,
                                               float& lam, float& bet, float& tot) {
  const int l = lane & 31;
  const bool valid = t0 + l < T;
  const float lf = valid ? log_forget(fpre, fexp) : 0.f;
  float A = lf, B = valid ? ipre : -1e30f;
  // the prefix over lanes 0-31 (and 32-63 alike) in the steps of wave_scan
  maxplus_step<0x111>(A, B);
  maxplus_step<0x112>(A, B);
  maxplus_step<0x114>(A, B);
  maxplus_step<0x118>(A, B);
  maxplus_step<0x142, 0xA>(A, B);
  mt = fmaxf(mst + A, B);
  float mp = dpp_or<0x138>(mt, mst);   // wave_shr:1, the previous token's m
  if (l == 0) mp = mst;
  la = valid ? fmaxf(lf + mp - mt, kLogFloorB) : 0.f;
  bet = valid ? __expf(ipre - mt) : 0.f;
  lam = wave_scan<32>(la, 0.f, ScanAdd{});
  tot = lane_bcast(lam, 31);
  mst = lane_bcast(mt, 31);
}

// ------------------------------------------------------------ reverse scan

// Per element of (G, gz) of one (b, h): the slot of segment u becomes G at
// u's end, carry = G_seg(u) + Gamma_u carry over the segments from the last;
// the final carry (G before the first token) is dS0 (dz0).
template <int D, bool DECAY>
__global__ __launch_bounds__(256) void bwd_rscan(float* gslot, const float* lgam, int nseg,
                                                 float* dS0, float* dz0) {
  constexpr int E = D * D + D;
  constexpr int PER = (E + 255) / 256;
  const int64_t bh = blockIdx.x / PER;
  const int e = (blockIdx.x % PER) * 256 + threadIdx.x;
  if (e >= E) return;
  float* base = gslot + bh * nseg * int64_t(E) + e;
  float carry = 0.f;
  for (int u = nseg - 1; u >= 0; --u) {
    const float x = base[int64_t(u) * E];
    base[int64_t(u) * E] = carry;
    carry = DECAY ? fmaf(__expf(lgam[bh * nseg + u]), carry, x) : carry + x;
  }
  if (dS0) {
    if (e < D * D) dS0[bh * D * D + e] = carry;
    else dz0[bh * D + (e - D * D)] = carry;
  }
}

// ------------------------------------------------ pass B, split states

// Pass B with the gradient state held twice in registers instead of staged
// in LDS: waves 0 .. NJ-1 ("value waves") hold G itself, rows f and the
// columns j of their 32-wide block, which as an MFMA operand contracts over
// f (dv); waves NJ .. 2 NJ-1 ("feature waves") hold G^T, rows j and the
// columns f of their block, which contracts over j (dk).  Each folds its own
// copy every chunk (the same products, the transposed way), so no state
// tile is split into LDS and read back, and the 64 KB that held it at D = 128
// double-buffer the staged tiles instead: the chunk after the current one is
// staged while the current one is computed, with one barrier per chunk.
// Two waves share each SIMD, one of each kind: value waves compute first and
// stage after, feature waves stage first, so one wave's VALU work meets the
// other's MFMAs.
//
// An accumulator used as an operand carries its k-index in the permuted
// order (perm_pos) of its rows: G's rows come from the columns of phi(q),
// G^T's from those of g.  The tiles are laid out so that every other operand
// meets that order: phi(k) is stored with its features at their perm_pos
// positions (against G in dv), and v is read at permuted positions (two
// 8-byte pieces, against G^T in dk); phi(q) and g stay in natural order, and
// the scores phi(q) . phi(k) read phi(q) at permuted positions to match
// phi(k).
template <int D, int DECAY>
struct BL2 {
  static constexpr int NJ = D / 32;          // 32-wide blocks of D
  static constexpr int NW = 2 * NJ;          // value waves, then feature waves
  static constexpr int NT = 64 * NW;         // threads per workgroup; each kind of wave stages two rows per thread
  static constexpr int BPR = D / 8;
  static constexpr int TILE = BCH * D * 2;
  // one buffer: token tiles (bf16, rows at perm_pos(token), tile_off<D>)
  static constexpr int Q = 0;                // phi(q) high (features in natural order)
  static constexpr int QL = Q + TILE;        // phi(q) low
  static constexpr int K = QL + TILE;        // phi(k) high (feature f at column perm_pos(f))
  static constexpr int KL = K + TILE;        // phi(k) low
  static constexpr int V = KL + TILE;        // v (natural)
  static constexpr int GH = V + TILE;        // g = r_t dout high
  static constexpr int GL = GH + TILE;       // g low
  static constexpr int WH = GL + TILE;       // with a decay: e^{l_t} g high
  static constexpr int WL = WH + TILE;       // and low
  static constexpr int FB = DECAY ? WL + TILE : WH;   // per-buffer scalars (floats from FB)
  static constexpr int LAM = 0;              // l_t [BCH]
  static constexpr int BET = LAM + BCH;      // beta_t [BCH]
  static constexpr int HT = BET + BCH;       // h_t [BCH]
  static constexpr int HW = HT + BCH;        // e^{l_t} h_t of the token at tile row p [BCH]
  static constexpr int TOT = HW + BCH;       // the chunk's total log-decay
  static constexpr int NFB = TOT + 4;
  static constexpr int BUF = FB + NFB * 4;   // bytes per buffer, a multiple of 16
  static constexpr int GZ = 2 * BUF;         // gz [D] (each feature wave its block)
  static constexpr int KP = GZ + D * 4;      // <phi(k), dphi(k)> / beta partials [2][NJ][BCH]
  static constexpr int LDS = KP + 2 * NJ * BCH * 4;
  static_assert(BUF % 16 == 0, "buffers stay 16-byte aligned");
};

// Row operand of k-step ks with the features in the permuted order: lane
// group g holds features 16 ks + perm_pos(8 g + e), e = 0..7, of row r (two
// 8-byte pieces of a tile stored in natural order).
template <int D>
__device__ __forceinline__ u32x4 row_operand_perm(const char* tile, int r, int ks, int g) {
  const int p0 = 16 * ks + perm_pos(8 * g), p1 = 16 * ks + perm_pos(8 * g + 4);
  const u32x2 x = *reinterpret_cast<const u32x2*>(tile + tile_off<D>(r, p0 >> 3) + ((p0 & 7) << 1));
  const u32x2 y = *reinterpret_cast<const u32x2*>(tile + tile_off<D>(r, p1 >> 3) + ((p1 & 7) << 1));
  return u32x4{x[0], x[1], y[0], y[1]};
}

// A load at a uniform base plus a 32-bit byte offset: the global load's
// scalar-address form, one offset register, where an element offset widened
// to 64 bits costs a 64-bit vector add per load.  The offsets here stay
// within a chunk's rows.
template <class V, class T>
__device__ __forceinline__ V ld_at(const T* base, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Pass B2's staging is split by kind of wave.  Each thread covers rows r0
// and r0 + 16 of feature block b (r0 = i / BPR, b = i % BPR, i = its index
// among the threads of its kind).  The value waves' threads stage phi(q),
// g = r_t dout (with a decay also e^{l_t} g), the decay's prefix, beta and
// total, and h_t; the feature waves' threads stage v.  The value waves
// stage after their products, the feature waves before theirs; the feature
// waves' products are the longer part of a chunk, so they get the least of
// the staging.  phi(k) goes with the value waves' part, except with identity
// features (mLSTM), where it is the raw k and costs little to stage: there
// the feature waves take it (measured faster both ways round).
template <int DECAY>
constexpr bool b2_k_on_value() { return DECAY != 3; }

// Raw inputs of one chunk for one thread of the split staging.
struct Raw2 {
  u32x4 x[2];         // value threads: q of both rows; feature threads: v
  u32x4 y[2];         // k of both rows (for the kind that stages phi(k))
  u32x4 d[2][2];      // value threads: dout of both rows as loaded (8 fp32: both words; 8 bf16: the first)
  float2 th[2];       // value threads: r_t and h_t of both rows (from pass A)
  float2 al;          // value threads: alpha of token lane % 32 (mLSTM: log alpha', beta', from pass A)
};

template <int D, int DECAY, bool DF32, bool VR>
__device__ __forceinline__ void load_raw2(const BwArgs& a, int64_t bh, int t0, int i, Raw2& x) {
  constexpr int BPR = D / 8;
  constexpr bool KH = VR == b2_k_on_value<DECAY>();   // phi(k) staged here
  const int r0 = i / BPR, b = i % BPR;
  // the chunk's first token (uniform), and 32-bit offsets within the chunk
  // (rows past the end read the last token)
  const int64_t tc = bh * int64_t(a.T) + t0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t tr = uint32_t(min(t0 + r0 + 16 * h, a.T - 1) - t0);
    const uint32_t off = tr * D + 8 * b;
    if constexpr (KH) x.y[h] = ld_at<u32x4>(a.k + tc * D, 2 * off);
    if constexpr (VR) {
      x.x[h] = ld_at<u32x4>(a.q + tc * D, 2 * off);
      x.th[h] = ld_at<float2>(a.tok + tc * 2, 8 * tr);
      if constexpr (DF32) {
        const float* dp = static_cast<const float*>(a.dout) + tc * D;
        x.d[h][0] = ld_at<u32x4>(dp, 4 * off);
        x.d[h][1] = ld_at<u32x4>(dp, 4 * off + 16);
      } else {
        x.d[h][0] = ld_at<u32x4>(static_cast<const bf16_t*>(a.dout) + tc * D, 2 * off);
      }
    } else {
      x.x[h] = ld_at<u32x4>(a.v + tc * D, 2 * off);
    }
  }
  if constexpr (VR) {
    x.al = make_float2(1.f, 1.f);
    const uint32_t ta = uint32_t(min(t0 + (i & 31), a.T - 1) - t0);
    if constexpr (DECAY == 3) x.al = ld_at<float2>(a.ab + tc * 2, 8 * ta);
    else if constexpr (DECAY != 0) x.al.x = ld_at<float>(a.decay + tc, 4 * ta);
  }
}

// Stage this thread's part of one chunk into buffer buf: phi(q) (high, low),
// phi(k) (high, low, at permuted feature positions), v, g = r_t dout (high,
// low; with a decay also e^{l_t} g), and the per-token scalars.  Rows past
// the end are zero (FULL: the chunk lies wholly inside the sequence, and no
// row is tested).
template <int D, int DECAY, bool DF32, bool VR, bool FULL = false>
__device__ __forceinline__ void stage2(const BwArgs& a, int t0, int i, const Raw2& x, char* buf) {
  using L = BL2<D, DECAY>;
  constexpr bool KH = VR == b2_k_on_value<DECAY>();   // phi(k) staged here
  float* F = reinterpret_cast<float*>(buf + L::FB);
  const int r0 = i / L::BPR, b = i % L::BPR, lane = i & 63;
  float lam = 0.f, bet = 1.f, tot = 0.f;
  if constexpr (VR) {
    if constexpr (DECAY == 3) {
      // log alpha' and beta' as pass A left them
      const bool vt = t0 + (lane & 31) < a.T;
      lam = wave_scan<32>(vt ? x.al.x : 0.f, 0.f, ScanAdd{});
      bet = vt ? x.al.y : 0.f;
      tot = lane_bcast(lam, 31);
    } else if constexpr (DECAY != 0) {
      chunk_decay<DECAY>(x.al.x, t0, a.T, lane, lam, bet, tot);
    }
    if (i < BCH) {
      F[L::LAM + i] = lam;
      F[L::BET + i] = bet;
      if (i == 0) F[L::TOT] = tot;
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 16 * h;
    const bool valid = FULL || t0 + r < a.T;
    const int pr = perm_pos(r);
    if constexpr (KH) {
      float fk[8];
      unpack8(x.y[h], fk, bf16_t{});
#pragma unroll
      for (int e = 0; e < 8; ++e) fk[e] = valid ? (DECAY == 3 ? fk[e] : elu1_fast(fk[e])) : 0.f;
      // identity features of bf16 inputs (mLSTM) are exact in bf16: no low parts
      const u32x4 kh = pack8(fk);
      row_write_perm<D>(buf + L::K, pr, b, kh);
      if constexpr (DECAY != 3) row_write_perm<D>(buf + L::KL, pr, b, low8(fk, kh));
    }
    if constexpr (VR) {
      float fq[8];
      unpack8(x.x[h], fq, bf16_t{});
#pragma unroll
      for (int e = 0; e < 8; ++e) fq[e] = valid ? (DECAY == 3 ? fq[e] : elu1_fast(fq[e])) : 0.f;
      const u32x4 qh = pack8(fq);
      blk_write<D>(buf + L::Q, pr, b, qh);
      if constexpr (DECAY != 3) blk_write<D>(buf + L::QL, pr, b, low8(fq, qh));
      float lr = 0.f;
      if constexpr (DECAY != 0) lr = __shfl(lam, r);
      const float rt = valid ? x.th[h].x : 0.f, ht = valid ? x.th[h].y : 0.f;
      float gv[8];
      if constexpr (DF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[e] = __uint_as_float(x.d[h][0][e]);
          gv[e + 4] = __uint_as_float(x.d[h][1][e]);
        }
      } else {
        unpack8(x.d[h][0], gv, bf16_t{});
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] *= rt;
      const u32x4 gh = pack8(gv);
      blk_write<D>(buf + L::GH, pr, b, gh);
      blk_write<D>(buf + L::GL, pr, b, low8(gv, gh));
      const float wq = DECAY ? __expf(lr) : 1.f;   // query weight from the chunk's start
      if constexpr (DECAY != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] *= wq;
        const u32x4 wh = pack8(gv);
        blk_write<D>(buf + L::WH, pr, b, wh);
        blk_write<D>(buf + L::WL, pr, b, low8(gv, wh));
      }
      if (b == 0) {
        F[L::HT + r] = ht;
        F[L::HW + pr] = wq * ht;
      }
    } else {
      blk_write<D>(buf + L::V, pr, b, valid ? x.x[h] : u32x4{0u, 0u, 0u, 0u});
    }
  }
}

// The causal weights of the score tile held by this lane (column s = n, rows
// t = 8 (i / 4) + 4 g + i % 4): e^{l_t - l_s} for t >= s, else 0.
template <int DECAY>
__device__ __forceinline__ void causal_weights(const float* F, int LAMOFF, int g, int n,
                                               float (&wt)[16]) {
  const float ls = DECAY ? F[LAMOFF + n] : 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    f32x4 lt = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DECAY != 0) lt = *reinterpret_cast<const f32x4*>(F + LAMOFF + 8 * q4 + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 8 * q4 + 4 * g + e;
      wt[4 * q4 + e] = t >= n ? (DECAY ? __expf(lt[e] - ls) : 1.f) : 0.f;
    }
  }
}

template <int D, int DECAY, bool DF32>
__global__ __launch_bounds__(128 * (D / 32)) void bwd_pass_b2(const BwArgs a) {
  using L = BL2<D, DECAY>;
  constexpr int NJ = L::NJ, KS = D / 16;
  constexpr bool XQ = DECAY == 3;   // exact phi(q), phi(k): no low parts (the header's precision note)
  __shared__ __align__(16) char smem[L::LDS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, n = lane & 31;
  const bool value_wave = w < NJ;
  const int wb = value_wave ? w : w - NJ;   // this wave's 32-wide block (j or f)
  const int64_t bh = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int T = a.T;
  const int nchunks = (T + BCH - 1) / BCH;
  const int c0 = seg * a.cps, c1 = min(c0 + a.cps, nchunks);
  if (c0 >= c1) return;   // the whole workgroup: no barrier is reached

  // G at the segment's end (slot layout rows f, columns j): value waves
  // hold X[fb] = rows f of block fb, columns j of block wb; feature waves
  // X[jb] = rows j of block jb, columns f of block wb
  f32x16 X[NJ];
  {
    const float* src = a.gslot + (bh * a.nseg + seg) * int64_t(D * D + D);
#pragma unroll
    for (int ob = 0; ob < NJ; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * ob + 8 * (i >> 2) + 4 * g + (i & 3), col = 32 * wb + n;
        X[ob][i] = value_wave ? src[row * D + col] : src[col * D + row];
      }
    if (!value_wave && g == 0)
      reinterpret_cast<float*>(smem + L::GZ)[32 * wb + n] = src[D * D + 32 * wb + n];
  }

  // the last chunk staged, the one before it loaded; each kind of wave its
  // part (si: the thread's index among the threads of its kind)
  Raw2 raw;
  const int si = tid & (64 * NJ - 1);
  auto first = [&](auto value_kind) {
    constexpr bool VR = decltype(value_kind)::value;
    load_raw2<D, DECAY, DF32, VR>(a, bh, (c1 - 1) * BCH, si, raw);
    stage2<D, DECAY, DF32, VR>(a, (c1 - 1) * BCH, si, raw, smem);
    if (c1 - 2 >= c0) load_raw2<D, DECAY, DF32, VR>(a, bh, (c1 - 2) * BCH, si, raw);
  };
  if (value_wave) first(std::true_type{});
  else first(std::false_type{});
  __syncthreads();

  // one loop per kind of wave (each keeps only its own loop-invariant
  // addresses live), the same barriers in both
  auto chunk = [&](int c, auto value_kind) {
    constexpr bool VW = decltype(value_kind)::value;
    const int t0 = c * BCH;
    const char* cur = smem + ((c1 - 1 - c) & 1) * L::BUF;
    char* nxt = smem + ((c1 - c) & 1) * L::BUF;
    const float* F = reinterpret_cast<const float*>(cur + L::FB);
    const bool more = c - 1 >= c0;
    // the next chunk (c - 1) into the other buffer, and its successor's raw
    // inputs in flight: feature waves before their products, value waves after
    auto stage_next = [&]() {
      if (more) {
        // the staging addresses are recomputed from an opaque copy of the
        // thread index: held across the loop with the products' addresses,
        // they would not fit the registers of two waves per SIMD
        int ts = tid;
        asm volatile("" : "+v"(ts));
        ts &= 64 * NJ - 1;
        stage2<D, DECAY, DF32, VW, true>(a, t0 - BCH, ts, raw, nxt);   // every chunk but the last is whole
        if (c - 2 >= c0) load_raw2<D, DECAY, DF32, VW>(a, bh, t0 - 2 * BCH, ts, raw);
      }
    };
    const bool vs = t0 + n < T;
    const float tot = DECAY ? F[L::TOT] : 0.f;
    const float es = DECAY ? __expf(tot - F[L::LAM + n]) : 1.f;   // key n to the chunk's end
    const float bet = DECAY >= 2 ? F[L::BET + n] : 1.f;
    const float ec = DECAY ? __expf(tot) : 1.f;
    float wt[16];
    constexpr int GA = DECAY ? L::WH : L::GH, GB = DECAY ? L::WL : L::GL;

    if constexpr (VW) {
      // dv^T / beta_s (rows j of block wb, columns s): e^{l_last - l_s}
      // G^T phi(k) + g^T A, with G from the registers (contracting over f);
      // the G products first, so that the state's split meets the scores'
      // MFMAs
      f32x16 dvt = zero16();
#pragma unroll
      for (int fb = 0; fb < NJ; ++fb) {
        u32x4 sh[2], sl[2], bk[2], bkl[2];
        split_acc(X[fb], sh, sl);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bk[ks] = row_operand<D>(cur + L::K, perm_pos(n), 2 * (2 * fb + ks) + g);
          if constexpr (!XQ) bkl[ks] = row_operand<D>(cur + L::KL, perm_pos(n), 2 * (2 * fb + ks) + g);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dvt = mfma(sh[ks], bk[ks], dvt);
          dvt = mfma(sl[ks], bk[ks], dvt);
          if constexpr (!XQ) dvt = mfma(sh[ks], bkl[ks], dvt);
        }
      }
      if constexpr (DECAY != 0) dvt *= es;

      // scores A (rows t, columns s = n): phi(q) at permuted feature
      // positions against phi(k) stored that way
      f32x16 at = zero16();
#pragma unroll
      for (int k0 = 0; k0 < KS; k0 += 2) {
        u32x4 aq[2], aql[2], bk[2], bkl[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          aq[kk] = row_operand_perm<D>(cur + L::Q, perm_pos(n), k0 + kk, g);
          bk[kk] = row_operand<D>(cur + L::K, perm_pos(n), 2 * (k0 + kk) + g);
          if constexpr (!XQ) {
            aql[kk] = row_operand_perm<D>(cur + L::QL, perm_pos(n), k0 + kk, g);
            bkl[kk] = row_operand<D>(cur + L::KL, perm_pos(n), 2 * (k0 + kk) + g);
          }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          at = mfma(aq[kk], bk[kk], at);
          if constexpr (!XQ) {
            at = mfma(aq[kk], bkl[kk], at);
            at = mfma(aql[kk], bk[kk], at);
          }
        }
      }
      causal_weights<DECAY>(F, L::LAM, g, n, wt);
#pragma unroll
      for (int i = 0; i < 16; ++i) at[i] *= wt[i];
      u32x4 ah[2], al[2];
      split_acc(at, ah, al);

      u32x4 ogt[2], oglt[2];
      tr_ops<D, 2>(cur + L::GH, 32 * wb, lane, ogt);
      tr_ops<D, 2>(cur + L::GL, 32 * wb, lane, oglt);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dvt = mfma(ogt[ks], ah[ks], dvt);
        dvt = mfma(ogt[ks], al[ks], dvt);
        dvt = mfma(oglt[ks], ah[ks], dvt);
      }
      if (vs) {
        float* dst = a.dv + (bh * T + t0) * D + uint32_t(n * D + 32 * wb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<f32x4*>(dst + 8 * r) =
              f32x4{bet * dvt[4 * r], bet * dvt[4 * r + 1], bet * dvt[4 * r + 2],
                    bet * dvt[4 * r + 3]};
      }

      // G (rows f, columns j of block wb) = e^{l_last} G + phi(Q)^T (e^{l_t} g)
      u32x4 ag[2], agl[2];
      if constexpr (DECAY != 0) {
        tr_ops<D, 2>(cur + GA, 32 * wb, lane, ag);
        tr_ops<D, 2>(cur + GB, 32 * wb, lane, agl);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          ag[ks] = ogt[ks];
          agl[ks] = oglt[ks];
        }
      }
#pragma unroll
      for (int fb = 0; fb < NJ; ++fb) {
        u32x4 bq[2], bql[2];
        tr_ops<D, 2>(cur + L::Q, 32 * fb, lane, bq);
        if constexpr (!XQ) tr_ops<D, 2>(cur + L::QL, 32 * fb, lane, bql);
        if constexpr (DECAY != 0) X[fb] *= ec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          X[fb] = mfma(bq[ks], ag[ks], X[fb]);
          if constexpr (!XQ) X[fb] = mfma(bql[ks], ag[ks], X[fb]);
          X[fb] = mfma(bq[ks], agl[ks], X[fb]);
        }
      }
      stage_next();
    } else {
      stage_next();
      // dphi(k)^T / beta_s (rows f of block wb, columns s): e^{l_last - l_s}
      // (G v + gz) + phi(Q)^T B, with G^T from the registers (contracting
      // over j) against v read at permuted positions; the G^T products first,
      // so that the state's split meets B's MFMAs
      f32x16 dkt = zero16();
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 sh[2], sl[2], ov[2];
        split_acc(X[jb], sh, sl);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) ov[ks] = row_operand_perm<D>(cur + L::V, perm_pos(n), 2 * jb + ks, g);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dkt = mfma(sh[ks], ov[ks], dkt);
          dkt = mfma(sl[ks], ov[ks], dkt);
        }
      }
      if constexpr (DECAY != 0) dkt *= es;

      // B (rows t, columns s = n): g_t . v_s + h_t
      f32x16 bt = zero16();
#pragma unroll
      for (int k0 = 0; k0 < KS; k0 += 2) {
        u32x4 gh[2], gl[2], ov[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          gh[kk] = row_operand<D>(cur + L::GH, perm_pos(n), 2 * (k0 + kk) + g);
          gl[kk] = row_operand<D>(cur + L::GL, perm_pos(n), 2 * (k0 + kk) + g);
          ov[kk] = row_operand<D>(cur + L::V, perm_pos(n), 2 * (k0 + kk) + g);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bt = mfma(gh[kk], ov[kk], bt);
          bt = mfma(gl[kk], ov[kk], bt);
        }
      }
      causal_weights<DECAY>(F, L::LAM, g, n, wt);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 h4 = *reinterpret_cast<const f32x4*>(F + L::HT + 8 * q4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) bt[4 * q4 + e] = (bt[4 * q4 + e] + h4[e]) * wt[4 * q4 + e];
      }
      u32x4 bh_[2], bl_[2];
      split_acc(bt, bh_, bl_);

      u32x4 oqt[2], oqlt[2];
      tr_ops<D, 2>(cur + L::Q, 32 * wb, lane, oqt);
      if constexpr (!XQ) tr_ops<D, 2>(cur + L::QL, 32 * wb, lane, oqlt);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dkt = mfma(oqt[ks], bh_[ks], dkt);
        dkt = mfma(oqt[ks], bl_[ks], dkt);
        if constexpr (!XQ) dkt = mfma(oqlt[ks], bh_[ks], dkt);
      }
      float* gzl = reinterpret_cast<float*>(smem + L::GZ);
      {
        float kdp = 0.f;   // <phi(k_s), dphi(k_s)> / beta_s over this lane's features
        float* dst = a.dk + (bh * T + t0) * D + uint32_t(n * D + 32 * wb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pc = perm_pos(32 * wb + 8 * r + 4 * g);   // stored column of these 4 features
          const int off = tile_off<D>(perm_pos(n), pc >> 3) + ((pc & 7) << 1);
          const f32x4 p4 = hilo4<XQ>(cur + L::K, cur + L::KL, off);
          const f32x4 z4 = *reinterpret_cast<const f32x4*>(gzl + 32 * wb + 8 * r + 4 * g);
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float raw_ = dkt[4 * r + e] + es * z4[e];
            o4[e] = DECAY == 3 ? bet * raw_ : bet * raw_ * fminf(p4[e], 1.f);
            kdp += p4[e] * raw_;
          }
          if (vs) *reinterpret_cast<f32x4*>(dst + 8 * r) = o4;
        }
        if constexpr (DECAY != 0) {
          kdp = swap_sum32(kdp);
          if (g == 0) reinterpret_cast<float*>(smem + L::KP)[((c & 1) * NJ + wb) * BCH + n] = kdp;
        }
      }

      // G^T (rows j, columns f of block wb) = e^{l_last} G^T + (e^{l_t} g)^T phi(Q)
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 ag[2], agl[2];
        tr_ops<D, 2>(cur + GA, 32 * jb, lane, ag);
        tr_ops<D, 2>(cur + GB, 32 * jb, lane, agl);
        if constexpr (DECAY != 0) X[jb] *= ec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          X[jb] = mfma(ag[ks], oqt[ks], X[jb]);
          X[jb] = mfma(agl[ks], oqt[ks], X[jb]);
          if constexpr (!XQ) X[jb] = mfma(ag[ks], oqlt[ks], X[jb]);
        }
      }
      // gz (feature 32 wb + n) = e^{l_last} gz + sum_t e^{l_t} h_t phi(q_t):
      // this lane's tokens are the tile rows of its phi(q) operands
      float inc = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(F + L::HW + 16 * ks + 8 * g);
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(F + L::HW + 16 * ks + 8 * g + 4);
        float ph[8];
        unpack8(oqt[ks], ph, bf16_t{});
        if constexpr (!XQ) {
          float pl[8];
          unpack8(oqlt[ks], pl, bf16_t{});
#pragma unroll
          for (int e = 0; e < 8; ++e) ph[e] += pl[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          inc += ph[e] * h0[e];
          inc += ph[e + 4] * h1[e];
        }
      }
      inc = swap_sum32(inc);
      if (g == 0) gzl[32 * wb + n] = fmaf(ec, gzl[32 * wb + n], inc);
    }
    __syncthreads();   // chunk c - 1 staged; every read of chunk c's buffer done
    if constexpr (DECAY != 0 && !VW) {
      if (w == NJ && lane < BCH && t0 + lane < T) {
        const float* kp = reinterpret_cast<const float*>(smem + L::KP) + (c & 1) * NJ * BCH;
        float s = 0.f;
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) s += kp[jb * BCH + lane];
        a.kd[bh * T + t0 + lane] = s;
      }
    }
  };
  if (value_wave)
    for (int c = c1 - 1; c >= c0; --c) chunk(c, std::true_type{});
  else
    for (int c = c1 - 1; c >= c0; --c) chunk(c, std::false_type{});
}

// ------------------------------------------------------------ pass A2

// Pass A with the state held twice in registers instead of staged in LDS
// (as pass B holds the gradient state): waves 0 .. NJ-1 ("value waves") hold
// S itself, rows f and the columns j of their 32-wide block, which as an
// MFMA operand contracts over f (the numerator phi(q) . S); waves NJ ..
// 2 NJ-1 ("feature waves") hold S^T, rows j and the columns f of their block,
// which contracts over j (dphi(q) = S g).  Each folds its own copy every
// chunk.  A chunk takes two phases, each ended by a barrier:
//   1. value waves: the scores, the read-out (r_t, the numerator) and g_t =
//      r_t dout_t into LDS with the partials of dout_t . o_t; feature waves
//      meanwhile stage the next chunk into the other buffer;
//   2. feature waves: h_t, B, dphi(q) and their fold; value waves their fold.
// Two waves share each SIMD, one of each kind, so one wave's VALU work meets
// the other's MFMAs.  The staging carries z one chunk ahead: staging chunk
// c + 1 forms z at its start from z at chunk c's start and the increments
// staged with chunk c, and phi(q) . z with it.  dout goes from global memory
// straight into the value waves' registers (loaded a chunk ahead).
//
// Operand orders: an accumulator used as an operand carries its k-index in
// the permuted order of its rows, so phi(q) (against S) and g (against S^T)
// are stored with their features at perm_pos positions; phi(k) and v stay
// natural, and are read at permuted positions where they meet phi(q) (the
// scores) or g (B).
template <int D, int DECAY>
struct BL3 {
  static constexpr int NJ = D / 32;          // 32-wide blocks of D
  static constexpr int NW = 2 * NJ;          // value waves, then feature waves
  static constexpr int BPR = D / 8;          // 16-byte blocks per bf16 row
  static constexpr int TILE = BCH * D * 2;
  static constexpr bool XQ = DECAY == 3;     // exact phi: no low tiles
  static constexpr bool WT = DECAY != 0;     // weighted key tiles (else phi(k) serves)
  // one buffer: token tiles (bf16, rows at perm_pos(token), tile_off<D>)
  static constexpr int Q = 0;                        // phi(q) high (features at perm_pos)
  static constexpr int QL = Q + TILE;                // phi(q) low
  static constexpr int K = XQ ? QL : QL + TILE;      // phi(k) high (natural)
  static constexpr int KL = K + TILE;                // phi(k) low
  static constexpr int V = XQ ? KL : KL + TILE;      // v (natural)
  static constexpr int WK = V + TILE;                // w_s phi(k_s) high, w_s = beta_s e^{l_last - l_s}
  static constexpr int WKL = WK + TILE;              // and low
  static constexpr int FB = WT ? WKL + TILE : WK;    // per-buffer scalars (floats from FB)
  static constexpr int LAM = 0;              // l_t [BCH]
  static constexpr int BET = LAM + BCH;      // beta_t [BCH]
  static constexpr int DI = BET + BCH;       // phi(q_t) . z, z at the chunk's start [BCH]
  static constexpr int MT = DI + BCH;        // mLSTM: m_t [BCH]
  static constexpr int TOT = MT + BCH;       // the chunk's total log-decay
  static constexpr int ZP = TOT + 4;         // per staging wave increments of z [NJ][D]
  static constexpr int NFB = ZP + NJ * D;
  static constexpr int BUF = FB + NFB * 4;   // bytes per buffer, a multiple of 16
  // shared by both buffers
  static constexpr int G = 2 * BUF;          // g = r_t dout high (features at perm_pos)
  static constexpr int GL = G + TILE;        // g low
  static constexpr int WG = GL + TILE;       // with a decay: e^{L + l_t} g_t high (L: the
                                             // log-decay from the segment's start to the chunk)
  static constexpr int WGL = WG + TILE;      // and low
  static constexpr int SC = WT ? WGL + TILE : WG;   // scalars (floats from SC)
  static constexpr int Z = 0;                // z at the start of chunks of parity p [2][D]
  static constexpr int HP = Z + 2 * D;       // dout . o partials [NJ][BCH]
  static constexpr int RT = HP + NJ * BCH;   // r_t [BCH]
  static constexpr int HF = RT + BCH;        // h_t / (dout_t . o_t) [BCH]
  static constexpr int QP = HF + BCH;        // <phi(q), dphi(q)> partials [NJ][BCH]
  static constexpr int NSC = QP + NJ * BCH;
  static constexpr int LDS = SC + NSC * 4;
  static_assert(BUF % 16 == 0, "buffers stay 16-byte aligned");
};

// Raw inputs of one chunk for a staging thread (feature waves): rows r and
// r + 16, block b; and token lane % 32's decay values.
struct Raw3 {
  u32x4 q[2], k[2], v[2];
  float al, ig;
};

template <int D, int DECAY>
__device__ __forceinline__ void load_raw3(const BwArgs& a, int64_t bh, int t0, int ft, Raw3& x) {
  constexpr int BPR = D / 8;
  const int r = ft / BPR, b = ft % BPR;
  const int64_t tc = bh * int64_t(a.T) + t0;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const uint32_t off = uint32_t(min(t0 + r + 16 * rr, a.T - 1) - t0) * D + 8 * b;
    x.q[rr] = ld_at<u32x4>(a.q + tc * D, 2 * off);
    x.k[rr] = ld_at<u32x4>(a.k + tc * D, 2 * off);
    x.v[rr] = ld_at<u32x4>(a.v + tc * D, 2 * off);
  }
  x.al = 1.f;
  x.ig = 0.f;
  const uint32_t ta = uint32_t(min(t0 + (ft & 31), a.T - 1) - t0);
  if constexpr (DECAY != 0) x.al = ld_at<float>(a.decay + tc, 4 * ta);
  if constexpr (DECAY == 3) x.ig = ld_at<float>(a.igate + tc, 4 * ta);
}

// dout of token t0 + n at features 32 wb + 8 r + 4 g .. + 3, r = 0..3, for a
// value wave: fp32 (one block per r) or bf16 (two r per block).
template <int D, bool DF32>
__device__ __forceinline__ void load_dout3(const BwArgs& a, int64_t bh, int t0, int wb, int n,
                                           int g, u32x4 (&d)[DF32 ? 4 : 2]) {
  const int64_t tc = bh * int64_t(a.T) + t0;
  const uint32_t off = uint32_t(min(t0 + n, a.T - 1) - t0) * D + 32 * wb + 4 * g;
  if constexpr (DF32) {
    const float* p = static_cast<const float*>(a.dout) + tc * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = ld_at<u32x4>(p, 4 * off + 32 * r);
  } else {
    const bf16_t* p = static_cast<const bf16_t*>(a.dout) + tc * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2 x = ld_at<u32x2>(p, 2 * off + 32 * h);
      const u32x2 y = ld_at<u32x2>(p, 2 * off + 32 * h + 16);
      d[h] = u32x4{x[0], x[1], y[0], y[1]};
    }
  }
}

template <bool DF32>
__device__ __forceinline__ f32x4 dout4(const u32x4 (&d)[DF32 ? 4 : 2], int r) {
  f32x4 o;
  if constexpr (DF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(d[r][e]);
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t w = d[r >> 1][2 * (r & 1) + e];
      o[2 * e] = __uint_as_float(w << 16);
      o[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
  return o;
}

// Stage one chunk into buffer buf (feature waves; ft = thread index among
// them): the decay (mLSTM: the gates in the stabilised frame, m_t carried in
// mst; log alpha', beta' to a.ab), phi(q) (high, low, features at perm_pos),
// phi(k) (high, low), v, with a decay the weighted keys w_s phi(k_s) (high,
// low), z at the chunk's start (from the previous chunk's buffer pbuf and z
// zprev, or zs for a segment's first chunk; null: zero) into znew, phi(q_t)
// . z and this wave's increments of z.  Rows past the end are zero.
template <int D, int DECAY>
__device__ __forceinline__ void stage3(const BwArgs& a, int64_t bh, int t0, int ft, const Raw3& x,
                                       char* buf, const char* pbuf, const float* zprev,
                                       float* znew, bool first, const float* zs, float& mst) {
  using L = BL3<D, DECAY>;
  float* F = reinterpret_cast<float*>(buf + L::FB);
  const int r0 = ft / L::BPR, b = ft % L::BPR, lane = ft & 63, fw = ft >> 6;
  float lam = 0.f, bet = 1.f, tot = 0.f, mt = 0.f;
  if constexpr (DECAY == 3) {
    float la;
    chunk_decay_ml(x.al, x.ig, a.fgate_exp, t0, a.T, lane, mst, mt, la, lam, bet, tot);
    if (fw == 0 && lane < BCH && t0 + lane < a.T)
      *reinterpret_cast<float2*>(a.ab + (bh * a.T + t0 + lane) * 2) = make_float2(la, bet);
  } else if constexpr (DECAY != 0) {
    chunk_decay<DECAY>(x.al, t0, a.T, lane, lam, bet, tot);
  }
  if (fw == 0 && lane < BCH) {
    F[L::LAM + lane] = lam;
    F[L::BET + lane] = bet;
    if constexpr (DECAY == 3) F[L::MT + lane] = mt;
    if (lane == 0) F[L::TOT] = tot;
  }
  // z at this chunk's start, features 8 b .. 8 b + 7
  float z[8];
  if (first) {
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = zs ? zs[8 * b + e] : 0.f;
  } else {
    const float* Fp = reinterpret_cast<const float*>(pbuf + L::FB);
    const float ep = DECAY ? __expf(Fp[L::TOT]) : 1.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 s = *reinterpret_cast<const f32x4*>(zprev + 8 * b + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] *= ep;
#pragma unroll
      for (int ww = 0; ww < L::NJ; ++ww) s += *reinterpret_cast<const f32x4*>(Fp + L::ZP + ww * D + 8 * b + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) z[4 * h + e] = s[e];
    }
  }
  if (r0 == 0) {
    *reinterpret_cast<f32x4*>(znew + 8 * b) = f32x4{z[0], z[1], z[2], z[3]};
    *reinterpret_cast<f32x4*>(znew + 8 * b + 4) = f32x4{z[4], z[5], z[6], z[7]};
  }
  float inc[8];   // set by the first row (adding to 0.f would cost an instruction each)
  // the rows; a chunk wholly inside the sequence takes no validity selects
  auto rows = [&](auto full_kind) {
    constexpr bool FULL = decltype(full_kind)::value;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = r0 + 16 * rr;
      const bool valid = FULL || t0 + r < a.T;
      const int pr = perm_pos(r);
      float lr = 0.f, br = 1.f;   // this row's log-prefix and beta
      if constexpr (DECAY != 0) {
        lr = __shfl(lam, r);
        br = __shfl(bet, r);
      }
      float fq[8], fk[8];
      unpack8(x.q[rr], fq, bf16_t{});
      unpack8(x.k[rr], fk, bf16_t{});
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fq[e] = valid ? (DECAY == 3 ? fq[e] : elu1_fast(fq[e])) : 0.f;
        fk[e] = valid ? (DECAY == 3 ? fk[e] : elu1_fast(fk[e])) : 0.f;
      }
      const u32x4 qh = pack8(fq);
      row_write_perm<D>(buf + L::Q, pr, b, qh);
      if constexpr (!L::XQ) row_write_perm<D>(buf + L::QL, pr, b, low8(fq, qh));
      const u32x4 kh = pack8(fk);
      blk_write<D>(buf + L::K, pr, b, kh);
      if constexpr (!L::XQ) blk_write<D>(buf + L::KL, pr, b, low8(fk, kh));
      blk_write<D>(buf + L::V, pr, b, valid ? x.v[rr] : u32x4{0u, 0u, 0u, 0u});
      const float wk = DECAY ? br * __expf(tot - lr) : 1.f;   // key weight to the chunk's end
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        part += fq[e] * z[e];
        inc[e] = rr == 0 ? wk * fk[e] : fmaf(wk, fk[e], inc[e]);
      }
      if constexpr (L::WT) {
        float wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = wk * fk[e];
        const u32x4 wh = pack8(wv);
        blk_write<D>(buf + L::WK, pr, b, wh);
        blk_write<D>(buf + L::WKL, pr, b, low8(wv, wh));
      }
      part = row_sum<L::BPR>(part);
      if (b == 0) F[L::DI + r] = part;
    }
  };
  if (t0 + BCH <= a.T) rows(std::true_type{});
  else rows(std::false_type{});
  wave_rows_sum8<L::BPR>(inc, lane, F + L::ZP + fw * D);
}

// The causal weights of a tile with rows s = 8 (i / 4) + 4 g + i % 4 and
// column t = n (token n's log-prefix lt): beta_s e^{l_t - l_s} for s <= t.
template <int DECAY>
__device__ __forceinline__ void causal_weights_st(const float* F, int LAMOFF, int BETOFF, float lt,
                                                  int g, int n, float (&wt)[16]) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    f32x4 ls = {0.f, 0.f, 0.f, 0.f}, bs = {1.f, 1.f, 1.f, 1.f};
    if constexpr (DECAY != 0) ls = *reinterpret_cast<const f32x4*>(F + LAMOFF + 8 * q4 + 4 * g);
    if constexpr (DECAY >= 2) bs = *reinterpret_cast<const f32x4*>(F + BETOFF + 8 * q4 + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 8 * q4 + 4 * g + e;
      wt[4 * q4 + e] = s <= n ? (DECAY ? bs[e] * __expf(lt - ls[e]) : 1.f) : 0.f;
    }
  }
}

template <int D, int DECAY, bool DF32>
__global__ __launch_bounds__(128 * (D / 32)) void bwd_pass_a2(const BwArgs a) {
  using L = BL3<D, DECAY>;
  constexpr int NJ = L::NJ, KS = D / 16;
  constexpr bool XQ = L::XQ;
  __shared__ __align__(16) char smem[L::LDS];
  float* Sc = reinterpret_cast<float*>(smem + L::SC);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, n = lane & 31;
  const bool value_wave = w < NJ;
  const int wb = value_wave ? w : w - NJ;   // this wave's 32-wide block (j or f)
  const int64_t bh = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int T = a.T;
  const int nchunks = (T + BCH - 1) / BCH;
  const int c0 = seg * a.cps, c1 = min(c0 + a.cps, nchunks);
  if (c0 >= c1) {
    // no chunks: a zero gradient state (the whole workgroup returns, no
    // barrier is reached)
    float* dst = a.gslot + (bh * a.nseg + seg) * int64_t(D * D + D);
    for (int e = tid; e < D * D + D; e += 64 * L::NW) dst[e] = 0.f;
    if (DECAY != 0 && tid == 0) a.lgam[bh * a.nseg + seg] = 0.f;
    return;
  }

  // the segment's start state (rows f, columns j): value waves hold X[fb] =
  // rows f of block fb, columns j of block wb; feature waves X[jb] = rows j
  // of block jb, columns f of block wb
  f32x16 X[NJ];
  {
    const float* Ss = a.S0 ? a.S0 + bh * a.s_bh + int64_t(seg) * a.s_seg : nullptr;
#pragma unroll
    for (int ob = 0; ob < NJ; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * ob + 8 * (i >> 2) + 4 * g + (i & 3), col = 32 * wb + n;
        X[ob][i] = !Ss ? 0.f : value_wave ? Ss[row * D + col] : Ss[col * D + row];
      }
  }
  const float* zs = a.z0 ? a.z0 + bh * a.z_bh + int64_t(seg) * a.s_seg : nullptr;
  const int ft = tid - 64 * NJ;   // index among the feature waves' threads
  const int wsg = __builtin_amdgcn_readfirstlane(w);   // the wave index, in a scalar register
  float mst = 0.f;                // mLSTM: the stabiliser before the chunk staged next
  if constexpr (DECAY == 3) mst = a.m0 ? a.m0[bh * a.m0_bh + seg] : 0.f;
  Raw3 raw;
  u32x4 dreg[DF32 ? 4 : 2];
  constexpr int WA = L::WT ? L::WK : L::K, WB = L::WT ? L::WKL : L::KL;

  // value waves: the read-out of the next chunk up to its factor, formed in
  // the previous chunk's second phase; the segment's gradient state G_seg^T
  // (rows j of block wb, columns f; both in the permuted order of the
  // features' stored positions) and this thread's share of gz_seg (tile rows
  // r0, r0 + 16, block b, by stored position); the log-decay from the
  // segment's start to the current chunk
  struct Prep {
    u32x4 ph[2], pl[2];   // the weighted scores P (rows s, column t = n), high and low
    float rt, hf, eq;     // r_t, h_t / (dout_t . o_t), e^{l_t}
  } pr;
  f32x16 Gs[NJ];
  float gzp[8];
  float Lseg = 0.f;
  if (value_wave) {
#pragma unroll
    for (int fb = 0; fb < NJ; ++fb) Gs[fb] = zero16();
#pragma unroll
    for (int e = 0; e < 8; ++e) gzp[e] = 0.f;
  }
  // the scores of chunk c (rows s, columns t = n): phi(k) at permuted
  // feature positions against phi(q) stored that way; the causal weights;
  // the denominator and the read-out factor
  auto prep = [&](int c) {
    // the operand addresses come from an opaque copy of the lane index:
    // held across the loop, they would not fit the registers
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = ln & 31, g = ln >> 5;
    const char* cur = smem + (c & 1) * L::BUF;
    const float* F = reinterpret_cast<const float*>(cur + L::FB);
    f32x16 sc = zero16();
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += 2) {
      u32x4 ak[2], akl[2], bq[2], bql[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        ak[kk] = row_operand_perm<D>(cur + L::K, perm_pos(n), k0 + kk, g);
        bq[kk] = row_operand<D>(cur + L::Q, perm_pos(n), 2 * (k0 + kk) + g);
        if constexpr (!XQ) {
          akl[kk] = row_operand_perm<D>(cur + L::KL, perm_pos(n), k0 + kk, g);
          bql[kk] = row_operand<D>(cur + L::QL, perm_pos(n), 2 * (k0 + kk) + g);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        sc = mfma(ak[kk], bq[kk], sc);
        if constexpr (!XQ) {
          sc = mfma(akl[kk], bq[kk], sc);
          sc = mfma(ak[kk], bql[kk], sc);
        }
      }
    }
    const float lt = DECAY ? F[L::LAM + n] : 0.f;   // token n's log-prefix
    pr.eq = DECAY ? __expf(lt) : 1.f;
    float wt[16];
    causal_weights_st<DECAY>(F, L::LAM, L::BET, lt, g, n, wt);
    float dsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] *= wt[i];
      dsum += sc[i];
    }
    dsum = swap_sum32(dsum);
    const float den = dsum + pr.eq * F[L::DI + n];
    const float mt = DECAY == 3 ? F[L::MT + n] : 0.f;
    // the read-out factor; with the mLSTM gates of the state scaled by
    // e^{-m_t}, whose max1 floor is e^{-m_t}
    pr.rt = DECAY == 3 ? readout_factor(a.norm, den, a.eps, mt)
            : a.norm == LA_NORM_NONE ? 1.f
            : a.norm == LA_NORM_MAX1 ? 1.f / fmaxf(fabsf(den), 1.f)
                                     : 1.f / (den + a.eps);
    pr.hf = 0.f;
    if (a.norm == LA_NORM_SUM) pr.hf = -pr.rt;
    else if (a.norm == LA_NORM_MAX1)
      pr.hf = fabsf(den) > (DECAY == 3 ? __expf(-mt) : 1.f) ? -copysignf(pr.rt, den) : 0.f;
    split_acc(sc, pr.ph, pr.pl);
  };

  if (value_wave) {
    load_dout3<D, DF32>(a, bh, c0 * BCH, wb, n, g, dreg);
  } else {
    load_raw3<D, DECAY>(a, bh, c0 * BCH, ft, raw);
    stage3<D, DECAY>(a, bh, c0 * BCH, ft, raw, smem + (c0 & 1) * L::BUF, nullptr, nullptr,
                     Sc + L::Z + (c0 & 1) * D, true, zs, mst);
    if (c0 + 1 < c1) load_raw3<D, DECAY>(a, bh, (c0 + 1) * BCH, ft, raw);
  }
  __syncthreads();
  if (value_wave) prep(c0);

  auto chunk = [&](int c, auto value_kind) {
    constexpr bool VW = decltype(value_kind)::value;
    const int t0 = c * BCH;
    const int64_t tc = bh * int64_t(T) + t0;
    const char* cur = smem + (c & 1) * L::BUF;
    const float* F = reinterpret_cast<const float*>(cur + L::FB);
    const bool vt = t0 + n < T;

    if constexpr (VW) {
      // ---- phase 1: the numerator^T (rows j of block wb, columns t):
      // e^{l_t} S^T phi(q) + V^T P, with S from the registers (contracting
      // over f) against phi(q) stored with its features permuted
      f32x16 nu = zero16();
#pragma unroll
      for (int fb = 0; fb < NJ; ++fb) {
        u32x4 sh[2], sl[2], bq[2], bql[2];
        split_acc(X[fb], sh, sl);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bq[ks] = row_operand<D>(cur + L::Q, perm_pos(n), 2 * (2 * fb + ks) + g);
          if constexpr (!XQ) bql[ks] = row_operand<D>(cur + L::QL, perm_pos(n), 2 * (2 * fb + ks) + g);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          nu = mfma(sh[ks], bq[ks], nu);
          nu = mfma(sl[ks], bq[ks], nu);
          if constexpr (!XQ) nu = mfma(sh[ks], bql[ks], nu);
        }
      }
      if constexpr (DECAY != 0) nu *= pr.eq;
      {
        u32x4 ov[2];
        tr_ops<D, 2>(cur + L::V, 32 * wb, lane, ov);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          nu = mfma(ov[ks], pr.ph[ks], nu);
          nu = mfma(ov[ks], pr.pl[ks], nu);
        }
      }

      // g = r_t dout into the shared tiles (feature j at perm_pos(j): the
      // values of r = 2 h2, 2 h2 + 1 fill one block), with a decay also
      // e^{L + l_t} g for the gradient-state fold; dout . o partials
      const float rt = vt ? pr.rt : 0.f;
      const float wg = DECAY ? __expf(Lseg) * pr.eq : 1.f;
      const int lg = lane_fresh(), ng = lg & 31, gg = lg >> 5;   // the tile offsets' lane
      float hp = 0.f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 gh, gl, wh, wl;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = 2 * h2 + rr;
          const f32x4 d4 = dout4<DF32>(dreg, r);
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hp += d4[e] * nu[4 * r + e];
            gv[e] = d4[e] * rt;
          }
          uint32_t h0, h1, l0, l1;
          split_bf16(gv[0], gv[1], h0, l0);
          split_bf16(gv[2], gv[3], h1, l1);
          gh[2 * rr] = h0;
          gh[2 * rr + 1] = h1;
          gl[2 * rr] = l0;
          gl[2 * rr + 1] = l1;
          if constexpr (DECAY != 0) {
            split_bf16(gv[0] * wg, gv[1] * wg, h0, l0);
            split_bf16(gv[2] * wg, gv[3] * wg, h1, l1);
            wh[2 * rr] = h0;
            wh[2 * rr + 1] = h1;
            wl[2 * rr] = l0;
            wl[2 * rr + 1] = l1;
          }
        }
        const int off = tile_off<D>(perm_pos(ng), 4 * wb + 2 * h2 + gg);
        *reinterpret_cast<u32x4*>(smem + L::G + off) = gh;
        *reinterpret_cast<u32x4*>(smem + L::GL + off) = gl;
        if constexpr (DECAY != 0) {
          *reinterpret_cast<u32x4*>(smem + L::WG + off) = wh;
          *reinterpret_cast<u32x4*>(smem + L::WGL + off) = wl;
        }
      }
      hp = swap_sum32(hp * pr.rt);
      if (g == 0) Sc[L::HP + wb * BCH + n] = hp;
      if (wb == 0 && g == 0) {
        Sc[L::RT + n] = pr.rt;
        Sc[L::HF + n] = pr.hf;
      }

      // the fold, after the numerator's reads of S: S (rows f, columns j of
      // block wb) = e^{l_last} S + (w phi(K))^T V
      const float tot = DECAY ? F[L::TOT] : 0.f;
      {
        const float ec = DECAY ? __expf(tot) : 1.f;
        u32x4 bv[2];
        tr_ops<D, 2>(cur + L::V, 32 * wb, lane, bv);
#pragma unroll
        for (int fb = 0; fb < NJ; ++fb) {
          u32x4 aw[2], awl[2];
          tr_ops<D, 2>(cur + WA, 32 * fb, lane, aw);
          tr_ops<D, 2>(cur + WB, 32 * fb, lane, awl);
          if constexpr (DECAY != 0) X[fb] *= ec;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            X[fb] = mfma(aw[ks], bv[ks], X[fb]);
            X[fb] = mfma(awl[ks], bv[ks], X[fb]);
          }
        }
      }
      // the segment's gradient state, G_seg^T += (e^{L + l} g)^T phi(Q): the
      // columns j of this wave's block are the ones it wrote (a wave's LDS
      // accesses complete in order, so no barrier is needed)
      {
        constexpr int GA = DECAY ? L::WG : L::G, GB = DECAY ? L::WGL : L::GL;
        u32x4 ag[2], agl[2];
        tr_ops<D, 2>(smem + GA, 32 * wb, lane, ag);
        tr_ops<D, 2>(smem + GB, 32 * wb, lane, agl);
#pragma unroll
        for (int fb = 0; fb < NJ; ++fb) {
          u32x4 bq[2], bql[2];
          tr_ops<D, 2>(cur + L::Q, 32 * fb, lane, bq);
          if constexpr (!XQ) tr_ops<D, 2>(cur + L::QL, 32 * fb, lane, bql);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            Gs[fb] = mfma(ag[ks], bq[ks], Gs[fb]);
            Gs[fb] = mfma(agl[ks], bq[ks], Gs[fb]);
            if constexpr (!XQ) Gs[fb] = mfma(ag[ks], bql[ks], Gs[fb]);
          }
        }
      }
      __syncthreads();   // g tiles and partials; the next chunk staged

      // ---- phase 2: the next chunk's dout; gz_seg += sum_t e^{L + l_t} h_t
      // phi(q_t); the next chunk's scores and read-out factor
      const bool more = c + 1 < c1;
      if (more) load_dout3<D, DF32>(a, bh, t0 + BCH, wb, n, g, dreg);
      {
        const float eL = DECAY ? __expf(Lseg) : 1.f;
        const int r0 = tid / L::BPR, b = tid % L::BPR;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = r0 + 16 * rr;
          float dot = 0.f;
#pragma unroll
          for (int ww = 0; ww < NJ; ++ww) dot += Sc[L::HP + ww * BCH + r];
          float ht = t0 + r < T ? Sc[L::HF + r] * dot : 0.f;
          if constexpr (DECAY != 0) ht *= eL * __expf(F[L::LAM + r]);
          float x[8];
          hilo8<D, XQ>(cur + L::Q, cur + L::QL, perm_pos(r), b, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) gzp[e] += x[e] * ht;
        }
      }
      if (more) prep(c + 1);
      Lseg += tot;
      __syncthreads();   // every read of chunk c's buffer and of g done
    } else {
      // ---- phase 1: the previous chunk's <phi(q), dphi(q)>, and the next
      // chunk staged into the other buffer (its addresses formed from a
      // fresh lane index: held across the loop, they would not fit the
      // registers of two waves per SIMD, and a reload of a spilled one waits
      // for every store and prefetch in flight)
      if constexpr (DECAY != 0) {
        if (wb == 0 && c > c0 && lane < BCH && t0 - BCH + lane < T) {
          float s = 0.f;
#pragma unroll
          for (int ww = 0; ww < NJ; ++ww) s += Sc[L::QP + ww * BCH + lane];
          a.qd[tc - BCH + lane] = s;
        }
      }
      if (c + 1 < c1) {
        const int fs = 64 * (wsg - NJ) + lane_fresh();
        stage3<D, DECAY>(a, bh, t0 + BCH, fs, raw, smem + ((c + 1) & 1) * L::BUF, cur,
                         Sc + L::Z + (c & 1) * D, Sc + L::Z + ((c + 1) & 1) * D, false, zs, mst);
        if (c + 2 < c1) load_raw3<D, DECAY>(a, bh, t0 + 2 * BCH, fs, raw);
      }
      __syncthreads();   // g tiles and partials; the next chunk staged

      // ---- phase 2: h_t, B, dphi(q), the fold
      const float lt = DECAY ? F[L::LAM + n] : 0.f;   // token n's log-prefix
      const float eq = DECAY ? __expf(lt) : 1.f;
      float dot = 0.f;
#pragma unroll
      for (int ww = 0; ww < NJ; ++ww) dot += Sc[L::HP + ww * BCH + n];
      const float h = vt ? Sc[L::HF + n] * dot : 0.f;
      if (wb == 0 && g == 0 && vt)
        *reinterpret_cast<float2*>(a.tok + (tc + n) * 2) = make_float2(Sc[L::RT + n], h);

      // dphi(q)^T (rows f of block wb, columns t): e^{l_t} (S g + z h) +
      // phi(K)^T B, with S^T from the registers (contracting over j); the
      // S g products first, so that the state's split meets B's MFMAs
      f32x16 dqt = zero16();
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 sh[2], sl[2], gh[2], gl[2];
        split_acc(X[jb], sh, sl);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          gh[ks] = row_operand<D>(smem + L::G, perm_pos(n), 2 * (2 * jb + ks) + g);
          gl[ks] = row_operand<D>(smem + L::GL, perm_pos(n), 2 * (2 * jb + ks) + g);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dqt = mfma(sh[ks], gh[ks], dqt);
          dqt = mfma(sl[ks], gh[ks], dqt);
          dqt = mfma(sh[ks], gl[ks], dqt);
        }
      }
      if constexpr (DECAY != 0) dqt *= eq;

      // B (rows s, columns t = n): (v_s . g_t + h_t) beta_s e^{l_t - l_s}
      f32x16 bs = zero16();
#pragma unroll
      for (int k0 = 0; k0 < KS; k0 += 2) {
        u32x4 ov[2], gh[2], gl[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          ov[kk] = row_operand_perm<D>(cur + L::V, perm_pos(n), k0 + kk, g);
          gh[kk] = row_operand<D>(smem + L::G, perm_pos(n), 2 * (k0 + kk) + g);
          gl[kk] = row_operand<D>(smem + L::GL, perm_pos(n), 2 * (k0 + kk) + g);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bs = mfma(ov[kk], gh[kk], bs);
          bs = mfma(ov[kk], gl[kk], bs);
        }
      }
      {
        float wt[16];
        causal_weights_st<DECAY>(F, L::LAM, L::BET, lt, g, n, wt);
#pragma unroll
        for (int i = 0; i < 16; ++i) bs[i] = (bs[i] + h) * wt[i];
      }
      u32x4 bh_[2], bl_[2];
      split_acc(bs, bh_, bl_);

      {
        u32x4 okt[2], oklt[2];
        tr_ops<D, 2>(cur + L::K, 32 * wb, lane, okt);
        if constexpr (!XQ) tr_ops<D, 2>(cur + L::KL, 32 * wb, lane, oklt);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dqt = mfma(okt[ks], bh_[ks], dqt);
          dqt = mfma(okt[ks], bl_[ks], dqt);
          if constexpr (!XQ) dqt = mfma(oklt[ks], bh_[ks], dqt);
        }
      }
      // the fold, issued before dphi(q)'s epilogue (its VALU work meets
      // these MFMAs): S^T (rows j, columns f of block wb) = e^{l_last} S^T +
      // V^T (w phi(K))
      const float ec = DECAY ? __expf(F[L::TOT]) : 1.f;
      u32x4 bw[2], bwl[2];
      tr_ops<D, 2>(cur + WA, 32 * wb, lane, bw);
      tr_ops<D, 2>(cur + WB, 32 * wb, lane, bwl);
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        u32x4 av[2];
        tr_ops<D, 2>(cur + L::V, 32 * jb, lane, av);
        if constexpr (DECAY != 0) X[jb] *= ec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          X[jb] = mfma(av[ks], bw[ks], X[jb]);
          X[jb] = mfma(av[ks], bwl[ks], X[jb]);
        }
      }
      {
        // the epilogue's addresses from a fresh lane index (as the staging's)
        const int le = lane_fresh(), n = le & 31, g = le >> 5;
        float qdp = 0.f;   // <phi(q_t), dphi(q_t)> over this lane's features
        const float* zc = Sc + L::Z + (c & 1) * D;
        float* dst = a.dq + tc * D + uint32_t(n * D + 32 * wb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pc = perm_pos(32 * wb + 8 * r + 4 * g);   // stored column of these 4 features
          const int off = tile_off<D>(perm_pos(n), pc >> 3) + ((pc & 7) << 1);
          const f32x4 p4 = hilo4<XQ>(cur + L::Q, cur + L::QL, off);
          const f32x4 z4 = *reinterpret_cast<const f32x4*>(zc + 32 * wb + 8 * r + 4 * g);
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float dphi = dqt[4 * r + e] + eq * z4[e] * h;
            // elu+1 has slope 1 above 0 and e^x = phi(x) below: min(phi, 1);
            // identity features (mLSTM): 1
            o4[e] = XQ ? dphi : dphi * fminf(p4[e], 1.f);
            qdp += p4[e] * dphi;
          }
          if (vt) *reinterpret_cast<f32x4*>(dst + 8 * r) = o4;
        }
        if constexpr (DECAY != 0) {
          qdp = swap_sum32(qdp);
          if (g == 0) Sc[L::QP + wb * BCH + n] = qdp;
        }
      }

      __syncthreads();   // every read of chunk c's buffer and of g done
    }
  };
  if (value_wave)
    for (int c = c0; c < c1; ++c) chunk(c, std::true_type{});
  else
    for (int c = c0; c < c1; ++c) chunk(c, std::false_type{});

  // the segment's gradient state into its slot: G_seg (rows f, columns j),
  // gz_seg, the segment's total log-decay
  float* dst = a.gslot + (bh * a.nseg + seg) * int64_t(D * D + D);
  float* gzw = reinterpret_cast<float*>(smem + L::FB) + L::ZP;   // [NJ][D], free now
  if (value_wave) {
#pragma unroll
    for (int fb = 0; fb < NJ; ++fb) {
      const int f = perm_pos(32 * fb + n);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f32x4*>(dst + f * D + perm_pos(32 * wb + 8 * r + 4 * g)) =
            f32x4{Gs[fb][4 * r], Gs[fb][4 * r + 1], Gs[fb][4 * r + 2], Gs[fb][4 * r + 3]};
    }
    wave_rows_sum8<L::BPR>(gzp, lane, gzw + wb * D);
    if (DECAY != 0 && tid == 0) a.lgam[bh * a.nseg + seg] = Lseg;
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NJ; ++ww) s += gzw[ww * D + tid];
    dst[D * D + perm_pos(tid)] = s;
  }

  // the last chunk's <phi(q), dphi(q)>
  if constexpr (DECAY != 0) {
    const int tl = (c1 - 1) * BCH + lane;
    if (w == NJ && lane < BCH && tl < T) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NJ; ++ww) s += Sc[L::QP + ww * BCH + lane];
      a.qd[bh * int64_t(T) + tl] = s;
    }
  }
}

// ----------------------------------------------------- decay gradient

// dL/dlog alpha_r = R_r = sum_{t >= r} (qd_t - beta_t kd_t), then dL/da_r =
// R_r / a_r (SSD) or dL/dg_r = R_r / g_r - kd_r (RFA: alpha = g, beta =
// 1 - g); for a_r below kDecayExact, the exact <G_r, S_{r-1}> term comes
// from decay_exact_kernel instead of R_r / a_r.  mLSTM gates (beta = beta'
// of the stabilised frame): dL/dfgate_r = R_r (1 - f_r), or R_r for the
// exponential forget gate, with no division, and dL/ditilde_r = beta'_r
// kd_r.  Two passes over tiles of DG_TILE tokens of every (b, h): the
// tiles' totals, then per tile a suffix scan (4 tokens per thread, waves by
// shuffles, the workgroup through LDS) plus the totals of the later tiles.
constexpr int DG_TILE = 1024;

struct DgArgs {
  const float* decay;   // alpha, the gate, or the mLSTM forget pre-activation
  const float* ab;      // mLSTM: log alpha', beta' per token
  const float* qd;
  const float* kd;
  float* part;
  float* dd;
  float* digate;        // mLSTM
  int T, ntile, fexp;
};

template <int DECAY>
__device__ __forceinline__ float beta_of(const DgArgs& g, int64_t i) {
  if constexpr (DECAY == 2) return 1.f - g.decay[i];
  if constexpr (DECAY == 3) return g.ab[2 * i + 1];
  return 1.f;
}

template <int DECAY>
__device__ __forceinline__ float dl_term(const DgArgs& g, int64_t i) {
  return g.qd[i] - beta_of<DECAY>(g, i) * g.kd[i];
}

// Sum over the 256 threads of a workgroup, returned to every thread.
__device__ __forceinline__ float block_sum256(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();   // red free from any earlier use
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <int DECAY>
__global__ __launch_bounds__(256) void bwd_decay_tile_sums(const DgArgs g) {
  __shared__ float red[4];
  const int T = g.T, ntile = g.ntile;
  const int64_t bh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  float s = 0.f;
  for (int i = threadIdx.x; i < DG_TILE; i += 256) {
    const int t = tile * DG_TILE + i;
    if (t < T) s += dl_term<DECAY>(g, bh * T + t);
  }
  s = block_sum256(s, red);
  if (threadIdx.x == 0) g.part[bh * ntile + tile] = s;
}

template <int DECAY>
__global__ __launch_bounds__(256) void bwd_decay_grad(const DgArgs g) {
  __shared__ float red[4];
  const int T = g.T, ntile = g.ntile;
  const float* part = g.part;
  const int64_t bh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // the later tiles' totals
  float c = 0.f;
  for (int u = tile + 1 + tid; u < ntile; u += 256) c += part[bh * ntile + u];
  const float carry = block_sum256(c, red);
  // this thread's 4 tokens, their suffix sums within the thread
  const int t0 = tile * DG_TILE + 4 * tid;
  float x[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = t0 + e < T ? dl_term<DECAY>(g, bh * T + t0 + e) : 0.f;
  float suf[4];
  suf[3] = x[3];
#pragma unroll
  for (int e = 2; e >= 0; --e) suf[e] = x[e] + suf[e + 1];
  // sum over the later threads of the wave (inclusive suffix, then less this
  // thread's own total)
  float v = suf[0];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_down(v, off);
    if (lane + off < 64) v += y;
  }
  __syncthreads();
  if (lane == 0) red[w] = v;   // the wave's total
  __syncthreads();
  float later = v - suf[0];
  for (int ww = w + 1; ww < 4; ++ww) later += red[ww];
  const float base = carry + later;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = t0 + e;
    if (t < T) {
      const int64_t i = bh * T + t;
      const float R = base + suf[e];
      if constexpr (DECAY == 3) {
        // 1 - sigmoid(x) = 1 / (1 + e^x)
        g.dd[i] = g.fexp ? R : R / (1.f + __expf(g.decay[i]));
        g.digate[i] = g.ab[2 * i + 1] * g.kd[i];
      } else {
        // near-zero decays: the exact term is added by decay_exact_kernel
        const float da = g.decay[i] < kDecayExact ? 0.f : R / g.decay[i];
        g.dd[i] = DECAY == 2 ? da - g.kd[i] : da;
      }
    }
  }
}

template <int D, int DECAY>
hipError_t launch_d(const Problem& pb, const BwArgs& a, float* dS0, float* dz0, float* ddecay,
                    hipStream_t st) {
  const unsigned nwg = unsigned(pb.BH() * a.nseg);
  if (a.dout_f32) bwd_pass_a2<D, DECAY, true><<<dim3(nwg), dim3(128 * (D / 32)), 0, st>>>(a);
  else bwd_pass_a2<D, DECAY, false><<<dim3(nwg), dim3(128 * (D / 32)), 0, st>>>(a);
  constexpr int PER = (D * D + D + 255) / 256;
  bwd_rscan<D, DECAY != 0><<<dim3(unsigned(pb.BH() * PER)), dim3(256), 0, st>>>(
      a.gslot, a.lgam, a.nseg, dS0, dz0);
  if (a.dout_f32) bwd_pass_b2<D, DECAY, true><<<dim3(nwg), dim3(128 * (D / 32)), 0, st>>>(a);
  else bwd_pass_b2<D, DECAY, false><<<dim3(nwg), dim3(128 * (D / 32)), 0, st>>>(a);
  if constexpr (DECAY != 0) {
    const int ntile = (a.T + DG_TILE - 1) / DG_TILE;
    const unsigned nb = unsigned(pb.BH() * ntile);
    DgArgs dg;
    dg.decay = a.decay; dg.ab = a.ab; dg.qd = a.qd; dg.kd = a.kd; dg.part = a.dpart;
    dg.dd = ddecay; dg.digate = a.digate; dg.T = a.T; dg.ntile = ntile; dg.fexp = a.fgate_exp;
    bwd_decay_tile_sums<DECAY><<<dim3(nb), dim3(256), 0, st>>>(dg);
    bwd_decay_grad<DECAY><<<dim3(nb), dim3(256), 0, st>>>(dg);
    if constexpr (DECAY == 3) return hipGetLastError();   // no division by a decay
    // near-zero decays: the exact gradient from each segment's start state
    // and the gradient state at its end (the reverse scan's slots)
    DecayExactArgs x;
    x.q = a.q; x.k = a.k; x.v = a.v; x.decay = a.decay; x.decay_kind = int(pb.decay_kind);
    x.phi = LA_PHI_ELU1; x.mode = 0; x.tok = a.tok; x.dout = a.dout; x.dout_f32 = a.dout_f32;
    x.ws = nullptr; x.S0 = a.S0; x.z0 = a.z0; x.s_bh = a.s_bh; x.z_bh = a.z_bh;
    x.s_seg = a.s_seg; x.gafter = a.gslot; x.nseg = a.nseg; x.seg_len = a.cps * BCH;
    x.dd = ddecay; x.T = a.T; x.dh = D; x.dv = D; x.dp = D;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decay_exact(x, LA_BF16, pb.BH(), st);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kind(const Problem& pb, const BwArgs& a, float* dS0, float* dz0, float* ddecay,
                       hipStream_t st) {
  switch (pb.decay_kind) {
    case LA_DECAY_NONE: return launch_d<D, 0>(pb, a, dS0, dz0, ddecay, st);
    case LA_DECAY_SSD: return launch_d<D, 1>(pb, a, dS0, dz0, ddecay, st);
    case LA_GATE_RFA: return launch_d<D, 2>(pb, a, dS0, dz0, ddecay, st);
    case LA_GATE_MLSTM: return launch_d<D, 3>(pb, a, dS0, dz0, ddecay, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

size_t r256(size_t b) { return (b + 255) / 256 * 256; }

struct BwLayout {
  size_t fwd, sinit, zinit, minit, gslot, tok, lgam, qd, kd, dpart, ab, total;
};

// Workspace: the prefill's (for the segment start states), a copy of the
// initial state, one gradient state per segment, two floats per token; with
// a decay also the segments' log-decays, two more floats per token and one
// per tile of DG_TILE tokens; with the mLSTM gates two more floats per token
// (log alpha', beta') and a zero start stabiliser per (b, h) for the
// prefill's stages when no initial state is given.
BwLayout layout_of(const Problem& pb) {
  int cps, nseg, nsub, nslot;
  mfma_split(pb, &cps, &nseg, &nsub, &nslot);
  const size_t BH = size_t(pb.BH()), D = size_t(pb.dv), T = size_t(pb.T);
  const bool dec = pb.decay_kind != LA_DECAY_NONE;
  BwLayout l;
  size_t off = 0;
  l.fwd = off;
  off += r256(mfma_workspace_bytes(pb));
  l.sinit = off;
  off += r256(BH * D * D * 4);
  l.zinit = off;
  off += r256(BH * D * 4);
  l.minit = off;
  if (pb.decay_kind == LA_GATE_MLSTM) off += r256(BH * 4);
  l.gslot = off;
  off += r256(BH * nseg * (D * D + D) * 4);
  l.tok = off;
  off += r256(BH * T * 2 * 4);
  l.lgam = l.qd = l.kd = l.dpart = l.ab = off;
  if (dec) {
    off += r256(BH * nseg * 4);
    l.qd = off;
    off += r256(BH * T * 4);
    l.kd = off;
    off += r256(BH * T * 4);
    l.dpart = off;
    off += r256(BH * ((T + DG_TILE - 1) / DG_TILE) * 4);
    l.ab = off;
    if (pb.decay_kind == LA_GATE_MLSTM) off += r256(BH * T * 2 * 4);
  }
  l.total = off;
  return l;
}

}  // namespace

bool backward_chunked(const Problem& p) {
  const bool gates = (p.phi == LA_PHI_ELU1 &&
                      (p.decay_kind == LA_DECAY_NONE || p.decay_kind == LA_DECAY_SSD ||
                       p.decay_kind == LA_GATE_RFA)) ||
                     (p.phi == LA_PHI_IDENTITY && p.decay_kind == LA_GATE_MLSTM);
  return p.path == 1 && p.dtype == LA_BF16 && gates && !p.noncausal && p.T > 0 &&
         p.dp == p.dv && (p.dv == 64 || p.dv == 128);
}

Problem backward_plan(const Problem& p) {
  Problem pb = p;
  if (p.chunk != BCH) {
    pb.chunk = BCH;
    pb.segments = mfma_default_segments(pb);
  }
  return pb;
}

size_t backward_chunked_workspace_bytes(const Problem& p) { return layout_of(backward_plan(p)).total; }

hipError_t launch_backward_chunked(const Problem& p, const void* q, const void* k, const void* v,
                                   const float* S0, const float* z0, const void* dout, float* dq,
                                   float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                                   void* ws, hipStream_t stream) {
  const Problem pb = backward_plan(p);
  const BwLayout l = layout_of(pb);
  char* base = static_cast<char*>(ws);
  int cps, nseg, nsub, nslot;
  mfma_split(pb, &cps, &nseg, &nsub, &nslot);
  const int64_t D = pb.dv, E = D * D + D;
  BwArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k);
  a.v = static_cast<const bf16_t*>(v);
  a.dout = dout;
  a.decay = pb.decay;
  a.dout_f32 = pb.out_dtype == LA_F32 ? 1 : 0;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.gslot = reinterpret_cast<float*>(base + l.gslot);
  a.tok = reinterpret_cast<float*>(base + l.tok);
  a.lgam = reinterpret_cast<float*>(base + l.lgam);
  a.qd = reinterpret_cast<float*>(base + l.qd);
  a.kd = reinterpret_cast<float*>(base + l.kd);
  a.dpart = reinterpret_cast<float*>(base + l.dpart);
  const bool ml = pb.decay_kind == LA_GATE_MLSTM;
  a.ab = ml ? reinterpret_cast<float*>(base + l.ab) : nullptr;
  a.igate = ml ? pb.igate : nullptr;
  a.fgate_exp = ml ? pb.fgate_exp : 0;
  a.digate = ml ? ddecay + pb.BH() * pb.T : nullptr;   // the second half of ddecay
  // the start state's stabiliser (one segment; null: a zero state, m = 0)
  a.m0 = ml && S0 ? pb.stab : nullptr;
  a.m0_bh = 1;
  a.T = pb.T;
  a.cps = cps;
  a.nseg = nseg;
  a.norm = pb.norm;
  a.eps = pb.eps;
  if (nseg > 1) {
    // the forward's stages 1 and 2 from a copy of the initial state (the scan
    // writes the final state over it): every segment's start state
    float* Si = reinterpret_cast<float*>(base + l.sinit);
    float* zi = reinterpret_cast<float*>(base + l.zinit);
    hipError_t e;
    if (S0) {
      e = hipMemcpyAsync(Si, S0, size_t(pb.BH()) * D * D * 4, hipMemcpyDeviceToDevice, stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(zi, z0, size_t(pb.BH()) * D * 4, hipMemcpyDeviceToDevice, stream);
    } else {
      // no initial state: zero, with the mLSTM gates also its stabiliser
      // (the caller's stab is read only with a state)
      float* mi = reinterpret_cast<float*>(base + l.minit);
      e = launch_state_init(Si, pb.BH() * D * D, zi, pb.BH() * D, ml ? mi : nullptr,
                            ml ? pb.BH() : 0, stream);
    }
    if (e != hipSuccess) return e;
    Problem pf = pb;
    if (ml && !S0) pf.stab = reinterpret_cast<float*>(base + l.minit);
    void* fws = base + l.fwd;
    e = launch_mfma_stage(pf, 1, q, k, v, Si, zi, nullptr, fws, stream);
    if (e != hipSuccess) return e;
    e = launch_mfma_stage(pf, 2, q, k, v, Si, zi, nullptr, fws, stream);
    if (e != hipSuccess) return e;
    const float* slots = reinterpret_cast<const float*>(fws);
    if (ml) {
      a.m0 = mfma_ws_m0(pb, fws);
      a.m0_bh = nseg + 1;
    }
    a.S0 = slots;
    a.z0 = slots + D * D;
    a.s_bh = a.z_bh = int64_t(nslot) * E;
    a.s_seg = int64_t(nsub) * E;
  } else {
    a.S0 = S0;
    a.z0 = z0;
    a.s_bh = D * D;
    a.z_bh = D;
    a.s_seg = 0;
  }
  if (D == 128) return launch_kind<128>(pb, a, dS0, dz0, ddecay, stream);
  return launch_kind<64>(pb, a, dS0, dz0, ddecay, stream);
}

}  // namespace la
