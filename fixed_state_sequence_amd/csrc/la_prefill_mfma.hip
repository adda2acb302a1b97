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
// mLSTM gates (wikillm "Linear attention", Variants / mLSTM; identity
// features, alpha = f, beta = e^{itilde}): the state is held scaled by e^{-m},
// m the stabiliser m_t = max(log f_t + m_{t-1}, itilde_t).  Inside a chunk
// that starts from (S', z', m0), with a_s = itilde_s - lc_s and the running
// maximum mu_t = max(m0, max_{s<=t} a_s), the stabiliser is m_t = lc_t + mu_t
// and every factor is at most 1:
//   inter-chunk read-out  e^{m0 - mu_t},   key s at query t  e^{a_s - mu_t},
//   carry  e^{m0 - mu_last},   fold weight  e^{a_s - mu_last};
// they take the places of e^{lc_t}, e^{lc_t - lc_s} beta_s, e^{lc_last} and
// w_s above (with "lc_t" := m0 - mu_t and beta_s := e^{a_s - mu_s}), and the
// read-out divides by max(|den'|, e^{-m_t}) (or den' + eps e^{-m_t}).
//
// Parallel schedule.  Each (b, h) sequence is cut into `segments` runs of
// whole chunks.  Stage 1: one workgroup per sub-segment (half a segment)
// folds its chunks into a sub-segment state (S_u, z_u, log Gamma_u).  Stage 2:
// per element of the state, a scan over the sub-segments, starting from the
// caller's initial state, gives each segment's start state and the final
// state.  Stage 3: one workgroup per segment walks its chunks again from its
// start state and writes the outputs (with a single segment, stages 1 and 2
// are skipped and stage 3 writes the final state).
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
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

// Floor on log(alpha) so that alpha = 0 (a full reset) stays finite in the
// within-chunk log-prefix; e^-80 ~ 1.8e-35 is the smallest decay applied.
constexpr float kLogFloor = -80.0f;

// The output stage holds its carried state as S = e^lp acc and lets the
// chunks' decays accumulate in lp (the fold operands take e^-lp instead)
// while |lp| stays within this bound; past it the accumulators take the
// factor and lp restarts from 0.  e^30 ~ 1e13 leaves fp32 ample range.
constexpr float kDeferLog = 30.0f;

template <int D, int C, bool VS, bool DMT = false>
struct Cfg {
  static constexpr int NW = D / 32;          // waves, 32 value columns each
  static constexpr int NT = 64 * NW;         // threads per workgroup (= 2 D)
  static constexpr int FB = D / 8;           // 16-byte feature blocks per row
  static constexpr int RPT = C * FB / NT;    // token rows per thread when loading (= C / 16)
  static constexpr int TB = C / 32;          // 32-token blocks of a chunk
  static constexpr int KS = D / 16;          // 16-feature k-steps
  static constexpr int KT = C / 16;          // 16-token k-steps
  static constexpr int MT = D / 32;          // 32-feature tiles of the state
  static constexpr int ND = C > 64 ? 2 : 1;  // decay values per lane (token lane, lane + 64)
  static constexpr int TILE = C * 2 * D;     // one C x D bf16 tile
  // Raw q, k, v of the next DEPTH chunks are held in registers (3 RPT
  // 16-byte blocks per thread and chunk) while the current one is computed,
  // so about 3 x 24 KB per compute unit stay in flight at C = 32.
  // DEPTH = 0: each chunk is loaded when it is staged.
  static constexpr int DEPTH = RPT <= 2 ? 3 : 0;
  static constexpr int RING = DEPTH > 0 ? DEPTH : 1;
  // Every tile is token-major (one row per token, D bf16 per row, 16-byte
  // blocks XOR-swizzled per row by blk_swz):
  //   Q, K   phi(q), phi(k); row = token, features at perm_pos order (read
  //          row-wise as the k = feature operands of the read-out and scores)
  //   KR     the bf16 low part phi(k) - K, laid out as K, in the chunks that
  //          start before token EXACT: their scores take phi(q) . (K + KR).
  //          An output there averages few values, so a rounding error in one
  //          weight passes to the output nearly undamped; later outputs
  //          average hundreds of weights and their rounding errors cancel.
  //   QR     the bf16 low part phi(q) - Q, laid out as Q, in the chunks that
  //          read the state out at high precision: those that start before
  //          token PRECISE without a decay, before EXACT with one (the scores
  //          of the first EXACT tokens take QR too).  Without a decay the
  //          outputs shrink like 1/sqrt(t) while the rounding of the
  //          inter-chunk read-out stays a fixed fraction of each output, so it
  //          is the first outputs' rounding that shows against the rms of a
  //          long sequence.  A decay keeps the outputs from shrinking once it
  //          has cut off the sequence's start, so with one these chunks also
  //          need the decay since the segment's start to be above e^PREC_LOG
  //          (decays of 1 behave as no decay).  They read the state out as
  //          (S_hi + S_lo)^T (Q + QR) (three products); the chunks before
  //          EXACT also fold w phi(k) as high + low parts.
  //   KH, KL w phi(k) as bf16 high/low parts; row = perm_pos(token), natural
  //          features (read transposed: the k = token operand of the fold)
  //   VH, VL v (high/low parts only for fp16 inputs); row = perm_pos(token),
  //          natural features (read transposed for P V and the fold)
  // followed by per-token fp32 arrays and the per-wave z increments.
  static constexpr int B_Q = 0;
  static constexpr int B_K = B_Q + TILE;
  static constexpr int B_KR = B_K + TILE;
  static constexpr int B_QR = B_KR + TILE;
  static constexpr int B_KH = B_QR + TILE;
  static constexpr int B_KL = B_KH + TILE;
  static constexpr int B_VH = B_KL + TILE;
  static constexpr int B_VL = B_VH + TILE;
  static constexpr int B_L = B_VL + (VS ? TILE : 0);  // lc_t, fp32 [C]
  static constexpr int EXACT = 128;
  static constexpr int PRECISE = 1024;
  static constexpr float PREC_LOG = -8.f;
  static constexpr int B_B = B_L + 4 * C;             // beta_t, fp32 [C]
  static constexpr int B_DEN = B_B + 4 * C;           // inter-chunk denominators, fp32 [C]
  static constexpr int B_M = B_DEN + 4 * C;           // mLSTM stabiliser m_t, fp32 [C]
  static constexpr int B_DZ = B_M + 4 * C;            // per-wave z increments, fp32 [NW][DZS]
  // z increment of feature 8 fb + e at dz_index: 4 floats of padding after
  // the first 64, so that feature blocks fb and fb + 8 (read together by a
  // wave) fall in different banks
  static constexpr int DZS = D + (D > 64 ? 4 : 0);
  // DM (DMT: decays with 32-token chunks): the chunk's decay mask
  // e^{lc_t - lc_s} beta_s (0 for s > t), fp32, row t = query token, DMS
  // floats per row (rows 16-byte aligned, 8 rows cover the 32 banks)
  static constexpr bool HAS_DM = DMT;
  static constexpr int DMS = C + 4;
  static constexpr int B_DM = B_DZ + 4 * NW * DZS;
  static constexpr int BUF = B_DM + (DMT ? 4 * C * DMS : 0);
  // The output stage: producer waves stage chunk c + 1 into one buffer while
  // consumer waves compute chunk c from the other, when two buffers fit; each
  // buffer also carries the chunk's total log-decay.
  static constexpr int B_LT = BUF;
  static constexpr int BUF3 = BUF + 16;
  static constexpr int NBUF = 2 * BUF3 <= 160 * 1024 ? 2 : 1;
  static constexpr int LDS = NBUF * BUF3;
  // producer prefetch depth (registers are not shared with the consumers'
  // accumulators, so it can be deeper)
  static constexpr int PDEPTH = RPT <= 2 ? 2 : 1;
  // stage 1: KH, KL, VH (VL), two buffers
  static constexpr int S1_KH = 0;
  static constexpr int S1_KL = S1_KH + TILE;
  static constexpr int S1_VH = S1_KL + TILE;
  static constexpr int S1_VL = S1_VH + TILE;
  static constexpr int S1_BUF = S1_VL + (VS ? TILE : 0);
  static constexpr int S1_LDS = 2 * S1_BUF;
  // stage-1 producer prefetch depth (chunks of k, v held in registers)
  static constexpr int S1_PD = RPT <= 2 ? 3 : 1;
  static_assert(RPT == C / 16, "row split");
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "width");
  static_assert(PRECISE >= EXACT && PRECISE % 128 == 0, "the QR tile covers the exact scores");
  static_assert(LDS <= 160 * 1024 && S1_LDS <= 160 * 1024, "LDS");
};

// p += (low parts of phi(k), key rows kr) . phi(q) (query row qr), over all
// feature k-steps: the second half of the scores phi(q) . (K + KR).
template <int D, int KS>
__device__ __forceinline__ f32x16 low_scores(const char* kr_tile, const char* q_tile, int kr,
                                             int qr, int g, f32x16 p) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    p = mfma(row_operand<D>(kr_tile, kr, 2 * ks + g), row_operand<D>(q_tile, qr, 2 * ks + g), p);
  return p;
}

struct PfArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* S;          // caller's state [BH, D, D] (initial in, final out)
  float* z;          // caller's normaliser [BH, D]
  const float* decay;  // [BH, T] or null (mLSTM: forget-gate pre-activations)
  const float* igate;  // [BH, T] mLSTM input-gate pre-activations, or null
  float* stab;         // [BH] mLSTM stabiliser (initial in, final out), or null
  int fgate_exp;       // mLSTM forget gate: sigmoid (0) or exp (1)
  // Workspace, per (b, h), NSLOT = nsub nseg slots of D*D + D floats (with
  // more than one segment): stage 1 writes sub-segment u's state into slot u
  // (each segment is cut into nsub sub-segments, so that stage 1 has enough
  // workgroups); the scan turns slot nsub s into the start state of segment s
  // and writes the final state, carried past the last slot, into (S, z).
  float* ws_state;   // [BH, NSLOT, D*D + D]
  float* ws_logg;    // [BH, NSLOT]: log Gamma of each sub-segment
  float* ws_m;       // [BH, NSLOT]: mLSTM stabiliser of each sub-segment's state
  float* ws_m0;      // [BH, nseg + 1]: mLSTM start stabiliser of each segment, then the final one
  int T;
  int nseg;
  int cps;           // chunks per segment
  int nsub;          // stage-1 sub-segments per segment
  int cps_sub;       // chunks per sub-segment (the last one of a segment may be shorter)
  int nslot;         // nsub nseg
  int out_f32;       // out is fp32 (else the input type)
  int norm;          // read-out form (LA_NORM_*)
  int nc;            // non-causal: every output reads the whole sequence's state
  float eps;
};

// The raw inputs of one chunk as this thread loads them: RPT 16-byte blocks
// (8 features of one token row) of q, k and v, and the decay/gate value of
// token `lane` (and `lane + 64`) of the chunk (with the mLSTM gates, the
// forget and the input pre-activation).  The loads are unconditional (rows
// past the end of the sequence read the last row) so that the compiler can
// count the loads still in flight exactly when a later chunk's data is used;
// clean_chunk() then zeroes those rows (and sets their decay to 1).
template <int RPT, int ND, bool HAS_Q, bool HAS_KV = true, bool HAS_I = false>
struct RawChunk {
  u32x4 q[HAS_Q ? RPT : 1], k[HAS_KV ? RPT : 1], v[HAS_KV ? RPT : 1];
  float d[ND];
  float ig[HAS_I ? ND : 1];
};

template <int C, int D, int RPT, int ND, bool HAS_Q, int DECAY, typename DT, bool HAS_KV,
          bool HAS_I>
__device__ __forceinline__ void fetch_chunk(RawChunk<RPT, ND, HAS_Q, HAS_KV, HAS_I>& r,
                                            const DT* qg, const DT* kg, const DT* vg,
                                            const float* dg, const float* igp, int tok0, int T,
                                            int rg, int fb, int lane) {
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int t = min(tok0 + RPT * rg + i, T - 1);
    // 32-bit byte offsets within the (b, h) slab (T D < 2^31 elements of 2
    // bytes is checked on the host), so that each load takes the slab's
    // uniform base as its scalar address and one offset register
    static_assert(sizeof(DT) == 2, "bf16 or fp16 inputs");
    const uint32_t ob = (uint32_t(t) * D + 8 * fb) * uint32_t(sizeof(DT));
    auto at = [&](const DT* base) {
      return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + ob);
    };
    if constexpr (HAS_Q) r.q[i] = at(qg);
    if constexpr (HAS_KV) {
      r.k[i] = at(kg);
      r.v[i] = at(vg);
    }
  }
  if constexpr (DECAY != 0) {
#pragma unroll
    for (int j = 0; j < ND; ++j) r.d[j] = dg[min(tok0 + lane + 64 * j, T - 1)];
  }
  if constexpr (DECAY == 3) {
#pragma unroll
    for (int j = 0; j < ND; ++j) r.ig[j] = igp[min(tok0 + lane + 64 * j, T - 1)];
  }
}

// Rows past the end of the sequence become 0 and decay values of tokens
// outside the chunk or the sequence become 1 (the loads read in-bounds
// stand-ins).  The row pass runs only for the chunk holding the end.  With
// the mLSTM gates the forget pre-activation becomes log f (0 outside) and
// the input pre-activation of a token outside becomes kNoToken.
template <int C, int RPT, int ND, bool HAS_Q, int DECAY, bool HAS_KV, bool HAS_I>
__device__ __forceinline__ void clean_chunk(RawChunk<RPT, ND, HAS_Q, HAS_KV, HAS_I>& r, int tok0,
                                            int T, int rg, int lane, int fgate_exp = 0) {
  if (tok0 + C > T) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      if (tok0 + RPT * rg + i >= T) {
        if constexpr (HAS_Q) r.q[i] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (HAS_KV) {
          r.k[i] = u32x4{0u, 0u, 0u, 0u};
          r.v[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
  }
  if constexpr (DECAY == 3) {
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int rr = lane + 64 * j;
      const bool out = rr >= C || tok0 + rr >= T;
      r.d[j] = out ? 0.f : log_forget(r.d[j], fgate_exp);
      if (out) r.ig[j] = kNoToken;
    }
  } else if constexpr (DECAY != 0) {
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int rr = lane + 64 * j;
      if (rr >= C || tok0 + rr >= T) r.d[j] = 1.f;
    }
  }
}

// Within-chunk inclusive log-prefix of the decay, one wave: every wave of the
// workgroup computes it redundantly (no barrier needed).  Returns lc for
// token `lane` (and `lane + 64` in hi for C = 128) and the chunk total.
// Tokens past the end of the chunk or the sequence contribute log 1 = 0.
// IS_LOG: d already holds log alpha (the mLSTM forget gate).
template <int C, int ND, bool IS_LOG = false>
__device__ __forceinline__ void chunk_logprefix(const float (&d)[ND], int lane, float& lo,
                                                float& hi, float& total) {
  lo = IS_LOG ? d[0] : fmaxf(__logf(d[0]), kLogFloor);
  hi = ND > 1 ? (IS_LOG ? d[ND - 1] : fmaxf(__logf(d[ND - 1]), kLogFloor)) : 0.f;
  (void)lane;
  lo = wave_scan<C <= 32 ? 32 : 64>(lo, 0.f, ScanAdd{});
  if constexpr (C > 64) {
    hi = wave_scan<64>(hi, 0.f, ScanAdd{}) + lane_bcast(lo, 63);
    total = lane_bcast(hi, 63);
  } else {
    total = lane_bcast(lo, C - 1);
  }
}

// mLSTM stabiliser inside one chunk, one wave (every wave redundantly): from
// the inclusive log-forget prefix lc (lo, hi) and the input pre-activations,
// a_t = itilde_t - lc_t and the running maximum mu_t = max(m0, max_{s<=t} a_s)
// of token `lane` (and `lane + 64` in the hi values), and mu at the chunk's
// last token.  Tokens outside hold kNoToken and never raise the maximum.
template <int C, int ND>
__device__ __forceinline__ void chunk_runmax(const float (&ig)[ND], float lo, float hi, float m0,
                                             int lane, float& alo, float& ahi, float& mlo,
                                             float& mhi, float& mend) {
  alo = ig[0] - lo;
  ahi = ND > 1 ? ig[ND - 1] - hi : kNoToken;
  (void)lane;
  mlo = fmaxf(wave_scan<C <= 32 ? 32 : 64>(alo, kNoToken, ScanMax{}), m0);
  if constexpr (C > 64) {
    mhi = fmaxf(wave_scan<64>(ahi, kNoToken, ScanMax{}), lane_bcast(mlo, 63));
    mend = lane_bcast(mhi, 63);
  } else {
    mhi = ahi;
    mend = lane_bcast(mlo, C - 1);
  }
}

template <int C>
__device__ __forceinline__ float lane_value(float lo, float hi, int r) {
  const float a = __shfl(lo, r & 63);
  if constexpr (C > 64) {
    const float b = __shfl(hi, r & 63);
    return r >= 64 ? b : a;
  } else {
    return a;
  }
}

// ---------------------------------------------------------------- stage 1

// Segment state: S_seg = sum_s w_s phi(k_s) v_s^T over the segment's tokens
// with w_s = beta_s prod_{r > s in the segment} alpha_r (and z_seg alike),
// plus log Gamma_seg = sum of log alpha over the segment.  The chunks are
// walked back to front, so the weight of a token is the decay of the chunks
// already folded (lsuf) times its within-chunk suffix, and the first chunks
// of the segment are the most recently read when the output stage starts.
//
// Warp-specialised like the output stage: NW producer waves load k, v
// S1_PD chunks ahead into registers, form w phi(k) (bf16 high and low parts)
// and the v tiles in one of two LDS buffers, and keep their share of z; NW
// consumer waves fold each staged chunk into the state held in their
// accumulators (32 value columns each).  One barrier per chunk.
// M16: the consumers fold on v_mfma_f32_16x16x32_bf16 (16 x 16 result tiles,
// the whole 32-token chunk as one k-block) instead of 32x32x16 (32 x 32
// tiles, two 16-token k-steps); the same sums in another order.  Kept to
// measure the shape choice (LA_STAGE1_MFMA=16x16x32).
template <int D, int C, int DECAY, typename DT, bool M16 = false>
__global__ __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(4, 4)))
void segment_state_kernel(const PfArgs a) {
  constexpr bool VS = __is_same(DT, f16_t);   // fp16 v needs a bf16 low part too
  using G = Cfg<D, C, VS>;
  __shared__ __align__(16) char smem[G::S1_LDS];
  __shared__ __align__(16) float zl[G::NW][D];
  // mLSTM: factor e^{M_old - M_new} that rescales the state before the
  // chunk in buffer i & 1 is folded in (the running maximum grew)
  __shared__ float s1_scale[2];
  const int bh = blockIdx.x / a.nslot;
  const int u = blockIdx.x % a.nslot;   // sub-segment: segment u / nsub, part u % nsub
  const int nchunks = (a.T + C - 1) / C;
  const int seg_first = (u / a.nsub) * a.cps;
  const int c0 = seg_first + (u % a.nsub) * a.cps_sub;
  const int c1 = min(min(c0 + a.cps_sub, seg_first + a.cps), nchunks);
  const int n = max(c1 - c0, 0);   // chunks to fold (a sub-segment can be empty)
  float* dst = a.ws_state + (int64_t(bh) * a.nslot + u) * (D * D + D);
  auto buffer = [&](int i) -> char* { return smem + (i & 1) * G::S1_BUF; };

  const int wave_id = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  if (wave_id >= G::NW) {
    // =================================================== producer waves
    const int ts = threadIdx.x - G::NT, lane = ts & 63, wave = ts >> 6;
    const int fb = ts % G::FB, rg = ts / G::FB;
    const DT* kg = static_cast<const DT*>(a.k) + int64_t(bh) * a.T * D;
    const DT* vg = static_cast<const DT*>(a.v) + int64_t(bh) * a.T * D;
    const float* dg = DECAY ? a.decay + int64_t(bh) * a.T : nullptr;
    const float* igp = DECAY == 3 ? a.igate + int64_t(bh) * a.T : nullptr;
    // this thread's share of z (features 8 fb .. 8 fb + 7, its own rows of
    // every chunk): the weights already carry the decay, so z is a plain
    // sum, reduced over the threads once at the end
    float zp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lsuf = 0.f;   // log-decay of the chunks already staged (later in the segment)
    // mLSTM: running maximum of the log weights itilde_s + (log decay from s
    // to the sub-segment's end) over the chunks staged so far; the state and
    // zp are held scaled by e^{-M}
    float M = kNoToken;
    using Raw = RawChunk<G::RPT, G::ND, false, true, DECAY == 3>;
    // walk step i stages chunk c1 - 1 - i; steps past the segment's first
    // chunk load a repeat of it (clamped), so the loads are the same on every
    // path, and add nothing
    auto fetch = [&](Raw& r, int i) {
      fetch_chunk<C, D, G::RPT, G::ND, false, DECAY>(r, (const DT*)nullptr, kg, vg, dg, igp,
                                                      max(c1 - 1 - i, c0) * C, a.T, rg, fb, lane);
    };
    // [A] chunk c into buffer buf: w phi(k) high/low and v as token-major
    // tiles; this thread's rows added to zp.  Rows past the end have k = v =
    // 0: phi(k) = 1 there and v = 0, so they add nothing to S; without decay
    // their 1s are taken off z at the end.
    auto stage = [&](Raw& raw, int i, char* buf) {
      const int c = c1 - 1 - i;
      const bool live = i < n;
      const int tok0 = max(c, c0) * C;
      clean_chunk<C, G::RPT, G::ND, false, DECAY>(raw, tok0, a.T, rg, lane, a.fgate_exp);
      float lo = 0.f, hi = 0.f, ltot = 0.f;
      if constexpr (DECAY != 0) chunk_logprefix<C, G::ND, DECAY == 3>(raw.d, lane, lo, hi, ltot);
      // mLSTM: the chunk's largest log weight relative to the sub-segment's
      // end raises the running maximum; the state folded so far is rescaled
      float alo = 0.f, ahi = 0.f, Mn = M;
      if constexpr (DECAY == 3) {
        alo = raw.ig[0] - lo;
        ahi = G::ND > 1 ? raw.ig[G::ND - 1] - hi : kNoToken;
        const float cm = lane_bcast(wave_scan<64>(fmaxf(alo, ahi), kNoToken, ScanMax{}), 63);
        Mn = fmaxf(M, cm + lsuf + ltot);
        const float sc = __expf(M - Mn);
        if (live && sc != 1.f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) zp[e] *= sc;
        }
        if (ts == 0) s1_scale[i & 1] = sc;
      }
#pragma unroll
      for (int ii = 0; ii < G::RPT; ++ii) {
        const int r = G::RPT * rg + ii;
        float kx[8];
        unpack8(raw.k[ii], kx, DT{});
        // The cross-lane reads run in every lane, outside the per-row
        // condition: a lane left out of a shuffle does not supply its value,
        // and the rows past the end belong to lanes whose token values the
        // last valid rows still need.
        float w = 1.f;
        if constexpr (DECAY == 3) {
          const float ar = lane_value<C>(alo, ahi, r);
          w = tok0 + r < a.T ? __expf(ar + lsuf + ltot - Mn) : 0.f;
        } else if constexpr (DECAY != 0) {
          const float lcr = lane_value<C>(lo, hi, r);
          w = tok0 + r < a.T ? __expf(lsuf + ltot - lcr) : 0.f;
          if constexpr (DECAY == 2)
            w *= 1.f - lane_value<C>(raw.d[0], G::ND > 1 ? raw.d[G::ND - 1] : 0.f, r);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (DECAY != 3) kx[e] = elu1_fast(kx[e]);   // mLSTM: identity
          if constexpr (DECAY != 0) kx[e] *= w;
          if (live) zp[e] += kx[e];
        }
        const u32x4 kh = pack8(kx);
        blk_write<D>(buf + G::S1_KH, perm_pos(r), fb, kh);
        blk_write<D>(buf + G::S1_KL, perm_pos(r), fb, low8(kx, kh));
        if constexpr (VS) {
          float vx[8];
          unpack8(raw.v[ii], vx, DT{});
          const u32x4 vh = pack8(vx);
          blk_write<D>(buf + G::S1_VH, perm_pos(r), fb, vh);
          blk_write<D>(buf + G::S1_VL, perm_pos(r), fb, low8(vx, vh));
        } else {
          blk_write<D>(buf + G::S1_VH, perm_pos(r), fb, raw.v[ii]);
        }
      }
      if (live) {
        lsuf += ltot;
        M = Mn;
      }
      // refill this register set with the step S1_PD further on
      fetch(raw, i + G::S1_PD);
    };

    Raw raw[G::S1_PD];
#pragma unroll
    for (int j = 0; j < G::S1_PD; ++j) fetch(raw[j], j);
    stage(raw[0], 0, buffer(0));
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += G::S1_PD) {
#pragma unroll
      for (int j = 0; j < G::S1_PD; ++j) {
        const int i = i0 + j;
        stage(raw[(j + 1) % G::S1_PD], i + 1, buffer(i + 1));
        if (i < n) __syncthreads();   // chunk i folded, chunk i + 1 staged
      }
    }
    // z: the shares summed within each wave, then over the producer waves;
    // less the 1s of the rows past the end (no decay)
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = group_sum<G::FB>(zp[e]);
    if (lane < G::FB) {
      *reinterpret_cast<f32x4*>(&zl[wave][8 * fb]) = f32x4{zp[0], zp[1], zp[2], zp[3]};
      *reinterpret_cast<f32x4*>(&zl[wave][8 * fb + 4]) = f32x4{zp[4], zp[5], zp[6], zp[7]};
    }
    __syncthreads();
    if (ts < D) {
      float zs = (DECAY == 0 && n > 0 && c1 == nchunks) ? -float(nchunks * C - a.T) : 0.f;
#pragma unroll
      for (int w = 0; w < G::NW; ++w) zs += zl[w][ts];
      dst[D * D + ts] = zs;
    }
    if (ts == 0) {
      a.ws_logg[int64_t(bh) * a.nslot + u] = lsuf;
      if constexpr (DECAY == 3) a.ws_m[int64_t(bh) * a.nslot + u] = M;
    }
  } else {
    // =================================================== consumer waves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if constexpr (M16) {
      static_assert(C == 32 && !VS && DECAY != 3, "the 16x16x32 fold covers 32-token bf16 chunks");
      // rows = features 16 ft + 4 (lane / 16) + r, columns = 32 wave + 16 nt + lane % 16
      f32x4 acc16[D / 16][2];
#pragma unroll
      for (int ft = 0; ft < D / 16; ++ft) acc16[ft][0] = acc16[ft][1] = f32x4{};
      __syncthreads();   // the producers' first chunk
      for (int i = 0; i < n; ++i) {
        const char* buf = buffer(i);
        u32x4 vb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) vb[nt] = tr_operand16<D>(buf + G::S1_VH, 0, 32 * wave + 16 * nt, lane);
#pragma unroll
        for (int ft = 0; ft < D / 16; ++ft) {
          const u32x4 kh = tr_operand16<D>(buf + G::S1_KH, 0, 16 * ft, lane);
          const u32x4 kl = tr_operand16<D>(buf + G::S1_KL, 0, 16 * ft, lane);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            acc16[ft][nt] = mfma16(kh, vb[nt], acc16[ft][nt]);
            acc16[ft][nt] = mfma16(kl, vb[nt], acc16[ft][nt]);
          }
        }
        __syncthreads();
      }
      const int q = lane >> 4, nn = lane & 15;
#pragma unroll
      for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dst[(16 * ft + 4 * q + r) * D + 32 * wave + 16 * nt + nn] = acc16[ft][nt][r];
      __syncthreads();   // matches the producers' z barrier
      return;
    }
    f32x16 acc[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc[mt] = f32x16{};
    // [B] fold the staged chunk into S; the weights already carry the decay
    // (mLSTM: the state is first rescaled to the new running maximum)
    auto fold = [&](const char* buf, int i) {
      if constexpr (DECAY == 3) {
        // the running maximum seldom grows after the segment's last chunks
        // (folded first), so the factor is mostly exactly 1: skip it then
        const float sc = s1_scale[i & 1];
        if (sc != 1.f) {
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt) acc[mt] *= sc;
        }
      }
      u32x4 vh[G::KT], vl[G::KT];
#pragma unroll
      for (int kk = 0; kk < G::KT; ++kk) {
        vh[kk] = tr_operand<D>(buf + G::S1_VH, 16 * kk, 32 * wave, lane);
        if constexpr (VS) vl[kk] = tr_operand<D>(buf + G::S1_VL, 16 * kk, 32 * wave, lane);
      }
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
        for (int kk = 0; kk < G::KT; ++kk) {
          const u32x4 kh = tr_operand<D>(buf + G::S1_KH, 16 * kk, 32 * mt, lane);
          const u32x4 kl = tr_operand<D>(buf + G::S1_KL, 16 * kk, 32 * mt, lane);
          acc[mt] = mfma(kh, vh[kk], acc[mt]);
          acc[mt] = mfma(kl, vh[kk], acc[mt]);
          if constexpr (VS) acc[mt] = mfma(kh, vl[kk], acc[mt]);
        }
      }
    };
    __syncthreads();   // the producers' first chunk
    for (int i = 0; i < n; ++i) {
      fold(buffer(i), i);
      __syncthreads();
    }
    // the state, row-major [f][v]
    const int g = lane >> 5, nn = lane & 31;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        dst[f * D + 32 * wave + nn] = acc[mt][r];
      }
    __syncthreads();   // matches the producers' z barrier
  }
}

// ---------------------------------------------------------------- stage 2

// Exclusive scan of the sub-segment states of one (b, h), one state element
// per thread: carry = Gamma_u carry + S_u over the slots in order, starting
// from the caller's initial state; the carry before slot nsub s is the start
// state of segment s (written in place) and the carry after the last slot is
// the final state (written over the initial one).  Slot values are loaded U
// at a time (all of them, for up to U slots), all in flight together, then
// folded in order.
// ML (mLSTM gates): every state is held scaled by e^{-m}; slot u carries its
// own stabiliser m_u, and carry (S', m) then slot u combine as
//   m <- max(m + log Gamma_u, m_u),
//   S' <- e^{m_old + log Gamma_u - m} S' + e^{m_u - m} S'_u,
// the max-plus form of the stabiliser's recurrence.  The start stabiliser
// of each segment and the final one go to ws_m0 (the output stage copies
// the final one to the caller's, after every block here has read it).
template <int D, int U, bool ML>
__global__ __launch_bounds__(256) void segment_scan_kernel(const PfArgs a) {
  // four consecutive state elements per thread (16-byte loads and stores)
  constexpr int E = D * D + D;
  constexpr int E4 = E / 4;
  static_assert(E % 4 == 0 && (D * D) % 4 == 0, "float4 elements");
  const int per_bh = (E4 + 255) / 256;
  const int bh = blockIdx.x / per_bh;
  const int e = 4 * ((blockIdx.x % per_bh) * 256 + int(threadIdx.x));
  if (e >= E) return;
  float* init = e < D * D ? a.S + int64_t(bh) * D * D + e : a.z + int64_t(bh) * D + (e - D * D);
  f32x4 carry = *reinterpret_cast<const f32x4*>(init);
  float mc = ML ? a.stab[bh] : 0.f;
  float* base = a.ws_state + int64_t(bh) * a.nslot * E + e;
  const float* lg = a.ws_logg + int64_t(bh) * a.nslot;
  const float* mg = ML ? a.ws_m + int64_t(bh) * a.nslot : nullptr;
  float* m0g = ML ? a.ws_m0 + int64_t(bh) * (a.nseg + 1) : nullptr;
  for (int s0 = 0; s0 < a.nslot; s0 += U) {
    f32x4 x[U];
    float gm[U], mu[ML ? U : 1];
    // unconditional loads (slot index clamped), so that all are in flight
    // together
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int uc = min(s0 + j, a.nslot - 1);
      x[j] = *reinterpret_cast<const f32x4*>(base + int64_t(uc) * E);
      gm[j] = lg[uc];
      if constexpr (ML) mu[j] = mg[uc];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = s0 + j;
      if (u < a.nslot) {
        if (u % a.nsub == 0) {
          *reinterpret_cast<f32x4*>(base + int64_t(u) * E) = carry;
          if (ML && e == 0) m0g[u / a.nsub] = mc;
        }
        if constexpr (ML) {
          const float mn = fmaxf(mc + gm[j], mu[j]);
          const float f0 = __expf(mc + gm[j] - mn), f1 = __expf(mu[j] - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) carry[i] = fmaf(f0, carry[i], f1 * x[j][i]);
          mc = mn;
        } else {
          const float g = __expf(gm[j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) carry[i] = fmaf(g, carry[i], x[j][i]);
        }
      }
    }
  }
  *reinterpret_cast<f32x4*>(init) = carry;
  if (ML && e == 0) m0g[a.nseg] = mc;
}

// ---------------------------------------------------------------- stage 3

// Output stage, warp-specialised: a workgroup of 2 NW waves holds NW
// consumer waves (the MFMA work: read-out, scores, P V, fold; each owns 32
// value columns of the state in accumulators) and NW producer waves (the
// loads and the VALU staging: feature maps, bf16 splits, tiles, denominators
// and z).  With two LDS buffers the producers stage chunk c + 1 while the
// consumers compute chunk c, one barrier per chunk; each role fits in 256
// registers, so a producer and a consumer wave share every SIMD.
// NC: the non-causal read-out.  Every segment starts from the state of the
// whole sequence (stage 1 and the scan leave it in S, z), so the producers
// stage phi(q) and the denominators only, and the consumers do the read-out
// alone: no scores, no P V, no fold.
template <int D, int C, int DECAY, typename DT, bool NC = false>
__global__ __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(2, 2)))
void output_kernel(const PfArgs a) {
  constexpr bool VS = __is_same(DT, f16_t);   // fp16 v needs a bf16 low part too
  // decays with 32-token chunks take the decay mask from the producers (DM)
  using G = Cfg<D, C, VS, DECAY != 0 && C == 32 && !NC>;
  __shared__ __align__(16) char smem[G::LDS];
  const int nseg = a.nseg;
  const int bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int nchunks = (a.T + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(c0 + a.cps, nchunks);
  const int nc = c1 - c0;
  // With several segments the final state comes from stage 1 and the scan
  // (which fold w phi(k) as bf16 high + low parts); the output stage then
  // folds only the high parts, as its state feeds this segment's outputs
  // alone.  A single segment folds both parts and writes the final state.
  const bool fin = !NC && nseg == 1;
  const bool from_ws = !NC && nseg > 1;
  const float* Sstart = from_ws ? a.ws_state + (int64_t(bh) * a.nslot + a.nsub * seg) * (D * D + D)
                                : a.S + int64_t(bh) * D * D;
  const float* zstart = from_ws ? Sstart + D * D : a.z + int64_t(bh) * D;
  auto buffer = [&](int i) -> char* { return smem + (G::NBUF == 2 ? (i & 1) * G::BUF3 : 0); };

  // the role is uniform per wave: tell the compiler, so the two roles are
  // separate paths rather than one masked sequence with both live sets
  const int wave_id = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  if (wave_id >= G::NW) {
    // =================================================== producer waves
    const int ts = threadIdx.x - G::NT, lane = ts & 63, wave = ts >> 6;
    const int fb = ts % G::FB;
    // Row group of this thread (rows RPT rg .. RPT rg + RPT - 1 of a chunk).
    // At 16 feature blocks and 2 rows per thread, bits 0 and 1 of the group
    // index are swapped: the two row groups a half-wave writes (8-byte
    // pieces of the Q and K rows) are then 4 rows apart, and the XOR
    // swizzle puts them in disjoint banks.
    const int rg0 = ts / G::FB;
    const int rg = (G::FB == 16 && G::RPT == 2) ? ((rg0 & ~3) | ((rg0 & 1) << 1) | ((rg0 >> 1) & 1))
                                                : rg0;
    const DT* qg = static_cast<const DT*>(a.q) + int64_t(bh) * a.T * D;
    const DT* kg = static_cast<const DT*>(a.k) + int64_t(bh) * a.T * D;
    const DT* vg = static_cast<const DT*>(a.v) + int64_t(bh) * a.T * D;
    const float* dg = DECAY ? a.decay + int64_t(bh) * a.T : nullptr;
    const float* igp = DECAY == 3 ? a.igate + int64_t(bh) * a.T : nullptr;
    float zf[8];   // z of features 8 fb .. 8 fb + 7 before the chunk being staged
    *reinterpret_cast<f32x4*>(zf) = *reinterpret_cast<const f32x4*>(zstart + 8 * fb);
    *reinterpret_cast<f32x4*>(zf + 4) = *reinterpret_cast<const f32x4*>(zstart + 8 * fb + 4);
    // mLSTM: stabiliser of the state before the chunk being staged
    float m0 = 0.f;
    if constexpr (DECAY == 3) m0 = from_ws ? a.ws_m0[int64_t(bh) * (nseg + 1) + seg] : a.stab[bh];
    // log of the decay from the segment's start to the chunk being staged
    float lrun = 0.f;
    // the consumers' state scale after the chunks staged so far (S = e^lp acc)
    float lp = 0.f;

    using Raw = RawChunk<G::RPT, G::ND, true, !NC, DECAY == 3>;
    auto fetch = [&](Raw& r, int c) {
      fetch_chunk<C, D, G::RPT, G::ND, true, DECAY>(r, qg, kg, vg, dg, igp, c * C, a.T, rg, fb,
                                                     lane);
    };
    // [A] chunk c into buf: phi(q), phi(k) and w phi(k) high/low, v tiles;
    // the inter-chunk denominators e^{lc_t} phi(q_t).z; lc_t, beta_t; the
    // per-wave z increments; the chunk's total log-decay.  Rows past the end
    // of the sequence hold k = v = 0 (phi = 1, no contribution to S; their
    // 1s are taken off z without decay) and their outputs are not stored.
    // Past the segment's last chunk this stages a repeat of it into a buffer
    // nobody reads, so that the loads are the same on every path.
    auto stage = [&](Raw& raw, int c, char* buf) -> float {
      const int tok0 = c * C;
      clean_chunk<C, G::RPT, G::ND, true, DECAY>(raw, tok0, a.T, rg, lane, a.fgate_exp);
      float lo = 0.f, hi = 0.f, ltot = 0.f;
      if constexpr (DECAY != 0) chunk_logprefix<C, G::ND, DECAY == 3>(raw.d, lane, lo, hi, ltot);
      float alo = 0.f, ahi = 0.f, mlo = 0.f, mhi = 0.f, mend = 0.f;
      if constexpr (DECAY == 3) chunk_runmax<C, G::ND>(raw.ig, lo, hi, m0, lane, alo, ahi, mlo, mhi, mend);
      float* Ll = reinterpret_cast<float*>(buf + G::B_L);
      float* Bl = reinterpret_cast<float*>(buf + G::B_B);
      float* denl = reinterpret_cast<float*>(buf + G::B_DEN);
      float* Ml = reinterpret_cast<float*>(buf + G::B_M);
      if constexpr (NC) {
        // phi(q) and phi(q) . z of the whole sequence
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) {
          const int r = G::RPT * rg + i;
          float qx[8];
          unpack8(raw.q[i], qx, DT{});
          float den = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            qx[e] = elu1_fast(qx[e]);
            den = fmaf(qx[e], zf[e], den);
          }
          row_write_perm<D>(buf + G::B_Q, r, fb, pack8(qx));
          den = row_sum<G::FB>(den);
          if (fb == 0) denl[r] = den;
        }
        fetch(raw, min(c + G::PDEPTH, c1 - 1));
        return 0.f;
      }
      // this thread's z increments: its first row sets them (adding to 0.f
      // would cost an instruction each, kept for the sign of zero)
      float dz[8];
      // the chunks read out (prec) and folded (exact) at high + low precision (see QR)
      const bool prec = DECAY != 3 && tok0 < G::PRECISE && (DECAY == 0 || lrun > G::PREC_LOG);
      const bool exact = DECAY != 3 && tok0 < G::EXACT;
      // log of the carry factor: the chunk's total log-decay (mLSTM: m0 - mu_last)
      const float lgam = DECAY == 3 ? m0 - mend : ltot;
      // the consumers keep the state at scale e^lp: while |lp + lgam| stays
      // within kDeferLog the decay goes into lp and the fold weights take
      // e^-(lp + lgam); past it the consumers apply the factor (lp = 0)
      const float lnew = lp + lgam;
      const float lsc = DECAY != 0 && fabsf(lnew) <= kDeferLog ? lnew : 0.f;
      // mLSTM with one token per lane (C <= 64): the per-token factors below
      // are formed once, in the token's lane, and the rows read them from
      // there (the same operations on the same values as forming them per row)
      constexpr bool TOKF = DECAY == 3 && G::ND == 1;
      float wl = 0.f, efl = 0.f;
      if constexpr (TOKF) {
        const float lctl = m0 - mlo;
        wl = tok0 + lane < a.T ? __expf(alo - mend - lsc) : 0.f;
        efl = __expf(lctl);
        if (wave == 0 && lane < C) {
          Ll[lane] = lctl;
          Bl[lane] = G::HAS_DM ? 1.f : __expf(alo - mlo);
          Ml[lane] = lo + mlo;
        }
      }
#pragma unroll
      for (int i = 0; i < G::RPT; ++i) {
        const int r = G::RPT * rg + i;
        float qx[8], kx[8];
        unpack8(raw.q[i], qx, DT{});
        unpack8(raw.k[i], kx, DT{});
        float lct = 0.f, w = 1.f, beta = 1.f, mt = 0.f, ef = 1.f;
        if constexpr (TOKF) {
          w = lane_value<C>(wl, 0.f, r);
          ef = lane_value<C>(efl, 0.f, r);
        } else if constexpr (DECAY == 3) {
          // lct := m0 - mu_t (inter-chunk factor e^{lct}); beta := e^{a_t - mu_t},
          // so that e^{lct_t - lct_s} beta_s = e^{a_s - mu_t}; m_t = lc_t + mu_t
          const float mu = lane_value<C>(mlo, mhi, r), at = lane_value<C>(alo, ahi, r);
          lct = m0 - mu;
          if constexpr (!G::HAS_DM) beta = __expf(at - mu);   // else in the decay mask
          w = tok0 + r < a.T ? __expf(at - mend - lsc) : 0.f;
          mt = lane_value<C>(lo, hi, r) + mu;
        } else if constexpr (DECAY != 0) {
          lct = lane_value<C>(lo, hi, r);
          if constexpr (DECAY == 2)
            beta = 1.f - lane_value<C>(raw.d[0], G::ND > 1 ? raw.d[G::ND - 1] : 0.f, r);
          w = tok0 + r < a.T ? beta * __expf(ltot - lct - lsc) : 0.f;
        }
        float den = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (DECAY != 3) {   // mLSTM: identity features
            qx[e] = elu1_fast(qx[e]);
            kx[e] = elu1_fast(kx[e]);
          }
          den = fmaf(qx[e], zf[e], den);
        }
        // identity features of bf16 inputs (mLSTM): the tiles are the inputs
        constexpr bool RAW = DECAY == 3 && __is_same(DT, bf16_t);
        const u32x4 qp = RAW ? raw.q[i] : pack8(qx);
        row_write_perm<D>(buf + G::B_Q, r, fb, qp);
        if (prec || exact) row_write_perm<D>(buf + G::B_QR, r, fb, low8(qx, qp));
        const u32x4 kp = RAW ? raw.k[i] : pack8(kx);
        row_write_perm<D>(buf + G::B_K, r, fb, kp);
        if (tok0 < G::EXACT) row_write_perm<D>(buf + G::B_KR, r, fb, low8(kx, kp));
        if constexpr (DECAY != 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kx[e] *= w;
            dz[e] = i == 0 ? kx[e] : dz[e] + kx[e];
          }
          const u32x4 kh = pack8(kx);
          blk_write<D>(buf + G::B_KH, perm_pos(r), fb, kh);
          if (fin || DECAY == 3 || exact)
            blk_write<D>(buf + G::B_KL, perm_pos(r), fb, low8(kx, kh));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) dz[e] = i == 0 ? kx[e] : dz[e] + kx[e];
          blk_write<D>(buf + G::B_KH, perm_pos(r), fb, kp);
          if (fin || exact) blk_write<D>(buf + G::B_KL, perm_pos(r), fb, low8(kx, kp));
        }
        if constexpr (VS) {
          float vx[8];
          unpack8(raw.v[i], vx, DT{});
          const u32x4 vh = pack8(vx);
          blk_write<D>(buf + G::B_VH, perm_pos(r), fb, vh);
          blk_write<D>(buf + G::B_VL, perm_pos(r), fb, low8(vx, vh));
        } else {
          blk_write<D>(buf + G::B_VH, perm_pos(r), fb, raw.v[i]);
        }
        den = row_sum<G::FB>(den);
        if (fb == 0) {
          if constexpr (TOKF) {
            denl[r] = den * ef;
          } else {
            if constexpr (DECAY != 0) den *= __expf(lct);
            denl[r] = den;
            Ll[r] = lct;
            Bl[r] = beta;
            if constexpr (DECAY == 3) Ml[r] = mt;
          }
        }
      }
      {
        float s0, s1;
        const int base = reduce_scatter8<G::FB>(dz, lane, s0, s1);
        if constexpr (DECAY != 0) {   // z itself is kept at scale 1
          const float f = __expf(lsc);
          s0 *= f;
          s1 *= f;
        }
        if (G::FB == 16 || !(lane & 8))
          *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(buf + G::B_DZ) + wave * G::DZS +
                                    dz_index(fb, base)) = f32x2{s0, s1};
      }
      if constexpr (G::HAS_DM) {
        // the decay mask of the chunk's scores, DM[t][s] = e^{lc_t - lc_s}
        // beta_s for s <= t (mLSTM: e^{a_s - mu_t}), else 0; four entries per
        // thread and pass, every lane in every cross-lane read
#pragma unroll
        for (int idx = ts; idx < C * C / 4; idx += G::NT) {
          const int t = idx / (C / 4), s0 = 4 * (idx % (C / 4));
          const float rt = DECAY == 3 ? lane_value<C>(mlo, mhi, t) : lane_value<C>(lo, hi, t);
          f32x4 dm;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x;
            if constexpr (DECAY == 3) {
              x = __expf(lane_value<C>(alo, ahi, s0 + e) - rt);
            } else {
              x = __expf(rt - lane_value<C>(lo, hi, s0 + e));
              if constexpr (DECAY == 2)
                x *= 1.f - lane_value<C>(raw.d[0], G::ND > 1 ? raw.d[G::ND - 1] : 0.f, s0 + e);
            }
            dm[e] = s0 + e <= t ? x : 0.f;
          }
          *reinterpret_cast<f32x4*>(buf + G::B_DM + 4 * (t * G::DMS + s0)) = dm;
        }
      }
      if (ts == 0) *reinterpret_cast<float*>(buf + G::B_LT) = lgam;
      if constexpr (DECAY == 3) {
        if (c < c1) m0 = ltot + mend;   // the stabiliser after this chunk
      } else if constexpr (DECAY != 0) {
        if (c < c1) lrun += ltot;
      }
      if (c < c1) lp = lsc;
      // refill this register set with the chunk PDEPTH ahead (clamped)
      fetch(raw, min(c + G::PDEPTH, c1 - 1));
      return lgam;
    };
    // z after chunk c (staged in buf): zf = e^{ltot} zf + sum of the increments
    auto zstep = [&](int c, const char* buf, float ltot) {
      if constexpr (NC) return;   // z is the whole sequence's throughout
      const float* dzl = reinterpret_cast<const float*>(buf + G::B_DZ);
      const float gam = DECAY ? __expf(ltot) : 1.f;
      const float pad = DECAY ? 0.f : float(max(c * C + C - a.T, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float s = -pad;
#pragma unroll
        for (int w = 0; w < G::NW; ++w) s += dzl[w * G::DZS + dz_index(fb, e)];
        zf[e] = fmaf(gam, zf[e], s);
      }
    };

    Raw raw[G::PDEPTH];
#pragma unroll
    for (int j = 0; j < G::PDEPTH; ++j) fetch(raw[j], min(c0 + j, c1 - 1));
    if constexpr (G::NBUF == 2) {
      float lt = stage(raw[0], c0, buffer(0));
      __syncthreads();
      for (int i0 = 0; i0 < nc; i0 += G::PDEPTH) {
#pragma unroll
        for (int j = 0; j < G::PDEPTH; ++j) {
          const int i = i0 + j;
          if (i < nc) zstep(c0 + i, buffer(i), lt);   // zf: the normaliser after chunk c0 + i
          lt = stage(raw[(j + 1) % G::PDEPTH], c0 + i + 1, buffer(i + 1));
          if (i < nc) __syncthreads();
        }
      }
    } else {
      for (int i0 = 0; i0 < nc; i0 += G::PDEPTH) {
#pragma unroll
        for (int j = 0; j < G::PDEPTH; ++j) {
          const int i = i0 + j;
          const float lt = stage(raw[j], c0 + i, buffer(0));
          if (i < nc) {
            __syncthreads();
            zstep(c0 + i, buffer(0), lt);
            __syncthreads();
          }
        }
      }
    }
    if (fin && rg == 0) {
      float* zd = a.z + int64_t(bh) * D + 8 * fb;
      *reinterpret_cast<f32x4*>(zd) = f32x4{zf[0], zf[1], zf[2], zf[3]};
      *reinterpret_cast<f32x4*>(zd + 4) = f32x4{zf[4], zf[5], zf[6], zf[7]};
    }
    if constexpr (DECAY == 3) {
      // the final stabiliser: this segment's (one segment) or the scan's
      if (ts == 0 && (fin || seg == 0))
        a.stab[bh] = fin ? m0 : a.ws_m0[int64_t(bh) * (nseg + 1) + nseg];
    }
  } else {
    // =================================================== consumer waves
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    DT* og = static_cast<DT*>(a.out) + int64_t(bh) * a.T * D;
    float* ogf = static_cast<float*>(a.out) + int64_t(bh) * a.T * D;
    f32x16 acc[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        acc[mt][r] = Sstart[f * D + 32 * wave + n];
      }

    // log of the decay from the segment's start to the chunk being computed
    // (the producers' lrun, from the chunks' totals)
    float lrun = 0.f;
    // the state is S = e^lp acc (decays only; the producers track lp alike)
    float lp = 0.f;
    // [B] read-out of the carried state, masked intra-chunk attention,
    // normalise and store, then fold the chunk into S.
    auto compute = [&](int c, const char* buf) {
      const int tok0 = c * C;
      const float* Ll = reinterpret_cast<const float*>(buf + G::B_L);
      const float* Bl = reinterpret_cast<const float*>(buf + G::B_B);
      const float* denl = reinterpret_cast<const float*>(buf + G::B_DEN);
      const float* Ml = reinterpret_cast<const float*>(buf + G::B_M);
      u32x4 vh[G::KT], vl[G::KT];
#pragma unroll
      for (int kk = 0; kk < G::KT; ++kk) {
        if constexpr (NC) break;
        vh[kk] = tr_operand<D>(buf + G::B_VH, 16 * kk, 32 * wave, lane);
        if constexpr (VS) vl[kk] = tr_operand<D>(buf + G::B_VL, 16 * kk, 32 * wave, lane);
      }
      // Fold this chunk into the carried state: w phi(k) high parts, and
      // (fold_lo) the low parts when this one segment also produces the
      // final state (`fin`).  With one 32-token block the high-part fold
      // follows the read-out directly (which has consumed the state by
      // then), so its MFMA chains overlap the masking and P V work.
      auto fold_hi = [&]() {
        if constexpr (DECAY != 0) {
          // the chunk's decay goes into lp, or into the accumulators once
          // |lp| would pass kDeferLog (the producers, who scaled the fold
          // weights by e^-lp, made the same choice from the same values)
          const float lnew = lp + *reinterpret_cast<const float*>(buf + G::B_LT);
          if (fabsf(lnew) <= kDeferLog) {
            lp = lnew;
          } else {
            const float gam = __expf(lnew);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt) acc[mt] *= gam;
            lp = 0.f;
          }
        }
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
          for (int kk = 0; kk < G::KT; ++kk) {
            const u32x4 kh = tr_operand<D>(buf + G::B_KH, 16 * kk, 32 * mt, lane);
            acc[mt] = mfma(kh, vh[kk], acc[mt]);
            if constexpr (VS) acc[mt] = mfma(kh, vl[kk], acc[mt]);
          }
        }
      };
      auto fold_lo = [&]() {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int kk = 0; kk < G::KT; ++kk)
            acc[mt] = mfma(tr_operand<D>(buf + G::B_KL, 16 * kk, 32 * mt, lane), vh[kk], acc[mt]);
      };
      // the chunks read out (prec, as the producers decided) and folded
      // (exact) at high + low precision (see QR)
      bool prec = !NC && DECAY == 0 && tok0 < G::PRECISE;
      if constexpr (!NC && DECAY != 0 && DECAY != 3) prec = tok0 < G::PRECISE && lrun > G::PREC_LOG;
      const bool exact = !NC && DECAY != 3 && tok0 < G::EXACT;
      const float lp0 = lp;   // the scale of the state this chunk reads out
#pragma unroll
      for (int tb = 0; tb < G::TB; ++tb) {
        const int tl = 32 * tb + n;   // this lane's query token within the chunk
        // read-out of the carried state O^T = S^T phi(Q)^T (the fp32
        // accumulators become bf16 operands, k = features) and the diagonal
        // score block in one pass over the feature k-steps
        f32x16 o = f32x16{}, p = f32x16{};
        auto readout = [&](auto split_tag) {
          constexpr bool SPLIT = decltype(split_tag)::value;
#pragma unroll
          for (int ks = 0; ks < G::KS; ++ks) {
            const u32x4 qf = row_operand<D>(buf + G::B_Q, tl, 2 * ks + g);
            const f32x16& sa = acc[ks >> 1];
            const int j0 = 8 * (ks & 1);
            if constexpr (DECAY == 3 || SPLIT) {
              // the state as bf16 high + low parts: identity features cancel
              // in phi(q) . S (mLSTM), and the first outputs of a long
              // sequence stand out against its rms (elu+1 features are
              // positive and average the rounding out further on)
              u32x4 sh, sl;
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                uint32_t x, y;
                split_bf16(sa[j0 + 2 * h], sa[j0 + 2 * h + 1], x, y);
                sh[h] = x;
                sl[h] = y;
              }
              o = mfma(sh, qf, o);
              o = mfma(sl, qf, o);
              if constexpr (SPLIT) o = mfma(sh, row_operand<D>(buf + G::B_QR, tl, 2 * ks + g), o);
            } else {
              const u32x4 sf = {pack_bf16(sa[j0 + 0], sa[j0 + 1]), pack_bf16(sa[j0 + 2], sa[j0 + 3]),
                                pack_bf16(sa[j0 + 4], sa[j0 + 5]), pack_bf16(sa[j0 + 6], sa[j0 + 7])};
              o = mfma(sf, qf, o);
            }
            if constexpr (!NC) p = mfma(row_operand<D>(buf + G::B_K, 32 * tb + n, 2 * ks + g), qf, p);
          }
        };
        if constexpr (NC || DECAY == 3) {
          readout(std::false_type{});
        } else {
          if (prec) readout(std::true_type{});
          else readout(std::false_type{});
        }
        if (!NC && tok0 < G::EXACT) {
          p = low_scores<D, G::KS>(buf + G::B_KR, buf + G::B_Q, 32 * tb + n, tl, g, p);
          if constexpr (DECAY != 3)
            p = low_scores<D, G::KS>(buf + G::B_K, buf + G::B_QR, 32 * tb + n, tl, g, p);
        }
        if constexpr (!NC && G::TB == 1) fold_hi();
        float lct = 0.f;
        if constexpr (DECAY != 0) {
          lct = Ll[tl];
          o *= __expf(lct + lp0);
        }
        float dsum = 0.f;
#pragma unroll
        for (int sb = tb; sb >= 0; --sb) {
          if constexpr (NC) break;
          if (sb != tb) {
            p = f32x16{};
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks)
              p = mfma(row_operand<D>(buf + G::B_K, 32 * sb + n, 2 * ks + g),
                       row_operand<D>(buf + G::B_Q, tl, 2 * ks + g), p);
            if (tok0 < G::EXACT) {
              p = low_scores<D, G::KS>(buf + G::B_KR, buf + G::B_Q, 32 * sb + n, tl, g, p);
              if constexpr (DECAY != 3)
                p = low_scores<D, G::KS>(buf + G::B_K, buf + G::B_QR, 32 * sb + n, tl, g, p);
            }
          }
          if constexpr (G::HAS_DM) {
            // one 32-token block: the producers' decay mask, causal zeros included
            const float* dml = reinterpret_cast<const float*>(buf + G::B_DM) + tl * G::DMS + 4 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 m = *reinterpret_cast<const f32x4*>(dml + 8 * j);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x = p[4 * j + e] * m[e];
                p[4 * j + e] = x;
                dsum += x;
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int sl = 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
              float x = p[r];
              if constexpr (DECAY != 0) x *= __expf(lct - Ll[sl]) * Bl[sl];
              if (sb == tb && sl > tl) x = 0.f;
              p[r] = x;
              dsum += x;
            }
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
        if constexpr (!NC) dsum = swap_sum32(dsum);
        const float dn = denl[tl] + dsum;
        float inv;
        if constexpr (DECAY == 3) {
          // state scaled by e^{-m_t}: the read-out's floor and eps scale with it
          const float mt = Ml[tl];
          inv = a.norm == LA_NORM_NONE ? __expf(mt)
              : a.norm == LA_NORM_MAX1 ? __builtin_amdgcn_rcpf(fmaxf(fabsf(dn), __expf(-mt)))
                                       : __builtin_amdgcn_rcpf(dn + a.eps * __expf(-mt));
        } else {
          inv = a.norm == LA_NORM_NONE ? 1.f
              : a.norm == LA_NORM_MAX1 ? __builtin_amdgcn_rcpf(fmaxf(fabsf(dn), 1.f))
                                       : __builtin_amdgcn_rcpf(dn + a.eps);
        }
        const int t = tok0 + tl;
        if (t < a.T) {
          const uint32_t orow = uint32_t(t) * D + 32 * wave + 4 * g;
          if (a.out_f32) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<f32x4*>(ogf + orow + 8 * j) =
                  f32x4{o[4 * j] * inv, o[4 * j + 1] * inv, o[4 * j + 2] * inv, o[4 * j + 3] * inv};
          } else {
            // lane (g, n) holds value columns 8 j + 4 g .. + 3 (j = 0..3) of
            // token n; a half-wave swap of the odd and even groups leaves
            // lane g with columns 16 m + 8 g .. + 7 (m = 0, 1): 16-byte stores
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float y0 = o[4 * j] * inv, y1 = o[4 * j + 1] * inv;
              const float y2 = o[4 * j + 2] * inv, y3 = o[4 * j + 3] * inv;
              if constexpr (__is_same(DT, bf16_t)) {
                w[2 * j] = pack_bf16(y0, y1);
                w[2 * j + 1] = pack_bf16(y2, y3);
              } else {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                w[2 * j] = __builtin_bit_cast(uint32_t, h2{(f16_t)y0, (f16_t)y1});
                w[2 * j + 1] = __builtin_bit_cast(uint32_t, h2{(f16_t)y2, (f16_t)y3});
              }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              swap_halves(w[4 * m], w[4 * m + 2]);
              swap_halves(w[4 * m + 1], w[4 * m + 3]);
              *reinterpret_cast<u32x4*>(og + uint32_t(t) * D + 32 * wave + 16 * m + 8 * g) =
                  u32x4{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
            }
          }
        }
      }
      if constexpr (!NC) {
        if constexpr (G::TB > 1) fold_hi();
        if (fin || DECAY == 3 || exact) fold_lo();   // mLSTM: the state always as high + low
      }
      if constexpr (DECAY != 0 && DECAY != 3) lrun += *reinterpret_cast<const float*>(buf + G::B_LT);
    };

    if constexpr (G::NBUF == 2) {
      __syncthreads();   // the producers' first chunk
      for (int i0 = 0; i0 < nc; i0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int i = i0 + j;
          if (i < nc) {
            compute(c0 + i, smem + j * G::BUF3);
            __syncthreads();
          }
        }
      }
    } else {
      for (int i = 0; i < nc; ++i) {
        __syncthreads();   // chunk c0 + i staged
        compute(c0 + i, smem);
        __syncthreads();
      }
    }
    if (fin) {
      float* Sd = a.S + int64_t(bh) * D * D;
      const float sc = DECAY != 0 ? __expf(lp) : 1.f;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int f = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
          Sd[f * D + 32 * wave + n] = acc[mt][r] * sc;
        }
    }
  }
}

// ---------------------------------------------------------------- dispatch

// LA_STAGE1_MFMA=16x16x32 in the environment selects the stage-1 fold on
// v_mfma_f32_16x16x32_bf16 for the 128-wide, 32-token, bf16 prefill without
// a decay (the configuration its measurement covers); read at every launch.
bool stage1_mfma16() {
  const char* e = std::getenv("LA_STAGE1_MFMA");
  return e && std::strcmp(e, "16x16x32") == 0;
}

template <int D, int C, int DECAY, typename DT>
hipError_t launch3(const PfArgs& a, int64_t BH, int stage, hipStream_t st) {
  using G = Cfg<D, C, __is_same(DT, f16_t)>;
  // a causal prefill of one segment needs neither stage 1 nor the scan (the
  // output stage carries the state itself); a non-causal one always does
  const bool scan = a.nseg > 1 || a.nc;
  if (stage == 1) {
    if (!scan) return hipSuccess;
    if constexpr (D == 128 && C == 32 && DECAY == 0 && __is_same(DT, bf16_t)) {
      if (stage1_mfma16()) {
        segment_state_kernel<D, C, DECAY, DT, true>
            <<<dim3(unsigned(BH * a.nslot)), dim3(2 * G::NT), 0, st>>>(a);
        return hipGetLastError();
      }
    }
    segment_state_kernel<D, C, DECAY, DT><<<dim3(unsigned(BH * a.nslot)), dim3(2 * G::NT), 0, st>>>(a);
  } else if (stage == 2) {
    if (!scan) return hipSuccess;
    const int per_bh = ((D * D + D) / 4 + 255) / 256;
    // 16 slots of four elements in flight at once per thread (64 registers)
    if constexpr (DECAY == 3)
      segment_scan_kernel<D, 16, true><<<dim3(unsigned(BH * per_bh)), dim3(256), 0, st>>>(a);
    else
      segment_scan_kernel<D, 16, false><<<dim3(unsigned(BH * per_bh)), dim3(256), 0, st>>>(a);
  } else if (a.nc) {
    if constexpr (DECAY != 0) return hipErrorInvalidValue;   // rejected on the host
    else output_kernel<D, C, 0, DT, true><<<dim3(unsigned(BH * a.nseg)), dim3(2 * G::NT), 0, st>>>(a);
  } else {
    output_kernel<D, C, DECAY, DT><<<dim3(unsigned(BH * a.nseg)), dim3(2 * G::NT), 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int D, int C, typename DT>
hipError_t launch_decay(const PfArgs& a, int64_t BH, la_decay kind, int stage, hipStream_t st) {
  switch (kind) {
    case LA_DECAY_NONE: return launch3<D, C, 0, DT>(a, BH, stage, st);
    case LA_DECAY_SSD: return launch3<D, C, 1, DT>(a, BH, stage, st);
    case LA_GATE_RFA: return launch3<D, C, 2, DT>(a, BH, stage, st);
    case LA_GATE_MLSTM: return launch3<D, C, 3, DT>(a, BH, stage, st);
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

// Chunk bookkeeping of a plan: chunks per segment, segment count, stage-1
// sub-segments per segment (two when a segment has at least two chunks, so
// that stage 1 runs two workgroups per compute unit) and workspace slots.
struct Split {
  int cps, nseg, nsub, cps_sub, nslot;
};

Split split_of(const Problem& p) {
  Split q;
  const int nchunks = (p.T + p.chunk - 1) / p.chunk;
  q.cps = (nchunks + p.segments - 1) / p.segments;
  q.nseg = q.cps > 0 ? (nchunks + q.cps - 1) / q.cps : 1;
  q.nsub = q.cps >= 2 ? 2 : 1;
  q.cps_sub = (q.cps + q.nsub - 1) / q.nsub;
  q.nslot = q.nsub * q.nseg;
  return q;
}

}  // namespace

void mfma_split(const Problem& p, int* cps, int* nseg, int* nsub, int* nslot) {
  const Split sp = split_of(p);
  *cps = sp.cps;
  *nseg = sp.nseg;
  *nsub = sp.nsub;
  *nslot = sp.nslot;
}

bool mfma_supported(const Problem& p) {
  // elu+1 with no decay, SSD decay or the RFA gate (bf16 or fp16 inputs);
  // identity features with the mLSTM gates, bf16 inputs only: the MFMA
  // operands are bf16, which holds bf16 q, k exactly, while fp16 q, k would
  // be rounded, and identity features cancel in q.k (elu+1 features are
  // positive and average that rounding out)
  const bool mlstm = p.decay_kind == LA_GATE_MLSTM;
  const bool pair = mlstm ? p.phi == LA_PHI_IDENTITY && p.dtype == LA_BF16
                          : p.phi == LA_PHI_ELU1 && (p.dtype == LA_BF16 || p.dtype == LA_F16);
  return pair && p.dp == p.dv && (p.dv == 64 || p.dv == 128);
}

// Chunks whose stage-3 tiles fit in the 160 KB of LDS of one compute unit.
bool mfma_chunk_fits(int d, int chunk) { return chunk <= 64 || d <= 64; }

// The output stage holds one 8-wave workgroup per compute unit at d = 128
// (two 4-wave ones at d = 64): aim for exactly that many workgroups on the
// 256 compute units, with at least two chunks per segment.
int mfma_default_segments(const Problem& p) {
  const int64_t target_wg = p.dv == 128 ? 256 : 512;
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

// Workspace: the slot states, then three fp32 arrays each rounded up to 256
// bytes: log Gamma per slot, the mLSTM stabiliser per slot, and the mLSTM
// start stabiliser per segment plus the final one (reserved for every decay
// kind, so the size does not depend on it).
static size_t round256(size_t bytes) { return ((bytes + 255) / 256) * 256; }

size_t mfma_workspace_bytes(const Problem& p) {
  if (p.path != 1 || (p.segments <= 1 && !p.noncausal)) return 0;
  const size_t E = size_t(p.dv) * p.dv + p.dv;
  const Split sp = split_of(p);
  const size_t n = size_t(p.BH()) * sp.nslot;
  return n * E * sizeof(float) + 2 * round256(n * sizeof(float)) +
         round256(size_t(p.BH()) * (sp.nseg + 1) * sizeof(float));
}

float* mfma_ws_m0(const Problem& p, void* ws) {
  const Split sp = split_of(p);
  const size_t E = size_t(p.dv) * p.dv + p.dv;
  const size_t n = size_t(p.BH()) * sp.nslot;
  return reinterpret_cast<float*>(static_cast<char*>(ws) + n * E * sizeof(float) +
                                  2 * round256(n * sizeof(float)));
}

hipError_t launch_mfma_stage(const Problem& p, int stage, const void* q, const void* k,
                             const void* v, float* S, float* z, void* out, void* ws,
                             hipStream_t stream) {
  PfArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.S = S; a.z = z; a.decay = p.decay;
  a.igate = p.igate; a.stab = p.stab; a.fgate_exp = p.fgate_exp;
  a.T = p.T;
  const Split sp = split_of(p);
  a.cps = sp.cps;
  a.nseg = sp.nseg;
  a.nsub = sp.nsub;
  a.cps_sub = sp.cps_sub;
  a.nslot = sp.nslot;
  a.eps = p.eps;
  a.norm = p.norm;
  a.nc = p.noncausal;
  a.out_f32 = p.out_dtype == LA_F32 ? 1 : 0;
  a.ws_logg = nullptr;
  a.ws_state = nullptr;
  a.ws_m = nullptr;
  a.ws_m0 = nullptr;
  if (a.nseg > 1 || a.nc) {
    const size_t E = size_t(p.dv) * p.dv + p.dv;
    const size_t n = size_t(p.BH()) * a.nslot;
    char* base = static_cast<char*>(ws);
    a.ws_state = reinterpret_cast<float*>(base);
    base += n * E * sizeof(float);
    a.ws_logg = reinterpret_cast<float*>(base);
    base += round256(n * sizeof(float));
    a.ws_m = reinterpret_cast<float*>(base);
    a.ws_m0 = mfma_ws_m0(p, ws);
  }
  if (p.dv == 128) {
    return p.dtype == LA_BF16 ? launch_chunk<128, bf16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream)
                              : launch_chunk<128, f16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream);
  }
  return p.dtype == LA_BF16 ? launch_chunk<64, bf16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream)
                            : launch_chunk<64, f16_t>(a, p.BH(), p.chunk, p.decay_kind, stage, stream);
}

}  // namespace la
