// Internal declarations shared by the host API and the kernel translation
// units of the linattn library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "linattn.h"

namespace la {

// A validated problem description (every field already checked on the host).
struct Problem {
  int B = 0, H = 0, T = 0;
  int dh = 0, dv = 0, dp = 0;   // query/key width, value width, feature width d'
  la_dtype dtype = LA_BF16;
  la_dtype out_dtype = LA_BF16;
  la_phi phi = LA_PHI_ELU1;
  int D = 0;                    // RFF pairs
  const float* W = nullptr;     // [H, D, dh]
  la_decay decay_kind = LA_DECAY_NONE;
  const float* decay = nullptr; // prefill [B,H,T], decode [B,H]
  float eps = 1e-6f;
  int norm = 0;                 // read-out form: LA_NORM_SUM, LA_NORM_NONE or LA_NORM_MAX1
  const float* igate = nullptr; // mLSTM input-gate pre-activations, shaped like decay
  int fgate_exp = 0;            // mLSTM forget gate: 0 sigmoid(decay), 1 exp(decay)
  float* stab = nullptr;        // mLSTM stabiliser m [B, H]
  int noncausal = 0;            // 1: non-causal prefill (every output reads the whole state)
  int chunk = 64;               // prefill chunk length (MFMA path)
  int segments = 1;             // prefill segments per (b,h) (MFMA path)
  int path = 0;                 // 1 = chunked MFMA, 0 = per-token recurrent kernel
  int64_t BH() const { return int64_t(B) * H; }
};

// Per-token recurrent kernel (decode step, and the general prefill path).
// The same device code runs T tokens with the state held in registers.
bool recurrent_supported(int dh, int dp, int dv);
hipError_t launch_recurrent(const Problem& p, const void* q, const void* k, const void* v,
                            float* S, float* z, void* out, hipStream_t stream);

// Decode step, one wave per state (d_v in {64, 128}, d' in {64, 128, 256};
// RFF with d_h <= 128, or elu+1 with d_h = d').  Other shapes take the
// recurrent kernel with T = 1.
bool decode_supported(const Problem& p);
hipError_t launch_decode(const Problem& p, const void* q, const void* k, const void* v,
                         float* S, float* z, void* out, hipStream_t stream);

// Gradients of the causal prefill (per-token, two passes per sequence):
// elu+1 or identity features, no decay / SSD / RFA, every read-out.
bool backward_supported(const Problem& p);
size_t backward_workspace_bytes(const Problem& p);
hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v,
                           const float* S0, const float* z0, const void* dout, float* dq,
                           float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                           void* ws, hipStream_t stream);

// Chunked gradients (la_backward_mfma.hip): bf16 inputs, elu+1, no decay,
// the SSD decay or the RFA gate, d' = d_v in {64, 128}, T > 0.  The plan is
// the prefill's with 32-token chunks.
bool backward_chunked(const Problem& p);
Problem backward_plan(const Problem& p);
size_t backward_chunked_workspace_bytes(const Problem& p);
hipError_t launch_backward_chunked(const Problem& p, const void* q, const void* k, const void* v,
                                   const float* S0, const float* z0, const void* dout, float* dq,
                                   float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                                   void* ws, hipStream_t stream);

// Decay or gate values below this take the exact decay gradient.  Both
// backward paths form dL/dalpha_r as a suffix sum of per-token terms divided
// by alpha_r; that sum is alpha_r <G_r, S_{r-1}> computed as a difference of
// O(1) terms, so its rounding is magnified by 1 / alpha_r (and alpha_r = 0,
// a full reset, gives 0/0).  For alpha_r below the threshold the backward
// writes only the gate's beta term and launch_decay_exact adds
// <G_r, S_{r-1}> + <gz_r, z_{r-1}>, the gradient's definition, by walking the
// state and the read-outs around token r.
constexpr float kDecayExact = 1.0f / 256.0f;

// Inputs of the exact decay gradient for near-zero decays.  The sequence of
// (b, h) is cut into segments of seg_len tokens (the last may be shorter);
// segment s starts from the state (S, z) at S0 + bh s_bh + s s_seg and
// z0 + bh z_bh + s s_seg (zero if S0 is null), and the gradient state
// carried in from beyond its end is (G, gz) at gafter + (bh nseg + s)
// (dp dv + dp) (zero if null).  The read-out's gradient of token t is
// g_t = gs_t gv_t (a dv-vector) and h_t: mode 0 reads gs_t, h_t from
// tok[2 (bh T + t)] and gv_t from dout (fp32 if dout_f32, else the input
// type); mode 1 reads gv_t and h_t from the rows of ws ((dv + 2) floats per
// token) with gs_t = 1.
struct DecayExactArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* decay;
  int decay_kind;
  int phi;
  int mode;
  const float* tok;
  const void* dout;
  int dout_f32;
  const float* ws;
  const float* S0;
  const float* z0;
  int64_t s_bh, z_bh, s_seg;
  const float* gafter;
  int nseg, seg_len;
  float* dd;
  int T, dh, dv, dp;
};
hipError_t launch_decay_exact(const DecayExactArgs& a, la_dtype dtype, int64_t BH,
                              hipStream_t stream);

// Zero-fill of the state (m may be null).
hipError_t launch_state_init(float* S, int64_t nS, float* z, int64_t nz, float* m, int64_t nm,
                             hipStream_t stream);

// Chunked MFMA prefill (16-bit inputs, d' = d_v in {64, 128}; elu+1 with no
// decay, SSD decay or the RFA gate, or the identity map with the mLSTM gates).
bool mfma_supported(const Problem& p);
bool mfma_chunk_fits(int d, int chunk);
int mfma_default_segments(const Problem& p);
size_t mfma_workspace_bytes(const Problem& p);
// The plan's chunk bookkeeping: chunks per segment, segments, stage-1
// sub-segments per segment and workspace slots per (b, h); after stage 2,
// slot nsub * s of (b, h) holds segment s's start state (S then z, D*D + D
// floats per slot, at the start of the workspace).
void mfma_split(const Problem& p, int* cps, int* nseg, int* nsub, int* nslot);
// With more than one segment: the mLSTM stabiliser of each segment's start
// state after stage 2, [BH, nseg + 1] floats in the workspace ws (the final
// one last).
float* mfma_ws_m0(const Problem& p, void* ws);
hipError_t launch_mfma_stage(const Problem& p, int stage, const void* q, const void* k,
                             const void* v, float* S, float* z, void* out, void* ws,
                             hipStream_t stream);

// Device address of this GPU's static scratch array (LA_NOALLOC_SCRATCH_BYTES;
// la_noalloc.hip), looked up on the first call per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace la
