// Host side of the linattn C ABI: argument validation, execution planning and
// dispatch to the kernels.  Nothing here allocates, copies or synchronises;
// every check runs before the first HIP call, so a rejected call has no effect.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "la_internal.h"

namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;  // bound on any tensor's element count

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return *out <= kMaxElems;
}

// Validate the descriptor and fill a Problem.  `prefill` selects which fields
// matter (T and the prefill plan) and how the decay array is shaped.
la_status check_desc(const la_desc* d, bool prefill, la::Problem* p) {
  if (!d) return fail(LA_EINVAL, "desc is NULL");
  if (d->B < 1 || d->H < 1) return fail(LA_EINVAL, "B and H must be >= 1 (got %d, %d)", d->B, d->H);
  if (prefill && d->T < 0) return fail(LA_EINVAL, "T must be >= 0 (got %d)", d->T);
  if (d->d_h < 1 || d->d_v < 1)
    return fail(LA_EINVAL, "d_h and d_v must be >= 1 (got %d, %d)", d->d_h, d->d_v);
  if (d->dtype != LA_F32 && d->dtype != LA_BF16 && d->dtype != LA_F16)
    return fail(LA_EINVAL, "unknown dtype %d", int(d->dtype));
  if (d->out_dtype != d->dtype && d->out_dtype != LA_F32)
    return fail(LA_EINVAL, "out_dtype must equal dtype or be LA_F32 (got %d)", int(d->out_dtype));
  int dp = 0;
  if (d->phi == LA_PHI_ELU1) {
    if (d->rff_D != 0 || d->rff_W != nullptr)
      return fail(LA_EINVAL, "elu+1 feature map takes no rff_D / rff_W");
    dp = d->d_h;
  } else if (d->phi == LA_PHI_IDENTITY) {
    if (d->rff_D != 0 || d->rff_W != nullptr)
      return fail(LA_EINVAL, "identity feature map takes no rff_D / rff_W");
    dp = d->d_h;
  } else if (d->phi == LA_PHI_RFF) {
    if (d->rff_D < 1) return fail(LA_EINVAL, "RFF needs rff_D >= 1 (got %d)", d->rff_D);
    if (!d->rff_W) return fail(LA_EINVAL, "RFF needs rff_W");
    if (!aligned(d->rff_W, 4)) return fail(LA_EINVAL, "rff_W must be 4-byte aligned");
    if (d->rff_D > (1 << 20)) return fail(LA_EINVAL, "rff_D too large");
    dp = 2 * d->rff_D;
  } else {
    return fail(LA_EINVAL, "unknown feature map %d", int(d->phi));
  }
  if (d->decay_kind == LA_DECAY_NONE) {
    if (d->decay) return fail(LA_EINVAL, "decay array given with LA_DECAY_NONE");
  } else if (d->decay_kind == LA_DECAY_SSD || d->decay_kind == LA_GATE_RFA ||
             d->decay_kind == LA_GATE_MLSTM) {
    if (!d->decay) return fail(LA_EINVAL, "decay/gate array missing");
    if (!aligned(d->decay, 4)) return fail(LA_EINVAL, "decay must be 4-byte aligned");
  } else {
    return fail(LA_EINVAL, "unknown decay kind %d", int(d->decay_kind));
  }
  if (d->decay_kind == LA_GATE_MLSTM) {
    if (!d->igate) return fail(LA_EINVAL, "mLSTM gates need igate (input-gate pre-activations)");
    if (!aligned(d->igate, 4)) return fail(LA_EINVAL, "igate must be 4-byte aligned");
    if (!d->stab) return fail(LA_EINVAL, "mLSTM gates need stab (stabiliser state [B, H])");
    if (!aligned(d->stab, 4)) return fail(LA_EINVAL, "stab must be 4-byte aligned");
    if (d->fgate_exp != 0 && d->fgate_exp != 1)
      return fail(LA_EINVAL, "fgate_exp must be 0 or 1 (got %d)", d->fgate_exp);
  } else if (d->igate || d->stab || d->fgate_exp) {
    return fail(LA_EINVAL, "igate, stab and fgate_exp are for LA_GATE_MLSTM only");
  }
  if (!std::isfinite(d->eps)) return fail(LA_EINVAL, "eps must be finite");
  if (d->norm != LA_NORM_SUM && d->norm != LA_NORM_NONE && d->norm != LA_NORM_MAX1)
    return fail(LA_EINVAL, "unknown read-out form %d", int(d->norm));
  if (d->noncausal != 0 && d->noncausal != 1)
    return fail(LA_EINVAL, "noncausal must be 0 or 1 (got %d)", d->noncausal);
  if (d->noncausal && d->decay_kind != LA_DECAY_NONE)
    return fail(LA_EINVAL, "the non-causal form takes no decay or gate");
  if (prefill) {
    if (d->chunk != 0 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128)
      return fail(LA_EINVAL, "chunk must be 0, 32, 64 or 128 (got %d)", d->chunk);
    if (d->segments < 0) return fail(LA_EINVAL, "segments must be >= 0 (got %d)", d->segments);
  }
  int64_t n = 0;
  const int64_t T = prefill ? d->T : 1;
  const int64_t wmax = d->d_h > d->d_v ? d->d_h : d->d_v;
  if (!mul_ok(int64_t(d->B) * d->H, T, &n) || !mul_ok(n, wmax, &n))
    return fail(LA_EINVAL, "tensor too large");
  if (!mul_ok(int64_t(d->B) * d->H, int64_t(dp) * d->d_v, &n)) return fail(LA_EINVAL, "state too large");

  p->B = d->B; p->H = d->H; p->T = prefill ? d->T : 1;
  p->dh = d->d_h; p->dv = d->d_v; p->dp = dp;
  p->dtype = d->dtype; p->out_dtype = d->out_dtype; p->phi = d->phi; p->D = d->rff_D; p->W = d->rff_W;
  p->decay_kind = d->decay_kind; p->decay = d->decay; p->eps = d->eps;
  p->norm = int(d->norm);
  p->igate = d->igate;
  p->fgate_exp = d->fgate_exp;
  p->stab = d->stab;
  p->noncausal = d->noncausal;
  p->chunk = d->chunk ? d->chunk : 32;
  p->segments = 1;
  p->path = 0;
  if (prefill) {
    p->path = la::mfma_supported(*p) ? 1 : 0;
    if (p->path == 1 && !la::mfma_chunk_fits(p->dv, p->chunk))
      return fail(LA_EUNSUPPORTED, "chunk %d needs d' = d_v <= 64 (LDS)", p->chunk);
    if (p->path == 1 && int64_t(p->T) * p->dv >= (int64_t(1) << 31))
      return fail(LA_EUNSUPPORTED, "T * d_v must be < 2^31 per (b, h) for the chunked kernels");
    if (p->path == 1) {
      // effective count: ceil(nchunks / cps) with cps = ceil(nchunks / requested),
      // so that no segment is empty
      const int nchunks = (p->T + p->chunk - 1) / p->chunk;
      int seg = d->segments ? d->segments : la::mfma_default_segments(*p);
      if (seg > nchunks) seg = nchunks;
      if (seg < 1) seg = 1;
      const int cps = (nchunks + seg - 1) / seg;
      p->segments = cps > 0 ? (nchunks + cps - 1) / cps : 1;
    }
  }
  if (p->path == 0 && !la::recurrent_supported(d->d_h, dp, d->d_v))
    return fail(LA_EUNSUPPORTED,
                "unsupported widths d_h=%d d'=%d d_v=%d (need d_h, d', d_v <= 256, d_v/4 a "
                "power of two, d' * d_v <= 32768)", d->d_h, dp, d->d_v);
  return LA_OK;
}

la_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(LA_EINVAL, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(LA_EINVAL, "%s must be 16-byte aligned", name);
  return LA_OK;
}

la_status launched(hipError_t e) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(LA_EHIP, "HIP launch failed: %s", hipGetErrorString(e));
  return LA_OK;
}

#define LA_TRY(expr)                   \
  do {                                 \
    la_status s_ = (expr);             \
    if (s_ != LA_OK) return s_;        \
  } while (0)

la_status check_prefill_ptrs(const la::Problem& p, const void* q, const void* k, const void* v,
                             float* S, float* z, void* out) {
  LA_TRY(check_ptr(S, "S"));
  LA_TRY(check_ptr(z, "z"));
  if (p.T > 0) {
    LA_TRY(check_ptr(q, "q"));
    LA_TRY(check_ptr(k, "k"));
    LA_TRY(check_ptr(v, "v"));
    LA_TRY(check_ptr(out, "out"));
  }
  return LA_OK;
}

la_status check_prefill_args(const la_desc* desc, const void* q, const void* k, const void* v,
                             float* S, float* z, void* out, void* ws, size_t ws_bytes,
                             la::Problem* p) {
  LA_TRY(check_desc(desc, true, p));
  LA_TRY(check_prefill_ptrs(*p, q, k, v, S, z, out));
  const size_t need = p->path == 1 ? la::mfma_workspace_bytes(*p) : 0;
  if (need > 0) {
    if (!ws) return fail(LA_EINVAL, "workspace is NULL (need %zu bytes)", need);
    if (!aligned(ws, 16)) return fail(LA_EINVAL, "workspace must be 16-byte aligned");
    if (ws_bytes < need)
      return fail(LA_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  }
  return LA_OK;
}

la_status run_stage(const la::Problem& p, int stage, const void* q, const void* k,
                    const void* v, float* S, float* z, void* out, void* ws, hipStream_t st) {
  if (p.T == 0) return LA_OK;
  if (p.path == 1) return launched(la::launch_mfma_stage(p, stage, q, k, v, S, z, out, ws, st));
  if (stage != 3) return LA_OK;
  return launched(la::launch_recurrent(p, q, k, v, S, z, out, st));
}

}  // namespace

extern "C" {

int la_feature_dim(const la_desc* desc) {
  la::Problem p;
  if (check_desc(desc, false, &p) != LA_OK) return -1;
  return p.dp;
}

la_status la_state_init(const la_desc* desc, float* S, float* z, void* stream) {
  la::Problem p;
  LA_TRY(check_desc(desc, false, &p));
  LA_TRY(check_ptr(S, "S"));
  LA_TRY(check_ptr(z, "z"));
  (void)hipGetLastError();
  return launched(la::launch_state_init(S, p.BH() * p.dp * p.dv, z, p.BH() * p.dp, p.stab,
                                        p.stab ? p.BH() : 0, static_cast<hipStream_t>(stream)));
}

la_status la_prefill_workspace_size(const la_desc* desc, size_t* bytes) {
  if (!bytes) return fail(LA_EINVAL, "bytes is NULL");
  la::Problem p;
  LA_TRY(check_desc(desc, true, &p));
  *bytes = p.path == 1 ? la::mfma_workspace_bytes(p) : 0;
  return LA_OK;
}

la_status la_prefill_plan(const la_desc* desc, int* chunk, int* segments, int* path) {
  la::Problem p;
  LA_TRY(check_desc(desc, true, &p));
  if (chunk) *chunk = p.path == 1 ? p.chunk : 1;
  if (segments) *segments = p.segments;
  if (path) *path = p.path;
  return LA_OK;
}

la_status la_prefill(const la_desc* desc, const void* q, const void* k, const void* v,
                     float* S, float* z, void* out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  la::Problem p;
  LA_TRY(check_prefill_args(desc, q, k, v, S, z, out, workspace, workspace_bytes, &p));
  (void)hipGetLastError();
  for (int stage = 1; stage <= 3; ++stage)
    LA_TRY(run_stage(p, stage, q, k, v, S, z, out, workspace, static_cast<hipStream_t>(stream)));
  return LA_OK;
}

la_status la_prefill_noalloc(const la_desc* desc, const void* q, const void* k, const void* v,
                             float* S, float* z, void* out, void* stream) {
  la::Problem p;
  LA_TRY(check_desc(desc, true, &p));
  LA_TRY(check_prefill_ptrs(p, q, k, v, S, z, out));
  const size_t need = p.path == 1 ? la::mfma_workspace_bytes(p) : 0;
  if (need > LA_NOALLOC_SCRATCH_BYTES)
    return fail(LA_EINVAL,
                "la_prefill_noalloc: this prefill needs %zu bytes of workspace, above the "
                "%zu-byte static scratch; use la_prefill with a caller workspace",
                need, size_t(LA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0 && p.T > 0) {
    const hipError_t e = la::noalloc_scratch(&ws);
    if (e != hipSuccess)
      return fail(LA_EHIP, "la_prefill_noalloc: scratch lookup failed: %s", hipGetErrorString(e));
  }
  (void)hipGetLastError();
  for (int stage = 1; stage <= 3; ++stage)
    LA_TRY(run_stage(p, stage, q, k, v, S, z, out, ws, static_cast<hipStream_t>(stream)));
  return LA_OK;
}

la_status la_prefill_stage(const la_desc* desc, int stage, const void* q, const void* k,
                           const void* v, float* S, float* z, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 3) return fail(LA_EINVAL, "stage must be 1, 2 or 3 (got %d)", stage);
  la::Problem p;
  LA_TRY(check_prefill_args(desc, q, k, v, S, z, out, workspace, workspace_bytes, &p));
  (void)hipGetLastError();
  return run_stage(p, stage, q, k, v, S, z, out, workspace, static_cast<hipStream_t>(stream));
}

la_status la_prefill_backward_workspace_size(const la_desc* desc, size_t* bytes) {
  if (!bytes) return fail(LA_EINVAL, "bytes is NULL");
  la::Problem p;
  LA_TRY(check_desc(desc, true, &p));
  *bytes = la::backward_workspace_bytes(p);
  return LA_OK;
}

la_status la_prefill_backward(const la_desc* desc, const void* q, const void* k, const void* v,
                              const float* S0, const float* z0, const void* dout, float* dq,
                              float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                              void* workspace, size_t workspace_bytes, void* stream) {
  la::Problem p;
  LA_TRY(check_desc(desc, true, &p));
  if (!la::backward_supported(p))
    return fail(LA_EUNSUPPORTED,
                "backward: needs a causal prefill with elu+1 or identity features, no decay, "
                "SSD decay or the RFA gate, and widths the per-token kernel takes");
  if ((S0 == nullptr) != (z0 == nullptr)) return fail(LA_EINVAL, "S0 and z0 go together");
  if ((dS0 == nullptr) != (dz0 == nullptr)) return fail(LA_EINVAL, "dS0 and dz0 go together");
  if (S0) {
    LA_TRY(check_ptr(S0, "S0"));
    LA_TRY(check_ptr(z0, "z0"));
  }
  if (dS0) {
    LA_TRY(check_ptr(dS0, "dS0"));
    LA_TRY(check_ptr(dz0, "dz0"));
  }
  if ((p.decay_kind != LA_DECAY_NONE) != (ddecay != nullptr))
    return fail(LA_EINVAL, "ddecay is required with a decay or gate, and only then");
  if (ddecay && !aligned(ddecay, 4)) return fail(LA_EINVAL, "ddecay must be 4-byte aligned");
  if (p.T > 0) {
    LA_TRY(check_ptr(q, "q"));
    LA_TRY(check_ptr(k, "k"));
    LA_TRY(check_ptr(v, "v"));
    LA_TRY(check_ptr(dout, "dout"));
    LA_TRY(check_ptr(dq, "dq"));
    LA_TRY(check_ptr(dk, "dk"));
    LA_TRY(check_ptr(dv, "dv"));
  }
  const size_t need = la::backward_workspace_bytes(p);
  if (need > 0) {
    if (!workspace) return fail(LA_EINVAL, "workspace is NULL (need %zu bytes)", need);
    if (!aligned(workspace, 16)) return fail(LA_EINVAL, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(LA_EINVAL, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                  need);
  }
  (void)hipGetLastError();
  return launched(la::launch_backward(p, q, k, v, S0, z0, dout, dq, dk, dv, ddecay, dS0, dz0,
                                      workspace, static_cast<hipStream_t>(stream)));
}

la_status la_decode_step(const la_desc* desc, const void* q, const void* k, const void* v,
                         float* S, float* z, void* out, void* stream) {
  la::Problem p;
  LA_TRY(check_desc(desc, false, &p));
  if (p.noncausal) return fail(LA_EINVAL, "decode is causal: noncausal must be 0");
  LA_TRY(check_ptr(q, "q"));
  LA_TRY(check_ptr(k, "k"));
  LA_TRY(check_ptr(v, "v"));
  LA_TRY(check_ptr(out, "out"));
  LA_TRY(check_ptr(S, "S"));
  LA_TRY(check_ptr(z, "z"));
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (la::decode_supported(p)) return launched(la::launch_decode(p, q, k, v, S, z, out, st));
  return launched(la::launch_recurrent(p, q, k, v, S, z, out, st));
}

const char* la_status_str(la_status status) {
  switch (status) {
    case LA_OK: return "LA_OK";
    case LA_EINVAL: return "LA_EINVAL";
    case LA_EUNSUPPORTED: return "LA_EUNSUPPORTED";
    case LA_EHIP: return "LA_EHIP";
  }
  return "LA_UNKNOWN";
}

const char* la_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
