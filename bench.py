"""Benchmark of the causal linear attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]      (defaults K = 200, W = 50)
                    [--chunk C] [--prefill-only] [--no-decode] [--no-cpu-baseline]

A step is one causal elu+1 prefill over the long-context workload
(B=1, H=8, T=102400, d_h = d' = d_v = 128, bf16 q, k, v ~ N(0, 1)/sqrt(2),
fp32 state, eps = 1e-6): la_state_init, then la_prefill (feature map,
chunking, intra-chunk MFMA contraction, chunk-local state contribution,
segment scan, inter-chunk read-out and normalisation).  Inputs are generated
on the device before timing.  W untimed warm-up steps are followed by exactly
K timed steps between two synchronisations, with HIP events on the stream the
library launches on.  The step time settles only after a few milliseconds of
back-to-back work (the clocks first dip, then recover), hence the defaults
of 50 warm-up and 200 timed steps (about 0.1 s of GPU time).

Printed as one JSON line:
  value        tokens/s (B*T tokens per step) over the K steps;
  roofline     the output kernel (la_prefill stage 3, the one that dominates),
               algorithmic bytes (q, k, v read + out written, bf16, plus the
               state) over its average duration, timed with events around
               that stage alone, against the 8 TB/s HBM peak; `traffic` is
               the HBM bytes per launch the counters measured (committed
               summary under profiles/), null once the kernel source changed;
  mfma         algorithmic FLOPs of the recurrence, 4 d' d_v + 4 d' per
               token-head, over the step time, against the 2.5 PFLOP/s bf16
               dense peak;
  decode       the gated random-feature decode workload (256 sequences x 16
               heads, d_h = d_v = 64, D = 64 sine/cosine pairs so d' = 128,
               fp32, 1024 one-token steps): state GB/s against 8 TB/s, and the
               same with 1024 sequences so the state (545 MB) exceeds the
               256 MB last-level cache;
  normaliser_free  the same prefill with the read-out phi(q)^T S alone;
  noncausal    the same prefill in the non-causal form;
  mlstm        the same shape with the mLSTM gates: identity features,
               sigmoid forget gate, exponential input gate (pre-activations
               N(3, 1) and N(0, 1), fp32), read-out divided by
               max(|q.z|, 1), stabilised state; algorithmic bytes add the
               two gate arrays;
  backward     la_prefill_backward (dq, dk, dv of L = sum <dout, out>) on the
               same long-context prefill, and on the elu+1 prefill shape
               B=4 H=8 T=2048 d=64, and on the SSD-decay shape B=2 H=16
               T=8192 d=128 with its decay: the chunked path (segment start states
               from the prefill's stages 1 and 2, a pass in token order for
               dq, a reverse scan of the segments' gradient states, a pass
               in reverse order for dk and dv), and on the mLSTM prefill
               above (dL/dfgate and dL/digate too); algorithmic bytes are q, k,
               v, dout read once (bf16) and dq, dk, dv written once (fp32);
  configs      the other prefill workloads, forward: the elu+1 prefill
               (B=4 H=8 T=2048 d=64) and the SSD-decay prefill (B=2 H=16
               T=8192 d=128, a = sigmoid(N(3, 1))), and the long-context one
               again, each timed per call (state zeroing + la_prefill) warm
               (back to back) and cold (a 1 GiB scrub written between calls,
               outside the timed region, so nothing of the inputs is left in
               the 256 MB last-level cache); median and minimum, algorithmic
               bytes (q, k, v read and out written once, the decay, the state
               read and written) and their fraction of the HBM peak;
  mfma_peak    a measured dense bf16 MFMA rate (libla_probe.so: every wave
               issues independent chains of v_mfma_f32_32x32x16_bf16, and of
               v_mfma_f32_16x16x32_bf16) beside the 2.5 PFLOP/s spec;
  mfma.executed  MFMA instructions per dispatch of the three prefill stages
               from the committed rocprofv3 counters (null once a kernel source
               changed) times their FLOPs, over the step time;
  cpu_baseline the fp64 oracle (the CPU reference the tests check against),
               on a bounded sample of the same prefill workload, one worker
               process per head.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published

# the long-context prefill workload
PF = dict(B=1, H=8, T=102400, d=128, scale=2.0 ** -0.5, eps=1e-6)
# the gated random-feature decode workload
DEC = dict(N=256, H=16, d_h=64, d_v=64, D=64, steps=1024)


# --------------------------------------------------------------------- CPU leg

_SAMPLE = None   # the oracle's inputs, made in the parent and inherited by the forked workers


def _oracle_head(h):
    """One head of the prefill sample through the fp64 oracle (worker process)."""
    from threadpoolctl import threadpool_limits
    from oracle import linattn_oracle as O
    x = _SAMPLE
    q, k, v = x.q[:, h:h + 1], x.k[:, h:h + 1], x.v[:, h:h + 1]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        O.causal_linear_attention(q, k, v, eps=PF["eps"])
        return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(T_sample: int):
    """Time the oracle on the first T_sample tokens of all H heads, one process
    per head (the heads are independent), before the GPU is touched.  Input
    generation is outside the timed region; the rate is taken over the slowest
    worker's oracle time."""
    global _SAMPLE
    import multiprocessing as mp
    from fixed_state_sequence_amd import inputs as I
    _SAMPLE = I.prefill_inputs(PF["B"], PF["H"], T_sample, PF["d"], dtype="bf16", seed=0,
                               scale=PF["scale"])
    workers = min(PF["H"], os.cpu_count() or 1)
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        per_head = pool.map(_oracle_head, range(PF["H"]))
    _SAMPLE = None
    wall = max(per_head) if workers >= PF["H"] else sum(per_head) / workers
    tokens = PF["B"] * T_sample
    return {
        "value": tokens / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
        "sample": (f"first {T_sample} of {PF['T']} tokens of the same workload, all {PF['H']} "
                   f"heads, fp64 numpy recurrence, one process per head with 1 BLAS thread; "
                   f"per-head oracle time {min(per_head):.2f}-{max(per_head):.2f} s; "
                   f"CPU {_cpu_model()}; "
                   f"{os.cpu_count()} host cores visible"),
    }


# ------------------------------------------------------ HBM traffic (counters)

TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "output_kernel_t102400_d128_hbm_traffic.txt")
# the sources the output kernel's device code is compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "fixed_state_sequence_amd", "csrc", f)
                  for f in ("la_prefill_mfma.hip", "la_mfma_common.h", "la_device.h")]


def kernel_source_sha256():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


MFMA_PROFILE = os.path.join(ROOT, "profiles", "prefill_t102400_d128_mfma_counters.txt")


def _profile_kv(path):
    """`key = value` lines of a committed counter summary, or None when the
    prefill kernels' sources no longer match the hash recorded there."""
    try:
        with open(path) as f:
            lines = f.read().splitlines()
        src = kernel_source_sha256()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if "=" in ln and not ln[:1].isspace():
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv if kv.get("source_sha256") == src else None


def profiled_mfma_insts():
    """MFMA instructions per dispatch of stages 1, 2 and 3 of the long-context
    prefill (SQ_INSTS_MFMA; every one a 32x32x16 bf16 MFMA), or None."""
    kv = _profile_kv(MFMA_PROFILE)
    if kv is None:
        return None
    try:
        return [float(kv[f"mfma_insts_stage{i}"]) for i in (1, 2, 3)]
    except (KeyError, ValueError):
        return None


def profiled_traffic():
    """HBM bytes per output-kernel launch, from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by what the counter
    reads for a streaming kernel of known size).  None when the kernel's
    source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = f.read().splitlines()
        src = kernel_source_sha256()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if "=" in ln and not ln[:1].isspace():
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != src or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


# --------------------------------------------------------------------- GPU leg

def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_prefill(torch, la, I, steps, warmup, normalize=True, stages=True, causal=True,
                  mlstm=False, chunk=0):
    dev = torch.device("cuda:0")
    B, H, T, d = PF["B"], PF["H"], PF["T"], PF["d"]
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=0, scale=PF["scale"], device=dev,
                         decay="mlstm" if mlstm else None)
    q, k, v = x.q, x.k, x.v
    stab = torch.empty(B, H, dtype=torch.float32, device=dev) if mlstm else None
    if mlstm:
        desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16, phi="identity", eps=PF["eps"],
                            normalize="max1", igate=x.igate, fgate=x.fgate, stab=stab,
                            chunk=chunk)
    else:
        desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16, eps=PF["eps"], normalize=normalize,
                            causal=causal, chunk=chunk)
    chunk, segments, path = la.prefill_plan(desc)
    if path != 1:
        raise RuntimeError("the long-context prefill did not take the chunked MFMA path")
    nws = la.prefill_workspace_size(desc)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    out = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    z = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    L = la._lib.lib()
    P = ctypes.c_void_p
    ptr = lambda t: P(t.data_ptr())
    stream = P(torch.cuda.current_stream(dev).cuda_stream)
    dref = ctypes.byref(desc)
    args = (ptr(q), ptr(k), ptr(v), ptr(S), ptr(z), ptr(out))

    def step():
        la._lib.check(L.la_state_init(dref, ptr(S), ptr(z), stream))
        la._lib.check(L.la_prefill(dref, *args, ptr(ws), nws, stream))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    if not stages:
        return dict(ms=ms, wall=wall, chunk=chunk, segments=segments)

    # per-stage durations: the same calls back to back (no synchronisation
    # between repetitions, so the clocks stay where the timed steps had them),
    # with events between the stages
    reps = max(steps, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps):
        L.la_state_init(dref, ptr(S), ptr(z), stream)
        evs[r][0].record()
        for s in (1, 2, 3):
            la._lib.check(L.la_prefill_stage(dref, s, *args, ptr(ws), nws, stream))
            evs[r][s].record()
    torch.cuda.synchronize()
    stage_ms = [sum(evs[r][s].elapsed_time(evs[r][s + 1]) for r in range(reps)) / reps
                for s in range(3)]
    # per-repetition totals of the three stages: median and minimum
    per = sorted(evs[r][0].elapsed_time(evs[r][3]) for r in range(reps))
    return dict(ms=ms, wall=wall, stage_ms=stage_ms, chunk=chunk, segments=segments,
                rep_median_ms=per[len(per) // 2], rep_min_ms=per[0])


def bench_backward(torch, la, I, B, H, T, d, reps, decay=None, scale=PF["scale"]):
    """ms per la_prefill_backward call (bf16 inputs and dout): elu+1 with no
    decay or the SSD decay a = sigmoid(N(3, 1)); or decay="mlstm", identity
    features with the mLSTM gates (the prefill's mLSTM workload) and the
    max(|q.z|, 1) read-out."""
    dev = torch.device("cuda:0")
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=0, scale=scale, device=dev,
                         decay=decay)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    do = torch.randn(B, H, T, d, generator=g, device=dev).to(torch.bfloat16)
    if decay == "mlstm":
        stab = torch.zeros(B, H, dtype=torch.float32, device=dev)
        desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16, phi="identity", normalize="max1",
                            igate=x.igate, fgate=x.fgate, stab=stab)
        kw = dict(phi="identity", normalize="max1", igate=x.igate, fgate=x.fgate)
    else:
        desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16, decay=x.decay)
        kw = dict(decay=x.decay)
    n = ctypes.c_size_t(0)
    la._lib.check(la._lib.lib().la_prefill_backward_workspace_size(ctypes.byref(desc),
                                                                   ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=dev)
    for _ in range(3):                                 # warm-up
        la.prefill_backward(x.q, x.k, x.v, do, workspace=ws, **kw)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        la.prefill_backward(x.q, x.k, x.v, do, workspace=ws, **kw)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # algorithmic bytes: q, k, v, dout read (bf16), dq, dk, dv written (fp32)
    nbytes = B * H * T * d * (4 * 2 + 3 * 4)
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), GBs=nbytes / (ms * 1e-3) / 1e9,
                algorithmic_bytes=nbytes)


def bench_config(torch, la, I, name, reps=25, warmup=5, scrub_bytes=1 << 30, chunk=0,
                 segments=0):
    """One forward prefill workload, per call (state zeroing + la_prefill):
    warm (calls back to back) and cold (a scrub buffer larger than the
    last-level cache written before every call, outside the events)."""
    dev = torch.device("cuda:0")
    x = I.workload_inputs(name, seed=0, device=dev)
    B, H, T, d = x.q.shape
    dv = x.v.shape[-1]
    desc = la.make_desc(B, H, T, d, dv, la._lib.LA_BF16, eps=PF["eps"], decay=x.decay,
                        chunk=chunk, segments=segments)
    chunk, segments, path = la.prefill_plan(desc)
    nws = la.prefill_workspace_size(desc)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    out = torch.empty(B, H, T, dv, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, d, dv, dtype=torch.float32, device=dev)
    z = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    scrub = torch.empty(scrub_bytes // 4, dtype=torch.float32, device=dev)
    L = la._lib.lib()
    P = ctypes.c_void_p
    ptr = lambda t: P(t.data_ptr())
    stream = P(torch.cuda.current_stream(dev).cuda_stream)
    dref = ctypes.byref(desc)
    args = (ptr(x.q), ptr(x.k), ptr(x.v), ptr(S), ptr(z), ptr(out))

    def call():
        la._lib.check(L.la_state_init(dref, ptr(S), ptr(z), stream))
        la._lib.check(L.la_prefill(dref, *args, ptr(ws), nws, stream))

    def timed(cold):
        evs = [_events(torch) for _ in range(reps)]
        for r in range(reps):
            if cold:
                scrub.fill_(float(r))
            evs[r][0].record()
            call()
            evs[r][1].record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    warm = timed(False)
    cold = timed(True)
    TH = B * H * T
    nbytes = TH * (2 * d + 2 * dv) * 2      # q, k, v read and out written, bf16
    nbytes += 2 * B * H * (d * dv + d) * 4 + (TH * 4 if x.decay is not None else 0)
    res = {"B": B, "H": H, "T": T, "d": d, "decay": "ssd" if x.decay is not None else None,
           "chunk": chunk, "segments": segments, "algorithmic_bytes": nbytes, "reps": reps}
    for tag, ts in (("warm", warm), ("cold", cold)):
        med = ts[len(ts) // 2]
        res[tag] = {"median_ms": med, "min_ms": ts[0], "tokens_per_s": B * T / (med * 1e-3),
                    "GBs": nbytes / (med * 1e-3) / 1e9,
                    "hbm_frac": nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


# libla_probe.so shapes: (id, MFMA, independent accumulator chains per wave, FLOPs per MFMA)
PROBE_SHAPES = ((0, "32x32x16", 4, 32768), (2, "32x32x16", 2, 32768), (1, "16x16x32", 8, 16384),
                (3, "16x16x32", 16, 16384))


def _probe_lib():
    from fixed_state_sequence_amd import build as B_
    if not os.path.exists(B_.PROBE_LIB_PATH):
        return None
    lib = ctypes.CDLL(B_.PROBE_LIB_PATH)
    lib.la_probe_mfma.restype = ctypes.c_int
    lib.la_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    return lib


def _probe_rate(torch, lib, shape, nblocks, iters, reps):
    """TFLOP/s of one probe configuration (events around `reps` launches)."""
    dev = torch.device("cuda:0")
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _, _, ch, per = next(p for p in PROBE_SHAPES if p[0] == shape)
    call = lambda: lib.la_probe_mfma(shape, nblocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                     stream)
    if call() != 0:
        return None
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return nblocks * 4 * ch * iters * per / (ms * 1e-3) / 1e12


def mfma_peak(torch, nblocks=512, iters=32768, reps=5):
    """Measured dense bf16 MFMA rate (TFLOP/s) of libla_probe.so's loops, two
    workgroups of 4 waves per compute unit, a few milliseconds per launch:
    v_mfma_f32_32x32x16_bf16 with 4 independent chains per wave, and
    v_mfma_f32_16x16x32_bf16 with 16 (it needs about twice the chains, and
    accumulator registers, to approach the same rate)."""
    lib = _probe_lib()
    if lib is None:
        return None
    r32 = _probe_rate(torch, lib, 0, nblocks, iters, reps)
    r16 = _probe_rate(torch, lib, 3, nblocks, iters, reps)
    if r32 is None or r16 is None:
        return None
    return {"unit": "TFLOP/s", "bf16_32x32x16": r32, "bf16_16x16x32": r16,
            "spec": BF16_PEAK_TFLOPS,
            "loop": f"{nblocks} workgroups x 4 waves, operands in registers, {iters} MFMAs per "
                    f"chain; 4 chains per wave (32x32x16), 16 (16x16x32)"}


def mfma_sweep(torch):
    """Every probe shape and chain count over 1 to 16 workgroups per compute
    unit (printed, one line each)."""
    lib = _probe_lib()
    for shape, name, ch, _ in PROBE_SHAPES:
        for nb in (256, 512, 1024, 2048, 4096):
            r = _probe_rate(torch, lib, shape, nb, 16384 * 1024 // nb, 5)
            print(f"v_mfma_f32_{name}_bf16, {ch} chains per wave, {nb} workgroups of 4 waves: "
                  f"{r:.0f} TFLOP/s", flush=True)


def issue_probe(torch, nblocks=256, mf_iters=20000, va_iters=10000, reps=5):
    """libla_probe.so's issue-overlap probe (one 8-wave workgroup per compute
    unit, waves w and w + 4 on one SIMD): ms per launch of MFMA waves alone
    (2 chains x mf_iters v_mfma_f32_32x32x16_bf16 each), one VALU wave per
    SIMD (32 chains x va_iters fp32 FMAs), two VALU waves per SIMD (twice the
    VALU work), and one MFMA plus one VALU wave per SIMD (printed)."""
    lib = _probe_lib()
    if lib is None:
        print("libla_probe.so is not built", flush=True)
        return None
    lib.la_probe_issue.restype = ctypes.c_int
    lib.la_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    sink = torch.empty(nblocks * 512, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ms = {}
    for mode in (0, 1, 2, 3):
        call = lambda: lib.la_probe_issue(mode, nblocks, mf_iters, va_iters,
                                          ctypes.c_void_p(sink.data_ptr()), stream)
        if call() != 0:
            return None
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms[mode] = e0.elapsed_time(e1) / reps
    print(f"MFMA waves alone (one per SIMD, {2 * mf_iters} MFMAs each): {ms[0]:.3f} ms", flush=True)
    print(f"one VALU wave per SIMD ({32 * va_iters} FMAs each): {ms[1]:.3f} ms", flush=True)
    print(f"two VALU waves per SIMD (twice the work): {ms[2]:.3f} ms = {ms[2] / ms[1]:.2f} x one wave's",
          flush=True)
    print(f"one MFMA and one VALU wave per SIMD: {ms[3]:.3f} ms = {ms[3] / ms[1]:.2f} x the VALU wave "
          f"alone, {ms[3] / (ms[0] + ms[1]):.2f} x the two alone in turn", flush=True)
    return ms


def hbm_copy(torch, nbytes=1 << 30, reps=10):
    """Device-to-device streaming of `nbytes` (read + write) by two kernels,
    torch's copy and its vectorised negation (16 bytes per lane, like the
    path's kernels): the faster is the achievable HBM bandwidth this box
    shows for plain streaming, the reference beside the 8 TB/s spec.  The
    negation is also the known-size kernel the traffic counters are scaled
    by."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = None
    for name, fn in (("copy", lambda: dst.copy_(src)), ("neg", lambda: torch.neg(src, out=dst))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = dict(bytes=2 * nbytes, ms=ms, gbs=gbs, kernel=name)
    return best


def bench_decode(torch, la, I, N, steps, warmup=64):
    """`steps` one-token steps for N sequences; inputs for every step are made
    on the device beforehand.  Returns ms per step."""
    dev = torch.device("cuda:0")
    H, d_h, d_v, D = DEC["H"], DEC["d_h"], DEC["d_v"], DEC["D"]
    dp = 2 * D
    W = I.rff_projection(H, D, d_h, seed=0, device=dev)
    nin = steps   # a distinct input set for every timed step
    x = I.rfa_decode_batch(nin, N, H, d_h, d_v, seed=1, device=dev)
    q, k, v, gate = x.q, x.k, x.v, x.gate
    S, z = la.state_init(N, H, dp, d_v, dev)
    out = torch.empty(N, H, d_v, dtype=torch.float32, device=dev)
    desc = la.make_desc(N, H, 1, d_h, d_v, la._lib.LA_F32, phi="rff", W=W, gate=gate[0],
                        eps=1e-6)
    L = la._lib.lib()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(dev).cuda_stream)
    dref = ctypes.byref(desc)
    qp = [P(q[i].data_ptr()) for i in range(nin)]
    kp = [P(k[i].data_ptr()) for i in range(nin)]
    vp = [P(v[i].data_ptr()) for i in range(nin)]
    gp = [gate[i].data_ptr() for i in range(nin)]
    Sp, zp, op = P(S.data_ptr()), P(z.data_ptr()), P(out.data_ptr())

    def run(n):
        for t in range(n):
            i = t % nin
            desc.decay = gp[i]
            rc = L.la_decode_step(dref, qp[i], kp[i], vp[i], Sp, zp, op, stream)
            if rc:
                la._lib.check(rc)

    run(warmup)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    state_b = N * H * (dp * d_v + dp) * 4
    io_b = N * H * (2 * d_h + 2 * d_v + 1) * 4 + H * D * d_h * 4
    bytes_step = 2 * state_b + io_b
    return dict(ms_per_step=ms, bytes_per_step=bytes_step, gbs=bytes_step / (ms * 1e-3) / 1e9,
                state_mb=state_b / 1e6)


def executed_mfma(pf, peak):
    """Executed MFMA work of the prefill step from the committed counters:
    per stage and in total, as TFLOP/s over the measured stage and step times
    and as fractions of the spec and the measured 32x32x16 peak."""
    insts = profiled_mfma_insts()
    if insts is None:
        return None
    per = 2 * 32 * 32 * 16              # FLOPs of one v_mfma_f32_32x32x16_bf16
    st = pf["stage_ms"]
    stages = [n * per / (ms * 1e-3) / 1e12 if ms > 0 else 0.0 for n, ms in zip(insts, st)]
    total = sum(insts) * per / (pf["ms"] * 1e-3) / 1e12
    meas = peak["bf16_32x32x16"] if peak else None
    return {"flops_per_step": sum(insts) * per, "stage_TFLOPs": stages, "achieved": total,
            "frac": total / BF16_PEAK_TFLOPS, "frac_of_measured": total / meas if meas else None,
            "stage3_frac": stages[2] / BF16_PEAK_TFLOPS}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=102400,
                    help="tokens per head in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--chunk", type=int, default=0,
                    help="prefill chunk length (0: the library's default plan)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the long-context prefill alone (no variants, backward, decode)")
    ap.add_argument("--issue-probe", action="store_true",
                    help="time the VALU/MFMA issue-overlap probe (libla_probe.so) and exit")
    ap.add_argument("--mfma-sweep", action="store_true",
                    help="only sweep the MFMA peak probe (shapes, chains, workgroups) and exit")
    ap.add_argument("--config", default=None,
                    help="only time this forward prefill workload (inputs.WORKLOADS name), with "
                         "--chunk and --segments, warm and cold, and print its line")
    ap.add_argument("--segments", type=int, default=0,
                    help="segments per sequence for --config (0: the library's default plan)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the path needs no second GPU; heads and sequences shard with no exchange)",
              file=sys.stderr)
        return 2

    cpu = None
    if not (a.no_cpu_baseline or a.prefill_only or a.config or a.mfma_sweep or a.issue_probe):
        print(f"[bench] cpu baseline: oracle on {a.cpu_tokens} tokens x {PF['H']} heads",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(a.cpu_tokens)

    import torch
    import fixed_state_sequence_amd as la
    from fixed_state_sequence_amd import inputs as I
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    la._lib.lib()
    if a.issue_probe:
        issue_probe(torch)
        return 0
    if a.mfma_sweep:
        mfma_sweep(torch)
        return 0
    if a.config:
        line = bench_config(torch, la, I, a.config, reps=max(a.steps, 5), warmup=a.warmup,
                            chunk=a.chunk, segments=a.segments)
        print(json.dumps({"config": a.config, **line}), flush=True)
        return 0

    print(f"[bench] prefill B={PF['B']} H={PF['H']} T={PF['T']} d={PF['d']}: "
          f"{a.warmup} warm-up + {a.steps} timed steps", file=sys.stderr, flush=True)
    pf = bench_prefill(torch, la, I, a.steps, a.warmup, chunk=a.chunk)
    B, H, T, d = PF["B"], PF["H"], PF["T"], PF["d"]
    TH = B * H * T
    tokens_per_s = B * T / (pf["ms"] * 1e-3)
    state_bytes = B * H * (d * d + d) * 4
    stage3_bytes = TH * 4 * d * 2 + 2 * state_bytes      # q, k, v in, out out (bf16); state
    s3 = pf["stage_ms"][2]
    achieved = stage3_bytes / (s3 * 1e-3) / 1e9
    flops = TH * (4 * d * d + 4 * d)
    tflops = flops / (pf["ms"] * 1e-3) / 1e12
    step_bytes = TH * 4 * d * 2 + 2 * state_bytes

    cp = hbm_copy(torch)
    peak = mfma_peak(torch)
    configs = None
    if not a.prefill_only:
        print("[bench] forward configs, warm and cold", file=sys.stderr, flush=True)
        configs = {n: bench_config(torch, la, I, n) for n in
                   ("elu_prefill_b4_h8_t2048_d64", "ssd_prefill_b2_h16_t8192_d128",
                    "long_prefill_b1_h8_t102400_d128")}
    dec = dec_big = None
    if a.prefill_only:
        extras = None
    else:
        print("[bench] prefill, normaliser-free read-out", file=sys.stderr, flush=True)
        pf_nn = bench_prefill(torch, la, I, a.steps, a.warmup, normalize=False, stages=False,
                              chunk=a.chunk)
        print("[bench] prefill, non-causal form", file=sys.stderr, flush=True)
        pf_nc = bench_prefill(torch, la, I, a.steps, a.warmup, stages=False, causal=False,
                              chunk=a.chunk)
        print("[bench] prefill, mLSTM gates", file=sys.stderr, flush=True)
        pf_ml = bench_prefill(torch, la, I, a.steps, a.warmup, mlstm=True, chunk=a.chunk)
        ml_bytes = step_bytes + TH * 2 * 4 + 2 * B * H * 4     # + the two gates, the stabiliser
        print("[bench] backward", file=sys.stderr, flush=True)
        bw_long = bench_backward(torch, la, I, B, H, T, d, 20)
        bw_small = bench_backward(torch, la, I, 4, 8, 2048, 64, 50)
        bw_ssd = bench_backward(torch, la, I, 2, 16, 8192, 128, 20, decay="ssd", scale=1.0)
        bw_ml = bench_backward(torch, la, I, B, H, T, d, 20, decay="mlstm")
        extras = True
    if not a.no_decode and not a.prefill_only:
        print(f"[bench] decode {DEC['N']} x {DEC['H']}, {DEC['steps']} steps", file=sys.stderr,
              flush=True)
        dec = bench_decode(torch, la, I, DEC["N"], DEC["steps"])
        print("[bench] decode 1024 x 16, 256 steps", file=sys.stderr, flush=True)
        dec_big = bench_decode(torch, la, I, 1024, 256)

    res = {
        "metric": "linear-attn fwd tokens/s + % MFMA peak at T=100K,d=128; decode state GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long-context causal elu+1 prefill", "B": B, "H": H, "T": T,
                   "d_h": d, "d_prime": d, "d_v": d, "in_dtype": "bf16", "out_dtype": "bf16",
                   "state_dtype": "fp32", "eps": PF["eps"], "decay": None,
                   "chunk": pf["chunk"], "segments": pf["segments"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "path_frac": step_bytes / (pf["rep_median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": profiled_traffic() if pf["chunk"] == 32 else None,
                     "kernel": "output_kernel (la_prefill stage 3)",
                     "kernel_ms": s3, "algorithmic_bytes": stage3_bytes,
                     "measured_copy_GBs": cp["gbs"], "copy_kernel": cp["kernel"],
                     "frac_of_copy": achieved / cp["gbs"]},
        "step": {"stage_ms": pf["stage_ms"], "prefill_median_ms": pf["rep_median_ms"],
                 "prefill_min_ms": pf["rep_min_ms"], "algorithmic_bytes": step_bytes,
                 "GBs": step_bytes / (pf["ms"] * 1e-3) / 1e9,
                 "hbm_frac": step_bytes / (pf["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "mfma": {"algorithmic_flops": flops, "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                 "executed": executed_mfma(pf, peak)},
        "mfma_peak": peak,
        "cpu_baseline": cpu,
    }
    if configs is not None:
        res["configs"] = configs
    if extras:
        res.update({
            "normaliser_free": {
                "workload": "the same prefill, read-out phi(q)^T S without the normaliser",
                "ms_per_step": pf_nn["ms"], "tokens_per_s": B * T / (pf_nn["ms"] * 1e-3),
                "GBs": step_bytes / (pf_nn["ms"] * 1e-3) / 1e9,
                "hbm_frac": step_bytes / (pf_nn["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "noncausal": {
                "workload": "the same prefill in the non-causal form: the whole sequence into "
                            "the state, then every token reads it out",
                "ms_per_step": pf_nc["ms"], "tokens_per_s": B * T / (pf_nc["ms"] * 1e-3),
                "GBs": step_bytes / (pf_nc["ms"] * 1e-3) / 1e9,
                "hbm_frac": step_bytes / (pf_nc["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "mlstm": {
                "workload": "the same shape with the mLSTM gates: identity features, sigmoid "
                            "forget and exponential input gates (fp32 pre-activations), "
                            "max(|q.z|, 1) read-out, stabilised state",
                "ms_per_step": pf_ml["ms"], "tokens_per_s": B * T / (pf_ml["ms"] * 1e-3),
                "stage_ms": pf_ml["stage_ms"], "algorithmic_bytes": ml_bytes,
                "GBs": ml_bytes / (pf_ml["ms"] * 1e-3) / 1e9,
                "hbm_frac": ml_bytes / (pf_ml["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "stage3_GBs": (stage3_bytes + TH * 2 * 4) / (pf_ml["stage_ms"][2] * 1e-3) / 1e9},
            "backward": {
                "workload": "la_prefill_backward, elu+1, bf16 q, k, v, dout; fp32 dq, dk, dv (and "
                            "dL/da with the SSD decay); chunked: prefill stages 1-2, dq pass, reverse "
                            "scan, dk/dv pass (with a decay, a suffix-sum pass for dL/da)",
                "algorithmic_bytes_per_token_head": 4 * 2 * d + 3 * 4 * d,
                "long_context": {"B": B, "H": H, "T": T, "d": d, "ms": bw_long["ms"],
                                 "tokens_per_s": bw_long["tokens_per_s"],
                                 "GBs": bw_long["GBs"],
                                 "hbm_frac": bw_long["GBs"] / HBM_PEAK_GBS},
                "elu_prefill_shape": {"B": 4, "H": 8, "T": 2048, "d": 64, "ms": bw_small["ms"],
                                      "tokens_per_s": bw_small["tokens_per_s"],
                                      "GBs": bw_small["GBs"]},
                "ssd_prefill_shape": {"B": 2, "H": 16, "T": 8192, "d": 128, "decay": "ssd",
                                      "ms": bw_ssd["ms"], "tokens_per_s": bw_ssd["tokens_per_s"],
                                      "GBs": bw_ssd["GBs"]},
                "mlstm_long_context": {"B": B, "H": H, "T": T, "d": d, "gates": "mlstm",
                                       "ms": bw_ml["ms"], "tokens_per_s": bw_ml["tokens_per_s"],
                                       "GBs": bw_ml["GBs"]}},
        })
    if dec is not None:
        res["decode"] = {
            "workload": "gated random-feature decode, fp32, D=64 pairs, d'=128, d_v=64",
            "sequences": DEC["N"], "heads": DEC["H"], "steps": DEC["steps"],
            "ms_per_step": dec["ms_per_step"], "bytes_per_step": dec["bytes_per_step"],
            "achieved": dec["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec["gbs"] / HBM_PEAK_GBS, "state_MB": dec["state_mb"],
            "frac_of_copy": dec["gbs"] / cp["gbs"],
            "note": ("the 136 MB state fits the 256 MB last-level cache and stays there "
                     "between the back-to-back steps (normal loads and stores); 'large' is the "
                     "same step on a state set that streams from HBM every step"),
            "large": {"sequences": 1024, "steps": 256, "ms_per_step": dec_big["ms_per_step"],
                      "achieved": dec_big["gbs"], "frac": dec_big["gbs"] / HBM_PEAK_GBS,
                      "frac_of_copy": dec_big["gbs"] / cp["gbs"],
                      "state_MB": dec_big["state_mb"], "accesses": "streamed (non-temporal)"},
        }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
