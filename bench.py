"""Benchmark of the MLA prolog hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = one full mla_prolog_v2 call (down projection, RmsNorms, c^KV /
k^R cache scatter, up projection with RoPE, per-head W^UK product) over one
batch of seeded synthetic tokens.  The headline workload is DeepSeek-V3-
shaped decode, T = 32 tokens (bf16).  Inputs are resident in HBM before the
timed region; steps rotate over several independent copies of weights,
activations, caches and outputs so the working set exceeds the 256 MB
last-level cache and bytes really come from HBM.  The timed decode steps
are a HIP-graph replay of prepared calls (how decode steps are served: no
host launch gaps); an eager pass over the same steps records per-kernel
phase events.

Prints ONE JSON line.  Besides the headline value it carries:
* roofline - the dominant kernel (the c^Q . [W^UQ | W^QR] up projection),
  its algorithmic bytes over its average duration, measured with HIP events
  the library records on the launch stream between its kernels;
* step_roofline - the whole call's algorithmic bytes over the step time;
* prefill - the same prolog at T = 4096 (bf16 MFMA-bound);
* qkv_rmsnorm_rope_cache - the fused qkv op on its (B=64, S=128) workload;
* preprocess_decode - MlaPreprocessV2 at the DeepSeek-V3 dims (32 heads),
  decode T = 32;
* cpu_baseline - the float64 NumPy oracle timed on this host on a bounded
  sample of the decode workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
DECODE_TARGET_FRAC = 0.60      # decode T=32: fraction of HBM peak on bytes moved
PREFILL_TARGET_FRAC = 0.50     # prefill T=4096: fraction of bf16 MFMA peak
METRIC = ("MLA-prolog tokens/s at decode T=32 & prefill T=4096; "
          "%HBM BW / %MFMA peak")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=12,
                    help="independent input sets cycled by the decode steps")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-qkv", action="store_true")
    ap.add_argument("--no-full-quant", action="store_true")
    ap.add_argument("--no-partial-quant", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--no-preprocess", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm single-input-set decode line")
    ap.add_argument("--regions", type=int, default=5,
                    help="separately timed regions of --steps calls each "
                         "(the value is their median)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="first run a plain device copy of MB megabytes "
                         "(a known-size reference for HBM traffic counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (bytes / flops the method must move / do per call)
# ---------------------------------------------------------------------------

def mla_bytes(c, wb_uq=2, cache_b=2):
    T = c.T
    weights = (c.He * c.Hcq + c.He * (c.Hckv + c.Dr)) * 2 \
        + c.Hcq * c.N * (c.D + c.Dr) * wb_uq + c.N * c.D * c.Hckv * 2
    gammas = (c.Hcq + c.Hckv) * 2
    per_tok = (c.He * 2 + 2 * c.Dr * 2 + 8 + c.N * c.Hckv * 2
               + c.N * c.Dr * 2 + (c.Hckv + c.Dr) * cache_b)
    return weights + gammas + T * per_tok


def mla_partial_bytes(c):
    """Partial quantisation with int8 caches: bf16 x and down-projection
    weights, int8 W^UQ_QR, bf16 W^UK, fp32 scales; bf16 query and query_rope,
    int8 kv / kr cache rows."""
    T = c.T
    weights = c.He * (c.Hcq + c.Hckv + c.Dr) * 2 + c.Hcq * c.N * (c.D + c.Dr) \
        + c.N * c.D * c.Hckv * 2
    scales = (c.N * (c.D + c.Dr) + c.Hcq + c.Hckv + c.Dr) * 4 \
        + (c.Hcq + c.Hckv) * 2
    per_tok = (c.He * 2 + 2 * c.Dr * 2 + 8 + c.N * c.Hckv * 2
               + c.N * c.Dr * 2 + c.Hckv + c.Dr)
    return weights + scales + T * per_tok


def mla_full_bytes(c):
    """Full quantisation with the int8 kv_cache: int8 x, down-projection
    and up-projection weights, bf16 W^UK, fp32 scales; int8 query with a
    per-(token, head) scale, bf16 query_rope and kr_cache, int8 kv_cache."""
    T = c.T
    weights = c.He * (c.Hcq + c.Hckv + c.Dr) + c.Hcq * c.N * (c.D + c.Dr) \
        + c.N * c.D * c.Hckv * 2
    scales = (c.Hcq + (c.Hckv + c.Dr) + c.N * (c.D + c.Dr) + c.Hcq
              + c.Hckv) * 4 + (c.Hcq + c.Hckv) * 2
    per_tok = (c.He + 4 + 2 * c.Dr * 2 + 8 + c.N * c.Hckv + c.N * 4
               + c.N * c.Dr * 2 + c.Hckv + c.Dr * 2)
    return weights + scales + T * per_tok


def mla_flops(c):
    return 2 * c.T * (c.He * (c.Hcq + c.Hckv + c.Dr)
                      + c.Hcq * c.N * (c.D + c.Dr) + c.N * c.D * c.Hckv)


def uqqr_bytes(c):
    """Algorithmic bytes of the up-projection launch: its share of the
    call's algorithmic bytes (W^UQ_QR, the cos/sin rows its RoPE reads, the
    query_rope rows it writes).  c^Q in and q^C out are workspace traffic
    between the library's own kernels, counted in uqqr_workspace_bytes."""
    return c.Hcq * c.N * (c.D + c.Dr) * 2 + c.T * (
        2 * c.Dr * 2 + c.N * c.Dr * 2)


def uqqr_workspace_bytes(c, merged=False):
    """Workspace bytes the up-projection launch also moves: c^Q (bf16) in,
    q^C (bf16) out, and with the W^UK product in the same launch q^C read
    back once per 128-column W^UK tile of each head."""
    back = (c.Hckv + 127) // 128 * c.T * c.N * c.D * 2 if merged else 0
    return c.T * (c.Hcq * 2 + c.N * c.D * 2) + back


def uk_bytes(c):
    """Algorithmic bytes of the W^UK product: W^UK in, the query out."""
    return c.N * c.D * c.Hckv * 2 + c.T * c.N * c.Hckv * 2


def uqqr_flops(c):
    return 2 * c.T * c.Hcq * c.N * (c.D + c.Dr)


def uk_flops(c):
    return 2 * c.T * c.N * c.D * c.Hckv


def preprocess_bytes(c):
    """MlaPreprocessV2 algorithmic bytes: bf16 x, gammas, W^UK, cos/sin,
    outputs and cache rows; int8 W^DQKV and W^UQ_QR; fp32 biases, dequant
    scales and the two quant scales; int64 index."""
    ntot = c.Hcq + c.Hckv + c.Dr
    nuq = c.N * (c.D + c.Dr)
    weights = c.He * ntot + c.Hcq * nuq + c.N * c.D * c.Hckv * 2
    params = (c.He + c.Hcq + c.Hckv) * 2 + (c.He + c.Hcq + ntot + nuq + 2) * 4
    per_tok = (c.He * 2 + 2 * c.Dr * 2 + 8 + c.N * c.Hckv * 2
               + c.N * c.Dr * 2 + (c.Hckv + c.Dr) * 2)
    return weights + params + c.T * per_tok


def qkv_bytes(c, n_valid):
    T = c.T
    return T * ((c.Nq + c.Nk + c.Nv) * c.D * 2 + 2 * c.D * 2 + 8
                + c.Nq * c.D * 2) + n_valid * (c.Nk + c.Nv) * c.D \
        + 2 * c.D * 2 + (c.Nk + c.Nv) * c.D * 4


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel, as measured by the rocprofv3 counter
# runs recorded under profiles/ (FETCH_SIZE and WRITE_SIZE, scaled by the
# counters of a plain copy of known size).  Reported only while the kernel
# source still hashes to what was profiled; otherwise null.

TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                            "profiles", "mla_decode_up_uk_hbm_traffic.md")
KERNEL_SOURCES = ("qkv_norm_rope_amd/csrc/mla_prolog_v2.hip",
                  "qkv_norm_rope_amd/csrc/device_common.h",
                  "qkv_norm_rope_amd/csrc/mla_device.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """(bytes per launch, source hash) from the traffic summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        for key in ("traffic_bytes_per_launch", "source_sha256"):
            if line.strip().startswith(key + " ="):
                vals[key] = line.split("=", 1)[1].strip()
    if len(vals) != 2:
        return None
    return float(vals["traffic_bytes_per_launch"]), vals["source_sha256"]


def calibrate_copy(torch, mb):
    n = mb * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# scale tensors of the quantised scenarios, passed by name when present
MLA_SCALES = ("dequant_scale_w_uq_qr", "smooth_scales_cq", "quant_scale_ckv",
              "quant_scale_ckr", "dequant_scale_x", "dequant_scale_w_dq",
              "dequant_scale_w_dkv_kr", "dequant_scale_q_nope")


def prepare_mla_sets(w, n_sets, torch, qn, gh):
    """Upload one seeded workload, pack its weights, and clone it n_sets-1
    times into distinct allocations."""
    cfg = w.cfg
    d = gh.upload(w)
    base = {
        "token_x": d["token_x"].view(cfg.B, cfg.S, cfg.He),
        "weight_dq": qn.mla_pack_weight(d["weight_dq"]),
        "weight_dkv_kr": qn.mla_pack_weight(d["weight_dkv_kr"]),
        "weight_uq_qr": qn.mla_pack_weight_uq_qr(d["weight_uq_qr"], cfg.N,
                                                 cfg.D, cfg.Dr),
        "weight_uk": qn.mla_pack_weight_uk(d["weight_uk"]),
    }
    for k in ("rmsnorm_gamma_cq", "rmsnorm_gamma_ckv", "rope_sin", "rope_cos",
              "cache_index", "kv_cache", "kr_cache") + MLA_SCALES:
        if k in d:
            base[k] = d[k]
    sets = [base]
    for _ in range(1, n_sets):
        sets.append({k: v.clone() for k, v in base.items()})
    q8 = cfg.quant_mode == "full_kv_int8"
    for s in sets:
        s["query"] = torch.empty((cfg.B, cfg.S, cfg.N, cfg.Hckv),
                                 dtype=torch.int8 if q8 else torch.bfloat16,
                                 device="cuda")
        s["query_rope"] = torch.empty((cfg.B, cfg.S, cfg.N, cfg.Dr),
                                      dtype=torch.bfloat16, device="cuda")
        if q8:
            s["dequant_scale_q_nope"] = torch.empty(
                (cfg.B, cfg.S, cfg.N, 1), dtype=torch.float32, device="cuda")
    return sets


class HipEvents:
    """Timing events created with a device-scope release (no L2 writeback at
    each record), through the HIP runtime torch already loaded."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [
            ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [
            ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    class Event:
        def __init__(self, handle):
            self.cuda_event = handle

    def create(self, flags=None):
        h = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(
            self.ct.byref(h), self.RELEASE_TO_DEVICE if flags is None else flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return self.Event(h.value)

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev.cuda_event, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a.cuda_event,
                                        b.cuda_event) != 0:
            self.hip.hipGetLastError()  # do not leave the error to torch
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev.cuda_event)


def _hold_gpu(torch, ms=20.0):
    """Keep the GPU busy for ~ms so the host can enqueue the whole timed
    region before it starts (no host launch gaps inside it)."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def _spread(ms_list):
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return med, xs[0], xs[-1]


def run_mla(cfg, sets, steps, warmup, torch, qn, graph=True, regions=5):
    """Time `steps` calls cycling over the sets, in `regions` separately
    timed regions of exactly `steps` calls each.

    Returns a dict: ms (median ms per call over the regions), ms_min,
    ms_max, regions, steps; phase_ms and kernel_ms (per-call averages from
    an instrumented eager region of the same `steps` calls: the library's
    phase events between its launches and each main kernel's own start/stop
    events, read only for the kernels the library reports it launches);
    ms_eager (that region's ms per call).  The timed regions are HIP-graph
    replays of one graph holding the `steps` calls (graph=True), or eager
    launches of them (graph=False), each bracketed by a device
    synchronisation on both sides.
    """
    nph = len(qn.MLA_PHASES)
    nk = len(qn.MLA_KERNELS)
    kw = dict(quant_mode=cfg.quant_mode, rmsnorm_epsilon_cq=cfg.eps_cq,
              rmsnorm_epsilon_ckv=cfg.eps_ckv)
    names = ("token_x", "weight_dq", "weight_uq_qr", "weight_uk",
             "weight_dkv_kr", "rmsnorm_gamma_cq", "rmsnorm_gamma_ckv",
             "rope_sin", "rope_cos", "cache_index", "kv_cache", "kr_cache",
             "query", "query_rope")
    def scales(s):
        return {k: s[k] for k in MLA_SCALES if k in s}
    calls = [qn.PreparedMlaPrologV2(*[s[k] for k in names], **kw, **scales(s))
             for s in sets[:1]]
    ws = calls[0].workspace
    calls += [qn.PreparedMlaPrologV2(*[s[k] for k in names], workspace=ws,
                                     **kw, **scales(s)) for s in sets[1:]]
    seq = [calls[i % len(calls)] for i in range(steps)]
    # the kernels whose start/stop events a call records
    launched = qn.mla_prolog_v2_kernels(calls[0].args)
    stream = torch.cuda.current_stream()
    he = HipEvents()
    ev = [[he.create() for _ in range(nph)] for _ in range(steps)]
    kev = [[he.create(0) for _ in range(2 * nk)] for _ in range(steps)]
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t0, t1 = he.create(), he.create()
    _hold_gpu(torch, 5.0 + 0.1 * steps)
    he.record(t0, stream)
    for i, c in enumerate(seq):
        c(phase_events=ev[i], kernel_events=kev[i])
    he.record(t1, stream)
    torch.cuda.synchronize()
    ms_eager = he.elapsed_ms(t0, t1) / steps
    phase_ms = [0.0] * (nph - 1)
    for row in ev:
        for p in range(nph - 1):
            phase_ms[p] += he.elapsed_ms(row[p], row[p + 1]) / steps
    kernel_ms = [None] * nk
    for k, name in enumerate(qn.MLA_KERNELS):
        if name in launched:
            kernel_ms[k] = sum(he.elapsed_ms(row[2 * k], row[2 * k + 1])
                               for row in kev) / steps
    for row in ev + kev:
        for e in row:
            he.destroy(e)
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in seq:
                c()
        g.replay()  # untimed: first replay
        torch.cuda.synchronize()
    times = []
    for _ in range(regions):
        torch.cuda.synchronize()
        _hold_gpu(torch, 2.0 if graph else 5.0 + 0.1 * steps)
        he.record(t0, stream)
        if graph:
            g.replay()
        else:
            for c in seq:
                c()
        he.record(t1, stream)
        torch.cuda.synchronize()
        times.append(he.elapsed_ms(t0, t1) / steps)
    del g
    he.destroy(t0)
    he.destroy(t1)
    med, lo, hi = _spread(times)
    return {"ms": med, "ms_min": lo, "ms_max": hi, "regions": regions,
            "steps": steps, "phase_ms": phase_ms, "kernel_ms": kernel_ms,
            "ms_eager": ms_eager}


def bench_qkv(steps, warmup, torch, qn, gh, make_workload, regions=5):
    """The qkv op on its (B=64, S=128) workload: `regions` HIP-graph
    replays, each of one graph holding `steps` calls alternating two input
    sets, timed separately; median, min and max ms per call."""
    w = make_workload(4)
    cfg = w.cfg
    sets = []
    for _ in range(2):
        d = gh.upload(w)
        d["q_out"] = torch.empty((cfg.T, cfg.Nq, cfg.D), dtype=torch.float16,
                                 device="cuda")
        sets.append(d)

    def call(d):
        qn.qkv_rmsnorm_rope_cache(
            d["qkv"], d["gamma_q"], d["gamma_k"], d["cos"], d["sin"],
            d["index"], d["k_cache"], d["v_cache"], Nq=cfg.Nq, Nk=cfg.Nk,
            Nv=cfg.Nv, quant_mode=cfg.quant_mode, epsilon=cfg.eps,
            k_scale=d["k_scale"], v_scale=d["v_scale"], q_out=d["q_out"],
            B=cfg.B, S=cfg.S)

    for i in range(warmup):
        call(sets[i % 2])
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            call(sets[i % 2])
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(regions):
        torch.cuda.synchronize()
        _hold_gpu(torch, 2.0)
        t0.record(s)
        g.replay()
        t1.record(s)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) / steps)
    del g
    ms, lo, hi = _spread(times)
    n_valid = int((w.arrays["index"] >= 0).sum())
    nbytes = qkv_bytes(cfg, n_valid)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": cfg.name, "tokens_per_s": cfg.T / (ms * 1e-3),
            "ms_per_step": ms, "ms_min": lo, "ms_max": hi, "steps": steps,
            "regions": regions, "algorithmic_bytes": nbytes,
            "achieved_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "timing": f"median of {regions} HIP-graph replays of {steps} "
                      "calls each"}


def bench_preprocess(steps, warmup, rotate, torch, qn, gh, make_workload,
                     regions=5):
    """MlaPreprocessV2 at the DeepSeek-V3 dims with 32 heads, decode
    T = 32: `regions` HIP-graph replays of one graph holding `steps` calls
    over `rotate` independent input sets (packed weights); median, min and
    max ms per call."""
    w = make_workload("pre_dsv3")
    cfg = w.cfg
    d0 = gh.upload(w)
    base = dict(d0)
    base["weight_dqkv"] = qn.mla_pack_weight(d0["weight_dqkv"])
    base["weight_uq_qr"] = qn.mla_pack_weight_uq_qr(d0["weight_uq_qr"], cfg.N,
                                                    cfg.D, cfg.Dr)
    base["weight_uk"] = qn.mla_pack_weight_uk(d0["weight_uk"])
    del d0
    sets = [base] + [{k: v.clone() for k, v in base.items()}
                     for _ in range(rotate - 1)]
    qsx = float(w.arrays["quant_scale_x"][0])
    qsc = float(w.arrays["quant_scale_cq"][0])
    for st in sets:
        st["query"] = torch.empty((cfg.T, cfg.N, cfg.Hckv),
                                  dtype=torch.bfloat16, device="cuda")
        st["query_rope"] = torch.empty((cfg.T, cfg.N, cfg.Dr),
                                       dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")

    def call(st):
        qn.mla_preprocess_v2(
            st["token_x"], st["gamma_x"], st["bias_x"], qsx,
            st["weight_dqkv"], st["dequant_scale_dqkv"], st["gamma_cq"],
            st["bias_cq"], qsc, st["weight_uq_qr"], st["dequant_scale_uq_qr"],
            st["weight_uk"], st["gamma_ckv"], st["rope_sin"], st["rope_cos"],
            st["cache_index"], st["kv_cache"], st["kr_cache"],
            epsilon=cfg.eps, query=st["query"], query_rope=st["query_rope"],
            workspace=ws)

    for i in range(warmup):
        call(sets[i % rotate])
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            call(sets[i % rotate])
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(regions):
        torch.cuda.synchronize()
        _hold_gpu(torch, 2.0)
        t0.record(s)
        g.replay()
        t1.record(s)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) / steps)
    del g
    ms, lo, hi = _spread(times)
    nbytes = preprocess_bytes(cfg)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": cfg.name, "tokens_per_s": cfg.T / (ms * 1e-3),
            "ms_per_step": ms, "ms_min": lo, "ms_max": hi, "steps": steps,
            "regions": regions, "algorithmic_bytes": nbytes,
            "achieved_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "timing": f"median of {regions} HIP-graph replays of {steps} "
                      f"calls over {rotate} rotating input sets"}


def measure_peaks(torch, qn, mib=1024):
    """Achievable rates on this GPU: a streaming read (the library's read
    probe) and a plain device copy (read + write) of `mib` MiB, and the
    library's MFMA-only bf16 loop; best of 5 event-timed runs each."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(5):
            t0.record(s)
            fn()
            t1.record(s)
            torch.cuda.synchronize()
            out.append(t0.elapsed_time(t1))
        return min(out)
    read_ms = best(lambda: qn.mla_probe_read(src, sink))
    copy_ms = best(lambda: dst.copy_(src))
    iters = 20000
    flop = qn.mla_probe_mfma_bf16(iters, sink)  # warm-up call; returns the flop count
    torch.cuda.synchronize()
    mfma_ms = best(lambda: qn.mla_probe_mfma_bf16(iters, sink))
    del src, dst
    torch.cuda.empty_cache()
    return {"read_GBps": n / (read_ms * 1e-3) / 1e9,
            "copy_GBps": 2 * n / (copy_ms * 1e-3) / 1e9,
            "mfma_bf16_TFLOPs": flop / (mfma_ms * 1e-3) / 1e12,
            "how": f"streaming read and device copy of {mib} MiB (copy "
                   "counts read + write bytes); dense bf16 MFMA loop with no "
                   "memory traffic; best of 5"}


def _blas_info():
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # pragma: no cover - older numpy
        return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        return len(os.sched_getaffinity(0))


def _time_oracle(fn, seconds, reps=3):
    """Median wall time of fn over at least `reps` runs, stopping once
    `seconds` have passed after the third."""
    ts = []
    t_start = time.perf_counter()
    while len(ts) < reps or time.perf_counter() - t_start < seconds:
        t = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t)
        if len(ts) >= reps and time.perf_counter() - t_start >= seconds:
            break
    ts.sort()
    return ts[len(ts) // 2], len(ts)


def cpu_baseline(w, seconds):
    """The float64 NumPy oracle on the host cores: whole T = 32 decode
    calls for about `seconds`; tokens/s from the median call time."""
    import oracle
    cfg = w.cfg
    dims = dict(He=cfg.He, Hcq=cfg.Hcq, N=cfg.N, D=cfg.D, Hckv=cfg.Hckv,
                Dr=cfg.Dr)
    med, n = _time_oracle(lambda: oracle.mla_prolog_v2(
        w.arrays, w.dtypes, dims, cfg.quant_mode, cfg.eps_cq, cfg.eps_ckv),
        seconds)
    return {"value": cfg.T / med, "unit": "tokens/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "blas": _blas_info(),
            "sample": f"median of {n} float64 NumPy oracle calls of the full "
                      f"T={cfg.T} decode workload"}


def cpu_baseline_other(make_workload, seconds):
    """The oracle on the other workloads, median of 3 calls each: tiny
    (config 0) whole; partial quant (config 3) on its first 16 tokens and
    prefill (config 2) on its first 512 (tokens are independent; the
    oracle's exact int64 product makes a whole config-3 call take seconds);
    the qkv op (config 4) whole.  tokens/s each."""
    import numpy as np
    import oracle
    from workloads import sub_workload
    out = {}
    for key, sample in ((0, None), (3, 16), (2, 512)):
        w = make_workload(key)
        cfg = w.cfg
        if sample:
            w = sub_workload(w, np.arange(sample))
        dims = dict(He=cfg.He, Hcq=cfg.Hcq, N=cfg.N, D=cfg.D, Hckv=cfg.Hckv,
                    Dr=cfg.Dr)
        ww = w
        med, n = _time_oracle(lambda: oracle.mla_prolog_v2(
            ww.arrays, ww.dtypes, dims, cfg.quant_mode, cfg.eps_cq,
            cfg.eps_ckv), 0.0)
        T = ww.cfg.T
        out[cfg.name] = {"tokens_per_s": T / med, "median_s": med,
                         "calls": n, "tokens_per_call": T}
    w = make_workload(4)
    cfg = w.cfg
    med, n = _time_oracle(lambda: oracle.qkv_rmsnorm_rope_cache(
        w.arrays, w.dtypes, dict(Nq=cfg.Nq, Nk=cfg.Nk, Nv=cfg.Nv, D=cfg.D),
        cfg.quant_mode, cfg.eps), 0.0)
    out[cfg.name] = {"tokens_per_s": cfg.T / med, "median_s": med,
                     "calls": n, "tokens_per_call": cfg.T}
    return out


def progress(msg):
    """One line on stderr per finished section (the JSON line is stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the prolog would shard by token or by head; the "
              "library implements no collective)", file=sys.stderr)
        return 2
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import qkv_norm_rope_amd as qn
    from workloads import device as gh
    from workloads import get_config, make_workload

    qn.load_library()  # fail loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.calibrate_copy > 0:
        calibrate_copy(torch, args.calibrate_copy)

    # ---- decode, T = 32 -------------------------------------------------
    w = make_workload(1)
    cfg = w.cfg
    sets = prepare_mla_sets(w, args.rotate, torch, qn, gh)
    r = run_mla(cfg, sets, args.steps, args.warmup, torch, qn,
                regions=args.regions)
    ms = r["ms"]
    kernel_ms = r["kernel_ms"]
    step_bytes = mla_bytes(cfg)
    a6_ms = kernel_ms[2]  # the up projection's own start/stop events
    # bf16 decode at T <= 32 runs the W^UK product inside the same launch
    merged = kernel_ms[3] is None
    a6_bytes = uqqr_bytes(cfg) + (uk_bytes(cfg) if merged else 0)
    a6_gbs = a6_bytes / (a6_ms * 1e-3) / 1e9
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    rec = recorded_traffic()
    traffic = rec[0] if rec is not None and rec[1] == kernel_source_hash() \
        else None
    out = {
        "metric": METRIC,
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, random-init weights of the DeepSeek-V3 "
                "MLA shapes)",
        "config": {"workload": cfg.name, "T": cfg.T, "B": cfg.B, "S": cfg.S,
                   "He": cfg.He, "Hcq": cfg.Hcq, "N": cfg.N, "D": cfg.D,
                   "Hckv": cfg.Hckv, "Dr": cfg.Dr, "block_num": cfg.block_num,
                   "block_size": cfg.block_size, "quant_mode": cfg.quant_mode,
                   "weight_layout": "packed_k16",
                   "rotating_input_sets": args.rotate},
        "timing": {"value": f"median over {r['regions']} separately timed "
                            f"regions, each one HIP-graph replay of exactly "
                            f"{args.steps} prepared calls (steps) cycling "
                            f"over {args.rotate} input sets, device "
                            "synchronised before and after each region",
                   "ms_per_step_min": r["ms_min"],
                   "ms_per_step_max": r["ms_max"],
                   "regions": r["regions"],
                   "calls_per_region": args.steps,
                   "kernel_us": "start/stop events taken by each main "
                                "kernel's own dispatch (hipExtLaunchKernel, "
                                "on the launch stream) in an eager region "
                                "of the same calls",
                   "phase_us": "events recorded between the launches "
                               "(kernel plus dispatch)"},
        "roofline": {"kernel": "up projection c^Q.[W^UQ|W^QR] + RoPE q^R"
                               + (" + per-head q^C.W^UK (one launch)"
                                  if merged else ""),
                     "bound": "hbm", "achieved": a6_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": a6_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": a6_bytes,
                     "workspace_bytes": uqqr_workspace_bytes(cfg, merged),
                     "avg_launch_us": a6_ms * 1e3,
                     "duration": "average over the eager region's calls of "
                                 "the kernel's own start/stop events"},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": step_bytes,
                          "achieved": step_gbs, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                          "target_frac": DECODE_TARGET_FRAC,
                          "gap_to_target": DECODE_TARGET_FRAC
                          - step_gbs / HBM_PEAK_GBS},
        "kernel_us": dict(zip(qn.MLA_KERNELS, [None if k is None else k * 1e3
                                               for k in kernel_ms])),
        "phase_us": dict(zip(("down", "norm_cache", "up_qr", "uk"),
                             [p * 1e3 for p in r["phase_ms"]])),
        "eager": {"ms_per_step": r["ms_eager"],
                  "tokens_per_s": cfg.T / (r["ms_eager"] * 1e-3)},
    }
    del sets
    torch.cuda.empty_cache()
    progress(f"decode T=32: {ms * 1e3:.2f} us/step")

    # ---- the same decode calls on one input set (a secondary line) -------
    # Its 122.6 MB of weights fit the 256 MB Infinity Cache, so after the
    # warm-up the weight bytes come from there rather than from HBM.
    if not args.no_warm:
        sets1 = prepare_mla_sets(w, 1, torch, qn, gh)
        rw = run_mla(cfg, sets1, args.steps, args.warmup, torch, qn,
                     regions=args.regions)
        wms = rw["ms"]
        out["decode_warm_single_set"] = {
            "workload": cfg.name, "tokens_per_s": cfg.T / (wms * 1e-3),
            "ms_per_step": wms, "ms_min": rw["ms_min"], "ms_max": rw["ms_max"],
            "hbm_frac_of_algorithmic_bytes": step_bytes / (wms * 1e-3) / 1e9
            / HBM_PEAK_GBS,
            "timing": "as the headline line, with one input set instead of "
                      f"{args.rotate} (secondary: weights stay in the MALL)",
        }
        del sets1
        torch.cuda.empty_cache()
        progress(f"decode T=32, one input set: {wms * 1e3:.2f} us/step")

    # ---- prefill, T = 4096 ------------------------------------------------
    if not args.no_prefill:
        wp = make_workload(2)
        pc = wp.cfg
        psets = prepare_mla_sets(wp, 1, torch, qn, gh)
        psteps = max(10, args.steps // 2)
        pr = run_mla(pc, psets, psteps, max(2, args.warmup // 2), torch, qn,
                     graph=False, regions=3)
        pms, pk = pr["ms"], pr["kernel_ms"]
        fl = mla_flops(pc)
        # The prefill plan fuses q^C.W^UK into the q^C tiles of the up
        # projection and runs the q^R tiles in the same launch: everything
        # after the norm phase is one roofline unit (one launch, or two).
        upf = uqqr_flops(pc) + uk_flops(pc)
        up_ms = sum(k for k in pk[2:4] if k is not None)
        frac = fl / (pms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
        out["prefill"] = {
            "workload": pc.name, "tokens_per_s": pc.T / (pms * 1e-3),
            "ms_per_step": pms, "ms_min": pr["ms_min"], "ms_max": pr["ms_max"],
            "steps": psteps, "regions": pr["regions"],
            "timing": f"median of {pr['regions']} eager regions of {psteps} "
                      "calls each",
            "algorithmic_flops": fl,
            "step_TFLOPs": fl / (pms * 1e-3) / 1e12,
            "mfma_frac": frac, "target_mfma_frac": PREFILL_TARGET_FRAC,
            "gap_to_target": PREFILL_TARGET_FRAC - frac,
            "kernel_us": dict(zip(("down", "norm", "up_qr_rope",
                                   "up_qc_uk_qr"),
                                  [None if k is None else k * 1e3 for k in pk])),
            "phase_us": dict(zip(("down", "norm_cache", "up_qr_rope",
                                  "up_qc_uk"),
                                 [p * 1e3 for p in pr["phase_ms"]])),
            "roofline": {"kernel": "up projections c^Q.[W^UQ|W^QR] with "
                                   "RoPE q^R and the fused per-head "
                                   "q^C.W^UK",
                         "bound": "mfma",
                         "achieved": upf / (up_ms * 1e-3) / 1e12,
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": upf / (up_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "algorithmic_flops": upf, "traffic": None},
        }
        del psets
        torch.cuda.empty_cache()
        progress(f"prefill T=4096: {pms * 1e3:.1f} us/step")

    # ---- partial quantisation at prefill size: T = 4096 ---------------------
    if not args.no_prefill and not args.no_partial_quant:
        wpq = make_workload(get_config(2).replace(
            name="mla_prefill_T4096_dsv3_partial_kv_int8",
            quant_mode="partial_kv_int8", seed=1102))
        pqc = wpq.cfg
        pqsets = prepare_mla_sets(wpq, 1, torch, qn, gh)
        psteps = max(10, args.steps // 2)
        pqr = run_mla(pqc, pqsets, psteps, max(2, args.warmup // 2), torch, qn,
                      graph=False, regions=3)
        pqms = pqr["ms"]
        # bf16 products (x.W^DQ_KR, q^C.W^UK) at the bf16 peak, the int8
        # c^Q.W^UQ_QR at the int8 peak
        t_peak = (2 * pqc.T * (pqc.He * (pqc.Hcq + pqc.Hckv + pqc.Dr)
                               + pqc.N * pqc.D * pqc.Hckv)) / (BF16_PEAK_TFLOPS * 1e12) \
            + uqqr_flops(pqc) / (INT8_PEAK_TOPS * 1e12)
        out["prefill_partial_quant"] = {
            "workload": pqc.name, "quant_mode": pqc.quant_mode,
            "tokens_per_s": pqc.T / (pqms * 1e-3), "ms_per_step": pqms,
            "ms_min": pqr["ms_min"], "ms_max": pqr["ms_max"],
            "steps": psteps, "regions": pqr["regions"],
            "algorithmic_ops": mla_flops(pqc),
            "mixed_peak_frac": t_peak / (pqms * 1e-3),
            "mixed_peak": "bf16 products at 2.5 PFLOP/s, the int8 up "
                          "projection at 5.0 POP/s",
            "kernel_us": dict(zip(qn.MLA_KERNELS,
                                  [None if k is None else k * 1e3
                                   for k in pqr["kernel_ms"]])),
            "timing": f"median of {pqr['regions']} eager regions of {psteps} "
                      "calls each",
        }
        del pqsets
        torch.cuda.empty_cache()
        progress(f"prefill partial quant T=4096: {pqms * 1e3:.1f} us/step")

    # ---- partial quantisation, int8 caches: T = 64, 32 heads -------------
    if not args.no_partial_quant:
        wq = make_workload(3)
        qc = wq.cfg
        qsets = prepare_mla_sets(wq, args.rotate, torch, qn, gh)
        qr = run_mla(qc, qsets, args.steps, max(5, args.warmup // 2), torch,
                     qn, regions=args.regions)
        qms, qk = qr["ms"], qr["kernel_ms"]
        qb = mla_partial_bytes(qc)
        out["partial_quant"] = {
            "workload": qc.name, "quant_mode": qc.quant_mode,
            "tokens_per_s": qc.T / (qms * 1e-3), "ms_per_step": qms,
            "ms_min": qr["ms_min"], "ms_max": qr["ms_max"],
            "algorithmic_bytes": qb,
            "achieved_GBps": qb / (qms * 1e-3) / 1e9,
            "hbm_frac": qb / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_us": dict(zip(qn.MLA_KERNELS, [None if k is None else k * 1e3
                                                   for k in qk])),
            "timing": f"median of {qr['regions']} HIP-graph replays of "
                      f"{args.steps} calls over {args.rotate} rotating "
                      "input sets",
        }
        del qsets
        torch.cuda.empty_cache()
        progress(f"partial quant T=64: {qms * 1e3:.2f} us/step")

    # ---- full quantisation (int8 kv_cache and query), T = 32 -------------
    if not args.no_full_quant:
        wf = make_workload(cfg.replace(quant_mode="full_kv_int8", seed=1101))
        fc = wf.cfg
        fsets = prepare_mla_sets(wf, args.rotate, torch, qn, gh)
        fr = run_mla(fc, fsets, args.steps, max(5, args.warmup // 2), torch,
                     qn, regions=args.regions)
        fms, fk = fr["ms"], fr["kernel_ms"]
        fb = mla_full_bytes(fc)
        out["full_quant_decode"] = {
            "workload": fc.name + "_full_kv_int8",
            "quant_mode": "full_kv_int8",
            "tokens_per_s": fc.T / (fms * 1e-3), "ms_per_step": fms,
            "ms_min": fr["ms_min"], "ms_max": fr["ms_max"],
            "algorithmic_bytes": fb,
            "achieved_GBps": fb / (fms * 1e-3) / 1e9,
            "hbm_frac": fb / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_us": dict(zip(qn.MLA_KERNELS, [None if k is None else k * 1e3
                                                   for k in fk])),
            "timing": f"median of {fr['regions']} HIP-graph replays of "
                      f"{args.steps} calls over {args.rotate} rotating input "
                      "sets; int8 x, weights (W^UK bf16), kv_cache and query",
        }
        del fsets
        torch.cuda.empty_cache()
        progress(f"full quant T=32: {fms * 1e3:.2f} us/step")

    if not args.no_preprocess:
        out["preprocess_decode"] = bench_preprocess(
            args.steps, max(5, args.warmup // 2), args.rotate, torch, qn, gh,
            make_workload, regions=args.regions)
        progress("preprocess T=32: %.2f us/step"
                 % (out["preprocess_decode"]["ms_per_step"] * 1e3))
        torch.cuda.empty_cache()

    if not args.no_qkv:
        out["qkv_rmsnorm_rope_cache"] = bench_qkv(
            max(20, args.steps), max(3, args.warmup // 2), torch, qn, gh,
            make_workload, regions=args.regions)
        progress("qkv op: %.2f us/step"
                 % (out["qkv_rmsnorm_rope_cache"]["ms_per_step"] * 1e3))

    if not args.no_peaks:
        out["achievable_peaks"] = measure_peaks(torch, qn)
        progress(f"achievable peaks: {out['achievable_peaks']}")

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        progress("cpu baseline (decode) done")
        out["cpu_baseline_other_workloads"] = cpu_baseline_other(
            make_workload, args.cpu_seconds)
        progress("cpu baseline (other workloads) done")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
