"""Benchmark: int4-g128 MoE FFN decode on one MI355X.

Workload (one "step" = one forward of one MoE layer over a decode batch):
DeepSeek-V3-shaped layer, hidden 7168, expert intermediate 2048, 256 routed
experts + 1 shared, top-8 routing with softmax over the selected logits, all
weights int4 with groups of 128 (one binary16 scale and one 4-bit zero per
group), bf16 activations, fp32 accumulation, bf16 output.  Two independent
layers are alternated step by step (11.8 GB of packed weights) so each step
reads its experts from HBM rather than from the 256 MB last-level cache, and
every step routes a different batch of tokens.  Inputs are seeded synthetic
data already resident in HBM when timing starts.

The timed step is one `moe_ffn_int4` call through the C ABI (routing with the
permutation and the layer input's fp16 rows in one launch, grouped gate/up +
SiLU, h rows, grouped down, combine).  The same steps then run once more as
the stage calls (`moe_route_sort`, `moe_expert_gate_up`, `moe_expert_down`,
`moe_combine`: the same kernels and launch shapes), where HIP events on the
launch stream time each grouped GEMM; those times give the roofline.  The events are created without a
system-scope fence (TimingEvent): a fenced event writes back and invalidates the
caches at every record, a 5-6 us gap that no real forward pays.  The JSON line
reports tokens/s of the main batch size, the roofline of the dominant kernel (grouped gate/up),
and the oracle's CPU time on a bounded sample as a baseline.  Extra fields
report the other decode batch sizes, the T=2048 prefill step (Zipf-skewed
routing), with a cold last-level cache the dense linears (the Llama-7B-shaped
decode stack at T=1 and the skinny sweep), the latency of the small float32
GEMV, the load-time quantizer, the router projection with its top-k, and the
main decode step with 64-wide groups and with one group per row.  `probes`
holds the ceilings measured on the same machine (a 2 GiB streaming read and
the fp16 matrix cores with no memory traffic), beside the published peaks the
fractions are quoted against.  The CPU baseline gives the host's CPU model and
a one-thread leg beside the all-thread one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, decimal GB/s
BF16_MFMA_PEAK = 2.5166e15   # MI355X dense fp16/bf16 MFMA, flop/s
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "moe_decode_t32_hbm_traffic.md")
GEMM_SOURCES = ["ffn_int4_g128_amd/csrc/qi4_dev.h", "ffn_int4_g128_amd/csrc/qi4_gemm.h",
                "ffn_int4_g128_amd/csrc/qi4_gemm.hip"]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    or None when the GEMM sources changed since the counters were taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_SUMMARY).read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in lines if ": " in l and l.split(": ", 1)[0] in
              ("kernel-source-sha256", "gate-up-traffic-bytes-per-launch"))
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if kv.get("kernel-source-sha256") != h.hexdigest():
        return None
    return float(kv["gate-up-traffic-bytes-per-launch"])


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on the
    launch stream.  torch.cuda.Event records with a system-scope release: the
    whole last-level cache hierarchy is written back and invalidated at every
    record, which costs about 5-6 us and shows up as a gap before the next
    kernel.  An event used only for timing needs no such fence, so these
    events add no gap between the kernels they bracket."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            import torch
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._h = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._lib().hipEventRecord(self._h, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if getattr(self, "_h", None) and self._hip is not None:
            self._hip.hipEventDestroy(self._h)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=32, help="tokens of the main decode batch")
    ap.add_argument("--sweep", type=str, default="1,8", help="other decode batch sizes to report")
    ap.add_argument("--layers", type=int, default=2)
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed prefill steps (T=2048, Zipf-skewed routing); 0 to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-linear measurements")
    ap.add_argument("--no-w4a8", action="store_true", help="skip the W4A8 MoE decode step")
    ap.add_argument("--no-groups", action="store_true",
                    help="skip the decode step with other group sizes and 8-bit codes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(c, layer, q, torch):
    import numpy as np
    import workloads
    ex = workloads.moe_experts(c["seed"], layer, c["E"], c["H"], c["I"], *c["scale"])
    sh = workloads.moe_shared(c["seed"], layer, c["H"], c["I"], *c["scale"])
    mw = q.pack_moe(ex, sh, c["E"], c["H"], c["I"], device="cuda")
    torch.cuda.synchronize()
    del ex, sh
    return mw


def build_layer_quantized(c, layer, q, torch, group, fmt=0):
    """A layer of the same shape for another group size or code width (fmt
    QI4_INT8: 8-bit codes): seeded random bf16 weights (N(0, 0.02^2)) quantized
    on the GPU and packed, expert by expert (fast to build; the values feed
    timing only)."""
    E, H, I = c["E"], c["H"], c["I"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 * c["seed"] + 17 * layer + group + 7 * fmt)

    def one(N, K, flags, out):
        w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32)
        w = w.mul_(0.02).to(torch.bfloat16)
        qw, sc, zr = q.quantize(w, group=group, flags=fmt)
        return q.pack(qw, sc, zr, N, K, flags | fmt, out=out, group=group)

    gu_b = q.packed_bytes(2 * I, H, q.QI4_PACK_GATEUP | fmt, group)
    dn_b = q.packed_bytes(H, I, fmt, group)
    w_gu = torch.empty(E * gu_b, dtype=torch.uint8, device="cuda")
    w_dn = torch.empty(E * dn_b, dtype=torch.uint8, device="cuda")
    for e in range(E):
        one(2 * I, H, q.QI4_PACK_GATEUP, w_gu[e * gu_b:(e + 1) * gu_b])
        one(H, I, 0, w_dn[e * dn_b:(e + 1) * dn_b])
    sgu = one(2 * I, H, q.QI4_PACK_GATEUP, None)
    sdn = one(H, I, 0, None)
    torch.cuda.synchronize()
    return q.MoeWeights(E, H, I, w_gu, w_dn, sgu, sdn, group, fmt)


def run_group_variants(q, torch, c, T, steps, warmup):
    """The decode step at batch T with 64-wide groups, with one group per row
    (group_size 0) and with 8-bit codes (groups of 128), two layers each, as the
    main measurement."""
    res = []
    for group, fmt in ((64, 0), (0, 0), (128, q.QI4_INT8)):
        layers = [build_layer_quantized(c, l, q, torch, group, fmt) for l in range(2)]
        r = run_batch(q, torch, layers, c, T, steps, warmup)
        res.append({"group_size": group, "bits": 8 if fmt else 4, "T": T,
                    "tokens_per_s": r["tokens_per_s"],
                    "ms_per_step": r["ms_per_step"], "gate_up_GBps": r["gate_up_GBps"],
                    "gate_up_hbm_frac": r["gate_up_GBps"] / HBM_PEAK_GBPS,
                    "down_GBps": r["down_GBps"], "step_GBps": r["step_GBps"]})
        del layers
        torch.cuda.empty_cache()
    return res


class Stepper:
    """One MoE forward through the C ABI, either as the one call
    (`moe_ffn_int4`: routing with the permutation and the input rows, gate/up,
    down, combine) or as the stage calls with events around the two grouped
    GEMMs (the same kernels and launch shapes)."""

    def __init__(self, q, torch, layers, T, top_k, n_batches, c, zipf=None):
        import numpy as np
        import workloads
        self.q, self.torch, self.layers, self.T, self.k = q, torch, layers, T, top_k
        self.c = c
        E, H = c["E"], c["H"]
        self.x = [q_bf16(torch, workloads.activations(c["seed"], 500 + 10 * b + T, T, H, "bf16"))
                  for b in range(n_batches)]
        if zipf is None:
            lg = [workloads.logits_normal(c["seed"], 600 + 10 * b + T, T, E) for b in range(n_batches)]
        else:
            lg = [workloads.logits_zipf(c["seed"], 600 + 10 * b + T, T, E, zipf) for b in range(n_batches)]
        self.logits = [torch.from_numpy(v).cuda() for v in lg]
        dev = "cuda"
        P = T * top_k
        R = P + T
        self.ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        self.wts = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        self.sp = torch.empty(P, dtype=torch.int32, device=dev)
        self.off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.inv = torch.empty(P, dtype=torch.int32, device=dev)
        self.act = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.h = torch.empty((R, 2, c["I"]), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((R, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.ws = q.moe_workspace(layers[0], top_k, T, dev)
        self.n_batches = n_batches

    def step(self, i, ev=None):
        q, torch = self.q, self.torch
        mw = self.layers[i % len(self.layers)]
        b = (i // len(self.layers)) % self.n_batches
        L = q.lib()
        d = mw.desc(self.k)
        import ctypes
        dref = ctypes.byref(d)
        st = q._stream()
        P = q._ptr
        T, E = self.T, self.c["E"]
        q._check(L.moe_route_sort(P(self.logits[b]), T, E, self.k, P(self.ids), P(self.wts),
                                  P(self.sp), P(self.off), P(self.inv), P(self.act), st),
                 "route_sort")
        if ev is not None:
            ev[0].record()
        q._check(L.moe_expert_gate_up(dref, P(self.x[b]), T, P(self.sp), P(self.off), P(self.act),
                                      P(mw.w_gate_up), P(mw.shared_gate_up), P(self.h), P(self.ws),
                                      self.ws.numel(), st), "gate_up")
        if ev is not None:
            ev[1].record()
        q._check(L.moe_expert_down(dref, P(self.h), T, P(self.off), P(self.act), P(mw.w_down),
                                   P(mw.shared_down), P(self.y), P(self.ws), self.ws.numel(), st),
                 "down")
        if ev is not None:
            ev[2].record()
        q._check(L.moe_combine(dref, P(self.y), P(self.wts), P(self.inv), T, P(self.out), st),
                 "combine")

    def call(self, i):
        """Step i as one moe_ffn_int4 call."""
        q = self.q
        mw = self.layers[i % len(self.layers)]
        b = (i // len(self.layers)) % self.n_batches
        import ctypes
        d = mw.desc(self.k)
        P = q._ptr
        q._check(q.lib().moe_ffn_int4(ctypes.byref(d), P(self.x[b]), self.T, P(self.logits[b]),
                                      None, None, P(mw.w_gate_up), P(mw.w_down),
                                      P(mw.shared_gate_up), P(mw.shared_down), P(self.out),
                                      P(self.ws), self.ws.numel(), q._stream()), "moe_ffn_int4")

    def timed_calls(self, steps, warmup):
        """Wall seconds of `steps` one-call steps after `warmup` untimed ones,
        bracketed by device synchronizations."""
        for i in range(warmup):
            self.call(i)
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.call(i)
        self.torch.cuda.synchronize()
        return time.perf_counter() - t0

    def touched(self, i):
        """Routed experts touched by step i (read back outside any timed region)."""
        self.step(i)
        self.torch.cuda.synchronize()
        return int(self.act[0].item())


def q_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def run_batch(q, torch, layers, c, T, steps, warmup, n_batches=8):
    import workloads
    k = c["top_k"]
    s = Stepper(q, torch, layers, T, k, n_batches, c)
    period = len(layers) * n_batches
    touched = [s.touched(i) for i in range(period)]
    # the step: one moe_ffn_int4 call
    wall = s.timed_calls(steps, warmup)
    # the same steps through the stage calls, events around the grouped GEMMs
    for i in range(warmup):
        s.step(i)
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s.step(i, evs[i])
    torch.cuda.synchronize()
    wall_stages = time.perf_counter() - t0
    gu_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    H, I = c["H"], c["I"]
    # bytes per weight of the gate/up (groups along H) and down (along I) matrices
    g, bits = layers[0].group, 8 if layers[0].flags & q.QI4_INT8 else 4
    pw_gu = workloads.packed_weight_bytes(1, g or H, bits)
    pw_dn = workloads.packed_weight_bytes(1, g or I, bits)
    gu_w, dn_w = 2 * I * H, H * I
    # algorithmic bytes per step: weights of the touched experts + the shared one,
    # activations in, outputs out, router logits in
    gu_bytes, dn_bytes, step_bytes = [], [], []
    for i in range(steps):
        n_e = touched[i % period] + 1
        gu_bytes.append(n_e * gu_w * pw_gu + T * H * 2 + T * (k + 1) * 2 * I * 2)
        dn_bytes.append(n_e * dn_w * pw_dn + T * (k + 1) * 2 * I * 2 + T * (k + 1) * H * 4)
        step_bytes.append(n_e * (gu_w * pw_gu + dn_w * pw_dn) + 2 * T * H * 2 + T * c["E"] * 4)
    mean = lambda v: sum(v) / len(v)
    ms_step = wall * 1e3 / steps
    return {
        "T": T, "ms_per_step": ms_step, "tokens_per_s": T * steps / wall,
        "stages_ms_per_step": wall_stages * 1e3 / steps,
        "experts_touched_mean": mean([touched[i % period] for i in range(steps)]) + 1,
        "step_GBps": mean(step_bytes) / (ms_step * 1e-3) / 1e9,
        "gate_up_us": mean(gu_ms) * 1e3, "down_us": mean(dn_ms) * 1e3,
        "gate_up_GBps": mean(gu_bytes) / (mean(gu_ms) * 1e-3) / 1e9,
        "down_GBps": mean(dn_bytes) / (mean(dn_ms) * 1e-3) / 1e9,
        "gate_up_bytes": mean(gu_bytes),
    }


def run_w4a8_decode(q, torch, layers, c, Ts, steps, warmup, n_batches=4):
    """The MoE decode step with W4A8 (moe_ffn_w4a8, one call per step: routing,
    int8 x, gate/up writing int8 h, down, combine) on the same 4-bit layers.
    Static scales: x_scale = max|x| / 127 of the batches; h_scale = max|h| / 127
    of h from the bf16 path's gate/up on the first batch (calibration, outside
    the timed region).  Fence-free events around each step."""
    import ctypes
    import workloads
    k, E, H, I = c["top_k"], c["E"], c["H"], c["I"]
    res = []
    for T in Ts:
        xs = [workloads.activations(c["seed"], 700 + 10 * b + T, T, H, "bf16") for b in range(n_batches)]
        x_scale = max(float(abs(workloads.bf16_bits_to_f32(v)).max()) for v in xs) / 127.0
        xt = [q_bf16(torch, v) for v in xs]
        lg = [torch.from_numpy(workloads.logits_normal(c["seed"], 800 + 10 * b + T, T, E)).cuda()
              for b in range(n_batches)]
        ids, wts, sp, off, inv, act = q.moe_route_sort(lg[0], k)
        h = q.moe_gate_up(xt[0], layers[0], k, sp, off, act).float()
        h_scale = float((h[:, 0] + h[:, 1]).abs().max()) / 127.0
        del h
        ws = torch.empty(q.lib().moe_ffn_w4a8_workspace_bytes(ctypes.byref(layers[0].desc(k)), T),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

        def step(i):
            b = (i // len(layers)) % n_batches
            q.moe_ffn_w4a8(xt[b], layers[i % len(layers)], k, x_scale, h_scale, logits=lg[b],
                           workspace=ws, out=out)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        evs = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            step(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        med = us[len(us) // 2]
        res.append({"T": T, "us_per_step": med, "tokens_per_s": T / (med * 1e-6),
                    "x_scale": x_scale, "h_scale": h_scale})
    return res


def run_prefill(q, torch, layers, steps, warmup, n_batches=2):
    """Prefill: T=2048 tokens of one layer, top-8 routing with Zipf(1.1) skew."""
    import workloads
    p = dict(workloads.MOE_PREFILL)
    c = dict(workloads.MOE_DECODE)
    T, k, H, I = p["T"], p["top_k"], p["H"], p["I"]
    s = Stepper(q, torch, layers, T, k, n_batches, c, zipf=p["zipf"])
    period = len(layers) * n_batches
    touched = [s.touched(i) for i in range(period)]
    wall = s.timed_calls(steps, warmup)
    for i in range(warmup):
        s.step(i)
    evs = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s.step(i, evs[i])
    torch.cuda.synchronize()
    wall_stages = time.perf_counter() - t0
    gu = sum(e[0].elapsed_time(e[1]) for e in evs) / steps * 1e-3
    dn = sum(e[1].elapsed_time(e[2]) for e in evs) / steps * 1e-3
    per_w = workloads.packed_weight_bytes(1)
    rows = T * k + T
    flop_gu, flop_dn = 2.0 * rows * 2 * I * H, 2.0 * rows * H * I
    n_e = sum(touched[i % period] for i in range(steps)) / steps + 1
    bytes_step = n_e * 3 * I * H * per_w + 2 * T * H * 2
    ms = wall * 1e3 / steps
    return {"T": T, "workload": "moe_ffn_prefill_deepseekv3_shape_zipf1.1", "ms_per_step": ms,
            "stages_ms_per_step": wall_stages * 1e3 / steps,
            "tokens_per_s": T * steps / wall, "experts_touched_mean": n_e,
            "mfma_frac_step": (flop_gu + flop_dn) / (ms * 1e-3) / BF16_MFMA_PEAK,
            "hbm_GBps_step": bytes_step / (ms * 1e-3) / 1e9,
            "gate_up_ms": gu * 1e3, "down_ms": dn * 1e3,
            "gate_up_mfma_frac": flop_gu / gu / BF16_MFMA_PEAK,
            "down_mfma_frac": flop_dn / dn / BF16_MFMA_PEAK}


def _dense_pack(q, torch, w, flags=0):
    dev = lambda a: torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda()
    return q.pack(dev(w["qweight"]), dev(w["scales"]), dev(w["zeros"]), w["N"], w["K"], flags)


def run_dense(q, torch, reps=100):
    """Dense int4-g128 linears, cold cache: before each timed rep 1 GiB is read
    (outside the event pair), so no weight is served from the 256 MB last-level
    cache.  A read, not a write: a 1 GiB write would leave that cache full of
    dirty lines whose write-back the next kernel's reads would pay for.  The
    events are enqueued while the flush runs, so the host adds no gaps.  Median
    over reps, with the 10th and 90th percentiles, and beside it a warm number
    (50 launches back to back, no flush, mean).  Workloads: the Llama-7B-shaped decode stack at T=1 (QKV, O,
    gate/up with SiLU*up, down: four launches back to back, and the same four
    replayed from a captured HIP graph) and the skinny sweep (5120->13824 and
    13824->5120 at T = 1..32, one launch per event pair).  The event pair is a
    fence-free TimingEvent pair, so it adds no cache write-back to the time."""
    import statistics
    import workloads
    per_w = workloads.packed_weight_bytes(1)
    rd = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    acc = torch.empty((), dtype=torch.float32, device="cuda")

    spread = {}
    sink = torch.empty(q.PROBE_READ_SINK_WORDS, dtype=torch.int32, device="cuda")

    def read_probe_us(nbytes):
        """Cold median (us) of the read probe over a buffer of nbytes: a plain
        streaming read of the same number of bytes, the floor for one launch
        that reads a matrix of that size."""
        buf = torch.ones((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
        fn = lambda: q.probe_stream_read(buf, sink)
        t = timed(fn)
        spread.pop(fn)
        return t * 1e6

    def timed(fn):
        """Cold median in seconds; its p10 / p90 and the warm mean (us) are kept
        in spread[fn] for the caller's record."""
        ts = []
        for r in range(reps + 3):
            torch.sum(rd, dim=0, out=acc)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if r >= 3:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        ts.sort()
        w0, w1 = TimingEvent(), TimingEvent()
        fn()
        torch.cuda.synchronize()
        w0.record()
        for _ in range(50):
            fn()
        w1.record()
        torch.cuda.synchronize()
        spread[fn] = {"p10_us": ts[len(ts) // 10] * 1e6, "p90_us": ts[(9 * len(ts)) // 10] * 1e6,
                      "warm_us": w0.elapsed_time(w1) * 1e3 / 50}
        return statistics.median(ts)

    c1 = workloads.LLAMA7B_STACK
    lin = []
    for i, (name, K, N, epi) in enumerate(c1["linears"]):
        w = workloads.weights(c1["seed"], 10 + i, N, K, *c1["scale"])
        flags = q.QI4_PACK_GATEUP if epi == "silu_mul" else 0
        e = q.QI4_EPI_SILU_MUL if epi == "silu_mul" else q.QI4_EPI_NONE
        x = q_bf16(torch, workloads.activations(c1["seed"], 20 + i, 1, K, "bf16"))
        n_out = N // 2 if epi == "silu_mul" else N
        y = torch.empty((1, n_out), dtype=torch.bfloat16, device="cuda")
        lin.append((name, N, K, n_out, _dense_pack(q, torch, w, flags), flags, e, x, y))
    calls = [lambda l=l: q.qlinear(l[7], l[4], l[1], flags=l[5], epilogue=l[6], out=l[8]) for l in lin]

    def stack():
        for f in calls:
            f()
    stack()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack()
    t_eager, t_graph = timed(stack), timed(graph.replay)
    eager_spread, graph_spread = spread.pop(stack), spread.pop(graph.replay)
    stack_bytes, per = 0.0, []
    for (name, N, K, n_out, *_), f in zip(lin, calls):
        b = N * K * per_w + K * 2 + n_out * 2
        stack_bytes += b
        t = timed(f)
        pr = read_probe_us(int(N * K * per_w))
        per.append({"linear": name, "N": N, "K": K, "us": t * 1e6,
                    "GBps": b / t / 1e9, **spread.pop(f), "read_probe_us": pr,
                    "frac_of_read_probe": pr / (t * 1e6)})
    del graph, lin, calls
    stack = {"workload": "llama7b_decode_stack_t1", "bytes": stack_bytes,
             "eager_us": t_eager * 1e6, "eager_tokens_per_s": 1.0 / t_eager,
             "eager_GBps": stack_bytes / t_eager / 1e9,
             "graph_us": t_graph * 1e6, "graph_tokens_per_s": 1.0 / t_graph,
             "graph_GBps": stack_bytes / t_graph / 1e9,
             "graph_hbm_frac": stack_bytes / t_graph / 1e9 / HBM_PEAK_GBPS,
             "eager_spread": eager_spread, "graph_spread": graph_spread, "linears": per,
             "read_probe_us": sum(l["read_probe_us"] for l in per)}
    stack["frac_of_read_probe"] = stack["read_probe_us"] / stack["eager_us"]

    c2 = workloads.SKINNY_SWEEP
    sweep = []
    for i, (K, N) in enumerate(c2["shapes"]):
        w = workloads.weights(c2["seed"], 10 + i, N, K, *c2["scale"])
        pw = _dense_pack(q, torch, w)
        pr = read_probe_us(int(N * K * per_w))
        for T in c2["T"]:
            x = q_bf16(torch, workloads.activations(c2["seed"], 20 + 10 * i + T, T, K, "bf16",
                                                    c2["x_scale"]))
            y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
            fn = lambda: q.qlinear(x, pw, N, out=y)
            t = timed(fn)
            b = N * K * per_w + T * K * 2 + T * N * 2
            sweep.append({"K": K, "N": N, "T": T, "us": t * 1e6,
                          "GBps": b / t / 1e9, "hbm_frac": b / t / 1e9 / HBM_PEAK_GBPS,
                          "tokens_per_s": T / t, **spread.pop(fn), "read_probe_us": pr,
                          "frac_of_read_probe": pr / (t * 1e6)})
        del pw
    # the same shapes with 8-bit codes (groups of 128), quantized on the GPU
    # from N(0, 0.02^2) bf16 weights
    sweep8 = []
    per_w8 = workloads.packed_weight_bytes(1, 128, 8)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    for i, (K, N) in enumerate(c2["shapes"]):
        wf = (torch.randn((N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
        qw, sc, zr = q.quantize(wf, flags=q.QI4_INT8)
        pw = q.pack(qw, sc, zr, N, K, q.QI4_INT8)
        del wf, qw, sc, zr
        for T in (1, 8, 32):
            x = q_bf16(torch, workloads.activations(c2["seed"], 20 + 10 * i + T, T, K, "bf16",
                                                    c2["x_scale"]))
            y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
            fn = lambda: q.qlinear(x, pw, N, flags=q.QI4_INT8, out=y)
            t = timed(fn)
            b = N * K * per_w8 + T * K * 2 + T * N * 2
            sweep8.append({"K": K, "N": N, "T": T, "us": t * 1e6,
                           "GBps": b / t / 1e9, "hbm_frac": b / t / 1e9 / HBM_PEAK_GBPS,
                           "tokens_per_s": T / t, **spread.pop(fn)})
        del pw
    # W4A8: the 4-bit matrices of the sweep with int8 activations (static
    # scale max|x| / 127); the time includes the activation-quantizing launch
    sweep_w4a8 = []
    for i, (K, N) in enumerate(c2["shapes"]):
        w = workloads.weights(c2["seed"], 10 + i, N, K, *c2["scale"])
        pw = _dense_pack(q, torch, w)
        for T in (1, 8, 32):
            xb = workloads.activations(c2["seed"], 20 + 10 * i + T, T, K, "bf16", c2["x_scale"])
            sx = float(abs(workloads.bf16_bits_to_f32(xb)).max()) / 127.0
            x = q_bf16(torch, xb)
            y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(q.lib().qlinear_w4a8_workspace_bytes(T, K), dtype=torch.uint8,
                             device="cuda")
            fn = lambda: q.qlinear_w4a8(x, sx, pw, N, out=y, workspace=ws)
            t = timed(fn)
            b = N * K * per_w + T * K * 2 + T * N * 2
            sweep_w4a8.append({"K": K, "N": N, "T": T, "us": t * 1e6,
                               "GBps": b / t / 1e9, "hbm_frac": b / t / 1e9 / HBM_PEAK_GBPS,
                               "tokens_per_s": T / t, **spread.pop(fn)})
        del pw
    del rd
    torch.cuda.empty_cache()
    return {"protocol": "1 GiB read before each rep (outside the events); median of "
                        f"{reps} reps (us), with p10_us / p90_us; warm_us: mean of 50 launches "
                        "back to back without the flush; read_probe_us: the read probe over "
                        "the matrix's packed bytes, same protocol", "llama7b_stack": stack, "skinny_sweep": sweep,
            "skinny_sweep_int8": sweep8, "skinny_sweep_w4a8": sweep_w4a8}


def run_router(q, torch, reps=20):
    """Router projection (bf16 [E][H] matrix, DeepSeek-V3 shape) plus top-8 through
    moe_router_topk, with a cold last-level cache (1 GiB read before each rep,
    outside the fence-free event pair); median over reps."""
    import statistics
    import workloads
    c = workloads.MOE_DECODE
    E, H, k = c["E"], c["H"], c["top_k"]
    w = q_bf16(torch, workloads.router_weights(c["seed"], 900, E, H))
    rd = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    res = []
    for T in (1, 32, 2048):
        x = q_bf16(torch, workloads.activations(c["seed"], 901 + T, T, H, "bf16"))
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ts = []
        for r in range(reps + 3):
            torch.sum(rd, dim=0, out=acc)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            q.moe_router_topk(x, w, k, logits=logits)
            e1.record()
            torch.cuda.synchronize()
            if r >= 3:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        t = statistics.median(ts)
        b = E * H * 2 + T * H * 2 + T * E * 4 + T * k * 8
        res.append({"T": T, "us": t * 1e6, "GBps": b / t / 1e9, "tokens_per_s": T / t,
                    "mfma_TFLOPs": 2 * T * E * H / t / 1e12})
    del rd
    return {"workload": "router_deepseekv3_shape_e256_h7168_top8", "protocol": "cold last-level "
            f"cache, median of {reps} reps; moe_router_topk (projection + top-k)", "points": res}


def run_quantize(q, torch, reps=10):
    """Load-time quantizer throughput: bf16 weights [16384][7168] (four experts'
    gate/up rows of the MoE layer), N(0, 0.02), cold cache (1 GiB read before each
    rep, outside the events); median of reps."""
    import statistics
    import workloads
    N, K = 16384, 7168
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    rd = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    q.quantize(w)
    ts = []
    for r in range(reps + 2):
        torch.sum(rd, dim=0, out=acc)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        q.quantize(w)
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(e0.elapsed_time(e1) * 1e-3)
    t = statistics.median(ts)
    b = N * K * (2 + workloads.packed_weight_bytes(1))
    del w, rd
    torch.cuda.empty_cache()
    return {"workload": "quantize_bf16_16384x7168_g128", "us": t * 1e6,
            "weights_per_s": N * K / t, "GBps": b / t / 1e9, "hbm_frac": b / t / 1e9 / HBM_PEAK_GBPS}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c, T, target_s):
    """The oracle (fp64 C, OpenMP over output rows) on a bounded sample of the
    same workload: n tokens of layer 0, n chosen for about target_s seconds on
    all the host threads this process may use; then one token (or more, for
    about target_s / 4 seconds) on a single thread."""
    import numpy as np
    import oracle
    import workloads
    oracle.lib()
    ex = workloads.moe_experts(c["seed"], 0, c["E"], c["H"], c["I"], *c["scale"])
    sh = workloads.moe_shared(c["seed"], 0, c["H"], c["I"], *c["scale"])
    Tmax = 256
    x = workloads.activations(c["seed"], 700, Tmax, c["H"], "bf16")
    logits = workloads.logits_normal(c["seed"], 701, Tmax, c["E"])
    ids, p = oracle.topk_softmax(logits, c["top_k"])
    threads = oracle.default_threads()
    x64 = oracle.widen(x, "bf16")
    t0 = time.perf_counter()
    oracle.moe(x64[:1], ids[:1], p[:1], ex, sh, c["H"], c["I"], c["E"], threads=threads)
    one = time.perf_counter() - t0
    n = int(max(1, min(Tmax, target_s // max(one, 1e-3))))
    t0 = time.perf_counter()
    oracle.moe(x64[:n], ids[:n], p[:n], ex, sh, c["H"], c["I"], c["E"], threads=threads)
    dt = time.perf_counter() - t0
    # one thread: one token, then more tokens if that took under target_s / 4
    t0 = time.perf_counter()
    oracle.moe(x64[n:n + 1], ids[n:n + 1], p[n:n + 1], ex, sh, c["H"], c["I"], c["E"], threads=1)
    one1 = time.perf_counter() - t0
    n1 = int(max(1, min(Tmax - n - 1, (target_s / 4) // max(one1, 1e-3))))
    if n1 > 1:
        t0 = time.perf_counter()
        oracle.moe(x64[n + 1:n + 1 + n1], ids[n + 1:n + 1 + n1], p[n + 1:n + 1 + n1], ex, sh,
                   c["H"], c["I"], c["E"], threads=1)
        dt1 = time.perf_counter() - t0
    else:
        n1, dt1 = 1, one1
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} tokens through the full layer 0 (routing, 8 experts + shared each), "
                      "one at a time as in decode",
            "seconds": dt, "cpu_model": cpu_model(),
            "one_thread": {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} other tokens of the same layer", "seconds": dt1}}


def run_copy(torch, mib=1024, reps=20):
    """Context for the HBM roofline: a plain device-to-device copy (torch's copy
    kernel, 1 GiB read + 1 GiB written per launch), bytes moved / time."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del a, b
    return {"bytes_per_launch": 2 * n, "us": us, "GBps": 2 * n / (us * 1e-6) / 1e9}


def run_probes(q, torch, reps=10):
    """The two ceilings, measured on this machine with the library's probes
    (include/qi4_probe.h): a streaming read of a 2 GiB buffer (8x the 256 MB
    last-level cache, so it comes from HBM) and the fp16 matrix cores on every
    SIMD with no memory traffic (1024 workgroups of four waves, eight
    independent MFMA 16x16x32 chains each).  Medians over reps, fence-free events."""
    import statistics
    buf = torch.ones(1 << 29, dtype=torch.float32, device="cuda")   # 2 GiB
    nbytes = buf.numel() * 4
    sink = torch.empty(q.PROBE_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    q.probe_stream_read(buf, sink)
    ts = []
    for _ in range(reps):
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        q.probe_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t_read = statistics.median(ts)
    del buf
    torch.cuda.empty_cache()
    fsink = torch.empty(1, dtype=torch.float32, device="cuda")
    iters, wgs = 4096, 1024
    q.probe_mfma(64, wgs, fsink)
    ts = []
    for _ in range(5):
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        flops = q.probe_mfma(iters, wgs, fsink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t_mfma = statistics.median(ts)
    return {"stream_read": {"bytes": nbytes, "us": t_read * 1e6, "GBps": nbytes / t_read / 1e9,
                            "frac_of_published": nbytes / t_read / 1e9 / HBM_PEAK_GBPS},
            "mfma_f16": {"flops": flops, "us": t_mfma * 1e6, "TFLOPs": flops / t_mfma / 1e12,
                         "frac_of_published": flops / t_mfma / BF16_MFMA_PEAK}}


def run_gemv_small(q, torch, reps=200):
    """The small GEMV (T=1, K=256, N=128, float32 in and out, groups of 128):
    a latency figure only (its 18.6 KB take nanoseconds at HBM speed).  Median of
    single launches (warm), fence-free events enqueued behind a GPU spin."""
    import statistics
    import workloads
    c = workloads.GEMV_SMALL
    w = workloads.weights(c["seed"], 0, c["N"], c["K"], *c["scale"])
    pw = _dense_pack(q, torch, w)
    x = torch.from_numpy(workloads.activations(c["seed"], 0, c["T"], c["K"], "f32")).cuda()
    y = torch.empty((c["T"], c["N"]), dtype=torch.float32, device="cuda")
    for _ in range(5):
        q.qlinear(x, pw, c["N"], out=y)
    ts = []
    for _ in range(reps):
        e0, e1 = TimingEvent(), TimingEvent()
        # the GPU spins while the events and the launch are enqueued, so the
        # interval holds the kernel and not the host's call
        torch.cuda._sleep(200000)
        e0.record()
        q.qlinear(x, pw, c["N"], out=y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return {"workload": c["name"], "us_median": statistics.median(ts),
            "us_p10": ts[len(ts) // 10], "us_p90": ts[(9 * len(ts)) // 10]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import ffn_int4_g128_amd as q
    import workloads
    c = dict(workloads.MOE_DECODE)
    log(f"building {args.layers} layers of packed weights ...")
    t0 = time.perf_counter()
    layers = [build_layer(c, l, q, torch) for l in range(args.layers)]
    log(f"  done in {time.perf_counter() - t0:.1f} s")

    copy = run_copy(torch)
    log(f"copy: {json.dumps(copy)}")
    probes = run_probes(q, torch)
    log(f"probes: {json.dumps(probes)}")
    main_r = run_batch(q, torch, layers, c, args.T, args.steps, args.warmup)
    log(f"T={args.T}: {json.dumps(main_r)}")
    sweep = []
    for t in [int(v) for v in args.sweep.split(",") if v.strip()]:
        if t == args.T:
            continue
        r = run_batch(q, torch, layers, c, t, max(10, args.steps), args.warmup)
        log(f"T={t}: {json.dumps(r)}")
        sweep.append(r)

    prefill = None
    if args.prefill_steps > 0:
        prefill = run_prefill(q, torch, layers, args.prefill_steps, 2)
        mfma_probe = probes["mfma_f16"]["TFLOPs"] * 1e12
        prefill["mfma_frac_of_probe"] = prefill["mfma_frac_step"] * BF16_MFMA_PEAK / mfma_probe
        log(f"prefill: {json.dumps(prefill)}")

    dense = None
    if not args.no_dense:
        dense = run_dense(q, torch)
        log(f"dense: {json.dumps(dense)}")

    quant = run_quantize(q, torch)
    log(f"quantize: {json.dumps(quant)}")

    gemv = run_gemv_small(q, torch)
    log(f"gemv small: {json.dumps(gemv)}")

    router = run_router(q, torch)
    log(f"router: {json.dumps(router)}")

    w4a8 = None
    if not args.no_w4a8:
        w4a8 = run_w4a8_decode(q, torch, layers, c, [1, 8, 32], max(10, args.steps), args.warmup)
        log(f"w4a8 decode: {json.dumps(w4a8)}")

    groups = None
    if not args.no_groups:
        groups = run_group_variants(q, torch, c, args.T, max(10, args.steps // 2), args.warmup)
        log(f"format variants: {json.dumps(groups)}")

    cpu = None
    if not args.no_cpu_baseline:
        del layers
        torch.cuda.empty_cache()
        log("timing the oracle on a CPU sample ...")
        cpu = cpu_baseline(c, args.T, args.cpu_seconds)
        log(f"  {json.dumps(cpu)}")

    gu_gbps = main_r["gate_up_GBps"]
    out = {
        "metric": "int4-g128 MoE FFN decode tokens/s (DeepSeek-V3-shaped layer)",
        "value": main_r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded int4 weights, N(0,1) bf16 activations and router logits)",
        "config": {"workload": "moe_ffn_decode_deepseekv3_shape", "T": args.T, "hidden": c["H"],
                   "inter": c["I"], "experts": c["E"], "shared_experts": 1, "top_k": c["top_k"],
                   "group": 128, "layers_alternated": args.layers},
        "roofline": {"bound": "hbm", "kernel": "moe grouped gate/up + SiLU (qgemm_kernel)",
                     "achieved": gu_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gu_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "launch_us": main_r["gate_up_us"], "bytes_per_launch": main_r["gate_up_bytes"],
                     "copy_GBps": copy["GBps"], "frac_of_copy": gu_gbps / copy["GBps"],
                     "probe_read_GBps": probes["stream_read"]["GBps"],
                     "frac_of_probe_read": gu_gbps / probes["stream_read"]["GBps"]},
        "probes": probes,
        "step_GBps": main_r["step_GBps"],
        "experts_touched_mean": main_r["experts_touched_mean"],
        "down_GBps": main_r["down_GBps"],
        "sweep": [{k: r[k] for k in ("T", "tokens_per_s", "ms_per_step", "step_GBps", "gate_up_GBps",
                                     "down_GBps", "experts_touched_mean")} for r in sweep],
        "prefill": prefill,
        "dense": dense,
        "gemv_small_latency": gemv,
        "quantize": quant,
        "format_variants": groups,
        "w4a8_moe_decode": w4a8,
        "router": router,
        "cpu_baseline": cpu,
    }
    # the headline figures of the sections above, rounded, last in the line (a
    # reader that sees only the end of the output still finds them)
    r3 = lambda v: None if v is None else round(v, 3)
    out["summary"] = {
        "decode_tokens_per_s": {str(r["T"]): round(r["tokens_per_s"]) for r in
                                [*sweep, {"T": args.T, "tokens_per_s": main_r["tokens_per_s"]}]},
        "gate_up_hbm_frac": r3(gu_gbps / HBM_PEAK_GBPS),
        "gate_up_frac_of_probe_read": r3(gu_gbps / probes["stream_read"]["GBps"]),
        "prefill_ms_per_step": r3(prefill["ms_per_step"]) if prefill else None,
        "prefill_mfma_frac": r3(prefill["mfma_frac_step"]) if prefill else None,
        "dense_stack_us": r3(dense["llama7b_stack"]["eager_us"]) if dense else None,
        "dense_stack_frac_of_read_probe": r3(dense["llama7b_stack"]["frac_of_read_probe"]) if dense else None,
        "quantize_us": r3(quant["us"]) if quant else None,
        "cpu_tokens_per_s": r3(cpu["value"]) if cpu else None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
