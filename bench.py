"""Throughput of the SSD chunked-scan forward on one MI355X.

One step = one pass of the whole forward (plan, chunk_cumsum, bmm_chunk,
chunk_state, state_passing, chunk_scan) over one batch of synthetic input
already resident in HBM.  Default workload: the Mamba-2 layer shape (batch 2,
seqlen 4096, 24 heads, headdim 64, dstate 128, 1 group, chunk 256, bf16
x/B/C, fp32 accumulation).

Prints ONE JSON line.  `value` is tokens/s over the K timed steps, replayed
back to back from a HIP graph between two HIP events; the median, p10 and
p90 of one step come from 20 further samples of 5 replays each (the clova.ai
page reports the median of 100 runs after 10 warm-ups, section "So how much
faster is it?").  `roofline` covers the slowest launch of the step, timed
live with HIP events on the stream its kernel runs on, warm and after the
last-level cache is evicted; `cpu_baseline` is the fp64 CPU oracle timed on
this host's cores on the same workload.  `workloads` repeats the step and
launch timings on the other full-size configurations (training batch, long
context, packed batch).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD forward tokens/s per MI355X; achieved HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA bf16, published
F32_PEAK_TFLOPS = 157.3        # dense MFMA fp32, published
STAGE_ORDER = ("plan", "chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing", "chunk_scan")
# What one bf16 forward step launches: stages 1-3 run as one fused launch.
STEP_LAUNCHES = ("plan", "front", "state_passing", "chunk_scan")
FLUSH_BYTES = 1 << 30          # written before a cold measurement: 4x the last-level cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(prob, nchunks):
    """Bytes each stage must move and flops it must do (see the design notes):
    inputs read once, outputs written once, intermediates at their stored
    precision, CB only on and below the diagonal."""
    tok = prob.batch * prob.seqlen
    H, P, N, G, L = prob.nheads, prob.headdim, prob.dstate, prob.ngroups, prob.chunk_size
    e = 2 if prob.dtype == "bf16" else 4
    nst = prob.nseq
    tri = L * (L + 1) // 2
    has_init = 1   # workloads 4-5 read initial states; harmless upper bound otherwise
    work = {
        "plan": (0, 0),
        # chunk_cumsum + bmm_chunk + chunk_state in one launch: the step and its
        # running sum are formed in-kernel (dt in, delta and sums out once)
        # (B is read once: the bmm tiles and the state workgroups share it)
        "front": (4 * tok * H + 8 * nchunks * H * L
                  + 2 * e * tok * G * N + e * nchunks * G * tri
                  + e * tok * H * P + 4 * nchunks * H * P * N,
                  2 * N * tri * nchunks * G + 2 * L * P * N * nchunks * H),
        "chunk_cumsum": (4 * tok * H + 8 * nchunks * H * L, 0),
        "bmm_chunk": (2 * e * tok * G * N + e * nchunks * G * tri, 2 * N * tri * nchunks * G),
        "chunk_state": (e * tok * H * P + e * tok * G * N + 8 * nchunks * H * L
                        + 4 * nchunks * H * P * N, 2 * L * P * N * nchunks * H),
        "state_passing": ((4 + e) * nchunks * H * P * N + 4 * (1 + has_init) * nst * H * P * N,
                          2 * P * N * nchunks * H),
        "chunk_scan": (2 * e * tok * H * P + e * tok * G * N + e * nchunks * G * tri
                       + 8 * nchunks * H * L + e * nchunks * H * P * N,
                       (2 * P * tri + 2 * L * N * P) * nchunks * H),
    }
    return work


def fused_minimum_bytes(prob):
    """What any forward must move: x, dt, B, C and the initial states read,
    y and the final states written."""
    tok = prob.batch * prob.seqlen
    H, P, N, G = prob.nheads, prob.headdim, prob.dstate, prob.ngroups
    e = 2 if prob.dtype == "bf16" else 4
    return 2 * e * tok * H * P + 4 * tok * H + 2 * e * tok * G * N + 8 * prob.nseq * H * P * N


STAGE_SOURCE = {"plan": ("ssd_prep.hip",), "chunk_cumsum": ("ssd_prep.hip",),
                "front": ("ssd_chunk_state.hip", "ssd_state_tile.h"),
                "bmm_chunk": ("ssd_bmm.hip",),
                "chunk_state": ("ssd_chunk_state.hip", "ssd_state_tile.h"),
                "state_passing": ("ssd_state_passing.hip",),
                "chunk_scan": ("ssd_chunk_scan.hip", "ssd_scan_tile.h", "ssd_gate.h")}
COMMON_HEADERS = ("ssd_common.h", "ssd_device.h", "ssd_kernels.h")


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and blank space removed) of a kernel's
    source files and of the headers every kernel includes."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "state_space_model_ssd_amd", "csrc")
    h = hashlib.sha256()
    for f in STAGE_SOURCE[kernel] + COMMON_HEADERS:
        text = open(os.path.join(csrc, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload_tag: str):
    """HBM bytes per launch from the committed counter summary
    profiles/<kernel>_<workload>_traffic.md (FETCH_SIZE and WRITE_SIZE passes,
    scaled by a plain copy of known size), or None when there is none or the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return int(fields["traffic_bytes_per_launch"])


def measured_counters(kernel: str, workload_tag: str):
    """Counter figures of one launch (matrix-core busy fraction of SIMD time,
    LDS bank-conflict cycles per active LDS cycle, L2 hit rate) from the
    committed summary profiles/counters_<workload>.md, or None when there is
    none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload_tag}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.split(":", 1)
        if len(parts) != 2:
            continue
        key = parts[0].split()
        if len(key) == 2 and key[1] == kernel:
            vals[key[0]] = parts[1].strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return {"mfma_busy": float(vals["mfma_busy"]),
                "lds_conflict_ratio": float(vals["lds_conflict_ratio"]),
                "l2_hit": float(vals["l2_hit"]), "source": f"profiles/counters_{workload_tag}.md"}
    except (KeyError, ValueError):
        return None


def env_info():
    info = {"host": platform.node(), "nproc": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except Exception:
        pass
    return info


def percentiles(vals):
    """median, p10, p90 (nearest rank) of a list of numbers."""
    v = sorted(vals)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "n": len(v)}


class Workload:
    """One workload's device inputs, buffers and a HIP graph of one step."""

    def __init__(self, k, torch, binding, tuning_arg=None):
        from state_space_model_ssd_amd.inputs import workload_inputs, WORKLOAD_NAMES
        from state_space_model_ssd_amd import tuning
        self.torch, self.binding, self.k = torch, binding, k
        dev = torch.device("cuda:0")
        log(f"[bench] workload {k}: drawing inputs")
        self.prob, self.inp = workload_inputs(k)
        prob = self.prob
        self.name = WORKLOAD_NAMES[k]
        self.d = {n: (v.to(dev) if isinstance(v, torch.Tensor) else v) for n, v in self.inp.items()}
        self.cprob = binding.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim,
                                          prob.dstate, prob.ngroups, prob.chunk_size,
                                          1 if prob.dtype == "bf16" else 0,
                                          nseq=len(prob.seq_lens) if prob.seq_lens else 0)
        self.lay = binding.workspace_layout(self.cprob)
        self.pinned = tuning_arg
        self.tuned = tuning_arg if tuning_arg is not None else tuning.lookup(self.cprob)
        self.tune_arg = tuning_arg if tuning_arg is not None else "config"
        self.tuning_record = {"source": "pinned" if tuning_arg is not None else
                              "tuned config" if self.tuned else "library's own choice",
                              "key": tuning.shape_key(self.cprob), "choice": self.tuned or {},
                              "library_choice": binding.fwd_choices(self.cprob)}
        self.ws = torch.empty(self.lay.total_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(self.d["x"])
        self.fin = torch.empty((prob.nseq, prob.nheads, prob.headdim, prob.dstate),
                               dtype=torch.float32, device=dev)
        self.tokens = prob.batch * prob.seqlen
        self.graph = None

    def step(self, stages=None):
        b = self.binding
        self.binding.ssd_fwd(self.d["x"], self.d["dt"], self.d["A"], self.d["B"], self.d["C"],
                             self.prob.chunk_size, D=self.d["D"], dt_bias=self.d["dt_bias"],
                             initial_states=self.d["init"], cu_seqlens=self.d["cu_seqlens"],
                             out=self.out, final_states=self.fin, workspace=self.ws,
                             stages=b.STAGE_ALL if stages is None else stages,
                             tuning=self.tune_arg)

    def nchunks(self):
        if self.prob.seq_lens:
            return int(self.binding.intermediates(self.ws, self.cprob)["seq_chunks"][-1].item())
        return self.lay.max_chunks

    def capture(self, warmup):
        torch = self.torch
        for _ in range(max(warmup, 1)):
            self.step()
        torch.cuda.synchronize()
        self.ref_out = self.out.clone()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            self.step()                  # settle on the side stream before capture
            torch.cuda.synchronize()
            with torch.cuda.graph(self.graph, stream=stream):
                self.step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(self.out, self.ref_out):
            raise RuntimeError("graph replay differs from the eager forward")

    def time_replays(self, steps):
        """K replays back to back between two HIP events: (total ms, wall s)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.perf_counter() - wall0

    def step_samples(self, batches, per_batch):
        """Per-step ms of `batches` samples, each the mean of `per_batch`
        replays back to back between two HIP events (an event recorded
        between every two replays would add its own cost to each step)."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(batches):
            for _ in range(per_batch):
                self.graph.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) / per_batch for i in range(batches)]

    def time_cold(self, reps, flush, fn):
        """Median over reps of fn() timed alone, each after a write of the
        flush buffer evicts the last-level cache (ms list)."""
        torch = self.torch
        cur = torch.cuda.current_stream()
        res = []
        for _ in range(reps):
            flush.fill_(1.0)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(cur)
            fn()
            c1.record(cur)
            torch.cuda.synchronize()
            res.append(c0.elapsed_time(c1))
        return res

    def time_launches(self, names, reps):
        """Average us of each launch: reps back-to-back launches between two
        HIP events on the launch stream, queued behind a GPU sleep so the CPU
        is never the limit."""
        torch, b = self.torch, self.binding
        cur = torch.cuda.current_stream()
        masks = dict(b.STAGES)
        masks["front"] = b.STAGES["chunk_cumsum"] | b.STAGES["bmm_chunk"] | b.STAGES["chunk_state"]
        res = {}
        for name in names:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            try:
                torch.cuda._sleep(20_000_000)
            except Exception:
                pass
            e0.record(cur)
            for _ in range(reps):
                self.step(masks[name])
            e1.record(cur)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / reps
        return res

    def masks(self):
        b = self.binding
        m = dict(b.STAGES)
        m["front"] = b.STAGES["chunk_cumsum"] | b.STAGES["bmm_chunk"] | b.STAGES["chunk_state"]
        return m


def stage_record(work, name, us, dtype):
    nbytes, flops = work[name]
    rec = {"us": round(us, 3), "alg_bytes": int(nbytes),
           "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
           "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if flops:
        peak = BF16_PEAK_TFLOPS if dtype == "bf16" else F32_PEAK_TFLOPS
        rec["tflops"] = round(flops / (us * 1e-6) / 1e12, 2)
        rec["mfma_frac"] = round(flops / (us * 1e-6) / 1e12 / peak, 4)
    return rec


def fused_step(k, torch, binding, steps, warmup):
    """Median step of workload k with the fused forward pinned
    (ssd_tuning_t.fused = 2), or None where the shape has none."""
    w = Workload(k, torch, binding, {"fused": 2})
    if w.prob.dtype != "bf16" or w.prob.chunk_size not in (128, 256):
        return None
    w.capture(warmup)
    w.time_replays(steps)
    per = w.step_samples(10, 5)
    med = percentiles(per)["median"] * 1e3
    del w
    torch.cuda.empty_cache()
    return round(med, 2)


def gated_norm_record(w, torch, binding, reps):
    """The gated RMS norm after the forward on workload w's output: the
    standalone forward and backward kernels over rows of H*P channels (one
    group per token, and one group per head), and the forward step with the
    norm fused into chunk_scan's store (groups of one head) against the plain
    step.  Algorithmic bytes: y, z read and out written (forward); y, z, dout
    read and dy, dz written (backward)."""
    prob = w.prob
    if prob.dtype != "bf16":
        return None
    tokens, C, P = w.tokens, prob.nheads * prob.headdim, prob.headdim
    gen = torch.Generator().manual_seed(77)
    z = torch.randn(w.d["x"].shape, generator=gen).to(torch.bfloat16).to(w.d["x"].device)
    wt = torch.ones(C, device=z.device)
    y = w.out.view(tokens, C)
    zz = z.view(tokens, C)
    dout = torch.randn((tokens, C), generator=gen).to(torch.bfloat16).to(z.device)
    cur = torch.cuda.current_stream()
    res = {"rows": tokens, "channels": C}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    nb = 2 * tokens * C
    for gs in (C, P):
        out = torch.empty_like(y)
        ws = torch.empty(1 << 26, dtype=torch.uint8, device=z.device)
        fus = timed(lambda: binding.gated_norm_fwd(y, zz, wt, gs, out=out))
        bus = timed(lambda: binding.gated_norm_bwd(y, zz, wt, dout, gs, workspace=ws))
        res[f"group{gs}"] = {
            "fwd_us": round(fus, 2), "fwd_alg_bytes": 3 * nb,
            "fwd_hbm_frac": round(3 * nb / (fus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_us": round(bus, 2), "bwd_alg_bytes": 5 * nb,
            "bwd_hbm_frac": round(5 * nb / (bus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    d = w.d
    gout = torch.empty_like(d["x"])

    def gated_step():
        binding.ssd_fwd_gated(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, z, wt, P,
                              D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                              cu_seqlens=d["cu_seqlens"], out=gout, final_states=w.fin,
                              workspace=w.ws)
    g_us = timed(gated_step)
    plain_us = timed(lambda: w.step())
    res["fused_epilogue"] = {"group_size": P, "step_us": round(g_us, 2),
                             "plain_step_us": round(plain_us, 2),
                             "note": "eager back-to-back calls (not graph replays)"}
    return res


def side_workload(k, torch, binding, flush, steps, warmup, reps, compare_fused=False):
    """Step and launch timings of another full-size workload (warm and cold)."""
    w = Workload(k, torch, binding)
    w.capture(warmup)
    total, _ = w.time_replays(steps)
    per = w.step_samples(10, 5)
    cold = w.time_cold(5, flush, w.graph.replay)
    nch = w.nchunks()
    work = algorithmic_work(w.prob, nch)
    launches = [n for n in STEP_LAUNCHES if n != "plan" or w.prob.seq_lens]
    us = w.time_launches(launches, reps)
    if not torch.equal(w.out, w.ref_out):
        raise RuntimeError(f"workload {k}: stage-by-stage run differs from the eager forward")
    step_pct = {q: round(v * 1e3, 2) for q, v in percentiles(per).items() if q != "n"}
    cold_pct = {q: round(v * 1e3, 2) for q, v in percentiles(cold).items() if q != "n"}
    rec = {"workload": w.name, "tokens": w.tokens, "chunks": nch,
           "tokens_per_s": round(w.tokens / (step_pct["median"] * 1e-6), 1),
           "step_us_warm": step_pct, "step_us_cold": cold_pct,
           "step_us_mean_warm": round(total * 1e3 / steps, 2),
           "fused_minimum_bytes": fused_minimum_bytes(w.prob),
           "launches": {n: dict(stage_record(work, n, us[n], w.prob.dtype),
                                counters=measured_counters(n, w.name.split()[0]))
                        for n in launches},
           "tuning": w.tuning_record}
    del w
    torch.cuda.empty_cache()
    if compare_fused:
        rec["fused_step_us_warm_median"] = fused_step(k, torch, binding, steps, warmup)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="1..6")
    ap.add_argument("--tuning", default=None, metavar="JSON",
                    help='pin kernel choices, e.g. \'{"sp_blocks": 1}\' (default: the tuned '
                         'config, else the library\'s own choice)')
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward (ssd_bwd) on the same workload")
    ap.add_argument("--backward-reps", type=int, default=5)
    ap.add_argument("--side-workloads", default="3,4,5",
                    help="comma-separated other workloads to time after the main one "
                         "('' for none)")
    ap.add_argument("--fused-workloads", default="2,4",
                    help="workloads whose step is also timed with the fused forward pinned")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy a buffer of MIB MiB three times (a plain copy "
                         "kernel of known size, for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_model_ssd_amd import binding

    torch.cuda.init()
    dev = torch.device("cuda:0")
    binding.load_library()
    pinned = json.loads(args.tuning) if args.tuning else None
    w = Workload(args.workload, torch, binding, pinned)
    prob, inp, d = w.prob, w.inp, w.d
    log("[bench] warmup")
    w.capture(args.warmup)
    nchunks = w.nchunks()

    # --- whole step: a HIP graph of one forward, replayed back to back
    log(f"[bench] timing {args.steps} graph replays")
    total_ms, wall = w.time_replays(args.steps)
    ms_per_step = total_ms / args.steps
    per_ms = w.step_samples(20, 5)
    tokens = w.tokens
    value = tokens / (ms_per_step * 1e-3)
    step_pct = {q: round(v * 1e3, 2) for q, v in percentiles(per_ms).items() if q != "n"}

    # --- the same step with cold caches (a 1 GiB write evicts the 256 MB
    # last-level cache before each replay; only the replay is timed), and
    # what a plain device copy sustains on this GPU
    log("[bench] cold-cache steps and copy bandwidth")
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    cold = w.time_cold(20, flush, w.graph.replay)
    cold_pct = {q: round(v * 1e3, 2) for q, v in percentiles(cold).items() if q != "n"}
    dst = torch.empty_like(flush)
    dst.copy_(flush)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(flush)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * flush.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst

    # --- per launch, warm: R back-to-back launches between two events
    log("[bench] per-launch timing")
    work = algorithmic_work(prob, nchunks)
    fused = prob.dtype == "bf16"
    step_launches = [n for n in (STEP_LAUNCHES if fused else STAGE_ORDER)
                     if n != "plan" or prob.seq_lens]
    singles_names = [n for n in STAGE_ORDER if n not in step_launches and n != "plan"]
    us = w.time_launches(step_launches + singles_names, args.stage_reps)
    stages = {n: stage_record(work, n, us[n], prob.dtype) for n in step_launches}
    singles = {n: stage_record(work, n, us[n], prob.dtype) for n in singles_names}
    wtag = w.name.split()[0]
    for n in stages:
        stages[n]["counters"] = measured_counters(n, wtag)
    if not torch.equal(w.out, w.ref_out):
        raise RuntimeError("stage-by-stage run differs from the eager forward")
    dom = max(stages, key=lambda k: stages[k]["us"])
    ds = stages[dom]
    # the dominant launch alone after the cache is evicted: what it reads
    # comes from HBM (the stages before it have left their outputs in place)
    masks = w.masks()
    cold_dom = w.time_cold(20, flush, lambda: w.step(masks[dom]))
    cold_dom_us = percentiles(cold_dom)["median"] * 1e3
    cold_rec = stage_record(work, dom, cold_dom_us, prob.dtype)
    traffic = measured_traffic(dom, wtag)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": ds["gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ds["hbm_frac"], "traffic": traffic,
                "traffic_unit": "bytes per launch", "launch_us": ds["us"],
                "alg_bytes_per_launch": ds["alg_bytes"], "counters": ds["counters"],
                "cold": {"launch_us_median": round(cold_dom_us, 3), "achieved": cold_rec["gbs"],
                         "frac": cold_rec["hbm_frac"]}}
    total_bytes = sum(work[n][0] for n in step_launches)
    del flush

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # --- the backward on the same inputs: seeded output gradients, R calls
    # between HIP events (the forward's stages 0-4 are recomputed inside)
    backward = None
    if not args.no_backward:
        log("[bench] backward")
        cur = torch.cuda.current_stream()
        gb = torch.Generator().manual_seed(12345)
        dy = torch.randn(inp["x"].shape, generator=gb).to(inp["x"].dtype).to(dev)
        dfin = torch.randn((prob.nseq, prob.nheads, prob.headdim, prob.dstate), generator=gb).to(dev)

        def bstep(wsb=None, after_fwd=False):
            return binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy,
                                   dfin, D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                                   cu_seqlens=d["cu_seqlens"], workspace=wsb, after_fwd=after_fwd)
        wsb = bstep()["workspace"]
        bstep(wsb)
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(20_000_000)
        except Exception:
            pass
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(cur)
        for _ in range(args.backward_reps):
            bstep(wsb)
        b1.record(cur)
        torch.cuda.synchronize()
        bus = b0.elapsed_time(b1) * 1e3 / args.backward_reps
        e = 2 if prob.dtype == "bf16" else 4
        H, P, N, G = prob.nheads, prob.headdim, prob.dstate, prob.ngroups
        # the fused minimum: x, dy read and dx written; dt read and ddt
        # written; B, C read and dB, dC written; init, dfinal read, dinit written
        bbytes = (3 * e * tokens * H * P + 8 * tokens * H + 4 * e * tokens * G * N
                  + 12 * prob.nseq * H * P * N)
        # ssd_bwd_after_fwd: the same gradients from the intermediates a
        # forward call left in the workspace (the training order)
        binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                        dt_bias=d["dt_bias"], initial_states=d["init"], cu_seqlens=d["cu_seqlens"],
                        workspace=wsb, tuning=None)
        bstep(wsb, True)
        torch.cuda.synchronize()
        b0.record(cur)
        for _ in range(args.backward_reps):
            bstep(wsb, True)
        b1.record(cur)
        torch.cuda.synchronize()
        aus = b0.elapsed_time(b1) * 1e3 / args.backward_reps
        backward = {"us": round(bus, 1), "tokens_per_s": round(tokens / (bus * 1e-6), 1),
                    "alg_bytes_fused_minimum": int(bbytes),
                    "hbm_frac_of_fused_minimum": round(bbytes / (bus * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
                    "us_after_fwd": round(aus, 1),
                    "reps": args.backward_reps,
                    "note": "ssd_bwd: gradients of every input; recomputes the forward's "
                            "stages 0-4 (us_after_fwd: ssd_bwd_after_fwd, which reuses a "
                            "forward's intermediates); per-kernel times in profiles/"}
        del wsb, dy, dfin
    log("[bench] gated norm")
    gnorm = gated_norm_record(w, torch, binding, max(5, args.stage_reps // 5))
    main_tuning = w.tuning_record
    del w
    torch.cuda.empty_cache()

    # --- the fused forward (ssd_tuning_t.fused = 2) on the main workload
    fused_list = [v.strip() for v in args.fused_workloads.split(",") if v.strip()]
    fused_main = None
    if str(args.workload) in fused_list and pinned is None:
        log("[bench] fused forward")
        fused_main = fused_step(args.workload, torch, binding, 20, 3)

    # --- the other full-size workloads: warm and cold step, per launch
    side = {}
    for k in [int(v) for v in args.side_workloads.split(",") if v.strip()]:
        if k == args.workload:
            continue
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        side[str(k)] = side_workload(k, torch, binding, flush, steps=20,
                                     warmup=3, reps=max(5, args.stage_reps // 5),
                                     compare_fused=str(k) in fused_list)
        del flush
        torch.cuda.empty_cache()

    # --- CPU baseline: the fp64 oracle on this host's cores, same workload
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        from oracle.recurrence import ssd_recurrence, max_threads
        heads = list(range(prob.nheads))
        reps, t_cpu = 0, 0.0
        while reps < 1 or (t_cpu < args.cpu_seconds and reps < 10000):
            c0 = time.perf_counter()
            ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                           inp["D"], init=inp["init"], cu_seqlens=inp["cu_seqlens"], heads=heads)
            t_cpu += time.perf_counter() - c0
            reps += 1
        cpu = {"value": round(tokens * reps / t_cpu, 1), "unit": "tokens/s",
               "cores": max_threads(), "kind": "oracle",
               "sample": f"whole workload ({tokens} tokens x {prob.nheads} heads) repeated "
                         f"{reps} time(s), {t_cpu:.1f} s, each including the fp64 upcast"}

    from state_space_model_ssd_amd.inputs import WORKLOAD_NAMES
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": prob.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "batch": prob.batch,
                   "seqlen": prob.seqlen, "nheads": prob.nheads, "headdim": prob.headdim,
                   "dstate": prob.dstate, "ngroups": prob.ngroups,
                   "chunk_size": prob.chunk_size, "tokens": tokens, "chunks": nchunks},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_us_warm": step_pct,
        "step_us_cold": cold_pct,
        "tokens_per_s_median": round(tokens / (step_pct["median"] * 1e-6), 1),
        "fused_step_us_warm_median": fused_main,
        "gated_norm": gnorm,
        "tuning": main_tuning,
        "stages": stages,
        "stages_unfused": singles,
        "backward": backward,
        "step_alg_bytes": int(total_bytes),
        "step_alg_gbs": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "fused_minimum_bytes": fused_minimum_bytes(prob),
        "workloads": side,
        "timing": "value: tokens over the mean of K HIP-graph replays back to back between "
                  "two HIP events (warm caches); step_us_warm: median/p10/p90 over 20 "
                  "samples, each the mean of 5 replays back to back between two events; "
                  "cold: each replay (or launch) alone after a "
                  "1 GiB write evicts the last-level cache; per launch: "
                  f"{args.stage_reps} back-to-back launches between HIP events; 'stages' are "
                  "the launches of one step, 'stages_unfused' the stages a fused launch "
                  "covers, run alone",
        "wall_s_timed_region": round(wall, 4),
        "context": {"device_copy_gbs": round(copy_gbs, 1),
                    "note": "copy: torch device-to-device copy of 1 GiB, read + write bytes "
                            "(measured, not the roofline peak)"},
        "env": env_info(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
