"""Throughput of the SSD chunked-scan forward on one MI355X.

One step = one pass of the whole forward (plan, chunk_cumsum, bmm_chunk,
chunk_state, state_passing, chunk_scan) over one batch of synthetic input
already resident in HBM.  Default workload: the Mamba-2 layer shape (batch 2,
seqlen 4096, 24 heads, headdim 64, dstate 128, 1 group, chunk 256, bf16
x/B/C, fp32 accumulation).

Prints ONE JSON line.  `value` is tokens/s of back-to-back steps replayed
from a HIP graph; `roofline` covers the slowest stage, timed live with HIP
events on the stream its kernel runs on; `cpu_baseline` is the fp64 CPU
oracle timed on this host's cores on the same workload.
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


STAGE_SOURCE = {"plan": "ssd_prep.hip", "chunk_cumsum": "ssd_prep.hip", "front": "ssd_chunk_state.hip",
                "bmm_chunk": "ssd_bmm.hip", "chunk_state": "ssd_chunk_state.hip",
                "state_passing": "ssd_state_passing.hip", "chunk_scan": "ssd_chunk_scan.hip"}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and blank space removed) of a kernel's
    source file and of the headers every kernel includes."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "state_space_model_ssd_amd", "csrc")
    h = hashlib.sha256()
    for f in (STAGE_SOURCE[kernel], "ssd_common.h", "ssd_device.h", "ssd_kernels.h"):
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
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = kernel_source_hash(kernel)
    if fields.get("kernel_source_sha256_16") != sha:
        return None
    return int(fields["traffic_bytes_per_launch"])


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
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
    from state_space_model_ssd_amd.inputs import workload_inputs, WORKLOAD_NAMES

    torch.cuda.init()
    dev = torch.device("cuda:0")
    binding.load_library()
    log(f"[bench] workload {args.workload}: drawing inputs")
    prob, inp = workload_inputs(args.workload)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cprob = binding.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate,
                                 prob.ngroups, prob.chunk_size, 1 if prob.dtype == "bf16" else 0,
                                 nseq=len(prob.seq_lens) if prob.seq_lens else 0)
    lay = binding.workspace_layout(cprob)
    from state_space_model_ssd_amd import tuning
    pinned = json.loads(args.tuning) if args.tuning else None
    tuned = pinned if pinned is not None else tuning.lookup(cprob)
    tune_arg = pinned if pinned is not None else "config"   # the binding's own lookup
    ws = torch.empty(lay.total_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["x"])
    fin = torch.empty((prob.nseq, prob.nheads, prob.headdim, prob.dstate), dtype=torch.float32,
                      device=dev)

    def step(stages=binding.STAGE_ALL):
        binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                        dt_bias=d["dt_bias"], initial_states=d["init"],
                        cu_seqlens=d["cu_seqlens"], out=out, final_states=fin, workspace=ws,
                        stages=stages, tuning=tune_arg)

    log("[bench] warmup")
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    nchunks = int(binding.intermediates(ws, cprob)["seq_chunks"][-1].item()) \
        if prob.seq_lens else lay.max_chunks
    ref_out = out.clone()

    # --- whole step: a HIP graph of one forward, replayed back to back
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step()                       # settle on the side stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref_out):
        raise RuntimeError("graph replay differs from the eager forward")
    log(f"[bench] timing {args.steps} graph replays")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    tokens = prob.batch * prob.seqlen
    value = tokens / (ms_per_step * 1e-3)

    # --- context: the same step with cold caches (a 1 GiB write evicts the
    # 256 MB last-level cache before each replay; only the replay is timed),
    # and what a plain device copy sustains on this GPU
    log("[bench] cold-cache steps and copy bandwidth")
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(10):
        flush.fill_(1.0)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        graph.replay()
        c1.record()
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    ms_cold = sorted(cold)[len(cold) // 2]
    src = flush
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del flush, src, dst

    # --- per stage: R back-to-back launches between two events on the
    # launch stream, queued behind a GPU sleep so the CPU is never the limit
    log("[bench] per-stage timing")
    work = algorithmic_work(prob, nchunks)
    R = args.stage_reps
    stages, singles = {}, {}
    cur = torch.cuda.current_stream()
    fused = prob.dtype == "bf16"
    step_launches = STEP_LAUNCHES if fused else STAGE_ORDER
    masks = dict(binding.STAGES)
    masks["front"] = binding.STAGES["chunk_cumsum"] | binding.STAGES["bmm_chunk"] | \
        binding.STAGES["chunk_state"]
    names = list(step_launches) + ([n for n in STAGE_ORDER if n not in step_launches])
    for name in names:
        if name == "plan" and not prob.seq_lens:
            continue
        bit = masks[name]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(20_000_000)
        except Exception:
            pass
        e0.record(cur)
        for _ in range(R):
            step(bit)
        e1.record(cur)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / R
        nbytes, flops = work[name]
        rec = {"us": round(us, 3), "alg_bytes": int(nbytes),
               "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
               "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if flops:
            peak = BF16_PEAK_TFLOPS if prob.dtype == "bf16" else F32_PEAK_TFLOPS
            rec["tflops"] = round(flops / (us * 1e-6) / 1e12, 2)
            rec["mfma_frac"] = round(flops / (us * 1e-6) / 1e12 / peak, 4)
        (stages if name in step_launches else singles)[name] = rec
    if not torch.equal(out, ref_out):
        raise RuntimeError("stage-by-stage run differs from the eager forward")
    dom = max(stages, key=lambda k: stages[k]["us"])
    ds = stages[dom]
    wtag = WORKLOAD_NAMES[args.workload].split()[0]
    traffic = measured_traffic(dom, wtag)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": ds["gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ds["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch", "launch_us": ds["us"],
                "alg_bytes_per_launch": ds["alg_bytes"]}
    total_bytes = sum(work[n][0] for n in step_launches if n in work and
                      (n != "plan" or prob.seq_lens))

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
        gb = torch.Generator().manual_seed(12345)
        dy = torch.randn(inp["x"].shape, generator=gb).to(inp["x"].dtype).to(dev)
        dfin = torch.randn((prob.nseq, prob.nheads, prob.headdim, prob.dstate), generator=gb).to(dev)

        def bstep(wsb=None):
            return binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy,
                                   dfin, D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                                   cu_seqlens=d["cu_seqlens"], workspace=wsb)
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

        def astep():
            return binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy,
                                   dfin, D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                                   cu_seqlens=d["cu_seqlens"], workspace=wsb, after_fwd=True)
        astep()
        torch.cuda.synchronize()
        b0.record(cur)
        for _ in range(args.backward_reps):
            astep()
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
        del wsb

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
        "tuning": {"source": "pinned" if pinned is not None else
                   "tuned config" if tuned else "library's own choice",
                   "key": tuning.shape_key(cprob), "choice": tuned or {}},
        "stages": stages,
        "stages_unfused": singles,
        "backward": backward,
        "step_alg_bytes": int(total_bytes),
        "step_alg_gbs": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "timing": "HIP-graph replays back to back (warm caches); per launch: "
                  f"{R} back-to-back launches between HIP events; 'stages' are the launches "
                  "of one step, 'stages_unfused' the stages a fused launch covers, run alone",
        "wall_s_timed_region": round(wall, 4),
        "context": {"ms_per_step_cold_cache": round(ms_cold, 5),
                    "tokens_per_s_cold_cache": round(tokens / (ms_cold * 1e-3), 1),
                    "device_copy_gbs": round(copy_gbs, 1),
                    "note": "cold: median of 10 replays, each after a 1 GiB write that evicts "
                            "the last-level cache; copy: torch device-to-device copy of 1 GiB, "
                            "read + write bytes (measured, not the roofline peak)"},
        "env": env_info(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
