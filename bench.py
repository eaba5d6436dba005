#!/usr/bin/env python3
"""Benchmark of the GDN decode hot path on one MI355X.

One step = one gdn_decode_layer call (conv update, gates, delta-rule state update and
readout, gated RMSNorm) over the whole batch, inputs resident in HBM. The workload is
the Qwen3.5-style layer (H_k = 16, H_v = 32, d_k = d_v = 128, K = 4, bf16 activations,
fp32 state) at B = 512: its 1 GiB of state exceeds the 256 MB Infinity Cache, so the
bandwidth figure is a cold-HBM one. 32 distinct steps of inputs are drawn and reused
cyclically; the state keeps evolving. B = 1 and B = 64 are reported in "sweep" (each
step called from the host, for B = 1 also with the binding's per-call tensor checks
off, 64 steps captured in one HIP graph and replayed, and for B = 64 single steps with
the caches flushed), the B = 8 x T = 4096 multi-token call in
"sequence", speculative verification (B = 64, 4 draft tokens) in "verify", the
projections around the layer in "proj"; each leg carries a roofline block. The
bandwidth reference is the benchmark's own streaming copy (libgdn_bench.so), and
"cpu_baseline" times the fp64 oracle on the host cores beside each leg.

Prints one JSON line. `value` = sequences x steps / second (seq-layer steps/s).
The roofline figure uses algorithmic bytes (state read once and written once, every
input read once, output written once) over the kernel's average duration, timed
with HIP events on the stream the kernel is launched on.

    python bench.py [--steps K] [--warmup W] [--no-sweep] [--no-cpu-baseline]
    python bench.py --copy-calibration     # streaming copy of known size (PMC scaling)
    python bench.py --summarize DIR        # summarise rocprofv3 CSV output in DIR
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN decode steps/s (seq·layer) at B=1/64/512 + achieved HBM GB/s vs peak"
UNIT = "seq·layer steps/s"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix peak of MI355X
# sources the decode kernel is built from (the traffic record is keyed on them)
KERNEL_SRCS = [os.path.join(ROOT, "gated_deltanet_linear_causal_amd", "csrc", f)
               for f in ("gdn_kernels.hip", "gdn_device.h", "gdn_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gdn_decode_fused_B512_traffic.txt")


def algorithmic_bytes(cfg, T=1) -> int:
    """Bytes one call must move: per sequence the fp32 state read and written once,
    the conv state read and rolled, qkv / z / a / b of each token read, the output
    written (fp32); plus the shared conv taps, A_log, dt_bias and norm weight."""
    ea = 2 if cfg.act_dtype == "bf16" else 4
    Hv, dk, dv, K, C = cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim, cfg.conv_kernel, cfg.channels
    per_seq = 2 * Hv * dk * dv * 4 + 2 * (K - 1) * C * ea
    per_tok = C * ea + Hv * dv * ea + 2 * Hv * ea + Hv * dv * 4
    shared = C * K * ea + 2 * Hv * 4 + dv * 4
    return cfg.batch * (per_seq + T * per_tok) + shared


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed PMC summary, only if the counters were
    taken on the current kernel source (else None)."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    kv = dict(ln.split(":", 1) for ln in lines if ln and not ln.startswith("#") and ":" in ln)
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_inputs(cfg, steps, torch):
    import numpy as np
    from gated_deltanet_linear_causal_amd import inputs as I
    data = I.generate(cfg, steps=steps)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    d = {k: dev(v) for k, v in data.items()}
    return data, d


def time_decode(cfg, d, steps, warmup, torch, gdn, validate=True):
    """Average seconds per gdn_decode_layer launch over `steps` timed launches. The
    per-step input views are taken before the timed loop; validate=False skips the
    binding's per-call tensor checks (the buffers are the same on every call)."""
    s = gdn.make_shape(cfg.batch, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                       cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps, cfg.act_dtype, "f32")
    nin = d["qkv"].shape[0]
    out = torch.empty((cfg.batch, cfg.z_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    views = [(d["qkv"][j], d["a"][j], d["b"][j], d["z"][j]) for j in range(nin)]

    def step(i):
        qkv, a, b, z = views[i % nin]
        gdn.gdn_decode_layer(s, d["conv_state"], d["state"], qkv, d["conv_w"], a, b, z, d["A_log"], d["dt_bias"],
                             d["norm_w"], out, stream=stream, validate=validate)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def time_decode_cold(cfg, d, steps, torch, gdn, flush_bytes=512 << 20):
    """Average seconds per gdn_decode_layer launch with the caches cold: before each step
    the benchmark's streaming copy moves flush_bytes through L2 and the Infinity Cache
    with the default policy (evicting the state), and only the step itself is timed
    (HIP events around it)."""
    lib = bench_library()
    s = gdn.make_shape(cfg.batch, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                       cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps, cfg.act_dtype, "f32")
    nin = d["qkv"].shape[0]
    out = torch.empty((cfg.batch, cfg.z_dim), dtype=torch.float32, device="cuda")
    src = torch.zeros(flush_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    total = 0.0
    for i in range(steps + 2):
        if lib.gdn_bench_stream_copy(src.data_ptr(), dst.data_ptr(), flush_bytes, 0, stream.cuda_stream) != 0:
            raise RuntimeError("gdn_bench_stream_copy failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        j = i % nin
        e0.record(stream)
        gdn.gdn_decode_layer(s, d["conv_state"], d["state"], d["qkv"][j], d["conv_w"], d["a"][j], d["b"][j],
                             d["z"][j], d["A_log"], d["dt_bias"], d["norm_w"], out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:  # the first two are warm-up
            total += e0.elapsed_time(e1) / 1e3
    del src, dst
    return total / steps


def time_decode_graph(cfg, d, steps, torch, gdn, replays=5):
    """Average seconds per gdn_decode_layer step when `steps` consecutive steps are
    captured in one HIP graph and replayed: the device time of a step without the
    host's per-call launch cost (which bounds small batches when called one by one)."""
    s = gdn.make_shape(cfg.batch, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                       cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps, cfg.act_dtype, "f32")
    nin = d["qkv"].shape[0]
    out = torch.empty((cfg.batch, cfg.z_dim), dtype=torch.float32, device="cuda")

    def step(i, st):
        j = i % nin
        gdn.gdn_decode_layer(s, d["conv_state"], d["state"], d["qkv"][j], d["conv_w"], d["a"][j], d["b"][j],
                             d["z"][j], d["A_log"], d["dt_bias"], d["norm_w"], out, stream=st)

    side = torch.cuda.Stream()  # warm-up off the default stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(4):
            step(i, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for i in range(steps):
            step(i, st)
    g.replay()  # untimed
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / 1e3 / (replays * steps)


def time_pooled(cfg, d, pool, steps, warmup, torch, gdn):
    """gdn_decode_layer_pooled: the batch's states are B distinct random slots of a
    pool of `pool` states (the batch's own states are copied into those slots)."""
    g = torch.Generator(device="cpu").manual_seed(7)
    slots = torch.randperm(pool, generator=g)[:cfg.batch].to(torch.int32).cuda()
    st_pool = torch.zeros((pool,) + tuple(d["state"].shape[1:]), dtype=torch.float32, device="cuda")
    cs_pool = torch.zeros((pool,) + tuple(d["conv_state"].shape[1:]), dtype=d["conv_state"].dtype, device="cuda")
    st_pool[slots.long()] = d["state"]
    cs_pool[slots.long()] = d["conv_state"]
    s = gdn.make_shape(cfg.batch, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                       cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps, cfg.act_dtype, "f32")
    nin = d["qkv"].shape[0]
    out = torch.empty((cfg.batch, cfg.z_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % nin
        gdn.gdn_decode_layer_pooled(s, slots, cs_pool, st_pool, d["qkv"][j], d["conv_w"], d["a"][j], d["b"][j],
                                    d["z"][j], d["A_log"], d["dt_bias"], d["norm_w"], out, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    del st_pool, cs_pool
    return e0.elapsed_time(e1) / 1e3 / steps


def time_sequence(cfg, d, reps, torch, gdn):
    s = gdn.make_shape(cfg.batch, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                       cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps, cfg.act_dtype, "f32")
    out = torch.empty((cfg.batch, cfg.steps, cfg.z_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ws_bytes = gdn.gdn_sequence_workspace_bytes(s, cfg.steps)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None

    def run():
        gdn.gdn_sequence(s, cfg.steps, d["conv_state"], d["state"], d["qkv"], d["conv_w"], d["a"], d["b"], d["z"],
                         d["A_log"], d["dt_bias"], d["norm_w"], out, workspace=ws, stream=stream)

    for _ in range(20):  # untimed: the clock settles over the first calls
        run()
    torch.cuda.synchronize()
    # median of batches of `reps` calls (single calls of this kernel vary by up to ~30 %
    # from call to call on a busy clock)
    batches = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        batches.append(e0.elapsed_time(e1) / 1e3 / reps)
    return sorted(batches)[len(batches) // 2]


def chunk_flops(cfg, C=32):
    """Useful flops of the chunked form per chunk and v-head (d = d_k = d_v): K K^T and
    Q K^T (2 C^2 d each), K H0 and Q H0 (2 C d^2 each), P Delta (2 C^2 d) and K^T E Delta
    (2 C d^2). The kernel evaluates each product as three fp16 MFMAs (split operands)."""
    d = cfg.head_k_dim
    return 2 * (2 * C * C * d) + 2 * (2 * C * d * d) + 2 * C * C * d + 2 * C * d * d


def time_events(fn, reps, torch, warmup=3):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def time_verify(cfg, T, reps, torch, gdn):
    """gdn_decode_verify of T draft tokens per sequence, then gdn_decode_commit of all
    T (the commit's worst case: every state rewritten)."""
    from gated_deltanet_linear_causal_amd import inputs as I
    c = cfg.with_(mode="sequence", steps=T)
    _, d = build_inputs(c, T, torch)
    s = gdn.make_shape(c.batch, c.num_k_heads, c.num_v_heads, c.head_k_dim, c.head_v_dim, c.conv_kernel,
                       c.l2_eps, c.rms_eps, c.act_dtype, "f32")
    out = torch.empty((c.batch, T, c.z_dim), dtype=torch.float32, device="cuda")
    trail = torch.empty(gdn.gdn_verify_trail_bytes(s, T), dtype=torch.uint8, device="cuda")
    acc = torch.full((c.batch,), T, dtype=torch.int32, device="cuda")

    def verify(st):
        gdn.gdn_decode_verify(s, T, d["conv_state"], d["state"], d["qkv"], d["conv_w"], d["a"], d["b"], d["z"],
                              d["A_log"], d["dt_bias"], d["norm_w"], out, trail, stream=st)

    def commit(st):
        gdn.gdn_decode_commit(s, T, acc, d["conv_state"], d["state"], d["qkv"], trail, stream=st)

    vsec = time_events(verify, reps, torch)
    csec = time_events(commit, reps, torch)
    B, Hk, Hv, dk, dv, K, C = c.batch, c.num_k_heads, c.num_v_heads, c.head_k_dim, c.head_v_dim, c.conv_kernel, c.channels
    trail_b = 4 * B * T * (Hv * dv + Hk * dk + Hv)
    vbytes = B * (Hv * dk * dv * 4 + (K - 1) * C * 2 + T * (C * 2 + Hv * dv * 2 + 2 * Hv * 2 + Hv * dv * 4)) + trail_b
    cbytes = B * (2 * Hv * dk * dv * 4 + 2 * (K - 1) * C * 2 + min(T, K - 1) * C * 2) + trail_b
    del d, out, trail
    return {"workload": "B=%d, T=%d draft tokens: gdn_decode_verify, then gdn_decode_commit of all T" % (B, T),
            "verify_us": round(vsec * 1e6, 2), "commit_us": round(csec * 1e6, 2),
            "draft_tokens_per_s": round(B * T / vsec, 1),
            "verify_GB_s": round(vbytes / vsec / 1e9, 1), "commit_GB_s": round(cbytes / csec / 1e9, 1),
            "verify_algorithmic_bytes": vbytes, "commit_algorithmic_bytes": cbytes,
            "verify_roofline": roofline_block("hbm", vbytes / vsec / 1e9, HBM_PEAK_GBS, "GB/s"),
            "commit_roofline": roofline_block("hbm", cbytes / csec / 1e9, HBM_PEAK_GBS, "GB/s"),
            "note": "the B=64 states (128 MiB) fit the 256 MB Infinity Cache: effective (cache-assisted) GB/s"}


def time_proj(cfg, B, reps, torch, gdn):
    """gdn_in_proj and gdn_out_proj at batch B (hidden = inputs.HIDDEN), synthetic
    bf16 weights; bytes = weights + x + y, flops = 2 B N K."""
    import numpy as np
    from gated_deltanet_linear_causal_amd import inputs as I
    c = cfg.with_(batch=B)
    H = I.HIDDEN
    P = I.generate_projections(c, H)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    w = {k: dv(v) for k, v in P.items()}
    s = gdn.make_shape(B, c.num_k_heads, c.num_v_heads, c.head_k_dim, c.head_v_dim, c.conv_kernel,
                       c.l2_eps, c.rms_eps, "bf16", "bf16")
    C, Hv, zd = c.channels, c.num_v_heads, c.z_dim
    qkv = torch.empty((B, C), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((B, zd), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((B, Hv), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((B, Hv), dtype=torch.bfloat16, device="cuda")
    gated = torch.randn((B, zd), device="cuda").to(torch.bfloat16)
    y = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")

    def inp(st):
        gdn.gdn_in_proj(s, H, w["x_norm"], w["w_qkv"], w["w_z"], w["w_a"], w["w_b"], qkv, z, a, b, stream=st)

    def outp(st):
        gdn.gdn_out_proj(s, H, gated, w["w_out"], y, stream=st)

    isec = time_events(inp, reps, torch)
    osec = time_events(outp, reps, torch)
    n_in = C + zd + 2 * Hv
    ib = 2 * (n_in * H + B * H + B * n_in)
    ob = 2 * (H * zd + B * zd + B * H)
    res = {}
    for name, sec, nb, fl in (("in_proj", isec, ib, 2 * B * n_in * H), ("out_proj", osec, ob, 2 * B * H * zd)):
        # the binding roof: HBM when the bytes take longer at peak than the flops
        hbm_bound = nb / (HBM_PEAK_GBS * 1e9) >= fl / (MFMA_PEAK_TFLOPS * 1e12)
        res[name] = {"us": round(sec * 1e6, 2), "GB_s": round(nb / sec / 1e9, 1),
                     "hbm_frac": round(nb / sec / 1e9 / HBM_PEAK_GBS, 4), "TFLOP_s": round(fl / sec / 1e12, 2),
                     "mfma_frac": round(fl / sec / 1e12 / MFMA_PEAK_TFLOPS, 4), "algorithmic_bytes": nb, "flops": fl,
                     "roofline": (roofline_block("hbm", nb / sec / 1e9, HBM_PEAK_GBS, "GB/s") if hbm_bound else
                                  roofline_block("mfma", fl / sec / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s"))}
    del w, qkv, z, a, b, gated, y
    return res


def cpu_info():
    """Host CPU model (from /proc/cpuinfo), logical CPUs and the CPUs this process may use."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def time_oracle(cfg, data, nseq, steps, target_s):
    """Seconds per run of the fp64 oracle over the first `nseq` sequences and `steps`
    tokens of `data` (decode inputs [S][B][...] or sequence inputs [B][T][...]), from the
    initial states; the run is repeated until about target_s has been measured.
    Returns (seconds per run, runs)."""
    import numpy as np
    from gated_deltanet_linear_causal_amd import inputs as I
    from oracle import oracle as O
    idx = np.arange(nseq)
    s = O.shape_of(cfg, batch=nseq)
    if cfg.mode == "sequence":
        sl = lambda k: np.ascontiguousarray(I.widen(data[k][idx, :steps], cfg.act_dtype))
    else:
        sl = lambda k: np.ascontiguousarray(np.swapaxes(I.widen(data[k][:steps][:, idx], cfg.act_dtype), 0, 1))
    args = (sl("qkv"), I.widen(data["conv_w"], cfg.act_dtype), sl("a"), sl("b"), sl("z"))
    cs0 = I.widen(data["conv_state"][idx], cfg.act_dtype).astype(np.float64)
    st0 = data["state"][idx].astype(np.float64)
    total, runs = 0.0, 0
    while total < target_s:
        cs, st = cs0.copy(), st0.copy()
        t0 = time.perf_counter()
        O.sequence(s, steps, cs, st, args[0], args[1], args[2], args[3], args[4], data["A_log"], data["dt_bias"],
                   data["norm_w"])
        total += time.perf_counter() - t0
        runs += 1
    return total / runs, runs


def cpu_baseline(cfg, data, seq_cfg=None, seq_data=None, target_s=8.0):
    """The fp64 oracle, as it is, on the GPU machine's host cores, in the units of the GPU
    figures and on bounded samples of the same workloads (about 20 s of CPU time).
    Headline: the B = 512 decode workload (seq-layer steps/s), all usable cores. Also:
    the same with one thread; B = 1, one step (seq-layer steps/s); B = 64, its 32 steps;
    and the B = 8 x T = 4096 sequence (tokens/s), on a sample of its sequences and
    tokens."""
    from gated_deltanet_linear_causal_amd import inputs as I
    from oracle import oracle as O
    info = cpu_info()
    threads = O.threads(info["usable_cpus"] or 1)
    S = data["qkv"].shape[0]
    # headline: grow the sample of B = 512 sequences until one run takes >= 1 s
    n = 8
    while True:
        sec, runs = time_oracle(cfg, data, n, S, target_s / 8)
        if sec >= 1.0 or n >= cfg.batch:
            break
        n = min(cfg.batch, n * 4)
    sec, runs = time_oracle(cfg, data, n, S, target_s)
    res = {"value": n * S / sec, "unit": UNIT, "cores": threads, "kind": "oracle",
           "sample": "first %d of the %d sequences x %d decode steps of the B=512 workload's inputs, run %d time(s) "
                     "from the initial states, fp64 C oracle (OpenMP over sequence x k-head units) on %d threads, "
                     "%.1f s" % (n, cfg.batch, S, runs, threads, sec * runs)}
    res.update(info)
    legs = {}
    O.threads(1)
    sec1, runs1 = time_oracle(cfg, data, 8, S, target_s / 4)
    legs["B512_1_thread"] = {"steps_per_s": round(8 * S / sec1, 1), "threads": 1,
                             "sample": "8 sequences x %d steps, %d run(s)" % (S, runs1)}
    O.threads(threads)
    for i, name in ((1, "B1"), (2, "B64")):
        c = I.config(i)
        d = I.generate(c)
        sec_c, runs_c = time_oracle(c, d, c.batch, c.steps, target_s / 8)
        legs[name] = {"steps_per_s": round(c.batch * c.steps / sec_c, 1), "threads": threads,
                      "sample": "all %d sequence(s) x %d step(s), %d run(s)" % (c.batch, c.steps, runs_c)}
    if seq_cfg is not None:
        T = min(seq_cfg.steps, 512)
        sec_s, runs_s = time_oracle(seq_cfg, seq_data, seq_cfg.batch, T, target_s / 4)
        legs["B8_T4096"] = {"tokens_per_s": round(seq_cfg.batch * T / sec_s, 1), "threads": threads,
                            "sample": "all %d sequences, first %d of the %d tokens, %d run(s)"
                                      % (seq_cfg.batch, T, seq_cfg.steps, runs_s)}
    res["legs"] = legs
    return res


def bench_library():
    """The benchmark's own streaming-copy library (libgdn_bench.so, built with libgdn.so)."""
    import ctypes
    path = os.path.join(ROOT, "gated_deltanet_linear_causal_amd", "libgdn_bench.so")
    if not os.path.exists(path):
        raise RuntimeError("libgdn_bench.so is not built; run `python -m gated_deltanet_linear_causal_amd.build`")
    lib = ctypes.CDLL(path)
    lib.gdn_bench_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.gdn_bench_stream_copy.restype = ctypes.c_int
    return lib


def copy_bandwidth(torch, nbytes=1 << 30, reps=20):
    """Achievable-bandwidth reference: the streaming copy of `nbytes` (read + write
    counted) with 128-bit buffer loads and stores, the access path of the decode kernel,
    with the non-temporal and with the default cache policy; GB/s of each, HIP events."""
    lib = bench_library()
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    res = {}
    for name, nt in (("nt", 1), ("default", 0)):
        def run():
            rc = lib.gdn_bench_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, nt, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("gdn_bench_stream_copy failed (%d)" % rc)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = 2 * nbytes / (e0.elapsed_time(e1) / 1e3 / reps) / 1e9
    assert torch.equal(src, dst)
    del src, dst
    return res


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A streaming copy of known size (nt policy) for scaling the PMC traffic counters."""
    lib = bench_library()
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        if lib.gdn_bench_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, 1, stream.cuda_stream) != 0:
            raise RuntimeError("gdn_bench_stream_copy failed")
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                      "reps": reps, "kernel": "stream_copy<2> (nt)"}))


def roofline_block(bound, achieved, peak, unit):
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4)}


def summarize(path):
    """Per-kernel summary of rocprofv3 CSV output found under `path`."""
    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        print("==", os.path.relpath(f, path))
        for row in csv.DictReader(open(f)):
            print("%-70.70s calls %6s  avg %10.1f us  min %10.1f us  max %10.1f us  %5.1f%%" % (
                row["Name"], row["Calls"], float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3,
                float(row["MaxNs"]) / 1e3, float(row["Percentage"])))
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        print("==", os.path.relpath(f, path))
        acc = {}
        for row in csv.DictReader(open(f)):
            key = (row.get("Kernel_Name", row.get("Kernel-Name", "?"))[:70], row["Counter_Name"])
            acc.setdefault(key, []).append(float(row["Counter_Value"]))
        for (k, c), v in sorted(acc.items()):
            print("%-70.70s %-12s dispatches %5d  mean %14.1f" % (k, c, len(v), sum(v) / len(v)))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-sweep", action="store_true", help="skip the B=1 / B=64 / sequence figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the GDN core shards "
              "by sequence and k-head with no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from gated_deltanet_linear_causal_amd import gdn
    from gated_deltanet_linear_causal_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    gdn.library()  # fail loudly if the HIP library is missing
    if args.copy_calibration:
        copy_calibration(torch)
        return 0

    cfg = I.config(3)  # B = 512
    data, d = build_inputs(cfg, 32, torch)
    sec = time_decode(cfg, d, args.steps, args.warmup, torch, gdn)
    nbytes = algorithmic_bytes(cfg)
    gbs = nbytes / sec / 1e9
    value = cfg.batch / sec
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded; recipe in inputs.py)",
        "config": {"workload": "GDN decode, Qwen3.5-style layer, B=512", "batch": cfg.batch,
                   "num_k_heads": cfg.num_k_heads, "num_v_heads": cfg.num_v_heads, "head_k_dim": cfg.head_k_dim,
                   "head_v_dim": cfg.head_v_dim, "conv_kernel": cfg.conv_kernel,
                   "activations": "bf16", "state": "fp32", "output": "fp32", "distinct_step_inputs": 32},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(),
                     "kernel": "gdn_step_fast<128, 2, fused, bf16, K=4>", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(sec * 1e6, 2)},
    }
    if not args.no_sweep:
        pool = 2 * cfg.batch
        psec = time_pooled(cfg, d, pool, args.steps, args.warmup, torch, gdn)
        result["pooled"] = {"workload": "B=512 active sequences in random distinct slots of a %d-state pool" % pool,
                            "us_per_step": round(psec * 1e6, 2), "steps_per_s": round(cfg.batch / psec, 1),
                            "GB_s": round(nbytes / psec / 1e9, 1), "frac": round(nbytes / psec / 1e9 / HBM_PEAK_GBS, 4)}
    del d
    torch.cuda.empty_cache()
    if not args.no_sweep:
        sweep = {}
        for i in (1, 2):
            c = I.config(i)
            _, dd = build_inputs(c, 32, torch)
            ssec = time_decode(c, dd, max(args.steps, 200), args.warmup, torch, gdn)
            b = algorithmic_bytes(c)
            gsec = time_decode_graph(c, dd, 64, torch, gdn)
            sweep["B%d" % c.batch] = {"steps_per_s": round(c.batch / ssec, 1), "us_per_step": round(ssec * 1e6, 2),
                                      "GB_s": round(b / ssec / 1e9, 1), "frac": round(b / ssec / 1e9 / HBM_PEAK_GBS, 4),
                                      "graph_us_per_step": round(gsec * 1e6, 2),
                                      "graph_GB_s": round(b / gsec / 1e9, 1)}
            if c.batch == 1:
                usec = time_decode(c, dd, max(args.steps, 200), args.warmup, torch, gdn, validate=False)
                sweep["B1"]["unchecked_us_per_step"] = round(usec * 1e6, 2)
                sweep["B1"]["note"] = ("launch-latency bound; graph_us_per_step is the device time per step; "
                                       "unchecked_us_per_step calls the binding with validate=False (no per-call "
                                       "tensor checks in Python)")
            elif c.batch * c.num_v_heads * c.head_k_dim * c.head_v_dim * 4 <= (256 << 20):
                csec = time_decode_cold(c, dd, 20, torch, gdn)
                sweep["B%d" % c.batch].update({
                    "cold_us_per_step": round(csec * 1e6, 2), "cold_GB_s": round(b / csec / 1e9, 1),
                    "cold_frac": round(b / csec / 1e9 / HBM_PEAK_GBS, 4),
                    "note": "us_per_step / GB_s are effective (cache-assisted): the state fits the 256 MB Infinity "
                            "Cache; cold_* times single steps after a 512 MiB streaming copy evicted it"})
            del dd
        result["sweep"] = sweep
        torch.cuda.empty_cache()
        cb = copy_bandwidth(torch)
        result["roofline"]["copy_GB_s"] = round(max(cb.values()), 1)
        result["roofline"]["copy_nt_GB_s"] = round(cb["nt"], 1)
        result["roofline"]["copy_default_GB_s"] = round(cb["default"], 1)
        c = I.config(4)
        seq_cfg = c
        seq_data, dd = build_inputs(c, c.steps, torch)
        ssec = time_sequence(c, dd, 20, torch, gdn)
        b = algorithmic_bytes(c, T=c.steps)
        fl = chunk_flops(c) * ((c.steps + 31) // 32) * c.batch * c.num_v_heads
        result["sequence"] = {"workload": "B=8 x T=4096 gdn_sequence (chunked MFMA form, 32-token chunks); "
                                          "median of 5 batches of 20 calls",
                              "ms": round(ssec * 1e3, 3), "tokens_per_s": round(c.batch * c.steps / ssec, 1),
                              "GB_s": round(b / ssec / 1e9, 1), "hbm_frac": round(b / ssec / 1e9 / HBM_PEAK_GBS, 4),
                              "useful_TFLOP_s": round(fl / ssec / 1e12, 2),
                              "mfma_issued_TFLOP_s": round(3 * fl / ssec / 1e12, 2),
                              "mfma_frac": round(3 * fl / ssec / 1e12 / MFMA_PEAK_TFLOPS, 4),
                              "algorithmic_bytes": b,
                              # the bytes at peak (173 us) take longer than the issued fp16 products
                              # at peak (155 us): HBM is the binding roof
                              "roofline": roofline_block("hbm", b / ssec / 1e9, HBM_PEAK_GBS, "GB/s")}
        del dd
        torch.cuda.empty_cache()
        result["verify"] = time_verify(I.config(2), 4, 50, torch, gdn)
        torch.cuda.empty_cache()
        result["proj"] = {"hidden": I.HIDDEN}
        for B in (1, 64, 512):
            result["proj"]["B%d" % B] = time_proj(I.config(2), B, 50, torch, gdn)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        if args.no_sweep:
            seq_cfg = I.config(4).with_(steps=512)
            seq_data = I.generate(seq_cfg)
        result["cpu_baseline"] = cpu_baseline(cfg, data, seq_cfg, seq_data)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
