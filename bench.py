#!/usr/bin/env python3
"""Throughput of the residual-compression hot path on one MI355X.

One step = rc_compress + rc_decompress over the whole batch of a workload (the
sender's fused residual / compress / error-feedback pass and the receiver's
decode-and-accumulate pass), with every input already resident in HBM. Default
workload: the FLUX-like share, 57 bf16 tensors of 1152 x 3072, 2-bit groups of
128. The other workloads (2:16, video-like 1-bit, both low-rank settings) are
measured the same way and reported under "workloads".

Prints ONE JSON line. `value` = input-activation GB/s of the default workload
(bf16 bytes of a_t per step / wall time per step over the timed steps).
`roofline` = the dominant kernel (the sender kernel) against HBM: algorithmic
bytes per launch / its mean duration from HIP events on the launch stream.
`cpu_baseline` = the single-threaded CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
# kernel-name prefixes (as rocprofv3 reports them) of each workload's sender kernel
SENDER_KERNEL = {
    "flux_q2": "q_compress_kernel<unsigned short, 128, 2,",
    "flux_nm": "nm_compress_kernel<unsigned short,",
    "video_q1": "q_compress_kernel<unsigned short, 64, 1,",
    "tiny_q1": "q_compress_kernel<float, 64, 1,",
}
LR_CONTRACTIONS = {  # (kernel, launches per step) of the bf16 MFMA products, whole-batch launches
    "flux_lr": [("lr_rq_kernel<unsigned short, true, 32>", 1), ("lr_rq_kernel<unsigned short, false, 32>", 1),
                ("lr_rtp_kernel<32, false>", 1), ("lr_rtp_kernel<32, true>", 1)],
    "video_lr": [("lr_rq_kernel<unsigned short, true, 48>", 1), ("lr_rq_kernel<unsigned short, false, 48>", 1),
                 ("lr_rtp_kernel<48, false>", 1), ("lr_rtp_kernel<48, true>", 1)],
}


# Sources a kernel's traffic and duration depend on: its own file, the shared
# device headers, and the host code that lays out the packed stream and drives
# the launches.
COMMON_SOURCES = ("device_common.hpp", "launch.hpp", "plan.cpp")
KERNEL_SOURCES = {"q_": "quant.hip", "nm_": "nm.hip", "lr_": "lowrank.hip", "bs_": "blocksel.hip"}


def _fresh_profile(name, kernel_prefix=None):
    """A committed profile JSON, or None when sources it depends on changed since
    it was taken: every kernel source, or (kernel_prefix) only that kernel's file
    and the common ones."""
    import json as _json
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    data = _json.load(open(path))
    from activation_residual_compression_amd.profsummary import source_hashes
    now, then = source_hashes(), data.get("sources") or {}
    if kernel_prefix is None:
        return data if then == now else None
    own = [f for p, f in KERNEL_SOURCES.items() if kernel_prefix.startswith(p)]
    files = list(COMMON_SOURCES) + own
    if len(own) != 1 or any(f not in now or then.get(f) != now[f] for f in files):
        return None
    return data


def hbm_probe(n, log):
    """Measured HBM ceilings of the path's access patterns (reference kernels) on
    buffers of the default workload's size: a bf16 [n], b and c fp32 [n]."""
    import torch
    from activation_residual_compression_amd import librescomp as rc
    n = n // 8 * 8
    a = torch.zeros(n, dtype=torch.bfloat16, device="cuda:0")
    b = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    c = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    out = {}
    for kind, name, bpe, src in ((rc.RCX_PROBE_COPY, "copy", 8, b), (rc.RCX_PROBE_READ, "read", 4, b),
                                 (rc.RCX_PROBE_WRITE, "write", 4, b),
                                 (rc.RCX_PROBE_SENDER_MIX, "sender_mix", 14, a),
                                 (rc.RCX_PROBE_RECEIVER_RMW, "receiver_rmw", 8, a)):
        dst, aux = (c, b) if kind in (rc.RCX_PROBE_COPY, rc.RCX_PROBE_READ) else (b, c)
        for _ in range(2):
            rc.rcx_hbm_probe(kind, src, dst, aux, n)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            rc.rcx_hbm_probe(kind, src, dst, aux, n)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        out[name] = n * bpe / (ms * 1e6)
    log("[bench] HBM reference kernels on %d elements (GB/s): " % n
        + ", ".join("%s %.0f" % kv for kv in out.items()))
    del a, b, c
    torch.cuda.empty_cache()
    return out


def algorithmic_bytes(scheme, n_elem, in_bytes, group=None, rank=None, rows=None, cols=None, iters=None,
                      batch=None, keep=None):
    """Bytes each call must move at minimum (all tensors): compress and decompress."""
    N = n_elem
    if scheme == "bs":
        # score pass reads a, ahat and the previous activation, writes e and the
        # new previous activation everywhere; the sent fraction of the blocks is
        # copied into the packed stream and written to ahat (and e = 0); the
        # receiver reads the sent blocks and writes them into its state
        frac = keep / (rows // 64)
        return dict(compress=N * (3 * in_bytes + 8) + N * frac * (2 * in_bytes + 8),
                    decompress=N * frac * (in_bytes + 4))
    if scheme == "q1":
        meta = N / 8 + 4 * N / group
    elif scheme == "q2":
        meta = N / 4 + 8 * N / group
    elif scheme == "nm":
        meta = 5 * N / 16
    else:
        meta = None
    if meta is not None:
        return dict(compress=N * (in_bytes + 12) + meta, decompress=meta + 8 * N)
    # low rank: residual + first product (a, ahat in; R out), later products re-read R,
    # reconstruct reads a, ahat and writes ahat, e; receiver reads/writes its state.
    factors = batch * (rows + cols) * rank // 2 + batch * 8 * rank
    compress = N * (in_bytes + 4 + 2) + N * 2 * (2 * iters - 1) + N * (in_bytes + 12) + factors
    return dict(compress=compress, decompress=factors + 8 * N)


def lr_flops(rows, cols, rank, iters, batch):
    """bf16 MFMA flops of the two tall-skinny products per iteration."""
    return batch * iters * 2 * (2.0 * rows * cols * rank)


_FRAMES = {}  # host frames per workload sequence, shared by the schemes measured on it


def _probe_on(kind, a, b, c, n, reps=5):
    import torch
    from activation_residual_compression_amd import librescomp as rc
    for _ in range(2):
        rc.rcx_hbm_probe(kind, a, b, c, n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        rc.rcx_hbm_probe(kind, a, b, c, n)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _r_probe_on(plan, pattern, reps=5):
    """ms per read of a low-rank plan's R in one product's pattern (after two
    untimed reads, so R's lines are clean, as for the later passes)."""
    import torch
    for _ in range(2):
        plan.r_probe(pattern)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        plan.r_probe(pattern)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def exchange_timing(plan, seq, ahat, e, packed, chunks, reps=7):
    """Sender step plus hand-off of the packed stream (rc_compress_send): compress
    alone, copy alone, both in sequence, and the chunked pipeline, to a device
    buffer (stand-in for a peer's receive buffer) and to pinned host memory (a
    PCIe link). Times are medians over `reps` calls after two untimed ones, from
    an event on the compute stream before the call to an event on the copy
    stream after it (the first chunked copies into a fresh pinned buffer can
    take several times longer than later ones)."""
    import torch
    stream = torch.cuda.current_stream()
    cs = torch.cuda.Stream()
    dsts = {"device": torch.empty_like(packed),
            "host": torch.empty(packed.numel(), dtype=torch.uint8, pin_memory=True)}
    out = {}

    def timed(fn):
        fn(0)
        fn(0)
        torch.cuda.synchronize()
        t = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            cs.wait_event(e0)
            fn(i + 1)
            e1.record(cs)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    def compress(i):
        plan.compress(seq[i % len(seq)], ahat, e, packed, stream)
        cs.wait_stream(stream)

    t_c = timed(compress)
    out["compress_ms"] = t_c
    for name, dst in dsts.items():
        def copy(i, dst=dst):
            with torch.cuda.stream(cs):
                dst.copy_(packed, non_blocking=True)

        def serial(i, dst=dst):
            plan.compress(seq[i % len(seq)], ahat, e, packed, stream)
            cs.wait_stream(stream)
            with torch.cuda.stream(cs):
                dst.copy_(packed, non_blocking=True)

        t_x, t_s = timed(copy), timed(serial)
        r = dict(copy_ms=t_x, serial_ms=t_s, copy_GBps=packed.numel() / (t_x * 1e6))
        for ch in chunks:
            def pipe(i, dst=dst, ch=ch):
                plan.compress_send(seq[i % len(seq)], ahat, e, packed, dst, ch, cs, stream)
            t_p = timed(pipe)
            r["pipeline_chunk%d_ms" % ch] = t_p
            # share of the shorter phase hidden by the pipeline (< 0: chunking costs more)
            r["hidden_frac_chunk%d" % ch] = (t_s - t_p) / min(t_c, t_x)
        out[name] = r
    return out


def _ms(x):
    return "-" if x is None else "%.3f" % x


def measure(config, steps, warmup, max_frames, log, exchange_chunks=(), overlap=True,
            lr_one_stream=False, parity=True):
    import numpy as np
    import torch

    from activation_residual_compression_amd import librescomp as rc
    from activation_residual_compression_amd import synth

    spec = synth.CONFIGS[config]
    wl = synth.make(config)
    nframes = max(2, min(1 + warmup + steps, wl.steps, max_frames))
    dev = torch.device("cuda:0")
    B, n, m = wl.nb, wl.n, wl.m
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    host = _FRAMES.setdefault(wl.name, [])
    if len(host) < nframes:
        log("[bench] %s: generating %d frames of %dx%dx%d %s" % (config, nframes, B, n, m, wl.dtype))
        for _ in range(len(host)):
            wl.next()
        while len(host) < nframes:
            host.append(wl.next()[1])
    frames = []
    for a in host[:nframes]:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if wl.dtype == "bf16" else \
            torch.from_numpy(a)
        frames.append(t.to(dev))
    kw = {k: spec[k] for k in ("group", "nm_keep", "nm_block", "rank", "iters", "grid_w", "keep_blocks")
          if k in spec}
    if spec["scheme"] == "lr":
        kw["q0"] = wl.q0(spec["rank"])
        if lr_one_stream:
            kw["flags"] = rc.RC_LR_ONE_STREAM
    plan = rc.Plan((B, n, m), wl.dtype, spec["scheme"], **kw)
    ahat = frames[0].float().clone()
    recon = ahat.clone()
    e = torch.zeros_like(ahat)
    packed = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    seq = [frames[1 + i % (nframes - 1)] for i in range(warmup + steps)]
    for i in range(warmup):
        plan.compress(seq[i], ahat, e, packed, stream)
        plan.decompress(packed, recon, stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        plan.compress(seq[warmup + i], ahat, e, packed, stream)
        ev[i][1].record(stream)
        plan.decompress(packed, recon, stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    c_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)) / steps
    d_ms = sum(ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)) / steps
    same = bool(torch.equal(ahat, recon))
    in_bytes = 2 if wl.dtype == "bf16" else 4
    N = B * n * m
    alg = algorithmic_bytes(spec["scheme"], N, in_bytes, group=spec.get("group"), rank=spec.get("rank"),
                            rows=n, cols=m, iters=spec.get("iters"), batch=B,
                            keep=spec.get("keep_blocks"))
    out = dict(config=config, scheme=spec["scheme"], shape=[B, n, m], dtype=wl.dtype,
               frames=nframes, steps=steps, ms_per_step=ms_step, compress_ms=c_ms,
               decompress_ms=d_ms, input_GBps=N * in_bytes / (ms_step * 1e6),
               compress_GBps=alg["compress"] / (c_ms * 1e6),
               decompress_GBps=alg["decompress"] / (d_ms * 1e6),
               alg_bytes_compress=alg["compress"], alg_bytes_decompress=alg["decompress"],
               sender_equals_receiver=same)
    out["hbm_frac_step"] = (alg["compress"] + alg["decompress"]) / (ms_step * 1e6) / HBM_PEAK_GBS
    if spec["scheme"] == "lr":
        fl = lr_flops(n, m, spec["rank"], spec["iters"], B)
        out["tensors_per_ms"] = B / ms_step
        out["compress_streams"] = 1 if (lr_one_stream or B < 2) else 2
        out["mfma_flops"] = fl
        out["mfma_util_whole_compress"] = fl / (c_ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    # Steady state of one GPU in a sequence-parallel group: its own compress of
    # step t+1 (stream) runs while the receiver decodes step t (second stream);
    # the two touch disjoint state, so only the packed buffer is double-buffered.
    out["overlapped_ms_per_step"] = None
    if overlap:
        s2 = torch.cuda.Stream()
        packed2 = torch.empty_like(packed)
        bufs = (packed, packed2)
        done_c = [torch.cuda.Event() for _ in range(2)]
        done_d = [torch.cuda.Event() for _ in range(2)]
        for ev in done_d:
            ev.record(stream)
        o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        o0.record(stream)
        for i in range(steps):
            k = i & 1
            stream.wait_event(done_d[k])          # the decode that read this buffer is done
            plan.compress(seq[warmup + i], ahat, e, bufs[k], stream)
            done_c[k].record(stream)
            s2.wait_event(done_c[k])
            plan.decompress(bufs[k], recon, s2)
            done_d[k].record(s2)
        stream.wait_stream(s2)
        o1.record(stream)
        torch.cuda.synchronize()
        out["overlapped_ms_per_step"] = o0.elapsed_time(o1) / steps
    # the same step captured once in a HIP graph and replayed (launch gaps removed)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            plan.compress(seq[0], ahat, e, packed, cap)
            plan.decompress(packed, recon, cap)
    stream.wait_stream(cap)
    for _ in range(2):
        g.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(steps):
        g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    out["graph_ms_per_step"] = g0.elapsed_time(g1) / steps
    del g
    if exchange_chunks:
        out["exchange"] = exchange_timing(plan, seq, ahat, e, packed, exchange_chunks)
        log("[bench] %s exchange: %s" % (config, json.dumps(out["exchange"])))
    if parity:
        out["parity"] = parity_sample(config, plan, seq[-1], ahat, e, recon, packed, log, q0=kw.get("q0"))
    # reference kernels on these very buffers, after the timed region (the state is
    # no longer needed): the HBM ceiling of the sender and receiver access patterns
    if wl.dtype == "bf16" and N % 8 == 0:
        from activation_residual_compression_amd import librescomp as rc
        out["ref_sender_mix_GBps"] = 14.0 * N / (_probe_on(rc.RCX_PROBE_SENDER_MIX, seq[0], ahat, e, N) * 1e6)
        out["ref_receiver_rmw_GBps"] = 8.0 * N / (_probe_on(rc.RCX_PROBE_RECEIVER_RMW, None, recon, None, N) * 1e6)
    if spec["scheme"] == "lr":
        # the passes that read R alone: R's bytes in each product's pattern
        from activation_residual_compression_amd import librescomp as rc
        out["ref_r_read_GBps"] = {
            "rq_pattern": 2.0 * N / (_r_probe_on(plan, rc.RCX_R_PROBE_RQ) * 1e6),
            "rtp_pattern": 2.0 * N / (_r_probe_on(plan, rc.RCX_R_PROBE_RTP) * 1e6)}
    plan.close()
    del frames, seq, ahat, recon, e, packed
    torch.cuda.empty_cache()
    return out


def parity_summary(results):
    """Totals of the per-workload sampled oracle checks."""
    checks = {k: r["parity"] for k, r in results.items() if "parity" in r}
    if not checks:
        return None
    exact = {k: p for k, p in checks.items() if "eps_gap_max" not in p}
    lr = {k: p for k, p in checks.items() if "eps_gap_max" in p}
    return dict(
        workloads_checked=sorted(checks),
        mismatched_packed_bytes=sum(p["mismatched_packed_bytes"] for p in exact.values()),
        mismatched_state_elements=sum(p["mismatched_state_elements"] for p in exact.values()),
        boundary_elements=sum(p["boundary_elements"] for p in exact.values()),
        max_rel_err_state=max([p["max_rel_err_state"] for p in exact.values()] or [0.0]),
        lowrank_eps_gap_max=max([p["eps_gap_max"] for p in lr.values()] or [0.0]),
        receiver_equals_sender=all(p["receiver_equals_sender"] for p in checks.values()))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(config, budget_s, log, ntensors=24):
    """The oracle, untuned, single-threaded, on a bounded sample of the workload
    (its first ntensors tensors, step after step, until budget_s is spent)."""
    import numpy as np

    import oracle
    from activation_residual_compression_amd import synth

    spec = synth.CONFIGS[config]
    kw = {k: spec[k] for k in ("group",) if k in spec}
    if spec["scheme"] == "lr":
        kw.update(rank=spec["rank"], iters=spec["iters"])
    oracle.build(force=False)
    full = synth.make(config, tensors=[0])
    tensors = list(range(min(ntensors, full.batch)))
    wl = synth.make(config, tensors=tensors)
    _, a0 = wl.next()
    f32 = lambda a: (a.astype(np.uint32) << 16).view(np.float32) if wl.dtype == "bf16" else a
    ahat = [f32(a0)[i].copy() for i in range(len(tensors))]
    recon = [x.copy() for x in ahat]
    prev = [x.copy() for x in ahat]
    visited = [np.zeros(wl.n // 64, bool) for _ in tensors]
    q0 = wl.q0(spec["rank"]) if spec["scheme"] == "lr" else None
    done, elapsed, t = 0, 0.0, 0
    log("[bench] cpu baseline: oracle %s" % config)
    while elapsed < budget_s and t + 1 < wl.steps:
        _, a = wl.next()
        t += 1
        af = f32(a)
        for i in range(len(tensors)):
            s = time.perf_counter()
            if spec["scheme"] == "bs":
                o = oracle.bs_compress_tensor(af[i], ahat[i], grid_w=spec["grid_w"], keep=spec["keep_blocks"],
                                              visited=visited[i], prev=prev[i], in_dtype=wl.dtype)
                recon[i] = oracle.bs_decompress_tensor(o["packed"], recon[i], grid_w=spec["grid_w"],
                                                       keep=spec["keep_blocks"], in_dtype=wl.dtype)
                visited[i], prev[i] = o["visited"], af[i]
            else:
                extra = dict(q0=q0[i]) if q0 is not None else {}
                o = oracle.compress_tensor(spec["scheme"], af[i], ahat[i], **kw, **extra)
                recon[i] = oracle.decompress_tensor(spec["scheme"], o["packed"], recon[i],
                                                    group=kw.get("group"), rank=kw.get("rank"))
            elapsed += time.perf_counter() - s
            ahat[i] = o["ahat"]
            done += 1
            if elapsed >= budget_s:
                break
    in_bytes = 2 if wl.dtype == "bf16" else 4
    gbps = done * wl.n * wl.m * in_bytes / elapsed / 1e9
    return dict(value=gbps, unit="GB/s", cores=1, kind="oracle", cpu_model=_cpu_model(),
                host_cpus=os.cpu_count(), tensors_per_s=done / elapsed,
                sample="%s: %d tensor-steps of %dx%d (tensors 0-%d, steps 1-%d), compress+decompress, "
                       "%.1f s single-threaded" % (config, done, wl.n, wl.m, len(tensors) - 1, t, elapsed))


def parity_sample(config, plan, frame, ahat, e, recon, packed, log, q0=None):
    """One more step after the timed region, checked against the oracle on the
    first and last tensor of the batch, teacher-forced (the oracle starts from
    the GPU's state before the step). Bit-exact schemes: packed bytes, e and
    ahat compared element by element; the count of elements within 1e-6
    (relative) of a quantiser decision boundary is reported, as those are the
    only ones where a code may differ. Low rank: the relative Frobenius error
    of ahat, GPU against oracle. Block selection: the plan's round is restarted
    first, so the oracle starts from an empty round too."""
    import numpy as np
    import torch

    import oracle
    from activation_residual_compression_amd import synth

    spec = synth.CONFIGS[config]
    scheme = spec["scheme"]
    B, n, m = plan.shape
    bf16 = plan.dtype == "bf16"
    f32 = lambda t: t.float().cpu().numpy()
    checked = sorted({0, B - 1})
    if scheme == "bs":
        plan.reset_state()
    recon.copy_(ahat)   # the receiver starts where the sender does (timing runs may have parted them)
    before = ahat.cpu().numpy()
    plan.compress(frame, ahat, e, packed)
    plan.decompress(packed, recon)
    torch.cuda.synchronize()
    af, pk, ah, eh, rh = f32(frame), packed.cpu().numpy(), ahat.cpu().numpy(), e.cpu().numpy(), recon.cpu().numpy()
    ts = plan.tensor_packed_bytes
    out = dict(tensors_checked=checked, mismatched_packed_bytes=0, mismatched_state_elements=0,
               max_rel_err_state=0.0, boundary_elements=0,
               receiver_equals_sender=bool(np.array_equal(rh.view(np.uint32), ah.view(np.uint32))))
    kw = {k: spec[k] for k in ("group",) if k in spec}
    for b in checked:
        r = (af[b] - before[b]).astype(np.float32)
        if scheme == "lr":
            o = oracle.compress_tensor("lr", af[b], before[b], rank=spec["rank"], iters=spec["iters"],
                                       q0=q0[b])
            eg = float(np.linalg.norm(af[b].astype(np.float64) - ah[b]) / np.linalg.norm(af[b]))
            eo = float(np.linalg.norm(af[b].astype(np.float64) - o["ahat"]) / np.linalg.norm(af[b]))
            out.setdefault("eps_gpu", []).append(eg)
            out.setdefault("eps_oracle", []).append(eo)
            out["eps_gap_max"] = max(out.get("eps_gap_max", 0.0), abs(eg - eo))
            continue
        if scheme == "bs":
            o = oracle.bs_compress_tensor(af[b], before[b], grid_w=spec["grid_w"], keep=spec["keep_blocks"],
                                          visited=np.zeros(n // 64, bool), in_dtype=plan.dtype)
        else:
            o = oracle.compress_tensor(scheme, af[b], before[b], **kw)
        out["mismatched_packed_bytes"] += int(np.count_nonzero(pk[b * ts:(b + 1) * ts] != o["packed"]))
        for g, w in ((ah[b], o["ahat"]), (eh[b], o["e"])):
            out["mismatched_state_elements"] += int(np.count_nonzero(g.view(np.uint32) != w.view(np.uint32)))
            den = max(float(np.abs(w).max()), 1e-30)
            out["max_rel_err_state"] = max(out["max_rel_err_state"], float(np.abs(g.astype(np.float64) - w).max()) / den)
        out["boundary_elements"] += boundary_count(scheme, r, o, n, m, kw)
    log("[bench] %s parity sample: %s" % (config, json.dumps(out)))
    return out


def boundary_count(scheme, r, o, n, m, kw):
    """Elements whose pre-quantisation value lies within 1e-6 (relative) of a
    decision boundary of the oracle's encoding (where a code may flip)."""
    import numpy as np

    import oracle
    if scheme == "q1":
        s = oracle.unpack_fields("q1", o["packed"], n, m, group=kw["group"])["scale"]
        s = np.repeat(s, kw["group"]).reshape(n, m)
        return int(np.count_nonzero(np.abs(r) <= 1e-6 * s))
    if scheme == "q2":
        f = oracle.unpack_fields("q2", o["packed"], n, m, group=kw["group"])
        mn = np.repeat(f["mn"], kw["group"]).reshape(n, m).astype(np.float64)
        d = np.repeat(f["d"], kw["group"]).reshape(n, m).astype(np.float64)
        cnt = 0
        for k in range(3):
            mid = mn + (k + 0.5) * d
            cnt += int(np.count_nonzero((np.abs(r - mid) <= 1e-6 * np.maximum(np.abs(mid), 3 * d)) & (d > 0)))
        return cnt
    if scheme == "nm":
        blk = np.sort(np.abs(r.reshape(-1, 16).astype(np.float64)), axis=1)[:, ::-1]
        return int(np.count_nonzero(blk[:, 1] - blk[:, 2] <= 1e-6 * blk[:, 1]) * 2)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flux_q2")
    ap.add_argument("--also", default="flux_nm,video_q1,flux_lr,video_lr,latent_bs,tiny_q1",
                    help="other workloads to measure ('' for none)")
    ap.add_argument("--also-frames", type=int, default=4,
                    help="distinct input frames for the other workloads (cycled)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cpu-budget-each", type=float, default=4.0,
                    help="seconds of oracle time on each of the other workloads (reported "
                         "under workloads.<name>.cpu_baseline; 0 to skip)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the sampled oracle check after each workload's timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-probe", action="store_true")
    ap.add_argument("--no-exchange", action="store_true",
                    help="skip the compress + hand-off pipeline timing and the two-stream "
                         "compress/decode overlap (both run kernels concurrently)")
    ap.add_argument("--lr-one-stream", action="store_true",
                    help="low-rank plans keep every compress kernel on one stream (per-kernel "
                         "traces without the two half-batch streams overlapping)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path has no inter-GPU step in this library "
              "(--gpus %d / WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    log = lambda s: print(s, file=sys.stderr, flush=True)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            dst.copy_(src)
        ev0.record()
        for _ in range(5):
            dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / 5
        log("[bench] copy 1 GiB -> 1 GiB: %.3f ms, %.0f GB/s (read+write)" % (ms, 2 * (1 << 30) / ms / 1e6))
        del src, dst
        torch.cuda.empty_cache()

    from activation_residual_compression_amd import synth as _synth
    _wl = _synth.make(args.workload, tensors=[0])
    ceiling = None if args.no_hbm_probe else hbm_probe(_wl.batch * _wl.n * _wl.m, log)
    main_res = measure(args.workload, args.steps, args.warmup, 64, log,
                       exchange_chunks=() if args.no_exchange else (4, 8, 19),
                       overlap=not args.no_exchange, lr_one_stream=args.lr_one_stream,
                       parity=not args.no_parity)
    log("[bench] %s: %.3f ms/step, %.1f GB/s input, compress %.3f ms (%.0f GB/s alg), "
        "graph replay %.3f ms/step, compress/decode overlapped %s ms/step" % (
            args.workload, main_res["ms_per_step"], main_res["input_GBps"], main_res["compress_ms"],
            main_res["compress_GBps"], main_res["graph_ms_per_step"], _ms(main_res["overlapped_ms_per_step"])))
    others = {}
    for cfg in [c for c in args.also.split(",") if c and c != args.workload]:
        r = measure(cfg, args.steps, args.warmup, args.also_frames, log,
                    exchange_chunks=(8, 19) if (cfg == "flux_lr" and not args.no_exchange) else (),
                    overlap=not args.no_exchange, lr_one_stream=args.lr_one_stream,
                    parity=not args.no_parity)
        log("[bench] %s: %.3f ms/step, %.1f GB/s input (graph replay %.3f, compress/decode "
            "overlapped %s ms/step)" % (cfg, r["ms_per_step"], r["input_GBps"],
                                       r["graph_ms_per_step"], _ms(r["overlapped_ms_per_step"])))
        others[cfg] = r

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_budget, log)
        main_res["cpu_baseline"] = cpu
        if args.cpu_budget_each > 0:
            for cfg, res in others.items():
                res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget_each, log,
                                                   ntensors=4 if res["scheme"] == "lr" else 8)

    ach = main_res["compress_GBps"]
    traffic = None
    prefix = SENDER_KERNEL.get(args.workload)
    pmc = _fresh_profile("bench_workloads_hbm_traffic.json", prefix) if prefix else None
    kname = None
    if pmc:
        hits = [k for k in pmc["kernels"] if k.startswith(prefix)]
        if len(hits) == 1:
            kname = hits[0]
            traffic = pmc["kernels"][kname]["bytes"]
    # the low-rank products' durations come from the one-stream trace (one
    # launch per kernel for the whole batch, nothing overlapping)
    trace = _fresh_profile("lowrank_flux_video_kernel_trace.json", "lr_")
    for cfg, res in others.items():
        if cfg in LR_CONTRACTIONS and trace:
            ks = LR_CONTRACTIONS[cfg]
            if all(k in trace["kernels"] for k, _ in ks):
                us = sum(trace["kernels"][k]["avg_us"] * cnt for k, cnt in ks)
                res["mfma_util_contractions"] = res["mfma_flops"] / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                res["contraction_us_per_step"] = us
            # HBM fraction of the streaming passes (whole-batch launches):
            # algorithmic bytes per element x elements / average duration
            B, n, m = res["shape"]
            k = int(ks[0][0].split(",")[-1].strip(" >"))
            passes = {"first_product": ("lr_rq_kernel<unsigned short, true, %d>" % k, 8, None),
                      "reconstruct_sender": ("lr_recon_kernel<unsigned short, true, %d, %d, false," % (k, k), 14,
                                             None),
                      "reconstruct_receiver": ("lr_recon_kernel<float, false, %d, %d, false," % (k, k), 8, None),
                      "r_only_rq": ("lr_rq_kernel<unsigned short, false, %d>" % k, 2, "rq_pattern"),
                      "r_only_rtp_first": ("lr_rtp_kernel<%d, false>" % k, 2, "rtp_pattern"),
                      "r_only_rtp_last": ("lr_rtp_kernel<%d, true>" % k, 2, "rtp_pattern")}
            frac, of_probe = {}, {}
            ref = res.get("ref_r_read_GBps") or {}
            for name, (prefix, bpe, pat) in passes.items():
                hits = [v for kn, v in trace["kernels"].items() if kn.startswith(prefix)]
                if len(hits) == 1:
                    gbs = bpe * B * n * m / (hits[0]["avg_us"] * 1e3)
                    frac[name] = gbs / HBM_PEAK_GBS
                    if pat in ref:
                        of_probe[name] = gbs / ref[pat]
            res["streaming_pass_hbm_frac"] = frac
            if of_probe:
                res["r_only_pass_frac_of_r_probe"] = of_probe
    roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": kname or ((prefix + " ...>") if prefix else "sender kernel (rc_compress)"),
            "alg_bytes_per_launch": main_res["alg_bytes_compress"]}
    if "ref_sender_mix_GBps" in main_res:
        roof["measured_ceiling"] = main_res["ref_sender_mix_GBps"]
        roof["frac_of_measured_ceiling"] = ach / main_res["ref_sender_mix_GBps"]
    line = {
        "metric": "compress+decompress GB/s of activations per GPU (% HBM peak); low-rank MFMA util",
        "value": main_res["input_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %d %s tensors [%d x %d] per step, scheme %s" % (
            args.workload, main_res["shape"][0], main_res["dtype"], *main_res["shape"][1:], main_res["scheme"]),
            "input_dtype": main_res["dtype"], "state_dtype": "f32",
            "steps_per_sequence": _synth.make(args.workload, tensors=[0]).steps,
            "parallelism": "single GPU",
            "headline": "the FLUX-like sequence-parallel share (2-bit), the first full-size "
                        "setting of the metric; every other setting, the largest (video-like "
                        "1-bit, 256 M elements per step) included, is measured in the same run "
                        "under workloads"},
        "roofline": roof,
        "hbm_reference_kernels_GBps": ceiling,
        "hbm_frac_step": main_res["hbm_frac_step"],
        "cpu_baseline": cpu,
        "parity": parity_summary({args.workload: main_res, **others}),
        "workloads": {args.workload: main_res, **others},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
