"""Rank x iterations x factor-precision sweep of the low-rank path on one GPU.

The low-rank strategy of the CompactFusion notes (Key designs / Low-rank
strategy for extreme compression) trades three things against each other:
rank (how much of the residual the factors can cover), subspace iterations (how
close the factors get to the best rank-k subspace) and factor precision (INT4
with per-column scales, or bf16: at one payload, bf16 factors of rank k cost as
much as INT4 factors of rank 4k). This script runs every combination through
the library on a synthetic workload and reports, per configuration:

  payload_B      packed bytes per tensor (rc_tensor_packed_bytes)
  ratio          bf16 activation bytes / payload
  res_relF       mean over tensors and steps of ||e_t|| / ||r_t||: the share of
                 the residual the compressor leaves behind
  eps            mean ||a_t - ahat_t|| / ||a_t|| after the step
  ms_per_step    compress + decompress of the whole batch (HIP events)
  tensors_per_ms batch / ms_per_step

Usage: python -m activation_residual_compression_amd.lr_sweep [--workload flux_lr]
       [--ranks 8,16,32,48,64] [--iters 1,2,3,4] [--factors int4,bf16] [--md OUT]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run(config, ranks, iters_list, factors_list, frames=3, reps=5, log=print):
    import numpy as np
    import torch

    from activation_residual_compression_amd import librescomp as rc
    from activation_residual_compression_amd import synth

    wl = synth.make(config)
    B, n, m = wl.nb, wl.n, wl.m
    dev = torch.device("cuda:0")
    log("[sweep] %s: generating %d frames of %dx%dx%d %s" % (config, frames, B, n, m, wl.dtype))
    host = [wl.next()[1] for _ in range(frames)]

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    seq = [to_dev(a) for a in host]
    in_bytes = 2 if wl.dtype == "bf16" else 4
    stream = torch.cuda.current_stream()
    rows = []
    for factors in factors_list:
        for rank in ranks:
            q0 = wl.q0(rank)
            for iters in iters_list:
                flags = rc.RC_LR_BF16_FACTORS if factors == "bf16" else 0
                with rc.Plan((B, n, m), wl.dtype, "lr", rank=rank, iters=iters, q0=q0, flags=flags) as plan:
                    ahat = seq[0].float().clone()
                    recon = ahat.clone()
                    e = torch.zeros_like(ahat)
                    packed = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=dev)
                    res, eps = [], []
                    for t in range(1, frames):
                        a = seq[t]
                        r = a.float() - ahat
                        plan.compress(a, ahat, e, packed, stream)
                        plan.decompress(packed, recon, stream)
                        rn = torch.linalg.vector_norm(r.double(), dim=(1, 2))
                        en = torch.linalg.vector_norm(e.double(), dim=(1, 2))
                        an = torch.linalg.vector_norm(a.double(), dim=(1, 2))
                        dn = torch.linalg.vector_norm((a.float() - ahat).double(), dim=(1, 2))
                        res.append((en / rn).mean().item())
                        eps.append((dn / an).mean().item())
                    same = bool(torch.equal(ahat, recon))
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    ev[0].record(stream)
                    for i in range(reps):
                        a = seq[1 + i % (frames - 1)]
                        plan.compress(a, ahat, e, packed, stream)
                        plan.decompress(packed, recon, stream)
                    ev[1].record(stream)
                    torch.cuda.synchronize()
                    ms = ev[0].elapsed_time(ev[1]) / reps
                    row = dict(workload=config, factors=factors, rank=rank, iters=iters,
                               payload_B=plan.tensor_packed_bytes,
                               ratio=n * m * in_bytes / plan.tensor_packed_bytes,
                               res_relF=float(np.mean(res)), eps=float(np.mean(eps)),
                               ms_per_step=ms, tensors_per_ms=B / ms, sender_equals_receiver=same)
                    log(json.dumps(row))
                    rows.append(row)
    return rows


def markdown(rows):
    lines = ["| factors | rank | iters | payload B/tensor | ratio vs bf16 | residual left ‖e‖/‖r‖ | ε after step | ms/step | tensors/ms |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: (r["payload_B"], r["factors"], r["iters"])):
        lines.append("| %s | %d | %d | %d | %.1f× | %.4f | %.4f | %.3f | %.1f |" % (
            r["factors"], r["rank"], r["iters"], r["payload_B"], r["ratio"], r["res_relF"], r["eps"],
            r["ms_per_step"], r["tensors_per_ms"]))
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="flux_lr")
    ap.add_argument("--ranks", default="8,16,32,48,64")
    ap.add_argument("--iters", default="1,2,3,4")
    ap.add_argument("--factors", default="int4,bf16")
    ap.add_argument("--frames", type=int, default=3)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--md")
    args = ap.parse_args(argv)
    rows = run(args.workload, [int(x) for x in args.ranks.split(",")],
               [int(x) for x in args.iters.split(",")], args.factors.split(","),
               frames=args.frames, reps=args.reps,
               log=lambda s: print(s, flush=True))
    text = markdown(rows)
    print(text)
    if args.md:
        open(args.md, "w").write(text + "\n")


if __name__ == "__main__":
    main()
