"""Where the prefill kernels' time goes, phase by phase, from their own clocks.

    python -m linear_attention_prefill_amd.build --phase-clocks
    python -m linear_attention_prefill_amd.phase_clocks [--workload packed|single|short] [--conv]

Runs one prefill call of a synthetic workload (the generators of
``workloads``) with ``libkda_clocks.so``, whose intra-chunk and fused
kernels record the core clock counter at every phase boundary of workgroup
0 (``kda_phase_clocks`` in ``include/kda.h``), and whose state scan does
the same for the steps of its workgroup 0 (the longest sequence's first
slice group), and prints for each wave the clocks an item spends in each
phase and in the barrier that ends it, averaged over the items the
workgroup ran.  Waves w and w + 4 of the 8-wave kernels share a SIMD.
The records cost a few instructions a phase; times are for attribution, the
uninstrumented library's times are ``bench.py``'s.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np
import torch

from . import kda as K
from . import workloads as W

# (name, first mark, last mark) of each interval of an item
INTERVALS = [("factors", 0, 1), ("bar", 1, 2), ("A blocks", 2, 3), ("bar", 3, 4),
             ("level 1", 4, 5), ("bar", 5, 6), ("level 2", 6, 7), ("bar", 7, 8),
             ("w, u", 8, 9), ("bar", 9, 10), ("state", 10, 11), ("bar", 11, 12),
             ("chain", 12, 13)]
# a scan step: publish the state tiles (and the barrier), U = u - w S with
# the Q~ S part of o, publish U (decay, refills, barrier), the state update
# and the o store
SCAN_INTERVALS = [("S out+bar", 0, 1), ("U, Q~S", 1, 2), ("U out+bar", 2, 3), ("S, o", 3, 4)]


def workload(name: str):
    if name == "packed":
        return W.packed_varlen_prefill()
    if name == "single":
        return W.single_seq_prefill()
    if name == "short":
        return W.packed_varlen_prefill(n=128, num_slots=128)
    raise ValueError(name)


def run_call(c, conv: bool, reps: int):
    dt = torch.bfloat16 if c.io_dtype == "bf16" else torch.float32
    d = lambda x: torch.from_numpy(x).to("cuda")
    q, k, v = d(c.q).to(dt), d(c.k).to(dt), d(c.v).to(dt)
    g, beta, cu = d(c.g), d(c.beta), d(c.cu_seqlens)
    slots = d(c.slots) if c.slots is not None else None
    pool = (d(c.state_pool) if c.state_pool is not None
            else torch.zeros((1, c.H, c.d_v, c.d_k), dtype=torch.float32, device="cuda"))
    kw = {}
    if conv:
        weight, window = W.draw_conv(11, pool.shape[0], c.H, c.d_k, c.d_v, c.io_dtype)
        kw = dict(conv_weight=d(weight), conv_window=d(window).to(dt), conv_activation="silu")
    o = torch.empty((c.T, c.H, c.d_v), dtype=dt, device="cuda")
    for _ in range(reps):
        K.chunk_prefill(q, k, v, g, beta, cu, state_in=pool if c.state_pool is not None else None,
                        state_out=pool, o=o, slots=slots, scale=c.scale, **kw)
    torch.cuda.synchronize()


def table(clk: np.ndarray, fused: bool, intervals=None) -> list:
    """Per-wave mean clocks of each interval over the items whose marks are
    all recorded and in order, and whose next item's top mark came later in
    the same launch.  The last item has no next top mark; a call of several
    windows launches the intra-chunk kernel once per window, and each launch
    rewrites the items it reaches, so an item left from an earlier launch
    (its top mark earlier than the item before it) ends the run."""
    iv = intervals if intervals is not None else [x for x in INTERVALS if fused or x[2] <= 10]
    names = [n for n, a, b in iv]
    lines = ["%-5s %5s %8s " % ("wave", "items", "item") + " ".join("%9s" % n for n in names)]
    for w in range(clk.shape[0]):
        rows = []
        for i in range(clk.shape[1] - 1):
            c0, c1 = clk[w, i], clk[w, i + 1]
            if c0[0] == 0 or c1[0] == 0:
                continue
            marks = [m for _, a, b in iv for m in (a, b)]
            if any(c0[m] == 0 for m in marks) or c1[0] <= c0[0]:
                continue
            if any(c0[b] < c0[a] for n, a, b in iv):
                continue
            rows.append([c1[0] - c0[0]] + [c0[b] - c0[a] for n, a, b in iv])
        if not rows:
            continue
        r = np.mean(np.array(rows, dtype=np.float64), axis=0)
        lines.append("%-5d %5d %8.0f " % (w, len(rows), r[0]) + " ".join("%9.0f" % x for x in r[1:]))
    return lines


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="packed", choices=["packed", "single", "short"])
    ap.add_argument("--conv", action="store_true", help="with the short conv front end (SiLU)")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.stderr.write("phase_clocks needs a GPU\n")
        return 1
    K.LIB_PATH = K.CLOCKS_LIB_PATH
    K.load_library()
    c = workload(args.workload)
    run_call(c, args.conv, 3)
    for kern in (K.KDA_CLOCK_INTRA, K.KDA_CLOCK_FUSED, K.KDA_CLOCK_SCAN):
        K.phase_clocks(kern, clear=True)
    run_call(c, args.conv, 1)
    print("phase clocks (core clocks an item, workgroup 0): %s%s, H=%d, d_k=%d, d_v=%d, %s"
          % (c.name, " + conv (SiLU)" if args.conv else "", c.H, c.d_k, c.d_v, c.io_dtype))
    for kern, label in ((K.KDA_CLOCK_INTRA, "intra-chunk kernel"), (K.KDA_CLOCK_FUSED, "fused prefill"),
                        (K.KDA_CLOCK_SCAN, "state scan (steps of the longest chain)")):
        clk = K.phase_clocks(kern)
        if not clk.any():
            print("%s: no items" % label)
            continue
        print("%s:" % label)
        print("\n".join(table(clk, kern == K.KDA_CLOCK_FUSED,
                               SCAN_INTERVALS if kern == K.KDA_CLOCK_SCAN else None)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
