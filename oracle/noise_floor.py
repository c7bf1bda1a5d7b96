"""Noise floor of the parity gates: the oracle against itself.

TEST INFRASTRUCTURE ONLY (see oracle.py).  The "kern" page, section "The
harness", judges a candidate against a noise floor measured by replaying the
reference against itself.  Here the reference is the fp64 token loop, and two
floors bound what any implementation can reach on the same inputs:

* arithmetic: the same loop run in fp32 (kda_oracle.c built with
  KDA_REAL=float) against fp64, i.e. what fp32 arithmetic alone costs;
* output dtype: the fp64 output rounded to bf16 (ties to even) against
  itself, which no bf16-output path can beat.

Errors are normwise per (sequence, head), max|x - ref| / max|ref|, as the
parity tests measure them.

    python -m oracle.noise_floor [--configs tiny,single,long] [--threads N]

prints one JSON object.  The long-context figure runs the 32 calls of the
262,144-token workload in both precisions, state carried, and takes about a
minute on 16 threads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_attention_prefill_amd import workloads as W  # noqa: E402  (inputs only)
from oracle import oracle  # noqa: E402


def _rel(x, ref):
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den else num


def head_floor(o32, o64, s32, s64):
    """Max over heads of the normwise errors of o [T, H, d_v] and of final
    states [H, d_v, d_k] (one sequence)."""
    H = o64.shape[1]
    eo = max(_rel(o32[:, h], o64[:, h]) for h in range(H))
    es = max(_rel(s32[h], s64[h]) for h in range(H))
    return eo, es


def bf16_output_floor(o64):
    r = W.round_to_bf16(o64.astype(np.float32)).astype(np.float64)
    return max(_rel(r[:, h], o64[:, h]) for h in range(o64.shape[1]))


def one_call(case, threads):
    out = {}
    t0 = time.perf_counter()
    o64, s64 = oracle.recurrence(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                 threads=threads)
    o32, s32 = oracle.recurrence(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                 threads=threads, precision="f32")
    eo, es = head_floor(o32, o64, s32[0], s64[0])
    out["fp32_vs_fp64"] = {"o": eo, "state": es}
    if case.io_dtype == "bf16":
        out["bf16_output_rounding"] = {"o": bf16_output_floor(o64)}
    out["seconds"] = time.perf_counter() - t0
    return out


def long_context(threads):
    t0 = time.perf_counter()
    cu = np.array([0, 8192], dtype=np.int32)
    s64 = s32 = None
    for c in range(W.LONG_CONTEXT_CALLS):
        case = W.long_context_call(c)
        o64, s64 = oracle.recurrence(case.q, case.k, case.v, case.g, case.beta, cu, s0=s64,
                                     threads=threads)
        o32, s32 = oracle.recurrence(case.q, case.k, case.v, case.g, case.beta, cu, s0=s32,
                                     threads=threads, precision="f32")
    eo, es = head_floor(o32, o64, s32[0], s64[0])
    return {"fp32_vs_fp64": {"o_last_call": eo, "final_state": es},
            "bf16_output_rounding": {"o_last_call": bf16_output_floor(o64)},
            "seconds": time.perf_counter() - t0}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--configs", default="tiny,single,long")
    ap.add_argument("--threads", type=int, default=None)
    args = ap.parse_args()
    threads = args.threads or oracle.default_threads()
    res = {"threads": threads}
    for name in args.configs.split(","):
        if name == "tiny":
            res["tiny_prefill_T256_H2_d64_f32"] = one_call(W.tiny_prefill(), threads)
        elif name == "single":
            res["single_seq_prefill_T8192_H32_d128_bf16"] = one_call(W.single_seq_prefill(),
                                                                     threads)
        elif name == "long":
            res["long_context_32x8192_H32_d128_bf16"] = long_context(threads)
        else:
            raise SystemExit("unknown config %s" % name)
        sys.stderr.write("[noise-floor] %s done\n" % name)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
