"""Phase timeline of the verify-attention kernel, read from the trace build.

    python -m speculative_decoding_verification_attn_amd.build --trace     # on the build host
    python -m speculative_decoding_verification_attn_amd.phase_trace llama3_70b_tree llama31_8b_chain b64

For each workload (a name of workloads.CONFIGS, or bN for the Llama-3-70B
chain shape at batch N) the attention with transposed V pages runs a few
times, then once more with the timeline cleared; every wave of every range
recorded its phase boundaries (spec_verify_attn_phase_trace).  Printed per
phase: how often it occurred, its median and mean length in shader cycles,
and its summed length per wave in microseconds at --ghz.  The trace build
waits for a whole round's K/V before computing its block and requests the
next page ids after it (so the timestamps do not wait on them); its timing
is therefore close to, not equal to, the production kernel's."""
from __future__ import annotations

import argparse
import collections
import os
import sys

import numpy as np

PHASES = [
    ((1, 2), "prologue: first unit's page ids, K/V loads out, Q staged"),
    ((2, 3), "loop entry"),
    ((3, 4), "issue the next round's K/V loads"),
    ((4, 5), "wait for this round's K/V"),
    ((5, 6), "compute the block (all tiles)"),
    ((6, 3), "page ids of round g+2, next round"),
    ((6, 7), "finish a unit: merge the waves in LDS, write rows"),
    ((7, 8), "enter the next unit: walk, Q staged"),
    ((8, 3), "loop entry after a unit"),
    ((7, 9), "range done"),
]


def phase_table(trace: np.ndarray, ghz: float) -> tuple[list[tuple], int]:
    """Per phase (name, count, median cycles, mean cycles, us per wave) from
    a [ranges, 4, events] timeline; consecutive events of one wave only."""
    iv = collections.defaultdict(list)
    waves = 0
    for w in range(trace.shape[0]):
        for wv in range(trace.shape[1]):
            ev = trace[w, wv]
            ev = ev[ev != 0]
            if len(ev) < 2:
                continue
            waves += 1
            t = (ev >> np.uint64(8)).astype(np.int64)
            c = (ev & np.uint64(255)).astype(np.int64)
            for k in range(1, len(c)):
                iv[(int(c[k - 1]), int(c[k]))].append(int(t[k] - t[k - 1]))
    rows = []
    for key, name in PHASES:
        v = np.array(iv.get(key, []), dtype=np.float64)
        if len(v) == 0:
            continue
        rows.append((name, len(v), float(np.median(v)), float(v.mean()), float(v.sum() / waves / ghz / 1e3)))
    return rows, waves


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--ghz", type=float, default=2.4, help="shader clock for the microsecond column")
    args = ap.parse_args(argv)

    import torch
    from . import build, ops, workloads as W
    if not os.path.exists(build.TRACE_LIB):
        print(f"{build.TRACE_LIB} is missing: python -m speculative_decoding_verification_attn_amd.build --trace",
              file=sys.stderr)
        return 2
    ops.LIB_PATH = build.TRACE_LIB
    ops.load_library()
    dev = "cuda:0"
    for name in args.workloads:
        batch, wl = None, name
        if name.startswith("b") and name[1:].isdigit():
            batch, wl = int(name[1:]), "llama3_70b_b256"
        big = wl in ("qwen3_8b_ragged", "llama3_70b_b256")
        case = W.make_case(wl, None, kv_device=dev if big else None, logits_device=dev if big else None, batch=batch)
        k = case.k_cache_dev if big else torch.from_numpy(case.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
        v = case.v_cache_dev if big else torch.from_numpy(case.v_cache.view(np.int16)).to(dev).view(torch.bfloat16)
        v = v.transpose(-1, -2).contiguous()
        i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)
        q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
        bt, ctx, cu = i32(case.block_tables), i32(case.context_lens), i32(case.cu_q)
        par = None if case.tree_parent is None else i32(case.tree_parent)
        for _ in range(3):
            ops.spec_verify_attn_vt(q, k, v, bt, ctx, cu, par)
        torch.cuda.synchronize()
        ops.spec_verify_attn_phase_trace(clear=True)
        ops.spec_verify_attn_vt(q, k, v, bt, ctx, cu, par)
        torch.cuda.synchronize()
        rows, waves = phase_table(ops.spec_verify_attn_phase_trace(clear=True), args.ghz)
        print(f"## {name}: {waves} waves\n")
        print("| phase | count | median cycles | mean cycles | us per wave |")
        print("|---|---|---|---|---|")
        for nm, cnt, med, mean, us in rows:
            print(f"| {nm} | {cnt} | {med:.0f} | {mean:.0f} | {us:.2f} |")
        print(flush=True)
        del k, v, case
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
