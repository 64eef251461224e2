#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verification step on one MI355X.

One step = the whole hot path over one batch: verify attention for every
layer of the model (K/V of distinct layers rotate through `--kv-copies`
resident caches), then full-vocabulary greedy acceptance, then KV compaction
over the resident caches.  Inputs are seeded synthetic tensors already in HBM
when the timed region starts.  Each phase is captured once as a HIP graph and
replayed every step (--eager launches every kernel from the host instead).

Prints ONE JSON line on stdout; progress goes to stderr.
Default workload: Llama-3-70B attention geometry, batch 256, gamma 3
(the spec shape), 80 layers per step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak, TFLOP/s
MI355X_SIMDS = 256 * 4  # compute units x SIMDs
MI355X_XCDS = 8
KV_RESIDENT_LIMIT = 96e9  # bytes of per-layer caches the bench keeps resident at most
SWEEP_BATCHES = (16, 32, 64, 128, 256)  # 70B-shape batch sweep (the last is the default workload)

WORKLOAD_TEXT = {
    "tiny_chain": "tiny chain verify: B=1, gamma=4, 8/2 heads, D=64, L=256, V=1024",
    "llama31_8b_chain": "Llama-3.1-8B geometry chain verify: B=1, gamma=5, 32/8 heads, D=128, L=4096, V=128256",
    "llama3_70b_tree": "Llama-3-70B geometry tree verify: B=1, 64-node depth-6 tree, 64/8 heads, D=128, L=8192, V=128256",
    "qwen3_8b_ragged": "Qwen3-8B geometry ragged batch: B=64, gamma_i~U[1,8], 32/8 heads, D=128, L log-uniform [512,32768], V=151936",
    "llama3_70b_b256": "Llama-3-70B geometry large-batch chain verify: B=256, gamma=3, 64/8 heads, D=128, L~U[2048,8192], V=128256",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama3_70b_b256")
    ap.add_argument("--layers", type=int, default=None, help="attention layers per step (default: the model's)")
    ap.add_argument("--kv-copies", type=int, default=None, help="distinct resident layer caches")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--batch", type=int, default=None, help="override the request count (batch sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host each step instead of replaying HIP graphs")
    ap.add_argument("--cpu-sample-requests", type=int, default=0,
                    help="requests of the workload the CPU oracle is timed on (0 = all)")
    ap.add_argument("--v-layout", choices=("transposed", "token-major"), default="transposed",
                    help="V page layout of the timed step: transposed page blocks (the *_vt calls) or "
                         "token-major pages (the plain calls); the other layout's attention is timed beside it")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 70B-shape batch sweep (and the SPS table built from it)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MB "
                         "(reference for the HBM traffic counters)")
    ap.add_argument("--stochastic", action="store_true",
                    help="stochastic acceptance (speculative sampling) instead of greedy; synthetic drafter "
                         "distributions = softmax of perturbed logits")
    ap.add_argument("--fused", action="store_true",
                    help="acceptance and compaction as one launch (spec_accept_compact)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="time chunked verification with early pruning (FASER) in chunks of this many "
                         "verify tokens instead of the default step")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU run: turn the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE outputs of a "
                         "--calibrate-copy-mb run into profiles/verify_attn_<config>_traffic.json")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR", default=None,
                    help="no GPU run: turn a rocprofv3 --pmc run of SQ_INSTS_MFMA, "
                         "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (among others) into "
                         "profiles/verify_attn_<config>_mfma.json")
    ap.add_argument("--sps-summary", metavar="BENCH_JSON", default=None,
                    help="no GPU run: turn the sps_table of a default run's JSON line into "
                         "profiles/sps_table_llama3_70b.json (the verify-budget scheduler's cost table)")
    args = ap.parse_args()
    if args.sps_summary:
        write_sps_summary(args.sps_summary)
        return
    if args.mfma_summary:
        write_mfma_summary(args.config, args.mfma_summary, vt=args.v_layout == "transposed")
        return
    if args.pmc_summary:
        write_traffic_summary(args.config, *args.pmc_summary, copy_mb=args.calibrate_copy_mb or 1024,
                              vt=args.v_layout == "transposed")
        return

    if args.gpus != 1:
        print(json.dumps({"error": "the verify step runs on one GPU; --gpus must be 1 "
                                   "(the path shards by request or KV head across GPUs, not implemented here)"}))
        sys.exit(2)

    import torch
    from speculative_decoding_verification_attn_amd import ops
    from speculative_decoding_verification_attn_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    ops.load_library()
    dev = "cuda:0"
    name = args.config
    layers = args.layers or W.MODEL_LAYERS[name]
    big = name in ("qwen3_8b_ragged", "llama3_70b_b256")
    t0 = time.time()
    case = W.make_case(name, args.seed, kv_device=dev if big else None,
                       logits_device=dev if big else None, batch=args.batch)
    log(f"generated {name}: B={case.batch} T={case.total_q} pages={case.num_pages} "
        f"({time.time() - t0:.1f}s)")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    kv_bytes = case.kv_bytes_per_layer()
    if args.kv_copies:
        copies = args.kv_copies
    elif layers * kv_bytes <= KV_RESIDENT_LIMIT:
        # every layer's cache resident: attention never hits the 256 MB
        # last-level cache and compaction covers all layers in one call
        copies = layers
    else:
        # distinct caches so layers do not hit in the 256 MB last-level cache
        copies = min(layers, max(2, int(np.ceil(1.0e9 / max(kv_bytes, 1)))))
    vt = args.v_layout == "transposed"
    attn_run = ops.spec_verify_attn_run_vt if vt else ops.spec_verify_attn_run
    compact = ops.kv_compact_vt if vt else ops.kv_compact
    accept_compact = ops.spec_accept_compact_vt if vt else ops.spec_accept_compact
    chunk_run = ops.spec_verify_attn_chunk_run_vt if vt else ops.spec_verify_attn_chunk_run
    k0 = case.k_cache_dev if big else bf16(case.k_cache)
    # generated pools are token-major; the *_vt calls take each V page block transposed
    v0 = case.v_cache_dev if big else bf16(case.v_cache)
    if vt:
        v0 = v0.transpose(-1, -2).contiguous()
    K = torch.empty((copies,) + tuple(k0.shape), dtype=torch.bfloat16, device=dev)
    V = torch.empty((copies,) + tuple(v0.shape), dtype=torch.bfloat16, device=dev)
    for c in range(copies):
        K[c].copy_(k0)
        V[c].copy_(v0)
    del k0, v0
    case.k_cache_dev = case.v_cache_dev = None
    q = bf16(case.q)
    bt, ctx, cu = i32(case.block_tables), i32(case.context_lens), i32(case.cu_q)
    par = None if case.tree_parent is None else i32(case.tree_parent)
    logits = case.logits_dev if big else torch.from_numpy(case.logits).to(dev)
    draft = i32(case.draft_tokens)
    out = torch.empty_like(q)
    B, T = case.batch, case.total_q
    ws_attn = torch.empty(ops.spec_verify_attn_workspace_size(B, T, case.num_q_heads, case.num_kv_heads,
                                                              case.head_dim), dtype=torch.uint8, device=dev)
    ws_acc = torch.empty(ops.spec_accept_workspace_size(B, T, case.vocab), dtype=torch.uint8, device=dev)
    t_arg = torch.empty(T, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(T, dtype=torch.int32, device=dev)
    toks = torch.empty(T, dtype=torch.int32, device=dev)
    new_len = torch.empty(B, dtype=torch.int32, device=dev)
    if args.stochastic:
        g = torch.Generator(device=dev).manual_seed(1234)
        # each draft row a perturbed copy of the target row that predicts its token
        # (the previous token's row; in a tree, the parent's)
        src = np.arange(T, dtype=np.int64)
        for i in range(B):
            o, o1 = int(case.cu_q[i]), int(case.cu_q[i + 1])
            ks = np.arange(1, o1 - o)
            src[o + ks] = o + (ks - 1 if case.tree_parent is None else case.tree_parent[o + ks])
        src_rows = torch.from_numpy(src).to(dev)
        dprobs = torch.softmax(logits[src_rows] + 0.3 * torch.randn(logits.shape, device=dev, generator=g), dim=-1)
        u_acc = torch.rand(T, device=dev, generator=g)
        w_smp = torch.rand(B, device=dev, generator=g)
        ws_sto = torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, case.vocab), dtype=torch.uint8,
                             device=dev)
    ws_fused = torch.zeros(ops.spec_accept_compact_workspace_size(B, T, case.vocab), dtype=torch.uint8,
                           device=dev) if args.fused else None
    stream = torch.cuda.current_stream()
    log(f"resident: {copies} KV copies x {kv_bytes / 1e9:.3f} GB, logits {T * case.vocab * 4 / 1e6:.1f} MB")

    timings = {"plan": [], "attn": [], "accept": [], "compact": []}

    def mark():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    # the four phases of a step; `st` None = the current stream (a capturing
    # stream inside graph capture)
    def phase_plan(st):
        # one plan per step serves every layer (it depends only on the batch metadata)
        ops.spec_verify_attn_plan(ctx, cu, max_blocks_per_seq=bt.shape[1], num_q_heads=case.num_q_heads,
                                  num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                                  num_pages=case.num_pages, total_q=T, workspace=ws_attn, stream=st)

    def phase_layer(layer, st):
        c = layer % copies
        attn_run(q, K[c], V[c], bt, ctx, cu, par, out=out, workspace=ws_attn, stream=st)

    def phase_accept(st):
        if args.stochastic:
            if par is None:
                ops.spec_accept_stochastic(logits, dprobs, draft, u_acc, w_smp, cu, workspace=ws_sto,
                                           accept_len=acc, accepted_path=path, out_tokens=toks, stream=st)
            else:
                ops.spec_accept_stochastic_tree(logits, dprobs, draft, par, u_acc, w_smp, cu, workspace=ws_sto,
                                                accept_len=acc, accepted_path=path, out_tokens=toks, stream=st)
            return
        if args.fused:  # acceptance and compaction in one launch; the compact phase is then empty
            accept_compact(logits, draft, cu, par, K, V, bt, ctx, workspace=ws_fused, num_layers=copies,
                           target_argmax=t_arg, accept_len=acc, accepted_path=path, out_tokens=toks,
                           new_context_lens=new_len, stream=st)
            return
        ops.spec_accept(logits, draft, cu, par, target_argmax=t_arg, accept_len=acc, accepted_path=path,
                        out_tokens=toks, workspace=ws_acc, stream=st)

    def phase_compact(st):
        if args.fused:
            return
        compact(K, V, bt, ctx, cu, path, acc, num_layers=copies, new_context_lens=new_len, stream=st)

    def step_eager(record):
        e0 = mark() if record else None
        phase_plan(stream)
        if record:
            timings["plan"].append((e0, mark()))
        for layer in range(layers):
            e0 = mark() if record else None
            phase_layer(layer, stream)
            if record:
                timings["attn"].append((e0, mark()))
        e0 = mark() if record else None
        phase_accept(stream)
        e1 = mark() if record else None
        phase_compact(stream)
        if record:
            timings["accept"].append((e0, e1))
            timings["compact"].append((e1, mark()))

    for _ in range(args.warmup):
        step_eager(False)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    if args.chunk > 0:
        print(json.dumps(chunked_bench(args, case, ops, dict(
            K=K, V=V, copies=copies, q=q, bt=bt, ctx=ctx, cu=cu, par=par, logits=logits, draft=draft,
            layers=layers, stream=stream, step_eager=step_eager, acc=acc, chunk_run=chunk_run))), flush=True)
        return

    graphs = None
    if not args.eager:
        # One HIP graph per phase: a step replays them back to back, with
        # timing events between the replays (outside the graphs).  Batch-1
        # kernels run for a few microseconds, less than a host-side launch,
        # so eager launches would leave the GPU idle between layers.
        phases = ("plan", "attn", "accept") if args.fused else ("plan", "attn", "accept", "compact")
        graphs = {k: torch.cuda.CUDAGraph() for k in phases}
        with torch.cuda.graph(graphs["plan"]):
            phase_plan(None)
        with torch.cuda.graph(graphs["attn"]):
            for layer in range(layers):
                phase_layer(layer, None)
        with torch.cuda.graph(graphs["accept"]):
            phase_accept(None)
        if "compact" in graphs:
            with torch.cuda.graph(graphs["compact"]):
                phase_compact(None)
        for _ in range(2):
            for k in phases:
                graphs[k].replay()
        torch.cuda.synchronize()
        log("captured one graph per phase")

    def step_graph():
        e0 = mark()
        graphs["plan"].replay()
        e1 = mark()
        graphs["attn"].replay()
        e2 = mark()
        graphs["accept"].replay()
        e3 = mark()
        if "compact" in graphs:
            graphs["compact"].replay()
        e4 = mark()
        timings["plan"].append((e0, e1))
        timings["attn"].append((e1, e2))
        timings["accept"].append((e2, e3))
        timings["compact"].append((e3, e4))

    # timed region: exactly `steps` steps, synchronized on both sides
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        if graphs is None:
            step_eager(True)
        else:
            step_graph()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    def avg_ms(pairs):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) if pairs else float("nan")

    plan_ms = avg_ms(timings["plan"])
    attn_ms = avg_ms(timings["attn"]) / (1 if graphs is None else layers)
    accept_ms = avg_ms(timings["accept"])
    compact_ms = avg_ms(timings["compact"])
    acc_np = acc.cpu().numpy()

    # algorithmic bytes (what the method must move)
    bt_bytes = int(sum(((int(L) + int(qq) + 15) // 16) * 4 for L, qq in zip(case.context_lens, case.q_lens)))
    attn_bytes = kv_bytes + case.qo_bytes() + bt_bytes
    logits_bytes = T * case.vocab * 4
    step_bytes = layers * attn_bytes + logits_bytes
    attn_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
    # algorithmic flops: S = QK^T and O = PV over every verify row and its
    # L_i + q_i keys (masked keys included), 2 flops per multiply-add
    attn_flops = case.attn_flops()
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    intensity = attn_flops / attn_bytes
    mfma_bound = intensity > PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    verified_tok_s = float(acc_np.sum()) / (ms_per_step * 1e-3)

    ceiling = read_ceiling(case, ops, K[0], V[0], stream, kv_bytes / (attn_ms * 1e-3) / 1e9)
    kv_for_cpu = None
    if not args.no_cpu_baseline:
        # host copy of layer 0 for the oracle (V in token-major order)
        v_host = V[0].view(torch.int16).cpu().numpy().view(np.uint16)
        kv_for_cpu = (K[0].view(torch.int16).cpu().numpy().view(np.uint16),
                      np.ascontiguousarray(np.swapaxes(v_host, -1, -2)) if vt else v_host)
        del v_host
    # the other V page layout's attention on the same pages, same plan
    other_us = other_layout_us_per_layer(ops, not vt, q, K, V, bt, ctx, cu, par, out, ws_attn, copies,
                                         min(layers, 20))
    layouts = {("v_transposed" if vt else "token_major"): {"us_per_layer": round(attn_ms * 1e3, 2),
                                                           "pct_hbm_peak": round(100 * attn_gbs / PEAK_HBM_GBS, 1)},
               ("token_major" if vt else "v_transposed"): {
                   "us_per_layer": round(other_us, 2),
                   "pct_hbm_peak": round(100 * attn_bytes / (other_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 1)}}
    log(f"other V layout: {other_us:.2f} us/layer")

    if args.calibrate_copy_mb > 0:
        nbytes = args.calibrate_copy_mb * (1 << 20)
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {nbytes} bytes read, {nbytes} bytes written")
        del src, dst

    sweep = None
    if name == "llama3_70b_b256" and not args.no_sweep and args.batch is None:
        main_point = {"batch": B, "verify_rows": T, "us_per_layer": round(attn_ms * 1e3, 2),
                      "pct_hbm_peak": round(100 * attn_gbs / PEAK_HBM_GBS, 1),
                      "attn_kv_frac_of_ceiling": None if ceiling is None else ceiling["attn_kv_frac_of_ceiling"],
                      "accept_us": round(accept_ms * 1e3, 2), "compact_us": round(compact_ms * 1e3, 2),
                      "plan_us": round(plan_ms * 1e3, 2)}
        del K, V
        torch.cuda.empty_cache()
        main_point["other_layout_us_per_layer"] = round(other_us, 2)
        sweep = batch_sweep(args, ops, W, main_point, layers, vt)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, kv_for_cpu, logits, args.cpu_sample_requests, layers)

    traffic = measured_traffic(name, vt)
    mfma = measured_mfma(name, vt)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4),
                "algorithmic_flops": attn_flops}
    else:
        roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(attn_gbs / PEAK_HBM_GBS, 4)}
    rec = {
        "metric": "verify-step µs/layer & KV-stream HBM GB/s (% peak), Llama-3-70B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; bf16 Q/K/V, fp32 logits)",
        "launch": "eager" if graphs is None else "one HIP graph per phase (plan, layers, accept, compact)",
        "config": {"workload": WORKLOAD_TEXT.get(name, name), "name": name, "batch": B, "total_q": T,
                   "layers_per_step": layers, "kv_copies": copies, "compact_layers_per_call": copies,
                   "kv_bytes_per_layer": kv_bytes, "logits_bytes": logits_bytes},
        "us_per_layer": round(attn_ms * 1e3, 2),
        "plan_us_per_step": round(plan_ms * 1e3, 2),
        "kv_stream_gbs": round(attn_gbs, 1),
        "pct_hbm_peak": round(100 * attn_gbs / PEAK_HBM_GBS, 1),
        "accept_us": round(accept_ms * 1e3, 2),
        "accept_gbs": round(logits_bytes / (accept_ms * 1e-3) / 1e9, 1),
        "compact_us": round(compact_ms * 1e3, 2),
        "accept_compact": "one launch (spec_accept_compact)" if args.fused else "two calls (spec_accept, kv_compact)",
        "acceptance": "stochastic (speculative sampling)" if args.stochastic else "greedy",
        "verified_tokens_per_s": round(verified_tok_s, 1),
        "mean_accept_len": round(float(acc_np.mean()), 4),
        "attn_tflops": round(attn_tflops, 1),
        "attn_flop_per_byte": round(intensity, 1),
        "mfma": {"algorithmic_frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4), "peak_tflops": PEAK_MFMA_TFLOPS,
                 "counters": mfma},
        "v_layout": "transposed V page blocks (spec_verify_attn_run_vt)" if vt
                    else "token-major V pages (spec_verify_attn_run)",
        "layouts": layouts,
        "roofline": {"kernel": "%s (verify_attn_kernel + attn_merge_kernel, per layer)"
                               % ("spec_verify_attn_run_vt" if vt else "spec_verify_attn_run"),
                     **roof,
                     "algorithmic_bytes": attn_bytes,
                     "traffic": None if traffic is None else traffic["total_bytes"],
                     "traffic_detail": traffic},
        "read_ceiling": ceiling,
        "sweep": None if sweep is None else sweep["points"],
        "sps_table": None if sweep is None else sweep["sps_table"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def read_ceiling(case, ops, k_cache, v_cache, stream, attn_kv_gbs, reps=10):
    """What a pure read kernel reaches on the pages the attention streams:
    spec_hbm_read_probe over every (page, KV head) block of K and V that the
    step's units read, in the attention's order (request, head, page) and
    with its load pattern, timed with HIP events on the launch stream.  Only
    for caches far larger than the 256 MB last-level cache (else None)."""
    import torch
    if case.kv_bytes_per_layer() < 1e9:
        return None
    hkv = case.num_kv_heads
    lists = []
    for i in range(case.batch):
        npg = (int(case.context_lens[i]) + int(case.q_lens[i]) + 15) // 16
        pg = case.block_tables[i, :npg].astype(np.int64)
        lists.append((pg[None, :] * hkv + np.arange(hkv)[:, None]).ravel())
    chunks = torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(k_cache.device)
    sink = torch.zeros(ops.PROBE_SINK_WORDS, dtype=torch.int32, device=k_cache.device)
    for _ in range(3):
        ops.spec_hbm_read_probe(k_cache, v_cache, chunks, sink=sink, stream=stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ops.spec_hbm_read_probe(k_cache, v_cache, chunks, sink=sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = int(chunks.numel()) * 2 * 16 * case.head_dim * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "us": round(us, 2),
            "bytes": nbytes, "attn_kv_gbs": round(attn_kv_gbs, 1),
            "attn_kv_frac_of_ceiling": round(attn_kv_gbs / gbs, 4),
            "probe": "spec_hbm_read_probe: the step's K and V (page, head) blocks in the attention's order, "
                     "16-byte nontemporal loads, 1 KB per instruction, one pair of blocks in flight per wave"}


def chunked_bench(args, case, ops, r):
    """One verify step as a chunk loop (FASER, "Early Token Pruning"): per chunk, the
    attention of every layer over the chunk's rows, then chunk acceptance, which drops
    the requests already rejected.  The loop runs on the device from start to end: a
    chunk's rows are read and written in place in q, out and logits, the kernels read
    the chunk's row count on the device, and the host issues ceil(max q_i / C)
    iterations (it knows the draft lengths), the ones after every request has ended
    doing nothing; the whole step is captured as one graph and replayed."""
    import torch
    dev = "cuda:0"
    B, T, Vv = case.batch, case.total_q, case.vocab
    Hq, Hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    C = args.chunk
    n_iter = -(-int(np.max(case.q_lens)) // C)
    ws_a = torch.empty(ops.spec_verify_attn_workspace_size(B, T, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(ops.spec_accept_chunk_workspace_size(B, T, Vv), dtype=torch.uint8, device=dev)
    t_arg = torch.empty(T, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(T, dtype=torch.int32, device=dev)
    toks = torch.empty(T, dtype=torch.int32, device=dev)
    bufs = [(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B + 1, dtype=torch.int32, device=dev))
            for _ in range(2)]
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)

    def step(observe=None):
        ops.spec_chunk_start(r["cu"], C, total_q=T, chunk_begin=bufs[0][0], cu_chunk=bufs[0][1])
        for k in range(n_iter):
            (b, cu), (nb, ncu) = bufs[k % 2], bufs[(k + 1) % 2]
            if observe is not None:
                observe.append(int(cu[B].item()))  # (the untimed pass that counts the chunks' rows)
            ops.spec_verify_attn_chunk_plan(r["ctx"], r["cu"], b, cu, total_q=T,
                                            max_blocks_per_seq=r["bt"].shape[1], num_q_heads=Hq,
                                            num_kv_heads=Hkv, head_dim=D, num_pages=case.num_pages,
                                            workspace=ws_a)
            for layer in range(r["layers"]):
                c = layer % r["copies"]
                r["chunk_run"](r["q"], r["K"][c], r["V"][c], r["bt"], r["ctx"], r["cu"], b, cu, r["par"],
                               total_q=T, out=out, workspace=ws_a)
            ops.spec_accept_chunk(r["logits"], r["draft"], r["cu"], b, cu, r["par"], chunk_size=C,
                                  target_argmax=t_arg, accept_len=acc, accepted_path=path, out_tokens=toks,
                                  next_begin=nb, next_cu=ncu, workspace=ws_c)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / args.steps
    acc_np = acc.cpu().numpy()
    rows = []
    step(rows)
    torch.cuda.synchronize()
    # the same step unchunked (eager launches, wall clock) for comparison
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r["step_eager"](False)
    torch.cuda.synchronize()
    full_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ref_acc = r["acc"].cpu().numpy()
    return {
        "metric": "chunked verify step (FASER early pruning): ms per step, one graph replay",
        "value": round(graph_ms, 3), "unit": "ms", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"workload": WORKLOAD_TEXT.get(case.name, case.name), "name": case.name, "batch": B,
                   "total_q": T, "layers_per_step": r["layers"], "chunk_size": C},
        "iterations_per_step": n_iter,
        "chunks_with_rows_per_step": int(sum(1 for x in rows if x > 0)),
        "rows_verified_per_step": int(sum(rows)),
        "eager_ms_per_step": round(eager_ms, 3),
        "unchunked_ms_per_step_eager": round(full_ms, 3),
        "same_acceptance_as_unchunked": bool(np.array_equal(acc_np, ref_acc)),
        "mean_accept_len": round(float(acc_np.mean()), 4),
    }


TRAFFIC_SOURCES = ["speculative_decoding_verification_attn_amd/csrc/verify_attn.hip",
                   "speculative_decoding_verification_attn_amd/csrc/sv_device.h",
                   "speculative_decoding_verification_attn_amd/csrc/sv_internal.h"]


def _sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def _pmc_per_kernel(run_dir, counter):
    """({kernel name: [value per dispatch]}, value of the last dispatch) from a
    rocprofv3 --pmc csv directory."""
    import csv
    import glob
    out, last = {}, (-1, None)
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                v = float(r["Counter_Value"])
                out.setdefault(r["Kernel_Name"], []).append(v)
                if int(r["Dispatch_Id"]) > last[0]:
                    last = (int(r["Dispatch_Id"]), v)
    if not out:
        raise SystemExit(f"no {counter} records under {run_dir}")
    return out, last[1]


def _timed_attention_kernel(per_kernel, vt):
    """The attention kernel instantiation of the timed V layout (template
    argument true: transposed V page blocks); the run also launches the other
    layout's instantiation for its side-by-side timing."""
    tag = "true>" if vt else "false>"
    names = [k for k in per_kernel if "verify_attn_kernel" in k and tag in k]
    return names[0] if names else None


def write_traffic_summary(name, fetch_dir, write_dir, copy_mb, vt=True):
    """HBM traffic per launch of the attention kernel: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for
    the plain device copy of copy_mb MiB that the profiled run ends with."""
    # the calibration copy is the profiled run's last dispatch
    fetch, fetch_copy = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write, write_copy = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mb * (1 << 20)
    fetch_scale = copy_bytes / (fetch_copy * 1024.0)
    write_scale = copy_bytes / (write_copy * 1024.0)
    kname = _timed_attention_kernel(fetch, vt)
    if kname is None:
        raise SystemExit(f"{fetch_dir}: no attention kernel of the {'transposed' if vt else 'token-major'} layout")
    f_kib = float(np.mean(fetch[kname]))
    w_kib = float(np.mean(write[kname]))
    rec = {
        "kernel": kname, "workload": name, "v_transposed": vt,
        "source_sha256": _sources_sha256(TRAFFIC_SOURCES), "sources": TRAFFIC_SOURCES,
        "fetch_kib_per_launch": round(f_kib, 1), "write_kib_per_launch": round(w_kib, 1),
        "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
        "read_bytes_per_launch": int(f_kib * 1024 * fetch_scale),
        "write_bytes_per_launch": int(w_kib * 1024 * write_scale),
        "calibration": {"copy_bytes": copy_bytes, "fetch_kib": round(fetch_copy, 1),
                        "write_kib": round(write_copy, 1)},
        "other_kernels_kib_per_launch": {k: {"fetch": round(float(np.mean(v)), 1),
                                             "write": round(float(np.mean(write.get(k, [0]))), 1)}
                                         for k, v in fetch.items() if "sv::" in k and k != kname},
    }
    path = os.path.join(ROOT, "profiles", f"verify_attn_{name}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def write_sps_summary(bench_json):
    """The SPS(B) table of a default run (70B-shape batch sweep) as the cost table
    the verify-budget scheduler reads: verify rows -> verify steps per second."""
    line = [ln for ln in open(bench_json).read().splitlines() if ln.strip().startswith("{")][-1]
    rec = json.loads(line)
    t = rec["sps_table"]
    out = {"workload": "Llama-3-70B attention geometry (64/8 heads, D=128), chains gamma=3, contexts U[2048,8192], "
                       "batch 16..256",
           "rows": t["rows"], "steps_per_s": t["steps_per_s"], "definition": t["definition"],
           "points": rec["sweep"], "v_layout": rec.get("v_layout"),
           "command": "python bench.py  (default run; this file: python bench.py --sps-summary <its JSON line>)"}
    path = os.path.join(ROOT, "profiles", "sps_table_llama3_70b.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def write_mfma_summary(name, pmc_dir, vt=True):
    """MFMA use of the attention kernel from one rocprofv3 --pmc run.
    SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs (a 32x32x16 bf16 MFMA
    counts 32 cycles, so 1024 SIMDs busy all the time is the 2.5 PFLOP/s
    peak); GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the dispatch lasted
    GRBM_GUI_ACTIVE / 8 cycles (profiler set-up included, which inflates it
    for short kernels).  SQ_WAVE_CYCLES counts the kernel's resident
    wave-cycles in units of 4 cycles; with one wave per SIMD that is the SIMD
    time the kernel held."""
    counters = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU",
                "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_WAVES", "SQ_BUSY_CYCLES"]
    got = {}
    kname = None
    for c in counters:
        try:
            per, _ = _pmc_per_kernel(pmc_dir, c)
        except SystemExit:
            continue
        k = _timed_attention_kernel(per, vt)
        if k is None:
            continue
        kname = k
        got[c] = float(np.mean(per[k]))
    need = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
    if kname is None or any(c not in got for c in need):
        raise SystemExit(f"{pmc_dir}: needs {need} for the attention kernel")
    busy = got["SQ_VALU_MFMA_BUSY_CYCLES"] / (got["GRBM_GUI_ACTIVE"] / MI355X_XCDS * MI355X_SIMDS)
    rec = {"kernel": kname, "workload": name, "v_transposed": vt,
           "source_sha256": _sources_sha256(TRAFFIC_SOURCES), "sources": TRAFFIC_SOURCES,
           "counters_per_launch": {c: round(v, 1) for c, v in got.items()},
           "simds": MI355X_SIMDS, "xcds": MI355X_XCDS,
           "mfma_busy_frac": round(busy, 4),
           "mfma_busy_cycles_per_instruction": round(got["SQ_VALU_MFMA_BUSY_CYCLES"] / got["SQ_INSTS_MFMA"], 2)}
    if "SQ_WAVE_CYCLES" in got:
        rec["mfma_busy_frac_of_resident_wave_cycles"] = round(
            got["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * got["SQ_WAVE_CYCLES"]), 4)
    if "SQ_WAVE_CYCLES" in got and "SQ_ACTIVE_INST_VALU" in got:
        rec["valu_active_frac_of_wave_cycles"] = round(got["SQ_ACTIVE_INST_VALU"] / got["SQ_WAVE_CYCLES"], 4)
    if "SQ_WAVE_CYCLES" in got and "SQ_WAIT_ANY" in got:
        rec["wait_frac_of_wave_cycles"] = round(got["SQ_WAIT_ANY"] / got["SQ_WAVE_CYCLES"], 4)
    path = os.path.join(ROOT, "profiles", f"verify_attn_{name}_mfma.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def measured_mfma(name, vt):
    """MFMA busy fraction of the attention kernel from the committed counter
    summary, if taken on this workload, V layout and the current kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"verify_attn_{name}_mfma.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if _sources_sha256(rec["sources"]) != rec["source_sha256"] or rec.get("v_transposed") != vt:
        return None
    return {"busy_frac": rec["mfma_busy_frac"],
            "busy_frac_of_resident_wave_cycles": rec.get("mfma_busy_frac_of_resident_wave_cycles"),
            "source": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs x %d SIMDs)"
                      % (rec["xcds"], rec["simds"])}


def measured_traffic(name, vt):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on this
    workload, V layout and the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"verify_attn_{name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if _sources_sha256(rec["sources"]) != rec["source_sha256"] or rec.get("v_transposed") != vt:
        return None
    return {"read_bytes": rec["read_bytes_per_launch"], "write_bytes": rec["write_bytes_per_launch"],
            "total_bytes": rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"],
            "source": "rocprofv3 --pmc FETCH_SIZE x%.4f, WRITE_SIZE x%.4f (plain-copy calibration)"
                      % (rec["fetch_scale"], rec["write_scale"])}


def _oracle_step_times(oracle, case, k, v, logits, n_req):
    """One layer of the oracle's verify attention over the first n_req requests
    and argmax + acceptance of their rows: (attention s, acceptance s, keys,
    rows)."""
    n_req = min(n_req or case.batch, case.batch)
    rows = np.arange(int(case.cu_q[0]), int(case.cu_q[n_req]))
    cu = case.cu_q[:n_req + 1]
    tp = None if case.tree_parent is None else case.tree_parent[rows]
    t0 = time.perf_counter()
    oracle.verify_attn(case.q[rows], k, v, case.block_tables[:n_req], case.context_lens[:n_req], cu, tp,
                       num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                       head_dim=case.head_dim, page_size=case.page_size, num_pages=case.num_pages)
    t_attn = time.perf_counter() - t0
    t0 = time.perf_counter()
    tg = oracle.argmax(logits[rows])
    oracle.accept(case.draft_tokens[rows], tg, cu, tp)
    t_acc = time.perf_counter() - t0
    keys = int(np.sum(case.context_lens[:n_req].astype(np.int64) + case.q_lens[:n_req]))
    return t_attn, t_acc, keys, len(rows)


def cpu_baseline(case, kv_host, logits_dev, n_req, layers):
    """The oracle, as it stands, on the same workload: verify attention of the
    whole batch (one layer, scaled to the step's layers) plus argmax and
    acceptance of every row, on the host's cores (OpenMP over (request, KV
    head); the thread count is OpenMP's default, i.e. OMP_NUM_THREADS when
    set).  Reported in GB/s of the same algorithmic bytes as the GPU figure.
    Also one thread on each of the three batch-1 workloads."""
    import oracle
    from speculative_decoding_verification_attn_amd import workloads as W

    k, v = kv_host
    lg = logits_dev.cpu().numpy() if case.logits is None else case.logits
    threads = oracle.set_threads(0)
    t_attn, t_acc, keys, n_rows = _oracle_step_times(oracle, case, k, v, lg, n_req)
    n = min(n_req or case.batch, case.batch)
    attn_bytes = keys * case.num_kv_heads * case.head_dim * 4 + n_rows * case.num_q_heads * case.head_dim * 4
    logit_bytes = n_rows * case.vocab * 4
    t_step = layers * t_attn + t_acc
    gbs = (layers * attn_bytes + logit_bytes) / t_step / 1e9
    log(f"cpu oracle: {n} requests on {threads} threads, attention {t_attn:.2f}s/layer, accept {t_acc:.3f}s")
    single = {}
    oracle.set_threads(1)
    try:
        for nm in ("tiny_chain", "llama31_8b_chain", "llama3_70b_tree"):
            c = W.make_case(nm)
            ta, tc, _, _ = _oracle_step_times(oracle, c, c.k_cache, c.v_cache, c.logits, 0)
            single[nm] = {"attn_s_per_layer": round(ta, 4), "accept_s": round(tc, 4)}
            log(f"cpu oracle, 1 thread, {nm}: attention {ta:.3f}s/layer, accept {tc:.4f}s")
    finally:
        oracle.set_threads(threads)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model,
            "cpus_in_affinity": affinity,
            "sample": f"{'all' if n == case.batch else 'first %d of' % n} {case.batch} requests "
                      f"({n_rows} verify rows, {keys} keys/layer): one layer of fp64 verify attention timed "
                      f"and scaled to {layers} layers, plus argmax+acceptance of those rows; C oracle, "
                      f"attention in parallel over (request, KV head) on {threads} threads",
            "attn_s_per_layer": round(t_attn, 3), "accept_s": round(t_acc, 4),
            "single_thread": single}


def other_layout_us_per_layer(ops, vt, q, K, V, bt, ctx, cu, par, out, ws, copies, n_layers, reps=5):
    """Attention time per layer with the other V page layout: the resident V
    copies re-laid out, then a graph of n_layers runs (the plan already in ws)
    replayed `reps` times."""
    import torch
    Vo = torch.empty(tuple(V.shape[:-2]) + (V.shape[-1], V.shape[-2]), dtype=V.dtype, device=V.device)
    for c in range(copies):
        Vo[c].copy_(V[c].transpose(-1, -2))
    run = ops.spec_verify_attn_run_vt if vt else ops.spec_verify_attn_run

    def layers_fn():
        for layer in range(n_layers):
            c = layer % copies
            run(q, K[c], Vo[c], bt, ctx, cu, par, out=out, workspace=ws)

    layers_fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layers_fn()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps / n_layers
    del g, Vo
    torch.cuda.empty_cache()
    return us


def batch_sweep(args, ops, W, main_point, layers, vt, timed_layers=20, reps=5):
    """Verify-attention time per layer at the Llama-3-70B shape over batches
    (the large-batch workload's distributions, batch overridden), each in its
    own run of graph replays over resident caches, with acceptance,
    compaction and the plan of one step; the read-ceiling probe beside it for
    caches of 1 GB or more.  The largest batch is the main measurement.  From
    the points: the verify path's steps per second at each row count (the
    SPS table a verify-budget scheduler consumes; the model's GEMMs are not
    part of it)."""
    import torch
    dev = "cuda:0"
    points = []
    for Bs in SWEEP_BATCHES:
        if Bs == main_point["batch"]:
            points.append(main_point)
            continue
        case = W.make_case("llama3_70b_b256", None, kv_device=dev, logits_device=dev, batch=Bs)
        kvb = case.kv_bytes_per_layer()
        copies = max(2, int(np.ceil(1.0e9 / kvb)))
        v_src = case.v_cache_dev.transpose(-1, -2) if vt else case.v_cache_dev
        K = torch.empty((copies,) + tuple(case.k_cache_dev.shape), dtype=torch.bfloat16, device=dev)
        V = torch.empty((copies,) + tuple(v_src.shape), dtype=torch.bfloat16, device=dev)
        for c in range(copies):
            K[c].copy_(case.k_cache_dev)
            V[c].copy_(v_src)
        del v_src
        case.k_cache_dev = case.v_cache_dev = None
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        q = torch.from_numpy(np.ascontiguousarray(case.q).view(np.int16)).to(dev).view(torch.bfloat16)
        bt, ctx, cu = i32(case.block_tables), i32(case.context_lens), i32(case.cu_q)
        draft = i32(case.draft_tokens)
        T = case.total_q
        out = torch.empty_like(q)
        ws = torch.empty(ops.spec_verify_attn_workspace_size(Bs, T, case.num_q_heads, case.num_kv_heads,
                                                             case.head_dim), dtype=torch.uint8, device=dev)
        ws_acc = torch.empty(ops.spec_accept_workspace_size(Bs, T, case.vocab), dtype=torch.uint8, device=dev)
        acc = torch.empty(Bs, dtype=torch.int32, device=dev)
        path = torch.empty(T, dtype=torch.int32, device=dev)

        def plan():
            ops.spec_verify_attn_plan(ctx, cu, max_blocks_per_seq=bt.shape[1], num_q_heads=case.num_q_heads,
                                      num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                                      num_pages=case.num_pages, total_q=T, workspace=ws)

        def attn():
            for layer in range(timed_layers):
                c = layer % copies
                (ops.spec_verify_attn_run_vt if vt else ops.spec_verify_attn_run)(
                    q, K[c], V[c], bt, ctx, cu, None, out=out, workspace=ws)

        def accept():
            ops.spec_accept(case.logits_dev, draft, cu, None, accept_len=acc, accepted_path=path, workspace=ws_acc)

        def compact():
            (ops.kv_compact_vt if vt else ops.kv_compact)(K, V, bt, ctx, cu, path, acc, num_layers=copies)

        plan(); attn(); accept(); compact()
        torch.cuda.synchronize()
        graphs = {}
        for nm, fn in (("plan", plan), ("attn", attn), ("accept", accept), ("compact", compact)):
            graphs[nm] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[nm]):
                fn()
        us = {}
        for nm, g in graphs.items():
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us[nm] = e0.elapsed_time(e1) * 1e3 / reps
        us_layer = us["attn"] / timed_layers
        attn_bytes = kvb + case.qo_bytes() + int(sum(((int(L) + int(qq) + 15) // 16) * 4
                                                     for L, qq in zip(case.context_lens, case.q_lens)))
        gbs = attn_bytes / (us_layer * 1e-6) / 1e9
        ceiling = read_ceiling(case, ops, K[0], V[0], torch.cuda.current_stream(), kvb / (us_layer * 1e-6) / 1e9)
        other = other_layout_us_per_layer(ops, not vt, q, K, V, bt, ctx, cu, None, out, ws, copies, timed_layers)
        pt = {"batch": Bs, "verify_rows": T, "us_per_layer": round(us_layer, 2),
              "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1), "other_layout_us_per_layer": round(other, 2),
              "attn_kv_frac_of_ceiling": None if ceiling is None else ceiling["attn_kv_frac_of_ceiling"],
              "accept_us": round(us["accept"], 2), "compact_us": round(us["compact"], 2),
              "plan_us": round(us["plan"], 2)}
        points.append(pt)
        log(f"sweep B={Bs}: {pt['us_per_layer']} us/layer, {pt['pct_hbm_peak']} % of 8 TB/s")
        del K, V, graphs, case
        torch.cuda.empty_cache()
    rows, sps = [], []
    for pt in points:
        t_step_us = layers * pt["us_per_layer"] + pt["accept_us"] + pt["compact_us"] + pt["plan_us"]
        pt["verify_steps_per_s"] = round(1e6 / t_step_us, 2)
        rows.append(pt["verify_rows"])
        sps.append(pt["verify_steps_per_s"])
    table = {"rows": rows, "steps_per_s": sps,
             "definition": f"verify steps per second of this path at the Llama-3-70B shape ({layers} layers of "
                           "verify attention + plan + acceptance + compaction per step, graph replays); the "
                           "model's GEMMs are not included"}
    return {"points": points, "sps_table": table}


if __name__ == "__main__":
    main()
