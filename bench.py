#!/usr/bin/env python3
"""Benchmark: block top-k sparse decode attention, one layer, one MI355X.

A step is one whole sparse decode step of one layer for a batch of
sequences, run through the C ABI of libkin.so back to back on one stream:
newest-block summary update -> block scores -> top-k -> sparse attention
(+ split combine).  Steps rotate over several independent layers (each with
its own cache, summaries and queries) so that consecutive steps never find
the previous step's bytes in the 256 MB Infinity Cache, as in a real decode
where the other layers run in between.  Inputs are resident in HBM before
the timed region starts.

Prints ONE JSON line (rank 0).  value = queries/s/layer = batch / step time.
"""
import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_top_sparse_amd import binding as kb  # noqa: E402
from block_top_sparse_amd import synth, workloads  # noqa: E402
from block_top_sparse_amd.buffers import LayerBuffers  # noqa: E402

METRIC = "sparse decode-attn queries/s/layer + achieved HBM GB/s vs peak (1 GPU)"
PEAK_HBM_GBS = 8000.0


# committed HBM counter summaries of the step kernel, per workload
TRAFFIC_FILES = {
    workloads.QWEN3_8B.name: "k_decode_step_qwen3-8b_counters.md",
    workloads.QWEN3_14B.name: "k_decode_step_qwen3-14b_counters.md",
    workloads.QWEN3_32B.name: "k_decode_step_qwen3-32b_counters.md",
}


def stored_traffic(w):
    """HBM bytes per launch of k_decode_step from the committed rocprofv3
    counter summary under profiles/ (FETCH_SIZE + WRITE_SIZE, each scaled by
    a plain copy's reading), only for the workload it was taken on and only
    while the kernel sources still hash to the recorded value; else None.
    Returns (bytes, file name)."""
    import hashlib

    name = TRAFFIC_FILES.get(w.name)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None, None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    try:
        srcs = fields["kernel_sources"].split()
        h = hashlib.sha256()
        for src in srcs:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None, None
        return int(fields["traffic_bytes_per_launch"]), "profiles/" + name
    except (KeyError, OSError, ValueError):
        return None, None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_layers(w, n_layers, with_dense):
    layers = []
    for l in range(n_layers):
        inp = synth.make_inputs(w, device="cuda", seed=w.seed + 7919 * l)
        bufs = LayerBuffers(w, with_dense=with_dense)
        kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, w.ctx_len)  # prefill
        layers.append((inp, bufs))
        torch.cuda.synchronize()
        log(f"layer {l}: cache {w.cache_bytes() / 2**30:.2f} GiB ready")
    return layers


def sparse_step(w, inp, bufs, ev=None, scores=False):
    """One decode step of one layer through kin_sparse_decode_step (one
    kernel when there are enough pairs, else two), events around it.  The
    step returns idx and out; the fp64 scores are written out only with
    scores=True (they are not part of the method's output)."""
    if ev is not None:
        ev[0].record()
    kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S,
                              bufs.scores if scores else None, bufs.k, bufs.idx, bufs.out,
                              bufs.ws)
    if ev is not None:
        ev[1].record()


def two_kernel_step(w, inp, bufs, ev=None):
    """The same step as its two fused halves, an event between them."""
    d = bufs.desc
    if ev is not None:
        ev[0].record()
    kb.kin_decode_update_score(d, inp["q"], inp["K"], bufs.S, bufs.scores)
    if ev is not None:
        ev[1].record()
    kb.kin_decode_select_attend(d, inp["q"], inp["K"], inp["V"], bufs.scores, bufs.k, bufs.idx,
                                bufs.out, bufs.ws)
    if ev is not None:
        ev[2].record()


def unfused_step(w, inp, bufs, ev=None):
    """The same step as four separate calls (one kernel each, plus combine)."""
    d, L = bufs.desc, w.ctx_len
    kb.kin_block_summary_update(d, inp["K"], bufs.S, L - 1, L)
    kb.kin_block_score(d, inp["q"], bufs.S, bufs.scores)
    kb.kin_block_topk(d, bufs.scores, bufs.k, bufs.idx)
    kb.kin_sparse_decode_attn(d, inp["q"], inp["K"], inp["V"], bufs.idx, bufs.k, bufs.out,
                              bufs.ws)


def dense_step(w, inp, bufs, ev=None):
    kb.kin_dense_decode_attn(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.out_dense,
                             bufs.ws_dense)


def time_steps(fn, layers, steps, warmup, n_events=0):
    """fn(inp, bufs, events_or_None); returns (ms per step, per-stage ms)."""
    for s in range(warmup):
        fn(*layers[s % len(layers)], None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        fn(*layers[s % len(layers)], evs[s] if n_events else None)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    stage_ms = []
    if n_events:
        for i in range(n_events - 1):
            stage_ms.append(sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps)
    return total_ms / steps, stage_ms


def step_distribution(fn, layers, steps):
    """A second pass of `steps` steps with an event recorded before each step
    and after the last one (same stream, no host gap): per-step durations in
    microseconds -> median, p10, p90 (nearest rank), mean, std."""
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for s_ in range(steps):
        evs[s_].record()
        fn(*layers[s_ % len(layers)], None)
    evs[steps].record()
    torch.cuda.synchronize()
    us = sorted(evs[i].elapsed_time(evs[i + 1]) * 1000.0 for i in range(steps))
    n = len(us)

    def rank(p):
        return us[min(n - 1, max(0, math.ceil(p * n) - 1))]

    mean = sum(us) / n
    std = math.sqrt(sum((x - mean) ** 2 for x in us) / max(1, n - 1))
    return {"n": n, "median_us": round(rank(0.5), 2), "p10_us": round(rank(0.1), 2),
            "p90_us": round(rank(0.9), 2), "mean_us": round(mean, 2), "std_us": round(std, 2)}


def read_peak(nbytes=4 * 2**30, reps=20):
    """Measured read bandwidth of this device: kin_hbm_read_probe (a plain
    streaming read of every 16-byte word once) over a buffer far larger than
    the Infinity Cache, the median of `reps` timed launches.  Returns GB/s."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        kb.kin_hbm_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        kb.kin_hbm_read_probe(buf, nbytes, sink)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)[reps // 2]
    del buf
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def layers_for(w, requested=0):
    """Layers rotated: enough that one round of steps moves >= 1 GiB (so the
    Infinity Cache holds no previous step's bytes), within 150 GiB of HBM."""
    n = requested or max(2, min(8, math.ceil(2**30 / w.bytes_sparse_step())))
    cap = max(1, int(150 * 2**30 // (w.cache_bytes() + w.summary_bytes())))
    return min(n, cap)


def single_kernel(w, num_cu):
    return w.dtype == "bf16" and w.pairs >= num_cu and w.nb <= 8192 and w.topk <= 2048


def step_kernels(w, num_cu):
    """The launches of one kin_sparse_decode_step without a scores output, as
    the library plans them: "one" (the whole step per pair), "one-f32" (the
    fp32 step of at most 1 MiB per pair in one kernel, split over several
    workgroups per pair), "one-split" (a step that keeps every block, few
    pairs: select + split attention alone), "two" (score tiles, then select
    + split attention), "four" (more than 2048 kept blocks: scores or the
    newest row, top-k, attention, combine)."""
    if single_kernel(w, num_cu):
        return "one"
    if w.topk > 2048:
        return "four"
    if w.dtype == "f32":
        keff = min(w.topk, w.nb)
        small = w.nb <= 8192 and w.nb * 512 + keff * w.block * 1024 <= 1 << 20
        return "one-f32" if small else "two"
    return "one-split" if w.topk >= w.nb else "two"


def run_sweep(args):
    """The budget/length grid: per point, kin_sparse_decode_step timed back to
    back over rotated layers, as for the headline workload."""
    pts = workloads.sweep()
    if args.sweep == "big":
        pts = [w for w in pts if w.bytes_sparse_step() >= 256 * 2**20]
    if args.sweep_batch:
        pts = [w for w in pts if w.batch == args.sweep_batch]
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    for w in pts:
        n_layers = layers_for(w, args.layers)
        layers = make_layers(w, n_layers, with_dense=False)
        est_us = w.bytes_sparse_step() / 5e12 * 1e6
        steps = max(10, min(args.steps, int(2e5 / est_us)))
        ms, _ = time_steps(lambda i, b, e: sparse_step(w, i, b, None), layers, steps,
                           max(3, steps // 5))
        gbs = w.bytes_sparse_step() / (ms * 1e-3) / 1e9
        print(json.dumps({"workload": w.name, "batch": w.batch, "ctx_len": w.ctx_len,
                          "block": w.block, "topk_blocks": w.topk, "pairs": w.pairs,
                          "step_bytes": w.bytes_sparse_step(), "steps": steps,
                          "layers_rotated": n_layers, "ms_per_step": round(ms, 5),
                          "queries_per_s": round(w.batch / (ms * 1e-3), 1),
                          "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                          "kernels": step_kernels(w, num_cu)}), flush=True)
        del layers
        torch.cuda.empty_cache()


def run_token(args, w):
    """Token-level top-k (block 1): kin_token_decode_step timed like the
    block step, over rotated layers; one JSON line."""
    n_layers = layers_for(w, args.layers)
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    nws = kb.kin_token_ws_bytes(desc, w.topk)
    layers = []
    for l in range(n_layers):
        inp = synth.make_inputs(w, device="cuda", seed=w.seed + 7919 * l)
        bufs = {"idx": torch.empty((w.batch, w.hkv, w.topk), dtype=torch.int32, device="cuda"),
                "out": torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda"),
                "ws": torch.zeros(nws, dtype=torch.uint8, device="cuda")}
        layers.append((inp, bufs))
        torch.cuda.synchronize()
        log(f"layer {l}: cache {w.cache_bytes() / 2**30:.2f} GiB ready")

    def step(inp, b, ev):
        kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], None, w.topk, b["idx"],
                                 b["out"], b["ws"])

    ms, _ = time_steps(step, layers, args.steps, args.warmup)
    step_bytes = w.bytes_sparse_step()
    gbs = step_bytes / (ms * 1e-3) / 1e9
    res = {"metric": METRIC, "value": round(w.batch / (ms * 1e-3), 1), "unit": "queries/s/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": dict(w.describe(), layers_rotated=n_layers,
                          step_outputs="out, idx (fp64 scores not written)"),
           "step_bytes": step_bytes, "hbm_gbs": round(gbs, 1),
           "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "roofline": {"bound": "hbm", "kernel": "k_tok_score + k_tok_select_attend (two "
                        "launches)", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "bytes_per_launch": step_bytes, "avg_us": round(ms * 1000, 2)}}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, layers[0], args.cpu_seqs)
    print(json.dumps(res), flush=True)


def run_paged(args, w):
    """Variable lengths in a paged cache: kin_paged_decode_step timed like the
    block step over rotated layers; lengths drawn once (seeded) from
    N(ctx_len - 3 sd, sd) clipped to [1, ctx_len]; every sequence's pages
    scattered over one shuffled pool.  Algorithmic bytes are summed over the
    sequences' own lengths.  One JSON line."""
    n_layers = layers_for(w, args.layers)
    g = torch.Generator().manual_seed(w.seed)
    mean = w.ctx_len - 3 * w.len_std
    lens = (torch.randn(w.batch, generator=g) * w.len_std + mean).round().clamp(1, w.ctx_len)
    lens = lens.to(torch.int32)
    P = w.page_size
    max_pages = (w.ctx_len + P - 1) // P
    cap = max_pages * P
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, cap, w.ctx_len, w.block, torch.bfloat16)
    used = [(int(L) + P - 1) // P for L in lens.tolist()]
    layers = []
    for l in range(n_layers):
        inp = synth.make_inputs(w.scaled(t_cap=cap), device="cuda", seed=w.seed + 7919 * l)
        num_pages = sum(used)
        perm = torch.randperm(num_pages, generator=g).tolist()
        table = torch.zeros((w.batch, max_pages), dtype=torch.int32)
        Kp = torch.empty((num_pages, w.hkv, P, 128), dtype=torch.bfloat16, device="cuda")
        Vp = torch.empty_like(Kp)
        nxt = 0
        for b in range(w.batch):
            for p_ in range(used[b]):
                pg = perm[nxt]
                nxt += 1
                Kp[pg] = inp["K"][b, :, p_ * P:(p_ + 1) * P]
                Vp[pg] = inp["V"][b, :, p_ * P:(p_ + 1) * P]
                table[b, p_] = pg
        lens_d, table_d = lens.cuda(), table.cuda()
        pages = kb.make_pages(lens_d, table_d, P, max_pages, num_pages)
        bufs = LayerBuffers(w.scaled(t_cap=cap))
        kb.kin_paged_summary_update(desc, pages, Kp, bufs.S, 0, w.ctx_len)
        q = inp["q"]
        del inp
        layers.append(({"q": q, "K": Kp, "V": Vp},
                       {"bufs": bufs, "pages": pages, "keep": (lens_d, table_d)}))
        torch.cuda.synchronize()
        log(f"layer {l}: {num_pages} pages of {P} tokens ready")

    def step(inp, b, ev):
        d = b["bufs"]
        kb.kin_paged_decode_step(desc, b["pages"], inp["q"], inp["K"], inp["V"], d.S, None, d.k,
                                 d.idx, d.out, d.ws)

    ms, _ = time_steps(step, layers, args.steps, args.warmup)
    step_bytes = sum(w.scaled(batch=1, ctx_len=int(L)).bytes_sparse_step() for L in lens.tolist())
    gbs = step_bytes / (ms * 1e-3) / 1e9
    res = {"metric": METRIC, "value": round(w.batch / (ms * 1e-3), 1), "unit": "queries/s/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": dict(w.describe(), page_size=P, len_mean=round(float(lens.float().mean()), 1),
                          len_std=round(float(lens.float().std()), 1), len_min=int(lens.min()),
                          len_max=int(lens.max()), layers_rotated=n_layers),
           "step_bytes": step_bytes, "hbm_gbs": round(gbs, 1),
           "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    print(json.dumps(res), flush=True)


def run_quest(args, w):
    """Quest-style representative: kin_quest_decode_step timed like the
    block step over rotated layers; one JSON line."""
    n_layers = layers_for(w, args.layers)
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, w.block, torch.bfloat16)
    nws = kb.kin_quest_ws_bytes(desc, w.topk)
    layers = []
    for l in range(n_layers):
        inp = synth.make_inputs(w, device="cuda", seed=w.seed + 7919 * l)
        Sq = torch.empty((w.batch, w.hkv, w.nb_cap, 2, 128), dtype=torch.bfloat16, device="cuda")
        kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, w.ctx_len)
        bufs = {"Sq": Sq,
                "idx": torch.empty((w.batch, w.hkv, w.topk), dtype=torch.int32, device="cuda"),
                "out": torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda"),
                "ws": torch.zeros(nws, dtype=torch.uint8, device="cuda")}
        layers.append((inp, bufs))
        torch.cuda.synchronize()
        log(f"layer {l}: cache {w.cache_bytes() / 2**30:.2f} GiB ready")

    def step(inp, b, ev):
        kb.kin_quest_decode_step(desc, inp["q"], inp["K"], inp["V"], b["Sq"], None, w.topk,
                                 b["idx"], b["out"], b["ws"])

    ms, _ = time_steps(step, layers, args.steps, args.warmup)
    step_bytes = w.bytes_sparse_step()
    gbs = step_bytes / (ms * 1e-3) / 1e9
    res = {"metric": METRIC, "value": round(w.batch / (ms * 1e-3), 1), "unit": "queries/s/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": dict(w.describe(), representative="quest (channel-wise min/max)",
                          layers_rotated=n_layers),
           "step_bytes": step_bytes, "hbm_gbs": round(gbs, 1),
           "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "roofline": {"bound": "hbm", "kernel": "k_quest_tiles + k_select_attend (two "
                        "launches)", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "bytes_per_launch": step_bytes, "avg_us": round(ms * 1000, 2)}}
    print(json.dumps(res), flush=True)


def run_shared(args, w):
    """Shared-prompt Best-of-N: kin_shared_decode_step timed like the block
    step over rotated layers (each with its own prompts and samples), and the
    same tokens laid out as one contiguous cache per sample through
    kin_sparse_decode_step for comparison; one JSON line."""
    n_layers = layers_for(w, args.layers)
    P, n_prompts = w.prompt_len, w.batch // w.share_n
    wp = workloads.Workload(w.name + "-prompts", batch=n_prompts, hq=w.hq, hkv=w.hkv,
                            ctx_len=P, block=w.block, topk=1, dtype=w.dtype, seed=w.seed + 1)
    desc_p = kb.make_desc(n_prompts, w.hkv, w.gqa, P, P, w.block, torch.bfloat16)
    layers = []
    for l in range(n_layers):
        own = synth.make_inputs(w, device="cuda", seed=w.seed + 7919 * l)
        pr = synth.make_inputs(wp, device="cuda", seed=wp.seed + 7919 * l)
        grp = torch.arange(w.batch, device="cuda") // w.share_n
        own["K"][:, :, :P] = pr["K"][grp]  # the contiguous copy holds the prompt too
        own["V"][:, :, :P] = pr["V"][grp]
        bufs = LayerBuffers(w)
        kb.kin_block_summary_update(bufs.desc, own["K"], bufs.S, 0, w.ctx_len)
        Sp = torch.empty((n_prompts, w.hkv, P // w.block, 128), dtype=torch.bfloat16,
                         device="cuda")
        kb.kin_block_summary_update(desc_p, pr["K"], Sp, 0, P)
        share = kb.make_share(w.share_n, P, pr["K"], pr["V"], Sp)
        layers.append((own, {"bufs": bufs, "share": share, "keep": (pr, Sp)}))
        torch.cuda.synchronize()
        log(f"layer {l}: cache {w.cache_bytes() / 2**30:.2f} GiB ready")

    def shared_step(inp, b, ev):
        d = b["bufs"]
        kb.kin_shared_decode_step(d.desc, b["share"], inp["q"], inp["K"], inp["V"], d.S, None,
                                  d.k, d.idx, d.out, d.ws)

    def plain_step(inp, b, ev):
        d = b["bufs"]
        kb.kin_sparse_decode_step(d.desc, inp["q"], inp["K"], inp["V"], d.S, None, d.k, d.idx,
                                  d.out, d.ws)

    ms, _ = time_steps(shared_step, layers, args.steps, args.warmup)
    ms_plain, _ = time_steps(plain_step, layers, args.steps, args.warmup)
    step_bytes = w.bytes_sparse_step()
    gbs = step_bytes / (ms * 1e-3) / 1e9
    plain_bytes = workloads.Workload(w.name, batch=w.batch, hq=w.hq, hkv=w.hkv, ctx_len=w.ctx_len,
                                     block=w.block, topk=w.topk, dtype=w.dtype,
                                     seed=w.seed).bytes_sparse_step()
    res = {"metric": METRIC, "value": round(w.batch / (ms * 1e-3), 1), "unit": "queries/s/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": dict(w.describe(), share_n=w.share_n, prompt_len=P,
                          layers_rotated=n_layers),
           "step_bytes": step_bytes, "hbm_gbs": round(gbs, 1),
           "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "unshared": {"ms_per_step": round(ms_plain, 5), "step_bytes": plain_bytes,
                        "hbm_gbs": round(plain_bytes / (ms_plain * 1e-3) / 1e9, 1)},
           "speedup_vs_unshared": round(ms_plain / ms, 3)}
    print(json.dumps(res), flush=True)


def cpu_share():
    """Threads the oracle may use: the CPUs this process may run on, at most
    16 (the host CPU share that comes with one GPU; the host's other CPUs
    belong to other GPUs' work).  Returns (threads, host CPUs, usable CPUs)."""
    host = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = host
    return max(1, min(16, usable)), host, usable


def _oracle_rate(w, q, K, V, S, nthreads, min_seconds):
    """Time the oracle's step (newest-block summary update + scores + top-k +
    attention) over the given sequences until min_seconds have passed."""
    import oracle

    n = q.shape[0]
    reps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        S, _ = oracle.block_summary(K, w.block, w.ctx_len, t_begin=w.ctx_len - 1, t_end=w.ctx_len,
                                    S=S, nthreads=nthreads)
        sc = oracle.block_score(q, S, w.gqa, w.nb, nthreads=nthreads)
        idx, _ = oracle.block_topk(sc, w.nb, w.topk, nthreads=nthreads)
        oracle.decode_attention(q, K, V, w.gqa, w.ctx_len, w.block, idx=idx, nthreads=nthreads)
        dt += time.perf_counter() - t0
        reps += 1
    return n * reps / dt, reps, dt


def cpu_baseline(w, layer, max_seqs, min_seconds=10.0, single_seqs=2, single_seconds=5.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    newest-block summary update + scores + selection + attention for the
    first `max_seqs` sequences of one layer (all their KV heads), summaries
    prebuilt outside the timed region; repeated until at least min_seconds
    of CPU work have been timed, the rate averaged over all repetitions.
    Run on the host's CPU share (cpu_share), and once more on one thread
    over the first `single_seqs` sequences."""
    import oracle

    inp = layer[0]
    n = min(max_seqs, w.batch)
    nthreads, host, usable = cpu_share()
    q = inp["q"][:n].cpu()
    K = inp["K"][:n].cpu()
    V = inp["V"][:n].cpu()
    S, _ = oracle.block_summary(K, w.block, w.ctx_len, nthreads=nthreads)
    rate, reps, dt = _oracle_rate(w, q, K, V, S, nthreads, min_seconds)
    n1 = min(single_seqs, n)
    rate1, reps1, dt1 = _oracle_rate(w, q[:n1].contiguous(), K[:n1].contiguous(),
                                     V[:n1].contiguous(), S[:n1].contiguous(), 1, single_seconds)
    return {"value": rate, "unit": "queries/s/layer", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} of {w.batch} sequences x {w.hkv} KV heads of one layer (summary "
                      f"update + scores + top-k + attention, fp64), {reps} repetitions, "
                      f"{dt:.1f} s on {nthreads} threads",
            "host_cpus": host, "usable_cpus": usable,
            "single_thread": {"value": rate1, "unit": "queries/s/layer", "cores": 1,
                              "sample": f"{n1} sequences x {w.hkv} KV heads, {reps1} "
                                        f"repetitions, {dt1:.1f} s"}}


KERNEL_NAMES = {"one": "k_decode_step",
                "one-f32": "k_decode_step_f32 (one launch, splits per pair)",
                "one-split": "k_select_attend (one launch)",
                "two": "k_score_tiles + k_select_attend (two launches)",
                "two-f32": "k_block_score + k_select_attend (two launches)",
                "four": "scores or newest row, top-k, attention, combine (four launches)"}


def measure(w, args, layers, num_cu):
    """Time kin_sparse_decode_step on workload w over the rotated layers:
    the K timed steps bracketed by one event pair (ms_per_step), then a
    second pass with an event between steps for the per-step spread."""
    step = lambda i, b, e: sparse_step(w, i, b, None)  # noqa: E731
    ms, _ = time_steps(step, layers, args.steps, args.warmup)
    dist = step_distribution(step, layers, args.steps)
    step_bytes = w.bytes_sparse_step()
    gbs = step_bytes / (ms * 1e-3) / 1e9
    form = step_kernels(w, num_cu)
    kern = KERNEL_NAMES["two-f32" if form == "two" and w.dtype == "f32" else form]
    traffic, traffic_src = stored_traffic(w) if form == "one" else (None, None)
    # the step is one launch of the dominant kernel when form == "one": its
    # average launch duration is the event time over the K back-to-back steps
    roofline = {"bound": "hbm", "kernel": kern, "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic, "bytes_per_launch": step_bytes, "avg_us": round(ms * 1000, 2),
                "avg_us_source": "HIP events on the launch stream around the K timed steps"}
    if traffic is not None:
        roofline["traffic_source"] = (f"{traffic_src}: rocprofv3 FETCH_SIZE + WRITE_SIZE of this "
                                      "kernel, copy-calibrated, sources hash-matched")
    return {"value": round(w.batch / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "per_step": dist, "step_bytes": step_bytes, "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "kernels": form, "roofline": roofline}


OTHER_WORKLOADS = [workloads.QWEN3_8B.name, workloads.QWEN3_32B.name, workloads.TINY.name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=workloads.QWEN3_14B.name)
    ap.add_argument("--others", default=",".join(OTHER_WORKLOADS),
                    help="comma-separated workloads also timed (same protocol) and reported "
                         "under 'other_workloads'; empty for none")
    ap.add_argument("--layers", type=int, default=0, help="layers rotated (0: auto)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--sweep", choices=["big", "all"], default=None,
                    help="time the budget/length grid instead (big: the points of at least "
                         "256 MiB per step), one JSON line per point")
    ap.add_argument("--sweep-batch", type=int, default=0, help="only grid points of this batch")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU (use --gpus 1): the step shards by sequence or KV "
              "head with no exchange between GPUs, and runs on several GPUs are not "
              "measured here.", file=sys.stderr)
        sys.exit(2)

    torch.cuda.set_device(0)
    if args.sweep:
        run_sweep(args)
        return
    w = workloads.by_name(args.workload)
    if w.block == 1:
        run_token(args, w)
        return
    if w.share_n:
        run_shared(args, w)
        return
    if w.quest:
        run_quest(args, w)
        return
    if w.page_size:
        run_paged(args, w)
        return
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_layers = layers_for(w, args.layers)
    log(f"workload {w.name}: {n_layers} layers rotated, step bytes "
        f"{w.bytes_sparse_step() / 2**20:.1f} MiB")
    layers = make_layers(w, n_layers, with_dense=not args.no_dense)

    # timed region: K steps of kin_sparse_decode_step back to back on one
    # stream, one HIP event pair around all of them (measure()); the
    # per-step spread comes from a second pass with an event between steps
    m = measure(w, args, layers, num_cu)
    res = {"metric": METRIC, "value": m["value"], "unit": "queries/s/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
           "config": dict(w.describe(), layers_rotated=n_layers,
                          step_outputs="out, idx, S row (fp64 scores not written)"),
           "per_step": m["per_step"], "step_bytes": m["step_bytes"], "hbm_gbs": m["hbm_gbs"],
           "hbm_frac": m["hbm_frac"], "kernels": m["kernels"], "roofline": m["roofline"]}
    gbs = m["hbm_gbs"]
    ms = m["ms_per_step"]

    # the same step also writing the fp64 scores (an inspection output)
    sms, _ = time_steps(lambda i, b, e: sparse_step(w, i, b, None, scores=True), layers,
                        max(5, args.steps // 4), 5)
    res["with_scores_ms_per_step"] = round(sms, 5)

    if not args.no_unfused:
        n = max(5, args.steps // 5)
        tms, tst = time_steps(lambda i, b, e: two_kernel_step(w, i, b, e), layers, n, 2,
                              n_events=3)
        res["two_kernel"] = {"ms_per_step": round(tms, 5),
                             "update_score_us": round(tst[0] * 1000, 2),
                             "select_attend_us": round(tst[1] * 1000, 2)}
        ums, _ = time_steps(lambda i, b, e: unfused_step(w, i, b, e), layers, n, 2)
        res["four_call_ms_per_step"] = round(ums, 5)

    dense_gbs = None
    if not args.no_dense:
        dms, _ = time_steps(lambda i, b, e: dense_step(w, i, b), layers,
                            max(5, args.steps // 5), 2)
        dbytes = w.bytes_dense()
        dense_gbs = dbytes / (dms * 1e-3) / 1e9
        res["dense"] = {"queries_per_s": round(w.batch / (dms * 1e-3), 1),
                        "ms_per_step": round(dms, 5), "hbm_gbs": round(dense_gbs, 1)}
        res["speedup_vs_dense"] = round(dms / ms, 2)

    if args.calib_copy:
        # a plain copy kernel of known size: reads 1 GiB and writes 1 GiB, so
        # its FETCH_SIZE / WRITE_SIZE counters calibrate the step kernel's
        src = torch.empty(2**30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = 2**30
        del src, dst

    # the oracle is timed last, after every GPU measurement: a GPU left idle
    # for its ~15 s would start the next measurements from a lower clock
    cpu_layer = layers[0]
    del layers
    torch.cuda.empty_cache()

    # the other configurations, same protocol, one entry each
    others = {}
    for name in [x for x in args.others.split(",") if x]:
        wo = workloads.by_name(name)
        if wo.name == w.name:
            continue
        nl = layers_for(wo, args.layers)
        lo = make_layers(wo, nl, with_dense=False)
        mo = measure(wo, args, lo, num_cu)
        mo["config"] = dict(wo.describe(), layers_rotated=nl)
        others[wo.name] = mo
        del lo
        torch.cuda.empty_cache()
    if others:
        res["other_workloads"] = others

    # the step against this device's measured streaming rate as well: the
    # read probe, or the in-house dense attention when that streamed faster
    if not args.no_probe:
        peak = read_peak()
        best, src = (peak, "k_read_probe")
        if dense_gbs is not None and dense_gbs > best:
            best, src = (dense_gbs, "dense attention (kin_dense_decode_attn)")
        res["read_peak"] = {"probe_gbs": round(peak, 1),
                            "dense_gbs": round(dense_gbs, 1) if dense_gbs else None,
                            "gbs": round(best, 1), "source": src,
                            "frac_of_published": round(best / PEAK_HBM_GBS, 4),
                            "step_frac": round(gbs / best, 4)}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, cpu_layer, args.cpu_seqs)
    del cpu_layer
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
