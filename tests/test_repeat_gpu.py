"""Repeated calls on one workspace: the split forms count their workgroups'
arrivals in workspace words that are either cleared by the step's first
kernel or were left at zero by the previous call on the workspace, so a word
left by an earlier call must never be mistaken for a current arrival.  Each form runs 100 times back
to back on the same workspace (no synchronisation between the calls) and
every call's idx and output must equal the first call's bit for bit."""
import zlib

import pytest
import torch

from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.buffers import LayerBuffers
from block_top_sparse_amd.workloads import Workload

from parity_util import bits, gpu_inputs, say

pytestmark = pytest.mark.gpu

REPEATS = 100


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _repeat(call, outs):
    """call() enqueues one step; outs() returns the tensors to compare."""
    call()
    torch.cuda.synchronize()
    first = [t.clone() for t in outs()]
    got = []
    for _ in range(REPEATS - 1):
        call()
        got.append([t.clone() for t in outs()])  # device copies, enqueued in order
    torch.cuda.synchronize()
    for i, g in enumerate(got):
        for a, b in zip(first, g):
            assert torch.equal(bits(a) if a.is_floating_point() else a,
                               bits(b) if b.is_floating_point() else b), f"call {i + 2}"


BLOCK = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap, scores
    ("rep-two-kernel", 3, 16, 2, 5000, 16, 100, "bf16", 5120, True),     # kernel 1 clears words
    ("rep-two-kernel-nosc", 3, 16, 2, 5000, 16, 100, "bf16", 5120, False),
    ("rep-two-kernel-one-split", 2, 64, 8, 3000, 64, 1, "bf16", 3072, False),  # one split per pair
    ("rep-two-kernel-cand", 2, 16, 4, 100000, 16, 120, "bf16", 100096, False),  # tile candidates
    ("rep-keepall", 2, 16, 4, 2000, 16, 125, "bf16", 2048, False),       # one launch
    ("rep-f32-split", 3, 2, 2, 4730, 16, 292, "f32", 4793, True),        # fp32 kernel 1 clears
    ("rep-f32-one", 1, 8, 2, 4096, 16, 32, "f32", 4096, False),          # fp32 one kernel, splits
]


@pytest.mark.parametrize("case", BLOCK, ids=[c[0] for c in BLOCK])
def test_block_step_repeated_on_one_workspace(case):
    name, b, hq, hkv, L, B, k, dt, cap, with_scores = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    inp = gpu_inputs(w)
    bufs = LayerBuffers(w, k=k)
    assert bufs.ws is not None, "a split form needs a workspace"
    kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, (w.nb - 1) * B)
    say(f"case {name}: {REPEATS} calls")

    def call():
        kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S,
                                  bufs.scores if with_scores else None, k, bufs.idx, bufs.out,
                                  bufs.ws)

    _repeat(call, lambda: (bufs.idx, bufs.out))


@pytest.mark.parametrize("k", [500, 100], ids=["all-words", "tile-candidates"])
def test_token_step_repeated_on_one_workspace(k):
    # 4 pairs: the two-kernel form; k = 100: the score tiles pick candidates
    w = Workload("rep-token", batch=2, hq=8, hkv=2, ctx_len=20000, block=1, topk=k,
                 dtype="bf16", seed=913, t_cap=20000)
    inp = synth.make_inputs(w, device="cuda")
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    idx = torch.empty((w.batch, w.hkv, k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(kb.kin_token_ws_bytes(desc, k), dtype=torch.uint8, device="cuda")
    _repeat(lambda: kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], None, k, idx,
                                             out, ws),
            lambda: (idx, out))


def test_quest_step_repeated_on_one_workspace():
    w = Workload("rep-quest", batch=3, hq=16, hkv=2, ctx_len=4000, block=16, topk=60,
                 dtype="bf16", seed=914, t_cap=4096)  # 6 pairs: the two-kernel form
    inp = synth.make_inputs(w, device="cuda")
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 16, torch.bfloat16)
    Sq = torch.empty((w.batch, w.hkv, w.nb_cap, 2, 128), dtype=torch.bfloat16, device="cuda")
    kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, w.ctx_len)
    idx = torch.empty((w.batch, w.hkv, 60), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(kb.kin_quest_ws_bytes(desc, 60), dtype=torch.uint8, device="cuda")
    _repeat(lambda: kb.kin_quest_decode_step(desc, inp["q"], inp["K"], inp["V"], Sq, None, 60,
                                             idx, out, ws),
            lambda: (idx, out))


def test_two_streams_at_once_match_one_after_the_other():
    """Two different few-pair problems (a bf16 two-kernel step and a keep-all
    one-launch step), each with its own workspace, stepped 20 times on two
    streams at once: the results equal those of the same calls made one
    after the other on the default stream (the library keeps no state
    between calls besides the caller's buffers)."""
    cases = [("conc-a", 3, 16, 2, 5000, 16, 100, 5120), ("conc-b", 2, 16, 4, 2000, 16, 125, 2048)]
    jobs = []
    for name, b, hq, hkv, L, B, k, cap in cases:
        w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype="bf16",
                     seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
        inp = gpu_inputs(w)
        bufs = LayerBuffers(w, k=k)
        kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, (w.nb - 1) * B)
        jobs.append((w, inp, bufs, k))

    def step(job, stream=None):
        w, inp, bufs, k = job
        kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S, None, k,
                                  bufs.idx, bufs.out, bufs.ws, stream=stream)

    for job in jobs:
        step(job)
    torch.cuda.synchronize()
    want = [(j[2].idx.clone(), j[2].out.clone()) for j in jobs]
    for j in jobs:
        j[2].idx.fill_(-7)
        j[2].out.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(20):
        for job, st in zip(jobs, streams):
            step(job, stream=st)
    torch.cuda.synchronize()
    for (idx, out), job in zip(want, jobs):
        assert torch.equal(job[2].idx, idx)
        assert torch.equal(bits(job[2].out), bits(out))


def test_one_workspace_zeroed_once_serves_every_split_form():
    """One workspace, zeroed once, used in turn by split forms of different
    shapes and entry points: the keep-all one-launch step, the bf16 two-kernel
    step (its first kernel clears the second's words), the standalone
    second half (kin_decode_select_attend), the fp32 two-kernel step, the
    standalone split attention, the token-level two-kernel step (over every
    token's word, and with the score tiles' candidates) and the Quest
    two-kernel step.
    After every call the first 8 KiB (the arrival words) are zero again, and
    every result equals the same call's on a fresh zeroed workspace."""
    calls = []

    def block_case(name, b, hq, hkv, L, B, k, dt, cap, kind):
        w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                     seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
        inp = gpu_inputs(w)
        bufs = LayerBuffers(w, k=k)
        kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, w.ctx_len)
        d = bufs.desc
        if kind == "step":
            def call(ws):
                kb.kin_sparse_decode_step(d, inp["q"], inp["K"], inp["V"], bufs.S, None, k,
                                          bufs.idx, bufs.out, ws)
        elif kind == "half":
            kb.kin_block_score(d, inp["q"], bufs.S, bufs.scores)

            def call(ws):
                kb.kin_decode_select_attend(d, inp["q"], inp["K"], inp["V"], bufs.scores, k,
                                            bufs.idx, bufs.out, ws)
        else:  # the standalone split attention over a fixed index list
            kb.kin_block_score(d, inp["q"], bufs.S, bufs.scores)
            kb.kin_block_topk(d, bufs.scores, k, bufs.idx)

            def call(ws):
                kb.kin_sparse_decode_attn(d, inp["q"], inp["K"], inp["V"], bufs.idx, k, bufs.out,
                                          ws)
        need = kb.kin_sparse_ws_bytes(d, k)
        # the standalone attention reads idx (an input there): compare out only
        outs = (lambda: (bufs.out,)) if kind == "attn" else (lambda: (bufs.idx, bufs.out))
        calls.append((name, call, need, outs))

    block_case("ws-keepall", 2, 16, 4, 2000, 16, 125, "bf16", 2048, "step")
    block_case("ws-two-kernel", 1, 8, 2, 40000, 32, 64, "bf16", 40000, "step")
    block_case("ws-half", 3, 16, 2, 5000, 16, 100, "bf16", 5120, "half")
    block_case("ws-f32", 3, 2, 2, 4730, 16, 292, "f32", 4793, "step")
    block_case("ws-attn", 2, 8, 2, 6000, 32, 150, "bf16", 6016, "attn")
    block_case("ws-f32-one", 1, 8, 2, 4096, 16, 32, "f32", 4096, "step")

    wt = Workload("ws-token", batch=2, hq=8, hkv=2, ctx_len=20000, block=1, topk=500,
                  dtype="bf16", seed=915, t_cap=20000)
    it = synth.make_inputs(wt, device="cuda")
    dt_ = kb.make_desc(wt.batch, wt.hkv, wt.gqa, wt.cap, wt.ctx_len, 1, torch.bfloat16)
    for tk, tname in ((500, "ws-token"), (100, "ws-token-tiles")):
        tidx = torch.empty((wt.batch, wt.hkv, tk), dtype=torch.int32, device="cuda")
        tout = torch.empty((wt.batch, wt.hq, 128), dtype=torch.bfloat16, device="cuda")
        calls.append((tname,
                      lambda ws, tk=tk, tidx=tidx, tout=tout: kb.kin_token_decode_step(
                          dt_, it["q"], it["K"], it["V"], None, tk, tidx, tout, ws),
                      kb.kin_token_ws_bytes(dt_, tk), lambda tidx=tidx, tout=tout: (tidx, tout)))

    wq = Workload("ws-quest", batch=3, hq=16, hkv=2, ctx_len=4000, block=16, topk=60,
                  dtype="bf16", seed=916, t_cap=4096)
    iq = synth.make_inputs(wq, device="cuda")
    dq = kb.make_desc(wq.batch, wq.hkv, wq.gqa, wq.cap, wq.ctx_len, 16, torch.bfloat16)
    Sq = torch.empty((wq.batch, wq.hkv, wq.nb_cap, 2, 128), dtype=torch.bfloat16, device="cuda")
    kb.kin_quest_summary_update(dq, iq["K"], Sq, 0, wq.ctx_len)
    qidx = torch.empty((wq.batch, wq.hkv, 60), dtype=torch.int32, device="cuda")
    qout = torch.empty((wq.batch, wq.hq, 128), dtype=torch.bfloat16, device="cuda")
    calls.append(("ws-quest",
                  lambda ws: kb.kin_quest_decode_step(dq, iq["q"], iq["K"], iq["V"], Sq, None, 60,
                                                      qidx, qout, ws),
                  kb.kin_quest_ws_bytes(dq, 60), lambda: (qidx, qout)))

    for name, _, need, _ in calls:
        assert need >= 8192, f"{name}: a split form's workspace holds the arrival words"
    torch.cuda.synchronize()
    # references, each on a workspace of its own
    want = {}
    for name, call, need, outs in calls:
        call(torch.zeros(need, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        want[name] = [t.clone() for t in outs()]
    shared = torch.zeros(max(c[2] for c in calls), dtype=torch.uint8, device="cuda")
    for rnd in range(3):
        for name, call, need, outs in calls:
            say(f"round {rnd}: {name}")
            for t in outs():
                t.fill_(-7 if not t.is_floating_point() else float("nan"))
            call(shared)
            torch.cuda.synchronize()
            assert int(shared[:8192].count_nonzero()) == 0, f"{name} left arrival words set"
            for a, b in zip(want[name], outs()):
                assert torch.equal(bits(a) if a.is_floating_point() else a,
                                   bits(b) if b.is_floating_point() else b), name
