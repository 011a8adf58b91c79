"""Repeated calls on one workspace: the split forms count their workgroups'
arrivals in workspace words that are either cleared by the step's first
kernel or tagged with each call's round, so a word left by an earlier call
must never be mistaken for a current arrival.  Each form runs 100 times back
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
    ("rep-keepall", 2, 16, 4, 2000, 16, 125, "bf16", 2048, False),       # one launch, round tags
    ("rep-f32-split", 3, 2, 2, 4730, 16, 292, "f32", 4793, True),        # fp32: round tags
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


def test_token_step_repeated_on_one_workspace():
    w = Workload("rep-token", batch=2, hq=8, hkv=2, ctx_len=20000, block=1, topk=500,
                 dtype="bf16", seed=913, t_cap=20000)  # 4 pairs: the two-kernel form
    inp = synth.make_inputs(w, device="cuda")
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    idx = torch.empty((w.batch, w.hkv, 500), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kb.kin_token_ws_bytes(desc, 500), dtype=torch.uint8, device="cuda")
    _repeat(lambda: kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], None, 500, idx,
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
    ws = torch.empty(kb.kin_quest_ws_bytes(desc, 60), dtype=torch.uint8, device="cuda")
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
