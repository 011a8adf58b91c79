"""The decode steps captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library allocates nothing, never synchronises and records no
memset, so a captured step replays; the split forms count their
workgroups' arrivals in workspace words that each call (and each replay)
must leave at zero for the next one.
Each form is replayed four times back to back, with new query values
written eagerly before each replay, and every replay must equal an eager
call on the same inputs bit for bit."""
import zlib

import pytest
import torch

from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.buffers import LayerBuffers
from block_top_sparse_amd.workloads import Workload

from parity_util import bits, gpu_inputs, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _check_replays(call, q, outs, seed):
    """Replays back to back (new queries written eagerly before each, no
    eager step in between, so each replay finds the arrival words exactly
    as the previous replay left them), then the eager references."""
    call()  # eager warm-up (the library caches the device's CU count)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    qs = [torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype) for _ in range(REPLAYS)]
    got = []
    for r in range(REPLAYS):
        q.copy_(qs[r])  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append([t.clone() for t in outs()])
    for r in range(REPLAYS):
        q.copy_(qs[r])
        call()
        torch.cuda.synchronize()
        for a, b in zip(got[r], outs()):
            assert torch.equal(bits(a) if a.is_floating_point() else a,
                               bits(b) if b.is_floating_point() else b), f"replay {r}"
    say(f"  {REPLAYS} replays equal eager calls")


BLOCK = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap, scores
    ("graph-one-kernel", 64, 16, 4, 2000, 16, 20, "bf16", 2048, False),   # 256 pairs
    ("graph-two-kernel", 3, 16, 2, 5000, 16, 100, "bf16", 5120, True),
    ("graph-two-kernel-nosc", 1, 8, 2, 40000, 32, 64, "bf16", 40000, False),  # scores in ws
    ("graph-two-kernel-cand", 2, 16, 4, 100000, 16, 120, "bf16", 100096, False),  # tile candidates
    ("graph-keepall", 2, 16, 4, 2000, 16, 125, "bf16", 2048, False),       # one launch, splits
    ("graph-f32-split", 3, 2, 2, 4730, 16, 292, "f32", 4793, True),        # fp32 split step
    ("graph-f32-one", 1, 8, 2, 4096, 16, 32, "f32", 4096, False),          # fp32 one kernel
]


@pytest.mark.parametrize("case", BLOCK, ids=[c[0] for c in BLOCK])
def test_block_step_replayed_from_a_graph(case):
    name, b, hq, hkv, L, B, k, dt, cap, with_scores = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}")
    inp = gpu_inputs(w)
    bufs = LayerBuffers(w, k=k)
    kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, (w.nb - 1) * B)

    def call():
        kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S,
                                  bufs.scores if with_scores else None, k, bufs.idx, bufs.out,
                                  bufs.ws)

    _check_replays(call, inp["q"], lambda: (bufs.idx, bufs.out), w.seed)


@pytest.mark.parametrize("k", [500, 100], ids=["all-words", "tile-candidates"])
def test_token_step_replayed_from_a_graph(k):
    """4 pairs over 53 score tiles: with k = 500 the splits share a
    selection over every token's word, with k = 100 each tile first keeps
    its own 100 best."""
    w = Workload("graph-token", batch=2, hq=8, hkv=2, ctx_len=20000, block=1, topk=k,
                 dtype="bf16", seed=915, t_cap=20000)
    inp = synth.make_inputs(w, device="cuda")
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    idx = torch.empty((w.batch, w.hkv, k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(kb.kin_token_ws_bytes(desc, k), dtype=torch.uint8, device="cuda")
    _check_replays(lambda: kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], None,
                                                    k, idx, out, ws),
                   inp["q"], lambda: (idx, out), 915)


def test_quest_step_replayed_from_a_graph():
    w = Workload("graph-quest", batch=3, hq=16, hkv=2, ctx_len=4000, block=16, topk=60,
                 dtype="bf16", seed=916, t_cap=4096)
    inp = synth.make_inputs(w, device="cuda")
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 16, torch.bfloat16)
    Sq = torch.empty((w.batch, w.hkv, w.nb_cap, 2, 128), dtype=torch.bfloat16, device="cuda")
    kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, w.ctx_len)
    idx = torch.empty((w.batch, w.hkv, 60), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(kb.kin_quest_ws_bytes(desc, 60), dtype=torch.uint8, device="cuda")
    _check_replays(lambda: kb.kin_quest_decode_step(desc, inp["q"], inp["K"], inp["V"], Sq, None,
                                                    60, idx, out, ws),
                   inp["q"], lambda: (idx, out), 916)


def test_paged_keepall_step_replayed_from_a_graph():
    """Variable lengths in a paged pool, few pairs, every block kept and no
    scores: the one-launch form whose splits count in words left at zero."""
    from test_paged_gpu import Case

    c = Case("graph-paged-keepall", 3, 2, 4, 16, 64, 600, 40, "rand")
    pg = c.pages()
    kb.kin_paged_summary_update(c.desc, pg, c.Kp, c.S, 0, c.w.ctx_len)

    def call():
        kb.kin_paged_decode_step(c.desc, pg, c.q, c.Kp, c.Vp, c.S, None, c.k, c.idx, c.out, c.ws)

    _check_replays(call, c.q, lambda: (c.idx, c.out), 917)


def test_shared_prompt_step_replayed_from_a_graph():
    """Samples sharing a prompt, few pairs (two kernels)."""
    from test_shared_gpu import build

    c = build(("graph-shared", 2, 2, 2, 8, 64, 512, 3000, 10))
    w, k, P = c["w"], c["k"], c["P"]
    S = torch.empty((w.batch, w.hkv, w.nb_cap, 128), dtype=torch.bfloat16, device="cuda")
    kb.kin_block_summary_update(c["desc"], c["K"], S, P, w.ctx_len)
    idx = torch.empty((w.batch, w.hkv, k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(kb.kin_sparse_ws_bytes(c["desc"], k), 16), dtype=torch.uint8,
                     device="cuda")
    share = kb.make_share(c["n_share"], P, c["Kp"], c["Vp"], c["Sp"])

    def call():
        kb.kin_shared_decode_step(c["desc"], share, c["q"], c["K"], c["V"], S, None, k, idx, out,
                                  ws)

    _check_replays(call, c["q"], lambda: (idx, out), 918)
