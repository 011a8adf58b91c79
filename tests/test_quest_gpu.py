"""GPU parity of the Quest-style step against the oracle.

The oracle's Quest summaries (channel-wise minimum and maximum) and bound
are pinned on the CPU (test_oracle_pins.py); here the GPU's summaries must
match them bit for bit, its bounds within 1e-13 relative, its selection
exactly (after the margin certificate), and its outputs within the bf16
tolerance.  Each case prefills every block but the newest, spoils the
newest block's rows, and lets the step rebuild them.
"""
import zlib

import pytest
import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.workloads import Workload

from parity_util import GAP_MIN, TOL, bits, say

pytestmark = pytest.mark.gpu

NAN = float("nan")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


QUEST = [
    # name, batch, hq, hkv, ctx, block, k, t_cap
    ("q-few-g4-b16-ragged", 3, 16, 4, 5000, 16, 40, 5120),   # 12 pairs: split attention
    ("q-many-g8-b32", 32, 64, 8, 3000, 32, 16, 3072),        # 256 pairs
    ("q-g1-b64-k1", 2, 2, 2, 1000, 64, 1, 1024),
    ("q-g4-b16-kpast", 2, 8, 2, 200, 16, 20, 208),           # k > nb
    ("q-g8-b128-short", 2, 16, 2, 100, 128, 2, 128),         # one partial block
    ("q-g5-b16-nb8192", 1, 10, 2, 131072, 16, 300, 131072),
    # at least as many pairs as CUs: the whole step in one kernel
    ("q-single-4w-g4-b16", 128, 16, 4, 2000, 16, 20, 2048),   # 512 pairs: the 4-wave step
    ("q-single-g4-b64-keepall", 64, 16, 4, 1000, 64, 20, 1024),
    ("q-single-g2-b16-nb8192", 64, 8, 4, 131072, 16, 300, 131072),  # 256 pairs, 8192 blocks
]


def run(w, inp, k, scores=True):
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, w.block, torch.bfloat16)
    Sq = torch.full((w.batch, w.hkv, w.nb_cap, 2, 128), NAN, dtype=torch.bfloat16, device="cuda")
    newest0 = (w.nb - 1) * w.block
    if newest0 > 0:
        kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, newest0)
    Sq[:, :, w.nb - 1] = 5.0  # stale newest rows: the step rebuilds them
    sc = torch.full((w.batch, w.hkv, w.nb_cap), NAN, dtype=torch.float64,
                    device="cuda") if scores else None
    idx = torch.full((w.batch, w.hkv, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.hq, 128), NAN, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(kb.kin_quest_ws_bytes(desc, k), dtype=torch.uint8, device="cuda")
    kb.kin_quest_decode_step(desc, inp["q"], inp["K"], inp["V"], Sq, sc, k, idx, out, ws)
    torch.cuda.synchronize()
    return Sq, sc, idx, out


@pytest.mark.parametrize("case", QUEST, ids=[c[0] for c in QUEST])
def test_quest_step_against_oracle(case):
    name, b, hq, hkv, L, B, k, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype="bf16",
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}, nb {w.nb}, k {k}")
    inp = synth.make_inputs(w, device="cuda", tail_fill=NAN)
    Sq, sc, idx, out = run(w, inp, k)
    nb = w.nb
    worst = 0.0
    for s in sorted({0, b // 2, b - 1}):
        qb, Kb, Vb = inp["q"][s:s + 1].cpu(), inp["K"][s:s + 1].cpu(), inp["V"][s:s + 1].cpu()
        Sq_or = oracle.quest_summary(Kb, B, L)
        assert torch.equal(bits(Sq[s:s + 1, :, :nb].cpu()), bits(Sq_or[:, :, :nb])), \
            f"summaries differ, seq {s}"
        sc_or = oracle.quest_score(qb, Sq_or, w.gqa, nb)
        ref = sc_or[:, :, :nb]
        scale = ref.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
        assert ((sc[s:s + 1, :, :nb].cpu() - ref).abs() / scale).max() < 1e-13, f"bounds, seq {s}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), nb, k)
        assert (gap > GAP_MIN).all(), f"margin certificate fails, seq {s}"
        assert torch.equal(idx[s:s + 1].cpu(), idx_or), f"selection differs, seq {s}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, L, B, idx=idx_or)
        og = out[s:s + 1].cpu().double()
        assert torch.isfinite(og).all(), f"unwritten output, seq {s}"
        err = (og - o).abs().max().item()
        assert err <= TOL["bf16"], f"output error {err}, seq {s}"
        worst = max(worst, err)
    if k > nb:
        assert (idx[:, :, nb:] == -1).all()
    # every pair's selection, and the call without a scores buffer
    _, _, idx2, out2 = run(w, inp, k, scores=False)
    assert torch.equal(idx2, idx)
    assert torch.equal(bits(out2), bits(out))
    say(f"  ok, max err {worst:.3e}")


def test_quest_summary_update_whole_cache():
    w = Workload("q-sum", batch=3, hq=4, hkv=2, ctx_len=777, block=32, topk=4, dtype="bf16",
                 seed=313, t_cap=800)
    inp = synth.make_inputs(w, device="cuda", tail_fill=NAN)
    desc = kb.make_desc(3, 2, 2, 800, 777, 32, torch.bfloat16)
    Sq = torch.full((3, 2, w.nb_cap, 2, 128), NAN, dtype=torch.bfloat16, device="cuda")
    kb.kin_quest_summary_update(desc, inp["K"], Sq, 100, 500)  # blocks 3 .. 15
    kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, 100)
    kb.kin_quest_summary_update(desc, inp["K"], Sq, 500, 800)
    torch.cuda.synchronize()
    ref = oracle.quest_summary(inp["K"].cpu(), 32, 777)
    assert torch.equal(bits(Sq[:, :, :w.nb].cpu()), bits(ref[:, :, :w.nb]))
    assert torch.isnan(Sq[:, :, w.nb:].float()).all()
