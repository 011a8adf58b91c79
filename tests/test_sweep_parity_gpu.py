"""GPU parity on EVERY point of the budget/length grid (the Qwen3-32B head
layout: 64 query / 8 KV heads, head_dim 128, bf16): batch 8, 32, 128 x
context 8K, 32K, 128K x block 16, 32, 64 x token budget 256, 1024, 4096,
8192 (k = budget / block, the pages' budget = block size x kept blocks),
plus the keep-every-block point of each (batch, context, block): 135 points.

Each test covers one (batch, context, block) group: one seeded cache (the
seed of the group's budget-256 point) and its five points.  Every point runs
the benchmarked call, kin_sparse_decode_step with no scores buffer, on that
cache.  Then the CPU oracle, fed the same bytes a few sequences at a time,
gives the summaries (compared bit for bit with the S the steps left), the
scores and, per point, the selection of EVERY (sequence, KV head) pair
(compared bit for bit after the margin certificate), and the outputs of two
sequences (the first and the last) per point, within the bf16 tolerance.
"""
import pytest
import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth, workloads

from parity_util import GAP_MIN, TOL, bits, say

pytestmark = pytest.mark.gpu

GROUPS = [(b, L, B) for b in workloads.SWEEP_BATCH for L in workloads.SWEEP_CTX
          for B in workloads.SWEEP_BLOCK]
CHUNK_BYTES = 2 << 30  # K bytes copied to the host per oracle call


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _group_points(b, L, B):
    pts = [w for w in workloads.sweep() if (w.batch, w.ctx_len, w.block) == (b, L, B)]
    assert len(pts) == len(workloads.SWEEP_BUDGET) + 1
    return pts


@pytest.mark.parametrize("b,L,B", GROUPS, ids=[f"b{b}-ctx{L}-blk{B}" for b, L, B in GROUPS])
def test_sweep_group_every_point(b, L, B):
    pts = _group_points(b, L, B)
    base = pts[0]
    say(f"group b{b} ctx{L} blk{B}: cache {base.cache_bytes() / 2**30:.1f} GiB, "
        f"points {[w.topk for w in pts]}")
    inp = synth.make_inputs(base, device="cuda")
    dt = torch.bfloat16
    nb, hkv, gqa = base.nb, base.hkv, base.gqa
    S = torch.empty((b, hkv, base.nb_cap, 128), dtype=dt, device="cuda")
    S[:, :, nb - 1] = 7.0  # stale newest row: every step rebuilds it
    desc = kb.make_desc(b, hkv, gqa, L, L, B, dt)
    if nb > 1:
        kb.kin_block_summary_update(desc, inp["K"], S, 0, (nb - 1) * B)
    sample = sorted({0, b - 1})
    gpu_idx, gpu_out = {}, {}
    for w in pts:
        k = w.topk
        idx = torch.full((b, hkv, k), -9, dtype=torch.int32, device="cuda")
        out = torch.full((b, w.hq, 128), float("nan"), dtype=dt, device="cuda")
        n = kb.kin_sparse_ws_bytes(desc, k)
        ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda") if n else None
        kb.kin_sparse_decode_step(desc, inp["q"], inp["K"], inp["V"], S, None, k, idx, out, ws)
        torch.cuda.synchronize()
        gpu_idx[w.name] = idx.cpu()
        gpu_out[w.name] = out[sample].cpu()
        del idx, out, ws
    say("  gpu steps done; oracle over every pair")

    q_all = inp["q"].cpu()
    per_seq = hkv * L * 128 * 2
    step = max(1, CHUNK_BYTES // per_seq)
    min_gap = float("inf")
    worst = 0.0
    for s0 in range(0, b, step):
        s1 = min(b, s0 + step)
        Kc = inp["K"][s0:s1].cpu()
        qc = q_all[s0:s1].contiguous()
        S_or, _ = oracle.block_summary(Kc, B, L)
        assert torch.equal(bits(S[s0:s1, :, :nb].cpu()), bits(S_or[:, :, :nb])), \
            f"summaries differ in sequences {s0}..{s1 - 1}"
        sc = oracle.block_score(qc, S_or, gqa, nb)
        here = {sq: inp["V"][sq:sq + 1].cpu() for sq in sample if s0 <= sq < s1}
        for w in pts:
            idx_or, gap = oracle.block_topk(sc, nb, w.topk)
            if w.topk < nb:
                g = gap.min().item()
                min_gap = min(min_gap, g)
                assert (gap > GAP_MIN).all(), f"{w.name}: margin certificate fails ({g})"
            assert torch.equal(gpu_idx[w.name][s0:s1], idx_or), \
                f"{w.name}: selection differs in sequences {s0}..{s1 - 1}"
            for i, sq in enumerate(sample):
                if not s0 <= sq < s1:
                    continue
                r = sq - s0
                o = oracle.decode_attention(qc[r:r + 1].contiguous(), Kc[r:r + 1].contiguous(),
                                            here[sq], gqa, L, B, idx=idx_or[r:r + 1].contiguous())
                og = gpu_out[w.name][i:i + 1].double()
                assert torch.isfinite(og).all(), f"{w.name}: unwritten output, seq {sq}"
                err = (og - o).abs().max().item()
                worst = max(worst, err)
                assert err <= TOL["bf16"], f"{w.name}: output error {err} at seq {sq}"
        say(f"  sequences {s0}..{s1 - 1}: summaries, selections of {len(pts)} points ok")
        del Kc, S_or, sc, here
    say(f"  ok: {len(pts)} points, every pair's selection exact, min gap {min_gap:.3g}, "
        f"max output error {worst:.3g} on sequences {sample}")
    del inp, S
    torch.cuda.empty_cache()
