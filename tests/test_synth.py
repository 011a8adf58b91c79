"""The seeded input generator against its stated recipe (CPU): streams are
reproducible and independent of each other, q and V are standard normal,
the keys' block means carry one N(0, 0.5^2) offset direction per (sequence,
KV head) on top of the N(0, 1/B) noise of a block mean, heavy blocks are
shifted by +2 along the unit group-query direction, and cache rows past the
context hold the tail fill."""
import math

import torch

from block_top_sparse_amd import synth
from block_top_sparse_amd.workloads import Workload


def _w(**kw):
    base = dict(name="synth", batch=1, hq=8, hkv=2, ctx_len=16384, block=16, topk=8,
                dtype="f32", seed=77)
    base.update(kw)
    return Workload(**base)


def test_same_seed_same_bytes_and_other_seed_differs():
    w = _w(ctx_len=500, t_cap=512, dtype="bf16")
    a, b = synth.make_inputs(w), synth.make_inputs(w)
    for k in ("q", "K", "V"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
    c = synth.make_inputs(w, seed=78)
    assert not torch.equal(a["K"][:, :, :500], c["K"][:, :, :500])


def test_query_and_values_are_standard_normal():
    inp = synth.make_inputs(_w(hq=64, hkv=8, ctx_len=4096))
    for x in (inp["q"], inp["V"]):
        x = x.double().flatten()
        n = x.numel()
        assert abs(x.mean().item()) < 5 / math.sqrt(n)
        assert abs(x.std().item() - 1.0) < 0.01


def test_block_means_have_one_offset_direction_of_variance_one_quarter():
    w = _w()
    K = synth.make_inputs(w)["K"].double()  # [1][hkv][L][d]
    B = w.block
    for g in range(w.hkv):
        means = K[0, g].view(w.nb, B, w.head_dim).mean(dim=1)  # [nb][d]
        cov = torch.cov(means.T)
        ev = torch.linalg.eigvalsh(cov)  # ascending
        # top: 0.25 (the offset) + 1/B (noise of a mean of B unit normals);
        # the rest: the noise alone, spread by the finite sample
        assert abs(ev[-1].item() - (0.25 + 1 / B)) < 0.05, ev[-1]
        assert ev[-2].item() < 0.15, ev[-2]
        assert abs(ev[: w.head_dim // 2].mean().item() - 1 / B) < 0.03


def test_heavy_blocks_are_shifted_by_two_along_the_group_query():
    w = _w(heavy_blocks=4, ctx_len=8192)
    inp = synth.make_inputs(w)
    ids = synth.heavy_block_ids(w)
    q = inp["q"][0].double().view(w.hkv, w.gqa, w.head_dim).sum(dim=1)
    qhat = q / q.norm(dim=1, keepdim=True)
    K = inp["K"][0].double()
    for g in range(w.hkv):
        proj = K[g].view(w.nb, w.block, w.head_dim).mean(dim=1) @ qhat[g]  # [nb]
        heavy = torch.zeros(w.nb, dtype=torch.bool)
        heavy[ids[0][g]] = True
        assert heavy.sum() == 4
        shift = proj[heavy].mean() - proj[~heavy].mean()
        assert abs(shift.item() - 2.0) < 0.6, shift


def test_rows_past_the_context_hold_the_tail_fill():
    w = _w(ctx_len=1000, t_cap=1024, dtype="bf16")
    inp = synth.make_inputs(w)
    assert torch.isnan(inp["K"][:, :, 1000:].float()).all()
    assert torch.isnan(inp["V"][:, :, 1000:].float()).all()
    assert torch.isfinite(inp["K"][:, :, :1000].float()).all()
    inp0 = synth.make_inputs(w, tail_fill=0.0)
    assert (inp0["V"][:, :, 1000:] == 0).all()
    # the context's rows do not depend on the fill
    assert torch.equal(inp0["K"][:, :, :1000].view(torch.int16),
                       inp["K"][:, :, :1000].view(torch.int16))
