"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle step to a closed form, a library routine, brute
force or an invariant, so that a plausible slip (a dropped 1/sqrt(d), a
wrong GQA mapping, max instead of sum over the group, a reversed tie-break,
an off-by-one partial block, a wrong rounding) fails at least one of them.

Steps (sources): the skill summary page "Kinetics: Memory-Aware Test-Time
Scaling", Implementation / BlockTopKAttention (scores q.k/sqrt(d), mean
score per block, torch.topk, mask then softmax . V); the rebuttal page
"Kinetics: Rethinking Test-Time Scaling Law", Q4 "KV block size and grouping
strategy" (KV blocks, budget = block size x top-k blocks).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from block_top_sparse_amd import synth
from block_top_sparse_amd.workloads import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "constructed_examples.json")


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32)


def _torch_two_step(x64, dtype):
    # library casts: fp64 -> fp32 (RNE) and, for bf16, fp32 -> bf16 (RNE)
    x = x64.to(torch.float32)
    return x if dtype == torch.float32 else x.to(torch.bfloat16)


# ---------------------------------------------------------------- rounding

def test_round_matches_torch_casts_including_halfway_cases():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(20000, generator=g, dtype=torch.float64) * 10.0 ** torch.randint(
        -6, 7, (20000,), generator=g).double()
    # exact halfway cases for bf16: fp32 values whose low 16 bits are 0x8000,
    # with even and odd kept parts, positive and negative
    hi = torch.randint(0, 0x1800, (4000,), generator=g, dtype=torch.int64) + 0x3000
    u = ((hi << 16) | 0x8000).to(torch.int64)
    halves = torch.from_numpy(u.numpy().astype(np.uint32).view(np.float32).astype(np.float64))
    x = torch.cat([x, halves, -halves, torch.tensor([0.0, -0.0, 1e-30, 3.0e38])])
    for dt in (torch.float32, torch.bfloat16):
        got = oracle.round_to(x, dt)
        ref = _torch_two_step(x, dt)
        assert torch.equal(_bits(got), _bits(ref)), dt


# ---------------------------------------------------------------- O1 summaries

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("block,ctx_len", [(16, 256), (16, 250), (32, 97), (64, 64), (4, 3)])
def test_summary_is_rounded_block_mean(dtype, block, ctx_len):
    g = torch.Generator().manual_seed(block * 1000 + ctx_len)
    cap = ctx_len + 13
    # values exact in bf16 so the fp64 sum is exact in any order
    K = torch.randn((2, 3, cap, 8), generator=g).to(torch.bfloat16).to(dtype)
    S, S64 = oracle.block_summary(K, block, ctx_len, want_f64=True)
    nb = oracle.nblocks(ctx_len, block)
    for j in range(nb):
        t0, t1 = j * block, min((j + 1) * block, ctx_len)
        mean = K[:, :, t0:t1].double().mean(dim=2)
        assert torch.equal(S64[:, :, j], mean)
        assert torch.equal(_bits(S[:, :, j]), _bits(_torch_two_step(mean, dtype)))
    # rows past the context are never summarised
    assert torch.count_nonzero(S[:, :, nb:].float()) == 0


def test_summary_fp32_random_values_close_to_library_mean():
    g = torch.Generator().manual_seed(3)
    K = torch.randn((1, 2, 200, 16), generator=g)
    S, S64 = oracle.block_summary(K, 16, 200, want_f64=True)
    for j in range(oracle.nblocks(200, 16)):
        mean = K[:, :, j * 16:min(200, (j + 1) * 16)].double().mean(dim=2)
        assert torch.allclose(S64[:, :, j], mean, rtol=1e-15, atol=1e-16)


def test_summary_range_update_touches_only_intersecting_blocks():
    g = torch.Generator().manual_seed(5)
    K = torch.randn((2, 2, 128, 8), generator=g).to(torch.bfloat16)
    sentinel = torch.full((2, 2, 8, 8), 7.0, dtype=torch.bfloat16)
    # decode step: newest token 99 is in block 6 (block size 16)
    S, _ = oracle.block_summary(K, 16, 100, t_begin=99, t_end=100, S=sentinel.clone())
    full, _ = oracle.block_summary(K, 16, 100)
    for j in range(8):
        if j == 6:
            assert torch.equal(_bits(S[:, :, j]), _bits(full[:, :, j]))
        else:
            assert torch.equal(_bits(S[:, :, j]), _bits(sentinel[:, :, j]))
    # building piecewise equals building at once (idempotent, no drift)
    S2 = sentinel.clone()
    for t in range(0, 100, 7):
        S2, _ = oracle.block_summary(K, 16, 100, t_begin=t, t_end=min(100, t + 7), S=S2)
    assert torch.equal(_bits(S2[:, :, :7]), _bits(full[:, :, :7]))


def test_summary_invariant_to_token_order_within_block():
    g = torch.Generator().manual_seed(11)
    K = torch.randn((1, 1, 64, 16), generator=g).to(torch.bfloat16)
    Kp = K.clone()
    for j in range(4):
        perm = torch.randperm(16, generator=g) + 16 * j
        Kp[0, 0, 16 * j:16 * (j + 1)] = K[0, 0, perm]
    a, _ = oracle.block_summary(K, 16, 64)
    b, _ = oracle.block_summary(Kp, 16, 64)
    assert torch.equal(_bits(a), _bits(b))


# ---------------------------------------------------------------- O2 scores

def test_scores_equal_exact_rational_mean_of_token_scores():
    # small integers, power-of-two block: every mean is exact, so the score
    # must equal the exact rational  sum_h mean_t (q_h . k_t)
    inp = synth.small_int_inputs(2, 6, 2, 8, 32, 4, seed=1)
    q, K = inp["q"], inp["K"]
    gqa, B, L = 3, 4, 32
    S, _ = oracle.block_summary(K, B, L)
    sc = oracle.block_score(q, S, gqa, L // B)
    qi, Ki = q.long(), K.long()
    for b in range(2):
        for gk in range(2):
            for j in range(L // B):
                num = 0
                for h in range(gk * gqa, (gk + 1) * gqa):
                    for t in range(j * B, (j + 1) * B):
                        num += int((qi[b, h] * Ki[b, gk, t]).sum())
                assert sc[b, gk, j].item() == num / B


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_scores_match_numpy_einsum_on_random_inputs(dtype):
    w = Workload("t", batch=2, hq=8, hkv=2, ctx_len=300, block=16, topk=4, dtype=
                 "bf16" if dtype == torch.bfloat16 else "f32", seed=21, head_dim=32)
    inp = synth.make_inputs(w)
    S, _ = oracle.block_summary(inp["K"], 16, 300)
    sc = oracle.block_score(inp["q"], S, w.gqa, w.nb)
    qn = inp["q"].double().numpy().reshape(2, 2, 4, 32)
    Sn = S.double().numpy()[:, :, : w.nb]
    ref = np.einsum("bghc,bgjc->bgj", qn, Sn)
    np.testing.assert_allclose(sc.numpy()[:, :, : w.nb], ref, rtol=1e-12, atol=1e-12)


def test_negative_zero_score_is_canonical():
    q = torch.tensor([[[1.0, 0.0]]])
    S = torch.tensor([[[[-0.0, 5.0], [0.0, 5.0]]]])
    sc = oracle.block_score(q, S, 1, 2)
    assert not math.copysign(1.0, sc[0, 0, 0].item()) < 0
    idx, _ = oracle.block_topk(sc, 2, 1)
    assert idx.tolist() == [[[0]]]


# ---------------------------------------------------------------- O3 selection

def _brute_force_topk(s, k):
    best = None
    for sub in itertools.combinations(range(len(s)), k):
        tot = sum(s[j] for j in sub)
        if best is None or tot > best[0] or (tot == best[0] and sub < best[1]):
            best = (tot, sub)
    return list(best[1])


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_brute_force_subset_search(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 13))
    # few distinct values, so ties are common
    s = rng.integers(-3, 4, size=nb).astype(np.float64)
    scores = torch.zeros((1, 1, 16), dtype=torch.float64)
    scores[0, 0, :nb] = torch.from_numpy(s)
    for k in range(1, nb + 1):
        idx, _ = oracle.block_topk(scores, nb, k)
        assert idx[0, 0].tolist() == _brute_force_topk(list(s), k)


@pytest.mark.parametrize("seed", range(4))
def test_topk_equals_numpy_lexsort(seed):
    rng = np.random.default_rng(100 + seed)
    nb, k = 2048, 64
    s = np.round(rng.normal(size=(3, 2, nb)) * 8) / 8  # many exact ties
    idx, gap = oracle.block_topk(torch.from_numpy(s), nb, k)
    for b in range(3):
        for g in range(2):
            j = np.arange(nb)
            order = np.lexsort((j, -s[b, g]))[:k]
            assert idx[b, g].tolist() == sorted(order.tolist())
            srt = np.sort(s[b, g])[::-1]
            assert gap[b, g].item() == pytest.approx((srt[k - 1] - srt[k]) / np.abs(s[b, g]).max())


def test_topk_pads_when_k_exceeds_blocks_and_gap_is_infinite():
    s = torch.tensor([[[3.0, 1.0, 2.0, 0.0]]], dtype=torch.float64)
    idx, gap = oracle.block_topk(s, 3, 5)  # only 3 valid blocks
    assert idx.tolist() == [[[0, 1, 2, -1, -1]]]
    assert math.isinf(gap.item())


def test_topk_all_equal_scores_keep_lowest_indices():
    s = torch.full((1, 1, 10), 2.5, dtype=torch.float64)
    idx, gap = oracle.block_topk(s, 10, 4)
    assert idx.tolist() == [[[0, 1, 2, 3]]]
    assert gap.item() == 0.0


def test_duplicated_block_tie_goes_to_lower_index():
    g = torch.Generator().manual_seed(9)
    K = torch.randn((1, 1, 64, 8), generator=g).to(torch.bfloat16)
    K[0, 0, 48:64] = K[0, 0, 16:32]          # block 3 duplicates block 1
    q = torch.zeros((1, 1, 8), dtype=torch.bfloat16)
    S, _ = oracle.block_summary(K, 16, 64)
    q[0, 0] = S[0, 0, 1] * 4                 # make block 1 (and 3) the best
    sc = oracle.block_score(q, S, 1, 4)
    assert sc[0, 0, 1] == sc[0, 0, 3]
    idx, _ = oracle.block_topk(sc, 4, 1)
    assert idx.tolist() == [[[1]]]


def test_heavy_blocks_are_always_selected():
    w = Workload("heavy", batch=3, hq=40, hkv=8, ctx_len=2048, block=32, topk=8, dtype="bf16",
                 seed=1003, heavy_blocks=4)
    inp = synth.make_inputs(w)
    res = oracle.sparse_decode(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len, w.block, w.topk)
    heavy = synth.heavy_block_ids(w)
    for b in range(w.batch):
        for g in range(w.hkv):
            assert set(heavy[b][g]) <= set(res["idx"][b, g].tolist())
    assert (res["gap"] > 1e-12).all()


# ---------------------------------------------------------------- O4 attention

def _sdpa(q, K, V, gqa, ctx_len, mask=None):
    """Library reference: scaled_dot_product_attention in fp64 on CPU."""
    b, hq, d = q.shape
    Kr = K[:, :, :ctx_len].double().repeat_interleave(gqa, dim=1).contiguous()
    Vr = V[:, :, :ctx_len].double().repeat_interleave(gqa, dim=1).contiguous()
    qq = q.double()[:, :, None, :]
    if mask is not None:
        mask = mask.repeat_interleave(gqa, dim=1)[:, :, None, :ctx_len]
    return F.scaled_dot_product_attention(qq, Kr, Vr, attn_mask=mask)[:, :, 0, :]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dense_and_keep_all_equal_sdpa(dtype):
    w = Workload("t", batch=2, hq=10, hkv=2, ctx_len=203, block=16, topk=13,
                 dtype="bf16" if dtype == torch.bfloat16 else "f32", seed=31, t_cap=240)
    inp = synth.make_inputs(w)
    ref = _sdpa(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len)
    dense = oracle.decode_attention(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len, w.block)
    res = oracle.sparse_decode(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len, w.block, w.topk)
    assert res["idx"][0, 0].tolist() == list(range(13))
    assert torch.allclose(dense, ref, rtol=0, atol=1e-13)
    assert torch.allclose(res["out"], ref, rtol=0, atol=1e-13)
    assert torch.isfinite(dense).all()  # NaN tail past ctx_len is never read


@pytest.mark.parametrize("block", [1, 16, 32])
def test_sparse_equals_masked_sdpa(block):
    w = Workload("t", batch=2, hq=8, hkv=2, ctx_len=250, block=block, topk=5, dtype="bf16",
                 seed=40 + block, t_cap=256)
    inp = synth.make_inputs(w)
    res = oracle.sparse_decode(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len, block, w.topk)
    mask = torch.zeros((2, 2, w.cap), dtype=torch.bool)
    for b in range(2):
        for g in range(2):
            for j in res["idx"][b, g].tolist():
                if j >= 0:
                    mask[b, g, j * block:(j + 1) * block] = True
    ref = _sdpa(inp["q"], inp["K"], inp["V"], w.gqa, w.ctx_len, mask=mask)
    assert torch.allclose(res["out"], ref, rtol=0, atol=1e-13)


def test_random_index_list_equals_masked_sdpa():
    # the attention step on its own, with a hand-made (not top-k) selection
    w = Workload("t", batch=1, hq=4, hkv=1, ctx_len=100, block=16, topk=3, dtype="f32", seed=77)
    inp = synth.make_inputs(w)
    idx = torch.tensor([[[2, 6, -1]]], dtype=torch.int32)  # block 6 is partial (96..99)
    out = oracle.decode_attention(inp["q"], inp["K"], inp["V"], 4, 100, 16, idx=idx)
    mask = torch.zeros((1, 1, 100), dtype=torch.bool)
    mask[0, 0, 32:48] = True
    mask[0, 0, 96:100] = True
    ref = _sdpa(inp["q"], inp["K"], inp["V"], 4, 100, mask=mask)
    assert torch.allclose(out, ref, rtol=0, atol=1e-13)


def test_constant_values_and_single_token():
    g = torch.Generator().manual_seed(2)
    q = torch.randn((1, 4, 16), generator=g)
    K = torch.randn((1, 2, 64, 16), generator=g)
    V = torch.empty((1, 2, 64, 16))
    V[0, 0] = torch.arange(16.0)        # every token of KV head 0 holds 0..15
    V[0, 1] = -torch.arange(16.0) / 4   # KV head 1: -(0..15)/4
    out = oracle.decode_attention(q, K, V, 2, 64, 16, idx=torch.tensor([[[0, 3], [2, -1]]],
                                                                      dtype=torch.int32))
    # constant V over the kept tokens: the output is that row (to rounding)
    assert torch.allclose(out[0, :2], V[0, 0, :2].double().expand(2, 16), rtol=1e-15, atol=0)
    assert torch.allclose(out[0, 2:], V[0, 1, :2].double().expand(2, 16), rtol=1e-15, atol=0)
    one = oracle.decode_attention(q, K, V, 2, 1, 16)
    assert torch.equal(one[0, 0], V[0, 0, 0].double())
    assert torch.equal(one[0, 3], V[0, 1, 0].double())


def test_block_of_one_is_token_level_topk():
    # block = 1: the kept set is the k tokens with the largest group score
    w = Workload("t", batch=1, hq=6, hkv=2, ctx_len=90, block=1, topk=7, dtype="bf16", seed=55)
    inp = synth.make_inputs(w)
    res = oracle.sparse_decode(inp["q"], inp["K"], inp["V"], w.gqa, 90, 1, 7)
    qsum = inp["q"].double().view(1, 2, 3, 128).sum(dim=2)
    tok = torch.einsum("bgc,bgtc->bgt", qsum, inp["K"].double())
    for g in range(2):
        top = torch.topk(tok[0, g], 7).indices.sort().values.tolist()
        assert res["idx"][0, g].tolist() == top


# ---------------------------------------------------------------- constructed examples

def _closed_forms():
    r2 = math.sqrt(2.0)
    return {"1": 1.0, "b": math.exp(r2), "c": math.exp(3 / r2), "e": math.exp(1 / r2),
            "f": math.exp(-1 / r2), "g": math.exp(-3 / r2), "h": math.exp(3 * r2),
            "i": math.exp(-2 * r2)}


def _eval_form(expr, env):
    import re
    py = re.sub(r"(\d)([a-z])", r"\1*\2", expr)
    return eval(py, {"__builtins__": {}}, env)  # fixture text written in this repo


@pytest.mark.parametrize("name", ["A1", "A2"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_constructed_examples(name, dtype):
    ex = json.load(open(GOLDEN))[name]
    gqa = ex["gqa"]
    q = torch.tensor(ex["q"], dtype=dtype)[None]
    K = torch.tensor(ex["K"], dtype=dtype)[None, None]
    V = torch.tensor(ex["V"], dtype=dtype)[None, None]
    S, _ = oracle.block_summary(K, 2, 8)
    assert S[0, 0].float().tolist() == ex["summaries"]
    sc = oracle.block_score(q, S, gqa, 4)
    assert sc[0, 0].tolist() == ex["scores"]
    env = _closed_forms()
    for case in ex["cases"]:
        idx, _ = oracle.block_topk(sc, 4, case["k"])
        assert idx[0, 0].tolist() == case["idx"]
        if "out" not in case:
            continue
        out = oracle.decode_attention(q, K, V, gqa, 8, 2, idx=idx)
        forms = case["closed_form"]
        if gqa == 1:
            forms = [forms]
        for h in range(gqa):
            for c in range(2):
                cf = _eval_form(forms[h][c], env)
                assert cf == pytest.approx(case["out"][h][c], abs=1e-10)
                assert out[0, h, c].item() == pytest.approx(cf, abs=1e-13)


# ---------------------------------------------------------------- Quest-style bound

QUEST_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quest_example.json")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("block,ctx_len", [(16, 256), (16, 250), (32, 97), (4, 3), (1, 40)])
def test_quest_summary_is_blockwise_min_and_max(dtype, block, ctx_len):
    g = torch.Generator().manual_seed(block * 1000 + ctx_len)
    cap = (ctx_len + block - 1) // block * block
    K = torch.randn((2, 3, cap, 16), generator=g).to(dtype)
    K[:, :, ctx_len:] = float("nan")  # never read
    Sq = oracle.quest_summary(K, block, ctx_len)
    for j in range((ctx_len + block - 1) // block):
        part = K[:, :, j * block:min((j + 1) * block, ctx_len)].float()
        assert torch.equal(Sq[:, :, j, 0].float(), part.amin(dim=2))
        assert torch.equal(Sq[:, :, j, 1].float(), part.amax(dim=2))


def test_quest_score_bounds_every_token_of_its_block():
    # the bound is at least the group score of every key inside the block
    g = torch.Generator().manual_seed(91)
    q = torch.randn((2, 8, 32), generator=g)
    K = torch.randn((2, 2, 96, 32), generator=g)
    Sq = oracle.quest_summary(K, 16, 96)
    sc = oracle.quest_score(q, Sq, 4, 6)
    tok = torch.einsum("bgc,bgtc->bgt", q.double().view(2, 2, 4, 32).sum(dim=2), K.double())
    for j in range(6):
        worst = tok[:, :, j * 16:(j + 1) * 16].amax(dim=2)
        assert (worst <= sc[:, :, j] + 1e-12 * sc.abs().max()).all()
    # and each head's part is attained by the corner key that picks, per
    # channel, the minimum or the maximum by the sign of that head's query
    qd = q.double().view(2, 2, 4, 32)
    lo, hi = Sq[:, :, :, 0].double(), Sq[:, :, :, 1].double()
    corner = torch.where(qd[:, :, :, None, :] >= 0, hi[:, :, None], lo[:, :, None])
    attained = (qd[:, :, :, None, :] * corner).sum(dim=(2, 4))
    assert torch.allclose(attained, sc[:, :, :6], rtol=1e-13, atol=0)


def test_quest_block_of_one_is_the_token_score():
    # one key per block: the box is that key, the bound is q.k exactly
    w = Workload("t", batch=1, hq=6, hkv=2, ctx_len=50, block=1, topk=5, dtype="bf16", seed=66)
    inp = synth.make_inputs(w)
    Sq = oracle.quest_summary(inp["K"], 1, 50)
    S, _ = oracle.block_summary(inp["K"], 1, 50)
    assert torch.equal(oracle.quest_score(inp["q"], Sq, 3, 50), oracle.block_score(inp["q"], S, 3, 50))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quest_constructed_example(dtype):
    ex = json.load(open(QUEST_GOLDEN))
    q = torch.tensor([ex["q"]], dtype=dtype)                 # [1][2][2]
    K = torch.tensor([[ex["K"]]], dtype=dtype)               # [1][1][6][2]
    Sq = oracle.quest_summary(K, 2, 6)
    assert Sq[0, 0].float().tolist() == ex["minmax"]
    sc = oracle.quest_score(q, Sq, ex["gqa"], 3)
    assert sc[0, 0].tolist() == ex["scores"]
    for case in ex["cases"]:
        idx, _ = oracle.block_topk(sc, 3, case["k"])
        assert idx[0, 0].tolist() == case["idx"]
