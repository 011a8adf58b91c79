"""GPU parity of the token-level step (block = 1) against the oracle.

The oracle runs the same method with blocks of one token: its summaries are
then the keys themselves, its scores, top-k and attention are the ones the
block tests use.  Cases cover several rounds of the streaming selection,
split attention (few pairs) and one workgroup per pair, k = 1, k past the
context, the largest k, and exact ties (all keys equal: the lowest indices
are kept).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.workloads import Workload

from parity_util import GAP_MIN, TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def run_token(w, inp, k, scores=True):
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    idx = torch.full((w.batch, w.hkv, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    sc = torch.full((w.batch, w.hkv, w.cap), float("nan"), dtype=torch.float64,
                    device="cuda") if scores else None
    ws = torch.zeros(kb.kin_token_ws_bytes(desc, k), dtype=torch.uint8, device="cuda")
    kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], sc, k, idx, out, ws)
    torch.cuda.synchronize()
    return idx, out, sc


def check(w, inp, k, idx, out, sc, seqs, certify=True):
    L = w.ctx_len
    worst = 0.0
    for b in seqs:
        qb, Kb, Vb = inp["q"][b:b + 1].cpu(), inp["K"][b:b + 1].cpu(), inp["V"][b:b + 1].cpu()
        S_or, _ = oracle.block_summary(Kb, 1, L)  # block 1: the keys themselves
        assert torch.equal(S_or[:, :, :L].view(torch.int16), Kb[:, :, :L].view(torch.int16))
        sc_or = oracle.block_score(qb, S_or, w.gqa, L)
        if sc is not None:
            got = sc[b:b + 1, :, :L].cpu()
            scale = sc_or[:, :, :L].abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
            assert ((got - sc_or[:, :, :L]).abs() / scale).max() < 1e-13, f"scores, seq {b}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), L, k)
        if certify:
            assert (gap > GAP_MIN).all(), f"margin certificate fails at seq {b}"
        assert torch.equal(idx[b:b + 1].cpu(), idx_or), f"selection differs, seq {b}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, L, 1, idx=idx_or)
        og = out[b:b + 1].cpu().double()
        assert torch.isfinite(og).all(), f"unwritten output, seq {b}"
        err = (og - o).abs().max().item()
        assert err <= TOL["bf16"], f"output error {err}, seq {b}"
        worst = max(worst, err)
    return worst


TOKEN = [
    # name, batch, hq, hkv, ctx, k, t_cap
    ("tok-few-g4-ragged", 3, 16, 4, 5000, 100, 5120),      # 12 pairs: split attention
    ("tok-few-g8-k1", 2, 16, 2, 3000, 1, 3072),
    ("tok-few-g2-kpast", 2, 8, 4, 300, 400, 320),          # k > ctx: all kept, -1 after
    ("tok-many-g4-k1024", 64, 16, 4, 20000, 1024, 20480),  # 256 pairs: one workgroup each
    ("tok-long-g2-k2048", 1, 4, 2, 131072, 2048, 131072),  # 256 rounds of the select
    ("tok-tiles-g8-L131072", 2, 32, 4, 131072, 1000, 131072),  # each tile picks candidates
    ("tok-kmax-g4", 2, 4, 1, 40000, 8192, 40000),          # the largest k
    ("tok-g16-short", 2, 32, 2, 33, 32, 48),               # one round, ragged
    # at least as many pairs as CUs, at most 32768 tokens and 2048 kept: one kernel
    ("tok-single-g8-k2048-L32768", 32, 64, 8, 32768, 2048, 32768),
    ("tok-single-g1-kpast", 128, 2, 2, 700, 900, 704),     # k > ctx: all kept, -1 after
    ("tok-single-g2-k1-ragged", 128, 4, 2, 1001, 1, 1024),
]


@pytest.mark.parametrize("case", TOKEN, ids=[c[0] for c in TOKEN])
def test_token_step_against_oracle(case):
    name, b, hq, hkv, L, k, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=1, topk=k, dtype="bf16",
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}, ctx {L}, k {k}")
    inp = synth.make_inputs(w, device="cuda", tail_fill=float("nan"))
    idx, out, sc = run_token(w, inp, k)
    seqs = sorted({0, b // 2, b - 1})
    err = check(w, inp, k, idx, out, sc, seqs)
    if k > L:
        assert (idx[:, :, L:] == -1).all()
    # no scores buffer: the same selection and bits
    idx2, out2, _ = run_token(w, inp, k, scores=False)
    assert torch.equal(idx2, idx)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    say(f"  ok, max err {err:.3e}")


def test_token_step_exact_ties_keep_lowest_indices():
    """Every key equal: all scores tie, the k lowest token indices are kept
    and the output is the mean of their values."""
    w = Workload("tok-ties", batch=2, hq=8, hkv=2, ctx_len=3000, block=1, topk=300,
                 dtype="bf16", seed=4242, t_cap=3072)
    inp = synth.make_inputs(w, device="cuda", tail_fill=float("nan"))
    inp["K"][:, :, :3000] = inp["K"][:, :, :1].clone()
    idx, out, sc = run_token(w, inp, 300)
    want = torch.arange(300, dtype=torch.int32, device="cuda").expand(2, 2, 300)
    assert torch.equal(idx, want)
    check(w, inp, 300, idx, out, sc, [0, 1], certify=False)


def test_token_tile_candidates_exact_ties_keep_lowest_indices():
    """Few pairs and many tiles per pair, so every score tile selects its own
    candidates: every key equal, all scores tie in every tile and across
    them, and the k lowest token indices (all of the first tile's) are
    kept."""
    w = Workload("tok-ties-tiles", batch=2, hq=8, hkv=2, ctx_len=20000, block=1, topk=300,
                 dtype="bf16", seed=4245, t_cap=20000)
    inp = synth.make_inputs(w, device="cuda", tail_fill=float("nan"))
    inp["K"][:, :, :20000] = inp["K"][:, :, :1].clone()
    idx, out, sc = run_token(w, inp, 300)
    want = torch.arange(300, dtype=torch.int32, device="cuda").expand(2, 2, 300)
    assert torch.equal(idx, want)
    check(w, inp, 300, idx, out, sc, [0, 1], certify=False)


def test_token_single_kernel_exact_ties_keep_lowest_indices():
    """256 pairs (the one-kernel step): every key of a pair equal, so all
    top words tie, the low words are recomputed for every key and tie as
    well; the k lowest indices are kept."""
    w = Workload("tok-single-ties", batch=128, hq=8, hkv=2, ctx_len=3000, block=1, topk=300,
                 dtype="bf16", seed=4243, t_cap=3072)
    inp = synth.make_inputs(w, device="cuda", tail_fill=float("nan"))
    inp["K"][:, :, :3000] = inp["K"][:, :, :1].clone()
    idx, out, sc = run_token(w, inp, 300)
    want = torch.arange(300, dtype=torch.int32, device="cuda").expand(128, 2, 300)
    assert torch.equal(idx, want)
    check(w, inp, 300, idx, out, sc, [0, 127], certify=False)


def _order_key_top(x):
    """Top 32 bits of the order-preserving key of fp64 values (numpy)."""
    u = x.view(np.uint64)
    neg = (u >> np.uint64(63)) == 1
    key = np.where(neg, ~u, u | np.uint64(1 << 63))
    return key >> np.uint64(32)


def _plant_near_tie(inp, w, b, g, k, exact, above=False):
    """Overwrite a low-ranked key of pair (b, g) with the rank-k key (exact)
    or with that key moved by one bf16 step in two channels whose effects on
    the score nearly cancel: a score that agrees with the k-th in its top 32
    key bits and lies just above it (above) or just below it."""
    L = w.ctx_len
    q = inp["q"][b, g * w.gqa:(g + 1) * w.gqa].cpu().double().numpy()
    qs = q.sum(0)
    Kp = inp["K"][b, g, :L].cpu()
    sc = Kp.double().numpy() @ qs
    order = np.argsort(-sc, kind="stable")
    a, c = int(order[k - 1]), int(order[k + 20])
    row = Kp[a].clone()
    if not exact:
        bits16 = row.view(torch.int16).numpy().astype(np.int32)
        vals = row.double().numpy()
        steps = []  # per channel, the change of one bf16 step up or down in the bits
        for s in (1, -1):
            stepped = torch.from_numpy((bits16 + s).astype(np.int16)).view(torch.bfloat16)
            steps.append((stepped.double().numpy() - vals, s))
        cand = []
        for dv1, s1 in steps:
            for dv2, s2 in steps:
                d = np.add.outer(qs * dv1, qs * dv2)  # channel c1 moved by s1, c2 by s2
                np.fill_diagonal(d, np.nan)
                cand.append((d, s1, s2))
        target = abs(sc[a])
        pick = None
        for d, s1, s2 in cand:
            # below the top word's resolution (2^-20 relative), far above fp64 rounding
            ok = np.isfinite(d) & (np.abs(d) > 1e-12 * target) & (np.abs(d) < 4e-7 * target)
            ii = np.argwhere(ok)
            for c1, c2 in ii[:200]:
                new = row.view(torch.int16).clone()
                new[c1] += s1
                new[c2] += s2
                nv = float(new.view(torch.bfloat16).double().numpy() @ qs)
                if _order_key_top(np.array([nv])) == _order_key_top(np.array([sc[a]])) \
                        and (nv > sc[a] if above else nv < sc[a]):
                    pick = new.view(torch.bfloat16)
                    break
            if pick is not None:
                break
        assert pick is not None, "no near tie found"
        row = pick
    inp["K"][b, g, c] = row.cuda()


@pytest.mark.parametrize("batch,k", [(64, 100), (2, 100), (2, 200)],
                         ids=["one-kernel", "two-kernel-tile-candidates", "two-kernel-all-words"])
def test_token_near_ties_below_the_top_word(batch, k):
    """Planted keys whose scores equal the k-th score in the top 32 bits of
    the order key (near ties: they differ below; exact ties: they do not):
    the recomputed low words must order them as the oracle does, in the
    one-kernel step (256 pairs: the top words in LDS) and in the two-kernel
    step (8 pairs): with k = 100 each of the 16 score tiles selects its own
    100 candidates first (their top words handed over in memory), with k =
    200 the tiles' candidates would outnumber the 2000 tokens, so every
    token's top word is handed over."""
    w = Workload(f"tok-near-b{batch}-k{k}", batch=batch, hq=16, hkv=4, ctx_len=2000, block=1,
                 topk=k, dtype="bf16", seed=4244, t_cap=2048)
    inp = synth.make_inputs(w, device="cuda", tail_fill=float("nan"))
    last = batch - 1
    # (sequence, KV head, exact tie, planted key just above the k-th)
    planted = [(0, 0, False, False), (0, 1, True, False), (last, 2, False, True),
               (last, 3, True, False), (last, 0, False, True)]
    for b, g, exact, above in planted:
        _plant_near_tie(inp, w, b, g, k, exact, above)
    idx, out, sc = run_token(w, inp, k)
    check(w, inp, k, idx, out, sc, sorted({p[0] for p in planted}), certify=False)
    idx2, out2, _ = run_token(w, inp, k, scores=False)
    assert torch.equal(idx2, idx)
