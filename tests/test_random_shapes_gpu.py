"""GPU parity on seeded random shapes: the decode steps (block, token-level,
Quest-style, paged with variable lengths, shared prompts) over drawn batch
sizes, GQA ratios, block and page sizes, context lengths and budgets, so
that every launch form the library picks (one kernel with 8 or 4 waves,
two kernels with split attention, the separate calls past 2048 kept
blocks, fp32) meets shapes no hand-written case names.  Each case checks
sequences against the oracle with the rules of the other parity tests, and
the call without a scores buffer bit for bit against the call with one.
"""
import random
import zlib

import pytest
import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.workloads import Workload

from parity_util import GAP_MIN, TOL, bits, check_sequences, gpu_inputs, run_gpu, say
from test_paged_gpu import check_paged_case
from test_shared_gpu import check_shared_case

pytestmark = pytest.mark.gpu

NAN = float("nan")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _draw_block_case(rng, i):
    kind = rng.choice(["few", "few", "many", "many4w", "f32"])
    block = rng.choice([16, 32, 64, 128])
    gqa = rng.choice([1, 2, 3, 4, 5, 8, 16])
    if kind == "f32":
        batch, hkv, dt = rng.randint(1, 3), rng.choice([1, 2]), "f32"
    elif kind == "few":
        batch, hkv, dt = rng.randint(1, 6), rng.choice([1, 2, 4, 8]), "bf16"
    elif kind == "many":  # at least as many pairs as CUs: one kernel
        hkv = rng.choice([2, 4, 8])
        batch, dt = 256 // hkv + rng.randint(0, 40), "bf16"
    else:  # two pairs per CU: the 4-wave shape (blocks of at most 64)
        hkv, block = rng.choice([4, 8]), rng.choice([16, 32, 64])
        batch, dt = 512 // hkv + rng.randint(0, 20), "bf16"
    ctx = rng.randint(1, 6000 if kind in ("few", "f32") else 2500)
    cap = ctx + rng.randint(0, 150)
    nb = (ctx + block - 1) // block
    k = rng.randint(1, nb + 3)
    if rng.random() < 0.15:
        k = nb  # every block kept
    return (f"rand{i}-{kind}-b{batch}-g{gqa}-kv{hkv}-B{block}-L{ctx}-k{k}", batch, gqa * hkv, hkv,
            ctx, block, k, dt, cap)


BLOCK_CASES = [_draw_block_case(random.Random(9000 + i), i) for i in range(24)]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_random_block_step(case):
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}, nb {w.nb}")
    inp = gpu_inputs(w)
    step = run_gpu(w, inp, step=True)
    seqs = sorted({0, b // 2, b - 1})
    r = check_sequences(w, inp, step, seqs)
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, step.idx)
    assert torch.equal(bits(quiet.out), bits(step.out))
    if k > w.nb:
        assert (step.idx[:, :, w.nb:] == -1).all()
    say(f"  ok {r}")


def _draw_token_case(rng, i):
    if rng.random() < 0.5:  # one kernel: pairs cover the chip, ctx <= 32768, k <= 2048
        hkv = rng.choice([2, 4, 8])
        batch = 256 // hkv + rng.randint(0, 16)
        ctx = rng.randint(1, 12000)
        k = rng.randint(1, 2048)
    else:
        hkv, batch = rng.choice([1, 2, 4]), rng.randint(1, 4)
        ctx = rng.randint(1, 50000)
        k = rng.randint(1, 4000)
    gqa = rng.choice([1, 2, 4, 8])
    cap = ctx + rng.randint(0, 100)
    return (f"tok{i}-b{batch}-g{gqa}-kv{hkv}-L{ctx}-k{k}", batch, gqa * hkv, hkv, ctx, k, cap)


def _draw_token_tile_case(rng, i):
    """Few pairs, long contexts and k below a score tile's length: the
    shapes for which each score tile first keeps its own k best tokens."""
    hkv = rng.choice([2, 4, 8])
    batch = max(1, rng.choice([16, 32, 64, 128]) // hkv + rng.randint(-1, 1))
    ctx = rng.randint(8000, 100000)
    rows = ctx * batch * hkv // 256  # about one tile's tokens
    k = rng.randint(1, max(1, min(8192, rows // 2)))
    gqa = rng.choice([1, 2, 4, 8])
    cap = ctx + rng.randint(0, 100)
    return (f"toktile{i}-b{batch}-g{gqa}-kv{hkv}-L{ctx}-k{k}", batch, gqa * hkv, hkv, ctx, k, cap)


TOKEN_CASES = [_draw_token_case(random.Random(9100 + i), i) for i in range(10)] + \
    [_draw_token_tile_case(random.Random(9200 + i), i) for i in range(4)]


def _run_token(w, inp, k, scores):
    desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, 1, torch.bfloat16)
    idx = torch.full((w.batch, w.hkv, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.hq, 128), NAN, dtype=torch.bfloat16, device="cuda")
    sc = torch.full((w.batch, w.hkv, w.cap), NAN, dtype=torch.float64,
                    device="cuda") if scores else None
    ws = torch.zeros(max(kb.kin_token_ws_bytes(desc, k), 16), dtype=torch.uint8, device="cuda")
    kb.kin_token_decode_step(desc, inp["q"], inp["K"], inp["V"], sc, k, idx, out, ws)
    torch.cuda.synchronize()
    return idx, out, sc


@pytest.mark.parametrize("case", TOKEN_CASES, ids=[c[0] for c in TOKEN_CASES])
def test_random_token_step(case):
    name, b, hq, hkv, L, k, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=1, topk=k, dtype="bf16",
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}")
    inp = synth.make_inputs(w, device="cuda", tail_fill=NAN)
    idx, out, sc = _run_token(w, inp, k, True)
    for s in sorted({0, b - 1}):
        qb, Kb, Vb = inp["q"][s:s + 1].cpu(), inp["K"][s:s + 1].cpu(), inp["V"][s:s + 1].cpu()
        S_or, _ = oracle.block_summary(Kb, 1, L)
        sc_or = oracle.block_score(qb, S_or, w.gqa, L)
        ref = sc_or[:, :, :L]
        scale = ref.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
        assert ((sc[s:s + 1, :, :L].cpu() - ref).abs() / scale).max() < 1e-13, f"scores, seq {s}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), L, k)
        assert (gap > GAP_MIN).all(), f"margin certificate fails, seq {s}"
        assert torch.equal(idx[s:s + 1].cpu(), idx_or), f"selection differs, seq {s}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, L, 1, idx=idx_or)
        og = out[s:s + 1].cpu().double()
        assert torch.isfinite(og).all(), f"unwritten output, seq {s}"
        assert (og - o).abs().max().item() <= TOL["bf16"], f"output, seq {s}"
    idx2, out2, _ = _run_token(w, inp, k, False)
    assert torch.equal(idx2, idx)
    assert torch.equal(bits(out2), bits(out))
    say("  ok")


def _draw_quest_case(rng, i):
    block = rng.choice([16, 32, 64, 128])
    gqa = rng.choice([1, 2, 4, 8])
    if rng.random() < 0.5:
        hkv = rng.choice([2, 4, 8])
        batch = 256 // hkv + rng.randint(0, 20)
        if block <= 64 and rng.random() < 0.5:
            batch = 512 // hkv + rng.randint(0, 10)  # the 4-wave shape
        ctx = rng.randint(1, 2500)
    else:
        hkv, batch = rng.choice([1, 2, 4]), rng.randint(1, 4)
        ctx = rng.randint(1, 6000)
    nb = (ctx + block - 1) // block
    k = min(rng.randint(1, nb + 3), 2048)
    cap = ctx + rng.randint(0, 150)
    return (f"quest{i}-b{batch}-g{gqa}-kv{hkv}-B{block}-L{ctx}-k{k}", batch, gqa * hkv, hkv, ctx,
            block, k, cap)


QUEST_CASES = [_draw_quest_case(random.Random(9200 + i), i) for i in range(8)]


@pytest.mark.parametrize("case", QUEST_CASES, ids=[c[0] for c in QUEST_CASES])
def test_random_quest_step(case):
    name, b, hq, hkv, L, B, k, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype="bf16",
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: pairs {w.pairs}, nb {w.nb}")
    inp = synth.make_inputs(w, device="cuda", tail_fill=NAN)
    desc = kb.make_desc(b, hkv, w.gqa, w.cap, L, B, torch.bfloat16)
    ws = torch.zeros(kb.kin_quest_ws_bytes(desc, k), dtype=torch.uint8, device="cuda")

    def run(scores):
        Sq = torch.full((b, hkv, w.nb_cap, 2, 128), NAN, dtype=torch.bfloat16, device="cuda")
        newest0 = (w.nb - 1) * B
        if newest0 > 0:
            kb.kin_quest_summary_update(desc, inp["K"], Sq, 0, newest0)
        sc = torch.full((b, hkv, w.nb_cap), NAN, dtype=torch.float64,
                        device="cuda") if scores else None
        idx = torch.full((b, hkv, k), -7, dtype=torch.int32, device="cuda")
        out = torch.full((b, hq, 128), NAN, dtype=torch.bfloat16, device="cuda")
        kb.kin_quest_decode_step(desc, inp["q"], inp["K"], inp["V"], Sq, sc, k, idx, out, ws)
        torch.cuda.synchronize()
        return Sq, sc, idx, out

    Sq, sc, idx, out = run(True)
    nb = w.nb
    for s in sorted({0, b - 1}):
        qb, Kb, Vb = inp["q"][s:s + 1].cpu(), inp["K"][s:s + 1].cpu(), inp["V"][s:s + 1].cpu()
        Sq_or = oracle.quest_summary(Kb, B, L)
        assert torch.equal(bits(Sq[s:s + 1, :, :nb].cpu()), bits(Sq_or[:, :, :nb])), f"rows {s}"
        sc_or = oracle.quest_score(qb, Sq_or, w.gqa, nb)
        ref = sc_or[:, :, :nb]
        scale = ref.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
        assert ((sc[s:s + 1, :, :nb].cpu() - ref).abs() / scale).max() < 1e-13, f"bounds {s}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), nb, k)
        assert (gap > GAP_MIN).all(), f"margin certificate fails, seq {s}"
        assert torch.equal(idx[s:s + 1].cpu(), idx_or), f"selection differs, seq {s}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, L, B, idx=idx_or)
        og = out[s:s + 1].cpu().double()
        assert torch.isfinite(og).all(), f"unwritten output, seq {s}"
        assert (og - o).abs().max().item() <= TOL["bf16"], f"output, seq {s}"
    _, _, idx2, out2 = run(False)
    assert torch.equal(idx2, idx)
    assert torch.equal(bits(out2), bits(out))
    say("  ok")


def _draw_paged_case(rng, i):
    kind = rng.choice(["few", "few", "many", "many4w"])
    block = rng.choice([16, 32, 64, 128])
    gqa = rng.choice([1, 2, 3, 4, 8, 16])
    if kind == "few":
        batch, hkv, max_len = rng.randint(1, 6), rng.choice([1, 2, 4]), rng.randint(1, 6000)
    elif kind == "many":  # at least as many pairs as CUs: one kernel
        hkv = 8
        batch, max_len = 32 + rng.randint(0, 6), rng.randint(1, 2500)
    else:  # two pairs per CU: the 4-wave shape
        hkv, block = 8, rng.choice([16, 32, 64])
        batch, max_len = 64 + rng.randint(0, 4), rng.randint(1, 1500)
    page = max(16, block) << rng.randint(0, 3)
    nb = (max_len + block - 1) // block
    k = min(rng.randint(1, nb + 3), 2048)
    lens = rng.choice(["rand", "edge"])
    return (f"paged{i}-{kind}-b{batch}-g{gqa}-kv{hkv}-B{block}-P{page}-L{max_len}-k{k}-{lens}",
            batch, hkv, gqa, block, page, max_len, k, lens)


PAGED_CASES = [_draw_paged_case(random.Random(9300 + i), i) for i in range(8)]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_random_paged_step(case):
    check_paged_case(case)


def _draw_shared_case(rng, i):
    block = rng.choice([16, 32, 64, 128])
    gqa = rng.choice([1, 2, 4, 5, 8])
    if rng.random() < 0.5:  # at least as many pairs as CUs
        hkv = 8
        n_prompts, n_share = rng.choice([(4, 8), (8, 4), (2, 16), (3, 11)])
        ctx = rng.randint(2 * block, 3000)
    else:
        hkv = rng.choice([1, 2, 4])
        n_prompts, n_share = rng.randint(1, 3), rng.randint(1, 4)
        ctx = rng.randint(2 * block, 5000)
    prompt = block * rng.randint(1, (ctx - 1) // block)
    nb = (ctx + block - 1) // block
    k = min(rng.randint(1, nb + 3), 2048)
    return (f"shared{i}-p{n_prompts}x{n_share}-g{gqa}-kv{hkv}-B{block}-P{prompt}-L{ctx}-k{k}",
            n_prompts, n_share, hkv, gqa, block, prompt, ctx, k)


SHARED_CASES = [_draw_shared_case(random.Random(9400 + i), i) for i in range(8)]


@pytest.mark.parametrize("case", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_random_shared_step(case):
    check_shared_case(case)
