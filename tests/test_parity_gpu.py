"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases run the whole oracle (several tiles, ragged tails, every block
size, GQA 1..16, k from 1 past nb, NaN-filled cache tails); the workload
shapes run at full size with every sequence's selection checked bit-exactly
and outputs checked on sampled sequences.
"""
import zlib

import pytest
import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth, workloads
from block_top_sparse_amd.buffers import LayerBuffers
from block_top_sparse_amd.workloads import Workload

from parity_util import TOL, bits, check_sequences, gpu_inputs, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()  # loud failure if the library is missing


SMALL = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap
    ("f32-g4-b16", 2, 8, 2, 1000, 16, 9, "f32", 1024),
    ("f32-g1-b32-k1", 3, 2, 2, 333, 32, 1, "f32", 400),
    ("f32-g16-b64", 1, 32, 2, 700, 64, 3, "f32", 704),
    ("bf16-g4-b16", 2, 8, 2, 2000, 16, 17, "bf16", 2048),
    ("bf16-g5-b32", 2, 10, 2, 1500, 32, 8, "bf16", 1600),
    ("bf16-g8-b64", 2, 16, 2, 4000, 64, 5, "bf16", 4096),
    ("bf16-g16-b128", 1, 32, 2, 2100, 128, 4, "bf16", 2176),
    ("bf16-g1-b16-k1", 2, 3, 3, 99, 16, 1, "bf16", 100),
    ("bf16-g3-b16-allm1", 2, 6, 2, 250, 16, 15, "bf16", 256),   # k = nb - 1
    ("bf16-g4-b32-keepall", 2, 8, 2, 290, 32, 10, "bf16", 320),  # k = nb (ragged last block)
    ("bf16-g4-b16-kpast", 1, 8, 2, 100, 16, 12, "bf16", 128),    # k > nb: -1 padding
    ("f32-g2-b16-short", 1, 4, 2, 5, 16, 2, "f32", 16),          # one partial block
    ("bf16-g8-b16-manyblk", 2, 16, 2, 40000, 16, 64, "bf16", 40000),  # nb 2500: 5 keys/thread
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_against_oracle(case):
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt, seed=
                 zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, dense=True)
    r = check_sequences(w, inp, bufs, range(b), check_dense=True)
    idx = bufs.idx.cpu()
    if k > w.nb:
        assert (idx[:, :, w.nb:] == -1).all()
    say(f"  ok {r}")


FUSED = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap
    ("fused-bf16-many-pairs", 40, 32, 8, 4096, 16, 32, "bf16", 4096),   # one workgroup per pair
    ("fused-bf16-few-pairs", 2, 16, 2, 8000, 16, 100, "bf16", 8192),    # split + combine
    ("fused-bf16-ragged-b64", 3, 24, 3, 5000, 64, 20, "bf16", 5120),
    ("fused-bf16-keepall", 2, 8, 2, 1000, 32, 40, "bf16", 1024),        # k > nb
    ("fused-bf16-g1-k1", 2, 2, 2, 77, 16, 1, "bf16", 80),
    ("fused-bf16-bigk-fallback", 1, 8, 2, 40000, 16, 2100, "bf16", 40000),  # k > LDS list
    ("fused-f32-tiny", 1, 8, 2, 4096, 16, 32, "f32", 4096),
    ("fused-f32-ragged", 2, 12, 2, 999, 32, 7, "f32", 1024),
]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_fused_step_halves_against_oracle(case):
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, fused=True)
    r = check_sequences(w, inp, bufs, range(b))
    # the fused halves select exactly what the separate calls select
    sep = run_gpu(w, inp)
    assert torch.equal(sep.idx, bufs.idx)
    assert torch.equal(bits(sep.S[:, :, :w.nb]), bits(bufs.S[:, :, :w.nb]))
    say(f"  ok {r}")


SINGLE = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap  (>= 256 pairs: one kernel per step)
    ("step-g4-b16-ragged", 64, 16, 4, 2000, 16, 20, "bf16", 2048),
    ("step-g5-b32-k1", 32, 40, 8, 1111, 32, 1, "bf16", 1152),
    ("step-g8-b64-kpast", 32, 64, 8, 700, 64, 15, "bf16", 704),      # k > nb
    ("step-g1-b16-manyblk", 256, 1, 1, 60000, 16, 100, "bf16", 60000),  # nb 3750
    ("step-g16-b128-short", 16, 256, 16, 100, 128, 2, "bf16", 128),  # a single partial block
    # >= 2 pairs per CU, nb <= 2048, block <= 64: the 4-wave step, two per CU
    ("step4w-g4-b16-ragged", 128, 16, 4, 2000, 16, 20, "bf16", 2048),
    ("step4w-g8-b64-kpast", 64, 64, 8, 700, 64, 15, "bf16", 704),    # k > nb
    ("step4w-g5-b32-k1", 130, 20, 4, 1111, 32, 1, "bf16", 1152),
    ("step4w-g2-b16-nb2048", 512, 2, 1, 32768, 16, 64, "bf16", 32768),
]


@pytest.mark.parametrize("case", SINGLE, ids=[c[0] for c in SINGLE])
def test_single_kernel_step_against_oracle(case):
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, step=True)
    seqs = sorted({0, 1, b // 2, b - 1})
    r = check_sequences(w, inp, bufs, seqs)
    sep = run_gpu(w, inp)
    assert torch.equal(sep.idx, bufs.idx)
    assert torch.equal(bits(sep.S[:, :, :w.nb]), bits(bufs.S[:, :, :w.nb]))
    assert torch.equal(sep.scores[:, :, :w.nb], bufs.scores[:, :, :w.nb])
    # without a scores buffer: the same selection and output, scores untouched
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, bufs.idx)
    assert torch.equal(bits(quiet.out), bits(bufs.out))
    assert torch.equal(bits(quiet.S[:, :, :w.nb]), bits(bufs.S[:, :, :w.nb]))
    assert torch.isnan(quiet.scores).all()
    say(f"  ok {r}")


FEW_PAIRS = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap  (bf16, fewer pairs than CUs: the
    # two-kernel step)
    ("few-g4-b16-ragged", 3, 16, 4, 5000, 16, 40, "bf16", 5120),
    ("few-255-pairs", 51, 20, 5, 3000, 16, 30, "bf16", 3008),       # one CU short of one per pair
    ("few-g8-b64-k1", 2, 64, 8, 3000, 64, 1, "bf16", 3072),         # one split
    ("few-g5-b32-kpast", 4, 20, 4, 700, 32, 40, "bf16", 704),       # k > nb
    ("few-g1-b16-nb8192", 1, 2, 2, 131072, 16, 512, "bf16", 131072),
    # more than 4096 blocks per pair, k below a tile's length: the score
    # tiles hand over their own k best (a tail tile shorter than k pads)
    ("few-g4-b16-cand", 2, 16, 4, 100000, 16, 120, "bf16", 100096),
    ("few-g2-b32-cand-ragged", 4, 8, 4, 150000, 32, 200, "bf16", 150016),
    ("few-g16-b128", 2, 64, 4, 20000, 128, 10, "bf16", 20096),
]


@pytest.mark.parametrize("case", FEW_PAIRS, ids=[c[0] for c in FEW_PAIRS])
def test_few_pair_step_against_oracle(case):
    """kin_sparse_decode_step with few pairs (split attention): the selection
    must equal the four-call path's, the output the oracle's, and repeated
    calls on the same workspace must agree bitwise, with or without a scores
    buffer."""
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    ref = run_gpu(w, inp)  # four calls
    step = run_gpu(w, inp, step=True)
    assert torch.equal(step.idx, ref.idx)
    assert torch.equal(step.scores[:, :, :w.nb], ref.scores[:, :, :w.nb])
    r = check_sequences(w, inp, step, range(b))
    out1 = step.out.clone()
    again = run_gpu(w, inp, step=True, bufs=step)
    assert torch.equal(bits(again.out), bits(out1))
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, ref.idx)
    assert torch.equal(bits(quiet.out), bits(out1))
    say(f"  ok {r}")


NEWEST_ROW = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap
    ("newest-single-nb1", 16, 256, 16, 100, 128, 2, "bf16", 128),   # one kernel, one block
    ("newest-single-nb2", 32, 64, 8, 150, 128, 1, "bf16", 256),     # one kernel, two blocks
    ("newest-few-nb1", 2, 16, 4, 90, 128, 3, "bf16", 128),          # two kernels
    ("newest-few-nb3", 2, 16, 4, 40, 16, 1, "bf16", 48),
    ("newest-few-keepall-split", 2, 16, 4, 700, 32, 40, "bf16", 704),  # two splits per pair
    ("newest-two-kernel-f32", 2, 8, 2, 70, 64, 1, "f32", 128),      # update + score kernel
]


@pytest.mark.parametrize("case", NEWEST_ROW, ids=[c[0] for c in NEWEST_ROW])
def test_newest_row_independent_of_old_contents(case):
    """The step rewrites the newest block's summary row while it scores the
    other rows; the row must come out as the oracle's whatever S held before
    (no load of that row may be in flight while it is stored)."""
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    S_or, _ = oracle.block_summary(inp["K"].cpu(), w.block, w.ctx_len)
    want = bits(S_or[:, :, :w.nb])
    for fill in (0.0, 1.0, -3.0, float("nan")):
        for scores in (True, False):
            bufs = LayerBuffers(w)
            newest0 = (w.nb - 1) * w.block
            if newest0 > 0:
                kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, newest0)
            bufs.S[:, :, w.nb - 1:].fill_(fill)
            kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S,
                                      bufs.scores if scores else None, bufs.k, bufs.idx,
                                      bufs.out, bufs.ws)
            torch.cuda.synchronize()
            got = bits(bufs.S[:, :, :w.nb].cpu())
            assert torch.equal(got, want), f"fill {fill}, scores {scores}"
    say("  ok")


NO_SCORES_TWO_KERNEL = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap  (few pairs: two kernels)
    ("nosc-g4-b16", 2, 8, 2, 3000, 16, 24, "bf16", 3072),
    ("nosc-g5-b32-f32", 3, 10, 2, 999, 32, 7, "f32", 1024),
    ("nosc-g8-b64-kpast", 1, 16, 2, 500, 64, 20, "bf16", 512),
]


@pytest.mark.parametrize("case", NO_SCORES_TWO_KERNEL, ids=[c[0] for c in NO_SCORES_TWO_KERNEL])
def test_two_kernel_step_without_scores_buffer(case):
    """scores == NULL in the two-kernel form: the scores live in the
    workspace; idx and out equal those of the call with a scores buffer."""
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    ref = run_gpu(w, inp, step=True)
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, ref.idx)
    assert torch.equal(bits(quiet.out), bits(ref.out))
    assert torch.isnan(quiet.scores).all()
    r = check_sequences(w, inp, quiet, range(b), check_scores=False)
    say(f"  ok {r}")


F32_SPLIT = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap  (few pairs, several splits)
    ("f32split-g1-b16-k292", 3, 2, 2, 4730, 16, 292, "f32", 4793),
    ("f32split-g4-b128-k14", 2, 8, 2, 5401, 128, 14, "f32", 5500),
    ("f32split-g5-b16-keepall", 3, 10, 2, 5936, 16, 371, "f32", 5999),
]


@pytest.mark.parametrize("case", F32_SPLIT, ids=[c[0] for c in F32_SPLIT])
def test_f32_two_kernel_step_splits_on_a_stale_workspace(case):
    """The fp32 two-kernel step with its attention split over several
    workgroups per pair: its scoring kernel clears the arrival words the
    splits count in, so even a workspace holding other bytes (here all ones,
    then the first call's own) gives the same result."""
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    bufs = LayerBuffers(w, k=k)
    assert bufs.ws is not None, "the plan must split (a workspace is needed)"
    bufs.ws.fill_(0xFF)
    step = run_gpu(w, inp, step=True, bufs=bufs)
    r = check_sequences(w, inp, step, range(b))
    first = (step.idx.clone(), step.out.clone())
    again = run_gpu(w, inp, step=True, bufs=bufs)  # the workspace as the first call left it
    assert torch.equal(again.idx, first[0])
    assert torch.equal(bits(again.out), bits(first[1]))
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(bits(quiet.out), bits(first[1]))
    say(f"  ok {r}")


def test_tiny_workload_full_parity():
    w = workloads.TINY
    say(f"workload {w.name}")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, dense=True)
    r = check_sequences(w, inp, bufs, range(w.batch), check_dense=True)
    say(f"  ok {r}")


def test_keep_all_blocks_equals_dense_bitwise():
    # with every block kept the token list is [0, ctx_len) in the same order
    # and the same split plan, so sparse and dense agree to the bit
    for dt in ("bf16", "f32"):
        w = Workload(f"keepall-{dt}", batch=2, hq=16, hkv=2, ctx_len=2048, block=32, topk=64,
                     dtype=dt, seed=71)
        inp = gpu_inputs(w)
        bufs = run_gpu(w, inp, dense=True)
        assert bufs.idx.cpu()[0, 0].tolist() == list(range(64))
        assert torch.equal(bits(bufs.out), bits(bufs.out_dense)), dt
        check_sequences(w, inp, bufs, [1], check_dense=True)


def test_deterministic_and_stream_ordered():
    w = Workload("det", batch=4, hq=32, hkv=8, ctx_len=8192, block=16, topk=64, dtype="bf16",
                 seed=81)
    inp = gpu_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = run_gpu(w, inp, stream=s)
        out1, idx1 = a.out.clone(), a.idx.clone()
        a = run_gpu(w, inp, stream=s, bufs=a)
    assert torch.equal(idx1, a.idx)
    assert torch.equal(bits(out1), bits(a.out))
    check_sequences(w, inp, a, [0, 3])


def test_decode_steps_update_newest_block():
    # grow the context one token at a time: the newest-block update must give
    # the same summaries as a full rebuild, and the fused step entry must
    # match the oracle at every step
    w0 = Workload("decode", batch=2, hq=8, hkv=2, ctx_len=600, block=16, topk=6, dtype="bf16",
                  seed=91, t_cap=700)
    inp = gpu_inputs(w0.scaled(ctx_len=700))  # rows 600..699 are the tokens to come
    bufs = LayerBuffers(w0, k=w0.topk)
    kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, w0.ctx_len)
    for L in range(601, 642):
        w = w0.scaled(ctx_len=L)
        d = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, L, w.block, torch.bfloat16)
        bufs.desc = d
        kb.kin_sparse_decode_step(d, inp["q"], inp["K"], inp["V"], bufs.S, bufs.scores, w.topk,
                                  bufs.idx, bufs.out, bufs.ws)
        torch.cuda.synchronize()
        if L % 8 == 1 or L == 641:
            check_sequences(w, inp, bufs, range(w.batch))
    full = LayerBuffers(w, k=w.topk)
    kb.kin_block_summary_update(full.desc, inp["K"], full.S, 0, w.ctx_len)
    torch.cuda.synchronize()
    assert torch.equal(bits(full.S[:, :, :w.nb]), bits(bufs.S[:, :, :w.nb]))


def test_workspace_too_small_is_rejected():
    w = workloads.QWEN3_8B.scaled(ctx_len=4096, batch=2)
    inp = gpu_inputs(w)
    bufs = LayerBuffers(w)
    n = kb.kin_sparse_ws_bytes(bufs.desc, w.topk)
    if n == 0:
        pytest.skip("no workspace needed for this plan")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kb.KinError) as e:
        kb.kin_sparse_decode_attn(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.idx, w.topk,
                                  bufs.out, small)
    assert e.value.status == -6
    # the two-kernel step without a scores buffer keeps the scores in ws
    with pytest.raises(kb.KinError) as e:
        kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S, None,
                                  w.topk, bufs.idx, bufs.out, small)
    assert e.value.status == -6
    kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, w.ctx_len)
    kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S, None, w.topk,
                              bufs.idx, bufs.out, bufs.ws)  # kin_sparse_ws_bytes is enough
    torch.cuda.synchronize()
    check_sequences(w, inp, bufs, [0, 1], check_scores=False)


@pytest.mark.parametrize("w", [workloads.QWEN3_8B, workloads.QWEN3_14B, workloads.QWEN3_32B],
                         ids=lambda w: w.name)
def test_full_size_workloads(w):
    say(f"workload {w.name}: generating {w.cache_bytes() / 2**30:.1f} GiB cache")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, dense=True)
    say("  gpu done; checking every sequence's selection")
    r = check_sequences(w, inp, bufs, range(w.batch), check_out=False)
    sample = [0, w.batch // 2, w.batch - 1]
    r2 = check_sequences(w, inp, bufs, sample, check_out=True, check_dense=True)
    # the decode-step forms (the benchmarked path) on the same inputs
    fused = run_gpu(w, inp, fused=True)
    assert torch.equal(fused.idx, bufs.idx)
    check_sequences(w, inp, fused, sample, check_out=True)
    step = run_gpu(w, inp, step=True)
    assert torch.equal(step.idx, bufs.idx)
    assert torch.equal(step.scores[:, :, :w.nb], bufs.scores[:, :, :w.nb])
    check_sequences(w, inp, step, sample, check_out=True)
    quiet = run_gpu(w, inp, step=True, no_scores=True)  # the benchmarked call
    assert torch.equal(quiet.idx, bufs.idx)
    assert torch.equal(bits(quiet.out), bits(step.out))
    if w.heavy_blocks:
        heavy = synth.heavy_block_ids(w, device="cuda")
        idx = bufs.idx.cpu()
        for b in range(w.batch):
            for g in range(w.hkv):
                assert set(heavy[b][g]) <= set(idx[b, g].tolist())
    say(f"  ok min_gap={r['min_gap']:.3g} {r2}")


SWEEP_SAMPLE = ["sweep-b8-ctx131072-blk16-budget8192", "sweep-b128-ctx8192-blk64-budget256",
                "sweep-b32-ctx32768-blk32-budget1024", "sweep-b8-ctx8192-blk32-allblocks",
                "sweep-b32-ctx131072-blk64-budget4096",
                "sweep-b8-ctx131072-blk16-allblocks"]  # 8192 kept blocks: four launches


@pytest.mark.parametrize("name", SWEEP_SAMPLE)
def test_sweep_points(name):
    w = workloads.by_name(name)
    say(f"workload {w.name}: cache {w.cache_bytes() / 2**30:.1f} GiB")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp)
    seqs = sorted({0, w.batch // 2, w.batch - 1})
    r = check_sequences(w, inp, bufs, seqs)
    fused = run_gpu(w, inp, fused=True)
    assert torch.equal(fused.idx, bufs.idx)
    check_sequences(w, inp, fused, seqs)
    step = run_gpu(w, inp, step=True)
    assert torch.equal(step.idx, bufs.idx)
    check_sequences(w, inp, step, seqs)
    # the benchmarked call: no scores output (a step that keeps every block
    # then has no scoring launch at all when the pairs are few)
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, bufs.idx)
    check_sequences(w, inp, quiet, seqs, check_scores=False)
    say(f"  ok {r}")


def _crafted_scores(kind, pairs, nb, gen):
    if kind == "normal":
        return torch.randn((pairs, nb), generator=gen, dtype=torch.float64) * 6
    if kind == "ties":
        return torch.round(torch.randn((pairs, nb), generator=gen, dtype=torch.float64) * 4) / 8
    if kind == "equal":
        return torch.full((pairs, nb), 2.5, dtype=torch.float64)
    if kind == "wide":  # exponents far apart: the k-th key lies > 255 binades below the max
        e = torch.randint(-1000, 1000, (pairs, nb), generator=gen).double()
        s = torch.where(torch.rand((pairs, nb), generator=gen) < 0.5, -1.0, 1.0).double()
        return s * torch.pow(torch.tensor(2.0, dtype=torch.float64), e)
    if kind == "zeros":  # +0, -0, denormals and their negatives
        v = torch.tensor([0.0, -0.0, 5e-324, -5e-324, 1e-310, -1e-310, 1.0], dtype=torch.float64)
        return v[torch.randint(0, len(v), (pairs, nb), generator=gen)]
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "wide", "zeros"])
@pytest.mark.parametrize("nb", [37, 2048, 8192])
def test_topk_crafted_scores_bit_exact(kind, nb):
    gen = torch.Generator().manual_seed(zlib.crc32(f"{kind}-{nb}".encode()))
    pairs = 24
    sc = _crafted_scores(kind, pairs, nb, gen).view(4, 6, nb).contiguous()
    d = kb.make_desc(4, 6, 1, nb * 16, nb * 16, 16, torch.bfloat16)
    sc_gpu = sc.cuda()
    for k in sorted({1, 2, 7, 64, nb - 1, nb, nb + 3}):
        if k < 1:
            continue
        idx = torch.full((4, 6, k), -9, dtype=torch.int32, device="cuda")
        kb.kin_block_topk(d, sc_gpu, k, idx)
        torch.cuda.synchronize()
        ref, _ = oracle.block_topk(sc, nb, k)
        assert torch.equal(idx.cpu(), ref), (kind, nb, k)


def _tied_cache(b, hkv, gqa, L, B, scales, seed):
    """A cache whose blocks are copies of a few block patterns per pair: one
    pattern of all zeros (its score is +0 or -0 before canonicalisation) and
    one random N(0,1) pattern per entry of `scales`, multiplied by that power
    of two (exact in bf16).  Every block copies one pattern (drawn at
    random), so blocks of one pattern have identical summaries and their
    scores tie exactly; selection among them is decided by index alone."""
    g = torch.Generator().manual_seed(seed)
    d = 128
    nb = (L + B - 1) // B
    gd = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((b, hkv * gqa, d), generator=gd, device="cuda").to(torch.bfloat16)
    K = torch.empty((b, hkv, L, d), dtype=torch.bfloat16, device="cuda")
    V = torch.randn((b, hkv, L, d), generator=gd, device="cuda").to(torch.bfloat16)
    for p in range(b * hkv):
        pats = torch.randn((len(scales), B, d), generator=g) * torch.tensor(scales)[:, None, None]
        pats = torch.cat([torch.zeros((1, B, d)), pats]).to(torch.bfloat16).cuda()
        cls = torch.randint(0, len(scales) + 1, (nb,), generator=g).cuda()
        K[p // hkv, p % hkv] = pats[cls].reshape(nb * B, d)[:L]
    return {"q": q, "K": K, "V": V}


TIES = [
    # name, batch, hkv, gqa, ctx, block, k, scales, check outputs
    ("ties-one-kernel-8w", 32, 8, 4, 4096, 16, 40, [1.0] * 5, True),
    ("ties-one-kernel-4w", 64, 8, 5, 2048, 32, 20, [1.0] * 4, True),
    ("ties-one-kernel-nb2048", 32, 8, 4, 32768, 16, 64, [1.0] * 6, True),
    ("ties-few-pairs", 2, 4, 8, 8192, 16, 100, [1.0] * 5, True),
    ("ties-few-pairs-nb8192", 1, 2, 4, 131072, 16, 300, [1.0] * 5, True),
    # the score tiles' own candidates (6250 blocks per pair, 25 tiles)
    ("ties-few-pairs-cand", 2, 4, 8, 100000, 16, 120, [1.0] * 5, True),
    # exponents far apart (scores spread over ~400 binades of both signs)
    ("wide-one-kernel-8w", 32, 8, 4, 4096, 16, 40, [2.0**-100, 2.0**-40, 1.0, 2.0**40, 2.0**100],
     False),
    ("wide-one-kernel-4w", 64, 8, 5, 2048, 32, 20, [2.0**-90, 1.0, 2.0**90], False),
    ("wide-few-pairs", 2, 4, 8, 8192, 16, 100, [2.0**-100, 2.0**-40, 1.0, 2.0**40, 2.0**100],
     False),
    ("wide-few-pairs-cand", 2, 4, 8, 100000, 16, 120,
     [2.0**-100, 2.0**-40, 1.0, 2.0**40, 2.0**100], False),
]


@pytest.mark.parametrize("case", TIES, ids=[c[0] for c in TIES])
def test_step_kernels_exact_ties_signed_zeros_and_wide_exponents(case):
    """kin_sparse_decode_step (with and without a scores buffer: one kernel
    when the pairs cover the chip, in both workgroup shapes, else the
    two-kernel form) on caches full of exactly tied blocks: the selection of
    every pair equals the oracle's selection on its own scores bit for bit
    (no margin certificate: the ties are the point), and tied blocks get
    bitwise equal scores."""
    name, b, hkv, gqa, L, B, k, scales, check_out = case
    say(f"case {name}")
    inp = _tied_cache(b, hkv, gqa, L, B, scales, zlib.crc32(name.encode()) % 10000)
    w = Workload(name, batch=b, hq=hkv * gqa, hkv=hkv, ctx_len=L, block=B, topk=k,
                 dtype="bf16", seed=0)
    nb = w.nb
    for no_scores in (False, True):
        bufs = run_gpu(w, inp, step=True, no_scores=no_scores)
        qc, Kc = inp["q"].cpu(), inp["K"].cpu()
        S_or, _ = oracle.block_summary(Kc, B, L)
        assert torch.equal(bits(bufs.S[:, :, :nb].cpu()), bits(S_or[:, :, :nb]))
        sc = oracle.block_score(qc, S_or, gqa, nb)
        idx_or, _ = oracle.block_topk(sc, nb, k)
        assert torch.equal(bufs.idx.cpu(), idx_or), f"{name}: selection differs"
        if not no_scores:
            sg = bufs.scores[:, :, :nb].cpu()
            # equal summaries -> bitwise equal scores (and -0 written as +0)
            assert not torch.any((sg == 0) & torch.signbit(sg))
            Sb = bits(S_or[:, :, :nb]).view(b * hkv, nb, 128)
            sgp = sg.view(b * hkv, nb)
            for p in range(0, b * hkv, max(1, b * hkv // 16)):
                _, inv = torch.unique(Sb[p], dim=0, return_inverse=True)
                for c in inv.unique().tolist():
                    vals = sgp[p][inv == c]
                    assert torch.equal(vals, vals[:1].expand_as(vals)), f"{name}: tied scores"
            scale = sc[:, :, :nb].abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
            assert ((sg - sc[:, :, :nb]).abs() / scale).max() < 1e-13
        if check_out:
            for s_ in sorted({0, b - 1}):
                o = oracle.decode_attention(qc[s_:s_ + 1], Kc[s_:s_ + 1],
                                            inp["V"][s_:s_ + 1].cpu(), gqa, L, B,
                                            idx=idx_or[s_:s_ + 1].contiguous())
                err = (bufs.out[s_:s_ + 1].cpu().double() - o).abs().max().item()
                assert err <= TOL["bf16"], f"{name}: output error {err} at seq {s_}"
    say(f"  ok")


F32_STEP = [
    # name, batch, hq, hkv, ctx, block, k, dtype, t_cap  (small per-pair bytes: one kernel)
    ("f32step-tiny-shape", 1, 8, 2, 4096, 16, 32, "f32", 4096),
    ("f32step-g1-b32-ragged", 3, 2, 2, 1000, 32, 5, "f32", 1024),
    ("f32step-g16-b64-k1", 2, 32, 2, 700, 64, 1, "f32", 704),
    ("f32step-g5-b16-kpast", 2, 10, 2, 100, 16, 9, "f32", 112),      # k > nb
    ("f32step-g8-b128-keepall", 1, 16, 2, 300, 128, 3, "f32", 384),  # k = nb, partial block
    ("f32step-g3-b16-one-block", 2, 6, 2, 7, 16, 2, "f32", 16),      # nb = 1
    ("f32step-g4-b16-nb1024", 1, 8, 2, 16384, 16, 8, "f32", 16384),  # KPT 2
]


@pytest.mark.parametrize("case", F32_STEP, ids=[c[0] for c in F32_STEP])
def test_f32_one_kernel_step_against_oracle(case):
    """kin_sparse_decode_step in fp32 with small per-pair bytes: one kernel
    per step (newest-row rebuild, scores, selection, attention); with and
    without a scores buffer, against the oracle on every sequence, and equal
    (selection, summaries, scores) to the separate calls."""
    name, b, hq, hkv, L, B, k, dt, cap = case
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    say(f"case {name}: {w.describe()}")
    inp = gpu_inputs(w)
    bufs = run_gpu(w, inp, step=True)
    assert bufs.ws is None or kb.kin_sparse_ws_bytes(bufs.desc, k) >= 0
    r = check_sequences(w, inp, bufs, range(b))
    sep = run_gpu(w, inp)
    assert torch.equal(sep.idx, bufs.idx)
    assert torch.equal(bits(sep.S[:, :, :w.nb]), bits(bufs.S[:, :, :w.nb]))
    assert torch.equal(sep.scores[:, :, :w.nb], bufs.scores[:, :, :w.nb])
    quiet = run_gpu(w, inp, step=True, no_scores=True)
    assert torch.equal(quiet.idx, bufs.idx)
    assert torch.equal(bits(quiet.out), bits(bufs.out))
    assert torch.isnan(quiet.scores).all()
    say(f"  ok {r}")
