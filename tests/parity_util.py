"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it, sequence by sequence, with the CPU oracle on the same bytes.

Agreement rules: summaries bit-exact, block indices bit-exact (after the
oracle's margin certificate shows the k-th and (k+1)-th scores of every pair
are apart by more than 1e-12 relative), outputs within max-abs 2e-2 (bf16)
or 1e-4 (fp32) of the oracle's unrounded fp64 result.
"""
import sys

import torch

import oracle
from block_top_sparse_amd import binding as kb
from block_top_sparse_amd import synth
from block_top_sparse_amd.buffers import LayerBuffers

TOL = {"bf16": 2e-2, "f32": 1e-4}
GAP_MIN = 1e-12


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def gpu_inputs(w, tail_fill=float("nan")):
    return synth.make_inputs(w, device="cuda", tail_fill=tail_fill)


def run_gpu(w, inp, k=None, dense=False, stream=None, prefill=True, bufs=None, fused=False,
            step=False, no_scores=False):
    """Prefill summaries, then scores -> top-k -> sparse attention (and dense).
    fused: the decode-step halves instead (newest-block update + scores in
    one launch, top-k + attention in the next); step: kin_sparse_decode_step
    (one kernel when there are at least as many pairs as CUs), with no scores
    buffer if no_scores."""
    bufs = bufs or LayerBuffers(w, k=k, with_dense=dense)
    d = bufs.desc
    bufs.out.fill_(float("nan"))  # every output must be written
    bufs.idx.fill_(-7)
    bufs.scores.fill_(float("nan"))
    if fused or step:
        # summaries of every block but the newest come from the prefill; the
        # newest is rebuilt by the step itself
        newest0 = (w.nb - 1) * w.block
        if prefill and newest0 > 0:
            kb.kin_block_summary_update(d, inp["K"], bufs.S, 0, newest0, stream=stream)
        if step:
            kb.kin_sparse_decode_step(d, inp["q"], inp["K"], inp["V"], bufs.S,
                                      None if no_scores else bufs.scores, bufs.k, bufs.idx,
                                      bufs.out, bufs.ws, stream=stream)
        else:
            kb.kin_decode_update_score(d, inp["q"], inp["K"], bufs.S, bufs.scores,
                                       stream=stream)
            kb.kin_decode_select_attend(d, inp["q"], inp["K"], inp["V"], bufs.scores, bufs.k,
                                        bufs.idx, bufs.out, bufs.ws, stream=stream)
    else:
        if prefill:
            kb.kin_block_summary_update(d, inp["K"], bufs.S, 0, w.ctx_len, stream=stream)
        kb.kin_block_score(d, inp["q"], bufs.S, bufs.scores, stream=stream)
        kb.kin_block_topk(d, bufs.scores, bufs.k, bufs.idx, stream=stream)
        kb.kin_sparse_decode_attn(d, inp["q"], inp["K"], inp["V"], bufs.idx, bufs.k, bufs.out,
                                  bufs.ws, stream=stream)
    if dense:
        bufs.out_dense.fill_(float("nan"))
        kb.kin_dense_decode_attn(d, inp["q"], inp["K"], inp["V"], bufs.out_dense, bufs.ws_dense,
                                 stream=stream)
    torch.cuda.synchronize()
    return bufs


def check_sequences(w, inp, bufs, seqs, check_out=True, check_dense=False, nthreads=None,
                    check_scores=True):
    """Compare sequences `seqs` of one GPU run with the oracle.  Returns the
    largest output error and the smallest margin seen.  check_scores=False
    for a run that wrote no scores."""
    nb, k = w.nb, bufs.k
    worst, min_gap, worst_dense = 0.0, float("inf"), 0.0
    for b in seqs:
        qb = inp["q"][b:b + 1].cpu()
        Kb = inp["K"][b:b + 1].cpu()
        S_or, _ = oracle.block_summary(Kb, w.block, w.ctx_len, nthreads=nthreads)
        S_gpu = bufs.S[b:b + 1, :, :nb].cpu()
        assert torch.equal(bits(S_gpu), bits(S_or[:, :, :nb])), f"summaries differ, seq {b}"
        sc_or = oracle.block_score(qb, S_or, w.gqa, nb, nthreads=nthreads)[:, :, :nb]
        if check_scores:
            sc_gpu = bufs.scores[b:b + 1, :, :nb].cpu()
            scale = sc_or.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
            assert ((sc_gpu - sc_or).abs() / scale).max() < 1e-13, f"scores differ, seq {b}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), nb, k, nthreads=nthreads)
        min_gap = min(min_gap, gap.min().item())
        assert (gap > GAP_MIN).all(), f"margin certificate fails at seq {b}: {gap.min().item()}"
        idx_gpu = bufs.idx[b:b + 1].cpu()
        assert torch.equal(idx_gpu, idx_or), f"selection differs, seq {b}"
        if check_out:
            Vb = inp["V"][b:b + 1].cpu()
            o = oracle.decode_attention(qb, Kb, Vb, w.gqa, w.ctx_len, w.block, idx=idx_or,
                                        nthreads=nthreads)
            og = bufs.out[b:b + 1].cpu().double()
            assert torch.isfinite(og).all(), f"unwritten or non-finite output, seq {b}"
            err = (og - o).abs().max().item()
            worst = max(worst, err)
            assert err <= TOL[w.dtype], f"sparse output error {err} at seq {b}"
            if check_dense:
                od = oracle.decode_attention(qb, Kb, Vb, w.gqa, w.ctx_len, w.block,
                                             nthreads=nthreads)
                ogd = bufs.out_dense[b:b + 1].cpu().double()
                assert torch.isfinite(ogd).all()
                errd = (ogd - od).abs().max().item()
                worst_dense = max(worst_dense, errd)
                assert errd <= TOL[w.dtype], f"dense output error {errd} at seq {b}"
    return {"max_err": worst, "max_err_dense": worst_dense, "min_gap": min_gap}
