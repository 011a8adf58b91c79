"""GPU parity of the shared-prompt Best-of-N step against the oracle.

Each group of n_share samples shares a prompt whose K/V and block summaries
are stored once; every sample's own cache holds NaN where the prompt would
be, so a read of it shows.  The oracle runs per sample on the sample's full
contiguous cache (its prompt followed by its own tokens), and the same
caches laid out contiguously must give kin_sparse_decode_step's bits.
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


SHARED = [
    # name, prompts, n_share, hkv, gqa, block, prompt_len, ctx_len, k
    ("shr-1k-g4-b16", 4, 8, 8, 4, 16, 1024, 4000, 40),       # 256 pairs: one kernel, XCD order
    ("shr-4w-g2-b32", 8, 8, 8, 2, 32, 2048, 5000, 24),       # 512 pairs: the 4-wave step
    ("shr-few-g8-b64", 2, 2, 2, 8, 64, 512, 3000, 10),       # 8 pairs: two kernels
    ("shr-odd-g3-b16", 3, 16, 6, 3, 16, 256, 2000, 30),      # 18 units: launch order unchanged
    ("shr-few-keepall", 2, 3, 2, 4, 16, 160, 300, 40),       # k > nb
]


def build(case):
    name, n_prompts, n_share, hkv, gqa, B, P, L, k = case
    seed = zlib.crc32(name.encode()) % 10000
    batch = n_prompts * n_share
    cap = (L + 63) // 64 * 64
    w = Workload(name, batch=batch, hq=hkv * gqa, hkv=hkv, ctx_len=L, block=B, topk=k,
                 dtype="bf16", seed=seed, t_cap=cap)
    wp = Workload(name + "-prompt", batch=n_prompts, hq=hkv * gqa, hkv=hkv, ctx_len=P, block=B,
                  topk=1, dtype="bf16", seed=seed + 1)
    own = synth.make_inputs(w, device="cuda", tail_fill=NAN)
    pr = synth.make_inputs(wp, device="cuda")
    Kp, Vp = pr["K"], pr["V"]
    grp = torch.arange(batch, device="cuda") // n_share
    Kfull, Vfull = own["K"].clone(), own["V"].clone()
    Kfull[:, :, :P] = Kp[grp]
    Vfull[:, :, :P] = Vp[grp]
    K, V = own["K"], own["V"]
    K[:, :, :P] = NAN  # the samples' own arrays hold nothing of the prompt
    V[:, :, :P] = NAN
    desc = kb.make_desc(batch, hkv, gqa, cap, L, B, torch.bfloat16)
    desc_p = kb.make_desc(n_prompts, hkv, gqa, P, P, B, torch.bfloat16)
    Sp = torch.empty((n_prompts, hkv, P // B, 128), dtype=torch.bfloat16, device="cuda")
    kb.kin_block_summary_update(desc_p, Kp, Sp, 0, P)
    return dict(w=w, q=own["q"], K=K, V=V, Kfull=Kfull, Vfull=Vfull, Kp=Kp, Vp=Vp, Sp=Sp,
                desc=desc, n_share=n_share, P=P, k=k)


def run(c, shared=True, with_scores=True):
    w, k = c["w"], c["k"]
    nb_cap = w.nb_cap
    S = torch.full((w.batch, w.hkv, nb_cap, 128), NAN, dtype=torch.bfloat16, device="cuda")
    K = c["K"] if shared else c["Kfull"]
    V = c["V"] if shared else c["Vfull"]
    # summaries of each sample's own blocks (all blocks for the contiguous run)
    kb.kin_block_summary_update(c["desc"], K, S, c["P"] if shared else 0, w.ctx_len)
    S[:, :, w.nb - 1] = 3.0  # stale newest row: the step rebuilds it
    scores = torch.full((w.batch, w.hkv, nb_cap), NAN, dtype=torch.float64, device="cuda")
    idx = torch.full((w.batch, w.hkv, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.hq, 128), NAN, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(kb.kin_sparse_ws_bytes(c["desc"], k), 16), dtype=torch.uint8,
                     device="cuda")
    if shared:
        share = kb.make_share(c["n_share"], c["P"], c["Kp"], c["Vp"], c["Sp"])
        kb.kin_shared_decode_step(c["desc"], share, c["q"], K, V, S,
                                  scores if with_scores else None, k, idx, out, ws)
    else:
        kb.kin_sparse_decode_step(c["desc"], c["q"], K, V, S, scores, k, idx, out, ws)
    torch.cuda.synchronize()
    return S, scores, idx, out


def check_shared_case(case):
    """One shared-prompt step against the oracle on each sample's full
    cache, then the same tokens in contiguous caches (bit for bit) and
    without a scores buffer."""
    c = build(case)
    w, k, P = c["w"], c["k"], c["P"]
    say(f"case {w.name}: pairs {w.pairs}, prompt {P} of {w.ctx_len}")
    S, scores, idx, out = run(c)
    nb, pb = w.nb, P // w.block
    seqs = sorted({0, 1, w.batch // 2, w.batch - 1})
    worst = 0.0
    for b in seqs:
        qb, Kb, Vb = c["q"][b:b + 1].cpu(), c["Kfull"][b:b + 1].cpu(), c["Vfull"][b:b + 1].cpu()
        S_or, _ = oracle.block_summary(Kb, w.block, w.ctx_len)
        g = b // c["n_share"]
        assert torch.equal(bits(c["Sp"][g].cpu()), bits(S_or[0, :, :pb])), f"prompt rows, seq {b}"
        assert torch.equal(bits(S[b, :, pb:nb].cpu()), bits(S_or[0, :, pb:nb])), f"own rows {b}"
        sc_or = oracle.block_score(qb, S_or, w.gqa, nb)
        ref = sc_or[:, :, :nb]
        scale = ref.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
        assert ((scores[b:b + 1, :, :nb].cpu() - ref).abs() / scale).max() < 1e-13
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), nb, k)
        assert (gap > GAP_MIN).all(), f"margin certificate fails, seq {b}"
        assert torch.equal(idx[b:b + 1].cpu(), idx_or), f"selection differs, seq {b}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, w.ctx_len, w.block, idx=idx_or)
        og = out[b:b + 1].cpu().double()
        assert torch.isfinite(og).all(), f"unwritten output, seq {b}"
        err = (og - o).abs().max().item()
        assert err <= TOL["bf16"], f"output error {err}, seq {b}"
        worst = max(worst, err)
    # the same tokens in contiguous caches: bit for bit the same step
    S2, sc2, idx2, out2 = run(c, shared=False)
    assert torch.equal(idx2, idx)
    assert torch.equal(bits(out2), bits(out))
    assert torch.equal(bits(S2[:, :, pb:nb]), bits(S[:, :, pb:nb]))
    assert torch.equal(sc2[:, :, :nb].view(torch.int64), scores[:, :, :nb].view(torch.int64))
    # no scores buffer: the same selection, output and rebuilt rows
    S3, _, idx3, out3 = run(c, with_scores=False)
    assert torch.equal(idx3, idx)
    assert torch.equal(bits(out3), bits(out))
    assert torch.equal(bits(S3[:, :, pb:nb]), bits(S[:, :, pb:nb]))
    say(f"  ok, max err {worst:.3e}")


@pytest.mark.parametrize("case", SHARED, ids=[c[0] for c in SHARED])
def test_shared_prompt_step_against_oracle(case):
    check_shared_case(case)
