"""GPU parity of the variable-length and paged-cache calls against the oracle.

Each sequence of a batch holds its own number of tokens; the K/V caches are
either contiguous [batch][hkv][t_cap][d] or scattered over a page pool
[num_pages][hkv][page_size][d] in a shuffled page order.  The oracle runs
per sequence on that sequence's contiguous cache and its own length, so the
paged addressing is checked against plain indexing.  Unused pages and every
cache slot past a sequence's length hold NaN: a read of any of them that
reaches a result shows up.
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


def draw_lens(name, batch, max_len, block, page_size, kind):
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    if kind == "edge":
        base = [1, block - 1, block, block + 1, 2 * block - 1, page_size, page_size + 1,
                max_len - 1, max_len, max_len // 2 + 3]
        lens = [min(max(x, 1), max_len) for x in base]
        while len(lens) < batch:
            lens.append(int(torch.randint(1, max_len + 1, (1,), generator=g)))
        return lens[:batch]
    lens = torch.randint(max(1, max_len // 8), max_len + 1, (batch,), generator=g).tolist()
    lens[0] = max_len  # the bound is reached by one sequence
    return lens


class Case:
    """Inputs of one variable-length batch: contiguous caches with NaN past
    each sequence's length, the same tokens scattered over a page pool, and
    the device buffers of the calls."""

    def __init__(self, name, batch, hkv, gqa, block, page_size, max_len, k, kind, seed=None,
                 lens=None, unused_entry="spare"):
        self.name, self.block, self.page_size, self.k = name, block, page_size, k
        self.lens = lens or draw_lens(name, batch, max_len, block, page_size, kind)
        max_pages = (max_len + page_size - 1) // page_size
        cap = max_pages * page_size
        seed = zlib.crc32(name.encode()) % 10000 if seed is None else seed
        self.w = Workload(name, batch=batch, hq=hkv * gqa, hkv=hkv, ctx_len=max_len, block=block,
                          topk=k, dtype="bf16", seed=seed, t_cap=cap)
        w = self.w
        inp = synth.make_inputs(w, device="cuda", tail_fill=NAN)
        for b, L in enumerate(self.lens):
            inp["K"][b, :, L:] = NAN
            inp["V"][b, :, L:] = NAN
        self.q, self.K, self.V = inp["q"], inp["K"], inp["V"]
        # page pool: every sequence's pages in one shuffled order, spare NaN pages
        used = [(L + page_size - 1) // page_size for L in self.lens]
        spare = 3
        num_pages = sum(used) + spare
        gen = torch.Generator().manual_seed(seed + 1)
        perm = torch.randperm(num_pages, generator=gen).tolist()
        spare_pages = perm[sum(used):]
        table = torch.empty((batch, max_pages), dtype=torch.int32)
        Kp = torch.full((num_pages, hkv, page_size, 128), NAN, dtype=torch.bfloat16, device="cuda")
        Vp = torch.full_like(Kp, NAN)
        nxt = 0
        for b in range(batch):
            for p in range(max_pages):
                if p < used[b]:
                    pg = perm[nxt]
                    nxt += 1
                    sl = slice(p * page_size, (p + 1) * page_size)
                    Kp[pg] = self.K[b, :, sl]
                    Vp[pg] = self.V[b, :, sl]
                else:
                    # never holds a token of the sequence
                    pg = spare_pages[p % spare] if unused_entry == "spare" else 1 << 30
                table[b, p] = pg
        self.Kp, self.Vp = Kp, Vp
        self.table = table.cuda()
        self.lens_t = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.num_pages, self.max_pages = num_pages, max_pages
        self.desc = kb.make_desc(batch, hkv, gqa, cap, max_len, block, torch.bfloat16)
        nb_cap = cap // block
        self.S = torch.empty((batch, hkv, nb_cap, 128), dtype=torch.bfloat16, device="cuda")
        self.scores = torch.empty((batch, hkv, nb_cap), dtype=torch.float64, device="cuda")
        self.idx = torch.empty((batch, hkv, k), dtype=torch.int32, device="cuda")
        self.out = torch.empty((batch, hkv * gqa, 128), dtype=torch.bfloat16, device="cuda")
        n = kb.kin_sparse_ws_bytes(self.desc, k)
        self.ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")

    def pages(self, paged=True, varlen=True):
        return kb.make_pages(self.lens_t if varlen else None, self.table if paged else None,
                             self.page_size, self.max_pages, self.num_pages)

    def nb(self, b):
        return oracle.nblocks(self.lens[b], self.block)

    def run(self, paged=True, varlen=True, no_scores=False, prefill_split=None):
        """Prefill the summaries, spoil each sequence's newest row (the step
        must rebuild it), then one decode step.  Returns copies of
        (S, scores, idx, out)."""
        pg = self.pages(paged, varlen)
        K, V = (self.Kp, self.Vp) if paged else (self.K, self.V)
        self.S.fill_(NAN)
        self.scores.fill_(NAN)
        self.idx.fill_(-7)
        self.out.fill_(NAN)
        T = self.w.ctx_len
        cuts = [0] + ([prefill_split] if prefill_split else []) + [T]
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            kb.kin_paged_summary_update(self.desc, pg, K, self.S, t0, t1)
        for b in range(self.w.batch):
            self.S[b, :, self.nb(b) - 1] = 3.0 if b % 2 else NAN
        kb.kin_paged_decode_step(self.desc, pg, self.q, K, V, self.S,
                                 None if no_scores else self.scores, self.k, self.idx, self.out,
                                 self.ws)
        torch.cuda.synchronize()
        return self.S.clone(), self.scores.clone(), self.idx.clone(), self.out.clone()


def check_against_oracle(c, S, scores, idx, out, check_scores=True):
    w, k = c.w, c.k
    worst = 0.0
    for b, L in enumerate(c.lens):
        nb = c.nb(b)
        qb, Kb, Vb = c.q[b:b + 1].cpu(), c.K[b:b + 1].cpu(), c.V[b:b + 1].cpu()
        S_or, _ = oracle.block_summary(Kb, c.block, L)
        assert torch.equal(bits(S[b:b + 1, :, :nb].cpu()), bits(S_or[:, :, :nb])), \
            f"{c.name}: summaries differ, seq {b} (len {L})"
        sc_or = oracle.block_score(qb, S_or, w.gqa, nb)
        if check_scores:
            sc = scores[b:b + 1, :, :nb].cpu()
            ref = sc_or[:, :, :nb]
            scale = ref.abs().amax(dim=2, keepdim=True).clamp_min(1e-300)
            assert ((sc - ref).abs() / scale).max() < 1e-13, f"{c.name}: scores differ, seq {b}"
        idx_or, gap = oracle.block_topk(sc_or.contiguous(), nb, k)
        assert (gap > GAP_MIN).all(), f"{c.name}: margin certificate fails, seq {b}"
        assert torch.equal(idx[b:b + 1].cpu(), idx_or), f"{c.name}: selection differs, seq {b}"
        o = oracle.decode_attention(qb, Kb, Vb, w.gqa, L, c.block, idx=idx_or)
        og = out[b:b + 1].cpu().double()
        assert torch.isfinite(og).all(), f"{c.name}: unwritten or non-finite output, seq {b}"
        err = (og - o).abs().max().item()
        assert err <= TOL["bf16"], f"{c.name}: output error {err}, seq {b} (len {L})"
        worst = max(worst, err)
    return worst


def assert_same(r1, r2, c, what):
    S1, sc1, i1, o1 = r1
    S2, sc2, i2, o2 = r2
    for b in range(c.w.batch):
        nb = c.nb(b)
        assert torch.equal(bits(S1[b, :, :nb]), bits(S2[b, :, :nb])), f"{what}: S, seq {b}"
        assert torch.equal(sc1[b, :, :nb].view(torch.int64), sc2[b, :, :nb].view(torch.int64)), \
            f"{what}: scores, seq {b}"
    assert torch.equal(i1, i2), f"{what}: idx"
    assert torch.equal(bits(o1), bits(o2)), f"{what}: out"


PAGED = [
    # name, batch, hkv, gqa, block, page_size, max_len, k, lens
    ("few-g4-b16-p64", 3, 2, 4, 16, 64, 3000, 32, "rand"),
    ("edge-g2-b16-p16", 12, 2, 2, 16, 16, 1000, 8, "edge"),
    ("few-g8-b64-p128-k1", 2, 2, 8, 64, 128, 5000, 1, "rand"),
    ("few-g5-b32-p256-kpast", 4, 2, 5, 32, 256, 2000, 40, "rand"),
    ("few-g4-b16-p64-keepall", 3, 2, 4, 16, 64, 600, 40, "rand"),  # every block kept
    ("few-g16-b128-p128", 2, 2, 16, 128, 128, 3000, 5, "edge"),
    ("many-g4-b16-p256", 40, 8, 4, 16, 256, 4096, 64, "rand"),    # 320 pairs: one kernel
    ("many-g8-b32-p64", 36, 8, 8, 32, 64, 3000, 16, "edge"),       # 288 pairs: one kernel
    ("many4w-g2-b32-p64", 64, 8, 2, 32, 64, 1500, 16, "edge"),     # 512 pairs: 4-wave step
]


def check_paged_case(case):
    """One paged, variable-length step against the oracle, then the same
    tokens in contiguous caches (bit for bit) and without a scores buffer."""
    name, batch, hkv, gqa, block, ps, L, k, kind = case
    c = Case(name, batch, hkv, gqa, block, ps, L, k, kind)
    say(f"case {name}: pairs {batch * hkv}, lens {c.lens[:12]}")
    r_paged = c.run(paged=True)
    err = check_against_oracle(c, *r_paged)
    # same tokens, contiguous caches: bit for bit the same results
    r_contig = c.run(paged=False)
    assert_same(r_paged, r_contig, c, "paged vs contiguous")
    # no scores buffer (every block kept: one kernel, which also rebuilds the newest rows)
    r_ns = c.run(paged=True, no_scores=True)
    assert torch.equal(r_ns[2], r_paged[2]) and torch.equal(bits(r_ns[3]), bits(r_paged[3]))
    for b in range(c.w.batch):
        assert torch.equal(bits(r_ns[0][b, :, :c.nb(b)]), bits(r_paged[0][b, :, :c.nb(b)])), \
            f"no scores: S, seq {b}"
    say(f"case {name}: max err {err:.3e}")


@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_paged_step_against_oracle(case):
    check_paged_case(case)


def test_paged_table_entries_past_the_length_are_not_used():
    """Entries of the page table past a sequence's pages may hold anything
    (here far outside the pool): results do not change."""
    args = ("few-g4-b16-p64", 3, 2, 4, 16, 64, 3000, 32, "rand")
    a = Case(*args)
    b = Case(*args, unused_entry="far")
    assert_same(a.run(paged=True), b.run(paged=True), a, "unused page-table entries")


def test_paged_summary_update_in_pieces():
    """Summaries built in two calls split inside a block equal the oracle's."""
    c = Case("sum-g2-b32-p64", 6, 2, 2, 32, 64, 2000, 8, "edge")
    pg = c.pages()
    c.S.fill_(NAN)
    kb.kin_paged_summary_update(c.desc, pg, c.Kp, c.S, 0, 777)
    kb.kin_paged_summary_update(c.desc, pg, c.Kp, c.S, 777, 2000)
    torch.cuda.synchronize()
    for b, L in enumerate(c.lens):
        nb = c.nb(b)
        S_or, _ = oracle.block_summary(c.K[b:b + 1].cpu(), c.block, L)
        assert torch.equal(bits(c.S[b:b + 1, :, :nb].cpu()), bits(S_or[:, :, :nb])), f"seq {b}"
        assert torch.isnan(c.S[b, :, nb:].float()).all(), f"rows past seq {b} were written"


def test_equal_lengths_match_the_contiguous_step():
    """No lengths and no page table: the same bits as kin_sparse_decode_step."""
    for name, batch, hkv in (("eq-few", 3, 2), ("eq-many", 40, 8)):
        c = Case(name, batch, hkv, 4, 16, 64, 2000, 16, "rand", lens=[2000] * batch)
        r1 = c.run(paged=False, varlen=False)
        S2 = torch.full_like(c.S, NAN)
        kb.kin_block_summary_update(c.desc, c.K, S2, 0, 2000)
        S2[:, :, c.nb(0) - 1] = NAN
        sc2 = torch.full_like(c.scores, NAN)
        idx2 = torch.full_like(c.idx, -7)
        out2 = torch.full_like(c.out, NAN)
        kb.kin_sparse_decode_step(c.desc, c.q, c.K, c.V, S2, sc2, c.k, idx2, out2, c.ws)
        torch.cuda.synchronize()
        assert_same(r1, (S2, sc2, idx2, out2), c, name)
        check_against_oracle(c, *r1)
