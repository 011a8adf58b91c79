"""ctypes wrapper of the CPU oracle (oracle/kin_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg import this package.  The product path
never does, and the oracle shares no code with the HIP library.

All arrays are CPU torch tensors, contiguous, in the layouts documented in
kin_oracle.c.  bf16 tensors are passed as their raw 16-bit patterns; the
oracle reads every stored element as its exact value.  Results are fp64
(means, scores, attention outputs) or int32 (block indices).

Function -> step of the method (sources: the skill summary page "Kinetics:
Memory-Aware Test-Time Scaling", Implementation / BlockTopKAttention, and
the rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", answer Q4
"KV block size and grouping strategy"):
  block_summary     mean key of each KV block (the block representative)
  block_score       sum over a GQA group of q_h . mean key
  block_topk        the k best blocks, ties to the lower index, ascending
  decode_attention  exact softmax(q.k/sqrt(d)) . v over the kept tokens
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KIN_ORACLE_LIB: another build of the same source to load instead (the
# mutation test points it at copies with a planted mistake, which the pins
# must then catch)
_LIB_PATH = os.environ.get("KIN_ORACLE_LIB") or os.path.join(_HERE, "libkin_oracle.so")
_lib = None

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.kor_block_summary.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I]
        lib.kor_block_score.argtypes = [P, P, P, I, I, I, I, I, I, I, I]
        lib.kor_block_topk.argtypes = [P, P, P, I, I, I, I, I, I]
        lib.kor_decode_attention.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, I, I]
        lib.kor_round.argtypes = [P, P, ctypes.c_size_t, I]
        lib.kor_quest_summary.argtypes = [P, P, I, I, I, I, I, I, I, I, I, I]
        lib.kor_quest_score.argtypes = [P, P, P, I, I, I, I, I, I, I, I]
        for f in ("kor_block_summary", "kor_block_score", "kor_block_topk",
                  "kor_decode_attention", "kor_round", "kor_version", "kor_quest_summary",
                  "kor_quest_score"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(t):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous(), "oracle takes contiguous CPU tensors"
    return ctypes.c_void_p(t.data_ptr())


def _dt(t):
    return _DTYPES[t.dtype]


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def nblocks(length: int, block: int) -> int:
    return (length + block - 1) // block


def block_summary(K, block, ctx_len, t_begin=0, t_end=None, S=None, want_f64=False, nthreads=None):
    """Mean key of every block meeting [t_begin, t_end) and [0, ctx_len).

    K: [batch][hkv][t_cap][d] (fp32 or bf16).  Returns (S, S64): S in K's
    dtype, shape [batch][hkv][nb_cap][d] (blocks outside the range keep the
    values of the S passed in, zeros otherwise); S64 the unrounded fp64 means
    when want_f64, else None."""
    b, hkv, t_cap, d = K.shape
    nb_cap = nblocks(t_cap, block)
    if t_end is None:
        t_end = ctx_len
    if S is None:
        S = torch.zeros((b, hkv, nb_cap, d), dtype=K.dtype)
    S64 = torch.zeros((b, hkv, nb_cap, d), dtype=torch.float64) if want_f64 else None
    rc = _load().kor_block_summary(_ptr(K), _ptr(S), _ptr(S64), _dt(K), b, hkv, t_cap, d,
                                   ctx_len, block, t_begin, t_end,
                                   nthreads or default_threads())
    _check(rc, "block_summary")
    return S, S64


def block_score(q, S, gqa, nb, nthreads=None):
    """scores[b][g][j] (fp64, [batch][hkv][nb_cap]) for j < nb; the rest 0."""
    b, hq, d = q.shape
    _, hkv, nb_cap, _ = S.shape
    assert hq == hkv * gqa and q.dtype == S.dtype
    scores = torch.zeros((b, hkv, nb_cap), dtype=torch.float64)
    rc = _load().kor_block_score(_ptr(q), _ptr(S), _ptr(scores), _dt(q), b, hkv, gqa, d,
                                 nb_cap, nb, nthreads or default_threads())
    _check(rc, "block_score")
    return scores


def quest_summary(K, block, ctx_len, t_begin=0, t_end=None, Sq=None, nthreads=None):
    """Quest-style summaries (reading R9 of kin_oracle.c): channel-wise minimum
    and maximum of the keys of every block meeting [t_begin, t_end) and
    [0, ctx_len).  Returns Sq [batch][hkv][nb_cap][2][d] in K's dtype (row 0
    minimum, row 1 maximum); blocks outside the range keep Sq's values
    (zeros when Sq is None)."""
    b, hkv, t_cap, d = K.shape
    nb_cap = nblocks(t_cap, block)
    if t_end is None:
        t_end = ctx_len
    if Sq is None:
        Sq = torch.zeros((b, hkv, nb_cap, 2, d), dtype=K.dtype)
    rc = _load().kor_quest_summary(_ptr(K), _ptr(Sq), _dt(K), b, hkv, t_cap, d, ctx_len, block,
                                   t_begin, t_end, nthreads or default_threads())
    _check(rc, "quest_summary")
    return Sq


def quest_score(q, Sq, gqa, nb, nthreads=None):
    """Quest bound of every block (fp64, [batch][hkv][nb_cap]) for j < nb:
    sum over the group's heads and channels of max(q*min, q*max)."""
    b, hq, d = q.shape
    _, hkv, nb_cap, two, _ = Sq.shape
    assert two == 2 and hq == hkv * gqa and q.dtype == Sq.dtype
    scores = torch.zeros((b, hkv, nb_cap), dtype=torch.float64)
    rc = _load().kor_quest_score(_ptr(q), _ptr(Sq), _ptr(scores), _dt(q), b, hkv, gqa, d, nb_cap,
                                 nb, nthreads or default_threads())
    _check(rc, "quest_score")
    return scores


def block_topk(scores, nb, k, nthreads=None):
    """(idx int32 [batch][hkv][k], gap fp64 [batch][hkv])."""
    b, hkv, nb_cap = scores.shape
    assert scores.dtype == torch.float64
    idx = torch.empty((b, hkv, k), dtype=torch.int32)
    gap = torch.empty((b, hkv), dtype=torch.float64)
    rc = _load().kor_block_topk(_ptr(scores), _ptr(idx), _ptr(gap), b, hkv, nb_cap, nb, k,
                                nthreads or default_threads())
    _check(rc, "block_topk")
    return idx, gap


def decode_attention(q, K, V, gqa, ctx_len, block, idx=None, nthreads=None):
    """fp64 [batch][hq][d]: softmax attention over the kept blocks (dense if idx is None)."""
    b, hq, d = q.shape
    _, hkv, t_cap, _ = K.shape
    assert hq == hkv * gqa and K.dtype == q.dtype == V.dtype and V.shape == K.shape
    k = 0
    if idx is not None:
        assert idx.dtype == torch.int32 and idx.shape[:2] == (b, hkv)
        k = idx.shape[2]
    out = torch.zeros((b, hq, d), dtype=torch.float64)
    rc = _load().kor_decode_attention(_ptr(q), _ptr(K), _ptr(V), _ptr(idx), k, _ptr(out), _dt(q),
                                      b, hkv, gqa, d, t_cap, ctx_len, block,
                                      nthreads or default_threads())
    _check(rc, "decode_attention")
    return out


def round_to(x64, dtype):
    """fp64 tensor -> dtype with the oracle's rounding (fp64->fp32 RNE, then ->bf16 RNE)."""
    x64 = x64.contiguous()
    out = torch.empty(x64.shape, dtype=dtype)
    _check(_load().kor_round(_ptr(x64), _ptr(out), x64.numel(), _DTYPES[dtype]), "round")
    return out


def sparse_decode(q, K, V, gqa, ctx_len, block, k, nthreads=None):
    """Whole method from the cache: summaries -> scores -> selection -> attention.

    Returns a dict with S, scores, idx, gap and out (fp64)."""
    nb = nblocks(ctx_len, block)
    S, _ = block_summary(K, block, ctx_len, nthreads=nthreads)
    scores = block_score(q, S, gqa, nb, nthreads=nthreads)
    idx, gap = block_topk(scores, nb, k, nthreads=nthreads)
    out = decode_attention(q, K, V, gqa, ctx_len, block, idx=idx, nthreads=nthreads)
    return {"S": S, "scores": scores, "idx": idx, "gap": gap, "out": out}
