"""Host-side checks of libkin.so that need no GPU.

The library loads, exports every entry point include/kin.h declares, and
rejects bad arguments on the host with the documented status before
anything is enqueued (each case here fails validation, so no HIP call is
made).
"""
import ctypes
import os
import re

import pytest

from block_top_sparse_amd import binding as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kin.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kb.LIB_PATH), reason="libkin.so not built")

FAKE = 0x100000  # an aligned, never dereferenced address: validation fails first
MISALIGNED = 0x100008


def header_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KIN_API\s+[\w\s\*]+?\b(kin_\w+)\s*\(", text)))


def test_every_declared_entry_point_is_exported():
    declared = header_entry_points()
    assert len(declared) == 23, declared
    lib = ctypes.CDLL(kb.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(kb.exported_names()) == declared


def test_version_and_status_strings():
    assert kb.kin_version() == 1
    for code, name in [(0, "KIN_OK"), (-1, "KIN_ERR_NULL"), (-2, "KIN_ERR_SHAPE"),
                       (-5, "KIN_ERR_UNSUPPORTED"), (-6, "KIN_ERR_WORKSPACE"), (-7, "KIN_ERR_HIP")]:
        assert kb.kin_status_str(code) == name


def _desc(**kw):
    base = dict(batch=2, hkv=2, gqa=4, t_cap=256, ctx_len=200, block=16, dtype=kb.KIN_BF16)
    base.update(kw)
    return kb.make_desc(**base)


def _raw(name, *args):
    return getattr(kb.lib(), name)(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(batch=0), -2),
    (dict(gqa=0), -2),
    (dict(ctx_len=0), -2),
    (dict(ctx_len=300), -2),          # beyond t_cap
    (dict(head_dim=64), -5),
    (dict(block=24), -5),
    (dict(block=8), -5),
    (dict(gqa=17), -5),
])
def test_bad_descriptor_is_rejected(kw, code):
    d = _desc(**kw)
    rc = _raw("kin_block_score", ctypes.byref(d), FAKE, FAKE, FAKE, None)
    assert rc == code, kb.kin_last_error()
    assert kb.kin_last_error()


def test_null_and_misaligned_pointers_are_rejected():
    d = _desc()
    assert _raw("kin_block_score", None, FAKE, FAKE, FAKE, None) == -1
    assert _raw("kin_block_score", ctypes.byref(d), None, FAKE, FAKE, None) == -1
    assert "q is NULL" in kb.kin_last_error()
    assert _raw("kin_block_score", ctypes.byref(d), FAKE, MISALIGNED, FAKE, None) == -4
    assert _raw("kin_block_topk", ctypes.byref(d), FAKE, 4, None, None) == -1
    assert _raw("kin_sparse_decode_attn", ctypes.byref(d), FAKE, FAKE, FAKE, None, 4, FAKE,
                None, 0, None) == -1
    assert _raw("kin_dense_decode_attn", ctypes.byref(d), FAKE, FAKE, None, FAKE, None, 0,
                None) == -1


def test_bad_ranges_and_k_are_rejected():
    d = _desc()
    assert _raw("kin_block_summary_update", ctypes.byref(d), FAKE, FAKE, -1, 5, None) == -2
    assert _raw("kin_block_summary_update", ctypes.byref(d), FAKE, FAKE, 10, 5, None) == -2
    assert _raw("kin_block_summary_update", ctypes.byref(d), FAKE, FAKE, 0, 257, None) == -2
    assert _raw("kin_block_topk", ctypes.byref(d), FAKE, 0, FAKE, None) == -2
    assert _raw("kin_sparse_decode_attn", ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                None, 0, None) == -2
    assert _raw("kin_sparse_decode_step", ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                FAKE, FAKE, None, 0, None) == -2
    big = _desc(t_cap=16 * 20000, ctx_len=16 * 20000)
    assert _raw("kin_block_topk", ctypes.byref(big), FAKE, 4, FAKE, None) == -5


def test_paged_calls_validate_on_the_host():
    """kin_pages rules (include/kin.h): bf16 only, page_size a power of two
    >= 16 and a multiple of block, t_cap = max_pages * page_size, k <= 2048."""
    bf = _desc(dtype=1)  # t_cap 256, block 16
    ok = kb.kin_pages(None, FAKE, 64, 4, 8)
    step = lambda d, p, k=4: _raw("kin_paged_decode_step", ctypes.byref(d), p, FAKE, FAKE,  # noqa
                                  FAKE, FAKE, FAKE, k, FAKE, FAKE, None, 0, None)
    assert step(bf, None) == -1
    assert step(_desc(dtype=0), ctypes.byref(ok)) == -5          # fp32
    for bad in (kb.kin_pages(None, FAKE, 48, 4, 8),              # not a power of two
                kb.kin_pages(None, FAKE, 8, 32, 8),              # below 16
                kb.kin_pages(None, FAKE, 64, 3, 8),              # t_cap != 3 * 64
                kb.kin_pages(None, FAKE, 64, 4, 0)):             # empty pool
        assert step(bf, ctypes.byref(bad)) == -2, bad
    big_block = _desc(dtype=1, block=128)
    assert step(big_block, ctypes.byref(kb.kin_pages(None, FAKE, 64, 4, 8))) == -2  # 64 % 128
    assert step(bf, ctypes.byref(kb.kin_pages(MISALIGNED + 2, None, 0, 0, 0))) == -4
    assert step(bf, ctypes.byref(ok), k=4096) == -5
    assert step(bf, ctypes.byref(ok), k=0) == -2
    assert _raw("kin_paged_summary_update", ctypes.byref(bf), ctypes.byref(ok), FAKE, FAKE, 0,
                300, None) == -2


def test_shared_prompt_step_validates_on_the_host():
    """kin_shared_prompt rules (include/kin.h): bf16, n_share divides batch,
    prompt_len a multiple of block, >= one block, < ctx_len; k <= 2048."""
    bf = _desc(dtype=1)  # batch 2, ctx 200, block 16
    ok = kb.kin_shared_prompt(2, 64, FAKE, FAKE, FAKE)
    step = lambda d, sh, k=4: _raw("kin_shared_decode_step", ctypes.byref(d), sh, FAKE,  # noqa
                                   FAKE, FAKE, FAKE, None, k, FAKE, FAKE, None, 0, None)
    assert step(bf, None) == -1
    assert step(_desc(dtype=0), ctypes.byref(ok)) == -5
    for bad in (kb.kin_shared_prompt(3, 64, FAKE, FAKE, FAKE),    # 3 does not divide 2
                kb.kin_shared_prompt(0, 64, FAKE, FAKE, FAKE),
                kb.kin_shared_prompt(2, 40, FAKE, FAKE, FAKE),    # not a multiple of 16
                kb.kin_shared_prompt(2, 0, FAKE, FAKE, FAKE),
                kb.kin_shared_prompt(2, 208, FAKE, FAKE, FAKE)):  # not below ctx_len
        assert step(bf, ctypes.byref(bad)) == -2
    assert step(bf, ctypes.byref(ok), k=4096) == -5
    assert step(bf, ctypes.byref(kb.kin_shared_prompt(2, 64, None, FAKE, FAKE))) == -1
    assert step(bf, ctypes.byref(kb.kin_shared_prompt(2, 64, FAKE, MISALIGNED, FAKE))) == -4


def test_quest_calls_validate_on_the_host():
    """Quest calls (include/kin.h): bf16 only, k in 1..2048, a workspace."""
    bf = _desc(dtype=1)
    step = lambda d, k=4, Sq=FAKE: _raw("kin_quest_decode_step", ctypes.byref(d), FAKE, FAKE,  # noqa
                                        FAKE, Sq, None, k, FAKE, FAKE, None, 0, None)
    assert step(_desc(dtype=0)) == -5
    assert step(bf, Sq=None) == -1
    assert step(bf, k=0) == -2
    assert step(bf, k=4096) == -5
    assert step(bf) == -1  # no workspace (the scores live there)
    assert kb.kin_quest_ws_bytes(bf, 4) >= 2 * 2 * 16 * 8
    assert _raw("kin_quest_summary_update", ctypes.byref(_desc(dtype=0)), FAKE, FAKE, 0, 16,
                None) == -5
    assert _raw("kin_quest_summary_update", ctypes.byref(bf), FAKE, FAKE, 0, 300, None) == -2


def test_token_calls_validate_on_the_host():
    """Token-level step (include/kin.h): block must be 1, bf16 only,
    1 <= k <= 8192, ctx_len <= 262144."""
    tok = _desc(block=1)
    step = lambda d, k=4, q=FAKE: _raw("kin_token_decode_step", ctypes.byref(d), q, FAKE,  # noqa
                                       FAKE, None, k, FAKE, FAKE, None, 0, None)
    assert step(_desc(block=16)) == -2
    assert step(_desc(block=1, dtype=0)) == -5
    assert step(tok, k=0) == -2
    assert step(tok, k=8193) == -5
    assert step(_desc(block=1, t_cap=300000, ctx_len=262145)) == -5
    assert step(tok, q=None) == -1
    assert step(tok, q=MISALIGNED) == -4
    assert step(tok) == -1  # no workspace
    n = kb.kin_token_ws_bytes(tok, 64)
    assert n >= 2 * 2 * 256 * 8  # the scores at least
    with pytest.raises(kb.KinError):
        kb.kin_token_ws_bytes(_desc(block=2), 64)


def test_workspace_query_rejects_bad_descriptor():
    with pytest.raises(kb.KinError):
        kb.kin_sparse_ws_bytes(_desc(gqa=0), 4)
    with pytest.raises(kb.KinError):
        kb.kin_dense_ws_bytes(_desc(dtype=9))


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kb, "_lib", None)
    with pytest.raises(ImportError):
        kb.kin_version()


def test_read_probe_argument_checks():
    """kin_hbm_read_probe rejects NULL or misaligned buffers and sizes that are
    not a positive multiple of 16, before any launch."""
    L = ctypes.CDLL(kb.LIB_PATH)
    f = L.kin_hbm_read_probe
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    null, shape, align = -1, -2, -4
    assert f(None, 64, FAKE, None) == null
    assert f(FAKE, 64, None, None) == null
    assert f(MISALIGNED, 64, FAKE, None) == align
    assert f(FAKE, 0, FAKE, None) == shape
    assert f(FAKE, 40, FAKE, None) == shape


def test_noalloc_step_rejects_a_step_beyond_its_scratch():
    """kin_sparse_decode_step_noalloc checks, on the host and before any
    launch, that the step fits its scratch array: 192 pairs of 16384 blocks
    with no scores buffer keep 24 MiB of scores in the workspace, more than
    KIN_NOALLOC_SCRATCH_BYTES (16 MiB), so the call returns KIN_ERR_WORKSPACE."""
    d = kb.make_desc(64, 3, 4, 262144, 262144, 16, kb.KIN_BF16)
    rc = _raw("kin_sparse_decode_step_noalloc", ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 64,
              FAKE, FAKE, None)
    assert rc == -6
    assert "scratch" in kb.kin_last_error()
    # the argument checks of kin_sparse_decode_step come first
    rc = _raw("kin_sparse_decode_step_noalloc", ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0,
              FAKE, FAKE, None)
    assert rc == -2
    rc = _raw("kin_sparse_decode_step_noalloc", ctypes.byref(d), None, FAKE, FAKE, FAKE, None, 64,
              FAKE, FAKE, None)
    assert rc == -1
