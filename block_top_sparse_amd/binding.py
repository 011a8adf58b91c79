"""Python binding of libkin.so (include/kin.h): argument marshalling only.

Every function has the name of the C entry point it calls and takes torch
device tensors (or None) plus an optional stream (a torch.cuda.Stream, a raw
hipStream_t handle, or None for torch's current stream).  Nothing here
computes: every step runs in the HIP kernels of libkin.so.  A non-zero
status raises KinError with the library's own message.  If libkin.so has not
been built the first call raises; there is no fallback.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkin.so")

KIN_F32, KIN_BF16 = 0, 1
_STATUS = {0: "KIN_OK", -1: "KIN_ERR_NULL", -2: "KIN_ERR_SHAPE", -3: "KIN_ERR_DTYPE",
           -4: "KIN_ERR_ALIGN", -5: "KIN_ERR_UNSUPPORTED", -6: "KIN_ERR_WORKSPACE",
           -7: "KIN_ERR_HIP"}
_DT = {torch.float32: KIN_F32, torch.bfloat16: KIN_BF16}


class KinError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class kin_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hkv", ctypes.c_int32), ("gqa", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("t_cap", ctypes.c_int32),
                ("ctx_len", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return "kin_desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class kin_pages(ctypes.Structure):
    """Variable lengths / paged caches: device pointers (ctx_lens [batch],
    page_table [batch][max_pages], int32, or None) and the page geometry."""
    _fields_ = [("ctx_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class kin_shared_prompt(ctypes.Structure):
    """Shared prompts: samples per prompt, prompt tokens, and the prompts'
    K, V and summaries (device pointers)."""
    _fields_ = [("n_share", ctypes.c_int32), ("prompt_len", ctypes.c_int32),
                ("Kp", ctypes.c_void_p), ("Vp", ctypes.c_void_p), ("Sp", ctypes.c_void_p)]


def make_share(n_share, prompt_len, Kp, Vp, Sp):
    """A kin_shared_prompt from torch device tensors."""
    return kin_shared_prompt(n_share, prompt_len, Kp.data_ptr(), Vp.data_ptr(), Sp.data_ptr())


def make_pages(ctx_lens=None, page_table=None, page_size=0, max_pages=0, num_pages=0):
    """A kin_pages from torch int32 device tensors (or None)."""
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return kin_pages(ptr(ctx_lens), ptr(page_table), page_size, max_pages, num_pages)


def make_desc(batch, hkv, gqa, t_cap, ctx_len, block, dtype, head_dim=128) -> kin_desc:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return kin_desc(batch, hkv, gqa, head_dim, t_cap, ctx_len, block, dt)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(or python block_top_sparse_amd/build.py) first")
        L = ctypes.CDLL(LIB_PATH)
        D, P, I, Z = ctypes.POINTER(kin_desc), ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        G = ctypes.POINTER(kin_pages)
        H = ctypes.POINTER(kin_shared_prompt)
        sig = {
            "kin_block_summary_update": (I, [D, P, P, I, I, P]),
            "kin_block_score": (I, [D, P, P, P, P]),
            "kin_block_topk": (I, [D, P, I, P, P]),
            "kin_sparse_decode_attn": (I, [D, P, P, P, P, I, P, P, Z, P]),
            "kin_dense_decode_attn": (I, [D, P, P, P, P, P, Z, P]),
            "kin_sparse_decode_step": (I, [D, P, P, P, P, P, I, P, P, P, Z, P]),
            "kin_decode_update_score": (I, [D, P, P, P, P, P]),
            "kin_decode_select_attend": (I, [D, P, P, P, P, I, P, P, P, Z, P]),
            "kin_sparse_ws_bytes": (Z, [D, I]),
            "kin_dense_ws_bytes": (Z, [D]),
            "kin_hbm_read_probe": (I, [P, Z, P, P]),
            "kin_status_str": (ctypes.c_char_p, [I]),
            "kin_last_error": (ctypes.c_char_p, []),
            "kin_version": (I, []),
            "kin_paged_summary_update": (I, [D, G, P, P, I, I, P]),
            "kin_paged_decode_step": (I, [D, G, P, P, P, P, P, I, P, P, P, Z, P]),
            "kin_token_decode_step": (I, [D, P, P, P, P, I, P, P, P, Z, P]),
            "kin_shared_decode_step": (I, [D, H, P, P, P, P, P, I, P, P, P, Z, P]),
            "kin_quest_summary_update": (I, [D, P, P, I, I, P]),
            "kin_quest_decode_step": (I, [D, P, P, P, P, P, I, P, P, P, Z, P]),
            "kin_quest_ws_bytes": (Z, [D, I]),
            "kin_token_ws_bytes": (Z, [D, I]),
            "kin_sparse_decode_step_noalloc": (I, [D, P, P, P, P, P, I, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def exported_names():
    return ["kin_block_summary_update", "kin_block_score", "kin_block_topk",
            "kin_sparse_decode_attn", "kin_dense_decode_attn", "kin_sparse_decode_step",
            "kin_decode_update_score", "kin_decode_select_attend",
            "kin_sparse_ws_bytes", "kin_dense_ws_bytes", "kin_status_str", "kin_last_error",
            "kin_version", "kin_paged_summary_update", "kin_paged_decode_step",
            "kin_token_decode_step", "kin_token_ws_bytes", "kin_shared_decode_step",
            "kin_quest_summary_update", "kin_quest_decode_step", "kin_quest_ws_bytes",
            "kin_hbm_read_probe", "kin_sparse_decode_step_noalloc"]


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check(rc):
    if rc != 0:
        raise KinError(rc, lib().kin_last_error().decode())


def kin_block_summary_update(desc, K, S, t_begin, t_end, stream=None):
    _check(lib().kin_block_summary_update(ctypes.byref(desc), _p(K), _p(S), t_begin, t_end,
                                          _s(stream)))


def kin_block_score(desc, q, S, scores, stream=None):
    _check(lib().kin_block_score(ctypes.byref(desc), _p(q), _p(S), _p(scores), _s(stream)))


def kin_block_topk(desc, scores, k, idx, stream=None):
    _check(lib().kin_block_topk(ctypes.byref(desc), _p(scores), k, _p(idx), _s(stream)))


def kin_sparse_decode_attn(desc, q, K, V, idx, k, out, ws=None, stream=None):
    _check(lib().kin_sparse_decode_attn(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(idx), k,
                                        _p(out), _p(ws), _nbytes(ws), _s(stream)))


def kin_dense_decode_attn(desc, q, K, V, out, ws=None, stream=None):
    _check(lib().kin_dense_decode_attn(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(out), _p(ws),
                                       _nbytes(ws), _s(stream)))


def kin_sparse_decode_step(desc, q, K, V, S, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_sparse_decode_step(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(S),
                                        _p(scores), k, _p(idx), _p(out), _p(ws), _nbytes(ws),
                                        _s(stream)))


def kin_sparse_decode_step_noalloc(desc, q, K, V, S, scores, k, idx, out, stream=None):
    _check(lib().kin_sparse_decode_step_noalloc(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(S),
                                                _p(scores), k, _p(idx), _p(out), _s(stream)))


def kin_paged_summary_update(desc, pages, K, S, t_begin, t_end, stream=None):
    _check(lib().kin_paged_summary_update(ctypes.byref(desc), ctypes.byref(pages), _p(K), _p(S),
                                          t_begin, t_end, _s(stream)))


def kin_paged_decode_step(desc, pages, q, K, V, S, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_paged_decode_step(ctypes.byref(desc), ctypes.byref(pages), _p(q), _p(K),
                                       _p(V), _p(S), _p(scores), k, _p(idx), _p(out), _p(ws),
                                       _nbytes(ws), _s(stream)))


def kin_shared_decode_step(desc, share, q, K, V, S, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_shared_decode_step(ctypes.byref(desc), ctypes.byref(share), _p(q), _p(K),
                                        _p(V), _p(S), _p(scores), k, _p(idx), _p(out), _p(ws),
                                        _nbytes(ws), _s(stream)))


def kin_quest_summary_update(desc, K, Sq, t_begin, t_end, stream=None):
    _check(lib().kin_quest_summary_update(ctypes.byref(desc), _p(K), _p(Sq), t_begin, t_end,
                                          _s(stream)))


def kin_quest_decode_step(desc, q, K, V, Sq, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_quest_decode_step(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(Sq),
                                       _p(scores), k, _p(idx), _p(out), _p(ws), _nbytes(ws),
                                       _s(stream)))


def kin_quest_ws_bytes(desc, k) -> int:
    n = lib().kin_quest_ws_bytes(ctypes.byref(desc), k)
    if n == ctypes.c_size_t(-1).value:
        raise KinError(-2, lib().kin_last_error().decode())
    return n


def kin_token_decode_step(desc, q, K, V, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_token_decode_step(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(scores), k,
                                       _p(idx), _p(out), _p(ws), _nbytes(ws), _s(stream)))


def kin_token_ws_bytes(desc, k) -> int:
    n = lib().kin_token_ws_bytes(ctypes.byref(desc), k)
    if n == ctypes.c_size_t(-1).value:
        raise KinError(-2, lib().kin_last_error().decode())
    return n


def kin_decode_update_score(desc, q, K, S, scores, stream=None):
    _check(lib().kin_decode_update_score(ctypes.byref(desc), _p(q), _p(K), _p(S), _p(scores),
                                         _s(stream)))


def kin_decode_select_attend(desc, q, K, V, scores, k, idx, out, ws=None, stream=None):
    _check(lib().kin_decode_select_attend(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(scores), k,
                                          _p(idx), _p(out), _p(ws), _nbytes(ws), _s(stream)))


def kin_sparse_ws_bytes(desc, k) -> int:
    n = lib().kin_sparse_ws_bytes(ctypes.byref(desc), k)
    if n == ctypes.c_size_t(-1).value:
        raise KinError(-2, lib().kin_last_error().decode())
    return n


def kin_hbm_read_probe(buf, nbytes, sink, stream=None):
    """Stream nbytes of buf (a measurement helper); XOR-folds into sink."""
    _check(lib().kin_hbm_read_probe(_p(buf), nbytes, _p(sink), _s(stream)))


def kin_dense_ws_bytes(desc) -> int:
    n = lib().kin_dense_ws_bytes(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise KinError(-2, lib().kin_last_error().decode())
    return n


def kin_status_str(status) -> str:
    return lib().kin_status_str(status).decode()


def kin_last_error() -> str:
    return lib().kin_last_error().decode()


def kin_version() -> int:
    return lib().kin_version()
