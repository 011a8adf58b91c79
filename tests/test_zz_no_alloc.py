"""kin_sparse_decode_step_noalloc (the step for callers that cannot allocate:
its workspace is the library's per-device scratch array) against
kin_sparse_decode_step with a workspace of its own, through the C ABI: two
calls in a row on the scratch array, the second with a smaller input, each
equal to the workspace call bit for bit (the same kernels on the same
inputs), for each form that uses a workspace."""
import zlib

import pytest
import torch

from block_top_sparse_amd import binding as kb
from block_top_sparse_amd.buffers import LayerBuffers
from block_top_sparse_amd.workloads import Workload

from parity_util import bits, check_sequences, gpu_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


def _case(name, b, hq, hkv, L, B, k, dt, cap):
    w = Workload(name, batch=b, hq=hq, hkv=hkv, ctx_len=L, block=B, topk=k, dtype=dt,
                 seed=zlib.crc32(name.encode()) % 10000, t_cap=cap)
    inp = gpu_inputs(w)
    return w, inp


def _run(w, inp, k, scores, noalloc):
    bufs = LayerBuffers(w, k=k)
    bufs.out.fill_(float("nan"))
    bufs.idx.fill_(-7)
    bufs.scores.fill_(float("nan"))
    if w.nb > 1:
        kb.kin_block_summary_update(bufs.desc, inp["K"], bufs.S, 0, (w.nb - 1) * w.block)
    sc = bufs.scores if scores else None
    if noalloc:
        kb.kin_sparse_decode_step_noalloc(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S, sc, k,
                                          bufs.idx, bufs.out)
    else:
        kb.kin_sparse_decode_step(bufs.desc, inp["q"], inp["K"], inp["V"], bufs.S, sc, k,
                                  bufs.idx, bufs.out, bufs.ws)
    torch.cuda.synchronize()
    return bufs


# (larger, smaller) shapes of each form that takes a workspace
PAIRS = [
    ("two-kernel-bf16",
     ("na-a", 4, 32, 4, 20000, 16, 300, "bf16", 20480), ("na-b", 2, 16, 2, 5000, 16, 100, "bf16", 5120)),
    ("keep-all-one-launch",
     ("na-c", 3, 32, 4, 4000, 32, 125, "bf16", 4096), ("na-d", 2, 16, 4, 2000, 16, 125, "bf16", 2048)),
    ("fp32-split",
     ("na-e", 3, 4, 2, 9000, 16, 500, "f32", 9024), ("na-f", 3, 2, 2, 4730, 16, 292, "f32", 4793)),
    ("fp32-one-kernel",
     ("na-i", 1, 8, 2, 4096, 16, 32, "f32", 4096), ("na-j", 1, 4, 2, 2048, 16, 16, "f32", 2048)),
    ("four-launch-bf16",
     ("na-g", 1, 8, 2, 40000, 16, 2100, "bf16", 40000), ("na-h", 1, 8, 2, 36000, 16, 2050, "bf16", 36000)),
]


@pytest.mark.parametrize("scores", [False, True], ids=["no-scores", "scores"])
@pytest.mark.parametrize("pair", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_step_equals_workspace_step_twice_second_smaller(pair, scores):
    form, big, small = pair
    for i, spec in enumerate((big, small)):
        w, inp = _case(*spec)
        k = spec[6]
        need = kb.kin_sparse_ws_bytes(LayerBuffers(w, k=k).desc, k)
        say(f"{form} call {i + 1}: {spec[0]} (workspace {need} bytes)")
        assert 0 < need <= 16 << 20
        ref = _run(w, inp, k, scores, noalloc=False)
        got = _run(w, inp, k, scores, noalloc=True)
        assert torch.equal(got.idx, ref.idx), f"{form}: selection"
        assert torch.equal(bits(got.out), bits(ref.out)), f"{form}: output"
        assert torch.equal(bits(got.S[:, :, :w.nb]), bits(ref.S[:, :, :w.nb])), f"{form}: S"
        if scores:
            assert torch.equal(got.scores[:, :, :w.nb], ref.scores[:, :, :w.nb])
        check_sequences(w, inp, got, [0, w.batch - 1], check_scores=scores)


def test_noalloc_one_kernel_step_needs_no_scratch():
    """With enough pairs the step is one kernel and takes no workspace: the
    no-allocation call equals the workspace call bit for bit."""
    w, inp = _case("na-one", 32, 32, 8, 4096, 16, 32, "bf16", 4096)
    ref = _run(w, inp, 32, False, noalloc=False)
    got = _run(w, inp, 32, False, noalloc=True)
    assert torch.equal(got.idx, ref.idx)
    assert torch.equal(bits(got.out), bits(ref.out))
