"""The read-bandwidth probe (a measurement helper): it reads every 16-byte
word of the buffer exactly once, so the sink ends up holding the XOR of the
whole buffer; a size that is not a multiple of the grid stride covers the
tail loop."""
import numpy as np
import pytest
import torch

from block_top_sparse_amd import binding as kb

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kb.lib()


@pytest.mark.parametrize("nbytes", [16, 4096 + 16 * 37, 3 * 2**20 + 16 * 37, 64 * 2**20])
def test_read_probe_reads_every_word_once(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    kb.kin_hbm_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert (sink.cpu().numpy().view(np.uint32) == want).all()
    # XOR-accumulated: a second pass over the same buffer cancels the first
    kb.kin_hbm_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 0).all()
