"""Device buffers for one decode layer (torch allocations; plumbing only).

Allocates what the C ABI takes -- summaries, scores, indices, output and
workspace -- in the layouts of include/kin.h, for a Workload whose q, K, V
already sit on the device.
"""
import torch

from . import binding as kb
from .workloads import Workload


class LayerBuffers:
    def __init__(self, w: Workload, device="cuda", k=None, with_dense=False):
        self.w = w
        self.k = w.topk if k is None else k
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        self.desc = kb.make_desc(w.batch, w.hkv, w.gqa, w.cap, w.ctx_len, w.block, dt,
                                 head_dim=w.head_dim)
        self.S = torch.empty((w.batch, w.hkv, w.nb_cap, w.head_dim), device=device, dtype=dt)
        self.scores = torch.empty((w.batch, w.hkv, w.nb_cap), device=device, dtype=torch.float64)
        self.idx = torch.empty((w.batch, w.hkv, self.k), device=device, dtype=torch.int32)
        self.out = torch.empty((w.batch, w.hq, w.head_dim), device=device, dtype=dt)
        n = kb.kin_sparse_ws_bytes(self.desc, self.k)
        self.ws = torch.zeros(max(n, 16), device=device, dtype=torch.uint8) if n else None
        self.out_dense = None
        self.ws_dense = None
        if with_dense:
            self.out_dense = torch.empty_like(self.out)
            nd = kb.kin_dense_ws_bytes(self.desc)
            self.ws_dense = torch.zeros(max(nd, 16), device=device, dtype=torch.uint8) if nd else None
