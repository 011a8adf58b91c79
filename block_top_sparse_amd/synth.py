"""Seeded synthetic decode inputs.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  The tests, the benchmark and the smoke check use
it to make the bytes that BOTH the HIP library and the CPU oracle read.

Recipe (a stand-in for Qwen3-style long-CoT / Best-of-N decode caches; no
dataset is used):
  q, V  ~ N(0, 1)
  keys  k_t = z_t + c_j * u,  z_t ~ N(0, I_d),  c_j ~ N(0, 0.5^2) per
        (sequence, KV head, block), u a random unit vector per
        (sequence, KV head); the offset makes block scores distinct.
  heavy (optional) h distinct blocks per (sequence, KV head), drawn
        uniformly; every key of those blocks gets + 2 * q_hat, where q_hat
        is the unit vector of the sum of the group's stored (already
        rounded) query heads.
Values are drawn in fp32 and then rounded to the cache dtype by torch's
cast (round to nearest even); the stored bytes ARE the inputs.  Cache rows
at or beyond ctx_len (when the capacity is larger) are filled with
`tail_fill` (NaN by default) so that any read past the context shows.

Streams: component i of a workload with seed s draws from a generator
seeded with s * 8 + i (0: q, 1: z, 2: V, 3: c, 4: u, 5: heavy).  Large
caches are generated one sequence at a time to bound the fp32 scratch.
"""
import torch

from .workloads import Workload

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(w: Workload):
    return _TORCH_DTYPE[w.dtype]


def _gen(seed: int, comp: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 8 + comp)
    return g


def make_inputs(w: Workload, device="cpu", tail_fill=float("nan"), seed=None):
    """Return dict(q, K, V) for workload w on `device`.

    q: [batch][hq][d], K and V: [batch][hkv][cap][d], all in w's dtype."""
    seed = w.seed if seed is None else seed
    dt = torch_dtype(w)
    d, L, cap, B = w.head_dim, w.ctx_len, w.cap, w.block
    nb = w.nb
    gq, gz, gv, gc, gu, gh = (_gen(seed, i, device) for i in range(6))

    q = torch.randn((w.batch, w.hq, d), generator=gq, device=device, dtype=torch.float32).to(dt)
    K = torch.empty((w.batch, w.hkv, cap, d), device=device, dtype=dt)
    V = torch.empty((w.batch, w.hkv, cap, d), device=device, dtype=dt)

    for b in range(w.batch):
        z = torch.randn((w.hkv, L, d), generator=gz, device=device, dtype=torch.float32)
        c = torch.randn((w.hkv, nb), generator=gc, device=device, dtype=torch.float32) * 0.5
        u = torch.randn((w.hkv, d), generator=gu, device=device, dtype=torch.float32)
        u = u / u.norm(dim=1, keepdim=True)
        off = c.repeat_interleave(B, dim=1)[:, :L]           # [hkv][L]
        z += off[:, :, None] * u[:, None, :]
        if w.heavy_blocks:
            qs = q[b].float().view(w.hkv, w.gqa, d).sum(dim=1)  # [hkv][d]
            qhat = qs / qs.norm(dim=1, keepdim=True)
            for g in range(w.hkv):
                pick = torch.randperm(nb, generator=gh, device=device)[: w.heavy_blocks]
                for j in pick.tolist():
                    z[g, j * B: min((j + 1) * B, L)] += 2.0 * qhat[g]
        K[b, :, :L] = z.to(dt)
        del z
        V[b, :, :L] = torch.randn((w.hkv, L, d), generator=gv, device=device,
                                  dtype=torch.float32).to(dt)
        if cap > L:
            K[b, :, L:] = tail_fill
            V[b, :, L:] = tail_fill
    return {"q": q, "K": K, "V": V}


def heavy_block_ids(w: Workload, device="cpu", seed=None):
    """Re-draw the heavy block ids of make_inputs (same stream, same order)
    as a list over batch of [hkv] lists, for the heavy-block invariant."""
    seed = w.seed if seed is None else seed
    gh = _gen(seed, 5, device)
    out = []
    for _b in range(w.batch):
        row = []
        for _g in range(w.hkv):
            row.append(sorted(torch.randperm(w.nb, generator=gh, device=device)[: w.heavy_blocks]
                              .tolist()))
        out.append(row)
    return out


def small_int_inputs(batch, hq, hkv, d, ctx_len, block, seed, lo=-3, hi=4, cap=None,
                     dtype=torch.float32):
    """Small-integer q, K, V (exact in bf16 and fp32) for hand-checkable pins."""
    g = torch.Generator().manual_seed(seed)
    cap = cap or ctx_len
    q = torch.randint(lo, hi, (batch, hq, d), generator=g).to(dtype)
    K = torch.randint(lo, hi, (batch, hkv, cap, d), generator=g).to(dtype)
    V = torch.randint(lo, hi, (batch, hkv, cap, d), generator=g).to(dtype)
    return {"q": q, "K": K, "V": V}
