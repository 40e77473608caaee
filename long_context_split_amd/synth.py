"""Seeded synthetic inputs for verification attention over a paged E4M3 KV cache.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  It serves both the HIP path (tests, benchmark) and the CPU oracle
(which receives the same arrays, copied to the host).

Recipe (the workload shapes of the pages, which measure q8 / six query heads /
one KV head / head dim 256 with E4M3 KV and FP16 activations over sixteen
distinct layer KV allocations at up to 261888 context tokens):

* Q: FP16 draws of N(0, 1), shape [B, q, 6, 256].
* K, V: FP32 draws of N(0, 1), divided by the per-layer scale, clamped to
  +-448 and cast to OCP E4M3 with round-to-nearest-even (torch's
  ``float8_e4m3fn`` cast).  ``key_mix`` > 0 draws each key *token* from N(0, 2^2)
  with that probability instead (peaky softmax rows).
* Scales: fixed (e.g. 1/8) or U(0.05, 0.2) per layer, separately for K and V.
* Paging: 16-token pages.  Logical pages of all sequences are placed on a seeded
  random permutation of physical pages.  A few spare physical pages hold the
  E4M3 NaN code 0x7F and are never mapped; slots past the context end in a
  sequence's last page also hold 0x7F, and block-table entries past the
  sequence's last page point at a poison page.  Any read of unmapped data
  therefore shows up as NaN in the results.
* Draw order per layer: scales, K, key mixture, V, permutation, Q.  Generation
  runs on ``device`` with a ``torch.Generator`` seeded by
  ``seed_base * 1_000_003 + layer``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

HQ = 6
HKV = 1
HEAD_DIM = 256
BLOCK_SIZE = 16
E4M3_MAX = 448.0
POISON_CODE = 0x7F
SPARE_PAGES = 2


@dataclass
class LayerInputs:
    q: torch.Tensor              # float16 [B, nq, 6, 256]
    k_cache: torch.Tensor        # uint8   [num_blocks, 16, 1, 256]
    v_cache: torch.Tensor        # uint8   [num_blocks, 16, 1, 256]
    block_table: torch.Tensor    # int32   [B, max_blocks]
    context_lens: torch.Tensor   # int32   [B]
    k_scale: torch.Tensor        # float32 [1]
    v_scale: torch.Tensor        # float32 [1]
    softmax_scale: float
    meta: dict = field(default_factory=dict)

    def to(self, device) -> "LayerInputs":
        return LayerInputs(self.q.to(device), self.k_cache.to(device), self.v_cache.to(device),
                           self.block_table.to(device), self.context_lens.to(device),
                           self.k_scale.to(device), self.v_scale.to(device), self.softmax_scale,
                           dict(self.meta))

    def numpy(self) -> dict:
        """Host copies as numpy arrays, in the argument order of the oracle."""
        return dict(q=self.q.cpu().numpy(), k_cache=self.k_cache.cpu().numpy(),
                    v_cache=self.v_cache.cpu().numpy(), block_table=self.block_table.cpu().numpy(),
                    context_lens=self.context_lens.cpu().numpy(),
                    k_scale=float(self.k_scale.cpu()[0]), v_scale=float(self.v_scale.cpu()[0]),
                    softmax_scale=self.softmax_scale)


def quantize_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """E4M3 codes of x / scale, clamped to the finite range, cast with RNE."""
    return (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def make_layer(context_lens: Sequence[int], num_q: int, *, seed_base: int, layer: int = 0,
               device="cpu", scales: Optional[tuple] = None, key_mix: float = 0.0,
               max_blocks: Optional[int] = None, head_dim: int = HEAD_DIM,
               softmax_scale: Optional[float] = None) -> LayerInputs:
    """One layer's inputs for a batch of sequences with the given context lengths."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_base * 1_000_003 + layer)
    lens = [int(x) for x in context_lens]
    B = len(lens)
    if any(L < num_q for L in lens):
        raise ValueError("each context must hold the q query tokens")
    pages = [-(-L // BLOCK_SIZE) for L in lens]
    if max_blocks is None:
        max_blocks = max(pages)
    if max_blocks < max(pages):
        raise ValueError("max_blocks too small for the longest context")
    total_pages = sum(pages)
    num_blocks = total_pages + SPARE_PAGES

    u = torch.rand(2, generator=gen, device=device, dtype=torch.float32)
    if scales is None:
        k_scale = float(0.05 + 0.15 * u[0].item())
        v_scale = float(0.05 + 0.15 * u[1].item())
    else:
        k_scale, v_scale = float(scales[0]), float(scales[1])
    k_scale = float(torch.tensor(k_scale, dtype=torch.float32))
    v_scale = float(torch.tensor(v_scale, dtype=torch.float32))

    n_tok = total_pages * BLOCK_SIZE
    kx = torch.randn(n_tok, head_dim, generator=gen, device=device, dtype=torch.float32)
    if key_mix > 0.0:
        wide = torch.rand(n_tok, generator=gen, device=device) < key_mix
        kx[wide] *= 2.0
    k_codes = quantize_e4m3(kx, k_scale)
    del kx
    vx = torch.randn(n_tok, head_dim, generator=gen, device=device, dtype=torch.float32)
    v_codes = quantize_e4m3(vx, v_scale)
    del vx

    perm = torch.randperm(num_blocks, generator=gen, device=device)
    q = torch.randn(B, num_q, HQ, head_dim, generator=gen, device=device,
                    dtype=torch.float32).to(torch.float16)

    k_cache = torch.full((num_blocks, BLOCK_SIZE, HKV, head_dim), POISON_CODE, dtype=torch.uint8,
                         device=device)
    v_cache = torch.full_like(k_cache, POISON_CODE)
    poison_page = int(perm[total_pages].item())
    block_table = torch.full((B, max_blocks), poison_page, dtype=torch.int32, device=device)
    off = 0
    for b, (L, npg) in enumerate(zip(lens, pages)):
        phys = perm[off:off + npg]
        tok = slice(off * BLOCK_SIZE, (off + npg) * BLOCK_SIZE)
        kc = k_codes[tok].clone().view(npg, BLOCK_SIZE, head_dim)
        vc = v_codes[tok].clone().view(npg, BLOCK_SIZE, head_dim)
        tail = npg * BLOCK_SIZE - L
        if tail:
            kc.view(-1, head_dim)[L:] = POISON_CODE
            vc.view(-1, head_dim)[L:] = POISON_CODE
        k_cache[phys, :, 0, :] = kc
        v_cache[phys, :, 0, :] = vc
        block_table[b, :npg] = phys.to(torch.int32)
        off += npg

    if softmax_scale is None:
        softmax_scale = 1.0 / (head_dim ** 0.5)
    return LayerInputs(
        q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
        context_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        k_scale=torch.tensor([k_scale], dtype=torch.float32, device=device),
        v_scale=torch.tensor([v_scale], dtype=torch.float32, device=device),
        softmax_scale=float(softmax_scale),
        meta=dict(seed_base=seed_base, layer=layer, key_mix=key_mix, num_q=num_q))


def make_periodic_layer(context_len: int, num_q: int, period: int, *, seed_base: int, device="cpu",
                        scales=(0.125, 0.125)) -> LayerInputs:
    """One sequence whose key and value rows repeat with `period` tokens.

    Token t holds row t mod period of a K pattern and of a V pattern (each drawn
    and quantized as in :func:`make_layer`); pages are placed on a seeded random
    permutation with the same poison as there.  A long context then needs only
    the patterns to describe it (``meta["k_pattern"]``, ``meta["v_pattern"]``:
    uint8 [period, 256]).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_base * 1_000_003 + period)
    L = int(context_len)
    if L < num_q:
        raise ValueError("the context must hold the q query tokens")
    k_scale = float(torch.tensor(float(scales[0]), dtype=torch.float32))
    v_scale = float(torch.tensor(float(scales[1]), dtype=torch.float32))
    kp = quantize_e4m3(torch.randn(period, HEAD_DIM, generator=gen, device=device), k_scale)
    vp = quantize_e4m3(torch.randn(period, HEAD_DIM, generator=gen, device=device), v_scale)
    npg = -(-L // BLOCK_SIZE)
    num_blocks = npg + SPARE_PAGES
    perm = torch.randperm(num_blocks, generator=gen, device=device)
    q = torch.randn(1, num_q, HQ, HEAD_DIM, generator=gen, device=device, dtype=torch.float32).to(torch.float16)
    k_cache = torch.full((num_blocks, BLOCK_SIZE, HKV, HEAD_DIM), POISON_CODE, dtype=torch.uint8, device=device)
    v_cache = torch.full_like(k_cache, POISON_CODE)
    phys = perm[:npg]
    step = 1 << 16                                   # pages per write, bounds the temporaries
    for p0 in range(0, npg, step):
        p1 = min(npg, p0 + step)
        t = torch.arange(p0 * BLOCK_SIZE, p1 * BLOCK_SIZE, device=device)
        kr = kp[t % period]
        vr = vp[t % period]
        past = t >= L
        kr[past] = POISON_CODE
        vr[past] = POISON_CODE
        k_cache[phys[p0:p1], :, 0, :] = kr.view(p1 - p0, BLOCK_SIZE, HEAD_DIM)
        v_cache[phys[p0:p1], :, 0, :] = vr.view(p1 - p0, BLOCK_SIZE, HEAD_DIM)
    block_table = phys.to(torch.int32).view(1, npg).clone()
    return LayerInputs(
        q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
        context_lens=torch.tensor([L], dtype=torch.int32, device=device),
        k_scale=torch.tensor([k_scale], dtype=torch.float32, device=device),
        v_scale=torch.tensor([v_scale], dtype=torch.float32, device=device),
        softmax_scale=1.0 / (HEAD_DIM ** 0.5),
        meta=dict(seed_base=seed_base, period=period, num_q=num_q, k_pattern=kp, v_pattern=vp))


# Named workloads: the pages' q8 / Hq6 / Hkv1 / D256 verification attention at the
# context lengths they measure (up to the 261888-token capacity boundary).
WORKLOADS = {
    "tiny_ctx4096": dict(layers=1, context=4096, num_q=(8,), scales=(0.125, 0.125), key_mix=0.0, seed=1),
    "ctx32768_16layer": dict(layers=16, context=32768, num_q=(8,), scales=None, key_mix=0.0, seed=2),
    "ctx131072_peaky_16layer": dict(layers=16, context=131072, num_q=(8,), scales=None, key_mix=0.05, seed=3),
    "ctx261888_16layer": dict(layers=16, context=261888, num_q=(8,), scales=None, key_mix=0.0, seed=4),
    "ctx261888_smallq_16layer": dict(layers=16, context=261888, num_q=(1, 2, 3, 4, 5, 6, 7), scales=None,
                                     key_mix=0.0, seed=5),
}


def workload_layer(name: str, layer: int, num_q: Optional[int] = None, device="cpu",
                   context: Optional[int] = None) -> LayerInputs:
    w = WORKLOADS[name]
    nq = num_q if num_q is not None else w["num_q"][0]
    L = context if context is not None else w["context"]
    return make_layer([L], nq, seed_base=w["seed"] * 100 + nq, layer=layer, device=device,
                      scales=w["scales"], key_mix=w["key_mix"])
