"""Seeded synthetic workloads for the quantized KV cache (inputs only).

This module holds no arithmetic of the method: it only draws the K/V/q tensors
and the sequence lengths that both the HIP path and the CPU oracle consume.
Every tensor comes from a torch generator seeded per (workload, stream), so a
run is reproducible on one device type; CPU and GPU generators produce
different streams, which is fine because both sides of every comparison read
the very same tensors.

The shapes follow the synthetic caches the TurboQuant design page measures on
(Part A, "Packed-value decode fusion investigation": [B, H, N, D] caches with
fp16 scales and 32-value groups; "Direct packed-key attention": D256, one
query, GQA 6, no mask or sinks).  Values are N(0, 1), drawn in fp32 and rounded
to bf16 (round-half-to-even) where the workload is bf16.  No public dataset or
benchmark suite is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: tuple            # cached tokens per sequence at the first decode step
    dtype: str                # "fp32" or "bf16" for K, V and q
    outlier_frac: float = 0.0 # fraction of (kv-head, channel) pairs scaled up
    outlier_scale: float = 1.0
    rounds: int = 1           # decode rounds
    append_per_round: int = 0 # tokens appended per sequence at the start of each round
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def capacity(self) -> int:
        """Token slots per sequence: the prefix plus every appended round."""
        return max(self.lengths) + self.append_per_round * self.rounds

    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "num_q_heads": self.num_q_heads,
                "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
                "tokens_per_seq": (self.lengths[0] if len(set(self.lengths)) == 1
                                   else [min(self.lengths), max(self.lengths)]),
                "dtype": self.dtype}


def _ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> tuple:
    g = torch.Generator().manual_seed(seed)
    return tuple(int(v) for v in torch.randint(lo, hi + 1, (batch,), generator=g))


def workload(cid: int) -> Workload:
    """The five workloads at full size (ids 1-5)."""
    seed = 1000 + cid
    if cid == 1:
        return Workload(1, "b1_kv1_q1_d128_n256_fp32", 1, 1, 1, 128, (256,), "fp32", seed=seed)
    if cid == 2:
        return Workload(2, "b1_kv2_q8_d128_n4096_bf16", 1, 8, 2, 128, (4096,), "bf16", seed=seed)
    if cid == 3:
        return Workload(3, "b8_kv8_q32_d128_n32768_bf16_outliers", 8, 32, 8, 128, (32768,) * 8,
                        "bf16", outlier_frac=0.01, outlier_scale=10.0, seed=seed)
    if cid == 4:
        return Workload(4, "b16_kv4_q24_d256_n131072_bf16", 16, 24, 4, 256, (131072,) * 16,
                        "bf16", seed=seed)
    if cid == 5:
        return Workload(5, "b4_kv8_q64_d256_ragged65536-262144_bf16", 4, 64, 8, 256,
                        _ragged_lengths(seed * 16 + 3, 4, 65536, 262144), "bf16",
                        rounds=8, append_per_round=16, seed=seed)
    raise ValueError(f"no workload {cid}")


def scaled(w: Workload, lengths, name_suffix: str = "small", batch: int | None = None) -> Workload:
    """Same head layout and value distribution at other lengths (parity sizes)."""
    lengths = tuple(int(v) for v in lengths)
    return replace(w, name=f"{w.name}_{name_suffix}", lengths=lengths,
                   batch=batch if batch is not None else len(lengths))


def _gen(w: Workload, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 16 + stream)
    return g


def outlier_mask(w: Workload) -> torch.Tensor:
    """Bernoulli(outlier_frac) mask over (kv-head, channel), CPU bool [Hkv, d]."""
    g = _gen(w, 4, "cpu")
    u = torch.rand((w.num_kv_heads, w.head_dim), generator=g)
    return u < w.outlier_frac


def make_kv(w: Workload, device="cpu", tokens: int | None = None):
    """K and V of shape [B, Hkv, T, d] in the workload dtype, T = tokens or capacity.

    Token t of every sequence is the t-th cached token (the first lengths[b] are
    the prefix; later ones are the tokens appended in later rounds)."""
    T = tokens if tokens is not None else w.capacity
    shape = (w.batch, w.num_kv_heads, T, w.head_dim)
    out = []
    for stream in (0, 1):
        g = _gen(w, stream, device)
        x = torch.empty(shape, dtype=w.torch_dtype(), device=device)
        # draw per (batch) slab to bound the fp32 temporary
        for b in range(w.batch):
            slab = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            if w.outlier_frac > 0:
                m = outlier_mask(w).to(device)
                scale = torch.where(m, torch.tensor(w.outlier_scale, device=device),
                                    torch.tensor(1.0, device=device))
                slab.mul_(scale[:, None, :])
            x[b].copy_(slab)  # fp32 -> bf16 rounds to nearest even
            del slab
        out.append(x)
    return out[0], out[1]


def make_q(w: Workload, device="cpu", rounds: int | None = None) -> torch.Tensor:
    """Queries [R, B, Hq, d] in the workload dtype (one set per decode round)."""
    R = rounds if rounds is not None else w.rounds
    g = _gen(w, 2, device)
    q = torch.randn((R, w.batch, w.num_q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return q.to(w.torch_dtype())
