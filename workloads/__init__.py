"""Seeded synthetic inputs for large-head-dim attention workloads.

This module is shared by the HIP path's tests/bench and by the float64 oracle's
tests. It draws random numbers and fixes shapes; it contains no attention
arithmetic (no products, no softmax, no reductions).

Shapes follow the benchmark tables of "FFPA Attention Benchmark"
(ffpa-attn.readthedocs.io, section "More Benchmark": self-attn, cross-attn,
decode-attn, gqa, causal, attn-mask, dropout, non-aligned rows at D=512 and
D=320).
The pages state no value distribution, so every tensor is i.i.d. N(0, 1).
The additive mask is the compact key-position bias of shape [1, 1, 1, Nkv]
named in the "Quick Start" section of the same page; 10% of its entries are
-inf (exactly round(0.1 * Nkv) positions, picked by a seeded permutation).

Seeding: every [N, D] slice of tensor t at (b, h) is drawn from its own
generator seeded with 10**6 * cfg_id + 10**4 * t + 10**2 * b + h
(t: q=1, k=2, v=3, dO=4, mask=5), as float32, then rounded to the storage
dtype (round-to-nearest-even through ``Tensor.to``). The bf16 variant of a
workload reuses the same float32 draws as the fp16 one. A slice drawn on a
CUDA device uses torch's device generator with the same seed; its values
differ from the CPU draw, so a test compares the HIP result against the
oracle run on the very tensors the kernel read (copied back to the host).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

T_Q, T_K, T_V, T_DO, T_MASK = 1, 2, 3, 4, 5

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, options and the seed family it draws from."""

    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str = "fp16"
    accum: str = "f32"
    causal: bool = False
    mask: Optional[str] = None  # None | "key" ([1,1,1,Nkv]) | "query" ([1,1,Nq,Nkv])
    mask_neg_inf_frac: float = 0.1
    backward: bool = False
    # dropout on the probabilities: the pages' tables run a "dropout" case but
    # state no probability; 0.1 is taken here (the seed is the cfg_id)
    dropout_p: float = 0.0

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to float32: the value both sides receive."""
        return float(torch.tensor(1.0 / (self.D ** 0.5), dtype=torch.float32).item())

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(name, cfg_id, B, Hq, Hkv, Nq, Nkv, D, **kw) -> Workload:
    return Workload(name, cfg_id, B, Hq, Hkv, Nq, Nkv, D, **kw)


# The five workload families. Variant families share a cfg_id (their seeds are
# therefore related, which is harmless: each is deterministic on its own).
WORKLOADS = {
    "tiny": _w("tiny", 0, 1, 2, 2, 256, 256, 320),
    "self": _w("self", 1, 1, 32, 32, 8192, 8192, 512),
    "self_bf16": _w("self_bf16", 1, 1, 32, 32, 8192, 8192, 512, dtype="bf16"),
    "self_acc16": _w("self_acc16", 1, 1, 32, 32, 8192, 8192, 512, accum="f16"),
    "cross": _w("cross", 2, 1, 32, 32, 1024, 8192, 512),
    "gqa": _w("gqa", 2, 1, 32, 8, 8192, 8192, 512),
    "causal": _w("causal", 2, 1, 32, 32, 8192, 8192, 512, causal=True),
    "nonaligned": _w("nonaligned", 2, 1, 32, 32, 8191, 8191, 512),
    "mask": _w("mask", 2, 1, 32, 32, 8192, 8192, 512, mask="key"),
    "decode": _w("decode", 3, 16, 32, 32, 1, 8192, 512),
    "bwd": _w("bwd", 4, 1, 32, 32, 8192, 8192, 512, dtype="bf16", backward=True),
    "bwd_causal": _w("bwd_causal", 4, 1, 32, 32, 8192, 8192, 512, dtype="bf16", causal=True,
                     backward=True),
    # the backward at the top of the head-dimension range
    "bwd_d1024": _w("bwd_d1024", 4, 1, 32, 32, 8192, 8192, 1024, dtype="bf16", backward=True),
    "bwd_d1024_causal": _w("bwd_d1024_causal", 4, 1, 32, 32, 8192, 8192, 1024, dtype="bf16",
                           causal=True, backward=True),
}
# 16K sequences (the CuTeDSL tables of "FFPA Attention Benchmark" at 16K, D = 512)
WORKLOADS.update({
    "self16k": _w("self16k", 5, 1, 32, 32, 16384, 16384, 512),
    "self16k_bf16": _w("self16k_bf16", 5, 1, 32, 32, 16384, 16384, 512, dtype="bf16"),
    "causal16k": _w("causal16k", 5, 1, 32, 32, 16384, 16384, 512, causal=True),
    "nonaligned16k": _w("nonaligned16k", 5, 1, 32, 32, 16383, 16383, 512),
    "bwd16k": _w("bwd16k", 6, 1, 32, 32, 16384, 16384, 512, dtype="bf16", backward=True),
    "bwd16k_causal": _w("bwd16k_causal", 6, 1, 32, 32, 16384, 16384, 512, dtype="bf16",
                        causal=True, backward=True),
})
# the backward of the other rows of the backward tables (bf16, 8K, D = 512)
WORKLOADS.update({
    "bwd_cross": _w("bwd_cross", 4, 1, 32, 32, 1024, 8192, 512, dtype="bf16", backward=True),
    "bwd_decode": _w("bwd_decode", 4, 16, 32, 32, 1, 8192, 512, dtype="bf16", backward=True),
    "bwd_gqa": _w("bwd_gqa", 4, 1, 32, 8, 8192, 8192, 512, dtype="bf16", backward=True),
    "bwd_mask": _w("bwd_mask", 4, 1, 32, 32, 8192, 8192, 512, dtype="bf16", mask="key", backward=True),
    "bwd_nonaligned": _w("bwd_nonaligned", 4, 1, 32, 32, 8191, 8191, 512, dtype="bf16", backward=True),
})
# the "dropout" rows of the same tables (forward and backward), 8K, D = 512
WORKLOADS.update({
    "dropout": _w("dropout", 2, 1, 32, 32, 8192, 8192, 512, dropout_p=0.1),
    "bwd_dropout": _w("bwd_dropout", 4, 1, 32, 32, 8192, 8192, 512, dtype="bf16", backward=True,
                      dropout_p=0.1),
})
# the shapes of the fp8 benchmark of "FFPA Attention Benchmark" ("FP8 and FP4":
# D = 128 at N = 16K and 32K; B and H are not printed, B = 1 and H = 32 as above)
WORKLOADS.update({
    "d128_16k": _w("d128_16k", 7, 1, 32, 32, 16384, 16384, 128),
    "d128_32k": _w("d128_32k", 7, 1, 32, 32, 32768, 32768, 128),
})
# bf16 variants of the variant family (same float32 draws as the fp16 ones)
for _n in ("cross", "gqa", "causal", "nonaligned", "mask", "dropout"):
    WORKLOADS[f"{_n}_bf16"] = WORKLOADS[_n].replace(name=f"{_n}_bf16", dtype="bf16")
for _d in (320, 448, 512, 576, 768, 1024):
    for _acc in ("f32", "f16"):
        WORKLOADS[f"dsweep{_d}_{_acc}"] = _w(f"dsweep{_d}_{_acc}", 3, 1, 32, 32, 8192, 8192, _d,
                                              accum=_acc)


def seed_of(cfg_id: int, t: int, b: int, h: int) -> int:
    return 10 ** 6 * cfg_id + 10 ** 4 * t + 10 ** 2 * b + h


def _slice(seed: int, n: int, d: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(n, d, generator=g, dtype=torch.float32, device=device)


def draw(cfg_id: int, t: int, B: int, H: int, N: int, D: int, dtype: str = "fp16",
         device="cpu") -> torch.Tensor:
    """A [B, H, N, D] tensor in ``dtype``; slice (b, h) from seed_of(cfg_id, t, b, h)."""
    out = torch.empty(B, H, N, D, dtype=DTYPES[dtype], device=device)
    for b in range(B):
        for h in range(H):
            out[b, h] = _slice(seed_of(cfg_id, t, b, h), N, D, device).to(DTYPES[dtype])
    return out


def draw_key_bias(cfg_id: int, nkv: int, dtype: str = "fp16", neg_inf_frac: float = 0.1,
                  rows: int = 1, device="cpu") -> torch.Tensor:
    """Additive mask of shape [rows, Nkv] (rows=1: key bias; rows=Nq: per-query mask).

    N(0, 1) entries; in every row exactly round(neg_inf_frac * Nkv) positions,
    chosen by a seeded permutation, are set to -inf.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(cfg_id, T_MASK, 0, 0))
    vals = torch.randn(rows, nkv, generator=g, dtype=torch.float32)
    n_inf = int(round(neg_inf_frac * nkv))
    for r in range(rows):
        idx = torch.randperm(nkv, generator=g)[:n_inf]
        vals[r, idx] = float("-inf")
    return vals.to(DTYPES[dtype]).to(device)


def make_inputs(w: Workload, device="cpu", with_grad_out: Optional[bool] = None) -> dict:
    """q, k, v (and mask, dout) for workload ``w`` on ``device``."""
    out = {
        "q": draw(w.cfg_id, T_Q, w.B, w.Hq, w.Nq, w.D, w.dtype, device),
        "k": draw(w.cfg_id, T_K, w.B, w.Hkv, w.Nkv, w.D, w.dtype, device),
        "v": draw(w.cfg_id, T_V, w.B, w.Hkv, w.Nkv, w.D, w.dtype, device),
        "mask": None,
    }
    if w.mask is not None:
        rows = 1 if w.mask == "key" else w.Nq
        out["mask"] = draw_key_bias(w.cfg_id, w.Nkv, w.dtype, w.mask_neg_inf_frac, rows, device)
    if with_grad_out if with_grad_out is not None else w.backward:
        out["dout"] = draw(w.cfg_id, T_DO, w.B, w.Hq, w.Nq, w.D, w.dtype, device)
    return out
