"""Float64 CPU oracle for scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` call it. It shares no code with the HIP kernels and their
bindings.

What it computes, and where that is defined:

* The forward is the plain, materialised definition printed under "naive_math"
  in section "3. Attention Variants" of the attention-kernel-profiler design
  document (page "JohnScheuer/attention-kernel-profiler generate_docs.py"):
  scores = Q K^T / sqrt(d_head), optional causal mask, softmax, out = attn V.
  Two generalisations come from "FFPA Attention Benchmark"
  (ffpa-attn.readthedocs.io): the scale is an argument (its default, applied by
  callers, is 1/sqrt(D)), and an additive mask is added to the scaled scores,
  either a key-position bias [1, 1, 1, Nkv] or a per-query bias [1, 1, Nq, Nkv]
  (section "Quick Start").
* Grouped-query attention follows "gqa_4kv" in the same section 3 of the
  profiler document: K/V heads are repeat_interleave'd, so query head h reads
  K/V head h // (Hq / Hkv).
* Readings where the pages are silent (each is listed in the design doc as well):
  causal masking is top-left aligned (query i sees keys j <= i, also when
  Nq != Nkv); a row whose every score is -inf returns O = 0 and lse = -inf;
  lse is the natural-log log-sum-exp of the scaled, masked scores.
* The backward is the gradient of that forward, written out from the chain
  rule of softmax: dV = P^T dO, dP = dO V^T, delta_i = sum_j P_ij dP_ij,
  dS = P * (dP - delta), dQ = scale dS K, dK = scale dS^T Q, with dK and dV
  of a K/V head summed over the query heads that share it (the gradient of
  repeat_interleave). The mask receives no gradient.

All arithmetic is float64. Inputs are the exact fp16/bf16 values widened to
float64; ``scale`` is the float32 value the GPU receives, widened.
The softmax is materialised for blocks of ``row_block`` query rows.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attn_fwd", "attn_bwd", "attn_probs", "to_f64"]


def to_f64(x) -> np.ndarray:
    """Widen a torch tensor (any device, any float dtype) or array to a float64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch  # local: the oracle itself only needs numpy

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v, mask):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nkv, D] with the q batch and D")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if mask is not None and (mask.ndim != 2 or mask.shape[1] != Nkv):
        raise ValueError("mask must be [1, Nkv] (key bias) or [Nq, Nkv] (per query)")
    return B, Hq, Hkv, Nq, Nkv, D


def _scores(qb, kh, scale, mask, causal, rows):
    """Scaled, masked scores for query rows ``rows`` (absolute positions) of one head.

    S = scale * Q K^T, then + mask (broadcast over rows for a key bias), then
    -inf above the top-left causal diagonal (j > i).
    """
    s = scale * (qb @ kh.T)
    if mask is not None:
        s = s + (mask[0][None, :] if mask.shape[0] == 1 else mask[rows, :])
    if causal:
        j = np.arange(kh.shape[0])
        s = np.where(j[None, :] > rows[:, None], -np.inf, s)
    return s


def _softmax_rows(s):
    """Row softmax and log-sum-exp; an all -inf row gives P = 0 and lse = -inf."""
    m = np.max(s, axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked entries
    l = np.sum(e, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(dead[:, None], 0.0, e / np.where(dead, 1.0, l)[:, None])
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return p, lse


def attn_fwd(q, k, v, scale, causal=False, mask=None, q_pos=None, row_block=1024):
    """O = softmax(scale * Q K^T + mask) V and the per-row log-sum-exp.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nkv, D]; mask: None, [1, Nkv] or [Nq_total, Nkv].
    q_pos: absolute query positions of the Nq rows given (default 0..Nq-1);
    they select the causal diagonal and the per-query mask rows, so a subset
    of rows can be checked on its own (rows are independent).
    Returns (o [B, Hq, Nq, D], lse [B, Hq, Nq]) as float64.
    """
    q, k, v, mask = to_f64(q), to_f64(k), to_f64(v), to_f64(mask)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v, mask)
    g = Hq // Hkv
    pos = np.arange(Nq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    scale = float(scale)
    o = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                s = _scores(q[b, h, r0:r1], k[b, hk], scale, mask, causal, pos[r0:r1])
                p, lse[b, h, r0:r1] = _softmax_rows(s)
                o[b, h, r0:r1] = p @ v[b, hk]
    return o, lse


def attn_bwd(q, k, v, dout, scale, causal=False, mask=None, row_block=1024):
    """Gradients (dq, dk, dv) of sum(dout * attn_fwd(q, k, v)[0]) in float64.

    P is recomputed from q, k, v here; nothing from a GPU forward is used.
    dk, dv of K/V head hk accumulate over the query heads h with h // g == hk.
    """
    q, k, v, dout, mask = to_f64(q), to_f64(k), to_f64(v), to_f64(dout), to_f64(mask)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v, mask)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    g = Hq // Hkv
    pos = np.arange(Nq)
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                s = _scores(q[b, h, r0:r1], k[b, hk], scale, mask, causal, pos[r0:r1])
                p, _ = _softmax_rows(s)
                do = dout[b, h, r0:r1]
                dv[b, hk] += p.T @ do
                dp = do @ v[b, hk].T
                delta = np.sum(p * dp, axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, h, r0:r1] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def attn_probs(q, k, scale, causal=False, mask=None):
    """The materialised softmax P [B, Hq, Nq, Nkv] (float64) of attn_fwd.

    For small shapes only (P is held whole). Tests use it to size rounding
    bounds; it is the same _scores/_softmax_rows path attn_fwd takes.
    """
    q, k, mask = to_f64(q), to_f64(k), to_f64(mask)
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    pos = np.arange(Nq)
    p = np.zeros((B, Hq, Nq, Nkv))
    for b in range(B):
        for h in range(Hq):
            s = _scores(q[b, h], k[b, h // g], float(scale), mask, causal, pos)
            p[b, h], _ = _softmax_rows(s)
    return p
