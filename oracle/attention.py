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

* Dropout (the "dropout" rows of the benchmark tables of "FFPA Attention
  Benchmark", section "More Benchmark"; the pages name neither the rate nor
  the random numbers). Reading: as PyTorch SDPA's dropout_p, which the pages
  compare against, the attention probabilities are dropped after the softmax
  and before the product with V, the kept ones scaled up by the inverse of
  the keep probability; the logsumexp is that of the undropped scores. The
  random numbers come from the counter-based generator Philox-4x32-10
  (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
  3", SC 2011), keyed by the 64-bit seed: one call per block of 4 query rows
  x 4 keys of a head, counter (j // 4, i // 4, b * Hq + h, 0), one byte per
  element (word i % 4, byte j % 4 of the output). An element is kept when its
  byte is >= t = round(256 p) (keep probability (256 - t) / 256) and kept
  elements are scaled by 256 / (256 - t).

All arithmetic is float64. Inputs are the exact fp16/bf16 values widened to
float64; ``scale`` is the float32 value the GPU receives, widened.
The softmax is materialised for blocks of ``row_block`` query rows.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attn_fwd", "attn_bwd", "attn_probs", "to_f64", "philox4x32_10", "dropout_threshold",
           "dropout_keep"]


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


# Philox-4x32-10 (Salmon et al., SC 2011): a 4-word counter and a 2-word key;
# each of the 10 rounds multiplies two counter words by fixed odd constants,
# recombines the 64-bit products' halves with the other two words and the key,
# and the key is bumped by two further constants ("Weyl" increments) between
# rounds.
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox-4x32-10 of counters (c0, c1, c2, c3) (arrays of equal shape) under
    the key (k0, k1); returns the four 32-bit output words as uint64 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0) & _MASK32, np.uint64(k1) & _MASK32
    for _ in range(10):
        p0 = np.uint64(_PHILOX_M[0]) * c[0]  # < 2^64: both factors are below 2^32
        p1 = np.uint64(_PHILOX_M[1]) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _MASK32, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & _MASK32]
        k0 = (k0 + np.uint64(_PHILOX_W[0])) & _MASK32
        k1 = (k1 + np.uint64(_PHILOX_W[1])) & _MASK32
    return c


def dropout_threshold(p):
    """t = round(256 p) for the float32 value of p: an element is dropped when
    its random byte is below t."""
    p = float(np.float32(p))
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(256.0 * p + 0.5)), 255)


def dropout_keep(seed, bh, rows, cols, t):
    """Keep mask [len(rows), len(cols)] of head bh = b Hq + h: element (i, j) is
    kept when byte j % 4 of word i % 4 of Philox(j // 4, i // 4, bh, 0; seed)
    is at least t."""
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.asarray(cols, dtype=np.uint64)[None, :]
    i, j = np.broadcast_arrays(i, j)
    words = philox4x32_10(j >> np.uint64(2), i >> np.uint64(2), np.full(i.shape, bh, np.uint64),
                          np.zeros(i.shape, np.uint64), int(seed) & 0xFFFFFFFF, int(seed) >> 32)
    w = np.choose((i & np.uint64(3)).astype(np.int64), words)
    byte = (w >> (np.uint64(8) * (j & np.uint64(3)))) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def attn_fwd(q, k, v, scale, causal=False, mask=None, q_pos=None, row_block=1024, dropout_p=0.0,
             seed=0, bh0=0):
    """O = softmax(scale * Q K^T + mask) V and the per-row log-sum-exp.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nkv, D]; mask: None, [1, Nkv] or [Nq_total, Nkv].
    q_pos: absolute query positions of the Nq rows given (default 0..Nq-1);
    they select the causal diagonal, the per-query mask rows and the dropout
    counters, so a subset of rows can be checked on its own (rows are
    independent).
    dropout_p, seed: the dropout of the module docstring (0: none). The
    counter of head (b, h) given is bh0 + b Hq + h: bh0 = 0 for a whole
    problem; a single head (b', h') of a larger one, passed alone, takes
    bh0 = b' Hq' + h' (its place in that problem).
    Returns (o [B, Hq, Nq, D], lse [B, Hq, Nq]) as float64.
    """
    q, k, v, mask = to_f64(q), to_f64(k), to_f64(v), to_f64(mask)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v, mask)
    g = Hq // Hkv
    pos = np.arange(Nq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    scale = float(scale)
    t = dropout_threshold(dropout_p)
    o = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                s = _scores(q[b, h, r0:r1], k[b, hk], scale, mask, causal, pos[r0:r1])
                p, lse[b, h, r0:r1] = _softmax_rows(s)
                if t > 0:
                    keep = dropout_keep(seed, bh0 + b * Hq + h, pos[r0:r1], np.arange(Nkv), t)
                    p = np.where(keep, p * (256.0 / (256 - t)), 0.0)
                o[b, h, r0:r1] = p @ v[b, hk]
    return o, lse


def attn_bwd(q, k, v, dout, scale, causal=False, mask=None, row_block=1024, dropout_p=0.0, seed=0,
             bh0=0):
    """Gradients (dq, dk, dv) of sum(dout * attn_fwd(q, k, v)[0]) in float64.

    P is recomputed from q, k, v here; nothing from a GPU forward is used.
    dk, dv of K/V head hk accumulate over the query heads h with h // g == hk.
    With dropout (keep mask Z, scale c = 256 / (256 - t)) the output is
    (P o Z c) V, so dV = (P o Z c)^T dO, dP = (dO V^T) o Z c, and the rest as
    without: delta_i = sum_j P_ij dP_ij, dS = P o (dP - delta). bh0: as in
    attn_fwd.
    """
    q, k, v, dout, mask = to_f64(q), to_f64(k), to_f64(v), to_f64(dout), to_f64(mask)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v, mask)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    g = Hq // Hkv
    pos = np.arange(Nq)
    scale = float(scale)
    t = dropout_threshold(dropout_p)
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
                zc = 1.0
                if t > 0:
                    keep = dropout_keep(seed, bh0 + b * Hq + h, pos[r0:r1], np.arange(Nkv), t)
                    zc = np.where(keep, 256.0 / (256 - t), 0.0)
                dv[b, hk] += (p * zc).T @ do
                dp = (do @ v[b, hk].T) * zc
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
