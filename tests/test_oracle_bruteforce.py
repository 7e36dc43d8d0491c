"""Pin the float64 oracle to a literal per-element definition on tiny inputs.

The brute force below is written independently of ``oracle.attention``: pure
Python loops, ``math.fsum`` for every sum and ``math.exp``/``math.log``,
following the "naive_math" definition in section "3. Attention Variants" of the
attention-kernel-profiler design document (scores = QK^T scale, mask, softmax,
attn V) with the additive mask of "FFPA Attention Benchmark" ("Quick Start")
and the repeat_interleave head map of "gqa_4kv" (same section 3).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import attn_fwd

NEG_INF = float("-inf")


def brute_fwd(q, k, v, scale, causal, mask):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    o = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Nq):
                s = []
                for j in range(Nkv):
                    dot = math.fsum(float(q[b, h, i, d]) * float(k[b, hk, j, d]) for d in range(D))
                    val = scale * dot
                    if mask is not None:
                        val = val + float(mask[0 if mask.shape[0] == 1 else i, j])
                    if causal and j > i:
                        val = NEG_INF
                    s.append(val)
                mx = max(s)
                if mx == NEG_INF:
                    lse[b, h, i] = NEG_INF
                    continue
                e = [math.exp(x - mx) if x != NEG_INF else 0.0 for x in s]
                tot = math.fsum(e)
                lse[b, h, i] = mx + math.log(tot)
                for d in range(D):
                    o[b, h, i, d] = math.fsum(e[j] / tot * float(v[b, hk, j, d]) for j in range(Nkv))
    return o, lse


def _rand(rng, *shape):
    return rng.standard_normal(shape)


CASES = list(itertools.product(
    [(1, 2, 2), (2, 4, 2), (1, 4, 1)],  # (B, Hq, Hkv)
    [(5, 5), (3, 7), (7, 3), (1, 6), (4, 1)],  # (Nq, Nkv)
    [False, True],  # causal
    [None, "key", "query"],  # mask
))


@pytest.mark.parametrize("bh,n,causal,mask_kind", CASES)
def test_oracle_matches_brute_force(bh, n, causal, mask_kind):
    B, Hq, Hkv = bh
    Nq, Nkv = n
    D = 6
    rng = np.random.default_rng(1000 * Nq + 10 * Nkv + Hq)
    q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D)
    mask = None
    if mask_kind is not None:
        rows = 1 if mask_kind == "key" else Nq
        mask = _rand(rng, rows, Nkv)
        if Nkv > 1:
            mask[rng.random((rows, Nkv)) < 0.3] = NEG_INF
    scale = 0.37
    o, lse = attn_fwd(q, k, v, scale, causal=causal, mask=mask)
    ob, lseb = brute_fwd(q, k, v, scale, causal, mask)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lseb))
    fin = np.isfinite(lseb)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


def test_fully_masked_rows_give_zero_and_neg_inf():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 5, 4)
    mask = np.zeros((3, 5))
    mask[1, :] = NEG_INF  # row 1 sees nothing
    o, lse = attn_fwd(q, k, v, 0.5, mask=mask)
    ob, lseb = brute_fwd(q, k, v, 0.5, False, mask)
    assert lse[0, 0, 1] == NEG_INF and lseb[0, 0, 1] == NEG_INF
    assert np.all(o[0, 0, 1] == 0.0)
    np.testing.assert_allclose(o, ob, atol=1e-12, rtol=0)


def test_causal_decode_row_sees_key_zero_only():
    # Top-left causal alignment with Nq = 1: the lone query (position 0) sees key 0.
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 1, 8), _rand(rng, 1, 2, 9, 8), _rand(rng, 1, 2, 9, 8)
    o, lse = attn_fwd(q, k, v, 0.3, causal=True)
    np.testing.assert_array_equal(o[0, :, 0], v[0, :, 0])
    np.testing.assert_allclose(lse[0, :, 0], 0.3 * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]),
                               atol=1e-14, rtol=0)
