"""Closed forms, special cases and structural invariants of attention, checked
on the float64 oracle (each is a fact of the mathematics, not of the code).

Forward: Q = 0 gives the mean of V and lse = ln Nkv; causal Q = 0 gives the
prefix mean and lse = ln(i + 1); Nkv = 1 returns V[0]; causal row 0 returns
V[0]; constant V rows return the constant; each softmax row sums to one;
a -inf bias equals deleting those keys; a constant bias shift moves only lse;
GQA equals MHA on repeat_interleave'd K/V ("gqa_4kv", section 3 of the
attention-kernel-profiler design document); rows are independent; permuting
keys (with their values and bias) changes nothing without causality.
Backward: sum_j dK_j = 0, sum_j dV_j = sum over the group's heads and rows of
dO, and Q = 0 gives dV_j = mean_i dO_i.
"""
import math

import numpy as np
import pytest

from oracle import attn_bwd, attn_fwd


def _qkv(seed, B=1, Hq=2, Hkv=2, Nq=24, Nkv=40, D=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, Nq, D)), rng.standard_normal((B, Hkv, Nkv, D)),
            rng.standard_normal((B, Hkv, Nkv, D)), rng)


def test_zero_query_gives_mean_of_v_and_log_n():
    q, k, v, _ = _qkv(1)
    q[:] = 0.0
    o, lse = attn_fwd(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(k.shape[2]), atol=1e-14, rtol=0)


def test_zero_query_causal_gives_prefix_mean():
    q, k, v, _ = _qkv(2, Nq=40, Nkv=40)
    q[:] = 0.0
    o, lse = attn_fwd(q, k, v, 0.25, causal=True)
    pref = np.cumsum(v, axis=2) / np.arange(1, 41)[None, None, :, None]
    np.testing.assert_allclose(o, pref, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 41)), atol=1e-14, rtol=0)


def test_single_key_returns_v0_exactly():
    q, k, v, rng = _qkv(3, Nkv=1)
    mask = rng.standard_normal((1, 1))
    o, lse = attn_fwd(q, k, v, 0.3, mask=mask)
    assert np.array_equal(o, np.broadcast_to(v[:, :, :1], o.shape))
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]) + mask[0, 0],
                               atol=1e-13, rtol=0)


def test_causal_row0_is_v0_exactly():
    q, k, v, _ = _qkv(4, Nq=30, Nkv=30)
    o, lse = attn_fwd(q, k, v, 0.3, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-13, rtol=0)


def test_constant_v_rows_return_the_constant():
    q, k, v, _ = _qkv(5)
    c = np.linspace(-2, 2, v.shape[-1])
    v[:] = c
    o, _ = attn_fwd(q, k, v, 0.7, causal=False)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one_through_lse(causal):
    q, k, v, rng = _qkv(6, Nq=33, Nkv=33)
    mask = rng.standard_normal((1, 33))
    mask[0, 5] = -np.inf
    _, lse = attn_fwd(q, k, v, 0.4, causal=causal, mask=mask)
    s = 0.4 * np.einsum("bhid,bhjd->bhij", q, k) + mask[0]
    if causal:
        s = np.where(np.triu(np.ones((33, 33), bool), 1), -np.inf, s)
    tot = np.exp(s - lse[..., None]).sum(axis=-1)
    np.testing.assert_allclose(tot, 1.0, atol=1e-13, rtol=0)


def test_neg_inf_bias_equals_deleting_keys():
    q, k, v, rng = _qkv(7)
    drop = np.zeros(40, bool)
    drop[rng.permutation(40)[:9]] = True
    mask = np.where(drop, -np.inf, 0.0)[None]
    o, lse = attn_fwd(q, k, v, 0.5, mask=mask)
    o2, lse2 = attn_fwd(q, k[:, :, ~drop], v[:, :, ~drop], 0.5)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


def test_constant_bias_shift_moves_only_lse():
    q, k, v, rng = _qkv(8)
    mask = rng.standard_normal((1, 40))
    o, lse = attn_fwd(q, k, v, 0.5, mask=mask)
    o2, lse2 = attn_fwd(q, k, v, 0.5, mask=mask + 1.75)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse2, lse + 1.75, atol=1e-13)


@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_on_repeat_interleave(g, causal):
    q, k, v, _ = _qkv(9, B=2, Hq=8, Hkv=8 // g, Nq=20, Nkv=20)
    o, lse = attn_fwd(q, k, v, 0.3, causal=causal)
    o2, lse2 = attn_fwd(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.3, causal=causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    do = np.random.default_rng(1).standard_normal(q.shape)
    dq, dk, dv = attn_bwd(q, k, v, do, 0.3, causal=causal)
    dq2, dke, dve = attn_bwd(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, 0.3,
                             causal=causal)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    B, Hkv, N, D = dk.shape
    np.testing.assert_allclose(dk, dke.reshape(B, Hkv, g, N, D).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dve.reshape(B, Hkv, g, N, D).sum(axis=2), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_are_independent(causal):
    q, k, v, rng = _qkv(10, Nq=50, Nkv=50)
    mask = rng.standard_normal((50, 50))
    o, lse = attn_fwd(q, k, v, 0.3, causal=causal, mask=mask)
    rows = np.array([0, 7, 8, 31, 49])
    o2, lse2 = attn_fwd(q[:, :, rows], k, v, 0.3, causal=causal, mask=mask, q_pos=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, :, rows], atol=1e-14)
    # decode: a lone query row against all keys equals that row of the full problem
    o3, _ = attn_fwd(q[:, :, 31:32], k, v, 0.3, causal=False)
    o4, _ = attn_fwd(q, k, v, 0.3, causal=False)
    np.testing.assert_allclose(o3[:, :, 0], o4[:, :, 31], atol=1e-14)


def test_key_permutation_invariance():
    q, k, v, rng = _qkv(11)
    mask = rng.standard_normal((1, 40))
    perm = rng.permutation(40)
    o, lse = attn_fwd(q, k, v, 0.5, mask=mask)
    o2, lse2 = attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.5, mask=mask[:, perm])
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sum_rules(causal):
    q, k, v, rng = _qkv(12, Hq=4, Hkv=2, Nq=30, Nkv=30)
    do = rng.standard_normal(q.shape)
    dq, dk, dv = attn_bwd(q, k, v, do, 0.4, causal=causal)
    # sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # sum_j P_ij = 1, hence sum_j dV_j = sum over the group's heads and rows of dO
    grp = do.reshape(1, 2, 2, 30, -1).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), grp, atol=1e-12)


def test_backward_zero_query_dv_is_mean_of_dout():
    q, k, v, rng = _qkv(13, Nq=10, Nkv=25)
    q[:] = 0.0
    do = rng.standard_normal(q.shape)
    _, _, dv = attn_bwd(q, k, v, do, 0.4)
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=2, keepdims=True) / 25, dv.shape),
                               atol=1e-14)


def test_attn_probs_rows_and_product():
    # the materialised softmax: rows sum to 1 (0 for a dead row) and P V is attn_fwd's O
    from oracle import attn_probs

    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 2, 9, 16))
    k = rng.standard_normal((1, 1, 7, 16))
    v = rng.standard_normal((1, 1, 7, 16))
    mask = rng.standard_normal((1, 7))
    mask[0, 0] = -np.inf
    p = attn_probs(q, k, 0.25, causal=True, mask=mask)
    o, _ = attn_fwd(q, k, v, 0.25, causal=True, mask=mask)
    sums = p.sum(axis=-1)
    assert np.allclose(sums[:, :, 1:], 1.0, atol=1e-12)
    assert np.all(sums[:, :, 0] == 0.0)  # row 0 sees only key 0, which is masked
    assert np.allclose(p @ v[0, 0], o, atol=1e-12)
