"""Pins of the oracle's dropout (CPU only).

The pages show dropout only as benchmark rows ("FFPA Attention Benchmark",
"More Benchmark"); they fix neither the rate nor the random numbers, so the
reading (SDPA's dropout_p semantics, Philox-4x32-10 bytes, threshold
t = round(256 p)) is pinned by what mathematics and statistics fix:

* p = 0 is the undropped attention, bit for bit;
* the keep mask: its rate is (256 - t) / 256 within binomial error, its bytes
  are uniform (chi-square), neighbouring elements are independent, it
  changes with the seed, the head and the position;
* placement: with V = I (Nkv = D) the output row is P o Z c itself, which
  puts each drop at its (query, key) and pins the scale c = 256 / (256 - t);
* E[O] over seeds equals the undropped O (inverted dropout is unbiased);
* the backward: torch float64 autograd of the same dropped product, and
  central finite differences of the oracle's own forward with a fixed seed;
* planted mistakes (unscaled output, transposed mask, dP not masked, the
  scale applied to dV twice, the counter ignoring the head) are rejected.

The Philox block function itself follows the published definition; the pages
print no random numbers, so its bit pattern is pinned against rocRAND's
Philox-4x32-10 in tests/test_oracle_philox.py (the HIP path implements the
same definition independently and must agree with this oracle bit for bit).
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.attention as oracle_mod
from oracle import attn_bwd, attn_fwd, attn_probs, dropout_keep, dropout_threshold, philox4x32_10


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_threshold_is_round_256p():
    assert dropout_threshold(0.0) == 0
    assert dropout_threshold(0.1) == 26
    assert dropout_threshold(0.5) == 128
    assert dropout_threshold(0.999) == 255
    with pytest.raises(ValueError):
        dropout_threshold(1.0)


def test_p_zero_is_the_undropped_attention():
    rng = np.random.default_rng(0)
    q, k, v, do = _rand(rng, 1, 4, 9, 8), _rand(rng, 1, 2, 11, 8), _rand(rng, 1, 2, 11, 8), _rand(rng, 1, 4, 9, 8)
    o0, l0 = attn_fwd(q, k, v, 0.3, causal=True)
    o1, l1 = attn_fwd(q, k, v, 0.3, causal=True, dropout_p=0.0, seed=77)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    for a, b in zip(attn_bwd(q, k, v, do, 0.3), attn_bwd(q, k, v, do, 0.3, dropout_p=0.0, seed=5)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate(p):
    t = dropout_threshold(p)
    keep = dropout_keep(2024, 3, np.arange(1024), np.arange(1024), t)
    n = keep.size
    rate = (256 - t) / 256
    sigma = math.sqrt(rate * (1 - rate) / n)
    assert abs(keep.mean() - rate) < 5 * sigma


def test_bytes_are_uniform_and_independent():
    # all bytes of 2^16 calls: a chi-square over 256 bins, 255 degrees of freedom
    c = np.arange(1 << 16, dtype=np.uint64)
    words = philox4x32_10(c, np.zeros_like(c), np.full_like(c, 7), np.zeros_like(c), 0x1234, 0x5678)
    b = np.concatenate([(w >> np.uint64(8 * s)) & np.uint64(0xFF) for w in words for s in range(4)])
    counts = np.bincount(b.astype(np.int64), minlength=256)
    exp = b.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert 160 < chi2 < 370  # 255 +- ~6 sigma
    # keep decisions of horizontally and vertically adjacent elements are independent
    keep = dropout_keep(99, 0, np.arange(512), np.arange(512), 128).astype(np.float64)
    for a, bb in ((keep[:, :-1], keep[:, 1:]), (keep[:-1, :], keep[1:, :])):
        corr = np.corrcoef(a.ravel(), bb.ravel())[0, 1]
        assert abs(corr) < 5 / math.sqrt(a.size)


def test_mask_changes_with_seed_head_and_position():
    t = 128
    base = dropout_keep(1, 0, np.arange(64), np.arange(64), t)
    assert not np.array_equal(base, dropout_keep(2, 0, np.arange(64), np.arange(64), t))
    assert not np.array_equal(base, dropout_keep(1, 1, np.arange(64), np.arange(64), t))
    assert not np.array_equal(base, dropout_keep(1, 0, np.arange(64) + 64, np.arange(64), t))
    # rows given out of order pick the same elements (the mask is a function of position)
    rows = np.array([5, 3, 60, 0])
    assert np.array_equal(dropout_keep(1, 0, rows, np.arange(64), t), base[rows])
    # the seed's high word matters too
    assert not np.array_equal(base, dropout_keep(1 + (1 << 32), 0, np.arange(64), np.arange(64), t))


def test_identity_values_expose_placement_and_scale():
    # Nkv = D and V = I: O[i, :] = (P o Z c)[i, :], element by element
    rng = np.random.default_rng(1)
    n, p, seed = 24, 0.3, 4242
    q, k = _rand(rng, 1, 2, 20, n), _rand(rng, 1, 2, n, n)
    v = np.broadcast_to(np.eye(n), (1, 2, n, n)).copy()
    o, _ = attn_fwd(q, k, v, 0.25, dropout_p=p, seed=seed)
    P = attn_probs(q, k, 0.25)
    t = dropout_threshold(p)
    for h in range(2):
        keep = dropout_keep(seed, h, np.arange(20), np.arange(n), t)
        assert np.all(o[0, h][~keep] == 0.0)
        np.testing.assert_allclose(o[0, h][keep], P[0, h][keep] * 256 / (256 - t), rtol=1e-12)


def test_dropout_is_unbiased_over_seeds():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 1, 6, 8), _rand(rng, 1, 1, 40, 8), _rand(rng, 1, 1, 40, 8)
    o_ref, _ = attn_fwd(q, k, v, 0.35)
    samples = np.stack([attn_fwd(q, k, v, 0.35, dropout_p=0.25, seed=s)[0] for s in range(400)])
    mean, sem = samples.mean(axis=0), samples.std(axis=0) / math.sqrt(len(samples))
    assert np.all(np.abs(mean - o_ref) <= 6 * sem + 1e-12)


def _torch_dropped(q, k, v, scale, keep_c, causal):
    s = scale * q @ k.transpose(-1, -2)
    if causal:
        n, m = s.shape[-2:]
        s = s.masked_fill(torch.arange(m)[None, :] > torch.arange(n)[:, None], float("-inf"))
    return (torch.softmax(s, dim=-1) * keep_c) @ v


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    # GQA g = 2: the mask of query head h uses bh = h (not its kv head)
    g = torch.Generator().manual_seed(8)
    q = torch.randn(1, 4, 7, 6, generator=g, dtype=torch.float64)
    k = torch.randn(1, 2, 9, 6, generator=g, dtype=torch.float64)
    v = torch.randn(1, 2, 9, 6, generator=g, dtype=torch.float64)
    do = torch.randn(1, 4, 7, 6, generator=g, dtype=torch.float64)
    p, seed = 0.3, 31337
    t = dropout_threshold(p)
    keep_c = torch.stack([torch.from_numpy(np.where(dropout_keep(seed, h, np.arange(7), np.arange(9), t),
                                                    256 / (256 - t), 0.0)) for h in range(4)])[None]
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = _torch_dropped(qa, ka.repeat_interleave(2, 1), va.repeat_interleave(2, 1), 0.4, keep_c, causal)
    out.backward(do)
    o, _ = attn_fwd(q, k, v, 0.4, causal=causal, dropout_p=p, seed=seed)
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12)
    for a, b in zip(attn_bwd(q, k, v, do, 0.4, causal=causal, dropout_p=p, seed=seed), (qa, ka, va)):
        np.testing.assert_allclose(a, b.grad.numpy(), atol=1e-10)


def test_backward_matches_central_differences():
    rng = np.random.default_rng(9)
    q, k, v, do = _rand(rng, 1, 2, 5, 4), _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 2, 5, 4)
    kw = dict(causal=True, dropout_p=0.4, seed=12)
    grads = attn_bwd(q, k, v, do, 0.5, **kw)
    eps = 1e-6
    for x, gx in zip((q, k, v), grads):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fp = (attn_fwd(*args_p, 0.5, **kw)[0] * do).sum()
            fm = (attn_fwd(*args_m, 0.5, **kw)[0] * do).sum()
            fd[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(gx, fd, rtol=1e-6, atol=1e-8)


SRC = inspect.getsource(oracle_mod)
MUTANTS = {
    "output_unscaled": ("p = np.where(keep, p * (256.0 / (256 - t)), 0.0)", "p = np.where(keep, p, 0.0)"),
    "mask_transposed": ("keep = dropout_keep(seed, bh0 + b * Hq + h, pos[r0:r1], np.arange(Nkv), t)\n"
                        "                    p = np.where",
                        "keep = dropout_keep(seed, bh0 + b * Hq + h, np.arange(Nkv), pos[r0:r1], t).T\n"
                        "                    p = np.where"),
    "counter_ignores_head": ("np.full(i.shape, bh, np.uint64)", "np.full(i.shape, 0, np.uint64)"),
    "bwd_dp_not_masked": ("dp = (do @ v[b, hk].T) * zc", "dp = (do @ v[b, hk].T)"),
    "bwd_dv_scaled_twice": ("dv[b, hk] += (p * zc).T @ do", "dv[b, hk] += (p * zc * zc).T @ do"),
}


def _mutant(old, new):
    assert old in SRC, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_dropout_mutant")
    exec(compile(SRC.replace(old, new), "oracle_dropout_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """Compact dropout pins against module ``mod``: placement and scale with
    V = I over two heads, and the backward against torch autograd."""
    rng = np.random.default_rng(11)
    try:
        n, p, seed = 12, 0.3, 4242
        q, k = _rand(rng, 1, 2, 10, n), _rand(rng, 1, 2, n, n)
        v = np.broadcast_to(np.eye(n), (1, 2, n, n)).copy()
        o, _ = mod.attn_fwd(q, k, v, 0.25, dropout_p=p, seed=seed)
        P = attn_probs(q, k, 0.25)
        t = dropout_threshold(p)
        for h in range(2):
            keep = dropout_keep(seed, h, np.arange(10), np.arange(n), t)
            if not np.allclose(o[0, h], np.where(keep, P[0, h] * 256 / (256 - t), 0.0), atol=1e-12):
                return False
        g = torch.Generator().manual_seed(8)
        q = torch.randn(1, 2, 7, 6, generator=g, dtype=torch.float64)
        k = torch.randn(1, 2, 9, 6, generator=g, dtype=torch.float64)
        v = torch.randn(1, 2, 9, 6, generator=g, dtype=torch.float64)
        do = torch.randn(1, 2, 7, 6, generator=g, dtype=torch.float64)
        keep_c = torch.stack([torch.from_numpy(np.where(dropout_keep(seed, h, np.arange(7), np.arange(9), t),
                                                        256 / (256 - t), 0.0)) for h in range(2)])[None]
        qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
        _torch_dropped(qa, ka, va, 0.4, keep_c, False).backward(do)
        for a, b in zip(mod.attn_bwd(q, k, v, do, 0.4, dropout_p=p, seed=seed), (qa, ka, va)):
            if not np.allclose(a, b.grad.numpy(), atol=1e-10):
                return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_the_dropout_pins():
    assert _pins_pass(oracle_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_dropout_pins_reject_planted_mistake(name):
    old, new = MUTANTS[name]
    assert not _pins_pass(_mutant(old, new)), f"dropout pins did not catch mutant {name}"


def test_one_head_alone_with_its_offset_is_that_head():
    # a head (b, h) checked alone takes bh0 = b Hq + h: the same output and
    # gradients as in the whole problem (B = 2, Hq = 3, GQA g = 3)
    rng = np.random.default_rng(11)
    q, k, v, do = (_rand(rng, 2, 3, 9, 8), _rand(rng, 2, 1, 12, 8), _rand(rng, 2, 1, 12, 8),
                   _rand(rng, 2, 3, 9, 8))
    kw = dict(dropout_p=0.4, seed=31)
    o, lse = attn_fwd(q, k, v, 0.3, **kw)
    grads = attn_bwd(q, k, v, do, 0.3, **kw)
    for b, h in [(0, 0), (1, 2), (1, 0)]:
        one = lambda t, hh: t[b:b + 1, hh:hh + 1]
        o1, _ = attn_fwd(one(q, h), one(k, 0), one(v, 0), 0.3, bh0=b * 3 + h, **kw)
        np.testing.assert_array_equal(o1[0, 0], o[b, h])
        dq1, _, _ = attn_bwd(one(q, h), one(k, 0), one(v, 0), one(do, h), 0.3, bh0=b * 3 + h, **kw)
        np.testing.assert_array_equal(dq1[0, 0], grads[0][b, h])
        # without the offset the head would draw head 0's mask
        if b * 3 + h:
            o0, _ = attn_fwd(one(q, h), one(k, 0), one(v, 0), 0.3, **kw)
            assert not np.array_equal(o0[0, 0], o[b, h])
