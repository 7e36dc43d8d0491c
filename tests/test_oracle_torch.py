"""Pin the float64 oracle to library routines: torch's CPU float64
scaled_dot_product_attention (forward), torch.logsumexp (lse) and
torch.autograd (backward), plus central finite differences of the oracle's
own forward for the backward.

torch's ``is_causal`` masks j > i (top-left), the reading the oracle takes;
its float ``attn_mask`` is added to the scaled scores, the additive-mask
convention of "FFPA Attention Benchmark" ("Quick Start").
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn_bwd, attn_fwd


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, mask_kind):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, Nq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, Nkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, Nkv, D, generator=g, dtype=torch.float64)
    do = torch.randn(B, Hq, Nq, D, generator=g, dtype=torch.float64)
    mask = None
    if mask_kind is not None:
        rows = 1 if mask_kind == "key" else Nq
        mask = torch.randn(rows, Nkv, generator=g, dtype=torch.float64)
        # -inf on a few keys, never a whole row (torch would return NaN there)
        mask[:, ::7] = float("-inf")
    return q, k, v, do, mask


def _torch_ref(q, k, v, scale, causal, mask):
    g = q.shape[1] // k.shape[1]
    ke = k.repeat_interleave(g, dim=1)
    ve = v.repeat_interleave(g, dim=1)
    am = None if mask is None else mask[None, None]
    o = F.scaled_dot_product_attention(q, ke, ve, attn_mask=am, is_causal=causal, scale=scale)
    s = scale * (q @ ke.transpose(-1, -2))
    if am is not None:
        s = s + am
    if causal:
        Nq, Nkv = q.shape[2], k.shape[2]
        s = s.masked_fill(torch.ones(Nq, Nkv, dtype=torch.bool).triu(1), float("-inf"))
    return o, torch.logsumexp(s, dim=-1)


SHAPES = [
    (1, 2, 2, 64, 64, 32),
    (2, 4, 2, 37, 91, 48),   # GQA, cross, ragged
    (1, 8, 2, 80, 80, 64),   # GQA g = 4
    (1, 2, 1, 1, 130, 40),   # decode-like
    (1, 2, 2, 129, 33, 16),  # Nq > Nkv
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mask_kind", [None, "key", "query"])
def test_forward_matches_torch_sdpa_f64(shape, causal, mask_kind):
    B, Hq, Hkv, Nq, Nkv, D = shape
    if causal and mask_kind is not None:
        pass  # both combine fine; covered
    q, k, v, _, mask = _inputs(sum(shape), B, Hq, Hkv, Nq, Nkv, D, mask_kind)
    if causal and mask is not None:
        mask[:, 0] = 0.0  # key 0 stays visible so no row is fully masked
    scale = 1.0 / np.sqrt(D)
    o, lse = attn_fwd(q, k, v, scale, causal=causal, mask=mask, row_block=17)
    ot, lset = _torch_ref(q, k, v, scale, causal, mask)
    np.testing.assert_allclose(o, ot.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(lse, lset.numpy(), atol=1e-10, rtol=0)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mask_kind", [None, "key"])
def test_backward_matches_torch_autograd_f64(shape, causal, mask_kind):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v, do, mask = _inputs(7 + sum(shape), B, Hq, Hkv, Nq, Nkv, D, mask_kind)
    if causal and mask is not None:
        mask[:, 0] = 0.0
    scale = 0.9 / np.sqrt(D)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    ot, _ = _torch_ref(qa, ka, va, scale, causal, mask)
    ot.backward(do)
    dq, dk, dv = attn_bwd(q, k, v, do, scale, causal=causal, mask=mask, row_block=19)
    np.testing.assert_allclose(dq, qa.grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(dk, ka.grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(dv, va.grad.numpy(), atol=1e-10, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Nq, Nkv, D = 1, 4, 2, 4, 5, 3
    q = rng.standard_normal((B, Hq, Nq, D))
    k = rng.standard_normal((B, Hkv, Nkv, D))
    v = rng.standard_normal((B, Hkv, Nkv, D))
    do = rng.standard_normal((B, Hq, Nq, D))
    mask = rng.standard_normal((1, Nkv))
    scale = 0.61
    dq, dk, dv = attn_bwd(q, k, v, do, scale, causal=causal, mask=mask)

    def loss(q_, k_, v_):
        return float(np.sum(do * attn_fwd(q_, k_, v_, scale, causal=causal, mask=mask)[0]))

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)
