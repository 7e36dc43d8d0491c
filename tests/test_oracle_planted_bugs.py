"""Mutation check of the oracle's pins: plant a plausible mistake in a copy of
the oracle (on the CPU, by editing its source text), and show that the pins
(brute force, torch float64 SDPA/autograd, closed forms) reject the mutant.
A pin set that let any of these through would be too weak to trust.
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as oracle_mod
from test_oracle_bruteforce import brute_fwd

SRC = inspect.getsource(oracle_mod)

MUTANTS = {
    "gqa_map_modulo": ("hk = h // g", "hk = h % Hkv"),
    "dropped_scale": ("s = scale * (qb @ kh.T)", "s = (qb @ kh.T)"),
    "causal_off_by_one": ("j[None, :] > rows[:, None]", "j[None, :] >= rows[:, None]"),
    "mask_sign": ("s = s + (mask[0][None, :]", "s = s - (mask[0][None, :]"),
    "query_mask_rows": ("else mask[rows, :])", "else mask[::-1][rows, :])"),
    "pv_wrong_operand": ("o[b, h, r0:r1] = p @ v[b, hk]", "o[b, h, r0:r1] = p @ k[b, hk]"),
    "lse_dropped_log": ("m_safe + np.log(np.where(dead, 1.0, l))", "m_safe + 0.0 * l"),
    "softmax_unnormalised": ("e / np.where(dead, 1.0, l)[:, None]", "e"),
    "bwd_dropped_delta": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "bwd_dv_no_group_sum": ("dv[b, hk] += (p * zc).T @ do", "dv[b, hk] = (p * zc).T @ do"),
    "bwd_dk_dropped_scale": ("dk[b, hk] += scale * (ds.T", "dk[b, hk] += (ds.T"),
    "bwd_dq_transposed": ("dq[b, h, r0:r1] = scale * (ds @ k[b, hk])",
                          "dq[b, h, r0:r1] = scale * (ds @ v[b, hk])"),
}


def _mutant(old, new):
    assert old in SRC, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    """A compact run of the pins against ``mod``; False as soon as one fails."""
    rng = np.random.default_rng(5)
    try:
        # brute force: GQA + cross + causal + key bias + per-query mask
        for causal, mk in ((False, "key"), (True, "query"), (True, None)):
            q = rng.standard_normal((1, 4, 5, 3))
            k = rng.standard_normal((1, 2, 6, 3))
            v = rng.standard_normal((1, 2, 6, 3))
            mask = None if mk is None else rng.standard_normal((1 if mk == "key" else 5, 6))
            o, lse = mod.attn_fwd(q, k, v, 0.45, causal=causal, mask=mask)
            ob, lseb = brute_fwd(q, k, v, 0.45, causal, mask)
            if not (np.allclose(o, ob, atol=1e-10) and np.allclose(lse, lseb, atol=1e-10)):
                return False
        # backward vs autograd on SDPA (GQA, causal)
        for causal in (False, True):
            g = torch.Generator().manual_seed(3)
            q = torch.randn(1, 4, 6, 5, generator=g, dtype=torch.float64)
            k = torch.randn(1, 2, 6, 5, generator=g, dtype=torch.float64)
            v = torch.randn(1, 2, 6, 5, generator=g, dtype=torch.float64)
            do = torch.randn(1, 4, 6, 5, generator=g, dtype=torch.float64)
            qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
            F.scaled_dot_product_attention(qa, ka.repeat_interleave(2, 1), va.repeat_interleave(2, 1),
                                           is_causal=causal, scale=0.4).backward(do)
            dq, dk, dv = mod.attn_bwd(q, k, v, do, 0.4, causal=causal)
            for a, b in ((dq, qa.grad), (dk, ka.grad), (dv, va.grad)):
                if not np.allclose(a, b.numpy(), atol=1e-10):
                    return False
        # closed form: Q = 0 gives mean of V, lse = ln Nkv
        q = np.zeros((1, 1, 3, 4))
        k = rng.standard_normal((1, 1, 9, 4))
        v = rng.standard_normal((1, 1, 9, 4))
        o, lse = mod.attn_fwd(q, k, v, 0.5)
        if not (np.allclose(o, v.mean(axis=2, keepdims=True)) and np.allclose(lse, math.log(9))):
            return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_the_compact_pins():
    assert _pins_pass(oracle_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    old, new = MUTANTS[name]
    assert not _pins_pass(_mutant(old, new)), f"pins did not catch mutant {name}"
