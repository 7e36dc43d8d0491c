"""Parity of the fp8 forward (ffpa_attn_fwd_fp8, HIP through the C ABI)
against oracle/fp8.py, the quantised attention the header specifies.

Both sides quantise Q, K and V identically (per-head amax in float32, the
product in float32, e4m3 round to nearest even) and quantise P against the
same per-row running reference (blocks of 64 keys, rise by more than 2.5 ln 2),
so the kernel differs from the oracle only in its arithmetic: the
matrix core's sums of exact fp8 products, the fast exp2, and the decisions
these move (a P on an e4m3 rounding tie, a block maximum at the rise
threshold). Such a decision moves one quantised p by one e4m3 step, at most
2^-3 of p, so the element bound is
    |O - O*| <= 2^-3 sum_j p_j |v8_j| (amax_V / 448) / l  +  u |O*|  +  1e-4,
the first term computed by the oracle itself on |V| (|V| quantises to the
magnitudes of V's codes), u the unit roundoff of the output type. Such flips
are rare, so the relative L2 error is held to 1e-2 (observed about 1e-3).
lse within 2e-3. The distance to the exact (unquantised) attention is printed
beside it (about 5 % at these sizes: e4m3's own rounding).

A power-of-two ramp (every quantised P exact) must match the exact attention
to the output rounding plus the matrix core's own summation error: the fp8
MFMA (32x32x64) adds its 64 products with an internal adder that truncates
each product about 17 bits below the largest one (measured: 448 + 63 x 2^-9
comes out as 448.109, 448^2 + 63 x 1.125 as 200767), so one instruction's
sum is off by at most 64 x 2^-17 = 2^-11 of the sum of its |products|; over
the 64-key tiles that is at most 2^-11 sum_j p_j |v_j| / l, and the test
allows twice that.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attn_fwd, to_f64
from oracle.fp8 import attn_fwd_fp8

pytestmark = pytest.mark.gpu

UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype):
    return (W.draw(seed, W.T_Q, B, Hq, Nq, D, dtype), W.draw(seed, W.T_K, B, Hkv, Nkv, D, dtype),
            W.draw(seed, W.T_V, B, Hkv, Nkv, D, dtype))


def check(o, lse, q, k, v, scale, causal, dtype, label, heads=None):
    """Compare o, lse (the kernel's) with the oracle on the given (b, h) heads
    (default all), each with its own kv head."""
    B, Hq = q.shape[:2]
    g = Hq // k.shape[1]
    heads = heads or [(b, h) for b in range(B) for h in range(Hq)]
    sq_e = sq_r = worst = worst_l = 0.0
    exact_e = 0.0
    for b, h in heads:
        hk = h // g
        qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1]
        oo, lo = attn_fwd_fp8(qs, ks, vs, scale, causal=causal)
        pv, _ = attn_fwd_fp8(qs, ks, to_f64(vs).__abs__(), scale, causal=causal)
        og, lg = to_f64(o[b, h]), to_f64(lse[b, h])
        assert np.isfinite(og).all(), f"{label}: non-finite output"
        d = np.abs(og - oo[0, 0])
        bound = 2.0 ** -3 * pv[0, 0] + UNIT[dtype] * np.abs(oo[0, 0]) + 1e-4
        worst = max(worst, float((d / bound).max()))
        sq_e += float((d * d).sum())
        sq_r += float((oo[0, 0] ** 2).sum())
        fin = np.isfinite(lo[0, 0])
        worst_l = max(worst_l, float(np.abs(lg[fin] - lo[0, 0][fin]).max()) if fin.any() else 0.0)
        ex, _ = attn_fwd(qs, ks, vs, scale, causal=causal)
        exact_e = max(exact_e, float(np.linalg.norm(og - ex[0, 0]) / max(np.linalg.norm(ex[0, 0]), 1e-30)))
    rel = (sq_e / max(sq_r, 1e-30)) ** 0.5
    print(f"{label}: err/bound={worst:.3f} relL2={rel:.3e} max|dlse|={worst_l:.3e} "
          f"relL2 to exact attention={exact_e:.3e}", flush=True)
    assert worst <= 1.0, f"{label}: error exceeds the bound by {worst:.3f}x"
    assert rel <= 1e-2, f"{label}: rel L2 {rel}"
    assert worst_l <= 2e-3, f"{label}: lse error {worst_l}"


CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 200, 150, 320),
    (1, 4, 1, 300, 257, 512),   # GQA g = 4, ragged
    (2, 2, 2, 130, 200, 128),
    (1, 2, 2, 64, 64, 448),
    (1, 3, 1, 100, 1000, 192),  # Nkv > Nq, GQA g = 3
    (1, 2, 2, 1, 77, 256),      # one query row
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_matches_oracle(lib, shape, dtype, causal):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v = _inputs(500 + D + Nkv, B, Hq, Hkv, Nq, Nkv, D, dtype)
    scale = 1.0 / math.sqrt(D)
    o, lse = lib.attention_fp8(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    check(o.cpu(), lse.cpu(), q, k, v, scale, causal, dtype, f"fp8 {shape} {dtype} causal={causal}")


def test_fp8_zero_query_and_zero_values(lib):
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 96, 200, 256
    q, k, v = _inputs(9, B, Hq, Hkv, Nq, Nkv, D, "fp16")
    q = torch.zeros_like(q)
    v[:, 1] = 0  # an all-zero head: codes 0, scale 1
    o, lse = lib.attention_fp8(q.cuda(), k.cuda(), v.cuda(), return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.count_nonzero(o[:, 1]).item() == 0
    np.testing.assert_allclose(to_f64(lse), math.log(Nkv), atol=2e-4)
    check(o, lse, q, k, v, 1.0 / math.sqrt(D), False, "fp16", "fp8 Q = 0")


def test_fp8_power_of_two_ramp_is_exact(lib):
    """Scores c ln 2 with integer c whose 64-key block maxima rise by 3 from
    each block to the next (K[:, 0] = 16 c with a 448 pin in another column,
    so K is its own e4m3 code; Q = e_0; scale = ln 2 / 16; V on its grid): the
    running reference rises at every tile by exactly 3 ln 2 (past the 2.5 ln 2
    threshold), every quantised P is an exact power of two, so O is the exact
    attention (to the output's rounding and the matrix core's summation) and
    lse = ln sum 2^c. The rows span several tiles and a ragged tail (Nkv is
    not a multiple of 64; the last block is cut short)."""
    B, H, Nq, N, D = 1, 2, 96, 300, 128
    rng = np.random.default_rng(11)
    c = np.array([3 * (j // 64) - (j % 64) % 4 for j in range(N)], dtype=np.float64)
    k = np.zeros((B, H, N, D))
    k[..., 0] = 16 * c
    k[..., 0, 1] = 448.0
    q = np.zeros((B, H, Nq, D))
    q[..., 0] = 1.0
    codes = np.array([m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                      for e in range(16) for m in range(8) if not (e == 15 and m == 7)])
    v = rng.choice(np.concatenate([codes, -codes]), size=(B, H, N, D)) * 2.0 ** -5
    v[..., 0, 0] = 448 * 2.0 ** -5
    qt, kt, vt = (torch.from_numpy(x).to(torch.float16) for x in (q, k, v))
    assert np.array_equal(vt.double().numpy(), v) and np.array_equal(kt.double().numpy(), k)
    scale = math.log(2.0) / 16
    o, lse = lib.attention_fp8(qt.cuda(), kt.cuda(), vt.cuda(), scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ref, lref = attn_fwd(qt, kt, vt, scale)
    og = to_f64(o.cpu())
    err = np.abs(og - ref)
    print(f"power-of-two ramp: max|dO|={err.max():.3e} max|dlse|={np.abs(to_f64(lse.cpu()) - lref).max():.3e}")
    pv_abs, _ = attn_fwd(qt, kt, vt.abs(), scale)
    assert np.all(err <= UNIT["fp16"] * np.abs(ref) + 2.0 ** -10 * pv_abs + 1e-6)
    np.testing.assert_allclose(to_f64(lse.cpu()), lref, atol=1e-5)


def test_fp8_validation(lib):
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(lib.FFPAError):
        lib.attention_fp8(q, q, q)  # D = 64 is not built for fp8
    q = torch.zeros(1, 2, 8, 576, dtype=torch.float16, device="cuda")
    with pytest.raises(lib.FFPAError):
        lib.attention_fp8(q, q, q)


@pytest.mark.parametrize("name", ["self", "self_bf16", "d128_16k"])
def test_fp8_full_size(lib, name):
    """The benchmark workloads (B1 H32 N8192 D512, and the pages' fp8 shape
    B1 H32 D128 at N = 16K): two whole heads. (At 32K the oracle's score
    matrix of one head alone takes 8 GiB of float64.)"""
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device="cuda")
    o, lse = lib.attention_fp8(inp["q"], inp["k"], inp["v"], scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (w.B - 1, w.Hq - 1)]
    sl = lambda t, h: t[:, h:h + 1].cpu()
    for b, h in heads:
        check(o[:, h:h + 1].cpu(), lse[:, h:h + 1].cpu(), sl(inp["q"], h), sl(inp["k"], h), sl(inp["v"], h),
              w.scale, False, w.dtype, f"fp8 {name} head {h}")
