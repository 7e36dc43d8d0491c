"""Pins of the fp8 oracle (oracle/fp8.py), CPU only.

* e4m3 rounding against a brute-force search over all 256 codes (OCP e4m3:
  bias 7, 3 mantissa bits, subnormals from 2^-9, largest finite 448): nearest
  value, ties to the even code; known values; every code is a fixed point.
* Per-head quantisation: the largest element maps to +-448 exactly, every
  code stays in range, the relative error of normal values is <= 2^-4.
* Closed forms of the quantised attention: Q = 0 gives P = 1 (64 P exact),
  so O is the mean of the dequantised V and lse = ln Nkv; with V on the e4m3
  grid of its own scale (amax = 448 * 2^k) that mean is the plain mean of V.
  One key: O = V[0] (on the grid) and lse = the dequantised score.
* Against the exact float64 attention (oracle/attention.py) on N(0, 1) data:
  the quantised result is attention to within the fp8 rounding (relative L2
  about 5 %, gate 10 %), causal and GQA included.
* The running reference: scores c ln 2 (integer c) whose block maxima rise by
  3 ln 2 from block to block (past the 2.5 ln 2 threshold), with Q, K and V
  on their e4m3 grids, make every quantised P and every rescale exact: the
  result must be the exact attention to float64 rounding.
* Planted mistakes (a dropped K dequantisation factor, the P scale not taken
  out, ties rounded away from zero, the row sum over quantised P replaced by
  its square, O not rescaled when the reference rises) are rejected by these
  pins.
"""
import inspect
import math
import types

import numpy as np
import pytest

import oracle.fp8 as fp8_mod
from oracle import attn_fwd
from oracle.fp8 import attn_fwd_fp8, e4m3_round, quantize_head


def e4m3_codes():
    """All finite e4m3 values, from the bit layout."""
    vals = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue  # NaN
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append((-v if s else v, c))
    return vals


def brute_round(x):
    best, bc, bd = 0.0, 0, math.inf
    for v, c in e4m3_codes():
        d = abs(v - x)
        if d < bd or (d == bd and (c & 1) == 0 and (bc & 1) == 1):
            best, bc, bd = v, c, d
    return math.copysign(abs(best), x) if best == 0 else best


def test_rounding_matches_brute_force():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.uniform(-448, 448, 400), rng.normal(0, 1, 400), rng.normal(0, 0.01, 200),
                         2.0 ** rng.uniform(-12, 8.7, 300) * rng.choice([-1, 1], 300)])
    # ties: midpoints between neighbouring codes
    pos = sorted({v for v, _ in e4m3_codes() if v >= 0})
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    xs = np.concatenate([xs, mids, -np.array(mids)])
    got = e4m3_round(xs)
    want = np.array([brute_round(float(x)) for x in xs])
    assert np.array_equal(got, want)


def test_known_values_and_fixed_points():
    assert e4m3_round(448.0) == 448.0
    assert e4m3_round(1.0625) == 1.0     # tie between 1 (even) and 1.125
    assert e4m3_round(1.1875) == 1.25    # tie between 1.125 and 1.25 (even)
    assert e4m3_round(2.0 ** -9) == 2.0 ** -9   # smallest subnormal
    assert e4m3_round(2.0 ** -10) == 0.0        # half of it: tie to 0
    assert e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8  # 1.5 steps: tie to the even 2 steps
    vals = np.array([v for v, _ in e4m3_codes()])
    assert np.array_equal(e4m3_round(vals), vals)
    assert len({v for v in vals if v > 0}) == 126 and vals.max() == 448.0


def test_quantize_head_range_and_error():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, (64, 48)).astype(np.float16)
    x8, amax = quantize_head(x)
    assert amax == float(np.abs(x.astype(np.float32)).max())
    assert np.abs(x8).max() == 448.0
    s = np.float32(448) / np.float32(amax)
    y = np.asarray(x, np.float32).astype(np.float64) * float(s)
    normal = np.abs(y) >= 2.0 ** -6
    assert np.all(np.abs(x8[normal] - y[normal]) <= 2.0 ** -4 * np.abs(y[normal]) * (1 + 1e-6))
    z8, za = quantize_head(np.zeros((4, 8), np.float16))
    assert za == 0.0 and not np.any(z8)


def _grid_v(rng, shape, k=-5):
    """Values on the e4m3 grid of a head whose amax is 448 * 2^k (scale 2^-k exact)."""
    codes = np.array([v for v, _ in e4m3_codes()])
    v = rng.choice(codes, size=shape) * 2.0 ** k
    v.reshape(-1)[0] = 448 * 2.0 ** k  # pin the amax
    return v


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(2)
    B, H, Nq, Nkv, D = 1, 2, 5, 37, 16
    q = np.zeros((B, H, Nq, D))
    k = rng.normal(size=(B, H, Nkv, D))
    v = np.stack([[_grid_v(rng, (Nkv, D)) for _ in range(H)]])
    o, lse = attn_fwd_fp8(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(Nkv), rtol=1e-12)


def test_single_key():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(1, 1, 4, 8))
    k = rng.normal(size=(1, 1, 1, 8))
    v = _grid_v(rng, (1, 1, 1, 8))
    o, lse = attn_fwd_fp8(q, k, v, 0.5)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (4, 8)), rtol=1e-12)
    q8, aq = quantize_head(q[0, 0])
    k8, ak = quantize_head(k[0, 0])
    np.testing.assert_allclose(lse[0, 0], (q8 @ k8.T)[:, 0] * (aq / 448) * (ak / 448) * 0.5, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_close_to_exact_attention(causal):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, Nq, Nkv, D = 1, 4, 2, 48, 64, 32
    q = rng.normal(size=(B, Hq, Nq, D)).astype(np.float16)
    k = rng.normal(size=(B, Hkv, Nkv, D)).astype(np.float16)
    v = rng.normal(size=(B, Hkv, Nkv, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    o8, l8 = attn_fwd_fp8(q, k, v, scale, causal=causal)
    o, l = attn_fwd(q, k, v, scale, causal=causal)
    # e4m3 keeps 3 mantissa bits: V alone carries a relative rounding error of
    # up to 2^-4 (rms about 2^-4 / sqrt(3) = 3.6 %), and Q, K and P add theirs:
    # a relative L2 error of about 5 % is the fp8 result itself; 10 % is the gate
    rel = np.linalg.norm(o8 - o) / np.linalg.norm(o)
    assert rel < 0.1, rel
    assert np.abs(l8 - l).max() < 0.1


def ramp_scores(n_blocks=5):
    """Integer c per key: in block b (64 keys), c = 3 b - (j % 4), so block b's
    maximum is 3 b: the reference rises by 3 (past the 2.5 threshold) at every
    block, and every c lies in -3 .. 12 (|16 c| <= 192 is an e4m3 value)."""
    return np.array([3 * (j // 64) - (j % 64) % 4 for j in range(64 * n_blocks)], dtype=np.float64)


def _rising_case(rng, n_blocks=5, D=16):
    """Scores c ln 2 (ramp_scores): K[:, 0] = 16 c and K[0, 1] = 448 (so
    amax_K = 448, the scale is 1 and K is its own code), Q = e_0 (code 448,
    amax 1), scale = ln 2 / 16: the score is exactly c ln 2 up to the float64
    rounding of the dequantisation. V on its grid: each quantised
    64 P = 64 x 2^(c - 3 b) is an exact e4m3 value and each rescale an exact
    power of 2, so the result is the exact attention to float64 rounding."""
    c = ramp_scores(n_blocks)
    N = c.size
    k = np.zeros((1, 1, N, D))
    k[0, 0, :, 0] = 16 * c
    k[0, 0, 0, 1] = 448.0
    q = np.zeros((1, 1, 3, D))
    q[..., 0] = 1.0
    v = _grid_v(rng, (1, 1, N, D))
    return q, k, v, math.log(2.0) / 16


def test_rising_reference_is_exact_on_a_power_of_two_ramp():
    q, k, v, scale = _rising_case(np.random.default_rng(5))
    o8, l8 = attn_fwd_fp8(q, k, v, scale)
    o, l = attn_fwd(q, k, v, scale)
    np.testing.assert_allclose(o8, o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l8, l, rtol=1e-12)


SRC = inspect.getsource(fp8_mod)
MUTANTS = {
    "k_dequant_dropped": ("(aq / E4M3_MAX) * (ak / E4M3_MAX)", "(aq / E4M3_MAX)"),
    "p_scale_kept": ("/ (P_SCALE * l[:, None])", "/ l[:, None]"),
    "no_rescale_on_rise": ("acc *= alpha[:, None]", "acc *= 1.0"),
    "ties_away": ("r = np.rint(a / step) * step", "r = np.floor(a / step + 0.5) * step"),
    "sum_of_quantised_sq": ("l += p.sum(axis=1)", "l += (p * p).sum(axis=1)"),
}


def _mutant(old, new):
    assert old in SRC, old
    mod = types.ModuleType("fp8_mutant")
    mod.__dict__["__name__"] = "oracle.fp8_mutant"
    src = SRC.replace(old, new).replace("from .attention import to_f64", "from oracle.attention import to_f64")
    exec(compile(src, "fp8_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    try:
        if not all(mod.e4m3_round(x) == brute_round(x) for x in (1.0625, 1.1875, 3 * 2.0 ** -10, 0.3, 17.0)):
            return False
        rng = np.random.default_rng(2)
        q = np.zeros((1, 1, 3, 16))
        k = rng.normal(size=(1, 1, 21, 16))
        v = _grid_v(rng, (1, 1, 21, 16))
        o, lse = mod.attn_fwd_fp8(q, k, v, 0.25)
        if not np.allclose(o, v.mean(axis=2, keepdims=True), rtol=1e-12, atol=1e-15):
            return False
        if not np.allclose(lse, math.log(21), rtol=1e-12):
            return False
        q = rng.normal(size=(1, 2, 24, 16)).astype(np.float16)
        k = (3 * rng.normal(size=(1, 2, 40, 16))).astype(np.float16)
        v = rng.normal(size=(1, 2, 40, 16)).astype(np.float16)
        o8, _ = mod.attn_fwd_fp8(q, k, v, 0.25)
        o, _ = attn_fwd(q, k, v, 0.25)
        if not np.linalg.norm(o8 - o) / np.linalg.norm(o) < 0.1:
            return False
        q, k, v, scale = _rising_case(rng)
        o8, _ = mod.attn_fwd_fp8(q, k, v, scale)
        o, _ = attn_fwd(q, k, v, scale)
        return bool(np.allclose(o8, o, rtol=1e-12, atol=1e-15))
    except Exception:
        return False


def test_unmutated_oracle_passes_the_pins():
    assert _pins_pass(fp8_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    assert not _pins_pass(_mutant(*MUTANTS[name])), name
