"""Oracle of the fp8 forward (quantised attention) on the CPU.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by the tests,
never by the product path; it shares no code with the HIP kernels.

The pages list fp8 attention kernels beside the 16-bit ones ("FFPA Attention
Benchmark", section "FP8 and FP4") but state no quantisation. The reading
taken (the same as the library's header states):

* e4m3 is the OCP 8-bit float with 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals down to 2^-9 and largest finite value 448 (no infinities).
  Rounding is to nearest, ties to even mantissa.
* Each head's Q, each kv head's K and V get one scale: amax = max |x| over the
  head; the code of x is e4m3(x * s) with s = 448 / amax computed in float32
  and the product rounded to float32 first (an all-zero head: s = 1).
* Scores S = scale * (Q8 K8^T) * (amax_Q / 448) * (amax_K / 448), with the
  causal mask (top-left) as in ``attention.py``.
* P = exp(S - m) is quantised as e4m3(64 P) against a running reference m
  per row: going over the keys in blocks of 64, in order, m rises to a
  block's largest score when that exceeds m by more than 2.5 ln(2), and only
  then (the partial O and l are rescaled by exp(m_old - m_new)); so P <= 2^2.5
  and 64 P stays inside e4m3's range (64 x 2^2.5 < 448). The row sum l takes
  the unquantised P; O = (sum of P8 V8) (amax_V / 448) / (64 l), and
  lse = m + ln l.

Everything after the quantisation of the inputs is float64.
"""
from __future__ import annotations

import numpy as np

from .attention import to_f64

__all__ = ["e4m3_round", "quantize_head", "attn_fwd_fp8"]

E4M3_MAX = 448.0
P_SCALE = 64.0


def e4m3_round(x) -> np.ndarray:
    """Nearest e4m3 value of each element of x (ties to even mantissa); |x| must
    not exceed 448 plus half a step (the callers scale into range)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # step of the grid at |x|: 2^(e - 3) for normal numbers (|x| >= 2^-6), 2^-9 below
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    r = np.rint(a / step) * step  # np.rint rounds half to even: even multiple of the step
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the e4m3 range")
    return np.copysign(r, x)


def quantize_head(x) -> tuple[np.ndarray, float]:
    """(codes as float64 values, amax) of one head's tensor x (any shape)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x32))) if x32.size else 0.0
    s = np.float32(E4M3_MAX) / np.float32(amax) if amax > 0 else np.float32(1.0)
    return e4m3_round((x32 * s).astype(np.float32)), amax


BLOCK = 64  # keys per block of the running reference
RISE = 2.5 * np.log(2.0)  # the reference rises when a block's max exceeds it by more


def attn_fwd_fp8(q, k, v, scale, causal=False):
    """The fp8 forward of the module docstring: (o [B, Hq, Nq, D], lse [B, Hq, Nq])."""
    q, k, v = (to_f64(t) for t in (q, k, v))
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    o = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    kq = [[quantize_head(k[b, hk]) for hk in range(Hkv)] for b in range(B)]
    vq = [[quantize_head(v[b, hk]) for hk in range(Hkv)] for b in range(B)]
    for b in range(B):
        for h in range(Hq):
            q8, aq = quantize_head(q[b, h])
            k8, ak = kq[b][h // g]
            v8, av = vq[b][h // g]
            s = (q8 @ k8.T) * (aq / E4M3_MAX) * (ak / E4M3_MAX) * float(scale)
            if causal:
                s = np.where(np.arange(Nkv)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
            m = np.full(Nq, -np.inf)  # running reference per row
            acc = np.zeros((Nq, D))   # sum of P8 V8 (codes)
            l = np.zeros(Nq)
            for j0 in range(0, Nkv, BLOCK):
                sb = s[:, j0:j0 + BLOCK]
                bm = sb.max(axis=1)
                rise = bm > m + RISE
                with np.errstate(invalid="ignore"):
                    alpha = np.where(rise, np.exp(m - np.where(rise, bm, m)), 1.0)
                alpha = np.where(rise & np.isneginf(m), 0.0, alpha)
                m = np.where(rise, bm, m)
                acc *= alpha[:, None]
                l *= alpha
                with np.errstate(invalid="ignore"):
                    p = np.where(np.isfinite(m)[:, None], np.exp(sb - m[:, None]), 0.0)
                acc += e4m3_round(P_SCALE * p) @ v8[j0:j0 + BLOCK]
                l += p.sum(axis=1)
            live = l > 0
            with np.errstate(divide="ignore", invalid="ignore"):
                o[b, h] = np.where(live[:, None], acc * (av / E4M3_MAX) / (P_SCALE * l[:, None]), 0.0)
                lse[b, h] = np.where(live, m + np.log(l), -np.inf)
    return o, lse
