"""Dropout parity: ffpa_attn_fwd_dropout and ffpa_attn_bwd_dropout (HIP, through
the C ABI) against the float64 oracle with the same dropout_p and seed.

The keep mask is a function of (seed, head, query, key) alone (Philox-4x32-10,
one call per 4 x 4 block; see include/ffpa_attn.h), so the oracle regenerates
it and the comparison is element by element, with the bounds of the plain
forward and backward tests (the dropped P enters the same products).

Exact mask checks: with Q = 0 every score is 0 and P = 1/Nkv; with V (or K) the
identity on the first Nkv columns, each output element is either 0 or c/Nkv
(c the keep scale), so the kernels' keep mask is read back bit for bit from
O (forward), from dV (the dK/dV kernel) and from dQ (the dQ kernels of both
backward paths) and compared with the oracle's mask.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attn_bwd, attn_fwd, attn_probs, dropout_keep, dropout_threshold, to_f64
from test_gpu_bwd import REL as BREL, TOL as BTOL, UNIT as BUNIT, _compare as _bcompare, _inputs as _binputs
from test_gpu_fwd import _compare, _inputs

pytestmark = pytest.mark.gpu

DT = {"fp16": torch.float16, "bf16": torch.bfloat16}

FWD_CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 200, 150, 320),    # prefill, V staged as is, ragged
    (1, 4, 1, 1024, 300, 512),   # prefill reading the transposed V (Nq Hq >= 3072 Hkv)
    (2, 4, 2, 130, 257, 384),    # GQA, ragged
    (1, 2, 2, 100, 80, 576),     # D split across wave pairs
    (1, 2, 1, 70, 130, 1024),    # the same, GQA
    (2, 3, 3, 1, 300, 512),      # decode
    (1, 2, 1, 1, 77, 1024),      # decode, GQA
]


@pytest.mark.parametrize("shape", FWD_CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask"])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_forward_dropout_matches_oracle(lib, shape, dtype, variant, p):
    B, Hq, Hkv, Nq, Nkv, D = shape
    seed = 1000 + Nkv + D
    q, k, v, mask = _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, "key" if variant == "mask" else None)
    causal = variant == "causal"
    scale = 1.0 / math.sqrt(D)
    o, lse = lib.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                           mask=None if mask is None else mask.cuda(), scale=scale, return_lse=True,
                           dropout_p=p, seed=0xDEADBEEF12345 + seed)
    torch.cuda.synchronize()
    _compare(o, lse, q, k, v, scale, causal, mask, dtype, "f32", f"{shape}-{dtype}-{variant}-p{p}",
             dropout_p=p, seed=0xDEADBEEF12345 + seed)


def test_zero_probability_is_the_plain_path(lib):
    q, k, v, _ = _inputs(7, 1, 2, 2, 200, 150, 512, "fp16")
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o0 = lib.attention(qc, kc, vc)
    o1 = lib.attention(qc, kc, vc, dropout_p=1e-4, seed=3)  # t = round(0.0256) = 0: no dropout
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)


def test_seed_and_probability_change_the_output(lib):
    q, k, v, _ = _inputs(8, 1, 2, 2, 128, 128, 512, "fp16")
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    a = lib.attention(qc, kc, vc, dropout_p=0.2, seed=1)
    b = lib.attention(qc, kc, vc, dropout_p=0.2, seed=1)
    c = lib.attention(qc, kc, vc, dropout_p=0.2, seed=2)
    d = lib.attention(qc, kc, vc, dropout_p=0.2, seed=1 << 40)  # the high seed word counts
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, d)


def _identity_kv(Nkv, D, dtype):
    eye = torch.zeros(Nkv, D)
    eye[:, :Nkv] = torch.eye(Nkv)
    return eye.to(DT[dtype])


@pytest.mark.parametrize("Nq,Nkv,D", [(96, 512, 512), (70, 320, 320), (64, 1024, 1024), (40, 576, 576),
                                      (1, 512, 512), (1, 1024, 1024)])
@pytest.mark.parametrize("p", [0.1, 0.7])
def test_forward_keep_mask_is_exact(lib, Nq, Nkv, D, p):
    B, Hq, Hkv, dtype = 2, 2, 1, "fp16"
    seed = 0x0123456789ABCDEF
    q = torch.zeros(B, Hq, Nq, D, dtype=torch.float16)
    v = _identity_kv(Nkv, D, dtype).expand(B, Hkv, Nkv, D).contiguous()
    k = torch.zeros_like(v)
    o = lib.attention(q.cuda(), k.cuda(), v.cuda(), dropout_p=p, seed=seed).cpu()
    torch.cuda.synchronize()
    t = dropout_threshold(p)
    c = 256.0 / (256 - t)
    for b in range(B):
        for h in range(Hq):
            got = to_f64(o[b, h, :, :Nkv]) > 0.5 * c / Nkv
            want = dropout_keep(seed, b * Hq + h, range(Nq), range(Nkv), t)
            assert np.array_equal(got, want), f"head {b},{h}: {np.sum(got != want)} mask bits differ"
            kept = to_f64(o[b, h, :, :Nkv])[want]
            np.testing.assert_allclose(kept, c / Nkv, rtol=2 ** -10)


@pytest.mark.parametrize("Nq,Nkv,D", [(96, 512, 512), (130, 320, 320), (64, 1024, 1024), (40, 576, 576)])
@pytest.mark.parametrize("store_ds", [True, False])
def test_backward_keep_mask_is_exact(lib, Nq, Nkv, D, store_ds):
    """Q = 0 (P = 1/Nkv), V = K = identity, dO = ones: dV[j, i] = Z_ij c / Nkv
    (the dK/dV kernel's mask) and dQ[i, j] = scale (Z_ij c - delta_i) / Nkv
    (the mask of the dQ kernel of the path)."""
    B, Hq, Hkv, dtype, p = 1, 2, 2, "fp16", 0.3
    seed = 99
    assert Nq <= D
    q = torch.zeros(B, Hq, Nq, D, dtype=torch.float16)
    kv = _identity_kv(Nkv, D, dtype).expand(B, Hkv, Nkv, D).contiguous()
    dout = torch.zeros(B, Hq, Nq, D, dtype=torch.float16)
    dout[..., :Nkv] = 1.0
    scale = 1.0 / math.sqrt(D)
    qc, kc, vc = q.cuda(), kv.cuda(), kv.cuda()
    o, lse = lib.attention(qc, kc, vc, scale=scale, return_lse=True, dropout_p=p, seed=seed)
    dq, dk, dv = lib.attention_backward(dout.cuda(), qc, kc, vc, o, lse, scale=scale, store_ds=store_ds,
                                        dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    t = dropout_threshold(p)
    c = 256.0 / (256 - t)
    dvh, dqh, oh = to_f64(dv.cpu()), to_f64(dq.cpu()), to_f64(o.cpu())
    for h in range(Hq):
        want = dropout_keep(seed, h, range(Nq), range(Nkv), t)
        # dV[key j] = sum_i Z_ij c / Nkv dO_i: column d of dO is ones for d < Nkv,
        # so dV[j, d] = c / Nkv * (number of queries keeping j), the same for
        # every d < Nkv; the per-query bits come from dQ instead
        np.testing.assert_allclose(dvh[0, h, :, 0], c / Nkv * want.sum(axis=0), rtol=2e-3)
        delta = oh[0, h, :, :Nkv].sum(axis=1)
        mid = scale * (0.5 * c - delta) / Nkv
        got = dqh[0, h, :, :Nkv] > mid[:, None]
        assert np.array_equal(got, want), f"head {h}: {np.sum(got != want)} mask bits differ"


BWD_CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 100, 80, 128),
    (2, 4, 2, 160, 200, 320),    # GQA, ragged
    (1, 2, 2, 200, 150, 512),    # several tiles each way, ragged
    (1, 2, 2, 1, 70, 512),       # one query row
    (1, 2, 2, 100, 80, 576),
    (1, 2, 1, 70, 130, 1024),    # GQA
]


def _drop_bounds(q, k, v, do, scale, causal, mask, refs, dtype, p, seed, bh0=0):
    """The bf16 rounding bounds of the plain backward test with P o Z c in
    place of P where the dropped probabilities enter (bh0: as in the oracle,
    for one head of a larger problem)."""
    u = BUNIT[dtype]
    qd, kd, vd, dod = (to_f64(t) for t in (q, k, v, do))
    B, Hq, Nq, D = qd.shape
    Hkv, Nkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    t = dropout_threshold(p)
    c = 256.0 / (256 - t)
    P = attn_probs(q, k, scale, causal=causal, mask=mask)
    bq, bk, bv = np.zeros_like(qd), np.zeros_like(kd), np.zeros_like(vd)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            zc = dropout_keep(seed, bh0 + b * Hq + h, range(Nq), range(Nkv), t) * c
            pd = P[b, h] * zc
            dp = (dod[b, h] @ vd[b, hk].T) * zc
            delta = np.sum(P[b, h] * dp, axis=1)
            ds = np.abs(P[b, h] * (dp - delta[:, None]))
            e = np.sum(np.abs(dod[b, h]) * np.abs(pd @ vd[b, hk]), axis=1)
            bv[b, hk] += pd.T @ np.abs(dod[b, h])
            bk[b, hk] += scale * (ds.T @ np.abs(qd[b, h]) + (P[b, h] * e[:, None]).T @ np.abs(qd[b, h]))
            bq[b, h] = scale * (ds @ np.abs(kd[b, hk]) + e[:, None] * (P[b, h] @ np.abs(kd[b, hk])))
    rq, rk, rv = refs
    return {"dQ": BTOL + 2 * u * (bq + np.abs(rq)), "dK": BTOL + 2 * u * (bk + np.abs(rk)),
            "dV": BTOL + 2 * u * (bv + np.abs(rv))}


@pytest.mark.parametrize("shape", BWD_CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask"])
@pytest.mark.parametrize("store_ds", [True, False])
def test_backward_dropout_matches_oracle(lib, shape, dtype, variant, store_ds):
    B, Hq, Hkv, Nq, Nkv, D = shape
    p, seed = 0.2, 4242 + D
    causal = variant == "causal"
    q, k, v, do, mask = _binputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, variant == "mask")
    scale = 1.0 / math.sqrt(D)
    m2 = None if mask is None else mask.view(-1, Nkv)
    o_ref, lse_ref = attn_fwd(q, k, v, scale, causal=causal, mask=m2, dropout_p=p, seed=seed)
    o_in = torch.from_numpy(o_ref).to(DT[dtype]).cuda()
    lse_in = torch.from_numpy(lse_ref).to(torch.float32).cuda()
    dq, dk, dv = lib.attention_backward(do.cuda(), q.cuda(), k.cuda(), v.cuda(), o_in, lse_in,
                                        causal=causal, mask=None if mask is None else mask.cuda(),
                                        scale=scale, store_ds=store_ds, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    refs = attn_bwd(q, k, v, do, scale, causal=causal, mask=m2, dropout_p=p, seed=seed)
    label = f"{shape}-{dtype}-{variant}-{'stored' if store_ds else 'recomputed'} dS-p{p}"
    print(label, flush=True)
    bounds = _drop_bounds(q, k, v, do, scale, causal, m2, refs, dtype, p, seed) if dtype == "bf16" else {}
    for name, got, ref in (("dV", dv, refs[2]), ("dK", dk, refs[1]), ("dQ", dq, refs[0])):
        _bcompare(name, got, ref, dtype, label, bounds.get(name))


def test_backward_dropout_chunks_agree(lib):
    """The stored-dS path over chunks of one kv head gives the bits of one chunk."""
    B, Hq, Hkv, Nq, Nkv, D = 2, 4, 2, 130, 160, 512
    q, k, v, do, _ = _binputs(5, B, Hq, Hkv, Nq, Nkv, D, "fp16", False)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.attention(qc, kc, vc, return_lse=True, dropout_p=0.25, seed=77)
    full = lib.attention_backward(dc, qc, kc, vc, o, lse, dropout_p=0.25, seed=77)
    mn = lib.ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, 0)
    kt = B * Hkv * D * 192 * 2
    ds1 = (Hq // Hkv) * math.ceil(Nq / 32) * math.ceil(Nkv / 32) * 2048
    one = lib.attention_backward(dc, qc, kc, vc, o, lse, dropout_p=0.25, seed=77,
                                 workspace_bytes=mn + kt + ds1)
    torch.cuda.synchronize()
    for a, b in zip(full, one):
        assert torch.equal(a, b)
