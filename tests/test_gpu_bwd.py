"""Backward parity: ffpa_attn_bwd (HIP, through the C ABI) against the float64 oracle.

Small shapes: seeded inputs; O and lse handed to the kernel are the oracle's
(rounded to the storage type and to fp32), so the kernels under test are the
backward ones alone; the expected dQ, dK, dV are oracle.attn_bwd on the same
16-bit values widened to float64 (the oracle recomputes P itself).

Gate (fp32 accumulation): max |d - d_oracle| <= 1e-2 for each of dQ, dK, dV
(fp16 here, and every type at the benchmark sizes in test_gpu_full.py). The
relative L2 error is asserted as well.

bf16 at small shapes: the MFMA operands P and dS must be rounded to bf16
(unit roundoff u = 2^-8), and O enters delta as the rounded bf16 output. On
short causal rows the gradients reach |dV| ~ 4, where those roundings alone
exceed 1e-2. The bound there is elementwise, 1e-2 + 2 x the rounding error
terms, each computed from the oracle's P:
    dV: u (P^T |dO| + |dV|)
    dK: u (scale |dS|^T |Q| + scale (P o e)^T |Q| + |dK|)
    dQ: u (scale |dS| |K| + scale e o (P |K|) + |dQ|)
with e_i = sum_d |dO_id| |O_id| (the rounding of O in delta).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attn_bwd, attn_fwd, attn_probs, to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-2
REL = {"fp16": 4e-3, "bf16": 2.5e-2}
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, with_mask, mask_rows=1):
    q = W.draw(seed, W.T_Q, B, Hq, Nq, D, dtype)
    k = W.draw(seed, W.T_K, B, Hkv, Nkv, D, dtype)
    v = W.draw(seed, W.T_V, B, Hkv, Nkv, D, dtype)
    do = W.draw(seed, W.T_DO, B, Hq, Nq, D, dtype)
    mask = W.draw_key_bias(seed, Nkv, dtype, 0.1, rows=mask_rows) if with_mask else None
    return q, k, v, do, mask


UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _rounding_bounds(q, k, v, do, scale, causal, mask, refs, dtype):
    """Elementwise bounds on dV, dK, dQ (see the module docstring)."""
    u = UNIT[dtype]
    qd, kd, vd, dod = (to_f64(t) for t in (q, k, v, do))
    B, Hq, Nq, D = qd.shape
    Hkv = kd.shape[1]
    g = Hq // Hkv
    P = attn_probs(q, k, scale, causal=causal, mask=mask)
    bq = np.zeros_like(qd)
    bk = np.zeros_like(kd)
    bv = np.zeros_like(vd)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            p = P[b, h]
            dp = dod[b, h] @ vd[b, hk].T
            delta = np.sum(p * dp, axis=1)
            ds = np.abs(p * (dp - delta[:, None]))
            e = np.sum(np.abs(dod[b, h]) * np.abs(p @ vd[b, hk]), axis=1)
            bv[b, hk] += p.T @ np.abs(dod[b, h])
            bk[b, hk] += scale * (ds.T @ np.abs(qd[b, h]) + (p * e[:, None]).T @ np.abs(qd[b, h]))
            bq[b, h] = scale * (ds @ np.abs(kd[b, hk]) + e[:, None] * (p @ np.abs(kd[b, hk])))
    rq, rk, rv = refs
    return {"dQ": TOL + 2 * u * (bq + np.abs(rq)), "dK": TOL + 2 * u * (bk + np.abs(rk)),
            "dV": TOL + 2 * u * (bv + np.abs(rv))}


def _compare(name, got, ref, dtype, label, bound=None):
    g = to_f64(got)
    assert np.isfinite(g).all(), f"{label}: non-finite {name}"
    diff = np.abs(g - ref)
    err = diff.max()
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"  {label} {name}: max|d|={err:.3e} relL2={rel:.3e} max|ref|={np.abs(ref).max():.3e}",
          flush=True)
    if bound is None:
        assert err <= TOL, f"{label}: {name} max abs error {err}"
    else:
        worst = (diff / bound).max()
        assert worst <= 1.0, f"{label}: {name} error exceeds the bound by {worst:.3f}x (max abs {err})"
    if np.abs(ref).max() >= TOL:  # a (near-)zero reference makes the ratio meaningless
        assert rel <= REL[dtype], f"{label}: {name} rel L2 {rel}"


def _run_case(lib, shape, dtype, causal, with_mask, seed, mask_rows=1, store_ds=True):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v, do, mask = _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, with_mask,
                                mask_rows=Nq if mask_rows != 1 else 1)
    scale = 1.0 / math.sqrt(D)
    m2 = None if mask is None else mask.view(-1, Nkv)
    o_ref, lse_ref = attn_fwd(q, k, v, scale, causal=causal, mask=m2)
    o_in = torch.from_numpy(o_ref).to(DT[dtype]).cuda()
    lse_in = torch.from_numpy(lse_ref).to(torch.float32).cuda()
    dq, dk, dv = lib.attention_backward(do.cuda(), q.cuda(), k.cuda(), v.cuda(), o_in, lse_in,
                                        causal=causal,
                                        mask=None if mask is None else mask.cuda(), scale=scale,
                                        store_ds=store_ds)
    torch.cuda.synchronize()
    rq, rk, rv = attn_bwd(q, k, v, do, scale, causal=causal, mask=m2)
    path = {True: "stored dS", False: "recomputed dS", None: "default workspace"}[store_ds]
    label = f"{shape}-{dtype}-{'causal' if causal else 'full'}-{'mask' if with_mask else 'nomask'}-{path}"
    print(label, flush=True)
    bounds = (_rounding_bounds(q, k, v, do, scale, causal, m2, (rq, rk, rv), dtype)
              if dtype == "bf16" else {})
    _compare("dV", dv, rv, dtype, label, bounds.get("dV"))
    _compare("dK", dk, rk, dtype, label, bounds.get("dK"))
    _compare("dQ", dq, rq, dtype, label, bounds.get("dQ"))


CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 64, 64, 64),
    (1, 2, 2, 100, 80, 128),     # ragged queries and keys
    (2, 4, 2, 160, 200, 256),    # GQA g = 2, ragged
    (1, 4, 1, 96, 130, 320),     # GQA g = 4
    (1, 2, 2, 200, 150, 512),    # several tiles each way, ragged
    (1, 2, 2, 1, 70, 512),       # one query row
    (1, 1, 1, 256, 256, 448),
    (1, 2, 2, 64, 300, 192),     # Nkv > Nq
    (1, 2, 2, 70, 33, 384),      # Nq > Nkv
    # above 512: D in four parts per workgroup, zero-padded to a multiple of 128
    (1, 2, 2, 100, 80, 576),     # padded to 640, ragged
    (1, 2, 1, 70, 130, 1024),    # GQA g = 2
    (1, 1, 1, 64, 64, 640),
    (1, 2, 2, 40, 90, 960),      # padded to 1024
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask", "causal_mask", "qmask", "causal_qmask"])
def test_backward_matches_oracle(lib, shape, dtype, variant):
    _run_case(lib, shape, dtype, "causal" in variant, "mask" in variant, 300 + sum(shape),
              mask_rows="q" if "qmask" in variant else 1)


# With only the minimal workspace, the dQ pass recomputes S and dP instead of
# reading back the dS that the dK/dV pass stored.
@pytest.mark.parametrize("shape", [CASES[1], CASES[2], CASES[4], CASES[9], CASES[10]],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", ["plain", "causal_mask", "causal_qmask"])
def test_backward_minimal_workspace_matches_oracle(lib, shape, variant):
    _run_case(lib, shape, "bf16", "causal" in variant, "mask" in variant, 300 + sum(shape),
              mask_rows="q" if "qmask" in variant else 1, store_ds=False)


def test_backward_deterministic(lib):
    B, Hq, Hkv, Nq, Nkv, D = 1, 4, 2, 150, 170, 512
    q, k, v, do, _ = _inputs(77, B, Hq, Hkv, Nq, Nkv, D, "bf16", False)
    q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.attention(q, k, v, return_lse=True)
    r1 = lib.attention_backward(do, q, k, v, o, lse)
    r2 = lib.attention_backward(do, q, k, v, o, lse)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_backward_zero_dout_gives_zero(lib):
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 96, 96, 256
    q, k, v, do, _ = _inputs(78, B, Hq, Hkv, Nq, Nkv, D, "fp16", False)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o, lse = lib.attention(q, k, v, return_lse=True)
    dq, dk, dv = lib.attention_backward(torch.zeros_like(q), q, k, v, o, lse)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t).item() == 0


def test_backward_causal_keys_past_queries_get_zero(lib):
    # top-left causal with Nkv > Nq: keys >= Nq are seen by no row
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 70, 200, 128
    q, k, v, do, _ = _inputs(79, B, Hq, Hkv, Nq, Nkv, D, "bf16", False)
    q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.attention(q, k, v, causal=True, return_lse=True)
    dq, dk, dv = lib.attention_backward(do, q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk[:, :, Nq:]).item() == 0
    assert torch.count_nonzero(dv[:, :, Nq:]).item() == 0


@pytest.mark.parametrize("shape,causal,mask_rows", [
    ((2, 6, 3, 150, 170, 512), False, 0),   # 6 kv heads over two batches: chunks cross b
    ((1, 8, 2, 100, 130, 320), True, 1),    # GQA g = 4, causal, key bias
    ((1, 3, 3, 70, 90, 1024), False, 70),   # D above 512, per-query mask
])
def test_backward_chunks_give_the_same_bits(lib, shape, causal, mask_rows):
    """The stored-dS path runs the dK/dV and dQ passes over chunks of kv heads
    that fit the dS room of the workspace. Chunks of 1 and 2 kv heads (room for
    exactly that much dS) must give the bits of the one-chunk default, and the
    default must match the oracle."""
    B, Hq, Hkv, Nq, Nkv, D = shape
    dtype = "bf16"
    q, k, v, do, mask = _inputs(90 + sum(shape), B, Hq, Hkv, Nq, Nkv, D, dtype, mask_rows > 0,
                                mask_rows=max(mask_rows, 1))
    q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    mk = None if mask is None else mask.cuda()
    scale = 1.0 / math.sqrt(D)
    o, lse = lib.attention(q, k, v, causal=causal, mask=mk, scale=scale, return_lse=True)
    ref = lib.attention_backward(do, q, k, v, o, lse, causal=causal, mask=mk, scale=scale)
    dt = lib.BF16
    base = lib.ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dt)
    kt = B * Hkv * D * ((Nkv + 63) // 64 * 64) * 2
    nqt, nkt = (Nq + 31) // 32, (Nkv + 31) // 32
    per = (Hq // Hkv) * nqt * nkt * 2048
    full = lib.ffpa_attn_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt)
    assert full == base + kt + B * Hkv * per  # small problems: one chunk
    for chunk in (1, 2):
        print(f"case {shape} causal={causal} mask_rows={mask_rows} chunk={chunk}", flush=True)
        got = lib.attention_backward(do, q, k, v, o, lse, causal=causal, mask=mk, scale=scale,
                                     workspace_bytes=base + kt + chunk * per + per - 1)
        torch.cuda.synchronize()
        for nm, a_, b_ in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a_, b_), f"chunk {chunk}: {nm} differs from the one-chunk result"
    m2 = None if mask is None else mask.view(-1, Nkv)
    qc, kc, vc, doc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    refs = attn_bwd(qc, kc, vc, doc, scale, causal=causal, mask=m2)
    bounds = _rounding_bounds(qc, kc, vc, doc, scale, causal, m2, refs, dtype)
    for nm, g_, r_ in zip(("dQ", "dK", "dV"), ref, refs):
        _compare(nm, g_, r_, dtype, f"chunks-{shape}", bounds[nm])


@pytest.mark.parametrize("shape", [(1, 2, 2, 2048, 2048, 512), (1, 2, 1, 1024, 1024, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("store_ds", [True, False])
def test_backward_causal_few_heads_long_rows(lib, shape, store_ds):
    """Causal with few heads and long rows: the blocks of one head fill several
    XCD ranges, whose causal work order interleaves them."""
    _run_case(lib, shape, "fp16", True, False, 31, store_ds=store_ds)


# One query row with the default workspace: the decode backward (dQ partials
# per key range, dK and dV written once per key) where it is built (G = Hq /
# Hkv up to 4 at D <= 512, up to 2 above), the minimal-workspace kernels
# otherwise (G = 8 below).
DECODE_CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 1, 70, 512),      # one key range, ragged
    (2, 4, 2, 1, 1000, 320),    # G = 2, four ranges, the last one shorter
    (1, 8, 2, 1, 4097, 128),    # G = 4, 17 ranges of 248 keys
    (1, 2, 1, 1, 600, 1024),    # G = 2, two granules per lane
    (1, 3, 3, 1, 517, 576),     # a lane's second granule only in lanes 0 .. 7
    (3, 2, 2, 1, 33, 64),       # 8 lanes hold the row
    (1, 2, 2, 1, 1, 256),       # one key: dV = dO, dK = dQ = 0
    (1, 8, 1, 1, 300, 128),     # G = 8: no decode backward, the minimal path
]


@pytest.mark.parametrize("shape", DECODE_CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask", "causal_mask"])
def test_decode_backward_matches_oracle(lib, shape, dtype, variant):
    B, Hq, Hkv, Nq, Nkv, D = shape
    dt = lib.BF16 if dtype == "bf16" else lib.F16
    size = lib.ffpa_attn_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt)
    if Hq // Hkv <= (4 if D <= 512 else 2):
        # the default holds the dQ partials, not the stored-dS path's K^T and dS
        assert lib.ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dt) <= size < \
            lib.ffpa_attn_bwd_workspace_size_stored(B, Hq, Hkv, Nq, Nkv, D, dt)
    _run_case(lib, shape, dtype, "causal" in variant, "mask" in variant, 500 + sum(shape), store_ds=None)


def test_decode_backward_deterministic_and_zero_dout(lib):
    """The decode backward gives the same bits on every call (dQ partials are
    summed in range order), and zero gradients for dO = 0."""
    B, Hq, Hkv, Nq, Nkv, D = 2, 8, 4, 1, 3000, 512
    q, k, v, do, _ = _inputs(81, B, Hq, Hkv, Nq, Nkv, D, "bf16", False)
    q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.attention(q, k, v, return_lse=True)
    r1 = lib.attention_backward(do, q, k, v, o, lse)
    r2 = lib.attention_backward(do, q, k, v, o, lse)
    z = lib.attention_backward(torch.zeros_like(do), q, k, v, o, lse)
    torch.cuda.synchronize()
    for a_, b_ in zip(r1, r2):
        assert torch.equal(a_, b_)
    for t in z:
        assert torch.count_nonzero(t).item() == 0



def test_decode_backward_fully_masked_row(lib):
    """A row that sees no key (every bias -inf) has lse = -inf and no gradient."""
    B, Hq, Hkv, Nq, Nkv, D = 1, 4, 2, 1, 300, 128
    q, k, v, do, _ = _inputs(82, B, Hq, Hkv, Nq, Nkv, D, "fp16", False)
    q, k, v, do = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    mask = torch.full((1, 1, 1, Nkv), float("-inf"), dtype=torch.float16, device="cuda")
    o, lse = lib.attention(q, k, v, mask=mask, return_lse=True)
    dq, dk, dv = lib.attention_backward(do, q, k, v, o, lse, mask=mask)
    torch.cuda.synchronize()
    assert torch.isinf(lse).all() and (lse < 0).all()
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t).item() == 0
