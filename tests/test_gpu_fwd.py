"""Forward parity: the HIP kernels (through the C ABI) against the float64 oracle.

Every case draws seeded inputs (``workloads``), runs ``ffpa_attn_fwd`` on the
GPU and compares O element by element, and lse, with the oracle run on the very
same fp16/bf16 values widened to float64. The gate is the stated tolerance on
max |O - O_oracle|: 1e-2 with fp32 accumulation, 5e-2 with fp16 accumulation.
Diagnostics that are sharper than the gate are asserted too: the relative L2
error of O, the lse error, and exact results where the mathematics fixes them.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attn_fwd, to_f64

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-2, "f16": 5e-2}
# relative L2 bounds expected from output rounding (not the gate)
REL = {("fp16", "f32"): 4e-3, ("bf16", "f32"): 1.6e-2, ("fp16", "f16"): 1.2e-2,
       ("bf16", "f16"): 2e-2}


def _run(lib, q, k, v, *, causal=False, mask=None, accum="f32", scale=None):
    o, lse = lib.attention(q, k, v, causal=causal, mask=mask, scale=scale, accum=accum,
                           return_lse=True)
    torch.cuda.synchronize()
    return o, lse


# unit roundoff of the 16-bit storage type (round to nearest even)
UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _compare(o, lse, q, k, v, scale, causal, mask, dtype, accum, label, flat_gate=False,
             dropout_p=0.0, seed=0):
    """Element-wise parity of O and lse against the oracle.

    flat_gate: the judged workloads' bound, max |dO| <= TOL[accum]. Otherwise
    the bound also admits the two roundings every 16-bit kernel must make,
    each at most one unit roundoff u of the storage type: O rounded on store
    (u |O|) and P rounded to the MFMA operand type (u sum_j p_j |v_j|). They
    matter only where |O| is large, e.g. the first rows of a causal pass on
    a short sequence; at N(0, 1) and N = 8192, |O| is ~0.02 and the flat gate
    applies.
    """
    m2 = None if mask is None else mask.view(-1, k.shape[2])
    drop = dict(dropout_p=dropout_p, seed=seed)
    oo, lo = attn_fwd(q, k, v, scale, causal=causal, mask=m2, **drop)
    og = to_f64(o)
    lg = to_f64(lse)
    assert np.isfinite(og).all(), f"{label}: non-finite output"
    diff = np.abs(og - oo)
    err = diff.max()
    rel = np.linalg.norm(og - oo) / max(np.linalg.norm(oo), 1e-30)
    fin = np.isfinite(lo)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lo)), f"{label}: -inf lse pattern differs"
    lerr = np.abs(lg[fin] - lo[fin]).max() if fin.any() else 0.0
    print(f"{label}: max|dO|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}", flush=True)
    if flat_gate:
        assert err <= TOL[accum], f"{label}: max abs error {err} > {TOL[accum]}"
    else:
        pv_abs, _ = attn_fwd(q, k, to_f64(v).__abs__(), scale, causal=causal, mask=m2, **drop)
        bound = TOL[accum] + UNIT[dtype] * (np.abs(oo) + pv_abs)
        worst = (diff / bound).max()
        assert worst <= 1.0, f"{label}: error exceeds the bound by {worst:.3f}x (max abs {err})"
    assert rel <= REL[(dtype, accum)], f"{label}: rel L2 {rel}"
    assert lerr <= 2e-3, f"{label}: lse error {lerr}"


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, mask_kind=None):
    q = W.draw(seed, W.T_Q, B, Hq, Nq, D, dtype)
    k = W.draw(seed, W.T_K, B, Hkv, Nkv, D, dtype)
    v = W.draw(seed, W.T_V, B, Hkv, Nkv, D, dtype)
    mask = None
    if mask_kind == "key":
        mask = W.draw_key_bias(seed, Nkv, dtype, 0.1, rows=1)
    elif mask_kind == "query":
        mask = W.draw_key_bias(seed, Nkv, dtype, 0.1, rows=Nq)
    return q, k, v, mask


def test_tiny_config(lib):
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = _run(lib, q, k, v, scale=w.scale)
    _compare(o, lse, inp["q"], inp["k"], inp["v"], w.scale, False, None, "fp16", "f32", "tiny",
             flat_gate=True)


CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D)
    (1, 2, 2, 256, 256, 320),
    (1, 2, 2, 200, 333, 512),   # ragged, several tiles
    (2, 4, 2, 130, 130, 448),   # GQA g=2, ragged
    (1, 8, 2, 64, 192, 384),    # GQA g=4, cross
    (1, 2, 2, 384, 64, 256),    # Nq > Nkv
    (1, 3, 3, 1, 517, 512),     # decode-like
    (1, 2, 1, 129, 1, 128),     # single key
    (1, 1, 1, 77, 700, 64),
    (1, 2, 2, 100, 100, 192),
    (1, 2, 2, 200, 333, 576),   # D above 512: D split across wave pairs
    (2, 4, 2, 130, 77, 768),    # GQA, Nq > Nkv
    (1, 2, 2, 64, 300, 1024),
    (1, 3, 1, 100, 100, 640),   # GQA g = 3
    (1, 2, 2, 70, 20, 832),     # D above 512, one partial key tile
    (1, 2, 1, 90, 1, 896),      # D above 512, a single key
    (1, 2, 2, 33, 64, 960),     # D above 512, two whole key tiles
    (1, 2, 2, 300, 250, 704),   # fp16 accumulation: three 128-row blocks, the last ragged
    (1, 4, 2, 129, 96, 576),    # fp16 accumulation: one row past a 128-row block
    (1, 2, 2, 260, 200, 640),   # fp16 accumulation at 640: 64-key tiles fill the LDS
    (1, 1, 1, 130, 8300, 576),  # the key bias no longer fits beside 64-key tiles at 576
]


# Up to D = 512 the library stages V from a transposed copy when a head's
# queries are many compared with its keys (Nq * Hq >= 3072 * Hkv), and reads V
# with transposed LDS reads otherwise: the shapes above take the second layout
# (and D > 512 always the copy), these the first.
CASES_VT = [
    (1, 1, 1, 3100, 100, 512),   # ragged queries and keys
    (1, 4, 1, 800, 200, 320),    # GQA g = 4
    (1, 1, 1, 3072, 64, 64),     # exactly at the threshold
    (1, 2, 2, 3200, 150, 448),
]


@pytest.mark.parametrize("shape", CASES + CASES_VT, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("accum", ["f32", "f16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask", "causal_mask", "qmask", "causal_qmask"])
def test_forward_matches_oracle(lib, shape, dtype, accum, variant):
    B, Hq, Hkv, Nq, Nkv, D = shape
    causal = "causal" in variant
    mk = "query" if "qmask" in variant else "key" if "mask" in variant else None
    seed = 100 + sum(shape)
    q, k, v, mask = _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, mk)
    if mask is not None:
        mask[:, 0] = 0.0  # key 0 stays visible: a causal row 0 is then never empty
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=causal,
                  mask=None if mask is None else mask.cuda(), accum=accum, scale=scale)
    _compare(o, lse, q, k, v, scale, causal, mask, dtype, accum, f"{shape}-{dtype}-{accum}-{variant}")


@pytest.mark.parametrize("D", [64, 320, 512, 576, 640, 704, 1024])
@pytest.mark.parametrize("accum", ["f32", "f16"])
def test_zero_query_gives_mean_and_log_n(lib, D, accum):
    _, k, v, _ = _inputs(7, 1, 2, 2, 8, 300, D, "fp16")
    q = torch.zeros(1, 2, 130, D, dtype=torch.float16)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), accum=accum)
    mean = to_f64(v).mean(axis=2, keepdims=True)
    assert np.abs(to_f64(o) - mean).max() <= 2e-3
    assert np.abs(to_f64(lse) - math.log(300)).max() <= 1e-5


@pytest.mark.parametrize("D", [320, 576, 640, 768, 960])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("accum", ["f32", "f16"])
def test_single_key_returns_v0_exactly(lib, D, dtype, accum):
    q, k, v, _ = _inputs(8, 1, 2, 2, 150, 1, D, dtype)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), accum=accum)
    want_o = v
    if accum == "f16" and dtype == "bf16":  # the fp16 accumulator holds V rounded to fp16
        want_o = v.to(torch.float16).to(torch.bfloat16)
    assert torch.equal(o.cpu(), want_o.expand_as(o)), "Nkv = 1 must return V[0] bit-exactly"
    scale = float(np.float32(1.0 / math.sqrt(D)))
    want = scale * np.einsum("bhnd,bhd->bhn", to_f64(q), to_f64(k)[:, :, 0])
    np.testing.assert_allclose(to_f64(lse), want, atol=2e-4, rtol=0)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_causal_row0_is_v0_exactly(lib, dtype):
    q, k, v, _ = _inputs(9, 1, 4, 2, 300, 300, 448, dtype)
    o, _ = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=True)
    assert torch.equal(o[:, :, 0].cpu(), v.repeat_interleave(2, dim=1)[:, :, 0])


@pytest.mark.parametrize("D,accum", [(320, "f32"), (576, "f16"), (768, "f16"), (1024, "f32")])
def test_fully_masked_rows_give_zero_and_neg_inf(lib, D, accum):
    q, k, v, _ = _inputs(10, 1, 2, 2, 70, 90, D, "fp16")
    mask = torch.full((1, 90), float("-inf"), dtype=torch.float16)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), mask=mask.cuda(), accum=accum)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("D,accum", [(512, "f32"), (640, "f16"), (1024, "f16")])
def test_mask_equals_deleting_keys(lib, D, accum):
    q, k, v, _ = _inputs(11, 1, 2, 2, 96, 200, D, "fp16")
    keep = torch.ones(200, dtype=torch.bool)
    keep[torch.randperm(200, generator=torch.Generator().manual_seed(1))[:37]] = False
    mask = torch.where(keep, 0.0, float("-inf")).to(torch.float16)[None]
    o1, l1 = _run(lib, q.cuda(), k.cuda(), v.cuda(), mask=mask.cuda(), accum=accum)
    o2, l2 = _run(lib, q.cuda(), k[:, :, keep].contiguous().cuda(), v[:, :, keep].contiguous().cuda(),
                  accum=accum)
    assert (o1 - o2).abs().max().item() <= 2e-3
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_deterministic(lib):
    q, k, v, _ = _inputs(12, 1, 4, 4, 256, 512, 512, "bf16")
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = _run(lib, q, k, v, causal=True)
    o2, l2 = _run(lib, q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("slope", [0.05, 0.5])
@pytest.mark.parametrize("D", [128, 512, 640, 1024])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("accum", ["f32", "f16"])
def test_growing_row_max(lib, slope, D, dtype, accum):
    """A key-bias ramp raises every row's running max tile after tile (by up to
    46 in log2 units per 64-key tile at slope 0.5), which forces the online
    softmax off its first reference max again and again."""
    q, k, v, _ = _inputs(13, 1, 2, 2, 200, 512, D, dtype)
    ramp = (slope * torch.arange(512, dtype=torch.float32)).to(W.DTYPES[dtype])[None]
    scale = 1.0 / math.sqrt(D)
    for causal in (False, True):
        o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=causal, mask=ramp.cuda(),
                      accum=accum, scale=scale)
        _compare(o, lse, q, k, v, scale, causal, ramp, dtype, accum,
                 f"ramp{slope}-D{D}-{dtype}-{accum}-causal{causal}")


DECODE_CASES = [
    # (B, Hq, Hkv, 1, Nkv, D): the split-KV decode kernels
    (2, 8, 2, 1, 1000, 1024),   # GQA g = 4, D = 1024 (two granules per lane)
    (1, 4, 4, 1, 3, 96),        # fewer keys than one step
    (3, 2, 1, 1, 4097, 576),    # ragged last range
    (1, 1, 1, 1, 1, 64),        # one key
    (2, 16, 16, 1, 8192, 512),  # the decode shape, fewer heads
    (1, 2, 2, 1, 300, 320),     # D / 8 not a multiple of 64 lanes
]


@pytest.mark.parametrize("shape", DECODE_CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("variant", ["plain", "causal", "mask"])
def test_decode_matches_oracle(lib, shape, dtype, variant):
    B, Hq, Hkv, Nq, Nkv, D = shape
    causal = variant == "causal"
    mk = "key" if variant == "mask" else None
    q, k, v, mask = _inputs(500 + sum(shape), B, Hq, Hkv, Nq, Nkv, D, dtype, mk)
    if mask is not None:
        mask[0, 0] = 0.0
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=causal,
                  mask=None if mask is None else mask.cuda(), scale=scale)
    _compare(o, lse, q, k, v, scale, causal, mask, dtype, "f32", f"decode-{shape}-{dtype}-{variant}")


def test_decode_fully_masked_row(lib):
    # every key masked: O = 0 and lse = -inf (the oracle's reading of a dead row)
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 1, 700, 512
    q, k, v, _ = _inputs(600, B, Hq, Hkv, Nq, Nkv, D, "fp16")
    mask = torch.full((1, Nkv), float("-inf"), dtype=torch.float16)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), mask=mask.cuda())
    assert torch.count_nonzero(o).item() == 0
    assert torch.isneginf(lse).all()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_key_bias_too_long_for_lds(lib, dtype):
    # 20000 keys: the bias (40000 B) does not fit beside the 128 KiB of tiles,
    # so the kernel reads it from global memory like a per-query mask
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 70, 20000, 512
    q, k, v, mask = _inputs(700, B, Hq, Hkv, Nq, Nkv, D, dtype, "key")
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=False, mask=mask.cuda(), scale=scale)
    _compare(o, lse, q, k, v, scale, False, mask, dtype, "f32", f"longbias-{dtype}")


@pytest.mark.parametrize("shape", [(1, 2, 2, 130, 300, 512), (1, 2, 1, 100, 77, 1024), (2, 2, 2, 64, 64, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_query_mask_equals_deleting_keys_per_row(lib, shape):
    # a per-query mask of 0 / -inf equals running each row with its own key set:
    # checked against the oracle on rows whose masks differ
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v, _ = _inputs(710 + sum(shape), B, Hq, Hkv, Nq, Nkv, D, "fp16")
    g = torch.Generator().manual_seed(711)
    keep = torch.rand(Nq, Nkv, generator=g) > 0.5
    keep[:, 0] = True
    mask = torch.where(keep, torch.zeros(()), torch.full((), float("-inf"))).to(torch.float16)
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), mask=mask.cuda(), scale=scale)
    for r in (0, Nq // 2, Nq - 1):
        ks = keep[r].nonzero().flatten()
        oo, lo = attn_fwd(q[:, :, r:r + 1], k[:, :, ks], v[:, :, ks], scale)
        assert np.abs(to_f64(o[:, :, r:r + 1]) - oo).max() <= 1e-2
        assert np.abs(to_f64(lse[:, :, r:r + 1]) - lo).max() <= 2e-3


@pytest.mark.parametrize("D", [320, 576, 768, 1024])
def test_bf16_inputs_with_the_fp16_accumulator(lib, D):
    """bf16 inputs with FFPA_ACC_F16 accumulate O in fp16 (the reading of
    "fp16 accumulation" the header documents). Inside fp16's range the result
    is right to the rounding of an fp16 accumulator, also at |V| ~ 6e4; a
    column of V whose products reach fp16 infinity (|v| = 1e5) makes that
    output column non-finite and leaves the others untouched; fp32
    accumulation gets it right."""
    q, k, v, _ = _inputs(31, 1, 2, 2, 150, 200, D, "bf16")
    scale = 1.0 / math.sqrt(D)
    big = v.clone()
    big[:, :, :, 5] = 6.0e4
    o, lse = _run(lib, q.cuda(), k.cuda(), big.cuda(), accum="f16", scale=scale)
    oo, lo = attn_fwd(q, k, big, scale)
    og = to_f64(o)
    others = [c for c in range(D) if c != 5]
    assert np.abs(og[..., others] - oo[..., others]).max() <= TOL["f16"]
    # fp16 spacing is 32 there; one rounding per fold of a key tile, 4-7 folds here
    assert np.abs(og[..., 5] - oo[..., 5]).max() <= 2.0 ** -7 * 6.0e4
    huge = v.clone()
    huge[:, :, :, 5] = 1.0e5
    o, lse = _run(lib, q.cuda(), k.cuda(), huge.cuda(), accum="f16", scale=scale)
    oo, lo = attn_fwd(q, k, huge, scale)
    og = to_f64(o)
    assert not np.isfinite(og[..., 5]).any()
    assert np.abs(og[..., others] - oo[..., others]).max() <= TOL["f16"]
    assert np.abs(to_f64(lse) - lo).max() <= 2e-3
    o32, _ = _run(lib, q.cuda(), k.cuda(), huge.cuda(), accum="f32", scale=scale)
    assert np.abs(to_f64(o32)[..., 5] - oo[..., 5]).max() <= 2.0 ** -8 * 1.0e5 * 2


@pytest.mark.parametrize("D", [512, 1024])
@pytest.mark.parametrize("accum", ["f32", "f16"])
def test_causal_few_heads_long_rows(lib, D, accum):
    """Causal with two heads of 4096 rows: each head's query blocks fill
    several XCD ranges (for D above 512 the kernel then interleaves a head's
    blocks over those ranges)."""
    q, k, v, _ = _inputs(23, 1, 2, 2, 4096, 4096, D, "fp16")
    o, lse = _run(lib, q.cuda(), k.cuda(), v.cuda(), causal=True, accum=accum)
    _compare(o, lse, q, k, v, 1.0 / math.sqrt(D), True, None, "fp16", accum, f"causal-2x4096-D{D}-{accum}")
