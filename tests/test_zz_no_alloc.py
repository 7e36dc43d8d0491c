"""ffpa_attn_fwd_noalloc (the forward that allocates nothing) against
ffpa_attn_fwd, through the C ABI, two calls in a row per case, the second on
a smaller problem (the shared scratch array keeps the first call's contents).

Where the regular call's workspace fits the 32 MiB scratch, the two entry
points run the same kernels on the same data: the outputs must be identical
bit for bit. Where it does not (a D <= 512 prefill whose V^T copy would exceed
it), the no-alloc call stages V as is, and its outputs must meet the parity
bar against the regular call's: max |dO| <= 1e-2 (fp32 accumulation) and the
relative L2 bound of the fp16 parity tests, lse within 2e-3.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import to_f64

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20


def _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, mask_kind):
    q = W.draw(seed, W.T_Q, B, Hq, Nq, D, dtype, device="cuda")
    k = W.draw(seed, W.T_K, B, Hkv, Nkv, D, dtype, device="cuda")
    v = W.draw(seed, W.T_V, B, Hkv, Nkv, D, dtype, device="cuda")
    mask = None
    if mask_kind is not None:
        mask = W.draw_key_bias(seed, Nkv, dtype, 0.1, rows=1 if mask_kind == "key" else Nq,
                               device="cuda")
        mask[:, 0] = 0.0
    return q, k, v, mask


def _noalloc(lib, q, k, v, causal, mask, accum, scale):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=q.device)
    dt = lib.BF16 if q.dtype == torch.bfloat16 else lib.F16
    rows = 0 if mask is None else mask.numel() // Nkv
    st = lib.ffpa_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, scale, int(causal),
                                   0 if mask is None else mask.data_ptr(), rows,
                                   lib.ACC_F16 if accum == "f16" else lib.ACC_F32, dt,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ffpa_last_error()
    return o, lse


# (first problem, second smaller problem): (B, Hq, Hkv, Nq, Nkv, D, dtype, accum, causal, mask)
PAIRS = [
    # decode: split-KV partials in the scratch
    ((4, 16, 8, 1, 3000, 512, "fp16", "f32", False, None),
     (2, 8, 8, 1, 700, 256, "bf16", "f32", False, "key")),
    # prefill with the transposed copy of V in the scratch
    ((1, 2, 2, 3100, 300, 512, "fp16", "f32", True, None),
     (1, 1, 1, 3072, 64, 320, "bf16", "f16", False, "key")),
    # above D = 512 (the transposed copy in blocks of 32 keys), both accumulators
    ((1, 2, 2, 200, 333, 768, "fp16", "f16", False, "query"),
     (1, 2, 1, 70, 40, 640, "bf16", "f32", True, None)),
    # no transposed copy needed (few queries per key)
    ((1, 8, 8, 1024, 2048, 512, "fp16", "f32", False, "key"),
     (1, 2, 2, 64, 90, 128, "fp16", "f16", True, None)),
]


def _fits(p):
    B, Hq, Hkv, Nq, Nkv, D, dtype = p[:7]
    import head_dim_attention_flash_amd as ffpa
    return ffpa.ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, 0) <= SCRATCH


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][3]}x{p[0][4]}x{p[0][5]}")
def test_noalloc_matches_fwd_bitwise(lib, pair):
    for i, p in enumerate(pair):
        B, Hq, Hkv, Nq, Nkv, D, dtype, accum, causal, mk = p
        print(f"noalloc call {i}: {p}", flush=True)
        assert _fits(p)
        q, k, v, mask = _inputs(40 + i + sum(p[:6]), B, Hq, Hkv, Nq, Nkv, D, dtype, mk)
        scale = 1.0 / math.sqrt(D)
        o_ref, l_ref = lib.attention(q, k, v, causal=causal, mask=mask, scale=scale, accum=accum,
                                     return_lse=True)
        o, lse = _noalloc(lib, q, k, v, causal, mask, accum, scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i}: O differs from ffpa_attn_fwd"
        assert torch.equal(torch.nan_to_num(lse, nan=7.0), torch.nan_to_num(l_ref, nan=7.0)), \
            f"call {i}: lse differs from ffpa_attn_fwd"


def test_noalloc_without_transposed_copy(lib):
    """A prefill whose V^T copy exceeds the scratch (B1 H8 N8192 D512: 64 MiB)
    stages V as is; then a smaller problem that fits reuses the scratch."""
    for i, p in enumerate([(1, 8, 8, 8192, 8192, 512, "fp16", "f32", False, "key"),
                           (1, 2, 2, 3100, 500, 512, "fp16", "f32", True, None)]):
        B, Hq, Hkv, Nq, Nkv, D, dtype, accum, causal, mk = p
        print(f"noalloc call {i}: {p}", flush=True)
        q, k, v, mask = _inputs(60 + i, B, Hq, Hkv, Nq, Nkv, D, dtype, mk)
        scale = 1.0 / math.sqrt(D)
        o_ref, l_ref = lib.attention(q, k, v, causal=causal, mask=mask, scale=scale, accum=accum,
                                     return_lse=True)
        o, lse = _noalloc(lib, q, k, v, causal, mask, accum, scale)
        torch.cuda.synchronize()
        if _fits(p):
            assert torch.equal(o, o_ref)
            continue
        d = to_f64(o) - to_f64(o_ref)
        rel = np.linalg.norm(d) / np.linalg.norm(to_f64(o_ref))
        print(f"  max|dO|={np.abs(d).max():.3e} relL2={rel:.3e}", flush=True)
        assert np.isfinite(to_f64(o)).all()
        assert np.abs(d).max() <= 1e-2 and rel <= 4e-3
        assert (lse - l_ref).abs().max().item() <= 2e-3


def test_noalloc_rejects_what_does_not_fit(lib):
    """Above D = 512 the transposed copy is required: B1 H4 N8192 D1024 needs
    64 MiB and is refused before any launch (the output stays untouched)."""
    q = torch.zeros(1, 4, 4096, 1024, dtype=torch.float16, device="cuda")
    k = torch.zeros(1, 4, 8192, 1024, dtype=torch.float16, device="cuda")
    o = torch.full_like(q, 3.0)
    st = lib.ffpa_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), 0,
                                   1, 4, 4, 4096, 8192, 1024, 0.03125, 0, 0, 0, lib.ACC_F32, lib.F16,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == lib.ERR_WORKSPACE
    assert "scratch" in lib.ffpa_last_error()
    assert torch.all(o == 3.0)
