"""Forward variants and the tuner (ffpa_attn_fwd_variant, ffpa_attn_fwd_tune)
through the C ABI.

Every variant of a problem is checked against the float64 oracle with the
bounds of test_gpu_fwd (fp16-accumulator variants with the fp16 accumulator's
bound). The tuner must pick a variant that exists, time only the variants
that fit, and make later ffpa_attn_fwd calls of the same problem give exactly
the bits of that variant (and the default's again after ffpa_attn_tune_reset).
"""
import math

import pytest
import torch

from test_gpu_fwd import _compare, _inputs

pytestmark = pytest.mark.gpu


def run_variant(lib, q, k, v, variant, *, causal=False, accum="f32"):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    dt = lib.BF16 if q.dtype == torch.bfloat16 else lib.F16
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    ws_bytes = lib.ffpa_attn_fwd_variant_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt, int(causal), variant)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    st = lib.ffpa_attn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   B, Hq, Hkv, Nq, Nkv, D, 1.0 / math.sqrt(D), int(causal), 0, 0,
                                   lib.ACC_F16 if accum == "f16" else lib.ACC_F32, dt, variant,
                                   ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ffpa_last_error()
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (shape (B, Hq, Hkv, Nq, Nkv, D), accum, variants)
    ((1, 2, 2, 200, 150, 320), "f32", (1, 2)),
    ((1, 4, 1, 300, 257, 512), "f16", (1, 2)),
    ((1, 2, 2, 200, 150, 576), "f16", (1, 2, 3)),
    ((1, 2, 1, 130, 100, 704), "f16", (1, 2, 3)),
    ((2, 2, 2, 100, 90, 768), "f16", (1, 2, 3)),
    ((1, 2, 2, 100, 80, 832), "f16", (1, 3)),
    ((1, 2, 1, 70, 130, 1024), "f16", (1, 3)),
    ((1, 2, 2, 100, 80, 640), "f32", (1,)),
    ((2, 4, 2, 1, 3000, 512), "f32", (1, 2, 3)),   # decode: key ranges / 1, 2, 4
    ((1, 2, 2, 1, 700, 1024), "f32", (1, 2, 3)),
]


@pytest.mark.parametrize("shape,accum,variants", CASES, ids=lambda c: str(c))
@pytest.mark.parametrize("causal", [False, True])
def test_every_variant_matches_oracle(lib, shape, accum, variants, causal):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v, _ = _inputs(400 + D, B, Hq, Hkv, Nq, Nkv, D, "fp16")
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    for var in variants:
        # the fp32-accumulator wide variant is also what an fp16 request may get
        acc = "f32" if (D > 512 and var == 1) or Nq == 1 else accum
        o, lse = run_variant(lib, qc, kc, vc, var, causal=causal, accum=accum)
        _compare(o, lse, q, k, v, 1.0 / math.sqrt(D), causal, None, "fp16", acc,
                 f"{shape}-{accum}-variant{var}-{'causal' if causal else 'full'}")


@pytest.mark.parametrize("shape,accum", [((1, 8, 8, 512, 2048, 512), "f32"), ((1, 4, 4, 256, 1024, 640), "f16"),
                                         ((4, 8, 8, 1, 8192, 512), "f32")], ids=str)
@pytest.mark.parametrize("level", [1, 2])
def test_tuner_choice_is_used_by_later_calls(lib, shape, accum, level):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v, _ = _inputs(77, B, Hq, Hkv, Nq, Nkv, D, "fp16")
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    lib.ffpa_attn_tune_reset()
    try:
        default = lib.attention(qc, kc, vc, accum=accum)
        chosen, times = lib.tune_forward(qc, kc, vc, accum=accum, level=level)
        print(f"{shape} {accum} level {level}: chosen {chosen}, ms {times}", flush=True)
        assert chosen in times and all(t > 0 for t in times.values())
        assert times[chosen] == min(times.values())
        tuned = lib.attention(qc, kc, vc, accum=accum)
        explicit, _ = run_variant(lib, qc, kc, vc, chosen, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(tuned, explicit)
    finally:
        lib.ffpa_attn_tune_reset()
    again = lib.attention(qc, kc, vc, accum=accum)
    torch.cuda.synchronize()
    assert torch.equal(again, default)
