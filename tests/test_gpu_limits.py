"""The largest problems the library accepts, through the C ABI.

The API takes (N + 128) D < 2^31 elements per (b, h) slice, so that every
byte offset inside a slice (and inside the transposed copies of V and K,
padded to whole tiles) fits the 32-bit offsets of the buffer loads. These
tests run right under that limit, where a 32-bit overflow anywhere in the
addressing would show: Nkv = 2^31 / D - 129 keys (ragged, not a multiple of
the tile), at D = 1024 and 512.

The float64 oracle cannot hold 2 M x 1024 keys, so the checks are properties
that hold at any size: K is zero except one key per target, at 10 in a
column c, and query i is 8 e_c for its target's column, so (scale 1) query i
scores 80 on its target key and 0 on every other one. Its softmax weight on
the others is e^-80 per key (2e-35: under fp16's range, so P puts exactly
0 there), hence O_i = V[target] exactly and lse_i = 80 to fp32 rounding. The
targets sit at the first and last keys, at tile boundaries and in the middle.
The backward of the same problem has dV[target] = the sum of dO over the
queries that attend it, dV = 0 on every other key, and dQ, dK = 0 up to the
rounding of dP - delta (dS = P (dP - delta) vanishes when P is one-hot);
with bf16 operands P keeps 2^-115 on the other keys, so their dV is ~1e-33
rather than 0. The decode backward (one query row) is checked the same way."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

D_LIMITS = {1024: (1 << 31) // 1024 - 129, 512: (1 << 31) // 512 - 129}


def _problem(D, Hq, Nq, dtype=torch.float16):
    """q, k, v on the GPU (B = 1, Hkv = 1), the target key of each query and
    the column each query uses."""
    Nkv = D_LIMITS[D]
    targets = [0, 1, 63, 64, Nkv // 2, Nkv - 65, Nkv - 2, Nkv - 1]
    k = torch.zeros(1, 1, Nkv, D, dtype=dtype, device="cuda")
    for c, t in enumerate(targets):
        k[0, 0, t, c] = 10.0
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    v = torch.randn(1, 1, Nkv, D, generator=g, device="cuda", dtype=torch.float32).to(dtype)
    q = torch.zeros(1, Hq, Nq, D, dtype=dtype, device="cuda")
    cols = [(h * Nq + i) % len(targets) for h in range(Hq) for i in range(Nq)]
    qi = torch.tensor(cols, device="cuda").view(Hq, Nq)
    q[0].scatter_(2, qi.unsqueeze(-1), 8.0)
    return q, k, v, targets, qi


def _run_variant(lib, q, k, v, variant, accum):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    dt = lib.BF16 if q.dtype == torch.bfloat16 else lib.F16
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device="cuda")
    ws_bytes = lib.ffpa_attn_fwd_variant_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt, 0, variant)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    st = lib.ffpa_attn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   B, Hq, Hkv, Nq, Nkv, D, 1.0, 0, 0, 0,
                                   lib.ACC_F16 if accum == "f16" else lib.ACC_F32, dt, variant,
                                   ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ffpa_last_error()
    torch.cuda.synchronize()
    del ws
    return o, lse


def _check_forward(o, lse, v, targets, qi, label):
    want = v[0, 0][torch.tensor(targets, device="cuda")[qi]]  # [Hq, Nq, D]
    diff = (o[0].float() - want.float()).abs().max().item()
    dl = (lse[0] - 80.0).abs().max().item()
    print(f"{label}: max|O - V[target]| = {diff:.3e}, max|lse - 80| = {dl:.3e}", flush=True)
    assert diff == 0.0, label
    assert dl <= 1e-4, label


@pytest.mark.parametrize("D,accum,variant", [(1024, "f32", 1), (1024, "f16", 3), (512, "f32", 1),
                                             (512, "f32", 2)], ids=str)
def test_forward_at_the_size_limit(lib, D, accum, variant):
    print(f"case limit forward D={D} Nkv={D_LIMITS[D]} accum={accum} variant={variant}", flush=True)
    q, k, v, targets, qi = _problem(D, Hq=8, Nq=256)
    o, lse = _run_variant(lib, q, k, v, variant, accum)
    _check_forward(o, lse, v, targets, qi, f"forward D={D} {accum} variant {variant}")


def test_decode_at_the_size_limit(lib):
    D = 1024
    print(f"case limit decode D={D} Nkv={D_LIMITS[D]}", flush=True)
    q, k, v, targets, qi = _problem(D, Hq=32, Nq=1)
    o, lse = lib.attention(q, k, v, scale=1.0, return_lse=True)
    torch.cuda.synchronize()
    _check_forward(o, lse, v, targets, qi, "decode D=1024")


def test_backward_at_the_size_limit(lib):
    D = 1024
    print(f"case limit backward D={D} Nkv={D_LIMITS[D]}", flush=True)
    q, k, v, targets, qi = _problem(D, Hq=8, Nq=256, dtype=torch.bfloat16)
    o, lse = lib.attention(q, k, v, scale=1.0, return_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = lib.attention_backward(dout, q, k, v, o, lse, scale=1.0)
    torch.cuda.synchronize()
    t_idx = torch.tensor(targets, device="cuda")
    # dV on the targets: sum of dO over the queries (of every head) attending each
    want = torch.zeros(len(targets), D, device="cuda")
    want.index_add_(0, qi.reshape(-1), dout[0].reshape(-1, D).float())
    got = dv[0, 0, t_idx].float()
    err = (got - want).abs().max().item()
    scale_ref = want.abs().max().item()
    print(f"backward D=1024: max|dV[target] - sum dO| = {err:.3e} (max |sum| {scale_ref:.2f})", flush=True)
    assert err <= 1e-2 + 2.0 ** -8 * scale_ref
    mask = torch.ones(dv.shape[2], dtype=torch.bool, device="cuda")
    mask[t_idx] = False
    # bf16 P keeps 2^-115 (fp32's exponent range): the other keys get ~1e-33
    assert dv[0, 0][mask].abs().max().item() <= 1e-30
    dk_max, dq_max = dk.abs().max().item(), dq.abs().max().item()
    print(f"backward D=1024: max|dK| = {dk_max:.3e}, max|dQ| = {dq_max:.3e}", flush=True)
    assert dk_max <= 5e-2 and dq_max <= 1e-2


def test_decode_backward_at_the_size_limit(lib):
    """One query row per head at the largest Nkv: the decode backward's key
    ranges and row offsets span the whole 2^31-element slice."""
    D = 1024
    print(f"case limit decode backward D={D} Nkv={D_LIMITS[D]}", flush=True)
    q, k, v, targets, qi = _problem(D, Hq=8, Nq=1, dtype=torch.bfloat16)
    o, lse = lib.attention(q, k, v, scale=1.0, return_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(98)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = lib.attention_backward(dout, q, k, v, o, lse, scale=1.0)
    torch.cuda.synchronize()
    t_idx = torch.tensor(targets, device="cuda")
    want = torch.zeros(len(targets), D, device="cuda")
    want.index_add_(0, qi.reshape(-1), dout[0].reshape(-1, D).float())
    err = (dv[0, 0, t_idx].float() - want).abs().max().item()
    scale_ref = want.abs().max().item()
    print(f"decode backward D=1024: max|dV[target] - sum dO| = {err:.3e} (max |sum| {scale_ref:.2f})", flush=True)
    assert err <= 1e-2 + 2.0 ** -8 * scale_ref
    mask = torch.ones(dv.shape[2], dtype=torch.bool, device="cuda")
    mask[t_idx] = False
    # P of the other keys is e^-80 in fp32 (the decode backward keeps P in
    # fp32): their dV is ~1e-35
    assert dv[0, 0][mask].abs().max().item() <= 1e-30
    dk_max, dq_max = dk.abs().max().item(), dq.abs().max().item()
    print(f"decode backward D=1024: max|dK| = {dk_max:.3e}, max|dQ| = {dq_max:.3e}", flush=True)
    assert dk_max <= 5e-2 and dq_max <= 1e-2
