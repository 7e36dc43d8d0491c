"""The C-ABI library loads, exports every function include/ffpa_attn.h declares,
and rejects invalid arguments before touching the GPU (no compute call is made:
every case below fails validation, which runs before any HIP call).
"""
import os
import re
import subprocess

import pytest

import head_dim_attention_flash_amd as ffpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffpa_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ffpa.LIB_PATH),
                                reason="library not built (python -m head_dim_attention_flash_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ffpa_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(ffpa.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ffpa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in declared_functions() if f not in syms]
    assert not missing, f"not exported: {missing}"
    lib = ffpa.load()
    for f in declared_functions():
        assert hasattr(lib, f)


def test_version_and_empty_error():
    assert ffpa.ffpa_version() >= 100
    assert isinstance(ffpa.ffpa_last_error(), str)


P = 0x10000  # a fake, 16-byte aligned non-null pointer value; never dereferenced


def fwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nkv=8, D=64, scale=0.125,
                causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0, workspace=0,
                workspace_bytes=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_fwd(*args.values())


def bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=2, Nq=8,
                Nkv=8, D=64, scale=0.125, causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0,
                workspace=0, workspace_bytes=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_bwd(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), ffpa.ERR_INVALID_ARG),
    (dict(o=0), ffpa.ERR_INVALID_ARG),
    (dict(B=0), ffpa.ERR_INVALID_ARG),
    (dict(Nq=0), ffpa.ERR_INVALID_ARG),
    (dict(Nkv=-3), ffpa.ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), ffpa.ERR_INVALID_ARG),
    (dict(causal=2), ffpa.ERR_INVALID_ARG),
    (dict(mask=P, mask_rows=3), ffpa.ERR_INVALID_ARG),
    (dict(dtype=7), ffpa.ERR_UNSUPPORTED),
    (dict(accum_dtype=5), ffpa.ERR_UNSUPPORTED),
    (dict(D=48), ffpa.ERR_UNSUPPORTED),
    (dict(D=1056), ffpa.ERR_UNSUPPORTED),
    (dict(k=P + 8), ffpa.ERR_INVALID_ARG),
    (dict(lse=P + 4), ffpa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), ffpa.ERR_INVALID_ARG),
    # many queries per key: the transposed copy of V lives in the workspace
    (dict(Nq=4096, workspace=0, workspace_bytes=0), ffpa.ERR_WORKSPACE),
    (dict(Nq=4096, workspace=P, workspace_bytes=64 * 64 * 2 * 2 - 1), ffpa.ERR_WORKSPACE),
    (dict(Nq=4096, workspace=P + 8, workspace_bytes=1 << 20), ffpa.ERR_INVALID_ARG),
])
def test_forward_validation(kw, code):
    assert fwd(**kw) == code
    assert ffpa.ffpa_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(dq=0), ffpa.ERR_INVALID_ARG),
    (dict(lse=0), ffpa.ERR_INVALID_ARG),
    (dict(Hq=4, Hkv=3), ffpa.ERR_INVALID_ARG),
    (dict(D=1100), ffpa.ERR_UNSUPPORTED),
    (dict(accum_dtype=1), ffpa.ERR_UNSUPPORTED),
    (dict(dv=P + 8), ffpa.ERR_INVALID_ARG),
    (dict(workspace=0, workspace_bytes=1 << 20), ffpa.ERR_WORKSPACE),
    (dict(workspace=P, workspace_bytes=16), ffpa.ERR_WORKSPACE),
    (dict(workspace=P, workspace_bytes=1 << 30, mask=P, mask_rows=5), ffpa.ERR_INVALID_ARG),
    (dict(workspace=P, workspace_bytes=1 << 30, D=544), ffpa.ERR_UNSUPPORTED),
    (dict(workspace=P, workspace_bytes=1 << 30, D=96), ffpa.ERR_UNSUPPORTED),
])
def test_backward_validation(kw, code):
    assert bwd(**kw) == code
    assert ffpa.ffpa_last_error() != ""


def test_forward_workspace_holds_transposed_v():
    # V^T of the size of V with Nkv rounded up to 64, in the 16-bit input type, when the
    # problem has Nq * Hq >= 3072 * Hkv (up to D = 512) or D > 512
    assert ffpa.ffpa_attn_fwd_workspace_size(1, 2, 2, 3072, 8, 64, 0) == 2 * 64 * 64 * 2
    assert ffpa.ffpa_attn_fwd_workspace_size(1, 2, 2, 3071, 8, 64, 0) == 0
    assert ffpa.ffpa_attn_fwd_workspace_size(2, 32, 8, 8192, 8191, 512, 1) == 2 * 8 * 512 * 8192 * 2
    assert ffpa.ffpa_attn_fwd_workspace_size(1, 4, 1, 800, 65, 320, 0) == 320 * 128 * 2
    assert ffpa.ffpa_attn_fwd_workspace_size(1, 32, 32, 1024, 8192, 512, 0) == 0  # cross-attention
    assert ffpa.ffpa_attn_fwd_workspace_size(1, 2, 2, 100, 300, 1024, 0) == 2 * 1024 * 320 * 2


def test_workspace_queries_are_pure_functions():
    a = ffpa.ffpa_attn_fwd_workspace_size(16, 32, 32, 1, 8192, 512, 0)
    b = ffpa.ffpa_attn_fwd_workspace_size(16, 32, 32, 1, 8192, 512, 0)
    assert a == b and a >= 0
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 32, 32, 8192, 8192, 512, 1) >= 32 * 8192 * 4


def test_backward_workspace_sizes():
    # the minimum: delta and lse * log2(e) per query row, rows padded to 64
    assert ffpa.ffpa_attn_bwd_workspace_size_min(2, 4, 2, 100, 70, 320, 0) == 2 * 2 * 4 * 128 * 4
    # stored dS: + K^T (keys padded to 64) + 2 KiB per 32 x 32 block of the heads of
    # one chunk; small problems are one chunk
    full = ffpa.ffpa_attn_bwd_workspace_size(2, 4, 2, 100, 70, 320, 0)
    assert full == 2 * 2 * 4 * 128 * 4 + 2 * 2 * 320 * 128 * 2 + 2 * 4 * 4 * 3 * 2048
    # 8K: 128 MiB of dS per head, at most 1 GiB of it: 4 chunks of 8 heads
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 32, 32, 8192, 8192, 512, 1) == (
        2 * 32 * 8192 * 4 + 32 * 512 * 8192 * 2 + 8 * 256 * 256 * 2048)
    # 16K: 512 MiB per head; 2 would fit 1 GiB, but a chunk's dQ pass needs 512
    # workgroups of 128 rows: 4 heads per chunk. GQA 32/8: a kv head's group is 4
    # query heads (2 GiB, 512 dQ workgroups)
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 32, 32, 16384, 16384, 512, 0) == (
        2 * 32 * 16384 * 4 + 32 * 512 * 16384 * 2 + 4 * 512 * 512 * 2048)
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 32, 8, 16384, 16384, 512, 0) == (
        2 * 32 * 16384 * 4 + 8 * 512 * 16384 * 2 + 1 * 4 * 512 * 512 * 2048)
    # 33 heads of 128 MiB: chunks of up to 8 (1 GiB, and 512 dQ workgroups of 64
    # rows), so 5 chunks, the heads spread evenly over them: 7 each
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 33, 33, 8192, 8192, 64, 0) == (
        2 * 33 * 8192 * 4 + 33 * 64 * 8192 * 2 + 7 * 256 * 256 * 2048)
    # up to 64 query rows: the minimum (dQ recomputes; no K transpose) ...
    assert ffpa.ffpa_attn_bwd_workspace_size(16, 32, 32, 64, 8192, 512, 0) == \
        ffpa.ffpa_attn_bwd_workspace_size_min(16, 32, 32, 64, 8192, 512, 0)
    # ... but one row takes the decode backward: fp32 dQ partials of 4 key
    # ranges per head (2048 waves over 16 x 32 kv heads)
    assert ffpa.ffpa_attn_bwd_workspace_size(16, 32, 32, 1, 8192, 512, 0) == 16 * 32 * 4 * 512 * 4
    # a group of 8 query heads per kv head has no decode backward: the minimum
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 8, 1, 1, 8192, 512, 0) == \
        ffpa.ffpa_attn_bwd_workspace_size_min(1, 8, 1, 1, 8192, 512, 0)
    # sizes of no valid problem are 0 (and compute nothing that divides by them)
    for dims in ((0, 2, 2, 1, 100, 64), (1, 0, 2, 1, 100, 64), (1, 2, 2, 0, 100, 64), (-1, 2, 2, 1, 100, 64)):
        assert ffpa.ffpa_attn_bwd_workspace_size(*dims, 0) == 0
    # and never less than the minimum (one short range, D = 64)
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 2, 2, 1, 100, 64, 0) == \
        ffpa.ffpa_attn_bwd_workspace_size_min(1, 2, 2, 1, 100, 64, 0)
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 2, 2, 65, 100, 64, 0) > \
        ffpa.ffpa_attn_bwd_workspace_size_min(1, 2, 2, 65, 100, 64, 0)
    # the stored-dS size whatever Nq: K^T (Nkv padded to 128) and dS of both kv
    # heads (32 x 32 blocks of 2048 bytes) on top of the minimum
    for nq in (1, 64, 65):
        assert ffpa.ffpa_attn_bwd_workspace_size_stored(1, 2, 2, nq, 100, 64, 0) == (
            ffpa.ffpa_attn_bwd_workspace_size_min(1, 2, 2, nq, 100, 64, 0) + 2 * 128 * 64 * 2
            + 2 * ((nq + 31) // 32) * 4 * 2048)
    assert ffpa.ffpa_attn_bwd_workspace_size_stored(1, 32, 32, 8192, 8192, 512, 1) == \
        ffpa.ffpa_attn_bwd_workspace_size(1, 32, 32, 8192, 8192, 512, 1)
    # D = 1024: 64 dQ rows per workgroup, so 4 heads suffice; the 1 GiB budget's 8 win
    assert ffpa.ffpa_attn_bwd_workspace_size(1, 32, 32, 8192, 8192, 1024, 1) == (
        2 * 32 * 8192 * 4 + 32 * 1024 * 8192 * 2 + 8 * 256 * 256 * 2048)


def fwd_noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nkv=8, D=64, scale=0.125,
                causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_fwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), ffpa.ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), ffpa.ERR_INVALID_ARG),
    (dict(D=1056), ffpa.ERR_UNSUPPORTED),
    (dict(lse=P + 4), ffpa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), ffpa.ERR_INVALID_ARG),
    # above D = 512 the transposed copy of V is required: 64 MiB > the 32 MiB scratch
    (dict(B=1, Hq=4, Hkv=4, Nq=4096, Nkv=8192, D=1024), ffpa.ERR_WORKSPACE),
    # decode partials of 8192 heads x 1 key range x 1025 floats > 32 MiB
    (dict(B=1024, Hq=8, Hkv=8, Nq=1, Nkv=4096, D=1024), ffpa.ERR_WORKSPACE),
])
def test_forward_noalloc_validation(kw, code):
    assert fwd_noalloc(**kw) == code
    assert ffpa.ffpa_last_error() != ""


def fwd_drop(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nkv=8, D=64, scale=0.125,
                causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0, dropout_p=0.1, seed=7,
                workspace=0, workspace_bytes=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_fwd_dropout(*args.values())


def bwd_drop(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=2, Nq=8,
                Nkv=8, D=64, scale=0.125, causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0,
                dropout_p=0.1, seed=7, workspace=0, workspace_bytes=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_bwd_dropout(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), ffpa.ERR_INVALID_ARG),
    (dict(D=1056), ffpa.ERR_UNSUPPORTED),
    (dict(lse=P + 4), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=1.0), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=-0.01), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=float("nan")), ffpa.ERR_INVALID_ARG),
    # p is checked before the workspace; the fp16 accumulator has no dropout
    (dict(dropout_p=2.0, Nq=4096), ffpa.ERR_INVALID_ARG),
    (dict(accum_dtype=1), ffpa.ERR_UNSUPPORTED),
    (dict(accum_dtype=1, D=1024), ffpa.ERR_UNSUPPORTED),
    (dict(Nq=4096), ffpa.ERR_WORKSPACE),
])
def test_forward_dropout_validation(kw, code):
    assert fwd_drop(**kw) == code
    assert ffpa.ffpa_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(dq=0), ffpa.ERR_INVALID_ARG),
    (dict(accum_dtype=1), ffpa.ERR_UNSUPPORTED),
    (dict(dv=P + 8), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=1.5), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=float("inf")), ffpa.ERR_INVALID_ARG),
    (dict(dropout_p=0.5), ffpa.ERR_WORKSPACE),
    (dict(dropout_p=0.5, workspace=P, workspace_bytes=16), ffpa.ERR_WORKSPACE),
])
def test_backward_dropout_validation(kw, code):
    assert bwd_drop(**kw) == code
    assert ffpa.ffpa_last_error() != ""


def test_binding_rejects_bad_seed():
    with pytest.raises(ValueError):
        ffpa._seed(-1)
    with pytest.raises(ValueError):
        ffpa._seed(1 << 64)
    assert ffpa._seed((1 << 64) - 1) == (1 << 64) - 1


def fwd_var(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nkv=8, D=64, scale=0.125,
                causal=0, mask=0, mask_rows=0, accum_dtype=0, dtype=0, variant=1, workspace=0,
                workspace_bytes=0, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_fwd_variant(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), ffpa.ERR_INVALID_ARG),
    (dict(variant=4), ffpa.ERR_INVALID_ARG),
    (dict(variant=-1), ffpa.ERR_INVALID_ARG),
    (dict(variant=3), ffpa.ERR_INVALID_ARG),                      # prefill has variants 1 and 2
    (dict(variant=2), ffpa.ERR_WORKSPACE),                        # V^T needs workspace
    (dict(variant=2, D=640), ffpa.ERR_INVALID_ARG),               # fp16-accumulator shape, fp32 asked
    (dict(variant=2, D=832, accum_dtype=1), ffpa.ERR_INVALID_ARG),  # all of D in a wave: D <= 768
    (dict(variant=3, D=832, accum_dtype=1), ffpa.ERR_WORKSPACE),
    (dict(variant=3, Nq=1), ffpa.ERR_WORKSPACE),                  # decode, fewer key ranges
])
def test_forward_variant_validation(kw, code):
    assert fwd_var(**kw) == code
    assert ffpa.ffpa_last_error() != ""


def test_variant_workspace_sizes():
    vt = 2 * 8 * 640 * 512 * 2  # V^T of B=2, Hkv=8, Nkv=600 (padded to 640), D=512, fp16
    assert ffpa.ffpa_attn_fwd_variant_workspace_size(2, 8, 8, 100, 600, 512, 0, 0, 1) == 0
    assert ffpa.ffpa_attn_fwd_variant_workspace_size(2, 8, 8, 100, 600, 512, 0, 0, 2) == vt
    assert ffpa.ffpa_attn_fwd_variant_workspace_size(2, 8, 8, 100, 600, 512, 0, 0, 0) == \
        ffpa.ffpa_attn_fwd_workspace_size(2, 8, 8, 100, 600, 512, 0)
    # decode: the default key ranges / 1, 2, 4 (never more than the default size)
    sizes = [ffpa.ffpa_attn_fwd_variant_workspace_size(1, 4, 4, 1, 65536, 512, 0, 0, v) for v in (1, 2, 3)]
    assert sizes[0] == ffpa.ffpa_attn_fwd_workspace_size(1, 4, 4, 1, 65536, 512, 0)
    assert sizes[0] >= sizes[1] >= sizes[2] > 0
    assert ffpa.ffpa_attn_fwd_variant_workspace_size(1, 4, 4, 1, 64, 512, 0, 0, 9) == 0


def test_tune_validation():
    st, _, _ = ffpa.ffpa_attn_fwd_tune(P, P, P, P, P, 1, 2, 2, 8, 8, 64, 0.125, 0, 0, 0, 0, 0, 0, 0, 3, 0)
    assert st == ffpa.ERR_INVALID_ARG  # level must be 1 or 2
    st, _, _ = ffpa.ffpa_attn_fwd_tune(0, P, P, P, P, 1, 2, 2, 8, 8, 64, 0.125, 0, 0, 0, 0, 0, 0, 0, 1, 0)
    assert st == ffpa.ERR_INVALID_ARG
    # D above 512: every variant needs the transposed copy of V; none fits no workspace
    st, _, ms = ffpa.ffpa_attn_fwd_tune(P, P, P, P, P, 1, 2, 2, 8, 8, 640, 0.125, 0, 0, 0, 0, 0, 0, 0, 1, 0)
    assert st == ffpa.ERR_WORKSPACE and ms == [-1.0, -1.0, -1.0]
    ffpa.ffpa_attn_tune_reset()


def fp8(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nkv=8, D=128, scale=0.125,
                causal=0, dtype=0, workspace=P, workspace_bytes=1 << 30, stream=0)
    args.update(kw)
    return ffpa.ffpa_attn_fwd_fp8(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), ffpa.ERR_INVALID_ARG),
    (dict(Nq=0), ffpa.ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), ffpa.ERR_INVALID_ARG),
    (dict(k=P + 8), ffpa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), ffpa.ERR_INVALID_ARG),
    (dict(dtype=7), ffpa.ERR_UNSUPPORTED),
    (dict(D=64), ffpa.ERR_UNSUPPORTED),      # built for D = 128 .. 512, multiples of 64
    (dict(D=160), ffpa.ERR_UNSUPPORTED),
    (dict(D=576), ffpa.ERR_UNSUPPORTED),
    (dict(workspace=P + 8), ffpa.ERR_INVALID_ARG),
    (dict(workspace=0), ffpa.ERR_WORKSPACE),
    (dict(workspace_bytes=1024), ffpa.ERR_WORKSPACE),
])
def test_fp8_validation(kw, code):
    assert fp8(**kw) == code
    assert ffpa.ffpa_last_error() != ""


def test_fp8_workspace_size():
    """amax (3 B Hq floats, 256-aligned), Q8, K8 and V8^T (keys padded to 64),
    each 256-byte aligned; 0 for invalid sizes."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hq, Hkv, Nq, Nkv, D in ((1, 32, 32, 8192, 8192, 512), (2, 4, 1, 100, 130, 192), (1, 1, 1, 1, 1, 128)):
        want = up(3 * B * Hq * 4) + up(B * Hq * Nq * D) + up(B * Hkv * Nkv * D) + up(B * Hkv * ((Nkv + 63) // 64) * 64 * D)
        assert ffpa.ffpa_attn_fwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nkv, D) == want
    assert ffpa.ffpa_attn_fwd_fp8_workspace_size(1, 2, 2, 0, 8, 128) == 0
