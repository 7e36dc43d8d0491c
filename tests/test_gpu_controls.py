"""Negative controls of the parity gate, and a bounded fuzz of the HIP path.

Negative controls (Tiny configuration, B1 H2 N256 D320 fp16; a GQA variant
Hq=4/Hkv=2 for the head map): the library's output, which passes the gate
against the oracle, must FAIL the same gate against an oracle with a planted
mistake of the kind a kernel could make. The mistakes are planted on the CPU,
in what the oracle is given: the other GQA head map (h % Hkv instead of
h // g), the last key tile (64 keys) dropped, the causal diagonal off by one,
and an all-zero output. The gate is the judged one (max |dO| <= 1e-2) with
the relative L2 bound of the parity tests (4e-3 for fp16).

Fuzz: hypothesis draws small shapes and options (batch, heads and GQA group,
lengths down to 1 and ragged, D, dtype, accumulator, causal, either mask
shape) and checks the forward against the oracle with the element-wise bound
of test_gpu_fwd; derandomized, 60 examples, and no shrinking, so that a
failure stops the run at the first failing case (printed before it runs).
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import workloads as W
from oracle import attn_fwd, to_f64
from test_gpu_fwd import _compare, _inputs

pytestmark = pytest.mark.gpu


def gate_passes(o, ref, tol=1e-2, rel_bound=4e-3):
    """The parity gate: max abs error and relative L2 error."""
    d = to_f64(o) - ref
    err = np.abs(d).max()
    rel = np.linalg.norm(d) / np.linalg.norm(ref)
    return err <= tol and rel <= rel_bound, err, rel


@pytest.fixture(scope="module")
def tiny(lib):
    w = W.WORKLOADS["tiny"]
    inp = W.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = lib.attention(q.cuda(), k.cuda(), v.cuda(), scale=w.scale).cpu()
    oc = lib.attention(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True).cpu()
    torch.cuda.synchronize()
    return w, q, k, v, o, oc


def test_tiny_passes_its_own_gate(tiny):
    w, q, k, v, o, oc = tiny
    ok, err, rel = gate_passes(o, attn_fwd(q, k, v, w.scale)[0])
    assert ok, (err, rel)
    ok, err, rel = gate_passes(oc, attn_fwd(q, k, v, w.scale, causal=True)[0])
    assert ok, (err, rel)


def test_control_dropped_last_key_tile_fails(tiny):
    w, q, k, v, o, _ = tiny
    ok, err, rel = gate_passes(o, attn_fwd(q, k[:, :, :-64], v[:, :, :-64], w.scale)[0])
    print(f"dropped last key tile: max|dO|={err:.3e} relL2={rel:.3e}")
    assert not ok


def test_control_off_by_one_causal_fails(tiny):
    w, q, k, v, _, oc = tiny
    # the diagonal one key late: query i sees keys j <= i + 1 (a planted mask)
    n = q.shape[2]
    shifted = torch.where(torch.arange(n)[None, :] <= torch.arange(n)[:, None] + 1, 0.0,
                          float("-inf")).to(torch.float16)
    ok, err, rel = gate_passes(oc, attn_fwd(q, k, v, w.scale, mask=shifted)[0])
    print(f"off-by-one causal: max|dO|={err:.3e} relL2={rel:.3e}")
    assert not ok


def test_control_zero_output_fails(tiny):
    w, q, k, v, o, _ = tiny
    ok, err, rel = gate_passes(torch.zeros_like(o), attn_fwd(q, k, v, w.scale)[0])
    print(f"zero output: max|dO|={err:.3e} relL2={rel:.3e}")
    assert not ok


def test_control_wrong_gqa_map_fails(lib):
    w = W.WORKLOADS["tiny"]
    q, k, v, _ = _inputs(w.cfg_id, 1, 4, 2, 256, 256, 320, "fp16")
    o = lib.attention(q.cuda(), k.cuda(), v.cuda(), scale=w.scale).cpu()
    torch.cuda.synchronize()
    ok, err, rel = gate_passes(o, attn_fwd(q, k, v, w.scale)[0])
    assert ok, (err, rel)
    # planted: query head h reads kv head h % Hkv instead of h // (Hq / Hkv)
    kk = k[:, [0, 1, 0, 1]].contiguous()
    vv = v[:, [0, 1, 0, 1]].contiguous()
    ok, err, rel = gate_passes(o, attn_fwd(q, kk, vv, w.scale)[0])
    print(f"wrong GQA map: max|dO|={err:.3e} relL2={rel:.3e}")
    assert not ok


@st.composite
def problems(draw):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 3))
    g = draw(st.sampled_from([1, 2, 4]))
    Nq = draw(st.one_of(st.just(1), st.integers(2, 300)))
    Nkv = draw(st.integers(1, 300))
    # Nq > 1 is built for D a multiple of 64; decode for every multiple of 32
    D = draw(st.sampled_from(range(64, 1025, 64) if Nq > 1 else range(32, 1025, 32)))
    dtype = draw(st.sampled_from(["fp16", "bf16"]))
    accum = draw(st.sampled_from(["f32", "f16"]))
    causal = draw(st.booleans())
    mask = draw(st.sampled_from([None, "key", "query"]))
    seed = draw(st.integers(0, 10 ** 6))
    return B, Hkv * g, Hkv, Nq, Nkv, D, dtype, accum, causal, mask, seed


@settings(max_examples=60, deadline=None, derandomize=True, phases=[Phase.generate],
          report_multiple_bugs=False, suppress_health_check=list(HealthCheck))
@given(problems())
def test_fuzz_forward_matches_oracle(lib, p):
    B, Hq, Hkv, Nq, Nkv, D, dtype, accum, causal, mk, seed = p
    print(f"fuzz case B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} {dtype} acc={accum} "
          f"causal={causal} mask={mk} seed={seed}", flush=True)
    q, k, v, mask = _inputs(seed, B, Hq, Hkv, Nq, Nkv, D, dtype, mk)
    if mask is not None:
        mask[:, 0] = 0.0  # key 0 stays visible: a causal row 0 is never empty
    scale = 1.0 / math.sqrt(D)
    o, lse = lib.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                           mask=None if mask is None else mask.cuda(), scale=scale, accum=accum,
                           return_lse=True)
    torch.cuda.synchronize()
    _compare(o, lse, q, k, v, scale, causal, mask, dtype, accum, "fuzz")
