"""Benchmark of the large-head-dimension attention forward on one MI355X.

Default workload (the headline metric): self-attention forward, B=1, Hq=Hkv=32,
Nq=Nkv=8192, D=512, fp16 inputs, N(0, 1) synthetic data, fp32 output
accumulation. One "step" is one forward call (every kernel of the path).

TFLOPS follow the convention of "FFPA Attention Benchmark" (section "More
Benchmark"): the forward counts 2 GEMMs = 4 B Hq Nq Nkv D flops, the backward
the standard 5 = 10 B Hq Nq Nkv D, and a causal pass half of that.

Prints ONE JSON line. Besides the headline forward it carries, under
"paths", the other two parts of the hot path measured in the same run:
the backward (B=1, H=32, N=8192, D=512, bf16, dQ/dK/dV after this library's
forward; TFLOPS counted as 5 GEMMs) and the decode forward (B=16, H=32,
Nq=1, Nkv=8192, D=512, fp16; HBM GB/s of its algorithmic bytes against the
8 TB/s HBM3E peak). ``--suite`` instead times every workload family and
prints one line per workload (not the headline contract).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6}  # MI355X dense MFMA, published
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("head_dim_attention_flash_amd/csrc/fwd_prefill.hpp",
                  "head_dim_attention_flash_amd/csrc/fwd_vt.hpp",
                  "head_dim_attention_flash_amd/csrc/fwd_vt.hip",
                  "head_dim_attention_flash_amd/csrc/ffpa_common.hpp")
COPY_BYTES = 1 << 30  # the calibration copy moves 1 GiB in and 1 GiB out


CSRC = "head_dim_attention_flash_amd/csrc/"
# sources each family of recorded counters was taken on
COUNTER_SOURCES = {
    "fwd": KERNEL_SOURCES,
    "wide": KERNEL_SOURCES + (CSRC + "fwd_wide.hpp",),
    "wide16": KERNEL_SOURCES + (CSRC + "fwd_wide.hpp", CSRC + "fwd_wide16.hpp"),
    "bwd": (CSRC + "bwd.hpp", CSRC + "ffpa_common.hpp", CSRC + "fwd_vt.hpp", CSRC + "fwd_vt.hip"),
    "decode": (CSRC + "decode.hpp", CSRC + "ffpa_common.hpp"),
    "dec_bwd": (CSRC + "dec_bwd.hpp", CSRC + "decode.hpp", CSRC + "ffpa_common.hpp"),
    "fp8": (CSRC + "fwd_fp8.hpp", CSRC + "ffpa_common.hpp"),
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the code in `sources`, comments and blank lines left out (a
    record taken on a kernel stays valid through edits of its comments)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = re.sub(r"//.*", "", line).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch recorded by rocprofv3 counters for `key`, or None if
    the record is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_hash():
        return None
    return int(rec["hbm_bytes"])


def recorded_counters(key: str):
    """rocprofv3 counter values recorded in profiles/counters.json for `key`
    (MFMA utilisation, HBM bytes), or None if missing or taken on other sources."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    family = rec.get("family") if rec else None
    if not rec or family not in COUNTER_SOURCES or \
            rec.get("source_sha") != kernel_source_hash(COUNTER_SOURCES[family]):
        return None
    return {k: v for k, v in rec.items() if k not in ("family", "source_sha", "command")}


def counted_flops(B, Hq, Nq, Nkv, D, causal=False, backward=False) -> float:
    """Flops credited to one pass: 2 (fwd) or 5 (bwd) GEMMs of 2 B Hq Nq Nkv D, halved if causal."""
    f = (10.0 if backward else 4.0) * B * Hq * Nq * Nkv * D
    return f * 0.5 if causal else f


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, heads: int) -> dict:
    """The float64 oracle timed on the host on `heads` query heads of the workload.

    The inputs are copied to the host and widened to float64 before the clock
    starts; the timed region is the oracle's arithmetic alone. The value is the
    sample's own throughput (counted flops of the heads timed / time), not an
    extrapolation: the heads are independent and identical in work."""
    from oracle import attn_fwd, to_f64

    g = w.Hq // w.Hkv
    hk = max(1, (heads + g - 1) // g)
    q = to_f64(inp["q"][:, :heads])
    k = to_f64(inp["k"][:, :hk])
    v = to_f64(inp["v"][:, :hk])
    mask = None if inp.get("mask") is None else to_f64(inp["mask"])
    t0 = time.perf_counter()
    attn_fwd(q, k, v, w.scale, causal=w.causal, mask=mask)
    dt = time.perf_counter() - t0
    fl = counted_flops(1, heads, w.Nq, w.Nkv, w.D, w.causal)
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": _blas_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{heads} of {w.B * w.Hq} (b, h) heads of the same workload, float64 numpy, "
                      f"{dt:.2f} s"}


def time_forward(ffpa, w, inp, accum, steps, warmup, any_variant=False):
    import torch

    q, k, v, mask = inp["q"], inp["k"], inp["v"], inp.get("mask")
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Nq, dtype=torch.float32, device=q.device)
    # caller-owned workspace, allocated once (the transposed V of the prefill
    # path); any_variant: room for whichever variant a tuning run picked
    dt = ffpa.BF16 if w.dtype == "bf16" else ffpa.F16
    ws_bytes = ffpa.ffpa_attn_fwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, dt)
    if any_variant:
        ws_bytes = max(ffpa.ffpa_attn_fwd_variant_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, dt,
                                                                 int(w.causal), var) for var in range(4))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)

    def step():
        ffpa.attention(q, k, v, causal=w.causal, mask=mask, scale=w.scale, accum=accum, out=o,
                       lse_out=lse, workspace=ws, dropout_p=w.dropout_p, seed=w.cfg_id)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return per, wall


def _time_calls(call, steps, warmup):
    """Per-call durations (ms, sorted) of `call` with HIP events on the current
    stream, the stream every library call is launched on."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def run_backward(ffpa, W, name, steps, warmup):
    """dQ, dK, dV at the backward workload; O and lse from this library's forward."""
    import torch

    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device="cuda")
    q, k, v, do, mask = inp["q"], inp["k"], inp["v"], inp["dout"], inp["mask"]
    o, lse = ffpa.attention(q, k, v, causal=w.causal, mask=mask, scale=w.scale, return_lse=True,
                            dropout_p=w.dropout_p, seed=w.cfg_id)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dt = ffpa.BF16 if w.dtype == "bf16" else ffpa.F16
    ws_bytes = ffpa.ffpa_attn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.scale,
            int(w.causal), mask.data_ptr() if mask is not None else 0,
            (1 if w.mask == "key" else w.Nq) if mask is not None else 0, ffpa.ACC_F32, dt)
    tail = (ws.data_ptr(), ws_bytes, stream)

    def call():
        if w.dropout_p:
            st = ffpa.ffpa_attn_bwd_dropout(*args, w.dropout_p, w.cfg_id, *tail)
        else:
            st = ffpa.ffpa_attn_bwd(*args, *tail)
        if st != 0:
            raise ffpa.FFPAError(st, ffpa.ffpa_last_error())

    per = _time_calls(call, steps, warmup)
    mean_ms = sum(per) / len(per)
    flops = counted_flops(w.B, w.Hq, w.Nq, w.Nkv, w.D, w.causal, backward=True)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    nbytes = backward_bytes(w)
    if flops / nbytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        # below the ridge point (few query rows per key, e.g. Nq = 1): the
        # bound is HBM, against the bytes every call must move
        gbs = nbytes / (mean_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4)}
    stored = ffpa.ffpa_attn_bwd_workspace_size_stored(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, dt)
    minimum = ffpa.ffpa_attn_bwd_workspace_size_min(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, dt)
    if ws_bytes >= stored:
        kernels = "prep + K^T copy + per chunk of kv heads: dK/dV (stores dS) + dQ from dS"
    elif w.Nq == 1 and ws_bytes > minimum and not w.dropout_p:
        kernels = "decode backward (dK, dV and dQ partials per key range, vector ALUs) + dQ sum"
    else:
        kernels = "prep + dK/dV + dQ (recomputes S and dP)"
    del inp, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"workload": f"{name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nkv={w.Nkv} D={w.D} {w.dtype} "
                        f"causal={w.causal} mask={w.mask}" + (f" dropout_p={w.dropout_p}" if w.dropout_p else ""),
            "value": round(tflops, 2), "unit": "TFLOPS (5 GEMMs counted)",
            "ms_per_call": round(mean_ms, 4),
            "kernels": kernels,
            "workspace_bytes": ws_bytes,
            "roofline": roof,
            "rocprof": recorded_counters(name)}


def backward_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: q, k, v, o, dO and lse read,
    dq, dk, dv written once each."""
    e = 2
    return e * (4 * w.B * w.Hq * w.Nq * w.D + 4 * w.B * w.Hkv * w.Nkv * w.D) + 4 * w.B * w.Hq * w.Nq


def decode_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode call: q, K, V read once, O and lse written."""
    e = 2
    return (w.B * w.Hq * w.D * e * 2 + 2 * w.B * w.Hkv * w.Nkv * w.D * e + w.B * w.Hq * 4)


def run_decode(ffpa, W, steps, warmup):
    import torch

    w = W.WORKLOADS["decode"]
    inp = W.make_inputs(w, device="cuda")
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, 1, dtype=torch.float32, device="cuda")
    dt = ffpa.BF16 if w.dtype == "bf16" else ffpa.F16
    ws_bytes = ffpa.ffpa_attn_fwd_workspace_size(w.B, w.Hq, w.Hkv, 1, w.Nkv, w.D, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        st = ffpa.ffpa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), w.B, w.Hq, w.Hkv, 1, w.Nkv, w.D, w.scale, 0, 0, 0,
                                ffpa.ACC_F32, dt, ws.data_ptr(), ws_bytes, stream)
        if st != 0:
            raise ffpa.FFPAError(st, ffpa.ffpa_last_error())

    per = _time_calls(call, steps, warmup)
    mean_ms = sum(per) / len(per)
    gbs = decode_bytes(w) / (mean_ms * 1e-3) / 1e9
    del inp, o, lse, ws
    torch.cuda.empty_cache()
    return {"workload": f"decode: B={w.B} H={w.Hq} Nq=1 Nkv={w.Nkv} D={w.D} {w.dtype}",
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(mean_ms, 4),
            "kernels": "split-KV + combine",
            "tflops": round(counted_flops(w.B, w.Hq, 1, w.Nkv, w.D) / (mean_ms * 1e-3) / 1e12, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
            "rocprof": recorded_counters("decode")}


def run_fp8(ffpa, W, name, steps, warmup):
    """The fp8 forward (ffpa_attn_fwd_fp8) on a 16-bit workload: per-head amax,
    e4m3 quantisation of Q, K and V^T into the workspace, then the fp8 attention
    kernel; every kernel is inside the timed call. TFLOPS counted like the
    16-bit forward, against the dense fp8 MFMA peak."""
    import torch

    w = W.WORKLOADS[name]
    if w.mask is not None or w.dropout_p:
        raise ValueError(f"the fp8 forward takes no mask and no dropout: {name}")
    inp = W.make_inputs(w, device="cuda")
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.empty_like(q)
    ws = torch.empty(ffpa.ffpa_attn_fwd_fp8_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D),
                     dtype=torch.uint8, device="cuda")

    def call():
        ffpa.attention_fp8(q, k, v, causal=w.causal, scale=w.scale, out=o, workspace=ws)

    per = _time_calls(call, steps, warmup)
    mean_ms = sum(per) / len(per)
    tflops = counted_flops(w.B, w.Hq, w.Nq, w.Nkv, w.D, w.causal) / (mean_ms * 1e-3) / 1e12
    ws_bytes = ws.numel()
    del inp, o, ws
    torch.cuda.empty_cache()
    return {"workload": f"{name} fp8: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nkv={w.Nkv} D={w.D} "
                        f"{w.dtype} in/out, e4m3 QK^T and PV, causal={w.causal}",
            "value": round(tflops, 2), "unit": "TFLOPS" + (" (causal: half counted)" if w.causal else ""),
            "ms_per_call": round(mean_ms, 4),
            "kernels": "f8_zero + f8_amax + f8_quant_qk + f8_quant_vt + fwd_fp8_kernel",
            "workspace_bytes": ws_bytes,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4)},
            "rocprof": recorded_counters("fp8:" + name)}


def timed_call(w, accum="f32", variant=0) -> str:
    """The kernels one timed forward call enqueues (mirrors the library's
    choice for `variant`, 0 = the default)."""
    if w.Nq == 1:
        return "dec_split_kernel + dec_combine_kernel" + (f" (key ranges / {2 ** (variant - 1)})" if variant else "")
    if w.D > 512:
        if variant == 0:
            variant = 1 if (accum != "f16" or w.dropout_p) else (2 if w.D <= 768 else 3)
        if variant == 2 and w.D <= 640:
            return ("fwd_vt_kernel (V transposed into the workspace) + "
                    "fwd_prefill_kernel (fp16 accumulator, a wave holds all of D, 128 rows)")
        return ("fwd_vt_kernel (V transposed, blocks of 32 keys) + " +
                {1: "fwd_wide_kernel (fp32 accumulator, 64 rows)",
                 2: "fwd_wide16_kernel (a wave holds all of D, 128 rows)",
                 3: "fwd_wide16_kernel (a wave pair splits D, 64 rows)"}[variant])
    if variant == 2 or (variant == 0 and w.Nq * w.Hq >= 3072 * w.Hkv):
        return "fwd_vt_kernel (V transposed into the workspace) + fwd_prefill_kernel"
    return "fwd_prefill_kernel (V staged as is)"


def run_one(ffpa, W, name, accum, steps, warmup, with_cpu, cpu_heads):
    import torch

    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device="cuda")
    per, wall = time_forward(ffpa, w, inp, accum, steps, warmup)
    mean_ms = sum(per) / len(per)
    fl = counted_flops(w.B, w.Hq, w.Nq, w.Nkv, w.D, w.causal)
    tflops = fl / (mean_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    line = {
        "metric": "attention fwd TFLOPS at N=8192, D=512 fp16; % of MI355X MFMA fp16 peak",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": f"{name}: self-attention forward" if name == "self" else name,
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nkv": w.Nkv, "D": w.D,
                   "causal": w.causal, "mask": w.mask, "accum": accum, "parallelism": "none"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": measured_traffic(f"{name}:{accum}")},
        "kernel_ms": {"mean": round(mean_ms, 4), "median": round(per[len(per) // 2], 4),
                      "min": round(per[0], 4)},
        "timed_call": timed_call(w, accum),
        "rocprof": recorded_counters(f"{name}:{accum}"),
    }
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(w, inp, cpu_heads)
    del inp
    torch.cuda.empty_cache()
    return line


def run_forward_path(ffpa, W, name, accum, steps, warmup, tune=False):
    """One forward workload timed like the headline (whole call, HIP events).
    tune: ffpa_attn_fwd_tune (level 2, "max") on the workload first, so that
    the timed calls run the variant it picked."""
    import torch

    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, device="cuda")
    tuned = None
    if tune:
        chosen, ms = ffpa.tune_forward(inp["q"], inp["k"], inp["v"], causal=w.causal, mask=inp["mask"],
                                       scale=w.scale, accum=accum, level=2)
        tuned = {"chosen_variant": chosen, "ms_per_variant": {str(k): round(t, 4) for k, t in ms.items()}}
    per, _ = time_forward(ffpa, w, inp, accum, steps, warmup, any_variant=tune)
    if tune:
        ffpa.ffpa_attn_tune_reset()
    mean_ms = sum(per) / len(per)
    tflops = counted_flops(w.B, w.Hq, w.Nq, w.Nkv, w.D, w.causal) / (mean_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    del inp
    torch.cuda.empty_cache()
    return {"workload": f"{name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nkv={w.Nkv} D={w.D} "
                        f"{w.dtype} causal={w.causal} mask={w.mask} accum={accum}"
                        + (f" dropout_p={w.dropout_p}" if w.dropout_p else ""),
            "value": round(tflops, 2), "unit": "TFLOPS" + (" (causal: half counted)" if w.causal else ""),
            "ms_per_call": round(mean_ms, 4),
            "timed_call": timed_call(w, accum, tuned["chosen_variant"] if tuned else 0),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tflops / peak, 4)},
            **({"tuned": tuned} if tuned else {})}


# Forward workloads the default line measures beside the headline: every
# variant in both dtypes, the fp16 accumulator, the head-dimension sweep with
# both accumulators, and 16K sequences.
FWD_PATHS = ([("self_bf16", "f32"), ("self", "f16"), ("self_bf16", "f16")] +
             [(n, "f32") for n in ("cross", "gqa", "causal", "nonaligned", "mask", "dropout")] +
             [(n + "_bf16", "f32") for n in ("cross", "gqa", "causal", "nonaligned", "mask", "dropout")] +
             [(f"dsweep{d}_{a}", a) for d in (320, 448, 512, 576, 768, 1024) for a in ("f32", "f16")] +
             [("self16k", "f32"), ("self16k_bf16", "f32"), ("causal16k", "f32"), ("nonaligned16k", "f32")] +
             [("d128_16k", "f32"), ("d128_32k", "f32")])
# Forward workloads measured again after tuning (the variants differ most there)
TUNED_PATHS = [("cross", "f32"), ("gqa", "f32"), ("dsweep576_f16", "f16"), ("dsweep768_f16", "f16"),
               ("dsweep1024_f16", "f16")]
# 16-bit workloads timed again through the fp8 forward
FP8_PATHS = ("self", "self_bf16", "causal", "dsweep320_f32", "d128_16k", "d128_32k")
BWD_PATHS = ("bwd_causal", "bwd_cross", "bwd_decode", "bwd_gqa", "bwd_mask", "bwd_nonaligned", "bwd_dropout",
             "bwd_d1024", "bwd16k", "bwd16k_causal")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 25 forward calls (~0.1 s at the headline size): the clock ramps up over the first ~10
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default="self")
    ap.add_argument("--accum", default=None, choices=["f32", "f16"],
                    help="output accumulator of the headline call (default: the workload's)")
    # 16 of the 32 heads: about 10 s of the oracle on a 16-core host
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="(b, h) heads the oracle CPU baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true", help="time every workload family")
    ap.add_argument("--no-paths", action="store_true",
                    help="headline forward only (skip the backward and decode measurements)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of 1 GiB (for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import head_dim_attention_flash_amd as ffpa
    import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    ffpa.load()
    if args.suite:
        names = ["tiny", "self", "self_bf16", "cross", "gqa", "causal", "nonaligned", "mask"] + \
                [f"dsweep{d}_f32" for d in (320, 448, 512, 576, 768, 1024)]
        for n in names:
            for acc in ("f32", "f16"):
                line = run_one(ffpa, W, n, acc, args.steps, args.warmup, False, 0)
                print(json.dumps(line), flush=True)
        for n in ("bwd", "bwd_causal", "bwd_d1024", "bwd_d1024_causal"):
            print(json.dumps(run_backward(ffpa, W, n, max(3, args.steps // 2), 2)), flush=True)
        return 0
    if args.workload.startswith("bwd"):
        print(json.dumps(run_backward(ffpa, W, args.workload, args.steps, args.warmup)), flush=True)
        return 0
    if args.workload.startswith("fp8:"):
        print(json.dumps(run_fp8(ffpa, W, args.workload[4:], args.steps, args.warmup)), flush=True)
        return 0
    if args.workload == "decode":
        print(json.dumps(run_decode(ffpa, W, args.steps, args.warmup)), flush=True)
        return 0
    paths = None

    def done(section, name, rec):
        # one progress line per measured path on stderr (stdout carries only
        # the JSON line)
        print(f"bench: {section} {name}: {rec['value']} {rec['unit']}", file=sys.stderr, flush=True)
        return rec

    if not args.no_paths:
        # the backward first: its calls (~0.2 s of GPU work) also bring the
        # clock past its ramp before the headline's warm-up steps
        paths = {"backward": done("backward", "bwd", run_backward(ffpa, W, "bwd", max(3, args.steps // 2), 5))}
    accum = args.accum or W.WORKLOADS[args.workload].accum
    line = run_one(ffpa, W, args.workload, accum, args.steps, args.warmup,
                   not args.no_cpu_baseline, args.cpu_heads)
    done("headline", args.workload, line)
    if paths is not None:
        for name in BWD_PATHS:
            # 5 warm-up calls: the first calls of a backward shape run measurably slower
            paths["backward" + name[3:]] = done("backward", name,
                                                run_backward(ffpa, W, name, max(3, args.steps // 2), 5))
        paths["decode"] = done("decode", "decode", run_decode(ffpa, W, args.steps, max(args.warmup, 50)))
        paths["forward"] = {f"{n}:{a}": done("forward", f"{n}:{a}",
                                             run_forward_path(ffpa, W, n, a, args.steps, args.warmup))
                            for n, a in FWD_PATHS}
        paths["forward_tuned"] = {f"{n}:{a}": done("forward_tuned", f"{n}:{a}",
                                                   run_forward_path(ffpa, W, n, a, args.steps, args.warmup,
                                                                    tune=True))
                                  for n, a in TUNED_PATHS}
        paths["forward_fp8"] = {n: done("forward_fp8", n, run_fp8(ffpa, W, n, args.steps, args.warmup))
                                for n in FP8_PATHS}
        line["paths"] = paths
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_BYTES}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
