#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X (gfx950).

One step is the forward and the backward of exact causal attention on the
bf16 training/prefill workload B=2, H=16, N=4096, d=128 (seeded synthetic
N(0,1) inputs, resident in device memory before timing starts), through
the public calls flash_attn_fwd and flash_attn_bwd; the timed region holds
exactly the K steps and no other event.  Then K more steps run the same
kernels through the phase entry points (forward; dQ, which also computes
the per-row terms; dK/dV) with a HIP event between each two on the
library's stream: they time every kernel separately (each event adds a few
microseconds between kernels, so these steps do not give the step time).
The roofline object describes whichever kernel takes the most time.

The same run also times, each reported under its own key: the same step on
the grouped-query shape (`gqa`), on a packed batch of variable-length
sequences (`varlen`), a chunked prefill over a paged KV cache
(`prefill_paged`), the FP8 (E4M3) forward (`fp8`), the split-KV paged decode
workload (B=8, Hq=32, Hkv=8, 32768 cached tokens per sequence, 16-token
pages) against the HBM roof (`decode`), and the float64 CPU oracle on a
bounded sample of every configuration (its `cpu_baseline` leg; the only
place this file touches the oracle).  The headline step is timed after the
other GPU legs, so that its kernels run at the clock the GPU settles at
under this work.

Prints one JSON line.  `--gpus` above 1 is refused: the library is measured on a
single GPU.

Helper modes produce the measured HBM traffic and counter figures that the
roofline objects report (see `profiles/`):
  python bench.py --profile-once [--profile-repeats R]
      runs every kernel of the step, the decode and the FP8 forward once (or
      R times), plus a 1 GiB device copy whose byte count calibrates the
      counters; run it under `rocprofv3 --pmc FETCH_SIZE` and again under
      `--pmc WRITE_SIZE`;
  python bench.py --traffic-from FETCH.csv WRITE.csv
      turns the two counter CSVs into profiles/traffic.json (bytes per launch,
      scaled by the copy's known bytes, tagged with the kernels' source hash)
      and profiles/hbm_traffic_mha_bf16_4k_decode_fp8.md;
  python bench.py --util-from COUNTERS.csv
      turns a counter CSV of --profile-once (MFMA busy cycles, GRBM active
      cycles, LDS bank conflicts) into profiles/mfma_util.json, from the last
      launch of each kernel.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2516.6  # TFLOP/s: 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_MFMA_FP8 = 5033.2   # TFLOP/s: dense fp8, twice the bf16 rate
PEAK_MFMA_F32 = 157.3    # TFLOP/s: dense fp32 matrix cores
PEAK_HBM = 8000.0        # GB/s: MI355X HBM3E
METRIC = "attention fwd/bwd TFLOP/s (bf16, N=4096, d=128, causal) + % of MFMA peak"


# ---------------------------------------------------------------------------
# Algorithmic work (what the method computes; the N x N work it avoids is not
# counted).  Per visible (query, key) pair and head:
#   forward   4d flops (S = QKᵀ and O = PV, 2 flops per multiply-add)
#   dK/dV     8d flops (S recomputed, dP, dV, dK)
#   dQ        2d flops (dQ; its own recomputation of S and dP is not counted)
# so the backward is 10d = 2.5x the forward.
# ---------------------------------------------------------------------------
def visible_pairs(nq: int, nk: int, causal: bool) -> int:
    if not causal:
        return nq * nk
    diag = nk - nq
    # row i sees keys 0 .. i + diag (clipped to [0, nk])
    total = 0
    lo = max(0, -diag)              # first row that sees any key
    full = max(lo, nk - diag)       # rows from here on see all nk keys
    full = min(full, nq)
    if full > lo:                   # rows lo..full-1 see i + diag + 1 keys
        a, b = lo + diag + 1, full - 1 + diag + 1
        total += (a + b) * (full - lo) // 2
    total += (nq - full) * nk
    return total


def attention_flops(B, Hq, nq, nk, d, causal):
    pairs = B * Hq * visible_pairs(nq, nk, causal)
    return {"fwd": 4 * d * pairs, "dkdv": 8 * d * pairs, "dq": 2 * d * pairs}


def decode_bytes(B, Hq, Hkv, seq_len, d, es, block_size=16):
    kv = 2 * B * Hkv * seq_len * d * es
    pages = -(-seq_len // block_size)
    return kv + 2 * B * Hq * d * es + B * Hq * 4 + B * pages * 4 + B * 4  # + Q, O, LSE, table, lengths


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_47_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "exact_io_aware_47_amd", "csrc", "fa_device.hpp"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"fwd": ("fa_fwd.hip",), "prep": ("fa_bwd.hip",), "dkdv": ("fa_bwd.hip",), "dq": ("fa_bwd.hip",),
                  "decode": ("fa_decode.hip",), "fp8": ("fa_fwd_fp8.hip",)}


def measured_util(kernel: str):
    """Counter-based MFMA busy fraction, shader clock and LDS bank conflicts of
    one launch, from the committed rocprofv3 summary, or None when there is
    none or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "mfma_util.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_hash") != source_hash(*KERNEL_SOURCES[kernel]):
        return None
    out = {k: rec.get(k) for k in ("mfma_busy", "clock_ghz", "lds_bank_conflicts_per_access")}
    if out["clock_ghz"] is not None and out["clock_ghz"] > MAX_SHADER_GHZ:
        out["mfma_busy"] = out["clock_ghz"] = None  # counter window longer than the launch
    return out


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(kernel)
    if not rec or rec.get("source_hash") != source_hash(*KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def mfma_roof():
    """Build bench_mfma_roof.hip for gfx950 into _build/ and run it (2048
    work-groups of 8 waves, 4000 iterations per wave)."""
    import subprocess
    exe = os.path.join(ROOT, "_build", "bench_mfma_roof")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(ROOT, "bench_mfma_roof.hip"), "-o", exe], check=True)
    return subprocess.run([exe, "2048", "4000"]).returncode


def ensure_library():
    from exact_io_aware_47_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from exact_io_aware_47_amd import build
        build.build()


def prepare_inputs(torch, si):
    """Every leg's seeded inputs, generated on the host and copied to the GPU
    before the first leg runs, so that the legs follow each other with no
    idle gap on the GPU (an MI355X resuming heavy work after a pause runs
    the first tens of calls ~10-20% slower while its power management
    settles)."""
    dev = lambda ts: tuple(t.to("cuda") for t in ts)
    inputs = {}
    for name in ("mha_f32_small", "mha_f16", "mha_bf16_16k", "gqa_bf16_4k", "mha_bf16_4k"):
        inputs[name] = dev(si.workload_attention_inputs(si.WORKLOADS[name]))
    inputs["varlen_bf16"] = dev(si.workload_packed_inputs(si.WORKLOADS["varlen_bf16"]))
    inputs["prefill_paged_bf16"] = dev(si.workload_prefill_inputs(si.WORKLOADS["prefill_paged_bf16"]))
    wf = si.WORKLOADS["mha_fp8_4k"]
    q, k, v, desc = si.make_fp8_inputs(wf.B, wf.Hq, wf.Hkv, wf.Nq, wf.Nk, wf.d, wf.seed)
    inputs["mha_fp8_4k"] = dev((q, k, v)) + (desc,)
    inputs["decode_gqa_paged"] = dev(si.workload_decode_inputs(si.WORKLOADS["decode_gqa_paged"]))
    torch.cuda.synchronize()
    return inputs


def bench_training(torch, fa, si, steps, warmup, inputs, name="mha_bf16_4k", causal=True):
    w = si.WORKLOADS[name]
    q, k, v, do = inputs[name]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[w.dtype]
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, code), dtype=torch.uint8,
                     device="cuda")

    # One step through the public calls: flash_attn_fwd, then flash_attn_bwd
    # (dQ computing the row terms D_i and LSE_i*log2(e) into the workspace,
    # then dK/dV reading them).
    def step():
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    # The same kernels through the phase entry points, with an event between
    # each two so that every kernel is timed on its own.  Each event costs the
    # stream a few microseconds between kernels, so these steps give the
    # per-kernel times, not the step time.
    def step_split(ev):
        ev[0].record()
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
        ev[1].record()
        fa.bwd_phase("dq_rowterms", q, k, v, o, do, lse, dq, None, None, ws, causal)
        ev[2].record()
        fa.bwd_phase("dkdv", q, k, v, None, do, None, None, dk, dv, ws, causal)
        ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step_split(evs[i])
    torch.cuda.synchronize()
    names = ["fwd", "dq", "dkdv"]
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names)}
    return w, total_ms / steps, per, wall


def bench_varlen(torch, fa, si, steps, warmup, inputs):
    """Forward + backward of the packed variable-length workload; the backward
    runs as one flash_attn_bwd_varlen call.  The step time comes from steps
    with no event inside them, the forward and backward times from as many
    more steps with an event between the two calls.  Returns (workload,
    lengths, ms per step, {fwd, bwd: ms})."""
    w = si.WORKLOADS["varlen_bf16"]
    q, k, v, do, cu_q, cu_k = inputs["varlen_bf16"]
    lens = (cu_q[1:] - cu_q[:-1]).tolist()
    mx = max(lens)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    tq = q.shape[0] // w.Hq
    ws = torch.empty(fa.bwd_varlen_workspace_bytes(w.B, w.Hq, w.Hkv, tq, tq, mx, mx, w.d, fa.FA_BF16),
                     dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev: ev[0].record()
        fa.fwd_varlen(q, k, v, cu_q, cu_k, w.Hq, w.Hkv, mx, mx, causal=w.causal, out=o, lse=lse)
        if ev: ev[1].record()
        fa.bwd_varlen(q, k, v, o, do, lse, cu_q, cu_k, w.Hq, w.Hkv, mx, mx, causal=w.causal, dq=dq, dk=dk, dv=dv,
                      workspace=ws)
        if ev: ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(("fwd", "bwd"))}
    return w, lens, t0.elapsed_time(t1) / steps, per


def bench_prefill(torch, fa, si, steps, warmup, inputs):
    """Chunked prefill over the paged cache: one flash_attn_prefill_paged call per step."""
    w = si.WORKLOADS["prefill_paged_bf16"]
    q, kc, vc, table, lens = inputs["prefill_paged_bf16"]
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        fa.prefill_paged(q, kc, vc, table, lens, causal=w.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fa.prefill_paged(q, kc, vc, table, lens, causal=w.causal, out=out, lse=lse)
    t1.record()
    torch.cuda.synchronize()
    return w, t0.elapsed_time(t1) / steps


def bench_fp8(torch, fa, si, steps, warmup, inputs):
    """FP8 forward on the training shape: one flash_attn_fwd_fp8 call per step
    (its V-staging pre-pass included)."""
    w = si.WORKLOADS["mha_fp8_4k"]
    q, k, v, desc = inputs["mha_fp8_4k"]
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fwd_fp8_workspace_bytes(w.B, w.Hkv, w.Nk, w.d), dtype=torch.uint8, device="cuda")
    call = lambda: fa.fwd_fp8(q, k, v, *desc, causal=True, out=out, lse=lse, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    return w, t0.elapsed_time(t1) / steps


def bench_decode(torch, fa, si, steps, warmup, inputs):
    w = si.WORKLOADS["decode_gqa_paged"]
    q, kc, vc, table, lens = inputs["decode_gqa_paged"]
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.max_blocks), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        fa.decode_paged(q, kc, vc, table, lens, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fa.decode_paged(q, kc, vc, table, lens, out=out, lse=lse, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return w, ms


def _blas_info():
    """(BLAS threads, BLAS vendor) of numpy, via threadpoolctl when present."""
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return int(p.get("num_threads") or 0), f"{p.get('internal_api')} {p.get('version') or ''}".strip()
    except Exception:
        pass
    return 0, "unknown"


def _visible_rows_pairs(rows, nq, nk, causal):
    """Visible (query, key) pairs of the given query rows."""
    if not causal:
        return len(rows) * nk
    return int(sum(max(0, min(nk, r + 1 + nk - nq)) for r in rows))


def cpu_baseline(si):
    """The float64 oracle, as it stands, timed on the host on bounded samples
    of every configuration: forward and backward wall-clock separately (one
    run for the two bf16 training shapes, the median of 3 for the others),
    with the rate on the same algorithmic flop count as the GPU (visible pairs
    only; the oracle itself evaluates every pair).  The line's value is the
    mha_bf16_4k sample's forward + backward rate."""
    import numpy as np
    from oracle import attention_f64 as orc
    threads, vendor = _blas_info()
    if not threads:
        threads = len(os.sched_getaffinity(0))
    per = {}

    def timed(fn, repeats):
        ts = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def attention_leg(key, name, causal, heads, rows, repeats):
        w = si.WORKLOADS[name]
        q, k, v, do = (t.double().numpy() for t in si.workload_attention_inputs(w))
        g = w.Hq // w.Hkv
        sel_rows = np.arange(w.Nq) if rows is None else rows
        fwd_s = bwd_s = 0.0
        for b, h in heads:
            qs, ks, vs, dos = (q[b:b + 1, h:h + 1], k[b:b + 1, h // g:h // g + 1], v[b:b + 1, h // g:h // g + 1],
                               do[b:b + 1, h:h + 1])
            kw = {} if rows is None else {"row_ids": rows, "nq_total": w.Nq}
            if rows is not None:
                qs, dos = qs[:, :, rows], dos[:, :, rows]
            fwd_s += timed(lambda: orc.attention_fwd(qs, ks, vs, w.scale, causal, **kw), repeats)
            bwd_s += timed(lambda: orc.attention_bwd(qs, ks, vs, dos, w.scale, causal, **kw), repeats)
        pairs = len(heads) * _visible_rows_pairs(sel_rows, w.Nq, w.Nk, causal)
        fwd_fl, bwd_fl = 4 * w.d * pairs, 10 * w.d * pairs
        frac = len(heads) * len(sel_rows) / (w.B * w.Hq * w.Nq)
        per[key] = {"sample": f"{len(heads)} of {w.B * w.Hq} heads" +
                              ("" if rows is None else f", query rows {int(rows[0])}..{int(rows[-1])} of {w.Nq}"),
                    "repeats": repeats, "fwd_s": round(fwd_s, 4), "bwd_s": round(bwd_s, 4),
                    "fwd_gflops": round(fwd_fl / fwd_s / 1e9, 3), "bwd_gflops": round(bwd_fl / bwd_s / 1e9, 3),
                    "whole_config_fwd_s_est": round(fwd_s / frac, 4), "whole_config_bwd_s_est": round(bwd_s / frac, 4)}
        return fwd_fl + bwd_fl, fwd_s + bwd_s

    t_all = time.perf_counter()
    attention_leg("mha_f32_small", "mha_f32_small", False, [(0, 0)], None, 3)
    heads8 = [(b, h) for b in range(4) for h in (0, 7)]
    attention_leg("mha_f16_causal", "mha_f16", True, heads8, None, 3)
    attention_leg("mha_f16_noncausal", "mha_f16", False, heads8, None, 3)
    fl3, s3 = attention_leg("mha_bf16_4k", "mha_bf16_4k", True, [(0, 0), (0, 9), (1, 4), (1, 15)], None, 1)
    w4 = si.WORKLOADS["mha_bf16_16k"]
    attention_leg("mha_bf16_16k", "mha_bf16_16k", True, [(0, 15)], np.arange(w4.Nq - 1024, w4.Nq), 1)
    # Decode: two of the eight sequences, gathered through the block table.
    wd = si.WORKLOADS["decode_gqa_paged"]
    q, kc, vc, table, lens = si.workload_decode_inputs(wd)
    q, kc, vc = q.double().numpy(), kc.float().numpy(), vc.float().numpy()
    seqs = [0, wd.B - 1]
    dec_s = timed(lambda: orc.decode_paged(q[seqs], kc, vc, table.numpy()[seqs], lens.numpy()[seqs], wd.scale), 3)
    dbytes = decode_bytes(len(seqs), wd.Hq, wd.Hkv, wd.seq_len, wd.d, 2)
    per["decode_gqa_paged"] = {"sample": f"{len(seqs)} of {wd.B} sequences", "repeats": 3, "fwd_s": round(dec_s, 4),
                               "GB/s": round(dbytes / dec_s / 1e9, 3),
                               "whole_config_fwd_s_est": round(dec_s * wd.B / len(seqs), 2)}
    del kc, vc
    total = time.perf_counter() - t_all
    return {"value": round(fl3 / s3 / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "mha_bf16_4k: 4 of 32 (batch, head) slices, causal forward + backward in float64 numpy "
                      f"({s3:.1f} s), flops counted as for the GPU (visible pairs only); per_config holds every "
                      f"configuration's forward and backward seconds ({total:.1f} s of oracle work in all)",
            "os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "blas": vendor,
            "blas_threads": int(threads), "per_config": per}


def profile_once(torch, fa, si, repeats=1):
    """``repeats`` launches of every kernel of the training step (forward, dQ
    with the row terms, dK/dV; also the separate row-term kernel of the
    preprocess phase), of the decode and of the FP8 forward, then a 1 GiB
    device-to-device copy (counter calibration).  Counter readers take the last launch of each kernel (util)
    or the mean over launches (bytes, which do not change between launches)."""
    w = si.WORKLOADS["mha_bf16_4k"]
    q, k, v, do = (t.to("cuda") for t in si.workload_attention_inputs(w))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, fa.FA_BF16), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for _ in range(repeats):
        o, lse = fa.fwd(q, k, v, causal=True)
        fa.bwd_phase("preprocess", None, None, None, o, do, lse, None, None, None, ws, True)
        fa.bwd_phase("dq_rowterms", q, k, v, o, do, lse, dq, None, None, ws, True)
        fa.bwd_phase("dkdv", q, k, v, None, do, None, None, dk, dv, ws, True)
    torch.cuda.synchronize()
    del q, k, v, do, o, lse, ws, dq, dk, dv
    wd = si.WORKLOADS["decode_gqa_paged"]
    args = [t.to("cuda") for t in si.workload_decode_inputs(wd)]
    for _ in range(repeats):
        fa.decode_paged(*args)
    torch.cuda.synchronize()
    del args
    wf = si.WORKLOADS["mha_fp8_4k"]
    q, k, v, desc = si.make_fp8_inputs(wf.B, wf.Hq, wf.Hkv, wf.Nq, wf.Nk, wf.d, wf.seed)
    q, k, v = q.to("cuda"), k.to("cuda"), v.to("cuda")
    for _ in range(repeats):
        fa.fwd_fp8(q, k, v, *desc, causal=True)
    torch.cuda.synchronize()
    del q, k, v
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print("profile-once done", flush=True)


COPY_BYTES = 1 << 30
# rocprofv3 kernel names -> the keys used above (the decode is split + reduce).
KERNEL_KEYS = (("fwd_kernel", "fwd"), ("bwd_prep_kernel", "prep"), ("bwd_dkdv_kernel", "dkdv"), ("bwd_dkdv16_kernel", "dkdv"),
               ("bwd_dq_kernel", "dq"), ("decode_split_kernel", "decode"), ("decode_reduce_kernel", "decode"),
               ("fp8_vt_kernel", "fp8"), ("fwd_fp8_kernel", "fp8"))


# The benchmark's legs in the order main() runs them, with the kernel
# dispatches of one step of each (warm-up and timed steps alike).
# The training legs (fwd + bwd) run their timed steps twice: once through the
# public calls for the step time, then through the phase entry points with
# events between the kernels for the per-kernel times.
LEG_ORDER = (("mha_f32_small (non-causal)", 3), ("mha_f16 (causal)", 3), ("mha_f16 (non-causal)", 3),
             ("mha_bf16_16k", 3), ("varlen_bf16", 3), ("prefill_paged_bf16", 1), ("mha_fp8_4k", 2),
             ("decode_gqa_paged", 2), ("gqa_bf16_4k", 3), ("mha_bf16_4k", 3))
TWO_PASS_LEGS = ("mha_f32_small (non-causal)", "mha_f16 (causal)", "mha_f16 (non-causal)", "mha_bf16_16k",
                 "varlen_bf16", "gqa_bf16_4k", "mha_bf16_4k")
ATTENTION_KERNEL = ("fwd_kernel", "fwd_keysplit_kernel", "fwd_keysplit_plain_kernel", "fwd_fp8_kernel",
                    "fp8_vt_kernel", "bwd_prep_kernel",
                    "bwd_dkdv16_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "decode_split_kernel",
                    "decode_reduce_kernel")


def _short_kernel_name(n):
    """Kernel name with its template arguments, from a mangled or demangled name."""
    import re
    m = re.search(r"N_1\d+(\w+?_kernel)I(.*?)EEv", n)
    if m:
        args = []
        for tok in re.findall(r"DF16b|DF16_|Lb[01]E|Li\d+E|^f|(?<=E)f", m.group(2)):
            args.append({"DF16b": "bf16", "DF16_": "f16", "f": "float", "Lb1E": "1", "Lb0E": "0"}.get(
                tok, tok[2:-1] if tok.startswith("Li") else tok))
        return f"{m.group(1)}<{', '.join(args)}>"
    m = re.search(r"::(\w+_kernel)<([^>]*)>", n)
    return f"{m.group(1)}<{m.group(2).replace('true', '1').replace('false', '0')}>" if m else n[:60]


def trace_summary(trace_csv, steps, warmup):
    """Markdown table of a rocprofv3 kernel trace of one default benchmark
    run: every attention dispatch labelled with its leg (legs run in
    LEG_ORDER, each with warmup + steps steps, the training legs with
    another `steps` steps for their per-kernel times), per (leg, kernel) the
    call count, the average over all calls and over the last `steps` calls
    (the ones the per-kernel events cover), min, max and total."""
    import collections
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    legs = [(n, k * (warmup + steps * (2 if n in TWO_PASS_LEGS else 1))) for n, k in LEG_ORDER]
    leg_i, used = 0, 0
    g = collections.defaultdict(list)
    for r in rows:
        n = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        if not any(k in n for k in ATTENTION_KERNEL):
            g[("(torch / runtime)", _short_kernel_name(n))].append(dur)
            continue
        while leg_i < len(legs) and used >= legs[leg_i][1]:
            leg_i, used = leg_i + 1, 0
        leg = legs[leg_i][0] if leg_i < len(legs) else "?"
        used += 1
        g[(leg, _short_kernel_name(n))].append(dur)
    tot = sum(sum(v) for v in g.values())
    out = [f"| workload | kernel (template arguments) | calls | avg us | avg us, last {steps} (timed) calls | "
           "min us | max us | total us | % |", "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (leg, k), v in sorted(g.items(), key=lambda kv: -sum(kv[1])):
        t = v[-steps:]
        out.append(f"| {leg} | `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {sum(t) / len(t):.2f} | {min(v):.2f} | "
                   f"{max(v):.2f} | {sum(v):.1f} | {100 * sum(v) / tot:.1f} |")
    text = "\n".join(out)
    print(text)
    return text


def _counter_sums(path, counter):
    """{dispatch id: (kernel name, counter value in KiB)} from a rocprofv3 CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, val = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, val + float(r["Counter_Value"]))
    return out


SIMDS, XCDS = 1024, 8  # MI355X: 256 compute units x 4 SIMDs, 8 XCDs
MAX_SHADER_GHZ = 2.4   # MI355X peak engine clock


def util_from(csv_path, out_dir=None):
    """profiles/mfma_util.json from one rocprofv3 counter CSV of --profile-once:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x SIMDs)
    (rocprofv3's MfmaUtil), clock = GRBM_GUI_ACTIVE per XCD / duration, LDS bank
    conflicts per access = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - conflicts)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {},
                                                       "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rec = {"_definition": util_from.__doc__.split("\n", 1)[1].strip()}
    for _, d in sorted(per.items()):
        # One launch per key: the last dispatch of its main kernel (the decode's
        # split kernel, the FP8 forward rather than its V staging), the earlier
        # ones being the warm-up.
        if "decode_reduce" in d["name"] or "fp8_vt" in d["name"]:
            continue
        key = next((k for pat, k in KERNEL_KEYS if pat in d["name"]), None)
        if key is None:
            continue
        c = d["c"]
        grbm = c["GRBM_GUI_ACTIVE"] / XCDS
        clock = grbm / (d["us"] * 1e3)
        # GRBM cycles beyond what the launch's duration allows at the top shader
        # clock mean that the counter window outlasted a short launch: the busy
        # fraction and the clock derived from them would be wrong, so neither is
        # reported.
        valid = clock <= MAX_SHADER_GHZ
        rec[key] = {"mfma_busy": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (grbm * SIMDS), 4) if valid else None,
                    "clock_ghz": round(clock, 3) if valid else None,
                    "lds_bank_conflicts_per_access": round(
                        c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"]), 4),
                    "us": round(d["us"], 2), "source_hash": source_hash(*KERNEL_SOURCES[key])}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "mfma_util.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return rec


# Labels of the counter tables, and the algorithmic flops each kernel's work
# amounts to on its workload (mha_bf16_4k for the training kernels and the FP8
# forward's shape; the decode is HBM-bound).
COUNTER_ROWS = (("fwd", "fwd (`fwd_kernel<bf16,128,causal>`)", "1.375e11"), ("prep", "prep", "—"),
                ("dkdv", "dkdv (`bwd_dkdv16_kernel`)", "2.750e11"),
                ("dq", "dq (`bwd_dq_kernel`, computing the row terms)", "0.687e11 (2d; S and dP recomputed)"),
                ("decode", "decode (`decode_split_kernel`)", "— (HBM-bound)"),
                ("fp8", "fp8 (`fwd_fp8_kernel`)", "1.375e11"))


def _last_launch_counters(csv_path):
    """{key: (counters, us)} of the last dispatch of each kernel key (decode:
    its split kernel; FP8: its forward kernel, not the V staging)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": {},
                                                       "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    last = {}
    for _, d in sorted(per.items()):
        if "decode_reduce" in d["name"] or "fp8_vt" in d["name"]:
            continue
        key = next((k for pat, k in KERNEL_KEYS if pat in d["name"]), None)
        if key is not None:
            last[key] = (d["c"], d["us"])
    return last


def util_table(csv_path):
    """Markdown rows of the MFMA-busy / clock / LDS counter table (last launch of each kernel)."""
    last = _last_launch_counters(csv_path)
    rows = ["| kernel | µs | MFMA busy | clock GHz | LDS bank conflicts / access | LDS wait / LDS active | "
            "executed flops | algorithmic flops |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for key, label, alg in COUNTER_ROWS:
        if key not in last:
            continue
        c, us = last[key]
        grbm = c["GRBM_GUI_ACTIVE"] / XCDS
        clock = grbm / (us * 1e3)
        valid = clock <= MAX_SHADER_GHZ
        busy = f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (grbm * SIMDS):.1f}%" if valid else "—"
        bc = c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"])
        wa = c["SQ_WAIT_INST_LDS"] / max(1.0, c["SQ_ACTIVE_INST_LDS"])
        fl = c["SQ_INSTS_VALU_MFMA_MOPS_F8" if key == "fp8" else "SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        fls = (f"{fl:.3e}" + (" (F8)" if key == "fp8" else "")) if fl else "0"
        rows.append(f"| {label} | {us:.1f} | {busy} | {f'{clock:.2f}' if valid else '—'} | {bc:.3f} | {wa:.2f} | "
                    f"{fls} | {alg} |")
    return "\n".join(rows)


def issue_table(csv_path):
    """Markdown rows of where the waves' time goes (SQ counters over SQ_WAVE_CYCLES, last launch)."""
    last = _last_launch_counters(csv_path)
    rows = ["| kernel | µs | issuing | waiting on a dependency | waiting for an issue slot | VALU | LDS | VMEM |",
            "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for key, label, _ in COUNTER_ROWS:
        if key not in last:
            continue
        c, us = last[key]
        w = max(1.0, c["SQ_WAVE_CYCLES"])
        f = lambda n: f"{100 * c[n] / w:.0f}%"
        rows.append(f"| {label} | {us:.1f} | {f('SQ_ACTIVE_INST_ANY')} | {f('SQ_WAIT_ANY')} | {f('SQ_WAIT_INST_ANY')} | "
                    f"{f('SQ_ACTIVE_INST_VALU')} | {f('SQ_ACTIVE_INST_LDS')} | {100 * c['SQ_ACTIVE_INST_VMEM'] / w:.1f}% |")
    return "\n".join(rows)


def traffic_from(fetch_csv, write_csv, out_dir=None):
    fetch, write = _counter_sums(fetch_csv, "FETCH_SIZE"), _counter_sums(write_csv, "WRITE_SIZE")
    def per_key(rows):
        acc, copy = {}, []
        for name, kib in rows.values():
            if "copy" in name.lower() or "elementwise" in name.lower():
                copy.append(kib)
                continue
            for pat, key in KERNEL_KEYS:
                if pat in name:
                    acc.setdefault(key, {}).setdefault(pat, []).append(kib)
        # bytes per launch: mean over dispatches of each kernel, summed over the key's kernels
        return {k: sum(sum(v) / len(v) for v in pats.values()) * 1024 for k, pats in acc.items()}, copy
    fb, fcopy = per_key(fetch)
    wb, wcopy = per_key(write)
    if not fcopy or not wcopy:
        raise SystemExit("no calibration copy kernel found in the counter files")
    f_factor = COPY_BYTES / (max(fcopy) * 1024)
    w_factor = COPY_BYTES / (max(wcopy) * 1024)
    rec = {"_calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": round(f_factor, 4),
                            "write_factor": round(w_factor, 4),
                            "note": "counter KiB x 1024 x factor = bytes; factor = copy bytes / copy counter bytes"}}
    for key in sorted(set(fb) | set(wb)):
        fbytes, wbytes = fb.get(key, 0.0) * f_factor, wb.get(key, 0.0) * w_factor
        rec[key] = {"fetch_bytes": round(fbytes), "write_bytes": round(wbytes),
                    "hbm_bytes_per_launch": round(fbytes + wbytes),
                    "source_hash": source_hash(*KERNEL_SOURCES[key])}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    # Text summary next to it.
    w = None
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Workloads: mha_bf16_4k (B=2, H=16, N=4096, d=128, causal, bf16) for fwd / prep / dkdv / dq;",
             "decode_gqa_paged (B=8, Hq=32, Hkv=8, Nk=32768, d=128, bf16, 16-token pages) for decode;",
             "mha_fp8_4k (B=2, H=16, N=4096, d=128, causal, E4M3 in, bf16 out) for fp8 (V staging + forward).", "",
             "Commands (from the repository root, on the GPU; $OUT is any output directory):", "",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o p -- python3 bench.py --profile-once",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o p -- python3 bench.py --profile-once",
             "    python3 bench.py --traffic-from $OUT/pmc_fetch/p_counter_collection.csv $OUT/pmc_write/p_counter_collection.csv",
             "",
             f"Calibration: a {COPY_BYTES >> 20} MiB device copy reads and writes {COPY_BYTES} bytes; the counters report "
             f"{max(fcopy):.0f} KiB fetched and {max(wcopy):.0f} KiB written, so fetch counts scale by {f_factor:.4f} "
             f"and write counts by {w_factor:.4f}.", "",
             "| kernel | fetch bytes | write bytes | total per launch |", "|---|---:|---:|---:|"]
    for key in ("fwd", "prep", "dkdv", "dq", "decode", "fp8"):
        if key in rec:
            r = rec[key]
            lines.append(f"| {key} | {r['fetch_bytes']:,} | {r['write_bytes']:,} | {r['hbm_bytes_per_launch']:,} |")
    with open(os.path.join(out_dir, "hbm_traffic_mha_bf16_4k_decode_fp8.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # A burst of attention kernels on an idle MI355X runs about 7% slower for
    # its first ~50 ms (5 warm-up steps: 642 TFLOP/s; 200: 686), so the
    # default warm-up covers that before the timed steps.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--profile-once", action="store_true", help="launch every kernel once (for rocprofv3 counters)")
    ap.add_argument("--profile-repeats", type=int, default=1, metavar="R",
                    help="with --profile-once: launch every kernel R times (the first ones warm the GPU up)")
    ap.add_argument("--util-from", metavar="COUNTER_CSV",
                    help="write profiles/mfma_util.json from a rocprofv3 counter CSV of --profile-once")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 counter CSVs")
    ap.add_argument("--mfma-roof", action="store_true",
                    help="build and run bench_mfma_roof.hip: the bf16 MFMA rate sustained with constant and random operands")
    ap.add_argument("--util-table", metavar="COUNTER_CSV", help="print the MFMA-busy / LDS counter table")
    ap.add_argument("--issue-table", metavar="COUNTER_CSV", help="print the issue-breakdown counter table")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print the per-leg table of a rocprofv3 kernel trace of a run with these --steps/--warmup")
    args = ap.parse_args(argv)
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps, args.warmup)
        return 0
    if args.util_table:
        print(util_table(args.util_table))
        return 0
    if args.issue_table:
        print(issue_table(args.issue_table))
        return 0
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return 0
    if args.util_from:
        util_from(args.util_from)
        return 0
    if args.mfma_roof:
        return mfma_roof()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention kernels here are "
              "built and timed on a single MI355X and no multi-GPU path exists.", file=sys.stderr)
        return 2

    import torch
    import synth_inputs as si
    ensure_library()
    import exact_io_aware_47_amd as fa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    props = torch.cuda.get_device_properties(0)
    if args.profile_once:
        profile_once(torch, fa, si, max(1, args.profile_repeats))
        return 0

    inputs = prepare_inputs(torch, si)
    # The legs run in LEG_ORDER: the headline step is timed last, right after
    # the grouped-query step, which runs the same kernels, so that it meets a
    # GPU whose clock has settled under this work (an idle MI355X runs these
    # kernels ~10% slower over its first tens of milliseconds of such a burst).
    extra = {}
    # The other attention configurations, same step, each against its dtype's matrix peak.
    extra["configs"] = {}
    for cname, causal in (("mha_f32_small", False), ("mha_f16", True), ("mha_f16", False), ("mha_bf16_16k", True)):
        wc, ms_c, per_c, _ = bench_training(torch, fa, si, args.steps, args.warmup, inputs, cname, causal)
        flc = attention_flops(wc.B, wc.Hq, wc.Nq, wc.Nk, wc.d, causal)
        peak = PEAK_MFMA_F32 if wc.dtype == "f32" else PEAK_MFMA_BF16
        fwd_tf = flc["fwd"] / (per_c["fwd"] * 1e-3) / 1e12
        bwd_tf = (flc["dkdv"] + flc["dq"]) / ((per_c["dkdv"] + per_c["dq"]) * 1e-3) / 1e12
        extra["configs"][f"{cname}_{'causal' if causal else 'noncausal'}"] = {
            "shape": f"B={wc.B} H={wc.Hq} N={wc.Nq} d={wc.d} {wc.dtype}" + (f" Q,K x{wc.qk_mult:g}" if wc.qk_mult != 1 else ""),
            "fwd_us": round(per_c["fwd"] * 1e3, 2), "bwd_us": round((per_c["dkdv"] + per_c["dq"]) * 1e3, 2),
            "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2), "peak": peak,
            "fwd_frac": round(fwd_tf / peak, 4), "bwd_frac": round(bwd_tf / peak, 4)}
    # Packed variable-length batch (16 causal sequences of seeded lengths), same step.
    wv, lens_v, ms_v, per_v = bench_varlen(torch, fa, si, args.steps, args.warmup, inputs)
    flv = {"fwd": 0, "dkdv": 0, "dq": 0}
    for n in lens_v:
        for key, val in attention_flops(1, wv.Hq, n, n, wv.d, wv.causal).items():
            flv[key] += val
    extra["varlen"] = {"workload": f"varlen_bf16: packed batch of {wv.B} causal sequences, Hq=Hkv={wv.Hq}, d={wv.d} "
                                  f"bf16, {sum(lens_v)} tokens, lengths uniform in [1, {wv.max_len}]",
                      "lengths": lens_v, "seed": wv.seed,
                      "TFLOP/s": round((flv["fwd"] + flv["dkdv"] + flv["dq"]) / (ms_v * 1e-3) / 1e12, 2),
                      "fwd_tflops": round(flv["fwd"] / (per_v["fwd"] * 1e-3) / 1e12, 2),
                      "bwd_tflops": round((flv["dkdv"] + flv["dq"]) / (per_v["bwd"] * 1e-3) / 1e12, 2),
                      "ms_per_step": round(ms_v, 4), "us": {n: round(v * 1e3, 2) for n, v in per_v.items()}}
    # Chunked prefill over the paged cache (queries are each sequence's last Nq positions).
    wp, ms_p = bench_prefill(torch, fa, si, args.steps, args.warmup, inputs)
    flp = attention_flops(wp.B, wp.Hq, wp.Nq, wp.seq_len, wp.d, wp.causal)["fwd"]
    extra["prefill_paged"] = {"workload": f"prefill_paged_bf16: B={wp.B} Hq={wp.Hq} Hkv={wp.Hkv}, a chunk of {wp.Nq} "
                                         f"queries over {wp.seq_len} cached tokens, d={wp.d} bf16 causal, "
                                         "16-token pages via a permuted table",
                             "us": round(ms_p * 1e3, 2), "TFLOP/s": round(flp / (ms_p * 1e-3) / 1e12, 2),
                             "flops": flp, "seed": wp.seed}
    # FP8 (E4M3) forward on the same shape.
    wf, ms_f = bench_fp8(torch, fa, si, args.steps, args.warmup, inputs)
    flf = attention_flops(wf.B, wf.Hq, wf.Nq, wf.Nk, wf.d, True)["fwd"]
    tf = flf / (ms_f * 1e-3) / 1e12
    extra["fp8"] = {"workload": "mha_fp8_4k: causal forward, B=2 H=16 N=4096 d=128, E4M3 Q/K/V with per-tensor "
                               "descales, bf16 O", "us": round(ms_f * 1e3, 2), "TFLOP/s": round(tf, 2),
                   "roofline": {"kernel": "fwd_fp8 (V staging + forward)", "bound": "mfma", "achieved": round(tf, 2),
                                "peak": PEAK_MFMA_FP8, "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_FP8, 4),
                                "traffic": measured_traffic("fp8"), "counters": measured_util("fp8")}}
    if not args.no_decode:
        wd, ms_dec = bench_decode(torch, fa, si, args.steps, args.warmup, inputs)
        nbytes = decode_bytes(wd.B, wd.Hq, wd.Hkv, wd.seq_len, wd.d, 2)
        gbs = nbytes / (ms_dec * 1e-3) / 1e9
        extra["decode"] = {"workload": "decode_gqa_paged: B=8 Hq=32 Hkv=8 Nk=32768 d=128 bf16, 16-token pages",
                          "us": round(ms_dec * 1e3, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
                          "roofline": {"kernel": "decode (split + reduce)", "bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM, "unit": "GB/s", "frac": round(gbs / PEAK_HBM, 4),
                                       "traffic": measured_traffic("decode")}}
    # The grouped-query training shape (four query heads per K/V head), same step.
    wg, ms_g, per_g, _ = bench_training(torch, fa, si, args.steps, args.warmup, inputs, "gqa_bf16_4k")
    flg = attention_flops(wg.B, wg.Hq, wg.Nq, wg.Nk, wg.d, True)
    extra["gqa"] = {"workload": "gqa_bf16_4k: causal forward + backward, B=2 Hq=32 Hkv=8 N=4096 d=128 bf16",
                   "TFLOP/s": round((flg["fwd"] + flg["dkdv"] + flg["dq"]) / (ms_g * 1e-3) / 1e12, 2),
                   "ms_per_step": round(ms_g, 4), "us": {n: round(v * 1e3, 2) for n, v in per_g.items()}}
    w, ms_step, per, wall = bench_training(torch, fa, si, args.steps, args.warmup, inputs)
    fl = attention_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, True)
    step_flops = fl["fwd"] + fl["dkdv"] + fl["dq"]
    value = step_flops / (ms_step * 1e-3) / 1e12

    work = {"fwd": ("mfma", fl["fwd"]), "dkdv": ("mfma", fl["dkdv"]), "dq": ("mfma", fl["dq"])}

    def roofline(name, ms):
        bound, amount = work[name]
        if bound == "mfma":
            ach, peak, unit = amount / (ms * 1e-3) / 1e12, PEAK_MFMA_BF16, "TFLOP/s"
        else:
            ach, peak, unit = amount / (ms * 1e-3) / 1e9, PEAK_HBM, "GB/s"
        return {"kernel": name, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": measured_traffic(name), "avg_us": round(ms * 1e3, 2),
                "counters": measured_util(name)}

    dominant = max(per, key=per.get)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mha_bf16_4k: causal attention forward + backward, bf16 in, fp32 accumulation",
                   "B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d, "causal": True, "seed": w.seed,
                   "flops_per_step": step_flops},
        "pct_mfma_peak": round(100 * value / PEAK_MFMA_BF16, 2),
        "roofline": roofline(dominant, per[dominant]),
        "kernels": {n: roofline(n, per[n]) for n in per},
        "fwd_tflops": round(fl["fwd"] / (per["fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round((fl["dkdv"] + fl["dq"]) / ((per["dkdv"] + per["dq"]) * 1e-3) / 1e12, 2),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "host_wall_s_timed": round(wall, 4),
    }
    line.update(extra)
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(si)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
