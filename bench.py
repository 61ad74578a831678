"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass of the whole path over synthetic inputs already resident
in HBM:
  * prefill: causal bf16 attention, B=1, H=32, N=16384, d=128 (fa_fwd);
  * decode: paged GQA decode, 64 sequences with KV lengths U[512, 32768]
    (seed 4), page size 16, 32 query / 8 KV heads, d=128 (fa_decode_paged).
``value`` is the prefill throughput in TFLOP/s (4*B*H*N^2*d/2 per call);
the decode line reports KV bytes read per second. Each call is timed with
HIP events on the stream it is launched on; ``ms_per_step`` is the wall
time of the timed steps divided by their number.

After the timed steps, the outputs of the last timed calls are checked
against the fp64 oracle: the prefill on every head at four rows of every
256-row query tile (each row's full score row), the decode on every sequence
and query head. The errors, tolerances and a pass flag go into the JSON line
(``parity``); a failed check makes the run exit with status 1 after printing
it.

The CPU baseline is the fp64 oracle run on a bounded sample of the same
prefill workload (whole heads, every row) on this host's cores.

``roofline.sustained_prefill`` and ``roofline.gemm_bf16_ceiling`` are the
prefill and the vendor bf16 GEMM (random operands) each run back to back for
a few seconds after the timed steps, with the board's power and GFX clocks
read once by amd-smi halfway through: the rates the board holds under its
power limit, as fractions of the datasheet peak and of the peak at the
sampled clock.

``roofline.traffic`` is the HBM bytes per call from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters calibrated on a copy of known size, as recorded in
profiles/hbm_traffic.txt; it is null when the kernel sources no longer
match the ones those counters were taken on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (prefill) & KV GB/s (paged decode), % of MI355X peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_CLOCK_MHZ = 2400.0     # the engine clock the bf16 peak is quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "io_aware_exact_flashattention_amd", "csrc")
KERNEL_SOURCES = {
    "prefill": ["fa_fwd.hip", "fa_device.h", "fa_internal.h", "fa_api.cpp"],
    "decode": ["fa_decode.hip", "fa_device.h", "fa_internal.h", "fa_api.cpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def sources_sha256(which: str) -> str:
    """SHA-256 of the path's source files with comments and whitespace
    removed, so that editing a comment does not retire recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(CSRC, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()


def measured_traffic(which: str):
    """HBM bytes per call (FETCH_SIZE + WRITE_SIZE, calibrated against a copy
    of known size) recorded for the current kernel sources; None when the
    sources changed since the counters were taken, or none were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    sha = sources_sha256(which)
    for ln in lines:
        if not ln.startswith("path="):
            continue
        kv = dict(f.split("=", 1) for f in ln.split())
        if kv.get("path") == which and kv.get("sources_sha256") == sha:
            return {"bytes_per_call": int(kv["hbm_bytes_per_call"]),
                    "fetch_bytes": int(kv["fetch_bytes_per_call"]),
                    "write_bytes": int(kv["write_bytes_per_call"])}
    return None


def host_info():
    """CPU model, core count and the BLAS library NumPy's products run on."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = int(i.get("num_threads", 1))
                break
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "host_cores": os.cpu_count(), "blas": blas, "blas_threads": threads}


def cpu_baseline(x, heads: int):
    """fp64 oracle on `heads` whole heads of the prefill workload."""
    import fa_inputs as fi
    import oracle
    info = host_info()
    B, Nq, Nk, Hq, Hkv, d = x.shape
    t0 = time.perf_counter()
    for h in range(heads):
        qh = fi.to_f64(x.q[0, :, h], "bf16")
        kh = fi.to_f64(x.k[0, :, h], "bf16")
        vh = fi.to_f64(x.v[0, :, h], "bf16")
        oracle.attention_head(qh, kh, vh, x.scale, True)
    dt = time.perf_counter() - t0
    flops = fi.prefill_flops([Nq], [Nk], heads, d, True)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(info["blas_threads"] or 1), "kind": "oracle",
            "sample": f"{heads} of 32 heads of the causal N=16384 d=128 prefill, all rows, "
                      f"fp64 NumPy (matrix products on {info['blas_threads']} BLAS threads, "
                      f"element-wise passes on one), {dt:.1f} s",
            "seconds": dt, **info}


def device_info():
    """CU count and engine clock of the GPU as rocminfo reports them."""
    import subprocess

    import torch
    prop = torch.cuda.get_device_properties(0)
    out = {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
           "compute_units": prop.multi_processor_count, "max_clock_mhz": None}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        agent = txt.split("gfx950", 1)[1] if "gfx950" in txt else ""
        for ln in agent.splitlines():
            if "Max Clock Freq" in ln:
                out["max_clock_mhz"] = int(ln.split(":", 1)[1].split()[0])
                break
    except Exception:  # pragma: no cover
        pass
    if out["max_clock_mhz"]:
        # dense 16-bit MFMA: 4096 flop per clock per CU (32x32x16 in 32 clocks per SIMD)
        out["bf16_peak_from_clock_tflops"] = (out["compute_units"] * 4096 *
                                              out["max_clock_mhz"] * 1e6 / 1e12)
    return out


def check_prefill(x, o, lse):
    """Oracle on every head at four rows of each 256-row query tile (the
    first and last row of the tile and two seeded ones); each row's full
    score row is formed."""
    import numpy as np

    import fa_inputs as fi
    from tests import full_oracle
    from tests.util import LSE_TOL, O_TOL, lse_error, o_error, to_f64
    B, Nq, Nk, Hq, Hkv, d = x.shape
    rng = np.random.default_rng(2024)
    rows = []
    for t0 in range(0, Nq, 256):
        t1 = min(Nq, t0 + 256)
        rows += [t0, t1 - 1] + rng.integers(t0, t1, 2).tolist()
    rows = np.unique(rows)
    O, L = full_oracle.dense_heads(x, range(Hq), rows=rows)
    og = to_f64(o[0, torch_index(rows, o.device)])
    lg = to_f64(lse[0, torch_index(rows, o.device)])
    eo = o_error(og, O, np.array([np.abs(fi.to_f64(x.v, "bf16")).max()]))
    el = lse_error(lg, L)
    return {"err_O": eo, "err_LSE": el, "tol_O": O_TOL["bf16"], "tol_LSE": LSE_TOL["bf16"],
            "finite": bool(np.isfinite(og).all()),
            "pass": bool(eo <= O_TOL["bf16"] and el <= LSE_TOL["bf16"] and np.isfinite(og).all()),
            "checked": f"all {Hq} heads x {len(rows)} of {Nq} rows (4 per 256-row query tile)"}


def torch_index(rows, device):
    import torch
    return torch.as_tensor(rows, dtype=torch.long, device=device)


def check_decode(p, o, lse):
    """Oracle on every sequence and query head, fed each sequence's
    contiguous K/V (no page table)."""
    import numpy as np

    import fa_inputs as fi
    from tests import full_oracle
    from tests.util import LSE_TOL, O_TOL, lse_error, o_error, to_f64
    seq = lambda src: (lambda b: src[p.cu_k[b]:p.cu_k[b + 1]])
    O, L = full_oracle.decode_all(p.q, seq(p.k_seq), seq(p.v_seq), "bf16", p.scale)
    og, lg = to_f64(o), to_f64(lse)
    eo = o_error(og, O, np.array([np.abs(fi.to_f64(p.v_seq, "bf16")).max()]))
    el = lse_error(lg, L)
    B, Hq, _ = p.q.shape
    return {"err_O": eo, "err_LSE": el, "tol_O": O_TOL["bf16"], "tol_LSE": LSE_TOL["bf16"],
            "finite": bool(np.isfinite(og).all()),
            "pass": bool(eo <= O_TOL["bf16"] and el <= LSE_TOL["bf16"] and np.isfinite(og).all()),
            "checked": f"all {B} sequences x {Hq} query heads"}


PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector, published


def other_configs(torch, fa, fi, to_dev, dev, reps=20):
    """Throughput of the remaining parity workloads (reported, not part of
    `value`): HIP events around each call on the current stream, after
    warm-up calls."""
    import numpy as np
    stream = torch.cuda.current_stream(dev)
    res = {}

    def timed(fn):
        for _ in range(10):  # clocks ramp up after the small cases before
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        return float(np.mean(ms)), float(np.min(ms))

    def dense_case(key, x, peak, desc):
        B, Nq, Nk, Hq, Hkv, d = x.shape
        q, k, v = to_dev(x.q, x.dtype), to_dev(x.k, x.dtype), to_dev(x.v, x.dtype)
        o, l = fa.fwd(q, k, v, causal=x.causal, scale=x.scale)
        mean, mn = timed(lambda: fa.fwd(q, k, v, causal=x.causal, scale=x.scale, out=o, lse=l))
        flops = fi.prefill_flops([Nq] * B, [Nk] * B, Hq, d, x.causal)
        tf = flops / (mean * 1e-3) / 1e12
        res[key] = {"workload": desc, "dtype": x.dtype, "ms_mean": mean, "ms_min": mn,
                    "tflops": tf, "peak_tflops": peak, "frac": tf / peak}

    dense_case("cfg0", fi.cfg0(), PEAK_FP32_VALU_TFLOPS,
               "fp32 B=1 H=1 N=256 d=64, no mask (fwd_f32_kernel; launch-latency bound)")
    dense_case("cfg1_bf16", fi.cfg1(), PEAK_BF16_TFLOPS, "causal bf16 B=4 H=16 N=2048 d=64")
    dense_case("cfg1_bf16_qx8", fi.cfg1(q_mult=8.0), PEAK_BF16_TFLOPS,
               "causal bf16 B=4 H=16 N=2048 d=64, Q x8 (logits to about +-45)")
    dense_case("cfg1_f16", fi.cfg1(dtype="f16"), PEAK_BF16_TFLOPS, "causal fp16 B=4 H=16 N=2048 d=64")

    x = fi.cfg3()
    q, k, v = to_dev(x.q, x.dtype), to_dev(x.k, x.dtype), to_dev(x.v, x.dtype)
    cq, ck = to_dev(x.cu_q, "i32"), to_dev(x.cu_k, "i32")
    o, l = fa.fwd_varlen(q, k, v, cq, ck, x.max_q, x.max_k, causal=True, scale=x.scale)
    mean, mn = timed(lambda: fa.fwd_varlen(q, k, v, cq, ck, x.max_q, x.max_k, causal=True,
                                           scale=x.scale, out=o, lse=l))
    lq = np.diff(x.cu_q)
    flops = fi.prefill_flops(lq, np.diff(x.cu_k), x.q.shape[1], x.q.shape[2], True)
    tf = flops / (mean * 1e-3) / 1e12
    res["cfg3"] = {"workload": "ragged causal GQA bf16, 8 sequences U[128,4096] seed 3, Hq=32 Hkv=8 d=128",
                   "dtype": "bf16", "ms_mean": mean, "ms_min": mn, "tflops": tf,
                   "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}

    # chunked prefill over a paged cache: work = 4 Hq d x (visible query-key
    # pairs), query i of a chunk seeing Lk - Lq + i + 1 keys
    lq, lk = fi.chunked_prefill_lengths()
    x = fi.paged_prefill(lq, lk, 32, 8, 128, "bf16", seed=5)
    kv = x.kv
    q, kp, vp = to_dev(x.q, "bf16"), to_dev(kv.k_pool, "bf16"), to_dev(kv.v_pool, "bf16")
    cq, pt, sl = to_dev(x.cu_q, "i32"), to_dev(kv.page_table, "i32"), to_dev(kv.seq_lens, "i32")
    o, l = fa.fwd_paged(q, kp, vp, cq, pt, sl, x.max_q, scale=kv.scale)
    mean, mn = timed(lambda: fa.fwd_paged(q, kp, vp, cq, pt, sl, x.max_q, scale=kv.scale,
                                          out=o, lse=l))
    pairs = float(np.sum(lq * (lk - lq) + lq * (lq + 1) / 2))
    tf = 4.0 * 32 * 128 * pairs / (mean * 1e-3) / 1e12
    res["chunked_prefill_paged"] = {
        "workload": "fa_fwd_paged: 16 chunks U[1,2048] after cached prefixes U[0,8192] seed 5, "
                    "page 16 (permuted pool), Hq=32 Hkv=8 d=128, causal",
        "dtype": "bf16", "ms_mean": mean, "ms_min": mn, "tflops": tf,
        "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}

    # appending the chunks' K/V rows to the paged cache (the step before the
    # chunked prefill above): bytes = K and V rows read once and written once
    lens_before = (lk - lq).astype(np.int32)
    cu_new = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    k_new = np.concatenate([kv.k_seq[kv.cu_k[s] + lens_before[s]:kv.cu_k[s + 1]] for s in range(len(lq))])
    v_new = np.concatenate([kv.v_seq[kv.cu_k[s] + lens_before[s]:kv.cu_k[s + 1]] for s in range(len(lq))])
    kn, vn = to_dev(k_new, "bf16"), to_dev(v_new, "bf16")
    cn, lb = to_dev(cu_new, "i32"), to_dev(lens_before, "i32")
    a_mean, a_min = timed(lambda: fa.kv_append(kn, vn, kp, vp, cn, pt, lb))
    moved = 2 * 2 * k_new.size * 2  # K and V, read and written, 2 bytes each
    res["kv_append_chunks"] = {
        "workload": "fa_kv_append: the 16 chunks above (U[1,2048] tokens after cached prefixes "
                    "U[0,8192]) written into the permuted page pool, Hkv=8 d=128",
        "dtype": "bf16", "ms_mean": a_mean, "ms_min": a_min, "tokens": int(k_new.shape[0]),
        "gbs": moved / (a_mean * 1e-3) / 1e9, "peak_gbs": PEAK_HBM_GBS,
        "frac": moved / (a_mean * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del kn, vn, cn, lb

    # backward pass (fa_bwd): work = the five products of the chain rule
    # (S, dP, dV, dK, dQ: 10 * Hq * Nq * Nk * d flops, halved when causal);
    # the kernels recompute S and dP once more (seven products)
    for key, x, desc in (
            ("bwd_long_context", fi.cfg2(),
             "fa_bwd: causal bf16 B=1 H=32 N=16384 d=128 (dQ kernel + dK/dV kernel)"),
            ("bwd_causal_B4_H16_N2048_d64", fi.cfg1(),
             "fa_bwd: causal bf16 B=4 H=16 N=2048 d=64 (dQ kernel + dK/dV kernel)")):
        B, Nq, Nk, Hq, Hkv, d = x.shape
        q, k, v = to_dev(x.q, x.dtype), to_dev(x.k, x.dtype), to_dev(x.v, x.dtype)
        o, l = fa.fwd(q, k, v, causal=True, scale=x.scale)
        g_out = to_dev(fi.grad_out((B, Nq, Hq, d), x.dtype, 2), x.dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wsb = torch.empty(fa.bwd_workspace_size(B, Nq, Hq), dtype=torch.uint8, device=dev)
        mean, mn = timed(lambda: fa.bwd(q, k, v, o, l, g_out, causal=True, scale=x.scale, dq=dq,
                                        dk=dk, dv=dv, workspace=wsb))
        flops = 2.5 * fi.prefill_flops([Nq] * B, [Nk] * B, Hq, d, True)
        tf = flops / (mean * 1e-3) / 1e12
        res[key] = {"workload": desc, "dtype": "bf16", "ms_mean": mean, "ms_min": mn,
                    "tflops": tf, "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS,
                    "flops_per_call": flops}
        del q, k, v, o, l, g_out, dq, dk, dv, wsb

    # shared-prompt decode: 64 sequences on one 16384-token prefix; the
    # unique K/V bytes (prefix once + suffixes) and the bytes a plain paged
    # decode would read (prefix once per sequence)
    rng = np.random.default_rng(83)
    suf = rng.integers(1, 2048, 64, endpoint=True)
    c = fi.cascade(16384, suf, 32, 8, 128, "bf16", seed=83)
    cp = c.pool
    cq, ckp, cvp = to_dev(c.q, "bf16"), to_dev(cp.k_pool, "bf16"), to_dev(cp.v_pool, "bf16")
    cpp, cpt, csl = to_dev(c.prefix_pages, "i32"), to_dev(c.page_table, "i32"), to_dev(c.seq_lens, "i32")
    o2, l2 = fa.decode_cascade(cq, ckp, cvp, cpp, c.prefix_len, cpt, csl, scale=cp.scale)
    c_mean, c_min = timed(lambda: fa.decode_cascade(cq, ckp, cvp, cpp, c.prefix_len, cpt, csl,
                                               scale=cp.scale, out=o2, lse=l2))
    row = 8 * 128 * 2 * 2  # K + V bytes per token
    unique = (c.prefix_len + int(suf.sum())) * row
    plain = (64 * c.prefix_len + int(suf.sum())) * row
    res["cascade_decode_shared_prompt"] = {
        "workload": "fa_decode_cascade: 64 sequences sharing a 16384-token prefix, suffixes "
                    "U[1,2048] seed 83, page 16, Hq=32 Hkv=8 d=128",
        "dtype": "bf16", "ms_mean": c_mean, "ms_min": c_min,
        "unique_kv_gbs": unique / (c_mean * 1e-3) / 1e9,
        "plain_decode_equivalent_gbs": plain / (c_mean * 1e-3) / 1e9}
    del cq, ckp, cvp, cpp, cpt, csl, o2, l2

    return res


def board_sample():
    """The board's socket power (W) and the GFX clock of each XCD (MHz), read
    once with amd-smi; None when amd-smi is missing or prints no clocks."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0"], capture_output=True,
                           text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    clks = [int(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
    if not clks:
        return None
    pw = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", r.stdout)
    return {"socket_power_w": float(pw.group(1)) if pw else None, "gfx_clock_mhz": clks,
            "mean_gfx_clock_mhz": sum(clks) / len(clks)}


def sustained(torch, fn, flops, seconds):
    """Runs fn back to back for about `seconds`, reading the board's power
    and clocks once halfway through: the rate a kernel holds under the
    board's power limit, and the clock it holds it at. The matrix-core peak
    at that clock is the datasheet peak scaled by clock / 2.4 GHz."""
    import threading
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        fn()
    e1.record()
    torch.cuda.synchronize()
    calls = max(10, int(seconds * 1e3 / (e0.elapsed_time(e1) / 5)))
    box = {}

    def sample():
        time.sleep(seconds / 2)
        box["board"] = board_sample()

    th = threading.Thread(target=sample)
    th.start()
    e0.record()
    for _ in range(calls):
        fn()
    e1.record()
    torch.cuda.synchronize()
    th.join()
    ms = e0.elapsed_time(e1) / calls
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"calls": calls, "ms_per_call": ms, "tflops": tflops,
           "frac_of_datasheet": tflops / PEAK_BF16_TFLOPS, "board": box.get("board")}
    if out["board"]:
        clk_peak = PEAK_BF16_TFLOPS * out["board"]["mean_gfx_clock_mhz"] / PEAK_CLOCK_MHZ
        out["clock_peak_tflops"] = clk_peak
        out["frac_of_clock_peak"] = tflops / clk_peak
    return out


def gemm_ceiling(torch, dev, seconds=2.0, n=8192):
    """Sustained rate of the vendor bf16 GEMM (torch.matmul, which calls
    hipBLASLt) on N(0,1) operands, M = N = K = n: the dense bf16 matrix-core
    rate this board holds under its power limit, reported next to the
    datasheet peak."""
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    res = sustained(torch, lambda: torch.matmul(a, b, out=c), 2.0 * n ** 3, seconds)
    res["kernel"] = f"torch.matmul bf16 (hipBLASLt) M=N=K={n}, N(0,1) operands"
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle check of the timed outputs (profiling runs)")
    ap.add_argument("--only", choices=["prefill", "decode", "both"], default="both")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the throughput report of the other parity workloads")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the sustained vendor bf16 GEMM rate reported beside the prefill roofline")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, copy this many MiB device-to-device once (a kernel of "
                         "known traffic, to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(it runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fa_inputs as fi
    import io_aware_exact_flashattention_amd as fa
    from tests.util import to_dev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    do_pre = args.only in ("prefill", "both")
    do_dec = args.only in ("decode", "both")

    log("[bench] generating prefill inputs")
    x = fi.cfg2()
    B, Nq, Nk, Hq, Hkv, d = x.shape
    pre_flops = fi.prefill_flops([Nq] * B, [Nk] * B, Hq, d, True)
    if do_pre:
        q, k, v = to_dev(x.q, "bf16"), to_dev(x.k, "bf16"), to_dev(x.v, "bf16")
        o = torch.empty_like(q)
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=dev)

    if do_dec:
        log("[bench] generating decode inputs")
        p = fi.cfg4()
        dq, dkp, dvp = to_dev(p.q, "bf16"), to_dev(p.k_pool, "bf16"), to_dev(p.v_pool, "bf16")
        dpt, dsl = to_dev(p.page_table, "i32"), to_dev(p.seq_lens, "i32")
        kv_bytes = fi.decode_kv_bytes(p.seq_lens, p.k_pool.shape[2], p.k_pool.shape[3], "bf16")
        Bd, Hqd, dd = p.q.shape
        ws = torch.empty(fa.decode_workspace_size(Bd, Hqd, dd, p.max_pages), dtype=torch.uint8,
                         device=dev)
        do_ = torch.empty_like(dq)
        dl = torch.empty((Bd, Hqd), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if do_pre:
            if ev is not None:
                ev[0].record(stream)
            fa.fwd(q, k, v, causal=True, scale=x.scale, out=o, lse=lse)
            if ev is not None:
                ev[1].record(stream)
        if do_dec:
            if ev is not None:
                ev[2].record(stream)
            fa.decode_paged(dq, dkp, dvp, dpt, dsl, scale=p.scale, workspace=ws, out=do_, lse=dl)
            if ev is not None:
                ev[3].record(stream)

    # the first call of each entry point in this process (kernel code loaded
    # on first launch), timed alone
    torch.cuda.synchronize()
    cold_ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_cold = time.perf_counter()
    step(cold_ev)
    torch.cuda.synchronize()
    cold = {"wall_ms": (time.perf_counter() - t_cold) * 1e3}
    if do_pre:
        cold["prefill_ms"] = cold_ev[0].elapsed_time(cold_ev[1])
    if do_dec:
        cold["decode_ms"] = cold_ev[2].elapsed_time(cold_ev[3])

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [e[0].elapsed_time(e[1]) for e in events] if do_pre else []
    dec_ms = [e[2].elapsed_time(e[3]) for e in events] if do_dec else []
    out = {
        "metric": METRIC,
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal bf16 prefill B=1 H=32 N=16384 d=128 (fa_fwd) + paged GQA decode "
                        "64 seqs KV U[512,32768] seed 4, page 16, Hq=32 Hkv=8 d=128 (fa_decode_paged)",
            "prefill": {"B": B, "N": Nq, "H": Hq, "d": d, "causal": True, "flops_per_call": pre_flops},
        },
        "cold_first_call": cold,
        "device": device_info(),
    }
    if do_pre:
        avg = float(np.mean(pre_ms))
        tflops = pre_flops / (avg * 1e-3) / 1e12
        out["value"] = tflops
        out["prefill_ms"] = {"mean": avg, "median": float(np.median(pre_ms)), "min": float(np.min(pre_ms))}
        tr = measured_traffic("prefill")
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                           "traffic": tr["bytes_per_call"] if tr else None,
                           "kernel": "fwd_mfma_kernel<Bf16,128,causal>"}
    if do_dec:
        avg = float(np.mean(dec_ms))
        tr_dec = measured_traffic("decode")
        gbs = kv_bytes / (avg * 1e-3) / 1e9
        out["decode"] = {
            "value": gbs, "unit": "GB/s", "kv_bytes_per_call": kv_bytes,
            "ms": {"mean": avg, "median": float(np.median(dec_ms)), "min": float(np.min(dec_ms))},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": tr_dec["bytes_per_call"] if tr_dec else None,
                         "kernel": "decode_split_kernel + decode_combine_kernel"},
        }
    if do_pre and not args.no_ceiling:
        log("[bench] prefill held back to back for 3 s, board power and clocks sampled")
        burst = sustained(torch, lambda: fa.fwd(q, k, v, causal=True, scale=x.scale, out=o, lse=lse),
                          pre_flops, 3.0)
        burst["kernel"] = "fwd_mfma_kernel<Bf16,128,causal>, the timed workload"
        out["roofline"]["sustained_prefill"] = burst
        log("[bench] sustained bf16 GEMM rate (matrix-core ceiling under the power limit)")
        ceil = gemm_ceiling(torch, dev)
        ceil["prefill_frac_of_gemm"] = out["value"] / ceil["tflops"]
        out["roofline"]["gemm_bf16_ceiling"] = ceil
    parity_ok = True
    if not args.no_check:
        out["parity"] = {}
        if do_pre:
            log("[bench] checking the timed prefill output against the oracle")
            out["parity"]["prefill"] = check_prefill(x, o, lse)
            parity_ok &= out["parity"]["prefill"]["pass"]
        if do_dec:
            log("[bench] checking the timed decode output against the oracle")
            out["parity"]["decode"] = check_decode(p, do_, dl)
            parity_ok &= out["parity"]["decode"]["pass"]
        out["parity"]["pass"] = bool(parity_ok)
    if do_dec:
        del p.k_seq, p.v_seq
    if not args.no_other:
        log("[bench] other workloads")
        out["other_configs"] = other_configs(torch, fa, fi, to_dev, dev)
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_heads)
        # the same work rate on the GPU over the oracle's on the host
        out["cpu_baseline"]["gpu_over_oracle"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)
    if not parity_ok:
        log("[bench] the timed outputs do not match the oracle")
        sys.exit(1)


if __name__ == "__main__":
    main()
