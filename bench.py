"""Benchmark of the Pingala-8 hot path on one MI355X.

Headline workload: the 36-layer Qwen3-4B-shaped linear stack at batch 1
(uniform random trellis bitstreams, fp16 U(0.005, 0.05) scales, fp16 N(0,1)
input fed layer to layer; 965,099,520 coded bytes per token).  One step is
one token through the whole stack: per layer four launches of the fused
stage kernel (RMS normalisation + activation rotation + qgemv; qkv and
gate/up merged), replayed from a HIP graph.  Inputs are resident in HBM
before timing starts.

Printed: one JSON line.  `value` is the whole-job compressed-weight GB/s of
the headline stack (bytes per token x tokens per second).  `roofline` is the
stage kernel's: coded bytes per launch over its average launch duration,
timed with HIP events around every weight-reading launch on the launch
stream.  Extra keys carry the other measurements: the Llama-3.1-8B-shaped
stack at batch 1 and 4, the 512 x 2048 layer's microseconds per call (warm
and cold), each Qwen3-4B matrix's cold GB/s, a streaming-read kernel's HBM
bandwidth, the prompt path's matrix-core fraction, the GPU encoder, and the
CPU oracle on one core and on all the host cores given to this process.
"""
from __future__ import annotations

import os

# the CPU oracle is timed per core: one BLAS thread per process
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

import argparse  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "qgemv compressed-weight GB/s (% HBM peak) + linear-stack tok/s at batch 1"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0          # dense bf16
FP64_OPS_PEAK_T = 39.3             # fp64 vector instructions per second (78.6 TFLOP/s counts an FMA as two)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading),
    or None when there is none or the kernel's source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "kernel_source:", "kernel_source_sha256:")))
    # the kernel's source files, hashed in the order listed
    srcs = [os.path.join(ROOT, f) for f in fields.get("kernel_source", "").split()]
    if not srcs or not all(os.path.exists(f) for f in srcs):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if h.hexdigest() != fields.get("kernel_source_sha256", "").strip():
        return None
    return int(fields["traffic_bytes_per_launch"])


def host_cores() -> int:
    """Host cores this process may use (capped at 16, the share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# ------------------------------------------------------------------ CPU oracle

def _oracle_chunk(args):
    from oracle import p8f
    codes, scales, x = args
    t0 = time.perf_counter()
    p8f.gemv_ref(codes, scales, x)
    return codes.nbytes + scales.nbytes, time.perf_counter() - t0


def cpu_baseline(seconds: float = 12.0, cores: int = 1):
    """The oracle (numpy fp64 decode + product), as it stands, on a bounded
    sample of the stack: the layer-0 launch groups of the Qwen3-4B-shaped
    stack, repeated until `seconds` have passed.  cores = 1: one process;
    cores > 1: a process pool over 256-row chunks of the same products."""
    import numpy as np

    from qgemv_amd import synth

    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    x = {s: synth.activations_f32(1, merged[s][0].shape[1] * 4) for s in merged}
    if cores <= 1:
        from oracle import p8f
        done_bytes, t0, mats = 0, time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for site in ("o", "qkv", "down", "gu"):
                codes, scales = merged[site]
                p8f.gemv_ref(codes, scales, x[site])
                done_bytes += codes.nbytes + scales.nbytes
                mats += 1
                if time.perf_counter() - t0 >= seconds:
                    break
        dt = time.perf_counter() - t0
        gbs = done_bytes / dt / 1e9
        return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{mats} launch-group products of layer 0 (decode + fp64 GEMV, batch 1) in {dt:.1f} s "
                          f"on one core; {done_bytes} coded bytes",
                # the 36-layer stack's coded bytes per token at this rate (extrapolated from layer 0)
                "stack_tok_per_s_extrapolated": gbs * 1e9 / (36 * sum(
                    n * k // 4 + n * k // 64 for n, k in synth.merged_shapes(synth.qwen3_4b_shapes()).values()))}
    import multiprocessing as mp
    jobs = []
    for site in ("o", "qkv", "down", "gu"):
        codes, scales = merged[site]
        for r in range(0, codes.shape[0], 256):
            jobs.append((np.ascontiguousarray(codes[r:r + 256]), np.ascontiguousarray(scales[r:r + 256]), x[site]))
    ctx = mp.get_context("spawn")                  # workers hold no GPU state
    done_bytes, rounds = 0, 0
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_chunk, jobs[:cores])                 # start the workers
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for nb, _ in pool.imap_unordered(_oracle_chunk, jobs):
                done_bytes += nb
            rounds += 1
        dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{rounds} passes over the layer-0 launch groups (decode + fp64 GEMV, batch 1), 256-row chunks "
                      f"over a pool of {cores} processes, in {dt:.1f} s; {done_bytes} coded bytes"}


def cpu_qgemm(seconds: float = 6.0, m: int = 64):
    """The oracle's prompt product (decode + fp64 matrix product) on one
    core, on a bounded sample of the prompt workload: m rotated bf16 rows
    against each Qwen3-4B layer-0 launch group, repeated until `seconds` have
    passed; GFLOP/s = 2 m n k per second."""
    import numpy as np

    from oracle import p8f
    from qgemv_amd import synth

    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    xs = {s: p8f.bf16_bits_to_float(synth.bf16_activations_bits(m, merged[s][0].shape[1] * 4, seed=m))
          for s in merged}
    flop, mats, t0 = 0.0, 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for site in ("o", "qkv", "down", "gu"):
            codes, scales = merged[site]
            p8f.gemm_ref(codes, scales, xs[site])
            flop += 2.0 * m * codes.shape[0] * codes.shape[1] * 4
            mats += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return {"value": flop / dt / 1e9, "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{mats} launch-group products of layer 0 at m = {m} (decode + fp64 product) in {dt:.1f} s "
                      f"on one core"}


# ----------------------------------------------------------------- GPU stacks

def time_launches(st, stream, reps: int = 10):
    """Average duration of the weight-reading launches of each site: one HIP
    graph per site holding that site's product launch of every layer, replayed
    `reps` times between HIP events on the launch stream (launch-to-launch
    time of back-to-back launches, dispatch included; no event inside)."""
    import torch
    per, nlaunch = {}, 0
    calls = {}
    for kind, layer, site, call in st.launches():       # the stream current at call time (the capture's)
        if kind == "product":
            calls.setdefault(site, []).append(call)
    for site, cs in calls.items():
        g = _graph_of(cs)
        per[site] = 1e3 * _time_graph(g, reps) / len(cs)
        nlaunch += reps * len(cs)
        del g
    torch.cuda.synchronize()
    return per, nlaunch


def run_stack(st, steps: int, warmup: int, use_graph: bool = True):
    """Whole-job timing of `steps` tokens: HIP events on the launch stream
    around exactly `steps` replays (graph) or eager tokens, synchronised on
    both sides."""
    import torch
    stream = torch.cuda.current_stream()
    if use_graph:
        st.capture()
    step = st.replay if use_graph else st.token
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    return max(gpu_ms, wall * 1e3) / steps, gpu_ms, wall * 1e3


def stack_result(st, ms_per_step: float, batch: int, per_site_us: dict):
    """Throughput of a stack and its per-launch figures."""
    bytes_tok = st.bytes_per_token
    sizes = {s: 0 for s in per_site_us}
    for layer in range(st.layers):
        for s in per_site_us:
            sizes[s] += st.codes[layer][s].numel() + st.scales[layer][s].numel() * 2
    per = {}
    for s, us in per_site_us.items():
        b = sizes[s] // st.layers
        per[s] = {"n": st.shapes[s][0], "k": st.shapes[s][1], "coded_bytes": b, "us": round(us, 3),
                  "gbs": round(b / (us * 1e-6) / 1e9, 1)}
    launches = 4 * st.layers
    avg_us = sum(per_site_us[s] for s in per_site_us) / len(per_site_us)
    value = bytes_tok * (1e3 / ms_per_step) / 1e9
    return {"ms_per_step": round(ms_per_step, 4), "tok_per_s": round(batch * 1e3 / ms_per_step, 2),
            "gbs": round(value, 2), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "bytes_per_token": bytes_tok, "weight_launches_per_token": launches,
            "avg_weight_launch_us": round(avg_us, 3), "per_site": per}


def codebook_tensor(table: str):
    """Device codebook table for the table-driven path: "v1" is P8F v1's own
    (pg_codebook_table), "gauss" a seeded rounded-Gaussian int8 table, "r23"
    the rate-2/3 variant's own (read on its trellis)."""
    import numpy as np
    import torch

    import qgemv_amd as q
    from qgemv_amd import synth
    if table == "r23":
        t = q.pg_codebook_table_ex(q.PG_FLAG_RATE23)
    else:
        t = q.pg_codebook_table() if table == "v1" else synth.random_codebook_table(22, "gauss")
    return torch.from_numpy(np.ascontiguousarray(t)).cuda()


def build_stack(workload: str, batch: int, path: str, carry: bool, table: str = "none"):
    from qgemv_amd import _lib as L
    from qgemv_amd import synth
    from qgemv_amd.stack import Stack
    shapes = synth.qwen3_4b_shapes() if workload == "qwen36" else synth.llama31_8b_shapes()
    layers = 36 if workload == "qwen36" else 32
    fused = path in ("fused", "hybrid")
    split_above = 4096 if path == "hybrid" else None
    tab = codebook_tensor(table) if table != "none" else None
    return Stack(shapes, layers, batch=batch, x_dtype=L.PG_Q16, fused=fused, carry=carry, split_above=split_above,
                 table=tab, rate23=table == "r23")


def run_table_stacks(steps: int, warmup: int):
    """The Qwen3-4B-shaped 36-layer stack at batch 1 with every launch group
    through a codebook table in LDS (pg_rot_qgemv_table): P8F v1's own table
    and a rounded-Gaussian one, and the rate-2/3 trellis with its own table,
    each timed as the headline."""
    import torch
    out = {}
    for table in ("v1", "gauss", "r23"):
        st = build_stack("qwen36", 1, "fused", False, table)
        ms, _, _ = run_stack(st, steps, warmup)
        per, _ = time_launches(st, torch.cuda.current_stream(), reps=5)
        out[table] = {"kernel": "k_rot_qgemv1<TAB=1> (pg_rot_qgemv_table)", **stack_result(st, ms, 1, per)}
        log(f"table {table}: {out[table]['ms_per_step']} ms/step, {out[table]['gbs']} GB/s")
        del st
        torch.cuda.empty_cache()
    return out


def auto_path(batch: int, carry: bool) -> str:
    # the v_dot4 fused stage at batch 1; from batch 2 on the matrix cores,
    # whose cost hardly grows with the batch: the fused stage where the
    # batch's rotated activations fit in LDS (k <= 4096), the rotation +
    # product elsewhere (hybrid)
    return "fused" if batch <= 1 or carry else "hybrid"


# ------------------------------------------------------- single-matrix timing

def _graph_of(calls):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls[:2]:
            c()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    return g


def _time_graph(g, reps: int):
    import torch
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def matrix_timing(codes, scales, n: int, k: int, x, x_dt: int, flags: int, signs, min_bytes: int = 1 << 30,
                  launches: int = 200):
    """Microseconds per pg_rot_qgemv call (batch 1) on one matrix: warm (the
    same copy every call, cache-resident) and cold (cycling through distinct
    device copies that together hold >= min_bytes, more than four times the
    256 MB last-level cache)."""
    import torch
    import qgemv_amd as q
    per = codes.numel() + scales.numel() * 2
    copies = max(1, -(-min_bytes // per))
    cbig = codes.repeat(copies, 1)          # copy i is rows [i n, (i + 1) n)
    sbig = scales.repeat(copies, 1)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    warm = [lambda: q.pg_rot_qgemv(codes, scales, n, k, x, x_dt, k, signs, flags, 1, y)] * launches
    cold = []
    for i in range(min(copies, 4096)):
        ci, si = cbig[i * n:(i + 1) * n], sbig[i * n:(i + 1) * n]
        cold.append(lambda ci=ci, si=si: q.pg_rot_qgemv(ci, si, n, k, x, x_dt, k, signs, flags, 1, y))
    while len(cold) < launches:
        cold = cold + cold
    gw, gc = _graph_of(warm), _graph_of(cold)
    us_w = 1e3 * _time_graph(gw, 5) / len(warm)
    us_c = 1e3 * _time_graph(gc, 2) / len(cold)
    del cbig, sbig
    return {"coded_bytes": per, "warm_us": round(us_w, 3), "cold_us": round(us_c, 3),
            "warm_gbs": round(per / (us_w * 1e-6) / 1e9, 1), "cold_gbs": round(per / (us_c * 1e-6) / 1e9, 1),
            "cold_copies": copies, "cold_bytes": copies * per}


def run_single_layer():
    """The 512 x 2048 layer (W ~ N(0,1) from seed 0, encoded by pg_encode),
    batch-1 fp16 input, no normalisation: one pg_rot_qgemv per call."""
    import torch
    import qgemv_amd as q
    from qgemv_amd import synth
    w = synth.single_layer_weights()
    n, k = w.shape
    sb = torch.from_numpy(synth.site_sign_bits(0, 0, k)).cuda()
    c = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    s = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode(torch.from_numpy(w).cuda(), n, k, sb, c, s)
    x = torch.from_numpy(synth.activations_fp16(1, k)).cuda()
    r = matrix_timing(c, s, n, k, x, q.PG_F16, 0, sb)
    r["workload"] = "512 x 2048 layer, N(0,1) weights encoded on the GPU, batch-1 fp16 input, pg_rot_qgemv"
    return r


def run_layer_cold():
    """Each matrix of one Qwen3-4B-shaped layer (0.02 N(0,1) weights with
    0.1% outliers x20, encoded by pg_encode), batch-1 fp32 input with the RMS
    normalisation, timed cold over >= 1 GB of distinct copies."""
    import torch
    import qgemv_amd as q
    from qgemv_amd import synth
    out = {}
    x32 = None
    for name in synth.MATS:
        w = synth.qwen_layer_weights(name)
        n, k = w.shape
        sb = torch.from_numpy(synth.site_sign_bits(0, synth.SITE_OF[name], k)).cuda()
        c = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
        s = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
        q.pg_encode(torch.from_numpy(w).cuda(), n, k, sb, c, s)
        x32 = torch.from_numpy(synth.activations_f32(1, k)).cuda()
        r = matrix_timing(c, s, n, k, x32, q.PG_F32, q.PG_FLAG_RMSNORM, sb)
        out[name] = {"n": n, "k": k, **r}
        del c, s
    return out


def run_hbm_read(nbytes: int = 4 << 30, reps: int = 5):
    """pg_hbm_read over a 4 GiB buffer: the bandwidth a plain streaming read
    reaches, checked against the XOR of the buffer."""
    import numpy as np
    import torch
    import qgemv_amd as q
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.random_()
    ref = int(np.bitwise_xor.reduce(buf[: 1 << 24].cpu().numpy().view(np.uint32)))
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.pg_hbm_read(buf[: 1 << 24], 1 << 26, out)
    torch.cuda.synchronize()
    ok = (int(out.item()) & 0xFFFFFFFF) == ref
    stream = torch.cuda.current_stream()
    q.pg_hbm_read(buf, nbytes, out)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        q.pg_hbm_read(buf, nbytes, out)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return {"kernel": "k_hbm_read (pg_hbm_read)", "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "xor_check": ok}


def run_qgemm(stream_iters: int = 10, rounds_n: int = 5):
    """Prompt path on the matrix cores: pg_qgemm_ex on the Qwen3-4B layer-0
    launch groups (random codes and scales as in the stack), X = bf16 N(0,1)
    rows rotated once by pg_fwht_rotate (bf16 -> bf16), at m = 512 and 4096,
    with the workspace pg_qgemm_workspace_bytes asks for (allocated before the
    timed calls; shapes whose tiles fill the chip in whole rounds ask for none
    and run unsplit).  Each product is timed alone with HIP events on the launch
    stream: after 3 warm-up calls, `rounds_n` rounds of `stream_iters`
    back-to-back calls (the split sum included), the median round per call
    (the first calls of a shape run slower while the clocks settle); the
    fraction is 2 m n k per second over the 2.5 PFLOP/s dense bf16 peak."""
    import numpy as np
    import torch

    import qgemv_amd as q
    from qgemv_amd import synth

    shapes = synth.qwen3_4b_shapes()
    merged = synth.random_layer_merged(0, shapes)
    site_no = {"qkv": 0, "o": 1, "gu": 2, "down": 3}
    stream = torch.cuda.current_stream()
    out = {"bound": "mfma", "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16 x bf16 -> f32",
           "kernel": "k_qgemm_v7<8,4,128> (+ k_qgemm_sum when split) (pg_qgemm_ex)", "workload": "Qwen3-4B layer-0 launch groups qkv/o/gu/down, "
           "random trellis bitstreams, bf16 N(0,1) rows", "per_m": {}}
    for m in (512, 4096):
        tot_flop = tot_us = 0.0
        per = {}
        for site, (codes, scales) in merged.items():
            n, k = codes.shape[0], codes.shape[1] * 4
            cd = torch.from_numpy(codes).cuda()
            sc = torch.from_numpy(scales.view(np.int16)).cuda()
            xb = torch.from_numpy(synth.bf16_activations_bits(m, k, seed=m + k).view(np.int16)).cuda()
            xr = torch.empty_like(xb)
            sb = torch.from_numpy(synth.site_sign_bits(0, site_no[site], k)).cuda()
            q.pg_fwht_rotate(xb, q.PG_BF16, xr, q.PG_BF16, sb, m, k, 0)
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            wsb = q.pg_qgemm_workspace_bytes(n, k, m)
            ws = torch.empty((max(wsb, 16) // 4,), dtype=torch.float32, device="cuda")
            for _ in range(3):
                q.pg_qgemm_ex(cd, sc, n, k, xr, m, y, ws, wsb)
            torch.cuda.synchronize()
            rounds = []
            for _ in range(rounds_n):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(stream_iters):
                    q.pg_qgemm_ex(cd, sc, n, k, xr, m, y, ws, wsb)
                e1.record(stream)
                torch.cuda.synchronize()
                rounds.append(1e3 * e0.elapsed_time(e1) / stream_iters)
            us = float(np.median(rounds))
            flop = 2.0 * m * n * k
            tf = flop / (us * 1e-6) / 1e12
            per[site] = {"n": n, "k": k, "us": round(us, 2), "us_min_max": [round(min(rounds), 2), round(max(rounds), 2)],
                         "tflops": round(tf, 1),
                         "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "workspace_bytes": wsb}
            tot_flop += flop
            tot_us += us
        tf = tot_flop / (tot_us * 1e-6) / 1e12
        out["per_m"][str(m)] = {"achieved": round(tf, 1), "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                                "gflop": round(tot_flop / 1e9, 1), "us": round(tot_us, 1), "sites": per}
        log(f"qgemm m={m}: {tf:.1f} TFLOP/s ({100 * tf / MFMA_PEAK_TFLOPS:.1f}% of peak)")
    return out


def run_encode():
    """Offline side: the GPU trellis encoder (pg_encode) on the seven
    Qwen3-4B-shaped matrices of one layer (0.02 N(0,1) weights with 0.1%
    outliers x20), each timed alone with HIP events on the launch stream, and
    the host reference encoder (pg_encode_ref, all host cores) on 64 rows of
    each as the CPU figure.  The search scores 128 points of 4 values in each
    of 4 cosets per group of 4 weights: 4 x 128 x 11 / 4 = 1408 fp64
    operations per weight (none fused), the encoder's algorithmic work, set
    against the fp64 instruction rate (78.6 TFLOP/s counts an FMA as two
    operations; the encoder issues none, so its peak is 39.3 T operations/s)."""
    import numpy as np
    import torch

    import qgemv_amd as q
    from qgemv_amd import synth

    stream = torch.cuda.current_stream()
    tot_w = tot_ms = cpu_w = cpu_s = 0.0
    per = {}
    for name in synth.MATS:
        w = synth.qwen_layer_weights(name)
        n, k = w.shape
        sb = synth.site_sign_bits(0, synth.SITE_OF[name], k)
        wd = torch.from_numpy(w).cuda()
        sbd = torch.from_numpy(sb).cuda()
        c = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
        q.pg_encode(wd, n, k, sbd, c, sc)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        q.pg_encode(wd, n, k, sbd, c, sc)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        rows = 64
        hc = np.zeros((rows, k // 4), np.uint8)
        hs = np.zeros((rows, k // 128), np.uint16)
        t0 = time.perf_counter()
        q.pg_encode_ref(np.ascontiguousarray(w[:rows]), rows, k, sb, hc, hs, host_cores())
        cpu_s += time.perf_counter() - t0
        cpu_w += rows * k
        if not np.array_equal(c[:rows].cpu().numpy(), hc):
            raise SystemExit(f"pg_encode differs from pg_encode_ref on {name}")
        per[name] = {"n": n, "k": k, "ms": round(ms, 3), "gweights_per_s": round(n * k / ms / 1e6, 2)}
        tot_w += n * k
        tot_ms += ms
    gws = tot_w / tot_ms / 1e6
    tops = 1408.0 * gws * 1e9 / 1e12
    log(f"encode: {gws:.2f} Gweights/s on the GPU")
    # the encoder through a codebook table on the q matrix: every byte of every
    # state scored, 8 x 256 x 15 / 4 = 7680 fp64 operations per weight
    w = synth.qwen_layer_weights("q")
    n, k = w.shape
    wd = torch.from_numpy(w).cuda()
    sbd = torch.from_numpy(synth.site_sign_bits(0, 0, k)).cuda()
    c = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    sc = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    tables = {"gauss table, P8F v1 trellis": (torch.from_numpy(synth.random_codebook_table(22, "gauss")).cuda(), 0),
              "rate-2/3 table and trellis": (torch.from_numpy(q.pg_codebook_table_ex(q.PG_FLAG_RATE23)).cuda(),
                                             q.PG_FLAG_RATE23)}
    tab_res = {}
    for label, (tt, fl) in tables.items():
        q.pg_encode_table(wd, n, k, sbd, tt, fl, c, sc)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        q.pg_encode_table(wd, n, k, sbd, tt, fl, c, sc)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        g = n * k / ms / 1e6
        tab_res[label] = {"ms": round(ms, 3), "gweights_per_s": round(g, 3),
                          "t_ops_per_s": round(7680.0 * g / 1e3, 2)}
    log(f"table encode: {tab_res}")
    return {"kernel": "k_encode (pg_encode)", "workload": "Qwen3-4B-shaped layer, 7 matrices, "
            f"{int(tot_w)} weights", "ms": round(tot_ms, 3), "gweights_per_s": round(gws, 2),
            "roofline": {"bound": "alu", "achieved": round(tops, 2), "peak": FP64_OPS_PEAK_T,
                         "unit": "T fp64 operations/s (no FMA)", "frac": round(tops / FP64_OPS_PEAK_T, 4),
                         "ops_per_weight": 1408},
            "cpu_reference": {"mweights_per_s": round(cpu_w / cpu_s / 1e6, 2), "threads": host_cores(),
                              "kind": "pg_encode_ref (host C++, bit-identical output)",
                              "sample": "64 rows of each matrix"},
            "matrices": per,
            "table_encoder": {"kernel": "k_encode_table (pg_encode_table)", "workload": "Qwen3-4B q matrix 4096 x 2560",
                              "ops_per_weight": 7680, **tab_res}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen36", choices=["qwen36", "llama32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 4 times (HBM-counter calibration) and exit")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "split", "hybrid"],
                    help="fused: one pg_rot_qgemv per stage; split: pg_fwht_rotate_ex + pg_qgemv per stage; "
                         "hybrid: fused where k <= 4096, split above; auto: fused at batch 1, hybrid from batch 2")
    ap.add_argument("--batch", type=int, default=1, help="activation rows per step (1..8)")
    ap.add_argument("--carry", action="store_true",
                    help="read the codes as the carried-state variant (state runs on across blocks; fused path)")
    ap.add_argument("--only-stack", action="store_true", help="only the headline stack (for profiling runs)")
    ap.add_argument("--table", default="none", choices=["none", "v1", "gauss", "r23"],
                    help="run the headline stack through a codebook table (pg_rot_qgemv_table; batch 1)")
    ap.add_argument("--only-qgemm", action="store_true",
                    help="only the prompt-path products, printed as one JSON line (for profiling runs)")
    ap.add_argument("--no-qgemm", action="store_true", help="skip the prompt-path (pg_qgemm) measurement")
    ap.add_argument("--no-encode", action="store_true", help="skip the GPU encoder (pg_encode) measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the Llama stack, single-matrix, HBM-read and all-core CPU measurements")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libpingala runs the hot path on a single MI355X "
              "and has no multi-GPU path; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 256 << 20, "bytes_written": 256 << 20,
                          "launches": 4}), flush=True)
        return
    if args.only_qgemm:
        log("timing the prompt path (pg_qgemm)")
        print(json.dumps({"qgemm": run_qgemm()}), flush=True)
        return
    if args.only_stack:
        args.no_qgemm = args.no_encode = args.no_extra = args.no_cpu_baseline = True

    # ---- the headline stack
    path = args.path if args.path != "auto" else auto_path(args.batch, args.carry)
    log(f"building {args.workload}: batch {args.batch}, {path} path")
    if args.table != "none" and (args.batch != 1 or path != "fused"):
        print("--table runs the fused batch-1 path only", file=sys.stderr)
        sys.exit(2)
    st = build_stack(args.workload, args.batch, path, args.carry, args.table)
    stream = torch.cuda.current_stream()
    ms, gpu_ms, wall_ms = run_stack(st, args.steps, args.warmup, use_graph=not args.no_graph)
    log(f"timed {args.steps} steps: {gpu_ms:.2f} ms (events), {wall_ms:.2f} ms (wall)")
    per_site_us, nlaunch = time_launches(st, stream)
    head = stack_result(st, ms, args.batch, per_site_us)
    fused_b1 = path == "fused" and args.batch <= 1
    if args.table != "none":
        kname, kdesc = "k_rot_qgemv1", f"k_rot_qgemv1<TAB=1> (pg_rot_qgemv_table, {args.table} codebook table in LDS)"
    elif fused_b1 and not args.carry:
        kname, kdesc = "k_rot_qgemv1", "k_rot_qgemv1 (pg_rot_qgemv at batch 1: RMS norm + rotation + qgemv, one launch per stage)"
    elif path == "fused":
        kname, kdesc = "k_rot_qgemv", "k_rot_qgemv (pg_rot_qgemv: RMS norm + rotation + qgemv, one launch per stage)"
    elif path == "hybrid":
        kname, kdesc = "k_rot_qmma", ("k_rot_qmma (pg_rot_qgemv at batch 2..8, int8 matrix cores) where k <= 4096, "
                                      "k_qgemv_mma after k_fwht above")
    else:
        kname = "k_qgemv_q16" if args.batch == 1 else "k_qgemv_mma"
        kdesc = f"{kname} (pg_qgemv on PG_Q16 activations, after k_fwht)"
    wl = ("qwen3-4b-36L" if args.workload == "qwen36" else "llama3.1-8b-32L") + f"-b{args.batch}"
    if args.table != "none":
        wl += f"-table-{args.table}"
    bytes_per_launch = st.bytes_per_token // head["weight_launches_per_token"]
    avg_us = head["avg_weight_launch_us"]
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": head["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "i8xi8->i32 (levels x 16-bit activation digits), f32 rotation and scales",
        "data": "synthetic",
        "config": {"workload": f"{'Qwen3-4B' if args.workload == 'qwen36' else 'Llama-3.1-8B'}-shaped "
                               f"{st.layers}-layer linear stack, batch {args.batch}, random trellis bitstreams",
                   "layers": st.layers, "batch": args.batch, "bytes_per_token": st.bytes_per_token,
                   "tok_per_s": head["tok_per_s"], "pct_hbm_peak": head["pct_hbm_peak"],
                   "hip_graphs": not args.no_graph, "path": path,
                   "format": ("carried-state variant" if args.carry else "P8F v1") +
                             (f", {args.table} codebook table" if args.table != "none" else "")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(kname, wl),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": bytes_per_launch, "kernel": kdesc,
                     "launches_timed": nlaunch, "avg_launch_us": avg_us,
                     "timing": "per site, a HIP graph of that site's launch in every layer, replayed between "
                               "HIP events on the launch stream; launch-to-launch duration",
                     "per_site": head["per_site"]},
        "stack": head,
    }
    log(f"stack: {head['ms_per_step']} ms/step, {head['gbs']} GB/s, {avg_us} us per weight launch")
    del st
    torch.cuda.empty_cache()
    if not args.no_extra:
        log("timing the streaming-read ceiling (pg_hbm_read)")
        res["hbm_read"] = run_hbm_read()
        if args.workload == "qwen36" and args.batch == 1:
            log("timing the Llama-3.1-8B-shaped stack at batch 1 and 4")
            ll = {}
            base = build_stack("llama32", 1, "fused", False)
            for b in (1, 4):
                s2 = base if b == 1 else base.with_batch(b)
                if b > 1:
                    s2.fused, s2.split_above = True, 4096       # the batched (hybrid) path
                ms2, _, _ = run_stack(s2, max(5, args.steps // 2), args.warmup)
                per2, _ = time_launches(s2, stream, reps=5)
                ll[f"b{b}"] = {"path": "fused" if b == 1 else "hybrid", **stack_result(s2, ms2, b, per2)}
                log(f"llama32 b{b}: {ll[f'b{b}']['ms_per_step']} ms/step")
                del s2
            del base
            torch.cuda.empty_cache()
            res["llama32"] = ll
            log("timing the stack through codebook tables (pg_rot_qgemv_table)")
            res["table"] = run_table_stacks(max(5, args.steps // 2), args.warmup)
            log("timing the 512 x 2048 layer warm and cold")
            res["single_layer"] = run_single_layer()
            log("timing each Qwen3-4B matrix cold")
            res["layer_cold"] = run_layer_cold()
            torch.cuda.empty_cache()
    if not args.no_qgemm:
        log("timing the prompt path (pg_qgemm)")
        res["qgemm"] = run_qgemm()
    if not args.no_encode:
        log("timing the GPU encoder (pg_encode)")
        res["encode"] = run_encode()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline()
        if not args.no_extra:
            res["cpu_all_cores"] = cpu_baseline(seconds=10.0, cores=host_cores())
            res["cpu_qgemm"] = cpu_qgemm()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
