"""Benchmark of the Pingala-8 hot path on one MI355X.

Default workload: the 36-layer Qwen3-4B-shaped linear stack at batch 1
(uniform random trellis bitstreams, fp16 U(0.005, 0.05) scales, fp16 N(0,1)
input fed layer to layer; 965,099,520 coded bytes per token).  One step is
one token through the whole stack: per layer four launches of the fused
stage kernel (RMS normalisation + activation rotation + qgemv; qkv and
gate/up merged), replayed from a HIP graph.  Inputs are resident in HBM before timing starts.

Printed: one JSON line with the whole-job compressed-weight GB/s
(bytes per token x tokens per second), tokens per second, the roofline of
the stage kernel (coded bytes per launch over its average duration, from
the HIP events around the timed region), the prompt path's matrix-core
fraction (pg_qgemm on the Qwen3-4B layer shapes at m = 512 and 4096), the
GPU encoder's throughput on one Qwen3-4B-shaped layer, and the oracle's CPU
throughput on a bounded sample of the stack workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "qgemv compressed-weight GB/s (% HBM peak) + linear-stack tok/s at batch 1"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0          # dense bf16


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


def cpu_baseline(seconds: float = 12.0):
    """The oracle (numpy fp64 decode + product), as it stands, on a bounded
    sample of the stack: layer-0 launch groups of the Qwen3-4B-shaped stack,
    repeated until `seconds` have passed.  numpy runs these ops on one
    thread."""
    import numpy as np

    from oracle import p8f
    from qgemv_amd import synth

    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    x = {s: synth.activations_f32(1, merged[s][0].shape[1] * 4) for s in merged}
    done_bytes, t0, mats = 0, time.perf_counter(), 0
    while True:
        for site in ("o", "qkv", "down", "gu"):
            codes, scales = merged[site]
            p8f.gemv_ref(codes, scales, x[site])
            done_bytes += codes.nbytes + scales.nbytes
            mats += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{mats} launch-group products of layer 0 (decode + fp64 GEMV, batch 1) in {dt:.1f} s; "
                      f"{done_bytes} coded bytes"}


def run_stack(args):
    import torch

    import qgemv_amd as q
    from qgemv_amd import synth
    from qgemv_amd.stack import ORDER, Stack

    shapes = synth.qwen3_4b_shapes() if args.workload == "qwen36" else synth.llama31_8b_shapes()
    layers = 36 if args.workload == "qwen36" else 32
    # auto: the v_dot4 fused stage at batch 1; from batch 2 on the matrix
    # cores, whose cost hardly grows with the batch: the fused stage where
    # the batch's rotated activations fit in LDS (k <= 4096), the rotation +
    # product elsewhere (hybrid)
    path = args.path if args.path != "auto" else ("fused" if args.batch <= 1 or args.carry else "hybrid")
    fused = path in ("fused", "hybrid")
    split_above = 4096 if path == "hybrid" else None
    log(f"building {args.workload}: {layers} layers, batch {args.batch}, {path} path")
    st = Stack(shapes, layers, batch=args.batch, x_dtype=q.PG_Q16, fused=fused, carry=args.carry,
               split_above=split_above)
    stream = torch.cuda.current_stream()
    use_graph = not args.no_graph
    if use_graph:
        st.capture()
    step = st.replay if use_graph else st.token
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done (hip graph: {use_graph})")
    # timed region: exactly `steps` tokens (one step = one pass of the batch
    # through every layer), HIP events on the launch stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    log(f"timed {args.steps} steps: {gpu_ms:.2f} ms (events), {wall * 1e3:.2f} ms (wall)")

    n_split = sum(1 for _, k in st.shapes.values() if split_above is not None and k > split_above)
    launches_per_step = (4 + n_split if fused else 8) * layers
    bytes_per_launch = st.bytes_per_token // (4 * layers)
    if fused:
        # every launch of the step is the fused stage kernel: its average
        # duration is the timed region over the launches (gaps included)
        avg_us = 1e3 * gpu_ms / (args.steps * launches_per_step)
        if args.batch <= 1 or args.carry:
            kname = "k_rot_qgemv"
            kdesc = "k_rot_qgemv (pg_rot_qgemv: RMS norm + rotation + qgemv, one launch per stage)"
        else:
            kname = "k_rot_qmma"
            kdesc = ("k_rot_qmma (pg_rot_qgemv at batch 2..8: RMS norm + rotation + int8 matrix-core product) "
                     "where k <= 4096" + ("; k_fwht + k_qgemv_mma above" if n_split else
                                          "; k_rot_qgemv above" if path == "fused" else ""))
        nlaunch = args.steps * launches_per_step
    else:
        # split path: events around every product launch of a separate pass;
        # a spin kernel queued first holds the GPU while the host enqueues, so
        # the events time back-to-back GPU work, not the host's launch rate
        evs = []
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.25))
        for _ in range(2):
            for layer in range(layers):
                for site in ORDER:
                    n, k = st.shapes[site]
                    first = site == "qkv" and layer == 0
                    prev = {"qkv": "down", "o": "qkv", "gu": "o", "down": "gu"}[site]
                    q.pg_fwht_rotate_ex(st.h0 if first else st.out[prev], q.PG_F16 if first else q.PG_F32,
                                        k if first else st.shapes[prev][0], st.xrot, q.PG_Q16, st.signs[layer][site],
                                        args.batch, k, 0 if first else q.PG_FLAG_RMSNORM)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    q.pg_qgemv(st.codes[layer][site], st.scales[layer][site], n, k, st.xrot, q.PG_Q16, args.batch,
                               st.out[site])
                    b.record(stream)
                    evs.append((a, b))
        torch.cuda.synchronize()
        avg_us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        if args.batch == 1:
            kname = "k_qgemv_q16"
            kdesc = "k_qgemv_q16 (pg_qgemv on PG_Q16 activations)"
        else:
            kname = "k_qgemv_mma"
            kdesc = "k_qgemv_mma (pg_qgemv on PG_Q16 activations, int8 matrix cores, batch 2..8)"
        nlaunch = len(evs)
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    wl = ("qwen3-4b-36L" if args.workload == "qwen36" else "llama3.1-8b-32L") + f"-b{args.batch}"
    traffic = committed_traffic(kname, wl)
    tok_s = args.batch * 1e3 / ms_per_step
    value = st.bytes_per_token * (1e3 / ms_per_step) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("i8xi8->i32 (levels x 16-bit activation digits), f16 MFMA rotation, f32 scales" if fused or
                  args.batch == 1 else "i8xi8->i32 MFMA (level planes x 16-bit activation digits), f32 scales"),
        "data": "synthetic",
        "config": {"workload": f"{'Qwen3-4B' if args.workload == 'qwen36' else 'Llama-3.1-8B'}-shaped "
                               f"{layers}-layer linear stack, batch {args.batch}, random trellis bitstreams",
                   "layers": layers, "batch": args.batch, "bytes_per_token": st.bytes_per_token,
                   "tok_per_s": round(tok_s, 2), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "hip_graphs": use_graph, "launches_per_token": launches_per_step, "path": path,
                   "format": "carried-state variant" if args.carry else "P8F v1"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": bytes_per_launch, "kernel": kdesc,
                     "launches": nlaunch, "avg_launch_us": round(avg_us, 3)},
    }
    return res


def run_qgemm(stream_iters: int = 10):
    """Prompt path on the matrix cores: pg_qgemm_ex on the Qwen3-4B layer-0
    launch groups (random codes and scales as in the stack), X = bf16 N(0,1)
    rows rotated once by pg_fwht_rotate (bf16 -> bf16), at m = 512 and 4096,
    with the workspace pg_qgemm_workspace_bytes asks for (allocated before the
    timed calls; shapes whose tiles fill the chip in whole rounds ask for none
    and run unsplit).  Each product is timed alone with HIP events on the launch
    stream over `stream_iters` back-to-back calls, the split sum included;
    the fraction is 2 m n k per second over the 2.5 PFLOP/s dense bf16 peak."""
    import numpy as np
    import torch

    import qgemv_amd as q
    from qgemv_amd import synth

    shapes = synth.qwen3_4b_shapes()
    merged = synth.random_layer_merged(0, shapes)
    site_no = {"qkv": 0, "o": 1, "gu": 2, "down": 3}
    stream = torch.cuda.current_stream()
    out = {"bound": "mfma", "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16 x bf16 -> f32",
           "kernel": "k_qgemm_v2 + k_qgemm_sum (pg_qgemm_ex)", "workload": "Qwen3-4B layer-0 launch groups qkv/o/gu/down, "
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
            for _ in range(2):
                q.pg_qgemm_ex(cd, sc, n, k, xr, m, y, ws, wsb)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(stream_iters):
                q.pg_qgemm_ex(cd, sc, n, k, xr, m, y, ws, wsb)
            e1.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / stream_iters
            flop = 2.0 * m * n * k
            tf = flop / (us * 1e-6) / 1e12
            per[site] = {"n": n, "k": k, "us": round(us, 2), "tflops": round(tf, 1),
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
    operations per weight, the encoder's algorithmic work."""
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
        q.pg_encode_ref(np.ascontiguousarray(w[:rows]), rows, k, sb, hc, hs, 0)
        cpu_s += time.perf_counter() - t0
        cpu_w += rows * k
        if not np.array_equal(c[:rows].cpu().numpy(), hc):
            raise SystemExit(f"pg_encode differs from pg_encode_ref on {name}")
        per[name] = {"n": n, "k": k, "ms": round(ms, 3), "gweights_per_s": round(n * k / ms / 1e6, 2)}
        tot_w += n * k
        tot_ms += ms
    gws = tot_w / tot_ms / 1e6
    tflops = 1408.0 * gws * 1e9 / 1e12
    log(f"encode: {gws:.2f} Gweights/s on the GPU")
    return {"kernel": "k_encode (pg_encode)", "workload": "Qwen3-4B-shaped layer, 7 matrices, "
            f"{int(tot_w)} weights", "ms": round(tot_ms, 3), "gweights_per_s": round(gws, 2),
            "roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": 78.6, "unit": "TFLOP/s (fp64)",
                         "frac": round(tflops / 78.6, 4), "flop_per_weight": 1408},
            "cpu_reference": {"mweights_per_s": round(cpu_w / cpu_s / 1e6, 2), "threads": os.cpu_count(),
                              "kind": "pg_encode_ref (host C++, bit-identical output)",
                              "sample": "64 rows of each matrix"},
            "matrices": per}


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
    ap.add_argument("--no-qgemm", action="store_true", help="skip the prompt-path (pg_qgemm) measurement")
    ap.add_argument("--no-encode", action="store_true", help="skip the GPU encoder (pg_encode) measurement")
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
    res = run_stack(args)
    if not args.no_qgemm:
        log("timing the prompt path (pg_qgemm)")
        res["qgemm"] = run_qgemm()
    if not args.no_encode:
        log("timing the GPU encoder (pg_encode)")
        res["encode"] = run_encode()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
