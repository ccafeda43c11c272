"""Throughput of the libfattn hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * bf16 forward, non-causal, B=2 H=16 N=8192 d=128   (fattn_fwd)
  * bf16 forward, causal,     B=8 H=16 N=2048 d=128   (fattn_fwd; causal tile skipping)
  * bf16 backward, causal,   B=4 H=16 N=4096 d=128   (fattn_bwd)
  * fp8 forward with Hadamard rotation, non-causal, B=4 H=16 N=4096 d=128
    (fattn_fwd_fp8)
value = algorithmic FLOP of the step / time of the step, in TFLOP/s
(forward 4·B·H·N²·d, backward 2.5× that, halved under causal).

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16 = 2500.0      # TFLOP/s, MI355X dense bf16 MFMA
PEAK_FP8 = 5000.0       # TFLOP/s, MI355X dense fp8 MFMA

PARTS = ["fwd", "fwd_causal", "bwd", "fp8"]
PART_WORKLOAD = {"fwd": 3, "fwd_causal": 2, "bwd": 4, "fp8": 5}
KERNEL_SOURCES = {
    "fwd": ["fwd_bf16.hip", "fattn_device.hpp", "fattn_launch.h"],
    "fwd_causal": ["fwd_bf16.hip", "fattn_device.hpp", "fattn_launch.h"],
    "bwd": ["bwd_bf16.hip", "fattn_device.hpp", "fattn_launch.h"],
    "fp8": ["fwd_fp8.hip", "fattn_device.hpp", "fattn_launch.h"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--parts", default=",".join(PARTS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--no-exp-variants", action="store_true",
                    help="skip the separate hw/poly/split exp2 timing of the forward")
    ap.add_argument("--exp-mode", default="auto", choices=["auto", "hw", "poly", "split"],
                    help="exp2 variant of the timed forward and fp8 calls (default: auto)")
    ap.add_argument("--fp8-error-rows", type=int, default=64,
                    help="rows per head of the fp8 output compared with the oracle, with and "
                         "without the rotation, in the cpu_baseline leg (0: skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the sequence-length / head-dimension sweep: N = 4096 to "
                         "32768 at a fixed B*H*N = 262144 tokens, d = 64 and 128")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a device-to-device copy of this many bytes "
                         "(calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def copy_calibration(nbytes, reps):
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch_read": n * 4, "write": n * 4, "launches": reps}))


def source_hash(part):
    """Hash of the kernel sources of a bench part and of the compile flags,
    ignoring comments and blank lines (a comment edit does not change the
    compiled kernels, a code-generation flag can)."""
    import re
    from tiled_attention_fattn_amd.build import FLAGS
    h = hashlib.sha256()
    h.update(" ".join(f for f in FLAGS if not f.startswith("/")).encode())
    for f in KERNEL_SOURCES[part]:
        with open(os.path.join(HERE, "tiled_attention_fattn_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def committed_traffic(part):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the
    kernel source has not changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(part)
    if not rec or rec.get("source_hash") != source_hash(part):
        return None
    return rec.get("bytes_per_launch")


def part_peak(part):
    return PEAK_FP8 if part == "fp8" else PEAK_BF16


def part_flops(part):
    from tiled_attention_fattn_amd.inputs import WORKLOADS, flops_bwd, flops_fwd
    w = WORKLOADS[PART_WORKLOAD[part]]
    args = (w["B"], w["H"], w["N"], w["d"], w["causal"])
    return flops_bwd(*args) if part == "bwd" else flops_fwd(*args)


def setup_part(part, torch, fa, exp_mode="auto"):
    """Resident inputs/outputs for one part; returns a launch closure."""
    from tiled_attention_fattn_amd.inputs import WORKLOADS, gen_workload, to_device_bf16
    k = PART_WORKLOAD[part]
    w = WORKLOADS[k]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    names = ("q", "k", "v", "do") if part == "bwd" else ("q", "k", "v")
    inp = gen_workload(k, names=names)
    t = {n: to_device_bf16(inp[n][1]) for n in names}
    del inp
    scale = d ** -0.5
    if w["kind"] == "fwd":
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        return lambda mode=exp_mode: fa.fwd(t["q"], t["k"], t["v"], causal=w["causal"],
                                            scale=scale, exp_mode=mode, out=o, lse=lse)
    if part == "bwd":
        o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=w["causal"], scale=scale)
        grads = tuple(torch.empty_like(t["q"]) for _ in range(3))
        ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        return lambda: fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w["causal"],
                              scale=scale, workspace=ws, out=grads)
    o = torch.empty_like(t["q"])
    o2 = torch.empty_like(t["q"])
    ws = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")

    def run(mode="full", em=exp_mode):
        if mode == "attend":  # the attention step alone on the operands of the last full call
            return fa.fwd_fp8_attend(t["q"], ws, causal=w["causal"], scale=scale,
                                     rotate=w["rotate"], seed=k, want_lse=False, out=o2,
                                     exp_mode=em)
        if mode == "outputs":  # O with and without the rotation (outside the timed region)
            outs = {}
            for rot in (True, False):
                outs[rot] = fa.fwd_fp8(t["q"], t["k"], t["v"], causal=w["causal"], scale=scale,
                                       rotate=rot, seed=k, want_lse=False, workspace=ws,
                                       exp_mode=em)[0]
            return outs
        return fa.fwd_fp8(t["q"], t["k"], t["v"], causal=w["causal"], scale=scale,
                          rotate=w["rotate"], seed=k, want_lse=False, workspace=ws, out=o,
                          exp_mode=em)
    return run


def fp8_error_sample(run, rows_per_head):
    """Sampled rows of the fp8 output with and without the rotation, copied to
    the host for the oracle leg: (rows, {rotate: float64 [B, H, rows, d]})."""
    import torch
    w = WORKLOADS_CACHE()[PART_WORKLOAD["fp8"]]
    outs = run("outputs")
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    N = w["N"]
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, rows_per_head, replace=False)]))
    idx = torch.as_tensor(rows, device=outs[True].device)
    got = {rot: o[:, :, idx].float().cpu().numpy().astype(np.float64) for rot, o in outs.items()}
    return rows, got


def WORKLOADS_CACHE():
    from tiled_attention_fattn_amd.inputs import WORKLOADS
    return WORKLOADS


def fp8_error_vs_oracle(rows, got):
    """Relative RMS of the fp8 output against the float64 oracle's exact
    attention on the unrotated bf16 inputs, on the sampled rows of every head,
    with and without the rotation (the checker's side: oracle code only)."""
    from oracle.attention import attention_forward_rows
    from tiled_attention_fattn_amd.inputs import gen_workload
    k = PART_WORKLOAD["fp8"]
    w = WORKLOADS_CACHE()[k]
    x = gen_workload(k, names=("q", "k", "v"))
    scale = w["d"] ** -0.5
    ref = np.empty_like(got[True])
    for b in range(w["B"]):
        for h in range(w["H"]):
            ref[b, h] = attention_forward_rows(x["q"][0], x["k"][0], x["v"][0], w["causal"],
                                               scale, b, h, rows)[0]
    den = np.linalg.norm(ref)
    err = {rot: float(np.linalg.norm(g - ref) / den) for rot, g in got.items()}
    return {"rel_rms_rotate": round(err[True], 5), "rel_rms_no_rotate": round(err[False], 5),
            "ratio_no_rotate_over_rotate": round(err[False] / err[True], 3), "bound": 6e-2,
            "sample": f"{len(rows)} rows of each of the {w['B'] * w['H']} heads of "
                      f"{w['name']}, against float64 exact attention (oracle)"}


def cpu_baseline(parts, heads):
    """The float64 oracle on a bounded sample (`heads` heads of each part's workload)."""
    from oracle.attention import attention_backward, attention_forward
    from oracle.fp8_model import fp8_attention_model
    from tiled_attention_fattn_amd.inputs import WORKLOADS, flops_bwd, flops_fwd, gen_workload
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    flop = 0.0
    secs = 0.0
    for part in parts:
        k = PART_WORKLOAD[part]
        w = WORKLOADS[k]
        shape = (1, heads, w["N"], w["d"])
        names = ("q", "k", "v", "do") if part == "bwd" else ("q", "k", "v")
        x = gen_workload(k, names=names, shape=shape)
        scale = w["d"] ** -0.5
        t0 = time.perf_counter()
        if w["kind"] == "fwd":
            attention_forward(x["q"][0], x["k"][0], x["v"][0], w["causal"], scale)
        elif part == "bwd":
            attention_backward(x["q"][0], x["k"][0], x["v"][0], x["do"][0], w["causal"], scale)
        else:
            fp8_attention_model(x["q"][0], x["k"][0], x["v"][0], w["causal"], scale,
                                rotate=True, seed=k)
        secs += time.perf_counter() - t0
        f = (flops_bwd if part == "bwd" else flops_fwd)(1, heads, w["N"], w["d"], w["causal"])
        flop += f
    return {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} head(s) of each part's workload ({', '.join(parts)}), "
                      f"float64 numpy, {secs:.1f} s"}


SWEEP_TOKENS = 262144   # B·H·N per point (that of the B=2 H=16 N=8192 forward)
SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)


def sweep(args):
    """Throughput over sequence length and head dimension at a fixed token count.

    For each N and d, B·H = 262144 / N heads (B = 1) of seeded N(0,1) inputs
    rounded to bf16; forward non-causal and causal, backward causal, and the
    fp8 attention step (non-causal, on operands quantised with the rotation).
    Prints one JSON line with every point.
    """
    import torch
    import tiled_attention_fattn_amd as fa
    from tiled_attention_fattn_amd.inputs import flops_bwd, flops_fwd
    torch.cuda.set_device(0)
    reps, warm = 10, 3
    points = []

    def timed(fn):
        # Median of per-call event timings: one slow call (a rare stall of the
        # box) must not move a point the way it moves a mean.
        for _ in range(warm):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    # Bring the shader clock up before the first point (a few calls are not
    # enough for the first configuration measured).
    g = torch.Generator(device="cuda").manual_seed(999)
    x = torch.randn(1, 64, 4096, 128, device="cuda", generator=g).to(torch.bfloat16)
    for _ in range(300):
        fa.fwd(x, x, x)
    torch.cuda.synchronize()
    del x

    for d in (128, 64):
        for N in SWEEP_N:
            H = SWEEP_TOKENS // N
            g = torch.Generator(device="cuda").manual_seed(1000 + N + d)
            q, k, v, do = (torch.randn(1, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
                           for _ in range(4))
            scale = d ** -0.5
            o = torch.empty_like(q)
            lse = torch.empty((1, H, N), dtype=torch.float32, device="cuda")
            for causal in (False, True):
                ms = timed(lambda: fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse))
                tf = flops_fwd(1, H, N, d, causal) / (ms * 1e-3) / 1e12
                points.append({"part": "fwd", "causal": causal, "B": 1, "H": H, "N": N, "d": d,
                               "ms": round(ms, 4), "tflops": round(tf, 1),
                               "frac_of_peak": round(tf / PEAK_BF16, 4)})
            # The backward consumes the causal forward's O and LSE (left in o, lse).
            grads = tuple(torch.empty_like(q) for _ in range(3))
            ws = torch.empty(fa.bwd_workspace_bytes(1, H, N, d), dtype=torch.uint8, device="cuda")
            ms = timed(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale,
                                      workspace=ws, out=grads))
            tf = flops_bwd(1, H, N, d, True) / (ms * 1e-3) / 1e12
            points.append({"part": "bwd", "causal": True, "B": 1, "H": H, "N": N, "d": d,
                           "ms": round(ms, 4), "tflops": round(tf, 1),
                           "frac_of_peak": round(tf / PEAK_BF16, 4)})
            del grads, ws
            ws8 = torch.empty(fa.fp8_workspace_bytes(1, H, N, d), dtype=torch.uint8, device="cuda")
            fa.fwd_fp8(q, k, v, scale=scale, rotate=True, seed=N, want_lse=False, workspace=ws8,
                       out=o)
            ms = timed(lambda: fa.fwd_fp8_attend(q, ws8, scale=scale, rotate=True, seed=N,
                                                 want_lse=False, out=o))
            tf = flops_fwd(1, H, N, d, False) / (ms * 1e-3) / 1e12
            points.append({"part": "fp8_attend", "causal": False, "B": 1, "H": H, "N": N, "d": d,
                           "ms": round(ms, 4), "tflops": round(tf, 1),
                           "frac_of_peak": round(tf / PEAK_FP8, 4)})
            print(f"[sweep] d={d} N={N} done", file=sys.stderr, flush=True)
            del q, k, v, do, o, lse, ws8
    # Packed variable-length sequences: B = 1, H = 8, N = 32768 rows split into
    # segments of seeded lengths uniform in [1, 8192] (the last one cut to fit).
    rng = np.random.default_rng(2024)
    lengths = []
    while sum(lengths) < 32768:
        lengths.append(int(min(rng.integers(1, 8193), 32768 - sum(lengths))))
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device="cuda")
    H, N, d = 8, 32768, 128
    g = torch.Generator(device="cuda").manual_seed(77)
    q, k, v, do = (torch.randn(1, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((1, H, N), dtype=torch.float32, device="cuda")
    maxl = max(lengths)
    scale = d ** -0.5
    for causal in (False, True):
        ms = timed(lambda: fa.fwd_varlen(q, k, v, cu, maxl, causal=causal, scale=scale, out=o,
                                         lse=lse))
        fl = sum(flops_fwd(1, H, n, d, causal) for n in lengths)
        points.append({"part": "fwd_varlen", "causal": causal, "B": 1, "H": H, "N": N, "d": d,
                       "segments": len(lengths), "max_seqlen": maxl, "ms": round(ms, 4),
                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                       "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16, 4)})
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(1, H, N, d), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: fa.bwd_varlen(q, k, v, o, lse, do, cu, maxl, causal=True, scale=scale,
                                     workspace=ws, out=grads))
    fl = sum(flops_bwd(1, H, n, d, True) for n in lengths)
    points.append({"part": "bwd_varlen", "causal": True, "B": 1, "H": H, "N": N, "d": d,
                   "segments": len(lengths), "max_seqlen": maxl, "ms": round(ms, 4),
                   "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                   "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16, 4)})
    del grads, ws
    # The fp8 forward over the same packing (whole call: per-segment K/V
    # quantisation, then attention).
    ws8 = torch.empty(fa.fp8_varlen_workspace_bytes(1, H, N, d, len(lengths), maxl),
                      dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        ms = timed(lambda: fa.fwd_fp8_varlen(q, k, v, cu, maxl, causal=causal, scale=scale,
                                             rotate=True, seed=5, want_lse=False, workspace=ws8,
                                             out=o))
        fl = sum(flops_fwd(1, H, n, d, causal) for n in lengths)
        points.append({"part": "fp8_varlen", "causal": causal, "B": 1, "H": H, "N": N, "d": d,
                       "segments": len(lengths), "max_seqlen": maxl, "ms": round(ms, 4),
                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                       "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP8, 4)})
    del ws8
    print(f"[sweep] varlen done ({len(lengths)} segments, max {maxl})", file=sys.stderr,
          flush=True)

    # Block masks over 128x128 blocks: B = 2, H = 16, N = 8192, d = 128, seeded
    # random masks with the diagonal block always visible, at several densities.
    B, H, N, d = 2, 16, 8192, 128
    g = torch.Generator(device="cuda").manual_seed(78)
    q, k, v, do = (torch.randn(B, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    ws8 = torch.empty(fa.fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    nb = N // 128
    scale = d ** -0.5
    for dens in (1.0, 0.5, 0.25, 0.1):
        m = (np.random.default_rng(3).random((nb, nb)) < dens).astype(np.uint8)
        m[np.arange(nb), np.arange(nb)] = 1
        mt = torch.as_tensor(m, device="cuda")
        vis = float(m.sum()) * 128 * 128 * B * H  # visible (query, key) pairs
        ms_f = timed(lambda: fa.fwd_blocksparse(q, k, v, mt, scale=scale, out=o, lse=lse))
        ms_b = timed(lambda: fa.bwd_blocksparse(q, k, v, o, lse, do, mt, scale=scale,
                                                workspace=ws, out=grads))
        # fp8 whole call (quantisation over all keys, attention over the
        # visible blocks).
        ms_8 = timed(lambda: fa.fwd_fp8_blocksparse(q, k, v, mt, scale=scale, rotate=True, seed=5,
                                                    want_lse=False, workspace=ws8, out=o))
        for part, ms, fl, peak in (("fwd_blocksparse", ms_f, 4 * d * vis, PEAK_BF16),
                                   ("bwd_blocksparse", ms_b, 10 * d * vis, PEAK_BF16),
                                   ("fp8_blocksparse", ms_8, 4 * d * vis, PEAK_FP8)):
            tf = fl / (ms * 1e-3) / 1e12
            points.append({"part": part, "causal": False, "B": B, "H": H, "N": N, "d": d,
                           "density": round(float(m.mean()), 4), "ms": round(ms, 4),
                           "tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4)})
    print("[sweep] block masks done", file=sys.stderr, flush=True)

    print(json.dumps({"sweep": "tokens per point B*H*N = %d, B = 1" % SWEEP_TOKENS,
                      "data": "synthetic: seeded N(0,1) rounded to bf16", "reps": reps,
                      "warmup": warm, "points": points}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, max(1, args.steps))
        return
    if args.sweep:
        sweep(args)
        return
    import torch
    import tiled_attention_fattn_amd as fa

    parts = [p for p in args.parts.split(",") if p]
    torch.cuda.set_device(0)
    clocks_before = gpu_clocks()
    launch = {p: setup_part(p, torch, fa, args.exp_mode) for p in parts}
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for p in parts:
            launch[p]()
    torch.cuda.synchronize()

    ev = {p: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for p in parts}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        for p in parts:
            ev[p][i][0].record()
            launch[p]()
            ev[p][i][1].record()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    samples = {p: [a.elapsed_time(b) for a, b in ev[p]] for p in parts}
    part_ms = {p: float(np.mean(samples[p])) for p in parts}
    flops = {p: part_flops(p) for p in parts}
    step_flop = sum(flops.values())
    value = step_flop / (ms_per_step * 1e-3) / 1e12

    info = {}
    for p in parts:
        tf = flops[p] / (part_ms[p] * 1e-3) / 1e12
        peak = part_peak(p)
        info[p] = {"workload": fa_workload_name(p), "ms": round(part_ms[p], 4),
                   "ms_median": round(float(np.median(samples[p])), 4),
                   "ms_min": round(float(np.min(samples[p])), 4),
                   "tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4)}

    # The C3 forward is also reported with each exp2 variant. The variants are
    # timed in interleaved rounds (order reversed every other round) so that
    # clock drift over the run does not favour whichever variant runs last.
    if "fwd" in parts and not args.no_exp_variants:
        modes = ("hw", "poly", "split")
        for mode in modes:
            for _ in range(2):
                launch["fwd"](mode)
        times = {m: [] for m in modes}
        for r in range(6):
            for mode in (modes if r % 2 == 0 else modes[::-1]):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(4):
                    launch["fwd"](mode)
                b.record()
                torch.cuda.synchronize()
                times[mode].append(a.elapsed_time(b) / 4)
        info["fwd"]["tflops_by_exp2"] = {
            m: round(flops["fwd"] / (float(np.median(t)) * 1e-3) / 1e12, 1) for m, t in times.items()}

    # The roofline is reported for the step's longest single kernel: the C3
    # forward is one launch of one kernel (the bwd and fp8 parts are several
    # launches each, and their longest kernels are shorter in the rocprofv3
    # kernel statistics kept under profiles/), so its event timing is that
    # kernel's duration.
    dom = "fwd" if "fwd" in parts else max(parts, key=lambda p: part_ms[p])
    dom_peak = PEAK_FP8 if dom == "fp8" else PEAK_BF16
    achieved = flops[dom] / (part_ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": dom_peak, "unit": "TFLOP/s", "frac": round(achieved / dom_peak, 4),
                "traffic": committed_traffic(dom)}

    # The fp8 attention step alone (after the quantisation the timed calls did),
    # with the default exp2 and, in interleaved rounds, with each variant.
    if "fp8" in parts:
        for _ in range(3):
            launch["fp8"]("attend")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            launch["fp8"]("attend")
        b.record()
        torch.cuda.synchronize()
        ams = a.elapsed_time(b) / 20
        atf = flops["fp8"] / (ams * 1e-3) / 1e12
        info["fp8"]["attention_only"] = {"ms": round(ams, 4), "tflops": round(atf, 1),
                                         "frac_of_peak": round(atf / PEAK_FP8, 4)}
        if not args.no_exp_variants:
            modes = ("hw", "poly", "split")
            times = {m: [] for m in modes}
            for r in range(6):
                for mode in (modes if r % 2 == 0 else modes[::-1]):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for _ in range(4):
                        launch["fp8"]("attend", mode)
                    b.record()
                    torch.cuda.synchronize()
                    times[mode].append(a.elapsed_time(b) / 4)
            info["fp8"]["attention_only"]["tflops_by_exp2"] = {
                m: round(flops["fp8"] / (float(np.median(t)) * 1e-3) / 1e12, 1)
                for m, t in times.items()}
    clocks = gpu_clocks()
    if clocks_before or clocks:
        info["gpu_clock_mhz"] = {"before": clocks_before, "after": clocks}

    # GPU outputs for the fp8 error check (after all timing).
    fp8_sample = None
    if "fp8" in parts and not args.no_cpu_baseline and args.fp8_error_rows > 0:
        fp8_sample = fp8_error_sample(launch["fp8"], args.fp8_error_rows)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(parts, args.cpu_heads)
        if fp8_sample is not None:
            # The checker's leg: the oracle's exact attention on the sampled rows.
            info["fp8"]["error_vs_oracle"] = fp8_error_vs_oracle(*fp8_sample)

    dtype = "bf16" if "fp8" not in parts else ("fp8" if parts == ["fp8"] else "bf16+fp8")
    line = {
        "metric": "attention TFLOP/s (bf16 fwd, bwd; fp8 fwd) and % of MI355X MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic: seeded N(0,1) rounded to bf16 (fp8 part: 0.1% x20 outliers in Q, K)",
        "config": {"workload": "+".join(fa_workload_name(p) for p in parts),
                   "step_tflop": round(step_flop / 1e12, 4), "parallelism": "single GPU"},
        "parts": info, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gpu_clocks():
    """Current shader clock (MHz) of GPU 0, or None.

    Read in-process from the amdgpu driver's sysfs DPM table of that device
    (the line marked '*' of pp_dpm_sclk under its PCI address): nothing is
    spawned from this process once it has touched the GPU."""
    import re
    import torch
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        with open(f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk") as fh:
            text = fh.read()
    except Exception:  # noqa: BLE001 (no sysfs entry: report nothing)
        return None
    m = re.search(r"(\d+)\s*Mhz\s*\*", text, re.IGNORECASE)
    return int(m.group(1)) if m else None


def fa_workload_name(p):
    from tiled_attention_fattn_amd.inputs import WORKLOADS
    return WORKLOADS[PART_WORKLOAD[p]]["name"]


if __name__ == "__main__":
    main()
