"""Benchmark of the FFF layer forward pass on one MI355X.

One step = one fff_forward call (routing through every tree, the fused
GELU*v accumulation into the concatenated buffer, the output projection)
over one batch of synthetic tokens already resident in HBM.  The default
workload is the OPT-1.3B-shaped depth-6 layer (T=16384, d=2048, P=32, D=6,
h=128, bf16).  Input sets are rotated between steps so that the 256 MB
Infinity Cache cannot serve a repeated call; a second, shorter pass on one
input set gives the warm figure beside it.

Prints one JSON line: tokens/s from K steps with nothing else on the
stream; the roofline of the dominant kernel, picked by measured time among
the stages the library brackets with HIP events on the stream it launches
on (dense top levels, deep levels, H build, projection), in
a second pass of the same K steps (each event costs about 3 us of GPU time,
so the headline pass carries none), with every stage's roofline beside it;
and the CPU oracle's throughput on the same workload, whose output also
gives the run's routing flips and y error.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FFF layer tokens/sec (bf16, OPT-1.3B d=6 shape) + % of HBM/MFMA roofline"
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="opt1p3b_d6")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--split-level", type=int, default=-1)
    ap.add_argument("--chunk-tokens", type=int, default=0)
    ap.add_argument("--variant", default="fff", choices=["fff", "post"],
                    help="GELU per node (fff) or on the summed tree output (post)")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0 = by footprint)")
    ap.add_argument("--prune", type=float, default=0.0,
                    help="statically prune this fraction of each tree's paths (seeded random "
                         "leaf mask) and run fff_forward_pruned (with --backward: "
                         "fff_backward_pruned)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle budget: three timed runs of about a third of this each")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time fff_backward (gradients of sum(y * dy)) on the workload instead")
    ap.add_argument("--depth-sweep", action="store_true",
                    help="time the layer at depths 0..11 (the headline's T, d, P, h) beside a "
                         "dense FF block of width 4d; one JSON line per depth")
    ap.add_argument("--sweep-depths", default="0-11")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of 256 MiB (3 times), the reference "
                         "for scaling the HBM byte counters")
    return ap.parse_args()


def algorithmic_work(s, U):
    """Flops and bytes the method itself must do (not the work it avoids,
    and not intermediate round trips): per visited node a length-d dot
    product and an h-vector update, the projection, and one read of x, the
    visited node rows, W_out, plus the writes of y and path_out."""
    e = 2 if s.dtype == "bf16" else 4
    flops_route = s.T * s.P * (s.D + 1) * 2 * (s.d + s.h)
    flops_proj = 2 * s.T * s.P * s.h * s.d
    bytes_alg = e * (2 * s.T * s.d + U * (s.d + s.h + 1) + s.P * s.h * s.d) + 4 * s.T * s.P
    return flops_route, flops_proj, bytes_alg


# Sources each dominant kernel's device code is built from (its own file,
# which also holds its launcher, and the device headers it includes):
# counter figures taken on other sources do not describe it.
KERNEL_SOURCES = {
    "proj_direct": ("k_proj.hip", "mfma_tile.hpp", "common.hpp"),
    "decode": ("k_decode.hip", "mfma_tile.hpp", "common.hpp"),
    "subtree": ("k_subtree.hip", "mfma_tile.hpp", "common.hpp"),
    "route_top": ("k_route.hip", "mfma_tile.hpp", "common.hpp"),
    "hbuild": ("k_route.hip", "mfma_tile.hpp", "common.hpp"),
}


def kernel_source_hash(kernel: str):
    """Hash of a kernel's device sources with comments and blank lines
    dropped, so that editing a comment does not retire its counter figures."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_tree_structured_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
        h.update(f.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def calibrate_copy():
    """A plain device-to-device copy of known size: FETCH_SIZE and WRITE_SIZE
    of its dispatches give the factor from counter bytes to real bytes."""
    import torch

    n = 256 << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "dispatches": 3}), flush=True)


def cpu_baseline(inp, budget_s, variant=0, leaf_alive=None):
    """The CPU oracle (plain float64 C, every host thread) on the first n
    tokens of the workload, n chosen so that three runs take about
    `budget_s`; returns the median of the three and the oracle output of the
    last run (for the parity figures)."""
    import numpy as np

    import oracle

    f = inp.as_f64()
    threads = oracle.default_threads()
    T = inp.shape.T

    def run(n, **kw):
        t0 = time.perf_counter()
        r = oracle.forward(f["x"][:n], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                           nthreads=threads, variant=variant, leaf_alive=leaf_alive, **kw)
        return time.perf_counter() - t0, r

    pilot = min(T, max(threads, 256))
    tp, _ = run(pilot)
    n = int(min(T, max(pilot, pilot * (budget_s / 3) / max(tp, 1e-6))))
    times = [run(n)[0] for _ in range(3)]
    dt = float(np.median(times))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    _, ref = run(n, want_records=True)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the same workload (seed 0), full forward "
                      f"(routing + projection) in float64, median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in times)} s) on {cpu}",
            "seconds": dt, "tokens": n}, ref


def parity_figures(inp, ref, n, path_dev, y_dev, variant=0, leaf_alive=None):
    """Routing flips and y error of the device output on the oracle's tokens
    (flipped tokens checked along the device's own paths)."""
    import numpy as np

    import oracle
    from oracle.compare import check_path_signs, classify_paths, node_alive_from_leaves, y_error

    s = inp.shape
    cls = classify_paths(path_dev[:n], ref, s.D)
    err = y_error(y_dev[:n], ref["y"], cls["tokens_ok"])
    flipped = np.flatnonzero(~cls["tokens_ok"])
    out = {"tokens_checked": int(n), "flips_near_tie": int(cls["flips_near_tie"]),
           "mismatches_beyond_tie": len(cls["bad"]), "tokens_excluded": 0,
           "tokens_flipped": int(len(flipped)), "y_err": err["err"],
           "y_err_unfloored": err["err_unfloored"], "y_err_normwise": err["normwise"]}
    if len(flipped):
        f = inp.as_f64()
        fr = oracle.forward(f["x"][flipped], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                            forced=np.ascontiguousarray(path_dev[flipped], dtype=np.int32),
                            want_records=True, variant=variant)
        alive = node_alive_from_leaves(leaf_alive, s.D) if leaf_alive is not None else None
        out["flipped_paths_valid"] = not check_path_signs(path_dev[flipped], fr, s.D, alive)
        out["y_err_flipped"] = y_error(y_dev[flipped], fr["y"])["err"]
    return out


def _events_ms(torch, fn, steps, warmup):
    """Median milliseconds of fn(i) over `steps` calls, each bracketed by
    events on the current stream, after at least `warmup` calls and 0.3 s of
    warm-up work (the clocks ramp up after the idle input generation)."""
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < 0.3:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def event_floor_us(torch, steps=200):
    """Median interval between two events on the current stream around the
    smallest kernel (a one-element add): the floor under any per-launch time
    taken this way, whatever the kernel does."""
    x = torch.zeros(1, device="cuda:0")
    return 1e3 * _events_ms(torch, lambda i: x.add_(1.0), steps, 20)


def depth_sweep(args):
    """Speed against tree depth, the MI355X counterpart of the paper page's
    Figure 5 and Table 5: the headline workload's T, d, P and h at depths
    D = 0..11 (AUTO plan), beside a dense FF block (x W1^T + b1, tanh GELU,
    then W2) of width 4d, which the pages do not state.  Depth 0 is itself a
    dense layer of P units.  Inputs: x and W_out from the headline generator
    (seed 0), W_node, b_node, V_node drawn per depth (seed 100 + depth); between
    timed calls the sets rotate through copies with tokens and trees
    permuted, so the 256 MB Infinity Cache cannot serve a repeated call."""
    import numpy as np
    import torch

    import sparse_tree_structured_amd as fff
    import workloads

    dev = torch.device("cuda:0")
    base, opts = workloads.WORKLOADS["opt1p3b_d6"]
    T, d, P, h = base.T, base.d, base.P, base.h
    lo, _, hi = args.sweep_depths.partition("-")
    depths = range(int(lo), int(hi or lo) + 1)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    gen0 = workloads.make_inputs(dataclasses_replace(base, D=0), seed=0, **opts)
    x0, wo0 = bf16(gen0.x), bf16(gen0.W_out)
    g = torch.Generator(device="cpu")
    g.manual_seed(1234)
    steps, warmup = args.steps, args.warmup

    # Dense comparator: d_ff = 4d, bf16 weights N(0, 1/fan_in), torch's
    # matrix products (hipBLASLt) and tanh GELU.
    dff = 4 * d
    w1 = (torch.randn(dff, d, generator=g) / d ** 0.5).to(torch.bfloat16).to(dev)
    b1 = (0.1 * torch.randn(dff, generator=g)).to(torch.bfloat16).to(dev)
    w2 = (torch.randn(d, dff, generator=g) / dff ** 0.5).to(torch.bfloat16).to(dev)
    xs = [x0] + [x0[torch.randperm(T, generator=g).to(dev)].contiguous() for _ in range(3)]

    def dense(i):
        hid = torch.nn.functional.gelu(torch.nn.functional.linear(xs[i % len(xs)], w1, b1),
                                       approximate="tanh")
        return torch.nn.functional.linear(hid, w2)

    t_dense = _events_ms(torch, dense, steps, warmup)
    dense_flops = 4 * T * d * dff
    print(json.dumps({"sweep": "dense_ff", "d_ff": dff, "T": T, "d": d, "ms": t_dense,
                      "tokens_per_s": T / (t_dense * 1e-3),
                      "tflops": dense_flops / (t_dense * 1e-3) / 1e12,
                      "impl": "torch linear (hipBLASLt) + tanh GELU, bf16"}), flush=True)
    # The same block with this library's matrix-core product (fff_project_ws,
    # y = H . W with W row-major [K, N], the kernel of the layer's own
    # projection) for both products; bias and GELU in torch between them.
    w1t, w2t = w1.t().contiguous(), w2.t().contiguous()
    hid = torch.empty((T, dff), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    pws = max(fff.project_workspace_size(fff.make_shape(T, dff, 1, 0, d, fff.DTYPE_BF16)),
              fff.project_workspace_size(fff.make_shape(T, d, 1, 0, dff, fff.DTYPE_BF16)))
    pws = torch.empty(pws, dtype=torch.uint8, device=dev) if pws else None

    def dense_ours(i):
        fff.project(xs[i % len(xs)], w1t, y=hid, workspace=pws)
        h2 = torch.nn.functional.gelu(hid + b1, approximate="tanh")
        fff.project(h2, w2t, y=yd, workspace=pws)

    t_ours = _events_ms(torch, dense_ours, steps, warmup)
    print(json.dumps({"sweep": "dense_ff_ours", "d_ff": dff, "T": T, "d": d, "ms": t_ours,
                      "tokens_per_s": T / (t_ours * 1e-3),
                      "tflops": dense_flops / (t_ours * 1e-3) / 1e12,
                      "impl": "fff_project_ws (matrix-core) x2 + torch bias and tanh GELU, bf16"}),
          flush=True)
    del xs, hid, yd, w1t, w2t, pws

    for D in depths:
        shape = dataclasses_replace(base, D=D)
        gen = workloads.make_inputs(dataclasses_replace(shape, T=1), seed=100 + D, **opts)
        W, b, V = bf16(gen.W_node), bf16(gen.b_node), bf16(gen.V_node)
        footprint = (T * d + P * shape.N * (d + h + 1) + P * h * d) * 2
        rotate = int(min(8, max(2, -(-600_000_000 // footprint))))
        sets = [(x0, W, b, V, wo0)]
        for _ in range(rotate - 1):
            tp = torch.randperm(P, generator=g).to(dev)
            rows = (tp[:, None] * h + torch.arange(h, device=dev)[None, :]).reshape(-1)
            sets.append((x0[torch.randperm(T, generator=g).to(dev)].contiguous(),
                         W[tp].contiguous(), b[tp].contiguous(), V[tp].contiguous(),
                         wo0[rows].contiguous()))
        fshape = fff.shape_of(x0, W, V)
        plan = fff.resolve_plan(fshape, fff.make_plan("auto"))
        ws, _ = fff.alloc_workspace(fshape, plan, dev)
        y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)

        def step(i):
            xx, WW, bb, VV, oo = sets[i % rotate]
            fff.forward(xx, WW, bb, VV, oo, workspace=ws, y=y, want_path=False)

        t = _events_ms(torch, step, steps, warmup)
        f_route, f_proj, _ = algorithmic_work(shape, 0)
        # Levels evaluated as one dense product: 2^L columns per tree.
        L = min(plan.split_level, D + 1)
        dense_route = 2 * T * P * (1 << L) * d
        print(json.dumps({
            "sweep": "fff", "D": D, "T": T, "d": d, "P": P, "h": h, "ms": t,
            "tokens_per_s": T / (t * 1e-3), "algo": fff.algo_name(plan.algo),
            "split_level": plan.split_level, "rotated_sets": rotate,
            "alg_gflop": (f_route + f_proj) / 1e9,
            "dense_levels": L, "dense_route_gflop": dense_route / 1e9,
            "speedup_vs_dense": t_dense / t,
            "alg_flops_vs_dense": (f_route + f_proj) / dense_flops}), flush=True)
        del sets, ws, W, b, V
        torch.cuda.empty_cache()


def backward_bench(args):
    """fff_backward on the workload: one step is the whole backward pass
    (routing again, dH, the masked products for dx, dW, dW_out, dV) for one
    batch, inputs and dy resident in HBM, input sets rotated."""
    import numpy as np
    import torch

    import sparse_tree_structured_amd as fff
    import workloads

    dev = torch.device("cuda:0")
    shape, opts = workloads.WORKLOADS[args.workload]
    footprint = (shape.T * shape.d * 2 + shape.P * shape.N * (shape.d + shape.h + 1)
                 + shape.P * shape.h * shape.d) * 2
    rotate = args.rotate or int(min(8, max(2, -(-600_000_000 // footprint))))

    def upload(inp, seed):
        out = [torch.from_numpy(getattr(inp, k).view(np.int16)).view(torch.bfloat16).to(dev)
               for k in ("x", "W_node", "b_node", "V_node", "W_out")]
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        out.append((torch.randn(shape.T, shape.d, generator=g) / shape.d ** 0.5)
                   .to(torch.bfloat16).to(dev))
        return out

    sets = [upload(workloads.make_inputs(shape, seed=s, **opts), s) for s in range(rotate)]
    variant = fff.VARIANTS[args.variant]
    fshape = fff.shape_of(sets[0][0], sets[0][1], sets[0][3], variant)
    plan = fff.make_plan(args.algo)
    prunings = None
    if args.prune > 0:
        # One table per input set, packed for every level dense (the
        # matrix-core backward's routing); each tree keeps at least one path.
        rng = np.random.default_rng(0)
        mask = (rng.random((shape.P, 1 << shape.D)) >= args.prune).astype(np.uint8)
        mask[np.arange(shape.P), rng.integers(0, 1 << shape.D, size=shape.P)] = 1
        prunings = [fff.prune_prepare(mask, st[1], st[3], algo="prefill", split_level=shape.D + 1,
                                      T=shape.T) for st in sets]
        nbytes = fff.backward_pruned_workspace_size(fshape, plan, prunings[0][0])
    else:
        nbytes = fff.backward_workspace_size(fshape, plan)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(sets[0][0]), "dW_node": torch.empty(sets[0][1].shape, **f32),
           "db_node": torch.empty(sets[0][2].shape, **f32),
           "dV_node": torch.empty(sets[0][3].shape, **f32),
           "dW_out": torch.empty(sets[0][4].shape, **f32)}

    def step(i):
        x, W, b, V, Wo, dy = sets[i % rotate]
        if prunings is not None:
            fff.backward_pruned(x, W, b, V, Wo, dy, prunings[i % rotate][0], algo=args.algo,
                                workspace=ws, out=out, variant=variant)
            return
        fff.backward(x, W, b, V, Wo, dy, algo=args.algo, workspace=ws, out=out, variant=variant)

    t_ms = _events_ms(torch, step, args.steps, args.warmup)
    s = shape
    L = s.D + 1
    # The backward's matrix products as the method needs them (visited nodes
    # only) and as the masked form executes them (every node of the levels).
    alg = 2 * 2 * s.T * s.P * s.h * s.d + 2 * 2 * s.T * s.P * L * s.d + 2 * s.T * s.P * L * s.h
    executed = 2 * 2 * s.T * s.P * s.h * s.d + 2 * 2 * s.T * (s.P << L) * s.d + \
        2 * s.T * (s.P << L) * s.h
    print(json.dumps({
        "metric": "FFF layer backward tokens/sec (bf16)", "value": s.T / (t_ms * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_ms, "higher_is_better": True, "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic", "config": {"workload": args.workload, "T": s.T, "d": s.d, "P": s.P,
                                        "D": s.D, "h": s.h, "variant": args.variant,
                                        "algo": args.algo, "rotated_sets": rotate,
                                        **({"pruning": {"ratio": args.prune,
                                                        "alive_leaves": float(mask.mean())}}
                                           if prunings is not None else {})},
        "flops": {"algorithmic": alg, "executed": executed,
                  "executed_tflops": executed / (t_ms * 1e-3) / 1e12}}), flush=True)


def dataclasses_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.depth_sweep:
        depth_sweep(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by tokens with no communication, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_tree_structured_amd as fff
    import workloads

    dev = torch.device("cuda:0")
    shape, opts = workloads.WORKLOADS[args.workload]
    footprint = (shape.T * shape.d + shape.P * shape.N * (shape.d + shape.h + 1)
                 + shape.P * shape.h * shape.d) * (2 if shape.dtype == "bf16" else 4)
    rotate = args.rotate or max(2, -(-600_000_000 // max(footprint, 1)))
    rotate = min(rotate, 64)

    def upload(inp):
        out = []
        for k in ("x", "W_node", "b_node", "V_node", "W_out"):
            a = getattr(inp, k)
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if shape.dtype == "bf16" \
                else torch.from_numpy(a)
            out.append(t.to(dev))
        return out

    inp0 = workloads.make_inputs(shape, seed=0, **opts)
    sets = [upload(inp0)] + [upload(workloads.make_inputs(shape, seed=s, **opts))
                             for s in range(1, rotate)]
    torch.cuda.synchronize()

    variant = fff.VARIANTS[args.variant]
    fshape = fff.shape_of(sets[0][0], sets[0][1], sets[0][3], variant)
    plan = fff.resolve_plan(fshape, fff.make_plan(args.algo, args.split_level, args.chunk_tokens))
    ws, nbytes = fff.alloc_workspace(fshape, plan, dev)
    y = torch.empty((shape.T, shape.d), dtype=sets[0][0].dtype, device=dev)
    path = torch.empty((shape.T, shape.P), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    prunings = None
    if args.prune > 0:
        # Each tree keeps at least one path; one table per input set.
        rng = np.random.default_rng(0)
        mask = (rng.random((shape.P, 1 << shape.D)) >= args.prune).astype(np.uint8)
        mask[np.arange(shape.P), rng.integers(0, 1 << shape.D, size=shape.P)] = 1
        prunings = [fff.prune_prepare(mask, st[1], st[3], algo=plan.algo,
                                      split_level=plan.split_level,
                                      chunk_tokens=plan.chunk_tokens, T=shape.T)
                    for st in sets]
        torch.cuda.synchronize()

    def step(i, ev=None):
        x, W, b, V, Wo = sets[i % rotate]
        if prunings is not None:
            fff.forward_pruned(x, W, b, V, Wo, prunings[i % rotate][0], algo=plan.algo,
                               split_level=plan.split_level, chunk_tokens=plan.chunk_tokens,
                               workspace=ws, y=y, path_out=path, stream=stream, events=ev,
                               variant=variant)
            return
        fff.forward(x, W, b, V, Wo, algo=plan.algo, split_level=plan.split_level,
                    chunk_tokens=plan.chunk_tokens, workspace=ws, y=y, path_out=path, stream=stream,
                    events=ev, variant=variant)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # HIP events (torch-created, so profilers see ordinary events) that the
    # library records on `stream` at its stage boundaries.  Record each once
    # so the underlying event exists before its handle is passed on.
    nev = len(fff.StageEvents.NAMES)

    def clean_pass(nsteps):
        # The headline: K steps on rotating input sets, no events inside.
        t0 = time.perf_counter()
        for i in range(nsteps):
            step(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def staged_pass(nsteps, rotating):
        # The same steps with the library's stage events on the stream.  An
        # event costs about 3 us of GPU time, so this pass is timed apart
        # from the headline one; it gives each stage's (kernel's) duration.
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(nev))
               for _ in range(nsteps)]
        for ev in evs:
            for e in ev:
                e.record(stream)
        torch.cuda.synchronize()
        sev = [fff.StageEvents(*[e.cuda_event for e in ev]) for ev in evs]
        t0 = time.perf_counter()
        for i in range(nsteps):
            step(i if rotating else 0, sev[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # per step: the intervals between consecutive stage events (ms)
        stages = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(nev - 1)] for ev in evs])
        fwd = np.array([ev[0].elapsed_time(ev[-1]) for ev in evs])
        return elapsed, stages, fwd

    elapsed = clean_pass(args.steps)
    staged_elapsed, stages_ms, fwd_ms = staged_pass(args.steps, True)
    _, _, warm_ms = staged_pass(max(5, args.steps // 2), False)

    # Device output on input set 0 (paths for the distinct visited nodes, the
    # empty-leaf fraction and the parity figures).
    step(0)
    torch.cuda.synchronize()
    leaves = path.cpu().numpy().astype(np.int64)
    y0 = y.float().cpu().numpy().astype(np.float64)
    visited = set()
    used_leaves = 0
    for p in range(shape.P):
        lfs = np.unique(leaves[:, p])
        used_leaves += len(lfs)
        for lf in lfs:
            n = int(lf) + (1 << shape.D) - 1
            while True:
                visited.add((p, n))
                if n == 0:
                    break
                n = (n - 1) // 2
    U = len(visited)
    empty_leaf_frac = 1.0 - used_leaves / float(shape.P << shape.D)
    f_route, f_proj, b_alg = algorithmic_work(shape, U)
    ms_step = 1e3 * elapsed / args.steps
    tokens_per_s = shape.T * args.steps / elapsed

    # Stage rooflines.  Work per stage is what the method itself needs there:
    # the routing stages' logits only along the paths (T*P per level, 2d
    # flops each) and each stage's own operand and result bytes (the H build:
    # its records in, H out; the projection: H, W_out and y).
    e = 2 if shape.dtype == "bf16" else 4
    T, d, P, D, h, K = shape.T, shape.d, shape.P, shape.D, shape.h, shape.P * shape.h
    k = plan.split_level if plan.algo == fff.ALGO_PREFILL else D + 1
    k = min(k, D + 1)
    x_bytes = T * d * e
    rows_top = P * ((1 << k) - 1)
    rows_deep = P * ((1 << (D + 1)) - (1 << k))
    stage_work = {
        # name: (flops, bytes)
        "top": (2 * T * P * k * d, x_bytes + rows_top * (d + 1) * e + 4 * T * P * (k + 1)),
        "deep": (2 * T * P * (D + 1 - k) * d,
                 x_bytes + rows_deep * (d + 1) * e + 4 * T * P * (D + 2 - k)),
        "hbuild": (2 * T * P * (D + 1) * h,
                   4 * T * P * (D + 2) + P * shape.N * h * e + T * K * e + 4 * T * P),
        "proj": (f_proj, T * K * e + K * d * e + T * d * e),
    }
    fused = plan.algo == fff.ALGO_DECODE
    # Intervals between the library's events: start-prepared (nothing is
    # prepared: the two events are recorded back to back, so it is counted
    # with the top levels), prepared-top, top-deep, deep-routed, routed-done.
    intervals = {"top": (0, 2), "deep": (2, 3), "hbuild": (3, 4), "proj": (4, 5)}
    stage_us = {n: float(np.mean(stages_ms[:, a:b].sum(axis=1))) * 1e3
                for n, (a, b) in intervals.items()}
    if fused:  # one kernel: its time sits in the first interval
        stage_us = {"decode": float(np.mean(stages_ms[:, 0])) * 1e3}
        stage_work = {"decode": (f_route + f_proj, b_alg)}
    stages = {}
    for n, us in stage_us.items():
        fl, by = stage_work[n]
        t_mfma = fl / (PEAK_MFMA_BF16_TFLOPS * 1e12)
        t_hbm = by / (PEAK_HBM_GBPS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        t = max(us, 1e-3) * 1e-6
        stages[n] = {"us": us, "flops": fl, "bytes": by, "bound": bound,
                     "tflops": fl / t / 1e12, "gbps": by / t / 1e9,
                     "frac": max(t_mfma, t_hbm) / t}
    dom = max(stages, key=lambda n: stages[n]["us"])
    ds = stages[dom]
    kernel_of = {"top": "route_top", "deep": "subtree", "hbuild": "hbuild",
                 "proj": "proj_direct", "decode": "decode"}
    traffic = measured_traffic(kernel_of[dom], args.workload)
    if ds["bound"] == "mfma":
        roof = {"bound": "mfma", "kernel": kernel_of[dom], "stage": dom, "achieved": ds["tflops"],
                "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ds["frac"],
                "traffic": traffic, "per_launch": {"flops": ds["flops"], "avg_us": ds["us"]}}
    else:
        roof = {"bound": "hbm", "kernel": kernel_of[dom], "stage": dom, "achieved": ds["gbps"],
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ds["frac"], "traffic": traffic,
                "per_launch": {"bytes": ds["bytes"], "avg_us": ds["us"]}}
    if traffic:
        roof["traffic_gbps"] = traffic / (ds["us"] * 1e-6) / 1e9

    t_roof = max(b_alg / (PEAK_HBM_GBPS * 1e9), (f_route + f_proj) / (PEAK_MFMA_BF16_TFLOPS * 1e12))
    t_med = float(np.median(fwd_ms)) * 1e-3
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the named shape)",
        "config": {"workload": args.workload, "T": shape.T, "d": shape.d, "P": shape.P,
                   "D": shape.D, "h": shape.h, "variant": args.variant,
                   "algo": fff.algo_name(plan.algo),
                   "split_level": plan.split_level, "chunk_tokens": plan.chunk_tokens,
                   "rotated_sets": rotate,
                   "parallelism": "none (1 GPU)",
                   **({"pruning": {"ratio": args.prune, "alive_leaves": float(mask.mean()),
                                   "col_tiles": int(prunings[0][0].col_tiles),
                                   "unpruned_col_tiles": -(-(shape.P << plan.split_level) // 256)
                                   if plan.algo == fff.ALGO_PREFILL else None}}
                      if prunings is not None else {})},
        "roofline": roof,
        "stages": stages,
        "layer": {"F_alg": f_route + f_proj, "B_alg": b_alg, "U": U,
                  "t_roof_us": t_roof * 1e6, "roof_frac": t_roof / (ms_step * 1e-3),
                  "hbm_frac": b_alg / (ms_step * 1e-3) / (PEAK_HBM_GBPS * 1e9),
                  "mfma_frac_proj": stages["proj"]["frac"] if "proj" in stages else None,
                  "empty_leaf_frac": empty_leaf_frac,
                  "route_us": float(np.mean(stages_ms[:, :4].sum(axis=1))) * 1e3,
                  "proj_us": float(np.mean(stages_ms[:, 4])) * 1e3,
                  "t_us_median": t_med * 1e6,
                  "t_us_p10": float(np.percentile(fwd_ms, 10)) * 1e3,
                  "t_us_p90": float(np.percentile(fwd_ms, 90)) * 1e3,
                  "rotated": True,
                  "staged_pass_us_per_step": 1e6 * staged_elapsed / args.steps,
                  "warm_t_us_median": float(np.median(warm_ms)) * 1e3,
                  "warm_tokens_per_s": shape.T / (float(np.median(warm_ms)) * 1e-3),
                  "event_floor_us": event_floor_us(torch)},
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        cb, ref = cpu_baseline(inp0, args.cpu_seconds, variant,
                               mask if prunings is not None else None)
        out["cpu_baseline"] = cb
        out["parity"] = parity_figures(inp0, ref, cb["tokens"], leaves, y0, variant,
                                       mask if prunings is not None else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
