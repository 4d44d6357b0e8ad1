#!/usr/bin/env python3
"""Throughput of the POET-X linear layer (fwd + bwd) on one MI355X.

One step is the whole hot path over one batch: the CNP blocks of both sides of
every linear of a Llama-8B decoder layer (one poetx_cnp_build_batch), the
forward of the seven linears (q, k, v, o, gate, up, down), then their backward
(poetx_linear_bwd_dx) and the CNP chain rule of all sides down to packed dq
(one poetx_cnp_backward_batch).  T = 8192 tokens, b = 512, bf16 activations and
weights with fp32 accumulation.  Inputs are seeded synthetic tensors already
resident in HBM when timing starts.

Prints one JSON line: tokens/s of the whole step, the roofline figure of the
dominant kernel class (the W~ contractions) from hipEvents recorded around its
launches during the timed steps, and the fp64 CPU oracle timed on a bounded
sample of the same workload as a baseline.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload llama8b]
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # dense MFMA: 256 CU x 2.4 GHz x 4096 (bf16) / 256 (fp32) flop/clk
HBM_PEAK_GBS = 8000.0
METRIC = "POET-X linear fwd+bwd tokens/s at Llama-8B shapes; % MFMA peak (1 GPU)"
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_MD = os.path.join(ROOT, "profiles", "llama8b_gemm_traffic.md")
CLASSES_MD = os.path.join(ROOT, "profiles", "llama8b_kernel_classes.md")
COPY_PROBE_BYTES = 256 << 20  # device-to-device copy of known size, the counters' calibration


def side_sums(d, b):
    nb = -(-d // b)
    r = d - (nb - 1) * b
    return (nb - 1) * b * b + r * r, (nb - 1) * b**3 + r**3


def step_flops(wl, T):
    """Algorithmic flops of one fwd+bwd step: W~ contractions, block products, CNP."""
    gemm = apply = cnp = 0.0
    for L in wl.linears:
        gemm += 4.0 * T * L.m * L.n
        r2R, r3R = side_sums(L.m, wl.b)
        r2P, r3P = side_sums(L.n, wl.b)
        apply += 6.0 * T * (r2R + r2P)  # fwd R, P; bwd P apply, P grad, R grad, R apply
        cnp += 16.0 * (r3R + r3P)  # build (2 products) + chain rule (6 products)
    return gemm, apply, cnp


def describe(wl):
    shapes = ", ".join(f"{L.name} {L.m}x{L.n}" for L in wl.linears)
    return f"{wl.description}: linears {shapes}"


def cpu_baseline(inp, wl, lin_flops, total_flops):
    """fp64 oracle, untuned, on one linear of the workload at full T; scaled to
    the whole layer by algorithmic flops."""
    import oracle as O
    from threadpoolctl import threadpool_info

    X = O.to_f64(inp.X, inp.act)
    dZ = O.to_f64(inp.dZ, inp.act)
    W = O.to_f64(inp.W0, inp.w, inp.w_scale)
    q_R, q_P = inp.q_R.astype(np.float64), inp.q_P.astype(np.float64)
    t0 = time.perf_counter()
    G_R, G_P = O.side_G(q_R, inp.m, inp.b), O.side_G(q_P, inp.n, inp.b)
    O.forward(X, W, inp.perm_R, inp.perm_P, G_R, G_P)
    O.backward(X, dZ, W, inp.perm_R, inp.perm_P, q_R, q_P, inp.b)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    layer_seconds = dt * total_flops / lin_flops
    return {
        "value": inp.T / layer_seconds,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (
            f"linear {inp.m}x{inp.n} of the same layer, all {inp.T} tokens, fwd + bwd incl. CNP "
            f"({dt:.1f} s); scaled to the 7-linear layer by algorithmic flops x{total_flops / lin_flops:.2f}"
        ),
        "seconds": dt,
        "host_cpus": os.cpu_count(),
    }


def kernel_source_hash():
    """sha256 over the HIP sources and headers: counter figures are only valid for the code they measured."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "orthogonal_reparameterized_cnp_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter_csv(d):
    """[(dispatch id, kernel name, KiB)] from a rocprofv3 --pmc output directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


def summarize_traffic(fetch_dir, write_dir, cmd_fetch, cmd_write):
    """Turn one FETCH_SIZE run and one WRITE_SIZE run of `bench.py --copy-probe` into per-launch HBM
    bytes of the W~ contractions, each counter scaled by what it reads for the copy probe."""
    res = {}
    for key, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = read_counter_csv(d)
        # the probe is the last device copy before the step's first CNP kernel (warm-up 0)
        first_step = min((i for i, n, _ in rows if "k_unpack_q" in n), default=None)
        copies = [v for i, n, v in rows if "copyBuffer" in n and first_step is not None and i < first_step]
        gemm = [v for _, n, v in rows if "k_gemm<" in n or "k_gemm_group<" in n]
        if not copies or not gemm or copies[-1] * 1024 < COPY_PROBE_BYTES / 4:
            raise SystemExit(f"{d}: copy probe or k_gemm dispatches missing")
        # the probe reads and writes COPY_PROBE_BYTES once
        factor = COPY_PROBE_BYTES / (copies[-1] * 1024)
        res[key] = {"factor": factor, "launches": len(gemm), "bytes_per_launch": sum(gemm) * 1024 * factor / len(gemm)}
    traffic = res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"]
    line = {
        "kernel_source_hash": kernel_source_hash(),
        "traffic_bytes_per_launch": traffic,
        "fetch_bytes_per_launch": res["fetch"]["bytes_per_launch"],
        "write_bytes_per_launch": res["write"]["bytes_per_launch"],
        "fetch_scale": res["fetch"]["factor"],
        "write_scale": res["write"]["factor"],
        "launches": res["fetch"]["launches"],
    }
    txt = f"""# W~ contractions (k_gemm): HBM traffic per launch (rocprofv3 counters)

Workload: one step of bench.py's default (7 POET-X linears of a Llama-8B decoder layer, T = 8192, b = 512,
bf16), with a {COPY_PROBE_BYTES >> 20} MiB device-to-device copy before the step as calibration.

Commands (from the repository root on one MI355X, one counter per run):

    {cmd_fetch}
    {cmd_write}
    python bench.py --summarize-traffic {fetch_dir} {write_dir}

Each counter is scaled by the factor that maps its reading for the copy probe to the probe's true
bytes: FETCH_SIZE x{res['fetch']['factor']:.3f}, WRITE_SIZE x{res['write']['factor']:.3f}.

| | per k_gemm launch (mean of {res['fetch']['launches']}) |
|---|---|
| bytes fetched | {res['fetch']['bytes_per_launch'] / 1e9:.4f} GB |
| bytes written | {res['write']['bytes_per_launch'] / 1e9:.4f} GB |
| traffic | {traffic / 1e9:.4f} GB |

bench.py reports `roofline.traffic` from the line below while the kernel sources still hash to the same value.

traffic-json: {json.dumps(line)}
"""
    with open(TRAFFIC_MD, "w") as fh:
        fh.write(txt)
    print(txt)


KERNEL_CLASSES = (  # kernel-name prefix -> class, as in --breakdown
    ("k_gemm<", "W~ contractions"),
    ("k_gemm_group<", "W~ contractions"),
    ("k_apply<", "block products"),
    ("k_apply_stream<", "block products"),
    ("k_block_grads", "block gradients"),
    ("k_cnp_", "CNP products"),
    ("k_unpack_q", "CNP pack/unpack"),
    ("k_pack_dq", "CNP pack/unpack"),
    ("k_permute", "permutations"),
    ("k_inverse_perm", "permutations"),
    ("k_scatter", "permutations"),
    ("k_adam<", "optimiser step"),
)
N_XCC = 8  # GRBM_GUI_ACTIVE is reported once per XCD; the counter CSV holds their sum


def kernel_class(name):
    for prefix, cls in KERNEL_CLASSES:
        if prefix in name:
            return cls
    return None


def read_counter_rows(d):
    """{dispatch id: {"name", "ns", counter: value}} from a rocprofv3 --pmc output directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                e = out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                          "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_classes(mfma_dir, fetch_dir, write_dir, cmds):
    """Per kernel class of one bench step: MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs and
    the XCDs' busy cycles) and copy-calibrated HBM bytes and rates (FETCH_SIZE, WRITE_SIZE)."""
    n_simd = 256 * 4
    rows = {k: read_counter_rows(d) for k, d in (("mfma", mfma_dir), ("fetch", fetch_dir), ("write", write_dir))}
    scale = {}
    for key in ("fetch", "write"):
        r = rows[key]
        first_step = min((i for i, e in r.items() if "k_unpack_q" in e["name"]), default=None)
        copies = [(i, e) for i, e in sorted(r.items()) if "copyBuffer" in e["name"] and first_step and i < first_step]
        ctr = "FETCH_SIZE" if key == "fetch" else "WRITE_SIZE"
        if not copies:
            raise SystemExit(f"{key}: copy probe missing")
        scale[key] = COPY_PROBE_BYTES / (copies[-1][1][ctr] * 1024)
    cls = {}
    for key, ctr in (("mfma", None), ("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        for i, e in rows[key].items():
            c = kernel_class(e["name"])
            if c is None:
                continue
            a = cls.setdefault(c, {"n": 0, "ns_mfma": 0, "busy": 0.0, "gui": 0.0, "ns_fetch": 0, "fetch": 0.0,
                                   "ns_write": 0, "write": 0.0})
            if key == "mfma":
                a["n"] += 1
                a["ns_mfma"] += e["ns"]
                a["busy"] += e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                a["gui"] += e.get("GRBM_GUI_ACTIVE", 0.0)
            else:
                a["ns_" + key] += e["ns"]
                a[key] += e[ctr] * 1024 * scale[key]
    # one k_pack_dq launch ends every step: the timed steps and the separate pass that times the contractions
    steps = sum(1 for e in rows["mfma"].values() if "k_pack_dq" in e["name"]) or 1
    lines = []
    for c in dict.fromkeys(c for _, c in KERNEL_CLASSES):
        a = cls.get(c)
        if not a:
            continue
        busy = a["busy"] / (a["gui"] / N_XCC * n_simd) if a["gui"] else 0.0
        gbs = lambda k: a[k] / (a["ns_" + k] * 1e-9) / 1e9 if a["ns_" + k] else 0.0
        lines.append(f"| {c} | {a['n'] / steps:g} | {a['ns_mfma'] / 1e6 / steps:.3f} | {100 * busy:.1f}% | "
                     f"{a['fetch'] / 1e9 / steps:.3f} | {a['write'] / 1e9 / steps:.3f} | {gbs('fetch') + gbs('write'):.0f} |")
    txt = f"""# One bench step by kernel class: MFMA busy and HBM traffic (rocprofv3 counters)

Workload: bench.py's default step (7 POET-X linears of a Llama-8B decoder layer, T = 8192, b = 512,
bf16), warm-up 0; the FETCH_SIZE and WRITE_SIZE runs add a {COPY_PROBE_BYTES >> 20} MiB device copy as calibration.

Commands (from the repository root on one MI355X, one counter set per run):

    {cmds[0]}
    {cmds[1]}
    {cmds[2]}
    python bench.py --summarize-classes {mfma_dir} {fetch_dir} {write_dir}

- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES summed over all {n_simd} SIMDs / ({n_simd} x the XCDs' busy cycles, GRBM_GUI_ACTIVE
  summed over {N_XCC} XCDs / {N_XCC}). It counts cycles with the matrix pipe occupied, at the clock the chip ran.
- Bytes between the L2s and memory (HBM or the Infinity Cache; the counters do not tell them apart):
  FETCH_SIZE x{scale['fetch']:.3f} and WRITE_SIZE x{scale['write']:.3f} (the factors that map each counter's
  reading for the copy probe to its true bytes); rates divide by the same run's kernel durations.
- Durations are those of the counter run (the profiler serialises dispatches), not the bench timing.
- Each run holds {steps} steps (the timed step and the pass that times the W~ contractions); launches, ms and GB
  are per step. The optimiser step runs after the timed steps, outside them.

| class | launches / step | ms / step | MFMA busy | GB fetched | GB written | GB/s (fetch + write) |
|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"
    with open(CLASSES_MD, "w") as fh:
        fh.write(txt)
    print(txt)


def committed_traffic():
    """Per-launch HBM bytes of the W~ contractions from the committed counter summary, or None when the
    summary is missing or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_MD) as fh:
            for l in fh:
                if l.startswith("traffic-json: "):
                    d = json.loads(l[len("traffic-json: "):])
                    if d.get("kernel_source_hash") == kernel_source_hash():
                        return d["traffic_bytes_per_launch"]
    except OSError:
        pass
    return None


def time_merge(key, to_dev, dev, layers=None):
    """poetx_merge_reinit of every linear of one decoder layer of workload `key` (merge-then-reinitialise:
    fold R and P into the weight, requantise int8 per column, draw new permutations, zero q), timed with
    events around the calls after one untimed merge; amortised over the workload's merge period.
    `layers`: the workload's PoetxLinear objects if already built (their weights are merged in place)."""
    import torch

    from orthogonal_reparameterized_cnp_amd.layer import PoetxLinear
    from workloads import WORKLOADS, make_linear_inputs

    wl = WORKLOADS[key]
    if layers is None:
        layers = []
        for i in range(len(wl.linears)):
            inp = make_linear_inputs(wl, i, T=1)
            lay = PoetxLinear(inp.m, inp.n, inp.b, inp.act, inp.w)
            scale = to_dev(inp.w_scale, "f32") if inp.w == "i8" else None
            lay.load(to_dev(inp.W0, inp.w), scale, to_dev(inp.perm_R, "i32"), to_dev(inp.perm_P, "i32"),
                     to_dev(inp.q_R, "f32"), to_dev(inp.q_P, "f32"))
            layers.append(lay)
    for lay in layers:
        lay.build()
        lay._ws(lay.ws_bytes(1))
    torch.cuda.synchronize()

    def merge_all(seed):
        for j, lay in enumerate(layers):
            lay.merge_reinit(seed + 2 * j, seed + 2 * j + 1)

    merge_all(1)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    merge_all(1001)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    flops = 0.0
    for L in wl.linears:
        flops += 2.0 * (L.n * side_sums(L.m, wl.b)[0] + L.m * side_sums(L.n, wl.b)[0])
    period = wl.merge_every or 1
    print(f"[bench] merge {key}: {ms:.3f} ms per layer merge ({flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s fp32 MFMA), "
          f"every {period} steps: {ms / period:.4f} ms per step", file=sys.stderr, flush=True)
    return {
        "workload": describe(wl),
        "weights": wl.w,
        "ms_per_layer_merge": ms,
        "every_steps": period,
        "amortised_ms_per_step": ms / period,
        "tflops_fp32": flops / (ms * 1e-3) / 1e12,
    }


def time_spo(T, d, b, act, to_dev):
    """One extra SPO factor of each kind on token rows at T x d (poetx_spo_fwd + poetx_spo_bwd), timed with
    events after one untimed call: the cost of each factor a chain of c > 1 factors per side adds."""
    import torch

    from orthogonal_reparameterized_cnp_amd.layer import PoetxSpoFactor
    from workloads.gen import spo_inputs

    out = {}
    for kind in ("block", "full"):
        inp = spo_inputs(d, b, kind, T, act, 0.005, seed=7)
        f = PoetxSpoFactor(d, b, kind, act)
        f.load(to_dev(inp.idx, "i32"), to_dev(inp.q, "f32"))
        f.build()
        X, dY = to_dev(inp.X, act), to_dev(inp.dY, act)
        Y, dX = torch.empty_like(X), torch.empty_like(X)
        dq = torch.empty_like(f.q)
        f.forward(X, Y)
        f.backward(dY, dX, dq)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record()
        f.forward(X, Y)
        ev[1].record()
        f.backward(dY, dX, dq)
        ev[2].record()
        torch.cuda.synchronize()
        fwd, bwd = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
        de = f.d_eff
        r2, r3 = side_sums(de, b)
        fl_f, fl_b = 2.0 * T * r2, 4.0 * T * r2 + 12.0 * r3
        out[kind] = {"d": d, "b": b, "T": T, "columns_transformed": de, "fwd_ms": fwd, "bwd_ms": bwd,
                     "fwd_tflops": fl_f / (fwd * 1e-3) / 1e12, "bwd_tflops": fl_b / (bwd * 1e-3) / 1e12}
        print(f"[bench] spo {kind} d={d} b={b} T={T}: fwd {fwd:.3f} ms, bwd {bwd:.3f} ms", file=sys.stderr, flush=True)
        del X, dY, Y, dX, f
    return out


class WorkloadStep:
    """One decoder layer of a workload on the GPU: seeded inputs resident in HBM, and step(), the
    whole hot path over one batch (batched CNP build, the forwards, the backwards to dX and the block
    gradients, the batched CNP chain rule to every side's packed dq, and optionally the Adam step)."""

    def __init__(self, wl, mode, to_dev, dev, optimizer=False, batch_grads=True, grouped=True):
        import torch

        from orthogonal_reparameterized_cnp_amd.layer import PoetxAdam, PoetxGroup, PoetxLinear
        from workloads import make_linear_inputs

        self.wl, self.mode, self.T = wl, mode, wl.T
        self.layers, self.Xs, self.dZs, self.inputs0 = [], [], [], None
        for i in range(len(wl.linears)):
            inp = make_linear_inputs(wl, i)
            lay = PoetxLinear(inp.m, inp.n, inp.b, inp.act, inp.w, mode=mode)
            scale = to_dev(inp.w_scale, "f32") if inp.w == "i8" else None
            lay.load(to_dev(inp.W0, inp.w), scale, to_dev(inp.perm_R, "i32"), to_dev(inp.perm_P, "i32"),
                     to_dev(inp.q_R, "f32"), to_dev(inp.q_P, "f32"))
            lay.reserve(self.T)
            self.layers.append(lay)
            # linears that read one input (q, k, v; gate, up) share the tensor of the first of them
            first = next(g[0] for g in wl.input_groups if i in g)
            self.Xs.append(self.Xs[first] if first != i else to_dev(inp.X, inp.act))
            self.dZs.append(to_dev(inp.dZ, inp.act))
            if i == 0:
                self.inputs0 = inp
        dt = self.Xs[0].dtype
        self.Ys = [torch.empty(self.T, L.n, dtype=dt, device=dev) for L in wl.linears]
        self.dXs = [torch.empty(self.T, L.m, dtype=dt, device=dev) for L in wl.linears]
        self.dqs = [(torch.empty_like(l.q_R), torch.empty_like(l.q_P)) for l in self.layers]
        # The layer's seven linears share their CNP work: every side's G is built in one batch, and the
        # block gradients and the chain rule to dq run once for all sides after the backward of the
        # last linear (batch_grads; without it the block gradients run per linear and the results are
        # bit-identical to per-linear calls).
        self.batch_grads = batch_grads
        self.group = PoetxGroup(self.layers, batch_grads=batch_grads)
        # grouped: the linears that share an input run as one group call (their block products in shared
        # launches, their W~ contractions in one launch where that fills the GPU); bit-identical outputs
        self.grouped = grouped and batch_grads
        self.calls = wl.input_groups if self.grouped else tuple((i,) for i in range(len(wl.linears)))
        if self.grouped:
            # the linears of a call read one input: they share its gradient, the sum of theirs
            for g in self.calls:
                for i in g[1:]:
                    self.dXs[i] = self.dXs[g[0]]
        # Adam on every side's packed q (lr small enough that the timed steps stay near the start)
        self.opt = PoetxAdam(self.layers, lr=1e-5)
        self.optimizer = optimizer
        torch.cuda.synchronize()

    def step(self):
        self.group.build()
        if not self.grouped:
            for lay, X, Y in zip(self.layers, self.Xs, self.Ys):
                lay.forward(X, Y)
            for i in reversed(range(len(self.layers))):
                self.group.backward_dx(i, self.Xs[i], self.dZs[i], self.dXs[i],
                                       Y=self.Ys[i] if self.mode == "xout" else None)
        else:
            for g in self.calls:
                self.group.forward(g, [self.Xs[i] for i in g], [self.Ys[i] for i in g])
            for g in reversed(self.calls):
                self.group.backward_dx_many(g, [self.dZs[i] for i in g], [self.dXs[i] for i in g],
                                            Ys=[self.Ys[i] for i in g] if self.mode == "xout" else None)
        self.group.backward_q(self.dqs)
        if self.optimizer:
            self.opt.step(self.dqs)


def timed(fn, steps):
    """Average ms per call of fn over `steps` calls between two events on the current stream, with a
    device synchronisation before and after; also the host wall time of the region."""
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - t0


def weight_centric_flops(wl, T):
    """Algorithmic flops of one weight-centric step: the three block products over the weight, the
    forward contraction, dX and the weight gradient dM, the block gradients from dM, the CNP work."""
    tot = 0.0
    for L in wl.linears:
        r2R, r3R = side_sums(L.m, wl.b)
        r2P, r3P = side_sums(L.n, wl.b)
        tot += 2.0 * L.n * r2R + 4.0 * L.m * r2P  # U^T, V, M
        tot += 6.0 * T * L.m * L.n  # Y, dX, dM
        tot += 2.0 * L.n * r2R + 2.0 * L.m * r2P  # dG_R, dG_P
        tot += 16.0 * (r3R + r3P)
    return tot


def time_weight_centric(ws, steps, ic_ms):
    """The same step computed weight-centric (poetx_wc_fwd / poetx_wc_bwd on the same layers: the factors
    applied to the weight, dense contractions, the full weight gradient), timed like the headline."""
    import torch

    from orthogonal_reparameterized_cnp_amd.layer import PoetxWeightCentric

    wcs = [PoetxWeightCentric(l) for l in ws.layers]
    for wc in wcs:
        wc.reserve(ws.T)

    def wstep():
        ws.group.build()
        for wc, X, Y in zip(wcs, ws.Xs, ws.Ys):
            wc.forward(X, Y)
        for i in reversed(range(len(wcs))):
            wcs[i].backward(ws.dZs[i], ws.dXs[i], *ws.dqs[i])

    for _ in range(2):
        wstep()
    ms, _ = timed(wstep, steps)
    fl = weight_centric_flops(ws.wl, ws.T)
    print(f"[bench] weight-centric step: {ms:.3f} ms ({ms / ic_ms:.2f}x the input-centric step)",
          file=sys.stderr, flush=True)
    del wcs
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms,
        "ratio_to_input_centric": ms / ic_ms,
        "tflop_per_step": fl / 1e12,
        "tflops": fl / (ms * 1e-3) / 1e12,
        "what": "poetx_wc_fwd / poetx_wc_bwd on the same layers and inputs: M = Diag(G_R) W~ Diag(G_P) built "
                "every step, dense contractions with M, the weight gradient dM = Xt^T dZt, block gradients "
                "from dM; CNP build batched as in the headline, CNP chain rule per linear",
    }


SECONDARY = ("linear256_fp32", "llama60m", "llama1p3b", "llama13b_int8")


def time_secondary(key, to_dev, dev):
    """One step of another workload (same structure as the headline), timed after two warm-up steps; the
    int8 Llama-13B layer also times its merge-then-reinitialise, amortised over its merge period."""
    import torch

    from workloads import WORKLOADS

    wl = WORKLOADS[key]
    ws = WorkloadStep(wl, "xfast", to_dev, dev)
    for _ in range(2):
        ws.step()
    steps = 50 if wl.T * sum(L.m * L.n for L in wl.linears) < 1e10 else 5
    ms, _ = timed(ws.step, steps)
    g, a, c = step_flops(wl, wl.T)
    tf = (g + a + c) / (ms * 1e-3) / 1e12
    out = {"workload": describe(wl), "weights": wl.w, "tokens": wl.T, "b": wl.b, "steps": steps, "ms_per_step": ms,
           "tokens_per_s": wl.T / (ms * 1e-3), "tflops": tf, "mfma_peak_frac": tf / PEAK_TFLOPS[wl.act],
           "peak": f"{wl.act} dense MFMA {PEAK_TFLOPS[wl.act]} TFLOP/s"}
    print(f"[bench] {key}: {ms:.3f} ms per step, {out['tokens_per_s']:.0f} tokens/s, {tf:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    if wl.merge_every:
        out["merge"] = time_merge(key, to_dev, dev, layers=ws.layers)
    del ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="per kernel class timings on stderr")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the weight-centric comparison and the other workloads' lines")
    ap.add_argument("--mode", choices=("xfast", "xmem", "xout"), default="xfast",
                    help="xfast saves H for the backward; xmem saves only the gathered input and recomputes H; "
                         "xout saves only the gathered input and takes H back from the output")
    ap.add_argument("--grads", choices=("batched", "per-linear"), default="batched",
                    help="block gradients of all sides in shared launches after the last backward (dq equal to "
                         "the per-linear calls' to fp32 rounding), or inside each linear's backward")
    ap.add_argument("--calls", choices=("grouped", "per-linear"), default="grouped",
                    help="the linears that read one input (q, k, v; gate, up) as one group call (bit-identical "
                         "outputs, shared launches), or one call per linear; grouped needs --grads batched")
    ap.add_argument("--merge", metavar="WORKLOAD", nargs="?", const="llama13b_int8", default=None,
                    help="also time poetx_merge_reinit of every linear of WORKLOAD (default llama13b_int8) and "
                         "report it amortised over the workload's merge period")
    ap.add_argument("--optimizer", action="store_true",
                    help="end every step with the Adam step on all packed q (poetx_adam_step_batch)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time its replays (the W~ contraction rate then "
                         "comes from an eager pass of the same length)")
    ap.add_argument("--spo", action="store_true",
                    help="also time one extra SPO factor of each kind (block, full) at the widest side")
    ap.add_argument("--copy-probe", action="store_true",
                    help=f"run a {COPY_PROBE_BYTES >> 20} MiB device copy before the steps (counter calibration)")
    ap.add_argument("--summarize-classes", nargs=3, metavar=("MFMA_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the per-kernel-class counter summary from three rocprofv3 --pmc runs")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the k_gemm traffic summary from two rocprofv3 --pmc runs and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_traffic:
        base = "rocprofv3 --pmc {c} --output-format csv -d {d} -o llama8b -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --headline-only --copy-probe"
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                          base.format(c="FETCH_SIZE", d=args.summarize_traffic[0]),
                          base.format(c="WRITE_SIZE", d=args.summarize_traffic[1]))
        return
    if args.summarize_classes:
        m, f, w = args.summarize_classes
        base = "rocprofv3 --pmc {c} --output-format csv -d {d} -o llama8b -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --headline-only"
        summarize_classes(m, f, w, (base.format(c="SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE", d=m),
                                    base.format(c="FETCH_SIZE", d=f) + " --copy-probe",
                                    base.format(c="WRITE_SIZE", d=w) + " --copy-probe"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from orthogonal_reparameterized_cnp_amd import binding as B
    from workloads import WORKLOADS

    B.lib()
    wl = WORKLOADS[args.workload]
    T = wl.T
    dev = torch.device("cuda:0")

    def to_dev(a, kind):
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t_gen = time.perf_counter()
    ws = WorkloadStep(wl, args.mode, to_dev, dev, optimizer=args.optimizer, batch_grads=args.grads == "batched",
                      grouped=args.calls == "grouped")
    layers, inputs0, opt, dqs, step = ws.layers, ws.inputs0, ws.opt, ws.dqs, ws.step
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] copy probe: {COPY_PROBE_BYTES} bytes device to device", file=sys.stderr, flush=True)

    gemm_f, apply_f, cnp_f = step_flops(wl, T)
    total_f = gemm_f + apply_f + cnp_f
    graph = None
    if args.graph:
        if args.optimizer:
            raise SystemExit("--graph does not take --optimizer: the Adam step count is a launch argument")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()

    # the timed steps run with the library's measurement timer off
    if graph is not None:
        ms, wall = timed(graph.replay, args.steps)
    ms_eager, wall_eager = timed(step, args.steps)
    if graph is None:
        ms, wall = ms_eager, wall_eager
    # the W~ contraction rate: a separate pass of the same number of steps with hipEvents recorded
    # around every k_gemm launch on its stream
    B.poetx_timer_enable(B.POETX_KC_GEMM)
    B.poetx_timer_read()
    timed(step, args.steps)
    n_launch, k_ms, k_flops, k_bytes = B.poetx_timer_read()
    B.poetx_timer_enable(B.POETX_KC_NONE)

    peak = PEAK_TFLOPS[wl.act]
    achieved = k_flops / (k_ms * 1e-3) / 1e12 if k_ms > 0 else 0.0
    result = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act,
        "data": "synthetic (seeded normalized-Gaussian W0, N(0,1) X and dZ, N(0, std^2) packed q)",
        "config": {
            "workload": describe(wl),
            "tokens": T,
            "b": wl.b,
            "weights": wl.w,
            "mode": args.mode,
            "optimizer_in_step": "adam" if args.optimizer else None,
            "block_grads": args.grads,
            "calls": " | ".join(",".join(wl.linears[i].name for i in g) for g in ws.calls)
                     + (" (one input per call, its gradient the sum over the call's linears)" if ws.grouped else ""),
            "launch": "hip graph replay" if args.graph else "eager",
        },
        "tflops": total_f / (ms * 1e-3) / 1e12,
        "mfma_peak_frac": total_f / (ms * 1e-3) / 1e12 / peak,
        "step_tflop": {"w_contractions": gemm_f / 1e12, "block_products": apply_f / 1e12, "cnp": cnp_f / 1e12},
        "roofline": {
            "kernel": "W~ contractions (k_gemm: forward against the stored W~^T and backward, both NT)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": committed_traffic(),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "launches": n_launch,
            "avg_launch_ms": k_ms / max(n_launch, 1),
            "algorithmic_gb_per_launch": k_bytes / max(n_launch, 1) / 1e9,
        },
        "wall_s_timed": wall,
        "ms_per_step_eager": ms_eager,
        "timing": "step timed with the library's launch timer off; roofline.achieved from a separate pass of "
                  "the same number of steps with hipEvents around every W~ contraction launch",
    }

    # the optimiser step on its own (outside the timed region): HBM-bound, 28 bytes per packed slot;
    # one untimed call first, so that the kernel's first launch in the process is not timed
    opt.step(dqs)
    torch.cuda.synchronize()
    B.poetx_timer_enable(B.POETX_KC_OPTIM)
    B.poetx_timer_read()
    opt.step(dqs)
    torch.cuda.synchronize()
    n_o, o_ms, _, o_bytes = B.poetx_timer_read()
    B.poetx_timer_enable(B.POETX_KC_NONE)
    result["optimizer_step"] = {
        "kernel": "k_adam (Adam with decoupled decay on every side's packed q, one launch)",
        "launches": n_o,
        "ms": o_ms,
        "slots": int(o_bytes / 28),
        "algorithmic_gb": o_bytes / 1e9,
        "gb_per_s": o_bytes / (o_ms * 1e-3) / 1e9 if o_ms > 0 else None,
        "hbm_frac": o_bytes / (o_ms * 1e-3) / 8.0e12 if o_ms > 0 else None,
    }

    if args.breakdown:
        for name, kc in (("gemm", B.POETX_KC_GEMM), ("apply", B.POETX_KC_APPLY), ("dgrad", B.POETX_KC_DGRAD),
                         ("cnp", B.POETX_KC_CNP), ("permute", B.POETX_KC_PERMUTE),
                         ("optim", B.POETX_KC_OPTIM)):
            B.poetx_timer_enable(kc)
            B.poetx_timer_read()
            step()
            torch.cuda.synchronize()
            n, kms, kf, kb = B.poetx_timer_read()
            B.poetx_timer_enable(B.POETX_KC_NONE)
            rate = kf / (kms * 1e-3) / 1e12 if kms else 0
            bw = kb / (kms * 1e-3) / 1e9 if kms else 0
            print(f"[bench] {name:8s} launches={n:3d} ms/step={kms:8.3f} TFLOP/s={rate:7.1f} "
                  f"alg GB/s={bw:7.1f}", file=sys.stderr, flush=True)

    if not args.headline_only:
        result["weight_centric"] = time_weight_centric(ws, args.steps, ms)
    if args.merge:
        result["merge"] = time_merge(args.merge, to_dev, dev)
    if args.spo:
        result["spo_factor"] = time_spo(T, max(max(L.m, L.n) for L in wl.linears), wl.b, wl.act, to_dev)

    if not args.headline_only and args.workload == "llama8b":
        del ws, layers, opt, dqs, step
        torch.cuda.empty_cache()
        result["other_workloads"] = {k: time_secondary(k, to_dev, dev) for k in SECONDARY}

    if not args.no_cpu_baseline:
        lin_f = 4.0 * T * inputs0.m * inputs0.n
        r2R, r3R = side_sums(inputs0.m, wl.b)
        r2P, r3P = side_sums(inputs0.n, wl.b)
        lin_f += 6.0 * T * (r2R + r2P) + 16.0 * (r3R + r3P)
        result["cpu_baseline"] = cpu_baseline(inputs0, wl, lin_f, total_f)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
