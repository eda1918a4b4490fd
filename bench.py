"""Benchmark of the MoonEP hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at
the bench shape (R=8 virtual ranks, S=8192 tokens/rank, E=384, K=8,
H=7168, H'=2048, B=E/R=48, bf16, Zipf-biased routing tuned to maxvio 1):

    plan (moe_plan_run: the deterministic Theorem-1 construction) ->
    prefetch_weight -> dispatch -> grouped GEMM (all 8 ranks, one launch) ->
    combine -> weight-grad GEMM -> reduce_grad

All inputs are resident in HBM before timing starts.  W untimed warmup
steps, then K timed steps bracketed by device synchronisation; every entry
point is also bracketed by HIP events on the stream it runs on, giving each
step's average duration.  After the timed steps the data backward of the
layer (combine backward -> data-gradient GEMM -> dispatch backward) is timed
the same way and reported beside the step ("data_backward"), outside
`value`, and so are: the same step with the largest-first planner
("step_largest_first"); the step at every maxvio of the sweep 0.2 / 1 / 10 /
20 from one shared seed with both planners ("maxvio_sweep"); the
two-projection SwiGLU expert's kernels at the same
shape ("swiglu_expert": first projection [E+B, 7168, 2*2048] fused with
the activation, second projection [E+B, 2048, 7168], activation backward),
a two-layer backward sharing one prefetch pool ("prefetch_pool"), one
rank's product shape as a single segment beside hipBLASLt through
torch.matmul on the same operands (a comparator only,
"vendor_gemm_context"), the
Theorem-2 worst case at the same shape, training and inference B=4
("theorem2"), and the
Large-E shape (R=64, S=4096, E=896, K=16): plan, dispatch and combine over
all 64 ranks and one rank's grouped GEMM ("large_e").
Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--maxvio 1.0]
                    [--no-sweep] [--no-cpu-baseline] [--no-extras] [--swiglu-only]
                    [--vendor-only]
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_expert_load_amd as mx  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "plan µs + dispatch/combine GB/s + grouped-GEMM TFLOP/s @S8192 E384 K8 R8"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
STEPS = ("plan", "prefetch", "dispatch", "gemm", "combine", "wgrad", "reduce_grad")
# The step plans with the deterministic Theorem-1 construction
# (moe_plan_run: ascending experts); the largest-remaining-first donor policy
# is timed beside it.
PLAN_POLICY = mx.PLAN_ASCENDING
POLICY_NAMES = {mx.PLAN_ASCENDING: "ascending", mx.PLAN_LARGEST_FIRST: "largest_first"}


def run_plan(c, ids, plan, policy):
    """The planner entry point of a policy: moe_plan_run for the construction
    as the proof states it, moe_plan_run_policy otherwise."""
    if policy == mx.PLAN_ASCENDING:
        return mx.moe_plan_run(c, ids, plan)
    return mx.moe_plan_run_policy(c, ids, plan, policy)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_bench_shape.txt")
KERNEL_SOURCES = {"k_gemm<0>": "moe_expert_load_amd/csrc/gemm.hip",
                  "k_wgrad": "moe_expert_load_amd/csrc/gemm.hip",
                  "k_gemm<2>": "moe_expert_load_amd/csrc/gemm.hip",
                  "k_gemm<3>": "moe_expert_load_amd/csrc/gemm.hip",
                  "k_swiglu_bwd": "moe_expert_load_amd/csrc/swiglu.hip",
                  "k_combine_bwd": "moe_expert_load_amd/csrc/copy.hip",
                  "k_dispatch_bwd": "moe_expert_load_amd/csrc/copy.hip",
                  "k_dispatch": "moe_expert_load_amd/csrc/copy.hip",
                  "k_combine": "moe_expert_load_amd/csrc/copy.hip",
                  "k_prefetch": "moe_expert_load_amd/csrc/copy.hip",
                  "k_reduce_grad": "moe_expert_load_amd/csrc/copy.hip",
                  "k_count": "moe_expert_load_amd/csrc/plan.hip",
                  "k_plan": "moe_expert_load_amd/csrc/plan.hip",
                  "k_route": "moe_expert_load_amd/csrc/plan.hip"}


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so an edit
    to comments alone does not void the counters taken for the code."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[kernel], "moe_expert_load_amd/csrc/common.hpp"):
        h.update(_code_only(open(os.path.join(ROOT, rel), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's source changed after the counters were taken."""
    try:
        rec = json.loads(open(TRAFFIC_FILE).read().split("\n", 1)[1])
    except (OSError, ValueError, IndexError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_digest") != source_digest(kernel):
        return None
    return k["traffic_bytes"]


def _short_kernel(name):
    import re
    m = re.search(r"moonep::(k_\w+)(?:<(\d+)(?:,\s*(\d+))?>)?", name)
    if m:
        # k_gemm<MODE, CLASS> / k_sched<MODE> keep their mode, and k_gemm its
        # tile class when it is a small one (k_gemm<0>c2: the forward's
        # class-2 launch); other templates are tuning variants of one kernel
        k = m.group(1)
        if k not in ("k_gemm", "k_sched") or m.group(2) is None:
            return k
        cls = m.group(3)
        return "%s<%s>%s" % (k, m.group(2), "c" + cls if cls and cls != "4" else "")
    if name.startswith("Cijk_"):
        # the vendor library's GEMM (comparator only): keep its macro tile
        # and matrix instruction from the kernel name
        t = re.search(r"_MT(\w+?)_", name)
        mi = re.search(r"_MI(\w+?)_", name)
        return "hipBLASLt %s MT%s MI%s" % (name.split("_")[0], t.group(1) if t else "?",
                                            mi.group(1) if mi else "?")
    return "copyBuffer" if "copyBuffer" in name else None


def summarize_traffic(fetch_csv, write_csv, cmd_fetch, cmd_write):
    """rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs -> TRAFFIC_FILE."""
    import csv
    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = _short_kernel(r["Kernel_Name"])
            if k:
                acc.setdefault(k, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        # the calibration copy (--calibrate-copy) is the first copyBuffer
        # dispatch of the run; later ones are other blocks' copies
        return {k: (min(v)[1] if k == "copyBuffer" else sum(x for _, x in v) / len(v))
                for k, v in acc.items()}
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = float(1 << 20)                     # the 1 GiB calibration copy
    sf, sw = copy_kib / f["copyBuffer"], copy_kib / w["copyBuffer"]
    out = {"calibration": {"kernel": "__amd_rocclr_copyBuffer (1 GiB device copy)",
                           "FETCH_SIZE_KiB": f["copyBuffer"], "WRITE_SIZE_KiB": w["copyBuffer"],
                           "fetch_scale": sf, "write_scale": sw},
           "commands": [cmd_fetch, cmd_write], "kernels": {}}
    for k in sorted(set(f) & set(w)):
        if k == "copyBuffer" or k not in KERNEL_SOURCES:
            continue
        out["kernels"][k] = {"FETCH_SIZE_KiB": f[k], "WRITE_SIZE_KiB": w[k],
                             "read_bytes": f[k] * 1024 * sf, "write_bytes": w[k] * 1024 * sw,
                             "traffic_bytes": (f[k] * sf + w[k] * sw) * 1024,
                             "source_digest": source_digest(k)}
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("# HBM traffic per launch at the bench shape, from rocprofv3 FETCH_SIZE and "
                 "WRITE_SIZE (KiB per dispatch, averaged), scaled by the same counters on a "
                 "1 GiB copy; JSON below\n")
        fh.write(json.dumps(out, indent=1))
    return out


def summarize_pmc(sq_csv, tcc_csv, cmd_sq, cmd_tcc, out_md):
    """Two rocprofv3 --pmc counter CSVs -> clock, matrix-pipe and L2 summary."""
    import csv
    def per_kernel(path):
        acc, dur = {}, {}
        for r in csv.DictReader(open(path)):
            k = _short_kernel(r["Kernel_Name"])
            if not k or k == "copyBuffer":
                continue
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, {})[r["Dispatch_Id"]] = (float(r["End_Timestamp"]) -
                                                       float(r["Start_Timestamp"]))
        mean = lambda v: sum(v) / len(v)
        return ({k: {c: mean(v) for c, v in cs.items()} for k, cs in acc.items()},
                {k: mean(list(v.values())) for k, v in dur.items()})
    sq, dur = per_kernel(sq_csv)
    tcc, _ = per_kernel(tcc_csv)
    lines = ["# Clock, matrix pipe and L2 at the bench shape (rocprofv3 --pmc)", "",
             "Commands (`<repo>` = repository root, `<out>` = output directory):", "",
             "- `%s`" % cmd_sq, "- `%s`" % cmd_tcc, "",
             "Summary written by `python bench.py --summarize-pmc`.  Per kernel, averaged over its "
             "dispatches: clock = GRBM_GUI_ACTIVE / 8 XCDs / kernel time; matrix pipe busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8); waiting = "
             "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS). "
             "Kernel times are under the profiler.", "",
             "| kernel | time us | clock GHz | matrix pipe busy | waves waiting | L2 hit rate |",
             "|---|---|---|---|---|---|"]
    for k in sorted(sq):
        m, t = sq[k], tcc.get(k, {})
        if "GRBM_GUI_ACTIVE" not in m or k not in dur or dur[k] <= 0:
            continue
        active = m["GRBM_GUI_ACTIVE"] / 8
        hit = t.get("TCC_HIT_sum", 0.0)
        tot = hit + t.get("TCC_MISS_sum", 0.0)
        lines.append("| %s | %.0f | %.2f | %.3f | %.3f | %s |" % (
            k, dur[k] / 1e3, active / dur[k], m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / active,
            m["SQ_WAIT_INST_ANY"] / max(m["SQ_WAVE_CYCLES"], 1.0),
            ("%.3f" % (hit / tot)) if tot else "-"))
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_stats(stats_csv, cmd, out_md):
    """rocprofv3 --kernel-trace --stats kernel_stats.csv -> a short markdown table."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel time at the bench shape (rocprofv3 --kernel-trace --stats)", "",
             "Command (`<repo>` = repository root, `<out>` = output directory): `%s`" % cmd,
             "", "Summary written by `python bench.py --summarize-stats`.", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        k = _short_kernel(r["Name"])
        if not k or k == "copyBuffer":
            continue
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            k, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    open(out_md, "w").write("\n".join(lines) + "\n")


class Path:
    """Buffers and calls of one layer at one shape."""

    def __init__(self, shape, ids, gates, seed=0, policy=PLAN_POLICY):
        self.shape = s = shape
        self.policy = policy
        self.c = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
        dev = "cuda"
        self.ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
        self.gates = torch.from_numpy(np.ascontiguousarray(gates, np.float32)).to(dev)
        self.plan = mx.Plan(self.c, dev)
        self.x = W.randn_bf16((s.tokens, s.H), seed + 1, dev)
        self.w_home = W.randn_bf16((s.E, s.H, s.Hp), seed + 2, dev, chunk_rows=1)
        self.dy = W.randn_bf16((s.R * s.SK, s.Hp), seed + 3, dev)
        self.w_pref = torch.empty((s.R * s.B, s.H, s.Hp), dtype=torch.bfloat16, device=dev)
        self.xperm = torch.empty((s.R * s.SK, s.H), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((s.R * s.SK, s.Hp), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((s.tokens, s.Hp), dtype=torch.bfloat16, device=dev)
        self.gh = torch.zeros((s.E, s.H, s.Hp), dtype=torch.float32, device=dev)
        self.gp = torch.zeros((s.R * s.B, s.H, s.Hp), dtype=torch.float32, device=dev)
        self.ws = torch.empty(mx.moe_gemm_workspace_size(self.c), dtype=torch.uint8, device=dev)
        # data backward
        self.dout = W.randn_bf16((s.tokens, s.Hp), seed + 4, dev)
        self.dy_b = torch.empty((s.R * s.SK, s.Hp), dtype=torch.bfloat16, device=dev)
        self.dgates = torch.empty((s.tokens, s.K), dtype=torch.float32, device=dev)
        self.dxperm = torch.empty((s.R * s.SK, s.H), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((s.tokens, s.H), dtype=torch.bfloat16, device=dev)
        # dedup dispatch
        self.route_enc = torch.empty(s.tokens * s.K, dtype=torch.int32, device=dev)

    def backward_calls(self):
        c, p = self.c, self.plan
        return (
            ("combine_bwd", lambda: mx.moe_combine_backward(c, p, self.dout, self.y, self.gates,
                                                            self.dy_b, self.dgates)),
            ("dgrad", lambda: mx.moe_grouped_gemm_dgrad(c, self.dy_b, self.w_home, self.w_pref,
                                                        p.cu_seqlens, self.dxperm, 0,
                                                        self.shape.R, self.ws)),
            ("dispatch_bwd", lambda: mx.moe_dispatch_backward(c, p, self.dxperm, self.dx)),
        )

    def calls(self):
        c, p = self.c, self.plan
        return (
            ("plan", lambda: run_plan(c, self.ids, p, self.policy)),
            ("prefetch", lambda: mx.moe_prefetch_weight(c, p, self.w_home, self.w_pref)),
            ("dispatch", lambda: mx.moe_dispatch(c, p, self.x, self.xperm)),
            ("gemm", lambda: mx.moe_grouped_gemm(c, self.xperm, self.w_home, self.w_pref,
                                                 p.cu_seqlens, self.y, 0, self.shape.R, self.ws)),
            ("combine", lambda: mx.moe_combine(c, p, self.y, self.gates, self.out)),
            ("wgrad", lambda: mx.moe_grouped_gemm_wgrad(c, p, self.xperm, self.dy, self.gh,
                                                        self.gp, self.ws)),
            ("reduce_grad", lambda: mx.moe_reduce_grad(c, p, self.gh, self.gp)),
        )

    def run(self, steps, timed, only=None, backward=False):
        calls = [(n, f) for n, f in (self.backward_calls() if backward else self.calls())
                 if only is None or n in only]
        ev = []
        for _ in range(steps):
            row = []
            for name, f in calls:
                if timed:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    f()
                    b.record()
                    row.append((name, a, b))
                else:
                    f()
            ev.append(row)
        return ev


def work_units(shape, plan_views):
    """Algorithmic bytes / flops of each step (what the method must move)."""
    s = shape
    H, Hp, K, T = s.H, s.Hp, s.K, s.tokens
    slot_expert = plan_views["slot_expert"].cpu().numpy()
    n_slots = int((slot_expert >= 0).sum())
    n_cons = int(len(np.unique(slot_expert[slot_expert >= 0])))
    rows = s.R * s.SK
    return {
        "plan": ("bytes", 8.0 * rows),                       # read id, write route
        "prefetch": ("bytes", 2.0 * 2 * H * Hp * n_slots),   # read + write each slot
        "dispatch": ("bytes", float(T) * (2 * H * (1 + K) + 4 * K)),
        "gemm": ("flops", 2.0 * H * Hp * rows),
        "combine": ("bytes", float(T) * (2 * Hp * (K + 1) + 8 * K)),
        "wgrad": ("flops", 2.0 * H * Hp * rows),
        "reduce_grad": ("bytes", 8.0 * H * Hp * (n_slots + n_cons)),
        # data backward: read dout and K y rows, write K dy rows, gates/routes
        # in and gate gradients out; data-gradient GEMM; K rows in, one out
        "combine_bwd": ("bytes", float(T) * (2 * Hp * (1 + 2 * K) + 12 * K)),
        "dgrad": ("flops", 2.0 * H * Hp * rows),
        "dispatch_bwd": ("bytes", float(T) * (2 * H * (K + 1) + 4 * K)),
    }, {"slots": n_slots, "experts_with_slots": n_cons}


def cpu_baseline(shape, ids, gates, path, policy):
    """The oracle as it stands, on the host, scaled to one step.

    plan (``oracle.plan.make_plan``) and dispatch (``oracle.dataflow.dispatch``)
    run at full size; combine runs through the oracle's sampled form on a
    quarter of the tokens, reduce_grad through ``oracle.dataflow.reduce_grad``
    on 1/64 of every gradient row (all experts, all slots), the grouped GEMM
    through ``gemm_rows`` on 4096 sampled rows and the weight gradient through
    ``wgrad_entries`` on 4 segments x 512 h rows, each extrapolated to the
    step as stated in ``sample``.  The NumPy element-wise parts run on one
    thread; the float64 products on BLAS threads (capped at 8).
    """
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import bf16, dataflow
    from oracle.plan import Cfg, make_plan

    s = shape
    oc = Cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
    affinity = len(os.sched_getaffinity(0))
    blas = min(8, affinity)
    rng = np.random.default_rng(0)
    sec, note = {}, {}
    with threadpool_limits(limits=blas):
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
        t0 = time.perf_counter()
        ref = make_plan(ids, oc, policy)
        sec["plan"] = time.perf_counter() - t0
        note["plan"] = "full size"
        # dispatch at full size, on the step's x copied to the host
        xb = W.bf16_bits(path.x)
        t0 = time.perf_counter()
        dataflow.dispatch(xb, ref, oc)
        sec["dispatch"] = time.perf_counter() - t0
        note["dispatch"] = "full size"
        # combine: a quarter of the tokens, the step's generated dy as y rows
        yb = W.bf16_bits(path.dy)
        toks = np.sort(rng.choice(s.tokens, s.tokens // 4, replace=False))
        t0 = time.perf_counter()
        dataflow.combine_tokens(toks, yb, gates, ref, oc)
        sec["combine"] = (time.perf_counter() - t0) * s.tokens / toks.size
        note["combine"] = "combine_tokens on %d of %d tokens, x%d" % (toks.size, s.tokens,
                                                                      s.tokens // toks.size)
        del xb, yb
        # reduce_grad: every expert and slot, 1/64 of each [H, H'] gradient
        hs = s.H // 64
        gh = rng.standard_normal((s.E, hs, s.Hp)).astype(np.float32)
        gp = rng.standard_normal((s.R, s.B, hs, s.Hp)).astype(np.float32)
        t0 = time.perf_counter()
        dataflow.reduce_grad(gh, gp, ref, oc)
        sec["reduce_grad"] = (time.perf_counter() - t0) * 64
        note["reduce_grad"] = "reduce_grad on [:, :%d, :] of every gradient, x64" % hs
        del gh, gp
        # grouped GEMM: 4096 sampled rows (first and last row of sampled
        # segments plus seeded rows); the weight conversion is counted once
        # per active segment, the float64 product per row
        nz = [(r, int(j)) for r in range(s.R) for j in np.nonzero(ref.seg_len[r])[0]]
        pick = [nz[i] for i in rng.choice(len(nz), min(48, len(nz)), replace=False)]
        rows = []
        for r, j in pick:
            lo, hi = int(ref.cu_seqlens[r, j]), int(ref.cu_seqlens[r, j + 1])
            rows += [r * s.SK + lo, r * s.SK + hi - 1]
        while len(rows) < 4096:
            r, j = pick[int(rng.integers(len(pick)))]
            rows.append(r * s.SK + int(rng.integers(ref.cu_seqlens[r, j], ref.cu_seqlens[r, j + 1])))
        rows = np.unique(np.array(rows, np.int64))
        wr, xr = _DevRows(path.w_home), _DevRows(path.x)
        w0 = wr[0]
        t_conv = min(_timed(lambda: bf16.bits_to_f64(w0)) for _ in range(3))
        nseg = len(pick)
        t0 = time.perf_counter()
        dataflow.gemm_rows(rows, xr, wr, _OraclePref(wr, ref), ref, oc)
        t_rows = time.perf_counter() - t0
        per_row = max(t_rows - nseg * t_conv, 0.0) / rows.size
        sec["gemm"] = t_conv * len(nz) + per_row * s.R * s.SK
        note["gemm"] = ("gemm_rows on %d rows of %d segments (%.1fs); extrapolated as %d active "
                        "segments x %.3fs weight conversion + %d rows x %.2fms"
                        % (rows.size, nseg, t_rows, len(nz), t_conv, s.R * s.SK, per_row * 1e3))
        # weight gradient: 4 home segments, 512 h rows each
        home = [(r, j) for r, j in nz if j < s.E]
        wpick = [home[i] for i in rng.choice(len(home), 4, replace=False)]
        dr = _DevRows(path.dy)
        nh = 512
        t0 = time.perf_counter()
        nrows = 0
        for r, j in wpick:
            hsel = np.sort(rng.choice(s.H, nh, replace=False))
            dataflow.wgrad_entries(r, j, hsel, xr, dr, ref, oc)
            nrows += int(ref.seg_len[r, j])
        t_w = time.perf_counter() - t0
        sec["wgrad"] = t_w * (s.H / nh) * (s.R * s.SK) / max(nrows, 1)
        note["wgrad"] = ("wgrad_entries on %d segments (%d rows) x %d of %d h rows (%.1fs); "
                         "extrapolated per h row and per segment row" % (len(wpick), nrows, nh,
                                                                         s.H, t_w))
    total = sum(sec.values())
    return {
        "value": s.tokens / total,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("oracle on the host, one step extrapolated to %.1fs: " % total +
                   "; ".join("%s %s (%.2fs)" % (k, note[k], sec[k]) for k in sec)),
        "seconds": sec,
        "threads": {"plan": 1, "dispatch": 1, "combine": 1, "reduce_grad": 1,
                    "gemm": int(blas_threads), "wgrad": int(blas_threads)},
        "host_cpus": {"affinity": affinity, "cpu_count": os.cpu_count(),
                      "blas_threads": int(blas_threads)},
    }


def _timed(f):
    t0 = time.perf_counter()
    f()
    return time.perf_counter() - t0


class _OraclePref:
    def __init__(self, w, plan):
        self.w, self.plan = w, plan

    def __getitem__(self, rb):
        return self.w[int(self.plan.slot_expert[rb[0], rb[1]])]


class _DevRows:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, i):
        if np.isscalar(i):
            return W.bf16_bits(self.t[int(i)])
        return W.bf16_bits(self.t.index_select(0, torch.as_tensor(np.asarray(i),
                                                                  device=self.t.device)))


def measure(path, steps, warmup):
    path.run(warmup, timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = path.run(steps, timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [] for n in STEPS}
    for row in ev:
        for name, a, b in row:
            per[name].append(a.elapsed_time(b))
    ms = {n: float(np.mean(v)) for n, v in per.items() if v}
    stats = {n: {"mean": float(np.mean(v)), "median": float(np.median(v)),
                 "min": float(np.min(v))} for n, v in per.items() if v}
    span = ev[0][0][1].elapsed_time(ev[-1][-1][2])
    return ms, span / steps, wall / steps * 1e3, stats


def step_summary(path, ms, span_ms):
    """Per-step figures of one measured configuration of the step."""
    units, st = work_units(path.shape, path.plan.views())
    v = path.plan.views()
    status = v["status"].cpu().numpy()
    out = {"step_ms": span_ms, "ms": ms, "redundant_slots": st["slots"],
           "max_redundant": int(v["n_redundant"].max().item()), "moves": int(status[1]),
           "plan_us": ms["plan"] * 1e3}
    for name in ("prefetch", "dispatch", "combine", "reduce_grad"):
        out[name + "_GBps"] = units[name][1] / ms[name] / 1e6 if ms[name] > 0 else None
    for name in ("gemm", "wgrad"):
        out[name + "_TFLOPs"] = units[name][1] / ms[name] / 1e9
    return out


def measure_policy(path, policy, steps):
    """The whole step with another planner policy on the same routing; the
    step's own policy is restored afterwards."""
    saved = path.policy
    path.policy = policy
    ms, span, _, _ = measure(path, steps, 2)
    out = {"policy": POLICY_NAMES[policy]}
    out.update(step_summary(path, ms, span))
    path.policy = saved
    path.run(1, timed=False)
    torch.cuda.synchronize()
    return out


def measure_sweep(path, routings, steps):
    """The whole step at every maxvio of the bench sweep (one shared seed:
    only the Zipf strength changes), with both planner policies -- the pages'
    comparison of communication time under growing skew.  Restores the
    step's routing afterwards."""
    saved = (path.ids, path.gates, path.policy)
    out = {}
    for t, (ids2, gates2, s_bias, mv2) in routings.items():
        path.ids = torch.from_numpy(np.ascontiguousarray(ids2, np.int32)).cuda()
        path.gates = torch.from_numpy(np.ascontiguousarray(gates2, np.float32)).cuda()
        row = {"maxvio": mv2, "zipf_s": s_bias}
        for p, name in POLICY_NAMES.items():
            path.policy = p
            ms, span, _, _ = measure(path, steps, 1)
            row[name] = step_summary(path, ms, span)
        out["%g" % t] = row
        log("sweep", t, {k: (v["step_ms"], v["redundant_slots"]) for k, v in row.items()
                         if isinstance(v, dict)})
    path.ids, path.gates, path.policy = saved
    path.run(1, timed=False)
    torch.cuda.synchronize()
    return out


def measure_theorem2(path, steps):
    """The Theorem-2 worst case at the bench shape (round-robin routing over
    the experts of ranks 1..7, gates 1/K): the training step with B = 48
    (rank 0 receives 42 experts from one donor, 168 slots in all), and the
    inference forward with B = 4 (four slots per rank, the other redundant
    experts read from their home rows).  Restores the step's routing and plan
    afterwards.
    """
    s, dev = path.shape, "cuda"
    saved = (path.ids, path.gates)
    path.ids = torch.from_numpy(np.ascontiguousarray(W.routing_theorem2(s), np.int32)).to(dev)
    path.gates = torch.from_numpy(W.gates_uniform(s)).to(dev)
    ms, span, _, _ = measure(path, steps, 1)
    units, stats = work_units(s, path.plan.views())
    nred = path.plan.views()["n_redundant"].cpu().numpy().tolist()
    out = {"workload": "bench shape, Theorem-2 routing (slot i -> expert E/R + i mod (E - E/R)), "
                       "gates 1/K",
           "train": {"n_redundant": nred, "slots": stats["slots"], "step_ms": span,
                     "ms": ms,
                     "prefetch_GB": units["prefetch"][1] / 1e9,
                     "prefetch_GBps": units["prefetch"][1] / ms["prefetch"] / 1e6,
                     "reduce_grad_GB": units["reduce_grad"][1] / 1e9,
                     "reduce_grad_GBps": units["reduce_grad"][1] / ms["reduce_grad"] / 1e6,
                     "gemm_TFLOPs": units["gemm"][1] / ms["gemm"] / 1e9,
                     "wgrad_TFLOPs": units["wgrad"][1] / ms["wgrad"] / 1e9}}
    # inference, B = 4: the step's buffers with a 4-slot view of w_pref
    ci = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, 4, mx.MODE_INFER)
    pi = mx.Plan(ci, dev)
    wpi = path.w_pref[:s.R * 4]
    calls = (("plan", lambda: run_plan(ci, path.ids, pi, path.policy)),
             ("prefetch", lambda: mx.moe_prefetch_weight(ci, pi, path.w_home, wpi)),
             ("dispatch", lambda: mx.moe_dispatch(ci, pi, path.x, path.xperm)),
             ("gemm", lambda: mx.moe_grouped_gemm(ci, path.xperm, path.w_home, wpi,
                                                  pi.cu_seqlens, path.y, 0, s.R, path.ws)),
             ("combine", lambda: mx.moe_combine(ci, pi, path.y, path.gates, path.out)))
    for _, f in calls:
        f()
    torch.cuda.synchronize()
    ts = {n: [] for n, _ in calls}
    for _ in range(steps):
        for n, f in calls:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts[n].append(a.elapsed_time(b))
    v = pi.views()
    out["inference_B4"] = {
        "ms": {n: float(np.mean(t)) for n, t in ts.items()},
        "n_redundant": v["n_redundant"].cpu().numpy().tolist(),
        "gemm_TFLOPs": units["gemm"][1] / float(np.mean(ts["gemm"])) / 1e9}
    path.ids, path.gates = saved
    run_plan(path.c, path.ids, path.plan, path.policy)
    mx.moe_prefetch_weight(path.c, path.plan, path.w_home, path.w_pref)
    mx.moe_dispatch(path.c, path.plan, path.x, path.xperm)
    torch.cuda.synchronize()
    return out


def measure_dedup(path, steps):
    """Route encoding and the two-phase dispatch, beside the plain dispatch."""
    s, c, p = path.shape, path.c, path.plan
    enc_f = lambda: mx.moe_route_encode(c, p, path.route_enc)
    disp_f = lambda: mx.moe_dispatch_dedup(c, path.route_enc, path.x, path.xperm)
    for f in (enc_f, disp_f):
        f()
    torch.cuda.synchronize()
    ts = {"route_encode": [], "dispatch_dedup": []}
    for _ in range(steps):
        for name, f in (("route_encode", enc_f), ("dispatch_dedup", disp_f)):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts[name].append(a.elapsed_time(b))
    enc = path.route_enc.view(-1, s.K).cpu().numpy().astype(np.int64)
    route = p.views()["route"].cpu().numpy().reshape(-1, s.K).astype(np.int64)
    src = (np.arange(s.tokens) // s.S)[:, None]
    off_rank = (route // s.SK) != src
    sent = enc >= 0
    n_slots = route.size
    d_total = int(sent.sum())
    row = 2.0 * s.H
    ms_d = float(np.mean(ts["dispatch_dedup"]))
    algo = s.tokens * row + d_total * row + (n_slots - d_total) * 2 * row + 4.0 * n_slots
    return {
        "route_encode_us": float(np.mean(ts["route_encode"])) * 1e3,
        "dispatch_dedup_ms": ms_d,
        "dispatch_dedup_GBps": algo / (ms_d * 1e-3) / 1e9,
        "payload_rows": {"plain": int(n_slots), "dedup": d_total},
        "cross_rank_payload_GB": {"plain": float(off_rank.sum()) * row / 1e9,
                                  "dedup": float((off_rank & sent).sum()) * row / 1e9},
        "note": "on one GPU the send pass writes one row per (token, rank) and the receive "
                "pass copies the repeats locally; cross_rank_payload_GB is what would cross "
                "xGMI links with one rank per GPU",
    }


def measure_swiglu(path, steps):
    """Kernels of the two-projection SwiGLU expert at the bench shape.

    H' = 2048 is the intermediate size: W13 [E+B, 7168, 4096] (gate | up),
    W2 [E+B, 2048, 7168].  Times the fused first projection with and without
    the stored h13, the plain grouped GEMM over the same [H, 2H'] weights
    (same flops, plain epilogue), the second projection and the activation
    backward, each averaged over ``steps`` launches after one warm-up.
    """
    s, p, c = path.shape, path.plan, path.c
    Hi, dev, rows = s.Hp, "cuda", s.R * s.SK
    bf = dict(dtype=torch.bfloat16, device=dev)
    c13 = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, 2 * Hi, s.B, s.mode)
    c2 = mx.make_cfg(s.R, s.S, s.E, s.K, Hi, s.H, s.B, s.mode)
    w13 = W.randn_bf16((s.E, s.H, 2 * Hi), 11, dev, chunk_rows=1)
    w13p = torch.empty((s.R * s.B, s.H, 2 * Hi), **bf)
    w2 = W.randn_bf16((s.E, Hi, s.H), 12, dev, chunk_rows=1)
    w2p = torch.empty((s.R * s.B, Hi, s.H), **bf)
    act, h13, dh13 = (torch.empty((rows, Hi), **bf), torch.empty((rows, 2 * Hi), **bf),
                      torch.empty((rows, 2 * Hi), **bf))
    y2 = torch.empty((rows, s.H), **bf)
    dact = W.randn_bf16((rows, Hi), 13, dev)
    ws = torch.empty(max(mx.moe_gemm_workspace_size(x) for x in (c13, c2)), dtype=torch.uint8,
                     device=dev)
    mx.moe_prefetch_weight(c13, p, w13, w13p)
    mx.moe_prefetch_weight(c2, p, w2, w2p)
    flop_up, flop_down = 2.0 * s.H * 2 * Hi * rows, 2.0 * Hi * s.H * rows
    calls = (
        ("swiglu_gemm", "k_gemm<3>", "flops", flop_up,
         lambda: mx.moe_grouped_gemm_swiglu(c, path.xperm, w13, w13p, p.cu_seqlens, act, h13,
                                            0, s.R, ws)),
        ("swiglu_gemm_act_only", "k_gemm<3>", "flops", flop_up,
         lambda: mx.moe_grouped_gemm_swiglu(c, path.xperm, w13, w13p, p.cu_seqlens, act, None,
                                            0, s.R, ws)),
        ("plain_gemm_2h", "k_gemm<0>", "flops", flop_up,
         lambda: mx.moe_grouped_gemm(c13, path.xperm, w13, w13p, p.cu_seqlens, h13, 0, s.R, ws)),
        ("down_gemm", "k_gemm<0>", "flops", flop_down,
         lambda: mx.moe_grouped_gemm(c2, act, w2, w2p, p.cu_seqlens, y2, 0, s.R, ws)),
        # read h13 and d act, write d h13
        ("swiglu_bwd", "k_swiglu_bwd", "bytes", 10.0 * Hi * rows,
         lambda: mx.moe_swiglu_backward(c, h13, dact, dh13)),
    )
    out = {"workload": "bench shape, SwiGLU expert: W13 [E+B, 7168, 4096] (gate | up), "
                       "W2 [E+B, 2048, 7168], %d rows" % rows}
    for name, kern, kind, amount, f in calls:
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = float(np.mean(ts))
        if kind == "flops":
            ach = amount / (ms * 1e-3) / 1e12
            out[name] = {"kernel": kern, "bound": "mfma", "ms": ms, "achieved": ach,
                         "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                         "frac": ach / BF16_PEAK_TFLOPS}
        else:
            ach = amount / (ms * 1e-3) / 1e9
            out[name] = {"kernel": kern, "bound": "hbm", "ms": ms, "achieved": ach,
                         "unit": "GB/s", "peak": HBM_PEAK_GBPS, "frac": ach / HBM_PEAK_GBPS}
    del w13, w13p, w2, w2p, act, h13, dh13, y2, dact, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_pool(path, reps):
    """Two layers of one projection sharing one prefetch pool, backward pass.

    The pages' prefetch slots come from one pool shared by all layers: here
    w_pref and grad_pref of the step serve two layers.  Layer 0 (fresh
    weights and activations, Theorem-2 routing: the most slots) and layer 1
    (the step's own buffers and plan) run forward in order, so the pool ends
    with layer 1's slots.  Their backward runs layer 1 then layer 0; before
    layer 0's data-gradient GEMM its slots must be prefetched again.  Timed
    two ways: the re-prefetch serialized on the compute stream, and on a
    second stream that starts once layer 1's data-gradient GEMM (the last
    reader of the slots) is done, meant to overlap layer 1's weight gradient,
    reduce_grad and dispatch backward.  (It cannot: the persistent GEMM
    keeps one 512-register wave on every SIMD, so no other kernel's waves fit
    on any CU until it ends; "hidden_ms" measures what overlap there is.)
    """
    s, c, dev = path.shape, path.c, "cuda"
    bf = dict(dtype=torch.bfloat16, device=dev)
    rows = s.R * s.SK
    L0 = {"ids": torch.from_numpy(np.ascontiguousarray(W.routing_theorem2(s), np.int32)).to(dev),
          "gates": torch.from_numpy(W.gates_uniform(s)).to(dev), "plan": mx.Plan(c, dev),
          "x": W.randn_bf16((s.tokens, s.H), 21, dev),
          "w": W.randn_bf16((s.E, s.H, s.Hp), 22, dev, chunk_rows=1),
          "dout": W.randn_bf16((s.tokens, s.Hp), 23, dev),
          "xperm": torch.empty((rows, s.H), **bf), "y": torch.empty((rows, s.Hp), **bf),
          "out": torch.empty((s.tokens, s.Hp), **bf),
          "gh": torch.zeros((s.E, s.H, s.Hp), dtype=torch.float32, device=dev)}
    L1 = {"ids": path.ids, "gates": path.gates, "plan": path.plan, "x": path.x,
          "w": path.w_home, "dout": path.dout, "xperm": path.xperm, "y": path.y, "out": path.out,
          "gh": path.gh}
    w_pool, g_pool, ws = path.w_pref, path.gp, path.ws
    compute, copy = torch.cuda.current_stream(), torch.cuda.Stream()   # default priority
    run_plan(c, L0["ids"], L0["plan"], path.policy)
    for L in (L0, L1):
        mx.moe_prefetch_weight(c, L["plan"], L["w"], w_pool)
        mx.moe_dispatch(c, L["plan"], L["x"], L["xperm"])
        mx.moe_grouped_gemm(c, L["xperm"], L["w"], w_pool, L["plan"].cu_seqlens, L["y"], 0, s.R,
                            ws)
        mx.moe_combine(c, L["plan"], L["y"], L["gates"], L["out"])
    torch.cuda.synchronize()

    def layer_bwd_head(L):
        mx.moe_combine_backward(c, L["plan"], L["dout"], L["y"], L["gates"], path.dy_b,
                                path.dgates)
        mx.moe_grouped_gemm_dgrad(c, path.dy_b, L["w"], w_pool, L["plan"].cu_seqlens,
                                  path.dxperm, 0, s.R, ws)

    def layer_bwd_tail(L):
        mx.moe_grouped_gemm_wgrad(c, L["plan"], L["xperm"], path.dy_b, L["gh"], g_pool, ws)
        mx.moe_reduce_grad(c, L["plan"], L["gh"], g_pool)
        mx.moe_dispatch_backward(c, L["plan"], path.dxperm, path.dx)

    def backward(overlap):
        layer_bwd_head(L1)
        if overlap:
            released, filled = torch.cuda.Event(), torch.cuda.Event()
            released.record(compute)
            copy.wait_event(released)
            mx.moe_prefetch_weight(c, L0["plan"], L0["w"], w_pool, stream=copy)
            filled.record(copy)
            layer_bwd_tail(L1)
            compute.wait_event(filled)
        else:
            layer_bwd_tail(L1)
            mx.moe_prefetch_weight(c, L0["plan"], L0["w"], w_pool)
        layer_bwd_head(L0)
        layer_bwd_tail(L0)

    out = {"workload": "two layers of one projection at the bench shape sharing one slot buffer "
                       "[R*B, 7168, 2048] bf16 and one reduce buffer (fp32): 33.8 GB in all, "
                       "instead of 33.8 GB per layer; layer 0 Theorem-2 routing, layer 1 the "
                       "step's routing; backward of both layers"}
    sv = {k: L["plan"].views()["slot_expert"].cpu().numpy() for k, L in (("layer0", L0),
                                                                         ("layer1", L1))}
    out["slots"] = {k: int((v >= 0).sum()) for k, v in sv.items()}
    out["reprefetch_GB"] = 4.0 * s.H * s.Hp * out["slots"]["layer0"] / 1e9
    for name, overlap in (("serialized", False), ("overlapped", True), ("serialized_2", False),
                          ("overlapped_2", True)):
        ts = []
        for _ in range(reps + 1):
            mx.moe_prefetch_weight(c, L1["plan"], L1["w"], w_pool)    # pool back to layer 1
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(compute)
            backward(overlap)
            b.record(compute)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[name + "_ms"] = float(np.mean(ts[1:]))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(compute)
    mx.moe_prefetch_weight(c, L0["plan"], L0["w"], w_pool)
    b.record(compute)
    torch.cuda.synchronize()
    out["reprefetch_alone_ms"] = a.elapsed_time(b)
    ser = (out["serialized_ms"] + out["serialized_2_ms"]) / 2
    ovl = (out["overlapped_ms"] + out["overlapped_2_ms"]) / 2
    out["hidden_ms"] = ser - ovl
    # leave the step's buffers as they were: the pool holds layer 1's slots
    mx.moe_prefetch_weight(c, L1["plan"], L1["w"], w_pool)
    del L0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _time_calls(f, reps):
    f()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        f()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def measure_ceilings(reps=5, gib=4):
    """Context for the HBM fractions: what plain device kernels reach on this
    card (torch's own copy, fill and sum over 4 GiB; not the path): a copy
    reads and writes every byte, a fill only writes, a sum only reads."""
    n = gib << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    av = a.view(torch.float32)
    out = {"workload": "%d GiB buffers; median of %d calls" % (gib, reps)}
    t = _time_calls(lambda: b.copy_(a), reps)
    out["copy_GBps"] = 2.0 * n / t / 1e6
    t = _time_calls(lambda: b.fill_(3), reps)
    out["fill_GBps"] = 1.0 * n / t / 1e6
    t = _time_calls(lambda: av.sum(), reps)
    out["read_GBps"] = 1.0 * n / t / 1e6
    out["note"] = ("torch device kernels on this card, for context; nothing on the path uses "
                   "them; read_GBps is torch's sum, a reduction kernel rather than a pure read")
    del a, b, av
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_vendor(path, reps):
    """Context for the GEMM's roofline fraction: the same product shape as one
    rank's work (65,536 rows x H=7168 -> H'=2048, 1.924 TFLOP) as (a) this
    library's kernel on a single segment (a one-rank, one-expert layout),
    (b) hipBLASLt through torch.matmul on the same operands (a comparator
    only; nothing on the path calls it), and (c) this library's grouped GEMM
    on rank 0 of the step's plan (ragged segments)."""
    s, dev = path.shape, "cuda"
    rows = s.SK
    flops = 2.0 * rows * s.H * s.Hp
    c1 = mx.make_cfg(1, rows, 1, 1, s.H, s.Hp, 0, mx.MODE_INFER)
    cu1 = torch.tensor([0, rows], dtype=torch.int32, device=dev)
    ws1 = torch.empty(mx.moe_gemm_workspace_size(c1), dtype=torch.uint8, device=dev)
    xp = path.xperm[:rows]
    w0 = path.w_home[0]
    y1 = torch.empty((rows, s.Hp), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty_like(y1)
    ours = _time_calls(lambda: mx.moe_grouped_gemm(c1, xp, path.w_home[:1], None, cu1, y1, 0, 1,
                                                   ws1), reps)
    vendor = _time_calls(lambda: torch.matmul(xp, w0, out=y2), reps)
    grouped = _time_calls(lambda: mx.moe_grouped_gemm(path.c, path.xperm, path.w_home,
                                                      path.w_pref, path.plan.cu_seqlens, path.y,
                                                      0, 1, path.ws), reps)
    torch.cuda.synchronize()
    same = bool(torch.allclose(y1.float()[:4096], y2.float()[:4096], rtol=2e-2, atol=2e-2))
    out = {"workload": "one rank's product shape: [65536, 7168] x [7168, 2048] bf16, fp32 "
                       "accumulation, bf16 output (1.924 TFLOP); median of %d calls" % reps,
           "this_library_one_segment": {"ms": ours, "TFLOPs": flops / ours / 1e9},
           "hipblaslt_torch_matmul": {"ms": vendor, "TFLOPs": flops / vendor / 1e9,
                                      "note": "comparator only, not on the path"},
           "this_library_rank0_grouped": {"ms": grouped, "TFLOPs": flops / grouped / 1e9,
                                          "note": "rank 0 of the step's plan, ragged segments"},
           "outputs_agree_first_4096_rows": same}
    del y1, y2, ws1
    return out


def measure_graph(path, reps):
    """The step captured once as a HIP graph (static shapes, no host sync in
    any call) and replayed, against the same calls issued eagerly: at the
    bench shape (the whole training step) and at the tiny and skewed shapes
    (plan -> prefetch -> dispatch -> GEMM -> combine), where launches weigh
    most.  Median of ``reps`` after a warm-up.
    """
    out = {}
    step = lambda: path.run(1, timed=False)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    out["bench_step"] = {"eager_ms": _time_calls(step, reps), "graph_ms": _time_calls(g.replay, reps)}
    dev = "cuda"
    for s, t in ((W.TINY, None), (W.SKEWED, 1.0)):
        c = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
        ids, gates = W.routing_uniform(s) if t is None else W.routing_zipf(s, t)[:2]
        bf = dict(dtype=torch.bfloat16, device=dev)
        ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
        g_t = torch.from_numpy(np.ascontiguousarray(gates, np.float32)).to(dev)
        plan = mx.Plan(c, dev)
        x, w = W.randn_bf16((s.tokens, s.H), 41, dev), W.randn_bf16((s.E, s.H, s.Hp), 42, dev)
        wp = torch.empty((s.R * s.B, s.H, s.Hp), **bf)
        xp, y = torch.empty((s.R * s.SK, s.H), **bf), torch.empty((s.R * s.SK, s.Hp), **bf)
        o = torch.empty((s.tokens, s.Hp), **bf)
        ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device=dev)

        def fwd():
            run_plan(c, ids_t, plan, PLAN_POLICY)
            mx.moe_prefetch_weight(c, plan, w, wp)
            mx.moe_dispatch(c, plan, x, xp)
            mx.moe_grouped_gemm(c, xp, w, wp, plan.cu_seqlens, y, 0, s.R, ws)
            mx.moe_combine(c, plan, y, g_t, o)
        fwd()
        torch.cuda.synchronize()
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            fwd()
        torch.cuda.synchronize()
        out[s.name + "_forward"] = {"eager_us": _time_calls(fwd, reps) * 1e3,
                                    "graph_us": _time_calls(gs.replay, reps) * 1e3}
    return out


def measure_small(reps):
    """The tiny (R=4, S=16, E=8, K=2, H=128, H'=64) and skewed (R=8, S=1024,
    E=64, K=4, H=1024, H'=512; zipf maxvio 0.2 / 1 / 10 / 15) shapes: the
    forward path's calls in microseconds.  Their working sets fit in the
    256 MB memory-side cache, so no HBM fraction is claimed.
    """
    dev = "cuda"
    out = {"note": "working sets fit in the memory-side cache: times only, no HBM fraction"}
    cases = [(W.TINY, None)] + [(W.SKEWED, t) for t in W.MAXVIO_SWEEP["skewed"]]
    for s, t in cases:
        c = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
        if t is None:
            ids, gates = W.routing_uniform(s)
            name = "tiny"
        else:
            ids, gates, _, _ = W.routing_zipf(s, t)
            name = "skewed_maxvio_%g" % t
        bf = dict(dtype=torch.bfloat16, device=dev)
        ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
        g_t = torch.from_numpy(np.ascontiguousarray(gates, np.float32)).to(dev)
        plan = mx.Plan(c, dev)
        x = W.randn_bf16((s.tokens, s.H), 41, dev)
        w = W.randn_bf16((s.E, s.H, s.Hp), 42, dev)
        wp = torch.empty((max(1, s.R * s.B), s.H, s.Hp), **bf)
        xp = torch.empty((s.R * s.SK, s.H), **bf)
        y = torch.empty((s.R * s.SK, s.Hp), **bf)
        o = torch.empty((s.tokens, s.Hp), **bf)
        ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device=dev)
        calls = (("plan", lambda: run_plan(c, ids_t, plan, PLAN_POLICY)),
                 ("prefetch", lambda: mx.moe_prefetch_weight(c, plan, w, wp)),
                 ("dispatch", lambda: mx.moe_dispatch(c, plan, x, xp)),
                 ("gemm", lambda: mx.moe_grouped_gemm(c, xp, w, wp, plan.cu_seqlens, y, 0, s.R,
                                                      ws)),
                 ("combine", lambda: mx.moe_combine(c, plan, y, g_t, o)))
        for _, f in calls:
            f()
        torch.cuda.synchronize()
        ts = {n: [] for n, _ in calls}
        for _ in range(reps):
            for n, f in calls:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                f()
                b.record()
                torch.cuda.synchronize()
                ts[n].append(a.elapsed_time(b) * 1e3)
        out[name] = {n + "_us": float(np.median(v)) for n, v in ts.items()}
    return out


def measure_schedule(reps):
    """The forward and data-gradient GEMMs where the tile-class schedule
    acts: the bench's experts (E=384, K=8, H=7168, H'=2048) at decode sizes
    (S = 256, 1024, 2048 tokens per rank: about 42, 168 and 335 rows per
    segment) and the skewed shape at maxvio 15, each planned by moe_plan_run
    from zipf routing (maxvio 1 for the decode sizes).  Reports the median of
    ``reps`` calls and the scheduler's choice for the step, read from the
    workspace header: row tiles per class launch (4: any tile, 2: at most
    128 rows, 1: at most 64 rows), the folds taken and the predicted time.
    """
    dev = "cuda"
    out = {"note": "class 4 tiles multiply all 8 MFMA row blocks, class 2 four, class 1 two; "
                   "small classes run as their own launches only when segments average under "
                   "512 rows"}
    cases = [("decode_S256", W.BENCH.with_(name="decode256", S=256), 1.0),
             ("decode_S1024", W.BENCH.with_(name="decode1024", S=1024), 1.0),
             ("decode_S2048", W.BENCH.with_(name="decode2048", S=2048), 1.0),
             ("skewed_maxvio15", W.SKEWED, 15.0)]
    for name, s, t in cases:
        c = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
        ids, _, _, mv = W.routing_zipf(s, t)
        plan = mx.Plan(c, dev)
        mx.moe_plan_run(c, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev), plan)
        bf = dict(dtype=torch.bfloat16, device=dev)
        x = W.randn_bf16((s.tokens, s.H), 51, dev)
        w = W.randn_bf16((s.E, s.H, s.Hp), 52, dev, chunk_rows=1)
        dy = W.randn_bf16((s.R * s.SK, s.Hp), 53, dev)
        wp = torch.empty((s.R * s.B, s.H, s.Hp), **bf)
        xp = torch.empty((s.R * s.SK, s.H), **bf)
        y = torch.empty((s.R * s.SK, s.Hp), **bf)
        dxp = torch.empty((s.R * s.SK, s.H), **bf)
        ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device=dev)
        mx.moe_prefetch_weight(c, plan, w, wp)
        mx.moe_dispatch(c, plan, x, xp)
        fwd = lambda: mx.moe_grouped_gemm(c, xp, w, wp, plan.cu_seqlens, y, 0, s.R, ws)
        dgr = lambda: mx.moe_grouped_gemm_dgrad(c, dy, w, wp, plan.cu_seqlens, dxp, 0, s.R, ws)
        tf = _time_calls(fwd, reps)
        hf = ws[:20].view(torch.int32).cpu().tolist()
        tb = _time_calls(dgr, reps)
        hb = ws[:20].view(torch.int32).cpu().tolist()
        flop = 2.0 * s.H * s.Hp * s.R * s.SK
        seg = np.diff(plan.views()["cu_seqlens"].cpu().numpy(), axis=1)
        nseg = int((seg > 0).sum())
        dec = lambda h: {"class4_row_tiles": h[0], "class2_row_tiles": h[1],
                         "class1_row_tiles": h[2],
                         "folded": {"class2_into_4": bool(h[3] & 1), "class1": bool(h[3] & 2),
                                    "class1_into_4": bool(h[3] & 4)},
                         "predicted_ms": h[4] * 1e-6}
        out[name] = {"maxvio": mv, "segments": nseg, "rows_per_segment": s.R * s.SK / nseg,
                     "forward_ms": tf, "forward_TFLOPs": flop / tf / 1e9,
                     "forward_weight_GBps": nseg * s.H * s.Hp * 2.0 / tf / 1e6,
                     "forward_schedule": dec(hf),
                     "dgrad_ms": tb, "dgrad_TFLOPs": flop / tb / 1e9, "dgrad_schedule": dec(hb)}
        log("schedule", name, {k: v for k, v in out[name].items() if "schedule" not in k})
        del x, w, dy, wp, xp, y, dxp, ws, plan
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def measure_large_e(reps):
    """The Large-E shape: R=64 virtual ranks, S=4096, E=896, K=16, H=7168,
    H'=2048, B=14, train mode, zipf maxvio 1 and 10.

    Plan, dispatch and combine run over all 64 ranks; the grouped GEMM of
    one rank -- the one with the most active segments (ties: lowest id), and
    rank 0 -- against its [910, 7168, 2048] view (896 home rows + its 14
    prefetch rows).  Each call is timed with HIP events, mean of ``reps``
    calls after one warm-up.
    """
    s, dev = W.LARGE_E, "cuda"
    c = mx.make_cfg(s.R, s.S, s.E, s.K, s.H, s.Hp, s.B, s.mode)
    bf = dict(dtype=torch.bfloat16, device=dev)
    rows = s.R * s.SK
    x = W.randn_bf16((s.tokens, s.H), 31, dev)
    w_home = W.randn_bf16((s.E, s.H, s.Hp), 32, dev, chunk_rows=1)
    w_pref = torch.empty((s.R * s.B, s.H, s.Hp), **bf)
    xperm = torch.empty((rows, s.H), **bf)
    y = W.randn_bf16((rows, s.Hp), 33, dev)
    out = torch.empty((s.tokens, s.Hp), **bf)
    ws = torch.empty(mx.moe_gemm_workspace_size(c), dtype=torch.uint8, device=dev)
    plan = mx.Plan(c, dev)
    T = s.tokens

    def timed(f):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.mean(ts))

    res = {"workload": "Large-E: R=64 virtual ranks, S=4096 tokens/rank, E=896, K=16, H=7168, "
                       "H'=2048, B=14, train mode; plan/dispatch/combine over all ranks, grouped "
                       "GEMM of one rank's 65536 rows against its [910, 7168, 2048] view"}
    disp_b = T * (2.0 * s.H * (1 + s.K) + 4 * s.K)
    comb_b = T * (2.0 * s.Hp * (s.K + 1) + 8 * s.K)
    flop = 2.0 * s.H * s.Hp * s.SK
    for t in W.MAXVIO_SWEEP["large_e"]:
        ids, gates, _, mv = W.routing_zipf(s, t)
        ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
        g_t = torch.from_numpy(np.ascontiguousarray(gates, np.float32)).to(dev)
        r_plan = plan_latency(s, t, ids=ids, maxvio=mv)
        run_plan(c, ids_t, plan, PLAN_POLICY)
        mx.moe_prefetch_weight(c, plan, w_home, w_pref)
        torch.cuda.synchronize()
        seg = np.diff(plan.views()["cu_seqlens"].cpu().numpy(), axis=1)
        active = (seg > 0).sum(axis=1)
        r_hot = int(np.argmax(active))
        ms_d = timed(lambda: mx.moe_dispatch(c, plan, x, xperm))
        ms_c = timed(lambda: mx.moe_combine(c, plan, y, g_t, out))
        ms_g = timed(lambda: mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y,
                                                 r_hot, r_hot + 1, ws))
        ms_g0 = timed(lambda: mx.moe_grouped_gemm(c, xperm, w_home, w_pref, plan.cu_seqlens, y,
                                                  0, 1, ws))
        res["maxvio_%g" % t] = {
            "maxvio": mv, "plan_us": r_plan["plan_us_median"],
            "max_redundant": r_plan["max_redundant"],
            "dispatch_ms": ms_d, "dispatch_GBps": disp_b / ms_d / 1e6,
            "dispatch_frac": disp_b / ms_d / 1e6 / HBM_PEAK_GBPS,
            "combine_ms": ms_c, "combine_GBps": comb_b / ms_c / 1e6,
            "combine_frac": comb_b / ms_c / 1e6 / HBM_PEAK_GBPS,
            "gemm_rank": r_hot, "gemm_rank_active_segments": int(active[r_hot]),
            "gemm_ms": ms_g, "gemm_TFLOPs": flop / ms_g / 1e9,
            "gemm_frac": flop / ms_g / 1e9 / BF16_PEAK_TFLOPS,
            "gemm_rank0_ms": ms_g0, "gemm_rank0_TFLOPs": flop / ms_g0 / 1e9}
        log("large_e", t, res["maxvio_%g" % t])
    del x, w_home, w_pref, xperm, y, out, ws, plan
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_backward(path, steps, warmup):
    path.run(warmup, timed=False, backward=True)
    torch.cuda.synchronize()
    ev = path.run(steps, timed=True, backward=True)
    torch.cuda.synchronize()
    per = {}
    for row in ev:
        for name, a, b in row:
            per.setdefault(name, []).append(a.elapsed_time(b))
    return {n: float(np.mean(v)) for n, v in per.items()}


def plan_latency(shape, target, runs=20, policy=PLAN_POLICY, ids=None, maxvio=None):
    """Plan µs (every planner launch) at one routing of one shape; ``maxvio``
    is the achieved maxvio of ``ids`` when they are passed in."""
    mv = maxvio
    if ids is None:
        ids, _, _, mv = W.routing_zipf(shape, target)
    c = mx.make_cfg(shape.R, shape.S, shape.E, shape.K, shape.H, shape.Hp, shape.B, shape.mode)
    plan = mx.Plan(c)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    for _ in range(3):
        run_plan(c, ids_t, plan, policy)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(runs):
        a.record()
        run_plan(c, ids_t, plan, policy)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    v = plan.views()
    st = v["status"].cpu().numpy()
    return {"maxvio": mv, "plan_us_median": float(np.median(ts)), "plan_us_min": float(min(ts)),
            "fills": int(st[0]), "moves": int(st[1]), "status": int(st[2]),
            "max_redundant": int(v["n_redundant"].max().item())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--maxvio", type=float, default=1.0)
    ap.add_argument("--no-sweep", action="store_true", help="skip the maxvio sweep (the step "
                    "with both planner policies at maxvio 0.2 / 1 / 10 / 20)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the blocks after the step's own (small shapes, graph replay, "
                         "Theorem-2, SwiGLU expert, prefetch pool, vendor GEMM context, Large-E: "
                         "they launch the step's kernels at other shapes; profiles of the step "
                         "use this)")
    ap.add_argument("--vendor-only", action="store_true",
                    help="plan and dispatch once, then only the vendor GEMM context block")
    ap.add_argument("--swiglu-only", action="store_true",
                    help="plan and dispatch once, then only the SwiGLU-expert block")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                          "CMD_FETCH", "CMD_WRITE"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "CMD", "OUT_MD"),
                    help="write a kernel-time summary from rocprofv3 --stats and exit")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("SQ_CSV", "TCC_CSV", "CMD_SQ", "CMD_TCC",
                                                      "OUT_MD"),
                    help="write the clock / matrix-pipe / L2 summary from two --pmc runs and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(*args.summarize_traffic)["calibration"]))
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the R expert-parallel ranks are virtual ranks "
              "inside one GPU's memory; --gpus %d is not supported" % args.gpus)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mx.load()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    shape = W.BENCH
    log("routing: zipf maxvio target", args.maxvio)
    ids, gates, s_bias, mv = W.routing_zipf(shape, args.maxvio)
    log("allocating and generating inputs")
    path = Path(shape, ids, gates)
    torch.cuda.synchronize()
    if args.vendor_only:
        path.run(1, timed=False, only=("plan", "prefetch", "dispatch"))
        torch.cuda.synchronize()
        print(json.dumps({"vendor_gemm_context": measure_vendor(path, 8)}), flush=True)
        return
    if args.swiglu_only:
        path.run(1, timed=False, only=("plan", "dispatch"))
        torch.cuda.synchronize()
        print(json.dumps({"swiglu_expert": measure_swiglu(path, max(3, args.steps // 4))}),
              flush=True)
        return
    log("warmup + timed steps")
    ms, span_ms, wall_ms, step_stats = measure(path, args.steps, args.warmup)
    st = path.plan.views()["status"].cpu().numpy()
    if st[2] != 0:
        raise RuntimeError("plan status bits %d" % st[2])
    units, plan_stats = work_units(shape, path.plan.views())
    comps = {}
    roof = []
    for name in STEPS:
        kind, amount = units[name]
        t = ms[name] * 1e-3
        if kind == "flops":
            ach = amount / t / 1e12
            roof.append({"step": name, "bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "ms": ms[name]})
            comps[name + "_TFLOPs"] = ach
        else:
            ach = amount / t / 1e9
            bound = "latency" if name == "plan" else "hbm"
            roof.append({"step": name, "bound": bound, "achieved": ach, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "ms": ms[name]})
            comps[name + "_GBps"] = ach
    comps["plan_us"] = ms["plan"] * 1e3
    step_kernel = {"gemm": "k_gemm<0>", "wgrad": "k_wgrad", "dispatch": "k_dispatch",
                   "combine": "k_combine", "prefetch": "k_prefetch",
                   "reduce_grad": "k_reduce_grad", "plan": None}
    for r in roof:
        k = step_kernel[r["step"]]
        r["traffic"] = measured_traffic(k) if k else None
    dom = max((r for r in roof if r["step"] != "plan"), key=lambda r: r["ms"])
    kernel_of = {"gemm": "k_gemm<0> (grouped GEMM, 256x256 MFMA tiles)",
                 "wgrad": "k_wgrad (weight-grad GEMM, 384x256 MFMA tiles)",
                 "dispatch": "k_dispatch", "combine": "k_combine",
                 "prefetch": "k_prefetch", "reduce_grad": "k_reduce_grad"}
    gemm_units = units[dom["step"]][1]
    dom_kernel = {"gemm": "k_gemm<0>", "wgrad": "k_wgrad", "dispatch": "k_dispatch",
                  "combine": "k_combine", "prefetch": "k_prefetch",
                  "reduce_grad": "k_reduce_grad"}[dom["step"]]
    roofline = {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                "unit": dom["unit"], "frac": dom["frac"],
                "traffic": measured_traffic(dom_kernel),
                "kernel": kernel_of[dom["step"]],
                "algorithmic_per_launch": gemm_units, "avg_launch_ms": dom["ms"]}
    line = {
        "metric": METRIC,
        "value": shape.tokens / (span_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": span_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bench shape: R=8 virtual ranks, S=8192 tokens/rank, E=384, K=8, "
                               "H=7168, H'=2048, B=48, train mode, zipf routing maxvio %.3f, "
                               "planner moe_plan_run (ascending Theorem-1 construction)" % mv,
                   "R": shape.R, "S": shape.S, "E": shape.E, "K": shape.K, "H": shape.H,
                   "Hp": shape.Hp, "B": shape.B, "maxvio": mv, "zipf_s": s_bias,
                   "redundant_slots": plan_stats["slots"], "planner": POLICY_NAMES[PLAN_POLICY]},
        "components": comps,
        "step_ms": ms,
        "step_ms_stats": step_stats,
        "wall_ms_per_step": wall_ms,
        "roofline": roofline,
        "rooflines": roof,
    }
    log("HBM ceilings of plain device kernels (context)")
    line["hbm_ceilings"] = measure_ceilings()
    log("the step with the largest-first planner")
    line["step_largest_first"] = measure_policy(path, mx.PLAN_LARGEST_FIRST,
                                                max(3, args.steps // 2))
    log("planner policies at the bench shape")
    routings = {t: W.routing_zipf(shape, t) for t in W.MAXVIO_SWEEP["bench"]}
    pol = {}
    for t in W.MAXVIO_SWEEP["bench"]:
        ids_t2, _, _, mv_t = routings[t]
        pol["maxvio_%g" % t] = {
            name: plan_latency(shape, t, policy=p, ids=ids_t2, maxvio=mv_t)
            for p, name in POLICY_NAMES.items()}
    line["plan_policies"] = pol
    if not args.no_sweep:
        log("maxvio sweep, both planner policies")
        line["maxvio_sweep"] = measure_sweep(path, routings, max(3, args.steps // 4))
    log("plan latency at the Large-E shape")
    le = {"workload": "Large-E: R=64, S=4096, E=896, K=16, B=14 (plan only)"}
    for t in W.MAXVIO_SWEEP["large_e"]:
        ids_le, _, _, mv_le = W.routing_zipf(W.LARGE_E, t)
        le["maxvio_%g" % t] = {
            name: plan_latency(W.LARGE_E, t, policy=p, ids=ids_le, maxvio=mv_le)
            for p, name in POLICY_NAMES.items()}
    line["plan_large_e"] = le
    log("data backward")
    bms = measure_backward(path, max(3, args.steps // 2), 1)
    bwd = []
    for name, kern in (("combine_bwd", "k_combine_bwd"), ("dgrad", "k_gemm<2>"),
                       ("dispatch_bwd", "k_dispatch_bwd")):
        kind, amount = units[name]
        t = bms[name] * 1e-3
        if kind == "flops":
            ach = amount / t / 1e12
            bwd.append({"step": name, "kernel": kern, "bound": "mfma", "achieved": ach,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / BF16_PEAK_TFLOPS, "ms": bms[name]})
        else:
            ach = amount / t / 1e9
            bwd.append({"step": name, "kernel": kern, "bound": "hbm", "achieved": ach,
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                        "ms": bms[name]})
    line["data_backward"] = bwd
    log("dedup dispatch")
    line["dedup_dispatch"] = measure_dedup(path, max(3, args.steps // 2))
    if not args.no_extras:
        log("vendor GEMM context (one rank's product shape)")
        line["vendor_gemm_context"] = measure_vendor(path, 5)
        log("tiny and skewed shapes")
        line["small_shapes"] = measure_small(10)
        log("graph capture and replay")
        line["graph_replay"] = measure_graph(path, 10)
        log("theorem-2 worst case (train B=48, inference B=4)")
        line["theorem2"] = measure_theorem2(path, max(3, args.steps // 4))
        log("swiglu expert")
        line["swiglu_expert"] = measure_swiglu(path, max(3, args.steps // 4))
        log("prefetch pool (two layers, backward)")
        line["prefetch_pool"] = measure_pool(path, 2)
        log("GEMM tile-class schedule at decode sizes and under skew")
        line["gemm_schedule"] = measure_schedule(10)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host, bounded sample)")
        line["cpu_baseline"] = cpu_baseline(shape, ids, gates, path, PLAN_POLICY)
    if not args.no_extras:
        log("large-E shape (the step's buffers released first)")
        del path
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["large_e"] = measure_large_e(5)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
