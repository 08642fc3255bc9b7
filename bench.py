#!/usr/bin/env python3
"""Benchmark of the Q8_0 GEMV / sparse-MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--act int8|f32|x2]

A step is one pass of the hot path over one batch of synthetic input.  The
headline workload is the batch-1 MoE FFN block at the Qwen3-30B-A3B-like shape
(d 2048, dff 768, 128 experts, top 8) in one-word int8 numerics, fed by its
producer, as one moe_ffn_block call a step (add + norm fused into the router's
logits, the top-K taken inside the gate-up launch, then down-combine);
--separate runs the same block as the separate calls

    add_rmsnorm_q8 -> moe_route_topk -> moe_gate_up -> moe_down_combine

Inputs are resident in HBM before timing starts.  Weight reads are kept
cache-cold: the steps rotate over `copies` copies of every weight array (more
bytes between two uses of a copy than two 256 MB Infinity Caches hold) and
over a pool of different input rows (so the chosen experts change from step
to step).

Timing: exactly W untimed steps, then exactly K timed steps, each run as one
HIP graph of that many consecutive steps (step i on copy i mod C); HIP events
on the graph's stream bracket the K steps, with a device synchronisation on
both sides.  The spread (p10 / median / p90) comes from --spread single steps,
each timed alone between two events.  Each of the step's calls is then timed
alone (a graph of its launches, one per copy, replayed back to back), beside
the time the library's plain streaming reader (q8s_stream_read) takes for the
same weight bytes, cold.  The dominant kernel's average launch time gives the
roofline object, on its algorithmic bytes (the weight bytes one launch must
read) against the 8 TB/s HBM peak.

By default the run goes on to every other workload and numerics (the suite),
each with the same measurements at 400 steps, into config.workloads; the CPU
oracle is timed on a bounded sample of the headline workload, on one core and
on every available core at once (one thread each).  --warm (context only)
keeps one weight copy and one input row, so the weights stay cache-resident.

Prints one JSON line on stdout; details go to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs and effective HBM GB/s per batch-1 MoE FFN block / Q8_0 GEMV (% of peak)"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
ACT_CODE = {"f32": 0, "int8": 1, "x2": 2}  # the library's activation modes
# the oracle tolerance of each mode's output (two words: one 128th of a
# one-word code flip, with a margin of 16 flips)
TOL = {"f32": 1e-5, "int8": 2e-3, "x2": 2.5e-4}
MALL_BYTES = 256 << 20
DEFAULT_WORKLOAD = "moe_d2048_dff768_e128_k8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# dominant kernel of each workload kind, and the sources that define it
DOMINANT = {
    "moe": ("k_route_gate_up", ("q8_gemv_sparse_amd/csrc/q8s_moe.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")),
    "chunk": ("k_chunk_gate_up", ("q8_gemv_sparse_amd/csrc/q8s_moe_chunk.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")),
    "moe_shared": ("k_route_gate_up", ("q8_gemv_sparse_amd/csrc/q8s_moe.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")),
    "norm_gemv": ("k_norm_gemv", ("q8_gemv_sparse_amd/csrc/q8s_gemv.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h",
                                  "q8_gemv_sparse_amd/csrc/q8s_norm_row.h")),
}


def chunk_kernels(cfg, act):
    """The grouped gate-up and down kernels a chunk workload runs (the
    library's own rule: q8s_moe_path)."""
    import q8_gemv_sparse_amd as q8
    path = q8.q8s_moe_path(cfg["rows"], cfg["d"], cfg["dff"], cfg["E"], cfg["k"], ACT_CODE[act])
    if path == q8.PATH_GROUPED_MFMA:
        return "k_grouped_mfma", "k_grouped_mfma"
    if path != q8.PATH_GROUPED:
        raise SystemExit("workload %s does not run the grouped chunk kernels" % cfg)
    return "k_chunk_gate_up", ("k_chunk_down2" if cfg["dff"] <= 1024 else "k_chunk_down")


def kernel_pattern(kernel):
    """The dispatches a counter file covers: the kernel's instantiations, or
    for the matrix-core grouped kernel only its gate-up (PAIR) ones."""
    if kernel == "k_grouped_mfma":
        return r"q8s::k_grouped_mfma<\d+, true, (true|false)>"
    return r"q8s::%s\b" % kernel


def counters_path(kernel, workload, act):
    return os.path.join(ROOT, "profiles", "%s_%s_%s_counters.txt" % (kernel, workload, act))


def summarize_counters(args):
    """Turns two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE; counter_collection.csv files, KiB per dispatch) into the HBM
    bytes one launch of the workload's dominant kernel moves.  Each counter is
    scaled by what it reads for the run's plain device copy of known size
    (--calib-copy-mib): the last copy dispatch of that size."""
    import csv
    import re
    import synthetic
    cfg = synthetic.CONFIGS[args.workload]
    kernel, srcs = DOMINANT[cfg["kind"]]
    if cfg["kind"] == "chunk":
        kernel = chunk_kernels(cfg, args.act)[0]
    calib = args.calib_copy_mib * 1024  # KiB moved each way by the copy
    run = ("python3 bench.py --workload %s --act %s --no-graph --steps 28 --warmup 14 --kernel-launches 14 "
           "--spread 0 --suite none --no-cpu --no-ceiling --calib-copy-mib %d"
           % (args.workload, args.act, args.calib_copy_mib))
    out = {"kernel": kernel, "workload": args.workload, "act": args.act,
           "source_digest": src_digest(*srcs), "calib_copy_kib": calib,
           "commands": ["rocprofv3 --pmc %s -f csv -d <out> -o run -- %s" % (c, run)
                        for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                       ["python3 bench.py --workload %s --act %s --calib-copy-mib %d --summarize-counters "
                        "<FETCH_SIZE counter_collection.csv> <WRITE_SIZE counter_collection.csv>"
                        % (args.workload, args.act, args.calib_copy_mib)]}
    for counter, path in (("FETCH_SIZE", args.summarize_counters[0]), ("WRITE_SIZE", args.summarize_counters[1])):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        mine = [float(r["Counter_Value"]) for r in rows if re.search(kernel_pattern(kernel), r["Kernel_Name"])]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        # the calibration copy is the run's last copy dispatch
        ref = copies[-1]
        scale = calib / ref
        out[counter] = {"dispatches": len(mine), "kib_per_dispatch": sum(mine) / len(mine),
                        "copy_kib": ref, "scale": scale,
                        "scaled_bytes_per_dispatch": sum(mine) / len(mine) * scale * 1024}
    out["hbm_bytes_per_launch"] = int(out["FETCH_SIZE"]["scaled_bytes_per_dispatch"] +
                                      out["WRITE_SIZE"]["scaled_bytes_per_dispatch"])
    dst = counters_path(kernel, args.workload, args.act)
    with open(dst, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--act", choices=["int8", "f32", "x2"], default="int8",
                   help="activation numerics: one-word int8, float32, or two-word int8 (norm + GEMV workload)")
    p.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough to defeat the MALL)")
    p.add_argument("--kernel-launches", type=int, default=400, help="launches timed for the dominant kernel")
    p.add_argument("--spread", type=int, default=200, help="single steps timed one by one for the spread (0: none)")
    p.add_argument("--suite", choices=["auto", "all", "none"], default="auto",
                   help="after the headline, measure every other workload and numerics into config.workloads "
                        "(auto: only for the default headline)")
    p.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for the CPU baseline")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads for the all-cores oracle run (0: every CPU available; 1: single-core only)")
    p.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    p.add_argument("--warm", action="store_true",
                   help="context only: every step on weight copy 0 and input row 0, so the weights stay cache-resident")
    p.add_argument("--ceiling-only", action="store_true",
                   help="measure only the streaming-read ceiling (2 GiB and the default workload's gate-up bytes)")
    p.add_argument("--no-graph", action="store_true",
                   help="launch every step eagerly instead of replaying a captured graph (for counter runs, which "
                        "profile each dispatch)")
    p.add_argument("--separate", action="store_true",
                   help="the separate calls a step instead of one moe_ffn_block / add_rmsnorm_gemv call")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU run: summarise two counter passes of this script into the traffic file")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (a known-size kernel for counter scaling)")
    return p.parse_args()


def src_digest(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workloads


class Workload:
    name = ""
    dominant = ""          # kernel symbol stem of the dominant kernel
    dominant_src = ()      # sources that define it (for the counter-file check)
    dominant_timed = "the dominant kernel alone"  # what the graph of its launches runs

    def step(self, c):
        raise NotImplementedError

    def launch_dominant(self, c):
        raise NotImplementedError

    def prepare_dominant(self):
        """Anything the dominant kernel's launches read that the steps leave
        elsewhere (called once before they are captured)."""


_MOE_MEMO = {}


def _moe_inputs(d, dff, E, k):
    """synthetic.moe_inputs(seed 0) of one shape, kept for the next workload
    of the same shape (the suite measures each shape in several numerics)."""
    import synthetic
    key = (d, dff, E, k)
    if key not in _MOE_MEMO:
        _MOE_MEMO.clear()
        _MOE_MEMO[key] = synthetic.moe_inputs(0, d, dff, E, k, rows=1)
    return _MOE_MEMO[key]


def _copies(step_bytes, want):
    """Weight copies to rotate so that more than two MALLs' worth of weight
    traffic passes between two uses of one copy."""
    if want:
        return want
    return max(2, min(64, -(-(2 * MALL_BYTES) // max(step_bytes, 1)) + 1))


class MoeBlock(Workload):
    """The mixture block of a layer, `rows` rows: add + norm -> router + top-K
    -> gate-up -> down-combine.  By default one moe_ffn_block call a step
    (three launches: norm fused into the router, top-K inside gate-up,
    down-combine); with separate=True the five calls add_rmsnorm_q8,
    moe_route_topk, moe_gate_up, moe_down_combine (five launches)."""

    dominant_src = ("q8_gemv_sparse_amd/csrc/q8s_moe.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")

    def __init__(self, name, cfg, act, copies, rows=1, pool=64, separate=False):
        import numpy as np
        import torch

        import q8_gemv_sparse_amd as q8
        import synthetic
        self.q8, self.torch, self.np = q8, torch, np
        self.name, self.act = name, act
        self.separate = separate
        self.dominant = "k_gate_up" if separate else "k_route_gate_up"
        d, dff, E, k = cfg["d"], cfg["dff"], cfg["E"], cfg["k"]
        self.d, self.dff, self.E, self.k, self.rows = d, dff, E, k, rows
        t0 = time.time()
        m = _moe_inputs(d, dff, E, k)
        self.host_w = m
        rng = np.random.default_rng(1)
        self.norm_w = rng.uniform(0.5, 1.5, size=d).astype(np.float32)
        self.pool_h = [synthetic.normal(rng, rows, d) for _ in range(pool)]
        self.pool_r = [synthetic.normal(rng, rows, d) for _ in range(pool)]
        log("[bench] generated inputs in %.1fs" % (time.time() - t0))
        per_expert = 3 * dff * d + 3 * dff * (d // 32) * 4
        self.bytes_all = E * d * 4 + E * per_expert
        # rotate enough copies that a copy was last touched more than two
        # MALLs of traffic ago
        step_bytes = E * d * 4 + min(E, rows * k) * per_expert
        self.copies = copies or _copies(step_bytes, 0)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [dev(a) for a in (m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)]
        self.W = [base] + [[t.clone() for t in base] for _ in range(self.copies - 1)]
        self.w = dev(self.norm_w)
        self.h = [dev(a) for a in self.pool_h]
        self.r = [dev(a) for a in self.pool_r]
        self.pool = pool
        z = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device="cuda")
        self.sum = z(rows, d)
        self.y = z(rows, d)
        self.xq, self.xs = z(rows, d, dt=torch.int8), z(rows, d // 32)
        self.xl = z(rows, d, dt=torch.int8)  # two words: the low words of x and of the hidden rows
        self.idx = [z(rows, k, dt=torch.int32) for _ in range(self.copies)]
        self.wts = [z(rows, k) for _ in range(self.copies)]
        self.hf = z(rows, k, dff)
        self.hq, self.hs = z(rows, k, dff, dt=torch.int8), z(rows, k, dff // 32)
        self.hl = z(rows, k, dff, dt=torch.int8)
        self.out = z(rows, d)
        self.rscratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_ROUTE, rows, d, dff, E, k), dtype=torch.uint8,
                                    device="cuda")
        dn = q8.q8s_scratch_bytes(q8.FN_DOWN, rows, d, dff, E, k)
        self.dscratch = torch.zeros(dn, dtype=torch.uint8, device="cuda") if dn else None
        a = ACT_CODE[act]
        self.bscratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_BLOCK, rows, d, dff, E, k, a), dtype=torch.uint8,
                                    device="cuda")
        self.logits = [z(rows, E, dt=torch.float64) for _ in range(self.copies)]
        torch.cuda.synchronize()
        log("[bench] %s: %d weight copies of %.1f MB on the device" % (name, self.copies, self.bytes_all / 1e6))

    # one pass; copy c, input c % pool
    def step(self, c):
        q8 = self.q8
        W = self.W[c % self.copies]
        i = c % self.pool
        a = ACT_CODE[self.act]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        if not self.separate:
            q8.moe_ffn_block(self.h[i], self.r[i], self.w, 1e-6, *W, self.k, act=a, sum=self.sum, idx=idx, wts=wts,
                             out=self.out, scratch=self.bscratch)
            return
        self._norm(c)
        self._mixture(c)

    def _norm(self, c):
        q8 = self.q8
        i = c % self.pool
        a = ACT_CODE[self.act]
        q8.add_rmsnorm_q8(self.h[i], self.r[i], self.w, 1e-6, sum=self.sum, y=self.y,
                          yq=self.xq if a == q8.ACT_INT8 else None, ys=self.xs if a == q8.ACT_INT8 else None,
                          want_q8=(a == q8.ACT_INT8))

    def _mixture(self, c):
        """The separate calls after the norm: route, gate-up, down-combine."""
        q8 = self.q8
        W = self.W[c % self.copies]
        a = ACT_CODE[self.act]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        q8.moe_route_topk(self.y, W[0], self.k, idx=idx, wts=wts, scratch=self.rscratch)
        self._gate_up(c, a)
        if a == q8.ACT_INT8:
            q8.moe_down_combine(W[5], W[6], idx, wts, self.E, hq=self.hq, hs=self.hs, y=self.out, act=a,
                                scratch=self.dscratch)
        else:
            q8.moe_down_combine(W[5], W[6], idx, wts, self.E, h=self.hf, y=self.out, act=a, scratch=self.dscratch)

    def _gate_up(self, c, a):
        q8 = self.q8
        W = self.W[c % self.copies]
        idx = self.idx[c % self.copies]
        if a == q8.ACT_INT8:
            q8.moe_gate_up(W[1], W[2], W[3], W[4], idx, self.E, xq=self.xq, xs=self.xs, hq=self.hq, hs=self.hs,
                           h=self.hf if self.rows > 1 else None, act=a, want_h=False)
        else:
            q8.moe_gate_up(W[1], W[2], W[3], W[4], idx, self.E, x=self.y, h=self.hf, act=a)

    def prepare_dominant(self):
        """The fused gate-up reads router logits: form each copy's from its
        own input row (as its steps do), so its choices rotate like theirs."""
        if self.separate:
            return
        q8 = self.q8
        for c in range(self.copies):
            i = c % self.pool
            x2 = self.act == "x2"
            q8.add_rmsnorm_router(self.h[i], self.r[i], self.w, 1e-6, self.W[c][0], sum=self.sum, x=self.y,
                                  xq=None if x2 else self.xq, xs=None if x2 else self.xs, logits=self.logits[c],
                                  want_q8=not x2)
            if x2:
                q8.q8_quantize_rows_x2(self.y, xq=self.xq, xl=self.xl, xs=self.xs)
        self.torch.cuda.synchronize()

    def launch_dominant(self, c):
        q8 = self.q8
        a = ACT_CODE[self.act]
        if self.separate:
            self._gate_up(c, a)
            return
        W = self.W[c % self.copies]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        if a == ACT_CODE["x2"]:
            q8.moe_topk_gate_up_x2(self.logits[c % self.copies], W[1], W[2], W[3], W[4], self.k, self.xq, self.xl,
                                   self.xs, idx=idx, wts=wts, hq=self.hq, hl=self.hl, hs=self.hs)
        elif a == q8.ACT_INT8:
            q8.moe_topk_gate_up(self.logits[c % self.copies], W[1], W[2], W[3], W[4], self.k, xq=self.xq, xs=self.xs,
                                idx=idx, wts=wts, hq=self.hq, hs=self.hs, act=a, want_h=False)
        else:
            q8.moe_topk_gate_up(self.logits[c % self.copies], W[1], W[2], W[3], W[4], self.k, x=self.y, idx=idx,
                                wts=wts, h=self.hf, act=a)

    def stages(self):
        """The step's launches, each as a call of its own (one kernel each
        for one row): (label, launch(c), weight bytes of one launch)."""
        q8 = self.q8
        a = ACT_CODE[self.act]
        d, dff, E, k = self.d, self.dff, self.E, self.k
        q8b = lambda n_out, n_in: n_out * n_in + n_out * (n_in // 32) * 4
        if self.separate or self.rows > 1:
            return []

        def norm_router(c):
            i = c % self.pool
            x2 = self.act == "x2"
            q8.add_rmsnorm_router(self.h[i], self.r[i], self.w, 1e-6, self.W[c % self.copies][0], sum=self.sum,
                                  x=self.y, xq=None if x2 else self.xq, xs=None if x2 else self.xs,
                                  logits=self.logits[c % self.copies], want_q8=not x2)

        def down(c):
            W = self.W[c % self.copies]
            idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
            if a == q8.ACT_INT8:
                q8.moe_down_combine(W[5], W[6], idx, wts, E, hq=self.hq, hs=self.hs, y=self.out, act=a)
            else:
                q8.moe_down_combine(W[5], W[6], idx, wts, E, h=self.hf, y=self.out, act=a)
        out = [("add_rmsnorm_router (k_norm_logits)", norm_router, E * d * 4),
               ("moe_topk_gate_up (k_route_gate_up)", self.launch_dominant, k * 2 * q8b(dff, d))]
        if self.act != "x2":  # the two-word down projection runs inside moe_ffn_block only
            out.append(("moe_down_combine (k_down)", down, k * q8b(d, dff)))
        return out

    def distinct_experts(self, c):
        """Experts chosen by copy c's last route (for the bytes a chunk reads)."""
        return int(self.torch.unique(self.idx[c % self.copies]).numel())

    def weight_bytes(self, c=None):
        """Weight bytes one step must read: the router and each distinct chosen
        expert's gate, up and down (quants + scales)."""
        d, dff, E = self.d, self.dff, self.E
        per_expert = 3 * (dff * d + dff * (d // 32) * 4)
        u = self.k if self.rows == 1 else self.distinct_experts(c)
        return E * d * 4 + u * per_expert

    def dominant_bytes(self, c=None):
        d, dff = self.d, self.dff
        u = self.k if self.rows == 1 else self.distinct_experts(c)
        return u * 2 * (dff * d + dff * (d // 32) * 4)

    def verify(self):
        """One eager step against the oracle (the same input, every stage)."""
        import oracle
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        m = self.host_w
        s, y64 = oracle.add_rmsnorm(self.pool_h[0], self.pool_r[0], self.norm_w, 1e-6)
        x = y64.astype(np.float32)
        a = ACT_CODE[self.act]
        ridx, rw, rh, ry = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a)
        got = self.out.cpu().numpy()
        err = float(np.max(np.abs(got - ry)) / np.max(np.abs(ry)))
        same_idx = bool(np.array_equal(self.idx[0].cpu().numpy(), ridx))
        return {"idx_equal": same_idx, "max_rel_err": err, "tol": TOL[self.act]}

    def cpu_baseline(self, budget):
        import oracle
        np = self.np
        m = self.host_w
        a = ACT_CODE[self.act]
        n, t0 = 0, time.perf_counter()
        while True:
            i = n % self.pool
            s, y64 = oracle.add_rmsnorm(self.pool_h[i], self.pool_r[i], self.norm_w, 1e-6)
            x = y64.astype(np.float32)
            if a == 2:
                oracle.quantize_x2(x)
            elif a:
                oracle.quantize(x)
            oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or n >= 100000:
                break
        per_step = el / n
        return per_step, "%d steps (rows %d, inputs from the same pool), %.1f s" % (n, self.rows, el)


class NormGemv(Workload):
    """The residual add + RMSNorm feeding the 2048 -> 4096 batch-1 projection:
    one add_rmsnorm_gemv call a step (one launch; add_rmsnorm_gemv_x2 in
    two-word numerics); with separate=True the calls add_rmsnorm_q8 ->
    q8_gemv (two words: add_rmsnorm_q8 -> q8_quantize_rows_x2 -> q8_gemv_x2)."""

    dominant_src = ("q8_gemv_sparse_amd/csrc/q8s_gemv.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h",
                    "q8_gemv_sparse_amd/csrc/q8s_norm_row.h")

    def __init__(self, name, cfg, act, copies, pool=64, separate=False):
        import numpy as np
        import torch

        import q8_gemv_sparse_amd as q8
        import synthetic
        self.q8, self.torch, self.np = q8, torch, np
        self.name, self.act = name, act
        # two words: add_rmsnorm_gemv_x2 (one launch), or with separate=True
        # add_rmsnorm_q8 (float32 row) -> q8_quantize_rows_x2 -> q8_gemv_x2
        self.separate = separate
        self.dominant = "k_gemv_rows" if self.separate else "k_norm_gemv"
        d, n_out = cfg["d"], cfg["n_out"]
        self.d, self.n_out = d, n_out
        inp = synthetic.norm_gemv_inputs(0, d, n_out, rows=1)
        self.inp = inp
        rng = np.random.default_rng(1)
        self.pool_h = [synthetic.normal(rng, 1, d) for _ in range(pool)]
        self.pool_r = [synthetic.normal(rng, 1, d) for _ in range(pool)]
        self.pool = pool
        wbytes = n_out * d + n_out * (d // 32) * 4
        self.copies = copies or _copies(wbytes, 0)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [dev(inp.Wq), dev(inp.Ws)]
        self.W = [base] + [[t.clone() for t in base] for _ in range(self.copies - 1)]
        self.w = dev(inp.w)
        self.h = [dev(a) for a in self.pool_h]
        self.r = [dev(a) for a in self.pool_r]
        z = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device="cuda")
        self.sum, self.y = z(1, d), z(1, d)
        self.xq, self.xs = z(1, d, dt=torch.int8), z(1, d // 32)
        self.xl = z(1, d, dt=torch.int8)
        self.out = z(1, n_out)
        self.wbytes = wbytes
        torch.cuda.synchronize()

    def step(self, c):
        q8 = self.q8
        i = c % self.pool
        a = q8.ACT_INT8 if self.act == "int8" else q8.ACT_F32
        if not self.separate and self.act == "x2":
            W = self.W[c % self.copies]
            q8.add_rmsnorm_gemv_x2(self.h[i], self.r[i], self.w, 1e-6, W[0], W[1], sum=self.sum, y=self.y,
                                   yq=self.xq, yl=self.xl, ys=self.xs, out=self.out)
            return
        if not self.separate:
            W = self.W[c % self.copies]
            q8.add_rmsnorm_gemv(self.h[i], self.r[i], self.w, 1e-6, W[0], W[1], act=a, sum=self.sum,
                                y=None if a else self.y, yq=self.xq if a else None, ys=self.xs if a else None,
                                out=self.out)
            return
        x2 = self.act == "x2"
        q8.add_rmsnorm_q8(self.h[i], self.r[i], self.w, 1e-6, sum=self.sum, y=self.y,
                          yq=self.xq if a and not x2 else None, ys=self.xs if a and not x2 else None,
                          want_q8=bool(a) and not x2)
        if x2:
            q8.q8_quantize_rows_x2(self.y, xq=self.xq, xl=self.xl, xs=self.xs)
        self.launch_dominant(c)

    def launch_dominant(self, c):
        q8 = self.q8
        if not self.separate:
            self.step(c)  # the step is the one fused launch
            return
        W = self.W[c % self.copies]
        if self.act == "x2":
            q8.q8_gemv_x2(W[0], W[1], self.xq, self.xl, self.xs, y=self.out)
        elif self.act == "int8":
            q8.q8_gemv(W[0], W[1], xq=self.xq, xs=self.xs, y=self.out, act=q8.ACT_INT8)
        else:
            q8.q8_gemv(W[0], W[1], x=self.y, y=self.out, act=q8.ACT_F32)

    def weight_bytes(self, c=None):
        return self.wbytes

    def dominant_bytes(self, c=None):
        return self.wbytes

    def stages(self):
        if self.separate:
            return [("q8_gemv (k_gemv_rows)", self.launch_dominant, self.wbytes)]
        return [("add_rmsnorm_gemv%s (k_norm_gemv)" % ("_x2" if self.act == "x2" else ""), self.step, self.wbytes)]

    def verify(self):
        import oracle
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        s, y64 = oracle.add_rmsnorm(self.pool_h[0], self.pool_r[0], self.inp.w, 1e-6)
        x = y64.astype(np.float32)
        if self.act == "x2":
            q, lo, sc = oracle.quantize_x2(x)
            ref = oracle.gemv_i8x2(self.inp.Wq, self.inp.Ws, q, lo, sc)
        elif self.act == "int8":
            q, sc = oracle.quantize(x)
            ref = oracle.gemv_i8(self.inp.Wq, self.inp.Ws, q, sc)
        else:
            ref = oracle.gemv_f32(self.inp.Wq, self.inp.Ws, x)
        got = self.out.cpu().numpy()
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        return {"max_rel_err": err, "tol": 2e-3 if self.act == "int8" else 1e-5}

    def cpu_baseline(self, budget):
        import oracle
        np = self.np
        n, t0 = 0, time.perf_counter()
        while True:
            i = n % self.pool
            s, y64 = oracle.add_rmsnorm(self.pool_h[i], self.pool_r[i], self.inp.w, 1e-6)
            x = y64.astype(np.float32)
            if self.act == "x2":
                q, lo, sc = oracle.quantize_x2(x)
                oracle.gemv_i8x2(self.inp.Wq, self.inp.Ws, q, lo, sc)
            elif self.act == "int8":
                q, sc = oracle.quantize(x)
                oracle.gemv_i8(self.inp.Wq, self.inp.Ws, q, sc)
            else:
                oracle.gemv_f32(self.inp.Wq, self.inp.Ws, x)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return el / n, "%d steps, %.1f s" % (n, el)


class Gemv(Workload):
    """One batch-1 Q8_0 GEMV a step, float32 activations (the 512 x 256
    matrix: 147 KB, which the caches hold; latency, not bandwidth, bounds
    it).  The step rotates over 64 weight copies and as many input rows."""

    dominant_src = ("q8_gemv_sparse_amd/csrc/q8s_gemv.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")
    dominant = "k_gemv_rows"

    def __init__(self, name, cfg, act, copies):
        import numpy as np
        import torch

        import q8_gemv_sparse_amd as q8
        import synthetic
        if act != "f32":
            raise SystemExit("workload %s is the float32-activation GEMV" % name)
        self.q8, self.torch, self.np = q8, torch, np
        self.name, self.act = name, act
        n_out, n_in = cfg["n_out"], cfg["n_in"]
        self.inp = synthetic.gemv_inputs(0, n_out, n_in, m=1)
        self.copies = copies or 64
        rng = np.random.default_rng(1)
        self.pool_x = [synthetic.normal(rng, 1, n_in) for _ in range(self.copies)]
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [dev(self.inp.Wq), dev(self.inp.Ws)]
        self.W = [base] + [[t.clone() for t in base] for _ in range(self.copies - 1)]
        self.x = [dev(a) for a in self.pool_x]
        self.out = torch.empty((1, n_out), dtype=torch.float32, device="cuda")
        self.wbytes = n_out * n_in + n_out * (n_in // 32) * 4
        self.cache = "warm: the 64 copies (9.4 MB) fit the Infinity Cache; a latency figure"
        torch.cuda.synchronize()

    def step(self, c):
        W = self.W[c % self.copies]
        self.q8.q8_gemv(W[0], W[1], x=self.x[c % self.copies], y=self.out, act=self.q8.ACT_F32)

    launch_dominant = step

    def weight_bytes(self, c=None):
        return self.wbytes

    dominant_bytes = weight_bytes

    def stages(self):
        return [("q8_gemv (k_gemv_rows)", self.step, self.wbytes)]

    def verify(self):
        import oracle
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        ref = oracle.gemv_f32(self.inp.Wq, self.inp.Ws, self.pool_x[0])
        got = self.out.cpu().numpy()
        return {"max_rel_err": float(np.max(np.abs(got - ref)) / np.max(np.abs(ref))), "tol": 1e-5}

    def cpu_baseline(self, budget):
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.gemv_f32(self.inp.Wq, self.inp.Ws, self.pool_x[n % self.copies])
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return el / n, "%d steps, %.1f s" % (n, el)


class ChunkBlock(MoeBlock):
    """A prefill chunk (64, 128 or 256 rows) through the MoE block (choices
    grouped by expert, int8 activations: the vector-unit grouped kernels at 4
    choices an expert, the matrix-core ones from 8), then the dense Q8_0
    projection of the same rows' Q8_0 form on the matrix cores."""

    dominant = "k_chunk_gate_up"
    dominant_src = ("q8_gemv_sparse_amd/csrc/q8s_moe_chunk.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")

    def __init__(self, name, cfg, act, copies):
        # the separate calls: the dense projection reads the chunk's Q8_0 rows
        # that add_rmsnorm_q8 writes (in two words: add_rmsnorm_q8_x2's
        # two-word form), and the grouped gate-up is the dominant kernel
        if act == "f32":
            raise SystemExit("workload %s runs in int8 numerics (one or two words)" % name)
        super().__init__(name, cfg, act, copies, rows=cfg["rows"], pool=8, separate=True)
        self.gu_kernel, self.dn_kernel = chunk_kernels(cfg, act)
        self.dominant = self.gu_kernel
        self.dominant_timed = "moe_gate_up without the hidden rows' Q8_0 pass: %s alone" % self.gu_kernel
        import synthetic
        np, torch = self.np, self.torch
        rng = np.random.default_rng(2)
        Dq, Ds = synthetic.q8_matrix(rng, cfg["n_dense"], cfg["d"])
        self.Dq_h, self.Ds_h = Dq, Ds
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [dev(Dq), dev(Ds)]
        self.D = [base] + [[t.clone() for t in base] for _ in range(self.copies - 1)]
        self.dense_out = torch.empty((cfg["rows"], cfg["n_dense"]), dtype=torch.float32, device="cuda")
        self.dense_bytes = cfg["n_dense"] * cfg["d"] + cfg["n_dense"] * (cfg["d"] // 32) * 4
        torch.cuda.synchronize()

    def step(self, c):
        # the dense projection reads the same normed rows as the router, so
        # one call runs both, the top-K inside the projection's launch (a
        # parallel graph branch for the projection instead, forked after the
        # norm and joined at the step's end, measured 173.2 against 161.7 us
        # a step: the fork and join cost more than the overlap gained)
        self._norm(c)
        self._route_dense(c)
        self._gate_up(c, None)
        self._down(c)

    def _route_dense(self, c):
        W, (Dq, Ds) = self.W[c % self.copies], self.D[c % self.copies]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        self.q8.moe_route_topk_gemv(self.y, W[0], self.k, Dq, Ds, self.xq, self.xs,
                                    xl=self.xl if self.act == "x2" else None, idx=idx, wts=wts, y=self.dense_out,
                                    scratch=self.rscratch)

    def _norm(self, c):
        if self.act != "x2":
            return super()._norm(c)
        i = c % self.pool
        self.q8.add_rmsnorm_q8_x2(self.h[i], self.r[i], self.w, 1e-6, sum=self.sum, y=self.y, yq=self.xq, yl=self.xl,
                                  ys=self.xs)

    def _gate_up(self, c, a, want_q8=True):
        if self.act != "x2":
            W = self.W[c % self.copies]
            return self.q8.moe_gate_up(W[1], W[2], W[3], W[4], self.idx[c % self.copies], self.E, xq=self.xq,
                                       xs=self.xs, hq=self.hq if want_q8 else None, hs=self.hs if want_q8 else None,
                                       h=self.hf, act=self.q8.ACT_INT8, want_q8=want_q8)
        W = self.W[c % self.copies]
        self.q8.moe_gate_up_x2(W[1], W[2], W[3], W[4], self.idx[c % self.copies], self.E, self.xq, self.xl, self.xs,
                               h=self.hf, hq=self.hq if want_q8 else None, hl=self.hl if want_q8 else None,
                               hs=self.hs if want_q8 else None, want_q8=want_q8)

    def _down(self, c):
        W = self.W[c % self.copies]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        if self.act == "x2":
            self.q8.moe_down_combine_x2(W[5], W[6], idx, wts, self.E, self.hq, self.hl, self.hs, y=self.out,
                                        scratch=self.dscratch)
        else:
            self.q8.moe_down_combine(W[5], W[6], idx, wts, self.E, hq=self.hq, hs=self.hs, y=self.out,
                                     act=self.q8.ACT_INT8, scratch=self.dscratch)

    def launch_dominant(self, c):
        # the grouped gate-up kernel alone: the float32 hidden rows, without
        # the quantise pass the step runs after it
        self._gate_up(c, None, want_q8=False)

    def weight_bytes(self, c=None):
        return super().weight_bytes(c) + self.dense_bytes

    def stages(self):
        """The chunk's calls in step order, each timed alone over the copies
        (the routing each copy's last step left in place)."""
        d, dff, E = self.d, self.dff, self.E
        q8b = lambda n_out, n_in: n_out * n_in + n_out * (n_in // 32) * 4
        u = lambda c: self.distinct_experts(c)
        C = self.copies
        avg_u = sum(u(c) for c in range(C)) / C

        x2 = self.act == "x2"
        sfx = "_x2" if x2 else ""
        rows, n_dense = self.rows, self.dense_out.shape[1]
        return [("add_rmsnorm_q8%s (k_add_rmsnorm_q8, %d rows)" % ("_x2" if x2 else "", rows), self._norm, 0),
                ("moe_route_topk_gemv%s: router + dense %d x %d -> %d (k_logits_tile + k_gemm_i8 carrying the "
                 "top-K)" % (" (two words)" if x2 else "", rows, d, n_dense), self._route_dense,
                 E * d * 4 + self.dense_bytes),
                ("moe_gate_up%s (%s + k_quantize_rows%s)" % (sfx, self.gu_kernel, sfx),
                 lambda c: self._gate_up(c, None), int(avg_u * 2 * q8b(dff, d))),
                ("moe_down_combine%s (%s + k_chunk_combine)" % (sfx, self.dn_kernel), self._down,
                 int(avg_u * q8b(d, dff)))]

    def verify(self):
        import oracle
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        m = self.host_w
        s, y64 = oracle.add_rmsnorm(self.pool_h[0], self.pool_r[0], self.norm_w, 1e-6)
        x = y64.astype(np.float32)
        a = ACT_CODE[self.act]
        ridx, rw, rh, ry = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a)
        got = self.out.cpu().numpy()
        err = float(np.max(np.abs(got - ry)) / np.max(np.abs(ry)))
        if a == 2:
            dref = oracle.gemv_i8x2(self.Dq_h, self.Ds_h, *oracle.quantize_x2(x))
        else:
            dref = oracle.gemv_i8(self.Dq_h, self.Ds_h, *oracle.quantize(x))
        derr = float(np.max(np.abs(self.dense_out.cpu().numpy() - dref)) / np.max(np.abs(dref)))
        return {"idx_equal": bool(np.array_equal(self.idx[0].cpu().numpy(), ridx)), "max_rel_err": err,
                "dense_max_rel_err": derr, "tol": TOL[self.act]}

    def cpu_baseline(self, budget):
        import oracle
        np = self.np
        m = self.host_w
        n, t0 = 0, time.perf_counter()
        a = ACT_CODE[self.act]
        while True:
            i = n % self.pool
            s, y64 = oracle.add_rmsnorm(self.pool_h[i], self.pool_r[i], self.norm_w, 1e-6)
            x = y64.astype(np.float32)
            oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a)
            if a == 2:
                oracle.gemv_i8x2(self.Dq_h, self.Ds_h, *oracle.quantize_x2(x))
            else:
                oracle.gemv_i8(self.Dq_h, self.Ds_h, *oracle.quantize(x))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return el / n, "%d chunks of %d rows, %.1f s" % (n, self.rows, el)


class MoeSharedBlock(MoeBlock):
    """The mixture block with its linked variants: the router as Q8_0 rows
    and an always-on shared expert, one moe_ffn_block_ex call a step (three
    launches; the shared expert's tiles ride in the gate-up launch, its slices
    in the down-combine).  The dominant kernel is that gate-up
    (moe_topk_gate_up_ex on logits from add_rmsnorm_router_q8)."""

    def __init__(self, name, cfg, act, copies, separate=False):
        if separate:
            raise SystemExit("workload %s runs as one moe_ffn_block_ex call a step" % name)
        super().__init__(name, cfg, act, copies)
        import synthetic
        np, torch, q8 = self.np, self.torch, self.q8
        d, E, sdff = cfg["d"], cfg["E"], cfg["sdff"]
        self.sdff = sdff
        rng = np.random.default_rng(3)
        self.Wrq_h = synthetic.quants(rng, E, d)
        self.Wrs_h = rng.uniform(2e-4, 5e-4, size=(E, d // 32)).astype(np.float32)
        S = []
        for rows_, cols in ((sdff, d), (sdff, d), (d, sdff)):
            S.extend(synthetic.q8_matrix(rng, rows_, cols))
        self.S_h = S
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [dev(self.Wrq_h), dev(self.Wrs_h)] + [dev(a) for a in S]
        self.V = [base] + [[t.clone() for t in base] for _ in range(self.copies - 1)]
        hw = self.k * self.dff + sdff
        z = lambda *s_, dt=torch.float32: torch.empty(s_, dtype=dt, device="cuda")
        self.hf, self.hq, self.hs = z(1, hw), z(1, hw, dt=torch.int8), z(1, hw // 32)
        a = q8.ACT_INT8 if act == "int8" else q8.ACT_F32
        self.bscratch = torch.zeros(q8.q8s_block_scratch_bytes(1, d, self.dff, sdff, E, self.k, a),
                                    dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def step(self, c):
        q8 = self.q8
        W = self.W[c % self.copies]
        V = self.V[c % self.copies]
        i = c % self.pool
        a = q8.ACT_INT8 if self.act == "int8" else q8.ACT_F32
        q8.moe_ffn_block_ex(self.h[i], self.r[i], self.w, 1e-6, *W[1:], self.k, self.E, act=a, Wrq=V[0], Wrs=V[1],
                            shared=tuple(V[2:]), sum=self.sum, idx=self.idx[c % self.copies],
                            wts=self.wts[c % self.copies], out=self.out, scratch=self.bscratch)

    def prepare_dominant(self):
        q8 = self.q8
        a = q8.ACT_INT8 if self.act == "int8" else q8.ACT_F32
        for c in range(self.copies):
            i = c % self.pool
            V = self.V[c]
            q8.add_rmsnorm_router_q8(self.h[i], self.r[i], self.w, 1e-6, V[0], V[1], act=a, sum=self.sum, x=self.y,
                                     xq=self.xq, xs=self.xs, logits=self.logits[c])
        self.torch.cuda.synchronize()

    def launch_dominant(self, c):
        q8 = self.q8
        a = q8.ACT_INT8 if self.act == "int8" else q8.ACT_F32
        W = self.W[c % self.copies]
        V = self.V[c % self.copies]
        idx, wts = self.idx[c % self.copies], self.wts[c % self.copies]
        kw = dict(xq=self.xq, xs=self.xs, hq=self.hq, hs=self.hs, want_h=False) if a == q8.ACT_INT8 else \
            dict(x=self.y, h=self.hf)
        q8.moe_topk_gate_up_ex(self.logits[c % self.copies], W[1], W[2], W[3], W[4], self.k, shared=tuple(V[2:6]),
                               idx=idx, wts=wts, act=a, **kw)

    def _q8(self, n_out, n_in):
        return n_out * n_in + n_out * (n_in // 32) * 4

    def stages(self):
        q8 = self.q8
        a = q8.ACT_INT8 if self.act == "int8" else q8.ACT_F32
        d, dff, E, k, sdff = self.d, self.dff, self.E, self.k, self.sdff
        C = self.copies

        def norm_router(c):
            i = c % self.pool
            V = self.V[c % C]
            q8.add_rmsnorm_router_q8(self.h[i], self.r[i], self.w, 1e-6, V[0], V[1], act=a, sum=self.sum, x=self.y,
                                     xq=self.xq, xs=self.xs, logits=self.logits[c % C])

        def down(c):
            W = self.W[c % C]
            V = self.V[c % C]
            kw = dict(hq=self.hq, hs=self.hs) if a == q8.ACT_INT8 else dict(h=self.hf)
            q8.moe_down_combine_ex(W[5], W[6], self.idx[c % C], self.wts[c % C], E, shared=tuple(V[6:8]), y=self.out,
                                   act=a, **kw)
        return [("add_rmsnorm_router_q8 (k_norm_logits)", norm_router, self._q8(E, d)),
                ("moe_topk_gate_up_ex (k_route_gate_up)", self.launch_dominant, self.dominant_bytes()),
                ("moe_down_combine_ex (k_down)", down, self._q8(d, k * dff + sdff))]

    def weight_bytes(self, c=None):
        d, dff, E, k, sdff = self.d, self.dff, self.E, self.k, self.sdff
        return self._q8(E, d) + k * 3 * self._q8(dff, d) + 3 * self._q8(sdff, d)

    def dominant_bytes(self, c=None):
        return 2 * self._q8(self.k * self.dff + self.sdff, self.d)

    def _oracle_step(self, i):
        import oracle
        np = self.np
        m = self.host_w
        s, y64 = oracle.add_rmsnorm(self.pool_h[i], self.pool_r[i], self.norm_w, 1e-6)
        x = y64.astype(np.float32)
        a = 1 if self.act == "int8" else 0
        return oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a, Wrq=self.Wrq_h,
                                 Wrs=self.Wrs_h, shared=self.S_h)

    def verify(self):
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        ridx, rw, rh, ry = self._oracle_step(0)
        got = self.out.cpu().numpy()
        err = float(np.max(np.abs(got - ry)) / np.max(np.abs(ry)))
        same_idx = bool(np.array_equal(self.idx[0].cpu().numpy(), ridx))
        return {"idx_equal": same_idx, "max_rel_err": err, "tol": 2e-3 if self.act == "int8" else 1e-5}

    def cpu_baseline(self, budget):
        n, t0 = 0, time.perf_counter()
        while True:
            self._oracle_step(n % self.pool)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return el / n, "%d steps (rows 1, inputs from the same pool), %.1f s" % (n, el)


class StackBlocks(Workload):
    """L layers of the mixture block in a row, each with weights of its own:
    one moe_ffn_stack call a step (3 launches a layer; each layer's residual
    add deferred into the next layer's add + norm launch, the last one's into
    its down-combine).  Stage: one moe_ffn_block call, a layer alone."""

    dominant = "k_route_gate_up"
    dominant_src = ("q8_gemv_sparse_amd/csrc/q8s_moe.hip", "q8_gemv_sparse_amd/csrc/q8s_device.h")

    def __init__(self, name, cfg, act, copies, pool=64):
        import numpy as np
        import torch

        import q8_gemv_sparse_amd as q8
        import synthetic
        self.q8, self.torch, self.np = q8, torch, np
        self.name, self.act = name, act
        d, dff, E, k, L = cfg["d"], cfg["dff"], cfg["E"], cfg["k"], cfg["layers"]
        self.d, self.dff, self.E, self.k, self.L = d, dff, E, k, L
        t0 = time.time()
        self.blocks = [synthetic.block_inputs(100 + l, d, dff, E, k, 1) for l in range(L)]
        rng = np.random.default_rng(1)
        self.pool_h = [synthetic.normal(rng, 1, d) for _ in range(pool)]
        self.pool_r = [synthetic.normal(rng, 1, d) for _ in range(pool)]
        self.pool = pool
        log("[bench] generated inputs in %.1fs" % (time.time() - t0))
        per_expert = 3 * dff * d + 3 * dff * (d // 32) * 4
        self.layer_bytes = E * d * 4 + k * per_expert
        self.copies = copies or _copies(L * self.layer_bytes, 0)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        base = [tuple(dev(a) for a in (b.w, b.moe.Wr, b.moe.Wgq, b.moe.Wgs, b.moe.Wuq, b.moe.Wus, b.moe.Wdq,
                                       b.moe.Wds)) for b in self.blocks]
        self.W = [base] + [[tuple(t.clone() for t in lw) for lw in base] for _ in range(self.copies - 1)]
        self.h = [dev(a) for a in self.pool_h]
        self.r = [dev(a) for a in self.pool_r]
        z = lambda *s_, dt=torch.float32: torch.empty(s_, dtype=dt, device="cuda")
        self.out = z(1, d)
        self.idx = [z(L, 1, k, dt=torch.int32) for _ in range(self.copies)]
        self.wts = [z(L, 1, k) for _ in range(self.copies)]
        a = ACT_CODE[act]
        self.scratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_STACK, 1, d, dff, E, k, a), dtype=torch.uint8,
                                   device="cuda")
        self.bscratch = torch.zeros(q8.q8s_scratch_bytes(q8.FN_BLOCK, 1, d, dff, E, k, a), dtype=torch.uint8,
                                    device="cuda")
        self.bsum, self.bidx, self.bwts, self.bout = z(1, d), z(1, k, dt=torch.int32), z(1, k), z(1, d)
        torch.cuda.synchronize()
        log("[bench] %s: %d layers, %d weight copies of %.1f MB on the device"
            % (name, L, self.copies, L * (E * d * 4 + E * per_expert) / 1e6))

    def step(self, c):
        i = c % self.pool
        self.q8.moe_ffn_stack(self.h[i], self.r[i], self.W[c % self.copies], self.k, 1e-6, act=ACT_CODE[self.act],
                              out=self.out, idx=self.idx[c % self.copies], wts=self.wts[c % self.copies],
                              scratch=self.scratch)

    def one_block(self, c):
        """Layer 0 of copy c alone, as one moe_ffn_block call."""
        i = c % self.pool
        lw = self.W[c % self.copies][0]
        self.q8.moe_ffn_block(self.h[i], self.r[i], lw[0], 1e-6, *lw[1:], self.k, act=ACT_CODE[self.act],
                              sum=self.bsum, idx=self.bidx, wts=self.bwts, out=self.bout, scratch=self.bscratch)

    launch_dominant = one_block

    def weight_bytes(self, c=None):
        return self.L * self.layer_bytes

    def dominant_bytes(self, c=None):
        return self.layer_bytes

    def stages(self):
        return [("moe_ffn_block (one layer alone, for the per-layer comparison)", self.one_block, self.layer_bytes)]

    def verify(self):
        """One eager step against the oracle's chain add_rmsnorm -> moe a layer."""
        import oracle
        np = self.np
        self.step(0)
        self.torch.cuda.synchronize()
        a = ACT_CODE[self.act]
        hh, rr = self.pool_h[0], self.pool_r[0]
        same = True
        for l, b in enumerate(self.blocks):
            s, y64 = oracle.add_rmsnorm(hh, rr, b.w, 1e-6)
            m = b.moe
            ridx, _, _, ry = oracle.moe(y64.astype(np.float32), m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds,
                                        self.k, a)
            same = same and bool(np.array_equal(self.idx[0][l].cpu().numpy(), ridx))
            hh, rr = ry.astype(np.float32), s
        ref = rr.astype(np.float64) + hh.astype(np.float64)
        got = self.out.cpu().numpy()
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        return {"idx_equal": same, "max_rel_err": err, "tol": self.L * TOL[self.act]}

    def cpu_baseline(self, budget):
        import oracle
        np = self.np
        a = ACT_CODE[self.act]
        n, t0 = 0, time.perf_counter()
        while True:
            hh, rr = self.pool_h[n % self.pool], self.pool_r[n % self.pool]
            for b in self.blocks:
                s, y64 = oracle.add_rmsnorm(hh, rr, b.w, 1e-6)
                m = b.moe
                ry = oracle.moe(y64.astype(np.float32), m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, self.k, a)[3]
                hh, rr = ry.astype(np.float32), s
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return el / n, "%d steps of %d layers, %.1f s" % (n, self.L, el)


def make_workload(name, act, copies, separate=False):
    import synthetic
    cfg = synthetic.CONFIGS[name]
    if act == "x2" and (cfg["kind"] not in ("norm_gemv", "moe", "stack", "chunk") or (cfg["kind"] == "moe" and separate)):
        raise SystemExit("two-word activations are built for the norm + GEMV and the mixture block's one call")
    if cfg["kind"] == "moe":
        return MoeBlock(name, cfg, act, copies, separate=separate)
    if cfg["kind"] == "norm_gemv":
        return NormGemv(name, cfg, act, copies, separate=separate)
    if cfg["kind"] == "chunk":
        return ChunkBlock(name, cfg, act, copies)
    if cfg["kind"] == "moe_shared":
        return MoeSharedBlock(name, cfg, act, copies, separate=separate)
    if cfg["kind"] == "gemv":
        return Gemv(name, cfg, act, copies)
    if cfg["kind"] == "stack":
        return StackBlocks(name, cfg, act, copies)
    raise SystemExit("workload %s is not a bench workload" % name)


# ---------------------------------------------------------------------------


def cpu_all_cores(wl, budget, threads):
    """The same oracle steps on every host core at once: `threads` Python
    threads, each running the workload's baseline loop for `budget` seconds
    (the oracle is C called through ctypes, which releases the interpreter
    lock, so the threads' steps run in parallel).  Returns the seconds per
    step of all threads together."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        per = list(ex.map(lambda _: wl.cpu_baseline(budget)[0], range(threads)))
    return 1.0 / sum(1.0 / p for p in per)


def host_cpu():
    """The host's CPU model and the CPUs this process may run on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return "%s, %d CPUs available" % (model, len(os.sched_getaffinity(0)))


class Ceiling:
    """What a plain read reaches on this device: the library's streaming
    reader (q8s_stream_read, which computes nothing of the method) over a
    2 GiB buffer -- eight times the 256 MB Infinity Cache -- and over cold
    slices of it of a given size, each slice a launch of its own, every slice
    read once per pass over the buffer."""

    def __init__(self, torch, q8, stream, eager):
        self.torch, self.q8, self.stream, self.eager = torch, q8, stream, eager
        self.total = 2 << 30
        self.buf = torch.zeros(self.total, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(q8.STREAM_WGS, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        whole_ms = self._timed(lambda: q8.q8s_stream_read(self.buf, out=self.out), 20)
        self.gbs = round(self.total / (whole_ms * 1e-3) / 1e9, 1)
        self.memo = {}

    def _timed(self, fn, reps):
        torch, stream = self.torch, self.stream
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            t0.record(stream)
            for _ in range(reps):
                fn()
            t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    def same_bytes(self, nbytes):
        """(µs, GB/s) of a launch that only reads `nbytes` cold bytes."""
        n = max(16, int(nbytes) // 16 * 16)
        if n in self.memo:
            return self.memo[n]
        torch, q8 = self.torch, self.q8
        span = -(-n // 256) * 256
        slices = max(1, min(4096, self.total // span))
        views = [self.buf[i * span:i * span + n] for i in range(slices)]

        def read_slices():
            for v in views:
                q8.q8s_stream_read(v, out=self.out)
        if self.eager:
            pass_fn = read_slices
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                read_slices()
            pass_fn = g.replay
        reps = max(1, -(-200 // slices))
        us = self._timed(pass_fn, reps) / slices * 1e3
        self.memo[n] = (round(us, 3), round(n / (us * 1e-6) / 1e9, 1))
        return self.memo[n]

    def describe(self, nbytes):
        us, gbs = self.same_bytes(nbytes)
        return {"what": "q8s_stream_read: 16-byte non-temporal loads, each byte once",
                "stream_read_gbs": self.gbs, "stream_read_bytes": self.total,
                "same_bytes_us": us, "same_bytes_gbs": gbs, "same_bytes": int(nbytes),
                "same_bytes_timing": "cold slices of a 2 GiB buffer, one launch each, %s"
                                     % ("eager" if self.eager else "a graph of one pass replayed")}


def _capture(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def _pct(vals, q):
    vals = sorted(vals)
    return round(vals[min(len(vals) - 1, int(q * len(vals)))], 3)


def _timing_events(torch, n, inside):
    return [torch.cuda.Event(enable_timing=True, external=inside) for _ in range(n)]


def measure(wl, steps, warmup, stream, eager=False, spread_n=200):
    """Times exactly `steps` steps after exactly `warmup` untimed ones, each
    group run as one graph of that many consecutive steps (step i on weight
    copy i mod C), a device synchronisation on both sides.  The two events
    that bracket the timed steps are recorded inside their graph, right
    before the first step's launches and right after the last one's, so the
    graph's own launch is not counted.  The spread: a graph of `spread_n`
    further steps with an event recorded between every two, each step's time
    the gap between its two events.  Without graphs (or where a graph cannot
    hold event records) the events go on the stream around the launches."""
    torch = wl.torch
    ver = wl.verify()
    ver["ok"] = bool(ver.get("idx_equal", True) and ver["max_rel_err"] <= ver["tol"] and
                     ver.get("dense_max_rel_err", 0.0) <= ver["tol"])
    log("[bench] %s %s: verify against the oracle: %s" % (wl.name, wl.act, ver))
    if not ver["ok"]:
        log("[bench] WARNING: the step does not match the oracle; its figures measure a wrong result")
    C = wl.copies
    with torch.cuda.stream(stream):
        for c in range(C):  # eager warm-up of every copy on the timing stream
            wl.step(c)
    torch.cuda.synchronize()

    def steps_fn(n, evs=None, first=0):
        # n steps from step `first`; evs: events recorded before step 0 and
        # after every step (len n + 1), or only around all (len 2)
        def fn():
            if evs is not None:
                evs[0].record(stream)
            for i in range(n):
                wl.step((first + i) % C)
                if evs is not None and (len(evs) == n + 1 or i == n - 1):
                    evs[i + 1 if len(evs) == n + 1 else 1].record(stream)
        return fn

    inside = not eager
    if inside:
        try:
            ek = _timing_events(torch, 2, True)
            gk = _capture(torch, stream, steps_fn(steps, ek))
        except Exception as exc:  # a runtime whose graphs do not take event records
            log("[bench] event records inside a graph refused (%s): events around the replay instead" % exc)
            inside = False
    gw = None
    if not eager and warmup > 0:
        gw = _capture(torch, stream, steps_fn(warmup))
    if not inside:
        ek = _timing_events(torch, 2, False)
        if not eager:
            gk = _capture(torch, stream, steps_fn(steps))
    with torch.cuda.stream(stream):
        if gw is not None:
            gw.replay()
        elif eager:
            steps_fn(warmup)()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        if inside:
            gk.replay()
        else:
            ek[0].record(stream)
            gk.replay() if not eager else steps_fn(steps)()
            ek[1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = ek[0].elapsed_time(ek[1]) / steps
    # the timed run's last step equals the same step run eagerly
    last = wl.out.clone()
    with torch.cuda.stream(stream):
        wl.step((steps - 1) % C)
    torch.cuda.synchronize()
    graph_matches = bool(torch.equal(last, wl.out))

    per_step_us = [float("nan")]
    if spread_n:
        es = _timing_events(torch, spread_n + 1, inside)
        if inside:
            gs = _capture(torch, stream, steps_fn(spread_n, es, steps))
            with torch.cuda.stream(stream):
                gs.replay()
        else:
            # eager steps with an event between every two, queued behind about
            # 30 ms of other GPU work (replays of the timed graph), so the
            # host's launches run ahead and no step waits for its submission
            fill = 0 if eager else max(1, int(30.0 / max(ms_per_step * steps, 1e-3)))
            with torch.cuda.stream(stream):
                for _ in range(fill):
                    gk.replay()
                steps_fn(spread_n, es, steps)()
        torch.cuda.synchronize()
        per_step_us = [es[i].elapsed_time(es[i + 1]) * 1e3 for i in range(spread_n)]
    step_bytes = sum(wl.weight_bytes(c) for c in range(C)) / C
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    return {
        "workload": wl.name, "act": wl.act, "rows": getattr(wl, "rows", 1),
        "steps": steps, "warmup": warmup,
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_p10_p50_p90": [_pct(per_step_us, 0.1), _pct(per_step_us, 0.5), _pct(per_step_us, 0.9)],
        "spread_samples": spread_n,
        "spread_timing": ("%d consecutive steps in one graph, an event recorded between every two; each step's "
                          "time includes one event record" if inside else
                          "%d consecutive steps launched eagerly behind queued GPU work, an event on the stream "
                          "between every two; each step's time includes one event record") % spread_n,
        "weight_bytes_per_step": int(step_bytes),
        "gbs": round(value, 2),
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "weight_copies": C,
        "timing": ("eager launches, %d steps, events on the stream around them" % steps if eager else
                   "one HIP graph of %d steps, its events recorded inside the graph" % steps if inside else
                   "one HIP graph of %d steps, events on the stream around its replay" % steps),
        "verified": ver,
        "graph_equals_eager": graph_matches,
        "cache": getattr(wl, "cache", "cold: weight copies and input rows rotate past the Infinity Cache"),
        "wall_s": round(t_wall, 4),
    }


def time_launches(torch, stream, fn, C, launches, eager=False):
    """µs per launch of fn(c): `launches` launches cycling over the C copies,
    captured as one graph (a graph replay has a fixed cost of its own, several
    µs, so a graph holds many launches), replayed once untimed and once
    between two events."""
    n = max(C, launches // C * C)

    def run_all():
        for i in range(n):
            fn(i % C)
    g = run_all if eager else _capture(torch, stream, run_all).replay
    with torch.cuda.stream(stream):
        g()
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        k0.record(stream)
        g()
        k1.record(stream)
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / n * 1e3


def time_stages(wl, stream, ceil, eager=False, launches=400):
    """Each of the step's calls alone: a graph of its launches, one per weight
    copy (on the routing and activations the steps left for that copy),
    replayed back to back between two events; with the time a plain read of
    the same weight bytes takes."""
    torch = wl.torch
    wl.prepare_dominant()
    C = wl.copies
    out = []
    for label, fn, nbytes in wl.stages():
        us = time_launches(torch, stream, fn, C, launches, eager)
        ent = {"call": label, "us_per_launch": round(us, 3), "weight_bytes": int(nbytes)}
        if nbytes:
            ent["gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            ent["hbm_frac_of_peak"] = round(ent["gbs"] / HBM_PEAK_GBS, 4)
            if ceil is not None:
                pu, pg = ceil.same_bytes(nbytes)
                ent["plain_read_us"] = pu
                ent["frac_of_plain_read"] = round(pu / us, 4)
        out.append(ent)
    return out


# The suite one default run measures after the headline: every workload the
# configs name, in each numerics it is built for.
SUITE = [
    ("gemv_512x256", "f32"),
    ("norm_gemv_2048x4096", "int8"),
    ("norm_gemv_2048x4096", "f32"),
    ("norm_gemv_2048x4096", "x2"),
    ("moe_d2048_dff768_e128_k8", "f32"),
    ("moe_d2048_dff768_e128_k8", "x2"),
    ("moe_d4096_dff14336_e8_k2", "int8"),
    ("moe_d4096_dff14336_e8_k2", "f32"),
    ("moe_d4096_dff14336_e8_k2", "x2"),
    ("chunk64_moe_d2048_dense4096", "int8"),
    ("chunk64_moe_d2048_dense4096", "x2"),
    ("chunk128_moe_d2048_dense4096", "int8"),
    ("chunk128_moe_d2048_dense4096", "x2"),
    ("chunk256_moe_d2048_dense4096", "int8"),
    ("moe_shared_d2048_dff1408_e60_k4_s5632", "int8"),
    ("moe_shared_d2048_dff1408_e60_k4_s5632", "f32"),
    ("stack4_moe_d2048_dff768_e128_k8", "int8"),
]
SUITE_STEPS = 400
SUITE_WARMUP = 20


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import gc

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import q8_gemv_sparse_amd as q8
    stream = torch.cuda.Stream()
    if args.ceiling_only:
        ceil = Ceiling(torch, q8, stream, args.no_graph)
        print(json.dumps({"ceiling": ceil.describe(28311552)}), flush=True)
        return
    ceil = None if args.no_ceiling else Ceiling(torch, q8, stream, args.no_graph)
    t_start = time.perf_counter()
    wl = make_workload(args.workload, args.act, args.copies, args.separate)
    if args.warm:
        # every step (and every dominant launch) on copy 0 with input row 0:
        # the same weights each time, resident in the Infinity Cache
        step0, dom0 = wl.step, wl.launch_dominant
        wl.step = lambda c: step0(0)
        wl.launch_dominant = lambda c: dom0(0)
        wl.cache = "warm: one weight copy and one input row every step (cache-resident, context only)"
    head = measure(wl, args.steps, args.warmup, stream, args.no_graph, args.spread)
    C = wl.copies

    # the dominant kernel: a graph of its launches on each copy (the routing
    # each copy's last step left in place), replayed back to back; HIP events
    # on the replay stream around the replays
    wl.prepare_dominant()
    n_dom = max(C, args.kernel_launches // C * C)
    kms = time_launches(torch, stream, wl.launch_dominant, C, args.kernel_launches, args.no_graph) / 1e3
    dom_bytes = sum(wl.dominant_bytes(i % C) for i in range(C)) / C
    achieved = dom_bytes / (kms * 1e-3) / 1e9
    head["stages"] = [] if args.warm else time_stages(wl, stream, ceil, args.no_graph)
    ceiling = ceil.describe(dom_bytes) if ceil else None

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy: %d MiB" % args.calib_copy_mib)

    traffic = None
    cfile = counters_path(wl.dominant, wl.name, args.act)
    if os.path.exists(cfile):
        with open(cfile) as fh:
            cnt = json.load(fh)
        if cnt.get("source_digest") == src_digest(*wl.dominant_src):
            traffic = cnt.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        step_bytes = head["weight_bytes_per_step"]
        per_step, sample = wl.cpu_baseline(args.cpu_budget)
        cpu = {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": sample + "; %.1f ms per step" % (per_step * 1e3), "host": host_cpu()}
        threads = args.cpu_threads or len(os.sched_getaffinity(0))
        if threads > 1:
            per_all = cpu_all_cores(wl, args.cpu_budget, threads)
            cpu["all_cores"] = {"value": round(step_bytes / per_all / 1e9, 4), "unit": "GB/s", "cores": threads,
                                "sample": "%d threads, each its own steps for %.0f s; %.2f ms per step together"
                                          % (threads, args.cpu_budget, per_all * 1e3)}
    wl_rows, dom_name = getattr(wl, "rows", 1), wl.dominant
    del wl
    gc.collect()
    torch.cuda.empty_cache()

    suite = []
    run_suite = args.suite == "all" or (args.suite == "auto" and args.workload == DEFAULT_WORKLOAD and
                                        args.act == "int8" and not (args.warm or args.separate or args.no_graph))
    if run_suite:
        for name, act in SUITE:
            log("[bench] suite: %s %s" % (name, act))
            w2 = make_workload(name, act, 0)
            ent = measure(w2, SUITE_STEPS, SUITE_WARMUP, stream, False, args.spread)
            ent["stages"] = time_stages(w2, stream, ceil)
            suite.append(ent)
            del w2
            gc.collect()
            torch.cuda.empty_cache()

    value = head["gbs"]
    cfg = dict(head)
    for k_ in ("gbs", "steps", "warmup"):
        cfg.pop(k_)
    cfg["workloads"] = suite
    cfg["run_s"] = round(time.perf_counter() - t_start, 1)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": round(head["us_per_step"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "i8", "x2": "i8x2", "f32": "f32"}[args.act],
        "data": "synthetic",
        "config": cfg,
        "roofline": {
            "bound": "hbm",
            "kernel": dom_name,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(dom_bytes),
            "us_per_launch": round(kms * 1e3, 3),
            "timed": "one graph of %d of its launches back to back, cycling over the %d weight copies" % (n_dom, C),
            "ceiling": ceiling,
            "frac_of_stream_ceiling": round(achieved / ceiling["stream_read_gbs"], 4) if ceiling else None,
        },
        "cpu_baseline": cpu,
    }
    log("[bench] timed region %.4fs for %d steps (rows %d)" % (head["wall_s"], head["steps"], wl_rows))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
