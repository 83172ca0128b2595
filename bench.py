"""Throughput of the speculative verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of the library on one batch of synthetic inputs already resident in
HBM.  The default workload is linear speculative sampling with B=64 sequences, k=5
draft tokens and a 32000-token bfloat16 vocabulary; the metric is verified draft
positions per second (B*k per step).  Other workloads (--workload) print their own line.

Inputs are rotated over enough device copies (>= 1 GiB in total by default) that the
256 MB Infinity Cache cannot serve a step from the previous step's reads.  The K timed
steps are recorded once into a HIP graph (one launch per step, rotating the inputs) and
the graph is replayed, so the host's per-call cost (about 10 us of Python and ctypes per
call) does not set the pace; if capture fails the steps are launched one by one.  Timing
uses HIP events recorded on the stream the kernels run on, around exactly K steps, with a
device synchronisation on both sides.  The JSON line carries a roofline block for the
dominant kernel (algorithmic bytes per launch / average launch time, against 8 TB/s), the
same bytes against a device copy measured in the same run, and the CPU oracle timed on a
bounded sample of the same workload on host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Sources that determine each kernel family's code and launch shape.  The HBM traffic table
# under profiles/ records the digest of the family a workload's dominant kernel belongs to;
# a row whose digest no longer matches is stale and reported as null.
_CSRC = "speculative_sampling_verify_03_amd/csrc/"
KERNEL_SOURCES = {
    "rows": [_CSRC + f for f in ("verify_rows.hip", "verify_split.hip", "sv_device.hpp", "sv_launch.hpp", "api.hip",
                                 "validate.hpp")],
    "greedy": [_CSRC + f for f in ("verify_greedy.hip", "sv_device.hpp", "sv_launch.hpp", "api.hip",
                                   "validate.cpp")],
    "lmhead": [_CSRC + f for f in ("lmhead_gemm.hip", "lmhead_verify.hip", "sv_device.hpp", "sv_launch.hpp")]
              + ["speculative_sampling_verify_03_amd/build.py"],
    "lookup": [_CSRC + f for f in ("lookup.hip", "sv_device.hpp", "sv_launch.hpp")],
}


def kernel_family(workload: str) -> str:
    if workload.startswith("greedy"):
        return "greedy"
    if workload.startswith("lmhead"):
        return "lmhead"
    if workload.startswith("lookup"):
        return "lookup"
    return "rows"


def kernel_digest(family: str = "rows") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="linear-b64-k5-v32000",
                    choices=["linear-b64-k5-v32000", "linear-b1-k4-v1024", "linear-b1000-k4-v1024",
                             "linear-b256-k8-v128256", "greedy-b256-k8-v128256", "tree-b16-n61-v128256", "tree-lossless-b16-n61-v128256",
                             "lmhead-b32-k5-h8192-v128256", "linear-b256-k1-v128256", "linear-plug-b64-k5-v32000",
                             "lookup-b64-l8192-n3-k5", "copy-probe"])
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true", help="launch the timed steps one by one (no graph)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- workloads
class Linear:
    ws_kind = 0  # SV_KIND_LINEAR

    def __init__(self, name, make_case, seeds, dtype_name, temperature):
        self.name = name
        self.make_case = make_case
        self.seeds = seeds
        self.dtype_name = dtype_name
        self.T = temperature

    def setup(self, sv, torch, rotate_bytes):
        self.sv = sv
        self.torch = torch
        self.cases = [self.make_case(s) for s in self.seeds]
        c0 = self.cases[0]
        self.B, self.R, self.V = c0.logits.shape
        self.k = self.R - 1
        per_set = c0.logits.numel() * c0.logits.element_size() + c0.draft_probs.numel() * c0.draft_probs.element_size()
        nsets = max(len(self.cases), int(np.ceil(rotate_bytes / per_set)))
        self.sets = []
        for i in range(nsets):
            c = self.cases[i % len(self.cases)]
            self.sets.append((c.logits.cuda(), c.draft_probs.cuda(), c.draft_tokens.cuda(), i % len(self.cases)))
        self.tokens = torch.empty((self.B, self.R), dtype=torch.int32, device="cuda")
        self.alen = torch.empty((self.B,), dtype=torch.int32, device="cuda")
        self.ws = sv.new_workspace(self.ws_kind, self.B, self.k, self.V)
        self.resident_bytes = per_set * nsets
        # realised rejections per distinct input (compulsory q-row reads)
        self.rejected = []
        for lg, q, x, _ in self.sets[:len(self.cases)]:
            self.launch_set(lg, q, x)
            torch.cuda.synchronize()
            self.rejected.append(int((self.alen < self.k).sum()))
        # Only the split kernel writes the workspace's fixed prefix past its status word (its
        # generation counters and tagged words); the row kernel leaves it at zero.
        prefix = sv.spec_verify_workspace_bytes(self.ws_kind, 0, self.k, self.V)
        self.split_path = int(self.ws[4:prefix].count_nonzero()) > 0

    def launch_set(self, lg, q, x):
        self.sv.spec_verify_linear(lg, q, x, self.T, 0, 0, self.tokens, self.alen, None, None, self.ws)

    def launch(self, i):
        lg, q, x, _ = self.sets[i % len(self.sets)]
        self.launch_set(lg, q, x)

    def positions(self):
        return self.B * self.k

    def algorithmic_bytes(self):
        c0 = self.cases[0]
        el = c0.logits.element_size()
        eq = c0.draft_probs.element_size()
        rej = float(np.mean(self.rejected))
        return (self.B * self.R * self.V * el          # every target logit row once
                + rej * self.V * eq                     # the draft row at each rejection
                + self.B * self.k * (eq + 4)            # q(x) gathers and draft tokens
                + self.B * self.R * 4 + self.B * 4)     # outputs

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_len": self.k, "vocab": self.V,
                "logits_dtype": self.dtype_name, "temperature": self.T}

    def oracle_sample(self, budget_s):
        from oracle import verify_linear
        from synthetic import to_numpy_f64
        c = self.cases[0]
        L = to_numpy_f64(c.logits)
        Q = to_numpy_f64(c.draft_probs)
        X = c.draft_tokens.numpy()
        done = 0
        t0 = time.perf_counter()
        while True:
            b = done % self.B
            verify_linear(L[b:b + 1], Q[b:b + 1], X[b:b + 1], self.T, 0, 0)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        return done * self.k / el, f"{done} sequences of the first input batch ({done * self.k} positions), one at a time"


class LinearPlug(Linear):
    """Linear verification followed by the on-device token plug of its outputs (the next
    step's inputs are set up without reading accept_len back to the host)."""

    def setup(self, sv, torch, rotate_bytes):
        super().setup(sv, torch, rotate_bytes)
        self.cap = 16384
        self.seq_len = torch.zeros(self.B, dtype=torch.int32, device="cuda")
        self.history = torch.zeros((self.B, self.cap), dtype=torch.int32, device="cuda")
        self.next_token = torch.zeros(self.B, dtype=torch.int32, device="cuda")

    def launch(self, i):
        super().launch(i)
        self.sv.spec_plug_tokens(self.tokens, self.alen, self.seq_len, self.history, self.next_token)

    def launch_verify_only(self, i):
        super().launch(i)


class Greedy(Linear):
    def launch_set(self, lg, q, x):
        self.sv.spec_verify_greedy(lg, x, self.tokens, self.alen, self.ws)

    ws_kind = 1  # SV_KIND_GREEDY

    def setup(self, sv, torch, rotate_bytes):
        super().setup(sv, torch, rotate_bytes)
        self.sets = [(lg, q, self.cases[ci].greedy_tokens.cuda(), ci) for lg, q, x, ci in self.sets]

    def algorithmic_bytes(self):
        # The rows the sequential rule examines: positions 0..n of every sequence (n its
        # accept length), counted on the inputs and averaged over the input sets; the kernels
        # read no row after a sequence's first mismatch once they know of it, so counting
        # every row would put the figure above what the chip can stream.
        if not hasattr(self, "_examined"):
            rows = []
            for c in self.cases:
                g = c.logits.float().argmax(dim=-1).numpy()
                miss = g[:, :self.k] != c.greedy_tokens.numpy()
                n = np.where(miss.any(axis=1), miss.argmax(axis=1), self.k)
                rows.append(float((n + 1).sum()))
            self._examined = sum(rows) / len(rows)
        el = self.cases[0].logits.element_size()
        return int(self._examined * self.V * el) + self.B * self.k * 4 + self.B * self.R * 4 + self.B * 4

    def oracle_sample(self, budget_s):
        from oracle import verify_greedy
        from synthetic import to_numpy_f64
        c = self.cases[0]
        L = to_numpy_f64(c.logits)
        X = c.greedy_tokens.numpy()
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = done % self.B
            verify_greedy(L[b:b + 1], X[b:b + 1])
            done += 1
        el = time.perf_counter() - t0
        return done * self.k / el, f"{done} sequences, one at a time"


class Tree:
    lossless = False

    def __init__(self, name, seeds):
        self.name = name
        self.seeds = seeds

    def setup(self, sv, torch, rotate_bytes):
        from synthetic import cfg5_case
        self.sv = sv
        self.torch = torch
        self.cases = [cfg5_case(seed=s) for s in self.seeds]
        c0 = self.cases[0]
        self.B, self.N, self.V = c0.logits.shape
        self.par = c0.parents.tolist()
        depth = [0] * self.N
        for c in range(1, self.N):
            depth[c] = depth[self.par[c]] + 1
        self.D = max(depth)
        per_set = c0.logits.numel() * 2 + (0 if self.lossless else c0.draft_probs.numel() * 2)
        nsets = max(len(self.cases), int(np.ceil(rotate_bytes / per_set)))
        self.sets = [(self.cases[i % len(self.cases)].logits.cuda(),
                      None if self.lossless else self.cases[i % len(self.cases)].draft_probs.cuda(),
                      self.cases[i % len(self.cases)].node_tokens.cuda()) for i in range(nsets)]
        self.tokens = torch.empty((self.B, self.D + 1), dtype=torch.int32, device="cuda")
        self.alen = torch.empty((self.B,), dtype=torch.int32, device="cuda")
        self.path = torch.empty((self.B, self.D + 1), dtype=torch.int32, device="cuda")
        self.ws = sv.new_workspace(sv.SV_KIND_TREE, self.B, self.N, self.V)
        self.resident_bytes = per_set * nsets

    def launch(self, i):
        lg, q, t = self.sets[i % len(self.sets)]
        if self.lossless:
            self.sv.spec_verify_tree_lossless(lg, t, self.par, 1.0, 0, 0, self.tokens, self.alen, self.path, self.ws)
        else:
            self.sv.spec_verify_tree(lg, q, t, self.par, 1.0, 0, 0, self.tokens, self.alen, self.path, self.ws)

    def positions(self):
        return self.B * (self.N - 1)

    def algorithmic_bytes(self):
        # every logits row once; the children's q(x) gathers (not read by the lossless
        # rule), node tokens and outputs
        return (self.B * self.N * self.V * 2 + self.B * (self.N - 1) * ((0 if self.lossless else 2) + 4)
                + self.B * (self.D + 1) * 8 + self.B * 4)

    def config(self):
        return {"workload": self.name, "batch": self.B, "tree_nodes": self.N, "vocab": self.V,
                "logits_dtype": "bf16", "temperature": 1.0}

    def oracle_sample(self, budget_s):
        from oracle import verify_tree, verify_tree_lossless
        from synthetic import to_numpy_f64
        c = self.cases[0]
        L = to_numpy_f64(c.logits)
        Q = None if self.lossless else to_numpy_f64(c.draft_probs)
        T_ = c.node_tokens.numpy()
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = done % self.B
            if self.lossless:
                verify_tree_lossless(L[b:b + 1], T_[b:b + 1], c.parents, 1.0, 0, 0)
            else:
                verify_tree(L[b:b + 1], Q[b:b + 1], T_[b:b + 1], c.parents, 1.0, 0, 0)
            done += 1
        el = time.perf_counter() - t0
        return done * (self.N - 1) / el, f"{done} sequences, one at a time"


class TreeLossless(Tree):
    """The same 61-node tree and inputs, verified by the lossless sibling rule (no q rows)."""
    lossless = True


class LMHead:
    name = "lmhead-b32-k5-h8192-v128256"

    def setup(self, sv, torch, rotate_bytes):
        from synthetic import cfg4_case
        self.sv = sv
        self.torch = torch
        self.case = cfg4_case()
        c = self.case
        self.B, self.R, self.H = c.hidden.shape
        self.k = self.R - 1
        self.V = c.weight.shape[1]
        self.h = c.hidden.cuda()
        self.w = c.weight.cuda()  # 2.1 GB: larger than every cache level on its own
        self.q = c.draft_probs.cuda()
        self.x = c.draft_tokens.cuda()
        self.logits = torch.empty((self.B, self.R, self.V), dtype=torch.float32, device="cuda")
        self.tokens = torch.empty((self.B, self.R), dtype=torch.int32, device="cuda")
        self.alen = torch.empty((self.B,), dtype=torch.int32, device="cuda")
        self.ws = sv.new_workspace(sv.SV_KIND_LMHEAD, self.B, self.k, self.V, self.H)
        self.resident_bytes = self.w.numel() * 2
        self.launch(0)
        torch.cuda.synchronize()
        self.rejected = int((self.alen < self.k).sum())

    def launch(self, i):
        self.sv.spec_lmhead_verify(self.h, self.w, self.q, self.x, 1.0, 0, i, self.logits, self.tokens,
                                   self.alen, None, None, self.ws)

    def launch_gemm_only(self, i):
        self.sv.spec_lmhead_logits(self.h, self.w, self.logits)

    def positions(self):
        return self.B * self.k

    def gemm_bytes(self):
        M = self.B * self.R
        return self.H * self.V * 2 + M * self.H * 2 + M * self.V * 4

    def gemm_flops(self):
        return 2.0 * self.B * self.R * self.H * self.V

    def algorithmic_bytes(self):
        return self.gemm_bytes() + self.rejected * self.V * 2 + self.B * self.k * 6 + self.B * self.R * 4

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_len": self.k, "hidden": self.H, "vocab": self.V,
                "weight_dtype": "bf16", "temperature": 1.0}

    def oracle_sample(self, budget_s):
        from oracle import verify_lmhead
        from synthetic import to_numpy_f64
        c = self.case
        hid = to_numpy_f64(c.hidden[:1])
        Q = to_numpy_f64(c.draft_probs[:1])
        X = c.draft_tokens[:1].numpy()
        t0 = time.perf_counter()
        done = 0
        W = None
        while time.perf_counter() - t0 < budget_s or done == 0:
            if W is None:
                W = to_numpy_f64(c.weight)
            verify_lmhead(hid, W, Q, X, 1.0, 0, 0)
            done += 1
        el = time.perf_counter() - t0
        return done * self.k / el, f"{done} sequence(s) of 6 rows, float64 GEMM + verification"


class Lookup:
    """Prompt-lookup drafting over token histories that echo their own prompt (a document
    followed by a response that copies spans of it), B sequences of up to `cap` tokens,
    phrase lengths min_ngram..max_ngram, k drafts per sequence."""
    metric = "proposed draft positions/sec"

    def __init__(self, name, B, cap, min_ngram, max_ngram, k, seeds):
        self.name, self.B, self.cap = name, B, cap
        self.mn, self.mx, self.k = min_ngram, max_ngram, k
        self.seeds = seeds

    def setup(self, sv, torch, rotate_bytes):
        from synthetic import lookup_histories
        self.sv, self.torch = sv, torch
        self.cases = [lookup_histories(self.B, self.cap, seed=s) for s in self.seeds]
        per_set = self.B * self.cap * 4
        nsets = max(len(self.cases), int(np.ceil(rotate_bytes / per_set)))
        self.sets = []
        for i in range(nsets):
            h, L = self.cases[i % len(self.cases)]
            self.sets.append((torch.as_tensor(h, dtype=torch.int32).cuda(),
                              torch.as_tensor(L, dtype=torch.int32).cuda()))
        self.drafts = torch.empty((self.B, self.k), dtype=torch.int32, device="cuda")
        self.count = torch.empty((self.B,), dtype=torch.int32, device="cuda")
        self.resident_bytes = per_set * nsets

    def launch(self, i):
        h, L = self.sets[i % len(self.sets)]
        self.sv.spec_lookup_drafts(h, L, self.mn, self.mx, self.drafts, self.count)

    def positions(self):
        return self.B * self.k

    def _extent(self, h, length):
        """Tokens a scan must read: up to the end of the longest phrase's earliest earlier
        occurrence when there is one (it decides and ends the scan), else the whole history."""
        if length - 1 < self.mx:
            return length
        from numpy.lib.stride_tricks import sliding_window_view
        win = sliding_window_view(h[:length - 1], self.mx)
        hit = np.flatnonzero((win == h[length - self.mx:length]).all(axis=1))
        return int(hit[0]) + self.mx if hit.size else length

    def algorithmic_bytes(self):
        tot = 0.0
        for h, L in self.cases:
            tot += sum(self._extent(h[b], int(L[b])) for b in range(self.B)) * 4
        return tot / len(self.cases) + self.B * 4 + self.B * (self.k + 1) * 4

    def config(self):
        return {"workload": self.name, "batch": self.B, "history_cap": self.cap, "min_ngram": self.mn,
                "max_ngram": self.mx, "draft_len": self.k}

    def oracle_sample(self, budget_s):
        from oracle import lookup_drafts
        h, L = self.cases[0]
        done = 0
        t0 = time.perf_counter()
        while True:
            b = done % self.B
            lookup_drafts(h[b:b + 1], L[b:b + 1], self.mn, self.mx, self.k)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        return done * self.k / el, f"{done} sequences of the first history batch, one at a time"


def make_workload(name):
    from synthetic import cfg1_case, cfg2_case, cfg3_case, mtp_case
    if name == "linear-b64-k5-v32000":
        return Linear(name, lambda s: cfg2_case(seed=s), [2, 102, 202, 302], "bf16", 1.0)
    if name == "linear-b1-k4-v1024":
        return Linear(name, lambda s: cfg1_case(B=1, seed=s), [1], "f32", 1.0)
    if name == "linear-b1000-k4-v1024":
        return Linear(name, lambda s: cfg1_case(B=1000, seed=s), [1, 101], "f32", 1.0)
    if name == "linear-b256-k8-v128256":
        return Linear(name, lambda s: cfg3_case(seed=s), [3], "bf16", 0.7)
    if name == "linear-b256-k1-v128256":  # single-token MTP regime: 2 rows per sequence
        return Linear(name, lambda s: mtp_case(seed=s), [6, 106], "bf16", 1.0)
    if name == "linear-plug-b64-k5-v32000":
        return LinearPlug(name, lambda s: cfg2_case(seed=s), [2, 102, 202, 302], "bf16", 1.0)
    if name == "greedy-b256-k8-v128256":
        return Greedy(name, lambda s: cfg3_case(seed=s), [3], "bf16", 0.7)
    if name == "tree-b16-n61-v128256":
        return Tree(name, [5, 105])
    if name == "tree-lossless-b16-n61-v128256":
        return TreeLossless(name, [5, 105])
    if name == "lmhead-b32-k5-h8192-v128256":
        return LMHead()
    if name == "lookup-b64-l8192-n3-k5":
        return Lookup(name, 64, 8192, 1, 3, 5, [7, 107])
    raise ValueError(name)


def traffic_for(name):
    """HBM bytes per launch from the committed rocprofv3 counter table, if the counters were
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest = kernel_digest(kernel_family(name))
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == name and cells[1] == digest:
            try:
                return int(cells[4])
            except ValueError:
                return None
    return None


def copy_probe(torch, steps):
    """A plain device copy of known size for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(3, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}), flush=True)


class Stepper:
    """Runs K consecutive steps fn(0..K-1) on the current stream: as one replay of a graph
    that recorded them (mode "hip_graph"), or launched one by one ("eager") when capture is
    refused.  Each step's inputs are fixed when it is recorded, so a replay repeats exactly
    the launches an eager loop would make."""

    def __init__(self, torch, fn, K, use_graph=True):
        self.torch, self.fn, self.K = torch, fn, K
        self.graph = None
        self.mode = "eager"
        if use_graph:
            try:
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    fn(0)  # first launches (per-device set-up) outside the capture
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=side):
                    for i in range(K):
                        fn(i)
                torch.cuda.synchronize()
                self.graph = g
                self.mode = "hip_graph"
            except Exception as exc:  # capture refused: eager launches
                self.mode = f"eager ({type(exc).__name__})"
                torch.cuda.synchronize()

    def run(self):
        if self.graph is not None:
            self.graph.replay()
        else:
            for i in range(self.K):
                self.fn(i)

    def time_ms(self, stream):
        torch = self.torch
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        self.run()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)


def copy_gbs(torch, stream, nbytes=1 << 30, reps=5):
    """Device-to-device copy bandwidth (bytes read + written per second), the practical
    streaming ceiling the verification kernels are compared with."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import speculative_sampling_verify_03_amd as sv
    torch.cuda.set_device(0)
    if args.workload == "copy-probe":
        copy_probe(torch, args.steps)
        return

    wl = make_workload(args.workload)
    wl.setup(sv, torch, args.rotate_gib * (1 << 30))
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        wl.launch(i)
    torch.cuda.synchronize()
    stepper = Stepper(torch, wl.launch, args.steps, use_graph=not args.eager)
    stepper.run()  # one untimed pass of the recorded steps
    ms_total = stepper.time_ms(stream)
    ms_step = ms_total / args.steps

    extra = {"launch": stepper.mode}
    if isinstance(wl, LinearPlug):
        # the plug's own cost: the step minus verification alone
        vs = Stepper(torch, wl.launch_verify_only, args.steps, use_graph=not args.eager)
        vs.run()
        extra["verify_ms"] = round(vs.time_ms(stream) / args.steps, 5)
        extra["plug_ms"] = round(ms_step - extra["verify_ms"], 5)
    if isinstance(wl, LMHead):
        # the GEMM dominates: timed alone (spec_lmhead_logits, the same kernel without the
        # softmax partials); the rest of the step is verification (partials, decide, draw)
        gs = Stepper(torch, wl.launch_gemm_only, args.steps, use_graph=not args.eager)
        gs.run()
        ms_gemm = gs.time_ms(stream) / args.steps
        ms_verify = ms_step - ms_gemm
        achieved = wl.gemm_bytes() / (ms_gemm * 1e-3) / 1e9
        tflops = wl.gemm_flops() / (ms_gemm * 1e-3) / 1e12
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(wl.name),
                    "kernel": "lmhead_gemm_dma_kernel", "kernel_ms": round(ms_gemm, 4),
                    "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
        extra["verify_ms"] = round(ms_verify, 4)
    else:
        kernel_ms = extra.get("verify_ms", ms_step)  # with the plug: the verification kernel alone
        achieved = wl.algorithmic_bytes() / (kernel_ms * 1e-3) / 1e9
        kname = {"Greedy": "greedy_flat_kernel", "Tree": "row_verify_kernel(tree)", "Lookup": "lookup_kernel",
                 "TreeLossless": "row_verify_kernel(tree, lossless)"}.get(type(wl).__name__,
                                                                                   "row_verify_kernel(linear)")
        if type(wl).__name__ in ("Linear", "LinearPlug") and getattr(wl, "split_path", False):
            kname = "row_split_kernel(linear)"
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(wl.name),
                    "kernel": kname, "kernel_ms": round(kernel_ms, 5),
                    "algorithmic_bytes_per_launch": int(wl.algorithmic_bytes())}

    value = wl.positions() / (ms_step * 1e-3)
    cpu = None
    if not args.no_cpu:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                cpu_value, sample = wl.oracle_sample(args.cpu_seconds)
        except ImportError:
            cpu_value, sample = wl.oracle_sample(args.cpu_seconds)
        cpu = {"value": round(cpu_value, 2), "unit": getattr(wl, "metric", "verified draft positions/sec").replace("/sec", "/s"), "cores": 1, "kind": "oracle",
               "sample": sample, "host_cores_available": len(os.sched_getaffinity(0))}
    copy_peak = copy_gbs(torch, stream)
    roofline["copy_gbs"] = round(copy_peak, 1)
    roofline["frac_of_copy"] = round(roofline["achieved"] / copy_peak, 4)
    line = {
        "metric": getattr(wl, "metric", "verified draft positions/sec"),
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type: the verification kernels compute in float32 whatever the input
        # dtype; the LM-head GEMM multiplies bf16 on the matrix cores (fp32 accumulation)
        "dtype": "bf16" if isinstance(wl, LMHead) else "int32" if isinstance(wl, Lookup) else "f32",
        "data": "synthetic",
        "config": wl.config(),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_gbs": roofline["achieved"],
        "hbm_frac": roofline["frac"],
        "resident_input_bytes": int(wl.resident_bytes),
        "kernel_digest": kernel_digest(kernel_family(wl.name)),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
