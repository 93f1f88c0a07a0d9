"""Benchmark of the per-round WhiFlash verify-and-route step on one MI355X.

One step = one speculation round over a batch: the neural router
(whiflash_route) followed by greedy verification of that batch's candidates
(argmax sweep over every logits row, chain / tree acceptance, emission), on
one HIP stream.

Workloads:
  sweep (default): the throughput sweep: 256 DFlash chains, K = 16, bf16 logits
      [256, 17, 151936] (1.32 GB per round) plus the router on bf16 hidden
      [256, 2560] (MFMA path); 100 rounds with fresh seeded logits, drafts and
      hidden states each, all resident in HBM (132 GB) and cycled.
  routed: 128 sequences, bf16 hidden [128, 2560] through the router
      (2560 -> 1024 -> 1, threshold 1.0, exact 64/64 split); 64 DFlash chains of
      K = 16 (17 rows) and 64 EAGLE-3 trees of 61 nodes, packed into 4,992 bf16
      logits rows of 151,936 (1.517 GB per round); one step is
      whiflash_round_routed.
  llama: the throughput sweep at Llama-3.1-8B shapes: 256 chains, K = 10, bf16
      logits [256, 11, 128256] (722 MB per round), router 4096 -> 512 -> 1;
      100 resident rounds.
  single: one DFlash chain, K = 16, float32 logits [17, 151936] and the router
      on one float32 hidden state; a launch-latency-bound size, so every figure
      comes from replaying a captured HIP graph of 16 resident rounds.
  chain32: 32 DFlash chains, K = 16, bf16 logits [32, 17, 151936] with the
      router (its tiles share the sweep's launch).
  trees: 8 EAGLE-3 trees of 61 nodes over bf16 logits, no router; one step is
      whiflash_verify_tree.

Prints one JSON line (rounds/s, logits GB/s, roofline of the argmax sweep and
the CPU oracle baseline).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "argmax_sweep_traffic.json")
# Sources of the argmax sweep kernel: a change to any of them voids the stored counters.
SWEEP_SRCS = [os.path.join(ROOT, "drafter_routing_verification_amd", "csrc", f)
              for f in ("sweep.hip", "sweep_body.h", "elem.h", "dpp.h")]


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", choices=["sweep", "routed", "llama", "single", "chain32", "trees"],
                   default="sweep",
                   help="sweep: 256 chains at Qwen3-4B shapes (default); routed: the 64/64 "
                        "chain/tree mix; llama: 256 chains at Llama-3.1-8B shapes; single: one "
                        "sequence, K = 16, float32 logits and router (latency-bound; timed by "
                        "replaying a captured HIP graph of the steps); chain32: 32 chains of "
                        "K = 16 with the router; trees: 8 EAGLE-3 trees of 61 nodes, no router")
    p.add_argument("--pool", type=int, default=None,
                   help="distinct rounds resident in HBM (default: 100 for the sweep workload, "
                        "4 for the routed early-exit mode)")
    p.add_argument("--mode", choices=["fused", "separate", "early-exit", "entropy",
                                      "entropy-separate"], default="fused",
                   help="sweep workload: whiflash_round_chain (fused) or whiflash_route then "
                        "whiflash_verify_chain (separate); routed workload: "
                        "whiflash_round_routed, whiflash_route then "
                        "whiflash_verify_routed, or whiflash_round_routed_early_exit over a pool "
                        "of --pool rounds; entropy: the WhiFlash-Entropy round "
                        "whiflash_verify_routed_entropy (entropy-separate: whiflash_verify_routed "
                        "then whiflash_route_entropy); sweep workload: early-exit verifies with "
                        "whiflash_verify_chain_early_exit (rows up to the first mismatch only)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-touch", action="store_true",
                   help="skip the setup pass that reads every resident round once before the "
                        "warm-up (the first sweep over a freshly written round runs slower)")
    p.add_argument("--no-size-fit", action="store_true",
                   help="skip the sweep launches over partial rounds (profiler runs use this, so "
                        "every argmax_sweep_kernel dispatch they record covers whole rounds)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--router-width", type=int, default=None,
                   help="router hidden width m for the chain workloads (sweep, chain32, llama); "
                        "default 1024 (512 for llama).  The paper's router uses m = d/8: 320 "
                        "at the Qwen3-4B hidden size 2560")
    return p.parse_args()


def _to_dev(a, torch, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def _sweep_source_hash() -> str:
    h = hashlib.sha256()
    for path in SWEEP_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, launches_bytes: float):
    """HBM bytes per launch of the sweep kernel alone (the unit `achieved` is timed on), from
    the committed counter summary, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("sweep_source_sha256_16") != _sweep_source_hash():
        return None
    return entry.get("sweep_kernel_hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU oracle baseline


def _argmax_worker(conn, raw, dtype):
    """Child process of the parallel CPU baseline: the oracle's row argmax over its own block
    of logits rows, once per request on the pipe, until it is told to stop."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        while conn.recv():
            conn.send(oracle.row_argmax(raw, dtype))
    conn.close()


def _cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo)."""
    import subprocess
    try:
        res = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in res.stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The GPU hosts give one job with one GPU a share of 16 CPUs, however many the host has or
# os.sched_getaffinity shows, so the parallel oracle leg runs at most this many processes.
CPU_SHARE = 16


def _cpu_baseline(raw, dtype, route, accept, what, budget_s):
    """Whole rounds of the oracle (route() -> (delta_al, choices); the row argmax of every
    logits row; accept(t, choices) -> dict of results), timed on the host cores in two ways:
    one process on one thread, and P processes (P - 1 children each take a contiguous block of
    rows for the argmax while the parent runs the router, then the parent runs the
    acceptance).  Process start-up and the hand-over of the rows to the children are outside
    the timed rounds.  Returns (baseline, results of the first round), the latter for the
    bench's parity check of the same round on the GPU."""
    import multiprocessing as mp
    import oracle
    from threadpoolctl import threadpool_limits
    rounds, spent, first = 0, 0.0, None
    with threadpool_limits(limits=1):
        while spent < budget_s:
            t0 = time.perf_counter()
            dal, choice = route()
            t = oracle.row_argmax(raw, dtype)
            res = accept(t, choice)
            spent += time.perf_counter() - t0
            rounds += 1
            if first is None:
                first = dict(res, rows=t, dal=dal, choice=choice)
    affinity = len(os.sched_getaffinity(0))
    P = min(CPU_SHARE, affinity)
    out = {"value": rounds / spent, "unit": "rounds/s", "cores": 1, "kind": "oracle",
           "sample": f"{rounds} whole rounds ({what}); {spent:.1f} s of CPU work on one thread",
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
           "parallel_cap": f"{CPU_SHARE} processes: the CPU share a one-GPU job gets on the "
                           "GPU host"}
    if P < 2:
        return out, first
    ctx = mp.get_context("spawn")
    conns, procs = [], []
    try:
        for blk in np.array_split(np.arange(raw.shape[0]), P - 1):
            parent_end, child_end = ctx.Pipe()
            pr = ctx.Process(target=_argmax_worker, daemon=True,
                             args=(child_end, raw[blk[0]:blk[-1] + 1], dtype))
            pr.start()
            conns.append(parent_end)
            procs.append(pr)
        for c in conns:                      # one untimed round: the children are ready
            c.send(True)
        for c in conns:
            c.recv()
        prounds, pspent = 0, 0.0
        with threadpool_limits(limits=1):
            while pspent < budget_s / 2:
                t0 = time.perf_counter()
                for c in conns:
                    c.send(True)
                _, choice = route()
                accept(np.concatenate([c.recv() for c in conns]), choice)
                pspent += time.perf_counter() - t0
                prounds += 1
    finally:
        for c in conns:
            try:
                c.send(False)
            except OSError:
                pass
        for pr in procs:
            pr.join(timeout=30)
    out["parallel"] = {"value": prounds / pspent, "unit": "rounds/s", "cores": P,
                       "processes": P, "kind": "oracle",
                       "sample": f"{prounds} whole rounds; {P - 1} processes split the rows for "
                                 f"the argmax while the parent runs the router; {pspent:.1f} s"}
    return out, first


def _parity(gpu: dict, ref: dict, tau, rtol: float) -> dict:
    """Round 0 of the timed workload on the GPU against the oracle's first baseline round.
    Bit-exact: accept lengths, bonus tokens, best nodes and every row argmax (rows an
    early-exit schedule skipped hold -1 and are not compared); routing choices too, except
    for sequences whose exact gain lies within 1e-3 of the threshold (those, and what they
    route to, are not compared); delta-AL within rtol * max(|ref|, 1)."""
    bad = []
    detail = {"round": 0}
    far = None
    if ref.get("dal") is not None and gpu.get("dal") is not None:
        e = np.asarray(ref["dal"], np.float64)
        err = np.abs(np.asarray(gpu["dal"], np.float64) - e) / np.maximum(np.abs(e), 1.0)
        detail["dal_max_rel_err"] = float(err.max())
        detail["dal_tolerance"] = rtol
        if not err.max() <= rtol:
            bad.append(f"delta-AL error {err.max():.3e} > {rtol}")
        far = np.abs(e - float(np.float32(tau))) >= 1e-3
        detail["sequences_within_1e-3_of_threshold"] = int((~far).sum())
        if not np.array_equal(np.asarray(gpu["choice"])[far], np.asarray(ref["choice"])[far]):
            bad.append("routing choices differ")
    # Routed rounds verify with the GPU's own choices; sequences in the band may go either way.
    seq = far if (far is not None and gpu.get("routed")) else slice(None)
    for key in ("al", "bonus", "best"):
        if key in ref:
            g, r = np.asarray(gpu[key]), np.asarray(ref[key])
            if not np.array_equal(g[seq], r[seq]):
                bad.append(f"{key} differs at {int((g[seq] != r[seq]).sum())} sequences")
    g_rows, r_rows = np.asarray(gpu["rows"]), np.asarray(ref["rows"])
    read = g_rows != -1
    detail["rows_compared"] = int(read.sum())
    if not np.array_equal(g_rows[read], r_rows[read]):
        bad.append(f"row argmax differs at {int((g_rows[read] != r_rows[read]).sum())} rows")
    detail["sequences"] = int(np.asarray(ref["al"]).shape[0])
    detail["status"] = "ok" if not bad else "FAILED: " + "; ".join(bad)
    return detail


# ----------------------------------------------------------------------------- workloads


class Routed:
    name = "routed_bf16"

    def __init__(self, torch, dev, pool=1):
        """Round 0 is the seeded routed workload itself.  With pool > 1, rounds 1.. keep its
        router, layout and d2t table and draw fresh drafts and planted tokens (same generator,
        next round index), with their logits generated on the device."""
        from synth import make_config, make_routed_batch
        from synth.workloads import CONFIGS, PLANT_BOOST
        import drafter_routing_verification_amd as wf
        t0 = time.time()
        batch, r = make_config("routed_bf16")
        self.batch, self.router = batch, r
        self.V, self.rows, self.B = batch.V, batch.rows, batch.B
        self.d, self.m = r.d, r.m
        T = lambda a: _to_dev(a, torch, dev)
        self.hidden, self.W1, self.W2 = T(r.hidden), T(r.W1), T(r.W2)
        self.b1 = T(r.b1)
        self.b2 = torch.tensor([r.b2], dtype=torch.float32, device=dev)
        self.offsets, self.d2t = T(batch.offsets), T(batch.d2t)
        self.pool = [dict(logits=T(batch.logits), chain_draft=T(batch.chain_draft),
                          parent=T(batch.parent), draft_ids=T(batch.draft_ids))]
        c = CONFIGS["routed_bf16"]
        g = torch.Generator(device=dev)
        for rnd in range(1, pool):
            rb = make_routed_batch(c["seed"], batch.layout_choice, c["K"], c["N"], self.V,
                                   batch.d2t.shape[0], "bf16", 0.8, 0.7, rnd, logits=False)
            g.manual_seed(c["seed"] * 1_000_003 + rnd)
            x = torch.randn((self.rows, self.V), generator=g, device=dev, dtype=torch.float32)
            planted = torch.from_numpy(np.concatenate(rb.planted).astype(np.int64)).to(dev)
            x[torch.arange(self.rows, device=dev), planted] += PLANT_BOOST
            self.pool.append(dict(logits=x.to(torch.bfloat16), chain_draft=T(rb.chain_draft),
                                  parent=T(rb.parent), draft_ids=T(rb.draft_ids)))
            del x
        B = self.B
        self.dal = torch.empty(B, dtype=torch.float32, device=dev)
        self.choice = torch.empty(B, dtype=torch.int32, device=dev)
        self.al = torch.empty(B, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(B, dtype=torch.int32, device=dev)
        self.best = torch.empty(B, dtype=torch.int32, device=dev)
        self.rws = torch.empty(wf.route_workspace_bytes(B, r.m), dtype=torch.uint8, device=dev)
        self.vws = torch.empty(wf.verify_workspace_bytes(self.rows, self.V), dtype=torch.uint8,
                               device=dev)
        self.sweep_out = torch.empty(self.rows * wf.argmax_sweep_plan(self.rows, self.V)[0] * 2,
                                     dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.fws = torch.empty(wf.round_workspace_bytes(B, r.m, self.rows, self.V),
                               dtype=torch.uint8, device=dev)
        K, N = batch.K, batch.N
        self.ews = torch.empty(wf.routed_early_exit_workspace_bytes(B, K, N, self.rows, self.V),
                               dtype=torch.uint8, device=dev)
        self.efws = torch.empty(wf.round_early_exit_workspace_bytes(B, r.m, K, N, self.rows, self.V),
                                dtype=torch.uint8, device=dev)
        self.layout = T(batch.layout_choice)
        self.ent = torch.empty(B, dtype=torch.float32, device=dev)
        self.nxt = torch.empty(B, dtype=torch.int32, device=dev)
        self.entws = torch.empty(wf.verify_routed_entropy_workspace_bytes(B, self.rows, self.V),
                                 dtype=torch.uint8, device=dev)
        self.erws = torch.empty(wf.entropy_workspace_bytes(B, self.V), dtype=torch.uint8,
                                device=dev)
        self.early = False
        self.wf = wf
        self.setup_s = time.time() - t0
        esz = 2
        self.logits_bytes = self.rows * self.V * esz
        self.router_bytes = (r.hidden.size + r.W1.size + r.W2.size) * esz + r.b1.size * 4
        meta = (batch.offsets.size + B * batch.K + 2 * B * batch.N + batch.d2t.size + 5 * B) * 4
        self.step_bytes = self.logits_bytes + self.router_bytes + meta

    def use_early_exit(self):
        """Verify with the early-exit schedule; the bytes a round needs are those of the rows
        of its accepted nodes (the sum of accept lengths: sibling tokens are distinct, so the
        accepted nodes form one path), averaged over the pool."""
        self.early = True
        self.route(0)
        need = []
        for i in range(len(self.pool)):
            self.verify(i)
            need.append(int(self.al.sum().item()) * self.V * 2)
        self.needed_bytes = sum(need) / len(need)

    def route(self, i):
        r = self.router
        self.wf.route(self.hidden, self.W1, self.b1, self.W2, self.b2, r.tau, delta_al=self.dal,
                      choice=self.choice, workspace=self.rws)

    def sweep(self, i, rows=None):
        """The argmax sweep kernel alone over this round's logits (whiflash_argmax_sweep),
        or over its first `rows` rows."""
        p = self.pool[i % len(self.pool)]
        self.wf.argmax_sweep(p["logits"] if rows is None else p["logits"][:rows],
                             partials=self.sweep_out)

    def stream(self, i):
        """The sweep's reads without its comparisons (whiflash_stream_read)."""
        p = self.pool[i % len(self.pool)]
        self.wf.stream_read(p["logits"], sink=self.sink)

    def verify(self, i):
        p = self.pool[i % len(self.pool)]
        fn = self.wf.verify_routed_early_exit if self.early else self.wf.verify_routed
        fn(p["logits"], self.offsets, self.rows, self.choice, p["chain_draft"], p["parent"],
           p["draft_ids"], self.d2t, row_argmax=False, accept_len=self.al, bonus=self.bonus,
           best_node=self.best, workspace=self.ews if self.early else self.vws)

    # Entropy-policy threshold (nats): any fixed value; the decision is not fed back.
    TAU_ENTROPY = 6.0

    def entropy_step(self, i):
        """One WhiFlash-Entropy round: verify with this round's choices, and the entropy at each
        accepted row deciding the next round's drafter (one call)."""
        p = self.pool[i % len(self.pool)]
        self.wf.verify_routed_entropy(p["logits"], self.offsets, self.rows, self.layout, p["chain_draft"],
                                      p["parent"], p["draft_ids"], self.d2t, self.TAU_ENTROPY,
                                      row_argmax=False, accept_len=self.al, bonus=self.bonus,
                                      best_node=self.best, entropy=self.ent, next_choice=self.nxt,
                                      workspace=self.entws)

    def entropy_separate_step(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.verify_routed(p["logits"], self.offsets, self.rows, self.layout, p["chain_draft"],
                              p["parent"], p["draft_ids"], self.d2t, row_argmax=False,
                              accept_len=self.al, bonus=self.bonus, best_node=self.best,
                              workspace=self.vws)
        self.entropy_only(i)

    def entropy_only(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.route_entropy(p["logits"], self.best, self.TAU_ENTROPY, row0=self.offsets,
                              entropy=self.ent, choice=self.nxt, workspace=self.erws)

    def fused_step(self, i):
        r = self.router
        p = self.pool[i % len(self.pool)]
        fn = self.wf.round_routed_early_exit if self.early else self.wf.round_routed
        fn(self.hidden, self.W1, self.b1, self.W2, self.b2, r.tau, p["logits"], self.offsets,
           self.rows, p["chain_draft"], p["parent"], p["draft_ids"], self.d2t, row_argmax=False,
           delta_al=self.dal, choice=self.choice, accept_len=self.al, bonus=self.bonus,
           best_node=self.best, workspace=self.efws if self.early else self.fws)

    def check(self):
        al = self.al.cpu().numpy()
        ch = self.choice.cpu().numpy()
        assert np.array_equal(ch, self.batch.layout_choice), "router choice differs from the layout"
        assert al.min() >= 1, "a sequence came out malformed"
        return float(al.mean())

    def cpu_baseline(self, budget_s):
        """The oracle on whole rounds of this workload (router, argmax of every row, chain and
        tree acceptance), repeated until the CPU budget is spent."""
        import oracle
        b, r = self.batch, self.router

        def route():
            return oracle.route(r.hidden, r.W1, r.b1, r.W2, r.b2, r.tau, r.dtype)

        def accept(t, choice):
            al, bo, be = oracle.verify_routed(t, b.offsets, choice, b.K, b.chain_draft, b.N,
                                              b.parent, b.draft_ids, b.d2t, b.V)
            return {"al": al, "bonus": bo, "best": be}
        what = (f"router on {b.B} hidden states, argmax of all {self.rows} rows, routed "
                "acceptance")
        return _cpu_baseline(b.logits, b.dtype, route, accept, what, budget_s)

    def gpu_round0(self, fused, entropy):
        """Round 0 through the timed step's own entry point, with every row's argmax."""
        r, p, wf = self.router, self.pool[0], self.wf
        H = lambda t: t.cpu().numpy()
        common = (p["logits"], self.offsets, self.rows)
        tree = (p["chain_draft"], p["parent"], p["draft_ids"], self.d2t)
        if entropy:
            al, bo, be, rows = wf.verify_routed(*common, self.layout, *tree)[:4]
            return {"al": H(al), "bonus": H(bo), "best": H(be), "rows": H(rows)}
        if fused:
            fn = wf.round_routed_early_exit if self.early else wf.round_routed
            dal, ch, al, bo, be, rows = fn(self.hidden, self.W1, self.b1, self.W2, self.b2, r.tau,
                                           *common, *tree)
        else:
            dal, ch = wf.route(self.hidden, self.W1, self.b1, self.W2, self.b2, r.tau)
            fn = wf.verify_routed_early_exit if self.early else wf.verify_routed
            al, bo, be, rows = fn(*common, ch, *tree)
        return {"dal": H(dal), "choice": H(ch), "al": H(al), "bonus": H(bo), "best": H(be),
                "rows": H(rows), "routed": True}


class Sweep:
    name = "sweep_bf16"

    @staticmethod
    def shape():
        """(seed, B, K, V, d, m) of the throughput sweep at the Qwen3-4B shapes."""
        from synth.workloads import CONFIGS, D_QWEN3, ROUTER_M, V_QWEN3
        c = CONFIGS["sweep_bf16"]
        return c["seed"], c["B"], c["K"], V_QWEN3, D_QWEN3, ROUTER_M

    def __init__(self, torch, dev, pool, router_width=None):
        from synth import make_chain_batch, make_router_inputs
        from synth.workloads import PLANT_BOOST
        import drafter_routing_verification_amd as wf
        t0 = time.time()
        seed, self.B, self.K, self.V, self.d, m = self.shape()
        if router_width:
            m = router_width
        self.rows = self.B * (self.K + 1)
        self.pool = []
        g = torch.Generator(device=dev)
        for rnd in range(pool):
            cb = make_chain_batch(seed, self.B, self.K, self.V, "bf16", 0.8, rnd, logits=False)
            r = make_router_inputs(seed, self.B, self.d, m, dtype="bf16", rnd=rnd)
            g.manual_seed(seed * 1_000_003 + rnd)
            x = torch.randn((self.rows, self.V), generator=g, device=dev, dtype=torch.float32)
            planted = torch.from_numpy(cb.planted.reshape(-1).astype(np.int64)).to(dev)
            x[torch.arange(self.rows, device=dev), planted] += PLANT_BOOST
            logits = x.to(torch.bfloat16)
            del x
            self.pool.append(dict(logits=logits, draft=_to_dev(cb.draft, torch, dev),
                                  hidden=_to_dev(r.hidden, torch, dev)))
            if rnd == 0:
                self.W1, self.W2 = _to_dev(r.W1, torch, dev), _to_dev(r.W2, torch, dev)
                self.b1 = _to_dev(r.b1, torch, dev)
                self.m, self.tau = r.m, r.tau
                self.router_bytes = (r.hidden.size + r.W1.size + r.W2.size) * 2 + r.b1.size * 4
        self.dal = torch.empty(self.B, dtype=torch.float32, device=dev)
        self.choice = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.al = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.rws = torch.empty(wf.route_workspace_bytes(self.B, self.m), dtype=torch.uint8, device=dev)
        self.vws = torch.empty(wf.verify_workspace_bytes(self.rows, self.V), dtype=torch.uint8,
                               device=dev)
        self.sweep_out = torch.empty(self.rows * wf.argmax_sweep_plan(self.rows, self.V)[0] * 2,
                                     dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ews = torch.empty(wf.early_exit_workspace_bytes(self.B, self.K, self.V),
                               dtype=torch.uint8, device=dev)
        self.cws = torch.empty(wf.round_chain_workspace_bytes(self.B, self.m, self.K, self.V),
                               dtype=torch.uint8, device=dev)
        self.ecws = torch.empty(
            wf.round_chain_early_exit_workspace_bytes(self.B, self.m, self.K, self.V),
            dtype=torch.uint8, device=dev)
        self.early = False
        self.wf = wf
        self.setup_s = time.time() - t0
        self.logits_bytes = self.rows * self.V * 2
        self.step_bytes = self.logits_bytes + self.router_bytes + (self.B * self.K + 4 * self.B) * 4

    def use_early_exit(self):
        """Verify with the early-exit schedule; the bytes it needs per round are those of
        rows 0..n of every sequence (sum of accept lengths), averaged over the pool."""
        self.early = True
        need = []
        for i in range(len(self.pool)):
            self.verify(i)
            need.append(int(self.al.sum().item()) * self.V * 2)
        self.needed_bytes = sum(need) / len(need)

    def route(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.route(p["hidden"], self.W1, self.b1, self.W2, None, self.tau, delta_al=self.dal,
                      choice=self.choice, workspace=self.rws)

    def fused_step(self, i):
        """route + verify_chain in one call (whiflash_round_chain, or its early-exit form)."""
        p = self.pool[i % len(self.pool)]
        fn = self.wf.round_chain_early_exit if self.early else self.wf.round_chain
        fn(p["hidden"], self.W1, self.b1, self.W2, None, self.tau, p["logits"], p["draft"],
           row_argmax=False, delta_al=self.dal, choice=self.choice, accept_len=self.al,
           bonus=self.bonus, workspace=self.ecws if self.early else self.cws)

    def sweep(self, i, rows=None):
        """The argmax sweep kernel alone over this round's logits (whiflash_argmax_sweep),
        or over its first `rows` rows."""
        p = self.pool[i % len(self.pool)]
        self.wf.argmax_sweep(p["logits"] if rows is None else p["logits"][:rows],
                             partials=self.sweep_out)

    def stream(self, i):
        """The sweep's reads without its comparisons (whiflash_stream_read)."""
        p = self.pool[i % len(self.pool)]
        self.wf.stream_read(p["logits"], sink=self.sink)

    def verify(self, i):
        p = self.pool[i % len(self.pool)]
        if self.early:
            self.wf.verify_chain_early_exit(p["logits"], p["draft"], row_argmax=False,
                                            accept_len=self.al, bonus=self.bonus,
                                            workspace=self.ews)
        else:
            self.wf.verify_chain(p["logits"], p["draft"], row_argmax=False, accept_len=self.al,
                                 bonus=self.bonus, workspace=self.vws)

    def check(self):
        al = self.al.cpu().numpy()
        assert al.min() >= 1 and al.max() <= self.K + 1
        return float(al.mean())

    def cpu_baseline(self, budget_s):
        """The oracle on round 0 of the pool (router, argmax of every row, chain acceptance),
        repeated until the CPU budget is spent."""
        import oracle
        import torch
        p = self.pool[0]
        raw = p["logits"].view(torch.int16).cpu().numpy().view(np.uint16)
        draft = p["draft"].cpu().numpy()
        bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        hidden, W1, W2, b1 = bits(p["hidden"]), bits(self.W1), bits(self.W2), self.b1.cpu().numpy()

        def route():
            return oracle.route(hidden, W1, b1, W2, 0.0, self.tau, "bf16")

        def accept(t, choice):
            al, bo = oracle.verify_chain(t.reshape(self.B, self.K + 1), draft)
            return {"al": al, "bonus": bo}
        what = f"router on {self.B} hidden states, argmax of all {self.rows} rows, chain acceptance"
        return _cpu_baseline(raw, "bf16", route, accept, what, budget_s)

    def gpu_round0(self, fused, entropy=False):
        """Round 0 through the timed step's own entry point, with every row's argmax."""
        p, wf = self.pool[0], self.wf
        H = lambda t: t.cpu().numpy()
        if fused:
            fn = wf.round_chain_early_exit if self.early else wf.round_chain
            dal, ch, al, bo, rows = fn(p["hidden"], self.W1, self.b1, self.W2, None, self.tau,
                                       p["logits"], p["draft"])
        else:
            dal, ch = wf.route(p["hidden"], self.W1, self.b1, self.W2, None, self.tau)
            fn = wf.verify_chain_early_exit if self.early else wf.verify_chain
            al, bo, rows = fn(p["logits"], p["draft"])
        return {"dal": H(dal), "choice": H(ch), "al": H(al), "bonus": H(bo), "rows": H(rows)}


class LlamaSweep(Sweep):
    """The same throughput sweep at Llama-3.1-8B shapes: DFlash blocks of 10 drafts (WhiFlash
    paper, Appendix A, Table 7), a 128,256-token vocabulary, hidden 4096 and a router of
    width 512 (the paper's d/8 rule)."""
    name = "llama_sweep_bf16"

    @staticmethod
    def shape():
        return 6, 256, 10, 128_256, 4_096, 512


class Chain32(Sweep):
    """32 DFlash chains of K = 16 over the 151,936-token vocabulary with the 2560 -> 1024
    router: the batched chain configuration, 170.7 MB of bf16 logits per round."""
    name = "batched_chain_bf16"

    @staticmethod
    def shape():
        from synth.workloads import CONFIGS, D_QWEN3, ROUTER_M, V_QWEN3
        c = CONFIGS["batched_chain_bf16"]
        return c["seed"], c["B"], c["K"], V_QWEN3, D_QWEN3, ROUTER_M


class Trees:
    """EAGLE-3 tree verification alone: 8 trees of 61 nodes (root + 60 drafts, depth <= 8,
    <= 10 children per node) over the 151,936-token vocabulary with the 32,000-entry d2t
    remap, bf16 logits (148.3 MB per round).  This configuration has no router."""
    name = "tree_bf16"

    def __init__(self, torch, dev, pool):
        from synth import make_tree_batch
        from synth.workloads import CONFIGS, PLANT_BOOST, V_QWEN3, VD_EAGLE3
        import drafter_routing_verification_amd as wf
        t0 = time.time()
        c = CONFIGS["tree_bf16"]
        self.B, self.N, self.V = c["B"], c["N"], V_QWEN3
        self.rows = self.B * self.N
        self.depth_bound = 8
        self.d = self.m = None
        self.pool = []
        g = torch.Generator(device=dev)
        for rnd in range(pool):
            tb = make_tree_batch(c["seed"], self.B, self.N, self.V, VD_EAGLE3, "bf16", 0.7,
                                 self.depth_bound, 10, rnd, logits=False)
            g.manual_seed(c["seed"] * 1_000_003 + rnd)
            x = torch.randn((self.rows, self.V), generator=g, device=dev, dtype=torch.float32)
            planted = torch.from_numpy(tb.planted.reshape(-1).astype(np.int64)).to(dev)
            x[torch.arange(self.rows, device=dev), planted] += PLANT_BOOST
            self.pool.append(dict(logits=x.to(torch.bfloat16),
                                  parent=_to_dev(tb.parent, torch, dev),
                                  ids=_to_dev(tb.draft_ids, torch, dev)))
            del x
            if rnd == 0:
                self.d2t = _to_dev(tb.d2t, torch, dev)
        new = lambda: torch.empty(self.B, dtype=torch.int32, device=dev)
        self.al, self.bonus, self.best = new(), new(), new()
        self.vws = torch.empty(wf.verify_workspace_bytes(self.rows, self.V), dtype=torch.uint8,
                               device=dev)
        self.sweep_out = torch.empty(self.rows * wf.argmax_sweep_plan(self.rows, self.V)[0] * 2,
                                     dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.early = False
        self.wf = wf
        self.setup_s = time.time() - t0
        self.logits_bytes = self.rows * self.V * 2
        self.step_bytes = self.logits_bytes + 2 * self.rows * 4 + 5 * self.B * 4 + tb.d2t.size * 4

    def route(self, i):
        """No router in this configuration."""

    def verify(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.verify_tree(p["logits"], p["parent"], p["ids"], self.d2t, row_argmax=False,
                            accept_len=self.al, bonus=self.bonus, best_node=self.best,
                            workspace=self.vws)

    sweep = Sweep.sweep
    stream = Sweep.stream

    def check(self):
        al = self.al.cpu().numpy()
        assert al.min() >= 1 and al.max() <= self.depth_bound + 1
        return float(al.mean())

    def cpu_baseline(self, budget_s):
        """The oracle on round 0 of the pool (argmax of every row, tree acceptance with the
        d2t remap), repeated until the CPU budget is spent."""
        import oracle
        import torch
        p = self.pool[0]
        raw = p["logits"].view(torch.int16).cpu().numpy().view(np.uint16)
        parent, ids, d2t = p["parent"].cpu().numpy(), p["ids"].cpu().numpy(), self.d2t.cpu().numpy()

        def accept(t, choice):
            al, bo, be = oracle.verify_tree(t.reshape(self.B, self.N), parent, ids, d2t, self.V)
            return {"al": al, "bonus": bo, "best": be}
        what = f"argmax of all {self.rows} rows, acceptance of {self.B} trees"
        return _cpu_baseline(raw, "bf16", lambda: (None, None), accept, what, budget_s)

    def gpu_round0(self, fused=False, entropy=False):
        p = self.pool[0]
        H = lambda t: t.cpu().numpy()
        al, bo, be, rows = self.wf.verify_tree(p["logits"], p["parent"], p["ids"], self.d2t)
        return {"al": H(al), "bonus": H(bo), "best": H(be), "rows": H(rows)}


class Single:
    """One sequence: a DFlash block of 16 drafts over 151,936 float32 logits and the router
    2560 -> 1024 on one float32 hidden state.  A launch-latency-bound step, so its launches
    are timed by replaying a captured HIP graph: the Python binding's per-call overhead would
    otherwise set the pace.  The pool's rounds (16 x 20.8 MB) exceed the 256 MB Infinity Cache."""
    name = "single_chain_f32"
    graph = True

    def __init__(self, torch, dev, pool):
        from synth import make_config
        import drafter_routing_verification_amd as wf
        t0 = time.time()
        self.pool = []
        for rnd in range(pool):
            batch, r = make_config("single_chain_f32", rnd=rnd)
            self.pool.append(dict(logits=_to_dev(batch.logits, torch, dev),
                                  draft=_to_dev(batch.draft, torch, dev),
                                  hidden=_to_dev(r.hidden, torch, dev),
                                  W1=_to_dev(r.W1, torch, dev), W2=_to_dev(r.W2, torch, dev),
                                  b1=_to_dev(r.b1, torch, dev)))
            if rnd == 0:
                self.B, self.K, self.V = batch.B, batch.K, batch.V
                self.d, self.m, self.tau = r.d, r.m, r.tau
                self.router_bytes = (r.hidden.size + r.W1.size + r.W2.size + r.b1.size) * 4
                self.host0 = (batch, r)
        self.rows = self.B * (self.K + 1)
        self.dal = torch.empty(self.B, dtype=torch.float32, device=dev)
        self.choice = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.al = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.rws = torch.empty(wf.route_workspace_bytes(self.B, self.m), dtype=torch.uint8, device=dev)
        self.vws = torch.empty(wf.verify_workspace_bytes(self.rows, self.V), dtype=torch.uint8,
                               device=dev)
        self.cws = torch.empty(wf.round_chain_workspace_bytes(self.B, self.m, self.K, self.V),
                               dtype=torch.uint8, device=dev)
        self.sweep_out = torch.empty(self.rows * wf.argmax_sweep_plan(self.rows, self.V)[0] * 2,
                                     dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.early = False
        self.wf = wf
        self.setup_s = time.time() - t0
        self.logits_bytes = self.rows * self.V * 4
        self.step_bytes = self.logits_bytes + self.router_bytes + (self.B * self.K + 4 * self.B) * 4

    def fused_step(self, i):
        """route + verify_chain in one call (whiflash_round_chain: two launches at one sequence)."""
        p = self.pool[i % len(self.pool)]
        self.wf.round_chain(p["hidden"], p["W1"], p["b1"], p["W2"], None, self.tau, p["logits"],
                            p["draft"], row_argmax=False, delta_al=self.dal, choice=self.choice,
                            accept_len=self.al, bonus=self.bonus, workspace=self.cws)

    def route(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.route(p["hidden"], p["W1"], p["b1"], p["W2"], None, self.tau, delta_al=self.dal,
                      choice=self.choice, workspace=self.rws)

    def verify(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.verify_chain(p["logits"], p["draft"], row_argmax=False, accept_len=self.al,
                             bonus=self.bonus, workspace=self.vws)

    def sweep(self, i, rows=None):
        p = self.pool[i % len(self.pool)]
        self.wf.argmax_sweep(p["logits"] if rows is None else p["logits"][:rows],
                             partials=self.sweep_out)

    def stream(self, i):
        p = self.pool[i % len(self.pool)]
        self.wf.stream_read(p["logits"], sink=self.sink)

    def check(self):
        al = self.al.cpu().numpy()
        assert al.min() >= 1 and al.max() <= self.K + 1
        return float(al.mean())

    def cpu_baseline(self, budget_s):
        """The oracle on round 0 (router in float64, argmax of the 17 rows, chain acceptance)."""
        import oracle
        batch, r = self.host0

        def route():
            return oracle.route(r.hidden, r.W1, r.b1, r.W2, np.float32(r.b2), r.tau, "f32")

        def accept(t, choice):
            al, bo = oracle.verify_chain(t.reshape(self.B, self.K + 1), batch.draft)
            return {"al": al, "bonus": bo}
        what = f"router on one float32 hidden state, argmax of all {self.rows} float32 rows, chain acceptance"
        return _cpu_baseline(batch.logits, "f32", route, accept, what, budget_s)

    def gpu_round0(self, fused=True, entropy=False):
        p = self.pool[0]
        H = lambda t: t.cpu().numpy()
        dal, ch, al, bo, rows = self.wf.round_chain(p["hidden"], p["W1"], p["b1"], p["W2"], None,
                                                    self.tau, p["logits"], p["draft"])
        return {"dal": H(dal), "choice": H(ch), "al": H(al), "bonus": H(bo), "rows": H(rows)}


def _graph_loop(torch, work, fn, outs, n):
    """Average duration of fn(i) when len(work.pool) consecutive calls are captured in one HIP
    graph and the graph is replayed back to back (n calls in all, at least one replay).  Before
    timing, three replays are checked against eager calls: `outs` are the tensors fn writes,
    which hold the graph's last call's results after a replay."""
    k = len(work.pool)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(k):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(k):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(3):
        fn(k - 1)
        torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        for t in outs:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(outs, want)):
            raise RuntimeError("a graph replay differs from the eager calls")
    reps = max(1, n // k)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * k) / 1000.0


def _bench_graph(args, torch, work):
    """The single-sequence line: every figure from HIP graph replay (see _graph_loop)."""
    for i in range(args.warmup):
        work.fused_step(i)
    torch.cuda.synchronize()
    mean_al = work.check()
    k = len(work.pool)
    reps = max(1, -(-args.steps // k))
    steps = reps * k
    T = lambda fn, outs: _graph_loop(torch, work, fn, outs, steps)
    step_s = T(work.fused_step, (work.al, work.bonus, work.dal, work.choice))
    work.check()
    route_s = T(work.route, (work.dal, work.choice))
    verify_s = T(work.verify, (work.al, work.bonus))
    sweep_s = T(work.sweep, (work.sweep_out,))
    stream_s = T(work.stream, (work.sink,))
    # For context: the same step launched from Python, back to back.
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        work.fused_step(i)
    b.record()
    torch.cuda.synchronize()
    python_us = a.elapsed_time(b) / steps * 1000.0
    B_ = work.logits_bytes
    return {
        "metric": "verify+route rounds/s and logits HBM GB/s (fraction of MI355X peak), 1 GPU",
        "value": round(1.0 / step_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; planted-argmax logits, random router weights)",
        "config": {"workload": work.name, "mode": "whiflash_round_chain, HIP graph replay",
                   "batch": work.B, "logits_rows": work.rows, "vocab": work.V,
                   "hidden": work.d, "router_width": work.m, "rounds_resident": len(work.pool),
                   "logits_bytes_per_round": B_, "bytes_per_round": work.step_bytes},
        "logits_GBps": round(B_ / verify_s / 1e9, 1),
        "route_us": round(route_s * 1e6, 2),
        "verify_us": round(verify_s * 1e6, 2),
        "sweep_us": round(sweep_s * 1e6, 2),
        "stream_read": {"what": "whiflash_stream_read, graph replay", "us": round(stream_s * 1e6, 2),
                        "GBps": round(B_ / stream_s / 1e9, 1),
                        "frac": round(B_ / stream_s / 1e9 / HBM_PEAK_GBS, 4)},
        "python_launch_us": round(python_us, 2),
        "mean_accept_len": round(mean_al, 3),
        "roofline": {
            "kernel": "argmax_sweep_kernel alone (whiflash_argmax_sweep), graph replay; bytes = "
                      "the 17 float32 logits rows; a launch-latency-bound size",
            "bound": "hbm",
            "achieved": round(B_ / sweep_s / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(B_ / sweep_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }


# ----------------------------------------------------------------------------- main


# Workgroups resident at once on the GPU: 256 CUs x 8 workgroups of 4 waves (32 waves per CU).
RESIDENT_WORKGROUPS = 2048


def _sweep_size_fit(work, timed_loop, n):
    """Least-squares line through the sweep kernel's durations at four launch sizes.  A
    launch under two rounds of the resident workgroups is latency-bound (its duration barely
    grows with its bytes), so when the smallest size is one the fit is skipped."""
    sizes = [work.rows * q // 4 for q in (1, 2, 3, 4)]
    smallest = sizes[0] * work.wf.argmax_sweep_plan(sizes[0], work.V)[0]
    if smallest < 2 * RESIDENT_WORKGROUPS:
        return {"skipped": f"a quarter round is {smallest} workgroups, under two rounds of the "
                           f"{RESIDENT_WORKGROUPS} resident slots: too small for a linear fit"}
    us = [timed_loop(lambda i, r=r: work.sweep(i, rows=r), n) * 1e6 for r in sizes]
    nbytes = [r * work.V * 2 for r in sizes]
    slope, fixed = np.polyfit(np.array(nbytes, np.float64), np.array(us, np.float64), 1)
    rate = 1e-3 / slope  # GB/s
    return {"what": "whiflash_argmax_sweep over the first rows of each resident round, "
                    "back-to-back launches; duration = fixed_us + bytes / steady_GBps",
            "rows": sizes, "us": [round(u, 2) for u in us],
            "fixed_us": round(float(fixed), 2), "steady_GBps": round(float(rate), 1),
            "steady_frac": round(float(rate) / HBM_PEAK_GBS, 4)}


def _touch_pool(torch, work):
    """Setup, before the warm-up: one streaming read (whiflash_stream_read, no comparisons,
    nothing kept) over the logits of every resident round.  The first sweep over a round that
    was just written runs measurably slower than later ones, and the timed steps should see
    rounds the way a serving loop sees its reused buffers.  Returns the pass's duration."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(len(work.pool)):
        work.stream(i)
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) * 1e3, 2)


def main():
    args = _parse()
    if args.router_width is not None and (args.router_width < 1 or
                                          args.workload not in ("sweep", "chain32", "llama")):
        print("--router-width takes a positive width and applies to the sweep, chain32 and "
              "llama workloads", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (sequences are "
              "independent, so N GPUs would each run this step on B/N sequences)", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload == "routed":
        work = Routed(torch, dev, (args.pool or 4) if args.mode == "early-exit" else 1)
    elif args.workload == "llama":
        work = LlamaSweep(torch, dev, args.pool or 100, args.router_width)
    elif args.workload == "single":
        if args.mode != "fused":
            print("--workload single times whiflash_round_chain (--mode fused) only",
                  file=sys.stderr)
            sys.exit(2)
        work = Single(torch, dev, args.pool or 16)
        print(f"# workload {work.name}: inputs resident in HBM ({work.setup_s:.1f} s setup)",
              file=sys.stderr, flush=True)
        out = _bench_graph(args, torch, work)
        _finish(out, work, args, fused=True, entropy=False, rtol=1e-4, tau=work.tau)
        return
    elif args.workload == "chain32":
        work = Chain32(torch, dev, args.pool or 100, args.router_width)
    elif args.workload == "trees":
        if args.mode not in ("fused", "separate"):
            print("--workload trees times whiflash_verify_tree only", file=sys.stderr)
            sys.exit(2)
        work = Trees(torch, dev, args.pool or 100)
    else:
        work = Sweep(torch, dev, args.pool or 100, args.router_width)
    stream = torch.cuda.current_stream()
    print(f"# workload {work.name}: inputs resident in HBM ({work.setup_s:.1f} s setup)",
          file=sys.stderr, flush=True)
    touch_ms = None if args.no_touch else _touch_pool(torch, work)

    early = args.mode == "early-exit"
    entropy = args.mode in ("entropy", "entropy-separate")
    if entropy and not hasattr(work, "entropy_step"):
        print("--mode entropy applies to the routed workload", file=sys.stderr)
        sys.exit(2)
    # The early-exit step of either workload is its fused early-exit round.
    fused = args.mode in ("fused", "early-exit") and hasattr(work, "fused_step")
    if early:
        work.use_early_exit()
    if entropy:
        # This round's drafter choices are the layout's; the entropy decides the next round's.
        work.choice.copy_(work.layout)
        entropy_step = work.entropy_step if args.mode == "entropy" else work.entropy_separate_step

    def step(i):
        if entropy:
            entropy_step(i)
        elif fused:
            work.fused_step(i)
        else:
            work.route(i)
            work.verify(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    mean_al = work.check()

    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_total_ms = start.elapsed_time(end)
    work.check()

    # Diagnostics outside the timed region: the same calls, one kind at a time,
    # back to back on the same stream, bracketed by one pair of HIP events.
    def timed_loop(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n / 1000.0

    def step_distribution(fn, n):
        """Per-step durations (HIP events around each step, launched back to back)."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(n):
            fn(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1000.0 for i in range(n)])
        return {"p10": round(float(np.percentile(us, 10)), 2),
                "p50": round(float(np.percentile(us, 50)), 2),
                "p90": round(float(np.percentile(us, 90)), 2), "steps": n}

    step_us = step_distribution(step, min(K, 200))
    if entropy:
        # The whole entropy round is the verify call; "route" is the separate entropy pass.
        verify_s = timed_loop(entropy_step, K)
        route_s = timed_loop(work.entropy_only, K)
    else:
        verify_s = timed_loop(work.verify, K)
        route_s = timed_loop(work.route, K) if work.m else None
    # The dominant kernel alone: whiflash_argmax_sweep launches only the argmax sweep, on the
    # same stream, over the same resident rounds.
    sweep_s = None if early else timed_loop(work.sweep, K)
    # A streaming-read ceiling on the same buffers: the sweep's loads without its comparisons.
    stream_s = None if early else timed_loop(work.stream, K)

    # The sweep kernel's fixed cost per launch (ramp-up, drain, dispatch) and its steady
    # streaming rate: the same launches over the first quarter, half, three quarters and all
    # of each resident round's rows, fitted as duration = fixed + bytes / rate.
    size_fit = None if early or args.no_size_fit else _sweep_size_fit(work, timed_loop, K)

    ms_per_step = gpu_total_ms / K
    rounds_per_s = 1000.0 / ms_per_step
    # Algorithmic bytes of the verify call: every logits row, or with the early-exit
    # schedule only rows 0..n of each sequence (what it must read at the least).
    alg_bytes = work.needed_bytes if early else work.logits_bytes
    achieved = alg_bytes / verify_s / 1e9
    # Roofline of the dominant kernel: the argmax sweep's launches on their own (the
    # early-exit schedules interleave their sweep with preparation and acceptance, so there
    # the whole call is the unit).
    kernel_bytes_per_s = alg_bytes / (verify_s if early else sweep_s)
    traffic = None if early else _traffic(work.name, work.logits_bytes)
    mode = ("whiflash_verify_routed_entropy" if args.mode == "entropy" else
            "whiflash_verify_routed + whiflash_route_entropy" if args.mode == "entropy-separate" else
            "whiflash_round_routed_early_exit" if fused and early and isinstance(work, Routed) else
            "whiflash_round_chain_early_exit" if fused and early else
            "whiflash_round_routed" if fused and isinstance(work, Routed) else
            "whiflash_round_chain" if fused else
            "whiflash_route + whiflash_verify_chain_early_exit" if early else
            "whiflash_verify_tree" if isinstance(work, Trees) else
            "whiflash_route + whiflash_verify_*")
    out = {
        "metric": "verify+route rounds/s and logits HBM GB/s (fraction of MI355X peak), 1 GPU",
        "value": round(rounds_per_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; planted-argmax logits, random trees, random router weights)",
        "config": {"workload": work.name, "mode": mode, "batch": work.B, "logits_rows": work.rows,
                   "vocab": work.V, "hidden": work.d, "router_width": work.m,
                   "rounds_resident": len(work.pool),
                   "logits_bytes_per_round": work.logits_bytes,
                   "bytes_per_round": work.step_bytes},
        "logits_GBps": round(achieved, 1),
        "route_us": None if route_s is None else round(route_s * 1e6, 2),
        "verify_us": round(verify_s * 1e6, 2),
        **({} if early else {"sweep_us": round(sweep_s * 1e6, 2)}),
        **({} if early else {"stream_read": {
            "what": "whiflash_stream_read: the sweep's chunks and loads without its comparisons, "
                    "back-to-back launches over the same resident rounds",
            "us": round(stream_s * 1e6, 2),
            "GBps": round(work.logits_bytes / stream_s / 1e9, 1),
            "frac": round(work.logits_bytes / stream_s / 1e9 / HBM_PEAK_GBS, 4),
            "sweep_over_stream": round(sweep_s / stream_s, 4)}}),
        **({} if size_fit is None else {"sweep_size_fit": size_fit}),
        "wall_ms_per_step": round(wall * 1000 / K, 5),
        "setup_touch_ms": touch_ms,
        "step_us": step_us,
        "mean_accept_len": round(mean_al, 3),
        **({"logits_bytes_needed_per_round": round(alg_bytes)} if early else {}),
        "roofline": {
            "kernel": ("whiflash_verify_*_early_exit call: preparation + early-exit sweep + "
                       "acceptance, back to back; bytes = rows of accepted nodes" if early else
                       "argmax_sweep_kernel alone (whiflash_argmax_sweep), back-to-back launches; "
                       "bytes = every logits row of the round"),
            "bound": "hbm",
            "achieved": round(kernel_bytes_per_s / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kernel_bytes_per_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    tau = work.router.tau if isinstance(work, Routed) else getattr(work, "tau", None)
    _finish(out, work, args, fused=fused, entropy=entropy, rtol=2e-2, tau=tau)


def _finish(out, work, args, fused, entropy, rtol, tau):
    """The CPU baseline and, from its first round, the parity check of round 0; then the line.
    A parity failure prints the line with the failure and exits with status 1."""
    if args.no_cpu_baseline:
        out["parity"] = "not checked (--no-cpu-baseline: the oracle runs in the CPU baseline)"
        print(json.dumps(out), flush=True)
        return
    gpu0 = work.gpu_round0(fused, entropy)
    out["cpu_baseline"], ref0 = work.cpu_baseline(args.cpu_seconds)
    detail = _parity(gpu0, ref0, tau, rtol)
    out["parity"] = "ok" if detail["status"] == "ok" else detail["status"]
    out["parity_detail"] = detail
    print(json.dumps(out), flush=True)
    if detail["status"] != "ok":
        sys.exit(1)


if __name__ == "__main__":
    main()
