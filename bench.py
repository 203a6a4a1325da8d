"""Benchmark of the trie-constrained sparse decode on one MI355X.

One bench step = one whole answer for one batch of the product-scale workload
(V=151936, H=2048 bf16 tied embedding, 42-tool catalog, k=3, B=1): the decode
state is reset and the device-resident loop (one kernel, one workgroup per
sequence, the reset applied inside it) runs until every sequence has emitted
exactly k pointers.  The K timed answers are captured once into a HIP graph
(as a serving loop would) and replayed; each replay is bracketed by HIP events
on the stream the kernels run on, and by device synchronisations.  value =
decode steps per second = steps per answer / median time per answer; the
eager per-call figures (Python launches, host in the loop) are reported beside
it.  The graph's outputs are checked against an eager answer before any number
is reported.

Also on the same line: the loop kernel's roofline (the unique rows and hidden
vectors the head steps must read, over the kernel's duration), the batch-64
and batch-256 workloads (unique-row rates: rows shared by sequences are read
once), the character-level catalogs (host compile time, valid tokens per node
by depth, decode rates), the per-step kernel graph (the form a caller with its own forward pass
uses), the gather-GEMV bandwidth stress shapes next to a hand-written
streaming-read kernel timed on the same byte counts, the dense+mask step, and
the CPU oracle on every host thread (cpu_baseline, the only place the oracle
is used here).  --only copyref runs a 256 MiB device copy that calibrates the
HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "constrained decode steps/sec (sparse head) at B=1/64; achieved HBM GB/s"


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _kernel_hash():
    """Kernel sources and the build script (compile flags): counters taken with
    another build are not reported."""
    h = hashlib.sha256()
    for f in ("csrc/kernels.hip", "csrc/kernels.h", "build.py"):
        with open(os.path.join(ROOT, "trie_masked_sparse_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _to_dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _graph_time(fn, n_inner: int, reps: int):
    """Capture n_inner calls of fn into one HIP graph and replay it reps times,
    each replay between two events on the replay stream; returns (median
    microseconds per inner call, every replay's per-call microseconds)."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for _ in range(n_inner):
            fn()
    torch.cuda.synchronize()
    g.replay()  # first replay: uploads the graph
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / n_inner)
    return statistics.median(per), per, g


class Workload:
    """Device copies of one seeded workload plus a state for it."""

    def __init__(self, cid, B=None):
        import torch

        import trie_masked_sparse_amd as tms
        from synth import CONFIGS, catalog, embedding, hidden_states
        self.c = c = CONFIGS[cid]
        self.cid = cid
        self.B = c.batch if B is None else B
        cat = catalog(cid)
        self.trie = tms.Trie(cat, c.vocab, c.sep, c.stop)
        self.info = self.trie.info
        self.T = c.k * (self.info["max_depth"] + 1)
        self.emb_np = embedding(cid)
        self.emb = _to_dev(self.emb_np)
        self.hid_np = hidden_states(cid, self.T, self.B)
        self.hid = _to_dev(self.hid_np)
        self.state = tms.State(self.trie, self.B, c.k, self.emb)
        begin = self.trie.csr()["begin"]
        # the library groups root steps across sequences for B >= 8 and a root of >= 64 edges
        self.grouped = self.B >= 8 and int(begin[1] - begin[0]) >= 64
        self.tokens = torch.empty((self.B, self.T), dtype=torch.int32, device="cuda")
        self.len = torch.empty(self.B, dtype=torch.int32, device="cuda")
        self.entries = torch.empty((self.B, c.k), dtype=torch.int32, device="cuda")
        self.esz = 2 if c.dtype == "bf16" else 4

    def decode(self):
        """One bench step: reset (applied inside the loop kernel), then the
        whole answer; asynchronous."""
        import trie_masked_sparse_amd as tms
        self.state.reset()
        tms.decode_k_pointers(self.state, self.hid, self.tokens, self.len, self.entries, check=False)

    def outputs(self):
        return self.tokens.cpu().numpy().copy(), self.len.cpu().numpy().copy(), self.entries.cpu().numpy().copy()

    def byte_profile(self):
        """Bytes per answer along the decode's own path, from the library's
        materialiser over host-driven steps.  Per step and sequence with legal
        set L: a head step (|L| >= 2) reads |L| rows and one hidden vector; a
        forced step (|L| = 1) reads nothing (its token is determined).
        head_gathered: every sequence reads its own rows; head_node_grouped: the
        sequences standing at the same node share its rows (what the node-grouped
        step requests: the union of their legal sets, per node); head_unique: a
        row needed by several sequences in the same step counted once (the union
        of the legal sets, the least that must come from memory);
        sec8d_gathered: every step counted, forced ones included."""
        import numpy as np
        import torch

        import trie_masked_sparse_amd as tms
        cap = self.info["cap"]
        legal = torch.empty((self.B, cap), dtype=torch.int32, device="cuda")
        nleg = torch.empty(self.B, dtype=torch.int32, device="cuda")
        tok = torch.empty(self.B, dtype=torch.int32, device="cuda")
        loop_tokens = self.tokens.cpu().numpy().copy()  # the resident loop's last answer
        self.state.reset()
        row = self.c.hidden * self.esz
        g_head = u_head = g_all = n_head = 0
        head_steps = rows_head = 0
        walk = np.full((self.B, self.T), -1, np.int32)
        for t in range(self.T):
            tms.legal_set(self.state, legal, nleg)
            lg, nl = legal.cpu().numpy(), nleg.cpu().numpy()
            act = nl >= 0
            g_all += int(nl[act].sum()) + int(act.sum())
            head = np.nonzero(nl >= 2)[0]
            node = self.state.export()["node"]
            u, by_node = set(), {}
            for b in head:
                u.update(lg[b, :nl[b]].tolist())
                by_node.setdefault(int(node[b]), set()).update(lg[b, :nl[b]].tolist())
            n_head += sum(len(x) for x in by_node.values()) + len(head)
            g_head += int(nl[head].sum()) + len(head)
            rows_head += int(nl[head].sum())
            u_head += len(u) + len(head)
            head_steps += len(head)
            tms.decode_step_sparse(self.state, self.hid[t], tok, check=False)
            walk[:, t] = tok.cpu().numpy()
        torch.cuda.synchronize()
        # the per-step walk and the resident loop decode the same answers (a
        # cheap consistency check outside the timed region, reported, not
        # asserted: a root step on the matrix cores may resolve a numerical
        # tie differently)
        same = bool(np.array_equal(walk, loop_tokens[:, :self.T]))
        return {"head_gathered": g_head * row, "head_node_grouped": n_head * row, "head_unique": u_head * row,
                "sec8d_gathered": g_all * row,
                "head_steps": head_steps, "head_rows": rows_head, "flops": 2 * self.c.hidden * rows_head,
                "step_walk_matches_loop": same}

    def close(self):
        self.state.close()
        self.trie.close()


def time_answers(w: Workload, steps: int, warmup: int, reps: int = 5):
    """Eager answers (host launch per call) and graph-replayed answers."""
    import numpy as np
    import torch
    for _ in range(warmup):
        w.decode()
    torch.cuda.synchronize()
    ref = w.outputs()
    assert (w.state.status() == 0).all(), "decode reported a device error"
    # eager: one event pair per call, and the wall clock over all of them
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        w.decode()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)
    # graph: the same K answers captured once, replayed
    per_answer_us, per_rep, g = _graph_time(w.decode, steps, reps)
    torch.cuda.synchronize()
    got = w.outputs()
    for x, y in zip(ref, got):
        assert np.array_equal(x, y), "graph-replayed answers differ from the eager answer"
    assert (w.state.status() == 0).all(), "decode reported a device error"
    del g
    steps_per_call = int(ref[1].max())  # lockstep steps that emitted a token
    tokens_per_call = int(ref[1].sum())
    return {
        "us_per_answer": per_answer_us, "us_per_answer_each_replay": per_rep,
        "steps_per_s": steps_per_call / (per_answer_us * 1e-6), "tokens_per_s": tokens_per_call / (per_answer_us * 1e-6),
        "eager_event_median_us": eager_us, "eager_wall_us_per_call": wall * 1e6 / steps,
        "eager_steps_per_s": steps_per_call * steps / wall,
        "steps_per_call": steps_per_call, "tokens_per_call": tokens_per_call,
        "launches_per_answer": 2 * w.c.k if w.grouped else 1,
    }


def loop_rates(w: Workload, r: dict, prof: dict):
    t = r["us_per_answer"] * 1e-6
    return {"unique_GBps": prof["head_unique"] / t / 1e9, "gathered_GBps": prof["head_gathered"] / t / 1e9,
            "unique_bytes_per_answer": prof["head_unique"], "gathered_bytes_per_answer": prof["head_gathered"],
            "node_grouped_bytes_per_answer": prof["head_node_grouped"],
            "sec8d_gathered_bytes_per_answer": prof["sec8d_gathered"], "head_steps_per_answer": prof["head_steps"],
            "flops_per_answer": prof["flops"], "step_walk_matches_loop": prof["step_walk_matches_loop"]}


def graph_mode(w: Workload, steps: int, warmup: int):
    """The same answers through the hipGraph of per-step kernels (one launch
    per step, the form a caller whose forward pass sits between steps uses)."""
    import torch

    import trie_masked_sparse_amd as tms
    tms.state_set_loop(w.state, tms.LOOP_GRAPH)
    for _ in range(warmup):
        w.decode()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        w.decode()
    e1.record()
    torch.cuda.synchronize()
    tms.state_set_loop(w.state, tms.LOOP_RESIDENT)
    per = e0.elapsed_time(e1) * 1e3 / steps
    spc = int(w.len.max().item())
    return {"us_per_answer": per, "steps_per_s": spc / (per * 1e-6), "us_per_step_kernel": per / w.T,
            "step_kernel_launches_per_answer": w.T}


def launch_floor(w: Workload, reps: int = 20):
    """Per-launch cost of the step kernel when it has nothing to do: the
    hipGraph of T step kernels replayed on a finished state."""
    import torch

    import trie_masked_sparse_amd as tms
    tms.state_set_loop(w.state, tms.LOOP_GRAPH)
    w.decode()  # build the graph; every sequence finishes
    tms.decode_k_pointers(w.state, w.hid, w.tokens, w.len, w.entries, check=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tms.decode_k_pointers(w.state, w.hid, w.tokens, w.len, w.entries, check=False)
    e1.record()
    torch.cuda.synchronize()
    tms.state_set_loop(w.state, tms.LOOP_RESIDENT)
    per_call = e0.elapsed_time(e1) * 1e3 / reps
    return {"us_per_step_kernel": per_call / (w.T + 1), "launches_per_call": w.T + 1, "us_per_call": per_call}


READ_REF = {"grid": 0, "unroll": 4}  # set by streaming_read_reference's sweep


def stress_sizes(V: int, H: int, esz: int = 2):
    """Row bytes per launch of the two stress shapes (64 sequences x 256 or
    x 887 distinct rows), and the byte counts the streaming reference reads:
    the same two, plus the 64 x 256 shape's whole working set (its disjoint
    row sets together), every one within the V x H table."""
    sizes = {R: 64 * R * H * esz for R in (256, 887)}
    working_set = (V // (64 * 256)) * sizes[256]
    ref = sorted(set(sizes.values())) + [working_set]
    assert max(ref) <= V * H * esz
    return sizes, ref


def streaming_read_reference(table, sizes, reps: int = 5):
    """The in-tree streaming-read kernel (tms_read_reference) on contiguous
    slices of the table, cycling through disjoint slices as the stress gathers
    cycle through disjoint row sets.  The launch shape (workgroups, loads in
    flight) is the best of a small sweep at the largest size."""
    import torch

    import trie_masked_sparse_amd as tms
    flat = table.view(-1)
    total = flat.numel() * flat.element_size()
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")

    def run(nbytes, grid, unroll):
        n_sl = max(1, total // nbytes)
        el = nbytes // flat.element_size()
        slices = [flat[i * el:(i + 1) * el] for i in range(n_sl)]
        assert all(x.numel() == el for x in slices), "a slice runs past the table"
        it = iter(range(1 << 30))

        def one():
            tms.read_reference(slices[next(it) % n_sl], out, grid, unroll, nbytes)
        us, _, g = _graph_time(one, n_sl * 2, reps)
        del g
        return us, nbytes / (us * 1e-6) / 1e9, n_sl

    for n in sizes:
        if n > total:
            raise ValueError(f"reference size {n} exceeds the {total}-byte table")
    big = max(sizes)
    sweep = {}
    for grid in (0, 1024, 2048, 4096, 8192):
        for unroll in (2, 4, 8):
            sweep[f"grid={grid},unroll={unroll}"] = run(big, grid, unroll)[1]
    best = max(sweep, key=sweep.get)
    READ_REF["grid"], READ_REF["unroll"] = (int(x.split("=")[1]) for x in best.split(","))
    res = {"kernel": "read_ref_kernel (tms_read_reference)", "launch": dict(READ_REF), "sweep_GBps": sweep}
    for n in sizes:
        us, gbps, n_sl = run(n, READ_REF["grid"], READ_REF["unroll"])
        res[f"{n}"] = {"bytes": n, "us": us, "GBps": gbps, "disjoint_slices": n_sl}
    return res


def stress_gemv(steps: int, emb, emb_np, rows_per_seq: int, reps: int = 5):
    """64 sequences x rows_per_seq distinct rows per launch, cycling through
    disjoint row sets so that no launch re-reads a row of the previous one;
    the launches are graph-replayed (no host gap between them)."""
    import numpy as np
    import torch

    import trie_masked_sparse_amd as tms
    from synth import bf16_bits_from_f32, stress_rows
    V, H = emb_np.shape
    B, R = 64, rows_per_seq
    S = V // (B * R)
    sets = [_to_dev(np.ascontiguousarray(s)) for s in stress_rows(V, B, R, S)]
    rng = np.random.Generator(np.random.PCG64(5))
    hid = _to_dev(bf16_bits_from_f32(rng.standard_normal((B, H), dtype=np.float32)))
    n = torch.full((B,), R, dtype=torch.int32, device="cuda")
    out = torch.empty((B, R), dtype=torch.float32, device="cuda")
    it = iter(range(1 << 30))

    def one():
        tms.gather_gemv(emb, hid, sets[next(it) % S], n, out)
    us, per, g = _graph_time(one, S * max(2, steps // 10), reps)
    del g
    nbytes = B * R * H * 2 + B * H * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"shape": f"64 seq x {R} distinct rows, H={H} bf16, {S} disjoint sets ({S * B * R * H * 2 >> 20} MiB)",
            "kernel": "gather_gemv_kernel", "avg_launch_us": us, "alg_bytes_per_launch": nbytes,
            "achieved_GBps": gbps, "frac_of_8TBps": gbps / HBM_PEAK_GBPS,
            "traffic": _pmc_traffic("gather_gemv", f"stress64x{R}"),
            "seeds": {"rows": 4242, "hidden": 5, "table": "the product-scale embedding's"}}


def copy_reference(reps: int = 5):
    """A plain device-to-device copy of 256 MiB (torch's copy kernel): the known
    byte count that calibrates the HBM counters FETCH_SIZE and WRITE_SIZE."""
    import torch
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": src.numel(), "bytes_written": dst.numel(), "reps": reps}


def environment():
    import platform

    import torch
    p = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "gpu": p.name,
            "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "host_cpu": cpu, "host_threads": os.cpu_count(), "python": platform.python_version()}


def mask_fed_head_us(w: Workload, reps=20):
    """The bitmask-fed head at the reset state (every sequence at the root):
    vocabulary mask of the legal sets, popcount-scan materialiser, gather-GEMV
    over the materialised rows; each timed on its own over reps launches."""
    import torch

    import trie_masked_sparse_amd as tms
    B, V, cap = w.B, w.c.vocab, w.info["cap"]
    W = (V + 31) // 32
    mask = torch.empty((B, W), dtype=torch.int32, device="cuda")
    rows = torch.empty((B, cap), dtype=torch.int32, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, cap), dtype=torch.float32, device="cuda")
    w.state.reset()
    calls = {
        "legal_mask": lambda: tms.legal_mask(w.state, mask),
        "mask_to_rows": lambda: tms.mask_to_rows(mask, V, rows, n),
        "gather_gemv": lambda: tms.gather_gemv(w.emb, w.hid[0], rows, n, out),
    }
    res = {"B": B, "V": V, "mask_bytes": B * W * 4}
    for name, f in calls.items():
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_us"] = e0.elapsed_time(e1) * 1e3 / reps
    res["rows_per_seq"] = float(n.float().mean().item())
    res["mask_to_rows_GBps"] = res["mask_bytes"] / (res["mask_to_rows_us"] * 1e-6) / 1e9
    return res


def dense_step_us(w: Workload, reps=5):
    import torch

    import trie_masked_sparse_amd as tms
    tok = torch.empty(w.B, dtype=torch.int32, device="cuda")
    w.state.reset()
    tms.decode_step_dense_masked(w.state, w.hid[0], tok, check=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w.state.reset()
    e0.record()
    n = min(reps, w.T)
    for t in range(n):
        tms.decode_step_dense_masked(w.state, w.hid[t], tok, check=False)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    table = w.c.vocab * w.c.hidden * w.esz
    flops = 2.0 * w.B * w.c.vocab * w.c.hidden
    mfma = w.B > 1 and w.c.dtype == "bf16"
    gbps, tflops = table / (us * 1e-6) / 1e9, flops / (us * 1e-6) / 1e12
    # a whole dense step (mask, head, advance) against the table read once and
    # the matrix cores' dense bf16 peak (the vector head's fp32 peak otherwise)
    return {"B": w.B, "us_per_step": us, "table_GBps": gbps, "frac_of_8TBps": gbps / HBM_PEAK_GBPS,
            "head": "matrix cores (v_mfma_f32_16x16x32_bf16)" if mfma else "vector units",
            "TFLOPs": tflops, "frac_of_compute_peak": tflops / (2500.0 if mfma else 157.3)}


def cpu_baseline(w: Workload, seconds: float, copies: int = 64):
    """The oracle (plain C, fp64) decoding the bench's answer on every host
    thread: each thread decodes batches of `copies` copies of the same
    sequence (one C call per batch, so the interpreter lock is not the
    limit) until `seconds` of wall time have passed; value = steps over all
    threads / wall time.  The single-thread rate is measured the same way."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    from synth import catalog
    otr = oracle.Trie(catalog(w.cid), w.c.vocab, w.c.sep, w.c.stop)
    hid = np.ascontiguousarray(np.repeat(w.hid_np, copies, axis=1))
    one = oracle.decode(otr, w.c.k, w.emb_np, w.hid_np[:, :1])
    steps_per_answer = int(one["len"][0])

    def worker(deadline):
        n = 0
        while time.perf_counter() < deadline:
            out = oracle.decode(otr, w.c.k, w.emb_np, hid)
            n += int(out["len"].sum())
        return n

    def run(threads, secs):
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            total = sum(ex.map(worker, [t0 + secs] * threads))
        return total / (time.perf_counter() - t0)

    single = run(1, max(1.0, seconds / 4))
    # the threads this process may run on (the box's share of the host)
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    many = run(n, seconds)
    return {"value": many, "unit": "steps/s", "cores": n, "kind": "oracle",
            "sample": f"the product decode ({steps_per_answer} steps per answer, B=1) repeated on {n} host threads, "
                      f"{copies} copies of the sequence per oracle call, for {seconds:.1f} s of wall time "
                      f"({seconds * n:.0f} thread-seconds); gcc -O2 scalar fp64; single thread: {single:,.0f} steps/s"}


def _pmc_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken with the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("kernel_sources_sha256_16") != _kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _rocprof_rows(folder: str, kind: str):
    """Rows of the rocprofv3 CSV output (kernel_trace or counter_collection)
    under folder."""
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(folder, "**", f"*{kind}.csv"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{kind}.csv under {folder}")
    rows = []
    for p in paths:
        with open(p, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _dim(row, key):
    if row.get(key) not in (None, ""):
        return int(row[key])
    return int(row[key + "_X"]) * int(row.get(key + "_Y") or 1) * int(row.get(key + "_Z") or 1)


def _kernel_key(row):
    """(short kernel name, workgroups) of a rocprofv3 dispatch row."""
    name = row["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "").replace("tms::", "")
    name = name.split("(")[0].strip()
    return name, _dim(row, "Grid_Size") // max(1, _dim(row, "Workgroup_Size"))


def summarize_trace(folder: str):
    """Per (kernel, workgroups): dispatches, mean and median duration in
    microseconds (End - Start of each dispatch)."""
    groups = {}
    for r in _rocprof_rows(folder, "kernel_trace"):
        groups.setdefault(_kernel_key(r), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    print(f"{'kernel':<48}{'WGs':>6}{'calls':>8}{'mean us':>10}{'median us':>11}")
    for (k, wg), d in sorted(groups.items()):
        print(f"{k:<48}{wg:>6}{len(d):>8}{statistics.mean(d):>10.2f}{statistics.median(d):>11.2f}")


DECODE_KERNELS = ("loop_kernel", "root_mfma_kernel", "root_head_kernel")


def summarize_counters(folder: str, bench_json=None):
    """HBM bytes per launch from rocprofv3 counter runs, one run per workload
    and counter in folder/<workload>_<FETCH_SIZE|WRITE_SIZE>/.  Both counters
    are in KiB per dispatch; each is scaled by what it reads for the 256 MiB
    device copy of the copyref run (bytes known).  Writes the per-launch
    traffic of the product loop and of the two stress gathers to profiles/
    (with the kernel-source hash recorded by the GPU run, which must be the
    current one) and prints the per-kernel table and the decode kernels'
    memory fills per answer of every workload."""
    import glob

    from synth import CHAR_CONFIGS, CONFIGS
    hash_file = os.path.join(folder, "kernel_hash.txt")
    run_hash = open(hash_file).read().strip() if os.path.exists(hash_file) else None
    if run_hash != _kernel_hash():
        raise SystemExit(f"counters were taken with kernel sources {run_hash}, the tree has {_kernel_hash()}")
    data = {}  # (workload, counter) -> {(kernel, WGs): [KiB per dispatch]}
    for d in sorted(glob.glob(os.path.join(folder, "*_*_SIZE"))):
        wl, ctr = os.path.basename(d).rsplit("_", 2)[0], "_".join(os.path.basename(d).rsplit("_", 2)[1:])
        g = data.setdefault((wl, ctr), {})
        for r in _rocprof_rows(d, "counter_collection"):
            if r["Counter_Name"] == ctr:
                g.setdefault(_kernel_key(r), []).append(float(r["Counter_Value"]))
    copy_kib = 256 * 1024.0
    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        g = data[("copyref", ctr)]
        big = max((k for k in g if k[0].startswith("__amd_rocclr_copyBuffer")), key=lambda k: k[1])
        scale[ctr] = copy_kib / statistics.median(g[big])
    print(f"calibration (256 MiB device copy): FETCH_SIZE x{scale['FETCH_SIZE']:.3f}, "
          f"WRITE_SIZE x{scale['WRITE_SIZE']:.3f}")
    print(f"{'workload':<16}{'kernel':<44}{'WGs':>6}{'calls':>7}{'FETCH KiB':>12}{'WRITE KiB':>11}{'MB/launch':>11}")
    per_launch = {}
    for wl in sorted({w for w, _ in data}):
        f, wr = data.get((wl, "FETCH_SIZE"), {}), data.get((wl, "WRITE_SIZE"), {})
        for key in sorted(set(f) | set(wr)):
            fk = statistics.mean(f[key]) if key in f else float("nan")
            wk = statistics.mean(wr[key]) if key in wr else float("nan")
            mb = (fk * scale["FETCH_SIZE"] + wk * scale["WRITE_SIZE"]) * 1024 / 1e6
            per_launch[(wl, key)] = (fk, wk, len(f.get(key, [])))
            print(f"{wl:<16}{key[0]:<44}{key[1]:>6}{len(f.get(key, [])):>7}{fk:>12.1f}{wk:>11.1f}{mb:>11.3f}")

    def hbm_bytes(wl, key):
        fk, wk, _ = per_launch[(wl, key)]
        return (fk * scale["FETCH_SIZE"] + wk * scale["WRITE_SIZE"]) * 1024

    def write(kernel, workload, wl, key):
        out = {"kernel_sources_sha256_16": run_hash, "hbm_bytes_per_launch": hbm_bytes(wl, key),
               "fetch_bytes_per_launch": per_launch[(wl, key)][0] * scale["FETCH_SIZE"] * 1024,
               "write_bytes_per_launch": per_launch[(wl, key)][1] * scale["WRITE_SIZE"] * 1024,
               "dispatches": per_launch[(wl, key)][2], "kernel": key[0], "workgroups": key[1],
               "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"]}
        with open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json"), "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")

    loops = [k for (wl, k) in per_launch if wl == "headline" and k[0].startswith("loop_kernel") and k[1] == 1]
    if loops:
        write("loop", "product", "headline", loops[0])
    gathers = sorted((k for (wl, k) in per_launch if wl == "stress" and k[0].startswith("gather_gemv_kernel")),
                     key=lambda k: per_launch[("stress", k)][0])
    if len(gathers) == 2:  # the 64 x 256 shape reads fewer bytes per launch than 64 x 887
        write("gather_gemv", "stress64x256", "stress", gathers[0])
        write("gather_gemv", "stress64x887", "stress", gathers[1])
    line = json.load(open(bench_json)) if bench_json else None
    keys = {"headline": ("product_answer", "product"), "structured": ("structured_B64", "structured"),
            "unstructured": ("unstructured_B64", "unstructured"), "large": ("large_B256", "large"),
            "charset_tools": ("charset_tools_B64", "charset_tools"), "charset_hex": ("charset_hex_B64", "charset_hex")}
    print()
    print("decode kernels (loop_kernel, root heads) per answer:")
    print(f"{'workload':<16}{'launches':>9}{'us/answer':>11}{'unique MB':>11}{'fills MB':>10}{'writes MB':>11}"
          f"{'fills/unique':>14}{'U/t TB/s':>10}{'fills/t TB/s':>14}")
    for wl, (jk, cid) in keys.items():
        ks = [k for (w, k) in per_launch if w == wl and k[0].split("<")[0] in DECODE_KERNELS]
        if not ks:
            continue
        loop_calls = sum(per_launch[(wl, k)][2] for k in ks if k[0].startswith("loop_kernel"))
        heads = sum(per_launch[(wl, k)][2] for k in ks if not k[0].startswith("loop_kernel"))
        c = CONFIGS.get(cid) or CHAR_CONFIGS[cid]
        answers = loop_calls / c.k if heads else loop_calls
        fill = sum(per_launch[(wl, k)][0] * per_launch[(wl, k)][2] for k in ks) * scale["FETCH_SIZE"] * 1024 / answers
        wr = sum(per_launch[(wl, k)][1] * per_launch[(wl, k)][2] for k in ks) * scale["WRITE_SIZE"] * 1024 / answers
        us = ub = None
        if line and jk in line.get("also", {}):
            a = line["also"][jk]
            us, ub = a["us_per_answer"], a.get("unique_bytes_per_answer")
        lp = c.k * 2 if heads else 1
        row = f"{wl:<16}{lp:>9}"
        row += f"{us:>11.1f}" if us else f"{'':>11}"
        row += f"{ub / 1e6:>11.2f}" if ub else f"{'':>11}"
        row += f"{fill / 1e6:>10.2f}{wr / 1e6:>11.2f}"
        row += f"{fill / ub:>14.2f}" if ub else f"{'':>14}"
        row += f"{ub / (us * 1e-6) / 1e12:>10.3f}{fill / (us * 1e-6) / 1e12:>14.3f}" if (us and ub) else ""
        print(row)


class CharWorkload(Workload):
    """A character-level catalog (byte strings, byte-string vocabulary), one
    string per answer, rows from the product-scale embedding."""

    def __init__(self, cid):
        import torch

        import trie_masked_sparse_amd as tms
        from synth import CHAR_CONFIGS, char_catalog, char_hidden, char_vocab, embedding
        self.c = c = CHAR_CONFIGS[cid]
        self.cid = cid
        self.B = c.batch
        strings, vocab = char_catalog(cid), char_vocab(cid)
        t0 = time.perf_counter()
        h = tms.charset_build(strings, vocab, c.sep, c.stop)  # host compile only, timed
        self.compile_ms = (time.perf_counter() - t0) * 1e3
        csr = tms.trie_export_csr(h)
        tms.trie_free(h)
        self.valid_by_depth = _valid_by_depth(csr, vocab)
        self.trie = tms.Trie.from_charset(strings, vocab, c.sep, c.stop)
        self.info = self.trie.info
        self.T = self.info["max_depth"] + 1
        self.emb_np = embedding(c.emb_cid)
        self.emb = _to_dev(self.emb_np)
        self.hid_np = char_hidden(cid, self.T)
        self.hid = _to_dev(self.hid_np)
        self.state = tms.State(self.trie, self.B, 1, self.emb)
        self.grouped = self.B >= 8 and int(csr["begin"][1] - csr["begin"][0]) >= 64
        self.tokens = torch.empty((self.B, self.T), dtype=torch.int32, device="cuda")
        self.len = torch.empty(self.B, dtype=torch.int32, device="cuda")
        self.entries = torch.empty((self.B, 1), dtype=torch.int32, device="cuda")
        self.esz = 2


def _valid_by_depth(csr, vocab):
    """Mean and largest number of valid tokens per trie node, by the node's
    depth in bytes (the page's measure of how fast the valid sets shrink)."""
    import numpy as np
    b = csr["begin"]
    depth = {0: 0}
    order = [0]
    for n in order:
        for e in range(b[n], b[n + 1]):
            ch = int(csr["child"][e])
            if ch >= 0 and ch not in depth:
                depth[ch] = depth[n] + len(vocab[int(csr["tok"][e])])
                order.append(ch)
    sizes = {}
    for n, d in depth.items():
        k = int(np.sum(csr["child"][b[n]:b[n + 1]] >= 0))
        sizes.setdefault(d, []).append(k)
    return {str(d): {"nodes": len(v), "mean": float(np.mean(v)), "max": int(max(v))}
            for d, v in sorted(sizes.items()) if d <= 6}


def workload_line(cid: str, steps: int, warmup: int, per_step_graph: bool = True):
    """Resident-loop rates of one batched workload."""
    import trie_masked_sparse_amd as tms
    _log(f"{cid} workload")
    w = CharWorkload(cid) if cid.startswith("charset") else Workload(cid)
    r = time_answers(w, steps, warmup)
    prof = w.byte_profile()
    rates = loop_rates(w, r, prof)
    d = {"B": w.B, "steps_per_s": r["steps_per_s"], "tokens_per_s": r["tokens_per_s"],
         "us_per_answer": r["us_per_answer"], "steps_per_call": r["steps_per_call"],
         "launches_per_answer": r["launches_per_answer"],
         "path": "fast" if w.info["path"] == tms.PATH_FAST else "global",
         "root_steps": "grouped" if w.grouped else "per sequence",
         "unique_frac_of_8TBps": rates["unique_GBps"] / HBM_PEAK_GBPS, **rates,
         "eager_event_median_us": r["eager_event_median_us"],
         "seeds": {"catalog": w.c.cat_seed, "hidden": w.c.hid_seed,
                   "embedding": getattr(w.c, "emb_seed", None), "vocabulary": getattr(w.c, "voc_seed", None)}}
    if isinstance(w, CharWorkload):
        d.update({"host_compile_ms": w.compile_ms, "valid_tokens_by_depth": w.valid_by_depth,
                  "trie": {k: w.info[k] for k in ("n_nodes", "n_edges", "cap", "max_depth")}})
    if per_step_graph:
        d["per_step_kernel_graph"] = graph_mode(w, max(5, steps // 5), 2)
        if w.B > 1:
            # the same graph with every shared node grouped (requests
            # node_grouped_bytes_per_answer of rows instead of gathered)
            tms.state_set_step_grouping(w.state, tms.STEP_GROUP_NODES)
            d["per_step_kernel_graph_node_grouped"] = graph_mode(w, max(5, steps // 5), 2)
            tms.state_set_step_grouping(w.state, tms.STEP_GROUP_AUTO)
    w.close()
    _log(f"{cid}: {d['steps_per_s']:.0f} steps/s, {d['us_per_answer']:.1f} us per answer, "
         f"unique {d['unique_GBps']:.0f} GB/s")
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=2.0)
    ap.add_argument("--only", default="",
                    help="comma list of headline,b64,large,charset,stress,dense,cpu, or single workloads "
                         "structured,unstructured,charset_tools,charset_hex; copyref (the counter calibration) and "
                         "dense_large (the dense step at B=256, H=4096) run only when named (default: all others)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel durations from a rocprofv3 --kernel-trace run's CSV in DIR; no GPU")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="summarize rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR (one subfolder "
                         "<workload>_<counter> per run) and write profiles/*_pmc.json; no GPU")
    ap.add_argument("--bench-json", metavar="FILE", help="with --summarize-counters: a bench line of the "
                    "same kernels, for times and unique bytes per answer")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.bench_json)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs on one GPU. "
              "Sequences shard across GPUs with no per-step exchange; run one process per GPU.", file=sys.stderr)
        sys.exit(2)
    only = set(filter(None, args.only.split(",")))

    def want(x):  # copyref and dense_large (profiling aids) only when asked for
        return (not only and x not in ("copyref", "dense_large")) or x in only

    import torch

    import trie_masked_sparse_amd as tms
    tms.lib()
    torch.cuda.init()
    _log(f"device {torch.cuda.get_device_name(0)}")

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    also = {}
    _log("product-scale workload")
    w = Workload("product")
    if want("headline"):
        r = time_answers(w, args.steps, args.warmup)
        prof = w.byte_profile()
        rates = loop_rates(w, r, prof)
        line.update({"value": r["steps_per_s"], "unit": "steps/s",
                     "ms_per_step": r["us_per_answer"] / r["steps_per_call"] * 1e-3,
                     "tokens_per_s": r["tokens_per_s"]})
        line["config"] = {
            "workload": "product-scale: V=151936, H=2048 bf16 tied embedding (622 MB), 42-tool catalog "
                        f"({w.info['n_nodes']} trie nodes, cap {w.info['cap']}), k=3, B=1; one bench step = "
                        "state reset + one whole answer from the resident device loop (one kernel; "
                        f"{r['steps_per_call']} steps, {prof['head_steps']} of them head steps); the K answers are "
                        "captured in one HIP graph and replayed; bf16 inputs, fp32 accumulation",
            "path": "fast" if w.info["path"] == tms.PATH_FAST else "global",
            "steps_per_call": r["steps_per_call"], "tokens_per_call": r["tokens_per_call"],
            "seeds": {"catalog": w.c.cat_seed, "embedding": w.c.emb_seed, "hidden": w.c.hid_seed}}
        _log(f"headline {r}")
        line["roofline"] = {"bound": "hbm", "kernel": "loop_kernel", "achieved": rates["unique_GBps"],
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": rates["unique_GBps"] / HBM_PEAK_GBPS,
                            "traffic": _pmc_traffic("loop", "product"),
                            "alg_bytes_per_launch": prof["head_unique"],
                            "avg_launch_us": r["us_per_answer"]}
        also["product_answer"] = {**rates, "us_per_answer": r["us_per_answer"],
                                  "us_per_answer_each_replay": r["us_per_answer_each_replay"],
                                  "eager_event_median_us": r["eager_event_median_us"],
                                  "eager_wall_us_per_call": r["eager_wall_us_per_call"],
                                  "eager_steps_per_s": r["eager_steps_per_s"]}
        also["product_per_step_kernel_graph"] = graph_mode(w, args.steps, args.warmup)
        also["product_launch_floor"] = launch_floor(w)
        _log(f"roofline {line['roofline']}; per-step graph {also['product_per_step_kernel_graph']}")
    for cid in ("structured", "unstructured"):
        if want("b64") or want(cid):
            also[f"{cid}_B64"] = workload_line(cid, max(10, args.steps // 2), args.warmup)
    if want("large"):
        also["large_B256"] = workload_line("large", max(5, args.steps // 5), 2, per_step_graph=False)
    for cid in ("charset_tools", "charset_hex"):
        if want("charset") or want(cid):
            also[f"{cid}_B64"] = workload_line(cid, max(10, args.steps // 2), args.warmup)
    if want("dense"):
        also["dense_masked_product_B1"] = dense_step_us(w)
        wd = Workload("structured")
        also["dense_masked_structured_B64"] = dense_step_us(wd)
        also["mask_fed_head_structured_B64"] = mask_fed_head_us(wd)
        wd.close()
        _log(f"dense {also['dense_masked_product_B1']} / {also['dense_masked_structured_B64']}")
    if want("dense_large"):
        wl = Workload("large")
        also["dense_masked_large_B256"] = dense_step_us(wl)
        wl.close()
        _log(f"dense large {also['dense_masked_large_B256']}")
    if want("stress"):
        sizes, ref_sizes = stress_sizes(w.c.vocab, w.c.hidden)
        ref = streaming_read_reference(w.emb, ref_sizes)
        also["streaming_read_reference"] = ref
        for R, nb in sizes.items():
            d = stress_gemv(args.steps, w.emb, w.emb_np, R)
            d["streaming_read_same_bytes_GBps"] = ref[f"{nb}"]["GBps"]
            d["frac_of_streaming_read"] = d["achieved_GBps"] / ref[f"{nb}"]["GBps"]
            also[f"gather_gemv_stress_64x{R}"] = d
            _log(f"stress {d}")
        _log(f"streaming read {ref}")
    if want("copyref"):
        also["copy_reference"] = copy_reference()
    if want("cpu"):
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        _log(f"cpu {line['cpu_baseline']}")
    also["environment"] = environment()
    line["also"] = also
    w.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
