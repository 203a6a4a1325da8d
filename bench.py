"""Benchmark of the trie-constrained sparse decode on one MI355X.

One bench step = one whole answer for one batch of the product-scale workload
(V=151936, H=2048 bf16 tied embedding, 42-tool catalog, k=3, B=1): reset the
decode state, then the device-resident loop (one kernel, one workgroup per
sequence) until every sequence has emitted exactly k pointers.  value = decode
steps per second (lockstep steps that emitted a token), over K timed steps
after W warmup steps, bracketed by device synchronisations.

Also reported on the same line: the loop kernel's roofline (algorithmic bytes
of one answer / that launch's duration, timed with HIP events on the launch
stream), the same answers through the hipGraph of per-step kernels, the
batch-64 workloads, the gather-GEMV bandwidth stress shapes (64 sequences x
256 or x 887 distinct rows per launch, cycling through disjoint row sets of
the 622 MB table), the dense+mask step, and the CPU oracle timed on this host
(cpu_baseline leg, the only place the oracle is used here).  --only copyref
runs a 256 MiB device copy that calibrates the HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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


class Workload:
    """Device copies of one seeded workload plus a state for it."""

    def __init__(self, cid, B=None):
        import numpy as np
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
        self.np = np

    def decode(self, ev=None):
        """One bench step: reset, then the whole answer.  ev: optional pair of
        events recorded around the decode launch (after the reset)."""
        import trie_masked_sparse_amd as tms
        self.state.reset()
        if ev:
            ev[0].record()
        tms.decode_k_pointers(self.state.h, self.hid, self.tokens, self.len, self.entries, check=False)
        if ev:
            ev[1].record()

    def legal_profile(self):
        """Per step: legal-set sizes and unique rows, from the library's own
        materialiser, along the decode's own path (host-driven steps)."""
        import torch

        import trie_masked_sparse_amd as tms
        np = self.np
        cap = self.info["cap"]
        legal = torch.empty((self.B, cap), dtype=torch.int32, device="cuda")
        nleg = torch.empty(self.B, dtype=torch.int32, device="cuda")
        tok = torch.empty(self.B, dtype=torch.int32, device="cuda")
        self.state.reset()
        n_rows, n_active, n_unique = [], [], []
        for t in range(self.T):
            tms.legal_set(self.state.h, legal, nleg)
            lg, nl = legal.cpu().numpy(), nleg.cpu().numpy()
            act = nl >= 0
            n_active.append(int(act.sum()))
            n_rows.append(int(nl[act].sum()))
            u = set()
            for b in np.nonzero(act)[0]:
                u.update(lg[b, :nl[b]].tolist())
            n_unique.append(len(u))
            tms.decode_step_sparse(self.state.h, self.hid[t], tok)
        torch.cuda.synchronize()
        return np.array(n_rows), np.array(n_active), np.array(n_unique)

    def close(self):
        self.state.close()
        self.trie.close()


def _to_dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_decode(w: Workload, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        w.decode()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        w.decode()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    # a second pass of the same bench steps with an event pair around each
    # decode launch: the loop kernel's own duration, for the roofline (kept out
    # of the region above, where the extra markers would lengthen the timeline)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        w.decode(evs[i])
    torch.cuda.synchronize()
    decode_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / steps
    ln = w.len.cpu().numpy()
    assert (w.state.status() == 0).all(), "decode reported a device error"
    steps_per_call = int(ln.max())  # lockstep steps that emitted a token
    tokens_per_call = int(ln.sum())
    return {
        "wall_s": wall, "gpu_ms": gpu_ms, "ms_per_call": wall * 1e3 / steps, "decode_launch_us": decode_us,
        "steps_per_s": steps_per_call * steps / wall, "tokens_per_s": tokens_per_call * steps / wall,
        "steps_per_call": steps_per_call, "tokens_per_call": tokens_per_call, "launches_per_call": w.T,
    }


def loop_roofline(w: Workload, timed: dict, steps: int):
    """Algorithmic bytes of one whole answer (the resident loop kernel's launch)
    over that launch's average duration.  A bench step is exactly one launch of
    the loop kernel (the state reset is carried out inside it), so the duration
    is the timed region's GPU time (HIP events on the launch stream) over the
    number of steps; the event pairs recorded around single launches in a
    second pass are reported beside it (they also count the dispatch)."""
    n_rows, n_act, n_uni = w.legal_profile()
    H, esz = w.c.hidden, w.esz
    gathered = float(((n_rows + n_act) * H * esz).sum())   # legal rows + hidden vectors
    unique = float(((n_uni + n_act) * H * esz).sum())
    launch_us = timed["gpu_ms"] * 1e3 / steps
    return {
        "kernel": "loop_kernel", "avg_launch_us": launch_us, "event_pair_us": timed["decode_launch_us"],
        "alg_bytes_per_launch": gathered, "unique_bytes_per_launch": unique,
        "achieved_GBps": gathered / (launch_us * 1e-6) / 1e9, "unique_GBps": unique / (launch_us * 1e-6) / 1e9,
        "flops_per_launch": float(2 * H * n_rows.sum()),
        "rows_per_step": [int(x) for x in n_rows],
    }


def graph_mode(w: Workload, steps: int, warmup: int):
    """The same answers through the hipGraph of per-step kernels."""
    import trie_masked_sparse_amd as tms
    tms.state_set_loop(w.state.h, tms.LOOP_GRAPH)
    r = time_decode(w, steps, warmup)
    tms.state_set_loop(w.state.h, tms.LOOP_RESIDENT)
    return {"steps_per_s": r["steps_per_s"], "ms_per_call": r["ms_per_call"],
            "step_kernel_launches_per_call": w.T}


def stress_gemv(steps: int, warmup: int, emb, emb_np, rows_per_seq: int):
    """64 sequences x rows_per_seq distinct rows per launch, cycling through
    disjoint row sets so that no launch re-reads a row of the previous one."""
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
    for i in range(warmup * S):
        tms.gather_gemv(emb, hid, sets[i % S], n, out)
    torch.cuda.synchronize()
    iters = max(steps, 1) * S
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        tms.gather_gemv(emb, hid, sets[i % S], n, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters  # back-to-back launches on the launch stream
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


def streaming_read_reference(nbytes: int = 604 << 20, reps: int = 5):
    """A plain streaming read of a buffer the size of the stress working set,
    the reference the gathers are compared with: torch's row sums over a
    [n / 4096, 4096] fp32 view (the fastest of the library's plain reductions
    measured here: sum, amax and row sums in bf16/fp32; full sums reach only
    3.3-3.8 TB/s)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda").view(-1, 4096)
    x.sum(dim=1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        x.sum(dim=1)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"bytes": nbytes, "us": us, "GBps": nbytes / (us * 1e-6) / 1e9, "kernel": "torch row sums (fp32)"}


def launch_floor(w: Workload, reps: int = 20):
    """Per-launch cost of the step kernel when it has nothing to do: the
    hipGraph of T step kernels replayed on a finished state."""
    import torch

    import trie_masked_sparse_amd as tms
    tms.state_set_loop(w.state.h, tms.LOOP_GRAPH)
    w.decode()  # build the graph; every sequence finishes
    tms.decode_k_pointers(w.state.h, w.hid, w.tokens, w.len, w.entries, check=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tms.decode_k_pointers(w.state.h, w.hid, w.tokens, w.len, w.entries, check=False)
    e1.record()
    torch.cuda.synchronize()
    tms.state_set_loop(w.state.h, tms.LOOP_RESIDENT)
    per_call = e0.elapsed_time(e1) * 1e3 / reps
    return {"us_per_step_kernel": per_call / (w.T + 1), "launches_per_call": w.T + 1, "us_per_call": per_call}


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
        "legal_mask": lambda: tms.legal_mask(w.state.h, mask),
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
    tms.decode_step_dense_masked(w.state.h, w.hid[0], tok)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w.state.reset()
    e0.record()
    n = min(reps, w.T)
    for t in range(n):
        tms.decode_step_dense_masked(w.state.h, w.hid[t], tok, check=False)
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


def cpu_baseline(w: Workload, min_seconds: float):
    """The oracle (plain C, fp64, one thread) decoding the same batch, repeated."""
    import oracle
    otr = oracle.Trie(__import__("synth").catalog(w.cid), w.c.vocab, w.c.sep, w.c.stop)
    reps, t0 = 0, time.perf_counter()
    steps = 0
    while True:
        out = oracle.decode(otr, w.c.k, w.emb_np, w.hid_np)
        reps += 1
        steps += int(out["len"].max())
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": steps / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} repetitions of the full {w.cid} decode (B={w.B}, {int(out['len'].max())} steps, "
                      f"{int(out['len'].sum())} tokens each), {el:.1f} s, single thread, gcc -O2 fp64"}


def cpu_baseline_threads(w: Workload, seq_sample=None):
    """The oracle decoding the same batch once: on one thread, and with the
    sequences split over the host's threads (ctypes releases the GIL around
    each call).  seq_sample: decode only these sequences (large batches)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    otr = oracle.Trie(__import__("synth").catalog(w.cid), w.c.vocab, w.c.sep, w.c.stop)
    hid = w.hid_np if seq_sample is None else np.ascontiguousarray(w.hid_np[:, seq_sample, :])
    t0 = time.perf_counter()
    oracle.decode(otr, w.c.k, w.emb_np, hid)
    one = time.perf_counter() - t0
    n = min(os.cpu_count() or 1, hid.shape[1])
    parts = [np.ascontiguousarray(hid[:, i::n, :]) for i in range(n)]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(n) as ex:
        list(ex.map(lambda h: oracle.decode(otr, w.c.k, w.emb_np, h), parts))
    many = time.perf_counter() - t0
    return {"seconds_1_thread": one, "seconds_n_threads": many, "threads": n, "sequences": int(hid.shape[1])}


def config_table(steps: int, warmup: int, cids=("tiny", "product", "product_deep", "structured", "unstructured",
                                                 "large")):
    """Every workload: the resident decode's steps/s and tokens/s, gathered
    bytes per second, the dense+mask step, and the oracle's time for the
    same batch (the results table of the bench's plan)."""
    import numpy as np
    out = {}
    for cid in cids:
        _log(f"table: {cid}")
        w = Workload(cid)
        r = time_decode(w, steps, warmup)
        n_rows, n_act, n_uniq = w.legal_profile()
        gathered = float(((n_rows + n_act) * w.c.hidden * w.esz).sum())
        unique = float(((n_uniq + n_act) * w.c.hidden * w.esz).sum())
        sample = None if w.B <= 64 else list(range(0, w.B, w.B // 24))[:24]
        row = {"B": w.B, "seeds": {"catalog": w.c.cat_seed, "embedding": w.c.emb_seed, "hidden": w.c.hid_seed},
               "steps_per_s": r["steps_per_s"], "tokens_per_s": r["tokens_per_s"],
               "ms_per_call": r["ms_per_call"], "gathered_TBps": gathered / (r["gpu_ms"] * 1e-3 / steps) / 1e12,
               "unique_TBps": unique / (r["gpu_ms"] * 1e-3 / steps) / 1e12,
               "gathered_bytes_per_call": gathered, "unique_bytes_per_call": unique,
               "dense_mask_step_us": dense_step_us(w)["us_per_step"],
               "oracle": cpu_baseline_threads(w, sample)}
        out[cid] = row
        _log(f"table: {cid} {row}")
        w.close()
    return out


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--configs", default="tiny,product,product_deep,structured,unstructured,large",
                    help="workloads of the --only configs table")
    ap.add_argument("--only", default="",
                    help="comma list of headline,b64,stress,dense,cpu,copyref,configs (default: all but copyref, configs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Sequences shard across GPUs with no per-step exchange; run one process per GPU.", file=sys.stderr)
        sys.exit(2)
    only = set(filter(None, args.only.split(",")))

    def want(x):
        return (not only and x != "copyref") or x in only

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
        r = time_decode(w, args.steps, args.warmup)
        line.update({"value": r["steps_per_s"], "unit": "steps/s", "ms_per_step": r["ms_per_call"],
                     "tokens_per_s": r["tokens_per_s"]})
        line["config"] = {
            "workload": "product-scale: V=151936, H=2048 bf16 tied embedding (622 MB), 42-tool catalog "
                        f"({w.info['n_nodes']} trie nodes, cap {w.info['cap']}), k=3, B=1; one bench step = "
                        "state reset + one whole answer from the resident device loop "
                        f"(up to {w.T} steps); bf16 inputs, fp32 accumulation",
            "path": "fast" if w.info["path"] == tms.PATH_FAST else "global",
            "steps_per_call": r["steps_per_call"], "tokens_per_call": r["tokens_per_call"],
            "seeds": {"catalog": w.c.cat_seed, "embedding": w.c.emb_seed, "hidden": w.c.hid_seed}}
        _log(f"headline {r}")
        rf = loop_roofline(w, r, args.steps)
        line["roofline"] = {"bound": "hbm", "kernel": rf["kernel"], "achieved": rf["achieved_GBps"],
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": rf["achieved_GBps"] / HBM_PEAK_GBPS,
                            "traffic": _pmc_traffic("loop", "product"),
                            "alg_bytes_per_launch": rf["alg_bytes_per_launch"],
                            "avg_launch_us": rf["avg_launch_us"]}
        also["product_loop_detail"] = rf
        also["product_graph_mode"] = graph_mode(w, args.steps, args.warmup)
        also["product_launch_floor"] = launch_floor(w)
        _log(f"roofline {line['roofline']}; graph {also['product_graph_mode']}")
    if want("dense"):
        also["dense_masked_product_B1"] = dense_step_us(w)
        _log(f"dense {also['dense_masked_product_B1']}")
        wd = Workload("structured")
        also["dense_masked_structured_B64"] = dense_step_us(wd)
        _log(f"dense B=64 {also['dense_masked_structured_B64']}")
        also["mask_fed_head_structured_B64"] = mask_fed_head_us(wd)
        _log(f"mask-fed head B=64 {also['mask_fed_head_structured_B64']}")
        wd.close()
    if want("stress"):
        for rows in (256, 887):
            also[f"gather_gemv_stress_64x{rows}"] = stress_gemv(max(3, args.steps // 5), 2, w.emb, w.emb_np, rows)
            _log(f"stress {also[f'gather_gemv_stress_64x{rows}']}")
        ref = streaming_read_reference()
        also["streaming_read_reference"] = ref
        for rows in (256, 887):
            d = also[f"gather_gemv_stress_64x{rows}"]
            d["frac_of_streaming_read"] = d["achieved_GBps"] / ref["GBps"]
        _log(f"streaming read {ref}")
    if want("copyref"):
        also["copy_reference"] = copy_reference()
    if want("b64"):
        for cid in ("structured", "unstructured"):
            _log(f"{cid} workload")
            wb = Workload(cid)
            nb = max(5, args.steps // 2)
            rb = time_decode(wb, nb, args.warmup)
            rfb = loop_roofline(wb, rb, nb)
            also[f"{cid}_B64"] = {"steps_per_s": rb["steps_per_s"], "tokens_per_s": rb["tokens_per_s"],
                                  "ms_per_call": rb["ms_per_call"], "steps_per_call": rb["steps_per_call"],
                                  "path": "fast" if wb.info["path"] == tms.PATH_FAST else "global",
                                  "root_steps": "grouped" if wb.grouped else "per sequence",
                                  "loop_kernel": {k: v for k, v in rfb.items() if k != "rows_per_step"},
                                  "graph_mode": graph_mode(wb, nb, args.warmup)}
            _log(f"{cid} {also[f'{cid}_B64']['steps_per_s']:.0f} steps/s")
            wb.close()
    if args.only and "configs" in args.only.split(","):
        also["configs"] = config_table(args.steps, args.warmup, tuple(filter(None, args.configs.split(","))))
    if want("cpu"):
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        _log(f"cpu {line['cpu_baseline']}")
    also["environment"] = environment()
    line["also"] = also
    w.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
