"""CPU-only checks of the HIP library: it loads, exports every symbol its header
declares, and its host-side catalog compiler produces exactly the oracle's
canonical CSR (no GPU call is made here)."""
import os
import re

import numpy as np
import pytest

import oracle
import trie_masked_sparse_amd as tms
from synth import CONFIGS, catalog, random_catalog

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tms.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tms.LIB_PATH):
        pytest.fail("libtms.so is not built (python -m trie_masked_sparse_amd.build)")
    return tms.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(tms_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(L):
    decl = declared_symbols()
    assert decl == sorted(tms.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_binding_constants_match_header():
    """Every enumerator and the no-allocation limit that include/tms.h
    defines has the same value in the Python binding (TMS_X -> tms.X)."""
    hdr = open(os.path.join(os.path.dirname(tms.__file__), os.pardir, "include", "tms.h")).read()
    seen = 0
    for body in re.findall(r"typedef enum\s*\{(.*?)\}", hdr, re.S):
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        for name, value in re.findall(r"TMS_([A-Z0-9_]+)\s*=\s*(\d+)", body):
            assert getattr(tms, name) == int(value), name
            seen += 1
    assert seen == 27  # status 11, dtype 2, path 3, loop 5, no-repeat 2, step grouping 4
    m = re.search(r"#define TMS_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", hdr)
    assert tms.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_status_strings(L):
    for code in range(11):
        assert tms.status_str(code) not in ("", "unknown status")
    assert tms.status_str(99) == "unknown status"


def _csr_equal(entries, V, sep, stop):
    h = tms.trie_build(entries, V, sep, stop)
    try:
        got = tms.trie_export_csr(h)
        info = tms.trie_info_get(h)
    finally:
        tms.trie_free(h)
    ref = oracle.Trie(entries, V, sep, stop)
    want = ref.csr()
    for key in ("begin", "entry", "tok", "child", "live0"):
        assert np.array_equal(got[key], want[key]), key
    assert (info["n_nodes"], info["n_edges"], info["n_entries"], info["cap"], info["max_depth"]) == \
        (ref.n_nodes, ref.n_edges, ref.n_entries, ref.cap, ref.max_depth)
    assert info["path"] == tms.PATH_AUTO and info["device_bytes"] == 0
    return info


def test_builder_matches_oracle_small(L, oracle_lib):
    cases = [([[1], [1, 2], [1, 2, 3], [4]], 16, 14, 15), ([[3, 3], [3], [3, 3, 3]], 16, 0, 15),
             ([[5, 6], [5], [7], [5, 6, 7]], 16, 15, 1), ([[0]], 4, 2, 3)]
    for seed in range(60):
        rng = np.random.Generator(np.random.PCG64(seed))
        K = int(rng.integers(1, 40))
        V = int(rng.integers(8, 64))
        sep, stop = (V - 2, V - 1) if seed % 2 else (0, V // 2)
        ids = [v for v in range(V) if v not in (sep, stop)]
        cat = random_catalog(seed, K, 6, len(ids))
        cases.append(([[ids[t] for t in e] for e in cat], V, sep, stop))
    for entries, V, sep, stop in cases:
        _csr_equal(entries, V, sep, stop)


@pytest.mark.parametrize("cid", ["tiny", "product", "product_deep", "structured", "unstructured", "large"])
def test_builder_matches_oracle_configs(L, oracle_lib, cid):
    c = CONFIGS[cid]
    info = _csr_equal(catalog(cid), c.vocab, c.sep, c.stop)
    assert info["n_entries"] == len(catalog(cid))


def test_builder_rejects_bad_catalogs(L):
    V, sep, stop = 16, 14, 15
    for entries in ([[1], []], [[1], [16]], [[1], [-1]], [[1], [2, 14]], [[15]], [[1, 2], [1, 2]]):
        with pytest.raises(tms.TmsError) as ei:
            tms.trie_build(entries, V, sep, stop)
        assert ei.value.code == tms.ERR_CATALOG, entries
    for args in ((16, 14, 14), (16, 16, 1), (1, 0, 0)):
        with pytest.raises(tms.TmsError) as ei:
            tms.trie_build([[1]], *args)
        assert ei.value.code == tms.ERR_INVALID_ARG


def test_state_needs_device_copy(L):
    """A host-only trie cannot back a decode state (checked before any HIP call)."""
    import ctypes as C
    h = tms.trie_build([[1], [2]], 16, 14, 15)
    try:
        out = C.c_void_p()
        rc = L.tms_state_create(h, 1, 1, C.c_void_p(16), 0, 64, None, C.byref(out))
        assert rc == tms.ERR_INVALID_ARG
        assert b"device copy" in L.tms_last_error()
    finally:
        tms.trie_free(h)


def test_bench_reference_sizes_fit_the_table():
    """The streaming reference reads slices of the product table: every byte
    count it is given must fit inside the table."""
    import bench
    V, H = CONFIGS["product"].vocab, CONFIGS["product"].hidden
    sizes, ref = bench.stress_sizes(V, H)
    assert all(n <= V * H * 2 for n in ref)
    assert sizes[256] in ref and sizes[887] in ref


def test_read_reference_refuses_bytes_past_the_tensor():
    import torch
    with pytest.raises(ValueError):
        tms.read_reference(torch.zeros(16, dtype=torch.int32), torch.zeros(1024, dtype=torch.int32), nbytes=65)


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summaries_from_rocprof_csv(tmp_path, capsys, monkeypatch):
    """bench.py's --summarize-trace and --summarize-counters on small
    synthetic rocprofv3 outputs: durations per (kernel, workgroups), the copy
    calibration of FETCH_SIZE / WRITE_SIZE, the traffic JSON it writes, and
    the refusal of counters taken with other kernel sources."""
    import json

    import bench
    trace_hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
                 "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]
    loop = "void tms::(anonymous namespace)::loop_kernel<1, 4, 1, true, true, false>(tms::DevTrie, tms::DevState)"
    _write_csv(str(tmp_path / "trace" / "run_kernel_trace.csv"), trace_hdr,
               [["KERNEL_DISPATCH", loop, 1000, 15000, 512, 1, 1, 512, 1, 1],
                ["KERNEL_DISPATCH", loop, 20000, 33000, 512, 1, 1, 512, 1, 1],
                ["KERNEL_DISPATCH", loop, 40000, 52000, 512 * 64, 1, 1, 512, 1, 1]])
    bench.summarize_trace(str(tmp_path / "trace"))
    out = capsys.readouterr().out
    lines = [l for l in out.splitlines() if l.startswith("loop_kernel")]
    assert len(lines) == 2
    one = [l for l in lines if l.split()[-4] == "1"][0].split()
    assert one[-3] == "2" and float(one[-2]) == 13.5  # two dispatches of 14 and 13 us
    # counters: a copy of 256 MiB reading FETCH 131072 KiB (scale 2) and writing 262144 KiB (scale 1)
    ctr_hdr = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    pmc = tmp_path / "pmc"
    for w, ctr, rows_ in (
            ("copyref", "FETCH_SIZE", [["__amd_rocclr_copyBuffer", 256 * 512, 512, "FETCH_SIZE", 131072.0]]),
            ("copyref", "WRITE_SIZE", [["__amd_rocclr_copyBuffer", 256 * 512, 512, "WRITE_SIZE", 262144.0]]),
            ("headline", "FETCH_SIZE", [[loop, 512, 512, "FETCH_SIZE", 50.0], [loop, 512, 512, "FETCH_SIZE", 70.0]]),
            ("headline", "WRITE_SIZE", [[loop, 512, 512, "WRITE_SIZE", 1.5], [loop, 512, 512, "WRITE_SIZE", 1.5]])):
        _write_csv(str(pmc / f"{w}_{ctr}" / "run_counter_collection.csv"), ctr_hdr, rows_)
    (pmc / "kernel_hash.txt").write_text("not-the-tree\n")
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(pmc))
    tree = bench._kernel_hash()
    (pmc / "kernel_hash.txt").write_text(tree + "\n")
    monkeypatch.setattr(bench, "_kernel_hash", lambda: tree)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))  # the JSON goes to tmp_path/profiles
    os.makedirs(tmp_path / "profiles")
    bench.summarize_counters(str(pmc))
    d = json.loads((tmp_path / "profiles" / "loop_product_pmc.json").read_text())
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["hbm_bytes_per_launch"] == (60.0 * 2.0 + 1.5) * 1024
    assert d["dispatches"] == 2 and d["workgroups"] == 1
