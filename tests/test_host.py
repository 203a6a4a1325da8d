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
