"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Tokens must be identical (bit-exact) except at steps the oracle's own top-two
margin explains (see tests/gpu_util.py); logits within 2e-3 relative plus the
fp32 summation bound.  Paths of the library itself (graph loop vs host loop,
fast vs global trie store, any workgroup split, any batch order, dense+mask vs
sparse) must agree bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import trie_masked_sparse_amd as tms
from gpu_util import (compare, config_case, dev_embedding, gamma, oracle_trie, ref_decode, run_k_pointers,
                      run_step_loop, to_dev)
from synth import CONFIGS, bf16_bits_from_f32, catalog, embedding, random_catalog, stress_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_lib):
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    tms.lib()
    yield
    torch.cuda.synchronize()


def _rand_table(rng, V, H, dtype, scale=0.02):
    x = rng.standard_normal((V, H), dtype=np.float32) * np.float32(scale)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


def _rand_hidden(rng, T, B, H, dtype):
    x = rng.standard_normal((T, B, H), dtype=np.float32)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid", ["tiny", "product", "product_deep", "structured", "unstructured"])
def test_config_parity(cid):
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    tok_g, len_g, ent_g = run_k_pointers(st, hd)
    assert (st.status() == 0).all()
    ref = ref_decode(otr, c.k, embedding(cid), hid)
    assert (ref["status"] == 0).all()
    flips = compare(tok_g, ref, c.hidden, None, len_g, ent_g, where=cid)
    # the host-driven loop: identical tokens, logits within tolerance
    st.reset()
    tok_h, lg_h = run_step_loop(st, hd)
    assert np.array_equal(tok_h, tok_g)
    compare(tok_h, ref, c.hidden, lg_h, where=cid + "/host")
    print(f"{cid}: path={trie.info['path']} nodes={trie.info['n_nodes']} tie flips={flips}")
    st.close()
    trie.close()


def test_large_parity():
    """Large workload at full size (B=256, H=4096, 100k entries, global path):
    every sequence against the oracle, tokens, lengths and entries, with no
    tie-explained flip."""
    cid = "large"
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    assert trie.info["path"] == tms.PATH_GLOBAL
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    tok_g, len_g, ent_g = run_k_pointers(st, hd)
    assert (st.status() == 0).all()
    ref = ref_decode(otr, c.k, embedding(cid), hid)
    assert (ref["status"] == 0).all()
    flips = compare(tok_g, ref, c.hidden, None, len_g, ent_g, where=cid)
    for b in range(c.batch):
        e = ent_g[b]
        assert len(set(e.tolist())) == c.k and (e >= 0).all()
    print(f"large: {c.batch} sequences, {int(len_g.sum())} tokens, tie flips={flips}")
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# Small random cases: ragged hidden sizes, both store paths, prefix pairs
# ---------------------------------------------------------------------------

CASES = [("f32", 100), ("f32", 256), ("f32", 300), ("f32", 4096), ("bf16", 8), ("bf16", 520), ("bf16", 1000),
         ("bf16", 2048), ("bf16", 4096), ("bf16", 8192)]


@pytest.mark.parametrize("dtype,H", CASES)
@pytest.mark.parametrize("path", [tms.PATH_FAST, tms.PATH_GLOBAL])
def test_random_catalog_parity(dtype, H, path):
    rng = np.random.Generator(np.random.PCG64(H * 7 + path))
    V = 700
    sep, stop = (V - 2, V - 1) if (H // 4) % 2 == 0 else (3, 500)
    ids = [v for v in range(V) if v not in (sep, stop)]
    # small id range -> heavy prefix sharing and prefix pairs
    cat = [[ids[t] for t in e] for e in random_catalog(H + path, 60, 6, 24)]
    B, k = 7, 4
    otr = oracle.Trie(cat, V, sep, stop)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, dtype)
    hid = _rand_hidden(rng, T, B, H, dtype)
    trie = tms.Trie(cat, V, sep, stop, path=path)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    tok_g, len_g, ent_g = run_k_pointers(st, hd)
    ref = ref_decode(otr, k, emb, hid)
    compare(tok_g, ref, H, None, len_g, ent_g, where=f"{dtype}/{H}/{path}")
    st.reset()
    tok_h, lg_h = run_step_loop(st, hd)
    assert np.array_equal(tok_h, tok_g)
    compare(tok_h, ref, H, lg_h, where=f"{dtype}/{H}/{path}/host")


@pytest.mark.parametrize("fan,path", [(250, tms.PATH_FAST), (250, tms.PATH_GLOBAL), (650, tms.PATH_GLOBAL)])
def test_wide_nodes(fan, path):
    """A root with hundreds of edges (several edge batches per wavefront)."""
    rng = np.random.Generator(np.random.PCG64(fan))
    V, H, B, k = 1024, 512, 9, 3
    firsts = rng.choice(V - 2, size=fan, replace=False)
    cat = [[int(f)] + [int(x) for x in rng.integers(0, V - 2, size=int(rng.integers(0, 3)))] for f in firsts]
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "bf16")
    hid = _rand_hidden(rng, T, B, H, "bf16")
    trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
    st = tms.State(trie, B, k, to_dev(emb))
    tok_h, lg_h = run_step_loop(st, to_dev(hid))
    compare(tok_h, ref_decode(otr, k, emb, hid), H, lg_h, where=f"wide{fan}")


def test_exact_ties_lower_id_wins():
    """Legal tokens with identical rows tie exactly; the lower id must win."""
    rng = np.random.Generator(np.random.PCG64(3))
    V, H = 512, 256
    emb = _rand_table(rng, V, H, "bf16")
    toks = sorted(rng.choice(V - 2, size=40, replace=False).tolist())
    for a in (5, 9, 17):
        emb[toks[a]] = emb[toks[30]]
    cat = [[t] for t in toks]
    k = 4
    h = emb[toks[30]].copy()
    hid = np.broadcast_to(h, (2 * k, 2, H)).copy()
    for path in (tms.PATH_FAST, tms.PATH_GLOBAL):
        trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
        st = tms.State(trie, 2, k, to_dev(emb))
        tok, ln, ent = run_k_pointers(st, to_dev(hid))
        for b in range(2):
            assert list(tok[b][::2]) == [toks[5], toks[9], toks[17], toks[30]]
    ref = ref_decode(oracle.Trie(cat, V, V - 2, V - 1), k, emb, hid)
    compare(tok, ref, H, where="ties")


def test_zero_hidden_lexicographic():
    """h = 0: every logit is +0, so the answer is the lexicographic minimum."""
    cid = "structured"
    c, otr, T, hid = config_case(cid, B=4)
    zero = np.zeros_like(hid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 4, c.k, dev_embedding(cid))
    tok, lg = run_step_loop(st, to_dev(zero))
    ref = ref_decode(otr, c.k, embedding(cid), zero)
    assert np.array_equal(tok, ref["tokens"])
    live = lg[tok >= 0]
    assert np.all(live == 0.0) and not np.any(np.signbit(live))


# ---------------------------------------------------------------------------
# Bit identity between the library's own paths
# ---------------------------------------------------------------------------

def test_paths_splits_graph_and_shuffle_identical():
    cid = "structured"
    c, otr, T, hid = config_case(cid, B=16)
    hd = to_dev(hid)
    emb = dev_embedding(cid)
    base = None
    for path in (tms.PATH_FAST, tms.PATH_GLOBAL):
        trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop, path=path)
        st = tms.State(trie, 16, c.k, emb)
        for split in (1, 2, 3, 8, 0):
            tms.state_set_split(st.h, split)
            st.reset()
            tok, lg = run_step_loop(st, hd)
            if base is None:
                base = (tok, lg)
            assert np.array_equal(tok, base[0]), (path, split)
            assert np.array_equal(lg, base[1], equal_nan=True), (path, split)
            # every loop form; graph replays with eager work and syncs in between
            for mode in (tms.LOOP_RESIDENT, tms.LOOP_GRAPH, tms.LOOP_STREAM):
                tms.state_set_loop(st.h, mode)
                for rep in range(3 if mode == tms.LOOP_GRAPH else 1):
                    st.reset()
                    torch.cuda.synchronize()
                    g_tok, g_len, g_ent = run_k_pointers(st, hd)
                    assert np.array_equal(g_tok, base[0]), (path, split, mode, rep)
                    ex = st.export(live=True)
                    if mode == tms.LOOP_RESIDENT:
                        ref_state = ex
                    else:
                        for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
                            assert np.array_equal(ex[key], ref_state[key]), (key, mode)
        st.close()
        trie.close()
    # batch shuffle: permuting the sequences permutes the outputs, nothing else
    perm = np.random.Generator(np.random.PCG64(1)).permutation(16)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 16, c.k, emb)
    tok, lg = run_step_loop(st, to_dev(np.ascontiguousarray(hid[:, perm, :])))
    assert np.array_equal(tok, base[0][perm])
    assert np.array_equal(lg, base[1][perm], equal_nan=True)


@pytest.mark.parametrize("cid", ["product", "unstructured"])
def test_resident_loop_in_captured_graph(cid):
    """The resident decode (one kernel, or grouped root heads plus loop
    kernels) captured in a caller's HIP graph with the reset inside it:
    several replays, with the caller's own eager work and synchronisations in
    between, each equal to the eager answer."""
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    want = run_k_pointers(st, hd)
    tok = torch.full((c.batch, T), -7, dtype=torch.int32, device="cuda")
    ln = torch.zeros(c.batch, dtype=torch.int32, device="cuda")
    ent = torch.zeros((c.batch, c.k), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for _ in range(3):
            st.reset()
            tms.decode_k_pointers(st, hd, tok, ln, ent, check=False)
    torch.cuda.synchronize()
    for rep in range(3):
        tok.fill_(-7)
        ln.zero_()
        ent.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = (tok.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy())
        for a, b in zip(got, want):
            assert np.array_equal(a, b), (cid, rep)
        assert (st.status() == 0).all()
        # eager work on the same state between replays
        st.reset()
        e = run_k_pointers(st, hd)
        assert all(np.array_equal(a, b) for a, b in zip(e, want))
    del g
    st.close()
    trie.close()


@pytest.mark.parametrize("loop", [tms.LOOP_GRAPH, tms.LOOP_STREAM])
def test_step_loops_in_captured_graph(loop):
    """The step-kernel forms of the whole decode (the library's own graph of
    step kernels, or the launches one by one) recorded in a caller's graph,
    root grouped (the unstructured catalog's wide root), reset inside it:
    the kernels are recorded themselves, each grouped step after a snapshot
    of its own, so that several replays, with the caller's eager work and a
    fresh eager decode in between, each give the eager answer."""
    cid = "unstructured"
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    tms.state_set_loop(st, loop)
    hd = to_dev(hid)
    want = run_k_pointers(st, hd)
    compare(want[0], ref_decode(otr, c.k, embedding(cid), hid), c.hidden, where=f"{cid} eager, loop {loop}")
    tok = torch.full((c.batch, T), -7, dtype=torch.int32, device="cuda")
    ln = torch.zeros(c.batch, dtype=torch.int32, device="cuda")
    ent = torch.zeros((c.batch, c.k), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        st.reset()
        tms.decode_k_pointers(st, hd, tok, ln, ent, check=False)
    torch.cuda.synchronize()
    for rep in range(3):
        tok.fill_(-7)
        ln.zero_()
        ent.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = (tok.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy())
        for a, b in zip(got, want):
            assert np.array_equal(a, b), (loop, rep)
        assert (st.status() == 0).all()
        st.reset()
        e = run_k_pointers(st, hd)
        assert all(np.array_equal(a, b) for a, b in zip(e, want)), (loop, rep)
    del g
    st.close()
    trie.close()


def test_graph_loop_follows_grouping_and_split_changes():
    """The graph form with the same buffers on every call, the grouping and
    the split changed between calls: each change records the graph again
    (another kernel or grid in the same shape), and every answer equals the
    first, with the exported state."""
    cid = "unstructured"
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    tms.state_set_loop(st, tms.LOOP_GRAPH)
    hd = to_dev(hid)
    tok = torch.empty((c.batch, T), dtype=torch.int32, device="cuda")
    ln = torch.empty(c.batch, dtype=torch.int32, device="cuda")
    ent = torch.empty((c.batch, c.k), dtype=torch.int32, device="cuda")
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    first = None
    for mode, split in ((tms.STEP_GROUP_OFF, 0), (tms.STEP_GROUP_ROOT, 0), (tms.STEP_GROUP_ROOT, 3),
                        (tms.STEP_GROUP_NODES, 3), (tms.STEP_GROUP_OFF, 2), (tms.STEP_GROUP_NODES, 0)):
        tms.state_set_step_grouping(st, mode)
        tms.state_set_split(st, split)
        for _ in range(2):
            st.reset()
            tms.decode_k_pointers(st, hd, tok, ln, ent)
            torch.cuda.synchronize()
            got = (tok.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy(), st.export(live=True))
            if first is None:
                first = got
                compare(got[0], ref_decode(otr, c.k, embedding(cid), hid), c.hidden, gpu_len=got[1],
                        gpu_entries=got[2], where="graph form, grouping off")
            for a, b in zip(got[:3], first[:3]):
                assert np.array_equal(a, b), (mode, split)
            for key in keys:
                assert np.array_equal(got[3][key], first[3][key]), (mode, split, key)
    st.close()
    trie.close()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_check_refused_while_recording():
    """The fail-loud check synchronises, which a stream being recorded into a
    graph cannot do: every checked call refuses before recording anything,
    and the state then decodes as if nothing had happened."""
    cid = "tiny"
    c, otr, T, hid = config_case(cid, B=4)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 4, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    tok = torch.empty(4, dtype=torch.int32, device="cuda")
    toks = torch.empty((4, T), dtype=torch.int32, device="cuda")
    calls = [lambda: tms.decode_step_sparse(st, hd[0], tok),
             lambda: tms.decode_step_dense_masked(st, hd[0], tok),
             lambda: tms.decode_k_pointers(st, hd, toks),
             lambda: tms.advance_forced(st, tok)]
    for call in calls:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with pytest.raises(tms.TmsError, match="recorded"):
            with torch.cuda.graph(g, capture_error_mode="relaxed"):
                call()
        del g
        torch.cuda.synchronize()
    got = run_k_pointers(st, hd)
    ref = ref_decode(otr, c.k, embedding(cid), hid)
    compare(got[0], ref, c.hidden, gpu_len=got[1], gpu_entries=got[2], where="after refused recordings")
    st.close()
    trie.close()


@pytest.mark.parametrize("mode", [tms.STEP_GROUP_ROOT, tms.STEP_GROUP_NODES])
def test_grouped_step_recorded_once_replayed_per_token(mode):
    """One grouped step recorded in a caller's graph and replayed once per
    token, the hidden vectors copied into its input between replays (a
    serving loop's pattern): each replay snapshots the nodes it starts from,
    so every step's tokens and logits equal the eager steps', bit for bit;
    and an eager step right after the recording (before any replay) still
    reads a current snapshot."""
    cid = "unstructured"
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    tms.state_set_step_grouping(st, mode)
    hd = to_dev(hid)
    st.reset()
    want_t, want_l = (a.T for a in run_step_loop(st, hd))  # [T][B]
    h_in = torch.empty_like(hd[0])
    tok = torch.empty(c.batch, dtype=torch.int32, device="cuda")
    lg = torch.empty(c.batch, dtype=torch.float32, device="cuda")
    st.reset()
    st.status()  # the pending reset runs now, outside the recording
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        tms.decode_step_sparse(st, h_in, tok, lg, check=False)
    torch.cuda.synchronize()
    # nothing recorded has run: an eager first step reads a fresh snapshot
    t0 = torch.empty_like(tok)
    l0 = torch.empty_like(lg)
    tms.decode_step_sparse(st, hd[0], t0, l0)
    torch.cuda.synchronize()
    assert np.array_equal(t0.cpu().numpy(), want_t[0]) and np.array_equal(l0.cpu().numpy(), want_l[0], equal_nan=True)
    for t in range(1, T):
        h_in.copy_(hd[t])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), want_t[t]), (mode, t)
        assert np.array_equal(lg.cpu().numpy(), want_l[t], equal_nan=True), (mode, t)
    assert (st.status() == 0).all()
    del g
    st.close()
    trie.close()


def test_two_tries_no_contamination():
    """Interleaved steps on two tries and two states give the same results as
    running each alone (each grammar owns its store)."""
    outs = {}
    for cid in ("product", "structured"):
        c, otr, T, hid = config_case(cid, B=4)
        trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
        st = tms.State(trie, 4, c.k, dev_embedding(cid))
        outs[cid] = (run_step_loop(st, to_dev(hid)), trie, st, to_dev(hid), T)
    (pa, ta, sa, ha, Ta), (pb, tb, sb, hb, Tb) = outs["product"], outs["structured"]
    sa.reset()
    sb.reset()
    toks = {n: torch.empty((T, 4), dtype=torch.int32, device="cuda") for n, T in (("a", Ta), ("b", Tb))}
    for t in range(max(Ta, Tb)):
        if t < Ta:
            tms.decode_step_sparse(sa.h, ha[t], toks["a"][t])
        if t < Tb:
            tms.decode_step_sparse(sb.h, hb[t], toks["b"][t])
    torch.cuda.synchronize()
    assert np.array_equal(toks["a"].cpu().numpy().T, pa[0])
    assert np.array_equal(toks["b"].cpu().numpy().T, pb[0])


def test_states_on_concurrent_streams():
    """Four states on four streams with their work in flight at once: the
    resident loop (one kernel, and grouped root heads with loop phases) and
    the root-grouped step kernels, each decoding repeatedly from resets, with
    no synchronisation between the streams.  Every answer equals the one the
    same state gives alone: states share nothing on the device."""
    jobs = []
    for cid, loop in (("product", tms.LOOP_RESIDENT), ("unstructured", tms.LOOP_RESIDENT),
                      ("structured", tms.LOOP_STREAM), ("unstructured", tms.LOOP_GRAPH)):
        c, otr, T, hid = config_case(cid)
        trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
        st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
        tms.state_set_loop(st, loop)
        hd = to_dev(hid)
        want = run_k_pointers(st, hd)
        outs = [tuple(torch.full(a.shape, -7, dtype=torch.int32, device="cuda") for a in want) for _ in range(3)]
        jobs.append((cid, loop, trie, st, hd, want, outs, torch.cuda.Stream()))
    torch.cuda.synchronize()
    for rep in range(3):
        for cid, loop, trie, st, hd, want, outs, stream in jobs:
            with torch.cuda.stream(stream):
                st.reset(stream)
                tms.decode_k_pointers(st, hd, *outs[rep], stream=stream, check=False)
    torch.cuda.synchronize()
    for cid, loop, trie, st, hd, want, outs, stream in jobs:
        for rep in range(3):
            for a, b in zip(outs[rep], want):
                assert np.array_equal(a.cpu().numpy(), b), (cid, loop, rep)
        assert (st.status() == 0).all(), (cid, loop)
        st.close()
        trie.close()


# ---------------------------------------------------------------------------
# Dense + mask cross-check
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,B", [("tiny", 1), ("product", 1), ("structured", 8), ("unstructured", 4),
                                   ("structured", 24), ("structured", 64), ("large", 24), ("structured", 128),
                                   ("large", 256)])
def test_dense_masked_matches_sparse(cid, B, monkeypatch):
    """Dense head + mask against the sparse step and the oracle.  B = 1 (and the
    vector head at any B) uses the sparse head's per-row arithmetic, so logits
    and tokens are bit-identical; the matrix-core head at B > 1 sums in its own
    order, so it is held to the oracle with the any-order tolerance and tie
    rule."""
    c, otr, T, hid = config_case(cid, B=B)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    hd = to_dev(hid)
    st = tms.State(trie, B, c.k, dev_embedding(cid))
    s_tok, s_lg = run_step_loop(st, hd)
    st.reset()
    nfull = min(T, 3)
    full = torch.zeros((T, B, c.vocab), dtype=torch.float32, device="cuda") if B * c.vocab * T <= 60_000_000 else None
    d_tok, d_lg = run_step_loop(st, hd, dense=True, full=full)
    ref = ref_decode(otr, c.k, embedding(cid), hid)
    mfma = B > 1 and c.dtype == "bf16"
    if not mfma:
        assert np.array_equal(d_tok, s_tok)
        assert np.array_equal(d_lg, s_lg, equal_nan=True)
    flips = compare(d_tok, ref, c.hidden, d_lg, where=cid + "/dense", depth=c.hidden + 1 if mfma else None,
                    max_flips=2 if mfma else 0)
    print(f"{cid} B={B} dense: tie flips={flips}", flush=True)
    if mfma:
        # the vector head at the same B: bit-identical to the sparse step
        monkeypatch.setenv("TMS_DENSE_VECTOR", "1")
        st2 = tms.State(trie, B, c.k, dev_embedding(cid))
        v_tok, v_lg = run_step_loop(st2, hd, dense=True)
        assert np.array_equal(v_tok, s_tok)
        assert np.array_equal(v_lg, s_lg, equal_nan=True)
        st2.close()
    if full is not None:
        fl = full.cpu().numpy()
        emb_np = embedding(cid)
        rng = np.random.Generator(np.random.PCG64(9))
        for t in range(nfull):
            for b in sorted(set([0, B - 1])):
                rows = np.arange(c.vocab) if c.vocab <= 8192 else rng.choice(c.vocab, 512, replace=False)
                for v in rows:
                    want, sa = oracle.logit(emb_np, int(v), hid[t, b])
                    tol = 2e-3 * abs(want) + gamma(c.hidden + 1) * sa
                    assert abs(float(fl[t, b, v]) - want) <= tol, (cid, t, b, v)
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# Materialiser, advance and state against the oracle under teacher forcing
# ---------------------------------------------------------------------------

def _forced_walk(cat, V, sep, stop, k, B, path, seed, check_live=True):
    otr = oracle.Trie(cat, V, sep, stop)
    trie = tms.Trie(cat, V, sep, stop, path=path)
    emb = torch.zeros((V, 8), dtype=torch.float32, device="cuda")
    st = tms.State(trie, B, k, emb)
    orefs = [oracle.State(otr, k) for _ in range(B)]
    rng = np.random.Generator(np.random.PCG64(seed))
    cap = trie.info["cap"]
    legal = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
    nleg = torch.zeros(B, dtype=torch.int32, device="cuda")
    forced = torch.zeros(B, dtype=torch.int32, device="cuda")
    T = k * (otr.max_depth + 1)
    for step in range(T + 1):
        tms.legal_set(st.h, legal, nleg)
        torch.cuda.synchronize()
        lg, nl = legal.cpu().numpy(), nleg.cpu().numpy()
        choice = np.full(B, -1, np.int32)
        for b in range(B):
            want = orefs[b].legal()
            if want is None:
                assert nl[b] == -1, (step, b)
                continue
            assert list(lg[b, :nl[b]]) == list(want[0]), (step, b)
            choice[b] = int(want[0][rng.integers(0, len(want[0]))])
        if (choice < 0).all():
            break
        forced.copy_(torch.from_numpy(choice))
        tms.advance_forced(st.h, forced)
        for b in range(B):
            if choice[b] >= 0:
                assert orefs[b].advance(int(choice[b])) == oracle.OK
        ex = st.export(live=check_live)
        for b in range(B):
            oi = orefs[b].info()
            got = (ex["node"][b], ex["depth"][b], ex["done"][b], ex["finished"][b], ex["status"][b], ex["n_emitted"][b])
            assert got == (oi["node"], oi["depth"], oi["done"], oi["finished"], oi["status"], oi["n_emitted"]), (step, b)
            assert list(ex["entries"][b]) == list(orefs[b].entries())
            if check_live:
                assert np.array_equal(ex["live"][b], orefs[b].live()), (step, b)
    assert all(o.info()["finished"] for o in orefs)


@pytest.mark.parametrize("path", [tms.PATH_FAST, tms.PATH_GLOBAL])
def test_teacher_forced_small(path):
    cases = [([[1], [1, 2], [1, 2, 3], [4]], 16, 14, 15, 3), ([[3, 3], [3], [3, 3, 3]], 16, 0, 15, 3),
             ([[5, 6], [5], [7], [5, 6, 7]], 16, 15, 1, 4)]
    for seed in range(12):
        cat = random_catalog(seed, 12, 4, 6)
        cases.append((cat, 16, 14, 15, 1 + seed % 4))
    for i, (cat, V, sep, stop, k) in enumerate(cases):
        _forced_walk(cat, V, sep, stop, min(k, len(cat)), 6, path, i)


def test_teacher_forced_structured():
    c = CONFIGS["structured"]
    _forced_walk(catalog("structured"), c.vocab, c.sep, c.stop, c.k, 16, tms.PATH_AUTO, 5)


@pytest.mark.parametrize("cid", ["product", "product_deep", "structured", "unstructured"])
def test_steps_without_logits_match_steps_with_logits(cid):
    """Host-driven steps asked for tokens only take the steps a node record
    decides (a single edge; a leaf terminal's sep or stop) without the head:
    tokens and the exported state after every step identical to steps that
    return logits, and the oracle's tokens (fast store, global store, and the
    root grouped in the step launch on the unstructured catalog)."""
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    tok_l, lg = run_step_loop(st, hd)
    x_l = st.export(live=True)
    st.reset()
    tok_n, lg_n = run_step_loop(st, hd, logits=False)
    x_n = st.export(live=True)
    assert np.array_equal(tok_l, tok_n)
    assert np.isnan(lg_n).all()
    for key in keys:
        assert np.array_equal(x_l[key], x_n[key]), key
    compare(tok_n, ref_decode(otr, c.k, embedding(cid), hid), c.hidden, None, where=f"{cid} tokens only")
    st.close()
    trie.close()


@pytest.mark.parametrize("split", [3, 8])
def test_steps_without_logits_many_workgroups_per_sequence(split):
    """Headless steps when each sequence has several workgroups and the grid
    (512 sequences x split) is larger than the chip holds at once, so that
    some workgroups of a sequence start after others have finished: every
    workgroup must decide from the same state.  Tokens-only steps equal steps
    with logits, in the plain and the root-grouped step, and the GRAPH loop
    (tokens only) equals the resident loop and the oracle."""
    rng = np.random.Generator(np.random.PCG64(900 + split))
    V, H, k, B = 4000, 64, 2, 512
    cat = random_catalog(901, 400, 12, V - 2, min_len=6)  # long single-edge chains below the root
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "fp32")
    hid = _rand_hidden(rng, T, B, H, "fp32")
    ref = ref_decode(otr, k, emb, hid)
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    tms.state_set_split(st, split)
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    for mode in (tms.STEP_GROUP_OFF, tms.STEP_GROUP_ROOT, tms.STEP_GROUP_NODES):
        tms.state_set_step_grouping(st, mode)
        st.reset()
        tok_l, lg = run_step_loop(st, hd)
        x_l = st.export(live=True)
        st.reset()
        tok_n, _ = run_step_loop(st, hd, logits=False)
        x_n = st.export(live=True)
        assert np.array_equal(tok_l, tok_n), mode
        for key in keys:
            assert np.array_equal(x_l[key], x_n[key]), (mode, key)
        compare(tok_n, ref, H, None, where=f"split {split} grouping {mode} tokens only")
        tms.state_set_loop(st, tms.LOOP_GRAPH)
        st.reset()
        tok_g, ln_g, ent_g = run_k_pointers(st, hd)
        tms.state_set_loop(st, tms.LOOP_RESIDENT_SOLO)
        st.reset()
        tok_r, ln_r, ent_r = run_k_pointers(st, hd)
        assert np.array_equal(tok_g, tok_r) and np.array_equal(ent_g, ent_r), mode
        compare(tok_g, ref, H, None, ln_g, ent_g, where=f"split {split} grouping {mode} graph")
        tms.state_set_loop(st, tms.LOOP_RESIDENT)
    st.close()
    trie.close()


def test_steps_without_logits_empty_and_spent_nodes():
    """The headless steps' statuses: a single edge whose live count is zero is
    an empty legal set (EMPTY_MASK), the same as the head reports; and every
    tiny catalog (prefix pairs, leaf terminals, k = K) stepped with and
    without logits gives the same tokens and state."""
    V, H = 16, 64
    rng = np.random.Generator(np.random.PCG64(77))
    emb = rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.2)
    cases = [([[1, 2, 3]], 1), ([[1], [1, 2], [1, 2, 3], [4]], 4), ([[3, 3], [3], [3, 3, 3]], 3),
             ([[5, 6], [5], [7], [5, 6, 7]], 2)] + [(random_catalog(300 + i, 10, 4, 12), 1 + i % 4) for i in range(10)]
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    for i, (cat, k) in enumerate(cases):
        k = min(k, len(cat))
        trie = tms.Trie(cat, V, V - 2, V - 1, path=tms.PATH_FAST if i % 2 else tms.PATH_GLOBAL)
        T = k * (trie.info["max_depth"] + 1)
        hid = rng.standard_normal((T, 3, H), dtype=np.float32)
        st = tms.State(trie, 3, k, to_dev(emb))
        hd = to_dev(hid)
        out = []
        for logits in (True, False):
            st.reset()
            if i == 0:  # the edge after token 1 (a single-edge node) has no live pointer for sequence 1
                tms.debug_set_live(st.h, 1, int(trie.csr()["begin"][1]), 0)
            tok, _ = run_step_loop(st, hd, check=False, logits=logits)
            out.append((tok, st.export(live=True)))
        assert np.array_equal(out[0][0], out[1][0]), i
        for key in keys:
            assert np.array_equal(out[0][1][key], out[1][1][key]), (i, key)
        if i == 0:
            assert list(out[1][1]["status"]) == [0, tms.ERR_EMPTY_MASK, 0]
        st.close()
        trie.close()


def _loop_forms(st, hd, check=True):
    """(name, tokens, len, entries, status) of decode_k_pointers in every
    loop form on a reset state."""
    out = []
    for name, mode in (("resident", tms.LOOP_RESIDENT), ("solo", tms.LOOP_RESIDENT_SOLO),
                       ("grouped", tms.LOOP_RESIDENT_GROUPED), ("graph", tms.LOOP_GRAPH),
                       ("stream", tms.LOOP_STREAM)):
        tms.state_set_loop(st, mode)
        st.reset()
        tok, ln, ent = run_k_pointers(st, hd, check=check)
        out.append((name, tok, ln, ent, st.status().copy()))
    tms.state_set_loop(st, tms.LOOP_RESIDENT)
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_large_batch_every_loop_form(dtype):
    """700 sequences: far more workgroups than compute units in every form,
    175 member tiles of 4 at the grouped root head (its vector form at
    H = 128) and 44 tiles of 16 in the grouped step, root row tiles padded to
    a multiple of 8; every loop form, and host-driven steps with and without
    logits, against the oracle."""
    rng = np.random.Generator(np.random.PCG64(700 + len(dtype)))
    V, H, k, B = 3000, 128, 2, 700
    cat = random_catalog(4242, 600, 6, V - 2, min_len=2)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    b = otr.csr()["begin"]
    assert b[1] - b[0] >= 64
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, dtype)
    hid = _rand_hidden(rng, T, B, H, dtype)
    ref = ref_decode(otr, k, emb, hid)
    assert (ref["status"] == 0).all()
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    for name, tok, ln, ent, status in _loop_forms(st, hd):
        compare(tok, ref, H, None, ln, ent, where=f"B={B} {dtype} {name}")
        assert (status == 0).all(), name
    st.reset()
    tok_h, lg_h = run_step_loop(st, hd)
    compare(tok_h, ref, H, lg_h, where=f"B={B} {dtype} steps")
    st.reset()
    tok_n, _ = run_step_loop(st, hd, logits=False)
    assert np.array_equal(tok_n, tok_h)
    st.close()
    trie.close()


def test_graph_loop_alternating_buffers():
    """The GRAPH loop form called with two sets of buffers in turn, with no
    synchronisation between the calls (the instantiated graph takes each
    call's pointers in place), then with a longer step budget (the graph is
    rebuilt): every answer against the oracle."""
    rng = np.random.Generator(np.random.PCG64(57))
    V, H, k, B = 500, 64, 2, 12
    cat = random_catalog(57, 90, 6, V - 2, min_len=1)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    emb = _rand_table(rng, V, H, "fp32")
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    tms.state_set_loop(st, tms.LOOP_GRAPH)
    T0 = k * (otr.max_depth + 1)
    for T in (T0, T0 + 3):
        hids = [_rand_hidden(rng, T, B, H, "fp32") for _ in range(2)]
        refs = [ref_decode(otr, k, emb, h) for h in hids]
        devs = [to_dev(h) for h in hids]
        outs = [(torch.full((B, T), -7, dtype=torch.int32, device="cuda"), torch.zeros(B, dtype=torch.int32, device="cuda"),
                 torch.zeros((B, k), dtype=torch.int32, device="cuda")) for _ in range(6)]
        for i, (tok, ln, ent) in enumerate(outs):  # A, B, A, B, ...: no host wait between calls
            st.reset()
            tms.decode_k_pointers(st, devs[i % 2], tok, ln, ent, check=False)
        torch.cuda.synchronize()
        assert (st.status() == 0).all()
        for i, (tok, ln, ent) in enumerate(outs):
            compare(tok.cpu().numpy(), refs[i % 2], H, None, ln.cpu().numpy(), ent.cpu().numpy(),
                    where=f"graph call {i} T={T}")
    st.close()
    trie.close()


def test_short_budget_refused_in_every_form():
    """decode_k_pointers needs T >= k * (max_depth + 1) steps (enough for
    every answer to stop): every loop form refuses one step less on the host
    (INVALID_ARG, nothing enqueued), and the state then decodes the full
    budget to the oracle's answer."""
    rng = np.random.Generator(np.random.PCG64(31))
    V, H, k, B = 400, 96, 3, 24
    cat = random_catalog(31, 120, 7, V - 2, min_len=1)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    emb = _rand_table(rng, V, H, "fp32")
    T = k * (otr.max_depth + 1)
    hid = _rand_hidden(rng, T, B, H, "fp32")
    ref = ref_decode(otr, k, emb, hid)
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    for mode in (tms.LOOP_RESIDENT, tms.LOOP_RESIDENT_SOLO, tms.LOOP_RESIDENT_GROUPED, tms.LOOP_GRAPH,
                 tms.LOOP_STREAM):
        tms.state_set_loop(st, mode)
        st.reset()
        with pytest.raises(tms.TmsError) as ei:
            run_k_pointers(st, hd[:T - 1])
        assert ei.value.code == tms.ERR_INVALID_ARG
        tok, ln, ent = run_k_pointers(st, hd)
        compare(tok, ref, H, None, ln, ent, where=f"after a refused call, loop form {mode}")
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# Fail loudly
# ---------------------------------------------------------------------------

def test_device_errors_are_sticky_and_isolated():
    c, otr, T, hid = config_case("tiny", B=3)
    trie = tms.Trie(catalog("tiny"), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 3, c.k, dev_embedding("tiny"))
    csr = trie.csr()
    # empty mask for sequence 1: no live pointer below any root edge
    for e in range(csr["begin"][0], csr["begin"][1]):
        tms.debug_set_live(st.h, 1, e, 0)
    tok, lg = run_step_loop(st, to_dev(hid), check=False)
    status = st.status()
    assert list(status) == [0, tms.ERR_EMPTY_MASK, 0]
    assert (tok[1] == -1).all() and np.isnan(lg[1]).all()
    ref = ref_decode(otr, c.k, embedding("tiny"), hid[:, [0, 2], :])
    compare(tok[[0, 2]], ref, c.hidden, lg[[0, 2]], where="isolated")
    with pytest.raises(tms.TmsError) as ei:
        tms.state_sync_status(st.h, 3, check=True)
    assert ei.value.code == tms.ERR_EMPTY_MASK
    # unwalkable forced token
    st.reset()
    forced = torch.tensor([c.stop, -1, c.sep], dtype=torch.int32, device="cuda")
    tms.advance_forced(st.h, forced, check=False)
    assert list(st.status()) == [tms.ERR_NOT_WALKABLE, 0, tms.ERR_NOT_WALKABLE]
    # the same through the checked call: it raises without a status query
    st.reset()
    with pytest.raises(tms.TmsError) as ei:
        tms.advance_forced(st, forced)
    assert ei.value.code == tms.ERR_NOT_WALKABLE and "2 of 3 sequences" in str(ei.value)
    # the trie cannot be freed while a state uses it
    with pytest.raises(tms.TmsError) as ei:
        tms.trie_free(trie.h)
    assert ei.value.code == tms.ERR_BUSY
    st.close()
    trie.close()


@pytest.mark.parametrize("mode", ["resident", "grouped", "graph", "step", "dense"])
def test_decode_raises_on_empty_mask(mode):
    """The decode calls fail loudly by default: with every root edge of one
    sequence emptied, the call itself raises TmsError(EMPTY_MASK) naming that
    sequence, with no status query by the caller."""
    c, otr, T, hid = config_case("tiny", B=3)
    trie = tms.Trie(catalog("tiny"), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 3, c.k, dev_embedding("tiny"))
    loop = {"resident": tms.LOOP_RESIDENT_SOLO, "grouped": tms.LOOP_RESIDENT_GROUPED, "graph": tms.LOOP_GRAPH}
    if mode in loop:
        tms.state_set_loop(st, loop[mode])
    csr = trie.csr()
    st.reset()
    st.export()  # carries out the reset, so the live counts below stick
    for e in range(csr["begin"][0], csr["begin"][1]):
        tms.debug_set_live(st, 1, e, 0)
    hd = to_dev(hid)
    tok = torch.empty((3, T), dtype=torch.int32, device="cuda")
    with pytest.raises(tms.TmsError) as ei:
        if mode == "step":
            tms.decode_step_sparse(st, hd[0], tok[:, 0].contiguous())
        elif mode == "dense":
            tms.decode_step_dense_masked(st, hd[0], tok[:, 0].contiguous())
        else:
            tms.decode_k_pointers(st, hd, tok)
    assert ei.value.code == tms.ERR_EMPTY_MASK
    assert "sequence 1" in str(ei.value) and "1 of 3 sequences" in str(ei.value)
    st.close()
    trie.close()


def test_host_side_errors():
    c = CONFIGS["unstructured"]
    emb = dev_embedding("unstructured")
    with pytest.raises(tms.TmsError) as ei:
        tms.Trie(catalog("unstructured"), c.vocab, c.sep, c.stop, path=tms.PATH_FAST)
    assert ei.value.code == tms.ERR_FANOUT
    trie = tms.Trie(catalog("unstructured"), c.vocab, c.sep, c.stop)
    assert trie.info["path"] == tms.PATH_GLOBAL
    with pytest.raises(tms.TmsError) as ei:
        tms.State(trie, 2, 1001, emb)
    assert ei.value.code == tms.ERR_K
    with pytest.raises(tms.TmsError) as ei:
        tms.State(trie, 2, 2, emb.reshape(-1)[: c.vocab * 2044].view(c.vocab, 2044))
    assert ei.value.code in (tms.ERR_INVALID_ARG,)
    st = tms.State(trie, 2, 2, emb)
    short = torch.zeros((3, 2, c.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tms.TmsError) as ei:
        tms.decode_k_pointers(st.h, short, torch.zeros((2, 3), dtype=torch.int32, device="cuda"))
    assert ei.value.code == tms.ERR_INVALID_ARG
    # the bitmask no-repeat state needs a catalog of at most 128 entries
    with pytest.raises(tms.TmsError) as ei:
        tms.state_set_norepeat(st, tms.NOREPEAT_BITMASK)
    assert ei.value.code == tms.ERR_INVALID_ARG
    tms.state_set_norepeat(st, tms.NOREPEAT_LIVE)
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# The sparse head on its own
# ---------------------------------------------------------------------------

def test_gather_gemv_rows():
    cid = "product"
    emb_np, emb = embedding(cid), dev_embedding(cid)
    V, H = emb_np.shape
    rng = np.random.Generator(np.random.PCG64(21))
    B, cap = 6, 300
    n_rows = np.array([0, 1, 150, 300, 37, 299], np.int32)
    rows = rng.integers(0, V, size=(B, cap)).astype(np.int32)
    rows[2, 10] = -5
    rows[3, 7] = V + 3
    rows[4, 3] = rows[4, 30]  # duplicate row -> identical logit
    hid = bf16_bits_from_f32(rng.standard_normal((B, H), dtype=np.float32))
    out = torch.full((B, cap), 1234.5, dtype=torch.float32, device="cuda")
    tms.gather_gemv(emb, to_dev(hid), to_dev(rows), to_dev(n_rows), out)
    o = out.cpu().numpy()
    for b in range(B):
        assert (o[b, n_rows[b]:] == 1234.5).all()
        for j in range(n_rows[b]):
            r = rows[b, j]
            if r < 0 or r >= V:
                assert math.isnan(o[b, j])
                continue
            want, sa = oracle.logit(emb_np, int(r), hid[b])
            assert abs(float(o[b, j]) - want) <= 2e-3 * abs(want) + gamma(H + 1) * sa, (b, j)
    assert o[4, 3] == o[4, 30]


@pytest.mark.parametrize("grid,unroll", [(0, 2), (1024, 2), (7, 8), (4096, 4), (3, 1)])
def test_read_reference_reads_every_byte_once(grid, unroll):
    """The streaming-read reference kernel behind the bandwidth comparisons:
    the XOR of its 1024 output words is the XOR of every 32-bit word of the
    bytes asked for (each read exactly once, none past them), for byte counts
    that leave ragged passes and a tail, and a prefix of a larger buffer."""
    rng = np.random.Generator(np.random.PCG64(90 + grid + unroll))
    data = rng.integers(-2**31, 2**31, size=(3 << 20) + 12, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(data).cuda()
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for nbytes in (16, 4096 + 16, (1 << 20) + 48, (3 << 20) * 4 - 32, data.nbytes):
        out.zero_()
        tms.read_reference(src, out, grid, unroll, nbytes)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(data[:nbytes // 4])
        got = np.bitwise_xor.reduce(out.cpu().numpy())
        assert got == want, (grid, unroll, nbytes)
    with pytest.raises(ValueError):
        tms.read_reference(src, out, grid, unroll, data.nbytes + 16)


def test_gather_gemv_stress_shape_sampled():
    """The bandwidth stress shape (64 sequences x 256 distinct rows), sampled."""
    cid = "product"
    emb_np, emb = embedding(cid), dev_embedding(cid)
    V, H = emb_np.shape
    sets = stress_rows(V, 64, 256, 9)
    rng = np.random.Generator(np.random.PCG64(8))
    hid = bf16_bits_from_f32(rng.standard_normal((64, H), dtype=np.float32))
    out = torch.zeros((64, 256), dtype=torch.float32, device="cuda")
    hd = to_dev(hid)
    n = torch.full((64,), 256, dtype=torch.int32, device="cuda")
    for si in (0, 8):
        tms.gather_gemv(emb, hd, to_dev(np.ascontiguousarray(sets[si])), n, out)
        o = out.cpu().numpy()
        for _ in range(300):
            b, j = int(rng.integers(0, 64)), int(rng.integers(0, 256))
            want, sa = oracle.logit(emb_np, int(sets[si, b, j]), hid[b])
            assert abs(float(o[b, j]) - want) <= 2e-3 * abs(want) + gamma(H + 1) * sa


# ---------------------------------------------------------------------------
# Resident-loop variants: register-held path/entry lists and their memory
# fallbacks, live counts in LDS or in device memory
# ---------------------------------------------------------------------------

def _loop_forms_agree(cat, V, k, B, H, path, seed, where):
    rng = np.random.Generator(np.random.PCG64(seed))
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "bf16")
    hid = _rand_hidden(rng, T, B, H, "bf16")
    trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    tok_r, len_r, ent_r = run_k_pointers(st, hd)
    ex_r = st.export(live=True)
    compare(tok_r, ref_decode(otr, k, emb, hid), H, None, len_r, ent_r, where=where)
    tms.state_set_loop(st.h, tms.LOOP_GRAPH)
    st.reset()
    tok_g, len_g, ent_g = run_k_pointers(st, hd)
    ex_g = st.export(live=True)
    assert np.array_equal(tok_r, tok_g) and np.array_equal(len_r, len_g) and np.array_equal(ent_r, ent_g)
    for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
        assert np.array_equal(ex_r[key], ex_g[key]), (where, key)
    return trie.info


def test_loop_deep_entries():
    """Entries longer than a wavefront (path kept in device memory)."""
    rng = np.random.Generator(np.random.PCG64(40))
    cat = [[int(x) for x in rng.integers(0, 100, size=int(rng.integers(60, 81)))] for _ in range(20)]
    info = _loop_forms_agree(cat, 600, 3, 3, 256, tms.PATH_AUTO, 1, "deep")
    assert info["max_depth"] > 64


def test_loop_many_pointers():
    """k above a wavefront (completed entries kept in device memory)."""
    cat = random_catalog(41, 100, 3, 300)
    _loop_forms_agree(cat, 600, 70, 3, 256, tms.PATH_AUTO, 2, "many_k")


def test_loop_fast_store_live_in_memory():
    """A fast-path trie whose live counts do not fit LDS."""
    cat = random_catalog(42, 3000, 6, 200, min_len=3)
    info = _loop_forms_agree(cat, 1024, 4, 5, 512, tms.PATH_FAST, 3, "fast_global_live")
    assert info["path"] == tms.PATH_FAST and info["n_edges"] * 4 > 65536


@pytest.mark.parametrize("cat,k", [([[7]], 1), ([list(range(3, 73))], 1), ([[4, 5], [4]], 2), ([[4], [4, 5]], 1),
                                   ([[9, 1], [9, 2], [8], [9, 1, 3], [2]], 5)])
def test_loop_degenerate_catalogs(cat, k):
    """Degenerate catalogs through the resident loop: one entry (every step
    forced, one of them a run of more than 64 tokens), an entry that is a
    prefix of the other (its terminal is not a leaf), and k equal to the
    catalog size (the last pointer has one entry left).  Tokens, lengths,
    entries and final state against the oracle and the per-step form."""
    V, H, B = 128, 256, 3
    rng = np.random.Generator(np.random.PCG64(70 + len(cat) + k))
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "bf16")
    hid = _rand_hidden(rng, T, B, H, "bf16")
    ref = ref_decode(otr, k, emb, hid)
    for path in (tms.PATH_FAST, tms.PATH_GLOBAL):
        trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
        st = tms.State(trie, B, k, to_dev(emb))
        hd = to_dev(hid)
        tok, ln, ent = run_k_pointers(st, hd)
        compare(tok, ref, H, None, ln, ent, where=f"degenerate {cat} k={k} path={path}")
        ex = st.export(live=True)
        tms.state_set_loop(st.h, tms.LOOP_STREAM)
        st.reset()
        tok2, ln2, ent2 = run_k_pointers(st, hd)
        assert np.array_equal(tok, tok2) and np.array_equal(ln, ln2) and np.array_equal(ent, ent2)
        ex2 = st.export(live=True)
        for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
            assert np.array_equal(ex[key], ex2[key]), (cat, k, path, key)
        st.close()
        trie.close()


def test_random_sweep_repeated_decodes():
    """Seeded random catalogs (sizes, depths, id ranges, hidden sizes, batch
    sizes, k, both stores, every resident loop form): three decodes on one
    state with resets between (the later ones restore only released paths),
    each against the oracle and with identical exported state, then the
    per-step form."""
    rng = np.random.Generator(np.random.PCG64(12345))
    n = 0
    while n < 48:
        seed = int(rng.integers(1 << 30))
        K, maxlen, idhi = int(rng.choice([3, 20, 150, 900])), int(rng.choice([3, 6, 12, 40, 80])), \
            int(rng.choice([6, 30, 300, 2000]))
        V = (max(idhi + 2, 64) + 7) // 8 * 8
        try:
            cat = random_catalog(seed, K, maxlen, idhi)
        except ValueError:
            continue  # not that many distinct strings in this id range
        H, B = int(rng.choice([64, 256])), int(rng.choice([1, 3, 8, 17]))
        k = int(rng.integers(1, min(len(cat), 6) + 1))
        path = int(rng.choice([tms.PATH_AUTO, tms.PATH_GLOBAL]))
        mode = int(rng.choice([tms.LOOP_RESIDENT, tms.LOOP_RESIDENT_SOLO, tms.LOOP_RESIDENT_GROUPED]))
        otr = oracle.Trie(cat, V, V - 2, V - 1)
        T = k * (otr.max_depth + 1)
        r2 = np.random.Generator(np.random.PCG64(seed + 1))
        emb, hid = _rand_table(r2, V, H, "bf16"), _rand_hidden(r2, T, B, H, "bf16")
        ref = ref_decode(otr, k, emb, hid)
        trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
        st = tms.State(trie, B, k, to_dev(emb))
        tms.state_set_loop(st.h, mode)
        hd = to_dev(hid)
        where = f"seed={seed} K={K} maxlen={maxlen} idhi={idhi} H={H} B={B} k={k} path={path} mode={mode}"
        first = None
        for rep in range(3):
            st.reset()
            tok, ln, ent = run_k_pointers(st, hd)
            compare(tok, ref, H, None, ln, ent, where=f"{where} rep={rep}")
            ex = st.export(live=True)
            first = first or ex
            for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
                assert np.array_equal(ex[key], first[key]), (where, rep, key)
        tms.state_set_loop(st.h, tms.LOOP_STREAM)
        st.reset()
        tok2, ln2, ent2 = run_k_pointers(st, hd)
        assert np.array_equal(tok, tok2) and np.array_equal(ln, ln2) and np.array_equal(ent, ent2), where
        st.close()
        trie.close()
        n += 1


def test_dense_odd_vocab_sweep():
    """The matrix-core dense head (H = 2048, B in 2..64) on vocabularies that
    are not a multiple of its 128-row blocks (a partial last block), seeded
    random catalogs: tokens against the oracle with the any-order tie bound,
    full logits sampled against the oracle's."""
    rng = np.random.Generator(np.random.PCG64(777))
    H = 2048
    for _ in range(12):
        seed = int(rng.integers(1 << 30))
        V = int(rng.integers(66, 3000))
        cat = random_catalog(seed, int(rng.integers(3, 60)), 6, V - 2)
        B = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(len(cat), 4) + 1))
        otr = oracle.Trie(cat, V, V - 2, V - 1)
        T = k * (otr.max_depth + 1)
        r2 = np.random.Generator(np.random.PCG64(seed + 1))
        emb, hid = _rand_table(r2, V, H, "bf16"), _rand_hidden(r2, T, B, H, "bf16")
        ref = ref_decode(otr, k, emb, hid)
        trie = tms.Trie(cat, V, V - 2, V - 1)
        st = tms.State(trie, B, k, to_dev(emb))
        full = torch.zeros((T, B, V), dtype=torch.float32, device="cuda")
        where = f"seed={seed} V={V} B={B} k={k}"
        tok, lg = run_step_loop(st, to_dev(hid), dense=True, full=full)
        flips = compare(tok, ref, H, lg, where=where, depth=H + 1, max_flips=2)
        print(where, f"tie flips={flips}", flush=True)
        fl = full.cpu().numpy()
        for b in (0, B - 1):
            for v in r2.choice(V, 64, replace=False):
                want, sa = oracle.logit(emb, int(v), hid[0, b])
                assert abs(float(fl[0, b, v]) - want) <= 2e-3 * abs(want) + gamma(H + 1) * sa, (where, b, v)
        st.close()
        trie.close()


def test_dense_wide_batch_sweep():
    """The matrix-core dense head for 64 < B <= 256 (H a multiple of 256):
    batches that leave the last member tile partly empty (its lanes read a copy
    of the last member and are dropped), both member-tile counts (8 and 16),
    several hidden sizes and vocabularies that end inside a 128-row workgroup
    block; seeded random catalogs.  Tokens against the oracle with the any-order
    tie bound, full logits of the first and last sequence sampled against the
    oracle's."""
    rng = np.random.Generator(np.random.PCG64(4242))
    for case in range(8):
        seed = int(rng.integers(1 << 30))
        H = int(rng.choice([256, 512, 1024, 2048]))
        B = int(rng.integers(65, 257)) if case else 255
        V = int(rng.integers(66, 3000))
        cat = random_catalog(seed, int(rng.integers(3, 60)), 6, V - 2)
        k = int(rng.integers(1, min(len(cat), 3) + 1))
        otr = oracle.Trie(cat, V, V - 2, V - 1)
        T = k * (otr.max_depth + 1)
        r2 = np.random.Generator(np.random.PCG64(seed + 1))
        emb, hid = _rand_table(r2, V, H, "bf16"), _rand_hidden(r2, T, B, H, "bf16")
        ref = ref_decode(otr, k, emb, hid)
        trie = tms.Trie(cat, V, V - 2, V - 1)
        st = tms.State(trie, B, k, to_dev(emb))
        full = torch.zeros((T, B, V), dtype=torch.float32, device="cuda")
        where = f"seed={seed} V={V} B={B} H={H} k={k}"
        print(where, flush=True)
        tok, lg = run_step_loop(st, to_dev(hid), dense=True, full=full)
        flips = compare(tok, ref, H, lg, where=where, depth=H + 1, max_flips=2)
        print(where, f"tie flips={flips}", flush=True)
        fl = full.cpu().numpy()
        for b in (0, B - 1):
            for v in r2.choice(V, 64, replace=False):
                want, sa = oracle.logit(emb, int(v), hid[0, b])
                assert abs(float(fl[0, b, v]) - want) <= 2e-3 * abs(want) + gamma(H + 1) * sa, (where, b, v)
        st.close()
        trie.close()


def test_dense_large_batch_other_hidden_sizes():
    """The matrix-core dense head for 64 < B <= 256 when H is not a multiple of
    256: H % 128 == 0 (the K-streamed kernel) and H % 128 != 0 (the per-block
    kernel), with partial member tiles and ragged vocabularies; tokens against
    the oracle with the any-order tie bound, sampled full logits against the
    oracle's."""
    rng = np.random.Generator(np.random.PCG64(5151))
    for H in (96, 160, 384, 640, 96, 384):
        seed = int(rng.integers(1 << 30))
        B = int(rng.integers(65, 257))
        V = int(rng.integers(66, 2500))
        cat = random_catalog(seed, int(rng.integers(3, 50)), 6, V - 2)
        k = int(rng.integers(1, min(len(cat), 3) + 1))
        otr = oracle.Trie(cat, V, V - 2, V - 1)
        T = k * (otr.max_depth + 1)
        r2 = np.random.Generator(np.random.PCG64(seed + 1))
        emb, hid = _rand_table(r2, V, H, "bf16"), _rand_hidden(r2, T, B, H, "bf16")
        ref = ref_decode(otr, k, emb, hid)
        trie = tms.Trie(cat, V, V - 2, V - 1)
        st = tms.State(trie, B, k, to_dev(emb))
        full = torch.zeros((T, B, V), dtype=torch.float32, device="cuda")
        where = f"seed={seed} V={V} B={B} H={H} k={k}"
        print(where, flush=True)
        tok, lg = run_step_loop(st, to_dev(hid), dense=True, full=full)
        flips = compare(tok, ref, H, lg, where=where, depth=H + 1, max_flips=2)
        print(where, f"tie flips={flips}", flush=True)
        fl = full.cpu().numpy()
        for b in (0, B - 1):
            for v in r2.choice(V, 64, replace=False):
                want, sa = oracle.logit(emb, int(v), hid[0, b])
                assert abs(float(fl[0, b, v]) - want) <= 2e-3 * abs(want) + gamma(H + 1) * sa, (where, b, v)
        st.close()
        trie.close()


def test_bf16_pair_product_rounding():
    """How one v_dot2_f32_bf16 rounds (an in-bounds check through the sparse
    head with H = 8, where lane 0 holds the whole row): 1.0 from the first
    pair, then products 2^-24 and 2^-25 from the second pair.  A single
    rounding of the pair sum (or of the exact three-term sum) gives 1 + 2^-23;
    adding the products to the running sum one at a time gives 1.0.  Either way
    a pair costs at most two roundings, the assumption behind the tie bound."""
    from synth import bf16_bits_from_f32
    h = np.zeros((1, 8), np.float32)
    e = np.zeros((2, 8), np.float32)
    h[0, :4] = [1.0, 0.0, 2.0 ** -12, 2.0 ** -13]
    e[0, :4] = [1.0, 0.0, 2.0 ** -12, 2.0 ** -12]
    hb, eb = bf16_bits_from_f32(h), bf16_bits_from_f32(e)
    out = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    tms.gather_gemv(to_dev(eb), to_dev(hb), torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"),
                    torch.tensor([1], dtype=torch.int32, device="cuda"), out)
    got = float(out[0, 0])
    assert got in (1.0 + 2.0 ** -23, 1.0), got
    print("v_dot2_f32_bf16 pair:", "single rounding" if got != 1.0 else "sequential")


def _chain_catalog(seed, n, V):
    """Entries with long single-child runs and a few branch points: most steps
    have one legal token, so the resident loop's forced steps dominate."""
    rng = np.random.Generator(np.random.PCG64(seed))
    stems = [[int(x) for x in rng.integers(0, V - 2, size=int(rng.integers(20, 70)))] for _ in range(4)]
    cat = []
    while len(cat) < n:
        st = stems[int(rng.integers(0, len(stems)))]
        cut = int(rng.integers(1, len(st)))
        tail = [int(x) for x in rng.integers(0, V - 2, size=int(rng.integers(1, 30)))]
        e = st[:cut] + tail
        if e not in cat:
            cat.append(e)
    return cat


@pytest.mark.parametrize("path", [tms.PATH_FAST, tms.PATH_GLOBAL])
def test_loop_forced_spans_from_mid_answer(path):
    """The resident loop skips the head on steps with one legal token.  Start
    it from states left by `cut` host-driven steps (inside a forced run, at a
    branch, after a completion, past the 64-token flush boundary): tokens and
    final state must match a whole-answer loop, the per-step loop form (which
    always runs the head) and the oracle."""
    V, H, k, B = 700, 256, 3, 4
    cat = _chain_catalog(50 + path, 40, V)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    rng = np.random.Generator(np.random.PCG64(60 + path))
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "bf16")
    hid = _rand_hidden(rng, T, B, H, "bf16")
    ref = ref_decode(otr, k, emb, hid)
    trie = tms.Trie(cat, V, V - 2, V - 1, path=path)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    tok_full, len_full, ent_full = run_k_pointers(st, hd)
    ex_full = st.export(live=True)
    compare(tok_full, ref, H, None, len_full, ent_full, where="forced full")
    n_forced = int((ref["nlegal"] == 1).sum())
    assert n_forced >= 0.6 * int(ref["len"].sum())  # most steps are forced here
    for cut in (1, 5, 37, 63, 64, 65, 100, T - 1):
        if cut >= T:
            continue
        # hidden vectors of the remaining steps, padded to the loop's minimum T
        rest = torch.zeros_like(hd)
        rest[: T - cut] = hd[cut:]
        for mode in (tms.LOOP_RESIDENT, tms.LOOP_STREAM):
            tms.state_set_loop(st.h, mode)
            st.reset()
            a, _ = run_step_loop(st, hd[:cut])
            b_, ln, en = run_k_pointers(st, rest)
            whole = np.concatenate([a, b_[:, : T - cut]], axis=1)
            assert np.array_equal(whole, tok_full), (cut, mode)
            assert (b_[:, T - cut:] == -1).all(), (cut, mode)
            assert np.array_equal(ln, len_full) and np.array_equal(en, ent_full), (cut, mode)
            ex = st.export(live=True)
            for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
                assert np.array_equal(ex[key], ex_full[key]), (cut, mode, key)
    st.close()
    trie.close()


def test_deferred_reset_is_applied_by_every_next_call():
    """tms_state_reset is carried out by the next call on the state: inside
    the resident loop, or as a reset kernel before any other call."""
    c, otr, T, hid = config_case("tiny", B=3)
    trie = tms.Trie(catalog("tiny"), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 3, c.k, dev_embedding("tiny"))
    hd = to_dev(hid)
    fresh = st.export(live=True)
    assert (fresh["node"] == 0).all() and (fresh["entries"] == -1).all()
    tok0, len0, ent0 = run_k_pointers(st, hd)
    for follow in ("export", "step", "loop", "stream", "legal"):
        run_k_pointers(st, hd)  # leave a finished state behind
        st.reset()
        if follow == "export":
            ex = st.export(live=True)
            for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
                assert np.array_equal(ex[key], fresh[key]), (follow, key)
        elif follow == "step":
            tok, _ = run_step_loop(st, hd)
            assert np.array_equal(tok, tok0), follow
        elif follow == "legal":
            n = torch.zeros(3, dtype=torch.int32, device="cuda")
            lt = torch.zeros((3, trie.info["cap"]), dtype=torch.int32, device="cuda")
            tms.legal_set(st.h, lt, n)
            torch.cuda.synchronize()
            root = trie.csr()
            assert (n.cpu().numpy() == root["begin"][1] - root["begin"][0]).all(), follow
        else:
            tms.state_set_loop(st.h, tms.LOOP_RESIDENT if follow == "loop" else tms.LOOP_STREAM)
            tok, ln, ent = run_k_pointers(st, hd)
            assert np.array_equal(tok, tok0) and np.array_equal(ln, len0) and np.array_equal(ent, ent0), follow
            tms.state_set_loop(st.h, tms.LOOP_RESIDENT)
    st.close()
    trie.close()


@pytest.mark.parametrize("mode", ["grouped", "solo", "stream"])
def test_reset_restores_released_paths(mode):
    """A reset after decoding restores only the live counts on the completed
    entries' root paths (all that completions take off); after
    tms_debug_set_live, or on a fresh state, it rewrites whole rows.  Both,
    inside the resident loop and as a reset kernel, leave every sequence's
    state equal to a fresh one's, and a decode after them repeats the first."""
    B = 64
    c, otr, T, hid = config_case("structured", B=B)
    trie = tms.Trie(catalog("structured"), c.vocab, c.sep, c.stop)
    st = tms.State(trie, B, c.k, dev_embedding("structured"))
    tms.state_set_loop(st.h, {"grouped": tms.LOOP_RESIDENT_GROUPED, "solo": tms.LOOP_RESIDENT_SOLO,
                              "stream": tms.LOOP_STREAM}[mode])
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live", "spent")
    fresh = st.export(live=True)
    r0 = run_k_pointers(st, hd)
    ex0 = st.export(live=True)
    assert (ex0["live"] != fresh["live"]).any() and (ex0["done"] == c.k).all()

    def same(a, b, where):
        for key in keys:
            if key in a:
                assert np.array_equal(a[key], b[key]), (mode, where, key)

    st.reset()  # carried out by the next decode
    r1 = run_k_pointers(st, hd)
    for x, y in zip(r0, r1):
        assert np.array_equal(x, y), (mode, "decode after reset")
    same(st.export(live=True), ex0, "state after reset and decode")
    st.reset()  # carried out by the export (reset kernel)
    same(st.export(live=True), fresh, "reset kernel")
    root = trie.csr()
    e = int(root["begin"][0])
    run_k_pointers(st, hd)
    tms.debug_set_live(st.h, 3, e, 0)
    st.reset()
    same(st.export(live=True), fresh, "reset kernel after set_live")
    run_k_pointers(st, hd)
    tms.debug_set_live(st.h, 5, e + 1, 0)
    st.reset()
    r2 = run_k_pointers(st, hd)
    for x, y in zip(r0, r2):
        assert np.array_equal(x, y), (mode, "decode after set_live and reset")
    same(st.export(live=True), ex0, "state after set_live, reset and decode")
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# The fused step with the root grouped across sequences
# ---------------------------------------------------------------------------

def _step_answers(st, hd, mode, loop=None):
    """Host-driven steps (or a loop form) under a root-grouping mode; tokens,
    winner logits and the exported state."""
    tms.state_set_step_grouping(st, mode)
    st.reset()
    if loop is None:
        tok, lg = run_step_loop(st, hd)
    else:
        tms.state_set_loop(st, loop)
        tok, _, _ = run_k_pointers(st, hd)
        lg = None
        tms.state_set_loop(st, tms.LOOP_RESIDENT)
    return tok, lg, st.export(live=True)


@pytest.mark.parametrize("dtype,H,B", [("bf16", 2048, 64), ("fp32", 256, 37), ("bf16", 8192, 20), ("bf16", 520, 200),
                                       ("fp32", 4096, 9)])
def test_step_root_grouping_bit_identical(dtype, H, B):
    """The grouped step (root rows read once per tile of members) against the
    per-sequence step: identical tokens, bit-identical winner logits and
    identical state after every answer, host-driven and in the graph of step
    kernels; tokens against the oracle.  Batches that leave the last member
    tile partly filled, hidden sizes that need 1 to 16 chunks per lane."""
    rng = np.random.Generator(np.random.PCG64(H * 3 + B))
    V, k = 2000, 3
    cat = random_catalog(700 + H + B, 400, 5, V - 2, min_len=2)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    b = otr.csr()["begin"]
    assert b[1] - b[0] >= 64
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, dtype)
    hid = _rand_hidden(rng, T, B, H, dtype)
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    t0, l0, x0 = _step_answers(st, hd, tms.STEP_GROUP_OFF)
    t1, l1, x1 = _step_answers(st, hd, tms.STEP_GROUP_ROOT)
    assert np.array_equal(t0, t1) and np.array_equal(l0, l1, equal_nan=True)
    for key in keys:
        assert np.array_equal(x0[key], x1[key]), key
    t2, _, x2 = _step_answers(st, hd, tms.STEP_GROUP_ROOT, loop=tms.LOOP_GRAPH)
    assert np.array_equal(t2, t0)
    for key in keys:
        assert np.array_equal(x2[key], x0[key]), key
    # every shared node grouped, host-driven and in the graph
    t3, l3, x3 = _step_answers(st, hd, tms.STEP_GROUP_NODES)
    assert np.array_equal(t0, t3) and np.array_equal(l0, l3, equal_nan=True)
    for key in keys:
        assert np.array_equal(x0[key], x3[key]), key
    t4, _, x4 = _step_answers(st, hd, tms.STEP_GROUP_NODES, loop=tms.LOOP_GRAPH)
    assert np.array_equal(t4, t0)
    for key in keys:
        assert np.array_equal(x4[key], x0[key]), key
    compare(t1, ref_decode(otr, k, emb, hid), H, l1, where=f"grouped step {dtype} H={H} B={B}")
    split, grid = tms.state_get_launch(st)
    assert grid > B * split  # the root workgroups are part of the grid
    st.close()
    trie.close()


@pytest.mark.parametrize("cid", ["unstructured", "structured"])
def test_step_root_grouping_workloads(cid):
    """The batch-64 workloads through the grouped step, root only and at
    every shared node (forced on for the structured catalog, whose root has 8
    edges): the per-sequence step's tokens and logits bit for bit, and the
    oracle's tokens."""
    c, otr, T, hid = config_case(cid)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, c.batch, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    t0, l0, x0 = _step_answers(st, hd, tms.STEP_GROUP_OFF)
    for mode in (tms.STEP_GROUP_ROOT, tms.STEP_GROUP_NODES):
        t1, l1, x1 = _step_answers(st, hd, mode)
        assert np.array_equal(t0, t1) and np.array_equal(l0, l1, equal_nan=True), mode
        for key in ("node", "done", "status", "n_emitted", "entries", "live"):
            assert np.array_equal(x0[key], x1[key]), (mode, key)
    compare(t1, ref_decode(otr, c.k, embedding(cid), hid), c.hidden, l1, where=f"{cid}/grouped step")
    st.close()
    trie.close()


def test_step_root_grouping_empty_mask_isolated():
    """An empty root mask for one member under the grouped step: that sequence
    alone gets EMPTY_MASK, the others decode as without it."""
    rng = np.random.Generator(np.random.PCG64(99))
    V, H, B, k = 1500, 256, 12, 2
    cat = random_catalog(4242, 300, 4, V - 2, min_len=2)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "fp32")
    hid = _rand_hidden(rng, T, B, H, "fp32")
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    tms.state_set_step_grouping(st, tms.STEP_GROUP_ROOT)
    csr = trie.csr()
    st.reset()
    st.export()
    for e in range(csr["begin"][0], csr["begin"][1]):
        tms.debug_set_live(st, 5, e, 0)
    tok, lg = run_step_loop(st, to_dev(hid), check=False)
    status = st.status()
    assert status[5] == tms.ERR_EMPTY_MASK and (np.delete(status, 5) == 0).all()
    assert (tok[5] == -1).all()
    keep = [i for i in range(B) if i != 5]
    compare(tok[keep], ref_decode(otr, k, emb, np.ascontiguousarray(hid[:, keep])), H, lg[keep],
            where="grouped step isolated")
    st.close()
    trie.close()


def _two_prefix_catalog(seed, K, max_len, V, prefixes):
    """Entries that all start with one of a few tokens, so that after the
    first step whole blocks of sequences stand at the same node."""
    rest = random_catalog(seed, K, max_len, V - 2 - len(prefixes), min_len=1)
    return [[prefixes[i % len(prefixes)]] + [x + len(prefixes) for x in r] for i, r in enumerate(rest)]


@pytest.mark.parametrize("split", [1, 3])
def test_step_node_grouping_large_groups(split):
    """Groups of more than 64 sequences at one node (150 sequences over a root
    of two edges, whose children have about 60 edges each: many member tiles,
    each over several row tiles whose keys meet in device memory, and below
    them nodes of one row tile), with one and three workgroups per sequence:
    the per-sequence step's tokens, logits and state bit for bit, host-driven,
    in the graph and in the stream of step launches; tokens against the
    oracle."""
    rng = np.random.Generator(np.random.PCG64(515 + split))
    V, H, B, k = 3000, 128, 150, 2
    cat = _two_prefix_catalog(516, 120, 5, V, [0, 1])
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    assert otr.csr()["begin"][1] - otr.csr()["begin"][0] == 2
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "fp32")
    hid = _rand_hidden(rng, T, B, H, "fp32")
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    tms.state_set_split(st, split)
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    t0, l0, x0 = _step_answers(st, hd, tms.STEP_GROUP_OFF)
    t1, l1, x1 = _step_answers(st, hd, tms.STEP_GROUP_NODES)
    assert np.array_equal(t0, t1) and np.array_equal(l0, l1, equal_nan=True)
    for key in keys:
        assert np.array_equal(x0[key], x1[key]), key
    for loop in (tms.LOOP_GRAPH, tms.LOOP_STREAM):
        t2, _, x2 = _step_answers(st, hd, tms.STEP_GROUP_NODES, loop=loop)
        assert np.array_equal(t2, t0), loop
        for key in keys:
            assert np.array_equal(x2[key], x0[key]), (loop, key)
    compare(t1, ref_decode(otr, k, emb, hid), H, l1, where=f"node groups > 64, split {split}")
    st.close()
    trie.close()


def test_step_node_grouping_empty_mask_isolated():
    """Every sequence at the root's only child after the first step; one of
    them has every edge there emptied: under node grouping that sequence alone
    gets EMPTY_MASK at its second step, the others decode as without it."""
    rng = np.random.Generator(np.random.PCG64(77))
    V, H, B, k = 1500, 256, 12, 2
    cat = _two_prefix_catalog(4343, 200, 4, V, [0])
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    csr = otr.csr()
    assert csr["begin"][1] - csr["begin"][0] == 1
    c1 = int(csr["child"][csr["begin"][0]])
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, "fp32")
    hid = _rand_hidden(rng, T, B, H, "fp32")
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    tms.state_set_step_grouping(st, tms.STEP_GROUP_NODES)
    st.reset()
    st.export()
    for e in range(int(csr["begin"][c1]), int(csr["begin"][c1 + 1])):
        tms.debug_set_live(st, 5, e, 0)
    tok, lg = run_step_loop(st, to_dev(hid), check=False)
    status = st.status()
    assert status[5] == tms.ERR_EMPTY_MASK and (np.delete(status, 5) == 0).all()
    assert tok[5, 0] == cat[0][0] and (tok[5, 1:] == -1).all()
    keep = [i for i in range(B) if i != 5]
    compare(tok[keep], ref_decode(otr, k, emb, np.ascontiguousarray(hid[:, keep])), H, lg[keep],
            where="node-grouped step isolated")
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# Root steps grouped across sequences (one phase per pointer)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,B", [("tiny", 5), ("structured", 64), ("unstructured", 64)])
def test_grouped_root_matches_solo_and_oracle(cid, B):
    """The grouped root head reads each root row once for all sequences at the
    root.  fp32 tables (vector units, the per-row order of the other kernels)
    give answers and final states bit-identical to the one-workgroup-per-
    sequence loop; bf16 tables with H = 2048 go through the matrix cores, so
    tokens are held to the oracle with the any-order tie bound (depth H + 1)
    and must equal the solo loop's wherever neither run has a tie-explained
    flip.  From a reset state (k phases) and from mid-answer states (k + 1)."""
    c, otr, T, hid = config_case(cid, B=B)
    mfma = c.dtype == "bf16" and c.hidden in (2048, 4096)
    depth = c.hidden + 1 if mfma else None
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, B, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    ref = ref_decode(otr, c.k, embedding(cid), hid)
    out = {}
    for mode in (tms.LOOP_RESIDENT_SOLO, tms.LOOP_RESIDENT_GROUPED, tms.LOOP_RESIDENT_GROUPED):
        tms.state_set_loop(st.h, mode)
        st.reset()
        r = run_k_pointers(st, hd)
        ex = st.export(live=True)
        if mode in out:  # a second grouped call: nothing left behind by the first
            assert all(np.array_equal(a, b) for a, b in zip(r, out[mode][0]))
        out[mode] = (r, ex)
    (ts, ls, es), exs = out[tms.LOOP_RESIDENT_SOLO]
    (tg, lg, eg), exg = out[tms.LOOP_RESIDENT_GROUPED]
    fs = compare(ts, ref, c.hidden, None, ls, es, where=cid + "/solo")
    fg = compare(tg, ref, c.hidden, None, lg, eg, where=cid + "/grouped", depth=depth)
    if not fs and not fg:
        assert np.array_equal(tg, ts) and np.array_equal(lg, ls) and np.array_equal(eg, es), cid
        for key in keys:
            assert np.array_equal(exg[key], exs[key]), (cid, key)
    # from states left by host-driven steps: some sequences mid-pointer
    for cut in (1, 3, T // 2):
        rest = torch.zeros_like(hd)
        rest[: T - cut] = hd[cut:]
        res = {}
        for mode in (tms.LOOP_RESIDENT_SOLO, tms.LOOP_RESIDENT_GROUPED):
            tms.state_set_loop(st.h, mode)
            st.reset()
            a, _ = run_step_loop(st, hd[:cut])
            b_, ln, en = run_k_pointers(st, rest)
            whole = np.concatenate([a, b_[:, : T - cut]], axis=1)
            flips = compare(whole, ref, c.hidden, None, ln, en, where=f"{cid}/cut{cut}/{mode}",
                            depth=depth if mode == tms.LOOP_RESIDENT_GROUPED else None)
            res[mode] = (whole, ln, en, st.export(live=True), flips)
        s_, g_ = res[tms.LOOP_RESIDENT_SOLO], res[tms.LOOP_RESIDENT_GROUPED]
        assert (b_[:, T - cut:] == -1).all()
        if not s_[4] and not g_[4]:
            assert np.array_equal(g_[0], s_[0]) and np.array_equal(g_[1], s_[1]) and np.array_equal(g_[2], s_[2])
            for key in keys:
                assert np.array_equal(g_[3][key], s_[3][key]), (cid, cut, key)
    st.close()
    trie.close()


def test_grouped_root_empty_mask_is_per_sequence():
    c, otr, T, hid = config_case("tiny", B=3)
    trie = tms.Trie(catalog("tiny"), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 3, c.k, dev_embedding("tiny"))
    tms.state_set_loop(st.h, tms.LOOP_RESIDENT_GROUPED)
    csr = trie.csr()
    st.reset()
    st.export()  # carries out the reset, so the live counts below stick
    for e in range(csr["begin"][0], csr["begin"][1]):
        tms.debug_set_live(st.h, 1, e, 0)
    tok, ln, ent = run_k_pointers(st, to_dev(hid), check=False)
    assert list(st.status()) == [0, tms.ERR_EMPTY_MASK, 0]
    assert (tok[1] == -1).all()
    ref = ref_decode(otr, c.k, embedding("tiny"), hid[:, [0, 2], :])
    compare(tok[[0, 2]], ref, c.hidden, None, ln[[0, 2]], ent[[0, 2]], where="grouped isolated")
    st.close()
    trie.close()


@pytest.mark.parametrize("cid", ["tiny", "product", "product_deep"])
def test_bitmask_state_matches_live_counts(cid):
    """Catalogs of at most 128 entries run the resident loop on the bitmask
    no-repeat state (an edge is live iff one of the entries below it is not
    spent).  Tokens, lengths, entries and the exported state (live counts
    rewritten from the masks) are bit-identical to the live-count loop and to
    the per-step kernel, from a reset state and from mid-answer states."""
    c, otr, T, hid = config_case(cid, B=4)
    assert len(catalog(cid)) <= 128
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, 4, c.k, dev_embedding(cid))
    hd = to_dev(hid)
    keys = ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live")
    for cut in (0, 1, 4, T // 2):
        rest = torch.zeros_like(hd)
        rest[: T - cut] = hd[cut:]
        res = []
        for mode, kind in ((tms.LOOP_RESIDENT_SOLO, tms.NOREPEAT_BITMASK), (tms.LOOP_RESIDENT_SOLO, tms.NOREPEAT_LIVE),
                           (tms.LOOP_STREAM, tms.NOREPEAT_LIVE)):
            tms.state_set_norepeat(st, kind)
            tms.state_set_loop(st.h, mode)
            st.reset()
            a, _ = run_step_loop(st, hd[:cut]) if cut else (np.zeros((4, 0), np.int32), None)
            b_, ln, en = run_k_pointers(st, rest)
            res.append((np.concatenate([a, b_[:, : T - cut]], axis=1), ln, en, st.export(live=True)))
        for other in res[1:]:
            assert np.array_equal(res[0][0], other[0]) and np.array_equal(res[0][1], other[1])
            assert np.array_equal(res[0][2], other[2])
            for key in keys:
                assert np.array_equal(res[0][3][key], other[3][key]), (cid, cut, key)
        if cut == 0:
            compare(res[0][0], ref_decode(otr, c.k, embedding(cid), hid), c.hidden, None, res[0][1], res[0][2],
                    where=cid + "/mask")
    st.close()
    trie.close()


# ---------------------------------------------------------------------------
# Bitmask-fed materialiser: vocabulary mask -> sorted rows -> head
# ---------------------------------------------------------------------------

def test_mask_to_rows_random_masks():
    """Popcount scan against numpy: ascending ids of the set bits, bits at or
    past V ignored, truncation at cap with the full count reported."""
    rng = np.random.Generator(np.random.PCG64(70))
    for V, B, dens in ((1000, 5, 0.05), (4096, 3, 0.5), (151936, 4, 0.003), (33, 2, 0.9), (1, 1, 1.0)):
        W = (V + 31) // 32
        bits = rng.random((B, W * 32)) < dens
        words = np.packbits(bits.reshape(B, W, 32)[:, :, ::-1], axis=-1, bitorder="big").view(">u4")
        mask = words.reshape(B, W).astype(np.uint32).view(np.int32)
        want = [np.flatnonzero(bits[s, :V]) for s in range(B)]
        for cap in (max(1, max(len(w) for w in want)), 3):
            rows = torch.full((B, cap), -5, dtype=torch.int32, device="cuda")
            n = torch.full((B,), -5, dtype=torch.int32, device="cuda")
            tms.mask_to_rows(to_dev(np.ascontiguousarray(mask)), V, rows, n)
            torch.cuda.synchronize()
            r, nn = rows.cpu().numpy(), n.cpu().numpy()
            for s in range(B):
                assert nn[s] == len(want[s]), (V, s)
                m = min(cap, len(want[s]))
                assert np.array_equal(r[s, :m], want[s][:m]), (V, s, cap)
                assert (r[s, m:] == -5).all()


@pytest.mark.parametrize("cid,B", [("tiny", 3), ("structured", 8)])
def test_mask_fed_head_matches_sparse_step(cid, B):
    """Along each answer: the legal mask has exactly the oracle's legal tokens;
    the materialised rows equal the library's legal set; the head over those
    rows (the same per-row arithmetic) picks the sparse step's token with a
    bit-identical logit."""
    c, otr, T, hid = config_case(cid, B=B)
    trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
    st = tms.State(trie, B, c.k, dev_embedding(cid))
    emb = dev_embedding(cid)
    W = (c.vocab + 31) // 32
    cap = trie.info["cap"]
    mask = torch.empty((B, W), dtype=torch.int32, device="cuda")
    rows = torch.empty((B, cap), dtype=torch.int32, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    lt = torch.empty((B, cap), dtype=torch.int32, device="cuda")
    ln = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, cap), dtype=torch.float32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    lg = torch.empty(B, dtype=torch.float32, device="cuda")
    ostates = [oracle.State(otr, c.k) for _ in range(B)]
    st.reset()
    for t in range(T):
        hd = to_dev(np.ascontiguousarray(hid[t]))
        tms.legal_mask(st.h, mask)
        tms.legal_set(st.h, lt, ln)
        tms.mask_to_rows(mask, c.vocab, rows, n)
        tms.gather_gemv(emb, hd, rows, n, out)
        tms.decode_step_sparse(st.h, hd, tok, lg)
        torch.cuda.synchronize()
        m = mask.cpu().numpy().view(np.uint32)
        r, nn, ltn, lnn = rows.cpu().numpy(), n.cpu().numpy(), lt.cpu().numpy(), ln.cpu().numpy()
        o, tk, lgv = out.cpu().numpy(), tok.cpu().numpy(), lg.cpu().numpy()
        for s in range(B):
            ol = ostates[s].legal()
            legal = [] if ol is None else sorted(int(x) for x in ol[0])
            bits = np.flatnonzero(np.unpackbits(m[s].view(np.uint8), bitorder="little"))
            assert list(bits) == legal, (cid, t, s)
            if lnn[s] < 0:  # finished or in error
                assert nn[s] == 0 and tk[s] == -1
                continue
            assert nn[s] == lnn[s] and list(r[s, : nn[s]]) == list(ltn[s, : lnn[s]]) == legal, (cid, t, s)
            j = int(np.argmax(o[s, : nn[s]]))  # first maximum: the lowest token id among ties
            assert r[s, j] == tk[s] and o[s, j] == lgv[s], (cid, t, s)
            ostates[s].advance(int(tk[s]))
    st.close()
    trie.close()


@pytest.mark.parametrize("dtype,H", [("bf16", 4096), ("bf16", 1024), ("fp32", 512), ("bf16", 2048)])
def test_grouped_root_random_tables(dtype, H):
    """Grouped root heads on catalogs with a wide root: the matrix-core head
    for bf16 with H = 2048 or 4096 (16 and 32 steps per quarter), the vector
    head otherwise; B = 24 gives a full and a partial member tile.  Checked
    against the oracle (tie depth H + 1 for the matrix cores) and against the
    per-sequence loop (bit-identical for the vector head)."""
    rng = np.random.Generator(np.random.PCG64(80 + H))
    V, B, k = 2000, 24, 3
    cat = random_catalog(90 + H, 400, 5, V - 2, min_len=2)
    otr = oracle.Trie(cat, V, V - 2, V - 1)
    b = otr.csr()["begin"]
    assert b[1] - b[0] >= 64  # a wide root
    T = k * (otr.max_depth + 1)
    emb = _rand_table(rng, V, H, dtype)
    hid = _rand_hidden(rng, T, B, H, dtype)
    ref = ref_decode(otr, k, emb, hid)
    mfma = dtype == "bf16" and H in (2048, 4096)
    trie = tms.Trie(cat, V, V - 2, V - 1)
    st = tms.State(trie, B, k, to_dev(emb))
    hd = to_dev(hid)
    out = {}
    for mode in (tms.LOOP_RESIDENT_GROUPED, tms.LOOP_RESIDENT_SOLO):
        tms.state_set_loop(st.h, mode)
        st.reset()
        out[mode] = run_k_pointers(st, hd) + (st.export(live=True),)
    tg, lg, eg, exg = out[tms.LOOP_RESIDENT_GROUPED]
    ts, ls, es, exs = out[tms.LOOP_RESIDENT_SOLO]
    fg = compare(tg, ref, H, None, lg, eg, where=f"grouped {dtype} H={H}", depth=H + 1 if mfma else None)
    fs = compare(ts, ref, H, None, ls, es, where=f"solo {dtype} H={H}")
    if not mfma or (not fg and not fs):
        assert np.array_equal(tg, ts) and np.array_equal(eg, es)
        for key in ("node", "depth", "done", "status", "finished", "n_emitted", "entries", "live"):
            assert np.array_equal(exg[key], exs[key]), key
    st.close()
    trie.close()
