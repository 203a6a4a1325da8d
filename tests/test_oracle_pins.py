"""Pins of the CPU oracle against things other than itself.

The oracle (oracle/tms_oracle.c) is trusted only because of these checks:
  * the next-token mask it computes equals Mask(u) = {v : exists w, u v w in L}
    obtained by enumerating the answer language L_k(C) outright (the mask
    definition of "Constrained decoding with weighted automata", applied to
    the exactly-k / no-repeat language of "Constraint made cheaper than no
    constraint", section "Masked sampling inside the sampler");
  * closed forms of the trie (node count = distinct prefixes + 1, breadth-first
    numbering, live counts = entries below an edge);
  * a hand-derived worked example (tests/golden/prefix_pairs.json);
  * logits against the exact dot product (math.fsum of exact products) within
    the fp64 summation bound, and special inputs whose logits are known exactly
    (zero hidden state, one-hot rows);
  * decodes that reduce to textbook results (top-k of a flat catalog via
    numpy.lexsort, lexicographic minimum of L_k(C) for a zero hidden state,
    a permutation of the catalog when k = K);
  * the per-step statistics the GPU comparison relies on (winner, top-two
    margin, the larger sum|p| of the top two) against a recomputation from
    exact dot products (math.fsum) over the legal set;
  * teacher forcing: along random answers drawn from L_k(C) itself, the
    oracle's pick at every step is the first maximum of the exact logits over
    Mask(u), and an illegal forced token is refused;
  * negative controls: each planted oracle mistake must fail at least one pin.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import CONFIGS, bf16_bits_from_f32, bf16_bits_to_f32, catalog, random_catalog

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, scope="module")
def _built(oracle_lib):
    oracle.set_mutant(0)
    yield
    oracle.set_mutant(0)


# ----------------------------------------------------------------------------
# Independent helpers written from the definitions (no oracle code)
# ----------------------------------------------------------------------------

def language(cat, k, sep, stop):
    """Every string of L_k(C): k distinct entries joined by sep, ended by stop."""
    out = []
    for perm in itertools.permutations(range(len(cat)), k):
        s = []
        for i, p in enumerate(perm):
            s.extend(cat[p])
            s.append(sep if i < k - 1 else stop)
        out.append(tuple(s))
    return out


def mask_by_definition(L, u):
    n = len(u)
    return sorted({s[n] for s in L if len(s) > n and s[:n] == u})


def force(trie, k, u):
    st = oracle.State(trie, k)
    for t in u:
        rc = st.advance(t)
        if rc != oracle.OK:
            return st, rc
    return st, oracle.OK


def tiny_cases():
    """Random tiny catalogs (K <= 6, lengths <= 4, V = 16) plus hand-made
    prefix-pair catalogs, with both placements of the control ids."""
    cases = [
        ([[1], [1, 2], [1, 2, 3], [4]], 16, 14, 15),
        ([[1], [1, 2]], 16, 14, 15),
        ([[3, 3], [3], [3, 3, 3]], 16, 0, 15),
        ([[5, 6], [5], [7], [5, 6, 7]], 16, 15, 1),
    ]
    for seed in range(36):
        rng = np.random.Generator(np.random.PCG64(seed))
        K = int(rng.integers(1, 7))
        sep, stop = (14, 15) if seed % 3 else (2, 9)
        ids = [v for v in range(16) if v not in (sep, stop)]
        cat = random_catalog(seed, K, 4, len(ids))
        cat = [[ids[t] for t in e] for e in cat]
        cases.append((cat, 16, sep, stop))
    return cases


# ----------------------------------------------------------------------------
# Pins (plain functions so the negative controls can run them under a mutant)
# ----------------------------------------------------------------------------

def pin_mask_brute_force():
    for cat, V, sep, stop in tiny_cases():
        trie = oracle.Trie(cat, V, sep, stop)
        for k in range(1, min(3, len(cat)) + 1):
            L = language(cat, k, sep, stop)
            Lset = set(L)
            prefixes = {s[:i] for s in L for i in range(len(s) + 1)}
            for u in prefixes:
                st, rc = force(trie, k, u)
                assert rc == oracle.OK, (cat, k, u)
                got = st.legal()
                if u in Lset:
                    assert got is None and st.info()["finished"] == 1, (cat, k, u)
                    continue
                want = mask_by_definition(L, u)
                assert got is not None and list(got[0]) == want, (cat, k, u, got, want)
                assert not (sep in want and stop in want)
                # every token outside the mask is refused
                for v in range(V):
                    if v not in want:
                        st2, _ = force(trie, k, u)
                        assert st2.advance(v) == oracle.ERR_NOT_WALKABLE, (cat, k, u, v)


def pin_golden_prefix_pairs():
    g = json.load(open(os.path.join(GOLDEN, "prefix_pairs.json")))
    trie = oracle.Trie(g["catalog"], g["vocab"], g["sep"], g["stop"])
    csr = trie.csr()
    for key in ("begin", "entry", "tok", "child", "live0"):
        assert list(csr[key]) == g["csr"][key], key
    st = oracle.State(trie, g["k"])
    for step in g["zero_hidden_trace"]:
        toks, _ = st.legal()
        assert list(toks) == step["legal"]
        assert st.advance(step["take"]) == oracle.OK
    assert st.info()["finished"] == 1
    assert list(st.entries()) == g["zero_hidden_entries"]
    assert list(st.live()) == g["zero_hidden_live_after"]
    # the same walk through the decoder with a zero hidden state
    emb = np.ones((g["vocab"], 4), np.float32)
    hid = np.zeros((len(g["zero_hidden_trace"]), 1, 4), np.float32)
    out = oracle.decode(trie, g["k"], emb, hid)
    assert list(out["tokens"][0]) == [s["take"] for s in g["zero_hidden_trace"]]
    assert list(out["entries"][0]) == g["zero_hidden_entries"]


def pin_live_counts():
    """live[e] = entries below e that are not emitted yet, along random walks."""
    for ci, (cat, V, sep, stop) in enumerate(tiny_cases()):
        trie = oracle.Trie(cat, V, sep, stop)
        csr = trie.csr()
        # prefix (token path) reaching each node, by walking the CSR from root
        node_path = {0: ()}
        for n in range(trie.n_nodes):
            for e in range(csr["begin"][n], csr["begin"][n + 1]):
                if csr["child"][e] >= 0:
                    node_path[int(csr["child"][e])] = node_path[n] + (int(csr["tok"][e]),)
        k = min(3, len(cat))
        rng = np.random.Generator(np.random.PCG64(100 + ci))
        st = oracle.State(trie, k)
        emitted = []
        while True:
            lg = st.legal()
            if lg is None:
                break
            toks, _ = lg
            t = int(toks[rng.integers(0, len(toks))])
            info = st.info()
            if t in (sep, stop):
                emitted.append(int(csr["entry"][info["node"]]))
            assert st.advance(t) == oracle.OK
            live = st.live()
            for e in range(trie.n_edges):
                c = int(csr["child"][e])
                if c < 0:
                    continue
                pre = node_path[c]
                want = sum(1 for j, ent in enumerate(cat)
                           if tuple(ent[:len(pre)]) == pre and j not in emitted)
                assert live[e] == want, (cat, e)


def pin_trie_closed_forms(cats):
    for cat, V, sep, stop in cats:
        trie = oracle.Trie(cat, V, sep, stop)
        csr = trie.csr()
        prefixes = {tuple(e[:i]) for e in cat for i in range(1, len(e) + 1)}
        assert trie.n_nodes == len(prefixes) + 1
        assert trie.n_edges == len(prefixes) + 2 * len(cat)
        assert trie.max_depth == max(len(e) for e in cat)
        b = csr["begin"]
        assert trie.cap == int(np.max(np.diff(b)))
        # ranges sorted by token; breadth-first numbering: content children in
        # CSR edge order are exactly 1, 2, ..., N-1
        for n in range(trie.n_nodes):
            assert all(np.diff(csr["tok"][b[n]:b[n + 1]]) > 0)
        kids = csr["child"][csr["child"] >= 0]
        assert list(kids) == list(range(1, trie.n_nodes))
        # walking the CSR from the root spells exactly the catalog
        spelled = {}
        stack = [(0, ())]
        while stack:
            n, p = stack.pop()
            if csr["entry"][n] >= 0:
                spelled[int(csr["entry"][n])] = p
            for e in range(b[n], b[n + 1]):
                if csr["child"][e] >= 0:
                    stack.append((int(csr["child"][e]), p + (int(csr["tok"][e]),)))
                else:
                    assert csr["entry"][n] >= 0 and csr["tok"][e] in (sep, stop)
                    assert (csr["child"][e] == -1) == (csr["tok"][e] == sep)
        assert spelled == {i: tuple(e) for i, e in enumerate(cat)}
        # live0 of a content edge = entries whose string passes through it
        counts = {}
        for e in cat:
            for i in range(1, len(e) + 1):
                counts[tuple(e[:i])] = counts.get(tuple(e[:i]), 0) + 1
        node_pre = {0: ()}
        for n in range(trie.n_nodes):
            for e in range(b[n], b[n + 1]):
                c = int(csr["child"][e])
                if c >= 0:
                    node_pre[c] = node_pre[n] + (int(csr["tok"][e]),)
                    assert csr["live0"][e] == counts[node_pre[c]]
                else:
                    assert csr["live0"][e] == 0


def _exact_dot(h, row):
    return math.fsum((h.astype(np.float64) * row.astype(np.float64)).tolist())


def pin_logits_exact():
    rng = np.random.Generator(np.random.PCG64(7))
    u = 2.0 ** -53
    for dt, H in (("f32", 256), ("f32", 37), ("bf16", 2048), ("bf16", 1000)):
        V = 64
        x = rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02)
        h = rng.standard_normal(H, dtype=np.float32)
        if dt == "bf16":
            emb, hh = bf16_bits_from_f32(x), bf16_bits_from_f32(h)
            ef, hf = bf16_bits_to_f32(emb), bf16_bits_to_f32(hh)
        else:
            emb, hh, ef, hf = x, h, x, h
        gamma = (H - 1) * u / (1 - (H - 1) * u)
        dense = oracle.dense_logits(emb, hh)
        for v in range(V):
            exact = _exact_dot(hf, ef[v])
            sabs = math.fsum(np.abs(hf.astype(np.float64) * ef[v].astype(np.float64)).tolist())
            got, a = oracle.logit(emb, v, hh)
            assert abs(got - exact) <= gamma * sabs, (dt, H, v)
            assert dense[v] == got
            assert abs(a - sabs) <= gamma * sabs
    # zero hidden state: every logit is exactly zero
    emb = rng.standard_normal((32, 64), dtype=np.float32)
    assert np.all(oracle.dense_logits(emb, np.zeros(64, np.float32)) == 0.0)
    # one-hot rows E_v = e_pi(v): the logit is h[pi(v)] exactly, in any order
    H = 48
    perm = rng.permutation(H)
    emb = np.zeros((H, H), np.float32)
    emb[np.arange(H), perm] = 1.0
    h = rng.standard_normal(H, dtype=np.float32)
    assert np.array_equal(oracle.dense_logits(emb, h), h[perm].astype(np.float64))


def pin_flat_topk():
    """All entries one token long, one hidden vector for every step: the k
    pointers are the top-k catalog tokens by <h, E_v>, ties to the lower id."""
    rng = np.random.Generator(np.random.PCG64(11))
    V, H, sep, stop = 512, 64, 510, 511
    emb = bf16_bits_from_f32(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    toks = sorted(rng.choice(V - 2, size=40, replace=False).tolist())
    # duplicate rows: two tokens share a row, so their logits tie exactly
    emb = emb.copy()
    emb[toks[5]] = emb[toks[30]]
    emb[toks[9]] = emb[toks[30]]
    h = bf16_bits_from_f32(rng.standard_normal(H, dtype=np.float32))
    ef, hf = bf16_bits_to_f32(emb).astype(np.float64), bf16_bits_to_f32(h).astype(np.float64)
    scores = np.array([ef[t] @ hf for t in toks])
    for k in (1, 3, 8):
        for sign in (1, -1):
            hs = h if sign > 0 else bf16_bits_from_f32(-bf16_bits_to_f32(h))
            sc = scores if sign > 0 else -scores
            order = np.lexsort((np.array(toks), -sc))[:k]
            want = []
            for i, j in enumerate(order):
                want += [toks[j], sep if i < k - 1 else stop]
            trie = oracle.Trie([[t] for t in toks], V, sep, stop)
            hid = np.broadcast_to(hs, (2 * k, 1, H)).copy()
            out = oracle.decode(trie, k, emb, hid)
            assert list(out["tokens"][0]) == want, (k, sign)
    # the tie itself: with h aligned to the shared row, the three tied tokens
    # come out in ascending id order
    hs = emb[toks[30]].copy()
    trie = oracle.Trie([[t] for t in toks], V, sep, stop)
    hid = np.broadcast_to(hs, (6, 1, H)).copy()
    out = oracle.decode(trie, 3, emb, hid)
    assert list(out["tokens"][0][::2]) == [toks[5], toks[9], toks[30]]
    assert out["margin"][0][0] == 0.0


def pin_zero_hidden_lexicographic():
    """With h = 0 every logit ties, so the answer is min L_k(C) in token order."""
    for cat, V, sep, stop in tiny_cases():
        trie = oracle.Trie(cat, V, sep, stop)
        for k in range(1, min(3, len(cat)) + 1):
            want = min(language(cat, k, sep, stop))
            T = k * (trie.max_depth + 1)
            out = oracle.decode(trie, k, np.ones((V, 3), np.float32), np.zeros((T, 1, 3), np.float32))
            got = tuple(int(x) for x in out["tokens"][0] if x >= 0)
            assert got == want, (cat, k)
            assert out["status"][0] == oracle.OK


def _check_answer(tokens, cat, k, sep, stop, entries, length):
    """The emitted string is in L_k(C) and agrees with entries and length."""
    s = [int(x) for x in tokens if x >= 0]
    assert len(s) == length and s[-1] == stop and s.count(stop) == 1
    pieces, cur = [], []
    for t in s[:-1]:
        if t == sep:
            pieces.append(tuple(cur))
            cur = []
        else:
            cur.append(t)
    pieces.append(tuple(cur))
    assert len(pieces) == k
    index = {tuple(e): i for i, e in enumerate(cat)}
    ids = [index[p] for p in pieces]
    assert len(set(ids)) == k
    assert list(entries) == ids
    assert length == sum(len(p) for p in pieces) + k


def pin_decode_invariants():
    rng = np.random.Generator(np.random.PCG64(5))
    for cid in ("tiny", "product", "structured", "unstructured"):
        c = CONFIGS[cid]
        cat = catalog(cid)
        trie = oracle.Trie(cat, c.vocab, c.sep, c.stop)
        H = 8
        emb = rng.standard_normal((c.vocab, H), dtype=np.float32)
        B = 16
        T = c.k * (trie.max_depth + 1)
        hid = rng.standard_normal((T, B, H), dtype=np.float32)
        out = oracle.decode(trie, c.k, emb, hid)
        for b in range(B):
            assert out["status"][b] == oracle.OK
            _check_answer(out["tokens"][b], cat, c.k, c.sep, c.stop, out["entries"][b], out["len"][b])
        assert np.all(out["margin"][out["tokens"] >= 0] >= 0)
    # k = K: a permutation of the whole catalog; k = 1: one entry then stop
    cat = random_catalog(3, 6, 4, 100)
    trie = oracle.Trie(cat, 128, 126, 127)
    for k in (1, 6):
        T = k * (trie.max_depth + 1)
        out = oracle.decode(trie, k, rng.standard_normal((128, 4), dtype=np.float32),
                            rng.standard_normal((T, 4, 4), dtype=np.float32))
        for b in range(4):
            _check_answer(out["tokens"][b], cat, k, 126, 127, out["entries"][b], out["len"][b])
            if k == 6:
                assert sorted(out["entries"][b]) == list(range(6))


def _exact_logit(ef, hf, v):
    """(exact dot product rounded once, exact sum |p|) of token v."""
    p = ef[v].astype(np.float64) * hf.astype(np.float64)
    return math.fsum(p.tolist()), math.fsum(np.abs(p).tolist())


def _top_two(cands, ef, hf):
    """First maximum (ties to the lower id) and runner-up of exact logits over
    the candidate tokens, with each one's exact sum |p|."""
    vals = sorted(((-_exact_logit(ef, hf, v)[0], v) for v in cands))
    top = vals[0][1]
    second = vals[1][1] if len(vals) > 1 else None
    return top, second


def pin_step_statistics():
    """Winner, margin and sum|p| recorded at every step of seeded decodes equal
    a recomputation from exact dot products over the legal set (the legal set
    itself is pinned by the brute-force mask check)."""
    rng = np.random.Generator(np.random.PCG64(23))
    u = 2.0 ** -53
    cases = [("tiny", "f32", 64), ("structured", "bf16", 96)]
    checked = 0
    for cid, dt, H in cases:
        c = CONFIGS[cid]
        cat = catalog(cid)
        trie = oracle.Trie(cat, c.vocab, c.sep, c.stop)
        x = rng.standard_normal((c.vocab, H), dtype=np.float32) * np.float32(0.02)
        B = 6
        T = c.k * (trie.max_depth + 1)
        hx = rng.standard_normal((T, B, H), dtype=np.float32)
        if dt == "bf16":
            emb, hid = bf16_bits_from_f32(x), bf16_bits_from_f32(hx)
            ef, hf = bf16_bits_to_f32(emb), bf16_bits_to_f32(hid)
        else:
            emb, hid, ef, hf = x, hx, x, hx
        # exact ties: a few tokens share one row
        first = [e[0] for e in cat]
        emb = emb.copy()
        ef = ef.copy()
        for v in first[1:4]:
            emb[v] = emb[first[0]]
            ef[v] = ef[first[0]]
        out = oracle.decode(trie, c.k, emb, hid)
        g = (H - 1) * u / (1 - (H - 1) * u)
        for b in range(B):
            st = oracle.State(trie, c.k)
            for t in range(T):
                lg = st.legal()
                if lg is None:
                    assert out["tokens"][b, t] == -1
                    continue
                cands = [int(v) for v in lg[0]]
                top, second = _top_two(cands, ef, hf[t, b])
                l1, a1 = _exact_logit(ef, hf[t, b], top)
                assert out["tokens"][b, t] == top, (cid, b, t)
                assert out["nlegal"][b, t] == len(cands)
                assert abs(out["best"][b, t] - l1) <= g * a1
                if second is None:
                    assert out["margin"][b, t] == math.inf
                    assert abs(out["sumabs"][b, t] - a1) <= g * a1
                else:
                    l2, a2 = _exact_logit(ef, hf[t, b], second)
                    assert abs(out["margin"][b, t] - (l1 - l2)) <= 2 * g * max(a1, a2), (cid, b, t)
                    assert abs(out["sumabs"][b, t] - max(a1, a2)) <= g * max(a1, a2), (cid, b, t)
                checked += 1
                assert st.advance(top) == oracle.OK
    assert checked > 100


def pin_teacher_forcing():
    """Forced along random strings of L_k(C): at every step the recorded pick
    is the first maximum of exact logits over Mask(u) (the language
    definition), the state follows the forced string to its entries, and a
    token outside Mask(u) is refused at the step where it is forced."""
    rng = np.random.Generator(np.random.PCG64(31))
    for ci, (cat, V, sep, stop) in enumerate(tiny_cases()[:24]):
        trie = oracle.Trie(cat, V, sep, stop)
        H = 5
        emb = rng.standard_normal((V, H), dtype=np.float32)
        emb[3] = emb[4]  # an exact tie between two tokens
        for k in range(1, min(3, len(cat)) + 1):
            L = language(cat, k, sep, stop)
            s = L[int(rng.integers(0, len(L)))]
            T = k * (trie.max_depth + 1)
            hid = rng.standard_normal((T, 1, H), dtype=np.float32)
            follow = np.full((1, T), -1, np.int32)
            follow[0, :len(s)] = s
            out = oracle.decode(trie, k, emb, hid, follow=follow)
            for t in range(len(s)):
                want = mask_by_definition(L, tuple(s[:t]))
                top, _ = _top_two(want, emb, hid[t, 0])
                assert out["tokens"][0, t] == top, (ci, k, t)
            assert (out["tokens"][0, len(s):] == -1).all()
            assert out["status"][0] == oracle.OK and out["len"][0] == len(s)
            pieces, cur = [], []
            for x in s[:-1]:
                if x == sep:
                    pieces.append(tuple(cur))
                    cur = []
                else:
                    cur.append(x)
            pieces.append(tuple(cur))
            index = {tuple(e): i for i, e in enumerate(cat)}
            ids = [index[p] for p in pieces]
            assert list(out["entries"][0]) == ids, (ci, k)
            # a token outside the mask, forced at a random step, is refused there
            t = int(rng.integers(0, len(s)))
            want = mask_by_definition(L, tuple(s[:t]))
            bad = [v for v in range(V) if v not in want]
            if bad:
                f2 = follow.copy()
                f2[0, t] = bad[int(rng.integers(0, len(bad)))]
                o2 = oracle.decode(trie, k, emb, hid, follow=f2)
                assert o2["status"][0] == oracle.ERR_NOT_WALKABLE, (ci, k, t)
                assert (o2["tokens"][0, t + 1:] == -1).all()
                assert np.array_equal(o2["tokens"][0, :t + 1], out["tokens"][0, :t + 1])


# ----------------------------------------------------------------------------
# Tests
# ----------------------------------------------------------------------------

def test_mask_matches_language_definition():
    pin_mask_brute_force()


def test_golden_prefix_pairs():
    pin_golden_prefix_pairs()


def test_live_counts_match_definition():
    pin_live_counts()


def test_trie_closed_forms_small():
    pin_trie_closed_forms(tiny_cases())


def test_trie_closed_forms_configs():
    cats = []
    for cid in ("tiny", "product", "product_deep", "structured", "unstructured", "large"):
        c = CONFIGS[cid]
        cats.append((catalog(cid), c.vocab, c.sep, c.stop))
    pin_trie_closed_forms(cats)


def test_logits_exact():
    pin_logits_exact()


def test_flat_catalog_topk():
    pin_flat_topk()


def test_zero_hidden_is_lexicographic_minimum():
    pin_zero_hidden_lexicographic()


def test_decode_invariants():
    pin_decode_invariants()


def test_step_statistics_exact():
    pin_step_statistics()


def test_teacher_forcing_follows_language():
    pin_teacher_forcing()


def test_catalog_validation():
    V, sep, stop = 16, 14, 15
    bad = [
        [[1], []],            # empty entry
        [[1], [16]],          # token out of range
        [[1], [-1]],
        [[1], [2, 14]],       # contains sep
        [[15]],               # contains stop
        [[1, 2], [1, 2]],     # duplicate
    ]
    for cat in bad:
        with pytest.raises(oracle.OracleError) as ei:
            oracle.Trie(cat, V, sep, stop)
        assert ei.value.code == oracle.ERR_CATALOG, cat
    trie = oracle.Trie([[1], [2]], V, sep, stop)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.decode(trie, 3, np.ones((V, 2), np.float32), np.zeros((4, 1, 2), np.float32))
    assert ei.value.code == oracle.ERR_K
    # too few steps: the sequence is reported as not done
    out = oracle.decode(trie, 2, np.ones((V, 2), np.float32), np.zeros((2, 1, 2), np.float32))
    assert out["status"][0] == oracle.ERR_NOT_DONE


ALL_PINS = [pin_mask_brute_force, pin_golden_prefix_pairs, pin_live_counts, pin_logits_exact,
            pin_flat_topk, pin_zero_hidden_lexicographic, pin_step_statistics, pin_teacher_forcing]


@pytest.mark.parametrize("mutant", [oracle.MUT_TIE_HIGHER_ID, oracle.MUT_NO_LIVE_DECREMENT,
                                    oracle.MUT_NO_SPENT_FLAG, oracle.MUT_ROW_OFF_BY_ONE,
                                    oracle.MUT_SEP_STOP_SWAPPED, oracle.MUT_DROP_LAST_TERM,
                                    oracle.MUT_MARGIN_ZERO, oracle.MUT_SUMABS_WINNER,
                                    oracle.MUT_FOLLOW_IGNORED])
def test_negative_controls(mutant):
    """Each planted oracle mistake must be rejected by at least one pin."""
    caught = []
    oracle.set_mutant(mutant)
    try:
        for pin in ALL_PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError, KeyError, IndexError, ValueError):
                caught.append(pin.__name__)
    finally:
        oracle.set_mutant(0)
    assert caught, f"mutant {mutant} passed every pin"
