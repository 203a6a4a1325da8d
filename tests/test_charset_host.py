"""CPU checks of the library's character-catalog compiler (tms_charset_build:
a byte trie plus one Aho-Corasick automaton over the vocabulary) against the
oracle's plain definition of the legal set, with no GPU call.

For each node of the compiled trie, the bytes spelled on the way to it are
recovered by walking the exported CSR from the root (any token path to a node
spells the same bytes: nodes are byte-trie nodes); the node's legal set with
one string to choose (its token edges, plus stop where a string ends) must
equal oracle.CharCatalog.mask of those bytes, token for token."""
import numpy as np
import pytest

import oracle
import trie_masked_sparse_amd as tms
from synth import CHAR_CONFIGS, char_catalog, char_vocab

from test_charset_oracle import tiny_cases


@pytest.fixture(scope="module")
def L():
    return tms.lib()


def _node_bytes(csr, vocab):
    """Bytes spelled from the root to every node (breadth-first walk)."""
    b = csr["begin"]
    pre = {0: b""}
    order = [0]
    for n in order:
        for e in range(b[n], b[n + 1]):
            c = int(csr["child"][e])
            if c >= 0 and c not in pre:
                pre[c] = pre[n] + vocab[int(csr["tok"][e])]
                order.append(c)
    return pre


def _check(strings, vocab, sep, stop, sample=None, seed=0):
    h = tms.charset_build(strings, vocab, sep, stop)
    try:
        csr = tms.trie_export_csr(h)
        info = tms.trie_info_get(h)
    finally:
        tms.trie_free(h)
    cc = oracle.CharCatalog(strings, vocab, sep, stop)
    pre = _node_bytes(csr, vocab)
    N = info["n_nodes"]
    assert len(pre) == N, "every node is reached from the root"
    # node count: distinct non-empty prefixes of the strings, plus the root
    assert N == len({s[:i] for s in strings for i in range(1, len(s) + 1)}) + 1
    nodes = range(N) if sample is None else \
        sorted(set([0]) | set(np.random.Generator(np.random.PCG64(seed)).choice(N, min(sample, N), replace=False)))
    b = csr["begin"]
    for n in nodes:
        toks = [int(t) for t in csr["tok"][b[n]:b[n + 1]]]
        kids = [int(c) for c in csr["child"][b[n]:b[n + 1]]]
        assert toks == sorted(toks) and len(set(toks)) == len(toks)
        legal = [t for t, c in zip(toks, kids) if c >= 0 or c == -2]  # k = 1: stop, never sep
        assert list(cc.mask(pre[n])) == legal, (n, pre[n])
        ent = int(csr["entry"][n])
        assert (ent >= 0) == (pre[n] in set(strings))
        if ent >= 0:
            assert strings[ent] == pre[n] and -1 in kids and -2 in kids
        for t, c in zip(toks, kids):
            if c >= 0:
                assert pre[c] == pre[n] + vocab[t]
    return info


def test_tiny_catalogs_every_node(L):
    for strings, vocab, sep, stop in tiny_cases():
        _check(strings, vocab, sep, stop)


@pytest.mark.parametrize("cid", sorted(CHAR_CONFIGS))
def test_workload_catalogs_sampled_nodes(L, cid):
    c = CHAR_CONFIGS[cid]
    info = _check(char_catalog(cid), char_vocab(cid), c.sep, c.stop, sample=250, seed=7)
    print(cid, info)


def test_rejected_catalogs(L):
    V = [b"a", b"b", b"", b""]
    for strings in ([b"ab", b"ac"], [b"a", b""], [b"ab", b"ab"]):
        with pytest.raises(tms.TmsError) as ei:
            tms.charset_build(strings, V, 2, 3)
        assert ei.value.code == tms.ERR_CATALOG, strings
    with pytest.raises(tms.TmsError) as ei:
        tms.charset_build([b"a"], V, 2, 2)
    assert ei.value.code == tms.ERR_INVALID_ARG
