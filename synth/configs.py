"""Seeded generators for the five workload shapes and for small test cases.

Every draw uses numpy's ``Generator(PCG64(seed))``.  Seeds: catalog 1000+c,
embedding 2000+c (the batched structured and unstructured workloads reuse the
product-scale table, seed 2002), hidden states 3000+c.

Shapes (vocabulary V, hidden size H, element type, catalog, k pointers, batch B):

1 tiny            V=4096,   H=256,  fp32, 42 tools of 2-6 tokens sharing
                  namespace prefixes, k=3, B=1
2 product         V=151936, H=2048, bf16, 42 tools of 2-8 tokens, k=3, B=1
2b product_deep   as 2 with 14-18 tokens per tool (about 610 trie nodes, close
                  to the node count quoted for the 42-tool product catalog)
3 structured      as 2, 1000 names namespace.verb_noun of 3-10 tokens,
                  prefix-sharing ratio about 0.38 (28 noun bases), k=4, B=64
4 unstructured    as 2, 1000 random strings of 10-16 tokens over a 4096-id
                  subset (root fan-out about 887), k=2, B=64
5 large           V=151936, H=4096, bf16, 100000 four-level names of 4-14
                  tokens, sibling first tokens distinct, k=5, B=256

The separator and stop ids are V-2 and V-1 and never appear inside an entry.
The embedding is N(0, 0.02^2) and the hidden states N(0, 1); bf16 values are
the fp32 draw rounded to nearest even on the bit pattern.
"""
from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Config:
    cid: str
    vocab: int
    hidden: int
    dtype: str          # "f32" or "bf16"
    k: int
    batch: int
    emb_seed: int
    cat_seed: int
    hid_seed: int

    @property
    def sep(self) -> int:
        return self.vocab - 2

    @property
    def stop(self) -> int:
        return self.vocab - 1


CONFIGS = {
    "tiny": Config("tiny", 4096, 256, "f32", 3, 1, 2001, 1001, 3001),
    "product": Config("product", 151936, 2048, "bf16", 3, 1, 2002, 1002, 3002),
    "product_deep": Config("product_deep", 151936, 2048, "bf16", 3, 1, 2002, 1012, 3012),
    "structured": Config("structured", 151936, 2048, "bf16", 4, 64, 2002, 1003, 3003),
    "unstructured": Config("unstructured", 151936, 2048, "bf16", 2, 64, 2002, 1004, 3004),
    "large": Config("large", 151936, 4096, "bf16", 5, 256, 2005, 1005, 3005),
}


# ----------------------------------------------------------------------------
# bf16 bit handling (round to nearest even on the fp32 bit pattern)
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.
    Inputs are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float, dtype: str, chunk_rows: int = 4096):
    """Draw N(0, scale^2) row blocks in a fixed order; return fp32 or bf16 bits."""
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[r0:r1] = x if dtype == "f32" else bf16_bits_from_f32(x)
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# Catalogs
# ----------------------------------------------------------------------------

def pack_catalog(entries):
    """List of token lists -> (tokens int32 [sum len], offsets int64 [K+1])."""
    offs = np.zeros(len(entries) + 1, dtype=np.int64)
    offs[1:] = np.cumsum([len(e) for e in entries])
    toks = np.fromiter((t for e in entries for t in e), dtype=np.int32, count=int(offs[-1]))
    return toks, offs


def _ids(rng, n, hi):
    return [int(x) for x in rng.integers(0, hi, size=n)]


def _namespaced(rng, n_tools, n_ns, ns_len, tool_len, id_hi):
    """Tools = one of n_ns namespace prefixes + a random suffix; total length in tool_len."""
    spaces = []
    while len(spaces) < n_ns:
        s = tuple(_ids(rng, int(rng.integers(ns_len[0], ns_len[1] + 1)), id_hi))
        if s not in spaces:
            spaces.append(s)
    seen, out = set(), []
    while len(out) < n_tools:
        ns = spaces[int(rng.integers(0, n_ns))]
        lo = max(tool_len[0], len(ns) + 1)
        total = int(rng.integers(lo, max(lo, tool_len[1]) + 1))
        tool = ns + tuple(_ids(rng, total - len(ns), id_hi))
        if tool not in seen:
            seen.add(tool)
            out.append(list(tool))
    return out


def _structured(rng, n_tools, id_hi, n_ns=8, n_verb=10, n_base=28):
    """namespace(1-3) ++ verb(1-3) ++ noun, noun = base(1 token) + tail(0-3)."""
    def pool(n, lo, hi):
        p = []
        while len(p) < n:
            s = tuple(_ids(rng, int(rng.integers(lo, hi + 1)), id_hi))
            if s not in p:
                p.append(s)
        return p
    spaces, verbs = pool(n_ns, 1, 3), pool(n_verb, 1, 3)
    bases = [(b,) for b in rng.choice(id_hi, size=n_base, replace=False).tolist()]
    seen, out = set(), []
    while len(out) < n_tools:
        ns = spaces[int(rng.integers(0, n_ns))]
        vb = verbs[int(rng.integers(0, n_verb))]
        base = bases[int(rng.integers(0, n_base))]
        tail = tuple(_ids(rng, int(rng.integers(0, 4)), id_hi))
        tool = ns + vb + base + tail
        if tool not in seen:
            seen.add(tool)
            out.append(list(tool))
    return out


def _unstructured(rng, n, id_hi, lens=(10, 16), subset=4096):
    alphabet = rng.choice(id_hi, size=subset, replace=False)
    seen, out = set(), []
    while len(out) < n:
        L = int(rng.integers(lens[0], lens[1] + 1))
        s = tuple(int(x) for x in alphabet[rng.integers(0, subset, size=L)])
        if s not in seen:
            seen.add(s)
            out.append(list(s))
    return out


def _hierarchical(rng, n_total, id_hi, fan=(48, 24, 12)):
    """Four levels; siblings get distinct first tokens, so no entry is a prefix
    of another and every fan-out is bounded by the level sizes."""
    def children(n):
        firsts = rng.choice(id_hi, size=n, replace=False)
        comps = []
        for f in firsts.tolist():
            L = int(rng.integers(1, 4))
            comps.append([f] + _ids(rng, L - 1, id_hi))
        return comps
    groups = []
    for c1 in children(fan[0]):
        for c2 in children(fan[1]):
            for c3 in children(fan[2]):
                groups.append(c1 + c2 + c3)
    n_groups = len(groups)
    base = n_total // n_groups
    extra = n_total - base * n_groups
    out = []
    for gi, prefix in enumerate(groups):
        n_leaf = base + (1 if gi < extra else 0)
        firsts = rng.choice(id_hi, size=n_leaf, replace=False).tolist()
        for f in firsts:
            L = int(rng.integers(1, 6))
            out.append(prefix + [f] + _ids(rng, L - 1, id_hi))
    return out


def catalog(cid: str):
    """Entries of one named workload as a list of token lists (deterministic)."""
    return [list(e) for e in _catalog_cached(cid)]


@functools.lru_cache(maxsize=None)
def _catalog_cached(cid: str):
    c = CONFIGS[cid]
    rng = np.random.Generator(np.random.PCG64(c.cat_seed))
    hi = c.vocab - 2          # ids in [0, V-2): the two control ids never appear
    if cid == "tiny":
        e = _namespaced(rng, 42, 6, (1, 2), (2, 6), hi)
    elif cid == "product":
        e = _namespaced(rng, 42, 6, (1, 3), (2, 8), hi)
    elif cid == "product_deep":
        e = _namespaced(rng, 42, 6, (1, 3), (14, 18), hi)
    elif cid == "structured":
        e = _structured(rng, 1000, hi)
    elif cid == "unstructured":
        e = _unstructured(rng, 1000, hi)
    elif cid == "large":
        e = _hierarchical(rng, 100000, hi)
    else:
        raise KeyError(cid)
    return tuple(tuple(x) for x in e)


def random_catalog(seed: int, K: int, max_len: int, id_hi: int, min_len: int = 1):
    """Small random catalog of K distinct strings (tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seen, out = set(), []
    tries = 0
    while len(out) < K:
        tries += 1
        if tries > 100000:
            raise ValueError("cannot draw that many distinct strings")
        L = int(rng.integers(min_len, max_len + 1))
        s = tuple(_ids(rng, L, id_hi))
        if s not in seen:
            seen.add(s)
            out.append(list(s))
    return out


# ----------------------------------------------------------------------------
# Tables and hidden states
# ----------------------------------------------------------------------------

@functools.lru_cache(maxsize=2)
def _embedding_cached(vocab, hidden, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    e = _normal(rng, (vocab, hidden), 0.02, dtype)
    e.setflags(write=False)
    return e


def embedding(cid: str) -> np.ndarray:
    """[V][H] table: float32 values, or uint16 bf16 bit patterns."""
    c = CONFIGS[cid]
    return _embedding_cached(c.vocab, c.hidden, c.dtype, c.emb_seed)


def hidden_states(cid: str, T: int, B: int | None = None, seed: int | None = None) -> np.ndarray:
    """[T][B][H] hidden states, one fresh N(0,1) vector per (step, sequence)."""
    c = CONFIGS[cid]
    B = c.batch if B is None else B
    rng = np.random.Generator(np.random.PCG64(c.hid_seed if seed is None else seed))
    return _normal(rng, (T * B, c.hidden), 1.0, c.dtype).reshape(T, B, c.hidden)


def stress_rows(vocab: int, batch: int, per_seq: int, n_sets: int, seed: int = 4242) -> np.ndarray:
    """[n_sets][batch][per_seq] distinct row ids: every row id appears once over
    all sets, so cycling through the sets never re-reads a row."""
    need = batch * per_seq * n_sets
    if need > vocab:
        raise ValueError("not enough distinct rows")
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.permutation(vocab)[:need].astype(np.int32)
    return ids.reshape(n_sets, batch, per_seq)
