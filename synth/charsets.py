"""Seeded character-level catalogs and byte-string vocabularies.

Stand-ins for the finite sets and tokenizers of the review of arXiv
2608.12574 (no tokenizer or enum file is available): a byte-level vocabulary
of V ids in which every byte value is a token of its own, followed by
multi-byte tokens drawn BPE-like from the catalog (its most frequent
substrings of 2 to 8 bytes) and filler byte strings, with the two control ids
last (empty byte strings).  Catalogs:
  charset_tools  1000 tool names "namespace.verb_noun" in lowercase ASCII
                 (8 namespaces, 12 verbs, 40 nouns, optional suffixes),
                 the prefix-structured kind the page measures;
  charset_hex    1000 random 32-character hex strings, the unstructured set
                 the page's falsifier and referee ask for.
Seeds: catalog 1100 + n, vocabulary 1200 + n.  Only draws inputs: no trie,
no matcher, no mask, no arithmetic of the decode.
"""
from __future__ import annotations

import functools
from collections import Counter
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class CharConfig:
    cid: str
    vocab: int
    hidden: int
    batch: int
    cat_seed: int
    voc_seed: int
    hid_seed: int
    emb_cid: str  # the token workload whose embedding table the rows come from

    @property
    def k(self) -> int:
        return 1  # one string per answer

    @property
    def sep(self) -> int:
        return self.vocab - 2

    @property
    def stop(self) -> int:
        return self.vocab - 1


CHAR_CONFIGS = {
    "charset_tools": CharConfig("charset_tools", 151936, 2048, 64, 1101, 1201, 3101, "product"),
    "charset_hex": CharConfig("charset_hex", 151936, 2048, 64, 1102, 1202, 3102, "product"),
}


def _word(rng, lo, hi):
    return "".join(chr(97 + int(x)) for x in rng.integers(0, 26, int(rng.integers(lo, hi + 1))))


def tool_strings(seed: int, n: int = 1000):
    rng = np.random.Generator(np.random.PCG64(seed))
    spaces = sorted({_word(rng, 3, 8) for _ in range(8)})
    verbs = sorted({_word(rng, 3, 7) for _ in range(12)})
    nouns = sorted({_word(rng, 3, 9) for _ in range(40)})
    out, seen = [], set()
    while len(out) < n:
        s = f"{spaces[int(rng.integers(len(spaces)))]}.{verbs[int(rng.integers(len(verbs)))]}_" \
            f"{nouns[int(rng.integers(len(nouns)))]}"
        if rng.random() < 0.3:
            s += "_" + _word(rng, 2, 5)
        if s not in seen:
            seen.add(s)
            out.append(s.encode())
    return out


def hex_strings(seed: int, n: int = 1000, length: int = 32):
    rng = np.random.Generator(np.random.PCG64(seed))
    out, seen = [], set()
    while len(out) < n:
        s = "".join("0123456789abcdef"[int(x)] for x in rng.integers(0, 16, length)).encode()
        if s not in seen:
            seen.add(s)
            out.append(s)
    return out


def byte_vocab(strings, V: int, seed: int, n_merges: int | None = None):
    """V byte strings: the 256 single bytes, then the catalog's most frequent
    substrings of 2-8 bytes (ties by the bytes), then distinct filler strings
    of 2-8 printable bytes; the last two ids (the separator and stop) are
    empty.  Token ids are shuffled except the control ids, so that a token's
    id says nothing of its bytes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_merges = (V - 258) // 4 if n_merges is None else n_merges
    items = [bytes([b]) for b in range(256)]
    have = set(items)
    cnt = Counter()
    for s in strings:
        for L in range(2, 9):
            for i in range(len(s) - L + 1):
                cnt[s[i:i + L]] += 1
    for sub, _ in sorted(cnt.items(), key=lambda kv: (-kv[1], kv[0]))[:n_merges]:
        if sub not in have:
            have.add(sub)
            items.append(sub)
    while len(items) < V - 2:
        x = bytes(int(c) for c in rng.integers(33, 127, int(rng.integers(2, 9))))
        if x not in have:
            have.add(x)
            items.append(x)
    items = items[:V - 2]
    perm = rng.permutation(len(items))
    return [items[i] for i in perm] + [b"", b""]


@functools.lru_cache(maxsize=4)
def char_catalog(cid: str):
    c = CHAR_CONFIGS[cid]
    return tool_strings(c.cat_seed) if cid == "charset_tools" else hex_strings(c.cat_seed)


@functools.lru_cache(maxsize=4)
def char_vocab(cid: str):
    c = CHAR_CONFIGS[cid]
    return byte_vocab(char_catalog(cid), c.vocab, c.voc_seed)


def char_hidden(cid: str, T: int, B: int | None = None) -> np.ndarray:
    from .configs import _normal
    c = CHAR_CONFIGS[cid]
    B = c.batch if B is None else B
    rng = np.random.Generator(np.random.PCG64(c.hid_seed))
    return _normal(rng, (T * B, c.hidden), 1.0, "bf16").reshape(T, B, c.hidden)
