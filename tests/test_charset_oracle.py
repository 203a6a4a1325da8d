"""Pins of the character-catalog oracle (oracle.CharCatalog) against things
other than itself.

The catalog is a set of byte strings; the vocabulary maps token ids to byte
strings (the review of arXiv 2608.12574, fields pith_extraction.key_machinery
and core_discovery).  An answer is one catalog string spelled by tokens, then
stop.  The legal set after tokens u is, by the next-token mask definition of
"GLRMask - constrained decoding with weighted automata", the set of tokens v
such that u v continues some answer.  The pins:
  * brute force on tiny inputs: every tokenization of every catalog string is
    enumerated outright, the legal set after every prefix of every answer is
    read off that list, and every token outside it is refused when forced;
  * a zero hidden state ties every logit, so the answer is the
    lexicographically smallest answer by token ids, a closed form;
  * winner, top-two margin and sum|p| at every step of seeded decodes against
    exact dot products (math.fsum) over the legal set;
  * catalogs the reading rejects (a byte no single-byte token spells, empty or
    duplicate strings);
  * negative controls: each planted mistake fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
from synth import bf16_bits_from_f32, bf16_bits_to_f32


@pytest.fixture(autouse=True, scope="module")
def _built(oracle_lib):
    oracle.set_mutant(0)
    yield
    oracle.set_mutant(0)


def _tokenizations(s: bytes, vocab):
    """Every sequence of content token ids whose bytes concatenate to s."""
    out = []

    def rec(pos, acc):
        if pos == len(s):
            out.append(tuple(acc))
            return
        for v, b in enumerate(vocab):
            if b and s.startswith(b, pos):
                rec(pos + len(b), acc + [v])
    rec(0, [])
    return out


def tiny_cases():
    """Tiny catalogs over a small alphabet with prefix pairs, and vocabularies
    of every single byte plus random merges (control ids last or first)."""
    rng = np.random.Generator(np.random.PCG64(404))
    cases = [([b"ab", b"abc", b"b"], [b"a", b"b", b"c", b"ab", b"bc", b"abc"]),
             ([b"aa", b"a", b"aaa"], [b"a", b"aa"]),
             ([b"x"], [b"x", b"xx"])]
    for _ in range(30):
        alpha = b"abcd"[: int(rng.integers(2, 5))]
        K = int(rng.integers(1, 6))
        strings = set()
        while len(strings) < K:
            n = int(rng.integers(1, 5))
            strings.add(bytes(alpha[int(i)] for i in rng.integers(0, len(alpha), n)))
        vocab = [bytes([c]) for c in alpha]
        for _ in range(int(rng.integers(0, 6))):
            n = int(rng.integers(2, 4))
            m = bytes(alpha[int(i)] for i in rng.integers(0, len(alpha), n))
            if m not in vocab:
                vocab.append(m)
        order = rng.permutation(len(vocab))
        cases.append((sorted(strings), [vocab[i] for i in order]))
    out = []
    for i, (strings, vocab) in enumerate(cases):
        if i % 2:
            full, sep, stop = [b"", b""] + vocab, 0, 1  # control ids first
        else:
            full, sep, stop = vocab + [b"", b""], len(vocab), len(vocab) + 1
        out.append((strings, full, sep, stop))
    return out


def pin_mask_brute_force():
    for strings, vocab, sep, stop in tiny_cases():
        cc = oracle.CharCatalog(strings, vocab, sep, stop)
        answers = [w + (stop,) for s in strings for w in _tokenizations(s, vocab)]
        prefixes = {a[:i] for a in answers for i in range(len(a))}
        for u in prefixes:
            want = sorted({a[len(u)] for a in answers if a[:len(u)] == u})
            pre = b"".join(vocab[v] for v in u)
            got = list(cc.mask(pre))
            assert got == want, (strings, vocab, u, got, want)
            assert sep not in got
        # a forced token outside the mask is refused at that step
        rng = np.random.Generator(np.random.PCG64(len(strings) * 7 + len(vocab)))
        V, H = len(vocab), 3
        emb = rng.standard_normal((V, H), dtype=np.float32)
        a = answers[int(rng.integers(0, len(answers)))]
        T = len(a) + 1
        hid = rng.standard_normal((T, 1, H), dtype=np.float32)
        follow = np.full((1, T), -1, np.int32)
        follow[0, :len(a)] = a
        out = cc.decode(emb, hid, follow)
        assert out["status"][0] == oracle.OK and out["len"][0] == len(a)
        assert strings[out["entry"][0]] == b"".join(vocab[v] for v in a[:-1])
        t = int(rng.integers(0, len(a)))
        legal = set(cc.mask(b"".join(vocab[v] for v in a[:t])))
        bad = [v for v in range(V) if v not in legal]
        if bad:
            f2 = follow.copy()
            f2[0, t] = bad[int(rng.integers(0, len(bad)))]
            o2 = cc.decode(emb, hid, f2)
            assert o2["status"][0] == oracle.ERR_NOT_WALKABLE
            assert (o2["tokens"][0, t + 1:] == -1).all()


def pin_zero_hidden_lexicographic():
    for strings, vocab, sep, stop in tiny_cases():
        cc = oracle.CharCatalog(strings, vocab, sep, stop)
        answers = [w + (stop,) for s in strings for w in _tokenizations(s, vocab)]
        want = min(answers)
        T = max(len(a) for a in answers) + 1
        out = cc.decode(np.ones((len(vocab), 2), np.float32), np.zeros((T, 1, 2), np.float32))
        got = tuple(int(x) for x in out["tokens"][0] if x >= 0)
        assert got == want, (strings, vocab, got, want)
        assert out["status"][0] == oracle.OK


def pin_step_statistics():
    rng = np.random.Generator(np.random.PCG64(17))
    u = 2.0 ** -53
    for strings, vocab, sep, stop in tiny_cases()[:12]:
        cc = oracle.CharCatalog(strings, vocab, sep, stop)
        V, H, B = len(vocab), 40, 3
        T = cc.max_len + 1
        x = rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.1)
        hx = rng.standard_normal((T, B, H), dtype=np.float32)
        emb, hid = bf16_bits_from_f32(x), bf16_bits_from_f32(hx)
        ef, hf = bf16_bits_to_f32(emb).astype(np.float64), bf16_bits_to_f32(hid).astype(np.float64)
        out = cc.decode(emb, hid)
        g = (H - 1) * u / (1 - (H - 1) * u)
        for b in range(B):
            pre = b""
            for t in range(T):
                if out["tokens"][b, t] < 0:
                    break
                legal = cc.mask(pre)
                ex = sorted(((-math.fsum((ef[v] * hf[t, b]).tolist()), int(v)) for v in legal))
                top = ex[0][1]
                assert out["tokens"][b, t] == top
                a1 = math.fsum(np.abs(ef[top] * hf[t, b]).tolist())
                assert abs(out["best"][b, t] + ex[0][0]) <= g * a1
                if len(ex) > 1:
                    a2 = math.fsum(np.abs(ef[ex[1][1]] * hf[t, b]).tolist())
                    assert abs(out["margin"][b, t] - (ex[1][0] - ex[0][0])) <= 2 * g * max(a1, a2)
                    assert abs(out["sumabs"][b, t] - max(a1, a2)) <= g * max(a1, a2)
                if top != stop:
                    pre += vocab[top]


def test_mask_matches_language_definition():
    pin_mask_brute_force()


def test_zero_hidden_is_lexicographic_minimum():
    pin_zero_hidden_lexicographic()


def test_step_statistics_exact():
    pin_step_statistics()


def test_rejected_catalogs():
    V = [b"a", b"b", b"", b""]
    for strings in ([b"ab", b"ac"], [b"a", b""], [b"ab", b"ab"]):
        with pytest.raises(oracle.OracleError) as ei:
            oracle.CharCatalog(strings, V, 2, 3)
        assert ei.value.code == oracle.ERR_CATALOG, strings
    with pytest.raises(oracle.OracleError):
        oracle.CharCatalog([b"a"], V, 2, 2)


@pytest.mark.parametrize("mutant", [oracle.MUT_CS_FIRST_BYTE, oracle.MUT_CS_STOP_LEAF_ONLY])
def test_negative_controls(mutant):
    caught = []
    oracle.set_mutant(mutant)
    try:
        for pin in (pin_mask_brute_force, pin_zero_hidden_lexicographic, pin_step_statistics):
            try:
                pin()
            except (AssertionError, oracle.OracleError):
                caught.append(pin.__name__)
    finally:
        oracle.set_mutant(0)
    assert caught, f"mutant {mutant} passed every pin"
