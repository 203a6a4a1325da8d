"""Python view of the CPU oracle (oracle/tms_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
bench's CPU-baseline leg, never by the library.  It shares no code with the HIP
path.  ``build()`` compiles the C file with gcc (-O2, no fast-math, so every
sum keeps its written order).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tms_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_INVALID_ARG, ERR_CATALOG, ERR_FANOUT, ERR_K, ERR_EMPTY_MASK, ERR_NOT_WALKABLE, ERR_NOT_DONE = range(8)
CHILD_SEP, CHILD_STOP = -1, -2

# planted mistakes for negative-control tests
MUT_NONE, MUT_TIE_HIGHER_ID, MUT_NO_LIVE_DECREMENT, MUT_NO_SPENT_FLAG, MUT_ROW_OFF_BY_ONE, \
    MUT_SEP_STOP_SWAPPED, MUT_DROP_LAST_TERM, MUT_MARGIN_ZERO, MUT_SUMABS_WINNER, MUT_FOLLOW_IGNORED, \
    MUT_CS_FIRST_BYTE, MUT_CS_STOP_LEAF_ONLY = range(12)


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.orc_trie_build.argtypes = [P, P, i32, i32, i32, i32, C.POINTER(P)]
        L.orc_trie_build.restype = C.c_int
        L.orc_trie_free.argtypes = [P]
        L.orc_trie_info.argtypes = [P, P]
        L.orc_trie_csr.argtypes = [P, P, P, P, P, P]
        L.orc_state_new.argtypes = [P, i32]
        L.orc_state_new.restype = P
        L.orc_state_free.argtypes = [P]
        L.orc_state_legal.argtypes = [P, P, P]
        L.orc_state_legal.restype = i32
        L.orc_state_advance.argtypes = [P, i32]
        L.orc_state_advance.restype = i32
        L.orc_state_info.argtypes = [P, P]
        L.orc_state_live.argtypes = [P, P]
        L.orc_state_entries.argtypes = [P, P]
        L.orc_logit.argtypes = [P, C.c_int, i32, i32, P, C.POINTER(C.c_double)]
        L.orc_logit.restype = C.c_double
        L.orc_dense_logits.argtypes = [P, C.c_int, i32, i32, P, P]
        L.orc_decode.argtypes = [P, i32, P, C.c_int, i32, i32, P, i32, i32] + [P] * 9
        L.orc_decode.restype = C.c_int
        L.orc_set_mutant.argtypes = [C.c_int]
        L.orc_cs_build.argtypes = [P, P, i32, P, P, i32, i32, i32, C.POINTER(P)]
        L.orc_cs_build.restype = C.c_int
        L.orc_cs_free.argtypes = [P]
        L.orc_cs_info.argtypes = [P, P]
        L.orc_cs_mask.argtypes = [P, P, i64, P]
        L.orc_cs_mask.restype = i32
        L.orc_cs_decode.argtypes = [P, P, C.c_int, i32, P, i32, i32] + [P] * 9
        L.orc_cs_decode.restype = C.c_int
        _lib = L
    return _lib


def set_mutant(m: int) -> None:
    lib().orc_set_mutant(int(m))


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return 0
    if arr.dtype == np.uint16:
        return 1
    raise TypeError("tables are float32 or uint16 bf16 bit patterns")


class OracleError(RuntimeError):
    def __init__(self, code, what=""):
        super().__init__(f"oracle status {code} {what}")
        self.code = code


class Trie:
    """Canonical CSR trie of a catalog (see tms_oracle.c for the reading)."""

    def __init__(self, entries, vocab: int, sep: int, stop: int):
        if isinstance(entries, tuple) and len(entries) == 2 and isinstance(entries[0], np.ndarray):
            toks, offs = entries
        else:
            offs = np.zeros(len(entries) + 1, dtype=np.int64)
            offs[1:] = np.cumsum([len(e) for e in entries]) if len(entries) else []
            toks = np.array([t for e in entries for t in e] or [0], dtype=np.int32)
        self._toks = np.ascontiguousarray(toks, dtype=np.int32)
        self._offs = np.ascontiguousarray(offs, dtype=np.int64)
        h = C.c_void_p()
        rc = lib().orc_trie_build(_ptr(self._toks), _ptr(self._offs), len(self._offs) - 1, vocab,
                                  sep, stop, C.byref(h))
        if rc != OK:
            raise OracleError(rc, "trie build")
        self._h = h
        info = np.zeros(8, dtype=np.int32)
        lib().orc_trie_info(self._h, _ptr(info))
        (self.n_nodes, self.n_edges, self.n_entries, self.cap, self.max_depth,
         self.sep, self.stop, self.vocab) = (int(x) for x in info)

    def __del__(self):
        # at interpreter exit the module globals (lib among them) may already
        # be gone; the process is ending and frees the memory anyway
        if getattr(self, "_h", None) and lib is not None:
            lib().orc_trie_free(self._h)
            self._h = None

    def csr(self):
        b = np.zeros(self.n_nodes + 1, np.int32)
        en = np.zeros(self.n_nodes, np.int32)
        t = np.zeros(self.n_edges, np.int32)
        c = np.zeros(self.n_edges, np.int32)
        l0 = np.zeros(self.n_edges, np.int32)
        lib().orc_trie_csr(self._h, _ptr(b), _ptr(en), _ptr(t), _ptr(c), _ptr(l0))
        return {"begin": b, "entry": en, "tok": t, "child": c, "live0": l0}


class State:
    """One sequence's decode state over a Trie."""

    def __init__(self, trie: Trie, k: int):
        self.trie = trie
        self.k = k
        self._h = lib().orc_state_new(trie._h, k)

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_state_free(self._h)
            self._h = None

    def legal(self):
        """(tokens, edges) legal now, ascending token order; None when inactive."""
        toks = np.zeros(max(self.trie.cap, 1), np.int32)
        edges = np.zeros(max(self.trie.cap, 1), np.int32)
        n = lib().orc_state_legal(self._h, _ptr(toks), _ptr(edges))
        if n < 0:
            return None
        return toks[:n].copy(), edges[:n].copy()

    def advance(self, tok: int) -> int:
        return int(lib().orc_state_advance(self._h, int(tok)))

    def info(self):
        a = np.zeros(6, np.int32)
        lib().orc_state_info(self._h, _ptr(a))
        return dict(zip(("node", "depth", "done", "finished", "status", "n_emitted"), (int(x) for x in a)))

    def live(self):
        a = np.zeros(self.trie.n_edges, np.int32)
        lib().orc_state_live(self._h, _ptr(a))
        return a

    def entries(self):
        a = np.zeros(self.k, np.int32)
        lib().orc_state_entries(self._h, _ptr(a))
        return a


def logit(emb: np.ndarray, v: int, h: np.ndarray):
    """(fp64 logit of token v, sum |h_i E_vi|)."""
    emb = np.ascontiguousarray(emb)
    h = np.ascontiguousarray(h, dtype=emb.dtype)
    a = C.c_double()
    val = lib().orc_logit(_ptr(emb), _dtype_code(emb), emb.shape[1], int(v), _ptr(h), C.byref(a))
    return float(val), float(a.value)


def dense_logits(emb: np.ndarray, h: np.ndarray) -> np.ndarray:
    emb = np.ascontiguousarray(emb)
    h = np.ascontiguousarray(h, dtype=emb.dtype)
    out = np.zeros(emb.shape[0], np.float64)
    lib().orc_dense_logits(_ptr(emb), _dtype_code(emb), emb.shape[0], emb.shape[1], _ptr(h), _ptr(out))
    return out


def decode(trie: Trie, k: int, emb: np.ndarray, hidden: np.ndarray, follow: np.ndarray | None = None):
    """Greedy decode of hidden [T][B][H]; returns a dict of numpy arrays.

    follow: optional [B][T] int32 tokens to advance by (teacher forcing): the
    oracle records its own greedy pick and statistics at every step, then
    advances by follow[b][t] where that is >= 0 (NOT_WALKABLE if it is not
    legal there) and by its own pick elsewhere."""
    emb = np.ascontiguousarray(emb)
    hidden = np.ascontiguousarray(hidden, dtype=emb.dtype)
    T, B, H = hidden.shape
    if H != emb.shape[1]:
        raise ValueError("hidden size mismatch")
    if follow is not None:
        follow = np.ascontiguousarray(follow, dtype=np.int32)
        if follow.shape != (B, T):
            raise ValueError(f"follow must be [B][T] = [{B}][{T}], got {follow.shape}")
    out = {
        "tokens": np.full((B, T), -1, np.int32),
        "len": np.zeros(B, np.int32),
        "entries": np.full((B, k), -1, np.int32),
        "status": np.zeros(B, np.int32),
        "best": np.zeros((B, T), np.float64),
        "margin": np.zeros((B, T), np.float64),
        "sumabs": np.zeros((B, T), np.float64),
        "nlegal": np.zeros((B, T), np.int32),
    }
    rc = lib().orc_decode(trie._h, k, _ptr(emb), _dtype_code(emb), emb.shape[0], H, _ptr(hidden), B, T,
                          _ptr(follow), *(_ptr(out[n]) for n in ("tokens", "len", "entries", "status", "best",
                                                                  "margin", "sumabs", "nlegal")))
    if rc != OK:
        raise OracleError(rc, "decode")
    return out


# ---------------------------------------------------------------------------
# Character-level catalogs (the review of arXiv 2608.12574): one string of a
# byte-string catalog, spelled by tokens whose byte strings are given.
# ---------------------------------------------------------------------------

def pack_bytes(items):
    """list of bytes -> (uint8 concatenation, int64 offsets)."""
    off = np.zeros(len(items) + 1, np.int64)
    off[1:] = np.cumsum([len(x) for x in items])
    buf = np.frombuffer(b"".join(items) or b"\0", np.uint8).copy()
    return buf, off


class CharCatalog:
    """A catalog of byte strings with a token vocabulary (token v spells
    vocab[v]; b"" for control and unused tokens)."""

    def __init__(self, strings, vocab, sep: int, stop: int):
        self.strings = [bytes(x) for x in strings]
        self.vocab = [bytes(x) for x in vocab]
        self.V, self.sep, self.stop = len(self.vocab), sep, stop
        self._sb, self._so = pack_bytes(self.strings)
        self._tb, self._to = pack_bytes(self.vocab)
        h = C.c_void_p()
        rc = lib().orc_cs_build(_ptr(self._sb), _ptr(self._so), len(self.strings), _ptr(self._tb), _ptr(self._to),
                                self.V, sep, stop, C.byref(h))
        if rc != OK:
            raise OracleError(rc, "character catalog")
        self._h = h
        info = np.zeros(3, np.int32)
        lib().orc_cs_info(self._h, _ptr(info))
        self.max_len, self.max_tok, self.n_content = (int(x) for x in info)

    def __del__(self):
        if getattr(self, "_h", None) and lib is not None:
            lib().orc_cs_free(self._h)
            self._h = None

    def mask(self, prefix: bytes) -> np.ndarray:
        """Legal token ids (ascending) after the emitted bytes prefix."""
        out = np.zeros(self.V, np.int32)
        p = np.frombuffer(bytes(prefix) or b"\0", np.uint8).copy()
        n = lib().orc_cs_mask(self._h, _ptr(p), len(prefix), _ptr(out))
        return out[:n].copy()

    def decode(self, emb: np.ndarray, hidden: np.ndarray, follow: np.ndarray | None = None):
        """Greedy decode (one string) of hidden [T][B][H]; dict of arrays as
        for decode(), with entry [B] instead of entries."""
        emb = np.ascontiguousarray(emb)
        hidden = np.ascontiguousarray(hidden, dtype=emb.dtype)
        T, B, H = hidden.shape
        if emb.shape[0] != self.V or emb.shape[1] != H:
            raise ValueError("table must be [V][H] with the hidden size")
        if follow is not None:
            follow = np.ascontiguousarray(follow, dtype=np.int32)
            if follow.shape != (B, T):
                raise ValueError("follow must be [B][T]")
        out = {"tokens": np.full((B, T), -1, np.int32), "len": np.zeros(B, np.int32),
               "entry": np.full(B, -1, np.int32), "status": np.zeros(B, np.int32),
               "best": np.zeros((B, T)), "margin": np.zeros((B, T)), "sumabs": np.zeros((B, T)),
               "nlegal": np.zeros((B, T), np.int32)}
        rc = lib().orc_cs_decode(self._h, _ptr(emb), _dtype_code(emb), H, _ptr(hidden), B, T, _ptr(follow),
                                 *(_ptr(out[n]) for n in ("tokens", "len", "entry", "status", "best", "margin",
                                                          "sumabs", "nlegal")))
        if rc != OK:
            raise OracleError(rc, "character decode")
        return out
