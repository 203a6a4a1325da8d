"""Python binding of libtms.so (include/tms.h): argument marshalling only.

Every function here forwards to the C entry point of the same name (without
the ``tms_`` prefix); all compute runs in the HIP kernels of the library.
Device buffers are torch tensors (only their data pointers are passed), the
stream defaults to torch's current stream.  There is no fallback: if the
library is not built, or no GPU is present, calls raise.

Fail loudly (page "Constraint made cheaper than no constraint", section
"Masked sampling inside the sampler": an empty mask or an unwalkable token is
an error, never a silent pick): the decode calls (decode_step_sparse,
decode_step_dense_masked, decode_k_pointers, advance_forced) synchronise the
stream after enqueueing their work and raise TmsError when any sequence holds a
device error (EMPTY_MASK, NOT_WALKABLE, NOT_DONE), unless called with
check=False, which leaves them asynchronous (for timed loops and for tests of
the error paths; State.status() then reports the per-sequence codes).  A state
is passed as a State or as its raw handle.

torch is imported before the library is loaded so that both use the same HIP
runtime (torch ships its own libamdhip64 with the same soname).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtms.so")

OK, ERR_INVALID_ARG, ERR_CATALOG, ERR_FANOUT, ERR_K, ERR_EMPTY_MASK, ERR_NOT_WALKABLE, ERR_NOT_DONE, \
    ERR_BUSY, ERR_OOM, ERR_HIP = range(11)
F32, BF16 = 0, 1
PATH_AUTO, PATH_FAST, PATH_GLOBAL = 0, 1, 2
LOOP_RESIDENT, LOOP_GRAPH, LOOP_STREAM, LOOP_RESIDENT_SOLO, LOOP_RESIDENT_GROUPED = 0, 1, 2, 3, 4

# every symbol declared in include/tms.h
EXPORTS = (
    "tms_trie_build", "tms_trie_upload", "tms_charset_build", "tms_charset_upload", "tms_trie_info_get",
    "tms_trie_export_csr", "tms_trie_free",
    "tms_state_create", "tms_state_reset", "tms_state_sync_status", "tms_state_export", "tms_state_free",
    "tms_decode_step_sparse", "tms_decode_step_dense_masked", "tms_decode_k_pointers",
    "tms_advance_forced", "tms_legal_set", "tms_legal_mask", "tms_mask_to_rows", "tms_gather_gemv",
    "tms_debug_set_live",
    "tms_state_set_split", "tms_state_set_loop", "tms_state_set_norepeat", "tms_state_set_step_grouping",
    "tms_state_get_launch",
    "tms_decode_k_pointers_noalloc", "tms_read_reference", "tms_status_str", "tms_last_error",
)
NOREPEAT_LIVE, NOREPEAT_BITMASK = 0, 1
STEP_GROUP_AUTO, STEP_GROUP_OFF, STEP_GROUP_ROOT, STEP_GROUP_NODES = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 32 << 20


class TmsError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        super().__init__(f"{where}: status {code} ({status_str(code)}) {detail}".rstrip())


class TrieInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_nodes", "n_edges", "n_entries", "cap", "max_depth", "sep", "stop",
                                         "vocab", "path")] + [("device_bytes", C.c_int64)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m trie_masked_sparse_amd.build")
        L = C.CDLL(LIB_PATH)
        P, i32 = C.c_void_p, C.c_int32
        PP = C.POINTER(C.c_void_p)
        sig = {
            "tms_trie_build": [P, P, i32, i32, i32, i32, PP],
            "tms_trie_upload": [P, P, i32, i32, i32, i32, C.c_int, P, PP],
            "tms_charset_build": [P, P, i32, P, P, i32, i32, i32, PP],
            "tms_charset_upload": [P, P, i32, P, P, i32, i32, i32, C.c_int, P, PP],
            "tms_trie_info_get": [P, C.POINTER(TrieInfo)],
            "tms_trie_export_csr": [P, P, P, P, P, P],
            "tms_trie_free": [P],
            "tms_state_create": [P, i32, i32, P, C.c_int, i32, P, PP],
            "tms_state_reset": [P, P],
            "tms_state_sync_status": [P, P, P],
            "tms_state_export": [P, P, P, P, P, P, P, P, P, P],
            "tms_state_free": [P],
            "tms_decode_step_sparse": [P, P, P, P, P],
            "tms_decode_step_dense_masked": [P, P, P, P, P, P],
            "tms_decode_k_pointers": [P, P, i32, P, P, P, P],
            "tms_advance_forced": [P, P, P],
            "tms_legal_set": [P, P, P, P],
            "tms_legal_mask": [P, P, P],
            "tms_mask_to_rows": [P, i32, i32, i32, P, P, P],
            "tms_gather_gemv": [P, C.c_int, i32, i32, P, P, P, i32, i32, P, P],
            "tms_debug_set_live": [P, i32, i32, i32, P],
            "tms_state_set_split": [P, i32],
            "tms_state_set_loop": [P, i32],
            "tms_state_set_norepeat": [P, i32],
            "tms_state_set_step_grouping": [P, i32],
            "tms_read_reference": [P, C.c_int64, P, i32, i32, P],
            "tms_decode_k_pointers_noalloc": [P, P, C.c_int, i32, i32, i32, P, i32, P, P, P, P, P],
            "tms_state_get_launch": [P, P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.tms_status_str.argtypes = [C.c_int]
        L.tms_status_str.restype = C.c_char_p
        L.tms_last_error.argtypes = []
        L.tms_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().tms_status_str(int(code)).decode()


def _check(rc: int, where: str):
    if rc != OK:
        raise TmsError(rc, where, lib().tms_last_error().decode())


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _dev(t, dtype=None, name="tensor"):
    """Data pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return C.c_void_p(t.data_ptr())


def _host_i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _catalog_arrays(entries):
    if isinstance(entries, tuple) and len(entries) == 2:
        toks, offs = entries
    else:
        offs = np.zeros(len(entries) + 1, dtype=np.int64)
        offs[1:] = np.cumsum([len(e) for e in entries])
        toks = np.array([t for e in entries for t in e] or [0], dtype=np.int32)
    return _host_i32(toks), np.ascontiguousarray(offs, dtype=np.int64)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError("embedding and hidden states are float32 or bfloat16 (raw 16-bit patterns allowed)")


# --------------------------------------------------------------------------- tries

def trie_build(entries, vocab: int, sep: int, stop: int):
    toks, offs = _catalog_arrays(entries)
    h = C.c_void_p()
    _check(lib().tms_trie_build(toks.ctypes.data, offs.ctypes.data, len(offs) - 1, vocab, sep, stop, C.byref(h)),
           "trie_build")
    return h


def trie_upload(entries, vocab: int, sep: int, stop: int, path: int = PATH_AUTO, stream=None):
    toks, offs = _catalog_arrays(entries)
    h = C.c_void_p()
    _check(lib().tms_trie_upload(toks.ctypes.data, offs.ctypes.data, len(offs) - 1, vocab, sep, stop, path,
                                 _stream(stream), C.byref(h)), "trie_upload")
    return h


def _bytes_arrays(items):
    off = np.zeros(len(items) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(x) for x in items])
    buf = np.frombuffer(b"".join(bytes(x) for x in items) or b"\0", np.uint8).copy()
    return buf, off


def charset_build(strings, vocab, sep: int, stop: int):
    """strings: catalog byte strings; vocab: byte string of every token id."""
    sb, so = _bytes_arrays(strings)
    tb, to = _bytes_arrays(vocab)
    h = C.c_void_p()
    _check(lib().tms_charset_build(sb.ctypes.data, so.ctypes.data, len(strings), tb.ctypes.data, to.ctypes.data,
                                   len(vocab), sep, stop, C.byref(h)), "charset_build")
    return h


def charset_upload(strings, vocab, sep: int, stop: int, path: int = PATH_AUTO, stream=None):
    sb, so = _bytes_arrays(strings)
    tb, to = _bytes_arrays(vocab)
    h = C.c_void_p()
    _check(lib().tms_charset_upload(sb.ctypes.data, so.ctypes.data, len(strings), tb.ctypes.data, to.ctypes.data,
                                    len(vocab), sep, stop, path, _stream(stream), C.byref(h)), "charset_upload")
    return h


def trie_info_get(trie) -> dict:
    info = TrieInfo()
    _check(lib().tms_trie_info_get(trie, C.byref(info)), "trie_info_get")
    return {n: getattr(info, n) for n, _ in TrieInfo._fields_}


def trie_export_csr(trie) -> dict:
    i = trie_info_get(trie)
    out = {"begin": np.zeros(i["n_nodes"] + 1, np.int32), "entry": np.zeros(i["n_nodes"], np.int32),
           "tok": np.zeros(i["n_edges"], np.int32), "child": np.zeros(i["n_edges"], np.int32),
           "live0": np.zeros(i["n_edges"], np.int32)}
    _check(lib().tms_trie_export_csr(trie, *(out[n].ctypes.data for n in ("begin", "entry", "tok", "child",
                                                                            "live0"))), "trie_export_csr")
    return out


def trie_free(trie):
    _check(lib().tms_trie_free(trie), "trie_free")


# --------------------------------------------------------------------------- states

def state_create(trie, B: int, k: int, emb: torch.Tensor, stream=None):
    if emb.dim() != 2:
        raise ValueError("emb must be [V][H]")
    h = C.c_void_p()
    _check(lib().tms_state_create(trie, B, k, _dev(emb, name="emb"), _dtype_code(emb), emb.shape[1],
                                  _stream(stream), C.byref(h)), "state_create")
    return h


def state_reset(st, stream=None):
    _check(lib().tms_state_reset(_handle(st), _stream(stream)), "state_reset")


def state_sync_status(st, B: int, stream=None, check: bool = True) -> np.ndarray:
    out = np.zeros(B, np.int32)
    rc = lib().tms_state_sync_status(_handle(st), out.ctypes.data, _stream(stream))
    if rc not in (OK, ERR_EMPTY_MASK, ERR_NOT_WALKABLE, ERR_NOT_DONE) or (check and rc != OK):
        _check(rc, "state_sync_status")
    return out


def state_export(st, B: int, k: int, n_edges: int, live: bool = False, stream=None) -> dict:
    out = {n: np.zeros(B, np.int32) for n in ("node", "depth", "done", "status", "finished", "n_emitted")}
    out["entries"] = np.zeros((B, k), np.int32)
    lv = np.zeros((B, n_edges), np.int32) if live else None
    _check(lib().tms_state_export(_handle(st), *(out[n].ctypes.data for n in ("node", "depth", "done", "status", "finished",
                                                                      "n_emitted", "entries")),
                                  lv.ctypes.data if live else None, _stream(stream)), "state_export")
    if live:
        out["live"] = lv
    return out


def state_free(st):
    _check(lib().tms_state_free(_handle(st)), "state_free")


def state_set_split(st, split: int):
    _check(lib().tms_state_set_split(_handle(st), split), "state_set_split")


def state_set_loop(st, mode: int):
    _check(lib().tms_state_set_loop(_handle(st), mode), "state_set_loop")


def state_set_norepeat(st, kind: int):
    _check(lib().tms_state_set_norepeat(_handle(st), kind), "state_set_norepeat")


def state_set_step_grouping(st, mode: int):
    _check(lib().tms_state_set_step_grouping(_handle(st), mode), "state_set_step_grouping")


def state_get_launch(st):
    s, g = C.c_int32(), C.c_int32()
    _check(lib().tms_state_get_launch(_handle(st), C.byref(s), C.byref(g)), "state_get_launch")
    return s.value, g.value


# --------------------------------------------------------------------------- decode

_HID = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)


def _handle(st):
    return st.h if isinstance(st, State) else st


def _recording(stream) -> bool:
    """Whether the stream (default: the current one) is being recorded into a
    graph; False for a raw handle, which torch cannot ask about."""
    if stream is None:
        return torch.cuda.is_current_stream_capturing()
    if isinstance(stream, torch.cuda.Stream):
        with torch.cuda.stream(stream):
            return torch.cuda.is_current_stream_capturing()
    return False


def _refuse_check_while_recording(check: bool, stream, where: str):
    """check=True synchronises the stream, which a recording cannot do: refuse
    before anything is recorded, with what to do instead."""
    if check and _recording(stream):
        raise TmsError(ERR_INVALID_ARG, where, "check=True synchronises the stream, which is being recorded into a "
                       "graph: pass check=False and read State.status() after a replay")


def _raise_device_errors(st, stream, where: str):
    """Synchronise the stream and raise TmsError if any sequence of st holds a
    device error; the message names the first such sequence and, for a State,
    lists every sequence's status."""
    B = st.B if isinstance(st, State) else 0
    buf = np.zeros(max(B, 1), np.int32)
    rc = lib().tms_state_sync_status(_handle(st), buf.ctypes.data if B else None, _stream(stream))
    if rc != OK:
        detail = lib().tms_last_error().decode()
        if B:
            bad = {i: int(x) for i, x in enumerate(buf) if x != OK}
            detail += f"; {len(bad)} of {B} sequences in error: {dict(list(bad.items())[:16])}"
        raise TmsError(rc, where, detail)


def decode_step_sparse(st, hidden, tok, logit=None, stream=None, check: bool = True):
    _refuse_check_while_recording(check, stream, "decode_step_sparse")
    _check(lib().tms_decode_step_sparse(_handle(st), _dev(hidden, _HID, "hidden"), _dev(tok, torch.int32, "tok"),
                                        _dev(logit, torch.float32, "logit"), _stream(stream)),
           "decode_step_sparse")
    if check:
        _raise_device_errors(st, stream, "decode_step_sparse")


def decode_step_dense_masked(st, hidden, tok, logit=None, full_logits=None, stream=None, check: bool = True):
    _refuse_check_while_recording(check, stream, "decode_step_dense_masked")
    _check(lib().tms_decode_step_dense_masked(_handle(st), _dev(hidden, _HID, "hidden"),
                                              _dev(tok, torch.int32, "tok"), _dev(logit, torch.float32, "logit"),
                                              _dev(full_logits, torch.float32, "full_logits"), _stream(stream)),
           "decode_step_dense_masked")
    if check:
        _raise_device_errors(st, stream, "decode_step_dense_masked")


def decode_k_pointers(st, hidden_seq, tokens, len=None, entries=None, stream=None, check: bool = True):  # noqa: A002
    _refuse_check_while_recording(check, stream, "decode_k_pointers")
    T = hidden_seq.shape[0]
    _check(lib().tms_decode_k_pointers(_handle(st), _dev(hidden_seq, _HID, "hidden_seq"), T,
                                       _dev(tokens, torch.int32, "tokens"), _dev(len, torch.int32, "len"),
                                       _dev(entries, torch.int32, "entries"), _stream(stream)),
           "decode_k_pointers")
    if check:
        _raise_device_errors(st, stream, "decode_k_pointers")


def decode_k_pointers_noalloc(trie, emb, k: int, hidden_seq, tokens, status, len=None, entries=None,  # noqa: A002
                              stream=None, check: bool = True):
    """One whole answer per sequence with the decode state in the library's
    per-GPU scratch (no state handle, no allocation).  status: dev int32 [B].
    check: synchronise and raise TmsError on any per-sequence device error."""
    T, B, H = hidden_seq.shape
    if emb.dim() != 2 or emb.shape[1] != H:
        raise ValueError("emb must be [V][H] with the hidden size of hidden_seq")
    _refuse_check_while_recording(check, stream, "decode_k_pointers_noalloc")
    _check(lib().tms_decode_k_pointers_noalloc(trie.h if isinstance(trie, Trie) else trie, _dev(emb, name="emb"),
                                               _dtype_code(emb), H, B, k, _dev(hidden_seq, _HID, "hidden_seq"), T,
                                               _dev(tokens, torch.int32, "tokens"), _dev(len, torch.int32, "len"),
                                               _dev(entries, torch.int32, "entries"),
                                               _dev(status, torch.int32, "status"), _stream(stream)),
           "decode_k_pointers_noalloc")
    if check:
        torch.cuda.synchronize()
        bad = status.cpu().numpy()
        if (bad != OK).any():
            first = int(np.nonzero(bad != OK)[0][0])
            raise TmsError(int(bad[first]), "decode_k_pointers_noalloc",
                           f"sequence {first}; {int((bad != OK).sum())} of {B} sequences in error")


def advance_forced(st, tok, stream=None, check: bool = True):
    _refuse_check_while_recording(check, stream, "advance_forced")
    _check(lib().tms_advance_forced(_handle(st), _dev(tok, torch.int32, "tok"), _stream(stream)), "advance_forced")
    if check:
        _raise_device_errors(st, stream, "advance_forced")


def legal_set(st, legal_tok, n_legal, stream=None):
    _check(lib().tms_legal_set(_handle(st), _dev(legal_tok, torch.int32, "legal_tok"), _dev(n_legal, torch.int32, "n_legal"),
                               _stream(stream)), "legal_set")


def legal_mask(st, mask, stream=None):
    _check(lib().tms_legal_mask(_handle(st), _dev(mask, torch.int32, "mask"), _stream(stream)), "legal_mask")


def mask_to_rows(mask, V: int, rows, n_rows, stream=None):
    B, cap = rows.shape
    _check(lib().tms_mask_to_rows(_dev(mask, torch.int32, "mask"), B, V, cap, _dev(rows, torch.int32, "rows"),
                                  _dev(n_rows, torch.int32, "n_rows"), _stream(stream)), "mask_to_rows")


def gather_gemv(emb, hidden, rows, n_rows, out, stream=None):
    B, cap = rows.shape
    _check(lib().tms_gather_gemv(_dev(emb, _HID, "emb"), _dtype_code(emb), emb.shape[0], emb.shape[1],
                                 _dev(hidden, _HID, "hidden"), _dev(rows, torch.int32, "rows"),
                                 _dev(n_rows, torch.int32, "n_rows"), B, cap, _dev(out, torch.float32, "out"),
                                 _stream(stream)), "gather_gemv")


def read_reference(src, out, grid: int = 0, unroll: int = 0, nbytes: int | None = None, stream=None):
    """Streaming read of src (a contiguous GPU tensor; nbytes of it, default
    all) into the XOR words out (int32 [1024]): the bandwidth reference."""
    have = src.numel() * src.element_size()
    n = have if nbytes is None else int(nbytes)
    if n > have:
        raise ValueError(f"read_reference: {n} bytes asked of a {have}-byte tensor")
    if out.numel() < 1024:
        raise ValueError("read_reference: out must hold 1024 words")
    _check(lib().tms_read_reference(_dev(src, name="src"), n, _dev(out, torch.int32, "out"), grid, unroll,
                                    _stream(stream)), "read_reference")


def debug_set_live(st, s: int, edge: int, value: int, stream=None):
    _check(lib().tms_debug_set_live(_handle(st), s, edge, value, _stream(stream)), "debug_set_live")


# --------------------------------------------------------------------------- handles

class Trie:
    """Owning wrapper of a tms_trie handle."""

    def __init__(self, entries, vocab: int, sep: int, stop: int, path: int = PATH_AUTO, upload: bool = True,
                 stream=None, _handle=None):
        if _handle is not None:
            self.h = _handle
        else:
            self.h = trie_upload(entries, vocab, sep, stop, path, stream) if upload else \
                trie_build(entries, vocab, sep, stop)
        self.info = trie_info_get(self.h)

    @classmethod
    def from_charset(cls, strings, vocab, sep: int, stop: int, path: int = PATH_AUTO, upload: bool = True,
                     stream=None):
        """A character-level catalog: byte strings and the byte string of
        every token id (answers pick one string, k = 1)."""
        h = charset_upload(strings, vocab, sep, stop, path, stream) if upload else \
            charset_build(strings, vocab, sep, stop)
        return cls(None, 0, 0, 0, _handle=h)

    def csr(self):
        return trie_export_csr(self.h)

    def close(self):
        if getattr(self, "h", None) is not None:
            trie_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class State:
    """Owning wrapper of a tms_state handle; keeps the embedding tensor alive."""

    def __init__(self, trie: Trie, B: int, k: int, emb: torch.Tensor, stream=None):
        self.trie, self.B, self.k, self.emb = trie, B, k, emb
        self.h = state_create(trie.h, B, k, emb, stream)

    def reset(self, stream=None):
        state_reset(self.h, stream)

    def status(self, stream=None, check: bool = False):
        return state_sync_status(self.h, self.B, stream, check)

    def export(self, live: bool = False, stream=None):
        return state_export(self.h, self.B, self.k, self.trie.info["n_edges"], live, stream)

    def close(self):
        if getattr(self, "h", None) is not None:
            state_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
