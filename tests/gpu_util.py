"""Shared helpers for the GPU parity tests: seeded inputs on the device and the
comparison rules against the oracle.

Comparison rules (fp32 accumulation on the GPU, fp64 in the oracle):
  * tokens must be identical.  The only allowed difference is a numerical tie:
    a step where the GPU's token g is legal (in the oracle's mask at the GPU's
    own prefix) and its exact logit is within the worst-case fp32 error of the
    kernel's declared summation order of the best one,
        best - logit(g) <= 2 * gamma_d * max(sum|p| of the top two, sum|p| of g),
    gamma_d = d u / (1 - d u), u = 2^-24, d the summation depth (per-lane
    chains of ceil(H/64) roundings then a 6-level butterfly for the vector
    kernels: d = ceil(H/64) + 6; H + 1 for the matrix cores, whose order is the
    hardware's).  After such a flip the oracle is teacher-forced along the
    GPU's tokens ("Understanding Inference for Systems Engineers", Part 8
    "Correctness") and the rest of the sequence is still compared step by
    step, lengths and entries included.  Flips are counted; a comparison
    allows none unless the caller states a bound;
  * a logit must satisfy |l_gpu - l_ref| <= 2e-3 |l_ref| + gamma_{H+1} sum|p|,
    the stated relative tolerance plus the any-order fp32 summation bound so
    that near-zero logits do not fail the relative test.
"""
from __future__ import annotations

import functools
import math
import warnings

import numpy as np
import torch

import oracle
import trie_masked_sparse_amd as tms
from synth import CONFIGS, catalog, embedding, hidden_states

U32 = 2.0 ** -24


def gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def tree_depth(H: int) -> int:
    return math.ceil(H / 64) + 6


def to_dev(a: np.ndarray) -> torch.Tensor:
    # cached inputs are read-only arrays; the host tensor wrapping them is only
    # copied to the device, never written, so torch's warning about that is moot
    with warnings.catch_warnings():
        warnings.filterwarnings("ignore", message="The given NumPy array is not writable")
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@functools.lru_cache(maxsize=2)
def dev_embedding(cid: str) -> torch.Tensor:
    return to_dev(embedding(cid))


@functools.lru_cache(maxsize=8)
def oracle_trie(cid: str) -> oracle.Trie:
    c = CONFIGS[cid]
    return oracle.Trie(catalog(cid), c.vocab, c.sep, c.stop)


def run_k_pointers(state: tms.State, hid_dev: torch.Tensor, check: bool = True):
    T, B = hid_dev.shape[0], hid_dev.shape[1]
    tokens = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    ln = torch.zeros(B, dtype=torch.int32, device="cuda")
    ent = torch.zeros((B, state.k), dtype=torch.int32, device="cuda")
    tms.decode_k_pointers(state, hid_dev, tokens, ln, ent, check=check)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy()


def run_step_loop(state: tms.State, hid_dev: torch.Tensor, dense: bool = False, full=None, check: bool = True,
                  logits: bool = True):
    """T host-driven steps; returns tokens [B][T] and winner logits [B][T]
    (NaN throughout when logits=False: the steps are asked for tokens only)."""
    T, B = hid_dev.shape[0], hid_dev.shape[1]
    toks = torch.empty((T, B), dtype=torch.int32, device="cuda")
    lg = torch.full((T, B), float("nan"), dtype=torch.float32, device="cuda")
    for t in range(T):
        if dense:
            tms.decode_step_dense_masked(state, hid_dev[t], toks[t], lg[t], None if full is None else full[t],
                                         check=check)
        else:
            tms.decode_step_sparse(state, hid_dev[t], toks[t], lg[t] if logits else None, check=check)
    torch.cuda.synchronize()
    return toks.cpu().numpy().T.copy(), lg.cpu().numpy().T.copy()


def ref_decode(otr: oracle.Trie, k: int, emb: np.ndarray, hid: np.ndarray):
    """The oracle's greedy decode, keeping what compare() needs to
    teacher-force it along the GPU's tokens after a numerical-tie flip."""
    ref = oracle.decode(otr, k, emb, hid)
    ref["_emb"], ref["_hid"] = emb, hid
    ref["_follow"] = lambda b, row: oracle.decode(otr, k, emb, np.ascontiguousarray(hid[:, b:b + 1]),
                                                  follow=np.ascontiguousarray(row))
    return ref


def ref_decode_chars(cc: oracle.CharCatalog, emb: np.ndarray, hid: np.ndarray):
    """The same for a character catalog (one string per answer: entries [B][1])."""
    def as_ref(out):
        out["entries"] = out["entry"][:, None].copy()
        return out
    ref = as_ref(cc.decode(emb, hid))
    ref["_emb"], ref["_hid"] = emb, hid
    ref["_follow"] = lambda b, row: as_ref(cc.decode(emb, np.ascontiguousarray(hid[:, b:b + 1]),
                                                     follow=np.ascontiguousarray(row)))
    return ref


def compare(gpu_tokens, ref, H, gpu_logits=None, gpu_len=None, gpu_entries=None, where="", depth=None,
            max_flips=0):
    """Apply the comparison rules; returns the list of tie-explained flips
    (sequence, step, gpu token, oracle token, oracle margin, bound).
    depth: summation depth behind the tie bound (default: the vector kernels'
    declared tree).  max_flips: how many flips the caller allows (default none).
    ref must come from ref_decode when any flip is to be excused."""
    B, T = ref["tokens"].shape
    d = tree_depth(H) if depth is None else depth
    flips = []
    for b in range(B):
        cur, row = ref, b          # switches to the teacher-forced run after a flip
        for t in range(T):
            g, r = int(gpu_tokens[b, t]), int(cur["tokens"][row, t])
            if g != r:
                assert r >= 0 and g >= 0, f"{where} seq {b} step {t}: gpu token {g}, oracle {r}"
                assert "_follow" in ref, f"{where} seq {b} step {t}: gpu token {g}, oracle {r} (no oracle inputs)"
                emb, hid = ref["_emb"], ref["_hid"]
                if cur is ref:
                    cur = ref["_follow"](b, gpu_tokens[b:b + 1, :T])
                    row = 0
                    assert int(cur["tokens"][0, t]) == r  # same prefix, same pick
                lg, ag = oracle.logit(emb, g, hid[t, b])
                best, sa = float(cur["best"][row, t]), float(cur["sumabs"][row, t])
                bound = 2 * gamma(d) * max(sa, ag)
                assert best - lg <= bound, (
                    f"{where} seq {b} step {t}: gpu token {g} (oracle logit {lg:.6e}), oracle {r} "
                    f"(best {best:.6e}, margin {cur['margin'][row, t]:.3e}) beyond the tie bound {bound:.3e}")
                flips.append((b, t, g, r, float(cur["margin"][row, t]), float(bound)))
                if gpu_logits is not None:
                    tol = 2e-3 * abs(lg) + gamma(H + 1) * ag
                    assert abs(float(gpu_logits[b, t]) - lg) <= tol, (where, b, t)
                continue
            if gpu_logits is not None and r >= 0:
                ref_l = cur["best"][row, t]
                tol = 2e-3 * abs(ref_l) + gamma(H + 1) * cur["sumabs"][row, t]
                assert abs(float(gpu_logits[b, t]) - ref_l) <= tol, (
                    f"{where} seq {b} step {t}: logit {gpu_logits[b, t]!r} vs oracle {ref_l!r} (tol {tol:.3e})")
            if gpu_logits is not None and r < 0:
                assert math.isnan(float(gpu_logits[b, t]))
        if cur is not ref:
            # every GPU token was legal where it was taken
            assert cur["status"][0] in (oracle.OK, oracle.ERR_NOT_DONE), (where, b, int(cur["status"][0]))
            assert cur["status"][0] == ref["status"][b], (where, b)
        if gpu_len is not None:
            assert gpu_len[b] == cur["len"][row], (where, b)
        if gpu_entries is not None:
            assert list(gpu_entries[b]) == list(cur["entries"][row]), (where, b)
    assert len(flips) <= max_flips, f"{where}: {len(flips)} tie-explained flips (allowed {max_flips}): {flips[:8]}"
    return flips


def config_case(cid: str, B: int | None = None, seqs=None, T: int | None = None):
    """(config, catalog, trie info from oracle, hidden numpy [T][B][H])."""
    c = CONFIGS[cid]
    otr = oracle_trie(cid)
    T = c.k * (otr.max_depth + 1) if T is None else T
    hid = hidden_states(cid, T, B)
    return c, otr, T, hid
