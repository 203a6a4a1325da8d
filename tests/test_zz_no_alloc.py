"""The allocation-free decode entry point (tms_decode_k_pointers_noalloc)
against the state-based one (tms_state_create + tms_decode_k_pointers from a
reset state): the same kernels, so tokens, lengths, entries and statuses must
be bit-identical.  Two calls in a row on one GPU, the second with a smaller
batch and another catalog, so the second runs on scratch the first left
behind; the device memory in use does not change across a call; a batch whose
state exceeds the scratch limit is refused before anything is launched."""
import numpy as np
import pytest
import torch

import trie_masked_sparse_amd as tms
from gpu_util import compare, config_case, dev_embedding, ref_decode, to_dev
from synth import catalog, embedding

pytestmark = pytest.mark.gpu


def _state_based(trie, cid, B, k, hd):
    st = tms.State(trie, B, k, dev_embedding(cid))
    T = hd.shape[0]
    tok = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    ln = torch.zeros(B, dtype=torch.int32, device="cuda")
    ent = torch.zeros((B, k), dtype=torch.int32, device="cuda")
    tms.decode_k_pointers(st, hd, tok, ln, ent, check=False)
    status = st.status()
    st.close()
    return tok.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy(), status


def _noalloc(trie, cid, B, k, hd):
    T = hd.shape[0]
    tok = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    ln = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ent = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    status = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    emb = dev_embedding(cid)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    tms.decode_k_pointers_noalloc(trie, emb, k, hd, tok, status, ln, ent, check=False)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return (tok.cpu().numpy(), ln.cpu().numpy(), ent.cpu().numpy(), status.cpu().numpy()), free0 - free1


def test_noalloc_matches_state_entry_point():
    # first call: the unstructured workload (global trie, grouped root heads);
    # second: a smaller batch of the structured one (trie image in LDS);
    # third: smaller again (tiny, fp32), after the two above
    for i, (cid, B) in enumerate((("unstructured", 64), ("structured", 16), ("tiny", 3))):
        c, otr, T, hid = config_case(cid, B=B)
        print(f"noalloc call {i}: {cid} B={B}", flush=True)
        trie = tms.Trie(catalog(cid), c.vocab, c.sep, c.stop)
        hd = to_dev(hid)
        if i == 0:  # the first use on this GPU takes the scratch address
            _noalloc(trie, cid, B, c.k, hd)
        got, used = _noalloc(trie, cid, B, c.k, hd)
        want = _state_based(trie, cid, B, c.k, hd)
        for name, a, b in zip(("tokens", "len", "entries", "status"), got, want):
            assert np.array_equal(a, b), (cid, name)
        assert (got[3] == tms.OK).all()
        assert used == 0, f"{cid}: device memory in use grew by {used} bytes during the call"
        compare(got[0], ref_decode(otr, c.k, embedding(cid), hid), c.hidden, None, got[1], got[2],
                where=f"noalloc {cid}")
        trie.close()


def test_noalloc_refuses_oversized_batch():
    c, otr, T, _ = config_case("large", B=1)
    trie = tms.Trie(catalog("large"), c.vocab, c.sep, c.stop)
    B = 256  # 256 rows of ~530k live counts: far above the scratch limit
    hd = torch.zeros((T, B, c.hidden), dtype=torch.bfloat16, device="cuda")
    tok = torch.empty((B, T), dtype=torch.int32, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    with pytest.raises(tms.TmsError) as ei:
        tms.decode_k_pointers_noalloc(trie, dev_embedding("large"), c.k, hd, tok, status)
    assert ei.value.code == tms.ERR_INVALID_ARG and "allocation-free limit" in str(ei.value)
    trie.close()


def test_noalloc_status_and_host_checks():
    """status is the call's only error report: it is overwritten for every
    sequence (all OK on a valid batch); too few steps are refused on the host
    before anything is launched."""
    c, otr, T, hid = config_case("tiny", B=2)
    trie = tms.Trie(catalog("tiny"), c.vocab, c.sep, c.stop)
    hd = to_dev(hid)
    tok = torch.empty((2, T - 1), dtype=torch.int32, device="cuda")
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(tms.TmsError) as ei:
        tms.decode_k_pointers_noalloc(trie, dev_embedding("tiny"), c.k, hd[: T - 1].contiguous(), tok, status)
    assert ei.value.code == tms.ERR_INVALID_ARG
    assert (status.cpu().numpy() == -7).all()
    tok = torch.empty((2, T), dtype=torch.int32, device="cuda")
    tms.decode_k_pointers_noalloc(trie, dev_embedding("tiny"), c.k, hd, tok, status)
    assert (status.cpu().numpy() == tms.OK).all()
    trie.close()
