"""GPU parity of the character-level catalogs (the review of arXiv
2608.12574): the library compiles byte strings and a byte-string vocabulary
into a trie of per-node valid tokens (tms_charset_upload) and decodes it with
the same kernels as the token catalogs, one string per answer (k = 1).  The
oracle is oracle.CharCatalog (the plain definition of the legal set, no trie,
no matcher).  Comparison rules as in gpu_util.compare: identical tokens,
lengths and chosen strings, no tie-explained flip on the workloads, logits
within tolerance."""
import numpy as np
import pytest
import torch

import oracle
import trie_masked_sparse_amd as tms
from gpu_util import compare, dev_embedding, ref_decode_chars, run_k_pointers, run_step_loop, to_dev
from synth import CHAR_CONFIGS, bf16_bits_from_f32, char_catalog, char_hidden, char_vocab, embedding

from test_charset_oracle import tiny_cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_lib):
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    tms.lib()
    yield
    torch.cuda.synchronize()


def _case(cid, B=None):
    c = CHAR_CONFIGS[cid]
    strings, vocab = char_catalog(cid), char_vocab(cid)
    cc = oracle.CharCatalog(strings, vocab, c.sep, c.stop)
    T = cc.max_len + 1
    hid = char_hidden(cid, T, B)
    return c, strings, vocab, cc, T, hid


@pytest.mark.parametrize("cid", sorted(CHAR_CONFIGS))
def test_charset_workload_parity(cid):
    """Full size (V = 151936, H = 2048 bf16, B = 64): the resident loop
    (grouped root head: matrix cores, tie depth H + 1) and the host-driven
    fused step (per-row order, logits checked), every sequence against the
    oracle."""
    c, strings, vocab, cc, T, hid = _case(cid)
    trie = tms.Trie.from_charset(strings, vocab, c.sep, c.stop)
    assert trie.info["path"] == tms.PATH_GLOBAL  # roots of hundreds to thousands of valid tokens
    emb = dev_embedding(c.emb_cid)
    st = tms.State(trie, c.batch, 1, emb)
    hd = to_dev(hid)
    ref = ref_decode_chars(cc, embedding(c.emb_cid), hid)
    assert (ref["status"] == 0).all()
    tok, ln, ent = run_k_pointers(st, hd)
    flips = compare(tok, ref, c.hidden, None, ln, ent, where=cid, depth=c.hidden + 1)
    st.reset()
    tok_h, lg_h = run_step_loop(st, hd)
    compare(tok_h, ref, c.hidden, lg_h, where=cid + "/step")
    # every shared node grouped (wide nodes of hundreds of valid tokens, read
    # once per step for the sequences standing there): bit for bit the same,
    # host-driven and in the graph of step kernels
    tms.state_set_step_grouping(st, tms.STEP_GROUP_NODES)
    st.reset()
    tok_g, lg_g = run_step_loop(st, hd)
    assert np.array_equal(tok_g, tok_h) and np.array_equal(lg_g, lg_h, equal_nan=True)
    tms.state_set_loop(st, tms.LOOP_GRAPH)
    st.reset()
    tok_gg, ln_gg, ent_gg = run_k_pointers(st, hd)
    assert np.array_equal(tok_gg, tok_h) and np.array_equal(ent_gg, ent)
    tms.state_set_loop(st, tms.LOOP_RESIDENT)
    # every answer is a catalog string, spelled by its tokens
    for b in range(c.batch):
        spelled = b"".join(vocab[t] for t in tok_h[b] if t >= 0 and t != c.stop)
        assert spelled == strings[ent[b, 0]]
    print(f"{cid}: nodes={trie.info['n_nodes']} edges={trie.info['n_edges']} root cap={trie.info['cap']} "
          f"tokens={int(ln.sum())} tie flips={flips}")
    st.close()
    trie.close()


@pytest.mark.parametrize("path", [tms.PATH_FAST, tms.PATH_GLOBAL])
def test_charset_tiny_catalogs(path):
    """Every tiny catalog of the oracle's pins (prefix pairs, both control-id
    placements), fp32 and bf16, through every loop form and the step."""
    rng = np.random.Generator(np.random.PCG64(61 + path))
    for i, (strings, vocab, sep, stop) in enumerate(tiny_cases()):
        cc = oracle.CharCatalog(strings, vocab, sep, stop)
        V, B, H = len(vocab), 5, 64 if i % 2 else 96
        T = cc.max_len + 1
        x = rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.2)
        h = rng.standard_normal((T, B, H), dtype=np.float32)
        emb, hid = (bf16_bits_from_f32(x), bf16_bits_from_f32(h)) if i % 2 else (x, h)
        trie = tms.Trie.from_charset(strings, vocab, sep, stop, path=path)
        st = tms.State(trie, B, 1, to_dev(emb))
        ref = ref_decode_chars(cc, emb, hid)
        hd = to_dev(hid)
        for mode in (tms.LOOP_RESIDENT_SOLO, tms.LOOP_RESIDENT_GROUPED, tms.LOOP_GRAPH, tms.LOOP_STREAM):
            tms.state_set_loop(st, mode)
            st.reset()
            tok, ln, ent = run_k_pointers(st, hd)
            compare(tok, ref, H, None, ln, ent, where=f"tiny {i} mode {mode}", depth=H + 1)
        st.reset()
        tok, lg = run_step_loop(st, hd)
        compare(tok, ref, H, lg, where=f"tiny {i} step")
        st.close()
        trie.close()


def test_charset_dense_matches_sparse():
    """Dense head plus the vocabulary mask on a character catalog: the vector
    head (B = 1) is bit-identical to the sparse step."""
    c, strings, vocab, cc, T, hid = _case("charset_tools", B=1)
    trie = tms.Trie.from_charset(strings, vocab, c.sep, c.stop)
    st = tms.State(trie, 1, 1, dev_embedding(c.emb_cid))
    hd = to_dev(hid)
    s_tok, s_lg = run_step_loop(st, hd)
    st.reset()
    d_tok, d_lg = run_step_loop(st, hd, dense=True)
    assert np.array_equal(s_tok, d_tok) and np.array_equal(s_lg, d_lg, equal_nan=True)
    compare(d_tok, ref_decode_chars(cc, embedding(c.emb_cid), hid), c.hidden, d_lg, where="charset dense")
    st.close()
    trie.close()


def test_charset_errors_and_state():
    """One string per answer: k != 1 is refused; a reset after a decode leaves
    the live rows untouched (nothing is released) and a repeat decode equal."""
    c, strings, vocab, cc, T, hid = _case("charset_tools", B=4)
    trie = tms.Trie.from_charset(strings, vocab, c.sep, c.stop)
    emb = dev_embedding(c.emb_cid)
    with pytest.raises(tms.TmsError) as ei:
        tms.State(trie, 4, 2, emb)
    assert ei.value.code == tms.ERR_K
    st = tms.State(trie, 4, 1, emb)
    fresh = st.export(live=True)
    hd = to_dev(hid)
    r0 = run_k_pointers(st, hd)
    ex = st.export(live=True)
    assert np.array_equal(ex["live"], fresh["live"]) and (ex["finished"] == 1).all()
    st.reset()
    r1 = run_k_pointers(st, hd)
    assert all(np.array_equal(a, b) for a, b in zip(r0, r1))
    st.close()
    trie.close()
