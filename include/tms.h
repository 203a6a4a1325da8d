/*
 * tms.h - trie-constrained sparse decode step for finite-set outputs (tool
 * catalogs), MI355X (gfx950) HIP library with a plain C ABI.
 *
 * The method (web page "Constraint made cheaper than no constraint"):
 *   - section "The grammar as a trie over tokens": a catalog of token-id
 *     strings is compiled into a trie in CSR form with sentinel children for a
 *     separator edge and a stop edge;
 *   - section "Masked sampling inside the sampler": each step builds the legal
 *     set at the current node, takes the argmax with ties to the lower token
 *     id, fails loudly on an empty mask or an unwalkable winner, and advances;
 *     exactly k pointers come out because sep is legal only while another
 *     pointer is owed and stop only when none is; live counts per edge,
 *     decremented along a completed pointer's path, keep pointers from
 *     repeating; a per-terminal spent flag handles entries that are prefixes
 *     of other entries;
 *   - section "The sparse output layer": the head computes one dot product per
 *     legal token against the tied embedding instead of all V logits; the
 *     dense head stays as a cross-check with the same tie rule and transitions;
 *   - section "The whole loop on the device": the decode loop runs without the
 *     host between steps.
 * The mask semantics are Mask(u) = {v : some w makes u v w an answer} (page
 * "GLRMask - constrained decoding with weighted automata", the next-token
 * mask), and the greedy tie rule is the one of page "Understanding Inference
 * for Systems Engineers", section 3.8.
 *
 * Conventions for every call:
 *   - Every function returns a tms_status and never throws.  On failure
 *     tms_last_error() gives a thread-local message.
 *   - "dev" pointers are device memory owned by the caller (for example
 *     torch.Tensor.data_ptr()); "host" pointers are host memory owned by the
 *     caller.  The library never frees caller memory.
 *   - stream is a hipStream_t (NULL = the legacy default stream).  Decode
 *     calls only enqueue work on it and return; they allocate nothing (the
 *     GRAPH loop form instantiates its graph on its first call for a step
 *     count, and waits for the device when it is called with new buffers).
 *   - Device-detected errors (EMPTY_MASK, NOT_WALKABLE, NOT_DONE) are recorded
 *     per sequence and are sticky: that sequence stops, the others continue.
 *     tms_state_sync_status() synchronises the stream and reports them.
 *   - Element type of the embedding and of every hidden-state buffer: fp32, or
 *     bf16 as raw 16-bit patterns.  Products and sums are fp32.
 *   - Rows must be 16-byte aligned: H*elem_size % 16 == 0 and the embedding and
 *     hidden base pointers 16-byte aligned.  H <= 8192 (bf16) or 4096 (fp32).
 */
#ifndef TMS_H
#define TMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TMS_OK = 0,
  TMS_ERR_INVALID_ARG = 1,  /* bad pointer, size, alignment or dtype */
  TMS_ERR_CATALOG = 2,      /* empty entry, token outside [0,V), control token inside an entry, duplicate */
  TMS_ERR_FANOUT = 3,       /* fast path forced on a trie whose widest node has more than 256 edges */
  TMS_ERR_K = 4,            /* k outside [1, K] */
  TMS_ERR_EMPTY_MASK = 5,   /* device: a step found no legal token */
  TMS_ERR_NOT_WALKABLE = 6, /* device: the chosen or forced token is not a live edge of the node */
  TMS_ERR_NOT_DONE = 7,     /* device: no stop token within the steps given */
  TMS_ERR_BUSY = 8,         /* trie freed while states still use it */
  TMS_ERR_OOM = 9,          /* device allocation failed */
  TMS_ERR_HIP = 10          /* any other HIP runtime failure (no device, launch failure, ...) */
} tms_status;

typedef enum { TMS_F32 = 0, TMS_BF16 = 1 } tms_dtype;

/* Trie store path.  FAST: every node has at most 256 edges and the hot CSR
 * arrays (begin, tok, child) fit in 64 KiB; the step reads edge records with
 * wave-uniform scalar loads (the MI355X stand-in for the constant-memory trie of
 * section "The grammar as a trie over tokens").  GLOBAL: any fan-out; edge records are
 * read with per-lane vector loads in batches of 64 per wavefront.  AUTO picks
 * FAST when both FAST conditions hold.  Both paths give bit-identical results. */
typedef enum { TMS_PATH_AUTO = 0, TMS_PATH_FAST = 1, TMS_PATH_GLOBAL = 2 } tms_path;

typedef struct tms_trie tms_trie;
typedef struct tms_state tms_state;

typedef struct {
  int32_t n_nodes, n_edges, n_entries;
  int32_t cap;        /* widest node's edge count, control edges included */
  int32_t max_depth;  /* longest entry, in tokens */
  int32_t sep, stop, vocab;
  int32_t path;       /* TMS_PATH_FAST or TMS_PATH_GLOBAL once uploaded, TMS_PATH_AUTO for a host-only trie */
  int64_t device_bytes;
} tms_trie_info;

/* ---------------------------------------------------------------- tries -- */

/* Compile a catalog on the host only (no device memory; usable without a GPU).
 * tokens: host int32 [offsets[K]]; offsets: host int64 [K+1], offsets[0] = 0,
 * entry i is tokens[offsets[i] .. offsets[i+1]).  sep and stop are two distinct
 * ids in [0, vocab) that no entry may contain.  Errors: INVALID_ARG, CATALOG.
 * Canonical CSR: nodes numbered breadth first from root 0, children in
 * ascending token order; a node's edge range holds its content edges and, for
 * a terminal, the sep and stop edges, all in ascending token order; control
 * edges have child -1 (sep) or -2 (stop); live0 of a content edge is the
 * number of entries whose string passes through it, 0 for control edges. */
tms_status tms_trie_build(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab,
                          int32_t sep, int32_t stop, tms_trie** out);

/* tms_trie_build plus a device copy owned by the handle (allocated and copied
 * on `stream`, which is synchronised before returning).  path selects the
 * store layout; FAST on a trie with cap > 256 is TMS_ERR_FANOUT. */
tms_status tms_trie_upload(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab,
                           int32_t sep, int32_t stop, tms_path path, void* stream, tms_trie** out);

/* Character-level catalogs (the review of arXiv 2608.12574, fields
 * pith_extraction.key_machinery and core_discovery): the catalog is K byte
 * strings (bytes [offsets[K]], offsets [K+1], string i = bytes[offsets[i] ..
 * offsets[i+1])) and the vocabulary gives each of the V token ids a byte
 * string (token_bytes / token_offsets alike; an empty string marks a control
 * or unused token).  An answer is one catalog string spelled by tokens,
 * then stop.  The compiler builds a trie over the strings' bytes and, with
 * one Aho-Corasick automaton over the vocabulary's byte strings carried along
 * a walk of the trie, every node's set of tokens whose bytes can be read
 * downward from it; the result is a trie of the same form as the token
 * catalogs' (nodes = the byte trie's, breadth first; a node's edges = its
 * valid tokens in ascending id order, each leading to the node where the
 * token ends; sep and stop edges where a string ends), decoded by every call
 * below with k = 1 (TMS_ERR_K otherwise).  Every byte that occurs in a string
 * must be spelled by a single-byte token (as in byte-level vocabularies), so
 * that every legal token leaves a remainder that can be spelled.  Errors:
 * INVALID_ARG (sizes, control ids), CATALOG (empty or duplicate string, a
 * byte with no single-byte token).  Host arrays, caller-owned. */
tms_status tms_charset_build(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                             const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, tms_trie** out);
/* tms_charset_build plus the device copy, as tms_trie_upload. */
tms_status tms_charset_upload(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                              const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, tms_path path,
                              void* stream, tms_trie** out);

tms_status tms_trie_info_get(const tms_trie* trie, tms_trie_info* info);

/* Copy the canonical CSR to host arrays sized from tms_trie_info:
 * begin [n_nodes+1], entry [n_nodes], tok/child/live0 [n_edges].  NULL skips. */
tms_status tms_trie_export_csr(const tms_trie* trie, int32_t* begin, int32_t* entry, int32_t* tok,
                               int32_t* child, int32_t* live0);

/* Free a trie.  TMS_ERR_BUSY (and nothing freed) while a state uses it. */
tms_status tms_trie_free(tms_trie* trie);

/* --------------------------------------------------------------- states -- */

/* Decode state for B sequences that each must emit exactly k distinct
 * catalog entries.  emb: dev [V][H] tied embedding (V = trie vocab), dtype
 * fp32 or bf16, kept by pointer (caller keeps it alive).  Allocates all device
 * memory the decode calls will need (per-sequence live counts [B][E], spent
 * flags, path stack, argmax slots) and leaves the state reset.
 * Errors: INVALID_ARG (upload-less trie, bad sizes, alignment), K, OOM, HIP. */
tms_status tms_state_create(tms_trie* trie, int32_t B, int32_t k, const void* emb, tms_dtype dtype,
                            int32_t H, void* stream, tms_state** out);

/* Every sequence back to the root: live = live0, spent cleared, no pointers
 * done, status OK, nothing emitted.  The reset is deferred: the next call on
 * st carries it out on that call's stream before its own work (the resident
 * device loop of tms_decode_k_pointers does it inside its kernel; every other
 * call enqueues a reset kernel first, no memset).  stream is not used.
 * Cost: a completed pointer only ever lowers the live counts on its entry's
 * root path (section "Masked sampling inside the sampler" of the page above),
 * so the reset of a decoded state rewrites just those edges from live0 and
 * clears just those spent words; whole rows are rewritten on a new state and
 * after tms_debug_set_live. */
tms_status tms_state_reset(tms_state* st, void* stream);

/* Synchronise stream, copy per-sequence status to host_status [B] (may be
 * NULL) and return the status of the lowest-numbered sequence in error, or
 * TMS_OK. */
tms_status tms_state_sync_status(tms_state* st, int32_t* host_status, void* stream);

/* Copy the state to host arrays after synchronising stream (tests/debug).
 * node, depth, done, status, finished, n_emitted: [B]; entries: [B][k] (-1 for
 * pointers not yet done); live: [B][n_edges] (may be NULL). */
tms_status tms_state_export(tms_state* st, int32_t* node, int32_t* depth, int32_t* done,
                            int32_t* status, int32_t* finished, int32_t* n_emitted,
                            int32_t* entries, int32_t* live, void* stream);

tms_status tms_state_free(tms_state* st);

/* --------------------------------------------------------------- decode -- */

/* One decode step for all B sequences (section "The sparse output layer").
 * hidden: dev [B][H] (state dtype).  For each active sequence s: legal set at
 * its node, logit = sum_i hidden[s][i]*emb[v][i] in fp32 for each legal v,
 * argmax with ties to the lower token id, advance.  Outputs: tok dev int32 [B]
 * (the emitted token, -1 if s was inactive or failed), logit dev fp32 [B] or
 * NULL (the winner's logit, NaN when nothing was emitted).  With logit NULL, a
 * step whose legal set the node alone decides (a node with one edge; a leaf
 * terminal, where sep or stop is the one legal token) takes that token
 * without computing logits (sections "Masked sampling inside the sampler"
 * and "The sparse output layer": the argmax over one legal token is that
 * token); tokens and state are the same either way.
 * One fused kernel; fixed grid per state, so it can be graph-captured.  With
 * the root or node grouping on, a step recorded into a caller's graph is
 * preceded by a snapshot kernel of the sequences' nodes, so that each replay
 * reads the nodes it starts from. */
tms_status tms_decode_step_sparse(tms_state* st, const void* hidden, int32_t* tok, float* logit,
                                  void* stream);

/* The same step computed the post-logit way (cross-check; section "Masked
 * sampling inside the sampler", and section 3.8 "The head: from hidden state
 * to token" of "Understanding Inference for Systems Engineers"): all V
 * logits, illegal tokens masked out, full-vocabulary argmax with the same tie
 * rule, same advance.  full_logits: dev fp32 [B][V] or NULL (written
 * unmasked).  One sequence, or fp32 tables, use the sparse head's per-row
 * arithmetic (bit-identical logits); bf16 with B > 1 runs on the matrix
 * cores, whose summation order differs, so logits agree with the sparse
 * head's within the any-order rounding bound and the argmax can differ only
 * where two logits are within it.  Errors as for tms_decode_step_sparse. */
tms_status tms_decode_step_dense_masked(tms_state* st, const void* hidden, int32_t* tok, float* logit,
                                        float* full_logits, void* stream);

/* The device-resident loop (section "The whole loop on the device"): T sparse
 * steps from the current state with no host work in between.  By default one
 * kernel runs the whole loop with one workgroup per sequence (state kept on
 * chip between steps), or, for B >= 8 and a root of at least 64 edges, one
 * grouped root head plus one such kernel per pointer; see tms_state_set_loop
 * for the other forms.  hidden_seq: dev
 * [T][B][H], step t uses hidden_seq[t].  Outputs: tokens dev int32 [B][T]
 * (token of step t, -1 where a sequence was inactive), len dev int32 [B]
 * (tokens emitted since the last reset), entries dev int32 [B][k] (catalog
 * index of each completed pointer, -1 if missing).  Sequences still unfinished
 * after T steps get NOT_DONE.  T must be >= k*(max_depth+1) (INVALID_ARG).
 * Bit-identical to T calls of tms_decode_step_sparse, except that a grouped
 * root head on the matrix cores (bf16, H = 2048 or 4096) sums the root steps'
 * logits in the matrix cores' order: the same tokens unless two root logits
 * are closer than that order's rounding. */
tms_status tms_decode_k_pointers(tms_state* st, const void* hidden_seq, int32_t T, int32_t* tokens,
                                 int32_t* len, int32_t* entries, void* stream);

/* Teacher forcing: advance sequence s by token tok[s] (dev int32 [B]); tok[s] <
 * 0 leaves s unchanged.  A token that is not a legal edge of the current node
 * sets NOT_WALKABLE for that sequence. */
tms_status tms_advance_forced(tms_state* st, const int32_t* tok, void* stream);

/* The legal set of every sequence at its current node (the materialiser on
 * its own).  legal_tok: dev int32 [B][cap] (cap from tms_trie_info), ascending
 * token order; n_legal: dev int32 [B], -1 for an inactive sequence. */
tms_status tms_legal_set(tms_state* st, int32_t* legal_tok, int32_t* n_legal, void* stream);

/* The legal set of every sequence as a vocabulary bitmask ("Understanding
 * Inference for Systems Engineers", Part 7's masked head; the next-token mask
 * of "GLRMask"): mask dev uint32 [B][ceil(V/32)], bit t of sequence s set iff
 * token t is legal; all zero for an inactive sequence.  V up to 2^19 (one mask in 64 KiB). */
tms_status tms_legal_mask(tms_state* st, uint32_t* mask, void* stream);

/* Bitmask-fed materialiser (same page, Part 7: a popcount scan over the V/32
 * words gives the sorted row list the head then reads): for each of B rows of
 * mask (dev uint32 [B][ceil(V/32)], bits at or past V ignored), rows[s][j] =
 * the j-th set bit's token id in ascending order for j < min(n, cap), and
 * n_rows[s] = n, the number of set bits (which may exceed cap; slots past n
 * are not written).  rows dev int32 [B][cap]; n_rows dev int32 [B].  Feeds
 * tms_gather_gemv directly.  V up to 2^19 (INVALID_ARG above). */
tms_status tms_mask_to_rows(const uint32_t* mask, int32_t B, int32_t V, int32_t cap, int32_t* rows,
                            int32_t* n_rows, void* stream);

/* The sparse head on its own (a gather-GEMV over explicit row lists, as for a
 * restricted vocabulary projection): out[s][j] = sum_i hidden[s][i] *
 * emb[rows[s][j]][i] for j < min(n_rows[s], cap), same fp32 arithmetic and
 * summation order as the decode step.  emb dev [V][H]; hidden dev [B][H];
 * rows dev int32 [B][cap]; n_rows dev int32 [B]; out dev fp32 [B][cap].  Row
 * ids outside [0, V) give NaN and are not read.  Slots j >= n_rows[s] are not
 * written. */
tms_status tms_gather_gemv(const void* emb, tms_dtype dtype, int32_t V, int32_t H, const void* hidden,
                           const int32_t* rows, const int32_t* n_rows, int32_t B, int32_t cap,
                           float* out, void* stream);

/* Measurement reference, not part of the decode path: a plain streaming read
 * of `bytes` (a positive multiple of 16) of device memory at src, the kernel
 * the sparse head's achieved bandwidth is compared with ("Understanding
 * Inference for Systems Engineers", Part 9 "Profiling": bandwidth against a
 * measured plain streaming kernel).  Each wavefront XORs what it read into
 * one word of out (dev uint32 [1024], caller-owned), so the loads cannot be
 * dropped.  grid:
 * workgroups of 256 threads (0: enough for one pass); unroll: loads in flight
 * per thread, 1, 2, 4 or 8 (0: 4).  Errors: INVALID_ARG, HIP. */
tms_status tms_read_reference(const void* src, int64_t bytes, uint32_t* out, int32_t grid, int32_t unroll,
                              void* stream);

/* Negative tests: set live[s][edge] = value on the device. */
tms_status tms_debug_set_live(tms_state* st, int32_t s, int32_t edge, int32_t value, void* stream);

/* Tuning knob (also read from the TMS_SPLIT environment variable at create):
 * workgroups per sequence in the fused step; 0 restores the default.
 * This setter, tms_state_set_loop and tms_state_set_step_grouping discard the
 * GRAPH form's instantiated graph, if there is one, after waiting for the
 * device to finish (a replay of it may still be queued). */
tms_status tms_state_set_split(tms_state* st, int32_t split);

/* How tms_decode_k_pointers runs its T steps (all bit-identical, up to the
 * matrix-core root head noted at tms_decode_k_pointers):
 * RESIDENT_SOLO: one launch, one workgroup per sequence loops over the steps;
 * RESIDENT_GROUPED: one phase per pointer; each phase first takes the root
 *   step of every sequence standing at the root in one grouped launch (each
 *   root row read once for all of them, "The batched engine"), then runs the
 *   resident loop until each sequence is back at the root (the last phase
 *   runs to the end): 2k launches from a reset state, 2(k+1) otherwise;
 * RESIDENT: GROUPED when B >= 8 and the root has at least 64 edges, else SOLO;
 * GRAPH: a hipGraph of T step kernels (as tms_decode_step_sparse), built and
 *   instantiated on the first call for a given T and replayed afterwards; a
 *   call with other buffers and the same T updates the instantiated graph's
 *   kernel arguments in place (after waiting for the device to drain, so
 *   that no queued replay reads them) instead of instantiating it again;
 *   a grouping or split set since the last call records the graph again;
 *   while the caller records the stream into a graph, the step kernels are
 *   recorded as STREAM launches them;
 * STREAM: the same T step kernels launched directly on the stream.
 * Also read from the TMS_LOOP environment variable (0..4) at create. */
typedef enum {
  TMS_LOOP_RESIDENT = 0,
  TMS_LOOP_GRAPH = 1,
  TMS_LOOP_STREAM = 2,
  TMS_LOOP_RESIDENT_SOLO = 3,
  TMS_LOOP_RESIDENT_GROUPED = 4
} tms_loop_mode;
tms_status tms_state_set_loop(tms_state* st, int32_t mode);

/* The no-repeat state the resident loop keeps (page "Constraint made cheaper
 * than no constraint", section "The batched engine": a per-sequence set of
 * spent pointers and, per edge, the set of pointers below it).  LIVE: the
 * per-edge live counts of section "Masked sampling inside the sampler" (any
 * catalog).  BITMASK: an edge is legal iff its set of entries minus the
 * sequence's spent set is non-empty (catalogs of at most 128 entries, else
 * INVALID_ARG); bit-identical results, live counts rewritten from the sets at
 * the end of each call.  Default LIVE, or BITMASK when the environment holds
 * TMS_BITMASK=1 at create and the catalog allows it.  Applies to the resident
 * loop forms of tms_decode_k_pointers; the step kernels always use the live
 * counts (and so does a call after tms_debug_set_live until the next reset). */
typedef enum { TMS_NOREPEAT_LIVE = 0, TMS_NOREPEAT_BITMASK = 1 } tms_norepeat;
tms_status tms_state_set_norepeat(tms_state* st, int32_t kind);

/* Node grouping of the fused step (tms_decode_step_sparse and the GRAPH and
 * STREAM loop forms; page "Constraint made cheaper than no constraint",
 * sections "The sparse output layer" and "The batched engine": the rows a
 * step needs are the union of the sequences' legal sets).  ROOT: the
 * sequences standing at the root in a step are served together in the same
 * launch: each root row is read once per tile of up to 16 of them and dotted
 * with each one's hidden vector.  NODES: as ROOT, and the sequences that
 * stand together at any other node share their workgroups: each row legal
 * for any of them is read once per tile of up to 4 of them and dotted with
 * each one's vector; a sequence alone at its node takes its own step.
 * Both keep the per-row arithmetic, so tokens, logits and state are
 * bit-identical to OFF (every sequence reads its own node's rows).  AUTO:
 * ROOT when B >= 8 and the root has at least 256 edges.  Always available for
 * the hidden sizes the library accepts (one member's vector, at most 16 KiB,
 * fits the LDS).  Also read from the TMS_STEP_GROUP environment variable
 * (0..3) at create. */
typedef enum {
  TMS_STEP_GROUP_AUTO = 0,
  TMS_STEP_GROUP_OFF = 1,
  TMS_STEP_GROUP_ROOT = 2,
  TMS_STEP_GROUP_NODES = 3
} tms_step_group;
tms_status tms_state_set_step_grouping(tms_state* st, int32_t mode);

/* Workgroups per sequence used by the fused step (per sequence off the root
 * when the root is grouped), and its grid size. */
tms_status tms_state_get_launch(const tms_state* st, int32_t* split, int32_t* grid);

/* ------------------------------------------------------ no allocation -- */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one whole
 * answer per sequence, exactly as tms_state_create + tms_decode_k_pointers on
 * a reset state (same kernels, bit-identical outputs), but with no state
 * handle: the per-sequence decode state (live counts, spent flags, path,
 * entries, argmax slots) lives in a device array of the library,
 * TMS_NOALLOC_SCRATCH_BYTES per GPU, allocated with the code object when the
 * library is first used on a GPU and held until the process ends.  The call
 * allocates nothing; the kernels initialise every word of the scratch they
 * read, so nothing carries over from an earlier call.
 * trie: uploaded on the current device; emb dev [V][H] (dtype, H as for
 * tms_state_create); hidden_seq dev [T][B][H]; outputs as for
 * tms_decode_k_pointers plus status dev int32 [B] (required: the per-sequence
 * tms_status, the only error report of the device for this call).
 * Errors: INVALID_ARG (as tms_state_create / tms_decode_k_pointers, null
 * status, or a batch whose state needs more than TMS_NOALLOC_SCRATCH_BYTES:
 * about B * (4 * n_edges + 4 * max_depth + 8 * k + 2 * root edges + 64)
 * bytes), K, HIP.  All calls on one GPU share its scratch: calls that overlap
 * on that GPU (other streams, other host threads) race, so serialise them. */
#define TMS_NOALLOC_SCRATCH_BYTES (32ll << 20)
tms_status tms_decode_k_pointers_noalloc(const tms_trie* trie, const void* emb, tms_dtype dtype, int32_t H,
                                         int32_t B, int32_t k, const void* hidden_seq, int32_t T,
                                         int32_t* tokens, int32_t* len, int32_t* entries, int32_t* status,
                                         void* stream);

const char* tms_status_str(tms_status s);
const char* tms_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TMS_H */
