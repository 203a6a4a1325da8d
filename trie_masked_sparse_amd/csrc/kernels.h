// Plain views of device buffers shared by the host API and the HIP kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tms {

// Sequence status codes written by the device (same values as tms_status).
enum : int32_t { kSeqOk = 0, kSeqEmptyMask = 5, kSeqNotWalkable = 6, kSeqNotDone = 7 };
enum : int32_t { kChildSep = -1, kChildStop = -2 };

// One 16-byte record per node: its edge range [b0, b1) and the catalog entry
// ending there (-1 if none).
struct alignas(16) NodeRec {
  int32_t b0, b1, ent, pad;
};

// One 16-byte record per edge: the child node (kChildSep/kChildStop for
// control edges), the token, and the child's edge range [b0, b1) (0, 0 for
// control edges).  With the child's entry (a separate array) one read of an
// edge gives everything a step needs to move along it.
struct alignas(16) EdgeRec {
  int32_t child, tok, b0, b1;
};

struct DevTrie {
  const int32_t* begin;  // [n_nodes+1]
  const int32_t* entry;  // [n_nodes]
  const int32_t* tok;    // [n_edges]
  const int32_t* child;  // [n_edges]
  const int32_t* live0;  // [live_stride], zero padded past n_edges
  const NodeRec* node_rec;  // [n_nodes]
  const EdgeRec* erec;      // [n_edges]
  const int32_t* cent;      // [live_stride] entry of the edge's child (-1: none or control edge), -1 padded
  // Forced runs.  A node with a single edge (a content edge: terminals carry
  // two control edges) leaves one legal token whenever it is reached along a
  // legal edge, since that edge and the next count the same live pointers.
  // Each maximal chain of such nodes is stored once, edges and tokens in
  // order; run[e] = (offset << 7) | length (at most 64) of the part of a chain
  // that follows edge e, 0 if e's child has more than one edge.
  const int32_t* run;       // [live_stride]
  const int32_t* run_edge;  // [n_run]
  const int32_t* run_tok;   // [n_run]
  // Where a run ends: for run position p, {child, child's first edge, child's
  // end edge, entry at the child} of run_edge[p] (one read lands a whole run).
  const int4* run_land;     // [n_run]
  int32_t n_run;            // nodes with a single edge
  // Bitmask no-repeat state (catalogs of at most 128 entries, else null): for
  // each edge the set of entries below it, 4 words, bit j = entry j.
  const uint32_t* emask;    // [n_edges][4]
  // Root path of every entry (its content edges from the root to its terminal,
  // in order): entry j's edges are ent_path[ent_off[j] .. ent_off[j+1]).  Null
  // when the catalog's tokens do not fit int32 offsets.
  const int32_t* ent_off;   // [n_entries + 1]
  const int32_t* ent_path;  // [ent_off[n_entries]]
  // erec, cent, run, run_edge, run_tok, run_land and emask (when present) are laid out
  // back to back from erec (each part a multiple of 16 bytes): image_words
  // int32 words in all
  int32_t image_words;
  int32_t n_nodes, n_edges, n_entries, cap, max_depth, sep, stop, vocab;
  int32_t live_stride;   // n_edges rounded up to a multiple of 4
  // 1: a completed pointer releases the live counts on its path (token
  // catalogs, k pointers); 0: an answer is one string (character catalogs),
  // so nothing is released and the live rows stay equal to live0
  int32_t release;
};

// Struct-of-arrays decode state for B sequences.
struct DevState {
  int32_t B, k;
  int32_t path_stride;   // >= max_depth
  int32_t spent_words;   // ceil(n_entries / 32)
  int32_t mask_words;    // ceil(vocab / 32)
  int32_t* node;         // [B] current trie node
  int32_t* depth;        // [B] content edges on the current pointer's path
  int32_t* done;         // [B] pointers completed
  int32_t* status;       // [B] kSeq* code, sticky
  int32_t* finished;     // [B] 1 after stop
  int32_t* nemit;        // [B] tokens emitted since reset
  int32_t* path;         // [B][path_stride] edge ids root -> node
  int32_t* entries;      // [B][k] completed catalog indices, -1 unused
  unsigned long long* key;  // [B] packed (logit, id) argmax slot, 0 = empty
  uint32_t* arrive;      // [B] workgroups of the current step that finished
  int32_t* tstep;        // [B] steps taken so far in the current phased decode call
  unsigned long long* rkey;  // [root_tiles][B] best key of each grouped-root row tile per sequence
  int32_t root_tiles;        // row tiles of the root (4 wavefronts x 1..4 rows each), upper bound
  int32_t* live;         // [B][live_stride]
  uint32_t* spent;       // [B][spent_words] one bit per catalog entry
  uint32_t* mask;        // [B][mask_words] dense-path vocabulary bitmask
  // [2][B] each sequence's node at the start of a root-grouped step (-1:
  // finished or in error), by launch parity: the step reads half p, which no
  // one writes during it, and writes half 1-p (null where unused)
  int32_t* snap;
};

// Per-step inputs and outputs.
struct StepIO {
  const void* emb;       // [V][H]
  const void* hidden;    // [B][H] for this step
  int32_t H, V;
  int32_t* out_tok;      // [B] or null
  float* out_logit;      // [B] or null
  int32_t* tokens_bt;    // [B][T] or null: column t receives this step's token
  int32_t T, t;
};

// Inputs and outputs of the resident device loop.
struct LoopIO {
  const void* emb;         // [V][H]
  const void* hidden_seq;  // [T][B][H]
  int32_t H, V, T;
  int32_t* tokens_bt;      // [B][T]
  int32_t* len;            // [B] or null
  int32_t* entries;        // [B][k] or null
  int32_t reset;           // kReset*: reset each sequence's state before the first step
  int32_t flags;           // kLoop* bits (phased runs of the resident loop)
  int32_t root_tiles;      // row tiles written by the last grouped root head (kLoopRootKey)
};

// Phased resident loop (one phase per pointer, the root steps grouped across
// sequences by launch_root_head): kLoopLater: not the first phase of the call
// (step index from DevState::tstep); kLoopExitAtRoot: a sequence that comes
// back to the root stops there (every phase but the last); kLoopRootKey: the
// root step of every sequence standing at the root was computed into key[s].
enum { kLoopLater = 1, kLoopExitAtRoot = 2, kLoopRootKey = 4 };

// Reset kinds.  kResetFull copies every live count from live0; kResetPaths
// relies on the stored live counts differing from live0 only on the root
// paths of the stored completed entries (what completions release), and
// restores just those edges and the entries' spent words.
// kResetState (tries that never release, see DevTrie::release): the live
// rows are untouched, only the sequences' state and spent flags are reset.
enum { kResetNone = 0, kResetFull = 1, kResetPaths = 2, kResetState = 3 };

// dtype: 0 fp32, 1 bf16.  Every launcher returns hipGetLastError().
hipError_t launch_reset(const DevTrie& tr, const DevState& st, int kind, hipStream_t s);
// Root grouping of the fused step (step_grouped_kernel): split workgroups per
// sequence not at the root, rt root row tiles of step_group_rows() rows each,
// mtiles member tiles of mt members (mt <= 16).
struct StepGroup {
  int split, rt, mt, mtiles;
  int parity;  // which half of DevState::snap holds the nodes at the start of this step
  int nodes;   // also group the sequences that share any other node
  int gmt;     // members per tile of those node groups
};
// snap[parity] <- every sequence's node (-1 if finished or in error).
hipError_t launch_snapshot(const DevState& st, int parity, hipStream_t s);
// grp null: the plain fused step (step_sparse_kernel, split workgroups per
// sequence); otherwise the step with the root grouped across sequences.
hipError_t launch_step_sparse(const DevTrie& tr, const DevState& st, const StepIO& io, int dtype,
                              bool fast, int split, hipStream_t s, const StepGroup* grp = nullptr);
// Workgroups of a grouped root launch with rt row tiles and mtiles member
// tiles: rt padded to a multiple of 8, so that the member tiles of a row tile
// share an XCD (root_tile in the kernels).
inline int root_tile_grid(int rt, int mtiles) { return (rt + 7) / 8 * 8 * mtiles; }
// LDS bytes of a root workgroup of the grouped step (nq = 16-byte chunks per row).
size_t step_group_lds(int nq, int mt);
// Root rows per root workgroup of the grouped step.
int step_group_rows(int dtype, int H);
// Variants of the resident loop: trie, live counts and spent bits in LDS
// (fast path); trie through the scalar cache with live counts in device
// memory (fast path, too big for LDS); vector edge reads with live counts in
// LDS, or in device memory (global path).
// kLoopTrieMask: as kLoopTrieLds with the bitmask no-repeat state.
enum { kLoopTrieLds = 0, kLoopFastGlobal = 1, kLoopVectorLds = 2, kLoopVectorGlobal = 3, kLoopTrieMask = 4 };
// The root step of every sequence at the root (or of all, with io.reset), for
// the step each is at: per row tile and sequence the best key into st.rkey
// (the root's edges are [root_b0, root_b0 + root_edges)).
hipError_t launch_root_head(const DevTrie& tr, const DevState& st, const LoopIO& io, int dtype, int root_b0,
                            int root_edges, hipStream_t s);
// Row tiles the grouped root head uses for this hidden size (io.root_tiles).
int root_head_tiles(int dtype, int H, int root_edges);
hipError_t launch_loop(const DevTrie& tr, const DevState& st, const LoopIO& io, int dtype, int mode,
                       hipStream_t s);
// LDS bytes of the resident loop's per-sequence copy (live counts, spent bits,
// and the trie arrays when trie = true).
size_t loop_lds_bytes(const DevTrie& tr, const DevState& st, bool trie);
// Dense step: bitmask, all-V head, masked argmax, advance.  With mfma and a
// bf16 table, 2 <= B <= 256 and H % 32 == 0 the head runs on the matrix cores;
// otherwise on the vector units with the sparse head's per-row arithmetic
// (grid workgroups; 0: sized from V).
hipError_t launch_dense_step(const DevTrie& tr, const DevState& st, const StepIO& io, int dtype,
                             float* full_logits, int grid, bool mfma, hipStream_t s);
bool dense_uses_mfma(int dtype, int B, int H);
// The vocabulary bitmask of each sequence's legal set ([B][ceil(V/32)]).
hipError_t launch_legal_mask(const DevTrie& tr, const DevState& st, uint32_t* out, hipStream_t s);
// Sorted token ids of the set bits of each mask row, at most cap of them.
hipError_t launch_mask_rows(const uint32_t* mask, int B, int V, int cap, int32_t* rows, int32_t* n_rows,
                            hipStream_t s);
hipError_t launch_forced(const DevTrie& tr, const DevState& st, const int32_t* forced, hipStream_t s);
hipError_t launch_legal_set(const DevTrie& tr, const DevState& st, int32_t* legal_tok,
                            int32_t* n_legal, hipStream_t s);
hipError_t launch_gather_gemv(const void* emb, int dtype, int32_t V, int32_t H, const void* hidden,
                              const int32_t* rows, const int32_t* n_rows, int32_t B, int32_t cap,
                              float* out, int split, hipStream_t s);
hipError_t launch_finalize(const DevState& st, int32_t* len, int32_t* entries, hipStream_t s);
// Streaming read of bytes (a multiple of 16) from src; grid workgroups of 256
// threads (0: one pass per thread), unroll 1/2/4/8 loads in flight per thread.
hipError_t launch_read_reference(const void* src, int64_t bytes, uint32_t* out, int grid, int unroll,
                                 hipStream_t s);
hipError_t launch_set_live(const DevTrie& tr, const DevState& st, int32_t seq, int32_t edge,
                           int32_t value, hipStream_t s);

// Chunks of 16 bytes per lane needed for a row of H elements (0 if too wide).
int chunks_for(int dtype, int H);

}  // namespace tms
