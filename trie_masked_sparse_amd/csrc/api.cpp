// C ABI of the trie-constrained sparse decode library (declared in include/tms.h).
// Handles own their device memory; decode calls only enqueue kernels on the
// caller's stream.  The device loop runs as one resident kernel (or one grouped
// root head plus one resident kernel per pointer), or as T step kernels, either
// launched directly or as a hipGraph captured on a private stream and replayed
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "charset_build.h"
#include "handles.h"

namespace {

thread_local std::string g_err;

tms_status fail(tms_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

tms_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? TMS_ERR_OOM : TMS_ERR_HIP;
}

#define TMS_HIP(call, what)                       \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Carve typed sub-buffers out of one allocation.
struct Carve {
  size_t off = 0;
  template <typename T>
  size_t take(size_t n) {
    const size_t o = off;
    off = align256(off + sizeof(T) * std::max<size_t>(n, 1));
    return o;
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == TMS_F32 ? 4 : 2; }

// Workgroups per sequence of the fused step: a step is a chain of dependent
// loads, and combining workgroups costs two device-scope atomics plus a third
// read on that chain (measured: split 1 against the former 3-4 workgroups per
// sequence, product 3.5 vs 4.9 us per step, structured B = 64 4.8 vs 8.1), so
// a sequence gets more than one workgroup only when its widest node needs more
// than two passes of its wavefronts' rows (4 wavefronts x rows_per_pass rows),
// and never more than a chip-filling 4096 wavefronts over the batch.
// Workgroups per sequence of the fused step: enough for one pass over the
// widest node's rows, but only while the grid stays within one workgroup per
// free compute unit (wgs_free): beyond that the extra workgroups share compute
// units and their key exchange costs more than the passes they save.  Per-step
// graph, old rule -> this one: large B = 256 (split 3 -> 1) 21.5 -> 9.3 us,
// charset_tools B = 64 (11 -> 4) 5.6 -> 4.0, charset_hex root-grouped (9 -> 1)
// 10.1 -> 5.6; structured and unstructured keep 1.
int default_split(int B, int cap, int rows_per_wg, int wgs_free) {
  const int by_cus = std::max(1, wgs_free / B);
  const int by_cap = std::max(1, (cap + rows_per_wg - 1) / rows_per_wg);
  return std::min(by_cus, by_cap);
}

// Gather-GEMV workgroups per sequence: 4096 wavefronts for short lists (one
// pass of rows each), 2048 for long ones (several double-buffered passes),
// the faster choice in measurements at 64 x 256 and 64 x 887 rows.
int gemv_split(int B, int cap) {
  const int target_waves = int64_t(B) * cap <= 32768 ? 4096 : 2048;
  int s = (target_waves + 4 * B - 1) / (4 * B);
  s = std::min(s, std::max(1, (cap + 3) / 4));
  return std::max(1, s);
}

void destroy_graph(tms_state* st) {
  // a replay may still be queued (a setter called without a synchronisation):
  // it finishes before its graph goes
  if (st->gexec) {
    (void)hipDeviceSynchronize();
    (void)hipGraphExecDestroy(st->gexec);
  }
  if (st->graph) (void)hipGraphDestroy(st->graph);
  st->gexec = nullptr;
  st->graph = nullptr;
  st->g_hidden = nullptr;
}

// The root grouping of the fused step, when it applies to this state.
tms::StepGroup* step_group(tms_state* st) {
  const int mode = st->step_group_mode;
  const bool on = mode == TMS_STEP_GROUP_ROOT || mode == TMS_STEP_GROUP_NODES ? st->step_group_ok
                  : mode == TMS_STEP_GROUP_OFF                               ? false
                                                                             : st->step_group_auto;
  st->grp.nodes = mode == TMS_STEP_GROUP_NODES ? 1 : 0;
  st->grp.gmt = st->grp_mt_nodes;
  return on ? &st->grp : nullptr;
}

const tms::StepGroup* step_group(const tms_state* st) { return step_group(const_cast<tms_state*>(st)); }

tms::StepIO make_io(const tms_state* st, const void* hidden) {
  tms::StepIO io{};
  io.emb = st->emb;
  io.hidden = hidden;
  io.H = st->H;
  io.V = st->trie->host.vocab;
  return io;
}

}  // namespace

namespace tms {

tms_status api_fail(tms_status s, const std::string& msg) { return fail(s, msg); }
tms_status api_hip_fail(hipError_t e, const char* what) { return hip_fail(e, what); }

hipError_t enqueue_resident(const tms_trie* trie, const DevState& dev, LoopIO io, int dtype, bool fast,
                            int loop_mode, bool fresh, bool bitmask, hipStream_t s) {
  // LDS budget per workgroup for the loop's on-chip copy (the part offers
  // 160 KiB; a little is left for the kernel's own shared variables)
  const size_t budget = 160 * 1024 - 2048;
  int mode;
  if (fast) {
    mode = loop_lds_bytes(trie->dev, dev, true) <= budget ? kLoopTrieLds : kLoopFastGlobal;
    // the bitmask no-repeat state, on request (measured slower than the live
    // counts for the product catalog: 17.4 vs 15.6 us per answer)
    if (mode == kLoopTrieLds && trie->dev.emask && bitmask) mode = kLoopTrieMask;
  } else {
    mode = loop_lds_bytes(trie->dev, dev, false) <= budget ? kLoopVectorLds : kLoopVectorGlobal;
  }
  // Root steps grouped across sequences: one phase per pointer (every
  // pointer starts at the root), each a grouped root head then the loop up
  // to the next return to the root; the last phase runs to the end.  Worth
  // it where the root is wide and shared by many sequences.
  const HostTrie& h = trie->host;
  const int root_edges = h.begin[1] - h.begin[0];
  const bool group = loop_mode == TMS_LOOP_RESIDENT_GROUPED ||
                     (loop_mode == TMS_LOOP_RESIDENT && dev.B >= 8 && root_edges >= 64);
  if (!group) return launch_loop(trie->dev, dev, io, dtype, mode, s);
  // after a grouped root step a phase reads few live counts: keep them in
  // device memory rather than copying them through LDS every phase
  if (mode == kLoopVectorLds) mode = kLoopVectorGlobal;
  const int reset = io.reset;
  const int phases = fresh ? dev.k : dev.k + 1;
  for (int p = 0; p < phases; ++p) {
    io.reset = p == 0 ? reset : kResetNone;
    io.flags = (p > 0 ? kLoopLater : 0) | (p + 1 < phases ? kLoopExitAtRoot : 0) | kLoopRootKey;
    io.root_tiles = root_head_tiles(dtype, io.H, root_edges);
    if (hipError_t e = launch_root_head(trie->dev, dev, io, dtype, h.begin[0], root_edges, s); e != hipSuccess)
      return e;
    if (hipError_t e = launch_loop(trie->dev, dev, io, dtype, mode, s); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tms

extern "C" {

const char* tms_status_str(tms_status s) {
  switch (s) {
    case TMS_OK: return "ok";
    case TMS_ERR_INVALID_ARG: return "invalid argument";
    case TMS_ERR_CATALOG: return "invalid catalog";
    case TMS_ERR_FANOUT: return "node fan-out above 256 on the fast path";
    case TMS_ERR_K: return "k outside [1, K]";
    case TMS_ERR_EMPTY_MASK: return "empty mask";
    case TMS_ERR_NOT_WALKABLE: return "token not walkable";
    case TMS_ERR_NOT_DONE: return "sequence not done";
    case TMS_ERR_BUSY: return "trie still in use";
    case TMS_ERR_OOM: return "out of device memory";
    case TMS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tms_last_error(void) { return g_err.c_str(); }

tms_status tms_trie_build(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab, int32_t sep,
                          int32_t stop, tms_trie** out) {
  if (!out) return fail(TMS_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  tms_trie* t = new tms_trie();
  std::string err;
  const int rc = tms::build_trie(tokens, offsets, K, vocab, sep, stop, &t->host, &err);
  if (rc != 0) {
    delete t;
    return fail(static_cast<tms_status>(rc), err);
  }
  *out = t;
  return TMS_OK;
}

// The device copy of a built trie, owned by t (freed with t on failure).
// tokens/offsets: the token catalog the trie was built from, for the
// per-entry tables (bitmask state, reset by paths); null for a character
// catalog, whose entries have no single token path.
static tms_status upload_host(tms_trie* t, const int32_t* tokens, const int64_t* offsets, int32_t K, tms_path path,
                              void* stream, tms_trie** out) {
  const tms::HostTrie& h = t->host;
  // hot CSR bytes read by the step: begin, tok, child
  const int64_t hot = 4ll * (h.n_nodes + 1) + 8ll * h.n_edges;
  const bool fast_ok = h.cap <= 256 && hot <= 65536;
  if (h.n_edges >= (1 << 29)) {
    delete t;
    return fail(TMS_ERR_CATALOG, "trie has 2^29 or more edges");
  }
  if (path == TMS_PATH_FAST && h.cap > 256) {
    delete t;
    return fail(TMS_ERR_FANOUT, "fast path needs every node to have at most 256 edges; widest has " +
                                    std::to_string(h.cap));
  }
  t->path = path == TMS_PATH_GLOBAL ? TMS_PATH_GLOBAL
            : path == TMS_PATH_FAST ? TMS_PATH_FAST
            : (fast_ok ? TMS_PATH_FAST : TMS_PATH_GLOBAL);
  const int32_t live_stride = (h.n_edges + 3) & ~3;
  Carve c;
  const size_t o_begin = c.take<int32_t>(h.n_nodes + 1);
  const size_t o_entry = c.take<int32_t>(h.n_nodes);
  const size_t o_tok = c.take<int32_t>(h.n_edges);
  const size_t o_child = c.take<int32_t>(h.n_edges);
  const size_t o_live0 = c.take<int32_t>(live_stride);
  const size_t o_rec = c.take<int32_t>(size_t(h.n_nodes) * 4);
  // forced runs: chains of nodes with a single edge, each stored once
  std::vector<int32_t> run(live_stride, 0), run_edge, run_tok;
  {
    auto unary = [&](int32_t n) { return h.begin[n + 1] - h.begin[n] == 1; };
    std::vector<int32_t> chain;
    for (int32_t n = 0; n < h.n_nodes; ++n) {
      if (n != 0 && unary(n)) continue;  // edges of single-edge nodes belong to their head's chain
      for (int32_t x = h.begin[n]; x < h.begin[n + 1]; ++x) {
        chain.clear();
        for (int32_t y = x; h.child[y] >= 0 && unary(h.child[y]);) {
          y = h.begin[h.child[y]];
          chain.push_back(y);
        }
        if (chain.empty()) continue;
        const int32_t p = static_cast<int32_t>(run_edge.size());
        for (size_t i = 0; i < chain.size(); ++i) {
          run_edge.push_back(chain[i]);
          run_tok.push_back(h.tok[chain[i]]);
        }
        // edge x is followed by the whole chain, chain[i] by what follows it
        const int32_t m = static_cast<int32_t>(chain.size());
        for (int32_t i = -1; i < m; ++i) {
          const int32_t edge = i < 0 ? x : chain[i];
          const int32_t len = std::min(m - 1 - i, 64);
          run[edge] = len > 0 ? ((p + i + 1) << 7) | len : 0;
        }
      }
    }
    if (run_edge.size() >= (size_t(1) << 24)) std::fill(run.begin(), run.end(), 0);  // offsets must fit
  }
  const int32_t n_run = static_cast<int32_t>(run_edge.size());
  // bitmask no-repeat state for catalogs of at most 128 entries: the entries
  // below each content edge (the edges of each entry's root path)
  const bool with_mask = tokens && h.n_entries <= 128;
  std::vector<uint32_t> emask(with_mask ? size_t(h.n_edges) * 4 : 0, 0u);
  // each entry's root path, for resets that restore only what completions
  // released (int32 offsets: at most 2^31 - 1 catalog tokens)
  const int64_t n_path = tokens ? offsets[K] - offsets[0] : 0;
  const bool with_paths = tokens && n_path < (int64_t(1) << 31);
  std::vector<int32_t> ent_off(with_paths ? size_t(K) + 1 : 0, 0), ent_path(with_paths ? size_t(n_path) : 0, 0);
  if (with_mask || with_paths) {
    for (int32_t j = 0; j < K; ++j) {
      int32_t n = 0;
      if (with_paths) ent_off[j] = static_cast<int32_t>(offsets[j] - offsets[0]);
      for (int64_t p = offsets[j]; p < offsets[j + 1]; ++p) {
        const int32_t* lo = h.tok.data() + h.begin[n];
        const int32_t* hi = h.tok.data() + h.begin[n + 1];
        const int32_t x = static_cast<int32_t>(std::lower_bound(lo, hi, tokens[p]) - h.tok.data());
        if (with_mask) emask[4 * size_t(x) + (j >> 5)] |= 1u << (j & 31);
        if (with_paths) ent_path[size_t(p - offsets[0])] = x;
        n = h.child[x];
      }
    }
    if (with_paths) ent_off[K] = static_cast<int32_t>(n_path);
  }
  // edge records, children's entries and run tables in one block, in the
  // order (and word offsets) the resident loop keeps them in LDS, so that
  // one copy loop brings them on chip
  const size_t w_erec = 0, w_cent = w_erec + 4 * size_t(h.n_edges), w_run = w_cent + live_stride,
               w_run_edge = w_run + live_stride, w_run_tok = w_run_edge + ((n_run + 3) & ~3),
               w_run_land = w_run_tok + ((n_run + 3) & ~3), w_emask = w_run_land + 4 * size_t(n_run),
               w_image = w_emask + emask.size();
  const size_t o_image = c.take<int32_t>(w_image);
  const size_t o_erec = o_image + 4 * w_erec, o_cent = o_image + 4 * w_cent, o_run = o_image + 4 * w_run,
               o_run_edge = o_image + 4 * w_run_edge, o_run_tok = o_image + 4 * w_run_tok,
               o_run_land = o_image + 4 * w_run_land,
               o_emask = o_image + 4 * w_emask;
  const size_t o_ent_off = c.take<int32_t>(ent_off.size()), o_ent_path = c.take<int32_t>(ent_path.size());
  // where each run position lands: the child of run_edge[p] and its record
  std::vector<int32_t> run_land(4 * size_t(n_run), 0);
  for (int32_t p = 0; p < n_run; ++p) {
    const int32_t ch = h.child[run_edge[p]];
    run_land[4 * size_t(p)] = ch;
    if (ch >= 0) {
      run_land[4 * size_t(p) + 1] = h.begin[ch];
      run_land[4 * size_t(p) + 2] = h.begin[ch + 1];
      run_land[4 * size_t(p) + 3] = h.entry[ch];
    } else {
      run_land[4 * size_t(p) + 3] = -1;
    }
  }
  run_edge.resize((n_run + 3) & ~3, 0);
  run_tok.resize((n_run + 3) & ~3, 0);
  hipError_t e = hipGetDevice(&t->device);
  if (e == hipSuccess) e = hipMalloc(&t->dmem, c.off);
  if (e != hipSuccess) {
    delete t;
    return hip_fail(e, "trie upload");
  }
  t->dbytes = c.off;
  char* base = static_cast<char*>(t->dmem);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> live0(live_stride, 0);
  std::copy(h.live0.begin(), h.live0.end(), live0.begin());
  std::vector<int32_t> rec(size_t(h.n_nodes) * 4, 0);
  for (int32_t n = 0; n < h.n_nodes; ++n) {
    rec[4 * size_t(n)] = h.begin[n];
    rec[4 * size_t(n) + 1] = h.begin[n + 1];
    rec[4 * size_t(n) + 2] = h.entry[n];
  }
  std::vector<int32_t> erec(size_t(h.n_edges) * 4, 0);
  std::vector<int32_t> cent(live_stride, -1);
  for (int32_t x = 0; x < h.n_edges; ++x) {
    const int32_t ch = h.child[x];
    erec[4 * size_t(x)] = ch;
    erec[4 * size_t(x) + 1] = h.tok[x];
    if (ch >= 0) {
      erec[4 * size_t(x) + 2] = h.begin[ch];
      erec[4 * size_t(x) + 3] = h.begin[ch + 1];
      cent[x] = h.entry[ch];
    }
  }
  e = hipMemcpyAsync(base + o_begin, h.begin.data(), 4 * h.begin.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_entry, h.entry.data(), 4 * h.entry.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_tok, h.tok.data(), 4 * h.tok.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_child, h.child.data(), 4 * h.child.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_live0, live0.data(), 4 * live0.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_rec, rec.data(), 4 * rec.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_erec, erec.data(), 4 * erec.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_cent, cent.data(), 4 * cent.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_run, run.data(), 4 * run.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !run_edge.empty())
    e = hipMemcpyAsync(base + o_run_edge, run_edge.data(), 4 * run_edge.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !run_tok.empty())
    e = hipMemcpyAsync(base + o_run_tok, run_tok.data(), 4 * run_tok.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !run_land.empty())
    e = hipMemcpyAsync(base + o_run_land, run_land.data(), 4 * run_land.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && with_mask)
    e = hipMemcpyAsync(base + o_emask, emask.data(), 4 * emask.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && with_paths)
    e = hipMemcpyAsync(base + o_ent_off, ent_off.data(), 4 * ent_off.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && with_paths && !ent_path.empty())
    e = hipMemcpyAsync(base + o_ent_path, ent_path.data(), 4 * ent_path.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(t->dmem);
    delete t;
    return hip_fail(e, "trie upload copy");
  }
  tms::DevTrie& d = t->dev;
  d.begin = reinterpret_cast<const int32_t*>(base + o_begin);
  d.entry = reinterpret_cast<const int32_t*>(base + o_entry);
  d.tok = reinterpret_cast<const int32_t*>(base + o_tok);
  d.child = reinterpret_cast<const int32_t*>(base + o_child);
  d.live0 = reinterpret_cast<const int32_t*>(base + o_live0);
  d.node_rec = reinterpret_cast<const tms::NodeRec*>(base + o_rec);
  d.erec = reinterpret_cast<const tms::EdgeRec*>(base + o_erec);
  d.cent = reinterpret_cast<const int32_t*>(base + o_cent);
  d.run = reinterpret_cast<const int32_t*>(base + o_run);
  d.run_edge = reinterpret_cast<const int32_t*>(base + o_run_edge);
  d.run_tok = reinterpret_cast<const int32_t*>(base + o_run_tok);
  d.run_land = reinterpret_cast<const int4*>(base + o_run_land);
  d.image_words = static_cast<int32_t>(w_image);
  d.emask = with_mask ? reinterpret_cast<const uint32_t*>(base + o_emask) : nullptr;
  d.ent_off = with_paths ? reinterpret_cast<const int32_t*>(base + o_ent_off) : nullptr;
  d.ent_path = with_paths ? reinterpret_cast<const int32_t*>(base + o_ent_path) : nullptr;
  d.n_run = n_run;
  d.n_nodes = h.n_nodes;
  d.n_edges = h.n_edges;
  d.n_entries = h.n_entries;
  d.cap = h.cap;
  d.max_depth = h.max_depth;
  d.sep = h.sep;
  d.stop = h.stop;
  d.vocab = h.vocab;
  d.live_stride = live_stride;
  d.release = t->charset ? 0 : 1;
  *out = t;
  return TMS_OK;
}

tms_status tms_trie_upload(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab, int32_t sep,
                           int32_t stop, tms_path path, void* stream, tms_trie** out) {
  if (!out) return fail(TMS_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (path != TMS_PATH_AUTO && path != TMS_PATH_FAST && path != TMS_PATH_GLOBAL)
    return fail(TMS_ERR_INVALID_ARG, "unknown path");
  tms_trie* t = nullptr;
  tms_status rc = tms_trie_build(tokens, offsets, K, vocab, sep, stop, &t);
  if (rc != TMS_OK) return rc;
  return upload_host(t, tokens, offsets, K, path, stream, out);
}

tms_status tms_charset_build(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                             const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, tms_trie** out) {
  if (!out) return fail(TMS_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  tms_trie* t = new tms_trie();
  t->charset = true;
  std::string err;
  const int rc = tms::build_charset(bytes, offsets, K, token_bytes, token_offsets, V, sep, stop, &t->host, &err);
  if (rc != 0) {
    delete t;
    return fail(static_cast<tms_status>(rc), err);
  }
  *out = t;
  return TMS_OK;
}

tms_status tms_charset_upload(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                              const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, tms_path path,
                              void* stream, tms_trie** out) {
  if (!out) return fail(TMS_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (path != TMS_PATH_AUTO && path != TMS_PATH_FAST && path != TMS_PATH_GLOBAL)
    return fail(TMS_ERR_INVALID_ARG, "unknown path");
  tms_trie* t = nullptr;
  tms_status rc = tms_charset_build(bytes, offsets, K, token_bytes, token_offsets, V, sep, stop, &t);
  if (rc != TMS_OK) return rc;
  return upload_host(t, nullptr, nullptr, 0, path, stream, out);
}

tms_status tms_trie_info_get(const tms_trie* t, tms_trie_info* info) {
  if (!t || !info) return fail(TMS_ERR_INVALID_ARG, "null argument");
  const tms::HostTrie& h = t->host;
  info->n_nodes = h.n_nodes;
  info->n_edges = h.n_edges;
  info->n_entries = h.n_entries;
  info->cap = h.cap;
  info->max_depth = h.max_depth;
  info->sep = h.sep;
  info->stop = h.stop;
  info->vocab = h.vocab;
  info->path = t->path;
  info->device_bytes = static_cast<int64_t>(t->dbytes);
  return TMS_OK;
}

tms_status tms_trie_export_csr(const tms_trie* t, int32_t* begin, int32_t* entry, int32_t* tok, int32_t* child,
                               int32_t* live0) {
  if (!t) return fail(TMS_ERR_INVALID_ARG, "null trie");
  const tms::HostTrie& h = t->host;
  if (begin) std::memcpy(begin, h.begin.data(), 4 * h.begin.size());
  if (entry) std::memcpy(entry, h.entry.data(), 4 * h.entry.size());
  if (tok) std::memcpy(tok, h.tok.data(), 4 * h.tok.size());
  if (child) std::memcpy(child, h.child.data(), 4 * h.child.size());
  if (live0) std::memcpy(live0, h.live0.data(), 4 * h.live0.size());
  return TMS_OK;
}

tms_status tms_trie_free(tms_trie* t) {
  if (!t) return TMS_OK;
  if (t->refs > 0) return fail(TMS_ERR_BUSY, std::to_string(t->refs) + " state(s) still use this trie");
  if (t->dmem) (void)hipFree(t->dmem);
  delete t;
  return TMS_OK;
}

tms_status tms_state_create(tms_trie* trie, int32_t B, int32_t k, const void* emb, tms_dtype dtype, int32_t H,
                            void* stream, tms_state** out) {
  if (!out) return fail(TMS_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (!trie || !trie->dmem) return fail(TMS_ERR_INVALID_ARG, "trie has no device copy (use tms_trie_upload)");
  if (B < 1 || B > 65535) return fail(TMS_ERR_INVALID_ARG, "B must be in [1, 65535]");
  if (k < 1 || k > trie->host.n_entries)
    return fail(TMS_ERR_K, "k = " + std::to_string(k) + " outside [1, " + std::to_string(trie->host.n_entries) + "]");
  if (trie->charset && k != 1) return fail(TMS_ERR_K, "a character catalog answers with one string (k = 1)");
  if (dtype != TMS_F32 && dtype != TMS_BF16) return fail(TMS_ERR_INVALID_ARG, "dtype must be fp32 or bf16");
  if (!emb || !aligned16(emb)) return fail(TMS_ERR_INVALID_ARG, "embedding pointer null or not 16-byte aligned");
  if (tms::chunks_for(dtype, H) == 0)
    return fail(TMS_ERR_INVALID_ARG, "H must be a positive multiple of " + std::to_string(16 / elem_size(dtype)) +
                                         " and at most " + std::to_string(dtype == TMS_F32 ? 4096 : 8192));
  int dev = -1;
  TMS_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != trie->device) return fail(TMS_ERR_INVALID_ARG, "trie was uploaded on another device");
  int cus = 0;
  TMS_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "compute unit count");
  cus = std::max(cus, 1);

  tms_state* st = new tms_state();
  st->trie = trie;
  st->B = B;
  st->k = k;
  st->H = H;
  st->dtype = dtype;
  st->emb = emb;
  st->device = dev;
  st->fast = trie->path == TMS_PATH_FAST;
  const tms::HostTrie& h = trie->host;
  const int32_t path_stride = std::max(1, h.max_depth);
  const int32_t spent_words = (h.n_entries + 31) / 32;
  const int32_t mask_words = (h.vocab + 31) / 32;
  const int64_t live_stride = trie->dev.live_stride;
  Carve c;
  const size_t o_node = c.take<int32_t>(B), o_depth = c.take<int32_t>(B), o_done = c.take<int32_t>(B);
  const size_t o_status = c.take<int32_t>(B), o_fin = c.take<int32_t>(B), o_nemit = c.take<int32_t>(B);
  const size_t o_path = c.take<int32_t>(size_t(B) * path_stride);
  const size_t o_entries = c.take<int32_t>(size_t(B) * k);
  const size_t o_key = c.take<unsigned long long>(B);
  const size_t o_arrive = c.take<uint32_t>(B);
  const size_t o_tstep = c.take<int32_t>(B);
  // grouped root head: one key per (row tile, sequence); at most one tile per 4 rows
  const int32_t root_tiles = (trie->host.begin[1] - trie->host.begin[0] + 3) / 4;
  const size_t o_rkey = c.take<unsigned long long>(size_t(root_tiles) * B);
  const size_t o_live = c.take<int32_t>(size_t(B) * live_stride);
  const size_t o_spent = c.take<uint32_t>(size_t(B) * spent_words);
  const size_t o_mask = c.take<uint32_t>(size_t(B) * mask_words);
  const size_t o_snap = c.take<int32_t>(2 * size_t(B));
  hipError_t e = hipMalloc(&st->dmem, c.off);
  if (e != hipSuccess) {
    delete st;
    return hip_fail(e, "state allocation");
  }
  st->dbytes = c.off;
  char* base = static_cast<char*>(st->dmem);
  tms::DevState& d = st->dev;
  d.B = B;
  d.k = k;
  d.path_stride = path_stride;
  d.spent_words = spent_words;
  d.mask_words = mask_words;
  d.node = reinterpret_cast<int32_t*>(base + o_node);
  d.depth = reinterpret_cast<int32_t*>(base + o_depth);
  d.done = reinterpret_cast<int32_t*>(base + o_done);
  d.status = reinterpret_cast<int32_t*>(base + o_status);
  d.finished = reinterpret_cast<int32_t*>(base + o_fin);
  d.nemit = reinterpret_cast<int32_t*>(base + o_nemit);
  d.path = reinterpret_cast<int32_t*>(base + o_path);
  d.entries = reinterpret_cast<int32_t*>(base + o_entries);
  d.key = reinterpret_cast<unsigned long long*>(base + o_key);
  d.arrive = reinterpret_cast<uint32_t*>(base + o_arrive);
  d.tstep = reinterpret_cast<int32_t*>(base + o_tstep);
  d.rkey = reinterpret_cast<unsigned long long*>(base + o_rkey);
  d.root_tiles = root_tiles;
  d.live = reinterpret_cast<int32_t*>(base + o_live);
  d.spent = reinterpret_cast<uint32_t*>(base + o_spent);
  d.mask = reinterpret_cast<uint32_t*>(base + o_mask);
  d.snap = reinterpret_cast<int32_t*>(base + o_snap);
  st->split_default = default_split(B, h.cap, tms::step_group_rows(dtype, H), cus);
  st->split = st->split_default;
  {
    // root grouping of the fused step: sequences off the root need only the
    // widest other node's edges; root workgroups take tiles of root rows x
    // members, as many members per tile (at most 16) as fit 128 KiB of LDS
    int cap_rest = 1;
    for (int32_t n = 1; n < h.n_nodes; ++n) cap_rest = std::max(cap_rest, h.begin[n + 1] - h.begin[n]);
    const int root_edges = h.begin[1] - h.begin[0];
    const int nq = H / (dtype == TMS_F32 ? 4 : 8);
    const int mt = std::max(1, std::min(16, int((128 * 1024 - 64) / (16 * size_t(nq)))));
    const int rows = tms::step_group_rows(dtype, H);
    st->grp.rt = (root_edges + rows - 1) / rows;
    // members per root tile: the fewest (shorter chains of member pairs per
    // workgroup) that keep the root tiles within about five workgroups per
    // compute unit.  Per-step graph, B = 64, 16 / 8 / 4 members: unstructured
    // 7.25 / 7.00 / 6.47 us, charset_tools 6.36 / 5.95 / 5.91, charset_hex (160
    // row tiles) 10.79 / 10.00 / 10.97.  Node groups (NODES) take 4 members per
    // tile: per-step graph with 16 / 4 / 2 (1), structured 9.11 / 8.48 / 8.07,
    // large (B = 256) 14.77 / 14.75 / (19.94); unstructured and the catalogs
    // within 1 % of each other.
    st->grp_mt_nodes = std::min(mt, 4);
    st->grp_mt_root = mt;
    for (int m = 4; m < mt; m *= 2)
      if (tms::root_tile_grid(st->grp.rt, (B + m - 1) / m) <= 5 * cus) {
        st->grp_mt_root = m;
        break;
      }
    st->grp.mt = st->grp_mt_root;
    st->grp.mtiles = (B + st->grp.mt - 1) / st->grp.mt;
    // the sequences off the root split over the compute units the root tiles leave
    const int root_wgs = tms::root_tile_grid(st->grp.rt, st->grp.mtiles);
    st->grp_split_default = default_split(B, cap_rest, rows, std::max(cus - root_wgs, 0));
    st->grp.split = st->grp_split_default;
    st->step_group_ok = root_edges > 0 && tms::step_group_lds(nq, mt) <= 160 * 1024 - 1024;
    // automatic for wide roots: per-step graph at B = 64, per sequence / root
    // grouped, unstructured (884 root edges) 19.3 / 6.6 us, charset_hex (2470)
    // 12.8 / 10.0, charset_tools (191) 5.5 / 5.8
    st->step_group_auto = st->step_group_ok && B >= 8 && root_edges >= 256;
  }
  if (const char* env = std::getenv("TMS_SPLIT")) {
    const int v = std::atoi(env);
    if (v > 0) st->split = st->grp.split = v;
  }
  if (const char* env = std::getenv("TMS_DENSE_VECTOR")) st->dense_mfma = std::atoi(env) == 0;
  if (const char* env = std::getenv("TMS_LOOP")) {
    const int v = std::atoi(env);
    if (v >= TMS_LOOP_RESIDENT && v <= TMS_LOOP_RESIDENT_GROUPED) st->loop_mode = v;
  }
  if (const char* env = std::getenv("TMS_STEP_GROUP")) {
    const int v = std::atoi(env);
    const bool needs_fit = v == TMS_STEP_GROUP_ROOT || v == TMS_STEP_GROUP_NODES;
    if (v >= TMS_STEP_GROUP_AUTO && v <= TMS_STEP_GROUP_NODES && (!needs_fit || st->step_group_ok))
      st->step_group_mode = v;
  }
  if (const char* env = std::getenv("TMS_BITMASK"))
    if (env[0] == '1' && trie->dev.emask) st->norepeat = TMS_NOREPEAT_BITMASK;
  st->host_status.assign(B, 0);
  e = hipStreamCreateWithFlags(&st->capture, hipStreamNonBlocking);
  if (e != hipSuccess) {
    (void)hipFree(st->dmem);
    delete st;
    return hip_fail(e, "capture stream");
  }
  trie->refs++;
  *out = st;
  tms_status rc = tms_state_reset(st, stream);
  if (rc != TMS_OK) {
    tms_state_free(st);
    *out = nullptr;
    return rc;
  }
  return TMS_OK;
}

// Carries out a pending reset before another call reads or writes the state.
// The kind of reset a pending reset takes.
static int reset_kind(const tms_state* st) {
  if (!st->reset_pending) return tms::kResetNone;
  if (!st->trie->dev.release) return st->live_by_paths ? tms::kResetState : tms::kResetFull;
  return st->live_by_paths && st->trie->dev.ent_path ? tms::kResetPaths : tms::kResetFull;
}

// A pending reset was enqueued: afterwards the live rows follow the stored
// entries again.
static void reset_enqueued(tms_state* st) {
  st->reset_pending = false;
  st->live_by_paths = true;
}

// Carries out a pending reset before another call reads or writes the state.
static tms_status flush_reset(tms_state* st, void* stream) {
  if (!st->reset_pending) return TMS_OK;
  TMS_HIP(tms::launch_reset(st->trie->dev, st->dev, reset_kind(st), static_cast<hipStream_t>(stream)),
          "reset launch");
  reset_enqueued(st);
  st->snap_valid = true;  // the reset kernel put every sequence at the root in half 0
  st->snap_parity = 0;
  return TMS_OK;
}

// Whether the caller is recording stream s into a graph.  Recorded work runs
// at each replay, not now, so what the host tracks about the device (the
// snapshot below) does not hold for it.
static bool is_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

// The grouped step's snapshot must hold the current nodes in half `parity`
// before a grouped step reads it; rewrites it from the state when stale, and
// always when recorded into a graph, so that every replay starts from a
// snapshot of its own (the callers then mark it stale for the eager calls
// that follow the recording).
static tms_status ensure_snapshot(tms_state* st, int parity, hipStream_t s) {
  if (st->snap_valid && st->snap_parity == parity && !is_capturing(s)) return TMS_OK;
  TMS_HIP(tms::launch_snapshot(st->dev, parity, s), "snapshot launch");
  st->snap_valid = true;
  st->snap_parity = parity;
  return TMS_OK;
}

tms_status tms_state_reset(tms_state* st, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  (void)stream;
  st->reset_pending = true;
  st->live_dirty = false;
  return TMS_OK;
}

#define TMS_FLUSH_RESET(st, stream)                   \
  do {                                                \
    const tms_status frs = flush_reset(st, stream);   \
    if (frs != TMS_OK) return frs;                    \
  } while (0)

tms_status tms_state_sync_status(tms_state* st, int32_t* host_status, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  TMS_FLUSH_RESET(st, stream);
  TMS_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "stream synchronize");
  TMS_HIP(hipMemcpy(st->host_status.data(), st->dev.status, 4 * st->B, hipMemcpyDeviceToHost), "status copy");
  if (host_status) std::memcpy(host_status, st->host_status.data(), 4 * st->B);
  for (int s = 0; s < st->B; ++s) {
    if (st->host_status[s] != 0) {
      g_err = "sequence " + std::to_string(s) + ": " + tms_status_str(static_cast<tms_status>(st->host_status[s]));
      return static_cast<tms_status>(st->host_status[s]);
    }
  }
  return TMS_OK;
}

tms_status tms_state_export(tms_state* st, int32_t* node, int32_t* depth, int32_t* done, int32_t* status,
                            int32_t* finished, int32_t* n_emitted, int32_t* entries, int32_t* live, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  TMS_FLUSH_RESET(st, stream);
  TMS_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "stream synchronize");
  const size_t b4 = 4 * size_t(st->B);
  const tms::DevState& d = st->dev;
  if (node) TMS_HIP(hipMemcpy(node, d.node, b4, hipMemcpyDeviceToHost), "export");
  if (depth) TMS_HIP(hipMemcpy(depth, d.depth, b4, hipMemcpyDeviceToHost), "export");
  if (done) TMS_HIP(hipMemcpy(done, d.done, b4, hipMemcpyDeviceToHost), "export");
  if (status) TMS_HIP(hipMemcpy(status, d.status, b4, hipMemcpyDeviceToHost), "export");
  if (finished) TMS_HIP(hipMemcpy(finished, d.finished, b4, hipMemcpyDeviceToHost), "export");
  if (n_emitted) TMS_HIP(hipMemcpy(n_emitted, d.nemit, b4, hipMemcpyDeviceToHost), "export");
  if (entries) TMS_HIP(hipMemcpy(entries, d.entries, b4 * st->k, hipMemcpyDeviceToHost), "export");
  if (live) {
    const int E = st->trie->host.n_edges;
    const int64_t ls = st->trie->dev.live_stride;
    TMS_HIP(hipMemcpy2D(live, 4 * size_t(E), d.live, 4 * size_t(ls), 4 * size_t(E), st->B, hipMemcpyDeviceToHost),
            "export live");
  }
  return TMS_OK;
}

tms_status tms_state_free(tms_state* st) {
  if (!st) return TMS_OK;
  destroy_graph(st);
  if (st->capture) (void)hipStreamDestroy(st->capture);
  if (st->dmem) (void)hipFree(st->dmem);
  if (st->trie) st->trie->refs--;
  delete st;
  return TMS_OK;
}

tms_status tms_decode_step_sparse(tms_state* st, const void* hidden, int32_t* tok, float* logit, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  if (!hidden || !aligned16(hidden)) return fail(TMS_ERR_INVALID_ARG, "hidden null or not 16-byte aligned");
  TMS_FLUSH_RESET(st, stream);
  tms::StepIO io = make_io(st, hidden);
  io.out_tok = tok;
  io.out_logit = logit;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool cap = is_capturing(s);
  tms::StepGroup* g = step_group(st);
  if (g) {
    const tms_status rs = ensure_snapshot(st, st->snap_parity, s);
    if (rs != TMS_OK) return rs;
    g->parity = st->snap_parity;
  }
  TMS_HIP(tms::launch_step_sparse(st->trie->dev, st->dev, io, st->dtype, st->fast, st->split, s, g),
          "sparse step launch");
  if (g && !cap) st->snap_parity ^= 1;  // the step wrote the other half
  else st->snap_valid = false;
  return TMS_OK;
}

tms_status tms_decode_step_dense_masked(tms_state* st, const void* hidden, int32_t* tok, float* logit,
                                        float* full_logits, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  if (!hidden || !aligned16(hidden)) return fail(TMS_ERR_INVALID_ARG, "hidden null or not 16-byte aligned");
  if (size_t(st->dev.mask_words) * 4 > 65536) return fail(TMS_ERR_INVALID_ARG, "vocabulary too large for the dense mask");
  TMS_FLUSH_RESET(st, stream);
  tms::StepIO io = make_io(st, hidden);
  io.out_tok = tok;
  io.out_logit = logit;
  st->snap_valid = false;
  TMS_HIP(tms::launch_dense_step(st->trie->dev, st->dev, io, st->dtype, full_logits, 0, st->dense_mfma,
                                 static_cast<hipStream_t>(stream)),
          "dense step launch");
  return TMS_OK;
}

tms_status tms_decode_k_pointers(tms_state* st, const void* hidden_seq, int32_t T, int32_t* tokens, int32_t* len,
                                 int32_t* entries, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  if (!hidden_seq || !aligned16(hidden_seq) || !tokens)
    return fail(TMS_ERR_INVALID_ARG, "hidden_seq or tokens null, or hidden_seq not 16-byte aligned");
  const int32_t need = st->k * (st->trie->host.max_depth + 1);
  if (T < need)
    return fail(TMS_ERR_INVALID_ARG, "T = " + std::to_string(T) + " < k*(max_depth+1) = " + std::to_string(need));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool resident = st->loop_mode == TMS_LOOP_RESIDENT || st->loop_mode == TMS_LOOP_RESIDENT_SOLO ||
                        st->loop_mode == TMS_LOOP_RESIDENT_GROUPED;
  if (resident) {
    tms::LoopIO io{};
    io.emb = st->emb;
    io.hidden_seq = hidden_seq;
    io.H = st->H;
    io.V = st->trie->host.vocab;
    io.T = T;
    io.tokens_bt = tokens;
    io.len = len;
    io.entries = entries;
    const bool fresh = st->reset_pending;  // every sequence starts at the root
    io.reset = reset_kind(st);             // the kernel resets its sequence first
    const bool bitmask = st->norepeat == TMS_NOREPEAT_BITMASK && !st->live_dirty;
    st->snap_valid = false;
    TMS_HIP(tms::enqueue_resident(st->trie, st->dev, io, st->dtype, st->fast, st->loop_mode, fresh, bitmask, s),
            "loop launch");
    if (fresh) reset_enqueued(st);
    return TMS_OK;
  }
  TMS_FLUSH_RESET(st, stream);
  const size_t step_bytes = size_t(st->B) * st->H * elem_size(st->dtype);
  tms::StepGroup* grp = step_group(st);
  // grouped steps alternate the snapshot halves: step t of a call starting at
  // half p0 reads half (p0 + t) & 1 (the captured graph always starts at 0)
  auto enqueue = [&](hipStream_t q, int p0) -> hipError_t {
    for (int32_t t = 0; t < T; ++t) {
      tms::StepIO io = make_io(st, static_cast<const char*>(hidden_seq) + step_bytes * t);
      io.tokens_bt = tokens;
      io.T = T;
      io.t = t;
      tms::StepGroup g{};
      if (grp) {
        g = *grp;
        g.parity = (p0 + t) & 1;
      }
      hipError_t e = tms::launch_step_sparse(st->trie->dev, st->dev, io, st->dtype, st->fast, st->split, q,
                                             grp ? &g : nullptr);
      if (e != hipSuccess) return e;
    }
    return tms::launch_finalize(st->dev, len, entries, q);
  };
  // a caller recording the stream into a graph records the step kernels
  // themselves (the library's own graph is not launched into a recording)
  const bool cap = is_capturing(s);
  if (st->loop_mode == TMS_LOOP_STREAM || cap) {
    const int p0 = st->snap_valid ? st->snap_parity : 0;
    if (grp) {
      const tms_status rs = ensure_snapshot(st, p0, s);
      if (rs != TMS_OK) return rs;
    }
    TMS_HIP(enqueue(s, p0), "step loop launch");
    if (grp && !cap) st->snap_parity = (p0 + T) & 1;
    else st->snap_valid = false;
    return TMS_OK;
  }
  const bool same = st->gexec && st->g_hidden == hidden_seq && st->g_T == T && st->g_tokens == tokens &&
                    st->g_len == len && st->g_entries == entries;
  if (!same) {
    TMS_HIP(hipStreamBeginCapture(st->capture, hipStreamCaptureModeRelaxed), "begin capture");
    const hipError_t le = enqueue(st->capture, 0);
    hipGraph_t g = nullptr;
    const hipError_t ce = hipStreamEndCapture(st->capture, &g);
    if (le != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      return hip_fail(le, "capture launch");
    }
    TMS_HIP(ce, "end capture");
    // the same step count keeps the graph's shape: only kernel arguments
    // (buffer pointers) differ, so the instantiated graph takes them in place;
    // otherwise (first call, another T, an update refused) it is rebuilt
    bool updated = false;
    if (st->gexec && st->g_T == T) {
      // a launch of the old arguments may still be queued: let it finish first
      TMS_HIP(hipDeviceSynchronize(), "graph update wait");
      hipGraphExecUpdateResult ur = hipGraphExecUpdateError;
      hipGraphNode_t bad = nullptr;
      updated = hipGraphExecUpdate(st->gexec, g, &bad, &ur) == hipSuccess && ur == hipGraphExecUpdateSuccess;
      if (!updated) (void)hipGetLastError();  // clear the refused update's error
    }
    if (updated) {
      (void)hipGraphDestroy(st->graph);
      st->graph = g;
    } else {
      if (st->gexec) TMS_HIP(hipDeviceSynchronize(), "graph rebuild wait");
      destroy_graph(st);
      st->graph = g;
      TMS_HIP(hipGraphInstantiate(&st->gexec, g, nullptr, nullptr, 0), "graph instantiate");
    }
    st->g_hidden = hidden_seq;
    st->g_T = T;
    st->g_tokens = tokens;
    st->g_len = len;
    st->g_entries = entries;
  }
  if (grp) {
    const tms_status rs = ensure_snapshot(st, 0, s);
    if (rs != TMS_OK) return rs;
  }
  TMS_HIP(hipGraphLaunch(st->gexec, s), "graph launch");
  if (grp) st->snap_parity = T & 1;
  else st->snap_valid = false;
  return TMS_OK;
}

tms_status tms_advance_forced(tms_state* st, const int32_t* tok, void* stream) {
  if (!st || !tok) return fail(TMS_ERR_INVALID_ARG, "null argument");
  TMS_FLUSH_RESET(st, stream);
  st->snap_valid = false;
  TMS_HIP(tms::launch_forced(st->trie->dev, st->dev, tok, static_cast<hipStream_t>(stream)), "forced launch");
  return TMS_OK;
}

tms_status tms_legal_set(tms_state* st, int32_t* legal_tok, int32_t* n_legal, void* stream) {
  if (!st || !legal_tok || !n_legal) return fail(TMS_ERR_INVALID_ARG, "null argument");
  TMS_FLUSH_RESET(st, stream);
  TMS_HIP(tms::launch_legal_set(st->trie->dev, st->dev, legal_tok, n_legal, static_cast<hipStream_t>(stream)),
          "legal set launch");
  return TMS_OK;
}

tms_status tms_legal_mask(tms_state* st, uint32_t* mask, void* stream) {
  if (!st || !mask) return fail(TMS_ERR_INVALID_ARG, "null argument");
  if (size_t(st->dev.mask_words) * 4 > 65536) return fail(TMS_ERR_INVALID_ARG, "vocabulary too large for the mask");
  TMS_FLUSH_RESET(st, stream);
  TMS_HIP(tms::launch_legal_mask(st->trie->dev, st->dev, mask, static_cast<hipStream_t>(stream)), "legal mask launch");
  return TMS_OK;
}

tms_status tms_mask_to_rows(const uint32_t* mask, int32_t B, int32_t V, int32_t cap, int32_t* rows,
                            int32_t* n_rows, void* stream) {
  if (!mask || !rows || !n_rows) return fail(TMS_ERR_INVALID_ARG, "null argument");
  if (B < 1 || V < 1 || cap < 0) return fail(TMS_ERR_INVALID_ARG, "B and V must be positive, cap not negative");
  if (V > (1 << 19)) return fail(TMS_ERR_INVALID_ARG, "V above 2^19 (a mask row is staged in 64 KiB of LDS)");
  TMS_HIP(tms::launch_mask_rows(mask, B, V, cap, rows, n_rows, static_cast<hipStream_t>(stream)), "mask rows launch");
  return TMS_OK;
}

tms_status tms_gather_gemv(const void* emb, tms_dtype dtype, int32_t V, int32_t H, const void* hidden,
                           const int32_t* rows, const int32_t* n_rows, int32_t B, int32_t cap, float* out,
                           void* stream) {
  if (!emb || !hidden || !rows || !n_rows || !out) return fail(TMS_ERR_INVALID_ARG, "null argument");
  if (!aligned16(emb) || !aligned16(hidden)) return fail(TMS_ERR_INVALID_ARG, "emb/hidden not 16-byte aligned");
  if (dtype != TMS_F32 && dtype != TMS_BF16) return fail(TMS_ERR_INVALID_ARG, "dtype must be fp32 or bf16");
  if (V < 1 || B < 1 || cap < 1 || B > (1 << 24)) return fail(TMS_ERR_INVALID_ARG, "bad sizes");
  if (tms::chunks_for(dtype, H) == 0) return fail(TMS_ERR_INVALID_ARG, "unsupported H");
  // workgroups per sequence: each wavefront owns at most 64 consecutive slots
  static const int env_split = [] {
    const char* e = std::getenv("TMS_GEMV_SPLIT");
    return e ? std::atoi(e) : 0;
  }();
  int split = env_split > 0 ? env_split : gemv_split(B, cap);
  split = std::max(split, (cap + 255) / 256);
  if (int64_t(B) * split > (int64_t(1) << 31) - 1) return fail(TMS_ERR_INVALID_ARG, "grid too large");
  TMS_HIP(tms::launch_gather_gemv(emb, dtype, V, H, hidden, rows, n_rows, B, cap, out, split,
                                  static_cast<hipStream_t>(stream)),
          "gather gemv launch");
  return TMS_OK;
}

tms_status tms_read_reference(const void* src, int64_t bytes, uint32_t* out, int32_t grid, int32_t unroll,
                              void* stream) {
  if (!src || !out || !aligned16(src)) return fail(TMS_ERR_INVALID_ARG, "src or out null, or src not 16-byte aligned");
  if (bytes < 16 || bytes % 16) return fail(TMS_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (grid < 0 || (unroll != 0 && unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8))
    return fail(TMS_ERR_INVALID_ARG, "grid must be >= 0 and unroll one of 0, 1, 2, 4, 8");
  TMS_HIP(tms::launch_read_reference(src, bytes, out, grid, unroll, static_cast<hipStream_t>(stream)),
          "read reference launch");
  return TMS_OK;
}

tms_status tms_debug_set_live(tms_state* st, int32_t s, int32_t edge, int32_t value, void* stream) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  if (s < 0 || s >= st->B || edge < 0 || edge >= st->trie->host.n_edges)
    return fail(TMS_ERR_INVALID_ARG, "sequence or edge out of range");
  TMS_FLUSH_RESET(st, stream);
  st->live_dirty = true;
  st->live_by_paths = false;
  TMS_HIP(tms::launch_set_live(st->trie->dev, st->dev, s, edge, value, static_cast<hipStream_t>(stream)),
          "set live launch");
  return TMS_OK;
}

tms_status tms_state_set_split(tms_state* st, int32_t split) {
  if (!st || split < 0 || split > 4096) return fail(TMS_ERR_INVALID_ARG, "split must be in [0, 4096]");
  st->split = split == 0 ? st->split_default : split;
  st->grp.split = split == 0 ? st->grp_split_default : split;
  destroy_graph(st);
  return TMS_OK;
}

tms_status tms_state_set_step_grouping(tms_state* st, int32_t mode) {
  if (!st || mode < TMS_STEP_GROUP_AUTO || mode > TMS_STEP_GROUP_NODES)
    return fail(TMS_ERR_INVALID_ARG, "unknown step grouping mode");
  if ((mode == TMS_STEP_GROUP_ROOT || mode == TMS_STEP_GROUP_NODES) && !st->step_group_ok)
    return fail(TMS_ERR_INVALID_ARG, "step grouping does not fit this state (LDS for the members' vectors)");
  st->step_group_mode = mode;
  destroy_graph(st);
  return TMS_OK;
}

tms_status tms_state_set_loop(tms_state* st, int32_t mode) {
  if (!st || mode < TMS_LOOP_RESIDENT || mode > TMS_LOOP_RESIDENT_GROUPED)
    return fail(TMS_ERR_INVALID_ARG, "unknown loop mode");
  st->loop_mode = mode;
  destroy_graph(st);
  return TMS_OK;
}

tms_status tms_state_set_norepeat(tms_state* st, int32_t kind) {
  if (!st || (kind != TMS_NOREPEAT_LIVE && kind != TMS_NOREPEAT_BITMASK))
    return fail(TMS_ERR_INVALID_ARG, "unknown no-repeat state");
  if (kind == TMS_NOREPEAT_BITMASK && !st->trie->dev.emask)
    return fail(TMS_ERR_INVALID_ARG, "the bitmask no-repeat state needs a catalog of at most 128 entries");
  st->norepeat = kind;
  return TMS_OK;
}

tms_status tms_state_get_launch(const tms_state* st, int32_t* split, int32_t* grid) {
  if (!st) return fail(TMS_ERR_INVALID_ARG, "null state");
  const tms::StepGroup* g = step_group(st);
  if (split) *split = g ? g->split : st->split;
  if (grid) *grid = g ? st->B * g->split + tms::root_tile_grid(g->rt, g->mtiles) : st->B * st->split;
  return TMS_OK;
}

}  // extern "C"
