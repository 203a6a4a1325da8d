// Catalog compiler: validated token-id strings -> canonical CSR trie.
//
// Follows "Constraint made cheaper than no constraint", section "The grammar
// as a trie over tokens": the registry becomes a trie over the model's token
// ids in compressed-sparse-row form (an edge range per node, a token and a
// child per edge) with two sentinel children for the control edges
// (separator -> -1, stop -> -2).  Each content edge carries the number of
// catalog entries below it, the starting value of the per-sequence live count
// of section "Masked sampling inside the sampler".
//
// Canonical form (so that any correct builder produces identical arrays):
// nodes are numbered breadth first from root 0, children visited in ascending
// token order; a node's edge range lists its content edges and, for a
// terminal, the sep and stop edges, all in ascending token order.
//
// Construction: sort the entries lexicographically, then create nodes in
// depth-first preorder from the longest common prefix of neighbouring entries
// (children appear in ascending token order for free), count terminals per
// subtree in reverse preorder, and finally renumber breadth first.
#include "trie_build.h"

#include <algorithm>
#include <numeric>

namespace tms {

namespace {
enum { kOk = 0, kInvalidArg = 1, kCatalog = 2 };
}

int build_trie(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab,
               int32_t sep, int32_t stop, HostTrie* out, std::string* err) {
  if (!tokens || !offsets || !out) { *err = "null argument"; return kInvalidArg; }
  if (K < 1) { *err = "catalog needs at least one entry"; return kInvalidArg; }
  if (vocab < 2 || sep < 0 || sep >= vocab || stop < 0 || stop >= vocab || sep == stop) {
    *err = "sep and stop must be distinct ids in [0, vocab)";
    return kInvalidArg;
  }
  if (offsets[0] != 0) { *err = "offsets[0] must be 0"; return kCatalog; }
  const int64_t total = offsets[K];
  if (total >= (int64_t(1) << 30)) { *err = "catalog too large (>= 2^30 tokens)"; return kCatalog; }
  int32_t max_depth = 0;
  for (int32_t i = 0; i < K; ++i) {
    const int64_t a = offsets[i], b = offsets[i + 1];
    if (b <= a) { *err = "entry " + std::to_string(i) + " is empty"; return kCatalog; }
    max_depth = std::max<int32_t>(max_depth, int32_t(b - a));
    for (int64_t j = a; j < b; ++j) {
      const int32_t t = tokens[j];
      if (t < 0 || t >= vocab) {
        *err = "entry " + std::to_string(i) + " has token " + std::to_string(t) + " outside [0, vocab)";
        return kCatalog;
      }
      if (t == sep || t == stop) {
        *err = "entry " + std::to_string(i) + " contains a control token";
        return kCatalog;
      }
    }
  }

  // lexicographic order of the entries
  std::vector<int32_t> order(K);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return std::lexicographical_compare(tokens + offsets[x], tokens + offsets[x + 1],
                                        tokens + offsets[y], tokens + offsets[y + 1]);
  });

  // preorder tree: node 0 is the root
  std::vector<int32_t> in_tok(1, -1), term(1, -1), first_child(1, -1), next_sib(1, -1),
      last_child(1, -1);
  in_tok.reserve(total + 1);
  std::vector<int32_t> path(1, 0);  // path[d] = node at depth d of the previous entry
  const int32_t* prev = nullptr;
  int64_t prev_len = 0;
  for (int32_t oi = 0; oi < K; ++oi) {
    const int32_t e = order[oi];
    const int32_t* x = tokens + offsets[e];
    const int64_t len = offsets[e + 1] - offsets[e];
    int64_t lcp = 0;
    if (prev) {
      const int64_t m = std::min(len, prev_len);
      while (lcp < m && x[lcp] == prev[lcp]) ++lcp;
      if (lcp == len && len == prev_len) {
        *err = "duplicate entry " + std::to_string(e);
        return kCatalog;
      }
    }
    path.resize(size_t(lcp) + 1);
    for (int64_t d = lcp; d < len; ++d) {
      const int32_t id = int32_t(in_tok.size());
      const int32_t par = path.back();
      in_tok.push_back(x[d]);
      term.push_back(-1);
      first_child.push_back(-1);
      next_sib.push_back(-1);
      last_child.push_back(-1);
      if (last_child[par] < 0) first_child[par] = id;
      else next_sib[last_child[par]] = id;
      last_child[par] = id;
      path.push_back(id);
    }
    term[path.back()] = e;
    prev = x;
    prev_len = len;
  }
  const int32_t N = int32_t(in_tok.size());

  // terminals per subtree: children have larger preorder ids than parents
  std::vector<int32_t> below(N, 0);
  for (int32_t n = N - 1; n >= 0; --n) {
    int32_t s = term[n] >= 0 ? 1 : 0;
    for (int32_t c = first_child[n]; c >= 0; c = next_sib[c]) s += below[c];
    below[n] = s;
  }

  // breadth-first renumbering
  std::vector<int32_t> bfs(N), bfs_id(N);
  int32_t head = 0, tail = 0;
  bfs[tail++] = 0;
  while (head < tail) {
    const int32_t n = bfs[head++];
    for (int32_t c = first_child[n]; c >= 0; c = next_sib[c]) bfs[tail++] = c;
  }
  for (int32_t i = 0; i < N; ++i) bfs_id[bfs[i]] = i;

  HostTrie& t = *out;
  t = HostTrie();
  t.n_nodes = N;
  t.n_entries = K;
  t.max_depth = max_depth;
  t.sep = sep;
  t.stop = stop;
  t.vocab = vocab;
  t.n_edges = (N - 1) + 2 * K;
  t.begin.resize(size_t(N) + 1);
  t.entry.resize(N);
  t.tok.resize(t.n_edges);
  t.child.resize(t.n_edges);
  t.live0.resize(t.n_edges);
  const int32_t lo_tok = std::min(sep, stop), hi_tok = std::max(sep, stop);
  const int32_t lo_child = lo_tok == sep ? -1 : -2, hi_child = lo_tok == sep ? -2 : -1;
  int32_t e = 0, cap = 0;
  for (int32_t i = 0; i < N; ++i) {
    const int32_t n = bfs[i];
    t.begin[i] = e;
    t.entry[i] = term[n];
    const bool terminal = term[n] >= 0;
    bool lo_done = !terminal, hi_done = !terminal;
    auto put_ctl = [&](int32_t tk, int32_t ch) {
      t.tok[e] = tk; t.child[e] = ch; t.live0[e] = 0; ++e;
    };
    for (int32_t c = first_child[n]; c >= 0; c = next_sib[c]) {
      if (!lo_done && lo_tok < in_tok[c]) { put_ctl(lo_tok, lo_child); lo_done = true; }
      if (!hi_done && hi_tok < in_tok[c]) { put_ctl(hi_tok, hi_child); hi_done = true; }
      t.tok[e] = in_tok[c];
      t.child[e] = bfs_id[c];
      t.live0[e] = below[c];
      ++e;
    }
    if (!lo_done) put_ctl(lo_tok, lo_child);
    if (!hi_done) put_ctl(hi_tok, hi_child);
    cap = std::max(cap, e - t.begin[i]);
  }
  t.begin[N] = e;
  t.cap = cap;
  return kOk;
}

}  // namespace tms
