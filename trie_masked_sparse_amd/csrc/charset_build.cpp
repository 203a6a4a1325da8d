// Character-level catalog compiler (source: the review of arXiv 2608.12574,
// fields pith_extraction.key_machinery and core_discovery).
//
// The catalog is a set of byte strings and the tokenizer maps each token id to
// a byte string.  A trie over the strings' bytes gets, for every node, the set
// valid[node] of tokens whose bytes can be read downward from that node
// without running off the trie, each with the node where its bytes end.  The
// sets come from one Aho-Corasick automaton over the vocabulary's byte
// strings: a depth-first walk of the trie carries the automaton's state, and
// every token the automaton reports as ending at trie node m, L bytes long, is
// a valid token of m's ancestor L bytes up (its bytes lie on the path between
// them).  That is one pass over the trie plus the automaton's construction,
// instead of testing every token at every node.
//
// The result is the trie form the decode kernels run (tms::HostTrie): nodes
// are the character trie's nodes (root 0, breadth-first), the edges of a node
// are its valid tokens in ascending id order, each leading to the node where
// the token's bytes end, and a node where a string ends carries the sep and
// stop control edges.  live0 of a token edge is the number of strings at or
// below the node it leads to.  Decoding then picks one string (k = 1): the
// legal set at a node is its valid tokens, plus stop where a string ends.
#include "charset_build.h"

#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

namespace tms {

namespace {

enum { kOk = 0, kInvalidArg = 1, kCatalog = 2 };
constexpr int32_t kSepChild = -1, kStopChild = -2;  // control-edge children, as in the token tries

// Aho-Corasick automaton over the content tokens' byte strings.
struct Matcher {
  std::vector<std::unordered_map<uint8_t, int32_t>> next;  // trie of the patterns
  std::vector<int32_t> fail;   // longest proper suffix that is a state
  std::vector<int32_t> dict;   // nearest state along the fail chain that ends a pattern (-1: none)
  std::vector<int32_t> depth;  // length of the state's string
  std::vector<std::vector<int32_t>> out;  // token ids whose bytes are exactly this state's string

  int32_t add_state(int32_t d) {
    next.emplace_back();
    fail.push_back(0);
    dict.push_back(-1);
    depth.push_back(d);
    out.emplace_back();
    return static_cast<int32_t>(next.size()) - 1;
  }

  void build(const std::vector<std::pair<const uint8_t*, int64_t>>& pats, const std::vector<int32_t>& ids) {
    add_state(0);
    for (size_t p = 0; p < pats.size(); ++p) {
      int32_t s = 0;
      for (int64_t i = 0; i < pats[p].second; ++i) {
        const uint8_t b = pats[p].first[i];
        auto it = next[s].find(b);
        if (it == next[s].end()) {
          const int32_t n = add_state(depth[s] + 1);
          next[s][b] = n;
          s = n;
        } else {
          s = it->second;
        }
      }
      out[s].push_back(ids[p]);
    }
    // fail and dictionary links, breadth first
    std::deque<int32_t> q;
    for (auto& kv : next[0]) q.push_back(kv.second);
    while (!q.empty()) {
      const int32_t s = q.front();
      q.pop_front();
      const int32_t f = fail[s];
      dict[s] = out[f].empty() ? dict[f] : f;
      for (auto& kv : next[s]) {
        const int32_t c = kv.second;
        int32_t g = f;
        for (;;) {
          auto it = next[g].find(kv.first);
          if (it != next[g].end() && it->second != c) {
            fail[c] = it->second;
            break;
          }
          if (g == 0) {
            fail[c] = 0;
            break;
          }
          g = fail[g];
        }
        q.push_back(c);
      }
    }
  }

  int32_t step(int32_t s, uint8_t b) const {
    for (;;) {
      auto it = next[s].find(b);
      if (it != next[s].end()) return it->second;
      if (s == 0) return 0;
      s = fail[s];
    }
  }
};

}  // namespace

int build_charset(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                  const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, HostTrie* out,
                  std::string* err) {
  if (!bytes || !offsets || !token_bytes || !token_offsets || !out) { *err = "null argument"; return kInvalidArg; }
  if (K < 1 || V < 2) { *err = "need at least one string and two tokens"; return kInvalidArg; }
  if (sep < 0 || sep >= V || stop < 0 || stop >= V || sep == stop) {
    *err = "sep and stop must be distinct ids in [0, V)";
    return kInvalidArg;
  }
  if (offsets[0] != 0 || token_offsets[0] != 0) { *err = "offsets must start at 0"; return kInvalidArg; }
  // content tokens: non-empty byte strings other than the control ids
  std::vector<std::pair<const uint8_t*, int64_t>> pats;
  std::vector<int32_t> ids;
  bool single[256] = {false};
  for (int32_t v = 0; v < V; ++v) {
    const int64_t L = token_offsets[v + 1] - token_offsets[v];
    if (L < 0) { *err = "token offsets decrease"; return kInvalidArg; }
    if (L == 0 || v == sep || v == stop) continue;
    pats.emplace_back(token_bytes + token_offsets[v], L);
    ids.push_back(v);
    if (L == 1) single[token_bytes[token_offsets[v]]] = true;
  }
  // character trie of the strings (children per node in a small sorted list)
  struct CNode {
    std::vector<std::pair<uint8_t, int32_t>> kids;
    int32_t entry = -1, depth = 0;
  };
  std::vector<CNode> cn(1);
  int32_t max_len = 0;
  for (int32_t i = 0; i < K; ++i) {
    const int64_t L = offsets[i + 1] - offsets[i];
    if (L <= 0) { *err = "string " + std::to_string(i) + " is empty"; return kCatalog; }
    max_len = std::max<int32_t>(max_len, static_cast<int32_t>(L));
    int32_t n = 0;
    for (int64_t j = offsets[i]; j < offsets[i + 1]; ++j) {
      const uint8_t b = bytes[j];
      if (!single[b]) {
        *err = "byte " + std::to_string(b) + " of string " + std::to_string(i) + " is no token of its own";
        return kCatalog;
      }
      auto& k = cn[n].kids;
      auto it = std::lower_bound(k.begin(), k.end(), std::make_pair(b, int32_t(-1)));
      if (it != k.end() && it->first == b) {
        n = it->second;
      } else {
        const int32_t c = static_cast<int32_t>(cn.size());
        k.insert(it, {b, c});
        cn.push_back(CNode{});
        cn[c].depth = cn[n].depth + 1;
        n = c;
      }
    }
    if (cn[n].entry >= 0) { *err = "string " + std::to_string(i) + " is a duplicate"; return kCatalog; }
    cn[n].entry = i;
  }
  const int32_t N = static_cast<int32_t>(cn.size());
  // breadth-first numbering
  std::vector<int32_t> order, bfs(N);
  order.reserve(N);
  order.push_back(0);
  for (size_t h = 0; h < order.size(); ++h)
    for (auto& kv : cn[order[h]].kids) order.push_back(kv.second);
  for (int32_t i = 0; i < N; ++i) bfs[order[i]] = i;
  // strings at or below each node (children come after parents in `order`)
  std::vector<int32_t> below(N, 0);
  for (int32_t i = N - 1; i >= 0; --i) {
    const int32_t n = order[i];
    below[n] = cn[n].entry >= 0 ? 1 : 0;
    for (auto& kv : cn[n].kids) below[n] += below[kv.second];
  }
  // valid tokens per node: the matcher carried along a depth-first walk
  Matcher ac;
  ac.build(pats, ids);
  std::vector<std::vector<std::pair<int32_t, int32_t>>> valid(N);  // (token, node where it ends)
  std::vector<int32_t> path;                                       // path[d] = node at depth d
  struct Frame {
    int32_t node, state;
    size_t next_kid;
  };
  std::vector<Frame> stack{{0, 0, 0}};
  path.push_back(0);
  while (!stack.empty()) {
    Frame& f = stack.back();
    if (f.next_kid == cn[f.node].kids.size()) {
      stack.pop_back();
      path.pop_back();
      continue;
    }
    const auto kid = cn[f.node].kids[f.next_kid++];
    const int32_t m = kid.second, s = ac.step(f.state, kid.first);
    path.push_back(m);
    const int32_t dm = cn[m].depth;
    for (int32_t t = ac.out[s].empty() ? ac.dict[s] : s; t > 0; t = ac.dict[t])
      for (const int32_t v : ac.out[t]) valid[path[dm - ac.depth[t]]].push_back({v, m});
    stack.push_back({m, s, 0});
  }
  // the CSR the kernels read
  HostTrie& h = *out;
  h = HostTrie{};
  h.n_nodes = N;
  h.n_entries = K;
  h.sep = sep;
  h.stop = stop;
  h.vocab = V;
  h.max_depth = max_len;
  h.begin.assign(N + 1, 0);
  h.entry.assign(N, -1);
  for (int32_t id = 0; id < N; ++id) {
    const int32_t n = order[id];
    auto& vs = valid[n];
    if (cn[n].entry >= 0) {
      vs.push_back({sep, kSepChild});
      vs.push_back({stop, kStopChild});
    }
    std::sort(vs.begin(), vs.end());
    h.entry[id] = cn[n].entry;
    h.begin[id] = static_cast<int32_t>(h.tok.size());
    for (auto& e : vs) {
      h.tok.push_back(e.first);
      if (e.second < 0) {
        h.child.push_back(e.second);
        h.live0.push_back(0);
      } else {
        h.child.push_back(bfs[e.second]);
        h.live0.push_back(below[e.second]);
      }
    }
    h.cap = std::max<int32_t>(h.cap, static_cast<int32_t>(vs.size()));
  }
  h.n_edges = static_cast<int32_t>(h.tok.size());
  h.begin[N] = h.n_edges;
  return kOk;
}

}  // namespace tms
