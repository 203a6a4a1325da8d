// Sanitizer driver for the library's host-side catalog compiler
// (trie_masked_sparse_amd/csrc/trie_build.cpp): built under
// -fsanitize=address,undefined and run by tests/test_sanitize.py.  Seeded
// random catalogs (shared prefixes, prefix pairs, duplicates, wide nodes,
// both placements of the control ids) and rejected inputs; each built trie is
// checked against its own contract (ranges cover the edges, breadth-first
// children, tokens ascending within a node, control edges only on terminals,
// live0 = entries below a content edge).  Prints "ok <tries>".
#include <cstdint>
#include <cstdio>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "trie_build.h"

static int fail(const char* what, int c) {
  std::fprintf(stderr, "case %d: %s\n", c, what);
  return 1;
}

int main() {
  std::mt19937_64 rng(20261202);
  int built = 0;
  for (int c = 0; c < 1500; ++c) {
    const int32_t V = 8 + int32_t(rng() % 1500);
    const bool high = c & 1;
    const int32_t sep = high ? V - 2 : 0, stop = high ? V - 1 : 1;
    const int32_t want = 1 + int32_t(rng() % 300);
    const int32_t maxlen = 1 + int32_t(rng() % 8);
    const int32_t idr = 2 + int32_t(rng() % std::min<int32_t>(V - 4, c % 3 == 0 ? 600 : 10));
    // distinct entries (every 7th case keeps one duplicate, which must be rejected)
    std::set<std::vector<int32_t>> seen;
    std::vector<int64_t> off(1, 0);
    std::vector<int32_t> tok;
    for (int32_t i = 0; i < 4 * want && int32_t(off.size()) <= want; ++i) {
      std::vector<int32_t> e(1 + rng() % maxlen);
      for (auto& x : e) x = 2 + int32_t(rng() % idr);  // never 0/1 or V-2/V-1
      if (!seen.insert(e).second && !(c % 7 == 0 && off.size() == 2)) continue;
      tok.insert(tok.end(), e.begin(), e.end());
      off.push_back(int64_t(tok.size()));
    }
    const int32_t K = int32_t(off.size()) - 1;
    if (tok.empty()) tok.push_back(2);
    tms::HostTrie h;
    std::string err;
    const int rc = tms::build_trie(tok.data(), off.data(), K, V, sep, stop, &h, &err);
    if (rc != 0) {
      if (err.empty()) return fail("error without a message", c);
      continue;  // duplicates are rejected
    }
    ++built;
    if (int(h.begin.size()) != h.n_nodes + 1 || h.begin[h.n_nodes] != h.n_edges) return fail("ranges", c);
    int32_t next_child = 1;
    std::vector<int32_t> below(h.n_nodes, 0);
    for (int32_t n = 0; n < h.n_nodes; ++n) {
      for (int32_t e = h.begin[n]; e < h.begin[n + 1]; ++e) {
        if (e > h.begin[n] && h.tok[e] <= h.tok[e - 1]) return fail("tokens not ascending", c);
        if (h.child[e] >= 0) {
          if (h.child[e] != next_child++) return fail("not breadth first", c);
        } else if (h.entry[n] < 0 || (h.child[e] == -1) != (h.tok[e] == sep)) {
          return fail("control edge", c);
        }
      }
    }
    if (next_child != h.n_nodes) return fail("node count", c);
    // live0 of a content edge = entries ending at or below its child
    for (int32_t n = h.n_nodes - 1; n >= 0; --n) {
      int32_t s = h.entry[n] >= 0 ? 1 : 0;
      for (int32_t e = h.begin[n]; e < h.begin[n + 1]; ++e)
        if (h.child[e] >= 0) {
          s += below[h.child[e]];
          if (h.live0[e] != below[h.child[e]]) return fail("live0", c);
        }
      below[n] = s;
    }
    if (below[0] != K) return fail("entries", c);
  }
  // rejected inputs
  {
    tms::HostTrie h;
    std::string err;
    const int32_t tok[3] = {5, 6, 7};
    const int64_t off_empty[3] = {0, 1, 1};
    if (tms::build_trie(tok, off_empty, 2, 16, 14, 15, &h, &err) == 0) return fail("empty entry", -1);
    const int64_t off1[2] = {0, 3};
    const int32_t bad[3] = {5, 15, 7};
    if (tms::build_trie(bad, off1, 1, 16, 14, 15, &h, &err) == 0) return fail("stop inside an entry", -1);
    const int32_t big[3] = {5, 16, 7};
    if (tms::build_trie(big, off1, 1, 16, 14, 15, &h, &err) == 0) return fail("token outside V", -1);
    if (tms::build_trie(tok, off1, 1, 16, 15, 15, &h, &err) == 0) return fail("sep == stop", -1);
    if (tms::build_trie(nullptr, off1, 1, 16, 14, 15, &h, &err) == 0) return fail("null tokens", -1);
  }
  std::printf("ok %d\n", built);
  return 0;
}
