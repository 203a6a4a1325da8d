// Host-side catalog compiler: token-id strings -> canonical CSR trie.
// HIP-free so that it builds and runs without a GPU.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

namespace tms {

// Canonical CSR (see the public header for the layout contract).
struct HostTrie {
  int32_t n_nodes = 0, n_edges = 0, n_entries = 0, cap = 0, max_depth = 0;
  int32_t sep = 0, stop = 0, vocab = 0;
  std::vector<int32_t> begin;  // [n_nodes + 1]
  std::vector<int32_t> entry;  // [n_nodes]
  std::vector<int32_t> tok;    // [n_edges]
  std::vector<int32_t> child;  // [n_edges]; -1 sep, -2 stop
  std::vector<int32_t> live0;  // [n_edges]
};

// Returns 0 on success, otherwise a tms_status code with a message in *err.
int build_trie(const int32_t* tokens, const int64_t* offsets, int32_t K, int32_t vocab,
               int32_t sep, int32_t stop, HostTrie* out, std::string* err);

}  // namespace tms
