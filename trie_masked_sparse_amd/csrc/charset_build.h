// Host-side compiler of character-level catalogs (byte strings + a token
// vocabulary of byte strings) into the trie form the decode kernels read.
// HIP-free so that it builds and runs without a GPU.
#pragma once
#include <cstdint>
#include <string>

#include "trie_build.h"

namespace tms {

// Returns 0 on success, otherwise a tms_status code with a message in *err.
int build_charset(const uint8_t* bytes, const int64_t* offsets, int32_t K, const uint8_t* token_bytes,
                  const int64_t* token_offsets, int32_t V, int32_t sep, int32_t stop, HostTrie* out,
                  std::string* err);

}  // namespace tms
