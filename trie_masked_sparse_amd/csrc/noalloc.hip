// Allocation-free form of the device loop (tms_decode_k_pointers_noalloc).
//
// The per-sequence decode state of one whole answer (node, path, live counts,
// spent flags, entries, argmax slots) is scratch for a call that starts every
// sequence from the reset state, so it is carved out of one file-scope device
// array instead of a state handle's allocation.  Each GPU holds its own copy
// of the array (allocated with the code object, kept until the process ends);
// its device address is taken once per GPU with hipGetSymbolAddress and only
// that address is handed to kernels.  The resident loop is launched with a
// full reset, which writes every word of the state it later reads (live counts
// from live0, spent flags, entries, node and counters), so the array needs no
// clearing and nothing carries over between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "handles.h"

namespace {
constexpr size_t kScratchBytes = static_cast<size_t>(TMS_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;
}  // namespace

// The scratch array.  In host code this name is only a stand-in for the
// symbol: host code uses the per-device address below, never the name.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of scratch on device dev (the current device), taken on the
// first call for that device.
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Offsets of the state arrays inside the scratch, 256-byte aligned each, in
// the order of the state handle's own layout (the dense path's mask is not
// used by the loop and has no place here).
struct Layout {
  size_t node, depth, done, status, fin, nemit, path, entries, key, arrive, tstep, rkey, live, spent, total;
};

Layout layout(const tms::HostTrie& h, int64_t live_stride, int B, int k, int root_tiles) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  const size_t b4 = 4 * size_t(B);
  L.node = take(b4);
  L.depth = take(b4);
  L.done = take(b4);
  L.status = take(b4);
  L.fin = take(b4);
  L.nemit = take(b4);
  L.path = take(b4 * size_t(std::max(1, h.max_depth)));
  L.entries = take(b4 * size_t(k));
  L.key = take(8 * size_t(B));
  L.arrive = take(b4);
  L.tstep = take(b4);
  L.rkey = take(8 * size_t(root_tiles) * size_t(B));
  L.live = take(b4 * size_t(live_stride));
  L.spent = take(b4 * size_t((h.n_entries + 31) / 32));
  L.total = off;
  return L;
}

}  // namespace

extern "C" tms_status tms_decode_k_pointers_noalloc(const tms_trie* trie, const void* emb, tms_dtype dtype,
                                                    int32_t H, int32_t B, int32_t k, const void* hidden_seq,
                                                    int32_t T, int32_t* tokens, int32_t* len, int32_t* entries,
                                                    int32_t* status, void* stream) {
  using tms::api_fail;
  if (!trie || !trie->dmem) return api_fail(TMS_ERR_INVALID_ARG, "trie has no device copy (use tms_trie_upload)");
  if (B < 1 || B > 65535) return api_fail(TMS_ERR_INVALID_ARG, "B must be in [1, 65535]");
  const tms::HostTrie& h = trie->host;
  if (k < 1 || k > h.n_entries)
    return api_fail(TMS_ERR_K, "k = " + std::to_string(k) + " outside [1, " + std::to_string(h.n_entries) + "]");
  if (trie->charset && k != 1) return api_fail(TMS_ERR_K, "a character catalog answers with one string (k = 1)");
  if (dtype != TMS_F32 && dtype != TMS_BF16) return api_fail(TMS_ERR_INVALID_ARG, "dtype must be fp32 or bf16");
  auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!emb || !aligned16(emb)) return api_fail(TMS_ERR_INVALID_ARG, "embedding pointer null or not 16-byte aligned");
  if (tms::chunks_for(dtype, H) == 0) return api_fail(TMS_ERR_INVALID_ARG, "unsupported H for this dtype");
  if (!hidden_seq || !aligned16(hidden_seq) || !tokens || !status)
    return api_fail(TMS_ERR_INVALID_ARG, "hidden_seq, tokens or status null, or hidden_seq not 16-byte aligned");
  const int32_t need = k * (h.max_depth + 1);
  if (T < need)
    return api_fail(TMS_ERR_INVALID_ARG, "T = " + std::to_string(T) + " < k*(max_depth+1) = " + std::to_string(need));
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return tms::api_hip_fail(e, "hipGetDevice");
  if (dev != trie->device) return api_fail(TMS_ERR_INVALID_ARG, "trie was uploaded on another device");
  if (dev < 0 || dev >= kMaxDevices) return api_fail(TMS_ERR_INVALID_ARG, "device index above the supported range");
  const int root_tiles = (h.begin[1] - h.begin[0] + 3) / 4;
  const Layout L = layout(h, trie->dev.live_stride, B, k, root_tiles);
  if (L.total > kScratchBytes)
    return api_fail(TMS_ERR_INVALID_ARG, "this batch needs " + std::to_string(L.total) +
                                             " bytes of decode state, above the allocation-free limit of " +
                                             std::to_string(kScratchBytes));
  void* base_v = nullptr;
  if (hipError_t e = scratch_address(dev, &base_v); e != hipSuccess) return tms::api_hip_fail(e, "scratch address");
  char* base = static_cast<char*>(base_v);
  tms::DevState d{};
  d.B = B;
  d.k = k;
  d.path_stride = std::max(1, h.max_depth);
  d.spent_words = (h.n_entries + 31) / 32;
  d.mask_words = (h.vocab + 31) / 32;
  d.node = reinterpret_cast<int32_t*>(base + L.node);
  d.depth = reinterpret_cast<int32_t*>(base + L.depth);
  d.done = reinterpret_cast<int32_t*>(base + L.done);
  d.status = status;  // the caller's status array is the state's: written by the kernels before any read
  d.finished = reinterpret_cast<int32_t*>(base + L.fin);
  d.nemit = reinterpret_cast<int32_t*>(base + L.nemit);
  d.path = reinterpret_cast<int32_t*>(base + L.path);
  d.entries = reinterpret_cast<int32_t*>(base + L.entries);
  d.key = reinterpret_cast<unsigned long long*>(base + L.key);
  d.arrive = reinterpret_cast<uint32_t*>(base + L.arrive);
  d.tstep = reinterpret_cast<int32_t*>(base + L.tstep);
  d.rkey = reinterpret_cast<unsigned long long*>(base + L.rkey);
  d.root_tiles = root_tiles;
  d.live = reinterpret_cast<int32_t*>(base + L.live);
  d.spent = reinterpret_cast<uint32_t*>(base + L.spent);
  d.mask = nullptr;
  tms::LoopIO io{};
  io.emb = emb;
  io.hidden_seq = hidden_seq;
  io.H = H;
  io.V = h.vocab;
  io.T = T;
  io.tokens_bt = tokens;
  io.len = len;
  io.entries = entries;
  io.reset = tms::kResetFull;
  const hipError_t e = tms::enqueue_resident(trie, d, io, dtype, trie->path == TMS_PATH_FAST, TMS_LOOP_RESIDENT,
                                             /*fresh=*/true, /*bitmask=*/false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return tms::api_hip_fail(e, "loop launch");
  return TMS_OK;
}
