// Internal definitions shared by the C ABI's translation units (not part of
// the public header): the handle types and the launch of the resident device
// loop, which both tms_decode_k_pointers and the allocation-free entry point
// enqueue.
#pragma once
#include <hip/hip_runtime_api.h>

#include <string>
#include <vector>

#include "kernels.h"
#include "tms.h"
#include "trie_build.h"

struct tms_trie {
  tms::HostTrie host;
  bool charset = false;  // built from a character catalog (one string per answer)
  int path = TMS_PATH_AUTO;  // FAST or GLOBAL once uploaded
  int device = -1;
  void* dmem = nullptr;
  size_t dbytes = 0;
  tms::DevTrie dev{};
  int refs = 0;
};

struct tms_state {
  tms_trie* trie = nullptr;
  int B = 0, k = 0, H = 0, dtype = 0, device = -1;
  const void* emb = nullptr;
  void* dmem = nullptr;
  size_t dbytes = 0;
  tms::DevState dev{};
  int split = 1, split_default = 1;
  // root grouping of the fused step (TMS_STEP_GROUP_*), its launch shape and
  // whether the state's trie and batch allow it
  int step_group_mode = TMS_STEP_GROUP_AUTO;
  bool step_group_ok = false, step_group_auto = false;
  tms::StepGroup grp{};
  int grp_split_default = 1;
  int grp_mt_root = 16, grp_mt_nodes = 4;  // members per root tile; per node-group tile
  // the grouped step's snapshot (DevState::snap): the half that holds every
  // sequence's current node, and whether it is up to date (any other call
  // that moves sequences makes it stale; the reset kernel rewrites half 0)
  int snap_parity = 0;
  bool snap_valid = false;
  bool fast = false;
  int loop_mode = TMS_LOOP_RESIDENT;
  bool dense_mfma = true;  // matrix-core dense head where it applies
  // A reset asked for and not yet carried out: the next call on the state
  // applies it on that call's stream (inside the resident loop's kernel when
  // that is the next call, otherwise as a reset kernel launched first).
  bool reset_pending = false;
  // live counts changed by tms_debug_set_live since the last reset: the
  // bitmask state (which derives liveness from the spent set) does not apply
  bool live_dirty = false;
  // the no-repeat state the resident loop keeps (TMS_NOREPEAT_*)
  int norepeat = TMS_NOREPEAT_LIVE;
  // every live row equals live0 except on the root paths of the row's stored
  // completed entries (false until the first reset has run, and after
  // tms_debug_set_live): a reset may then restore just those paths
  bool live_by_paths = false;
  hipStream_t capture = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  const void* g_hidden = nullptr;
  int32_t g_T = 0;
  int32_t *g_tokens = nullptr, *g_len = nullptr, *g_entries = nullptr;
  std::vector<int32_t> host_status;
};

namespace tms {

// Sets a thread-local error message and returns s.
tms_status api_fail(tms_status s, const std::string& msg);
tms_status api_hip_fail(hipError_t e, const char* what);

// Enqueues the resident device loop over io.T steps for the sequences of dev
// (io.reset says how their state starts; fresh: every sequence starts at the
// root): one loop kernel, or, for B >= 8 and a root of at least 64 edges (or
// TMS_LOOP_RESIDENT_GROUPED), one grouped root head plus one loop kernel per
// pointer.  bitmask: keep the bitmask no-repeat state where the trie has one.
hipError_t enqueue_resident(const tms_trie* trie, const DevState& dev, LoopIO io, int dtype, bool fast,
                            int loop_mode, bool fresh, bool bitmask, hipStream_t s);

}  // namespace tms
