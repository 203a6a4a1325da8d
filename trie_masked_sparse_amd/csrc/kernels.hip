// HIP kernels for gfx950 (CDNA4, 64-wide wavefronts): the trie-constrained
// sparse decode step, its device loop, and the dense-plus-mask cross-check.
//
// Sources (web page "Constraint made cheaper than no constraint"):
//   section "The grammar as a trie over tokens"  - CSR trie, sentinel children;
//   section "Masked sampling inside the sampler" - filter the node's edges,
//     argmax with ties to the lower token id, fail loudly on an empty mask or
//     an unwalkable winner, exactly-k rule, live counts decremented along the
//     completed pointer's path, per-terminal spent flag;
//   section "The sparse output layer" - one dot product per legal token against
//     the tied embedding; the dense head kept as a cross-check with the same
//     tie rule and transitions; no head on steps with a single legal token;
//   section "The whole loop on the device" - the steps run on the device with
//     token, node and no-repeat state in device memory;
//   section "The batched engine" - rows shared by sequences at the same node
//     read once (the grouped root head); the bitmask no-repeat state.
// Dense-plus-mask semantics: page "GLRMask" (mask the logits, then take the
// argmax) and page "Understanding Inference for Systems Engineers", Part 7
// (the post-logit bitmask and the row list read off it).
//
// Arithmetic contract of the vector kernels (every logit of the sparse
// paths, the B = 1 dense head, the vector grouped root head):
//   lane l of a wavefront owns 16-byte chunks c = 0,1,.. of a row, i.e. the
//   elements [c*CH + l*EL, c*CH + l*EL + EL) with EL = 4 (fp32) or 8 (bf16) and
//   CH = 64*EL; it accumulates h[i]*E[v][i] in fp32 in ascending element order
//   (fp32: one fused multiply-add per element; bf16: one v_dot2_f32_bf16 per
//   pair of adjacent elements); the 64 partial sums are then combined by a fixed
//   6-level tree (see wave_sum).  The order depends only on H, never on the
//   workgroup, slot, batch size or path, so these kernels give bit-identical
//   logits.  The matrix-core heads (dense at B > 1, grouped root for bf16 with
//   H = 2048 or 4096) sum in the hardware's order, fixed for a given shape.
//
// Argmax: a 64-bit key (order-preserving fp32 bits, -0 folded into +0, in the
// high word; 0xFFFFFFFF - id in the low word) so that an unsigned max picks
// the largest logit and, among equal logits, the lowest id.  Unsigned max is
// associative and commutative, so combining per-wavefront and per-workgroup
// maxima with atomics gives the same result in any order.
#include <hip/hip_runtime.h>
#include <math.h>

#include <map>
#include <mutex>
#include <utility>

#include "kernels.h"

namespace tms {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// scalar-load views: wave-uniform addresses read through the scalar cache
typedef const __attribute__((address_space(4))) int32_t* cint_p;
typedef const __attribute__((address_space(4))) uint32_t* cuint_p;

// node record through the scalar cache (three adjacent dwords of a 16-byte record)
__device__ __forceinline__ NodeRec rec_scalar(const NodeRec* recs, int n) {
  const cint_p p = (cint_p)(recs + n);
  return NodeRec{p[0], p[1], p[2], 0};
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

__host__ __device__ constexpr int rows_per_pass(int nc) { return nc <= 4 ? 4 : (nc == 8 ? 2 : 1); }


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t h, uint32_t e, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h), __builtin_bit_cast(bf16x2_t, e), acc,
                                         false);
}

// acc += h . e over one 16-byte chunk in ascending element order: fp32 rows
// one fused multiply-add per element; bf16 rows one v_dot2_f32_bf16 per pair
// of adjacent elements (both products added to the fp32 running sum).
template <int DT>
__device__ __forceinline__ float fma_chunk(const uint4& h, const uint4& e, float acc) {
  if constexpr (DT == 0) {
    acc = fmaf(__uint_as_float(h.x), __uint_as_float(e.x), acc);
    acc = fmaf(__uint_as_float(h.y), __uint_as_float(e.y), acc);
    acc = fmaf(__uint_as_float(h.z), __uint_as_float(e.z), acc);
    acc = fmaf(__uint_as_float(h.w), __uint_as_float(e.w), acc);
  } else {
    acc = dot2_bf16(h.x, e.x, acc);
    acc = dot2_bf16(h.y, e.y, acc);
    acc = dot2_bf16(h.z, e.z, acc);
    acc = dot2_bf16(h.w, e.w, acc);
  }
  return acc;
}

// Sum over the 64 lanes in a fixed tree of depth 6: four in-row DPP levels
// (partner lane i^1, i^2, then the mirror lane within 8 and within 16, so
// each level adds two equal-size partial sums and every lane of a 16-lane row
// ends with the same row sum), then (row0 + row1) + (row2 + row3).  The result
// is wave-uniform.
#define TMS_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl), 0xF, 0xF, false))
__device__ __forceinline__ float wave_sum(float v) {
  v += TMS_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
  v += TMS_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
  v += TMS_DPP(v, 0x141);  // row_half_mirror
  v += TMS_DPP(v, 0x140);  // row_mirror
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}
#undef TMS_DPP

// Workgroup barrier that orders LDS only: outstanding global loads and stores
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Row loads of up to U rows (rows[u] < 0 skips row u).  Lanes past the end of
// a partial chunk re-read the row's first chunk and are zeroed afterwards, so
// the loads need no per-lane branches; chunks past the row end are skipped.
// NT marks the loads non-temporal (rows read once per launch: the explicit
// row-list head and the dense head); the decode step keeps rows cacheable
// because sequences at the same node share them.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int NC, int U, bool NT = false>
__device__ __forceinline__ void issue_rows(const uint4* __restrict__ emb, int nq, const int (&rows)[U],
                                           uint4 (&raw)[U][NC], int lane) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (rows[u] < 0) continue;
    const uint4* p = emb + (int64_t)rows[u] * nq;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c * kWave >= nq) break;
      const int i = c * kWave + lane;
      const uint4* a = p + (i < nq ? i : 0);
      if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a));
        raw[u][c] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        raw[u][c] = *a;
      }
    }
  }
}

// Finish the dot products started by issue_rows (fixed order, see above).
template <int DT, int NC, int U>
__device__ __forceinline__ void finish_rows(int nq, const int (&rows)[U], const uint4 (&raw)[U][NC],
                                            const uint4 (&hq)[NC], float (&out)[U], int lane) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    out[u] = 0.0f;
    if (rows[u] < 0) continue;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c * kWave >= nq) break;
      if ((c + 1) * kWave <= nq) {
        acc = fma_chunk<DT>(hq[c], raw[u][c], acc);  // full chunk
      } else {
        const float a = fma_chunk<DT>(hq[c], raw[u][c], acc);
        acc = (c * kWave + lane < nq) ? a : acc;
      }
    }
    out[u] = wave_sum(acc);
  }
}

// After a pass's dot products every row load of the pass has been consumed.
// Saying so with an explicit wait (which then waits for nothing) keeps the
// compiler's wait analysis from carrying loads of a branch it cannot prove
// consumed (row u issued, its dot product skipped: the same rows[u] < 0 test
// guards both) around the scan loops, where it otherwise waits for every
// older load, the hidden vector and the previous row included, before
// reusing a row's registers.
// (the builtin, not inline asm: the compiler's wait analysis reads the
// builtin's counts; 0x0F70 = vmcnt 0, expcnt and lgkmcnt unconstrained)
__device__ __forceinline__ void rows_consumed() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DT, int NC, int U, bool NT = false>
__device__ __forceinline__ void dot_rows(const uint4* __restrict__ emb, int nq, const int (&rows)[U],
                                         const uint4 (&hq)[NC], float (&out)[U], int lane) {
  uint4 raw[U][NC];
  issue_rows<NC, U, NT>(emb, nq, rows, raw, lane);
  finish_rows<DT, NC, U>(nq, rows, raw, hq, out, lane);
}

template <int NC>
__device__ __forceinline__ void load_hidden(const uint4* __restrict__ h, int nq, uint4 (&hq)[NC], int lane) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = c * kWave + lane;
    hq[c] = c * kWave < nq ? h[i < nq ? i : 0] : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ unsigned long long pack_key(float x, uint32_t id) {
  uint32_t b = __float_as_uint(x);
  if (x == 0.0f) b = 0u;  // -0 and +0 are the same logit
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ float key_logit(unsigned long long k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint32_t key_id(unsigned long long k) { return 0xFFFFFFFFu - (uint32_t)k; }

// Per-sequence view at the start of a step.
struct Seq {
  int node, depth, done, b0, b1;
  bool sep_ok, stop_ok;  // control edges of the current node (terminal, not spent, exactly-k rule)
};

// Reads the sequence record with scalar loads; false when s is finished or in
// error.  Section "Masked sampling inside the sampler": sep is legal at an
// unspent terminal only while another pointer is owed, stop only when none is.
__device__ __forceinline__ bool load_seq(const DevTrie& tr, const DevState& st, int s, Seq& q) {
  if (((cint_p)st.status)[s] != kSeqOk || ((cint_p)st.finished)[s] != 0) return false;
  q.node = ((cint_p)st.node)[s];
  q.depth = ((cint_p)st.depth)[s];
  q.done = ((cint_p)st.done)[s];
  const NodeRec rec = rec_scalar(tr.node_rec, q.node);
  q.b0 = rec.b0;
  q.b1 = rec.b1;
  const int ent = rec.ent;
  bool ctl = false;
  if (ent >= 0) {
    const uint32_t w = ((cuint_p)st.spent)[(int64_t)s * st.spent_words + (ent >> 5)];
    ctl = ((w >> (ent & 31)) & 1u) == 0u;
  }
  const bool more = q.done + 1 < st.k;
  q.sep_ok = ctl && more;
  q.stop_ok = ctl && !more;
  return true;
}

__device__ __forceinline__ bool edge_ok(int child, int live, const Seq& q) {
  return child >= 0 ? live > 0 : (child == kChildSep ? q.sep_ok : q.stop_ok);
}

// edge_ok without short-circuit evaluation
__device__ __forceinline__ bool edge_ok_bits(int child, int live, const Seq& q) {
  return ((child >= 0) & (live > 0)) | ((child == kChildSep) & q.sep_ok) | ((child == kChildStop) & q.stop_ok);
}

// The edge a step takes whatever the logits, when the node record decides it
// (sections "Masked sampling inside the sampler" and "The sparse output
// layer": the argmax over a single legal token is that token): a node with
// one edge holds a content edge (terminals carry two control edges), legal iff
// its live count is positive; a terminal with two edges has no content edge,
// and of its control edges sep or stop is legal by the exactly-k rule (edges
// in ascending token order).  -2: nothing is legal; -3: the head decides.
__device__ __forceinline__ int forced_edge(const DevTrie& tr, const int32_t* live, const Seq& q) {
  const int f = q.b1 - q.b0;
  if (f == 1) return ((cint_p)live)[q.b0] > 0 ? q.b0 : -2;
  if (f == 2 && (q.sep_ok || q.stop_ok)) return q.b0 + (q.sep_ok == (tr.sep < tr.stop) ? 0 : 1);
  return -3;
}

// A headless step of a sequence served by split workgroups: the advance must
// wait until every one of them has read the sequence's state (a workgroup
// that started late would otherwise read the advanced state and decide
// another step), so each counts itself into arrive[s] and the last one,
// which clears the counter, advances.  True in that workgroup only.
__device__ __forceinline__ bool forced_last(const DevState& st, int s, int split) {
  if (split == 1) return true;
  __shared__ int s_flast;
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&st.arrive[s], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (uint32_t)(split - 1);
    if (last) __hip_atomic_store(&st.arrive[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flast = last;
  }
  __syncthreads();
  return s_flast != 0;
}

__device__ __forceinline__ void write_step_out(const StepIO& io, int s, int tok, float logit) {
  if (io.out_tok) io.out_tok[s] = tok;
  if (io.out_logit) io.out_logit[s] = tok >= 0 ? logit : NAN;
  if (io.tokens_bt) io.tokens_bt[(int64_t)s * io.T + io.t] = tok;
}

// Advance sequence s along edge e (executed by one whole wavefront).
// e == -2: the mask was empty.  e outside the node's range or not legal:
// the winner is not walkable.  Both set a sticky error and stop the sequence.
// Completing a pointer: its terminal is marked spent, every content edge on
// its path loses one live pointer, and the catalog index is recorded.
// Returns the sequence's node after the step, -1 once it is finished or in error.
__device__ int advance(const DevTrie& tr, const DevState& st, const StepIO* io, int s, const Seq& q, int e,
                       float logit, int lane) {
  int status = kSeqOk, tok = -1, next = -1;
  int32_t* live = st.live + (int64_t)s * tr.live_stride;
  if (e == -2) {
    status = kSeqEmptyMask;
  } else {
    bool ok = e >= q.b0 && e < q.b1;
    int c = 0;
    if (ok) {
      c = tr.child[e];
      ok = edge_ok(c, c >= 0 ? live[e] : 0, q);
    }
    if (!ok) {
      status = kSeqNotWalkable;
    } else {
      tok = tr.tok[e];
      if (c >= 0) {
        next = c;
        if (lane == 0) {
          st.path[(int64_t)s * st.path_stride + q.depth] = e;
          st.depth[s] = q.depth + 1;
          st.node[s] = c;
        }
      } else {
        next = c == kChildStop ? -1 : 0;
        const int ent = tr.entry[q.node];
        const int32_t* path = st.path + (int64_t)s * st.path_stride;
        if (tr.release)
          for (int i = lane; i < q.depth; i += kWave) live[path[i]] -= 1;  // distinct edges
        if (lane == 0) {
          st.spent[(int64_t)s * st.spent_words + (ent >> 5)] |= 1u << (ent & 31);
          st.entries[(int64_t)s * st.k + q.done] = ent;
          st.done[s] = q.done + 1;
          st.depth[s] = 0;
          if (c == kChildStop) st.finished[s] = 1;
          else st.node[s] = 0;
        }
      }
      if (lane == 0) st.nemit[s] = st.nemit[s] + 1;
    }
  }
  if (lane == 0) {
    if (status != kSeqOk) st.status[s] = status;
    if (io) write_step_out(*io, s, tok, logit);
  }
  return status == kSeqOk ? next : -1;
}

// First edge of the node's range labelled tok, or -1 (one wavefront).
__device__ __forceinline__ int find_edge(const DevTrie& tr, const Seq& q, int tok, int lane) {
  for (int base = q.b0; base < q.b1; base += kWave) {
    const int e = base + lane;
    const unsigned long long m = __ballot(e < q.b1 && tr.tok[e] == tok);
    if (m) return base + (int)__builtin_ctzll(m);
  }
  return -1;
}

// How a scan reads live counts: through the scalar cache (state not written
// earlier in the same kernel), from LDS, with ordinary vector loads, or as
// the bitmask no-repeat state (kLiveMask: `live` is the per-edge mask of the
// entries below each edge, 128 bits, and an edge is live iff one of them is
// not in the sequence's banned set; section "The batched engine").
enum { kLiveScalar = 0, kLiveLds = 1, kLiveVector = 2, kLiveMask = 3 };

// The banned set of the bitmask state: spent entries, one bit each (K <= 128).
struct Ban {
  uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ bool mask_live(const uint4& m, const Ban& b) {
  return ((m.x & ~b.w0) | (m.y & ~b.w1) | (m.z & ~b.w2) | (m.w & ~b.w3)) != 0u;
}

template <int LIVE>
__device__ __forceinline__ int read_live_uniform(const int32_t* live, int e, const Ban& ban) {
  if constexpr (LIVE == kLiveScalar) {
    return ((cint_p)live)[e];
  } else if constexpr (LIVE == kLiveMask) {
    const uint4 m = reinterpret_cast<const uint4*>(live)[e];
    const uint4 u = make_uint4(__builtin_amdgcn_readfirstlane(m.x), __builtin_amdgcn_readfirstlane(m.y),
                               __builtin_amdgcn_readfirstlane(m.z), __builtin_amdgcn_readfirstlane(m.w));
    return mask_live(u, ban) ? 1 : 0;
  } else {
    return __builtin_amdgcn_readfirstlane(live[e]);
  }
}

// A wavefront's best candidate, carried to the advance so that it needs no
// further trie reads: the edge's child, its token and the child's record.
struct Cand {
  int child, tok, b0, b1, ent, run;
};

// Where a scan reads edge records: through the scalar cache from device
// memory (FAST), from a copy of the trie in LDS (FAST inside the resident
// loop), or with per-lane vector loads (GLOBAL).
enum { kMetaScalar = 0, kMetaLds = 1, kMetaVector = 2 };

// The trie arrays a scan reads (device memory, or their LDS copies): edge
// records and the entries of the edges' children.
struct TrieView {
  const EdgeRec* erec;
  const int32_t* cent;
  const int32_t* run;
  const int32_t* run_edge;
  const int32_t* run_tok;
  const int4* run_land;
};

// A wave-uniform edge record: scalar loads (kMetaScalar) or one 16-byte read
// whose fields are moved to scalar registers.
template <int META>
__device__ __forceinline__ EdgeRec erec_uniform(const EdgeRec* p, int i) {
  if constexpr (META == kMetaScalar) {
    const cint_p q = (cint_p)(p + i);
    return EdgeRec{q[0], q[1], q[2], q[3]};
  } else {
    const EdgeRec r = p[i];
    return EdgeRec{__builtin_amdgcn_readfirstlane(r.child), __builtin_amdgcn_readfirstlane(r.tok),
                   __builtin_amdgcn_readfirstlane(r.b0), __builtin_amdgcn_readfirstlane(r.b1)};
  }
}

// Resident-loop keys carry the wavefront index in their three low bits (below
// the edge order, so the tie rule is unchanged: edges are distinct): one LDS
// max then names both the winner and the wavefront holding its payload.
__device__ __forceinline__ unsigned long long pack_key_wave(float x, uint32_t edge, int wv) {
  const unsigned long long k = pack_key(x, 0u);
  return (k & 0xFFFFFFFF00000000ull) | (unsigned long long)(((0x1FFFFFFFu - edge) << 3) | (uint32_t)wv);
}
__device__ __forceinline__ uint32_t key_wave_edge(unsigned long long k) {
  return 0x1FFFFFFFu - ((uint32_t)k >> 3);
}

template <int META>
__device__ __forceinline__ int meta_uniform(const int32_t* p, int i) {
  if constexpr (META == kMetaScalar) return ((cint_p)p)[i];
  else return __builtin_amdgcn_readfirstlane(p[i]);
}

// Scan the current node's edge range for this wavefront's share of the
// edges (b0+wv, b0+wv+W, ...), compute a logit for every legal edge and
// return the wavefront's best packed key (0 if it had no legal edge).
// kMetaScalar/kMetaLds: wave-uniform edge records, U edges per pass, all
// requested before one wait.  kMetaVector: 64 edges per pass through per-lane
// vector loads, the legal ones compacted with a ballot, U rows in flight.
// With CAND the child's node record is fetched alongside the row gathers and
// returned in cand, and keys carry the wavefront index (pack_key_wave).
template <int DT, int NC, int META, int LIVE, bool CAND>
__device__ __forceinline__ unsigned long long scan_node(const DevTrie& tr, const TrieView& tv, const Seq& q,
                                                        const int32_t* live, const uint4* __restrict__ emb,
                                                        int nq, const uint4 (&hq)[NC], int wv, int W, int lane,
                                                        Cand& cand, const Ban& ban = Ban{0u, 0u, 0u, 0u}) {
  constexpr int U = rows_per_pass(NC);
  unsigned long long best = 0;
  auto key_of = [&](float l, int e) -> unsigned long long {
    if constexpr (CAND) return pack_key_wave(l, (uint32_t)e, wv);
    else return pack_key(l, (uint32_t)e);
  };
  if constexpr (META != kMetaVector) {
    auto pass = [&](int e0) {
      int rows[U], edges[U], chs[U];
      // edge records for all U slots first (indices clamped into the range,
      // out-of-range slots masked afterwards), then one wait
      EdgeRec rs[U];
      int lvs[U], ces[U], rns[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * W;
        const int ee = e < q.b1 ? e : q.b1 - 1;  // every node has at least one edge
        rs[u] = erec_uniform<META>(tv.erec, ee);
        lvs[u] = read_live_uniform<LIVE>(live, ee, ban);  // control edges hold 0
        ces[u] = CAND ? meta_uniform<META>(tv.cent, ee) : -1;
        rns[u] = CAND ? meta_uniform<META>(tv.run, ee) : 0;
      }
      // consume every record here so that all of them are requested together,
      // before the first row gather (the compiler would otherwise sink them)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        asm volatile("" ::"s"(rs[u].child), "s"(rs[u].tok), "s"(lvs[u]));
        if constexpr (CAND) asm volatile("" ::"s"(rs[u].b0), "s"(rs[u].b1), "s"(ces[u]), "s"(rns[u]));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * W;
        // bitwise, so that every record load above is used unconditionally
        const bool ok = (e < q.b1) & edge_ok_bits(rs[u].child, lvs[u], q);
        edges[u] = e;
        rows[u] = rs[u].tok | -(int)!ok;
        chs[u] = ok ? rs[u].child : -3;
      }
      uint4 raw[U][NC];
      issue_rows<NC, U>(emb, nq, rows, raw, lane);
      float l[U];
      finish_rows<DT, NC, U>(nq, rows, raw, hq, l, lane);
      rows_consumed();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (rows[u] < 0) continue;
        const unsigned long long k = key_of(l[u], edges[u]);
        if (k > best) {
          best = k;
          if constexpr (CAND) cand = Cand{chs[u], rows[u], rs[u].b0, rs[u].b1, ces[u], rns[u]};
        }
      }
    };
    pass(q.b0 + wv);
    for (int e0 = q.b0 + wv + U * W; e0 < q.b1; e0 += U * W) pass(e0);
  } else {
    for (int base = q.b0 + wv; base < q.b1; base += kWave * W) {
      const int e = base + lane * W;
      int tk = -1, ch = -3, rn = 0;
      NodeRec rec{0, 0, -1, 0};
      {
        const int ee = e < q.b1 ? e : q.b1 - 1;
        const EdgeRec r = tr.erec[ee];
        const int lv = live[ee];  // control edges hold 0
        const bool ok = (e < q.b1) & edge_ok_bits(r.child, lv, q);
        tk = r.tok | -(int)!ok;
        ch = ok ? r.child : -3;
        if constexpr (CAND) {
          rec = NodeRec{r.b0, r.b1, tr.cent[ee], 0};
          rn = tr.run[ee];
        }
      }
      unsigned long long m = __ballot(tk >= 0);
      while (m) {
        int rows[U], edges[U], chs[U], r0[U], r1[U], r2[U], r3[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (m) {
            const int j = (int)__builtin_ctzll(m);
            m &= m - 1;
            rows[u] = __builtin_amdgcn_readlane(tk, j);
            edges[u] = base + j * W;
            if constexpr (CAND) {
              chs[u] = __builtin_amdgcn_readlane(ch, j);
              r0[u] = __builtin_amdgcn_readlane(rec.b0, j);
              r1[u] = __builtin_amdgcn_readlane(rec.b1, j);
              r2[u] = __builtin_amdgcn_readlane(rec.ent, j);
              r3[u] = __builtin_amdgcn_readlane(rn, j);
            }
          } else {
            rows[u] = -1;
            edges[u] = 0;
            chs[u] = r0[u] = r1[u] = r2[u] = r3[u] = 0;
          }
        }
        float l[U];
        dot_rows<DT, NC, U>(emb, nq, rows, hq, l, lane);
        rows_consumed();
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (rows[u] < 0) continue;
          const unsigned long long k = key_of(l[u], edges[u]);
          if (k > best) {
            best = k;
            if constexpr (CAND) cand = Cand{chs[u], rows[u], r0[u], r1[u], r2[u], r3[u]};
          }
        }
      }
    }
  }
  return best;
}

// ---------------------------------------------------------------------------
// Fused sparse step (the host-argument form): materialise the legal set,
// gather-GEMV, argmax, advance, in one launch.
// Grid: B * split workgroups of 256 threads; workgroup g serves sequence
// g / split and its wavefronts take a strided share of the node's edges.  The
// last workgroup of a sequence to finish (arrival counter) reads the combined
// key and advances; with split == 1 no cross-workgroup traffic is needed.
// ---------------------------------------------------------------------------
template <int DT, int NC, bool FAST>
__global__ __launch_bounds__(kBlock) void step_sparse_kernel(DevTrie tr, DevState st, StepIO io, int split) {
  constexpr int EL = DT == 0 ? 4 : 8;
  const int g = blockIdx.x;
  const int s = g / split;
  const int w = g - s * split;
  const int lane = __lane_id();
  const int wv = w * kWavesPerBlock + wave_id();
  const int W = split * kWavesPerBlock;
  Seq q;
  if (!load_seq(tr, st, s, q)) {
    if (w == 0 && threadIdx.x == 0) write_step_out(io, s, -1, NAN);
    return;
  }
  const int32_t* live = st.live + (int64_t)s * tr.live_stride;
  // no logit asked for: a step the node record decides takes no head
  if (io.out_logit == nullptr) {
    const int fe = forced_edge(tr, live, q);
    if (fe != -3) {
      if (forced_last(st, s, split)) {
        if (threadIdx.x < kWave) advance(tr, st, &io, s, q, fe, NAN, lane);
      }
      return;
    }
  }
  const int nq = io.H / EL;
  uint4 hq[NC];
  load_hidden<NC>((const uint4*)io.hidden + (int64_t)s * nq, nq, hq, lane);
  Cand unused;
  const TrieView tv{tr.erec, tr.cent, tr.run, tr.run_edge, tr.run_tok, tr.run_land};
  const unsigned long long best = scan_node<DT, NC, FAST ? kMetaScalar : kMetaVector, kLiveScalar, false>(
      tr, tv, q, live, (const uint4*)io.emb, nq, hq, wv, W, lane, unused);

  __shared__ unsigned long long s_best[kWavesPerBlock];
  __shared__ unsigned long long s_key;
  __shared__ int s_last;
  if (lane == 0) s_best[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long b = s_best[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) b = max(b, s_best[i]);
    if (split == 1) {
      s_last = 1;
      s_key = b;
    } else {
      if (b) __hip_atomic_fetch_max(&st.key[s], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t prev = __hip_atomic_fetch_add(&st.arrive[s], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int last = prev == (uint32_t)(split - 1);
      s_last = last;
      if (last) s_key = __hip_atomic_load(&st.key[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!s_last || threadIdx.x >= kWave) return;
  const unsigned long long key = s_key;
  advance(tr, st, &io, s, q, key ? (int)key_id(key) : -2, key ? key_logit(key) : NAN, lane);
  if (lane == 0 && split > 1) {
    __hip_atomic_store(&st.key[s], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&st.arrive[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Row tile x and member tile y of root workgroup r of a launch with rt row
// tiles and mtiles member tiles.  Workgroups go to the eight XCDs in launch
// order, round robin, and each XCD has its own L2; numbering the member tiles
// of one row tile eight apart puts them on one XCD, whose L2 then fetches the
// tile's rows once instead of once per member tile.  The row tiles are padded
// to a multiple of 8 (false: a padding workgroup, which does nothing).
__device__ __forceinline__ bool root_tile(int r, int rt, int mtiles, int& x, int& y) {
  const int per = 8 * mtiles;
  const int q = r / per, rem = r - q * per;
  y = rem >> 3;
  x = q * 8 + (rem & 7);
  return x < rt;
}

// ---------------------------------------------------------------------------
// Node-grouped head below the root (sections "The batched engine" and "The
// sparse output layer": the rows a batch needs are the union of the legal
// sets, so a row legal for several sequences standing at the same node is
// read once for all of them).  The n_mem sequences at `node` (ranked by id)
// share the work of their split workgroups each: the node's edges in row
// tiles of one pass of the workgroup's rows (U per wavefront) times the
// members in tiles of mt, tile i taken by the group's workgroup i mod
// (n_mem * split).  A tile stages its members' hidden vectors in LDS, reads
// its rows once, and dots every (row, member) pair with the per-row
// arithmetic of the other kernels, so every logit, key and token is the one
// step_sparse_kernel computes; an edge's legality for the tile's members is
// one ballot (lane j: member j).  With one row tile the workgroup that takes a
// member tile holds its members' keys and advances them; with more, the keys
// meet in key[] with an atomic max and the last row tile of a member tile to
// arrive advances its members.
// ---------------------------------------------------------------------------
// rank: the rank of this workgroup's sequence among the members; mask0: with
// B <= 64, bit q set where sequence q is a member (the caller's ballot over
// the snapshot), so member lists need no second read of it.
template <int DT, int NC>
__device__ void node_group_step(const DevTrie& tr, const DevState& st, const StepIO& io, int node, int n_mem,
                                int rank, unsigned long long mask0, int split, int w,
                                const int32_t* snap_in, int32_t* snap_out, uint4* sh, int mt) {
  constexpr int EL = DT == 0 ? 4 : 8;
  constexpr int U = rows_per_pass(NC);
  constexpr int MPW = 4;  // members staged per wavefront per round
  constexpr int RT = U * kWavesPerBlock;  // rows per tile
  const int lane = __lane_id();
  const int wv = wave_id();
  const int nq = io.H / EL;
  const NodeRec rec = rec_scalar(tr.node_rec, node);
  const int f = rec.b1 - rec.b0;
  const int nrt = max(1, (f + RT - 1) / RT), nmt = (n_mem + mt - 1) / mt;
  const int n_wg = n_mem * split, me = rank * split + w;
  __shared__ int s_gm[kWave];
  __shared__ unsigned long long s_gbest[kWave];
  __shared__ int s_glast;
  // s_gm <- the ids of members r0 .. r0+cnt-1 (cnt <= 64), s_gbest <- 0
  // (wavefront 0; the caller's barrier publishes them)
  auto members = [&](int r0, int cnt) {
    if (wv != 0) return;
    s_gbest[lane] = 0ull;
    int rk = 0;
    for (int c = 0; c < st.B; c += kWave) {
      const int q = c + lane;
      const bool in = st.B <= kWave ? ((mask0 >> lane) & 1ull) != 0ull : q < st.B && snap_in[q] == node;
      const unsigned long long m = __ballot(in);
      const int r = rk + __popcll(m & ((1ull << lane) - 1ull)) - r0;
      if (in && r >= 0 && r < cnt) s_gm[r] = q;
      rk += __popcll(m);
    }
  };
  const uint4* hid = (const uint4*)io.hidden;
  for (int i = me; i < nrt * nmt; i += n_wg) {
    const int xr = i % nrt, m0 = (i / nrt) * mt;
    const int tc = min(mt, n_mem - m0);
    members(m0, tc);
    __syncthreads();
    const int mj = lane < tc ? s_gm[lane] : -1;
    // member j's control edges here: terminal, entry not spent, exactly-k rule
    Seq qj{node, 0, 0, rec.b0, rec.b1, false, false};
    if (mj >= 0) {
      qj.done = st.done[mj];
      bool ctl = false;
      if (rec.ent >= 0)
        ctl = ((st.spent[(int64_t)mj * st.spent_words + (rec.ent >> 5)] >> (rec.ent & 31)) & 1u) == 0u;
      const bool more = qj.done + 1 < st.k;
      qj.sep_ok = ctl && more;
      qj.stop_ok = ctl && !more;
    }
    const int32_t* mlive = st.live + (int64_t)(mj >= 0 ? mj : 0) * tr.live_stride;
    const int e0 = rec.b0 + xr * RT + wv;
    int rows[U];
    unsigned long long legal[U];  // bit j: legal for member j of the tile
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kWavesPerBlock;
      const bool in = e < rec.b1;
      const EdgeRec r = erec_uniform<kMetaScalar>(tr.erec, in ? e : rec.b0);
      const int lv = (in && mj >= 0) ? mlive[e] : 0;  // control edges hold 0
      legal[u] = __ballot(in && mj >= 0 && edge_ok_bits(r.child, lv, qj));
      rows[u] = legal[u] ? r.tok : -1;  // the union over the tile's members
    }
    uint4 raw[U][NC];
    issue_rows<NC, U>((const uint4*)io.emb, nq, rows, raw, lane);
    for (int jb = wv; jb < tc; jb += kWavesPerBlock * MPW) {
      uint4 v[MPW][NC];
#pragma unroll
      for (int u = 0; u < MPW; ++u) {
        const int j = jb + u * kWavesPerBlock;
        if (j < tc) load_hidden<NC>(hid + (int64_t)s_gm[j] * nq, nq, v[u], lane);
      }
#pragma unroll
      for (int u = 0; u < MPW; ++u) {
        const int j = jb + u * kWavesPerBlock;
        if (j >= tc) continue;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c * kWave + lane < nq) sh[j * nq + c * kWave + lane] = v[u][c];
      }
    }
    __syncthreads();  // staged vectors visible
    // two members per pass: independent accumulation chains side by side
    for (int j = 0; j < tc; j += 2) {
      const int j1 = min(j + 1, tc - 1);
      uint4 hq0[NC], hq1[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ii = c * kWave + lane < nq ? c * kWave + lane : 0;
        hq0[c] = c * kWave < nq ? sh[j * nq + ii] : make_uint4(0, 0, 0, 0);
        hq1[c] = c * kWave < nq ? sh[j1 * nq + ii] : make_uint4(0, 0, 0, 0);
      }
      float l0[U], l1[U];
      finish_rows<DT, NC, U>(nq, rows, raw, hq0, l0, lane);
      finish_rows<DT, NC, U>(nq, rows, raw, hq1, l1, lane);
      unsigned long long k0 = 0ull, k1 = 0ull;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = (uint32_t)(e0 + u * kWavesPerBlock);
        if ((legal[u] >> j) & 1ull) k0 = max(k0, pack_key(l0[u], e));
        if ((legal[u] >> j1) & 1ull) k1 = max(k1, pack_key(l1[u], e));
      }
      if (lane == 0) {
        if (k0) __hip_atomic_fetch_max(&s_gbest[j], k0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (k1 && j1 != j) __hip_atomic_fetch_max(&s_gbest[j1], k1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    rows_consumed();
    __syncthreads();  // the tile's keys are complete
    bool last = true;  // one row tile: this workgroup holds the members' final keys
    if (nrt > 1) {
      // the member tile's keys meet in key[]; the last of its nrt row tiles
      // to arrive (counted in the arrival slot of its first member) advances
      // its members.  The maxima are acknowledged (no-return atomics count in
      // vmcnt) before the arrival is issued.
      if (wv == 0 && lane < tc && s_gbest[lane])
        __hip_atomic_fetch_max(&st.key[mj], s_gbest[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (threadIdx.x == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t prev = __hip_atomic_fetch_add(&st.arrive[s_gm[0]], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_glast = prev == (uint32_t)(nrt - 1);
      }
      __syncthreads();
      last = s_glast;
    }
    if (last) {
      for (int j = wv; j < tc; j += kWavesPerBlock) {
        const int m = s_gm[j];
        const unsigned long long key =
            nrt > 1 ? __hip_atomic_load(&st.key[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : s_gbest[j];
        Seq q;
        if (!load_seq(tr, st, m, q)) {  // not expected: it stood at the node when the step began
          if (lane == 0) {
            write_step_out(io, m, -1, NAN);
            snap_out[m] = -1;
          }
        } else {
          const int next = advance(tr, st, &io, m, q, key ? (int)key_id(key) : -2, key ? key_logit(key) : NAN, lane);
          if (lane == 0) snap_out[m] = next;
        }
        if (nrt > 1 && lane == 0) __hip_atomic_store(&st.key[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (nrt > 1 && threadIdx.x == 0)
        __hip_atomic_store(&st.arrive[s_gm[0]], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // before the next tile rewrites s_gm, s_gbest and the staged vectors
  }
}

// NODES: sequences standing together at any other node are grouped as well
// (node_group_step); a sequence alone at its node takes its own step.
template <int DT, int NC, bool FAST, bool NODES = false>
__global__ __launch_bounds__(kBlock) void step_grouped_kernel(DevTrie tr, DevState st, StepIO io, int split,
                                                              int rt, int mt, int mtiles, int parity, int gmt) {
  constexpr int EL = DT == 0 ? 4 : 8;
  constexpr int U = rows_per_pass(NC);
  constexpr int MPW = 4;  // members staged per wavefront per round
  const int lane = __lane_id();
  const int wv = wave_id();
  const int nq = io.H / EL;
  const int nseq_wg = st.B * split;
  // who stands where at the start of the step: read from one half of snap,
  // which no workgroup writes during this launch (advances happen during it)
  const int32_t* snap_in = st.snap + (int64_t)parity * st.B;
  int32_t* snap_out = st.snap + (int64_t)(1 - parity) * st.B;
  __shared__ unsigned long long s_best[16];
  __shared__ unsigned long long s_key;
  __shared__ int s_last;
  __shared__ int s_cnt[kWavesPerBlock];
  if ((int)blockIdx.x < nseq_wg) {
    const int g = blockIdx.x;
    const int s = g / split;
    const int w = g - s * split;
    const int wq = w * kWavesPerBlock + wv;
    const int W = split * kWavesPerBlock;
    // the hidden vector first on the scalar-trie path (the edge records come
    // through the scalar cache and do not queue behind it), unless steps
    // without a head are possible: their advance would wait behind it
    uint4 hq[NC];
    const bool early = FAST && io.out_logit != nullptr;
    if (early) load_hidden<NC>((const uint4*)io.hidden + (int64_t)s * nq, nq, hq, lane);
    const int node0 = ((cint_p)snap_in)[s];
    Seq q;
    const bool active = load_seq(tr, st, s, q);  // issued with the snapshot read
    if (node0 == 0) return;  // a member: the root workgroups take its step
    if constexpr (NODES) {
      // the sequences at the same node take their steps together (the
      // workgroups of all of them share the work).  Decided from the snapshot
      // alone, before this sequence's own state: the group's last workgroup
      // may already be advancing it
      int n_mem = 0, rank = 0;
      unsigned long long mask0 = 0ull;
      for (int c = 0; node0 > 0 && c < st.B; c += kWave) {
        const int q2 = c + lane;
        const unsigned long long m = __ballot(q2 < st.B && snap_in[q2] == node0);
        if (c == 0) mask0 = m;
        if (c + kWave <= s) rank += __popcll(m);
        else if (c <= s) rank += __popcll(m & ((1ull << (s - c)) - 1ull));
        n_mem += __popcll(m);
      }
      if (n_mem > 1) {
        extern __shared__ uint4 sh_g[];
        node_group_step<DT, NC>(tr, st, io, node0, n_mem, rank, mask0, split, w, snap_in, snap_out, sh_g, gmt);
        return;
      }
    }
    if (node0 < 0 || !active) {
      if (w == 0 && threadIdx.x == 0) {
        write_step_out(io, s, -1, NAN);
        snap_out[s] = -1;
      }
      return;
    }
    const int32_t* live = st.live + (int64_t)s * tr.live_stride;
    // no logit asked for: a step the node record decides takes no head
    if (io.out_logit == nullptr) {
      const int fe = forced_edge(tr, live, q);
      if (fe != -3) {
        if (forced_last(st, s, split) && threadIdx.x < kWave) {
          const int next = advance(tr, st, &io, s, q, fe, NAN, lane);
          if (lane == 0) snap_out[s] = next;
        }
        return;
      }
    }
    if (!early) load_hidden<NC>((const uint4*)io.hidden + (int64_t)s * nq, nq, hq, lane);
    Cand unused;
    const TrieView tv{tr.erec, tr.cent, tr.run, tr.run_edge, tr.run_tok, tr.run_land};
    const unsigned long long best = scan_node<DT, NC, FAST ? kMetaScalar : kMetaVector, kLiveScalar, false>(
        tr, tv, q, live, (const uint4*)io.emb, nq, hq, wq, W, lane, unused);
    if (lane == 0) s_best[wv] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long b = s_best[0];
#pragma unroll
      for (int i = 1; i < kWavesPerBlock; ++i) b = max(b, s_best[i]);
      if (split == 1) {
        s_last = 1;
        s_key = b;
      } else {
        if (b) __hip_atomic_fetch_max(&st.key[s], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t prev = __hip_atomic_fetch_add(&st.arrive[s], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == (uint32_t)(split - 1);
        s_last = last;
        if (last) s_key = __hip_atomic_load(&st.key[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= kWave) return;
    const unsigned long long key = s_key;
    const int next = advance(tr, st, &io, s, q, key ? (int)key_id(key) : -2, key ? key_logit(key) : NAN, lane);
    if (lane == 0) {
      snap_out[s] = next;
      if (split > 1) {
        __hip_atomic_store(&st.key[s], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&st.arrive[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }
  // root workgroup (x, y); [mt][nq] members' hidden vectors in LDS, then their ids
  extern __shared__ uint4 sh[];
  int* s_mem = reinterpret_cast<int*>(sh + (size_t)mt * nq);
  int x, y;
  if (!root_tile((int)blockIdx.x - nseq_wg, rt, mtiles, x, y)) return;
  const int m0 = y * mt;
  if (threadIdx.x < 16) s_best[threadIdx.x] = 0ull;
  // this wavefront's root edges and their tokens, requested before the member
  // scan (they do not depend on it)
  const int r1 = tr.begin[1];
  const int e0 = tr.begin[0] + (x * kWavesPerBlock + wv) * U;
  int rows[U];
#pragma unroll
  for (int u = 0; u < U; ++u) rows[u] = e0 + u < r1 ? tr.tok[e0 + u] : -1;
  // members of this tile: ranks m0 .. m0+mt-1 among the sequences at the root
  int n_mem = 0;
  for (int s0 = 0; s0 < st.B; s0 += kBlock) {
    const int s = s0 + (int)threadIdx.x;
    const bool ok = s < st.B && snap_in[s] == 0;
    const unsigned long long m = __ballot(ok);
    if (lane == 0) s_cnt[wv] = __popcll(m);
    lds_barrier();
    int off = n_mem;
    for (int i = 0; i < wv; ++i) off += s_cnt[i];
    if (ok) {
      const int idx = off + __popcll(m & ((1ull << lane) - 1ull)) - m0;
      if (idx >= 0 && idx < mt) s_mem[idx] = s;
    }
    for (int i = 0; i < kWavesPerBlock; ++i) n_mem += s_cnt[i];
    lds_barrier();
  }
  const int cnt = min(mt, n_mem - m0);
  if (cnt <= 0) return;  // the same for the whole workgroup
  uint4 raw[U][NC];
  issue_rows<NC, U>((const uint4*)io.emb, nq, rows, raw, lane);
  // lane j reads member j's live counts of the wavefront's edges, requested
  // with the rows (used after the staging below)
  int lv[U];
  {
    const int32_t* my_live = lane < cnt ? st.live + (int64_t)s_mem[lane] * tr.live_stride : nullptr;
#pragma unroll
    for (int u = 0; u < U; ++u) lv[u] = rows[u] >= 0 && lane < cnt ? my_live[e0 + u] : 0;
  }
  // stage the members' vectors: every load of a round before its stores
  const uint4* hid = (const uint4*)io.hidden;
  for (int jb = wv; jb < cnt; jb += kWavesPerBlock * MPW) {
    uint4 v[MPW][NC];
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int j = jb + u * kWavesPerBlock;
      if (j < cnt) load_hidden<NC>(hid + (int64_t)s_mem[j] * nq, nq, v[u], lane);
    }
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int j = jb + u * kWavesPerBlock;
      if (j >= cnt) continue;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c * kWave + lane < nq) sh[j * nq + c * kWave + lane] = v[u][c];
    }
  }
  unsigned long long legal[U];
#pragma unroll
  for (int u = 0; u < U; ++u) legal[u] = __ballot(lv[u] > 0);
  lds_barrier();  // staged vectors visible
  // two members per pass: independent accumulation chains side by side
  for (int j = 0; j < cnt; j += 2) {
    const int j1 = min(j + 1, cnt - 1);
    uint4 hq0[NC], hq1[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = c * kWave + lane;
      const int ii = i < nq ? i : 0;
      hq0[c] = c * kWave < nq ? sh[j * nq + ii] : make_uint4(0, 0, 0, 0);
      hq1[c] = c * kWave < nq ? sh[j1 * nq + ii] : make_uint4(0, 0, 0, 0);
    }
    float l0[U], l1[U];
    finish_rows<DT, NC, U>(nq, rows, raw, hq0, l0, lane);
    finish_rows<DT, NC, U>(nq, rows, raw, hq1, l1, lane);
    unsigned long long b0 = 0ull, b1 = 0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((legal[u] >> j) & 1ull) b0 = max(b0, pack_key(l0[u], (uint32_t)(e0 + u)));
      if ((legal[u] >> j1) & 1ull) b1 = max(b1, pack_key(l1[u], (uint32_t)(e0 + u)));
    }
    if (lane == 0) {
      if (b0) __hip_atomic_fetch_max(&s_best[j], b0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (b1 && j1 != j) __hip_atomic_fetch_max(&s_best[j1], b1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  lds_barrier();
  if (wv != 0) return;
  // combine this tile's best keys into the members' slots; the last of the rt
  // root workgroups to arrive for a member advances it.  Everything they
  // exchange goes through device-scope atomics (the key max and the arrival
  // count), which are performed where they are coherent for the whole device:
  // waiting for the max to complete before the arrival is issued orders the
  // two, so the last arrival finds every tile's max in key[s].  A device-scope release and acquire would instead write back and
  // invalidate this XCD's L2 in each of the rt x mtiles root workgroups.
  bool last = false;
  int sm = 0;
  if (lane < cnt) {
    sm = s_mem[lane];
    const unsigned long long b = s_best[lane];
    if (b) __hip_atomic_fetch_max(&st.key[sm], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the max is acknowledged (vector memory counter drained) before the
  // arrival is issued; no-return atomics count in vmcnt on this part
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane < cnt) {
    const uint32_t prev = __hip_atomic_fetch_add(&st.arrive[sm], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (uint32_t)(rt - 1);
  }
  if (!last) return;
  // The advance of a member, one lane each (what advance() does for a
  // sequence at the root: the root has content edges only, so a legal winner
  // pushes its edge as the path's first and moves to the child; nothing is
  // released).  Empty mask: EMPTY_MASK; a winner that is not a live root edge:
  // NOT_WALKABLE.
  const unsigned long long key = __hip_atomic_load(&st.key[sm], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int status = kSeqOk, tok = -1, next = -1;
  if (!key) {
    status = kSeqEmptyMask;
  } else {
    const int e = (int)key_id(key);
    const int c = e >= tr.begin[0] && e < r1 ? tr.child[e] : -3;
    if (c < 0 || st.live[(int64_t)sm * tr.live_stride + e] <= 0) {
      status = kSeqNotWalkable;
    } else {
      next = c;
      tok = tr.tok[e];
      st.path[(int64_t)sm * st.path_stride] = e;
      st.depth[sm] = 1;
      st.node[sm] = c;
      st.nemit[sm] = st.nemit[sm] + 1;
    }
  }
  if (status != kSeqOk) st.status[sm] = status;
  snap_out[sm] = next;
  write_step_out(io, sm, tok, key ? key_logit(key) : NAN);
  __hip_atomic_store(&st.key[sm], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&st.arrive[sm], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The edges of a node of at most 64 edges, one lane per edge (lane i: edge
// b0+i; lanes past the range hold a record that matches no edge kind), and
// the ballot of the legal ones.  Every wavefront of the resident loop loads
// the same copy, so all of them take the same decisions from it without a
// barrier.
struct NodeLanes {
  EdgeRec r;
  int lv, ce, rn;
  unsigned long long m;  // bit i: edge b0+i is legal
};

template <bool MASK>
__device__ __forceinline__ NodeLanes node_lanes(const TrieView& tv, const int32_t* live, const Seq& q, int lane,
                                                const Ban& ban) {
  const int f = q.b1 - q.b0;
  const int e = q.b0 + lane;
  NodeLanes n{EdgeRec{kChildSep - 8, 0, 0, 0}, 0, -1, 0, 0ull};
  if (lane < f) {
    n.r = tv.erec[e];
    // read for every edge (in range of the live array), used for content edges
    if constexpr (MASK) n.lv = mask_live(reinterpret_cast<const uint4*>(live)[e], ban) ? 1 : 0;
    else n.lv = live[e];
    n.ce = tv.cent[e];
    n.rn = tv.run[e];
  }
  n.m = __ballot(edge_ok_bits(n.r.child, n.lv, q));
  return n;
}

__device__ __forceinline__ Cand lane_cand(const NodeLanes& n, int w) {
  return Cand{__builtin_amdgcn_readlane(n.r.child, w), __builtin_amdgcn_readlane(n.r.tok, w),
              __builtin_amdgcn_readlane(n.r.b0, w),    __builtin_amdgcn_readlane(n.r.b1, w),
              __builtin_amdgcn_readlane(n.ce, w),      __builtin_amdgcn_readlane(n.rn, w)};
}

// Head scan of a node held as NodeLanes (sections "The sparse output layer"
// and "The batched engine": logits of the legal edges only): wavefront wv
// takes lanes wv, wv+W, ..., U per pass, and requests their rows straight
// from the lanes' records, with no second read of records or live counts.
// Same keys as scan_node, so the winner does not depend on which scan ran.
template <int DT, int NC, bool CAND>
__device__ __forceinline__ unsigned long long scan_lanes(const Seq& q, const NodeLanes& n,
                                                         const uint4* __restrict__ emb, int nq,
                                                         const uint4 (&hq)[NC], int wv, int W, int lane,
                                                         Cand& cand) {
  constexpr int U = rows_per_pass(NC);
  const int f = q.b1 - q.b0;
  unsigned long long best = 0;
  for (int j0 = wv; j0 < f; j0 += U * W) {
    int rows[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * W;
      const bool ok = j < f && ((n.m >> (j & 63)) & 1ull);
      rows[u] = ok ? __builtin_amdgcn_readlane(n.r.tok, j & 63) : -1;
    }
    uint4 raw[U][NC];
    issue_rows<NC, U>(emb, nq, rows, raw, lane);
    float l[U];
    finish_rows<DT, NC, U>(nq, rows, raw, hq, l, lane);
    rows_consumed();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (rows[u] < 0) continue;
      const int j = j0 + u * W;
      const uint32_t e = (uint32_t)(q.b0 + j);
      const unsigned long long k = CAND ? pack_key_wave(l[u], e, wv) : pack_key(l[u], e);
      if (k > best) {
        best = k;
        if constexpr (CAND) cand = lane_cand(n, j);
      }
    }
  }
  return best;
}

// ---------------------------------------------------------------------------
// Resident device loop (section "The whole loop on the device"): one
// workgroup per sequence runs every step of the answer without returning to
// the host or launching again; token, node, path and no-repeat state stay on
// the device.  Each step is the same scan, arithmetic and tie rule as the
// step kernel, so the two forms give bit-identical results.  Only this
// workgroup touches its sequence's state, so steps need no cross-workgroup
// synchronisation, only workgroup barriers.  FAST: the sequence's live counts
// and spent flags are copied into LDS for the duration of the loop; GLOBAL:
// they stay in device memory.
// ---------------------------------------------------------------------------
constexpr int kLoopBlock = 512;

// A 64-bit uniform value parked in lanes 2I and 2I+1 of a vector register
// while the resident loop runs, and read back after it: values used only
// before and after the loop then leave the scalar registers to the loop's
// own state (which otherwise gets spilled inside the loop).
template <int I>
__device__ __forceinline__ void park64(int& reg, const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  asm volatile("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(reg) : "s"(lo), "n"(2 * I));
  asm volatile("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(reg) : "s"(hi), "n"(2 * I + 1));
}
template <typename T, int I>
__device__ __forceinline__ T* unpark64(int reg) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(reg, 2 * I);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(reg, 2 * I + 1);
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
constexpr int kLoopWaves = kLoopBlock / kWave;

// LDS layout of the resident loop (in int32 words, each part a multiple of 4):
// live counts, spent bits and, with the trie in LDS, edge records, the
// entries of the edges' children and the forced-run tables.
struct LoopLds {
  int live, spent, erec, cent, run, run_edge, run_tok, land, emask, total;
};
__host__ __device__ inline int round4(int n) { return (n + 3) & ~3; }
__host__ __device__ inline LoopLds loop_lds_layout(const DevTrie& tr, const DevState& st, bool trie) {
  LoopLds o;
  o.live = 0;
  o.spent = o.live + tr.live_stride;
  o.erec = o.spent + round4(st.spent_words);
  o.cent = o.erec + (trie ? 4 * tr.n_edges : 0);
  o.run = o.cent + (trie ? tr.live_stride : 0);
  o.run_edge = o.run + (trie ? tr.live_stride : 0);
  o.run_tok = o.run_edge + (trie ? round4(tr.n_run) : 0);
  o.land = o.run_tok + (trie ? round4(tr.n_run) : 0);
  o.emask = o.land + (trie ? 4 * tr.n_run : 0);
  o.total = o.emask + (trie && tr.emask ? 4 * tr.n_edges : 0);
  return o;
}

// Reset of sequence s by its completed entries (kResetPaths): each completion
// took one live count off every edge of the entry's root path and set the
// entry's spent bit, so giving those edges their live0 counts back and
// clearing those spent words restores the initial state.  An edge on several
// paths gets the same value from each writer.  Wavefront wv of nw.  The
// caller orders these stores before anything reads the counts or clears the
// stored entries.
__device__ __forceinline__ void restore_paths(const DevTrie& tr, const DevState& st, int s, int32_t* g_live,
                                              uint32_t* g_spent, int wv, int nw, int lane) {
  const int32_t* ent = st.entries + (int64_t)s * st.k;
  const int od = min(max(st.done[s], 0), st.k);
  for (int j = wv; j < od; j += nw) {
    const int x = __builtin_amdgcn_readfirstlane(ent[j]);
    if (x < 0 || x >= tr.n_entries) continue;
    const int p1 = tr.ent_off[x + 1];
    for (int p = tr.ent_off[x] + lane; p < p1; p += kWave) {
      const int e = tr.ent_path[p];
      g_live[e] = tr.live0[e];
    }
    if (lane == 0) g_spent[x >> 5] = 0u;
  }
}

// Two blocks of n0 and n1 int32 words from device memory into LDS as
// 16-byte moves through registers, every load of a round issued before its
// stores.
__device__ __forceinline__ void copy2_regs(int32_t* d0, const int32_t* s0, int n0, int32_t* d1,
                                           const int32_t* s1, int n1) {
  const int a = (n0 + 3) >> 2, b = (n1 + 3) >> 2;
  const int4* S0 = reinterpret_cast<const int4*>(s0);
  const int4* S1 = reinterpret_cast<const int4*>(s1);
  int4* D0 = reinterpret_cast<int4*>(d0);
  int4* D1 = reinterpret_cast<int4*>(d1);
  for (int base = 0; base < max(a, b); base += 2 * kLoopBlock) {
    const int i0 = base + (int)threadIdx.x, i1 = i0 + kLoopBlock;
    int4 v0, v1, v2, v3;
    if (i0 < a) v0 = S0[i0];
    if (i1 < a) v1 = S0[i1];
    if (i0 < b) v2 = S1[i0];
    if (i1 < b) v3 = S1[i1];
    if (i0 < a) D0[i0] = v0;
    if (i1 < a) D0[i1] = v1;
    if (i0 < b) D1[i0] = v2;
    if (i1 < b) D1[i1] = v3;
  }
}

// n int32 words from device memory into LDS with direct loads: each
// wavefront moves 1 KB per instruction, lane l's 16 bytes landing at byte
// 16 l of the chunk, with no register round trip and no LDS store
// instruction (the caller waits for the loads).
__device__ __forceinline__ void lds_chunks(int32_t* d, const int32_t* s, int n, int wv, int lane) {
  const int q = (n + 3) >> 2;  // 16-byte units
  const int4* S = reinterpret_cast<const int4*>(s);
  for (int c = wv * kWave; c < q; c += kLoopWaves * kWave) {
    if (c + lane < q)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(S + c + lane),
                                       (__attribute__((address_space(3))) void*)(d + 4 * c), 16, 0, 0);
  }
}
// Two blocks of n0 and n1 int32 words from device memory into LDS (the
// device buffers are padded to 256 bytes and the LDS parts to 4 words).  A
// large image goes with direct loads (lds_chunks); a small one (the product
// catalog's 8 KB) through registers, measured the faster of the two there.
// The caller's barrier follows.
__device__ __forceinline__ void copy2_to_lds(int32_t* d0, const int32_t* s0, int n0, int32_t* d1,
                                             const int32_t* s1, int n1) {
  if (n0 + n1 >= 4096) {  // 16 KB
    const int wv = wave_id(), lane = __lane_id();
    lds_chunks(d0, s0, n0, wv, lane);
    lds_chunks(d1, s1, n1, wv, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    copy2_regs(d0, s0, n0, d1, s1, n1);
  }
}

// Every wavefront of the loop holds the same copy of the sequence's state
// (node, depth, pointers done, the node's record and control-edge flags) and
// takes every decision itself from the same inputs, so the steps need
// barriers only where LDS is written: once per step that reads the head
// (winning keys and payloads go through LDS) and around the release of a
// completed pointer's live counts.  Wavefront 0 alone keeps the path and the
// completed entries and stores the emitted tokens.
//   Keys rotate over three LDS slots and payloads over two, indexed by the
// number of head steps so far: the slot a step fills was last read two head
// steps earlier, before the barrier of the previous head step, and is cleared
// by wavefront 0 before that of the current one.
// SMALL: path, completed entries and spent flags are known to fit the
// register-held lists (depth, k and spent words at most 64); the general
// instantiations decide at run time.
// MASK: the bitmask no-repeat state replaces the live counts inside the loop
// (legality from the edges' entry masks and the banned set; no counts to
// copy in or release); the counts are rewritten from the masks at the end.
template <int DT, int NC, int META, bool LDS_LIVE, bool SMALL, bool MASK>
__global__ __launch_bounds__(kLoopBlock) void loop_kernel(DevTrie tr, DevState st, LoopIO io) {
  constexpr int EL = DT == 0 ? 4 : 8;
  constexpr bool TRIE_LDS = META == kMetaLds;
  static_assert(!MASK || (TRIE_LDS && SMALL), "the bitmask state comes with the LDS trie and register lists");
  constexpr int LIVE_KIND = MASK ? kLiveMask : (LDS_LIVE ? kLiveLds : kLiveVector);
  // With the trie in LDS the winner's record is read again from LDS after the
  // barrier; otherwise each wavefront's best candidate carries it (PAYLOAD).
  constexpr bool PAYLOAD = !TRIE_LDS;
  static_assert(!TRIE_LDS || LDS_LIVE, "the LDS trie comes with LDS live counts");
  extern __shared__ __attribute__((aligned(16))) int32_t lds[];
  __shared__ unsigned long long s_key[3];
  __shared__ Cand s_cand[2][kLoopWaves];
  __shared__ NodeRec s_root;
  const int s = blockIdx.x;
  const int lane = __lane_id();
  const int wv = wave_id();
  const int W = kLoopWaves;
  const int nq = io.H / EL;
  const int64_t ls = tr.live_stride;
  const LoopLds lay = loop_lds_layout(tr, st, TRIE_LDS);
  int32_t* g_live = st.live + (int64_t)s * ls;
  uint32_t* g_spent = st.spent + (int64_t)s * st.spent_words;
  int32_t* live = LDS_LIVE ? lds + lay.live : g_live;
  uint32_t* spent = LDS_LIVE ? reinterpret_cast<uint32_t*>(lds + lay.spent) : g_spent;
  // spent flags of up to 2048 entries live in a register of every wavefront
  // (lane l: word l); beyond that in LDS or device memory
  const bool sreg_ok = SMALL || st.spent_words <= kWave;
  // io.reset: start from the reset state (full live counts, nothing spent,
  // no entries, root) instead of the stored one
  const bool rst = io.reset != 0;
  const bool later = (io.flags & kLoopLater) != 0;
  const bool exit_root = (io.flags & kLoopExitAtRoot) != 0;
  const bool root_key = (io.flags & kLoopRootKey) != 0;
  __shared__ unsigned long long s_pre_key;
  uint32_t sreg = 0u;
  if (sreg_ok && lane < st.spent_words && !rst) sreg = g_spent[lane];
  TrieView tv{tr.erec, tr.cent, tr.run, tr.run_edge, tr.run_tok, tr.run_land};
  if constexpr (LDS_LIVE) {
    // live counts, and the trie image when it is kept in LDS
    copy2_to_lds(lds + lay.live, rst ? tr.live0 : g_live, MASK ? 0 : (int)ls, lds + lay.erec,
                 reinterpret_cast<const int32_t*>(tr.erec), TRIE_LDS ? tr.image_words : 0);
    if (!sreg_ok)
      for (int i = threadIdx.x; i < st.spent_words; i += kLoopBlock) spent[i] = rst ? 0u : g_spent[i];
  } else if (io.reset == kResetPaths) {
    restore_paths(tr, st, s, g_live, g_spent, wv, W, lane);
    __syncthreads();  // the stored entries are read before they are cleared below
  } else if (rst) {
    if (io.reset == kResetFull)
      for (int i = threadIdx.x; i < (int)(ls / 4); i += kLoopBlock)
        reinterpret_cast<int4*>(g_live)[i] = reinterpret_cast<const int4*>(tr.live0)[i];
    if (!sreg_ok)
      for (int i = threadIdx.x; i < st.spent_words; i += kLoopBlock) g_spent[i] = 0u;
  }
  if constexpr (TRIE_LDS) {
    tv = TrieView{reinterpret_cast<const EdgeRec*>(lds + lay.erec), lds + lay.cent, lds + lay.run,
                  lds + lay.run_edge, lds + lay.run_tok, reinterpret_cast<const int4*>(lds + lay.land)};
  }
  int node = 0, depth = 0, done = 0, status = kSeqOk, fin = 0, nemit = 0;
  if (!rst) {
    node = st.node[s];
    depth = st.depth[s];
    done = st.done[s];
    status = st.status[s];
    fin = st.finished[s];
    nemit = st.nemit[s];
  }
  int32_t* path = st.path + (int64_t)s * st.path_stride;
  int32_t* entries = st.entries + (int64_t)s * st.k;
  if (rst) {
    for (int j = threadIdx.x; j < st.k; j += kLoopBlock) entries[j] = -1;
    if (threadIdx.x == 0) {
      st.key[s] = 0ull;
      st.arrive[s] = 0u;
    }
  }
  int32_t* tokens = io.tokens_bt + (int64_t)s * io.T;
  int t = later ? st.tstep[s] : 0;
  // Wavefront 0 keeps the current path (lane d: edge at depth d) and the
  // completed entries (lane j: entry j) in registers; they reach device
  // memory at the end.  Tokens are stored as they are emitted (stores are not
  // waited for by the LDS barriers).
  const bool reg_lists = SMALL || (st.path_stride <= kWave && st.k <= kWave);
  int my_path = -1, my_ent = -1;
  if (wv == 0 && reg_lists) {
    if (lane < depth) my_path = path[lane];
    if (lane < done) my_ent = entries[lane];
  }
  NodeRec rec = rec_scalar(tr.node_rec, node);
  if (threadIdx.x == 0) {
    s_root = rec_scalar(tr.node_rec, 0);
    s_key[0] = s_key[1] = s_key[2] = 0ull;
  }
  if (root_key && wv == 0) {
    // this sequence's root step from the grouped head: max over its row tiles
    unsigned long long m = 0ull;
    for (int i = lane; i < io.root_tiles; i += kWave) m = max(m, st.rkey[(int64_t)i * st.B + s]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)m, d);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(m >> 32), d);
      m = max(m, ((unsigned long long)hi << 32) | lo);
    }
    if (lane == 0) s_pre_key = m;
  }
  __syncthreads();  // also orders the reset's stores before their first reads
  int parked = 0;
  park64<0>(parked, path);
  park64<1>(parked, entries);
  park64<2>(parked, g_spent);
  park64<3>(parked, g_live);
  park64<4>(parked, st.tstep + s);
  park64<5>(parked, st.node + s);
  park64<6>(parked, st.depth + s);
  park64<7>(parked, st.done + s);
  park64<8>(parked, st.status + s);
  park64<9>(parked, st.finished + s);
  park64<10>(parked, st.nemit + s);
  park64<11>(parked, io.len ? io.len + s : nullptr);
  park64<12>(parked, io.entries ? io.entries + (int64_t)s * st.k : nullptr);
  auto is_spent = [&](int ent) -> bool {
    const uint32_t w = sreg_ok ? (uint32_t)__builtin_amdgcn_readlane((int)sreg, ent >> 5)
                               : (uint32_t)__builtin_amdgcn_readfirstlane(spent[ent >> 5]);
    return ((w >> (ent & 31)) & 1u) != 0u;
  };
  // the banned set of the bitmask state: spent words 0..3 (uniform)
  Ban ban{0u, 0u, 0u, 0u};
  if constexpr (MASK)
    ban = Ban{(uint32_t)__builtin_amdgcn_readlane((int)sreg, 0), (uint32_t)__builtin_amdgcn_readlane((int)sreg, 1),
              (uint32_t)__builtin_amdgcn_readlane((int)sreg, 2), (uint32_t)__builtin_amdgcn_readlane((int)sreg, 3)};
  const int32_t* lsrc = MASK ? lds + lay.emask : live;  // what scans read for liveness
  bool ctl0 = rec.ent >= 0 && !is_spent(rec.ent);
  bool sep_ok = ctl0 && done + 1 < st.k, stop_ok = ctl0 && done + 1 >= st.k;
  const uint4* hid = (const uint4*)io.hidden_seq;
  const uint4* emb = (const uint4*)io.emb;
  const int t_enter = t;
  int nhead = 0;  // steps so far that read the head
  // Step t emits control edge `kind` (token tok) at the current terminal:
  // wavefront 0 releases the path's live counts, records the entry and
  // spends the terminal; the barrier after it publishes the new counts.
  // sync_first: some wavefront may still be reading live counts of this
  // answer (no barrier since its last read), so wait for all of them first.
  auto complete = [&](int kind, int tok, bool sync_first) {
    if (sync_first) {
      if constexpr (LDS_LIVE) lds_barrier();
      else __syncthreads();
    }
    const int ent = rec.ent;
    if constexpr (MASK) {
      const uint32_t bit = 1u << (ent & 31);
      const int w = ent >> 5;
      ban.w0 |= w == 0 ? bit : 0u;
      ban.w1 |= w == 1 ? bit : 0u;
      ban.w2 |= w == 2 ? bit : 0u;
      ban.w3 |= w == 3 ? bit : 0u;
    }
    if (wv == 0) {
      if (lane == 0) tokens[t] = tok;
      if (reg_lists) {
        if (!MASK && lane < depth && tr.release) atomicSub(&live[my_path], 1);  // distinct edges; no value returned
        if (lane == done) my_ent = ent;
      } else {
        if (tr.release)
          for (int i = lane; i < depth; i += kWave) atomicSub(&live[path[i]], 1);
        if (lane == 0) entries[done] = ent;
      }
      if (!sreg_ok && lane == 0) spent[ent >> 5] |= 1u << (ent & 31);
      // live counts in device memory are read again by this kernel unless the
      // sequence stops here or the phase ends at the root; spent flags and
      // entries in device memory are read back in any case
      const bool reread = kind != kChildStop && !exit_root;
      if ((!LDS_LIVE && reread) || !reg_lists || !sreg_ok) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (sreg_ok && lane == (ent >> 5)) sreg |= 1u << (ent & 31);
    if constexpr (LDS_LIVE) lds_barrier();
    else __syncthreads();
    done += 1;
    depth = 0;
    nemit += 1;
    if (kind == kChildStop) {
      fin = 1;
    } else {
      node = 0;
      rec = s_root;
    }
  };
  // Step t takes edge e with payload c (every wavefront).  After a content
  // edge, the forced run that follows it (single-edge nodes) is emitted at
  // once, and a leaf terminal reached with its entry unspent completes in
  // the next step (its only legal edge is sep or stop); each of these counts
  // as steps and stops at the step budget.
  auto take = [&](int e, const Cand& c, bool sync_release) {
    if (c.child < 0) {
      complete(c.child, c.tok, sync_release);
    } else {
      if (wv == 0) {
        if (lane == 0) tokens[t] = c.tok;
        if (reg_lists) {
          if (lane == depth) my_path = e;
        } else {
          if (lane == 0) path[depth] = e;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // read back by this wavefront
        }
      }
      depth += 1;
      node = c.child;
      rec = NodeRec{c.b0, c.b1, c.ent, 0};
      nemit += 1;
      int ri = c.run;
      while ((ri & 127) != 0 && t + 1 < io.T) {
        const int rl = ri & 127;
        const int ra = (int)((uint32_t)ri >> 7);
        const int L = min(rl, io.T - 1 - t);
        if (wv == 0) {
          if (lane < L) tokens[t + 1 + lane] = tv.run_tok[ra + lane];
          if (reg_lists) {
            const int i = lane - depth;
            if (i >= 0 && i < L) my_path = tv.run_edge[ra + i];
          } else {
            if (lane < L) path[depth + lane] = tv.run_edge[ra + lane];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // read back by this wavefront
          }
        }
        if (L == rl && rl < 64) {
          // the whole run, and it ends the chain (a run of 64 may continue):
          // land on the child of its last edge in one read
          const int4 d = tv.run_land[ra + rl - 1];
          node = __builtin_amdgcn_readfirstlane(d.x);
          rec = NodeRec{__builtin_amdgcn_readfirstlane(d.y), __builtin_amdgcn_readfirstlane(d.z),
                        __builtin_amdgcn_readfirstlane(d.w), 0};
          ri = 0;
        } else {
          const int el = __builtin_amdgcn_readfirstlane(tv.run_edge[ra + L - 1]);
          const EdgeRec r = tv.erec[el];
          const int ce = __builtin_amdgcn_readfirstlane(tv.cent[el]);
          const int rn = __builtin_amdgcn_readfirstlane(tv.run[el]);
          node = __builtin_amdgcn_readfirstlane(r.child);
          rec = NodeRec{__builtin_amdgcn_readfirstlane(r.b0), __builtin_amdgcn_readfirstlane(r.b1), ce, 0};
          ri = L == rl ? rn : 0;
        }
        depth += L;
        t += L;
        nemit += L;
      }
      if (rec.ent >= 0 && rec.b1 - rec.b0 == 2 && t + 1 < io.T && !is_spent(rec.ent)) {
        t += 1;
        const bool more = done + 1 < st.k;
        complete(more ? kChildSep : kChildStop, more ? tr.sep : tr.stop, sync_release);
      }
    }
    // control edges of the node reached: terminal, not yet spent, exactly-k rule
    const bool ctl = rec.ent >= 0 && !fin && !is_spent(rec.ent);
    sep_ok = ctl && done + 1 < st.k;
    stop_ok = ctl && done + 1 >= st.k;
  };
  if (root_key) {
    const unsigned long long pre_key = s_pre_key;
    if (status == kSeqOk && !fin && node == 0 && depth == 0 && t < io.T) {
      // the root step from the grouped head (same arithmetic and tie rule)
      const uint32_t klo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pre_key);
      const uint32_t khi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(pre_key >> 32));
      if ((klo | khi) == 0u) {
        status = kSeqEmptyMask;
        if (wv == 0 && lane == 0) tokens[t] = -1;
      } else {
        const int e = (int)key_id(((unsigned long long)khi << 32) | klo);
        const EdgeRec r = tv.erec[e];
        const Cand c{__builtin_amdgcn_readfirstlane(r.child), __builtin_amdgcn_readfirstlane(r.tok),
                     __builtin_amdgcn_readfirstlane(r.b0),    __builtin_amdgcn_readfirstlane(r.b1),
                     __builtin_amdgcn_readfirstlane(tv.cent[e]), __builtin_amdgcn_readfirstlane(tv.run[e])};
        take(e, c, false);
      }
      t += 1;
    }
  }
  for (; t < io.T && status == kSeqOk && !fin; ++t) {
    // a phase before the last ends where the sequence is back at the root:
    // the next phase's grouped head takes that step
    if (exit_root && node == 0 && depth == 0 && t > t_enter) break;
    Seq q;
    q.node = node;
    q.depth = depth;
    q.done = done;
    q.b0 = rec.b0;
    q.b1 = rec.b1;
    q.sep_ok = sep_ok;
    q.stop_ok = stop_ok;
    // A node of at most 64 edges is loaded once, one lane per edge: with a
    // single legal edge the step is forced (sections "Masked sampling inside
    // the sampler" and "The sparse output layer": the argmax over one legal
    // token is that token whatever the logits) and takes no rows, no
    // reduction and no barrier unless a pointer completes (forced steps have
    // no barrier of their own, so a release first waits for every
    // wavefront); otherwise the head scan starts from the same lanes.
    const bool narrow = q.b1 - q.b0 <= kWave;
    NodeLanes nl{};
    if (narrow) {
      nl = node_lanes<MASK>(tv, lsrc, q, lane, ban);
      if (__popcll(nl.m) == 1) {
        const int w = (int)__builtin_ctzll(nl.m);
        take(q.b0 + w, lane_cand(nl, w), true);
        continue;
      }
    }
    // this step's hidden vector, requested before the edge records and rows:
    // it arrives alongside them (a copy carried from earlier steps would have
    // to be moved and waited for on every forced step)
    uint4 hq[NC];
    load_hidden<NC>(hid + ((int64_t)t * st.B + s) * nq, nq, hq, lane);
    const int slot = nhead % 3;
    if (threadIdx.x == 0) s_key[(nhead + 1) % 3] = 0ull;  // the next head step's slot
    Cand cand{0, 0, 0, 0, 0, 0};
    const unsigned long long best =
        narrow ? scan_lanes<DT, NC, PAYLOAD>(q, nl, emb, nq, hq, wv, W, lane, cand)
               : scan_node<DT, NC, META, LIVE_KIND, PAYLOAD>(tr, tv, q, lsrc, emb, nq, hq, wv, W, lane, cand, ban);
    if (lane == 0) {
      if (best) __hip_atomic_fetch_max(&s_key[slot], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if constexpr (PAYLOAD) s_cand[nhead & 1][wv] = cand;
    }
    lds_barrier();
    const unsigned long long key = s_key[slot];
    const uint32_t klo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)key);
    const uint32_t khi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(key >> 32));
    nhead += 1;
    if ((klo | khi) == 0u) {
      status = kSeqEmptyMask;
      if (wv == 0 && lane == 0) tokens[t] = -1;
    } else if constexpr (PAYLOAD) {
      const Cand w = s_cand[(nhead - 1) & 1][klo & 7u];
      const Cand c{__builtin_amdgcn_readfirstlane(w.child), __builtin_amdgcn_readfirstlane(w.tok),
                   __builtin_amdgcn_readfirstlane(w.b0),    __builtin_amdgcn_readfirstlane(w.b1),
                   __builtin_amdgcn_readfirstlane(w.ent),   __builtin_amdgcn_readfirstlane(w.run)};
      take((int)key_wave_edge(((unsigned long long)khi << 32) | klo), c, false);
    } else {
      const int e = (int)key_id(((unsigned long long)khi << 32) | klo);  // plain keys carry the edge
      const EdgeRec r = tv.erec[e];
      const Cand c{__builtin_amdgcn_readfirstlane(r.child), __builtin_amdgcn_readfirstlane(r.tok),
                   __builtin_amdgcn_readfirstlane(r.b0),    __builtin_amdgcn_readfirstlane(r.b1),
                   __builtin_amdgcn_readfirstlane(tv.cent[e]), __builtin_amdgcn_readfirstlane(tv.run[e])};
      take(e, c, false);
    }
  }
  {
    int32_t* const p_path = unpark64<int32_t, 0>(parked);
    int32_t* const p_entries = unpark64<int32_t, 1>(parked);
    uint32_t* const p_spent = unpark64<uint32_t, 2>(parked);
    if (wv == 0) {
      if (reg_lists) {
        if (lane < depth) p_path[lane] = my_path;
        if (lane < done) p_entries[lane] = my_ent;
      }
      if (sreg_ok && lane < st.spent_words) p_spent[lane] = sreg;
    }
    if (!exit_root) {
      for (int i = t + threadIdx.x; i < io.T; i += kLoopBlock) tokens[i] = -1;
      if (status == kSeqOk && !fin) status = kSeqNotDone;
    }
    if (threadIdx.x == 0) {
      *unpark64<int32_t, 4>(parked) = t;
      *unpark64<int32_t, 5>(parked) = node;
      *unpark64<int32_t, 6>(parked) = depth;
      *unpark64<int32_t, 7>(parked) = done;
      *unpark64<int32_t, 8>(parked) = status;
      *unpark64<int32_t, 9>(parked) = fin;
      *unpark64<int32_t, 10>(parked) = nemit;
      int32_t* const p_len = unpark64<int32_t, 11>(parked);
      if (p_len) *p_len = nemit;
    }
    int32_t* const p_out = unpark64<int32_t, 12>(parked);
    if (wv == 0 && p_out) {
      for (int j = lane; j < st.k; j += kWave)
        p_out[j] = (reg_lists && j < kWave) ? (j < done ? my_ent : p_entries[j]) : p_entries[j];
    }
  }
  int32_t* const g_live_out = unpark64<int32_t, 3>(parked);
  if constexpr (MASK) {
    // live counts from the masks: entries below each edge not yet spent
    const uint4* em = reinterpret_cast<const uint4*>(lds + lay.emask);
    for (int e = threadIdx.x; e < (int)ls; e += kLoopBlock) {
      int c = 0;
      if (e < tr.n_edges) {
        const uint4 m = em[e];
        c = __popc(m.x & ~ban.w0) + __popc(m.y & ~ban.w1) + __popc(m.z & ~ban.w2) + __popc(m.w & ~ban.w3);
      }
      g_live_out[e] = c;
    }
  } else if constexpr (LDS_LIVE) {
    __syncthreads();
    int4* dst = reinterpret_cast<int4*>(g_live_out);
    for (int i = threadIdx.x; i < (int)(ls / 4); i += kLoopBlock) dst[i] = reinterpret_cast<const int4*>(live)[i];
    if (!sreg_ok)
      for (int i = threadIdx.x; i < st.spent_words; i += kLoopBlock) g_spent[i] = spent[i];
  }
}

// ---------------------------------------------------------------------------
// Node-grouped head at the root (sections "The batched engine" and "The sparse
// output layer": the rows a batch needs are the union of the legal sets, so a
// row shared by sequences at the same node is read once for all of them).
// Every pointer starts at the root, the widest node of a catalog with many
// first tokens.  Before each pointer phase of the resident loop this kernel
// takes the root step of every sequence standing there ("members"), each with
// the hidden vector of its own current step: workgroup (x, y) loads 4*U root
// rows once and dots them with the vectors of members [y*mt, y*mt+mt) staged in
// LDS, in the fixed per-row order of the other kernels (bit-identical logits),
// and each member's legal edges go into key[s] with an atomic max.
// ---------------------------------------------------------------------------
template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void root_head_kernel(DevTrie tr, DevState st, LoopIO io, int mt, int rt, int mtiles) {
  constexpr int EL = DT == 0 ? 4 : 8;
  constexpr int U = rows_per_pass(NC);
  constexpr int MPW = 4;  // members staged per wavefront per round
  // [mt][nq] members' hidden vectors, then int64 hidden offsets[B], int members[B]
  extern __shared__ uint4 sh[];
  __shared__ int s_cnt[kWavesPerBlock];
  __shared__ unsigned long long s_best[16];
  const int lane = __lane_id();
  const int wv = wave_id();
  const int nq = io.H / EL;
  int64_t* s_off = reinterpret_cast<int64_t*>(sh + (size_t)mt * nq);
  int* s_mem = reinterpret_cast<int*>(s_off + st.B);
  const bool rst = io.reset != 0;
  const bool later = (io.flags & kLoopLater) != 0;
  int tx, ty;
  if (!root_tile((int)blockIdx.x, rt, mtiles, tx, ty)) return;
  if (threadIdx.x < 16) s_best[threadIdx.x] = 0ull;
  // this wavefront's U root edges (the root is not a terminal: content edges
  // only); their rows are requested first, so that the member bookkeeping
  // below overlaps the gathers
  const int r1 = tr.begin[1];
  const int e0 = tr.begin[0] + (tx * kWavesPerBlock + wv) * U;
  int rows[U];
#pragma unroll
  for (int u = 0; u < U; ++u) rows[u] = e0 + u < r1 ? tr.tok[e0 + u] : -1;
  uint4 raw[U][NC];
  issue_rows<NC, U>((const uint4*)io.emb, nq, rows, raw, lane);
  // members in ascending sequence order (every workgroup builds the same list),
  // with the offset of the hidden vector of each one's current step
  int n_mem = 0;
  for (int s0 = 0; s0 < st.B; s0 += kBlock) {
    const int s = s0 + (int)threadIdx.x;
    bool ok = false;
    int t = 0;
    if (s < st.B) {
      t = later ? st.tstep[s] : 0;
      const int stat = st.status[s], fin = st.finished[s], nd = st.node[s], dp = st.depth[s];
      ok = t < io.T && (rst || (stat == kSeqOk && fin == 0 && nd == 0 && dp == 0));
    }
    const unsigned long long m = __ballot(ok);
    if (lane == 0) s_cnt[wv] = __popcll(m);
    lds_barrier();
    int off = n_mem;
    for (int w = 0; w < wv; ++w) off += s_cnt[w];
    if (ok) {
      const int idx = off + __popcll(m & ((1ull << lane) - 1ull));
      s_mem[idx] = s;
      s_off[idx] = ((int64_t)t * st.B + s) * nq;
    }
    for (int w = 0; w < kWavesPerBlock; ++w) n_mem += s_cnt[w];
    lds_barrier();
  }
  const int m0 = ty * mt;
  const int cnt = min(mt, n_mem - m0);
  if (cnt <= 0) return;  // the same for the whole workgroup
  // stage the members' vectors: every load of a round before its stores
  const uint4* hid = (const uint4*)io.hidden_seq;
  for (int jb = wv; jb < cnt; jb += kWavesPerBlock * MPW) {
    uint4 v[MPW][NC];
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int j = jb + u * kWavesPerBlock;
      if (j < cnt) load_hidden<NC>(hid + s_off[m0 + j], nq, v[u], lane);
    }
#pragma unroll
    for (int u = 0; u < MPW; ++u) {
      const int j = jb + u * kWavesPerBlock;
      if (j >= cnt) continue;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c * kWave + lane < nq) sh[j * nq + c * kWave + lane] = v[u][c];
    }
  }
  // lane j checks member j's live counts of the wavefront's edges
  const int32_t* my_live = nullptr;
  if (lane < cnt) my_live = rst ? tr.live0 : st.live + (int64_t)s_mem[m0 + lane] * tr.live_stride;
  unsigned long long legal[U];
#pragma unroll
  for (int u = 0; u < U; ++u) legal[u] = __ballot(rows[u] >= 0 && lane < cnt && my_live[e0 + u] > 0);
  lds_barrier();  // staged vectors visible
  // two members per pass: independent accumulation chains side by side
  for (int j = 0; j < cnt; j += 2) {
    const int j1 = min(j + 1, cnt - 1);
    uint4 hq0[NC], hq1[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = c * kWave + lane;
      const int ii = i < nq ? i : 0;
      hq0[c] = c * kWave < nq ? sh[j * nq + ii] : make_uint4(0, 0, 0, 0);
      hq1[c] = c * kWave < nq ? sh[j1 * nq + ii] : make_uint4(0, 0, 0, 0);
    }
    float l0[U], l1[U];
    finish_rows<DT, NC, U>(nq, rows, raw, hq0, l0, lane);
    finish_rows<DT, NC, U>(nq, rows, raw, hq1, l1, lane);
    unsigned long long b0 = 0ull, b1 = 0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((legal[u] >> j) & 1ull) b0 = max(b0, pack_key(l0[u], (uint32_t)(e0 + u)));
      if ((legal[u] >> j1) & 1ull) b1 = max(b1, pack_key(l1[u], (uint32_t)(e0 + u)));
    }
    if (lane == 0) {
      if (b0) __hip_atomic_fetch_max(&s_best[j], b0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (b1 && j1 != j) __hip_atomic_fetch_max(&s_best[j1], b1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  lds_barrier();
  // this tile's best per member (0: none legal); the loop takes the max over tiles
  if ((int)threadIdx.x < cnt) st.rkey[(int64_t)tx * st.B + s_mem[m0 + threadIdx.x]] = s_best[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Dense cross-check: vocabulary bitmask, all-V head, masked argmax, advance.
// ---------------------------------------------------------------------------

// One workgroup per sequence builds its V-bit mask in LDS, then stores it.
__global__ __launch_bounds__(kBlock) void dense_mask_kernel(DevTrie tr, DevState st, uint32_t* out) {
  extern __shared__ uint32_t smask[];
  const int s = blockIdx.x;
  const int mw = st.mask_words;
  for (int i = threadIdx.x; i < mw; i += kBlock) smask[i] = 0u;
  __syncthreads();
  Seq q;
  if (load_seq(tr, st, s, q)) {
    const int32_t* live = st.live + (int64_t)s * tr.live_stride;
    for (int e = q.b0 + threadIdx.x; e < q.b1; e += kBlock) {
      const int c = tr.child[e];
      if (edge_ok(c, c >= 0 ? live[e] : 0, q)) {
        const int t = tr.tok[e];
        atomicOr(&smask[t >> 5], 1u << (t & 31));
      }
    }
  }
  __syncthreads();
  uint32_t* dst = (out ? out : st.mask) + (int64_t)s * mw;
  for (int i = threadIdx.x; i < mw; i += kBlock) dst[i] = smask[i];
}

// Bitmask-fed materialiser ("Understanding Inference for Systems Engineers",
// the masked head of Part 7: the legal rows are read off a vocabulary bitmask
// with a popcount scan, then only those rows go through the head).  One
// workgroup per sequence: thread i counts the set bits of its run of words,
// an exclusive scan over the workgroup gives each run's first slot, and the
// runs write their token ids in ascending order.  Bits at or past V are not
// tokens and are ignored.
__global__ __launch_bounds__(kBlock) void mask_rows_kernel(const uint32_t* mask, int W, int V, int cap,
                                                           int32_t* rows, int32_t* n_rows) {
  __shared__ int s_scan[kBlock];
  extern __shared__ uint32_t s_words[];  // the sequence's mask row, staged with coalesced loads
  const int s = blockIdx.x;
  {
    const uint32_t* g = mask + (int64_t)s * W;
    constexpr int L = 16;  // loads per thread in flight
    for (int base = 0; base < W; base += L * kBlock) {
      uint32_t v[L];
#pragma unroll
      for (int u = 0; u < L; ++u) {
        const int w = base + u * kBlock + (int)threadIdx.x;
        v[u] = w < W ? g[w] : 0u;
      }
#pragma unroll
      for (int u = 0; u < L; ++u) {
        const int w = base + u * kBlock + (int)threadIdx.x;
        if (w < W) s_words[w] = v[u];
      }
    }
    __syncthreads();
  }
  const uint32_t* m = s_words;
  const int per = (W + kBlock - 1) / kBlock;
  const int w0 = min(W, (int)threadIdx.x * per), w1 = min(W, w0 + per);
  auto word = [&](int w) -> uint32_t {
    uint32_t x = m[w];
    const int lo = w * 32;
    if (lo + 32 > V) x &= (V - lo) >= 32 ? 0xFFFFFFFFu : ((1u << (V - lo)) - 1u);
    return x;
  };
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(word(w));
  s_scan[threadIdx.x] = c;
  __syncthreads();
  for (int d = 1; d < kBlock; d <<= 1) {  // inclusive scan
    const int v = threadIdx.x >= (unsigned)d ? s_scan[threadIdx.x - d] : 0;
    __syncthreads();
    s_scan[threadIdx.x] += v;
    __syncthreads();
  }
  int off = s_scan[threadIdx.x] - c;
  int32_t* out = rows + (int64_t)s * cap;
  for (int w = w0; w < w1 && off < cap; ++w) {
    uint32_t x = word(w);
    while (x && off < cap) {
      out[off++] = w * 32 + __builtin_ctz(x);
      x &= x - 1u;
    }
  }
  if (threadIdx.x == kBlock - 1) n_rows[s] = s_scan[kBlock - 1];
}

// Every logit of every sequence; masked-in ones feed the per-sequence key.
// Grid-stride over groups of U consecutive rows per wavefront.
template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void dense_head_kernel(DevState st, StepIO io, float* full_logits) {
  constexpr int U = rows_per_pass(NC);
  constexpr int EL = DT == 0 ? 4 : 8;
  const int lane = __lane_id();
  const int gw = blockIdx.x * kWavesPerBlock + wave_id();
  const int nw = gridDim.x * kWavesPerBlock;
  const int nq = io.H / EL;
  const int V = io.V;
  const uint4* emb = (const uint4*)io.emb;
  const cuint_p cmask = (cuint_p)st.mask;
  uint4 hq[NC];
  if (st.B == 1) load_hidden<NC>((const uint4*)io.hidden, nq, hq, lane);
  for (int v0 = gw * U; v0 < V; v0 += nw * U) {
    int rows[U];
#pragma unroll
    for (int u = 0; u < U; ++u) rows[u] = v0 + u < V ? v0 + u : -1;
    for (int b = 0; b < st.B; ++b) {
      if (st.B > 1) load_hidden<NC>((const uint4*)io.hidden + (int64_t)b * nq, nq, hq, lane);
      float l[U];
      dot_rows<DT, NC, U, true>(emb, nq, rows, hq, l, lane);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (rows[u] < 0) continue;
        const int v = rows[u];
        if (full_logits && lane == u) full_logits[(int64_t)b * V + v] = l[u];
        const uint32_t word = cmask[(int64_t)b * st.mask_words + (v >> 5)];
        if (((word >> (v & 31)) & 1u) && lane == 0)
          __hip_atomic_fetch_max(&st.key[b], pack_key(l[u], (uint32_t)v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Dense head for B > 1 on the matrix cores (the one dense contraction of the
// path: [B x H] . [H x V]).  logits = h . E^T through v_mfma_f32_16x16x32_bf16
// (fp32 accumulation in the matrix core's own order).  A workgroup of four
// wavefronts takes 64*MT vocabulary rows, MT tiles of 16 per wavefront
// (operand A: lane l holds row l%16, elements 8*(l/16)..+8 of the current
// 32-wide K step); all B sequences go in tiles of 16 (operand B from LDS,
// where the hidden vectors of each 128-wide K block are staged with padded
// rows, 17 KB at B = 64 so that eight workgroups fit a compute unit); the
// table operand is loaded one K step ahead; the result tile has
// lane l holding sequence l%16, rows 4*(l/16)+i.  Masked-in logits go to
// the per-sequence key with an atomic max; full logits are written if asked.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kDenseKB = 128;                   // K block staged in LDS
constexpr int kDenseStride = kDenseKB / 8 + 1;  // uint4 per staged row (+1 against bank conflicts)

// Stage the hidden vectors' K block [kb, kb + kDenseKB) into an LDS buffer.
__device__ __forceinline__ void stage_hidden(uint4* buf, const uint4* hid, int B, int nseq, int nq, int kb) {
  const int qb = kb / 8;
  for (int idx = threadIdx.x; idx < nseq * (kDenseKB / 8); idx += kBlock) {
    const int sq = idx / (kDenseKB / 8), qq = idx % (kDenseKB / 8);
    buf[sq * kDenseStride + qq] = (sq < B && qb + qq < nq) ? hid[(int64_t)sq * nq + qb + qq] : make_uint4(0, 0, 0, 0);
  }
}

template <int MAXT, int MT>
__global__ __launch_bounds__(kBlock) void dense_mfma_kernel(DevState st, StepIO io, float* full_logits, int ntiles) {
  extern __shared__ uint4 sh[];  // [ntiles*16][kDenseStride]
  const int lane = __lane_id();
  const int wv = wave_id();
  const int V = io.V, H = io.H, B = st.B;
  const int nq = H / 8;
  const uint4* emb = (const uint4*)io.emb;
  const uint4* hid = (const uint4*)io.hidden;
  const int nseq = ntiles * 16;
  constexpr int kRows = 4 * MT * 16;  // rows per workgroup
  const int nblk = (V + kRows - 1) / kRows;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int m0 = blk * kRows + wv * (MT * 16);
    const uint4* arow_p[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) arow_p[m] = emb + (int64_t)min(m0 + m * 16 + (lane & 15), V - 1) * nq;
    f32x4_t acc[MT][MAXT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < MAXT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Operand A one K step ahead.  One load covers 64 bytes of each of 16
    // rows, half a 128-byte line: the next K step reads the other half, so
    // these are ordinary (cached) loads; a non-temporal hint costs ~18% here.
    u32x4_t an[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      an[m] = *reinterpret_cast<const u32x4_t*>(arow_p[m] + (lane >> 4));
    for (int kb = 0; kb < H; kb += kDenseKB) {
      __syncthreads();  // the previous block is consumed
      stage_hidden(sh, hid, B, nseq, nq, kb);
      __syncthreads();
      const int kend = min(kDenseKB, H - kb);
      for (int ks = 0; ks < kend; ks += 32) {
        bf16x8_t a[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) a[m] = __builtin_bit_cast(bf16x8_t, an[m]);
        const int kn = kb + ks + 32;  // next K step
        if (kn < H) {
#pragma unroll
          for (int m = 0; m < MT; ++m)
            an[m] = *reinterpret_cast<const u32x4_t*>(arow_p[m] + kn / 8 + (lane >> 4));
        }
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t < ntiles) {
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, sh[(t * 16 + (lane & 15)) * kDenseStride + ks / 8 + (lane >> 4)]);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b, acc[m][t], 0, 0, 0);
          }
        }
      }
    }
    // epilogue: tile m, sequence t*16 + lane%16, rows m0 + m*16 + 4*(lane/16) + i
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r0 = m0 + m * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= ntiles) continue;
        const int sq = t * 16 + (lane & 15);
        if (sq >= B) continue;
        const uint32_t word = r0 < V ? st.mask[(int64_t)sq * st.mask_words + (r0 >> 5)] : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          if (r >= V) continue;
          const float l = acc[m][t][i];
          if (full_logits) full_logits[(int64_t)sq * V + r] = l;
          if ((word >> ((r0 & 31) + i)) & 1u)
            __hip_atomic_fetch_max(&st.key[sq], pack_key(l, (uint32_t)r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Grouped root head on the matrix cores (bf16, H = 128 * KS): workgroup
// (x, y) takes root rows [16x, 16x+16) and members [16y, 16y+16).  The four
// wavefronts split the hidden dimension in quarters; each requests all of its
// quarter of the 16 rows up front (operand A, KS steps of 32) and reads the
// members' vectors from LDS (operand B); the four partial 16 x 16 tiles are
// summed in a fixed order ((w0 + w1) + (w2 + w3)), so results do not depend on
// scheduling, and each member's best legal edge of the tile goes to rkey.
template <int KS>
__global__ __launch_bounds__(kBlock) void root_mfma_kernel(DevTrie tr, DevState st, LoopIO io, int rb0, int rb1,
                                                           int rt, int mtiles) {
  extern __shared__ uint4 sh[];  // int64 offsets[B], then int members[B]
  __shared__ f32x4_t s_part[3][kWave];
  __shared__ int s_cnt[kWavesPerBlock];
  const int lane = __lane_id();
  const int wv = wave_id();
  const int nq = io.H / 8;
  int64_t* s_off = reinterpret_cast<int64_t*>(sh);
  int* s_mem = reinterpret_cast<int*>(s_off + st.B);
  const bool rst = io.reset != 0;
  const bool later = (io.flags & kLoopLater) != 0;
  int tx, ty;
  if (!root_tile((int)blockIdx.x, rt, mtiles, tx, ty)) return;
  const int r1 = rb1;  // the root's edges are [rb0, rb1)
  const int eb = rb0 + tx * 16;
  // the states of the member list's first sequences and this lane's root
  // token, requested together (loads complete in order: the states are not
  // to wait behind the rows)
  int f_t = 0, f_stat = 0, f_fin = 1, f_nd = 0, f_dp = 0;
  if ((int)threadIdx.x < st.B) {
    f_t = later ? st.tstep[threadIdx.x] : 0;
    f_stat = st.status[threadIdx.x];
    f_fin = st.finished[threadIdx.x];
    f_nd = st.node[threadIdx.x];
    f_dp = st.depth[threadIdx.x];
  }
  const int my_e = min(eb + (lane & 15), r1 - 1);
  const int my_tok = tr.tok[my_e];
  // operand A: lane l holds row l % 16, elements 8 (l / 16) .. + 8 of each
  // 32-wide step of this wavefront's quarter
  const uint4* arow = (const uint4*)io.emb + (int64_t)my_tok * nq + wv * (KS * 4) + (lane >> 4);
  u32x4_t a[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) a[j] = *reinterpret_cast<const u32x4_t*>(arow + j * 4);
  // members in ascending sequence order (every workgroup builds the same
  // list); the first chunk from the states requested above, outside the loop,
  // so that no path to it waits for the rows
  int n_mem = 0;
  auto chunk = [&](int s, int t, int stat, int fin, int nd, int dp) {
    const bool ok = s < st.B && t < io.T && (rst || (stat == kSeqOk && fin == 0 && nd == 0 && dp == 0));
    const unsigned long long m = __ballot(ok);
    if (lane == 0) s_cnt[wv] = __popcll(m);
    lds_barrier();
    int off = n_mem;
    for (int w = 0; w < wv; ++w) off += s_cnt[w];
    if (ok) {
      const int idx = off + __popcll(m & ((1ull << lane) - 1ull));
      s_mem[idx] = s;
      s_off[idx] = ((int64_t)t * st.B + s) * nq;
    }
    for (int w = 0; w < kWavesPerBlock; ++w) n_mem += s_cnt[w];
    lds_barrier();
  };
  chunk((int)threadIdx.x, f_t, f_stat, f_fin, f_nd, f_dp);
  for (int s0 = kBlock; s0 < st.B; s0 += kBlock) {
    const int s = s0 + (int)threadIdx.x;
    int t = 0, stat = 0, fin = 1, nd = 0, dp = 0;
    if (s < st.B) {
      t = later ? st.tstep[s] : 0;
      stat = st.status[s];
      fin = st.finished[s];
      nd = st.node[s];
      dp = st.depth[s];
    }
    chunk(s, t, stat, fin, nd, dp);
  }
  const int m0 = ty * 16;
  const int cnt = min(16, n_mem - m0);
  if (cnt <= 0) return;  // the same for the whole workgroup
  // live counts of this lane's four (row, member) results (wavefront 0 uses them)
  const int col = lane & 15;
  int lv[4] = {0, 0, 0, 0};
  if (wv == 0 && col < cnt) {
    const int32_t* live = rst ? tr.live0 : st.live + (int64_t)s_mem[m0 + col] * tr.live_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = eb + 4 * (lane >> 4) + i;
      lv[i] = e < r1 ? live[e] : 0;
    }
  }
  // operand B straight from the members' vectors: wavefront wv needs only its
  // quarter of each, so there is nothing to share through LDS (lane l: member
  // l % 16, elements 8 (l / 16) .. + 8 of each 32-wide step; missing members
  // re-read member m0's vector and are zeroed)
  const bool have = col < cnt;
  const uint4* bsrc = (const uint4*)io.hidden_seq + s_off[m0 + (have ? col : 0)] + wv * (KS * 4) + (lane >> 4);
  u32x4_t bq[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) bq[j] = *reinterpret_cast<const u32x4_t*>(bsrc + j * 4);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const u32x4_t bj = have ? bq[j] : u32x4_t{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[j]), __builtin_bit_cast(bf16x8_t, bj),
                                                  acc, 0, 0, 0);
  }
  if (wv > 0) s_part[wv - 1][lane] = acc;
  lds_barrier();
  if (wv != 0) return;
  acc = (acc + s_part[0][lane]) + (s_part[1][lane] + s_part[2][lane]);
  // lane l: member col, rows 4 (l / 16) + i
  unsigned long long best = 0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lv[i] > 0) best = max(best, pack_key(acc[i], (uint32_t)(eb + 4 * (lane >> 4) + i)));
#pragma unroll
  for (int d = 16; d < kWave; d <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, d);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), d);
    best = max(best, ((unsigned long long)hi << 32) | lo);
  }
  if (lane < cnt) st.rkey[(int64_t)tx * st.B + s_mem[m0 + lane]] = best;
}

// The same contraction with the K loop outside (H a multiple of 128): each
// wavefront keeps T row tiles of 16 in accumulators for the whole of H, so a
// workgroup stages each 128-wide K block of the hidden vectors once for its
// 64*T rows (double-buffered: the next block's slice and table data are in
// flight while the current one is multiplied, one barrier per block).  A lane
// reads four consecutive K steps of its row per block, i.e. 64 bytes; the
// four lanes of a row cover a full 256-byte run, so no line is read twice.
// Sums in the same K order as dense_mfma_kernel.
template <int MAXT, int T>
__global__ __launch_bounds__(kBlock) void dense_mfma_kstream_kernel(DevState st, StepIO io, float* full_logits,
                                                                     int ntiles, int nblk) {
  extern __shared__ uint4 sh[];  // two buffers of [ntiles*16][kDenseStride]
  const int lane = __lane_id();
  const int wv = wave_id();
  const int V = io.V, H = io.H, B = st.B;
  const int nq = H / 8;
  const uint4* emb = (const uint4*)io.emb;
  const uint4* hid = (const uint4*)io.hidden;
  const int nseq = ntiles * 16;
  const int bufsz = nseq * kDenseStride;
  constexpr int kRows = 4 * T * 16;
  const int nkb = H / kDenseKB;
  uint4 hv[MAXT];  // this thread's share of a staged block: entries tid + 256u
  auto hload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      const int sq = idx >> 4, qq = idx & 15;
      hv[u] = (idx < nseq * 16 && sq < B) ? hid[(int64_t)sq * nq + kb * 16 + qq] : make_uint4(0, 0, 0, 0);
    }
  };
  auto hstore = [&](uint4* buf) {
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      if (idx < nseq * 16) buf[(idx >> 4) * kDenseStride + (idx & 15)] = hv[u];
    }
  };
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int m0 = blk * kRows + wv * (T * 16);
    const uint4* rp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) rp[t] = emb + (int64_t)min(m0 + t * 16 + (lane & 15), V - 1) * nq + (lane >> 4);
    f32x4_t acc[T][MAXT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < MAXT; ++m) acc[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t a[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[t][j] = *reinterpret_cast<const u32x4_t*>(rp[t] + j * 4);
    hload(0);
    __syncthreads();  // the buffers of the previous row block are consumed
    hstore(sh);
    int cur = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      const bool more = kb + 1 < nkb;
      u32x4_t an[T][4];
      if (more) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) an[t][j] = *reinterpret_cast<const u32x4_t*>(rp[t] + (kb + 1) * 16 + j * 4);
        hload(kb + 1);
      }
      lds_barrier();  // block kb staged; every wavefront is done with the other buffer
      const uint4* hb = sh + cur * bufsz;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
          if (m < ntiles) {
            const bf16x8_t b =
                __builtin_bit_cast(bf16x8_t, hb[(m * 16 + (lane & 15)) * kDenseStride + j * 4 + (lane >> 4)]);
#pragma unroll
            for (int t = 0; t < T; ++t)
              acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[t][j]), b, acc[t][m],
                                                                   0, 0, 0);
          }
        }
      }
      if (more) {
        hstore(sh + (cur ^ 1) * bufsz);
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) a[t][j] = an[t][j];
      }
      cur ^= 1;
    }
    // epilogue: tile t, sequence m*16 + lane%16, rows m0 + t*16 + 4*(lane/16) + i
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int r0 = m0 + t * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int m = 0; m < MAXT; ++m) {
        if (m >= ntiles) continue;
        const int sq = m * 16 + (lane & 15);
        if (sq >= B) continue;
        const uint32_t word = r0 < V ? st.mask[(int64_t)sq * st.mask_words + (r0 >> 5)] : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          if (r >= V) continue;
          const float l = acc[t][m][i];
          if (full_logits) full_logits[(int64_t)sq * V + r] = l;
          if ((word >> ((r0 & 31) + i)) & 1u)
            __hip_atomic_fetch_max(&st.key[sq], pack_key(l, (uint32_t)r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// The K-streamed contraction with every load requested two K blocks ahead
// (B <= 64): table fragments in a ring of three register slots and hidden
// slices in a ring of two per wavefront.  The K loop is fully unrolled (NKB
// blocks of KB: H fixed per instantiation), so each slot keeps its role
// without copies (a copy of a fragment still in flight would wait for it) and
// every wait counts exactly how many younger loads may stay in flight (loads
// complete in issue order): the products of block kb wait only for loads
// issued two blocks earlier.  All MAXT member tiles are computed (missing
// members are zeros), which keeps the unrolled body free of branches.  Same
// products and K order as the kernel above, so bit-identical logits.
template <int MAXT, int T, int KB, int NKB>
__global__ __launch_bounds__(kBlock) void dense_mfma_kring_kernel(DevState st, StepIO io, float* full_logits,
                                                                   int ntiles, int nblk) {
  extern __shared__ uint4 sh[];  // two buffers of [ntiles*16][KS]
  constexpr int KQ = KB / 8;     // uint4 per staged row
  constexpr int KS = KQ + 1;     // staged row stride (+1 against bank conflicts)
  constexpr int KJ = KB / 32;    // matrix-core K steps per block
  const int lane = __lane_id();
  const int wv = wave_id();
  const int V = io.V, H = io.H, B = st.B;
  const int nq = H / 8;
  const uint4* emb = (const uint4*)io.emb;
  const uint4* hid = (const uint4*)io.hidden;
  constexpr int nseq = MAXT * 16;  // every member tile is computed (missing members are zeros): no branches
  (void)ntiles;
  const int bufsz = nseq * KS;
  constexpr int kRows = 4 * T * 16;
  constexpr int nkb = NKB;  // H / KB, fixed so that the K loop unrolls fully
  typedef u32x4_t Frag[T][KJ];
  constexpr int HV = MAXT * KQ / 16;  // this thread's share of a staged block
  typedef uint4 Slice[HV];
  Slice hv0, hv1;  // hidden slices, two blocks in flight
  auto hload = [&](Slice& hv, int kb) {
#pragma unroll
    for (int u = 0; u < HV; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      const int sq = idx / KQ, qq = idx % KQ;
      hv[u] = (idx < nseq * KQ && sq < B) ? hid[(int64_t)sq * nq + kb * KQ + qq] : make_uint4(0, 0, 0, 0);
    }
  };
  auto hstore = [&](uint4* buf, const Slice& hv) {
#pragma unroll
    for (int u = 0; u < HV; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      if (idx < nseq * KQ) buf[(idx / KQ) * KS + idx % KQ] = hv[u];
    }
  };
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int m0 = blk * kRows + wv * (T * 16);
    const uint4* rp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) rp[t] = emb + (int64_t)min(m0 + t * 16 + (lane & 15), V - 1) * nq + (lane >> 4);
    f32x4_t acc[T][MAXT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < MAXT; ++m) acc[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto fetch = [&](Frag& f, int kb) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int j = 0; j < KJ; ++j) f[t][j] = *reinterpret_cast<const u32x4_t*>(rp[t] + kb * KQ + j * 4);
    };
    Frag f0, f1, f2;
    hload(hv0, 0);
    fetch(f0, 0);
    if (nkb > 1) {
      hload(hv1, 1);
      fetch(f1, 1);
    }
    __syncthreads();  // the buffers of the previous row block are consumed
    hstore(sh, hv0);
    // block kb: its fragments are in `cur`; the hidden slice of block kb + 2
    // goes into `hnext` (free: block kb's slice was staged in the previous
    // step) and its table fragments into `ahead`
    auto step = [&](const Frag& cur, Frag& ahead, Slice& hnext, const Slice& hstage, int kb) {
      if (kb + 2 < nkb) {
        hload(hnext, kb + 2);
        fetch(ahead, kb + 2);
      }
      lds_barrier();  // block kb staged; every wavefront is done with the other buffer
      const uint4* hb = sh + (kb & 1) * bufsz;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
          const bf16x8_t b = __builtin_bit_cast(bf16x8_t, hb[(m * 16 + (lane & 15)) * KS + j * 4 + (lane >> 4)]);
#pragma unroll
          for (int t = 0; t < T; ++t)
            acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[t][j]), b, acc[t][m],
                                                                 0, 0, 0);
        }
      }
      if (kb + 1 < nkb) hstore(sh + ((kb + 1) & 1) * bufsz, hstage);
    };
#pragma unroll
    for (int kb = 0; kb < nkb; ++kb) {
      const int r = kb % 3;
      step(r == 0 ? f0 : r == 1 ? f1 : f2, r == 0 ? f2 : r == 1 ? f0 : f1, (kb & 1) ? hv1 : hv0, (kb & 1) ? hv0 : hv1,
           kb);
    }
    // epilogue: tile t, sequence m*16 + lane%16, rows m0 + t*16 + 4*(lane/16) + i
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int r0 = m0 + t * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int m = 0; m < MAXT; ++m) {
        const int sq = m * 16 + (lane & 15);
        if (sq >= B) continue;
        const uint32_t word = r0 < V ? st.mask[(int64_t)sq * st.mask_words + (r0 >> 5)] : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          if (r >= V) continue;
          const float l = acc[t][m][i];
          if (full_logits) full_logits[(int64_t)sq * V + r] = l;
          if ((word >> ((r0 & 31) + i)) & 1u)
            __hip_atomic_fetch_max(&st.key[sq], pack_key(l, (uint32_t)r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// The contraction for 64 < B <= 256 (H a multiple of KB * R): each wavefront
// keeps T row tiles x MAXT member tiles of accumulators for the whole of H.
// The hidden slice of a KB-wide K block goes through registers into one of
// two LDS buffers (requested one block ahead, stored after the products);
// the table fragments rotate over a ring of R register slots, requested R - 1
// blocks ahead.  The K loop is unrolled by R so that every slot keeps its
// role without copies, and its body has no branches: the requests past the
// last block repeat the last block (cached, unused).  All MAXT member tiles are
// computed (missing members read a copy of the last one and are dropped).
// At 8 member tiles the kernel fits 256 registers, so two workgroups share a
// compute unit; at 16 the accumulators take the accumulation registers and
// one workgroup runs per unit.  Same products and K order as the kernels
// above, so bit-identical logits.
template <int MAXT, int T, int KB, int R>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(MAXT <= 8 ? 2 : 1, 2)))
void dense_mfma_wide_kernel(DevState st, StepIO io, float* full_logits, int nblk) {
  extern __shared__ uint4 sh[];  // two buffers of [MAXT*16][KS]
  constexpr int KQ = KB / 8;     // uint4 per staged row
  constexpr int KS = KQ + 1;     // staged row stride (+1 against bank conflicts)
  constexpr int KJ = KB / 32;    // matrix-core K steps per block
  constexpr int nseq = MAXT * 16;
  constexpr int bufsz = nseq * KS;
  constexpr int HV = nseq * KQ / kBlock;
  constexpr int kRows = 4 * T * 16;
  static_assert(nseq * KQ % kBlock == 0, "whole staging rounds");
  const int lane = __lane_id();
  const int wv = wave_id();
  const int V = io.V, B = st.B;
  const int nq = io.H / 8;
  const int nkb = io.H / KB;  // a multiple of R
  const uint4* emb = (const uint4*)io.emb;
  const uint4* hid = (const uint4*)io.hidden;
  typedef u32x4_t Frag[T][KJ];
  u32x4_t hv[HV];  // a vector type: copies of uint4 (a struct) would go through private memory
  auto hload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < HV; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      const int sq = idx / KQ, qq = idx % KQ;
      hv[u] = *reinterpret_cast<const u32x4_t*>(hid + (int64_t)min(sq, B - 1) * nq + kb * KQ + qq);
    }
  };
  // LDS position (in uint4) of member row `row`, 16-byte column `col` of a staged block
  auto lpos = [](int row, int col) { return row * KS + col; };
  auto hstore = [&](uint4* buf) {
#pragma unroll
    for (int u = 0; u < HV; ++u) {
      const int idx = u * kBlock + (int)threadIdx.x;
      *reinterpret_cast<u32x4_t*>(buf + lpos(idx / KQ, idx % KQ)) = hv[u];
    }
  };
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int m0 = blk * kRows + wv * (T * 16);
    const uint4* rp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) rp[t] = emb + (int64_t)min(m0 + t * 16 + (lane & 15), V - 1) * nq + (lane >> 4);
    auto fetch = [&](Frag& f, int kb) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int j = 0; j < KJ; ++j) f[t][j] = *reinterpret_cast<const u32x4_t*>(rp[t] + kb * KQ + j * 4);
    };
    f32x4_t acc[T][MAXT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < MAXT; ++m) acc[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Frag f[R];
    hload(0);
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) fetch(f[r], r);
    __syncthreads();  // the buffers of the previous row block are consumed
    hstore(sh);
    // block kb from slot kb % R; block kb + R - 1 goes into the slot block
    // kb - 1 used, and the hidden slice of block kb + 1 is requested first
    for (int k0 = 0; k0 < nkb; k0 += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int kb = k0 + r;
        hload(min(kb + 1, nkb - 1));
        fetch(f[(r + R - 1) % R], min(kb + R - 1, nkb - 1));
        lds_barrier();  // block kb staged; every wavefront is done with the other buffer
        const uint4* hb = sh + (kb & 1) * bufsz;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
#pragma unroll
          for (int m = 0; m < MAXT; ++m) {
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, hb[lpos(m * 16 + (lane & 15), j * 4 + (lane >> 4))]);
#pragma unroll
            for (int t = 0; t < T; ++t)
              acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f[r][t][j]), b,
                                                                   acc[t][m], 0, 0, 0);
          }
        }
        // schedule: kAhead LDS reads first, then one read per T products, so
        // that at most kAhead + 1 hidden fragments occupy registers
        constexpr int kAhead = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int g = 0; g < KJ * MAXT - kAhead; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, T, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead * T, 0);
        hstore(sh + ((kb + 1) & 1) * bufsz);  // after the last block: a copy into the free buffer, unused
      }
    }
    // epilogue: tile t, sequence m*16 + lane%16, rows m0 + t*16 + 4*(lane/16) + i.
    // The mask pointer passes through an empty asm statement so that the
    // addresses below are formed here, not kept in registers across the K
    // loop.  A lane's four rows of a tile share one mask word (r0 % 4 == 0);
    // bits past V are never set.  Each lane combines its masked-in keys of a
    // member tile (the unsigned max is order-independent) into one atomic.
    const uint32_t* mask = st.mask;
    asm volatile("" : "+s"(mask));
    const int rl = m0 + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
      const int sq = m * 16 + (lane & 15);
      const uint32_t* mrow = mask + (int64_t)min(sq, B - 1) * st.mask_words;
      unsigned long long best = 0ull;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int r0 = rl + t * 16;
        const uint32_t bits = r0 < V ? (mrow[r0 >> 5] >> (r0 & 31)) & 15u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((bits >> i) & 1u) best = max(best, pack_key(acc[t][m][i], (uint32_t)(r0 + i)));
      }
      if (sq < B && best)
        __hip_atomic_fetch_max(&st.key[sq], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (full_logits) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
          const int sq = m * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rl + t * 16 + i;
            if (sq < B && r < V) full_logits[(int64_t)sq * V + r] = acc[t][m][i];
          }
        }
    }
  }
}

// One wavefront per sequence: winner token from the key, its edge, advance.
__global__ __launch_bounds__(kWave) void dense_advance_kernel(DevTrie tr, DevState st, StepIO io) {
  const int s = blockIdx.x;
  const int lane = __lane_id();
  Seq q;
  if (!load_seq(tr, st, s, q)) {
    if (lane == 0) write_step_out(io, s, -1, NAN);
    return;
  }
  const unsigned long long key = st.key[s];
  int e = -2;
  float lg = NAN;
  if (key) {
    e = find_edge(tr, q, (int)key_id(key), lane);
    lg = key_logit(key);
  }
  advance(tr, st, &io, s, q, e, lg, lane);
  if (lane == 0) st.key[s] = 0ull;
}

// Teacher forcing: one wavefront per sequence.
__global__ __launch_bounds__(kWave) void forced_kernel(DevTrie tr, DevState st, const int32_t* forced) {
  const int s = blockIdx.x;
  const int lane = __lane_id();
  const int t = forced[s];
  Seq q;
  if (t < 0 || !load_seq(tr, st, s, q)) return;
  advance(tr, st, nullptr, s, q, find_edge(tr, q, t, lane), NAN, lane);
}

// The legal set alone, compacted in ascending token order (one wavefront per sequence).
__global__ __launch_bounds__(kWave) void legal_set_kernel(DevTrie tr, DevState st, int32_t* legal_tok,
                                                          int32_t* n_legal) {
  const int s = blockIdx.x;
  const int lane = __lane_id();
  Seq q;
  if (!load_seq(tr, st, s, q)) {
    if (lane == 0) n_legal[s] = -1;
    return;
  }
  const int32_t* live = st.live + (int64_t)s * tr.live_stride;
  int cnt = 0;
  for (int base = q.b0; base < q.b1; base += kWave) {
    const int e = base + lane;
    bool ok = false;
    int t = 0;
    if (e < q.b1) {
      const int c = tr.child[e];
      ok = edge_ok(c, c >= 0 ? live[e] : 0, q);
      t = tr.tok[e];
    }
    const unsigned long long m = __ballot(ok);
    if (ok) legal_tok[(int64_t)s * tr.cap + cnt + __popcll(m & ((1ull << lane) - 1ull))] = t;
    cnt += __popcll(m);
  }
  if (lane == 0) n_legal[s] = cnt;
}

// The sparse head alone over explicit row lists (same arithmetic as the step).
// Wavefront wv of a sequence's W = 4*split wavefronts owns the R consecutive
// list slots [wv*R, wv*R + R) (R <= 64): one coalesced load brings all its
// row ids, the count is read alongside, and the rows go through passes of U
// with the next pass's gathers in flight while the current pass is reduced.
template <int U>
__device__ __forceinline__ void pop_rows(unsigned long long& m, int id, int (&rows)[U], int (&slots)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (m) {
      const int j = (int)__builtin_ctzll(m);
      m &= m - 1;
      rows[u] = __builtin_amdgcn_readlane(id, j);
      slots[u] = j;
    } else {
      rows[u] = -1;
      slots[u] = 0;
    }
  }
}

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void gather_gemv_kernel(const uint4* __restrict__ emb, int V, int H,
                                                             const uint4* __restrict__ hidden,
                                                             const int32_t* rows_in, const int32_t* n_rows,
                                                             int cap, float* out, int split, int R) {
  constexpr int U = rows_per_pass(NC);
  constexpr int EL = DT == 0 ? 4 : 8;
  const int g = blockIdx.x;
  const int s = g / split;
  const int w = g - s * split;
  const int lane = __lane_id();
  const int wv = w * kWavesPerBlock + wave_id();
  const int j0 = wv * R;
  if (j0 >= cap) return;
  const int jl = j0 + lane;
  const bool in_cap = lane < R && jl < cap;
  const int id = in_cap ? rows_in[(int64_t)s * cap + jl] : -1;  // slots inside [B][cap]
  const int n = min(((cint_p)n_rows)[s], cap);
  const int nq = H / EL;
  uint4 hq[NC];
  load_hidden<NC>(hidden + (int64_t)s * nq, nq, hq, lane);
  float* o = out + (int64_t)s * cap + j0;
  const bool listed = in_cap && jl < n;
  const bool valid = listed && id >= 0 && id < V;
  if (listed && !valid) o[lane] = NAN;
  unsigned long long m = __ballot(valid);
  int rows_a[U], slots_a[U], rows_b[U], slots_b[U];
  uint4 raw_a[U][NC], raw_b[U][NC];
  float l[U];
  pop_rows<U>(m, id, rows_a, slots_a);
  issue_rows<NC, U, true>(emb, nq, rows_a, raw_a, lane);
  while (rows_a[0] >= 0) {
    pop_rows<U>(m, id, rows_b, slots_b);
    issue_rows<NC, U, true>(emb, nq, rows_b, raw_b, lane);
    finish_rows<DT, NC, U>(nq, rows_a, raw_a, hq, l, lane);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (rows_a[u] >= 0 && lane == u) o[slots_a[u]] = l[u];
    if (rows_b[0] < 0) break;
    pop_rows<U>(m, id, rows_a, slots_a);
    issue_rows<NC, U, true>(emb, nq, rows_a, raw_a, lane);
    finish_rows<DT, NC, U>(nq, rows_b, raw_b, hq, l, lane);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (rows_b[u] >= 0 && lane == u) o[slots_b[u]] = l[u];
  }
}

// ---------------------------------------------------------------------------
// Streaming-read reference ("Understanding Inference for Systems Engineers",
// Part 9 "Profiling": an achieved bandwidth is judged against what a plain
// streaming kernel reaches on the same machine, not only against the data
// sheet).  Every thread reads 16-byte words of one contiguous buffer in a
// grid-stride loop with U non-temporal loads in flight, XORs them together,
// and each wavefront XORs its result into one of 1024 words of out (spread so
// that the atomics do not queue on one address), so no load is dead code.
// ---------------------------------------------------------------------------

template <int U>
__global__ __launch_bounds__(kBlock) void read_ref_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t x = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i));
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
  if (__lane_id() == 0) atomicXor(out + ((blockIdx.x * kWavesPerBlock + wave_id()) & 1023u), x);
}

// ---------------------------------------------------------------------------
// State maintenance
// ---------------------------------------------------------------------------

// grid (x, B): row s = blockIdx.y.  kResetFull: live row copied from live0
// with 16-byte stores, spent row cleared; kResetPaths (grid x = 1): only the
// root paths of the stored entries.
__global__ __launch_bounds__(kBlock) void reset_kernel(DevTrie tr, DevState st, int kind) {
  const int s = blockIdx.y;
  uint32_t* sp = st.spent + (int64_t)s * st.spent_words;
  if (kind == kResetPaths) {
    restore_paths(tr, st, s, st.live + (int64_t)s * tr.live_stride, sp, wave_id(), kWavesPerBlock, __lane_id());
    __syncthreads();  // the stored entries are read before they are cleared below
  } else {
    if (kind == kResetFull) {
      const int q4 = tr.live_stride / 4;
      const int4* src = (const int4*)tr.live0;
      int4* dst = (int4*)(st.live + (int64_t)s * tr.live_stride);
      for (int i = blockIdx.x * kBlock + threadIdx.x; i < q4; i += gridDim.x * kBlock) dst[i] = src[i];
    }
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < st.spent_words; i += gridDim.x * kBlock) sp[i] = 0u;
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < st.k; i += kBlock) st.entries[(int64_t)s * st.k + i] = -1;
    if (threadIdx.x == 0) {
      st.node[s] = 0;
      st.depth[s] = 0;
      st.done[s] = 0;
      st.status[s] = kSeqOk;
      st.finished[s] = 0;
      st.nemit[s] = 0;
      st.key[s] = 0ull;
      st.arrive[s] = 0u;
      if (st.snap) st.snap[s] = 0;  // at the root, half 0 of the grouped step's snapshot
    }
  }
}

__global__ __launch_bounds__(kBlock) void snapshot_kernel(DevState st, int parity) {
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= st.B) return;
  st.snap[(int64_t)parity * st.B + s] = st.status[s] == kSeqOk && st.finished[s] == 0 ? st.node[s] : -1;
}

__global__ __launch_bounds__(kBlock) void finalize_kernel(DevState st, int32_t* len, int32_t* entries) {
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= st.B) return;
  if (st.status[s] == kSeqOk && st.finished[s] == 0) st.status[s] = kSeqNotDone;
  if (len) len[s] = st.nemit[s];
  if (entries)
    for (int j = 0; j < st.k; ++j) entries[(int64_t)s * st.k + j] = st.entries[(int64_t)s * st.k + j];
}

__global__ void set_live_kernel(DevTrie tr, DevState st, int32_t s, int32_t e, int32_t v) {
  if (threadIdx.x == 0) st.live[(int64_t)s * tr.live_stride + e] = v;
}

// ---------------------------------------------------------------------------
// Dispatch on (dtype, chunks per lane)
// ---------------------------------------------------------------------------
template <template <int, int> class F, typename... A>
hipError_t dispatch(int dtype, int nc, A&&... a) {
#define TMS_CASE(D, N) \
  if (dtype == D && nc == N) return F<D, N>::run(static_cast<A&&>(a)...);
  TMS_CASE(0, 1) TMS_CASE(0, 2) TMS_CASE(0, 4) TMS_CASE(0, 8) TMS_CASE(0, 16)
  TMS_CASE(1, 1) TMS_CASE(1, 2) TMS_CASE(1, 4) TMS_CASE(1, 8) TMS_CASE(1, 16)
#undef TMS_CASE
  return hipErrorInvalidValue;
}

hipError_t allow_lds(const void* k, size_t lds);

template <int DT, int NC>
struct StepLaunch {
  static hipError_t run(const DevTrie& tr, const DevState& st, const StepIO& io, bool fast, int split,
                        const StepGroup* grp, hipStream_t s) {
    const dim3 block(kBlock);
    if (!grp) {
      const dim3 grid((unsigned)(st.B * split));
      if (fast) hipLaunchKernelGGL((step_sparse_kernel<DT, NC, true>), grid, block, 0, s, tr, st, io, split);
      else hipLaunchKernelGGL((step_sparse_kernel<DT, NC, false>), grid, block, 0, s, tr, st, io, split);
      return hipGetLastError();
    }
    constexpr int EL = DT == 0 ? 4 : 8;
    const size_t lds = step_group_lds(io.H / EL, grp->nodes ? max(grp->mt, grp->gmt) : grp->mt);
    auto* k = grp->nodes ? (fast ? &step_grouped_kernel<DT, NC, true, true> : &step_grouped_kernel<DT, NC, false, true>)
                         : (fast ? &step_grouped_kernel<DT, NC, true> : &step_grouped_kernel<DT, NC, false>);
    if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
    const dim3 grid((unsigned)(st.B * grp->split + root_tile_grid(grp->rt, grp->mtiles)));
    hipLaunchKernelGGL(k, grid, block, lds, s, tr, st, io, grp->split, grp->rt, grp->mt, grp->mtiles, grp->parity,
                       grp->gmt);
    return hipGetLastError();
  }
};

// Raises a kernel's dynamic LDS limit on the current device when a launch
// needs more than the default 64 KB.  Remembered per (kernel, device), under a
// lock, so concurrent host threads and several devices are handled.
hipError_t allow_lds(const void* k, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> raised;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = raised[{k, dev}];
  if (lds <= have) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) have = lds;
  return e;
}

template <int DT, int NC>
struct LoopLaunch {
  template <int META, bool LIVE, bool SMALL, bool MASK = false>
  static hipError_t go(const DevTrie& tr, const DevState& st, const LoopIO& io, hipStream_t s) {
    const size_t lds = LIVE ? sizeof(int32_t) * (size_t)loop_lds_layout(tr, st, META == kMetaLds).total : 0;
    auto* k = &loop_kernel<DT, NC, META, LIVE, SMALL, MASK>;
    if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)st.B), dim3(kLoopBlock), lds, s, tr, st, io);
    return hipGetLastError();
  }
  static hipError_t run(const DevTrie& tr, const DevState& st, const LoopIO& io, int mode, hipStream_t s) {
    const bool small = st.path_stride <= kWave && st.k <= kWave && st.spent_words <= kWave;
    switch (mode) {
      case kLoopTrieMask:
        if (small && tr.emask) return go<kMetaLds, true, true, true>(tr, st, io, s);
        [[fallthrough]];
      case kLoopTrieLds:
        return small ? go<kMetaLds, true, true>(tr, st, io, s) : go<kMetaLds, true, false>(tr, st, io, s);
      case kLoopFastGlobal: return go<kMetaScalar, false, false>(tr, st, io, s);
      case kLoopVectorLds:
        return small ? go<kMetaVector, true, true>(tr, st, io, s) : go<kMetaVector, true, false>(tr, st, io, s);
      default: return go<kMetaVector, false, false>(tr, st, io, s);
    }
  }
};

template <int DT, int NC>
struct DenseLaunch {
  // grid 0: at most two groups of rows per wavefront, so that every
  // wavefront has the same number of groups or one fewer (with ~9.3 groups
  // each at 1024 workgroups, a quarter of them ran a tenth: the product
  // table's dense step took 109.8 us against 101.6 at two groups each)
  static hipError_t run(const DevState& st, const StepIO& io, float* full, int grid, hipStream_t s) {
    if (grid <= 0) {
      const int groups = (io.V + rows_per_pass(NC) - 1) / rows_per_pass(NC);
      grid = (groups + 2 * kWavesPerBlock - 1) / (2 * kWavesPerBlock);
    }
    hipLaunchKernelGGL((dense_head_kernel<DT, NC>), dim3(grid), dim3(kBlock), 0, s, st, io, full);
    return hipGetLastError();
  }
};

template <int DT, int NC>
struct GemvLaunch {
  static hipError_t run(const void* emb, int V, int H, const void* hidden, const int32_t* rows,
                        const int32_t* n_rows, int B, int cap, float* out, int split, hipStream_t s) {
    const int W = split * kWavesPerBlock;
    const int R = (cap + W - 1) / W;
    hipLaunchKernelGGL((gather_gemv_kernel<DT, NC>), dim3((unsigned)(B * split)), dim3(kBlock), 0, s,
                       (const uint4*)emb, V, H, (const uint4*)hidden, rows, n_rows, cap, out, split, R);
    return hipGetLastError();
  }
};

}  // namespace

int chunks_for(int dtype, int H) {
  const int el = dtype == 0 ? 4 : 8;
  if (H <= 0 || H % el) return 0;
  const int need = (H / el + kWave - 1) / kWave;
  for (int nc = 1; nc <= 16; nc *= 2)
    if (need <= nc) return nc;
  return 0;
}

hipError_t launch_reset(const DevTrie& tr, const DevState& st, int kind, hipStream_t s) {
  const int q4 = tr.live_stride / 4;
  int gx = (q4 + kBlock * 8 - 1) / (kBlock * 8);
  gx = kind != kResetFull || gx < 1 ? 1 : (gx > 256 ? 256 : gx);
  hipLaunchKernelGGL(reset_kernel, dim3(gx, st.B), dim3(kBlock), 0, s, tr, st, kind);
  return hipGetLastError();
}

hipError_t launch_step_sparse(const DevTrie& tr, const DevState& st, const StepIO& io, int dtype, bool fast,
                              int split, hipStream_t s, const StepGroup* grp) {
  return dispatch<StepLaunch>(dtype, chunks_for(dtype, io.H), tr, st, io, fast, split, grp, s);
}

size_t step_group_lds(int nq, int mt) { return sizeof(uint4) * (size_t)mt * nq + sizeof(int) * (size_t)mt; }

int step_group_rows(int dtype, int H) { return kWavesPerBlock * rows_per_pass(chunks_for(dtype, H)); }

hipError_t launch_loop(const DevTrie& tr, const DevState& st, const LoopIO& io, int dtype, int mode,
                       hipStream_t s) {
  return dispatch<LoopLaunch>(dtype, chunks_for(dtype, io.H), tr, st, io, mode, s);
}

constexpr int kRootMembers = 4;  // members per workgroup of the grouped root head

// The matrix-core root head takes bf16 tables with H = 2048 or 4096.
bool root_uses_mfma(int dtype, int H) { return dtype == 1 && (H == 2048 || H == 4096); }

int root_head_tiles(int dtype, int H, int root_edges) {
  const int rows_per_wg = root_uses_mfma(dtype, H) ? 16 : kWavesPerBlock * rows_per_pass(chunks_for(dtype, H));
  return (root_edges + rows_per_wg - 1) / rows_per_wg;
}

template <int KS>
hipError_t launch_root_mfma(const DevTrie& tr, const DevState& st, const LoopIO& io, int root_b0, int root_edges,
                            hipStream_t s) {
  const size_t lds = (sizeof(int64_t) + sizeof(int)) * (size_t)st.B;
  auto* k = &root_mfma_kernel<KS>;
  if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
  const int rt = (root_edges + 15) / 16, mtiles = (st.B + 15) / 16;
  hipLaunchKernelGGL(k, dim3((unsigned)root_tile_grid(rt, mtiles)), dim3(kBlock), lds, s, tr, st, io, root_b0,
                     root_b0 + root_edges, rt, mtiles);
  return hipGetLastError();
}

template <int DT, int NC>
struct RootLaunch {
  static hipError_t run(const DevTrie& tr, const DevState& st, const LoopIO& io, int root_edges, hipStream_t s) {
    constexpr int EL = DT == 0 ? 4 : 8;
    const int nq = io.H / EL;
    // members per workgroup: as many hidden vectors as fit 64 KiB of LDS, 1..16
    const int mt = max(1, min(kRootMembers, 65536 / (nq * 16)));
    const size_t lds = sizeof(uint4) * (size_t)mt * nq + (sizeof(int64_t) + sizeof(int)) * (size_t)st.B;
    auto* k = &root_head_kernel<DT, NC>;
    if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
    const int rows_per_wg = kWavesPerBlock * rows_per_pass(NC);
    const int rt = (root_edges + rows_per_wg - 1) / rows_per_wg, mtiles = (st.B + mt - 1) / mt;
    hipLaunchKernelGGL(k, dim3((unsigned)root_tile_grid(rt, mtiles)), dim3(kBlock), lds, s, tr, st, io, mt, rt,
                       mtiles);
    return hipGetLastError();
  }
};

hipError_t launch_root_head(const DevTrie& tr, const DevState& st, const LoopIO& io, int dtype, int root_b0,
                            int root_edges, hipStream_t s) {
  if (root_edges <= 0) return hipSuccess;
  if (root_uses_mfma(dtype, io.H))
    return io.H == 2048 ? launch_root_mfma<16>(tr, st, io, root_b0, root_edges, s)
                        : launch_root_mfma<32>(tr, st, io, root_b0, root_edges, s);
  return dispatch<RootLaunch>(dtype, chunks_for(dtype, io.H), tr, st, io, root_edges, s);
}

size_t loop_lds_bytes(const DevTrie& tr, const DevState& st, bool trie) {
  return sizeof(int32_t) * (size_t)loop_lds_layout(tr, st, trie).total;
}

template <int MAXT, int MT>
hipError_t launch_dense_mfma(const DevState& st, const StepIO& io, float* full, hipStream_t s) {
  const int ntiles = (st.B + 15) / 16;
  const size_t lds = sizeof(uint4) * (size_t)ntiles * 16 * kDenseStride;
  auto* k = &dense_mfma_kernel<MAXT, MT>;
  if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
  const int nblk = (io.V + 64 * MT - 1) / (64 * MT);
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(kBlock), lds, s, st, io, full, ntiles);
  return hipGetLastError();
}

template <int MAXT, int T>
hipError_t launch_dense_kstream(const DevState& st, const StepIO& io, float* full, hipStream_t s) {
  const int ntiles = (st.B + 15) / 16;
  const size_t lds = 2 * sizeof(uint4) * (size_t)ntiles * 16 * kDenseStride;  // double buffer
  auto* k = &dense_mfma_kstream_kernel<MAXT, T>;
  if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
  const int nblk = (io.V + 64 * T - 1) / (64 * T);
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(kBlock), lds, s, st, io, full, ntiles, nblk);
  return hipGetLastError();
}

template <int MAXT, int T, int KB, int NKB>
hipError_t launch_dense_kring(const DevState& st, const StepIO& io, float* full, hipStream_t s) {
  const int ntiles = (st.B + 15) / 16;
  const size_t lds = 2 * sizeof(uint4) * (size_t)MAXT * 16 * (KB / 8 + 1);  // double buffer
  auto* k = &dense_mfma_kring_kernel<MAXT, T, KB, NKB>;
  if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
  const int nblk = (io.V + 64 * T - 1) / (64 * T);
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(kBlock), lds, s, st, io, full, ntiles, nblk);
  return hipGetLastError();
}

template <int MAXT, int T, int KB, int R>
hipError_t launch_dense_wide(const DevState& st, const StepIO& io, float* full, hipStream_t s) {
  const size_t lds = 2 * sizeof(uint4) * (size_t)MAXT * 16 * (KB / 8 + 1);  // double buffer
  auto* k = &dense_mfma_wide_kernel<MAXT, T, KB, R>;
  if (hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
  const int nblk = (io.V + 64 * T - 1) / (64 * T);
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(kBlock), lds, s, st, io, full, nblk);
  return hipGetLastError();
}

bool dense_uses_mfma(int dtype, int B, int H) { return dtype == 1 && B >= 2 && B <= 256 && H % 32 == 0; }

hipError_t launch_dense_step(const DevTrie& tr, const DevState& st, const StepIO& io, int dtype, float* full,
                             int grid, bool mfma, hipStream_t s) {
  hipLaunchKernelGGL(dense_mask_kernel, dim3(st.B), dim3(kBlock), st.mask_words * sizeof(uint32_t), s, tr, st,
                     nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mfma && dense_uses_mfma(dtype, st.B, io.H)) {
    // one 16-row tile per wavefront keeps many workgroups (2374 at V = 151936)
    // for balance and latency hiding
    if (st.B <= 64 && io.H == 16 * kDenseKB)
      // loads two blocks ahead: 166 -> 136 us at B = 64, H = 2048 (V = 151936);
      // at H = 4096 the unrolled body needs more than 256 registers
      err = launch_dense_kring<4, 2, kDenseKB, 16>(st, io, full, s);
    else if (st.B > 64 && io.H % 256 == 0)
      // hidden slices 64 wide through registers, table fragments three blocks
      // ahead: 939 -> 545 us at B = 256, H = 4096; 319 -> 179 us at B = 128,
      // H = 2048 (two workgroups per compute unit fit at 8 member tiles)
      err = st.B <= 128 ? launch_dense_wide<8, 2, 64, 4>(st, io, full, s)
                        : launch_dense_wide<16, 2, 64, 4>(st, io, full, s);
    else if (io.H % kDenseKB == 0)
      // two row tiles per wavefront: measured best (1/2/3/4/8 swept at B = 64)
      err = st.B <= 64 ? launch_dense_kstream<4, 2>(st, io, full, s)
          : st.B <= 128 ? launch_dense_kstream<8, 2>(st, io, full, s)
                        : launch_dense_kstream<16, 2>(st, io, full, s);
    else
      err = st.B <= 64 ? launch_dense_mfma<4, 1>(st, io, full, s)
          : st.B <= 128 ? launch_dense_mfma<8, 1>(st, io, full, s)
                        : launch_dense_mfma<16, 1>(st, io, full, s);
  } else {
    err = dispatch<DenseLaunch>(dtype, chunks_for(dtype, io.H), st, io, full, grid, s);
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dense_advance_kernel, dim3(st.B), dim3(kWave), 0, s, tr, st, io);
  return hipGetLastError();
}

hipError_t launch_legal_mask(const DevTrie& tr, const DevState& st, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(dense_mask_kernel, dim3(st.B), dim3(kBlock), st.mask_words * sizeof(uint32_t), s, tr, st, out);
  return hipGetLastError();
}

hipError_t launch_mask_rows(const uint32_t* mask, int B, int V, int cap, int32_t* rows, int32_t* n_rows,
                            hipStream_t s) {
  const int W = (V + 31) / 32;
  hipLaunchKernelGGL(mask_rows_kernel, dim3((unsigned)B), dim3(kBlock), sizeof(uint32_t) * (size_t)W, s, mask, W, V,
                     cap, rows, n_rows);
  return hipGetLastError();
}

hipError_t launch_forced(const DevTrie& tr, const DevState& st, const int32_t* forced, hipStream_t s) {
  hipLaunchKernelGGL(forced_kernel, dim3(st.B), dim3(kWave), 0, s, tr, st, forced);
  return hipGetLastError();
}

hipError_t launch_legal_set(const DevTrie& tr, const DevState& st, int32_t* legal_tok, int32_t* n_legal,
                            hipStream_t s) {
  hipLaunchKernelGGL(legal_set_kernel, dim3(st.B), dim3(kWave), 0, s, tr, st, legal_tok, n_legal);
  return hipGetLastError();
}

hipError_t launch_gather_gemv(const void* emb, int dtype, int32_t V, int32_t H, const void* hidden,
                              const int32_t* rows, const int32_t* n_rows, int32_t B, int32_t cap, float* out,
                              int split, hipStream_t s) {
  return dispatch<GemvLaunch>(dtype, chunks_for(dtype, H), emb, V, H, hidden, rows, n_rows, B, cap, out, split,
                              s);
}

hipError_t launch_read_reference(const void* src, int64_t bytes, uint32_t* out, int grid, int unroll,
                                 hipStream_t s) {
  const int64_t n16 = bytes / 16;
  auto go = [&](auto k, int u) {
    int64_t g = grid > 0 ? grid : (n16 + (int64_t)kBlock * u - 1) / ((int64_t)kBlock * u);
    g = g < 1 ? 1 : (g > (1 << 20) ? (1 << 20) : g);
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(kBlock), 0, s, (const uint4*)src, n16, out);
    return hipGetLastError();
  };
  switch (unroll) {
    case 1: return go(read_ref_kernel<1>, 1);
    case 2: return go(read_ref_kernel<2>, 2);
    case 8: return go(read_ref_kernel<8>, 8);
    default: return go(read_ref_kernel<4>, 4);
  }
}

hipError_t launch_snapshot(const DevState& st, int parity, hipStream_t s) {
  hipLaunchKernelGGL(snapshot_kernel, dim3((st.B + kBlock - 1) / kBlock), dim3(kBlock), 0, s, st, parity);
  return hipGetLastError();
}

hipError_t launch_finalize(const DevState& st, int32_t* len, int32_t* entries, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3((st.B + kBlock - 1) / kBlock), dim3(kBlock), 0, s, st, len, entries);
  return hipGetLastError();
}

hipError_t launch_set_live(const DevTrie& tr, const DevState& st, int32_t seq, int32_t edge, int32_t value,
                           hipStream_t s) {
  hipLaunchKernelGGL(set_live_kernel, dim3(1), dim3(kWave), 0, s, tr, st, seq, edge, value);
  return hipGetLastError();
}

}  // namespace tms
