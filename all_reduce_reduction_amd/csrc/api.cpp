// api.cpp -- the C ABI of libsimar.so: argument validation, the library
// context (scratch, LL buffer, epoch, device error word), schedule-driven
// kernel launches and the selector.
//
// Validation mirrors the conditions under which the MSCCL runtime refuses
// to run a custom algorithm ("MSCCL, in depth ...", section "How the runtime
// decides to use your algorithm": op, collective, in-place-ness, rank
// count, divisibility, size window), except that a refusal here is an
// explicit error status and never a silent fallback to another schedule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.h"
#include "schedule.h"
#include "select.h"
#include "simar.h"

namespace simar {

int g_launch_device = 0;

namespace {

constexpr int kVersion = 1;
constexpr int64_t kMaxTiles = 1 << 20;  // cap on workgroups per transfer
// single-launch ring: FIFO geometry
constexpr int kFifoMaxChannels = 128;     // channels per rank
constexpr int kFifoMaxSlots = 8;          // slots per FIFO
// pointer table: distinct rank pointer sets kept in device memory
constexpr int kPtrSets = 512;
// single-launch ring: the LL protocol's default size limit (bytes per rank).
// Measured on MI355X (p = 8, bf16): the LL ring takes 13.7-14.9 us from
// 1 to 64 KiB per rank against 24-32 us for the FIFO protocol, 21.8 against
// 44.7 us at 128 KiB and 37.4 against 45.3 us at 256 KiB.
constexpr size_t kRingLLMaxBytes = 256 << 10;
// The phased one-shot (k_phased.hip) from this many bytes per rank on.
// Measured on MI355X, p = 8, against the fused one-shot (bf16; fp32):
// 12 MiB 36.2 against 35.3 us; 37.2 against 37.5, 16 MiB 44.5 against 46.3;
// 44.6 against 48.5, 32 MiB 84.7 against 94.1; 89.2 against 93.1, 64 MiB
// 174 against 201, 128 MiB 347 against 404.
constexpr size_t kPhasedMinBytes = 16 << 20;
// Polls before a phased one-shot barrier wait gives up.  A wait normally
// ends within the read half's tail (tens of polls); the barrier only orders
// traffic, so when something keeps the grid from being resident at once
// (another process's kernels) it is better to stop waiting early.
constexpr unsigned long long kPhasedSpinLimit = 1 << 13;

// A call's rank pointers as a hash key (p, then x[0..p), y[0..p)).
struct PtrKey {
  int p = 0;
  uintptr_t w[2 * SIM_MAX_RANKS] = {};
  bool operator==(const PtrKey& o) const {
    if (p != o.p) return false;
    for (int i = 0; i < 2 * p; i++)
      if (w[i] != o.w[i]) return false;
    return true;
  }
};
struct PtrKeyHash {
  size_t operator()(const PtrKey& k) const {
    uint64_t h = 0x9e3779b97f4a7c15ull ^ (uint64_t)k.p;
    for (int i = 0; i < 2 * k.p; i++) {
      h ^= (uint64_t)k.w[i] + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
    }
    return (size_t)h;
  }
};
// A table slot: written by an async copy, complete once `done` has fired
// (`ready` caches that).
struct PtrSlot {
  hipEvent_t done = nullptr;
  bool ready = false;
};

struct Ctx {
  bool init = false;
  int device = 0;
  int p_max = 0;
  int cu_count = 256;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  unsigned long long* ll = nullptr;
  int64_t ll_stride = 0;  // packets per rank
  int* err = nullptr;
  uint32_t epoch = 0;
  unsigned long long spin_limit = 1ull << 20;
  uint32_t wait_skew = 0;
  int log = 0;
  int force_wg = 0;
  int unroll = 0;  // forced vectors per lane (debug hook); 0: the launch table's, else 1
  int last_algo = -1;
  int env_algo = 0;
  int ll_occ[4][5] = {};
  uint32_t* fifo = nullptr;
  size_t fifo_bytes = 0;
  unsigned long long* fifo_sem = nullptr;
  uint32_t fifo_epoch = 0;
  int fifo_channels = 0;  // 0: heuristic
  int fifo_slots = 4;
  int fifo_withhold = 0;  // test hook: rank 0's workgroups leave at once
  int fifo_vecs = kFifoVecsPerLane;  // 16-byte vectors per lane per slot: 1, 2 or 4
  bool capturing = false;  // the current call's stream is being captured into a graph
  bool captured = false;   // some call has been captured since sim_init
  std::vector<void*> retired;  // outgrown scratch a captured graph may still use
  // pointer table (one-shot calls outside graph capture): slot i of `ptab`
  // holds a pointer set, copied from slot i of the pinned `ptab_host`; slots
  // are never rewritten or evicted, so no launch can see a slot change
  PtrSet* ptab = nullptr;
  PtrSet* ptab_host = nullptr;
  int ptab_used = 0;
  int ptab_on = 1;
  std::unordered_map<PtrKey, int, PtrKeyHash> ptab_index;
  std::vector<PtrSlot> ptab_slots;

  int fifo_occ[4][5] = {};
  int ring_ll_occ[4][5] = {};
  // the single-launch ring runs its LL protocol up to this many bytes per rank
  size_t ring_ll_max = kRingLLMaxBytes;
  int ap_occ[4][5][2] = {};  // persistent all-pairs: [dtype][op][p == 8]
  // phased kernels: barrier slots (per slot a counter, ph_gmax release
  // flags, then kPhasedGroups group counters, all kPhasedFlagStride words
  // apart), the count of barrier waits that gave up, and per slot the
  // counter, group counter and flag values the next call starts from
  unsigned long long* ph_mem = nullptr;
  int64_t ph_slot_words = 0;
  int ph_gmax = 0;
  unsigned int* ph_expired = nullptr;
  unsigned long long ph_ctr[kPhasedSlots] = {};
  unsigned long long ph_gctr[kPhasedSlots][kPhasedGroups] = {};
  unsigned long long ph_seq[kPhasedSlots] = {};
  unsigned ph_next = 0;
  int ph_occ[4][5][4][4] = {};  // [dtype][op][log2 p - 1][form]: resident workgroups per CU (-1: none)
  int phased_mode = 0;       // 0: from phased_min bytes per rank on, 1: always, 2: never
  size_t phased_min = kPhasedMinBytes;
  bool last_phased = false;  // the current (or last) call ran a phased fold
  bool last_whole = false;   // ... the phased one-shot in the whole-buffer layout
  int ph_layout = 0;         // 0: the one-shot's whole-buffer layout where it applies; 1: per chunk
  int ph_occ_whole[4][5][4] = {};  // that layout's kernel: workgroups per CU (0 = not asked yet, -1 = none)
  // the most recent phased launch with a barrier: its stream and sequence
  // number, and the pinned host word the workgroup that opens its last
  // barrier writes that number to
  unsigned long long* ph_host_done = nullptr;
  unsigned long long* ph_dev_done = nullptr;
  unsigned long long ph_launched = 0;
  hipStream_t ph_stream = nullptr;
  bool ph_any = false;
  Model model = default_model();
};

Ctx g;

int esize_of(int dtype) { return (dtype == SIM_FP16 || dtype == SIM_BF16) ? 2 : 4; }
const char* algo_name(int a) {
  static const char* n[] = {"auto",  "ring", "allpairs", "oneshot",    "oneshot_ll",         "ring_fifo",
                            "tree",  "rexch", "hier",    "hier_large", "allpairs_persistent"};
  return (a >= 0 && a < SIM_NUM_ALGOS) ? n[a] : "?";
}
constexpr int kLastAlgo = SIM_NUM_ALGOS - 1;
bool is_topology_algo(int a) { return a >= SIM_ALGO_TREE && a <= SIM_ALGO_HIER_LARGE; }

// The simulated topology of the tree / recursive-exchange / 2PH schedules:
// process-wide, kept across sim_init.
Topology g_topo;
// Workgroup budget of one launch (0: none); process-wide like the topology.
int g_max_wg = 0;

int64_t chunk_lo(int64_t n, int p, int c) { return (int64_t)(((__int128)c * n) / p); }

int hip_err(hipError_t e) { return e == hipSuccess ? SIM_OK : SIM_ERR_HIP; }

// Make the library's device current on the calling thread (only switches
// when another device is current: a per-call switch costs launch latency).
int use_device() {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SIM_ERR_HIP;
  if (cur != g.device && hipSetDevice(g.device) != hipSuccess) return SIM_ERR_HIP;
  return SIM_OK;
}

// ---- validation -------------------------------------------------------------
struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_scalars(int p, int dtype, int op, bool need_op) {
  if (!g.init) return SIM_ERR_NOT_INIT;
  if (p < 2 || p > g.p_max) return SIM_ERR_INVALID_ARG;
  if (dtype < SIM_INT32 || dtype > SIM_BF16) return SIM_ERR_INVALID_ARG;
  if (need_op && (op < SIM_SUM || op > SIM_AVG)) return SIM_ERR_INVALID_ARG;
  return SIM_OK;
}

// in-place iff out == in + inplace_off(r) for every rank (mixing is an error)
int check_buffers(const void* const* in, void* const* out, int p, size_t in_bytes, size_t out_bytes,
                  const size_t* inplace_off, bool* inplace) {
  if (!in || !out) return SIM_ERR_INVALID_ARG;
  int n_inplace = 0;
  for (int r = 0; r < p; r++) {
    if (!in[r] || !out[r]) return SIM_ERR_INVALID_ARG;
    if (((uintptr_t)in[r] | (uintptr_t)out[r]) & 15u) return SIM_ERR_ALIGN;
    if ((const char*)in[r] == (const char*)out[r] + (inplace_off ? inplace_off[r] : 0)) n_inplace++;
  }
  if (n_inplace != 0 && n_inplace != p) return SIM_ERR_INVALID_ARG;
  *inplace = (n_inplace == p);
  Range ins[SIM_MAX_RANKS], outs[SIM_MAX_RANKS];  // p <= SIM_MAX_RANKS (check_scalars)
  for (int r = 0; r < p; r++) {
    ins[r] = {(uintptr_t)in[r], (uintptr_t)in[r] + in_bytes};
    outs[r] = {(uintptr_t)out[r], (uintptr_t)out[r] + out_bytes};
  }
  for (int r = 0; r < p; r++) {
    for (int q = 0; q < p; q++) {
      if (q != r && overlap(outs[r], outs[q])) return SIM_ERR_ALIAS;
      if (*inplace) {
        if (q != r && overlap(outs[r], ins[q])) return SIM_ERR_ALIAS;
      } else if (overlap(outs[r], ins[q])) {
        return SIM_ERR_ALIAS;
      }
    }
  }
  return SIM_OK;
}

// ---- scratch ------------------------------------------------------------------
// Ring partial slots: [parity 0/1][rank] x (max chunk + 8) fp32/int32 values,
// each slot rounded to whole blocks of 512 values (the layout of 16-bit
// types' partials, see part_pos in device_common.h), so every slot also
// starts 2 KiB aligned.
size_t slot_elems(size_t n, int p) {
  const size_t e = (n + (size_t)p - 1) / (size_t)p + 8;
  return (e + 511) / 512 * 512;
}
size_t scratch_need(size_t n, int p) { return 2 * (size_t)p * slot_elems(n, p) * 4; }

// Grow the partial scratch.  Under stream capture it cannot grow (that would
// allocate, and the captured graph would keep the new address); once any
// call has been captured, an outgrown buffer is retired instead of freed,
// since a graph may still replay kernels that use it (all are freed by
// sim_finalize).
int ensure_scratch(size_t bytes) {
  if (bytes <= g.scratch_bytes) return SIM_OK;
  if (g.capturing) return SIM_ERR_UNSUPPORTED;
  if (g.scratch) {
    if (g.captured) {
      g.retired.push_back(g.scratch);
    } else {
      if (hipDeviceSynchronize() != hipSuccess) return SIM_ERR_HIP;
      if (hipFree(g.scratch) != hipSuccess) return SIM_ERR_HIP;
    }
    g.scratch = nullptr;
    g.scratch_bytes = 0;
  }
  if (hipMalloc(&g.scratch, bytes) != hipSuccess) {
    g.scratch = nullptr;
    (void)hipGetLastError();
    return SIM_ERR_NOMEM;
  }
  g.scratch_bytes = bytes;
  return SIM_OK;
}

float inv_p_of(int p) {
  volatile float one = 1.0f, fp = (float)p;
  return one / fp;
}

// ---- launch glue ----------------------------------------------------------------
struct Call {
  int coll, p, dtype, op, algo;
  size_t n;            // elements per rank (AR: buffer; RS: input; AG: output)
  const void* const* x;
  void* const* y;
  bool inplace;
  hipStream_t s;
  // allocation-free calls: partial slots in this fixed array (checked to be
  // large enough before anything is enqueued), no pointer-table entry
  void* fixed_scratch = nullptr;
  bool noalloc = false;
};

// Workgroups per transfer (gridDim.x) of a bulk kernel; every bulk kernel
// walks its transfer with a grid-stride loop, so any count >= 1 is correct.
// Measured on MI355X: streaming kernels run fastest with one short-lived
// workgroup per kBlock * unroll vectors (many waves in flight), so the
// default covers the transfer exactly.  The calibration's launch table, when
// it has an entry for this algo and was measured at this call's rank count,
// replaces that with the measured best total for the nearest message size
// (at p = 8 the one-shot's 2p streams per workgroup keep enough bytes in
// flight with far fewer workgroups than at p = 2); SIM_CONFIG_MAX_WORKGROUPS caps the total
// (T-CCL's restricted mode: communication given a fixed slice of the GPU);
// SIM_DEBUG_WORKGROUPS forces a total.
// 16-byte vectors per lane per pass of a bulk kernel: forced by the debug
// hook, else the calibration's launch table entry for this call, else 1.
// 16-byte vectors per lane per pass of a bulk kernel: SIM_DEBUG_UNROLL, else
// the launch table's entry, else 1; at most max_u (the kernel's largest form)
int unroll_for(const Call& c, int max_u = 2) {
  int u = g.unroll > 0 ? g.unroll : model_launch(g.model, c.algo, c.p, (double)c.n * esize_of(c.dtype)).unroll;
  if (u < 1) u = 1;
  return u < max_u ? u : max_u;
}

int tiles_for(const Call& c, int64_t vecs_per_unit, int units, int unroll) {
  int64_t t;
  if (g.force_wg > 0) {
    t = g.force_wg / units;
  } else {
    t = (vecs_per_unit + (int64_t)kBlock * unroll - 1) / ((int64_t)kBlock * unroll);
    const int total = model_workgroups(g.model, c.algo, c.p, (double)c.n * esize_of(c.dtype));
    if (total > 0) t = std::min<int64_t>(t, std::max(1, total / units));
  }
  if (g_max_wg > 0) t = std::min<int64_t>(t, g_max_wg / units);
  return (int)std::max<int64_t>(1, std::min<int64_t>(t, kMaxTiles));
}

// The device copy of the call's rank pointers, or nullptr when this call
// must carry them in its kernel arguments: under graph capture (a replay
// pays no launch cost, and a captured kernel keeps no reference into the
// table), when the table is full or off, or while the set's copy may still
// be in flight.  A new set is copied on the call's stream, so the launch
// that follows it is ordered after the copy; any later call uses the entry
// only once the copy's event has completed (a later call may come on
// another stream, or on a new stream that reuses the handle).
const PtrSet* ptr_set_for(const Call& c) {
  if (c.noalloc || !g.ptab_on || !g.ptab || g.capturing || c.p > SIM_MAX_RANKS) return nullptr;
  PtrKey k;
  k.p = c.p;
  for (int q = 0; q < c.p; q++) {
    k.w[q] = (uintptr_t)c.x[q];
    k.w[c.p + q] = (uintptr_t)c.y[q];
  }
  auto it = g.ptab_index.find(k);
  if (it != g.ptab_index.end()) {
    PtrSlot& sl = g.ptab_slots[it->second];
    if (!sl.ready) {
      if (hipEventQuery(sl.done) == hipSuccess) sl.ready = true;
      else (void)hipGetLastError();  // not yet complete: clear the query's status
    }
    return sl.ready ? g.ptab + it->second : nullptr;
  }
  if (g.ptab_used >= kPtrSets) return nullptr;
  // the slot is taken even if a call below fails: its staging entry may be
  // in use by a copy and is never written again
  const int i = g.ptab_used++;
  PtrSet& h = g.ptab_host[i];
  std::memset(&h, 0, sizeof h);
  for (int q = 0; q < c.p; q++) {
    h.x[q] = c.x[q];
    h.y[q] = c.y[q];
  }
  PtrSlot& sl = g.ptab_slots[i];
  if (hipEventCreateWithFlags(&sl.done, hipEventDisableTiming) != hipSuccess) {
    sl.done = nullptr;
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipMemcpyAsync(g.ptab + i, &h, sizeof h, hipMemcpyHostToDevice, c.s) != hipSuccess ||
      hipEventRecord(sl.done, c.s) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  g.ptab_index.emplace(k, i);
  return g.ptab + i;
}

// set: the call's entry in the pointer table, or nullptr.  With an entry the
// launch carries a 32-byte argument block; that form computes the standard
// chunk bounds itself and writes outputs unshifted, so it serves the
// one-shot and all-pairs step 1 of an all-reduce (not the reduce-scatter).
int run_fold(const Call& c, bool all_out, const int64_t* lo, const int64_t* out_shift,
             const PtrSet* set) {
  FoldArgs a;
  std::memset(&a, 0, sizeof a);
  const int V = 16 / esize_of(c.dtype);
  int64_t maxchunk = 0;
  for (int q = 0; q < c.p; q++) {
    a.x[q] = c.x[q];
    a.y[q] = c.y[q];
    a.out_shift[q] = out_shift ? out_shift[q] : 0;
    if (a.out_shift[q] % V == 0) a.vec_ok |= 1u << q;
    maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
  }
  for (int q = 0; q <= c.p; q++) a.lo[q] = lo[q];
  a.p = c.p;
  a.inv_p = inv_p_of(c.p);
  // The fold forms for p = 2, 4 and 8 have 2- and 4-vector forms.  Under a
  // workgroup budget below the CU count every workgroup has a CU to itself
  // and the fold runs at the bytes each one keeps in flight, so it takes 4
  // vectors per lane when the budget binds even at 4 (every budgeted
  // workgroup still gets a whole span); on smaller messages, which a budget
  // does not cap, the table's choice keeps the workgroup count up.  MI355X,
  // p = 8 bf16 one-shot, 1 / 2 / 4 vectors: 64 MiB per rank under 32
  // workgroups 691 / 810 / 608 us, under 128 234 / 270 / 213 us; 4 MiB under
  // 128 16.9 / 19.3 / 14.8 us; at a budget of 256 the three are within 6%.
  int unroll = 1;
  if (c.p == 2 || c.p == 4 || c.p == 8) {
    unroll = unroll_for(c, 4);
    const int64_t span4 = (int64_t)kBlock * 4, vecs = (maxchunk + V - 1) / V;
    if (g.unroll == 0 && g_max_wg > 0 && g_max_wg < g.cu_count &&
        (vecs + span4 - 1) / span4 >= std::max<int64_t>(1, g_max_wg / c.p))
      unroll = 4;
  }
  a.tiles = tiles_for(c, (maxchunk + V - 1) / V, c.p, unroll);
  if (set && out_shift == nullptr) {
    FoldTabArgs t;
    std::memset(&t, 0, sizeof t);
    t.set = set;
    t.n = (int64_t)c.n;
    t.p = c.p;
    t.tiles = a.tiles;
    t.inv_p = a.inv_p;
    return hip_err(launch_fold_tab(c.dtype, c.op, c.p, all_out, t, unroll, c.s));
  }
  return hip_err(launch_fold(c.dtype, c.op, c.p, all_out, a, unroll, c.s));
}

// The phased kernels, when this call may use one: the fold writing every
// output (kPhasedAll: the one-shot) or the owner's (kPhasedOwner: all-pairs
// step 1; the direct reduce-scatter, whose owner writes element i at i -
// out_shift[j]), or the direct all-gather's copy (kPhasedGather: output
// block j from rank j's input); p = 2, 4, 8 or 16, no workgroup budget, not
// under graph capture (the barrier counts are fixed at enqueue time) and
// not the allocation-free entry point; by default from phased_min bytes per
// rank on (of the input for the fold, of the output for the gather).
// Returns SIM_OK after enqueueing it, a negative value when the call should
// take the fused kernel instead, or an error.
// kPhasedFanout: all-pairs step 2, owner j's finished chunk from output j to
// the other outputs, with the gather's kernel.
enum PhasedForm { kPhasedAll = 0, kPhasedOwner = 1, kPhasedGather = 2, kPhasedFanout = 3 };
// Bytes per rank from which a call of a phased form runs phased (0: never),
// given the rank count, the switch (SIM_DEBUG_PHASED) and the workgroup
// budget (the persistent grid needs every CU).
size_t phased_threshold(int form, int p) {
  // Where the phased form pays, in units of the settable threshold
  // (g.phased_min, 16 MiB by default), by form (one-shot, owner-only fold,
  // copy) and rank count; 0 = never by default.  The owner-only fold writes
  // S bytes, not p S, and the copy reads only S / p, so their phase
  // separation gains less against the barriers' cost, and the copy's last
  // phase, not dealt out evenly (k_phased_gather.hip), leaves workgroups
  // idle.  At p = 2 the fused one-shot already runs at ~0.75 of peak.
  // Measured on MI355X, bf16, phased / fused (us):
  //   p = 2: one-shot 32 MiB 22.7 / 24.8, 64 MiB 42.7 / 43.4, 96 MiB
  //          68.5 / 65.7; reduce-scatter (input per rank) 24 MiB 13.1 / 12.5,
  //          32 MiB 17.0 / 18.1; all-gather (output per rank) 12 MiB
  //          10.5 / 9.7, 16 MiB 11.9 / 12.5
  //   p = 4: one-shot 12 MiB 18.7 / 17.8, 16 MiB 24.0 / 28.0; reduce-scatter
  //          24 MiB 21.4 / 19.8, 32 MiB 28.9 / 32.3; all-gather 16 MiB
  //          17.4 / 17.3, 48 MiB 46.1 / 44.5, 64 MiB 66.0 / 65.1
  //   p = 8: one-shot 8 MiB 24.9 / 23.1, 12 MiB 35.2 / 37.7; reduce-scatter
  //          16 MiB 23.8 / 22.5, 24 MiB 35.4 / 36.4; all-gather 16 MiB
  //          29.2 / 28.4, 24 MiB 42.4 / 45.0 (fp32 within 3% of bf16)
  //   p = 16: one-shot 8 MiB 48.4 / 49.5; reduce-scatter 8 MiB 24.4 / 24.3,
  //          12 MiB 34.5 / 35.7; all-gather 8 MiB 29.3 / 29.6, 12 MiB
  //          42.3 / 45.4
  static const double kFrom[3][4] = {
      // p = 2, 4, 8, 16
      {0.0, 1.0, 0.75, 0.5},   // one-shot
      {2.0, 2.0, 1.5, 0.75},   // owner-only fold (direct reduce-scatter, all-pairs step 1)
      {1.0, 0.0, 1.5, 0.75},   // copy (direct all-gather, all-pairs step 2)
  };
  if (g.phased_mode == 2 || g_max_wg > 0 || (p != 2 && p != 4 && p != 8 && p != 16)) return 0;
  if (g.phased_mode == 1) return 1;
  const int pi = p == 2 ? 0 : p == 4 ? 1 : p == 8 ? 2 : 3;
  const double from = kFrom[form == kPhasedAll ? 0 : form == kPhasedOwner ? 1 : 2][pi];
  return from == 0.0 ? 0 : std::max<size_t>(1, (size_t)(from * (double)g.phased_min));
}

int run_phased(const Call& c, const int64_t* lo, PhasedForm form, const int64_t* out_shift) {
  const int p = c.p;
  const bool all_out = form != kPhasedOwner;
  const bool copy = form == kPhasedGather || form == kPhasedFanout;
  if (!g.ph_mem || !g.ph_dev_done || c.noalloc || g.capturing || g_max_wg > 0 || g.phased_mode == 2) return -1;
  if (p != 2 && p != 4 && p != 8 && p != 16) return -1;
  const int E = esize_of(c.dtype);
  const size_t min_bytes = phased_threshold(form, p);
  if (min_bytes == 0) return -1;
  if (c.n * (size_t)E < min_bytes) return -1;
  // owner-only with shifted outputs, and the gather's inputs: whole 16-byte
  // vectors need 16-byte aligned offsets on both sides
  if (out_shift)
    for (int q = 0; q < p; q++)
      if (out_shift[q] % (16 / E) != 0) return -1;
  if (form == kPhasedGather)
    for (int q = 0; q < p; q++)
      if (lo[q] % (16 / E) != 0) return -1;
  // Two phased kernels in flight at once could each hold part of the CUs
  // while waiting at a barrier for workgroups the other keeps from being
  // resident (until their waits give up).  Calls on one stream are ordered;
  // a call on another stream takes the fused kernel until the last phased
  // launch has opened its last barrier (after which none of its workgroups
  // waits for anything, so its CUs drain on their own).
  if (g.ph_any && c.s != g.ph_stream &&
      __atomic_load_n(g.ph_host_done, __ATOMIC_ACQUIRE) != g.ph_launched)
    return -1;
  const int pi = p == 2 ? 0 : p == 4 ? 1 : p == 8 ? 2 : 3;
  int& occ = g.ph_occ[c.dtype][copy ? 0 : c.op][pi][form];
  if (occ == 0) {
    occ = copy ? gather_phased_blocks_per_cu(E, p, form == kPhasedFanout)
               : fold_phased_blocks_per_cu(c.dtype, c.op, p, all_out);
    if (occ < 1) occ = -1;
  }
  if (occ < 1) return -1;
  // every workgroup resident at once: at most two per CU (the VGPR budget
  // of a phase's results), fewer if the kernel fits fewer
  int64_t G = (int64_t)std::min(occ, 2) * g.cu_count;
  if (g.force_wg > 0) G = std::min<int64_t>(G, g.force_wg);
  G = std::min<int64_t>(G, g.ph_gmax);
  const int64_t tiles = std::max<int64_t>(1, G / p);
  G = tiles * p;
  if (G > g.ph_gmax) return -1;
  // The fold takes every whole block (kBlock 16-byte vectors) of the
  // largest chunk in phases of tiles * K blocks, the last one dealt out
  // evenly; the copy takes every whole span (K blocks) in phases of tiles
  // spans.  What is past them is done after the phases.
  const int V = 16 / E;
  const int64_t K = fold_phased_vecs_per_lane(p);
  int64_t nmax = 0;  // whole blocks (fold) or spans (copy) of the largest chunk
  for (int q = 0; q < p; q++) {
    int64_t head = (V - lo[q] % V) % V;
    head = std::min(head, lo[q + 1] - lo[q]);
    const int64_t nvec = (lo[q + 1] - lo[q] - head) / V;
    nmax = std::max(nmax, nvec / (copy ? kBlock * K : kBlock));
  }
  const int64_t per_phase = copy ? tiles : tiles * K;
  int64_t nphase = (nmax + per_phase - 1) / per_phase;
  // The one-shot's whole-buffer layout (phased_impl.h): when every chunk is
  // the same whole number of blocks, and no fewer blocks than the grid has
  // workgroups, the grid's workgroups take the whole buffer's blocks in
  // turn, G blocks per step, instead of each chunk's in turn.  (The same
  // layout for the direct all-gather's copy measured 1-7% slower on
  // MI355X, so that keeps its per-chunk layout.)
  const int64_t bel = (int64_t)kBlock * V;  // elements per block
  const int64_t n = lo[p];
  bool whole = form == kPhasedAll && g.ph_layout == 0 && lo[0] == 0 && n % (p * bel) == 0 &&
               n / (p * bel) >= G;
  for (int q = 1; whole && q < p; q++) whole = lo[q] == q * (n / p);
  if (whole) {  // its kernel must fit the same grid, all resident
    int& wocc = g.ph_occ_whole[c.dtype][c.op][pi];
    if (wocc == 0) {
      wocc = fold_phased_blocks_per_cu(c.dtype, c.op, p, true, true);
      if (wocc < 1) wocc = -1;
    }
    whole = wocc >= std::min(occ, 2);
  }
  if (whole) nphase = (n / bel + G * K - 1) / (G * K);
  const int64_t nbar = nphase > 0 ? 2 * nphase - 1 : 0;
  PhasedArgs a;
  std::memset(&a, 0, sizeof a);
  if (whole) {
    a.gblk = n / bel;
    a.gbpc = n / (p * bel);
  }
  for (int q = 0; q < p; q++) {
    // the fan-out's block q comes from output q itself (the kernel indexes
    // its source as x[q] - lo[q] by output element)
    a.x[q] = form == kPhasedFanout ? (const void*)((const char*)c.y[q] + lo[q] * E) : c.x[q];
    a.y[q] = c.y[q];
  }
  for (int q = 0; q <= p; q++) a.lo[q] = lo[q];
  if (out_shift)
    for (int q = 0; q < p; q++) a.out_shift[q] = out_shift[q];
  const unsigned slot = g.ph_next++ % kPhasedSlots;
  a.ctr = g.ph_mem + (int64_t)slot * g.ph_slot_words;
  a.flags = a.ctr + kPhasedFlagStride;
  a.gctr = a.flags + (int64_t)g.ph_gmax * kPhasedFlagStride;
  for (int q = 0; q < kPhasedGroups; q++) a.gbase[q] = g.ph_gctr[slot][q];
  a.base = g.ph_ctr[slot];
  a.seq = g.ph_seq[slot];
  a.spin_limit = std::min(g.spin_limit, kPhasedSpinLimit);
  a.expired = g.ph_expired;
  a.done = g.ph_dev_done;
  a.done_seq = g.ph_launched + 1;
  a.tiles = (int)tiles;
  a.nphase = (int)nphase;
  a.inv_p = inv_p_of(p);
  const int rc = hip_err(copy ? launch_gather_phased(E, p, form == kPhasedFanout, a, c.s)
                              : launch_fold_phased(c.dtype, c.op, p, all_out, a, c.s));
  if (rc) return rc;

  // the counts this call adds: every workgroup meets every barrier at its
  // group's counter (workgroup b in group b mod NG), every group completes
  // its share of every barrier once at the slot's counter.  A launch
  // without barriers (no whole block to phase) never waits, so it does not
  // hold up calls on other streams.
  const int64_t NG = std::min<int64_t>(G, kPhasedGroups);
  for (int64_t q = 0; q < NG; q++)
    g.ph_gctr[slot][q] += (unsigned long long)nbar * (unsigned long long)(G / NG + (q < G % NG ? 1 : 0));
  g.ph_ctr[slot] += (unsigned long long)nbar * (unsigned long long)NG;
  g.ph_seq[slot] += (unsigned long long)nbar;
  if (nbar > 0) {
    g.ph_launched = a.done_seq;
    g.ph_stream = c.s;
    g.ph_any = true;
  }
  g.last_phased = true;
  g.last_whole = whole;
  return SIM_OK;
}

int run_copy_step(const Call& c, const CopyXfer* xs, int count) {
  CopyArgs a;
  std::memset(&a, 0, sizeof a);
  const int e = esize_of(c.dtype), V = 16 / e;
  int64_t maxlen = 0;
  a.nx = count;
  for (int k = 0; k < count; k++) {
    a.x[k] = xs[k];
    a.x[k].vec_ok = (xs[k].src_shift % V == 0) && (xs[k].dst_shift % V == 0);
    maxlen = std::max(maxlen, xs[k].hi - xs[k].lo);
  }
  if (a.nx == 0) return SIM_OK;
  const int unroll = unroll_for(c);
  a.tiles = tiles_for(c, (maxlen + V - 1) / V, a.nx, unroll);
  return hip_err(launch_copy(e, a, unroll, c.s));
}

// Ring reduce-scatter half.  final_out_chunk: outputs are chunk-sized (RS).
int run_ring_rs(const Call& c, const Schedule& sch, int nsteps, bool final_out_chunk,
                const int64_t* lo) {
  const int p = c.p, e = esize_of(c.dtype), V = 16 / e;
  // 32-bit all-reduce keeps partials in the receiving rank's output (a chunk
  // it does not own yet); otherwise partials live in fp32/int32 scratch slots.
  const bool part_in_y = (e == 4) && !final_out_chunk;
  const size_t se = slot_elems(c.n, p);
  if (!part_in_y && p > 2 && !c.fixed_scratch) {
    int rc = ensure_scratch(scratch_need(c.n, p));
    if (rc) return rc;
  }
  char* const base = (char*)(c.fixed_scratch ? c.fixed_scratch : g.scratch);
  auto slot = [&](int parity, int rank) -> void* { return base + ((size_t)parity * p + rank) * se * 4; };
  int64_t maxchunk = 0;
  for (int q = 0; q < p; q++) maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
  for (int st = 0; st < nsteps; st++) {
    RingArgs a;
    std::memset(&a, 0, sizeof a);
    a.nx = (int)sch.steps[st].size();
    a.p = p;
    a.inv_p = inv_p_of(p);
    const bool first = (st == 0), last = (st == nsteps - 1);
    for (int k = 0; k < a.nx; k++) {
      const Xfer& xf = sch.steps[st][k];
      RingXfer& x = a.x[k];
      const int64_t l = lo[xf.chunk], h = lo[xf.chunk + 1];
      const int64_t slot_shift = l - (l % 8);
      x.lo = l;
      x.hi = h;
      if (first) {
        x.a = c.x[xf.src];
        x.a_shift = 0;
      } else if (part_in_y) {
        x.a = c.y[xf.src];
        x.a_shift = 0;
      } else {
        x.a = slot((st - 1) & 1, xf.src);
        x.a_shift = slot_shift;
      }
      x.b = c.x[xf.dst];
      if (last) {
        x.d = c.y[xf.dst];
        x.d_shift = final_out_chunk ? l : 0;
      } else if (part_in_y) {
        x.d = c.y[xf.dst];
        x.d_shift = 0;
      } else {
        x.d = slot(st & 1, xf.dst);
        x.d_shift = slot_shift;
      }
      x.vec_ok = (x.a_shift % V == 0) && (x.d_shift % V == 0);
    }
    const int unroll = unroll_for(c);
    a.tiles = tiles_for(c, (maxchunk + V - 1) / V, a.nx, unroll);
    int rc = hip_err(launch_ring_reduce(c.dtype, c.op, !first, last, a, unroll, c.s));
    if (rc) return rc;
  }
  return SIM_OK;
}

// The all-reduce ring from the pointer table: each of the 2(p-1) steps
// launches with a 48-byte argument block and derives its transfers from the
// step number, exactly as the ring's lowering lists them (the schedule
// verifier proves that list); partials as in run_ring_rs.
int run_ring_tab(const Call& c, const PtrSet* set, const int64_t* lo) {
  const int p = c.p, e = esize_of(c.dtype), V = 16 / e;
  const bool part_in_y = (e == 4);
  const size_t se = slot_elems(c.n, p);
  if (!part_in_y && p > 2) {
    int rc = ensure_scratch(scratch_need(c.n, p));
    if (rc) return rc;
  }
  int64_t maxchunk = 0;
  for (int q = 0; q < p; q++) maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
  const int unroll = unroll_for(c);
  RingTabArgs a;
  std::memset(&a, 0, sizeof a);
  a.set = set;
  a.scratch = (part_in_y || p == 2) ? nullptr : g.scratch;
  a.n = (int64_t)c.n;
  a.slot_elems = (int64_t)se;
  a.p = p;
  a.tiles = tiles_for(c, (maxchunk + V - 1) / V, p, unroll);
  a.inv_p = inv_p_of(p);
  for (int st = 0; st < p - 1; st++) {  // reduce-scatter
    a.step = st;
    int rc = hip_err(launch_ring_reduce_tab(c.dtype, c.op, st > 0, st == p - 2, a, unroll, c.s));
    if (rc) return rc;
  }
  for (int st = 0; st < p - 1; st++) {  // all-gather
    a.step = st;
    int rc = hip_err(launch_ring_copy_tab(e, a, unroll, c.s));
    if (rc) return rc;
  }
  return SIM_OK;
}

// The epoch of a call of a persistent kernel (the single-launch ring and
// all-pairs share the semaphore array and this one monotonic count, so a
// counter value left by any earlier call compares lower than anything the
// new call waits for).  On wrap every counter is cleared first.
int next_sem_epoch(const Call& c, uint32_t* epoch) {
  uint32_t e = g.fifo_epoch + 1;
  if (e == 0) {
    int rc = hip_err(launch_fill64(g.fifo_sem, 0ull, (int64_t)g.p_max * kFifoMaxChannels * 2, c.s));
    if (rc) return rc;
    e = 1;
  }
  g.fifo_epoch = e;
  *epoch = e;
  return SIM_OK;
}

// The epoch of a call that sends LL packets (the LL one-shot and the
// single-launch ring's LL protocol share the packet buffer and this count,
// so a packet left by any earlier call never carries a flag a new call
// accepts).  On wrap the buffer is cleared first.
int next_ll_epoch(const Call& c, uint32_t* epoch) {
  uint32_t e = g.epoch + 1;
  if (e == 0) {
    int rc = hip_err(launch_fill64(g.ll, 0ull, (int64_t)g.p_max * g.ll_stride, c.s));
    if (rc) return rc;
    e = 1;
  }
  g.epoch = e;
  *epoch = e;
  return SIM_OK;
}

// The whole ring in one launch with LL packets (k_ring_ll): p * C
// persistent workgroups, all co-resident; every hop is one polled packet.
int run_ring_ll(const Call& c, const int64_t* lo, int64_t maxchunk) {
  const int p = c.p;
  RingLLArgs a;
  std::memset(&a, 0, sizeof a);
  for (int q = 0; q < p; q++) {
    a.x[q] = c.x[q];
    a.y[q] = c.y[q];
  }
  for (int q = 0; q <= p; q++) a.lo[q] = lo[q];
  int& occ = g.ring_ll_occ[c.dtype][c.op];
  if (occ == 0) occ = ring_ll_blocks_per_cu(c.dtype, c.op);
  const int64_t resident = (int64_t)occ * g.cu_count;  // every workgroup must be resident at once
  // one element per thread and step while the slices allow it, at most 16 channels
  int64_t C = g.fifo_channels > 0 ? g.fifo_channels : (maxchunk + kBlock - 1) / kBlock;
  C = std::max<int64_t>(1, std::min<int64_t>(C, 16));
  C = std::min<int64_t>(C, std::max<int64_t>(1, resident / p));
  if (g_max_wg > 0) C = std::min<int64_t>(C, std::max(1, g_max_wg / p));  // at least one per rank
  int64_t Cg = (C + 7) / 8 * 8;  // rank-major grid padded to whole rounds of the 8 XCDs
  if ((int64_t)p * Cg > resident || g_max_wg > 0) Cg = C;
  uint32_t epoch = 0;
  int rc = next_ll_epoch(c, &epoch);
  if (rc) return rc;
  a.ll = g.ll;
  a.ll_stride = g.ll_stride;
  a.maxchunk = maxchunk;
  a.spin_limit = g.spin_limit;
  a.err = g.err;
  a.p = p;
  a.C = (int)C;
  a.Cg = (int)Cg;
  a.epoch = epoch;
  a.wait_epoch = epoch + g.wait_skew;
  a.inv_p = inv_p_of(p);
  a.withhold = g.fifo_withhold;
  return hip_err(launch_ring_ll(c.dtype, c.op, a, c.s));
}

// The two all-pairs steps in one launch (k_allpairs_persistent): p * C
// persistent workgroups, all co-resident; channel c of every rank handles
// the same slice of each chunk.
int run_allpairs_persistent(const Call& c, const int64_t* lo) {
  const int p = c.p;
  const int V = 16 / esize_of(c.dtype);
  AllPairsPArgs a;
  std::memset(&a, 0, sizeof a);
  int64_t maxchunk = 0;
  for (int q = 0; q < p; q++) {
    a.x[q] = c.x[q];
    a.y[q] = c.y[q];
    maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
  }
  for (int q = 0; q <= p; q++) a.lo[q] = lo[q];
  int& occ = g.ap_occ[c.dtype][c.op][p == 8 ? 1 : 0];
  if (occ == 0) occ = allpairs_persistent_blocks_per_cu(c.dtype, c.op, p);
  const int64_t resident = (int64_t)occ * g.cu_count;  // every workgroup must be resident at once
  // one pass (kAllPairsPVecsPerLane vectors per lane) per slice, but at
  // least 8 channels while a slice still holds a vector per lane: small
  // messages want the parallelism (measured on MI355X: 256 KiB per rank
  // 9.3 -> 8.2 us; one vector per lane everywhere cost 4 MiB 12%)
  const int64_t lane_elems = (int64_t)kBlock * V;
  const int64_t span = lane_elems * kAllPairsPVecsPerLane;
  int64_t C = std::max((maxchunk + span - 1) / span, std::min<int64_t>(8, (maxchunk + lane_elems - 1) / lane_elems));
  if (g.fifo_channels > 0) C = g.fifo_channels;
  C = std::max<int64_t>(C, 1);
  C = std::min<int64_t>(C, kFifoMaxChannels);
  C = std::min<int64_t>(C, std::max<int64_t>(1, resident / p));
  if (g_max_wg > 0) C = std::min<int64_t>(C, std::max(1, g_max_wg / p));  // at least one per rank
  int64_t Cg = (C + 7) / 8 * 8;  // rank-major grid padded to whole rounds of the 8 XCDs
  if ((int64_t)p * Cg > resident || g_max_wg > 0) Cg = C;
  uint32_t epoch = 0;
  int rc = next_sem_epoch(c, &epoch);
  if (rc) return rc;
  a.sem = g.fifo_sem;
  a.err = g.err;
  a.spin_limit = g.spin_limit;
  a.p = p;
  a.C = (int)C;
  a.Cg = (int)Cg;
  a.epoch = epoch;
  a.inv_p = inv_p_of(p);
  a.withhold = g.fifo_withhold;
  return hip_err(launch_allpairs_persistent(c.dtype, c.op, a, c.s));
}

// The whole ring in one launch (k_ring_fifo): p * C persistent workgroups,
// all co-resident, exchanging partials through bounded FIFOs.
int run_ring_fifo(const Call& c, const int64_t* lo) {
  const int p = c.p;
  {  // small messages: the LL protocol, when its packets fit the LL buffer
    int64_t maxchunk = 0;
    for (int q = 0; q < p; q++) maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
    if (c.n * (size_t)esize_of(c.dtype) <= g.ring_ll_max && (int64_t)(2 * p - 2) * maxchunk <= g.ll_stride)
      return run_ring_ll(c, lo, maxchunk);
  }
  const int V = 16 / esize_of(c.dtype);
  const int slot = kBlock * g.fifo_vecs * V;
  RingFifoArgs a;
  std::memset(&a, 0, sizeof a);
  int64_t maxchunk = 0;
  for (int q = 0; q < p; q++) {
    a.x[q] = c.x[q];
    a.y[q] = c.y[q];
    maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
  }
  for (int q = 0; q <= p; q++) a.lo[q] = lo[q];
  int& occ = g.fifo_occ[c.dtype][c.op];
  if (occ == 0) occ = ring_fifo_blocks_per_cu(c.dtype, c.op);
  const int64_t resident = (int64_t)occ * g.cu_count;  // every workgroup must be resident at once
  int64_t C = g.fifo_channels > 0 ? g.fifo_channels : std::max<int64_t>(1, (maxchunk + slot - 1) / slot);
  C = std::min<int64_t>(C, kFifoMaxChannels);
  C = std::min<int64_t>(C, std::max<int64_t>(1, resident / p));
  if (g_max_wg > 0) C = std::min<int64_t>(C, std::max(1, g_max_wg / p));  // at least one per rank
  // rank-major grid padded to whole rounds of the 8 XCDs (when the padded
  // grid still fits at once): the ranks of a channel run on one XCD
  int64_t Cg = (C + 7) / 8 * 8;
  if ((int64_t)p * Cg > resident || g_max_wg > 0) Cg = C;  // no padding under a budget
  // slots per channel slice: the longest slice over all chunks (same formula as the kernel)
  int64_t maxslice = 0;
  for (int q = 0; q < p; q++) {
    const int64_t clen = lo[q + 1] - lo[q];
    for (int64_t ch = 0; ch < C; ch++) {
      const int64_t s_lo = (clen * ch / C) / V * V;
      const int64_t s_hi = (ch + 1 == C) ? clen : (clen * (ch + 1) / C) / V * V;
      maxslice = std::max(maxslice, s_hi - s_lo);
    }
  }
  const int NS = g.fifo_slots;
  const size_t need = (size_t)p * C * NS * slot * 4;
  if (need > g.fifo_bytes) {  // grow (synchronises the device once)
    if (g.fifo) {
      if (hipDeviceSynchronize() != hipSuccess || hipFree(g.fifo) != hipSuccess) return SIM_ERR_HIP;
      g.fifo = nullptr;
      g.fifo_bytes = 0;
    }
    if (hipMalloc(&g.fifo, need) != hipSuccess) {
      g.fifo = nullptr;
      (void)hipGetLastError();
      return SIM_ERR_NOMEM;
    }
    g.fifo_bytes = need;
  }
  uint32_t epoch = 0;
  int rc = next_sem_epoch(c, &epoch);
  if (rc) return rc;
  a.fifo = g.fifo;
  a.sem = g.fifo_sem;
  a.err = g.err;
  a.spin_limit = g.spin_limit;
  a.p = p;
  a.C = (int)C;
  a.Cg = (int)Cg;
  a.NS = NS;
  a.nsub = (int)std::max<int64_t>(1, (maxslice + slot - 1) / slot);
  a.slot_elems = slot;
  a.epoch = epoch;
  a.inv_p = inv_p_of(p);
  a.withhold = g.fifo_withhold;
  return hip_err(launch_ring_fifo(c.dtype, c.op, a, c.s));
}

// Tree, recursive exchange and 2PH: every lowered step runs as fold
// launches (GATHER / EXCH transfers, the members of an exchange group
// sharing one transfer) and copy launches (MCAST).  Within a step no
// transfer touches a slot another one writes (the verifier proves it), so
// the step's transfers may run in any order and in one launch.  A rank's
// value of a chunk lives in its input until a fold replaces it with a
// partial, and in its output once finished.  Partials are accumulator-typed:
// 32-bit types keep them in the rank's own output buffer (the slot is only
// read by later steps, never by one that still needs the input there);
// fp16/bf16 keep fp32 partials in library scratch.
int run_sched(const Call& c, const Schedule& sch) {
  const int p = c.p, e = esize_of(c.dtype), V = 16 / e;
  const int nch = sch.nchunks;
  std::vector<int64_t> lo(nch + 1);
  for (int q = 0; q <= nch; q++) lo[q] = chunk_lo((int64_t)c.n, nch, q);
  void* part[SIM_MAX_RANKS] = {};
  if (e == 4) {
    for (int r = 0; r < p; r++) part[r] = c.y[r];
  } else {
    const size_t stride = (c.n + 511) / 512 * 512;  // fp32 elements per rank, whole 512-element blocks
    int rc = ensure_scratch((size_t)p * stride * 4);
    if (rc) return rc;
    for (int r = 0; r < p; r++) part[r] = (char*)g.scratch + (size_t)r * stride * 4;
  }
  enum { IN = 0, PART = 1, OUT = 2 };
  std::vector<uint8_t> loc((size_t)p * nch, IN);
  auto where = [&](int r, int ch) -> uint8_t& { return loc[(size_t)r * nch + ch]; };
  for (const auto& step : sch.steps) {
    std::vector<SchedXfer> folds;
    std::vector<std::pair<int, uint32_t>> group_key;  // (chunk, set) of exchange folds; -1 chunk otherwise
    std::vector<CopyXfer> copies;
    std::vector<std::pair<int, uint8_t>> moves;  // (slot index, new location), applied after the step
    for (const Xfer& xf : step) {
      const bool gather = (xf.kind == XK_GATHER || xf.kind == XK_GATHER_POST);
      const bool exch = (xf.kind == XK_EXCH || xf.kind == XK_EXCH_POST);
      if (gather || exch) {
        const bool fin = (xf.kind == XK_GATHER_POST || xf.kind == XK_EXCH_POST);
        moves.push_back({xf.dst * nch + xf.chunk, fin ? (uint8_t)OUT : (uint8_t)PART});
        if (exch) {
          bool merged = false;
          for (size_t k = 0; k < folds.size(); k++)
            if (group_key[k] == std::make_pair(xf.chunk, xf.mask)) {
              folds[k].dmask |= 1u << xf.dst;
              merged = true;
            }
          if (merged) continue;
        }
        SchedXfer f;
        std::memset(&f, 0, sizeof f);
        f.lo = lo[xf.chunk];
        f.hi = lo[xf.chunk + 1];
        f.dmask = 1u << xf.dst;
        f.final_ = fin ? 1 : 0;
        auto add = [&](int q) {
          const uint8_t w = where(q, xf.chunk);
          if (w == OUT) return false;  // finished values are never folded again
          f.order |= (uint64_t)q << (4 * f.nsrc);
          if (w == PART) f.from_part |= 1u << f.nsrc;
          f.nsrc++;
          return true;
        };
        if (gather && !add(xf.dst)) return SIM_ERR_VERIFY;
        for (int q = 0; q < p; q++)
          if ((xf.mask >> q) & 1u)
            if (!add(q)) return SIM_ERR_VERIFY;
        folds.push_back(f);
        group_key.push_back(exch ? std::make_pair(xf.chunk, xf.mask) : std::make_pair(-1, 0u));
      } else if (xf.kind == XK_MCAST) {
        if (where(xf.src, xf.chunk) != OUT) return SIM_ERR_VERIFY;
        CopyXfer x;
        std::memset(&x, 0, sizeof x);
        x.src = c.y[xf.src];
        for (int q = 0; q < p; q++)
          if ((xf.mask >> q) & 1u) {
            x.dst[x.ndst++] = c.y[q];
            moves.push_back({q * nch + xf.chunk, (uint8_t)OUT});
          }
        x.lo = lo[xf.chunk];
        x.hi = lo[xf.chunk + 1];
        if (x.hi > x.lo) copies.push_back(x);
      } else {
        return SIM_ERR_VERIFY;  // not a kind this executor runs
      }
    }
    // launch the folds, at most kSchedMaxXfers per launch (empty chunks skipped)
    folds.erase(std::remove_if(folds.begin(), folds.end(), [](const SchedXfer& f) { return f.hi <= f.lo; }),
                folds.end());
    for (size_t b = 0; b < folds.size(); b += kSchedMaxXfers) {
      SchedArgs a;
      std::memset(&a, 0, sizeof a);
      for (int r = 0; r < p; r++) {
        a.x[r] = c.x[r];
        a.y[r] = c.y[r];
        a.part[r] = part[r];
      }
      a.p = p;
      a.inv_p = inv_p_of(p);
      a.nx = (int)std::min<size_t>(kSchedMaxXfers, folds.size() - b);
      int64_t maxlen = 0;
      for (int k = 0; k < a.nx; k++) {
        a.xf[k] = folds[b + k];
        maxlen = std::max(maxlen, a.xf[k].hi - a.xf[k].lo);
      }
      a.tiles = tiles_for(c, (maxlen + V - 1) / V, a.nx, 1);
      int rc = hip_err(launch_sched_fold(c.dtype, c.op, a, c.s));
      if (rc) return rc;
    }
    for (size_t b = 0; b < copies.size(); b += SIM_MAX_RANKS) {
      const int count = (int)std::min<size_t>(copies.size() - b, SIM_MAX_RANKS);
      int rc = run_copy_step(c, copies.data() + b, count);
      if (rc) return rc;
    }
    for (auto& m : moves) loc[(size_t)m.first] = m.second;
  }
  return SIM_OK;
}

int run_allreduce(const Call& c) {
  std::string diag;
  const Schedule* sch = cached_schedule(COLL_ALLREDUCE, c.algo, c.p, g_topo, &diag);
  if (!sch) return SIM_ERR_VERIFY;
  if (is_topology_algo(c.algo)) return run_sched(c, *sch);
  const int p = c.p;
  int64_t lo[SIM_MAX_RANKS + 1];
  for (int q = 0; q <= p; q++) lo[q] = chunk_lo((int64_t)c.n, p, q);
  switch (c.algo) {
    case SIM_ALGO_ONESHOT: {
      const int rc = run_phased(c, lo, kPhasedAll, nullptr);
      if (rc >= 0) return rc;
      return run_fold(c, true, lo, nullptr, ptr_set_for(c));
    }
    case SIM_ALGO_ALLPAIRS: {
      const PtrSet* set = ptr_set_for(c);
      int rc = run_phased(c, lo, kPhasedOwner, nullptr);  // step 1: GATHER_REDUCE into each owner
      if (rc < 0) rc = run_fold(c, false, lo, nullptr, set);
      if (rc) return rc;
      const bool step1_phased = g.last_phased;
      rc = run_phased(c, lo, kPhasedFanout, nullptr);  // step 2 (FANOUT), phased
      if (rc >= 0) {
        g.last_phased = g.last_phased || step1_phased;
        return rc;
      }
      if (set) {  // step 2 (FANOUT) from the same table entry
        const int V = 16 / esize_of(c.dtype);
        int64_t maxchunk = 0;
        for (int q = 0; q < p; q++) maxchunk = std::max(maxchunk, lo[q + 1] - lo[q]);
        const int unroll = unroll_for(c);
        FanoutTabArgs f;
        std::memset(&f, 0, sizeof f);
        f.set = set;
        f.n = (int64_t)c.n;
        f.p = p;
        f.tiles = tiles_for(c, (maxchunk + V - 1) / V, p, unroll);
        return hip_err(launch_fanout_tab(esize_of(c.dtype), f, unroll, c.s));
      }
      CopyXfer xs[SIM_MAX_RANKS];                // step 2: FANOUT from each owner (p transfers)
      int nx = 0;
      for (const Xfer& xf : sch->steps[1]) {
        CopyXfer& x = xs[nx++];
        std::memset(&x, 0, sizeof x);
        x.src = c.y[xf.src];
        for (int r = 0; r < p; r++)
          if (r != xf.src) x.dst[x.ndst++] = c.y[r];
        x.lo = lo[xf.chunk];
        x.hi = lo[xf.chunk + 1];
      }
      return run_copy_step(c, xs, nx);
    }
    case SIM_ALGO_RING: {
      if (const PtrSet* set = ptr_set_for(c)) return run_ring_tab(c, set, lo);
      int rc = run_ring_rs(c, *sch, p - 1, false, lo);
      if (rc) return rc;
      for (int st = p - 1; st < 2 * (p - 1); st++) {
        CopyXfer xs[SIM_MAX_RANKS];  // p transfers per step
        int nx = 0;
        for (const Xfer& xf : sch->steps[st]) {
          CopyXfer& x = xs[nx++];
          std::memset(&x, 0, sizeof x);
          x.src = c.y[xf.src];
          x.dst[x.ndst++] = c.y[xf.dst];
          x.lo = lo[xf.chunk];
          x.hi = lo[xf.chunk + 1];
        }
        rc = run_copy_step(c, xs, nx);
        if (rc) return rc;
      }
      return SIM_OK;
    }
    case SIM_ALGO_RING_FIFO:
      return run_ring_fifo(c, lo);
    case SIM_ALGO_ALLPAIRS_PERSISTENT:
      return run_allpairs_persistent(c, lo);
    case SIM_ALGO_ONESHOT_LL: {
      LLArgs a;
      std::memset(&a, 0, sizeof a);
      const int e = esize_of(c.dtype);
      uint32_t epoch = 0;
      int rc = next_ll_epoch(c, &epoch);
      if (rc) return rc;
      for (int q = 0; q < p; q++) {
        a.x[q] = c.x[q];
        a.y[q] = c.y[q];
      }
      for (int q = 0; q <= p; q++) a.lo[q] = lo[q];
      a.ll = g.ll;
      a.ll_stride = g.ll_stride;
      a.n = (int64_t)c.n;
      a.nwords = ((int64_t)c.n * e + 3) / 4;
      // At least 16 tiles while a tile keeps 16 words, and consumers take
      // the tile 8 ahead: under the round-robin dispatch of workgroups to
      // the 8 XCDs the packets of a tile are then read on the XCD that wrote
      // them (with one tile per workgroup, or a workgroup count that is a
      // multiple of 8)
      int64_t tw = kBlock;
      while (tw > 16 && (a.nwords + tw - 1) / tw < 16) tw /= 2;
      a.tile_words = tw;
      a.ntiles = (a.nwords + a.tile_words - 1) / a.tile_words;
      a.spin_limit = g.spin_limit;
      a.err = g.err;
      a.p = p;
      a.epoch = epoch;
      a.wait_epoch = epoch + g.wait_skew;
      a.shift = a.ntiles >= 16 ? 8 : (a.ntiles > 1 ? 1 : 0);
      a.inv_p = inv_p_of(p);
      int& occ = g.ll_occ[c.dtype][c.op];
      if (occ == 0) occ = ll_blocks_per_cu(c.dtype, c.op);
      const int64_t resident = (int64_t)occ * g.cu_count;
      int64_t cap = resident;
      if (g_max_wg > 0) cap = std::min<int64_t>(cap, g_max_wg);
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(a.ntiles, cap));
      return hip_err(launch_ll(c.dtype, c.op, a, grid, c.s));
    }
  }
  return SIM_ERR_INVALID_ARG;
}

int run_reduce_scatter(const Call& c) {
  std::string diag;
  const Schedule* sch = cached_schedule(COLL_REDUCE_SCATTER, c.algo, c.p, g_topo, &diag);
  if (!sch) return SIM_ERR_VERIFY;
  const int p = c.p;
  std::vector<int64_t> lo(p + 1);
  for (int q = 0; q <= p; q++) lo[q] = chunk_lo((int64_t)c.n, p, q);
  if (c.algo == SIM_ALGO_ALLPAIRS) {
    std::vector<int64_t> shift(p);
    for (int q = 0; q < p; q++) shift[q] = lo[q];
    const int rc = run_phased(c, lo.data(), kPhasedOwner, shift.data());
    if (rc >= 0) return rc;
    return run_fold(c, false, lo.data(), shift.data(), nullptr);
  }
  return run_ring_rs(c, *sch, p - 1, true, lo.data());
}

int run_all_gather(const Call& c) {
  std::string diag;
  const Schedule* sch = cached_schedule(COLL_ALL_GATHER, c.algo, c.p, g_topo, &diag);
  if (!sch) return SIM_ERR_VERIFY;
  const int p = c.p;
  const int64_t nin = (int64_t)c.n / p;
  if (c.algo == SIM_ALGO_ALLPAIRS) {  // direct: output block q is rank q's input
    int64_t lo[SIM_MAX_RANKS + 1];
    for (int q = 0; q <= p; q++) lo[q] = q * nin;
    const int rc = run_phased(c, lo, kPhasedGather, nullptr);
    if (rc >= 0) return rc;
  }
  for (size_t st = 0; st < sch->steps.size(); st++) {
    // merge the step's transfers that share (source rank, block) into one
    // multi-destination copy: one load, several stores
    std::vector<CopyXfer> xs;
    std::vector<std::pair<int, int>> keys;
    for (const Xfer& xf : sch->steps[st]) {
      const int64_t l = xf.chunk * nin, h = l + nin;
      // the source block: the rank's own input for its own block at step 0
      // (ring) or for every block (direct); a finished output block otherwise
      const bool from_input = (c.algo == SIM_ALGO_ALLPAIRS) || (st == 0);
      auto key = std::make_pair(xf.src, xf.chunk);
      size_t idx = std::find(keys.begin(), keys.end(), key) - keys.begin();
      if (idx == keys.size()) {
        CopyXfer x;
        std::memset(&x, 0, sizeof x);
        if (from_input) {
          x.src = c.x[xf.src];
          x.src_shift = l;
        } else {
          x.src = c.y[xf.src];
          x.src_shift = 0;
        }
        x.lo = l;
        x.hi = h;
        xs.push_back(x);
        keys.push_back(key);
      }
      CopyXfer& x = xs[idx];
      auto add_dst = [&](int r) {
        void* d = c.y[r];
        // in place, the owner's block already holds the data
        if (c.inplace && (const char*)d + l * esize_of(c.dtype) == (const char*)c.x[xf.src]) return;
        x.dst[x.ndst++] = d;
      };
      if (xf.kind == XK_FANOUT) {
        for (int r = 0; r < p; r++) add_dst(r);  // every rank's output, the owner's included
      } else {
        add_dst(xf.dst);
      }
    }
    xs.erase(std::remove_if(xs.begin(), xs.end(), [](const CopyXfer& x) { return x.ndst == 0; }), xs.end());
    int rc = run_copy_step(c, xs.data(), (int)xs.size());
    if (rc) return rc;
  }
  return SIM_OK;
}

// legal candidates for AUTO / explicit requests
bool legal(int coll, int algo, int p, size_t n, int dtype) {
  // LL and the single-launch ring and all-pairs carry a per-call epoch in
  // their kernel arguments: a replayed graph would repeat it and accept
  // stale flags
  if (g.capturing && (algo == SIM_ALGO_ONESHOT_LL || algo == SIM_ALGO_RING_FIFO ||
                      algo == SIM_ALGO_ALLPAIRS_PERSISTENT))
    return false;
  if (coll == COLL_ALLREDUCE) {
    if (algo == SIM_ALGO_ONESHOT_LL) return n * (size_t)esize_of(dtype) <= SIM_LL_MAX_BYTES_PER_RANK;
    if (is_topology_algo(algo)) return cached_schedule(coll, algo, p, g_topo, nullptr) != nullptr;
    return algo >= SIM_ALGO_RING && algo <= kLastAlgo;
  }
  return algo == SIM_ALGO_RING || algo == SIM_ALGO_ALLPAIRS;
}

// AUTO weighs the single-node schedules; the tree, recursive-exchange and
// 2PH schedules model multi-node topologies and run when asked for by name
const int kAutoCandidates[] = {SIM_ALGO_RING,       SIM_ALGO_ALLPAIRS,  SIM_ALGO_ONESHOT,
                               SIM_ALGO_ONESHOT_LL, SIM_ALGO_RING_FIFO, SIM_ALGO_ALLPAIRS_PERSISTENT};
// the schedules the allocation-free entry point runs (no library buffers)
const int kNoAllocCandidates[] = {SIM_ALGO_RING, SIM_ALGO_ALLPAIRS, SIM_ALGO_ONESHOT};

// Bytes per rank from which the model prices an algo with its second regime
// (Model::hi; 0: one regime): the single-launch ring's FIFO protocol above
// the LL limit, and the one-shot from the size where it runs phased.
double model_hi_from(int coll, int algo, int p) {
  if (coll != COLL_ALLREDUCE) return 0.0;
  if (algo == SIM_ALGO_RING_FIFO) return (double)g.ring_ll_max + 1.0;
  if (algo == SIM_ALGO_ONESHOT) return (double)phased_threshold(kPhasedAll, p);
  return 0.0;
}

double predict(int coll, int algo, int p, double n, int esize) {
  return model_predict(g.model, coll, algo, p, n, esize, g_topo, g_max_wg, model_hi_from(coll, algo, p));
}

int pick(int coll, int p, size_t n, int dtype, int* algo, double* us, const int* cands = kAutoCandidates,
         int ncands = (int)(sizeof kAutoCandidates / sizeof kAutoCandidates[0])) {
  int best = -1;
  double bt = 0;
  for (int k = 0; k < ncands; k++) {
    const int a = cands[k];
    if (!legal(coll, a, p, n, dtype)) continue;
    const double t = predict(coll, a, p, (double)n, esize_of(dtype));
    if (best < 0 || t < bt) {
      best = a;
      bt = t;
    }
  }
  if (best < 0) return SIM_ERR_UNSUPPORTED;
  *algo = best;
  if (us) *us = bt;
  return SIM_OK;
}

int resolve_algo(int coll, int p, size_t n, int dtype, int* algo, double* us) {
  if (*algo < SIM_ALGO_AUTO || *algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  if (*algo == SIM_ALGO_AUTO && coll == COLL_ALLREDUCE && g.env_algo > 0) *algo = g.env_algo;
  if (*algo == SIM_ALGO_AUTO) return pick(coll, p, n, dtype, algo, us);
  if (!legal(coll, *algo, p, n, dtype)) return SIM_ERR_UNSUPPORTED;
  if (us) *us = predict(coll, *algo, p, (double)n, esize_of(dtype));
  return SIM_OK;
}

// Is `s` being captured into a graph?  Sets g.capturing for the current call.
int begin_call(void* stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return SIM_ERR_HIP;
  }
  g.capturing = (st != hipStreamCaptureStatusNone);
  if (g.capturing) g.captured = true;
  g.last_phased = false;
  g.last_whole = false;
  return SIM_OK;
}

void log_call(const char* what, const Call& c, double us) {
  if (!g.log) return;
  std::fprintf(stderr, "[simar] %s: %zu bytes/rank p %d -> algo %s%s steps %d predicted %.2f us\n", what,
               c.n * (size_t)esize_of(c.dtype), c.p, algo_name(c.algo),
               g.last_phased ? " (phased fold)" : "",
               model_launches(c.coll, c.algo, c.p, g_topo), us);
}

int parse_algo_env(const char* v) {
  if (!v) return 0;
  for (int a = 1; a <= kLastAlgo; a++)
    if (!std::strcmp(v, algo_name(a))) return a;
  return 0;
}

}  // namespace
}  // namespace simar

using namespace simar;

extern "C" {

int sim_version(void) { return kVersion; }

const char* sim_status_string(int status) {
  switch (status) {
    case SIM_OK: return "ok";
    case SIM_ERR_INVALID_ARG: return "invalid argument";
    case SIM_ERR_UNSUPPORTED: return "unsupported by the requested algorithm";
    case SIM_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case SIM_ERR_ALIAS: return "output overlaps an input or another output";
    case SIM_ERR_NOMEM: return "out of device memory for library scratch";
    case SIM_ERR_HIP: return "HIP runtime error";
    case SIM_ERR_TIMEOUT: return "a bounded device-side wait expired";
    case SIM_ERR_VERIFY: return "schedule failed verification";
    case SIM_ERR_NOT_INIT: return "library not initialised";
  }
  return "unknown status";
}

int sim_finalize(void) {
  // (also releases what a failed sim_init had allocated before it gave up)
  if (!g.init && !g.err && !g.ll && !g.fifo_sem && !g.scratch && !g.ptab && !g.ptab_host && !g.ph_mem &&
      !g.ph_host_done)
    return SIM_OK;
  // teardown is best effort: every allocation is released even if one call fails
  (void)hipSetDevice(g.device);
  (void)hipDeviceSynchronize();
  if (g.scratch) (void)hipFree(g.scratch);
  for (void* r : g.retired) (void)hipFree(r);
  if (g.ll) (void)hipFree(g.ll);
  if (g.fifo) (void)hipFree(g.fifo);
  if (g.fifo_sem) (void)hipFree(g.fifo_sem);
  if (g.ph_mem) (void)hipFree(g.ph_mem);
  if (g.ph_host_done) (void)hipHostFree(g.ph_host_done);
  if (g.err) (void)hipFree(g.err);
  for (PtrSlot& sl : g.ptab_slots)
    if (sl.done) (void)hipEventDestroy(sl.done);
  if (g.ptab) (void)hipFree(g.ptab);
  if (g.ptab_host) (void)hipHostFree(g.ptab_host);
  (void)hipGetLastError();
  Model keep = g.model;
  g = Ctx();
  g.model = keep;
  return SIM_OK;
}

int sim_init(int device, int p_max, size_t max_bytes_per_rank) {
  if (p_max < 2 || p_max > SIM_MAX_RANKS) return SIM_ERR_INVALID_ARG;
  sim_finalize();
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
    (void)hipGetLastError();
    return device < 0 ? SIM_ERR_INVALID_ARG : SIM_ERR_HIP;
  }
  if (hipSetDevice(device) != hipSuccess) return SIM_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SIM_ERR_HIP;
  g.device = device;
  g_launch_device = device;
  g.p_max = p_max;
  g.cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  if (hipMalloc(&g.err, 256) != hipSuccess) return SIM_ERR_NOMEM;
  if (hipMemset(g.err, 0, 256) != hipSuccess) return SIM_ERR_HIP;
  g.ll_stride = (int64_t)(2 * SIM_LL_MAX_BYTES_PER_RANK / 8);  // packets per rank
  if (hipMalloc(&g.ll, (size_t)p_max * g.ll_stride * 8) != hipSuccess) {
    sim_finalize();
    return SIM_ERR_NOMEM;
  }
  if (launch_fill64(g.ll, 0ull, (int64_t)p_max * g.ll_stride, nullptr) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    sim_finalize();
    return SIM_ERR_HIP;
  }
  const int64_t nsem = (int64_t)p_max * kFifoMaxChannels * 2;
  if (hipMalloc(&g.fifo_sem, (size_t)nsem * 8) != hipSuccess) {
    sim_finalize();
    return SIM_ERR_NOMEM;
  }
  if (launch_fill64(g.fifo_sem, 0ull, nsem, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    sim_finalize();
    return SIM_ERR_HIP;
  }
  // phased one-shot barrier slots, zeroed (the expired count sits after them)
  g.ph_gmax = 2 * g.cu_count;
  g.ph_slot_words = (int64_t)(1 + g.ph_gmax + kPhasedGroups) * kPhasedFlagStride;
  const int64_t ph_words = g.ph_slot_words * kPhasedSlots + kPhasedFlagStride;
  if (hipMalloc(&g.ph_mem, (size_t)ph_words * 8) != hipSuccess) {
    sim_finalize();
    return SIM_ERR_NOMEM;
  }
  if (launch_fill64(g.ph_mem, 0ull, ph_words, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    sim_finalize();
    return SIM_ERR_HIP;
  }
  g.ph_expired = (unsigned int*)(g.ph_mem + g.ph_slot_words * kPhasedSlots);
  // (no phased calls without the host word)
  if (hipHostMalloc((void**)&g.ph_host_done, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
      hipHostGetDevicePointer((void**)&g.ph_dev_done, g.ph_host_done, 0) != hipSuccess) {
    (void)hipGetLastError();
    if (g.ph_host_done) (void)hipHostFree(g.ph_host_done);
    g.ph_host_done = nullptr;
    g.ph_dev_done = nullptr;
  } else {
    *g.ph_host_done = 0;
  }
  // the pointer table only makes launches cheaper: without it every call
  // carries its pointers in its kernel arguments
  if (hipMalloc(&g.ptab, sizeof(PtrSet) * kPtrSets) != hipSuccess ||
      hipHostMalloc(&g.ptab_host, sizeof(PtrSet) * kPtrSets, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    if (g.ptab) (void)hipFree(g.ptab);
    g.ptab = nullptr;
    g.ptab_host = nullptr;
  }
  g.ptab_slots.assign(kPtrSets, PtrSlot());
  // the allocation-free entry point: its scratch array's address on this
  // device, and its schedules lowered and verified now, so that its calls
  // find them cached
  if (noalloc_setup(device) != SIM_OK) {
    sim_finalize();
    return SIM_ERR_HIP;
  }
  for (int p = 2; p <= p_max; p++)
    for (int a : kNoAllocCandidates) (void)cached_schedule(COLL_ALLREDUCE, a, p, g_topo, nullptr);
  g.init = true;
  if (max_bytes_per_rank > 0) {
    const size_t n = max_bytes_per_rank / 2;  // 16-bit elements need the most slots
    size_t need = 0;
    for (int p = 2; p <= p_max; p++) need = std::max(need, scratch_need(n, p));
    int rc = ensure_scratch(need);
    if (rc) {
      sim_finalize();
      return rc;
    }
  }
  const char* dbg = std::getenv("SIM_DEBUG");
  g.log = (dbg && dbg[0] == '1') ? 1 : 0;
  g.env_algo = parse_algo_env(std::getenv("SIM_ALGO"));
  const char* calib = std::getenv("SIM_CALIB");
  if (calib && calib[0]) {
    std::string err;
    if (!model_load_json(calib, &g.model, &err) && g.log)
      std::fprintf(stderr, "[simar] SIM_CALIB %s not loaded: %s\n", calib, err.c_str());
  }
  return SIM_OK;
}

int sim_allreduce(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n, int dtype,
                  int op, int algo, void* stream) {
  int rc = check_scalars(p, dtype, op, true);
  if (rc) return rc;
  if (algo < SIM_ALGO_AUTO || algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  if (n == 0) return SIM_OK;
  const size_t e = (size_t)esize_of(dtype);
  if (n > ((size_t)1 << 46) / e) return SIM_ERR_INVALID_ARG;
  bool inplace = false;
  rc = check_buffers(in_ptrs, out_ptrs, p, n * e, n * e, nullptr, &inplace);
  if (rc) return rc;
  double us = 0;
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  rc = begin_call(stream);
  if (rc) return rc;
  rc = resolve_algo(COLL_ALLREDUCE, p, n, dtype, &algo, &us);
  if (rc) return rc;
  Call c{COLL_ALLREDUCE, p, dtype, op, algo, n, in_ptrs, out_ptrs, inplace, (hipStream_t)stream};
  rc = run_allreduce(c);
  if (rc) return rc;
  g.last_algo = algo;
  log_call("AllReduce", c, us);
  return SIM_OK;
}

int sim_allreduce_noalloc(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n, int dtype,
                          int op, int algo, void* stream) {
  int rc = check_scalars(p, dtype, op, true);
  if (rc) return rc;
  if (algo < SIM_ALGO_AUTO || algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  if (algo != SIM_ALGO_AUTO && algo != SIM_ALGO_RING && algo != SIM_ALGO_ALLPAIRS && algo != SIM_ALGO_ONESHOT)
    return SIM_ERR_UNSUPPORTED;
  if (n == 0) return SIM_OK;
  const size_t e = (size_t)esize_of(dtype);
  if (n > ((size_t)1 << 46) / e) return SIM_ERR_INVALID_ARG;
  bool inplace = false;
  rc = check_buffers(in_ptrs, out_ptrs, p, n * e, n * e, nullptr, &inplace);
  if (rc) return rc;
  void* const fixed = noalloc_scratch(g.device);
  if (!fixed) return SIM_ERR_NOT_INIT;
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  rc = begin_call(stream);
  if (rc) return rc;
  double us = 0;
  if (algo == SIM_ALGO_AUTO) {
    rc = pick(COLL_ALLREDUCE, p, n, dtype, &algo, &us, kNoAllocCandidates,
              (int)(sizeof kNoAllocCandidates / sizeof kNoAllocCandidates[0]));
    if (rc) return rc;
  } else {
    us = predict(COLL_ALLREDUCE, algo, p, (double)n, (int)e);
  }
  // only the 16-bit ring (p > 2) keeps partials: they must fit the array
  if (algo == SIM_ALGO_RING && e == 2 && p > 2 && scratch_need(n, p) > SIM_NOALLOC_SCRATCH_BYTES)
    return SIM_ERR_NOMEM;
  Call c{COLL_ALLREDUCE, p, dtype, op, algo, n, in_ptrs, out_ptrs, inplace, (hipStream_t)stream};
  c.fixed_scratch = fixed;
  c.noalloc = true;
  rc = run_allreduce(c);
  if (rc) return rc;
  g.last_algo = algo;
  log_call("AllReduce (allocation-free)", c, us);
  return SIM_OK;
}

int sim_reduce_scatter(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n_out,
                       int dtype, int op, int algo, void* stream) {
  int rc = check_scalars(p, dtype, op, true);
  if (rc) return rc;
  if (algo < SIM_ALGO_AUTO || algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  if (n_out == 0) return SIM_OK;
  const size_t e = (size_t)esize_of(dtype);
  if (n_out > ((size_t)1 << 46) / e / (size_t)p) return SIM_ERR_INVALID_ARG;
  if (algo == SIM_ALGO_AUTO) algo = SIM_ALGO_ALLPAIRS;
  if (algo != SIM_ALGO_RING && algo != SIM_ALGO_ALLPAIRS) return SIM_ERR_UNSUPPORTED;
  std::vector<size_t> off(p);
  for (int r = 0; r < p; r++) off[r] = 0;
  // in place: out[r] is chunk r of in[r]  (in[r] == out[r] - r*chunk)
  bool inplace = false;
  {
    int n_inplace = 0;
    if (!in_ptrs || !out_ptrs) return SIM_ERR_INVALID_ARG;
    for (int r = 0; r < p; r++) {
      if (!in_ptrs[r] || !out_ptrs[r]) return SIM_ERR_INVALID_ARG;
      if ((const char*)out_ptrs[r] == (const char*)in_ptrs[r] + (size_t)r * n_out * e) n_inplace++;
    }
    if (n_inplace != 0 && n_inplace != p) return SIM_ERR_INVALID_ARG;
    inplace = (n_inplace == p);
  }
  if (inplace) {
    for (int r = 0; r < p; r++)
      if (((uintptr_t)in_ptrs[r] | (uintptr_t)out_ptrs[r]) & 15u) return SIM_ERR_ALIGN;
    // the input buffers must not overlap each other
    for (int r = 0; r < p; r++)
      for (int q = r + 1; q < p; q++)
        if (overlap({(uintptr_t)in_ptrs[r], (uintptr_t)in_ptrs[r] + p * n_out * e},
                    {(uintptr_t)in_ptrs[q], (uintptr_t)in_ptrs[q] + p * n_out * e}))
          return SIM_ERR_ALIAS;
  } else {
    bool ip2 = false;
    rc = check_buffers(in_ptrs, out_ptrs, p, (size_t)p * n_out * e, n_out * e, off.data(), &ip2);
    if (rc) return rc;
    if (ip2) return SIM_ERR_ALIAS;
  }
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  rc = begin_call(stream);
  if (rc) return rc;
  Call c{COLL_REDUCE_SCATTER, p, dtype, op, algo, (size_t)p * n_out, in_ptrs, out_ptrs, inplace,
         (hipStream_t)stream};
  rc = run_reduce_scatter(c);
  if (rc) return rc;
  g.last_algo = algo;
  log_call("ReduceScatter", c, predict(c.coll, algo, p, (double)c.n, (int)e));
  return SIM_OK;
}

int sim_all_gather(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n_in, int dtype,
                   int algo, void* stream) {
  int rc = check_scalars(p, dtype, SIM_SUM, false);
  if (rc) return rc;
  if (algo < SIM_ALGO_AUTO || algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  if (n_in == 0) return SIM_OK;
  const size_t e = (size_t)esize_of(dtype);
  if (n_in > ((size_t)1 << 46) / e / (size_t)p) return SIM_ERR_INVALID_ARG;
  if (algo == SIM_ALGO_AUTO) algo = SIM_ALGO_ALLPAIRS;
  if (algo != SIM_ALGO_RING && algo != SIM_ALGO_ALLPAIRS) return SIM_ERR_UNSUPPORTED;
  // in place: in[r] is block r of out[r]
  std::vector<size_t> off(p);
  for (int r = 0; r < p; r++) off[r] = (size_t)r * n_in * e;
  bool inplace = false;
  if (!in_ptrs || !out_ptrs) return SIM_ERR_INVALID_ARG;
  {
    int n_inplace = 0;
    for (int r = 0; r < p; r++) {
      if (!in_ptrs[r] || !out_ptrs[r]) return SIM_ERR_INVALID_ARG;
      if (((uintptr_t)in_ptrs[r] | (uintptr_t)out_ptrs[r]) & 15u) return SIM_ERR_ALIGN;
      if ((const char*)in_ptrs[r] == (const char*)out_ptrs[r] + off[r]) n_inplace++;
    }
    if (n_inplace != 0 && n_inplace != p) return SIM_ERR_INVALID_ARG;
    inplace = (n_inplace == p);
  }
  {
    std::vector<Range> outs(p), ins(p);
    for (int r = 0; r < p; r++) {
      outs[r] = {(uintptr_t)out_ptrs[r], (uintptr_t)out_ptrs[r] + (size_t)p * n_in * e};
      ins[r] = {(uintptr_t)in_ptrs[r], (uintptr_t)in_ptrs[r] + n_in * e};
    }
    for (int r = 0; r < p; r++)
      for (int q = 0; q < p; q++) {
        if (q != r && overlap(outs[r], outs[q])) return SIM_ERR_ALIAS;
        if (inplace ? (q != r && overlap(outs[r], ins[q])) : overlap(outs[r], ins[q])) return SIM_ERR_ALIAS;
      }
  }
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  rc = begin_call(stream);
  if (rc) return rc;
  Call c{COLL_ALL_GATHER, p, dtype, SIM_SUM, algo, (size_t)p * n_in, in_ptrs, out_ptrs, inplace,
         (hipStream_t)stream};
  rc = run_all_gather(c);
  if (rc) return rc;
  g.last_algo = algo;
  log_call("AllGather", c, predict(c.coll, algo, p, (double)c.n, (int)e));
  return SIM_OK;
}

int sim_select(int p, size_t n, int dtype, int op, int* algo_out, double* predicted_us) {
  if (!algo_out) return SIM_ERR_INVALID_ARG;
  if (p < 2 || p > SIM_MAX_RANKS) return SIM_ERR_INVALID_ARG;
  if (dtype < SIM_INT32 || dtype > SIM_BF16 || op < SIM_SUM || op > SIM_AVG) return SIM_ERR_INVALID_ARG;
  int a = SIM_ALGO_AUTO;
  double us = 0;
  g.capturing = false;  // the pick of an ordinary (not captured) call
  int rc = resolve_algo(COLL_ALLREDUCE, p, n, dtype, &a, &us);
  if (rc) return rc;
  *algo_out = a;
  if (predicted_us) *predicted_us = us;
  return SIM_OK;
}

int sim_last_algo(void) { return g.last_algo; }

int sim_model_load(const char* json_path) {
  if (!json_path) return SIM_ERR_INVALID_ARG;
  std::string err;
  if (!model_load_json(json_path, &g.model, &err)) {
    if (g.log) std::fprintf(stderr, "[simar] model %s not loaded: %s\n", json_path, err.c_str());
    return SIM_ERR_INVALID_ARG;
  }
  return SIM_OK;
}

int sim_model_predict(int algo, int p, int dtype, double bytes_per_rank, double* us_out) {
  if (!us_out || algo < SIM_ALGO_RING || algo > kLastAlgo || p < 2 || p > SIM_MAX_RANKS ||
      dtype < SIM_INT32 || dtype > SIM_BF16 || !(bytes_per_rank >= 0))
    return SIM_ERR_INVALID_ARG;
  if (is_topology_algo(algo) && !cached_schedule(COLL_ALLREDUCE, algo, p, g_topo, nullptr))
    return SIM_ERR_UNSUPPORTED;
  const int e = esize_of(dtype);
  *us_out = predict(COLL_ALLREDUCE, algo, p, bytes_per_rank / e, e);
  return SIM_OK;
}

int sim_model_set(int algo, double alpha_us, double steps, double bytes_factor, double gbps) {
  if (algo < SIM_ALGO_RING || algo > kLastAlgo || !(gbps > 0) || !(alpha_us >= 0))
    return SIM_ERR_INVALID_ARG;
  AlgoModel& m = g.model.a[algo];
  m.alpha_us = alpha_us;
  m.gbps = gbps;
  m.steps = steps;
  m.bytes_factor = bytes_factor;
  m.host_us = 0.0;  // the additive form as given; sim_model_set_host_overlap adds the host term
  g.model.has_hi[algo] = false;  // one line for every size
  g.model.source = "sim_model_set";
  return SIM_OK;
}

int sim_model_set_host_overlap(int algo, double host_us_per_launch) {
  if (algo < SIM_ALGO_RING || algo > kLastAlgo || !(host_us_per_launch >= 0)) return SIM_ERR_INVALID_ARG;
  g.model.a[algo].host_us = host_us_per_launch;
  g.model.hi[algo].host_us = host_us_per_launch;
  g.model.source = "sim_model_set_host_overlap";
  return SIM_OK;
}

int sim_model_set_workgroup_rate(int algo, double gbps_per_workgroup) {
  if (algo < SIM_ALGO_RING || algo > kLastAlgo || !(gbps_per_workgroup >= 0)) return SIM_ERR_INVALID_ARG;
  g.model.a[algo].wg_gbps = gbps_per_workgroup;
  g.model.hi[algo].wg_gbps = gbps_per_workgroup;
  g.model.source = "sim_model_set_workgroup_rate";
  return SIM_OK;
}

int sim_model_reset(void) {
  g.model = default_model();
  return SIM_OK;
}

int sim_check_error(void* stream) {
  if (!g.init) return SIM_ERR_NOT_INIT;
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SIM_ERR_HIP;
  int word = 0;
  if (hipMemcpy(&word, g.err, sizeof word, hipMemcpyDeviceToHost) != hipSuccess) return SIM_ERR_HIP;
  if (word != 0) {
    if (hipMemset(g.err, 0, sizeof word) != hipSuccess) return SIM_ERR_HIP;
    return word;
  }
  return SIM_OK;
}

int sim_copy_streams(const void* const* src_ptrs, void* const* dst_ptrs, int k, size_t bytes, int workgroups,
                     void* stream) {
  if (!g.init) return SIM_ERR_NOT_INIT;
  if (k < 1 || k > SIM_MAX_RANKS || workgroups < 0 || (bytes & 15u)) return SIM_ERR_INVALID_ARG;
  if (!src_ptrs || !dst_ptrs) return SIM_ERR_INVALID_ARG;
  if (bytes > ((size_t)1 << 46)) return SIM_ERR_INVALID_ARG;
  Range srcs[SIM_MAX_RANKS], dsts[SIM_MAX_RANKS];
  for (int q = 0; q < k; q++) {
    if (!src_ptrs[q] || !dst_ptrs[q]) return SIM_ERR_INVALID_ARG;
    if (((uintptr_t)src_ptrs[q] | (uintptr_t)dst_ptrs[q]) & 15u) return SIM_ERR_ALIGN;
    srcs[q] = {(uintptr_t)src_ptrs[q], (uintptr_t)src_ptrs[q] + bytes};
    dsts[q] = {(uintptr_t)dst_ptrs[q], (uintptr_t)dst_ptrs[q] + bytes};
  }
  for (int q = 0; q < k; q++)
    for (int r = 0; r < k; r++)
      if (overlap(dsts[q], srcs[r]) || (r != q && overlap(dsts[q], dsts[r]))) return SIM_ERR_ALIAS;
  if (bytes == 0) return SIM_OK;
  if (use_device() != SIM_OK) return SIM_ERR_HIP;
  CopyStreamsArgs a;
  std::memset(&a, 0, sizeof a);
  for (int q = 0; q < k; q++) {
    a.src[q] = src_ptrs[q];
    a.dst[q] = dst_ptrs[q];
  }
  a.k = k;
  a.nvec = (int64_t)(bytes / 16);
  int64_t wg = workgroups > 0 ? workgroups : (a.nvec + kBlock - 1) / kBlock;
  wg = std::max<int64_t>(1, std::min<int64_t>(wg, kMaxTiles));
  return hip_err(launch_copy_streams(a, (int)wg, (hipStream_t)stream));
}

int sim_config_set(int key, int value) {
  switch (key) {
    case SIM_CONFIG_RANKS_PER_NODE:
      if (value < 1 || value > SIM_MAX_RANKS) return SIM_ERR_INVALID_ARG;
      g_topo.ranks_per_node = value;
      return SIM_OK;
    case SIM_CONFIG_RADIX:
      if (value < 2 || value > SIM_MAX_RANKS) return SIM_ERR_INVALID_ARG;
      g_topo.radix = value;
      return SIM_OK;
    case SIM_CONFIG_MAX_WORKGROUPS:
      if (value < 0) return SIM_ERR_INVALID_ARG;
      g_max_wg = value;
      return SIM_OK;
  }
  return SIM_ERR_INVALID_ARG;
}

int sim_config_get(int key, int* value) {
  if (!value) return SIM_ERR_INVALID_ARG;
  switch (key) {
    case SIM_CONFIG_RANKS_PER_NODE: *value = g_topo.ranks_per_node; return SIM_OK;
    case SIM_CONFIG_RADIX: *value = g_topo.radix; return SIM_OK;
    case SIM_CONFIG_MAX_WORKGROUPS: *value = g_max_wg; return SIM_OK;
  }
  return SIM_ERR_INVALID_ARG;
}

int sim_tree_info(int tree, int p, int ranks_per_node, int rank, int* parent, int* children, int* nchildren) {
  if (tree < 0 || tree > 1 || p < 2 || p > SIM_MAX_RANKS || ranks_per_node < 1 || p % ranks_per_node != 0 ||
      rank < 0 || rank >= p || !parent || !children || !nchildren)
    return SIM_ERR_INVALID_ARG;
  *parent = rank_tree_parent(tree, p, ranks_per_node, rank);
  *nchildren = rank_tree_children(tree, p, ranks_per_node, rank, children);
  return SIM_OK;
}

// lowered (not cached) schedule of the current topology; SIM_ERR_UNSUPPORTED
// when (algo, p, topology) has none
static int lower_current(int algo, int p, Schedule* s) {
  if (p < 2 || p > SIM_MAX_RANKS || algo < SIM_ALGO_RING || algo > kLastAlgo) return SIM_ERR_INVALID_ARG;
  return lower(COLL_ALLREDUCE, algo, p, g_topo, s) ? SIM_OK : SIM_ERR_UNSUPPORTED;
}

int sim_schedule_info(int algo, int p, int* nsteps, int* nxfers, int* nchunks) {
  Schedule s;
  int rc = lower_current(algo, p, &s);
  if (rc) return rc;
  if (nsteps) *nsteps = (int)s.steps.size();
  if (nxfers) *nxfers = s.nxfers();
  if (nchunks) *nchunks = s.nchunks;
  return SIM_OK;
}

int sim_schedule_xfers(int algo, int p, int step, int* out, int max, int* count) {
  Schedule s;
  int rc = lower_current(algo, p, &s);
  if (rc) return rc;
  if (step < 0 || step >= (int)s.steps.size() || !count) return SIM_ERR_INVALID_ARG;
  int k = 0;
  for (const Xfer& x : s.steps[step]) {
    if (k >= max) break;
    if (out) {
      out[5 * k + 0] = x.kind;
      out[5 * k + 1] = x.src;
      out[5 * k + 2] = x.dst;
      out[5 * k + 3] = x.chunk;
      out[5 * k + 4] = (int)x.mask;
    }
    k++;
  }
  *count = k;
  return SIM_OK;
}

int sim_schedule_state(int algo, int p, int after_steps, uint32_t* masks) {
  Schedule s;
  if (!masks) return SIM_ERR_INVALID_ARG;
  int rc = lower_current(algo, p, &s);
  if (rc) return rc;
  std::string d;
  return symbolic_state(s, after_steps, masks, &d) ? SIM_OK : SIM_ERR_INVALID_ARG;
}

static void put_diag(const std::string& d, char* diag, size_t len) {
  if (!diag || len == 0) return;
  std::snprintf(diag, len, "%s", d.c_str());
}

int sim_verify_schedule(int algo, int p, char* diag, size_t diag_len) {
  Schedule s;
  int rc = lower_current(algo, p, &s);
  if (rc) {
    put_diag("no lowering for this (algo, p, topology)", diag, diag_len);
    return rc;
  }
  std::string d;
  const bool ok = verify(s, &d);
  put_diag(d, diag, diag_len);
  return ok ? SIM_OK : SIM_ERR_VERIFY;
}

int sim_verify_custom(int algo, int p, int nchunks, int rounds, int nsteps, const int* counts,
                      const int* xfers, char* diag, size_t diag_len) {
  if (p < 2 || p > SIM_MAX_RANKS || nsteps < 0 || (nsteps > 0 && (!counts || !xfers)) ||
      algo < SIM_ALGO_RING || algo > kLastAlgo || nchunks < 1 || nchunks > p)
    return SIM_ERR_INVALID_ARG;
  Schedule s;
  s.algo = algo;
  s.p = p;
  s.coll = COLL_ALLREDUCE;
  s.nchunks = nchunks;
  s.rounds = rounds;
  if (is_topology_algo(algo)) {
    if (algo == SIM_ALGO_REXCH) s.topo.radix = g_topo.radix;
    else s.topo.ranks_per_node = g_topo.ranks_per_node;
  }
  int k = 0;
  for (int st = 0; st < nsteps; st++) {
    if (counts[st] < 0) return SIM_ERR_INVALID_ARG;
    std::vector<Xfer> v;
    for (int j = 0; j < counts[st]; j++, k++) {
      const int* w = xfers + 5 * (size_t)k;
      if (w[0] < 0 || w[0] >= kNumXferKinds) {
        put_diag("unknown transfer kind", diag, diag_len);
        return SIM_ERR_VERIFY;
      }
      v.push_back({w[0], w[1], w[2], w[3], (uint32_t)w[4]});
    }
    s.steps.push_back(v);
  }
  std::string d;
  const bool ok = verify(s, &d);
  put_diag(d, diag, diag_len);
  return ok ? SIM_OK : SIM_ERR_VERIFY;
}

int sim_debug_set(int key, uint64_t value) {
  switch (key) {
    case SIM_DEBUG_EPOCH: g.epoch = (uint32_t)value; return SIM_OK;
    case SIM_DEBUG_SPIN_LIMIT: g.spin_limit = value; return SIM_OK;
    case SIM_DEBUG_LL_WAIT_SKEW: g.wait_skew = (uint32_t)value; return SIM_OK;
    case SIM_DEBUG_LOG: g.log = value ? 1 : 0; return SIM_OK;
    case SIM_DEBUG_WORKGROUPS: g.force_wg = (int)value; return SIM_OK;
    case SIM_DEBUG_UNROLL:
      if (value > 4 || value == 3) return SIM_ERR_INVALID_ARG;
      g.unroll = (int)value;
      return SIM_OK;
    case SIM_DEBUG_FIFO_CHANNELS:
      if (value > (uint64_t)kFifoMaxChannels) return SIM_ERR_INVALID_ARG;
      g.fifo_channels = (int)value;
      return SIM_OK;
    case SIM_DEBUG_FIFO_WITHHOLD: g.fifo_withhold = value ? 1 : 0; return SIM_OK;
    case SIM_DEBUG_PTR_TABLE: g.ptab_on = value ? 1 : 0; return SIM_OK;
    case SIM_DEBUG_RING_LL_MAX: g.ring_ll_max = (size_t)value; return SIM_OK;
    case SIM_DEBUG_PHASED:
      if (value > 2) return SIM_ERR_INVALID_ARG;
      g.phased_mode = (int)value;
      return SIM_OK;
    case SIM_DEBUG_PHASED_MIN: g.phased_min = (size_t)value; return SIM_OK;
    case SIM_DEBUG_PHASED_LAYOUT:
      if (value > 1) return SIM_ERR_INVALID_ARG;
      g.ph_layout = (int)value;
      return SIM_OK;
    case SIM_DEBUG_PHASED_EXPIRED: {
      if (value != 0) return SIM_ERR_INVALID_ARG;
      if (!g.init) return SIM_ERR_NOT_INIT;
      if (use_device() != SIM_OK || hipDeviceSynchronize() != hipSuccess ||
          hipMemset(g.ph_expired, 0, sizeof(unsigned int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return SIM_ERR_HIP;
      return SIM_OK;
    }
    case SIM_DEBUG_FIFO_VECS:
      if (value != 1 && value != 2 && value != (uint64_t)kFifoVecsPerLane) return SIM_ERR_INVALID_ARG;
      g.fifo_vecs = (int)value;
      return SIM_OK;

    case SIM_DEBUG_FIFO_SLOTS:
      // two slots are the minimum: with one, every rank waits for its
      // successor to consume before sending and the ring deadlocks
      if (value < 2 || value > (uint64_t)kFifoMaxSlots) return SIM_ERR_INVALID_ARG;
      g.fifo_slots = (int)value;
      return SIM_OK;
    case SIM_DEBUG_FILL_LL: {
      if (!g.init) return SIM_ERR_NOT_INIT;
      if (use_device() != SIM_OK) return SIM_ERR_HIP;
      if (launch_fill64(g.ll, (unsigned long long)value, (int64_t)g.p_max * g.ll_stride, nullptr) != hipSuccess)
        return SIM_ERR_HIP;
      return hipDeviceSynchronize() == hipSuccess ? SIM_OK : SIM_ERR_HIP;
    }
  }
  return SIM_ERR_INVALID_ARG;
}

int sim_debug_set_epoch(uint32_t epoch) { return sim_debug_set(SIM_DEBUG_EPOCH, epoch); }

int sim_debug_get(int key, uint64_t* value) {
  if (!value) return SIM_ERR_INVALID_ARG;
  switch (key) {
    case SIM_DEBUG_EPOCH: *value = g.epoch; return SIM_OK;
    case SIM_DEBUG_SPIN_LIMIT: *value = g.spin_limit; return SIM_OK;
    case SIM_DEBUG_LL_WAIT_SKEW: *value = g.wait_skew; return SIM_OK;
    case SIM_DEBUG_LOG: *value = (uint64_t)g.log; return SIM_OK;
    case SIM_DEBUG_WORKGROUPS: *value = (uint64_t)g.force_wg; return SIM_OK;
    case SIM_DEBUG_UNROLL: *value = (uint64_t)g.unroll; return SIM_OK;
    case SIM_DEBUG_FIFO_CHANNELS: *value = (uint64_t)g.fifo_channels; return SIM_OK;
    case SIM_DEBUG_FIFO_WITHHOLD: *value = (uint64_t)g.fifo_withhold; return SIM_OK;
    case SIM_DEBUG_FIFO_VECS: *value = (uint64_t)g.fifo_vecs; return SIM_OK;
    case SIM_DEBUG_FIFO_SLOTS: *value = (uint64_t)g.fifo_slots; return SIM_OK;
    case SIM_DEBUG_PTR_TABLE: *value = (uint64_t)g.ptab_on; return SIM_OK;
    case SIM_DEBUG_PTR_SETS: *value = (uint64_t)g.ptab_index.size(); return SIM_OK;
    case SIM_DEBUG_RING_LL_MAX: *value = (uint64_t)g.ring_ll_max; return SIM_OK;
    case SIM_DEBUG_PHASED: *value = (uint64_t)g.phased_mode; return SIM_OK;
    case SIM_DEBUG_PHASED_MIN: *value = (uint64_t)g.phased_min; return SIM_OK;
    case SIM_DEBUG_PHASED_LAST: *value = g.last_phased ? 1 : 0; return SIM_OK;
    case SIM_DEBUG_PHASED_LAYOUT: *value = (uint64_t)g.ph_layout; return SIM_OK;
    case SIM_DEBUG_PHASED_WHOLE_LAST: *value = g.last_whole ? 1 : 0; return SIM_OK;
    case SIM_DEBUG_PHASED_EXPIRED: {
      if (!g.init) return SIM_ERR_NOT_INIT;
      unsigned int v = 0;
      if (use_device() != SIM_OK || hipDeviceSynchronize() != hipSuccess ||
          hipMemcpy(&v, g.ph_expired, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
        return SIM_ERR_HIP;
      *value = v;
      return SIM_OK;
    }
  }
  return SIM_ERR_INVALID_ARG;
}

}  // extern "C"
