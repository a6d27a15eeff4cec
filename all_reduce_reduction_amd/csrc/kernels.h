// kernels.h -- kernel argument blocks and host-side launchers shared by the
// C-ABI layer (api.cpp) and the gfx950 kernels (k_*.hip).
//
// Every argument block is passed by value as the kernel's argument segment
// (at most 4 KiB).  Element indices are absolute within a rank's buffer;
// an operand with a `shift` is addressed at [i - shift] (chunk-sized outputs
// and scratch slots).  `vec_ok` says the 16-byte vector body is aligned for
// every operand of that transfer; otherwise the transfer runs element by
// element (only for ragged sizes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "simar.h"

namespace simar {

constexpr int kBlock = 256;  // threads per workgroup (4 wavefronts of 64)

// The device the library launches on (the one sim_init chose).  Launches
// keep their kernel handles per device index, up to kMaxDevices devices.
constexpr int kMaxDevices = 64;
extern int g_launch_device;

// Gather-fold of whole chunks: the fused one-shot (every rank's output
// written from the same registers) or all-pairs step 1 / direct
// reduce-scatter (only the owner's output written).
struct FoldArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  int64_t lo[SIM_MAX_RANKS + 1];     // chunk bounds
  int64_t out_shift[SIM_MAX_RANKS];  // owner-only mode: y[j] index = i - out_shift[j]
  uint32_t vec_ok;                   // bit j: chunk j may use the vector body
  int p;
  int tiles;                         // workgroups per chunk (gridDim.x)
  float inv_p;                       // fp32(1/p) for fp avg
};

// The fused one-shot (and all-pairs step 1) with its rank pointers in device memory: one entry of
// the library's pointer table, written (in stream order) before the first
// launch that uses it.  The argument block then fits the HIP runtime's
// small-argument launch path (<= 64 bytes), which measured ~1 us cheaper
// per launch on MI355X than argument blocks of 128 bytes or more.  Chunk j
// is [floor(j n / p), floor((j+1) n / p)), computed in the kernel.
struct PtrSet {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
};
struct FoldTabArgs {
  const PtrSet* set;  // device memory
  int64_t n;          // elements per rank (< 2^46)
  int p;
  int tiles;          // workgroups per chunk
  float inv_p;        // fp32(1/p) for fp avg
};
// The all-pairs fan-out (step 2) from the same table entry: chunk j of the
// owner's output y[j] to every other rank's output.
struct FanoutTabArgs {
  const PtrSet* set;
  int64_t n;
  int p;
  int tiles;
};
// One step of the all-reduce ring from the same table entry: the step's
// transfers follow from the step number (reduce-scatter step s: rank r
// sends chunk (r - 1 - s) mod p to r + 1; all-gather step s: rank r
// forwards chunk (r - s) mod p).
struct RingTabArgs {
  const PtrSet* set;
  void* scratch;       // fp16/bf16 partial slots [2][p][slot_elems] fp32; nullptr: partials in the outputs
  int64_t n;
  int64_t slot_elems;
  int p;
  int step;
  int tiles;
  float inv_p;
};

// One ring reduce-scatter step: p transfers, each over one chunk.
struct RingXfer {
  const void* a;    // running value from the predecessor: an input (first step) or a partial
  int64_t a_shift;
  const void* b;    // the receiving rank's own input, absolute index
  void* d;          // partial (not last step) or output (last step)
  int64_t d_shift;
  int64_t lo, hi;
  int vec_ok;
  int pad_;
};
struct RingArgs {
  RingXfer x[SIM_MAX_RANKS];
  int nx;
  int p;
  int tiles;
  float inv_p;
};

// Bit copies: ring all-gather forwards, all-pairs fan-out, all-gather.
struct CopyXfer {
  const void* src;
  int64_t src_shift;
  void* dst[SIM_MAX_RANKS];
  int64_t dst_shift;
  int64_t lo, hi;
  int ndst;
  int vec_ok;
};
struct CopyArgs {
  CopyXfer x[SIM_MAX_RANKS];
  int nx;
  int tiles;
};

// LL packet one-shot: producers write 8-byte {data, flag} packets, the
// consumers poll them and fold.
struct LLArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  unsigned long long* ll;   // packets: rank q's word k at ll[q * ll_stride + k]
  int64_t ll_stride;
  int64_t n;                // elements per rank
  int64_t nwords;           // 32-bit data words per rank
  int64_t lo[SIM_MAX_RANKS + 1];
  int64_t tile_words;       // words per tile (one workgroup's share)
  int64_t ntiles;
  unsigned long long spin_limit;
  int* err;                 // device error word
  int p;
  unsigned int epoch;       // flag the producers write
  unsigned int wait_epoch;  // flag the consumers accept (== epoch unless a test skews it)
  int shift;                // consumers take tile (t + shift) mod ntiles
  float inv_p;
};

// Single-launch ring: p * C persistent workgroups (grid p * Cg, rank-major),
// bounded FIFOs between neighbouring ranks, epoch-tagged monotonic
// semaphores.  A FIFO slot holds kBlock * U 16-byte vectors' worth of
// elements (one 32-bit word per element), U = 1, 2 or kFifoVecsPerLane:
// up to 8192 elements for 16-bit types, 4096 for 32-bit.
constexpr int kFifoVecsPerLane = 4;
constexpr int kFifoMaxSlotElems = kBlock * kFifoVecsPerLane * 8;
struct RingFifoArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  int64_t lo[SIM_MAX_RANKS + 1];
  uint32_t* fifo;              // [p][C][NS][slot_elems] 32-bit words
  unsigned long long* sem;     // [p][C][2]: posted, consumed
  int* err;
  unsigned long long spin_limit;
  int p;
  int C;                       // channels per rank
  int Cg;                      // channels in the grid: C rounded up to a multiple of 8 (rank-major grid)
  int NS;                      // slots per FIFO
  int nsub;                    // slots per channel slice of a chunk
  int slot_elems;              // kBlock * kFifoVecsPerLane * (16 / element bytes)
  unsigned int epoch;
  float inv_p;
  int withhold;                // test hook: rank 0 leaves at once, its partners' waits expire
};

// The single-launch ring with LL packets (small messages): p * C persistent
// workgroups, rank-major grid.  Every value that crosses from rank r to
// rank r+1 -- a partial of the reduce-scatter half (fp32 / int32 bits) or a
// finished element of the all-gather half (storage bits) -- travels as one
// 8-byte packet {low 32 bits payload, high 32 bits epoch} in the receiver's
// region of the LL buffer: send k (0 <= k < 2p-2) of chunk offset o at
// ll[(r+1) * ll_stride + k * maxchunk + o].  No counters: the receiver
// polls the packets themselves.
struct RingLLArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  int64_t lo[SIM_MAX_RANKS + 1];
  unsigned long long* ll;
  int64_t ll_stride;           // packets per rank region
  int64_t maxchunk;            // longest chunk (packets per send)
  unsigned long long spin_limit;
  int* err;
  int p;
  int C;                       // channels per rank
  int Cg;                      // channels in the grid (rank-major, C rounded up to a multiple of 8 when it fits)
  unsigned int epoch;          // flag the senders write
  unsigned int wait_epoch;     // flag the receivers accept (== epoch unless a test skews it)
  float inv_p;
  int withhold;                // test hook: rank 0 leaves at once, its partners' waits expire
};

// The all-pairs schedule in ONE launch: p * C persistent workgroups.
// Workgroup (rank r, channel c) folds its slice of chunk r from every
// rank's input into Y[r] (owner first, then ascending) and signals; then,
// for every other owner j, it waits for (j, c)'s signal and copies that
// slice of Y[j] into Y[r].
struct AllPairsPArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  int64_t lo[SIM_MAX_RANKS + 1];
  unsigned long long* sem;     // ready counter of (r, c) = word (r * C + c) * 2 (the ring's semaphore array)
  int* err;
  unsigned long long spin_limit;
  int p;
  int C;                       // channels per rank
  int Cg;                      // channels in the grid (C rounded up to a multiple of 8: rank-major grid)
  unsigned int epoch;
  float inv_p;
  int withhold;                // test hook: rank 0 leaves at once, its partners' waits expire
};
constexpr int kAllPairsPVecsPerLane = 2;  // 16-byte vectors per lane per pass

// One step of the tree, recursive-exchange and 2PH schedules: a set of
// folds, each over one chunk.  A fold's operands are ranks' current values
// in fold order -- an input (widened, avg-scaled as it is read) or an
// accumulator-typed partial -- and its result goes to every rank in
// `dmask`: post-processed and narrowed into the outputs, or as a partial.
constexpr int kSchedMaxXfers = 32;
struct SchedXfer {
  int64_t lo, hi;      // element range (a chunk)
  uint64_t order;      // operand ranks in fold order, 4 bits each
  uint32_t from_part;  // bit k: operand k is a partial
  uint32_t dmask;      // ranks that receive the result
  int nsrc;            // operands, 1..SIM_MAX_RANKS
  int final_;          // 1: post-processed output; 0: partial
};
struct SchedArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  void* part[SIM_MAX_RANKS];  // accumulator-typed partials, absolute element index, 16-byte aligned
  SchedXfer xf[kSchedMaxXfers];
  int nx;
  int p;
  int tiles;                  // workgroups per fold (gridDim.x = tiles * nx)
  float inv_p;
};

// k independent streaming copies (the ceiling of the one-shot's access
// pattern): dst[q][0 .. 16 nvec) = src[q][0 .. 16 nvec) for q < k.
// The phased kernels (k_phased.hip, k_phased_owner.hip, k_phased_gather.hip):
// the grid loads (and folds) a phase's blocks into VGPRs, meets at a grid
// barrier, writes them out, and meets again before the next phase.  Barrier state lives in one of kPhasedSlots slots (the
// host takes them in turn, call by call): a counter, one release flag per
// workgroup and kPhasedGroups group counters, kPhasedFlagStride 64-bit
// words (256 bytes) apart.
constexpr int kPhasedSlots = 4;
constexpr int kPhasedFlagStride = 32;
// Arrivals count first per group of workgroups (workgroup b in group b mod
// kPhasedGroups), each group on its own counter; the arrival that completes
// a group's share of a barrier then counts once at the slot's counter.
// Arrivals at one counter serialize (~12 ns each on MI355X), so 512
// workgroups on one counter took ~6 us per barrier.
constexpr int kPhasedGroups = 8;
struct PhasedArgs {
  const void* x[SIM_MAX_RANKS];
  void* y[SIM_MAX_RANKS];
  int64_t lo[SIM_MAX_RANKS + 1];  // chunk bounds
  int64_t out_shift[SIM_MAX_RANKS];  // owner-only mode: y[j] index = i - out_shift[j] (a multiple of 16 bytes)
  unsigned long long* ctr;        // the slot's counter: groups' completed shares
  unsigned long long* flags;      // the slot's release flags
  unsigned long long* gctr;       // the slot's group counters, kPhasedFlagStride words apart
  unsigned long long gbase[kPhasedGroups];  // the group counters' values when this call starts
  unsigned long long base;        // the slot counter's value when this call starts
  unsigned long long seq;         // the flags' value when this call starts
  unsigned long long spin_limit;  // polls before a barrier wait gives up
  unsigned int* expired;          // barrier waits that gave up (timing only, not an error)
  unsigned long long* done;       // host-visible word: the opener of the last barrier writes done_seq
  unsigned long long done_seq;
  int64_t gblk;                   // the one-shot's whole-buffer layout: the buffer's blocks (0: per chunk)
  int64_t gbpc;                   // whole-buffer layout: blocks per chunk (every chunk the same, >= the grid)
  int tiles;                      // workgroups per chunk (grid = tiles * p)
  int nphase;
  float inv_p;
  int pad_;
};

struct CopyStreamsArgs {
  const void* src[SIM_MAX_RANKS];
  void* dst[SIM_MAX_RANKS];
  int64_t nvec;  // 16-byte vectors per stream
  int k;
  int pad_;
};

static_assert(sizeof(FoldArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(CopyStreamsArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(PhasedArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(FoldTabArgs) <= 64, "must fit the small-argument launch path");
static_assert(sizeof(FanoutTabArgs) <= 64, "must fit the small-argument launch path");
static_assert(sizeof(RingTabArgs) <= 64, "must fit the small-argument launch path");
static_assert(sizeof(SchedArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(RingFifoArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(RingLLArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(AllPairsPArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(RingArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(CopyArgs) <= 4096, "kernel argument segment too large");
static_assert(sizeof(LLArgs) <= 4096, "kernel argument segment too large");

// Launchers: select the (dtype, op, ...) instantiation and enqueue.
hipError_t launch_fold(int dtype, int op, int p, bool all_out, const FoldArgs& a, int unroll,
                       hipStream_t s);
// all_out: the one-shot (every output); otherwise all-pairs step 1 (the owner's output only)
hipError_t launch_fold_tab(int dtype, int op, int p, bool all_out, const FoldTabArgs& a, int unroll, hipStream_t s);
hipError_t launch_fanout_tab(int esize, const FanoutTabArgs& a, int unroll, hipStream_t s);
hipError_t launch_ring_reduce_tab(int dtype, int op, bool a_partial, bool d_final, const RingTabArgs& a,
                                  int unroll, hipStream_t s);
hipError_t launch_ring_copy_tab(int esize, const RingTabArgs& a, int unroll, hipStream_t s);
hipError_t launch_ring_reduce(int dtype, int op, bool a_partial, bool d_final, const RingArgs& a,
                              int unroll, hipStream_t s);
hipError_t launch_copy(int esize, const CopyArgs& a, int unroll, hipStream_t s);
hipError_t launch_ll(int dtype, int op, const LLArgs& a, int grid, hipStream_t s);
hipError_t launch_copy_streams(const CopyStreamsArgs& a, int workgroups, hipStream_t s);
// The fixed scratch array of sim_allreduce_noalloc (noalloc.hip): look up its
// device address once per device, with that device current (SIM_OK or
// SIM_ERR_HIP), and read it back (nullptr before the lookup).
int noalloc_setup(int device);
void* noalloc_scratch(int device);
hipError_t launch_fill64(unsigned long long* p, unsigned long long v, int64_t n, hipStream_t s);
// Workgroups of the LL kernel (dtype, op) that fit on one CU at once.
int ll_blocks_per_cu(int dtype, int op);
hipError_t launch_ring_fifo(int dtype, int op, const RingFifoArgs& a, hipStream_t s);
hipError_t launch_sched_fold(int dtype, int op, const SchedArgs& a, hipStream_t s);
int ring_fifo_blocks_per_cu(int dtype, int op);
hipError_t launch_ring_ll(int dtype, int op, const RingLLArgs& a, hipStream_t s);
int ring_ll_blocks_per_cu(int dtype, int op);
hipError_t launch_allpairs_persistent(int dtype, int op, const AllPairsPArgs& a, hipStream_t s);
int allpairs_persistent_blocks_per_cu(int dtype, int op, int p);
// The phased fold for p = 2, 4, 8 or 16 (hipErrorInvalidValue otherwise):
// every output (the one-shot) or the owner's (all-pairs step 1, the direct
// reduce-scatter); its resident workgroups per CU, and its result vectors
// per lane per phase.
hipError_t launch_fold_phased(int dtype, int op, int p, bool all_out, const PhasedArgs& a, hipStream_t s);
// whole: the one-shot's whole-buffer layout (PhasedArgs::gblk > 0)
int fold_phased_blocks_per_cu(int dtype, int op, int p, bool all_out, bool whole = false);
int fold_phased_vecs_per_lane(int p);
// The phased copy (k_phased_gather.hip; out_shift unused, lo the output
// blocks, x[j] - lo[j] the source of block j indexed by output element):
// the direct all-gather (every output), or with skip_own the all-pairs
// fan-out (every output but j).
hipError_t launch_gather_phased(int esize, int p, bool skip_own, const PhasedArgs& a, hipStream_t s);
int gather_phased_blocks_per_cu(int esize, int p, bool skip_own);
// WHOLE: the one-shot's whole-buffer layout (only with ALL_OUT)
template <bool ALL_OUT, bool WHOLE>
hipError_t phased_launch(int dtype, int op, int p, const PhasedArgs& a, hipStream_t s);
template <bool ALL_OUT, bool WHOLE>
int phased_occupancy(int dtype, int op, int p);

}  // namespace simar
