// phased_impl.h -- the phased fold for large messages (gfx950): the one-shot
// all-reduce (every output) and all-pairs step 1 / the direct reduce-scatter
// (the owner's output only), included by k_phased.hip and
// k_phased_owner.hip, which instantiate one output mode each.
//
// It computes exactly what the fused one-shot computes ("MSCCL++ ...",
// section "The Collective Algorithm Library", 1PA: every rank reads every
// rank's data and reduces it in one phase; the fold in the all-pairs order of
// "MSCCL, in depth ...", section "Writing an algorithm in MSCCLang": owner of
// the chunk first, then the other ranks ascending), with the same 2 p S bytes
// -- only the order in which the whole GPU issues them differs.  The fused
// kernel keeps every workgroup reading and writing at once: the p input
// streams and p output streams of all workgroups share HBM the whole time.
// On MI355X that mix moves ~0.71 of the 8 TB/s peak, while the same
// workgroups reading alone reach ~0.87 and writing alone ~0.70 (measured,
// 64 MiB per rank, p = 8).  Here the grid takes turns instead:
//
//   read half:  every workgroup loads its K blocks of all p inputs (16-byte
//               loads, the next blocks' loads in flight while one folds;
//               the chunk's workgroups take its blocks in turn,
//               phase_blocks)
//               and keeps the folded result in VGPRs: K vectors per lane,
//               K * 16 * kBlock bytes per workgroup;
//   grid barrier;
//   write half: every workgroup stores its results to the p outputs, output
//               by output, the workgroups of chunk j starting at output j;
//   grid barrier (before the next phase's reads), and so on.
//
// The grid is persistent (two workgroups per CU, all resident), and a phase
// covers K * kBlock vectors of every workgroup: 64 MiB of results per phase
// on 256 CUs, one phase at 64 MiB per rank with p = 8.  Where every chunk is
// the same whole number of blocks (no fewer than the grid's workgroups), the
// one-shot lays the phases out over the whole buffer instead of chunk by
// chunk (the WHOLE form, see the phase loop).
//
// The barrier is for timing only: every element is read, folded and written
// by one lane, so no workgroup ever reads what another writes, and the
// result does not depend on when (or whether) a barrier opens.  A waiting
// workgroup therefore gives up after the spin limit and carries on (counted
// in *expired; never an error).  The barrier: each workgroup adds 1 to its
// group's arrival counter, the arrival that completes a group's share adds
// 1 to the slot's counter, and the one that completes that count raises
// every workgroup's own flag word (256 bytes apart) to the release value;
// each workgroup's lane 0 polls only its own flag (phased_arrive).  Polling one shared
// counter instead (every waiting workgroup on one address) measured ~29 us
// per barrier against ~4 us: the polls of hundreds of workgroups on one
// memory location slow the reads still in flight.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

namespace {

// result vectors per lane per phase, and load sets in flight while folding
// (with p = 16, 16 vectors per lane: the 16 operands of a fold take 64 VGPRs)
template <int P> struct PhasedShape {
  static constexpr int K = P <= 8 ? 32 : 16;
  static constexpr int D = P >= 16 ? 1 : 16 / P;  // about 16 loads in flight per lane
};

// One arrival per workgroup at each barrier, counted in two levels: at the
// counter of the workgroup's group (workgroup b in group b mod NG, NG =
// min(kPhasedGroups, G), n_g workgroups each), and, by the arrival that
// completes the group's share of a barrier, once at the slot's counter.  A
// group's share of barrier k is complete at its R_g-th arrival, R_g = n_g -
// n_g / 10 (the group's count reaching (k - 1) n_g + R_g); barrier k opens
// when all NG groups have completed theirs (the slot's count reaching k
// NG): that arrival raises every workgroup's flag to seq + k with an
// atomic max, so flags only grow even if a later release overtakes this
// one, and each group's last tenth passes straight through.  Waiting for
// the very last workgroup measured ~1.5% slower at 64 MiB per rank (the
// slowest readers' tail overlaps the first writes instead of idling the
// grid).  A call adds nbar n_g to each group's counter and nbar NG to the
// slot's.  When every wait completes, barrier k opens exactly when every
// group has its R_g-th arrival; after a give-up, workgroups running ahead
// may complete a count early and open a barrier early -- harmless, as the
// barrier guards no data -- and none is left closed, as every count passes
// all its thresholds on its way to its total.  The arrival that opens the
// last barrier also writes done_seq to the host-visible word: from then on
// no workgroup of the grid waits for anything, so another phased grid may
// start beside it.  (One counter for all G arrivals serialized them at
// ~12 ns each -- 512 workgroups, ~6 us per barrier; and workgroups do not
// arrive once more on leaving, which added a second such round to every
// call.)
__device__ __forceinline__ void phased_arrive(const PhasedArgs& a, unsigned long long nbar,
                                              unsigned long long* s_rel) {
  __syncthreads();
  const unsigned G = gridDim.x;
  if (threadIdx.x == 0) {
    const unsigned NG = G < (unsigned)kPhasedGroups ? G : (unsigned)kPhasedGroups;
    const unsigned gi = blockIdx.x % NG;
    const unsigned long long n = G / NG + (gi < G % NG ? 1u : 0u);  // workgroups in this group
    const unsigned long long R = n - n / 10;
    const unsigned long long old = __hip_atomic_fetch_add(a.gctr + (int64_t)gi * kPhasedFlagStride, 1ull,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long done = old + 1 - a.gbase[gi];  // this group's arrivals of this call, this one included
    unsigned long long rel = 0;
    if (done >= R && (done - R) % n == 0) {  // the group's share of a barrier is complete
      const unsigned long long told = __hip_atomic_fetch_add(a.ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long shares = told + 1 - a.base;
      if (shares % NG == 0) {  // every group's: the barrier opens
        const unsigned long long k = shares / NG;
        rel = a.seq + (k < nbar ? k : nbar);
        if (k == nbar) __hip_atomic_store(a.done, a.done_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    *s_rel = rel;
  }
  __syncthreads();
  const unsigned long long rel = *s_rel;
  if (rel) {
    for (unsigned i = threadIdx.x; i < G; i += kBlock)
      __hip_atomic_fetch_max(a.flags + (int64_t)i * kPhasedFlagStride, rel, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// barrier nb of the call: arrive, then wait (lane 0) until this
// workgroup's own flag reaches seq + nb, or the spin limit
__device__ __forceinline__ void phased_barrier(const PhasedArgs& a, unsigned long long nbar, unsigned long long nb,
                                               unsigned long long* s_rel) {
  phased_arrive(a, nbar, s_rel);
  if (threadIdx.x == 0) {
    const unsigned long long want = a.seq + nb;
    unsigned long long spins = 0;
    while (__hip_atomic_load(a.flags + (int64_t)blockIdx.x * kPhasedFlagStride, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < want) {
      if (++spins > a.spin_limit) {
        __hip_atomic_fetch_add(a.expired, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Which of its chunk's blocks (kBlock whole vectors, one per lane) a
// workgroup holds in phase ph.  A chunk has nblk whole blocks and a phase
// takes up to tiles * K of them; the chunk's tiles workgroups interleave
// block by block: the workgroup's block k is block k * tiles + t of the
// phase, so at each step of the write half the chunk's stores cover one
// contiguous range of the output rather than tiles ranges far apart
// (measured on MI355X, p = 8: one-shot 168-171 against 176-177 us at 64 MiB
// per rank, 715-721 against 737-740 us for fp32 at 256 MiB; direct
// reduce-scatter and all-gather 4-6% faster at 64 MiB).  The phase that
// reaches the chunk's end deals its blocks out evenly -- every workgroup
// left / tiles of them, the first left % tiles one more -- so no workgroup
// idles while others hold a full K.  The blocks of every workgroup of every
// phase cover the chunk's first min(nblk, nphase * tiles * K) blocks once.
struct PhaseBlocks {
  int64_t v0;  // the lane-0 vector of the workgroup's first block
  int kv;      // blocks held, 0 ... K (uniform over the workgroup)
};
template <int K>
__device__ __forceinline__ PhaseBlocks phase_blocks(int ph, int t, int tiles, int64_t nblk) {
  const int64_t pblk = (int64_t)tiles * K;  // a chunk's blocks per phase
  const int64_t left = nblk - (int64_t)ph * pblk;
  const int kv = left >= pblk ? K : left <= 0 ? 0 : (int)(left / tiles) + (t < left % tiles ? 1 : 0);
  return {((int64_t)ph * pblk + t) * kBlock, kv};
}

// A workgroup holding kv < K blocks takes them as runs of B = K/2, K/4, ...,
// 1 blocks, one per bit set in kv: the run of B covers blocks k0 ... k0 + B
// - 1 (k0 = the sum of kv's higher bits) and keeps its results in the fixed
// slots K - 2B ... K - B - 1 of the workgroup's K result registers, so every
// register index is a constant and no slot is loaded for nothing.  f is
// called with std::integral_constant<int, B> for B = TOP, TOP/2, ..., 1.
template <int B, class F>
__device__ __forceinline__ void for_each_run(F&& f) {
  if constexpr (B >= 1) {
    f(std::integral_constant<int, B>{});
    for_each_run<B / 2>(f);
  }
}

}  // namespace

// WHOLE (the one-shot only; the host sets a.gblk): the whole-buffer layout
// of a phase's blocks, see the phase loop below.
template <int DT, int OP, int P, bool ALL_OUT, bool WHOLE>
__global__ void __launch_bounds__(kBlock) k_fold_phased(PhasedArgs a) {
  static_assert(ALL_OUT || !WHOLE, "the whole-buffer layout writes every output");
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int V = epv<DT>();
  constexpr int E = Ty<DT>::E;
  constexpr int K = PhasedShape<P>::K;
  // load sets in flight while one folds: about 16 loads per lane, or about 8
  // in the whole-buffer layout, whose register selects per block ran better
  // with fewer sets ahead (p = 8 on MI355X, one set against two: 169.5
  // against 171.8-172.4 us at 64 MiB per rank, 337 against 343 us at 128 MiB,
  // fp32 at 32 MiB 89.5-90.3 against 93.4-93.6 us)
  constexpr int D = WHOLE ? (P >= 8 ? 1 : 8 / P) : PhasedShape<P>::D;
  const int j = (int)(blockIdx.x % (unsigned)P);
  const int t = (int)(blockIdx.x / (unsigned)P);
  const int64_t lo = a.lo[j], hi = a.lo[j + 1];
  const float inv_p = a.inv_p;
  __shared__ unsigned long long s_rel;

  // operand k of the fold: rank j for k == 0, then the ranks != j ascending.
  // The whole-buffer layout loads the ranks in their own order and puts each
  // block's operands in its chunk's order in registers (fold_in below).
  const void* xp[P];
#pragma unroll
  for (int k = 0; k < P; k++) xp[k] = WHOLE ? a.x[k] : a.x[(k == 0) ? j : (k <= j ? k - 1 : k)];
  // outputs: every rank's, or (owner-only) rank j's, element i at i - shift
  void* yp[ALL_OUT ? P : 1];
#pragma unroll
  for (int r = 0; r < (ALL_OUT ? P : 1); r++) yp[r] = a.y[ALL_OUT ? r : j];
  const int64_t oshift = ALL_OUT ? 0 : a.out_shift[j];

  // chunk j: scalar head up to the first 16-byte boundary, whole vectors,
  // scalar tail (every pointer is 16-byte aligned)
  int64_t head = (V - lo % V) % V;
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const uint32_t lane = lane_offset((uint32_t)tid * 16u);

  auto fold = [&](const u32x4* L) {
    A acc[V], tt[V];
    unpack<DT>(L[0], acc);
#pragma unroll
    for (int e = 0; e < V; e++) acc[e] = O::pre(acc[e], inv_p);
#pragma unroll
    for (int k = 1; k < P; k++) {
      unpack<DT>(L[k], tt);
#pragma unroll
      for (int e = 0; e < V; e++) acc[e] = O::comb(acc[e], O::pre(tt[e], inv_p));
    }
#pragma unroll
    for (int e = 0; e < V; e++) acc[e] = O::post(acc[e], P);
    return pack<DT>(acc);
  };
  // the same fold of a block of chunk c whose operands L[q] are rank q's:
  // rank c first, then the ranks != c ascending (c uniform: every select is
  // one v_cndmask per dword on a scalar condition)
  auto fold_in = [&](const u32x4* L, int c) {
    u32x4 Lc[P];
    Lc[0] = L[0];
#pragma unroll
    for (int q = 1; q < P; q++) Lc[0] = (q == c) ? L[q] : Lc[0];
#pragma unroll
    for (int k = 1; k < P; k++) Lc[k] = (k - 1 < c) ? L[k - 1] : L[k];
    return fold(Lc);
  };

  // read B blocks, k0 ... k0 + B - 1, into R[S0 ... S0 + B - 1]: D sets of
  // p loads in flight while one set folds.  The scheduling barriers keep
  // each set's p loads issued together, ahead of the fold that follows:
  // without them the compiler interleaved the 32-bit folds with their own
  // loads, waiting on every load (1-3 in flight per wave instead of ~16; the
  // fp32 phased reduce-scatter ran 1.5x slower than the bf16 one).
  // chunk_of(k): the chunk of the workgroup's block k of the phase (WHOLE)
  auto read_run = [&](auto b_tag, auto s_tag, u32x4* R, int64_t sbyte, int64_t kst, int k0, auto&& chunk_of)
                      __attribute__((always_inline)) {
    constexpr int B = decltype(b_tag)::value, S0 = decltype(s_tag)::value;
    constexpr int DR = D < B ? D : B;
    u32x4 L[DR][P];
#pragma unroll
    for (int d = 0; d < DR; d++)
#pragma unroll
      for (int q = 0; q < P; q++) L[d][q] = ld16u(xp[q], sbyte + (int64_t)(k0 + d) * kst, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < B; i++) {
      if constexpr (WHOLE)
        R[S0 + i] = fold_in(L[i % DR], chunk_of(k0 + i));
      else
        R[S0 + i] = fold(L[i % DR]);
      if (i + DR < B) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < P; q++) L[i % DR][q] = ld16u(xp[q], sbyte + (int64_t)(k0 + i + DR) * kst, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // store R[S0 ... S0 + B - 1] to blocks k0 ... k0 + B - 1 of one output
  auto write_run = [&](auto b_tag, auto s_tag, const u32x4* R, void* y, int64_t obyte, int64_t kst, int k0)
                       __attribute__((always_inline)) {
    constexpr int B = decltype(b_tag)::value, S0 = decltype(s_tag)::value;
#pragma unroll
    for (int i = 0; i < B; i++) st16u(y, obyte + (int64_t)(k0 + i) * kst, lane, R[S0 + i]);
  };
  // every block the workgroup holds in the phase, as one run of K or as the
  // runs of kv's bits (for_each_run)
  auto runs = [&](int kv, auto&& run) __attribute__((always_inline)) {
    if (kv == K) {
      run(std::integral_constant<int, K>{}, std::integral_constant<int, 0>{}, 0);
    } else if (kv > 0) {
      for_each_run<K / 2>([&](auto b_tag) __attribute__((always_inline)) {
        constexpr int B = decltype(b_tag)::value;
        if (kv & B) run(b_tag, std::integral_constant<int, K - 2 * B>{}, kv & ~(2 * B - 1));
      });
    }
  };

  // The layout of a phase's blocks.  Per chunk: workgroup (j, t) holds
  // blocks of chunk j, the chunk's workgroups taking its blocks in turn, so
  // each step of the write half covers p ranges of tiles blocks, a chunk
  // apart.  WHOLE (the one-shot, when every chunk is the same whole number
  // of blocks, no fewer than the grid's G workgroups): the grid takes the
  // whole buffer's blocks in turn, workgroup (j, t) at turn j tiles + t (so
  // each XCD's workgroups hold neighbouring blocks), and each step of the
  // write half covers one range of G blocks.  Each block keeps its own
  // chunk's fold order.  Measured on MI355X (p = 8, bf16, 64 MiB per rank,
  // same run): 170.0-170.5 against 174.3-174.8 us per call.
  const int G = a.tiles * P;
  const int lt = WHOLE ? G : a.tiles;                   // workgroups taking turns
  const int lpos = WHOLE ? j * a.tiles + t : t;         // this workgroup's turn
  const int64_t lblk = WHOLE ? a.gblk : nvec / kBlock;  // whole blocks laid out
  const int64_t lbyte = WHOLE ? 0 : vbeg * E;           // byte of the first
  const unsigned long long nbar = a.nphase > 0 ? 2ull * a.nphase - 1 : 0ull;  // barriers of this call
  unsigned long long nb = 0;
  const int64_t kst = (int64_t)lt * kBlock * 16;  // bytes from one of a workgroup's blocks to the next
  for (int ph = 0; ph < a.nphase; ph++) {
    const PhaseBlocks pb = phase_blocks<K>(ph, lpos, lt, lblk);
    const int64_t sbyte = lbyte + pb.v0 * 16;  // this workgroup's first block of the phase
    // WHOLE: the chunk of the workgroup's block k is c0 plus the bits of inc
    // up to k (its blocks are G apart and a chunk holds at least G blocks,
    // so the chunk grows by at most one from a block to the next)
    int c0 = 0;
    uint32_t inc = 0;
    if constexpr (WHOLE) {
      if (pb.kv > 0) {
        const int64_t g0 = pb.v0 / kBlock;
        c0 = (int)(g0 / a.gbpc);
        int64_t r = g0 - (int64_t)c0 * a.gbpc;
        for (int k = 1; k < pb.kv; k++) {
          r += G;
          if (r >= a.gbpc) {
            r -= a.gbpc;
            inc |= 1u << k;
          }
        }
      }
    }
    auto chunk_of = [&](int k) __attribute__((always_inline)) {
      return c0 + __builtin_popcount(inc & (0xFFFFFFFFu >> (31 - k)));
    };
    u32x4 R[K];  // the phase's results, in VGPRs from the read half to the write half
    runs(pb.kv, [&](auto b_tag, auto s_tag, int k0) __attribute__((always_inline)) {
      read_run(b_tag, s_tag, R, sbyte, kst, k0, chunk_of);
    });
    phased_barrier(a, nbar, ++nb, &s_rel);
    // write half: output by output; the workgroups of chunk j start at
    // output j, so at any moment each output takes one chunk's stores
    if constexpr (ALL_OUT) {
#pragma unroll
      for (int rr = 0; rr < P; rr++) {
        const int r = (rr + j) & (P - 1);  // P is a power of two
        void* yr = yp[0];
#pragma unroll
        for (int q = 1; q < P; q++)
          if (q == r) yr = yp[q];
        runs(pb.kv, [&](auto b_tag, auto s_tag, int k0) __attribute__((always_inline)) {
          write_run(b_tag, s_tag, R, yr, sbyte, kst, k0);
        });
      }
    } else {
      const int64_t obyte = sbyte - oshift * E;  // 16-byte aligned: the host checks oshift % V == 0
      runs(pb.kv, [&](auto b_tag, auto s_tag, int k0) __attribute__((always_inline)) {
        write_run(b_tag, s_tag, R, yp[0], obyte, kst, k0);
      });
    }
    if (ph + 1 < a.nphase) phased_barrier(a, nbar, ++nb, &s_rel);
  }

  if constexpr (WHOLE) return;  // every element sits in a whole block of the layout

  // the chunk's vectors past the blocks the phases hold (less than a block
  // when the grid runs enough phases), read, folded and written vector by
  // vector by all of the chunk's workgroups
  const int64_t nblk = nvec / kBlock;
  const int64_t held = (int64_t)a.nphase * a.tiles * K;
  for (int64_t v = (nblk < held ? nblk : held) * kBlock + (int64_t)t * kBlock + tid; v < nvec;
       v += (int64_t)a.tiles * kBlock) {
    const int64_t vb = (vbeg + v * V) * E;
    u32x4 L[P];
#pragma unroll
    for (int q = 0; q < P; q++) L[q] = ld16(xp[q], vb);
    const u32x4 out = fold(L);
    if constexpr (ALL_OUT) {
#pragma unroll
      for (int r = 0; r < P; r++) st16(yp[r], vb, out);
    } else {
      st16(yp[0], vb - oshift * E, out);
    }
  }

  // ragged chunk edges, element by element, in the same fold order
  for (int64_t s = (int64_t)t * kBlock + tid; s < nscalar; s += (int64_t)a.tiles * kBlock) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    A acc = O::pre(load_elem<DT>(xp[0], i), inv_p);
#pragma unroll
    for (int k = 1; k < P; k++) acc = O::comb(acc, O::pre(load_elem<DT>(xp[k], i), inv_p));
    acc = O::post(acc, P);
    if constexpr (ALL_OUT) {
#pragma unroll
      for (int r = 0; r < P; r++) store_elem<DT>(yp[r], i, acc);
    } else {
      store_elem<DT>(yp[0], i - oshift, acc);
    }
  }

}

namespace {

template <int DT, int OP, bool ALL_OUT, bool WHOLE>
hipError_t phased_by_p(int p, const PhasedArgs& a, hipStream_t s) {
  const dim3 g((unsigned)a.tiles * (unsigned)p), b(kBlock);
  switch (p) {
    case 2: return launch<k_fold_phased<DT, OP, 2, ALL_OUT, WHOLE>>(g, b, s, a);
    case 4: return launch<k_fold_phased<DT, OP, 4, ALL_OUT, WHOLE>>(g, b, s, a);
    case 8: return launch<k_fold_phased<DT, OP, 8, ALL_OUT, WHOLE>>(g, b, s, a);
    case 16: return launch<k_fold_phased<DT, OP, 16, ALL_OUT, WHOLE>>(g, b, s, a);
  }
  return hipErrorInvalidValue;
}

template <int DT, bool ALL_OUT, bool WHOLE>
hipError_t phased_by_op(int op, int p, const PhasedArgs& a, hipStream_t s) {
  switch (op) {
    case SIM_SUM: return phased_by_p<DT, SIM_SUM, ALL_OUT, WHOLE>(p, a, s);
    case SIM_PROD: return phased_by_p<DT, SIM_PROD, ALL_OUT, WHOLE>(p, a, s);
    case SIM_MIN: return phased_by_p<DT, SIM_MIN, ALL_OUT, WHOLE>(p, a, s);
    case SIM_MAX: return phased_by_p<DT, SIM_MAX, ALL_OUT, WHOLE>(p, a, s);
    case SIM_AVG: return phased_by_p<DT, SIM_AVG, ALL_OUT, WHOLE>(p, a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int OP, int P, bool ALL_OUT, bool WHOLE>
int occ_of() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)k_fold_phased<DT, OP, P, ALL_OUT, WHOLE>,
                                                   kBlock, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return nb;
}

template <int DT, int OP, bool ALL_OUT, bool WHOLE>
int occ_by_p(int p) {
  switch (p) {
    case 2: return occ_of<DT, OP, 2, ALL_OUT, WHOLE>();
    case 4: return occ_of<DT, OP, 4, ALL_OUT, WHOLE>();
    case 8: return occ_of<DT, OP, 8, ALL_OUT, WHOLE>();
    case 16: return occ_of<DT, OP, 16, ALL_OUT, WHOLE>();
  }
  return 0;
}

template <int DT, bool ALL_OUT, bool WHOLE>
int occ_by_op(int op, int p) {
  switch (op) {
    case SIM_SUM: return occ_by_p<DT, SIM_SUM, ALL_OUT, WHOLE>(p);
    case SIM_PROD: return occ_by_p<DT, SIM_PROD, ALL_OUT, WHOLE>(p);
    case SIM_MIN: return occ_by_p<DT, SIM_MIN, ALL_OUT, WHOLE>(p);
    case SIM_MAX: return occ_by_p<DT, SIM_MAX, ALL_OUT, WHOLE>(p);
    case SIM_AVG: return occ_by_p<DT, SIM_AVG, ALL_OUT, WHOLE>(p);
  }
  return 0;
}

}  // namespace

// the launcher and occupancy query of one output mode and layout (every
// dtype, op and p)
template <bool ALL_OUT, bool WHOLE>
hipError_t phased_launch(int dtype, int op, int p, const PhasedArgs& a, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return phased_by_op<SIM_INT32, ALL_OUT, WHOLE>(op, p, a, s);
    case SIM_FP32: return phased_by_op<SIM_FP32, ALL_OUT, WHOLE>(op, p, a, s);
    case SIM_FP16: return phased_by_op<SIM_FP16, ALL_OUT, WHOLE>(op, p, a, s);
    case SIM_BF16: return phased_by_op<SIM_BF16, ALL_OUT, WHOLE>(op, p, a, s);
  }
  return hipErrorInvalidValue;
}

template <bool ALL_OUT, bool WHOLE>
int phased_occupancy(int dtype, int op, int p) {
  switch (dtype) {
    case SIM_INT32: return occ_by_op<SIM_INT32, ALL_OUT, WHOLE>(op, p);
    case SIM_FP32: return occ_by_op<SIM_FP32, ALL_OUT, WHOLE>(op, p);
    case SIM_FP16: return occ_by_op<SIM_FP16, ALL_OUT, WHOLE>(op, p);
    case SIM_BF16: return occ_by_op<SIM_BF16, ALL_OUT, WHOLE>(op, p);
  }
  return 0;
}

}  // namespace simar
