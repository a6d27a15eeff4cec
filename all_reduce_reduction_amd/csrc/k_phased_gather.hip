// k_phased_gather.hip -- the direct all-gather and the all-pairs fan-out
// for large messages, phased (gfx950).
//
// The all-gather of "Inside NCCL all-reduce" (section "What all-reduce
// promises": reduce-scatter then all-gather; the all-gather alone gives every
// rank every rank's block): out[r][q n_in + i] = in[q][i].  Done directly it
// reads each block once and writes it p times, (p + 1) S bytes with S = the
// output per rank, almost all of them writes.  The phased form (the grid
// barrier and its slots are those of the phased fold, phased_impl.h): the
// grid's workgroups load their parts of the source blocks (laid out as the
// phased fold's, phase_span) into VGPRs -- 32
// (16 at p = 16) 16-byte vectors per lane, all in flight at once, no
// arithmetic -- meet at the grid barrier, then store them to the p outputs
// output by output (the workgroups of block j starting at output j), and
// meet again before the next phase.  Measured against the fused copy
// (one load, p stores per vector, every workgroup reading and writing at
// once) in the all-gather's own section of the design notes.
#include "phased_impl.h"

namespace simar {

namespace {

// Where a workgroup's K vectors per lane lie in phase ph of its block (nvec
// whole vectors, tiles workgroups, span = kBlock * K vectors each).  While
// the whole phase lies inside the block, the workgroups interleave as the
// phased fold's do (phase_blocks): the workgroup's k-th group of kBlock
// vectors is group k * tiles + t of the phase.  The phase that reaches the
// block's end gives each workgroup one contiguous span, used only if whole,
// and the vectors past the last whole span are copied one by one after the
// phases: the phases' whole spans cover exactly the block's first
// floor(nvec / span) * span vectors.  (Dealing that last phase out evenly,
// as the fold does, needs loads the workgroup may skip; the compiler then
// waited for every earlier access before each store -- one store in flight
// per wave -- and the all-gather at 64 MiB per rank ran 7% slower.)
struct PhaseSpan {
  int64_t v0;       // the lane-0 vector of the workgroup's first group
  int64_t vstride;  // vectors from one of its groups to the next
  bool whole;       // all K groups inside the block (uniform over the workgroup)
};
__device__ __forceinline__ PhaseSpan phase_span(int ph, int t, int tiles, int64_t nvec, int64_t span) {
  const int64_t ptile = (int64_t)tiles * span;  // a block's vectors per phase
  if ((int64_t)(ph + 1) * ptile <= nvec)
    return {(int64_t)ph * ptile + (int64_t)t * kBlock, (int64_t)tiles * kBlock, true};
  const int64_t s0 = ((int64_t)ph * tiles + t) * span;
  return {s0, (int64_t)kBlock, s0 + span <= nvec};
}

}  // namespace

// E: element bytes (the copy moves 16-byte vectors; E matters for the chunk
// bounds and the ragged edges only)
// SKIP_OWN: the all-pairs fan-out (step 2): block j is owner j's finished
// chunk, already in output j, copied to the other p - 1 outputs only.
template <int E, int P, bool SKIP_OWN>
__global__ void __launch_bounds__(kBlock) k_gather_phased(PhasedArgs a) {
  typedef typename std::conditional<E == 4, uint32_t, uint16_t>::type U;
  constexpr int V = 16 / E;
  constexpr int K = PhasedShape<P>::K;
  const int j = (int)(blockIdx.x % (unsigned)P);
  const int t = (int)(blockIdx.x / (unsigned)P);
  // output block j = [lo, hi) holds source rank j's input, element i of the
  // block at index i - lo of that input (lo is a multiple of V: the host
  // checks, so input and output offsets are both 16-byte aligned)
  const int64_t lo = a.lo[j], hi = a.lo[j + 1];
  const char* xj = (const char*)a.x[j] - lo * E;  // indexed by output element (only bytes >= lo*E are touched)
  __shared__ unsigned long long s_rel;
  void* yp[P];
#pragma unroll
  for (int r = 0; r < P; r++) yp[r] = a.y[r];

  int64_t head = (V - lo % V) % V;
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const int64_t span = (int64_t)kBlock * K;
  const uint32_t lane = lane_offset((uint32_t)tid * 16u);

  const unsigned long long nbar = a.nphase > 0 ? 2ull * a.nphase - 1 : 0ull;
  unsigned long long nb = 0;
  for (int ph = 0; ph < a.nphase; ph++) {
    const PhaseSpan sp = phase_span(ph, t, a.tiles, nvec, span);
    const int64_t sbyte = vbeg * E + sp.v0 * 16;
    const int64_t kst = sp.vstride * 16;
    const bool whole = sp.whole;
    u32x4 R[K];
    if (whole) {
#pragma unroll
      for (int k = 0; k < K; k++) R[k] = ld16u(xj, sbyte + (int64_t)k * kst, lane);
    }
    phased_barrier(a, nbar, ++nb, &s_rel);
    if (whole) {
#pragma unroll
      for (int rr = SKIP_OWN ? 1 : 0; rr < P; rr++) {
        const int r = (rr + j) & (P - 1);
        void* yr = yp[0];
#pragma unroll
        for (int q = 1; q < P; q++)
          if (q == r) yr = yp[q];
#pragma unroll
        for (int k = 0; k < K; k++) st16u(yr, sbyte + (int64_t)k * kst, lane, R[k]);
      }
    }
    if (ph + 1 < a.nphase) phased_barrier(a, nbar, ++nb, &s_rel);
  }

  // the block's vectors past its last whole span, then its ragged edges
  for (int64_t v = nvec / span * span + (int64_t)t * kBlock + tid; v < nvec; v += (int64_t)a.tiles * kBlock) {
    const int64_t vb = (vbeg + v * V) * E;
    const u32x4 w = ld16(xj, vb);
#pragma unroll
    for (int r = 0; r < P; r++)
      if (!SKIP_OWN || r != j) st16(yp[r], vb, w);
  }
  for (int64_t s = (int64_t)t * kBlock + tid; s < nscalar; s += (int64_t)a.tiles * kBlock) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    const U w = ((const U*)xj)[i];
#pragma unroll
    for (int r = 0; r < P; r++)
      if (!SKIP_OWN || r != j) ((U*)yp[r])[i] = w;
  }
}

namespace {

template <int E, bool SKIP_OWN>
hipError_t gather_by_p(int p, const PhasedArgs& a, hipStream_t s) {
  const dim3 g((unsigned)a.tiles * (unsigned)p), b(kBlock);
  switch (p) {
    case 2: return launch<k_gather_phased<E, 2, SKIP_OWN>>(g, b, s, a);
    case 4: return launch<k_gather_phased<E, 4, SKIP_OWN>>(g, b, s, a);
    case 8: return launch<k_gather_phased<E, 8, SKIP_OWN>>(g, b, s, a);
    case 16: return launch<k_gather_phased<E, 16, SKIP_OWN>>(g, b, s, a);
  }
  return hipErrorInvalidValue;
}

template <int E, int P, bool SKIP_OWN>
int gather_occ_of() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)k_gather_phased<E, P, SKIP_OWN>, kBlock, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return nb;
}

template <int E, bool SKIP_OWN>
int gather_occ(int p) {
  switch (p) {
    case 2: return gather_occ_of<E, 2, SKIP_OWN>();
    case 4: return gather_occ_of<E, 4, SKIP_OWN>();
    case 8: return gather_occ_of<E, 8, SKIP_OWN>();
    case 16: return gather_occ_of<E, 16, SKIP_OWN>();
  }
  return 0;
}

}  // namespace

hipError_t launch_gather_phased(int esize, int p, bool skip_own, const PhasedArgs& a, hipStream_t s) {
  if (esize == 4) return skip_own ? gather_by_p<4, true>(p, a, s) : gather_by_p<4, false>(p, a, s);
  if (esize == 2) return skip_own ? gather_by_p<2, true>(p, a, s) : gather_by_p<2, false>(p, a, s);
  return hipErrorInvalidValue;
}

int gather_phased_blocks_per_cu(int esize, int p, bool skip_own) {
  if (esize == 4) return skip_own ? gather_occ<4, true>(p) : gather_occ<4, false>(p);
  if (esize == 2) return skip_own ? gather_occ<2, true>(p) : gather_occ<2, false>(p);
  return 0;
}

}  // namespace simar
