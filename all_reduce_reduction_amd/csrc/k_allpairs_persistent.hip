// k_allpairs_persistent.hip -- the two-step all-pairs all-reduce in ONE
// launch, its steps joined by in-kernel signal / wait (gfx950).
//
// The two-phase all-pairs of "MSCCL++ ..." (section "The Collective
// Algorithm Library": every rank reduce-scatters its own chunk from all
// peers, then all-gathers the finished chunks) run as one kernel over
// MemoryChannel-style put / signal / wait (section 4): the step boundary is
// a per-slice counter instead of a kernel launch.
//   step 1 (GATHER_REDUCE): workgroup (rank r, channel c) folds its slice
//          of chunk r over every rank's input in the all-pairs order (owner
//          r first, then the other ranks ascending -- the order of the
//          scratch slots in the all-pairs program of "MSCCL, in depth ...",
//          section "Writing an algorithm in MSCCLang"), post-processes it
//          and writes it into Y[r] with device-scope stores; then it
//          signals ready(r, c).
//   step 2 (FANOUT, as each rank pulling from the owner): the workgroup
//          waits for ready(j, c) of every other owner j at once (one lane
//          per owner), then copies every owner's slice of Y[j] into Y[r],
//          reading it with device-scope loads -- each rank reading a peer's
//          finished chunk from the peer's buffer, as a GPU reads over its
//          links.  Each pass loads from all p - 1 owners before it stores.
// On one HBM this moves (3p - 1) S bytes (the 2-launch all-pairs fans out
// with one load and p - 1 stores: (2p + 1) S; the fused one-shot 2p S): it
// is the all-pairs schedule with its synchronisation inside the kernel,
// not a faster form of it.
//
// In place (Y[r] == X[r]) is safe: rank r overwrites X[r]'s slice c of
// chunk j only after ready(j, c), which owner j signals after its last read
// of that slice.  Every workgroup finishes step 1 (no waits) before it
// waits in step 2 and the host keeps the whole grid co-resident, so every
// wait is answered; each wait is still bounded, and on expiry the
// workgroup records SIM_ERR_TIMEOUT and leaves.  The grid is rank-major
// (workgroup r * Cg + c, Cg a multiple of 8), so the ranks of one channel
// share an XCD as in the single-launch ring.
#include "device_sync.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

template <int DT, int OP, int P>
__global__ void __launch_bounds__(kBlock) k_allpairs_persistent(AllPairsPArgs a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int E = Ty<DT>::E;
  constexpr int V = epv<DT>();
  constexpr int U = kAllPairsPVecsPerLane;
  constexpr int MAXP = P ? P : SIM_MAX_RANKS;
  constexpr int64_t kSpan = (int64_t)kBlock * U * V;  // elements per pass
  __shared__ int ok_flag;

  const int p = P ? P : a.p;
  const int r = (int)(blockIdx.x / (unsigned)a.Cg);
  const int ch = (int)(blockIdx.x % (unsigned)a.Cg);
  if (ch >= a.C) return;                  // grid padding
  if (a.withhold && r == 0) return;       // test hook: a partner that never shows up
  const int tid = threadIdx.x;
  const unsigned epoch = a.epoch;
  const float inv_p = a.inv_p;
  const int C = a.C;

  // channel ch's slice of chunk j: inner boundaries on whole vectors of the
  // chunk (the split of the single-launch ring)
  auto slice = [&](int j, int64_t* s_lo, int64_t* s_hi) {
    const int64_t clo = a.lo[j], chi = a.lo[j + 1], clen = chi - clo;
    *s_lo = clo + (clen * ch / C) / V * V;
    *s_hi = (ch + 1 == C) ? chi : clo + (clen * (ch + 1) / C) / V * V;
  };

  // ---- step 1: fold my slice of chunk r --------------------------------------
  {
    const void* xp[MAXP];  // operand k: rank r for k == 0, then the ranks != r ascending
#pragma unroll
    for (int k = 0; k < MAXP; k++) {
      const int q = (k == 0) ? r : (k <= r ? k - 1 : k);
      xp[k] = (k < p) ? a.x[q] : nullptr;
    }
    void* const yr = a.y[r];
    int64_t s_lo, s_hi;
    slice(r, &s_lo, &s_hi);
    const bool vec = (s_lo % V) == 0;  // absolute alignment (every pointer is 16-byte aligned)
    for (int64_t base = s_lo; base < s_hi; base += kSpan) {
      const int64_t len = min(s_hi - base, kSpan);
      const __amdgpu_buffer_rsrc_t my_y = out_rsrc(yr, base * E, len * E);
      u32x4 L[U][MAXP];
      bool full[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int64_t off = ((int64_t)u * kBlock + tid) * V;
        full[u] = vec && off + V <= len;
        if (full[u]) {
#pragma unroll
          for (int k = 0; k < MAXP; k++)
            if (k < p) L[u][k] = ld16(xp[k], (base + off) * E);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int64_t off = ((int64_t)u * kBlock + tid) * V;
        if (full[u]) {
          A acc[V], t[V];
          unpack<DT>(L[u][0], acc);
#pragma unroll
          for (int e = 0; e < V; e++) acc[e] = O::pre(acc[e], inv_p);
#pragma unroll
          for (int k = 1; k < MAXP; k++) {
            if (k < p) {
              unpack<DT>(L[u][k], t);
#pragma unroll
              for (int e = 0; e < V; e++) acc[e] = O::comb(acc[e], O::pre(t[e], inv_p));
            }
          }
#pragma unroll
          for (int e = 0; e < V; e++) acc[e] = O::post(acc[e], p);
          __builtin_amdgcn_raw_buffer_store_b128(pack<DT>(acc), my_y, (int)(off * E), 0, kSt);
        } else if (off < len) {  // ragged: element by element
          const int cnt = (int)min((int64_t)V, len - off);
          for (int e = 0; e < cnt; e++) {
            const int64_t i = base + off + e;
            A acc = O::pre(load_elem<DT>(xp[0], i), inv_p);
#pragma unroll
            for (int k = 1; k < MAXP; k++)
              if (k < p) acc = O::comb(acc, O::pre(load_elem<DT>(xp[k], i), inv_p));
            acc = O::post(acc, p);
            const int yoff = (int)((off + e) * E);
            if constexpr (E == 4) __builtin_amdgcn_raw_buffer_store_b32(narrow_bits<DT>(acc), my_y, yoff, 0, kSt);
            else __builtin_amdgcn_raw_buffer_store_b16((unsigned short)narrow_bits<DT>(acc), my_y, yoff, 0, kSt);
          }
        }
      }
    }
  }
  // signal: every wave's stores have completed before the barrier, and
  // only then does one lane store the counter
  wait_stores();
  __syncthreads();
  if (tid == 0)
    __hip_atomic_store(a.sem + ((int64_t)r * C + ch) * 2, tag(epoch, 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- step 2: pull every other owner's slice --------------------------------
  void* const yr = a.y[r];
  // wait for the p - 1 owners together (lane k polls owner r + 1 + k)
  if (!wait_all_geq(
          p - 1, [&](int k) { return a.sem + ((int64_t)((r + 1 + k) % p) * C + ch) * 2; }, tag(epoch, 1),
          a.spin_limit, &ok_flag))
    goto timeout;
  // Pass b covers offsets [b, b + kPull) of every owner's slice, one
  // vector per lane per owner: the loads of all p - 1 owners for the pass
  // are issued together, then stored, so a pass costs one device-scope
  // round trip instead of one per owner (at 8 KiB per rank a slice is a
  // single pass).
  {
    constexpr int64_t kPull = (int64_t)kBlock * V;
    int64_t o_lo[MAXP], o_len[MAXP];
    int64_t longest = 0;
#pragma unroll
    for (int jj = 1; jj < MAXP; jj++) {
      o_lo[jj] = 0;
      o_len[jj] = 0;
      if (jj < p) {
        int64_t s_lo, s_hi;
        slice((r + jj) % p, &s_lo, &s_hi);
        o_lo[jj] = s_lo;
        o_len[jj] = s_hi - s_lo;
        longest = max(longest, s_hi - s_lo);
      }
    }
    for (int64_t b = 0; b < longest; b += kPull) {
      u32x4 w[MAXP];
      bool full[MAXP];
#pragma unroll
      for (int jj = 1; jj < MAXP; jj++) {
        const int64_t len = (jj < p) ? min(max(o_len[jj] - b, (int64_t)0), kPull) : 0;
        const bool vec = (o_lo[jj] % V) == 0;
        const __amdgpu_buffer_rsrc_t src =
            out_rsrc(a.y[jj < p ? (r + jj) % p : r], (o_lo[jj] + b) * E, len * E);
        const int64_t off = (int64_t)tid * V;
        full[jj] = jj < p && vec && off + V <= len;
        if (full[jj]) w[jj] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(off * E), 0, kLd);
      }
#pragma unroll
      for (int jj = 1; jj < MAXP; jj++) {
        if (jj >= p) continue;
        const int64_t len = min(max(o_len[jj] - b, (int64_t)0), kPull);
        const int64_t base = o_lo[jj] + b;
        const __amdgpu_buffer_rsrc_t src = out_rsrc(a.y[(r + jj) % p], base * E, len * E);
        {
          const int64_t off = (int64_t)tid * V;
          if (full[jj]) {
            st16(yr, (base + off) * E, w[jj]);
          } else if (off < len) {  // ragged: element by element
            const int cnt = (int)min((int64_t)V, len - off);
            for (int e = 0; e < cnt; e++) {
              const int yoff = (int)((off + e) * E);
              if constexpr (E == 4) {
                ((uint32_t*)yr)[base + off + e] = __builtin_amdgcn_raw_buffer_load_b32(src, yoff, 0, kLd);
              } else {
                ((uint16_t*)yr)[base + off + e] =
                    (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(src, yoff, 0, kLd);
              }
            }
          }
        }
      }
    }
  }
  return;

timeout:
  if (tid == 0) __hip_atomic_store(a.err, (int)SIM_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int OP>
static hipError_t ap_go(const AllPairsPArgs& a, hipStream_t s) {
  const dim3 g((unsigned)(a.p * a.Cg)), b(kBlock);
  if (a.p == 8) return launch<k_allpairs_persistent<DT, OP, 8>>(g, b, s, a);
  return launch<k_allpairs_persistent<DT, OP, 0>>(g, b, s, a);
}

template <int DT>
static hipError_t ap_by_op(int op, const AllPairsPArgs& a, hipStream_t s) {
  switch (op) {
    case SIM_SUM: return ap_go<DT, SIM_SUM>(a, s);
    case SIM_PROD: return ap_go<DT, SIM_PROD>(a, s);
    case SIM_MIN: return ap_go<DT, SIM_MIN>(a, s);
    case SIM_MAX: return ap_go<DT, SIM_MAX>(a, s);
    case SIM_AVG: return ap_go<DT, SIM_AVG>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_allpairs_persistent(int dtype, int op, const AllPairsPArgs& a, hipStream_t s) {
  if (a.p < 2 || a.p > SIM_MAX_RANKS || a.C < 1 || a.Cg < a.C) return hipErrorInvalidValue;
  switch (dtype) {
    case SIM_INT32: return ap_by_op<SIM_INT32>(op, a, s);
    case SIM_FP32: return ap_by_op<SIM_FP32>(op, a, s);
    case SIM_FP16: return ap_by_op<SIM_FP16>(op, a, s);
    case SIM_BF16: return ap_by_op<SIM_BF16>(op, a, s);
  }
  return hipErrorInvalidValue;
}

// Workgroups of the (dtype, op, p) instantiation that fit on one CU at once.
template <int DT, int OP>
static int ap_occ(int p) {
  int nb = 0;
  const void* f = (p == 8) ? (const void*)k_allpairs_persistent<DT, OP, 8> : (const void*)k_allpairs_persistent<DT, OP, 0>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, kBlock, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  return nb > 0 ? nb : 1;
}

template <int DT>
static int ap_occ_op(int op, int p) {
  switch (op) {
    case SIM_SUM: return ap_occ<DT, SIM_SUM>(p);
    case SIM_PROD: return ap_occ<DT, SIM_PROD>(p);
    case SIM_MIN: return ap_occ<DT, SIM_MIN>(p);
    case SIM_MAX: return ap_occ<DT, SIM_MAX>(p);
    default: return ap_occ<DT, SIM_AVG>(p);
  }
}

int allpairs_persistent_blocks_per_cu(int dtype, int op, int p) {
  switch (dtype) {
    case SIM_INT32: return ap_occ_op<SIM_INT32>(op, p);
    case SIM_FP32: return ap_occ_op<SIM_FP32>(op, p);
    case SIM_FP16: return ap_occ_op<SIM_FP16>(op, p);
    default: return ap_occ_op<SIM_BF16>(op, p);
  }
}

}  // namespace simar
