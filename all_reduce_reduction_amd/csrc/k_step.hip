// k_step.hip -- per-step kernels of the multi-launch schedules (gfx950).
//
// k_ring_reduce runs one reduce-scatter step of the ring: for each of the
// step's transfers (one per rank), the arriving running value of
// the chunk is combined with the receiving rank's own element and written
// on -- the fused receive-reduce-send primitive of NCCL's runRing
// ("Inside NCCL all-reduce", section "The ring, exactly as the kernel runs
// it").  On the last step of the half the chunk completes: the post-op (the
// int avg divide, the one RNE narrowing of 16-bit types) is applied and the
// result goes to the owner's output.  Partials are accumulator-typed: for
// 32-bit types they live in the receiving rank's output buffer (the slot of
// a chunk that rank does not own yet); for fp16/bf16 they stay fp32, in
// library scratch, so each element is rounded to 16 bits exactly once.
//
// k_copy moves finished chunks: the ring's all-gather forwards, the
// all-pairs fan-out (one 16-byte load, up to p-1 stores from the same
// registers) and the standalone all-gather.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

// One reduce-scatter transfer's share for workgroup `tile` of `tiles`.
template <int DT, int OP, bool A_PART, bool D_FINAL, int U>
__device__ __forceinline__ void ring_reduce_xfer(const RingXfer& x, const int64_t tile, const int tiles, const int p,
                                                 const float inv_p) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int V = epv<DT>();
  constexpr int E = Ty<DT>::E;
  const int64_t lo = x.lo, hi = x.hi;
  int64_t head = x.vec_ok ? (int64_t)((V - (lo % V)) % V) : (hi - lo);
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const int64_t span = (int64_t)kBlock * U;
  const int64_t stride = (int64_t)tiles * span;

  // one span of U vectors per lane; GUARD: the span may run past nvec
  auto span_body = [&](int64_t base, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t v = base + u * kBlock + tid;
      if (!GUARD || v < nvec) {
        const int64_t i0 = vbeg + v * V;
        A in[V], own[V];
        if constexpr (A_PART) {
          load_part<DT>(x.a, i0 - x.a_shift, in);
        } else {
          unpack<DT>(ld16(x.a, i0 * E), in);
#pragma unroll
          for (int e = 0; e < V; e++) in[e] = O::pre(in[e], inv_p);
        }
        unpack<DT>(ld16(x.b, i0 * E), own);
#pragma unroll
        for (int e = 0; e < V; e++) in[e] = O::comb(in[e], O::pre(own[e], inv_p));
        if constexpr (D_FINAL) {
#pragma unroll
          for (int e = 0; e < V; e++) in[e] = O::post(in[e], p);
          st16(x.d, (i0 - x.d_shift) * E, pack<DT>(in));
        } else {
          store_part<DT>(x.d, i0 - x.d_shift, in);
        }
      }
    }
  };
  // whole spans unguarded (one straight-line block per span), then the
  // partial span, if any
  int64_t base = tile * span;
  for (; base + span <= nvec; base += stride) span_body(base, std::false_type());
  if (base < nvec) span_body(base, std::true_type());

  for (int64_t s = tile * kBlock + tid; s < nscalar; s += (int64_t)tiles * kBlock) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    A in;
    if constexpr (A_PART) in = ((const A*)x.a)[part_pos<DT>(i - x.a_shift)];
    else in = O::pre(load_elem<DT>(x.a, i), inv_p);
    A v = O::comb(in, O::pre(load_elem<DT>(x.b, i), inv_p));
    if constexpr (D_FINAL) store_elem<DT>(x.d, i - x.d_shift, O::post(v, p));
    else ((A*)x.d)[part_pos<DT>(i - x.d_shift)] = v;
  }
}

template <int DT, int OP, bool A_PART, bool D_FINAL, int U>
__global__ void __launch_bounds__(kBlock) k_ring_reduce(RingArgs args) {
  // 1-D grid, transfers interleaved: workgroup b runs tile b / nx of
  // transfer b mod nx, so the transfers in flight together cover every chunk
  const unsigned xi = blockIdx.x % (unsigned)args.nx;
  const int64_t tile = blockIdx.x / (unsigned)args.nx;
  const RingXfer x = args.x[xi];
  ring_reduce_xfer<DT, OP, A_PART, D_FINAL, U>(x, tile, args.tiles, args.p, args.inv_p);
}

// The same step of an all-reduce ring from the library's pointer table: the
// transfers follow from the step, as the ring's lowering defines them --
// at reduce-scatter step s rank r sends chunk (r - 1 - s) mod p to rank
// r + 1, which folds its own input in; fp16/bf16 partials alternate between
// two scratch slot sets by step parity (32-bit partials stay in the
// receiving rank's output).
template <int DT, int OP, bool A_PART, bool D_FINAL, int U>
__global__ void __launch_bounds__(kBlock) k_ring_reduce_tab(RingTabArgs a) {
  const int p = a.p;
  const int r = (int)(blockIdx.x % (unsigned)p);
  const int64_t tile = blockIdx.x / (unsigned)p;
  const int s = a.step;
  const int c = ((r - 1 - s) % p + p) % p;
  const int d = (r + 1 == p) ? 0 : r + 1;
  RingXfer x;
  x.lo = (int64_t)c * a.n / p;
  x.hi = (int64_t)(c + 1) * a.n / p;
  const int64_t slot_shift = x.lo - (x.lo % 8);
  auto slot = [&](int parity, int rank) -> void* {
    return (char*)a.scratch + ((int64_t)parity * p + rank) * a.slot_elems * 4;
  };
  if (!A_PART) {
    x.a = a.set->x[r];
    x.a_shift = 0;
  } else if (a.scratch) {
    x.a = slot((s - 1) & 1, r);
    x.a_shift = slot_shift;
  } else {
    x.a = a.set->y[r];
    x.a_shift = 0;
  }
  x.b = a.set->x[d];
  if (D_FINAL || !a.scratch) {
    x.d = a.set->y[d];
    x.d_shift = 0;
  } else {
    x.d = slot(s & 1, d);
    x.d_shift = slot_shift;
  }
  x.vec_ok = 1;  // every shift is a multiple of 8 elements and every pointer 16-byte aligned
  x.pad_ = 0;
  ring_reduce_xfer<DT, OP, A_PART, D_FINAL, U>(x, tile, a.tiles, p, a.inv_p);
}

// One transfer's share for workgroup `tile` of `tiles`: elements [lo, hi)
// of src (read at [i - src_shift]) to the nd destinations in dp (written at
// [i - dst_shift]).  The destination pointers sit in scalar registers,
// loaded once by the caller (a loop over a run-time count would re-load each
// one and wait for it before every store).
template <int E, int U, int ND>
__device__ __forceinline__ void copy_tiles(const void* const src, void* const (&dp)[ND], const int nd, const int64_t lo,
                                           const int64_t hi, const bool vec_ok, const int64_t src_shift,
                                           const int64_t dst_shift, const int64_t tile, const int tiles) {
  constexpr int V = 16 / E;
  int64_t head = vec_ok ? (int64_t)((V - (lo % V)) % V) : (hi - lo);
  if (head > hi - lo) head = hi - lo;
  const int64_t vbeg = lo + head;
  const int64_t nvec = (hi - vbeg) / V;
  const int64_t tail_beg = vbeg + nvec * V;
  const int64_t nscalar = head + (hi - tail_beg);
  const int tid = threadIdx.x;
  const int64_t span = (int64_t)kBlock * U;
  const int64_t stride = (int64_t)tiles * span;
  const int64_t src_off = src_shift * E, dst_off = dst_shift * E;
  // one span of U vectors per lane; GUARD: the span may run past nvec
  auto span_body = [&](int64_t base, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    const int64_t sb = (vbeg + base * V) * E;  // the span's first byte (uniform)
    const uint32_t lane = lane_offset((uint32_t)tid * 16u);
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; u++)
      if (!GUARD || base + u * kBlock + tid < nvec)
        w[u] = ld16u(src, sb - src_off + (int64_t)u * kBlock * 16, lane);
#pragma unroll
    for (int u = 0; u < U; u++)
      if (!GUARD || base + u * kBlock + tid < nvec) {
        const int64_t ub = sb - dst_off + (int64_t)u * kBlock * 16;
#pragma unroll
        for (int d = 0; d < ND; d++)
          if (d < nd) st16u(dp[d], ub, lane, w[u]);
      }
  };
  // whole spans unguarded (one straight-line block per span), then the
  // partial span, if any
  int64_t base = tile * span;
  for (; base + span <= nvec; base += stride) span_body(base, std::false_type());
  if (base < nvec) span_body(base, std::true_type());
  for (int64_t s = tile * kBlock + tid; s < nscalar; s += (int64_t)tiles * kBlock) {
    const int64_t i = (s < head) ? lo + s : tail_beg + (s - head);
    if constexpr (E == 4) {
      const uint32_t w = ((const uint32_t*)src)[i - src_shift];
#pragma unroll
      for (int d = 0; d < ND; d++)
        if (d < nd) ((uint32_t*)dp[d])[i - dst_shift] = w;
    } else {
      const uint16_t w = ((const uint16_t*)src)[i - src_shift];
#pragma unroll
      for (int d = 0; d < ND; d++)
        if (d < nd) ((uint16_t*)dp[d])[i - dst_shift] = w;
    }
  }
}

// ONE: every transfer of the launch has a single destination (the ring's
// all-gather steps).  Measured on MI355X: loading all 16 destination
// pointers up front costs such short-lived workgroups ~20% on a ring
// all-gather step, while it saves the fan-out ~4%.
template <int E, int U, bool ONE>
__global__ void __launch_bounds__(kBlock) k_copy(CopyArgs args) {
  const unsigned xi = blockIdx.x % (unsigned)args.nx;  // transfers interleaved, as above
  const int64_t tile = blockIdx.x / (unsigned)args.nx;
  const CopyXfer& x = args.x[xi];
  const int nd = x.ndst;
  constexpr int ND = ONE ? 1 : SIM_MAX_RANKS;
  void* dp[ND];
#pragma unroll
  for (int d = 0; d < ND; d++) dp[d] = (d < nd) ? x.dst[d] : nullptr;
  copy_tiles<E, U, ND>(x.src, dp, nd, x.lo, x.hi, x.vec_ok != 0, x.src_shift, x.dst_shift, tile, args.tiles);
}

// The all-pairs fan-out with its pointers in the library's pointer table:
// workgroup b copies tile b / p of chunk j = b mod p from the owner's
// output to every other rank's output (chunk j = [floor(j n / p),
// floor((j+1) n / p)), every pointer 16-byte aligned).
template <int E, int U>
__global__ void __launch_bounds__(kBlock) k_fanout_tab(FanoutTabArgs a) {
  const int p = a.p;
  const int j = (int)(blockIdx.x % (unsigned)p);
  const int64_t tile = blockIdx.x / (unsigned)p;
  void* dp[SIM_MAX_RANKS];
#pragma unroll
  for (int d = 0; d < SIM_MAX_RANKS; d++) dp[d] = (d < p - 1) ? a.set->y[d < j ? d : d + 1] : nullptr;
  const int64_t lo = (int64_t)j * a.n / p, hi = (int64_t)(j + 1) * a.n / p;
  copy_tiles<E, U, SIM_MAX_RANKS>(a.set->y[j], dp, p - 1, lo, hi, true, 0, 0, tile, a.tiles);
}

// A ring all-gather step from the pointer table: at step s rank r forwards
// its finished chunk (r - s) mod p to rank r + 1.
template <int E, int U>
__global__ void __launch_bounds__(kBlock) k_ring_copy_tab(RingTabArgs a) {
  const int p = a.p;
  const int r = (int)(blockIdx.x % (unsigned)p);
  const int64_t tile = blockIdx.x / (unsigned)p;
  const int c = ((r - a.step) % p + p) % p;
  void* dp[1] = {a.set->y[(r + 1 == p) ? 0 : r + 1]};
  const int64_t lo = (int64_t)c * a.n / p, hi = (int64_t)(c + 1) * a.n / p;
  copy_tiles<E, U, 1>(a.set->y[r], dp, 1, lo, hi, true, 0, 0, tile, a.tiles);
}

__global__ void __launch_bounds__(kBlock) k_fill64(unsigned long long* p, unsigned long long v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) p[i] = v;
}

// ---- launchers ----------------------------------------------------------------
template <int DT, int OP, int U>
static hipError_t ring_go(bool a_part, bool d_final, const RingArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.tiles * (unsigned)a.nx), block(kBlock);
  if (a_part) {
    if (d_final) return launch<k_ring_reduce<DT, OP, true, true, U>>(grid, block, s, a);
    return launch<k_ring_reduce<DT, OP, true, false, U>>(grid, block, s, a);
  }
  if (d_final) return launch<k_ring_reduce<DT, OP, false, true, U>>(grid, block, s, a);
  return launch<k_ring_reduce<DT, OP, false, false, U>>(grid, block, s, a);
}

template <int DT, int OP, int U>
static hipError_t ring_go(bool a_part, bool d_final, const RingTabArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.tiles * (unsigned)a.p), block(kBlock);
  if (a_part) {
    if (d_final) return launch<k_ring_reduce_tab<DT, OP, true, true, U>>(grid, block, s, a);
    return launch<k_ring_reduce_tab<DT, OP, true, false, U>>(grid, block, s, a);
  }
  if (d_final) return launch<k_ring_reduce_tab<DT, OP, false, true, U>>(grid, block, s, a);
  return launch<k_ring_reduce_tab<DT, OP, false, false, U>>(grid, block, s, a);
}

template <int DT, int OP, class Args>
static hipError_t ring_by_unroll(int unroll, bool ap, bool df, const Args& a, hipStream_t s) {
  return unroll == 2 ? ring_go<DT, OP, 2>(ap, df, a, s) : ring_go<DT, OP, 1>(ap, df, a, s);
}

template <int DT, class Args>
static hipError_t ring_by_op(int op, int unroll, bool ap, bool df, const Args& a, hipStream_t s) {
  switch (op) {
    case SIM_SUM: return ring_by_unroll<DT, SIM_SUM>(unroll, ap, df, a, s);
    case SIM_PROD: return ring_by_unroll<DT, SIM_PROD>(unroll, ap, df, a, s);
    case SIM_MIN: return ring_by_unroll<DT, SIM_MIN>(unroll, ap, df, a, s);
    case SIM_MAX: return ring_by_unroll<DT, SIM_MAX>(unroll, ap, df, a, s);
    case SIM_AVG: return ring_by_unroll<DT, SIM_AVG>(unroll, ap, df, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ring_reduce(int dtype, int op, bool a_partial, bool d_final, const RingArgs& a,
                              int unroll, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return ring_by_op<SIM_INT32>(op, unroll, a_partial, d_final, a, s);
    case SIM_FP32: return ring_by_op<SIM_FP32>(op, unroll, a_partial, d_final, a, s);
    case SIM_FP16: return ring_by_op<SIM_FP16>(op, unroll, a_partial, d_final, a, s);
    case SIM_BF16: return ring_by_op<SIM_BF16>(op, unroll, a_partial, d_final, a, s);
  }
  return hipErrorInvalidValue;
}

template <bool ONE>
static hipError_t copy_go(int esize, const CopyArgs& a, int unroll, hipStream_t s) {
  const dim3 grid((unsigned)a.tiles * (unsigned)a.nx), block(kBlock);
  if (esize == 4) {
    if (unroll == 2) return launch<k_copy<4, 2, ONE>>(grid, block, s, a);
    return launch<k_copy<4, 1, ONE>>(grid, block, s, a);
  }
  if (esize == 2) {
    if (unroll == 2) return launch<k_copy<2, 2, ONE>>(grid, block, s, a);
    return launch<k_copy<2, 1, ONE>>(grid, block, s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ring_reduce_tab(int dtype, int op, bool a_partial, bool d_final, const RingTabArgs& a,
                                  int unroll, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return ring_by_op<SIM_INT32>(op, unroll, a_partial, d_final, a, s);
    case SIM_FP32: return ring_by_op<SIM_FP32>(op, unroll, a_partial, d_final, a, s);
    case SIM_FP16: return ring_by_op<SIM_FP16>(op, unroll, a_partial, d_final, a, s);
    case SIM_BF16: return ring_by_op<SIM_BF16>(op, unroll, a_partial, d_final, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ring_copy_tab(int esize, const RingTabArgs& a, int unroll, hipStream_t s) {
  const dim3 grid((unsigned)a.tiles * (unsigned)a.p), block(kBlock);
  if (esize == 4) {
    if (unroll == 2) return launch<k_ring_copy_tab<4, 2>>(grid, block, s, a);
    return launch<k_ring_copy_tab<4, 1>>(grid, block, s, a);
  }
  if (esize == 2) {
    if (unroll == 2) return launch<k_ring_copy_tab<2, 2>>(grid, block, s, a);
    return launch<k_ring_copy_tab<2, 1>>(grid, block, s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy(int esize, const CopyArgs& a, int unroll, hipStream_t s) {
  bool one = true;  // every transfer has a single destination (ring all-gather steps)
  for (int k = 0; k < a.nx; k++) one = one && a.x[k].ndst <= 1;
  return one ? copy_go<true>(esize, a, unroll, s) : copy_go<false>(esize, a, unroll, s);
}

hipError_t launch_fanout_tab(int esize, const FanoutTabArgs& a, int unroll, hipStream_t s) {
  const dim3 grid((unsigned)a.tiles * (unsigned)a.p), block(kBlock);
  if (esize == 4) {
    if (unroll == 2) return launch<k_fanout_tab<4, 2>>(grid, block, s, a);
    return launch<k_fanout_tab<4, 1>>(grid, block, s, a);
  }
  if (esize == 2) {
    if (unroll == 2) return launch<k_fanout_tab<2, 2>>(grid, block, s, a);
    return launch<k_fanout_tab<2, 1>>(grid, block, s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fill64(unsigned long long* p, unsigned long long v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  return launch<k_fill64>(dim3((unsigned)blocks), dim3(kBlock), s, p, v, n);
}

}  // namespace simar
