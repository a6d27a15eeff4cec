// k_ring_fifo.hip -- the whole ring all-reduce in ONE launch (gfx950).
//
// NCCL's runRing ("Inside NCCL all-reduce", section "The ring, exactly as
// the kernel runs it") executed by persistent workgroups: workgroup
// (rank r, channel ch) runs rank r's primitive sequence
//     send, (p-2) x recvReduceSend, recvReduceCopySend(post-op),
//     (p-2) x recvCopySend, recv
// over its channel's slice of every chunk ("Channels: the ring is plural":
// each channel owns a slice of the buffer and its own FIFOs).  Partial sums
// of the reduce-scatter half move between neighbouring ranks through
// bounded FIFOs of NS slots (the 8-slot FIFO per peer of the same page,
// section "Why a 100 GB all-reduce doesn't OOM"), so a partial never
// round-trips a full-size buffer.  In the all-gather half a finished slice
// is final where it lands, so the successor reads it straight from this
// rank's output buffer (NCCL's direct read of a peer's buffer) at storage
// width instead of through a FIFO.
//
// Synchronisation is the MemoryChannel put / signal / wait of "MSCCL++ ...",
// section 4 (signal after the data, wait blocks, a monotonic expected value
// so a stale signal never satisfies a wait):
//   - posted[r][ch]   written by rank r-1 after it fills a slot of rank r's FIFO
//   - consumed[r][ch] written by rank r after it has read a slot
// Both hold (epoch << 32 | count) with a per-call epoch, so values left by
// an earlier call compare lower than anything this call waits for.  A
// sender may run at most NS FIFO slots ahead of its receiver (backpressure);
// output slices are written once per call and need none.
// Placement.  The grid is rank-major, workgroup b = r * Cg + ch with Cg the
// channel count rounded up to a multiple of 8 (padding workgroups leave at
// once).  Under the round-robin dispatch of workgroups to the 8 XCDs this
// keeps the ranks of one channel together on one XCD; the channel-major
// grid (rank r on XCD r) measured 12% slower at 64 MiB per rank.
//
// Memory ordering.  Each XCD has its own L2, not coherent with the others
// for plain accesses, and a CU's own cache is coherent only for its own
// waves.  FIFO words are therefore only ever read and written with
// device-scope (sc1) buffer instructions, coherent across CUs and XCDs
// without flushing or invalidating any cache; so are the output slices a
// successor will read.  (Keeping a channel's FIFO
// words in its XCD's L2 with workgroup-scope accesses and a CU-cache
// invalidate was tried: it returned stale words -- outside thread-group
// split mode that scope does not reach another CU.)  A producer wave issues
// its slot stores, waits for them to complete (s_waitcnt vmcnt(0)), the
// workgroup meets at a barrier, and only then does one lane store the
// counter (a relaxed agent-scope atomic, also sc1).  The consumer's lane 0
// polls the counter with agent-scope loads; the workgroup meets at a
// barrier; only then are the slot's words loaded.  (A release/acquire pair
// on the counter would add an L2 write-back and invalidate per step, which
// measured ~10 us per step.)
// Every wait is bounded by spin_limit polls; on expiry the workgroup writes
// SIM_ERR_TIMEOUT to the error word and leaves, so a missing partner (e.g.
// workgroups that could not be co-resident) ends in an error, never a hang.
#include "device_sync.h"
#include "kernels.h"
#include "launch.h"

namespace simar {

namespace {

// Byte offset in a FIFO slot of fp32 partial e (0 <= e < V) of vector u of
// lane t.  The slot holds 16-byte words ordered [u][e / 4][t], so each
// 16-byte store or load instruction of a wave covers one contiguous
// 1 KiB run.  (Laid out element by element, a lane's V = 8 partials of a
// 16-bit vector span 32 bytes and each instruction would cover every other
// 16 bytes: half lines, which the device-scope stores wrote through to
// memory as separate partial writes -- twice the FIFO bytes in the write
// counters.)  The producer and the consumer of a slot run the same (u, t, e)
// over the same elements, so the layout is private to this kernel.
template <int V>
__device__ __forceinline__ int fifo_off(int u, int t, int e) {
  return ((u * (V / 4) + e / 4) * kBlock + t) * 16 + (e % 4) * 4;
}

}  // namespace

template <int DT, int OP>
__global__ void __launch_bounds__(kBlock) k_ring_fifo(RingFifoArgs a) {
  typedef typename Ty<DT>::A A;
  typedef Op<DT, OP> O;
  constexpr int E = Ty<DT>::E;
  constexpr int V = epv<DT>();  // elements per 16-byte storage vector
  constexpr int U = kFifoVecsPerLane;  // a slot is exactly kBlock * U vectors
  __shared__ int ok_recv, ok_send;

  const int p = a.p;
  const int r = (int)(blockIdx.x / (unsigned)a.Cg);
  const int ch = (int)(blockIdx.x % (unsigned)a.Cg);
  if (ch >= a.C) return;  // grid padding: the channel count rounded up to whole XCD rounds
  const int nxt = (r + 1 == p) ? 0 : r + 1;
  const int prv = (r == 0) ? p - 1 : r - 1;
  const int tid = threadIdx.x;
  const unsigned epoch = a.epoch;
  const float inv_p = a.inv_p;
  const int64_t slot_words = a.slot_elems;  // one 32-bit word per element

  // my receive FIFO and counters, and my successor's
  uint32_t* my_fifo = a.fifo + ((int64_t)r * a.C + ch) * a.NS * slot_words;
  uint32_t* nx_fifo = a.fifo + ((int64_t)nxt * a.C + ch) * a.NS * slot_words;
  const __amdgpu_buffer_rsrc_t in_rs = fifo_rsrc(my_fifo, a.NS * slot_words * 4);
  const __amdgpu_buffer_rsrc_t out_rs = fifo_rsrc(nx_fifo, a.NS * slot_words * 4);
  // per (rank, channel): posted, consumed
  unsigned long long* my_posted = a.sem + ((int64_t)r * a.C + ch) * 2;
  unsigned long long* my_consumed = my_posted + 1;
  unsigned long long* nx_posted = a.sem + ((int64_t)nxt * a.C + ch) * 2;
  unsigned long long* nx_consumed = nx_posted + 1;

  const void* xr = a.x[r];
  void* yr = a.y[r];
  unsigned long long sent = 0, recvd = 0;
  if (a.withhold && r == 0) return;  // test hook: a partner that never shows up

  for (int k = 0; k < a.nsub; k++) {
    for (int step = 0; step < 2 * p - 1; step++) {
      // step 0: send; 1..p-2: recvReduceSend; p-1: recvReduceCopySend;
      // p..2p-3: recvCopySend; 2p-2: recv
      const bool do_recv = step > 0;
      const bool do_send = step < 2 * p - 2;
      const bool reduce = step < p;            // reduce-scatter half (incl. the finishing step)
      const bool finish = (step == p - 1);     // the chunk completes here: post-op + output
      const bool part_in = do_recv && reduce;  // a partial arrives through the FIFO
      const bool part_out = step < p - 1;      // a partial leaves through the FIFO
      const bool peer_out = do_send && !part_out;  // the output slice is what the successor reads next
      // chunk handled at this step
      int c;
      if (step < p) c = r - 1 - step;          // send0: r-1; recvReduceSend j: r-1-j; finishing: r
      else c = r - (step - p + 1);             // recvCopySend j: r-j; recv: r-(p-1)
      c = ((c % p) + p) % p;
      const int64_t clo = a.lo[c], chi = a.lo[c + 1];
      const int64_t clen = chi - clo;
      // channel slice of the chunk, its inner boundaries on whole vectors
      const int64_t s_lo = clo + (clen * ch / a.C) / V * V;
      const int64_t s_hi = (ch + 1 == a.C) ? chi : clo + (clen * (ch + 1) / a.C) / V * V;
      const int64_t e0 = s_lo + (int64_t)k * a.slot_elems;
      const int64_t e1 = min(s_hi, e0 + (int64_t)a.slot_elems);
      const int64_t len = e1 > e0 ? e1 - e0 : 0;
      // FIFO slots are used by the reduce-scatter sends only: use u of this
      // channel goes to slot u mod NS
      const unsigned long long use_out = (unsigned long long)k * (p - 1) + step;
      const unsigned long long use_in = (unsigned long long)k * (p - 1) + (step - 1);

      // ---- wait for the incoming slot / the predecessor's finished slice ----
      if (do_recv) {
        if (!wait_geq(my_posted, tag(epoch, recvd + 1), a.spin_limit, &ok_recv)) goto timeout;
      }
      // ---- wait until the successor has drained the slot about to be refilled ----
      if (part_out && use_out >= (unsigned long long)a.NS) {
        const unsigned long long u = use_out - a.NS;  // the earlier use of the same slot
        const unsigned long long drained = (u / (p - 1)) * (2 * p - 2) + (u % (p - 1)) + 1;
        if (!wait_geq(nx_consumed, tag(epoch, drained), a.spin_limit, &ok_send)) goto timeout;
      }
      if (len > 0) {
        const int in_base = (int)((use_in % a.NS) * slot_words * 4);   // byte offsets in the FIFOs
        const int out_base = (int)((use_out % a.NS) * slot_words * 4);
        // this slice of my output and of the predecessor's (device-scope access)
        const __amdgpu_buffer_rsrc_t my_y = out_rsrc(yr, e0 * E, len * E);
        const __amdgpu_buffer_rsrc_t pv_y = out_rsrc(a.y[prv], e0 * E, len * E);
        const bool vec = ((e0 % V) == 0);
        // phase 1: issue every load of this step (U vectors per lane)
        u32x4 xin[U];
        u32x4 fin[U][V / 4];
        bool full[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int64_t off = ((int64_t)u * kBlock + tid) * V;
          full[u] = vec && off + V <= len;
          if (full[u]) {
            if (reduce) xin[u] = ld16(xr, (e0 + off) * E);
            if (part_in) {
#pragma unroll
              for (int h = 0; h < V / 4; h++)
                fin[u][h] = __builtin_amdgcn_raw_buffer_load_b128(in_rs, in_base + fifo_off<V>(u, tid, 4 * h), 0, kLd);
            } else if (do_recv) {  // gather: the predecessor's finished storage vector
              fin[u][0] = __builtin_amdgcn_raw_buffer_load_b128(pv_y, (int)(off * E), 0, kLd);
            }
          }
        }
        // phase 2: fold, write the output and the outgoing partial
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int64_t off = ((int64_t)u * kBlock + tid) * V;
          const int64_t i0 = e0 + off;
          if (full[u]) {
            if (reduce) {
              A v[V];
              A own[V];
              unpack<DT>(xin[u], own);
              if (step == 0) {
#pragma unroll
                for (int e = 0; e < V; e++) v[e] = O::pre(own[e], inv_p);
              } else {
#pragma unroll
                for (int h = 0; h < V / 4; h++) {
#pragma unroll
                  for (int e = 0; e < 4; e++) {
                    const uint32_t bits = fin[u][h][e];
                    v[4 * h + e] = __builtin_bit_cast(A, bits);
                  }
                }
#pragma unroll
                for (int e = 0; e < V; e++) v[e] = O::comb(v[e], O::pre(own[e], inv_p));
              }
              if (finish) {
#pragma unroll
                for (int e = 0; e < V; e++) v[e] = O::post(v[e], p);
                __builtin_amdgcn_raw_buffer_store_b128(pack<DT>(v), my_y, (int)(off * E), 0, kSt);
              } else {
#pragma unroll
                for (int h = 0; h < V / 4; h++) {
                  u32x4 q;
#pragma unroll
                  for (int e = 0; e < 4; e++) q[e] = __builtin_bit_cast(uint32_t, v[4 * h + e]);
                  __builtin_amdgcn_raw_buffer_store_b128(q, out_rs, out_base + fifo_off<V>(u, tid, 4 * h), 0, kSt);
                }
              }
            } else {  // gather: keep the finished vector and pass it on through my output
              if (peer_out) __builtin_amdgcn_raw_buffer_store_b128(fin[u][0], my_y, (int)(off * E), 0, kSt);
              else st16(yr, i0 * E, fin[u][0]);
            }
          } else if (off < len) {  // ragged: element by element
            const int cnt = (int)min((int64_t)V, len - off);
            for (int e = 0; e < cnt; e++) {
              const int64_t i = i0 + e;
              const int yoff = (int)((off + e) * E);
              if (reduce) {
                A val;
                const A own = O::pre(load_elem<DT>(xr, i), inv_p);
                if (step == 0) {
                  val = own;
                } else {
                  const uint32_t bits =
                      __builtin_amdgcn_raw_buffer_load_b32(in_rs, in_base + fifo_off<V>(u, tid, e), 0, kLd);
                  val = O::comb(__builtin_bit_cast(A, bits), own);
                }
                if (finish) {
                  val = O::post(val, p);
                  if constexpr (E == 4) __builtin_amdgcn_raw_buffer_store_b32(narrow_bits<DT>(val), my_y, yoff, 0, kSt);
                  else __builtin_amdgcn_raw_buffer_store_b16((unsigned short)narrow_bits<DT>(val), my_y, yoff, 0, kSt);
                } else {
                  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), out_rs,
                                                        out_base + fifo_off<V>(u, tid, e), 0, kSt);
                }
              } else {
                uint32_t word;
                if constexpr (E == 4) word = __builtin_amdgcn_raw_buffer_load_b32(pv_y, yoff, 0, kLd);
                else word = __builtin_amdgcn_raw_buffer_load_b16(pv_y, yoff, 0, kLd);
                if (peer_out) {
                  if constexpr (E == 4) __builtin_amdgcn_raw_buffer_store_b32(word, my_y, yoff, 0, kSt);
                  else __builtin_amdgcn_raw_buffer_store_b16((unsigned short)word, my_y, yoff, 0, kSt);
                } else {
                  if constexpr (E == 4) ((uint32_t*)yr)[i] = word;
                  else ((uint16_t*)yr)[i] = (uint16_t)word;
                }
              }
            }
          }
        }
      }
      // Every wave waits for its own stores (and loads) to complete before
      // the barrier: a workgroup barrier alone does not wait for the other
      // waves' memory operations, so lane 0's signal could otherwise
      // overtake them.
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        if (do_send)
          __hip_atomic_store(nx_posted, tag(epoch, sent + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (do_recv)
          __hip_atomic_store(my_consumed, tag(epoch, recvd + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (do_send) sent++;
      if (do_recv) recvd++;
    }
  }
  return;

timeout:
  if (tid == 0) __hip_atomic_store(a.err, (int)SIM_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT>
static hipError_t fifo_by_op(int op, const RingFifoArgs& a, hipStream_t s) {
  const dim3 g((unsigned)(a.p * a.Cg)), b(kBlock);
  switch (op) {
    case SIM_SUM: return launch<k_ring_fifo<DT, SIM_SUM>>(g, b, s, a);
    case SIM_PROD: return launch<k_ring_fifo<DT, SIM_PROD>>(g, b, s, a);
    case SIM_MIN: return launch<k_ring_fifo<DT, SIM_MIN>>(g, b, s, a);
    case SIM_MAX: return launch<k_ring_fifo<DT, SIM_MAX>>(g, b, s, a);
    case SIM_AVG: return launch<k_ring_fifo<DT, SIM_AVG>>(g, b, s, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ring_fifo(int dtype, int op, const RingFifoArgs& a, hipStream_t s) {
  switch (dtype) {
    case SIM_INT32: return fifo_by_op<SIM_INT32>(op, a, s);
    case SIM_FP32: return fifo_by_op<SIM_FP32>(op, a, s);
    case SIM_FP16: return fifo_by_op<SIM_FP16>(op, a, s);
    case SIM_BF16: return fifo_by_op<SIM_BF16>(op, a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int OP>
static int occ1() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)k_ring_fifo<DT, OP>, kBlock, 0) !=
      hipSuccess)
    return 1;
  return nb > 0 ? nb : 1;
}

template <int DT>
static int occ_op(int op) {
  switch (op) {
    case SIM_SUM: return occ1<DT, SIM_SUM>();
    case SIM_PROD: return occ1<DT, SIM_PROD>();
    case SIM_MIN: return occ1<DT, SIM_MIN>();
    case SIM_MAX: return occ1<DT, SIM_MAX>();
    default: return occ1<DT, SIM_AVG>();
  }
}

int ring_fifo_blocks_per_cu(int dtype, int op) {
  switch (dtype) {
    case SIM_INT32: return occ_op<SIM_INT32>(op);
    case SIM_FP32: return occ_op<SIM_FP32>(op);
    case SIM_FP16: return occ_op<SIM_FP16>(op);
    default: return occ_op<SIM_BF16>(op);
  }
}

}  // namespace simar
