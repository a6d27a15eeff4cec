/*
 * simar.h -- C ABI of libsimar.so: a simulated all-reduce on one MI355X.
 *
 * p simulated ranks each hold a same-shaped buffer in the one HBM.  The
 * library combines them element-wise and leaves every rank's output buffer
 * holding the identical result, executing the chunked schedules the pages
 * describe with hand-written HIP kernels for gfx950:
 *   - the contract (sum, prod, min, max, avg; identical result on every
 *     rank): "Inside NCCL all-reduce" (rakshithvasudev.github.io), section
 *     "What all-reduce promises";
 *   - ring = reduce-scatter then all-gather, 2(p-1) steps: same page,
 *     section "The ring, exactly as the kernel runs it";
 *   - all-pairs (2 steps), one-shot (the two fused in one phase) and the LL
 *     packet protocol: "MSCCL++: Rethinking GPU Communication Abstractions
 *     for AI Inference", sections "The Collective Algorithm Library" (1PA,
 *     2PA, 2PR) and 4.2 (LL protocol); "MSCCL, in depth ...", section
 *     "Writing an algorithm in MSCCLang" (the all-pairs program);
 *   - the alpha-beta selector: "MSCCL, in depth ...", section "Why generic
 *     collectives leave time on the table"; "Inside NCCL all-reduce",
 *     section "How NCCL picks: a cost model, not a threshold".
 *
 * Conventions shared by every entry point:
 *   - Every function returns an int status: SIM_OK (0) or a negative
 *     SIM_ERR_* code.  Argument errors are detected synchronously and
 *     NOTHING is enqueued when an error is returned; there is no silent
 *     fallback to another schedule (the failure mode "MSCCL, in depth ...",
 *     section "How the runtime decides to use your algorithm", warns of).
 *   - Collectives are asynchronous and stream-ordered: they enqueue kernels
 *     on `stream` (a hipStream_t, or NULL for the null stream) and return.
 *     Device buffers are owned by the caller and must stay valid until the
 *     stream work completes.  `in_ptrs` / `out_ptrs` are caller-owned host
 *     arrays of p device pointers; the library copies them into kernel
 *     arguments and keeps no reference after returning.
 *   - Device pointers must be 16-byte aligned (SIM_ERR_ALIGN otherwise).
 *   - In-place means in_ptrs[r] == out_ptrs[r] for every rank; mixing
 *     in-place and out-of-place ranks is SIM_ERR_INVALID_ARG.  Any other
 *     overlap between an output and an input or another output is
 *     SIM_ERR_ALIAS.
 *   - n == 0 is a no-op that returns SIM_OK after the scalar arguments
 *     (p, dtype, op, algo) are checked.
 *   - Chunk c of an n-element buffer is [floor(c*n/p), floor((c+1)*n/p)).
 *   - One host thread per process drives the library (no internal locking).
 *     Calls make the library's device (the one given to sim_init) current
 *     on the calling thread when another one is.
 *   - Graph capture: a collective enqueued on a stream that is being
 *     captured (hipStreamBeginCapture, torch.cuda.graph) is recorded like
 *     any other kernel launch and may be replayed.  SIM_ALGO_ONESHOT_LL,
 *     SIM_ALGO_RING_FIFO and SIM_ALGO_ALLPAIRS_PERSISTENT carry a per-call
 *     epoch in their kernel arguments,
 *     which a replay would repeat: under capture they are
 *     SIM_ERR_UNSUPPORTED and AUTO skips them.  Library scratch cannot grow
 *     during capture (SIM_ERR_UNSUPPORTED): size it with sim_init's
 *     max_bytes_per_rank or make one uncaptured call of the same shape
 *     first.  Once a call has been captured, outgrown scratch is kept until
 *     sim_finalize, so recorded graphs stay valid until then (not after).
 *   - Co-residency: SIM_ALGO_RING_FIFO, SIM_ALGO_ALLPAIRS_PERSISTENT and
 *     SIM_ALGO_ONESHOT_LL run workgroups that wait on one another (the LL
 *     consumers poll packets other workgroups of the same launch write), so
 *     all of them must be resident on the GPU at once.  The library sizes the grid from the
 *     kernels' occupancy on an otherwise idle GPU; kernels running at the
 *     same time on other streams may hold CUs those workgroups need.  Every
 *     wait is bounded: such a call then ends with SIM_ERR_TIMEOUT (reported
 *     by sim_check_error; that call's outputs are undefined), never a hang;
 *     a workgroup whose wait expired gives up its remaining waits at once.
 *     AUTO does not pick these three schedules on MI355X (the calibrated
 *     model ranks the one-shot first at every size and under every budget
 *     the calibration checks), but it may with another calibration file:
 *     callers that run other kernels concurrently should name a schedule.
 *   - Phased kernels: SIM_ALGO_ONESHOT, step 1 of SIM_ALGO_ALLPAIRS and
 *     the direct (SIM_ALGO_ALLPAIRS) reduce-scatter (input bytes per rank;
 *     when n_out_per_rank fills whole 16-byte vectors), step 2 of
 *     SIM_ALGO_ALLPAIRS and the direct all-gather (output bytes per rank;
 *     when n_in_per_rank fills whole 16-byte vectors), each from a size per
 *     rank that depends on the form and on p (SIM_DEBUG_PHASED_MIN; at
 *     p = 8: one-shot 12 MiB, reduce-scatter and step 1 24 MiB, all-gather
 *     and step 2 24 MiB), for p = 2, 4, 8, 16
 *     and not under capture, under a workgroup budget or through
 *     sim_allreduce_noalloc, run as one persistent grid that meets at grid
 *     barriers between reading and writing.  The barriers order the traffic
 *     and guard no data (every element is read, folded and written by one
 *     lane), so its results never depend on co-residency: a wait that finds
 *     the grid not all resident gives up after a bounded number of polls
 *     and the call completes correctly, only slower.  A phased call on
 *     another stream while the previous phased grid may still run takes
 *     the fused kernel instead.  Its barrier state is library memory; calls
 *     on different streams may overlap.
 *   - Shared library buffers: the partial scratch (16-bit ring, tree,
 *     recursive exchange and 2PH all-reduces; the ring reduce-scatter), the
 *     LL packet buffer (the LL one-shot and the single-launch ring's LL
 *     protocol), and the FIFOs and counters of the single-launch ring and
 *     all-pairs belong to the library, one set per process.  Calls
 *     that use one of them must not run at the same time on different
 *     streams (calls on one stream are ordered); one-shot, all-pairs, the
 *     32-bit ring all-reduce, the ring all-gather and the all-pairs
 *     reduce-scatter / all-gather use none and may overlap freely.
 *   - Pointer table: the first 512 distinct (p, in_ptrs, out_ptrs) sets of
 *     SIM_ALGO_ONESHOT, SIM_ALGO_ALLPAIRS and SIM_ALGO_RING all-reduce calls
 *     made outside graph capture are copied once (asynchronously, on the
 *     call's stream) into a device-memory table
 *     that the library owns until sim_finalize; later calls with the same
 *     set launch with argument blocks of at most 64 bytes instead of the
 *     full pointer lists, which are cheaper to enqueue.  Entries hold addresses only (no
 *     ownership) and are never rewritten or evicted; other sets, captured
 *     calls, and calls made while a set's copy has not completed yet carry
 *     their pointers in the kernel arguments.  Results are the same either
 *     way.
 *
 * Results: int32 and fp32 results are bit-exact functions of the schedule:
 * ring chunk c (both ring executions) folds ranks c+1, c+2, ..., c+p
 * (mod p) left to right;
 * all-pairs, one-shot and LL fold the owner c first and then the other
 * ranks in ascending order; the tree folds each rank's own value and then
 * its children's subtree totals in ascending rank order; the recursive
 * exchange folds each group in ascending rank order, lowest base-k digit
 * first; 2PH folds a node's ranks starting with the rank that holds the
 * chunk, then the node partials (small form: nodes ascending; large form:
 * the owner's node first, then the others ascending).  Every rank's output
 * is the same bits.  fp16/bf16 are widened exactly to fp32,
 * accumulated in fp32 (ring partials are kept in fp32) and rounded once,
 * to nearest even, at the final write.  fp avg multiplies each operand by
 * fp32(1/p) as it is read; int32 avg divides the wrapped int32 sum by p
 * once (truncating).  int32 sum/prod wrap modulo 2^32.
 */
#ifndef SIMAR_H
#define SIMAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  SIM_OK = 0,
  SIM_ERR_INVALID_ARG = -1,  /* bad p, NULL pointer, unknown code, mixed in-place */
  SIM_ERR_UNSUPPORTED = -2,  /* legal call, but this algo cannot serve it (e.g. LL above its buffer) */
  SIM_ERR_ALIGN = -3,        /* a device pointer is not 16-byte aligned */
  SIM_ERR_ALIAS = -4,        /* an output overlaps an input or another output */
  SIM_ERR_NOMEM = -5,        /* library scratch could not be allocated */
  SIM_ERR_HIP = -6,          /* a HIP runtime call or kernel launch failed */
  SIM_ERR_TIMEOUT = -7,      /* a bounded device-side wait expired (reported by sim_check_error) */
  SIM_ERR_VERIFY = -8,       /* a schedule failed the symbolic verifier */
  SIM_ERR_NOT_INIT = -9      /* sim_init has not been called */
};

/* ---- element types, reduction ops, schedules -------------------------- */
enum { SIM_INT32 = 0, SIM_FP32 = 1, SIM_FP16 = 2, SIM_BF16 = 3 };
enum { SIM_SUM = 0, SIM_PROD = 1, SIM_MIN = 2, SIM_MAX = 3, SIM_AVG = 4 };
enum {
  SIM_ALGO_AUTO = 0,        /* alpha-beta argmin over the legal schedules 1..5 and 10
                               (the topology schedules 6..9 run only when named) */
  SIM_ALGO_RING = 1,        /* 2(p-1) steps, one launch per step */
  SIM_ALGO_ALLPAIRS = 2,    /* 2 steps: owner gather-reduce, then fan-out */
  SIM_ALGO_ONESHOT = 3,     /* the 2 all-pairs steps fused in one launch */
  SIM_ALGO_ONESHOT_LL = 4,  /* one-shot through 8-byte data+flag packets */
  SIM_ALGO_RING_FIFO = 5,   /* the ring in ONE launch: persistent workgroups, bounded
                               FIFOs between neighbours, in-kernel signal/wait; up to
                               SIM_DEBUG_RING_LL_MAX bytes per rank (256 KiB) every hop
                               is instead one polled LL packet (NCCL's LL protocol) */
  SIM_ALGO_TREE = 6,        /* double binary tree: each half of the buffer reduced up
                               and broadcast down one of two complementary trees */
  SIM_ALGO_REXCH = 7,       /* k-ary recursive exchange: log_k(p) rounds */
  SIM_ALGO_HIER = 8,        /* 2PH, small-message form: node-local reduce-scatter into
                               G chunks, all-pairs across nodes, node-local all-gather */
  SIM_ALGO_HIER_LARGE = 9,  /* 2PH, large-message form: p chunks; node-local and
                               cross-node reduce-scatter, then the two all-gathers */
  SIM_ALGO_ALLPAIRS_PERSISTENT = 10  /* the 2 all-pairs steps in ONE launch: persistent
                               workgroups, each owner signals its finished chunk and
                               the other ranks wait and pull it (in-kernel signal/wait) */
};
#define SIM_NUM_ALGOS 11

#define SIM_MAX_RANKS 16
/* LL packets carry 4 data bytes in 8: the LL buffer holds 2x the payload.
 * LL is legal for messages of at most this many bytes per rank. */
#define SIM_LL_MAX_BYTES_PER_RANK ((size_t)1 << 20)

/* ---- lifetime ---------------------------------------------------------- */

/* Initialise the library on HIP device `device` for up to p_max ranks
 * (2..SIM_MAX_RANKS).  Allocates the device error word, the LL packet
 * buffer (p_max * 2 * SIM_LL_MAX_BYTES_PER_RANK bytes), the single-launch
 * ring's semaphores (its FIFOs, p * channels * slots * 32 KiB at most,
 * are allocated on first use and grown when needed) and, when
 * max_bytes_per_rank > 0, the ring/reduce-scatter partial scratch for
 * messages up to that size (otherwise scratch grows on first need).
 * Calling it again re-initialises (finalize + init).  Errors:
 * SIM_ERR_INVALID_ARG, SIM_ERR_HIP, SIM_ERR_NOMEM. */
int sim_init(int device, int p_max, size_t max_bytes_per_rank);

/* Free everything sim_init allocated (synchronises the device first). */
int sim_finalize(void);

/* ---- collectives -------------------------------------------------------- */

/* All-reduce: out_ptrs[r][i] = X[0][i] (+) ... (+) X[p-1][i] for every rank
 * r, each buffer holding n elements of `dtype`, combined with `op` in the
 * fold order of `algo` (see the header comment).  algo SIM_ALGO_AUTO picks
 * the schedule with sim_select().  Ring on fp16/bf16 keeps fp32 partials in
 * library scratch (8 * ceil512(ceil(n/p) + 8) * p bytes).  Errors: every code
 * above except SIM_ERR_TIMEOUT/SIM_ERR_VERIFY (asynchronous device errors
 * come back through sim_check_error). */
int sim_allreduce(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n,
                  int dtype, int op, int algo, void* stream);

/* Allocation-free all-reduce, for callers that cannot allocate device
 * memory while they run: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same call as sim_allreduce, with
 * the same arguments, checks, fold orders and bit-identical results, for
 * algo SIM_ALGO_ONESHOT, SIM_ALGO_ALLPAIRS, SIM_ALGO_RING or SIM_ALGO_AUTO
 * (the selector's argmin over these three; sim_last_algo reports the
 * pick); any other schedule is SIM_ERR_UNSUPPORTED.  It allocates nothing:
 * no hipMalloc or hipFree, no scratch growth, no pointer-table entry (the
 * pointers travel in the kernel arguments).  The only scratch, the fp32
 * partial slots of the fp16/bf16 ring (p > 2), lives in a fixed device
 * array of SIM_NOALLOC_SCRATCH_BYTES that the library's code object holds
 * on every device it is loaded on until the process ends: the call needs
 * 8 p ceil512(ceil(n/p) + 8) bytes of it (ceil512: rounded up to a
 * multiple of 512): at p = 8 up to 8,388,544 elements per rank (16 MiB - 128 B of
 * bf16).  A larger message is SIM_ERR_NOMEM with nothing enqueued.  Nothing in
 * the array has to start at zero (every partial is written before it is
 * read).  The array is shared by every call of this entry point on one
 * device and keeps the last call's contents: calls that overlap in time on
 * one device (on different streams, or from different host threads) race
 * on it; calls on one stream are ordered.  Errors: as sim_allreduce, plus
 * SIM_ERR_NOMEM as above. */
#define SIM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sim_allreduce_noalloc(const void* const* in_ptrs, void* const* out_ptrs, int p, size_t n, int dtype,
                          int op, int algo, void* stream);

/* Reduce-scatter ("Inside NCCL all-reduce", "What all-reduce promises":
 * every rank ends owning the finished reduction of one slice): inputs hold
 * p * n_out_per_rank elements; out_ptrs[r] (n_out_per_rank elements)
 * receives the reduction of chunk r.  algo: SIM_ALGO_RING (the ring's
 * reduce-scatter half, p-1 steps, partials in library scratch) or
 * SIM_ALGO_ALLPAIRS (direct: each owner gathers and folds its chunk, one
 * step); SIM_ALGO_AUTO picks ALLPAIRS.  Fold orders as for sim_allreduce. */
int sim_reduce_scatter(const void* const* in_ptrs, void* const* out_ptrs, int p,
                       size_t n_out_per_rank, int dtype, int op, int algo, void* stream);

/* All-gather: out_ptrs[r][q*n_in_per_rank + i] = in_ptrs[q][i] for all r,
 * q (a bit copy).  algo: SIM_ALGO_RING (own block placed, then p-1
 * forwarding steps) or SIM_ALGO_ALLPAIRS (direct fan-out, one step);
 * SIM_ALGO_AUTO picks ALLPAIRS.  In-place is in_ptrs[r] == out_ptrs[r] +
 * r*n_in_per_rank*esize for every r. */
int sim_all_gather(const void* const* in_ptrs, void* const* out_ptrs, int p,
                   size_t n_in_per_rank, int dtype, int algo, void* stream);

/* ---- selection and the cost model ------------------------------------- */

/* The schedule SIM_ALGO_AUTO would run for this call, with its predicted
 * time in microseconds: argmin over legal algos of
 *   T_a = alpha_a * launches_a(p) + traffic_a(p, n, dtype) / B_a
 * (a launch cost plus bytes over bandwidth), traffic_a being the schedule's
 * algorithmic HBM bytes over all simulated ranks.  Under a workgroup budget
 * W (SIM_CONFIG_MAX_WORKGROUPS > 0) an algo with a per-workgroup rate b_a
 * (sim_model_set_workgroup_rate, or "wg_gbps" in the calibration file) is
 * priced with B_a replaced by (B_a^-3 + (W_a b_a)^-3)^(-1/3), the smooth
 * minimum of B_a and what W_a workgroups sustain; W_a = W, or max(W, p) for
 * SIM_ALGO_RING_FIFO and SIM_ALGO_ALLPAIRS_PERSISTENT, which keep one
 * workgroup per rank ("T-CCL ...", sections III-C3 and IV-B: restricted
 * mode).  The budget in effect is the current SIM_CONFIG_MAX_WORKGROUPS.
 * An algo with a host enqueue cost H_a per launch (sim_model_set_host_overlap,
 * or "host_us" in the calibration file) is priced max(H_a * launches_a, T_a):
 * calls issued back to back overlap the host's enqueue of one call with the
 * GPU's execution of the previous one, so a call costs whichever side is
 * slower; H_a = 0 leaves T_a as it is.  Two algos change kernels with the
 * size, and the model may hold a second (alpha, B, ...) entry for each,
 * used from that size on: SIM_ALGO_RING_FIFO above SIM_DEBUG_RING_LL_MAX
 * bytes per rank (the FIFO protocol instead of LL packets), and
 * SIM_ALGO_ONESHOT from the size where it runs phased (see "Phased
 * kernels"; never under a workgroup budget). */
int sim_select(int p, size_t n, int dtype, int op, int* algo_out, double* predicted_us);

/* The algo the most recent successful collective actually ran. */
int sim_last_algo(void);

/* Load per-algo alpha (us per launch) and B (GB/s) from a JSON file
 * written by the calibration sweep, and its optional launch table
 * ("workgroups": {algo: [[bytes per rank, total workgroups(, vectors per
 * lane)], ...]}, after T-CCL's ranked launch-configuration table, section
 * III-C3): bulk kernels of that algo then launch the measured best total of
 * the nearest size (log scale), never more than covers the transfer, with
 * the entry's 16-byte vectors per lane (1 or 2; 1 when absent).  A
 * top-level "p" (2..16) names the rank count the table was measured at;
 * calls with another rank count then ignore the table.  An algo
 * entry may carry "wg_gbps", its per-workgroup rate under a budget, and
 * "host_us", its host enqueue cost per launch (see sim_select; 0 when
 * absent).  An optional "algos_hi" object holds second entries of the same
 * form for the algos whose kernels change with the size (see sim_select);
 * an algo listed in "algos" but not in "algos_hi" gets one entry for every
 * size.  Errors: SIM_ERR_INVALID_ARG (the current model is kept). */
int sim_model_load(const char* json_path);

/* Predicted time of `algo` for `bytes_per_rank` bytes per rank of `dtype`
 * (the element size fixes the element count the traffic laws take), under
 * the current workgroup budget as sim_select prices it. */
int sim_model_predict(int algo, int p, int dtype, double bytes_per_rank, double* us_out);

/* Set one algo's host enqueue cost per launch (microseconds; 0 removes the
 * term).  Errors: SIM_ERR_INVALID_ARG (unknown algo, negative or NaN). */
int sim_model_set_host_overlap(int algo, double host_us_per_launch);

/* Set one algo's per-workgroup rate b (GB/s one workgroup sustains; 0
 * removes the budget term, so a budget leaves that algo's B unchanged).
 * Errors: SIM_ERR_INVALID_ARG (unknown algo, negative or NaN rate). */
int sim_model_set_workgroup_rate(int algo, double gbps_per_workgroup);

/* Override one algo's model: alpha_us and gbps always; `steps` (latency
 * units) and `bytes_factor` (bytes moved per byte of message) replace the
 * built-in laws when >= 0 -- e.g. the multi-GPU form 2(p-1) alpha +
 * 2(p-1)/p n / B.  Pass negative values to keep the built-in laws.  The
 * algo's host enqueue term is cleared (the additive form exactly as given);
 * its per-workgroup rate is kept; a second entry it had for large sizes is
 * dropped (this one then prices every size). */
int sim_model_set(int algo, double alpha_us, double steps, double bytes_factor, double gbps);

/* Restore the built-in default model. */
int sim_model_reset(void);

/* ---- device errors ------------------------------------------------------ */

/* Synchronise `stream`, then return and clear the device error word:
 * SIM_OK, or SIM_ERR_TIMEOUT if a bounded wait expired since the last
 * check (that call's outputs are undefined). */
int sim_check_error(void* stream);

/* ---- measurement --------------------------------------------------------- */

/* k independent copies in one launch: dst_ptrs[q][0 .. bytes) =
 * src_ptrs[q][0 .. bytes) for q < k, asynchronously on `stream`.  Each lane
 * moves 16-byte vectors with the same streaming loads and stores, address
 * split and grid-stride walk as the one-shot's fold, so k = p measures what
 * the one-shot's access pattern (p input and p output streams, "MSCCL++
 * ...", section "The Collective Algorithm Library", 1PA) can reach on this
 * GPU without its arithmetic, and k = 1 a plain copy: the same-GPU ceiling
 * the one-shot's HBM bandwidth is read against.  `workgroups` is the grid
 * size (0: one workgroup per 256 vectors of a stream, at most 2^20).
 * Pointers are caller-owned device memory, 16-byte aligned; no destination
 * may overlap a source or another destination.  Errors: SIM_ERR_NOT_INIT,
 * SIM_ERR_INVALID_ARG (k outside 1..SIM_MAX_RANKS, a NULL pointer, bytes
 * not a multiple of 16, workgroups < 0), SIM_ERR_ALIGN, SIM_ERR_ALIAS,
 * SIM_ERR_HIP; nothing is enqueued on an error.  bytes == 0 is a no-op. */
int sim_copy_streams(const void* const* src_ptrs, void* const* dst_ptrs, int k, size_t bytes, int workgroups,
                     void* stream);

/* ---- topology (host only; no device needed) ------------------------- */

/* The simulated topology that SIM_ALGO_TREE, SIM_ALGO_REXCH, SIM_ALGO_HIER
 * and SIM_ALGO_HIER_LARGE follow ("Inside NCCL all-reduce", section "The
 * double binary tree": trees link nodes, a node's ranks form a chain;
 * "MSCCL++ ...", section "The Collective Algorithm Library", 2PH: local
 * collectives inside a node; "Demystifying NVSHMEM", Fig. 7: k-ary
 * recursive exchange).  Process-wide settings, kept across sim_init.
 *   SIM_CONFIG_RANKS_PER_NODE  G: ranks kG .. kG+G-1 form node k.  1..16,
 *                              default 1.  Collectives with a G that does
 *                              not divide p are SIM_ERR_UNSUPPORTED for the
 *                              algos that use it.
 *   SIM_CONFIG_RADIX           k of the recursive exchange, 2..16, default
 *                              2; it needs p to be a power of k
 *                              (SIM_ERR_UNSUPPORTED otherwise).
 *   SIM_CONFIG_MAX_WORKGROUPS  workgroup budget of every launch (T-CCL's
 *                              restricted mode, "T-CCL ...", sections III-C3
 *                              and IV-B: communication limited to a fixed
 *                              number of thread blocks so the rest of the GPU
 *                              stays free for compute).  0 (default) = no cap;
 *                              the single-launch ring still uses at least one
 *                              workgroup per rank.  Below the CU count, where
 *                              it caps the launch, the fused fold (one-shot,
 *                              all-pairs step 1, direct reduce-scatter) keeps
 *                              4 vectors per lane in flight instead of the
 *                              launch table's 1 or 2.
 *                              Results do not depend on it.
 * Out-of-range values are SIM_ERR_INVALID_ARG and change nothing. */
enum { SIM_CONFIG_RANKS_PER_NODE = 0, SIM_CONFIG_RADIX = 1, SIM_CONFIG_MAX_WORKGROUPS = 2 };
int sim_config_set(int key, int value);
int sim_config_get(int key, int* value);

/* The rank tree SIM_ALGO_TREE runs for p ranks, G ranks per node.
 * tree 0: NCCL's bit-trick binary tree over the p/G nodes (node k's lowest
 * set bit fixes its height; its parent clears that bit and sets the next
 * one up, or only clears it at the edge of the range; its children are k
 * minus and plus half that bit); tree 1: its mirror image (node x plays
 * node p/G-1-x) for an even node count, the tree shifted by one node for an
 * odd one.  Node k's place is taken by rank kG; ranks kG+1 .. kG+G-1 hang
 * below it as a chain.  *parent gets -1 for the root; children[0..2] get
 * up to three children in ascending order, *nchildren their count. */
int sim_tree_info(int tree, int p, int ranks_per_node, int rank, int* parent, int* children,
                  int* nchildren);

/* ---- schedules and the verifier (host only; no device needed) --------- */

/* The all-reduce schedules below use the current topology settings.
 * Step and transfer counts of the lowered schedule of (algo, p), and the
 * number of chunks it cuts the buffer into (chunk c of nchunks is
 * [floor(c*n/nchunks), floor((c+1)*n/nchunks))).  SIM_ERR_UNSUPPORTED when
 * (algo, p, topology) has no schedule. */
int sim_schedule_info(int algo, int p, int* nsteps, int* nxfers, int* nchunks);

/* The transfers of one step: 5 ints each {kind, src rank, dst rank, chunk,
 * rank set}, kind 0 REDUCE, 1 REDUCE_POST, 2 COPY, 3 GATHER_REDUCE,
 * 4 FANOUT, 5 ONESHOT, 6 GATHER, 7 GATHER_POST, 8 EXCH, 9 EXCH_POST,
 * 10 MCAST; the rank set (bit q = rank q) is used by kinds 6..10:
 *   GATHER(_POST) dst folds into its own value the set's values, ascending;
 *   EXCH(_POST)   dst's value becomes the fold of the set's values
 *                 (the set contains dst), ascending, as before the step;
 *   MCAST         src's finished value is copied to every rank in the set.
 * _POST kinds complete the value.  `*count` gets the number written (at
 * most max). */
int sim_schedule_xfers(int algo, int p, int step, int* out, int max, int* count);

/* Symbolic state after `after_steps` steps: masks[r*nchunks + c] = bit
 * mask of the ranks whose contribution rank r's slot for chunk c holds. */
int sim_schedule_state(int algo, int p, int after_steps, uint32_t* masks);

/* Check() -- run the schedule symbolically and prove that every output
 * chunk holds each rank's contribution exactly once, in the documented
 * fold order, with no read/write hazard inside a step (members of one
 * exchange group excepted) and the closed-form round count.  Returns
 * SIM_OK or SIM_ERR_VERIFY with a message in diag. */
int sim_verify_schedule(int algo, int p, char* diag, size_t diag_len);

/* Same check on a caller-supplied all-reduce schedule over nchunks chunks
 * (nsteps steps; step s has counts[s] transfers laid out as in
 * sim_schedule_xfers, concatenated in xfers).  `algo` names the fold order
 * (and, for the topology algos, the current topology) the result must
 * follow; `rounds` is the round count the schedule claims. */
int sim_verify_custom(int algo, int p, int nchunks, int rounds, int nsteps, const int* counts,
                      const int* xfers, char* diag, size_t diag_len);

/* ---- test hooks --------------------------------------------------------- */
enum {
  SIM_DEBUG_EPOCH = 0,         /* set the LL epoch counter (next call uses value+1) */
  SIM_DEBUG_SPIN_LIMIT = 1,    /* polls before a bounded wait gives up */
  SIM_DEBUG_LL_WAIT_SKEW = 2,  /* consumers wait for epoch+value (0 = normal) */
  SIM_DEBUG_FILL_LL = 3,       /* fill the LL buffer with this 64-bit packet (synchronous) */
  SIM_DEBUG_LOG = 4,           /* 1: log one line per call to stderr (also SIM_DEBUG=1) */
  SIM_DEBUG_WORKGROUPS = 5,    /* force the workgroup count of bulk kernels (0 = heuristic) */
  SIM_DEBUG_UNROLL = 6,        /* 16-byte vectors per lane per pass in bulk kernels: 1, 2 or 4
                                  (4: the fused fold at p = 2, 4, 8; other kernels take 2);
                                  0, the default: the launch table's entry, else 1, and the
                                  fused fold takes 4 where a budget below the CU count caps it */
  SIM_DEBUG_FIFO_CHANNELS = 7, /* single-launch ring: channels per rank, <= 128 (0 = heuristic) */
  SIM_DEBUG_FIFO_SLOTS = 8,    /* single-launch ring: slots per FIFO, 2..8 (default 4) */
  SIM_DEBUG_FIFO_WITHHOLD = 9, /* 1: rank 0's ring workgroups leave at once (forces a bounded-wait expiry) */
  SIM_DEBUG_FIFO_VECS = 10,    /* single-launch ring: 16-byte vectors per lane per slot, 1, 2 or 4 (default 4) */
  SIM_DEBUG_PTR_TABLE = 11,    /* 0: all-reduce calls never use the pointer table (default 1) */
  SIM_DEBUG_PTR_SETS = 12,     /* get only: pointer sets the table holds */
  SIM_DEBUG_RING_LL_MAX = 13,  /* single-launch ring: largest message (bytes per rank) sent as
                                  LL packets (default 256 KiB; 0 = never) */
  SIM_DEBUG_PHASED = 14,       /* phased kernels (one-shot, all-pairs, direct reduce-scatter and
                                  all-gather):
                                  0 from SIM_DEBUG_PHASED_MIN bytes per rank on (default),
                                  1 whenever the call allows it, 2 never */
  SIM_DEBUG_PHASED_MIN = 15,   /* the unit of the phased kernels' thresholds (default 16 MiB):
                                  at p = 8 the one-shot runs phased from 3/4 unit per rank,
                                  all-pairs step 1 and the direct reduce-scatter (input bytes)
                                  and all-pairs step 2 and the direct all-gather (output bytes)
                                  from 1.5; other rank counts have their own multiples (never at
                                  p = 2 for the one-shot, never at p = 4 for the all-gather) */
  SIM_DEBUG_PHASED_EXPIRED = 16, /* phased fold barrier waits that gave up at the spin limit
                                  (synchronizes the device; set only to 0, which clears it) */
  SIM_DEBUG_PHASED_LAST = 17, /* get only: 1 if the last collective call ran a phased kernel */
  SIM_DEBUG_PHASED_LAYOUT = 18, /* the phased one-shot's block layout: 0 (default) the whole
                                  buffer's blocks in turn over the grid where every chunk is the
                                  same whole number of blocks, no fewer than the grid's
                                  workgroups; 1 each chunk's blocks over its own workgroups */
  SIM_DEBUG_PHASED_WHOLE_LAST = 19 /* get only: 1 if the last collective call ran the phased
                                  one-shot in the whole-buffer layout */
};
int sim_debug_set(int key, uint64_t value);
int sim_debug_get(int key, uint64_t* value);
/* The LL epoch hook under its own name: sim_debug_set(SIM_DEBUG_EPOCH,
 * epoch) -- the next LL call uses epoch + 1, so a value near 2^32 forces the
 * wrap (the packet buffer is cleared and the epoch restarts at 1). */
int sim_debug_set_epoch(uint32_t epoch);

const char* sim_status_string(int status);
int sim_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SIMAR_H */
