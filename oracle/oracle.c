/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the simulated
 * all-reduce.  TEST INFRASTRUCTURE ONLY: the product library never links,
 * loads or calls this file.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source with the HIP
 * library (its own enums, codecs and schedule rules, written from the pages).
 *
 * Sources (web pages; the title names the page):
 *  [NCCL]   "Inside NCCL all-reduce" (rakshithvasudev.github.io, 2026-08-02):
 *           section "What all-reduce promises" (the contract, the worked
 *           example, the avg rule), section "The ring, exactly as the kernel
 *           runs it" (the 3-GPU state table, the runRing step sequence).
 *  [MSCCL]  "MSCCL, in depth: custom GPU collective algorithms with MSCCLang,
 *           the XML IR and the selection rules ...": section "Writing an
 *           algorithm in MSCCLang" (the all-pairs program: scatter into
 *           scratch, local reduction, gather), section "Failure modes"
 *           (a different reduction order is not bitwise equal).
 *  [MSCCLPP] "MSCCL++: Rethinking GPU Communication Abstractions for AI
 *           Inference": section "The Collective Algorithm Library" (1PA, 2PA,
 *           2PR, and 2PH: local reduce-scatter, cross-node all-pairs, local
 *           all-gather; small- and large-message forms).
 *  [NCCL]   also section "The double binary tree" (the bit-trick tree, its
 *           14-rank drawing, the mirror/shift second tree, chains inside a
 *           node) and section "How NCCL picks" (the tree's latency count).
 *  [NVSHMEM] "Demystifying NVSHMEM" analysis, Fig. 7 (k-ary recursive
 *           exchange as the P2P all-reduce).
 *
 * Arithmetic.  Accumulation is fp32 for every floating type (the parity bar
 * fixes fp32 accumulation and bit-exact fp32 results in schedule order), and
 * uint32 (wrap mod 2^32) for int32 sum/prod.  Built with gcc -O2
 * -ffp-contract=off and no fast-math, so every a*b and a+b is one correctly
 * rounded IEEE binary32 operation (x86-64 SSE; FLT_EVAL_METHOD == 0).
 * OpenMP parallelises only over elements inside one chunk transfer; each
 * element's own sequence of operations is untouched by it.
 *
 * Readings of points the pages leave open:
 *  - chunk c = elements [floor(c*n/p), floor((c+1)*n/p)).
 *  - ring: at reduce-scatter step s rank r sends chunk (r-1-s) mod p to rank
 *    r+1, which folds its own contribution in (accumulator first); at
 *    all-gather step s rank r forwards chunk (r-s) mod p.  This reproduces
 *    every cell of the 3-GPU table in [NCCL].
 *  - all-pairs / one-shot / LL: owner j of chunk j folds its own element
 *    first, then the other ranks in ascending order (the scratch slots of the
 *    [MSCCL] program are appended in issue order, r1 ascending).
 *  - avg: fp operands are multiplied by fp32(1/p) as they are read; int32
 *    avg divides the wrapped int32 sum once at the end (C truncation).
 *  - 16-bit outputs: partials stay fp32 between ring hops; one RNE narrowing
 *    at the final write.
 *  - min/max: acc = (b < a) ? b : a  /  (b > a) ? b : a, a = accumulator.
 *  - double binary tree: chunk t (t = 0, 1) of the buffer cut in two runs on
 *    tree t; a rank adds its children's subtree totals to its own value in
 *    ascending child order; the root's total is post-processed and is every
 *    rank's result.  Tree two = tree one's mirror (node x plays n-1-x) for
 *    an even node count, tree one shifted by +1 node for an odd one (the
 *    pages move tree one over by a single rank but give no direction: the
 *    +1 is a reading, and parity is unpinned for that direction alone).  With
 *    G ranks per node, node k is rank kG and ranks kG+1..kG+G-1 hang below
 *    it as a chain.
 *  - recursive exchange: p must be k^m; round j (j = 0 first) folds the k
 *    ranks that differ only in base-k digit j, in ascending rank order.
 *  - 2PH: nodes are G consecutive ranks.  Small form: G chunks; chunk i is
 *    folded inside node K by rank (K, i) -- own element, then the node's
 *    others ascending -- and the node partials are folded in ascending node
 *    order.  Large form: p chunks; chunk c is owned by rank c = (K, i);
 *    node partials as above at position i; the owner's node partial first,
 *    then the other nodes' ascending.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- codes (kept numerically equal to the library's public enums) ---- */
enum { OR_INT32 = 0, OR_FP32 = 1, OR_FP16 = 2, OR_BF16 = 3 };
enum { OR_SUM = 0, OR_PROD = 1, OR_MIN = 2, OR_MAX = 3, OR_AVG = 4 };
enum { OR_RING = 1, OR_ALLPAIRS = 2, OR_ONESHOT = 3, OR_ONESHOT_LL = 4, OR_RING_FIFO = 5,
       OR_TREE = 6, OR_REXCH = 7, OR_HIER = 8, OR_HIER_LARGE = 9, OR_ALLPAIRS_PERSISTENT = 10 };
#define OR_MAXP 128
#define OR_EBADARG (-1)

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 / bfloat16 codecs, from the format definitions.   */
/* ------------------------------------------------------------------ */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 = the top 16 bits of a binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even.  The dropped low 16
 * bits are compared against one half unit of the kept part.  NaN stays NaN
 * (quiet bit set); a carry out of the mantissa bumps the exponent, which is
 * exactly the IEEE overflow-to-infinity rule. */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xffffu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept;
}

/* binary16 -> binary32 (exact): sign, 5-bit exponent (bias 15), 10-bit
 * fraction; subnormals are value = fraction * 2^-24. */
float oracle_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  if (e == 0x1fu) return u2f(sign | 0x7f800000u | (m << 13));  /* inf / NaN */
  if (e == 0) {
    if (m == 0) return u2f(sign);
    /* subnormal: m * 2^-24, exact in binary32 */
    float v = (float)m * u2f(0x33800000u); /* 2^-24 */
    return (sign ? -v : v);
  }
  return u2f(sign | ((e - 15u + 127u) << 23) | (m << 13));
}

/* binary32 -> binary16, round to nearest, ties to even.  Works in units of
 * the target's last place: normal results keep 10 fraction bits, subnormal
 * results are integer multiples of 2^-24. */
uint16_t oracle_f32_to_f16(float f) {
  uint32_t u = f2u(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t exp = (u >> 23) & 0xffu;
  uint32_t frac = u & 0x7fffffu;
  if (exp == 0xffu) return (uint16_t)(sign | (frac ? 0x7e00u : 0x7c00u));
  int e16 = (int)exp - 127 + 15;                 /* biased binary16 exponent */
  if (e16 >= 31) return (uint16_t)(sign | 0x7c00u);  /* too large: infinity */
  uint32_t q, rem, half;
  if (e16 <= 0) {
    /* subnormal (or zero) result: value / 2^-24 = sig * 2^(exp-127-23+24) */
    if (exp == 0) return sign;                   /* |f| < 2^-126: rounds to 0 */
    uint32_t sig = 0x800000u | frac;             /* 24 significant bits */
    int shift = 14 - e16;                        /* >= 14 */
    if (shift > 24) return sign;                 /* below half of 2^-24 */
    q = sig >> shift;
    rem = sig & ((1u << shift) - 1u);
    half = 1u << (shift - 1);
  } else {
    q = ((uint32_t)e16 << 10) | (frac >> 13);
    rem = frac & 0x1fffu;
    half = 0x1000u;
  }
  if (rem > half || (rem == half && (q & 1u))) q += 1u;  /* may carry into exp */
  return (uint16_t)(sign | q);
}

void oracle_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_bf16(x[i]);
}
void oracle_f32_to_f16_array(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_f16(x[i]);
}
void oracle_bf16_to_f32_array(const uint16_t* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = oracle_bf16_to_f32(x[i]);
}
void oracle_f16_to_f32_array(const uint16_t* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = oracle_f16_to_f32(x[i]);
}

/* ------------------------------------------------------------------ */
/* One accumulator value: either 32 raw integer bits or an fp32.       */
/* ------------------------------------------------------------------ */
typedef union { uint32_t u; int32_t i; float f; } acc_t;

typedef struct {
  int p, dtype, op;
  float inv_p;    /* fp32(1/p), correctly rounded */
} ctx_t;

static int esize(int dtype) { return (dtype == OR_FP16 || dtype == OR_BF16) ? 2 : 4; }

/* pre(): read element i of a rank's buffer into the accumulator type.
 * fp avg: the contribution is scaled by 1/p as it is read ([NCCL], "What
 * all-reduce promises"). */
static acc_t pre(const ctx_t* c, const void* buf, int64_t i) {
  acc_t a;
  switch (c->dtype) {
    case OR_INT32: a.i = ((const int32_t*)buf)[i]; return a;
    case OR_FP32:  a.f = ((const float*)buf)[i]; break;
    case OR_FP16:  a.f = oracle_f16_to_f32(((const uint16_t*)buf)[i]); break;
    default:       a.f = oracle_bf16_to_f32(((const uint16_t*)buf)[i]); break;
  }
  if (c->op == OR_AVG) {
    volatile float scaled = a.f * c->inv_p;   /* its own rounding step */
    a.f = scaled;
  }
  return a;
}

/* a (+) b, a = the running accumulator, b = the arriving operand. */
static acc_t combine(const ctx_t* c, acc_t a, acc_t b) {
  acc_t r;
  if (c->dtype == OR_INT32) {
    switch (c->op) {
      case OR_SUM: case OR_AVG: r.u = a.u + b.u; break;   /* wraps mod 2^32 */
      case OR_PROD: r.u = a.u * b.u; break;
      case OR_MIN: r.i = (b.i < a.i) ? b.i : a.i; break;
      default:     r.i = (b.i > a.i) ? b.i : a.i; break;
    }
  } else {
    switch (c->op) {
      case OR_SUM: case OR_AVG: r.f = a.f + b.f; break;
      case OR_PROD: r.f = a.f * b.f; break;
      case OR_MIN: r.f = (b.f < a.f) ? b.f : a.f; break;
      default:     r.f = (b.f > a.f) ? b.f : a.f; break;
    }
  }
  return r;
}

/* post(): the fix-up where a chunk's reduction completes: the int avg
 * divide (once, truncating) and the single RNE narrowing of 16-bit types. */
static void post_store(const ctx_t* c, acc_t v, void* buf, int64_t i) {
  switch (c->dtype) {
    case OR_INT32:
      ((int32_t*)buf)[i] = (c->op == OR_AVG) ? (int32_t)(v.i / c->p) : v.i;
      break;
    case OR_FP32: ((float*)buf)[i] = v.f; break;
    case OR_FP16: ((uint16_t*)buf)[i] = oracle_f32_to_f16(v.f); break;
    default:      ((uint16_t*)buf)[i] = oracle_f32_to_bf16(v.f); break;
  }
}

static int64_t chunk_lo(int64_t n, int p, int c) { return (int64_t)(((__int128)c * n) / p); }
static int64_t chunk_of(int64_t n, int p, int64_t i) {
  /* the c with chunk_lo(c) <= i < chunk_lo(c+1) */
  int c = (int)(((__int128)i * p) / (n > 0 ? n : 1));
  while (c > 0 && chunk_lo(n, p, c) > i) c--;
  while (c < p - 1 && chunk_lo(n, p, c + 1) <= i) c++;
  return c;
}

static int check_args(int p, int64_t n, int dtype, int op) {
  if (p < 2 || p > OR_MAXP || n < 0) return OR_EBADARG;
  if (dtype < OR_INT32 || dtype > OR_BF16) return OR_EBADARG;
  if (op < OR_SUM || op > OR_AVG) return OR_EBADARG;
  return 0;
}

static ctx_t make_ctx(int p, int dtype, int op) {
  ctx_t c; c.p = p; c.dtype = dtype; c.op = op;
  volatile float one = 1.0f, fp = (float)p;
  c.inv_p = one / fp;
  return c;
}

/* ------------------------------------------------------------------ */
/* Ring: reduce-scatter in p-1 steps, then all-gather in p-1 steps     */
/* ([NCCL] "The ring, exactly as the kernel runs it"; [MSCCLPP] 2PR).  */
/* P[r] holds rank r's accumulator-typed partial of whichever chunk it  */
/* last received.  Returns the number of steps executed.               */
/* ------------------------------------------------------------------ */
static int ring_reduce_scatter(const ctx_t* c, const void* const* X, void* const* Y,
                               int64_t n, int out_is_chunk) {
  const int p = c->p;
  acc_t* P = (acc_t*)malloc(sizeof(acc_t) * (size_t)(n > 0 ? n : 1) * (size_t)p);
  if (!P) return OR_EBADARG;
  int steps = 0;
  for (int s = 0; s <= p - 2; s++) {
    for (int r = 0; r < p; r++) {
      const int ch = ((r - 1 - s) % p + p) % p;    /* chunk rank r sends */
      const int d = (r + 1) % p;                   /* its ring successor */
      const int64_t lo = chunk_lo(n, p, ch), hi = chunk_lo(n, p, ch + 1);
      acc_t* Pr = P + (size_t)r * (size_t)n;
      acc_t* Pd = P + (size_t)d * (size_t)n;
      #pragma omp parallel for schedule(static)
      for (int64_t i = lo; i < hi; i++) {
        acc_t a = (s == 0) ? pre(c, X[r], i) : Pr[i];
        acc_t v = combine(c, a, pre(c, X[d], i));
        if (s == p - 2) {
          /* the chunk completes at its owner d == ch: postOp here */
          if (out_is_chunk) post_store(c, v, Y[d], i - lo);
          else post_store(c, v, Y[d], i);
        } else {
          Pd[i] = v;
        }
      }
    }
    steps++;
  }
  free(P);
  return steps;
}

static int ring_all_gather_inplace(const ctx_t* c, void* const* Y, int64_t n) {
  const int p = c->p, e = esize(c->dtype);
  int steps = 0;
  for (int s = 0; s <= p - 2; s++) {
    for (int r = 0; r < p; r++) {
      const int ch = ((r - s) % p + p) % p;
      const int d = (r + 1) % p;
      const int64_t lo = chunk_lo(n, p, ch), hi = chunk_lo(n, p, ch + 1);
      memcpy((char*)Y[d] + lo * e, (const char*)Y[r] + lo * e, (size_t)((hi - lo) * e));
    }
    steps++;
  }
  return steps;
}

/* ------------------------------------------------------------------ */
/* All-pairs: step 1, owner j gathers chunk j from every rank and folds  */
/* it (own element first, then the others ascending); step 2, owner j   */
/* sends the finished chunk to every other rank ([MSCCL] "Writing an    */
/* algorithm in MSCCLang"; [MSCCLPP] 2PA).  One-shot and LL compute the  */
/* same fold for every element in one phase ([MSCCLPP] 1PA), so the      */
/* oracle for them is this schedule.                                     */
/* ------------------------------------------------------------------ */
static void allpairs_fold_chunk(const ctx_t* c, const void* const* X, void* out,
                                int64_t n, int j, int64_t out_offset) {
  const int p = c->p;
  const int64_t lo = chunk_lo(n, p, j), hi = chunk_lo(n, p, j + 1);
  #pragma omp parallel for schedule(static)
  for (int64_t i = lo; i < hi; i++) {
    acc_t v = pre(c, X[j], i);
    for (int q = 0; q < p; q++) {
      if (q == j) continue;
      v = combine(c, v, pre(c, X[q], i));
    }
    post_store(c, v, out, i - out_offset);
  }
}

static int allpairs(const ctx_t* c, const void* const* X, void* const* Y, int64_t n) {
  const int p = c->p, e = esize(c->dtype);
  for (int j = 0; j < p; j++) allpairs_fold_chunk(c, X, Y[j], n, j, 0);   /* step 1 */
  for (int j = 0; j < p; j++) {                                           /* step 2 */
    const int64_t lo = chunk_lo(n, p, j), hi = chunk_lo(n, p, j + 1);
    for (int r = 0; r < p; r++) {
      if (r == j) continue;
      memcpy((char*)Y[r] + lo * e, (const char*)Y[j] + lo * e, (size_t)((hi - lo) * e));
    }
  }
  return 2;
}

/* ------------------------------------------------------------------ */
/* Topology schedules: each rank's result is computed element by element */
/* straight from the algorithm's definition.                             */
/* ------------------------------------------------------------------ */
typedef struct {
  int algo, G, k;              /* ranks per node, radix */
  int nchunks;
  int parent[2][OR_MAXP];      /* rank trees (double binary tree) */
} topo_t;

/* NCCL's tree over n nodes, by its parent rule only ([NCCL] "The double
 * binary tree"): the lowest set bit b of x is cleared and the next bit up is
 * set; if that leaves the node range, b is only cleared.  Node 0 is the
 * root.  Children are found by inverting this relation. */
static int bittree_parent(int n, int x) {
  if (x == 0) return -1;
  int b = 1;
  while (!(x & b)) b <<= 1;
  int up = (x & ~b) | (b << 1);
  if (up >= n) up = x & ~b;
  return up;
}

/* Node parent in tree t: t = 1 relabels tree one's nodes, x -> n-1-x when
 * n is even, x -> x+1 (mod n) when n is odd. */
static int node_parent(int t, int n, int x) {
  if (t == 0) return bittree_parent(n, x);
  if (n % 2 == 0) {
    int q = bittree_parent(n, n - 1 - x);
    return q < 0 ? -1 : n - 1 - q;
  }
  int q = bittree_parent(n, (x + n - 1) % n);
  return q < 0 ? -1 : (q + 1) % n;
}

static int topo_init(topo_t* T, int algo, int p, int G, int k) {
  memset(T, 0, sizeof *T);
  T->algo = algo; T->G = G; T->k = k;
  if (algo == OR_TREE || algo == OR_HIER || algo == OR_HIER_LARGE)
    if (G < 1 || p % G != 0) return OR_EBADARG;
  if (algo == OR_TREE) {
    const int nn = p / G;
    for (int t = 0; t < 2; t++)
      for (int r = 0; r < p; r++) {
        if (r % G != 0) { T->parent[t][r] = r - 1; continue; }   /* chain inside the node */
        int up = node_parent(t, nn, r / G);
        T->parent[t][r] = up < 0 ? -1 : up * G;
      }
    T->nchunks = 2;
  } else if (algo == OR_REXCH) {
    if (k < 2) return OR_EBADARG;
    int v = 1;
    while (v < p) v *= k;
    if (v != p) return OR_EBADARG;
    T->nchunks = 1;
  } else if (algo == OR_HIER) {
    T->nchunks = G;
  } else if (algo == OR_HIER_LARGE) {
    T->nchunks = p;
  } else {
    return OR_EBADARG;
  }
  return 0;
}

/* Subtree total of rank r in tree t: own value, then each child's subtree
 * total, children in ascending rank order. */
static acc_t subtree(const ctx_t* c, const topo_t* T, const void* const* X, int t, int r, int64_t i) {
  acc_t v = pre(c, X[r], i);
  for (int q = 0; q < c->p; q++)
    if (q != r && T->parent[t][q] == r) v = combine(c, v, subtree(c, T, X, t, q, i));
  return v;
}

/* Node K's partial of element i at local position pos: rank (K, pos) first,
 * then the node's other ranks ascending. */
static acc_t node_partial(const ctx_t* c, int G, const void* const* X, int K, int pos, int64_t i) {
  acc_t v = pre(c, X[K * G + pos], i);
  for (int j = 0; j < G; j++)
    if (j != pos) v = combine(c, v, pre(c, X[K * G + j], i));
  return v;
}

/* The value rank r ends with at element i (before post-processing). */
static acc_t topo_value(const ctx_t* c, const topo_t* T, const void* const* X, int64_t n, int r, int64_t i) {
  const int p = c->p;
  const int ch = (int)chunk_of(n, T->nchunks, i);
  switch (T->algo) {
    case OR_TREE: {
      int root = 0;
      while (T->parent[ch][root] >= 0) root = T->parent[ch][root];   /* walk up from rank 0 */
      return subtree(c, T, X, ch, root, i);
    }
    case OR_REXCH: {
      acc_t v[OR_MAXP], w[OR_MAXP];
      for (int q = 0; q < p; q++) v[q] = pre(c, X[q], i);
      for (int stride = 1; stride < p; stride *= T->k) {
        for (int q = 0; q < p; q++) {
          const int digit = (q / stride) % T->k;
          const int first = q - digit * stride;      /* the group's lowest rank */
          acc_t a = v[first];
          for (int m = 1; m < T->k; m++) a = combine(c, a, v[first + m * stride]);
          w[q] = a;
        }
        memcpy(v, w, sizeof(acc_t) * (size_t)p);
      }
      return v[r];
    }
    case OR_HIER: {
      acc_t a = node_partial(c, T->G, X, 0, ch, i);
      for (int K = 1; K < p / T->G; K++) a = combine(c, a, node_partial(c, T->G, X, K, ch, i));
      return a;
    }
    default: {   /* OR_HIER_LARGE: chunk ch is owned by rank ch */
      const int K0 = ch / T->G, pos = ch % T->G;
      acc_t a = node_partial(c, T->G, X, K0, pos, i);
      for (int K = 0; K < p / T->G; K++)
        if (K != K0) a = combine(c, a, node_partial(c, T->G, X, K, pos, i));
      return a;
    }
  }
}

/* Communication rounds: tree, 2 x the root's height (up, then down);
 * recursive exchange, log_k p; 2PH, one per phase that has work. */
static int topo_rounds(const topo_t* T, int p) {
  if (T->algo == OR_TREE) {
    int h = 0;
    for (int r = 0; r < p; r++) {       /* deepest rank in tree one */
      int d = 0;
      for (int q = r; T->parent[0][q] >= 0; q = T->parent[0][q]) d++;
      if (d > h) h = d;
    }
    return 2 * h;
  }
  if (T->algo == OR_REXCH) {
    int m = 0;
    for (int v = 1; v < p; v *= T->k) m++;
    return m;
  }
  const int local = T->G > 1, cross = p / T->G > 1;
  return (T->algo == OR_HIER) ? 2 * local + cross : 2 * local + 2 * cross;
}

static int topo_allreduce(const ctx_t* c, const void* const* X, void* const* Y, int64_t n,
                          int algo, int G, int k) {
  const int p = c->p;
  topo_t T;
  if (topo_init(&T, algo, p, G, k)) return OR_EBADARG;
  const int e = esize(c->dtype);
  /* results go to a separate buffer first so that in-place calls read
   * untouched inputs */
  char* out = (char*)malloc((size_t)(n > 0 ? n : 1) * (size_t)e * (size_t)p);
  if (!out) return OR_EBADARG;
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++)
    for (int r = 0; r < p; r++)
      post_store(c, topo_value(c, &T, X, n, r, i), out + (size_t)r * (size_t)n * (size_t)e, i);
  for (int r = 0; r < p; r++) memcpy(Y[r], out + (size_t)r * (size_t)n * (size_t)e, (size_t)n * (size_t)e);
  free(out);
  return topo_rounds(&T, p);
}

/* Parent of rank r in tree t (0 or 1) of the double binary tree over p
 * ranks with G ranks per node; -1 for the root, -2 for bad arguments. */
int oracle_tree_parent(int t, int p, int G, int r) {
  topo_t T;
  if (p < 1 || p > OR_MAXP || t < 0 || t > 1 || r < 0 || r >= p) return -2;
  if (topo_init(&T, OR_TREE, p, G, 2)) return -2;
  return T.parent[t][r];
}

/* ------------------------------------------------------------------ */
/* Public entry points.  X, Y: arrays of p host pointers.  In-place      */
/* (X[r] == Y[r]) is allowed.  Return: steps executed, or -1.            */
/* ------------------------------------------------------------------ */
int oracle_allreduce_topo(const void* const* X, void* const* Y, int p, int64_t n,
                          int dtype, int op, int algo, int ranks_per_node, int radix) {
  if (check_args(p, n, dtype, op)) return OR_EBADARG;
  ctx_t c = make_ctx(p, dtype, op);
  if (algo >= OR_TREE && algo <= OR_HIER_LARGE)
    return topo_allreduce(&c, X, Y, n, algo, ranks_per_node, radix);
  /* the single-launch ring runs the ring's schedule: same steps, same order */
  if (algo == OR_RING || algo == OR_RING_FIFO) {
    int s1 = ring_reduce_scatter(&c, X, Y, n, 0);
    if (s1 < 0) return s1;
    return s1 + ring_all_gather_inplace(&c, Y, n);
  }
  /* the single-launch all-pairs runs the all-pairs' two steps: same order */
  if (algo == OR_ALLPAIRS || algo == OR_ONESHOT || algo == OR_ONESHOT_LL || algo == OR_ALLPAIRS_PERSISTENT)
    return allpairs(&c, X, Y, n);
  return OR_EBADARG;
}

/* The schedules that take no topology (ring, all-pairs, one-shot, LL);
 * the topology ones with one rank per node and radix 2. */
int oracle_allreduce(const void* const* X, void* const* Y, int p, int64_t n,
                     int dtype, int op, int algo) {
  return oracle_allreduce_topo(X, Y, p, n, dtype, op, algo, 1, 2);
}

/* The plain definition Y[r][i] = X[0][i] (+) X[1][i] (+) ... (+) X[p-1][i]
 * ([NCCL] "What all-reduce promises"), left fold in rank order.  For the
 * exact cases (int32 sum/prod/min/max/avg, fp min/max) every schedule must
 * reach exactly this. */
int oracle_definition(const void* const* X, void* const* Y, int p, int64_t n,
                      int dtype, int op) {
  if (check_args(p, n, dtype, op)) return OR_EBADARG;
  ctx_t c = make_ctx(p, dtype, op);
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    acc_t v = pre(&c, X[0], i);
    for (int q = 1; q < p; q++) v = combine(&c, v, pre(&c, X[q], i));
    for (int r = 0; r < p; r++) post_store(&c, v, Y[r], i);
  }
  return 1;
}

/* Reduce-scatter: rank r ends with the reduction of chunk r (n_out
 * elements, inputs hold p*n_out).  Ring = the reduce-scatter half of the
 * ring; direct (ALLPAIRS) = all-pairs step 1. */
int oracle_reduce_scatter(const void* const* X, void* const* Y, int p, int64_t n_out,
                          int dtype, int op, int algo) {
  if (check_args(p, n_out, dtype, op)) return OR_EBADARG;
  ctx_t c = make_ctx(p, dtype, op);
  const int64_t n = n_out * p;
  if (algo == OR_RING) return ring_reduce_scatter(&c, X, Y, n, 1);
  if (algo == OR_ALLPAIRS) {
    for (int j = 0; j < p; j++) allpairs_fold_chunk(&c, X, Y[j], n, j, chunk_lo(n, p, j));
    return 1;
  }
  return OR_EBADARG;
}

/* All-gather: Y[r][q*n_in + i] = X[q][i] for every r, q.  Ring: each rank
 * places its own block, then p-1 forwarding steps; direct (ALLPAIRS): every
 * block is fanned out to all ranks in one step. */
int oracle_all_gather(const void* const* X, void* const* Y, int p, int64_t n_in,
                      int dtype, int algo) {
  if (check_args(p, n_in, dtype, OR_SUM)) return OR_EBADARG;
  const int e = esize(dtype);
  const int64_t n = n_in * p;
  if (algo == OR_RING) {
    ctx_t c = make_ctx(p, dtype, OR_SUM);
    for (int r = 0; r < p; r++)
      memmove((char*)Y[r] + (int64_t)r * n_in * e, X[r], (size_t)(n_in * e));
    return ring_all_gather_inplace(&c, Y, n);
  }
  if (algo == OR_ALLPAIRS) {
    for (int q = 0; q < p; q++)
      for (int r = 0; r < p; r++)
        if ((const void*)((char*)Y[r] + (int64_t)q * n_in * e) != X[q])
          memcpy((char*)Y[r] + (int64_t)q * n_in * e, X[q], (size_t)(n_in * e));
    return 1;
  }
  return OR_EBADARG;
}

/* Sampled all-reduce: the value every rank ends with at element idx[k],
 * obtained by running the algorithm's schedule on that one element.
 * Ring: the chunk ch of element i is sent at reduce-scatter step s by rank
 * (ch+1+s) mod p to its successor, which folds its own element in; the
 * all-gather half only copies.  All-pairs/one-shot/LL: owner first, then the
 * other ranks ascending.  out is dtype-typed, m elements. */
int oracle_allreduce_at_topo(const void* const* X, int p, int64_t n, int dtype, int op,
                             int algo, int ranks_per_node, int radix,
                             const int64_t* idx, int64_t m, void* out) {
  if (check_args(p, n, dtype, op)) return OR_EBADARG;
  if (algo < OR_RING || algo > OR_ALLPAIRS_PERSISTENT) return OR_EBADARG;
  ctx_t c = make_ctx(p, dtype, op);
  for (int64_t k = 0; k < m; k++) if (idx[k] < 0 || idx[k] >= n) return OR_EBADARG;
  if (algo >= OR_TREE && algo <= OR_HIER_LARGE) {   /* rank 0's value: every rank ends with the same */
    topo_t T;
    if (topo_init(&T, algo, p, ranks_per_node, radix)) return OR_EBADARG;
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < m; k++) post_store(&c, topo_value(&c, &T, X, n, 0, idx[k]), out, k);
    return 0;
  }
  #pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < m; k++) {
    const int64_t i = idx[k];
    const int ch = (int)chunk_of(n, p, i);
    acc_t v;
    if (algo == OR_RING || algo == OR_RING_FIFO) {
      v = pre(&c, X[(ch + 1) % p], i);
      for (int s = 0; s <= p - 2; s++) {
        const int r = (ch + 1 + s) % p;     /* sender of chunk ch at step s */
        v = combine(&c, v, pre(&c, X[(r + 1) % p], i));
      }
    } else {
      v = pre(&c, X[ch], i);
      for (int q = 0; q < p; q++) if (q != ch) v = combine(&c, v, pre(&c, X[q], i));
    }
    post_store(&c, v, out, k);
  }
  return 0;
}

int oracle_allreduce_at(const void* const* X, int p, int64_t n, int dtype, int op,
                        int algo, const int64_t* idx, int64_t m, void* out) {
  return oracle_allreduce_at_topo(X, p, n, dtype, op, algo, 1, 2, idx, m, out);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the element loops of later calls (timing only; results do
 * not depend on it).  Returns the count now in effect. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

int64_t oracle_chunk_lo(int64_t n, int p, int c) { return chunk_lo(n, p, c); }
