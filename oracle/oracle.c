/*
 * Plain CPU oracle for the Atom datapath: reduce, layout copy, variable-length copy.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The library under
 * reduce_atom_amd/ never does, and shares no code with it.
 *
 * Everything here is written for obviousness, not speed: one output at a time,
 * in the order the definitions state, with no blocking, vectorisation or fusion.
 *
 * Sources followed (Purlin: Separating Orchestration from the Datapath of
 * Collectives, Aimuyo, Gandhi, Kozyrakis):
 *  - reduce: the paper's section 3.3 ("The Atom", SCORE): each output element is
 *    owned by one thread that accumulates the sources in a fixed source order.
 *    The accumulation type (binary32) and the single final rounding to the element
 *    type follow the project's stated contract for the method (fp32 accumulation
 *    in rank order 0..W-1, one rounding at the end).
 *  - copy: section 3.1 ("Layouts"): a collective names an input and an output
 *    layout and copies between them; the offsets themselves come from the
 *    layout derivation in oracle/__init__.py.
 *  - copy_v: appendix C.4 ("Variable-Length Collectives") and section 4
 *    (partition sizes at run time, prefix sums): rows are packed per destination,
 *    in source-rank then row order, with counts and offsets emitted.
 *
 * Floating point: binary32 additions are the host's IEEE-754 additions (x86-64
 * SSE, round-to-nearest-even). The flush-to-zero and denormals-are-zero bits of
 * MXCSR are cleared for the duration of every call, whatever the calling process
 * set. Build with -O2 -ffp-contract=off -fno-fast-math.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in binary32 (FLT_EVAL_METHOD == 0)"
#endif

enum { OR_BF16 = 0, OR_F16 = 1, OR_F32 = 2 };

/* ---------------------------------------------------------------- MXCSR guard */
static unsigned int ieee_enter(void) {
  unsigned int old = _mm_getcsr();
  /* bit 15 = flush-to-zero, bit 6 = denormals-are-zero; rounding bits 13-14 = 0 (nearest) */
  _mm_setcsr(old & ~(0x8000u | 0x0040u | 0x6000u));
  return old;
}
static void ieee_leave(unsigned int old) { _mm_setcsr(old); }

/* ------------------------------------------------ 16-bit formats, by definition */
/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double bf16_value(uint16_t p) {
  int s = p >> 15, e = (p >> 7) & 0xFF, f = p & 0x7F;
  double v;
  if (e == 0xFF) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -126 - 7);          /* subnormal */
  else v = ldexp((double)(128 + f), e - 127 - 7);           /* normal */
  return s ? -v : v;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_value(uint16_t p) {
  int s = p >> 15, e = (p >> 10) & 0x1F, f = p & 0x3FF;
  double v;
  if (e == 0x1F) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -14 - 10);
  else v = ldexp((double)(1024 + f), e - 15 - 10);
  return s ? -v : v;
}

typedef struct {
  double (*value)(uint16_t);
  uint16_t pos_inf;      /* bit pattern of +inf; patterns 0..pos_inf-1 are +finite, increasing */
  double past_max;       /* the next value after the largest finite one, exponent unbounded */
  uint16_t quiet_nan;
} fmt16;

static const fmt16 FMT_BF16 = {bf16_value, 0x7F80, 0x1p128, 0x7FC0};
static const fmt16 FMT_F16 = {f16_value, 0x7C00, 0x1p16, 0x7E00};

/* Round x to the nearest value of the format; ties go to the even bit pattern.
 * Finite values are compared exactly in double: every value involved is a
 * binary32 value or a 16-bit-format value, so the differences are exact. */
static uint16_t round_to_fmt(const fmt16* F, float x) {
  if (isnan(x)) return (uint16_t)((signbit(x) ? 0x8000 : 0) | F->quiet_nan);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isinf(x)) return sign | F->pos_inf;
  double a = fabs((double)x);
  /* largest positive pattern p with value(p) <= a; value(0) = 0 <= a */
  uint32_t lo = 0, hi = (uint32_t)F->pos_inf - 1;
  if (F->value((uint16_t)hi) <= a) {
    lo = hi;
  } else {
    while (hi - lo > 1) { /* invariant: value(lo) <= a < value(hi) */
      uint32_t mid = lo + (hi - lo) / 2;
      if (F->value((uint16_t)mid) <= a) lo = mid; else hi = mid;
    }
  }
  uint32_t p = lo;
  double v_lo = F->value((uint16_t)p);
  if (v_lo == a) return sign | (uint16_t)p;
  double v_hi = (p + 1 == F->pos_inf) ? F->past_max : F->value((uint16_t)(p + 1));
  double d_lo = a - v_lo, d_hi = v_hi - a;
  uint32_t r;
  if (d_lo < d_hi) r = p;
  else if (d_hi < d_lo) r = p + 1;
  else r = (p & 1) ? p + 1 : p; /* tie: even pattern */
  return sign | (uint16_t)r;    /* p + 1 == pos_inf encodes overflow to infinity */
}

static float widen(int dtype, const void* base, int64_t i) {
  if (dtype == OR_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * i, 4);
    return f;
  }
  uint16_t p;
  memcpy(&p, (const char*)base + 2 * i, 2);
  double v = (dtype == OR_BF16) ? bf16_value(p) : f16_value(p);
  return (float)v; /* exact: every bf16/f16 value is a binary32 value */
}

static void narrow_store(int dtype, void* base, int64_t i, float a) {
  if (dtype == OR_F32) {
    memcpy((char*)base + 4 * i, &a, 4);
    return;
  }
  uint16_t p = round_to_fmt(dtype == OR_BF16 ? &FMT_BF16 : &FMT_F16, a);
  memcpy((char*)base + 2 * i, &p, 2);
}

/* ------------------------------------------------------------ exported: formats */
void oracle_widen(int dtype, const void* src, float* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = widen(dtype, src, i);
}

void oracle_narrow(int dtype, const float* src, void* dst, int64_t n) {
  unsigned int m = ieee_enter();
  for (int64_t i = 0; i < n; ++i) narrow_store(dtype, dst, i, src[i]);
  ieee_leave(m);
}

/* One binary32 addition, exported so tests can check the MXCSR guard. */
float oracle_add_f32(float a, float b) {
  unsigned int m = ieee_enter();
  float r = a + b;
  ieee_leave(m);
  return r;
}

/* --------------------------------------------------------------- exported: reduce
 * out[i] = round(((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{W-1}[i]) for i in [0, n):
 * the accumulator starts at source 0 and takes the others in source order, each
 * addition rounded to binary32; one rounding to the element type at the end.
 * srcs[w] points at source w's buffer; src_off[w] is the element offset of the
 * share inside it (0 for a packed contribution, rank * n for a scattered one).
 */
/* elements [i0, i1) of the definition above */
static void reduce_range(int dtype, int W, const void* const* srcs, const int64_t* src_off,
                         void* dst, int64_t i0, int64_t i1) {
  unsigned int m = ieee_enter();
  for (int64_t i = i0; i < i1; ++i) {
    float a = widen(dtype, srcs[0], src_off[0] + i);
    for (int w = 1; w < W; ++w) a = a + widen(dtype, srcs[w], src_off[w] + i);
    narrow_store(dtype, dst, i, a);
  }
  ieee_leave(m);
}

int oracle_reduce(int dtype, int W, const void* const* srcs, const int64_t* src_off,
                  void* dst, int64_t n) {
  if (W < 1 || dtype < 0 || dtype > 2 || n < 0) return -1;
  reduce_range(dtype, W, srcs, src_off, dst, 0, n);
  return 0;
}

/* ----------------------------------------------------------------- exported: copy
 * For every segment k: bytes [src_off[k], src_off[k] + len[k]) of source src[k]
 * go to bytes [dst_off[k], dst_off[k] + len[k]) of the output. */
int oracle_copy(int nseg, const void* const* srcs, const int32_t* seg_src,
                const int64_t* src_off, const int64_t* dst_off, const int64_t* len, void* dst) {
  for (int k = 0; k < nseg; ++k)
    memcpy((char*)dst + dst_off[k], (const char*)srcs[seg_src[k]] + src_off[k], (size_t)len[k]);
  return 0;
}

/* --------------------------------------------------------------- exported: copy_v
 * W sources; source s has rows[s] rows of row_bytes bytes and dest[s][i] in [0, W)
 * names the destination of its row i.
 *   counts[s*W + d]  = number of rows of source s bound for d
 *   offsets[d*W + s] = first output row of the block (d, s): all rows bound for a
 *                      smaller destination, then the rows bound for d from smaller
 *                      sources
 * Row i of source s lands at offsets[d*W + s] + (number of rows i' < i of source s
 * bound for the same d). Returns the total row count, or -1 on a bad destination. */

/* counts and offsets as defined above; returns the total row count or -1 */
static int64_t copy_v_counts_offsets(int W, const int64_t* rows, const int32_t* const* dest,
                                     int64_t* counts, int64_t* offsets) {
  for (int s = 0; s < W; ++s)
    for (int d = 0; d < W; ++d) counts[s * W + d] = 0;
  for (int s = 0; s < W; ++s)
    for (int64_t i = 0; i < rows[s]; ++i) {
      int32_t d = dest[s][i];
      if (d < 0 || d >= W) return -1;
      counts[s * W + d] += 1;
    }
  int64_t base = 0;
  for (int d = 0; d < W; ++d) {
    int64_t off = base;
    for (int s = 0; s < W; ++s) {
      offsets[d * W + s] = off;
      off += counts[s * W + d];
    }
    base = off;
  }
  return base;
}

/* Rows [i0, i1) of source s, in row order. A row's rank among the rows of its source
 * bound for the same destination is the number of earlier such rows, counted from
 * row 0 of the source. */
static void place_rows(int W, int s, const void* const* srcs, const int32_t* const* dest,
                       int64_t row_bytes, void* dst, const int64_t* offsets, int64_t i0, int64_t i1) {
  int64_t seen[64];
  for (int d = 0; d < W; ++d) seen[d] = 0;
  for (int64_t i = 0; i < i0; ++i) seen[dest[s][i]] += 1;
  for (int64_t i = i0; i < i1; ++i) {
    int32_t d = dest[s][i];
    int64_t out_row = offsets[d * W + s] + seen[d];
    seen[d] += 1;
    memcpy((char*)dst + out_row * row_bytes, (const char*)srcs[s] + i * row_bytes, (size_t)row_bytes);
  }
}

int64_t oracle_copy_v(int W, const void* const* srcs, const int64_t* rows,
                      const int32_t* const* dest, int64_t row_bytes, void* dst,
                      int64_t* counts, int64_t* offsets) {
  if (W < 1 || W > 64) return -1;
  int64_t total = copy_v_counts_offsets(W, rows, dest, counts, offsets);
  if (total < 0) return -1;
  for (int s = 0; s < W; ++s) place_rows(W, s, srcs, dest, row_bytes, dst, offsets, 0, rows[s]);
  return total;
}

/* ------------------------------------------------------- threaded variants
 * The same definitions with the work split over POSIX threads, only so that the
 * oracle can be timed on every host core. No element's arithmetic changes: each
 * output element, byte or row is produced by exactly one thread running the code of
 * the single-threaded function (reduce: reduce_range over a contiguous range of i;
 * copy: memcpy of a contiguous part of every segment; copy_v: counts and offsets on
 * the calling thread as oracle_copy_v computes them, then place_rows over contiguous
 * row ranges of one source). The results are those of the single-threaded calls bit
 * for bit; the tests check that. MXCSR is per thread, and reduce_range sets it in
 * the thread that runs it. */
#include <pthread.h>
#include <stdlib.h>
#include <unistd.h>

/* Logical CPUs online on this host (what std::thread::hardware_concurrency reports). */
int oracle_hardware_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* part k of [0, n) cut into `parts` contiguous ranges of nearly equal length */
static int64_t part_start(int64_t n, int parts, int k) { return (int64_t)((__int128)n * k / parts); }

/* Runs f on nparts argument blocks of `size` bytes, at most nthreads at a time (the
 * calling thread runs one of each group; a part whose thread cannot start runs here). */
static void run_parts(void* (*f)(void*), char* parts, size_t size, int nparts, int nthreads) {
  pthread_t th[256];
  if (nthreads > 256) nthreads = 256;
  for (int k0 = 0; k0 < nparts; k0 += nthreads) {
    int n = nparts - k0 < nthreads ? nparts - k0 : nthreads;
    int made[256];
    for (int k = 1; k < n; ++k) {
      made[k] = pthread_create(&th[k], NULL, f, parts + (size_t)(k0 + k) * size) == 0;
      if (!made[k]) f(parts + (size_t)(k0 + k) * size);
    }
    f(parts + (size_t)k0 * size);
    for (int k = 1; k < n; ++k)
      if (made[k]) pthread_join(th[k], NULL);
  }
}

typedef struct {
  int dtype, W;
  const void* const* srcs;
  const int64_t* src_off;
  void* dst;
  int64_t i0, i1;
} reduce_part;

static void* reduce_part_run(void* p) {
  const reduce_part* r = (const reduce_part*)p;
  reduce_range(r->dtype, r->W, r->srcs, r->src_off, r->dst, r->i0, r->i1);
  return NULL;
}

int oracle_reduce_mt(int dtype, int W, const void* const* srcs, const int64_t* src_off,
                     void* dst, int64_t n, int nthreads) {
  if (W < 1 || dtype < 0 || dtype > 2 || n < 0 || nthreads < 1) return -1;
  reduce_part* parts = (reduce_part*)calloc((size_t)nthreads, sizeof(reduce_part));
  if (!parts) return -1;
  for (int k = 0; k < nthreads; ++k) {
    reduce_part r = {dtype, W, srcs, src_off, dst, part_start(n, nthreads, k), part_start(n, nthreads, k + 1)};
    parts[k] = r;
  }
  run_parts(reduce_part_run, (char*)parts, sizeof(reduce_part), nthreads, nthreads);
  free(parts);
  return 0;
}

typedef struct {
  int nseg;
  const void* const* srcs;
  const int32_t* seg_src;
  const int64_t *src_off, *dst_off, *len;
  void* dst;
  int k, parts;
} copy_part;

static void* copy_part_run(void* p) {
  const copy_part* c = (const copy_part*)p;
  for (int s = 0; s < c->nseg; ++s) {
    int64_t a = part_start(c->len[s], c->parts, c->k), b = part_start(c->len[s], c->parts, c->k + 1);
    memcpy((char*)c->dst + c->dst_off[s] + a, (const char*)c->srcs[c->seg_src[s]] + c->src_off[s] + a,
           (size_t)(b - a));
  }
  return NULL;
}

int oracle_copy_mt(int nseg, const void* const* srcs, const int32_t* seg_src,
                   const int64_t* src_off, const int64_t* dst_off, const int64_t* len, void* dst,
                   int nthreads) {
  if (nthreads < 1) return -1;
  copy_part* parts = (copy_part*)calloc((size_t)nthreads, sizeof(copy_part));
  if (!parts) return -1;
  for (int k = 0; k < nthreads; ++k) {
    copy_part c = {nseg, srcs, seg_src, src_off, dst_off, len, dst, k, nthreads};
    parts[k] = c;
  }
  run_parts(copy_part_run, (char*)parts, sizeof(copy_part), nthreads, nthreads);
  free(parts);
  return 0;
}

typedef struct {
  int W, s;
  const void* const* srcs;
  const int32_t* const* dest;
  int64_t row_bytes;
  void* dst;
  const int64_t* offsets;
  int64_t i0, i1;
} copy_v_part;

static void* copy_v_part_run(void* p) {
  const copy_v_part* c = (const copy_v_part*)p;
  place_rows(c->W, c->s, c->srcs, c->dest, c->row_bytes, c->dst, c->offsets, c->i0, c->i1);
  return NULL;
}

int64_t oracle_copy_v_mt(int W, const void* const* srcs, const int64_t* rows,
                         const int32_t* const* dest, int64_t row_bytes, void* dst,
                         int64_t* counts, int64_t* offsets, int nthreads) {
  if (W < 1 || W > 64 || nthreads < 1) return -1;
  int64_t total = copy_v_counts_offsets(W, rows, dest, counts, offsets);
  if (total < 0) return -1;
  const int nparts = W * nthreads; /* nthreads row ranges of every source */
  copy_v_part* parts = (copy_v_part*)calloc((size_t)nparts, sizeof(copy_v_part));
  if (!parts) return -1;
  for (int s = 0; s < W; ++s)
    for (int k = 0; k < nthreads; ++k) {
      copy_v_part c = {W, s, srcs, dest, row_bytes, dst, offsets,
                       part_start(rows[s], nthreads, k), part_start(rows[s], nthreads, k + 1)};
      parts[s * nthreads + k] = c;
    }
  run_parts(copy_v_part_run, (char*)parts, sizeof(copy_v_part), nparts, nthreads);
  free(parts);
  return total;
}
