/* Host fuzz driver for the oracle (oracle/oracle.c), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_host_sanitize.py: seeded random inputs to
 * every exported function, with the buffers sized exactly, plus a few identities that
 * hold for any input (a 16-bit value survives widening and narrowing back, a reduce of
 * one source is that source, copy_v's counts add up to the rows and its output rows
 * are a permutation of the input rows). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_widen(int dtype, const void* src, float* dst, int64_t n);
void oracle_narrow(int dtype, const float* src, void* dst, int64_t n);
float oracle_add_f32(float a, float b);
int oracle_reduce(int dtype, int W, const void* const* srcs, const int64_t* src_off, void* dst, int64_t n);
int oracle_copy(int nseg, const void* const* srcs, const int32_t* seg_src, const int64_t* src_off,
                const int64_t* dst_off, const int64_t* len, void* dst);
int64_t oracle_copy_v(int W, const void* const* srcs, const int64_t* rows, const int32_t* const* dest,
                      int64_t row_bytes, void* dst, int64_t* counts, int64_t* offsets);

static uint64_t g_state;
static uint64_t next_u64(void) { /* SplitMix64 (Steele, Lea and Flood, 2014) */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static uint64_t below(uint64_t n) { return n ? next_u64() % n : 0; }
static void fill(void* p, size_t bytes) {
  for (size_t i = 0; i < bytes; ++i) ((uint8_t*)p)[i] = (uint8_t)next_u64();
}
#define CHECK(c, what)                                                  \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "iteration %d: check failed: %s (%s)\n", it, #c, what); \
      abort();                                                          \
    }                                                                   \
  } while (0)

static int is_nan16(int dtype, uint16_t p) {
  return dtype == 0 ? ((p & 0x7F80) == 0x7F80 && (p & 0x7F)) : ((p & 0x7C00) == 0x7C00 && (p & 0x3FF));
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 2000;
  g_state = argc > 2 ? strtoull(argv[2], NULL, 10) : 1;
  for (int it = 0; it < iters; ++it) {
    /* formats: widen then narrow gives back every non-NaN 16-bit pattern */
    {
      const int dtype = (int)below(2);
      const int64_t n = (int64_t)below(300);
      uint16_t* x = malloc(2 * (size_t)n + 2);
      float* f = malloc(4 * (size_t)n + 4);
      uint16_t* y = malloc(2 * (size_t)n + 2);
      fill(x, 2 * (size_t)n);
      oracle_widen(dtype, x, f, n);
      oracle_narrow(dtype, f, y, n);
      for (int64_t i = 0; i < n; ++i) CHECK(is_nan16(dtype, x[i]) || x[i] == y[i], "16-bit round trip");
      float* g = malloc(4 * (size_t)n + 4);
      fill(g, 4 * (size_t)n);
      oracle_widen(2, g, f, n);
      oracle_narrow(2, f, y, 0);
      free(x), free(f), free(y), free(g);
      (void)oracle_add_f32((float)below(100), -1.5f);
    }
    /* reduce: W sources with their own offsets; one source reduces to itself */
    {
      const int dtype = (int)below(3), W = 1 + (int)below(16), es = dtype == 2 ? 4 : 2;
      const int64_t n = (int64_t)below(400);
      void* srcs[16];
      int64_t off[16];
      for (int w = 0; w < W; ++w) {
        off[w] = (int64_t)below(64);
        srcs[w] = malloc((size_t)(off[w] + n) * es + 1);
        fill(srcs[w], (size_t)(off[w] + n) * es);
      }
      void* dst = malloc((size_t)n * es + 1);
      CHECK(oracle_reduce(dtype, W, (const void* const*)srcs, off, dst, n) == 0, "reduce");
      CHECK(oracle_reduce(dtype, 0, (const void* const*)srcs, off, dst, n) == -1, "W = 0 refused");
      if (W >= 1) {
        CHECK(oracle_reduce(dtype, 1, (const void* const*)srcs, off, dst, n) == 0, "reduce of one");
        if (dtype == 2) {
          for (int64_t i = 0; i < n; ++i) {
            float a, b;
            memcpy(&a, (char*)srcs[0] + (off[0] + i) * 4, 4);
            memcpy(&b, (char*)dst + i * 4, 4);
            CHECK(a != a || memcmp(&a, &b, 4) == 0, "one f32 source is its own reduction");
          }
        } else {
          for (int64_t i = 0; i < n; ++i) {
            uint16_t a, b;
            memcpy(&a, (char*)srcs[0] + (off[0] + i) * 2, 2);
            memcpy(&b, (char*)dst + i * 2, 2);
            CHECK(is_nan16(dtype, a) || a == b, "one 16-bit source is its own reduction");
          }
        }
      }
      for (int w = 0; w < W; ++w) free(srcs[w]);
      free(dst);
    }
    /* copy: an AllGather-shaped table with random segment lengths, packed output */
    {
      const int W = 1 + (int)below(8);
      void* srcs[8];
      int32_t seg_src[8];
      int64_t so[8], dof[8], len[8], total = 0;
      for (int s = 0; s < W; ++s) {
        len[s] = (int64_t)below(500);
        so[s] = (int64_t)below(32);
        srcs[s] = malloc((size_t)(so[s] + len[s]) + 1);
        fill(srcs[s], (size_t)(so[s] + len[s]));
        seg_src[s] = s;
        dof[s] = total;
        total += len[s];
      }
      uint8_t* dst = malloc((size_t)total + 1);
      CHECK(oracle_copy(W, (const void* const*)srcs, seg_src, so, dof, len, dst) == 0, "copy");
      for (int s = 0; s < W; ++s)
        CHECK(memcmp(dst + dof[s], (uint8_t*)srcs[s] + so[s], (size_t)len[s]) == 0, "segment landed");
      for (int s = 0; s < W; ++s) free(srcs[s]);
      free(dst);
    }
    /* copy_v: random destinations; counts add up; rows are moved, not invented */
    {
      const int W = 1 + (int)below(8);
      const int64_t row_bytes = 16 * (1 + (int64_t)below(4));
      void* srcs[8];
      int32_t* dest[8];
      int64_t rows[8], total = 0;
      for (int s = 0; s < W; ++s) {
        rows[s] = (int64_t)below(60);
        srcs[s] = malloc((size_t)(rows[s] * row_bytes) + 1);
        dest[s] = malloc(4 * (size_t)rows[s] + 4);
        for (int64_t i = 0; i < rows[s]; ++i) {
          memset((char*)srcs[s] + i * row_bytes, 0, (size_t)row_bytes);
          memcpy((char*)srcs[s] + i * row_bytes, &(int64_t){s * 1000000 + i}, 8);
          dest[s][i] = (int32_t)below((uint64_t)W);
        }
        total += rows[s];
      }
      uint8_t* dst = malloc((size_t)(total * row_bytes) + 1);
      int64_t counts[64], offsets[64];
      CHECK(oracle_copy_v(W, (const void* const*)srcs, rows, (const int32_t* const*)dest, row_bytes, dst, counts,
                          offsets) == total, "copy_v row count");
      int64_t sum = 0;
      for (int k = 0; k < W * W; ++k) sum += counts[k];
      CHECK(sum == total, "counts add up");
      uint8_t* seen = calloc((size_t)(8 * 60), 1);
      for (int64_t r = 0; r < total; ++r) {
        int64_t tag;
        memcpy(&tag, dst + r * row_bytes, 8);
        const int64_t s = tag / 1000000, i = tag % 1000000;
        CHECK(s >= 0 && s < W && i >= 0 && i < rows[s] && !seen[s * 60 + i], "output rows are the input rows");
        seen[s * 60 + i] = 1;
      }
      if (W > 1 && rows[0] > 0) { /* a destination out of range is refused */
        dest[0][0] = W;
        CHECK(oracle_copy_v(W, (const void* const*)srcs, rows, (const int32_t* const*)dest, row_bytes, dst,
                            counts, offsets) == -1, "bad destination refused");
      }
      free(seen);
      for (int s = 0; s < W; ++s) free(srcs[s]), free(dest[s]);
      free(dst);
    }
  }
  printf("oracle fuzz: %d iterations\n", iters);
  return 0;
}
