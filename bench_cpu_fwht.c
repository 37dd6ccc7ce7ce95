/*
 * CPU throughput baseline for the fused rotate + int4 quantize step: a fast
 * Walsh-Hadamard transform (O(n log n) add/sub butterflies) of every row after
 * the sign diagonal, the 1/sqrt(n) normalisation, then per-group symmetric
 * absmax int4 quantization with fp16 scales and nibble packing.
 *
 * What is computed follows "Experiment -- Hadamard rotation for int4 (W4A4)
 * accuracy", Method (a fast Walsh-Hadamard transform followed by the 1/sqrt(K)
 * normalisation; per-group symmetric quantization), with the randomized
 * Hadamard transform's sign diagonal applied first and the rules of the
 * library's hr_rotate_quant_int4: s32 = absmax / 7 in fp32, the stored scale
 * is s32 rounded to fp16, codes are y / s rounded half away from zero and
 * clamped to [-7, 7], two codes per byte (even element in the low nibble).
 *
 * This is the fair CPU number for the path (the library's oracle multiplies
 * by an explicit Hadamard matrix instead).  Rows run in parallel with OpenMP.
 *
 * Usage: bench_cpu_fwht <x.bf16> <signs.i8> <rows> <n> <group> <reps> [out]
 *   x.bf16   rows * n bfloat16 values (raw, row-major)
 *   signs.i8 n int8 values, each +1 or -1
 *   reps     timed passes over all rows (the best is reported)
 *   out      optional file: codes (rows * n / 2 bytes) then fp16 scales
 * Prints one JSON object: best and mean seconds per pass, rows, threads.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> fp16 bit pattern, round to nearest even (finite, non-negative
 * inputs: scales). */
static uint16_t f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  x &= 0x7fffffffu;
  if (x >= 0x47800000u) return 0x7c00u;                 /* >= 65536: infinity */
  if (x < 0x38800000u) {                                /* below 2^-14: subnormal */
    return (uint16_t)nearbyintf(f * 16777216.0f);       /* units of 2^-24, ties to even */
  }
  const uint32_t m = x - 0x38000000u;                   /* exponent bias 127 -> 15 */
  return (uint16_t)((m + 0x0fffu + ((m >> 13) & 1u)) >> 13);
}

static float f16_to_f32(uint16_t h) {
  const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
  if (e == 0) return (float)m * (1.0f / 16777216.0f);
  uint32_t u = ((e + 112u) << 23) | (m << 13);
  if (e == 31) u = 0x7f800000u | (m << 13);
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* One row: y = H (d * x) / sqrt(n), then group quantization. */
static void row_rotate_quant(const uint16_t* xr, const float* d, int n, int group, float norm,
                             float* y, uint8_t* codes, uint16_t* scales) {
  for (int i = 0; i < n; ++i) y[i] = bf16_to_f32(xr[i]) * d[i];
  for (int h = 1; h < n; h <<= 1) {
    for (int i = 0; i < n; i += 2 * h) {
      float* a = y + i;
      float* b = y + i + h;
      for (int j = 0; j < h; ++j) {
        const float u = a[j], v = b[j];
        a[j] = u + v;
        b[j] = u - v;
      }
    }
  }
  for (int i = 0; i < n; ++i) y[i] *= norm;
  for (int g = 0; g < n / group; ++g) {
    const float* yg = y + g * group;
    float amax = 0.0f;
    for (int e = 0; e < group; ++e) amax = fmaxf(amax, fabsf(yg[e]));
    const float s32 = amax / 7.0f;
    const uint16_t s16 = f32_to_f16(s32);
    scales[g] = s16;
    const float s = f16_to_f32(s16);
    uint8_t* cg = codes + g * (group / 2);
    for (int e = 0; e < group; e += 2) {
      int q[2];
      for (int k = 0; k < 2; ++k) {
        int v = 0;
        if (s > 0.0f) {
          const float t = yg[e + k] / s;
          v = (int)floorf(fabsf(t) + 0.5f);
          if (v > 7) v = 7;
          if (t < 0.0f) v = -v;
        }
        q[k] = v;
      }
      cg[e / 2] = (uint8_t)((q[0] & 0xf) | ((q[1] & 0xf) << 4));
    }
  }
}

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

int main(int argc, char** argv) {
  if (argc < 7) {
    fprintf(stderr, "usage: %s x.bf16 signs.i8 rows n group reps [out]\n", argv[0]);
    return 2;
  }
  const long rows = atol(argv[3]);
  const int n = atoi(argv[4]), group = atoi(argv[5]), reps = atoi(argv[6]);
  if (rows <= 0 || n <= 0 || (n & (n - 1)) || group <= 0 || n % group || group % 2 || reps <= 0) {
    fprintf(stderr, "bad sizes\n");
    return 2;
  }
  uint16_t* x = (uint16_t*)read_file(argv[1], (size_t)rows * n * 2);
  int8_t* s8 = (int8_t*)read_file(argv[2], (size_t)n);
  if (!x || !s8) {
    fprintf(stderr, "cannot read inputs\n");
    return 1;
  }
  float* d = (float*)malloc(sizeof(float) * n);
  for (int i = 0; i < n; ++i) d[i] = s8[i] < 0 ? -1.0f : 1.0f;
  uint8_t* codes = (uint8_t*)malloc((size_t)rows * n / 2);
  uint16_t* scales = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)rows * (n / group));
  const float norm = (float)(1.0 / sqrt((double)n));
  int threads = 1;
  double best = 1e30, total = 0.0;
  for (int r = 0; r < reps; ++r) {
    const double t0 = omp_get_wtime();
#pragma omp parallel
    {
      float* y = (float*)malloc(sizeof(float) * n);
#pragma omp single
      threads = omp_get_num_threads();
#pragma omp for schedule(static)
      for (long i = 0; i < rows; ++i)
        row_rotate_quant(x + i * n, d, n, group, norm, y, codes + i * (n / 2),
                         scales + i * (n / group));
      free(y);
    }
    const double dt = omp_get_wtime() - t0;
    total += dt;
    if (dt < best) best = dt;
  }
  if (argc > 7) {
    FILE* f = fopen(argv[7], "wb");
    if (!f) return 1;
    fwrite(codes, 1, (size_t)rows * n / 2, f);
    fwrite(scales, sizeof(uint16_t), (size_t)rows * (n / group), f);
    fclose(f);
  }
  printf("{\"best_s\": %.6f, \"mean_s\": %.6f, \"rows\": %ld, \"threads\": %d}\n", best, total / reps, rows,
         threads);
  free(x);
  free(s8);
  free(d);
  free(codes);
  free(scales);
  return 0;
}
