/*
 * gen.c — seeded synthetic inputs for QSA layer-step workloads.
 *
 * This file holds no arithmetic of the method: it only draws numbers and
 * stores them in the layouts the C ABI takes (paged caches, page tables,
 * query tensors).  Both the CPU oracle and the GPU library consume its
 * output bytes; neither links it.
 *
 * Random numbers: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) used as a
 * counter-based generator: draw i of a stream with key k is
 * mix64(k + (i + 1) * 0x9E3779B97F4A7C15), which is the (i+1)-th output of
 * SplitMix64 seeded with k.  Every element is therefore a pure function of
 * (seed, tensor id, logical index) and generation is order-independent and
 * parallel.  Normal deviates use the Box–Muller transform (Box & Muller,
 * 1958) on a pair of draws; uniforms take the top 24 or 53 bits.
 *
 * Element formats written here:
 *   bf16  round-to-nearest-even of the fp32 value (top 16 bits).
 *   fp8   OCP E4M3FN of value/scale, round-to-nearest-even, saturating to
 *         +-448 (the format has no infinity; code 0x7F is NaN).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of the stream for tensor `tensor_id` under `seed`. */
uint64_t wl_stream_key(uint64_t seed, uint64_t tensor_id) {
  return mix64(mix64(seed) ^ (tensor_id * GOLDEN + 0x51A0ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN);
}

/* Uniform in [0,1) with 24 random bits (exact in fp32). */
static inline float unif24(uint64_t key, uint64_t i) {
  return (float)(draw(key, i) >> 40) * (1.0f / 16777216.0f);
}

/* Normal deviate number n of the stream: Box–Muller on draws 2*(n/2) and
 * 2*(n/2)+1; even n takes the cosine branch, odd n the sine branch. */
static inline double normal(uint64_t key, uint64_t n) {
  uint64_t p = n >> 1;
  double u1 = ((double)(draw(key, 2 * p) >> 11) + 1.0) * 0x1.0p-53; /* (0,1] */
  double u2 = (double)(draw(key, 2 * p + 1) >> 11) * 0x1.0p-53;     /* [0,1) */
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (n & 1) ? r * sin(t) : r * cos(t);
}

/* Both deviates of Box–Muller pair p (normal numbers 2p and 2p+1). */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  double u1 = ((double)(draw(key, 2 * p) >> 11) + 1.0) * 0x1.0p-53;
  double u2 = (double)(draw(key, 2 * p + 1) >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

uint16_t wl_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0; /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP E4M3FN encoding of x (already divided by the scale). */
uint8_t wl_fp8_e4m3_rne(double x) {
  uint8_t s = 0;
  if (x != x) return 0x7F;
  if (x < 0 || (x == 0 && signbit(x))) { s = 0x80; x = -x; }
  if (x >= 448.0) return s | 0x7E;
  if (x < 0x1.0p-6) { /* subnormal range: multiples of 2^-9 */
    double m = rint(x * 512.0); /* round half to even */
    if (m >= 8.0) return s | 0x08; /* rounds up to the smallest normal */
    return s | (uint8_t)m;
  }
  int e2;
  double f = frexp(x, &e2);      /* x = f * 2^e2, f in [0.5,1) */
  int e = e2 - 1;                /* x = (2f) * 2^e, 2f in [1,2) */
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m >= 8.0) { m = 0.0; e += 1; }
  if (e > 8) return s | 0x7E;
  int be = e + 7;                /* biased exponent 1..15 */
  if (be == 15 && m == 7.0) return s | 0x7E; /* would be NaN: saturate */
  return s | (uint8_t)((be << 3) | (int)m);
}

/* --- dense tensors ------------------------------------------------------ */

void wl_fill_normal_f32(uint64_t key, int64_t n, float* out, int bf16_exact) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float v = (float)normal(key, (uint64_t)i);
    if (bf16_exact) {
      uint32_t u = (uint32_t)wl_bf16_rne(v) << 16;
      memcpy(&v, &u, 4);
    }
    out[i] = v;
  }
}

void wl_fill_normal_bf16(uint64_t key, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = wl_bf16_rne((float)normal(key, (uint64_t)i));
}

void wl_fill_uniform_f32(uint64_t key, int64_t n, float lo, float hi, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = lo + (hi - lo) * unif24(key, (uint64_t)i);
}

/* Integers uniform in [lo, hi] (inclusive). */
void wl_fill_uniform_int(uint64_t key, int64_t n, int32_t lo, int32_t hi, int32_t* out) {
  uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  for (int64_t i = 0; i < n; ++i) {
    double u = (double)(draw(key, (uint64_t)i) >> 11) * 0x1.0p-53;
    uint64_t k = (uint64_t)(u * (double)span);
    if (k >= span) k = span - 1;
    out[i] = (int32_t)((int64_t)lo + (int64_t)k);
  }
}

/* Fisher–Yates permutation of 0..n-1 (Durstenfeld's in-place form). */
void wl_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    double u = (double)(draw(key, (uint64_t)i) >> 11) * 0x1.0p-53;
    int32_t j = (int32_t)(u * (double)(i + 1));
    if (j > i) j = i;
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* --- paged caches ------------------------------------------------------- */
/* Logical element (request b, token t, kv head h, dim d) is normal number
 * ((b * 2^20 + t) * Hkv + h) * D + d of the stream.  Slots beyond a
 * request's stored length are filled with NaN codes so that any read of
 * them shows up in the results. */

static inline uint64_t kv_index(int b, int t, int h, int d, int Hkv, int D) {
  return ((((uint64_t)b << 20) + (uint64_t)t) * (uint64_t)Hkv + (uint64_t)h) * (uint64_t)D +
         (uint64_t)d;
}

/* Largest |value| over the stored tokens of every request (D even). */
double wl_kv_amax(uint64_t key, int B, const int32_t* lens, int Hkv, int D) {
  double amax = 0.0;
  for (int b = 0; b < B; ++b) {
    int64_t rows = (int64_t)lens[b] * Hkv;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      int t = (int)(r / Hkv), h = (int)(r % Hkv);
      uint64_t n0 = kv_index(b, t, h, 0, Hkv, D);
      for (int d = 0; d < D; d += 2) {
        double z0, z1;
        normal_pair(key, (n0 + (uint64_t)d) >> 1, &z0, &z1);
        double a0 = fabs((double)(float)z0), a1 = fabs((double)(float)z1);
        if (a0 > amax) amax = a0;
        if (a1 > amax) amax = a1;
      }
    }
  }
  return amax;
}

/* Fill a paged K or V cache [num_pages, page, Hkv, D] (D even).
 * dtype 0: bf16 of the normal value; dtype 1: fp8 e4m3 of value / scale.
 * Pages not referenced by any request are left untouched (caller zeroes). */
void wl_fill_kv_cache(uint64_t key, int B, const int32_t* lens, const int32_t* page_table,
                      int max_pages, int page, int Hkv, int D, int dtype, double scale,
                      void* out) {
  for (int b = 0; b < B; ++b) {
    int npages = (lens[b] + page - 1) / page;
#pragma omp parallel for schedule(static)
    for (int p = 0; p < npages; ++p) {
      int64_t phys = page_table[(int64_t)b * max_pages + p];
      for (int s = 0; s < page; ++s) {
        int t = p * page + s;
        for (int h = 0; h < Hkv; ++h) {
          int64_t base = ((phys * page + s) * Hkv + h) * (int64_t)D;
          uint64_t n0 = kv_index(b, t, h, 0, Hkv, D);
          for (int d = 0; d < D; d += 2) {
            double z0 = NAN, z1 = NAN;
            if (t < lens[b]) normal_pair(key, (n0 + (uint64_t)d) >> 1, &z0, &z1);
            if (dtype == 0) {
              uint16_t* o = (uint16_t*)out;
              o[base + d] = (t < lens[b]) ? wl_bf16_rne((float)z0) : (uint16_t)0x7FC0;
              o[base + d + 1] = (t < lens[b]) ? wl_bf16_rne((float)z1) : (uint16_t)0x7FC0;
            } else {
              uint8_t* o = (uint8_t*)out;
              o[base + d] = (t < lens[b]) ? wl_fp8_e4m3_rne((double)(float)z0 / scale) : (uint8_t)0x7F;
              o[base + d + 1] = (t < lens[b]) ? wl_fp8_e4m3_rne((double)(float)z1 / scale) : (uint8_t)0x7F;
            }
          }
        }
      }
    }
  }
}

/* Fill the paged compressed-key cache [num_pages, page/ratio, Hi, Di] f32.
 * Logical (b, g, h, d) is normal number ((b * 2^18 + g) * Hi + h) * Di + d.
 * Groups g < n_groups[b] get values; the remaining slots of the request's
 * pages get NaN.  bf16_exact rounds the values to bf16 first. */
void wl_fill_khat_cache(uint64_t key, int B, const int32_t* n_groups, const int32_t* page_table,
                        int max_pages, int gpp, int Hi, int Di, int bf16_exact, float* out) {
  for (int b = 0; b < B; ++b) {
    int npages = (n_groups[b] + gpp - 1) / gpp;
    if (npages == 0) continue;
#pragma omp parallel for schedule(static)
    for (int p = 0; p < npages; ++p) {
      int64_t phys = page_table[(int64_t)b * max_pages + p];
      for (int s = 0; s < gpp; ++s) {
        int g = p * gpp + s;
        for (int h = 0; h < Hi; ++h) {
          int64_t base = ((phys * gpp + s) * Hi + h) * (int64_t)Di;
          for (int d = 0; d < Di; ++d) {
            float v;
            if (g < n_groups[b]) {
              uint64_t n = ((((uint64_t)b << 18) + (uint64_t)g) * (uint64_t)Hi + (uint64_t)h) * (uint64_t)Di + (uint64_t)d;
              v = (float)normal(key, n);
              if (bf16_exact) {
                uint32_t u = (uint32_t)wl_bf16_rne(v) << 16;
                memcpy(&v, &u, 4);
              }
            } else {
              v = NAN;
            }
            out[base + d] = v;
          }
        }
      }
    }
  }
}

int wl_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
