/*
 * Seeded synthetic inputs for the attention forward: counter-based normals and
 * uniform words.  This file holds no attention arithmetic; it only fills host
 * buffers that both the GPU path and the CPU oracle then read.
 *
 * Generator: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), keyed by (seed, tensor_id).  Element i
 * of a tensor takes word i%4 of the block whose counter is (i/4 low 32 bits,
 * i/4 high 32 bits, 0, 0).  Normals come from the Box-Muller transform in
 * double precision over the word pairs (0,1) and (2,3) of a block; element
 * i%4 == 0 or 2 takes the cosine branch, 1 or 3 the sine branch.  The double
 * is rounded to float (round to nearest even) and, for bf16 output, the float
 * is rounded to bfloat16 (round to nearest even on the upper 16 bits).
 *
 * The seed of the pages' test protocol (1234) is a caller argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Raw Philox block, exported for known-answer tests. */
void attn_inputs_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  philox4x32_10(ctr, key, out);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);  /* quiet NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Exported for the bit-level rounding test. */
void attn_inputs_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

static const double TWO_PI = 6.283185307179586476925286766559;
static const double INV_2_32 = 1.0 / 4294967296.0;

/* The four normals of Philox block `blk` of stream (seed, tensor_id). */
static void normals_of_block(uint64_t blk, uint32_t seed, uint32_t tensor_id, double z[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
  uint32_t key[2] = {seed, tensor_id};
  uint32_t w[4];
  philox4x32_10(ctr, key, w);
  for (int pair = 0; pair < 2; ++pair) {
    double u1 = ((double)w[2 * pair] + 0.5) * INV_2_32;     /* in (0,1) */
    double u2 = ((double)w[2 * pair + 1] + 0.5) * INV_2_32; /* in (0,1) */
    double r = sqrt(-2.0 * log(u1));
    double t = TWO_PI * u2;
    z[2 * pair] = r * cos(t);
    z[2 * pair + 1] = r * sin(t);
  }
}

/* Calls emit(j, z) for every element j in [0, n) of the slice starting at
 * global index `offset`, visiting each Philox block once. */
#define FOR_EACH_NORMAL(n, offset, seed, tensor_id, threads, EMIT)                                   \
  do {                                                                                             \
    const uint64_t first = (uint64_t)(offset), last = (uint64_t)(offset) + (uint64_t)(n);          \
    const int64_t b0 = (int64_t)(first >> 2), b1 = (int64_t)((last + 3) >> 2);                     \
    _Pragma("omp parallel for schedule(static) num_threads(threads > 0 ? threads : omp_get_max_threads())") \
    for (int64_t blk = b0; blk < b1; ++blk) {                                                      \
      double z[4];                                                                                 \
      normals_of_block((uint64_t)blk, seed, tensor_id, z);                                         \
      for (int e = 0; e < 4; ++e) {                                                                \
        uint64_t i = ((uint64_t)blk << 2) + (uint64_t)e;                                           \
        if (i < first || i >= last) continue;                                                      \
        int64_t j = (int64_t)(i - first);                                                          \
        EMIT;                                                                                      \
      }                                                                                            \
    }                                                                                              \
  } while (0)

/* out[j] = bf16(float(normal(offset + j))) for j < n.  threads <= 0: runtime default. */
void attn_inputs_normal_bf16(uint16_t* out, int64_t n, int64_t offset, uint32_t seed, uint32_t tensor_id, int threads) {
  FOR_EACH_NORMAL(n, offset, seed, tensor_id, threads, out[j] = f32_to_bf16_rne((float)z[e]));
}

void attn_inputs_normal_f32(float* out, int64_t n, int64_t offset, uint32_t seed, uint32_t tensor_id, int threads) {
  FOR_EACH_NORMAL(n, offset, seed, tensor_id, threads, out[j] = (float)z[e]);
}

/* Uniform 32-bit words: out[j] = word (offset+j)%4 of block (offset+j)/4. */
void attn_inputs_u32(uint32_t* out, int64_t n, int64_t offset, uint32_t seed, uint32_t tensor_id) {
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = (uint64_t)(offset + j), blk = i >> 2;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
    uint32_t key[2] = {seed, tensor_id};
    uint32_t w[4];
    philox4x32_10(ctr, key, w);
    out[j] = w[i & 3];
  }
}
