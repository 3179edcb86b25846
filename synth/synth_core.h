/*
 * synth_core.h - counter-based draws for the seeded synthetic inputs.
 *
 * This header is the whole random part of the input generator. It holds no
 * arithmetic of the MoE layer: it only turns (seed, layer, tensor, sub-id,
 * attempt, element index) into a 14-bit table index. The value an index
 * stands for (a normal quantile already cast to the tensor's storage type)
 * comes from tables that the host computes once (synth_host.c) and that the
 * host and the device both read, so a host draw and a device draw of the same
 * element are the same bytes.
 *
 * The mixing function is the output function of SplitMix64 (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, with
 * the constants of Vigna's public-domain splitmix64.c). Only 64-bit integer
 * adds, xors, shifts and multiplies are used, so every compiler computes the
 * same bits.
 *
 * The includer defines SYNTH_FN (e.g. "static inline" for C, or
 * "__host__ __device__ static inline" for HIP) before including this file.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYNTH_FN
#error "define SYNTH_FN before including synth_core.h"
#endif

#define SYNTH_TABLE_BITS 14
#define SYNTH_TABLE_SIZE (1u << SYNTH_TABLE_BITS)
#define SYNTH_GAMMA_STEP 0x9E3779B97F4A7C15ull

/* tensor ids: each tensor of each layer draws from its own stream */
enum {
  SYNTH_T_X = 1,          /* layer input x, sub = token, attempt = redraw count */
  SYNTH_T_GAMMA = 2,      /* RMSNorm gain (only when a test asks for a random one) */
  SYNTH_T_ROUTER = 3,     /* router weight [E][H] */
  SYNTH_T_EXPERT_GU = 4,  /* expert gate/up weight [2I][H], sub = expert */
  SYNTH_T_EXPERT_D = 5,   /* expert down weight [H][I], sub = expert */
  SYNTH_T_SHARED_GU = 6,  /* shared gate/up [2Is][H] */
  SYNTH_T_SHARED_D = 7,   /* shared down [H][Is] */
  SYNTH_T_BIAS_PERM = 8,  /* permutation behind the log-Zipf router bias */
  SYNTH_T_SCALE_GU = 9,   /* fp8 scale class of each 128-row group of gate/up */
  SYNTH_T_SCALE_D = 10    /* fp8 scale class of each 128-row group of down */
};

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Stream key of one tensor. Distinct (seed, layer, tensor, sub, attempt)
 * tuples give unrelated streams. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor,
                            uint32_t sub, uint32_t attempt) {
  uint64_t k = synth_mix64(seed + SYNTH_GAMMA_STEP);
  k = synth_mix64(k ^ (((uint64_t)tensor << 48) | ((uint64_t)layer << 32) | sub));
  k = synth_mix64(k + (uint64_t)attempt * SYNTH_GAMMA_STEP);
  return k;
}

/* 64 random bits number n of a stream (SplitMix64 with state key + (n+1)*gamma). */
SYNTH_FN uint64_t synth_bits(uint64_t key, uint64_t n) {
  return synth_mix64(key + (n + 1u) * SYNTH_GAMMA_STEP);
}

/* Table index of element i: four 14-bit fields per 64-bit draw. */
SYNTH_FN uint32_t synth_index(uint64_t key, uint64_t i) {
  uint64_t h = synth_bits(key, i >> 2);
  return (uint32_t)(h >> (16u * (uint32_t)(i & 3u))) & (SYNTH_TABLE_SIZE - 1u);
}

#endif
