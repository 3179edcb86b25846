/*
 * moedecode_debug.h - the ordering-stress build of libmoedecode
 * (libmoedecode_delay.so: moedecode.hip compiled with -DMOE_DEBUG_DELAY).
 *
 * That build exports every entry point of moedecode.h unchanged, plus the
 * call below. It exists to test the kernel's cross-workgroup ordering under
 * timings that a fixed launch never produces: fixed-timing kernel tests can
 * miss ordering bugs that long runs expose, among them a compiler that moved
 * an activation load above a synchronisation wait (aiposthub.com article,
 * section on how vLLM verifies AI-written kernels). The production library
 * does not export it and contains none of its code.
 */
#ifndef MOEDECODE_DEBUG_H
#define MOEDECODE_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* For later launches of this process: seed != 0 injects seeded pauses (about
 * one call site in four, up to ~55 us, keyed by seed, workgroup, wave, site)
 * before barrier arrivals, published router logits, expert gate/up tasks,
 * output-row units, routing and the combine, and maps the hardware
 * workgroups onto the work shares through a seeded permutation; seed 0
 * disables both. grid > 0 launches that many workgroups instead of one per
 * compute unit (when smaller). Results must be bit-identical to an undelayed
 * launch with the same grid. Not thread-safe with concurrent launches. */
void moe_debug_set_delay(uint64_t seed, int32_t grid);

#ifdef __cplusplus
}
#endif

#endif /* MOEDECODE_DEBUG_H */
