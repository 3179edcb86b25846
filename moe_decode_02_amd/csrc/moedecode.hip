// moedecode.hip - libmoedecode: the MoE decode layer for MI355X (gfx950).
//
// One persistent kernel per call (moe_route, moe_decode_layer, moe_decode_stack),
// one 1024-thread workgroup per compute unit. The kernel fuses what the stock
// decode path launches one by one - normalisation, matmul, activation and
// routing ops (openai-hub.com "Kimi K3 ... 1.68x", section on why decode suits
// a megakernel) - and keeps the steps of a layer inside one launch. Per layer:
//
//   x-hat   RMSNorm. At B <= 2 every workgroup normalises all tokens into its
//           own LDS (x is 14 KB per token), so no grid barrier is needed; at
//           larger B workgroup t normalises token t into global memory and a
//           barrier publishes it.
//   P0      The router GEMV, split over K into slices of about 7 KB of weights
//           (partial logits, summed later in a fixed order), then the shared
//           expert's gate/up rows, which do not depend on routing; the pages
//           run the shared expert on its own stream beside routing (smzdm.com
//           post, section "what changed", MoE de-duplication item). Every wave
//           announces "router done" before its shared rows, so the router
//           barrier has completed by the time anyone waits on it.
//   P1      Every workgroup redoes softmax + top-k + renormalisation (same
//           inputs, same code, same result: no extra barrier), builds the
//           expert gather tables in LDS (union of selected experts, each
//           expert's token list), then streams the selected experts' gate/up
//           rows: h = SiLU(g) * u.
//   P2      Each workgroup owns a block of output rows. It first reduces the
//           shared expert's down rows (their input is ready since P0), which
//           fills the wait for the expert barrier, then every selected
//           expert's down rows, then combines in a fixed order with the
//           routing weights and the residual.
//   stack   Between layers one more barrier; while waiting for it, a
//           workgroup loads the next layer's router and shared-expert rows
//           that it will read first, so they come from cache.
//
// Weight rows stream through 16-byte non-temporal loads, whole chunks of 64
// lanes with no per-lane guard, all loads of a step in flight before the
// first use. Cross-lane sums and the top-k argmax use DPP row operations.
// All reductions are fixed-order (no float atomics), so identical router rows
// give bit-identical logits and repeated runs give identical outputs.
//
// Memory ordering across the 8 XCDs: every wave releases its stores at
// workgroup scope and counts itself in LDS; the workgroup's last wave releases
// at agent scope (L2 write-back) and adds one to the barrier's global counter.
// One wave per workgroup polls the counter, acquires at agent scope and raises
// an LDS flag for the others. Weights are static and may be loaded before a
// barrier; activations are read only after it (a compiler that hoisted an
// activation load above a sync wait was one of the bugs found in the pages'
// review: aiposthub.com article, section on how vLLM verifies AI-written
// kernels).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moedecode.h"

namespace {

// ---------------------------------------------------------------------------
// constants and parameter block

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

constexpr int kThreads = 1024;  // one workgroup per CU, 16 waves
constexpr int kWaves = kThreads / 64;
constexpr int kMaxB = 64;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
constexpr int kMaxL = 8;
constexpr int kTokGroup = 4;    // tokens whose partial sums a lane holds at once
constexpr int kRowBlock = 4;    // down-projection rows per unit
constexpr int kSmallB = 2;      // B <= kSmallB: x-hat and h staged in each workgroup's LDS

enum : int { BAR_XHAT = 0, BAR_ROUTER = 1, BAR_SHARED = 2, BAR_H = 3, BAR_LAYER = 4, kBarPerLayer = 5 };
constexpr int kMaxBarriers = kBarPerLayer * kMaxL;
constexpr int kCtrlStride = 16;  // words: each control word on its own 64-byte line
enum : int { CTRL_DONE = 0, CTRL_ERR = 1, CTRL_BAR = 2 };
constexpr size_t kCtrlBytes = (size_t)(CTRL_BAR + kMaxBarriers) * kCtrlStride * sizeof(unsigned);

struct LayerPtrs {
  const void *x;          // layer input [B][H] (act)
  void *y;                // layer output [B][H] (act)
  const void *gamma;      // [H] act
  const void *rw;         // [E][H] router dtype
  const float *rb;        // [E] or null
  const void *egu;        // [E][2I][H]
  const void *ed;         // [E][H][I]
  const uint16_t *egus;   // fp8: [E][2I/128]
  const uint16_t *eds;    // fp8: [E][H/128]
  const void *sgu;        // [2Is][H]
  const void *sd;         // [H][Is]
  int32_t *idx_out;       // [B][k] or null
  float *w_out;           // [B][k] or null
  float *logits_out;      // [B][E] or null (route mode)
};

struct Params {
  int H, E, k, I, Is, B, L;
  int route_only;
  int NSR;                // router K-slices
  int NSS;                // shared gate/up K-slices (small regime), else 1
  int G;                  // workgroups
  int rows_per_wg;        // P2 output rows per workgroup (multiple of kRowBlock)
  int pass_rows;          // P2 rows per LDS pass
  float eps;
  long long timeout_ticks;  // s_memrealtime ticks (100 MHz) before a barrier wait gives up
  unsigned *ctrl;         // control words, kCtrlStride apart
  float *xhat;            // [B][H] fp32 (general regime)
  void *xa;               // [B][H] act (general regime; == xhat for fp32 activations)
  float *rpart;           // [B][E][4]: slice s of expert e's logit at [t][e][s] (s < NSR)
  float *hspart;          // [NSS][B][2 Is] (small regime)
  void *hbuf;             // [B*k][I] act
  void *hsbuf;            // [B][Is] act (general regime)
  void *xbuf[2];          // [B][H] act, stack intermediates
  // LDS carve-up, byte offsets from the start of dynamic LDS
  int o_sel_idx, o_sel_w;           // routing of each token [B*k]
  int o_ulist, o_ucnt, o_ustart;    // gather tables per union slot [min(E, B*k)]
  int o_plist;                      // (token, rank) pairs grouped by expert [B*k]
  int o_cnt, o_start, o_tmask;      // per-expert scratch of the workgroup-wide table build [E]
  int o_xf, o_xa;                   // small regime: x-hat fp32 / act [B][H]
  int o_hs;                         // small regime: shared h [B][Is] (act)
  int o_h;                          // small regime: expert h [B*k][I] (act), over x-hat once P1 is done
  int o_part;                       // P2 partial sums [pass_rows][pstride] fp32
  LayerPtrs lp[kMaxL];
};

// fixed head of the dynamic LDS
struct SmemHead {
  int bar_cnt[kMaxBarriers];    // waves of this workgroup that arrived
  int bar_claim[kMaxBarriers];  // one wave polls the global counter
  int bar_flag[kMaxBarriers];   // raised once the barrier is passed
  float red[kWaves * kSmallB];
  int scan_tmp[2 * kWaves];
  int nU;
  int route_claim, route_ready;    // small regime: the first free wave does the routing
  int shared_claim, shared_ready;  // small regime: ... and the shared expert's h
  int unit_ctr[2];                 // small regime: P2 units handed out to waves
  unsigned cand_key[kWaves][2 * 64];  // top-k candidates of each wave (ordered logit bits), then the ranked k
  int cand_idx[kWaves][2 * 64];
  unsigned sink;
};

// Kernel parameters are read in place from the kernarg segment (address space 4).
#define KARG __attribute__((address_space(4)))
typedef const KARG Params *KParams;
typedef const KARG LayerPtrs *KLayer;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_t;

// ---------------------------------------------------------------------------
// numbers

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// OCP e4m3fn byte -> fp32, exact: the 7 magnitude bits land in the fp32
// exponent/mantissa fields (exponent bias 127 instead of 7, so a factor 2^-120),
// subnormal codes land on fp32 subnormals with the same factor.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const float mag = __uint_as_float((b & 0x7Fu) << 20) * 0x1p120f;
  return (b & 0x80u) ? -mag : mag;
}

template <int D> __device__ __forceinline__ float load_act(const void *p, size_t i) {
  if constexpr (D == DT_F32) return ((const float *)p)[i];
  else return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

template <int D> __device__ __forceinline__ void store_act(void *p, size_t i, float v) {
  if constexpr (D == DT_F32) ((float *)p)[i] = v;
  else ((uint16_t *)p)[i] = f32_to_bf16(v);
}

template <int D> __device__ __forceinline__ void store_act_lds(lds_t *p, size_t i, float v) {
  if constexpr (D == DT_F32) ((__attribute__((address_space(3))) float *)p)[i] = v;
  else ((__attribute__((address_space(3))) uint16_t *)p)[i] = f32_to_bf16(v);
}

// value of v once stored in dtype D
template <int D> __device__ __forceinline__ float round_act(float v) {
  if constexpr (D == DT_F32) return v;
  else return __uint_as_float((uint32_t)f32_to_bf16(v) << 16);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <int D> constexpr int dsz() { return D == DT_F32 ? 4 : D == DT_BF16 ? 2 : 1; }
template <int WD> constexpr int epl() { return 16 / dsz<WD>(); }  // weights per 16-byte chunk

// ---------------------------------------------------------------------------
// 16-byte weight chunk . activation chunk (EPL values, NX 16-byte vectors)

template <int WD, int XD> struct Chunk;

template <> struct Chunk<DT_BF16, DT_BF16> {
  static constexpr int NX = 1;
  __device__ static __forceinline__ float dot(const u32x4 &w, const u32x4 *x, float a) {
    a = dot2_bf16(w.x, x[0].x, a);
    a = dot2_bf16(w.y, x[0].y, a);
    a = dot2_bf16(w.z, x[0].z, a);
    a = dot2_bf16(w.w, x[0].w, a);
    return a;
  }
};

template <> struct Chunk<DT_F32, DT_F32> {
  static constexpr int NX = 1;
  __device__ static __forceinline__ float dot(const u32x4 &w, const u32x4 *x, float a) {
    a = fmaf(__uint_as_float(w.x), __uint_as_float(x[0].x), a);
    a = fmaf(__uint_as_float(w.y), __uint_as_float(x[0].y), a);
    a = fmaf(__uint_as_float(w.z), __uint_as_float(x[0].z), a);
    a = fmaf(__uint_as_float(w.w), __uint_as_float(x[0].w), a);
    return a;
  }
};

template <> struct Chunk<DT_BF16, DT_F32> {
  static constexpr int NX = 2;
  __device__ static __forceinline__ float dot(const u32x4 &w, const u32x4 *x, float a) {
    a = fmaf(bf_lo(w.x), __uint_as_float(x[0].x), a);
    a = fmaf(bf_hi(w.x), __uint_as_float(x[0].y), a);
    a = fmaf(bf_lo(w.y), __uint_as_float(x[0].z), a);
    a = fmaf(bf_hi(w.y), __uint_as_float(x[0].w), a);
    a = fmaf(bf_lo(w.z), __uint_as_float(x[1].x), a);
    a = fmaf(bf_hi(w.z), __uint_as_float(x[1].y), a);
    a = fmaf(bf_lo(w.w), __uint_as_float(x[1].z), a);
    a = fmaf(bf_hi(w.w), __uint_as_float(x[1].w), a);
    return a;
  }
};

template <> struct Chunk<DT_FP8, DT_BF16> {
  static constexpr int NX = 2;
  __device__ static __forceinline__ float dot4(uint32_t w, uint32_t x01, uint32_t x23, float a) {
    a = fmaf(e4m3_to_f32(w & 0xFFu), bf_lo(x01), a);
    a = fmaf(e4m3_to_f32((w >> 8) & 0xFFu), bf_hi(x01), a);
    a = fmaf(e4m3_to_f32((w >> 16) & 0xFFu), bf_lo(x23), a);
    a = fmaf(e4m3_to_f32(w >> 24), bf_hi(x23), a);
    return a;
  }
  __device__ static __forceinline__ float dot(const u32x4 &w, const u32x4 *x, float a) {
    a = dot4(w.x, x[0].x, x[0].y, a);
    a = dot4(w.y, x[0].z, x[0].w, a);
    a = dot4(w.z, x[1].x, x[1].y, a);
    a = dot4(w.w, x[1].z, x[1].w, a);
    return a;
  }
};

// weight chunk: streamed once, so loaded non-temporal
__device__ __forceinline__ u32x4 ldw(const char *p) { return __builtin_nontemporal_load((const u32x4 *)p); }

// activation chunk, from global memory (XL = false) or LDS (XL = true)
template <bool XL> struct XSrc;
template <> struct XSrc<false> {
  typedef const char *ptr;
  __device__ static __forceinline__ u32x4 ld(ptr p, size_t off) { return *(const u32x4 *)(p + off); }
};
template <> struct XSrc<true> {
  typedef const lds_t *ptr;
  __device__ static __forceinline__ u32x4 ld(ptr p, size_t off) {
    return *(const __attribute__((address_space(3))) u32x4 *)(p + off);
  }
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// DPP cross-lane operations (wave64). After the six steps below lane 63 holds
// the reduction of the whole wave: quad swaps, half-row and row mirrors give
// every lane its 16-lane row's result; row_bcast:15 folds row 0 into row 1 and
// row 2 into row 3; row_bcast:31 folds rows 0-1 into rows 2-3.

constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}

// sum of v over the wave, valid in lane 63 (fixed order: deterministic)
__device__ __forceinline__ float wave_sum63(float v) {
  v += dpp_f<DPP_QUAD_1032, 0xF>(0.f, v);
  v += dpp_f<DPP_QUAD_2301, 0xF>(0.f, v);
  v += dpp_f<DPP_ROW_HALF_MIRROR, 0xF>(0.f, v);
  v += dpp_f<DPP_ROW_MIRROR, 0xF>(0.f, v);
  v += dpp_f<DPP_ROW_BCAST15, 0xA>(0.f, v);
  v += dpp_f<DPP_ROW_BCAST31, 0xC>(0.f, v);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// (larger value, then lower index) wins
template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
  const float ov = dpp_f<CTRL, ROWS>(v, v);
  const int oi = dpp_i<CTRL, ROWS>(i, i);
  const bool take = ov > v || (ov == v && oi < i);
  v = take ? ov : v;
  i = take ? oi : i;
}

// wave-wide argmax of (v, i); the result is returned in every lane
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
  argmax_step<DPP_QUAD_1032, 0xF>(v, i);
  argmax_step<DPP_QUAD_2301, 0xF>(v, i);
  argmax_step<DPP_ROW_HALF_MIRROR, 0xF>(v, i);
  argmax_step<DPP_ROW_MIRROR, 0xF>(v, i);
  argmax_step<DPP_ROW_BCAST15, 0xA>(v, i);
  argmax_step<DPP_ROW_BCAST31, 0xC>(v, i);
  v = readlane_f(v, 63);
  i = __builtin_amdgcn_readlane(i, 63);
}

// ---------------------------------------------------------------------------
// GEMV core: NR weight rows times TG activation rows over columns [k0, k1).
// Lane l covers chunk c0 + s*CH + l*EPL of each step; a step issues all
// NR*SEG weight loads before the first use. Full steps carry no per-lane guard;
// the remainder runs chunk by chunk with one. Rows are 16-byte aligned and
// k0, k1 multiples of EPL. acc[r][t] receives lane partial sums.

template <int WD, int XD, bool XL, int NR, int SEG, int TG>
__device__ __forceinline__ void rows_dot(const char *const (&wrow)[NR], int k0, int k1,
                                         const typename XSrc<XL>::ptr (&xr)[TG], float (&acc)[NR][TG]) {
  constexpr int EPL = epl<WD>(), NX = Chunk<WD, XD>::NX, CH = 64 * EPL;
  constexpr int WB = dsz<WD>(), XB = dsz<XD>();
  const int lane = lane_id();
  int c0 = k0;
  for (; c0 + SEG * CH <= k1; c0 += SEG * CH) {
    u32x4 w[NR][SEG];
#pragma unroll
    for (int s = 0; s < SEG; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r][s] = ldw(wrow[r] + (size_t)(c0 + s * CH + lane * EPL) * WB);
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const size_t e = (size_t)(c0 + s * CH + lane * EPL);
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        u32x4 xv[NX];
#pragma unroll
        for (int q = 0; q < NX; ++q) xv[q] = XSrc<XL>::ld(xr[t], e * XB + 16 * q);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r][t] = Chunk<WD, XD>::dot(w[r][s], xv, acc[r][t]);
      }
    }
  }
  for (; c0 < k1; c0 += CH) {
    const int e = c0 + lane * EPL;
    if (e < k1) {
      u32x4 w[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r] = ldw(wrow[r] + (size_t)e * WB);
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        u32x4 xv[NX];
#pragma unroll
        for (int q = 0; q < NX; ++q) xv[q] = XSrc<XL>::ld(xr[t], (size_t)e * XB + 16 * q);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r][t] = Chunk<WD, XD>::dot(w[r], xv, acc[r][t]);
      }
    }
  }
}

// 16-byte weight loads per lane in flight per step. HBM read bandwidth on
// MI355X peaks (about 7.1-7.3 TB/s) with only ~28-32 KB in flight per CU and
// falls with more, while every extra in-flight byte lengthens the queue that
// the latency-critical loads (barrier polls, router partials) wait in; with
// 16 waves per CU, two 1 KB wave loads each is the measured optimum.
#ifndef MOE_LOADS_PER_STEP
#define MOE_LOADS_PER_STEP 2
#endif
constexpr int kLoadsPerStep = MOE_LOADS_PER_STEP;
// chunks per step of a gate/up pair (2 rows)
template <int WD, int TG> constexpr int seg_gu() { return kLoadsPerStep >= 4 ? kLoadsPerStep / 2 : 1; }
// rows of a 4-row down unit handled per pass, and chunks per step
constexpr int kDownRows = kLoadsPerStep >= 4 ? 4 : kLoadsPerStep >= 2 ? 2 : 1;
template <int WD, int TG> constexpr int seg_down() { return kLoadsPerStep / kDownRows > 0 ? kLoadsPerStep / kDownRows : 1; }
// chunks per step of a router row slice
template <int WD, int TG> constexpr int seg_router() { return kLoadsPerStep; }

// Run f.template operator()<TG>(t0, nt) over groups of up to kTokGroup of n
// tokens, with the smallest specialisation that holds each group.
template <class F>
__device__ __forceinline__ void for_token_groups(int n, F &&f) {
  for (int t0 = 0; t0 < n; t0 += kTokGroup) {
    const int nt = min(kTokGroup, n - t0);
    if (nt == 1) f.template operator()<1>(t0, nt);
    else if (nt == 2) f.template operator()<2>(t0, nt);
    else f.template operator()<4>(t0, nt);
  }
}

// ---------------------------------------------------------------------------
// grid barriers

__device__ __forceinline__ long long rt_now() { return (long long)__builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ unsigned *ctrl_word(KParams p, int w) { return p->ctrl + (size_t)w * kCtrlStride; }

// Small regime: values other workgroups read after a barrier are written
// with device-coherent stores (write-through past this XCD's L2), so the
// barrier does not need an L2 write-back, which costs several microseconds
// per workgroup while the memory system is streaming.
__device__ __forceinline__ void publish(float *q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wave is done with the work barrier b waits for, and every value it wrote
// for other workgroups went out through publish(): waiting for its stores to
// complete (they are then visible device-wide) replaces the L2 write-back.
// Readers still acquire at agent scope (L1/L2 invalidate) before reading.
__device__ void bar_arrive_published(KParams p, SmemHead &sh, int b) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane_id() == 0) {
    const int old = __hip_atomic_fetch_add(&sh.bar_cnt[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (old == kWaves - 1)
      __hip_atomic_fetch_add(ctrl_word(p, CTRL_BAR + b), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// A wave is done with the work barrier b waits for.
__device__ void bar_arrive(KParams p, SmemHead &sh, int b) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane_id() == 0) {
    const int old = __hip_atomic_fetch_add(&sh.bar_cnt[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (old == kWaves - 1) {
      // the whole workgroup's stores are in this XCD's L2: write them back for the other XCDs
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(ctrl_word(p, CTRL_BAR + b), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Wait until every workgroup arrived at barrier b.
__device__ void bar_wait(KParams p, SmemHead &sh, int b) {
  if (lane_id() == 0) {
    if (__hip_atomic_load(&sh.bar_flag[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
      const bool poller =
          __hip_atomic_exchange(&sh.bar_claim[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
      const long long t0 = rt_now();
      if (poller) {
        unsigned *cnt = ctrl_word(p, CTRL_BAR + b);
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)p->G) {
          __builtin_amdgcn_s_sleep(1);
          if (rt_now() - t0 > p->timeout_ticks) {
            __hip_atomic_store(ctrl_word(p, CTRL_ERR), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&sh.bar_flag[b], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        while (__hip_atomic_load(&sh.bar_flag[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          __builtin_amdgcn_s_sleep(1);
          if (rt_now() - t0 > 2 * p->timeout_ticks) break;
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// LDS views

struct Lds {
  unsigned char *base;
  __device__ SmemHead &head() const { return *reinterpret_cast<SmemHead *>(base); }
  template <class T> __device__ T *at(int off) const { return reinterpret_cast<T *>(base + off); }
  __device__ lds_t *raw(int off) const { return (lds_t *)(base + off); }
};

// ---------------------------------------------------------------------------
// x-hat

// Activation chunk c (16 bytes) of a row; chunks past the row's end read
// chunk 0 (always in bounds) and are masked by the caller.
template <int AD> constexpr int act_chunks_max() { return AD == DT_F32 ? 4 : 2; }  // (H <= 16384) / 1024 threads

template <int AD>
__device__ __forceinline__ void act_chunk_vals(const u32x4 &v, float (&f)[8]) {
  if constexpr (AD == DT_F32) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y); f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  }
}

// RMSNorm of NT tokens (rows x_t of `x`, t = tok[i]) by the whole workgroup:
// every load is issued before the first use (one round trip); out(t, h, v)
// receives x-hat. Chunk c of a row is handled by thread c mod 1024.
template <int AD, int NT, class Out>
__device__ __forceinline__ void rmsnorm_rows(KParams p, KLayer lp, SmemHead &sh, const int (&tok)[NT], Out &&out) {
  constexpr int EPC = 16 / dsz<AD>(), NC = act_chunks_max<AD>();
  const int H = p->H, tid = threadIdx.x, nch = H / EPC;
  u32x4 xv[NT][NC], gv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + c * kThreads;
    const int cc = ch < nch ? ch : 0;
    gv[c] = *(const u32x4 *)((const char *)lp->gamma + (size_t)cc * 16);
#pragma unroll
    for (int i = 0; i < NT; ++i) xv[i][c] = *(const u32x4 *)((const char *)lp->x + ((size_t)tok[i] * nch + cc) * 16);
  }
  float ss[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (tid + c * kThreads < nch) {
        float f[8];
        act_chunk_vals<AD>(xv[i][c], f);
#pragma unroll
        for (int q = 0; q < EPC; ++q) ss[i] = fmaf(f[q], f[q], ss[i]);
      }
    }
    ss[i] = readlane_f(wave_sum63(ss[i]), 63);
    if (lane_id() == 0) sh.red[i * kWaves + wave_id()] = ss[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float tot = 0.f;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sh.red[i * kWaves + w2];
    const float r = 1.0f / sqrtf(tot / (float)H + p->eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = tid + c * kThreads;
      if (ch < nch) {
        float f[8], g[8];
        act_chunk_vals<AD>(xv[i][c], f);
        act_chunk_vals<AD>(gv[c], g);
#pragma unroll
        for (int q = 0; q < EPC; ++q) out(i, ch * EPC + q, f[q] * r * g[q]);
      }
    }
  }
  __syncthreads();
}

// Small regime: this workgroup normalises every token into its own LDS:
// xf [B][H] fp32 (router input) and xa [B][H] act (FFN input).
template <int AD>
__device__ __attribute__((noinline)) void stage_xhat(KParams p, KLayer lp, const Lds &L) {
  const int H = p->H;
  float *xf = L.at<float>(p->o_xf);
  lds_t *xa = L.raw(p->o_xa);
  auto put = [&](int t, int h, float v) {
    xf[(size_t)t * H + h] = v;
    if constexpr (AD != DT_F32) store_act_lds<AD>(xa, (size_t)t * H + h, v);
  };
  if (p->B == 1) {
    const int tok[1] = {0};
    rmsnorm_rows<AD, 1>(p, lp, L.head(), tok, put);
  } else {
    const int tok[2] = {0, 1};
    rmsnorm_rows<AD, 2>(p, lp, L.head(), tok, put);
  }
}

// General regime: workgroup t normalises token t into global memory.
template <int AD>
__device__ __attribute__((noinline)) void produce_xhat(KParams p, KLayer lp, const Lds &L) {
  const int H = p->H;
  for (int t = blockIdx.x; t < p->B; t += p->G) {
    const int tok[1] = {t};
    rmsnorm_rows<AD, 1>(p, lp, L.head(), tok, [&](int, int h, float v) {
      p->xhat[(size_t)t * H + h] = v;
      if constexpr (AD != DT_F32) store_act<AD>(p->xa, (size_t)t * H + h, v);
    });
  }
}

// pointer to token t's row of x-hat (fp32 if F32X, else act) in LDS or global memory
template <bool XL, int AD, bool F32X>
__device__ __forceinline__ typename XSrc<XL>::ptr xhat_row(KParams p, const Lds &L, int t) {
  constexpr int XB = F32X ? 4 : dsz<AD>();
  if constexpr (XL) {
    const int off = (F32X || AD == DT_F32) ? p->o_xf : p->o_xa;
    return L.raw(off) + (size_t)t * p->H * XB;
  } else {
    const char *base = (F32X || AD == DT_F32) ? (const char *)p->xhat : (const char *)p->xa;
    return base + (size_t)t * p->H * XB;
  }
}

// ---------------------------------------------------------------------------
// P0: router slices and shared gate/up rows

// task (row e, slice s) -> rpart[s][t][e] for all tokens
template <int RD, bool XL>
__device__ __forceinline__ void router_task(KParams p, KLayer lp, const Lds &L, int e, int s) {
  const int H = p->H, E = p->E, B = p->B;
  const int Ks = H / p->NSR;
  const char *const wrow[1] = {(const char *)lp->rw + (size_t)e * H * dsz<RD>()};
  for_token_groups(B, [&]<int TG>(int t0, int nt) {
    typename XSrc<XL>::ptr xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) xr[t] = xhat_row<XL, DT_F32, true>(p, L, t0 + (t < nt ? t : 0));
    float acc[1][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = 0.f;
    rows_dot<RD, DT_F32, XL, 1, seg_router<RD, TG>(), TG>(wrow, s * Ks, (s + 1) * Ks, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float v = wave_sum63(acc[0][t]);
      if (t < nt && lane_id() == 63) {
        float *q = p->rpart + ((size_t)(t0 + t) * E + e) * 4 + s;
        if constexpr (XL) publish(q, v);
        else *q = v;
      }
    }
  });
}

// shared gate/up task (pair j, slice s). Small regime: partial g and u sums to
// hspart[s][t][j] and hspart[s][t][Is + j]. General regime (one slice): h.
template <int AD, int SD, bool XL>
__device__ __forceinline__ void shared_gu_task(KParams p, KLayer lp, const Lds &L, int j, int s) {
  const int H = p->H, B = p->B, Is = p->Is;
  const int Ks = H / p->NSS;
  const size_t rowb = (size_t)H * dsz<SD>();
  const char *const wrow[2] = {(const char *)lp->sgu + (size_t)j * rowb, (const char *)lp->sgu + (size_t)(Is + j) * rowb};
  for_token_groups(B, [&]<int TG>(int t0, int nt) {
    typename XSrc<XL>::ptr xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) xr[t] = xhat_row<XL, AD, false>(p, L, t0 + (t < nt ? t : 0));
    float acc[2][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = acc[1][t] = 0.f;
    rows_dot<SD, AD, XL, 2, seg_gu<SD, TG>(), TG>(wrow, s * Ks, (s + 1) * Ks, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float g = wave_sum63(acc[0][t]);
      const float u = wave_sum63(acc[1][t]);
      if (t < nt && lane_id() == 63) {
        if (p->NSS > 1 || XL) {
          float *hp = p->hspart + ((size_t)s * B + t0 + t) * 2 * Is;
          publish(hp + j, g);
          publish(hp + Is + j, u);
        } else {
          store_act<AD>(p->hsbuf, (size_t)(t0 + t) * Is + j, silu_mul(g, u));
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// top-k of one token (one wave): softmax over all E logits restricted to the
// k largest (ties to the lower index), renormalised.
//
// Lane l holds the logits of experts l, l+64, ... . The k-th largest of the 64
// lane maxima, T, is found by a bitwise search with wave ballots; at least k
// lanes reach T, so every one of the k largest logits is >= T and only the
// logits >= T (usually a few dozen) are candidates. The candidates are
// compacted into LDS and each is ranked against all others by (logit desc,
// index asc); ranks below k are the selection, in order. When more than 64
// logits tie at the threshold, a 64-round-free fallback runs k rounds of
// wave argmax instead.

// float -> unsigned with the same order (-0 and +0 are made equal first)
__device__ __forceinline__ unsigned ord_f32(float v) {
  const unsigned u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(unsigned o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

constexpr int kMaxCand = 64;

// Logits of token t for the experts of this lane (e = lane + 64 j), from the
// router partials: one 16-byte load per expert holds its K-slice partials,
// all loads issued before the first use. Slots past E read expert E-1.
__device__ __forceinline__ void load_logits(KParams p, KLayer lp, int t, float (&v)[kMaxE / 64]) {
  const int lane = lane_id(), E = p->E, NSR = p->NSR;
  constexpr int PER = kMaxE / 64;
  const u32x4 *base = (const u32x4 *)(p->rpart + (size_t)t * E * 4);
  u32x4 q[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) q[j] = base[min(lane + 64 * j, E - 1)];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    float s = __uint_as_float(q[j].x);
    if (NSR > 1) s += __uint_as_float(q[j].y);
    if (NSR > 2) s += __uint_as_float(q[j].z);
    if (NSR > 3) s += __uint_as_float(q[j].w);
    v[j] = s;
  }
  if (const float *rb = lp->rb) {
    float b[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) b[j] = rb[min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] += b[j];
  }
}

// Rare path (more than 64 logits tie at the threshold): k rounds of wave
// argmax over all logits. Returns the selection in lanes < k.
__device__ __attribute__((noinline)) void topk_rounds(KParams p, KLayer lp, int t, float &myv, int &myidx) {
  const int lane = lane_id(), E = p->E, k = p->k;
  constexpr int PER = kMaxE / 64;
  float v[PER];
  load_logits(p, lp, t, v);
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? ((v[j] == v[j]) ? v[j] : -INFINITY) : qnan;  // NaN never wins
  }
  for (int i = 0; i < k; ++i) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (v[j] > bv || (v[j] == bv && e < bi)) { bv = v[j]; bi = e; }
    }
    wave_argmax(bv, bi);
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (lane + 64 * j == bi) v[j] = qnan;  // taken
    if (lane == i) { myv = bv; myidx = bi; }
  }
}

__device__ __attribute__((noinline)) void topk_token(KParams p, KLayer lp, const Lds &L, int t, bool write_out) {
  const int lane = lane_id();
  const int E = p->E, k = p->k;
  constexpr int PER = kMaxE / 64;
  float v[PER];
  load_logits(p, lp, t, v);
  unsigned o[PER];
  unsigned omax = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    // a NaN logit ranks last but stays selectable; a slot past E ranks below every expert
    if (e < E) v[j] = (v[j] == v[j]) ? v[j] : -INFINITY;
    if (write_out && lp->logits_out && e < E) lp->logits_out[(size_t)t * E + e] = v[j];
    o[j] = e < E ? ord_f32(v[j]) : 0u;
    omax = max(omax, o[j]);
  }
  // T = k-th largest lane maximum (largest T with at least k lanes >= T)
  unsigned thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned c = thr | (1u << bit);
    if (__popcll(__ballot(omax >= c)) >= k) thr = c;
  }
  int nc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) nc += (lane + 64 * j < E && o[j] >= thr) ? 1 : 0;
  // exclusive prefix of the candidate counts over the lanes
  int incl = nc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  const int total = __shfl(incl, 63);
  int *sel_idx = L.at<int>(p->o_sel_idx);
  float *sel_w = L.at<float>(p->o_sel_w);
  int myidx = 0;
  float myv = -INFINITY;
  if (total <= kMaxCand) {
    unsigned *ck = L.head().cand_key[wave_id()];
    int *ci = L.head().cand_idx[wave_id()];
    int pos = incl - nc;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (e < E && o[j] >= thr) { ck[pos] = o[j]; ci[pos] = e; ++pos; }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    if (lane < total) {
      const unsigned mk = ck[lane];
      const int me = ci[lane];
      int rank = 0;
      for (int c = 0; c < total; ++c) {
        const unsigned ok = ck[c];
        const int oe = ci[c];
        rank += (ok > mk || (ok == mk && oe < me)) ? 1 : 0;
      }
      if (rank < k) {
        ck[kMaxCand + rank] = mk;
        ci[kMaxCand + rank] = me;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    if (lane < k) {
      myv = unord_f32(ck[kMaxCand + lane]);
      myidx = ci[kMaxCand + lane];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  } else {
    topk_rounds(p, lp, t, myv, myidx);
  }
  // renormalised softmax over the selection (the denominator over all E cancels)
  const bool mine = lane < k;
  const float lmax = readlane_f(myv, 0);
  const float ex = mine ? expf(myv - lmax) : 0.f;
  const float z = readlane_f(wave_sum63(ex), 63);
  if (mine) {
    const float wgt = ex / z;
    sel_idx[t * k + lane] = myidx;
    sel_w[t * k + lane] = wgt;
    if (write_out) {
      if (lp->idx_out) lp->idx_out[(size_t)t * k + lane] = myidx;
      if (lp->w_out) lp->w_out[(size_t)t * k + lane] = wgt;
    }
  }
}

// gather tables: union U of selected experts (ascending), each expert's pairs
// (t*k+i) in ascending token order.
__device__ __attribute__((noinline)) void build_tables(KParams p, const Lds &L) {
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int E = p->E, P = p->B * p->k;
  SmemHead &sh = L.head();
  int *cnt = L.at<int>(p->o_cnt), *start = L.at<int>(p->o_start), *ulist = L.at<int>(p->o_ulist);
  int *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  int *plist = L.at<int>(p->o_plist);
  const int *sel_idx = L.at<int>(p->o_sel_idx);
  unsigned long long *tmask = L.at<unsigned long long>(p->o_tmask);
  for (int e = tid; e < E; e += kThreads) { cnt[e] = 0; tmask[e] = 0ull; }
  __syncthreads();
  for (int q = tid; q < P; q += kThreads) {
    const int e = sel_idx[q];
    atomicAdd(&cnt[e], 1);
    atomicOr(&tmask[e], 1ull << (q / p->k));
  }
  __syncthreads();
  // block scan over e of (cnt, cnt > 0); E <= kThreads
  const int c = (tid < E) ? cnt[tid] : 0;
  const int f = c > 0 ? 1 : 0;
  int ci = c, fi = f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int uc = __shfl_up(ci, o), uf = __shfl_up(fi, o);
    if (lane >= o) { ci += uc; fi += uf; }
  }
  if (lane == 63) { sh.scan_tmp[wv] = ci; sh.scan_tmp[kWaves + wv] = fi; }
  __syncthreads();
  int bc = 0, bf = 0;
  for (int w2 = 0; w2 < wv; ++w2) { bc += sh.scan_tmp[w2]; bf += sh.scan_tmp[kWaves + w2]; }
  if (tid < E) {
    start[tid] = bc + ci - c;
    if (f) ulist[bf + fi - f] = tid;
  }
  if (tid == kThreads - 1) {
    int tot = 0;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sh.scan_tmp[kWaves + w2];
    sh.nU = tot;
  }
  __syncthreads();
  for (int q = tid; q < P; q += kThreads) {
    const int e = sel_idx[q];
    const int t = q / p->k;
    const unsigned long long below = (t == 0) ? 0ull : (tmask[e] & ((1ull << t) - 1ull));
    plist[start[e] + __popcll(below)] = q;
  }
  for (int u = tid; u < sh.nU; u += kThreads) {
    ucnt[u] = cnt[ulist[u]];
    ustart[u] = start[ulist[u]];
  }
  __syncthreads();
}

// The same tables built by one wave when B*k <= 64: the (expert, pair) keys
// are sorted across the lanes (bitonic), then each run of equal experts is a
// union slot. Pairs of one expert keep ascending order, hence ascending tokens.
__device__ __attribute__((noinline)) void build_tables_wave(KParams p, const Lds &L) {
  const int lane = lane_id(), P = p->B * p->k;
  const int *sel_idx = L.at<int>(p->o_sel_idx);
  int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  int *plist = L.at<int>(p->o_plist);
  unsigned key = lane < P ? ((unsigned)sel_idx[lane] << 6) | (unsigned)lane : 0xFFFFFFFFu;
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const unsigned o = (unsigned)__shfl_xor((int)key, j);
      const bool asc = (lane & kk) == 0, low = (lane & j) == 0;
      key = (asc == low) ? min(key, o) : max(key, o);
    }
  const bool valid = lane < P;
  const unsigned prev = (unsigned)__shfl_up((int)key, 1);
  const bool first = valid && (lane == 0 || (prev >> 6) != (key >> 6));
  const unsigned long long firsts = __ballot(first);
  if (valid) plist[lane] = (int)(key & 63u);
  if (first) {
    const int rank = __popcll(firsts & ((1ull << lane) - 1ull));
    const unsigned long long rest = lane < 63 ? firsts >> (lane + 1) : 0ull;
    const int nxt = rest ? lane + __ffsll((long long)rest) : P;
    ulist[rank] = (int)(key >> 6);
    ustart[rank] = lane;
    ucnt[rank] = nxt - lane;
  }
  if (lane == 0) L.head().nU = __popcll(firsts);
}

// ---------------------------------------------------------------------------
// P1: expert gate/up, task (expert u of U, pair j)

template <int AD, int ED, bool XL>
__device__ __forceinline__ void expert_gu_task(KParams p, KLayer lp, const Lds &L, int u, int j) {
  const int H = p->H, I = p->I, k = p->k;
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *plist = L.at<int>(p->o_plist);
  const int e = ulist[u];
  const int n = ucnt[u];
  const int *pl = plist + ustart[u];
  const size_t rowb = (size_t)H * dsz<ED>();
  const char *gu = (const char *)lp->egu + (size_t)e * 2 * I * rowb;
  const char *const wrow[2] = {gu + (size_t)j * rowb, gu + (size_t)(I + j) * rowb};
  float gs = 1.f, us = 1.f;
  if constexpr (ED == DT_FP8) {
    // e4m3_to_f32 is exact, so the bf16 row scale multiplies the finished dot
    const uint16_t *sc = lp->egus + (size_t)e * (2 * I / 128);
    gs = __uint_as_float((uint32_t)sc[j / 128] << 16);
    us = __uint_as_float((uint32_t)sc[(I + j) / 128] << 16);
  }
  for_token_groups(n, [&]<int TG>(int t0, int nt) {
    typename XSrc<XL>::ptr xr[TG];
    int slot[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      slot[t] = pl[t0 + (t < nt ? t : 0)];
      xr[t] = xhat_row<XL, AD, false>(p, L, slot[t] / k);
    }
    float acc[2][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = acc[1][t] = 0.f;
    rows_dot<ED, AD, XL, 2, seg_gu<ED, TG>(), TG>(wrow, 0, H, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float g = wave_sum63(acc[0][t]) * gs;
      const float uu = wave_sum63(acc[1][t]) * us;
      if (t < nt && lane_id() == 63) {
        const float h = silu_mul(g, uu);
        // small regime: fp32 copy of the act-rounded h, published; otherwise h in the act dtype
        if constexpr (XL) publish((float *)p->hbuf + (size_t)slot[t] * I + j, round_act<AD>(h));
        else store_act<AD>(p->hbuf, (size_t)slot[t] * I + j, h);
      }
    }
  });
}

// ---------------------------------------------------------------------------
// P2: down projections of this workgroup's rows

// Small regime, one wave: the shared expert's h for every token from the
// slice partials, into LDS. Lane l covers 4 consecutive columns per step; all
// partial loads of a step are issued before the first use.
template <int AD>
__device__ __attribute__((noinline)) void finish_shared_h_wave(KParams p, const Lds &L) {
  const int Is = p->Is, B = p->B, NSS = p->NSS, lane = lane_id();
  lds_t *hs = L.raw(p->o_hs);
  constexpr int U = 2;  // 16-byte groups per lane per step
  for (int t = 0; t < B; ++t) {
    for (int j0 = 0; j0 < Is; j0 += 64 * 4 * U) {
      u32x4 g[U][2], u[U][2];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int j = min(j0 + (q * 64 + lane) * 4, Is - 4);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float *hp = p->hspart + ((size_t)min(s2, NSS - 1) * B + t) * 2 * Is;
          g[q][s2] = *(const u32x4 *)(hp + j);
          u[q][s2] = *(const u32x4 *)(hp + Is + j);
        }
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int j = j0 + (q * 64 + lane) * 4;
        if (j < Is) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float gg = __uint_as_float(g[q][0][c]), uu = __uint_as_float(u[q][0][c]);
            if (NSS > 1) { gg += __uint_as_float(g[q][1][c]); uu += __uint_as_float(u[q][1][c]); }
            store_act_lds<AD>(hs, (size_t)t * Is + j + c, silu_mul(gg, uu));
          }
        }
      }
    }
  }
}

// Small regime: the expert h of every selected (token, expert) pair, from the
// published fp32 copy into LDS in the act dtype (values are already rounded).
// Every load is issued before the first use.
template <int AD>
__device__ __attribute__((noinline)) void stage_h(KParams p, const Lds &L) {
  const int n4 = p->B * p->k * p->I / 4;  // groups of 4 values
  constexpr int U = 8;                     // covers B*k*I <= 32768 values in one round
  const u32x4 *src = (const u32x4 *)p->hbuf;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = threadIdx.x + u * kThreads;
    v[u] = src[i < n4 ? i : 0];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i < n4) {
      if constexpr (AD == DT_F32) {
        *(__attribute__((address_space(3))) u32x4 *)(L.raw(p->o_h) + (size_t)i * 16) = v[u];
      } else {
        // the values are bf16-exact: their top halves are the bf16 patterns
        const uint32_t lo = (v[u].x >> 16) | (v[u].y & 0xFFFF0000u);
        const uint32_t hi = (v[u].z >> 16) | (v[u].w & 0xFFFF0000u);
        *(__attribute__((address_space(3))) u32x2 *)(L.raw(p->o_h) + (size_t)i * 8) = u32x2{lo, hi};
      }
    }
  }
  for (int i = threadIdx.x + U * kThreads; i < n4; i += kThreads) {  // larger shapes: rest, one by one
    const u32x4 w = src[i];
    if constexpr (AD == DT_F32) {
      *(__attribute__((address_space(3))) u32x4 *)(L.raw(p->o_h) + (size_t)i * 16) = w;
    } else {
      *(__attribute__((address_space(3))) u32x2 *)(L.raw(p->o_h) + (size_t)i * 8) =
          u32x2{(w.x >> 16) | (w.y & 0xFFFF0000u), (w.z >> 16) | (w.w & 0xFFFF0000u)};
    }
  }
}

// One 4-row unit of a [rows][K] down matrix: row pointers wrow, columns
// [0, I) of x rows xr (TG tokens); writes the row sums times sc[r] to
// part[(o0 + r - pr0) * pstride + col[t]].
template <int WD, int AD, bool XL, int TG>
__device__ __forceinline__ void down_unit(const char *const (&wrow)[kRowBlock], int I,
                                          const typename XSrc<XL>::ptr (&xr)[TG], const float (&sc)[kRowBlock],
                                          float *prow, int pstride, const int (&col)[TG], int nt) {
#pragma unroll
  for (int r0 = 0; r0 < kRowBlock; r0 += kDownRows) {
    const char *wr[kDownRows];
    float acc[kDownRows][TG];
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) {
      wr[r] = wrow[r0 + r];
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[r][t] = 0.f;
    }
    rows_dot<WD, AD, XL, kDownRows, seg_down<WD, TG>(), TG>(wr, 0, I, xr, acc);
#pragma unroll
    for (int r = 0; r < kDownRows; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float v = wave_sum63(acc[r][t]) * sc[r0 + r];
        if (t < nt && lane_id() == 63) prow[(r0 + r) * pstride + col[t]] = v;
      }
  }
}

// Next P2 unit of this wave: handed out through an LDS counter (DYN, small
// regime) or dealt round-robin from wave w0.
template <bool DYN>
__device__ __forceinline__ int next_unit(SmemHead &sh, int which, int &cur, int w0) {
  if constexpr (DYN) {
    int u = 0;
    if (lane_id() == 0) u = __hip_atomic_fetch_add(&sh.unit_ctr[which], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(u);
  } else {
    cur = (cur < 0) ? (wave_id() + kWaves - w0 % kWaves) % kWaves : cur + kWaves;
    return cur;
  }
}

// shared-expert units of rows [pr0, pr1): (row block, column block hf); the
// shared h comes from LDS (small regime) or global memory
template <int AD, int SD, bool SMALL>
__device__ __forceinline__ void shared_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int w0) {
  const int I = p->I, Is = p->Is, B = p->B;
  const int nsh = Is / I, P = B * p->k, pstride = P + B * nsh;
  const int nrb = (pr1 - pr0) / kRowBlock;
  float *part = L.at<float>(p->o_part);
  const float one[kRowBlock] = {1.f, 1.f, 1.f, 1.f};
  int cur = -1;
  for (int un = next_unit<SMALL>(L.head(), 0, cur, w0); un < nrb * nsh; un = next_unit<SMALL>(L.head(), 0, cur, w0)) {
    const int hf = un / nrb, rb = un % nrb;
    const int o0 = pr0 + rb * kRowBlock;
    const char *wrow[kRowBlock];
#pragma unroll
    for (int r = 0; r < kRowBlock; ++r)
      wrow[r] = (const char *)lp->sd + ((size_t)(o0 + r) * Is + (size_t)hf * I) * dsz<SD>();
    for_token_groups(B, [&]<int TG>(int t0, int nt) {
      typename XSrc<SMALL>::ptr xr[TG];
      int col[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const int tt = t0 + (t < nt ? t : 0);
        if constexpr (SMALL) xr[t] = L.raw(p->o_hs) + ((size_t)tt * Is + (size_t)hf * I) * dsz<AD>();
        else xr[t] = (const char *)p->hsbuf + ((size_t)tt * Is + (size_t)hf * I) * dsz<AD>();
        col[t] = P + (t0 + t) * nsh + hf;
      }
      down_unit<SD, AD, SMALL, TG>(wrow, I, xr, one, part + (size_t)(o0 - pr0) * pstride, pstride, col, nt);
    });
  }
}

// routed-expert units of rows [pr0, pr1): (expert slot, row block), expert-major
// so a wave's consecutive units read consecutive rows; h from LDS (small
// regime) or global memory
template <int AD, int ED, bool SMALL>
__device__ __forceinline__ void expert_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int w0) {
  const int H = p->H, I = p->I, B = p->B;
  const int nsh = p->Is / I, P = B * p->k, pstride = P + B * nsh;
  const int nU = L.head().nU;
  const int nrb = (pr1 - pr0) / kRowBlock;
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *plist = L.at<int>(p->o_plist);
  float *part = L.at<float>(p->o_part);
  int cur = -1;
  for (int un = next_unit<SMALL>(L.head(), 1, cur, w0); un < nrb * nU; un = next_unit<SMALL>(L.head(), 1, cur, w0)) {
    const int s = un / nrb, rb = un % nrb;
    const int o0 = pr0 + rb * kRowBlock;
    const int e = ulist[s];
    const int n = ucnt[s];
    const int *pl = plist + ustart[s];
    const char *wrow[kRowBlock];
    float sc[kRowBlock];
#pragma unroll
    for (int r = 0; r < kRowBlock; ++r) {
      wrow[r] = (const char *)lp->ed + ((size_t)e * H + o0 + r) * I * dsz<ED>();
      sc[r] = 1.f;
      if constexpr (ED == DT_FP8) sc[r] = __uint_as_float((uint32_t)lp->eds[(size_t)e * (H / 128) + (o0 + r) / 128] << 16);
    }
    for_token_groups(n, [&]<int TG>(int t0, int nt) {
      typename XSrc<SMALL>::ptr xr[TG];
      int col[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        col[t] = pl[t0 + (t < nt ? t : 0)];
        if constexpr (SMALL) xr[t] = L.raw(p->o_h) + (size_t)col[t] * I * dsz<AD>();
        else xr[t] = (const char *)p->hbuf + (size_t)col[t] * I * dsz<AD>();
      }
      down_unit<ED, AD, SMALL, TG>(wrow, I, xr, sc, part + (size_t)(o0 - pr0) * pstride, pstride, col, nt);
    });
  }
}

// y = x + shared + sum_i w_i d_i (rank order i) for rows [pr0, pr1)
template <int AD>
__device__ __forceinline__ void combine(KParams p, KLayer lp, const Lds &L, int pr0, int pr1) {
  const int H = p->H, k = p->k, B = p->B;
  const int nsh = p->Is / p->I, P = B * k, pstride = P + B * nsh;
  const float *part = L.at<float>(p->o_part);
  const float *sel_w = L.at<float>(p->o_sel_w);
  const int cells = (pr1 - pr0) * B;
  for (int c = threadIdx.x; c < cells; c += kThreads) {
    const int ro = c / B, t = c % B;
    const int o = pr0 + ro;
    const float *pp = part + (size_t)ro * pstride;
    float sh = 0.f;
    for (int hf = 0; hf < nsh; ++hf) sh += pp[P + t * nsh + hf];
    float rt = 0.f;
    for (int i = 0; i < k; ++i) rt = fmaf(sel_w[t * k + i], pp[t * k + i], rt);
    const float v = load_act<AD>(lp->x, (size_t)t * H + o) + sh + rt;
    store_act<AD>(lp->y, (size_t)t * H + o, v);
  }
}

// Bring the lines of [p, p + bytes) into the caches: one 4-byte load per
// 128-byte line, folded into a value that is never used.
__device__ __forceinline__ unsigned touch_lines(const char *p, size_t bytes) {
  unsigned acc = 0;
  for (size_t off = (size_t)lane_id() * 128; off < bytes; off += 64 * 128) acc ^= *(const unsigned *)(p + off);
  return acc;
}

// The weights this wave reads first in the next layer's P0 (its router and
// shared gate/up slices), loaded while the layer barrier is pending.
template <int RD, int SD>
__device__ __forceinline__ unsigned prefetch_p0(KParams p, KLayer nl, int W, int NW) {
  const int H = p->H, NSR = p->NSR, NSS = p->NSS, E = p->E, Is = p->Is;
  const int nrt = E * NSR;
  unsigned acc = 0;
  for (int tau = W; tau < nrt + Is * NSS; tau += NW) {
    if (tau < nrt) {
      const int e = tau / NSR, s = tau % NSR;
      const size_t ks = (size_t)(H / NSR) * dsz<RD>();
      acc ^= touch_lines((const char *)nl->rw + (size_t)e * H * dsz<RD>() + s * ks, ks);
    } else {
      const int j = (tau - nrt) / NSS, s = (tau - nrt) % NSS;
      const size_t ks = (size_t)(H / NSS) * dsz<SD>();
      const size_t rowb = (size_t)H * dsz<SD>();
      acc ^= touch_lines((const char *)nl->sgu + (size_t)j * rowb + s * ks, ks);
      acc ^= touch_lines((const char *)nl->sgu + (size_t)(Is + j) * rowb + s * ks, ks);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// the kernel

// Small regime: the first wave of the workgroup to get here (it has no P0
// work left) waits for the router barrier, routes every token and builds the
// gather tables; the other waves keep streaming their P0 rows meanwhile and
// pick the tables up from LDS when they are done.
template <bool FIRST_WAVE_ROUTES>
__device__ __forceinline__ void route_small(KParams p, KLayer lp, const Lds &L, int b_router) {
  SmemHead &sh = L.head();
  int claimed = 0;
  if (lane_id() == 0)
    claimed = __hip_atomic_exchange(&sh.route_claim, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
  claimed = __builtin_amdgcn_readfirstlane(claimed);
  if (claimed) {
    bar_wait(p, sh, b_router);
    for (int t = 0; t < p->B; ++t) topk_token(p, lp, L, t, blockIdx.x == 0);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    build_tables_wave(p, L);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane_id() == 0) __hip_atomic_store(&sh.route_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else if (lane_id() == 0) {
    while (__hip_atomic_load(&sh.route_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Small regime: the first wave done with P1 waits for the shared barrier and
// finishes the shared expert's h in LDS; the others wait for it.
template <int AD>
__device__ __forceinline__ void shared_h_small(KParams p, const Lds &L, int b_shared) {
  SmemHead &sh = L.head();
  int claimed = 0;
  if (lane_id() == 0)
    claimed = __hip_atomic_exchange(&sh.shared_claim, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
  claimed = __builtin_amdgcn_readfirstlane(claimed);
  if (claimed) {
    bar_wait(p, sh, b_shared);
    finish_shared_h_wave<AD>(p, L);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane_id() == 0) __hip_atomic_store(&sh.shared_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else if (lane_id() == 0) {
    while (__hip_atomic_load(&sh.shared_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int AD, int RD, int ED, int SD, bool SMALL>
__global__ void __launch_bounds__(kThreads, 1) moe_kernel(Params params) {
  // read the parameters in place in the kernarg segment (scalar loads; no private copy)
  (void)params;
  KParams p = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const Lds L{smem_raw};
  SmemHead &sh = L.head();
  const int tid = threadIdx.x, wv = wave_id();
  const int NW = p->G * kWaves;
  const int W = blockIdx.x * kWaves + wv;  // global wave id

  for (int i = tid; i < kMaxBarriers; i += kThreads) sh.bar_cnt[i] = sh.bar_claim[i] = sh.bar_flag[i] = 0;
  if (tid == 0) sh.sink = 0;

  unsigned sink = 0;
  for (int l = 0; l < p->L; ++l) {
    KLayer lp = &p->lp[l];
    const int b0 = kBarPerLayer * l;
    if (tid == 0) {
      sh.route_claim = sh.route_ready = sh.shared_claim = sh.shared_ready = 0;
      sh.unit_ctr[0] = sh.unit_ctr[1] = 0;
    }
    __syncthreads();

    // x-hat
    if constexpr (SMALL) {
      stage_xhat<AD>(p, lp, L);
    } else {
      produce_xhat<AD>(p, lp, L);
      bar_arrive(p, sh, b0 + BAR_XHAT);
      bar_wait(p, sh, b0 + BAR_XHAT);
    }

    // P0: router slices, then shared gate/up
    const int nrt = p->E * p->NSR;
    int tau = W;
    for (; tau < nrt; tau += NW) router_task<RD, SMALL>(p, lp, L, tau / p->NSR, tau % p->NSR);
    if constexpr (SMALL) bar_arrive_published(p, sh, b0 + BAR_ROUTER);
    else bar_arrive(p, sh, b0 + BAR_ROUTER);
    if (p->route_only) {
      bar_wait(p, sh, b0 + BAR_ROUTER);
      if (blockIdx.x == 0)
        for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, L, t, true);
      break;
    }
    for (; tau < nrt + p->Is * p->NSS; tau += NW)
      shared_gu_task<AD, SD, SMALL>(p, lp, L, (tau - nrt) / p->NSS, (tau - nrt) % p->NSS);
    if constexpr (SMALL) bar_arrive_published(p, sh, b0 + BAR_SHARED);
    else bar_arrive(p, sh, b0 + BAR_SHARED);

    // P1: routing, gather tables, expert gate/up
    if constexpr (SMALL) {
      route_small<true>(p, lp, L, b0 + BAR_ROUTER);
    } else {
      bar_wait(p, sh, b0 + BAR_ROUTER);
      for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, L, t, blockIdx.x == 0);
      __syncthreads();
      build_tables(p, L);
    }
    const int ntask = sh.nU * p->I;
    for (int q = W; q < ntask; q += NW) expert_gu_task<AD, ED, SMALL>(p, lp, L, q / p->I, q % p->I);
    if constexpr (SMALL) bar_arrive_published(p, sh, b0 + BAR_H);
    else bar_arrive(p, sh, b0 + BAR_H);

    // P2: this workgroup's output rows; the shared expert's rows first (their
    // input is complete since P0), which fills the wait for the expert barrier
    const int r0 = blockIdx.x * p->rows_per_wg;
    const int r1 = min(p->H, r0 + p->rows_per_wg);
    if constexpr (SMALL) {
      shared_h_small<AD>(p, L, b0 + BAR_SHARED);
      if (r0 < r1) shared_down_units<AD, SD, true>(p, lp, L, r0, r1, 0);
      bar_wait(p, sh, b0 + BAR_H);
      stage_h<AD>(p, L);
      __syncthreads();
      if (r0 < r1) expert_down_units<AD, ED, true>(p, lp, L, r0, r1, 0);
      __syncthreads();
      if (r0 < r1) combine<AD>(p, lp, L, r0, r1);
      __syncthreads();
    } else {
      const bool one_pass = p->pass_rows >= p->rows_per_wg;
      const int nsh = p->Is / p->I;
      bar_wait(p, sh, b0 + BAR_SHARED);
      if (one_pass && r0 < r1) shared_down_units<AD, SD, false>(p, lp, L, r0, r1, 0);
      bar_wait(p, sh, b0 + BAR_H);
      for (int pr0 = r0; pr0 < r1; pr0 += p->pass_rows) {
        const int pr1 = min(r1, pr0 + p->pass_rows);
        const int nrb = (pr1 - pr0) / kRowBlock;
        if (!one_pass) shared_down_units<AD, SD, false>(p, lp, L, pr0, pr1, 0);
        expert_down_units<AD, ED, false>(p, lp, L, pr0, pr1, one_pass ? 0 : nrb * nsh);
        __syncthreads();
        combine<AD>(p, lp, L, pr0, pr1);
        __syncthreads();
      }
    }

    if (l + 1 < p->L) {
      bar_arrive(p, sh, b0 + BAR_LAYER);
      sink ^= prefetch_p0<RD, SD>(p, &p->lp[l + 1], W, NW);
      bar_wait(p, sh, b0 + BAR_LAYER);
    }
  }
  if (sink == 0x9E3779B9u) sh.sink = sink;  // keeps the prefetch loads; practically never taken

  // last workgroup out resets the counters for the next launch on this workspace
  __syncthreads();
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(ctrl_word(p, CTRL_DONE), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (unsigned)p->G - 1u) {
      for (int b = 0; b < kBarPerLayer * p->L; ++b)
        __hip_atomic_store(ctrl_word(p, CTRL_BAR + b), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctrl_word(p, CTRL_DONE), 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// host runtime

thread_local char g_err[512] = "no error";

moe_status fail(moe_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

struct DevInfo {
  int cus = 0;
  int max_lds = 0;
};

DevInfo g_dev[64];

moe_status device_info(DevInfo &out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "hipGetDevice failed");
  if (g_dev[dev].cus == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed");
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 65536;
    g_dev[dev].max_lds = lds;
    g_dev[dev].cus = prop.multiProcessorCount;
  }
  out = g_dev[dev];
  return MOE_OK;
}

bool aligned16(const void *q) { return ((uintptr_t)q & 15u) == 0; }

int dsize(moe_dtype d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

moe_status check_desc(const moe_layer_desc *d) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->expert_inter <= 0 || d->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "non-positive size in desc");
  if (!(d->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARGUMENT, "rms_eps must be >= 0");
  if (d->hidden % 256 || d->hidden > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: need a multiple of 256, at most 16384", d->hidden);
  if (d->expert_inter % 128 || d->expert_inter > 4096)
    return fail(MOE_ERR_UNSUPPORTED, "expert_inter=%d: need a multiple of 128, at most 4096", d->expert_inter);
  if (d->shared_inter % d->expert_inter || d->shared_inter > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "shared_inter=%d: need 0 or a multiple of expert_inter, at most 8192",
                d->shared_inter);
  if (d->top_k > kMaxK || d->top_k > d->num_experts || d->num_experts > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "top_k=%d num_experts=%d: need 1<=k<=32, k<=E<=1024", d->top_k, d->num_experts);
  const bool f32set = d->act == MOE_F32 && d->router == MOE_F32 && d->expert == MOE_F32 && d->shared == MOE_F32;
  const bool bfset = d->act == MOE_BF16 && (d->router == MOE_F32 || d->router == MOE_BF16) &&
                     (d->expert == MOE_BF16 || d->expert == MOE_FP8_E4M3) && d->shared == MOE_BF16;
  if (!f32set && !bfset) return fail(MOE_ERR_UNSUPPORTED, "unsupported dtype combination");
  if (d->expert == MOE_FP8_E4M3 && d->scale_group != 128)
    return fail(MOE_ERR_UNSUPPORTED, "fp8 experts need scale_group 128");
  return MOE_OK;
}

// K-slices of a row of `hidden` elements of dtype dt: the most (of `most`,
// halving) that keep whole 64-lane chunks per slice and about 4 KB or more.
int k_slices(int hidden, moe_dtype dt, int most) {
  const int chunk = 64 * (16 / dsize(dt));
  for (int ns = most; ns > 1; ns /= 2)
    if ((hidden / ns) % chunk == 0 && (size_t)hidden * dsize(dt) / ns >= 4096) return ns;
  return 1;
}

bool small_regime(int B) { return B <= kSmallB; }

struct WsLayout {
  size_t xhat, xa, rpart, hspart, hbuf, hsbuf, xbuf0, xbuf1, total;
};

size_t up256(size_t v) { return (v + 255u) & ~(size_t)255u; }

WsLayout ws_layout(const moe_layer_desc *d, int B, int L) {
  WsLayout w{};
  size_t off = up256(kCtrlBytes);
  const size_t act = (size_t)dsize(d->act);
  const size_t is = (size_t)(d->shared_inter > 0 ? d->shared_inter : 1);
  w.xhat = off; off += up256((size_t)B * d->hidden * 4);
  w.xa = off; off += up256((size_t)B * d->hidden * act);
  w.rpart = off; off += up256((size_t)B * d->num_experts * 4 * 4);
  w.hspart = off; off += up256((size_t)2 * B * 2 * is * 4);
  w.hbuf = off; off += up256((size_t)B * d->top_k * d->expert_inter * 4);  // fp32 in the small regime
  w.hsbuf = off; off += up256((size_t)B * is * act);
  w.xbuf0 = off; off += (L > 1) ? up256((size_t)B * d->hidden * act) : 0;
  w.xbuf1 = off; off += (L > 2) ? up256((size_t)B * d->hidden * act) : 0;
  w.total = off;
  return w;
}

typedef void (*kernel_fn)(Params);

template <bool S>
kernel_fn pick_kernel_t(const moe_layer_desc *d) {
  if (d->act == MOE_F32) return moe_kernel<DT_F32, DT_F32, DT_F32, DT_F32, S>;
  if (d->expert == MOE_BF16)
    return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_BF16, DT_BF16, S>
                                : moe_kernel<DT_BF16, DT_BF16, DT_BF16, DT_BF16, S>;
  return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_FP8, DT_BF16, S>
                              : moe_kernel<DT_BF16, DT_BF16, DT_FP8, DT_BF16, S>;
}

kernel_fn pick_kernel(const moe_layer_desc *d, bool small) {
  return small ? pick_kernel_t<true>(d) : pick_kernel_t<false>(d);
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

moe_status check_weights(const moe_layer_desc *d, const moe_layer_weights *w) {
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  const void *req[] = {w->rms_gamma, w->router_w, w->expert_gate_up, w->expert_down};
  for (const void *q : req)
    if (!q) return fail(MOE_ERR_INVALID_ARGUMENT, "a required weight pointer is NULL");
  if (d->shared_inter > 0 && (!w->shared_gate_up || !w->shared_down))
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert weights are NULL but shared_inter > 0");
  if (d->expert == MOE_FP8_E4M3 && (!w->expert_gate_up_scale || !w->expert_down_scale))
    return fail(MOE_ERR_INVALID_ARGUMENT, "fp8 experts need both scale arrays");
  const void *all[] = {w->rms_gamma, w->router_w, w->router_bias, w->expert_gate_up, w->expert_down,
                       w->expert_gate_up_scale, w->expert_down_scale, w->shared_gate_up, w->shared_down};
  for (const void *q : all)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARGUMENT, "weight pointer %p is not 16-byte aligned", q);
  return MOE_OK;
}

size_t align16(size_t v) { return (v + 15u) & ~(size_t)15u; }

moe_status launch(const moe_layer_desc *d, const moe_layer_weights *layers, int L, const void *x, void *y, int B,
                  int32_t *idx, float *wts, float *logits, void *ws, size_t ws_bytes, void *stream, bool route_only) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (B < 1 || B > kMaxB) return fail(MOE_ERR_UNSUPPORTED, "batch %d outside 1..64", B);
  if (L < 1 || L > kMaxL) return fail(MOE_ERR_UNSUPPORTED, "layers %d outside 1..8", L);
  if (!layers) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  for (int l = 0; l < L; ++l)
    if ((st = check_weights(d, &layers[l])) != MOE_OK) return st;
  if (!x || !ws || (!route_only && !y)) return fail(MOE_ERR_INVALID_ARGUMENT, "x, y or workspace is NULL");
  if (route_only && (!idx || !wts)) return fail(MOE_ERR_INVALID_ARGUMENT, "topk_idx or topk_w is NULL");
  const void *ptrs[] = {x, y, idx, wts, logits, ws};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer %p is not 16-byte aligned", q);
  const size_t xbytes = (size_t)B * d->hidden * dsize(d->act);
  if (y && y != x && overlap(x, xbytes, y, xbytes)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and y partially overlap");
  const WsLayout wl = ws_layout(d, B, L);
  if (ws_bytes < wl.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  if (overlap(ws, wl.total, x, xbytes) || (y && overlap(ws, wl.total, y, xbytes)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace overlaps x or y");

  DevInfo di;
  if ((st = device_info(di)) != MOE_OK) return st;
  Params p;
  memset(&p, 0, sizeof p);
  p.H = d->hidden; p.E = d->num_experts; p.k = d->top_k; p.I = d->expert_inter; p.Is = d->shared_inter;
  p.B = B; p.L = L; p.route_only = route_only ? 1 : 0; p.eps = d->rms_eps;
  p.G = di.cus;
  if (p.G < 1) return fail(MOE_ERR_DEVICE, "device reports no compute units");
  const bool small = small_regime(B);
  p.NSR = k_slices(d->hidden, d->router, 4);
  p.NSS = small && d->shared_inter > 0 ? k_slices(d->hidden, d->shared, 2) : 1;
  int rpw = (p.H + p.G - 1) / p.G;
  rpw = (rpw + kRowBlock - 1) / kRowBlock * kRowBlock;
  p.rows_per_wg = rpw;

  // LDS carve-up
  const int E = d->num_experts, P = B * d->top_k, H = d->hidden;
  const int nsh = d->shared_inter > 0 ? d->shared_inter / d->expert_inter : 0;
  const int nslot = P < E ? P : E;
  const size_t act = (size_t)dsize(d->act);
  size_t o = align16(sizeof(SmemHead));
  p.o_sel_idx = (int)o; o = align16(o + (size_t)P * 4);
  p.o_sel_w = (int)o; o = align16(o + (size_t)P * 4);
  p.o_ulist = (int)o; o = align16(o + (size_t)nslot * 4);
  p.o_ucnt = (int)o; o = align16(o + (size_t)nslot * 4);
  p.o_ustart = (int)o; o = align16(o + (size_t)nslot * 4);
  p.o_plist = (int)o; o = align16(o + (size_t)P * 4);
  if (small) {
    if (P > 64) return fail(MOE_ERR_UNSUPPORTED, "small-batch routing needs batch*top_k <= 64");
    p.o_xf = (int)o; o = align16(o + (size_t)B * H * 4);
    p.o_xa = (int)o; o = align16(o + (d->act == MOE_F32 ? 0 : (size_t)B * H * act));
    p.o_hs = (int)o; o = align16(o + (size_t)B * (d->shared_inter > 0 ? d->shared_inter : 1) * act);
    // expert h lands over x-hat once every P1 task is done (after the expert
    // barrier), or after the other regions when it is the larger of the two
    const size_t hbytes = (size_t)P * d->expert_inter * act;
    if ((size_t)p.o_xf + hbytes <= (size_t)p.o_hs) {
      p.o_h = p.o_xf;
    } else {
      p.o_h = (int)o; o = align16(o + hbytes);
    }
  } else {
    p.o_cnt = (int)o; o = align16(o + (size_t)E * 4);
    p.o_start = (int)o; o = align16(o + (size_t)E * 4);
    p.o_tmask = (int)o; o = align16(o + (size_t)E * 8);
  }
  p.o_part = (int)o;
  const size_t per_row = (size_t)(P + B * nsh) * sizeof(float);
  const size_t lds_cap = (size_t)(di.max_lds > 0 ? di.max_lds : 65536);
  if (o + (size_t)kRowBlock * per_row > lds_cap)
    return fail(MOE_ERR_UNSUPPORTED, "shape needs more LDS than the device's %zu bytes", lds_cap);
  int pr = (int)((lds_cap - o) / per_row);
  pr = pr / kRowBlock * kRowBlock;
  p.pass_rows = pr < rpw ? pr : rpw;
  if (small && p.pass_rows < rpw)
    return fail(MOE_ERR_UNSUPPORTED, "small-batch layout needs one LDS pass over %d rows", rpw);
  const size_t lds = o + (size_t)p.pass_rows * per_row;

  p.timeout_ticks = 200000000LL;  // 2 s at 100 MHz
  // test hook: a tiny limit makes every barrier wait give up at once (no hang, no fault)
  if (const char *ev = getenv("MOE_DEBUG_BARRIER_TIMEOUT_TICKS")) p.timeout_ticks = atoll(ev);
  unsigned char *wsb = (unsigned char *)ws;
  p.ctrl = (unsigned *)wsb;
  p.xhat = (float *)(wsb + wl.xhat);
  p.xa = (d->act == MOE_F32) ? (void *)p.xhat : (void *)(wsb + wl.xa);
  p.rpart = (float *)(wsb + wl.rpart);
  p.hspart = (float *)(wsb + wl.hspart);
  p.hbuf = wsb + wl.hbuf;
  p.hsbuf = wsb + wl.hsbuf;
  p.xbuf[0] = wsb + wl.xbuf0;
  p.xbuf[1] = wsb + wl.xbuf1;
  for (int l = 0; l < L; ++l) {
    LayerPtrs &lp = p.lp[l];
    const moe_layer_weights &w = layers[l];
    lp.x = (l == 0) ? x : p.xbuf[(l - 1) & 1];
    lp.y = (l == L - 1) ? y : p.xbuf[l & 1];
    lp.gamma = w.rms_gamma; lp.rw = w.router_w; lp.rb = w.router_bias;
    lp.egu = w.expert_gate_up; lp.ed = w.expert_down;
    lp.egus = w.expert_gate_up_scale; lp.eds = w.expert_down_scale;
    lp.sgu = w.shared_gate_up; lp.sd = w.shared_down;
    lp.idx_out = idx ? idx + (size_t)l * B * d->top_k : nullptr;
    lp.w_out = wts ? wts + (size_t)l * B * d->top_k : nullptr;
    lp.logits_out = logits;
  }
  kernel_fn fn = pick_kernel(d, small);
  if (hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return fail(MOE_ERR_DEVICE, "hipFuncSetAttribute(%zu bytes of LDS) failed", lds);
  // the grid is persistent: one resident workgroup per CU is required
  int resident = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, (const void *)fn, kThreads, lds) != hipSuccess ||
      resident < 1)
    return fail(MOE_ERR_DEVICE, "a %d-thread workgroup with %zu bytes of LDS cannot be resident", kThreads, lds);
  hipLaunchKernelGGL(fn, dim3(p.G), dim3(kThreads), lds, (hipStream_t)stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens, int32_t num_layers) {
  if (check_desc(desc) != MOE_OK) return 0;
  if (max_tokens < 1 || max_tokens > kMaxB || num_layers < 1 || num_layers > kMaxL) return 0;
  return ws_layout(desc, max_tokens, num_layers).total;
}

moe_status moe_route(const moe_layer_desc *desc, const moe_layer_weights *weights, const void *x, int32_t B,
                     int32_t *topk_idx, float *topk_w, float *logits, void *ws, size_t ws_bytes, void *stream) {
  return launch(desc, weights, 1, x, nullptr, B, topk_idx, topk_w, logits, ws, ws_bytes, stream, true);
}

moe_status moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *weights, const void *x, void *y,
                            int32_t B, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  return launch(desc, weights, 1, x, y, B, topk_idx, topk_w, nullptr, ws, ws_bytes, stream, false);
}

moe_status moe_decode_stack(const moe_layer_desc *desc, const moe_layer_weights *layers, int32_t L, const void *x,
                            void *y, int32_t B, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                            void *stream) {
  return launch(desc, layers, L, x, y, B, topk_idx, topk_w, nullptr, ws, ws_bytes, stream, false);
}

moe_status moe_check_workspace(void *ws, size_t ws_bytes, void *stream) {
  if (!ws || ws_bytes < kCtrlBytes) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL or too small");
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return fail(MOE_ERR_DEVICE, "stream sync failed");
  unsigned err = 0;
  unsigned char *word = (unsigned char *)ws + (size_t)CTRL_ERR * kCtrlStride * sizeof(unsigned);
  if (hipMemcpy(&err, word, sizeof err, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MOE_ERR_DEVICE, "reading the error word failed");
  if (err) {
    const unsigned zero = 0;
    if (hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "clearing the error word failed");
    return fail(MOE_ERR_TIMEOUT, "a launch on this workspace stopped at its barrier watchdog");
  }
  return MOE_OK;
}

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    case MOE_ERR_TIMEOUT: return "MOE_ERR_TIMEOUT";
  }
  return "unknown moe_status";
}

const char *moe_last_error(void) { return g_err; }

}  // extern "C"
