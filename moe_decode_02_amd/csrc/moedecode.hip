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
//           (partial logits, summed in a fixed order), then the shared
//           expert's gate/up rows, which do not depend on routing; the pages
//           run the shared expert on its own stream beside routing (smzdm.com
//           post, section "what changed", MoE de-duplication item). From 8
//           tokens both run on MFMA tiles instead.
//   routing Softmax + top-k + renormalisation and the expert gather tables
//           (union of selected experts, each expert's token list) in LDS.
//           At B <= 2 one spare wave per workgroup polls the published logits
//           (no router barrier) while the others stream shared rows; at
//           larger B every workgroup routes the batch after a router barrier.
//   P1      The selected experts' gate/up rows, h = SiLU(g) * u: GEMV rows,
//           or MFMA tiles for experts that several tokens select. The work
//           falls into groups, each closed by its own barrier.
//   P2      Each workgroup owns a block of output rows. It reduces the shared
//           expert's down rows first (their input is ready since P0), then
//           each group's routed down rows once that group's barrier has
//           passed, overlapping later gate/up work, then combines in a fixed
//           order with the routing weights and the residual.
//   stack   Between layers one more barrier (published: the combine writes
//           the next layer's input with device-coherent stores).
//
// Weight rows stream through 16-byte non-temporal loads, whole chunks of 64
// lanes with no per-lane guard, all loads of a step in flight before the
// first use; fp8 codes become bf16 through the hardware conversion and meet
// the bf16 activations in dot2 instructions. Cross-lane sums and the top-k
// argmax use DPP row operations. All reductions are fixed-order (no float
// atomics), so identical router rows give bit-identical logits and repeated
// runs give identical outputs.
//
// Memory ordering across the 8 XCDs: every value one workgroup writes for
// others (x-hat, logits, shared and expert h, the next layer's x) goes out
// through device-coherent stores, written through past the XCD's L2. A wave
// arriving at a barrier waits for its own stores to complete and counts
// itself in LDS; the workgroup's last wave adds one to the barrier's global
// counter, with no L2 write-back. One wave per workgroup polls the counter,
// acquires at agent scope and raises an LDS flag for the others. Weights are static and may be loaded before a barrier;
// activations are read only after it (a compiler that hoisted an activation
// load above a sync wait was one of the bugs found in the pages' review:
// aiposthub.com article, section on how vLLM verifies AI-written kernels).
//
// The end of the file holds the multi-launch path (moe_decode_layer_unfused):
// the same layer as eleven kernel launches, the measured baseline of the fusion.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moedecode.h"
#ifdef MOE_DEBUG_DELAY
#include "moedecode_debug.h"
#endif

// The library's own workspace for moe_decode_layer_static (callers that
// cannot allocate device memory): every GPU the library runs on holds one copy
// until the process ends. Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

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
constexpr int kSmallB = 4;      // B <= kSmallB (and B * k <= 64): the small regime (x-hat in every workgroup's LDS)
constexpr int kMaxRounds = 32;  // rounds of P0 slices over the grid's waves

// expert barriers of the small regime: P1's rounds fall into up to kP1Groups
// groups, each with a barrier, so the down projections of the experts done in
// early groups run while later groups are still being computed
#ifndef MOE_P1_GROUPS
#define MOE_P1_GROUPS 4
#endif
constexpr int kP1Groups = MOE_P1_GROUPS;
enum : int { BAR_XHAT = 0, BAR_ROUTER = 1, BAR_SHARED = 2, BAR_LAYER = 3, BAR_H = 4, kBarPerLayer = 4 + kP1Groups };
constexpr int kMaxBarriers = kBarPerLayer * kMaxL;
constexpr int kCtrlStride = 16;  // words: each control word on its own 64-byte line
// router MFMA tiles (16 experts each) whose K range is split over workgroups:
// one arrival counter per tile, after the barrier counters
constexpr int kMaxRTiles = kMaxE / 16;
constexpr int kMaxRQ = 8;        // most K parts of a router tile
constexpr int kMaxStealG = 512;  // general regime: workgroups whose P1 tail others may take (larger grids: none)
enum : int {
  CTRL_DONE = 0,
  CTRL_ERR = 1,
  CTRL_BAR = 2,
  CTRL_RTILE = CTRL_BAR + kMaxBarriers,
  CTRL_P1 = CTRL_RTILE + kMaxRTiles,  // [workgroup][P1 group]: tasks taken from the shared tail of its share
};
constexpr size_t kCtrlBytes = (size_t)(CTRL_P1 + kMaxStealG * kP1Groups) * kCtrlStride * sizeof(unsigned);
// small-regime logit buffers (two layer parities), right after the control words
constexpr size_t kRlogOffset = (kCtrlBytes + 255u) & ~(size_t)255u;
constexpr size_t kRlogBytes = (size_t)2 * kSmallB * kMaxE * sizeof(float);

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
  float *lg;              // [B][E] router logits of this layer (see Params::rfin, Params::rlog)
};

struct Params {
  int H, E, k, I, Is, B, L;
  int nsh;                // shared down: column blocks of width <= I (ceil(Is / I)), each a partial-sum column
  int route_only;
  int mfma_min;           // general regime: experts with >= mfma_min tokens go through MFMA tiles (0: none)
  int mfma_sh;            // general regime: the router and the shared expert go through MFMA tiles
  int rq;                 // K parts of each router MFMA tile, one workgroup each
  int steal;              // general regime: P1 share tails taken through CTRL_P1 counters
  int tail_div;           // general regime: 1 / tail_div of each workgroup's P1 share is its stealable tail
  int p1_groups;          // general regime: P1 groups (each closed by a barrier), at most kP1Groups
  int p0_end;             // P0 task indices in [0, p0_end): router slices, then shared slices (VALU)
  int NSR;                // router K-slices
  int NSS;                // shared gate/up K-slices
  int s0;                 // first P0 task index of the shared slices (a multiple of the wave count of a workgroup)
  int slw;                // floats per wave and round in the LDS slice slots (B, or 2B with shared slices)
  int p0r, p0w;           // P0 rounds; waves per workgroup that take a task in the last round
  int G;                  // workgroups
  int rows_per_wg;        // P2 output rows per workgroup (multiple of kRowBlock)
  float eps;
  long long timeout_ticks;  // s_memrealtime ticks (100 MHz) before a barrier wait gives up
  // ordering-stress build only (MOE_DEBUG_DELAY): seed of the injected delays,
  // and the workgroup -> work permutation g -> (perm_a * g + perm_c) mod G
  unsigned long long dbg_seed;
  int perm_a, perm_c;
  int self_reset;         // the workspace is the library's static array: the launch also clears a watchdog stop's state
  unsigned *ctrl;         // control words, kCtrlStride apart
  float *xhat;            // [B][H] fp32 (general regime)
  void *xa;               // [B][H] act (general regime; == xhat for fp32 activations)
  float *rfin;            // [B][E]: the logits, general regime and route mode
  float *rlog;            // [2][kSmallB][E]: small-regime logits by layer parity, all-zero bits while
                          // unwritten (a written logit is never +0: +0 is stored as -0)
  float *hsh32;           // [B][Is]: the shared h, act-rounded, as fp32 (small regime)
  void *hbuf;             // [B*k][I] act
  void *hsbuf;             // [B][Is] act (general regime)
  float *partbuf;          // [pstride][H] P2 partial sums (general regime), column-major
  float *rpart;            // [rq][B][E] router partial logits of the K parts of the MFMA tiles
  void *xbuf[2];          // [B][H] act, stack intermediates
  // LDS carve-up, byte offsets from the start of dynamic LDS
  int o_sel_idx, o_sel_w;           // routing of each token [B*k]
  int o_ulist, o_ucnt, o_ustart;    // gather tables per union slot [min(E, B*k)]
  int o_plist;                      // (token, rank) pairs grouped by expert [B*k]
  int o_cnt, o_start, o_tmask;      // per-expert scratch of the workgroup-wide table build [E]
  int o_mslot, o_gslot;             // general regime: union slots on MFMA tiles / on GEMV [min(E, B*k)]
  int o_cpre;                       // general regime: P1 cost before each listed slot [min(E, B*k) + 1]
  int o_xf, o_xa;                   // small regime: x-hat fp32 [B][H] (fp32 activations) / act [B][H]
  int o_x, o_g;                     // small regime, bf16 activations: x [B][H] and gamma [H] as given
  int rx32;                         // small regime: the router's fp32 x-hat [B][H] is in LDS (o_xf); else formed from o_x, o_g
  int o_cand;                       // top-k candidates, then the ranked k: [slots][2 * 64] keys, then indices
  int o_hs;                         // small regime: shared h [B][Is] (act)
  int o_slc;                        // slice sums of P0 tasks [round][wave][slw]
  int o_scnt;                       // slices of a router row / shared pair done: [2][round][slice group] int
  int o_part;                       // small regime: P2 partial sums [rows_per_wg][pstride] fp32
  int o_red;                        // shared MFMA tiles: partial tiles of the waves [kWaves][16][B] fp32
  LayerPtrs lp[kMaxL];
};

// fixed head of the dynamic LDS
struct SmemHead {
  int bar_cnt[kMaxBarriers];    // waves of this workgroup that arrived
  int bar_claim[kMaxBarriers];  // one wave polls the global counter
  int bar_flag[kMaxBarriers];   // raised once the barrier is passed
  float red[kWaves * kSmallB];
  float rstd[kSmallB];             // small regime, bf16 activations: 1 / sqrt(mean(x^2) + eps) of each token
  int scan_tmp[2 * kWaves];
  int nU;
  int route_claim, route_ready;    // small regime: the first free wave does the routing
  int shared_claim, shared_ready;  // small regime: ... and the shared expert's h
  int unit_ctr[2 + kP1Groups];     // P2 units handed out to waves (shared, experts / expert group)
  int p1_ctr[kP1Groups];           // general regime: P1 tasks of the workgroup's share handed out, per group
  int nM, nG;                      // general regime: union slots on MFMA tiles, on GEMV
  int expired;                     // a wait of this workgroup gave up at its watchdog during this launch
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

// 8 e4m3 codes (two words) -> 8 bf16 (exact: e4m3 values are bf16 values)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  u32x4 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
  r.z = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
  r.w = __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
  return r;
}

// 16 e4m3 codes against 16 bf16 activations: the codes become bf16 pairs
// through the hardware conversion (exact), then bf16 dot2 as for bf16 weights
// (a software decode costs ~6 VALU operations per code, which made the fp8
// GEMV ALU-bound well below the HBM rate).
template <> struct Chunk<DT_FP8, DT_BF16> {
  static constexpr int NX = 2;
  __device__ static __forceinline__ float dot(const u32x4 &w, const u32x4 *x, float a) {
    const u32x4 lo = fp8x8_to_bf16(w.x, w.y), hi = fp8x8_to_bf16(w.z, w.w);
    a = dot2_bf16(lo.x, x[0].x, a);
    a = dot2_bf16(lo.y, x[0].y, a);
    a = dot2_bf16(lo.z, x[0].z, a);
    a = dot2_bf16(lo.w, x[0].w, a);
    a = dot2_bf16(hi.x, x[1].x, a);
    a = dot2_bf16(hi.y, x[1].y, a);
    a = dot2_bf16(hi.z, x[1].z, a);
    a = dot2_bf16(hi.w, x[1].w, a);
    return a;
  }
};

// A bf16 scale of fp8 weights is loaded when a task starts and applied when
// it ends. It stays a raw word until late_scale(), whose empty asm keeps the
// conversion, and with it the wait for the load, after the task's weight
// loads; converted at once, each scale load cost a full memory round trip
// before the first weight load was issued.
__device__ __forceinline__ float late_scale(uint32_t raw) {
  asm volatile("" : "+v"(raw));
  return __uint_as_float(raw << 16);
}

// weight chunk: streamed once, so loaded non-temporal
__device__ __forceinline__ u32x4 ldw(const char *p) { return __builtin_nontemporal_load((const u32x4 *)p); }

// activation chunk, from global memory (XS = 0), LDS (XS = 1), or, for the
// router in the small regime with bf16 activations, the fp32 x-hat formed
// from the token's bf16 x, bf16 gamma (both in LDS) and its fp32 r (XS = 2)
template <int XS> struct XSrc;
template <> struct XSrc<0> {
  typedef const char *ptr;
  __device__ static __forceinline__ u32x4 ld(ptr p, size_t off) { return *(const u32x4 *)(p + off); }
};
template <> struct XSrc<1> {
  typedef const lds_t *ptr;
  __device__ static __forceinline__ u32x4 ld(ptr p, size_t off) {
    return *(const __attribute__((address_space(3))) u32x4 *)(p + off);
  }
};
template <> struct XSrc<2> {
  struct ptr {
    const lds_t *x, *g;  // the token's row of x, and gamma, bf16
    float r;
  };
  // off: byte offset into an fp32 row; 4 elements, each (x * r) * gamma as
  // the normalisation computes it, so the router sees the same bits
  __device__ static __forceinline__ u32x4 ld(const ptr &p, size_t off) {
    const size_t b = off >> 1;
    const u32x2 xv = *(const __attribute__((address_space(3))) u32x2 *)(p.x + b);
    const u32x2 gv = *(const __attribute__((address_space(3))) u32x2 *)(p.g + b);
    u32x4 v;
    v.x = __float_as_uint(__uint_as_float(xv.x << 16) * p.r * __uint_as_float(gv.x << 16));
    v.y = __float_as_uint(__uint_as_float(xv.x & 0xFFFF0000u) * p.r * __uint_as_float(gv.x & 0xFFFF0000u));
    v.z = __float_as_uint(__uint_as_float(xv.y << 16) * p.r * __uint_as_float(gv.y << 16));
    v.w = __float_as_uint(__uint_as_float(xv.y & 0xFFFF0000u) * p.r * __uint_as_float(gv.y & 0xFFFF0000u));
    return v;
  }
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }
// The lane index computed where it is used (volatile, so the compiler neither
// hoists nor merges it): after a long MFMA loop a lane-derived value kept
// from before the loop can be spilled, and each reload's wait then also
// waits for every store in flight.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The work of "workgroup g" (every share of tasks, rows and tiles is keyed
// by it). The ordering-stress build maps the hardware workgroups onto these
// shares through a seeded permutation, so that which CU, XCD and launch
// position takes which share changes between runs; results must not.
__device__ __forceinline__ int wg_id(KParams p) {
#ifdef MOE_DEBUG_DELAY
  return (int)(((long long)p->perm_a * blockIdx.x + p->perm_c) % p->G);
#else
  (void)p;
  return (int)blockIdx.x;
#endif
}

// Ordering-stress build: a seeded pause of up to ~55 us for about one call in
// four, keyed by (seed, workgroup, wave, site, arg), before barrier arrivals,
// published logits, expert tasks, output units, routing and the combine.
// Every result must be bit-identical to the undelayed run. Other builds: no code.
enum : int { DLY_START = 0, DLY_ARRIVE, DLY_PUBLISH, DLY_P1, DLY_P2, DLY_COMBINE, DLY_ROUTE, DLY_STAGE, DLY_CLEAR };
__device__ __forceinline__ void dbg_delay(KParams p, int site, int arg) {
#ifdef MOE_DEBUG_DELAY
  if (p->dbg_seed == 0) return;
  unsigned long long z = p->dbg_seed ^ ((unsigned long long)site << 56) ^ ((unsigned long long)wg_id(p) << 40) ^
                         ((unsigned long long)wave_id() << 32) ^ (unsigned)arg;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;  // SplitMix64 output function (Steele, Lea, Flood)
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  if ((z & 3u) == 0) {
    const int n = 1 + (int)((z >> 8) & 15u);
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
  }
#else
  (void)p; (void)site; (void)arg;
#endif
}

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
constexpr int DPP_ROW_ROR8 = 0x128;    // row_ror:8 (lane s of a 16-lane row reads lane (s + 8) % 16)

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

template <int WD, int XD, int XL, int NR, int SEG, int TG>
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
// General regime (B > 4): chunks per step of a gate/up pair and of a down
// pass. Its x-hat rows come from L2, not LDS, so a step waits longer.
#ifndef MOE_GEN_GU_SEG
#define MOE_GEN_GU_SEG 1
#endif
#ifndef MOE_GEN_DOWN_SEG
#define MOE_GEN_DOWN_SEG 1
#endif
#ifndef MOE_GEN_DOWN_ROWS_FP8
#define MOE_GEN_DOWN_ROWS_FP8 4  // fp8 down units: rows per pass (all 4: one 4 KB step)
#endif
template <int WD, int TG, bool XL> constexpr int seg_gu_r() { return XL ? seg_gu<WD, TG>() : MOE_GEN_GU_SEG; }
template <int WD, int TG, bool XL> constexpr int seg_down_r() { return XL ? seg_down<WD, TG>() : MOE_GEN_DOWN_SEG; }
// P0 (router and shared gate/up slices): loads per step
#ifndef MOE_P0_LOADS_PER_STEP
#define MOE_P0_LOADS_PER_STEP MOE_LOADS_PER_STEP
#endif
constexpr int kP0LoadsPerStep = MOE_P0_LOADS_PER_STEP;
// chunks per step of a router row slice, of a shared gate/up pair's slice
template <int WD, int TG> constexpr int seg_router() { return kP0LoadsPerStep; }
template <int WD, int TG> constexpr int seg_p0gu() { return kP0LoadsPerStep >= 4 ? kP0LoadsPerStep / 2 : 1; }

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

// Values other workgroups read after a barrier are written with
// device-coherent stores (write-through past this XCD's L2), so no barrier
// needs an L2 write-back, which costs several microseconds per workgroup
// while the memory system is streaming (a workgroup's last wave wrote back
// 5-12 us after its router unit at 8 tokens, when the general regime still
// used it).
// +0 as -0 (equal in every comparison and product), so that all-zero bits
// can mark a value not yet written
__device__ __forceinline__ float nonzero_bits(float v) { return __float_as_uint(v) == 0u ? -0.0f : v; }

__device__ __forceinline__ void publish(float *q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// element i of an act-dtype array, published
template <int D> __device__ __forceinline__ void publish_act(void *p, size_t i, float v) {
  if constexpr (D == DT_F32) __hip_atomic_store((float *)p + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else __hip_atomic_store((uint16_t *)p + i, f32_to_bf16(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wave is done with the work barrier b waits for, and every value it wrote
// for other workgroups went out through publish(): waiting for its stores to
// complete (they are then visible device-wide) replaces the L2 write-back.
// Readers still acquire at agent scope (L1/L2 invalidate) before reading.
__device__ void bar_arrive_published(KParams p, SmemHead &sh, int b) {
  dbg_delay(p, DLY_ARRIVE, b);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane_id() == 0) {
    const int old = __hip_atomic_fetch_add(&sh.bar_cnt[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (old == kWaves - 1)
      __hip_atomic_fetch_add(ctrl_word(p, CTRL_BAR + b), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            __hip_atomic_store(&sh.expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&sh.bar_flag[b], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        while (__hip_atomic_load(&sh.bar_flag[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          __builtin_amdgcn_s_sleep(1);
          if (rt_now() - t0 > 2 * p->timeout_ticks) {
            __hip_atomic_store(&sh.expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
          }
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// The workspace's error word, read device-coherently. A wait that gave up
// stores it before its workgroup arrives at any later barrier (every wave's
// arrival first waits for its own stores), so a workgroup that passed a later
// barrier and then reads it sees every expiry that preceded that barrier.
__device__ __forceinline__ unsigned err_word(KParams p) {
  return __hip_atomic_load(ctrl_word(p, CTRL_ERR), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// LDS views

// The kernel's dynamic LDS. Every region is addressed from this symbol, never
// from a pointer held in memory, so the compiler sees LDS accesses (ds_*
// instructions) in every function, inlined or not, and no function reloads a
// base pointer from scratch memory.
extern __shared__ __align__(16) unsigned char smem_raw[];

struct Lds {
  __device__ SmemHead &head() const { return *reinterpret_cast<SmemHead *>(smem_raw); }
  template <class T> __device__ T *at(int off) const { return reinterpret_cast<T *>(smem_raw + off); }
  __device__ lds_t *raw(int off) const { return (lds_t *)(smem_raw + off); }
};

// Arguments of a non-inlined function arrive in vector registers even when
// they are uniform; re-reading them through lane 0 puts them back in scalar
// registers, so parameter reads are scalar loads and addresses built from
// them can use a scalar base (no memory round trip of vector loads first).
template <class T> __device__ __forceinline__ T uni(T v) {
  if constexpr (sizeof(T) == 8) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (T)(((unsigned long long)hi << 32) | lo);
  } else {
    return (T)__builtin_amdgcn_readfirstlane((int)v);
  }
}

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
// every load is issued before the first use (one round trip). Chunk c of a
// row is handled by thread c mod 1024; out(i, ch, xv, gv, r) receives token
// i's chunk ch of x and gamma (16 bytes each) and the token's
// r = 1 / sqrt(mean(x^2) + eps); x-hat is (x * r) * gamma, elementwise.
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
      if (ch < nch) out(i, ch, xv[i][c], gv[c], r);
    }
  }
  __syncthreads();
}

// x-hat values of one chunk: (x * r) * gamma
template <int AD>
__device__ __forceinline__ void xhat_chunk(const u32x4 &xv, const u32x4 &gv, float r, float (&v)[8]) {
  float f[8], g[8];
  act_chunk_vals<AD>(xv, f);
  act_chunk_vals<AD>(gv, g);
#pragma unroll
  for (int q = 0; q < 16 / dsz<AD>(); ++q) v[q] = f[q] * r * g[q];
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Small regime: this workgroup normalises every token into its own LDS. fp32
// activations: x-hat [B][H] (the router's and the FFNs' input). bf16: the
// FFNs' x-hat [B][H] in bf16, and either the router's fp32 x-hat [B][H]
// (rx32) or x [B][H] and gamma [H] as given with each token's r, from which
// the router forms its fp32 input (XSrc<2>). All loads are issued first; each
// raw x chunk goes straight to its x-hat slot in LDS, so no chunk stays in a
// register across the workgroup barrier, and after it each thread reads its
// own chunks back and normalises them in place.
template <int AD, int NT>
__device__ __forceinline__ void stage_tokens(KParams p, KLayer lp, const Lds &L) {
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  constexpr int EPC = 16 / dsz<AD>(), NC = act_chunks_max<AD>();
  constexpr int XSL = AD == DT_F32 ? 4 : 2;  // bytes per element of the x-hat slot
  SmemHead &sh = L.head();
  const int H = p->H, tid = threadIdx.x, nch = H / EPC;
  lds_t *slot = L.raw(AD == DT_F32 ? p->o_xf : p->o_xa);
  u32x4 xv[NT][NC], gv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + c * kThreads;
    const int cc = ch < nch ? ch : 0;
    gv[c] = *(const u32x4 *)((const char *)lp->gamma + (size_t)cc * 16);
#pragma unroll
    for (int i = 0; i < NT; ++i) xv[i][c] = *(const u32x4 *)((const char *)lp->x + ((size_t)i * nch + cc) * 16);
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = tid + c * kThreads;
      if (ch < nch) {
        float f[8];
        act_chunk_vals<AD>(xv[i][c], f);
#pragma unroll
        for (int q = 0; q < EPC; ++q) ss = fmaf(f[q], f[q], ss);
        *(lds_u32x4 *)(slot + ((size_t)i * H + (size_t)ch * EPC) * XSL) = xv[i][c];
      }
    }
    ss = readlane_f(wave_sum63(ss), 63);
    if (lane_id() == 0) sh.red[i * kWaves + wave_id()] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float tot = 0.f;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sh.red[i * kWaves + w2];
    const float r = 1.0f / sqrtf(tot / (float)H + p->eps);
    if constexpr (AD != DT_F32)
      if (tid == 0 && !p->rx32) sh.rstd[i] = r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = tid + c * kThreads;
      if (ch >= nch) continue;
      lds_u32x4 *sl = (lds_u32x4 *)(slot + ((size_t)i * H + (size_t)ch * EPC) * XSL);
      const u32x4 x = *sl;
      float v[8];
      xhat_chunk<AD>(x, gv[c], r, v);
      if constexpr (AD == DT_F32) {
        *sl = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
      } else {
        *sl = u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
        const size_t off = ((size_t)i * H + (size_t)ch * 8) * 2;
        if (p->rx32) {
          lds_u32x4 *xf = (lds_u32x4 *)(L.raw(p->o_xf) + off * 2);
          xf[0] = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
          xf[1] = u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
        } else {
          *(lds_u32x4 *)(L.raw(p->o_x) + off) = x;
          if (i == 0) *(lds_u32x4 *)(L.raw(p->o_g) + (size_t)ch * 16) = gv[c];
        }
      }
    }
  }
  __syncthreads();
}

// One or two tokens, and three or four, in separate non-inlined functions:
// the register footprint of the larger batches would otherwise make every
// call save and restore callee-saved registers through scratch memory.
template <int AD>
__device__ __attribute__((noinline)) void stage_xhat12(KParams p_arg, KLayer lp_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  if (p->B == 1) stage_tokens<AD, 1>(p, lp, L);
  else stage_tokens<AD, 2>(p, lp, L);
}
template <int AD>
__device__ __attribute__((noinline)) void stage_xhat34(KParams p_arg, KLayer lp_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  if (p->B == 3) stage_tokens<AD, 3>(p, lp, L);
  else stage_tokens<AD, 4>(p, lp, L);
}
template <int AD>
__device__ __forceinline__ void stage_xhat(KParams p, KLayer lp, const Lds &L) {
  if (p->B <= 2) stage_xhat12<AD>(p, lp, L);
  else stage_xhat34<AD>(p, lp, L);
}

// 16-byte device-coherent store (written through this XCD's L2, visible
// device-wide once complete), for values published before a barrier that
// needs no L2 write-back
__device__ __forceinline__ void publish16(void *q, const u32x4 &v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(q), "v"(v) : "memory");
}

// elements i .. i + 3 of an act-dtype array (i a multiple of 4), published
// with one store
template <int D> __device__ __forceinline__ void publish_act4(void *p, size_t i, const float (&v)[4]) {
  if constexpr (D == DT_F32) {
    publish16((float *)p + i, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
  } else {
    const u32x2 w = {(uint32_t)f32_to_bf16(v[0]) | (uint32_t)f32_to_bf16(v[1]) << 16,
                     (uint32_t)f32_to_bf16(v[2]) | (uint32_t)f32_to_bf16(v[3]) << 16};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"((uint16_t *)p + i), "v"(w) : "memory");
  }
}

// General regime: workgroup t normalises token t into global memory, fp32
// (the router's input) and in the act dtype (the FFNs'), published.
template <int AD>
__device__ __attribute__((noinline)) void produce_xhat(KParams p_arg, KLayer lp_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  const int H = p->H;
  constexpr int EPC = 16 / dsz<AD>();
  for (int t = wg_id(p); t < p->B; t += p->G) {
    const int tok[1] = {t};
    rmsnorm_rows<AD, 1>(p, lp, L.head(), tok, [&](int, int ch, const u32x4 &xv, const u32x4 &gv, float r) {
      float v[8];
      xhat_chunk<AD>(xv, gv, r, v);
      float *xf = p->xhat + (size_t)t * H + (size_t)ch * EPC;
      publish16(xf, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
      if constexpr (AD != DT_F32) {
        publish16(xf + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
        publish16((char *)p->xa + ((size_t)t * H + (size_t)ch * EPC) * 2,
                  u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])});
      }
    });
  }
}

// pointer to token t's row of the FFNs' x-hat (act dtype) in LDS or global memory
template <bool XL, int AD>
__device__ __forceinline__ typename XSrc<XL>::ptr xhat_row(KParams p, const Lds &L, int t) {
  constexpr int XB = dsz<AD>();
  if constexpr (XL) {
    const int off = AD == DT_F32 ? p->o_xf : p->o_xa;
    return L.raw(off) + (size_t)t * p->H * XB;
  } else {
    const char *base = AD == DT_F32 ? (const char *)p->xhat : (const char *)p->xa;
    return base + (size_t)t * p->H * XB;
  }
}

// the router's fp32 input: global x-hat (general regime), LDS x-hat (small
// regime, fp32 activations), or formed from LDS x, gamma and r (small regime,
// bf16 activations)
template <bool XL, int AD> constexpr int router_src() { return !XL ? 0 : AD == DT_F32 ? 1 : 2; }

template <bool XL, int AD>
__device__ __forceinline__ typename XSrc<router_src<XL, AD>()>::ptr router_row(KParams p, const Lds &L, int t) {
  constexpr int XS = router_src<XL, AD>();
  if constexpr (XS == 0) return (const char *)p->xhat + (size_t)t * p->H * 4;
  else if constexpr (XS == 1) return L.raw(p->o_xf) + (size_t)t * p->H * 4;
  else return typename XSrc<2>::ptr{L.raw(p->o_x) + (size_t)t * p->H * 2, L.raw(p->o_g), L.head().rstd[t]};
}

// ---------------------------------------------------------------------------
// P0: router slices and shared gate/up rows

// The K-slices of one router row (or shared gate/up pair) are P0 tasks of
// consecutive indices that waves of one workgroup handle in the same round
// (the slice count divides the workgroup's wave count and the first index is a
// multiple of it, so slice s is the group's wave s). Each wave leaves its
// slice sums in its LDS slot of the round; the wave that finishes the last
// slice of the group sums the slots in slice order (a fixed order: identical
// rows give identical logits) and writes the result for other workgroups.
__device__ __forceinline__ float *slice_slot(KParams p, const Lds &L, int round, int wave) {
  return L.at<float>(p->o_slc) + ((size_t)round * kWaves + wave) * p->slw;
}

// which = 0: router rows, 1: shared pairs
__device__ __forceinline__ bool last_slice(KParams p, const Lds &L, int which, int round, int NS) {
  if (NS == 1) return true;
  int *cnt = L.at<int>(p->o_scnt) + ((size_t)which * p->p0r + round) * kWaves;
  int old = 0;
  if (lane_id() == 0)
    old = __hip_atomic_fetch_add(&cnt[wave_id() / NS], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(old) == NS - 1;
}

// router task tau = (row e, slice s) of round `round`: slice sums of all
// tokens to this wave's LDS slot; the last slice's wave writes the logit rfin[t][e]
// (published in the small regime)
template <int AD, int RD, bool XL>
__device__ __forceinline__ void router_task(KParams p, KLayer lp, const Lds &L, int tau, int round);

// small regime, bf16 activations: the router reads the fp32 x-hat from LDS
// where it fits (XS = 1), else forms it from x, gamma and r (XS = 2)
template <int AD, int RD, bool XL>
__device__ __forceinline__ void router_task_any(KParams p, KLayer lp, const Lds &L, int tau, int round) {
  if constexpr (router_src<XL, AD>() == 2) {
    if (p->rx32) router_task<DT_F32, RD, XL>(p, lp, L, tau, round);
    else router_task<AD, RD, XL>(p, lp, L, tau, round);
  } else {
    router_task<AD, RD, XL>(p, lp, L, tau, round);
  }
}

template <int AD, int RD, bool XL>
__device__ __forceinline__ void router_task(KParams p, KLayer lp, const Lds &L, int tau, int round) {
  constexpr int XS = router_src<XL, AD>();
  const int H = p->H, E = p->E, B = p->B, NSR = p->NSR;
  const int e = tau / NSR, s = tau % NSR;
  const int Ks = H / NSR;
  const char *const wrow[1] = {(const char *)lp->rw + (size_t)e * H * dsz<RD>()};
  const float bias = lp->rb ? lp->rb[e] : 0.f;  // added to the finished fp32 dot product
  for_token_groups(B, [&]<int TG>(int t0, int nt) {
    typename XSrc<XS>::ptr xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) xr[t] = router_row<XL, AD>(p, L, t0 + (t < nt ? t : 0));
    float acc[1][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = 0.f;
    rows_dot<RD, DT_F32, XS, 1, seg_router<RD, TG>(), TG>(wrow, s * Ks, (s + 1) * Ks, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float v = wave_sum63(acc[0][t]);
      if (t < nt && lane_id() == 63) {
        if (NSR == 1) {
          dbg_delay(p, DLY_PUBLISH, e);
          if constexpr (XL) publish(lp->lg + (size_t)(t0 + t) * E + e, nonzero_bits(v + bias));
          else publish(lp->lg + (size_t)(t0 + t) * E + e, v + bias);
        } else {
          slice_slot(p, L, round, wave_id())[t0 + t] = v;
        }
      }
    }
  });
  if (NSR > 1 && last_slice(p, L, 0, round, NSR)) {
    dbg_delay(p, DLY_PUBLISH, e);
    const int w0 = wave_id() - s;
    for (int t = lane_id(); t < B; t += 64) {
      float sum = slice_slot(p, L, round, w0)[t];
      for (int s2 = 1; s2 < NSR; ++s2) sum += slice_slot(p, L, round, w0 + s2)[t];
      if constexpr (XL) publish(lp->lg + (size_t)t * E + e, nonzero_bits(sum + bias));
      else publish(lp->lg + (size_t)t * E + e, sum + bias);
    }
  }
}

// the shared expert's h for (token, pair) index i
template <int AD, bool XL>
__device__ __forceinline__ void shared_h_out(KParams p, size_t i, float h) {
  if constexpr (XL) publish(p->hsh32 + i, round_act<AD>(h));
  else publish_act<AD>(p->hsbuf, i, h);
}

// shared gate/up task tau = (pair j, slice s) of round `round`. Several
// slices: slice sums to the LDS slot, and the last slice's wave finishes h.
// h goes to hsh32 as act-rounded fp32, published (small regime), or to hsbuf
// in the act dtype (general regime).
template <int AD, int SD, bool XL>
__device__ __forceinline__ void shared_gu_task(KParams p, KLayer lp, const Lds &L, int tau, int round) {
  const int H = p->H, B = p->B, Is = p->Is, NSS = p->NSS;
  const int j = tau / NSS, s = tau % NSS;
  const int Ks = H / NSS;
  const size_t rowb = (size_t)H * dsz<SD>();
  const char *const wrow[2] = {(const char *)lp->sgu + (size_t)j * rowb, (const char *)lp->sgu + (size_t)(Is + j) * rowb};
  for_token_groups(B, [&]<int TG>(int t0, int nt) {
    typename XSrc<XL>::ptr xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) xr[t] = xhat_row<XL, AD>(p, L, t0 + (t < nt ? t : 0));
    float acc[2][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = acc[1][t] = 0.f;
    rows_dot<SD, AD, XL, 2, seg_p0gu<SD, TG>(), TG>(wrow, s * Ks, (s + 1) * Ks, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float g = wave_sum63(acc[0][t]);
      const float u = wave_sum63(acc[1][t]);
      if (t < nt && lane_id() == 63) {
        if (NSS == 1) {
          shared_h_out<AD, XL>(p, (size_t)(t0 + t) * Is + j, silu_mul(g, u));
        } else {
          float *q = slice_slot(p, L, round, wave_id()) + 2 * (t0 + t);
          q[0] = g;
          q[1] = u;
        }
      }
    }
  });
  if (NSS > 1 && last_slice(p, L, 1, round, NSS)) {
    const int w0 = wave_id() - s;
    for (int t = lane_id(); t < B; t += 64) {
      float g = slice_slot(p, L, round, w0)[2 * t], u = slice_slot(p, L, round, w0)[2 * t + 1];
      for (int s2 = 1; s2 < NSS; ++s2) {
        g += slice_slot(p, L, round, w0 + s2)[2 * t];
        u += slice_slot(p, L, round, w0 + s2)[2 * t + 1];
      }
      shared_h_out<AD, XL>(p, (size_t)t * Is + j, silu_mul(g, u));
    }
  }
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

// number of set bits of m in the lanes below this one
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// float -> unsigned with the same order (-0 and +0 are made equal first)
__device__ __forceinline__ unsigned ord_f32(float v) {
  const unsigned u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(unsigned o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

constexpr int kMaxCand = 64;

// Logits of token t for the experts of this lane (e = lane + 64 j), all
// loads issued before the first use. Slots past E read expert E-1.
// (32-bit byte offsets from a uniform base: one register per address)
__device__ __forceinline__ float ld_off(const float *base, unsigned i) {
  return *(const float *)((const char *)base + i * 4u);
}

// POLL (small regime): the logits are read device-coherently until none of
// this token's is still unwritten (all-zero bits); this wait replaces a grid
// barrier, so the data arrive with the same round trip that observes them.
template <bool POLL>
__device__ __forceinline__ void load_logits(KParams p, KLayer lp, int t, float (&v)[kMaxE / 64]) {
  const int lane = lane_id(), E = p->E;
  constexpr int PER = kMaxE / 64;
  static_assert(PER == 16, "the polled load's wait lists 16 values");
  const float *base = lp->lg + (size_t)t * E;
  if constexpr (!POLL) {
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = ld_off(base, (unsigned)min(lane + 64 * j, E - 1));
  } else {
    const long long t0 = rt_now();
    for (;;) {
      // device-coherent (sc1) loads with a scalar base and 32-bit offsets;
      // the wait names every result, so nothing reads them before they land
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const unsigned off = (unsigned)min(lane + 64 * j, E - 1) * 4u;
        asm volatile("global_load_dword %0, %1, %2 sc1" : "=v"(v[j]) : "v"(off), "s"(base) : "memory");
      }
      asm volatile("s_waitcnt vmcnt(0)"
                   : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                     "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                     "+v"(v[15])
                   :
                   : "memory");
      bool missing = false;
#pragma unroll
      for (int j = 0; j < PER; ++j) missing |= __float_as_uint(v[j]) == 0u;
      if (__ballot(missing) == 0ull) break;
      if (rt_now() - t0 > p->timeout_ticks) {
        if (lane == 0) {
          __hip_atomic_store(ctrl_word(p, CTRL_ERR), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&Lds{}.head().expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Rare path (more than 64 logits tie at the threshold): k rounds of wave
// argmax over all logits. Returns the selection in lanes < k.
template <bool POLL>
__device__ __forceinline__ void topk_rounds(KParams p_arg, KLayer lp_arg, int t_arg, float &myv, int &myidx) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  const int t = uni(t_arg);
  const int lane = lane_id(), E = p->E, k = p->k;
  constexpr int PER = kMaxE / 64;
  float v[PER];
  load_logits<POLL>(p, lp, t, v);
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

template <bool POLL>
__device__ __attribute__((noinline)) void topk_token(KParams p_arg, KLayer lp_arg, const Lds &L, int t_arg, bool write_out_arg) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  const int t = uni(t_arg);
  const bool write_out = uni(write_out_arg);
  const int lane = lane_id();
  const int E = p->E, k = p->k;
  constexpr int PER = kMaxE / 64;
  // order keys of the logits: a NaN logit ranks last but stays selectable; a
  // slot past E gets key 0, below every expert's (so it is never a candidate)
  unsigned o[PER];
  {
    float v[PER];
    load_logits<POLL>(p, lp, t, v);
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] = lane + 64 * j < E ? ord_f32((v[j] == v[j]) ? v[j] : -INFINITY) : 0u;
  }
  if (write_out && lp->logits_out) {
    float *lo = lp->logits_out + (size_t)t * E;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (lane + 64 * j < E) lo[lane + 64 * j] = unord_f32(o[j]);
  }
  unsigned omax = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) omax = max(omax, o[j]);
  // T = k-th largest lane maximum (largest T with at least k lanes >= T)
  unsigned thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned c = thr | (1u << bit);
    if (__popcll(__ballot(omax >= c)) >= (unsigned)k) thr = c;
  }
  // thr >= the key of -inf > 0: at least k lanes hold an expert
  int nc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) nc += o[j] >= thr ? 1 : 0;
  // exclusive prefix of the candidate counts over the lanes, from ballots of
  // their bits (nc <= PER < 32)
  int pre = 0, total = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const unsigned long long m = __ballot((nc >> b) & 1);
    pre += lanes_below(m) << b;
    total += __popcll(m) << b;
  }
  int *sel_idx = L.at<int>(p->o_sel_idx);
  float *sel_w = L.at<float>(p->o_sel_w);
  int myidx = 0;
  float myv = -INFINITY;
  if (total <= kMaxCand) {
    // the small regime's routing wave may be any wave: slot 0 (the only one there)
    unsigned *ck = L.at<unsigned>(p->o_cand) + (POLL ? 0 : wave_id()) * 4 * kMaxCand;
    int *ci = (int *)ck + 2 * kMaxCand;
    int pos = pre;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (o[j] >= thr) { ck[pos] = o[j]; ci[pos] = lane + 64 * j; ++pos; }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    // one candidate per lane; each is ranked against the others read back
    // from lane c through the scalar unit (no LDS round trip per candidate)
    const unsigned mk = lane < total ? ck[lane] : 0u;
    const int me = lane < total ? ci[lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int c = 0; c < total; ++c) {
      const unsigned ok = (unsigned)__builtin_amdgcn_readlane((int)mk, c);
      const int oe = __builtin_amdgcn_readlane(me, c);
      rank += (ok > mk || (ok == mk && oe < me)) ? 1 : 0;
    }
    if (lane < total) {
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
    topk_rounds<POLL>(p, lp, t, myv, myidx);
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
__device__ __attribute__((noinline)) void build_tables(KParams p_arg, const Lds &L) {
  const KParams p = uni(p_arg);
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
// are distinct, so each key's rank (read lane by lane through the scalar
// unit) is its sorted position; the sorted keys go through LDS, and each run
// of equal experts is a union slot. Pairs of one expert keep ascending order,
// hence ascending tokens.
__device__ __attribute__((noinline)) void build_tables_wave(KParams p_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const int lane = lane_id(), P = p->B * p->k;
  const int *sel_idx = L.at<int>(p->o_sel_idx);
  int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  int *plist = L.at<int>(p->o_plist);
  unsigned *sorted = L.at<unsigned>(p->o_cand);  // slot 0: the small regime's routing wave
  const bool valid = lane < P;
  const unsigned key = valid ? ((unsigned)sel_idx[lane] << 6) | (unsigned)lane : 0xFFFFFFFFu;
  int rank = 0;
  for (int c = 0; c < P; ++c) rank += ((unsigned)__builtin_amdgcn_readlane((int)key, c) < key) ? 1 : 0;
  if (valid) sorted[rank] = key;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  const unsigned k2 = valid ? sorted[lane] : 0xFFFFFFFFu;
  const unsigned prev = (valid && lane > 0) ? sorted[lane - 1] : 0xFFFFFFFFu;
  const bool first = valid && (lane == 0 || (prev >> 6) != (k2 >> 6));
  const unsigned long long firsts = __ballot(first);
  if (valid) plist[lane] = (int)(k2 & 63u);
  if (first) {
    const int slot = lanes_below(firsts);
    const unsigned long long rest = lane < 63 ? firsts >> (lane + 1) : 0ull;
    const int nxt = rest ? lane + __ffsll((long long)rest) : P;
    ulist[slot] = (int)(k2 >> 6);
    ustart[slot] = lane;
    ucnt[slot] = nxt - lane;
  }
  if (lane == 0) L.head().nU = __popcll(firsts);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

// ---------------------------------------------------------------------------
// P1: expert gate/up, task (expert u of U, pair j)

template <int AD, int ED, bool XL>
__device__ __forceinline__ void expert_gu_task(KParams p, KLayer lp, const Lds &L, int u, int j) {
  dbg_delay(p, DLY_P1, u * 4096 + j);
  const int H = p->H, I = p->I, k = p->k;
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *plist = L.at<int>(p->o_plist);
  const int e = ulist[u];
  const int n = ucnt[u];
  const int *pl = plist + ustart[u];
  const size_t rowb = (size_t)H * dsz<ED>();
  const char *gu = (const char *)lp->egu + (size_t)e * 2 * I * rowb;
  const char *const wrow[2] = {gu + (size_t)j * rowb, gu + (size_t)(I + j) * rowb};
  uint32_t graw = 0x3F80u, uraw = 0x3F80u;
  if constexpr (ED == DT_FP8) {
    // the code conversion is exact, so the bf16 row scale multiplies the finished dot
    const uint16_t *sc = lp->egus + (size_t)e * (2 * I / 128);
    graw = sc[j / 128];
    uraw = sc[(I + j) / 128];
  }
  for_token_groups(n, [&]<int TG>(int t0, int nt) {
    typename XSrc<XL>::ptr xr[TG];
    int slot[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      slot[t] = pl[t0 + (t < nt ? t : 0)];
      xr[t] = xhat_row<XL, AD>(p, L, slot[t] / k);
    }
    float acc[2][TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[0][t] = acc[1][t] = 0.f;
    rows_dot<ED, AD, XL, 2, seg_gu_r<ED, TG, XL>(), TG>(wrow, 0, H, xr, acc);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      float g = wave_sum63(acc[0][t]), uu = wave_sum63(acc[1][t]);
      if constexpr (ED == DT_FP8) {
        g *= late_scale(graw);
        uu *= late_scale(uraw);
      }
      if (t < nt && lane_id() == 63) {
        const float h = silu_mul(g, uu);
        publish_act<AD>(p->hbuf, (size_t)slot[t] * I + j, h);  // h in the act dtype, published
      }
    }
  });
}

// ---------------------------------------------------------------------------
// P2: down projections of this workgroup's rows

// Small regime, one wave: the shared expert's h of every token (published
// fp32, already act-rounded) into LDS in the act dtype. Every load of a step
// is issued before the first use.
template <int AD>
__device__ __forceinline__ void stage_shared_h_wave(KParams p, const Lds &L) {
  const int n4 = p->B * p->Is / 4, lane = lane_id();
  const u32x4 *src = (const u32x4 *)p->hsh32;
  lds_t *hs = L.raw(p->o_hs);
  constexpr int U = 8;
  for (int i0 = 0; i0 < n4; i0 += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * 64 + lane;
      v[u] = src[i < n4 ? i : 0];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * 64 + lane;
      if (i < n4) {
        if constexpr (AD == DT_F32) {
          *(__attribute__((address_space(3))) u32x4 *)(hs + (size_t)i * 16) = v[u];
        } else {
          *(__attribute__((address_space(3))) u32x2 *)(hs + (size_t)i * 8) =
              u32x2{(v[u].x >> 16) | (v[u].y & 0xFFFF0000u), (v[u].z >> 16) | (v[u].w & 0xFFFF0000u)};
        }
      }
    }
  }
}

// One 4-row unit of a down matrix: row pointers wrow, columns [0, K) of x
// rows xr (TG tokens); writes the row sums (fp8 weights: times
// the bf16 scale word sraw, common to the unit's rows) to
// prow[(o0 + r - o0) * rs + col[t] * cs] (rs, cs: row and column strides of
// the partial-sum buffer).
template <int WD, int AD, bool XL, int TG, int DR = kDownRows>
__device__ __forceinline__ void down_unit(const char *const (&wrow)[kRowBlock], int K,
                                          const typename XSrc<XL>::ptr (&xr)[TG], uint32_t sraw,
                                          float *prow, int rs, int cs, const int (&col)[TG], int nt) {
#pragma unroll
  for (int r0 = 0; r0 < kRowBlock; r0 += DR) {
    const char *wr[DR];
    float acc[DR][TG];
#pragma unroll
    for (int r = 0; r < DR; ++r) {
      wr[r] = wrow[r0 + r];
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[r][t] = 0.f;
    }
    rows_dot<WD, AD, XL, DR, seg_down_r<WD, TG, XL>(), TG>(wr, 0, K, xr, acc);
#pragma unroll
    for (int r = 0; r < DR; ++r)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        float v = wave_sum63(acc[r][t]);
        if constexpr (WD == DT_FP8) v *= late_scale(sraw);
        if (t < nt && lane_id() == 63) prow[(r0 + r) * rs + col[t] * cs] = v;
      }
  }
}

// partial sums of P2: the workgroup's rows in LDS, row-major (small regime),
// or all rows in the workspace, column-major so that a unit's rows of one
// column are contiguous (general regime)
template <bool SMALL>
__device__ __forceinline__ float *part_base(KParams p, const Lds &L) {
  if constexpr (SMALL) return L.at<float>(p->o_part);
  else return p->partbuf;
}
template <bool SMALL> __device__ __forceinline__ int part_rs(KParams, int pstride) { return SMALL ? pstride : 1; }
template <bool SMALL> __device__ __forceinline__ int part_cs(KParams p) { return SMALL ? 1 : p->H; }

// Next P2 unit of this wave, handed out through the workgroup's LDS counter
// `which` (so a wave that starts late takes fewer).
__device__ __forceinline__ int next_unit(KParams p, SmemHead &sh, int which) {
  int u = 0;
  if (lane_id() == 0) u = __hip_atomic_fetch_add(&sh.unit_ctr[which], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  u = __builtin_amdgcn_readfirstlane(u);
  dbg_delay(p, DLY_P2, which * 65536 + u);
  return u;
}

// shared-expert units of rows [pr0, pr1): (row block, column block hf); the
// shared h comes from LDS (small regime) or global memory
template <int AD, int SD, bool SMALL>
__device__ __forceinline__ void shared_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1) {
  const int I = p->I, Is = p->Is, B = p->B;
  const int nsh = p->nsh, P = B * p->k, pstride = P + B * nsh;
  const int nrb = (pr1 - pr0) / kRowBlock;
  float *part = part_base<SMALL>(p, L);
  const int prb = SMALL ? pr0 : 0;
  for (int un = next_unit(p, L.head(), 0); un < nrb * nsh; un = next_unit(p, L.head(), 0)) {
    const int hf = un / nrb, rb = un % nrb;
    const int o0 = pr0 + rb * kRowBlock;
    const int kw = min(I, Is - hf * I);  // columns of block hf (the last may be partial)
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
      down_unit<SD, AD, SMALL, TG>(wrow, kw, xr, 0x3F80u, part + (size_t)(o0 - prb) * part_rs<SMALL>(p, pstride),
                                   part_rs<SMALL>(p, pstride), part_cs<SMALL>(p), col, nt);
    });
  }
}

// ---------------------------------------------------------------------------
// MFMA tiles for the experts that many tokens of a batch select (general
// regime). v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+i] and
// B[8(l/16)+i][l%16] (i < 8) and receives D[4(l/16)+i][l%16] (i < 4). A is 16
// weight rows, B is 16 tokens of the activation; the weights are read once
// for all the expert's tokens. fp8 weights: a lane loads 16 codes of its row,
// converts them exactly to bf16 (gfx950's OCP e4m3 conversion) and feeds two
// MFMAs; B takes the matching activation columns, so the K order is the same
// permutation on both sides.

#ifndef MOE_MFMA_MIN
#define MOE_MFMA_MIN 2
#endif
#ifndef MOE_MFMA_SHARED_MIN
#define MOE_MFMA_SHARED_MIN 8
#endif
constexpr int kMfmaMin = MOE_MFMA_MIN;  // tokens of one expert from which its rows go through MFMA tiles
constexpr int kMfmaSharedMin = MOE_MFMA_SHARED_MIN;  // batch from which the shared expert goes through MFMA tiles

// workgroup g's contiguous share of n tasks
__device__ __forceinline__ int share_lo(int n, int g, int G) { return (int)((long long)n * g / G); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// 16-byte loads at a uniform base plus a per-lane 32-bit byte offset, issued
// as written (the compiler neither splits nor delays them); the results must
// not be read before mfma_wait().
__device__ __forceinline__ u32x4 ld16_nt(const char *base, unsigned off) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, %2 nt" : "=v"(v) : "v"(off), "s"(base) : "memory");
  return v;
}
__device__ __forceinline__ u32x4 ld16(const char *base, unsigned off) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(v) : "v"(off), "s"(base) : "memory");
  return v;
}
// waits for every load in flight; each value is then passed through an
// empty asm so no use of it can be scheduled above the wait
template <int A, int B2>
__device__ __forceinline__ void mfma_wait(u32x4 (&a)[A][B2]) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B2; ++j) asm volatile("" : "+v"(a[i][j]));
}

// Whole-line loads. An MFMA operand gives each lane one row (l%16) and
// 16 bytes of it, so a 16-byte load in operand order reads 64 bytes of each
// of 16 rows and every 128-byte line is split over two instructions; such
// loads stream at ~5.4 TB/s where whole-line loads of the same bytes reach
// ~6.9 (a read-rate probe on MI355X). The tiles therefore load lines: X, rows
// 0-7 of a 16-row tile, and Y, rows 8-15, each lane reading chunk c(l) of row
// l%8 (8 lanes cover a row's 128 bytes), and a rotation by 8 lanes within each
// 16-lane row (DPP row_ror:8) hands lane (kq = l/16, s = l%16) the chunks of
// row s that operand order gives it: with c(l) = kq + 4((l>>3)&1), chunks kq
// (a) and 4 + kq (b); with c(l) = 2kq + ((l>>3)&1), chunks 2kq and 2kq + 1.
// The MFMAs see the same operands as with operand-order loads, so the results
// do not change.
// (lane-derived offsets are computed per task from lane_here(): kept from
// the start of the kernel, they are what the register allocator spills)
__device__ __forceinline__ int line_row(int h) { return 8 * h + (lane_here() & 7); }  // the lane's row of half h
__device__ __forceinline__ unsigned line_chunk4() {
  const int l = lane_here();
  return (unsigned)((l >> 4) + 4 * ((l >> 3) & 1));
}
__device__ __forceinline__ unsigned line_chunk2() {
  const int l = lane_here();
  return (unsigned)(2 * (l >> 4) + ((l >> 3) & 1));
}
constexpr int kXH = 2;  // activation offsets per token tile: rows line_row(0) and line_row(1)
__device__ __forceinline__ int x_row(int h) { return line_row(h); }
// in place: X becomes operand a, Y operand b
__device__ __forceinline__ void lines_to_operands(u32x4 &X, u32x4 &Y) {
  const bool lo = (lane_id() & 8) == 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const unsigned xr = (unsigned)__builtin_amdgcn_mov_dpp((int)X[d], DPP_ROW_ROR8, 0xF, 0xF, false);
    const unsigned yr = (unsigned)__builtin_amdgcn_mov_dpp((int)Y[d], DPP_ROW_ROR8, 0xF, 0xF, false);
    X[d] = lo ? X[d] : yr;
    Y[d] = lo ? xr : Y[d];
  }
}

// acc[row tile r][token tile t] += W rows x activation rows over K columns
// (bf16 weights). Addresses are a uniform base plus a per-lane 32-bit byte
// offset: woff[r][h] is the lane's row line_row(h) of row tile r, xoff[t][h]
// its token row x_row(h) of token tile t. Each iteration covers 64 columns,
// one 128-byte line of every row, and issues every load of the iteration
// (4 KB of weights per wave for a gate/up pair) before one wait; operand
// chunks kq and 4 + kq feed the two MFMAs of a row tile.
template <int NR, int NT>
__device__ __forceinline__ void mfma_rows(const char *wbase, const unsigned (&woff)[NR][2], int K, const char *xbase,
                                          const unsigned (&xoff)[NT][kXH], f32x4 (&acc)[NR][NT]) {
  const unsigned ch = line_chunk4() * 16u;  // the lane's chunk of each row's line
  for (int k0 = 0; k0 < K; k0 += 64) {
    u32x4 w[NR][2], x[NT][2];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r][0] = ld16_nt(wbase, woff[r][0] + (unsigned)k0 * 2u + ch);
      w[r][1] = ld16_nt(wbase, woff[r][1] + (unsigned)k0 * 2u + ch);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      x[t][0] = ld16(xbase, xoff[t][0] + (unsigned)k0 * 2u + ch);
      x[t][1] = ld16(xbase, xoff[t][1] + (unsigned)k0 * 2u + ch);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mfma_wait(w);
    mfma_wait(x);
#pragma unroll
    for (int r = 0; r < NR; ++r) lines_to_operands(w[r][0], w[r][1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) lines_to_operands(x[t][0], x[t][1]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = mfma16(w[r][h], x[t][h], acc[r][t]);
  }
}

// mfma_rows with S 64-column steps per wait, for short K ranges whose steps
// would otherwise each be a round trip (K a multiple of 64; the last wait's
// steps past K load step K - 64 again, passed through the wait and unused).
// The MFMAs run step by step, so the results equal mfma_rows'.
template <int NR, int NT, int S>
__device__ __forceinline__ void mfma_rows_multi(const char *wbase, const unsigned (&woff)[NR][2], int K,
                                                const char *xbase, const unsigned (&xoff)[NT][kXH],
                                                f32x4 (&acc)[NR][NT]) {
  const unsigned ch = line_chunk4() * 16u;
  for (int k0 = 0; k0 < K; k0 += 64 * S) {
    u32x4 w[S * NR][2], x[S * NT][2];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const unsigned kb = (unsigned)min(k0 + 64 * st, K - 64) * 2u + ch;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        w[st * NR + r][0] = ld16_nt(wbase, woff[r][0] + kb);
        w[st * NR + r][1] = ld16_nt(wbase, woff[r][1] + kb);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        x[st * NT + t][0] = ld16(xbase, xoff[t][0] + kb);
        x[st * NT + t][1] = ld16(xbase, xoff[t][1] + kb);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mfma_wait(w);
    mfma_wait(x);
#pragma unroll
    for (int st = 0; st < S; ++st) {
      if (k0 + 64 * st < K) {
#pragma unroll
        for (int r = 0; r < NR; ++r) lines_to_operands(w[st * NR + r][0], w[st * NR + r][1]);
#pragma unroll
        for (int t = 0; t < NT; ++t) lines_to_operands(x[st * NT + t][0], x[st * NT + t][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[r][t] = mfma16(w[st * NR + r][h], x[st * NT + t][h], acc[r][t]);
      }
    }
  }
}

// fp8 weights (up to 2 token tiles): the same product with two 64-column
// steps per wait (K a multiple of 128), so that a row's 128 codes are one
// line: chunks kq and 4 + kq feed steps 0 and 1, and the activation's
// 32-byte pieces of the two steps (chunks 2kq and 2kq + 1 of each step's
// line) are loaded the same way. A lane's 16 codes are converted exactly to
// bf16 and feed two MFMAs. An fp8 step moves half the weight bytes of a
// bf16 step, so one step per wait would leave a tile waiting on latency.
// The MFMAs run step by step, so the results do not depend on how many
// steps share a wait.
template <int NR, int NT>
__device__ __forceinline__ void mfma_rows_fp8x2(const char *wbase, const unsigned (&woff)[NR][2], int K,
                                                const char *xbase, const unsigned (&xoff)[NT][kXH],
                                                f32x4 (&acc)[NR][NT]) {
  const unsigned wc = line_chunk4() * 16u, xc = line_chunk2() * 16u;
  for (int k0 = 0; k0 < K; k0 += 128) {
    u32x4 w[NR][2], x[2 * NT][2];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r][0] = ld16_nt(wbase, woff[r][0] + (unsigned)k0 + wc);
      w[r][1] = ld16_nt(wbase, woff[r][1] + (unsigned)k0 + wc);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const unsigned cb = ((unsigned)k0 + 64u * (unsigned)st) * 2u + xc;
        x[st * NT + t][0] = ld16(xbase, xoff[t][0] + cb);
        x[st * NT + t][1] = ld16(xbase, xoff[t][1] + cb);
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mfma_wait(w);
    mfma_wait(x);
#pragma unroll
    for (int r = 0; r < NR; ++r) lines_to_operands(w[r][0], w[r][1]);
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) lines_to_operands(x[i][0], x[i][1]);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 wr = w[r][st];
        const u32x4 lo = fp8x8_to_bf16(wr.x, wr.y), hi = fp8x8_to_bf16(wr.z, wr.w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[r][t] = mfma16(lo, x[st * NT + t][0], acc[r][t]);
          acc[r][t] = mfma16(hi, x[st * NT + t][1], acc[r][t]);
        }
      }
  }
}

// fp8 weights and 3 or 4 token tiles: a row's 128 codes are loaded as one
// line, as in mfma_rows_fp8x2, but the activations of the two 64-column
// steps are loaded one step at a time, in operand order (lane l: token row
// l%16, its 16 columns as two 16-byte pieces), so that the tile fits the
// registers without spilling inside the loop; the second step's
// activation loads (L2) are issued after the first step's MFMAs. Same MFMA
// order, so the same results.
template <int NR, int NT>
__device__ __forceinline__ void mfma_rows_fp8_split(const char *wbase, const unsigned (&woff)[NR][2], int K,
                                                    const char *xbase, const unsigned (&xoff)[NT][kXH],
                                                    f32x4 (&acc)[NR][NT]) {
  const unsigned wc = line_chunk4() * 16u, xc = ((unsigned)lane_here() >> 4) * 32u;
  const bool hs = (lane_here() & 8) != 0;
  unsigned xs[NT];  // the lane's token row l%16 of each token tile
#pragma unroll
  for (int t = 0; t < NT; ++t) xs[t] = hs ? xoff[t][1] : xoff[t][0];
  for (int k0 = 0; k0 < K; k0 += 128) {
    u32x4 w[NR][2];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r][0] = ld16_nt(wbase, woff[r][0] + (unsigned)k0 + wc);
      w[r][1] = ld16_nt(wbase, woff[r][1] + (unsigned)k0 + wc);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 x[NT][2];
      const unsigned cb = ((unsigned)k0 + 64u * (unsigned)st) * 2u + xc;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        x[t][0] = ld16(xbase, xs[t] + cb);
        x[t][1] = ld16(xbase, xs[t] + cb + 16u);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (st == 0) {
        mfma_wait(w);
#pragma unroll
        for (int r = 0; r < NR; ++r) lines_to_operands(w[r][0], w[r][1]);
      }
      mfma_wait(x);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 wr = w[r][st];
        const u32x4 lo = fp8x8_to_bf16(wr.x, wr.y), hi = fp8x8_to_bf16(wr.z, wr.w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[r][t] = mfma16(lo, x[t][0], acc[r][t]);
          acc[r][t] = mfma16(hi, x[t][1], acc[r][t]);
        }
      }
    }
  }
}

// The expert tiles' product: bf16 weights one 64-column step per wait, fp8
// weights two (one line per row), with both steps' activations loaded
// together up to 2 token tiles
template <int WD, int NR, int NT>
__device__ __forceinline__ void mfma_rows_expert(const char *wbase, const unsigned (&woff)[NR][2], int K,
                                                 const char *xbase, const unsigned (&xoff)[NT][kXH],
                                                 f32x4 (&acc)[NR][NT]) {
  if constexpr (WD != DT_FP8) mfma_rows<NR, NT>(wbase, woff, K, xbase, xoff, acc);
  else if constexpr (NT <= 2) mfma_rows_fp8x2<NR, NT>(wbase, woff, K, xbase, xoff, acc);
  else mfma_rows_fp8_split<NR, NT>(wbase, woff, K, xbase, xoff, acc);
}

// Run f.template operator()<NT>() with NT = ceil(n / 16) token tiles (1..4).
template <class F>
__device__ __forceinline__ void with_token_tiles(int n, F &&f) {
  const int nt = (n + 15) / 16;
  if (nt <= 1) f.template operator()<1>();
  else if (nt == 2) f.template operator()<2>();
  else if (nt == 3) f.template operator()<3>();
  else f.template operator()<4>();
}

// P1 MFMA task: rows [16 jb, 16 jb + 16) of union slot u's gate and up
// matrices for all of the expert's tokens; h = SiLU(g) * u to hbuf.
template <int AD, int ED>
__device__ __forceinline__ void mfma_gu_task(KParams p, KLayer lp, const Lds &L, int u, int jb) {
  dbg_delay(p, DLY_P1, u * 4096 + jb);
  const int H = p->H, I = p->I, k = p->k;
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *pl = L.at<int>(p->o_plist) + ustart[u];
  const int e = ulist[u], n = ucnt[u];
  const size_t rowb = (size_t)H * dsz<ED>();
  const char *gu = (const char *)lp->egu + (size_t)e * 2 * I * rowb;  // < 4 GB: 32-bit offsets
  unsigned wo[2][2];  // gate and up rows 16 jb + line_row(h)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    wo[0][h] = (unsigned)((16 * jb + line_row(h)) * rowb);
    wo[1][h] = (unsigned)((I + 16 * jb + line_row(h)) * rowb);
  }
  uint32_t graw = 0x3F80u, uraw = 0x3F80u;
  if constexpr (ED == DT_FP8) {
    const uint16_t *sc = lp->egus + (size_t)e * (2 * I / 128);
    graw = uni((uint32_t)sc[(16 * jb) / 128]);  // uniform: kept in scalar registers
    uraw = uni((uint32_t)sc[(I + 16 * jb) / 128]);
  }
  with_token_tiles(n, [&]<int NT>() {
    unsigned xo[NT][kXH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < kXH; ++h) {
        const int c = min(16 * t + x_row(h), n - 1);  // columns past n repeat a valid token; discarded
        xo[t][h] = (unsigned)(pl[c] / k) * (unsigned)H * 2u;
      }
    f32x4 acc[2][NT];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_rows_expert<ED, 2, NT>(uni(gu), wo, H, (const char *)p->xa, xo, acc);
    const int r = lane_here() & 15, kq = lane_here() >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = 16 * t + r;
      if (c < n) {
        const int slot = pl[c];
        float h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = silu_mul(acc[0][t][i] * late_scale(graw), acc[1][t][i] * late_scale(uraw));
        publish_act4<AD>(p->hbuf, (size_t)slot * I + 16 * jb + 4 * kq, h);
      }
    }
  });
}

// P2 MFMA tile: rows [o0, min(o0 + 16 NR, hi)) of union slot s's down matrix
// for all of the expert's tokens (NR row tiles of 16 rows), into the partial
// sums. Lanes of rows at or past hi (the workgroup's end) load row hi - 1
// again, whose lines a load of the same step fetches anyway, and their
// results are dropped: a partial tile reads no bytes beyond its rows. Two row tiles
// read the tokens' h once for 32 rows.
#ifndef MOE_P2_TILE_NR
#define MOE_P2_TILE_NR 2
#endif
template <int AD, int ED, int NR>
__device__ __forceinline__ void mfma_down_tile(KParams p, KLayer lp, const Lds &L, int s, int o0, int hi, float *part) {
  const int H = p->H, I = p->I, lane = lane_id();
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *pl = L.at<int>(p->o_plist) + ustart[s];
  const int e = ulist[s], n = ucnt[s];
  const int kq0 = lane >> 4;
  const char *wbase = (const char *)lp->ed + (size_t)e * H * I * dsz<ED>();  // < 4 GB: 32-bit offsets
  unsigned wo[NR][2];
#pragma unroll
  for (int q = 0; q < NR; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) wo[q][h] = (unsigned)((size_t)min(o0 + 16 * q + line_row(h), hi - 1) * I * dsz<ED>());
  // scale of the lane's output rows o0 + 16 q + 4 kq .. + 3 (one 128-row
  // group: the 4 rows start at a multiple of 4), applied after the tile
  uint32_t sraw[NR];
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    sraw[q] = 0x3F80u;
    if constexpr (ED == DT_FP8) sraw[q] = lp->eds[(size_t)e * (H / 128) + min(o0 + 16 * q + 4 * kq0, hi - 1) / 128];
  }
  with_token_tiles(n, [&]<int NT>() {
    unsigned xo[NT][kXH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < kXH; ++h) xo[t][h] = (unsigned)pl[min(16 * t + x_row(h), n - 1)] * (unsigned)I * 2u;
    f32x4 acc[NR][NT];
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_rows_expert<ED, NR, NT>(uni(wbase), wo, I, (const char *)p->hbuf, xo, acc);
    const int r = lane_here() & 15, kq = lane_here() >> 4;
    // the lane's 4 rows o0 + 16 q + 4 kq .. + 3 are all below hi or all at or
    // past it (hi - o0 is a multiple of 4): one 16-byte store per token column
    // (column-major partial sums, 16-byte aligned: H and o0 are multiples of 4)
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int ob = o0 + 16 * q + 4 * kq;
      if (ob < hi) {
        const float sc = ED == DT_FP8 ? late_scale(sraw[q]) : 1.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = 16 * t + r;
          if (c < n)
            *(f32x4 *)(part + (size_t)pl[c] * H + ob) =
                f32x4{acc[q][t][0] * sc, acc[q][t][1] * sc, acc[q][t][2] * sc, acc[q][t][3] * sc};
        }
      }
    }
  });
}

// P0 on MFMA tiles (general regime from kMfmaSharedMin tokens): first a
// router unit (one K part of a 16-expert tile, for all tokens), then shared
// gate/up tiles. Within a unit or tile the 16 waves split the K columns and
// sum their partial tiles in LDS in wave order.
__device__ __forceinline__ int router_tiles(int E) { return (E + 15) / 16; }
// Router units: each 16-expert tile's K range is split into p->rq parts, and
// unit u = tile * rq + q goes to workgroup u, so the router's bytes spread
// over nearly every CU (with one CU per whole tile, the router barrier waited
// for 56 CUs streaming 458 KB each while the rest streamed half of that).
__device__ __forceinline__ int router_units(KParams p) { return router_tiles(p->E) * p->rq; }
// first 16-column block of wave w's share of K part q
__device__ __forceinline__ int router_unit_blk(KParams p, int q, int w) {
  const int nb = p->H / 16;
  const int q0 = share_lo(nb, q, p->rq), q1 = share_lo(nb, q + 1, p->rq);
  return q0 + share_lo(q1 - q0, w, kWaves);
}

// Before the x-hat wait (general regime): one dword of every 128-byte line
// of this wave's share of its workgroup's first router unit is loaded, so
// that the unit's loads after the barrier find its lines in L2 instead of
// waiting on HBM while the barrier is pending anyway. Router weights are
// static, so loading them before a barrier is safe.
template <int RD>
__device__ __forceinline__ void router_touch(KParams p, KLayer lp) {
  const int u = wg_id(p);
  if (u >= router_units(p)) return;
  const int tile = u / p->rq, q = u % p->rq, wv = wave_id();
  const size_t lo = (size_t)router_unit_blk(p, q, wv) * 16 * dsz<RD>();
  const size_t hi = (size_t)router_unit_blk(p, q, wv + 1) * 16 * dsz<RD>();
  if (lo >= hi) return;
  const size_t l0 = lo & ~(size_t)127;
  const int nl = (int)((hi - l0 + 127) / 128);  // lines of each of the tile's 16 rows
  const size_t row_bytes = (size_t)p->H * dsz<RD>();
  for (int i = lane_id(); i < 16 * nl; i += 64) {
    const int row = min(16 * tile + i % 16, p->E - 1);
    const char *a = (const char *)lp->rw + (size_t)row * row_bytes + l0 + (size_t)128 * (i / 16);
    unsigned v;
    asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(a) : "memory");
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(v) : : "memory");
  }
}

// Router tile: v_mfma_f32_16x16x4_f32 with lane l holding A[l%16][l/16] and
// B[l/16][l%16] in fp32 (bf16 router weights widen exactly). In a 16-column
// block lane l loads columns 4(l/16) .. 4(l/16)+3 of its expert row and of
// its token row, and MFMA m of the block takes component m: k-slot q then
// holds column 4q + m on both sides. The logits (with the bias) go to rfin.
__device__ __forceinline__ f32x4 mfma4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8-byte load at a uniform base plus a per-lane byte offset (see ld16)
__device__ __forceinline__ u32x2 ld8_nt(const char *base, unsigned off) {
  u32x2 v;
  asm volatile("global_load_dwordx2 %0, %1, %2 nt" : "=v"(v) : "v"(off), "s"(base) : "memory");
  return v;
}
template <int A>
__device__ __forceinline__ void mfma_wait2(u32x2 (&a)[A]) {
#pragma unroll
  for (int i = 0; i < A; ++i) asm volatile("" : "+v"(a[i]));
}

template <int RD>
__device__ __attribute__((noinline)) void router_mfma(KParams p_arg, KLayer lp_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  const int H = p->H, E = p->E, B = p->B, lane = lane_id(), wv = wave_id(), tid = threadIdx.x;
  const int r = lane & 15, kq = lane >> 4, RQ = p->rq;
  SmemHead &sh = L.head();
  for (int u = wg_id(p); u < router_units(p); u += p->G) {
    const int tile = u / RQ, q = u % RQ;
    const int b0 = router_unit_blk(p, q, wv), b1 = router_unit_blk(p, q, wv + 1);
    const unsigned wo = (unsigned)((size_t)min(16 * tile + r, E - 1) * H * dsz<RD>()) + (unsigned)(kq * 4 * dsz<RD>());
    const char *wb = (const char *)lp->rw;
    const char *xb = (const char *)p->xhat;
    float *red = L.at<float>(p->o_red);  // [kWaves][16][B]
    with_token_tiles(B, [&]<int NT>() {
      unsigned xo[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) xo[t] = (unsigned)min(16 * t + r, B - 1) * (unsigned)H * 4u + (unsigned)kq * 16u;
      f32x4 acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      // RB 16-column blocks per wait (a wave's share is 7 blocks at H = 7168
      // and 4 K parts); blocks past b1 load block b1 - 1 again, unused
      constexpr int RB = NT == 1 ? 8 : NT == 2 ? 4 : 2;
      for (int blk = b0; blk < b1; blk += RB) {
        unsigned c[RB];
#pragma unroll
        for (int h = 0; h < RB; ++h) c[h] = (unsigned)min(blk + h, b1 - 1) * 16u;
        u32x4 x[RB][NT];
        float wf[RB][4];
        if constexpr (RD == DT_F32) {
          u32x4 w[RB];
#pragma unroll
          for (int h = 0; h < RB; ++h) w[h] = ld16_nt(uni(wb), wo + c[h] * 4u);
#pragma unroll
          for (int h = 0; h < RB; ++h)
#pragma unroll
            for (int t = 0; t < NT; ++t) x[h][t] = ld16(uni(xb), xo[t] + c[h] * 4u);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          u32x4 wt[1][RB];
#pragma unroll
          for (int h = 0; h < RB; ++h) wt[0][h] = w[h];
          mfma_wait(wt);
          mfma_wait(x);
#pragma unroll
          for (int h = 0; h < RB; ++h) {
            wf[h][0] = __uint_as_float(wt[0][h].x); wf[h][1] = __uint_as_float(wt[0][h].y);
            wf[h][2] = __uint_as_float(wt[0][h].z); wf[h][3] = __uint_as_float(wt[0][h].w);
          }
        } else {
          u32x2 w[RB];
#pragma unroll
          for (int h = 0; h < RB; ++h) w[h] = ld8_nt(uni(wb), wo + c[h] * 2u);
#pragma unroll
          for (int h = 0; h < RB; ++h)
#pragma unroll
            for (int t = 0; t < NT; ++t) x[h][t] = ld16(uni(xb), xo[t] + c[h] * 4u);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          mfma_wait2(w);
          mfma_wait(x);
#pragma unroll
          for (int h = 0; h < RB; ++h) {
            wf[h][0] = bf_lo(w[h].x); wf[h][1] = bf_hi(w[h].x);
            wf[h][2] = bf_lo(w[h].y); wf[h][3] = bf_hi(w[h].y);
          }
        }
#pragma unroll
        for (int h = 0; h < RB; ++h) {
          if (blk + h < b1) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const uint32_t xm = m == 0 ? x[h][t].x : m == 1 ? x[h][t].y : m == 2 ? x[h][t].z : x[h][t].w;
                acc[t] = mfma4f32(wf[h][m], __uint_as_float(xm), acc[t]);
              }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int cc = 16 * t + r;
        if (cc < B) {
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(size_t)(wv * 16 + 4 * kq + i) * B + cc] = acc[t][i];
        }
      }
    });
    __syncthreads();
    // this part's sums over the waves (wave order), published
    float *part = p->rpart + (size_t)q * B * E;
    for (int idx = tid; idx < 16 * B; idx += kThreads) {
      const int i = idx / B, t = idx % B, e = 16 * tile + i;
      float sum = 0.f;
      for (int w = 0; w < kWaves; ++w) sum += red[(size_t)(w * 16 + i) * B + t];
      if (e < E) publish(part + (size_t)t * E + e, sum);
    }
    // the last of the tile's RQ workgroups to arrive sums the parts in part
    // order (whoever it is, the same sums) and writes the logits with the bias
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(ctrl_word(p, CTRL_RTILE + tile), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sh.route_claim = old == (unsigned)RQ - 1u;
    }
    __syncthreads();
    if (sh.route_claim) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      for (int idx = tid; idx < 16 * B; idx += kThreads) {
        const int i = idx % 16, t = idx / 16, e = 16 * tile + i;
        if (e < E) {
          float sum = 0.f;
          for (int q2 = 0; q2 < RQ; ++q2) sum += p->rpart[((size_t)q2 * B + t) * E + e];
          publish(lp->lg + (size_t)t * E + e, sum + (lp->rb ? lp->rb[e] : 0.f));
        }
      }
      if (tid == 0) __hip_atomic_store(ctrl_word(p, CTRL_RTILE + tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
}

// Shared expert on MFMA tiles (bf16), after the router units. Gate/up tile
// j is one 16-row A operand: gate rows [8j, 8j + 8) over up rows [8j, 8j + 8),
// so that g and u of one h element land in the same tile; workgroup g takes
// tiles g, g + G, ..., and its waves split K in 64-column steps.
template <int NT> constexpr int kSharedSteps() { return NT == 1 ? 4 : NT == 2 ? 2 : 1; }
__device__ __forceinline__ int shared_tile_row(int Is, int j, int r) { return r < 8 ? 8 * j + r : Is + 8 * j + r - 8; }
__device__ __forceinline__ int shared_tile_k(int H, int w) { return share_lo(H / 64, w, kWaves) * 64; }

template <int AD>
__device__ __attribute__((noinline)) void shared_gu_mfma(KParams p_arg, KLayer lp_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  const KLayer lp = uni(lp_arg);
  const int H = p->H, Is = p->Is, B = p->B, wv = wave_id();
  const int k0 = shared_tile_k(H, wv), k1 = shared_tile_k(H, wv + 1);
  float *red = L.at<float>(p->o_red);  // [kWaves][16][B]
  const char *xa = (const char *)p->xa + (size_t)k0 * 2;
  for (int j = wg_id(p); j < Is / 8; j += p->G) {
    const char *wb = (const char *)lp->sgu + (size_t)k0 * 2;
    const unsigned wo[1][2] = {{(unsigned)((size_t)shared_tile_row(Is, j, line_row(0)) * H * 2),  // < 4 GB
                                (unsigned)((size_t)shared_tile_row(Is, j, line_row(1)) * H * 2)}};
    with_token_tiles(B, [&]<int NT>() {
      unsigned xo[NT][kXH];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < kXH; ++h) xo[t][h] = (unsigned)min(16 * t + x_row(h), B - 1) * (unsigned)H * 2u;
      f32x4 acc[1][NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      // a wave's share is a few steps (7 at H = 7168): up to 4 per wait
      mfma_rows_multi<1, NT, kSharedSteps<NT>()>(uni(wb), wo, k1 - k0, uni(xa), xo, acc);
      const int r = lane_here() & 15, kq = lane_here() >> 4;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = 16 * t + r;
        if (c < B) {
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(size_t)(wv * 16 + 4 * kq + i) * B + c] = acc[0][t][i];
        }
      }
    });
    __syncthreads();
    for (int q = threadIdx.x; q < 8 * B; q += kThreads) {
      const int jj = q / B, t = q % B;
      float g = 0.f, u = 0.f;
      for (int w = 0; w < kWaves; ++w) {
        g += red[(size_t)(w * 16 + jj) * B + t];
        u += red[(size_t)(w * 16 + 8 + jj) * B + t];
      }
      publish_act<AD>(p->hsbuf, (size_t)t * Is + 8 * j + jj, silu_mul(g, u));
    }
    __syncthreads();
  }
}

// Shared down on MFMA tiles (general regime, bf16): units (half hf of the
// shared intermediate columns, 16-row tile of rows [pr0, pr1)) through unit
// counter 0; the partial sums go to the shared expert's partial columns.
// Needs pr1 >= 16 (the launch enables this path only when every workgroup
// owns at least 16 rows).
template <int AD>
__device__ __forceinline__ void shared_down_mfma(KParams p, KLayer lp, const Lds &L, int pr0, int pr1) {
  const int H = p->H, I = p->I, Is = p->Is, B = p->B;
  const int nsh = p->nsh, P = B * p->k;
  const int ntile = (pr1 - pr0 + 15) / 16;
  float *part = p->partbuf;
  for (int un = next_unit(p, L.head(), 0); un < ntile * nsh; un = next_unit(p, L.head(), 0)) {
    const int hf = un / ntile, o0 = pr0 + 16 * (un % ntile);
    const char *wb = (const char *)lp->sd + (size_t)hf * I * 2;
    const char *xb = (const char *)p->hsbuf + (size_t)hf * I * 2;
    // lanes of rows past pr1 load row pr1 - 1 again (no extra bytes); their results are dropped
    const unsigned wo[1][2] = {{(unsigned)((size_t)min(o0 + line_row(0), pr1 - 1) * Is * 2),
                                (unsigned)((size_t)min(o0 + line_row(1), pr1 - 1) * Is * 2)}};
    with_token_tiles(B, [&]<int NT>() {
      unsigned xo[NT][kXH];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < kXH; ++h) xo[t][h] = (unsigned)min(16 * t + x_row(h), B - 1) * (unsigned)Is * 2u;
      f32x4 acc[1][NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      mfma_rows<1, NT>(uni(wb), wo, min(I, Is - hf * I), uni(xb), xo, acc);
      const int r = lane_here() & 15, kq = lane_here() >> 4;
      // as in mfma_down_tile: the lane's 4 rows are all valid or all past pr1
      if (o0 + 4 * kq < pr1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = 16 * t + r;
          if (c < B) *(f32x4 *)(part + (size_t)(P + c * nsh + hf) * H + o0 + 4 * kq) = acc[0][t];  // column-major
        }
      }
    });
  }
}

// P1 cost of a GEMV row pair of an expert with n tokens and of an MFMA tile
// (16 pairs, ceil(n/16) token tiles), in tenths of a one-token GEMV pair:
// per-task timings on MI355X at the K3 share (B=64, every wave streaming)
// for the GEMV pairs; the MFMA tile's from step times over a range of
// values (with whole-line loads a tile costs less than the timings of
// operand-order loads gave).
#ifndef MOE_COST_G2
#define MOE_COST_G2 15
#endif
#ifndef MOE_COST_M0
#define MOE_COST_M0 150
#endif
#ifndef MOE_COST_M1
#define MOE_COST_M1 24
#endif
__device__ __forceinline__ int gemv_pair_cost(int n) { return n <= 1 ? 10 : n == 2 ? MOE_COST_G2 : n <= 4 ? 21 : 11 + 4 * n; }
__device__ __forceinline__ int mfma_tile_cost(int n) { return MOE_COST_M0 + MOE_COST_M1 * ((n + 15) / 16); }
// all of a listed slot's P1 work
__device__ __forceinline__ int slot_cost(KParams p, bool mfma, int n) {
  return mfma ? (p->I / 16) * mfma_tile_cost(n) : p->I * gemv_pair_cost(n);
}

// Union slots split by token count: MFMA tiles (n >= mfma_min) and GEMV.
__device__ __attribute__((noinline)) void classify_slots(KParams p_arg, const Lds &L) {
  const KParams p = uni(p_arg);
  SmemHead &sh = L.head();
  if (wave_id() == 0) {
    const int lane = lane_id(), nU = sh.nU;
    const int *ucnt = L.at<int>(p->o_ucnt);
    int *mslot = L.at<int>(p->o_mslot), *gslot = L.at<int>(p->o_gslot);
    int nm = 0, ng = 0;
    for (int u0 = 0; u0 < nU; u0 += 64) {
      const int u = u0 + lane;
      const bool valid = u < nU;
      const bool m = valid && p->mfma_min > 0 && ucnt[u] >= p->mfma_min;
      const unsigned long long bm = __ballot(m), bg = __ballot(valid && !m);
      const unsigned long long below = (1ull << lane) - 1ull;
      if (m) mslot[nm + __popcll(bm & below)] = u;
      if (valid && !m) gslot[ng + __popcll(bg & below)] = u;
      nm += __popcll(bm);
      ng += __popcll(bg);
    }
    if (lane == 0) { sh.nM = nm; sh.nG = ng; }
    // cost prefix over the listed slots (MFMA slots, then GEMV slots)
    int *cpre = L.at<int>(p->o_cpre);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    int run = 0;
    for (int i0 = 0; i0 < nm + ng; i0 += 64) {
      const int i = i0 + lane;
      const int c = i < nm + ng ? slot_cost(p, i < nm, ucnt[i < nm ? mslot[i] : gslot[i - nm]]) : 0;
      int incl = c;  // inclusive prefix over the lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int up = __shfl_up(incl, d);
        if (lane >= d) incl += up;
      }
      if (i < nm + ng) cpre[i] = run + incl - c;
      run += __shfl(incl, 63);
    }
    if (lane == 0) cpre[nm + ng] = run;
  }
  __syncthreads();
}

// One routed expert's 4-row GEMV unit (slot s, rows [o0, o0+4)).
template <int AD, int ED, bool SMALL>
__device__ __forceinline__ void expert_down_gemv(KParams p, KLayer lp, const Lds &L, int s, int o0, float *prow,
                                                 int rs, int cs) {
  const int H = p->H, I = p->I;
  const int *ulist = L.at<int>(p->o_ulist), *ucnt = L.at<int>(p->o_ucnt), *ustart = L.at<int>(p->o_ustart);
  const int *plist = L.at<int>(p->o_plist);
  const int e = ulist[s];
  const int n = ucnt[s];
  const int *pl = plist + ustart[s];
  const char *wrow[kRowBlock];
#pragma unroll
  for (int r = 0; r < kRowBlock; ++r) wrow[r] = (const char *)lp->ed + ((size_t)e * H + o0 + r) * I * dsz<ED>();
  // o0 is a multiple of the row block, which divides the 128-row scale group
  uint32_t sraw = 0x3F80u;
  if constexpr (ED == DT_FP8) sraw = lp->eds[(size_t)e * (H / 128) + o0 / 128];
  for_token_groups(n, [&]<int TG>(int t0, int nt) {
    typename XSrc<false>::ptr xr[TG];
    int col[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      col[t] = pl[t0 + (t < nt ? t : 0)];
      xr[t] = (const char *)p->hbuf + (size_t)col[t] * I * dsz<AD>();
    }
    // fp8 rows are half as long: all 4 rows of the unit in one pass
    down_unit<ED, AD, false, TG, ED == DT_FP8 ? MOE_GEN_DOWN_ROWS_FP8 : kDownRows>(wrow, I, xr, sraw, prow, rs, cs, col, nt);
  });
}

// Small regime: routed-expert units of rows [pr0, pr1): (union slot, 4-row
// block) for the slots [ua, ub) of one expert group, slot-major so a wave's
// consecutive units read consecutive rows, handed out through counter uc.
template <int AD, int ED, bool SMALL>
__device__ __forceinline__ void expert_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int ua, int ub,
                                                  int uc) {
  const int B = p->B;
  const int nsh = p->nsh, P = B * p->k, pstride = P + B * nsh;
  const int nrb = (pr1 - pr0) / kRowBlock;
  float *part = part_base<SMALL>(p, L);
  const int prb = SMALL ? pr0 : 0;
  const int nu = ub - ua;
  for (int un = next_unit(p, L.head(), uc); un < nrb * nu; un = next_unit(p, L.head(), uc)) {
    const int s = ua + un / nrb, o0 = pr0 + (un % nrb) * kRowBlock;
    expert_down_gemv<AD, ED, SMALL>(p, lp, L, s, o0, part + (size_t)(o0 - prb) * part_rs<SMALL>(p, pstride),
                                    part_rs<SMALL>(p, pstride), part_cs<SMALL>(p));
  }
}

#ifndef MOE_P2_SPREAD
#define MOE_P2_SPREAD 1
#endif

// General regime: routed-expert units of rows [pr0, pr1) for listed slots
// [ia, ib) (MFMA slots first, then GEMV slots), handed out through unit
// counter uc: MFMA down tiles of 16 rows for the MFMA slots (GEMV units when
// the workgroup has fewer than 16 rows), 4-row GEMV units for the others.
template <int AD, int ED>
__device__ __forceinline__ void expert_down_listed(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int ia, int ib,
                                                   int uc) {
  const int nrb = (pr1 - pr0) / kRowBlock, nM = L.head().nM;
  float *part = p->partbuf;
  const int *mslot = L.at<int>(p->o_mslot), *gslot = L.at<int>(p->o_gslot);
  constexpr int TR = 16 * MOE_P2_TILE_NR;  // rows of a down tile
  const int ntile = (pr1 - pr0) >= 16 ? (pr1 - pr0 + TR - 1) / TR : 0;
  const int ma = min(ia, nM), mb = min(ib, nM);
  const int nmu = (mb - ma) * (ntile > 0 ? ntile : nrb);
  const int total = nmu + (max(ib, nM) - max(ia, nM)) * nrb;
  for (int u0 = next_unit(p, L.head(), uc); u0 < total; u0 = next_unit(p, L.head(), uc)) {
#if MOE_P2_SPREAD
    // MFMA units spread evenly over the claim order: unit j of nmu sits at
    // position floor(j * total / nmu), the GEMV units fill the rest in order
    int un;
    {
      const int j = (int)(((long long)u0 * nmu + total - 1) / total);  // MFMA positions before u0
      un = (j < nmu && (int)((long long)j * total / nmu) == u0) ? j : nmu + (u0 - j);
    }
#else
    const int un = u0;
#endif
    if (un < nmu && ntile > 0) {
      mfma_down_tile<AD, ED, MOE_P2_TILE_NR>(p, lp, L, mslot[ma + un / ntile], pr0 + TR * (un % ntile), pr1, part);
    } else {
      const int s = un < nmu ? mslot[ma + un / nrb] : gslot[max(ia, nM) - nM + (un - nmu) / nrb];
      const int o0 = pr0 + ((un < nmu ? un : un - nmu) % nrb) * kRowBlock;
      expert_down_gemv<AD, ED, false>(p, lp, L, s, o0, part + o0, 1, p->H);
    }
  }
}

// y = x + shared + sum_i w_i d_i (rank order i) for rows [pr0, pr1). pub:
// y is the next layer's input, written with device-coherent stores so that
// the layer barrier needs no L2 write-back. poison: a wait gave up during the
// launch, so the rows are written as NaN instead.
template <int AD, bool SMALL>
__device__ __forceinline__ void combine(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, bool pub, bool poison) {
  const int H = p->H, k = p->k, B = p->B;
  const int nsh = p->nsh, P = B * k, pstride = P + B * nsh;
  const float *part = part_base<SMALL>(p, L);
  const int prb = SMALL ? pr0 : 0;
  const float *sel_w = L.at<float>(p->o_sel_w);
  const int nr = pr1 - pr0, cells = nr * B;
  dbg_delay(p, DLY_COMBINE, 0);
  for (int c = threadIdx.x; c < cells; c += kThreads) {
    const int ro = c % nr, t = c / nr;  // consecutive threads: consecutive rows (coalesced x, y, partials)
    const int o = pr0 + ro;
    const int cs = part_cs<SMALL>(p);
    const float *pp = part + (size_t)(o - prb) * part_rs<SMALL>(p, pstride);
    // a cell's partial sums are loaded 8 at a time before they are used (one
    // at a time they were k + nsh dependent round trips); the sums keep
    // their order
    float sh = 0.f;
    for (int hf = 0; hf < nsh; ++hf) sh += pp[(size_t)(P + t * nsh + hf) * cs];
    float rt = 0.f;
    for (int i0 = 0; i0 < k; i0 += 8) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = pp[(size_t)(t * k + min(i0 + j, k - 1)) * cs];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i0 + j < k) rt = fmaf(sel_w[t * k + i0 + j], pv[j], rt);
    }
    // after a watchdog stop the rows are not trusted: NaN makes that visible in y
    const float v = poison ? __builtin_nanf("") : load_act<AD>(lp->x, (size_t)t * H + o) + sh + rt;
    if (pub) publish_act<AD>(lp->y, (size_t)t * H + o, v);
    else store_act<AD>(lp->y, (size_t)t * H + o, v);
  }
}

// P0 task of wave wv of workgroup g in round r, or -1. Every round but the
// last gives each workgroup kWaves consecutive task indices; the last gives
// each p0w (fewer when the tasks left do not need all waves), so the spare
// waves of every workgroup are free early and one of them routes the batch.
// The slices of a row stay within one workgroup and round: p0w and the
// shared tasks' first index are multiples of the slice counts.
__device__ __forceinline__ int p0_task(KParams p, int r, int g, int wv) {
  const int w = (r == p->p0r - 1) ? p->p0w : kWaves;
  return wv < w ? r * p->G * kWaves + g * w + wv : -1;
}

// ---------------------------------------------------------------------------
// the kernel

__device__ __forceinline__ void raise_flag(int &f) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane_id() == 0) __hip_atomic_store(&f, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void wait_flag(int &f) {
  if (lane_id() == 0)
    while (__hip_atomic_load(&f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// P0 of this wave: its router slices, arrival at the router barrier, its
// shared gate/up slices, arrival at the shared barrier. PUB: the small
// regime's published stores and arrivals; there the routing waves poll the
// logits themselves and no router barrier is kept.
template <int AD, int RD, int SD, bool PUB, bool MSH>
__device__ __forceinline__ void p0_tasks(KParams p, KLayer lp, const Lds &L, int b0) {
  SmemHead &sh = L.head();
  const int nrt = p->E * p->NSR, s0 = p->s0, end = p->p0_end;
  bool routed = false;  // arrived at the router barrier
  for (int r = 0; r < p->p0r; ++r) {
    const int tau = p0_task(p, r, wg_id(p), wave_id());
    if (tau < 0 || tau >= end) break;
    if (tau >= nrt && !routed) {
      if constexpr (!PUB) bar_arrive_published(p, sh, b0 + BAR_ROUTER);
      routed = true;
    }
    if (tau < nrt) router_task_any<AD, RD, PUB>(p, lp, L, tau, r);
    else if (!MSH && tau >= s0) shared_gu_task<AD, SD, PUB>(p, lp, L, tau - s0, r);
  }
  if constexpr (PUB) {
    bar_arrive_published(p, sh, b0 + BAR_SHARED);
  } else {
    if constexpr (MSH) router_mfma<RD>(p, lp, L);
    if (!routed) bar_arrive_published(p, sh, b0 + BAR_ROUTER);
    if constexpr (MSH) shared_gu_mfma<AD>(p, lp, L);
    bar_arrive_published(p, sh, b0 + BAR_SHARED);
  }
}

// General regime: the first listed slot of P1 group gi of nG: the first slot
// whose cost prefix reaches gi/nG of the total (gi = nG gives nL).
__device__ __forceinline__ int group_first_slot(const int *cpre, int nL, int gi, int nG) {
  if (gi >= nG) return nL;
  const int target = share_lo(cpre[nL], gi, nG);
  int a = 0, z = nL;  // first i with cpre[i] >= target
  while (a < z) {
    const int m = (a + z) >> 1;
    if (cpre[m] < target) a = m + 1; else z = m;
  }
  return a;
}

// General regime, P1 tasks numbered in listed order: the I/16 MFMA tiles of
// each MFMA slot, then the I row pairs of each GEMV slot. First task of
// listed slot i:
__device__ __forceinline__ int p1_task_base(KParams p, int nM, int i) {
  const int nb = p->I / 16;
  return i <= nM ? i * nb : nM * nb + (i - nM) * p->I;
}

// The first task of listed slots [ia, ib) whose starting cost is >= c
// (p1_task_base(ib) if none).
__device__ __forceinline__ int p1_task_at_cost(KParams p, const Lds &L, int ia, int ib, int c) {
  const int nM = L.head().nM;
  const int *mslot = L.at<int>(p->o_mslot), *gslot = L.at<int>(p->o_gslot);
  const int *ucnt = L.at<int>(p->o_ucnt), *cpre = L.at<int>(p->o_cpre);
  if (ia >= ib || c >= cpre[ib]) return p1_task_base(p, nM, ib);
  int a = ia, z = ib;  // the last i in [ia, ib) with cpre[i] <= c
  while (z - a > 1) {
    const int m = (a + z) >> 1;
    if (cpre[m] <= c) a = m; else z = m;
  }
  if (c <= cpre[a]) return p1_task_base(p, nM, a);
  const bool mf = a < nM;
  const int slot = mf ? mslot[a] : gslot[a - nM];
  const int uc = mf ? mfma_tile_cost(ucnt[slot]) : gemv_pair_cost(ucnt[slot]);
  // j <= the slot's task count, since c < cpre[a + 1]
  return p1_task_base(p, nM, a) + (c - cpre[a] + uc - 1) / uc;
}

// General regime: the P1 tasks [t0, t1) of this workgroup's cost share of
// one group, handed out to its waves one at a time through the group's LDS
// counter, so that waves that drew long tasks (MFMA tiles) take fewer and the
// workgroup's waves finish together.
template <int AD, int ED>
__device__ __forceinline__ void p1_claimed(KParams p, KLayer lp, const Lds &L, int t0, int t1, int gi) {
  SmemHead &sh = L.head();
  const int I = p->I, nb = I / 16, nM = sh.nM, mt = nM * nb;
  const int *mslot = L.at<int>(p->o_mslot), *gslot = L.at<int>(p->o_gslot);
  for (;;) {
    int q = 0;
    if (lane_id() == 0) q = __hip_atomic_fetch_add(&sh.p1_ctr[gi], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int t = t0 + __builtin_amdgcn_readfirstlane(q);
    if (t >= t1) break;
    if (t < mt) mfma_gu_task<AD, ED>(p, lp, L, mslot[t / nb], t % nb);
    else expert_gu_task<AD, ED, false>(p, lp, L, gslot[(t - mt) / I], (t - mt) % I);
  }
}

// General regime: the last part of every workgroup's share of a P1 group is
// taken through a counter in the workspace (CTRL_P1), so that a workgroup
// done with its own tasks takes the remaining tail tasks of others: first
// its own tail, then the tails of up to MOE_P1_STEAL workgroups g + 8, g + 16,
// ... (the same XCD when the grid is a multiple of 8). A task's result does
// not depend on which wave runs it. Each workgroup zeroes its counters at the
// start of every layer.
#ifndef MOE_P1_STEAL
#define MOE_P1_STEAL 4
#endif
#ifndef MOE_P1_TAIL_DIV
#define MOE_P1_TAIL_DIV 0  // 0: p->tail_div (a quarter of each share up to 16 tokens, a third above)
#endif
__device__ __forceinline__ void p1_share(KParams p, const Lds &L, int ia, int ib, int Clo, int Chi, int v, int &t0,
                                         int &tm, int &t1) {
  const int NW = p->G * kWaves;
  t0 = p1_task_at_cost(p, L, ia, ib, Clo + share_lo(Chi - Clo, v * kWaves, NW));
  t1 = p1_task_at_cost(p, L, ia, ib, Clo + share_lo(Chi - Clo, (v + 1) * kWaves, NW));
  tm = t1 - (t1 - t0) / (MOE_P1_TAIL_DIV > 0 ? MOE_P1_TAIL_DIV : p->tail_div);
}
template <int AD, int ED>
__device__ __forceinline__ void p1_stealing(KParams p, KLayer lp, const Lds &L, int ia, int ib, int Clo, int Chi,
                                            int gi) {
  SmemHead &sh = L.head();
  const int I = p->I, nb = I / 16, nM = sh.nM, mt = nM * nb, G = p->G, g = wg_id(p);
  const int *mslot = L.at<int>(p->o_mslot), *gslot = L.at<int>(p->o_gslot);
  int t0, tm, t1;
  p1_share(p, L, ia, ib, Clo, Chi, g, t0, tm, t1);
  p1_claimed<AD, ED>(p, lp, L, t0, tm, gi);  // the private part, through LDS
  for (int hop = 0; hop <= MOE_P1_STEAL && hop < G; ++hop) {
    const int v = (g + 8 * hop) % G;
    if (hop > 0) {
      if (v == g) break;
      p1_share(p, L, ia, ib, Clo, Chi, v, t0, tm, t1);
    }
    unsigned *ctr = ctrl_word(p, CTRL_P1 + v * kP1Groups + gi);
    for (;;) {
      int q = 0;
      if (lane_id() == 0) q = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int t = tm + __builtin_amdgcn_readfirstlane(q);
      if (t >= t1) break;
      if (t < mt) mfma_gu_task<AD, ED>(p, lp, L, mslot[t / nb], t % nb);
      else expert_gu_task<AD, ED, false>(p, lp, L, gslot[(t - mt) / I], (t - mt) % I);
    }
  }
}

// One layer at B <= 2. P0: router slices, then shared gate/up slices, dealt
// round-robin over all waves of the grid (every slice is ~7 KB, so the waves
// finish together). The first wave of each workgroup to run out of P0 work
// routes the batch and builds the gather tables (by then the memory system has
// drained, so its few dependent loads are fast), the others wait for the
// tables. P1 and P2 overlap: a wave done with P1 runs the shared expert's
// down rows and then the routed experts' down rows of every expert group
// whose barrier has passed, while slower waves finish the later groups. The
// first wave done with P1 stages the shared expert's h.
template <int AD, int RD, int ED, int SD>
__device__ __forceinline__ bool layer_small(KParams p, KLayer lp, const Lds &L, int b0, int W, int NW) {
  SmemHead &sh = L.head();
  const int G = p->G, g = wg_id(p);
  stage_xhat<AD>(p, lp, L);

  // P0
  p0_tasks<AD, RD, SD, true, false>(p, lp, L, b0);

  // routing, by the first wave out of P0 work
  int claimed = 0;
  if (lane_id() == 0)
    claimed = __hip_atomic_exchange(&sh.route_claim, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
  claimed = __builtin_amdgcn_readfirstlane(claimed);
  if (claimed) {
    dbg_delay(p, DLY_ROUTE, 0);
    for (int t = 0; t < p->B; ++t) topk_token<true>(p, lp, L, t, g == 0);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    build_tables_wave(p, L);
    raise_flag(sh.route_ready);
  } else {
    wait_flag(sh.route_ready);
  }

  // P1: the expert gate/up rows (union slot, pair) in slot order, round-robin
  // over the grid's waves; the rounds fall into nG groups, each closed by its
  // barrier, so a slot is complete once the group of its last round is
  const int I = p->I, N = sh.nU * I;
  const int R1 = (N + NW - 1) / NW, nG = min(kP1Groups, R1);
  for (int gi = 0; gi < nG; ++gi) {
    for (int r = share_lo(R1, gi, nG); r < share_lo(R1, gi + 1, nG); ++r) {
      const int q = W + r * NW;
      if (q < N) expert_gu_task<AD, ED, true>(p, lp, L, q / I, q % I);
    }
    bar_arrive_published(p, sh, b0 + BAR_H + gi);
  }

  // P2: the shared expert's rows first (input ready since P0), which fills the
  // wait for the expert barrier, then the routed experts' rows and the combine
  int sclaim = 0;
  if (lane_id() == 0)
    sclaim = __hip_atomic_exchange(&sh.shared_claim, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
  sclaim = __builtin_amdgcn_readfirstlane(sclaim);
  if (sclaim) {
    bar_wait(p, sh, b0 + BAR_SHARED);
    dbg_delay(p, DLY_STAGE, 0);
    stage_shared_h_wave<AD>(p, L);
    raise_flag(sh.shared_ready);
  } else {
    wait_flag(sh.shared_ready);
  }
  const int r0 = g * p->rows_per_wg;
  const int r1 = min(p->H, r0 + p->rows_per_wg);
  if (r0 < r1) shared_down_units<AD, SD, true>(p, lp, L, r0, r1);
  // the routed experts' rows, group by group: slots [ua, ub) end in group gi
  // (the last group always holds the last slot); the error word is read once
  // the last group's barrier has passed, its latency hidden by the down rows
  int ua = 0;
  unsigned gerr = 0;
  for (int gi = 0; gi < nG; ++gi) {
    const int rend = share_lo(R1, gi + 1, nG);
    int ub = ua;
    while (ub < sh.nU && ((ub + 1) * I - 1) / NW < rend) ++ub;
    if (ub > ua) {
      bar_wait(p, sh, b0 + BAR_H + gi);
      if (gi == nG - 1) gerr = err_word(p);
      if (r0 < r1) expert_down_units<AD, ED, true>(p, lp, L, r0, r1, ua, ub, 2 + gi);
    }
    ua = ub;
  }
  // every workgroup is past its routing (all arrived at the last expert
  // barrier): clear this workgroup's share of the layer's logits for the next
  // use of the buffer (the stores complete before the layer barrier or the
  // end of the launch)
  if (wave_id() == 0) {
    dbg_delay(p, DLY_CLEAR, 0);
    const int n = p->B * p->E;
    for (int i = share_lo(n, g, G) + lane_id(); i < share_lo(n, g + 1, G); i += 64) publish(lp->lg + i, 0.f);
  }
  // one decision for the whole workgroup (its waves read the error word separately)
  const bool poison = __syncthreads_or(gerr != 0 || sh.expired != 0);
  if (r0 < r1) combine<AD, true>(p, lp, L, r0, r1, b0 / kBarPerLayer + 1 < p->L, poison);
  __syncthreads();
  return poison;
}

// SMALL: B <= kSmallB. MSH: general regime with the shared expert on MFMA tiles.
template <int AD, int RD, int ED, int SD, bool SMALL, bool MSH>
__global__ void __launch_bounds__(kThreads, 1) moe_kernel(Params params) {
  // read the parameters in place in the kernarg segment (scalar loads; no private copy)
  (void)params;
  KParams p = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  const Lds L{};
  SmemHead &sh = L.head();
  const int tid = threadIdx.x, wv = wave_id();
  const int NW = p->G * kWaves;
  const int W = wg_id(p) * kWaves + wv;  // global wave id of this share

  for (int i = tid; i < kMaxBarriers; i += kThreads) sh.bar_cnt[i] = sh.bar_claim[i] = sh.bar_flag[i] = 0;
  if (tid == 0) sh.expired = 0;
  dbg_delay(p, DLY_START, 0);

  bool poisoned = false;  // a wait gave up during this launch (this workgroup's, or one before a barrier it passed)
  for (int l = 0; l < p->L; ++l) {
    KLayer lp = &p->lp[l];
    const int b0 = kBarPerLayer * l;
    for (int i = tid; i < 2 * p->p0r * kWaves; i += kThreads) L.at<int>(p->o_scnt)[i] = 0;
    if (tid == 0) {
      sh.route_claim = sh.route_ready = sh.shared_claim = sh.shared_ready = 0;
      for (int i = 0; i < 2 + kP1Groups; ++i) sh.unit_ctr[i] = 0;
      for (int i = 0; i < kP1Groups; ++i) sh.p1_ctr[i] = 0;
    }
    __syncthreads();

    if (p->route_only) {
      if constexpr (SMALL) {
        stage_xhat<AD>(p, lp, L);
      } else {
        produce_xhat<AD>(p, lp, L);
        bar_arrive_published(p, sh, b0 + BAR_XHAT);
        bar_wait(p, sh, b0 + BAR_XHAT);
      }
      for (int tau = W, r = 0; tau < p->E * p->NSR; tau += NW, ++r) router_task_any<AD, RD, SMALL>(p, lp, L, tau, r);
      bar_arrive_published(p, sh, b0 + BAR_ROUTER);
      bar_wait(p, sh, b0 + BAR_ROUTER);
      poisoned = err_word(p) != 0;
      if (wg_id(p) == 0)
        for (int t = wv; t < p->B; t += kWaves) topk_token<false>(p, lp, L, t, true);
      break;
    }

    if constexpr (SMALL) {
      poisoned |= layer_small<AD, RD, ED, SD>(p, lp, L, b0, W, NW);
    } else {
      // x-hat (published: the barrier needs no L2 write-back)
      // this workgroup's P1 tail counters start at zero: reset before it
      // arrives at the x-hat barrier, so before any wave takes a P1 task (all
      // wait for the router barrier first); the previous layer's and launch's
      // takes ended before their barriers or launch end (or the outputs are
      // already poisoned by a watchdog stop)
      if (p->steal && threadIdx.x < kP1Groups)
        __hip_atomic_store(ctrl_word(p, CTRL_P1 + wg_id(p) * kP1Groups + (int)threadIdx.x), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      produce_xhat<AD>(p, lp, L);
      bar_arrive_published(p, sh, b0 + BAR_XHAT);
      if constexpr (MSH) router_touch<RD>(p, lp);
      bar_wait(p, sh, b0 + BAR_XHAT);

      // P0: router slices, then shared gate/up
      p0_tasks<AD, RD, SD, false, MSH>(p, lp, L, b0);

      // P1: routing (one wave per token), gather tables, expert gate/up. The
      // tasks (MFMA tiles of the listed MFMA slots, then GEMV row pairs of the
      // GEMV slots) have measured costs. The listed slots fall into up to
      // kP1Groups groups of about equal cost, each closed by its barrier; in
      // every group each wave of the grid takes the tasks whose starting cost
      // falls in its equal share, so all waves finish group 0 first and the
      // down projections of early groups overlap the later gate/up work.
      bar_wait(p, sh, b0 + BAR_ROUTER);
      for (int t = wv; t < p->B; t += kWaves) topk_token<false>(p, lp, L, t, wg_id(p) == 0);
      __syncthreads();
      build_tables(p, L);
      classify_slots(p, L);
      const int nL = sh.nM + sh.nG, nGr = min(p->p1_groups, nL);
      const int *cpre = L.at<int>(p->o_cpre);
      for (int gi = 0; gi < nGr; ++gi) {
        const int ia = group_first_slot(cpre, nL, gi, nGr), ib = group_first_slot(cpre, nL, gi + 1, nGr);
        const int Clo = cpre[ia], Chi = cpre[ib];
        if (p->steal) {
          p1_stealing<AD, ED>(p, lp, L, ia, ib, Clo, Chi, gi);
        } else {
          const int g = wg_id(p), lo = Clo + share_lo(Chi - Clo, g * kWaves, NW);
          const int hi = Clo + share_lo(Chi - Clo, (g + 1) * kWaves, NW);
          p1_claimed<AD, ED>(p, lp, L, p1_task_at_cost(p, L, ia, ib, lo), p1_task_at_cost(p, L, ia, ib, hi), gi);
        }
        bar_arrive_published(p, sh, b0 + BAR_H + gi);
      }

      // P2: this workgroup's output rows, partial sums in global memory; the
      // shared expert's rows first, then each group's routed rows once its
      // barrier has passed
      const int r0 = wg_id(p) * p->rows_per_wg;
      const int r1 = min(p->H, r0 + p->rows_per_wg);
      bar_wait(p, sh, b0 + BAR_SHARED);
      if (r0 < r1) {
        if constexpr (MSH) shared_down_mfma<AD>(p, lp, L, r0, r1);
        else shared_down_units<AD, SD, false>(p, lp, L, r0, r1);
      }
      unsigned gerr = 0;
      for (int gi = 0; gi < nGr; ++gi) {
        bar_wait(p, sh, b0 + BAR_H + gi);
        // every take of this group ended before its barrier: back to zero, so
        // that the workspace is left as found (the layer start zeroes them
        // again, which covers a watchdog stop)
        if (p->steal && threadIdx.x == 0)
          __hip_atomic_store(ctrl_word(p, CTRL_P1 + wg_id(p) * kP1Groups + gi), 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (gi == nGr - 1) gerr = err_word(p);  // latency hidden by the last group's down rows
        const int ia = group_first_slot(cpre, nL, gi, nGr), ib = group_first_slot(cpre, nL, gi + 1, nGr);
        if (r0 < r1) expert_down_listed<AD, ED>(p, lp, L, r0, r1, ia, ib, 2 + gi);
      }
      const bool poison = __syncthreads_or(gerr != 0 || sh.expired != 0);
      poisoned |= poison;
      if (r0 < r1) combine<AD, false>(p, lp, L, r0, r1, l + 1 < p->L, poison);
      __syncthreads();
    }

    if (l + 1 < p->L) {
      // the next layer reads, before its own first barrier, only y (published
      // by the combine) and values published by this layer; its workspace
      // buffers are rewritten before other workgroups read them
      bar_arrive_published(p, sh, b0 + BAR_LAYER);
      bar_wait(p, sh, b0 + BAR_LAYER);
    }
  }

  // after a watchdog stop the routing outputs are not trusted either: the
  // workgroup that wrote them overwrites them with -1 / NaN
  const bool poison_out = __syncthreads_or(poisoned || sh.expired != 0);
  if (wg_id(p) == 0 && poison_out) {
    const int n = p->B * p->k;
    for (int l = 0; l < p->L; ++l) {
      KLayer lp = &p->lp[l];
      for (int i = tid; i < n; i += kThreads) {
        if (lp->idx_out) lp->idx_out[i] = -1;
        if (lp->w_out) lp->w_out[i] = __builtin_nanf("");
      }
      if (lp->logits_out)
        for (int i = tid; i < p->B * p->E; i += kThreads) lp->logits_out[i] = __builtin_nanf("");
    }
  }

  // last workgroup out resets the counters for the next launch on this
  // workspace. Every wave first waits for its own memory operations, barrier
  // increments included (a workgroup need not wait on every barrier it
  // arrived at), so all of a workgroup's increments are complete before it
  // counts itself out, and the reset follows every workgroup's increments. A
  // relaxed count then suffices; the end of the launch makes y visible. An
  // acquire-release count wrote back L2 on the last workgroup's critical path.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(ctrl_word(p, CTRL_DONE), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.route_claim = old == (unsigned)p->G - 1u;  // this workgroup is the last out
    if (old == (unsigned)p->G - 1u) {
      for (int b = 0; b < kBarPerLayer * p->L; ++b)
        __hip_atomic_store(ctrl_word(p, CTRL_BAR + b), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (sh.route_claim && tid == 0 && !p->self_reset)
    __hip_atomic_store(ctrl_word(p, CTRL_DONE), 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  if (p->self_reset) {
    // The static workspace has no moe_check_workspace: after a watchdog stop
    // (already visible as NaN outputs) the last workgroup out clears the
    // error word and the small-batch logit buffers itself.
    if (sh.route_claim) {
      if (err_word(p) != 0) {
        for (int i = tid; i < 2 * kSmallB * p->E; i += kThreads) publish(p->rlog + i, 0.f);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(ctrl_word(p, CTRL_ERR), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (tid == 0) __hip_atomic_store(ctrl_word(p, CTRL_DONE), 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// zero n words (the control words and logit buffers of a fresh workspace)
__global__ void __launch_bounds__(256) zero_words(unsigned *w, unsigned n) {
  for (unsigned i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) w[i] = 0u;
}


// ---------------------------------------------------------------------------
// Multi-launch path (moe_decode_layer_unfused): the same layer as eleven
// separate kernels with every intermediate (x-hat, logits, routing, expert
// grouping, gate/up outputs, h, down outputs, the shared expert's) in HBM, the
// way an unfused decode step runs it. It is the measured baseline of the
// fusion above. Its GEMVs use the same streaming core: one wave per weight
// row, activation rows from global memory; an align kernel groups the
// (token, expert) pairs by expert, so each selected expert's rows are read
// once per group of up to 4 of its tokens.

constexpr int kUfThreads = 256;
constexpr int kUfRows = kUfThreads / 64;  // GEMV kernels: one weight row per wave

// x-hat of token blockIdx.x (one 1024-thread workgroup, 16-byte chunks):
// fp32 (router input) and act (FFN input; for fp32 activations xa is xf)
template <int AD>
__global__ void __launch_bounds__(kThreads) uf_rmsnorm(const void *x, const void *gamma, int H, float eps,
                                                        float *xf, void *xa) {
  __shared__ float red[kWaves];
  constexpr int EPC = 16 / dsz<AD>(), NC = act_chunks_max<AD>();
  const size_t t = blockIdx.x;
  const int tid = threadIdx.x, nch = H / EPC;
  u32x4 xv[NC], gv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + c * kThreads, cc = ch < nch ? ch : 0;
    xv[c] = *(const u32x4 *)((const char *)x + (t * nch + cc) * 16);
    gv[c] = *(const u32x4 *)((const char *)gamma + (size_t)cc * 16);
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (tid + c * kThreads < nch) {
      float f[8];
      act_chunk_vals<AD>(xv[c], f);
#pragma unroll
      for (int q = 0; q < EPC; ++q) ss = fmaf(f[q], f[q], ss);
    }
  }
  ss = readlane_f(wave_sum63(ss), 63);
  if (lane_id() == 0) red[wave_id()] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kWaves; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = tid + c * kThreads;
    if (ch < nch) {
      float f[8], g[8];
      act_chunk_vals<AD>(xv[c], f);
      act_chunk_vals<AD>(gv[c], g);
#pragma unroll
      for (int q = 0; q < EPC; ++q) {
        const float v = f[q] * r * g[q];
        const size_t h = (size_t)ch * EPC + q;
        xf[t * H + h] = v;
        if constexpr (AD != DT_F32) store_act<AD>(xa, t * H + h, v);
      }
    }
  }
}

// Gathered GEMV. Job j (blockIdx.y) uses matrix m = idx ? idx[j] : 0 and,
// for TG = 1, activation row j / x_div; for TG > 1, rows TG j .. TG j + TG - 1
// (those below nx). out[row][r] = scale * sum_k W_m[r][k] X[row][k] + bias[r];
// fp8 weights take the bf16 scale of their 128-row group.
struct UfGemv {
  const char *w;          // matrix 0, rows of K elements
  size_t mat_bytes;       // bytes from one matrix to the next
  const int32_t *idx;     // [jobs] matrix of each job, or NULL
  int R, K;               // rows, columns
  const char *x;          // activation rows of K elements
  int x_div, nx;
  const uint16_t *scale;  // fp8: [m][R / 128] bf16
  const float *bias;      // [R] or NULL
  float *out;             // [rows][R]
};

template <int WD, int XD, int TG>
__global__ void __launch_bounds__(kUfThreads) uf_gemv(UfGemv a) {
  const int r = blockIdx.x * kUfRows + wave_id(), j = blockIdx.y;
  if (r >= a.R) return;
  const int m = a.idx ? a.idx[j] : 0;
  const char *const wrow[1] = {a.w + (size_t)m * a.mat_bytes + (size_t)r * a.K * dsz<WD>()};
  const char *xr[TG];
  int row[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    row[t] = TG == 1 ? j / a.x_div : min(TG * j + t, a.nx - 1);
    xr[t] = a.x + (size_t)row[t] * a.K * dsz<XD>();
  }
  float acc[1][TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) acc[0][t] = 0.f;
  rows_dot<WD, XD, false, 1, 2, TG>(wrow, 0, a.K, xr, acc);
  float sc = 1.f;
  if constexpr (WD == DT_FP8) sc = __uint_as_float((uint32_t)a.scale[(size_t)m * (a.R / 128) + r / 128] << 16);
  const float b = a.bias ? a.bias[r] : 0.f;
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const float v = wave_sum63(acc[0][t]) * sc + b;
    const int orow = TG == 1 ? j : TG * j + t;
    if (lane_id() == 63 && (TG == 1 || orow < a.nx)) a.out[(size_t)orow * a.R + r] = v;
  }
}

// top-k of token blockIdx.x (one wave): k rounds of wave argmax (larger
// logit, then lower index), then the softmax restricted to the selection
__global__ void __launch_bounds__(64) uf_topk(const float *logits, int E, int k, int32_t *idx, float *w) {
  const int t = blockIdx.x, lane = lane_id();
  float v[kMaxE / 64];  // slots past E hold -inf and never win against a logit
#pragma unroll
  for (int q = 0; q < kMaxE / 64; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? logits[(size_t)t * E + e] : -INFINITY;
  }
  float my_l = 0.f;
  int my_e = 0;
  for (int i = 0; i < k; ++i) {
    // the lane's best (strictly larger keeps the lower index), branch-free
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int q = 1; q < kMaxE / 64; ++q) {
      const bool take = v[q] > bv;
      bv = take ? v[q] : bv;
      bi = take ? lane + 64 * q : bi;
    }
    wave_argmax(bv, bi);
    if (lane == i) {
      my_l = bv;
      my_e = bi;
    }
#pragma unroll
    for (int q = 0; q < kMaxE / 64; ++q) v[q] = lane + 64 * q == bi ? -INFINITY : v[q];
  }
  const float lmax = readlane_f(my_l, 0);
  const float pe = lane < k ? expf(my_l - lmax) : 0.f;
  const float sum = readlane_f(wave_sum63(pe), 63);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = pe / sum;
  }
}

// Exclusive prefix of v over the 1024 threads of a workgroup (every thread
// calls it); total receives the sum.
__device__ __forceinline__ int uf_block_scan(int v, int *wtot, int &total) {
  const int lane = lane_id(), wv = wave_id();
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int t = wtot[w];
    if (w < wv) base += t;
    total += t;
  }
  __syncthreads();
  return base + incl - v;
}

// Expert grouping of the P (token, expert) pairs, one workgroup: the union of
// the selected experts in ascending order (ulist, *nU of them), and each
// expert's pairs in ascending pair order, so ascending tokens
// (plist[ustart[u] .. ustart[u + 1])).
__global__ void __launch_bounds__(kThreads) uf_align(const int32_t *idx, int P, int E, int *nU, int *ulist,
                                                      int *ustart, int *plist) {
  __shared__ int cnt[kMaxE], start[kMaxE], sidx[kMaxB * kMaxK], wtot[kWaves];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
  for (int q = tid; q < P; q += kThreads) sidx[q] = idx[q];
  __syncthreads();
  for (int q = tid; q < P; q += kThreads) atomicAdd(&cnt[sidx[q]], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0, f = c > 0 ? 1 : 0;
  int totc, totf;
  const int sc = uf_block_scan(c, wtot, totc);  // first pair position of expert tid
  const int sf = uf_block_scan(f, wtot, totf);  // union slot of expert tid
  if (tid < E) {
    start[tid] = sc;
    if (f) {
      ulist[sf] = tid;
      ustart[sf] = sc;
    }
  }
  if (tid == 0) {
    *nU = totf;
    ustart[totf] = totc;
  }
  __syncthreads();
  // stable placement: pair q follows the earlier pairs of its expert
  for (int q = tid; q < P; q += kThreads) {
    const int e = sidx[q];
    int r = 0;
    for (int q2 = 0; q2 < q; ++q2) r += sidx[q2] == e ? 1 : 0;
    plist[start[e] + r] = q;
  }
}

// Grouped GEMV over the union: job u (blockIdx.y) below *nU is expert
// ulist[u] with the pairs plist[ustart[u] .. ustart[u + 1]); each wave reads
// its weight row once per group of up to 4 pairs and writes out[pair][r].
// The activation row of pair q is q / x_div.
struct UfGroup {
  const char *w;          // matrix 0, rows of K elements
  size_t mat_bytes;       // bytes from one expert's matrix to the next
  int R, K;
  const char *x;          // activation rows of K elements
  int x_div;
  const uint16_t *scale;  // fp8: [e][R / 128] bf16
  const int *nU, *ulist, *ustart, *plist;
  float *out;             // [pairs][R]
};

template <int WD, int XD, int TG>
__device__ __forceinline__ void uf_group_pass(const UfGroup &a, const char *const (&wrow)[1], int r, int q, int nt,
                                              float sc) {
  const char *xr[TG];
  int pr[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    pr[t] = a.plist[q + min(t, nt - 1)];
    xr[t] = a.x + (size_t)(pr[t] / a.x_div) * a.K * dsz<XD>();
  }
  float acc[1][TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) acc[0][t] = 0.f;
  rows_dot<WD, XD, false, 1, 2, TG>(wrow, 0, a.K, xr, acc);
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const float v = wave_sum63(acc[0][t]) * sc;
    if (lane_id() == 63 && t < nt) a.out[(size_t)pr[t] * a.R + r] = v;
  }
}

template <int WD, int XD>
__global__ void __launch_bounds__(kUfThreads) uf_group_gemv(UfGroup a) {
  const int r = blockIdx.x * kUfRows + wave_id(), u = blockIdx.y;
  if (r >= a.R || u >= *a.nU) return;
  const int m = a.ulist[u], q0 = a.ustart[u], q1 = a.ustart[u + 1];
  const char *const wrow[1] = {a.w + (size_t)m * a.mat_bytes + (size_t)r * a.K * dsz<WD>()};
  float sc = 1.f;
  if constexpr (WD == DT_FP8) sc = __uint_as_float((uint32_t)a.scale[(size_t)m * (a.R / 128) + r / 128] << 16);
  for (int q = q0; q < q1; q += 4) {
    const int nt = min(4, q1 - q);
    if (nt == 1) uf_group_pass<WD, XD, 1>(a, wrow, r, q, nt, sc);
    else if (nt == 2) uf_group_pass<WD, XD, 2>(a, wrow, r, q, nt, sc);
    else uf_group_pass<WD, XD, 4>(a, wrow, r, q, nt, sc);
  }
}

// h[j][i] = act(SiLU(g) u) from the gate/up outputs gu[j] = (g[0..I), u[0..I))
template <int AD>
__global__ void __launch_bounds__(kUfThreads) uf_silu_mul(const float *gu, int I, int J, void *h) {
  const size_t n = (size_t)J * I;
  for (size_t q = (size_t)blockIdx.x * kUfThreads + threadIdx.x; q < n; q += (size_t)gridDim.x * kUfThreads) {
    const size_t j = q / I, i = q % I;
    store_act<AD>(h, q, silu_mul(gu[j * 2 * I + i], gu[j * 2 * I + I + i]));
  }
}

// y[t][h] = act(x + s + sum_i w[t][i] d[t k + i][h]) (s: shared expert or NULL)
template <int AD>
__global__ void __launch_bounds__(kUfThreads) uf_combine(const void *x, const float *s, const float *d,
                                                          const float *w, int H, int k, int B, void *y) {
  const size_t n = (size_t)B * H;
  for (size_t q = (size_t)blockIdx.x * kUfThreads + threadIdx.x; q < n; q += (size_t)gridDim.x * kUfThreads) {
    const size_t t = q / H, h = q % H;
    float rt = 0.f;
    for (int i = 0; i < k; ++i) rt = fmaf(w[t * k + i], d[(t * k + i) * H + h], rt);
    store_act<AD>(y, q, load_act<AD>(x, q) + (s ? s[q] : 0.f) + rt);
  }
}

// Side-stream prefetch of the next layer's dense weights (router, shared
// gate/up, shared down): ordinary (cache-allocating) 16-byte loads over each
// range, two in flight per lane, so that the lines are in the memory-side
// cache when the next layer streams them. The loaded words are folded into
// one value that is stored only if it equals a constant, which keeps the
// loads without writing anything in practice.
struct UfPrefetch {
  const u32x4 *p[3];
  size_t n16[3];
  unsigned *sink;
};

__global__ void __launch_bounds__(kUfThreads) uf_prefetch(UfPrefetch a) {
  const size_t stride = (size_t)gridDim.x * kUfThreads;
  unsigned acc = 0;
  for (int r = 0; r < 3; ++r) {
    const u32x4 *q = a.p[r];
    const size_t n = a.n16[r];
    size_t i = (size_t)blockIdx.x * kUfThreads + threadIdx.x;
    for (; i + stride < n; i += 2 * stride) {
      const u32x4 v0 = q[i], v1 = q[i + stride];
      acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    }
    if (i < n) {
      const u32x4 v = q[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == 0x9E3779B9u) a.sink[0] = acc;
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

// Per-device facts and launch preparation, filled on first use and then
// only read: the compute-unit count, the LDS limit, and for each kernel the
// largest dynamic LDS size for which its attribute is set and one resident
// workgroup per CU has been checked. One mutex guards it (calls are
// thread-safe); a call after the first takes it once and makes no HIP query.
constexpr int kMaxDevices = 64;
constexpr int kMaxKernels = 64;

struct KernelReady {
  const void *fn;
  size_t lds;
};

struct DevInfo {
  int cus = 0;
  int max_lds = 0;
  int nk = 0;
  KernelReady ready[kMaxKernels];
  hipEvent_t fork = nullptr, join = nullptr;  // cross-stream ordering of the side-stream variants
};

DevInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once set up

// every in-kernel wait gives up after this many ticks of the 100 MHz realtime counter
constexpr long long kDefaultWatchdogTicks = 200000000LL;  // 2 s
std::atomic<long long> g_watchdog_ticks{kDefaultWatchdogTicks};

#ifdef MOE_DEBUG_DELAY
// ordering-stress build: delay seed (0 = none) and grid size (0 = one workgroup per CU)
std::atomic<unsigned long long> g_dbg_seed{0};
std::atomic<int> g_dbg_grid{0};

int gcd_int(int a, int b) { while (b) { const int t = a % b; a = b; b = t; } return a; }
#endif

moe_status current_device(int &dev) {
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_DEVICE, "hipGetDevice failed");
  return MOE_OK;
}

moe_status device_info(int dev, int &cus, int &max_lds) {
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DevInfo &di = g_dev[dev];
  if (di.cus == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed");
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 65536;
    di.max_lds = lds;
    di.cus = prop.multiProcessorCount;
  }
  cus = di.cus;
  max_lds = di.max_lds;
  return MOE_OK;
}

// Set kernel fn's dynamic LDS limit to at least lds bytes and check that a
// workgroup of it fits on a CU (the persistent grid needs one per CU), once
// per (device, kernel, larger LDS size).
moe_status prepare_kernel(int dev, const void *fn, int threads, size_t lds) {
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DevInfo &di = g_dev[dev];
  int i = 0;
  while (i < di.nk && di.ready[i].fn != fn) ++i;
  if (i < di.nk && lds <= di.ready[i].lds) return MOE_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return fail(MOE_ERR_DEVICE, "hipFuncSetAttribute(%zu bytes of LDS) failed", lds);
  int resident = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, fn, threads, lds) != hipSuccess || resident < 1)
    return fail(MOE_ERR_DEVICE, "a %d-thread workgroup with %zu bytes of LDS cannot be resident", threads, lds);
  if (i == di.nk) {
    if (di.nk == kMaxKernels) return MOE_OK;  // not cached: checked again next time
    di.ready[di.nk++] = KernelReady{fn, lds};
  } else {
    di.ready[i].lds = lds;
  }
  return MOE_OK;
}

bool aligned16(const void *q) { return ((uintptr_t)q & 15u) == 0; }

int dsize(moe_dtype d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

moe_status check_desc(const moe_layer_desc *d) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->expert_inter <= 0 || d->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "non-positive size in desc");
  if (!(d->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARGUMENT, "rms_eps must be >= 0");
  if (d->hidden % 128 || d->hidden > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: need a multiple of 128, at most 16384", d->hidden);
  if (d->expert_inter % 128 || d->expert_inter > 4096)
    return fail(MOE_ERR_UNSUPPORTED, "expert_inter=%d: need a multiple of 128, at most 4096", d->expert_inter);
  if (d->shared_inter % 128 || d->shared_inter > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "shared_inter=%d: need 0 or a multiple of 128, at most 8192",
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

// column blocks of the shared down projection: width I, the last one partial
int shared_blocks(const moe_layer_desc *d) { return (d->shared_inter + d->expert_inter - 1) / d->expert_inter; }

struct WsLayout {
  size_t rlog, xhat, xa, rfin, hsh32, hbuf, hsbuf, partbuf, rpart, xbuf0, xbuf1, total;
};

size_t up256(size_t v) { return (v + 255u) & ~(size_t)255u; }

WsLayout ws_layout(const moe_layer_desc *d, int B, int L) {
  WsLayout w{};
  w.rlog = kRlogOffset;
  size_t off = up256(kRlogOffset + kRlogBytes);
  const size_t act = (size_t)dsize(d->act);
  const size_t is = (size_t)(d->shared_inter > 0 ? d->shared_inter : 1);
  w.xhat = off; off += up256((size_t)B * d->hidden * 4);
  w.xa = off; off += up256((size_t)B * d->hidden * act);
  w.rfin = off; off += up256((size_t)B * d->num_experts * 4);
  w.hsh32 = off; off += up256((size_t)B * is * 4);
  w.hbuf = off; off += up256((size_t)B * d->top_k * d->expert_inter * act);
  w.hsbuf = off; off += up256((size_t)B * is * act);
  const size_t pstride = (size_t)B * d->top_k + (size_t)B * shared_blocks(d);
  w.partbuf = off; off += up256((size_t)d->hidden * pstride * 4);
  // router partial logits of the MFMA tiles' K parts (batches that use them)
  w.rpart = off; off += (B >= kMfmaSharedMin) ? up256((size_t)kMaxRQ * B * d->num_experts * 4) : 0;
  w.xbuf0 = off; off += (L > 1) ? up256((size_t)B * d->hidden * act) : 0;
  w.xbuf1 = off; off += (L > 2) ? up256((size_t)B * d->hidden * act) : 0;
  w.total = off;
  return w;
}

typedef void (*kernel_fn)(Params);

template <bool S, bool M>
kernel_fn pick_kernel_t(const moe_layer_desc *d) {
  if (d->expert == MOE_BF16)
    return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_BF16, DT_BF16, S, M>
                                : moe_kernel<DT_BF16, DT_BF16, DT_BF16, DT_BF16, S, M>;
  return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_FP8, DT_BF16, S, M>
                              : moe_kernel<DT_BF16, DT_BF16, DT_FP8, DT_BF16, S, M>;
}

// msh: the shared expert on MFMA tiles (general regime, bf16 activations only)
kernel_fn pick_kernel(const moe_layer_desc *d, bool small, bool msh) {
  if (d->act == MOE_F32)
    return small ? moe_kernel<DT_F32, DT_F32, DT_F32, DT_F32, true, false>
                 : moe_kernel<DT_F32, DT_F32, DT_F32, DT_F32, false, false>;
  return small ? pick_kernel_t<true, false>(d) : msh ? pick_kernel_t<false, true>(d) : pick_kernel_t<false, false>(d);
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

// The device address of this device's copy of `scratch`; on the first call
// on a device (with it current) the symbol's address is looked up and a fill
// kernel on `stream` zeroes its control words and logit buffers.
moe_status static_workspace(int dev, void *stream, void *&ws) {
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    const unsigned words = (unsigned)((kRlogOffset + kRlogBytes) / sizeof(unsigned));
    hipLaunchKernelGGL(zero_words, dim3((words + 255u) / 256u), dim3(256), 0, (hipStream_t)stream, (unsigned *)ptr,
                       words);
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return fail(MOE_ERR_DEVICE, "clearing the static workspace failed: %s", hipGetErrorString(e2));
    g_scratch_ptr[dev] = ptr;
  }
  ws = g_scratch_ptr[dev];
  return MOE_OK;
}

// static_ws: the workspace is the library's `scratch` (ws must be NULL)
moe_status launch(const moe_layer_desc *d, const moe_layer_weights *layers, int L, const void *x, void *y, int B,
                  int32_t *idx, float *wts, float *logits, void *ws, size_t ws_bytes, void *stream, bool route_only,
                  bool static_ws = false) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (B < 1 || B > kMaxB) return fail(MOE_ERR_UNSUPPORTED, "batch %d outside 1..64", B);
  if (L < 1 || L > kMaxL) return fail(MOE_ERR_UNSUPPORTED, "layers %d outside 1..8", L);
  if (!layers) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  for (int l = 0; l < L; ++l)
    if ((st = check_weights(d, &layers[l])) != MOE_OK) return st;
  if (!x || (!static_ws && !ws) || (!route_only && !y))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x, y or workspace is NULL");
  if (route_only && (!idx || !wts)) return fail(MOE_ERR_INVALID_ARGUMENT, "topk_idx or topk_w is NULL");
  const void *ptrs[] = {x, y, idx, wts, logits, ws};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer %p is not 16-byte aligned", q);
  const size_t xbytes = (size_t)B * d->hidden * dsize(d->act);
  if (y && y != x && overlap(x, xbytes, y, xbytes)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and y partially overlap");
  const WsLayout wl = ws_layout(d, B, L);
  if (static_ws) {
    if (wl.total > kScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED, "this shape and batch need %zu bytes of workspace; the static workspace holds %zu",
                  wl.total, kScratchBytes);
  } else {
    if (ws_bytes < wl.total)
      return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, wl.total);
    if (overlap(ws, wl.total, x, xbytes) || (y && overlap(ws, wl.total, y, xbytes)))
      return fail(MOE_ERR_INVALID_ARGUMENT, "workspace overlaps x or y");
  }

  int dev = 0, cus = 0, max_lds = 0;
  if ((st = current_device(dev)) != MOE_OK || (st = device_info(dev, cus, max_lds)) != MOE_OK) return st;
  if (static_ws) {
    if ((st = static_workspace(dev, stream, ws)) != MOE_OK) return st;
    ws_bytes = kScratchBytes;
  }
  Params p;
  memset(&p, 0, sizeof p);
  p.H = d->hidden; p.E = d->num_experts; p.k = d->top_k; p.I = d->expert_inter; p.Is = d->shared_inter;
  p.B = B; p.L = L; p.route_only = route_only ? 1 : 0; p.eps = d->rms_eps;
  p.nsh = shared_blocks(d);
  p.G = cus;
  if (p.G < 1) return fail(MOE_ERR_DEVICE, "device reports no compute units");
  p.perm_a = 1;
  p.perm_c = 0;
  p.self_reset = static_ws ? 1 : 0;
#ifdef MOE_DEBUG_DELAY
  {
    const int grid = g_dbg_grid.load(std::memory_order_relaxed);
    if (grid > 0 && grid < p.G) p.G = grid;  // fewer workgroups than CUs: still all resident
    const unsigned long long seed = g_dbg_seed.load(std::memory_order_relaxed);
    p.dbg_seed = seed;
    if (seed != 0 && p.G > 1) {
      int a = (int)(((seed >> 17) * 2 + 1) % (unsigned long long)p.G);  // odd start, then the next unit mod G
      if (a < 1) a = 1;
      while (gcd_int(a, p.G) != 1) a = a % p.G + 1;
      p.perm_a = a;
      p.perm_c = (int)(seed % (unsigned long long)p.G);
    }
  }
#endif
  // the regime: B <= kSmallB with B * k <= 64 (one wave routes the batch and
  // builds the gather tables) keeps x-hat in every workgroup's LDS when it
  // fits; otherwise (or for larger B) the general regime
  bool small = small_regime(B) && B * d->top_k <= 64;
  p.rx32 = d->act == MOE_BF16 ? 1 : 0;  // first try: the router's fp32 x-hat in LDS (bf16 activations)
  size_t lds = 0;
  const size_t lds_cap = (size_t)(max_lds > 0 ? max_lds : 65536);
  for (;;) {
    // P2 output rows per workgroup, a multiple of the GEMV row block
    int rpw = (p.H + p.G - 1) / p.G;
    rpw = (rpw + kRowBlock - 1) / kRowBlock * kRowBlock;
    p.rows_per_wg = rpw;
    p.NSR = k_slices(d->hidden, d->router, 4);
    // general regime, bf16: the router and the shared expert on MFMA tiles
    // from kMfmaSharedMin tokens, when every workgroup owns at least 16 output
    // rows (a 16-row down tile over fewer rows would leave most lanes idle).
    p.mfma_sh = (!small && !route_only && d->act == MOE_BF16 && d->shared_inter > 0 && B >= kMfmaSharedMin &&
                 rpw >= 16)
                    ? 1
                    : 0;
    p.NSS = (d->shared_inter > 0 && !p.mfma_sh) ? k_slices(d->hidden, d->shared, 2) : 1;
    // K parts per router MFMA tile: as many as the grid holds one unit each (at most kMaxRQ)
    {
      const int ntr = (d->num_experts + 15) / 16;
      p.rq = p.mfma_sh ? std::max(1, std::min(kMaxRQ, p.G / ntr)) : 1;
    }
    // general regime: a workgroup's P2 rows follow its P1 tasks, so extra
    // groups mostly add barrier waits; 2 measured best up to 16 tokens, 3 above
    p.p1_groups = std::min(kP1Groups, B <= 16 ? 2 : 3);
    // P1 tail stealing: bf16 experts (fp8 tasks are half as long, and the
    // workspace atomics measured a little slower there)
    p.steal = (!small && !route_only && MOE_P1_STEAL > 0 && p.G <= kMaxStealG && d->expert == MOE_BF16) ? 1 : 0;
    // the stealable tail: a quarter of a share up to 16 tokens, a third above
    // (where a share holds fewer, longer MFMA tiles)
    p.tail_div = B <= 16 ? 4 : 3;
    // the slices of a row are one workgroup's waves of one round: the shared
    // tasks start at a multiple of the workgroup's wave count, and the rounds
    // must fit the per-round slice counters and LDS slots (else every row is
    // one slice)
    const int NW = p.G * kWaves;
    int rounds = 0;
    auto plan_slices = [&]() {
      p.s0 = (p.E * p.NSR + kWaves - 1) / kWaves * kWaves;
      p.slw = p.NSS > 1 ? 2 * B : B;
      const int ntask = p.mfma_sh ? 0 : p.s0 + p.Is * p.NSS;
      p.p0_end = ntask;
      p.p0r = (ntask + NW - 1) / NW;
      // last round: as few waves per workgroup as cover the tasks left, a
      // multiple of the slice counts of the rows in that round
      const int left = ntask - (p.p0r - 1) * NW;
      const int unit = (p.p0r - 1) * NW >= p.E * p.NSR ? p.NSS : (p.NSR > p.NSS ? p.NSR : p.NSS);
      p.p0w = ((left + p.G - 1) / p.G + unit - 1) / unit * unit;
      if (p.p0w > kWaves) p.p0w = kWaves;
      rounds = (p.NSR > 1 || p.NSS > 1) ? p.p0r : 0;
      if (ntask == 0) p.p0r = p.p0w = rounds = 0;
    };
    plan_slices();
    if (rounds > kMaxRounds || (size_t)rounds * kWaves * p.slw * sizeof(float) > 16384) {
      p.NSR = p.NSS = 1;
      plan_slices();
    }

    // LDS carve-up
    const int E = d->num_experts, P = B * d->top_k, H = d->hidden;
    const int nsh = shared_blocks(d);
    const int nslot = P < E ? P : E;
    const size_t act = (size_t)dsize(d->act);
    size_t o = align16(sizeof(SmemHead));
    p.o_sel_idx = (int)o; o = align16(o + (size_t)P * 4);
    p.o_sel_w = (int)o; o = align16(o + (size_t)P * 4);
    p.o_ulist = (int)o; o = align16(o + (size_t)nslot * 4);
    p.o_ucnt = (int)o; o = align16(o + (size_t)nslot * 4);
    p.o_ustart = (int)o; o = align16(o + (size_t)nslot * 4);
    p.o_plist = (int)o; o = align16(o + (size_t)P * 4);
    // top-k candidate slots of 1 KB: one per routing wave
    // (small regime: the one routing wave; its route-only launch: one wave per token)
    p.o_cand = (int)o; o = align16(o + (size_t)(small ? (route_only ? B : 1) : kWaves) * 4 * 64 * sizeof(unsigned));
    if (small) {
      if (d->act == MOE_F32) {
        p.o_xf = (int)o; o = align16(o + (size_t)B * H * 4);
      } else if (p.rx32) {
        p.o_xf = (int)o; o = align16(o + (size_t)B * H * 4);
        p.o_xa = (int)o; o = align16(o + (size_t)B * H * act);
      } else {
        p.o_x = (int)o; o = align16(o + (size_t)B * H * act);
        p.o_xa = (int)o; o = align16(o + (size_t)B * H * act);
        p.o_g = (int)o; o = align16(o + (size_t)H * act);
      }
      p.o_hs = (int)o; o = align16(o + (size_t)B * (d->shared_inter > 0 ? d->shared_inter : 1) * act);
    } else {
      p.o_cnt = (int)o; o = align16(o + (size_t)E * 4);
      p.o_start = (int)o; o = align16(o + (size_t)E * 4);
      p.o_tmask = (int)o; o = align16(o + (size_t)E * 8);
      p.o_mslot = (int)o; o = align16(o + (size_t)nslot * 4);
      p.o_gslot = (int)o; o = align16(o + (size_t)nslot * 4);
      p.o_cpre = (int)o; o = align16(o + (size_t)(nslot + 1) * 4);
    }
    p.o_slc = (int)o;
    o = align16(o + (size_t)rounds * kWaves * p.slw * sizeof(float));
    p.o_scnt = (int)o;
    o = align16(o + (size_t)2 * p.p0r * kWaves * sizeof(int));
    p.o_red = (int)o;
    if (p.mfma_sh) o = align16(o + (size_t)kWaves * 16 * B * sizeof(float));
    p.o_part = (int)o;
    // small regime: the workgroup's P2 partial sums stay in LDS (one pass over
    // its rows); general regime: they go to the workspace
    const size_t per_row = (size_t)(P + B * nsh) * sizeof(float);
    lds = small ? o + (size_t)rpw * per_row : o;
    p.mfma_min = (!small && d->expert != MOE_F32 && rpw >= 16) ? kMfmaMin : 0;
    if (lds <= lds_cap) break;
    if (!small) return fail(MOE_ERR_UNSUPPORTED, "shape needs more LDS than the device's %zu bytes", lds_cap);
    if (p.rx32) {  // the router's fp32 x-hat does not fit: form it from x, gamma and r instead
      p.rx32 = 0;
      continue;
    }
    // x-hat of every token does not fit a workgroup's LDS (H = 16384 at
    // B = 2, or the K3 share above B = 4): the general regime keeps it in
    // global memory instead
    small = false;
  }

  p.timeout_ticks = g_watchdog_ticks.load(std::memory_order_relaxed);
  unsigned char *wsb = (unsigned char *)ws;
  p.ctrl = (unsigned *)wsb;
  p.xhat = (float *)(wsb + wl.xhat);
  p.xa = (d->act == MOE_F32) ? (void *)p.xhat : (void *)(wsb + wl.xa);
  p.rfin = (float *)(wsb + wl.rfin);
  p.rlog = (float *)(wsb + wl.rlog);
  p.hsh32 = (float *)(wsb + wl.hsh32);
  p.hbuf = wsb + wl.hbuf;
  p.hsbuf = wsb + wl.hsbuf;
  p.partbuf = (float *)(wsb + wl.partbuf);
  p.rpart = (float *)(wsb + wl.rpart);
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
    lp.lg = (small && !route_only) ? p.rlog + (size_t)(l & 1) * kSmallB * d->num_experts : p.rfin;
  }
  kernel_fn fn = pick_kernel(d, small, p.mfma_sh != 0);
  // the grid is persistent: one resident workgroup per CU is required
  if ((st = prepare_kernel(dev, (const void *)fn, kThreads, lds)) != MOE_OK) return st;
  hipLaunchKernelGGL(fn, dim3(p.G), dim3(kThreads), lds, (hipStream_t)stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}


// workspace of the multi-launch path
struct UfLayout {
  size_t xf, xa, lg, idx, w, nu, ulist, ustart, plist, gu, h, d, sgu, hs, ds, sink, xbuf0, xbuf1, total;
};

// L > 1: the layer outputs between layers alternate between two [B][H] buffers
UfLayout uf_layout(const moe_layer_desc *d, int B, int L = 1) {
  UfLayout u{};
  const size_t act = (size_t)dsize(d->act), H = (size_t)d->hidden, P = (size_t)B * d->top_k;
  const size_t I = (size_t)d->expert_inter, Is = (size_t)d->shared_inter;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up256(bytes > 0 ? bytes : 1); return o; };
  u.xf = take((size_t)B * H * 4);
  u.xa = take((size_t)B * H * act);
  u.lg = take((size_t)B * d->num_experts * 4);
  u.idx = take(P * 4);
  u.w = take(P * 4);
  const size_t nslot = std::min(P, (size_t)d->num_experts);
  u.nu = take(4);
  u.ulist = take(nslot * 4);
  u.ustart = take((nslot + 1) * 4);
  u.plist = take(P * 4);
  u.gu = take(P * 2 * I * 4);
  u.h = take(P * I * act);
  u.d = take(P * H * 4);
  u.sgu = take((size_t)B * 2 * Is * 4);
  u.hs = take((size_t)B * Is * act);
  u.ds = take((size_t)B * H * 4);
  u.sink = take(4);
  if (L > 1) {
    u.xbuf0 = take((size_t)B * H * act);
    u.xbuf1 = take((size_t)B * H * act);
  }
  u.total = off;
  return u;
}

unsigned uf_blocks(size_t n) { return (unsigned)std::min<size_t>((n + kUfThreads - 1) / kUfThreads, 8192); }

#ifndef MOE_UF_PREFETCH_BLOCKS
#define MOE_UF_PREFETCH_BLOCKS 64  // workgroups of the side-stream prefetch (a quarter of the CUs)
#endif

// Work of a layer on the side stream of the multi-launch path.
struct UfSide {
  hipStream_t ss = nullptr;      // the side stream
  hipEvent_t fork = nullptr;     // recorded on the main stream after the RMSNorm; ss waits for it
  hipEvent_t join = nullptr;     // recorded on ss after the shared expert; the main stream waits before the combine
  bool shared = false;           // the shared expert's three launches run on ss
  const UfPrefetch *pf = nullptr;  // a prefetch launched on ss after them, or none
};

// The eleven launches of one layer on stream st; the shared expert and a
// prefetch of other weights optionally on a side stream (UfSide), concurrent
// with the routed path. Returns the first error of the event calls (launch
// errors are read with hipGetLastError).
template <int AD, int RD, int ED, int SD>
hipError_t uf_launch_all(const moe_layer_desc *d, const moe_layer_weights *wt, const void *x, void *y, int B,
                   int32_t *idx, float *wts, unsigned char *ws, const UfLayout &u, hipStream_t st,
                   const UfSide &sd = UfSide{}) {
  const int H = d->hidden, E = d->num_experts, k = d->top_k, I = d->expert_inter, Is = d->shared_inter;
  const int P = B * k;
  float *xf = (float *)(ws + u.xf);
  void *xa = AD == DT_F32 ? (void *)xf : (void *)(ws + u.xa);
  float *lg = (float *)(ws + u.lg), *gu = (float *)(ws + u.gu), *dd = (float *)(ws + u.d);
  float *sgu = (float *)(ws + u.sgu), *ds = (float *)(ws + u.ds);
  void *h = ws + u.h, *hs = ws + u.hs;
  const dim3 blk(kUfThreads);
  // 1. RMSNorm
  hipLaunchKernelGGL(uf_rmsnorm<AD>, dim3(B), dim3(kThreads), 0, st, x, wt->rms_gamma, H, d->rms_eps, xf, xa);
  // 8.-10. shared expert: gate/up, SiLU * mul, down
  auto shared_expert = [&](hipStream_t s) {
    UfGemv a{};
    a.w = (const char *)wt->shared_gate_up; a.R = 2 * Is; a.K = H; a.x = (const char *)xa; a.x_div = 1; a.nx = B;
    a.out = sgu;
    hipLaunchKernelGGL((uf_gemv<SD, AD, 1>), dim3((2 * Is + kUfRows - 1) / kUfRows, B), blk, 0, s, a);
    hipLaunchKernelGGL(uf_silu_mul<AD>, dim3(uf_blocks((size_t)B * Is)), blk, 0, s, (const float *)sgu, Is, B, hs);
    a = UfGemv{};
    a.w = (const char *)wt->shared_down; a.R = H; a.K = Is; a.x = (const char *)hs; a.x_div = 1; a.nx = B;
    a.out = ds;
    hipLaunchKernelGGL((uf_gemv<SD, AD, 1>), dim3((H + kUfRows - 1) / kUfRows, B), blk, 0, s, a);
  };
  const bool side = sd.shared && Is > 0;
  hipError_t er = hipSuccess;
  auto keep = [&](hipError_t e) { if (er == hipSuccess) er = e; };
  if (side || sd.pf) {
    keep(hipEventRecord(sd.fork, st));
    keep(hipStreamWaitEvent(sd.ss, sd.fork, 0));
    if (side) {
      shared_expert(sd.ss);
      keep(hipEventRecord(sd.join, sd.ss));
    }
    if (sd.pf) hipLaunchKernelGGL(uf_prefetch, dim3(MOE_UF_PREFETCH_BLOCKS), dim3(kUfThreads), 0, sd.ss, *sd.pf);
  }
  // 2. router: one weight row per wave for up to 4 tokens
  UfGemv a{};
  a.w = (const char *)wt->router_w; a.R = E; a.K = H; a.x = (const char *)xf; a.x_div = 1; a.nx = B;
  a.bias = wt->router_bias; a.out = lg;
  if (B > 1) hipLaunchKernelGGL((uf_gemv<RD, DT_F32, 4>), dim3((E + kUfRows - 1) / kUfRows, (B + 3) / 4), blk, 0, st, a);
  else hipLaunchKernelGGL((uf_gemv<RD, DT_F32, 1>), dim3((E + kUfRows - 1) / kUfRows, 1), blk, 0, st, a);
  // 3. top-k + softmax
  hipLaunchKernelGGL(uf_topk, dim3(B), dim3(64), 0, st, (const float *)lg, E, k, idx, wts);
  // 4. expert grouping: union of selected experts, each expert's pairs
  int *nU = (int *)(ws + u.nu), *ulist = (int *)(ws + u.ulist), *ustart = (int *)(ws + u.ustart);
  int *plist = (int *)(ws + u.plist);
  const int nslot = std::min(P, E);
  hipLaunchKernelGGL(uf_align, dim3(1), dim3(kThreads), 0, st, (const int32_t *)idx, P, E, nU, ulist, ustart, plist);
  // 5. expert gate/up, each selected expert's rows read once for its tokens
  UfGroup g{};
  g.w = (const char *)wt->expert_gate_up; g.mat_bytes = (size_t)2 * I * H * dsize(d->expert);
  g.R = 2 * I; g.K = H; g.x = (const char *)xa; g.x_div = k;
  g.scale = (const uint16_t *)wt->expert_gate_up_scale;
  g.nU = nU; g.ulist = ulist; g.ustart = ustart; g.plist = plist; g.out = gu;
  hipLaunchKernelGGL((uf_group_gemv<ED, AD>), dim3((2 * I + kUfRows - 1) / kUfRows, nslot), blk, 0, st, g);
  // 6. SiLU * mul
  hipLaunchKernelGGL(uf_silu_mul<AD>, dim3(uf_blocks((size_t)P * I)), blk, 0, st, (const float *)gu, I, P, h);
  // 7. expert down, grouped the same way
  g.w = (const char *)wt->expert_down; g.mat_bytes = (size_t)H * I * dsize(d->expert);
  g.R = H; g.K = I; g.x = (const char *)h; g.x_div = 1;
  g.scale = (const uint16_t *)wt->expert_down_scale; g.out = dd;
  hipLaunchKernelGGL((uf_group_gemv<ED, AD>), dim3((H + kUfRows - 1) / kUfRows, nslot), blk, 0, st, g);
  if (side) keep(hipStreamWaitEvent(st, sd.join, 0));
  else if (Is > 0) shared_expert(st);
  // 11. weighted combine + residual
  hipLaunchKernelGGL(uf_combine<AD>, dim3(uf_blocks((size_t)B * H)), blk, 0, st, x, Is > 0 ? (const float *)ds : nullptr,
                     (const float *)dd, (const float *)wts, H, k, B, y);
  return er;
}

// Dense weights of a layer that the side-stream prefetch reads: router, shared gate/up, shared down.
UfPrefetch uf_prefetch_args(const moe_layer_desc *d, const moe_layer_weights *wt, unsigned *sink) {
  const size_t H = (size_t)d->hidden, Is = (size_t)d->shared_inter;
  UfPrefetch a{};
  a.p[0] = (const u32x4 *)wt->router_w;
  a.n16[0] = (size_t)d->num_experts * H * dsize(d->router) / 16;
  a.p[1] = (const u32x4 *)wt->shared_gate_up;
  a.n16[1] = Is > 0 ? 2 * Is * H * dsize(d->shared) / 16 : 0;
  a.p[2] = (const u32x4 *)wt->shared_down;
  a.n16[2] = Is > 0 ? H * Is * dsize(d->shared) / 16 : 0;
  a.sink = sink;
  return a;
}

// L layers through the multi-launch path: layer l reads x (l = 0) or the
// previous layer's output in the workspace and writes y (l = L - 1) or the
// other workspace buffer. flags: MOE_UF_SHARED_SIDE puts each layer's shared
// expert on `side`; MOE_UF_PREFETCH_SIDE launches on `side`, once layer l's
// RMSNorm is done (and after its shared expert if that is there too), a
// prefetch of layer l + 1's router and shared weights.
// Work on `side` is joined back into `stream` before the call's last launch
// ends, so `stream` alone orders everything the call enqueued.
moe_status launch_unfused(const moe_layer_desc *d, const moe_layer_weights *layers, int L, const void *x, void *y,
                          int B, int32_t *idx, float *wts, void *ws, size_t ws_bytes, void *stream, void *side,
                          unsigned flags) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (B < 1 || B > kMaxB) return fail(MOE_ERR_UNSUPPORTED, "batch %d outside 1..64", B);
  if (!layers) return fail(MOE_ERR_INVALID_ARGUMENT, "layers is NULL");
  if (L < 1 || L > kMaxL) return fail(MOE_ERR_UNSUPPORTED, "%d layers outside 1..%d", L, kMaxL);
  if (flags & ~(unsigned)(MOE_UF_SHARED_SIDE | MOE_UF_PREFETCH_SIDE))
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
  if (flags && !side) return fail(MOE_ERR_INVALID_ARGUMENT, "side-stream flags need a side stream");
  for (int l = 0; l < L; ++l)
    if ((st = check_weights(d, &layers[l])) != MOE_OK) return st;
  if (!x || !y || !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "x, y or workspace is NULL");
  const void *ptrs[] = {x, y, idx, wts, ws};
  for (const void *q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer %p is not 16-byte aligned", q);
  const size_t xbytes = (size_t)B * d->hidden * dsize(d->act);
  if (y != x && overlap(x, xbytes, y, xbytes)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and y partially overlap");
  const UfLayout u = uf_layout(d, B, L);
  if (ws_bytes < u.total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, u.total);
  if (overlap(ws, u.total, x, xbytes) || overlap(ws, u.total, y, xbytes))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace overlaps x or y");
  unsigned char *wsb = (unsigned char *)ws;
  const int P = B * d->top_k;
  const hipStream_t s = (hipStream_t)stream, ss = (hipStream_t)side;
  hipEvent_t fork = nullptr, join = nullptr;
  std::unique_lock<std::mutex> order;  // one call at a time records and waits on the device's two events
  if (flags) {
    int dev = 0;
    if ((st = current_device(dev)) != MOE_OK) return st;
    std::unique_lock<std::mutex> lock(g_dev_mu);
    DevInfo &di = g_dev[dev];
    if (!di.fork && hipEventCreateWithFlags(&di.fork, hipEventDisableTiming) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "hipEventCreateWithFlags failed");
    if (!di.join && hipEventCreateWithFlags(&di.join, hipEventDisableTiming) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "hipEventCreateWithFlags failed");
    fork = di.fork;
    join = di.join;
    order = std::move(lock);
  }
  for (int l = 0; l < L; ++l) {
    const moe_layer_weights *wt = &layers[l];
    const void *xl = l == 0 ? x : (const void *)(wsb + ((l - 1) % 2 ? u.xbuf1 : u.xbuf0));
    void *yl = l == L - 1 ? y : (void *)(wsb + (l % 2 ? u.xbuf1 : u.xbuf0));
    int32_t *il = idx ? idx + (size_t)l * P : (int32_t *)(wsb + u.idx);
    float *wl = wts ? wts + (size_t)l * P : (float *)(wsb + u.w);
    UfSide sd;
    UfPrefetch pf;
    sd.ss = ss;
    sd.fork = fork;
    sd.join = join;
    sd.shared = (flags & MOE_UF_SHARED_SIDE) != 0;
    if ((flags & MOE_UF_PREFETCH_SIDE) && l + 1 < L) {
      pf = uf_prefetch_args(d, &layers[l + 1], (unsigned *)(wsb + u.sink));
      sd.pf = &pf;
    }
    hipError_t er;
    if (d->act == MOE_F32) {
      er = uf_launch_all<DT_F32, DT_F32, DT_F32, DT_F32>(d, wt, xl, yl, B, il, wl, wsb, u, s, sd);
    } else if (d->expert == MOE_BF16) {
      if (d->router == MOE_F32) er = uf_launch_all<DT_BF16, DT_F32, DT_BF16, DT_BF16>(d, wt, xl, yl, B, il, wl, wsb, u, s, sd);
      else er = uf_launch_all<DT_BF16, DT_BF16, DT_BF16, DT_BF16>(d, wt, xl, yl, B, il, wl, wsb, u, s, sd);
    } else {
      if (d->router == MOE_F32) er = uf_launch_all<DT_BF16, DT_F32, DT_FP8, DT_BF16>(d, wt, xl, yl, B, il, wl, wsb, u, s, sd);
      else er = uf_launch_all<DT_BF16, DT_BF16, DT_FP8, DT_BF16>(d, wt, xl, yl, B, il, wl, wsb, u, s, sd);
    }
    if (er != hipSuccess) return fail(MOE_ERR_DEVICE, "stream ordering failed: %s", hipGetErrorString(er));
  }
  if (flags) {
    hipError_t er = hipEventRecord(join, ss);
    if (er == hipSuccess) er = hipStreamWaitEvent(s, join, 0);
    if (er != hipSuccess) return fail(MOE_ERR_DEVICE, "stream ordering failed: %s", hipGetErrorString(er));
  }
  const hipError_t e = hipGetLastError();
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

moe_status moe_decode_layer_static(const moe_layer_desc *desc, const moe_layer_weights *weights, const void *x,
                                   void *y, int32_t B, int32_t *topk_idx, float *topk_w, void *stream) {
  return launch(desc, weights, 1, x, y, B, topk_idx, topk_w, nullptr, nullptr, 0, stream, false, true);
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
    // a stopped launch may have left small-batch logits behind: clear them
    if (ws_bytes >= kRlogOffset + kRlogBytes &&
        hipMemset((unsigned char *)ws + kRlogOffset, 0, kRlogBytes) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "clearing the logit buffers failed");
    return fail(MOE_ERR_TIMEOUT, "a launch on this workspace stopped at its barrier watchdog");
  }
  return MOE_OK;
}

size_t moe_unfused_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens) {
  if (check_desc(desc) != MOE_OK) return 0;
  if (max_tokens < 1 || max_tokens > kMaxB) return 0;
  return uf_layout(desc, max_tokens).total;
}

size_t moe_unfused_stack_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens, int32_t num_layers) {
  if (check_desc(desc) != MOE_OK) return 0;
  if (max_tokens < 1 || max_tokens > kMaxB || num_layers < 1 || num_layers > kMaxL) return 0;
  return uf_layout(desc, max_tokens, num_layers).total;
}

moe_status moe_decode_layer_unfused(const moe_layer_desc *desc, const moe_layer_weights *weights, const void *x,
                                    void *y, int32_t B, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                    void *stream) {
  return launch_unfused(desc, weights, 1, x, y, B, topk_idx, topk_w, ws, ws_bytes, stream, nullptr, 0);
}

moe_status moe_decode_stack_unfused(const moe_layer_desc *desc, const moe_layer_weights *layers, int32_t L,
                                    const void *x, void *y, int32_t B, int32_t *topk_idx, float *topk_w, void *ws,
                                    size_t ws_bytes, void *stream, void *side_stream, uint32_t flags) {
  return launch_unfused(desc, layers, L, x, y, B, topk_idx, topk_w, ws, ws_bytes, stream, side_stream, flags);
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

#ifdef MOE_DEBUG_DELAY
void moe_debug_set_delay(uint64_t seed, int32_t grid) {
  g_dbg_seed.store(seed, std::memory_order_relaxed);
  g_dbg_grid.store(grid < 0 ? 0 : grid, std::memory_order_relaxed);
}
#endif

void moe_set_watchdog_ticks(int64_t ticks) {
  g_watchdog_ticks.store(ticks < 0 ? kDefaultWatchdogTicks : (long long)ticks, std::memory_order_relaxed);
}

}  // extern "C"
