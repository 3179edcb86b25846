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
  float *rpart;           // [NSR][B][E]
  float *hspart;          // [NSS][B][2 Is] (small regime)
  void *hbuf;             // [B*k][I] act
  void *hsbuf;            // [B][Is] act (general regime)
  void *xbuf[2];          // [B][H] act, stack intermediates
  // LDS carve-up, byte offsets from the start of dynamic LDS
  int o_sel_idx, o_sel_w, o_cnt, o_start, o_tmask, o_ulist, o_plist;
  int o_xf, o_xa;         // small regime, P0-P1: x-hat fp32 / act [B][H]
  int o_hs, o_h;          // small regime, P2: shared h [B][Is], expert h [B*k][I] (act)
  int o_part;             // P2 partial sums [pass_rows][pstride] fp32
  LayerPtrs lp[kMaxL];
};

// fixed head of the dynamic LDS
struct SmemHead {
  int bar_cnt[kMaxBarriers];    // waves of this workgroup that arrived
  int bar_claim[kMaxBarriers];  // one wave polls the global counter
  int bar_flag[kMaxBarriers];   // raised once the barrier is passed
  float red[kWaves];
  int scan_tmp[2 * kWaves];
  int nU;
  unsigned sink;
};

// Kernel parameters are read in place from the kernarg segment (address space 4).
#define KARG __attribute__((address_space(4)))
typedef const KARG Params *KParams;
typedef const KARG LayerPtrs *KLayer;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// chunks per step of a gate/up pair (2 rows), sized to the register budget
template <int WD, int TG> constexpr int seg_gu() {
  return WD == DT_FP8 ? (TG <= 2 ? 7 : 3) : WD == DT_BF16 ? 7 : 4;
}
// chunks per step of a 4-row down unit
template <int WD, int TG> constexpr int seg_down() { return WD == DT_FP8 ? 1 : WD == DT_BF16 ? 2 : 2; }
// chunks per step of a router row slice
template <int WD, int TG> constexpr int seg_router() { return TG <= 2 ? 7 : 4; }

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

// Small regime: this workgroup normalises every token into its own LDS:
// xf [B][H] fp32 (router input) and xa [B][H] act (FFN input).
template <int AD>
__device__ __attribute__((noinline)) void stage_xhat(KParams p, KLayer lp, const Lds &L) {
  const int H = p->H, tid = threadIdx.x;
  SmemHead &sh = L.head();
  float *xf = L.at<float>(p->o_xf);
  for (int t = 0; t < p->B; ++t) {
    float ss = 0.f;
    for (int h = tid; h < H; h += kThreads) {
      const float v = load_act<AD>(lp->x, (size_t)t * H + h);
      ss = fmaf(v, v, ss);
    }
    ss = readlane_f(wave_sum63(ss), 63);
    if (lane_id() == 0) sh.red[wave_id()] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sh.red[w2];
    const float r = 1.0f / sqrtf(tot / (float)H + p->eps);
    for (int h = tid; h < H; h += kThreads) {
      const float xh = load_act<AD>(lp->x, (size_t)t * H + h) * r * load_act<AD>(lp->gamma, h);
      xf[(size_t)t * H + h] = xh;
      if constexpr (AD != DT_F32) store_act_lds<AD>(L.raw(p->o_xa), (size_t)t * H + h, xh);
    }
    __syncthreads();
  }
}

// General regime: workgroup t normalises token t into global memory.
template <int AD>
__device__ __attribute__((noinline)) void produce_xhat(KParams p, KLayer lp, const Lds &L) {
  const int H = p->H, tid = threadIdx.x;
  SmemHead &sh = L.head();
  for (int t = blockIdx.x; t < p->B; t += p->G) {
    float ss = 0.f;
    for (int h = tid; h < H; h += kThreads) {
      const float v = load_act<AD>(lp->x, (size_t)t * H + h);
      ss = fmaf(v, v, ss);
    }
    ss = readlane_f(wave_sum63(ss), 63);
    if (lane_id() == 0) sh.red[wave_id()] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sh.red[w2];
    const float r = 1.0f / sqrtf(tot / (float)H + p->eps);
    for (int h = tid; h < H; h += kThreads) {
      const float xh = load_act<AD>(lp->x, (size_t)t * H + h) * r * load_act<AD>(lp->gamma, h);
      p->xhat[(size_t)t * H + h] = xh;
      if constexpr (AD != DT_F32) store_act<AD>(p->xa, (size_t)t * H + h, xh);
    }
    __syncthreads();
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
      if (t < nt && lane_id() == 63) p->rpart[((size_t)s * B + t0 + t) * E + e] = v;
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
          hp[j] = g;
          hp[Is + j] = u;
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

__device__ __attribute__((noinline)) void topk_token(KParams p, KLayer lp, const Lds &L, int t, bool write_out) {
  const int lane = lane_id();
  const int E = p->E, k = p->k, B = p->B, NSR = p->NSR;
  constexpr int PER = kMaxE / 64;
  const float qnan = __builtin_nanf("");
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    float l = qnan;  // not an expert: never selected (NaN compares false)
    if (e < E) {
      float s = 0.f;
      for (int q = 0; q < NSR; ++q) s += p->rpart[((size_t)q * B + t) * E + e];
      if (lp->rb) s += lp->rb[e];
      l = (s == s) ? s : -INFINITY;  // a NaN logit ranks last but stays selectable
      if (write_out && lp->logits_out) lp->logits_out[(size_t)t * E + e] = l;
    }
    v[j] = l;
  }
  int *sel_idx = L.at<int>(p->o_sel_idx);
  float *sel_w = L.at<float>(p->o_sel_w);
  float lmax = 0.f, z = 0.f, selv = 0.f;
  int seli = 0;
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
    if (i == 0) lmax = bv;
    const float ex = expf(bv - lmax);
    z += ex;
    if (lane == i) { selv = ex; seli = bi; }
  }
  if (lane < k) {
    const float w = selv / z;
    sel_idx[t * k + lane] = seli;
    sel_w[t * k + lane] = w;
    if (write_out) {
      if (lp->idx_out) lp->idx_out[(size_t)t * k + lane] = seli;
      if (lp->w_out) lp->w_out[(size_t)t * k + lane] = w;
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
  __syncthreads();
}

// ---------------------------------------------------------------------------
// P1: expert gate/up, task (expert u of U, pair j)

template <int AD, int ED, bool XL>
__device__ __forceinline__ void expert_gu_task(KParams p, KLayer lp, const Lds &L, int u, int j) {
  const int H = p->H, I = p->I, k = p->k;
  const int *cnt = L.at<int>(p->o_cnt), *start = L.at<int>(p->o_start), *ulist = L.at<int>(p->o_ulist);
  const int *plist = L.at<int>(p->o_plist);
  const int e = ulist[u];
  const int n = cnt[e];
  const int *pl = plist + start[e];
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
      if (t < nt && lane_id() == 63) store_act<AD>(p->hbuf, (size_t)slot[t] * I + j, silu_mul(g, uu));
    }
  });
}

// ---------------------------------------------------------------------------
// P2: down projections of this workgroup's rows

// shared h for every token from the slice partials, into LDS (small regime)
template <int AD>
__device__ __attribute__((noinline)) void finish_shared_h(KParams p, const Lds &L) {
  const int Is = p->Is, B = p->B, NSS = p->NSS;
  lds_t *hs = L.raw(p->o_hs);
  for (int c = threadIdx.x; c < B * Is; c += kThreads) {
    const int t = c / Is, j = c % Is;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < NSS; ++s) {
      const float *hp = p->hspart + ((size_t)s * B + t) * 2 * Is;
      g += hp[j];
      u += hp[Is + j];
    }
    store_act_lds<AD>(hs, (size_t)t * Is + j, silu_mul(g, u));
  }
}

// expert h of every selected (token, expert) pair into LDS (small regime)
__device__ __attribute__((noinline)) void stage_h(KParams p, const Lds &L, int act_bytes) {
  const size_t n16 = (size_t)p->B * p->k * p->I * act_bytes / 16;
  const u32x4 *src = (const u32x4 *)p->hbuf;
  __attribute__((address_space(3))) u32x4 *dst = (__attribute__((address_space(3))) u32x4 *)L.raw(p->o_h);
  for (size_t i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
}

// One 4-row unit of a [rows][K] down matrix: row pointers wrow, columns
// [0, I) of x rows xr (TG tokens); writes the row sums times sc[r] to
// part[(o0 + r - pr0) * pstride + col[t]].
template <int WD, int AD, bool XL, int TG>
__device__ __forceinline__ void down_unit(const char *const (&wrow)[kRowBlock], int I,
                                          const typename XSrc<XL>::ptr (&xr)[TG], const float (&sc)[kRowBlock],
                                          float *prow, int pstride, const int (&col)[TG], int nt) {
  float acc[kRowBlock][TG];
#pragma unroll
  for (int r = 0; r < kRowBlock; ++r)
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[r][t] = 0.f;
  rows_dot<WD, AD, XL, kRowBlock, seg_down<WD, TG>(), TG>(wrow, 0, I, xr, acc);
#pragma unroll
  for (int r = 0; r < kRowBlock; ++r)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float v = wave_sum63(acc[r][t]) * sc[r];
      if (t < nt && lane_id() == 63) prow[r * pstride + col[t]] = v;
    }
}

// shared-expert units of rows [pr0, pr1): (row block, column block hf)
template <int AD, int SD, bool XL>
__device__ __forceinline__ void shared_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int w0) {
  const int I = p->I, Is = p->Is, B = p->B;
  const int nsh = Is / I, P = B * p->k, pstride = P + B * nsh;
  const int nrb = (pr1 - pr0) / kRowBlock;
  float *part = L.at<float>(p->o_part);
  const float one[kRowBlock] = {1.f, 1.f, 1.f, 1.f};
  for (int un = (wave_id() + kWaves - w0 % kWaves) % kWaves; un < nrb * nsh; un += kWaves) {
    const int rb = un / nsh, hf = un % nsh;
    const int o0 = pr0 + rb * kRowBlock;
    const char *wrow[kRowBlock];
#pragma unroll
    for (int r = 0; r < kRowBlock; ++r)
      wrow[r] = (const char *)lp->sd + ((size_t)(o0 + r) * Is + (size_t)hf * I) * dsz<SD>();
    for_token_groups(B, [&]<int TG>(int t0, int nt) {
      typename XSrc<XL>::ptr xr[TG];
      int col[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const int tt = t0 + (t < nt ? t : 0);
        if constexpr (XL) xr[t] = L.raw(p->o_hs) + ((size_t)tt * Is + (size_t)hf * I) * dsz<AD>();
        else xr[t] = (const char *)p->hsbuf + ((size_t)tt * Is + (size_t)hf * I) * dsz<AD>();
        col[t] = P + (t0 + t) * nsh + hf;
      }
      down_unit<SD, AD, XL, TG>(wrow, I, xr, one, part + (size_t)(o0 - pr0) * pstride, pstride, col, nt);
    });
  }
}

// routed-expert units of rows [pr0, pr1): (row block, expert slot)
template <int AD, int ED, bool XL>
__device__ __forceinline__ void expert_down_units(KParams p, KLayer lp, const Lds &L, int pr0, int pr1, int w0) {
  const int H = p->H, I = p->I, B = p->B;
  const int nsh = p->Is / I, P = B * p->k, pstride = P + B * nsh;
  const int nU = L.head().nU;
  const int nrb = (pr1 - pr0) / kRowBlock;
  const int *cnt = L.at<int>(p->o_cnt), *start = L.at<int>(p->o_start), *ulist = L.at<int>(p->o_ulist);
  const int *plist = L.at<int>(p->o_plist);
  float *part = L.at<float>(p->o_part);
  for (int un = (wave_id() + kWaves - w0 % kWaves) % kWaves; un < nrb * nU; un += kWaves) {
    const int rb = un / nU, s = un % nU;
    const int o0 = pr0 + rb * kRowBlock;
    const int e = ulist[s];
    const int n = cnt[e];
    const int *pl = plist + start[e];
    const char *wrow[kRowBlock];
    float sc[kRowBlock];
#pragma unroll
    for (int r = 0; r < kRowBlock; ++r) {
      wrow[r] = (const char *)lp->ed + ((size_t)e * H + o0 + r) * I * dsz<ED>();
      sc[r] = 1.f;
      if constexpr (ED == DT_FP8) sc[r] = __uint_as_float((uint32_t)lp->eds[(size_t)e * (H / 128) + (o0 + r) / 128] << 16);
    }
    for_token_groups(n, [&]<int TG>(int t0, int nt) {
      typename XSrc<XL>::ptr xr[TG];
      int col[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        col[t] = pl[t0 + (t < nt ? t : 0)];
        if constexpr (XL) xr[t] = L.raw(p->o_h) + (size_t)col[t] * I * dsz<AD>();
        else xr[t] = (const char *)p->hbuf + (size_t)col[t] * I * dsz<AD>();
      }
      down_unit<ED, AD, XL, TG>(wrow, I, xr, sc, part + (size_t)(o0 - pr0) * pstride, pstride, col, nt);
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
  __syncthreads();

  unsigned sink = 0;
  for (int l = 0; l < p->L; ++l) {
    KLayer lp = &p->lp[l];
    const int b0 = kBarPerLayer * l;

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
    bar_arrive(p, sh, b0 + BAR_ROUTER);
    if (!p->route_only) {
      for (; tau < nrt + p->Is * p->NSS; tau += NW)
        shared_gu_task<AD, SD, SMALL>(p, lp, L, (tau - nrt) / p->NSS, (tau - nrt) % p->NSS);
      bar_arrive(p, sh, b0 + BAR_SHARED);
    }
    bar_wait(p, sh, b0 + BAR_ROUTER);

    if (p->route_only) {
      if (blockIdx.x == 0)
        for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, L, t, true);
      break;
    }

    // P1: routing, gather tables, expert gate/up
    for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, L, t, blockIdx.x == 0);
    __syncthreads();
    build_tables(p, L);
    const int ntask = sh.nU * p->I;
    for (int q = W; q < ntask; q += NW) expert_gu_task<AD, ED, SMALL>(p, lp, L, q / p->I, q % p->I);
    bar_arrive(p, sh, b0 + BAR_H);

    // P2: this workgroup's output rows
    const int r0 = blockIdx.x * p->rows_per_wg;
    const int r1 = min(p->H, r0 + p->rows_per_wg);
    const bool one_pass = p->pass_rows >= p->rows_per_wg;
    const int nsh = p->Is / p->I;
    bar_wait(p, sh, b0 + BAR_SHARED);
    if constexpr (SMALL) {
      __syncthreads();  // x-hat in LDS is dead; its space now holds shared h and the partials
      finish_shared_h<AD>(p, L);
      __syncthreads();
    }
    if (one_pass && r0 < r1) shared_down_units<AD, SD, SMALL>(p, lp, L, r0, r1, 0);
    bar_wait(p, sh, b0 + BAR_H);
    if constexpr (SMALL) {
      stage_h(p, L, dsz<AD>());
      __syncthreads();
    }
    for (int pr0 = r0; pr0 < r1; pr0 += p->pass_rows) {
      const int pr1 = min(r1, pr0 + p->pass_rows);
      const int nrb = (pr1 - pr0) / kRowBlock;
      if (!one_pass) shared_down_units<AD, SD, SMALL>(p, lp, L, pr0, pr1, 0);
      expert_down_units<AD, ED, SMALL>(p, lp, L, pr0, pr1, one_pass ? 0 : nrb * nsh);
      __syncthreads();
      combine<AD>(p, lp, L, pr0, pr1);
      __syncthreads();
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
  w.rpart = off; off += up256((size_t)4 * B * d->num_experts * 4);
  w.hspart = off; off += up256((size_t)2 * B * 2 * is * 4);
  w.hbuf = off; off += up256((size_t)B * d->top_k * d->expert_inter * act);
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
  const size_t act = (size_t)dsize(d->act);
  size_t o = align16(sizeof(SmemHead));
  p.o_sel_idx = (int)o; o = align16(o + (size_t)P * 4);
  p.o_sel_w = (int)o; o = align16(o + (size_t)P * 4);
  p.o_cnt = (int)o; o = align16(o + (size_t)E * 4);
  p.o_start = (int)o; o = align16(o + (size_t)E * 4);
  p.o_tmask = (int)o; o = align16(o + (size_t)E * 8);
  p.o_ulist = (int)o; o = align16(o + (size_t)E * 4);
  p.o_plist = (int)o; o = align16(o + (size_t)P * 4);
  const size_t region = o;
  size_t need_a = 0, p2_fixed = 0;
  if (small) {
    p.o_xf = (int)region;
    size_t a = align16(region + (size_t)B * H * 4);
    p.o_xa = (int)a;
    need_a = (d->act == MOE_F32) ? a : align16(a + (size_t)B * H * act);
    p.o_hs = (int)region;
    size_t b = align16(region + (size_t)B * (d->shared_inter > 0 ? d->shared_inter : 1) * act);
    p.o_h = (int)b;
    b = align16(b + (size_t)P * d->expert_inter * act);
    p2_fixed = b;
  } else {
    p2_fixed = region;
  }
  p.o_part = (int)p2_fixed;
  const size_t per_row = (size_t)(P + B * nsh) * sizeof(float);
  const size_t lds_cap = (size_t)(di.max_lds > 0 ? di.max_lds : 65536);
  if (need_a > lds_cap || p2_fixed + (size_t)kRowBlock * per_row > lds_cap)
    return fail(MOE_ERR_UNSUPPORTED, "shape needs more LDS than the device's %zu bytes", lds_cap);
  int pr = (int)((lds_cap - p2_fixed) / per_row);
  pr = pr / kRowBlock * kRowBlock;
  p.pass_rows = pr < rpw ? pr : rpw;
  if (small && p.pass_rows < rpw)
    return fail(MOE_ERR_UNSUPPORTED, "small-batch layout needs one LDS pass over %d rows", rpw);
  size_t lds = p2_fixed + (size_t)p.pass_rows * per_row;
  if (need_a > lds) lds = need_a;

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
