// moedecode.hip - libmoedecode: the MoE decode layer for MI355X (gfx950).
//
// One persistent kernel per call (moe_route, moe_decode_layer, moe_decode_stack).
// The kernel fuses what the stock decode path launches one by one -
// normalisation, matmul, activation and routing ops (openai-hub.com "Kimi K3 ...
// 1.68x", section on why decode suits a megakernel) - and keeps the steps of
// one layer inside one launch, synchronised by grid barriers:
//
//   P0a  x-hat producers: workgroup t computes RMSNorm of token t, writes the
//        fp32 x-hat (router input) and its activation-dtype copy (FFN input).
//   B0   barrier
//   P0b  router GEMV, split over K (partial logits), then the shared expert's
//        gate/up rows, which do not depend on routing and fill the time the
//        router barrier takes (the pages move the shared expert onto its own
//        stream beside routing: smzdm.com post, section "what changed", MoE
//        de-duplication item).
//   B1   barrier (arrival after the router rows, wait after the shared rows)
//   P1   every workgroup redoes softmax + top-k + renormalisation (same inputs,
//        same code, same result - no extra barrier), builds the expert gather
//        tables in LDS (union of selected experts, each expert's token list),
//        then streams the selected experts' gate/up rows: h = SiLU(g) * u.
//   B2   barrier
//   P2   down projections: each workgroup owns a block of output rows and
//        reduces every selected expert and the shared expert for them, then
//        combines in a fixed order with the routing weights and the residual.
//   B3   barrier between layers of a stack.
//
// All reductions are fixed-order (no float atomics), so identical router rows
// give bit-identical logits and repeated runs give identical outputs.
//
// Memory ordering across the 8 XCDs: a wave publishes its stores with an
// agent-scope release fence before it counts itself in; a workgroup's last
// wave adds one to the global barrier counter; one wave per workgroup polls
// the counter, acquires at agent scope and raises an LDS flag for the others,
// which acquire again before they read what other workgroups wrote. Weights
// are static and may be loaded before a barrier; activations are only read
// after it (a compiler that hoisted an activation load above a sync wait was
// one of the bugs found in the pages' review: aiposthub.com article, section on
// how vLLM verifies AI-written kernels).
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

constexpr int kThreads = 1024;            // one workgroup per CU, 16 waves
constexpr int kWaves = kThreads / 64;
constexpr int kMaxB = 64;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
constexpr int kMaxL = 8;
constexpr int kTokGroup = 8;              // tokens whose partial sums a lane holds at once
constexpr int kRowBlock = 4;              // down-projection rows per unit
constexpr int kMaxBarriers = 4 * kMaxL + 4;
constexpr unsigned kCtrlBar = 0, kCtrlDone = 1, kCtrlErr = 2;
constexpr size_t kCtrlBytes = 256;

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
  int NS;                 // router K-splits
  int G;                  // workgroups
  int rows_per_wg;        // P2 output rows per workgroup (multiple of kRowBlock)
  int pass_rows;          // P2 rows per LDS pass
  float eps;
  long long timeout_ticks;  // s_memrealtime ticks (100 MHz) before a barrier wait gives up
  unsigned *ctrl;         // [0] barrier counter, [1] exit counter, [2] error word
  float *xhat;            // [B][H] fp32
  void *xa;               // [B][H] act (== xhat for fp32 activations)
  float *rpart;           // [NS][B][E]
  void *hbuf;             // [B*k][I] act
  void *hsbuf;            // [B][Is] act
  void *xbuf[2];          // [B][H] act, stack intermediates
  LayerPtrs lp[kMaxL];
};

// LDS layout (dynamic shared memory)
struct Smem {
  int bar_cnt[kMaxBarriers];   // waves of this workgroup that arrived
  int bar_claim[kMaxBarriers]; // one wave polls the global counter
  int bar_flag[kMaxBarriers];  // raised once the barrier is passed
  float red[kWaves];
  int nU;
  int sel_idx[kMaxB * kMaxK];
  float sel_w[kMaxB * kMaxK];
  int cnt[kMaxE];
  int start[kMaxE];
  unsigned long long tmask[kMaxE];
  int ulist[kMaxE];
  int plist[kMaxB * kMaxK];
  int scan_tmp[2 * kWaves];
  float part[1];               // P2 partial sums, sized at launch
};

// Kernel parameters are read in place from the kernarg segment (address space 4).
#define KARG __attribute__((address_space(4)))
typedef const KARG Params *KParams;
typedef const KARG LayerPtrs *KLayer;

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

// value of v once stored in dtype D
template <int D> __device__ __forceinline__ float round_act(float v) {
  if constexpr (D == DT_F32) return v;
  else return __uint_as_float((uint32_t)f32_to_bf16(v) << 16);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *(const uint4 *)p; }

// ---------------------------------------------------------------------------
// 16-byte weight chunk . activation chunk

template <int WD> constexpr int elems16() { return WD == DT_F32 ? 4 : WD == DT_BF16 ? 8 : 16; }
template <int XD> constexpr int xsize() { return XD == DT_F32 ? 4 : 2; }

template <int WD, int XD> struct Chunk;

template <> struct Chunk<DT_BF16, DT_BF16> {
  static constexpr int NX = 1;
  __device__ static __forceinline__ float dot(const uint4 &w, const uint4 *x, float a) {
    a = dot2_bf16(w.x, x[0].x, a);
    a = dot2_bf16(w.y, x[0].y, a);
    a = dot2_bf16(w.z, x[0].z, a);
    a = dot2_bf16(w.w, x[0].w, a);
    return a;
  }
};

template <> struct Chunk<DT_F32, DT_F32> {
  static constexpr int NX = 1;
  __device__ static __forceinline__ float dot(const uint4 &w, const uint4 *x, float a) {
    a = fmaf(__uint_as_float(w.x), __uint_as_float(x[0].x), a);
    a = fmaf(__uint_as_float(w.y), __uint_as_float(x[0].y), a);
    a = fmaf(__uint_as_float(w.z), __uint_as_float(x[0].z), a);
    a = fmaf(__uint_as_float(w.w), __uint_as_float(x[0].w), a);
    return a;
  }
};

template <> struct Chunk<DT_BF16, DT_F32> {
  static constexpr int NX = 2;
  __device__ static __forceinline__ float dot(const uint4 &w, const uint4 *x, float a) {
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
  __device__ static __forceinline__ float dot(const uint4 &w, const uint4 *x, float a) {
    a = dot4(w.x, x[0].x, x[0].y, a);
    a = dot4(w.y, x[0].z, x[0].w, a);
    a = dot4(w.z, x[1].x, x[1].y, a);
    a = dot4(w.w, x[1].z, x[1].w, a);
    return a;
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// grid barriers

__device__ __forceinline__ long long rt_now() { return (long long)__builtin_amdgcn_s_memrealtime(); }

// A wave is done with the work barrier b waits for.
__device__ void bar_arrive(KParams p, Smem &sm, int b) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (lane_id() == 0) {
    int old = __hip_atomic_fetch_add(&sm.bar_cnt[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (old == kWaves - 1)
      __hip_atomic_fetch_add(&p->ctrl[kCtrlBar], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until every workgroup arrived at barrier b (global barrier number nb).
__device__ void bar_wait(KParams p, Smem &sm, int b, int nb) {
  const unsigned target = (unsigned)p->G * (unsigned)(nb + 1);
  if (lane_id() == 0) {
    if (__hip_atomic_load(&sm.bar_flag[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
      const bool poller = __hip_atomic_exchange(&sm.bar_claim[b], 1, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
      const long long t0 = rt_now();
      if (poller) {
        while (__hip_atomic_load(&p->ctrl[kCtrlBar], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
          __builtin_amdgcn_s_sleep(2);
          if (rt_now() - t0 > p->timeout_ticks) {
            __hip_atomic_store(&p->ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&sm.bar_flag[b], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        while (__hip_atomic_load(&sm.bar_flag[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          __builtin_amdgcn_s_sleep(1);
          if (rt_now() - t0 > 2 * p->timeout_ticks) break;
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// ---------------------------------------------------------------------------
// GEMV pieces. Lane l of a wave covers elements [c*64*EPL + l*EPL, +EPL) of a
// K-long row for chunk c; rows are 16-byte aligned and K % EPL == 0.

// Dot products of one weight row segment [k0, k1) with TG activation rows
// xr[t] (element offsets as in the weight row), lane partials in acc[t].
template <int WD, int XD, int SEG, int TG>
__device__ __forceinline__ void row_dot(const void *wrow, int k0, int k1, const char *const *xr, float *acc) {
  constexpr int EPL = elems16<WD>();
  constexpr int NX = Chunk<WD, XD>::NX;
  const int lane = lane_id();
  for (int c0 = k0; c0 < k1; c0 += SEG * 64 * EPL) {
    uint4 w[SEG];
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const int e = c0 + (s * 64 + lane) * EPL;
      w[s] = (e < k1) ? ld16((const char *)wrow + (size_t)e * (16 / EPL)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const int e = c0 + (s * 64 + lane) * EPL;
      if (e < k1) {
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          uint4 xv[NX];
#pragma unroll
          for (int q = 0; q < NX; ++q) xv[q] = ld16(xr[t] + (size_t)e * xsize<XD>() + 16 * q);
          acc[t] = Chunk<WD, XD>::dot(w[s], xv, acc[t]);
        }
      }
    }
  }
}

// Run f.template operator()<TG>(t0, nt) over groups of up to 8 of n tokens,
// with the smallest specialisation that holds each group.
template <class F>
__device__ __forceinline__ void for_token_groups(int n, F &&f) {
  for (int t0 = 0; t0 < n; t0 += kTokGroup) {
    const int nt = min(kTokGroup, n - t0);
    if (nt == 1) f.template operator()<1>(t0, nt);
    else if (nt == 2) f.template operator()<2>(t0, nt);
    else if (nt <= 4) f.template operator()<4>(t0, nt);
    else f.template operator()<8>(t0, nt);
  }
}

// Gate/up pair task: rows j (gate) and inter+j (up) of a [2 inter][H] matrix
// for n tokens; writes h[slot][j] = act(SiLU(g * gs) * (u * us)). Tokens are
// list[q] / div with slot list[q] (expert pairs), or q with slot q (list null).
template <int AD, int WD>
__device__ __forceinline__ void gate_up_pair(KParams p, const void *gu, int inter, int j,
                                                       float gs, float us, const int *list, int div, int n,
                                                       void *hout, int hstride) {
  const int H = p->H;
  const size_t rowb = (size_t)H * (WD == DT_F32 ? 4 : WD == DT_BF16 ? 2 : 1);
  const void *grow = (const char *)gu + (size_t)j * rowb;
  const void *urow = (const char *)gu + (size_t)(inter + j) * rowb;
  for_token_groups(n, [&]<int TG>(int t0, int nt) {
    const char *xr[TG];
    int slot[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const int q = t0 + (t < nt ? t : 0);
      slot[t] = list ? list[q] : q;
      const int tok = list ? slot[t] / div : q;
      xr[t] = (const char *)p->xa + (size_t)tok * H * xsize<AD>();
    }
    float ag[TG], au[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) ag[t] = au[t] = 0.f;
    constexpr int SEG = (WD == DT_FP8) ? (TG <= 2 ? 4 : TG == 4 ? 2 : 1) : (TG <= 2 ? 7 : TG == 4 ? 4 : 2);
    row_dot<WD, AD, SEG, TG>(grow, 0, H, xr, ag);
    row_dot<WD, AD, SEG, TG>(urow, 0, H, xr, au);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      if (t < nt) {
        const float g = wave_sum(ag[t]) * gs;
        const float u = wave_sum(au[t]) * us;
        if (lane_id() == 0) store_act<AD>(hout, (size_t)slot[t] * hstride + j, g / (1.0f + expf(-g)) * u);
      }
    }
  });
}

// ---------------------------------------------------------------------------
// top-k of one token (one wave): softmax over all E logits restricted to the
// k largest (ties to the lower index), renormalised.

__device__ __attribute__((noinline)) void topk_token(KParams p, KLayer lp, Smem &sm, int t, bool write_out) {
  const int lane = lane_id();
  const int E = p->E, k = p->k;
  constexpr int PER = kMaxE / 64;
  float v[PER];
  unsigned taken = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    float l = -INFINITY;
    if (e < E) {
      float s = 0.f;
      for (int q = 0; q < p->NS; ++q) s += p->rpart[((size_t)q * p->B + t) * E + e];
      if (lp->rb) s += lp->rb[e];
      l = (s == s) ? s : -INFINITY;  // a NaN logit ranks last, so every pick is a valid expert
      if (write_out && lp->logits_out) lp->logits_out[(size_t)t * E + e] = l;
    } else {
      taken |= 1u << j;
    }
    v[j] = l;
  }
  float lmax = 0.f, z = 0.f;
  float selv = 0.f;
  int seli = 0;
  for (int i = 0; i < k; ++i) {
    // lane-local best: larger value, then lower index
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (!(taken & (1u << j)) && (v[j] > bv || (v[j] == bv && e < bi))) { bv = v[j]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (i == 0) lmax = bv;
    const float ex = expf(bv - lmax);
    z += ex;
    if (lane == i) { selv = ex; seli = bi; }
    if (lane == 0) sm.sel_idx[t * k + i] = bi;
  }
  if (lane < k) {
    const float w = selv / z;
    sm.sel_w[t * k + lane] = w;
    if (write_out) {
      if (lp->idx_out) lp->idx_out[(size_t)t * k + lane] = seli;
      if (lp->w_out) lp->w_out[(size_t)t * k + lane] = w;
    }
  }
}

// ---------------------------------------------------------------------------
// gather tables: union U of selected experts (ascending), each expert's pairs
// (t*k+i) in ascending token order.

__device__ __attribute__((noinline)) void build_tables(KParams p, Smem &sm) {
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int E = p->E, P = p->B * p->k;
  for (int e = tid; e < E; e += kThreads) { sm.cnt[e] = 0; sm.tmask[e] = 0ull; }
  __syncthreads();
  for (int q = tid; q < P; q += kThreads) {
    const int e = sm.sel_idx[q];
    atomicAdd(&sm.cnt[e], 1);
    atomicOr(&sm.tmask[e], 1ull << (q / p->k));
  }
  __syncthreads();
  // block scan over e of (cnt, cnt > 0); E <= kThreads
  int c = (tid < E) ? sm.cnt[tid] : 0;
  int f = c > 0 ? 1 : 0;
  int ci = c, fi = f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int uc = __shfl_up(ci, o), uf = __shfl_up(fi, o);
    if (lane >= o) { ci += uc; fi += uf; }
  }
  if (lane == 63) { sm.scan_tmp[wv] = ci; sm.scan_tmp[kWaves + wv] = fi; }
  __syncthreads();
  int bc = 0, bf = 0;
  for (int w2 = 0; w2 < wv; ++w2) { bc += sm.scan_tmp[w2]; bf += sm.scan_tmp[kWaves + w2]; }
  if (tid < E) {
    sm.start[tid] = bc + ci - c;
    if (f) sm.ulist[bf + fi - f] = tid;
  }
  if (tid == kThreads - 1) {
    int tot = 0;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sm.scan_tmp[kWaves + w2];
    sm.nU = tot;
  }
  __syncthreads();
  for (int q = tid; q < P; q += kThreads) {
    const int e = sm.sel_idx[q];
    const int t = q / p->k;
    const unsigned long long below = (t == 0) ? 0ull : (sm.tmask[e] & ((1ull << t) - 1ull));
    sm.plist[sm.start[e] + __popcll(below)] = q;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// P0a: RMSNorm producers

template <int AD>
__device__ __attribute__((noinline)) void produce_xhat(KParams p, KLayer lp, Smem &sm) {
  const int H = p->H, tid = threadIdx.x;
  for (int t = blockIdx.x; t < p->B; t += p->G) {
    float ss = 0.f;
    for (int h = tid; h < H; h += kThreads) {
      const float v = load_act<AD>(lp->x, (size_t)t * H + h);
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane_id() == 0) sm.red[wave_id()] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w2 = 0; w2 < kWaves; ++w2) tot += sm.red[w2];
    const float r = 1.0f / sqrtf(tot / (float)H + p->eps);
    for (int h = tid; h < H; h += kThreads) {
      const float xh = load_act<AD>(lp->x, (size_t)t * H + h) * r * load_act<AD>(lp->gamma, h);
      p->xhat[(size_t)t * H + h] = xh;
      if constexpr (AD != DT_F32) store_act<AD>(p->xa, (size_t)t * H + h, xh);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// the kernel

// ---------------------------------------------------------------------------
// phases

// P0b router: task tau = (row e, K-split s) -> partial logits rpart[s][t][e]
template <int RD>
__device__ __forceinline__ void router_phase(KParams p, KLayer lp, int W, int NW) {
  const int H = p->H, E = p->E, B = p->B, lane = lane_id();
  const int nrt = E * p->NS, Ks = H / p->NS;
  for (int tau = W; tau < nrt; tau += NW) {
    const int e = tau / p->NS, s = tau % p->NS;
    const void *wrow = (const char *)lp->rw + (size_t)e * H * (RD == DT_F32 ? 4 : 2);
    for_token_groups(B, [&]<int TG>(int t0, int nt) {
      const char *xr[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) xr[t] = (const char *)(p->xhat + (size_t)(t0 + (t < nt ? t : 0)) * H);
      float acc[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[t] = 0.f;
      constexpr int SEG = TG <= 2 ? 7 : TG == 4 ? 4 : 2;
      row_dot<RD, DT_F32, SEG, TG>(wrow, s * Ks, (s + 1) * Ks, xr, acc);
#pragma unroll
      for (int t = 0; t < TG; ++t)
        if (t < nt) {
          const float v = wave_sum(acc[t]);
          if (lane == 0) p->rpart[((size_t)s * B + t0 + t) * E + e] = v;
        }
    });
  }
}

// P0b shared expert gate/up: the P0 task list is [router tasks | shared pairs];
// wave W takes every NW-th task.
template <int AD, int SD>
__device__ __forceinline__ void shared_phase(KParams p, KLayer lp, int W, int NW) {
  const int nrt = p->E * p->NS;
  int tau = W;
  while (tau < nrt) tau += NW;
  for (; tau < nrt + p->Is; tau += NW)
    gate_up_pair<AD, SD>(p, lp->sgu, p->Is, tau - nrt, 1.f, 1.f, nullptr, 1, p->B, p->hsbuf, p->Is);
}

// P1 expert gate/up: task tau = (expert u of U, pair j)
template <int AD, int ED>
__device__ __forceinline__ void expert_phase(KParams p, KLayer lp, Smem &sm, int W,
                                                       int NW) {
  const int H = p->H, I = p->I, k = p->k;
  const int ntask = sm.nU * I;
  const size_t exp_gu = (size_t)2 * I * H;  // elements per expert
  for (int tau = W; tau < ntask; tau += NW) {
    const int u = tau / I, j = tau % I;
    const int e = sm.ulist[u];
    const int n = sm.cnt[e];
    const int *pl = &sm.plist[sm.start[e]];
    float gs = 1.f, us = 1.f;
    const void *gu;
    if constexpr (ED == DT_FP8) {
      // e4m3_to_f32 is exact, so the bf16 row scale multiplies the finished dot
      gu = (const uint8_t *)lp->egu + (size_t)e * exp_gu;
      const uint16_t *sc = lp->egus + (size_t)e * (2 * I / 128);
      gs = __uint_as_float((uint32_t)sc[j / 128] << 16);
      us = __uint_as_float((uint32_t)sc[(I + j) / 128] << 16);
    } else {
      gu = (const char *)lp->egu + (size_t)e * exp_gu * (ED == DT_F32 ? 4 : 2);
    }
    gate_up_pair<AD, ED>(p, gu, I, j, gs, us, pl, k, n, p->hbuf, I);
  }
}

// One P2 unit: rows [o0, o0+nr) of one expert's down matrix (or one I-wide
// column block hf of the shared down matrix) for its tokens; lane-reduced
// results go to LDS partials part[(o - pr0) * pstride + column].
template <int AD, int ED, int SD>
__device__ __forceinline__ void down_unit(KParams p, KLayer lp, Smem &sm, int s,
                                                    int o0, int nr, int pr0, int pstride) {
  const int H = p->H, I = p->I, Is = p->Is, B = p->B, lane = lane_id();
  const int nU = sm.nU, P = B * p->k;
  const int nsh = Is / I;
  if (s < nU) {
    const int e = sm.ulist[s];
    const int n = sm.cnt[e];
    const int *pl = &sm.plist[sm.start[e]];
    const size_t wexp = (size_t)H * I;
    for_token_groups(n, [&]<int TG>(int t0, int nt) {
      int slot[TG];
      const char *xr[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        slot[t] = pl[t0 + (t < nt ? t : 0)];
        xr[t] = (const char *)p->hbuf + (size_t)slot[t] * I * xsize<AD>();
      }
      for (int r = 0; r < nr; ++r) {
        const int o = o0 + r;
        float acc[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[t] = 0.f;
        const void *wrow = (const char *)lp->ed + (e * wexp + (size_t)o * I) * (ED == DT_F32 ? 4 : ED == DT_BF16 ? 2 : 1);
        row_dot<ED, AD, (ED == DT_FP8 ? 1 : 2), TG>(wrow, 0, I, xr, acc);
        float sc = 1.f;
        if constexpr (ED == DT_FP8) sc = __uint_as_float((uint32_t)lp->eds[(size_t)e * (H / 128) + o / 128] << 16);
#pragma unroll
        for (int t = 0; t < TG; ++t)
          if (t < nt) {
            const float v = wave_sum(acc[t]) * sc;
            if (lane == 0) sm.part[(o - pr0) * pstride + slot[t]] = v;
          }
      }
    });
  } else {
    const int hf = s - nU;
    for_token_groups(B, [&]<int TG>(int t0, int nt) {
      const char *xr[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t)
        xr[t] = (const char *)p->hsbuf + ((size_t)(t0 + (t < nt ? t : 0)) * Is + (size_t)hf * I) * xsize<AD>();
      for (int r = 0; r < nr; ++r) {
        const int o = o0 + r;
        float acc[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[t] = 0.f;
        const void *wrow = (const char *)lp->sd + ((size_t)o * Is + (size_t)hf * I) * (SD == DT_F32 ? 4 : 2);
        row_dot<SD, AD, 2, TG>(wrow, 0, I, xr, acc);
#pragma unroll
        for (int t = 0; t < TG; ++t)
          if (t < nt) {
            const float v = wave_sum(acc[t]);
            if (lane == 0) sm.part[(o - pr0) * pstride + P + (t0 + t) * nsh + hf] = v;
          }
      }
    });
  }
}

// P2: this workgroup's output rows: all units, then the fixed-order combine
// y = x + shared + sum_i w_i d_i (rank order i).
template <int AD, int ED, int SD>
__device__ __forceinline__ void down_phase(KParams p, KLayer lp, Smem &sm) {
  const int H = p->H, k = p->k, B = p->B, tid = threadIdx.x, wv = wave_id();
  const int nsh = p->Is > 0 ? p->Is / p->I : 0;
  const int r0 = blockIdx.x * p->rows_per_wg;
  const int r1 = min(H, r0 + p->rows_per_wg);
  const int P = B * k;
  const int pstride = P + B * nsh;
  const int nslot = sm.nU + nsh;
  for (int pr0 = r0; pr0 < r1; pr0 += p->pass_rows) {
    const int pr1 = min(r1, pr0 + p->pass_rows);
    const int nrb = (pr1 - pr0 + kRowBlock - 1) / kRowBlock;
    const int nunit = nrb * nslot;
    for (int un = wv; un < nunit; un += kWaves) {
      const int rb = un / nslot, s = un % nslot;
      const int o0 = pr0 + rb * kRowBlock;
      down_unit<AD, ED, SD>(p, lp, sm, s, o0, min(kRowBlock, pr1 - o0), pr0, pstride);
    }
    __syncthreads();
    const int cells = (pr1 - pr0) * B;
    for (int c = tid; c < cells; c += kThreads) {
      const int ro = c / B, t = c % B;
      const int o = pr0 + ro;
      const float *pp = &sm.part[ro * pstride];
      float sh = 0.f;
      for (int hf = 0; hf < nsh; ++hf) sh += pp[P + t * nsh + hf];
      float rt = 0.f;
      for (int i = 0; i < k; ++i) rt = fmaf(sm.sel_w[t * k + i], pp[t * k + i], rt);
      const float v = load_act<AD>(lp->x, (size_t)t * H + o) + sh + rt;
      store_act<AD>(lp->y, (size_t)t * H + o, v);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// the kernel

template <int AD, int RD, int ED, int SD>
__global__ void __launch_bounds__(kThreads, 1) moe_kernel(Params params) {
  // read the parameters in place in the kernarg segment (scalar loads; no private copy)
  (void)params;
  KParams p = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  const int tid = threadIdx.x, wv = wave_id();
  const int NW = p->G * kWaves;
  const int W = blockIdx.x * kWaves + wv;  // global wave id

  for (int i = tid; i < kMaxBarriers; i += kThreads) sm.bar_cnt[i] = sm.bar_claim[i] = sm.bar_flag[i] = 0;
  __syncthreads();

  int nb = 0;  // global barrier number
  for (int l = 0; l < p->L; ++l) {
    KLayer lp = &p->lp[l];
    const int b0 = 4 * l;

    produce_xhat<AD>(p, lp, sm);
    bar_arrive(p, sm, b0);
    bar_wait(p, sm, b0, nb++);

    router_phase<RD>(p, lp, W, NW);
    bar_arrive(p, sm, b0 + 1);
    if (!p->route_only) shared_phase<AD, SD>(p, lp, W, NW);
    bar_wait(p, sm, b0 + 1, nb++);

    if (p->route_only) {
      if (blockIdx.x == 0)
        for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, sm, t, true);
      break;
    }
    for (int t = wv; t < p->B; t += kWaves) topk_token(p, lp, sm, t, blockIdx.x == 0);
    __syncthreads();
    build_tables(p, sm);
    expert_phase<AD, ED>(p, lp, sm, W, NW);
    bar_arrive(p, sm, b0 + 2);
    bar_wait(p, sm, b0 + 2, nb++);

    down_phase<AD, ED, SD>(p, lp, sm);
    if (l + 1 < p->L) {
      bar_arrive(p, sm, b0 + 3);
      bar_wait(p, sm, b0 + 3, nb++);
    }
  }

  // last workgroup out resets the counters for the next launch on this workspace
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&p->ctrl[kCtrlDone], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (unsigned)p->G - 1u) {
      __hip_atomic_store(&p->ctrl[kCtrlBar], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p->ctrl[kCtrlDone], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MOE_ERR_DEVICE, "hipGetDevice failed");
  if (g_dev[dev].cus == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed");
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      lds = 65536;
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
    return fail(MOE_ERR_UNSUPPORTED, "top_k=%d num_experts=%d: need 1<=k<=32, k<=E<=1024", d->top_k,
                d->num_experts);
  const bool f32set = d->act == MOE_F32 && d->router == MOE_F32 && d->expert == MOE_F32 && d->shared == MOE_F32;
  const bool bfset = d->act == MOE_BF16 && (d->router == MOE_F32 || d->router == MOE_BF16) &&
                     (d->expert == MOE_BF16 || d->expert == MOE_FP8_E4M3) && d->shared == MOE_BF16;
  if (!f32set && !bfset) return fail(MOE_ERR_UNSUPPORTED, "unsupported dtype combination");
  if (d->expert == MOE_FP8_E4M3 && d->scale_group != 128)
    return fail(MOE_ERR_UNSUPPORTED, "fp8 experts need scale_group 128");
  return MOE_OK;
}

int router_splits(const moe_layer_desc *d) {
  const int chunk = 64 * (d->router == MOE_F32 ? 4 : 8);
  return ((d->hidden / 2) % chunk == 0) ? 2 : 1;
}

struct WsLayout {
  size_t xhat, xa, rpart, hbuf, hsbuf, xbuf0, xbuf1, total;
};

size_t up256(size_t v) { return (v + 255u) & ~(size_t)255u; }

WsLayout ws_layout(const moe_layer_desc *d, int B, int L) {
  WsLayout w{};
  size_t off = kCtrlBytes;
  const size_t act = (size_t)dsize(d->act);
  w.xhat = off; off += up256((size_t)B * d->hidden * 4);
  w.xa = off; off += up256((size_t)B * d->hidden * act);
  w.rpart = off; off += up256((size_t)2 * B * d->num_experts * 4);
  w.hbuf = off; off += up256((size_t)B * d->top_k * d->expert_inter * act);
  w.hsbuf = off; off += up256((size_t)B * (d->shared_inter > 0 ? d->shared_inter : 1) * act);
  w.xbuf0 = off; off += (L > 1) ? up256((size_t)B * d->hidden * act) : 0;
  w.xbuf1 = off; off += (L > 2) ? up256((size_t)B * d->hidden * act) : 0;
  w.total = off;
  return w;
}

typedef void (*kernel_fn)(Params);

kernel_fn pick_kernel(const moe_layer_desc *d) {
  if (d->act == MOE_F32) return moe_kernel<DT_F32, DT_F32, DT_F32, DT_F32>;
  if (d->expert == MOE_BF16)
    return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_BF16, DT_BF16>
                                : moe_kernel<DT_BF16, DT_BF16, DT_BF16, DT_BF16>;
  return d->router == MOE_F32 ? moe_kernel<DT_BF16, DT_F32, DT_FP8, DT_BF16>
                              : moe_kernel<DT_BF16, DT_BF16, DT_FP8, DT_BF16>;
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

moe_status launch(const moe_layer_desc *d, const moe_layer_weights *layers, int L, const void *x, void *y, int B,
                  int32_t *idx, float *wts, float *logits, void *ws, size_t ws_bytes, void *stream,
                  bool route_only) {
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
  p.NS = router_splits(d);
  p.G = di.cus;
  if (p.G < 1) return fail(MOE_ERR_DEVICE, "device reports no compute units");
  int rpw = (p.H + p.G - 1) / p.G;
  rpw = (rpw + kRowBlock - 1) / kRowBlock * kRowBlock;
  p.rows_per_wg = rpw;
  const int nsh = d->shared_inter > 0 ? d->shared_inter / d->expert_inter : 0;
  const size_t fixed = (offsetof(Smem, part) + 15) & ~(size_t)15;
  const size_t per_row = (size_t)(B * d->top_k + B * nsh) * sizeof(float);
  const size_t lds_cap = (size_t)(di.max_lds > 0 ? di.max_lds : 65536);
  size_t budget = lds_cap > fixed + 4096 ? lds_cap - fixed : 4096;
  int pr = (int)(budget / per_row);
  pr = pr / kRowBlock * kRowBlock;
  if (pr < kRowBlock) return fail(MOE_ERR_UNSUPPORTED, "LDS too small for batch %d", B);
  p.pass_rows = pr < rpw ? pr : rpw;
  p.timeout_ticks = 200000000LL;  // 2 s at 100 MHz
  // test hook: a tiny limit makes every barrier wait give up at once (no hang, no fault)
  if (const char *ev = getenv("MOE_DEBUG_BARRIER_TIMEOUT_TICKS")) p.timeout_ticks = atoll(ev);
  unsigned char *wsb = (unsigned char *)ws;
  p.ctrl = (unsigned *)wsb;
  p.xhat = (float *)(wsb + wl.xhat);
  p.xa = (d->act == MOE_F32) ? (void *)p.xhat : (void *)(wsb + wl.xa);
  p.rpart = (float *)(wsb + wl.rpart);
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
  const size_t lds = fixed + (size_t)p.pass_rows * per_row;
  kernel_fn fn = pick_kernel(d);
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
  if (hipMemcpy(&err, (unsigned char *)ws + kCtrlErr * sizeof(unsigned), sizeof err, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return fail(MOE_ERR_DEVICE, "reading the error word failed");
  if (err) {
    const unsigned zero = 0;
    if (hipMemcpy((unsigned char *)ws + kCtrlErr * sizeof(unsigned), &zero, sizeof zero, hipMemcpyHostToDevice) !=
        hipSuccess)
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
