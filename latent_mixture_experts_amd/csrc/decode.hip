// Decode / speculative-verify forward (T <= 8 tokens): four launches of
// dequant-in-register GEMVs over the tiled weight streams.
//
// Layer ("Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B table
// left on the SSD", section "A latent in front of the experts", the layer
// equation y = U_g(sum_e w_e E_e(D_g x)); "Edge0 145B and Edge0 120B" model
// page, "Model profile" and architecture tables):
//
//   phase 1  router logits in fp64 (bf16 weights), D_g x for every group,
//            shared-expert gate/up + SwiGLU; the last router block takes the
//            top K, the renormalized softmax and the (label, expert) stable
//            permutation of the assignments
//   phase 2  routed-expert gate/up + SwiGLU (NVFP4), one block per (distinct
//            expert, 32-row tile of gate/up pairs)
//   phase 3  routed-expert down (NVFP4) scaled by the routing weight; the last
//            block of each (group, 64-row tile) sums the group's outputs per
//            token in ascending k
//   phase 4  U_g over the per-group sums and the shared-expert down; the last
//            block of each 64-row tile of y adds the partials in a fixed order
//
// Every weight byte is read once per forward with 16-byte lane loads that
// form 1 KiB coalesced requests; activations are read through the scalar
// data path (uniform addresses), so the vector ALUs only decode and multiply.
// Cross-block steps use the "last block" pattern (release fence, counter,
// acquire fence); counters are reset by the block that consumes them, so
// forwards need no memset and the result is bit-reproducible.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace lm {
namespace {

typedef const __attribute__((address_space(4))) float* cf_t;     // uniform, read-only
typedef const __attribute__((address_space(4))) int* ci_t;
typedef const __attribute__((address_space(4))) uint8_t* cu8_t;

__device__ __forceinline__ cf_t cf(const float* p) { return (cf_t)p; }
__device__ __forceinline__ ci_t ci(const int* p) { return (ci_t)p; }

__device__ __forceinline__ uint4 ldw(const uint8_t* p) { return *(const uint4*)p; }

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// ---------------------------------------------------------------------------
// One wavefront, one super-step (up to 256 columns) of one 64-row tile.
// p points at the lane's 16 bytes of the super-step's first slot; xv[t] at
// column 0 of the super-step in input vector t; ncs = code slots present.
// acc[t] += sum over the super-step of row(lane) . xv[t].

template <int NT>
__device__ __forceinline__ void ss_q8(const uint8_t* p, int ncs, const cf_t (&xv)[NT],
                                      float (&acc)[NT]) {
  uint4 q[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < ncs) q[j] = ldw(p + j * kSlot);
  const uint4 sc = ldw(p + ncs * kSlot);
  const uint32_t s4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (2 * b < ncs) {
      float blk[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) blk[t] = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 w = q[2 * b + hh];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = (float)(int8_t)(ww[i] >> (8 * j));
            const int c = 32 * b + 16 * hh + 4 * i + j;
#pragma unroll
            for (int t = 0; t < NT; ++t) blk[t] = __builtin_fmaf(v, xv[t][c], blk[t]);
          }
      }
      const float d = h2f(s4[b >> 1] >> (16 * (b & 1)));
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(d, blk[t], acc[t]);
    }
  }
}

// Q4: each code slot is one block of 32 signed 4-bit codes (element 2m in the
// low nibble of byte m). Shifting a nibble into the top of a byte gives 16*q
// as an int8; the 1/16 folds into the block scale.
template <int NT>
__device__ __forceinline__ void ss_q4(const uint8_t* p, int ncs, const cf_t (&xv)[NT],
                                      float (&acc)[NT]) {
  uint4 q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < ncs) q[j] = ldw(p + j * kSlot);
  const uint4 sc = ldw(p + ncs * kSlot);
  const uint32_t s4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < ncs) {
      float blk[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) blk[t] = 0.f;
      const uint32_t ww[4] = {q[b].x, q[b].y, q[b].z, q[b].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (ww[i] << 4) & 0xF0F0F0F0u;   // elements 8i + 0, 2, 4, 6
        const uint32_t hi = ww[i] & 0xF0F0F0F0u;          // elements 8i + 1, 3, 5, 7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v0 = (float)(int8_t)(lo >> (8 * j));
          const float v1 = (float)(int8_t)(hi >> (8 * j));
          const int c = 32 * b + 8 * i + 2 * j;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            blk[t] = __builtin_fmaf(v0, xv[t][c], blk[t]);
            blk[t] = __builtin_fmaf(v1, xv[t][c + 1], blk[t]);
          }
        }
      }
      const float d = h2f(s4[b >> 1] >> (16 * (b & 1))) * 0.0625f;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(d, blk[t], acc[t]);
    }
  }
}

// NVFP4: each code slot is 32 E2M1 codes = two scale blocks of 16; the scale
// slot holds 16 E4M3 bytes. The gfx950 converters decode two E2M1 values of
// one byte (low nibble first) and two E4M3 values of one half-word.
template <int NT>
__device__ __forceinline__ void ss_fp4(const uint8_t* p, int ncs, const cf_t (&xv)[NT],
                                       float (&acc)[NT]) {
  uint4 q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < ncs) q[j] = ldw(p + j * kSlot);
  const uint4 sc = ldw(p + ncs * kSlot);
  const uint32_t s4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < ncs) {
      const uint32_t ww[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
      // scale bytes 2j and 2j+1 live in word j/2, half (j&1)
      const auto sf = (j & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(s4[j >> 1], true)
                              : __builtin_amdgcn_cvt_pk_f32_fp8(s4[j >> 1], false);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float blk[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) blk[t] = 0.f;
#pragma unroll
        for (int i = 2 * hb; i < 2 * hb + 2; ++i) {
#define LMOE_FP4_BYTE(m)                                                               \
  {                                                                                    \
    const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww[i], 1.0f, m);          \
    const int c = 32 * j + 8 * i + 2 * (m);                                            \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                   \
      blk[t] = __builtin_fmaf(f2[0], xv[t][c], blk[t]);                                \
      blk[t] = __builtin_fmaf(f2[1], xv[t][c + 1], blk[t]);                            \
    }                                                                                  \
  }
          LMOE_FP4_BYTE(0)
          LMOE_FP4_BYTE(1)
          LMOE_FP4_BYTE(2)
          LMOE_FP4_BYTE(3)
#undef LMOE_FP4_BYTE
        }
        const float s = hb ? sf[1] : sf[0];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(s, blk[t], acc[t]);
      }
    }
  }
}

// bf16 rows, fp32 accumulation; a super-step has up to 32 code slots, taken
// in two halves of 16 to bound live registers.
template <int NT>
__device__ __forceinline__ void ss_bf16(const uint8_t* p, int ncs, const cf_t (&xv)[NT],
                                        float (&acc)[NT]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (16 * half + j < ncs) q[j] = ldw(p + (16 * half + j) * kSlot);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (16 * half + j < ncs) {
        const uint32_t ww[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = __uint_as_float(ww[i] << 16);
          const float v1 = __uint_as_float(ww[i] & 0xFFFF0000u);
          const int c = 8 * (16 * half + j) + 2 * i;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[t] = __builtin_fmaf(v0, xv[t][c], acc[t]);
            acc[t] = __builtin_fmaf(v1, xv[t][c + 1], acc[t]);
          }
        }
      }
    }
  }
}

// Router: bf16 rows, fp64 products and sums, over a chunk of `nslot` (<= 8)
// slots of 8 columns.
template <int NT>
__device__ __forceinline__ void chunk_bf16_f64(const uint8_t* p, int nslot, const cf_t (&xv)[NT],
                                               double (&acc)[NT]) {
  uint4 q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < nslot) q[j] = ldw(p + j * kSlot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < nslot) {
      const uint32_t ww[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double v0 = (double)__uint_as_float(ww[i] << 16);
        const double v1 = (double)__uint_as_float(ww[i] & 0xFFFF0000u);
        const int c = 8 * j + 2 * i;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t] = __builtin_fma(v0, (double)xv[t][c], acc[t]);
          acc[t] = __builtin_fma(v1, (double)xv[t][c + 1], acc[t]);
        }
      }
    }
  }
}

// D/U matrices: Q8 or Q4 (uniform branch on the handle's format).
template <int NT>
__device__ __forceinline__ void ss_du(int fmt, const uint8_t* p, int ncs, const cf_t (&xv)[NT],
                                      float (&acc)[NT]) {
  if (fmt == kQ8) ss_q8<NT>(p, ncs, xv, acc);
  else ss_q4<NT>(p, ncs, xv, acc);
}

// Pointer to lane `lane`'s bytes of super-step `ss` of tile `tile`.
__device__ __forceinline__ const uint8_t* tile_ptr(const uint8_t* base, const Geom& g, int tile,
                                                   int ss, int lane) {
  return base + ((size_t)tile * g.tile_slots + (size_t)ss * g.full) * kSlot + lane * 16;
}
__device__ __forceinline__ int ss_codes(int fmt, const Geom& g, int ss) {
  return min(kSSCols, g.k - ss * kSSCols) / cols_per_slot(fmt);
}

// Sum the per-wave partials acc[t] of the block in wave order into wave 0.
// red: nwaves * NT * 64 floats of LDS. Returns true on wave 0.
template <int NT, typename V>
__device__ __forceinline__ bool block_reduce(V (&acc)[NT], V* red, int wave, int lane, int nwaves) {
#pragma unroll
  for (int t = 0; t < NT; ++t) red[(wave * NT + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (wave != 0) return false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    V s = red[t * 64 + lane];
    for (int w = 1; w < nwaves; ++w) s += red[(w * NT + t) * 64 + lane];
    acc[t] = s;
  }
  return true;
}

// Last-block protocol: every thread's global writes are released before one
// thread bumps the counter; the block that brings it to `expect` acquires and
// resets it.
__device__ __forceinline__ bool arrive_last(unsigned* ctr, unsigned expect, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old + 1 == expect);
    if (old + 1 == expect) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------------------
// Kernel arguments.

struct Dims {
  int T, H, L, E, K, G, F, Fs;
  int du_fmt;
};

struct P1 {
  Dims d;
  const float* x;          // [T][H]
  const float* rms;        // [T] or null: multiply dot products by rms[t]
  const uint8_t* router; Geom gr;
  const float* bias;
  const uint8_t* labels;
  const uint8_t* dmat; Geom gd;
  const uint8_t* sgu; Geom gs;
  int nrb, nch, cw;        // router blocks, column chunks per tile, columns per chunk
  int ndb;                 // D blocks
  Workspace ws;
};

struct P2 {
  Dims d;
  const uint8_t* experts; Geom ggu; size_t stride, ts_off;
  const uint8_t* labels;
  Workspace ws;
};

struct P3 {
  Dims d;
  const uint8_t* experts; Geom gdn; size_t stride, gu_bytes, ts_off;
  const uint8_t* labels;
  Workspace ws;
};

struct P4 {
  Dims d;
  const uint8_t* umat; Geom gu;
  const uint8_t* sdn; Geom gsd;
  float* y;
  int accumulate;          // y += result (block forward) instead of y = result
  Workspace ws;
};

// ---------------------------------------------------------------------------
// Routing, done by the last router block.

template <int T>
__device__ void routing(const P1& a, char* smem) {
  const Dims& d = a.d;
  const Workspace& ws = a.ws;
  const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nw = nth >> 6;
  const int Epad = a.gr.tiles * 64;

  // logits = sum of chunk partials in chunk order (+ bias)
  for (int i = tid; i < T * d.E; i += nth) {
    int t = i / d.E, e = i % d.E;
    double s = 0.0;
    for (int c = 0; c < a.nch; ++c) s += ws.part64[((size_t)c * T + t) * Epad + e];
    if (a.rms) s *= (double)a.rms[t];
    s += (double)a.bias[e];
    ws.logits[i] = s;
  }
  __syncthreads();

  // top K per token, one wavefront per token: K rounds of a wave arg-max over
  // (logit desc, expert asc); then the softmax of the kept logits
  for (int t = wave; t < T; t += nw) {
    double v[16];
    const int per = (d.E + 63) / 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int e = lane + 64 * i;
      v[i] = (i < per && e < d.E) ? ws.logits[t * d.E + e] : -INFINITY;
    }
    double kept[64];
    double l0 = 0.0;
    for (int k = 0; k < d.K; ++k) {
      double bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int e = lane + 64 * i;
        if (v[i] > bv || (v[i] == bv && e < bi)) { bv = v[i]; bi = e; }
      }
      for (int o = 32; o > 0; o >>= 1) {
        double ov = __shfl_xor(bv, o);
        int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i == (bi >> 6)) v[i] = -INFINITY;
      }
      if (k == 0) l0 = bv;
      if (lane == 0) ws.topk_idx[t * d.K + k] = bi;
      if (k < 64) kept[k] = bv;
    }
    if (lane == 0) {
      double z = 0.0;
      for (int k = 0; k < d.K; ++k) z += exp(kept[k] - l0);
      for (int k = 0; k < d.K; ++k) ws.topk_w[t * d.K + k] = (float)(exp(kept[k] - l0) / z);
    }
  }
  __syncthreads();

  // stable rank of each assignment by key (label, expert)
  const int n = T * d.K;
  int* key = (int*)smem;           // [n]
  int* sperm = key + n;            // [n]
  int* start = sperm + n;          // [n] slot start flags, then slot ids
  for (int i = tid; i < n; i += nth) {
    int e = ws.topk_idx[i];
    key[i] = (int)a.labels[e] * d.E + e;
  }
  __syncthreads();
  for (int i = tid; i < n; i += nth) {
    int ki = key[i], r = 0;
    for (int j = 0; j < n; ++j) {
      int kj = key[j];
      r += (kj < ki) || (kj == ki && j < i);
    }
    sperm[r] = i;
    ws.perm[r] = i;
    ws.inv[i] = r;
  }
  __syncthreads();
  for (int j = tid; j < n; j += nth)
    start[j] = (j == 0 || key[sperm[j]] != key[sperm[j - 1]]) ? 1 : 0;
  __syncthreads();
  for (int j = tid; j < n; j += nth) {
    if (!start[j]) continue;
    int sid = 0;
    for (int q = 0; q < j; ++q) sid += start[q];
    int end = j + 1;
    while (end < n && !start[end]) ++end;
    ws.slot_expert[sid] = key[sperm[j]] % d.E;
    ws.slot_start[sid] = j;
    ws.slot_count[sid] = end - j;
  }
  __syncthreads();
  if (tid == 0) {
    int ns = 0;
    for (int j = 0; j < n; ++j) ns += start[j];
    *ws.n_slots = ns;
  }
  for (int g = tid; g <= d.G; g += nth) {
    int gs = 0, ga = 0;
    for (int j = 0; j < n; ++j) {
      int lab = key[sperm[j]] / d.E;
      if (lab < g) {
        ga += 1;
        gs += start[j];
      }
    }
    ws.gslot_off[g] = gs;
    ws.group_off[g] = ga;
  }
  for (int e = tid; e < d.E; e += nth) {
    int c = 0;
    for (int j = 0; j < n; ++j) c += (key[j] % d.E) == e;
    ws.expert_count[e] = c;
  }
}

// ---------------------------------------------------------------------------
// Phase 1: router | D_g | shared gate/up, by block index range.

template <int T>
__global__ __launch_bounds__(1024) void k_phase1(P1 a) {
  extern __shared__ char smem[];
  const Dims& d = a.d;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int b = blockIdx.x;
  __shared__ int flag;

  if (b < a.nrb) {
    // router: tile r, column chunk c; wave w covers 64 columns
    const int r = b / a.nch, c = b % a.nch;
    const int col0 = c * a.cw + wave * 64;
    double acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0;
    if (col0 < d.H) {
      const int nslot = min(64, d.H - col0) / 8;
      const uint8_t* p = a.router + ((size_t)r * a.gr.tile_slots + col0 / 8) * kSlot + lane * 16;
      cf_t xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t] = cf(a.x + (size_t)t * d.H + col0);
      chunk_bf16_f64<T>(p, nslot, xv, acc);
    }
    double* red = (double*)smem;
    if (block_reduce<T>(acc, red, wave, lane, nw)) {
      const int Epad = a.gr.tiles * 64;
#pragma unroll
      for (int t = 0; t < T; ++t) a.ws.part64[((size_t)c * T + t) * Epad + r * 64 + lane] = acc[t];
    }
    if (arrive_last(a.ws.ctr_router, (unsigned)a.nrb, &flag)) routing<T>(a, smem);
    return;
  }

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
  float* red = (float*)smem;
  if (b < a.nrb + a.ndb) {
    // D_g, tile r; wave = super-step
    const int i = b - a.nrb;
    const int tiles = a.gd.tiles;
    const int g = i / tiles, r = i % tiles;
    if (wave < a.gd.nss) {
      const uint8_t* base = a.dmat + (size_t)g * a.gd.bytes();
      cf_t xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t] = cf(a.x + (size_t)t * d.H + wave * kSSCols);
      ss_du<T>(d.du_fmt, tile_ptr(base, a.gd, r, wave, lane), ss_codes(d.du_fmt, a.gd, wave),
                     xv, acc);
    }
    if (block_reduce<T>(acc, red, wave, lane, nw)) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float v = acc[t];
        if (a.rms) v *= a.rms[t];
        a.ws.xl[((size_t)t * d.G + g) * d.L + r * 64 + lane] = v;
      }
    }
    return;
  }
  // shared gate/up pairs, tile r: lanes 0..31 gate rows, 32..63 up rows
  const int r = b - a.nrb - a.ndb;
  if (wave < a.gs.nss) {
    cf_t xv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xv[t] = cf(a.x + (size_t)t * d.H + wave * kSSCols);
    ss_bf16<T>(tile_ptr(a.sgu, a.gs, r, wave, lane), ss_codes(kBF16, a.gs, wave), xv, acc);
  }
  if (block_reduce<T>(acc, red, wave, lane, nw)) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v = acc[t];
      if (a.rms) v *= a.rms[t];
      const float other = __shfl_xor(v, 32);
      const int f = r * 32 + lane;
      if (lane < 32 && f < d.Fs) a.ws.hs[(size_t)t * d.Fs + f] = silu(v) * other;
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 2: routed-expert gate/up + SwiGLU.

template <int NA>
__device__ __forceinline__ void expert_gateup(const P2& a, int e, int g, int start, int r,
                                              int wave, int lane, int nw, char* smem) {
  const Dims& d = a.d;
  float acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = 0.f;
  const uint8_t* base = a.experts + (size_t)e * a.stride;
  if (wave < a.ggu.nss) {
    cf_t xv[NA];
    ci_t perm = ci(a.ws.perm);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int t = perm[start + i] / d.K;
      xv[i] = cf(a.ws.xl + ((size_t)t * d.G + g) * d.L + wave * kSSCols);
    }
    ss_fp4<NA>(tile_ptr(base, a.ggu, r, wave, lane), ss_codes(kFP4, a.ggu, wave), xv, acc);
  }
  if (block_reduce<NA>(acc, (float*)smem, wave, lane, nw)) {
    cf_t ts = cf((const float*)(base + a.ts_off));
    const float s = lane < 32 ? ts[0] : ts[1];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const float v = acc[i] * s;
      const float other = __shfl_xor(v, 32);
      const int f = r * 32 + lane;
      if (lane < 32 && f < d.F) a.ws.hbuf[(size_t)(start + i) * d.F + f] = silu(v) * other;
    }
  }
}

template <int T>
__global__ __launch_bounds__(1024) void k_phase2(P2 a) {
  extern __shared__ char smem[];
  const int tiles = a.ggu.tiles;
  const int j = blockIdx.x / tiles, r = blockIdx.x % tiles;
  ci_t ns = ci(a.ws.n_slots);
  if (j >= ns[0]) return;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int e = ci(a.ws.slot_expert)[j], start = ci(a.ws.slot_start)[j];
  const int cnt = ci(a.ws.slot_count)[j];
  const int g = ((cu8_t)a.labels)[e];
  switch (cnt) {
    case 1: expert_gateup<1>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 2: if constexpr (T >= 2) expert_gateup<2>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 3: if constexpr (T >= 3) expert_gateup<3>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 4: if constexpr (T >= 4) expert_gateup<4>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 5: if constexpr (T >= 5) expert_gateup<5>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 6: if constexpr (T >= 6) expert_gateup<6>(a, e, g, start, r, wave, lane, nw, smem); break;
    case 7: if constexpr (T >= 7) expert_gateup<7>(a, e, g, start, r, wave, lane, nw, smem); break;
    default: if constexpr (T >= 8) expert_gateup<8>(a, e, g, start, r, wave, lane, nw, smem); break;
  }
}

// ---------------------------------------------------------------------------
// Phase 3: routed-expert down, scaled by the routing weight; per-group sums.

template <int NA>
__device__ __forceinline__ void expert_down(const P3& a, int e, int start, int r, int wave,
                                            int lane, int nw, char* smem) {
  const Dims& d = a.d;
  float acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = 0.f;
  const uint8_t* base = a.experts + (size_t)e * a.stride;
  if (wave < a.gdn.nss) {
    cf_t xv[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) xv[i] = cf(a.ws.hbuf + (size_t)(start + i) * d.F + wave * kSSCols);
    ss_fp4<NA>(tile_ptr(base + a.gu_bytes, a.gdn, r, wave, lane), ss_codes(kFP4, a.gdn, wave), xv,
               acc);
  }
  if (block_reduce<NA>(acc, (float*)smem, wave, lane, nw)) {
    cf_t ts = cf((const float*)(base + a.ts_off));
    ci_t perm = ci(a.ws.perm);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const float w = a.ws.topk_w[perm[start + i]];
      a.ws.obuf[(size_t)(start + i) * d.L + r * 64 + lane] = acc[i] * ts[2] * w;
    }
  }
}

template <int T>
__global__ __launch_bounds__(1024) void k_phase3(P3 a) {
  extern __shared__ char smem[];
  __shared__ int flag;
  const Dims& d = a.d;
  const int tiles = a.gdn.tiles;
  const int j = blockIdx.x / tiles, r = blockIdx.x % tiles;
  ci_t ns = ci(a.ws.n_slots);
  if (j >= ns[0]) return;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int e = ci(a.ws.slot_expert)[j], start = ci(a.ws.slot_start)[j];
  const int cnt = ci(a.ws.slot_count)[j];
  const int g = ((cu8_t)a.labels)[e];
  switch (cnt) {
    case 1: expert_down<1>(a, e, start, r, wave, lane, nw, smem); break;
    case 2: if constexpr (T >= 2) expert_down<2>(a, e, start, r, wave, lane, nw, smem); break;
    case 3: if constexpr (T >= 3) expert_down<3>(a, e, start, r, wave, lane, nw, smem); break;
    case 4: if constexpr (T >= 4) expert_down<4>(a, e, start, r, wave, lane, nw, smem); break;
    case 5: if constexpr (T >= 5) expert_down<5>(a, e, start, r, wave, lane, nw, smem); break;
    case 6: if constexpr (T >= 6) expert_down<6>(a, e, start, r, wave, lane, nw, smem); break;
    case 7: if constexpr (T >= 7) expert_down<7>(a, e, start, r, wave, lane, nw, smem); break;
    default: if constexpr (T >= 8) expert_down<8>(a, e, start, r, wave, lane, nw, smem); break;
  }
  ci_t gso = ci(a.ws.gslot_off);
  const unsigned expect = (unsigned)(gso[g + 1] - gso[g]);
  if (!arrive_last(a.ws.ctr_s + (size_t)g * tiles + r, expect, &flag)) return;
  // s[t][g][row] = sum over k ascending of o for token t's experts in group g
  if (wave == 0) {
    const int row = r * 64 + lane;
    for (int t = 0; t < T; ++t) {
      float s = 0.f;
      for (int k = 0; k < d.K; ++k) {
        const int ee = a.ws.topk_idx[t * d.K + k];
        if (a.labels[ee] == g) s += a.ws.obuf[(size_t)a.ws.inv[t * d.K + k] * d.L + row];
      }
      a.ws.s[((size_t)t * d.G + g) * d.L + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 4: U_g per used group and the shared down; ordered sum per row tile.

template <int T>
__global__ __launch_bounds__(1024) void k_phase4(P4 a) {
  extern __shared__ char smem[];
  __shared__ int flag;
  const Dims& d = a.d;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int tiles = a.gu.tiles;      // H / 64
  const int b = blockIdx.x;
  const int part = b / tiles, r = b % tiles;   // part < G: U_part; part == G: shared down
  ci_t gso = ci(a.ws.gslot_off);
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
  bool active;
  if (part < d.G) {
    active = gso[part + 1] > gso[part];
    if (active && wave < a.gu.nss) {
      cf_t xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t] = cf(a.ws.s + ((size_t)t * d.G + part) * d.L + wave * kSSCols);
      ss_du<T>(d.du_fmt, tile_ptr(a.umat + (size_t)part * a.gu.bytes(), a.gu, r, wave, lane),
                     ss_codes(d.du_fmt, a.gu, wave), xv, acc);
    }
  } else {
    active = true;
    if (wave < a.gsd.nss) {
      cf_t xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t] = cf(a.ws.hs + (size_t)t * d.Fs + wave * kSSCols);
      ss_bf16<T>(tile_ptr(a.sdn, a.gsd, r, wave, lane), ss_codes(kBF16, a.gsd, wave), xv, acc);
    }
  }
  if (active && block_reduce<T>(acc, (float*)smem, wave, lane, nw)) {
#pragma unroll
    for (int t = 0; t < T; ++t) a.ws.ypart[((size_t)part * T + t) * d.H + r * 64 + lane] = acc[t];
  }
  if (!arrive_last(a.ws.ctr_y + r, (unsigned)(d.G + 1), &flag)) return;
  if (wave == 0) {
    const int row = r * 64 + lane;
    for (int t = 0; t < T; ++t) {
      float y = 0.f;
      for (int g = 0; g < d.G; ++g)
        if (gso[g + 1] > gso[g]) y += a.ws.ypart[((size_t)g * T + t) * d.H + row];
      y += a.ws.ypart[((size_t)d.G * T + t) * d.H + row];
      float* dst = a.y + (size_t)t * d.H + row;
      *dst = a.accumulate ? *dst + y : y;
    }
  }
}

// 1/sqrt(mean(x^2) + eps) per row, fp64 sum.
__global__ void k_rms(const float* __restrict__ x, int H, float eps, float* __restrict__ out) {
  const int t = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    double v = x[(size_t)t * H + i];
    s += v * v;
  }
  __shared__ double red[1024];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double z = 0.0;
    for (int i = 0; i < (int)blockDim.x; ++i) z += red[i];
    out[t] = (float)(1.0 / sqrt(z / H + (double)eps));
  }
}

template <int T>
int launch_all(lmoe_t* h, const float* x, float* y, bool norm, hipStream_t st) {
  const lmoe_dims& dd = h->d;
  Dims d{T, dd.hidden, dd.latent, dd.n_experts, dd.top_k, dd.n_groups, dd.expert_ffn,
         dd.shared_ffn, dd.du_bits == 8 ? kQ8 : kQ4};
  Workspace ws = h->ws;
  const bool ev = h->phase_events.size() == (size_t)kDecodePhases + 1;
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[0], st));

  // phase 1
  P1 p1{};
  p1.d = d;
  p1.x = x;
  p1.rms = norm ? ws.rms : nullptr;
  p1.router = h->router; p1.gr = h->g_router;
  p1.bias = h->bias;
  p1.labels = h->labels;
  p1.dmat = h->dmat; p1.gd = h->g_d;
  p1.sgu = h->sgu; p1.gs = h->g_sgu;
  const int nw1 = h->g_d.nss;               // waves per phase-1 block = H / 256
  p1.cw = nw1 * 64;
  p1.nch = ws.nch;
  p1.nrb = h->g_router.tiles * p1.nch;
  p1.ndb = d.G * h->g_d.tiles;
  p1.ws = ws;
  const int nb1 = p1.nrb + p1.ndb + h->g_sgu.tiles;
  const int n = T * d.K;
  size_t sm1 = (size_t)nw1 * T * 64 * sizeof(double);
  sm1 = sm1 > (size_t)3 * n * sizeof(int) ? sm1 : (size_t)3 * n * sizeof(int);
  hipLaunchKernelGGL(k_phase1<T>, dim3(nb1), dim3(nw1 * 64), sm1, st, p1);
  LMOE_HIP(hipGetLastError());

  const int maxslots = n < d.E ? n : d.E;
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[1], st));
  // phase 2
  P2 p2{};
  p2.d = d; p2.experts = h->experts; p2.ggu = h->g_gu; p2.stride = h->expert_stride;
  p2.ts_off = h->ts_off; p2.labels = h->labels; p2.ws = ws;
  const int nw2 = h->g_gu.nss;
  hipLaunchKernelGGL(k_phase2<T>, dim3(maxslots * h->g_gu.tiles), dim3(nw2 * 64),
                     (size_t)nw2 * T * 64 * sizeof(float), st, p2);
  LMOE_HIP(hipGetLastError());

  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[2], st));
  // phase 3
  P3 p3{};
  p3.d = d; p3.experts = h->experts; p3.gdn = h->g_dn; p3.stride = h->expert_stride;
  p3.gu_bytes = h->g_gu.bytes(); p3.ts_off = h->ts_off; p3.labels = h->labels; p3.ws = ws;
  const int nw3 = h->g_dn.nss;
  hipLaunchKernelGGL(k_phase3<T>, dim3(maxslots * h->g_dn.tiles), dim3(nw3 * 64),
                     (size_t)nw3 * T * 64 * sizeof(float), st, p3);
  LMOE_HIP(hipGetLastError());

  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[3], st));
  // phase 4
  P4 p4{};
  p4.d = d; p4.umat = h->umat; p4.gu = h->g_u; p4.sdn = h->sdn; p4.gsd = h->g_sdn;
  p4.y = y; p4.accumulate = norm ? 1 : 0; p4.ws = ws;
  const int nw4 = h->g_u.nss > h->g_sdn.nss ? h->g_u.nss : h->g_sdn.nss;
  hipLaunchKernelGGL(k_phase4<T>, dim3((d.G + 1) * h->g_u.tiles), dim3(nw4 * 64),
                     (size_t)nw4 * T * 64 * sizeof(float), st, p4);
  LMOE_HIP(hipGetLastError());
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[4], st));
  return 0;
}

}  // namespace

int rms_rows(lmoe_t* h, const float* x, int T, float eps, hipStream_t st) {
  hipLaunchKernelGGL(k_rms, dim3(T), dim3(256), 0, st, x, h->d.hidden, eps, h->ws.rms);
  LMOE_HIP(hipGetLastError());
  return 0;
}

int forward_decode(lmoe_t* h, const float* x, int T, float* y, bool norm, hipStream_t st) {
  switch (T) {
    case 1: return launch_all<1>(h, x, y, norm, st);
    case 2: return launch_all<2>(h, x, y, norm, st);
    case 3: return launch_all<3>(h, x, y, norm, st);
    case 4: return launch_all<4>(h, x, y, norm, st);
    case 5: return launch_all<5>(h, x, y, norm, st);
    case 6: return launch_all<6>(h, x, y, norm, st);
    case 7: return launch_all<7>(h, x, y, norm, st);
    case 8: return launch_all<8>(h, x, y, norm, st);
    default: return LMOE_EUNSUPPORTED;
  }
}

}  // namespace lm
