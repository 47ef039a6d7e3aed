// Decode / speculative-verify forward (T <= 8 tokens): four launches built on
// a small-batch GEMV that runs its multiply-adds on the matrix cores.
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
// GEMV core: a wavefront takes one super-step (256 columns) of one 64-row
// tile. It reads the weights once with nontemporal 16-byte lane loads
// (1 KiB coalesced per slot), decodes them in registers to fp16 (Q8, Q4,
// NVFP4 with its E4M3 block scale folded in exactly) or uses bf16 as is, and
// multiplies them on v_mfma_f32_16x16x32_{f16,bf16} with the tokens on the
// M side (up to 16 tokens cost the same). Activations are split exactly
// enough to keep fp32 accuracy: fp16 hi + lo (22 bits) against fp16
// weights, three bf16 parts (exact) against bf16 weights. At T = 4 this
// leaves the vector ALUs about 24 instructions per KiB of weights, so the
// kernels are bound by HBM, not by decode arithmetic.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "internal.h"

namespace lm {
namespace {

typedef const __attribute__((address_space(4))) float* cf_t;     // uniform, read-only
typedef const __attribute__((address_space(4))) int* ci_t;
typedef const __attribute__((address_space(4))) uint8_t* cu8_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ cf_t cf(const float* p) { return (cf_t)p; }
__device__ __forceinline__ ci_t ci(const int* p) { return (ci_t)p; }

__device__ __forceinline__ uint4 ldw(const uint8_t* p) { return *(const uint4*)p; }
// weights are read once per forward: stream them past the caches
__device__ __forceinline__ uint4 ldnt(const uint8_t* p) {
  const u4v v = __builtin_nontemporal_load((const u4v*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Group label of expert e, read as a 32-bit scalar load (the label array is
// allocated in whole words).
__device__ __forceinline__ int label_of(const uint8_t* labels, int e) {
  typedef const __attribute__((address_space(4))) uint32_t* cu32_t;
  return (int)((((cu32_t)labels)[e >> 2] >> (8 * (e & 3))) & 0xFFu);
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

constexpr int kXStr = 264;        // staged activation row: 256 columns + 8 pad (halves)

// ---------------------------------------------------------------------------
// MFMA A operand: the token vectors of one super-step, staged per wavefront.

template <int NT>
struct XRegs {
  float4 v[NT];
};

// Lane l loads columns 4l..4l+3 of each of the n valid vectors (0 beyond).
template <int NT>
__device__ __forceinline__ void x_load(XRegs<NT>& r, const float* const (&src)[NT], int n,
                                       int cols, int lane) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    r.v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n && 4 * lane < cols) r.v[i] = *(const float4*)(src[i] + 4 * lane);
  }
}

// Maximum of a non-negative int over the wavefront, by DPP: row shifts give
// each row's maximum in its lane 15, two row broadcasts carry it to lane 63
// (lanes a shift or mask leaves out contribute 0).
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));   // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));   // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));   // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));   // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// fp16 hi/lo parts: xs[part][i][col], part 0 = hi, 1 = lo, of each vector
// scaled by an exact power of two 2^s_i chosen from its largest magnitude in
// this super-step (to [2^14, 2^15)) when that magnitude lies outside
// [2^-4, 2^14), so that neither part overflows or loses precision to the
// fp16 subnormals; inv[i] = 2^-s_i undoes it on the fp32 products.
// A vector whose largest magnitude is zero, subnormal, infinite or NaN is
// staged as is (inf and NaN then reach y, as in exact arithmetic).
template <int NT>
__device__ __forceinline__ bool x_stage_f16(const XRegs<NT>& r, _Float16* xs, int lane,
                                            float (&inv)[NT]) {
  bool any = false;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float v[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
    // largest |v| by its bit pattern (NaN sorts above inf)
    int mb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) mb = max(mb, (int)(__float_as_uint(v[j]) & 0x7FFFFFFFu));
    // A vector whose largest magnitude lies in [2^-4, 2^14) needs no scale
    // (its hi part cannot overflow, and the lo parts' absolute error of at
    // most 2^-25 is below 2^-21 of that magnitude): two ballots decide it,
    // and only other vectors pay for the exact wave maximum.
    const bool over = __ballot(mb >= 0x46800000) != 0ull;      // some |v| >= 2^14 (or inf, NaN)
    const bool some = __ballot(mb >= 0x3D800000) != 0ull;      // some |v| >= 2^-4
    int sh = 0;
    if (over || !some) {
      mb = wave_max_nonneg(mb);
      const int e = (mb >> 23) & 0xFF;                          // biased exponent of the maximum
      sh = (e == 0 || e == 255) ? 0 : max(-126, min(126, 141 - e));
    }
    const float sc = __int_as_float((127 + sh) << 23);
    inv[i] = __int_as_float((127 - sh) << 23);
    any = any || sh != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float u = v[j] * sc;
      const _Float16 hi = (_Float16)u;
      xs[(0 * NT + i) * kXStr + 4 * lane + j] = hi;
      xs[(1 * NT + i) * kXStr + 4 * lane + j] = (_Float16)(u - (float)hi);
    }
  }
  return any;
}

// The inverse scales of the tokens a lane holds in the MFMA D layout
// (tokens 4 (l / 16) + 0..3); 1 past NT.
template <int NT>
__device__ __forceinline__ f4 lane_inv(const float (&inv)[NT], int lane) {
  const int q = lane >> 4;
  f4 r = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (t / 4 == q) r[t % 4] = inv[t];
  return r;
}

// Three bf16 parts whose sum is the fp32 value exactly.
template <int NT>
__device__ __forceinline__ void x_stage_bf16(const XRegs<NT>& r, __bf16* xs, int lane) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float v[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 b1 = (__bf16)v[j];
      const float r1 = v[j] - (float)b1;
      const __bf16 b2 = (__bf16)r1;
      const __bf16 b3 = (__bf16)(r1 - (float)b2);
      xs[(0 * NT + i) * kXStr + 4 * lane + j] = b1;
      xs[(1 * NT + i) * kXStr + 4 * lane + j] = b2;
      xs[(2 * NT + i) * kXStr + 4 * lane + j] = b3;
    }
  }
}

template <int NT, typename E, typename V>
__device__ __forceinline__ V a_read(const E* xs, int part, int tok, int n, int col) {
  V z = {};
  return tok < n ? *(const V*)(xs + (part * NT + tok) * kXStr + col) : z;
}

// ---------------------------------------------------------------------------
// Weight decoding to MFMA B operands (8 values of one row).

// Q8 codes held offset-binary (q + 128): fp16 bits 0x6400 | u = 1024 + u,
// then minus 1152 gives q exactly.
__device__ __forceinline__ half8 dec_q8(uint32_t w0, uint32_t w1) {
  const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t d[4] = {__builtin_amdgcn_perm(0x64646464u, w0, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, w0, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, w1, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, w1, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(half2v, d[i]) - off;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// Q4: 8 offset-binary nibbles (q + 8); the device keeps element i in the low
// nibble of byte i and element i + 4 in its high nibble.
__device__ __forceinline__ half8 dec_q4(uint32_t w) {
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t d[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, lo, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, hi, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, hi, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(half2v, d[i]) - off;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// NVFP4: 8 E2M1 codes (element 2i in the low nibble of byte i) times their
// E4M3 block scale; e2m1 * e4m3 needs at most 6 significant bits and lies in
// [2^-10, 2688], so the fp16 product is exact.
__device__ __forceinline__ half8 dec_fp4(uint32_t w, _Float16 s) {
  const half2v ss = {s, s};
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// IQ4_NL: 8 indices into the format's 16-value table, in the Q4 nibble
// order. Four lookups per byte permute (indices 0..7 from the first half of
// the table, 8..15 from the second, picked by bit 3), the int8 values then
// offset-binary as for Q8; exact in fp16.
__device__ __forceinline__ uint32_t iq4_look(uint32_t ix) {
  constexpr uint32_t kT0 = 0xBFAD9881u, kT1 = 0xF6EADDCFu;     // -127 -104 -83 -65 | -49 -35 -22 -10
  constexpr uint32_t kT2 = 0x26190D01u, kT3 = 0x71594535u;     //    1   13  25  38 |  53  69  89 113
  const uint32_t sel = ix & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(kT1, kT0, sel), hi = __builtin_amdgcn_perm(kT3, kT2, sel);
  const uint32_t m = ((ix >> 3) & 0x01010101u) * 0xFFu;
  return ((hi & m) | (lo & ~m)) ^ 0x80808080u;
}
__device__ __forceinline__ half8 dec_iq4(uint32_t w) {
  const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t a = iq4_look(w & 0x0F0F0F0Fu), b = iq4_look((w >> 4) & 0x0F0F0F0Fu);
  const uint32_t d[4] = {__builtin_amdgcn_perm(0x64646464u, a, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, a, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, b, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, b, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(half2v, d[i]) - off;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// Q3_K: 8 weights of one 16-column run of a 32-column block: two low bits at
// bit sq of each byte of q0, q1, the high bit at bit sm of m0, m1; code
// u = low + 4 high in 0..7, weight (u - 4) times the run's integer scale
// s = scale - 32 (|product| <= 128: exact in fp16; the block's fp16 d is
// applied to the MFMA result).
__device__ __forceinline__ half8 dec_q3k(uint32_t q0, uint32_t q1, uint32_t m0, uint32_t m1, int sq,
                                         int sm, _Float16 s) {
  const half2v off = {(_Float16)1028.0f, (_Float16)1028.0f}, ss = {s, s};
  const uint32_t u0 = ((q0 >> sq) & 0x03030303u) | (((m0 >> sm) & 0x01010101u) << 2);
  const uint32_t u1 = ((q1 >> sq) & 0x03030303u) | (((m1 >> sm) & 0x01010101u) << 2);
  const uint32_t d[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, u0, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, u1, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, u1, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = (__builtin_bit_cast(half2v, d[i]) - off) * ss;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// One wavefront, one super-step of one 64-row tile (4 row groups of 16).
//
// Slot j of the super-step holds chunk j/4 of row group j%4; lane l owns row
// l%16 of the group and k-group l/16 of each 32-column block. The scale slot
// (scaled formats) holds, at lane-chunk 16*rg + r, the scales of row r of
// group rg. On return acc[rg] holds, in lane l, rows 16rg + l%16 for tokens
// 4(l/16) + 0..3 (the MFMA D layout).
//
// xs: this wave's staging area; src[i]: vector i at the super-step's first
// column; n: valid vectors; ncs: code slots present.
__host__ __device__ constexpr int cc_of(int fmt) {
  return fmt == kQ8 ? 64 : (fmt == kBF16 ? 32 : (fmt == kQ3K ? 256 : 128));
}

// SL: code slots the registers hold (a full super-step by default; fewer
// for waves that take only the first columns of one).
template <int FMT, int NT, int SL = FMT == kQ3K ? 6 : 4 * (kSSCols / cc_of(FMT))>
struct WRegs {
  static constexpr int CC = cc_of(FMT);   // columns per chunk
  static constexpr int NSL = SL;
  XRegs<NT> xr;
  uint4 sc[4];
  uint4 q[NSL];
};

// Issues the loads of one super-step: activations first, then scales, then
// the weight stream (loads are counted in order, so the staging waits only
// for its own data).
template <int FMT, int NT, int SL>
__device__ __forceinline__ void wave_load(WRegs<FMT, NT, SL>& R, const uint8_t* p, int ncs, int cols,
                                          const float* const (&src)[NT], int n, int lane) {
  const int tok = lane & 15;
  x_load<NT>(R.xr, src, n, cols, lane);
  if (FMT != kBF16) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) R.sc[rg] = ldw(p + ncs * kSlot + (rg * 16 + tok) * 16);
  }
#pragma unroll
  for (int j = 0; j < SL; ++j)
    if (j < ncs) R.q[j] = ldnt(p + j * kSlot + lane * 16);
}

// wave_load for loops over items: weights through resource w (the
// super-step's first slot at offset 0, ncs code slots then the scale slot),
// vector i of the activations at byte offset xoff[i] of resource x. All
// per-lane addresses are the one lane offset, which stays in a register
// across items instead of one 64-bit address per load.
// The weight half of wave_load_b: scales, then the code slots.
template <int FMT, int NT, int SL>
__device__ __forceinline__ void wave_load_wts(WRegs<FMT, NT, SL>& R, rsrc_t w, int ncs, int lane) {
  const int tok = lane & 15;
  if (FMT != kBF16) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) R.sc[rg] = ldb(w, 16 * tok, ncs * kSlot + rg * 256);
  }
#pragma unroll
  for (int j = 0; j < SL; ++j)
    if (j < ncs) R.q[j] = ldb<kAuxNT>(w, 16 * lane, j * kSlot);
}

template <int FMT, int NT, int SL>
__device__ __forceinline__ void wave_load_b(WRegs<FMT, NT, SL>& R, rsrc_t w, int ncs, rsrc_t x,
                                            const int (&xoff)[NT], int n, int cols, int lane) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    R.xr.v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n && 4 * lane < cols) {
      const uint4 v = ldb(x, 16 * lane, xoff[i]);
      R.xr.v[i] = __builtin_bit_cast(float4, v);
    }
  }
  wave_load_wts<FMT, NT, SL>(R, w, ncs, lane);
}

// The MFMAs of a loaded super-step (xs: this wave's staging area).
template <int FMT, int NT, int SL>
__device__ __forceinline__ void wave_compute(const WRegs<FMT, NT, SL>& R, int ncs, int n, void* xs,
                                             int lane, f4 (&acc)[4]) {
  constexpr int CC = WRegs<FMT, NT, SL>::CC;
  constexpr int MAXCH = SL / 4;
  const int tok = lane & 15, qg = lane >> 4;
  const uint4 (&sc)[4] = R.sc;
  const uint4 (&q)[SL] = R.q;
  float inv[NT];
  bool scaled = false;
  if (FMT == kBF16) x_stage_bf16<NT>(R.xr, (__bf16*)xs, lane);
  else scaled = x_stage_f16<NT>(R.xr, (_Float16*)xs, lane, inv);
  __builtin_amdgcn_wave_barrier();

  if constexpr (FMT == kQ3K) {
    // one super-block per row: slots 0..3 the low bits of row group rg,
    // slots 4, 5 the high-bit masks of row groups 0, 1 and 2, 3; the scale
    // slot the row's sub-block scales and d. The lane's k-group is half of
    // run qg / 2 of each 32-column block 4h + j, whose scale is number
    // 8h + 2j + qg / 2; d multiplies the chain of the super-step.
    const _Float16* x = (const _Float16*)xs;
    const int run = qg >> 1;
    f4 ch[4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) ch[rg] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int B = 0; B < 8; ++B) {
      const int h = B >> 2, j = B & 3;
      const int col = 32 * B + 8 * qg;
      const half8 ahb = a_read<NT, _Float16, half8>(x, 0, tok, n, col);
      const half8 alb = a_read<NT, _Float16, half8>(x, 1, tok, n, col);
      const int bsh = 8 * (2 * (j & 1) + run);       // the scale bytes' position for this run
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t lo4 = (word(sc[rg], j >> 1) >> (bsh + 4 * h)) & 0xFu;
        const uint32_t hi2 = (sc[rg].z >> (bsh + 2 * (2 * h + (j >> 1)))) & 3u;
        const _Float16 s = (_Float16)((int)(lo4 | (hi2 << 4)) - 32);
        const uint4& m = q[4 + (rg >> 1)];
        const half8 bw = dec_q3k(word(q[rg], 2 * h), word(q[rg], 2 * h + 1), word(m, 2 * (rg & 1)),
                                 word(m, 2 * (rg & 1) + 1), 2 * j, 4 * h + j, s);
        ch[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahb, bw, ch[rg], 0, 0, 0);
        ch[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alb, bw, ch[rg], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const float dd = h2f(sc[rg].w);
      if (!scaled) acc[rg] += dd * ch[rg];
      else acc[rg] += (dd * lane_inv<NT>(inv, lane)) * ch[rg];
    }
    return;
  }

  const int nch = ncs / 4;
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    if (c >= nch) break;
    if constexpr (FMT == kBF16) {
      const __bf16* x = (const __bf16*)xs;
      const int col = CC * c + 8 * qg;
      const bf16x8 a0 = a_read<NT, __bf16, bf16x8>(x, 0, tok, n, col);
      const bf16x8 a1 = a_read<NT, __bf16, bf16x8>(x, 1, tok, n, col);
      const bf16x8 a2 = a_read<NT, __bf16, bf16x8>(x, 2, tok, n, col);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, q[4 * c + rg]);
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[rg], 0, 0, 0);
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[rg], 0, 0, 0);
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b, acc[rg], 0, 0, 0);
      }
    } else {
      constexpr int NB = CC / 32;                      // 32-column blocks per chunk
      const _Float16* x = (const _Float16*)xs;
      // one 32-column block's A operands at a time; every acc[rg] still sums
      // in (chunk, block, hi before lo) order
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int col = CC * c + 32 * b + 8 * qg;
        const half8 ahb = a_read<NT, _Float16, half8>(x, 0, tok, n, col);
        const half8 alb = a_read<NT, _Float16, half8>(x, 1, tok, n, col);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const uint4 w = q[4 * c + rg];
          if constexpr (FMT == kFP4) {
            // block of 16 columns holding this lane's 8: 8c + 2b + qg/2
            const int k = 4 * c + b;                     // scale half-word index
            const uint32_t sb = (word(sc[rg], k >> 1) >> (16 * (k & 1) + 8 * (qg >> 1))) & 0xFFu;
            const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sb, 0);
            const half8 bw = dec_fp4(word(w, b), s);
            if (!scaled) {                               // wave-uniform
              acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahb, bw, acc[rg], 0, 0, 0);
              acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alb, bw, acc[rg], 0, 0, 0);
            } else {                                     // undo the token scales per block
              f4 d = {0.f, 0.f, 0.f, 0.f};
              d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahb, bw, d, 0, 0, 0);
              d = __builtin_amdgcn_mfma_f32_16x16x32_f16(alb, bw, d, 0, 0, 0);
              acc[rg] += d * lane_inv<NT>(inv, lane);
            }
          } else {
            const half8 bw = FMT == kQ8 ? dec_q8(word(w, 2 * b), word(w, 2 * b + 1))
                                        : FMT == kIQ4 ? dec_iq4(word(w, b)) : dec_q4(word(w, b));
            f4 d = {0.f, 0.f, 0.f, 0.f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahb, bw, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(alb, bw, d, 0, 0, 0);
            const int blk = NB * c + b;                  // fp16 scale of this 32-column block
            const float s = h2f(word(sc[rg], blk >> 1) >> (16 * (blk & 1)));
            if (!scaled) acc[rg] += s * d;
            else acc[rg] += (s * lane_inv<NT>(inv, lane)) * d;
          }
        }
      }
    }
  }
}

template <int FMT, int NT>
__device__ __forceinline__ void wave_ss(const uint8_t* p, int ncs, int cols,
                                        const float* const (&src)[NT], int n, void* xs,
                                        int lane, f4 (&acc)[4]) {
  WRegs<FMT, NT> R;
  wave_load<FMT, NT>(R, p, ncs, cols, src, n, lane);
  wave_compute<FMT, NT>(R, ncs, n, xs, lane, acc);
}

// Sum the per-wave MFMA accumulators of the block in wave order into wave 0.
// Only lane groups holding tokens < NT are exchanged. Returns true on wave 0.
template <int NT>
__device__ __forceinline__ bool block_reduce_mf(f4 (&acc)[4], f4* red, int wave, int lane, int nw) {
  constexpr int LN = 16 * ((NT + 3) / 4);
  if (lane < LN) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) red[(wave * 4 + rg) * LN + lane] = acc[rg];
  }
  __syncthreads();
  if (wave != 0) return false;
  if (lane < LN) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      f4 s = red[rg * LN + lane];
      for (int w = 1; w < nw; ++w) s += red[(w * 4 + rg) * LN + lane];
      acc[rg] = s;
    }
  }
  return true;
}

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

// Pointer to super-step `ss` of tile `tile` (lane offset not included).
__device__ __forceinline__ const uint8_t* ss_ptr(const uint8_t* base, const Geom& g, int tile,
                                                 int ss) {
  return base + ((size_t)tile * g.tile_slots + (size_t)ss * g.full) * kSlot;
}
__device__ __forceinline__ int ss_cols(const Geom& g, int ss) { return min(kSSCols, g.k - ss * kSSCols); }
__device__ __forceinline__ int ss_codes(int fmt, const Geom& g, int ss) {
  return ss_code_slots(fmt, ss_cols(g, ss));
}

// LDS bytes of one wave's staging area, and of the MFMA reduction.
template <int NT>
constexpr int stage_bytes() { return 3 * NT * kXStr * 2; }
template <int NT>
constexpr int red_bytes_per_wave() { return 4 * 16 * ((NT + 3) / 4) * 16; }

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
// Data handed from one block to another inside a kernel goes through
// coherent agent-scope accesses (they bypass the non-coherent cache levels
// of the XCDs), so no cache writeback or invalidation is needed.
template <typename V>
__device__ __forceinline__ void st_co(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V ld_co(const V* p) {
  return __hip_atomic_load((V*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-block protocol: each block waits until its coherent stores have
// completed, then one thread bumps the counter; the block that brings it to
// `expect` goes on (and resets the counter for the next forward).
__device__ __forceinline__ bool arrive_last(unsigned* ctr, unsigned expect, int* flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old + 1 == expect;
    *flag = last;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// Kernel arguments.

struct Dims {
  int T, H, L, E, K, G, F, Fs;
};

struct P1 {
  Dims d;
  const float* x;          // [T][H]
  float* rms;              // [T] or null (plain forward): block forward, 1/rms of
  double* rms64;           // each row, written by the routing for phase 2
  float eps;               // RMSNorm eps (block forward)
  const uint8_t* router; Geom gr;
  const float* bias;
  const uint8_t* labels;
  const uint8_t* dmat; Geom gd;
  const uint8_t* sgu; Geom gs;
  int nrb, nch, cw;        // router blocks, column chunks per tile, columns per chunk
  int ndb;                 // D tiles
  int nsh;                 // shared gate/up (tile, super-step) tasks
  Workspace ws;
};

struct P2 {
  Dims d;
  int nps;                 // shared gate/up partials (super-steps of H)
  const float* rms;        // [T] or null
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
  int hu;                  // super-steps of U's first half = waves of every block
  int nsb;                 // shared-down blocks per row tile
  const uint8_t* umat; Geom gu;
  const uint8_t* sdn; Geom gsd;
  float* y;
  int accumulate;          // y += result (block forward) instead of y = result
  Workspace ws;
};

// ---------------------------------------------------------------------------
// Routing, done by the last router block.

// Sum of a double over the wavefront (butterfly: every lane gets it).
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// LDS of the routing block: logits [T][Epad] (fp64, -inf past E), per-wave
// top-K scratch,
// then per assignment (at least 64 entries) key, sorted order, inverse,
// label and slot of each sorted position, expert and label; per expert a
// counter and its group label; the slot count.
__host__ __device__ constexpr size_t routing_lds_bytes(int T, int E, int Epad, int n, int nw) {
  return (size_t)T * Epad * 8 + (size_t)nw * 3 * 64 * 8 + (size_t)(7 * (n > 64 ? n : 64) + 2 * E + 8) * 4;
}

template <int T>
__device__ void routing(const P1& a, char* smem) {
  const Dims& d = a.d;
  const Workspace& ws = a.ws;
  const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nw = nth >> 6;
  const int Epad = a.gr.tiles * 64;
  const int n = T * d.K;
  const int na = n > 64 ? n : 64;  // assignment arrays, at least 64 entries
  double* lg = (double*)smem;      // [T][Epad] logits, -inf past E
  double* scr = lg + T * Epad;     // [nw][3][64] per-wave top-K scratch
  int* key = (int*)(scr + nw * 3 * 64);  // [n] (label * E + expert) * 64 + assignment % 64
  int* sperm = key + na;           // [n] sorted position -> assignment
  int* inv = sperm + na;           // [n] assignment -> sorted position
  int* slab = inv + na;            // [n] label at each sorted position
  int* sid = slab + na;            // [n] slot of each sorted position
  int* aexp = sid + na;            // [n] expert of each assignment
  int* alab = aexp + na;           // [n] group label of each assignment
  int* ecnt = alab + na;           // [E] assignments per expert
  int* elab = ecnt + d.E;          // [E] group label of each expert
  int* nslot = elab + d.E;         // [1]

  // block forward: 1/rms of each row from the router chunks' sums of x^2
  // (added in chunk order, fp64), kept for the logits and written for phase 2
  __shared__ double rr[kMaxDecodeT];
  if (a.rms) {
    if (tid < T) {
      double q = 0.0;
      for (int c = 0; c < a.nch; ++c) q += ld_co(ws.sqp + (size_t)c * T + tid);
      const double r = 1.0 / sqrt(q / d.H + (double)a.eps);
      rr[tid] = r;
      a.rms64[tid] = r;
      a.rms[tid] = (float)r;
    }
    __syncthreads();
  }
  // logits = the chunk partials summed in chunk order (scaled by 1/rms in the
  // block forward) + bias; the labels come in with the token-0 entries.
  // Every thread issues all its loads before summing.
  {
    constexpr int U = 4;
    const int total = T * d.E;
    for (int base = 0; base < total; base += U * nth) {
      double part[U][kRouterChunks];
      int lab[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = min(base + tid + u * nth, total - 1);
        const int t = i / d.E, e = i % d.E;
#pragma unroll
        for (int c = 0; c < kRouterChunks; ++c)
          part[u][c] = ld_co(ws.part64 + ((size_t)c * T + t) * Epad + e);
        lab[u] = t == 0 ? (int)a.labels[e] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + tid + u * nth;
        if (i < total) {
          const int t = i / d.E, e = i % d.E;
          double l = 0.0;
#pragma unroll
          for (int c = 0; c < kRouterChunks; ++c) l += part[u][c];
          if (a.rms) l *= rr[t];
          lg[t * Epad + e] = l + (double)a.bias[e];
          if (t == 0) elab[e] = lab[u];
        }
      }
    }
    for (int i = tid; i < T * (Epad - d.E); i += nth)
      lg[(i / (Epad - d.E)) * Epad + d.E + i % (Epad - d.E)] = -INFINITY;
  }
  for (int e = tid; e < d.E; e += nth) ecnt[e] = 0;
  __syncthreads();

  // Top K per token, one wavefront per token, exact. Candidates: the logits
  // whose fp32 rounding is >= theta32, the K-th largest fp32-rounded lane
  // maximum. Rounding is monotone, so theta32 = fl(K-th largest lane max)
  // <= fl(K-th largest logit) and every top-K logit is a candidate. The
  // candidates are ranked exactly in fp64 by (logit desc, expert asc): a
  // candidate's rank among them equals its rank among all experts when it is
  // in the top K. More than 64 candidates (heavy ties): rank among all
  // experts instead. A single wavefront runs this, so it is written for few
  // instructions: unique 64-bit keys, loops over the candidates only.
  const unsigned long long lower = (1ull << lane) - 1ull;
  for (int t = wave; t < T; t += nw) {
    const double* l = lg + t * Epad;
    const int per = Epad >> 6;
    unsigned long long* wk = (unsigned long long*)(scr + wave * 3 * 64);  // lane-max keys
    double* cv = scr + wave * 3 * 64 + 64;    // candidate values, then the picks
    int* we = (int*)(cv + 64);                // candidate experts, then the picks
    double m = -INFINITY;
#pragma unroll 8
    for (int j = 0; j < per; ++j) {
      const double x = l[j * 64 + lane];
      m = x > m ? x : m;
    }
    const float m32 = (float)m;
    const unsigned mb = __float_as_uint(m32);
    const unsigned mo = (mb & 0x80000000u) ? ~mb : (mb | 0x80000000u);   // order-preserving
    const unsigned long long mk = ((unsigned long long)mo << 6) | (unsigned)(63 - lane);
    wk[lane] = mk;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < 64; j += 2) {
      const ulonglong2 p = *(const ulonglong2*)(wk + j);
      r += (int)(p.x > mk) + (int)(p.y > mk);
    }
    // rank K - 1 exists (K <= 64) and is unique: its fp32 value is theta32
    const float theta = __shfl(m32, __builtin_ctzll(__ballot(r == d.K - 1)));
    int base = 0;
#pragma unroll 4
    for (int j = 0; j < per; ++j) {
      const double x = l[j * 64 + lane];
      const bool in = (float)x >= theta;
      const unsigned long long bm = __ballot(in);
      const int q = base + __popcll(bm & lower);
      if (in && q < 64) {
        cv[q] = x;
        we[q] = j * 64 + lane;
      }
      base += __popcll(bm);
    }
    const int c = base;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double kv = 0.0;
    int ki = 0;
    if (c <= 64) {
      const double mv = lane < c ? cv[lane] : 0.0;
      const int me = lane < c ? we[lane] : 0;
      int rank = 0;
#pragma unroll 4
      for (int q = 0; q < c; ++q) {
        const double x = cv[q];
        rank += (int)((x > mv) | ((x == mv) & (we[q] < me)));
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < c && rank < d.K) {
        cv[rank] = mv;
        we[rank] = me;
      }
    } else {
      __builtin_amdgcn_wave_barrier();
      for (int e0 = 0; e0 < d.E; e0 += 64) {
        const int e = e0 + lane;
        if (e < d.E) {
          const double x = l[e];
          int rk = 0;
          for (int j = 0; j < d.E; ++j) rk += (int)((l[j] > x) | ((l[j] == x) & (j < e)));
          if (rk < d.K) {
            cv[rk] = x;
            we[rk] = e;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane < d.K) {
      kv = cv[lane];
      ki = min(max(we[lane], 0), d.E - 1);   // in range even for NaN logits
    }
    // softmax over the K picks: exp relative to the largest, the denominator
    // summed in rank order
    const double ex = lane < d.K ? exp(kv - cv[0]) : 0.0;
    double* exs = (double*)wk;                // the lane-max keys are no longer needed
    if (lane < d.K) exs[lane] = ex;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double z = 0.0;
    for (int k = 0; k < d.K; ++k) z += exs[k];
    if (lane < d.K) {
      const int i = t * d.K + lane;
      const int g = elab[ki];
      ws.topk_idx[i] = ki;
      ws.topk_w[i] = (float)(ex / z);
      key[i] = (g * d.E + ki) * 64 + (i & 63);   // unique when n <= 64
      alab[i] = g;
      aexp[i] = ki;
      atomicAdd(&ecnt[ki], 1);
    }
  }
  __syncthreads();

  // stable order of the assignments by (label, expert): for n <= 64 the keys
  // are unique and an assignment's rank is the count of smaller keys; beyond,
  // ties in (label, expert) are broken by assignment index
  if (n <= 64) {
    if (wave == 0 && lane < n) {
      const int ki = key[lane];
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < n; ++j) r += (int)(key[j] < ki);
      sperm[r] = lane;
      inv[lane] = r;
      ws.perm[r] = lane;
    }
  } else {
    for (int i = tid; i < n; i += nth) {
      const int ki = key[i] >> 6;
      int r = 0;
      for (int j = 0; j < n; ++j) {
        const int kj = key[j] >> 6;
        r += (int)((kj < ki) | ((kj == ki) & (j < i)));
      }
      sperm[r] = i;
      inv[i] = r;
      ws.perm[r] = i;
    }
  }
  for (int e = tid; e < d.E; e += nth) ws.expert_count[e] = ecnt[e];
  __syncthreads();
  for (int j = tid; j < n; j += nth) slab[j] = alab[sperm[j]];
  // slot of each sorted position: prefix count of segment starts, by wave 0
  if (wave == 0) {
    int run = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool st = j < n && (j == 0 || (key[sperm[j]] >> 6) != (key[sperm[j - 1]] >> 6));
      const unsigned long long mk = __ballot(st);
      if (j < n) sid[j] = run + __popcll(mk & lower) + (st ? 0 : -1);
      run += __popcll(mk);
    }
    if (lane == 0) {
      *nslot = run;
      *ws.n_slots = run;
    }
  }
  __syncthreads();
  // slots: expert, first sorted position, count; group offsets (positions
  // and slots) from the boundaries of the sorted labels
  for (int j = tid; j < n; j += nth) {
    const int s0 = sid[j];
    if (j == 0 || sid[j - 1] != s0) {
      int end = j + 1;
      while (end < n && sid[end] == s0) ++end;
      ws.slot_expert[s0] = aexp[sperm[j]];
      ws.slot_start[s0] = j;
      ws.slot_count[s0] = end - j;
      // the xl rows (t * G + g) of the slot's tokens, padded with the first
      for (int i = 0; i < kMaxDecodeT; ++i)
        ws.slot_xrow[s0 * kMaxDecodeT + i] = (sperm[j + (j + i < end ? i : 0)] / d.K) * d.G + slab[j];
    }
    const int lo = j == 0 ? 0 : slab[j - 1] + 1;
    for (int g = lo; g <= slab[j]; ++g) {
      ws.group_off[g] = j;
      ws.gslot_off[g] = s0;
    }
    if (j == n - 1)
      for (int g = slab[j] + 1; g <= d.G; ++g) {
        ws.group_off[g] = n;
        ws.gslot_off[g] = *nslot;
      }
  }
  // for each (token, group): the sorted positions of its assignments, in
  // ascending k (the order the per-group sum takes)
  for (int q = tid; q < T * d.G; q += nth) {
    const int t = q / d.G, g = q % d.G;
    int c = 0;
    for (int k = 0; k < d.K; ++k)
      if (alab[t * d.K + k] == g) ws.tg_pos[q * d.K + c++] = inv[t * d.K + k];
    ws.tg_cnt[q] = c;
  }
}

// ---------------------------------------------------------------------------
// Shared expert gate/up, super-step ss of row tile r, by this wavefront
// alone: the partial pre-activations go to hsp[ss]; the start of phase 2
// adds them in super-step order and applies SwiGLU.

template <int T>
__device__ __forceinline__ void shared_gu_part(const P1& a, int r, int ss, char* xs, int lane) {
  const Dims& d = a.d;
  f4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = (f4){0.f, 0.f, 0.f, 0.f};
  const float* src[T];
#pragma unroll
  for (int t = 0; t < T; ++t) src[t] = a.x + (size_t)t * d.H + ss * kSSCols;
  wave_ss<kBF16, T>(ss_ptr(a.sgu, a.gs, r, ss), ss_codes(kBF16, a.gs, ss), ss_cols(a.gs, ss), src, T,
                    xs, lane, acc);
  float* out = a.ws.hsp + (size_t)ss * T * 2 * d.Fs;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 4 * (lane >> 4) + v;
      if (t < T) out[(size_t)t * 2 * d.Fs + r * 64 + rg * 16 + (lane & 15)] = acc[rg][v];
    }
}

// ---------------------------------------------------------------------------
// Phase 1: router | D_g (and on the first D blocks one shared gate/up
// super-step each), by block index range.

// W: most waves a block of this launch has (the register budget follows it)
template <int T, int DU, int W>
__global__ __launch_bounds__(64 * W) void k_phase1(P1 a) {
  extern __shared__ __align__(16) char smem[];
  const Dims& d = a.d;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int b = blockIdx.x;
  __shared__ int flag;

  if (b < a.nrb) {
    // router: tile r, column chunk c; wave w covers 64 columns (fp64)
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
    if (block_reduce<T>(acc, (double*)smem, wave, lane, nw)) {
      const int Epad = a.gr.tiles * 64;
#pragma unroll
      for (int t = 0; t < T; ++t)
        st_co(a.ws.part64 + ((size_t)c * T + t) * Epad + r * 64 + lane, acc[t]);
    }
    if (a.rms && r == 0) {
      // block forward: sum of x^2 over this chunk's columns (one a thread),
      // per token, fp64, for the routing's 1/rms
      __shared__ double sqw[16][kMaxDecodeT];
      const int col = c * a.cw + (int)threadIdx.x;
      double q[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const double v = (int)threadIdx.x < a.cw && col < d.H ? (double)a.x[(size_t)t * d.H + col] : 0.0;
        q[t] = wave_sum64(v * v);
      }
      if (lane == 0)
#pragma unroll
        for (int t = 0; t < T; ++t) sqw[wave][t] = q[t];
      __syncthreads();
      if ((int)threadIdx.x < T) {
        double sq = 0.0;
        for (int w = 0; w < nw; ++w) sq += sqw[w][threadIdx.x];
        st_co(a.ws.sqp + (size_t)c * T + threadIdx.x, sq);
      }
    }
    if (arrive_last(a.ws.ctr_router, (unsigned)a.nrb, &flag)) routing<T>(a, smem);
    return;
  }

  f4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = (f4){0.f, 0.f, 0.f, 0.f};
  char* xs = smem + wave * stage_bytes<T>();
  f4* red = (f4*)(smem + nw * stage_bytes<T>());
  const float* src[T];
#pragma unroll
  for (int t = 0; t < T; ++t) src[t] = a.x + (size_t)t * d.H + wave * kSSCols;

  // D_g, tile r; wave = super-step
  const int i = b - a.nrb;
  if (i < a.ndb) {
    const int g = i / a.gd.tiles, r = i % a.gd.tiles;
    if (wave < a.gd.nss)
      wave_ss<DU, T>(ss_ptr(a.dmat + (size_t)g * a.gd.bytes(), a.gd, r, wave),
                     ss_codes(DU, a.gd, wave), ss_cols(a.gd, wave), src, T, xs, lane, acc);
    // block forward: the block's waves cover every column (wave w: super-step
    // w), so the block forms each row's sum of x^2 itself (fp64)
    __shared__ double sqd[16][kMaxDecodeT];
    if (a.rms) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        double q = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = wave * kSSCols + 4 * lane + j;
          const double v = col < d.H ? (double)a.x[(size_t)t * d.H + col] : 0.0;
          q += v * v;
        }
        q = wave_sum64(q);
        if (lane == 0) sqd[wave][t] = q;
      }
    }
    if (block_reduce_mf<T>(acc, red, wave, lane, nw)) {
      float rt[T];
      if (a.rms) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          double q = 0.0;
          for (int w = 0; w < nw; ++w) q += sqd[w][t];
          rt[t] = (float)(1.0 / sqrt(q / d.H + (double)a.eps));
        }
      }
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 4 * (lane >> 4) + v;
          if (t < T) {
            float y = acc[rg][v];
            if (a.rms) y *= rt[t];
            a.ws.xl[((size_t)t * d.G + g) * d.L + r * 64 + rg * 16 + (lane & 15)] = y;
          }
        }
    }
  }
  // Then one wavefront of each of the first nsh of these blocks computes one
  // super-step of one shared gate/up tile: the D blocks end well before the
  // routing block, and spreading the shared weights over them keeps every
  // CU's share of the stream even.
  if (i < a.nsh && wave == i % nw) shared_gu_part<T>(a, i / a.gs.nss, i % a.gs.nss, xs, lane);
}

// ---------------------------------------------------------------------------
// Phases 2 to 4 run as many blocks as are resident at once; a block strides
// over the items (one item = one 64-row tile of one matrix, every wave one
// super-step of it) and issues the weight loads of its next item as soon as
// the MFMAs of the current one have consumed its registers, so that the
// reduction and the stores of an item overlap the loads of the next.
// The cross-wave reduction buffer alternates between two halves by item
// parity: wave 0 may still read one while the others fill the other.

// Phase 2: routed-expert gate/up + SwiGLU, item = (slot, tile).

// GU: the gate/up format (kFP4, or kQ3K for the Q3_K records)
template <int T, int GU>
__global__ __launch_bounds__(1024) void k_phase2(P2 a) {
  extern __shared__ __align__(16) char smem[];
  const Dims& d = a.d;
  const int tiles = a.ggu.tiles;
  ci_t ns = ci(a.ws.n_slots);
  const int nvalid = ns[0] * tiles;            // items of real slots come first
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  char* xs = smem + wave * stage_bytes<T>();
  f4* red0 = (f4*)(smem + nw * stage_bytes<T>());
  const int red_len = nw * red_bytes_per_wave<T>() / (int)sizeof(f4);
  const bool active = wave < a.ggu.nss;

  // activations: xl [T][G][L] fp32; item (slot j, tile r)
  const rsrc_t xr = rsrc(a.ws.xl, (uint32_t)((size_t)T * d.G * d.L * sizeof(float)));
  const int wbytes = (ss_codes(GU, a.ggu, wave) + scale_slots(GU)) * kSlot;
  // Item (slot j, tile r): every table entry it needs comes in one round of
  // scalar loads (expert, count, the xl rows of its tokens written by the
  // routing), so its weight and activation loads start one load latency in.
  auto issue = [&](int item, WRegs<GU, T>& R) {
    const int j = item / tiles;
    const int e = ci(a.ws.slot_expert)[j], cnt = ci(a.ws.slot_count)[j];
    ci_t xrow = ci(a.ws.slot_xrow + j * kMaxDecodeT);
    int xoff[T];
#pragma unroll
    for (int i = 0; i < T; ++i) xoff[i] = (int)((xrow[i] * d.L + wave * kSSCols) * sizeof(float));
    const uint8_t* base = a.experts + (size_t)e * a.stride;
    wave_load_b<GU, T>(R, rsrc(ss_ptr(base, a.ggu, item % tiles, wave), wbytes),
                         ss_codes(GU, a.ggu, wave), xr, xoff, cnt, ss_cols(a.ggu, wave), lane);
  };
  WRegs<GU, T> R;
  int it = blockIdx.x;
  if (it < nvalid && active) issue(it, R);
  for (int par = 0; it < nvalid; it += gridDim.x, par ^= 1) {
    const int j = it / tiles, r = it % tiles;
    const int start = ci(a.ws.slot_start)[j], cnt = ci(a.ws.slot_count)[j];
    const uint8_t* base = a.experts + (size_t)ci(a.ws.slot_expert)[j] * a.stride;
    f4 acc[4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) acc[rg] = (f4){0.f, 0.f, 0.f, 0.f};
    if (active) wave_compute<GU, T>(R, ss_codes(GU, a.ggu, wave), cnt, xs, lane, acc);
    __builtin_amdgcn_sched_barrier(0);   // the next loads reuse this item's registers
    const int nx = it + gridDim.x;
    if (nx < nvalid && active) issue(nx, R);
    if (block_reduce_mf<T>(acc, red0 + par * red_len, wave, lane, nw)) {
      cf_t ts = cf((const float*)(base + a.ts_off));
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 4 * (lane >> 4) + v;
          const int f = r * 32 + rg * 16 + (lane & 15);
          if (i < cnt && f < d.F)
            a.ws.hbuf[(size_t)(start + i) * d.F + f] = silu(acc[rg][v] * ts[0]) * (acc[rg + 2][v] * ts[1]);
        }
    }
  }
  // shared expert: hs[t][f] = silu(g) * u from the phase-1 partials, summed
  // in super-step order (gate row f % 32 of tile f / 32 at tile row f % 32,
  // the up row 32 rows below). Done by the blocks that had one item fewer
  // (all blocks when the items divide evenly), after their items.
  {
    const int rem = nvalid % (int)gridDim.x;
    const int nc = rem > 0 ? (int)gridDim.x - rem : (int)gridDim.x;
    const int cb = (int)blockIdx.x - (rem > 0 ? rem : 0);
    const int nps = a.nps, Fs2 = 2 * d.Fs;
    if (cb >= 0) {
      for (int v = cb + nc * (int)threadIdx.x; v < T * d.Fs; v += nc * (int)blockDim.x) {
        const int t = v / d.Fs, f = v % d.Fs;
        const int row = (f >> 5) * 64 + (f & 31);
        const float* p = a.ws.hsp + (size_t)t * Fs2 + row;
        float gv = 0.f, uv = 0.f;
        for (int k0 = 0; k0 < nps; k0 += 8) {
          float gp[8], up[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            gp[k] = k0 + k < nps ? p[(size_t)(k0 + k) * T * Fs2] : 0.f;
            up[k] = k0 + k < nps ? p[(size_t)(k0 + k) * T * Fs2 + 32] : 0.f;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            gv += gp[k];
            uv += up[k];
          }
        }
        if (a.rms) {
          gv *= a.rms[t];
          uv *= a.rms[t];
        }
        a.ws.hs[v] = silu(gv) * uv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 3: routed-expert down, scaled by the routing weight.
//
// One block per (slot, 64-row tile r of ell), one wave per super-step of the
// ffn width, so that every block's loads are in flight at once and the
// blocks spread over the whole chip whatever the group sizes. The weighted
// outputs go to obuf [sorted position][ell]; phase 4 forms the per-group
// sums from them as it stages U's activations.

constexpr size_t kLdsBytes = 160 * 1024;   // LDS of one CU

// LDS of the fp16-staged kernels: hi and lo parts only.
template <int NT>
constexpr int stage_bytes_f16() { return 2 * NT * kXStr * 2; }

// waves of a phase-3 block: one per super-step, fewer if the LDS is short
template <int T>
constexpr int phase3_waves(int nss) {
  int n = nss < 16 ? nss : 16;
  while (n > 1 && (size_t)n * (stage_bytes_f16<T>() + red_bytes_per_wave<T>()) > kLdsBytes) --n;
  return n;
}

// DN: the down format (kFP4, or kIQ4 for the Q3_K records)
template <int T, int W, int DN>
__global__ __launch_bounds__(64 * W) void k_phase3(P3 a) {
  extern __shared__ __align__(16) char smem[];
  const Dims& d = a.d;
  const int tiles = a.gdn.tiles;                     // ell / 64
  const int j = blockIdx.x / tiles, r = blockIdx.x % tiles;
  // the slot's entries are read with the slot count (j < T * K: in bounds,
  // stale past the count), so the loads below wait one round, not two
  const int e = ci(a.ws.slot_expert)[j], start = ci(a.ws.slot_start)[j];
  const int cnt = ci(a.ws.slot_count)[j];
  if (j >= ci(a.ws.n_slots)[0]) return;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  ci_t perm = ci(a.ws.perm);
  const uint8_t* rec = a.experts + (size_t)e * a.stride;
  char* xs = smem + wave * stage_bytes_f16<T>();
  f4* red = (f4*)(smem + nw * stage_bytes_f16<T>());
  f4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = (f4){0.f, 0.f, 0.f, 0.f};
  // wave w takes super-steps w, w + nw, ... (nw = all of them unless the
  // LDS is short)
  for (int ss = wave; ss < a.gdn.nss; ss += nw) {
    int xoff[T];
#pragma unroll
    for (int i = 0; i < T; ++i)
      xoff[i] = (int)(((size_t)(start + (i < cnt ? i : 0)) * d.F + ss * kSSCols) * sizeof(float));
    const int ncs = ss_codes(DN, a.gdn, ss);
    WRegs<DN, T> R;
    wave_load_b<DN, T>(R, rsrc(ss_ptr(rec + a.gu_bytes, a.gdn, r, ss), (ncs + scale_slots(DN)) * kSlot),
                         ncs, rsrc(a.ws.hbuf, (uint32_t)((size_t)T * d.K * d.F * sizeof(float))), xoff, cnt,
                         ss_cols(a.gdn, ss), lane);
    wave_compute<DN, T>(R, ncs, cnt, xs, lane, acc);
  }
  if (block_reduce_mf<T>(acc, red, wave, lane, nw)) {
    cf_t ts = cf((const float*)(rec + a.ts_off));
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 4 * (lane >> 4) + v;
        const int row = r * 64 + rg * 16 + (lane & 15);
        if (i < cnt && row < d.L)
          a.ws.obuf[(size_t)(start + i) * d.L + row] = acc[rg][v] * ts[2] * a.ws.topk_w[perm[start + i]];
      }
  }
}

// ---------------------------------------------------------------------------
// Phase 4: U_g per used group and the shared down; ordered sum per row tile.
//
// U_g's ell columns are split into two halves of super-steps, so an item is
// (group g, half h, row tile r) or (shared down block k, row tile r): small
// blocks, several per CU, so that every item's loads are in flight in one
// round. Item (g, h) writes partial 2g + h of row tile r, shared down block
// k partial 2G + k; the partials are added in that order, by k_ysum after
// the kernel (SUMK) or by the last of a row tile's items to finish.

// U's activations for group g, columns of super-step ss (lane l: 4 l ..
// 4 l + 3): s[t][g] = the sum over token t's experts in group g of their
// weighted outputs, added in ascending k (0 where t has none in g). Each
// token's first kPreRows rows are loaded together (three at up to four
// tokens, fewer beyond, for the registers); more are rare.
template <int T>
__device__ __forceinline__ void group_sums(const P4& a, int g, int ss, int lane, XRegs<T>& X) {
  constexpr int kPreRows = T <= 4 ? 3 : T <= 6 ? 2 : 1;
  const Dims& d = a.d;
  ci_t cnt_tab = ci(a.ws.tg_cnt);
  ci_t pos_tab = ci(a.ws.tg_pos);
  const bool on = 4 * lane < ss_cols(a.gu, ss);
  const float* ob = a.ws.obuf + ss * kSSCols + 4 * lane;
  // the counts and the first positions in one round of scalar loads (the
  // positions read whatever the count; entries past it are not used)
  int c[T], pr[T][kPreRows];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int q = t * d.G + g;
    c[t] = cnt_tab[q];
#pragma unroll
    for (int i = 0; i < kPreRows; ++i) pr[t][i] = i < d.K ? pos_tab[q * d.K + i] : 0;
  }
  float4 u[T][kPreRows];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < kPreRows; ++i)
      u[t][i] = on && i < c[t] ? *(const float4*)(ob + (size_t)pr[t][i] * d.L) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kPreRows; ++i)
      if (i < c[t]) {
        v.x += u[t][i].x; v.y += u[t][i].y; v.z += u[t][i].z; v.w += u[t][i].w;
      }
    for (int i = kPreRows; i < c[t]; ++i) {
      const float4 w = on ? *(const float4*)(ob + (size_t)pos_tab[(t * d.G + g) * d.K + i] * d.L)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    X.v[t] = v;
  }
}

template <int T, int DU, int W, bool SUMK>
__global__ __launch_bounds__(64 * W) void k_phase4(P4 a) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int flag;
  const Dims& d = a.d;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int tiles = a.gu.tiles;                      // H / 64
  const int nu = 2 * d.G * tiles;
  const int b = blockIdx.x;
  ci_t gso = ci(a.ws.gslot_off);
  char* xs = smem + wave * stage_bytes<T>();
  f4* red = (f4*)(smem + nw * stage_bytes<T>());
  f4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = (f4){0.f, 0.f, 0.f, 0.f};
  int part, r;
  bool active;
  if (b < nu) {
    const int gh = b / tiles, g = gh >> 1, h = gh & 1;
    r = b % tiles;
    part = gh;
    active = gso[g + 1] > gso[g];
    const int ss = h * a.hu + wave;
    if (active && wave < a.hu && ss < a.gu.nss) {
      const int ncs = ss_codes(DU, a.gu, ss);
      const uint8_t* p = ss_ptr(a.umat + (size_t)g * a.gu.bytes(), a.gu, r, ss);
      WRegs<DU, T> R;
      group_sums<T>(a, g, ss, lane, R.xr);
      wave_load_wts<DU, T>(R, rsrc(p, (ncs + scale_slots(DU)) * kSlot), ncs, lane);
      wave_compute<DU, T>(R, ncs, T, xs, lane, acc);
    }
  } else {
    // shared down, block k of row tile r: wave w takes half-step
    // k * nw + w, i.e. half hs % 2 (128 columns, 16 code slots) of
    // super-step hs / 2, which keeps a bf16 wave's weights at 64 VGPRs
    const int k = (b - nu) / tiles;
    r = (b - nu) % tiles;
    part = 2 * d.G + k;
    active = true;
    const int hs = k * nw + wave;
    const int ss = hs >> 1, hf = hs & 1;
    const int cols = ss < a.gsd.nss ? min(128, ss_cols(a.gsd, ss) - 128 * hf) : 0;
    if (cols > 0) {
      const float* src[T];
#pragma unroll
      for (int t = 0; t < T; ++t) src[t] = a.ws.hs + (size_t)t * d.Fs + ss * kSSCols + 128 * hf;
      const int ncs = ss_code_slots(kBF16, cols);
      WRegs<kBF16, T, 16> R;
      wave_load<kBF16, T>(R, ss_ptr(a.sdn, a.gsd, r, ss) + (size_t)16 * hf * kSlot, ncs, cols, src, T,
                          lane);
      wave_compute<kBF16, T>(R, ncs, T, xs, lane, acc);
    }
  }
  if (active && block_reduce_mf<T>(acc, red, wave, lane, nw)) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 4 * (lane >> 4) + v;
        if (t < T) {
          float* q = a.ws.ypart + ((size_t)part * T + t) * d.H + r * 64 + rg * 16 + (lane & 15);
          if constexpr (SUMK) *q = acc[rg][v];
          else st_co(q, acc[rg][v]);
        }
      }
  }
  if constexpr (SUMK) return;                        // k_ysum adds the partials
  const int np = 2 * d.G + a.nsb;
  if (!arrive_last(a.ws.ctr_y + r, (unsigned)np, &flag)) return;
  // Ordered sum of the partials: wave w fetches parts w, w + nw, ..., up to
  // eight per pass with all their loads in flight together (one pass at the
  // 145B shape), then wave 0 adds them in part order.
  const int row = r * 64 + lane;
  float* stage = (float*)smem;                       // [np][T][64]
  constexpr int PW = 8;
  for (int base = 0; base < np; base += PW * nw) {
    float v[PW][T];
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int p = base + wave + k * nw;
#pragma unroll
      for (int t = 0; t < T; ++t) v[k][t] = p < np ? ld_co(a.ws.ypart + ((size_t)p * T + t) * d.H + row) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int p = base + wave + k * nw;
      if (p < np)
#pragma unroll
        for (int t = 0; t < T; ++t) stage[(p * T + t) * 64 + lane] = v[k][t];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float y = 0.f;
      for (int g = 0; g < d.G; ++g)
        if (gso[g + 1] > gso[g]) {
          y += stage[((2 * g) * T + t) * 64 + lane];
          y += stage[((2 * g + 1) * T + t) * 64 + lane];
        }
      for (int p = 2 * d.G; p < np; ++p) y += stage[(p * T + t) * 64 + lane];
      float* dst = a.y + (size_t)t * d.H + row;
      *dst = a.accumulate ? *dst + y : y;
    }
  }
}

// The ordered sum of phase 4's partials as a kernel of its own: block r
// takes row tile r, thread (t, lane) row 64 r + lane of token t, all its
// partials' loads in flight, added in part order (used groups only).
template <int T>
__global__ __launch_bounds__(512) void k_ysum(P4 a) {
  const Dims& d = a.d;
  const int r = blockIdx.x, lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t >= T) return;
  ci_t gso = ci(a.ws.gslot_off);
  const int np = 2 * d.G + a.nsb, row = r * 64 + lane;
  float y = 0.f;
  for (int p0 = 0; p0 < np; p0 += 8) {
    float v[8];
    bool use[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = p0 + k;
      use[k] = p < np && (p >= 2 * d.G || gso[p / 2 + 1] > gso[p / 2]);
      v[k] = use[k] ? a.ws.ypart[((size_t)p * T + t) * d.H + row] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (use[k]) y += v[k];
  }
  float* dst = a.y + (size_t)t * d.H + row;
  *dst = a.accumulate ? *dst + y : y;
}



// Blocks of `kernel` the device holds at once with `threads` threads and
// `lds` dynamic LDS bytes (the persistent phases launch that many).
int resident_blocks(lmoe_t* h, const void* kernel, int threads, size_t lds) {
  for (const auto& r : h->resident)
    if (r.kernel == kernel && r.threads == threads && r.lds == lds) return r.blocks;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess)
    return -1;
  const int n = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  h->resident.push_back({kernel, threads, lds, n});
  return n;
}

// only: 0 launches every phase, k in 1..4 phase k alone (its inputs are in
// the workspace from an earlier forward of T tokens)
// Phase 4's ordered sum: from four tokens on, a kernel of its own after
// phase 4 (no store-completion waits, arrival counters or coherent loads:
// 145B T 4 phase 4 18.1 -> 17.0 us, 120B T 5 17.9 -> 15.8); for fewer
// tokens the last-arriving block of each row tile (MTP T 1: 11.7 against
// 12.5 us as a kernel).
template <int T>
constexpr bool ysum_kernel() { return T >= 4; }

template <int T, int DU>
int launch_all(lmoe_t* h, const float* x, float* y, bool norm, hipStream_t st, int only,
               const Workspace& ws) {
  const lmoe_dims& dd = h->d;
  Dims d{T, dd.hidden, dd.latent, dd.n_experts, dd.top_k, dd.n_groups, dd.expert_ffn,
         dd.shared_ffn};
  const bool ev = only == 0 && h->phase_events.size() == (size_t)kDecodePhases + 1;
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[0], st));

  // phase 1
  P1 p1{};
  p1.d = d;
  p1.x = x;
  p1.rms = norm ? ws.rms : nullptr;
  p1.rms64 = norm ? ws.rms64 : nullptr;
  p1.eps = h->rms_eps;
  p1.router = h->router; p1.gr = h->g_router;
  p1.bias = h->bias;
  p1.labels = h->labels;
  p1.dmat = h->dmat; p1.gd = h->g_d;
  p1.sgu = h->sgu; p1.gs = h->g_sgu;
  const int nw1 = h->g_d.nss;               // waves per phase-1 block = H / 256
  p1.cw = nw1 * 64;
  p1.nch = kRouterChunks;
  p1.nrb = h->g_router.tiles * p1.nch;
  p1.ndb = d.G * h->g_d.tiles;
  p1.ws = ws;
  p1.nsh = h->g_sgu.tiles * h->g_sgu.nss;
  const int nb1 = p1.nrb + (p1.ndb > p1.nsh ? p1.ndb : p1.nsh);
  const int n = T * d.K;
  size_t sm1 = (size_t)nw1 * (stage_bytes<T>() + red_bytes_per_wave<T>());
  const size_t sm_router = (size_t)nw1 * T * 64 * sizeof(double);
  const size_t sm_routing = routing_lds_bytes(T, d.E, h->g_router.tiles * 64, n, nw1);
  sm1 = sm1 > sm_router ? sm1 : sm_router;
  sm1 = sm1 > sm_routing ? sm1 : sm_routing;
  if (only == 0 || only == 1) {
    if (nw1 <= 10)
      hipLaunchKernelGGL((k_phase1<T, DU, 10>), dim3(nb1), dim3(nw1 * 64), sm1, st, p1);
    else
      hipLaunchKernelGGL((k_phase1<T, DU, 16>), dim3(nb1), dim3(nw1 * 64), sm1, st, p1);
  }
  LMOE_HIP(hipGetLastError());
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[1], st));

  const int maxslots = n < d.E ? n : d.E;
  // phase 2
  P2 p2{};
  p2.d = d; p2.experts = h->experts; p2.ggu = h->g_gu; p2.stride = h->expert_stride;
  p2.ts_off = h->ts_off; p2.labels = h->labels; p2.ws = ws;
  p2.nps = h->g_sgu.nss; p2.rms = norm ? ws.rms : nullptr;
  const int nw2 = h->g_gu.nss;
  const size_t sm2 = (size_t)nw2 * (stage_bytes<T>() + 2 * red_bytes_per_wave<T>());
  const int items2 = maxslots * h->g_gu.tiles;
  const bool q3k = dd.expert_format == LMOE_EXPERTS_Q3K;
  const void* k2 = q3k ? (const void*)k_phase2<T, kQ3K> : (const void*)k_phase2<T, kFP4>;
  const int res2 = resident_blocks(h, k2, nw2 * 64, sm2);
  if (res2 <= 0) { set_error("phase 2: occupancy query failed"); return LMOE_EHIP; }
  if (only == 0 || only == 2) {
    const dim3 g2(items2 < res2 ? items2 : res2), b2(nw2 * 64);
    if (q3k) hipLaunchKernelGGL((k_phase2<T, kQ3K>), g2, b2, sm2, st, p2);
    else hipLaunchKernelGGL((k_phase2<T, kFP4>), g2, b2, sm2, st, p2);
  }
  LMOE_HIP(hipGetLastError());
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[2], st));

  // phase 3
  P3 p3{};
  p3.d = d; p3.experts = h->experts; p3.gdn = h->g_dn; p3.stride = h->expert_stride;
  p3.gu_bytes = h->g_gu.bytes(); p3.ts_off = h->ts_off; p3.labels = h->labels; p3.ws = ws;
  // Blocks of at most eight waves are compiled for 512 threads: they then
  // fit in 94 registers, five waves per SIMD, and every item of the 145B
  // shape is resident at once (at four waves per SIMD the items past 1024
  // waited a whole round)
  const int nw3 = phase3_waves<T>(h->g_dn.nss);
  const size_t sm3 = (size_t)nw3 * (stage_bytes_f16<T>() + red_bytes_per_wave<T>());
  const dim3 grid3((unsigned)(maxslots * h->g_dn.tiles)), block3(nw3 * 64);
  if (only == 0 || only == 3) {
    if (q3k) {
      if (nw3 <= 8) hipLaunchKernelGGL((k_phase3<T, 8, kIQ4>), grid3, block3, sm3, st, p3);
      else hipLaunchKernelGGL((k_phase3<T, 16, kIQ4>), grid3, block3, sm3, st, p3);
    } else {
      if (nw3 <= 8) hipLaunchKernelGGL((k_phase3<T, 8, kFP4>), grid3, block3, sm3, st, p3);
      else hipLaunchKernelGGL((k_phase3<T, 16, kFP4>), grid3, block3, sm3, st, p3);
    }
  }
  LMOE_HIP(hipGetLastError());
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[3], st));

  // phase 4
  P4 p4{};
  p4.d = d; p4.umat = h->umat; p4.gu = h->g_u; p4.sdn = h->sdn; p4.gsd = h->g_sdn;
  p4.y = y; p4.accumulate = norm ? 1 : 0; p4.ws = ws;
  // every block has hu waves (one per SIMD for hu = 4, so several blocks
  // share a CU evenly); the shared down takes ceil(half-steps / hu) blocks
  const int hu = (h->g_u.nss + 1) / 2;
  const int nhs = (dd.shared_ffn + 127) / 128;        // shared-down half super-steps
  p4.hu = hu;
  p4.nsb = (nhs + hu - 1) / hu;
  const int nw4 = hu;
  size_t sm4 = (size_t)nw4 * (stage_bytes<T>() + red_bytes_per_wave<T>());
  const size_t sm4r = (size_t)(2 * d.G + p4.nsb) * T * 64 * sizeof(float);
  sm4 = sm4 > sm4r ? sm4 : sm4r;
  const int grid4 = (2 * d.G + p4.nsb) * h->g_u.tiles;
  if (only == 0 || only == 4) {
    // blocks of up to eight waves compiled for 512 threads: 4-wave bounds
    // let the compiler spend AGPRs and drop to three waves per SIMD
    if (ysum_kernel<T>()) {
      if (nw4 <= 8)
        hipLaunchKernelGGL((k_phase4<T, DU, 8, true>), dim3(grid4), dim3(nw4 * 64), sm4, st, p4);
      else
        hipLaunchKernelGGL((k_phase4<T, DU, 16, true>), dim3(grid4), dim3(nw4 * 64), sm4, st, p4);
      hipLaunchKernelGGL((k_ysum<T>), dim3(h->g_u.tiles), dim3(64 * T), 0, st, p4);
    } else if (nw4 <= 8) {
      hipLaunchKernelGGL((k_phase4<T, DU, 8, false>), dim3(grid4), dim3(nw4 * 64), sm4, st, p4);
    } else {
      hipLaunchKernelGGL((k_phase4<T, DU, 16, false>), dim3(grid4), dim3(nw4 * 64), sm4, st, p4);
    }
  }
  LMOE_HIP(hipGetLastError());
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[4], st));
  return 0;
}

template <int T>
int launch_t(lmoe_t* h, const float* x, float* y, bool norm, hipStream_t st, int only,
             const Workspace& ws) {
  return h->d.du_bits == 8 ? launch_all<T, kQ8>(h, x, y, norm, st, only, ws)
                           : launch_all<T, kQ4>(h, x, y, norm, st, only, ws);
}

// Largest dynamic LDS any of the four kernels asks for at T tokens (the
// same sizes launch_all computes).
template <int T>
size_t lds_need(const lmoe_dims& d) {
  const int nssH = (d.hidden + kSSCols - 1) / kSSCols, nssL = (d.latent + kSSCols - 1) / kSSCols;
  const int Epad = (d.n_experts + 63) / 64 * 64, n = T * d.top_k;
  size_t m = (size_t)nssH * (stage_bytes<T>() + red_bytes_per_wave<T>());
  m = std::max(m, (size_t)nssH * T * 64 * sizeof(double));
  m = std::max(m, routing_lds_bytes(T, d.n_experts, Epad, n, nssH));
  m = std::max(m, (size_t)nssL * (stage_bytes<T>() + 2 * red_bytes_per_wave<T>()));
  const int nssF = (d.expert_ffn + kSSCols - 1) / kSSCols;
  m = std::max(m, (size_t)phase3_waves<T>(nssF) * (stage_bytes_f16<T>() + red_bytes_per_wave<T>()));
  const int hu = (nssL + 1) / 2, nhs = (d.shared_ffn + 127) / 128, nsb = (nhs + hu - 1) / hu;
  m = std::max(m, (size_t)hu * (stage_bytes<T>() + red_bytes_per_wave<T>()));
  m = std::max(m, (size_t)(2 * d.n_groups + nsb) * T * 64 * sizeof(float));
  return m;
}

}  // namespace

size_t decode_lds_bytes(const lmoe_dims& d, int T) {
  switch (T) {
    case 1: return lds_need<1>(d);
    case 2: return lds_need<2>(d);
    case 3: return lds_need<3>(d);
    case 4: return lds_need<4>(d);
    case 5: return lds_need<5>(d);
    case 6: return lds_need<6>(d);
    case 7: return lds_need<7>(d);
    default: return lds_need<8>(d);
  }
}


int forward_decode(lmoe_t* h, const float* x, int T, float* y, bool norm, hipStream_t st, int only,
                   const Workspace* ws) {
  const Workspace& w = ws ? *ws : h->ws;
  switch (T) {
    case 1: return launch_t<1>(h, x, y, norm, st, only, w);
    case 2: return launch_t<2>(h, x, y, norm, st, only, w);
    case 3: return launch_t<3>(h, x, y, norm, st, only, w);
    case 4: return launch_t<4>(h, x, y, norm, st, only, w);
    case 5: return launch_t<5>(h, x, y, norm, st, only, w);
    case 6: return launch_t<6>(h, x, y, norm, st, only, w);
    case 7: return launch_t<7>(h, x, y, norm, st, only, w);
    case 8: return launch_t<8>(h, x, y, norm, st, only, w);
    default: return LMOE_EUNSUPPORTED;
  }
}

}  // namespace lm
