// Prefill forward (T > 8 tokens): the layer as MFMA GEMMs.
//
// The layer is the one of "Edge0-145B: a Qwen MoE with its experts squeezed,
// and a 51B table left on the SSD", section "A latent in front of the
// experts" (layer equation; D over all groups, U once per group a token
// routed into), with the shapes and formats of the "Edge0 145B and Edge0
// 120B" model page ("Model profile" and architecture tables).
//
//   prep     x (or x / rms(x)) staged once: fp16 for D, two bf16 parts for
//            the router and the shared expert, and |x|_2 per token
//   router   logits on MFMA (bf16 x bf16 products are exact, fp32 sums);
//            per token every expert whose fp32 logit lies within twice the
//            rounding bound of the K-th largest is rescored in fp64, and
//            top-K and softmax are taken on the fp64 logits. The bound holds
//            for any summation order, so the kept set is the one exact
//            arithmetic gives.
//   permute  stable order of the assignments by (group label, expert): per
//            64-token chunk a bitmask per expert gives each assignment its
//            rank among earlier tokens of the chunk; chunk counts are
//            prefix-summed per expert. No sort, no atomics on positions.
//   D        dense GEMM over the stacked D_g: xl[t][g] = D_g x[t] (fp16)
//   experts  grouped GEMMs over the (label, expert) segments, in pieces of
//            up to 128 assignments: gate/up with SwiGLU in the epilogue
//            (fp16 h), down scaled by the routing weight (fp32 o)
//   combine  s[t][g] = sum of token t's outputs in group g, ascending k
//            (fp16; zero for groups t did not route into)
//   U        dense GEMM with the G matrices concatenated along K, followed in
//            the same accumulators by the shared expert's down projection
//   shared   gate/up GEMM with SwiGLU in the epilogue
//
// GEMM tile: 128 tokens x 256 weight rows (four 64-row tiles of the tiled
// stream) per 512-thread workgroup, two waves per SIMD. Wave w takes weight
// tile w/2 for tokens 64*(w%2) .. +63 with v_mfma_f32_32x32x16 (2 x 2
// accumulators of 32 x 32); the two waves of a SIMD overlap each other's
// MFMAs with their loads, LDS traffic and weight decoding. Per stage (128
// columns, 64 for 16-bit weights) the activation rows and the raw weight
// slots go through a double-buffered LDS ring, loads running two stages
// ahead. Weights are decoded in registers right before use: NVFP4 to fp16
// exactly (e2m1 * e4m3 <= 6 significant bits), bf16 / fp16 as stored. D and
// U run on fp16 copies made at load time with the same rounding the Q8/Q4
// decode has (fp16(q * d)). 32-token blocks past the last valid token are
// skipped (ragged tails, small expert segments).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "internal.h"

namespace lm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

constexpr int NTH = 512;       // threads per GEMM workgroup (8 waves)
constexpr int BM = 128;        // tokens per GEMM tile
constexpr int WTOK = 64;       // tokens per wave
constexpr int MB = WTOK / 32;  // 32-token MFMA blocks per wave
constexpr int NTW = 4;         // 64-row weight tiles per workgroup (two waves each)
constexpr int CHUNK_T = 64;    // tokens per permutation chunk
constexpr int kShortT = 32;    // expert pieces of at most 32 (64) tokens run in k_grouped_short<1> (<2>)

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }
// 1 / v for v a power of two in [2^-126, 2^127]: exact, from the exponent
__device__ __forceinline__ float inv_pow2(float v) {
  return __builtin_bit_cast(float, 0x7F000000u - __builtin_bit_cast(uint32_t, v));
}

// ---------------------------------------------------------------------------
// Weight decoding: the 8 columns one lane holds of one 32-column block.

__device__ __forceinline__ half8 q8_row8(uint32_t w0, uint32_t w1, _Float16 d) {
  // offset-binary q + 128 as the low byte of fp16 1024 + u, minus 1152 = q
  const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const half2v dd = {d, d};
  const uint32_t p[4] = {__builtin_amdgcn_perm(0x64646464u, w0, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, w0, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, w1, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, w1, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = (__builtin_bit_cast(half2v, p[i]) - off) * dd;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

__device__ __forceinline__ half8 q4_row8(uint32_t w, _Float16 d) {
  // nibble i (low) and i + 4 (high) of byte i hold q + 8 of elements i, i + 4
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2v dd = {d, d};
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t p[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, lo, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, hi, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, hi, 0x05030402u)};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = (__builtin_bit_cast(half2v, p[i]) - off) * dd;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

__device__ __forceinline__ half8 fp4_row8(uint32_t w, _Float16 s) {
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

// ---------------------------------------------------------------------------
// The GEMM core.

template <int WF>
struct Fm {
  static constexpr bool W16 = WF == kBF16 || WF == kF16;  // 16-bit weights, no decode
  static constexpr int CC = chunk_cols(WF);               // columns per chunk (memory)
  static constexpr int SCOLS = W16 ? 64 : 128;            // columns per stage
  static constexpr int SC = SCOLS / CC;                   // chunks per stage
  static constexpr int KS = SCOLS / 16;                   // MFMA k-steps (16 columns) per stage
  static constexpr int BPC = CC / 32;                     // 32-column blocks per chunk
  static constexpr int NP = WF == kBF16 ? 2 : 1;          // activation parts
  static constexpr int AST = SCOLS + 8;                   // LDS row stride (elements)
  static constexpr int PPR = SCOLS / 8;                   // 16-byte pieces per row
  static constexpr int PPT = NP * BM * PPR / NTH;         // A pieces per thread
  static constexpr int NS = SC * 4;                       // weight slots per tile and stage
  static constexpr int BPW = NS / 2;                      // of which each wave of the pair loads
  static constexpr int LDSA = NP * BM * AST * 2;          // A bytes per stage
};

// One LDS stage: the activation tile, the raw weight slots of the four
// tiles, and the scale words of their rows.
constexpr int kAOff = 0;
constexpr int kABytes = Fm<kBF16>::LDSA > Fm<kFP4>::LDSA ? Fm<kBF16>::LDSA : Fm<kFP4>::LDSA;
constexpr int kBOff = kABytes;
constexpr int kBBytes = NTW * 8 * 1024;                  // NS <= 8 slots of 1 KB per tile
constexpr int kSOff = kBOff + kBBytes;
constexpr int kStage = kSOff + NTW * 64 * 8;
static_assert(Fm<kQ8>::LDSA <= kABytes && Fm<kQ4>::LDSA <= kABytes && Fm<kF16>::LDSA <= kABytes,
              "LDS sizing");
static_assert(Fm<kQ8>::NS <= 8 && Fm<kBF16>::NS <= 8 && Fm<kFP4>::NS <= 8 && Fm<kF16>::NS <= 8,
              "LDS sizing");
static_assert(2 * kStage <= 160 * 1024, "two stages fit the LDS");

// A weight operand: `nmat` matrices of one geometry concatenated along K
// (U_0 .. U_{G-1}); tile j of a matrix at base + j * tile_slots slots.
struct WMat {
  const uint8_t* base;
  Geom g;
  size_t mat_bytes;
  int nmat;
};

// An activation operand: element (row, part, col) of matrix m at
// p + row * rs + part * ps + m * kmat + col; 16-bit elements.
struct AMat {
  const uint16_t* p;
  size_t rs;
  int ps;
  int kmat;
};

// The global loads of one stage, held in registers until stored to LDS.
template <int WF>
struct Reg {
  uint4 a[Fm<WF>::PPT];
  uint4 b[Fm<WF>::BPW];
  uint2 sc;
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The thread's activation pieces, fixed for a whole GEMM: piece i is 16
// bytes of row m = (threadIdx.x + i * NTH) / PPR (modulo the tile, per part)
// at column c = 8 * (threadIdx.x % PPR) of each stage; p[i] points at that
// column of stage 0 of matrix 0 (padding rows at row 0), bit i of `valid`
// says the row exists.
template <int WF>
struct ARows {
  const uint16_t* p[Fm<WF>::PPT];
  uint32_t valid;
  int c;
};

template <int WF>
__device__ __forceinline__ ARows<WF> a_rows(const AMat& A, const int* arow) {
  using F = Fm<WF>;
  ARows<WF> R;
  R.valid = 0;
  R.c = 8 * (threadIdx.x % F::PPR);
#pragma unroll
  for (int i = 0; i < F::PPT; ++i) {
    const int p = threadIdx.x + i * NTH;
    const int part = p / (BM * F::PPR), m = (p % (BM * F::PPR)) / F::PPR;
    const int row = arow[m];
    R.valid |= (row >= 0 ? 1u : 0u) << i;
    R.p[i] = A.p + (size_t)max(row, 0) * A.rs + (size_t)part * A.ps + R.c;
  }
  return R;
}

// First tile row of activation piece i (its rows are that one and the next
// NTH / PPR - 1; the same rows in every part).
template <int WF>
__host__ __device__ constexpr int piece_row_lo(int i) {
  return ((NTH * i) % (BM * Fm<WF>::PPR)) / Fm<WF>::PPR;
}

// Issues the loads of stage s: the activation pieces (all threads); for the
// wave pair of a weight tile, alternate code slots each plus, from both, the
// scale word of lane-chunk `lane` (row group lane/16, row lane%16). Every
// load is issued: columns past k and a missing last chunk are clamped to
// valid ones (the values are masked when stored, or meet zero activations).
// The weight loads address the wave's tile through a buffer resource with a
// wave-uniform base, so only the lane offset lives in a vector register;
// BAUX is their cache policy. A stage at or past the range end (s >= nst)
// issues the loads of stage nst - 1 with an empty weight resource: its weight loads
// return zeros without a memory access and its activation loads hit the
// lines the same thread just fetched; no branch, so the compiler's counts of
// loads in flight stay exact. Only the pieces of the first SB 32-token
// blocks are staged (the rest of the tile is never read).
template <int WF, int BAUX, int SB>
__device__ __forceinline__ void fetch(const WMat& W, int tile, const AMat& A, const ARows<WF>& ar,
                                      int s, int nst, Reg<WF>& R) {
  const bool live = s < nst;
  s = min(s, nst - 1);
  using F = Fm<WF>;
  const int lane = threadIdx.x & 63, wm = wave_id() & 1;
  const int kmat = W.g.k;
  const int spm = (kmat + F::SCOLS - 1) / F::SCOLS;
  const int mat = s / spm, sm = s % spm;
  const int col0 = sm * F::SCOLS;
  const size_t aoff = (size_t)mat * A.kmat + min(col0, A.kmat - 8 - ar.c);
#pragma unroll
  for (int i = 0; i < F::PPT; ++i)
    if (piece_row_lo<WF>(i) < 32 * SB) R.a[i] = *(const uint4*)(ar.p[i] + aoff);
  const int cpm = (kmat + F::CC - 1) / F::CC;
  const int ss = col0 / kSSCols, cin0 = (col0 % kSSCols) / F::CC;
  const int ncs = ss_code_slots(WF, min(kSSCols, kmat - ss * kSSCols));
  const int jmax = cpm - 1 - sm * F::SC;
  const rsrc_t wt = rsrc(W.base + (size_t)mat * W.mat_bytes + (size_t)tile * W.g.tile_slots * kSlot,
                         live ? (uint32_t)(W.g.tile_slots * kSlot) : 0u);
  const int sso = ss * W.g.full * kSlot;
#pragma unroll
  for (int i2 = 0; i2 < F::BPW; ++i2) {
    const int i = 2 * i2 + wm;
    const int j = min(i / 4, jmax), rg = i % 4;
    R.b[i2] = ldb<BAUX>(wt, lane * 16, sso + ((cin0 + j) * 4 + rg) * kSlot);
  }
  if constexpr (!F::W16) {
    const int off = WF == kQ8 ? 4 * cin0 : 8 * cin0;
    R.sc = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(wt, lane * 16 + off,
                                                                           sso + ncs * kSlot, BAUX));
  }
}

template <int WF, int SB>
__device__ __forceinline__ void store(uint8_t* st, Reg<WF>& R, const AMat& A, const ARows<WF>& ar, int s) {
  using F = Fm<WF>;
  const int spm = (A.kmat + F::SCOLS - 1) / F::SCOLS;
  const int col0 = (s % spm) * F::SCOLS;
  const bool cok = col0 + ar.c < A.kmat;
  uint16_t* As = (uint16_t*)(st + kAOff);
#pragma unroll
  for (int i = 0; i < F::PPT; ++i) {
    if (piece_row_lo<WF>(i) >= 32 * SB) continue;
    const int p = threadIdx.x + i * NTH;
    const int part = p / (BM * F::PPR), m = (p % (BM * F::PPR)) / F::PPR;
    // masked with an AND rather than a select: the loaded value is always
    // used, so the compiler cannot sink the load down to this store
    const uint32_t mk = (cok && ((ar.valid >> i) & 1u)) ? ~0u : 0u;
    const uint4 v = make_uint4(R.a[i].x & mk, R.a[i].y & mk, R.a[i].z & mk, R.a[i].w & mk);
    *(uint4*)(As + (size_t)(part * BM + m) * F::AST + ar.c) = v;
  }
  const int lane = threadIdx.x & 63, w = wave_id(), tl = w >> 1, wm = w & 1;
  uint4* Bs = (uint4*)(st + kBOff);
#pragma unroll
  for (int i2 = 0; i2 < F::BPW; ++i2) Bs[(tl * 8 + 2 * i2 + wm) * 64 + lane] = R.b[i2];
  // both waves of the pair hold the same scale word and store it
  if constexpr (!F::W16) ((uint2*)(st + kSOff))[tl * 64 + lane] = R.sc;
}

// The B operand of v_mfma_f32_32x32x16 for weight rows 32*nb + l%32 and
// k-step ks: lane l needs columns 16*ks + 8*(l/32) .. +7. In the tiled stream
// those sit in row group 2*nb + (l%32)/16, in the lane-chunk of k-group
// 2*(ks%2) + l/32 and row l%16, of block (ks/2) % BPC of chunk (ks/2) / BPC.
__device__ __forceinline__ int b_lane(int nb, int kk, int lane) {
  return (((2 * nb + ((lane & 31) >> 4)) * 64) + 16 * (2 * kk + (lane >> 5)) + (lane & 15));
}

// decodes the 8 columns of block b held in raw word(s), with the scale word
// pair `sc` of the lane's row (k-group qg of the 32-column block)
template <int WF>
__device__ __forceinline__ uint4 decode_b(uint4 w, uint2 sc, int blk, int b, int qg) {
  if constexpr (Fm<WF>::W16) {
    return w;
  } else if constexpr (WF == kFP4) {
    const int byte = 2 * b + (qg >> 1);
    const uint32_t sw = byte < 4 ? sc.x : sc.y;
    const uint32_t code = (sw >> (8 * (byte & 3))) & 0xFFu;
    const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8(code, 0);
    return __builtin_bit_cast(uint4, fp4_row8(word(w, b), s));
  } else {
    const uint32_t sw = blk < 2 ? sc.x : sc.y;
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(sw >> (16 * (blk & 1))));
    if constexpr (WF == kQ8) return __builtin_bit_cast(uint4, q8_row8(word(w, 2 * b), word(w, 2 * b + 1), d));
    else return __builtin_bit_cast(uint4, q4_row8(word(w, b), d));
  }
}

// One stage of MFMAs for this wave over its first NMB 32-token blocks: per
// k-step the activation fragments are read, the two weight fragments (rows
// 0..31 and 32..63 of the wave's tile) decoded, then 2 * NMB MFMAs issued.
template <int WF, int NMB>
__device__ __forceinline__ void mfma_stage(const uint8_t* st, f16v (&acc)[MB][2]) {
  using F = Fm<WF>;
  const int lane = threadIdx.x & 63, w = wave_id(), tl = w >> 1, wm = w & 1;
  const int row = lane & 31, kh = lane >> 5;
  const uint16_t* As = (const uint16_t*)(st + kAOff);
  const uint4* Bs = (const uint4*)(st + kBOff) + tl * 8 * 64;
  // raw weight words: chunk j, row block nb, k-half kk (ks % 2)
  uint4 raw[F::SC][2][2];
#pragma unroll
  for (int j = 0; j < F::SC; ++j)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) raw[j][nb][kk] = Bs[j * 4 * 64 + b_lane(nb, kk, lane)];
  uint2 sc[2] = {make_uint2(0, 0), make_uint2(0, 0)};
  if constexpr (!F::W16) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      sc[nb] = ((const uint2*)(st + kSOff))[tl * 64 + 16 * (2 * nb + (row >> 4)) + (lane & 15)];
  }
  // activation fragments of k-step ks (rows of the wave's token blocks)
  const auto load_a = [&](int ks, uint4 (&a)[F::NP][NMB]) {
#pragma unroll
    for (int p = 0; p < F::NP; ++p)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        a[p][mb] = *(const uint4*)(As + (size_t)(p * BM + WTOK * wm + 32 * mb + row) * F::AST +
                                   16 * ks + 8 * kh);
  };
  // the fragments of k-step ks + 1 are read while ks computes; for the
  // decoded formats a scheduling barrier closes each k-step, so the compiler
  // does not hoist every read and decode of the stage ahead of the first MFMA
  // (that needs more registers than two waves per SIMD have)
  uint4 a[2][F::NP][NMB];
  load_a(0, a[0]);
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) {
    const int kk = ks & 1, c32 = ks >> 1;           // 32-column block of the stage
    const int j = c32 / F::BPC, b = c32 % F::BPC;   // chunk, block within the chunk
    if (ks + 1 < F::KS) load_a(ks + 1, a[(ks + 1) & 1]);
    const uint4 (&ac)[F::NP][NMB] = a[ks & 1];
    uint4 bw[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bw[nb] = decode_b<WF>(raw[j][nb][kk], sc[nb], F::BPC * j + b, b, 2 * kk + kh);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (WF == kBF16) {
#pragma unroll
          for (int p = 0; p < F::NP; ++p)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, ac[p][mb]), __builtin_bit_cast(bf16x8, bw[nb]), acc[mb][nb], 0, 0, 0);
        } else {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(half8, ac[0][mb]), __builtin_bit_cast(half8, bw[nb]), acc[mb][nb], 0, 0, 0);
        }
      }
    if constexpr (!F::W16) __builtin_amdgcn_sched_barrier(0);
  }
}

// Accumulates the tile's product over stages [sb, se) of W (stage s covers
// SCOLS columns of matrix s / stages-per-matrix) for the wave's first NMB
// token blocks (NMB 0: the wave only stages); `tile` is the wave's weight
// tile (a wave whose tile is past the last one computes on tile 0 and
// discards the result). Global loads run NSET - 1 stages ahead in NSET
// register sets; one barrier per stage: between two barriers a wave issues
// the global loads of stage s + NSET (into the set stage s left), the MFMAs
// of stage s (LDS buffer (s - sb) % 2) and the LDS stores of stage s + 1 (the
// other buffer, whose last readers finished before the barrier). The
// register set is the stage's index in the range modulo NSET (the body is
// unrolled NSET times, with one loop exit); the buffer is picked at run
// time. Every thread of the block takes part in the staging and the
// barriers (the range is the block's); the closing barrier also frees the
// buffers for a following call. An empty range does nothing. Only the first
// SB 32-token blocks of the tile are staged (SB >= the blocks any wave
// computes on).
template <int WF, int NMB, int BAUX, int NSET, int SB>
__device__ __forceinline__ void gemm_loop(const WMat& W, int tile, bool b_on, const AMat& A,
                                          const int* arow, uint8_t* smem, f16v (&acc)[MB][2],
                                          int sb, int se) {
  static_assert(NSET == 2 || NSET == 3, "two or three register sets");
  if (sb >= se) return;
  const int ld_tile = b_on ? tile : 0;     // a valid tile for the unused loads
  const ARows<WF> ar = a_rows<WF>(A, arow);
  Reg<WF> r[NSET];
#pragma unroll
  for (int i = 0; i < NSET; ++i) fetch<WF, BAUX, SB>(W, ld_tile, A, ar, sb + i, se, r[i]);
  store<WF, SB>(smem, r[0], A, ar, sb);
  __syncthreads();
  // stage s: loads of s + NSET into the set stage s left, MFMAs of s, stores
  // of s + 1 (past the last stage, a stale set into the buffer no wave reads
  // again); the body has no branch
  const auto step = [&](int s, Reg<WF>& mine, Reg<WF>& next) {
    fetch<WF, BAUX, SB>(W, ld_tile, A, ar, s + NSET, se, mine);
    if constexpr (NMB > 0) mfma_stage<WF, NMB>(smem + ((s - sb) & 1) * kStage, acc);
    store<WF, SB>(smem + ((s - sb + 1) & 1) * kStage, next, A, ar, min(s + 1, se - 1));
    __syncthreads();
  };
  int s0 = sb;
  for (; s0 + NSET <= se; s0 += NSET) {
#pragma unroll
    for (int i = 0; i < NSET; ++i) step(s0 + i, r[i], r[(i + 1) % NSET]);
  }
#pragma unroll
  for (int i = 0; i + 1 < NSET; ++i)
    if (s0 + i < se) step(s0 + i, r[i], r[(i + 1) % NSET]);
}

// stages of a weight operand: SCOLS-column steps of each of its matrices
template <int WF>
__host__ __device__ __forceinline__ int n_stages(const WMat& W) {
  return ((W.g.k + Fm<WF>::SCOLS - 1) / Fm<WF>::SCOLS) * W.nmat;
}

// runs gemm_loop over stages [sb, se) (default: all) with the wave's
// token-block count: 0, 1 or 2; BAUX is the cache policy of the weight
// loads, NSET the register sets of the prefetch
template <int WF, int BAUX = 0, int NSET = 3>
__device__ __forceinline__ void gemm_wave(const WMat& W, int tile, bool b_on, int nmb, const AMat& A,
                                          const int* arow, uint8_t* smem, f16v (&acc)[MB][2],
                                          int sb = 0, int se = -1) {
  if (se < 0) se = n_stages<WF>(W);
  if (nmb >= 2) gemm_loop<WF, 2, BAUX, NSET, 4>(W, tile, b_on, A, arow, smem, acc, sb, se);
  else if (nmb == 1) gemm_loop<WF, 1, BAUX, NSET, 4>(W, tile, b_on, A, arow, smem, acc, sb, se);
  else gemm_loop<WF, 0, BAUX, NSET, 4>(W, tile, b_on, A, arow, smem, acc, sb, se);
}

// gemm_wave for a tile of `count` tokens (1..BM) that stages only the
// 32-token blocks holding them: most expert pieces are short, and the
// vector memory path is what the stages wait on. The wave of each pair that
// covers tokens 0..63 computes min(2, blocks) blocks, the other the rest.
template <int WF, int BAUX = 0, int NSET = 3>
__device__ __forceinline__ void gemm_wave_count(const WMat& W, int tile, bool b_on, int count,
                                                const AMat& A, const int* arow, uint8_t* smem,
                                                f16v (&acc)[MB][2]) {
  const int se = n_stages<WF>(W), blocks = min(4, (count + 31) / 32);
  const bool lo = (wave_id() & 1) == 0;
  switch (blocks) {
    case 1:
      if (lo) gemm_loop<WF, 1, BAUX, NSET, 1>(W, tile, b_on, A, arow, smem, acc, 0, se);
      else gemm_loop<WF, 0, BAUX, NSET, 1>(W, tile, b_on, A, arow, smem, acc, 0, se);
      break;
    case 2:
      if (lo) gemm_loop<WF, 2, BAUX, NSET, 2>(W, tile, b_on, A, arow, smem, acc, 0, se);
      else gemm_loop<WF, 0, BAUX, NSET, 2>(W, tile, b_on, A, arow, smem, acc, 0, se);
      break;
    case 3:
      if (lo) gemm_loop<WF, 2, BAUX, NSET, 3>(W, tile, b_on, A, arow, smem, acc, 0, se);
      else gemm_loop<WF, 1, BAUX, NSET, 3>(W, tile, b_on, A, arow, smem, acc, 0, se);
      break;
    default:
      gemm_loop<WF, 2, BAUX, NSET, 4>(W, tile, b_on, A, arow, smem, acc, 0, se);
      break;
  }
}

__device__ __forceinline__ void zero_acc(f16v (&acc)[MB][2]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
}

// Lane l holds in acc[mb][nb][i] the tile-relative token
// 32*mb + 8*(i/4) + 4*(l/32) + i%4 and the row 32*nb + l%32 of its wave's
// weight tile (the v_mfma_f32_32x32x16 accumulator layout).
__device__ __forceinline__ int acc_tok(int lane, int mb, int i) {
  return 32 * mb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ---------------------------------------------------------------------------
// Dense GEMMs: router, D, shared gate/up, U (+ shared down).

enum Epi : int {
  kEpiLogits = 0,   // fp32 out[t][n], n < nvalid
  kEpiF16 = 1,      // fp16 out[t][n]
  kEpiSwigluB2 = 2, // paired gate/up tile: h = silu(g) * u as two bf16 parts
  kEpiY = 3,        // fp32 y[t][n] (+ residual)
};

struct Dense {
  WMat W;
  AMat A;
  WMat W2;       // kEpiY: the shared down projection, same accumulators
  AMat A2;
  int T, mtiles, ntiles, nquads;
  void* out;
  size_t ostride;
  int nvalid;
  const float* res;   // kEpiY: residual rows [T][ostride] or null
  const float* xsc;   // kEpiSwigluB2, kEpiY: range scale c per token (h gets c^2, y c^-2)
  // kEpiY and kEpiLogits: the first nfull logical tiles run whole; each of
  // the remaining nrem runs as nsplit blocks along k. Split sp covers a
  // balanced share of the stages of W (kEpiY: then W2, a W2 stage, bf16 in
  // two parts, counting twice). With nsplit > 1, kEpiY writes its BM x 256
  // sum to part + (sp * nrem + j) * BM * 256 for the j-th split tile, with
  // no residual (k_ytiles adds them up); kEpiLogits writes its sum to
  // out + sp * T * ostride (k_select adds them up).
  int nfull, nrem, nsplit;
  float* part;
  // D over the routed (token, group) pairs only: group g's rows are the
  // tokens gl_tok[g * gcap + i], i < gl_cnt[g]; its output goes to columns
  // g * gL .. of the token's row
  const int* gl_tok;
  const int* gl_cnt;
  int G, gcap, gL;
};

// XCD-aware order: block b of n runs on XCD b % 8; each XCD takes a
// contiguous range of the n logical indices
__device__ __forceinline__ int xcd_order(int b, int n) {
  const int xcd = b & 7, q = b >> 3, per = n >> 3, rem = n & 7;
  return xcd * per + min(xcd, rem) + q;
}

// logical tile L -> (token tile, weight quad): groups of 8 token tiles sweep
// the weight quads with the token tile fastest, so neighbours in time share
// A and B in L2
__device__ __forceinline__ void tile_of(int L, int mtiles, int nquads, int& mt, int& quad) {
  constexpr int GM = 8;
  const int span = GM * nquads;
  const int first = (L / span) * GM, gsz = min(mtiles - first, GM);
  mt = first + (L % span) % gsz;
  quad = (L % span) / gsz;
}

// the inverse: logical tile of (token tile mt, weight quad quad)
__device__ __forceinline__ int tile_index(int mt, int quad, int mtiles, int nquads) {
  constexpr int GM = 8;
  const int first = (mt / GM) * GM, gsz = min(mtiles - first, GM);
  return (mt / GM) * GM * nquads + quad * gsz + (mt - first);
}

// ---------------------------------------------------------------------------
// LDS DMA.

// 16 bytes per lane from r + voff + soff to LDS m0 + 16 lane. Written in
// assembly so that the compiler, which cannot tell which LDS bytes a DMA
// writes, does not wait for every DMA before each LDS read; the kernel waits
// for the stage it needs (vmcnt) itself. No vector register is written; m0
// (the LDS address) is, and is declared clobbered: the compiler reserves m0
// and sets it itself before each of its own uses, so it warns that a
// reserved register is listed (silenced here).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt operand that waits for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 at their maxima)
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

constexpr uint32_t kOob = 0xFFFFFFF0u;                   // a DMA offset past any resource: out of range

// the k_dense epilogues for the wave's accumulators (tile row block mt,
// weight tile `tile`, split sp of nsp of logical tile L)
template <int EPI>
__device__ __forceinline__ void dense_epilogue(const Dense& a, const f16v (&acc)[MB][2], int mt, int quad, int tile,
                                               int L, int sp, int nsp, int lane, int wm) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = mt * BM + WTOK * wm + acc_tok(lane, mb, v);
      if (t >= a.T) continue;
      if constexpr (EPI == kEpiSwigluB2) {
        // rows 0..31 of the tile are gate rows 32*tile + 0..31, rows 32..63
        // the up rows of the same indices
        const int f = 32 * tile + (lane & 31);
        const float c = a.xsc[t];
        const float hv = silu(acc[mb][0][v]) * acc[mb][1][v] * c * c;
        const __bf16 h0 = (__bf16)hv;
        const __bf16 h1 = (__bf16)(hv - (float)h0);
        __bf16* o = (__bf16*)a.out + (size_t)t * a.ostride;
        o[f] = h0;
        o[a.nvalid + f] = h1;
      } else {
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          const int n = 64 * tile + 32 * rg + (lane & 31);
          const float val = acc[mb][rg][v];
          if constexpr (EPI == kEpiLogits) {
            if (n < a.nvalid) ((float*)a.out)[((size_t)sp * a.T + t) * a.ostride + n] = val;
          } else if constexpr (EPI == kEpiF16) {
            ((_Float16*)a.out)[(size_t)t * a.ostride + n] = (_Float16)val;
          } else if (nsp > 1) {
            const size_t j = (size_t)sp * a.nrem + (L - a.nfull);
            a.part[(j * BM + (t - mt * BM)) * 256 + (n - 256 * quad)] = val;
          } else {
            const size_t i = (size_t)t * a.ostride + n;
            const float ic = inv_pow2(a.xsc[t]), yv = val * ic * ic;
            ((float*)a.out)[i] = a.res ? a.res[i] + yv : yv;
          }
        }
      }
    }
}

template <int WF, int EPI>
__global__ __launch_bounds__(NTH) void k_dense(Dense a) {
  __shared__ __align__(16) uint8_t smem[2 * kStage];
  __shared__ int arow[BM];
  constexpr bool SPLIT = EPI == kEpiY || EPI == kEpiLogits;
  const int nblk0 = a.mtiles * a.nquads;
  int L = 0, sp = 0, nsp = 1;
  if (!SPLIT || (int)blockIdx.x < a.nfull) {
    L = xcd_order(blockIdx.x, SPLIT ? a.nfull : nblk0);
  } else {
    // split blocks follow the whole tiles (nfull is a multiple of 8, so the
    // XCD of a block is still its index modulo 8); the split is slowest
    const int Ls = xcd_order(blockIdx.x - a.nfull, a.nrem * a.nsplit);
    sp = Ls / a.nrem;
    L = a.nfull + Ls % a.nrem;
    nsp = a.nsplit;
  }
  int mt, quad;
  tile_of(L, a.mtiles, a.nquads, mt, quad);

  if (threadIdx.x < BM) {
    const int t = mt * BM + threadIdx.x;
    arow[threadIdx.x] = t < a.T ? t : -1;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1;
  const int tile = NTW * quad + (wave >> 1);
  const bool b_on = tile < a.ntiles;
  const int nmb = min(MB, max(0, a.T - mt * BM - WTOK * wm + 31) / 32);
  f16v acc[MB][2];
  zero_acc(acc);
  if constexpr (EPI == kEpiY) {
    // unit boundaries of the split: W stages count one, W2 stages two
    const int n1 = n_stages<WF>(a.W), n2 = n_stages<kBF16>(a.W2), units = n1 + 2 * n2;
    const int c0 = (int)((long long)units * sp / nsp);
    const int c1 = (int)((long long)units * (sp + 1) / nsp);
    const auto w2_stage = [&](int c) { return min(n2, max(0, (c - n1 + 1) / 2)); };
    gemm_wave<WF>(a.W, tile, b_on, nmb, a.A, arow, smem, acc, min(c0, n1), min(c1, n1));
    gemm_wave<kBF16>(a.W2, tile, b_on, nmb, a.A2, arow, smem, acc, w2_stage(c0), w2_stage(c1));
  } else if constexpr (EPI == kEpiLogits) {
    const int n1 = n_stages<WF>(a.W);
    gemm_wave<WF>(a.W, tile, b_on, nmb, a.A, arow, smem, acc,
                  (int)((long long)n1 * sp / nsp), (int)((long long)n1 * (sp + 1) / nsp));
  } else {
    gemm_wave<WF>(a.W, tile, b_on, nmb, a.A, arow, smem, acc);
  }
  if (!b_on) return;
  dense_epilogue<EPI>(a, acc, mt, quad, tile, L, sp, nsp, lane, wm);
}

// ---------------------------------------------------------------------------
// The dense GEMMs of 16-bit weights (router, shared gate/up, U + shared
// down) with DMA-fed operands: the geometry and epilogues of k_dense, but
// 32-column stages copied global -> LDS by buffer DMA (activation rows of
// all parts and the weights' raw slots), three stages ahead in four 32 KB
// buffers, so the loop issues no vector loads or LDS stores of its own.
// Activation rows are 64 B, their four 16 B pieces XOR-swizzled by
// (row / 4) % 4: the fragment reads of 16 consecutive rows hit distinct
// banks. K of every matrix is a multiple of 64 (k_dense's stage unit), so
// stage s of k_dense is stages 2s and 2s + 1 here.

constexpr int kDdCols = 32, kDdBuf = 4, kDdStage = 32 * 1024, kDdB = 16 * 1024;

// stages [2 sb, 2 se) of W (sb, se in 64-column units); the wave's 64 tokens
// x 64-row tile as in gemm_wave, both 32-token blocks always computed
template <int WF>
__device__ __forceinline__ void gemm_wave_dma(const WMat& W, int tile, bool b_on, const AMat& A,
                                              const int* arow, uint8_t* smem, f16v (&acc)[MB][2],
                                              int sb64, int se64) {
  constexpr int NP = WF == kBF16 ? 2 : 1;
  static_assert(WF == kBF16 || WF == kF16, "16-bit weights");
  const int sb = 2 * sb64, se = 2 * se64;
  if (se <= sb) return;
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1, tl = wave >> 1;
  const int row = lane & 31, kh = lane >> 5;
  const int spm = W.g.k / kDdCols;
  // activation DMA: instruction (part p, i = wave) covers rows 16 i .. + 15;
  // lane l the piece at position l % 4 of row 16 i + l / 4
  const int r = 16 * wave + (lane >> 2);
  const int arw = arow[r];
  const int cch = 8 * ((lane & 3) ^ ((r >> 2) & 3));
  const uint32_t abase = arw >= 0 ? (uint32_t)((size_t)arw * A.rs * 2) : kOob;
  const rsrc_t ar = rsrc(A.p, kOob);
  const size_t wspan = (size_t)(W.nmat - 1) * W.mat_bytes + (size_t)W.g.tile_slots * kSlot;
  const rsrc_t wt = rsrc(W.base + (size_t)(b_on ? tile : 0) * W.g.tile_slots * kSlot, b_on ? (uint32_t)wspan : 0u);
  const rsrc_t wz = rsrc(W.base, 0u);
  const uint32_t sbase = lds_off(smem);
  const auto issue = [&](int s) {
    const bool live = s < se;
    const uint32_t st = sbase + (uint32_t)((s % kDdBuf) * kDdStage);
    s = min(s, se - 1);
    const int mat = s / spm, sm = s % spm;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t vo = (abase == kOob || !live)
                              ? kOob
                              : abase + (uint32_t)(2 * (p * A.ps + mat * A.kmat + sm * kDdCols + cch));
      dma16(ar, st + p * 8192 + wave * 1024, vo, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rg = 2 * wm + h;
      dma16(live ? wt : wz, st + kDdB + (tl * 4 + rg) * 1024, lane * 16,
            (uint32_t)((size_t)mat * W.mat_bytes + (size_t)(4 * sm + rg) * kSlot));
    }
  };
  // the buffers may still be read by a previous range's last stage
  __syncthreads();
  issue(sb);
  issue(sb + 1);
  issue(sb + 2);
  for (int s = sb; s < se; ++s) {
    // this wave's DMAs of stage s are done when at most those of s + 1 and
    // s + 2 are in flight; the barrier makes every wave's visible and ends
    // the reads of stage s - 1, whose buffer stage s + 3 refills
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * (NP + 2)));
    __syncthreads();
    issue(s + 3);
    const uint8_t* st = smem + (s % kDdBuf) * kDdStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + kh;
      uint4 af[NP][2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int m = WTOK * wm + 32 * mb + row;
          af[p][mb] = *(const uint4*)(st + (p * BM + m) * 64 + 16 * (c ^ ((m >> 2) & 3)));
        }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bf[nb] = *(const uint4*)(st + kDdB + ((tl * 4 + 2 * nb + (row >> 4)) * 64 + 16 * c + (lane & 15)) * 16);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if constexpr (WF == kBF16) {
#pragma unroll
            for (int p = 0; p < NP; ++p)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, af[p][mb]), __builtin_bit_cast(bf16x8, bf[nb]), acc[mb][nb], 0, 0, 0);
          } else {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8, af[0][mb]), __builtin_bit_cast(half8, bf[nb]), acc[mb][nb], 0, 0, 0);
          }
        }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
}

template <int WF, int EPI>
__global__ __launch_bounds__(NTH) void k_dense_dma(Dense a) {
  __shared__ __align__(1024) uint8_t smem[kDdBuf * kDdStage];
  __shared__ int arow[BM];
  constexpr bool SPLIT = EPI == kEpiY || EPI == kEpiLogits;
  const int nblk0 = a.mtiles * a.nquads;
  int L = 0, sp = 0, nsp = 1;
  if (!SPLIT || (int)blockIdx.x < a.nfull) {
    L = xcd_order(blockIdx.x, SPLIT ? a.nfull : nblk0);
  } else {
    const int Ls = xcd_order(blockIdx.x - a.nfull, a.nrem * a.nsplit);
    sp = Ls / a.nrem;
    L = a.nfull + Ls % a.nrem;
    nsp = a.nsplit;
  }
  int mt, quad;
  tile_of(L, a.mtiles, a.nquads, mt, quad);
  if (threadIdx.x < BM) {
    const int t = mt * BM + threadIdx.x;
    arow[threadIdx.x] = t < a.T ? t : -1;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1;
  const int tile = NTW * quad + (wave >> 1);
  const bool b_on = tile < a.ntiles;
  f16v acc[MB][2];
  zero_acc(acc);
  if constexpr (EPI == kEpiY) {
    const int n1 = n_stages<WF>(a.W), n2 = n_stages<kBF16>(a.W2), units = n1 + 2 * n2;
    const int c0 = (int)((long long)units * sp / nsp);
    const int c1 = (int)((long long)units * (sp + 1) / nsp);
    const auto w2_stage = [&](int c) { return min(n2, max(0, (c - n1 + 1) / 2)); };
    gemm_wave_dma<WF>(a.W, tile, b_on, a.A, arow, smem, acc, min(c0, n1), min(c1, n1));
    gemm_wave_dma<kBF16>(a.W2, tile, b_on, a.A2, arow, smem, acc, w2_stage(c0), w2_stage(c1));
  } else if constexpr (EPI == kEpiLogits) {
    const int n1 = n_stages<WF>(a.W);
    gemm_wave_dma<WF>(a.W, tile, b_on, a.A, arow, smem, acc,
                      (int)((long long)n1 * sp / nsp), (int)((long long)n1 * (sp + 1) / nsp));
  } else {
    gemm_wave_dma<WF>(a.W, tile, b_on, a.A, arow, smem, acc, 0, n_stages<WF>(a.W));
  }
  if (!b_on) return;
  dense_epilogue<EPI>(a, acc, mt, quad, tile, L, sp, nsp, lane, wm);
}

// ---------------------------------------------------------------------------
// Grouped GEMMs over the expert segments.

struct Piece {
  int expert, start, count, pad;
};

enum GEpi : int { kGateUp = 0, kDown = 1 };

struct Grouped {
  const uint8_t* experts;
  size_t estride;       // bytes per expert
  size_t woff;          // offset of this matrix in an expert
  size_t ts_off;        // offset of the three fp32 tensor scales
  Geom g;
  AMat A;
  const Piece* pieces;
  const int* npieces;   // [0] pieces, [1] the first of at most 64 tokens, [2] of at most 32
  int ntiles, nquads, G, F;
  const int* perm;      // [T*K] sorted position -> assignment t*K + k
  const float* topk_w;  // [T*K]
  const float* psc;     // [T*K] range scale of each sorted assignment's token
  const uint8_t* labels;
  int K;
  void* out;
  size_t ostride;
};

template <int EPI>
__global__ __launch_bounds__(NTH) void k_grouped(Grouped a) {
  __shared__ __align__(16) uint8_t smem[2 * kStage];
  __shared__ int arow[BM];
  // piece p runs on XCD p % 8, all its weight-tile quads back to back (the
  // pieces of a large expert spread over the XCDs, which balances them)
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int p = xcd + 8 * (q / a.nquads), quad = q % a.nquads;
  if (p >= a.npieces[1]) return;                     // pieces of more than 64 tokens
  const Piece pc = a.pieces[p];
  const int e = pc.expert;
  if (threadIdx.x < BM) {
    const int i = threadIdx.x;
    int row = -1;
    if (i < pc.count) {
      const int pos = pc.start + i;
      row = EPI == kGateUp ? (a.perm[pos] / a.K) * a.G + a.labels[e] : pos;
    }
    arow[i] = row;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1;
  const int tile = NTW * quad + (wave >> 1);
  const bool b_on = tile < a.ntiles;
  const uint8_t* base = a.experts + (size_t)e * a.estride;
  const WMat W{base + a.woff, a.g, 0, 1};
  f16v acc[MB][2];
  zero_acc(acc);
  // each expert's weights are streamed once per piece: non-temporal
  gemm_wave_count<kFP4, kAuxNT>(W, tile, b_on, pc.count, a.A, arow, smem, acc);
  if (!b_on) return;
  const float* ts = (const float*)(base + a.ts_off);

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = WTOK * wm + acc_tok(lane, mb, v);
      if (i >= pc.count) continue;
      const size_t pos = (size_t)pc.start + i;
      if constexpr (EPI == kGateUp) {
        const float tg = ts[0], tu = ts[1];
        const int f = 32 * tile + (lane & 31);
        // gate and up carry the token's range scale c: h = silu(g) u c^2
        const float c = a.psc[pos];
        const float hv = silu(acc[mb][0][v] * tg * inv_pow2(c)) * (acc[mb][1][v] * tu * c);
        ((_Float16*)a.out)[pos * a.ostride + f] = (_Float16)hv;
      } else {
        const float sc = a.topk_w[a.perm[pos]] * ts[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          const int n = 64 * tile + 32 * rg + (lane & 31);
          ((_Float16*)a.out)[pos * a.ostride + n] = (_Float16)(acc[mb][rg][v] * sc);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Expert gate/up for pieces of more than 64 tokens, operands fed by DMA. The
// geometry of k_grouped (128 tokens x 4 weight tiles, each wave 64 tokens x
// one 64-row tile), but no register staging: the activation rows (gathered
// through the permutation) and the weights' raw code and scale slots are
// copied global -> LDS by buffer DMA, two stages ahead in three buffers, so
// a wave's instruction stream in the loop is its LDS reads, decodes and
// MFMAs. Activation rows are 256 B (128 fp16 columns), their sixteen 16 B
// pieces XOR-swizzled by row % 16 through the DMA source address, so the
// fragment reads of 16 consecutive rows hit distinct banks. K is a multiple
// of 128 (every staged column real); rows past the piece may hold anything,
// their outputs are not stored.

constexpr int kGdA = BM * 256;                           // activation bytes per stage
constexpr int kGdB = NTW * 4 * kSlot;                    // code slots
constexpr int kGdS = NTW * kSlot;                        // scale slots
constexpr int kGdStage = kGdA + kGdB + kGdS;
constexpr int kGdBuf = 3;
static_assert(kGdBuf * kGdStage + BM * 4 <= 160 * 1024, "LDS");

template <int EPI>
__global__ __launch_bounds__(NTH) void k_grouped_dma(Grouped a) {
  __shared__ __align__(1024) uint8_t smem[kGdBuf * kGdStage];
  __shared__ int arow[BM];
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int p = xcd + 8 * (q / a.nquads), quad = q % a.nquads;
  if (p >= a.npieces[1]) return;                     // pieces of more than 64 tokens
  const Piece pc = a.pieces[p];
  const int e = pc.expert;
  if (threadIdx.x < BM) {
    const int i = threadIdx.x;
    int row = -1;
    if (i < pc.count) {
      const int pos = pc.start + i;
      row = EPI == kGateUp ? (a.perm[pos] / a.K) * a.G + a.labels[e] : pos;
    }
    arow[i] = row;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1, tl = wave >> 1;
  const int tile = NTW * quad + tl;
  const bool b_on = tile < a.ntiles;
  const uint8_t* base = a.experts + (size_t)e * a.estride;
  const WMat W{base + a.woff, a.g, 0, 1};
  using F = Fm<kFP4>;
  const int kmat = a.A.kmat, nst = n_stages<kFP4>(W);
  // activation DMA: instruction i = wave + 8 j covers rows 4 i .. + 3; lane
  // l the piece at position l % 16 of row 4 i + l / 16, which holds column
  // piece (l % 16) ^ (row % 16)
  const rsrc_t ar = rsrc(a.A.p, kOob);
  uint32_t aro[4];
  int acol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * (wave + 8 * j) + (lane >> 4);
    const int arw = arow[r];
    acol[j] = 8 * ((lane & 15) ^ (r & 15));
    aro[j] = arw >= 0 ? (uint32_t)((size_t)arw * a.A.rs * 2) : kOob;
  }
  const uint32_t sbase = lds_off(smem);
  const auto issue = [&](int s) {
    const bool live = s < nst;
    const uint32_t st = sbase + (uint32_t)((s % kGdBuf) * kGdStage);
    s = min(s, nst - 1);
    const int col0 = s * F::SCOLS;                 // one matrix: stage s covers columns col0 ..
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = col0 + acol[j];
      const uint32_t vo = (aro[j] == kOob || c >= kmat || !live) ? kOob : aro[j] + (uint32_t)(2 * c);
      dma16(ar, st + (wave + 8 * j) * 1024, vo, 0);
    }
    const int ss = col0 / kSSCols, cin0 = (col0 % kSSCols) / F::CC;
    const int ncs = ss_code_slots(kFP4, min(kSSCols, kmat - ss * kSSCols));
    const rsrc_t wt = rsrc(W.base + (size_t)min(tile, a.ntiles - 1) * W.g.tile_slots * kSlot,
                           live && b_on ? (uint32_t)(W.g.tile_slots * kSlot) : 0u);
    const uint32_t sso = (uint32_t)(ss * W.g.full * kSlot);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rg = 2 * wm + h;
      dma16(wt, st + kGdA + (tl * 4 + rg) * 1024, lane * 16, sso + (uint32_t)((cin0 * 4 + rg) * kSlot));
    }
    // the tile's scale slot, from the even wave of the pair (a DMA writes its
    // 64 lanes to consecutive 16 B: one slot per instruction)
    if (wm == 0) dma16(wt, st + kGdA + kGdB + tl * 1024, lane * 16, sso + (uint32_t)(ncs * kSlot));
  };
  f16v acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
  issue(0);
  issue(1);
  const int row = lane & 31, kh = lane >> 5;
  for (int s = 0; s < nst; ++s) {
    // this wave's DMAs of stage s (7 or 6) are done when at most 6 of s + 1
    // are in flight; the barrier makes every wave's visible and ends the
    // reads of stage s - 1, whose buffer stage s + 2 refills
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(6));
    __syncthreads();
    issue(s + 2);
    const uint8_t* st = smem + (s % kGdBuf) * kGdStage;
    const uint4* Bs = (const uint4*)(st + kGdA) + tl * 4 * 64;
    const uint8_t* Ss = st + kGdA + kGdB + tl * 1024;
    const int cin0 = ((s * F::SCOLS) % kSSCols) / F::CC;
    uint4 raw[2][2];
    uint2 sc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) raw[nb][kk] = Bs[(2 * nb + (row >> 4)) * 64 + 16 * (2 * kk + kh) + (lane & 15)];
      sc[nb] = *(const uint2*)(Ss + (16 * (2 * nb + (row >> 4)) + (lane & 15)) * 16 + 8 * cin0);
    }
    const auto afrag = [&](int ks, int mb) {
      const int m = WTOK * wm + 32 * mb + row, c = 2 * ks + kh;
      return *(const uint4*)(st + m * 256 + 16 * (c ^ (m & 15)));
    };
    uint4 av[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) av[0][mb] = afrag(0, mb);
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) {
      const int kk = ks & 1, b = ks >> 1;
      if (ks + 1 < F::KS)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) av[(ks + 1) & 1][mb] = afrag(ks + 1, mb);
      uint4 bw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bw[nb] = decode_b<kFP4>(raw[nb][kk], sc[nb], b, b, 2 * kk + kh);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, av[ks & 1][mb]),
                                                               __builtin_bit_cast(half8, bw[nb]), acc[mb][nb],
                                                               0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  if (!b_on) return;
  const float* ts = (const float*)(base + a.ts_off);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = WTOK * wm + acc_tok(lane, mb, v);
      if (i >= pc.count) continue;
      const size_t pos = (size_t)pc.start + i;
      const float tg = ts[0], tu = ts[1];
      const int f = 32 * tile + (lane & 31);
      // gate and up carry the token's range scale c: h = silu(g) u c^2
      const float c = a.psc[pos];
      const float hv = silu(acc[mb][0][v] * tg * inv_pow2(c)) * (acc[mb][1][v] * tu * c);
      ((_Float16*)a.out)[pos * a.ostride + f] = (_Float16)hv;
    }
}

// ---------------------------------------------------------------------------
// Narrow pieces of the expert GEMMs (at most 64 tokens). Most experts draw
// few tokens (the median of the 145B prefill input is 10), and in a
// 128-token tile such a piece leaves waves without MFMAs while every wave
// pair stages and decodes the same weight tile. Here a workgroup of NW waves
// takes 32 NMB tokens x 64 NW weight rows: each wave owns one 64-row tile
// and reads its weights straight from memory into the registers of its
// MFMA operands (the tiled stream holds the v_mfma_f32_32x32x16 B operand of
// a lane as one 16-byte lane-chunk: whole 256-byte segments per load),
// decodes them itself, and only the activation rows go through LDS, shared by
// all the workgroup's tiles. Activation and weight register sets rotate separately
// (three each), so no load targets registers the MFMAs in flight read, and
// each load has two stages to arrive; the body has no branch (empty weight
// resource past the last stage or tile).

constexpr int kSpAst = Fm<kFP4>::SCOLS + 8;            // LDS row stride of the activations
static_assert(Fm<kFP4>::PPR == 16, "16 activation pieces per row");
static_assert(Fm<kFP4>::SC == 1, "one chunk per stage");

template <int NMB>
constexpr int sp_stage_bytes() { return 32 * NMB * kSpAst * 2; }

struct SpB {
  uint4 b[2][2];   // raw FP4 words: row block nb (rows 32 nb .. + 31 of the tile), k-half kk
  uint2 sc[2];     // the scale words of the lane's row in each row block
};

// weights of stage s (past nst or !b_on: an empty resource, zeros). For row
// block nb and k-half kk lane l takes lane-chunk 16 (2 kk + l / 32) + l % 16
// of row group 2 nb + (l % 32) / 16: columns 16 ks + 8 (l / 32) .. + 7 of row
// 32 nb + l % 32 for the k-steps ks = kk (mod 2); the scale word from the
// same lane-chunk of the scale slot.
template <int BAUX>
__device__ __forceinline__ void sp_fetch_b(const WMat& W, int tile, bool b_on, int s, int nst, SpB& R) {
  using F = Fm<kFP4>;
  const bool live = s < nst && b_on;
  s = min(s, nst - 1);
  const int lane = threadIdx.x & 63;
  const int kmat = W.g.k;
  const int spm = (kmat + F::SCOLS - 1) / F::SCOLS;
  const int mat = s / spm, col0 = (s % spm) * F::SCOLS;
  const int ss = col0 / kSSCols, cin0 = (col0 % kSSCols) / F::CC;
  const int ncs = ss_code_slots(kFP4, min(kSSCols, kmat - ss * kSSCols));
  const rsrc_t wt = rsrc(W.base + (size_t)mat * W.mat_bytes + (size_t)tile * W.g.tile_slots * kSlot,
                         live ? (uint32_t)(W.g.tile_slots * kSlot) : 0u);
  const int sso = ss * W.g.full * kSlot;
  const int vb = ((lane & 31) >> 4) * kSlot + (16 * (lane >> 5) + (lane & 15)) * 16;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      R.b[nb][kk] = ldb<BAUX>(wt, vb, sso + (cin0 * 4 + 2 * nb) * kSlot + kk * 512);
  const int vs = (16 * ((lane & 31) >> 4) + (lane & 15)) * 16 + 8 * cin0;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    R.sc[nb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                             wt, vs, sso + ncs * kSlot + nb * 512, BAUX));
}

// Activation staging with NW waves: the 32 NMB x SCOLS tile of a stage is
// 512 NMB pieces of 8 columns; thread x stages pieces x + 64 NW i, i.e.
// columns c = 8 (x % 16) .. + 7 of rows m + 4 NW i (m = x / 16) below 32 NMB.
template <int NMB, int NW>
struct SpA {
  static constexpr int PPT = (512 * NMB + 64 * NW - 1) / (64 * NW);   // pieces per thread
  static constexpr int RS = 4 * NW;                                   // row step between them
  static constexpr int TT = 32 * NMB;
  __device__ static constexpr bool live(int i, int m) { return m + RS * i < TT; }
};

// the thread's activation pieces of stage s (ap[i] points at column c of its
// row, clamped into the row past k)
template <int NMB, int NW>
__device__ __forceinline__ void sp_fetch_a(const uint16_t* const (&ap)[SpA<NMB, NW>::PPT], int c, int kmat,
                                           int s, int nst, uint4 (&v)[SpA<NMB, NW>::PPT]) {
  s = min(s, nst - 1);
  const int spm = (kmat + Fm<kFP4>::SCOLS - 1) / Fm<kFP4>::SCOLS;
  const int col0 = (s % spm) * Fm<kFP4>::SCOLS;
#pragma unroll
  for (int i = 0; i < SpA<NMB, NW>::PPT; ++i) v[i] = *(const uint4*)(ap[i] + min(col0, kmat - 8 - c));
}

template <int NMB, int NW>
__device__ __forceinline__ void sp_store(uint8_t* st, const uint4 (&v)[SpA<NMB, NW>::PPT], int kmat, int c,
                                         int m, uint32_t rvalid, int s) {
  using P = SpA<NMB, NW>;
  const int spm = (kmat + Fm<kFP4>::SCOLS - 1) / Fm<kFP4>::SCOLS;
  const int col0 = (s % spm) * Fm<kFP4>::SCOLS;
#pragma unroll
  for (int i = 0; i < P::PPT; ++i) {
    if (!P::live(i, m)) continue;   // only the last piece of a thread can fall past the tile
    // an AND, not a select: the load cannot be sunk down to this store
    const uint32_t mk = (((rvalid >> i) & 1u) && col0 + c < kmat) ? ~0u : 0u;
    *(uint4*)((uint16_t*)st + (m + P::RS * i) * kSpAst + c) =
        make_uint4(v[i].x & mk, v[i].y & mk, v[i].z & mk, v[i].w & mk);
  }
}

// one stage: per k-step the activation fragments of the NMB token blocks
// (read one k-step ahead) against the two decoded weight fragments of the
// wave's tile
template <int NMB>
__device__ __forceinline__ void sp_mfma(const uint8_t* st, const SpB& R, f16v (&acc)[NMB][2]) {
  using F = Fm<kFP4>;
  const int lane = threadIdx.x & 63, row = lane & 31, kh = lane >> 5;
  const uint16_t* As = (const uint16_t*)st;
  uint4 a[2][NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) a[0][mb] = *(const uint4*)(As + (32 * mb + row) * kSpAst + 8 * kh);
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) {
    const int kk = ks & 1, b = ks >> 1;              // k-half, 32-column block of the chunk
    if (ks + 1 < F::KS)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        a[(ks + 1) & 1][mb] = *(const uint4*)(As + (32 * mb + row) * kSpAst + 16 * (ks + 1) + 8 * kh);
    uint4 bw[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bw[nb] = decode_b<kFP4>(R.b[nb][kk], R.sc[nb], b, b, 2 * kk + kh);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a[ks & 1][mb]),
                                                             __builtin_bit_cast(half8, bw[nb]), acc[mb][nb],
                                                             0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Pieces [npieces[lo], npieces[hi]) of at most 32 NMB tokens; NW waves, one
// 64-row weight tile each (a wave past the last tile computes on zero weights
// and stores nothing).
template <int EPI, int NMB, int NW>
__global__ __launch_bounds__(64 * NW) void k_grouped_short(Grouped a, int lo, int hi) {
  using P = SpA<NMB, NW>;
  constexpr int TT = P::TT;                            // tokens per workgroup
  __shared__ __align__(16) uint8_t smem[2 * sp_stage_bytes<NMB>()];
  __shared__ int arow[TT];
  // piece p runs on XCD p % 8, its weight-tile groups back to back
  const int nocts = (a.ntiles + NW - 1) / NW;
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int oct = q % nocts;
  const int p = a.npieces[lo] + xcd + 8 * (q / nocts);
  if (p >= a.npieces[hi]) return;
  const Piece pc = a.pieces[p];
  const int cnt = min(TT, pc.count);
  const int e = pc.expert;
  static_assert(64 * NW >= TT, "one thread per token row");
  if (threadIdx.x < TT) {
    const int i = threadIdx.x;
    int row = -1;
    if (i < cnt) {
      const int pos = pc.start + i;
      row = EPI == kGateUp ? (a.perm[pos] / a.K) * a.G + a.labels[e] : pos;
    }
    arow[i] = row;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int tile = NW * oct + wave;
  const bool b_on = tile < a.ntiles;
  const uint8_t* base = a.experts + (size_t)e * a.estride;
  const WMat W{base + a.woff, a.g, 0, 1};
  const int nst = n_stages<kFP4>(W), kmat = a.A.kmat;
  const int c = 8 * (threadIdx.x % 16), m = threadIdx.x / 16;
  const uint16_t* ap[P::PPT];
  uint32_t rvalid = 0;
#pragma unroll
  for (int i = 0; i < P::PPT; ++i) {
    const int arw = P::live(i, m) ? arow[m + P::RS * i] : -1;
    rvalid |= (arw >= 0 ? 1u : 0u) << i;
    ap[i] = a.A.p + (size_t)max(arw, 0) * a.A.rs + c;
  }
  f16v acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
  constexpr int SB = sp_stage_bytes<NMB>();
  uint4 ra[3][P::PPT];
  SpB rb[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) sp_fetch_a<NMB, NW>(ap, c, kmat, i, nst, ra[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) sp_fetch_b<kAuxNT>(W, tile, b_on, i, nst, rb[i]);
  sp_store<NMB, NW>(smem, ra[0], kmat, c, m, rvalid, 0);
  __syncthreads();
  // stage s with sets i = s % 3: weights of s + 2 into the set the MFMAs of
  // s - 1 read, activations of s + 3 into the set stored at s - 1, the
  // activations of s + 1 stored (past the end: a stale set into the buffer
  // no wave reads again), the MFMAs of s
  const auto step = [&](int s, int i) {
    sp_fetch_b<kAuxNT>(W, tile, b_on, s + 2, nst, rb[(i + 2) % 3]);
    sp_fetch_a<NMB, NW>(ap, c, kmat, s + 3, nst, ra[i]);
    sp_store<NMB, NW>(smem + ((s + 1) & 1) * SB, ra[(i + 1) % 3], kmat, c, m, rvalid, min(s + 1, nst - 1));
    sp_mfma<NMB>(smem + (s & 1) * SB, rb[i], acc);
    __syncthreads();
  };
  int s0 = 0;
  for (; s0 + 3 <= nst; s0 += 3) {
    step(s0, 0);
    step(s0 + 1, 1);
    step(s0 + 2, 2);
  }
  if (s0 < nst) step(s0, 0);
  if (s0 + 1 < nst) step(s0 + 1, 1);
  if (!b_on) return;
  const float* ts = (const float*)(base + a.ts_off);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = acc_tok(lane, mb, v);
      if (i >= cnt) continue;
      const size_t pos = (size_t)pc.start + i;
      if constexpr (EPI == kGateUp) {
        const float tg = ts[0], tu = ts[1];
        const int f = 32 * tile + (lane & 31);
        // gate and up carry the token's range scale c: h = silu(g) u c^2
        const float c = a.psc[pos];
        const float hv = silu(acc[mb][0][v] * tg * inv_pow2(c)) * (acc[mb][1][v] * tu * c);
        ((_Float16*)a.out)[pos * a.ostride + f] = (_Float16)hv;
      } else {
        const float sc = a.topk_w[a.perm[pos]] * ts[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          const int n = 64 * tile + 32 * rg + (lane & 31);
          ((_Float16*)a.out)[pos * a.ostride + n] = (_Float16)(acc[mb][rg][v] * sc);
        }
      }
    }
}

// Expert down projection with the activations resident in LDS. The down
// matrix has K = expert ffn (640 at the 145B shapes): five FP4 stages, too
// few for a per-tile pipeline to amortise its ramp and per-stage barriers.
// Here a workgroup of NW waves takes one 32 NMB-token block of a piece (its
// 32 NMB x K fp16 activations fit the LDS), stages it once, and each wave then
// walks its weight tiles (w, w + NW, ...) as one flat sequence of
// (tile, stage) items: weights read straight into MFMA operand registers
// two items ahead across tile boundaries, no barrier after the staging, and
// each tile's weighted outputs stored after its last stage.

constexpr int kResMaxK = 1024;                         // largest K kept resident
constexpr int kResAst = kResMaxK + 8;                  // LDS row stride (elements)

// weights of item `it` of the wave's sequence (past n: an empty resource)
__device__ __forceinline__ void res_fetch(const WMat& W, int wave, int nw, int it, int n, int nst, SpB& R) {
  const int j = min(it, n - 1);
  const int tile = wave + nw * (j / nst);
  sp_fetch_b<kAuxNT>(W, tile, it < n, j % nst, nst, R);
}

// pieces [npieces[lo], npieces[hi]) (lo < 0: from the first one) in nsub
// blocks of 32 NMB tokens
template <int NW, int NMB>
__global__ __launch_bounds__(64 * NW) void k_down_res(Grouped a, int lo, int hi, int nsub) {
  constexpr int kResTT = 32 * NMB;                     // tokens per workgroup
  __shared__ __align__(16) uint16_t As[kResTT * kResAst];
  __shared__ float tsc[kResTT];
  // piece p runs on XCD p % 8, its token blocks back to back
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int h = q % nsub, p = (lo < 0 ? 0 : a.npieces[lo]) + xcd + 8 * (q / nsub);
  if (p >= a.npieces[hi]) return;
  const Piece pc = a.pieces[p];
  const int t0 = kResTT * h, cnt = min(kResTT, pc.count - t0);
  if (cnt <= 0) return;
  const uint8_t* base = a.experts + (size_t)pc.expert * a.estride;
  const float* ts = (const float*)(base + a.ts_off);
  const WMat W{base + a.woff, a.g, 0, 1};
  const int nst = n_stages<kFP4>(W), kmat = a.A.kmat, kpad = nst * Fm<kFP4>::SCOLS;
  if (threadIdx.x < kResTT) {
    const int i = threadIdx.x;
    tsc[i] = i < cnt ? a.topk_w[a.perm[pc.start + t0 + i]] * ts[2] : 0.f;
  }
  // stage the block: rows past the piece and columns past K are zeros
  {
    const int ppr = kpad / 8, npc = kResTT * ppr;
    for (int x = threadIdx.x; x < npc; x += 64 * NW) {
      const int r = x / ppr, c = 8 * (x % ppr);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < cnt && c < kmat) v = *(const uint4*)(a.A.p + (size_t)(pc.start + t0 + r) * a.A.rs + c);
      *(uint4*)(As + r * kResAst + c) = v;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int ntw = (a.ntiles - wave + NW - 1) / NW;     // the wave's tiles
  const int n = ntw * nst;
  if (n <= 0) return;
  const int row = lane & 31, kh = lane >> 5;
  f16v acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
  SpB rb[3];
  res_fetch(W, wave, NW, 0, n, nst, rb[0]);
  res_fetch(W, wave, NW, 1, n, nst, rb[1]);
  // item it with set i = it % 3: weights of it + 2 into the set item it - 1
  // read, the MFMAs of it over the stage's columns of the resident block, and
  // after a tile's last stage its outputs
  const auto item = [&](int it, int i) {
    res_fetch(W, wave, NW, it + 2, n, nst, rb[(i + 2) % 3]);
    const int st = it % nst;
    const uint16_t* Ab = As + Fm<kFP4>::SCOLS * st + 8 * kh;
    uint4 av[2][NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) av[0][mb] = *(const uint4*)(Ab + (32 * mb + row) * kResAst);
#pragma unroll
    for (int ks = 0; ks < Fm<kFP4>::KS; ++ks) {
      const int kk = ks & 1, b = ks >> 1;
      if (ks + 1 < Fm<kFP4>::KS)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          av[(ks + 1) & 1][mb] = *(const uint4*)(Ab + (32 * mb + row) * kResAst + 16 * (ks + 1));
      uint4 bw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bw[nb] = decode_b<kFP4>(rb[i].b[nb][kk], rb[i].sc[nb], b, b, 2 * kk + kh);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, av[ks & 1][mb]),
                                                               __builtin_bit_cast(half8, bw[nb]), acc[mb][nb],
                                                               0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (st == nst - 1) {
      const int tile = wave + NW * (it / nst);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = acc_tok(lane, mb, v);
          const float sc = tsc[t];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (t < cnt)
              ((_Float16*)a.out)[(size_t)(pc.start + t0 + t) * a.ostride + 64 * tile + 32 * nb + (lane & 31)] =
                  (_Float16)(acc[mb][nb][v] * sc);
            acc[mb][nb][v] = 0.f;
          }
        }
    }
  };
  int i0 = 0;
  for (; i0 + 3 <= n; i0 += 3) {
    item(i0, 0);
    item(i0 + 1, 1);
    item(i0 + 2, 2);
  }
  if (i0 < n) item(i0, 0);
  if (i0 + 1 < n) item(i0 + 1, 1);
}

// Waves per k_grouped_short workgroup: 8, or 4 for a matrix of at most four
// 64-row tiles. Measured on the 145B prefill: 8-wave workgroups with idle
// waves in the last group (20 and 28 tiles) beat 5- and 7-wave ones that
// divide the tile count, which leave SIMD slots of the CU empty.
static int short_waves(int ntiles) { return ntiles <= 4 ? 4 : 8; }

template <int EPI, int NMB>
static int launch_short(const Grouped& a, unsigned npc, int lo, int hi, hipStream_t st) {
  const int nw = short_waves(a.ntiles);
  const unsigned grid = 8u * ((a.ntiles + nw - 1) / nw) * ((npc + 7) / 8);
  switch (nw) {
    case 8: hipLaunchKernelGGL((k_grouped_short<EPI, NMB, 8>), dim3(grid), dim3(64 * 8), 0, st, a, lo, hi); break;
    default: hipLaunchKernelGGL((k_grouped_short<EPI, NMB, 4>), dim3(grid), dim3(64 * 4), 0, st, a, lo, hi); break;
  }
  LMOE_HIP(hipGetLastError());
  return 0;
}

// The three grouped launches of one expert matrix: pieces of more than 64
// tokens in 128-token tiles, then those of 33..64 and of at most 32 tokens
// (each class holds at most one piece per expert).
template <int EPI>
static int launch_grouped(const Grouped& a, unsigned maxp, int E, hipStream_t st) {
  const unsigned ncls = std::min<unsigned>(maxp, E);
  if constexpr (EPI == kGateUp)
    if (a.A.kmat % Fm<kFP4>::SCOLS == 0) {
      hipLaunchKernelGGL(k_grouped_dma<EPI>, dim3(8u * a.nquads * ((maxp + 7) / 8)), dim3(NTH), 0, st, a);
      LMOE_HIP(hipGetLastError());
      if (int rc = launch_short<EPI, 2>(a, ncls, 1, 2, st)) return rc;
      return launch_short<EPI, 1>(a, ncls, 2, 0, st);
    }
  if (EPI == kDown && a.A.kmat <= kResMaxK) {
    // pieces of more than 32 tokens in 64-token blocks, the rest in 32
    hipLaunchKernelGGL((k_down_res<8, 2>), dim3(8u * 2 * ((maxp + 7) / 8)), dim3(512), 0, st, a, -1, 2, 2);
    LMOE_HIP(hipGetLastError());
    hipLaunchKernelGGL((k_down_res<8, 1>), dim3(8u * ((ncls + 7) / 8)), dim3(512), 0, st, a, 2, 0, 1);
    LMOE_HIP(hipGetLastError());
    return 0;
  }
  hipLaunchKernelGGL(k_grouped<EPI>, dim3(8u * a.nquads * ((maxp + 7) / 8)), dim3(NTH), 0, st, a);
  LMOE_HIP(hipGetLastError());
  if (int rc = launch_short<EPI, 2>(a, ncls, 1, 2, st)) return rc;
  return launch_short<EPI, 1>(a, ncls, 2, 0, st);
}

// ---------------------------------------------------------------------------
// Staging of the input rows.

struct Prep {
  const float* x;
  int T, H;
  int norm;
  float eps;
  _Float16* xh;     // [T][H]
  __bf16* xb;       // [T][2][H]
  double* xnorm;    // [T] |staged row|_2
  float* r;         // [T] the row scale (1/rms, or 1)
  double* r64;      // [T] the same in fp64 (exact 1/rms for the fp64 logits)
  float* xsc;       // [T] power-of-two scale of the fp16 rows
};

// Range of the fp16 activations. A staged row whose largest magnitude m lies
// outside [2^-3, 2^6) is multiplied by the power of two c that brings m into
// [4, 8) (|log2 c| <= 60), so that the fp16 copies of x, D x and of what
// follows neither overflow nor lose bits to subnormals. The path is linear in
// x up to the SwiGLU: D x, the gate and up rows carry c, h = silu(g) u is
// formed from the unscaled gate and carries c^2 (so do the expert outputs,
// the per-group sums and the shared expert's hidden row), and U's
// accumulators are multiplied by c^-2. Powers of two make every one of these
// steps exact, and c = 1 (every unit-scale and every normalized row) leaves
// the arithmetic as it is without them.
__device__ __forceinline__ float range_scale(float m) {
  if (!(m > 0.f) || !(m < 3.0e38f) || (m >= 0.125f && m < 64.f)) return 1.f;
  int ex;
  frexpf(m, &ex);                                       // m = f 2^ex, f in [0.5, 1)
  return ldexpf(1.f, max(-60, min(60, 3 - ex)));
}

// Sum / maximum over the block (at most 8 waves), every thread gets it.
__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  __syncthreads();
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

// One block per token, one 8-column chunk per thread (blockDim = H / 8
// rounded up to 64, H <= 4096): the row is read once and held in registers
// for the second pass.
__global__ __launch_bounds__(512) void k_prep(Prep a) {
  __shared__ double red[8];
  __shared__ float redm[8];
  const int t = blockIdx.x, c = threadIdx.x;
  const float* xr = a.x + (size_t)t * a.H;
  const bool own = c < a.H / 8;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (own) {
    const float4 u0 = *(const float4*)(xr + 8 * c), u1 = *(const float4*)(xr + 8 * c + 4);
    v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
    v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
  }
  float r = 1.0f;
  double r64 = 1.0;
  double s = 0.0;
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (a.norm) s += (double)v[j] * v[j];
    m = fmaxf(m, fabsf(v[j]));
  }
  m = block_max(m, redm);
  if (a.norm) {
    s = block_sum(s, red);
    r64 = 1.0 / sqrt(s / a.H + (double)a.eps);
    r = (float)r64;
  }
  // the largest staged magnitude, up to rounding (enough to pick the scale)
  const float xs = range_scale(m * r);
  double s2 = 0.0;
  half8 h;
  bf16x8 b0, b1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (a.norm) v[j] *= r;
    h[j] = (_Float16)(v[j] * xs);
    b0[j] = (__bf16)v[j];
    b1[j] = (__bf16)(v[j] - (float)b0[j]);
    s2 += (double)v[j] * v[j];
  }
  if (own) {
    *(half8*)(a.xh + (size_t)t * a.H + 8 * c) = h;
    *(bf16x8*)(a.xb + (size_t)t * 2 * a.H + 8 * c) = b0;
    *(bf16x8*)(a.xb + (size_t)t * 2 * a.H + a.H + 8 * c) = b1;
  }
  s2 = block_sum(s2, red);
  if (threadIdx.x == 0) {
    a.xnorm[t] = sqrt(s2);
    a.r[t] = r;
    a.r64[t] = r64;
    a.xsc[t] = xs;
  }
}

// ---------------------------------------------------------------------------
// Routing: certified candidates, fp64 rescoring, top-K, softmax.

struct Select {
  const float* logits;       // [nsplit][T][Epad] fp32 router GEMM partial sums
  int nsplit;
  int Epad, T, E, H, K;
  const float* bias;         // [E]
  const float* x;            // [T][H] raw input rows
  const double* r;           // [T] row scale (fp64)
  const double* xnorm;       // [T]
  const double* wmax;        // max_e |Wr_e|_2
  const uint16_t* wr;        // router bf16 [E][H] row-major
  double cbeta;              // rounding bound per unit |x| |w|
  int* idx;                  // [T][K]
  float* w;                  // [T][K]
};

__device__ __forceinline__ double bf16_to_f64(uint32_t bits) {
  return (double)__uint_as_float(bits << 16);
}

// The x row of a token in the registers of a wave: lane l holds columns
// 8 l + 512 j .. + 7 for j < NJ (H <= 512 NJ), zeros past H. Held in fp32
// (half the registers of fp64) and widened exactly at each product.
template <int NJ>
struct XRow {
  float v[NJ][8];
};

template <int NJ>
__device__ __forceinline__ XRow<NJ> load_xrow(const float* xr, int H) {
  const int lane = threadIdx.x & 63;
  XRow<NJ> X;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 8 * lane + 512 * j;
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (c < H) {
      x0 = *(const float4*)(xr + c);
      x1 = *(const float4*)(xr + c + 4);
    }
    X.v[j][0] = x0.x; X.v[j][1] = x0.y; X.v[j][2] = x0.z; X.v[j][3] = x0.w;
    X.v[j][4] = x1.x; X.v[j][5] = x1.y; X.v[j][6] = x1.z; X.v[j][7] = x1.w;
  }
  return X;
}

// wave arg-max over (value desc, index asc)
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  for (int o = 32; o > 0; o >>= 1) {
    const double ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

constexpr int kMaxE = 1024;
constexpr int kMaxG = 64;     // groups (the create-time limit)

// Sum over the wave, every lane gets it: DPP exchanges within each row of
// 16 lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row
// sums from lanes 0, 16, 32, 48, added in that order. Fixed order:
// deterministic.
__device__ __forceinline__ double dpp_f64(double v, int ctrl_id) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  switch (ctrl_id) {
    case 0: lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false); break;
    case 1: lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false); break;
    case 2: lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false); break;
    default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, false);
             hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64(v, 0);
  v += dpp_f64(v, 1);
  v += dpp_f64(v, 2);
  v += dpp_f64(v, 3);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// fp32 -> unsigned key with the same order (NaN lowest)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// NJ: 512-column chunks of a row (H <= 512 NJ); EPL: experts per lane
// (E <= 64 EPL), so the registers fit the layer
template <int NJ, int EPL>
__global__ __launch_bounds__(256, 4) void k_select(Select a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  // fp32 logits (the router GEMM's k-splits added in fp32, in split order:
  // one more fp32 summation order of the same products) + bias, exactly in
  // fp64; their fp32 roundings as ordered keys
  double v[EPL];
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < a.E) {
      float l = a.logits[(size_t)t * a.Epad + e];
      for (int k = 1; k < a.nsplit; ++k) l += a.logits[((size_t)k * a.T + t) * a.Epad + e];
      v[i] = (double)l + (double)a.bias[e];
      key[i] = order_key((float)v[i]);
    } else {
      v[i] = -INFINITY;
      key[i] = 0u;
    }
  }
  // the K-th largest fp32-rounded value, bit by bit from the top: the
  // largest key kt with at least K keys >= kt (ballots and popcounts, no
  // lane exchanges). Rounding is monotone, so it is the rounding of the
  // K-th largest v; one fp32 ulp (and a subnormal step) below it bounds
  // that v from below.
  uint32_t kt = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = kt | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) cnt += __popcll(__ballot(key[i] >= c));
    if (cnt >= a.K) kt = c;
  }
  const float fk = key_float(kt);
  const double vk = kt == 0u ? -INFINITY
                  : isinf(fk) ? (double)fk
                              : (double)fk - (fabs((double)fk) * 0x1p-23 + 0x1p-149);
  // every expert whose exact logit can reach the top K: its fp32 logit is
  // within 2 beta of the K-th largest (|fp32 - exact| <= beta for all e)
  const double beta = a.cbeta * a.xnorm[t] * *a.wmax + 1e-30;
  const double thr = vk - 2.0 * beta;
  const double rt = a.r[t];
  const XRow<NJ> X = load_xrow<NJ>(a.x + (size_t)t * a.H, a.H);   // read once for every candidate
  unsigned long long cm[EPL];                              // candidates, per slot (uniform)
  int nc = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    cm[i] = __ballot(lane + 64 * i < a.E && v[i] >= thr);
    nc += __popcll(cm[i]);
  }
  // the candidate after expert e (or -1): the next set bit in slot order
  const auto next_cand = [&](int e) {
    int i0 = (e + 1) >> 6;
    unsigned long long m0 = i0 < EPL ? cm[i0] & (~0ull << ((e + 1) & 63)) : 0ull;
    for (int i = i0; i < EPL; ++i) {
      const unsigned long long m = i == i0 ? m0 : cm[i];
      if (m) return 64 * i + __builtin_ctzll(m);
    }
    return -1;
  };
  // the lane's router words of expert e: columns 8 lane + 512 j .. + 7
  const auto load_row = [&](int e, uint4 (&w)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = 8 * lane + 512 * j;
      w[j] = c < a.H ? *(const uint4*)(a.wr + (size_t)e * a.H + c) : make_uint4(0, 0, 0, 0);
    }
  };
  // exact fp64 logits of the candidates, in expert order; the next
  // candidate's router row is loaded while the current one's dot product
  // runs. Lane c keeps candidate c (c < 64); ex[] keeps them by expert.
  double ex[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) ex[i] = -INFINITY;
  double cl = -INFINITY;
  int ce = 0x7FFFFFFF;
  bool nan_seen = false;
  int e = next_cand(-1), c = 0;
  uint4 wc[NJ];
  if (e >= 0) load_row(e, wc);
  while (e >= 0) {
    const int en = next_cand(e);
    uint4 wn[NJ];
    if (en >= 0) load_row(en, wn);
    double sd = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint4 w = wc[j];
      // widened here, per candidate (an empty asm keeps the compiler from
      // hoisting the conversions and holding the row in fp64 registers)
      float xv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xv[k] = X.v[j][k];
        asm volatile("" : "+v"(xv[k]));
      }
      sd = fma((double)xv[0], bf16_to_f64(w.x & 0xFFFFu), sd);
      sd = fma((double)xv[1], bf16_to_f64(w.x >> 16), sd);
      sd = fma((double)xv[2], bf16_to_f64(w.y & 0xFFFFu), sd);
      sd = fma((double)xv[3], bf16_to_f64(w.y >> 16), sd);
      sd = fma((double)xv[4], bf16_to_f64(w.z & 0xFFFFu), sd);
      sd = fma((double)xv[5], bf16_to_f64(w.z >> 16), sd);
      sd = fma((double)xv[6], bf16_to_f64(w.w & 0xFFFFu), sd);
      sd = fma((double)xv[7], bf16_to_f64(w.w >> 16), sd);
    }
    const double l = wave_sum_f64(sd) * rt + (double)a.bias[e];
    nan_seen |= l != l;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + 64 * i) ex[i] = l;
    if (lane == c) {
      cl = l;
      ce = e;
    }
    ++c;
    if (en >= 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) wc[j] = wn[j];
    }
    e = en;
  }
  double kv = 0.0, top = 0.0;
  int ki = 0;
  bool mine = false;   // this lane writes output slot `slot`
  int slot = 0;
  if (nc >= a.K && nc <= 64 && !nan_seen) {
    // rank of lane c's candidate among all: larger logit first, then lower
    // expert index; the K best go to slots 0 .. K-1
    int rank = 0;
    top = -INFINITY;
    for (int j = 0; j < nc; ++j) {
      const double lj = readlane_f64(cl, j);
      const int ej = __builtin_amdgcn_readlane(ce, j);
      top = fmax(top, lj);
      rank += (lj > cl || (lj == cl && ej < ce)) ? 1 : 0;
    }
    mine = lane < nc && rank < a.K;
    slot = rank;
    kv = cl;
    ki = ce;
  } else {
    // general case (more than 64 candidates, fewer than K, or a NaN): top K
    // of the exact logits by K wave arg-max rounds; lane k keeps the k-th.
    // Taken experts and e >= E are NaN (never chosen); experts outside the
    // candidate set stay at -inf, so K distinct valid experts come out even
    // for rows with NaN logits.
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i >= a.E) ex[i] = NAN;
    for (int k = 0; k < a.K; ++k) {
      double bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int ee = lane + 64 * i;
        if (ex[i] > bv || (ex[i] == bv && ee < bi)) {
          bv = ex[i];
          bi = ee;
        }
      }
      wave_argmax(bv, bi);
      if (k == 0) top = bv;
      if (lane == k) {
        kv = bv;
        ki = bi;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == bi) ex[i] = NAN;
    }
    mine = lane < a.K;
    slot = lane;
  }
  const double z = mine ? exp(kv - top) : 0.0;
  const double zs = wave_sum_f64(z);
  if (mine) {
    a.idx[(size_t)t * a.K + slot] = ki;
    a.w[(size_t)t * a.K + slot] = (float)(z / zs);
  }
}

// ---------------------------------------------------------------------------
// Permutation.

struct Perm {
  const int* idx;        // [T][K]
  int T, K, E, G, nchunk;
  unsigned long long* cmask;   // [nchunk][E]
  unsigned long long* gmask;   // [nchunk][G]: the chunk's tokens with an assignment in group g
  int* ccnt;             // [nchunk][E] tokens of the chunk per expert
  int* cbase;            // [nchunk][E] tokens of earlier chunks per expert
  const int* eorder;     // [E] experts in (label, expert) order
  const uint8_t* labels;
  int* seg_start;        // [E]
  int* expert_count;     // [E]
  int* group_off;        // [G+1]
  Piece* pieces;
  int* npieces;
  int* perm;             // [T*K]
  int* inv;              // [T*K]
  const float* xsc;      // [T] range scale per token
  float* psc;            // [T*K] the same per sorted position
  int* gl_tok;           // [G][gcap] each group's routed tokens, ascending
  int* gl_cnt;           // [G]
  int gcap;
};

__global__ __launch_bounds__(256) void k_perm_mask(Perm a) {
  __shared__ unsigned long long m[kMaxE];
  __shared__ unsigned long long gm[kMaxG];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) m[e] = 0ull;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x) gm[g] = 0ull;
  __syncthreads();
  const int n = CHUNK_T * a.K;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int t = c * CHUNK_T + j / a.K;
    if (t < a.T) atomicOr(&m[a.idx[(size_t)t * a.K + j % a.K]], 1ull << (t % CHUNK_T));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    a.cmask[(size_t)c * a.E + e] = m[e];
    a.ccnt[(size_t)c * a.E + e] = __popcll(m[e]);
    if (m[e]) atomicOr(&gm[a.labels[e]], m[e]);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < a.G; g += blockDim.x) a.gmask[(size_t)c * a.G + g] = gm[g];
}

// one block of kMaxE threads: chunk prefixes, segment starts, group offsets
// and the piece list of the grouped GEMMs
__device__ __forceinline__ void perm_scan_block(const Perm& a) {
  __shared__ int sc[kMaxE];
  __shared__ int sp[kMaxE];
  __shared__ int sf[kMaxE];
  __shared__ int sq[kMaxE];
  __shared__ int sm_[kMaxE];
  __shared__ int ss_[kMaxE];
  const int j = threadIdx.x;
  if (j < a.E) {
    // running count over the chunks, 16 chunk loads in flight at a time
    int cnt = 0;
    for (int c0 = 0; c0 < a.nchunk; c0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = c0 + u < a.nchunk ? a.ccnt[(size_t)(c0 + u) * a.E + j] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < a.nchunk) {
          a.cbase[(size_t)(c0 + u) * a.E + j] = cnt;
          cnt += v[u];
        }
    }
    a.expert_count[j] = cnt;
  }
  __syncthreads();
  // counts in (label, expert) order
  const int e = j < a.E ? a.eorder[j] : 0;
  const int c_e = j < a.E ? a.expert_count[e] : 0;
  const int np = (c_e + BM - 1) / BM;
  // piece order: the full pieces of all experts, then the partial last
  // pieces of more than 64 tokens, of 33 to 64, of at most 32 (the grouped
  // GEMMs dispatch their longest work items first; the last two classes go
  // to k_grouped_short)
  const int nf = c_e / BM, nq = np - nf, rem = c_e - nf * BM;
  const int cls = nq == 0 ? -1 : rem > 2 * kShortT ? 0 : rem > kShortT ? 1 : 2;
  sc[j] = c_e;
  sp[j] = np;
  sf[j] = nf;
  sq[j] = cls == 0;
  sm_[j] = cls == 1;
  ss_[j] = cls == 2;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    const int x0 = j >= o ? sc[j - o] : 0, x1 = j >= o ? sp[j - o] : 0;
    const int x2 = j >= o ? sf[j - o] : 0, x3 = j >= o ? sq[j - o] : 0;
    const int x4 = j >= o ? sm_[j - o] : 0, x5 = j >= o ? ss_[j - o] : 0;
    __syncthreads();
    sc[j] += x0;
    sp[j] += x1;
    sf[j] += x2;
    sq[j] += x3;
    sm_[j] += x4;
    ss_[j] += x5;
    __syncthreads();
  }
  const int nbig = sf[kMaxE - 1] + sq[kMaxE - 1];   // pieces of more than 64 tokens
  const int nmid = nbig + sm_[kMaxE - 1];           // ... and of 33 to 64
  const int start = sc[j] - c_e, fstart = sf[j] - nf;
  const int qstart = cls == 0 ? sf[kMaxE - 1] + sq[j] - 1 : cls == 1 ? nbig + sm_[j] - 1 : nmid + ss_[j] - 1;
  if (j < a.E) {
    a.seg_start[e] = start;
    for (int i = 0; i < np; ++i) {
      Piece p;
      p.expert = e;
      p.start = start + i * BM;
      p.count = min(BM, c_e - i * BM);
      p.pad = 0;
      a.pieces[i < nf ? fstart + i : qstart] = p;
    }
    // the first expert of each label opens its group's segment
    const int lab = a.labels[e];
    const int prev = j > 0 ? a.labels[a.eorder[j - 1]] : -1;
    for (int g = prev + 1; g <= lab; ++g) a.group_off[g] = start;
    if (j == a.E - 1) {
      for (int g = lab + 1; g <= a.G; ++g) a.group_off[g] = sc[j];
      a.npieces[0] = sp[j];
      a.npieces[1] = nbig;
      a.npieces[2] = nmid;
    }
  }
}

// each group's routed tokens in ascending order (defined with the prefill
// D over the routed pairs below)
__device__ __forceinline__ void group_list_block(const unsigned long long* gmask, int nchunk, int G,
                                                 int gcap, int* gl_tok, int* gl_cnt, int g);

// Block 0: the scan above; blocks 1 .. G: group g - 1's token list (from
// the per-chunk group bitmasks k_perm_mask wrote), which only the routed D
// reads: one launch for both.
__global__ __launch_bounds__(kMaxE) void k_perm_scan(Perm a) {
  if (blockIdx.x == 0) perm_scan_block(a);
  else group_list_block(a.gmask, a.nchunk, a.G, a.gcap, a.gl_tok, a.gl_cnt, (int)blockIdx.x - 1);
}

__global__ __launch_bounds__(256) void k_perm_scatter(Perm a) {
  const int n = a.T * a.K;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int t = i / a.K, e = a.idx[i];
  const size_t ci = (size_t)(t / CHUNK_T) * a.E + e;
  const unsigned long long below = (1ull << (t % CHUNK_T)) - 1ull;
  const int pos = a.seg_start[e] + a.cbase[ci] + __popcll(a.cmask[ci] & below);
  a.perm[pos] = i;
  a.inv[i] = pos;
  a.psc[pos] = a.xsc[t];
}

// ---------------------------------------------------------------------------
// Combine: s[t][g] = sum over k ascending of o[pos(t, k)] for label g.

struct Combine {
  const int* idx;
  const int* inv;
  const uint8_t* labels;
  const _Float16* o;  // [T*K][L] weighted expert outputs, fp16
  _Float16* s;        // [T][G][L]
  int K, G, L;
};

// One block per token; a thread owns 8 columns (one 16-byte chunk) of the
// ell outputs. The token's K assignments are put in (group, k) order (each
// ranked by its own thread, in LDS); a thread loads its chunk of up to
// 16 of them at once and walks them in that order with one running fp32
// sum, writing each group's sum (zeros for groups the token skips) when the
// walk passes it: every group's sum is over ascending k.
constexpr int kCombBatch = 16;

__global__ __launch_bounds__(256) void k_combine(Combine a) {
  __shared__ int pos[64];
  __shared__ int lab[64];
  __shared__ int ord[64];                  // assignment k in (group, k) order
  const int t = blockIdx.x;
  if (threadIdx.x < a.K) {
    const size_t i = (size_t)t * a.K + threadIdx.x;
    pos[threadIdx.x] = a.inv[i];
    lab[threadIdx.x] = a.labels[a.idx[i]];
  }
  __syncthreads();
  if (threadIdx.x < a.K) {
    // rank of assignment k: those of lower labels, then those of its label before it
    const int k = threadIdx.x, lk = lab[k];
    int rank = 0;
    for (int j = 0; j < a.K; ++j) rank += (lab[j] < lk) || (lab[j] == lk && j < k);
    ord[rank] = k;
  }
  __syncthreads();
  const int nc = a.L / 8;
  for (int q = threadIdx.x; q < nc; q += blockDim.x) {
    _Float16* out = a.s + (size_t)t * a.G * a.L + 8 * q;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int g = 0;
    const auto flush = [&]() {
      half8 h;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = (_Float16)acc[j];
        acc[j] = 0.f;
      }
      *(half8*)(out + (size_t)g * a.L) = h;
      ++g;
    };
    for (int k0 = 0; k0 < a.K; k0 += kCombBatch) {
      uint4 raw[kCombBatch];
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u)
        if (k0 + u < a.K) raw[u] = *(const uint4*)(a.o + (size_t)pos[ord[k0 + u]] * a.L + 8 * q);
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u) {
        if (k0 + u >= a.K) break;
        const int gi = lab[ord[k0 + u]];
        while (g < gi) flush();
        const half8 v = __builtin_bit_cast(half8, raw[u]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += (float)v[j];
      }
    }
    while (g < a.G) flush();
  }
}

// Load time: the Q8 / Q4 tiled stream of `nmat` matrices into the fp16
// tiled stream, with the decode the GEMM would do in registers (fp16(q * d),
// the same instructions), one thread per 16-byte lane-chunk of the output.
__global__ void k_dequant_du(const uint8_t* src, Geom gs, int fmt, uint8_t* dst, Geom gd, int nmat) {
  const size_t per_mat = (size_t)gd.tiles * gd.tile_slots * 64;
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_mat * nmat) return;
  const int mat = (int)(idx / per_mat);
  idx %= per_mat;
  const int lane = (int)(idx % 64);
  const int slot = (int)((idx / 64) % gd.tile_slots);
  const int tile = (int)(idx / 64 / gd.tile_slots);
  const int ss = slot / gd.full, j = slot % gd.full;
  const int c = j / 4, rg = j % 4;               // 32-column chunk of the super-step, row group
  const int cols = min(kSSCols, gd.k - ss * kSSCols);
  const uint8_t* sb = src + (size_t)mat * gs.bytes() + ((size_t)tile * gs.tile_slots + (size_t)ss * gs.full) * kSlot;
  const uint4 scw = *(const uint4*)(sb + (size_t)ss_code_slots(fmt, cols) * kSlot + (16 * rg + lane % 16) * 16);
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(word(scw, c >> 1) >> (16 * (c & 1))));
  uint4 out;
  if (fmt == kQ8) {
    const uint4 w = *(const uint4*)(sb + (size_t)((c / 2) * 4 + rg) * kSlot + lane * 16);
    const int b = c % 2;
    out = __builtin_bit_cast(uint4, q8_row8(word(w, 2 * b), word(w, 2 * b + 1), d));
  } else {
    const uint4 w = *(const uint4*)(sb + (size_t)((c / 4) * 4 + rg) * kSlot + lane * 16);
    out = __builtin_bit_cast(uint4, q4_row8(word(w, c % 4), d));
  }
  *(uint4*)(dst + (size_t)mat * gd.bytes() + ((size_t)tile * gd.tile_slots + slot) * kSlot + lane * 16) = out;
}

// fp16 latent rows to fp32 (debug copy)
// fp16 rows of `row` elements to fp32, the row's range scale taken out
__global__ void k_f16_to_f32(const _Float16* src, size_t n, size_t row, const float* xsc, float* dst) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (float)src[i] * inv_pow2(xsc[i / row]);
}

// max_e |Wr_e|_2 of the row-major bf16 router, fp64, one block
__global__ __launch_bounds__(1024) void k_router_wmax(const uint16_t* wr, int E, int H, double* out) {
  __shared__ double red[16];
  double mx = 0.0;
  for (int e = threadIdx.x >> 6; e < E; e += 16) {
    double s = 0.0;
    for (int c = threadIdx.x & 63; c < H; c += 64) {
      const double w = bf16_to_f64(wr[(size_t)e * H + c]);
      s += w * w;
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    mx = fmax(mx, sqrt(s));
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    double m = 0.0;
    for (int i = 0; i < 16; ++i) m = fmax(m, red[i]);
    // |w| is computed with relative error far below 1e-12; round it up
    *out = m * (1.0 + 1e-12);
  }
}

// y = residual + the NS partial sums of each split tile of a kEpiY launch,
// added in split order (deterministic): block b takes row b % BM of split
// tile b / BM, one column per thread; the NS loads are issued together.
// Plain float accesses: y and the residual are caller pointers with no
// alignment promise beyond float's.
// Block = 4 rows of one split tile, a thread 4 consecutive columns of one
// row (16-byte loads and stores); the partials are added in split order.
template <int NS>
__global__ __launch_bounds__(256) void k_ytiles(Dense a, const float* res) {
  constexpr int RPB = 4;                             // rows per block
  const int j = blockIdx.x / (BM / RPB), r = (blockIdx.x % (BM / RPB)) * RPB + (threadIdx.x >> 6);
  const int L = a.nfull + j, c = 4 * (threadIdx.x & 63);
  int mt, quad;
  tile_of(L, a.mtiles, a.nquads, mt, quad);
  const int t = mt * BM + r, n = 256 * quad + c;
  if (t >= a.T || n >= a.nvalid) return;
  const size_t tsz = (size_t)BM * 256, e = (size_t)r * 256 + c;
  const size_t i = (size_t)t * a.ostride + n;
  const float ic = inv_pow2(a.xsc[t]);
  float* out = (float*)a.out;
  if (n + 4 <= a.nvalid && (a.ostride & 3) == 0) {
    float4 p[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) p[k] = *(const float4*)(a.part + ((size_t)k * a.nrem + j) * tsz + e);
    float4 v = p[0];
#pragma unroll
    for (int k = 1; k < NS; ++k) {
      v.x += p[k].x; v.y += p[k].y; v.z += p[k].z; v.w += p[k].w;
    }
    v.x = v.x * ic * ic; v.y = v.y * ic * ic; v.z = v.z * ic * ic; v.w = v.w * ic * ic;
    if (res) {
      const float4 q = *(const float4*)(res + i);
      v.x = q.x + v.x; v.y = q.y + v.y; v.z = q.z + v.z; v.w = q.w + v.w;
    }
    *(float4*)(out + i) = v;
    return;
  }
  for (int u = 0; u < 4 && n + u < a.nvalid; ++u) {
    float v = a.part[((size_t)0 * a.nrem + j) * tsz + e + u];
#pragma unroll
    for (int k = 1; k < NS; ++k) v += a.part[((size_t)k * a.nrem + j) * tsz + e + u];
    v = v * ic * ic;
    out[i + u] = res ? res[i + u] + v : v;
  }
}

// ---------------------------------------------------------------------------
// Dense GEMM on fp16 weights with 128 x 128 wave tiles (the D projection):
// out[t][n] = sum_k A[t][k] W[n][k], fp16 out. A workgroup of 4 waves takes
// 256 tokens x 256 weight rows (4 tiles), wave (wm, wn) 128 tokens x 128 rows
// with its 256 accumulators in AGPRs (one wave per SIMD). Per 16-column
// k-step a wave reads 8 KB of fragments from LDS for 16 MFMAs, half of what
// the 64 x 64 wave tile of k_dense needs per MFMA, whose LDS bandwidth bounds
// it. Operands reach LDS by DMA (buffer_load ... lds: no registers, no LDS
// store instructions), 32 columns per stage in four buffers, issued three
// stages ahead. The weights' 1 KiB slots are copied as they are; activation
// rows are 64 B, their four 16 B pieces XOR-swizzled by (row / 2) % 4 so
// that fragment reads of 8 consecutive rows hit distinct banks.

constexpr int kWgT = 256, kWgN = 256, kWgCols = 32, kWgBuf = 4;
constexpr int kWgA = kWgT * kWgCols * 2;                 // activation bytes per stage
constexpr int kWgB = (kWgN / 64) * 4 * kSlot;            // weight bytes per stage
constexpr int kWgStage = kWgA + kWgB;
static_assert(kWgBuf * kWgStage <= 160 * 1024, "LDS");

// GATHER: D over the routed (token, group) pairs only. Blocks then take
// (group, 256-token tile of the group's tokens, quad), gather their rows by
// the DMA's per-lane source offsets and write each result row to its token's
// group columns; blocks past the last tile exit.
template <int EPI, bool GATHER>
__global__ __launch_bounds__(256) void k_dense16(Dense a) {
  __shared__ __align__(1024) uint8_t smem[kWgBuf * kWgStage];
  __shared__ int toks[GATHER ? kWgT : 1];
  const int nq = (a.ntiles + 3) / 4;
  int mt, quad, g = 0, nrows, sp = 0;
  const int nsp = EPI == kEpiY ? a.nsplit : 1;
  const uint8_t* wbase = a.W.base;
  if constexpr (!GATHER) {
    // kEpiY: split sp of the stages (the slowest index, so that the tiles
    // of one split that share rows sit together on an XCD)
    const int mtl = (a.T + kWgT - 1) / kWgT, ntl = mtl * nq;
    const int L0 = xcd_order(blockIdx.x, ntl * nsp);
    sp = L0 / ntl;
    tile_of(L0 % ntl, mtl, nq, mt, quad);
    nrows = min(kWgT, a.T - mt * kWgT);
  } else {
    // the grid is an upper bound; the work items (256-token tiles of the
    // groups' lists x quads) are ordered over the XCDs by their own count,
    // so that every XCD gets its share whatever the lists hold
    int nw = 0;
    for (int gg = 0; gg < a.G; ++gg) nw += (a.gl_cnt[gg] + kWgT - 1) / kWgT;
    nw *= nq;
    if ((int)blockIdx.x >= nw) return;
    const int L = xcd_order(blockIdx.x, nw);
    quad = L % nq;
    int lt = L / nq, c = 0;
    for (; g < a.G; ++g) {
      c = a.gl_cnt[g];
      const int nt = (c + kWgT - 1) / kWgT;
      if (lt < nt) break;
      lt -= nt;
    }
    if (g >= a.G) return;
    mt = lt;
    nrows = min(kWgT, c - mt * kWgT);
    wbase = a.W.base + (size_t)g * a.W.g.bytes();
    for (int i = threadIdx.x; i < kWgT; i += blockDim.x)
      toks[i] = i < nrows ? a.gl_tok[(size_t)g * a.gcap + (size_t)mt * kWgT + i] : 0;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = wave_id(), wm = wave & 1, wn = wave >> 1;
  // stages: 32 columns of W's nmat matrices one after another (their
  // activation columns contiguous), this block's share [st0, st1)
  const int spm = a.A.kmat / kWgCols, nst = spm * a.W.nmat;
  const int st0 = (int)((long long)nst * sp / nsp), st1 = (int)((long long)nst * (sp + 1) / nsp);
  // activation DMA: wave w stages rows 16 i .. + 15 for i = w + 4 j; lane l
  // the piece at position l % 4 of row 16 i + l / 4, which holds column
  // piece (l % 4) ^ ((row / 2) % 4). Rows past the tile's last read zeros.
  const rsrc_t ar = GATHER ? rsrc(a.A.p, (uint32_t)((size_t)a.T * a.A.rs * 2))
                           : rsrc(a.A.p + (size_t)mt * kWgT * a.A.rs, (uint32_t)(nrows * a.A.rs * 2));
  uint32_t avo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (wave + 4 * j) + (lane >> 2);
    const int pc = (lane & 3) ^ ((r >> 1) & 3);
    if constexpr (GATHER)
      avo[j] = r < nrows ? (uint32_t)(((size_t)toks[r] * a.A.rs + 8 * pc) * 2) : kOob;
    else
      avo[j] = (uint32_t)((r * a.A.rs + 8 * pc) * 2);
  }
  // weight DMA: wave w copies the 4 slots of stage s of tile 4 quad + w
  const int wt = 4 * quad + wave;
  const size_t wspan = (size_t)(a.W.nmat - 1) * a.W.mat_bytes + (size_t)a.W.g.tile_slots * kSlot;
  const rsrc_t br = rsrc(wbase + (size_t)min(wt, a.ntiles - 1) * a.W.g.tile_slots * kSlot,
                         wt < a.ntiles ? (uint32_t)wspan : 0u);
  const uint32_t sbase = lds_off(smem);
  const auto issue = [&](int s) {
    const int b = s & (kWgBuf - 1);
    const bool live = s < st1;
    const int sc = min(s, st1 - 1), mat = sc / spm, sm = sc % spm;
    const uint32_t col = (uint32_t)(sc * kWgCols * 2);
    const uint32_t st = sbase + b * kWgStage;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(live ? ar : rsrc(a.A.p, 0u), st + (wave + 4 * j) * 1024, avo[j], col);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      dma16(live ? br : rsrc(a.W.base, 0u), st + kWgA + (wave * 4 + rg) * 1024, lane * 16,
            (uint32_t)((size_t)mat * a.W.mat_bytes + (size_t)(4 * sm + rg) * kSlot));
  };
  f16v acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][j][v] = 0.f;
  const int row = lane & 31, kh = lane >> 5;
  // fragments of k-step ks (0, 1) of stage s
  const auto frags = [&](int s, int ks, uint4 (&af)[4], uint4 (&bf)[4]) {
    const uint8_t* st = smem + (s & (kWgBuf - 1)) * kWgStage;
    const uint16_t* As = (const uint16_t*)st;
    const uint4* Bs = (const uint4*)(st + kWgA);
    const int c = 2 * ks + kh;                       // 8-column piece of the stage
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = 128 * wm + 32 * mb + row;
      af[mb] = *(const uint4*)(As + m * kWgCols + 8 * (c ^ ((m >> 1) & 3)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = 2 * wn + (j >> 1), nb = j & 1;
      bf[j] = Bs[(tt * 4 + 2 * nb + (row >> 4)) * 64 + 16 * c + (lane & 15)];
    }
  };
  const auto mfmas = [&](const uint4 (&af)[4], const uint4 (&bf)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[mb][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, af[mb]),
                                                            __builtin_bit_cast(half8, bf[j]), acc[mb][j], 0, 0, 0);
  };
  issue(st0);
  issue(st0 + 1);
  issue(st0 + 2);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(16));             // this wave's first stage
  __syncthreads();
  uint4 a0[4], b0[4], a1[4], b1[4];
  frags(st0, 0, a0, b0);
  // stage s: second k-step's fragments read under the first's MFMAs; then
  // the wait for this wave's DMAs of stage s + 1 (those of s + 2, 8, may
  // stay in flight) and the barrier that makes every wave's visible and
  // ends all reads of stage s - 1, whose buffer stage s + 3 then refills;
  // the next stage's first fragments are read under the second k-step's
  // MFMAs (past the last stage they read a buffer of zeros, unused)
  // (scheduling barriers keep this order: the compiler would otherwise read
  // each fragment just before its MFMA and expose the LDS latency)
  for (int s = st0; s < st1; ++s) {
    frags(s, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(8));
    __syncthreads();
    issue(s + 3);
    frags(s + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the trailing DMAs (empty resources) write the buffers of stages past the
  // end, which no wave reads: let them land before the workgroup's LDS is freed
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 128 * wm + acc_tok(lane, mb, v);
      if (r >= nrows) continue;
      const size_t orow = GATHER ? (size_t)toks[r] * a.ostride + (size_t)g * a.gL
                                 : (size_t)(mt * kWgT + r) * a.ostride;
      const int t = mt * kWgT + r;
      // kEpiY: the 128-token half of the tile that holds row r, as a tile of
      // the kEpiY partial layout (BM tokens x 256 columns)
      const int L128 = EPI == kEpiY ? tile_index(2 * mt + wm, quad, a.mtiles, a.nquads) : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tile = 4 * quad + 2 * wn + (j >> 1);
        if (tile >= a.ntiles) continue;
        const int n = 64 * tile + 32 * (j & 1) + (lane & 31);
        if constexpr (EPI == kEpiF16) {
          ((_Float16*)a.out)[orow + n] = (_Float16)acc[mb][j][v];
        } else if constexpr (EPI == kEpiY) {
          if (nsp > 1) {
            const size_t jj = (size_t)sp * a.nrem + L128;
            a.part[(jj * BM + (t - (2 * mt + wm) * BM)) * 256 + (n - 256 * quad)] = acc[mb][j][v];
          } else {
            // y holds the shared down projection and the residual already
            const float ic = inv_pow2(a.xsc[t]);
            ((float*)a.out)[orow + n] += acc[mb][j][v] * ic * ic;
          }
        }
      }
    }
}

// Per group g, its tokens in ascending order (those with an assignment
// labelled g), from the per-chunk group masks of the permutation: one block
// per group, 1024 chunks of 64 tokens per pass; a block scan of the chunks'
// popcounts gives each chunk's first position, then wave w writes the tokens
// of chunks w, w + 16, ... (lane l: token 64 c + l).
__device__ __forceinline__ void group_list_block(const unsigned long long* gmask, int nchunk, int G,
                                                 int gcap, int* gl_tok, int* gl_cnt, int g) {
  __shared__ unsigned long long ms[1024];
  __shared__ int base[1024];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int run = 0;
  for (int c0 = 0; c0 < nchunk; c0 += 1024) {
    const int c = c0 + tid;
    const unsigned long long m = c < nchunk ? gmask[(size_t)c * G + g] : 0ull;
    const int n = __popcll(m);
    int v = n;                                        // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane == 63) wsum[w] = v;
    ms[tid] = m;
    __syncthreads();
    int off = run, tot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < w) off += wsum[i];
      tot += wsum[i];
    }
    base[tid] = off + v - n;
    __syncthreads();
    for (int cc = w; cc < 1024 && c0 + cc < nchunk; cc += 16) {
      const unsigned long long mm = ms[cc];
      if ((mm >> lane) & 1ull)
        gl_tok[(size_t)g * gcap + base[cc] + __popcll(mm & ((1ull << lane) - 1ull))] = (c0 + cc) * 64 + lane;
    }
    run += tot;
    __syncthreads();
  }
  if (tid == 0) gl_cnt[g] = run;
}

template <int WF, int EPI>
int launch_dense(const Dense& a, hipStream_t st) {
  const unsigned nblk = (unsigned)(EPI == kEpiY || EPI == kEpiLogits ? a.nfull + a.nrem * a.nsplit
                                                                     : a.mtiles * a.nquads);
  if (nblk == 0) return 0;
  if constexpr (WF == kF16 && EPI == kEpiF16)
    if (a.A.kmat % kWgCols == 0 && a.A.ps == 0 && a.W.nmat == 1) {
      const unsigned n16 = (unsigned)(((a.T + kWgT - 1) / kWgT) * ((a.ntiles + 3) / 4));
      hipLaunchKernelGGL((k_dense16<EPI, false>), dim3(n16), dim3(256), 0, st, a);
      LMOE_HIP(hipGetLastError());
      return 0;
    }
  if constexpr (WF == kF16 || WF == kBF16)
    if (a.W.g.k % 64 == 0 && (EPI != kEpiY || a.W2.g.k % 64 == 0)) {
      hipLaunchKernelGGL((k_dense_dma<WF, EPI>), dim3(nblk), dim3(NTH), 0, st, a);
      LMOE_HIP(hipGetLastError());
      return 0;
    }
  hipLaunchKernelGGL((k_dense<WF, EPI>), dim3(nblk), dim3(NTH), 0, st, a);
  LMOE_HIP(hipGetLastError());
  return 0;
}

}  // namespace

size_t prefill_max_pieces(int T, int K, int E) {
  const size_t n = (size_t)T * K;
  return n / BM + 1 + std::min<size_t>(n, (size_t)E);
}
int prefill_chunks(int T) { return (T + CHUNK_T - 1) / CHUNK_T; }
size_t prefill_piece_bytes() { return sizeof(Piece); }

int prefill_router_wmax(lmoe_t* h, hipStream_t st) {
  hipLaunchKernelGGL(k_router_wmax, dim3(1), dim3(1024), 0, st, (const uint16_t*)h->router_rm,
                     h->d.n_experts, h->d.hidden, h->pw.wmax);
  LMOE_HIP(hipGetLastError());
  return 0;
}

int prefill_dequant_du(lmoe_t* h, hipStream_t st) {
  const int fmt = h->d.du_bits == 8 ? kQ8 : kQ4, G = h->d.n_groups;
  for (int which = 0; which < 2; ++which) {
    const Geom& gs = which == 0 ? h->g_d : h->g_u;
    const Geom& gd = which == 0 ? h->g_d16 : h->g_u16;
    const size_t n = (size_t)gd.tiles * gd.tile_slots * 64 * G;
    hipLaunchKernelGGL(k_dequant_du, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const uint8_t*)(which == 0 ? h->dmat : h->umat), gs, fmt,
                       which == 0 ? h->dmat16 : h->umat16, gd, G);
    LMOE_HIP(hipGetLastError());
  }
  return 0;
}

int forward_prefill(lmoe_t* h, const float* x, int T, float* y, bool norm, float eps,
                    hipStream_t st) {
  const lmoe_dims& d = h->d;
  const PrefillWs& p = h->pw;
  const int H = d.hidden, L = d.latent, E = d.n_experts, K = d.top_k, G = d.n_groups,
            F = d.expert_ffn, Fs = d.shared_ffn;
  const int Epad = h->g_router_m.tiles * 64;
  const int mtiles = (T + BM - 1) / BM;
  const bool ev = h->phase_events.size() == (size_t)kPrefillPhases + 1;
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[0], st));

  // staging
  {
    Prep a{x, T, H, norm ? 1 : 0, eps, (_Float16*)p.xh, (__bf16*)p.xb, p.xnorm, p.r, p.r64, p.xsc};
    hipLaunchKernelGGL(k_prep, dim3(T), dim3((H / 8 + 63) / 64 * 64), 0, st, a);
    LMOE_HIP(hipGetLastError());
  }
  // D and the shared gate/up need only the staged rows: D runs on the aux
  // stream while the routing chain and then the shared gate/up run on the
  // caller's (D alone is longer than both). When phases are timed everything
  // runs on the caller's stream in phase order, so that each phase is
  // measured alone.
  // D over the routed (token, group) pairs (the handle's prefill-D option):
  // the gathered GEMM over the per-group token lists the permutation wrote
  const bool routed = h->prefill_d_routed && (size_t)T * H * 2 < (1ull << 31);
  auto routed_d = [&](hipStream_t sd) -> int {
    Dense a{};
    a.W = WMat{h->dmat16, h->g_d16, 0, 1};
    a.A = AMat{p.xh, (size_t)H, 0, H};
    a.T = T; a.ntiles = h->g_d16.tiles;
    a.out = p.xl; a.ostride = (size_t)G * L;
    a.gl_tok = p.gl_tok; a.gl_cnt = p.gl_cnt; a.G = G; a.gcap = p.tmax; a.gL = L;
    // at most sum_g ceil(cnt_g / 256) <= T min(K, G) / 256 + G tiles
    const size_t nt = (size_t)T * std::min(K, G) / kWgT + G;
    const size_t nb = nt * ((a.ntiles + 3) / 4);
    hipLaunchKernelGGL((k_dense16<kEpiF16, true>), dim3((unsigned)nb), dim3(256), 0, sd, a);
    LMOE_HIP(hipGetLastError());
    if (ev) LMOE_HIP(hipEventRecord(h->phase_events[3], sd));
    return 0;
  };
  // the shared down projection straight into y, with the token's range
  // unscaling and the residual: y = c^-2 (Sd h) (+ x); U is added later. It
  // follows the shared gate/up on that stream, unless phases are timed or y
  // is x (the block forward in place: the routing still reads x), then it
  // opens the U phase.
  const bool early_sd = !ev && y != x;
  auto shared_down = [&](hipStream_t sd) -> int {
    Dense a{};
    a.W = WMat{h->sdn, h->g_sdn, 0, 1};
    a.A = AMat{p.hsb, (size_t)2 * Fs, Fs, Fs};
    a.T = T; a.mtiles = mtiles; a.ntiles = h->g_sdn.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW;
    a.out = y; a.ostride = H; a.nvalid = H; a.res = norm ? x : nullptr; a.xsc = p.xsc;
    a.nsplit = 1; a.nfull = mtiles * a.nquads; a.nrem = 0;
    return launch_dense<kBF16, kEpiY>(a, sd);
  };
  auto dense_front = [&](hipStream_t sd, bool d_part, bool s_part) -> int {
    if (d_part) {
      Dense a{};
      a.W = WMat{h->dmat16, h->g_d16, 0, 1};
      a.A = AMat{p.xh, (size_t)H, 0, H};
      a.T = T; a.mtiles = mtiles; a.ntiles = G * h->g_d16.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW;
      a.out = p.xl; a.ostride = (size_t)G * L; a.nvalid = G * L;
      if (int rc = launch_dense<kF16, kEpiF16>(a, sd)) return rc;
      if (ev) LMOE_HIP(hipEventRecord(h->phase_events[3], sd));
    }
    if (s_part) {
      Dense a{};
      a.W = WMat{h->sgu, h->g_sgu, 0, 1};
      a.A = AMat{p.xb, (size_t)2 * H, H, H};
      a.T = T; a.mtiles = mtiles; a.ntiles = h->g_sgu.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW;
      a.out = p.hsb; a.ostride = (size_t)2 * Fs; a.nvalid = Fs;
      a.xsc = p.xsc;
      if (int rc = launch_dense<kBF16, kEpiSwigluB2>(a, sd)) return rc;
      if (ev) LMOE_HIP(hipEventRecord(h->phase_events[4], sd));
      else if (early_sd)
        if (int rc = shared_down(sd)) return rc;
    }
    return 0;
  };
  if (!ev) {
    // the second stream takes D over all groups, or (routed D, which waits
    // for the routing) the shared gate/up
    LMOE_HIP(hipEventRecord(h->ev_fork, st));
    LMOE_HIP(hipStreamWaitEvent(h->aux, h->ev_fork, 0));
    if (int rc = dense_front(h->aux, !routed, routed)) return rc;
    LMOE_HIP(hipEventRecord(h->ev_join, h->aux));
  }
  // router logits
  int rsplit = 1;
  {
    Dense a{};
    a.W = WMat{h->router_m, h->g_router_m, 0, 1};
    a.A = AMat{p.xb, (size_t)2 * H, H, H};
    a.T = T; a.mtiles = mtiles; a.ntiles = h->g_router_m.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW;
    a.ostride = Epad; a.nvalid = E;
    // split k so the launch fills the chip; the partial logits go to the
    // expert outputs' buffer, unused until the expert GEMMs
    const int nblk0 = mtiles * a.nquads;
    const size_t cap = (size_t)p.tmax * K * L / ((size_t)T * Epad);
    rsplit = (int)std::max<size_t>(1, std::min<size_t>({(size_t)8, cap, (size_t)std::max(1, h->ncu / nblk0)}));
    a.nsplit = rsplit;
    a.nfull = rsplit == 1 ? nblk0 : 0;
    a.nrem = rsplit == 1 ? 0 : nblk0;
    a.out = rsplit == 1 ? p.logits : p.o;
    if (int rc = launch_dense<kBF16, kEpiLogits>(a, st)) return rc;
  }
  // selection
  {
    Select a{};
    a.logits = rsplit == 1 ? p.logits : p.o; a.nsplit = rsplit;
    a.Epad = Epad; a.T = T; a.E = E; a.H = H; a.K = K;
    a.bias = h->bias; a.x = x; a.r = p.r64; a.xnorm = p.xnorm; a.wmax = p.wmax;
    a.wr = (const uint16_t*)h->router_rm;
    // |fp32 logit - exact| <= beta: 2H bf16 x bf16 products, each exact,
    // summed in fp32 in any order (each addition within 2 ulp, allowing
    // truncation): 2 * (2H + 1) * 2^-24 * sum |x_i w_i|; the two-part split
    // of the staged row leaves 2^-16 |x_i|, and the staged row is x * r
    // rounded (2^-24); sum |x_i w_i| <= |x|_2 |w|_2. Margin 2%.
    a.cbeta = 1.02 * (2.0 * (2.0 * H + 1.0) * ldexp(1.0, -24) + ldexp(1.0, -15));
    a.idx = p.idx; a.w = p.w;
    const dim3 g((T + 3) / 4), b(256);
    const int nj = (H + 511) / 512;
    if (E <= 512) {
      if (nj <= 4) hipLaunchKernelGGL((k_select<4, 8>), g, b, 0, st, a);
      else if (nj == 5) hipLaunchKernelGGL((k_select<5, 8>), g, b, 0, st, a);
      else hipLaunchKernelGGL((k_select<8, 8>), g, b, 0, st, a);
    } else {
      if (nj <= 4) hipLaunchKernelGGL((k_select<4, 16>), g, b, 0, st, a);
      else if (nj == 5) hipLaunchKernelGGL((k_select<5, 16>), g, b, 0, st, a);
      else hipLaunchKernelGGL((k_select<8, 16>), g, b, 0, st, a);
    }
    LMOE_HIP(hipGetLastError());
  }
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[1], st));
  // permutation
  {
    Perm a{};
    a.idx = p.idx; a.T = T; a.K = K; a.E = E; a.G = G; a.nchunk = prefill_chunks(T);
    a.cmask = p.cmask; a.gmask = p.gmask; a.ccnt = p.ccnt; a.cbase = p.cbase; a.eorder = p.eorder;
    a.labels = h->labels; a.seg_start = p.seg_start; a.expert_count = p.expert_count;
    a.group_off = p.group_off; a.pieces = (Piece*)p.pieces; a.npieces = p.npieces;
    a.perm = p.perm; a.inv = p.inv; a.xsc = p.xsc; a.psc = p.psc;
    a.gl_tok = p.gl_tok; a.gl_cnt = p.gl_cnt; a.gcap = p.tmax;
    hipLaunchKernelGGL(k_perm_mask, dim3(a.nchunk), dim3(256), 0, st, a);
    LMOE_HIP(hipGetLastError());
    // the group lists' blocks only when the routed D reads them
    hipLaunchKernelGGL(k_perm_scan, dim3(1 + (routed ? G : 0)), dim3(kMaxE), 0, st, a);
    LMOE_HIP(hipGetLastError());
    hipLaunchKernelGGL(k_perm_scatter, dim3((T * K + 255) / 256), dim3(256), 0, st, a);
    LMOE_HIP(hipGetLastError());
  }
  if (ev) {
    LMOE_HIP(hipEventRecord(h->phase_events[2], st));
    if (routed) {
      if (int rc = routed_d(st)) return rc;
    }
    if (int rc = dense_front(st, !routed, true)) return rc;
  } else {
    if (routed) {
      if (int rc = routed_d(st)) return rc;
    } else if (int rc = dense_front(st, false, true)) {
      return rc;
    }
    LMOE_HIP(hipStreamWaitEvent(st, h->ev_join, 0));
  }
  // experts
  const unsigned maxp = (unsigned)prefill_max_pieces(T, K, E);
  {
    Grouped a{};
    a.experts = h->experts; a.estride = h->expert_stride; a.woff = 0; a.ts_off = h->ts_off;
    a.g = h->g_gu; a.A = AMat{p.xl, (size_t)L, 0, L};
    a.pieces = (const Piece*)p.pieces; a.npieces = p.npieces;
    a.ntiles = h->g_gu.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW; a.G = G; a.F = F;
    a.perm = p.perm; a.topk_w = p.w; a.psc = p.psc; a.labels = h->labels; a.K = K;
    a.out = p.h; a.ostride = F;
    if (int rc = launch_grouped<kGateUp>(a, maxp, E, st)) return rc;
  }
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[5], st));
  {
    Grouped a{};
    a.experts = h->experts; a.estride = h->expert_stride; a.woff = h->g_gu.bytes();
    a.ts_off = h->ts_off; a.g = h->g_dn; a.A = AMat{p.h, (size_t)F, 0, F};
    a.pieces = (const Piece*)p.pieces; a.npieces = p.npieces;
    a.ntiles = h->g_dn.tiles; a.nquads = (a.ntiles + NTW - 1) / NTW; a.G = G; a.F = F;
    a.perm = p.perm; a.topk_w = p.w; a.psc = p.psc; a.labels = h->labels; a.K = K;
    a.out = p.o; a.ostride = L;
    if (int rc = launch_grouped<kDown>(a, maxp, E, st)) return rc;
  }
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[6], st));
  // combine
  {
    Combine a{p.idx, p.inv, h->labels, (const _Float16*)p.o, (_Float16*)p.s, K, G, L};
    hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, st, a);
    LMOE_HIP(hipGetLastError());
  }
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[7], st));
  // U over the concatenated groups on k_dense16, split along k; the splits'
  // partial sums (in the dead expert-output buffer) are added onto y, which
  // holds the shared down projection and the residual already
  {
    if (!early_sd)
      if (int rc = shared_down(st)) return rc;
    Dense a{};
    a.W = WMat{h->umat16, h->g_u16, h->g_u16.bytes(), G};
    a.A = AMat{p.s, (size_t)G * L, 0, L};
    a.T = T; a.mtiles = mtiles; a.ntiles = h->g_u16.tiles; a.nquads = (a.ntiles + 3) / 4;
    a.out = y; a.ostride = H; a.nvalid = H; a.xsc = p.xsc;
    // one 256 x 256 workgroup per CU at a time: the split minimising rounds
    // of the chip per split plus a small charge per split for writing and
    // re-reading its partial sums (as many as the buffer holds)
    const int nt16 = ((T + kWgT - 1) / kWgT) * a.nquads;
    a.nfull = 0;
    a.nrem = mtiles * a.nquads;
    const size_t cap = (size_t)p.tmax * K * L / ((size_t)a.nrem * BM * 256);
    const int smax = (int)std::max<size_t>(1, std::min<size_t>(8, cap));
    int ns = 1;
    double best = 1e30;
    for (int c = 1; c <= smax; ++c) {
      const double rounds = (double)((nt16 * c + h->ncu - 1) / h->ncu);
      const double cost = rounds / c + 0.05 * (c > 1 ? c : 0);
      if (cost < best - 1e-9) { best = cost; ns = c; }
    }
    a.nsplit = ns;
    a.part = p.o;
    hipLaunchKernelGGL((k_dense16<kEpiY, false>), dim3((unsigned)(nt16 * ns)), dim3(256), 0, st, a);
    LMOE_HIP(hipGetLastError());
    if (ns > 1) {
      const dim3 g(a.nrem * (BM / 4)), b(256);
      switch (ns) {
        case 2: hipLaunchKernelGGL(k_ytiles<2>, g, b, 0, st, a, (const float*)y); break;
        case 3: hipLaunchKernelGGL(k_ytiles<3>, g, b, 0, st, a, (const float*)y); break;
        case 4: hipLaunchKernelGGL(k_ytiles<4>, g, b, 0, st, a, (const float*)y); break;
        case 5: hipLaunchKernelGGL(k_ytiles<5>, g, b, 0, st, a, (const float*)y); break;
        case 6: hipLaunchKernelGGL(k_ytiles<6>, g, b, 0, st, a, (const float*)y); break;
        case 7: hipLaunchKernelGGL(k_ytiles<7>, g, b, 0, st, a, (const float*)y); break;
        default: hipLaunchKernelGGL(k_ytiles<8>, g, b, 0, st, a, (const float*)y); break;
      }
      LMOE_HIP(hipGetLastError());
    }
  }
  if (ev) LMOE_HIP(hipEventRecord(h->phase_events[8], st));
  return 0;
}

int prefill_debug_latent(lmoe_t* h, int T, float* dst, hipStream_t st) {
  const size_t n = (size_t)T * h->d.n_groups * h->d.latent;
  hipLaunchKernelGGL(k_f16_to_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const _Float16*)h->pw.xl, n, (size_t)h->d.n_groups * h->d.latent, h->pw.xsc, dst);
  LMOE_HIP(hipGetLastError());
  return 0;
}

}  // namespace lm
