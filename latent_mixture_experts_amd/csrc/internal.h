// Internal declarations of liblmoe: the device weight layout, the handle and
// the launchers. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "lmoe.h"

namespace lm {

// Raw buffer resource over [p, p + bytes): wave-uniform base in SGPRs, so a
// lane addresses it with one 32-bit offset register; loads past the end
// return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int kAuxNT = 2;   // cache policy: non-temporal
template <int AUX = 0>
__device__ __forceinline__ uint4 ldb(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

// ---------------------------------------------------------------------------
// Device weight layout: the "tiled stream".
//
// A weight matrix [rows][k] is cut into tiles of 64 rows (four row groups of
// 16). Along k, a tile is a sequence of 1 KiB slots, each read by one
// global_load_dwordx4 per lane as a single coalesced request. Columns are
// grouped in super-steps of 256 (the unit of work of one wavefront): a
// super-step holds its code slots, then, for scaled formats, one scale slot.
//
// Code slot j of a super-step holds chunk j/4 of row group j%4. Lane l owns
// row l%16 of the group and, in every 32-column block of the chunk, the 8
// columns 8*(l/16)..8*(l/16)+7: exactly the B operand of an MFMA
// 16x16x32 instruction for that row.
//
//   format  chunk   lane's 16 bytes                       scale slot (lane-chunk 16*rg + r)
//   Q8      64      2 blocks x 8 int8, held as q + 128     8 fp16 scales of row r (per 32 cols)
//   Q4      128     4 blocks x 8 nibbles, held as q + 8    8 fp16 scales of row r (per 32 cols)
//                   (element i in the low nibble of byte i, element i+4 in its high nibble)
//   FP4     128     4 blocks x 8 E2M1 codes (pairs per byte, low nibble first)
//                                                         16 E4M3 scales of row r (per 16 cols)
//   BF16    32      8 bf16                                none
//   IQ4     128     as Q4, the nibbles holding IQ4_NL table indices
//                                                         8 fp16 scales of row r (per 32 cols)
//   Q3K     256     (K a multiple of 256: one super-step is one Q3_K super-block
//                   per row; six code slots) slots 0..3, row group j: lane
//                   (r, k-group q) holds the 8 low-bit bytes 16 b + 8 (q % 2) + 0..7
//                   of half 0, then of half 1 (b = q / 2: the 16-column run of
//                   its k-group); slots 4, 5: row groups 2s and 2s + 1, each the
//                   lane's 8 high-bit-mask bytes 16 b + 8 (q % 2) + 0..7
//                                                         row r's 12 scale bytes and fp16 d
//
// The router keeps a plainer layout (BF16R) for its fp64 dot products: lane
// l of a slot holds 8 consecutive bf16 columns of row l of the tile. F16 is
// the BF16 layout holding fp16 values: the prefill path keeps D and U
// dequantized to fp16(q * d) in it.
enum Fmt : int { kQ8 = 0, kQ4 = 1, kFP4 = 2, kBF16 = 3, kBF16R = 4, kF16 = 5, kIQ4 = 6, kQ3K = 7 };
constexpr int kSSCols = 256;
constexpr int kSlot = 1024;
constexpr int kMaxDecodeT = 8;     // tokens the GEMV (decode) path takes per forward
constexpr int kMaxWaves = 16;
constexpr int kDecodePhases = 4;
constexpr int kPrefillPhases = 8;
constexpr int kMaxTokens = 1 << 20;   // largest max_tokens a handle accepts
constexpr int kRouterChunks = 4;  // router column chunks: H / (64 * H/256)

__host__ __device__ constexpr int chunk_cols(int f) {      // columns of one chunk
  return f == kQ8 ? 64 : ((f == kBF16 || f == kF16) ? 32 : (f == kBF16R ? 8 : (f == kQ3K ? 256 : 128)));
}
__host__ __device__ constexpr int scale_slots(int f) {
  return (f == kBF16 || f == kBF16R || f == kF16) ? 0 : 1;
}
// Code slots of a super-step of `cols` columns: four row groups per chunk
// (one slot per chunk for the router layout); a partial last chunk is
// padded with zero codes.
__host__ __device__ constexpr int ss_code_slots(int f, int cols) {
  return f == kBF16R ? cols / 8 : (f == kQ3K ? 6 : 4 * ((cols + chunk_cols(f) - 1) / chunk_cols(f)));
}

struct Geom {
  int rows = 0;        // real rows
  int tiles = 0;       // ceil(rows / 64)
  int k = 0;           // columns
  int nss = 0;         // super-steps
  int full = 0;        // slots of a full super-step
  int tile_slots = 0;  // slots of one tile
  __host__ __device__ size_t bytes() const { return (size_t)tiles * tile_slots * kSlot; }
};

inline Geom make_geom(int fmt, int rows, int k) {
  Geom g;
  g.rows = rows;
  g.tiles = (rows + 63) / 64;
  g.k = k;
  g.nss = (k + kSSCols - 1) / kSSCols;
  g.full = ss_code_slots(fmt, kSSCols) + scale_slots(fmt);
  int last = k - (g.nss - 1) * kSSCols;
  g.tile_slots = (g.nss - 1) * g.full + ss_code_slots(fmt, last) + scale_slots(fmt);
  return g;
}

// ---------------------------------------------------------------------------
// Workspace of one handle (device pointers). Decode buffers are sized for
// min(max_tokens, kMaxDecodeT) tokens.
struct Workspace {
  double* part64 = nullptr;      // [nch][T][Epad] router partial logits
  int* topk_idx = nullptr;       // [T][K]
  float* topk_w = nullptr;       // [T][K]
  int* perm = nullptr;           // [T*K]
  int* tg_cnt = nullptr;         // [T][G] assignments of token t in group g
  int* tg_pos = nullptr;         // [T][G][K] their sorted positions, ascending k
  int* slot_expert = nullptr;    // [T*K] distinct experts in (label, expert) order
  int* slot_start = nullptr;     // [T*K]
  int* slot_count = nullptr;     // [T*K]
  int* slot_xrow = nullptr;      // [T*K][8] xl rows t * G + g of each slot's tokens (padded)
  int* n_slots = nullptr;        // [1]
  int* gslot_off = nullptr;      // [G+1] first slot of each group
  int* group_off = nullptr;      // [G+1]
  int* expert_count = nullptr;   // [E]
  float* rms = nullptr;          // [T] 1/rms of the input rows (block forward)
  double* rms64 = nullptr;       // [T] the same in fp64, for the router logits
  double* sqp = nullptr;         // [nch][T] sums of x^2 over the router's column chunks
  float* xl = nullptr;           // [T][G][ell]
  float* hs = nullptr;           // [T][Fs] shared-expert hidden
  float* hsp = nullptr;          // [H/256][T][2 Fs] shared gate/up partials per super-step
  float* hbuf = nullptr;         // [T*K][F] expert hidden, sorted position order
  float* obuf = nullptr;         // [T*K][ell] weighted expert outputs, sorted position order
  float* ypart = nullptr;        // [2G + shared-down blocks][T][H] phase-4 partials
  unsigned* ctr_router = nullptr;  // [1]
  unsigned* ctr_y = nullptr;       // [H/64]
  int nch = 0;                   // router column chunks
  int tmax = 0;                  // tokens the decode buffers hold
};

// Workspace of the prefill path (T > kMaxDecodeT), sized for max_tokens.
struct PrefillWs {
  uint16_t* xh = nullptr;          // [T][H] fp16 staged rows (D input)
  uint16_t* xb = nullptr;          // [T][2][H] bf16 parts (router, shared gate/up)
  double* xnorm = nullptr;         // [T] 2-norm of the staged rows
  float* r = nullptr;              // [T] row scale (1/rms in the block forward, else 1)
  double* r64 = nullptr;           // [T] the same in fp64 (the fp64 rescoring of the logits)
  float* xsc = nullptr;            // [T] power-of-two range scale of the fp16 activations
  float* psc = nullptr;            // [T*K] the same per sorted assignment
  float* logits = nullptr;         // [T][Epad] fp32 router logits
  int* idx = nullptr;              // [T][K]
  float* w = nullptr;              // [T][K]
  unsigned long long* cmask = nullptr;  // [nchunk][E] tokens of a 64-token chunk per expert
  unsigned long long* gmask = nullptr;  // [nchunk][G] the same per group
  int* ccnt = nullptr;             // [nchunk][E]
  int* cbase = nullptr;            // [nchunk][E]
  int* eorder = nullptr;           // [E] experts in (label, expert) order
  int* seg_start = nullptr;        // [E]
  int* expert_count = nullptr;     // [E]
  int* group_off = nullptr;        // [G+1]
  void* pieces = nullptr;          // [max pieces] grouped-GEMM work list
  int* npieces = nullptr;          // [3] pieces, first of at most 64 tokens, of at most 32
  int* perm = nullptr;             // [T*K]
  int* inv = nullptr;              // [T*K] assignment -> sorted position
  uint16_t* xl = nullptr;          // [T][G][ell] fp16
  uint16_t* hsb = nullptr;         // [T][2][Fs] shared hidden, bf16 parts
  uint16_t* h = nullptr;           // [T*K][F] fp16 expert hidden, sorted order
  float* o = nullptr;              // [T*K][ell] weighted expert outputs (held as fp16, in
                                   // the first half); the router and U k-splits put
                                   // their fp32 partial sums here while it is unused
  uint16_t* s = nullptr;           // [T][G][ell] fp16 per-group sums
  int* gl_tok = nullptr;           // [G][T] each group's routed tokens (routed-pairs D)
  int* gl_cnt = nullptr;           // [G]
  double* wmax = nullptr;          // [1] max_e |Wr_e|_2
  int tmax = 0;                    // tokens the buffers hold (0: no prefill path)
};

}  // namespace lm

struct lmoe {
  lmoe_dims d{};
  int device = 0;
  int ncu = 1;                // compute units of the device
  bool loaded = false;
  bool prefill_d_routed = true;   // prefill D over the routed (t, g) pairs only (else all groups)
  lm::Geom g_router, g_d, g_u, g_gu, g_dn, g_sgu, g_sdn;
  lm::Geom g_router_m;        // router in the MFMA layout (prefill)
  lm::Geom g_d16, g_u16;      // D_g, U_g dequantized to fp16 (prefill)
  size_t expert_stride = 0;   // bytes per expert in device memory
  size_t ts_off = 0;          // offset of the three fp32 tensor scales
  uint8_t* router = nullptr;  // tiled bf16 [Epad][H]
  uint8_t* router_m = nullptr;  // prefill: router tiled for MFMA
  uint8_t* dmat16 = nullptr;    // prefill: G tiled fp16 D_g
  uint8_t* umat16 = nullptr;    // prefill: G tiled fp16 U_g
  uint16_t* router_rm = nullptr;  // prefill: router bf16 [E][H] row-major
  float* bias = nullptr;      // [E] (zeros without a bias)
  uint8_t* dmat = nullptr;    // G tiled D_g
  uint8_t* umat = nullptr;    // G tiled U_g
  uint8_t* experts = nullptr; // E experts: tiled gate/up pairs, tiled down, ts
  uint8_t* sgu = nullptr;     // tiled shared gate/up pairs
  uint8_t* sdn = nullptr;     // tiled shared down
  uint8_t* labels = nullptr;  // [E] device copy
  std::vector<uint8_t> labels_host;
  lm::Workspace ws;
  lm::PrefillWs pw;
  // prefill: a second stream (default priority) on which D and the shared
  // gate/up run while the router, top-K and permutation run on the caller's
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  std::vector<void*> allocations;
  std::vector<hipEvent_t> phase_events;   // empty: no phase timing
  int last_decode_T = 0;                  // T of the last plain decode forward (0: none)
  float rms_eps = 0.f;                    // eps of the block forward being launched
  // blocks of a kernel resident at once, by (kernel, threads, LDS bytes)
  struct Resident { const void* kernel; int threads; size_t lds; int blocks; };
  std::vector<Resident> resident;
};

namespace lm {

// layout.hip
int load_weights_impl(lmoe_t* h, const lmoe_weights* w, hipStream_t stream);
int pack_bf16_impl(const float* src, size_t n, uint16_t* dst, hipStream_t stream);
int pack_blocks_impl(const float* src, int rows, int cols, int bits, uint8_t* dst,
                     hipStream_t stream);
int pack_experts_impl(const float* gate, const float* up, const float* down, int n, int ell,
                      int f, uint8_t* dst, hipStream_t stream);

// decode.hip
// only: 0 runs the whole forward, 1..4 that phase alone
// ws: the workspace to run on (nullptr: the handle's)
int forward_decode(lmoe_t* h, const float* x, int T, float* y, bool norm, hipStream_t stream,
                   int only = 0, const Workspace* ws = nullptr);
// Largest dynamic LDS a decode kernel needs for T tokens (a handle whose
// decode path would need more than a CU has is refused at create).
size_t decode_lds_bytes(const lmoe_dims& d, int T);

// prefill.hip
int forward_prefill(lmoe_t* h, const float* x, int T, float* y, bool norm, float eps,
                    hipStream_t stream);
size_t prefill_max_pieces(int T, int K, int E);
int prefill_chunks(int T);
size_t prefill_piece_bytes();
int prefill_router_wmax(lmoe_t* h, hipStream_t stream);
int prefill_dequant_du(lmoe_t* h, hipStream_t stream);
int prefill_debug_latent(lmoe_t* h, int T, float* dst, hipStream_t stream);

// api.hip
void set_error(const std::string& msg);
size_t decode_ws_layout(const lmoe_t* h, int T, char* base, Workspace* out);
int hip_fail(hipError_t e, const char* what);

}  // namespace lm

#define LMOE_HIP(call)                                         \
  do {                                                         \
    hipError_t e_ = (call);                                    \
    if (e_ != hipSuccess) return lm::hip_fail(e_, #call);    \
  } while (0)
