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

// ---------------------------------------------------------------------------
// Device weight layout: the "tiled stream".
//
// A weight matrix [rows][k] is cut into tiles of 64 rows. One lane of a
// 64-wide wavefront owns one row of a tile, so a dot product never needs a
// cross-lane reduction. Along k, a tile is a sequence of 1 KiB slots; slot j
// holds 16 bytes of every lane's row, lane-major, so one global_load_dwordx4
// per lane reads one slot as a single coalesced 1 KiB request. Columns are
// grouped in super-steps of 256: the code slots of a super-step come first,
// then (for scaled formats) one slot holding that super-step's scales.
//
//   format  columns per code slot  scale slot (16 B per lane)
//   Q8      16 (int8)              8 fp16 scales, one per 32 columns
//   Q4      32 (4-bit two's compl) 8 fp16 scales, one per 32 columns
//   FP4     32 (E2M1)              16 E4M3 scales, one per 16 columns
//   BF16     8                     none
//
// A super-step is the unit of work of one wavefront in the GEMV kernels.
enum Fmt : int { kQ8 = 0, kQ4 = 1, kFP4 = 2, kBF16 = 3 };
constexpr int kSSCols = 256;
constexpr int kSlot = 1024;
constexpr int kMaxDecodeT = 8;     // tokens the GEMV (decode) path takes per forward
constexpr int kMaxWaves = 16;
constexpr int kDecodePhases = 4;

__host__ __device__ constexpr int cols_per_slot(int f) {
  return f == kQ8 ? 16 : (f == kBF16 ? 8 : 32);
}
__host__ __device__ constexpr int scale_slots(int f) { return f == kBF16 ? 0 : 1; }

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
  g.full = kSSCols / cols_per_slot(fmt) + scale_slots(fmt);
  int last = k - (g.nss - 1) * kSSCols;
  g.tile_slots = (g.nss - 1) * g.full + last / cols_per_slot(fmt) + scale_slots(fmt);
  return g;
}

// ---------------------------------------------------------------------------
// Workspace of one handle (device pointers). Decode buffers are sized for
// min(max_tokens, kMaxDecodeT) tokens.
struct Workspace {
  double* part64 = nullptr;      // [nch][T][Epad] router partial logits
  double* logits = nullptr;      // [T][E]
  int* topk_idx = nullptr;       // [T][K]
  float* topk_w = nullptr;       // [T][K]
  int* perm = nullptr;           // [T*K]
  int* inv = nullptr;            // [T*K] sorted position of assignment a
  int* slot_expert = nullptr;    // [T*K] distinct experts in (label, expert) order
  int* slot_start = nullptr;     // [T*K]
  int* slot_count = nullptr;     // [T*K]
  int* n_slots = nullptr;        // [1]
  int* gslot_off = nullptr;      // [G+1] first slot of each group
  int* group_off = nullptr;      // [G+1]
  int* expert_count = nullptr;   // [E]
  float* rms = nullptr;          // [T] 1/rms of the input rows (block forward)
  float* xl = nullptr;           // [T][G][ell]
  float* hs = nullptr;           // [T][Fs] shared-expert hidden
  float* hbuf = nullptr;         // [T*K][F] expert hidden, sorted position order
  float* obuf = nullptr;         // [T*K][ell] weighted expert outputs
  float* s = nullptr;            // [T][G][ell] per-group sums
  float* ypart = nullptr;        // [G+1][T][H]
  unsigned* ctr_router = nullptr;  // [1]
  unsigned* ctr_s = nullptr;       // [G][ell/64]
  unsigned* ctr_y = nullptr;       // [H/64]
  int nch = 0;                   // router column chunks
  int tmax = 0;                  // tokens the decode buffers hold
};

}  // namespace lm

struct lmoe {
  lmoe_dims d{};
  int device = 0;
  bool loaded = false;
  lm::Geom g_router, g_d, g_u, g_gu, g_dn, g_sgu, g_sdn;
  size_t expert_stride = 0;   // bytes per expert in device memory
  size_t ts_off = 0;          // offset of the three fp32 tensor scales
  uint8_t* router = nullptr;  // tiled bf16 [Epad][H]
  float* bias = nullptr;      // [E] (zeros without a bias)
  uint8_t* dmat = nullptr;    // G tiled D_g
  uint8_t* umat = nullptr;    // G tiled U_g
  uint8_t* experts = nullptr; // E experts: tiled gate/up pairs, tiled down, ts
  uint8_t* sgu = nullptr;     // tiled shared gate/up pairs
  uint8_t* sdn = nullptr;     // tiled shared down
  uint8_t* labels = nullptr;  // [E] device copy
  std::vector<uint8_t> labels_host;
  lm::Workspace ws;
  std::vector<void*> allocations;
  std::vector<hipEvent_t> phase_events;   // empty: no phase timing
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
int forward_decode(lmoe_t* h, const float* x, int T, float* y, bool norm, hipStream_t stream);
int rms_rows(lmoe_t* h, const float* x, int T, float eps, hipStream_t stream);

// api.hip
void set_error(const std::string& msg);
int hip_fail(hipError_t e, const char* what);

}  // namespace lm

#define LMOE_HIP(call)                                         \
  do {                                                         \
    hipError_t e_ = (call);                                    \
    if (e_ != hipSuccess) return lm::hip_fail(e_, #call);    \
  } while (0)
