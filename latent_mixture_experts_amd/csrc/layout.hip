// Load-time work: re-laying the packed weights into the tiled stream, and
// the device-side packers (fp32 masters -> bf16 / Q8 / Q4 / NVFP4 blobs).
//
// Packed formats are those of "Edge0-145B: a Qwen MoE with its experts
// squeezed, and a 51B table left on the SSD", section "What is 4-bit" (NVFP4
// expert records: FP4 values, an E4M3 scale per 16, a 16-byte tail; Q8_0 /
// Q4_0 D/U with one fp16 scale per 32), read as stated in include/lmoe.h.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <vector>

#include "internal.h"

namespace lm {
namespace {

// ---------------------------------------------------------------------------
// Re-layout into tiled streams.

// Where the rows of one source matrix live in packed form.
struct Src {
  const uint8_t* codes;   // row-major codes in the packed format; Q3K / IQ4: the blocks
  const uint8_t* scales;  // Q8/Q4: fp16 [rows][k/32]; FP4: E4M3 [rows][k/16]; else unused
  int rows;
};

constexpr int kQ3KBlock = 110, kIQ4Block = 18;   // bytes of a Q3_K (256) / IQ4_NL (32) block

// One 16-byte lane chunk of a Q3K super-step (layout in internal.h): slot j
// of super-step ss, lane (r16, qg) of the tile's row group(s).
__device__ void q3k_chunk(const Src& a, const Src& b, int pair, int k, int tile, int ss, int j,
                          int lane, uint8_t (&out)[16]) {
  const int r16 = lane % 16, qg = lane / 16, run = qg >> 1, part = qg & 1;
  const auto block = [&](int rg, int& rows_ok) -> const uint8_t* {
    const Src* s = (pair && rg >= 2) ? &b : &a;
    const int row = pair ? 32 * tile + 16 * (rg & 1) + r16 : 64 * tile + 16 * rg + r16;
    rows_ok = row < s->rows;
    return s->codes + ((size_t)row * (k / 256) + ss) * kQ3KBlock;
  };
  int ok;
  if (j < 4) {                                  // low bits, halves 0 and 1
    const uint8_t* p = block(j, ok);
    if (ok)
      for (int h = 0; h < 2; ++h)
        for (int i = 0; i < 8; ++i) out[8 * h + i] = p[32 + 32 * h + 16 * run + 8 * part + i];
  } else if (j < 6) {                           // high-bit masks of two row groups
    for (int t = 0; t < 2; ++t) {
      const uint8_t* p = block(2 * (j - 4) + t, ok);
      if (ok)
        for (int i = 0; i < 8; ++i) out[8 * t + i] = p[16 * run + 8 * part + i];
    }
  } else {                                      // lane-chunk 16 rg + r: scales and d of that row
    const uint8_t* p = block(lane / 16, ok);
    if (ok)
      for (int i = 0; i < 14; ++i) out[i] = p[96 + i];
  }
}

__device__ inline size_t code_offset(int fmt, int row, int k, int col) {
  size_t e = (size_t)row * k + col;
  return fmt == kQ8 ? e : ((fmt == kBF16 || fmt == kBF16R) ? 2 * e : e / 2);
}

// One thread writes one 16-byte lane chunk of one slot (layouts in
// internal.h). `pair` tiles take rows from two matrices: row groups 0,1 from
// a (rows 32*tile + 16*rg + r), row groups 2,3 from b (same rows), so the
// gate and up rows of the same index meet in one lane.
__global__ void k_tile(int fmt, Src a, Src b, int pair, int k, Geom g, uint8_t* __restrict__ dst) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t total = (size_t)g.tiles * g.tile_slots * 64;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  const int slot = (int)((idx / 64) % g.tile_slots);
  const int tile = (int)(idx / 64 / g.tile_slots);
  const int ss = slot / g.full;
  const int j = slot % g.full;
  const int cols = min(kSSCols, k - ss * kSSCols);
  const int ncs = ss_code_slots(fmt, cols);

  uint8_t out[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = 0;
  if (fmt == kQ3K) {
    q3k_chunk(a, b, pair, k, tile, ss, j, lane, out);
  } else if (fmt == kBF16R) {
    const int row = 64 * tile + lane;
    if (row < a.rows) {
      const uint8_t* p = a.codes + code_offset(fmt, row, k, ss * kSSCols + j * 8);
      for (int i = 0; i < 16; ++i) out[i] = p[i];
    }
  } else {
    // code slot: row group j%4, chunk j/4; scale slot: lane-chunk 16*rg + r
    const bool is_code = j < ncs;
    const int rg = is_code ? (j % 4) : (lane / 16);
    const int r16 = lane % 16;
    const Src* s = (pair && rg >= 2) ? &b : &a;
    const int row = pair ? 32 * tile + 16 * (rg & 1) + r16 : 64 * tile + 16 * rg + r16;
    if (row < s->rows) {
      if (is_code) {
        const int c = j / 4, qg = lane / 16;
        // 8-column pieces past k stay zero codes (k is a multiple of 32)
        if (fmt == kQ8) {
          for (int bb = 0; bb < 2; ++bb) {
            const int col = ss * kSSCols + 64 * c + 32 * bb + 8 * qg;
            if (col >= k) continue;
            const uint8_t* p = s->codes + code_offset(fmt, row, k, col);
            for (int i = 0; i < 8; ++i) out[8 * bb + i] = p[i] ^ 0x80;   // int8 -> q + 128
          }
        } else if (fmt == kBF16) {
          const int col = ss * kSSCols + 32 * c + 8 * qg;
          if (col < k) {
            const uint8_t* p = s->codes + code_offset(fmt, row, k, col);
            for (int i = 0; i < 16; ++i) out[i] = p[i];
          }
        } else {
          for (int bb = 0; bb < 4; ++bb) {
            const int col = ss * kSSCols + 128 * c + 32 * bb + 8 * qg;
            if (col >= k) {
              if (fmt == kQ4)
                for (int i = 0; i < 4; ++i) out[4 * bb + i] = 0x88;         // q = 0
              continue;
            }
            if (fmt == kIQ4) {
              // block col / 32 holds element o < 16 in the low nibble of
              // byte 2 + o, element 16 + o in its high nibble; the device
              // keeps element i low and element i + 4 high in byte i
              const uint8_t* blk = s->codes + ((size_t)row * (k / 32) + col / 32) * kIQ4Block;
              const int o = col % 32;
              uint8_t e[8];
              for (int i = 0; i < 8; ++i) {
                const int oo = o + i;
                e[i] = oo < 16 ? (blk[2 + oo] & 0xF) : (blk[2 + oo - 16] >> 4);
              }
              for (int i = 0; i < 4; ++i) out[4 * bb + i] = (uint8_t)(e[i] | (e[i + 4] << 4));
              continue;
            }
            const uint8_t* p = s->codes + code_offset(fmt, row, k, col);
            if (fmt == kFP4) {
              for (int i = 0; i < 4; ++i) out[4 * bb + i] = p[i];
            } else {
              // packed Q4: byte i = e(2i) | e(2i+1) << 4; device: e(i) | e(i+4) << 4
              uint8_t e[8];
              for (int i = 0; i < 4; ++i) {
                e[2 * i] = p[i] & 0xF;
                e[2 * i + 1] = p[i] >> 4;
              }
              for (int i = 0; i < 4; ++i) out[4 * bb + i] = (uint8_t)(e[i] | (e[i + 4] << 4));
            }
          }
        }
      } else {
        if (fmt == kFP4) {
          const uint8_t* p = s->scales + (size_t)row * (k / 16) + ss * 16;
          for (int i = 0; i < cols / 16; ++i) out[i] = p[i];
        } else if (fmt == kIQ4) {
          const uint8_t* blk = s->codes + ((size_t)row * (k / 32) + ss * 8) * kIQ4Block;
          for (int i = 0; i < cols / 32; ++i) {
            out[2 * i] = blk[i * kIQ4Block];
            out[2 * i + 1] = blk[i * kIQ4Block + 1];
          }
        } else {
          const uint8_t* p = s->scales + ((size_t)row * (k / 32) + ss * 8) * 2;
          for (int i = 0; i < 2 * (cols / 32); ++i) out[i] = p[i];
        }
      }
    }
  }
  uint4 v;
  v.x = out[0] | (out[1] << 8) | (out[2] << 16) | ((uint32_t)out[3] << 24);
  v.y = out[4] | (out[5] << 8) | (out[6] << 16) | ((uint32_t)out[7] << 24);
  v.z = out[8] | (out[9] << 8) | (out[10] << 16) | ((uint32_t)out[11] << 24);
  v.w = out[12] | (out[13] << 8) | (out[14] << 16) | ((uint32_t)out[15] << 24);
  *(uint4*)(dst + ((size_t)tile * g.tile_slots + slot) * kSlot + lane * 16) = v;
}

int launch_tile(int fmt, Src a, Src b, int pair, int k, const Geom& g, uint8_t* dst,
                hipStream_t st) {
  size_t total = (size_t)g.tiles * g.tile_slots * 64;
  unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(k_tile, dim3(blocks), dim3(256), 0, st, fmt, a, b, pair, k, g, dst);
  LMOE_HIP(hipGetLastError());
  return 0;
}

// Expert records: sections of one record (see include/lmoe.h).
struct RecOff {
  size_t gate_c, up_c, down_c, gate_s, up_s, down_s, tail;
};
inline RecOff rec_off(int ell, int f) {
  size_t n = (size_t)ell * f;
  RecOff r;
  r.gate_c = 0;
  r.up_c = n / 2;
  r.down_c = n;
  r.gate_s = 3 * n / 2;
  r.up_s = r.gate_s + n / 16;
  r.down_s = r.up_s + n / 16;
  r.tail = r.down_s + n / 16;
  return r;
}

__global__ void k_copy_ts(const uint8_t* __restrict__ recs, size_t rec_bytes, size_t tail,
                          int n, uint8_t* __restrict__ dst, size_t stride, size_t ts_off) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const uint8_t* p = recs + (size_t)e * rec_bytes + tail;
  float* q = (float*)(dst + (size_t)e * stride + ts_off);
  for (int i = 0; i < 3; ++i) {
    uint32_t v = p[4 * i] | (p[4 * i + 1] << 8) | (p[4 * i + 2] << 16) | ((uint32_t)p[4 * i + 3] << 24);
    q[i] = __uint_as_float(v);
  }
  q[3] = 0.f;
}

// Q3_K records carry no tensor scales: the device record's three are 1.
__global__ void k_unit_ts(int n, uint8_t* __restrict__ dst, size_t stride, size_t ts_off) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float* q = (float*)(dst + (size_t)e * stride + ts_off);
  q[0] = q[1] = q[2] = 1.f;
  q[3] = 0.f;
}

// ---------------------------------------------------------------------------
// Device packers. Rounding to a binary grid with `mb` fraction bits and
// exponent >= emin, ties to even, done in fp64 where every step is exact for
// these formats (the quotients are correctly rounded fp64 values far from
// the few-bit ties unless exactly on them).

__device__ inline double round_grid(double v, int mb, int emin) {
  if (v == 0.0) return 0.0;
  int ex;
  frexp(v, &ex);                 // v = f * 2^ex, f in [0.5, 1)
  int e = max(ex - 1, emin);     // exponent of the leading bit
  double q = rint(ldexp(v, mb - e));
  return ldexp(q, e - mb);
}

__device__ inline uint32_t e4m3_code(double v) {   // v >= 0
  double r = fmin(round_grid(v, 3, -6), 448.0);
  if (r < 0.015625) return (uint32_t)(r * 512.0);
  int ex;
  frexp(r, &ex);
  int e = ex - 1;
  return (uint32_t)(((e + 7) << 3) | (int)((ldexp(r, -e) - 1.0) * 8.0));
}

__device__ inline double e4m3_value(uint32_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  return e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
}

__device__ inline uint32_t e2m1_code(double v) {
  double mag = fmin(round_grid(fabs(v), 1, 0), 6.0);
  uint32_t c;
  if (mag < 1.0) {
    c = (uint32_t)(mag * 2.0);
  } else {
    int ex;
    frexp(mag, &ex);           // mag in [2^(ex-1), 2^ex)
    c = (uint32_t)((ex << 1) | (int)((ldexp(mag, -(ex - 1)) - 1.0) * 2.0));
  }
  if (v < 0 && mag != 0.0) c |= 8;
  return c;
}

__device__ inline uint32_t f16_bits(double v) {    // v >= 0, below 65504
  double r = round_grid(v, 10, -14);
  if (r < 6.103515625e-05) return (uint32_t)(r * 16777216.0);
  int ex;
  frexp(r, &ex);
  int e = ex - 1;
  return (uint32_t)(((e + 15) << 10) | (int)((ldexp(r, -e) - 1.0) * 1024.0));
}

__device__ inline double f16_value(uint32_t b) {
  int e = (b >> 10) & 31, m = b & 1023;
  return e == 0 ? ldexp(m / 1024.0, -14) : ldexp(1.0 + m / 1024.0, e - 15);
}

__global__ void k_pack_bf16(const float* __restrict__ src, size_t n, uint16_t* __restrict__ dst) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double v = (double)src[i];
  double mag = round_grid(fabs(v), 7, -126);
  uint32_t bits;
  if (mag == 0.0) {
    bits = 0;
  } else {
    // fp32 holds every bf16 value exactly: take its top 16 bits
    bits = __float_as_uint((float)mag) >> 16;
    if (v < 0) bits |= 0x8000u;
  }
  dst[i] = (uint16_t)bits;
}

// One thread per block of 32 along a row.
__global__ void k_pack_blocks(const float* __restrict__ src, int rows, int cols, int bits,
                              uint8_t* __restrict__ dst) {
  size_t nb = (size_t)rows * (cols / 32);
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nb) return;
  const float* p = src + i * 32;
  double amax = 0.0;
  for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs((double)p[j]));
  int qmax = bits == 8 ? 127 : 7, qmin = bits == 8 ? -127 : -8;
  uint32_t db = f16_bits(amax / qmax);
  double d = f16_value(db);
  uint8_t* codes = dst + i * 32 * bits / 8;
  uint8_t* sc = dst + (size_t)rows * cols * bits / 8 + i * 2;
  int q[32];
  for (int j = 0; j < 32; ++j) {
    int v = 0;
    if (d > 0) v = (int)fmin(fmax(rint((double)p[j] / d), (double)qmin), (double)qmax);
    q[j] = v;
  }
  if (bits == 8) {
    for (int j = 0; j < 32; ++j) codes[j] = (uint8_t)(q[j] & 0xFF);
  } else {
    for (int j = 0; j < 16; ++j) codes[j] = (uint8_t)((q[2 * j] + 8) | ((q[2 * j + 1] + 8) << 4));
  }
  sc[0] = (uint8_t)(db & 0xFF);
  sc[1] = (uint8_t)(db >> 8);
}

// amax of matrix m (blockIdx.y) into out[m * stride]; non-negative floats
// order like their bit patterns, so an integer max is exact.
__global__ void k_amax(const float* __restrict__ src, size_t per, unsigned* __restrict__ out,
                       int stride) {
  int m = blockIdx.y;
  const float* p = src + (size_t)m * per;
  float a = 0.f;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < per;
       i += (size_t)gridDim.x * blockDim.x)
    a = fmaxf(a, fabsf(p[i]));
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((threadIdx.x & 63) == 0) atomicMax(out + (size_t)m * stride, __float_as_uint(a));
}

__global__ void k_zero_u32(unsigned* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One thread per block of 16 of one matrix of one expert. which: 0 gate,
// 1 up, 2 down.
__global__ void k_pack_fp4(const float* __restrict__ gate, const float* __restrict__ up,
                           const float* __restrict__ down, int n, int ell, int f,
                           const unsigned* __restrict__ amax, uint8_t* __restrict__ dst,
                           size_t rec_bytes) {
  size_t per = (size_t)ell * f;
  size_t nb = per / 16;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  int which = blockIdx.y;
  int e = blockIdx.z;
  if (i >= nb || e >= n) return;
  const float* src = (which == 0 ? gate : which == 1 ? up : down) + (size_t)e * per + i * 16;
  double am = (double)__uint_as_float(amax[e * 3 + which]);
  float ts = am > 0 ? (float)(am / 2688.0) : 1.0f;
  double bmax = 0.0;
  for (int j = 0; j < 16; ++j) bmax = fmax(bmax, fabs((double)src[j]));
  uint32_t sb = e4m3_code(bmax / (6.0 * (double)ts));
  double s = e4m3_value(sb) * (double)ts;
  uint8_t* rec = dst + (size_t)e * rec_bytes;
  size_t n2 = per / 2;
  uint8_t* codes = rec + which * n2 + i * 8;
  uint8_t* scales = rec + 3 * n2 + which * nb + i;
  for (int j = 0; j < 8; ++j) {
    uint32_t c0 = s > 0 ? e2m1_code((double)src[2 * j] / s) : 0u;
    uint32_t c1 = s > 0 ? e2m1_code((double)src[2 * j + 1] / s) : 0u;
    codes[j] = (uint8_t)(c0 | (c1 << 4));
  }
  scales[0] = (uint8_t)sb;
  if (i == 0) {
    float* tail = (float*)(rec + 3 * n2 + 3 * nb);
    tail[which] = ts;
    if (which == 0) ((uint32_t*)tail)[3] = 0u;
  }
}

}  // namespace

// ---------------------------------------------------------------------------

int pack_bf16_impl(const float* src, size_t n, uint16_t* dst, hipStream_t st) {
  if (!n) return 0;
  hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, n, dst);
  LMOE_HIP(hipGetLastError());
  return 0;
}

int pack_blocks_impl(const float* src, int rows, int cols, int bits, uint8_t* dst,
                     hipStream_t st) {
  size_t nb = (size_t)rows * (cols / 32);
  if (!nb) return 0;
  hipLaunchKernelGGL(k_pack_blocks, dim3((unsigned)((nb + 127) / 128)), dim3(128), 0, st, src,
                     rows, cols, bits, dst);
  LMOE_HIP(hipGetLastError());
  return 0;
}

int pack_experts_impl(const float* gate, const float* up, const float* down, int n, int ell,
                      int f, uint8_t* dst, hipStream_t st) {
  if (n <= 0) return 0;
  unsigned* amax = nullptr;
  LMOE_HIP(hipMallocAsync((void**)&amax, sizeof(unsigned) * 3 * n, st));
  size_t per = (size_t)ell * f;
  size_t nb = per / 16;
  size_t rec = lmoe_expert_record_bytes(ell, f);
  hipLaunchKernelGGL(k_zero_u32, dim3((3 * n + 255) / 256), dim3(256), 0, st, amax, 3 * n);
  for (int e0 = 0; e0 < n; e0 += 65535) {
    int cnt = std::min(65535, n - e0);
    for (int which = 0; which < 3; ++which) {
      const float* src = (which == 0 ? gate : which == 1 ? up : down) + (size_t)e0 * per;
      hipLaunchKernelGGL(k_amax, dim3(64, cnt), dim3(256), 0, st, src, per,
                         amax + 3 * e0 + which, 3);
    }
    hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)((nb + 255) / 256), 3, cnt), dim3(256), 0, st,
                       gate + (size_t)e0 * per, up + (size_t)e0 * per, down + (size_t)e0 * per,
                       cnt, ell, f, amax + 3 * e0, dst + (size_t)e0 * rec, rec);
  }
  LMOE_HIP(hipGetLastError());
  LMOE_HIP(hipFreeAsync(amax, st));
  return 0;
}

// ---------------------------------------------------------------------------
// lmoe_load_weights

namespace {

struct DevTemp {
  void* p = nullptr;
  ~DevTemp() {
    if (p) (void)hipFree(p);
  }
};

int copy_in(DevTemp& t, const void* src, size_t bytes, hipStream_t st) {
  LMOE_HIP(hipMalloc(&t.p, bytes ? bytes : 1));
  LMOE_HIP(hipMemcpyAsync(t.p, src, bytes, hipMemcpyDefault, st));
  return 0;
}

}  // namespace

int load_weights_impl(lmoe_t* h, const lmoe_weights* w, hipStream_t st) {
  const lmoe_dims& d = h->d;
  const int E = d.n_experts, H = d.hidden, L = d.latent, G = d.n_groups, F = d.expert_ffn,
            Fs = d.shared_ffn, bits = d.du_bits;
  const int du_fmt = bits == 8 ? kQ8 : kQ4;
  if (!w->router_bf16 || !w->group_labels || !w->d_blob || !w->u_blob || !w->experts ||
      !w->shared_gate_bf16 || !w->shared_up_bf16 || !w->shared_down_bf16) {
    set_error("lmoe_load_weights: a required weight pointer is NULL");
    return LMOE_EINVAL;
  }
  if (d.has_router_bias && !w->router_bias) {
    set_error("lmoe_load_weights: has_router_bias is set but router_bias is NULL");
    return LMOE_EINVAL;
  }
  const size_t dg = lmoe_du_matrix_bytes(L, H, bits), ug = lmoe_du_matrix_bytes(H, L, bits);
  if (w->d_bytes != dg * G || w->u_bytes != ug * G) {
    set_error("lmoe_load_weights: d_bytes/u_bytes do not match G packed matrices");
    return LMOE_EINVAL;
  }
  const bool q3k = d.expert_format == LMOE_EXPERTS_Q3K;
  const size_t rec = lmoe_expert_record_bytes_fmt(L, F, d.expert_format);
  if (w->expert_record_bytes != rec) {
    set_error("lmoe_load_weights: expert_record_bytes does not match the expert format's record size");
    return LMOE_EINVAL;
  }
  std::vector<uint8_t> lab(E);
  LMOE_HIP(hipMemcpy(lab.data(), w->group_labels, E, hipMemcpyDefault));
  for (int e = 0; e < E; ++e)
    if (lab[e] >= G) {
      set_error("lmoe_load_weights: a group label is >= n_groups");
      return LMOE_EINVAL;
    }
  // From here on the device copies are overwritten: the handle refuses
  // forwards until every part of the new weights is in place, so a load that
  // fails midway cannot leave a mix of old and new weights in use.
  h->loaded = false;

  // router, bias, labels
  {
    DevTemp t;
    if (int rc = copy_in(t, w->router_bf16, (size_t)E * H * 2, st)) return rc;
    Src a{(const uint8_t*)t.p, nullptr, E};
    if (int rc = launch_tile(kBF16R, a, a, 0, H, h->g_router, h->router, st)) return rc;
    if (h->pw.tmax) {
      // prefill: the MFMA layout for the logits GEMM, the plain rows for the
      // fp64 rescoring, and max_e |Wr_e|_2 for its rounding bound
      if (int rc = launch_tile(kBF16, a, a, 0, H, h->g_router_m, h->router_m, st)) return rc;
      LMOE_HIP(hipMemcpyAsync(h->router_rm, t.p, (size_t)E * H * 2, hipMemcpyDeviceToDevice, st));
      if (int rc = prefill_router_wmax(h, st)) return rc;
      // experts in (label, expert) order
      std::vector<int> order(E);
      for (int e = 0; e < E; ++e) order[e] = e;
      std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lab[x] < lab[y]; });
      LMOE_HIP(hipMemcpyAsync(h->pw.eorder, order.data(), sizeof(int) * E, hipMemcpyHostToDevice, st));
      LMOE_HIP(hipStreamSynchronize(st));
    }
    if (d.has_router_bias)
      LMOE_HIP(hipMemcpyAsync(h->bias, w->router_bias, sizeof(float) * E, hipMemcpyDefault, st));
    else
      LMOE_HIP(hipMemsetAsync(h->bias, 0, sizeof(float) * E, st));
    LMOE_HIP(hipMemcpyAsync(h->labels, lab.data(), E, hipMemcpyHostToDevice, st));
    LMOE_HIP(hipStreamSynchronize(st));
  }
  // D and U
  for (int which = 0; which < 2; ++which) {
    DevTemp t;
    const uint8_t* blob = which == 0 ? w->d_blob : w->u_blob;
    const size_t gb = which == 0 ? dg : ug;
    const int rows = which == 0 ? L : H, k = which == 0 ? H : L;
    const Geom& g = which == 0 ? h->g_d : h->g_u;
    uint8_t* dst = which == 0 ? h->dmat : h->umat;
    if (int rc = copy_in(t, blob, gb * G, st)) return rc;
    for (int gi = 0; gi < G; ++gi) {
      const uint8_t* base = (const uint8_t*)t.p + gi * gb;
      Src a{base, base + (size_t)rows * k * bits / 8, rows};
      if (int rc = launch_tile(du_fmt, a, a, 0, k, g, dst + gi * g.bytes(), st)) return rc;
    }
    LMOE_HIP(hipStreamSynchronize(st));
  }
  if (h->pw.tmax) {
    if (int rc = prefill_dequant_du(h, st)) return rc;
    LMOE_HIP(hipStreamSynchronize(st));
  }
  // shared expert
  {
    DevTemp tg, tu, td;
    if (int rc = copy_in(tg, w->shared_gate_bf16, (size_t)Fs * H * 2, st)) return rc;
    if (int rc = copy_in(tu, w->shared_up_bf16, (size_t)Fs * H * 2, st)) return rc;
    if (int rc = copy_in(td, w->shared_down_bf16, (size_t)H * Fs * 2, st)) return rc;
    Src a{(const uint8_t*)tg.p, nullptr, Fs}, b{(const uint8_t*)tu.p, nullptr, Fs};
    if (int rc = launch_tile(kBF16, a, b, 1, H, h->g_sgu, h->sgu, st)) return rc;
    Src c{(const uint8_t*)td.p, nullptr, H};
    if (int rc = launch_tile(kBF16, c, c, 0, Fs, h->g_sdn, h->sdn, st)) return rc;
    LMOE_HIP(hipStreamSynchronize(st));
  }
  // experts, in chunks of records
  {
    const int chunk = 64;
    DevTemp t;
    LMOE_HIP(hipMalloc(&t.p, rec * chunk));
    const RecOff ro = rec_off(L, F);
    for (int e0 = 0; e0 < E; e0 += chunk) {
      int cnt = std::min(chunk, E - e0);
      LMOE_HIP(hipMemcpyAsync(t.p, w->experts + (size_t)e0 * rec, rec * cnt, hipMemcpyDefault, st));
      for (int i = 0; i < cnt; ++i) {
        const uint8_t* r = (const uint8_t*)t.p + (size_t)i * rec;
        uint8_t* dst = h->experts + (size_t)(e0 + i) * h->expert_stride;
        if (q3k) {
          // gate blocks [F][L/256], up blocks, down blocks [L][F/32]
          const size_t n1 = (size_t)F * (L / 256) * kQ3KBlock;
          Src ga{r, nullptr, F}, ua{r + n1, nullptr, F}, da{r + 2 * n1, nullptr, L};
          if (int rc = launch_tile(kQ3K, ga, ua, 1, L, h->g_gu, dst, st)) return rc;
          if (int rc = launch_tile(kIQ4, da, da, 0, F, h->g_dn, dst + h->g_gu.bytes(), st)) return rc;
          continue;
        }
        Src ga{r + ro.gate_c, r + ro.gate_s, F}, ua{r + ro.up_c, r + ro.up_s, F};
        if (int rc = launch_tile(kFP4, ga, ua, 1, L, h->g_gu, dst, st)) return rc;
        Src da{r + ro.down_c, r + ro.down_s, L};
        if (int rc = launch_tile(kFP4, da, da, 0, F, h->g_dn, dst + h->g_gu.bytes(), st)) return rc;
      }
      if (q3k)
        hipLaunchKernelGGL(k_unit_ts, dim3((cnt + 63) / 64), dim3(64), 0, st, cnt,
                           h->experts + (size_t)e0 * h->expert_stride, h->expert_stride, h->ts_off);
      else
        hipLaunchKernelGGL(k_copy_ts, dim3((cnt + 63) / 64), dim3(64), 0, st, (const uint8_t*)t.p,
                           rec, ro.tail, cnt, h->experts + (size_t)e0 * h->expert_stride,
                           h->expert_stride, h->ts_off);
      LMOE_HIP(hipGetLastError());
      LMOE_HIP(hipStreamSynchronize(st));
    }
  }
  h->labels_host = lab;
  h->loaded = true;
  return 0;
}

}  // namespace lm
