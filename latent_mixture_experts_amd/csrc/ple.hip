// PLE n-gram embedding gather ("Edge0-145B: a Qwen MoE with its experts
// squeezed, and a 51B table left on the SSD", section "The 51.2B the GPU
// never holds"): each token hashes its last two tokens into 8 rows and its
// last three into 8 more, of one table of E4M3 rows (160 bytes each at the
// Edge0 shapes, 2,560 bytes a token).
//
// The hash is this library's reading (the pages do not give it): head h's
// row is mix64(key) mod rows_h, key = sum over the n-gram's tokens, oldest
// first, of (id + 1) * K[h][j] mod 2^64, with mix64 the SplitMix64 output
// function and K[h][j] its output number 3h + j + 1 from seed 0 (Steele, Lea
// and Flood, OOPSLA 2014). Head h's rows follow those of heads < h.
//
// One wavefront per token: lanes 0..15 hash, then the 16 rows are copied in
// 16-byte pieces, one per lane and step, each decoded to bf16 (exact: E4M3
// has 3 mantissa bits and exponents inside bf16's range) and stored as 32
// bytes. The table is read once per forward: non-temporal loads.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace lm {
namespace {

constexpr int kHeads = 16, kHeadsPerGram = 8;
constexpr unsigned long long kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// bf16 bits of an E4M3 code (OCP E4M3FN: bias 7, no infinities, S.1111.111
// is NaN): normals keep their exponent (rebiased) and 3 mantissa bits;
// subnormals m * 2^-9 are normalized at their leading bit.
__device__ __forceinline__ uint32_t e4m3_bf16(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 8, e = (b >> 3) & 0xFu, m = b & 7u;
  if (e == 15u && m == 7u) return s | 0x7FC0u;
  if (e != 0u) return s | ((e + 120u) << 7) | (m << 4);
  if (m == 0u) return s;
  const uint32_t p = 31u - (uint32_t)__builtin_clz(m);   // leading bit of m
  return s | ((p + 118u) << 7) | ((m << (7u - p)) & 0x7Fu);
}

struct Ple {
  const int32_t* tokens;       // [T + 2]
  int T, row_bytes;
  const uint8_t* table;
  uint16_t* out;               // [T][16][row_bytes] bf16
  unsigned long long off[kHeads], rows[kHeads], key[kHeads][3];
};

__global__ __launch_bounds__(256) void k_ple(Ple a) {
  __shared__ unsigned long long rowsh[4][kHeads];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= a.T) return;                          // whole wavefronts
  if (lane < kHeads) {
    const int n = lane < kHeadsPerGram ? 2 : 3;
    unsigned long long key = 0;
    for (int j = 0; j < n; ++j)
      key += (unsigned long long)((long long)a.tokens[t + 3 - n + j] + 1) * a.key[lane][j];
    rowsh[w][lane] = a.off[lane] + mix64(key) % a.rows[lane];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int pieces = a.row_bytes >> 4, total = kHeads * pieces;
  for (int i = lane; i < total; i += 64) {
    const int h = i / pieces, c = i - h * pieces;
    const uint8_t* src = a.table + rowsh[w][h] * (unsigned long long)a.row_bytes + 16 * c;
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    const u4v v = __builtin_nontemporal_load((const u4v*)src);
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t word = v[q];
      o[2 * q] = e4m3_bf16(word & 0xFFu) | (e4m3_bf16((word >> 8) & 0xFFu) << 16);
      o[2 * q + 1] = e4m3_bf16((word >> 16) & 0xFFu) | (e4m3_bf16(word >> 24) << 16);
    }
    uint4* dst = (uint4*)(a.out + ((size_t)t * kHeads + h) * a.row_bytes + 16 * c);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

}  // namespace
}  // namespace lm

using namespace lm;

int lmoe_ple_gather(const int32_t* tokens, int32_t T, const uint8_t* table, const int64_t* head_rows,
                    int32_t row_bytes, uint16_t* out, void* stream) {
  if (T < 0 || !head_rows || row_bytes < 16 || row_bytes > 1024 || row_bytes % 16 ||
      (T > 0 && (!tokens || !table || !out))) {
    set_error("lmoe_ple_gather: bad argument (T >= 0, row_bytes a multiple of 16 in [16, 1024], "
              "non-NULL pointers)");
    return LMOE_EINVAL;
  }
  Ple a{};
  unsigned long long off = 0;
  for (int h = 0; h < kHeads; ++h) {
    if (head_rows[h] <= 0) {
      set_error("lmoe_ple_gather: every head needs at least one row");
      return LMOE_EINVAL;
    }
    a.off[h] = off;
    a.rows[h] = (unsigned long long)head_rows[h];
    off += a.rows[h];
    for (int j = 0; j < 3; ++j) a.key[h][j] = mix64((unsigned long long)(3 * h + j + 1) * kGolden);
  }
  if (T == 0) return LMOE_OK;
  a.tokens = tokens;
  a.T = T;
  a.row_bytes = row_bytes;
  a.table = table;
  a.out = out;
  hipLaunchKernelGGL(k_ple, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, (hipStream_t)stream, a);
  LMOE_HIP(hipGetLastError());
  return LMOE_OK;
}
