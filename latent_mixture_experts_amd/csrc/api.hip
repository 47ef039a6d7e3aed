// C ABI of liblmoe (declared and documented in include/lmoe.h): argument
// validation, device memory, and dispatch to the decode path.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <string>
#include <type_traits>

#include "internal.h"

namespace lm {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return LMOE_EHIP;
}

namespace {

int check_dims(const lmoe_dims& d) {
  auto bad = [](const char* m) {
    set_error(std::string("lmoe_create: ") + m);
    return LMOE_EINVAL;
  };
  auto unsup = [](const char* m) {
    set_error(std::string("lmoe_create: ") + m);
    return LMOE_EUNSUPPORTED;
  };
  if (d.hidden <= 0 || d.latent <= 0 || d.n_experts <= 0 || d.top_k <= 0 || d.n_groups <= 0 ||
      d.expert_ffn <= 0 || d.shared_ffn <= 0 || d.max_tokens <= 0)
    return bad("every dimension must be positive");
  if (d.du_bits != 8 && d.du_bits != 4) return bad("du_bits must be 8 or 4");
  if (d.top_k > d.n_experts) return bad("top_k exceeds n_experts");
  if (d.has_router_bias != 0 && d.has_router_bias != 1) return bad("has_router_bias must be 0 or 1");
  if (d.expert_format != LMOE_EXPERTS_NVFP4 && d.expert_format != LMOE_EXPERTS_Q3K)
    return bad("expert_format must be LMOE_EXPERTS_NVFP4 or LMOE_EXPERTS_Q3K");
  if (d.expert_format == LMOE_EXPERTS_Q3K && d.latent % 256)
    return unsup("Q3_K experts need latent % 256 == 0 (one super-block per 256 columns)");
  if (d.hidden % 256) return unsup("hidden must be a multiple of 256");
  if (d.latent % 64) return unsup("latent must be a multiple of 64");
  if (d.expert_ffn % 32 || d.shared_ffn % 32) return unsup("expert_ffn and shared_ffn must be multiples of 32");
  if (d.du_bits == 4 && d.latent % 128) return unsup("Q4 D/U needs latent % 128 == 0");
  if (d.hidden > 4096 || d.latent > 4096 || d.expert_ffn > 4096 || d.shared_ffn > 4096)
    return unsup("widths above 4096");
  if (d.n_experts > 1024 || d.top_k > 64 || d.n_groups > 64)
    return unsup("n_experts <= 1024, top_k <= 64, n_groups <= 64");
  if (d.max_tokens > kMaxTokens) return unsup("max_tokens above 1048576");
  // the decode kernels keep activations, partial sums, expert outputs and the
  // routing tables in LDS: refuse shapes whose blocks would not fit a CU
  const int Td = d.max_tokens < kMaxDecodeT ? d.max_tokens : kMaxDecodeT;
  if (decode_lds_bytes(d, Td) > 160 * 1024)
    return unsup("decode path: n_groups, T * top_k or the expert count too large for the LDS of a CU");
  return 0;
}

template <typename P>
int dalloc(lmoe_t* h, P** p, size_t bytes) {
  void* q = nullptr;
  hipError_t e = hipMalloc(&q, bytes ? bytes : 1);
  if (e != hipSuccess) {
    set_error(std::string("hipMalloc of ") + std::to_string(bytes) + " bytes: " + hipGetErrorString(e));
    return LMOE_ENOMEM;
  }
  h->allocations.push_back(q);
  *p = (P*)q;
  return 0;
}

void free_all(lmoe_t* h) {
  for (void* p : h->allocations) (void)hipFree(p);
  h->allocations.clear();
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->aux) (void)hipStreamDestroy(h->aux);
  h->ev_fork = h->ev_join = nullptr;
  h->aux = nullptr;
}

}  // namespace

// Lays out the decode workspace for up to T tokens at `base` (nullptr: only
// sizes it); returns its bytes. Each array starts on a 256-byte boundary.
size_t decode_ws_layout(const lmoe_t* h, int T, char* base, Workspace* out) {
  const lmoe_dims& d = h->d;
  const int E = d.n_experts, H = d.hidden, L = d.latent, G = d.n_groups, F = d.expert_ffn,
            Fs = d.shared_ffn, K = d.top_k;
  const int nss_d = (H + kSSCols - 1) / kSSCols, nss_s = nss_d;
  const int Epad = (E + 63) / 64 * 64;
  const int n = T * K;
  Workspace w;
  w.tmax = T;
  w.nch = (H + 64 * nss_d - 1) / (64 * nss_d);
  size_t off = 0;
  auto take = [&](auto*& p, size_t bytes) {
    off = (off + 255) / 256 * 256;
    p = base ? reinterpret_cast<std::remove_reference_t<decltype(p)>>(base + off) : nullptr;
    off += bytes ? bytes : 1;
  };
  take(w.part64, sizeof(double) * w.nch * T * Epad);
  take(w.topk_idx, sizeof(int) * n);
  take(w.topk_w, sizeof(float) * n);
  take(w.perm, sizeof(int) * n);
  take(w.tg_cnt, sizeof(int) * T * G);
  take(w.tg_pos, sizeof(int) * T * G * K);
  take(w.slot_expert, sizeof(int) * n);
  take(w.slot_start, sizeof(int) * n);
  take(w.slot_count, sizeof(int) * n);
  take(w.slot_xrow, sizeof(int) * n * kMaxDecodeT);
  take(w.n_slots, sizeof(int));
  take(w.gslot_off, sizeof(int) * (G + 1));
  take(w.group_off, sizeof(int) * (G + 1));
  take(w.expert_count, sizeof(int) * E);
  take(w.rms, sizeof(float) * T);
  take(w.rms64, sizeof(double) * T);
  take(w.sqp, sizeof(double) * w.nch * T);
  take(w.xl, sizeof(float) * T * G * L);
  take(w.hs, sizeof(float) * T * Fs);
  take(w.hsp, sizeof(float) * nss_s * T * 2 * Fs);
  take(w.hbuf, sizeof(float) * n * F);
  take(w.obuf, sizeof(float) * n * L);
  // 2G + shared-down blocks (at most one per half-step)
  take(w.ypart, sizeof(float) * (2 * G + (Fs + 127) / 128) * T * H);
  take(w.ctr_router, sizeof(unsigned));
  take(w.ctr_y, sizeof(unsigned) * (H / 64));
  if (out) *out = w;
  return (off + 255) / 256 * 256;
}

namespace {

int create_impl(lmoe_t* h) {
  const lmoe_dims& d = h->d;
  const int E = d.n_experts, H = d.hidden, L = d.latent, G = d.n_groups, F = d.expert_ffn,
            Fs = d.shared_ffn, K = d.top_k;
  const int du = d.du_bits == 8 ? kQ8 : kQ4;
  h->g_router = make_geom(kBF16R, E, H);
  h->g_d = make_geom(du, L, H);
  h->g_u = make_geom(du, H, L);
  const bool q3k = d.expert_format == LMOE_EXPERTS_Q3K;
  h->g_gu = make_geom(q3k ? kQ3K : kFP4, 2 * F, L);   // tiles of 32 gate + 32 up rows
  h->g_dn = make_geom(q3k ? kIQ4 : kFP4, L, F);
  h->g_sgu = make_geom(kBF16, 2 * Fs, H);
  h->g_sdn = make_geom(kBF16, H, Fs);
  h->ts_off = h->g_gu.bytes() + h->g_dn.bytes();
  h->expert_stride = (h->ts_off + 16 + 255) / 256 * 256;

  int rc;
#define A(p, n) if ((rc = dalloc(h, &(p), (n)))) return rc
  A(h->router, h->g_router.bytes());
  A(h->bias, sizeof(float) * E);
  A(h->labels, (size_t)(E + 3) / 4 * 4);   // whole 32-bit words: kernels read labels by word
  A(h->dmat, h->g_d.bytes() * G);
  A(h->umat, h->g_u.bytes() * G);
  A(h->experts, h->expert_stride * E);
  A(h->sgu, h->g_sgu.bytes());
  A(h->sdn, h->g_sdn.bytes());

  {
    const int T = d.max_tokens < kMaxDecodeT ? d.max_tokens : kMaxDecodeT;
    char* base = nullptr;
    A(base, decode_ws_layout(h, T, nullptr, nullptr));
    decode_ws_layout(h, T, base, &h->ws);
  }

  // prefill path (T > kMaxDecodeT): router copies and GEMM workspace (NVFP4
  // records; Q3_K records run larger batches as decode forwards of 8 tokens)
  if (d.max_tokens > kMaxDecodeT && !q3k) {
    PrefillWs& p = h->pw;
    const size_t Tp = (size_t)d.max_tokens, nk = Tp * K;
    const size_t nchunk = (size_t)prefill_chunks(d.max_tokens);
    h->g_router_m = make_geom(kBF16, E, H);
    const size_t Epm = (size_t)h->g_router_m.tiles * 64;
    p.tmax = d.max_tokens;
    A(h->router_m, h->g_router_m.bytes());
    h->g_d16 = make_geom(kF16, L, H);
    h->g_u16 = make_geom(kF16, H, L);
    A(h->dmat16, h->g_d16.bytes() * G);
    A(h->umat16, h->g_u16.bytes() * G);
    A(h->router_rm, sizeof(uint16_t) * E * H);
    A(p.wmax, sizeof(double));
    A(p.xh, 2 * Tp * H);
    A(p.xb, 4 * Tp * H);
    A(p.xnorm, sizeof(double) * Tp);
    A(p.r, sizeof(float) * Tp);
    A(p.r64, sizeof(double) * Tp);
    A(p.xsc, sizeof(float) * Tp);
    A(p.psc, sizeof(float) * nk);
    A(p.logits, sizeof(float) * Tp * Epm);
    A(p.idx, sizeof(int) * nk);
    A(p.w, sizeof(float) * nk);
    A(p.cmask, sizeof(unsigned long long) * nchunk * E);
    A(p.gmask, sizeof(unsigned long long) * nchunk * G);
    A(p.ccnt, sizeof(int) * nchunk * E);
    A(p.cbase, sizeof(int) * nchunk * E);
    A(p.eorder, sizeof(int) * E);
    A(p.seg_start, sizeof(int) * E);
    A(p.expert_count, sizeof(int) * E);
    A(p.group_off, sizeof(int) * (G + 1));
    A(p.pieces, prefill_piece_bytes() * prefill_max_pieces(d.max_tokens, K, E));
    A(p.npieces, 3 * sizeof(int));
    A(p.perm, sizeof(int) * nk);
    A(p.inv, sizeof(int) * nk);
    A(p.xl, 2 * Tp * G * L);
    A(p.hsb, 4 * Tp * Fs);
    A(p.h, 2 * nk * F);
    A(p.o, sizeof(float) * nk * L);
    A(p.s, 2 * Tp * G * L);
    A(p.gl_tok, sizeof(int) * Tp * G);
    A(p.gl_cnt, sizeof(int) * G);
    LMOE_HIP(hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking));
    LMOE_HIP(hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming));
    LMOE_HIP(hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming));
  }
#undef A
  LMOE_HIP(hipMemset(h->ws.ctr_router, 0, sizeof(unsigned)));
  LMOE_HIP(hipMemset(h->ws.ctr_y, 0, sizeof(unsigned) * (H / 64)));
  LMOE_HIP(hipDeviceSynchronize());
  return 0;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Exclusive scan of n counts into off[0..n] by one block (n <= 1024).
__global__ __launch_bounds__(1024) void k_exclusive_scan(const int* __restrict__ cnt, int n,
                                                         int* __restrict__ off) {
  __shared__ int buf[1024];
  const int i = threadIdx.x;
  buf[i] = i < n ? cnt[i] : 0;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {      // inclusive Hillis-Steele scan
    const int v = i >= d ? buf[i - d] : 0;
    __syncthreads();
    buf[i] += v;
    __syncthreads();
  }
  if (i < n) off[i + 1] = buf[i];
  if (i == 0) off[0] = 0;
}

int copy_debug(lmoe_t* h, const lmoe_debug* dbg, int T, hipStream_t st) {
  const lmoe_dims& d = h->d;
  const Workspace& w = h->ws;
  const PrefillWs& p = h->pw;
  const bool pre = T > kMaxDecodeT;
  const size_t n = (size_t)T * d.top_k;
  const auto D2D = hipMemcpyDeviceToDevice;
  if (dbg->topk_idx) LMOE_HIP(hipMemcpyAsync(dbg->topk_idx, pre ? p.idx : w.topk_idx, 4 * n, D2D, st));
  if (dbg->topk_w) LMOE_HIP(hipMemcpyAsync(dbg->topk_w, pre ? p.w : w.topk_w, 4 * n, D2D, st));
  if (dbg->perm) LMOE_HIP(hipMemcpyAsync(dbg->perm, pre ? p.perm : w.perm, 4 * n, D2D, st));
  if (dbg->expert_count)
    LMOE_HIP(hipMemcpyAsync(dbg->expert_count, pre ? p.expert_count : w.expert_count,
                            4 * (size_t)d.n_experts, D2D, st));
  if (dbg->expert_off) {
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(1024), 0, st,
                       (const int*)(pre ? p.expert_count : w.expert_count), d.n_experts,
                       dbg->expert_off);
    LMOE_HIP(hipGetLastError());
  }
  if (dbg->group_off)
    LMOE_HIP(hipMemcpyAsync(dbg->group_off, pre ? p.group_off : w.group_off,
                            4 * (size_t)(d.n_groups + 1), D2D, st));
  if (dbg->latent) {
    if (pre) return prefill_debug_latent(h, T, dbg->latent, st);
    LMOE_HIP(hipMemcpyAsync(dbg->latent, w.xl, 4 * (size_t)T * d.n_groups * d.latent, D2D, st));
  }
  return 0;
}

int check_forward(lmoe_t* h, const void* x, int T, const void* y) {
  if (!h) {
    set_error("NULL handle");
    return LMOE_EINVAL;
  }
  if (!h->loaded) {
    set_error("forward before lmoe_load_weights");
    return LMOE_ESTATE;
  }
  if (!x || !y) {
    set_error("NULL x or y");
    return LMOE_EINVAL;
  }
  if (T <= 0 || T > h->d.max_tokens) {
    set_error("T must be in [1, max_tokens]");
    return LMOE_EINVAL;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Allocation-free decode forwards: the workspace lives in one static device
// array per GPU (allocated by the loader with the code object, kept until the
// process ends). Host code never passes `scratch` itself to a kernel (its
// host-side name is only a stand-in): each device's address is looked up once
// with hipGetSymbolAddress and kept here.
constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per GPU
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};

// Looks up this device's copy of `scratch` (the device must be current).
int scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) {
    set_error("scratch: device index above the supported count");
    return LMOE_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[device]) return 0;
  void* p = nullptr;
  LMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
  if (!p) {
    set_error("scratch: hipGetSymbolAddress returned no address");
    return LMOE_EHIP;
  }
  g_scratch[device] = (char*)p;
  return 0;
}

char* scratch_of(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch[device];
}

// Zeroes n 32-bit words (the kernels' arrival counters must start at 0).
__global__ void k_fill_zero(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace
}  // namespace lm

using namespace lm;

extern "C" {

int lmoe_create(const lmoe_dims* dims, int hip_device, lmoe_t** out) {
  if (!dims || !out) {
    set_error("lmoe_create: NULL argument");
    return LMOE_EINVAL;
  }
  if (int rc = check_dims(*dims)) return rc;
  int ndev = 0;
  LMOE_HIP(hipGetDeviceCount(&ndev));
  if (hip_device < 0 || hip_device >= ndev) {
    set_error("lmoe_create: no such HIP device");
    return LMOE_EINVAL;
  }
  DeviceGuard g(hip_device);
  lmoe_t* h = new (std::nothrow) lmoe_t();
  if (!h) return LMOE_ENOMEM;
  h->d = *dims;
  h->device = hip_device;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, hip_device) == hipSuccess &&
      ncu > 0)
    h->ncu = ncu;
  if (int rc = scratch_setup(hip_device)) {
    delete h;
    return rc;
  }
  if (int rc = create_impl(h)) {
    free_all(h);
    delete h;
    return rc;
  }
  *out = h;
  return 0;
}

int lmoe_load_weights(lmoe_t* h, const lmoe_weights* w, void* stream) {
  if (!h || !w) {
    set_error("lmoe_load_weights: NULL argument");
    return LMOE_EINVAL;
  }
  DeviceGuard g(h->device);
  return load_weights_impl(h, w, (hipStream_t)stream);
}

// Q3_K records, T > 8: decode forwards of up to 8 tokens each (every output
// row depends on its own input row only); the debug outputs that describe
// the whole batch's permutation are refused.
static int forward_chunked(lmoe_t* h, const float* x, int T, float* y, bool norm, float eps,
                           const lmoe_debug* dbg, hipStream_t st) {
  if (dbg && (dbg->perm || dbg->expert_count || dbg->expert_off || dbg->group_off)) {
    set_error("Q3_K records, T > 8: perm, expert_count, expert_off and group_off are not produced "
              "(the batch runs as decode forwards of 8 tokens)");
    return LMOE_EUNSUPPORTED;
  }
  const lmoe_dims& d = h->d;
  const size_t H = d.hidden, K = d.top_k, GL = (size_t)d.n_groups * d.latent;
  const auto D2D = hipMemcpyDeviceToDevice;
  h->rms_eps = eps;
  for (int t0 = 0; t0 < T; t0 += kMaxDecodeT) {
    const int n = T - t0 < kMaxDecodeT ? T - t0 : kMaxDecodeT;
    if (int rc = forward_decode(h, x + t0 * H, n, y + t0 * H, norm, st)) return rc;
    if (dbg && dbg->topk_idx)
      LMOE_HIP(hipMemcpyAsync(dbg->topk_idx + t0 * K, h->ws.topk_idx, 4 * n * K, D2D, st));
    if (dbg && dbg->topk_w)
      LMOE_HIP(hipMemcpyAsync(dbg->topk_w + t0 * K, h->ws.topk_w, 4 * n * K, D2D, st));
    if (dbg && dbg->latent)
      LMOE_HIP(hipMemcpyAsync(dbg->latent + t0 * GL, h->ws.xl, 4 * n * GL, D2D, st));
  }
  h->last_decode_T = 0;                            // the workspace holds the last chunk only
  return 0;
}

int lmoe_forward(lmoe_t* h, const float* x, int32_t T, float* y, const lmoe_debug* dbg,
                 void* stream) {
  if (int rc = check_forward(h, x, T, y)) return rc;
  if (x == y) {
    set_error("lmoe_forward: x and y alias");
    return LMOE_EINVAL;
  }
  DeviceGuard g(h->device);
  hipStream_t st = (hipStream_t)stream;
  if (T > kMaxDecodeT && h->d.expert_format == LMOE_EXPERTS_Q3K)
    return forward_chunked(h, x, T, y, false, 0.0f, dbg, st);
  const int rc = T > kMaxDecodeT ? forward_prefill(h, x, T, y, false, 0.0f, st)
                                 : forward_decode(h, x, T, y, false, st);
  if (rc) return rc;
  h->last_decode_T = T > kMaxDecodeT ? h->last_decode_T : T;
  if (dbg) return copy_debug(h, dbg, T, st);
  return 0;
}

int lmoe_forward_noalloc(lmoe_t* h, const float* x, int32_t T, float* y, void* stream) {
  if (!h || !x || !y || x == y || T <= 0 || T > h->d.max_tokens) {
    set_error("lmoe_forward_noalloc: NULL or aliased x / y, or T outside [1, max_tokens]");
    return LMOE_EINVAL;
  }
  if (T > kMaxDecodeT) {
    set_error("lmoe_forward_noalloc: serves the decode path only (T <= 8)");
    return LMOE_EUNSUPPORTED;
  }
  const size_t need = decode_ws_layout(h, T, nullptr, nullptr);
  if (need > kScratchBytes) {
    set_error("lmoe_forward_noalloc: the layer needs " + std::to_string(need) +
              " bytes of workspace at this T, above the " + std::to_string(kScratchBytes) +
              "-byte static scratch");
    return LMOE_EUNSUPPORTED;
  }
  if (int rc = check_forward(h, x, T, y)) return rc;
  DeviceGuard g(h->device);
  char* base = scratch_of(h->device);
  if (!base) {
    set_error("lmoe_forward_noalloc: no scratch address for this device");
    return LMOE_EHIP;
  }
  Workspace ws;
  decode_ws_layout(h, T, base, &ws);
  hipStream_t st = (hipStream_t)stream;
  // the counters reset themselves at the end of a forward; clear them anyway,
  // in case another handle's forward on this device stopped short
  const int nctr = h->d.hidden / 64;
  hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(64), 0, st, ws.ctr_router, 1);
  hipLaunchKernelGGL(k_fill_zero, dim3((nctr + 255) / 256), dim3(256), 0, st, ws.ctr_y, nctr);
  LMOE_HIP(hipGetLastError());
  return forward_decode(h, x, T, y, false, st, 0, &ws);
}

int lmoe_forward_block(lmoe_t* h, float* x, int32_t T, float eps, void* stream) {
  if (int rc = check_forward(h, x, T, x)) return rc;
  if (!(eps >= 0.0f)) {
    set_error("lmoe_forward_block: rms_eps must be >= 0");
    return LMOE_EINVAL;
  }
  DeviceGuard g(h->device);
  hipStream_t st = (hipStream_t)stream;
  if (T > kMaxDecodeT && h->d.expert_format == LMOE_EXPERTS_Q3K)
    return forward_chunked(h, x, T, x, true, eps, nullptr, st);
  if (T > kMaxDecodeT) return forward_prefill(h, x, T, x, true, eps, st);
  h->rms_eps = eps;                                // phase 1 normalizes the rows itself
  h->last_decode_T = 0;                            // the decode workspace now holds a block forward
  return forward_decode(h, x, T, x, true, st);
}

int lmoe_set_phase_events(lmoe_t* h, void* const* events, int32_t n) {
  if (!h) {
    set_error("lmoe_set_phase_events: NULL handle");
    return LMOE_EINVAL;
  }
  if (!events) {
    h->phase_events.clear();
    return 0;
  }
  if (n != kDecodePhases + 1 && n != kPrefillPhases + 1) {
    set_error("lmoe_set_phase_events: n must be lmoe_phase_count(T) + 1");
    return LMOE_EINVAL;
  }
  h->phase_events.assign((hipEvent_t*)events, (hipEvent_t*)events + n);
  return 0;
}

int32_t lmoe_phase_count(int32_t T) { return T > kMaxDecodeT ? kPrefillPhases : kDecodePhases; }

int lmoe_run_phase(lmoe_t* h, const float* x, int32_t T, int32_t phase, float* y, void* stream) {
  if (int rc = check_forward(h, x, T, y)) return rc;
  if (x == y || T > kMaxDecodeT || phase < 1 || phase > kDecodePhases) {
    set_error("lmoe_run_phase: x and y alias, T above 8 or phase outside 1..4");
    return LMOE_EINVAL;
  }
  if (h->last_decode_T != T) {
    set_error("lmoe_run_phase: the last decode forward on this handle was not of T tokens");
    return LMOE_ESTATE;
  }
  DeviceGuard g(h->device);
  return forward_decode(h, x, T, y, false, (hipStream_t)stream, phase);
}

void lmoe_destroy(lmoe_t* h) {
  if (!h) return;
  {
    DeviceGuard g(h->device);
    (void)hipDeviceSynchronize();
    free_all(h);
  }
  delete h;
}

const char* lmoe_strerror(int code) {
  switch (code) {
    case LMOE_OK: return "success";
    case LMOE_EINVAL: return "invalid argument";
    case LMOE_ENOMEM: return "out of device memory";
    case LMOE_EHIP: return "HIP runtime error";
    case LMOE_ESTATE: return "handle not ready (weights not loaded)";
    case LMOE_EUNSUPPORTED: return "dimensions not supported";
    default: return "unknown error code";
  }
}

const char* lmoe_last_error(void) { return g_last_error.c_str(); }

size_t lmoe_expert_record_bytes_fmt(int32_t latent, int32_t expert_ffn, int32_t fmt) {
  if (fmt == LMOE_EXPERTS_NVFP4) return lmoe_expert_record_bytes(latent, expert_ffn);
  if (fmt != LMOE_EXPERTS_Q3K || latent <= 0 || expert_ffn <= 0 || latent % 256 || expert_ffn % 32) return 0;
  return 2 * (size_t)expert_ffn * (latent / 256) * 110 + (size_t)latent * (expert_ffn / 32) * 18;
}

size_t lmoe_expert_record_bytes(int32_t latent, int32_t expert_ffn) {
  size_t n = (size_t)latent * expert_ffn;
  return 3 * (n / 2) + 3 * (n / 16) + 16;
}

size_t lmoe_du_matrix_bytes(int32_t rows, int32_t cols, int32_t du_bits) {
  return (size_t)rows * cols * du_bits / 8 + (size_t)rows * (cols / 32) * 2;
}

int lmoe_pack_bf16(const float* src, size_t n, uint16_t* dst, void* stream) {
  if ((!src || !dst) && n) {
    set_error("lmoe_pack_bf16: NULL pointer");
    return LMOE_EINVAL;
  }
  return pack_bf16_impl(src, n, dst, (hipStream_t)stream);
}

int lmoe_pack_blocks(const float* src, int32_t rows, int32_t cols, int32_t bits, uint8_t* dst,
                     void* stream) {
  if (!src || !dst || rows < 0 || cols < 0 || cols % 32 || (bits != 8 && bits != 4)) {
    set_error("lmoe_pack_blocks: bad argument (cols % 32 == 0, bits 8 or 4)");
    return LMOE_EINVAL;
  }
  return pack_blocks_impl(src, rows, cols, bits, dst, (hipStream_t)stream);
}

int lmoe_pack_expert_records(const float* gate, const float* up, const float* down, int32_t n,
                             int32_t latent, int32_t ffn, uint8_t* dst, void* stream) {
  if (!gate || !up || !down || !dst || n < 0 || latent <= 0 || ffn <= 0 ||
      ((size_t)latent * ffn) % 256) {
    set_error("lmoe_pack_expert_records: bad argument (latent*ffn % 256 == 0)");
    return LMOE_EINVAL;
  }
  return pack_experts_impl(gate, up, down, n, latent, ffn, dst, (hipStream_t)stream);
}

}  // extern "C"

int lmoe_set_prefill_d(lmoe_t* h, int32_t routed_only) {
  if (!h || (routed_only != 0 && routed_only != 1)) {
    set_error("lmoe_set_prefill_d: NULL handle or a value other than 0 and 1");
    return LMOE_EINVAL;
  }
  h->prefill_d_routed = routed_only == 1;
  return LMOE_OK;
}
