/*
 * lmoe.h -- C ABI of liblmoe.so, the latent mixture-of-experts layer of the
 * Edge0 145B / 120B models on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title, then section / equation / table):
 *   LAYER    = "Edge0 145B and Edge0 120B" model page: "Model profile" table
 *              (512 routed experts plus one shared expert, top_k 10, latent
 *              compression with 8 groups of D/U chosen by each expert's group
 *              label, expert formats, D/U formats) and the "Edge0-145B
 *              architecture" / "Edge0-120B architecture" tables and text
 *              (SwiGLU width 640; D projects to ell per routing group; only
 *              the experts work at ell; U projects the combined result back).
 *   TEARDOWN = "Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B
 *              table left on the SSD": "A latent in front of the experts"
 *              (the layer equation y = U_g(sum_e w_e E_e(D_g x)); D runs over
 *              all groups, U once per group a token routed into; the router
 *              reads the full-width hidden state), "What is 4-bit" (NVFP4
 *              record: FP4 values, an E4M3 scale per 16, a 16-byte tail; Q8_0
 *              / Q4_0 D/U), "The base, byte for byte" (bf16 router weights).
 *
 * The layer, per token x (fp32, width H):
 *   l      = Wr x (+ b)                 router logits over E experts
 *   idx, w = top K of l (descending, ties to the lower index) and the
 *            softmax of the kept logits (= softmax over E, keep K, renormalize)
 *   for each kept expert e with group g = label[e]:
 *            h = silu(Wg_e (D_g x)) * (Wu_e (D_g x));   o = w * Wd_e h
 *   y      = sum over groups g used by x of U_g (sum of that group's o)
 *          + Ws_down (silu(Ws_gate x) * (Ws_up x))
 *
 * Packed input formats (host or device memory; the library copies them):
 *   router      bf16 [E][H] (uint16 bit patterns)
 *   router bias fp32 [E], optional
 *   labels      uint8 [E], each < G
 *   D blob      G matrices D_g [ell][H], one after another; each = codes then
 *               fp16 scales [ell][H/32]. Q8 codes: int8 [ell][H]; Q4 codes:
 *               bytes [ell][H/2] holding q+8, element 2i in the low nibble.
 *               Q8: x ~ q * d; Q4: x ~ (nibble - 8) * d. Blocks of 32 run
 *               along the row (the input dimension).
 *   U blob      G matrices U_g [H][ell], same block layout.
 *   experts     E fixed-size NVFP4 records, each: gate codes [F][ell/2],
 *               up codes [F][ell/2], down codes [ell][F/2] (E2M1, element 2i
 *               in the low nibble), gate scales [F][ell/16], up scales
 *               [F][ell/16], down scales [ell][F/16] (E4M3, one per 16 along
 *               the row), tail: fp32 ts_gate, ts_up, ts_down, uint32 0.
 *               Weight = e2m1 * e4m3 * ts. Record = 3*ell*F*9/16 + 16 bytes
 *               (1,935,376 B at ell 1792, F 640).
 *   shared      bf16 gate [Fs][H], up [Fs][H], down [H][Fs].
 *
 * Errors: every entry point returns 0 or a negative LMOE_E* code; argument
 * errors are found on the host before any launch. Device-side faults surface
 * as LMOE_EHIP at a later call. lmoe_last_error() gives the last message of
 * the calling thread.
 *
 * Threads and streams: a handle is not thread-safe. Forward calls on one
 * handle must be ordered (one stream, or explicit events): they share the
 * handle's workspace.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LMOE_OK            0
#define LMOE_EINVAL       -1   /* bad argument: NULL, size, T out of range, label >= G */
#define LMOE_ENOMEM       -2   /* device allocation failed */
#define LMOE_EHIP         -3   /* a HIP runtime call failed */
#define LMOE_ESTATE       -4   /* forward before load_weights */
#define LMOE_EUNSUPPORTED -5   /* dimensions the kernels do not cover */

/* Expert record formats ("Edge0 145B and Edge0 120B", "Model profile" row
 * "Expert formats"; teardown "What is 4-bit"):
 *   LMOE_EXPERTS_NVFP4  the NVFP4 record described below
 *   LMOE_EXPERTS_Q3K    Q3_K gate and up, IQ4_NL down: gate blocks [F][latent/256]
 *                       then up blocks (GGML Q3_K, 110 bytes a 256-weight block:
 *                       high-bit mask, low bits, 12 bytes of 6-bit sub-block scales,
 *                       fp16 d), then down blocks [latent][F/32] (GGML IQ4_NL, 18
 *                       bytes a 32-weight block: fp16 d, 16 bytes of table
 *                       indices); 1,630,720 bytes at latent 1792, F 640.
 *                       latent % 256 == 0. Batches of T > 8 run as decode
 *                       forwards of 8 tokens each (no prefill workspace is
 *                       allocated); their lmoe_debug perm, expert_count,
 *                       expert_off and group_off are refused
 *                       (LMOE_EUNSUPPORTED). */
#define LMOE_EXPERTS_NVFP4 0
#define LMOE_EXPERTS_Q3K   1

/* Layer dimensions, validated by lmoe_create.
 * Constraints: hidden % 256 == 0, latent % 64 == 0, expert_ffn % 32 == 0,
 * shared_ffn % 32 == 0, hidden <= 4096, latent <= 4096, expert_ffn <= 4096,
 * shared_ffn <= 4096, 1 <= top_k <= min(n_experts, 64), n_experts <= 1024,
 * 1 <= n_groups <= 64, du_bits in {8, 4}, 1 <= max_tokens <= 1048576. */
typedef struct lmoe_dims {
  int32_t hidden;          /* H */
  int32_t latent;          /* ell */
  int32_t n_experts;       /* E */
  int32_t top_k;           /* K */
  int32_t n_groups;        /* G */
  int32_t expert_ffn;      /* F, SwiGLU width of a routed expert */
  int32_t shared_ffn;      /* Fs, SwiGLU width of the shared expert */
  int32_t du_bits;         /* 8 = Q8, 4 = Q4 ("D/U formats", LAYER) */
  int32_t max_tokens;      /* largest T a forward may take; sizes the workspace */
  int32_t has_router_bias; /* 1: lmoe_weights.router_bias is read */
  int32_t expert_format;   /* LMOE_EXPERTS_NVFP4 (0) or LMOE_EXPERTS_Q3K */
} lmoe_dims;

/* Packed weights (layouts above). Pointers may be host or device memory;
 * lmoe_load_weights copies what it needs and keeps no pointer. */
typedef struct lmoe_weights {
  const uint16_t* router_bf16;
  const float*    router_bias;          /* NULL unless has_router_bias */
  const uint8_t*  group_labels;
  const uint8_t*  d_blob;  size_t d_bytes;
  const uint8_t*  u_blob;  size_t u_bytes;
  const uint8_t*  experts; size_t expert_record_bytes;   /* E records */
  const uint16_t* shared_gate_bf16;
  const uint16_t* shared_up_bf16;
  const uint16_t* shared_down_bf16;
} lmoe_weights;

/* Optional intermediate outputs of lmoe_forward; DEVICE pointers, each may
 * be NULL. Written on the forward's stream. */
typedef struct lmoe_debug {
  int32_t* topk_idx;       /* [T][K] expert ids, descending logit, ties to lower id */
  float*   topk_w;         /* [T][K] renormalized softmax weights */
  int32_t* perm;           /* [T*K]: stable sort of a = t*K+k by (label, expert) */
  int32_t* expert_count;   /* [E] assignments per expert */
  int32_t* expert_off;     /* [E+1] exclusive scan of expert_count in expert-id
                              order: expert_off[e] = sum of expert_count[e']
                              over e' < e, expert_off[E] = T*K */
  int32_t* group_off;      /* [G+1] start of each group's segment in perm */
  float*   latent;         /* [T][G][ell] D_g x; entries of (t, g) pairs that
                              token t does not use are unspecified. On the
                              prefill path (T > 8, NVFP4 records) these are
                              the fp16 values the experts read, widened */
} lmoe_debug;

typedef struct lmoe lmoe_t;

/* Create a handle on HIP device `hip_device`: validates dims, allocates the
 * workspace for max_tokens. *out is set only on success.
 * Two paths serve a forward: T <= 8 tokens run the decode path (weights
 * streamed once per call through a GEMV on matrix cores); T > 8 the prefill
 * path (MFMA GEMMs over the sorted assignments). The prefill workspace
 * exists only when max_tokens > 8 (and the records are NVFP4); it takes about
 *   T * (6H + 4 Epad + 8 G ell + K (2F + 4 ell + 48) + 4 Fs) bytes
 * for T = max_tokens (Epad = E rounded up to 64), e.g. 0.68 GB at T 4096
 * for the 145B shapes, plus a bf16 copy of the router in two layouts. */
int lmoe_create(const lmoe_dims* dims, int hip_device, lmoe_t** out);

/* Copy and re-lay the packed weights into device memory owned by the handle
 * (the device layout is internal). Synchronous with respect to the host: the
 * source buffers may be reused when it returns. `hip_stream` orders the
 * copies (NULL = default stream). EINVAL on a size mismatch or a label >= G. */
int lmoe_load_weights(lmoe_t* h, const lmoe_weights* w, void* hip_stream);

/* y[T][H] = layer(x[T][H]); x and y are device fp32, row-major, not
 * aliased. 1 <= T <= max_tokens. Asynchronous on `hip_stream`. `dbg` may be
 * NULL. Top-K indices and the permutation are those of exact arithmetic
 * (fp64 rescoring wherever fp32 cannot decide); y carries the rounding of the
 * path's arithmetic (fp32 on the decode path; fp16 activations on the
 * prefill path). */
int lmoe_forward(lmoe_t* h, const float* x_dev, int32_t T, float* y_dev,
                 const lmoe_debug* dbg, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as lmoe_forward for T <= 8 tokens (the decode path, same kernels,
 * bit-identical y), with its workspace in a static device array of 16 MiB per
 * GPU instead of the handle's. It calls no allocator. All calls on one GPU
 * share that array: calls that overlap on one GPU (other streams, other
 * handles) race and must be ordered by the caller. x and y are device fp32
 * [T][H], not aliased. LMOE_EUNSUPPORTED for T > 8 or when the layer's
 * workspace at this T exceeds the array (it holds the 145B shapes at T 8
 * several times over); LMOE_EINVAL / LMOE_ESTATE as lmoe_forward. No debug
 * outputs. */
int lmoe_forward_noalloc(lmoe_t* h, const float* x, int32_t T, float* y, void* hip_stream);

/* One block of a pre-norm residual stack, in place on device memory:
 *   x += layer(RMSNorm(x)),  RMSNorm(v) = v / sqrt(mean(v^2) + eps), unit gain.
 * (The stack arrangement is this library's reading; the pages give none.) */
int lmoe_forward_block(lmoe_t* h, float* x_inout_dev, int32_t T, float rms_eps,
                       void* hip_stream);

/* Profiling hook: when `events` is non-NULL, each following lmoe_forward /
 * lmoe_forward_block of T tokens with lmoe_phase_count(T) == n - 1 records
 * events[0] on its stream before its first kernel and events[i] after its
 * i-th phase (hipEvent_t handles owned by the caller). Decode (T <= 8) has 4
 * phases: router + D + shared gate/up, expert gate/up, expert down,
 * combine + U + shared down (the per-group sums formed in U's staging).
 * Prefill has 8: staging + router + top-K; permutation; D; shared gate/up;
 * expert gate/up; expert down; combine; U + shared down. Forwards of the other path record nothing. NULL switches
 * it off. EINVAL unless n is 5 or 9. */
int lmoe_set_phase_events(lmoe_t* h, void* const* events, int32_t n);
int32_t lmoe_phase_count(int32_t T);

/* Profiling hook: runs phase `phase` (1 .. 4) of a decode forward of
 * T <= 8 tokens by itself on the stream. It reads what the handle's last
 * decode forward left in its workspace, which must have been an
 * lmoe_forward of the same T (else LMOE_ESTATE), and writes what that phase
 * writes there (phase 4: y, as lmoe_forward does). Calls back to back time
 * one kernel as a forward runs it. x: [T][H] as given to that forward;
 * y: [T][H] (written by phase 4 only). EINVAL: NULL or aliased x/y, phase
 * outside 1..4, T outside 1..8 or above max_tokens. */
int lmoe_run_phase(lmoe_t* h, const float* x, int32_t T, int32_t phase, float* y, void* stream);

/* Prefill D variant ("Edge0-145B: a Qwen MoE with its experts squeezed, and
 * a 51B table left on the SSD", section "A latent in front of the experts":
 * the reference engine runs D for every group): 1 (the default) computes
 * D_g x only for the (token, group) pairs the routing uses, after the
 * routing (per-group token lists, a gathered GEMM), with the shared gate/up
 * on a second stream; the debug latent rows of unused pairs are then not
 * written. 0 computes D_g x for all G groups of every token, on the second
 * stream beside the routing (the reference engine's form). y is the same up
 * to fp32 rounding order. Applies to forwards of T > 8 on a handle created
 * with max_tokens > 8; batches with T * hidden * 2 >= 2^31 always take the
 * all-groups form. EINVAL for a NULL handle or another value. */
int lmoe_set_prefill_d(lmoe_t* h, int32_t routed_only);

void lmoe_destroy(lmoe_t* h);

const char* lmoe_strerror(int code);
const char* lmoe_last_error(void);

/* Bytes of one packed NVFP4 expert record and of one packed D_g / U_g. */
size_t lmoe_expert_record_bytes(int32_t latent, int32_t expert_ffn);
/* Bytes of one record in expert format `fmt` (0 for an unknown format). */
size_t lmoe_expert_record_bytes_fmt(int32_t latent, int32_t expert_ffn, int32_t fmt);
size_t lmoe_du_matrix_bytes(int32_t rows, int32_t cols, int32_t du_bits);

/* ---- PLE n-gram embedding gather --------------------------------------------
 * "Edge0-145B: a Qwen MoE with its experts squeezed, and a 51B table left on
 * the SSD", section "The 51.2B the GPU never holds": 16 hash heads, heads
 * 0..7 over each token's 2-gram (previous token, token) and heads 8..15 over
 * its 3-gram, each naming one row of row_bytes E4M3 (OCP E4M3FN) values in
 * one table (160 bytes a row, 2,560 bytes a token at the Edge0 shapes).
 * The hash is this library's reading (the pages do not give it): head h's
 * row is mix64(key) mod head_rows[h], key = sum over the n-gram's ids, oldest
 * first, of (id + 1) * K[h][j] mod 2^64, where mix64 is the SplitMix64
 * output function and K[h][j] its output number 3h + j + 1 from seed 0;
 * head h's rows follow those of heads 0..h-1 in the table.
 *   tokens     DEVICE int32 [T + 2]: the two ids before the batch (-1 where
 *              the sequence has not started), then the T ids of the batch
 *   table      DEVICE bytes [sum of head_rows][row_bytes]
 *   head_rows  HOST int64 [16], each >= 1
 *   row_bytes  multiple of 16 in [16, 1024]
 *   out        DEVICE bf16 bit patterns [T][16][row_bytes]: the decoded
 *              values (exact; NaN codes give NaN)
 * Asynchronous on hip_stream; no handle, the calling thread's device.
 * EINVAL for a bad argument (T == 0 is a no-op). Ids are hashed as given. */
int lmoe_ple_gather(const int32_t* tokens, int32_t T, const uint8_t* table,
                    const int64_t* head_rows, int32_t row_bytes, uint16_t* out,
                    void* hip_stream);

/* ---- Device-side packing of fp32 masters into the formats above ----------
 * For callers holding unquantized weights on the GPU. All pointers are
 * DEVICE memory; asynchronous on `hip_stream`. Rounding is to nearest, ties
 * to even, saturating:
 *   bf16:  RNE of each fp32 value.
 *   Q8/Q4: per 32 along the row, d = fp16(amax/127) (Q4: amax/7),
 *          q = clamp(round(x/d), -127, 127) (Q4: [-8, 7]); d == 0 -> q = 0.
 *   NVFP4: per matrix ts = fp32(amax/(6*448)) (1 for an all-zero matrix); per
 *          16 along the row s = E4M3(amax16/(6*ts)) saturating at 448;
 *          q = E2M1(x/(s*ts)) saturating at 6, magnitude 0 stored as +0.
 * These readings of the formats are this library's; the pages give only the
 * element and scale types and the block sizes. */
int lmoe_pack_bf16(const float* src, size_t n, uint16_t* dst, void* hip_stream);
/* One matrix [rows][cols] (cols % 32 == 0) into codes then fp16 scales, i.e.
 * lmoe_du_matrix_bytes(rows, cols, bits) bytes at dst. */
int lmoe_pack_blocks(const float* src, int32_t rows, int32_t cols, int32_t du_bits,
                     uint8_t* dst, void* hip_stream);
/* n expert records from gate [n][F][ell], up [n][F][ell], down [n][ell][F]
 * into dst (n * lmoe_expert_record_bytes(ell, F) bytes). */
int lmoe_pack_expert_records(const float* gate, const float* up, const float* down,
                             int32_t n, int32_t latent, int32_t expert_ffn,
                             uint8_t* dst, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* LMOE_H */
