/*
 * moe_mxfp4.h - C ABI of the routed MoE layer on MXFP4 expert weights (gfx950).
 *
 * What the layer computes (one call = N token rows):
 *   z[r][e]  = sum_i x[r][i] * W_r[e][i] (+ bias[e])          router logits
 *   s[r][e]  = sqrt(softplus(z[r][e]))                          router scores
 *   sel(r)   = the k experts with the largest s (top-k mode), or
 *              tid2eid[token_ids[r]][0..k) (hash mode); listed in ascending id
 *   g[r][j]  = s[r][sel_j] / sum_j' s[r][sel_j']                gates, sum 1
 *   FFN_e(v) = W_down[e] (silu(min(W_gate[e] v, L)) * clamp(W_up[e] v, -L, L))
 *   out[r]   = FFN_shared(x[r]) + route_scale * sum_j g[r][j] FFN_{sel_j}(x[r])
 * Optionally the layer first normalises its input, x <- RMSNorm(x) (norm_w),
 * and adds a residual row to its output (residual); see moe_args_t.
 * Sources (pages on DeepSeek V4 Flash):
 *   - top-6 of 256 routed experts plus one shared expert, sqrt-softplus routing
 *     with hash layers: TensorSharp "DeepSeek V4 Flash (deepseek4)", intro and
 *     "How TensorSharp runs it";
 *   - top-k = 6, hash routing, route_scale, swiglu_limit = 10: aimarketly model
 *     card "Deepseek-V4-Flash-Dspark-FST", "Model Architecture and Objective";
 *   - router weight/bias and per-expert w1/w2/w3 tensors plus shared experts:
 *     ds4 issue "DeepSeek-V4-Flash-DSpark", "Loader spec";
 *   - MXFP4 experts as 32-value blocks with one e8m0 scale: model card
 *     "Preprocessing"; FaStar README "Expert virtual memory"; TensorSharp
 *     "Getting a drafter" (per-32 E8M0 scales);
 *   - the weighted-sum epilogue over the selected experts: TensorSharp
 *     "Fitting the model" (moe_scatter_add); shared and routed FFN paths: pypto
 *     "DeepSeek V4-Flash, DSpark point", "MoE and output stages".
 * The pages do not fix gate normalisation, the placement of the swiglu clamp
 * or the bias semantics; this library normalises the selected scores to sum
 * 1, clamps the gate from above and the up projection on both sides at L, and
 * adds the bias to the logit before the score (or, with bias_mode
 * MOE_BIAS_SELECT, to the score for the selection only).
 *
 * Conventions for every entry point:
 *   - Return 0 (MOE_OK) or a negative MOE_ERR_* code.  Argument validation is
 *     done on the host before anything is enqueued: on error nothing runs.
 *   - Device pointers are caller-owned and must stay valid until the stream
 *     has executed the work; the library keeps no pointer after returning.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  No allocation, no host<->device copy, no host synchronisation.
 *   - Results are bitwise reproducible for identical inputs and sizes.
 *   - Concurrent calls are safe when their workspaces and outputs differ.
 *   - Buffers the layer writes (out, the workspace, the optional routing
 *     outputs) must not overlap any other buffer of the call: inputs, packed
 *     weights (each weight set over its full packed size), hash-mode token
 *     ids and the whole tid2eid table, or each other.  The one exception is a
 *     residual that is `out` itself.  Inputs may overlap each other.  A call
 *     that breaks this returns MOE_ERR_INVALID and enqueues nothing.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MXFP4_VERSION 5

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* null/misaligned pointer, bad enum, aliasing output */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported range */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  MOE_ERR_HIP = -4,         /* a HIP launch failed */
  MOE_ERR_SCRATCH = -5      /* moe_layer_forward_noalloc: the call needs more scratch than the library holds */
};

enum { MOE_ROUTING_TOPK = 0, MOE_ROUTING_HASH = 1 };
enum { MOE_BIAS_LOGIT = 0, MOE_BIAS_SELECT = 1 };
enum { MOE_SHARED_MXFP4 = 0, MOE_SHARED_BF16 = 1 };
enum { MOE_EXPERTS_MXFP4 = 0, MOE_EXPERTS_Q2K = 1 };

/* Supported shapes: d_model and d_ff multiples of 128 (>= 128, <= 65536),
 * 1 <= n_experts <= 1024, 1 <= top_k <= min(8, n_experts),
 * 0 <= n_rows <= MOE_MAX_ROWS. */
#define MOE_MAX_ROWS (1 << 20)

typedef struct moe_config {
  int32_t d_model;      /* d: hidden size */
  int32_t d_ff;         /* I: expert intermediate size */
  int32_t n_experts;    /* E: routed experts */
  int32_t top_k;        /* k: experts per row */
  int32_t routing;      /* MOE_ROUTING_TOPK or MOE_ROUTING_HASH */
  int32_t has_shared;   /* 1: one shared expert on every row; 0: none */
  float route_scale;    /* multiplies the routed sum only (1.0 = plain sum) */
  float swiglu_limit;   /* L; <= 0 disables the clamp */
  float norm_eps;       /* eps of the input RMSNorm (used when moe_args_t.norm_w != NULL); >= 0 */
  int32_t bias_mode;    /* router_bias: 0 (MOE_BIAS_LOGIT) added to the logits, so it shifts both the
                           selection and the gates; 1 (MOE_BIAS_SELECT) added to the scores for the
                           top-k selection only, the gates use the unbiased scores.  The pages name the
                           bias (gate.bias, ds4 issue "Loader spec") but not its use. */
  int32_t shared_format; /* weights of the shared expert: MOE_SHARED_MXFP4 (packed like the routed
                           experts, sh_*_q/s) or MOE_SHARED_BF16 (plain bf16 matrices, sh_*_w).  The
                           model card ("Preprocessing"; "Model Architecture and Objective") keeps the
                           expert blocks in MXFP4 and the shared tensors in Q8_0/BF16 without saying on
                           which side the per-layer shared expert falls; both are supported. */
  int32_t expert_format; /* weights of the routed experts: MOE_EXPERTS_MXFP4 (packed MXFP4, w.*_q and
                           w.*_s) or MOE_EXPERTS_Q2K (packed Q2_K, w.gate_q/up_q/down_q only; see
                           moe_pack_q2k).  Q2_K needs d and I multiples of 256 and a shared expert, if
                           any, in bf16 (MOE_SHARED_BF16); otherwise MOE_ERR_UNSUPPORTED.  TensorSharp
                           "Getting a drafter" names q2_k as the drafter's routed-expert type. */
} moe_config_t;

/*
 * Routed experts in the library's packed layout: MXFP4 (moe_pack_mxfp4) or,
 * with expert_format MOE_EXPERTS_Q2K, Q2_K (moe_pack_q2k, *_q pointers only,
 * 16-byte aligned, the *_s pointers ignored).  An MXFP4 matrix: a
 * matrix [rows][K] of E2M1 values with one E8M0 scale per 32 consecutive
 * values along K.  Each group of n_mat matrices is stored back to back.
 *   gate, up : routed, n_mat = E, each [I][d]   (w1 and w3 of each expert)
 *   down     : routed, n_mat = E, each [d][I]   (w2)
 *   sh_*_q/s : the shared expert, n_mat = 1 (used when has_shared == 1 and
 *              shared_format == MOE_SHARED_MXFP4)
 * q pointers 16-byte aligned, s pointers 4-byte aligned.
 * sh_*_w: the shared expert in bf16, row-major with K contiguous (used when
 * has_shared == 1 and shared_format == MOE_SHARED_BF16, else ignored):
 *   sh_gate_w, sh_up_w [I][d];  sh_down_w [d][I];  16-byte aligned.
 */
typedef struct moe_weights {
  const void *gate_q, *gate_s;
  const void *up_q, *up_s;
  const void *down_q, *down_s;
  const void *sh_gate_q, *sh_gate_s;
  const void *sh_up_q, *sh_up_s;
  const void *sh_down_q, *sh_down_s;
  const void *sh_gate_w, *sh_up_w, *sh_down_w;
} moe_weights_t;

typedef struct moe_args {
  int32_t n_rows;             /* N >= 0; N == 0 returns MOE_OK and enqueues nothing */
  const void* x;              /* bf16 [N][d], row-major, 16-byte aligned */
  const float* router_w;      /* fp32 [E][d], row-major, 16-byte aligned */
  const float* router_bias;   /* fp32 [E] added to the logits, or NULL */
  const int32_t* token_ids;   /* hash mode: int32 [N], each in [0, vocab) */
  const int32_t* tid2eid;     /* hash mode: int32 [vocab][k], k distinct ids in [0, E) per row.
                                 Invalid entries give an unspecified routing but never an
                                 out-of-bounds access (token and expert ids are clamped) */
  int64_t vocab;              /* hash mode: rows of tid2eid */
  moe_weights_t w;            /* packed expert weights */
  void* out;                  /* bf16 [N][d], 16-byte aligned; must not overlap x or any other buffer */
  /* Optional outputs (NULL to skip), for inspection of the routing:
   *   topk_idx [N][k] int32 ascending expert ids;  topk_w [N][k] fp32 gates;
   *   counts [E] rows per expert; offsets [E+1] exclusive prefix sum of counts;
   *   perm [N*k]: pair index r*k+j at each expert-major position (rows ascending
   *   within an expert); inv [N*k]: position of pair r*k+j. */
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  void* workspace;            /* device scratch, 256-byte aligned, >= moe_workspace_size(); must not
                                 overlap any other buffer of the call */
  size_t workspace_bytes;
  /* Optional stage timing (NULL to skip): MOE_N_STAGE_EVENTS hipEvent_t handles
   * created by the caller.  Event i is recorded on `stream` just before stage i
   * and the last one after the final stage; a NULL entry is not recorded
   * (each recorded event costs several microseconds of stream time, about 9 us
   * measured on MI355X between two kernels).  The
   * stages are 0 router logits + activation split, 1 top-k/hash selection +
   * routing bookkeeping, 2 gate/up GEMM, 3 down GEMM, 4 combine (a bf16 shared
   * expert's GEMMs run in stages 2 and 3). */
  void* const* stage_events;
  /* Input RMSNorm (the FFN input norm: ffn_norm in the ds4 issue's loader
   * spec; the rmsnorm step of the pypto DSpark pipeline).  norm_w: bf16 [d],
   * 16-byte aligned, or NULL (x is used as given).  The layer then runs on
   *   x'[r][i] = bf16((x[r][i] * rs[r]) * norm_w[i]),  rs[r] = 1/sqrt(sum_i x[r][i]^2 / d + norm_eps),
   * computed in fp32 and rounded once to nearest even, as an unfused bf16
   * pipeline would store it (the pages fix neither precision nor eps). */
  const void* norm_w;
  /* Residual: bf16 [N][d], 16-byte aligned, or NULL.  out[r] = bf16(residual[r]
   * + layer output), added in fp32 before the one rounding.  It may be `out`
   * itself (in-place update) or x, but not overlap `out` partially. */
  const void* residual;
  /* Optional (ABI version 5), with shared_format MOE_SHARED_BF16: the three
   * bf16 shared matrices also packed by moe_pack_bf16 into one buffer, back to
   * back: gate [I][d] at byte 0, up [I][d] at I*d*2, down [d][I] at 2*I*d*2
   * (3*I*d*2 bytes, 16-byte aligned), or NULL.  For batches of at least
   * MOE_SHARED_STREAM_ROWS rows with d % 512 == 0 and I % 256 == 0 the layer
   * then streams these fragments per wave instead of tiling sh_*_w through LDS
   * (the same values in the same summation order: identical results); sh_*_w
   * are still required. */
  const void* sh_packed;
} moe_args_t;

#define MOE_SHARED_STREAM_ROWS 2048

#define MOE_N_STAGES 5  /* the input RMSNorm, when asked for, belongs to stage 0 */
#define MOE_N_STAGE_EVENTS (MOE_N_STAGES + 1)

/* Library version (MOE_MXFP4_VERSION). */
int moe_version(void);

/* Static text for a status code (never NULL). */
const char* moe_status_string(int status);

/*
 * Bytes of one packed MXFP4 matrix [rows][K]: rows % 16 == 0, K % 128 == 0.
 * q_bytes = rows*K/2; s_bytes = (rows/16) * ceil(K/512) * 256.
 */
int moe_packed_mxfp4_bytes(int32_t rows, int32_t K, size_t* q_bytes, size_t* s_bytes);

/*
 * Re-lay n_mat MXFP4 matrices from the natural layout to the packed layout
 * (same values, one-time weight preparation, e.g. at checkpoint load).
 * Natural layout (device pointers): q [n_mat][rows][K/2] with element 2t in the
 * low nibble of byte t, s [n_mat][rows][K/32], one E8M0 byte per 32 values.
 * Packed layout, per matrix, with nks = K/128 and n_sg = ceil(nks/4):
 *   q_out: fragment (rt, ks) for rt < rows/16, ks < nks, at byte
 *          (rt*nks + ks)*1024; its lane l (0..63) holds 16 bytes = the 32
 *          values of row 16*rt + l%16 in the 32-block 4*ks + l/16.
 *   s_out: group (rt, sg) at byte (rt*n_sg + sg)*256; lane l holds 4 bytes,
 *          byte j = the scale of row 16*rt + l%16, 32-block 4*(4*sg + j) + l/16
 *          (127 where 4*sg + j >= nks).
 * q/q_out 16-byte aligned, s/s_out 4-byte aligned; outputs must not overlap
 * inputs.  Asynchronous on `stream`.
 */
int moe_pack_mxfp4(const void* q, const void* s, int32_t n_mat, int32_t rows, int32_t K, void* q_out,
                   void* s_out, void* stream);

/*
 * Q2_K matrices (MOE_EXPERTS_Q2K): GGUF's Q2_K super-blocks, 256 values of a
 * row in 84 bytes (the pages name the type, not its layout): bytes 0..15 one
 * byte per 16-value sub-block (scale in the low nibble, min in the high
 * nibble), bytes 16..79 the 2-bit quants (the block's two 128-value halves 32
 * bytes each; value 32j + i of a half in bits 2j..2j+1 of the half's byte i),
 * bytes 80..83 fp16 d then fp16 dmin; a value is d * scale * q - dmin * min.
 *
 * Bytes of one Q2_K matrix [rows][K], natural or packed (the same size):
 * rows * (K/256) * 84; rows % 16 == 0, K % 256 == 0.
 */
int moe_q2k_bytes(int32_t rows, int32_t K, size_t* bytes);

/*
 * Re-lay n_mat Q2_K matrices from the natural layout [n_mat][rows][K/256][84]
 * (row-major super-blocks) to the packed layout the layer reads (same values,
 * one-time weight preparation).  Packed, per matrix: the 16-row tile rt and
 * super-block b at byte (rt*(K/256) + b)*1344, holding
 *   [0, 1024)    lane l (0..63): quant bytes 8g..8g+7 of both halves (natural
 *                bytes 16+8g..+7 then 48+8g..+7) of row 16*rt + l%16, g = l/16;
 *   [1024, 1280) the 16 scale/min bytes of each of the 16 rows;
 *   [1280, 1344) d and dmin (4 bytes) of each of the 16 rows.
 * q 4-byte aligned, q_out 16-byte aligned, not overlapping.  Asynchronous on
 * `stream`.
 */
int moe_pack_q2k(const void* q, int32_t n_mat, int32_t rows, int32_t K, void* q_out, void* stream);

/*
 * Re-lay n_mat bf16 matrices [rows][K] (row-major, K contiguous) into the
 * fragment order of the bf16 matrix instruction (one-time weight preparation,
 * for moe_args_t.sh_packed): per matrix, fragment (rt, ks) for rt < rows/16,
 * ks < K/32 at byte (rt*(K/32) + ks)*1024; its lane l (0..63) holds 16 bytes =
 * the 8 values of row 16*rt + l%16 at columns 32*ks + 8*(l/16) .. +7.  Packed
 * size = natural size (rows*K*2 bytes per matrix).  rows % 16 == 0, K % 32 ==
 * 0 (each 16 .. 65536), else MOE_ERR_UNSUPPORTED; w and out 16-byte aligned,
 * not overlapping.  Asynchronous on `stream`.  The shared expert's gate and up
 * are [I][d] (rows I, K d), its down [d][I] (rows d, K I).
 */
int moe_pack_bf16(const void* w, int32_t n_mat, int32_t rows, int32_t K, void* out, void* stream);

/* Device workspace bytes that moe_layer_forward needs for n_rows rows. */
int moe_workspace_size(const moe_config_t* cfg, int32_t n_rows, size_t* bytes);

/* The whole layer (router, routing bookkeeping, expert FFNs, combine) on `stream`. */
int moe_layer_forward(const moe_config_t* cfg, const moe_args_t* args, void* stream);

/*
 * moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The layer runs on a static device array
 * of the library, MOE_NOALLOC_SCRATCH_BYTES per GPU, held from the library's
 * load until the process ends; this call allocates nothing and frees nothing.
 *   - args->workspace must be NULL and args->workspace_bytes 0 (else
 *     MOE_ERR_INVALID); every other argument as for moe_layer_forward.
 *   - A call is accepted when moe_workspace_size(cfg, n_rows) <=
 *     MOE_NOALLOC_SCRATCH_BYTES (at d 4096, I 2048, 256 experts top-6 + 1
 *     MXFP4 shared expert: up to 598 rows); a larger one returns
 *     MOE_ERR_SCRATCH and enqueues nothing.
 *   - Every call on one GPU uses that GPU's one scratch array: calls that can
 *     overlap in time on one GPU (different streams without ordering, or
 *     several host threads) race and give undefined results.  Order them on
 *     one stream or with events.  The array keeps the last call's contents;
 *     each call re-initialises what it reads.
 *   - The first call on each device looks up that device's copy of the array
 *     (hipGetSymbolAddress, no allocation); a failure returns MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (96u << 20)
int moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_args_t* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
