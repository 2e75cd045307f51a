/*
 * beam_moe.h -- C ABI of the Beam-1.0 mixture-of-experts block on one
 * AMD Instinct MI355X (gfx950).
 *
 * The block ("Welcome Beam: a 501B open model you can own, customize, and
 * scale", section "Mixture of Experts"; "Beam 1.0" miles recipes, section 1
 * "Model Introduction"):
 *   1. router GEMM in FP32 (router weights are kept in FP32; the same page's
 *      section "Residual Stream" lists the router among the FP32 computations),
 *   2. sigmoid score for every expert,
 *   3. experts split into num_groups contiguous groups; each group scored by the
 *      sum of its two best scores; the topk_groups best groups are kept,
 *   4. the topk best experts inside the kept groups are chosen,
 *   5. each chosen expert is a SwiGLU MLP (gate/up projection, SiLU(gate)*up
 *      in FP32, down projection), with no shared expert,
 *   6. the token's output is the sum of its experts' outputs, each weighted by
 *      its score over the sum of the chosen scores, times routed_scaling (2.5).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory; scratch space comes from the
 *     caller's workspace (size from moe_workspace_bytes).
 *   - bf16 tensors are passed as uint16_t bit patterns.  All tensors are dense
 *     row-major with the layouts stated per argument.  Tensor pointers and the
 *     workspace must be 16-byte aligned.
 *   - Every call validates its arguments on the host first.  On any error it
 *     enqueues nothing and returns a negative status; MOE_OK (0) otherwise.
 *     num_tokens == 0 is a valid no-op.  A failed kernel launch returns
 *     MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation of `stream`.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call never synchronises it.  Calls that share a workspace must be
 *     ordered on one stream.
 *   - Results are bitwise deterministic: no floating-point atomics.  They do
 *     not depend on the number of workgroups of the persistent expert GEMMs
 *     either; the environment variable BEAM_MOE_MAX_GRID=<n>, read at each
 *     launch, caps that number (for testing this).
 *   - Supported shapes: num_experts == 256; num_groups a power of two in
 *     [1, 64]; 1 <= topk_groups <= num_groups; 1 <= topk <= 8 and topk not
 *     above the experts in the kept groups; hidden a multiple of 256;
 *     intermediate a multiple of 128; num_tokens * topk < 2^31.  Other shapes return
 *     MOE_ERR_UNSUPPORTED.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, negative size, misalignment     */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside the shapes listed above     */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required    */
  MOE_ERR_HIP = -4,          /* HIP runtime error (no device, launch failure) */
  MOE_ERR_TOO_LARGE = -5     /* moe_layer_forward_noalloc: the call needs more
                                scratch than the library's static array holds */
};

/* Which entry point a workspace size is asked for. */
enum moe_entry {
  MOE_ENTRY_ROUTE = 0,
  MOE_ENTRY_PERMUTE = 1,
  MOE_ENTRY_EXPERT_FFN = 2,
  MOE_ENTRY_LAYER = 3,
  MOE_ENTRY_EXPERT_STAGE = 4,  /* moe_expert_gate_up or moe_expert_down */
  MOE_ENTRY_EXPERT_FFN_LORA = 5,
  MOE_ENTRY_LAYER_LORA = 6
};

typedef struct moe_config {
  int64_t num_tokens;     /* T >= 0 tokens in this call                           */
  int32_t hidden;         /* H: 5120 for Beam-1.0                                 */
  int32_t intermediate;   /* I: SwiGLU intermediate size, 2560 for Beam-1.0       */
  int32_t num_experts;    /* E = 256                                              */
  int32_t num_groups;     /* G = 8 groups of E/G contiguous experts               */
  int32_t topk_groups;    /* groups kept per token, 4                             */
  int32_t topk;           /* experts per token, 8                                 */
  int32_t renormalize;    /* 1: combine weight = score / sum of the topk chosen
                             scores (weights that sum to one); 0: raw score       */
  float routed_scaling;   /* factor applied to the combined output, 2.5          */
  int32_t weight_layout;  /* expert weight storage: MOE_LAYOUT_ROW_MAJOR or
                             MOE_LAYOUT_PACKED (written by moe_pack_weights) for
                             the bf16 expert calls, MOE_LAYOUT_FP8_PACKED for the
                             *_fp8 calls; calls that read no expert weights
                             accept any of the three                              */
} moe_config_t;

/* Expert weight layouts. */
enum moe_weight_layout {
  MOE_LAYOUT_ROW_MAJOR = 0,  /* w_gate_up [E, 2I, H], w_down [E, H, I], row-major    */
  MOE_LAYOUT_PACKED = 1,     /* same sizes, each expert's [N, K] matrix stored as
                                [N/16][K/32][64][8]: the 16 x 32 bf16 operand tiles of
                                the gfx950 matrix cores, lane-ordered, consecutive
                                along K (see moe_pack_weights)                        */
  MOE_LAYOUT_FP8_PACKED = 2  /* E4M3FN codes plus fp32 per-row scales (see
                                moe_quantize_fp8)                                     */
};

/* Bytes of workspace `entry` needs for `cfg` (written to *bytes). */
int moe_workspace_bytes(const moe_config_t* cfg, int entry, size_t* bytes);

/*
 * Router: logits = x . W_r^T in FP32 (bf16 inputs widened exactly), scores =
 * sigmoid(logits), group-limited top-k selection, combine weights.
 *   x         [T, H] bf16
 *   w_router  [E, H] fp32, one row per expert
 *   sel_bias  [E] fp32 or NULL: added to the scores for choosing only (the
 *             checkpoint's FP32 "expert biases" read as a selection bias); the
 *             combine weights always use the unbiased scores
 *   topk_ids  [T, topk] int32 out, ordered by (selection value desc, id asc)
 *   topk_w    [T, topk] fp32 out, combine weights WITHOUT routed_scaling
 * Ties between equal values go to the lower group / expert index.
 */
int moe_route(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
              const float* sel_bias, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routing replay: recompute scores and combine weights for caller-supplied
 * expert ids (e.g. recorded at rollout time), skipping selection.
 *   topk_ids  [T, topk] int32 in; an id outside [0, E) names no expert and is
 *             dropped, as moe_permute drops it: its weight is 0 and it is left
 *             out of the normalising sum (a token with no valid id gets all
 *             weights 0)
 *   topk_w    [T, topk] fp32 out
 * Replayed ids then go through moe_permute, the expert calls and moe_combine,
 * where a dropped slot contributes nothing.
 */
int moe_route_replay(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                     const int32_t* topk_ids, float* topk_w,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token permutation and per-expert histogram (stable counting sort of the
 * T*topk (token, slot) pairs by expert).
 *   topk_ids  [T, topk] int32 in; ids outside [0, E) are dropped (their
 *             perm_dst entry is -1 and they are not counted)
 *   counts    [E] int32 out: pairs routed to each expert
 *   offsets   [E + 1] int32 out: exclusive prefix sum of counts
 *   perm_src  [T*topk] int32 out: row r of the expert-major order holds pair
 *             perm_src[r] = t*topk + j; rows of one expert ascend in t
 *   perm_dst  [T*topk] int32 out: inverse, perm_dst[t*topk + j] = r
 */
int moe_permute(const moe_config_t* cfg, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* perm_src, int32_t* perm_dst,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expert SwiGLU MLPs over the permuted rows (bf16 grouped GEMMs with FP32
 * accumulation; SiLU(gate)*up in FP32, rounded to bf16 before the down GEMM).
 *   x          [T, H] bf16; row r reads token perm_src[r] / topk
 *   perm_src   [T*topk] int32, offsets [E + 1] int32 (from moe_permute)
 *   w_gate_up  [E, 2*I, H] bf16: rows [0, I) gate, rows [I, 2I) up
 *   w_down     [E, H, I] bf16
 *   (both in cfg->weight_layout)
 *   y_perm     [T*topk, H] bf16 out, expert-major row order
 * Experts with no rows read no weights.
 */
int moe_expert_ffn(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                   const int32_t* offsets, const uint16_t* w_gate_up, const uint16_t* w_down,
                   uint16_t* y_perm, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of moe_expert_ffn, for callers that time or schedule them
 * separately (same kernels, same results).
 *   moe_expert_gate_up: h [T*topk, I] bf16 out = bf16(SiLU(x_r . Wg^T) * (x_r . Wu^T))
 *   moe_expert_down:    y_perm [T*topk, H] bf16 out = bf16(h_r . Wd^T)
 * Each builds its own m-tile plan from `offsets` in its workspace
 * (moe_workspace_bytes with MOE_ENTRY_EXPERT_STAGE).
 */
int moe_expert_gate_up(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                       const int32_t* offsets, const uint16_t* w_gate_up, uint16_t* h,
                       void* workspace, size_t workspace_bytes, void* stream);
int moe_expert_down(const moe_config_t* cfg, const uint16_t* h, const int32_t* offsets,
                    const uint16_t* w_down, uint16_t* y_perm,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Weighted un-permute: out[t] = bf16(routed_scaling * sum_j topk_w[t, j] *
 * y_perm[perm_dst[t*topk + j]]), summed in FP32 in slot order.  Slots with
 * perm_dst < 0 contribute nothing.
 *   out  [T, H] bf16 out
 */
int moe_combine(const moe_config_t* cfg, const uint16_t* y_perm, const int32_t* perm_dst,
                const float* topk_w, uint16_t* out, void* stream);

/*
 * The whole block: route, permute, expert MLPs, combine.
 *   out           [T, H] bf16 out
 *   topk_ids_out  [T, topk] int32 out or NULL
 *   topk_w_out    [T, topk] fp32 out or NULL
 */
int moe_layer_forward(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                      const float* sel_bias, const uint16_t* w_gate_up, const uint16_t* w_down,
                      uint16_t* out, int32_t* topk_ids_out, float* topk_w_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with no workspace argument.  The
 * scratch comes from a static device array of 128 MiB inside the library, one
 * per GPU it runs on, held until the process ends; the call allocates nothing.
 *   - It serves configurations whose moe_workspace_bytes(MOE_ENTRY_LAYER) is at
 *     most 128 MiB (at the Beam shape, hidden 5120 and intermediate 2560:
 *     batches of up to 1,090 tokens); larger ones return MOE_ERR_TOO_LARGE
 *     and enqueue nothing.
 *   - It uses the array of the current device; `stream` must belong to it.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind: calls that overlap on one GPU (on different streams, or from
 *     several threads without ordering) race.  Order them on one stream.
 * Other arguments are those of moe_layer_forward.
 */
int moe_layer_forward_noalloc(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                              const float* sel_bias, const uint16_t* w_gate_up,
                              const uint16_t* w_down, uint16_t* out, int32_t* topk_ids_out,
                              float* topk_w_out, void* stream);

/*
 * Rewrites expert weights from MOE_LAYOUT_ROW_MAJOR into MOE_LAYOUT_PACKED
 * (a pure permutation of each expert's elements; run once at load time).
 *   w_gate_up, w_down            row-major inputs (shapes as above)
 *   packed_gate_up, packed_down  outputs of the same sizes; must not overlap
 *                                the inputs
 * Either pair may be NULL to skip it.  num_tokens and weight_layout are
 * ignored.
 */
int moe_pack_weights(const moe_config_t* cfg, const uint16_t* w_gate_up, const uint16_t* w_down,
                     uint16_t* packed_gate_up, uint16_t* packed_down, void* stream);

/*
 * FP8 per-channel expert weights (vLLM recipe JSON "Beam-1.0-501B-A23B",
 * precision variant fp8: FP8 per-channel weights, router unquantized).
 *
 * Each expert matrix row n (output channel) has one fp32 scale s[n] and
 * E4M3FN codes q[n, k] (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite value 448); the matrix the GEMMs use is
 * w[n, k] = s[n] * q[n, k].  Activations stay bf16, accumulation fp32, and
 * the scale multiplies the fp32 accumulator of its output column.  The
 * router, selection, permutation and combine are the bf16 path's.
 *
 * Code layout (MOE_LAYOUT_FP8_PACKED): each expert's [N, K] code matrix is
 * stored as [N/16][K/64][2][64][8] bytes; entry (b, s, h, l) holds the codes
 * of row 16b + l%16 at k = 64s + 32h + 8(l/16) .. +7.  Scales are plain
 * fp32 [E, N].
 *   q_gate_up [E, 2*I, H] codes, s_gate_up [E, 2*I]
 *   q_down    [E, H, I]   codes, s_down    [E, H]
 * The *_fp8 calls require cfg->weight_layout == MOE_LAYOUT_FP8_PACKED (else
 * MOE_ERR_INVALID_ARG).  Their workspace sizes are the ones moe_workspace_bytes
 * gives for MOE_ENTRY_EXPERT_FFN, MOE_ENTRY_EXPERT_STAGE and MOE_ENTRY_LAYER.
 */
/*
 * Quantise row-major bf16 expert weights: s[n] = fp32(max_k |w[n, k]|) / 448
 * in fp32 (1 for an all-zero row); q[n, k] = E4M3FN(clamp(w[n, k] / s[n],
 * -448, 448)) with fp32 division and round-to-nearest-even (ties to the even
 * code); codes are written in MOE_LAYOUT_FP8_PACKED.
 *   w_gate_up, w_down  row-major bf16 inputs [E, 2I, H], [E, H, I]
 *   q_*, s_*           outputs as above; must not overlap the inputs
 * Either set (w, q, s) may be all NULL to skip it.  num_tokens and
 * weight_layout are ignored.
 */
int moe_quantize_fp8(const moe_config_t* cfg, const uint16_t* w_gate_up, const uint16_t* w_down,
                     uint8_t* q_gate_up, float* s_gate_up, uint8_t* q_down, float* s_down,
                     void* stream);

/* moe_expert_ffn, moe_expert_gate_up, moe_expert_down and moe_layer_forward
 * with FP8 expert weights (arguments as in those calls). */
int moe_expert_ffn_fp8(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                       const int32_t* offsets, const uint8_t* q_gate_up, const float* s_gate_up,
                       const uint8_t* q_down, const float* s_down, uint16_t* y_perm,
                       void* workspace, size_t workspace_bytes, void* stream);
int moe_expert_gate_up_fp8(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                           const int32_t* offsets, const uint8_t* q_gate_up,
                           const float* s_gate_up, uint16_t* h,
                           void* workspace, size_t workspace_bytes, void* stream);
int moe_expert_down_fp8(const moe_config_t* cfg, const uint16_t* h, const int32_t* offsets,
                        const uint8_t* q_down, const float* s_down, uint16_t* y_perm,
                        void* workspace, size_t workspace_bytes, void* stream);
int moe_layer_forward_fp8(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                          const float* sel_bias, const uint8_t* q_gate_up, const float* s_gate_up,
                          const uint8_t* q_down, const float* s_down, uint16_t* out,
                          int32_t* topk_ids_out, float* topk_w_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expert LoRA ("Beam 1.0" miles recipes, section 5.5 "LoRA": an adapter of
 * rank 16 and alpha 32 on every routed expert, router frozen).  Each expert's
 * fused gate/up weight and its down weight carry one adapter; an adapted
 * weight W [out, in] computes W a + scale * B (A a).  The rank-wide first
 * factor is rounded once to bf16 after scaling: t = bf16(scale * fp32(a . A^T));
 * the second factor t . B^T accumulates in fp32 with the base GEMM before the
 * SwiGLU (gate/up) or the output rounding (down).  The down adapter reads the
 * bf16 h the base down GEMM reads.
 */
typedef struct moe_lora {
  const uint16_t* a_gate_up;  /* [E, r, H] bf16 row-major  */
  const uint16_t* b_gate_up;  /* [E, 2I, r] bf16 (rows as in w_gate_up: gate, then up) */
  const uint16_t* a_down;     /* [E, r, I] bf16            */
  const uint16_t* b_down;     /* [E, H, r] bf16            */
  int32_t rank;               /* r in {16, 32, 48, 64}; Beam's recipe uses 16 */
  float scale;                /* alpha / r; Beam's recipe: 32 / 16 = 2 */
} moe_lora_t;

/*
 * moe_expert_ffn and moe_layer_forward with expert LoRA on bf16 base weights
 * (base weights in cfg->weight_layout; adapters row-major, 16-byte aligned).
 * Workspace: MOE_ENTRY_EXPERT_FFN_LORA / MOE_ENTRY_LAYER_LORA.  A missing or
 * malformed `lora` returns MOE_ERR_INVALID_ARG.
 */
int moe_expert_ffn_lora(const moe_config_t* cfg, const uint16_t* x, const int32_t* perm_src,
                        const int32_t* offsets, const uint16_t* w_gate_up, const uint16_t* w_down,
                        const moe_lora_t* lora, uint16_t* y_perm,
                        void* workspace, size_t workspace_bytes, void* stream);
int moe_layer_forward_lora(const moe_config_t* cfg, const uint16_t* x, const float* w_router,
                           const float* sel_bias, const uint16_t* w_gate_up,
                           const uint16_t* w_down, const moe_lora_t* lora, uint16_t* out,
                           int32_t* topk_ids_out, float* topk_w_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code; never NULL. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
