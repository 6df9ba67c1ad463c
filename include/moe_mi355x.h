/*
 * moe_mi355x.h -- C ABI of the sparse top-k Mixture-of-Experts FFN forward
 * for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * Page legend (titles of the pages that define the operations):
 *   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
 *   [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
 *   [SonicMoE page]  "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"
 *
 * The block computes, for hidden states x [T,H]:
 *   1. router logits  l = x W_r^T + b      ([Hunyuan page] §二.1 gating formula)
 *   2. softmax over all E experts           (same formula; [Qwen3-MoE page] §1 forward listing)
 *   3. per-token top-k of the logits         ([Qwen3-MoE page] §1 forward listing)
 *   4. an expert-sorted permutation of the T*k assignments ([Qwen3-MoE page] §2.2)
 *   5. per expert, SwiGLU  h = silu(x Wg^T) * (x Wu^T), then y = h W2^T
 *      (one grouped compute over all experts: [Qwen3-MoE page] §2.1)
 *   6. out[t] = sum_j w[t,j] * y[row of (t,j)]   ([Qwen3-MoE page] §1, phase 4)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Device pointers point to memory of the current HIP device; host pointers
 *   are marked as such.  Arrays of the bulk dtype (x, weights, h, y, x_perm,
 *   out) and workspaces must be 16-byte aligned (the moe_forward workspace
 *   256-byte aligned); int32 and fp32 index/weight arrays 4-byte aligned.
 *   A misaligned pointer is rejected with MOE_ERR_INVALID_ARG.
 * - All arrays are dense, row-major, contiguous.  Weights are (out, in):
 *   w_router [E,H]; w13 [E,2I,H] holding, per expert, the I gate rows and
 *   then the I up rows; w2 [E,H,I].
 * - dtype MOE_DTYPE_BF16: x, weights, h, y, x_perm and out are bf16; every
 *   product is accumulated in fp32; h and y are rounded to bf16 once (round
 *   to nearest even).  MOE_DTYPE_F32: everything is fp32, computed with fp32
 *   fused multiply-adds (no reduced-precision matrix path).
 *   router_bias and topk_weights are always fp32; indices are int32.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   validates on the host and enqueues kernels on `stream`: it does not
 *   allocate, copy to the host or synchronise.  The caller owns every buffer;
 *   the library keeps no device memory and no mutable global state besides a
 *   per-device cache of device properties and the device array that
 *   moe_permute_static uses instead of a workspace, so calls on different
 *   streams may run concurrently as long as their buffers do not overlap
 *   (moe_permute_static calls on one GPU share that array and must not).
 * - Results are deterministic: identical inputs give bitwise identical
 *   outputs (no floating-point atomics anywhere).
 * - Limits: 1 <= k <= E, E <= 256, k <= 8, H and I multiples of 64,
 *   H <= 16384, I <= 65536, T*k <= 2^31-1.  T == 0 is a valid no-op.
 * - Errors are returned before anything is enqueued; the output buffers are
 *   then untouched.  moe_last_error() gives a message for the calling thread.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned pointer */
    MOE_ERR_UNSUPPORTED = 2,   /* outside the limits above, unknown dtype, not a gfx950 device */
    MOE_ERR_WORKSPACE = 3,     /* workspace null or smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,
    MOE_DTYPE_BF16 = 1
} moe_dtype;

typedef enum moe_entry {
    MOE_ENTRY_ROUTE = 0,
    MOE_ENTRY_PERMUTE = 1,
    MOE_ENTRY_GROUPED_GEMM = 2,
    MOE_ENTRY_COMBINE = 3,
    MOE_ENTRY_FORWARD = 4
} moe_entry;

/*
 * moe_route -- steps 1-3: router linear layer, softmax over all E experts,
 * per-token top-k.  Defined by the gating formula G(x) = Softmax(W_g x + b_g)
 * of [Hunyuan page] §二.1 and the softmax-then-topk of the forward listing of
 * [Qwen3-MoE page] §1.
 *
 *   x            [T,H] dtype, device.
 *   w_router     [E,H] dtype, device.
 *   router_bias  [E] fp32, device, or NULL for no bias.
 *   topk_ids     [T,k] int32, device, output.  Slot j holds the expert with
 *                the (j+1)-th largest logit; ties go to the lowest expert
 *                index.  The selection is that of the exact logits: tokens
 *                whose fp32 logits are too close to order safely (closer
 *                than a rigorous bound on the fp32 summation error) are
 *                re-ranked with float64 dot products.
 *   topk_weights [T,k] fp32, device, output: the softmax probability of the
 *                chosen expert; with renormalize != 0 divided by the sum of
 *                the token's k probabilities.
 *   workspace    device scratch of moe_workspace_size(MOE_ENTRY_ROUTE, ...)
 *                bytes; contents on entry are ignored.
 * x, w_router and router_bias must hold finite values (the error bound that
 * decides which tokens are re-ranked is built from their norms); with an
 * infinity or NaN among them the ids and weights are unspecified.  The same
 * holds for every entry point that routes.
 */
int moe_route(const void* x, const void* w_router, const float* router_bias,
              int64_t T, int32_t H, int32_t E, int32_t k, int32_t dtype,
              int32_t renormalize, int32_t* topk_ids, float* topk_weights,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute -- step 4: group the T*k assignments by expert
 * ([Qwen3-MoE page] §2.2: reorder tokens by their expert, gather the states,
 * scatter the results back).  With f = t*k + j the flat assignment index:
 *
 *   topk_ids       [T,k] int32, device; every id must lie in [0,E) (ids out
 *                  of range are a caller error with undefined results).
 *   expert_counts  [E] int32, device, output: assignments per expert.
 *   expert_offsets [E+1] int32, device, output: exclusive prefix sum of the
 *                  counts; rows of expert e are offsets[e]..offsets[e+1]-1.
 *   perm           [T*k] int32, device, output: perm[r] = f of row r, rows in
 *                  (expert, f) order -- a stable sort by expert.
 *   inv_perm       [T*k] int32, device, output: inv_perm[perm[r]] = r.
 *   x, x_perm      optional (both NULL or both set): x [T,H] dtype, device;
 *                  x_perm [T*k,H] dtype, device, output: x_perm[r] = x[perm[r]/k].
 *   workspace      moe_workspace_size(MOE_ENTRY_PERMUTE, ...) bytes, device.
 */
int moe_permute(const int32_t* topk_ids, const void* x, int64_t T, int32_t H,
                int32_t E, int32_t k, int32_t dtype, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                void* x_perm, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * moe_permute_static -- moe_permute for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * kernels as moe_permute without the workspace; the per-chunk expert
 * histograms live in a 4 MiB device array the library owns (one per GPU,
 * held until the process ends, its address looked up on the first call on
 * each device).  Nothing is allocated or freed, and every entry of that
 * array a call reads was written by the same call (no zeroing needed).
 *
 * Limit: ceil(T*k / 1024) * E <= 1048576 histogram entries (for E = 256,
 * T*k <= 4194304); larger problems return MOE_ERR_UNSUPPORTED before any
 * launch.  All calls on one GPU share the array: calls that overlap in
 * time on one GPU (different streams or host threads without ordering)
 * race and give undefined results.
 */
int moe_permute_static(const int32_t* topk_ids, const void* x, int64_t T,
                       int32_t H, int32_t E, int32_t k, int32_t dtype,
                       int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* perm, int32_t* inv_perm, void* x_perm,
                       void* stream);

/*
 * moe_grouped_swiglu_gemm -- steps 5-6: every expert's SwiGLU MLP over its
 * rows, in one grouped compute ([Qwen3-MoE page] §2.1: stacked expert
 * weights, one batched launch scheduled over the compute units).
 *
 *   x_perm          [M,H] dtype, device: rows grouped by expert.
 *   expert_offsets  [E+1] int32, device: rows of expert e are
 *                   offsets[e]..offsets[e+1]-1; offsets[0] = 0, offsets[E] = M,
 *                   non-decreasing (empty experts cost nothing and their
 *                   weights are never read).
 *   w13             [E,2I,H] dtype, device.   w2 [E,H,I] dtype, device.
 *   h               [M,I] dtype, device, output: silu(x Wg^T) * (x Wu^T).
 *   y               [M,H] dtype, device, output: h W2^T.
 *   workspace       moe_workspace_size(MOE_ENTRY_GROUPED_GEMM, T=M, ..., k=1)
 *                   bytes, device (tile schedule).
 */
int moe_grouped_swiglu_gemm(const void* x_perm, const int32_t* expert_offsets,
                            const void* w13, const void* w2, int64_t M,
                            int32_t H, int32_t I, int32_t E, int32_t dtype,
                            void* h, void* y, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * moe_combine -- step 7: out[t] = sum_{j<k} w[t,j] * y[inv_perm[t*k+j]],
 * the routing-weighted sum of expert outputs ([Qwen3-MoE page] §1 phase 4,
 * §2.2 scatter back).  Summed in fp32 in slot order j = 0..k-1 and rounded
 * once; no atomics.
 *
 *   y [T*k,H] dtype, inv_perm [T*k] int32, topk_weights [T,k] fp32,
 *   out [T,H] dtype (output); all device.
 */
int moe_combine(const void* y, const int32_t* inv_perm,
                const float* topk_weights, int64_t T, int32_t H, int32_t k,
                int32_t dtype, void* out, void* stream);

/*
 * moe_forward -- the whole block: route, permute, grouped SwiGLU, combine,
 * in the step order of the optimised forward pseudocode of [Qwen3-MoE page]
 * §2.2 (route, reorder the tokens by expert, batched expert compute, scatter
 * the results back and sum them with the routing weights; the block itself
 * is the forward listing of §1).  The grouped GEMM reads the rows of x through the permutation directly (no
 * x_perm copy), and its down projection writes each output row straight back
 * to token order (row perm[r]), so the combine reads every token's k rows
 * contiguously.  Every intermediate is left in the workspace at the offsets
 * moe_forward_workspace_layout() reports, so each step can be inspected.
 *
 *   x [T,H], w_router [E,H], router_bias [E] fp32 or NULL, w13 [E,2I,H],
 *   w2 [E,H,I], out [T,H] (output); all device.
 *   workspace  moe_workspace_size(MOE_ENTRY_FORWARD, ...) bytes, device.
 */
int moe_forward(const void* x, const void* w_router, const float* router_bias,
                const void* w13, const void* w2, int64_t T, int32_t H,
                int32_t I, int32_t E, int32_t k, int32_t dtype,
                int32_t renormalize, void* out, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * moe_forward_profiled -- moe_forward that also records caller-created HIP
 * events on `stream` around its stages, for per-kernel timing on the stream
 * the kernels run on.  events: host array of n_events hipEvent_t handles
 * (passed as void*), n_events == MOE_PROFILE_EVENTS.  events[i] is recorded
 * before stage i and events[MOE_PROFILE_EVENTS-1] after the last stage:
 *   0 router (logits, softmax, top-k, float64 re-rank)
 *   1 permutation (histogram, scan, stable scatter; also the grouped GEMMs'
 *     tile schedule)
 *   2 gate/up grouped GEMM with the SiLU(gate)*up epilogue
 *   3 down grouped GEMM
 *   4 combine
 * Arguments and results are otherwise those of moe_forward.
 */
#define MOE_PROFILE_EVENTS 6
int moe_forward_profiled(const void* x, const void* w_router,
                         const float* router_bias, const void* w13,
                         const void* w2, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, int32_t dtype,
                         int32_t renormalize, void* out, void* workspace,
                         size_t workspace_bytes, void* const* events,
                         int32_t n_events, void* stream);

/* Byte offsets of the intermediates inside the moe_forward workspace. */
typedef struct moe_forward_layout {
    size_t topk_ids;        /* [T,k] int32 */
    size_t topk_weights;    /* [T,k] fp32 */
    size_t expert_counts;   /* [E] int32 */
    size_t expert_offsets;  /* [E+1] int32 */
    size_t perm;            /* [T*k] int32 */
    size_t inv_perm;        /* [T*k] int32 */
    size_t h;               /* [T*k,I] dtype */
    size_t y;               /* [T*k,H] dtype, token order: row t*k+j is slot (t,j)'s
                               expert output (the down GEMM writes row r of the
                               expert-sorted order to row perm[r]) */
    size_t scratch;         /* internal */
    size_t total;           /* == moe_workspace_size(MOE_ENTRY_FORWARD, ...) */
} moe_forward_layout;

/* Host-only.  Fills *layout; same validation as moe_forward's sizes. */
int moe_forward_workspace_layout(int64_t T, int32_t H, int32_t I, int32_t E,
                                 int32_t k, int32_t dtype,
                                 moe_forward_layout* layout);

/*
 * moe_forward_train -- moe_forward that also keeps what the caching variant
 * of moe_backward needs: the gate/up GEMM writes, besides h, its gate and up
 * sums rounded to bf16.
 *   gate_up  [T*k, 2I] bf16, device, output, 16-byte aligned: row r (the
 *            expert-sorted row of the permutation) holds g (I values) then u.
 *   events   NULL, or MOE_PROFILE_EVENTS caller-created HIP events recorded
 *            as moe_forward_profiled records them (n_events must match).
 * dtype must be MOE_DTYPE_BF16.  Other arguments and results as moe_forward;
 * the workspace (moe_forward_workspace_layout) is the one moe_backward reads.
 */
int moe_forward_train(const void* x, const void* w_router,
                      const float* router_bias, const void* w13,
                      const void* w2, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t k, int32_t dtype, int32_t renormalize,
                      void* out, void* gate_up, void* workspace,
                      size_t workspace_bytes, void* const* events,
                      int32_t n_events, void* stream);

/*
 * moe_forward_shared -- moe_forward plus a shared expert.  [Hunyuan page]
 * §二.1 routes tokens through a shared-expert pool besides the gated experts
 * without giving its formula; the reading implemented here is a dense expert
 * of the routed experts' SwiGLU form applied to every token and added with
 * weight 1:
 *   out[t] = sum_{j<k} w[t,j] * Y_{t,j} + S(x_t),
 *   S(x)   = ws2 (silu(ws13[0:Is] x) * (ws13[Is:2Is] x)).
 * S is computed by the same grouped-GEMM kernels as one dense group, stored
 * as dtype like Y, and added after the k routed slots in the same fp32 sum,
 * rounded once.
 *
 *   ws13 [2*Is,H] dtype, ws2 [H,Is] dtype, device, 16-byte aligned; Is a
 *   multiple of 64, at most 65536.  Other arguments as moe_forward.
 *   workspace  moe_forward_shared_layout(...).total bytes, device.  The
 *              routed intermediates sit at the offsets of layout.routed, the
 *              shared expert's h and output at h_shared / y_shared.
 */
int moe_forward_shared(const void* x, const void* w_router,
                       const float* router_bias, const void* w13,
                       const void* w2, const void* ws13, const void* ws2,
                       int64_t T, int32_t H, int32_t I, int32_t Is, int32_t E,
                       int32_t k, int32_t dtype, int32_t renormalize,
                       void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * moe_forward_shared_profiled -- moe_forward_shared recording caller-created
 * HIP events around its stages (as moe_forward_profiled), n_events ==
 * MOE_PROFILE_EVENTS_SHARED: stages 0..3 as moe_forward_profiled, then
 *   4 shared expert (gate/up and down GEMMs over every token)
 *   5 combine (routed slots plus the shared output)
 */
#define MOE_PROFILE_EVENTS_SHARED 7
int moe_forward_shared_profiled(const void* x, const void* w_router,
                                const float* router_bias, const void* w13,
                                const void* w2, const void* ws13,
                                const void* ws2, int64_t T, int32_t H,
                                int32_t I, int32_t Is, int32_t E, int32_t k,
                                int32_t dtype, int32_t renormalize, void* out,
                                void* workspace, size_t workspace_bytes,
                                void* const* events, int32_t n_events,
                                void* stream);

/* Byte offsets inside the moe_forward_shared workspace. */
typedef struct moe_shared_layout {
    moe_forward_layout routed;  /* routed intermediates, as in moe_forward */
    size_t h_shared;            /* [T,Is] dtype */
    size_t y_shared;            /* [T,H] dtype: S(x) */
    size_t scratch;             /* internal */
    size_t total;               /* workspace bytes moe_forward_shared needs */
} moe_shared_layout;

/* Host-only.  Fills *layout; same validation as moe_forward_shared's sizes. */
int moe_forward_shared_layout(int64_t T, int32_t H, int32_t I, int32_t Is,
                              int32_t E, int32_t k, int32_t dtype,
                              moe_shared_layout* layout);

/*
 * moe_forward_rounded -- moe_forward with token rounding between the router
 * and the permutation.  [SonicMoE page] 核心差异 §3 rounds each expert's row
 * count down to a multiple of the GEMM row tile and gives the remaining
 * tokens to the least-loaded experts, so the grouped GEMM pads no tile.  The
 * rule implemented (all integer decisions, B = tile_rows):
 *   1. expert e keeps the first floor(c_e/B)*B of its assignments in flat
 *      order f = t*k + j; the others are pooled;
 *   2. the pool is handed out in rounds: a round with P pooled assignments
 *      left opens ceil(P/B) tiles of B rows and first picks their owners by
 *      water-filling (lowest row count, kept plus B per tile already planned,
 *      ties to the lowest id, skipping experts one of whose tiles came out
 *      empty); then, tile by tile, a tile takes up to B pooled assignments in
 *      flat order whose token holds its owner in no other slot, at most one
 *      slot per token (a token's first untaken pooled slot, or the slot that
 *      already holds the owner).  What a round leaves goes to the next one;
 *   3. a moved slot keeps its position j; its weight is the token's softmax
 *      probability of the new expert (renormalised over the token's k
 *      weights when renormalize != 0).  Unmoved tokens keep their weights.
 * No token ever holds an expert twice (needs k <= E, which is a limit anyway).
 *
 *   tile_rows  B >= 1; moe_gemm_tile_rows(dtype) is the row tile of this
 *              library's grouped GEMM, the value that removes its padding.
 *   workspace  moe_forward_rounded_layout(...).total bytes, device.
 * The workspace intermediates are those of moe_forward for the rounded
 * routing: topk_ids / topk_weights hold the rounded ids and weights, and the
 * counts, offsets and permutation are those of the rounded ids.  Other
 * arguments and results as moe_forward.  The tile hand-out is sequential by
 * nature and runs in one workgroup (its tiles pipelined across 16 waves); its
 * cost grows with the number of tiles handed out and the pool tokens each
 * tile walks.
 */
int moe_forward_rounded(const void* x, const void* w_router,
                        const float* router_bias, const void* w13,
                        const void* w2, int64_t T, int32_t H, int32_t I,
                        int32_t E, int32_t k, int32_t dtype,
                        int32_t renormalize, int32_t tile_rows, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward_rounded_profiled -- moe_forward_rounded recording caller-created
 * HIP events around its stages (as moe_forward_profiled), n_events ==
 * MOE_PROFILE_EVENTS_ROUNDED:
 *   0 router (also keeps every token's logits, softmax max and sum)
 *   1 token rounding (permutation of the routed ids, pooled slots, tile
 *     hand-out, new weights)
 *   2 permutation of the rounded ids (and the GEMMs' tile schedule)
 *   3..5 gate/up GEMM, down GEMM, combine
 */
#define MOE_PROFILE_EVENTS_ROUNDED 7
int moe_forward_rounded_profiled(const void* x, const void* w_router,
                                 const float* router_bias, const void* w13,
                                 const void* w2, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k,
                                 int32_t dtype, int32_t renormalize,
                                 int32_t tile_rows, void* out, void* workspace,
                                 size_t workspace_bytes, void* const* events,
                                 int32_t n_events, void* stream);

/* Host-only.  Fills *layout (same fields as moe_forward's; a larger scratch
 * and total); same validation as moe_forward's sizes. */
int moe_forward_rounded_layout(int64_t T, int32_t H, int32_t I, int32_t E,
                               int32_t k, int32_t dtype,
                               moe_forward_layout* layout);

/* Host-only.  Rows per tile of the grouped GEMM for dtype (bf16: 256, fp32:
 * 64); 0 for an unknown dtype (moe_last_error() then says so). */
int moe_gemm_tile_rows(int32_t dtype);

/*
 * MXFP8 expert GEMMs
 * ------------------
 * [Hunyuan page] §七.1 runs the experts in FP8 and asks for the routing to be
 * checked again under quantization.  Here the router stays on the bf16
 * inputs (its decisions are those of moe_forward) and the two expert GEMMs
 * run on MXFP8 operands, the OCP Microscaling v1.0 format: along the
 * reduction axis of each row, a block of 32 consecutive values shares one
 * E8M0 scale 2^e with e = floor(log2 amax) - 8 (8 = largest exponent of
 * e4m3), clamped to [-127, 127] (-127 for a block of zeros), and each value
 * is stored as the e4m3 code (bias 7, largest magnitude 448, no infinities)
 * nearest to value / 2^e, ties to the even code, saturating at +-448; a
 * value that rounds to zero gets the code of +0.  Scales are stored as the
 * biased exponent e + 127, one uint8 per block.
 */

/*
 * moe_mx_quantize -- MXFP8 codes and scales of a [rows, cols] matrix along
 * its rows (the format above).
 *   src     [rows, cols] dtype (bf16 or fp32), device, 16-byte aligned.
 *   cols    a multiple of 32; rows >= 0 (0: no-op).
 *   codes   [rows, cols] uint8, device, output, 16-byte aligned.
 *   scales  [rows, cols/32] uint8, device, output.
 * The expert weights of moe_forward_mxfp8 are w13 viewed as [E*2I, H] and
 * w2 as [E*H, I], each quantized along its input dimension.
 */
int moe_mx_quantize(const void* src, int64_t rows, int32_t cols, int32_t dtype,
                    uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_forward_mxfp8 -- the block of moe_forward with MXFP8 expert GEMMs:
 * routing and permutation as moe_forward (dtype must be MOE_DTYPE_BF16);
 * x quantized along H; per expert, h = silu(x Wg^T) * (x Wu^T) from the
 * block-scaled MFMA (products of the dequantized values, fp32 sums),
 * quantized along I; y = h W2^T (fp32 sums) rounded to bf16; the weighted
 * combine as moe_forward.  The GEMMs read the scales as stage-major 32-bit
 * words (the four scales of 128 consecutive K values of one row in one word,
 * the words of consecutive rows adjacent); the call writes those of x (in the
 * permuted row order) and of the weights into its workspace first.
 *   w13q [E,2I,H] uint8 codes, w13s [E,2I,H/32] uint8 scales;
 *   w2q [E,H,I] uint8 codes, w2s [E,H,I/32] uint8 scales (moe_mx_quantize
 *   of the expert weights); codes 16-byte aligned.
 *   H and I multiples of 128; T*H <= 2^32.
 *   workspace  moe_forward_mxfp8_layout(...).total bytes, device, 256-byte
 *              aligned; afterwards it holds the intermediates at the layout's
 *              offsets (y in token order: row t*k+j).
 * Other arguments, limits and results as moe_forward.
 */
int moe_forward_mxfp8(const void* x, const void* w_router,
                      const float* router_bias, const uint8_t* w13q,
                      const uint8_t* w13s, const uint8_t* w2q,
                      const uint8_t* w2s, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t k, int32_t dtype,
                      int32_t renormalize, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * moe_forward_mxfp8_profiled -- moe_forward_mxfp8 recording caller-created
 * HIP events around its stages (as moe_forward_profiled), n_events ==
 * MOE_PROFILE_EVENTS_MXFP8: 0 router, 1 permutation (and the GEMMs' tile
 * schedule), 2 quantization of x and the stage-major scale words, 3 gate/up
 * GEMM (with the quantization of h), 4 down GEMM, 5 combine.
 */
#define MOE_PROFILE_EVENTS_MXFP8 7
int moe_forward_mxfp8_profiled(const void* x, const void* w_router,
                               const float* router_bias, const uint8_t* w13q,
                               const uint8_t* w13s, const uint8_t* w2q,
                               const uint8_t* w2s, int64_t T, int32_t H,
                               int32_t I, int32_t E, int32_t k, int32_t dtype,
                               int32_t renormalize, void* out, void* workspace,
                               size_t workspace_bytes, void* const* events,
                               int32_t n_events, void* stream);

/* Byte offsets of the moe_forward_mxfp8 workspace regions (M = T*k). */
typedef struct moe_mxfp8_layout {
    size_t topk_ids;       /* [T,k] int32 */
    size_t topk_weights;   /* [T,k] fp32 */
    size_t expert_counts;  /* [E] int32 */
    size_t expert_offsets; /* [E+1] int32 */
    size_t perm;           /* [M] int32 */
    size_t inv_perm;       /* [M] int32 */
    size_t x_codes;        /* [T,H] uint8: x quantized along H */
    size_t x_scales;       /* [T,H/32] uint8 */
    size_t h_codes;        /* [M,I] uint8: h of the expert-sorted rows */
    size_t h_scales;       /* [I/128,M] uint32 words, stage-major: word (s,r)
                              holds the scales of blocks 4s..4s+3 of row r,
                              block 4s+b in byte b */
    size_t y;              /* [M,H] bf16: expert outputs, row t*k+j */
    size_t x_scale_words;  /* [H/128,M] uint32: x_scales of row perm[r]/k as
                              word (s,r), in the same stage-major form */
    size_t w13_scale_words;/* [H/128,E*2I] uint32: w13s, stage-major */
    size_t w2_scale_words; /* [I/128,E*H] uint32: w2s, stage-major */
    size_t scratch;        /* kernel scratch */
    size_t total;          /* bytes of the whole workspace */
} moe_mxfp8_layout;

/* Host-only.  Fills *layout; validates the sizes as moe_forward_mxfp8. */
int moe_forward_mxfp8_layout(int64_t T, int32_t H, int32_t I, int32_t E,
                             int32_t k, int32_t dtype,
                             moe_mxfp8_layout* layout);

/*
 * Backward
 * --------
 * moe_backward -- the gradients of L = sum(dout * out) for the block of
 * moe_forward, with the top-k choice held fixed (it is piecewise constant):
 * dx, the router weight and bias, W13 and W2.  Following [SonicMoE page]
 * 核心差异 §1, the forward keeps only its routing and its expert outputs y
 * (in the moe_forward workspace) and the backward recomputes the rest: g and
 * u by the grouped GEMM, h from them.  Per [Hunyuan page] §二.2 only the
 * experts a token activated get gradients (the others' come out zero).
 *   dw[t,j] = <dout_t, y_tj>;  through the renormalisation (renormalize != 0)
 *   and the softmax, dl = dL/dlogits; dx = sum_j [dg du] W13_e + dl W_r;
 *   dW_r = dl^T x; dbias = sum_t dl; dW2_e = sum (w dout)^T h;
 *   dW13_e = sum [dg du]^T x, with dh = (w dout) W2_e, dg = dh u silu'(g),
 *   du = dh silu(g).
 * dtype must be MOE_DTYPE_BF16 (bf16 operands, fp32 accumulation; g, u, dh,
 * dg, du, h and the per-slot dx rounded to bf16 once).
 *   x, w_router, router_bias, w13, w2, sizes, renormalize: exactly as passed
 *               to the moe_forward call whose workspace is given.
 *   forward_workspace  that call's workspace (moe_forward_workspace_layout
 *               size), left unchanged since; read only.
 *   gate_up     NULL: g and u are recomputed (the memory-saving variant of
 *               [SonicMoE page] 核心差异 §1); or the [T*k, 2I] bf16 sums the
 *               matching moe_forward_train call kept (the caching variant:
 *               one grouped GEMM less, 4*T*k*I bytes more kept), read only.
 *   dout        [T,H] bf16, device.
 *   dx          [T,H] bf16, device, output.
 *   dw_router   [E,H] fp32, device, output.
 *   dbias       [E] fp32, device, output, or NULL (not computed).
 *   dw13        [E,2I,H] fp32, device, output (layout of w13).
 *   dw2         [E,H,I] fp32, device, output (layout of w2).
 *   workspace   moe_backward_workspace_layout(...).total bytes, device, 256-byte
 *               aligned; afterwards it holds the intermediates at the
 *               layout's offsets.
 * Limits as moe_forward, plus T*H*2 <= 2^32.  Deterministic (no atomics).
 */
int moe_backward(const void* x, const void* w_router, const float* router_bias,
                 const void* w13, const void* w2, int64_t T, int32_t H, int32_t I,
                 int32_t E, int32_t k, int32_t dtype, int32_t renormalize,
                 const void* forward_workspace, size_t forward_workspace_bytes,
                 const void* gate_up, const void* dout, void* dx,
                 float* dw_router, float* dbias, float* dw13, float* dw2,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_backward_profiled -- moe_backward recording caller-created HIP events
 * around its stages, n_events == MOE_PROFILE_EVENTS_BACKWARD:
 *   0 router gradients (dw, the router's logits again, dl, dl W_r, dW_r, dbias)
 *   1 g and u again (grouped GEMM; empty when gate_up is given)
 *   2 dh (grouped GEMM reading W2 as stored) and the SwiGLU backward (dg, du, h)
 *   3 dx: [dg du] W13 (grouped GEMM reading W13 as stored) and the sum over
 *     a token's slots
 *   4 transposed operands of the weight-gradient GEMMs
 *   5 dW2 (grouped GEMM over each expert's rows)
 *   6 dW13 (same)
 */
#define MOE_PROFILE_EVENTS_BACKWARD 8
int moe_backward_profiled(const void* x, const void* w_router,
                          const float* router_bias, const void* w13,
                          const void* w2, int64_t T, int32_t H, int32_t I,
                          int32_t E, int32_t k, int32_t dtype,
                          int32_t renormalize, const void* forward_workspace,
                          size_t forward_workspace_bytes, const void* gate_up,
                          const void* dout, void* dx, float* dw_router,
                          float* dbias, float* dw13, float* dw2,
                          void* workspace, size_t workspace_bytes,
                          void* const* events, int32_t n_events, void* stream);

/* Byte offsets of the moe_backward workspace regions (M = T*k; ld = the
 * padded row count of the weight-gradient operands). */
typedef struct moe_backward_layout {
    size_t dw;           /* [T,k] fp32: dL/d(routing weight) */
    size_t dlogits;      /* [T,E] fp32: dL/d(router logit) */
    size_t dx_router;    /* [T,H] bf16: dl W_r */
    size_t gu;           /* [M,2I] bf16: g then u of each expert-sorted row */
    size_t dh;           /* [M,I] bf16: dout W2_e (before the routing weight) */
    size_t dgdu;         /* [M,2I] bf16: dg then du */
    size_t h;            /* [M,I] bf16: silu(g) u */
    size_t dx_slots;     /* [M,H] bf16: [dg du] W13_e, row t*k+j */
    size_t padded_offsets; /* [E+1] int32: column offsets of the experts in the operands below */
    size_t dyT;          /* [H,ld] bf16 */
    size_t hT;           /* [I,ld] bf16 */
    size_t dgduT;        /* [2I,ld] bf16 */
    size_t xT;           /* [H,ld] bf16 */
    size_t ld;           /* elements */
    size_t scratch;
    size_t total;
} moe_backward_layout;

/* Host-only.  Fills *layout; validates the sizes as moe_backward. */
int moe_backward_workspace_layout(int64_t T, int32_t H, int32_t I, int32_t E,
                                  int32_t k, int32_t dtype,
                                  moe_backward_layout* layout);

/*
 * Host-only.  Workspace bytes needed by `entry` (a moe_entry) for these
 * sizes, written to *bytes (host pointer).  For MOE_ENTRY_GROUPED_GEMM pass
 * T = M and k = 1.  Sizes that the entry ignores may be given as 1.
 */
int moe_workspace_size(int32_t entry, int64_t T, int32_t H, int32_t I,
                       int32_t E, int32_t k, int32_t dtype, size_t* bytes);

/* Host-only.  Static string naming a moe_status value. */
const char* moe_status_string(int status);

/* Host-only.  Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Host-only.  ABI version: major*100 + minor. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
