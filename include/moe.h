/*
 * moe.h - C ABI of the MI355X (gfx950) fine-grained Mixture-of-Experts layer
 * forward: router projection, sigmoid top-k / hash routing, token dispatch
 * permutation, grouped expert FFN with clamped SwiGLU, shared expert and
 * routing-weight combine.
 *
 * The operations follow these pages:
 *   [HP]  "HyperParallel accelerates DeepSeek-V4.1 multimodal 1M long-sequence
 *         training", section 2.3 (MegaKernel): MegaGate (score, bias ranking,
 *         Top-K, score extraction, normalisation, scaling; text and vision
 *         routing bias; projection matmul outside the gate) and MegaMoE (token
 *         dispatch, two expert matmuls, SwiGLU with the V4.1 clamp, result
 *         return, reused workspace).
 *   [TW]  "Twinkle x Ascend ... DeepSeek-V4 training", section "FSDP2-4D
 *         parallel engine adaptation": router output (logits, routing weights,
 *         selected experts); HashRouter ids = tid2eid[input_ids] weighted from
 *         the gate logits; one dispatch path for both routers; results merged
 *         by routing weight.
 *   [MS]  "MindSpore HyperParallel one-click DeepSeek-V4.1-Flash", section 01:
 *         one shared expert plus 384 routed experts, 6 routed per token.
 *   [CN]  "CANN DeepSeek-V4 training optimisation", outlook section,
 *         functional-expansion bullets: MxFP8 / MxFP4 low-precision weights.
 *
 * Conventions (all entry points):
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous.  bf16 tensors are passed as uint16_t bit patterns.  Pointers
 *     to bf16 data and fp32 matrices must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued: no entry point synchronises the host, allocates or frees.
 *   - Return 0 (MOE_OK) or a negative MOE_ERR_* code.  All argument checks run
 *     on the host before the first launch, so an error leaves no partial work
 *     queued.  Errors found in device data (ids out of range) do not abort:
 *     the offending token/pair is dropped and a bit is OR-ed into `*d_flags`
 *     (a device uint32, optional: NULL = not reported).  The caller clears it.
 *   - Scratch memory comes from a caller workspace `ws` of at least the
 *     size the matching *_workspace_size() returns (256-byte aligned).  Calls
 *     that share a workspace must not overlap in time.
 *   - Calls with distinct workspaces and outputs may come from several host
 *     threads at once, also as the first calls of a process: the library's
 *     one-time per-device set-up (kernel attributes, grid sizes) runs once
 *     per device under a lock, and the library keeps no other host state.
 *   - Results are deterministic: the same inputs give the same bits.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define MOE_ERR_UNSUPPORTED (-3) /* a mode or size outside the supported set */
#define MOE_ERR_WORKSPACE (-4)   /* workspace missing, misaligned or too small */
#define MOE_ERR_HIP (-5)         /* a HIP runtime call failed */
#define MOE_ERR_ALIGN (-6)       /* a tensor pointer is not 16-byte aligned */
#define MOE_ERR_SCRATCH (-7)     /* more scratch than the static array holds */

#define MOE_MODE_TOPK 0 /* sigmoid score + bias-ranked top-k */
#define MOE_MODE_HASH 1 /* ids from tid2eid[input_ids] */

#define MOE_OUT_BF16 0
#define MOE_OUT_F32 1

#define MOE_CLAMP_SYMMETRIC 0  /* gate and up clamped to [-L, L] */
#define MOE_CLAMP_GATE_UPPER 1 /* gate clamped to (-inf, L], up to [-L, L] */

#define MOE_FLAG_BAD_INPUT_ID 1u  /* an input id outside [0, V) */
#define MOE_FLAG_BAD_EXPERT_ID 2u /* an expert id outside [0, E) */

/* Limits: 1 <= k <= 8, k <= E, 1 <= E <= 1024 (route/permute/forward);
 * d, F multiples of 64 (expert FFN, forward); T * k < 2^31; G <= 4096.
 * The packed-weight expert GEMMs contract over at most 4,194,240 values (a
 * 256-row weight panel within 2 GiB): d, F, F_shared and K up to that,
 * 2 F and 2 F_shared too in moe_backward; larger sizes return
 * MOE_ERR_UNSUPPORTED. */
#define MOE_MAX_K 8
#define MOE_MAX_E 1024
#define MOE_MAX_GROUPS 4096

const char* moe_status_string(int status);

/* ------------------------------------------------------------------------
 * Router projection [HP 2.3 MegaGate: the projection matmul sits outside the
 * gate; TW: router computes logits from hidden states].
 *   logits[t,e] = fl32( sum_i x[t,i] * w_g[e,i]  (+ logit_offset[e]) )
 * bf16 products, fp32 accumulation on MFMA.
 *   x [T,d] bf16, w_g [E,d] bf16, logit_offset [E] fp32 or NULL,
 *   logits [T,E] fp32 (written).  d multiple of 64; 1 <= E <= 4096.
 */
int moe_gate_logits(const uint16_t* x, const uint16_t* w_g, const float* logit_offset,
                    int T, int d, int E, float* logits, void* stream);

/* ------------------------------------------------------------------------
 * Routing [HP 2.3 MegaGate order: score -> bias ranking -> Top-K -> score
 * extraction -> normalise -> scale; TW HashRouter].
 *   s[e] = S(logits[t,e]), S = binary32 sigmoid evaluated as a fixed sequence
 *          of IEEE operations (clamp to [-80,80]; n = rint(-x log2 e);
 *          Cody-Waite reduction; degree-7 Taylor polynomial by fma; scale by
 *          2^n; 1/(1+e) correctly rounded), so the scores are reproducible bit
 *          for bit on any IEEE machine.
 *   TOPK: r[e] = fl32(s[e] + score_bias[m(t), e]), m(t) = modality[t] ? 1 : 0
 *         when n_bias == 2 and modality != NULL, else 0 (no bias if NULL);
 *         topk_ids[t,:] = the k experts greatest under (r desc, index asc),
 *         in that order.
 *   HASH: topk_ids[t,j] = tid2eid[input_ids[t], j] (table order).  A token
 *         with input_ids[t] outside [0,V) or a table id outside [0,E) gets
 *         ids -1 and weights 0 and sets a flag bit.
 *   both: g_j = s[topk_ids[t,j]] (unbiased); S_t = ((g_0 + g_1) + ...) in
 *         fp32; topk_w[t,j] = fl32(fl32(g_j / S_t) * scale).
 *   logits [T,E] fp32; score_bias [n_bias,E] fp32 or NULL (n_bias 0..2);
 *   modality [T] u8 or NULL; input_ids [T] int32 and tid2eid [V,k] int32
 *   (HASH only); topk_ids [T,k] int32 and topk_w [T,k] fp32 (written).
 */
int moe_route(const float* logits, const float* score_bias, const uint8_t* modality,
              const int32_t* input_ids, const int32_t* tid2eid, int T, int E, int k,
              int n_bias, int V, int mode, float scale, int32_t* topk_ids, float* topk_w,
              uint32_t* d_flags, void* stream);

/* ------------------------------------------------------------------------
 * Routing backward [HP 2.3 MegaGate: the gradient chain of the gate's
 * normalisation and scaling, the first step of the gate's backward].
 * Given the forward's logits and routes and the gradient d_topk_w[t,j] of a
 * loss with respect to topk_w[t,j]:
 *   g_j = S(logits[t, topk_ids[t,j]]) (the forward's scores), G = sum_j g_j,
 *   d_logits[t, topk_ids[t,i]] = (scale / G) * (d_topk_w[t,i]
 *                                 - sum_j d_topk_w[t,j] g_j / G) * g_i (1 - g_i)
 *   and d_logits[t,e] = 0 for every expert the token did not select (the
 *   choice is piecewise constant in the logits; the ranking bias takes no
 *   part in the weights).  fp32 arithmetic, sums in slot order; the bracket
 *   is evaluated as sum_j g_j (d_topk_w[t,i] - d_topk_w[t,j]) / G, so it is
 *   exactly 0 when k = 1 or all d_topk_w of a token are equal.
 *   logits [T,E] fp32; topk_ids [T,k] int32; d_topk_w [T,k] fp32;
 *   d_logits [T,E] fp32 (every entry written).  A token with an id outside
 *   [0,E) (as the forward leaves dropped hash tokens) gets a zero row and
 *   sets MOE_FLAG_BAD_EXPERT_ID.  Same limits on E and k as moe_route.
 */
int moe_route_backward(const float* logits, const int32_t* topk_ids, const float* d_topk_w,
                       int T, int E, int k, float scale, float* d_logits, uint32_t* d_flags,
                       void* stream);

/* ------------------------------------------------------------------------
 * Token dispatch [TW: ids from either router -> expert_mask -> one dispatch
 * flow; HP 2.3 MegaMoE token dispatch].  On one device the expert-parallel
 * all-to-all becomes a stable counting sort of the (t, j) pairs, t-major, by
 * expert id, and a copy of each token row to its slots:
 *   counts[e]    = #{(t,j): topk_ids[t,j] = e}
 *   offsets[e]   = sum_{e' < e} counts[e'], offsets[E] = number of valid pairs
 *   dest[t*k+j]  = offsets[e] + #{earlier pairs with the same expert}, or -1
 *   src[row]     = t for filled rows, -1 for rows in [offsets[E], T*k)
 *   x_perm[row]  = x[src[row]] (exact copy; rows past offsets[E] untouched)
 * Pairs with an id outside [0,E) are dropped and set MOE_FLAG_BAD_EXPERT_ID.
 *   topk_ids [T,k] int32, x [T,d] bf16 (d multiple of 8); counts [E],
 *   offsets [E+1], dest [T*k], src [T*k] int32, x_perm [T*k,d] bf16.
 *   ws: moe_permute_workspace_size(T, k, E) bytes, 256-byte aligned (may be
 *   NULL when that size is 0, i.e. T = 0).
 */
size_t moe_permute_workspace_size(int T, int k, int E);
int moe_permute(const int32_t* topk_ids, const uint16_t* x, int T, int d, int E, int k,
                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                uint16_t* x_perm, uint32_t* d_flags, void* ws, size_t ws_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, results and errors as moe_permute, without the
 * workspace: the permutation's scratch (entry ranks and chunk histogram:
 * moe_permute_workspace_size(T, k, E) bytes) lives in a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs
 * on holds until the process ends.  The call allocates nothing; a call whose
 * scratch would exceed the array returns MOE_ERR_SCRATCH before any launch.
 * Every call on one GPU shares that GPU's array (no part of it needs to
 * start at zero; it keeps the last call's contents), so calls that overlap
 * in time on one GPU race: the caller serialises them (one stream, or
 * events between streams).  The first call on a device looks up the array's
 * device address once (a host call, not an allocation). */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_permute_noalloc(const int32_t* topk_ids, const uint16_t* x, int T, int d, int E, int k,
                        int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                        uint16_t* x_perm, uint32_t* d_flags, void* stream);

/* ------------------------------------------------------------------------
 * Grouped expert FFN [HP 2.3 MegaMoE: two expert matmuls with SwiGLU and the
 * V4.1 clamp between them].  For every group g and row r in
 * [offsets[g], offsets[g+1]):
 *   G_f = sum_i a[r,i] w_gate[g,f,i],  U_f = sum_i a[r,i] w_up[g,f,i]  (fp32)
 *   clamp with limit L (L = +inf: none): SYMMETRIC G,U <- clamp(., -L, L);
 *   GATE_UPPER G <- min(G, L), U <- clamp(U, -L, L)
 *   h[r,f] = bf16( silu(G_f) * U_f ),  silu(z) = z / (1 + e^-z)
 *   y[r,o] = sum_f h[r,f] w_down[g,o,f]  (fp32)
 *   a [rows,d] bf16; offsets [G+1] int32 in DEVICE memory, non-decreasing
 *   within [0, rows] (entries outside are clamped into range); w_gate, w_up
 *   [G,F,d] bf16; w_down [G,d,F] bf16; h [rows,F] bf16 and y [rows,d] fp32
 *   (written for rows inside a group only).  d, F multiples of 64.
 *   The shared expert is the G = 1, offsets = {0, T} call on x.
 */
int moe_expert_ffn(const uint16_t* a, const int32_t* offsets, int G, int rows, int d, int F,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   float clamp_limit, int clamp_mode, uint16_t* h, float* y, void* stream);

/* The same grouped FFN on weights in the moe_pack_weights layout (w_gate,
 * w_up with panel_rows 128, w_down with 256), computed by the expert GEMM
 * that moe_forward uses for packed weights.  Arguments, layouts
 * and results as moe_expert_ffn (h row-major).  It takes no
 * workspace, so its workgroups split the tiles statically (moe_forward
 * balances them with counters in its workspace); the arithmetic, and so every
 * result bit, is the same either way. */
int moe_expert_ffn_packed(const uint16_t* a, const int32_t* offsets, int G, int rows, int d,
                          int F, const uint16_t* w_gate, const uint16_t* w_up,
                          const uint16_t* w_down, float clamp_limit, int clamp_mode, uint16_t* h,
                          float* y, void* stream);

/* The grouped FFN in the A8W4 mode [CN outlook: A8W4 on MxFP8 / MxFP4] on
 * the scaled MX matrix cores: activations as MXFP8 (moe_quantize_mxfp8 of
 * a), weights as MXFP4 (moe_pack_weights_fp4 codes and scales; panel_rows
 * 128 for w_gate / w_up, 256 for w_down).  For every group g and row r:
 *   G, U as moe_expert_ffn on the dequantised a8 and weights (exact products,
 *   fp32 accumulation), clamped; h = bf16(silu(G) U), then h8 / h_scale =
 *   its MXFP8 quantisation along F (the rule of moe_quantize_mxfp8);
 *   y[r,o] = sum_f h8~[r,f] w_down~[g,o,f] (fp32), h8~ the dequantised h8.
 *   a8 [rows,d] uint8 codes + a_scale [rows,d/32] scale bytes; offsets [G+1]
 *   int32 in DEVICE memory (as moe_expert_ffn); h8 [rows,F] uint8 codes,
 *   h_scale [rows,F/32] scale bytes, y [rows,d] fp32 (written for rows
 *   inside a group only).  d, F multiples of 128; a8, h8, y and the weight
 *   codes 16-byte aligned, the scale arrays 4-byte aligned.  moe_forward
 *   with MOE_WEIGHTS_A8W4 runs this chain on the routed rows (gathered
 *   through the dispatch permutation). */
int moe_expert_ffn_a8w4(const uint8_t* a8, const uint8_t* a_scale, const int32_t* offsets, int G,
                        int rows, int d, int F, const uint8_t* w_gate, const uint8_t* w_up,
                        const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                        const uint8_t* s_down, float clamp_limit, int clamp_mode, uint8_t* h8,
                        uint8_t* h_scale, float* y, void* stream);

/* ------------------------------------------------------------------------
 * Weight packing (a one-time layout change at weight-load time, not part of
 * the per-step computation).  Rewrites G matrices W[g] of [N,K] bf16 ([out,
 * in], K multiple of 64) into the matrix-core fragment order the GEMM kernels
 * stream, in panels of P = panel_rows rows:
 *   [G][ceil(N/P)][K/64][P/32][4][64][8],  fragment (panel, s, b, q, lane) =
 *   W[panel*P + b*32 + lane%32][s*64 + 16q + 8(lane/32) .. +8], rows >= N zero.
 * One wave's fragments for one MFMA substep are 1 KB contiguous and one
 * workgroup's panel is contiguous per 64-wide K stage.  moe_forward expects
 * P = 128 for w_gate, w_up, s_gate, s_up and P = 256 for w_down, s_down, w_g.
 *   src [G,N,K] bf16; dst: moe_packed_weight_bytes(G,N,K,P) bytes, 16-byte
 *   aligned, not overlapping src; panel_rows 128 or 256 (else 0 /
 *   MOE_ERR_UNSUPPORTED).
 */
size_t moe_packed_weight_bytes(int G, int N, int K, int panel_rows);
int moe_pack_weights(const uint16_t* src, int G, int N, int K, int panel_rows, uint16_t* dst,
                     void* stream);

/* ------------------------------------------------------------------------
 * MXFP8 routed-expert weights (a one-time conversion at weight-load time).
 * The pages name MXFP8 / MXFP4 expert weights ("CANN DeepSeek-V4 training
 * optimisation", outlook section, functional-expansion bullets; the FP4/FP8
 * checkpoints in the quick start of "Twinkle x Ascend ... DeepSeek-V4
 * training");
 * MXFP8 is the OCP Microscaling format: blocks of 32 values along K (the
 * input dimension) share one power-of-two scale, each value an OCP E4M3
 * float (bias 7, subnormals, no infinities, largest finite 448).  Per block,
 * with the OCP specification's scale rule:
 *   X = floor(log2(max |W| over the block)) - 8, clamped to [-110, 110]
 *       (0 for an all-zero block);
 *   q = E4M3(W / 2^X), round to nearest even, saturating at +-448.
 * The dequantised weight E4M3(q) * 2^X is exactly a bf16 value; moe_forward
 * computes with it exactly (codes and scale decoded together to bf16 for the
 * matrix cores).
 *   Codes, panels of P rows: [G][ceil(N/P)][K/64][P/32][2][64][16 B]; chunk
 *   c of block b, lane l holds row panel*P + b*32 + l%32, columns
 *   64 s + 32 c + 8 (l/32) + {0..7} in bytes 0-7 and the same + 16 in bytes
 *   8-15; rows >= N are zero codes.
 *   Scales: one byte X + 127 per (row, block), [G][ceil(N/P)][K/32][P/32][32].
 *   src [G,N,K] bf16 (finite); dst moe_packed_fp8_weight_bytes(G,N,K,P)
 *   bytes; scales moe_packed_fp8_scale_bytes(G,N,K,P) bytes; both 16-byte
 *   aligned.  K multiple of 64; P 128 (gate, up) or 256 (down), else 0 /
 *   MOE_ERR_UNSUPPORTED.
 */
size_t moe_packed_fp8_weight_bytes(int G, int N, int K, int panel_rows);
size_t moe_packed_fp8_scale_bytes(int G, int N, int K, int panel_rows);
int moe_pack_weights_fp8(const uint16_t* src, int G, int N, int K, int panel_rows, uint8_t* dst,
                         uint8_t* scales, void* stream);

/* MXFP4 routed-expert weights (the pages' "MxFP4"; OCP Microscaling): blocks
 * of 32 values along K share one power-of-two scale, each value an OCP E2M1
 * float (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Per block:
 *   X = floor(log2(max |W| over the block)) - 2, clamped to [-110, 110]
 *       (0 for an all-zero block);
 *   q = E2M1(W / 2^X), nearest, ties to the even code, saturating at +-6.
 * The dequantised weight E2M1(q) * 2^X is exactly a bf16 value.
 *   Codes, panels of P rows: [G][ceil(N/P)][K/32][P/32][64][8 B]; lane l of
 *   the 512-byte chunk of (K block kb, 32-row block b) holds row
 *   panel*P + b*32 + l%32, columns 32 kb + 8 (l/32) + {0..7} in bytes 0-3
 *   and the same + 16 in bytes 4-7, two codes per byte, the lower column in
 *   the low nibble; rows >= N are zero codes.
 *   Scales: as moe_pack_weights_fp8 (moe_packed_fp8_scale_bytes bytes).
 *   src [G,N,K] bf16 (finite); dst moe_packed_fp4_weight_bytes(G,N,K,P)
 *   bytes; both 16-byte aligned.  K multiple of 64; P 128 (gate, up) or 256
 *   (down), else 0 / MOE_ERR_UNSUPPORTED.
 */
size_t moe_packed_fp4_weight_bytes(int G, int N, int K, int panel_rows);
int moe_pack_weights_fp4(const uint16_t* src, int G, int N, int K, int panel_rows, uint8_t* dst,
                         uint8_t* scales, void* stream);

/* MXFP8 quantisation of activation rows [CN outlook: A8W4, MxFP8 activations]
 * (the rule of moe_pack_weights_fp8, along K): for every row of a and block
 * of 32 consecutive values, X = floor(log2(max |v|)) - 8 clamped to
 * [-110, 110] (0 for an all-zero block), codes[r, c] = E4M3(a[r, c] / 2^X)
 * rounded to nearest even and saturated to +-448, scales[r, c / 32] = X + 127.
 *   a [rows, K] bf16 (16-byte aligned), codes [rows, K] uint8 (16-byte
 *   aligned), scales [rows, K / 32] uint8; rows >= 0, K > 0 a multiple of 32.
 * NaN inputs give unspecified codes.  Enqueued on `stream`; the caller owns
 * every buffer.  MOE_ERR_SHAPE / MOE_ERR_NULL / MOE_ERR_ALIGN on bad
 * arguments (nothing enqueued). */
int moe_quantize_mxfp8(const uint16_t* a, long long rows, int K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* ------------------------------------------------------------------------
 * Result return merged by routing weight [TW], plus the always-on shared
 * expert with weight 1 [MS]:
 *   y[t,o] = y_shared[t,o] + sum_j topk_w[t,j] * y_perm[dest[t,j], o]
 * in fp32 (pairs with dest < 0 skipped; y_shared may be NULL), written as
 * bf16 (MOE_OUT_BF16, round to nearest even) or fp32 (MOE_OUT_F32).
 *   y_perm [rows,d] fp32, dest [T*k] int32 (entries >= rows are skipped),
 *   topk_w [T*k] fp32, y_shared [T,d] fp32 or NULL, y [T,d].  d multiple of 8.
 */
int moe_combine(const float* y_perm, const int32_t* dest, const float* topk_w,
                const float* y_shared, int T, int d, int k, int rows, int out_dtype, void* y,
                void* stream);

/* ------------------------------------------------------------------------
 * Combine backward [TW: the merge by routing weight; its gradients feed
 * the expert outputs and, through moe_route_backward, the router].  For a
 * gradient dy of the layer output y = y_shared + sum_j w[t,j] y_perm[dest]:
 *   dy_perm[dest[t,j], o] = fl32(topk_w[t,j] * dy[t,o]),
 *   d_topk_w[t,j] = sum_o dy[t,o] * y_perm[dest[t,j], o]   (fp32 fma
 *                   partials reduced over the workgroup in a fixed order),
 *   and the shared expert's output gradient is dy itself (nothing to do).
 *   dy [T,d] fp32; y_perm [rows,d] fp32 (the forward's expert outputs);
 *   dest [T*k] int32; topk_w [T,k] fp32; dy_perm [rows,d] fp32 (rows that
 *   no pair maps to are left untouched); d_topk_w [T,k] fp32 (written).
 *   A pair with dest outside [0, rows) gets d_topk_w = 0 and writes no
 *   row.  d multiple of 8, k <= 8; dy, y_perm and dy_perm 16-byte aligned.
 */
int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                         const float* topk_w, int T, int d, int k, int rows, float* dy_perm,
                         float* d_topk_w, void* stream);

/* ------------------------------------------------------------------------
 * Clamped-SwiGLU backward [HP 2.3 MegaMoE: SwiGLU with the V4.1 clamp].
 * For h = silu(cg(gate)) * cu(up), the clamps of moe_expert_ffn (limit L,
 * clamp_mode), and a gradient dh of h, elementwise:
 *   dup   = dh * silu(cg(gate)) * [up inside [-L, L]],
 *   dgate = dh * cu(up) * silu'(cg(gate)) * [gate inside the gate clamp's
 *           range ([-L, L], or (-inf, L] for MOE_CLAMP_GATE_UPPER)],
 *   silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z); a clamp passes its
 *   gradient on the closed range.  fp32 arithmetic.
 *   gate, up, dh, dgate, dup: n fp32 values each (n a multiple of 4; the
 *   [rows, F] pre-activations of the gate/up matmul and their gradients),
 *   16-byte aligned.  L > 0 (+inf disables the clamp).
 */
int moe_swiglu_backward(const float* gate, const float* up, const float* dh, int64_t n,
                        float clamp_limit, int clamp_mode, float* dgate, float* dup,
                        void* stream);

/* ------------------------------------------------------------------------
 * Grouped matmul on packed weights [HP 2.3 MegaMoE: the expert matmuls].
 *   out[r, n] = sum_k a[r,k] * W[g, n, k]  for offsets[g] <= r < offsets[g+1],
 *   bf16 products, fp32 accumulation (the expert FFN's MFMA chain); rows
 *   outside every group are left untouched.  In the backward it gives the
 *   expert GEMMs' input gradients: dH = dY W_down with W = W_down^T
 *   ([G, F, d]), and the gate/up input gradient with W = [W_gate | W_up]^T.
 *   a [rows, K] bf16 row-major; offsets [G+1] int32 device; w_packed =
 *   moe_pack_weights(W [G, N, K], panel_rows 256); out [rows, N] fp32.
 *   K, N multiples of 64; a, w_packed, out 16-byte aligned.  No workspace.
 */
int moe_grouped_gemm_packed(const uint16_t* a, const int32_t* offsets, int G, int rows, int K,
                            int N, const uint16_t* w_packed, float* out, void* stream);

/* ------------------------------------------------------------------------
 * Grouped weight gradient [HP 2.3 MegaMoE: the expert matmuls, whose weights
 * the training step of HP 03 updates].  For the grouped matmul
 * out[r, :] = a[r, :] W_g^T on the rows of group g and a gradient dy of out:
 *   dw[g, m, k] = sum_{offsets[g] <= r < offsets[g+1]} dy[r, m] * a[r, k]
 * bf16 products, fp32 accumulation; a group without rows gets zeros (every
 * entry of dw is written).  dW_down = dY^T H (dy = dY [rows, d], a = H
 * [rows, F]), dW_gate = dG^T X and dW_up = dU^T X (dy = the pre-activation
 * gradients, a = the dispatched token rows), and with G = 1 the shared
 * expert's matrices and the router's dW_g = dlogits^T x.
 *   dy [rows, M] bf16, a [rows, K] bf16 row-major; offsets [G+1] int32 in
 *   DEVICE memory (entries clamped into [0, rows]; NULL allowed when G = 1:
 *   one group [0, rows)); dw [G, M, K] fp32.  M, K multiples of 8; dy, a, dw
 *   16-byte aligned.  No workspace.
 */
int moe_grouped_wgrad(const uint16_t* dy, const uint16_t* a, const int32_t* offsets, int G,
                      int rows, int M, int K, float* dw, void* stream);

/* ------------------------------------------------------------------------
 * Whole layer forward: gate logits -> route -> permute -> grouped FFN (routed
 * experts) and FFN (shared expert) -> combine.
 */
typedef struct moe_cfg {
    int T;            /* tokens */
    int d;            /* hidden size (multiple of 64) */
    int E;            /* routed experts (<= 1024) */
    int k;            /* routed experts per token (<= 8, <= E) */
    int F;            /* routed expert FFN width (multiple of 64) */
    int F_shared;     /* shared expert FFN width (multiple of 64), 0 = none */
    int mode;         /* MOE_MODE_TOPK or MOE_MODE_HASH */
    int n_bias;       /* routing bias rows: 0, 1 or 2 (text, vision) */
    int V;            /* HASH: tid2eid rows (vocabulary) */
    float scale;      /* routing weight scale */
    float clamp_limit;/* SwiGLU clamp L (> 0; +inf = none) */
    int clamp_mode;   /* MOE_CLAMP_* */
    int out_dtype;    /* MOE_OUT_BF16 or MOE_OUT_F32 */
} moe_cfg;

typedef struct moe_weights {
    int packed;                   /* 0: every bf16 matrix below is [out,in] as
                                     listed; 1: w_g, w_gate, w_up, w_down,
                                     s_gate, s_up, s_down hold the
                                     moe_pack_weights layout of those matrices
                                     (panel_rows 128 for the gate / up
                                     matrices, 256 for the others);
                                     MOE_WEIGHTS_FP8: as 1, except that w_gate,
                                     w_up, w_down hold moe_pack_weights_fp8
                                     MXFP8 codes (uint8) with the block
                                     scales below; MOE_WEIGHTS_FP4: the same
                                     with moe_pack_weights_fp4 MXFP4 codes;
                                     MOE_WEIGHTS_A8W4: the MXFP4 weights of
                                     MOE_WEIGHTS_FP4 and MXFP8 activations
                                     for both routed expert matmuls [CN
                                     outlook: A8W4 on MxFP8 / MxFP4]: each
                                     token's row of x is quantised along d
                                     (as moe_quantize_mxfp8) before gate/up
                                     and each routed row of h (the bf16
                                     SwiGLU output) along F before down, on
                                     the scaled MX matrix cores; d and F
                                     multiples of 128; the shared expert
                                     stays bf16 */
    const uint16_t* w_g;          /* [E,d] bf16 router projection */
    const float* logit_offset;    /* [E] fp32 or NULL, added to the logits */
    const float* score_bias;      /* [n_bias,E] fp32 or NULL (TOPK) */
    const int32_t* tid2eid;       /* [V,k] int32 (HASH) */
    const uint16_t* w_gate;       /* [E,F,d] bf16 */
    const uint16_t* w_up;         /* [E,F,d] bf16 */
    const uint16_t* w_down;       /* [E,d,F] bf16 */
    const uint16_t* s_gate;       /* [F_shared,d] bf16 (shared expert) */
    const uint16_t* s_up;         /* [F_shared,d] bf16 */
    const uint16_t* s_down;       /* [d,F_shared] bf16 */
    const uint8_t* w_gate_scale;  /* MOE_WEIGHTS_FP8 / FP4: block scales */
    const uint8_t* w_up_scale;    /* MOE_WEIGHTS_FP8 / FP4 */
    const uint8_t* w_down_scale;  /* MOE_WEIGHTS_FP8 / FP4 */
} moe_weights;
#define MOE_WEIGHTS_FP8 2
#define MOE_WEIGHTS_FP4 3
#define MOE_WEIGHTS_A8W4 4

/* Workspace for moe_forward (all intermediates: logits, routing, permutation,
 * x_perm, h, y_perm and the shared expert's h and y) [HP 2.3 MegaMoE: one
 * workspace reused across the fused chain].  moe_workspace_size is the same
 * size under the name of the layer's one workspace; 0 for an invalid cfg
 * (NULL, T < 0, E < 1 or k < 1). */
size_t moe_forward_workspace_size(const moe_cfg* cfg);
size_t moe_workspace_size(const moe_cfg* cfg);

/* Reads the device error-flag word (the MOE_FLAG_* bits that moe_route,
 * moe_permute, moe_route_backward and moe_forward OR into *d_flags) into
 * *out after all work queued on `stream` so far has completed.  Unlike every
 * other entry point it synchronises the host with the stream (a checking or
 * test call, not a per-step one).  d_flags is a device uint32; out a host
 * pointer.  MOE_ERR_NULL if either is NULL, MOE_ERR_HIP if the copy or the
 * synchronisation fails (then *out is not written). */
int moe_read_error_flags(const uint32_t* d_flags, void* stream, uint32_t* out);

/* x [T,d] bf16; input_ids [T] int32 (HASH) or NULL; modality [T] u8 or NULL;
 * y [T,d] (bf16 or fp32 per out_dtype).  Optional outputs (NULL = kept in the
 * workspace): logits_out [T,E] fp32, ids_out [T,k] int32, w_out [T,k] fp32. */
int moe_forward(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x,
                const int32_t* input_ids, const uint8_t* modality, void* y,
                float* logits_out, int32_t* ids_out, float* w_out, uint32_t* d_flags,
                void* ws, size_t ws_bytes, void* stream);

/* moe_forward that also records caller-created hipEvent_t handles on the
 * stream around its stages, for per-stage timing: events[0] before the first
 * stage and events[i + 1] after stage i, i < MOE_FORWARD_STAGES, in the order
 *   0 router projection, 1 routing, 2 dispatch permutation (+ row gather),
 *   3 routed gate/up GEMM + clamped SwiGLU, 4 shared gate/up GEMM,
 *   5 routed down GEMM, 6 shared down GEMM, 7 combine.
 * Stages that do no work (no shared expert) still record their event.
 * events may be NULL (= moe_forward). */
#define MOE_FORWARD_STAGES 8
int moe_forward_timed(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x,
                      const int32_t* input_ids, const uint8_t* modality, void* y,
                      float* logits_out, int32_t* ids_out, float* w_out, uint32_t* d_flags,
                      void* ws, size_t ws_bytes, void* stream, void* const* events);

/* ------------------------------------------------------------------------
 * Whole layer backward [HP 2.3: MegaGate's fused backward chain of the gate's
 * normalisation gradients, MegaMoE's expert matmuls; HP 03: the training run
 * whose step this is].  For an output gradient dy of moe_forward's output y,
 * the gradients of y with respect to x and every weight.  The forward's
 * intermediates are recomputed from x (router logits, routes, dispatch,
 * expert pre-activations, h, expert outputs); then, in reverse order:
 *   combine:      dy_perm[dest[t,j]] = w[t,j] dy[t], d_w[t,j] = <dy[t], y_perm[dest]>
 *   down:         dW_down[e] = dy_perm_e^T h_e,  dh = dy_perm W_down
 *   SwiGLU:       dG, dU from dh through the clamps (moe_swiglu_backward)
 *   gate / up:    dW_gate[e] = dG_e^T x_e, dW_up[e] = dU_e^T x_e,
 *                 dx_perm = dG W_gate + dU W_up
 *   dispatch:     dx[t] = sum_j dx_perm[dest[t,j]]
 *   routing:      d_logits from d_w (moe_route_backward)
 *   router:       dx[t] += d_logits[t] W_g, dW_g = d_logits^T x
 *   shared:       the same FFN chain on x with dy (dWs_*, dx += its input
 *                 gradient).
 * Gradients enter the matrix products as bf16 (round to nearest even), as
 * the activations do; every product accumulates in fp32; the outputs are
 * fp32.  The ranking bias and the logit offset get no gradient (the bias
 * only ranks; the offset is a fixed input), nor does the hash table.
 *   cfg, w: as moe_forward, with w->packed == 1 (bf16 packed weights); x,
 *   input_ids, modality: the forward's inputs; dy [T,d] fp32.
 *   bw: the weights in the layouts of the input-gradient products, each
 *   written once per weight update by moe_pack_weights with panel_rows 256:
 *     w_g        [E,d] bf16 router weights, plain row-major;
 *     w_down_t   W_down^T, [E,F,d];
 *     w_gu_t     [W_gate; W_up]^T per expert, [E,d,2F] (column o of
 *                expert e: W_gate[e][:,o] then W_up[e][:,o]);
 *     s_down_t   Ws_down^T [F_shared,d]; s_gu_t [Ws_gate; Ws_up]^T [d,2F_shared]
 *                (NULL when F_shared = 0).
 *   g: outputs, all fp32, every entry written: dx [T,d], dw_g [E,d], dw_gate
 *   and dw_up [E,F,d], dw_down [E,d,F], ds_gate and ds_up [F_shared,d],
 *   ds_down [d,F_shared] (NULL when F_shared = 0).
 *   ws: moe_backward_workspace_size(cfg) bytes, 256-byte aligned.  With T = 0
 *   nothing is written.  d multiple of 8; E <= 1024.
 */
typedef struct moe_bwd_weights {
    const uint16_t* w_g;
    const uint16_t* w_down_t;
    const uint16_t* w_gu_t;
    const uint16_t* s_down_t;
    const uint16_t* s_gu_t;
} moe_bwd_weights;

typedef struct moe_grads {
    float* dx;
    float* dw_g;
    float* dw_gate;
    float* dw_up;
    float* dw_down;
    float* ds_gate;
    float* ds_up;
    float* ds_down;
} moe_grads;

size_t moe_backward_workspace_size(const moe_cfg* cfg);
int moe_backward(const moe_cfg* cfg, const moe_weights* w, const moe_bwd_weights* bw,
                 const uint16_t* x, const int32_t* input_ids, const uint8_t* modality,
                 const float* dy, const moe_grads* g, uint32_t* d_flags, void* ws,
                 size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
