/*
 * mxmoe.h -- C ABI of the MXFP8 block-scaled top-k MoE expert layer for
 * AMD MI355X (gfx950).
 *
 * The layer (sources: "Quantization on Ascend", sglang docs, section on MXFP8
 * for LLM MoE models; "[WIP] Fix offline W8A8 MXFP8 quantization for Qwen3.5
 * on Ascend NPU", sglang PR 32266, commit adding the fused-experts chain):
 *
 *   moe_route_quant     top-k routing with the MX activation quant fused in
 *   gmm_swiglu_mxquant  grouped GEMM1 (gate + up) + SwiGLU + MX requant
 *   gmm_mx              grouped GEMM2 (down), bf16 output
 *   moe_finalize        weighted un-permute and sum of the top-k outputs
 *   moe_mxfp8_forward   the four steps above on one stream
 *   mx_quantize         stand-alone MX quantiser (weights at load time)
 *   moe_route_quant_noalloc
 *                       moe_route_quant without a workspace (allocates nothing)
 *   moe_router          top-k softmax router over a bf16 gate (upstream of
 *                       the layer: produces the ids and weights it takes)
 *   mx_linear           dense MXFP8 linear layer (activation quant + MX GEMM)
 *   mx_pack_weights, gmm_swiglu_mxquant_packed, gmm_mx_packed,
 *   moe_mxfp8_forward_packed
 *                       load-time weight cast into the GEMMs' tile layout,
 *                       and the GEMMs and the layer reading it
 *   mx_quantize_fp4     MXFP4 (e2m1) quantiser for the W4A8 path's weights
 *   gmm_swiglu_mxquant_w4a8, gmm_mx_w4a8, moe_w4a8_forward
 *                       the GEMMs and the layer with MXFP4 expert weights
 *
 * Formats.  MXFP8 = e4m3 payload bytes plus one e8m0 scale byte (exponent +
 * 127, value 2^(byte-127)) per 32 consecutive elements along the reduction
 * dimension.  A row of Kd elements has ceil(Kd/32) scales, padded with one
 * zero byte when that count is odd, stored as [ceil(Kd/64), 2] pairs: the
 * pair-split layout ("Quantization on Ascend", offline MoE path: [E,N,K/32]
 * scales viewed as [E,N,K/64,2]; PR 32266 Summary, offline partial block-scale
 * layout, worked example K = 4304 -> 135 -> 136 -> 68 pairs).  There is no zero
 * point.  Quantisation: s = floor(log2(amax)) - 8 clamped to [-127, 127]
 * (scale byte s + 127; an all-zero block gets byte 0), payload = e4m3 of
 * x * 2^-s rounded to nearest, ties to even, saturating at +-448, sign kept
 * (so -0 and negative values that round to zero give 0x80).
 *
 * Finite inputs only.  Every bf16/fp32 input (x, bf16 weights, topk_w) must
 * be finite: the pages fix no NaN or infinity convention for MX blocks and
 * the library does not check (a device-side scan would cost a full read).
 * What non-finite inputs produce is not part of the contract; with the
 * current kernels a NaN drops out of its block's amax and encodes as -448
 * times the block scale (code 0xFE), and an infinity sets its block's scale
 * byte to 247 and flushes the block's other elements to zero.  No error is
 * reported for either.
 *
 * Tensors.  Every pointer is a DEVICE pointer unless stated; all tensors are
 * dense row-major.  bf16 is passed as its 16-bit pattern.  Sizes are int64_t.
 *   x            bf16   [T, K]
 *   topk_ids     int32  [T, k]   expert ids in [0, E)
 *   topk_w       fp32   [T, k]   routing weights
 *   w13          uint8  [E, 2I, K]   e4m3; rows [0, I) gate, rows [I, 2I) up
 *   w13_s        uint8  [E, 2I, K/64, 2]
 *   w2           uint8  [E, K, I]    e4m3
 *   w2_s         uint8  [E, K, I/64, 2]
 *   group_list   int64  [E]  type 1: rows per expert (counts);
 *                            type 0: inclusive cumulative counts
 *   M = T*k expanded rows; expert e owns a contiguous run of rows in expert
 *   order, and inside one expert rows keep the order of the flat assignment
 *   index t*k + j (a stable sort).
 *
 * Ownership and execution.  The caller allocates every buffer, including
 * the workspaces (sized by the *_workspace_size queries).  The library never
 * allocates, frees or retains pointers and never synchronises the host.
 * Every call enqueues work on `stream` (a hipStream_t passed as void*; NULL =
 * the null stream) and returns at once; results are ready when the stream
 * reaches them.  Calls on different streams must not share output or
 * workspace buffers.
 *
 * Errors.  Every entry point returns MX_OK (0) or a negative mx_status.
 * Argument checks happen on the host before anything is enqueued; on error
 * nothing is enqueued and mx_last_error() (thread-local) describes why.
 * Data-dependent conditions are handled on the device without faulting:
 * an expert id outside [0, E) is dropped (its expanded_row_idx entry is -1,
 * it counts toward no expert, so sum(group_list) < T*k tells the caller), and
 * group lists are clamped to [0, M] rows.
 *
 * GPU shape limits (MX_ERR_UNSUPPORTED otherwise): every size argument at
 * most 2^31 - 1, and M = T*k at most 2^27 for routing and the layer (below
 * 2^31 for the GEMMs and finalize); GEMM reduction dims (K of GEMM1,
 * I of GEMM2) multiples of 128 and at most 2^20; GEMM2 output dim N a
 * multiple of 256;
 * GEMM1 intermediate size I a multiple of 128 (so the forward needs K % 256
 * == 0 and I % 128 == 0); routing needs K % 32 == 0, K <= 2^24,
 * 1 <= k <= 256 and E <= 1024; mx_quantize takes any Kd >= 1.
 *
 * Alignment (MX_ERR_UNSUPPORTED otherwise): e4m3 payload and bf16 tensors
 * that the GEMMs, routing and finalize read or write (x, xq, a, w, w13, w2,
 * hq, y, out, the forward workspace) start on 16-byte boundaries, their scale
 * tensors (a_s, w_s, w13_s, w2_s, hs) on 4-byte boundaries, h_f32_debug on 16.
 * mx_quantize accepts any alignment (a slower path handles the rest).
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, k > E, bad group_list_type */
  MX_ERR_UNSUPPORTED = -2, /* a shape the GPU kernels do not handle (see above) */
  MX_ERR_WORKSPACE = -3,   /* workspace smaller than the size query returned */
  MX_ERR_HIP = -4          /* a HIP runtime error at launch */
} mx_status;

/*
 * MX-quantise `rows` rows of `kd` bf16 elements (row stride `ld` elements,
 * ld >= kd) into e4m3 payload q [rows, kd] (row stride kd bytes) and scales
 * s [rows, ceil(kd/64), 2] (odd scale counts padded with a zero byte).
 * Used on expert weights at load time ("Quantization on Ascend", MoE online
 * path: bf16 [E, N, K] expert weights quantised once, 3-D input taken as
 * E*N rows) and for activations that bypass routing.
 */
int mx_quantize(const void* x_bf16, int64_t rows, int64_t kd, int64_t ld,
                void* q_u8, void* s_u8, void* stream);

/*
 * MXFP4-quantise `rows` rows of `kd` bf16 elements (row stride `ld`) into
 * packed e2m1 codes q [rows, kd/2] (element 2i in the low nibble of byte i)
 * and e8m0 scales s [rows, ceil(kd/64), 2]: the weights of the W4A8 path
 * ("Quantization on Ascend", W4A8 implementation notes: weights packed FP4,
 * float4_e2m1fn_x2, two nibbles per byte, one UE8M0 scale per 32 elements;
 * activations stay MXFP8).  Per 32-block: s = floor(log2(amax)) - 2 clamped
 * to [-127, 127] (byte s + 127, an all-zero block gets 0), codes = nearest of
 * +-{0, .5, 1, 1.5, 2, 3, 4, 6} to x * 2^-s, ties to the even code,
 * saturating at 6, sign kept.  kd % 32 == 0 (MX_ERR_UNSUPPORTED otherwise).
 */
int mx_quantize_fp4(const void* x_bf16, int64_t rows, int64_t kd, int64_t ld,
                    void* q_u8, void* s_u8, void* stream);

/* Workspace bytes moe_route_quant needs for T tokens, top-k, E experts
 * (0 when T*k <= 256: the call then accepts a null workspace). */
size_t moe_route_quant_workspace_size(int64_t T, int64_t k, int64_t E);

/*
 * Top-k routing with fused MX activation quant ("Quantization on Ascend",
 * MoE forward: routing quantises the activations in the same op; PR 32266,
 * commit on the fused routing quant: byte-identical to routing then
 * quantising).  Outputs, for M = T*k:
 *   xq                uint8 [M, K]        row p = MX payload of token sorted_row[p] / k
 *   xs                uint8 [M, K/64, 2]  its scales (pair-split)
 *   sorted_row        int32 [M]           flat assignment index t*k+j of row p
 *   expanded_row_idx  int32 [M]           row p of flat assignment i (-1 if its id was invalid)
 *   group_list        int64 [E]           rows per expert (count form, type 1)
 * Rows past sum(group_list) (only when ids were invalid) are left unwritten.
 * One kernel launch.  Its workgroups exchange per-chunk expert counts through
 * the workspace under flags tagged per call, so the workspace needs no
 * clearing; a workgroup that finds the counts not yet published after a
 * bounded number of polls (moe_route_quant_set_wait_limit) counts them from
 * topk_ids itself, so the call always ends and its output never depends on
 * the order the GPU runs the workgroups in.  Called while `stream` is
 * capturing, the call also records a one-thread kernel ahead of the routing
 * kernel that advances a generation word in the workspace, so that every
 * replay of the captured graph tags its flags afresh.
 */
int moe_route_quant(const void* x_bf16, const int32_t* topk_ids,
                    int64_t T, int64_t K, int64_t k, int64_t E,
                    void* xq_u8, void* xs_u8, int32_t* sorted_row,
                    int32_t* expanded_row_idx, int64_t* group_list,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_route_quant for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and results as moe_route_quant minus the workspace:
 * the routing scratch (per-chunk expert counts, the experts' offsets and
 * the flags that publish them) is a 4 MiB device array inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller still passes every input and
 * output.  Sizes whose scratch, moe_route_quant_workspace_size(T, k, E),
 * exceeds 4 MiB (4,194,304 bytes) are rejected with MX_ERR_UNSUPPORTED
 * before anything is enqueued (e.g. E = 128, k = 8: up to 261,056 tokens).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and must not be
 * issued; calls ordered on one stream are safe.  The array needs no
 * clearing: each call writes every count it reads before reading it, and
 * its flags match only the tag of the call that set them.
 */
int moe_route_quant_noalloc(const void* x_bf16, const int32_t* topk_ids,
                            int64_t T, int64_t K, int64_t k, int64_t E,
                            void* xq_u8, void* xs_u8, int32_t* sorted_row,
                            int32_t* expanded_row_idx, int64_t* group_list,
                            void* stream);

/*
 * How many times a routing workgroup polls for the published expert counts
 * before counting them from topk_ids itself (process-wide, default 2^18;
 * 0 makes every workgroup count for itself: much slower, same output).
 * Applies to launches enqueued after the call; returns the previous value.
 * Negative values are taken as 0.  Meant for tests of that path.
 */
int64_t moe_route_quant_set_wait_limit(int64_t polls);

/*
 * Grouped GEMM1 with SwiGLU and MX requant fused ("Quantization on Ascend",
 * MoE forward: GEMM1 fuses gate/up, SwiGLU and requant and hands back
 * quantised activations plus block scales; "PR #30768 report", key source
 * excerpt: it takes a cumulative group list, the dispatcher produces counts).
 * For expert e and its rows m:
 *   acc = A[m] . W13_e^T (fp32 accumulation), g = acc[:, :I], u = acc[:, I:],
 *   h = silu(g) * u (fp32), (hq, hs) = MX quantisation of h along I.
 *   a      uint8 [M, K], a_s [M, K/64, 2]
 *   hq     uint8 [M, I], hs  [M, I/64, 2]
 *   h_f32_debug  fp32 [M, I] or NULL: when given, also receives h.
 * group_list_type: 0 = cumulative, 1 = count.  Rows not owned by any expert
 * are not written.
 */
int gmm_swiglu_mxquant(const void* a_u8, const void* a_s,
                       const void* w13_u8, const void* w13_s,
                       const int64_t* group_list, int group_list_type,
                       int64_t M, int64_t K, int64_t I, int64_t E,
                       void* hq_u8, void* hs_u8, float* h_f32_debug,
                       void* stream);

/*
 * Grouped MX GEMM with bf16 output (GEMM2, down projection; "Quantization on
 * Ascend", MoE forward: the second grouped GEMM takes the count group list).
 *   y[m, :] = bf16_rne( A[m] . W_e^T )  for the expert e owning row m
 *   a  uint8 [M, Kd], a_s [M, Kd/64, 2];  w uint8 [E, N, Kd], w_s [E, N, Kd/64, 2]
 *   y  bf16 [M, N]
 */
int gmm_mx(const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
           const int64_t* group_list, int group_list_type,
           int64_t M, int64_t N, int64_t Kd, int64_t E,
           void* y_bf16, void* stream);

/*
 * Tile-packed expert weights: the weights' load-time cast into the layout
 * the GEMMs' LDS ring holds, the counterpart of the pages' cast of expert
 * weights into the matrix unit's tiled format once at load ("PR #30768
 * report", review highlights: the NZ format; PR 32266, the commit casting
 * weights to NZ).  mx_pack_weights rewrites e4m3 weights w [E, N, Kd] into
 * out (same size, E*N*Kd bytes, must not overlap w): for expert e, n-tile
 * nt = 0 .. N/256 - 1 and k stage ks = 0 .. Kd/128 - 1, the 32 KB block at
 * byte ((e*(N/256) + nt)*(Kd/128) + ks)*32768 holds 256 rows of 128 bytes,
 * 16-byte chunk c of block row r at chunk position c ^ ((r/2) % 8).  Block
 * row r is weight row 256*nt + r for kind 0 (GEMM2 weights w2 [E, K, I]);
 * for kind 1 (GEMM1 weights w13 [E, 2I, K], I = N/2) block rows
 * [128h, 128h+64) are gate rows 128*nt + 64h + (0..63) and block rows
 * [128h+64, 128h+128) up rows I + 128*nt + 64h + (0..63), h = 0, 1.
 * Scales are not packed: the *_packed calls take them in the usual
 * [E, N, Kd/64, 2] layout.  Needs N % 256 == 0, Kd % 128 == 0, E <= 1024.
 *
 * gmm_swiglu_mxquant_packed, gmm_mx_packed and moe_mxfp8_forward_packed
 * are gmm_swiglu_mxquant, gmm_mx and moe_mxfp8_forward with w13 packed as
 * kind 1 and w2 (w) packed as kind 0; arguments, results and limits are
 * otherwise the same (the results are identical byte for byte).
 */
int mx_pack_weights(const void* w_u8, int64_t E, int64_t N, int64_t Kd, int kind,
                    void* out_u8, void* stream);

int gmm_swiglu_mxquant_packed(const void* a_u8, const void* a_s,
                              const void* w13_packed, const void* w13_s,
                              const int64_t* group_list, int group_list_type,
                              int64_t M, int64_t K, int64_t I, int64_t E,
                              void* hq_u8, void* hs_u8, float* h_f32_debug,
                              void* stream);

int gmm_mx_packed(const void* a_u8, const void* a_s, const void* w_packed,
                  const void* w_s, const int64_t* group_list, int group_list_type,
                  int64_t M, int64_t N, int64_t Kd, int64_t E, void* y_bf16,
                  void* stream);

/*
 * Finalize: weighted un-permute and sum (PR 32266, fused-experts commit:
 * the chain ends with finalize routing).
 *   out[t, :] = bf16_rne( sum_{j=0}^{k-1} w[t, j] * y[expanded_row_idx[t*k+j], :] )
 * accumulated in fp32 in ascending j, each product and sum rounded to fp32.
 * Entries whose index is outside [0, M) are skipped.
 *   y bf16 [M, K], topk_w fp32 [T, k], expanded_row_idx int32 [T*k], out bf16 [T, K]
 */
int moe_finalize(const void* y_bf16, const float* topk_w,
                 const int32_t* expanded_row_idx, int64_t T, int64_t K,
                 int64_t k, int64_t M, void* out_bf16, void* stream);

/*
 * W4A8 variants ("Quantization on Ascend", W4A8 implementation notes: expert
 * weights packed FP4 with a UE8M0 scale per 32 elements, activations per-token
 * MXFP8).  Same arguments, semantics, limits and errors as gmm_swiglu_mxquant
 * and gmm_mx, except that the weight payload is packed e2m1 (mx_quantize_fp4):
 *   w13 uint8 [E, 2I, K/2] (gate rows [0, I), up rows [I, 2I)),
 *   w   uint8 [E, N, Kd/2]; element 2c in the low nibble of byte c.
 * Scales keep the [.., K/64, 2] layout.  GEMM1's output hq/hs stays MXFP8.
 */
int gmm_swiglu_mxquant_w4a8(const void* a_u8, const void* a_s,
                            const void* w13_u8, const void* w13_s,
                            const int64_t* group_list, int group_list_type,
                            int64_t M, int64_t K, int64_t I, int64_t E,
                            void* hq_u8, void* hs_u8, float* h_f32_debug,
                            void* stream);
int gmm_mx_w4a8(const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
                const int64_t* group_list, int group_list_type,
                int64_t M, int64_t N, int64_t Kd, int64_t E,
                void* y_bf16, void* stream);

/* Workspace bytes moe_mxfp8_forward needs (holds every intermediate). */
size_t moe_mxfp8_forward_workspace_size(int64_t T, int64_t K, int64_t I,
                                        int64_t E, int64_t k);

/*
 * The whole layer on one stream: moe_route_quant -> gmm_swiglu_mxquant ->
 * gmm_mx -> moe_finalize (PR 32266, fused-experts commit; "Quantization on
 * Ascend", MoE forward).  Weights are pre-quantised (see mx_quantize).
 * out bf16 [T, K].  Intermediates live in the workspace.
 */
int moe_mxfp8_forward(const void* x_bf16, const int32_t* topk_ids,
                      const float* topk_w, const void* w13_u8,
                      const void* w13_s, const void* w2_u8, const void* w2_s,
                      int64_t T, int64_t K, int64_t I, int64_t E, int64_t k,
                      void* out_bf16, void* workspace, size_t ws_bytes,
                      void* stream);

/* moe_mxfp8_forward with tile-packed weights (see mx_pack_weights). */
int moe_mxfp8_forward_packed(const void* x_bf16, const int32_t* topk_ids,
                             const float* topk_w, const void* w13_packed,
                             const void* w13_s, const void* w2_packed,
                             const void* w2_s, int64_t T, int64_t K, int64_t I,
                             int64_t E, int64_t k, void* out_bf16, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * The whole layer with MXFP4 expert weights (the W4A8 path): as
 * moe_mxfp8_forward with w13 uint8 [E, 2I, K/2] and w2 uint8 [E, K, I/2]
 * packed e2m1 (see gmm_swiglu_mxquant_w4a8); same workspace and layout.
 */
int moe_w4a8_forward(const void* x_bf16, const int32_t* topk_ids,
                     const float* topk_w, const void* w13_u8,
                     const void* w13_s, const void* w2_u8, const void* w2_s,
                     int64_t T, int64_t K, int64_t I, int64_t E, int64_t k,
                     void* out_bf16, void* workspace, size_t ws_bytes,
                     void* stream);

/* Byte offsets of the intermediates inside the forward workspace, so a caller
 * can inspect them after the stream has run.  Fills the 8 offsets in order:
 * xq, xs, sorted_row, expanded_row_idx, group_list, hq, hs, y. */
int moe_mxfp8_forward_workspace_layout(int64_t T, int64_t K, int64_t I,
                                       int64_t E, int64_t k,
                                       size_t* offsets_host);

/*
 * Top-k softmax router over a bf16 gate linear, the step upstream of
 * moe_route_quant ("Quantization on Ascend", MXFP8 for LLM MoE models,
 * implementation notes: the router gate is a plain linear layer, kept in bf16
 * on the online path).  For each token t:
 *   logits[e] = sum_c x[t,c] * gate[e,c] (+ bias[e])   fp32 accumulation of
 *               the exact bf16 products
 *   topk_ids[t, :] = the k largest logits, descending (equal logits: the
 *                    lower expert id first)
 *   topk_w[t, j]   = softmax(logits)[topk_ids[t, j]], divided by the sum of
 *                    the k selected when renormalize != 0
 *   x bf16 [T, K], gate bf16 [E, K], bias fp32 [E] or NULL (-inf allowed:
 *   that expert is never picked while a finite one is left);
 *   topk_ids int32 [T, k], topk_w fp32 [T, k] (the inputs of moe_route_quant,
 *   moe_finalize and moe_mxfp8_forward).
 * Limits: K % 64 == 0, E <= 256 (MX_ERR_UNSUPPORTED); 1 <= k <= E
 * (MX_ERR_INVALID_ARG); x and gate 16-byte aligned.
 */
int moe_router(const void* x_bf16, const void* gate_bf16, const float* bias,
               int64_t T, int64_t K, int64_t E, int64_t k, int renormalize,
               int32_t* topk_ids, float* topk_w, void* stream);

/* Workspace bytes mx_linear needs for T tokens of K features. */
size_t mx_linear_workspace_size(int64_t T, int64_t K);

/*
 * Dense MXFP8 linear layer ("Quantization on Ascend", MXFP8 (dense)
 * implementation notes: weights MX-quantised once at load (see mx_quantize),
 * activations MX-quantised per token at inference, block 32 along K, then the
 * quantised matmul):
 *   (xq, xs) = MX quantisation of x along K (as mx_quantize)
 *   y[t, n]  = bf16_rne( sum over 32-blocks b of 2^(sx[t,b] + sw[n,b]) * (xq[t,b] . wq[n,b]) )
 *   x bf16 [T, K]; w uint8 [N, K] e4m3; w_s uint8 [N, K/64, 2]; y bf16 [T, N].
 * The workspace (mx_linear_workspace_size, 256-byte aligned) holds xq and
 * xs.  Limits as gmm_mx with one group: K % 128 == 0,
 * N % 256 == 0.
 */
int mx_linear(const void* x_bf16, const void* w_u8, const void* w_s,
              int64_t T, int64_t K, int64_t N, void* y_bf16,
              void* workspace, size_t ws_bytes, void* stream);

/* Description of the last non-OK status returned on this thread. */
const char* mx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
