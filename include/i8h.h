/*
 * i8h — routed-expert gate_up of a weight-quantized MoE layer, on one
 * AMD Instinct MI355X (gfx950). C ABI of libi8h.so.
 *
 * The format comes from the model card "Gemma 4 26B-A4B-it + DFlash, int8
 * experts — radiance container" (model table, row "Weights"; section "How
 * this file was made", the recipe line of the routed experts' gate_up): int8
 * codes in -127..127 stored in the 128-wide Hadamard domain, one bf16 scale
 * per output row and per 128 of K. The FP8 variant comes from "Gemma 4
 * 26B-A4B-it + DFlash, FP8 experts — radiance container" (model table, row
 * "Weights"; its recipe): E4M3 codes per 128x128 block with one bf16 scale
 * per block.
 *
 * Conventions shared by every call:
 *   - All array pointers are DEVICE pointers, allocated and owned by the
 *     caller. The library allocates nothing and keeps no state between calls.
 *   - bf16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and return: no device synchronisation,
 *     no device-to-host copy, and grid sizes never depend on device data.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation error nothing is enqueued. I8H_EHIP reports a launch error
 *     from the HIP runtime. Faults during execution surface at the caller's
 *     next synchronisation.
 *   - T == 0 (no tokens) is a valid no-op that returns I8H_OK.
 *   - Calls are thread-safe and reentrant; calls on different streams may
 *     overlap as long as their output buffers do not alias.
 *   - Row-major layouts throughout; the last index is contiguous.
 *   - bf16 scale arrays (4-byte aligned, as each call requires) are read by
 *     the MFMA and GEMV kernels in aligned 4-byte words: when a scale array holds an
 *     odd number of elements, the 2 bytes after its last element are read
 *     (never used, never written). Allocations of HIP and torch are rounded
 *     to at least 256 bytes, so such a read stays inside the allocation.
 *
 * Sizes: T tokens, K hidden size (K % 128 == 0), E experts (1..1024),
 * topk experts per token (1..min(E, 32)), N = 2*I gate_up rows per expert
 * (rows 0..I-1 are the gate rows, rows I..2I-1 the matching up rows),
 * P = T*topk (token, slot) pairs, G = K/128 groups.
 */
#ifndef I8H_H
#define I8H_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I8H_OK = 0,
  I8H_EINVAL = -1,       /* invalid argument: null pointer, size, alignment */
  I8H_EUNSUPPORTED = -2, /* well-formed but outside what the kernels handle */
  I8H_EHIP = -3          /* the HIP runtime refused a launch */
} i8h_status;

/* Static, human-readable name of a status code. Never NULL. */
const char* i8h_status_string(int status);

/* Upper limits checked by every entry point. */
#define I8H_MAX_EXPERTS 1024
#define I8H_MAX_TOPK 32

/* ------------------------------------------------------------------------
 * Routing: top-k over router logits, per-expert histogram, exclusive scan
 * and a stable scatter of the (token, slot) pairs into expert-sorted order.
 *
 * The int8 card's model table (row "Weights") describes routed experts picked
 * by a router; it prints no rule, so: token t takes the topk experts of
 * largest logit, ties to the lower expert index, slot j = j-th in that order;
 * topk_w[t, j] = softmax over the topk chosen logits (float32 arithmetic).
 * Pair p = t*topk + j. expert_off is the exclusive scan of per-expert pair
 * counts (expert_off[E] = P); sorted_pairs[expert_off[e] .. expert_off[e+1])
 * lists expert e's pairs in increasing p; pair_pos[p] is the position of p
 * in sorted_pairs. All integer outputs are deterministic, bit for bit.
 *
 * logits      [T, E] float32. A NaN ranks after every number (-inf
 *             included), NaNs among themselves by index like ties, so every
 *             id is an expert in [0, E); a token whose chosen logits hold a
 *             NaN (or only -inf) gets NaN weights.
 * topk_ids    [T, topk] int32 out
 * topk_w      [T, topk] float32 out
 * expert_off  [E + 1] int32 out
 * sorted_pairs[P] int32 out
 * pair_pos    [P] int32 out
 * workspace   device scratch of at least moe_route_permute_workspace_size()
 *             bytes (may be NULL when that size is 0): one histogram of E
 *             int32 counts per chunk of c = max(1, min(floor(256 / topk),
 *             ceil(T / 32))) whole tokens, C = ceil(T / c) chunks (none for
 *             T <= 4); contents on entry are ignored. P must stay below
 *             2^31, and C * E too (else I8H_EUNSUPPORTED).
 * ---------------------------------------------------------------------- */
size_t moe_route_permute_workspace_size(int T, int E, int topk);
int moe_route_permute(const float* logits, int T, int E, int topk,
                      int32_t* topk_ids, float* topk_w, int32_t* expert_off,
                      int32_t* sorted_pairs, int32_t* pair_pos,
                      void* workspace, size_t workspace_bytes, void* stream);

/* moe_route_permute that also rotates the activation rows of the tokens it
 * routes: the int8 card's model table (row "Needs") puts the 128-wide
 * Hadamard rotation in the producer of the experts' input, and the routing
 * is that producer here. Same routing outputs, rules and workspace as
 * moe_route_permute, bit for bit; x_rot equals hadamard128_rotate(x) bit for
 * bit. x [T, K] bf16 (K % 128 == 0, rows contiguous, 16-B aligned), x_rot
 * [T, K] bf16 out (16-B aligned); x == x_rot (in place) is allowed, other
 * overlap is not; T*K < 2^31 (else I8H_EUNSUPPORTED). For many tokens the
 * rotation runs inside the routing kernel (one launch fewer than the two
 * calls); for T <= 4 it is a launch of its own after the routing. */
int moe_route_permute_rotate(const float* logits, const uint16_t* x, int T, int E, int topk, int K,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_off,
                             int32_t* sorted_pairs, int32_t* pair_pos, uint16_t* x_rot,
                             void* workspace, size_t workspace_bytes, void* stream);

/* moe_route_permute without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same inputs, outputs, rules and results,
 * bit for bit. The call allocates nothing: the histograms that the workspace
 * holds otherwise live in a fixed 1 MiB device array inside the library, one
 * per GPU, held until the process ends; so moe_route_permute_workspace_size
 * (T, E, topk) must not exceed 1 MiB (else I8H_EUNSUPPORTED; e.g. T*topk <=
 * 524,288 pairs at E = 128, topk = 8). The array's
 * device address is looked up on the first call on each device: the stream
 * must belong to the current device (else I8H_EHIP). Every call on one GPU
 * shares that array: calls that overlap on one GPU (on different streams, or
 * from several threads) race on it and give unspecified results; calls one
 * after another on a stream are safe (nothing in the array must start at
 * zero). */
int moe_route_permute_noalloc(const float* logits, int T, int E, int topk,
                              int32_t* topk_ids, float* topk_w, int32_t* expert_off,
                              int32_t* sorted_pairs, int32_t* pair_pos, void* stream);

/* ------------------------------------------------------------------------
 * Blockwise 128-wide Walsh-Hadamard rotation of bf16 activation rows.
 *
 * The int8 card's codes live in the 128-wide Hadamard domain (model table,
 * row "Weights"; recipe transform fwht128), so the activations must be
 * rotated the same way before the product; the card puts this in the
 * producer of the experts' input (row "Needs"). For every row t and block b:
 *   y[t, 128b + i] = bf16( sum_j H[i, j] * x[t, 128b + j] / sqrt(128) ),
 * H[i, j] = (-1)^popcount(i & j) (Sylvester, natural order). The butterflies
 * run in float32; the result is rounded once to bf16 (nearest even).
 *
 * x  [T, ldx] bf16, the first K columns are read; y [T, ldy] bf16 out.
 * ldx, ldy >= K and multiples of 8; x, y 16-byte aligned. x == y (in place)
 * is allowed; other overlap is not.
 * ---------------------------------------------------------------------- */
int hadamard128_rotate(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy,
                       int T, int K, void* stream);

/* ------------------------------------------------------------------------
 * Grouped int8 Hadamard-domain gate_up with the fused GELU-tanh epilogue.
 *
 * For the pair in expert-sorted row r (expert e = the run holding r,
 * token t = sorted_pairs[r] / topk):
 *   gu[r, n]  = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
 *   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i],  i < I = N/2,
 *   gelu_tanh(v) = v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3))).
 * The code-times-activation products are exact; sums are float32. Router
 * weights are not applied. Output rows stay in expert-sorted order.
 *
 * x_rot       [T, K] bf16, already rotated (hadamard128_rotate), 16-B aligned
 * codes       [E, N, K] int8 in -127..127, 16-B aligned
 * scales      [E, N, K/128] bf16, 4-byte aligned
 * expert_off  [E + 1], sorted_pairs [T*topk]: as moe_route_permute writes them
 * gate_up     [T*topk, N] float32 out, or NULL to skip storing it
 * act         [T*topk, N/2] float32 out, or NULL to skip storing it
 * N must be positive and even (odd: I8H_EINVAL); the kernels tile the gate
 * and up halves in 32-row pieces, so an N that is not a multiple of 64 is
 * I8H_EUNSUPPORTED.
 * ---------------------------------------------------------------------- */
int moe_gateup_i8h_grouped(const uint16_t* x_rot, int T, int K,
                           const int8_t* codes, const uint16_t* scales,
                           int E, int N, int topk,
                           const int32_t* expert_off, const int32_t* sorted_pairs,
                           float* gate_up, float* act, void* stream);

/* Same as moe_gateup_i8h_grouped with the kernel chosen by the caller:
 * I8H_PATH_AUTO (as the call above: GEMV for T <= 8 and K <= 4096, TALL when
 * the pairs average at least 32 per expert, else SKINNY), I8H_PATH_GEMV (the
 * decode-shaped kernel: VALU dot products streaming codes with 16-byte
 * loads), I8H_PATH_GEMM (bf16 MFMA, passes of 128 pairs, a second
 * accumulator per 128-K group) or I8H_PATH_TALL (bf16 MFMA, passes of 256
 * pairs, the running result kept in units of the current group's scale) or
 * I8H_PATH_SKINNY (bf16 MFMA for few pairs per expert: passes of 64 pairs,
 * units of 64 gate + 64 up columns, three workgroups per CU).
 * All give the same result to float32 rounding. TALL needs N*K < 2^31
 * (else I8H_EUNSUPPORTED); its running result spans 2^64 of scale range per
 * row: a group whose scale lies more than 2^64 below the largest scale before
 * it in the row contributes nothing (its terms are below 2^-64 of that
 * scale's), which keeps every intermediate finite for activations below 2^46
 * at K = 2048. */
enum { I8H_PATH_AUTO = 0, I8H_PATH_GEMV = 1, I8H_PATH_GEMM = 2, I8H_PATH_TALL = 3, I8H_PATH_SKINNY = 4 };
int moe_gateup_i8h_grouped_path(const uint16_t* x_rot, int T, int K,
                                const int8_t* codes, const uint16_t* scales,
                                int E, int N, int topk,
                                const int32_t* expert_off, const int32_t* sorted_pairs,
                                float* gate_up, float* act, int path, void* stream);

/* moe_gateup_i8h_grouped_path with act stored in bf16, the input the bf16
 * down projection takes (moe_down_bf16_combine_act_bf16): act_bf16
 * [T*topk, N/2] bf16 bits out, 2-B aligned, or NULL. Each value is the
 * float32 act of moe_gateup_i8h_grouped_path rounded to nearest even, so it
 * equals that call's act rounded the way the down projection rounds it;
 * gate_up stays float32. Same paths, limits and status codes. */
int moe_gateup_i8h_grouped_act_bf16(const uint16_t* x_rot, int T, int K,
                                    const int8_t* codes, const uint16_t* scales,
                                    int E, int N, int topk,
                                    const int32_t* expert_off, const int32_t* sorted_pairs,
                                    float* gate_up, uint16_t* act_bf16, int path, void* stream);

/* Same product with the rotation fused in: x is the UNROTATED bf16
 * activation [T, K]. The 128-wide Walsh-Hadamard rotation of
 * hadamard128_rotate is applied on the fly (the int8 card's model table, row
 * "Needs", puts the rotation in the producer of the experts' input; this call
 * is that fusion for callers whose producer does not rotate). For few tokens
 * (T <= 8, K <= 4096) the decode-shaped kernel rotates in its prologue and
 * the workspace is unused; otherwise the call rotates into the workspace and
 * runs the MFMA kernel. workspace: at least
 * moe_gateup_i8h_fused_workspace_size(T, K) bytes, 256-B aligned (may be NULL
 * when that size is 0). Results equal moe_gateup_i8h_grouped on the rotated
 * activations up to float32 rounding order in the rotation. */
size_t moe_gateup_i8h_fused_workspace_size(int T, int K);
int moe_gateup_i8h_grouped_fused(const uint16_t* x, int T, int K,
                                 const int8_t* codes, const uint16_t* scales,
                                 int E, int N, int topk,
                                 const int32_t* expert_off, const int32_t* sorted_pairs,
                                 float* gate_up, float* act,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Decode step in one launch: moe_route_permute, then
 * moe_gateup_i8h_grouped_fused, for a few tokens. Each workgroup ranks the
 * logits of every token itself and picks its expert from the result, so the
 * code stream starts without waiting for a routing kernel; one workgroup also
 * stores the routing outputs. Same inputs, outputs and rules as those two
 * calls (x is the UNROTATED activation), with the same bit-exact routing;
 * no workspace. Limits (else I8H_EUNSUPPORTED): T*topk <= 64, E <= 256,
 * K <= 4096. Needs at least one of gate_up and act; N even (odd: I8H_EINVAL)
 * and a multiple of 64 (else I8H_EUNSUPPORTED). */
int moe_route_gateup_i8h_decode(const float* logits, const uint16_t* x, int T, int K,
                                const int8_t* codes, const uint16_t* scales,
                                int E, int N, int topk,
                                int32_t* topk_ids, float* topk_w, int32_t* expert_off,
                                int32_t* sorted_pairs, int32_t* pair_pos,
                                float* gate_up, float* act, void* stream);

/* ------------------------------------------------------------------------
 * FP8 activation quantizer: per token and per 128 of K (one float32 scale
 * per token and 128 values, as the activations of the int8 12B card, header
 * table row "Format"):
 *   sx[t, g] = float32(amax_g / 448)            (IEEE single division)
 *   qx[t, kk] = E4M3FN(x[t, kk] / sx[t, g])      (nearest even, saturating
 *                                                at +-448; sign kept on zero)
 * a group with sx == 0 gets qx = 0. x [T, K] bf16 (16-B aligned); qx [T, K]
 * uint8 out (16-B aligned); sx [T, K/128] float32 out.
 * ---------------------------------------------------------------------- */
int fp8_quantize_activations(const uint16_t* x, int T, int K,
                             uint8_t* qx, float* sx, void* stream);

/* ------------------------------------------------------------------------
 * Grouped FP8 E4M3 128x128-block gate_up (FP8 card, model table row
 * "Weights"). Activations are unrotated bf16; the call first quantizes them
 * as fp8_quantize_activations does, into the workspace, then
 *   gu[r, n] = sum_g (sw[e, n/128, g] * sx[t, g])
 *                    * sum_{kk in g} E4M3(qw[e, n, kk]) * E4M3(qx[t, kk])
 * with the same epilogue, row order and outputs as moe_gateup_i8h_grouped.
 *
 * x [T, K] bf16; codes [E, N, K] E4M3FN bytes (finite); scales [E, N/128,
 * K/128] bf16, 4-byte aligned; N must be a positive multiple of 128 (whole 128-row scale
 * blocks). The products of decoded codes are exact and summed in float32
 * (the codes are expanded to bf16 for bf16 MFMA; gfx950's FP8 MFMA keeps
 * only about 13 bits below its largest product). Workspace (at least
 * moe_gateup_fp8blk_workspace_size(T, K) bytes, 256-B aligned base): qx
 * [T, K] uint8 at offset 0, sx [T, K/128] float32 at offset
 * A = round_up(T*K, 256), the exact bf16 values of qx [T, K] at offset
 * A + round_up(4*T*(K/128), 256). All are left there for the caller.
 * ---------------------------------------------------------------------- */
size_t moe_gateup_fp8blk_workspace_size(int T, int K);
int moe_gateup_fp8blk_grouped(const uint16_t* x, int T, int K,
                              const uint8_t* codes, const uint16_t* scales,
                              int E, int N, int topk,
                              const int32_t* expert_off, const int32_t* sorted_pairs,
                              float* gate_up, float* act,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Same as moe_gateup_fp8blk_grouped with the kernel chosen by the caller:
 * I8H_PATH_AUTO (as the call above: GEMM when the pairs average at least 32
 * per expert, else SKINNY), I8H_PATH_GEMM (bf16 MFMA, passes of 128 pairs,
 * units of 128 gate + 128 up columns) or I8H_PATH_SKINNY (bf16 MFMA for few
 * pairs per expert: passes of 64 pairs, units of 64 gate + 64 up columns,
 * several workgroups per CU). Both give the same result to float32 rounding
 * order. I8H_PATH_GEMV and I8H_PATH_TALL have no E4M3 form:
 * I8H_EUNSUPPORTED; any other value: I8H_EINVAL. */
int moe_gateup_fp8blk_grouped_path(const uint16_t* x, int T, int K,
                                   const uint8_t* codes, const uint16_t* scales,
                                   int E, int N, int topk,
                                   const int32_t* expert_off, const int32_t* sorted_pairs,
                                   float* gate_up, float* act,
                                   void* workspace, size_t workspace_bytes, int path,
                                   void* stream);

/* moe_gateup_fp8blk_grouped_path with act stored in bf16 (act_bf16
 * [T*topk, N/2] bf16 bits out, 2-B aligned, or NULL): each value the float32
 * act rounded to nearest even, as for moe_gateup_i8h_grouped_act_bf16. */
int moe_gateup_fp8blk_grouped_act_bf16(const uint16_t* x, int T, int K,
                                       const uint8_t* codes, const uint16_t* scales,
                                       int E, int N, int topk,
                                       const int32_t* expert_off, const int32_t* sorted_pairs,
                                       float* gate_up, uint16_t* act_bf16,
                                       void* workspace, size_t workspace_bytes, int path,
                                       void* stream);

/* ------------------------------------------------------------------------
 * The step after the path: bf16 grouped down projection of the routed
 * experts, then the weighted combine of each token's topk outputs.
 *
 * The int8 card's model table (row "Weights") keeps the experts' down
 * projections in bf16 as the checkpoint ships them; the pages show neither
 * that product nor the merge, so: W_down[e] is [H, I] (H = the hidden size);
 * the float32 act rows are rounded to bf16 (nearest even) for the product,
 * which accumulates in float32 (bf16 x bf16 products are exact there);
 *   y[r, h]   = sum_i W_down[e(r), h, i] * bf16(act[r, i])  (sorted row r)
 *   out[t, h] = sum_j topk_w[t, j] * y[pair_pos[t*topk + j], h]  (slot order)
 *
 * act        [P, I] float32, expert-sorted rows (the act of the gate_up calls),
 *            16-B aligned; I % 8 == 0
 * w_down     [E, H, I] bf16 bits, 16-B aligned; H % 8 == 0
 * topk_ids, topk_w, expert_off, pair_pos: as moe_route_permute wrote them
 * out        [T, H] float32 out, 16-B aligned
 * workspace  at least moe_down_bf16_workspace_size(T, I, H, topk) bytes,
 *            256-B aligned: the bf16 act rows and y, for the many-pairs form
 *            (unused, may be NULL, for the one-launch form)
 * Forms: for up to 64 pairs (and I <= 1024) one launch computes out directly
 * (a workgroup owns 8 rows h of a token and all its slots); otherwise act is
 * rounded into the workspace, a grouped bf16 MFMA GEMM writes y there
 * (needs I % 32 == 0, I >= 96, H % 256 == 0, P*I < 2^31) and a combine kernel merges
 * the slots. Outside both: I8H_EUNSUPPORTED. Results agree to float32
 * rounding order. */
size_t moe_down_bf16_workspace_size(int T, int I, int H, int topk);
int moe_down_bf16_combine(const float* act, int T, int I, const uint16_t* w_down,
                          int E, int H, int topk,
                          const int32_t* topk_ids, const float* topk_w,
                          const int32_t* expert_off, const int32_t* pair_pos,
                          float* out, void* workspace, size_t workspace_bytes, void* stream);

/* The same with the form chosen by the caller: I8H_DOWN_AUTO (as above),
 * I8H_DOWN_GEMV (the one-launch form, any T; I <= 1024) or I8H_DOWN_GEMM (the
 * GEMM + combine form; its limits above, workspace required). */
enum { I8H_DOWN_AUTO = 0, I8H_DOWN_GEMV = 1, I8H_DOWN_GEMM = 2 };
int moe_down_bf16_combine_path(const float* act, int T, int I, const uint16_t* w_down,
                               int E, int H, int topk,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_off, const int32_t* pair_pos,
                               float* out, void* workspace, size_t workspace_bytes,
                               int path, void* stream);

/* moe_down_bf16_combine_path on act already in bf16 (act_bf16 [P, I] bf16
 * bits, 16-B aligned, as moe_gateup_*_act_bf16 write it): the rounding step
 * is skipped, and the GEMM form reads act_bf16 directly, so its workspace
 * holds y only: at least moe_down_bf16_act_bf16_workspace_size(T, I, H, topk)
 * bytes, 256-B aligned (unused, may be NULL, for the one-launch form). Same
 * forms, limits and status codes; on act_bf16 = bf16(act) the results equal
 * moe_down_bf16_combine_path's on act bit for bit. */
size_t moe_down_bf16_act_bf16_workspace_size(int T, int I, int H, int topk);
int moe_down_bf16_combine_act_bf16(const uint16_t* act_bf16, int T, int I, const uint16_t* w_down,
                                   int E, int H, int topk,
                                   const int32_t* topk_ids, const float* topk_w,
                                   const int32_t* expert_off, const int32_t* pair_pos,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int path, void* stream);

/* ------------------------------------------------------------------------
 * Dense int8 linear with an f16 scale per row and 128 of K, no transform: the
 * DFlash drafter's linears and head on the int8 card (model table, row
 * "Speculator"; recipe lines `rtn codes=i8 group=128 scale=f16 clamp=sym`).
 *   y[t, n] = sum_g scales[n, g] * sum_{k in g} codes[n, k] * x[t, k]
 * x       [T, K] bf16 bits (unrotated), 16-B aligned; K % 128 == 0
 * codes   [N, K] int8 in -127..127, 16-B aligned; N % 16 == 0
 * scales  [N, K/128] f16 bits (IEEE binary16), 2-B aligned
 * y       [T, N] float32 out, 4-B aligned
 * Products exact in float32, float32 accumulation. Made for the drafter's
 * blocks of 16 positions: a workgroup owns 16 columns x 16 tokens, so larger
 * T re-reads the codes once per 16 tokens. No workspace. */
int linear_i8f16(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales,
                 int N, float* y, void* stream);

/* ------------------------------------------------------------------------
 * The W8A8 int8 g128 form ("Gemma 4 12B-it · int8 · for radiance", header
 * table row "Format", and "How it was made", step 2): int8 weights with one
 * bf16 scale per row and 128 of K, rounded to nearest, no rotation; int8
 * activations with one scale per token and 128 values. The int5 card's row
 * "Format" uses such activations above 64 rows: this is the prefill-shaped
 * form. Readings: the activation scale is float32,
 *   sx[t, g]   = float32(amax_g / 127)          (IEEE single division)
 *   qx[t, kk]  = round-half-even(float32(x / sx)), clamped to [-127, 127]
 * and a group with sx == 0 gets qx = 0. x [T, K] bf16 (16-B aligned), qx
 * [T, K] int8 out (8-B aligned), sx [T, K/128] float32 out (4-B aligned);
 * T*K < 2^31 (else I8H_EUNSUPPORTED).
 * ---------------------------------------------------------------------- */
int i8_quantize_activations(const uint16_t* x, int T, int K,
                            int8_t* qx, float* sx, void* stream);

/* Grouped gate_up in the W8A8 form: the call quantizes x (unrotated bf16
 * [T, K]) as i8_quantize_activations does into the workspace, then
 *   gu[r, n] = sum_g sw[e, n, g] * sx[t, g] * sum_{kk in g} qw[e, n, kk] * qx[t, kk]
 * with the epilogue, row order and outputs of moe_gateup_i8h_grouped. The
 * group sums are exact int32 (int8 MFMA); each is folded into the float32
 * result with sw * sx. codes [E, N, K] int8 in -127..127, 16-B aligned;
 * scales [E, N, K/128] bf16, 4-B aligned; N positive and even (odd:
 * I8H_EINVAL), a multiple of 64 and N*K < 2^31 (else I8H_EUNSUPPORTED).
 * Workspace: at least
 * moe_gateup_i8g_workspace_size(T, K) bytes, 256-B aligned: qx [T, K] int8
 * at offset 0, sx [T, K/128] float32 at offset round_up(T*K, 256), left there
 * for the caller. Passes of 192 pairs: one per expert at prefill sizes. */
size_t moe_gateup_i8g_workspace_size(int T, int K);
int moe_gateup_i8g_grouped(const uint16_t* x, int T, int K,
                           const int8_t* codes, const uint16_t* scales,
                           int E, int N, int topk,
                           const int32_t* expert_off, const int32_t* sorted_pairs,
                           float* gate_up, float* act,
                           void* workspace, size_t workspace_bytes, void* stream);

/* moe_gateup_i8g_grouped with act stored in bf16 (act_bf16 [T*topk, N/2] bf16
 * bits out, 2-B aligned, or NULL): each value the float32 act rounded to
 * nearest even, as for moe_gateup_i8h_grouped_act_bf16. */
int moe_gateup_i8g_grouped_act_bf16(const uint16_t* x, int T, int K,
                                    const int8_t* codes, const uint16_t* scales,
                                    int E, int N, int topk,
                                    const int32_t* expert_off, const int32_t* sorted_pairs,
                                    float* gate_up, uint16_t* act_bf16,
                                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* I8H_H */
