/*
 * moe_anyprec.h -- C ABI of libmoe_anyprec.so, a dynamic any-precision
 * Mixture-of-Experts FFN layer for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer whose expert weights are stored once as most-significant-bit
 * first bitplanes (up to 4 planes, per-group fp32 scale and zero point) and
 * read, per (token, expert) pair, at a bit-width chosen at run time from the
 * live router gate scores.  The steps follow these pages:
 *   - "DPA-MoE: A Runtime Precision Control Framework for MoE Inference"
 *     (abstract): prefix-decodable chunks, allocation after routing from
 *     live gate scores, one checkpoint at many budgets.
 *   - "MatMoE: Matryoshka Mixture-of-Experts with Dynamic Mixed-Precision
 *     Quantization for Efficient Inference" (abstract; review, Core
 *     Contribution): floor-and-compensation reads, a routing-score threshold
 *     set by binary search to hit a target average bit-width, bitplane
 *     storage.
 *   - "DuoRate: Two-Rate Per-Expert Precision Allocation for
 *     Mixture-of-Experts Serving" (abstract): a decode step pays only for
 *     the experts it selects; the stream is prefix-readable.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *     and allocates every buffer, workspaces included; the library never
 *     allocates, frees or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *     work is enqueued on it; outputs are valid once the stream completes.
 *   - bf16 values travel as uint16_t bit patterns.
 *   - The returned status reflects argument validation (done on the host in
 *     O(1), before any HIP call, so it works on a host without a GPU) and
 *     launch errors.  Data-dependent contract violations (an expert index
 *     out of range, a bit-width outside [1, b_max], duplicate experts in one
 *     token's top-k) never make a kernel read or write out of bounds: such
 *     pairs are dropped from the output (of duplicates, the first pair with a
 *     valid width is kept).
 *   - Where this interface departs from the plainest layer signature:
 *     the plane words are tiled (16-row tiles, 128-column blocks, see the
 *     bank struct) instead of row-major [N][K/32], and (scale, zero) is
 *     [N/16][K/group][2][16] instead of [N][K/group][2], so one 64-lane
 *     load reads a whole matrix-core operand; moe_route takes a workspace
 *     for its float64 logits; top_k is at most 8 (the combine keeps a
 *     token's slots in registers); `stream` is a void* so that the header
 *     needs no HIP include.
 *   - No C++ exception crosses the ABI.  The library keeps no state between
 *     calls except a cached device property, so calls are thread-safe; calls
 *     that share a workspace must be ordered on one stream.
 */
#ifndef MOE_ANYPREC_H
#define MOE_ANYPREC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL                          */
  MOE_ERR_SHAPE = 2,        /* a size is inconsistent (e.g. d not a multiple of 128) */
  MOE_ERR_ALIGN = 3,        /* a buffer is not 16-byte aligned                      */
  MOE_ERR_RANGE = 4,        /* an argument is outside its documented range          */
  MOE_ERR_WORKSPACE = 5,    /* workspace too small                                  */
  MOE_ERR_UNSUPPORTED = 6,  /* valid but not supported by this library              */
  MOE_ERR_HIP = 7           /* a HIP call failed; see moe_last_hip_error()          */
} moe_status;

/*
 * One bank of experts (routed or shared), described by a HOST struct whose
 * pointers are device pointers.  Storage format (the stored checkpoint; "one
 * encoded checkpoint" of the DPA-MoE abstract, "bitplane storage" of the
 * MatMoE review, Core Contribution):
 *
 *   Matrix W13 of an expert is 2*d_ff x d_model (rows 0..d_ff-1 gate
 *   projection, rows d_ff..2*d_ff-1 up projection); W2 is d_model x d_ff
 *   (down projection).  Each weight has an unsigned code q in
 *   [0, 2^b_max - 1]; plane p (p = 0 first) holds bit b_max-1-p of q.
 *
 *   *_planes: uint32 words [E][b_max][N/16 * 16*K/32] for an N x K matrix.
 *     Plane-major, so the first b planes of a matrix are one contiguous
 *     prefix.  Within a plane: 16-row tiles of 16*K/32 words each; within a
 *     tile, for 128-column block kb (K/128 blocks) and 32-column chunk j of
 *     it, row r of the tile has its word at  64*kb + 16*j + r,  and bit i of
 *     that word is column 128*kb + 32*j + i.
 *   *_sz: float32 [E][N/16][K/group][2][16]: for tile, quant group G (columns
 *     G*group .. G*group+group-1): the scales s of the tile's 16 rows, then
 *     their zero points z.  z is integer-valued in [0, 2^b_max - 1].  (s, z) is shared by every read
 *     width ("SharedScale", DPA-MoE abstract; "shared quantization
 *     parameters", MatMoE review).
 *
 *   Reading b planes gives, with delta = b_max - b, the floor-and-compensation
 *   weight (MatMoE review, Core Contribution, F&C paragraph):
 *       w = ((q >> delta) * 2^delta + (2^delta - 1)/2 - z) * s.
 *
 *   Requirements: 1 <= n_experts; d_model, d_ff multiples of 128; group in
 *   {64, 128}; 1 <= b_max <= 4; planes and sz 16-byte aligned.
 *
 *   Per-expert maximum width (MatMoE review, Core Contribution: each expert's
 *   maximum bit-width, 2/3/4, is chosen offline under a memory budget):
 *   plane_prefix is NULL for a uniform bank (every expert stores b_max
 *   planes), or a DEVICE int32 array [n_experts + 1] with plane_prefix[0] = 0
 *   for a ragged bank: expert e stores B_e = plane_prefix[e+1] -
 *   plane_prefix[e] planes (1 <= B_e <= b_max, b_max the largest), its codes
 *   are B_e-bit, and its planes are planes plane_prefix[e] ..
 *   plane_prefix[e+1]-1 of *_planes, viewed as [sum B_e][N/16 * 16*K/32]
 *   (the same tiled words per plane; (scale, zero) keep their [E] layout).
 *   A pair of width b reads min(b, B_e) planes, with floor and compensation
 *   relative to B_e.  Only routed banks may be ragged; the DuoRate and DPA
 *   bakes take uniform banks.  The prefix is not validated (a contract).
 */
typedef struct {
  int32_t n_experts;
  int32_t d_model;
  int32_t d_ff;
  int32_t group;
  int32_t b_max;
  const uint32_t* w13_planes;
  const float* w13_sz;
  const uint32_t* w2_planes;
  const float* w2_sz;
  const int32_t* plane_prefix;
} moe_expert_bank;

/* ------------------------------------------------------------------------ */
/* Router                                                                    */

/* Workspace bytes moe_route needs for T tokens and E experts (host, pure). */
size_t moe_route_workspace_bytes(int32_t T, int32_t E);

/*
 * Router: logits l[t][e] = sum_i W_r[e][i] * x[t][i] (+ logit_bias[e]),
 * accumulated in float64 from exact bf16/fp32 inputs; softmax over all E
 * experts; the top_k experts ordered by (logit descending, index
 * ascending); gate = softmax probability of each chosen expert, divided by
 * the sum over the chosen k if renorm_topk != 0.  ("routing each token to a
 * small set of experts", DPA-MoE abstract; "routing scores", MatMoE
 * abstract.)
 *   x          [T][d] bf16, 16-byte aligned
 *   w_router   [E][d] fp32, 16-byte aligned
 *   logit_bias [E] fp32 or NULL
 *   topk_idx   [T][top_k] int32 (output)
 *   topk_gate  [T][top_k] fp32  (output)
 *   workspace  >= moe_route_workspace_bytes(T, E) bytes, 16-byte aligned,
 *              any content: it receives the T x E float64 logits and is
 *              overwritten by every call (reusable without clearing).
 * Ranges: T >= 0 (T == 0 is a no-op), d multiple of 128, 1 <= E <= 256,
 * 1 <= top_k <= min(E, 8).
 */
moe_status moe_route(const uint16_t* x, int32_t T, int32_t d, const float* w_router,
                     int32_t E, const float* logit_bias, int32_t top_k, int32_t renorm_topk,
                     int32_t* topk_idx, float* topk_gate, void* workspace, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Bit allocation                                                            */

/*
 * Threshold allocation over the P live routed pairs (MatMoE abstract, item
 * (3), and review, Core Contribution: pairs whose routing score exceeds a
 * threshold read high precision, the rest low, the threshold found by binary
 * search to hit a target average bit-width; DPA-MoE abstract: allocation
 * after routing from live gate scores).
 *   n*   = floor(P * (target - b_lo) / (b_max - b_lo)), exact rational
 *          arithmetic on the float target, clamped to [0, P];
 *   tau  = the smallest fp32 value with #{gate > tau} <= n*, found on the
 *          device by bisection over the bit pattern of tau (32 steps);
 *   bits[i] = b_max if gate[i] > tau, else b_lo.
 * Equal gate scores are never split: the number of high pairs n_hi is the
 * largest count a threshold can realise that does not exceed n*.
 *   gate   [P] fp32 (any order; typically topk_gate viewed as [T*top_k])
 *   bits   [P] uint8 (output)
 *   tau_out  fp32 scalar or NULL (output; -inf when every pair is high)
 *   n_hi_out int32 scalar or NULL (output)
 * Ranges: P >= 0 (P == 0 is a no-op), 1 <= b_lo <= b_max <= 4,
 * b_lo <= target <= b_max.  Gates must not be NaN.
 */
moe_status moe_alloc_bits(const float* gate, int32_t P, int32_t b_lo, int32_t b_max,
                          float target_avg_bits, uint8_t* bits, float* tau_out,
                          int32_t* n_hi_out, void* stream);

/*
 * Calibration-threshold mode (MatMoE review, Core Contribution: the routing
 * score threshold is set on a calibration distribution of scores to meet the
 * target average, then applied to each pair as it is routed):
 *   bits[i] = b_max if gate[i] > tau (fp32 comparison), else b_lo
 * for i < P.  A threshold calibrated once (for instance the tau_out of
 * moe_alloc_bits over a calibration set of gate scores) is reused across
 * decode steps, so a step's average width varies around the target instead
 * of meeting it exactly.
 *   gate [P] fp32 device, bits [P] uint8 device (output), tau host scalar
 *   (-inf: every pair high).
 * Ranges: P >= 0, 1 <= b_lo <= b_max <= 4, tau not NaN; else MOE_ERR_RANGE.
 */
moe_status moe_bits_from_threshold(const float* gate, int32_t P, float tau, int32_t b_lo, int32_t b_max,
                                   uint8_t* bits, void* stream);

/*
 * The same widths with tau read from device memory (a float32 scalar), for a
 * controller that follows a changing target without a host round trip:
 * when the target changes, moe_alloc_bits over the stored calibration gate
 * scores writes the new tau to that scalar (its tau_out); every step then
 * calls this with the routed gates.  NaN tau is a contract violation (every
 * pair low).
 * Ranges: P >= 0, 1 <= b_lo <= b_max <= 4.
 */
moe_status moe_bits_from_threshold_device(const float* gate, int32_t P, const float* tau, int32_t b_lo,
                                          int32_t b_max, uint8_t* bits, void* stream);

/* n* computed on the host exactly as moe_alloc_bits does (pure). */
int32_t moe_budget_pairs(int32_t P, int32_t b_lo, int32_t b_max, float target_avg_bits);

/* ------------------------------------------------------------------------ */
/* Any-precision expert FFN                                                  */

/*
 * Workspace bytes for moe_anyprec_ffn / moe_permute (host, pure).  `shared`
 * may be NULL.  Returns 0 if the arguments are invalid.
 */
size_t moe_ffn_workspace_bytes(const moe_expert_bank* routed, const moe_expert_bank* shared,
                               int32_t T, int32_t top_k);

/*
 * The layer's expert computation at per-pair bit-widths:
 *   for every pair (t, j) with e = topk_idx[t][j], b = bits[t*top_k + j]:
 *     g = W_gate^(b) x_t,  u = W_up^(b) x_t   (fp32 accumulation)
 *     h = bf16_round(silu(g) * u)             (silu(v) = v / (1 + e^-v))
 *     o = W_down^(b) h
 *   y[t] = (accumulate ? y[t] : 0) + sum_j topk_gate[t][j] * o_(t,j)
 *          + sum_s FFN_shared_s^(b_max)(x_t)     (shared experts, weight 1)
 * where W^(b) is the floor-and-compensation read of the first b planes.
 * Each expert's planes are streamed once per group of up to 16 of its
 * pairs, at the largest width any of those pairs needs; every pair only
 * uses its own planes (the read is masked per pair), so the result is the
 * per-pair definition above ("pays only for the experts it selects",
 * DuoRate abstract; prefix reads, DPA-MoE abstract).
 *   x          [T][d_model] bf16, 16-byte aligned
 *   topk_idx   [T][top_k] int32, entries in [0, routed->n_experts), distinct per token
 *   topk_gate  [T][top_k] fp32
 *   bits       [T*top_k] uint8 in [1, routed->b_max]
 *   y          [T][d_model] fp32 (output; read too if accumulate != 0), 16-byte aligned
 *   workspace  >= moe_ffn_workspace_bytes(...), 256-byte aligned, any content
 * shared: NULL or a bank with the routed bank's d_model, group and b_max;
 * all of its n_experts experts are applied to every token at b_max planes.
 * Ranges: T >= 0 (T == 0 is a no-op), 1 <= top_k <= min(E, 8), E <= 256.
 */
moe_status moe_anyprec_ffn(const moe_expert_bank* routed, const moe_expert_bank* shared,
                           const uint16_t* x, int32_t T, int32_t top_k,
                           const int32_t* topk_idx, const float* topk_gate,
                           const uint8_t* bits, float* y, int32_t accumulate,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * The whole layer in one call: moe_route (without a separate workspace),
 * moe_alloc_bits over the call's T*top_k routed pairs, then moe_anyprec_ffn,
 * with the same results as those three calls in sequence (the passages they
 * cite).  For decode-sized batches (T*top_k <= 1024 and
 * n_experts*b_max*ceil(T/32) <= 4096) the allocation and the FFN's plan run
 * as one single-block kernel, with the softmax + top-k too when T <= 16.
 *   x, w_router, logit_bias, renorm_topk   as for moe_route (d = routed->d_model,
 *                                          E = routed->n_experts)
 *   b_lo, target_avg_bits                  as for moe_alloc_bits (b_max = routed->b_max)
 *   topk_idx [T][top_k], topk_gate [T][top_k], bits [T*top_k]   outputs, device
 *   y, accumulate                          as for moe_anyprec_ffn
 *   workspace  >= moe_layer_workspace_bytes(...), 256-byte aligned, any content
 * Ranges and errors: those of the three calls.
 */
size_t moe_layer_workspace_bytes(const moe_expert_bank* routed, const moe_expert_bank* shared, int32_t T,
                                 int32_t top_k);
moe_status moe_layer(const moe_expert_bank* routed, const moe_expert_bank* shared, const uint16_t* x, int32_t T,
                     int32_t top_k, const float* w_router, const float* logit_bias, int32_t renorm_topk,
                     int32_t b_lo, float target_avg_bits, int32_t* topk_idx, float* topk_gate, uint8_t* bits,
                     float* y, int32_t accumulate, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_layer for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as moe_layer, without the workspace: the
 * call uses a static device array of the library (its size is
 * moe_layer_static_scratch_bytes(), 64 MiB, enough for decode batches of up
 * to 256 tokens on the Qwen3-30B-A3B shape), and calls no allocating
 * routine.  A call whose moe_layer_workspace_bytes exceeds that size returns
 * MOE_ERR_WORKSPACE.  Each GPU holds one such array until the process ends,
 * shared by every call on that GPU and keeping the last call's contents:
 * no part of it needs to start at zero (every call writes what it reads),
 * but calls that overlap in time on one GPU (on different streams or host
 * threads) race on it and must be ordered by the caller.
 */
size_t moe_layer_static_scratch_bytes(void);
moe_status moe_layer_static(const moe_expert_bank* routed, const moe_expert_bank* shared, const uint16_t* x,
                            int32_t T, int32_t top_k, const float* w_router, const float* logit_bias,
                            int32_t renorm_topk, int32_t b_lo, float target_avg_bits, int32_t* topk_idx,
                            float* topk_gate, uint8_t* bits, float* y, int32_t accumulate, void* stream);

/*
 * The token-to-expert permutation and histogram step of moe_anyprec_ffn, on
 * its own, for inspection.  Pairs are ordered stably by (expert ascending,
 * bits descending, pair id ascending), pair id = t*top_k + j.
 *   slot_pair       [T*top_k] int32 (output): pair id at each sorted position
 *                   (the kept pairs first, then -1 once per dropped pair)
 *   expert_offsets  [E+1] int32 (output): first sorted position of each expert
 *   expert_maxbits  [E] int32 (output): largest bit-width among the expert's
 *                   pairs (0 for an expert with no pair)
 * The workspace is the same as for moe_anyprec_ffn.
 */
moe_status moe_permute(const int32_t* topk_idx, const uint8_t* bits, int32_t T, int32_t top_k,
                       int32_t E, int32_t b_max, int32_t* slot_pair, int32_t* expert_offsets,
                       int32_t* expert_maxbits, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* DuoRate: per-expert read widths for a workload                            */
/*
 * "DuoRate: Two-Rate Per-Expert Precision Allocation for Mixture-of-Experts
 * Serving" (abstract): the bank is stored once (one uniform tier of b_max
 * prefix-readable planes); offline a distortion tensor is baked from it;
 * online a prefill of the workload is profiled without labels, and each
 * expert's decode read width is chosen by a Lagrangian rate-distortion
 * solve under the decode rate (bits read per routed pair), in which routing
 * frequency cancels from every per-expert decision, at the cost of one dot
 * product per expert and width plus a bisection.  Decode steps then read
 * every pair of expert e at width b_e (moe_bits_from_expert_widths feeds
 * moe_anyprec_ffn unchanged).
 */

/*
 * Bake the distortion tensor of a bank (offline):
 *   delta[e][b-1][c] = sum over the 2*d_ff rows n of W13 of
 *                      (s(n, c) * (q(n, c) - qhat_b(n, c)))^2,
 * the squared change of input column c's gate/up weights when expert e is
 * read at b planes instead of all b_max (qhat_b: the floor-and-compensation
 * code of the first b planes; the zero-point terms of both reads cancel).
 *   delta  [n_experts][b_max][d_model] float64, device, 8-byte aligned (output)
 * Errors: those of the bank (see moe_expert_bank), MOE_ERR_NULL.
 */
moe_status moe_duorate_bake(const moe_expert_bank* bank, double* delta, void* stream);

/*
 * Profile a prefill batch (label-free): for every expert e,
 *   pair_count[e]    = number of routed pairs (t, j) with topk_idx[t][j] == e,
 *   act_energy[e][c] = sum over those pairs, in pair order, of x[t][c]^2 (float64).
 *   x [T][d] bf16, topk_idx [T][top_k] int32 (entries outside [0, E) are
 *   skipped), act_energy [E][d] float64 (output, 8-byte aligned),
 *   pair_count [E] int32 (output).  All device.
 * Ranges: T >= 0 (T == 0 writes zeros), d >= 1, top_k >= 1, 1 <= E <= 1024.
 */
moe_status moe_duorate_profile(const uint16_t* x, int32_t T, int32_t d, const int32_t* topk_idx, int32_t top_k,
                               int32_t E, double* act_energy, int32_t* pair_count, void* stream);

/*
 * Solve for per-expert widths:
 *   distortion[e][b-1] = <delta[e][b-1], act_energy[e]> / pair_count[e]
 *                        (0 when pair_count[e] == 0), the expected squared
 *                        error of the expert's gate/up pre-activations per
 *                        routed token, for b = 1..b_max;
 *   b_e(lam) = argmin over b in [b_lo, b_max] of distortion[e][b-1] + lam*b
 *              (float64, no fused multiply-add, ties to the smaller b);
 *   lam* = the smallest non-negative double with
 *          sum_e pair_count[e] * b_e(lam) <= floor(target_rate * sum_e pair_count[e]),
 *          found by bisection over the bit patterns of doubles in
 *          [0, 2 * max_e distortion[e][b_lo-1] + 1];
 *   expert_bits[e] = b_e(lam*); *lambda_out = lam* (if not NULL).
 *   delta       [E][b_max][d] float64 as baked from a bank with this b_max
 *   act_energy  [E][d] float64, pair_count [E] int32   (moe_duorate_profile)
 *   distortion  [E][b_max] float64 (output), expert_bits [E] uint8 (output),
 *   lambda_out  float64 scalar or NULL (output).  All device.
 * Ranges: 1 <= E <= 1024, d >= 1, 1 <= b_lo <= b_max <= 4,
 * b_lo <= target_rate <= b_max.
 */
moe_status moe_duorate_solve(const double* delta, const double* act_energy, const int32_t* pair_count, int32_t E,
                             int32_t d, int32_t b_lo, int32_t b_max, float target_rate, double* distortion,
                             uint8_t* expert_bits, double* lambda_out, void* stream);

/*
 * Per-pair widths of a batch from per-expert widths:
 *   bits[i] = expert_bits[topk_idx[i]] for i < P (topk_idx viewed as [P]),
 *   0 where the index is outside [0, E) (such pairs are dropped by the FFN).
 * Ranges: P >= 0, E >= 1.
 */
moe_status moe_bits_from_expert_widths(const int32_t* topk_idx, int32_t P, const uint8_t* expert_bits, int32_t E,
                                       uint8_t* bits, void* stream);

/* ------------------------------------------------------------------------ */
/* DPA-MoE: residual-aware chunk allocation over widths b_lo..b_max          */
/*
 * "DPA-MoE: A Runtime Precision Control Framework for MoE Inference"
 * (abstract): per-expert reconstruction residuals are profiled offline and
 * chunks (planes) are allocated at inference time from live router gate
 * scores, so one encoded checkpoint runs at many budgets.  The abstract
 * states no rule; the one built here: every pair reads b_lo planes, and the
 * extra planes go to the candidate (pair, plane) chunks that remove the most
 * gate-weighted residual.
 */

/* Workspace bytes of moe_dpa_residuals (host, pure; 0 for an invalid bank). */
size_t moe_dpa_residuals_workspace_bytes(const moe_expert_bank* bank);

/*
 * Offline residual profile of a bank:
 *   resid[e][b-1] = ||W_hat^(b_max) - W_hat^(b)||_F^2 over both matrices of
 *                   expert e (W13 and W2), float64, for b = 1..b_max
 *                   (resid[e][b_max-1] = 0); the stored uniform tier is the
 *                   reference.
 *   resid  [n_experts][b_max] float64, device, 8-byte aligned (output)
 *   workspace >= moe_dpa_residuals_workspace_bytes(bank), 256-byte aligned,
 *   any content (per-column sums of both matrices).
 */
moe_status moe_dpa_residuals(const moe_expert_bank* bank, double* resid, void* workspace, size_t ws_bytes,
                             void* stream);

/* Workspace bytes of moe_dpa_alloc for P pairs (host, pure). */
size_t moe_dpa_alloc_workspace_bytes(int32_t P, int32_t b_lo, int32_t b_max);

/*
 * Residual-aware widths of the P live routed pairs:
 *   score(p, k) = fp32(fp64(gate[p])^2 * (resid[e][k-2] - resid[e][k-1])),
 *                 e = topk_idx[p], for the extra planes k = b_lo+1..b_max
 *                 (0 for an index outside [0, E));
 *   budget      = floor(P * (target - b_lo)) extra planes, exact on the float
 *                 target, at most P * (b_max - b_lo);
 *   the candidates of highest score are chosen, as many as the budget allows
 *   without splitting equal scores (the threshold bisection of
 *   moe_alloc_bits, run over the candidates);
 *   bits[p] = b_lo + number of chosen candidates of pair p;
 *   *n_chunks_out = chosen candidates (device int32, or NULL).
 *   gate [P] fp32, topk_idx [P] int32, resid [E][b_max] float64
 *   (moe_dpa_residuals), bits [P] uint8 (output).  All device.
 *   workspace >= moe_dpa_alloc_workspace_bytes(P, b_lo, b_max), 256-byte
 *   aligned, any content.
 * Ranges: P >= 0, E >= 1, 1 <= b_lo <= b_max <= 4, b_lo <= target <= b_max,
 * P * (b_max - b_lo) < 2^30.
 */
moe_status moe_dpa_alloc(const float* gate, const int32_t* topk_idx, int32_t P, const double* resid, int32_t E,
                         int32_t b_lo, int32_t b_max, float target_avg_bits, uint8_t* bits, int32_t* n_chunks_out,
                         void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Helpers                                                                   */

/*
 * Materialise the floor-and-compensation weights of one matrix of one expert
 * read at `bits` planes: out[n][c] = fp32(((q>>delta)*2^delta + c_delta - z)*s)
 * with one rounding (MatMoE review, Core Contribution, F&C paragraph).
 *   matrix 0 = W13 (out [2*d_ff][d_model]), 1 = W2 (out [d_model][d_ff]).
 * Ranges: 0 <= expert < n_experts, 1 <= bits <= b_max.
 */
moe_status moe_dequant(const moe_expert_bank* bank, int32_t expert, int32_t matrix,
                       int32_t bits, float* out, void* stream);

/* x[i] = bf16_round_nearest_even(h[i]) for i < n: the next layer's input
 * from an fp32 residual stream.  n >= 0. */
moe_status moe_residual_to_bf16(const float* h, uint16_t* x, int64_t n, void* stream);

/*
 * The next layer's input from an fp32 residual stream with each row
 * RMS-normalised, as the Qwen3-MoE-shaped stacks do before every MoE layer
 * (the pages define the layer, not the stack around it; this is the reading
 * taken for a 48-layer stack, whose un-normalised residual overflows fp32
 * within a few SwiGLU layers):
 *   r = fp32(1 / sqrt(sum_c h[t][c]^2 / d + eps))   (squares and sum in fp64)
 *   x[t][c] = bf16_round_nearest_even(fp32(h[t][c] * r))
 * h [rows][d] fp32, x [rows][d] bf16 bits, both device, row-major, not
 * overlapping.  rows >= 0, d >= 1, 0 <= eps finite; otherwise MOE_ERR_RANGE.
 * A row of zeros needs eps > 0 (with eps = 0 its scale is infinite).
 */
moe_status moe_rmsnorm_to_bf16(const float* h, uint16_t* x, int32_t rows, int32_t d, float eps, void* stream);

/*
 * Measurement helper, for callers that compare a kernel's rate with what the
 * memory system can deliver: a pure streaming read of `bytes` bytes of `buf`
 * (16-byte loads, every byte read once, nothing else moved), the achievable
 * HBM read ceiling next to the 8 TB/s specification.  The loaded values are
 * folded into one uint32 per wave and written to sink[0 .. MOE_STREAM_SINK)
 * so the loads stay live; their values mean nothing.
 *   buf   device, 16-byte aligned, bytes a multiple of 16 (bytes >= 0)
 *   sink  device, MOE_STREAM_SINK uint32 entries, written
 */
#define MOE_STREAM_SINK 8192
moe_status moe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement hook for callers that time the two streaming kernels of the
 * FFN stage on their own (the roofline of the dominant kernel): while set,
 * every moe_anyprec_ffn and moe_layer call on this host thread records
 * w13_begin / w13_end on its stream right before / after the gate/up kernel,
 * and w2_begin / w2_end around the down kernel.  Arguments are hipEvent_t
 * handles (created and owned by the caller) passed as void*; NULL disables
 * that mark.  All NULL is the default.  Thread-local; no other effect.
 */
void moe_set_kernel_events(void* w13_begin, void* w13_end, void* w2_begin, void* w2_end);

/* Static description of a status code. */
const char* moe_status_string(moe_status status);

/* hipError_t of the last MOE_ERR_HIP returned on the calling thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ANYPREC_H */
