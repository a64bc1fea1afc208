// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Record a HIP error for moe_last_hip_error() on this thread; returns MOE_ERR_HIP (7).
int record_hip_error(hipError_t e);

// ---- router
size_t route_workspace_bytes(int T, int E);
hipError_t launch_route(const uint16_t* x, int T, int d, const float* W, int E, const float* bias, int k,
                        int renorm, int* idx, float* gate, void* ws, hipStream_t stream);
hipError_t launch_route_logits(const uint16_t* x, int T, int d, const float* W, int E, const float* bias,
                               double* logits, hipStream_t stream);
hipError_t launch_route_topk(const double* logits, int T, int E, int k, int renorm, int* idx, float* gate,
                             hipStream_t stream);

// ---- allocation
hipError_t launch_alloc(const float* gate, int P, int n_star, int b_lo, int b_max, uint8_t* bits, float* tau_out,
                        int* n_hi_out, hipStream_t stream);
hipError_t launch_bits_threshold(const float* gate, int P, float tau, int b_lo, int b_max, uint8_t* bits,
                                 hipStream_t stream);
hipError_t launch_bits_threshold_dev(const float* gate, int P, const float* tau, int b_lo, int b_max, uint8_t* bits,
                                     hipStream_t stream);

// ---- FFN workspace plan
struct FfnShape {
  int T, k, E, B, g;     // tokens, top-k, routed experts, b_max, quant group
  int d, f;              // routed hidden / intermediate
  int n_shared, fs;      // shared experts and their intermediate size (0 if none)
  int P, Pt;             // routed pairs, all pairs (routed + shared)
  int W;                 // 32-token words per bitmap row
  int max_rchunks;       // routed chunk capacity
  int n_schunks;         // shared chunks
  int fmax;              // max(f, fs)
  int cs;                // pairs per chunk: 16 (decode), or 64 (prefill: four 16-token blocks)
  int sub;               // 16-token blocks per chunk (cs / 16)
  const int* bprefix;    // routed bank's per-expert plane prefix [E+1] (device), or null (uniform)
  int act_shared;        // one token: the plan wrote one activation fragment that every chunk reads
};

struct FfnLayout {
  size_t pair_key, bitmap, prefix, colerr, keycnt, slot_pair, pair_slot, slot_info, chunks, chunk_cnt, meta,
      expert_off, expert_maxbits;
  size_t xg, xvg, hg, hsg, obuf;  // chunk activation fragments and sums, gate/up output, down output
  size_t hsgg;                    // wide chunks: group sums of the gate/up output
  size_t total;
};

FfnShape make_shape(int T, int k, int E, int B, int g, int d, int f, int n_shared, int fs);
FfnLayout make_layout(const FfnShape& s);

struct MatrixDev {
  const uint32_t* planes;
  const float* sz;
  int N, K;
};

// Plan: permutation, histogram, chunks.
hipError_t launch_plan(const FfnShape& s, const FfnLayout& L, char* ws, const int* idx, const uint8_t* bits,
                       hipStream_t stream);
// Fused decode control (softmax + top-k, allocation, plan) in one block.
struct FfnLayout;
bool control_fits(const FfnShape& s);
bool control_does_topk(const FfnShape& s);
hipError_t launch_control(const FfnShape& s, const FfnLayout& L, char* ws, const double* logits, int renorm,
                          int n_star, int b_lo, int b_max, int* idx, float* gate, uint8_t* bits,
                          hipStream_t stream);
// One token: softmax + top-k (when logits is not null; else idx and bits are
// inputs), allocation, plan and the token's activation fragment in one block.
bool one_token_fits(const FfnShape& s);
hipError_t launch_one(const FfnShape& s, const FfnLayout& L, char* ws, const uint16_t* x, const double* logits,
                      int renorm, int n_star, int b_lo, int b_max, int* idx, float* gate, uint8_t* bits,
                      hipStream_t stream);
// Activation fragments of every chunk (after the plan).
hipError_t launch_gather(const FfnShape& s, const FfnLayout& L, char* ws, const uint16_t* x, hipStream_t stream);
hipError_t launch_ffn_w13(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                          int num_cu, hipStream_t stream);
hipError_t launch_ffn_w2(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                         int num_cu, hipStream_t stream);
hipError_t launch_combine(const FfnShape& s, const FfnLayout& L, char* ws, const float* gate, float* y,
                          int accumulate, hipStream_t stream);

// ---- DuoRate per-expert widths
hipError_t launch_duo_bake(MatrixDev m, int B, int g, int E, double* delta, hipStream_t stream);
hipError_t launch_duo_profile(const uint16_t* x, int T, int d, const int* idx, int k, int E, double* a, int* n,
                              hipStream_t stream);
hipError_t launch_duo_solve(const double* delta, const double* a, const int* n, int E, int d, int B, int b_lo,
                            int b_max, long long tmant, int tshift, double* D, uint8_t* widths, double* lam_out,
                            hipStream_t stream);
hipError_t launch_bits_from_expert(const int* idx, int P, const uint8_t* w, int E, uint8_t* bits, hipStream_t stream);

// ---- DPA-MoE residual-aware chunk allocation
hipError_t launch_resid_sum(const double* d13, const double* d2, int E, int B, int d, int f, double* resid,
                            hipStream_t stream);
hipError_t launch_dpa_alloc(const float* gate, const int* idx, int P, const double* resid, int E, int B, int b_lo,
                            int n_chunks, float* scores, uint8_t* chosen, uint8_t* bits, int* n_chosen_out,
                            hipStream_t stream);

// ---- helpers
hipError_t launch_dequant(MatrixDev m, int B, int g, int expert, int bits, const int* bprefix, float* out,
                          hipStream_t stream);
hipError_t launch_residual_to_bf16(const float* h, uint16_t* x, int64_t n, hipStream_t stream);
hipError_t launch_rmsnorm_to_bf16(const float* h, uint16_t* x, int rows, int d, float eps, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int sink_len, hipStream_t stream);

}  // namespace moe
