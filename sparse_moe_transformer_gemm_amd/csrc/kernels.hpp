// Launchers of the non-GEMM kernels (top-k, permute, tile list, combine+norm).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

// Tokens handled by one permute work-group (one per thread).
constexpr int kPermTokens = 256;

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int k, int32_t* idx,
                       float* w, hipStream_t st);

hipError_t launch_permute(const int32_t* idx, int64_t T, int E, int k, int32_t* bcounts, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, hipStream_t st);

// launch_permute and launch_tiles (one list, token-tile height bt) in one
// work-group, for T <= kPermTokens and E <= 1024; the same results.
hipError_t launch_permute_small(const int32_t* idx, int64_t T, int E, int k, int32_t* offsets, int32_t* sorted,
                                int32_t* pos, int bt, int4* tiles, int32_t* cnt, hipStream_t st);

// Tile lists of the expert GEMMs for token-tile heights bt_a and bt_b (0: skip b).
hipError_t launch_tiles(const int32_t* offsets, int E, int bt_a, int4* tiles_a, int32_t* cnt_a, int bt_b,
                        int4* tiles_b, int32_t* cnt_b, hipStream_t st);

// c_out / r_out (optional, fp32): the combined rows and each row's 1/rms.
hipError_t launch_combine_norm(bool bf16, const void* O, const int32_t* pos, const float* w, const float* gamma,
                               int64_t T, int L, int k, float eps, void* n, hipStream_t st, float* c_out = nullptr,
                               float* r_out = nullptr);

// Quantile Balancing: bias[e] = -(1 - k/E) quantile of sigmoid(logits[:, e]);
// keys: T * E uint32 scratch.
hipError_t launch_quantile_bias(const float* logits, int64_t T, int E, int k, uint32_t* keys, float* bias,
                                hipStream_t st);

// W8A8 activations: x[R, C] (bf16, or fp32 when x_f32; C a multiple of 128,
// row stride C) -> e4m3fn codes q[R, C] and fp32 scales sc[C/128, R]
// (scale = amax / 448 per row per 128 columns; code = e4m3fn(x / scale)).
hipError_t launch_quant_1x128(const void* x, bool x_f32, int64_t R, int C, void* q, float* sc, hipStream_t st);

// out[b, a] = s_tok[b, sorted[a] / k] for b < nb, a < T * k (row scales of
// the token rows in expert order).
hipError_t launch_gather_scales(const float* s_tok, int64_t T, int nb, const int32_t* sorted, int k, float* out,
                                hipStream_t st);

}  // namespace lmoe
