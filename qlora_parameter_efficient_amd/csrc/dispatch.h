// Internal entry points of the kernel translation units, called by api.cpp
// after validation.  All shapes and pointers are already checked.
#pragma once

#include "common.h"

namespace lq {

int launch_nf4_quantize(const void* W, lq_dtype wdt, int64_t n, int32_t double_quant,
                        uint8_t* codes, uint8_t* q8, float* c2, float* absmax,
                        hipStream_t stream);
int launch_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* c2,
                          const float* absmax, int32_t double_quant, int64_t n, void* out,
                          lq_dtype odt, hipStream_t stream);
int launch_zero_f32(float* p, int64_t n, hipStream_t stream);

int f32_lora_fwd(const float* X, int64_t M, const lq_weight& W, const float* A, const float* B,
                 int64_t r, float s, float* Y, float* T, hipStream_t st);
int f32_lora_bwd(const float* dY, const float* X, int64_t M, const lq_weight& W, const float* A,
                 const float* B, int64_t r, float s, const float* T_saved, float* dX, float* dA,
                 float* dB, int accumulate, float* ws, hipStream_t st);
int f32_lora_merge(const lq_weight& W, const float* A, const float* B, int64_t r, float s,
                   float* Wout, hipStream_t st);

// Partial sums of T = X A^T kept by the decode path.
constexpr int kTParts = 8;

namespace dispatch {

size_t grad_partial_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
size_t multi_ws_bytes(int64_t T_tokens, int64_t r, int32_t n_adapters);

int bf16_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
             int64_t r, float s, void* Y, float* T_out, hipStream_t st);
// Decode path (M <= 16): T partial sums (kTParts x M x r floats) go to Tp;
// T_out (optional) receives T.
int decode_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T_out, float* Tp, hipStream_t st);
int bf16_bwd(const void* dY, const void* X, int64_t M, const lq_weight& W, const void* A,
             const void* B, int64_t r, float s, const float* T_saved, void* dX, float* dA,
             float* dB, int accumulate, void* ws, hipStream_t st);
int bf16_merge(const lq_weight& W, const void* A, const void* B, int64_t r, float s, void* Wout,
               hipStream_t st);
int bf16_fwd_multi(const void* X, int64_t T_tokens, const lq_weight& W, const void* A_stack,
                   const void* B_stack, int32_t n_adapters, int64_t r, float s,
                   const int32_t* seg_offsets, const int32_t* seg_adapter, int32_t n_seg, void* Y,
                   void* ws, hipStream_t st);

}  // namespace dispatch
}  // namespace lq
