// Internal entry points of the kernel translation units, called by api.cpp
// after validation.  All shapes and pointers are already checked.
#pragma once

#include "common.h"

namespace lq {

int launch_nf4_quantize(const void* W, lq_dtype wdt, int64_t n, int32_t double_quant,
                        int32_t codebook, uint8_t* codes, uint8_t* q8, float* c2, float* absmax,
                        hipStream_t stream);
int launch_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* c2,
                          const float* absmax, int32_t double_quant, int32_t codebook, int64_t n,
                          void* out, lq_dtype odt, hipStream_t stream);
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
// Layers one grouped decode call may take (layers that read the same X).
constexpr int kDecodeMaxGroup = 8;

namespace dispatch {

size_t grad_partial_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
size_t multi_ws_bytes(int64_t T_tokens, int64_t r, int32_t n_adapters);

int bf16_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
             int64_t r, float s, void* Y, float* T_out, hipStream_t st);
// Chunked decode path (16 < M <= 96, as 16-row chunks in one launch of each
// of two kernels): T partial sums (kTParts x M x r floats, M padded to a
// multiple of 16) go to Tp; T_out (optional) receives T.
int decode_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T_out, float* Tp, hipStream_t st);
// Decode forward for M <= 16 in one launch (the reduction split over
// workgroups, T formed inside; no workspace: decode1_floats is 0).
size_t decode1_floats(int64_t M, int64_t N, int64_t K, int64_t r);
int decode_fwd1(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
                int64_t r, float s, void* Y, float* T_out, float* part, hipStream_t st);
// The one-launch decode over n <= kDecodeMaxGroup layers that read the same
// X (M <= 16): layer g has weight W[g] (all with the same K, kind, constant
// format and codebook), factors A[g], B[g], scale s[g] and output Y[g];
// T_out (or T_out[g]) may be NULL.  Arguments are checked by the caller.
int decode_fwd_group(const void* X, int64_t M, int32_t n, const lq_weight* W,
                     const void* const* A, const void* const* B, int64_t r, const float* s,
                     void* const* Y, float* const* T_out, hipStream_t st);
// Bound (in polls) of a workgroup's wait for data another workgroup publishes
// (the decode kernel's T words, the split-K partner's partial sums): polls > 0
// sets it, 0 restores the default, < 0 makes every such wait give up at once
// (wait_limit() is then -1).  Every wait that gives up is counted (a decode
// workgroup then forms T itself; a split-K workgroup leaves its partner's
// partial sums unread); take_*_giveups return the device's count since the
// last read and clear it.
constexpr int32_t kDefaultWaitPolls = 1 << 22;
void set_wait_limit(int32_t polls);
int32_t wait_limit();
int take_g256_giveups(uint64_t* n);
int take_decode_giveups(uint64_t* n);
// big_ws: workspace of the large-tile dX path (big_dx_ws_bytes), or NULL for
// the fused kernel
int bf16_bwd(const void* dY, const void* X, int64_t M, const lq_weight& W, const void* A,
             const void* B, int64_t r, float s, const float* T_saved, void* dX, float* dA,
             float* dB, int accumulate, void* ws, void* big_ws, hipStream_t st);
int bf16_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
            int64_t r, float s, void* dX, float* U_out, hipStream_t st);

// Skinny products T = X A^T and U = dY B (float32, M x r), each result times
// oscale (a single float32 product).  zero / nzero: int words cleared by the
// first workgroup as a side job (the split-K flags of the large-tile kernel
// that follows), or NULL / 0.
int t_only(const void* X, int64_t M, int64_t K, const void* A, int64_t r, float* T,
           hipStream_t st, int32_t* zero, int nzero, float oscale = 1.0f);
int u_only(const void* dY, int64_t M, int64_t N, const void* B, int64_t r, float* U,
           hipStream_t st, int32_t* zero, int nzero, float oscale = 1.0f);
// The 8-wave shrink kernel behind t_only / u_only (gt: G is B, K x r; needs
// r % 4 == 0), with the older one-pass kernel as the fallback.
// row_ad / mt (optional, multi-adapter T): column j of row m kept, times the
// adapter's scale, only inside the columns of adapter row_ad[m], else 0;
// every stored result is then multiplied by mt->oscale.
bool shrink_eligible(bool gt, int64_t r);
// One launch: the NF4 weight W dequantised to bf16 at wout, and the shrink of
// launch_shrink (same arguments), the flag words cleared as well.
int launch_prep(const lq_weight& W, void* wout, const void* Z, int64_t M, int64_t K, const void* G,
                bool gt, int64_t r, float* out, int32_t* zero, int nzero, hipStream_t st,
                const int32_t* row_ad = nullptr, const MultiTab* mt = nullptr);
int launch_shrink(const void* Z, int64_t M, int64_t K, const void* G, bool gt, int64_t r,
                  float* out, int32_t* zero, int nzero, hipStream_t st,
                  const int32_t* row_ad = nullptr, const MultiTab* mt = nullptr);

// Large-M path: the NF4 weight dequantised to a bf16 workspace copy, then the
// 256 x 256-tile product with the rank-r expand fused.  Eligible when the
// product's output width is a multiple of 256 and there are enough rows.
bool big_fwd_eligible(int64_t M, int64_t N, int64_t K);
// The large-tile product would use 256 x 256 tiles (enough of them to fill
// the chip): there it outruns the K-loop NF4 products even with the copy of
// W0 (a Llama-2-7B block at M = 8192, r = 64: 862 against 668 TFLOP/s), so
// an NF4 call given the copy's workspace takes it.
bool big_wide_tiles(int64_t M, int64_t NI);
bool big_dx_eligible(int64_t M, int64_t N, int64_t K);
size_t big_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
size_t big_dx_ws_bytes(int64_t M, int64_t N, int64_t K);
// Xa: the adapter branch's input when it differs from X (dropout), whose T is
// then scaled by inv_keep.
int big_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
            float s, void* Y, float* T_out, void* ws, hipStream_t st, const void* Xa = nullptr,
            float inv_keep = 1.0f);
// Large-M NF4 forward with no copy of W0, in one launch: the 128 x 256-tile
// product that dequantises the codes inside its K loop, forms T = X A^T in the
// same loop (stored to T_out, M x r float32, when not NULL) and adds the
// expand in its epilogue.  Eligible for an NF4 weight with N % 128 == 0,
// K % 256 == 0 and at least 192 tiles.
bool inloop_fwd_eligible(const lq_weight& W, int64_t M);
int inloop_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T_out, hipStream_t st);
// Large-M NF4 dX with no copy of W0, in one launch: the 128 x 256-tile product
// that dequantises the codes inside its K loop (read back transposed), forms
// U = dY B in the same loop (stored to U_out, M x r float32, when not NULL)
// and adds the expand (s U) A in its epilogue.  Eligible for an NF4 weight
// with K % 256 == 0, N % 128 == 0, r % 8 == 0 and at least 192 tiles.
bool inloop_dx_eligible(const lq_weight& W, int64_t M, int64_t r);
int inloop_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
              int64_t r, float s, void* dX, float* U_out, hipStream_t st);
// Multi-adapter forward at large T (same eligibility as the forward).
size_t big_multi_ws_bytes(int64_t T, int64_t N, int64_t K, int64_t rc);
int big_fwd_multi(const void* X, int64_t T, const lq_weight& W, const void* A_cat,
                  const void* B_cat, const MultiTab& mt, const int32_t* seg_off,
                  const int32_t* seg_ad, int32_t n_seg, void* Y, void* ws, hipStream_t st);
// row_ad[m] = adapter of the segment holding row m
int launch_rowmap(const int32_t* seg_off, const int32_t* seg_ad, int32_t n_seg, int64_t T,
                  int32_t* row_ad, hipStream_t st);
// dX for at most 64 rows with an NF4 weight (K % 128 == 0, N % 64 == 0,
// r <= 64): the weight streamed once by (128-column, 512-row) pieces, float32
// partial sums of dY Wd and of U = dY B per row range in ws
// (small_dx_ws_bytes, carved from the large-tile dX workspace), added in a
// second launch that also writes U (M x r float32, when U is not NULL).
bool small_dx_eligible(const lq_weight& W, int64_t M, int64_t r);
size_t small_dx_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
int small_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
             int64_t r, float s, float* U, void* dX, void* ws, hipStream_t st);
// Forward for 16 < M <= 64 rows with an NF4 weight (N % 128 == 0, K % 512
// == 0, r <= 64): the weight streamed once by (128-row, 512-column) pieces,
// float32 partial sums of X Wd^T and of T per column range in ws
// (small_fwd_ws_bytes), added in a second launch that applies the expand and
// writes T (M x r float32, when T_out is not NULL).
bool small_fwd_eligible(const lq_weight& W, int64_t M, int64_t r);
size_t small_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
int small_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
              int64_t r, float s, void* Y, float* T_out, void* ws, hipStream_t st);
// U (M x r float32) is written as well, times uscale: the expand needs it.
int big_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
           float s, void* dX, float* U, void* ws, hipStream_t st, float uscale = 1.0f);
int bf16_merge(const lq_weight& W, const void* A, const void* B, int64_t r, float s, void* Wout,
               hipStream_t st);
int bf16_fwd_multi(const void* X, int64_t T_tokens, const lq_weight& W, const void* A_cat,
                   const void* B_cat, const MultiTab& mt, const int32_t* seg_offsets,
                   const int32_t* seg_adapter, int32_t n_seg, void* Y, void* ws, hipStream_t st);

// AdamW step over a list of tensors (adamw.hip); launches in groups of
// kAdamTensors tensors.  Arguments already validated.
constexpr int kAdamTensors = 24;
struct AdamHyper {
  float lr, beta1, beta2, eps, weight_decay, grad_scale;
  int64_t step;
};
int adamw_step(const lq_adamw_tensor* ts, int32_t n_tensors, bool bf16_grad, const AdamHyper& h,
               hipStream_t st);

// LoRA-input dropout (dropout.hip): X_d = X * keep; T *= inv_keep and
// optionally Tm = bf16(s T) padded to rp columns; dX += s ((U A) * keep).
int launch_keep_apply(const void* X, const uint8_t* keep, int64_t M, int64_t K, void* Xd,
                      hipStream_t st);
int launch_t_finish(float* T, int64_t M, int64_t r, float inv_keep, float s, void* Tm, int rp,
                    hipStream_t st);
int launch_dx_fixup(void* dX, const float* U, const void* A, const uint8_t* keep, int64_t M,
                    int64_t K, int64_t r, float s, hipStream_t st);
// The fused forward with the adapter factor given: Y = X W0^T + Tm B^T, Tm the
// bf16 M x rp matrix s T (columns past r zero).
int bf16_fwd_given_t(const void* X, int64_t M, const lq_weight& W, const void* B, int64_t r,
                     const void* Tm, void* Y, hipStream_t st);
// Dropout backward (lora_grad.hip); Xd is M x K bf16 scratch.
int bf16_bwd_dropout(const void* dY, const void* X, const uint8_t* keep, float inv_keep,
                     int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
                     float s, const float* T_saved, void* dX, float* dA, float* dB,
                     int accumulate, void* Xd, void* ws, void* big_ws, hipStream_t st);

// One gradient-style reduction (lora_grad.hip): out[j][c] += s sum_m
// V[m][j] Z[m][c] over M rows (Z bf16 M x C, V float32 M x r); part holds
// grad_one_bytes(M, C, r) bytes of split partials.
size_t grad_one_bytes(int64_t M, int64_t C, int64_t r);
int grad_one(const void* Z, const float* V, int64_t M, int64_t C, int r, float s, float* out,
             float* part, hipStream_t st);

// DoRA (dora.hip).  Weight side: row norms c of W0 + s B A (W0 given as the
// bf16 matrix the products use) and g = m / c, with the pieces the backward
// reuses.  Gradient side: G' = dY * g, h, dm, kappa and the kappa terms.
struct DoraSide {
  float* w0sq;  // N
  float* P0;    // N x r, W0 A^T
  float* Gram;  // r x r, A A^T
  float* Gpart; // dora_gblocks(K) x r x r partials of A A^T
  float* c;     // N
  float* g;     // N
};
struct DoraGrad {
  uint16_t* Gp;  // M x N bf16
  float* hpart;  // tiles x N
  float* kappa;  // N
  float* KB;     // N x r
  float* Rpart;  // dora_rblocks(N) x r x r
  float* R;      // r x r
  float* part;   // grad_one partials
};
int dora_tiles(int64_t M);
int dora_rblocks(int64_t N);
int dora_gblocks(int64_t K);
int dora_weight_side(const void* Wd, int64_t N, int64_t K, const void* A, const void* B,
                     int64_t r, float s, const float* m, const DoraSide& d, hipStream_t st);
int dora_g_from_c(const float* m, const DoraSide& d, int64_t N, hipStream_t st);
int launch_col_scale(const void* Z, const float* g, int64_t M, int64_t N, void* Y,
                     hipStream_t st);
int dora_grad_side(const void* dY, const void* Z, const float* m, const void* B, int64_t M,
                   int64_t N, int64_t r, const DoraSide& d, const DoraGrad& q, float* dm,
                   int accumulate, hipStream_t st);
int dora_fix(const void* Wd, const void* A, const void* B, int64_t N, int64_t K, int64_t r,
             float s, const DoraSide& d, const DoraGrad& q, float* dA, float* dB, hipStream_t st);

}  // namespace dispatch
}  // namespace lq
