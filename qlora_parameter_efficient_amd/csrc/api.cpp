// C ABI of liblq: argument validation, workspace carving and dispatch to the
// HIP kernels.  Nothing here computes; every step of the layer runs in the
// kernels of the .hip translation units.
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>

#include "common.h"
#include "dispatch.h"

namespace lq {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int hip_fail(hipError_t e, const char* where) {
  if (e == hipSuccess) return LQ_OK;
  set_error("%s: %s", where, hipGetErrorString(e));
  return LQ_ERR_HIP;
}

}  // namespace lq

using namespace lq;

#define REQUIRE(cond, code, ...)   \
  do {                             \
    if (!(cond)) {                 \
      set_error(__VA_ARGS__);      \
      return (code);               \
    }                              \
  } while (0)

namespace {

constexpr int64_t kMaxRank = 64;
constexpr int64_t kDecodeMaxM = 16;
// Forward rows that may run as 16-row decode chunks (one launch of each chunk
// kernel): each chunk streams W0 again, while the large-tile path's time
// barely grows with M at these sizes but leaves most compute units idle.
constexpr int64_t kDecodeChunkMaxM = 96;

// Where the chunks stop when the large-tile path is available (the LQ_OP_FWD
// workspace).  Measured, µs per graph-launched call at r = 16 (chunks / large
// tile): 4096 x 4096 NF4 M = 64 29.6 / 51.6, M = 96 42.1 / 51.6; 4096 x 4096
// bf16 M = 64 30.6 / 45.1, M = 96 43.4 / 45.4; 4096 x 11008 NF4 M = 96
// 107.4 / 116.7; 11008 x 4096 NF4 M = 32 41.9 / 58.7, M = 48 60.2 / 59.3,
// M = 64 73.4 / 59.6; 11008 x 4096 bf16 M = 17 47.4 / 46.0.  A wider output
// gives the large-tile path more tiles, while every chunk costs more.
int64_t chunk_max_m(int64_t N, bool nf4) {
  if (N <= 4096) return kDecodeChunkMaxM;
  return nf4 ? 32 : kDecodeMaxM;
}

int check_weight(const lq_weight* w, lq_dtype dt) {
  REQUIRE(w != nullptr, LQ_ERR_INVALID_ARG, "W0 descriptor is NULL");
  REQUIRE(w->N > 0 && w->K > 0, LQ_ERR_INVALID_ARG, "W0 has N=%lld K=%lld", (long long)w->N,
          (long long)w->K);
  REQUIRE(w->codebook == LQ_CB_NF4 || w->codebook == LQ_CB_NF4_SYMMETRIC, LQ_ERR_INVALID_ARG,
          "unknown W0 codebook %d", (int)w->codebook);
  REQUIRE(w->double_quant >= LQ_DQ_NONE && w->double_quant <= LQ_DQ_FP8, LQ_ERR_INVALID_ARG,
          "unknown W0 constant format %d", (int)w->double_quant);
  REQUIRE(w->dtype == dt, LQ_ERR_INVALID_ARG, "W0 dtype %d does not match call dtype %d",
          (int)w->dtype, (int)dt);
  if (w->kind == LQ_WEIGHT_DENSE) {
    REQUIRE(w->dense != nullptr, LQ_ERR_INVALID_ARG, "dense W0 pointer is NULL");
  } else if (w->kind == LQ_WEIGHT_NF4) {
    REQUIRE(w->codes != nullptr, LQ_ERR_INVALID_ARG, "NF4 codes pointer is NULL");
    if (w->double_quant) {
      REQUIRE(w->q8 && w->c2, LQ_ERR_INVALID_ARG, "NF4 double-quant constants are NULL");
    } else {
      REQUIRE(w->absmax != nullptr, LQ_ERR_INVALID_ARG, "NF4 absmax pointer is NULL");
    }
  } else {
    REQUIRE(false, LQ_ERR_INVALID_ARG, "unknown W0 kind %d", (int)w->kind);
  }
  return LQ_OK;
}

int check_bf16_shape(const lq_weight* w) {
  REQUIRE(w->K % 64 == 0, LQ_ERR_UNSUPPORTED, "bf16 path needs K %% 64 == 0 (K=%lld)",
          (long long)w->K);
  REQUIRE(w->N % 64 == 0, LQ_ERR_UNSUPPORTED, "bf16 path needs N %% 64 == 0 (N=%lld)",
          (long long)w->N);
  REQUIRE(w->K <= 65536 && w->N <= 65536, LQ_ERR_UNSUPPORTED,
          "bf16 path supports N, K <= 65536 (N=%lld K=%lld)", (long long)w->N, (long long)w->K);
  return LQ_OK;
}

// The bf16 kernels address activations with 32-bit byte offsets.
int check_bf16_rows(int64_t M, const lq_weight* w) {
  const int64_t lim = (int64_t)1 << 31;
  REQUIRE(M * w->K < lim && M * w->N < lim, LQ_ERR_UNSUPPORTED,
          "bf16 path needs M*K and M*N below 2^31 elements (M=%lld)", (long long)M);
  return LQ_OK;
}

size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  // U (M x r f32), T (M x r f32), dA / dB split partials
  return (size_t)(2 * M * r) * 4 + dispatch::grad_partial_bytes(M, N, K, r);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// The large-tile path of the bf16 forward / dX runs when the call's workspace
// holds its extra part (the bf16 weight copy and the split-K slots); with a
// smaller workspace the fused kernels run instead.
size_t fwd_big_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  return dispatch::big_fwd_eligible(M, N, K) ? dispatch::big_fwd_ws_bytes(M, N, K, r) : 0;
}

size_t bwd_big_bytes(int64_t M, int64_t N, int64_t K) {
  return dispatch::big_dx_eligible(M, N, K) ? dispatch::big_dx_ws_bytes(M, N, K) : 0;
}

size_t multi_big_bytes(int64_t T, int64_t N, int64_t K, int64_t rc) {
  return dispatch::big_fwd_eligible(T, N, K) ? dispatch::big_multi_ws_bytes(T, N, K, rc) : 0;
}

// Dropout workspaces: [X * keep, bf16 M x K][T, float32 M x r][the forward's
// large-tile part, or the fused path's bf16 M x rp Tm]; backward: [X * keep]
// [the backward's workspace][its large-tile part].
size_t drop_fwd_bytes(int64_t M, int64_t N, int64_t K, int64_t r, bool big) {
  const int64_t rp = r <= 32 ? 32 : 64;
  const size_t head = align256((size_t)(M * K) * 2) + align256((size_t)(M * r) * 4);
  return head + (big ? dispatch::big_fwd_ws_bytes(M, N, K, r) : (size_t)(M * rp) * 2);
}

size_t drop_bwd_bytes(int64_t M, int64_t N, int64_t K, int64_t r, bool big) {
  const size_t head = align256((size_t)(M * K) * 2) + align256(bwd_ws_bytes(M, N, K, r));
  return head + (big ? bwd_big_bytes(M, N, K) : 0);
}

bool drop_fwd_big(int64_t M, int64_t N, int64_t K) {
  return M > kDecodeMaxM && dispatch::big_fwd_eligible(M, N, K);
}

// Carves a caller workspace into 256-byte aligned pieces; with a null base it
// only measures (the size is then the final offset).
struct Bump {
  char* base;
  char* p;
  explicit Bump(void* b) : base((char*)b), p((char*)b) {}
  template <class T>
  T* take(size_t bytes) {
    T* r = (T*)p;
    p += align256(bytes);
    return r;
  }
  size_t used() const { return (size_t)(p - base); }
};

// DoRA weight side: [bf16 W0 (NF4 weights only)][w0sq][Gram partials][g] and,
// unless the caller's saved buffer holds them, [c][P0][Gram] (the saved
// buffer's layout: c[N], P0[N x r], Gram[r x r]).
void dora_side_take(Bump& b, bool nf4, int64_t N, int64_t K, int64_t r, const float* saved,
                    const void*& Wd, const void* dense, dispatch::DoraSide& d) {
  Wd = nf4 ? (const void*)b.take<uint16_t>((size_t)(N * K) * 2) : dense;
  d.w0sq = b.take<float>((size_t)N * 4);
  d.Gpart = b.take<float>((size_t)(dispatch::dora_gblocks(K) * r * r) * 4);
  d.g = b.take<float>((size_t)N * 4);
  float* sv = saved ? const_cast<float*>(saved)
                    : b.take<float>((size_t)(N + N * r + r * r) * 4);
  d.c = sv;
  d.P0 = sv + N;
  d.Gram = sv + N + N * r;
}

// Partial sums of T for the decode kernels: kTParts per row, 16-row chunks
// padded past 16 rows.
// Up to 16 rows: the one-launch decode kernel's partial sums and T; past 16
// rows: kTParts partial sums per row, 16-row chunks.
size_t decode_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M <= kDecodeMaxM) return dispatch::decode1_floats(M, N, K, r) * 4;
  const int64_t rows = (M + kDecodeMaxM - 1) / kDecodeMaxM * kDecodeMaxM;
  return (size_t)(kTParts * rows * r) * 4;
}

// The bf16 forward of up to kDecodeChunkMaxM rows by the decode kernels: one
// launch up to 16 rows, else one launch each of the two chunk kernels, 16-row
// chunks along the grid's second dimension.
int decode_chunks(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
                  int64_t r, float s, void* Y, float* T_out, float* Tp, hipStream_t st) {
  if (M <= kDecodeMaxM) return dispatch::decode_fwd1(X, M, W, A, B, r, s, Y, T_out, Tp, st);
  return dispatch::decode_fwd(X, M, W, A, B, r, s, Y, T_out, Tp, st);
}

size_t plain_fwd_bytes(int64_t M, int64_t N, int64_t K, int64_t r, bool big) {
  if (M <= kDecodeChunkMaxM) return decode_bytes(M, N, K, r);
  return big ? dispatch::big_fwd_ws_bytes(M, N, K, r) : 0;
}

bool dora_fwd_big(int64_t M, int64_t N, int64_t K) {
  return M > kDecodeChunkMaxM && dispatch::big_fwd_eligible(M, N, K);
}

size_t dora_fwd_bytes(int64_t M, int64_t N, int64_t K, int64_t r, bool nf4, bool big) {
  Bump b(nullptr);
  const void* Wd;
  dispatch::DoraSide d;
  dora_side_take(b, nf4, N, K, r, nullptr, Wd, nullptr, d);
  b.take<uint16_t>((size_t)(M * N) * 2);  // Z when the caller keeps none
  return b.used() + plain_fwd_bytes(M, N, K, r, big);
}

void dora_grad_take(Bump& b, int64_t M, int64_t N, int64_t K, int64_t r, dispatch::DoraGrad& q) {
  q.Gp = b.take<uint16_t>((size_t)(M * N) * 2);
  q.hpart = b.take<float>((size_t)(dispatch::dora_tiles(M) * N) * 4);
  q.kappa = b.take<float>((size_t)N * 4);
  q.KB = b.take<float>((size_t)(N * r) * 4);
  q.Rpart = b.take<float>((size_t)(dispatch::dora_rblocks(N) * r * r) * 4);
  q.R = b.take<float>((size_t)(r * r) * 4);
  q.part = b.take<float>(dispatch::grad_one_bytes(N, K, r));
}

size_t dora_bwd_bytes(int64_t M, int64_t N, int64_t K, int64_t r, bool nf4, bool big) {
  Bump b(nullptr);
  const void* Wd;
  dispatch::DoraSide d;
  dispatch::DoraGrad q;
  dora_side_take(b, nf4, N, K, r, nullptr, Wd, nullptr, d);
  dora_grad_take(b, M, N, K, r, q);
  b.take<char>(bwd_ws_bytes(M, N, K, r));
  return b.used() + (big ? bwd_big_bytes(M, N, K) : 0);
}

lq_weight dense_view(const lq_weight& W, const void* Wd) {
  lq_weight v{};
  v.kind = LQ_WEIGHT_DENSE;
  v.dtype = LQ_BF16;
  v.N = W.N;
  v.K = W.K;
  v.dense = Wd;
  return v;
}

// Column table of the multi-adapter forward from host rank offsets (n + 1
// entries, checked by the caller) and per-adapter scales.
MultiTab make_multi_tab(int32_t n, const int32_t* roff, const float* scales, int64_t N) {
  MultiTab t{};
  t.n_ad = n;
  t.rc = roff[n];
  for (int32_t a = 0; a <= n; ++a) t.roff[a] = roff[a];
  for (int32_t a = 0; a < n; ++a) {
    t.scale[a] = scales[a];
    for (int32_t c = roff[a]; c < roff[a + 1]; ++c) {
      t.col_base[c] = (int32_t)(N * roff[a] + (c - roff[a]));
      t.col_stride[c] = roff[a + 1] - roff[a];
    }
  }
  return t;
}

int multi_common(const void* X, int64_t T_tokens, const lq_weight* W0, const void* A_cat,
                 const void* B_cat, int32_t n_adapters, const int32_t* roff, const float* scales,
                 const int32_t* seg_offsets, const int32_t* seg_adapter, int32_t n_seg,
                 lq_dtype dt, void* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(dt == LQ_BF16, LQ_ERR_UNSUPPORTED, "multi-adapter forward supports bf16 only");
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  if ((rc = check_bf16_shape(W0))) return rc;
  REQUIRE(T_tokens >= 0 && n_seg >= 0, LQ_ERR_INVALID_ARG, "negative size");
  if ((rc = check_bf16_rows(T_tokens, W0))) return rc;
  if (T_tokens == 0) return LQ_OK;
  REQUIRE(n_seg >= 1, LQ_ERR_INVALID_ARG, "no segments for %lld tokens", (long long)T_tokens);
  REQUIRE(X && A_cat && B_cat && Y && seg_offsets && seg_adapter, LQ_ERR_INVALID_ARG,
          "a required pointer is NULL");
  const int64_t R = roff[n_adapters];
  const size_t need = dispatch::multi_ws_bytes(T_tokens, R, 1);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  const MultiTab mt = make_multi_tab(n_adapters, roff, scales, W0->N);
  const size_t big = multi_big_bytes(T_tokens, W0->N, W0->K, R);
  if (big && ws_bytes >= big)
    return dispatch::big_fwd_multi(X, T_tokens, *W0, A_cat, B_cat, mt, seg_offsets, seg_adapter,
                                   n_seg, Y, ws, stream);
  return dispatch::bf16_fwd_multi(X, T_tokens, *W0, A_cat, B_cat, mt, seg_offsets, seg_adapter,
                                  n_seg, Y, ws, stream);
}

}  // namespace

extern "C" {

const char* lq_last_error(void) { return g_err; }

int lq_debug_set_wait_limit(int32_t polls) {
  dispatch::set_wait_limit(polls);
  return LQ_OK;
}

int lq_debug_wait_giveups(int64_t* count) {
  REQUIRE(count != nullptr, LQ_ERR_INVALID_ARG, "count is NULL");
  int rc = hip_fail(hipDeviceSynchronize(), "hipDeviceSynchronize");
  uint64_t a = 0, b = 0;
  if (!rc) rc = dispatch::take_g256_giveups(&a);
  if (!rc) rc = dispatch::take_decode_giveups(&b);
  *count = rc ? 0 : (int64_t)(a + b);
  return rc;
}

int lq_nf4_codebook(int32_t codebook, float* out) {
  REQUIRE(out != nullptr, LQ_ERR_INVALID_ARG, "out is NULL");
  REQUIRE(codebook == LQ_CB_NF4 || codebook == LQ_CB_NF4_SYMMETRIC, LQ_ERR_INVALID_ARG,
          "unknown codebook %d", (int)codebook);
  std::memcpy(out, nf4_table(codebook).cb, sizeof(float) * 16);
  return LQ_OK;
}

int64_t lq_lora_num_params(int64_t N, int64_t K, int64_t r) { return r * (N + K); }

int lq_adamw_step(const lq_adamw_tensor* tensors, int32_t n_tensors, lq_dtype gdt, float lr,
                  float beta1, float beta2, float eps, float weight_decay, int64_t step,
                  float grad_scale, hipStream_t stream) {
  REQUIRE(n_tensors >= 0, LQ_ERR_INVALID_ARG, "n_tensors = %d", n_tensors);
  if (n_tensors == 0) return LQ_OK;
  REQUIRE(tensors != nullptr, LQ_ERR_INVALID_ARG, "tensor table is NULL");
  REQUIRE(gdt == LQ_F32 || gdt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad gradient dtype %d", (int)gdt);
  REQUIRE(step >= 1, LQ_ERR_INVALID_ARG, "step %lld (steps count from 1)", (long long)step);
  REQUIRE(std::isfinite(lr) && lr >= 0.0f, LQ_ERR_INVALID_ARG, "lr must be finite and >= 0");
  REQUIRE(std::isfinite(beta1) && beta1 >= 0.0f && beta1 < 1.0f, LQ_ERR_INVALID_ARG,
          "beta1 must be in [0, 1)");
  REQUIRE(std::isfinite(beta2) && beta2 >= 0.0f && beta2 < 1.0f, LQ_ERR_INVALID_ARG,
          "beta2 must be in [0, 1)");
  REQUIRE(std::isfinite(eps) && eps >= 0.0f, LQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
  REQUIRE(std::isfinite(weight_decay) && weight_decay >= 0.0f, LQ_ERR_INVALID_ARG,
          "weight_decay must be finite and >= 0");
  REQUIRE(std::isfinite(grad_scale), LQ_ERR_INVALID_ARG, "grad_scale must be finite");
  for (int32_t i = 0; i < n_tensors; ++i) {
    const lq_adamw_tensor& t = tensors[i];
    REQUIRE(t.n >= 0 && t.n <= ((int64_t)1 << 40), LQ_ERR_INVALID_ARG, "tensor %d: n = %lld", i,
            (long long)t.n);
    if (t.n == 0) continue;
    REQUIRE(t.master && t.m && t.v && t.grad, LQ_ERR_INVALID_ARG,
            "tensor %d: master, m, v and grad are required", i);
  }
  dispatch::AdamHyper h{lr, beta1, beta2, eps, weight_decay, grad_scale, step};
  return dispatch::adamw_step(tensors, n_tensors, gdt == LQ_BF16, h, stream);
}

int lq_check_segments(const int32_t* h_offsets, const int32_t* h_adapter, int32_t n_seg,
                      int64_t T_tokens, int32_t n_adapters) {
  REQUIRE(n_seg >= 0 && T_tokens >= 0 && n_adapters >= 1, LQ_ERR_INVALID_ARG,
          "bad segment counts");
  REQUIRE(h_offsets != nullptr, LQ_ERR_INVALID_ARG, "offsets NULL");
  REQUIRE(n_seg == 0 || h_adapter != nullptr, LQ_ERR_INVALID_ARG, "adapter ids NULL");
  REQUIRE(h_offsets[0] == 0, LQ_ERR_INVALID_ARG, "offsets[0] = %d, must be 0", h_offsets[0]);
  for (int32_t i = 0; i < n_seg; ++i) {
    REQUIRE(h_offsets[i + 1] >= h_offsets[i], LQ_ERR_INVALID_ARG,
            "offsets decrease at segment %d", i);
    REQUIRE(h_adapter[i] >= 0 && h_adapter[i] < n_adapters, LQ_ERR_INVALID_ARG,
            "segment %d adapter id %d out of range", i, h_adapter[i]);
  }
  REQUIRE(h_offsets[n_seg] == T_tokens, LQ_ERR_INVALID_ARG, "offsets end at %d, not %lld",
          h_offsets[n_seg], (long long)T_tokens);
  return LQ_OK;
}

size_t lq_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int64_t r,
                         int32_t n_adapters) {
  if (M < 0 || N < 0 || K < 0 || r < 0) return 0;
  switch (op) {
    case LQ_OP_FWD: {  // the decode path's partial sums of T, or float32 T
      // 17 to 64 rows of an NF4 weight in whole pieces: the weight-streaming
      // kernel's partial sums (the largest of the sizes those rows can use)
      const size_t sf = (M > kDecodeMaxM && M <= 64 && N % 128 == 0 && K % 512 == 0)
                            ? dispatch::small_fwd_ws_bytes(M, N, K, r)
                            : 0;
      // up to chunk_max_m rows (either format) never the large-tile path
      if (M <= kDecodeMaxM || M <= chunk_max_m(N, true)) {
        const size_t d = decode_bytes(M, N, K, r);
        return sf > d ? sf : d;
      }
      const size_t base = M <= kDecodeChunkMaxM ? decode_bytes(M, N, K, r) : (size_t)(M * r) * 4;
      const size_t big = fwd_big_bytes(M, N, K, r);
      const size_t mx = big > base ? big : base;
      return sf > mx ? sf : mx;
    }
    case LQ_OP_BWD: {
      const size_t big = bwd_big_bytes(M, N, K);
      return big ? align256(bwd_ws_bytes(M, N, K, r)) + big : bwd_ws_bytes(M, N, K, r);
    }
    case LQ_OP_FWD_MULTI: {
      const size_t base = dispatch::multi_ws_bytes(M, r, n_adapters);
      const size_t big = multi_big_bytes(M, N, K, r * (n_adapters > 0 ? n_adapters : 1));
      return big > base ? big : base;
    }
    case LQ_OP_FWD_DROPOUT:
      return drop_fwd_bytes(M, N, K, r, drop_fwd_big(M, N, K));
    case LQ_OP_FWD_DROPOUT_FUSED:
      return drop_fwd_bytes(M, N, K, r, false);
    case LQ_OP_BWD_DROPOUT:
      return drop_bwd_bytes(M, N, K, r, bwd_big_bytes(M, N, K) != 0);
    case LQ_OP_BWD_DROPOUT_FUSED:
      return drop_bwd_bytes(M, N, K, r, false);
    case LQ_OP_DORA_FWD:
      return dora_fwd_bytes(M, N, K, r, true, dora_fwd_big(M, N, K));
    case LQ_OP_DORA_FWD_FUSED:
      return dora_fwd_bytes(M, N, K, r, true, false);
    case LQ_OP_DORA_BWD:
      return dora_bwd_bytes(M, N, K, r, true, bwd_big_bytes(M, N, K) != 0);
    case LQ_OP_DORA_BWD_FUSED:
      return dora_bwd_bytes(M, N, K, r, true, false);
    case LQ_OP_FWD_FUSED:
      if (M <= kDecodeChunkMaxM) return decode_bytes(M, N, K, r);
      return (size_t)(M * r) * 4;
    case LQ_OP_BWD_FUSED:
      return bwd_ws_bytes(M, N, K, r);
    case LQ_OP_FWD_MULTI_FUSED:
      return dispatch::multi_ws_bytes(M, r, n_adapters);
    default:
      return 0;
  }
}

int lq_nf4_quantize(const void* W, lq_dtype wdt, int64_t n, int32_t double_quant,
                    int32_t codebook, uint8_t* codes, uint8_t* q8, float* c2, float* absmax,
                    hipStream_t stream) {
  REQUIRE(W != nullptr && codes != nullptr, LQ_ERR_INVALID_ARG, "W or codes is NULL");
  REQUIRE(n >= 1, LQ_ERR_INVALID_ARG, "n = %lld", (long long)n);
  REQUIRE(wdt == LQ_F32 || wdt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)wdt);
  REQUIRE(double_quant >= LQ_DQ_NONE && double_quant <= LQ_DQ_FP8, LQ_ERR_INVALID_ARG,
          "unknown constant format %d", (int)double_quant);
  REQUIRE(codebook == LQ_CB_NF4 || codebook == LQ_CB_NF4_SYMMETRIC, LQ_ERR_INVALID_ARG,
          "unknown codebook %d", (int)codebook);
  if (double_quant) {
    REQUIRE(q8 && c2, LQ_ERR_INVALID_ARG, "q8 or c2 is NULL");
  } else {
    REQUIRE(absmax != nullptr, LQ_ERR_INVALID_ARG, "absmax is NULL");
  }
  return launch_nf4_quantize(W, wdt, n, double_quant, codebook, codes, q8, c2, absmax, stream);
}

int lq_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* c2,
                      const float* absmax, int32_t double_quant, int32_t codebook, int64_t n,
                      void* out, lq_dtype odt, hipStream_t stream) {
  REQUIRE(codes != nullptr && out != nullptr, LQ_ERR_INVALID_ARG, "codes or out is NULL");
  REQUIRE(n >= 1, LQ_ERR_INVALID_ARG, "n = %lld", (long long)n);
  REQUIRE(odt == LQ_F32 || odt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)odt);
  REQUIRE(double_quant >= LQ_DQ_NONE && double_quant <= LQ_DQ_FP8, LQ_ERR_INVALID_ARG,
          "unknown constant format %d", (int)double_quant);
  REQUIRE(codebook == LQ_CB_NF4 || codebook == LQ_CB_NF4_SYMMETRIC, LQ_ERR_INVALID_ARG,
          "unknown codebook %d", (int)codebook);
  if (double_quant) {
    REQUIRE(q8 && c2, LQ_ERR_INVALID_ARG, "q8 or c2 is NULL");
  } else {
    REQUIRE(absmax != nullptr, LQ_ERR_INVALID_ARG, "absmax is NULL");
  }
  return launch_nf4_dequantize(codes, q8, c2, absmax, double_quant, codebook, n, out, odt,
                               stream);
}

int lq_lora_fwd(const void* X, int64_t M, const lq_weight* W0, const void* A, const void* B,
                int64_t r, float scale, lq_dtype dt, void* Y, float* T_out, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  if (dt == LQ_BF16 && (rc = check_bf16_shape(W0))) return rc;
  if (dt == LQ_BF16 && (rc = check_bf16_rows(M, W0))) return rc;
  if (M == 0) return LQ_OK;
  REQUIRE(X && A && B && Y, LQ_ERR_INVALID_ARG, "X, A, B or Y is NULL");
  if (dt == LQ_F32) {  // T crosses two kernels
    float* T = T_out;
    if (!T) {
      const size_t need = (size_t)(M * r) * 4;
      REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE,
              "workspace %zu bytes, need %zu", ws_bytes, need);
      T = (float*)ws;
    }
    return f32_lora_fwd((const float*)X, M, *W0, (const float*)A, (const float*)B, r, scale,
                        (float*)Y, T, stream);
  }
  // 17 to 64 rows of an NF4 weight, given the LQ_OP_FWD workspace: the
  // weight-streaming kernel (the weight read once, not once per 16 rows)
  if (M > kDecodeMaxM && dispatch::small_fwd_eligible(*W0, M, r) && ws &&
      ws_bytes >= dispatch::small_fwd_ws_bytes(M, W0->N, W0->K, r))
    return dispatch::small_fwd(X, M, *W0, A, B, r, scale, Y, T_out, ws, stream);
  const size_t big = fwd_big_bytes(M, W0->N, W0->K, r);
  const bool big_ok = big && ws && ws_bytes >= big;
  if (M <= kDecodeMaxM ||
      (M <= kDecodeChunkMaxM && (!big_ok || M <= chunk_max_m(W0->N, W0->kind == LQ_WEIGHT_NF4)))) {
    // partial sums of T cross two kernels, per 16-row chunk (none up to 16 rows)
    const size_t need = decode_bytes(M, W0->N, W0->K, r);
    REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), LQ_ERR_WORKSPACE,
            "workspace %zu bytes, need %zu", ws_bytes, need);
    return decode_chunks(X, M, *W0, A, B, r, scale, Y, T_out, (float*)ws, stream);
  }
  // an NF4 weight with enough 128 x 256 tiles: the product that dequantises
  // in its K loop and forms T in the same loop (no bf16 copy of W0, no
  // workspace) -- unless the copy's workspace was given and the large-tile
  // product would run 256 x 256 tiles, where it is the faster of the two
  if (dispatch::inloop_fwd_eligible(*W0, M) &&
      !(big_ok && dispatch::big_wide_tiles(M, W0->N)))
    return dispatch::inloop_fwd(X, M, *W0, A, B, r, scale, Y, T_out, stream);
  if (big_ok) return dispatch::big_fwd(X, M, *W0, A, B, r, scale, Y, T_out, ws, stream);
  return dispatch::bf16_fwd(X, M, *W0, A, B, r, scale, Y, T_out, stream);
}

int lq_lora_fwd_decode_layers(const void* X, int64_t M, int32_t n_layers, const lq_weight* W,
                              const void* const* A, const void* const* B, int64_t r,
                              const float* s, void* const* Y, float* const* T_out,
                              hipStream_t stream) {
  static_assert(LQ_DECODE_MAX_LAYERS == kDecodeMaxGroup, "layer limit");
  REQUIRE(n_layers >= 1 && n_layers <= LQ_DECODE_MAX_LAYERS, LQ_ERR_INVALID_ARG,
          "n_layers = %d outside [1, %d]", (int)n_layers, LQ_DECODE_MAX_LAYERS);
  REQUIRE(W && A && B && s && Y, LQ_ERR_INVALID_ARG, "W, A, B, s or Y array is NULL");
  REQUIRE(M >= 0 && M <= kDecodeMaxM, LQ_ERR_UNSUPPORTED, "M = %lld outside [0, %lld]",
          (long long)M, (long long)kDecodeMaxM);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  for (int g = 0; g < n_layers; ++g) {
    int rc = check_weight(&W[g], LQ_BF16);
    if (rc) return rc;
    if ((rc = check_bf16_shape(&W[g]))) return rc;
    if ((rc = check_bf16_rows(M, &W[g]))) return rc;
    REQUIRE(W[g].K == W[0].K, LQ_ERR_INVALID_ARG, "layer %d has K=%lld, layer 0 K=%lld", g,
            (long long)W[g].K, (long long)W[0].K);
    REQUIRE(W[g].kind == W[0].kind && (W[g].kind == LQ_WEIGHT_DENSE ||
                                       (W[g].double_quant == W[0].double_quant &&
                                        W[g].codebook == W[0].codebook)),
            LQ_ERR_INVALID_ARG, "layer %d's weight format differs from layer 0's", g);
    REQUIRE(M == 0 || (A[g] && B[g] && Y[g]), LQ_ERR_INVALID_ARG,
            "A, B or Y of layer %d is NULL", g);
  }
  if (M == 0) return LQ_OK;
  REQUIRE(X != nullptr, LQ_ERR_INVALID_ARG, "X is NULL");
  return dispatch::decode_fwd_group(X, M, n_layers, W, A, B, r, s, Y, T_out, stream);
}

int lq_lora_bwd(const void* dY, const void* X, int64_t M, const lq_weight* W0, const void* A,
                const void* B, int64_t r, float scale, lq_dtype dt, const float* T_saved,
                void* dX, float* dA, float* dB, int32_t accumulate, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  REQUIRE(A && B, LQ_ERR_INVALID_ARG, "A or B is NULL");
  REQUIRE((dA == nullptr) == (dB == nullptr), LQ_ERR_INVALID_ARG,
          "dA and dB must both be given or both be NULL");
  REQUIRE(dA || dX, LQ_ERR_INVALID_ARG, "nothing to compute: dX, dA and dB are NULL");
  REQUIRE(M == 0 || (dY && (X || !dA)), LQ_ERR_INVALID_ARG, "dY or X is NULL");
  if (dt == LQ_BF16 && (rc = check_bf16_shape(W0))) return rc;
  if (dt == LQ_BF16 && (rc = check_bf16_rows(M, W0))) return rc;
  const int64_t N = W0->N, K = W0->K;
  const size_t need = bwd_ws_bytes(M, N, K, r);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  if (dt == LQ_F32)
    return f32_lora_bwd((const float*)dY, (const float*)X, M, *W0, (const float*)A,
                        (const float*)B, r, scale, T_saved, (float*)dX, dA, dB, accumulate,
                        (float*)ws, stream);
  const size_t big = dX ? bwd_big_bytes(M, N, K) : 0;
  void* big_ws = nullptr;
  if (big && ws_bytes >= align256(need) + big) big_ws = (char*)ws + align256(need);
  return dispatch::bf16_bwd(dY, X, M, *W0, A, B, r, scale, T_saved, dX, dA, dB, accumulate, ws,
                            big_ws, stream);
}

int lq_lora_fwd_dropout(const void* X, int64_t M, const lq_weight* W0, const void* A,
                        const void* B, int64_t r, float scale, const uint8_t* keep, float p,
                        lq_dtype dt, void* Y, float* T_out, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  REQUIRE(dt == LQ_BF16, LQ_ERR_UNSUPPORTED, "dropout is implemented for bf16 only");
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  REQUIRE(std::isfinite(p) && p >= 0.0f && p < 1.0f, LQ_ERR_INVALID_ARG,
          "dropout probability must be in [0, 1)");
  if ((rc = check_bf16_shape(W0)) || (rc = check_bf16_rows(M, W0))) return rc;
  if (M == 0) return LQ_OK;
  REQUIRE(X && A && B && Y && keep, LQ_ERR_INVALID_ARG, "X, A, B, Y or keep is NULL");
  const int64_t N = W0->N, K = W0->K;
  const size_t need = drop_fwd_bytes(M, N, K, r, false);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  const bool big = drop_fwd_big(M, N, K) && ws_bytes >= drop_fwd_bytes(M, N, K, r, true);
  char* w = (char*)ws;
  void* Xd = w;
  w += align256((size_t)(M * K) * 2);
  float* T = T_out ? T_out : (float*)w;
  w += align256((size_t)(M * r) * 4);
  const float inv_keep = (float)(1.0 / (1.0 - (double)p));
  if ((rc = dispatch::launch_keep_apply(X, keep, M, K, Xd, stream))) return rc;
  if (big)
    return dispatch::big_fwd(X, M, *W0, A, B, r, scale, Y, T, w, stream, Xd, inv_keep);
  if ((rc = dispatch::t_only(Xd, M, K, A, r, T, stream, nullptr, 0))) return rc;
  const int rp = r <= 32 ? 32 : 64;
  if ((rc = dispatch::launch_t_finish(T, M, r, inv_keep, scale, w, rp, stream))) return rc;
  return dispatch::bf16_fwd_given_t(X, M, *W0, B, r, w, Y, stream);
}

int lq_lora_bwd_dropout(const void* dY, const void* X, int64_t M, const lq_weight* W0,
                        const void* A, const void* B, int64_t r, float scale,
                        const uint8_t* keep, float p, lq_dtype dt, const float* T_saved,
                        void* dX, float* dA, float* dB, int32_t accumulate, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  REQUIRE(dt == LQ_BF16, LQ_ERR_UNSUPPORTED, "dropout is implemented for bf16 only");
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  REQUIRE(std::isfinite(p) && p >= 0.0f && p < 1.0f, LQ_ERR_INVALID_ARG,
          "dropout probability must be in [0, 1)");
  REQUIRE(A && B, LQ_ERR_INVALID_ARG, "A or B is NULL");
  REQUIRE((dA == nullptr) == (dB == nullptr), LQ_ERR_INVALID_ARG,
          "dA and dB must both be given or both be NULL");
  REQUIRE(dA || dX, LQ_ERR_INVALID_ARG, "nothing to compute: dX, dA and dB are NULL");
  REQUIRE(M == 0 || (dY && keep && (X || !dA)), LQ_ERR_INVALID_ARG, "dY, keep or X is NULL");
  if ((rc = check_bf16_shape(W0)) || (rc = check_bf16_rows(M, W0))) return rc;
  const int64_t N = W0->N, K = W0->K;
  const size_t need = drop_bwd_bytes(M, N, K, r, false);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  char* w = (char*)ws;
  void* Xd = w;
  w += align256((size_t)(M * K) * 2);
  void* big_ws = nullptr;
  if (dX && bwd_big_bytes(M, N, K) && ws_bytes >= drop_bwd_bytes(M, N, K, r, true))
    big_ws = w + align256(bwd_ws_bytes(M, N, K, r));
  const float inv_keep = (float)(1.0 / (1.0 - (double)p));
  return dispatch::bf16_bwd_dropout(dY, X, keep, inv_keep, M, *W0, A, B, r, scale, T_saved, dX,
                                    dA, dB, accumulate, Xd, w, big_ws, stream);
}

int64_t lq_dora_saved_floats(int64_t N, int64_t r) { return N + N * r + r * r; }

int lq_dora_fwd(const void* X, int64_t M, const lq_weight* W0, const void* A, const void* B,
                int64_t r, float scale, const float* magnitude, lq_dtype dt, void* Y,
                void* Z_out, float* T_out, float* saved_out, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  REQUIRE(dt == LQ_BF16, LQ_ERR_UNSUPPORTED, "DoRA is implemented for bf16 only");
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  if ((rc = check_bf16_shape(W0)) || (rc = check_bf16_rows(M, W0))) return rc;
  if (M == 0) return LQ_OK;
  REQUIRE(X && A && B && Y && magnitude, LQ_ERR_INVALID_ARG, "X, A, B, Y or magnitude is NULL");
  const int64_t N = W0->N, K = W0->K;
  const bool nf4 = W0->kind == LQ_WEIGHT_NF4;
  const size_t need = dora_fwd_bytes(M, N, K, r, nf4, false);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  const bool big = dora_fwd_big(M, N, K) && ws_bytes >= dora_fwd_bytes(M, N, K, r, nf4, true);
  Bump b(ws);
  const void* Wd;
  dispatch::DoraSide d;
  dora_side_take(b, nf4, N, K, r, saved_out, Wd, W0->dense, d);
  void* Z = Z_out ? Z_out : (void*)b.take<uint16_t>((size_t)(M * N) * 2);
  void* rest = b.p;
  if (nf4 && (rc = launch_nf4_dequantize(W0->codes, W0->q8, W0->c2, W0->absmax,
                                         W0->double_quant, W0->codebook, N * K, (void*)Wd,
                                         LQ_BF16, stream)))
    return rc;
  if ((rc = dispatch::dora_weight_side(Wd, N, K, A, B, r, scale, magnitude, d, stream))) return rc;
  const lq_weight Wv = dense_view(*W0, Wd);
  if (M <= kDecodeChunkMaxM)
    rc = decode_chunks(X, M, Wv, A, B, r, scale, Z, T_out, (float*)rest, stream);
  else if (big)
    rc = dispatch::big_fwd(X, M, Wv, A, B, r, scale, Z, T_out, rest, stream);
  else
    rc = dispatch::bf16_fwd(X, M, Wv, A, B, r, scale, Z, T_out, stream);
  if (rc) return rc;
  return dispatch::launch_col_scale(Z, d.g, M, N, Y, stream);
}

int lq_dora_bwd(const void* dY, const void* X, int64_t M, const lq_weight* W0, const void* A,
                const void* B, int64_t r, float scale, const float* magnitude, lq_dtype dt,
                const void* Z_saved, const float* T_saved, const float* saved, void* dX,
                float* dA, float* dB, float* dmag, int32_t accumulate, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  REQUIRE(dt == LQ_BF16, LQ_ERR_UNSUPPORTED, "DoRA is implemented for bf16 only");
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(M >= 0, LQ_ERR_INVALID_ARG, "M = %lld", (long long)M);
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  REQUIRE(A && B && magnitude && dA && dB && dmag, LQ_ERR_INVALID_ARG,
          "A, B, magnitude, dA, dB and dmag are required");
  REQUIRE(M == 0 || (dY && X && Z_saved), LQ_ERR_INVALID_ARG, "dY, X or Z_saved is NULL");
  if ((rc = check_bf16_shape(W0)) || (rc = check_bf16_rows(M, W0))) return rc;
  const int64_t N = W0->N, K = W0->K;
  if (M == 0) {
    if (accumulate) return LQ_OK;
    if ((rc = launch_zero_f32(dA, r * K, stream)) || (rc = launch_zero_f32(dB, N * r, stream)))
      return rc;
    return launch_zero_f32(dmag, N, stream);
  }
  const bool nf4 = W0->kind == LQ_WEIGHT_NF4;
  const size_t need = dora_bwd_bytes(M, N, K, r, nf4, false);
  REQUIRE(ws != nullptr && ws_bytes >= need, LQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu",
          ws_bytes, need);
  const bool big = dX && bwd_big_bytes(M, N, K) &&
                   ws_bytes >= dora_bwd_bytes(M, N, K, r, nf4, true);
  Bump b(ws);
  const void* Wd;
  dispatch::DoraSide d;
  dispatch::DoraGrad q;
  dora_side_take(b, nf4, N, K, r, saved, Wd, W0->dense, d);
  dora_grad_take(b, M, N, K, r, q);
  void* bws = b.take<char>(bwd_ws_bytes(M, N, K, r));
  void* big_ws = big ? (void*)b.p : nullptr;
  if (nf4 && (rc = launch_nf4_dequantize(W0->codes, W0->q8, W0->c2, W0->absmax,
                                         W0->double_quant, W0->codebook, N * K, (void*)Wd,
                                         LQ_BF16, stream)))
    return rc;
  rc = saved ? dispatch::dora_g_from_c(magnitude, d, N, stream)
             : dispatch::dora_weight_side(Wd, N, K, A, B, r, scale, magnitude, d, stream);
  if (rc) return rc;
  if ((rc = dispatch::dora_grad_side(dY, Z_saved, magnitude, B, M, N, r, d, q, dmag, accumulate,
                                     stream)))
    return rc;
  const lq_weight Wv = dense_view(*W0, Wd);
  if ((rc = dispatch::bf16_bwd(q.Gp, X, M, Wv, A, B, r, scale, T_saved, dX, dA, dB, accumulate,
                               bws, big_ws, stream)))
    return rc;
  return dispatch::dora_fix(Wd, A, B, N, K, r, scale, d, q, dA, dB, stream);
}

int lq_lora_merge(const lq_weight* W0, const void* A, const void* B, int64_t r, float scale,
                  lq_dtype dt, void* W_out, hipStream_t stream) {
  REQUIRE(dt == LQ_F32 || dt == LQ_BF16, LQ_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
  int rc = check_weight(W0, dt);
  if (rc) return rc;
  REQUIRE(r >= 1 && r <= kMaxRank, LQ_ERR_UNSUPPORTED, "rank %lld outside [1, %lld]",
          (long long)r, (long long)kMaxRank);
  REQUIRE(A && B && W_out, LQ_ERR_INVALID_ARG, "A, B or W_out is NULL");
  if (dt == LQ_F32)
    return f32_lora_merge(*W0, (const float*)A, (const float*)B, r, scale, (float*)W_out, stream);
  if ((rc = check_bf16_shape(W0))) return rc;
  return dispatch::bf16_merge(*W0, A, B, r, scale, W_out, stream);
}

int lq_lora_fwd_multi(const void* X, int64_t T_tokens, const lq_weight* W0, const void* A_stack,
                      const void* B_stack, int32_t n_adapters, int64_t r, float scale,
                      const int32_t* seg_offsets, const int32_t* seg_adapter, int32_t n_seg,
                      lq_dtype dt, void* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(n_adapters >= 1, LQ_ERR_INVALID_ARG, "n_adapters = %d", n_adapters);
  REQUIRE(r >= 1 && r * n_adapters <= kMaxRank, LQ_ERR_UNSUPPORTED,
          "r * n_adapters = %lld exceeds %lld", (long long)(r * n_adapters), (long long)kMaxRank);
  int32_t roff[kMaxRankCols + 1];
  float scales[kMaxRankCols];
  for (int32_t a = 0; a <= n_adapters; ++a) roff[a] = (int32_t)(a * r);
  for (int32_t a = 0; a < n_adapters; ++a) scales[a] = scale;
  return multi_common(X, T_tokens, W0, A_stack, B_stack, n_adapters, roff, scales, seg_offsets,
                      seg_adapter, n_seg, dt, Y, ws, ws_bytes, stream);
}

int lq_lora_fwd_multi_ranks(const void* X, int64_t T_tokens, const lq_weight* W0,
                            const void* A_cat, const void* B_cat, int32_t n_adapters,
                            const int32_t* rank_offsets, const float* scales,
                            const int32_t* seg_offsets, const int32_t* seg_adapter,
                            int32_t n_seg, lq_dtype dt, void* Y, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  REQUIRE(n_adapters >= 1 && n_adapters <= kMaxRankCols, LQ_ERR_INVALID_ARG, "n_adapters = %d",
          n_adapters);
  REQUIRE(rank_offsets && scales, LQ_ERR_INVALID_ARG, "rank_offsets or scales is NULL");
  REQUIRE(rank_offsets[0] == 0, LQ_ERR_INVALID_ARG, "rank_offsets[0] = %d, must be 0",
          rank_offsets[0]);
  for (int32_t a = 0; a < n_adapters; ++a)
    REQUIRE(rank_offsets[a + 1] > rank_offsets[a], LQ_ERR_INVALID_ARG,
            "adapter %d has rank %d (ranks must be >= 1)", a,
            rank_offsets[a + 1] - rank_offsets[a]);
  REQUIRE(rank_offsets[n_adapters] <= kMaxRank, LQ_ERR_UNSUPPORTED,
          "total rank %d exceeds %lld", rank_offsets[n_adapters], (long long)kMaxRank);
  return multi_common(X, T_tokens, W0, A_cat, B_cat, n_adapters, rank_offsets, scales,
                      seg_offsets, seg_adapter, n_seg, dt, Y, ws, ws_bytes, stream);
}

}  // extern "C"
