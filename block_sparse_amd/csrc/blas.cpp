// The plain GEMMs around the attention (q/k/v and output projections of the
// Llama-3 attention block) run in rocBLAS: bf16 operands, fp32 accumulation,
// bf16 result, with the residual add folded in as beta * C.  A star_context
// owns the rocBLAS handle and a fixed device workspace handed to it, so the
// library keeps no global state and a GEMM call never allocates.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <cstdint>
#include <new>

#include "../../include/star_attn.h"
#include "internal.h"

struct star_context {
  rocblas_handle blas;
  void* workspace;
};

namespace {

bool matrix_ok(const star_tensor* t) {
  return t != nullptr && t->data != nullptr && t->dtype == STAR_BF16 && t->B == 1 && t->H == 1 &&
         t->S >= 0 && t->D >= 1 && t->sS >= t->D &&
         (reinterpret_cast<uintptr_t>(t->data) & 15u) == 0 && (t->sS * 2) % 16 == 0;
}

}  // namespace

extern "C" {

int star_context_create(star_context** ctx) {
  if (ctx == nullptr) return STAR_ERR_NULL;
  *ctx = nullptr;
  star_context* c = new (std::nothrow) star_context{nullptr, nullptr};
  if (c == nullptr) return STAR_ERR_UNSUPPORTED;
  if (rocblas_create_handle(&c->blas) != rocblas_status_success) {
    delete c;
    return STAR_ERR_BLAS;
  }
  // a user-owned workspace: rocBLAS uses it and allocates nothing itself
  if (hipMalloc(&c->workspace, STAR_BLAS_WORKSPACE_BYTES) != hipSuccess) {
    c->workspace = nullptr;
    rocblas_destroy_handle(c->blas);
    delete c;
    return STAR_ERR_HIP;
  }
  if (rocblas_set_workspace(c->blas, c->workspace, STAR_BLAS_WORKSPACE_BYTES) !=
      rocblas_status_success) {
    rocblas_destroy_handle(c->blas);
    (void)hipFree(c->workspace);
    delete c;
    return STAR_ERR_BLAS;
  }
  *ctx = c;
  return STAR_OK;
}

int star_context_destroy(star_context* ctx) {
  if (ctx == nullptr) return STAR_OK;
  const rocblas_status s = rocblas_destroy_handle(ctx->blas);
  const hipError_t e = ctx->workspace != nullptr ? hipFree(ctx->workspace) : hipSuccess;
  delete ctx;
  if (s != rocblas_status_success) return STAR_ERR_BLAS;
  return e == hipSuccess ? STAR_OK : STAR_ERR_HIP;
}

int star_linear(star_context* ctx, const star_tensor* x, const star_tensor* w,
                const star_tensor* residual, const star_tensor* y, void* stream) {
  if (ctx == nullptr || x == nullptr || w == nullptr || y == nullptr) return STAR_ERR_NULL;
  if (x->data == nullptr || w->data == nullptr || y->data == nullptr) return STAR_ERR_NULL;
  if (x->dtype != STAR_BF16 || w->dtype != STAR_BF16 || y->dtype != STAR_BF16) return STAR_ERR_DTYPE;
  if (residual != nullptr && (residual->data == nullptr)) return STAR_ERR_NULL;
  if (residual != nullptr && residual->dtype != STAR_BF16) return STAR_ERR_DTYPE;
  if (!matrix_ok(x) || !matrix_ok(w) || !matrix_ok(y) ||
      (residual != nullptr && !matrix_ok(residual)))
    return STAR_ERR_SHAPE;
  const int64_t M = x->S, K = x->D, N = w->S;
  if (w->D != K || y->S != M || y->D != N) return STAR_ERR_SHAPE;
  if (residual != nullptr && (residual->S != M || residual->D != N)) return STAR_ERR_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || x->sS > INT32_MAX ||
      w->sS > INT32_MAX || y->sS > INT32_MAX || (residual && residual->sS > INT32_MAX))
    return STAR_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return STAR_OK;
  if (rocblas_set_stream(ctx->blas, (hipStream_t)stream) != rocblas_status_success)
    return STAR_ERR_BLAS;
  // row-major y[M, N] = x[M, K] w[N, K]^T (+ r): in rocBLAS's column-major
  // terms y^T (N x M) = op(w) x^T with op = transpose of w's (K x N) view
  const float alpha = 1.f, beta = residual != nullptr ? 1.f : 0.f;
  const void* c = residual != nullptr ? residual->data : y->data;
  const int64_t ldc = residual != nullptr ? residual->sS : y->sS;
  const rocblas_status s = rocblas_gemm_ex(
      ctx->blas, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)N,
      (rocblas_int)M, (rocblas_int)K, &alpha, w->data, rocblas_datatype_bf16_r,
      (rocblas_int)w->sS, x->data, rocblas_datatype_bf16_r, (rocblas_int)x->sS, &beta, c,
      rocblas_datatype_bf16_r, (rocblas_int)ldc, y->data, rocblas_datatype_bf16_r,
      (rocblas_int)y->sS, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return s == rocblas_status_success ? STAR_OK : STAR_ERR_BLAS;
}

}  // extern "C"
