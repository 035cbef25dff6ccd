// Plain GEMMs through rocBLAS (the projection layer and the first layer of the
// compression MLP phi): one handle per device, row-major views.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "nsa_kernels.hpp"

namespace nsa {

namespace {

// One rocBLAS handle per device, created on first use with that device
// current; the mutex serialises setting the stream and enqueuing a GEMM.
std::mutex g_mu;
rocblas_handle g_handle[64];

rocblas_datatype rt(BlasType t) { return t == kBlasBF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r; }

}  // namespace

int blas_gemm(hipStream_t s, bool ta, bool tb, int M, int N, int K, const void* A, BlasType at, int lda,
              const void* B, BlasType bt, int ldb, float beta, void* C, BlasType ct, int ldc) {
  if (M == 0 || N == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 2;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_handle[dev] && rocblas_create_handle(&g_handle[dev]) != rocblas_status_success) {
    g_handle[dev] = nullptr;
    return 2;
  }
  rocblas_handle h = g_handle[dev];
  if (rocblas_set_stream(h, s) != rocblas_status_success) return 1;
  // rocBLAS is column-major, where a row-major matrix reads as its transpose:
  // C^T = op(B)^T op(A)^T, with the operands swapped
  const float alpha = 1.f;
  const rocblas_status st =
      rocblas_gemm_ex(h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                      ta ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &alpha, B, rt(bt), ldb, A,
                      rt(at), lda, &beta, C, rt(ct), ldc, C, rt(ct), ldc, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? 0 : 1;
}

}  // namespace nsa
