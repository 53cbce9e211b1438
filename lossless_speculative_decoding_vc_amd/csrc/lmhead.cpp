// Logits of hidden rows through a library GEMM (rocBLAS, bf16 in, fp32 out,
// fp32 accumulate).  The verify step's logits for every block row feed the
// greedy acceptance; the draft step's logits feed the drafter's argmax.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "../../include/vc.h"

namespace vc {

namespace {
std::mutex g_mu;
rocblas_handle g_handle = nullptr;
int g_device = -1;
}  // namespace

// Returns a rocBLAS status mapped to a HIP-style success flag; the caller
// reports errors through the C ABI.
int lm_head(int R, int Dm, int V, const void *h, const void *w, float *logits, hipStream_t s,
            const char **err) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { *err = "hipGetDevice failed"; return 1; }
  if (!g_handle || dev != g_device) {
    if (g_handle) rocblas_destroy_handle(g_handle);
    g_handle = nullptr;
    if (rocblas_create_handle(&g_handle) != rocblas_status_success) { *err = "rocblas_create_handle failed"; return 1; }
    g_device = dev;
  }
  if (rocblas_set_stream(g_handle, s) != rocblas_status_success) { *err = "rocblas_set_stream failed"; return 1; }
  const float alpha = 1.f, beta = 0.f;
  // Row-major logits[R][V] = h[R][Dm] W[Dm][V]  <=>  column-major
  // logits^T (V x R) = W^T (V x Dm) h^T (Dm x R) with no transposes.
  rocblas_status st = rocblas_gemm_ex(g_handle, rocblas_operation_none, rocblas_operation_none, V, R, Dm, &alpha,
                                      w, rocblas_datatype_bf16_r, V, h, rocblas_datatype_bf16_r, Dm, &beta, logits,
                                      rocblas_datatype_f32_r, V, logits, rocblas_datatype_f32_r, V,
                                      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) { *err = rocblas_status_to_string(st); return 1; }
  return 0;
}

}  // namespace vc
