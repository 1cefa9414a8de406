// Kernel launch helper shared by the device sources of libqgemv.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/qgemv.h"

namespace qg {

// The HIP error of the calling thread's last failed launch (returned by qg_last_hip_error).
extern thread_local hipError_t g_last_hip_error;

// hipLaunchKernel returns the launch status itself, so a stale error left in the runtime's
// last-error slot by an unrelated earlier call cannot be mistaken for a failed launch.
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args) {
  void *ptrs[] = {static_cast<void *>(&args)...};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shm, s);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return QG_ERR_LAUNCH;
  }
  return QG_OK;
}

// Dequant GEMM for larger m through LDS-staged fp16 tiles and MFMA (prefill.hip). Arguments
// are validated by the caller.
int launch_prefill(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
                   int64_t m, int64_t n, int64_t k, hipStream_t s);

// Tile shape the prefill GEMM takes for m x n (BM x BN; prefill.hip).
void prefill_tile(int64_t m, int64_t n, int *bm, int *bn);

// Dequant GEMM for up to 32 activation rows through fp16 MFMA (skinny.hip; qg_gemm sends it
// 5 <= m <= 16, and more rows in launches of up to 32 when skinny_us says so). Arguments are
// validated by the caller.
int launch_skinny(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
                  int64_t m, int64_t n, int64_t k, hipStream_t s);

// Estimated duration in microseconds of one launch_skinny of m <= 32 rows (a huge value for
// shapes it does not take).
double skinny_us(int fmt, int64_t m, int64_t n, int64_t k);

}  // namespace qg
