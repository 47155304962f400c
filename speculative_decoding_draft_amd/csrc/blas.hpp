// Plain GEMMs of the library on rocBLAS (internal to libdspark_attn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

namespace dspark {

// The rocBLAS handle of the calling thread on the current device, created
// on first use with atomics disabled (the same call gives the same bits) and
// kept for the life of the process; bound to `s` on return.
rocblas_status blas_handle(hipStream_t s, rocblas_handle* h);

// Row-major D[M][N] = A[M][K] B[N][K]^T + beta C[M][N] with fp32
// accumulation.  A and B have type in_t, C and D type out_t (bf16 or fp32);
// leading dimensions in elements.  C = nullptr: D itself (read only when
// beta != 0).  tune: time every solution rocBLAS offers for this shape (and
// its default) on the handle's stream -- synchronising it -- record the
// fastest for (device, shape, types), then run it; later calls with the same
// key use the recorded choice.  The trials rewrite D, so a tuned call with
// beta != 0 and C = nullptr (D accumulated in place) leaves D accumulated
// many times: the caller recomputes it.  Otherwise C must not alias D.
rocblas_status gemm_nt(rocblas_handle h, rocblas_datatype in_t, rocblas_datatype out_t, int M,
                       int N, int K, const void* A, int lda, const void* B, int ldb, float beta,
                       const void* C, int ldc, void* D, int ldd, bool tune);

}  // namespace dspark
