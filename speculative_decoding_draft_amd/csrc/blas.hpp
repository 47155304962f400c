// Plain GEMMs of the library on rocBLAS (internal to libdspark_attn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include "dspark_attn.h"

namespace dspark {

// The rocBLAS handle of the calling thread on the current device, created
// on first use with atomics disabled (the same call gives the same bits) and
// kept for the life of the process; bound to `s` on return.
rocblas_status blas_handle(hipStream_t s, rocblas_handle* h);

// rocBLAS works in the caller's memory (the MLA block's and the loss head's
// workspaces set DSPARK_BLAS_WORKSPACE_BYTES aside).  The handle keeps the
// pointer after the call returns; only the library uses the handle, and
// every call sets its own area before its first GEMM.  (Handing the handle
// back to rocBLAS's own memory after each call would let rocBLAS allocate
// and free device memory between calls.)
rocblas_status blas_use_workspace(rocblas_handle h, void* p, size_t n);

// The GEMMs of one call, in order: the i-th takes table->gemm[i] when its
// shape matches (tune = false), or times every solution rocBLAS offers for
// its shape (and rocBLAS's default) on the handle's stream -- synchronising
// it -- writes the fastest to table->gemm[i] and runs it (tune = true).
struct GemmPick {
    dspark_gemm_choices* table;    // nullptr: rocBLAS's own choice everywhere
    bool tune;
    int next;
};

// Row-major D[M][N] = A[M][K] B[N][K]^T + beta C[M][N] with fp32
// accumulation.  A and B have type in_t, C and D type out_t (bf16 or fp32);
// leading dimensions in elements.  C = nullptr: D itself (read only when
// beta != 0).  pick: nullptr (rocBLAS's choice) or the call's GemmPick.  The
// tuning trials rewrite D, so a tuned call with beta != 0 and C = nullptr (D
// accumulated in place) leaves D accumulated many times: the caller
// recomputes it.  Otherwise C must not alias D.
rocblas_status gemm_nt(rocblas_handle h, rocblas_datatype in_t, rocblas_datatype out_t, int M,
                       int N, int K, const void* A, int lda, const void* B, int ldb, float beta,
                       const void* C, int ldc, void* D, int ldd, GemmPick* pick);

}  // namespace dspark
