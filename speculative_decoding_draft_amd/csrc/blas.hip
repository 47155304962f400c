// rocBLAS handles, the caller's workspace for them, and the kernel choice of
// the library's GEMMs.
#define ROCBLAS_BETA_FEATURES_API   // rocblas_gemm_ex_get_solutions (kernel choice)
#pragma clang diagnostic ignored "-Wdeprecated-declarations"   // that beta call is marked so
#include "blas.hpp"

#include <vector>

namespace dspark {

namespace {

// one handle per (thread, device)
thread_local rocblas_handle t_handles[64] = {};

}  // namespace

rocblas_status blas_handle(hipStream_t s, rocblas_handle* h) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return rocblas_status_invalid_handle;
    if (!t_handles[dev]) {
        const rocblas_status st = rocblas_create_handle(&t_handles[dev]);
        if (st != rocblas_status_success) return st;
        rocblas_set_atomics_mode(t_handles[dev], rocblas_atomics_not_allowed);
    }
    *h = t_handles[dev];
    return rocblas_set_stream(*h, s);
}

rocblas_status blas_use_workspace(rocblas_handle h, void* p, size_t n) {
    return rocblas_set_workspace(h, p, n);
}

// In rocBLAS's column-major terms the row-major product is
// D^T = op_T(B^T) A^T, so B goes first.
rocblas_status gemm_nt(rocblas_handle h, rocblas_datatype in_t, rocblas_datatype out_t, int M,
                       int N, int K, const void* A, int lda, const void* B, int ldb, float beta,
                       const void* C, int ldc, void* D, int ldd, GemmPick* pick) {
    const float alpha = 1.f;
    const void* Cp = C ? C : D;
    const int ldcp = C ? ldc : ldd;
    auto run = [&](int sol) {
        return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, M, K,
                               &alpha, B, in_t, ldb, A, in_t, lda, &beta, Cp, out_t, ldcp, D,
                               out_t, ldd, rocblas_datatype_f32_r,
                               sol > 0 ? rocblas_gemm_algo_solution_index
                                       : rocblas_gemm_algo_standard,
                               sol > 0 ? sol : 0, 0);
    };
    if (!pick) return run(0);
    const int idx = pick->next++;
    dspark_gemm_choice* slot = (pick->table && idx < DSPARK_MAX_GEMMS) ? &pick->table->gemm[idx]
                                                                      : nullptr;
    if (!pick->tune) {
        const bool same = slot && idx < pick->table->n_gemms && slot->m == M && slot->n == N &&
                          slot->k == K;
        return run(same ? slot->solution : 0);
    }
    rocblas_int n = 0;
    rocblas_status st = rocblas_gemm_ex_get_solutions(
        h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &alpha, B, in_t, ldb, A,
        in_t, lda, &beta, Cp, out_t, ldcp, D, out_t, ldd, rocblas_datatype_f32_r,
        rocblas_gemm_algo_solution_index, 0, nullptr, &n);
    std::vector<rocblas_int> sols(n > 0 ? n : 0);
    if (st == rocblas_status_success && n > 0)
        st = rocblas_gemm_ex_get_solutions(
            h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &alpha, B, in_t, ldb,
            A, in_t, lda, &beta, Cp, out_t, ldcp, D, out_t, ldd, rocblas_datatype_f32_r,
            rocblas_gemm_algo_solution_index, 0, sols.data(), &n);
    sols.insert(sols.begin(), 0);              // rocBLAS's default
    hipStream_t s = nullptr;
    rocblas_get_stream(h, &s);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
        return rocblas_status_internal_error;
    int best = 0;
    float best_ms = 1e30f;
    for (int sol : sols) {
        if (run(sol) != rocblas_status_success) continue;      // warm-up; skips invalid ones
        (void)hipEventRecord(e0, s);
        bool ok = true;
        for (int i = 0; i < 3 && ok; ++i) ok = run(sol) == rocblas_status_success;
        (void)hipEventRecord(e1, s);
        (void)hipEventSynchronize(e1);
        float ms = 0.f;
        if (ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms < best_ms) {
            best_ms = ms;
            best = sol;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (slot) {
        *slot = dspark_gemm_choice{M, N, K, best};
        pick->table->n_gemms = idx + 1;
    }
    return run(best);
}

}  // namespace dspark
