// Debug index check on the device: every pick row of the given levels and
// every key of the given CSR levels is checked (index_check.hpp) and the
// flags of what failed are OR-ed into one status word.  Reads stay inside the
// lists' own buffers whatever their values, so corrupt lists can be checked
// before any kernel gathers through them.
#include "common.hpp"
#include "index_check.hpp"
#include "internal.hpp"

namespace llsa {

__global__ __launch_bounds__(64) void status_clear_kernel(uint32_t *__restrict__ status) {
    if (threadIdx.x == 0) status[0] = 0u;
}

// one thread per row of one level (all batch * heads matrices)
__global__ __launch_bounds__(256) void check_rows_kernel(const int32_t *__restrict__ idx,
                                                        const int32_t *__restrict__ parent, int n,
                                                        int k, int kp, int B, int64_t rows,
                                                        uint32_t *__restrict__ status) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    const int64_t b = r / n, i = r % n;
    const int32_t *par = parent != nullptr ? parent + (b * (n / B) + i / B) * kp : nullptr;
    const uint32_t f = check_pick_row(idx + r * k, k, n, par, kp, B);
    if (f != 0u) atomicOr(status, f);
}

// one thread per key of one CSR level (all batch * heads matrices)
__global__ __launch_bounds__(256) void check_csr_kernel(const int32_t *__restrict__ ptr,
                                                       const int32_t *__restrict__ col,
                                                       const int32_t *__restrict__ idx, int n,
                                                       int k, int64_t keys,
                                                       uint32_t *__restrict__ status) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= keys) return;
    const int64_t b = x / n;
    const int c = (int)(x % n);
    const uint32_t f = check_csr_key(ptr + b * (n + 1), col + b * (int64_t)n * k,
                                     idx + b * (int64_t)n * k, n, k, c);
    if (f != 0u) atomicOr(status, f);
}

hipError_t launch_status_clear(uint32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, s, status);
    return hipGetLastError();
}

hipError_t launch_check_indices(const Geometry &g, const int32_t *idx, const int32_t *csr_ptr,
                                const int32_t *csr_col, uint32_t *status, hipStream_t s) {
    for (int l = 1; l <= g.L; ++l) {
        const int64_t rows = (int64_t)g.bh * g.n[l];
        const int32_t *parent = l < g.L ? idx + g.idx_off[l + 1] : nullptr;
        const int kp = l < g.L ? g.kl[l + 1] : 0;
        hipLaunchKernelGGL(check_rows_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                           idx + g.idx_off[l], parent, g.n[l], g.kl[l], kp, g.B, rows, status);
    }
    if (csr_ptr != nullptr && csr_col != nullptr) {
        for (int l = 1; l <= g.Le + 1; ++l) {
            const int64_t keys = (int64_t)g.bh * g.n[l];
            hipLaunchKernelGGL(check_csr_kernel, dim3((unsigned)((keys + 255) / 256)), dim3(256), 0,
                               s, csr_ptr + g.ptr_off[l], csr_col + g.col_off[l], idx + g.idx_off[l],
                               g.n[l], g.kl[l], keys, status);
        }
    }
    return hipGetLastError();
}

uint32_t check_indices_host(const Geometry &g, const int32_t *idx, const int32_t *csr_ptr,
                            const int32_t *csr_col) {
    uint32_t f = 0;
    for (int l = 1; l <= g.L; ++l) {
        const int n = g.n[l], k = g.kl[l];
        const int kp = l < g.L ? g.kl[l + 1] : 0;
        for (int64_t r = 0; r < (int64_t)g.bh * n; ++r) {
            const int64_t b = r / n, i = r % n;
            const int32_t *par =
                l < g.L ? idx + g.idx_off[l + 1] + (b * (n / g.B) + i / g.B) * kp : nullptr;
            f |= check_pick_row(idx + g.idx_off[l] + r * k, k, n, par, kp, g.B);
        }
    }
    if (csr_ptr != nullptr && csr_col != nullptr) {
        for (int l = 1; l <= g.Le + 1; ++l) {
            const int n = g.n[l], k = g.kl[l];
            for (int b = 0; b < g.bh; ++b)
                for (int c = 0; c < n; ++c)
                    f |= check_csr_key(csr_ptr + g.ptr_off[l] + (int64_t)b * (n + 1),
                                       csr_col + g.col_off[l] + (int64_t)b * n * k,
                                       idx + g.idx_off[l] + (int64_t)b * n * k, n, k, c);
        }
    }
    return f;
}

}  // namespace llsa
