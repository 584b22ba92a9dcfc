// Checks of pick lists and key-major lists (CSR), shared by the device
// kernels of the debug index check and its host-side form.
//
// The attention kernels gather key and value rows through the pick lists, and
// the backward pass gathers query rows through the CSR ("Trainable Log-linear
// Sparse Attention for Efficient Diffusion Transformers", explainer "Step 3"
// and "Step 4"; the abstract: the operator is driven by sparse indices alone),
// so a value out of range is an out-of-bounds read.  These functions read only
// inside the row, key segment or parent row they are given.
#pragma once
#include <stdint.h>

#include "llsa.h"

namespace llsa {

// One pick row of a level with n tokens: k values, each in [0, n), strictly
// ascending, and (parent != nullptr) each a child of one of the kp parent
// picks, i.e. value / B is among them.
__host__ __device__ inline uint32_t check_pick_row(const int32_t *row, int k, int n,
                                                   const int32_t *parent, int kp, int B) {
    uint32_t f = 0;
    int prev = -1;
    for (int j = 0; j < k; ++j) {
        const int c = row[j];
        if (c < 0 || c >= n) {
            f |= LLSA_IDX_RANGE;
            continue;
        }
        if (c <= prev) f |= LLSA_IDX_ORDER;
        prev = c;
        if (parent != nullptr) {
            bool child = false;
            for (int m = 0; m < kp; ++m) child = child || parent[m] == c / B;
            if (!child) f |= LLSA_IDX_PARENT;
        }
    }
    return f;
}

// Key c of the CSR of one n x n pick matrix with k picks per row (n * k
// picks): ptr[0] = 0, ptr[n] = n * k, ptr[c] <= ptr[c+1]; the rows of key c's
// segment lie in [0, n), strictly ascend, and each of them picked c in idx
// (its row of k values).  With every pick row valid, all keys passing these
// checks make the CSR exactly the transpose of idx: n * k distinct (row, key)
// pairs, each one of the n * k pairs of idx.
__host__ __device__ inline uint32_t check_csr_key(const int32_t *ptr, const int32_t *col,
                                                  const int32_t *idx, int n, int k, int c) {
    const int total = n * k;
    uint32_t f = 0;
    const int a = ptr[c], e = ptr[c + 1];
    if (c == 0 && a != 0) f |= LLSA_IDX_CSR_PTR;
    if (c == n - 1 && e != total) f |= LLSA_IDX_CSR_PTR;
    if (a < 0 || e < a || e > total) return f | LLSA_IDX_CSR_PTR;
    int prev = -1;
    for (int x = a; x < e; ++x) {
        const int r = col[x];
        if (r < 0 || r >= n) {
            f |= LLSA_IDX_CSR_COL;
            continue;
        }
        if (r <= prev) f |= LLSA_IDX_CSR_COL;
        prev = r;
        bool hit = false;
        for (int j = 0; j < k; ++j) hit = hit || idx[(int64_t)r * k + j] == c;
        if (!hit) f |= LLSA_IDX_CSR_COL;
    }
    return f;
}

}  // namespace llsa
