/*
 * llsa.h -- C ABI of the MI355X (gfx950) Log-linear Sparse Attention library.
 *
 * The operator is the one described in "Trainable Log-linear Sparse Attention
 * for Efficient Diffusion Transformers" (howistudyai.com explainer): input
 * Q, K, V go through hierarchical compression, hierarchical Top-K selection
 * and sparse attention with hierarchical KV enrichment and reweighting to the
 * output O; a sparse index transpose drives the backward pass (explainer,
 * paragraph "At a high level", and "Step 1" .. "Step 4").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller, contiguous and
 *    row-major, at least 16-byte aligned.  The library never allocates or
 *    frees device memory and, outside the debug index check (see
 *    llsa_problem.index_status), never synchronises: each call enqueues its
 *    kernels on `stream` (a hipStream_t passed as void*, NULL = default
 *    stream) and returns.  It keeps no global state (except the static scratch
 *    of llsa_attn_bwd_noalloc) and is thread-safe.
 *  - Q, K, V, O, dO are [batch, heads, seq_len, head_dim] in `dtype`.
 *  - Level l = 1..L has n_l = seq_len / block^l tokens; level 0 is the input.
 *    Pyramids are float32, levels stored in order, each starting on a
 *    64-byte boundary:
 *        level l at float offset sizes.pyramid_offset[l], shape [batch*heads, n_l, d].
 *  - Index lists are int32, levels stored in order, each starting on a
 *    64-byte boundary:
 *        level l at offset sizes.index_offset[l], shape [batch*heads, n_l, K_l],
 *    with K_L = min(K, n_L) and K_l = min(K, B*K_{l+1}) for l < L; every row
 *    holds distinct indices in ascending order.
 *  - All shape, pointer and alignment checks run on the host before any HIP
 *    call; on an error status nothing is launched and no output is touched.
 *    Launch failures are reported as LLSA_ERR_HIP.
 *  - Index lists and CSR are trusted: outside the debug index check
 *    (llsa_problem.index_status) their values are not checked, and values
 *    other than the library's own make the kernels read out of bounds.  With
 *    the check on, a call that reads lists checks them on the device first and
 *    returns LLSA_ERR_INDEX, with nothing else launched, when they are
 *    invalid.
 *  - Supported set: head_dim = 64, block = 16 or 64, 1 <= levels <= 6,
 *    1 <= topk <= 32, seq_len < 2^25, batch * heads * seq_len < 2^31, dtype
 *    LLSA_F32 or LLSA_BF16, non-causal.  Other values give
 *    LLSA_ERR_UNSUPPORTED.
 */
#ifndef LLSA_H
#define LLSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLSA_MAX_LEVELS 6

enum llsa_status {
    LLSA_OK = 0,
    LLSA_ERR_INVALID = 1,      /* bad shape, null or misaligned pointer, inconsistent sizes */
    LLSA_ERR_UNSUPPORTED = 2,  /* valid but outside the supported set above               */
    LLSA_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than required          */
    LLSA_ERR_HIP = 4,          /* a kernel launch failed                                   */
    LLSA_ERR_INDEX = 5,        /* debug index check only: an index list or CSR is invalid   */
    LLSA_ERR_SCRATCH = 6       /* llsa_attn_bwd_noalloc: the problem needs more workspace
                                  than LLSA_NOALLOC_SCRATCH_BYTES                          */
};

/* Flags of the debug index check's status word (OR-ed). */
enum llsa_index_flag {
    LLSA_IDX_RANGE = 1,    /* a pick outside [0, n_l)                                      */
    LLSA_IDX_ORDER = 2,    /* a pick row not strictly ascending                            */
    LLSA_IDX_PARENT = 4,   /* a pick at level l < L that is no child of its parent's picks */
    LLSA_IDX_CSR_PTR = 8,  /* ptr[0] != 0, ptr[n_l] != n_l * K_l, or ptr decreasing        */
    LLSA_IDX_CSR_COL = 16  /* a CSR row outside [0, n_l), not ascending in its key's
                              segment, or not having picked that key                       */
};

enum llsa_dtype { LLSA_F32 = 0, LLSA_BF16 = 1 };

typedef struct llsa_problem {
    int32_t batch, heads, seq_len, head_dim;
    int32_t block;        /* B: tokens pooled into one token of the next level            */
    int32_t levels;       /* L: pooling steps; seq_len % block^levels == 0                */
    int32_t topk;         /* K: picks per query and level                                  */
    int32_t enrich;       /* Le: coarse levels 2..Le+1 enrich attention; -1 means L-1      */
    int32_t dtype;        /* llsa_dtype of Q, K, V, O, dO                                  */
    int32_t grad_dtype;   /* llsa_dtype of dQ, dK, dV                                      */
    float scale;          /* softmax scale; 0 means 1/sqrt(head_dim)                       */
    int32_t drop_covered; /* 1: leave out a coarse pick whose level-1 children are all
                             fine picks of the query block (then K = all blocks is exactly
                             dense attention); 0: keep every coarse pick                  */
    int32_t token_order;  /* 0: the sequence as stored.  1: seq_len = S*S pixels of an
                             image stored in raster order (S a power of two); the method
                             runs on the nested 2^i x 2^i patch sequence (Z order), so a
                             level-l token pools a 4^l x 4^l patch.  Q, K, V, O, dO, dQ,
                             dK, dV and lse stay in raster order; pyramids, index lists
                             and CSR are in patch-sequence order                          */
    int32_t *index_status; /* debug index check; NULL (the default) turns it off.  Else a
                             DEVICE pointer to one int32 status word.  llsa_attn_fwd,
                             llsa_index_transpose_levels and llsa_attn_bwd then check the
                             lists they read (as llsa_check_indices), wait for the check on
                             their stream and return LLSA_ERR_INDEX, launching nothing
                             else, when it fails; llsa_select and llsa_select_transpose
                             check the lists they wrote (after writing them) and also
                             report a parent pick outside its level, which the selection
                             otherwise reads as key 0.  The word is cleared by each such
                             call and holds the LLSA_IDX_* flags of what failed.  These
                             calls synchronise their stream, so the check is for debugging */
} llsa_problem;

typedef struct llsa_sizes {
    int32_t levels;                              /* L                                   */
    int32_t enrich;                              /* resolved Le                         */
    int32_t level_tokens[LLSA_MAX_LEVELS + 1];   /* [0] = seq_len, [l] = n_l            */
    int32_t level_k[LLSA_MAX_LEVELS + 1];        /* [l] = K_l, [0] unused               */
    int64_t pyramid_elems;                       /* floats in ONE pyramid (q, k or v)   */
    int64_t pyramid_offset[LLSA_MAX_LEVELS + 2]; /* float offset of level l             */
    int64_t index_elems;                         /* int32s in the index buffer          */
    int64_t index_offset[LLSA_MAX_LEVELS + 2];   /* int32 offset of level l             */
    int64_t csr_ptr_elems;                       /* int32s of all CSR ptr arrays        */
    int64_t csr_ptr_offset[LLSA_MAX_LEVELS + 2]; /* level l: [batch*heads, n_l + 1]     */
                                                 /* (CSR levels also 64-byte aligned)   */
    int64_t csr_col_elems;                       /* int32s of all CSR col arrays        */
    int64_t csr_col_offset[LLSA_MAX_LEVELS + 2]; /* level l: [batch*heads, n_l * K_l]   */
    int64_t lse_elems;                           /* floats of lse: batch*heads*seq_len  */
    size_t transpose_workspace_bytes;            /* per llsa_index_transpose call, max  */
    size_t bwd_workspace_bytes;                  /* llsa_attn_bwd                       */
} llsa_sizes;

/* Host only: derived sizes and layout offsets for problem `p`.  The CSR
 * arrays cover levels 1..Le+1 (the levels the backward pass reads). */
int llsa_sizes_query(const llsa_problem *p, llsa_sizes *out);

/*
 * Hierarchical compression (explainer "Step 1: Hierarchical Compression"):
 * level l token j is the mean of level l-1 tokens jB .. jB+B-1, for
 * l = 1..L, computed for Q, K and V in float32.
 * In : q, k, v [batch, heads, seq_len, head_dim] (dtype).
 * Out: pyr_q, pyr_k, pyr_v, each sizes.pyramid_elems floats (layout above).
 */
int llsa_pool(const llsa_problem *p, const void *q, const void *k, const void *v,
              float *pyr_q, float *pyr_k, float *pyr_v, void *stream);

/*
 * Hierarchical Top-K selection (explainer "Step 2: Hierarchical Top-K
 * Selection"): at level L every query scores all n_L keys; at level l < L
 * query i scores only the B children of each pick of its parent i/B at level
 * l+1.  A score is the float32 dot product of pooled query and pooled key;
 * the K_l highest scores are kept, ties going to the lower index; each row is
 * stored in ascending index order.
 * In : pyr_q, pyr_k from llsa_pool.
 * Out: idx, sizes.index_elems int32 (layout above).
 */
int llsa_select(const llsa_problem *p, const float *pyr_q, const float *pyr_k,
                int32_t *idx, void *stream);

/*
 * Sparse attention with hierarchical KV enrichment and reweighting (explainer
 * "Step 3: Hierarchical KV Enrichment + KV Reweighting"): query block i
 * (tokens iB .. iB+B-1) attends to every token of its K_1 fine picks
 * I^(1)[i] (weight 1) and, for l = 2..Le+1, to the pooled tokens K^(l)[c],
 * V^(l)[c] of the picks c of its level-l ancestor i / B^(l-1) (weight B^l,
 * i.e. logit + ln B^l; see drop_covered).  Logits are scale * q.k.  The
 * kernels read only the index lists, never a dense mask.
 * In : q, k, v (dtype), pyr_k, pyr_v (float32), idx.
 *      idx must be as llsa_select writes it: every row of level l holds K_l
 *      distinct values in [0, n_l), ascending.  The values are checked only
 *      in the debug index check (llsa_problem.index_status); otherwise others
 *      make the kernels read out of bounds.
 * Out: o [batch, heads, seq_len, head_dim] (dtype), lse [batch*heads*seq_len]
 *      float32 natural-log normaliser of every query row.
 */
int llsa_attn_fwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                  const float *pyr_k, const float *pyr_v, const int32_t *idx,
                  void *o, float *lse, void *stream);

/*
 * Sparse index transpose (explainer "Step 4: Efficient Sparse Index
 * Transpose"): query-major picks become key-major lists by counting the picks
 * of every key, an exclusive prefix sum of the counts, and a fill.
 * In : idx [n_batch, n_rows, k] int32, every value in [0, n_cols), rows of
 *      distinct values.
 * Out: csr_ptr [n_batch, n_cols + 1]: ptr[c] = number of picks of keys < c,
 *      so ptr[n_cols] = n_rows * k; csr_col [n_batch, n_rows * k]: the rows
 *      that picked key c, ascending, at csr_col[ptr[c] .. ptr[c+1]).
 * workspace: at least llsa_index_transpose_workspace(...) bytes of device
 *      memory.  Zero (workspace may be NULL) for matrices of at most 131072
 *      picks and 4096 keys, which one launch transposes; otherwise per-range
 *      histograms and totals of up to 4096 buckets, and above 4096 keys also
 *      a staging list of (key, row) pairs and sorted keys, 12 bytes per pick.
 * Limits: n_cols <= 2^24 and n_batch <= 65535 (LLSA_ERR_UNSUPPORTED).
 * An index outside [0, n_cols) is skipped: it is not listed, and ptr[n_cols]
 * then counts only the listed picks.  The output is deterministic.
 */
size_t llsa_index_transpose_workspace(int32_t n_batch, int32_t n_rows, int32_t k,
                                      int32_t n_cols);
int llsa_index_transpose(int32_t n_batch, int32_t n_rows, int32_t k, int32_t n_cols,
                         const int32_t *idx, int32_t *csr_ptr, int32_t *csr_col,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The index transposes the backward pass reads, for one problem: the CSR of
 * I^(l) for l = 1..Le+1, exactly as llsa_index_transpose(batch * heads, n_l,
 * K_l, n_l, idx + sizes.index_offset[l], ...) would write them at
 * sizes.csr_ptr_offset[l] / sizes.csr_col_offset[l].  The levels that fit the
 * one-launch transpose (at most 131072 picks and 4096 keys) share a single
 * launch; larger ones run in turn.
 * In : idx, every level as llsa_select writes it.
 * workspace: at least llsa_index_transpose_levels_workspace(p) bytes of
 *      device memory (16-byte aligned; zero bytes, NULL allowed, when every
 *      level fits the one-launch transpose).
 * Errors as llsa_select; LLSA_ERR_UNSUPPORTED also when batch * heads >
 * 65535.
 */
size_t llsa_index_transpose_levels_workspace(const llsa_problem *p);
int llsa_index_transpose_levels(const llsa_problem *p, const int32_t *idx, int32_t *csr_ptr,
                                int32_t *csr_col, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Selection and the index transposes the backward pass reads, fused
 * (explainer "Step 2" and "Step 4"): the same idx as llsa_select and the
 * same csr_ptr / csr_col for levels 1..Le+1 as llsa_index_transpose(batch *
 * heads, n_l, K_l, n_l, ...) at sizes.csr_*_offset[l].  When level 1 has at
 * most 4096 tokens (and its rows come eight 16-row groups to a workgroup), its
 * selection kernel also counts its picks per key, the first step of the
 * transpose, so the picks are not read back for it.
 * workspace: at least llsa_select_transpose_workspace(p) bytes of device
 *      memory (16-byte aligned), shared by the level transposes in turn.
 * Errors as llsa_select; LLSA_ERR_UNSUPPORTED also when batch * heads >
 * 65535.
 */
size_t llsa_select_transpose_workspace(const llsa_problem *p);
int llsa_select_transpose(const llsa_problem *p, const float *pyr_q, const float *pyr_k,
                          int32_t *idx, int32_t *csr_ptr, int32_t *csr_col, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Baseline for comparison with llsa_index_transpose: the same output built
 * from a dense bit mask of n_rows x n_cols per matrix (set every pick's bit,
 * then read every key's column): the mask-based route of explainer "Step 4",
 * whose time and memory grow with n_rows * n_cols, the square of the
 * sequence length.  Same arguments and output; rows ascend within a key.
 * workspace: at least llsa_index_transpose_mask_workspace(n_batch, n_rows,
 *      n_cols) bytes (the mask and per-key counts).
 */
size_t llsa_index_transpose_mask_workspace(int32_t n_batch, int32_t n_rows, int32_t n_cols);
int llsa_index_transpose_mask(int32_t n_batch, int32_t n_rows, int32_t k, int32_t n_cols,
                              const int32_t *idx, int32_t *csr_ptr, int32_t *csr_col,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward pass of llsa_attn_fwd for the loss <O, dO> with the picks held
 * fixed (Top-K has no gradient; pooled Q only feeds the picks), driven by the
 * key-major lists (explainer "Step 4"; "Sparse Index Transpose" building
 * block): dQ is computed query-major, dK and dV key-major from the CSR of
 * I^(1), pooled-token gradients of levels 2..Le+1 from the CSR of I^(l) and
 * then spread back to the B^l tokens under each pooled token (mean adjoint).
 * In : everything llsa_attn_fwd read, its outputs o and lse, dout (dtype),
 *      csr_ptr / csr_col for levels 1..Le+1 at sizes.csr_*_offset[l], each
 *      produced by llsa_index_transpose(batch*heads, n_l, K_l, n_l, ...) (or
 *      llsa_index_transpose_levels) from that same idx; like idx, the lists
 *      are checked only in the debug index check.
 * Out: dq, dk, dv [batch, heads, seq_len, head_dim] in grad_dtype.
 * workspace: at least sizes.bwd_workspace_bytes of device memory.
 */
int llsa_attn_bwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                  const float *pyr_k, const float *pyr_v, const int32_t *idx,
                  const int32_t *csr_ptr, const int32_t *csr_col,
                  const void *o, const float *lse, const void *dout,
                  void *dq, void *dk, void *dv,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * llsa_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and kernels without the workspace.  Its
 * workspace is a static device array of LLSA_NOALLOC_SCRATCH_BYTES bytes that
 * every GPU the library runs on holds until the process ends (its address is
 * looked up on the first call with that device current; the stream must
 * belong to the current device).  No allocation and no allocating library
 * routine is called.  Problems whose sizes.bwd_workspace_bytes exceed the
 * scratch are rejected on the host with LLSA_ERR_SCRATCH (nothing launched);
 * the 65536-token, 16-head, K = 8 problem needs 22 MiB.  Every call on one
 * GPU shares that GPU's scratch and leaves its contents behind (each call
 * writes every byte it reads, so nothing needs clearing): calls that overlap
 * on one GPU, on different streams or threads, race and must not be issued.
 */
#define LLSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int llsa_attn_bwd_noalloc(const llsa_problem *p, const void *q, const void *k, const void *v,
                          const float *pyr_k, const float *pyr_v, const int32_t *idx,
                          const int32_t *csr_ptr, const int32_t *csr_col,
                          const void *o, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, void *stream);

/*
 * Dense (full, non-causal) softmax attention in the same kernel style, the
 * comparator of the explainer's "Scoreboard" speed-up (full attention).
 * In : q, k, v [batch, heads, seq_len, head_dim] (dtype; only LLSA_BF16),
 *      scale as in llsa_problem (other fields ignored except batch, heads,
 *      seq_len, head_dim, dtype).
 * Out: o (dtype), lse float32 [batch*heads*seq_len].
 */
int llsa_dense_attn_fwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                        void *o, float *lse, void *stream);

/*
 * Dense backward comparator of llsa_dense_attn_fwd for the loss <O, dO>: a
 * query-major pass computes D = rowsum(dO * O) and dQ, a key-major pass dK
 * and dV, over all keys (no sparsity).  Same supported set as the forward.
 * In : q, k, v, o, dout [batch, heads, seq_len, 64] bf16; lse from
 *      llsa_dense_attn_fwd.
 * Out: dq, dk, dv float32 [batch, heads, seq_len, 64].
 * workspace: at least llsa_dense_attn_bwd_workspace(p) bytes (D, float32
 *      per query).
 */
size_t llsa_dense_attn_bwd_workspace(const llsa_problem *p);
int llsa_dense_attn_bwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                        const void *o, const float *lse, const void *dout, float *dq, float *dk,
                        float *dv, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The debug index check on its own (the pick lists of every level, and the CSR
 * of levels 1..Le+1 unless csr_ptr or csr_col is NULL).  Every pick row must
 * hold K_l distinct values in [0, n_l), ascending, each (below level L) a child
 * of one of its parent's picks; every CSR level must be exactly the transpose
 * of its pick list (ptr bounds and monotonicity, each listed row in range,
 * ascending within the key, and having picked the key).  The sparse lists drive
 * every gather of the forward and backward passes (abstract: the operator uses
 * only sparse indices in both passes), so a caller that builds or edits lists
 * itself can check them before use.
 * In : idx (sizes.index_elems int32), csr_ptr / csr_col (layout of sizes), all
 *      DEVICE pointers; reads stay inside these buffers whatever their values.
 * Out: *status (DEVICE int32): cleared, then the OR of LLSA_IDX_* flags of
 *      what failed (0: valid).  Asynchronous on `stream`; p->index_status is
 *      ignored.
 */
int llsa_check_indices(const llsa_problem *p, const int32_t *idx, const int32_t *csr_ptr,
                       const int32_t *csr_col, int32_t *status, void *stream);

/* The same check on HOST copies of the lists (no HIP call): *flags receives
 * the OR of LLSA_IDX_* flags (0: valid). */
int llsa_check_indices_host(const llsa_problem *p, const int32_t *idx, const int32_t *csr_ptr,
                            const int32_t *csr_col, int32_t *flags);

/* Human-readable name of a status code (static string). */
const char *llsa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LLSA_H */
