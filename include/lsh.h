/*
 * lsh.h -- C ABI of the MI355X (gfx950) shared-QK LSH attention library.
 *
 * The library computes the hot path of LSH attention as described in
 * "Reformer: The Efficient Transformer" (Kitaev, Kaiser, Levskaya): angular
 * LSH by random rotation, a stable sort by (bucket, position), attention over
 * chunks of the sorted order (each chunk sees itself and one chunk back, with
 * self and duplicate masking, and causal masking unless the problem is
 * non-causal), a logsumexp-weighted combine over the hash rounds with the
 * unsort, and the backward pass through the fixed permutation.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to contiguous row-major arrays,
 *     owned by the caller, at least 16-byte aligned.  The library allocates
 *     nothing and frees nothing; the results of a call depend on its
 *     arguments only.  The one process-wide setting is the instrumentation
 *     bracket of lsh_profile_kernel (HIP events recorded around launches; it
 *     changes no result).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and nothing synchronises with the host.  Outputs are valid once the
 *     stream reaches that point.
 *   - The return value is an lsh_status_t.  Arguments are validated before
 *     anything is launched: LSH_ERR_INVALID for malformed arguments (null
 *     pointer, bad size, too small a workspace), LSH_ERR_UNSUPPORTED for a
 *     well-formed problem outside what the kernels implement.  A failed
 *     launch returns LSH_ERR_HIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - Results are deterministic: the same inputs give the same bits.
 *
 * Shapes: B batch, H heads, L sequence length, d head dim, nh hash rounds,
 * nb buckets, m chunk length.  "dtype" below is problem.dtype (fp32 or bf16).
 */
#ifndef LSH_H
#define LSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LSH_OK = 0,
    LSH_ERR_INVALID = 1,
    LSH_ERR_UNSUPPORTED = 2,
    LSH_ERR_HIP = 3
} lsh_status_t;

typedef enum { LSH_F32 = 0, LSH_BF16 = 1 } lsh_dtype_t;

/* Bits of lsh_problem_t.flags. */
typedef enum {
    /* Drop the same-bucket condition from the attended sets: the chunks of
     * the sorted order alone restrict attention (the alternative reading of
     * "Reformer" §2, where restricting each query to its own bucket is what
     * sorting and chunking approximate). */
    LSH_FLAG_NO_BUCKET_MASK = 1,
    /* Count duplicates over bucket membership ("Reformer" App. A defines the
     * count N_ij through the rounds in which j is in i's bucket): a member
     * that the query attends to in k_ij rounds weighs k_ij / N_ij, N_ij =
     * rounds in which it shares the query's bucket.  Without this flag each
     * member of the union counts once.  The two agree unless a bucket is
     * cut by the chunk window.  Not with LSH_FLAG_NO_BUCKET_MASK. */
    LSH_FLAG_DUP_BY_BUCKET = 2
} lsh_flag_t;

/* Which call a workspace is for (lsh_workspace_bytes). */
typedef enum {
    LSH_WS_SORT = 0,
    LSH_WS_FWD = 1,
    LSH_WS_BWD = 2,
    LSH_WS_TRAIN = 3,
    LSH_WS_REHASH = 4
} lsh_ws_kind_t;

/*
 * Problem description, passed by pointer to every call.
 *   batch, heads, seq_len, head_dim: B, H, L, d.  Supported: d in {32, 64, 128};
 *       B >= 0, H >= 0, 0 <= L <= 65536.  A problem with B, H or L equal to 0
 *       is empty: every call on it returns LSH_OK at once, without reading
 *       its pointers or launching anything.
 *   n_hashes: nh >= 1 hash rounds (<= 16); B * H * nh <= 65535 and
 *       B * H * nh * L < 2^31 (else LSH_ERR_UNSUPPORTED).
 *   n_buckets: nb, even, 2 <= nb <= 4096; nb = 2 * columns of the rotation.
 *   chunk_len: m, 1 <= m, L % m == 0 (m == L gives one chunk).
 *   causal: 1 = causal sets ("Reformer" §2: a query attends to no position
 *       after its own); 0 = non-causal (encoder) sets, which the paper does
 *       not spell out and are read here as the causal ones without that one
 *       condition: same bucket, own chunk or the one before (no look-ahead
 *       into the next chunk, no wrap-around from the first chunk to the
 *       last), self only when nothing else is there.  Other values:
 *       LSH_ERR_INVALID.
 *   scale: the softmax scale applied to q_i . k_j (1/sqrt(d) for standard
 *       scaled dot-product attention).
 *   dtype: element type of q, v, rot, out, dout, dq, dv and o_rounds.
 *   flags: 0, LSH_FLAG_NO_BUCKET_MASK (round set of a query: every position
 *       of its own chunk and the one before, not after it when causal; the
 *       rest as above) or LSH_FLAG_DUP_BY_BUCKET (duplicate count over
 *       bucket membership, see lsh_flag_t).  Unknown bits, or both:
 *       LSH_ERR_INVALID.
 */
typedef struct {
    int32_t batch, heads, seq_len, head_dim;
    int32_t n_hashes, n_buckets, chunk_len;
    int32_t causal;
    float scale;
    int32_t dtype; /* lsh_dtype_t */
    int32_t flags; /* lsh_flag_t bits */
} lsh_problem_t;

/* Human-readable text of a status code (static storage). */
const char *lsh_status_string(int status);

/* Version of this ABI: major * 10000 + minor * 100 + patch. */
int lsh_version(void);

/* Bytes of device workspace that lsh_sort (LSH_WS_SORT), lsh_attn_fwd
 * (LSH_WS_FWD), lsh_attn_bwd (LSH_WS_BWD) or lsh_attn_bwd_rehash
 * (LSH_WS_REHASH) needs for `prob`, or that one workspace shared by
 * lsh_attn_fwd and a later lsh_attn_bwd_saved needs (LSH_WS_TRAIN); 0 if the
 * problem is invalid or empty.  Alignment of every
 * workspace pointer: 256 bytes. */
size_t lsh_workspace_bytes(const lsh_problem_t *prob, int kind);

/*
 * lsh_hash -- angular LSH by random rotation ("Reformer" §2, random
 * projections h(x) = argmax([xR; -xR])).
 *   q       [B][H][L][d] dtype: queries (keys are q/|q|; hashing q or q/|q|
 *           gives the same bucket).
 *   rot     [nh][d][nb/2] dtype: one rotation per round, shared by all (b, h).
 *   buckets [B][H][nh][L] int32 out: index in [0, nb) of the largest entry of
 *           [qR_r ; -qR_r]; entry j < nb/2 is +y_j, entry nb/2 + j is -y_j;
 *           ties go to the smaller index.
 * Products are formed exactly and summed in fp32.
 */
int lsh_hash(const lsh_problem_t *prob, const void *q, const void *rot, int32_t *buckets,
             void *stream);

/*
 * lsh_sort -- per (b, h, round), the stable sort of positions by bucket
 * ("Reformer" §2: sorting by bucket clusters same-bucket pairs; ties by
 * position), i.e. ascending order of the unique keys bucket * L + position.
 *   buckets [B][H][nh][L] int32 in, values in [0, nb).
 *   perm    [B][H][nh][L] int32 out: sorted index -> position.
 *   inv     [B][H][nh][L] int32 out: position -> sorted index.
 *   win_lo  [B][H][nh][L] int32 out, indexed by position t: the smallest
 *           sorted index of the round's attended set of t (same bucket, not
 *           after t, own chunk or the one before):
 *           max(first sorted index of t's bucket, (inv[t]/m - 1) * m).
 *           The causal set is exactly the sorted range [win_lo[t], inv[t]].
 *           The non-causal set starts at the same index and ends at the last
 *           sorted index of t's bucket inside t's chunk; lsh_attn_fwd and
 *           the backwards derive that end from perm and win_lo, so the
 *           output of lsh_sort is the same for both kinds of problem (and
 *           with LSH_FLAG_NO_BUCKET_MASK, whose sets the attention calls
 *           take from the chunks alone).
 *   ws      workspace of lsh_workspace_bytes(prob, LSH_WS_SORT) bytes.
 * Bucket values outside [0, nb) are not reported: the kernels clamp them into
 * [0, nb), so the outputs are then meaningless but every write stays inside
 * perm, inv, win_lo and the workspace.
 */
int lsh_sort(const lsh_problem_t *prob, const int32_t *buckets, int32_t *perm, int32_t *inv,
             int32_t *win_lo, void *ws, size_t ws_bytes, void *stream);

/*
 * lsh_sort_noalloc -- lsh_sort for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments as lsh_sort without
 * ws / ws_bytes and the same results bit for bit; the per-tile count matrix
 * (lsh_workspace_bytes(prob, LSH_WS_SORT) bytes) lives instead in a static
 * device array of the library, LSH_SORT_NOALLOC_MAX_BYTES on every GPU it
 * runs on, held until the process ends.  The call allocates nothing; its
 * first call on a GPU looks up that GPU's copy of the array (the GPU of
 * `stream`, or the current one for the null stream).
 *   Problems whose count matrix is larger than LSH_SORT_NOALLOC_MAX_BYTES:
 *   LSH_ERR_UNSUPPORTED, before anything is launched.
 *   Calls on one GPU share its array, which keeps the last call's counts
 *   (each call writes every count it reads, so nothing has to start at
 *   zero): calls that may overlap on one GPU (streams not ordered with each
 *   other) race and must not be issued.
 */
#define LSH_SORT_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int lsh_sort_noalloc(const lsh_problem_t *prob, const int32_t *buckets, int32_t *perm, int32_t *inv,
                     int32_t *win_lo, void *stream);

/*
 * lsh_attn_fwd -- per-round chunked attention ("Reformer" §2 and App. A):
 * in round r, query t attends to the members of its attended set (causal or
 * not, see lsh_problem_t) other than itself, with logits
 * scale * q_t . k_j, k_j = q_j / |q_j|.  A member j that
 * already belongs to the attended set of t in an earlier round is masked
 * (the duplicate correction of App. A, folded into the mask), so that the
 * rounds together count every member of the union once.  Outputs are
 * written at the original positions (the unsort).
 *   q, v       [B][H][L][d] dtype.
 *   perm, inv, win_lo  as produced by lsh_sort.
 *   o_rounds   [B][H][nh][L][d] dtype out: softmax-weighted average of v over
 *              the round's unmasked members (0 if there are none).
 *   lse_rounds [B][H][nh][L] fp32 out: log of the round's softmax
 *              denominator (-inf if there are no unmasked members).
 *   ws         workspace of lsh_workspace_bytes(prob, LSH_WS_FWD) bytes, or
 *              of LSH_WS_TRAIN bytes to keep what the forward derives from
 *              q, perm, inv and win_lo (packed sorted records, inverse norms,
 *              per-block key data; for non-causal problems also the window
 *              ends) for lsh_attn_bwd_saved.
 */
int lsh_attn_fwd(const lsh_problem_t *prob, const void *q, const void *v, const int32_t *perm,
                 const int32_t *inv, const int32_t *win_lo, void *o_rounds, float *lse_rounds,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * lsh_combine -- logsumexp-weighted combine over the rounds ("Reformer"
 * App. A: each round's output is independently computable and the outputs
 * are combined):  lse_t = log sum_r exp(lse_rounds[r][t]),
 * out_t = sum_r exp(lse_rounds[r][t] - lse_t) o_rounds[r][t].
 * A token with no member in any round (e.g. the first token) attends only to
 * itself: out_t = v_t and lse_t = scale * |q_t| ("Reformer" §2 and App. A
 * masking rule).
 *   q, v       [B][H][L][d] dtype (read only for such tokens).
 *   o_rounds, lse_rounds  as produced by lsh_attn_fwd.
 *   out        [B][H][L][d] dtype out.   lse  [B][H][L] fp32 out.
 */
int lsh_combine(const lsh_problem_t *prob, const void *q, const void *v, const void *o_rounds,
                const float *lse_rounds, void *out, float *lse, void *stream);

/*
 * lsh_attn_bwd -- gradient of the combined output with respect to q and v,
 * with the bucket assignment and sort order held fixed (no differentiation
 * through hashing or sorting, as the Reformer authors state in Hacker News
 * thread 22095523).  Gradient flows through both the query and the
 * normalised key k = q / |q|.
 *   q, v, out, dout  [B][H][L][d] dtype; out and lse as produced by
 *                    lsh_combine for the same q, v, perm, inv, win_lo.
 *   lse        [B][H][L] fp32.
 *   perm, inv, win_lo  as produced by lsh_sort.
 *   dq, dv     [B][H][L][d] dtype out.
 *   ws         workspace of lsh_workspace_bytes(prob, LSH_WS_BWD) bytes.
 */
int lsh_attn_bwd(const lsh_problem_t *prob, const void *q, const void *v, const void *out,
                 const void *dout, const float *lse, const int32_t *perm, const int32_t *inv,
                 const int32_t *win_lo, void *dq, void *dv, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * lsh_attn_bwd_rehash -- lsh_attn_bwd for the reversible-layer setting
 * ("Reformer" §3: activations are recovered in the backward pass instead of
 * being stored): the buckets, the sorted order and the window starts are
 * recomputed from q and rot (lsh_hash and lsh_sort inside the call), so the
 * caller keeps none of them between the forward and the backward.  Hashing
 * and sorting are deterministic, so the gradient is the same, bit for bit,
 * as lsh_attn_bwd's with the forward's perm, inv and win_lo.
 *   q, v, out, dout, lse, dq, dv  as for lsh_attn_bwd.
 *   rot        [nh][d][nb/2] dtype: the rotations the forward hashed with.
 *   ws         workspace of lsh_workspace_bytes(prob, LSH_WS_REHASH) bytes
 *              (scratch only; nothing in it is needed after the call).
 */
int lsh_attn_bwd_rehash(const lsh_problem_t *prob, const void *q, const void *v, const void *rot,
                        const void *out, const void *dout, const float *lse, void *dq, void *dv,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * lsh_attn_bwd_saved -- lsh_attn_bwd for a training step that keeps the
 * forward's workspace: the gradient is the same (bit for bit), but the
 * records that the forward derived from q, perm, inv and win_lo are read
 * from ws instead of being derived again.
 *   ws         workspace of at least lsh_workspace_bytes(prob, LSH_WS_TRAIN)
 *              bytes that was passed to lsh_attn_fwd for the same problem,
 *              q, perm, inv and win_lo, and that nothing has written to
 *              since (the caller's contract; it is not checked, and results
 *              are undefined if it does not hold).  Its first LSH_WS_FWD
 *              bytes are read, the rest is overwritten.
 *   other arguments as for lsh_attn_bwd.
 */
int lsh_attn_bwd_saved(const lsh_problem_t *prob, const void *q, const void *v, const void *out,
                       const void *dout, const float *lse, void *dq, void *dv, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * Chunked feed-forward layer ("Reformer" §3, Reversible Transformer: the
 * feed-forward computation is independent across positions, so it is split
 * into c chunks of positions, forward, recomputation and backward alike).
 * The layer is the standard Transformer one, y = relu(x W1 + b1) W2 + b2,
 * row by row; only one chunk's hidden activations (ceil(rows / c) x d_ff)
 * are held at a time, in the workspace.  Hidden activations and their
 * gradient are kept in bf16; products accumulate in fp32.
 *   rows: n >= 0 positions (B * L); rows == 0 is a no-op returning LSH_OK.
 *   d_model, d_ff: multiples of 8, at least 8.
 *   chunks: c >= 1.
 *   dtype: LSH_BF16 (x, w1, w2, y, dy, dx); LSH_F32 returns
 *       LSH_ERR_UNSUPPORTED.
 */
typedef struct {
    int32_t rows, d_model, d_ff, chunks;
    int32_t dtype; /* lsh_dtype_t */
} lsh_ff_t;

/* Workspace bytes of lsh_ff_fwd (backward = 0) or lsh_ff_bwd (backward = 1);
 * 0 if the description is invalid or empty.  Alignment: 256 bytes. */
size_t lsh_ff_workspace_bytes(const lsh_ff_t *ff, int backward);

/*
 * lsh_ff_fwd -- y = relu(x W1 + b1) W2 + b2, chunk by chunk.
 *   x  [n][d_model] bf16;  w1 [d_model][d_ff] bf16;  b1 [d_ff] fp32;
 *   w2 [d_ff][d_model] bf16;  b2 [d_model] fp32;  y [n][d_model] bf16 out.
 *   Device pointers, x, w1, w2, y 16-byte aligned; ws as returned by
 *   lsh_ff_workspace_bytes(ff, 0).
 */
int lsh_ff_fwd(const lsh_ff_t *ff, const void *x, const void *w1, const float *b1, const void *w2, const float *b2,
               void *y, void *ws, size_t ws_bytes, void *stream);

/*
 * lsh_ff_bwd -- gradients of sum(y * dy) for lsh_ff_fwd, chunk by chunk: the
 * hidden activations of a chunk are recomputed from x (nothing is kept from
 * the forward), then dH = (dy W2^T) * relu'(x W1 + b1), dx = dH W1^T, and the
 * weight and bias gradients are summed over the chunks in fp32.
 *   dy [n][d_model] bf16;  dx [n][d_model] bf16 out;
 *   dw1 [d_model][d_ff], db1 [d_ff], dw2 [d_ff][d_model], db2 [d_model]
 *   fp32 out (overwritten, not added to).
 *   ws as returned by lsh_ff_workspace_bytes(ff, 1).
 */
int lsh_ff_bwd(const lsh_ff_t *ff, const void *x, const void *w1, const float *b1, const void *w2, const void *dy,
               void *dx, float *dw1, float *db1, float *dw2, float *db2, void *ws, size_t ws_bytes, void *stream);

/*
 * Instrumentation (not needed to compute anything).
 *
 * Kernels of the library, for lsh_profile_kernel and lsh_kernel_name.
 */
typedef enum {
    LSH_KERNEL_HASH = 0,        /* lsh_hash: rotation + argmax                      */
    LSH_KERNEL_SORT_COUNT = 1,  /* lsh_sort: per-tile bucket counts                 */
    LSH_KERNEL_SORT_SCATTER = 2,/* lsh_sort: bucket starts and earlier-tile counts
                                   from the count matrix, stable ranks,
                                   perm / inv / win_lo                            */
    LSH_KERNEL_PREP = 3,        /* lsh_attn_fwd / lsh_attn_bwd: packed records,
                                   inverse norms, non-causal window ends (and
                                   dO . O in the backward; only that in
                                   lsh_attn_bwd_saved)                             */
    LSH_KERNEL_FWD = 4,         /* lsh_attn_fwd: per-round chunk attention          */
    LSH_KERNEL_COMBINE = 5,     /* lsh_combine                                      */
    LSH_KERNEL_BWD_DQ = 6,      /* lsh_attn_bwd: query-side gradient per round      */
    LSH_KERNEL_BWD_DKV = 7,     /* lsh_attn_bwd: key-side gradients per round       */
    LSH_KERNEL_BWD_REDUCE = 8,  /* lsh_attn_bwd: sum over rounds, key normalisation */
    LSH_KERNEL_TILES = 9,       /* lsh_attn_fwd / lsh_attn_bwd (bf16 matrix-core
                                   path): per-32-row metadata tiles             */
    LSH_KERNEL_COUNT = 10
} lsh_kernel_t;

/* Name of a kernel id (static storage), or NULL for an unknown id. */
const char *lsh_kernel_name(int kernel);

/*
 * lsh_profile_kernel -- bracket every later launch of `kernel` with
 * hipEventRecord(start_event) before it and hipEventRecord(stop_event) after
 * it, on the stream the kernel is launched on.  start_event and stop_event
 * are hipEvent_t handles owned by the caller; passing NULL for either clears
 * the bracket.  The setting is process-wide and not synchronised: set it from
 * the thread that launches, between calls.  Returns LSH_ERR_INVALID for an
 * unknown kernel id.
 */
int lsh_profile_kernel(int kernel, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* LSH_H */
