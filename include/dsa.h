/*
 * dsa.h -- C ABI of libdsa, the DeepSeek-Sparse-Attention (DSA) decode /
 * prefill path for AMD Instinct MI355X (gfx950).
 *
 * The path has three stages plus reuse of one index set across layers:
 *
 *   dsa_index_k_cache_write  index-cache writer: rope + fp8 keys with a
 *   dsa_index_q_quant        power-of-two scale (and the same for prefill
 *   dsa_index_front_end      index queries, or both in one launch), the step
 *                            in front of the indexer
 *   dsa_index_scores         lightning indexer: one fp32 score per visible
 *                            cached token for every query row
 *   dsa_topk                 per-row top-k (k <= DSA_TOPK_MAX) positions
 *   sparse_mla_decode        attention of H query heads over only the
 *   sparse_mla_prefill       selected rows of a latent KV cache
 *   sparse_mla_decode_shared several layers' sparse MLA over one index set
 *
 * Citations are to the reference pages by title and section:
 *   [anatomy]  "GLM-5.2 架构解剖" (GLM-5.2 anatomy);
 *   [guide]    "ATOM Model Support Guide";
 *   [pr2980]   ATOM pull request #2980 (FP8 weight planes in mono decode);
 *   [serving]  the ATOM serving and benchmarking guide.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer (HIP memory visible to
 *   the current device) unless its comment says "host".  The caller owns
 *   every buffer; the library keeps no pointer after a call returns and
 *   allocates no device memory.  Buffers must stay alive until the stream
 *   has executed the call.
 * Streams.  Every call only enqueues work on `stream` (a hipStream_t, NULL =
 *   the default stream) and never synchronises the host.
 * Errors.  All arguments are checked on the host first.  A failed check
 *   returns a negative dsa_status, sets the thread-local message read by
 *   dsa_last_error(), and launches nothing, so no output is partially
 *   written.  A failed launch returns DSA_ERR_HIP.  Device faults surface at
 *   the caller's next synchronisation.  No C++ exception crosses the ABI.
 * Determinism.  Identical inputs give bitwise-identical outputs.  There are
 *   no floating-point atomics; every reduction has a fixed order.
 * Preconditions the library does not check (they need device data):
 *   kv_indptr / q_indptr are non-decreasing, every context is >= 1 and
 *   <= max_ctx, q_len_b <= ctx_b; scales are finite and > 0; no fp8 NaN
 *   codes (0x7F, 0xFF); the indices given to sparse MLA were produced for the
 *   same layout (unique, < n_i, or -1; physical rows < cache_rows when
 *   paged); block-table entries address pages inside the caches.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2

/* Largest k accepted by dsa_topk and the sparse MLA entry points. */
#define DSA_TOPK_MAX 2048

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad stride          */
    DSA_ERR_UNSUPPORTED = -2, /* dtype / shape combination not implemented   */
    DSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
    DSA_ERR_HIP = -4          /* a HIP launch or query failed                */
} dsa_status;

typedef enum {
    DSA_F32 = 0,
    DSA_BF16 = 1,          /* bfloat16                                        */
    DSA_FP8_E4M3FN = 2     /* OCP E4M3, finite-only (max 448): the fp8 format
                              of gfx950 ([pr2980], Limitations)              */
} dsa_dtype;

/*
 * Ragged batch layout, shared by every call ([guide], DeepSeek V2/V3: MLA
 * attention metadata is tracked with kv_indptr).
 *
 * Sequence b has ctx_b = kv_indptr[b+1] - kv_indptr[b] cached tokens and
 * query rows q_indptr[b] .. q_indptr[b+1]-1 (q_len_b rows).  Query j of
 * sequence b sits at position p = ctx_b - q_len_b + j and sees the causal
 * prefix 0 .. p, i.e. n = p + 1 tokens.  q_indptr == NULL means one query per
 * sequence (decode): T = B and n = ctx_b.
 *
 * Where a token's row is.  Contiguous caches (block_table == NULL): token s of
 * sequence b is row kv_indptr[b] + s of every per-token cache (index keys and
 * each layer's latent KV).  Paged caches ([serving], server options: the KV
 * cache is kept in blocks, 16 tokens by default; [anatomy], verified
 * deployments, note on the SGLang plugin path: full layers write a shared
 * buffer of physical indices that shared layers read): token s of sequence b
 * is row
 *     block_table[b * block_table_stride + s / page_size] * page_size + s % page_size
 * of every per-token cache, and top-k indices and sparse-MLA indices are such
 * physical rows instead of positions.  The tuned kernels take power-of-two
 * page sizes up to 4096; other page sizes run the generic kernels.
 */
typedef struct {
    int32_t batch;             /* B >= 1                                      */
    int32_t total_q;           /* T: query rows (= q_indptr[B]; = B for decode) */
    int64_t max_ctx;           /* host upper bound of every ctx_b (>= 1)      */
    const int64_t *kv_indptr;  /* device [B+1]                                */
    const int32_t *q_indptr;   /* device [B+1], or NULL for decode            */
    const int32_t *block_table;   /* device [B][block_table_stride] page ids, or
                                     NULL for contiguous caches               */
    int32_t block_table_stride;   /* >= ceil(max_ctx / page_size) when paged  */
    int32_t page_size;            /* tokens per page (>= 1) when paged        */
    int64_t cache_rows;           /* rows of every per-token cache when paged
                                     (bounds the physical rows; > 0)          */
} dsa_layout;

/*
 * dsa_index_k_cache_write / dsa_index_q_quant -- index-cache writer ([anatomy],
 * full structure diagram, Indexer box: the index key takes interleaved rope,
 * then fp8 per-1x128 quantisation with a ue8m0 scale, and is written into the
 * 132-byte index cache; ATOM-side optimisations, fused indexer kernel: query
 * rope, fp8 quantisation and key-cache write in one pass, for 128-wide index
 * heads with 64 rope dims; section on the rope switches: GLM's indexer rope is
 * the interleaved style).  Each group of 128 values (one key, or one head of
 * an index query) is turned into
 *
 *   y     the group; if cos_sin is non-NULL, dims [rope_off, rope_off + 64)
 *         are rotated in interleaved pairs (2i, 2i+1), i < 32, with the table
 *         row c = cos_sin[pos * 64 + i], s = cos_sin[pos * 64 + 32 + i]:
 *         (y0, y1) = (x0*c - x1*s, x0*s + x1*c), each product and sum an fp32
 *         rounding of its own
 *   scale the smallest power of two 2^e with max|y| <= 448 * 2^e and
 *         e >= -126 (a normal fp32); 1 for an all-zero group
 *   codes y / scale rounded to the nearest OCP E4M3FN value, ties to the even
 *         code, with the sign kept (so -0 gives 0x80)
 *
 * Inputs are F32 or BF16 values, finite.  The codes are what dsa_index_scores
 * reads as FP8_E4M3FN keys with k_scale (and prefill queries with q_scale).
 *
 * dsa_index_k_cache_write writes n new keys:
 *   k, k_dt       key r (128 values) starts at byte r * k_row_stride of k; k
 *                 16-byte aligned, k_row_stride a multiple of 16 (a column
 *                 slice of a wider projection output works).
 *   positions     int64 [n] rope positions; required iff cos_sin is non-NULL.
 *   cos_sin       fp32 [rope_rows][64] (cos of the 32 frequencies, then their
 *                 sin), 16-byte aligned, or NULL for no rope.  rope_off is 0
 *                 or 64.  Positions outside [0, rope_rows) break the contract;
 *                 the kernel clamps them into the table and never reads past it.
 *   slots         int64 [n]: key r goes to cache row slots[r]; a negative slot
 *                 is skipped (padding).  Slots >= cache_rows break the contract
 *                 and are skipped too, so no write leaves the cache.
 *   cache         codes of row j at cache + j * cache_row_stride (bytes; a
 *                 multiple of 4, base 4-byte aligned).
 *   cache_scale   fp32 scale of row j at cache_scale[j * cache_scale_stride].
 *                 The interleaved 132-byte entries are cache_row_stride = 132,
 *                 cache_scale = (float *)(cache + 128), cache_scale_stride = 33.
 * Rows that no slot names keep their bytes.  Two keys with the same slot race.
 * n = 0 (or T = 0 below) is a no-op whose pointers may be NULL.
 *
 * dsa_index_q_quant quantises T index-query rows of H_I heads:
 *   q, q_dt       row t (H_I * 128 values, head-major) at byte t * q_row_stride
 *                 of q; 16-byte alignment as for k.
 *   positions, cos_sin, rope_rows, rope_off   as above, per row.
 *   q_fp8         uint8 [T][H_I][128] codes; q_scale fp32 [T][H_I] scales.
 */
dsa_status dsa_index_k_cache_write(int64_t n, dsa_dtype k_dt, const void *k, int64_t k_row_stride,
                                   const int64_t *positions, const float *cos_sin,
                                   int64_t rope_rows, int rope_off, const int64_t *slots,
                                   uint8_t *cache, int64_t cache_row_stride, float *cache_scale,
                                   int64_t cache_scale_stride, int64_t cache_rows, void *stream);
dsa_status dsa_index_q_quant(int64_t T, int H_I, dsa_dtype q_dt, const void *q, int64_t q_row_stride,
                             const int64_t *positions, const float *cos_sin, int64_t rope_rows,
                             int rope_off, uint8_t *q_fp8, float *q_scale, void *stream);

/*
 * dsa_index_front_end -- both of the above in one launch, the fused form of the
 * step ([anatomy], ATOM-side optimisations, fused indexer kernel: query rope,
 * fp8 quantisation and key-cache write as one kernel).  T new tokens, each with
 * H_I index-query heads (q, as for dsa_index_q_quant) and one index key (k, as
 * for dsa_index_k_cache_write), both of dtype dt and both roped at
 * positions[t].  The results are bitwise those of the two separate calls.
 */
dsa_status dsa_index_front_end(int64_t T, int H_I, dsa_dtype dt, const void *q, int64_t q_row_stride,
                               const void *k, int64_t k_row_stride, const int64_t *positions,
                               const float *cos_sin, int64_t rope_rows, int rope_off,
                               const int64_t *slots, uint8_t *cache, int64_t cache_row_stride,
                               float *cache_scale, int64_t cache_scale_stride, int64_t cache_rows,
                               uint8_t *q_fp8, float *q_scale, void *stream);

/*
 * dsa_index_scores -- lightning-indexer scores ([anatomy], full structure
 * diagram, Indexer box: 32 index heads x 128 dims, one key per token shared
 * by every index head, keys stored as fp8 with a per-token scale in a
 * 132-byte index-cache entry).  For every query row i and visible token
 * s < n_i:
 *
 *     score[i, s] = sum_h w[i,h] * ReLU( (q[i,h,:] . k[s,:]) * qs[i,h] * ks[s] )
 *
 * with qs = 1 when q_scale is NULL and ks = 1 when k_scale is NULL.
 *
 *   H_I, D_I      index heads and head dim (any H_I <= 64, D_I <= 256; the
 *                 tuned kernels take H_I = 32, D_I = 128).
 *   q_dt, q       [T][H_I][D_I] of q_dt (F32, BF16 or FP8_E4M3FN), contiguous.
 *   q_scale       [T][H_I] fp32, required iff q_dt is FP8_E4M3FN, else NULL.
 *   w             [T][H_I] fp32 head weights.
 *   k_dt, k       key row r (global cache row) starts at byte r * k_row_stride
 *                 of k and holds D_I elements of k_dt.  k_row_stride >= D_I *
 *                 elem size; 132 with k_scale = (float*)(k + 128) and
 *                 k_scale_stride = 33 reads the interleaved 132-byte entries.
 *   k_scale       fp32 scale of row r at k_scale[r * k_scale_stride];
 *                 required iff k_dt is FP8_E4M3FN.
 *   scores, ld    fp32 output, row i at scores + i * ld; ld >= max_ctx.  Only
 *                 s < n_i is written.
 * The fp8 x bf16 products are exact in fp32; sums are fp32.
 * The tuned kernels (H_I = 32, D_I = 128, fp8 keys) need k 4-byte aligned and
 * k_row_stride a multiple of 4, which the interleaved 132-byte entries meet;
 * other keys run the generic kernel.  The tuned fp8-query kernel addresses
 * keys with 32-bit offsets: it needs max_ctx * k_row_stride (cache_rows *
 * k_row_stride with paged caches) below 2^31; beyond it the generic kernel
 * runs (same results, slower).
 */
dsa_status dsa_index_scores(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt,
                            const void *q, const float *q_scale, const float *w,
                            dsa_dtype k_dt, const void *k, int64_t k_row_stride,
                            const float *k_scale, int64_t k_scale_stride, float *scores,
                            int64_t ld, void *stream);

/*
 * dsa_topk -- per-row top-k selection ([anatomy], Indexer box: top-k = 2048
 * written as int32 [tokens x 2048]; ATOM-side optimisations, stable_topk:
 * ties must not be broken arbitrarily; caveats: with fewer visible tokens
 * than k every token is taken).
 *
 * Row i considers scores[i * ld + s] for s < n_i and selects the first
 * min(k, n_i) positions under the strict order "higher score first; equal
 * scores (with -0 == +0) by lower position".  It writes them to
 * indices[i * k .. i * k + k - 1] in ascending position order (the attention
 * over them does not depend on the order; the pages fix the set, not its
 * listing), then -1 in the remaining slots.  Positions are logical (0 ..
 * ctx_b - 1 within the sequence), or with paged caches the tokens' physical
 * rows (see dsa_layout).  1 <= k <= DSA_TOPK_MAX.  NaN scores are outside the
 * contract.
 *   workspace     device scratch of dsa_topk_workspace_size() bytes, needed
 *                 when max_ctx exceeds what one block holds (32768): a
 *                 score histogram per row and, for up to 512 long rows, each
 *                 row's bitmap of selected positions, its threshold-bin
 *                 candidates and the threshold bin itself (handed from one
 *                 kernel to the next); may be NULL when the size is 0.  It must be
 *                 zero-filled before its first use; every completed call leaves
 *                 all of it zero again, whatever the layout.  Calls that overlap
 *                 in time must not share it.
 */
size_t dsa_topk_workspace_size(const dsa_layout *layout, int64_t ld, int k);
dsa_status dsa_topk(const dsa_layout *layout, const float *scores, int64_t ld, int k,
                    int32_t *indices, void *workspace, size_t workspace_bytes, void *stream);

/*
 * dsa_index_topk -- dsa_index_scores followed by dsa_topk as one call, with
 * the top-k's histogram pass folded into the indexer ([anatomy], ATOM's
 * GLM-5.2 optimisations: the indexer's steps fused into one kernel; stable
 * top-k).  Arguments: those of dsa_index_scores (scores is still written:
 * the selection reads it), then k, indices and workspace as for dsa_topk
 * (workspace of dsa_topk_workspace_size() bytes, zero before its first use,
 * left zero by every completed call).  Results: the same scores and indices,
 * bit for bit, as the two separate calls.  For bf16 index queries (the decode
 * indexer) and rows longer than 32768 scores, the indexer adds every row's
 * histogram of the top 11 bits of its score keys to the workspace while it
 * writes the scores, and the selection skips its own histogram pass; every
 * other shape runs the two separate launches.  Every check of both calls
 * runs before anything is launched.
 */
dsa_status dsa_index_topk(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt,
                          const void *q, const float *q_scale, const float *w, dsa_dtype k_dt,
                          const void *k, int64_t k_row_stride_bytes, const float *k_scale,
                          int64_t k_scale_stride, float *scores, int64_t ld_scores, int k_top,
                          int32_t *indices, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * dsa_index_scores_hist / dsa_topk_after_hist -- dsa_index_topk as two calls
 * (same passages), so that a caller can time the two stages or put other
 * work between them.
 *   dsa_index_scores_hist takes dsa_index_topk's arguments without indices
 *   and one more, hist_built (host int, not NULL): it writes the scores and,
 *   for the shapes where dsa_index_topk folds the histogram into the
 *   indexer, adds each row's histogram to the workspace and sets *hist_built
 *   to 1; otherwise it sets 0 (the workspace is then untouched).
 *   dsa_topk_after_hist takes dsa_topk's arguments and the hist_built value:
 *   with 1 it runs only the selection, on the histogram the indexer call
 *   left in the workspace; with 0 it is dsa_topk.
 * Between the two calls nothing else may use the workspace, and the layout,
 * scores, ld and workspace must be the same in both; hist_built = 1 without
 * a preceding dsa_index_scores_hist that returned it gives undefined indices.
 * Together they give dsa_index_topk's scores and indices, bit for bit, and
 * leave the workspace zero as it does.  Checks: those of dsa_index_topk
 * (hist_built NULL is DSA_ERR_INVALID_ARG), each before its own launch.
 */
dsa_status dsa_index_scores_hist(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt,
                                 const void *q, const float *q_scale, const float *w,
                                 dsa_dtype k_dt, const void *k, int64_t k_row_stride_bytes,
                                 const float *k_scale, int64_t k_scale_stride, float *scores,
                                 int64_t ld_scores, int k_top, void *workspace,
                                 size_t workspace_bytes, int *hist_built, void *stream);
dsa_status dsa_topk_after_hist(const dsa_layout *layout, const float *scores, int64_t ld, int k,
                               int32_t *indices, void *workspace, size_t workspace_bytes,
                               int hist_built, void *stream);

/*
 * sparse_mla_decode / sparse_mla_prefill -- attention over the selected
 * latent rows ([anatomy], full structure diagram, sparse MLA box: 64 heads
 * computed only on the 2048 selected rows of the latent KV cache, 576 = 512
 * latent + 64 rope values per token).  The absorbed form: the key is the
 * whole D_c + D_r row, the value is its first D_c entries, and the output
 * stays in latent space.  For every query row i and head h, with J the
 * non-negative entries of indices[i * k .. i * k + k - 1]:
 *
 *   z_j   = sm_scale * kv_scale * (q[i,h,:] . c[kv_indptr[b] + J_j, :])
 *           (c[J_j, :] with paged caches: J_j is then a physical row)
 *   o     = sum_j softmax(z)_j * kv_scale * c[kv_indptr[b] + J_j, 0:D_c]
 *   lse   = log sum_j exp(z_j)          (o = 0, lse = -inf when J is empty)
 *
 *   H, D_c, D_r   heads, latent width, rope width.  Tuned kernels: H = 64,
 *                 D_c = 512, D_r = 64, bf16 q, bf16 or fp8 KV.  Other shapes
 *                 (H <= 128, D_c <= 512, D_c + D_r <= 1024) run a generic
 *                 kernel.
 *   q             [T][H][D_c + D_r] of q_dt (F32 or BF16).
 *   kv            [rows][D_c + D_r] of kv_dt (F32, BF16 or FP8_E4M3FN) with
 *                 one per-tensor scale kv_scale (use 1 for F32 / BF16).
 *   indices, k    int32 [T][k] logical positions (< n_i) or -1.
 *   out           [T][H][D_c] of out_dt (F32 or BF16).
 *   lse           fp32 [T][H], or NULL.
 *   workspace     device scratch of sparse_mla_workspace_size() bytes (the
 *                 split partials of the index list; none is needed when one
 *                 block covers a whole row).  No initial contents are needed.
 *                 Calls that overlap in time must not share a workspace.
 * The tuned kernels need max_ctx * (D_c + D_r) * element size <= 4 GiB - 1 MiB
 * (cache_rows * (D_c + D_r) * element size with paged caches); beyond it the
 * generic kernel runs.
 * The two entries run the same code: the kernel and the split of each row's
 * index list follow the number of query rows T (half-head blocks for bf16 KV
 * up to 64 rows, full-head blocks beyond; key splits while T < 256), whatever
 * the entry, so a prefill chunk and a decode batch of the same T and dtypes
 * take the same path.  Both accept any layout; the two names mark the two
 * call sites of a model (a prefill chunk with q_len_b > 1, a decode step).
 */
size_t sparse_mla_workspace_size(const dsa_layout *layout, int H, int D_c, int D_r, int k,
                                 int n_layers);
dsa_status sparse_mla_decode(const dsa_layout *layout, int H, int D_c, int D_r, float sm_scale,
                             dsa_dtype q_dt, const void *q, dsa_dtype kv_dt, const void *kv,
                             float kv_scale, const int32_t *indices, int k, dsa_dtype out_dt,
                             void *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream);
dsa_status sparse_mla_prefill(const dsa_layout *layout, int H, int D_c, int D_r, float sm_scale,
                              dsa_dtype q_dt, const void *q, dsa_dtype kv_dt, const void *kv,
                              float kv_scale, const int32_t *indices, int k, dsa_dtype out_dt,
                              void *out, float *lse, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * sparse_mla_decode_no_alloc -- sparse_mla_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and result as
 * sparse_mla_decode (bit for bit: the same kernels), without the workspace:
 * the split partials live in a static device array of
 * DSA_NO_ALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The call allocates nothing and needs no initial
 * contents of that array.  Every call on one GPU uses the same array, so calls
 * that overlap in time on one GPU (several streams, several threads) race and
 * must be serialised by the caller.  A call whose split partials would exceed
 * the array (none with k <= DSA_TOPK_MAX under the library's split policy)
 * returns DSA_ERR_WORKSPACE and launches nothing.
 */
#define DSA_NO_ALLOC_SCRATCH_BYTES (64u << 20)
dsa_status sparse_mla_decode_no_alloc(const dsa_layout *layout, int H, int D_c, int D_r,
                                      float sm_scale, dsa_dtype q_dt, const void *q,
                                      dsa_dtype kv_dt, const void *kv, float kv_scale,
                                      const int32_t *indices, int k, dsa_dtype out_dt, void *out,
                                      float *lse, void *stream);

/*
 * sparse_mla_decode_shared -- IndexShare ([anatomy], layer scheduling:
 * "shared" layers carry no indexer and reuse the indices the previous "full"
 * layer selected; full structure diagram: one int32 [tokens x 2048] buffer is
 * read by every layer).  Runs sparse_mla_decode for n_layers layers, each
 * with its own q, latent KV, scale and outputs, over the same indices, in one
 * launch.  Layer l's result is bitwise equal to sparse_mla_decode on layer l.
 * The index set must have been written by a full layer before (a shared layer
 * cannot come first: it would read a buffer nobody wrote; [anatomy], layer
 * scheduling, invariant box); the library cannot check this.
 *   layers        HOST array of n_layers descriptors (1 <= n_layers <=
 *                 DSA_MAX_SHARED_LAYERS); every layer uses the same dtypes.
 */
#define DSA_MAX_SHARED_LAYERS 8
typedef struct {
    const void *q;   /* [T][H][D_c + D_r] */
    const void *kv;  /* [rows][D_c + D_r] */
    float kv_scale;
    void *out;       /* [T][H][D_c]       */
    float *lse;      /* [T][H] or NULL    */
} dsa_mla_layer;

dsa_status sparse_mla_decode_shared(const dsa_layout *layout, int H, int D_c, int D_r,
                                    float sm_scale, dsa_dtype q_dt, dsa_dtype kv_dt,
                                    dsa_dtype out_dt, int n_layers, const dsa_mla_layer *layers,
                                    const int32_t *indices, int k, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * dsa_gather_ceiling -- a measurement aid; no step of the method.  Gathers the
 * rows of a latent cache that an index set selects, with the buffer-to-LDS
 * loads and slot geometry of the tuned sparse-MLA kernels, and discards them:
 * the row traffic of the sparse-MLA stage without its arithmetic, so the
 * bandwidth it reaches on a workload's own indices bounds that stage.
 *   rows        device, n_rows rows of row_bytes bytes (576: fp8 latent
 *               rows, 1152: bf16), read only
 *   indices     device int32 [T][k]: rows of `rows` (absolute; -1 = none)
 *   sink        device, >= 4 bytes: receives one word of the gathered data
 *   stream      hipStream_t, or NULL for the default stream
 * One 512-thread block per 256 index slots of a row, three 32-row slots in
 * flight.  Errors: DSA_ERR_INVALID_ARG for NULL pointers, row_bytes other than
 * 576 or 1152, T < 1, k outside 1 .. DSA_TOPK_MAX, n_rows < 1 or a table of
 * 4 GiB - 1 MiB or more; DSA_ERR_HIP if the launch fails.  Nothing is
 * allocated.
 */
dsa_status dsa_gather_ceiling(const void *rows, int64_t n_rows, int row_bytes, const int32_t *indices,
                              int64_t T, int k, uint32_t *sink, void *stream);

/*
 * dsa_read_ceiling -- a measurement aid; no step of the method.  Reads the
 * index cache the way the tuned decode indexer streams it (the same share of
 * tokens per block, 32-token tiles per wave, two tiles in flight) and does no
 * arithmetic and no stores, so the bandwidth it reaches bounds the indexer.
 *   k, k_row_stride   device key rows as for dsa_index_scores (row r at byte
 *                     r * k_row_stride; >= 128, a multiple of 4, k 4-byte
 *                     aligned); the first 128 bytes of rows 0 .. n_tokens-1
 *                     are read
 *   k_scale, k_scale_stride  the rows' fp32 scales (k_scale[r * stride])
 *   pattern   0: the indexer's lanes for rows it cannot read as contiguous
 *             tiles (each 16-byte load of a wave touches 32 rows); 1: each
 *             load reads 1 KB of consecutive bytes; 2: as 1 with nontemporal
 *             loads, the indexer's stream for a 16-byte aligned plane of
 *             128-byte rows (1 and 2 need k_row_stride = 128 and k 16-byte
 *             aligned)
 *   blocks    the grid (the indexer streams with 512 blocks on MI355X)
 *   sink      device uint32 [blocks]: block b stores in sink[b] the xor of
 *             every word it read (so the xor of all entries is that of the
 *             first n_tokens key rows and scales)
 * Errors: DSA_ERR_INVALID_ARG for NULL pointers, n_tokens < 1, blocks
 * outside 1 .. 65536, another pattern or a layout the pattern cannot read;
 * DSA_ERR_HIP if the launch fails.  Nothing is allocated.
 */
dsa_status dsa_read_ceiling(const void *k, int64_t k_row_stride, const float *k_scale, int64_t k_scale_stride,
                            int64_t n_tokens, int pattern, int blocks, uint32_t *sink, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *dsa_last_error(void);

/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
