/*
 * ckv.h -- C ABI of libckv, cluster-granular recallable KV selection for
 * long-context decode on AMD Instinct MI355X (gfx950).
 *
 * Method: the page "ClusterKV: Manipulating LLM KV Cache in Semantic Space
 * for Recallable Compression" (summary of arXiv 2412.03213). Section names
 * are the page's headings, glossed:
 *   [Clustering in semantic space]  核心方法细节 / 语义空间中的聚类
 *   [Cluster-granular selection]    核心方法细节 / 语义聚类粒度的选择
 *   [Selection and indexing]        核心方法细节 / 选择与索引机制 (Fig. 8)
 *   [Long context & KV compression] 背景知识与设计原则 / 长上下文推理与KV缓存压缩
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or keeps them; the caller also provides the
 *     scratch workspace, sized by the matching *_workspace() query.
 *   - A workspace serves one call at a time: calls sharing one must be
 *     ordered on a stream. A zero-byte workspace may be passed as NULL.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is enqueued on it; no call synchronises the host. Calls on one
 *     stream run in order. Calls with distinct workspaces may run
 *     concurrently on different streams.
 *   - Arguments are checked on the host before anything is enqueued. On any
 *     error the call returns a non-zero ckv_status and has written nothing.
 *     A failure to launch returns CKV_ERR_LAUNCH. No C++ exception crosses
 *     this boundary.
 *   - Only head dimension d = 128 is supported, and at most 65535 heads per
 *     call (CKV_ERR_UNSUPPORTED otherwise). Element type: CKV_F32 or
 *     CKV_BF16 for keys, values and queries; centroids are always fp32,
 *     indices int32, the attention output fp32.
 *   - Rows are row-major with d contiguous elements. "Head stride" is the
 *     number of ELEMENTS between row 0 of one head and row 0 of the next.
 *     K, V, q and centroid pointers must be 16-byte aligned and head strides
 *     a multiple of 16 bytes (CKV_ERR_INVALID_ARG otherwise).
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CKV_OK = 0,
    CKV_ERR_INVALID_ARG = 1,  /* a pointer, size, stride or range is invalid */
    CKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d != 128) */
    CKV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    CKV_ERR_LAUNCH = 4        /* the HIP runtime refused a kernel launch */
} ckv_status;

typedef enum { CKV_F32 = 0, CKV_BF16 = 1 } ckv_dtype;

/* Assignment distance of ckv_cluster. The page clusters with the cosine
 * distance and reports L2 and inner-product distance as worse, because the
 * outlier channels of keys make them swing [Clustering in semantic space;
 * recall experiment, Fig. 11b]; the other two exist for that ablation. */
typedef enum { CKV_COSINE = 0, CKV_INNER_PRODUCT = 1, CKV_L2 = 2 } ckv_metric;

/* Static English text for a status code (never NULL). */
const char *ckv_status_string(int status);

/* Version of this ABI (structure layouts and call signatures). */
int ckv_abi_version(void);

/* ------------------------------------------------------------ cluster --
 * Semantic clustering of keys [Clustering in semantic space, Fig. 4]:
 * K-means with the cosine distance D(i,j) = 1 - <k_i,k_j>/(|k_i||k_j|) over
 * window rows n_sink .. L-1 of each head (the first n_sink rows are attention
 * sinks and are not clustered). Initial centroids are the keys at rows
 * n_sink + s*c, s = floor((L - n_sink) / C). Each of `iters` iterations
 * assigns every key to the centroid of largest cosine similarity (ties to
 * the lower id) and replaces every centroid by the mean of the raw keys
 * assigned to it (an empty cluster keeps its centroid). The returned
 * partition is the last iteration's and the centroids are its means.
 * The page's C0 = L/80 and, for decode-time increments, C+ = 4 clusters
 * over the newest m = 320 tokens with n_sink = 0, are the caller's choice.
 *
 * A key's cosine with mu is <k, mu/|mu|> / |k|, and |k| is common to all of
 * its scores, so the assignment takes the largest <k, mu/|mu|>: the key as
 * stored against the unit centroid (mu/|mu| in fp64, rounded to fp32, then
 * to bf16 for CKV_BF16 keys), with fp32 accumulation. Keys are never
 * normalised. Centroid means are accumulated in fp64 and stored as fp32.
 * Scores are fp32, so keys and centroids must keep |k|^2 and the scores
 * within fp32 range (|k| < 1.8e19).
 *
 * desc->metric selects the distance of the assignment (the update is the
 * mean of the raw keys for every metric):
 *   CKV_COSINE        largest cosine similarity, as above;
 *   CKV_INNER_PRODUCT largest <k, mu> on the raw key and the centroid
 *                     rounded to the key's type (bf16 or fp32);
 *   CKV_L2            smallest |k - mu|^2, evaluated as the largest
 *                     <k, mu> - |mu|^2 / 2 on the same operands (|mu|^2 an
 *                     fp64 sum of the rounded centroid's squares, halved
 *                     and stored as fp32).
 *
 * Outputs (per head h, all caller-owned device buffers):
 *   centroids   fp32 [H][c_cap][d]; slots c_base .. c_base+C-1 written.
 *   assign      int32 [H][L]; label of every window row, -1 for sinks.
 *   csr_offsets int32 [H][c_cap+1]; slots c_base .. c_base+C written with
 *               t_base + exclusive prefix sums of the cluster sizes, so
 *               cluster c_base+c owns tokens [off[c_base+c], off[c_base+c+1]).
 *   csr_tokens  int32 [H][t_cap]; slots t_base .. t_base+L-n_sink-1 written
 *               with absolute token ids (token_base + row), sorted by
 *               cluster, ascending inside a cluster.
 * Appending clusters of a later window (c_base > 0, t_base > 0) leaves the
 * earlier slots untouched, so one CSR can index prompt and decode clusters.
 * A bf16 window of at most 1024 clustered rows and 16 clusters (a decode
 * increment) runs as one launch with the same arithmetic and results.
 */
typedef struct {
    int32_t H;              /* independent KV-head problems (batch x KV heads), >= 1 */
    int32_t d;              /* head dimension, must be 128 */
    int64_t L;              /* rows in the clustering window, > n_sink */
    int64_t k_head_stride;  /* elements between heads of K, >= L*d */
    int64_t token_base;     /* absolute token id of window row 0, >= 0 */
    int32_t n_sink;         /* leading rows excluded from clustering, >= 0 */
    int32_t C;              /* clusters, 1 <= C <= min(L - n_sink, 2048) */
    int32_t iters;          /* K-means iterations, >= 1 */
    int32_t dtype;          /* ckv_dtype of K */
    int32_t c_base;         /* first centroid / offset slot written, >= 0 */
    int32_t c_cap;          /* centroid slots per head, >= c_base + C */
    int64_t t_base;         /* first token slot written, >= 0 */
    int64_t t_cap;          /* token slots per head, >= t_base + L - n_sink */
    int32_t metric;         /* ckv_metric of the assignment (0: cosine) */
} ckv_cluster_desc;

/* Bytes of workspace ckv_cluster needs for `desc`, whatever memory K is in
 * (0 if desc is invalid). Its last region holds a copy of the clustered rows
 * of keys in pinned host memory. */
size_t ckv_cluster_workspace(const ckv_cluster_desc *desc);

/* Bytes of workspace ckv_cluster needs for `desc` when K is device memory:
 * ckv_cluster_workspace() without the region for the copy of host keys
 * (H * (L - n_sink) * d * element bytes less, 64 MiB at 8 x 32768 bf16 rows).
 * ckv_cluster over pinned host keys with only this much returns
 * CKV_ERR_WORKSPACE before anything is enqueued. 0 if desc is invalid. */
size_t ckv_cluster_workspace_device(const ckv_cluster_desc *desc);

/* K: window row 0 of head 0, element type desc->dtype, row r of head h at
 * K + (h * k_head_stride + r) * d. Device memory, or pinned host memory (read
 * through its device mapping; its clustered rows are first copied to the last
 * region of the workspace); any other pointer is CKV_ERR_INVALID_ARG.
 * workspace_bytes below ckv_cluster_workspace_device(), or below
 * ckv_cluster_workspace() for host keys, is CKV_ERR_WORKSPACE. */
int ckv_cluster(const ckv_cluster_desc *desc, const void *K, float *centroids,
                int32_t *assign, int32_t *csr_offsets, int32_t *csr_tokens,
                void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------- select --
 * Cluster-granular selection for one decode step [Cluster-granular
 * selection; Selection and indexing, Fig. 8]. For KV head g, with
 * q_g = sum of its G query rows (fp64, in row order):
 *   s_c = q_g . mu_c for c < C, an fp64 inner product with a fixed
 *         association (32 fused-multiply-add chains over 4 consecutive
 *         channels, then a pairwise tree: run r + run r+16, +8, +4, +2, +1);
 *   clusters are ranked by (s_c descending, c ascending);
 *   walking the ranks, whole clusters are admitted until
 *   B_eff = B - n_sink - n_pending tokens are taken; the last admitted
 *   cluster is cut to its first (lowest-position) tokens that still fit.
 * idx[g] = [0 .. n_sink) ++ [pending_begin .. pending_begin + n_pending)
 *          ++ the admitted clusters' tokens, clusters in ascending id,
 *          each cluster's tokens in CSR order (ascending position; the
 *          cut cluster only its first ones),
 * then -1 up to B; n_sel[g] = number of valid entries. The pages fix which
 * tokens are taken, not the order attention sees them in; emitting by
 * cluster id lets the device find the cut cluster by a weighted select
 * instead of a full sort of the C scores, and lets every 64-slot window of
 * the row be written independently.
 * Pending tokens are decode tokens not yet clustered; they are always
 * selected and count toward the budget, like the sinks.
 *
 * Inputs: q [H*G][d] (dtype), centroids fp32 [H][c_cap][d], csr_offsets
 * int32 [H][c_cap+1] and csr_tokens int32 [H][t_cap] as written by
 * ckv_cluster. Offsets are clamped to [0, t_cap] on the device.
 * Outputs: idx int32 [H][B], n_sel int32 [H].
 * Two launches: the scores (32 clusters per workgroup) go to the workspace,
 * then one workgroup per 64 slots of each idx row finds the cut and writes
 * its slots. B is at most 2^20 (CKV_ERR_UNSUPPORTED above).
 */
typedef struct {
    int32_t H;              /* KV heads, >= 1 */
    int32_t G;              /* query heads per KV head, 1..8 */
    int32_t d;              /* must be 128 */
    int32_t C;              /* clusters in use, 1 <= C <= min(c_cap, 2048) */
    int32_t c_cap;          /* centroid slots per head (row stride) */
    int32_t n_sink;         /* always-selected leading tokens, >= 0 */
    int64_t t_cap;          /* token slots per head (row stride) */
    int64_t pending_begin;  /* first pending token id, >= 0 */
    int64_t n_pending;      /* pending token count, >= 0 */
    int32_t B;              /* budget incl. sinks and pending; idx row stride */
    int32_t dtype;          /* ckv_dtype of q */
} ckv_select_desc;

/* Bytes of workspace ckv_select needs: H * C fp64 scores, rounded up to 256
 * bytes (0 if desc is invalid). */
size_t ckv_select_workspace(const ckv_select_desc *desc);

int ckv_select(const ckv_select_desc *desc, const void *q, const float *centroids,
               const int32_t *csr_offsets, const int32_t *csr_tokens,
               int32_t *idx, int32_t *n_sel, void *workspace,
               size_t workspace_bytes, void *stream);

/* -------------------------------------------------------- sparse_attn --
 * Decode attention over the selected rows [Long context & KV compression]:
 * o_h = softmax(q_h K_S^T * scale) V_S, K_S and V_S the rows idx[g][0 ..
 * n_sel[g]) of KV head g = h / G, for every query head h. scale <= 0 means
 * 1/sqrt(d). The G query heads of a KV head share one gather of its rows.
 * Entries outside [0, kv_rows) are skipped (they contribute nothing);
 * n_sel is clamped to [0, B]; a head with nothing selected gets o = 0.
 * CKV_BF16 computes in fp32; CKV_F32 computes scores, softmax and sums in
 * fp64. The output is fp32.
 *
 * Inputs: q [H*G][d] (dtype), K and V (dtype; row r of head g at
 * (g * kv_head_stride + r) * d), idx int32 [H][B], n_sel int32 [H].
 * Output: o fp32 [H*G][d].
 * K and V may be device memory or the device mapping of pinned host memory
 * (ckv_device_view). The call reads the pointer's memory type: for host
 * memory the bf16 gather keeps more row requests in flight over the host
 * link. The result is the same either way.
 */
typedef struct {
    int32_t H;              /* KV heads, >= 1 */
    int32_t G;              /* query heads per KV head, 1..8 */
    int32_t d;              /* must be 128 */
    int32_t B;              /* idx row stride (max selected rows), 1..32768 */
    int64_t kv_head_stride; /* elements between heads of K and V, >= kv_rows*d */
    int64_t kv_rows;        /* valid rows per head, >= 1 */
    float scale;            /* softmax scale; <= 0 means 1/sqrt(d) */
    int32_t dtype;          /* ckv_dtype of q, K and V */
} ckv_attn_desc;

size_t ckv_attn_workspace(const ckv_attn_desc *desc);

int ckv_sparse_attn(const ckv_attn_desc *desc, const void *q, const void *K,
                    const void *V, const int32_t *idx, const int32_t *n_sel,
                    float *o, void *workspace, size_t workspace_bytes,
                    void *stream);

/* --------------------------------------------------------- select_attn --
 * One decode step: ckv_select followed by ckv_sparse_attn on its output
 * [Cluster-granular selection; Selection and indexing, Fig. 8; Long context
 * & KV compression], with one launch and one round trip of idx through
 * memory fewer: the workgroup that writes 64 slots of a head's idx row also
 * runs the attention over those 64 rows. idx, n_sel and o are bitwise the
 * values the two separate calls produce (same device code, same order),
 * for CKV_BF16 and CKV_F32 alike.
 *
 * sdesc and adesc describe the same step: equal H, G, B and dtype
 * (CKV_ERR_INVALID_ARG otherwise); each is also checked as by its own call.
 * Inputs: those of ckv_select, plus K and V as in ckv_sparse_attn (q is read
 * by both steps). Outputs: idx int32 [H][B], n_sel int32 [H], o fp32
 * [H*G][d]. Workspace: ckv_select_attn_workspace() bytes (the selection's
 * scores, then the attention's split partials).
 */
size_t ckv_select_attn_workspace(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc);

int ckv_select_attn(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc, const void *q,
                    const float *centroids, const int32_t *csr_offsets,
                    const int32_t *csr_tokens, const void *K, const void *V, int32_t *idx,
                    int32_t *n_sel, float *o, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------- select_attn_noalloc --
 * ckv_select_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments and results as ckv_select_attn (bitwise: the
 * same kernels), except that the workspace is a static device array of
 * CKV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends. Nothing is allocated or freed by the call.
 *
 * The caller still owns and passes every input and output. A step whose
 * workspace (ckv_select_attn_workspace) exceeds CKV_NOALLOC_SCRATCH_BYTES
 * returns CKV_ERR_WORKSPACE before anything is enqueued. The array of the
 * current device is used, so `stream` must belong to the current device.
 * All calls on one GPU share that array: calls that may overlap on one GPU
 * (on different streams, or from several threads) race and must not be
 * made; calls ordered on one stream are fine. The first call on a device
 * looks the array's address up once (hipGetSymbolAddress); if that fails
 * the call returns CKV_ERR_LAUNCH.
 */
#define CKV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

int ckv_select_attn_noalloc(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc,
                            const void *q, const float *centroids, const int32_t *csr_offsets,
                            const int32_t *csr_tokens, const void *K, const void *V,
                            int32_t *idx, int32_t *n_sel, float *o, void *stream);

/* --------------------------------------------------------------- cache --
 * Cluster-granular GPU cache of selected KV rows, for KV kept in host memory
 * [Caching the KV of selected tokens; system overview, Fig. 5]: the GPU keeps
 * the rows selected in the last R decode steps, and at each step only the
 * selected rows not in that cache are read from host memory.
 *
 * Contents after step s: exactly the rows selected in steps s-R+1 .. s.
 * Layout of a head's rows (a function of the ring below): slots
 * 0 .. n_sink-1 hold sink tokens 0 .. n_sink-1; then the clusters in
 * ascending id, cluster c holding the first N_c tokens of its CSR segment,
 * N_c = the largest number of c's rows any of those steps selected (a
 * selection takes a prefix of every admitted cluster).
 *
 * State (caller-owned device memory, kept between steps):
 *   ring      int32 [H][c_cap][R]: rows of every cluster selected in each of
 *             the last R steps (slot s % R); zero it before step 0.
 *   cache_K, cache_V  dtype [2][H][rows][d], rows = ckv_cache_rows(desc) =
 *             n_sink + R * (B - n_sink): step s writes buffer s & 1 from
 *             buffer (s - 1) & 1 and from K_src / V_src.
 *   cache_tok int32 [2][H][rows]: token id of every slot of either buffer
 *             (-1 for unused slots).
 * Steps must be numbered 0, 1, 2, ... for one sequence (step 0 loads the
 * sinks); R and the layout inputs stay fixed across its steps.
 *
 * Inputs of a step: this step's ckv_select output idx [H][B], n_sel [H];
 * the labels assign [H][L] of ckv_cluster (token id t is row t - token_base)
 * and the CSR csr_offsets [H][c_cap+1], csr_tokens [H][t_cap] the selection
 * used; K_src, V_src: every head's K and V, row t of head h at
 * (h * kv_head_stride + t * d), either device memory or pinned host memory
 * (hipHostMalloc; read through its device mapping). Any other pointer is
 * CKV_ERR_INVALID_ARG.
 *
 * Outputs: idx_cache int32 [H][B]: the slot of every selected entry in
 * buffer step & 1 (-1 past n_sel, and for entries that are neither a sink
 * nor a clustered row, such as pending decode rows, which the cache does not
 * hold); stats int32 [H][5]: cluster rows found in the cache, cluster rows
 * read from K_src/V_src, selected clusters found whole in the cache,
 * selected clusters, selected entries without a slot. ckv_sparse_attn with
 * K, V = buffer step & 1 (kv_head_stride rows * d, kv_rows = rows) and idx =
 * idx_cache leaves out every entry without a slot (-1). When a head has none
 * (stats[h][4] == 0, always the case for a selection without pending rows,
 * n_pending == 0), that attention is bitwise equal to the one over
 * K_src/V_src with idx (same rows, same order); with pending rows it is not,
 * and the caller must attend those rows from where they live.
 *
 * Workspace: ckv_cache_workspace() bytes. Two launches on `stream`.
 */
typedef struct {
    int32_t H;              /* KV heads, >= 1 */
    int32_t d;              /* must be 128 */
    int32_t C;              /* clusters in use, 1 <= C <= min(c_cap, 2048) */
    int32_t c_cap;          /* cluster slots per head (CSR and ring stride) */
    int32_t n_sink;         /* sink tokens, 0 <= n_sink <= B */
    int32_t B;              /* selection budget (idx row stride), <= 4096 */
    int32_t R;              /* steps a selected row stays cached, 1 .. 8 */
    int32_t dtype;          /* ckv_dtype of K_src, V_src and the cache */
    int64_t L;              /* rows of assign per head */
    int64_t token_base;     /* token id of assign row 0, >= 0 */
    int64_t t_cap;          /* CSR token slots per head */
    int64_t kv_head_stride; /* elements between heads of K_src / V_src */
    int64_t kv_rows;        /* rows per head of K_src / V_src */
} ckv_cache_desc;

/* Cache rows per head and buffer, n_sink + R * (B - n_sink) (0 if invalid). */
int64_t ckv_cache_rows(const ckv_cache_desc *desc);

/* Bytes of workspace ckv_cache_step needs (0 if desc is invalid). */
size_t ckv_cache_workspace(const ckv_cache_desc *desc);

int ckv_cache_step(const ckv_cache_desc *desc, int64_t step, const int32_t *idx,
                   const int32_t *n_sel, const int32_t *assign, const int32_t *csr_offsets,
                   const int32_t *csr_tokens, const void *K_src, const void *V_src,
                   int32_t *ring, void *cache_K, void *cache_V, int32_t *cache_tok,
                   int32_t *idx_cache, int32_t *stats, void *workspace, size_t workspace_bytes,
                   void *stream);

/* The address at which the library's kernels read `ptr`: itself for device
 * memory, the device mapping for pinned host memory (hipHostMalloc); any
 * other pointer is CKV_ERR_INVALID_ARG. Lets a caller hand host-resident K/V
 * to ckv_sparse_attn directly (every selected row read over the host link,
 * the no-cache baseline of the cache). */
int ckv_device_view(const void *ptr, const void **device_ptr);

#ifdef __cplusplus
}
#endif
#endif /* CKV_H */
