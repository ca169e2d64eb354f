// api.hip -- the C ABI of libckv (declared in include/ckv.h).
//
// Every entry point validates its descriptor and pointers on the host,
// carves the caller's workspace, and enqueues kernels on the caller's
// stream. Nothing is allocated, nothing is synchronised, no state is kept.
#include <math.h>
#include <string.h>

#include <atomic>

#include "ckv.h"
#include "cache_dev.h"
#include "ckv_dev.h"
#include "cluster_dev.h"

using namespace ckv;

namespace ckv {
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}
}  // namespace ckv

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(int32_t t) { return t == CKV_F32 || t == CKV_BF16; }

// heads beyond this do not fit the second grid dimension of some launches
constexpr int32_t kMaxHeads = 65535;

// Returns CKV_OK or the reason the cluster descriptor is rejected.
int check_cluster(const ckv_cluster_desc *d) {
    if (!d) return CKV_ERR_INVALID_ARG;
    if (d->H < 1 || !dtype_ok(d->dtype)) return CKV_ERR_INVALID_ARG;
    if (d->d != kD) return d->d < 1 ? CKV_ERR_INVALID_ARG : CKV_ERR_UNSUPPORTED;
    if (d->H > kMaxHeads) return CKV_ERR_UNSUPPORTED;
    if (d->n_sink < 0 || d->L <= d->n_sink) return CKV_ERR_INVALID_ARG;
    const int64_t Lp = d->L - d->n_sink;
    if (d->C < 1 || d->C > Lp || d->iters < 1) return CKV_ERR_INVALID_ARG;
    if (d->C > kMaxC) return CKV_ERR_UNSUPPORTED;
    if (d->k_head_stride < d->L * kD) return CKV_ERR_INVALID_ARG;
    if (d->token_base < 0 || d->token_base + d->L > INT32_MAX) return CKV_ERR_INVALID_ARG;
    if (d->c_base < 0 || (int64_t)d->c_cap < (int64_t)d->c_base + d->C) return CKV_ERR_INVALID_ARG;
    if (d->t_base < 0 || d->t_cap < d->t_base + Lp || d->t_cap > INT32_MAX)
        return CKV_ERR_INVALID_ARG;
    if (d->metric != CKV_COSINE && d->metric != CKV_INNER_PRODUCT && d->metric != CKV_L2)
        return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

// Workspace carve-up. *bytes: the whole workspace; *bytes_dev (if given): its
// prefix without the copy of pinned host keys, all that device keys need.
void plan_cluster(const ckv_cluster_desc *d, ClusterPlan *p, size_t *bytes, char *ws,
                  size_t *bytes_dev = nullptr) {
    p->H = d->H;
    p->C = d->C;
    p->Cpad = (d->C + 63) / 64 * 64;
    p->iters = d->iters;
    p->n_sink = d->n_sink;
    p->dtype = d->dtype;
    p->metric = d->metric;
    p->c_base = d->c_base;
    p->c_cap = d->c_cap;
    p->L = d->L;
    p->Lp = d->L - d->n_sink;
    p->k_head_stride = d->k_head_stride;
    p->token_base = d->token_base;
    p->t_base = d->t_base;
    p->t_cap = d->t_cap;
    p->ka = p->ku = nullptr;  // set by ckv_cluster once K is resolved
    p->ka_stride = p->ku_stride = p->ku_rows = p->ku_base = 0;
    p->csr_wide = d->C <= kCsrWideMaxC;
    const int tile = kCsrWideTile;
    p->ntiles = (p->Lp + tile - 1) / tile;
    const size_t es = d->dtype == CKV_BF16 ? 2 : 4;
    size_t o = 0;
    p->mt = ws ? ws + o : nullptr;
    o += align_up((size_t)p->H * p->Cpad * kD * es);
    p->mb = ws ? (float *)(ws + o) : nullptr;
    o += align_up((size_t)p->H * p->Cpad * sizeof(float));
    p->tile_hist = ws ? (int32_t *)(ws + o) : nullptr;
    o += align_up((size_t)p->H * p->ntiles * p->C * sizeof(int32_t));
    p->tile_rank = ws ? (int32_t *)(ws + o) : nullptr;
    o += align_up((size_t)p->H * p->Lp * sizeof(int32_t));
    p->counts = ws ? (int32_t *)(ws + o) : nullptr;
    o += align_up((size_t)p->H * p->C * sizeof(int32_t));
    if (bytes_dev) *bytes_dev = o;
    p->kt = ws ? ws + o : nullptr;            // last: only keys in host memory use it
    o += align_up((size_t)p->H * p->Lp * kD * es);
    *bytes = o;
}

int check_select(const ckv_select_desc *d) {
    if (!d) return CKV_ERR_INVALID_ARG;
    if (d->H < 1 || d->G < 1 || d->G > 8 || !dtype_ok(d->dtype)) return CKV_ERR_INVALID_ARG;
    if (d->d != kD) return d->d < 1 ? CKV_ERR_INVALID_ARG : CKV_ERR_UNSUPPORTED;
    if (d->H > kMaxHeads) return CKV_ERR_UNSUPPORTED;
    if (d->C < 1 || d->c_cap < d->C) return CKV_ERR_INVALID_ARG;
    if (d->C > kMaxC) return CKV_ERR_UNSUPPORTED;
    if (d->n_sink < 0 || d->n_pending < 0 || d->pending_begin < 0) return CKV_ERR_INVALID_ARG;
    if (d->pending_begin + d->n_pending > INT32_MAX) return CKV_ERR_INVALID_ARG;
    if (d->B < 1 || (int64_t)d->B < d->n_sink + d->n_pending) return CKV_ERR_INVALID_ARG;
    if (d->B > kMaxSelB) return CKV_ERR_UNSUPPORTED;
    if (d->t_cap < 1 || d->t_cap > INT32_MAX) return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

// the fp64 scores [H][C] pass from the scoring kernel to the cut kernel
size_t select_bytes(const ckv_select_desc *d) {
    return align_up((size_t)d->H * d->C * sizeof(double));
}

int check_attn(const ckv_attn_desc *d) {
    if (!d) return CKV_ERR_INVALID_ARG;
    if (d->H < 1 || d->G < 1 || d->G > 8 || !dtype_ok(d->dtype)) return CKV_ERR_INVALID_ARG;
    if (d->d != kD) return d->d < 1 ? CKV_ERR_INVALID_ARG : CKV_ERR_UNSUPPORTED;
    if (d->B < 1 || d->kv_rows < 1) return CKV_ERR_INVALID_ARG;
    if (d->H > kMaxHeads) return CKV_ERR_UNSUPPORTED;
    if (d->B > kMaxSplits * kAttnSplitRows) return CKV_ERR_UNSUPPORTED;
    if (d->kv_head_stride < d->kv_rows * kD) return CKV_ERR_INVALID_ARG;
    if (!(d->scale == d->scale) || isinf(d->scale)) return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

int attn_splits(const ckv_attn_desc *d) { return (d->B + kAttnSplitRows - 1) / kAttnSplitRows; }

// workspace: split partials [H*G][S][2+d]
size_t attn_bytes(const ckv_attn_desc *d) {
    const size_t es = d->dtype == CKV_BF16 ? sizeof(float) : sizeof(double);
    return align_up((size_t)d->H * d->G * attn_splits(d) * (kD + 2) * es);
}

int launch_status(hipError_t e) { return e == hipSuccess ? CKV_OK : CKV_ERR_LAUNCH; }

void plan_select(const ckv_select_desc *d, SelectPlan *p, void *scores) {
    p->H = d->H;
    p->G = d->G;
    p->C = d->C;
    p->c_cap = d->c_cap;
    p->n_sink = d->n_sink;
    p->B = d->B;
    p->dtype = d->dtype;
    p->t_cap = d->t_cap;
    p->pending_begin = d->pending_begin;
    p->n_pending = d->n_pending;
    p->scores = (double *)scores;
}

void plan_attn(const ckv_attn_desc *d, AttnPlan *p, void *partials) {
    p->H = d->H;
    p->G = d->G;
    p->B = d->B;
    p->dtype = d->dtype;
    p->S = attn_splits(d);
    p->kv_head_stride = d->kv_head_stride;
    p->kv_rows = d->kv_rows;
    p->scale = d->scale > 0.f ? (double)d->scale : 1.0 / sqrt((double)kD);
    p->partials = partials;
    p->host_kv = false;
}


// the two descriptors of one decode step describe the same problem
int check_select_attn(const ckv_select_desc *s, const ckv_attn_desc *a) {
    int st = check_select(s);
    if (st != CKV_OK) return st;
    st = check_attn(a);
    if (st != CKV_OK) return st;
    if (s->H != a->H || s->G != a->G || s->B != a->B || s->dtype != a->dtype)
        return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

// Kernels read rows with 16-byte vector loads.
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool stride_ok(int64_t elems, int32_t dtype) {
    return ((elems * (dtype == CKV_BF16 ? 2 : 4)) & 15) == 0;
}

int check_cache(const ckv_cache_desc *d) {
    if (!d) return CKV_ERR_INVALID_ARG;
    if (d->H < 1 || !dtype_ok(d->dtype)) return CKV_ERR_INVALID_ARG;
    if (d->d != kD) return d->d < 1 ? CKV_ERR_INVALID_ARG : CKV_ERR_UNSUPPORTED;
    if (d->H > kMaxHeads) return CKV_ERR_UNSUPPORTED;
    if (d->C < 1 || d->c_cap < d->C) return CKV_ERR_INVALID_ARG;
    if (d->C > kMaxC) return CKV_ERR_UNSUPPORTED;
    if (d->n_sink < 0 || d->B < 1 || d->B < d->n_sink) return CKV_ERR_INVALID_ARG;
    if (d->R < 1) return CKV_ERR_INVALID_ARG;
    if (d->R > kMaxCacheR || d->B > kMaxCacheB) return CKV_ERR_UNSUPPORTED;
    if (d->L < 1 || d->token_base < 0 || d->t_cap < 1 || d->t_cap > INT32_MAX)
        return CKV_ERR_INVALID_ARG;
    if (d->kv_rows < 1 || d->kv_rows > INT32_MAX || d->kv_head_stride < d->kv_rows * kD)
        return CKV_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)d->n_sink + (int64_t)d->R * (d->B - d->n_sink);
    if (rows < 1 || rows > INT32_MAX / 2) return CKV_ERR_UNSUPPORTED;
    return CKV_OK;
}

int64_t cache_rows(const ckv_cache_desc *d) {
    return (int64_t)d->n_sink + (int64_t)d->R * (d->B - d->n_sink);
}

size_t cache_bytes(const ckv_cache_desc *d) {
    return align_up((size_t)d->H * cache_rows(d) * sizeof(int32_t)) +
           align_up((size_t)d->H * sizeof(int32_t));
}

void plan_cache(const ckv_cache_desc *d, CachePlan *p, void *ws) {
    p->H = d->H;
    p->C = d->C;
    p->c_cap = d->c_cap;
    p->n_sink = d->n_sink;
    p->B = d->B;
    p->R = d->R;
    p->dtype = d->dtype;
    p->rows = (int)cache_rows(d);
    p->L = d->L;
    p->token_base = d->token_base;
    p->t_cap = d->t_cap;
    p->kv_head_stride = d->kv_head_stride;
    p->kv_rows = d->kv_rows;
    p->src = (int32_t *)ws;
    p->tot = (int32_t *)((char *)ws + align_up((size_t)d->H * p->rows * sizeof(int32_t)));
}

// The address at which a kernel reads `p`: device memory as is, pinned host
// memory (hipHostMalloc) through its device mapping. Anything else (pageable
// host memory, unknown pointers) is refused, so no kernel is handed an
// address it cannot read. *host (if given) tells which of the two it is.
int device_view(const void *p, const void **out, bool *host = nullptr) {
    if (!p) return CKV_ERR_INVALID_ARG;
    if (host) *host = false;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return CKV_ERR_INVALID_ARG;
    }
    if (a.type == hipMemoryTypeDevice) {
        *out = p;
        return CKV_OK;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        if (host) *host = true;
        const char *hb = (const char *)a.hostPointer;
        const char *db = (const char *)a.devicePointer;
        *out = (hb && (const char *)p >= hb) ? db + ((const char *)p - hb) : db;
        return CKV_OK;
    }
    return CKV_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

const char *ckv_status_string(int status) {
    switch (status) {
        case CKV_OK: return "ok";
        case CKV_ERR_INVALID_ARG: return "invalid argument";
        case CKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case CKV_ERR_WORKSPACE: return "workspace missing or too small";
        case CKV_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int ckv_abi_version(void) { return 4; }

size_t ckv_cluster_workspace(const ckv_cluster_desc *desc) {
    if (check_cluster(desc) != CKV_OK) return 0;
    ClusterPlan p;
    size_t bytes;
    plan_cluster(desc, &p, &bytes, nullptr);
    return bytes;
}

size_t ckv_cluster_workspace_device(const ckv_cluster_desc *desc) {
    if (check_cluster(desc) != CKV_OK) return 0;
    ClusterPlan p;
    size_t bytes, dev;
    plan_cluster(desc, &p, &bytes, nullptr, &dev);
    return dev;
}

int ckv_cluster(const ckv_cluster_desc *desc, const void *K, float *centroids,
                int32_t *assign, int32_t *csr_offsets, int32_t *csr_tokens, void *workspace,
                size_t workspace_bytes, void *stream) {
    const int st = check_cluster(desc);
    if (st != CKV_OK) return st;
    if (!K || !centroids || !assign || !csr_offsets || !csr_tokens) return CKV_ERR_INVALID_ARG;
    if (!aligned16(K) || !aligned16(centroids) || !stride_ok(desc->k_head_stride, desc->dtype))
        return CKV_ERR_INVALID_ARG;
    ClusterPlan p;
    size_t need, need_dev;
    plan_cluster(desc, &p, &need, (char *)workspace, &need_dev);
    if (!workspace || workspace_bytes < need_dev) return CKV_ERR_WORKSPACE;
    // K as the kernels read it: device memory, or pinned host memory through
    // its device mapping; pageable host memory and unknown pointers are refused
    const void *Kv;
    bool k_host = false;
    if (device_view(K, &Kv, &k_host) != CKV_OK || !aligned16(Kv)) return CKV_ERR_INVALID_ARG;
    if (k_host && workspace_bytes < need) return CKV_ERR_WORKSPACE;   // room for the copy
    K = Kv;
    p.n_cu = device_cu_count();
    hipStream_t s = (hipStream_t)stream;
    // the assignment and the update read device keys where they are; host
    // keys are copied to the workspace once, so the iterations do not cross
    // the host link
    const size_t es = p.dtype == CKV_BF16 ? 2 : 4;
    hipError_t e = hipSuccess;
    if (k_host) {
        p.ka = p.kt;
        p.ka_stride = p.Lp * kD;
        p.ku = p.kt;                          // row t - token_base - n_sink
        p.ku_stride = p.Lp * kD;
        p.ku_rows = p.Lp;
        p.ku_base = p.token_base + p.n_sink;
        e = launch_copy_keys(p, K, s);
        if (e != hipSuccess) return launch_status(e);
    } else {
        p.ka = (const char *)K + (size_t)p.n_sink * kD * es;
        p.ka_stride = p.k_head_stride;
        p.ku = K;
        p.ku_stride = p.k_head_stride;
        p.ku_rows = p.L;
        p.ku_base = p.token_base;
    }

    if (p.dtype == CKV_BF16 && p.Lp <= kSmallRows && p.C <= kSmallC)
        return launch_status(launch_cluster_small(p, K, centroids, assign, csr_offsets,
                                                  csr_tokens, s));
    e = launch_init_centroids(p, K, centroids, assign, s);
    for (int t = 0; t < p.iters && e == hipSuccess; ++t) {
        e = launch_assign(p, assign, s);
        if (e == hipSuccess) e = launch_csr(p, assign, csr_offsets, csr_tokens, s);
        if (e == hipSuccess) e = launch_update(p, csr_offsets, csr_tokens, centroids, s);
    }
    return launch_status(e);
}

size_t ckv_select_workspace(const ckv_select_desc *desc) {
    if (check_select(desc) != CKV_OK) return 0;
    return select_bytes(desc);
}

int ckv_select(const ckv_select_desc *desc, const void *q, const float *centroids,
               const int32_t *csr_offsets, const int32_t *csr_tokens, int32_t *idx,
               int32_t *n_sel, void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_select(desc);
    if (st != CKV_OK) return st;
    if (!q || !centroids || !csr_offsets || !csr_tokens || !idx || !n_sel)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(centroids)) return CKV_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < select_bytes(desc)) return CKV_ERR_WORKSPACE;
    SelectPlan p;
    plan_select(desc, &p, workspace);
    return launch_status(launch_select(p, q, centroids, csr_offsets, csr_tokens, idx, n_sel,
                                       (hipStream_t)stream));
}

size_t ckv_attn_workspace(const ckv_attn_desc *desc) {
    if (check_attn(desc) != CKV_OK) return 0;
    return attn_bytes(desc);
}

int ckv_sparse_attn(const ckv_attn_desc *desc, const void *q, const void *K, const void *V,
                    const int32_t *idx, const int32_t *n_sel, float *o, void *workspace,
                    size_t workspace_bytes, void *stream) {
    const int st = check_attn(desc);
    if (st != CKV_OK) return st;
    if (!q || !K || !V || !idx || !n_sel || !o) return CKV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) ||
        !stride_ok(desc->kv_head_stride, desc->dtype))
        return CKV_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < attn_bytes(desc)) return CKV_ERR_WORKSPACE;
    // K and V as the kernels read them (pinned host memory through its device
    // mapping; pageable host memory and unknown pointers are refused)
    const void *Kd, *Vd;
    bool hk, hv;
    if (device_view(K, &Kd, &hk) != CKV_OK || device_view(V, &Vd, &hv) != CKV_OK)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(Kd) || !aligned16(Vd)) return CKV_ERR_INVALID_ARG;
    AttnPlan p;
    plan_attn(desc, &p, workspace);
    p.host_kv = hk || hv;
    return launch_status(launch_attn(p, q, Kd, Vd, idx, n_sel, o, (hipStream_t)stream));
}

namespace {
// Workspace of ckv_select_attn_noalloc: one copy per device, for the life of
// the process. Its name is a host-side stand-in in host code; kernels get
// the device address found by hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[CKV_NOALLOC_SCRATCH_BYTES];

// scratch's device address on the current device (looked up once per
// device, with that device current), or nullptr if the lookup fails
void *scratch_ptr() {
    static std::atomic<void *> ptr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    if (dev < 64) {
        void *p = ptr[dev].load(std::memory_order_acquire);
        if (p) return p;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    if (dev < 64) ptr[dev].store(p, std::memory_order_release);
    return p;
}
}  // namespace

size_t ckv_select_attn_workspace(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc) {
    if (check_select_attn(sdesc, adesc) != CKV_OK) return 0;
    return select_bytes(sdesc) + attn_bytes(adesc);
}

int ckv_select_attn(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc, const void *q,
                    const float *centroids, const int32_t *csr_offsets,
                    const int32_t *csr_tokens, const void *K, const void *V, int32_t *idx,
                    int32_t *n_sel, float *o, void *workspace, size_t workspace_bytes,
                    void *stream) {
    const int st = check_select_attn(sdesc, adesc);
    if (st != CKV_OK) return st;
    if (!q || !centroids || !csr_offsets || !csr_tokens || !K || !V || !idx || !n_sel || !o)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(centroids) || !aligned16(q) || !aligned16(K) || !aligned16(V) ||
        !stride_ok(adesc->kv_head_stride, adesc->dtype))
        return CKV_ERR_INVALID_ARG;
    const size_t sb = select_bytes(sdesc);
    if (!workspace || workspace_bytes < sb + attn_bytes(adesc)) return CKV_ERR_WORKSPACE;
    const void *Kd, *Vd;
    bool hk, hv;
    if (device_view(K, &Kd, &hk) != CKV_OK || device_view(V, &Vd, &hv) != CKV_OK)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(Kd) || !aligned16(Vd)) return CKV_ERR_INVALID_ARG;
    SelectPlan sp;
    plan_select(sdesc, &sp, workspace);
    AttnPlan ap;
    plan_attn(adesc, &ap, (char *)workspace + sb);
    ap.host_kv = hk || hv;
    return launch_status(launch_select_attn(sp, ap, q, centroids, csr_offsets, csr_tokens, Kd,
                                            Vd, idx, n_sel, o, (hipStream_t)stream));
}

int ckv_select_attn_noalloc(const ckv_select_desc *sdesc, const ckv_attn_desc *adesc,
                            const void *q, const float *centroids, const int32_t *csr_offsets,
                            const int32_t *csr_tokens, const void *K, const void *V,
                            int32_t *idx, int32_t *n_sel, float *o, void *stream) {
    const int st = check_select_attn(sdesc, adesc);
    if (st != CKV_OK) return st;
    const size_t need = select_bytes(sdesc) + attn_bytes(adesc);
    if (need > CKV_NOALLOC_SCRATCH_BYTES) return CKV_ERR_WORKSPACE;
    if (!q || !centroids || !csr_offsets || !csr_tokens || !K || !V || !idx || !n_sel || !o)
        return CKV_ERR_INVALID_ARG;
    void *ws = scratch_ptr();
    if (!ws) return CKV_ERR_LAUNCH;
    return ckv_select_attn(sdesc, adesc, q, centroids, csr_offsets, csr_tokens, K, V, idx, n_sel,
                           o, ws, CKV_NOALLOC_SCRATCH_BYTES, stream);
}

int ckv_device_view(const void *ptr, const void **device_ptr) {
    if (!device_ptr) return CKV_ERR_INVALID_ARG;
    return device_view(ptr, device_ptr);
}

int64_t ckv_cache_rows(const ckv_cache_desc *desc) {
    return check_cache(desc) == CKV_OK ? cache_rows(desc) : 0;
}

size_t ckv_cache_workspace(const ckv_cache_desc *desc) {
    return check_cache(desc) == CKV_OK ? cache_bytes(desc) : 0;
}

int ckv_cache_step(const ckv_cache_desc *desc, int64_t step, const int32_t *idx,
                   const int32_t *n_sel, const int32_t *assign, const int32_t *csr_offsets,
                   const int32_t *csr_tokens, const void *K_src, const void *V_src,
                   int32_t *ring, void *cache_K, void *cache_V, int32_t *cache_tok,
                   int32_t *idx_cache, int32_t *stats, void *workspace, size_t workspace_bytes,
                   void *stream) {
    const int st = check_cache(desc);
    if (st != CKV_OK) return st;
    if (step < 0) return CKV_ERR_INVALID_ARG;
    if (!idx || !n_sel || !assign || !csr_offsets || !csr_tokens || !ring || !cache_K ||
        !cache_V || !cache_tok || !idx_cache || !stats)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(cache_K) || !aligned16(cache_V) ||
        !stride_ok(desc->kv_head_stride, desc->dtype))
        return CKV_ERR_INVALID_ARG;
    const void *Kd = nullptr, *Vd = nullptr;
    if (device_view(K_src, &Kd) != CKV_OK || device_view(V_src, &Vd) != CKV_OK)
        return CKV_ERR_INVALID_ARG;
    if (!aligned16(Kd) || !aligned16(Vd)) return CKV_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < cache_bytes(desc)) return CKV_ERR_WORKSPACE;
    CachePlan p;
    plan_cache(desc, &p, workspace);
    return launch_status(launch_cache_step(p, step, idx, n_sel, assign, csr_offsets, csr_tokens,
                                           Kd, Vd, ring, cache_K, cache_V, cache_tok, idx_cache,
                                           stats, (hipStream_t)stream));
}

}  // extern "C"
