// dsa_api.cpp -- the C ABI of libdsa: host-side argument checks, kernel choice, launch.
//
// Every entry point validates all of its arguments before touching HIP; a failed check
// returns a negative dsa_status with a thread-local message and launches nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "dsa_common.h"
#include "dsa_kernels.h"

// Scratch of the allocation-free entry point (sparse_mla_decode_no_alloc): one file-scope
// device array per GPU, holding the split partials that sparse_mla_decode keeps in a caller
// workspace.  Its size covers every single-layer call with k <= DSA_TOPK_MAX under the
// library's split policy (at most 510 (row, split) partials of 64 x 512 fp32 plus their
// (max, sum) pairs).  Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the address comes from hipGetSymbolAddress, once per device
// with that device current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[DSA_NO_ALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

dsa_status ok()
{
    g_err.clear();
    return DSA_OK;
}

dsa_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int elem_size(int dt)
{
    return dt == DSA_F32 ? 4 : dt == DSA_BF16 ? 2 : dt == DSA_FP8_E4M3FN ? 1 : 0;
}

bool aligned(const void *p, size_t a)
{
    return ((uintptr_t)p % a) == 0;
}

// "generic" forces the generic kernels (A/B checks); anything else picks the tuned ones.
bool force_generic()
{
    const char *v = getenv("DSA_KERNEL_VARIANT");
    return v && strcmp(v, "generic") == 0;
}

dsa_status check_layout(const dsa_layout *L)
{
    if (!L)
        return fail(DSA_ERR_INVALID_ARG, "layout is NULL");
    if (L->batch < 1)
        return fail(DSA_ERR_INVALID_ARG, "layout.batch must be >= 1 (got %d)", L->batch);
    if (L->total_q < 0)
        return fail(DSA_ERR_INVALID_ARG, "layout.total_q must be >= 0 (got %d)", L->total_q);
    if (L->max_ctx < 1)
        return fail(DSA_ERR_INVALID_ARG, "layout.max_ctx must be >= 1 (got %lld)", (long long)L->max_ctx);
    if (!L->kv_indptr)
        return fail(DSA_ERR_INVALID_ARG, "layout.kv_indptr is NULL");
    if (!L->q_indptr && L->total_q != L->batch)
        return fail(DSA_ERR_INVALID_ARG,
                    "layout.q_indptr is NULL (one query per sequence) but total_q %d != batch %d",
                    L->total_q, L->batch);
    if (L->max_ctx > (int64_t)INT32_MAX)
        return fail(DSA_ERR_UNSUPPORTED, "layout.max_ctx %lld exceeds int32 positions",
                    (long long)L->max_ctx);
    if (L->block_table) {
        if (L->page_size < 1)
            return fail(DSA_ERR_INVALID_ARG, "layout.page_size must be >= 1 with a block table");
        if ((int64_t)L->block_table_stride < (L->max_ctx + L->page_size - 1) / L->page_size)
            return fail(DSA_ERR_INVALID_ARG,
                        "layout.block_table_stride %d < pages of max_ctx (%lld tokens, page %d)",
                        L->block_table_stride, (long long)L->max_ctx, L->page_size);
        if (L->cache_rows < 1 || L->cache_rows > (int64_t)INT32_MAX)
            return fail(DSA_ERR_INVALID_ARG, "layout.cache_rows must be in [1, 2^31) with a block table");
        if (!aligned(L->block_table, 4))
            return fail(DSA_ERR_INVALID_ARG, "layout.block_table must be 4-byte aligned");
    }
    return DSA_OK;
}

// Paged caches whose page size the tuned kernels take (power of two, at most 4096).
bool tuned_pages(const dsa_layout *L)
{
    const int p = L->page_size;
    return !L->block_table || (p >= 1 && p <= 4096 && (p & (p - 1)) == 0);
}

dsa::LayoutDev to_dev(const dsa_layout *L)
{
    dsa::LayoutDev d;
    d.kv_indptr = L->kv_indptr;
    d.q_indptr = L->q_indptr;
    d.batch = L->batch;
    d.block_table = L->block_table;
    d.bt_stride = L->block_table ? L->block_table_stride : 0;
    d.page_size = L->block_table ? L->page_size : 1;
    d.cache_rows = L->block_table ? L->cache_rows : 0;
    return d;
}

struct MlaArgs {
    int H, Dc, Dr;
    int q_dt, kv_dt, out_dt;
    int k;
};

dsa_status check_mla_common(const dsa_layout *L, const MlaArgs &a, const int32_t *indices)
{
    dsa_status st = check_layout(L);
    if (st != DSA_OK)
        return st;
    if (a.H < 1 || a.Dc < 1 || a.Dr < 0)
        return fail(DSA_ERR_INVALID_ARG, "bad MLA shape H=%d D_c=%d D_r=%d", a.H, a.Dc, a.Dr);
    if (a.k < 1 || a.k > DSA_TOPK_MAX)
        return fail(DSA_ERR_INVALID_ARG, "k=%d outside [1, %d]", a.k, DSA_TOPK_MAX);
    if (!indices)
        return fail(DSA_ERR_INVALID_ARG, "indices is NULL");
    if (a.q_dt != DSA_F32 && a.q_dt != DSA_BF16)
        return fail(DSA_ERR_UNSUPPORTED, "MLA q dtype %d not supported (F32 or BF16)", a.q_dt);
    if (!elem_size(a.kv_dt))
        return fail(DSA_ERR_UNSUPPORTED, "MLA kv dtype %d not supported", a.kv_dt);
    if (a.out_dt != DSA_F32 && a.out_dt != DSA_BF16)
        return fail(DSA_ERR_UNSUPPORTED, "MLA out dtype %d not supported (F32 or BF16)", a.out_dt);
    return DSA_OK;
}

bool mla_tuned_shape(const MlaArgs &a)
{
    return a.H == 64 && a.Dc == 512 && a.Dr == 64 && a.q_dt == DSA_BF16 &&
           (a.kv_dt == DSA_BF16 || a.kv_dt == DSA_FP8_E4M3FN);
}

dsa_status check_mla_layer(const MlaArgs &a, const dsa_mla_layer &l, int idx, bool tuned)
{
    if (!l.q || !l.kv || !l.out)
        return fail(DSA_ERR_INVALID_ARG, "layer %d: q, kv and out must be non-NULL", idx);
    if (!(l.kv_scale > 0.f) || !std::isfinite(l.kv_scale))
        return fail(DSA_ERR_INVALID_ARG, "layer %d: kv_scale must be finite and > 0", idx);
    if (tuned && (!aligned(l.q, 16) || !aligned(l.kv, 16) || !aligned(l.out, 16)))
        return fail(DSA_ERR_INVALID_ARG, "layer %d: q, kv and out must be 16-byte aligned", idx);
    if (!aligned(l.q, (size_t)elem_size(a.q_dt)) || !aligned(l.kv, (size_t)elem_size(a.kv_dt)) ||
        !aligned(l.out, (size_t)elem_size(a.out_dt)) || (l.lse && !aligned(l.lse, 4)))
        return fail(DSA_ERR_INVALID_ARG, "layer %d: pointer not aligned to its element size", idx);
    return DSA_OK;
}

// The device address of `scratch` (declared above the namespace), kept per device.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch (looked up on the first call per device).
dsa_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(DSA_ERR_UNSUPPORTED, "device %d outside the %d devices the static scratch serves", dev,
                    MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

dsa_status run_mla(const dsa_layout *L, const MlaArgs &a, float sm_scale, int n_layers,
                   const dsa_mla_layer *layers, const int32_t *indices, void *workspace,
                   size_t ws_bytes, void *stream, bool static_scratch = false)
{
    dsa_status st = check_mla_common(L, a, indices);
    if (st != DSA_OK)
        return st;
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
        return fail(DSA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    if (n_layers < 1 || n_layers > DSA_MAX_SHARED_LAYERS)
        return fail(DSA_ERR_INVALID_ARG, "n_layers=%d outside [1, %d]", n_layers, DSA_MAX_SHARED_LAYERS);
    if (!layers)
        return fail(DSA_ERR_INVALID_ARG, "layers is NULL");
    // the tuned kernels address one sequence's rows (or, paged, the whole cache) with unsigned
    // 32-bit buffer offsets, keeping the top 1 MiB for the "no row" offset; larger ranges run
    // the generic kernel
    const int64_t rows_addressed = L->block_table ? L->cache_rows : L->max_ctx;
    const bool fits32 = rows_addressed * (int64_t)(a.Dc + a.Dr) * elem_size(a.kv_dt) <=
                        ((int64_t)1 << 32) - (1 << 20);
    const bool tuned = mla_tuned_shape(a) && !force_generic() && fits32;
    if (!tuned) {
        if (a.H > 128 || a.Dc > 512 || a.Dc + a.Dr > 1024)
            return fail(DSA_ERR_UNSUPPORTED,
                        "MLA shape H=%d D_c=%d D_r=%d exceeds the generic kernel (H<=128, D_c<=512, D_c+D_r<=1024)",
                        a.H, a.Dc, a.Dr);
    }
    for (int l = 0; l < n_layers; ++l) {
        st = check_mla_layer(a, layers[l], l, tuned);
        if (st != DSA_OK)
            return st;
    }
    if (!aligned(indices, 4))
        return fail(DSA_ERR_INVALID_ARG, "indices must be 4-byte aligned");
    const int64_t T = L->total_q;
    size_t need = tuned ? dsa::mla_workspace_bytes(T, n_layers, a.k) : 0;
    if (static_scratch) {
        if (need > DSA_NO_ALLOC_SCRATCH_BYTES)
            return fail(DSA_ERR_WORKSPACE,
                        "this call needs %zu bytes of split partials; the static scratch holds %zu "
                        "(call sparse_mla_decode with a workspace instead)",
                        need, (size_t)DSA_NO_ALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        ws_bytes = DSA_NO_ALLOC_SCRATCH_BYTES;
        if (need > 0 && T > 0) {
            st = scratch_address(&workspace);
            if (st != DSA_OK)
                return st;
        }
    }
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 256))
        return fail(DSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (T == 0)
        return ok();

    dsa::MlaLayersDev ld;
    memset(&ld, 0, sizeof ld);
    for (int l = 0; l < n_layers; ++l) {
        ld.l[l].q = layers[l].q;
        ld.l[l].kv = layers[l].kv;
        ld.l[l].kv_scale = layers[l].kv_scale;
        ld.l[l].out = layers[l].out;
        ld.l[l].lse = layers[l].lse;
    }
    const dsa::LayoutDev dl = to_dev(L);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (tuned)
        e = dsa::launch_mla_tuned(dl, T, ld, n_layers, a.kv_dt == DSA_FP8_E4M3FN, a.out_dt == DSA_F32,
                                  indices, a.k, sm_scale, workspace, s);
    else
        e = dsa::launch_mla_generic(dl, T, a.H, a.Dc, a.Dr, ld, n_layers, a.q_dt, a.kv_dt,
                                    a.out_dt == DSA_F32, indices, a.k, sm_scale, s);
    return hip_status(e, "sparse MLA launch");
}

// Shared checks of the two index-cache writer entry points (rows of H groups of 128 values).
dsa_status check_index_quant(int64_t rows, int H, dsa_dtype x_dt, const void *x, int64_t x_row_bytes,
                             const int64_t *positions, const float *cos_sin, int64_t rope_rows,
                             int rope_off, const void *codes, int64_t code_row_bytes,
                             const float *scales, int64_t scale_row_stride)
{
    if (rows < 0 || H < 1)
        return fail(DSA_ERR_INVALID_ARG, "bad writer shape rows=%lld H=%d", (long long)rows, H);
    if (x_dt != DSA_F32 && x_dt != DSA_BF16)
        return fail(DSA_ERR_UNSUPPORTED, "writer input dtype %d not supported (F32 or BF16)", x_dt);
    if (rows == 0)
        return DSA_OK;  // nothing to read or write: empty tensors may carry NULL pointers
    if (!x || !codes || !scales)
        return fail(DSA_ERR_INVALID_ARG, "input, codes and scales must be non-NULL");
    if (x_row_bytes < (int64_t)H * 128 * elem_size(x_dt) || x_row_bytes % 16 != 0 || !aligned(x, 16))
        return fail(DSA_ERR_INVALID_ARG,
                    "input rows must hold H * 128 values, start 16-byte aligned and have a "
                    "16-byte multiple stride (stride %lld)", (long long)x_row_bytes);
    if (code_row_bytes < (int64_t)H * 128 || code_row_bytes % 4 != 0 || !aligned(codes, 4))
        return fail(DSA_ERR_INVALID_ARG,
                    "code rows must hold H * 128 bytes, start 4-byte aligned and have a 4-byte "
                    "multiple stride (stride %lld)", (long long)code_row_bytes);
    if (scale_row_stride < H || !aligned(scales, 4))
        return fail(DSA_ERR_INVALID_ARG, "scale stride %lld < H or scales not 4-byte aligned",
                    (long long)scale_row_stride);
    if (cos_sin) {
        if (!positions)
            return fail(DSA_ERR_INVALID_ARG, "rope needs positions");
        if (rope_rows < 1 || !aligned(cos_sin, 16))
            return fail(DSA_ERR_INVALID_ARG, "rope table needs >= 1 row and 16-byte alignment");
        if (rope_off != 0 && rope_off != 64)
            return fail(DSA_ERR_INVALID_ARG, "rope_off must be 0 or 64 (got %d)", rope_off);
    }
    if (rows > ((int64_t)1 << 40) || rows * H > 16 * (int64_t)INT32_MAX)
        return fail(DSA_ERR_UNSUPPORTED, "too many groups for one launch (rows %lld x H %d)",
                    (long long)rows, H);
    return DSA_OK;
}

}  // namespace

// Checks of the top-k arguments (dsa_topk and the fused entry).
static dsa_status check_topk(const dsa_layout *layout, const float *scores, int64_t ld, int k,
                             int32_t *indices, void *workspace, size_t workspace_bytes)
{
    dsa_status st = check_layout(layout);
    if (st != DSA_OK)
        return st;
    if (k < 1 || k > DSA_TOPK_MAX)
        return fail(DSA_ERR_INVALID_ARG, "k=%d outside [1, %d]", k, DSA_TOPK_MAX);
    if (!scores || !indices)
        return fail(DSA_ERR_INVALID_ARG, "scores and indices must be non-NULL");
    if (ld < layout->max_ctx)
        return fail(DSA_ERR_INVALID_ARG, "ld %lld < max_ctx %lld", (long long)ld,
                    (long long)layout->max_ctx);
    if (!aligned(scores, 4) || !aligned(indices, 4))
        return fail(DSA_ERR_INVALID_ARG, "scores and indices must be 4-byte aligned");
    const size_t need = dsa::topk_workspace_bytes(layout->total_q, layout->max_ctx);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSA_ERR_WORKSPACE, "top-k workspace of %zu bytes required, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 256))
        return fail(DSA_ERR_WORKSPACE, "top-k workspace must be 256-byte aligned");
    return DSA_OK;
}

// The indexer entry; with hist != nullptr and the tuned decode kernel, the kernel also adds
// every row's score histogram to hist (*hist_used says whether it did).  Every check runs
// before the launch.
static dsa_status index_scores_impl(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt,
                                    const void *q, const float *q_scale, const float *w, dsa_dtype k_dt,
                                    const void *k, int64_t k_row_stride, const float *k_scale,
                                    int64_t k_scale_stride, float *scores, int64_t ld, void *stream,
                                    uint32_t *hist, bool *hist_used)
{
    if (hist_used)
        *hist_used = false;
    dsa_status st = check_layout(layout);
    if (st != DSA_OK)
        return st;
    if (H_I < 1 || D_I < 1)
        return fail(DSA_ERR_INVALID_ARG, "bad indexer shape H_I=%d D_I=%d", H_I, D_I);
    if (!elem_size(q_dt) || !elem_size(k_dt))
        return fail(DSA_ERR_UNSUPPORTED, "indexer dtypes q=%d k=%d not supported", q_dt, k_dt);
    if (!q || !w || !k || !scores)
        return fail(DSA_ERR_INVALID_ARG, "q, w, k and scores must be non-NULL");
    if ((q_dt == DSA_FP8_E4M3FN) != (q_scale != nullptr))
        return fail(DSA_ERR_INVALID_ARG, "q_scale is required for fp8 q and must be NULL otherwise");
    if ((k_dt == DSA_FP8_E4M3FN) && !k_scale)
        return fail(DSA_ERR_INVALID_ARG, "k_scale is required for fp8 keys");
    if (k_row_stride < (int64_t)D_I * elem_size(k_dt))
        return fail(DSA_ERR_INVALID_ARG, "k_row_stride %lld < D_I * element size",
                    (long long)k_row_stride);
    if (k_row_stride % elem_size(k_dt) != 0)
        return fail(DSA_ERR_INVALID_ARG, "k_row_stride must be a multiple of the key element size");
    if (k_scale && k_scale_stride < 1)
        return fail(DSA_ERR_INVALID_ARG, "k_scale_stride must be >= 1");
    if (ld < layout->max_ctx)
        return fail(DSA_ERR_INVALID_ARG, "ld %lld < max_ctx %lld", (long long)ld,
                    (long long)layout->max_ctx);
    if (!aligned(w, 4) || !aligned(scores, 4) || (k_scale && !aligned(k_scale, 4)) ||
        (q_scale && !aligned(q_scale, 4)) || !aligned(q, (size_t)elem_size(q_dt)) ||
        !aligned(k, (size_t)elem_size(k_dt)))
        return fail(DSA_ERR_INVALID_ARG, "pointer not aligned to its element size");

    // key rows 4-byte aligned: key planes, or 132-byte index-cache entries read in place (the
    // kernels' 16-byte key loads need only dword alignment)
    const bool shape32 = H_I == 32 && D_I == 128 && k_dt == DSA_FP8_E4M3FN && aligned(q, 16) &&
                         aligned(k, 4) && (k_row_stride % 4) == 0 && tuned_pages(layout);
    const bool tuned_decode = shape32 && q_dt == DSA_BF16 && !force_generic();
    // the prefill kernel addresses a sequence's keys with 32-bit buffer offsets
    const bool tuned_fp8 = shape32 && q_dt == DSA_FP8_E4M3FN && !force_generic() &&
                           (layout->block_table ? layout->cache_rows : layout->max_ctx) * k_row_stride <
                               (int64_t)INT32_MAX;
    if (!tuned_decode && !tuned_fp8 && (H_I > 64 || D_I > 256))
        return fail(DSA_ERR_UNSUPPORTED,
                    "indexer shape H_I=%d D_I=%d needs the generic kernel (H_I <= 64, D_I <= 256)",
                    H_I, D_I);
    const int64_t T = layout->total_q;
    if (T == 0)
        return ok();
    const dsa::LayoutDev dl = to_dev(layout);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (tuned_decode) {
        e = dsa::launch_index_decode(dl, T, layout->max_ctx, q, w, k, k_row_stride, k_scale,
                                     k_scale_stride, scores, ld, s, hist);
        if (hist_used)
            *hist_used = hist != nullptr;
    }
    else if (tuned_fp8)
        e = dsa::launch_index_fp8(dl, T, layout->max_ctx, q, q_scale, w, k, k_row_stride, k_scale,
                                  k_scale_stride, scores, ld, s);
    else
        e = dsa::launch_index_generic(dl, T, layout->max_ctx, H_I, D_I, q_dt, q, q_scale, w, k_dt, k,
                                      k_row_stride, k_scale, k_scale_stride, scores, ld, s);
    return hip_status(e, "indexer launch");
}

extern "C" {

const char *dsa_last_error(void)
{
    return g_err.c_str();
}

int dsa_abi_version(void)
{
    return DSA_ABI_VERSION;
}

dsa_status dsa_index_scores(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt,
                            const void *q, const float *q_scale, const float *w, dsa_dtype k_dt,
                            const void *k, int64_t k_row_stride, const float *k_scale,
                            int64_t k_scale_stride, float *scores, int64_t ld, void *stream)
{
    return index_scores_impl(layout, H_I, D_I, q_dt, q, q_scale, w, k_dt, k, k_row_stride, k_scale,
                             k_scale_stride, scores, ld, stream, nullptr, nullptr);
}

dsa_status dsa_index_k_cache_write(int64_t n, dsa_dtype k_dt, const void *k, int64_t k_row_stride,
                                   const int64_t *positions, const float *cos_sin,
                                   int64_t rope_rows, int rope_off, const int64_t *slots,
                                   uint8_t *cache, int64_t cache_row_stride, float *cache_scale,
                                   int64_t cache_scale_stride, int64_t cache_rows, void *stream)
{
    dsa_status st = check_index_quant(n, 1, k_dt, k, k_row_stride, positions, cos_sin, rope_rows,
                                      rope_off, cache, cache_row_stride, cache_scale,
                                      cache_scale_stride);
    if (st != DSA_OK)
        return st;
    if (n == 0)
        return ok();
    if (!slots)
        return fail(DSA_ERR_INVALID_ARG, "slots must be non-NULL");
    if (cache_rows < 0)
        return fail(DSA_ERR_INVALID_ARG, "cache_rows must be >= 0");
    hipError_t e = dsa::launch_index_quant(n, 1, k_dt == DSA_F32, k, k_row_stride, positions,
                                           cos_sin, rope_rows, rope_off, slots, cache_rows, cache,
                                           cache_row_stride, cache_scale, cache_scale_stride,
                                           (hipStream_t)stream);
    return hip_status(e, "index-cache writer launch");
}

dsa_status dsa_index_q_quant(int64_t T, int H_I, dsa_dtype q_dt, const void *q, int64_t q_row_stride,
                             const int64_t *positions, const float *cos_sin, int64_t rope_rows,
                             int rope_off, uint8_t *q_fp8, float *q_scale, void *stream)
{
    dsa_status st = check_index_quant(T, H_I, q_dt, q, q_row_stride, positions, cos_sin, rope_rows,
                                      rope_off, q_fp8, (int64_t)H_I * 128, q_scale, H_I);
    if (st != DSA_OK)
        return st;
    if (T == 0)
        return ok();
    hipError_t e = dsa::launch_index_quant(T, H_I, q_dt == DSA_F32, q, q_row_stride, positions,
                                           cos_sin, rope_rows, rope_off, nullptr, T, q_fp8,
                                           (int64_t)H_I * 128, q_scale, H_I, (hipStream_t)stream);
    return hip_status(e, "index-query quantiser launch");
}

dsa_status dsa_index_front_end(int64_t T, int H_I, dsa_dtype dt, const void *q, int64_t q_row_stride,
                               const void *k, int64_t k_row_stride, const int64_t *positions,
                               const float *cos_sin, int64_t rope_rows, int rope_off,
                               const int64_t *slots, uint8_t *cache, int64_t cache_row_stride,
                               float *cache_scale, int64_t cache_scale_stride, int64_t cache_rows,
                               uint8_t *q_fp8, float *q_scale, void *stream)
{
    dsa_status st = check_index_quant(T, H_I, dt, q, q_row_stride, positions, cos_sin, rope_rows,
                                      rope_off, q_fp8, (int64_t)H_I * 128, q_scale, H_I);
    if (st != DSA_OK)
        return st;
    st = check_index_quant(T, 1, dt, k, k_row_stride, positions, cos_sin, rope_rows, rope_off, cache,
                           cache_row_stride, cache_scale, cache_scale_stride);
    if (st != DSA_OK)
        return st;
    if (T == 0)
        return ok();
    if (!slots)
        return fail(DSA_ERR_INVALID_ARG, "slots must be non-NULL");
    if (cache_rows < 0)
        return fail(DSA_ERR_INVALID_ARG, "cache_rows must be >= 0");
    hipError_t e = dsa::launch_index_front(T, H_I, dt == DSA_F32, q, q_row_stride, k, k_row_stride,
                                           positions, cos_sin, rope_rows, rope_off, slots, cache_rows,
                                           cache, cache_row_stride, cache_scale, cache_scale_stride,
                                           q_fp8, q_scale, (hipStream_t)stream);
    return hip_status(e, "index front-end launch");
}

size_t dsa_topk_workspace_size(const dsa_layout *layout, int64_t ld, int k)
{
    (void)ld;
    (void)k;
    if (!layout || layout->total_q < 0)
        return 0;
    return dsa::topk_workspace_bytes(layout->total_q, layout->max_ctx);
}

dsa_status dsa_topk(const dsa_layout *layout, const float *scores, int64_t ld, int k,
                    int32_t *indices, void *workspace, size_t workspace_bytes, void *stream)
{
    dsa_status st = check_topk(layout, scores, ld, k, indices, workspace, workspace_bytes);
    if (st != DSA_OK)
        return st;
    const int64_t T = layout->total_q;
    if (T == 0)
        return ok();
    return hip_status(dsa::launch_topk(to_dev(layout), T, layout->max_ctx, scores, ld, k, indices, workspace,
                                       (hipStream_t)stream),
                      "top-k launch");
}

dsa_status dsa_index_scores_hist(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt, const void *q,
                                 const float *q_scale, const float *w, dsa_dtype k_dt, const void *k,
                                 int64_t k_row_stride, const float *k_scale, int64_t k_scale_stride,
                                 float *scores, int64_t ld, int k_top, void *workspace, size_t workspace_bytes,
                                 int *hist_built, void *stream)
{
    if (!hist_built)
        return fail(DSA_ERR_INVALID_ARG, "hist_built must not be NULL");
    *hist_built = 0;
    // the top-k's checks (indices aside: this call does not write them) come first
    int32_t probe;
    dsa_status st = check_topk(layout, scores, ld, k_top, &probe, workspace, workspace_bytes);
    if (st != DSA_OK)
        return st;
    const int64_t T = layout->total_q;
    uint32_t *hist = T > 0 ? dsa::topk_hist_of(workspace, T, layout->max_ctx) : nullptr;
    bool fused = false;
    st = index_scores_impl(layout, H_I, D_I, q_dt, q, q_scale, w, k_dt, k, k_row_stride, k_scale,
                           k_scale_stride, scores, ld, stream, hist, &fused);
    if (st == DSA_OK)
        *hist_built = fused ? 1 : 0;
    return st;
}

dsa_status dsa_topk_after_hist(const dsa_layout *layout, const float *scores, int64_t ld, int k,
                               int32_t *indices, void *workspace, size_t workspace_bytes, int hist_built,
                               void *stream)
{
    dsa_status st = check_topk(layout, scores, ld, k, indices, workspace, workspace_bytes);
    if (st != DSA_OK)
        return st;
    const int64_t T = layout->total_q;
    if (T == 0)
        return ok();
    return hip_status(dsa::launch_topk(to_dev(layout), T, layout->max_ctx, scores, ld, k, indices, workspace,
                                       (hipStream_t)stream, hist_built != 0),
                      "top-k launch");
}

dsa_status dsa_index_topk(const dsa_layout *layout, int H_I, int D_I, dsa_dtype q_dt, const void *q,
                          const float *q_scale, const float *w, dsa_dtype k_dt, const void *k,
                          int64_t k_row_stride, const float *k_scale, int64_t k_scale_stride,
                          float *scores, int64_t ld, int k_top, int32_t *indices, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    // both calls' checks first: the indexer launch is the first thing that runs
    dsa_status st = check_topk(layout, scores, ld, k_top, indices, workspace, workspace_bytes);
    if (st != DSA_OK)
        return st;
    int built = 0;
    st = dsa_index_scores_hist(layout, H_I, D_I, q_dt, q, q_scale, w, k_dt, k, k_row_stride, k_scale,
                               k_scale_stride, scores, ld, k_top, workspace, workspace_bytes, &built, stream);
    if (st != DSA_OK)
        return st;
    return dsa_topk_after_hist(layout, scores, ld, k_top, indices, workspace, workspace_bytes, built, stream);
}

size_t sparse_mla_workspace_size(const dsa_layout *layout, int H, int D_c, int D_r, int k,
                                 int n_layers)
{
    if (!layout || layout->total_q < 0 || n_layers < 1 || k < 1 || k > DSA_TOPK_MAX)
        return 0;
    if (!(H == 64 && D_c == 512 && D_r == 64))
        return 0;
    return dsa::mla_workspace_bytes((int64_t)layout->total_q, n_layers, k);
}

dsa_status sparse_mla_decode(const dsa_layout *layout, int H, int D_c, int D_r, float sm_scale,
                             dsa_dtype q_dt, const void *q, dsa_dtype kv_dt, const void *kv,
                             float kv_scale, const int32_t *indices, int k, dsa_dtype out_dt,
                             void *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    MlaArgs a{H, D_c, D_r, q_dt, kv_dt, out_dt, k};
    dsa_mla_layer l{q, kv, kv_scale, out, lse};
    return run_mla(layout, a, sm_scale, 1, &l, indices, workspace, workspace_bytes, stream);
}

dsa_status sparse_mla_decode_no_alloc(const dsa_layout *layout, int H, int D_c, int D_r, float sm_scale,
                                      dsa_dtype q_dt, const void *q, dsa_dtype kv_dt, const void *kv,
                                      float kv_scale, const int32_t *indices, int k, dsa_dtype out_dt,
                                      void *out, float *lse, void *stream)
{
    MlaArgs a{H, D_c, D_r, q_dt, kv_dt, out_dt, k};
    dsa_mla_layer l{q, kv, kv_scale, out, lse};
    return run_mla(layout, a, sm_scale, 1, &l, indices, nullptr, 0, stream, true);
}

// The same computation and launch choice as the decode entry (both follow T): one code path.
dsa_status sparse_mla_prefill(const dsa_layout *layout, int H, int D_c, int D_r, float sm_scale,
                              dsa_dtype q_dt, const void *q, dsa_dtype kv_dt, const void *kv,
                              float kv_scale, const int32_t *indices, int k, dsa_dtype out_dt,
                              void *out, float *lse, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    return sparse_mla_decode(layout, H, D_c, D_r, sm_scale, q_dt, q, kv_dt, kv, kv_scale, indices, k, out_dt,
                             out, lse, workspace, workspace_bytes, stream);
}

dsa_status sparse_mla_decode_shared(const dsa_layout *layout, int H, int D_c, int D_r,
                                    float sm_scale, dsa_dtype q_dt, dsa_dtype kv_dt,
                                    dsa_dtype out_dt, int n_layers, const dsa_mla_layer *layers,
                                    const int32_t *indices, int k, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    MlaArgs a{H, D_c, D_r, q_dt, kv_dt, out_dt, k};
    return run_mla(layout, a, sm_scale, n_layers, layers, indices, workspace, workspace_bytes,
                   stream);
}

dsa_status dsa_gather_ceiling(const void *rows, int64_t n_rows, int row_bytes, const int32_t *indices, int64_t T,
                              int k, uint32_t *sink, void *stream)
{
    if (!rows || !indices || !sink)
        return fail(DSA_ERR_INVALID_ARG, "rows, indices and sink must not be NULL");
    if (row_bytes != 576 && row_bytes != 1152)
        return fail(DSA_ERR_INVALID_ARG, "row_bytes must be 576 (fp8 rows) or 1152 (bf16 rows)");
    if (T < 1 || k < 1 || k > DSA_TOPK_MAX || n_rows < 1)
        return fail(DSA_ERR_INVALID_ARG, "need T >= 1, 1 <= k <= %d and n_rows >= 1", DSA_TOPK_MAX);
    if (n_rows > (int64_t)(0xFFFFFFFFu - (1u << 20)) / row_bytes)
        return fail(DSA_ERR_INVALID_ARG, "the row table must stay below 4 GiB - 1 MiB");
    return hip_status(dsa::launch_gather_ceiling(rows, n_rows, row_bytes, indices, T, k, sink, (hipStream_t)stream),
                      "gather ceiling launch");
}

dsa_status dsa_read_ceiling(const void *k, int64_t k_row_stride, const float *k_scale, int64_t k_scale_stride,
                            int64_t n_tokens, int pattern, int blocks, uint32_t *sink, void *stream)
{
    if (!k || !k_scale || !sink)
        return fail(DSA_ERR_INVALID_ARG, "k, k_scale and sink must not be NULL");
    if (n_tokens < 1 || blocks < 1 || blocks > 65536)
        return fail(DSA_ERR_INVALID_ARG, "need n_tokens >= 1 and 1 <= blocks <= 65536");
    if (pattern < 0 || pattern > 2)
        return fail(DSA_ERR_INVALID_ARG,
                    "pattern must be 0 (the indexer's lanes), 1 (1 KB per load) or 2 (1 KB per nontemporal load)");
    if (k_row_stride < 128 || k_row_stride % 4 != 0 || !aligned(k, 4) || !aligned(k_scale, 4) || k_scale_stride < 1)
        return fail(DSA_ERR_INVALID_ARG, "key rows of >= 128 bytes, 4-byte aligned, and a scale stride >= 1");
    if (pattern != 0 && (k_row_stride != 128 || !aligned(k, 16)))
        return fail(DSA_ERR_INVALID_ARG, "patterns 1 and 2 read a 16-byte aligned plane of 128-byte rows");
    return hip_status(dsa::launch_read_ceiling((const uint8_t *)k, k_row_stride, k_scale, k_scale_stride, n_tokens,
                                               pattern, blocks, sink, (hipStream_t)stream),
                      "read ceiling launch");
}

}  // extern "C"
