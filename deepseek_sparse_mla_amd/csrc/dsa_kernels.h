// dsa_kernels.h -- internal launchers of libdsa (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/dsa.h"

namespace dsa {

struct LayoutDev;

struct MlaLayerDev {
    const void *q;
    const void *kv;
    float kv_scale;
    void *out;
    float *lse;
};
struct MlaLayersDev {
    MlaLayerDev l[DSA_MAX_SHARED_LAYERS];
};

// Sparse-MLA split heuristic: enough (query row, split) blocks to give every CU one block.
constexpr int MLA_TARGET_BLOCKS = 256;

// hist: nullptr, or per-row histograms of the top 11 key bits of the scores to add to
// (the top-k workspace's, see topk_hist_of)
hipError_t launch_index_decode(const LayoutDev &L, int64_t T, int64_t max_ctx, const void *q,
                               const float *w, const void *k, int64_t kstride, const float *ks,
                               int64_t ks_stride, float *scores, int64_t ld, hipStream_t stream,
                               uint32_t *hist = nullptr);
hipError_t launch_index_fp8(const LayoutDev &L, int64_t T, int64_t max_ctx, const void *q,
                            const float *qs, const float *w, const void *k, int64_t kstride,
                            const float *ks, int64_t ks_stride, float *scores, int64_t ld,
                            hipStream_t stream);
hipError_t launch_index_generic(const LayoutDev &L, int64_t T, int64_t max_ctx, int H, int D,
                                int q_dt, const void *q, const float *qs, const float *w, int k_dt,
                                const void *k, int64_t kstride, const float *ks, int64_t ks_stride,
                                float *scores, int64_t ld, hipStream_t stream);
size_t topk_workspace_bytes(int64_t T, int64_t max_ctx);
// The per-row score histograms inside a top-k workspace (nullptr when the layout's rows take
// the single-block mode, which needs none).
uint32_t *topk_hist_of(void *workspace, int64_t T, int64_t max_ctx);
// hist_ready: the workspace's histograms already hold every row's scores (built by the
// indexer), so the histogram pass is skipped.
hipError_t launch_topk(const LayoutDev &L, int64_t T, int64_t max_ctx, const float *scores, int64_t ld,
                       int k, int32_t *indices, void *workspace, hipStream_t stream, bool hist_ready = false);

hipError_t launch_index_quant(int64_t rows, int H, bool in_f32, const void *x, int64_t x_row_bytes,
                              const int64_t *positions, const float *cos_sin, int64_t rope_rows,
                              int rope_off, const int64_t *dst_rows, int64_t out_rows,
                              uint8_t *codes, int64_t code_row_bytes, float *scales,
                              int64_t scale_row_stride, hipStream_t stream);

hipError_t launch_index_front(int64_t T, int H, bool in_f32, const void *q, int64_t q_row_bytes,
                              const void *k, int64_t k_row_bytes, const int64_t *positions,
                              const float *cos_sin, int64_t rope_rows, int rope_off,
                              const int64_t *slots, int64_t cache_rows, uint8_t *cache,
                              int64_t cache_row_bytes, float *cache_scale, int64_t cache_scale_stride,
                              uint8_t *q_fp8, float *q_scale, hipStream_t stream);

int mla_num_splits(int64_t T, int k, int min_tiles);
size_t mla_workspace_bytes(int64_t T, int n_layers, int k);
hipError_t launch_mla_tuned(const LayoutDev &L, int64_t T, const MlaLayersDev &layers, int n_layers,
                            bool kv_fp8, bool out_f32, const int32_t *indices, int k,
                            float sm_scale, void *workspace, hipStream_t stream);
hipError_t launch_read_ceiling(const uint8_t *k, int64_t kstride, const float *ks, int64_t ks_stride, int64_t N,
                               int pattern, int blocks, uint32_t *sink, hipStream_t stream);
hipError_t launch_gather_ceiling(const void *rows, int64_t n_rows, int row_bytes, const int32_t *indices, int64_t T,
                                 int k, uint32_t *sink, hipStream_t stream);
hipError_t launch_mla_generic(const LayoutDev &L, int64_t T, int H, int Dc, int Dr,
                              const MlaLayersDev &layers, int n_layers, int q_dt, int kv_dt,
                              bool out_f32, const int32_t *indices, int k, float sm_scale,
                              hipStream_t stream);

}  // namespace dsa
