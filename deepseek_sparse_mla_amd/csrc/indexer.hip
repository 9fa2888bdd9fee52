// indexer.hip -- lightning-indexer score kernels for gfx950.
//
// score[i, s] = sum_h w[i,h] * ReLU(q[i,h,:] . k[s,:] * qs[i,h] * ks[s])
// ("GLM-5.2 架构解剖", full structure diagram, Indexer box: 32 index heads x 128 dims
// with one key per token shared by all heads; fp8 keys with a per-token scale in a
// 132-byte index-cache entry).  Scales are positive, so ReLU(x * qs * ks) =
// qs * ks * ReLU(x): qs folds into the head weight and ks multiplies the head sum.
//
// Three kernels:
//  * idx_decode_kernel   bf16 q x fp8 k (H=32, D=128).  HBM stream of the index cache:
//    each lane loads 64 contiguous key bytes, widens them exactly to bf16 and feeds
//    v_mfma_f32_32x32x16_bf16 with the 32 heads as M and 32 tokens as N.
//  * idx_fp8_kernel      fp8 q x fp8 k (H=32, D=128): the prefill GEMM on
//    v_mfma_scale_f32_32x32x64_f8f6f4; 16 query rows per block share an LDS key tile.
//  * idx_generic_kernel  any dtypes / H <= 64 / D <= 256, one thread per token.
#include <cstdlib>

#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

// ReLU in one instruction (v_med3_f32); MFMA results are never NaN here.
__device__ __forceinline__ float relu(float x)
{
    return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f);
}

// ------------------------------------------------------------------------------------------
// bf16 q x fp8 k, H = 32, D = 128
//
// MFMA 32x32x16 bf16: lane l supplies A[row l%32][k-group l/32] and B[k-group l/32][col
// l%32]; D[row][col] lands in lane col + 32*((row/4)%2), register 4*(row/8) + row%4.
// Rows are heads, columns tokens.  The 128-long contraction is split so that lane half g
// owns dims [64g, 64g+64): MFMA t consumes dims 64g + 8t .. 64g + 8t + 7 of both q and k.
// ------------------------------------------------------------------------------------------
// 16 key bytes of a lane: rows need only be 4-byte aligned (a 132-byte index-cache entry puts
// the 128 code bytes of token r at byte 132 r); the loads are still single 16-byte loads.
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// Contiguous tiles (unpaged 128-byte rows, 16-byte aligned): a wave reads its 32-token tile
// as four 1 KB runs of consecutive bytes with nontemporal loads (lane l: token 8u + l / 8,
// bytes 16 (l % 8) of run u), which streams faster than the lane layout of the MFMA, and
// rearranges it through a wave-private LDS tile (rows of 144 bytes, so the eight lanes of a
// 16-byte LDS access hit disjoint banks).
constexpr int IDX_STAGE_ROWB = 144;
constexpr int IDX_STAGE_BYTES = 32 * IDX_STAGE_ROWB;  // per wave

// Tokens [s_begin, s_end) of query row i, whose keys start at cache row kv_base; with paged
// caches (pages != nullptr) token s is instead in row pages[(s >> lg) - p0] << lg | (s & page-1),
// the segment's block-table entries having been copied to LDS.  CONTIG: the keys are read as
// contiguous tiles and rearranged in the wave's LDS tile `stage`.
template <bool CONTIG>
__device__ __forceinline__ void idx_decode_segment(const uint16_t *__restrict__ q, const float *__restrict__ w,
                                                   const uint8_t *__restrict__ k, int64_t kstride,
                                                   const float *__restrict__ ks, int64_t ks_stride,
                                                   float *__restrict__ scores, int64_t ld, int64_t i,
                                                   int64_t kv_base, int64_t s_begin, int64_t s_end,
                                                   const int32_t *pages = nullptr, int lg = 0, int64_t p0 = 0,
                                                   uint32_t *wh = nullptr, char *stage = nullptr)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform loop bounds
    const int g = lane >> 5, j = lane & 31;

    bf16x8 a[8];
    const u32x4 *qp = (const u32x4 *)(q + ((i * 32 + j) * 128 + 64 * g));
#pragma unroll
    for (int t = 0; t < 8; ++t)
        a[t] = __builtin_bit_cast(bf16x8, qp[t]);
    float wr[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
        wr[rr] = w[i * 32 + 8 * (rr >> 2) + 4 * g + (rr & 3)];

    float *out = scores + i * ld;
    // Double-buffered: the next tile's 64 key bytes per lane (and its scale) are requested
    // before the current tile's MFMAs, so every wave keeps a tile in flight.
    auto load_tile = [&](int64_t s0, u32x4 (&kv)[4], float &ksv) {
        if constexpr (CONTIG) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t s = min(s0 + 8 * u + (lane >> 3), s_end - 1);
                kv[u] = __builtin_nontemporal_load((const u32x4 *)(k + (kv_base + s) * 128 + 16 * (lane & 7)));
            }
            ksv = ks[(kv_base + min(s0 + j, s_end - 1)) * ks_stride];
            return;
        }
        const int64_t s = s0 + j;
        const int64_t sc = s < s_end ? s : s_end - 1;
        const int64_t row = pages ? ((int64_t)pages[(sc >> lg) - p0] << lg) | (sc & ((1 << lg) - 1))
                                  : kv_base + sc;
        const u32x4a4 *kp = (const u32x4a4 *)(k + row * kstride + 64 * g);
        kv[0] = kp[0];
        kv[1] = kp[1];
        kv[2] = kp[2];
        kv[3] = kp[3];
        ksv = ks[row * ks_stride];
    };
    auto compute_tile = [&](const u32x4 (&kin)[4], float ksv) -> float {
        u32x4 kv[4];
        if constexpr (CONTIG) {  // to the MFMA layout: lane (g, j) takes bytes 64 g .. +63 of token j
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *(u32x4 *)(stage + (8 * u + (lane >> 3)) * IDX_STAGE_ROWB + 16 * (lane & 7)) = kin[u];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                kv[c] = *(const u32x4 *)(stage + j * IDX_STAGE_ROWB + 64 * g + 16 * c);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                kv[c] = kin[c];
        }
        f32x16 acc = {};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], fp8x8_to_bf16x8(kv[0][0], kv[0][1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], fp8x8_to_bf16x8(kv[0][2], kv[0][3]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], fp8x8_to_bf16x8(kv[1][0], kv[1][1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], fp8x8_to_bf16x8(kv[1][2], kv[1][3]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4], fp8x8_to_bf16x8(kv[2][0], kv[2][1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[5], fp8x8_to_bf16x8(kv[2][2], kv[2][3]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[6], fp8x8_to_bf16x8(kv[3][0], kv[3][1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[7], fp8x8_to_bf16x8(kv[3][2], kv[3][3]), acc, 0, 0, 0);
        float part = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            part = fmaf(wr[rr], relu(acc[rr]), part);
        part += __shfl_xor(part, 32, 64);
        return part * ksv;
    };
    auto put = [&](int64_t s0, float v) {
        const int64_t s = s0 + j;
        if (g == 0 && s < s_end) {
            out[s] = v;
            if (wh)  // the top-k's histogram bin of exactly the stored score (this wave's LDS copy)
                atomicAdd(&wh[score_key(v) >> SCORE_BIN_SHIFT], 1u);
        }
    };
    // Ping-pong over two register buffers (no copies, so only the tile being computed is
    // waited for while the other one is in flight).
    // The prefetches are unconditional (rows past the end are clamped to the last visible
    // row), so the loop body is straight-line code and only the computed tile is waited for.
    u32x4 bufA[4], bufB[4];
    float kA = 0.f, kB = 0.f;
    int64_t s0 = s_begin + wave * 32;
    if (s0 >= s_end)
        return;
    load_tile(s0, bufA, kA);
    // Long runs: sixteen tiles per round with their scores stored together at its end.  With
    // a store after every tile, the wait for the next tile's loads (issued before that store)
    // was placed so that it also waited for the store; storing once per sixteen tiles leaves
    // one such wait per round instead of one per two tiles (eight per round measured 2 us
    // slower on IndexShare with the histogram, 32 spilled).
    constexpr int NB = 16;
    for (; s0 + 128 * (NB - 1) < s_end; s0 += 128 * NB) {
        float vb[NB];
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
            load_tile(s0 + 256 * h + 128, bufB, kB);
            __builtin_amdgcn_sched_barrier(0);
            vb[2 * h] = compute_tile(bufA, kA);
            load_tile(s0 + 256 * h + 256, bufA, kA);
            __builtin_amdgcn_sched_barrier(0);
            vb[2 * h + 1] = compute_tile(bufB, kB);
        }
#pragma unroll
        for (int t = 0; t < NB; ++t)
            put(s0 + 128 * t, vb[t]);
    }
    for (; s0 < s_end; s0 += 256) {
        load_tile(s0 + 128, bufB, kB);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the wait below
        put(s0, compute_tile(bufA, kA));
        if (s0 + 128 >= s_end)
            break;
        load_tile(s0 + 256, bufA, kA);
        __builtin_amdgcn_sched_barrier(0);
        put(s0 + 128, compute_tile(bufB, kB));
    }
}

// Paged caches: a block copies the block-table entries of the tokens it is about to read to
// LDS (dynamic, sized by the host for the longest range a block covers, at most
// IDX_PAGE_TABLE_MAX entries).
constexpr int64_t IDX_PAGE_TABLE_MAX = 8192;
constexpr int64_t IDX_PAGED_SHARE = IDX_PAGE_TABLE_MAX - 32;  // tokens per page of a block's share, at most

// Two launch shapes.  Rows that are whole sequences (one query each, as in decode): the grid
// walks the concatenated token stream of all sequences, an equal share of it per block (a
// block may finish one sequence and start the next), so no block waits on a longer one.
// Otherwise: one block per (chunk, query row).
// With HIST the kernel also builds, for the top-k, each row's histogram of the top 11 key bits
// of its scores (SCORE_BINS bins, added to hist[row][bin] with integer atomics): per-wave
// histograms in LDS, summed and flushed once per (block, sequence segment).
constexpr int IDX_HIST_LDS = 4 * SCORE_BINS * (int)sizeof(uint32_t);  // 32 KB

template <bool HIST>
__device__ __forceinline__ void idx_hist_flush(uint32_t *lh, uint32_t *__restrict__ hist, int64_t row)
{
    if (!HIST)
        return;
    __syncthreads();  // every wave has added this segment's scores
    for (int b = threadIdx.x; b < SCORE_BINS; b += 256) {
        const uint32_t c = lh[b] + lh[SCORE_BINS + b] + lh[2 * SCORE_BINS + b] + lh[3 * SCORE_BINS + b];
        if (c)
            atomicAdd(&hist[row * SCORE_BINS + b], c);
        lh[b] = lh[SCORE_BINS + b] = lh[2 * SCORE_BINS + b] = lh[3 * SCORE_BINS + b] = 0u;
    }
    __syncthreads();
}

template <bool PAGED, bool HIST, bool CONTIG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void idx_decode_kernel(LayoutDev L, const uint16_t *__restrict__ q,
                                                         const float *__restrict__ w,
                                                         const uint8_t *__restrict__ k, int64_t kstride,
                                                         const float *__restrict__ ks, int64_t ks_stride,
                                                         float *__restrict__ scores, int64_t ld, int chunk,
                                                         int stream, uint32_t *__restrict__ hist)
{
    // dynamic LDS: with HIST the four waves' histograms, then (paged) a segment's table
    // entries or (CONTIG) the four waves' staging tiles
    static_assert(!(PAGED && CONTIG), "paged rows are not contiguous tiles");
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
    uint32_t *lh = s_dyn;
    int32_t *s_pages = (int32_t *)(s_dyn + (HIST ? 4 * SCORE_BINS : 0));
    char *stage = CONTIG ? (char *)s_pages + IDX_STAGE_BYTES * (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)
                         : nullptr;
    uint32_t *wh = HIST ? lh + SCORE_BINS * (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : nullptr;
    if (HIST) {
        for (int b = threadIdx.x; b < 4 * SCORE_BINS; b += 256)
            lh[b] = 0u;
        __syncthreads();
    }
    const int lg = PAGED ? 31 - __builtin_clz((unsigned)L.page_size) : 0;  // power of two (host)
    if (!stream) {
        const int64_t i = blockIdx.y;
        const RowInfo r = row_info(L, i);
        const int64_t s_begin = (int64_t)blockIdx.x * chunk;
        if (s_begin >= r.n)
            return;
        const int64_t s_end = min(s_begin + (int64_t)chunk, r.n);
        if (!PAGED) {
            idx_decode_segment<CONTIG>(q, w, k, kstride, ks, ks_stride, scores, ld, i, r.kv_base, s_begin, s_end,
                                       nullptr, 0, 0, wh, stage);
            idx_hist_flush<HIST>(lh, hist, i);
            return;
        }
        // paged caches: this chunk's block-table entries to LDS
        const int64_t p0 = s_begin >> lg, p1 = (s_end - 1) >> lg;
        for (int64_t p = p0 + threadIdx.x; p <= p1; p += 256)
            s_pages[p - p0] = L.block_table[(int64_t)r.b * L.bt_stride + p];
        __syncthreads();
        idx_decode_segment<false>(q, w, k, kstride, ks, ks_stride, scores, ld, i, 0, s_begin, s_end, s_pages, lg, p0,
                                  wh);
        idx_hist_flush<HIST>(lh, hist, i);
        return;
    }
    // stream: the grid's blocks split the N cached tokens evenly (N is known only here), in
    // ranges that are multiples of 32 tokens
    const int64_t N = L.kv_indptr[L.batch];
    const int64_t per = ((N + gridDim.x - 1) / gridDim.x + 31) & ~(int64_t)31;
    const int64_t t0 = (int64_t)blockIdx.x * per;
    if (t0 >= N)
        return;
    const int64_t t1 = min(t0 + per, N);
    int lo = 0, hi = L.batch - 1;  // the sequence holding token t0: largest b with kv_indptr[b] <= t0
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (L.kv_indptr[mid] <= t0)
            lo = mid;
        else
            hi = mid - 1;
    }
    for (int b = lo; b < L.batch; ++b) {
        const int64_t rb = L.kv_indptr[b], re = L.kv_indptr[b + 1];
        if (rb >= t1)
            break;
        const int64_t sb = max(t0, rb), se = min(t1, re);
        if (se <= sb)
            continue;
        if (!PAGED) {
            idx_decode_segment<CONTIG>(q, w, k, kstride, ks, ks_stride, scores, ld, b, rb, sb - rb, se - rb,
                                       nullptr, 0, 0, wh, stage);
            idx_hist_flush<HIST>(lh, hist, b);
            continue;
        }
        // paged caches: the segment's block-table entries to LDS, after every wave is done
        // with the previous segment's
        const int64_t s0 = sb - rb, s1 = se - rb, p0 = s0 >> lg, p1 = (s1 - 1) >> lg;
        __syncthreads();
        for (int64_t p = p0 + threadIdx.x; p <= p1; p += 256)
            s_pages[p - p0] = L.block_table[(int64_t)b * L.bt_stride + p];
        __syncthreads();
        idx_decode_segment<false>(q, w, k, kstride, ks, ks_stride, scores, ld, b, 0, s0, s1, s_pages, lg, p0, wh);
        idx_hist_flush<HIST>(lh, hist, b);
    }
}

// ------------------------------------------------------------------------------------------
// fp8 q x fp8 k, H = 32, D = 128 (prefill GEMM)
//
// Block = 8 waves x 2 query rows; the block streams CHUNK tokens of one sequence through two
// LDS tiles of 256 tokens (rows padded to 144 B so the 16-lane groups of ds_read_b128 hit
// disjoint banks), filled by buffer-to-LDS DMA one tile ahead of the MFMAs.  MFMA 32x32x64
// f8f6f4 (E4M3 on both sides, unit block scales): lane half g owns dims [64g, 64g+64) of q
// and k; MFMA t consumes 32 of them.  The weighted-ReLU head sum runs on the VALU.
// ------------------------------------------------------------------------------------------
constexpr int PF_WAVES = 8;                     // waves per block (two per SIMD)
constexpr int PF_QPW = 2;                       // query rows per wave
constexpr int PF_QPB = PF_WAVES * PF_QPW;       // query rows per block
constexpr int PF_STAGE = 256;                   // tokens per LDS tile
constexpr int PF_ROWB = 144;                    // LDS row stride in bytes (128 + pad)
constexpr int PF_TILEB = PF_STAGE * PF_ROWB;    // 36864
constexpr int PF_DMA = PF_TILEB / 1024;         // 36 wave-wide 1 KB loads per tile
constexpr int PF_DMA_PER_WAVE = (PF_DMA + PF_WAVES - 1) / PF_WAVES;  // 5 (the last only on waves 0-3)
constexpr int E8M0_ONE = 127;                   // block scale 2^0
// static LDS of the kernel (two tiles, their scales, row metadata, folded weights); paged
// caches add a table of up to PF_MAX_PAGES block-table entries, which keeps two blocks per CU
constexpr int PF_STATIC_LDS = 2 * PF_TILEB + 2 * PF_STAGE * 4 + PF_QPB * 3 * 8 + PF_QPB * 32 * 4;
constexpr int PF_MAX_PAGES = (160 * 1024 / 2 - PF_STATIC_LDS) / 4;
static_assert(PF_STAGE + 2 <= PF_MAX_PAGES, "a one-tile chunk of 1-token pages fits the table");

__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8 &a, const i32x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0, E8M0_ONE);
}

template <bool PAGED>
__global__ __launch_bounds__(64 * PF_WAVES) __attribute__((amdgpu_waves_per_eu(4))) void idx_fp8_kernel(LayoutDev L, int64_t T, const uint8_t *__restrict__ q,
                                                      const float *__restrict__ qs,
                                                      const float *__restrict__ w,
                                                      const uint8_t *__restrict__ k, int64_t kstride,
                                                      const float *__restrict__ ks, int64_t ks_stride,
                                                      float *__restrict__ scores, int64_t ld, int chunk)
{
    __shared__ __attribute__((aligned(16))) char ktile[2][PF_TILEB];
    __shared__ float kscale[2][PF_STAGE];
    __shared__ int64_t s_meta[PF_QPB][3];  // b, kv_base, n per block query row (b = -1: none)
    __shared__ __attribute__((aligned(16))) float s_wq[PF_QPB][32];  // folded head weights w * qs
    extern __shared__ int32_t s_pg[];  // paged: the segment's block-table entries (chunk / page + 2)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, j = lane & 31;
    const int64_t q0 = (int64_t)blockIdx.y * PF_QPB;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;

    if (tid < PF_QPB) {
        const int64_t qi = q0 + tid;
        if (qi < T) {
            RowInfo r = row_info(L, qi);
            s_meta[tid][0] = r.b;
            s_meta[tid][1] = r.kv_base;
            s_meta[tid][2] = r.n;
        } else {
            s_meta[tid][0] = -1;
            s_meta[tid][1] = 0;
            s_meta[tid][2] = 0;
        }
    }

    // A operands of this wave's query rows; the block's folded weights go to LDS (read back
    // as four 16-byte broadcasts per row and tile, which keeps the wave under 128 VGPRs:
    // two blocks per CU).
    i32x8 a[PF_QPW][2];
#pragma unroll
    for (int u = 0; u < PF_QPW; ++u) {
        const int64_t qi = q0 + wave * PF_QPW + u;
        const int64_t qq = qi < T ? qi : 0;
        const u32x4 *qp = (const u32x4 *)(q + (qq * 32 + j) * 128 + 64 * g);
        u32x4 v0 = qp[0], v1 = qp[1], v2 = qp[2], v3 = qp[3];
        a[u][0] = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
        a[u][1] = i32x8{(int)v2[0], (int)v2[1], (int)v2[2], (int)v2[3], (int)v3[0], (int)v3[1], (int)v3[2], (int)v3[3]};
    }
    for (int e = tid; e < PF_QPB * 32; e += 64 * PF_WAVES) {
        const int64_t qi = q0 + e / 32;
        const int64_t qq = qi < T ? qi : 0;
        s_wq[e / 32][e % 32] = w[qq * 32 + e % 32] * qs[qq * 32 + e % 32];
    }
    __syncthreads();

    // DMA geometry, fixed per lane: load qd of this wave covers tile bytes 1024 (8 qd + wave)
    // + 16 lane, i.e. one row and column (-1: pad columns, or a load past the tile).  A source
    // piece needs only dword alignment, so key rows of 132-byte entries are read in place.
    // (paged caches: toff holds row | col << 16 instead, the row mapped per tile)
    int toff[PF_DMA_PER_WAVE];
#pragma unroll
    for (int qd = 0; qd < PF_DMA_PER_WAVE; ++qd) {
        const int o = 1024 * (PF_WAVES * qd + wave) + 16 * lane;
        const int row = o / PF_ROWB, col = o - (o / PF_ROWB) * PF_ROWB;
        const bool real = o < PF_TILEB && col < 128;
        toff[qd] = !real ? -1 : PAGED ? (row | (col << 16)) : row * (int)kstride + col;
    }
    constexpr bool paged = PAGED;
    const int lg = PAGED ? 31 - __builtin_clz((unsigned)L.page_size) : 0;  // power of two (host)
    const uint32_t lds0 = lds_addr_of(&ktile[0][0]);

    // Query rows of one block may span several sequences: handle each in turn.
    int first = 0;
    while (first < PF_QPB) {
        const int64_t b = s_meta[first][0];
        if (b < 0)
            break;
        int last = first;
        int64_t nmax = s_meta[first][2];
        while (last + 1 < PF_QPB && s_meta[last + 1][0] == b) {
            ++last;
            nmax = max(nmax, s_meta[last][2]);
        }
        const int64_t kv_base = s_meta[first][1];
        const int64_t s_end = min(c0 + (int64_t)chunk, nmax);
        // this wave's rows in this segment: output from token c0 on, and how many of the
        // chunk's tokens each row sees (0: the row is not in this segment)
        // (lane half g stores the scores of the wave's row g)
        static_assert(PF_QPW == 2, "one row per lane half");
        float *myrow;
        int mylim;
        {
            const int qb = wave * PF_QPW + g;
            const int64_t nq = (qb >= first && qb <= last) ? s_meta[qb][2] : 0;
            mylim = (int)max((int64_t)0, min(nq - c0, (int64_t)chunk));
            myrow = scores + (q0 + qb) * ld + c0;
        }
        if (c0 >= s_end) {
            first = last + 1;
            continue;
        }
        // the sequence's key rows; offsets past nmax rows read zeros
        // the sequence's key rows (offsets past nmax rows read zeros), or with paged caches
        // the whole cache, addressed through the segment's block-table entries in LDS
        const i32x4 desc = paged ? buffer_desc(k, L.cache_rows * kstride)
                                 : buffer_desc(k + kv_base * kstride, nmax * kstride);
        const int64_t pg0 = c0 >> lg;
        if (PAGED) {
            const int64_t pg1 = (s_end - 1) >> lg;
            const int64_t b = s_meta[first][0];
            for (int64_t p = pg0 + tid; p <= pg1; p += 64 * PF_WAVES)
                s_pg[p - pg0] = L.block_table[b * L.bt_stride + p];
            __syncthreads();
        }
        auto prow = [&](int64_t s) -> int64_t {  // physical row of token s (paged)
            return ((int64_t)s_pg[(s >> lg) - pg0] << lg) | (s & ((1 << lg) - 1));
        };
        auto fetch = [&](int64_t st, int buf) {  // DMA of tokens st .. st+255 into ktile[buf]
            const int base = (int)(st * kstride);
#pragma unroll
            for (int qd = 0; qd < PF_DMA_PER_WAVE; ++qd) {
                const int u = PF_WAVES * qd + wave;
                int off = (int)0x80000000;
                if (toff[qd] >= 0) {
                    if (PAGED) {
                        const int64_t s = st + (toff[qd] & 0xffff);  // the table covers tokens < s_end
                        off = s < s_end ? (int)(prow(s) * kstride) + (toff[qd] >> 16) : (int)0x80000000;
                    } else {
                        off = base + toff[qd];
                    }
                }
                if (qd + 1 < PF_DMA_PER_WAVE || u < PF_DMA)
                    dma16(desc, lds0 + (uint32_t)(buf * PF_TILEB + 1024 * u), off);
            }
        };
        auto fetch_scale = [&](int64_t st) -> float {
            const int64_t s = st + tid;
            if (tid >= PF_STAGE || s >= (PAGED ? s_end : nmax))
                return 0.f;
            return ks[(PAGED ? prow(s) : kv_base + s) * ks_stride];
        };

        fetch(c0, 0);
        float sc = fetch_scale(c0);
        if (tid < PF_STAGE)
            kscale[0][tid] = sc;
        tile_barrier();
        int buf = 0;
        for (int64_t st = c0; st < s_end; st += PF_STAGE, buf ^= 1) {
            const bool more = st + PF_STAGE < s_end;
            if (more) {
                fetch(st + PF_STAGE, buf ^ 1);
                sc = fetch_scale(st + PF_STAGE);
            }
            const char *kt = &ktile[buf][0];
#pragma unroll
            for (int sub = 0; sub < PF_STAGE / 32; ++sub) {
                const int64_t sb = st + sub * 32;
                if (sb >= s_end)
                    break;
                const u32x4 *kr = (const u32x4 *)(kt + (sub * 32 + j) * PF_ROWB + 64 * g);
                const u32x4 v0 = kr[0], v1 = kr[1], v2 = kr[2], v3 = kr[3];
                const i32x8 b0 = {(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
                const i32x8 b1 = {(int)v2[0], (int)v2[1], (int)v2[2], (int)v2[3], (int)v3[0], (int)v3[1], (int)v3[2], (int)v3[3]};
                const float ksv = kscale[buf][sub * 32 + j];
                f32x16 acc[PF_QPW];
#pragma unroll
                for (int u = 0; u < PF_QPW; ++u) {
                    acc[u] = mfma_fp8_32x32x64(a[u][0], b0, f32x16{});
                    acc[u] = mfma_fp8_32x32x64(a[u][1], b1, acc[u]);
                }
                // epilogues unconditional (only the stores are masked), so both rows' MFMAs
                // issue back to back and the first epilogue overlaps the second row's MFMAs
                // (the empty asm pins both results here: no pass may sink an MFMA to its use)
                static_assert(PF_QPW == 2, "pin below");
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
                float part[PF_QPW];
#pragma unroll
                for (int u = 0; u < PF_QPW; ++u) {
                    const f32x4 *wrow = (const f32x4 *)&s_wq[wave * PF_QPW + u][4 * g];
                    part[u] = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        part[u] = fmaf(wrow[2 * (rr >> 2)][rr & 3], relu(acc[u][rr]), part[u]);
                }
                // one swap of the two halves: lanes of half 0 get (row 0 here, row 0 of lane +32),
                // lanes of half 1 get (row 1 of lane -32, row 1 here); each adds the (half 0,
                // half 1) pair and stores its row's score for token j
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                                 false, false);
                const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const int so = (int)(sb - c0) + j;  // offset in the chunk
                if (so < mylim)
                    myrow[so] = tot * ksv;
            }
            if (more && tid < PF_STAGE)
                kscale[buf ^ 1][tid] = sc;
            tile_barrier();  // the next tile has landed; this one is free
        }
        first = last + 1;
    }
}

// ------------------------------------------------------------------------------------------
// generic: any dtypes, H <= 64, D <= 256.  One thread per token; q row in LDS as fp32.
// ------------------------------------------------------------------------------------------
template <int QDT, int KDT>
__global__ __launch_bounds__(256) void idx_generic_kernel(LayoutDev L, int H, int D, const void *__restrict__ q,
                                                          const float *__restrict__ qs,
                                                          const float *__restrict__ w,
                                                          const uint8_t *__restrict__ k, int64_t kstride,
                                                          const float *__restrict__ ks, int64_t ks_stride,
                                                          float *__restrict__ scores, int64_t ld)
{
    extern __shared__ float sm[];  // [H*D] q, then [H] folded weights
    const int64_t i = blockIdx.y;
    const RowInfo r = row_info(L, i);
    const int64_t sblk = (int64_t)blockIdx.x * 256;
    if (sblk >= r.n)
        return;
    float *sq = sm, *sw = sm + H * D;
    for (int e = threadIdx.x; e < H * D; e += 256)
        sq[e] = load_elem<QDT>(q, i * H * D + e);
    for (int h = threadIdx.x; h < H; h += 256)
        sw[h] = w[i * H + h] * (qs ? qs[i * H + h] : 1.f);
    __syncthreads();
    const int64_t s = sblk + threadIdx.x;
    if (s >= r.n)
        return;
    const int64_t row = token_row(L, r.b, r.kv_base, s);
    const uint8_t *krow = k + row * kstride;
    float acc = 0.f;
    for (int h = 0; h < H; ++h) {
        float a = 0.f;
        for (int d = 0; d < D; ++d)
            a = fmaf(sq[h * D + d], load_elem<KDT>(krow, d), a);
        acc = fmaf(sw[h], fmaxf(a, 0.f), acc);
    }
    scores[i * ld + s] = acc * (ks ? ks[row * ks_stride] : 1.f);
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
constexpr int IDX_STREAM_BLOCKS = 512;  // two blocks per CU: measured as good as or better than four

hipError_t launch_index_decode(const LayoutDev &L, int64_t T, int64_t max_ctx, const void *q,
                               const float *w, const void *k, int64_t kstride, const float *ks,
                               int64_t ks_stride, float *scores, int64_t ld, hipStream_t stream,
                               uint32_t *hist)
{
    // Per (chunk, query row) blocks: waves of at most 16 tiles and enough blocks to cover the
    // chip several times, at least two 32-token tiles per wave (one tile per wave re-reads q
    // and w for too little work: 7.9 against 9.2 us on the 8-row decode).  DSA_INDEXER_CHUNK
    // (a power of two in [128, 8192]) overrides the tokens per block and DSA_INDEXER_BLOCKS
    // the stream's block count, for launch-shape tuning.
    int chunk = 2048;
    while (chunk > 256 && T * ((max_ctx + chunk - 1) / chunk) < 2048)
        chunk >>= 1;
    if (const char *env = getenv("DSA_INDEXER_CHUNK")) {
        const int c = atoi(env);
        if (c >= 128 && c <= 8192 && (c & (c - 1)) == 0)
            chunk = c;
    }
    while (L.block_table && chunk / L.page_size + 2 > IDX_PAGE_TABLE_MAX)  // paged: table fits LDS
        chunk >>= 1;
    const int64_t nchunks = (max_ctx + chunk - 1) / chunk;
    const bool as_stream = L.q_indptr == nullptr;  // rows are whole sequences
    // stream: two blocks per CU for long streams (one round; four per CU measured no
    // better), fewer blocks (at least 256 tokens each) for short ones; the kernel divides
    // the actual token count
    int64_t sblocks = min((int64_t)IDX_STREAM_BLOCKS, (T * max_ctx + 255) / 256);
    if (const char *env = getenv("DSA_INDEXER_BLOCKS")) {  // launch-shape tuning
        const int nb = atoi(env);
        if (nb >= 1 && nb <= 65536)
            sblocks = min((int64_t)nb, T * max_ctx);
    }
    // Paged: tokens [s0, s1) span at most (s1 - s0) / page + 2 pages.  A stream block's
    // share is at most per_max tokens (the kernel divides N <= T * max_ctx tokens the same
    // way); shares are kept to IDX_PAGED_SHARE pages' worth so the table stays in 32 KB.
    size_t lds = 0;
    if (L.block_table) {
        const int64_t page = L.page_size;
        int64_t span = chunk;
        if (as_stream) {
            sblocks = max(sblocks, (T * max_ctx + IDX_PAGED_SHARE * page - 1) / (IDX_PAGED_SHARE * page));
            span = (((T * max_ctx + sblocks - 1) / sblocks) + 31) & ~(int64_t)31;
        }
        lds = (size_t)(span / page + 2) * sizeof(int32_t);  // <= IDX_PAGE_TABLE_MAX entries
    }
    dim3 grid = as_stream ? dim3((unsigned)max((int64_t)1, sblocks)) : dim3((unsigned)nchunks, (unsigned)T);
    const int st = as_stream ? 1 : 0;
    const uint16_t *qh = (const uint16_t *)q;
    const uint8_t *kk = (const uint8_t *)k;
    // unpaged 128-byte rows at a 16-byte aligned base: contiguous tiles
    const bool contig = !L.block_table && kstride == 128 && ((uintptr_t)k & 15) == 0;
    if (hist)
        lds += IDX_HIST_LDS;
    if (contig)
        lds += 4 * IDX_STAGE_BYTES;
#define DSA_IDX_DECODE(P, H, C)                                                                                  \
    hipLaunchKernelGGL((idx_decode_kernel<P, H, C>), grid, dim3(256), lds, stream, L, qh, w, kk, kstride, ks, ks_stride, \
                       scores, ld, chunk, st, hist)
    if (L.block_table) {
        if (hist)
            DSA_IDX_DECODE(true, true, false);
        else
            DSA_IDX_DECODE(true, false, false);
    } else if (contig) {
        if (hist)
            DSA_IDX_DECODE(false, true, true);
        else
            DSA_IDX_DECODE(false, false, true);
    } else {
        if (hist)
            DSA_IDX_DECODE(false, true, false);
        else
            DSA_IDX_DECODE(false, false, false);
    }
#undef DSA_IDX_DECODE
    return hipGetLastError();
}

hipError_t launch_index_fp8(const LayoutDev &L, int64_t T, int64_t max_ctx, const void *q,
                            const float *qs, const float *w, const void *k, int64_t kstride,
                            const float *ks, int64_t ks_stride, float *scores, int64_t ld,
                            hipStream_t stream)
{
    // Long chunks amortise each block's start (q, weights, first tile); halve them only
    // while the grid would not fill two rounds of the chip's 512 block slots (2 per CU).
    int chunk = 8192;
    const int64_t qblocks = (T + PF_QPB - 1) / PF_QPB;
    while (chunk > PF_STAGE && qblocks * ((max_ctx + chunk - 1) / chunk) < 1024)
        chunk >>= 1;
    if (const char *env = getenv("DSA_INDEXER_CHUNK")) {  // launch-shape tuning (power of two)
        const int c = atoi(env);
        if (c >= PF_STAGE && c <= 8192 && (c & (c - 1)) == 0)
            chunk = c;
    }
    // paged: a chunk spans at most chunk / page + 2 pages, whose table entries go to LDS
    if (L.block_table)
        while (chunk > PF_STAGE && chunk / L.page_size + 2 > PF_MAX_PAGES)
            chunk >>= 1;
    const size_t lds = L.block_table ? (size_t)(chunk / L.page_size + 2) * sizeof(int32_t) : 0;
    dim3 grid((unsigned)((max_ctx + chunk - 1) / chunk), (unsigned)qblocks);
    if (L.block_table)
        hipLaunchKernelGGL(idx_fp8_kernel<true>, grid, dim3(64 * PF_WAVES), lds, stream, L, T, (const uint8_t *)q, qs, w,
                           (const uint8_t *)k, kstride, ks, ks_stride, scores, ld, chunk);
    else
        hipLaunchKernelGGL(idx_fp8_kernel<false>, grid, dim3(64 * PF_WAVES), 0, stream, L, T, (const uint8_t *)q, qs, w,
                           (const uint8_t *)k, kstride, ks, ks_stride, scores, ld, chunk);
    return hipGetLastError();
}

template <int QDT, int KDT>
static hipError_t launch_generic_t(const LayoutDev &L, int64_t T, int64_t max_ctx, int H, int D,
                                   const void *q, const float *qs, const float *w, const void *k,
                                   int64_t kstride, const float *ks, int64_t ks_stride, float *scores,
                                   int64_t ld, hipStream_t stream)
{
    dim3 grid((unsigned)((max_ctx + 255) / 256), (unsigned)T);
    size_t shmem = sizeof(float) * (size_t)(H * D + H);
    hipLaunchKernelGGL((idx_generic_kernel<QDT, KDT>), grid, dim3(256), shmem, stream, L, H, D, q, qs,
                       w, (const uint8_t *)k, kstride, ks, ks_stride, scores, ld);
    return hipGetLastError();
}

hipError_t launch_index_generic(const LayoutDev &L, int64_t T, int64_t max_ctx, int H, int D,
                                int q_dt, const void *q, const float *qs, const float *w, int k_dt,
                                const void *k, int64_t kstride, const float *ks, int64_t ks_stride,
                                float *scores, int64_t ld, hipStream_t stream)
{
#define DSA_IDX_CASE(QD, KD)                                                                     \
    if (q_dt == QD && k_dt == KD)                                                                \
        return launch_generic_t<QD, KD>(L, T, max_ctx, H, D, q, qs, w, k, kstride, ks, ks_stride, \
                                        scores, ld, stream);
    DSA_IDX_CASE(0, 0) DSA_IDX_CASE(0, 1) DSA_IDX_CASE(0, 2)
    DSA_IDX_CASE(1, 0) DSA_IDX_CASE(1, 1) DSA_IDX_CASE(1, 2)
    DSA_IDX_CASE(2, 0) DSA_IDX_CASE(2, 1) DSA_IDX_CASE(2, 2)
#undef DSA_IDX_CASE
    return hipErrorInvalidValue;
}

}  // namespace dsa
