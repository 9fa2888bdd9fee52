// topk.hip -- per-row top-k with a deterministic order, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram: top-k = 2048 written as int32
// [tokens x 2048]; ATOM-side optimisations, stable_topk: ties must resolve the same
// way every time; caveats: with fewer than k visible tokens every token is taken.)
//
// Order: higher score first; equal scores (with -0 == +0) by lower position.  Each score
// maps to a monotone 32-bit key (sign-flipped IEEE bits, -0 folded into +0) and each
// candidate to the 64-bit composite (key << 32) | ~position, which is unique per row, so
// "larger composite first" is exactly that order.
//
// Rows longer than CAP take two kernels:
//  K1  topk_hist_kernel   many blocks per row: an LDS histogram (one per wave) of the top 11
//                         key bits of a chunk, added into the row's global histogram with
//                         integer atomics (deterministic totals);
//  K2  topk_select_kernel one 1024-thread block per row: the histogram gives the bin that
//                         holds the k-th key; one pass gathers every score at or above that
//                         bin into LDS (when they fit), an exact radix select over the
//                         composites keeps exactly k, and a sort orders them (per-wave
//                         bitonic with shuffles, then four LDS merge levels).  K2 clears
//                         the row's histogram, so the workspace is zero again for the next
//                         call.  Rows with at most CAP scores skip K1 and load directly.
// If the scores at or above the threshold bin do not fit in LDS (heavily tied data), K2
// falls back to radix passes over the row in global memory and an ordered compaction of
// the ties (lowest positions first).
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAP = 8192;        // candidates held in LDS (64 KB of composites)
constexpr int TK_BINS = 2048;       // 11-bit digits
constexpr int TK_SORT = 2048;       // sort width (>= DSA_TOPK_MAX)
constexpr int H_THREADS = 256;      // histogram kernel
constexpr int H_CHUNK = 8192;       // scores per histogram block

__device__ __forceinline__ uint32_t score_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int64_t s)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s);
}

// Exclusive scan over the block (one value per thread, thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < TK_WAVES; ++w2) {
        const uint32_t t = wsum[w2];
        before += (w2 < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// Given a histogram of nb bins (counts of candidates matching the current prefix) and the
// number still needed, find the bin holding the need-th largest: returns the bin, the
// count strictly above it and its own count.  Thread t owns bins nb-1-2t and nb-2-2t.
struct DigitPick {
    uint32_t digit, above, count;
};
__device__ __forceinline__ DigitPick pick_digit(const uint32_t *hist, int nb, uint32_t need, uint32_t *wsum,
                                                uint32_t *sh)
{
    const int tid = threadIdx.x;
    const int d_hi = nb - 1 - 2 * tid;
    uint32_t c_hi = 0, c_lo = 0;
    if (2 * tid < nb) {
        c_hi = hist[d_hi];
        c_lo = hist[d_hi - 1];
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan(c_hi + c_lo, wsum, &tot);
    if (2 * tid < nb) {
        if (ex < need && need <= ex + c_hi) {
            sh[0] = (uint32_t)d_hi;
            sh[1] = ex;
            sh[2] = c_hi;
        } else if (ex + c_hi < need && need <= ex + c_hi + c_lo) {
            sh[0] = (uint32_t)(d_hi - 1);
            sh[1] = ex + c_hi;
            sh[2] = c_lo;
        }
    }
    __syncthreads();
    DigitPick p{sh[0], sh[1], sh[2]};
    __syncthreads();
    return p;
}

// ------------------------------------------------------------------------------------------
// K1: per-row histogram of the top 11 key bits
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(H_THREADS) void topk_hist_kernel(LayoutDev L, const float *__restrict__ scores,
                                                              int64_t ld, uint32_t *__restrict__ ghist)
{
    __shared__ uint32_t lh[H_THREADS / 64][TK_BINS];
    const int64_t i = blockIdx.y;
    const RowInfo r = row_info(L, i);
    const int64_t s0 = (int64_t)blockIdx.x * H_CHUNK;
    if (s0 >= r.n)
        return;
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int b = tid; b < (H_THREADS / 64) * TK_BINS; b += H_THREADS)
        (&lh[0][0])[b] = 0u;
    __syncthreads();
    const int64_t s1 = min(s0 + (int64_t)H_CHUNK, r.n);
    const float *row = scores + i * ld;
    for (int64_t s = s0 + 4 * tid; s < s1; s += 4 * H_THREADS) {
        if (s + 3 < s1 && ((uintptr_t)(row + s) & 15) == 0) {
            const f32x4 v = *(const f32x4 *)(row + s);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                atomicAdd(&lh[wave][score_key(v[e]) >> 21], 1u);
        } else {
            for (int e = 0; e < 4 && s + e < s1; ++e)
                atomicAdd(&lh[wave][score_key(row[s + e]) >> 21], 1u);
        }
    }
    __syncthreads();
    for (int b = tid; b < TK_BINS; b += H_THREADS) {
        uint32_t c = 0;
#pragma unroll
        for (int w2 = 0; w2 < H_THREADS / 64; ++w2)
            c += lh[w2][b];
        if (c)
            atomicAdd(&ghist[i * TK_BINS + b], c);
    }
}

// ------------------------------------------------------------------------------------------
// K2: gather, exact select, sort, emit
// ------------------------------------------------------------------------------------------
// Descending sort of TK_SORT unique composites.  Lane l of wave w holds positions
// 128w + 2l and 128w + 2l + 1: every wave first sorts its 128 with a bitonic network whose
// partners are in the same thread or wave (shuffles, no barrier); four merge levels then
// join runs of 128 -> 256 -> ... -> 2048 through LDS.  In a merge, an element's place is its
// index in its own run plus the number of larger elements in the partner run (binary
// search), which is exact because the composites are unique.  The result is left in buf
// (TK_SORT entries; `tmp` is a second buffer of the same size).
__device__ __forceinline__ void sort_2048_desc(uint64_t v[2], uint64_t *buf, uint64_t *tmp)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride == 1) {
                const int q = 2 * lane;
                const bool desc = (size == 128) || ((q & size) == 0);
                const uint64_t a = v[0], b = v[1];
                const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
                v[0] = desc ? hi : lo;
                v[1] = desc ? lo : hi;
            } else {
                const int ls = stride >> 1;  // partner lane distance
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const uint64_t o = __shfl_xor(v[rr], ls, 64);
                    const int q = 2 * lane + rr;
                    const bool lower = (q & stride) == 0;
                    const bool desc = (size == 128) || ((q & size) == 0);
                    const bool keep_max = (lower == desc);
                    v[rr] = keep_max ? (v[rr] > o ? v[rr] : o) : (v[rr] > o ? o : v[rr]);
                }
            }
        }
    }
    uint64_t *src = buf, *dst = tmp;
    src[128 * w + 2 * lane] = v[0];
    src[128 * w + 2 * lane + 1] = v[1];
    __syncthreads();
#pragma unroll 1
    for (int run = 128; run < TK_SORT; run <<= 1) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int p = 2 * tid + rr;
            const int pair0 = p & ~(2 * run - 1);      // start of the merged pair of runs
            const int in_b = (p & run) != 0;           // element sits in the second run
            const int own = p - pair0 - (in_b ? run : 0);
            const uint64_t *other = src + pair0 + (in_b ? 0 : run);
            const uint64_t x = src[p];
            int lo = 0, hi = run;                       // count of partner entries > x
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (other[mid] > x)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            dst[pair0 + own + lo] = x;
        }
        __syncthreads();
        uint64_t *t = src;
        src = dst;
        dst = t;
    }
    if (src != buf) {  // odd number of levels: copy back
        buf[2 * tid] = src[2 * tid];
        buf[2 * tid + 1] = src[2 * tid + 1];
        __syncthreads();
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_select_kernel(LayoutDev L, const float *__restrict__ scores,
                                                                 int64_t ld, int k, int32_t *__restrict__ out,
                                                                 uint32_t *__restrict__ ghist)
{
    __shared__ uint64_t cand[TK_CAP];
    __shared__ uint32_t hist[TK_BINS];
    __shared__ uint32_t wsum[TK_WAVES];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t sh_cnt;

    const int tid = threadIdx.x;
    const int64_t i = blockIdx.x;
    const RowInfo r = row_info(L, i);
    const int64_t n = r.n > 0 ? r.n : 0;
    const float *row = scores + i * ld;
    int32_t *orow = out + i * k;
    const uint32_t kk = (uint32_t)min((int64_t)k, n);

    if (tid == 0)
        sh_cnt = 0u;
    uint32_t m;  // candidates in cand
    if (n <= TK_CAP) {
        for (int64_t s = tid; s < n; s += TK_THREADS)
            cand[s] = composite(score_key(row[s]), s);
        m = (uint32_t)n;
        __syncthreads();
    } else {
        // threshold bin from the row histogram (then clear it for the next call)
        uint32_t *gh = ghist + i * TK_BINS;
        for (int b = tid; b < TK_BINS; b += TK_THREADS) {
            hist[b] = gh[b];
            gh[b] = 0u;
        }
        __syncthreads();
        const DigitPick p0 = pick_digit(hist, TK_BINS, kk, wsum, sh);
        const uint32_t count_ge = p0.above + p0.count;
        if (count_ge <= (uint32_t)TK_CAP) {
            const uint32_t lo_key = p0.digit << 21;
            for (int64_t s = tid; s < n; s += TK_THREADS) {
                const uint32_t key = score_key(row[s]);
                if (key >= lo_key)
                    cand[atomicAdd(&sh_cnt, 1u)] = composite(key, s);
            }
            m = count_ge;
            __syncthreads();
        } else {
            // Too many scores share the threshold bin: refine with two more passes over the
            // row, then take keys above tau and the lowest positions among its copies.
            uint32_t prefix = p0.digit, above = p0.above, need = kk - p0.above;
            int shift = 21;
            const int widths[2] = {11, 10};
            for (int pass = 0; pass < 2; ++pass) {
                const int width = widths[pass], nshift = shift - width;
                const uint32_t dmask = (1u << width) - 1u;
                for (int b = tid; b < TK_BINS; b += TK_THREADS)
                    hist[b] = 0u;
                __syncthreads();
                for (int64_t s = tid; s < n; s += TK_THREADS) {
                    const uint32_t key = score_key(row[s]);
                    if ((key >> shift) == prefix)
                        atomicAdd(&hist[(key >> nshift) & dmask], 1u);
                }
                __syncthreads();
                const DigitPick p = pick_digit(hist, 1 << width, need, wsum, sh);
                above += p.above;
                need -= p.above;
                prefix = (prefix << width) | p.digit;
                shift = nshift;
            }
            const uint32_t tau = prefix;
            for (int64_t s = tid; s < n; s += TK_THREADS) {
                const uint32_t key = score_key(row[s]);
                if (key > tau)
                    cand[atomicAdd(&sh_cnt, 1u)] = composite(key, s);
            }
            uint32_t taken = 0;
            for (int64_t base = 0; base < n && taken < need; base += TK_THREADS) {
                const int64_t s = base + tid;
                const uint32_t flag = (s < n && score_key(row[s]) == tau) ? 1u : 0u;
                uint32_t tot;
                const uint32_t rank = block_excl_scan(flag, wsum, &tot);
                if (flag && taken + rank < need)
                    cand[above + taken + rank] = composite(tau, s);
                taken += tot;
            }
            m = kk;
            __syncthreads();
        }
    }

    // ---- exact selection of the kk largest composites among the m candidates (unique)
    uint64_t lo_comp = 0;  // every selected composite is >= lo_comp
    if (m > kk) {
        uint64_t prefix = 0;
        uint32_t need = kk;
        int shift = 64;
        while (true) {
            const int width = shift >= 11 ? 11 : shift;
            const int nshift = shift - width;
            const uint64_t dmask = (1ull << width) - 1ull;
            for (int b = tid; b < TK_BINS; b += TK_THREADS)
                hist[b] = 0u;
            __syncthreads();
            for (uint32_t c = tid; c < m; c += TK_THREADS) {
                const uint64_t v = cand[c];
                if (shift == 64 || (v >> shift) == prefix)
                    atomicAdd(&hist[(uint32_t)((v >> nshift) & dmask)], 1u);
            }
            __syncthreads();
            const DigitPick p = pick_digit(hist, 1 << width, need, wsum, sh);
            prefix = (shift == 64 ? 0ull : (prefix << width)) | p.digit;
            shift = nshift;
            need -= p.above;
            if (p.count == need || shift == 0) {  // the whole bin is taken
                lo_comp = prefix << shift;
                break;
            }
        }
    }

    // ---- compact the selected composites into sort slots, pad, sort, emit
    uint64_t v[2];
    if (m > kk) {
        // move the selected composites to the front of cand: every thread reads its
        // candidates before the scan's barrier, then writes them to its ranked slots
        uint64_t mine[TK_CAP / TK_THREADS];
        uint32_t sel_mask = 0, cnt_mine = 0;
#pragma unroll
        for (int e = 0; e < TK_CAP / TK_THREADS; ++e) {
            const uint32_t c = tid + e * TK_THREADS;
            mine[e] = c < m ? cand[c] : 0ull;
            if (c < m && mine[e] >= lo_comp) {
                sel_mask |= 1u << e;
                ++cnt_mine;
            }
        }
        uint32_t tot;
        uint32_t pos = block_excl_scan(cnt_mine, wsum, &tot);
#pragma unroll
        for (int e = 0; e < TK_CAP / TK_THREADS; ++e)
            if (sel_mask & (1u << e))
                cand[pos++] = mine[e];
        __syncthreads();
    }
    // unique padding below every real composite (real keys are >= 0x007FFFFF)
    v[0] = (uint32_t)(2 * tid) < kk ? cand[2 * tid] : (uint64_t)(2 * tid);
    v[1] = (uint32_t)(2 * tid + 1) < kk ? cand[2 * tid + 1] : (uint64_t)(2 * tid + 1);
    __syncthreads();
    sort_2048_desc(v, cand, cand + TK_SORT);
    for (int t = tid; t < k; t += TK_THREADS)
        orow[t] = (uint32_t)t < kk ? (int32_t)(0xFFFFFFFFu - (uint32_t)(cand[t] & 0xFFFFFFFFull)) : -1;
}

// ------------------------------------------------------------------------------------------
size_t topk_workspace_bytes(int64_t T, int64_t max_ctx)
{
    return max_ctx > TK_CAP ? (size_t)T * TK_BINS * sizeof(uint32_t) : 0;
}

hipError_t launch_topk(const LayoutDev &L, int64_t T, int64_t max_ctx, const float *scores, int64_t ld,
                       int k, int32_t *indices, void *workspace, hipStream_t stream)
{
    uint32_t *ghist = (uint32_t *)workspace;
    if (max_ctx > TK_CAP) {
        dim3 hgrid((unsigned)((max_ctx + H_CHUNK - 1) / H_CHUNK), (unsigned)T);
        hipLaunchKernelGGL(topk_hist_kernel, hgrid, dim3(H_THREADS), 0, stream, L, scores, ld, ghist);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)T), dim3(TK_THREADS), 0, stream, L, scores, ld, k,
                       indices, ghist);
    return hipGetLastError();
}

}  // namespace dsa
