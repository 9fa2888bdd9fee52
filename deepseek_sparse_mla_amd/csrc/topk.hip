// topk.hip -- per-row top-k with a deterministic order, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram: top-k = 2048 written as int32
// [tokens x 2048]; ATOM-side optimisations, stable_topk: ties must resolve the same
// way every time; caveats: with fewer than k visible tokens every token is taken.)
//
// Selection order: higher score first; equal scores (with -0 == +0) by lower position.
// Each score maps to a monotone 32-bit key (sign-flipped IEEE bits, -0 folded into +0) and
// each candidate to the 64-bit composite (key << 32) | ~position, which is unique per row,
// so "larger composite first" is exactly that order.  The selected set is then written in
// ascending position order (the attention over it does not depend on the order, and the
// gathers it drives then walk the cache forwards).
//
// Rows longer than CAP take two kernels:
//  K1  topk_hist_kernel   many blocks per row: an LDS histogram (one per wave) of the top 11
//                         key bits of a chunk, added into the row's global histogram with
//                         integer atomics (deterministic totals);
//  K2  topk_select_kernel one 1024-thread block per row: the histogram gives the bin that
//                         holds the k-th key; one pass gathers every score at or above that
//                         bin into LDS (when they fit), an exact radix select over the
//                         composites finds the k-th largest, and the selected positions are
//                         marked in an LDS bitmap and compacted in position order.  K2
//                         clears the row's histogram, so the workspace is zero again for the
//                         next call.  Rows with at most CAP scores skip K1 and load directly.
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
constexpr int TK_BMAP_BITS = 1 << 15;  // positions marked per bitmap pass (4 KB: two blocks per CU)
constexpr int TK_BMAP_WORDS = TK_BMAP_BITS / 32;
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
__global__ __launch_bounds__(TK_THREADS) void topk_select_kernel(LayoutDev L, const float *__restrict__ scores,
                                                                 int64_t ld, int k, int32_t *__restrict__ out,
                                                                 uint32_t *__restrict__ ghist)
{
    __shared__ uint64_t cand[TK_CAP];
    __shared__ uint32_t hist[TK_BINS];
    __shared__ uint32_t bmap[TK_BMAP_WORDS];
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
            // one pass over the row: 16-byte loads, four in flight per thread, and one LDS
            // atomic per wave (ballot + popcount give each lane its slot)
            const uint32_t lo_key = p0.digit << 21;
            const int lane = tid & 63;
            const uint64_t below = (1ull << lane) - 1ull;
            auto take = [&](float x, int64_t s, bool in) {
                const uint32_t key = score_key(x);
                const bool hit = in && key >= lo_key;
                const uint64_t b = __ballot(hit);
                if (b == 0ull)
                    return;
                uint32_t base = 0;
                if (lane == 0)
                    base = atomicAdd(&sh_cnt, (uint32_t)__popcll(b));
                base = __shfl(base, 0, 64);
                if (hit)
                    cand[base + (uint32_t)__popcll(b & below)] = composite(key, s);
            };
            const int64_t head = (int64_t)((4 - (((uintptr_t)row >> 2) & 3)) & 3);  // to 16-B alignment
            const int64_t h = head < n ? head : n;
            take(tid < h ? row[tid] : 0.f, tid, tid < h);
            const float4 *row4 = (const float4 *)(row + h);
            const int64_t n4 = (n - h) >> 2;
            constexpr int U = 4;
            for (int64_t b4 = 0; b4 < n4; b4 += (int64_t)U * TK_THREADS) {
                float4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t j = b4 + (int64_t)u * TK_THREADS + tid;
                    v[u] = j < n4 ? row4[j] : float4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t j = b4 + (int64_t)u * TK_THREADS + tid;
                    const int64_t s0 = h + 4 * j;
                    const bool in = j < n4;
                    take(v[u].x, s0, in);
                    take(v[u].y, s0 + 1, in);
                    take(v[u].z, s0 + 2, in);
                    take(v[u].w, s0 + 3, in);
                }
            }
            const int64_t tail0 = h + 4 * n4;  // fewer than 4 scores left
            take(tail0 + tid < n ? row[tail0 + tid] : 0.f, tail0 + tid, tail0 + tid < n);
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

    // ---- list the selected positions in ascending order: mark them in a bitmap (one pass
    // per 2^15 positions), then a block scan over per-thread popcounts of consecutive
    // words gives every set bit its output slot.  The slots are staged in hist (kk <= 2048).
    static_assert(TK_BINS >= DSA_TOPK_MAX, "staging area");
    uint32_t *slots = hist;
    uint32_t done = 0;
    for (int64_t cb = 0; cb < n && done < kk; cb += TK_BMAP_BITS) {
        const int64_t len = min((int64_t)TK_BMAP_BITS, n - cb);
        const int nw = (int)((len + 31) >> 5);
        __syncthreads();  // previous pass's readers of bmap are done
        for (int w = tid; w < nw; w += TK_THREADS)
            bmap[w] = 0u;
        __syncthreads();
        for (uint32_t c = tid; c < m; c += TK_THREADS) {
            const uint64_t v = cand[c];
            if (m > kk && v < lo_comp)
                continue;
            const int64_t pos = (int64_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
            if (pos >= cb && pos < cb + len) {
                const uint32_t rel = (uint32_t)(pos - cb);
                atomicOr(&bmap[rel >> 5], 1u << (rel & 31));
            }
        }
        __syncthreads();
        const int wpt = (nw + TK_THREADS - 1) / TK_THREADS;  // consecutive words per thread
        const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
        uint32_t cnt = 0;
        for (int w = w0; w < w1; ++w)
            cnt += __popc(bmap[w]);
        uint32_t tot;
        uint32_t slot = done + block_excl_scan(cnt, wsum, &tot);
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = bmap[w];
            while (bits) {
                const int b = __ffs(bits) - 1;
                if (slot < (uint32_t)TK_BINS)
                    slots[slot] = (uint32_t)(cb + 32 * w + b);
                ++slot;
                bits &= bits - 1u;
            }
        }
        done += tot;
    }
    __syncthreads();
    for (int t = tid; t < k; t += TK_THREADS)
        orow[t] = (uint32_t)t < kk ? (int32_t)slots[t] : -1;
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
