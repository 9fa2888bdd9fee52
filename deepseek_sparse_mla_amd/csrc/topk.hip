// topk.hip -- per-row top-k with a deterministic order, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram: top-k = 2048 written as int32
// [tokens x 2048]; ATOM-side optimisations, stable_topk: ties must resolve the same
// way every time; caveats: with fewer than k visible tokens every token is taken.)
//
// Order: higher score first; equal scores (with -0 == +0) by lower position.  Each score
// maps to a monotone 32-bit key (sign-flipped IEEE bits, -0 folded into +0) and each
// candidate to the 64-bit composite (key << 32) | ~position, so "larger composite first"
// is exactly that order and a plain descending sort of composites gives the output.
//
// One 1024-thread block per query row:
//  1. rows with n <= CAP: load every candidate into LDS and sort.
//  2. otherwise an MSB-first radix select over the keys (digits of 11, 11, 10 bits, an LDS
//     histogram per pass read from the row in global memory) narrows the threshold until
//     the candidates at or above it fit in LDS (CAP); they are gathered and sorted.
//  3. if even the exact k-th key has too many copies, every key above it is gathered and
//     the ties are taken in position order by an ordered (block-scan) compaction.
// The sort is a bitonic network over the LDS buffer.  All choices depend only on the
// data, so the output is deterministic; integer LDS atomics only count.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_CAP = 4096;      // candidates sorted in LDS (32 KB of composites)
constexpr int TK_BINS = 2048;     // 11-bit digits

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

// Exclusive scan over 1024 threads (one value each), in thread order.  Returns the
// exclusive prefix; *total receives the sum.  `wsum` holds 16 partials.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < TK_THREADS / 64; ++w2) {
        const uint32_t t = wsum[w2];
        before += (w2 < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// Descending bitonic sort of buf[0 .. m2), m2 a power of two >= 2.
__device__ __forceinline__ void bitonic_desc(uint64_t *buf, int m2)
{
    for (int size = 2; size <= m2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (m2 >> 1); t += TK_THREADS) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = buf[lo], b = buf[hi];
                if ((a < b) == desc) {
                    buf[lo] = b;
                    buf[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(LayoutDev L, const float *__restrict__ scores,
                                                          int64_t ld, int k, int32_t *__restrict__ out)
{
    __shared__ uint64_t buf[TK_CAP];
    __shared__ uint32_t hist[TK_BINS];
    __shared__ uint32_t wsum[TK_THREADS / 64];
    __shared__ uint32_t sh_cnt, sh_digit, sh_above_d, sh_count_d;

    const int tid = threadIdx.x;
    const int64_t i = blockIdx.x;
    const RowInfo r = row_info(L, i);
    const int64_t n = r.n > 0 ? r.n : 0;
    const float *row = scores + i * ld;
    int32_t *orow = out + i * k;
    const int kk = (int)min((int64_t)k, n);

    int m = 0;  // number of composites in buf
    if (n <= TK_CAP) {
        for (int64_t s = tid; s < n; s += TK_THREADS)
            buf[s] = composite(score_key(row[s]), s);
        m = (int)n;
    } else {
        // ---- radix select ------------------------------------------------------------
        uint32_t prefix = 0;   // resolved high bits of the threshold key
        int shift = 32;        // low bits still unresolved
        uint32_t above = 0;    // candidates with key above the current prefix range
        uint32_t need = (uint32_t)kk;
        bool gathered = false;
        const int widths[3] = {11, 11, 10};
        for (int pass = 0; pass < 3; ++pass) {
            const int width = widths[pass];
            const int nshift = shift - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int b = tid; b < TK_BINS; b += TK_THREADS)
                hist[b] = 0u;
            __syncthreads();
            for (int64_t s = tid; s < n; s += TK_THREADS) {
                const uint32_t key = score_key(row[s]);
                const bool match = (pass == 0) || ((key >> shift) == prefix);
                if (match)
                    atomicAdd(&hist[(key >> nshift) & dmask], 1u);
            }
            __syncthreads();
            // suffix counts from the top digit down: thread t owns digits 2t, 2t+1
            // (reversed so that the scan runs from the largest digit)
            const int nb = 1 << width;
            const int d_hi = nb - 1 - 2 * tid;  // this thread's larger digit
            uint32_t c_hi = 0, c_lo = 0;
            if (2 * tid < nb) {
                c_hi = hist[d_hi];
                c_lo = hist[d_hi - 1];
            }
            uint32_t tot;
            const uint32_t ex = block_excl_scan(c_hi + c_lo, wsum, &tot);  // count above d_hi
            if (2 * tid < nb) {
                if (ex < need && need <= ex + c_hi) {
                    sh_digit = (uint32_t)d_hi;
                    sh_above_d = ex;
                    sh_count_d = c_hi;
                } else if (ex + c_hi < need && need <= ex + c_hi + c_lo) {
                    sh_digit = (uint32_t)(d_hi - 1);
                    sh_above_d = ex + c_hi;
                    sh_count_d = c_lo;
                }
            }
            __syncthreads();
            const uint32_t dstar = sh_digit;
            above += sh_above_d;
            need -= sh_above_d;
            prefix = (prefix << width) | dstar;
            shift = nshift;
            const uint32_t count_ge = above + sh_count_d;  // keys >= prefix << shift
            if (count_ge <= (uint32_t)TK_CAP) {
                const uint32_t lo_key = prefix << shift;
                if (tid == 0)
                    sh_cnt = 0u;
                __syncthreads();
                for (int64_t s = tid; s < n; s += TK_THREADS) {
                    const uint32_t key = score_key(row[s]);
                    if (key >= lo_key) {
                        const uint32_t pos = atomicAdd(&sh_cnt, 1u);
                        buf[pos] = composite(key, s);
                    }
                }
                __syncthreads();
                m = (int)count_ge;
                gathered = true;
                break;
            }
            __syncthreads();
        }
        if (!gathered) {
            // prefix is the exact threshold key tau; `above` keys exceed it and `need`
            // copies of tau are taken, lowest positions first.
            const uint32_t tau = prefix;
            if (tid == 0)
                sh_cnt = 0u;
            __syncthreads();
            for (int64_t s = tid; s < n; s += TK_THREADS) {
                const uint32_t key = score_key(row[s]);
                if (key > tau) {
                    const uint32_t pos = atomicAdd(&sh_cnt, 1u);
                    buf[pos] = composite(key, s);
                }
            }
            uint32_t taken = 0;
            for (int64_t base = 0; base < n && taken < need; base += TK_THREADS) {
                const int64_t s = base + tid;
                const uint32_t flag = (s < n && score_key(row[s]) == tau) ? 1u : 0u;
                uint32_t tot;
                const uint32_t rank = block_excl_scan(flag, wsum, &tot);
                if (flag && taken + rank < need)
                    buf[above + taken + rank] = composite(tau, s);
                taken += tot;
            }
            __syncthreads();
            m = (int)(above + need);
        }
    }

    // ---- sort and emit ------------------------------------------------------------------
    int m2 = 2;
    while (m2 < m)
        m2 <<= 1;
    for (int t = m + tid; t < m2; t += TK_THREADS)
        buf[t] = 0ull;  // below every real composite
    __syncthreads();
    bitonic_desc(buf, m2);
    for (int t = tid; t < k; t += TK_THREADS)
        orow[t] = t < kk ? (int32_t)(0xFFFFFFFFu - (uint32_t)(buf[t] & 0xFFFFFFFFull)) : -1;
}

hipError_t launch_topk(const LayoutDev &L, int64_t T, const float *scores, int64_t ld, int k,
                       int32_t *indices, hipStream_t stream)
{
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)T), dim3(TK_THREADS), 0, stream, L, scores, ld, k,
                       indices);
    return hipGetLastError();
}

}  // namespace dsa
