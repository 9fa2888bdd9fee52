// topk.hip -- per-row top-k with a deterministic order, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram: top-k = 2048 written as int32
// [tokens x 2048]; ATOM-side optimisations, stable_topk: ties must resolve the same
// way every time; caveats: with fewer than k visible tokens every token is taken.)
//
// Selection order: higher score first; equal scores (with -0 == +0) by lower position.
// Each score maps to a monotone 32-bit key (sign-flipped IEEE bits, -0 folded into +0) and
// each candidate to the 64-bit composite (key << 32) | ~position, which is unique per row,
// so "larger composite first" is exactly that order.  The selected set is written in
// ascending position order (the attention over it does not depend on the order, and the
// gathers it drives then walk the cache forwards).
//
// Method, per row of n scores (kk = min(k, n) are taken):
//  1. a histogram of the top 11 key bits gives the bin d that holds the kk-th largest key
//     and the count `above` of keys in higher bins;
//  2. every position whose bin is above d is marked in a bitmap (whole 32-bit words built
//     with one ballot per 64 positions, so no atomics); the keys in bin d (its "members")
//     are collected as composites;
//  3. an exact radix select over the members (11-bit digits below the first 11) finds the
//     (kk - above)-th largest; members at or above it are marked too;
//  4. a block scan over per-thread popcounts of consecutive bitmap words gives every marked
//     position its output slot.
// Three ways to run it:
//  DIRECT  rows of at most 32768 scores: one 1024-thread block per row holds its row in
//          registers and LDS and does everything; its histogram bins are equal-width value bins
//          over the row's range (see topk_direct_kernel), and it writes the output slots
//          from a block scan over the positions themselves, without a bitmap;
//  ROW     many rows (prefill): topk_hist_kernel builds the histogram with many blocks per
//          row; one block per row then reads its row once (bitmap in LDS);
//  MB      few long rows (decode): topk_hist_kernel, then topk_mark_kernel marks the bitmap
//          and collects the members with many blocks per row (global workspace), then one
//          block per row selects among the members and compacts.
// Integer atomics only; every result is bit-reproducible.  The kernels leave every byte of
// the workspace they wrote zero again, so it can be reused as is for any layout.  If a
// row's bin d holds more than 8192 keys (heavily tied scores), two more radix passes over
// the row find the exact kk-th key and its ties are taken in position order.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAP = 8192;          // members held in LDS (64 KB of composites)
constexpr int TK_BINS = 2048;         // 11-bit digits
constexpr int TK_ROW_BITS = 1 << 18;  // longest row of the ROW mode (32 KB LDS bitmap)
constexpr int TK_MB_ROWS = 512;       // up to this many rows, long rows use the MB mode
constexpr int TD_MAX_PER = 32;        // longest DIRECT row: 1024 threads x 32 = 32768 scores
constexpr int H_THREADS = 512;        // histogram kernel (256 threads x 8192 scores per block:
constexpr int H_CHUNK = 16384;        // IndexShare top-k 24.4 against 23.7 us)
constexpr int MK_THREADS = 1024;      // mark kernel: 16 waves per block (measured against
constexpr int MK_CHUNK = 16384;       // 256 x 8192, 512 x 8192 and 512 x 16384: all slower)

enum TkMode { TK_DIRECT = 0, TK_ROW = 1, TK_MB = 2 };

static int topk_mode(int64_t T, int64_t max_ctx)
{
    if (max_ctx <= (int64_t)TK_THREADS * TD_MAX_PER)
        return TK_DIRECT;
    if (T <= TK_MB_ROWS || max_ctx > TK_ROW_BITS)
        return TK_MB;
    return TK_ROW;
}

// Workspace of the ROW and MB modes (MB only: counters, bitmaps, member lists and picks).
struct TkWs {
    uint32_t *hist;  // [T][2048]
    uint32_t *cnt;   // [T]
    uint32_t *bits;  // [T][W]
    uint64_t *memb;  // [T][TK_CAP]
    uint32_t *pick;  // [T][2]: threshold bin d and the count above it, from the mark kernel
    int64_t W;       // bitmap words per row
};

static inline size_t al256(size_t x)
{
    return (x + 255) & ~(size_t)255;
}

size_t topk_workspace_bytes(int64_t T, int64_t max_ctx)
{
    const int mode = topk_mode(T, max_ctx);
    if (mode == TK_DIRECT)
        return 0;
    size_t b = al256((size_t)T * TK_BINS * 4);
    if (mode == TK_MB) {
        const size_t W = (size_t)((max_ctx + 31) / 32);
        b += al256((size_t)T * 4) + al256((size_t)T * W * 4) + al256((size_t)T * TK_CAP * 8) + al256((size_t)T * 8);
    }
    return b;
}

static TkWs carve(void *ws, int64_t T, int64_t max_ctx)
{
    TkWs w{};
    char *p = (char *)ws;
    w.W = (max_ctx + 31) / 32;
    w.hist = (uint32_t *)p;
    p += al256((size_t)T * TK_BINS * 4);
    w.cnt = (uint32_t *)p;
    p += al256((size_t)T * 4);
    w.bits = (uint32_t *)p;
    p += al256((size_t)T * w.W * 4);
    w.memb = (uint64_t *)p;
    p += al256((size_t)T * TK_CAP * 8);
    w.pick = (uint32_t *)p;  // MB mode only (the ROW mode's workspace ends at hist)
    return w;
}


__device__ __forceinline__ uint64_t composite(uint32_t key, int64_t s)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s);
}

__device__ __forceinline__ uint32_t comp_pos(uint64_t v)
{
    return 0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull);
}

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS round trips): shifts of
// 1, 2, 4, 8 inside each 16-lane row, then lane 15 of each row added into the next row
// (rows 1, 3) and lane 31 into rows 2, 3.  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive scan over the block (one value per thread, thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t x = wave_incl_scan(v, lane);
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


// Given a histogram of NB bins (a power of two, 256 .. 2048) and the number still needed
// (1 <= need <= total), find the bin holding the need-th largest entry: the bin, the count
// strictly above it and its own count.  Wave 0 works it out (lane l owns the NB/64 bins
// below NB - (NB/64) l, read as 16-byte vectors; a second scan resolves the bin inside the
// chosen lane's range); the result is broadcast through sh after a barrier that every
// thread of the block takes.
struct DigitPick {
    uint32_t digit, above, count;
};
// Barrier that waits only for this wave's LDS traffic (global loads stay in flight).
__device__ __forceinline__ void lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int NB>
__device__ __forceinline__ DigitPick pick_digit(const uint32_t *hist, uint32_t need, uint32_t *sh)
{
    static_assert(NB >= 256 && (NB & (NB - 1)) == 0, "bins");
    constexpr int PER = NB / 64, Q = PER / 4;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int lo = NB - PER * (lane + 1);  // lowest bin of this lane
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const u32x4 v = *(const u32x4 *)(hist + lo + 4 * ((q + lane) % Q));  // rotated
            c += v[0] + v[1] + v[2] + v[3];
        }
        const uint32_t incl = wave_incl_scan(c, lane);
        const uint64_t hit = __ballot(incl - c < need && need <= incl);
        const int L = hit ? __ffsll((long long)hit) - 1 : 0;  // one lane holds it (need <= total)
        const uint32_t exL = __shfl(incl - c, L, 64);
        const int topL = NB - 1 - PER * L;
        const uint32_t h = lane < PER ? hist[topL - lane] : 0u;
        const uint32_t inc2 = wave_incl_scan(h, lane);
        if (lane < PER && exL + inc2 - h < need && need <= exL + inc2) {
            sh[0] = (uint32_t)(topL - lane);
            sh[1] = exL + inc2 - h;
            sh[2] = h;
        }
    }
    lds_sync();
    return DigitPick{sh[0], sh[1], sh[2]};
}

// Four consecutive scores s .. s+3 of a row (zeros past n): one 16-byte load when aligned.
__device__ __forceinline__ f32x4 load4(const float *row, int64_t s, int64_t n)
{
    if (s + 3 < n && ((uintptr_t)(row + s) & 15) == 0)
        return *(const f32x4 *)(row + s);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        v[e] = s + e < n ? row[s + e] : 0.f;
    return v;
}

// One wave over positions base .. base+255 (base a multiple of 256; lane l holds base+4l ..
// +3): the bitmap words of the positions whose bin is above d (lanes 8w'.. 8w'+7 build word
// w' with three DPP moves; no atomics), and the keys of bin d either handed to store_member
// per element (a ballot and the lane's rank among the wave's members) or, with note_member
// given, only flagged per lane and element, for the caller to reserve once per wave.
struct NoNote {
    __device__ void operator()(int, bool) const {}
};
template <typename WordStore, typename MemberStore, typename MemberNote = NoNote>
__device__ __forceinline__ void take_wave(int64_t base, const f32x4 &x, int64_t n, uint32_t d, int lane,
                                          WordStore store_word, MemberStore store_member,
                                          MemberNote note_member = NoNote())
{
    const int64_t s0 = base + 4 * lane;
    uint32_t key[4], nib = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        key[e] = score_key(x[e]);
        if (s0 + e < n && (key[e] >> 21) > d)
            nib |= 1u << e;
    }
    // OR over each group of 8 lanes with DPP moves: the quad, then row_shr:4 (lanes 4-7 and
    // 12-15 of each 16-lane row then hold their 8-lane group's word)
    uint32_t word = nib << (4 * (lane & 7));
    word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xf, 0xf, false);  // quad_perm 1,0,3,2
    word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x4E, 0xf, 0xf, false);  // quad_perm 2,3,0,1
    word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x114, 0xf, 0xf, true);  // row_shr:4
    if ((lane & 7) == 7 && base + 32 * (lane >> 3) < n)
        store_word((base >> 5) + (lane >> 3), word);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool m = s0 + e < n && (key[e] >> 21) == d;
        if constexpr (std::is_same<MemberNote, NoNote>::value) {
            const uint64_t mb = __ballot(m);
            if (mb)
                store_member(mb, (uint32_t)__popcll(mb & below), m, composite(key[e], s0 + e));
        } else {
            note_member(e, m);
        }
    }
}

// ------------------------------------------------------------------------------------------
// K1: per-row histogram of the top 11 key bits (ROW and MB modes)
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
    constexpr int U = H_CHUNK / (4 * H_THREADS);  // 8 vectors per thread, all in flight
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = load4(row, s0 + 4 * (u * H_THREADS + tid), s1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t s = s0 + 4 * (u * H_THREADS + tid);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (s + e < s1)
                atomicAdd(&lh[wave][score_key(v[u][e]) >> 21], 1u);
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
// K2 (MB mode): mark the bitmap words and collect the members of one 16384-score chunk
// ------------------------------------------------------------------------------------------
template <bool AL16>  // every row 16-byte aligned (scores and ld): 16-byte loads
__global__ __launch_bounds__(MK_THREADS) void topk_mark_kernel(LayoutDev L, const float *__restrict__ scores,
                                                              int64_t ld, int k, TkWs ws)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS];
    __shared__ uint64_t lmem[MK_CHUNK];  // this chunk's members, before one reservation
    __shared__ uint32_t sh[4];
    __shared__ uint32_t lcnt, gbase;
    const int64_t i = blockIdx.y;
    const RowInfo r = row_info(L, i);
    const int64_t n = r.n > 0 ? r.n : 0;
    const int64_t s0 = (int64_t)blockIdx.x * MK_CHUNK;
    if (s0 >= n)
        return;
    const uint32_t kk = (uint32_t)min((int64_t)k, n);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *row = scores + i * ld;
    uint32_t *bits = ws.bits + i * ws.W;
    // the row's histogram first, then this chunk's scores: waiting for the histogram (in
    // issue order) leaves the score loads in flight through the digit pick
    const uint32_t *gh = ws.hist + i * TK_BINS;
    constexpr int HB = TK_BINS / MK_THREADS;
    uint32_t hv[HB];
#pragma unroll
    for (int e = 0; e < HB; ++e)
        hv[e] = gh[e * MK_THREADS + tid];
    constexpr int U = MK_CHUNK / (4 * MK_THREADS);  // 8 wave steps of 256 positions
    // unconditional buffer loads (zeros past n): the wait for the histogram above then leaves
    // every score load in flight through the digit pick
    const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(
        (void *)row, (short)0, __builtin_amdgcn_readfirstlane((int)(uint32_t)(n * 4)), 0x00020000);
    f32x4 v[U];
    if constexpr (AL16) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = (int)(s0 + (int64_t)u * 4 * MK_THREADS) + 256 * wave + 4 * lane;
            v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrow, 4 * sp, 0, 0));
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = (int)(s0 + (int64_t)u * 4 * MK_THREADS) + 256 * wave + 4 * lane;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrow, 4 * (sp + e), 0, 0));
        }
    }
#pragma unroll
    for (int e = 0; e < HB; ++e)
        hist[e * MK_THREADS + tid] = hv[e];
    if (tid == 0)
        lcnt = 0u;
    lds_sync();
    const DigitPick pk = pick_digit<TK_BINS>(hist, kk, sh);
    const uint32_t d = pk.digit;
    if (blockIdx.x == 0 && tid == 0) {  // handed to the select kernel, which then skips the pick
        ws.pick[2 * i] = d;
        ws.pick[2 * i + 1] = pk.above;
    }

    // bitmap words of this chunk; the members of bin d are noted per lane (bit 4u + e) and
    // appended to lmem with one LDS reservation per wave, in (lane, u, e) order
    // (unconditional: take_wave writes no word and notes no member at or past n, and a branch
    // here would leave the compiler unsure whether the scores had arrived, so that it waited
    // for them again below, behind the reservation)
    uint32_t mflag = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t base = s0 + (int64_t)u * 4 * MK_THREADS + 256 * wave;
        take_wave(
            base, v[u], n, d, lane, [&](int64_t w, uint32_t word) { bits[w] = word; },
            [&](uint64_t, uint32_t, bool m, uint64_t) {},
            [&](int e, bool m) { mflag |= (m ? 1u : 0u) << (4 * u + e); });
    }
    const uint32_t mc = (uint32_t)__popc(mflag);
    const uint32_t incl = wave_incl_scan(mc, lane);
    uint32_t wbase = 0;
    if (lane == 63 && incl != 0u)
        wbase = atomicAdd(&lcnt, incl);
    __syncthreads();  // every wave has reserved its slots: lcnt is the block's member count
    // one reservation per block in the row's member list (a device-wide atomic, whose
    // latency the members' copy to LDS overlaps), then a coalesced copy
    const uint32_t m = lcnt;
    if (m == 0u)
        return;
    uint32_t gb = 0;
    if (tid == 0) {
        // an address the compiler cannot prove uniform: it then issues the plain atomic, not
        // its wave-reduction form, which consumes the result (waits for it) on the spot
        int zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
        gb = atomicAdd(ws.cnt + i + zero, m);
    }
    uint32_t at = (uint32_t)__shfl((int)wbase, 63, 64) + incl - mc;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((mflag >> (4 * u + e)) & 1u)  // at < MK_CHUNK: one slot per position
                lmem[at++] = composite(score_key(v[u][e]), s0 + (int64_t)u * 4 * MK_THREADS + 256 * wave + 4 * lane + e);
    if (tid == 0)
        gbase = gb;
    __syncthreads();
    uint64_t *memb = ws.memb + i * TK_CAP;
    for (uint32_t e = tid; e < m; e += MK_THREADS) {
        const uint32_t at = gbase + e;
        if (at < (uint32_t)TK_CAP)
            memb[at] = lmem[e];
    }
}

// ------------------------------------------------------------------------------------------
// DIRECT mode: rows of at most 1024 PER scores (PER = 8, 16, 32, in registers), one
// 1024-thread block per row, which reads its row once.  Thread t owns the positions
// 4096 q + 4 t + e (q < PER / 4, e < 4): every load instruction reads 1 KB of consecutive
// scores.
//  1. the row's minimum and maximum cut [min, max] into 2048 bins of equal width; the bin of
//     a score, trunc((x - min) * 2048 / (max - min)) clamped to 2047, never decreases as the
//     score grows (each rounding step is monotone), so every score in a bin above the
//     threshold bin d is taken and none below it.  A row whose range is zero or not finite
//     uses the top 11 key bits instead (also monotone).  Equal-width bins spread typical
//     score rows far more evenly than the exponent-led key bits, so the LDS histogram
//     atomics rarely collide and bin d holds only a handful of members;
//  2. the members of bin d go to LDS as composites (up to CAP of them), and the
//     (kk - above)-th largest is found by counting (up to TD_COUNT members) or by an MSD radix
//     select over the composites (from LDS, or recomputed from the row when bin d holds more
//     than CAP members);
//  3. each thread marks its taken positions per group q (by composite alone when step 2
//     found an exact member, else by bin and composite); wave scans and one scan over the
//     (q, wave) totals give every position its output slot: ascending position order.
// ------------------------------------------------------------------------------------------
constexpr uint32_t TD_COUNT = 256;  // members ranked by counting up to this many

// Maximum / minimum over the 64 lanes of a wave, returned as a wave-uniform value: the DPP
// pattern of wave_incl_scan with max / min (lanes without a source read the identity), and
// lane 63 holds the result.
__device__ __forceinline__ float wave_max_f32(float x)
{
    constexpr int ID = (int)0xff800000u;  // -inf
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x111, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x112, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x114, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x118, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x142, 0xa, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float wave_min_f32(float x)
{
    constexpr int ID = (int)0x7f800000u;  // +inf
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x111, 0xf, 0xf, false)));
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x112, 0xf, 0xf, false)));
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x114, 0xf, 0xf, false)));
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x118, 0xf, 0xf, false)));
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x142, 0xa, 0xf, false)));
    x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(ID, __float_as_int(x), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// A block-uniform value made visibly uniform to the compiler (so branches on it are scalar).
__device__ __forceinline__ uint32_t uni(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ float uni(float x)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <int PER>
__global__ __launch_bounds__(TK_THREADS) void topk_direct_kernel(LayoutDev L, const float *__restrict__ scores,
                                                                 int64_t ld, int k, int32_t *__restrict__ out)
{
    static_assert(PER % 4 == 0 && PER >= 8 && PER <= TD_MAX_PER, "positions per thread");
    constexpr int NQ = PER / 4;                      // groups of 4 positions per thread
    constexpr int GROUP = 4 * TK_THREADS;            // positions per group (4096)
    constexpr int NB = NQ * TK_WAVES;                // (group, wave) totals
    constexpr int CAP = 2048;                        // members held in LDS (value bins: ~20 per row)
    constexpr int HC = 4;                            // histogram copies, one per lane & 3
    constexpr int HS = TK_BINS + 4;                  // copy stride: + a bin for positions past n
    static_assert(PER <= 32, "per-thread masks are 32 bits");
    __shared__ uint64_t cand[CAP];
    __shared__ __attribute__((aligned(16))) uint32_t hist[HC * HS];
    __shared__ float red[2][TK_WAVES];
    __shared__ uint32_t base[NB];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t sh_cnt;
    __shared__ uint64_t sh_lo;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t i = blockIdx.x;
    const RowInfo r = row_info(L, i);
    const int n32 = (int)uni((uint32_t)min(r.n > 0 ? r.n : (int64_t)0, (int64_t)TK_THREADS * PER));  // host: n <= 1024 PER
    int32_t *orow = out + i * k;
    const uint32_t kk = (uint32_t)min(k, n32);
    if (kk == 0) {
        for (int t = tid; t < k; t += TK_THREADS)
            orow[t] = -1;
        return;
    }
    const float *row = scores + i * ld;
    auto pos = [&](int q, int e) -> int { return GROUP * q + 4 * tid + e; };
    // bit 4q + e: position pos(q, e) is inside the row
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            valid |= (pos(q, e) < n32 ? 1u : 0u) << (4 * q + e);

    // ---- 0. the row, in registers: four dword loads per group through a buffer resource over
    // the n scores (zeros past the end), all issued before any is used.
    const __amdgpu_buffer_rsrc_t rrow =
        __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, n32 * 4, 0x00020000);
    auto load_group = [&](int q) -> f32x4 {
        const int p = pos(q, 0);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrow, 4 * (p + e), 0, 0));
        return v;
    };
    f32x4 xr[NQ];
    auto get = [&](int q) -> f32x4 { return xr[q]; };
    float mx = -INFINITY, mn = INFINITY;
    auto range_of = [&](const f32x4 &v, int q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = (valid >> (4 * q + e)) & 1u;
            mx = fmaxf(mx, ok ? v[e] : -INFINITY);
            mn = fminf(mn, ok ? v[e] : INFINITY);
        }
    };
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        xr[q] = load_group(q);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        range_of(xr[q], q);

    // ---- 1. range of the row, histogram of the value bins
    mx = wave_max_f32(mx);
    mn = wave_min_f32(mn);
    if (lane == 0) {
        red[0][wave] = mx;
        red[1][wave] = mn;
    }
    for (int b = tid; b < HC * HS; b += TK_THREADS)
        hist[b] = 0u;
    if (tid == 0)
        sh_cnt = 0u;
    __syncthreads();
    mx = red[0][0];
    mn = red[1][0];
#pragma unroll
    for (int w2 = 1; w2 < TK_WAVES; ++w2) {
        mx = fmaxf(mx, red[0][w2]);
        mn = fminf(mn, red[1][w2]);
    }
    mx = uni(mx);
    mn = uni(mn);
    const float range = mx - mn;
    float scale = 0.f;
    bool lin = range > 0.f && range < INFINITY;
    if (lin) {
        scale = (float)TK_BINS / range;
        lin = scale < INFINITY;
    }
    lin = uni(lin ? 1u : 0u) != 0u;
    scale = uni(scale);
    // The two bin functions, each straight-line; every pass below is instantiated for both
    // under one block-uniform branch, so no per-score branch is left.
    auto bin_lin = [&](float v) -> uint32_t { return min((uint32_t)((v - mn) * scale), (uint32_t)(TK_BINS - 1)); };
    auto bin_key = [&](float v) -> uint32_t { return score_key(v) >> 21; };
    auto with_bins = [&](auto &&pass) {
        if (lin)
            pass(bin_lin);
        else
            pass(bin_key);
    };
    // positions past n count into the spare bin TK_BINS (never read).  Scores crowd a few
    // bins near the row's mode, so the lanes of a wave add into four copies of the histogram
    // (lane & 3) to cut the LDS atomic collisions, then the copies are summed.
    uint32_t *hcopy = hist + (lane & 3) * HS;
    with_bins([&](auto bin_of) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f32x4 v = get(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t b = bin_of(v[e]);
                atomicAdd(&hcopy[((valid >> (4 * q + e)) & 1u) ? b : (uint32_t)TK_BINS], 1u);
            }
        }
    });
    __syncthreads();
    for (int b = tid; b < TK_BINS; b += TK_THREADS)
        hist[b] += hist[HS + b] + hist[2 * HS + b] + hist[3 * HS + b];
    __syncthreads();
    const DigitPick p0 = pick_digit<TK_BINS>(hist, kk, sh);
    const uint32_t d = uni(p0.digit), c = uni(p0.count);
    const uint32_t need = kk - uni(p0.above);  // 1 .. c members of bin d are taken

    // ---- 2. members of bin d into cand (a handful per row: one counter atomic each)
    const bool in_lds = c <= (uint32_t)CAP;
    uint32_t memb = 0;  // bit 4q + e: position pos(q, e) is a member of bin d
    if (need < c) {  // block-uniform
        with_bins([&](auto bin_of) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 v = get(q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    memb |= (bin_of(v[e]) == d ? 1u : 0u) << (4 * q + e);
            }
        });
        memb &= valid;
        if (in_lds) {
            if (memb) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const f32x4 v = get(q);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if ((memb >> (4 * q + e)) & 1u)
                            cand[atomicAdd(&sh_cnt, 1u)] = composite(score_key(v[e]), pos(q, e));
                }
            }
            __syncthreads();
        }
    }

    // ---- 3. lo: the need-th largest member (every member >= lo is taken)
    uint64_t lo = 0;
    const bool exact = need < c && in_lds && c <= TD_COUNT;  // lo is then a member's composite
    if (need < c) {
        if (exact) {
            if ((uint32_t)tid < c) {
                const uint64_t v = cand[tid];
                uint32_t above = 0;
                for (uint32_t u = 0; u < c; ++u)
                    above += cand[u] > v ? 1u : 0u;
                if (above == need - 1u)  // composites are unique: exactly one member
                    sh_lo = v;
            }
            __syncthreads();
            lo = sh_lo;
        } else {
            // MSD radix select over the 64-bit composites of the members: 11-bit digits from
            // the top, over cand or (too many members for it) over the row
            uint64_t prefix = 0;
            uint32_t nd = need;
            int shift = 64;
            while (true) {
                const int width = shift >= 11 ? 11 : shift;
                const int nshift = shift - width;
                const uint32_t nb = 1u << width;
                for (uint32_t b = tid; b < nb; b += TK_THREADS)
                    hist[b] = 0u;
                __syncthreads();
                auto count = [&](uint64_t v) {
                    if (shift == 64 || (v >> shift) == prefix)
                        atomicAdd(&hist[(uint32_t)((v >> nshift) & (uint64_t)(nb - 1))], 1u);
                };
                if (in_lds) {
                    for (uint32_t e = tid; e < c; e += TK_THREADS)
                        count(cand[e]);
                } else if (memb) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const f32x4 v = get(q);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if ((memb >> (4 * q + e)) & 1u)
                                count(composite(score_key(v[e]), pos(q, e)));
                    }
                }
                __syncthreads();
                const DigitPick p = nb == (uint32_t)TK_BINS ? pick_digit<TK_BINS>(hist, nd, sh)
                                                              : pick_digit<512>(hist, nd, sh);
                prefix = (prefix << width) | uni(p.digit);
                nd -= uni(p.above);
                shift = nshift;
                if (uni(p.count) == nd || shift == 0) {  // the whole sub-bin is taken
                    lo = prefix << shift;
                    break;
                }
            }
        }
    }
    lo = ((uint64_t)uni((uint32_t)(lo >> 32)) << 32) | uni((uint32_t)lo);

    // ---- 4. output slots in position order: group q of wave w starts at base[q][w].  With an
    // exact lo (a member's composite) the taken set is simply {composite >= lo}: every score of
    // a higher bin is larger than every member, every score of a lower bin smaller.
    // composite >= lo  <=>  x > x_lo, or x == x_lo at a position <= p_lo (float compares: -0 == +0
    // as for the keys; no NaN).  need == c takes the whole bin d and everything above it.
    const uint32_t lo_key = (uint32_t)(lo >> 32);
    const float x_lo = __uint_as_float((lo_key & 0x80000000u) ? (lo_key & 0x7FFFFFFFu) : ~lo_key);
    const int p_lo = (int)comp_pos(lo);
    uint32_t takes = 0;  // bit 4q + e: position pos(q, e) is taken
    if (exact) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f32x4 v = get(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool t = (v[e] > x_lo) | ((v[e] == x_lo) & (pos(q, e) <= p_lo));
                takes |= (t ? 1u : 0u) << (4 * q + e);
            }
        }
    } else {
        with_bins([&](auto bin_of) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 v = get(q);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t bn = bin_of(v[e]);
                    const bool t = (bn > d) | ((bn == d) & (composite(score_key(v[e]), pos(q, e)) >= lo));
                    takes |= (t ? 1u : 0u) << (4 * q + e);
                }
            }
        });
    }
    takes &= valid;
    uint32_t incl[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        incl[q] = wave_incl_scan((uint32_t)__popc((takes >> (4 * q)) & 15u), lane);
        if (lane == 63)
            base[q * TK_WAVES + wave] = incl[q];
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the NB totals in (group, wave) order
        constexpr int PL = (NB + 63) / 64;  // consecutive entries per lane
        uint32_t v[PL], s = 0;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int e = PL * lane + u;
            v[u] = e < NB ? base[e] : 0u;
            s += v[u];
        }
        uint32_t run = wave_incl_scan(s, lane) - s;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int e = PL * lane + u;
            if (e < NB)
                base[e] = run;
            run += v[u];
        }
    }
    __syncthreads();
    // Paged caches list physical rows.  When the page size is a multiple of 4 the four
    // positions of a group (which starts at a multiple of 4) share one page: one block-table
    // lookup per group, all issued before the stores (clamped into the row, so always valid).
    const bool quad_pages = L.block_table != nullptr && (L.page_size & 3) == 0;
    int32_t qrow[NQ];
    if (quad_pages) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            qrow[q] = (int32_t)token_row(L, r.b, 0, min(pos(q, 0), n32 - 1));
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const uint32_t m = (takes >> (4 * q)) & 15u, cnt = (uint32_t)__popc(m);
        uint32_t slot = base[q * TK_WAVES + wave] + incl[q] - cnt;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((m >> e) & 1u)
                orow[slot++] = quad_pages ? qrow[q] + e : (int32_t)token_row(L, r.b, 0, pos(q, e));
    }
    for (int t = (int)kk + tid; t < k; t += TK_THREADS)
        orow[t] = -1;
}

// ------------------------------------------------------------------------------------------
// K3 (ROW and MB modes): exact selection and ordered output, one 1024-thread block per row
// ------------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(TK_THREADS) void topk_select_kernel(LayoutDev L, const float *__restrict__ scores,
                                                                 int64_t ld, int k, int32_t *__restrict__ out,
                                                                 TkWs ws)
{
    __shared__ uint64_t cand[TK_CAP];
    __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS + 4];  // + a spare slot (see step 4)
    __shared__ uint32_t wsum[TK_WAVES];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t sh_cnt;
    extern __shared__ uint32_t bmap_lds[];  // the row's bitmap (ROW, and MB rows that fit)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t i = blockIdx.x;
    const RowInfo r = row_info(L, i);
    const int64_t n = r.n > 0 ? r.n : 0;
    const float *row = scores + i * ld;
    int32_t *orow = out + i * k;
    const uint32_t kk = (uint32_t)min((int64_t)k, n);
    if (kk == 0) {
        for (int t = tid; t < k; t += TK_THREADS)
            orow[t] = -1;
        return;
    }
    const int nw = (int)((n + 31) >> 5);
    // MB rows keep their bitmap in global memory unless it fits the LDS one
    const bool gbm = MODE == TK_MB && ws.W > TK_ROW_BITS / 32;
    uint32_t *gbits = ws.bits + i * ws.W;
    // bitmap access through typed pointers (a generic one would turn every LDS access into a
    // flat access waited for on its own)
    auto bm_or = [&](int64_t w, uint32_t bit) {
        if (gbm)
            atomicOr(&gbits[w], bit);
        else
            atomicOr(&bmap_lds[w], bit);
    };

    // MB: the member count, the bitmap words and the members (written by topk_mark_kernel) are
    // requested first, so their latency overlaps the histogram's and the digit pick
    constexpr int PB = TK_ROW_BITS / 32 / TK_THREADS, PM = TK_CAP / TK_THREADS;
    uint32_t bw[PB];
    uint64_t mv[PM];
    uint32_t c = 0;  // members of bin d
    if (MODE == TK_MB) {
        c = ws.cnt[i];
        if (!gbm) {
            const uint32_t *g = ws.bits + i * ws.W;
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const int w = tid + TK_THREADS * q;
                bw[q] = w < nw ? g[w] : 0u;
            }
        }
        const uint64_t *memb = ws.memb + i * TK_CAP;
        const uint32_t cm = min(c, (uint32_t)TK_CAP);
#pragma unroll
        for (int q = 0; q < PM; ++q) {
            const uint32_t e = tid + TK_THREADS * q;
            mv[q] = e < cm ? memb[e] : 0ull;
        }
    }

    // ---- 1. threshold bin d from the histogram of the top 11 key bits (MB: as the mark
    // kernel picked it from the same histogram)
    if (tid == 0)
        sh_cnt = 0u;
    uint32_t d, above;
    if (MODE == TK_MB) {
        d = ws.pick[2 * i];
        above = ws.pick[2 * i + 1];
        uint32_t *gh = ws.hist + i * TK_BINS;
        for (int b = tid; b < TK_BINS; b += TK_THREADS)
            gh[b] = 0u;  // the workspace is left zero for the next call
    } else {
        for (int b = tid; b < TK_BINS; b += TK_THREADS) {
            uint32_t *gh = ws.hist + i * TK_BINS;
            hist[b] = gh[b];
            gh[b] = 0u;
        }
        __syncthreads();
        const DigitPick p0 = pick_digit<TK_BINS>(hist, kk, sh);
        d = p0.digit;
        above = p0.above;
    }
    const uint32_t need = kk - above;  // 1 .. (count of bin d) members of bin d are taken

    // ---- 2. bitmap of the positions above bin d; members of bin d into cand
    if (MODE == TK_ROW) {
        constexpr int U = 4;  // 4 vectors per thread: 16384 positions per round
#pragma unroll 1
        for (int64_t b0 = 0; b0 < n; b0 += (int64_t)U * 4 * TK_THREADS) {
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = load4(row, b0 + (int64_t)u * 4 * TK_THREADS + 256 * wave + 4 * lane, n);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t base = b0 + (int64_t)u * 4 * TK_THREADS + 256 * wave;
                if (base < n)
                    take_wave(
                        base, v[u], n, d, lane, [&](int64_t w, uint32_t word) { bmap_lds[w] = word; },
                        [&](uint64_t mb, uint32_t rank, bool m, uint64_t comp) {
                            uint32_t at = 0;
                            if (lane == 0)
                                at = atomicAdd(&sh_cnt, (uint32_t)__popcll(mb));
                            at = (uint32_t)__builtin_amdgcn_readfirstlane((int)at) + rank;
                            if (m && at < (uint32_t)TK_CAP)
                                cand[at] = comp;
                        });
            }
        }
        __syncthreads();
        c = sh_cnt;
    } else {
        if (!gbm) {  // the bitmap into LDS, the global words left zero
            uint32_t *g = ws.bits + i * ws.W;
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                const int w = tid + TK_THREADS * q;
                if (w < nw) {
                    bmap_lds[w] = bw[q];
                    g[w] = 0u;
                }
            }
        }
        uint64_t *memb = ws.memb + i * TK_CAP;
#pragma unroll
        for (int q = 0; q < PM; ++q) {
            const uint32_t e = tid + TK_THREADS * q;
            if (e < min(c, (uint32_t)TK_CAP)) {
                if (c <= (uint32_t)TK_CAP)
                    cand[e] = mv[q];
                memb[e] = 0ull;  // everything this call wrote is left zero for the next one
            }
        }
        __syncthreads();
        if (tid == 0) {
            ws.cnt[i] = 0u;
            ws.pick[2 * i] = ws.pick[2 * i + 1] = 0u;
        }
    }

    // ---- 3. the need-th largest member; it and every member above it are marked
    if (c <= (uint32_t)TK_CAP) {
        uint64_t lo = 0;  // every selected member is >= lo
        if (need < c) {
            uint64_t prefix = d;
            uint32_t nd = need;
            int shift = 53;
            while (true) {
                const int width = shift >= 11 ? 11 : shift;
                const int nshift = shift - width;
                const int nb = 1 << width;
                for (int b = tid; b < nb; b += TK_THREADS)
                    hist[b] = 0u;
                __syncthreads();
                for (uint32_t e = tid; e < c; e += TK_THREADS) {
                    const uint64_t v = cand[e];
                    if ((v >> shift) == prefix)
                        atomicAdd(&hist[(uint32_t)((v >> nshift) & (uint64_t)(nb - 1))], 1u);
                }
                __syncthreads();
                const DigitPick p = nb == TK_BINS ? pick_digit<TK_BINS>(hist, nd, sh) : pick_digit<512>(hist, nd, sh);
                prefix = (prefix << width) | p.digit;
                nd -= p.above;
                shift = nshift;
                if (p.count == nd || shift == 0) {  // the whole sub-bin is taken
                    lo = prefix << shift;
                    break;
                }
            }
        }
        for (uint32_t e = tid; e < c; e += TK_THREADS) {
            const uint64_t v = cand[e];
            if (v >= lo) {
                const uint32_t pos = comp_pos(v);
                bm_or(pos >> 5, 1u << (pos & 31));
            }
        }
    } else {
        // Bin d holds more than TK_CAP keys: find the exact kk-th key tau with two more
        // radix passes over the row, mark the keys of bin d above tau, then the first ties
        // of tau in position order.
        uint32_t prefix = d, nd = need;
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
            const DigitPick p = width == 11 ? pick_digit<TK_BINS>(hist, nd, sh) : pick_digit<1024>(hist, nd, sh);
            nd -= p.above;
            prefix = (prefix << width) | p.digit;
            shift = nshift;
        }
        const uint32_t tau = prefix;
        for (int64_t s = tid; s < n; s += TK_THREADS) {
            const uint32_t key = score_key(row[s]);
            if ((key >> 21) == d && key > tau)
                bm_or(s >> 5, 1u << (s & 31));
        }
        uint32_t taken = 0;
        for (int64_t b0 = 0; b0 < n && taken < nd; b0 += TK_THREADS) {
            const int64_t s = b0 + tid;
            const uint32_t flag = (s < n && score_key(row[s]) == tau) ? 1u : 0u;
            uint32_t tot;
            const uint32_t rank = block_excl_scan(flag, wsum, &tot);
            if (flag && taken + rank < nd)
                bm_or(s >> 5, 1u << (s & 31));
            taken += tot;
        }
    }
    __syncthreads();

    // ---- 4. ordered output: per-thread popcounts of consecutive words, a block scan, then
    // every set bit its slot (staged in hist: kk <= 2048 slots)
    static_assert(TK_BINS >= DSA_TOPK_MAX, "staging area");
    uint32_t *slots = hist;
    const int wpt = (nw + TK_THREADS - 1) / TK_THREADS;
    const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    auto word = [&](int w) -> uint32_t {
        if (gbm)  // written by other CUs and by atomics: read past the L1
            return __hip_atomic_load(&gbits[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return bmap_lds[w];
    };
    uint32_t cnt_mine = 0;
    if (!gbm) {
        // LDS bitmap (at most 8192 words): this thread's words read once into registers, so
        // that neither pass waits on memory per word
        constexpr int WPT = TK_ROW_BITS / 32 / TK_THREADS;
        uint32_t wv[WPT];
#pragma unroll
        for (int q = 0; q < WPT; ++q)
            wv[q] = w0 + q < w1 ? bmap_lds[w0 + q] : 0u;
#pragma unroll
        for (int q = 0; q < WPT; ++q)
            cnt_mine += __popc(wv[q]);
        uint32_t tot;
        uint32_t slot = block_excl_scan(cnt_mine, wsum, &tot);
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            uint32_t b = wv[q];
            while (b) {  // slots past the k kept ones go to the spare entry: no branch
                slots[min(slot, (uint32_t)TK_BINS)] = (uint32_t)(32 * (w0 + q) + __ffs(b) - 1);
                ++slot;
                b &= b - 1u;
            }
        }
    } else {
        for (int w = w0; w < w1; ++w)
            cnt_mine += __popc(word(w));
        uint32_t tot;
        uint32_t slot = block_excl_scan(cnt_mine, wsum, &tot);
        for (int w = w0; w < w1; ++w) {
            uint32_t b = word(w);
            gbits[w] = 0u;  // left zero for the next call
            while (b) {
                slots[min(slot, (uint32_t)TK_BINS)] = (uint32_t)(32 * w + __ffs(b) - 1);
                ++slot;
                b &= b - 1u;
            }
        }
    }
    __syncthreads();
    for (int t = tid; t < k; t += TK_THREADS)  // positions, or physical rows (paged caches)
        orow[t] = (uint32_t)t < kk ? (int32_t)token_row(L, r.b, 0, (int64_t)slots[t]) : -1;
}

// ------------------------------------------------------------------------------------------
uint32_t *topk_hist_of(void *workspace, int64_t T, int64_t max_ctx)
{
    return topk_mode(T, max_ctx) == TK_DIRECT ? nullptr : carve(workspace, T, max_ctx).hist;
}

hipError_t launch_topk(const LayoutDev &L, int64_t T, int64_t max_ctx, const float *scores, int64_t ld,
                       int k, int32_t *indices, void *workspace, hipStream_t stream, bool hist_ready)
{
    const int mode = topk_mode(T, max_ctx);
    const TkWs ws = mode == TK_DIRECT ? TkWs{} : carve(workspace, T, max_ctx);
    const dim3 hgrid((unsigned)((max_ctx + H_CHUNK - 1) / H_CHUNK), (unsigned)T);
    if (mode != TK_DIRECT && !hist_ready) {
        hipLaunchKernelGGL(topk_hist_kernel, hgrid, dim3(H_THREADS), 0, stream, L, scores, ld, ws.hist);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (mode == TK_MB) {
        const dim3 mgrid((unsigned)((max_ctx + MK_CHUNK - 1) / MK_CHUNK), (unsigned)T);
        if (((uintptr_t)scores & 15) == 0 && (ld & 3) == 0)
            hipLaunchKernelGGL(topk_mark_kernel<true>, mgrid, dim3(MK_THREADS), 0, stream, L, scores, ld, k, ws);
        else
            hipLaunchKernelGGL(topk_mark_kernel<false>, mgrid, dim3(MK_THREADS), 0, stream, L, scores, ld, k, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const size_t dyn = max_ctx <= TK_ROW_BITS ? (size_t)((max_ctx + 31) / 32) * 4 : 0;
    if (mode == TK_DIRECT) {
        const dim3 g((unsigned)T), b(TK_THREADS);
        if (max_ctx <= 8 * TK_THREADS)
            hipLaunchKernelGGL((topk_direct_kernel<8>), g, b, 0, stream, L, scores, ld, k, indices);
        else if (max_ctx <= 16 * TK_THREADS)
            hipLaunchKernelGGL((topk_direct_kernel<16>), g, b, 0, stream, L, scores, ld, k, indices);
        else
            hipLaunchKernelGGL((topk_direct_kernel<32>), g, b, 0, stream, L, scores, ld, k, indices);
    } else if (mode == TK_ROW)
        hipLaunchKernelGGL(topk_select_kernel<TK_ROW>, dim3((unsigned)T), dim3(TK_THREADS), dyn, stream, L,
                           scores, ld, k, indices, ws);
    else
        hipLaunchKernelGGL(topk_select_kernel<TK_MB>, dim3((unsigned)T), dim3(TK_THREADS), dyn, stream, L,
                           scores, ld, k, indices, ws);
    return hipGetLastError();
}

}  // namespace dsa
