// sparse_mla.hip -- sparse MLA over the selected latent rows, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram, sparse MLA box: 64 heads computed only on
// the 2048 selected rows of the 576-wide latent cache, 512 latent + 64 rope; layer
// scheduling: shared layers read the same index buffer.)  Absorbed form: the key is the
// whole 576-wide row, the value its first 512 entries, the output stays in latent space.
//
//   z_j = sm_scale * kv_scale * q_h . c_j ;  o_h = kv_scale * sum_j softmax(z)_j c_j[0:512]
//
// Tuned kernels (H = 64, Dc = 512, Dr = 64, bf16 q, bf16 or fp8 latent rows):
//  * mla_fp8_kernel (fp8 rows) and mla_bf16_team_kernel (bf16 rows, more than 64 (row, layer)
//    pairs, e.g. prefill): 8-wave blocks of two wave teams a tile apart -- an S team (logits
//    over all 576 dims with Q^T in registers, softmax, P^T to LDS) and a PV team (gathers,
//    O^T for 128 dims of all 64 heads) -- rows gathered by buffer-to-LDS DMA into a ring of
//    32-row slots;
//  * mla_hh_kernel (bf16 rows, at most 64 (row, layer) pairs: small decode): one 4-wave block
//    per (row, split, head half), 32-key tiles, small enough for two blocks per CU;
//  * O^T[dims x heads] += V^T . P^T, V^T read straight from the row-major tile with
//    ds_read_b64_tr_b16 (4 consecutive keys of one dim per lane; _b8 for fp8 tiles);
//  * softmax reference: each head's reference max is fixed at its first non-empty tile and
//    never moves, so the accumulators are never rescaled; a split whose later logits
//    exceed the reference by more than 2^100 is rerun with the exact maximum (exact
//    either way, because l and O share the reference);
//  * with several splits per row, partial (O, m, l) go to the workspace and a second
//    kernel combines them in split order -- deterministic.
// Generic kernel: any H <= 128, Dc <= 512, Dqk <= 1024, fp32 everywhere, two passes.
#include <cstdlib>
#include <type_traits>

#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int M_H = 64;
constexpr int M_DC = 512;
constexpr int M_DQK = 576;
constexpr int M_TILE = 64;                 // gathered rows per tile
constexpr int M_ROWB = 1168;               // LDS row stride in bytes (1152 + 16 pad)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BUF_DWORD3 = 0x00020000;     // buffer descriptor word 3 for the gfx9 family

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr16(const char *lds_generic_ptr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(
            (__attribute__((address_space(3))) char *)(lds_generic_ptr)));
}

constexpr int M_THREADS = 256;             // 4 waves, one per SIMD (512 registers each)

// Byte offset of 16-byte piece `piece` of row `row` in a buffer of rows of `rowb` bytes, as
// the unsigned 32-bit offset a buffer load takes (buffers up to 4 GB); a row of -1 (no
// index) maps past every buffer's range, so its load returns zeros.
__device__ __forceinline__ int row_offset(int32_t row, uint32_t rowb, int piece)
{
    return row >= 0 ? (int)((uint32_t)row * rowb + 16u * (uint32_t)piece) : (int)0xFFFFFFF0u;
}

// Block -> (output row, split).  The (row, split) pairs are cut into 8 contiguous ranges,
// one per XCD (blocks are dispatched to the 8 XCDs round-robin), so all splits of a row
// -- which share the row's q -- and neighbouring rows -- which share many gathered
// latent rows -- run under one L2.
__device__ __forceinline__ int64_t xcd_pair(int64_t pairs_per_xcd)
{
    const int64_t b = blockIdx.x;
    return (b & 7) * pairs_per_xcd + (b >> 3);
}

// ------------------------------------------------------------------------------------------
// fp8 latent rows: one 8-wave block per group of consecutive splits of a row, two wave teams
// a tile apart.
//
// A 4-wave block that runs S, softmax and PV of a tile in sequence keeps each SIMD's matrix
// core idle through the softmax, the exchanges and the barriers.  Here each SIMD holds one
// wave of each team, and between two barriers the teams work on different tiles:
//   * the S team (waves 0-3, wave a: heads 32*(a & 1) .., keys 32*(a >> 1) .. of each tile)
//     computes S^T [32 keys x 32 heads] over all 576 dims (36 MFMA; the wave holds its heads'
//     Q^T), the softmax numerators against the split's fixed reference maximum and writes P^T
//     (bf16) to LDS: tile t in step t;
//   * the PV team (waves 4-7, wave b: dims 128*b .. +127 of all 64 heads) issues the gathers
//     and accumulates O^T [128 dims x 64 heads] += V^T . P^T (32 MFMA, each V element widened
//     once): tile t in step t + 1.
// One team's softmax and widening then run beside the other's MFMAs.  With all 576 dims in
// one wave the logits need no cross-wave sum; only the reference maximum (fixed at each
// split's first non-empty tile) is exchanged, once per split.
//
// Splits: the split count and boundaries come from the split policy alone; a block runs
// `group` consecutive splits of one row as one tile sequence (the S team restarts its softmax
// state and hands (row sum, reference maximum) over at each split boundary, the PV team
// stores the split's result and clears O), so grouping changes scheduling, not a bit of any
// result.  Q is loaded once per block: staged through LDS by all 512 threads.
//
// Gathers: rows land by buffer-to-LDS DMA in a ring of seven 32-row slots (half tiles), kept
// fp8 there and widened to bf16 in registers when read.  In step s the S team reads tile s,
// the PV team tile s - 1, and the half tiles 2s+2 .. 2s+4 are in flight: half tiles 2s+3 and
// 2s+4 are issued at the start of step s, into the slots tile s - 2 left, and the step ends
// once 2s+2 and 2s+3 have landed.
//
// Softmax without rescaling: the reference maximum is fixed at the split's first non-empty
// tile, so the fp32 O accumulators are never rescaled (exact either way, since l and O share
// the reference); a later logit above it by more than 2^100 makes that split run again (a
// cold second pass) with the exact maximum of the first pass.
// ------------------------------------------------------------------------------------------
constexpr int F_ROWB = 592;                      // fp8 LDS row stride (576 + 16 pad)
constexpr int TM_THREADS = 512;
constexpr int TM_HALF = 32;                      // gathered rows per ring slot (half a tile)
constexpr int TM_SLOTB = TM_HALF * F_ROWB;       // 18944 B
constexpr int TM_SLOTS = 7;
constexpr int TM_DMA = (TM_SLOTB + 1023) / 1024;     // 19 wave-wide loads per slot, the last half wide
constexpr int TM_DMA_PER_WAVE = (TM_DMA + 3) / 4;    // 5 (4 on the last PV wave)
constexpr int TM_PROWB = 144;                    // P^T row of one head: 64 keys bf16 + 16 pad
constexpr int TM_PBUFB = M_H * TM_PROWB;         // 9216 B
static_assert(TM_DMA == 19 && TM_SLOTB - 18 * 1024 == 512, "the last load of a slot is 32 lanes wide");

// Value of lane l ^ 32 (g = lane >> 5), through one v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float other_half(float x, int g)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(g ? r[0] : r[1]);
}

__device__ __forceinline__ i32x2 lds_tr8(const char *lds_generic_ptr)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (i32x2 __attribute__((address_space(3))) *)((__attribute__((address_space(3))) char *)(lds_generic_ptr)));
}

constexpr int F_IDX = 2048;  // index slots of one split (32 tiles) held in LDS
static_assert(F_IDX >= DSA_TOPK_MAX, "a split never holds more than k index slots");

// Gathers into a ring slot of 32 rows (fp8: 32 x 592 B, 19 wave-wide 1 KB loads; bf16:
// 32 x 1168 B, 37 loads; the last load of a slot is 32 lanes wide), shared by NW waves.  Load q
// of issuing wave w covers slot bytes 1024 (NW q + w) + 16 lane, i.e. row rc & 0xFF, column
// rc >> 8 (0xFFFF: the pad bytes, which read zeros); the row's source is index * RB (RB = 576
// or 1152 bytes).
template <int RB, int NW = 4>
struct SlotDma {
    static constexpr int ROWB = RB + 16;
    static constexpr int SLOTB = 32 * ROWB;
    static constexpr int LOADS = (SLOTB + 1023) / 1024;
    static constexpr int PER_WAVE = (LOADS + NW - 1) / NW;
    static_assert(SLOTB - (LOADS - 1) * 1024 == 512, "the last load of a slot is 32 lanes wide");

    __device__ static void geometry(int w, int lane, uint32_t (&rc)[PER_WAVE])
    {
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int o = 1024 * (NW * q + w) + 16 * lane;
            const int row = min(o / ROWB, 31);
            const int col = o - (o / ROWB) * ROWB;
            const bool real = o < SLOTB && col < RB;
            rc[q] = (uint32_t)row | ((real ? (uint32_t)col : 0xFFFFu) << 8);
        }
    }
    // Source offsets of this wave's loads for the 32 rows given by sidx (index -1: zeros).
    __device__ static void offsets(const int32_t *sidx, const uint32_t (&rc)[PER_WAVE], int (&voff)[PER_WAVE])
    {
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int32_t idx = sidx[rc[q] & 0xFFu];
            const uint32_t col = rc[q] >> 8;
            // unsigned 32-bit offsets (buffers up to 4 GB); pads and missing rows read zeros
            voff[q] = (col != 0xFFFFu && idx >= 0) ? (int)((uint32_t)idx * (uint32_t)RB + col) : (int)0xFFFFFFF0u;
        }
    }
    // Load q of wave w (nothing past the slot's last load).
    __device__ static void one(const i32x4 &seq, uint32_t lds_base, int w, int lane, int q, int voff)
    {
        const int u = NW * q + w;
        if (u < LOADS - 1)
            dma16(seq, lds_base + 1024u * (uint32_t)u, voff);
        else if (u == LOADS - 1 && lane < 32)
            dma16(seq, lds_base + 1024u * (uint32_t)u, voff);
    }
    // Gather this wave's share of the 32 rows given by sidx into the slot at lds_base.
    __device__ static void issue(const i32x4 &seq, uint32_t lds_base, const int32_t *sidx, int w, int lane,
                                 const uint32_t (&rc)[PER_WAVE])
    {
        int voff[PER_WAVE];
        offsets(sidx, rc, voff);
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q)
            one(seq, lds_base, w, lane, q, voff[q]);
    }
};
typedef SlotDma<576> Fp8Slot;
static_assert(Fp8Slot::SLOTB == TM_SLOTB && Fp8Slot::PER_WAVE == TM_DMA_PER_WAVE, "fp8 slot geometry");

// Wait until only the most recent fp8 slot's loads (5 on PV waves 0-2, 4 on wave 3) may still
// be outstanding: every earlier slot has landed.
__device__ __forceinline__ void wait_but_last_slot(int b)
{
    static_assert(TM_DMA_PER_WAVE == 5, "loads per wave and slot");
    if (b == 3)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}

// Partial (or, with one split, final) result of one split from the PV team's registers:
// wave b holds dims 128 b + 32 mt + 8 q4 + 4 g + 0..3 of heads j (nh = 0) and 32 + j (nh = 1).
// bf16 results are staged through LDS, 32 heads at a time, in bytes of the split's last tile
// that only this wave reads (its own V columns): stage(r, c) is the address of byte c of head
// r's 256-byte piece.  They are then stored as whole 256-byte pieces, four heads per
// instruction.  fp32 results are stored straight from the MFMA layout.
template <bool OUT_F32, typename Stage>
__device__ __forceinline__ void mla_team_store(const f32x16 (&O)[4][2], const float (&l)[2], const float (&m)[2],
                                               const MlaLayerDev &Ld, int64_t i, int64_t orow, int split, int nsplit,
                                               int b, int g, int j, int lane, Stage stage, float *__restrict__ ws_o,
                                               float *__restrict__ ws_ml)
{
    const int64_t base = (nsplit == 1) ? i * M_H * M_DC : (orow * nsplit + split) * M_H * M_DC;
#pragma unroll
    for (int nh = 0; nh < 2; ++nh) {
        const float inv = (l[nh] > 0.f) ? (nsplit == 1 ? Ld.kv_scale / l[nh] : 1.f / l[nh]) : 0.f;
        if (OUT_F32) {
            float *dst = ((nsplit == 1) ? (float *)Ld.out : ws_o) + base + (32 * nh + j) * M_DC;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x16 &o = O[mt][nh];
                    *(f32x4 *)(dst + 128 * b + 32 * mt + 8 * q4 + 4 * g) =
                        f32x4{o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv};
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x16 &o = O[mt][nh];
                    *(u32x2 *)stage(j, 2 * (32 * mt + 8 * q4 + 4 * g)) =
                        u32x2{pack_bf16x2(o[4 * q4] * inv, o[4 * q4 + 1] * inv),
                              pack_bf16x2(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv)};
                }
            uint16_t *dst = ((nsplit == 1) ? (uint16_t *)Ld.out : (uint16_t *)ws_o) + base + 128 * b;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 4 * u + (lane >> 4), c = 16 * (lane & 15);
                *(u32x4 *)((char *)(dst + (32 * nh + r) * M_DC) + c) = *(const u32x4 *)stage(r, c);
            }
        }
        if (b == 0 && g == 0) {
            const int head = 32 * nh + j;
            if (nsplit == 1) {
                if (Ld.lse)
                    Ld.lse[i * M_H + head] = (l[nh] > 0.f) ? (m[nh] + __log2f(l[nh])) * LN2 : -INFINITY;
            } else {
                float *pml = ws_ml + ((orow * nsplit + split) * M_H + head) * 2;
                pml[0] = m[nh];
                pml[1] = l[nh];
            }
        }
    }
}

constexpr int TM_MAX_GROUP = 4;       // consecutive splits of one row run by one block, at most
constexpr int TM_QROWB = 1168;        // Q staging row in LDS: 576 bf16 + 16 pad
constexpr int TM_QOFF = 3 * TM_SLOTB; // Q staged in slots 3..6 before the first gathers
static_assert(M_H * TM_QROWB <= 4 * TM_SLOTB, "Q staging fits slots 3..6");

template <bool OUT_F32>
__global__ __launch_bounds__(TM_THREADS, 1) void mla_fp8_kernel(LayoutDev L, int64_t T, int64_t n_rows,
                                                                MlaLayersDev layers,
                                                                const int32_t *__restrict__ indices, int k,
                                                                float sm_scale, int nsplit, int tiles_per_split,
                                                                int group, int64_t pairs_per_xcd,
                                                                float *__restrict__ ws_o, float *__restrict__ ws_ml)
{
    __shared__ __attribute__((aligned(16))) char ring[TM_SLOTS][TM_SLOTB];
    __shared__ __attribute__((aligned(16))) char pbuf[2][TM_PBUFB];  // P^T of tiles s, s - 1
    __shared__ int32_t sidx[F_IDX];                                   // the group's index slots
    __shared__ float xm[2][M_H];                  // reference-maximum exchange (key halves)
    __shared__ float xl[2][2][M_H];               // row sums of the key halves, by split parity
    __shared__ float xr[2][M_H];                  // reference maximum, by split parity
    __shared__ float xs[TM_MAX_GROUP][2][M_H];    // largest logit per split and key half (reruns)
    __shared__ uint32_t sh_ne, sh_ovf;            // non-empty tiles; splits to run again

    const int ngroups = nsplit / group;
    const int64_t pair = xcd_pair(pairs_per_xcd);
    if (pair >= n_rows * ngroups)
        return;
    const int64_t orow = pair / ngroups;
    const int split0 = (int)(pair % ngroups) * group;
    const int layer = (int)(orow / T);
    const int64_t i = orow % T;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tw = w & 3;  // wave within its team
    const int g = lane >> 5, j = lane & 31;
    const MlaLayerDev Ld = layers.l[layer];
    const RowInfo r = row_info(L, i);
    const float c2 = sm_scale * Ld.kv_scale * LOG2E;

    // the group's tiles: split split0 + gs covers tiles [gs tps, min(nt, (gs + 1) tps))
    const int tps = tiles_per_split;
    const int ntiles_all = (k + M_TILE - 1) / M_TILE;
    const int g_begin = split0 * tps;
    const int nt = max(0, min(ntiles_all, (split0 + group) * tps) - g_begin);
    const int32_t *irow = indices + i * k + (int64_t)g_begin * M_TILE;
    const int nidx = min(k - g_begin * M_TILE, nt * M_TILE);

    // ---- prologue (all 512 threads): the group's index list and the row's Q to LDS, slots
    //      0..2 cleared; the non-empty tiles noted
    {
        int32_t v[F_IDX / TM_THREADS];
#pragma unroll
        for (int u = 0; u < F_IDX / TM_THREADS; ++u) {
            const int e = tid + TM_THREADS * u;
            v[u] = e < nidx ? irow[e] : -1;
        }
        u32x4 qv[(M_H * 72 + TM_THREADS - 1) / TM_THREADS];
        const u32x4 *qsrc = (const u32x4 *)((const uint16_t *)Ld.q + i * M_H * M_DQK);
#pragma unroll
        for (int u = 0; u < (M_H * 72 + TM_THREADS - 1) / TM_THREADS; ++u) {
            const int c = tid + TM_THREADS * u;
            if (c < M_H * 72)
                qv[u] = qsrc[c];
        }
        for (int e = tid; e < 3 * TM_SLOTB / 16; e += TM_THREADS)
            ((u32x4 *)&ring[0][0])[e] = u32x4{0u, 0u, 0u, 0u};
        if (tid == 0) {
            sh_ne = 0u;
            sh_ovf = 0u;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < F_IDX / TM_THREADS; ++u) {
            const int e = tid + TM_THREADS * u;  // a wave covers one tile: e >> 6 is wave-uniform
            if (e < nt * M_TILE) {
                sidx[e] = v[u];
                if (__ballot(v[u] >= 0) != 0ull && lane == 0)
                    atomicOr(&sh_ne, 1u << (e >> 6));
            }
        }
#pragma unroll
        for (int u = 0; u < (M_H * 72 + TM_THREADS - 1) / TM_THREADS; ++u) {
            const int c = tid + TM_THREADS * u;
            if (c < M_H * 72)
                *(u32x4 *)(&ring[0][0] + TM_QOFF + (c / 72) * TM_QROWB + 16 * (c % 72)) = qv[u];
        }
        __syncthreads();
    }
    const uint32_t ne = sh_ne;
    // tile s is the first non-empty tile of its split
    auto first_of_split = [&](int s) __attribute__((always_inline)) {
        const int st = (s / tps) * tps;
        const uint32_t below = ((1u << s) - 1u) & ~((1u << st) - 1u);
        return ((ne >> s) & 1u) != 0u && (ne & below) == 0u;
    };
    auto last_of_split = [&](int s) __attribute__((always_inline)) {
        return s + 1 == nt || (s + 1) % tps == 0;
    };

    // The two teams run separate code (so that Q^T and O share registers) with the same
    // sequence of barriers: per pass two after the first gathers, one per step, two more in
    // the step of each split's first non-empty tile in the first pass; the rerun flag; per
    // rerun split a pass of its own.
    if (w < 4) {
        // ================================ S team ================================
        // wave a: heads 32 hh .. +31, keys 32 hi .. +31 of each tile
        const int hh = tw & 1, hi = tw >> 1, head = 32 * hh + j;
        // Q^T of its 32 heads over all 576 dims; k-step 2p + h of lane half g covers dims
        // 32p + 16g + 8h .. +7 (the K rows are read 16 bytes per lane in the same order)
        bf16x8 qT[36];
        const char *srow = &ring[0][0] + j * F_ROWB + 16 * g;  // S operand row j of slot 0
        float m_ref = -INFINITY, m_seen = -INFINITY, l_own = 0.f;
        bool ovf = false;

        // step s (tile s of the pass starting at tile t0): logits of this wave's key half,
        // softmax numerators against the split's reference maximum, P^T to LDS
        auto s_step = [&](int s, int t0, bool need_ref) __attribute__((always_inline)) {
            const int gs = s / tps;
            if (s % tps == 0 || s == t0) {  // a split starts
                m_ref = need_ref ? -INFINITY : fmaxf(xs[gs][0][head], xs[gs][1][head]);
                m_seen = -INFINITY;
                l_own = 0.f;
                ovf = false;
            }
            const int sl = (2 * (s - t0) + hi) % TM_SLOTS;
            const char *a = srow + sl * TM_SLOTB;
            char *prow = &pbuf[(s - t0) & 1][0] + head * TM_PROWB + 2 * (32 * hi + 4 * g);
            const uint64_t valid = __ballot(sidx[s * M_TILE + lane] >= 0);
            if (valid == 0ull) {  // no key of the tile: P = 0 (also before the reference is fixed)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(u32x2 *)(prow + 16 * q) = u32x2{0u, 0u};
            } else {
                f32x16 S = f32x16{};
                u32x4 A[2];
                A[0] = *(const u32x4 *)a;
#pragma unroll
                for (int p = 0; p < 18; ++p) {
                    if (p + 1 < 18)
                        A[(p + 1) & 1] = *(const u32x4 *)(a + 32 * (p + 1));
                    const u32x4 x = A[p & 1];
                    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(x[0], x[1]), qT[2 * p], S, 0, 0, 0);
                    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(x[2], x[3]), qT[2 * p + 1], S, 0, 0,
                                                                0);
                }
                // lane (g, j) holds keys 32 hi + 8 (rr >> 2) + 4 g + (rr & 3) of head 32 hh + j
                const uint32_t vkeys = (uint32_t)(valid >> (32 * hi)) >> (4 * g);
                const bool full = valid == ~0ull;
                float mloc = -INFINITY;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const bool ok = full || ((vkeys >> (8 * (rr >> 2) + (rr & 3))) & 1u);
                    S[rr] = ok ? S[rr] * c2 : -INFINITY;
                    mloc = fmaxf(mloc, S[rr]);
                }
                mloc = fmaxf(mloc, other_half(mloc, g));
                if (need_ref && first_of_split(s)) {  // the maximum over both key halves
                    if (g == 0)
                        xm[hi][head] = mloc;
                    lds_barrier();
                    m_ref = fmaxf(xm[0][head], xm[1][head]);
                    lds_barrier();
                }
                m_seen = fmaxf(m_seen, mloc);
                ovf |= mloc > m_ref + 100.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float p4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p4[e] = __builtin_amdgcn_exp2f(S[4 * q + e] - m_ref);  // masked: exp2(-inf) = 0
                    l_own += p4[0] + p4[1];
                    l_own += p4[2] + p4[3];
                    *(u32x2 *)(prow + 16 * q) = u32x2{pack_bf16x2(p4[0], p4[1]), pack_bf16x2(p4[2], p4[3])};
                }
            }
            if (last_of_split(s)) {  // (row sum, reference maximum) to the PV team
                const float l_pair = l_own + other_half(l_own, g);
                if (g == 0) {
                    xl[gs & 1][hi][head] = l_pair;
                    if (hi == 0)
                        xr[gs & 1][head] = m_ref;
                    if (need_ref)
                        xs[gs][hi][head] = m_seen;
                }
                if (ovf)
                    atomicOr(&sh_ovf, 1u << gs);
            }
        };
        // Q^T from LDS; the staging slots are cleared once every S wave has its copy
#pragma unroll
        for (int t = 0; t < 36; ++t)
            qT[t] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(&ring[0][0] + TM_QOFF + head * TM_QROWB +
                                                                64 * (t >> 1) + 32 * g + 16 * (t & 1)));
        // pass 0: every tile of the group; pass 1 + gs: split gs again, if it overflowed
        uint32_t rerun = 0u;
        for (int pass = 0; pass <= group; ++pass) {
            const int t0 = pass == 0 ? 0 : (pass - 1) * tps;
            const int t1 = pass == 0 ? nt : min(nt, pass * tps);
            if ((pass == 0 && nt > 0) || (pass > 0 && ((rerun >> (pass - 1)) & 1u))) {
                lds_barrier();
                if (pass == 0)
                    for (int e = tid; e < 4 * TM_SLOTB / 16; e += 256)
                        ((u32x4 *)(&ring[0][0] + TM_QOFF))[e] = u32x4{0u, 0u, 0u, 0u};
                lds_barrier();  // tile t0 has landed
                for (int s = t0; s <= t1; ++s) {
                    if (s < t1)
                        s_step(s, t0, pass == 0);
                    lds_barrier();
                }
            }
            if (pass == 0) {
                __syncthreads();
                rerun = sh_ovf;
            }
        }
    } else {
        // ================================ PV team ================================
        // wave b: dims 128 b .. +127 of all 64 heads
        const int b = tw;
        f32x16 O[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            O[mt][0] = O[mt][1] = f32x16{};

        // this sequence's rows, or with paged caches the whole cache (host: at most 4 GiB - 1 MiB)
        const bool paged = L.block_table != nullptr;
        const int64_t seq_bytes = (paged ? L.cache_rows : r.n) * 576;
        const i32x4 seq = buffer_desc((const uint8_t *)Ld.kv + (paged ? 0 : r.kv_base) * 576, seq_bytes);
        const uint32_t lds0 = lds_addr_of(&ring[0][0]);
        uint32_t rc[TM_DMA_PER_WAVE];
        Fp8Slot::geometry(b, lane, rc);
        // V^T read geometry: 16-lane group G covers dims +16 (G & 1), keys +8 (G >> 1)
        const int mq = lane & 15;
        const int voffs = (8 * g + (mq >> 1)) * F_ROWB + 128 * b + 16 * ((lane >> 4) & 1) + 8 * (mq & 1);

        // O^T += V^T . P^T over the 64 keys of tile t (pass starting at t0)
        auto pv_tile = [&](int t, int t0) __attribute__((always_inline)) {
            const int h0 = 2 * (t - t0);
            const char *v0 = &ring[0][0] + (h0 % TM_SLOTS) * TM_SLOTB + voffs;
            const char *v1 = &ring[0][0] + ((h0 + 1) % TM_SLOTS) * TM_SLOTB + voffs;
            const char *pb = &pbuf[(t - t0) & 1][0] + j * TM_PROWB + 16 * g;
            i32x2 V[2][4];
            auto v_load = [&](int u, i32x2 (&Vd)[4]) __attribute__((always_inline)) {
                const char *v = ((u >> 1) ? v1 : v0) + 16 * (u & 1) * F_ROWB;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Vd[mt] = lds_tr8(v + 32 * mt);
            };
            v_load(0, V[0]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u + 1 < 4)
                    v_load(u + 1, V[(u + 1) & 1]);
                // keys 16u + 8g .. +7 of heads j, 32 + j: the key order of the V^T operand
                const bf16x8 p0 = __builtin_bit_cast(bf16x8, *(const u32x4 *)(pb + 32 * u));
                const bf16x8 p1 = __builtin_bit_cast(bf16x8, *(const u32x4 *)(pb + 32 * TM_PROWB + 32 * u));
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const bf16x8 va = fp8x8_to_bf16x8((uint32_t)V[u & 1][mt][0], (uint32_t)V[u & 1][mt][1]);
                    O[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p0, O[mt][0], 0, 0, 0);
                    O[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1, O[mt][1], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the split of tile t (pass starting at t0) is complete: its result out, O cleared
        auto finish_split = [&](int t, int t0) __attribute__((always_inline)) {
            const int gs = t / tps;
            const int h0 = 2 * (t - t0);
            char *sa = &ring[0][0] + (h0 % TM_SLOTS) * TM_SLOTB, *sb = &ring[0][0] + ((h0 + 1) % TM_SLOTS) * TM_SLOTB;
            // head r's 256 bytes in stage rows 2r, 2r + 1 (rows 0..31 of sa, then of sb), the
            // wave's columns 128 b .. +127
            auto stage = [&](int r, int c) __attribute__((always_inline)) {
                const int R = 2 * r + (c >> 7);
                return (R < 32 ? sa : sb) + (R & 31) * F_ROWB + 128 * b + (c & 127);
            };
            float l[2], m[2];
#pragma unroll
            for (int nh = 0; nh < 2; ++nh) {
                l[nh] = xl[gs & 1][0][32 * nh + j] + xl[gs & 1][1][32 * nh + j];
                m[nh] = xr[gs & 1][32 * nh + j];
            }
            mla_team_store<OUT_F32>(O, l, m, Ld, i, orow, split0 + gs, nsplit, b, g, j, lane, stage, ws_o, ws_ml);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                O[mt][0] = O[mt][1] = f32x16{};
        };
        auto run = [&](int t0, int t1, bool need_ref) __attribute__((always_inline)) {
            const int nslots = 2 * (t1 - t0);
            for (int h = 0; h < min(3, nslots); ++h)
                Fp8Slot::issue(seq, lds0 + (uint32_t)h * TM_SLOTB, sidx + (2 * t0 + h) * TM_HALF, b, lane, rc);
            lds_barrier();  // (first pass: the S team has its copy of Q and clears slots 3..6)
            if (nslots > 2)
                wait_but_last_slot(b);  // tile t0 has landed
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            for (int s = t0; s <= t1; ++s) {
                const int hs = 2 * (s - t0);
                // half tiles hs+3, hs+4 into the slots of tile s - 2 (consumed in step s - 1)
                for (int h = hs + 3; h <= hs + 4; ++h)
                    if (h < nslots)
                        Fp8Slot::issue(seq, lds0 + (uint32_t)(h % TM_SLOTS) * TM_SLOTB, sidx + (2 * t0 + h) * TM_HALF,
                                       b, lane, rc);
                if (need_ref && s < t1 && first_of_split(s)) {
                    lds_barrier();  // the S team's two exchange barriers
                    lds_barrier();
                }
                if (s > t0)
                    pv_tile(s - 1, t0);
                // tile s + 1 (half tiles hs+2, hs+3) must have landed; hs+4 may stay in flight
                if (s + 1 < t1) {
                    if (hs + 4 < nslots)
                        wait_but_last_slot(b);
                    else
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                // after the wait, so that the result's stores are the newest memory operations
                // and the count-based waits of the next step do not wait for them
                if (s > t0 && last_of_split(s - 1))
                    finish_split(s - 1, t0);
                lds_barrier();
            }
        };
        uint32_t rerun = 0u;
        for (int pass = 0; pass <= group; ++pass) {
            const int t0 = pass == 0 ? 0 : (pass - 1) * tps;
            const int t1 = pass == 0 ? nt : min(nt, pass * tps);
            if ((pass == 0 && nt > 0) || (pass > 0 && ((rerun >> (pass - 1)) & 1u)))
                run(t0, t1, pass == 0);
            if (pass == 0) {
                __syncthreads();
                rerun = sh_ovf;
            }
        }
        // splits past the end of the index list (none under the split policy): empty results
        for (int gs = 0; gs < group; ++gs)
            if (gs * tps >= nt) {
                const float l[2] = {0.f, 0.f}, m[2] = {-INFINITY, -INFINITY};
                auto stage = [&](int r, int c) __attribute__((always_inline)) {
                    const int R = 2 * r + (c >> 7);
                    return &ring[R >> 5][0] + (R & 31) * F_ROWB + 128 * b + (c & 127);
                };
                mla_team_store<OUT_F32>(O, l, m, Ld, i, orow, split0 + gs, nsplit, b, g, j, lane, stage, ws_o, ws_ml);
            }
    }
}

// ------------------------------------------------------------------------------------------
// bf16 latent rows, more than MLA_HH_MAX_ROWS rows (prefill): the two-team layout of
// mla_fp8_kernel with 32-key steps.  A 32-row bf16 slot takes 37 KB, so the LDS ring holds
// three: in step s the S team reads tile s, the PV team tile s - 1, and tile s + 1 is in
// flight (issued at the start of step s into the slot tile s - 2 left).
//   * S team wave a: heads 32 (a & 1) .. +31 as two 16-head blocks, keys 16 (a >> 1) .. +15
//     of each 32-key tile: S^T [16 keys x 16 heads] per block over all 576 dims
//     (v_mfma_f32_16x16x32_bf16, 2 x 18 per step; the wave's Q^T in 144 registers, each K
//     operand shared by the two blocks);
//   * PV team wave b: dims 128 b .. +127 of all 64 heads, O^T += V^T . P^T over 2 steps of 16
//     keys (v_mfma_f32_32x32x16_bf16, 4 dim blocks x 2 head blocks each), V^T read with
//     ds_read_b64_tr_b16, P^T from LDS in the same key order.
// The gathers of tile s + 1 are shared by all eight waves and issued between the MFMAs of
// step s (the S team's between its k-steps, the PV team's between its key steps), so the
// address unit works through them while the matrix cores run.
// Splits, grouping, the reference maximum, the rerun and the staged split results are those
// of mla_fp8_kernel; split boundaries are the policy's 64-key tiles (two 32-key tiles each).
// ------------------------------------------------------------------------------------------
typedef SlotDma<1152, 8> Bf16Slot;  // all 8 waves gather: 5 loads on waves 0-4, 4 on 5-7
constexpr int TB_ROWB = Bf16Slot::ROWB;          // 1168
constexpr int TB_SLOTB = Bf16Slot::SLOTB;        // 37376
constexpr int TB_SLOTS = 3;
constexpr int TB_PROWB = 80;                     // P^T row of one head: 32 keys bf16 + 16 pad
constexpr int TB_PBUFB = M_H * TB_PROWB;         // 5120 B
constexpr int TB_QOFF = TB_SLOTB;                // Q staged in slots 1..2 before the first gathers
static_assert(M_H * TM_QROWB <= 2 * TB_SLOTB, "Q staging fits slots 1..2");
static_assert(TB_ROWB == TM_QROWB, "Q staging rows and K rows share the stride");

template <bool OUT_F32>
__global__ __launch_bounds__(TM_THREADS, 1) void mla_bf16_team_kernel(LayoutDev L, int64_t T, int64_t n_rows,
                                                                      MlaLayersDev layers,
                                                                      const int32_t *__restrict__ indices, int k,
                                                                      float sm_scale, int nsplit, int tiles_per_split,
                                                                      int group, int64_t pairs_per_xcd,
                                                                      float *__restrict__ ws_o,
                                                                      float *__restrict__ ws_ml)
{
    __shared__ __attribute__((aligned(16))) char ring[TB_SLOTS][TB_SLOTB];
    __shared__ __attribute__((aligned(16))) char pbuf[2][TB_PBUFB];  // P^T of tiles s, s - 1
    __shared__ int32_t sidx[F_IDX];                                   // the group's index slots
    __shared__ float xm[2][M_H];                  // reference-maximum exchange (key quarters)
    __shared__ float xl[2][2][M_H];               // row sums of the two S waves, by split parity
    __shared__ float xr[2][M_H];                  // reference maximum, by split parity
    __shared__ float xs[TM_MAX_GROUP][2][M_H];    // largest logit per split and S wave (reruns)
    __shared__ uint32_t sh_ne[2], sh_ovf;         // non-empty 32-key tiles; splits to run again

    const int ngroups = nsplit / group;
    const int64_t pair = xcd_pair(pairs_per_xcd);
    if (pair >= n_rows * ngroups)
        return;
    const int64_t orow = pair / ngroups;
    const int split0 = (int)(pair % ngroups) * group;
    const int layer = (int)(orow / T);
    const int64_t i = orow % T;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tw = w & 3;  // wave within its team
    const int g = lane >> 5, j = lane & 31;
    const MlaLayerDev Ld = layers.l[layer];
    const RowInfo r = row_info(L, i);
    const float c2 = sm_scale * Ld.kv_scale * LOG2E;

    // the group's 32-key tiles: split split0 + gs covers tiles [gs tps, min(nt, (gs + 1) tps))
    const int tps = tiles_per_split;
    const int ntiles_all = (k + 31) / 32;
    const int g_begin = split0 * tps;
    const int nt = max(0, min(ntiles_all, (split0 + group) * tps) - g_begin);
    const int32_t *irow = indices + i * k + (int64_t)g_begin * 32;
    const int nidx = min(k - g_begin * 32, nt * 32);

    // ---- prologue (all 512 threads): the group's index list and the row's Q to LDS, slot 0
    //      cleared; the non-empty tiles noted
    {
        int32_t v[F_IDX / TM_THREADS];
#pragma unroll
        for (int u = 0; u < F_IDX / TM_THREADS; ++u) {
            const int e = tid + TM_THREADS * u;
            v[u] = e < nidx ? irow[e] : -1;
        }
        u32x4 qv[(M_H * 72 + TM_THREADS - 1) / TM_THREADS];
        const u32x4 *qsrc = (const u32x4 *)((const uint16_t *)Ld.q + i * M_H * M_DQK);
#pragma unroll
        for (int u = 0; u < (M_H * 72 + TM_THREADS - 1) / TM_THREADS; ++u) {
            const int c = tid + TM_THREADS * u;
            if (c < M_H * 72)
                qv[u] = qsrc[c];
        }
        for (int e = tid; e < TB_SLOTB / 16; e += TM_THREADS)
            ((u32x4 *)&ring[0][0])[e] = u32x4{0u, 0u, 0u, 0u};
        if (tid < 2)
            sh_ne[tid] = 0u;
        if (tid == 0)
            sh_ovf = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < F_IDX / TM_THREADS; ++u) {
            const int e = tid + TM_THREADS * u;  // a wave covers tiles 2m, 2m + 1 (m = e >> 6)
            const bool in = e < nt * 32;
            if (in)
                sidx[e] = v[u];
            const uint64_t bal = __ballot(in && v[u] >= 0);
            if (lane == 0 && bal != 0ull) {
                const int t2 = (e >> 5) & ~1;  // this wave's even tile
                const uint32_t bits = ((uint32_t)bal != 0u ? 1u : 0u) | ((bal >> 32) != 0ull ? 2u : 0u);
                atomicOr(&sh_ne[t2 >> 5], bits << (t2 & 31));
            }
        }
#pragma unroll
        for (int u = 0; u < (M_H * 72 + TM_THREADS - 1) / TM_THREADS; ++u) {
            const int c = tid + TM_THREADS * u;
            if (c < M_H * 72)
                *(u32x4 *)(&ring[0][0] + TB_QOFF + (c / 72) * TM_QROWB + 16 * (c % 72)) = qv[u];
        }
        __syncthreads();
    }
    const uint64_t ne = ((uint64_t)sh_ne[1] << 32) | sh_ne[0];
    // tile s is the first non-empty tile of its split
    auto first_of_split = [&](int s) __attribute__((always_inline)) {
        const int st = (s / tps) * tps;
        const uint64_t below = ((1ull << s) - 1ull) & ~((1ull << st) - 1ull);
        return ((ne >> s) & 1ull) != 0ull && (ne & below) == 0ull;
    };
    auto last_of_split = [&](int s) __attribute__((always_inline)) {
        return s + 1 == nt || (s + 1) % tps == 0;
    };

    // The two teams run separate code with the same sequence of block barriers (see
    // mla_fp8_kernel).
    if (w < 4) {
        // ================================ S team ================================
        const int hh = tw & 1, kq = tw >> 1;
        const int hd0 = 32 * hh + (lane & 15);  // head of block 0 (block 1: + 16)
        const int qg = lane >> 4;               // key group: keys 16 kq + 4 qg + 0..3
        // Q^T of block hb: head hd0 + 16 hb, dims 32t + 8 qg .. +7 (the 16x16x32 B operand)
        bf16x8 qT[2][18];
        float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY}, l_own[2] = {0.f, 0.f};
        bool ovf = false;
        const bool paged = L.block_table != nullptr;
        const i32x4 seq = buffer_desc((const uint8_t *)Ld.kv + (paged ? 0 : r.kv_base) * 1152,
                                      (paged ? L.cache_rows : r.n) * 1152);
        const uint32_t lds0 = lds_addr_of(&ring[0][0]);
        uint32_t rc[Bf16Slot::PER_WAVE];
        Bf16Slot::geometry(tw, lane, rc);

        // step s (tile s of the pass starting at tile t0): logits of this wave's 16 keys for
        // its 32 heads, softmax numerators against the split's reference maximum, P^T to LDS;
        // with gather, this wave's share of tile s + 1 issued between the k-steps
        auto s_step = [&](int s, int t0, bool need_ref, bool gather) __attribute__((always_inline)) {
            int voff[Bf16Slot::PER_WAVE];
            const uint32_t nslot = lds0 + (uint32_t)((s + 1 - t0) % TB_SLOTS) * TB_SLOTB;
            if (gather)
                Bf16Slot::offsets(sidx + 32 * (s + 1), rc, voff);
            const int gs = s / tps;
            if (s % tps == 0 || s == t0) {  // a split starts
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int hd = hd0 + 16 * hb;
                    m_ref[hb] = need_ref ? -INFINITY : fmaxf(xs[gs][0][hd], xs[gs][1][hd]);
                    m_seen[hb] = -INFINITY;
                    l_own[hb] = 0.f;
                }
                ovf = false;
            }
            const char *slot = &ring[0][0] + ((s - t0) % TB_SLOTS) * TB_SLOTB;
            char *pw = &pbuf[(s - t0) & 1][0] + hd0 * TB_PROWB + 2 * (16 * kq + 4 * qg);
            const uint32_t valid = (uint32_t)__ballot(lane < 32 && sidx[s * 32 + (lane & 31)] >= 0);
            if (valid == 0u) {  // no key of the tile: P = 0 (also before the reference is fixed)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    *(u32x2 *)(pw + 16 * hb * TB_PROWB) = u32x2{0u, 0u};
                if (gather)
#pragma unroll
                    for (int q = 0; q < Bf16Slot::PER_WAVE; ++q)
                        Bf16Slot::one(seq, nslot, tw, lane, q, voff[q]);
            } else {
                f32x4 S[2] = {f32x4{}, f32x4{}};
                const char *arow = slot + (16 * kq + (lane & 15)) * TB_ROWB + 16 * qg;
                constexpr int AD = 4;  // K operands read this many k-steps ahead
                u32x4 A[AD];
#pragma unroll
                for (int t = 0; t < AD - 1; ++t)
                    A[t] = *(const u32x4 *)(arow + 64 * t);
#pragma unroll
                for (int t = 0; t < 18; ++t) {
                    if (t + AD - 1 < 18)
                        A[(t + AD - 1) % AD] = *(const u32x4 *)(arow + 64 * (t + AD - 1));
                    const bf16x8 a = __builtin_bit_cast(bf16x8, A[t % AD]);
                    S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qT[0][t], S[0], 0, 0, 0);
                    S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qT[1][t], S[1], 0, 0, 0);
                    if (gather && t % 3 == 1 && t / 3 < Bf16Slot::PER_WAVE)
                        Bf16Slot::one(seq, nslot, tw, lane, t / 3, voff[t / 3]);
                }
                // lane holds keys 16 kq + 4 qg + e of heads hd0 (S[0]) and hd0 + 16 (S[1])
                const bool full = valid == ~0u;
                float mloc[2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    mloc[hb] = -INFINITY;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = full || ((valid >> (16 * kq + 4 * qg + e)) & 1u);
                        S[hb][e] = ok ? S[hb][e] * c2 : -INFINITY;
                        mloc[hb] = fmaxf(mloc[hb], S[hb][e]);
                    }
                }
                if (need_ref && first_of_split(s)) {  // the maximum over all 32 keys of the tile
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb) {
                        float m = fmaxf(mloc[hb], __shfl_xor(mloc[hb], 16, 64));
                        m = fmaxf(m, __shfl_xor(m, 32, 64));
                        if (qg == 0)
                            xm[kq][hd0 + 16 * hb] = m;
                    }
                    lds_barrier();
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
                        m_ref[hb] = fmaxf(xm[0][hd0 + 16 * hb], xm[1][hd0 + 16 * hb]);
                    lds_barrier();
                }
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    m_seen[hb] = fmaxf(m_seen[hb], mloc[hb]);
                    ovf |= mloc[hb] > m_ref[hb] + 100.f;
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p[e] = __builtin_amdgcn_exp2f(S[hb][e] - m_ref[hb]);  // masked: exp2(-inf) = 0
                    l_own[hb] += p[0] + p[1];
                    l_own[hb] += p[2] + p[3];
                    *(u32x2 *)(pw + 16 * hb * TB_PROWB) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                }
            }
            if (last_of_split(s)) {  // (row sum, reference maximum) to the PV team
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    float l = l_own[hb] + __shfl_xor(l_own[hb], 16, 64);
                    l = l + __shfl_xor(l, 32, 64);
                    float ms = fmaxf(m_seen[hb], __shfl_xor(m_seen[hb], 16, 64));
                    ms = fmaxf(ms, __shfl_xor(ms, 32, 64));
                    const int hd = hd0 + 16 * hb;
                    if (qg == 0) {
                        xl[gs & 1][kq][hd] = l;
                        if (kq == 0)
                            xr[gs & 1][hd] = m_ref[hb];
                        if (need_ref)
                            xs[gs][kq][hd] = ms;
                    }
                }
                if (ovf)
                    atomicOr(&sh_ovf, 1u << gs);
            }
        };

        // Q^T from LDS; the staging slots are cleared once every S wave has its copy
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int t = 0; t < 18; ++t)
                qT[hb][t] = __builtin_bit_cast(
                    bf16x8, *(const u32x4 *)(&ring[0][0] + TB_QOFF + (hd0 + 16 * hb) * TM_QROWB + 64 * t + 16 * qg));
        // pass 0: every tile of the group; pass 1 + gs: split gs again, if it overflowed
        uint32_t rerun = 0u;
        for (int pass = 0; pass <= group; ++pass) {
            const int t0 = pass == 0 ? 0 : (pass - 1) * tps;
            const int t1 = pass == 0 ? nt : min(nt, pass * tps);
            if ((pass == 0 && nt > 0) || (pass > 0 && ((rerun >> (pass - 1)) & 1u))) {
                Bf16Slot::issue(seq, lds0, sidx + 32 * t0, tw, lane, rc);  // tile t0, this wave's share
                lds_barrier();
                if (pass == 0)
                    for (int e = tid; e < 2 * TB_SLOTB / 16; e += 256)
                        ((u32x4 *)(&ring[0][0] + TB_QOFF))[e] = u32x4{0u, 0u, 0u, 0u};
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                lds_barrier();  // tile t0 has landed
                for (int s = t0; s <= t1; ++s) {
                    if (s < t1)
                        s_step(s, t0, pass == 0, s + 1 < t1);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's share of tile s + 1
                    lds_barrier();
                }
            }
            if (pass == 0) {
                __syncthreads();
                rerun = sh_ovf;
            }
        }
    } else {
        // ================================ PV team ================================
        // wave b: dims 128 b .. +127 of all 64 heads
        const int b = tw;
        f32x16 O[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            O[mt][0] = O[mt][1] = f32x16{};

        // this sequence's rows, or with paged caches the whole cache (host: at most 4 GiB - 1 MiB)
        const bool paged = L.block_table != nullptr;
        const int64_t seq_bytes = (paged ? L.cache_rows : r.n) * 1152;
        const i32x4 seq = buffer_desc((const uint8_t *)Ld.kv + (paged ? 0 : r.kv_base) * 1152, seq_bytes);
        const uint32_t lds0 = lds_addr_of(&ring[0][0]);
        uint32_t rc[Bf16Slot::PER_WAVE];
        Bf16Slot::geometry(4 + b, lane, rc);
        // V^T read geometry (ds_read_b64_tr_b16): lane reads rows 4g + ((lane & 15) >> 2) and
        // +8 of a 16-key step at dims 128 b + 16 ((lane >> 4) & 1) + 4 (lane & 3) (+32 mt): the
        // operand's keys 4g + 0..3 and 8 + 4g + 0..3 of the step
        const int voffs = (4 * g + ((lane & 15) >> 2)) * TB_ROWB + 2 * (128 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

        // O^T += V^T . P^T over the 32 keys of tile t (pass starting at t0); with gather, this
        // wave's share of tile t + 2 issued between the MFMAs
        auto pv_tile = [&](int t, int t0, bool gather) __attribute__((always_inline)) {
            int voff[Bf16Slot::PER_WAVE];
            const uint32_t nslot = lds0 + (uint32_t)((t + 2 - t0) % TB_SLOTS) * TB_SLOTB;
            if (gather)
                Bf16Slot::offsets(sidx + 32 * (t + 2), rc, voff);
            const char *vb0 = &ring[0][0] + ((t - t0) % TB_SLOTS) * TB_SLOTB + voffs;
            const char *pb = &pbuf[(t - t0) & 1][0] + j * TB_PROWB + 8 * g;
            s16x4 V[2][4][2];
            auto v_load = [&](int u, s16x4 (&Vd)[4][2]) __attribute__((always_inline)) {
                const char *vb = vb0 + 16 * u * TB_ROWB;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    Vd[mt][0] = lds_tr16(vb + 64 * mt);
                    Vd[mt][1] = lds_tr16(vb + 8 * TB_ROWB + 64 * mt);
                }
            };
            v_load(0, V[0]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u + 1 < 2)
                    v_load(u + 1, V[1]);
                // keys 16u + 4g + 0..3 and 16u + 8 + 4g + 0..3 of heads j, 32 + j
                bf16x8 pp[2];
#pragma unroll
                for (int nh = 0; nh < 2; ++nh) {
                    const char *pr = pb + 32 * nh * TB_PROWB + 32 * u;
                    const u32x2 lo = *(const u32x2 *)pr, hi = *(const u32x2 *)(pr + 16);
                    pp[nh] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const s16x4 lo = V[u][mt][0], hi = V[u][mt][1];
                    typedef short s16x8 __attribute__((ext_vector_type(8)));
                    const bf16x8 va = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                    O[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[0], O[mt][0], 0, 0, 0);
                    O[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[1], O[mt][1], 0, 0, 0);
                    const int q = 4 * u + mt;  // loads 0..4 after the first five MFMA pairs
                    if (gather && q < Bf16Slot::PER_WAVE)
                        Bf16Slot::one(seq, nslot, 4 + b, lane, q, voff[q]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the split of tile t (pass starting at t0) is complete: its result out, O cleared
        auto finish_split = [&](int t, int t0) __attribute__((always_inline)) {
            const int gs = t / tps;
            char *slot = &ring[0][0] + ((t - t0) % TB_SLOTS) * TB_SLOTB;
            // head r's 256 bytes in row r of the tile's slot, the wave's columns 256 b .. +255
            auto stage = [&](int rr, int c) __attribute__((always_inline)) { return slot + rr * TB_ROWB + 256 * b + c; };
            float l[2], m[2];
#pragma unroll
            for (int nh = 0; nh < 2; ++nh) {
                l[nh] = xl[gs & 1][0][32 * nh + j] + xl[gs & 1][1][32 * nh + j];
                m[nh] = xr[gs & 1][32 * nh + j];
            }
            mla_team_store<OUT_F32>(O, l, m, Ld, i, orow, split0 + gs, nsplit, b, g, j, lane, stage, ws_o, ws_ml);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                O[mt][0] = O[mt][1] = f32x16{};
        };
        auto run = [&](int t0, int t1, bool need_ref) __attribute__((always_inline)) {
            Bf16Slot::issue(seq, lds0, sidx + 32 * t0, 4 + b, lane, rc);  // tile t0, this wave's share
            lds_barrier();  // (first pass: the S team has its copy of Q and clears slots 1..2)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();  // tile t0 has landed
            for (int s = t0; s <= t1; ++s) {
                // tile s + 1 goes into the slot of tile s - 2 (consumed in step s - 1)
                if (need_ref && s < t1 && first_of_split(s)) {
                    lds_barrier();  // the S team's two exchange barriers
                    lds_barrier();
                }
                if (s > t0)
                    pv_tile(s - 1, t0, s + 1 < t1);
                else if (s + 1 < t1)  // the pass's first step has no PV work
                    Bf16Slot::issue(seq, lds0 + (uint32_t)((s + 1 - t0) % TB_SLOTS) * TB_SLOTB, sidx + 32 * (s + 1),
                                    4 + b, lane, rc);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's share of tile s + 1
                // after the wait, so that the result's stores are the newest memory operations
                if (s > t0 && last_of_split(s - 1))
                    finish_split(s - 1, t0);
                lds_barrier();
            }
        };
        uint32_t rerun = 0u;
        for (int pass = 0; pass <= group; ++pass) {
            const int t0 = pass == 0 ? 0 : (pass - 1) * tps;
            const int t1 = pass == 0 ? nt : min(nt, pass * tps);
            if ((pass == 0 && nt > 0) || (pass > 0 && ((rerun >> (pass - 1)) & 1u)))
                run(t0, t1, pass == 0);
            if (pass == 0) {
                __syncthreads();
                rerun = sh_ovf;
            }
        }
        // splits past the end of the index list (none under the split policy): empty results
        for (int gs = 0; gs < group; ++gs)
            if (gs * tps >= nt) {
                const float l[2] = {0.f, 0.f}, m[2] = {-INFINITY, -INFINITY};
                auto stage = [&](int rr, int c) __attribute__((always_inline)) {
                    return &ring[0][0] + rr * TB_ROWB + 256 * b + c;
                };
                mla_team_store<OUT_F32>(O, l, m, Ld, i, orow, split0 + gs, nsplit, b, g, j, lane, stage, ws_o, ws_ml);
            }
    }
}

// ------------------------------------------------------------------------------------------
// bf16 latent rows, half the heads per block: one 4-wave block per (row, split, head half),
// 32-key tiles, ~56 KB of LDS and at most 256 registers per lane, so two blocks share a CU and
// one block's MFMAs run while the other waits on its softmax, exchanges or barriers.  The two
// head halves of a (row, split) gather the same rows; they are dealt to the same XCD, so the
// second gather hits L2.
// Wave w = dq: S^T partials [32 keys x 32 heads] over dims 144 dq .. +143 (9 MFMA), a 4-way
// exchange after which wave dq holds the full logits of keys 8 dq + 4 g + 0..3 (summed in wave
// order 0, 1, 2, 3), their softmax numerators, and O^T for dims 128 dq .. +127 of the 32 heads
// over all 32 keys (8 MFMA; P of keys 16 u + 4 g + e comes from wave 2u, of 16 u + 8 + 4 g + e
// from wave 2u + 1, in the key order of ds_read_b64_tr_b16).
// ------------------------------------------------------------------------------------------
constexpr int HH_TILE = 32;                          // keys per tile
// bf16 rows up to this many use mla_hh_kernel: measured on 8192-token decode, the half-head
// blocks win at 8-32 rows, tie at 64 and lose from 128 rows on (96.1 against 91.2 us at 128,
// 155 against 142 at 256), where the full-head kernel's single staging of each row pays
constexpr int64_t MLA_HH_MAX_ROWS = 64;
constexpr int HH_TILEB = HH_TILE * M_ROWB;           // 37376 B
constexpr int HH_PIECES = HH_TILE * 72;              // 16-byte pieces per tile
constexpr int HH_N = HH_PIECES / M_THREADS;          // 9 per thread
static_assert(HH_PIECES % M_THREADS == 0, "staging");
constexpr int HH_EROWB = 1040;                       // output staging row stride
static_assert(32 * HH_EROWB <= HH_TILEB, "output staging fits the tile buffer");

template <bool OUT_F32>
__global__ __launch_bounds__(M_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void mla_hh_kernel(
    LayoutDev L, int64_t T, int64_t n_rows, MlaLayersDev layers, const int32_t *__restrict__ indices, int k,
    float sm_scale, int nsplit, int tiles_per_split, int64_t pairs_per_xcd, float *__restrict__ ws_o,
    float *__restrict__ ws_ml)
{
    __shared__ __attribute__((aligned(16))) char kt[HH_TILEB];
    __shared__ __attribute__((aligned(16))) f32x4 xs[4][4][64];  // S^T quarter partials [from][to][lane]
    __shared__ __attribute__((aligned(16))) u32x2 xp[4][64];     // P of each wave's keys (4 bf16)
    __shared__ float xm[4][32];                                   // per-head stats across the waves
    __shared__ int32_t sidx[2][HH_TILE];
    __shared__ int sh_flag;

    const int64_t pair = xcd_pair(pairs_per_xcd);  // (row, split, head half), head half fastest
    if (pair >= n_rows * nsplit * 2)
        return;
    const int hh = (int)(pair & 1);
    const int64_t rs = pair >> 1;
    const int64_t orow = rs / nsplit;
    const int split = (int)(rs % nsplit);
    const int layer = (int)(orow / T);
    const int64_t i = orow % T;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, j = lane & 31;
    const int dq = w;
    const MlaLayerDev Ld = layers.l[layer];
    const RowInfo r = row_info(L, i);
    const float c2 = sm_scale * Ld.kv_scale * LOG2E;

    // this split's index slots [s0, s0 + nsl) as 32-key tiles
    const int s0 = split * tiles_per_split * M_TILE;
    const int nsl = max(0, min(k - s0, tiles_per_split * M_TILE));
    const int ntiles = (nsl + HH_TILE - 1) / HH_TILE;
    const int32_t *irow = indices + i * k + s0;
    auto load_idx = [&](int tt) -> int32_t {  // slot `tid` of tile tt (tid < 32)
        const int e = tt * HH_TILE + tid;
        return (tt < ntiles && e < nsl) ? irow[e] : -1;
    };
    int32_t i0 = -1, i1 = -1, i2 = -1;
    if (tid < HH_TILE) {
        i0 = load_idx(0);
        i1 = load_idx(1);
        i2 = load_idx(2);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Q^T: head 32 hh + j, dims 144 dq + 16 t + 8 g .. +7 (t < 9)
    bf16x8 qT[9];
    {
        const uint16_t *qp = (const uint16_t *)Ld.q + ((i * M_H + 32 * hh + j) * M_DQK + 144 * dq + 8 * g);
#pragma unroll
        for (int t = 0; t < 9; ++t)
            qT[t] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * t));
    }
    f32x16 O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        O[mt] = f32x16{};

    // this sequence's rows, or with paged caches the whole cache (host: at most 4 GiB - 1 MiB)
    const bool paged = L.block_table != nullptr;
    const int64_t seq_bytes = (paged ? L.cache_rows : r.n) * (2 * M_DQK);
    const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const uint8_t *)Ld.kv + (paged ? 0 : r.kv_base) * (2 * M_DQK)), (short)0, (int)(uint32_t)seq_bytes,
        BUF_DWORD3);
    u32x4 R[HH_N];
    // thread t stages tile row t >> 3, 16-byte pieces (t & 7) + 8 u (u < 9): one index per
    // thread and tile, and every load instruction reads whole 128-byte lines of 8 rows
    static_assert(HH_N * 8 == 72 && HH_TILE * 8 == M_THREADS, "one tile row per 8 threads");
    const int hrow = tid >> 3, hcol = tid & 7;
    auto gather = [&](int32_t row_idx) {  // this thread's pieces of the tile row row_idx
#pragma unroll
        for (int u = 0; u < HH_N; ++u)
            R[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 seq, row_offset(row_idx, 2 * M_DQK, hcol + 8 * u), 0, 0));
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < HH_N; ++u)
            *(u32x4 *)(kt + hrow * M_ROWB + 16 * (hcol + 8 * u)) = R[u];
    };

    const int aoffs = j * M_ROWB + 2 * (144 * dq + 8 * g);
    const int voffs = (4 * g + ((lane & 15) >> 2)) * M_ROWB + 2 * (128 * dq + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    float m_ref = -INFINITY;   // identical in the 4 waves (same reference for head j)
    float m_seen = -INFINITY;  // max over this wave's keys
    float l_own = 0.f;         // sum of p over this lane's keys
    bool ovf = false;

    auto run = [&]() {
        if (tid < HH_TILE) {
            sidx[0][tid] = i0;
            sidx[1][tid] = i1;
        }
        if (tid == 0)
            sh_flag = 0;
        int32_t idx_next = i2;
        lds_barrier();  // Q stays in flight
        if (ntiles > 0) {
            gather(sidx[0][hrow]);
            stage();
        }
        __builtin_amdgcn_s_waitcnt(0x0070);  // nothing known to the compiler stays in flight
        lds_barrier();
        for (int tt = 0; tt < ntiles; ++tt) {
            const int buf = tt & 1;
            const bool gather_next = tt + 1 < ntiles;
            if (gather_next)  // this thread's row of the next tile, requested before any compute
                gather(sidx[buf ^ 1][hrow]);
            const uint32_t valid = (uint32_t)__ballot(lane < HH_TILE && sidx[buf][lane & 31] >= 0);

            // ---- 1. S^T partial over this wave's 144 dims
            f32x16 S = f32x16{};
            {
                const char *arow = kt + aoffs;
                u32x4 A[2][3];
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    A[0][t] = *(const u32x4 *)(arow + 32 * t);
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const int cur = c & 1;
                    if (c + 1 < 3) {
#pragma unroll
                        for (int t = 0; t < 3; ++t)
                            A[cur ^ 1][t] = *(const u32x4 *)(arow + 32 * (3 * (c + 1) + t));
                    }
#pragma unroll
                    for (int t = 0; t < 3; ++t)
                        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A[cur][t]),
                                                                    qT[3 * c + t], S, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- 2. quarter exchange: s = sum over waves 0..3 of their partials of this wave's keys
            // (all four quarters go through LDS, own one included: no per-lane selects)
#pragma unroll
            for (int d2 = 0; d2 < 4; ++d2)
                xs[dq][d2][lane] = f32x4{S[4 * d2], S[4 * d2 + 1], S[4 * d2 + 2], S[4 * d2 + 3]};
            lds_barrier();
            float s[4];
            {
                const f32x4 p0 = xs[0][dq][lane], p1 = xs[1][dq][lane], p2 = xs[2][dq][lane], p3 = xs[3][dq][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[e] = ((p0[e] + p1[e]) + p2[e]) + p3[e];
            }

            // ---- 3. softmax numerators of keys 8 dq + 4 g + e of head j
            const uint32_t vk = (valid >> (8 * dq + 4 * g)) & 15u;
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[e] = ((vk >> e) & 1u) ? s[e] * c2 : -INFINITY;
                mloc = fmaxf(mloc, s[e]);
            }
            mloc = fmaxf(mloc, other_half(mloc, g));
            if (m_ref == -INFINITY && valid != 0u) {
                // first non-empty tile (block-uniform): the 4 waves agree on the reference
                if (g == 0)
                    xm[w][j] = mloc;
                lds_barrier();
                m_ref = fmaxf(fmaxf(xm[0][j], xm[1][j]), fmaxf(xm[2][j], xm[3][j]));
                lds_barrier();
            }
            m_seen = fmaxf(m_seen, mloc);
            ovf |= mloc > m_ref + 100.f;
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[e] - m_ref);
                l_own += p[e];
            }
            xp[w][lane] = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[0], p[1]}, bf16x2)),
                                __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2], p[3]}, bf16x2))};
            lds_barrier();

            // ---- 4. O^T += V^T . P^T over the 32 keys (2 steps of 16 keys x 4 dim blocks)
            {
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const char *vbase = kt + voffs;
                s16x4 V[2][4][2];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        V[u][mt][0] = lds_tr16(vbase + 16 * u * M_ROWB + 64 * mt);
                        V[u][mt][1] = lds_tr16(vbase + (16 * u + 8) * M_ROWB + 64 * mt);
                    }
                const u32x2 pa0 = xp[0][lane], pa1 = xp[1][lane], pa2 = xp[2][lane], pa3 = xp[3][lane];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const u32x2 lo2 = u ? pa2 : pa0, hi2 = u ? pa3 : pa1;
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const s16x4 lo = V[u][mt][0], hi = V[u][mt][1];
                        const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        O[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), bop, O[mt],
                                                                        0, 0, 0);
                    }
                }
            }
            lds_barrier();  // tile, partials and P consumed
            if (tt + 1 < ntiles)
                stage();
            if (tid < HH_TILE) {
                sidx[buf][tid] = idx_next;  // tile tt + 2
                idx_next = load_idx(tt + 3);
            }
            lds_barrier();
        }
    };
    run();
    if (ovf)
        sh_flag = 1;
    __syncthreads();
    if (sh_flag) {  // rare: rerun with the exact maximum of the first run as the reference
        if (g == 0)
            xm[w][j] = m_seen;
        __syncthreads();
        m_ref = fmaxf(fmaxf(xm[0][j], xm[1][j]), fmaxf(xm[2][j], xm[3][j]));
        l_own = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            O[mt] = f32x16{};
        __syncthreads();
        run();
    }

    // ---- row sum of head j over all keys: lane halves, then the 4 waves in order
    float l_w = l_own + other_half(l_own, g);
    __syncthreads();
    if (g == 0)
        xm[w][j] = l_w;
    __syncthreads();
    const float l_run = ((xm[0][j] + xm[1][j]) + xm[2][j]) + xm[3][j];

    // ---- epilogue: this block's 32 heads x 512 dims (O / l, or the normalised output)
    const int head = 32 * hh + j;
    const float inv = (l_run > 0.f) ? (nsplit == 1 ? Ld.kv_scale / l_run : 1.f / l_run) : 0.f;
    if (OUT_F32) {
        float *dst = (nsplit == 1) ? (float *)Ld.out + (i * M_H + head) * M_DC
                                   : ws_o + ((orow * nsplit + split) * M_H + head) * M_DC;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 128 * dq + 32 * mt + 8 * q4 + 4 * g;
                *(f32x4 *)(dst + d) = f32x4{O[mt][4 * q4] * inv, O[mt][4 * q4 + 1] * inv, O[mt][4 * q4 + 2] * inv,
                                            O[mt][4 * q4 + 3] * inv};
            }
    } else {
        __syncthreads();  // the tile buffer becomes the output staging area
        char *srow = kt + j * HH_EROWB;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 128 * dq + 32 * mt + 8 * q4 + 4 * g;
                *(u32x2 *)(srow + 2 * d) = u32x2{pack_bf16x2(O[mt][4 * q4] * inv, O[mt][4 * q4 + 1] * inv),
                                                 pack_bf16x2(O[mt][4 * q4 + 2] * inv, O[mt][4 * q4 + 3] * inv)};
            }
        __syncthreads();
        char *dst = (nsplit == 1) ? (char *)((uint16_t *)Ld.out + (i * M_H + 32 * hh) * M_DC)
                                  : (char *)((uint16_t *)ws_o + ((orow * nsplit + split) * M_H + 32 * hh) * M_DC);
#pragma unroll
        for (int u = 0; u < 32 * M_DC * 2 / (16 * M_THREADS); ++u) {
            const int c = tid + M_THREADS * u, h = c >> 6, c16 = c & 63;
            *(u32x4 *)(dst + h * (M_DC * 2) + 16 * c16) = *(const u32x4 *)(kt + h * HH_EROWB + 16 * c16);
        }
    }
    if (nsplit == 1) {
        if (Ld.lse && dq == 0 && g == 0)
            Ld.lse[i * M_H + head] = (l_run > 0.f) ? (m_ref + __log2f(l_run)) * LN2 : -INFINITY;
    } else if (dq == 0 && g == 0) {
        float *pml = ws_ml + ((orow * nsplit + split) * M_H + head) * 2;
        pml[0] = m_ref;
        pml[1] = l_run;
    }
}

constexpr int MLA_MAX_SPLITS = 32;  // the split count never exceeds this (mla_num_splits)
constexpr int MLA_MIN_TILES_BF16 = 2;  // fewest tiles per split (see mla_num_splits)
constexpr int MLA_MIN_TILES_FP8 = 8;

// Combine the split partials of every (output row, head), in split order.  One block of 4
// waves (or of 1 wave, when there are few rows) per (row, head group): wave w takes head
// (waves per block) blockIdx.y + w, lane l its dims 8l .. 8l + 7
// (16 bytes of a bf16 partial).  Partial s holds O_s / l_s, so its weight is l_s 2^(m_s - M) /
// sum over splits of the same; the wave works the weights out itself (lane s holds split s),
// so the block has no barrier.  NSB bounds the split count (register arrays).
template <bool OUT_F32, int NSB>
__global__ __launch_bounds__(256) void mla_combine_kernel(int64_t T, MlaLayersDev layers, int nsplit,
                                                          const float *__restrict__ ws_o,
                                                          const float *__restrict__ ws_ml)
{
    const int64_t orow = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int head = (int)(blockDim.x >> 6) * (int)blockIdx.y + (tid >> 6);
    const int layer = (int)(orow / T);
    const int64_t i = orow % T;
    const MlaLayerDev Ld = layers.l[layer];
    // every split's partial is requested first (independent of the weights), so their
    // latencies overlap each other and the weight computation
    const int64_t pbase = (orow * nsplit * M_H + head) * M_DC + 8 * lane;
    typedef typename std::conditional<OUT_F32, f32x4, u32x4>::type Piece;
    Piece pv[NSB][OUT_F32 ? 2 : 1];
#pragma unroll
    for (int sp = 0; sp < NSB; ++sp) {
        if (sp < nsplit) {
            const int64_t pe = pbase + (int64_t)sp * M_H * M_DC;
            if constexpr (OUT_F32) {
                pv[sp][0] = *(const f32x4 *)(ws_o + pe);
                pv[sp][OUT_F32 ? 1 : 0] = *(const f32x4 *)(ws_o + pe + 4);
            } else {
                pv[sp][0] = *(const u32x4 *)((const uint16_t *)ws_o + pe);
            }
        }
    }
    const float *ml = ws_ml + (orow * nsplit * M_H + head) * 2;
    const float ms = lane < nsplit ? ml[lane * M_H * 2] : -INFINITY;
    const float ls = lane < nsplit ? ml[lane * M_H * 2 + 1] : 0.f;
    const float mx = wave_max(ms);
    const float e = (mx == -INFINITY || lane >= nsplit) ? 0.f : exp2f(ms - mx);
    // fixed-order total: splits summed in index order (every lane the same sum)
    float tot = 0.f;
    for (int s2 = 0; s2 < nsplit; ++s2)
        tot += __shfl(e * ls, s2, 64);
    const float inv = tot > 0.f ? Ld.kv_scale / tot : 0.f;
    const float wl = e * ls * inv;  // split `lane`'s weight (partials are O / l)
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < NSB; ++sp) {
        if (sp < nsplit) {
            float v[8];
            if constexpr (OUT_F32) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    v[e2] = pv[sp][0][e2];
                    v[4 + e2] = pv[sp][OUT_F32 ? 1 : 0][e2];
                }
            } else {
                const u32x4 bw = pv[sp][0];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    v[2 * e2] = __uint_as_float(bw[e2] << 16);
                    v[2 * e2 + 1] = __uint_as_float(bw[e2] & 0xFFFF0000u);
                }
            }
            const float wgt = __shfl(wl, sp, 64);
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2)
                acc[e2] = fmaf(wgt, v[e2], acc[e2]);
        }
    }
    const int64_t o = (i * M_H + head) * M_DC + 8 * lane;
    if (OUT_F32) {
        *(f32x4 *)((float *)Ld.out + o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *(f32x4 *)((float *)Ld.out + o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
        *(u32x4 *)((uint16_t *)Ld.out + o) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
    if (Ld.lse && lane == 0)
        Ld.lse[i * M_H + head] = tot > 0.f ? (mx + __log2f(tot)) * LN2 : -INFINITY;
}

// ------------------------------------------------------------------------------------------
// generic kernel: one block per (query row, head, layer); fp32 math, two passes over keys.
// ------------------------------------------------------------------------------------------
constexpr int G_THREADS = 256;

template <int QDT, int KVDT, bool OUT_F32>
__global__ __launch_bounds__(G_THREADS) void mla_generic_kernel(LayoutDev L, int H, int Dc, int Dr,
                                                                MlaLayersDev layers,
                                                                const int32_t *__restrict__ indices,
                                                                int k, float sm_scale)
{
    extern __shared__ float gsm[];  // q [Dqk], z [k], red [G_THREADS/64]
    const int Dqk = Dc + Dr;
    const int64_t i = blockIdx.x;
    const int h = blockIdx.y, layer = blockIdx.z;
    const MlaLayerDev Ld = layers.l[layer];
    const RowInfo r = row_info(L, i);
    float *sq = gsm, *z = gsm + Dqk, *red = z + k;
    const int tid = threadIdx.x;
    for (int d = tid; d < Dqk; d += G_THREADS)
        sq[d] = load_elem<QDT>(Ld.q, ((int64_t)i * H + h) * Dqk + d);
    __syncthreads();
    const float zs = sm_scale * Ld.kv_scale;
    float mx = -INFINITY;
    for (int jj = tid; jj < k; jj += G_THREADS) {
        const int32_t idx = indices[i * k + jj];
        float zz = -INFINITY;
        if (idx >= 0) {
            const int64_t row = ((L.block_table ? 0 : r.kv_base) + idx) * Dqk;  // physical when paged
            float acc = 0.f;
            for (int d = 0; d < Dqk; ++d)
                acc = fmaf(sq[d], load_elem<KVDT>(Ld.kv, row + d), acc);
            zz = acc * zs;
        }
        z[jj] = zz;
        mx = fmaxf(mx, zz);
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int w2 = 1; w2 < G_THREADS / 64; ++w2)
        mx = fmaxf(mx, red[w2]);
    __syncthreads();
    float sum = 0.f;
    for (int jj = tid; jj < k; jj += G_THREADS) {
        const float p = (mx == -INFINITY || z[jj] == -INFINITY) ? 0.f : __expf(z[jj] - mx);
        z[jj] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if ((tid & 63) == 0)
        red[tid >> 6] = sum;
    __syncthreads();
    float tot = 0.f;
    for (int w2 = 0; w2 < G_THREADS / 64; ++w2)
        tot += red[w2];
    const float inv = tot > 0.f ? Ld.kv_scale / tot : 0.f;
    for (int e = tid; e < Dc; e += G_THREADS) {
        float acc = 0.f;
        for (int jj = 0; jj < k; ++jj) {
            const int32_t idx = indices[i * k + jj];
            if (idx >= 0)
                acc = fmaf(z[jj], load_elem<KVDT>(Ld.kv, ((L.block_table ? 0 : r.kv_base) + idx) * Dqk + e), acc);
        }
        const float o = acc * inv;
        const int64_t oo = ((int64_t)i * H + h) * Dc + e;
        if (OUT_F32)
            ((float *)Ld.out)[oo] = o;
        else
            ((uint16_t *)Ld.out)[oo] = (uint16_t)f32_to_bf16_bits(o);
    }
    if (Ld.lse && tid == 0)
        Ld.lse[i * H + h] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
// Key splits per (query row, layer).  They depend on the query rows T of one layer and on k
// only, never on the layer count: a layer run through the shared entry then sums its keys in
// exactly the same blocks and order as a single-layer call, and its output is the same bit
// for bit.  The shared entry adds (row, layer) blocks instead of changing the split.
//
// min_tiles: the fewest 64-key tiles a split may hold.  bf16 latent (half-head decode kernel):
// 2 -- a second tile hides the first one's fixed costs better than a second wave of split
// partials does (measured on 8-row decode).  fp8 latent: 8 -- a block's fixed costs (index
// list, Q, the first gathers' latency, the partial's store) are ~20K cycles against ~7.5K per
// tile, so 4-tile splits lose even with twice the blocks (64-row ragged decode: 512 blocks of 4
// tiles 59 us, 256 blocks of 8 tiles 48 us).
// ------------------------------------------------------------------------------------------
// Gather ceiling (a measurement aid, no method arithmetic): the row traffic of the sparse-MLA
// stage alone.  One 512-thread block per 256 index slots of one index row gathers those rows
// into LDS with the same buffer-to-LDS loads and slot geometry as the team kernels (eight
// waves share each 32-row slot, three slots in flight, then a wait), and discards them.
// ------------------------------------------------------------------------------------------
constexpr int GC_ROWS = 256;  // index slots per block
template <int RB>
__global__ __launch_bounds__(TM_THREADS) void gather_ceiling_kernel(const uint8_t *__restrict__ rows,
                                                                    int64_t n_rows,
                                                                    const int32_t *__restrict__ indices,
                                                                    int k, int chunks, uint32_t *sink)
{
    typedef SlotDma<RB, 8> Slot;
    __shared__ __attribute__((aligned(16))) char ring[3][Slot::SLOTB];
    __shared__ int32_t sidx[GC_ROWS];
    const int64_t row = blockIdx.x / chunks;
    const int c0 = (int)(blockIdx.x % chunks) * GC_ROWS;
    const int n = min(GC_ROWS, k - c0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < GC_ROWS)
        sidx[tid] = tid < n ? indices[row * k + c0 + tid] : -1;
    __syncthreads();
    const i32x4 seq = buffer_desc(rows, n_rows * RB);
    const uint32_t lds0 = lds_addr_of(&ring[0][0]);
    uint32_t rc[Slot::PER_WAVE];
    Slot::geometry(w, lane, rc);
    const int ntile = (n + 31) / 32;
    for (int t = 0; t < ntile; ++t) {
        Slot::issue(seq, lds0 + (uint32_t)(t % 3) * Slot::SLOTB, sidx + 32 * t, w, lane, rc);
        if (t % 3 == 2 || t + 1 == ntile) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    if (tid == 0 && blockIdx.x == 0)
        sink[0] = *(const uint32_t *)&ring[0][0];
}

hipError_t launch_gather_ceiling(const void *rows, int64_t n_rows, int row_bytes, const int32_t *indices, int64_t T,
                                 int k, uint32_t *sink, hipStream_t stream)
{
    const int chunks = (k + GC_ROWS - 1) / GC_ROWS;
    const dim3 grid((unsigned)(T * chunks));
    if (row_bytes == 576)
        hipLaunchKernelGGL(gather_ceiling_kernel<576>, grid, dim3(TM_THREADS), 0, stream, (const uint8_t *)rows,
                           n_rows, indices, k, chunks, sink);
    else
        hipLaunchKernelGGL(gather_ceiling_kernel<1152>, grid, dim3(TM_THREADS), 0, stream, (const uint8_t *)rows,
                           n_rows, indices, k, chunks, sink);
    return hipGetLastError();
}

int mla_num_splits(int64_t rows, int k, int min_tiles)
{
    const int ntiles = (k + M_TILE - 1) / M_TILE;
    if (rows <= 0)
        return 1;
    int64_t ns = (MLA_TARGET_BLOCKS + rows - 1) / rows;
    if (ns > ntiles / min_tiles)
        ns = ntiles / min_tiles;
    if (const char *env = getenv("DSA_MLA_SPLITS")) {  // tuning sweeps: a fixed split count
        const long v = strtol(env, nullptr, 10);
        if (v >= 1 && v <= MLA_MAX_SPLITS)
            ns = v;
    }
    if (ns > ntiles)
        ns = ntiles;
    if (ns > MLA_MAX_SPLITS)
        ns = MLA_MAX_SPLITS;
    if (ns < 1)
        ns = 1;
    const int tps = (ntiles + (int)ns - 1) / (int)ns;  // equal tiles per split
    return (ntiles + tps - 1) / tps;
}

size_t mla_workspace_bytes(int64_t T, int n_layers, int k)
{
    const size_t rows = (size_t)T * n_layers;
    // the most splits any tuned kernel takes (the bf16 policy), so one size serves both dtypes
    const int ns = mla_num_splits(T, k, MLA_MIN_TILES_BF16);
    if (ns <= 1)
        return 0;
    size_t o = rows * ns * M_H * M_DC * sizeof(float);
    size_t ml = rows * ns * M_H * 2 * sizeof(float);
    return o + ml;
}

hipError_t launch_mla_tuned(const LayoutDev &L, int64_t T, const MlaLayersDev &layers, int n_layers,
                            bool kv_fp8, bool out_f32, const int32_t *indices, int k,
                            float sm_scale, void *workspace, hipStream_t stream)
{
    const int64_t rows = T * n_layers;
    // from one layer's rows and the latent dtype: layer-count independent
    const int ns = mla_num_splits(T, k, kv_fp8 ? MLA_MIN_TILES_FP8 : MLA_MIN_TILES_BF16);
    const int ntiles = (k + M_TILE - 1) / M_TILE;
    const int tps = (ntiles + ns - 1) / ns;
    float *wo = nullptr, *wml = nullptr;
    if (ns > 1) {
        wo = (float *)workspace;
        wml = wo + (size_t)rows * ns * M_H * M_DC;
    }
    const int64_t pairs = rows * ns;
    if (kv_fp8) {
        // consecutive splits of a row share a block while that leaves a block per CU: the
        // splits (and so every result bit) stay those of the policy above, only their
        // scheduling changes
        int group = 1;
        while (group * 2 <= TM_MAX_GROUP && ns % (group * 2) == 0 && pairs / (group * 2) >= MLA_TARGET_BLOCKS)
            group *= 2;
        const int64_t gpx = (pairs / group + 7) / 8;
        dim3 fgrid((unsigned)(8 * gpx));
        if (out_f32)
            hipLaunchKernelGGL((mla_fp8_kernel<true>), fgrid, dim3(TM_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, tps, group, gpx, wo, wml);
        else
            hipLaunchKernelGGL((mla_fp8_kernel<false>), fgrid, dim3(TM_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, tps, group, gpx, wo, wml);
    } else if (T <= MLA_HH_MAX_ROWS) {
        // few rows (decode): half-head blocks, two per CU
        const int64_t hpairs = pairs * 2, hppx = (hpairs + 7) / 8;
        dim3 hgrid((unsigned)(8 * hppx));
        if (out_f32)
            hipLaunchKernelGGL((mla_hh_kernel<true>), hgrid, dim3(M_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, tps, hppx, wo, wml);
        else
            hipLaunchKernelGGL((mla_hh_kernel<false>), hgrid, dim3(M_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, tps, hppx, wo, wml);
    } else {
        // many rows (prefill): the two-team kernel, 32-key tiles (two per policy tile)
        int group = 1;
        while (group * 2 <= TM_MAX_GROUP && ns % (group * 2) == 0 && pairs / (group * 2) >= MLA_TARGET_BLOCKS)
            group *= 2;
        const int64_t gpx = (pairs / group + 7) / 8;
        dim3 bgrid((unsigned)(8 * gpx));
        if (out_f32)
            hipLaunchKernelGGL((mla_bf16_team_kernel<true>), bgrid, dim3(TM_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, 2 * tps, group, gpx, wo, wml);
        else
            hipLaunchKernelGGL((mla_bf16_team_kernel<false>), bgrid, dim3(TM_THREADS), 0, stream, L, T, rows, layers,
                               indices, k, sm_scale, ns, 2 * tps, group, gpx, wo, wml);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1)
        return e;
    // four heads per block, or one when that would leave fewer than 512 blocks
    const int hpb = rows * (M_H / 4) >= 512 ? 4 : 1;
    dim3 cgrid((unsigned)rows, M_H / hpb);
    const dim3 cblock(64 * hpb);
#define DSA_COMBINE(NSB)                                                                                         \
    do {                                                                                                         \
        if (out_f32)                                                                                             \
            hipLaunchKernelGGL((mla_combine_kernel<true, NSB>), cgrid, cblock, 0, stream, T, layers, ns, wo, wml); \
        else                                                                                                     \
            hipLaunchKernelGGL((mla_combine_kernel<false, NSB>), cgrid, cblock, 0, stream, T, layers, ns, wo, wml); \
    } while (0)
    if (ns <= 4)
        DSA_COMBINE(4);
    else if (ns <= 8)
        DSA_COMBINE(8);
    else if (ns <= 16)
        DSA_COMBINE(16);
    else
        DSA_COMBINE(MLA_MAX_SPLITS);
#undef DSA_COMBINE
    return hipGetLastError();
}

template <int QDT, int KVDT, bool OF>
static hipError_t launch_generic_t(const LayoutDev &L, int64_t T, int H, int Dc, int Dr,
                                   const MlaLayersDev &layers, int n_layers, const int32_t *indices,
                                   int k, float sm_scale, hipStream_t stream)
{
    dim3 grid((unsigned)T, (unsigned)H, (unsigned)n_layers);
    size_t shmem = sizeof(float) * (size_t)(Dc + Dr + k + G_THREADS / 64);
    hipLaunchKernelGGL((mla_generic_kernel<QDT, KVDT, OF>), grid, dim3(G_THREADS), shmem, stream, L,
                       H, Dc, Dr, layers, indices, k, sm_scale);
    return hipGetLastError();
}

hipError_t launch_mla_generic(const LayoutDev &L, int64_t T, int H, int Dc, int Dr,
                              const MlaLayersDev &layers, int n_layers, int q_dt, int kv_dt,
                              bool out_f32, const int32_t *indices, int k, float sm_scale,
                              hipStream_t stream)
{
#define DSA_MLA_G(QD, KD)                                                                        \
    if (q_dt == QD && kv_dt == KD)                                                               \
        return out_f32 ? launch_generic_t<QD, KD, true>(L, T, H, Dc, Dr, layers, n_layers, indices, \
                                                        k, sm_scale, stream)                     \
                       : launch_generic_t<QD, KD, false>(L, T, H, Dc, Dr, layers, n_layers,     \
                                                         indices, k, sm_scale, stream);
    DSA_MLA_G(0, 0) DSA_MLA_G(0, 1) DSA_MLA_G(0, 2)
    DSA_MLA_G(1, 0) DSA_MLA_G(1, 1) DSA_MLA_G(1, 2)
#undef DSA_MLA_G
    return hipErrorInvalidValue;
}

}  // namespace dsa
