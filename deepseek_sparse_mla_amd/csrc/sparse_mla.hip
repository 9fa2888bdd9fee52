// sparse_mla.hip -- sparse MLA over the selected latent rows, for gfx950.
//
// ("GLM-5.2 架构解剖", full structure diagram, sparse MLA box: 64 heads computed only on
// the 2048 selected rows of the 576-wide latent cache, 512 latent + 64 rope; layer
// scheduling: shared layers read the same index buffer.)  Absorbed form: the key is the
// whole 576-wide row, the value its first 512 entries, the output stays in latent space.
//
//   z_j = sm_scale * kv_scale * q_h . c_j ;  o_h = kv_scale * sum_j softmax(z)_j c_j[0:512]
//
// Tuned kernel (H = 64, Dc = 512, Dr = 64, bf16 q, bf16 or fp8 latent rows):
//  * one 256-thread block per (layer, query row, split of the index list); 4 waves,
//    wave w owns heads 32*(w&1) .. +31 and key half / output-dim half (w>>1);
//  * 64-row tiles of gathered latent rows are staged (fp8 widened exactly to bf16) into a
//    double-buffered LDS tile [64][576 (+8 pad)]; the next tile's rows are loaded into
//    registers while the current one is computed;
//  * S^T[keys x heads] = K . Q^T on v_mfma_f32_32x32x16_bf16 with Q^T held in registers,
//    so each lane owns one head column: the online-softmax max/sum need one cross-half
//    swap and one LDS exchange with the partner wave;
//  * O^T[dims x heads] += V^T . P^T, V^T read straight from the row-major tile with
//    ds_read_b64_tr_b16 (4 consecutive keys of one dim per lane);
//  * with several splits per row, partial (O, m, l) go to the workspace and the last block
//    to finish (integer counter) combines them in split order -- deterministic.
// Generic kernel: any H <= 128, Dc <= 512, Dqk <= 1024, fp32 everywhere, two passes.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int M_H = 64;
constexpr int M_DC = 512;
constexpr int M_DQK = 576;
constexpr int M_TILE = 64;                 // gathered rows per tile
constexpr int M_ROWB = 1168;               // LDS row stride in bytes (1152 + 16 pad)
constexpr int M_TILEB = M_TILE * M_ROWB;   // 74752 B per tile buffer
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr16(const char *lds_generic_ptr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(
            (__attribute__((address_space(3))) char *)(lds_generic_ptr)));
}

template <bool KV_FP8>
struct StageRegs {
    static constexpr int N = KV_FP8 ? 9 : 18;   // 16-byte pieces per thread per tile
    u32x4 v[N];
};

// Issue the global loads of one tile (rows given by sidx) into registers.
template <bool KV_FP8>
__device__ __forceinline__ void stage_load(StageRegs<KV_FP8> &R, const uint8_t *__restrict__ kv,
                                           int64_t kv_base, const int32_t *sidx, int tid)
{
    constexpr int PIECES = KV_FP8 ? 36 : 72;    // 16-byte pieces per row
    constexpr int ROWB = KV_FP8 ? 576 : 1152;   // bytes per row in HBM
#pragma unroll
    for (int u = 0; u < R.N; ++u) {
        const int c = tid + 256 * u;
        const int row = c / PIECES, col = c % PIECES;
        const int32_t idx = sidx[row];
        if (idx >= 0)
            R.v[u] = *(const u32x4 *)(kv + (kv_base + idx) * ROWB + col * 16);
        else
            R.v[u] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <bool KV_FP8>
__device__ __forceinline__ void stage_store(const StageRegs<KV_FP8> &R, char *tile, int tid)
{
    constexpr int PIECES = KV_FP8 ? 36 : 72;
#pragma unroll
    for (int u = 0; u < R.N; ++u) {
        const int c = tid + 256 * u;
        const int row = c / PIECES, col = c % PIECES;
        if (KV_FP8) {
            u32x4 lo, hi;
            lo[0] = fp8x2_to_bf16x2<false>(R.v[u][0]);
            lo[1] = fp8x2_to_bf16x2<true>(R.v[u][0]);
            lo[2] = fp8x2_to_bf16x2<false>(R.v[u][1]);
            lo[3] = fp8x2_to_bf16x2<true>(R.v[u][1]);
            hi[0] = fp8x2_to_bf16x2<false>(R.v[u][2]);
            hi[1] = fp8x2_to_bf16x2<true>(R.v[u][2]);
            hi[2] = fp8x2_to_bf16x2<false>(R.v[u][3]);
            hi[3] = fp8x2_to_bf16x2<true>(R.v[u][3]);
            u32x4 *dst = (u32x4 *)(tile + row * M_ROWB + col * 32);
            dst[0] = lo;
            dst[1] = hi;
        } else {
            *(u32x4 *)(tile + row * M_ROWB + col * 16) = R.v[u];
        }
    }
}

template <bool KV_FP8, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void mla_kernel(LayoutDev L, int64_t T, MlaLayersDev layers,
                                                     const int32_t *__restrict__ indices, int k,
                                                     float sm_scale, int nsplit, int tiles_per_split,
                                                     float *__restrict__ ws_o,
                                                     float *__restrict__ ws_ml,
                                                     int *__restrict__ ws_cnt)
{
    __shared__ __attribute__((aligned(16))) char kt[2][M_TILEB];
    __shared__ __attribute__((aligned(16))) u32x4 xch_p[4][64][2];   // P^T exchange (bf16)
    __shared__ float xch_m[4][32], xch_l[4][32];
    __shared__ int32_t sidx[2][M_TILE];
    __shared__ int sh_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, j = lane & 31;
    const int hh = wave & 1, kh = wave >> 1;  // head half; key half (S) and dim half (O)
    const int partner = wave ^ 2;
    const int split = blockIdx.x;
    const int64_t i = blockIdx.y;
    const int layer = blockIdx.z;
    const MlaLayerDev Ld = layers.l[layer];
    const RowInfo r = row_info(L, i);
    const float c2 = sm_scale * Ld.kv_scale * LOG2E;

    const int ntiles_all = (k + M_TILE - 1) / M_TILE;
    const int t_begin = split * tiles_per_split;
    const int t_end = min(ntiles_all, t_begin + tiles_per_split);
    const int ntiles = max(0, t_end - t_begin);
    const int32_t *irow = indices + i * k;

    // ---- Q^T operand: head 32*hh + j, dims 16t + 8g .. +7
    bf16x8 qT[36];
    {
        const uint16_t *qp = (const uint16_t *)Ld.q + ((i * M_H + 32 * hh + j) * M_DQK + 8 * g);
#pragma unroll
        for (int t = 0; t < 36; ++t)
            qT[t] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * t));
    }

    f32x16 O[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        O[mt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    auto load_idx = [&](int tt) -> int32_t {  // slot `tid` of tile tt (tid < 64)
        const int slot = (t_begin + tt) * M_TILE + tid;
        return (tt < ntiles && slot < k) ? irow[slot] : -1;
    };

    // ---- prologue: indices of tiles 0, 1; tile 0 staged
    if (tid < M_TILE) {
        sidx[0][tid] = load_idx(0);
        sidx[1][tid] = load_idx(1);
    }
    int32_t idx_next = tid < M_TILE ? load_idx(2) : -1;
    __syncthreads();
    StageRegs<KV_FP8> R;
    const uint8_t *kvb = (const uint8_t *)Ld.kv;
    if (ntiles > 0) {
        stage_load<KV_FP8>(R, kvb, r.kv_base, sidx[0], tid);
        stage_store<KV_FP8>(R, kt[0], tid);
    }
    __syncthreads();

    for (int tt = 0; tt < ntiles; ++tt) {
        const int buf = tt & 1;
        const char *tile = kt[buf];
        if (tt + 1 < ntiles)
            stage_load<KV_FP8>(R, kvb, r.kv_base, sidx[buf ^ 1], tid);

        const uint64_t valid = __ballot(sidx[buf][lane] >= 0);

        // ---- S^T = K . Q^T for this wave's 32 keys x 32 heads
        f32x16 s = {};
        {
            const char *arow = tile + (32 * kh + j) * M_ROWB + 16 * g;
#pragma unroll
            for (int t = 0; t < 36; ++t) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4 *)(arow + 32 * t));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qT[t], s, 0, 0, 0);
            }
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int key = 32 * kh + 8 * (rr >> 2) + 4 * g + (rr & 3);
            const float z = ((valid >> key) & 1ull) ? s[rr] * c2 : -INFINITY;
            s[rr] = z;
            mloc = fmaxf(mloc, z);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        if (g == 0)
            xch_m[wave][j] = mloc;
        __syncthreads();
        const float m_tile = fmaxf(mloc, xch_m[partner][j]);
        const float m_new = fmaxf(m_run, m_tile);
        float alpha, lloc = 0.f;
        uint32_t pk[8];
        if (m_new == -INFINITY) {
            alpha = 1.f;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                pk[q] = 0u;
        } else {
            alpha = exp2f(m_run - m_new);
            float p[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                p[rr] = exp2f(s[rr] - m_new);
                lloc += p[rr];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                pk[q] = pack_bf16x2(p[2 * q], p[2 * q + 1]);
        }
        lloc += __shfl_xor(lloc, 32, 64);
        xch_p[wave][lane][0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        xch_p[wave][lane][1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
        if (g == 0)
            xch_l[wave][j] = lloc;
        __syncthreads();
        const u32x4 pp0 = xch_p[partner][lane][0], pp1 = xch_p[partner][lane][1];
        const float lpart = xch_l[partner][j];
        l_run = l_run * alpha + (kh == 0 ? (lloc + lpart) : (lpart + lloc));
        m_run = m_new;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                O[mt][rr] *= alpha;

        // ---- O^T += V^T . P^T over the 64 keys (4 steps of 16)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int khu = u >> 1, jj = u & 1;
            u32x4 bw;
            if (khu == kh)
                bw = (jj == 0) ? u32x4{pk[0], pk[1], pk[2], pk[3]} : u32x4{pk[4], pk[5], pk[6], pk[7]};
            else
                bw = (jj == 0) ? pp0 : pp1;
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
            const int key0 = 32 * khu + 16 * jj + 4 * g + ((lane & 15) >> 2);
            const char *p0 = tile + key0 * M_ROWB;
            const char *p1 = p0 + 8 * M_ROWB;
            const int dcol = 256 * kh + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const int boff = 2 * (dcol + 32 * mt);
                const s16x4 lo = lds_tr16(p0 + boff);
                const s16x4 hi = lds_tr16(p1 + boff);
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                O[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), bop,
                                                                O[mt], 0, 0, 0);
            }
        }

        if (tt + 1 < ntiles)
            stage_store<KV_FP8>(R, kt[buf ^ 1], tid);
        if (tid < M_TILE) {
            sidx[buf][tid] = idx_next;  // tile tt + 2
            idx_next = load_idx(tt + 3);
        }
        __syncthreads();
    }

    // ---- epilogue
    const int64_t orow = (int64_t)layer * T + i;
    const int head = 32 * hh + j;
    if (nsplit == 1) {
        const float inv = (l_run > 0.f) ? Ld.kv_scale / l_run : 0.f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 256 * kh + 32 * mt + 8 * q4 + 4 * g;
                const int64_t o = (i * M_H + head) * M_DC + d;
                if (OUT_F32) {
                    *(f32x4 *)((float *)Ld.out + o) =
                        f32x4{O[mt][4 * q4] * inv, O[mt][4 * q4 + 1] * inv, O[mt][4 * q4 + 2] * inv,
                              O[mt][4 * q4 + 3] * inv};
                } else {
                    *(u32x2 *)((uint16_t *)Ld.out + o) =
                        u32x2{pack_bf16x2(O[mt][4 * q4] * inv, O[mt][4 * q4 + 1] * inv),
                              pack_bf16x2(O[mt][4 * q4 + 2] * inv, O[mt][4 * q4 + 3] * inv)};
                }
            }
        }
        if (Ld.lse && kh == 0 && g == 0)
            Ld.lse[i * M_H + head] = (l_run > 0.f) ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
        return;
    }

    // several splits: write the partial, count, and let the last block combine
    float *po = ws_o + ((orow * nsplit + split) * M_H + head) * M_DC;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 256 * kh + 32 * mt + 8 * q4 + 4 * g;
            *(f32x4 *)(po + d) = f32x4{O[mt][4 * q4], O[mt][4 * q4 + 1], O[mt][4 * q4 + 2], O[mt][4 * q4 + 3]};
        }
    if (kh == 0 && g == 0) {
        float *pml = ws_ml + ((orow * nsplit + split) * M_H + head) * 2;
        pml[0] = m_run;
        pml[1] = l_run;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int old = atomicAdd(&ws_cnt[orow], 1);
        sh_last = (old == nsplit - 1);
    }
    __syncthreads();
    if (!sh_last)
        return;
    __threadfence();

    // combine weights per (split, head) into LDS (the tile buffers are free now)
    float *wts = (float *)kt[0];          // [nsplit][64]
    float *hstat = wts + nsplit * M_H;    // [64] lse
    if (tid < M_H) {
        const float *ml = ws_ml + (orow * nsplit * M_H + tid) * 2;
        float mx = -INFINITY;
        for (int sp = 0; sp < nsplit; ++sp)
            mx = fmaxf(mx, ml[sp * M_H * 2]);
        float tot = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) {
            const float ms = ml[sp * M_H * 2];
            const float e = (mx == -INFINITY) ? 0.f : exp2f(ms - mx);
            wts[sp * M_H + tid] = e;
            tot += e * ml[sp * M_H * 2 + 1];
        }
        const float inv = tot > 0.f ? Ld.kv_scale / tot : 0.f;
        for (int sp = 0; sp < nsplit; ++sp)
            wts[sp * M_H + tid] *= inv;
        hstat[tid] = tot > 0.f ? (mx + __log2f(tot)) * LN2 : -INFINITY;
    }
    __syncthreads();
    const float *pbase = ws_o + orow * nsplit * M_H * M_DC;
    for (int e4 = tid; e4 < M_H * M_DC / 4; e4 += 256) {
        const int hd = (e4 * 4) / M_DC;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < nsplit; ++sp) {
            const f32x4 v = *(const f32x4 *)(pbase + (int64_t)sp * M_H * M_DC + e4 * 4);
            const float wgt = wts[sp * M_H + hd];
            acc[0] = fmaf(wgt, v[0], acc[0]);
            acc[1] = fmaf(wgt, v[1], acc[1]);
            acc[2] = fmaf(wgt, v[2], acc[2]);
            acc[3] = fmaf(wgt, v[3], acc[3]);
        }
        const int64_t o = i * M_H * M_DC + (int64_t)e4 * 4;
        if (OUT_F32)
            *(f32x4 *)((float *)Ld.out + o) = acc;
        else
            *(u32x2 *)((uint16_t *)Ld.out + o) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
    if (Ld.lse && tid < M_H)
        Ld.lse[i * M_H + tid] = hstat[tid];
    if (tid == 0)
        ws_cnt[orow] = 0;  // leave the counter zeroed for the next call
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
            const int64_t row = (r.kv_base + idx) * Dqk;
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
                acc = fmaf(z[jj], load_elem<KVDT>(Ld.kv, (r.kv_base + idx) * Dqk + e), acc);
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
// Splits depend on the query rows T only (not on the layer count), so a layer run through
// the shared entry takes exactly the same reduction path as a single-layer call.
int mla_num_splits(int64_t T, int k)
{
    const int ntiles = (k + M_TILE - 1) / M_TILE;
    if (T <= 0)
        return 1;
    int64_t ns = (MLA_TARGET_BLOCKS + T - 1) / T;
    if (ns > ntiles)
        ns = ntiles;
    if (ns < 1)
        ns = 1;
    const int tps = (ntiles + (int)ns - 1) / (int)ns;  // equal tiles per split
    return (ntiles + tps - 1) / tps;
}

size_t mla_workspace_bytes(int64_t T, int n_layers, int k)
{
    const int ns = mla_num_splits(T, k);
    if (ns <= 1)
        return 0;
    const size_t rows = (size_t)T * n_layers;
    size_t cnt = (rows * sizeof(int) + 255) & ~(size_t)255;
    size_t o = rows * ns * M_H * M_DC * sizeof(float);
    size_t ml = rows * ns * M_H * 2 * sizeof(float);
    return cnt + o + ml;
}

hipError_t launch_mla_tuned(const LayoutDev &L, int64_t T, const MlaLayersDev &layers, int n_layers,
                            bool kv_fp8, bool out_f32, const int32_t *indices, int k,
                            float sm_scale, void *workspace, hipStream_t stream)
{
    const int64_t rows = T * n_layers;
    const int ns = mla_num_splits(T, k);
    const int ntiles = (k + M_TILE - 1) / M_TILE;
    const int tps = (ntiles + ns - 1) / ns;
    int *cnt = nullptr;
    float *wo = nullptr, *wml = nullptr;
    if (ns > 1) {
        size_t cntb = ((size_t)rows * sizeof(int) + 255) & ~(size_t)255;
        cnt = (int *)workspace;
        wo = (float *)((char *)workspace + cntb);
        wml = wo + (size_t)rows * ns * M_H * M_DC;
    }
    dim3 grid((unsigned)ns, (unsigned)T, (unsigned)n_layers);
#define DSA_MLA_LAUNCH(F8, OF)                                                                   \
    hipLaunchKernelGGL((mla_kernel<F8, OF>), grid, dim3(256), 0, stream, L, T, layers, indices, k, \
                       sm_scale, ns, tps, wo, wml, cnt)
    if (kv_fp8) {
        if (out_f32)
            DSA_MLA_LAUNCH(true, true);
        else
            DSA_MLA_LAUNCH(true, false);
    } else {
        if (out_f32)
            DSA_MLA_LAUNCH(false, true);
        else
            DSA_MLA_LAUNCH(false, false);
    }
#undef DSA_MLA_LAUNCH
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
