// index_quant.hip -- index-cache writer: rope, ue8m0 scale and E4M3FN codes (gfx950).
//
// The step in front of the lightning indexer ("GLM-5.2 架构解剖", full structure
// diagram, Indexer box: the index key takes interleaved rope, is quantised to
// fp8 in 1x128 groups with a power-of-two (ue8m0) scale and is written into a
// 132-byte index-cache entry; section ATOM 侧, fused indexer kernel: query rope,
// fp8 quantisation and the key-cache write as one pass for 128-wide index heads
// with 64 rope dims).  One group is one head's 128 values:
//
//   y     = the group, with rope applied to dims [rope_off, rope_off + 64) in
//           interleaved pairs (2i, 2i+1) using table row cos_sin[pos] =
//           (cos_0 .. cos_31, sin_0 .. sin_31):  (y0, y1) = (x0 c - x1 s, x0 s + x1 c)
//   s     = smallest 2^e, e >= -126, with max|y| <= 448 * 2^e   (1 if y == 0)
//   code  = y / s rounded to the nearest E4M3FN value, ties to even
//
// The work is a stream: 256 B read (bf16) and 132 B written per group, so the
// kernel is bound by HBM.  Sixteen lanes own a group, 8 consecutive values per
// lane (one 16-byte load); a team of 16 lanes takes one group, or four
// consecutive groups with all their loads in flight together when the launch is
// large enough to fill the chip with 64-group blocks.  The rope
// products and sums are rounded one by one (no contraction) because their fp32
// results decide the 8-bit codes.  The scale comes from the bits of the group's
// largest magnitude, so it is exact and independent of denormal handling; y / s
// is a product with the exact power of two 1 / s; gfx950's converter rounds
// to OCP E4M3FN, nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int IQ_D = 128;          // values per group (one index head)
constexpr int IQ_DR = 64;          // rope dims per group
constexpr int IQ_LANES = 16;       // lanes per group
constexpr int IQ_BLOCK = 256;      // threads per block
constexpr int IQ_GROUPS = IQ_BLOCK / IQ_LANES;

static __device__ __forceinline__ void rope_pair(float &x0, float &x1, float c, float s)
{
#pragma clang fp contract(off)
    float a = x0 * c;
    float b = x1 * s;
    float d = x0 * s;
    float e = x1 * c;
    x0 = a - b;
    x1 = d + e;
}

// Maximum over each 16-lane DPP row (one team): swap neighbours, swap pairs (quad
// permutes), then mirror within 8 lanes and within the 16-lane row.
__device__ __forceinline__ uint32_t team_max(uint32_t x)
{
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
    x = t > x ? t : x;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
    x = t > x ? t : x;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false); // row_half_mirror
    x = t > x ? t : x;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false); // row_mirror
    x = t > x ? t : x;
    return x;
}

// This lane's 8 values of one group as raw words: 4 (bf16 pairs) or 8 (fp32).
template <bool IN_F32>
struct Raw {
    uint32_t w[IN_F32 ? 8 : 4];
};

template <bool IN_F32>
__device__ __forceinline__ Raw<IN_F32> load_raw(const uint8_t *src, int lane)
{
    Raw<IN_F32> a;
    if (IN_F32) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(src) + 2 * lane;
        u32x4 x0 = p[0], x1 = p[1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a.w[t] = x0[t];
            a.w[4 + t] = x1[t];
        }
    } else {
        u32x4 x0 = reinterpret_cast<const u32x4 *>(src)[lane];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            a.w[t] = x0[t];
    }
    return a;
}

template <bool IN_F32>
__device__ __forceinline__ void widen(const Raw<IN_F32> &a, float v[8])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (IN_F32) {
            v[2 * t] = __uint_as_float(a.w[2 * t]);
            v[2 * t + 1] = __uint_as_float(a.w[2 * t + 1]);
        } else {
            v[2 * t] = __uint_as_float(a.w[t] << 16);
            v[2 * t + 1] = __uint_as_float(a.w[t] & 0xffff0000u);
        }
    }
}

// One quantisation job: `groups` groups of 128 values, H per row of x; group (r, h) goes to
// row dst_rows[r] (r when NULL) of codes / scales, skipped when that row is outside
// [0, out_rows).
struct IqArgs {
    int64_t groups;
    int H;
    const uint8_t *x;
    int64_t x_row_bytes;
    const int64_t *positions;
    const float *cos_sin;
    int64_t rope_rows;
    int rope_off;
    const int64_t *dst_rows;
    int64_t out_rows;
    uint8_t *codes;
    int64_t code_row_bytes;
    float *scales;
    int64_t scale_row_stride;
};

// Each 16-lane team owns NG consecutive groups of ONE row (the launcher only picks NG > 1
// when H is a multiple of NG), so the row's destination, position and rope-table values
// are loaded once, and the team issues all NG loads of its groups before any arithmetic:
// a lane keeps NG 16-byte loads in flight.  Values are read for every existing group;
// only the writes depend on the destination row.  All lanes stay live to the end (no early
// return), so the cross-lane maximum always sees its partners; a team's lanes agree on
// every group's validity.
template <bool IN_F32, int NG, bool ROPE>
__device__ __forceinline__ void quant_block(const IqArgs &a, int64_t block)
{
    const int64_t groups = a.groups;
    const int H = a.H;
    const uint8_t *__restrict__ x = a.x;
    const int64_t x_row_bytes = a.x_row_bytes;
    const int64_t *__restrict__ positions = a.positions;
    const float *__restrict__ cos_sin = a.cos_sin;
    const int64_t rope_rows = a.rope_rows;
    const int rope_off = a.rope_off;
    const int64_t *__restrict__ dst_rows = a.dst_rows;
    const int64_t out_rows = a.out_rows;
    uint8_t *__restrict__ codes = a.codes;
    const int64_t code_row_bytes = a.code_row_bytes;
    float *__restrict__ scales = a.scales;
    const int64_t scale_row_stride = a.scale_row_stride;

    const int lane = threadIdx.x & (IQ_LANES - 1);
    const int64_t g0 = (block * IQ_GROUPS + (threadIdx.x >> 4)) * NG;
    // groups fit in 32 bits for every realistic call; the 64-bit division is the fallback
    const int64_t r = groups <= (int64_t)UINT32_MAX ? (int64_t)((uint32_t)g0 / (uint32_t)H) : g0 / H;
    const int h0 = (int)(g0 - r * H);
    const bool live = g0 < groups;  // a live team's NG groups all exist (H % NG == 0)

    // Loads in the order their results are needed: the rope position first (its table
    // row is a second, dependent load), then every group's values, then the table row;
    // the values stay in flight meanwhile.  The loads are unconditional (a team past the
    // end re-reads the first groups, and drops them) so the waits before the dependent
    // loads can count outstanding loads instead of draining them.
    const int64_t rr = live ? r : 0;  // row whose position and values are read
    const int hb = live ? h0 : 0;
    const int rl = 8 * lane - rope_off;  // first rope dim of this lane, relative
    const bool rope_lane = ROPE && rl >= 0 && rl < IQ_DR;
    int64_t pos = 0;
    if (ROPE)
        pos = positions[rr];

    Raw<IN_F32> raw[NG];
    const uint8_t *src = x + rr * x_row_bytes + (int64_t)hb * IQ_D * (IN_F32 ? 4 : 2);
#pragma unroll
    for (int j = 0; j < NG; ++j)
        raw[j] = load_raw<IN_F32>(src + j * IQ_D * (IN_F32 ? 4 : 2), lane);

    // Interleaved rope: this lane's dims 8*lane .. 8*lane+7 hold pairs
    // (8*lane - rope_off)/2 .. +3 when they fall in the rope range (other lanes read the
    // row's first entries and ignore them).
    f32x4 rc = {1.f, 1.f, 1.f, 1.f}, rs = {0.f, 0.f, 0.f, 0.f};
    if (ROPE) {
        pos = pos < 0 ? 0 : pos >= rope_rows ? rope_rows - 1 : pos;
        const float *row = cos_sin + pos * IQ_DR + (rope_lane ? rl / 2 : 0);
        rc = *reinterpret_cast<const f32x4 *>(row);
        rs = *reinterpret_cast<const f32x4 *>(row + IQ_DR / 2);
    }
    const int64_t dst = live ? (dst_rows ? dst_rows[r] : r) : -1;
    const bool row_ok = dst >= 0 && dst < out_rows;

#pragma unroll
    for (int j = 0; j < NG; ++j) {
        float v[8];
        widen<IN_F32>(raw[j], v);
        if (rope_lane) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                rope_pair(v[2 * t], v[2 * t + 1], rc[t], rs[t]);
        }
        // Largest magnitude as an integer max over the sign-cleared bits (monotone for
        // non-negative floats, subnormals included), then over the team's 16 lanes.
        uint32_t amax = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            uint32_t m = __float_as_uint(v[t]) & 0x7fffffffu;
            amax = m > amax ? m : amax;
        }
        amax = team_max(amax);
        if (!row_ok)
            continue;

        // amax = 1.M * 2^E: 448 * 2^e >= amax  <=>  e >= E - 8 when 1.M <= 1.75, else E - 7.
        int e;
        if (amax == 0) {
            e = 0;
        } else {
            int E = (int)(amax >> 23) - 127;
            e = E - 8 + ((amax & 0x7fffffu) > 0x600000u ? 1 : 0);
            e = e < -126 ? -126 : e;  // also covers subnormal amax (E = -127)
        }
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
        uint32_t w0 = 0, w1 = 0;
        w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, (int)w0, false);
        w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, (int)w0, true);
        w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, (int)w1, false);
        w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, (int)w1, true);

        const int h = h0 + j;
        uint32_t *out = reinterpret_cast<uint32_t *>(codes + dst * code_row_bytes +
                                                     (int64_t)h * IQ_D) + 2 * lane;
        out[0] = w0;
        out[1] = w1;
        if (lane == 0)
            scales[dst * scale_row_stride + h] = __uint_as_float((uint32_t)(127 + e) << 23);
    }
}

template <bool IN_F32, int NG, bool ROPE>
__global__ void __launch_bounds__(IQ_BLOCK) index_quant_kernel(IqArgs a)
{
    quant_block<IN_F32, NG, ROPE>(a, blockIdx.x);
}

// The fused front end: the first qblocks blocks quantise the index queries (NGQ groups per
// team), the rest write the keys (one group per team), in one launch.
template <bool IN_F32, int NGQ, bool ROPE>
__global__ void __launch_bounds__(IQ_BLOCK) index_front_kernel(IqArgs q, IqArgs k, int64_t qblocks)
{
    if ((int64_t)blockIdx.x < qblocks)
        quant_block<IN_F32, NGQ, ROPE>(q, blockIdx.x);
    else
        quant_block<IN_F32, 1, ROPE>(k, (int64_t)blockIdx.x - qblocks);
}

// Groups per team: four when the heads of a row split into fours and there are enough
// groups for 256 blocks of 64, else one.
constexpr int IQ_NG_WIDE = 4;

static bool iq_wide(int64_t groups, int H)
{
    return H % IQ_NG_WIDE == 0 && groups >= (int64_t)256 * IQ_GROUPS * IQ_NG_WIDE;
}

static int64_t iq_blocks(int64_t groups, bool wide)
{
    const int64_t per_block = (int64_t)IQ_GROUPS * (wide ? IQ_NG_WIDE : 1);
    return (groups + per_block - 1) / per_block;
}

hipError_t launch_index_quant(int64_t rows, int H, bool in_f32, const void *x, int64_t x_row_bytes,
                              const int64_t *positions, const float *cos_sin, int64_t rope_rows,
                              int rope_off, const int64_t *dst_rows, int64_t out_rows,
                              uint8_t *codes, int64_t code_row_bytes, float *scales,
                              int64_t scale_row_stride, hipStream_t stream)
{
    const IqArgs a{rows * H, H, (const uint8_t *)x, x_row_bytes, positions, cos_sin, rope_rows,
                   rope_off, dst_rows, out_rows, codes, code_row_bytes, scales, scale_row_stride};
    if (a.groups == 0)
        return hipSuccess;
    const bool wide = iq_wide(a.groups, H), rope = cos_sin != nullptr;
    const dim3 grid((unsigned)iq_blocks(a.groups, wide));
#define IQ_LAUNCH(F32, NG, ROPE) index_quant_kernel<F32, NG, ROPE><<<grid, IQ_BLOCK, 0, stream>>>(a)
#define IQ_LAUNCH_NG(F32, ROPE)                                                                   \
    do {                                                                                          \
        if (wide)                                                                                 \
            IQ_LAUNCH(F32, IQ_NG_WIDE, ROPE);                                                     \
        else                                                                                      \
            IQ_LAUNCH(F32, 1, ROPE);                                                              \
    } while (0)
    if (in_f32) {
        if (rope)
            IQ_LAUNCH_NG(true, true);
        else
            IQ_LAUNCH_NG(true, false);
    } else {
        if (rope)
            IQ_LAUNCH_NG(false, true);
        else
            IQ_LAUNCH_NG(false, false);
    }
#undef IQ_LAUNCH_NG
#undef IQ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_index_front(int64_t T, int H, bool in_f32, const void *q, int64_t q_row_bytes,
                              const void *k, int64_t k_row_bytes, const int64_t *positions,
                              const float *cos_sin, int64_t rope_rows, int rope_off,
                              const int64_t *slots, int64_t cache_rows, uint8_t *cache,
                              int64_t cache_row_bytes, float *cache_scale, int64_t cache_scale_stride,
                              uint8_t *q_fp8, float *q_scale, hipStream_t stream)
{
    const IqArgs qa{T * H, H, (const uint8_t *)q, q_row_bytes, positions, cos_sin, rope_rows,
                    rope_off, nullptr, T, q_fp8, (int64_t)H * IQ_D, q_scale, H};
    const IqArgs ka{T, 1, (const uint8_t *)k, k_row_bytes, positions, cos_sin, rope_rows, rope_off,
                    slots, cache_rows, cache, cache_row_bytes, cache_scale, cache_scale_stride};
    if (T == 0)
        return hipSuccess;
    const bool wide = iq_wide(qa.groups, H), rope = cos_sin != nullptr;
    const int64_t qblocks = iq_blocks(qa.groups, wide);
    const dim3 grid((unsigned)(qblocks + iq_blocks(ka.groups, false)));
#define IQ_LAUNCH(F32, NG, ROPE) index_front_kernel<F32, NG, ROPE><<<grid, IQ_BLOCK, 0, stream>>>(qa, ka, qblocks)
#define IQ_LAUNCH_NG(F32, ROPE)                                                                   \
    do {                                                                                          \
        if (wide)                                                                                 \
            IQ_LAUNCH(F32, IQ_NG_WIDE, ROPE);                                                     \
        else                                                                                      \
            IQ_LAUNCH(F32, 1, ROPE);                                                              \
    } while (0)
    if (in_f32) {
        if (rope)
            IQ_LAUNCH_NG(true, true);
        else
            IQ_LAUNCH_NG(true, false);
    } else {
        if (rope)
            IQ_LAUNCH_NG(false, true);
        else
            IQ_LAUNCH_NG(false, false);
    }
#undef IQ_LAUNCH_NG
#undef IQ_LAUNCH
    return hipGetLastError();
}

}  // namespace dsa
