// dsa_common.h -- device-side helpers shared by the libdsa kernels (gfx950 only).
//
// Vector types for the CDNA4 matrix cores, exact fp8 -> bf16 / fp32 widening,
// bf16 rounding and the ragged-layout row lookup used by every stage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Kernel-side copy of dsa_layout (host sizes other than the paging ones are launch params).
struct LayoutDev {
    const int64_t *kv_indptr;
    const int32_t *q_indptr;  // nullptr: one query per sequence
    int32_t batch;
    const int32_t *block_table;  // nullptr: contiguous caches
    int32_t bt_stride;
    int32_t page_size;
    int64_t cache_rows;
};

// Cache row of token s of sequence b: kv_base + s for contiguous caches, the page table's
// physical row for paged ones.  With kv_base = 0 on contiguous caches it is the position
// itself: the form top-k writes (positions, or physical rows when paged).
// Positions are below 2^31 (the host checks max_ctx), so the page split runs in 32 bits: a
// shift and a mask for power-of-two pages, else one unsigned division.
__device__ __forceinline__ int64_t token_row(const LayoutDev &L, int b, int64_t kv_base, int64_t s)
{
    if (L.block_table == nullptr)
        return kv_base + s;
    const uint32_t ps = (uint32_t)L.page_size, si = (uint32_t)s;
    uint32_t pg, off;
    if ((ps & (ps - 1u)) == 0u) {
        pg = si >> __builtin_ctz(ps);
        off = si & (ps - 1u);
    } else {
        pg = si / ps;
        off = si - pg * ps;
    }
    return (int64_t)L.block_table[(int64_t)b * L.bt_stride + pg] * ps + off;
}

struct RowInfo {
    int32_t b;
    int64_t kv_base;  // first cache row of the sequence
    int64_t n;        // visible tokens of this query row (causal, inclusive)
};

// Query row i -> (sequence, first cache row, visible count).  Query j of a
// q_len-long chunk at the end of a ctx-long sequence sees ctx - q_len + j + 1
// tokens; with no q_indptr every sequence has one query that sees all of it.
__device__ __forceinline__ RowInfo row_info(const LayoutDev &L, int64_t i)
{
    RowInfo r;
    if (L.q_indptr == nullptr) {
        r.b = (int32_t)i;
        r.kv_base = L.kv_indptr[i];
        r.n = L.kv_indptr[i + 1] - r.kv_base;
        return r;
    }
    int lo = 0, hi = L.batch - 1;  // largest b with q_indptr[b] <= i
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)L.q_indptr[mid] <= i)
            lo = mid;
        else
            hi = mid - 1;
    }
    r.b = lo;
    r.kv_base = L.kv_indptr[lo];
    int64_t ctx = L.kv_indptr[lo + 1] - r.kv_base;
    int64_t qlen = (int64_t)L.q_indptr[lo + 1] - L.q_indptr[lo];
    r.n = ctx - qlen + (i - L.q_indptr[lo]) + 1;
    return r;
}

// ---- conversions -------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Two E4M3FN codes (bytes 0,1 or 2,3 of `word`) -> two bf16; exact, since every
// E4M3FN value is a bf16 value.  gfx950's converter reads OCP E4M3FN.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word)
{
    bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// 8 E4M3FN codes (two dwords) -> 8 bf16 operand lanes for a bf16 MFMA.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    u32x4 r;
    r[0] = fp8x2_to_bf16x2<false>(w0);
    r[1] = fp8x2_to_bf16x2<true>(w0);
    r[2] = fp8x2_to_bf16x2<false>(w1);
    r[3] = fp8x2_to_bf16x2<true>(w1);
    return __builtin_bit_cast(bf16x8, r);
}

// One E4M3FN code -> fp32, exact.
__device__ __forceinline__ float fp8_to_f32(uint32_t code)
{
    f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false);
    return v[0];
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Element loaders used by the generic kernels.
template <int DT> __device__ __forceinline__ float load_elem(const void *base, int64_t idx);
template <> __device__ __forceinline__ float load_elem<0>(const void *base, int64_t idx)
{
    return ((const float *)base)[idx];
}
template <> __device__ __forceinline__ float load_elem<1>(const void *base, int64_t idx)
{
    return bf16_bits_to_f32(((const uint16_t *)base)[idx]);
}
template <> __device__ __forceinline__ float load_elem<2>(const void *base, int64_t idx)
{
    return fp8_to_f32(((const uint8_t *)base)[idx]);
}

// Monotone 32-bit key of a score (sign-flipped IEEE bits, -0 folded into +0): a > b as floats
// iff key(a) > key(b), and -0 == +0 share a key.  The top 11 bits are the top-k's histogram bin.
__device__ __forceinline__ uint32_t score_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int SCORE_BINS = 2048;  // 11-bit key digits
constexpr int SCORE_BIN_SHIFT = 21;

// ---- wave / block reductions (wave64) -----------------------------------------------------

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}


// Barrier that waits only for this wave's LDS traffic (global loads and LDS DMA stay in
// flight).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Barrier that also waits for this wave's global loads and LDS DMA.  The wait is issued
// through the builtin as well so that the compiler's own wait-count tracking sees every
// load as complete (it does not read inline asm) and adds no waits for them later.
__device__ __forceinline__ void tile_barrier()
{
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer descriptor (stride 0, range = bytes) over base; every field uniform.
__device__ __forceinline__ i32x4 buffer_desc(const void *base, int64_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    d[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)bytes);  // unsigned range, up to 4 GiB - 1
    d[3] = 0x00020000;  // buffer descriptor word 3 for the gfx9 family
    return d;
}

// One wave-wide 16-byte-per-lane load from a buffer straight into LDS: lane l writes LDS
// bytes lds_addr + 16 l .. +15 with the bytes at voff of the buffer (zeros when voff is past
// its range).  Issued as inline asm, so the compiler neither tracks it nor orders LDS reads
// of other buffers after it: tile_barrier() waits for it.  M0 holds the LDS destination
// (one wait state after writing it); nothing else in these kernels uses M0, so clobbering
// the reserved register is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const i32x4 &desc, uint32_t lds_addr, int voff)
{
    // the LDS address is wave-uniform; readfirstlane keeps it in an SGPR whatever the compiler's
    // uniformity analysis concluded
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(desc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object (for M0).
__device__ __forceinline__ uint32_t lds_addr_of(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

}  // namespace dsa
