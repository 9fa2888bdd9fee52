// read_ceiling.hip -- a measurement aid for gfx950, no step of the method: the decode
// indexer's load stream over the index cache (its block shares, 32-token tiles, lanes and
// scale loads) with no arithmetic and no stores, to bound idx_decode_kernel.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

// 16 key bytes of a lane: rows need only be 4-byte aligned (132-byte entries work in place).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// ------------------------------------------------------------------------------------------
// The N tokens are cut into equal shares, one per block (multiples of 32 tokens); a
// wave takes 32-token tiles of its block's share, waves interleaved, two tiles in flight.
// pattern 0: the decode kernel's lanes for rows it cannot read as contiguous tiles (lane
// (g, j): token j, bytes 64 g .. +63, as four 16-byte loads) and its scale load; pattern 1:
// each load instruction reads 1 KB of consecutive bytes (rows of exactly 128 bytes), scales
// as in pattern 0; pattern 2: pattern 1 with nontemporal loads, the decode kernel's stream
// for contiguous tiles.  Every byte read is
// folded once into an xor; block b stores its xor in sink[b] (plain stores: one address
// shared by every block would serialise the grid's atomics), so the host can check that
// exactly the N rows and their scales were read.  One instantiation per pattern: a load and
// its nontemporal twin in one kernel could be merged into a plain load.
// ------------------------------------------------------------------------------------------
template <int pattern>
__global__ __launch_bounds__(256) void idx_read_ceiling_kernel(const uint8_t *__restrict__ k, int64_t kstride,
                                                               const float *__restrict__ ks, int64_t ks_stride,
                                                               int64_t N, uint32_t *sink)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, j = lane & 31;
    const int64_t per = ((N + gridDim.x - 1) / gridDim.x + 31) & ~(int64_t)31;
    const int64_t t0 = (int64_t)blockIdx.x * per, t1 = min(t0 + per, N);
    uint32_t acc = 0;
    auto load = [&](int64_t s0, u32x4 (&v)[4], uint32_t &sc) {
        if constexpr (pattern == 0) {
            const int64_t s = min(s0 + j, t1 - 1);
            const u32x4a4 *kp = (const u32x4a4 *)(k + s * kstride + 64 * g);
            v[0] = kp[0];
            v[1] = kp[1];
            v[2] = kp[2];
            v[3] = kp[3];
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = 1024 * u + 16 * lane;  // byte of the 4 KB tile
                const int64_t s = min(s0 + b / 128, t1 - 1);
                const u32x4 *p = (const u32x4 *)(k + s * 128 + (b & 127));
                if constexpr (pattern == 1)
                    v[u] = *p;
                else
                    v[u] = __builtin_nontemporal_load(p);
            }
        }
        sc = __float_as_uint(ks[min(s0 + j, t1 - 1) * ks_stride]);
    };
    auto fold = [&](int64_t s0, const u32x4 (&v)[4], uint32_t sc) {  // tokens past t1 (clamped) are left out
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t s = pattern == 0 ? s0 + j : s0 + (1024 * u + 16 * lane) / 128;
            if (s < t1)
                acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
        if (g == 0 && s0 + j < t1)
            acc ^= sc;
    };
    int64_t s0 = t0 + 32 * wave;
    if (s0 < t1) {
        u32x4 a[4], b[4];
        uint32_t sa, sb;
        load(s0, a, sa);
        for (; s0 < t1; s0 += 256) {
            load(s0 + 128, b, sb);
            fold(s0, a, sa);
            load(s0 + 256, a, sa);
            fold(s0 + 128, b, sb);
        }
    }
    __shared__ uint32_t wx[4];
    for (int o = 32; o > 0; o >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0)
        wx[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

hipError_t launch_read_ceiling(const uint8_t *k, int64_t kstride, const float *ks, int64_t ks_stride, int64_t N,
                               int pattern, int blocks, uint32_t *sink, hipStream_t stream)
{
    if (pattern == 0)
        hipLaunchKernelGGL(idx_read_ceiling_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, k, kstride, ks,
                           ks_stride, N, sink);
    else if (pattern == 1)
        hipLaunchKernelGGL(idx_read_ceiling_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, k, kstride, ks,
                           ks_stride, N, sink);
    else
        hipLaunchKernelGGL(idx_read_ceiling_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, k, kstride, ks,
                           ks_stride, N, sink);
    return hipGetLastError();
}

}  // namespace dsa
