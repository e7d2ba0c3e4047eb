// Low-bit records of streamed experts, expanded on the GPU.
//
// The experts.rs page streams experts that are not kept resident ("transient
// misses") in the layout of its low-bit store (fn prepare_expert_jobs:
// miss_layout; fn read_expert_batch keeps 4-bit and low-bit reads apart).
// Here a miss record crosses the host link with 2-bit codes (about 56% of
// the 4-bit record's bytes at the large chunk's shape) and, once in device
// memory, k_expand2 rewrites it exactly as the 4-bit record that the grouped
// GEMMs read: the codes 0..3 are a subset of 0..15 and the scale/bias
// sections are the same, so the weights, and every result, are unchanged.
//
// Code tiles: a 2-bit tile (512 bytes) gives each lane two 32-bit words,
// word j at byte 256 j + 4 L, code c in word c/16 at bit 2((c%16)/2) +
// 16(c%2); the 4-bit tile (1024 bytes) gives lane L 16 bytes at 16 L, code c
// in word c/8 at bit 4((c%8)/2) + 16(c%2).  Output word m holds codes 8m ..
// 8m+7, which sit in input word m/2 shifted right by 8 (m%2): there code 2u
// is at bit 2u and code 2u+1 at bit 16 + 2u, and they move to bits 4u and
// 16 + 4u.  One thread converts one (tile, lane): two coalesced 4-byte loads,
// one coalesced 16-byte store.  Scale/bias sections are copied 16 bytes a
// thread.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t spread2to4(uint32_t w) {
    uint32_t o = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) o |= ((w >> (2 * u)) & 0x00030003u) << (4 * u);
    return o;
}

__global__ void __launch_bounds__(256) k_expand2(ExpandArgs a) {
    const ExpandJob job = a.job[blockIdx.y];
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    uint64_t base = 0;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const uint64_t n = (uint64_t)a.tiles[m] * 64;
        if (i >= base && i < base + n) {
            const uint64_t q = i - base, tile = q >> 6, lane = q & 63;
            const uint8_t *src = job.src + a.src_w[m] + tile * 512 + lane * 4;
            const uint32_t w0 = *reinterpret_cast<const uint32_t *>(src);
            const uint32_t w1 = *reinterpret_cast<const uint32_t *>(src + 256);
            uint4 o;
            o.x = spread2to4(w0);
            o.y = spread2to4(w0 >> 8);
            o.z = spread2to4(w1);
            o.w = spread2to4(w1 >> 8);
            *reinterpret_cast<uint4 *>(job.dst + a.dst_w[m] + tile * 1024 + lane * 16) = o;
            return;
        }
        base += n;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const uint64_t n = a.sb_bytes[m] / 16;
        if (i >= base && i < base + n) {
            const uint64_t q = i - base;
            *reinterpret_cast<uint4 *>(job.dst + a.dst_sb[m] + q * 16) =
                *reinterpret_cast<const uint4 *>(job.src + a.src_sb[m] + q * 16);
            return;
        }
        base += n;
    }
}

}  // namespace

hipError_t launch_expand2(const ExpandArgs &a, hipStream_t s) {
    uint64_t items = 0;
    for (int m = 0; m < 3; ++m) items += (uint64_t)a.tiles[m] * 64 + a.sb_bytes[m] / 16;
    const dim3 grid((unsigned)((items + 255) / 256), (unsigned)a.n);
    hipLaunchKernelGGL(k_expand2, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// Offsets and sizes of the expansion from the miss layout L2 (2-bit) to the
// routed layout L4 (4-bit) of the same shape.
ExpandArgs expand_args(const moe_layout *L4, const moe_layout *L2) {
    ExpandArgs a;
    a.n = 0;
    const uint64_t w4[3] = {L4->gate_w, L4->up_w, L4->down_w}, sb4[3] = {L4->gate_sb, L4->up_sb, L4->down_sb};
    const uint64_t w2[3] = {L2->gate_w, L2->up_w, L2->down_w}, sb2[3] = {L2->gate_sb, L2->up_sb, L2->down_sb};
    const uint64_t tiles = (uint64_t)(L4->hidden / 32) * (L4->inter / 64);  // every matrix: h*I/2048 tiles
    for (int m = 0; m < 3; ++m) {
        a.dst_w[m] = w4[m];
        a.dst_sb[m] = sb4[m];
        a.src_w[m] = w2[m];
        a.src_sb[m] = sb2[m];
        a.tiles[m] = (uint32_t)tiles;
        a.sb_bytes[m] = (uint32_t)((uint64_t)L4->hidden * L4->inter / L4->group * 4);
    }
    return a;
}

}  // namespace moe
