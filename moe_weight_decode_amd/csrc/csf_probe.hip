// Measurement kernels for the CSF decoder on gfx950: the ceilings and floors
// its timings are read against.  Nothing here decodes; these kernels move
// bytes in the decoder's patterns so that its speed can be stated as a
// fraction of what the chip does with the same streams (the pages time the
// decode warm and with flushed caches, "finegrained-kernels: decode
// losslessly compressed NVFP4 scales (CSF)", kernels-community PR 1236,
// measurements paragraph).
//
//   csf_probe_mix_kernel    up to three read streams and one write stream,
//                           split into the same number of tiles; workgroup
//                           tiles grid-stride, every lane loads 16 bytes per
//                           instruction and stores 16-byte runs (a wave
//                           store covers 1 KiB), the decoder's access shape
//                           without its LDS work.
//   csf_probe_chain_kernel  per workgroup, a chain of dependent 4-byte loads
//                           (each address read from the previous load) and
//                           then one 16-byte store per lane: a launch with k
//                           dependent round trips to memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <chrono>

#include "csf.h"
#include "csf_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kBlock = 256;
constexpr uint32_t kRuns = 4;          // 16-byte output runs per lane per tile
constexpr uint32_t kTile = kBlock * 16 * kRuns;  // 16 KiB of output per tile
constexpr uint32_t kLoads = 4;         // 16-byte loads per lane per read stream and tile (at most)
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

struct MixArgs {
    const uint8_t *src[3];
    uint64_t src_bytes[3];
    uint8_t *dst;
    uint64_t dst_bytes;
    uint32_t tiles;
    uint32_t nsrc;
    uint32_t flags;
    uint32_t pad_;
};

// Tile u's byte range of a stream of n bytes cut into `tiles` pieces on
// 16-byte boundaries.
__device__ __forceinline__ void piece(uint64_t n, uint32_t u, uint32_t tiles, uint64_t &lo, uint64_t &hi) {
    lo = ((n * u) / tiles) & ~15ull;
    hi = u + 1 == tiles ? n : (((n * (u + 1)) / tiles) & ~15ull);
}

__global__ __launch_bounds__(kBlock) void csf_probe_mix_kernel(MixArgs a) {
    const bool nt_store = (a.flags & CSF_PROBE_NT_STORES) != 0;
    for (uint32_t u = blockIdx.x; u < a.tiles; u += gridDim.x) {
        u32x4 acc = {0u, 0u, 0u, 0u};
        u32x4 v[3][kLoads];
#pragma unroll
        for (uint32_t s = 0; s < 3; ++s) {
            uint64_t lo = 0, hi = 0;
            if (s < a.nsrc) piece(a.src_bytes[s], u, a.tiles, lo, hi);
            const rsrc_t r = make_rsrc(a.src[s] + lo, (uint32_t)(hi - lo));
            const bool nt = (a.flags & (CSF_PROBE_NT_LOADS0 << s)) != 0;
#pragma unroll
            for (uint32_t i = 0; i < kLoads; ++i) {
                const int off = (int)(16u * (i * kBlock + threadIdx.x));
                v[s][i] = __builtin_bit_cast(
                    u32x4, nt ? __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal)
                              : __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
            }
        }
#pragma unroll
        for (uint32_t s = 0; s < 3; ++s)
#pragma unroll
            for (uint32_t i = 0; i < kLoads; ++i) acc ^= v[s][i];
        uint64_t lo = 0, hi = 0;
        piece(a.dst_bytes, u, a.tiles, lo, hi);
        const rsrc_t w = make_rsrc(a.dst + lo, (uint32_t)(hi - lo));
#pragma unroll
        for (uint32_t i = 0; i < kRuns; ++i) {
            const uint32_t j = i * kBlock + threadIdx.x;
            const i32x4 out = __builtin_bit_cast(i32x4, acc ^ (u32x4){j, u, i, 0u});
            if (nt_store)
                __builtin_amdgcn_raw_buffer_store_b128(out, w, (int)(16u * j), 0, kNonTemporal);
            else
                __builtin_amdgcn_raw_buffer_store_b128(out, w, (int)(16u * j), 0, 0);
        }
    }
}

// hops dependent loads from a chain of indices (buf[i] < words for every i),
// starting at a position set by the workgroup and the seed; then, when out is
// not null, one 16-byte store per lane at out + 16 * global thread index.
__global__ __launch_bounds__(1024) void csf_probe_chain_kernel(const uint32_t *buf, uint64_t words, uint32_t seed,
                                                               uint32_t hops, uint8_t *out) {
    uint32_t i = (uint32_t)((((uint64_t)blockIdx.x * 2654435761u) ^ ((uint64_t)seed * 40503u)) % words);
    const rsrc_t r = make_rsrc(buf, (uint32_t)(4u * words));
    // buffer loads: vector memory instructions, as the decoder's loads are
    for (uint32_t h = 0; h < hops; ++h)
        i = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(r, (int)(4u * i), 0, 0));
    if (out != nullptr) {
        const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
        *reinterpret_cast<u32x4 *>(out + 16 * t) = (u32x4){i, (uint32_t)t, hops, seed};
    }
}

}  // namespace

extern "C" {

csf_status csf_probe_mix(const uint8_t *const *src, const uint64_t *src_bytes, uint32_t nsrc, uint8_t *dst,
                         uint64_t dst_bytes, uint32_t grid, uint32_t flags, void *hip_stream) {
    if (nsrc > 3 || dst == nullptr || dst_bytes == 0 || grid == 0 || dst_bytes >= (1ull << 40)) return CSF_E_SIZE;
    if (nsrc > 0 && (src == nullptr || src_bytes == nullptr)) return CSF_E_NULL;
    MixArgs a = {};
    a.dst = dst;
    a.dst_bytes = dst_bytes;
    a.tiles = (uint32_t)((dst_bytes + kTile - 1) / kTile);
    a.nsrc = nsrc;
    a.flags = flags;
    if ((dst_bytes + kTile - 1) / kTile >= (1ull << 31)) return CSF_E_SIZE;
    for (uint32_t s = 0; s < nsrc; ++s) {
        if (src[s] == nullptr) return CSF_E_NULL;
        if (src_bytes[s] >= (1ull << 40)) return CSF_E_SIZE;
        // every tile's piece of a stream must fit the loads a lane issues
        if ((src_bytes[s] + a.tiles - 1) / a.tiles + 16 > uint64_t(kLoads) * kBlock * 16) return CSF_E_SIZE;
        a.src[s] = src[s];
        a.src_bytes[s] = src_bytes[s];
    }
    for (uint32_t s = nsrc; s < 3; ++s) a.src[s] = dst;  // never read: zero-length pieces
    (void)hipGetLastError();
    hipLaunchKernelGGL(csf_probe_mix_kernel, dim3(grid), dim3(kBlock), 0, static_cast<hipStream_t>(hip_stream), a);
    return hipGetLastError() == hipSuccess ? CSF_OK : CSF_E_HIP;
}

csf_status csf_probe_chain(const uint32_t *buf, uint64_t words, uint32_t seed, uint32_t hops, uint8_t *out,
                           uint32_t grid, uint32_t block, void *hip_stream) {
    if (grid == 0 || block == 0 || block > 1024 || block % 64 != 0 || words >= (1ull << 30)) return CSF_E_SIZE;
    if (hops > 0 && (buf == nullptr || words == 0)) return CSF_E_NULL;
    if (words == 0) words = 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(csf_probe_chain_kernel, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(hip_stream),
                       buf, words, seed, hops, out);
    return hipGetLastError() == hipSuccess ? CSF_OK : CSF_E_HIP;
}

double csf_probe_host_ns(const csf_stack *first, uint8_t *ws_first, const csf_stack *second, uint8_t *ws_second,
                         const int32_t *expert_start, uint32_t calls, void *hip_stream) {
    if (calls == 0) return -1.0;
    const auto t0 = std::chrono::steady_clock::now();
    for (uint32_t i = 0; i < calls; ++i) {
        const csf_status st = second ? csf_decode_paired(first, ws_first, second, ws_second, expert_start, hip_stream)
                                     : csf_decode(first, ws_first, expert_start, hip_stream);
        if (st != CSF_OK) return -1.0 - double(st);
    }
    const auto t1 = std::chrono::steady_clock::now();
    return std::chrono::duration<double, std::nano>(t1 - t0).count() / calls;
}

}  // extern "C"
