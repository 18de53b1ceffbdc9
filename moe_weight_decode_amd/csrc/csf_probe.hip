// Measurement kernels for the CSF decoder on gfx950: the ceilings and floors
// its timings are read against.  Nothing here decodes; these kernels move
// bytes in the decoder's patterns so that its speed can be stated as a
// fraction of what the chip does with the same streams (the pages time the
// decode warm and with flushed caches, "finegrained-kernels: decode
// losslessly compressed NVFP4 scales (CSF)", kernels-community PR 1236,
// measurements paragraph).
//
//   csf_probe_mix_kernel    up to three read streams and one write stream,
//                           split into the same number of tiles; workgroups
//                           take tiles grid-stride, every lane loads 16 bytes
//                           per instruction and stores 16-byte runs (a wave
//                           store covers 1 KiB), the next tile's loads issued
//                           before this tile's stores: the decoder's access
//                           shape and schedule without its LDS work.
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
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

struct MixArgs {
    const uint8_t *src[3];
    uint64_t src_bytes[3];
    double per_tile[3];     // src_bytes[s] / tiles
    uint8_t *dst;
    uint64_t dst_bytes;
    uint32_t tiles;
    uint32_t nsrc;
    uint32_t flags;
    uint32_t pad_;
};

// Piece u of a stream of n bytes cut into `tiles` pieces on 16-byte
// boundaries (boundary u at floor(u * n / tiles) rounded down to 16; f = n /
// tiles; the same expression gives both ends of neighbouring pieces).
__device__ __forceinline__ uint64_t boundary(double f, uint32_t u) {
    return (uint64_t)((double)u * f) & ~15ull;
}

__device__ __forceinline__ void piece(uint64_t n, double f, uint32_t u, uint32_t tiles, uint64_t &lo, uint64_t &hi) {
    lo = boundary(f, u);
    hi = u + 1 == tiles ? n : boundary(f, u + 1);
}

// One tile's loads: stream s's piece in L[s] 16-byte loads per lane (lane t
// loads chunks t, t + 256, ...), through a buffer resource that covers the
// piece exactly, so loads past it read 0 without touching memory.  Every
// load is issued unconditionally; POLICY is the cache policy.
template <uint32_t L0, uint32_t L1, uint32_t L2>
struct TileIn {
    u32x4 v0[L0 ? L0 : 1], v1[L1 ? L1 : 1], v2[L2 ? L2 : 1];
};

template <uint32_t L, int POLICY>
__device__ __forceinline__ void load_piece(const MixArgs &a, uint32_t s, uint32_t u, u32x4 *v) {
    uint64_t lo = 0, hi = 0;
    piece(a.src_bytes[s], a.per_tile[s], u, a.tiles, lo, hi);
    const rsrc_t r = make_rsrc(a.src[s] + lo, (uint32_t)(hi - lo));
#pragma unroll
    for (uint32_t i = 0; i < L; ++i)
        v[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(16u * (i * kBlock + threadIdx.x)), 0, POLICY));
}

template <uint32_t L0, uint32_t L1, uint32_t L2, int NT1>
__device__ __forceinline__ void load_tile(const MixArgs &a, uint32_t u, TileIn<L0, L1, L2> &in) {
    if constexpr (L0 > 0) load_piece<L0, 0>(a, 0, u, in.v0);
    if constexpr (L1 > 0) load_piece<L1, NT1 ? kNonTemporal : 0>(a, 1, u, in.v1);
    if constexpr (L2 > 0) load_piece<L2, 0>(a, 2, u, in.v2);
}

template <uint32_t L0, uint32_t L1, uint32_t L2>
__device__ __forceinline__ u32x4 fold(const TileIn<L0, L1, L2> &in) {
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (uint32_t i = 0; i < L0; ++i) acc ^= in.v0[i];
#pragma unroll
    for (uint32_t i = 0; i < L1; ++i) acc ^= in.v1[i];
#pragma unroll
    for (uint32_t i = 0; i < L2; ++i) acc ^= in.v2[i];
    return acc;
}

// Workgroups take tiles grid-stride; the next tile's loads go out before
// this tile's stores (as in the decoder's pipelined loop); stores are
// non-temporal, as the decoder's.
template <uint32_t L0, uint32_t L1, uint32_t L2, int NT1>
__global__ __launch_bounds__(kBlock) void csf_probe_mix_kernel(MixArgs a) {
    uint32_t u = blockIdx.x;
    if (u >= a.tiles) return;
    TileIn<L0, L1, L2> in;
    load_tile<L0, L1, L2, NT1>(a, u, in);
    while (true) {
        const u32x4 acc = fold(in);
        const uint32_t un = u + gridDim.x;
        if (un < a.tiles) load_tile<L0, L1, L2, NT1>(a, un, in);
        uint64_t lo = 0, hi = 0;
        lo = uint64_t(kTile) * u;
        hi = min(lo + kTile, a.dst_bytes);
        const rsrc_t w = make_rsrc(a.dst + lo, (uint32_t)(hi - lo));
#pragma unroll
        for (uint32_t i = 0; i < kRuns; ++i) {
            const uint32_t j = i * kBlock + threadIdx.x;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc ^ (u32x4){j, u, i, 0u}), w,
                                                   (int)(16u * j), 0, kNonTemporal);
        }
        if (un >= a.tiles) break;
        u = un;
    }
}

// Instantiations: loads per lane of each stream's largest piece (stream 0:
// 1-2, stream 1: 0-3, stream 2: 0-1) and the entry stream's policy.
template <uint32_t L0, uint32_t L1, uint32_t L2>
void launch_mix_nt(const MixArgs &a, bool nt1, uint32_t grid, hipStream_t st) {
    if (nt1)
        hipLaunchKernelGGL((csf_probe_mix_kernel<L0, L1, L2, 1>), dim3(grid), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((csf_probe_mix_kernel<L0, L1, L2, 0>), dim3(grid), dim3(kBlock), 0, st, a);
}

template <uint32_t L0, uint32_t L1>
void launch_mix_l2(const MixArgs &a, uint32_t l2, bool nt1, uint32_t grid, hipStream_t st) {
    if (l2 == 0)
        launch_mix_nt<L0, L1, 0>(a, nt1, grid, st);
    else
        launch_mix_nt<L0, L1, 1>(a, nt1, grid, st);
}

template <uint32_t L0>
void launch_mix_l1(const MixArgs &a, uint32_t l1, uint32_t l2, bool nt1, uint32_t grid, hipStream_t st) {
    switch (l1) {
        case 0: launch_mix_l2<L0, 0>(a, l2, nt1, grid, st); break;
        case 1: launch_mix_l2<L0, 1>(a, l2, nt1, grid, st); break;
        case 2: launch_mix_l2<L0, 2>(a, l2, nt1, grid, st); break;
        default: launch_mix_l2<L0, 3>(a, l2, nt1, grid, st); break;
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
    if (nsrc == 0 || nsrc > 3 || dst == nullptr || dst_bytes == 0 || grid == 0 || dst_bytes >= (1ull << 40))
        return CSF_E_SIZE;
    if (nsrc > 0 && (src == nullptr || src_bytes == nullptr)) return CSF_E_NULL;
    MixArgs a = {};
    a.dst = dst;
    a.dst_bytes = dst_bytes;
    a.tiles = (uint32_t)((dst_bytes + kTile - 1) / kTile);
    a.nsrc = nsrc;
    a.flags = flags;
    if ((dst_bytes + kTile - 1) / kTile >= (1ull << 31)) return CSF_E_SIZE;
    uint32_t loads[3] = {0u, 0u, 0u};
    for (uint32_t s = 0; s < nsrc; ++s) {
        if (src[s] == nullptr) return CSF_E_NULL;
        if (src_bytes[s] >= (1ull << 40)) return CSF_E_SIZE;
        // the largest piece (the kernel's boundaries, computed the same way),
        // in loads of 4 KiB per workgroup
        a.per_tile[s] = double(src_bytes[s]) / double(a.tiles);
        uint64_t piece_bytes = 0, lo = 0;
        for (uint32_t u = 0; u < a.tiles; ++u) {
            const uint64_t hi = u + 1 == a.tiles ? src_bytes[s] : (uint64_t)(double(u + 1) * a.per_tile[s]) & ~15ull;
            piece_bytes = hi - lo > piece_bytes ? hi - lo : piece_bytes;
            lo = hi;
        }
        const uint64_t l = (piece_bytes + 4095) / 4096;
        if (l > (s == 0 ? 2u : s == 1 ? 3u : 1u)) return CSF_E_SIZE;
        loads[s] = uint32_t(l);
        a.src[s] = src[s];
        a.src_bytes[s] = src_bytes[s];
    }
    for (uint32_t s = nsrc; s < 3; ++s) a.src[s] = dst;  // never read
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    const bool nt1 = (flags & CSF_PROBE_NT_ENTRIES) != 0;
    if (loads[0] <= 1)
        launch_mix_l1<1>(a, loads[1], loads[2], nt1, grid, st);
    else
        launch_mix_l1<2>(a, loads[1], loads[2], nt1, grid, st);
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
