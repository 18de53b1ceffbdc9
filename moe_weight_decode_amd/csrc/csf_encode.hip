// CSF encoder on gfx950: the preparation step run on the GPU, as the pages'
// preparation does ("Load native FP4 experts with optional lossless CSF
// scales", vLLM PR 964, preparation paragraphs: encoding plus the index on the
// GPU).  Output is byte-identical to the host encoder for every input: the
// base of a row is the row value v with the most row values in
// [v, v + 2^w - 1], ties to the smallest v; offsets, exception entries,
// prefix and tile index follow the layout in include/csf.h.
//
// Four kernels, all byte streams bound by HBM bandwidth:
//   csf_enc_bases_kernel    one wave per 4 rows at a time: a 256-bin
//                           histogram per row in LDS (4 bins per lane),
//                           window counts as differences of a wave prefix
//                           over the bins, arg-max by a wave reduction.
//   csf_enc_pack_kernel     one lane per 16-byte offset group: fields packed
//                           in the contiguous-decoding order; each index
//                           tile's out-of-window count reduced across lanes.
//   csf_enc_scan_kernel     one workgroup: exclusive scan of the per-tile
//                           counts, in place, into tile_index and prefix.
//   csf_enc_entries_kernel  one wave per index tile: out-of-window positions
//                           ranked by a wave prefix and written in ascending
//                           order at the tile's index.
// The pack and entries kernels read the dense bytes 16 at a time when the
// stack is 16-byte aligned and R*C is a multiple of 16, else byte by byte.
#include "csf_launch.h"

namespace csf {
namespace {

constexpr uint32_t kWave = 64;
constexpr uint32_t kScanThreads = 1024;

__device__ __forceinline__ uint32_t div_exact(uint32_t n, double rcp) {
    return (uint32_t)(((double)n + 0.5) * rcp);
}

// Dense bytes plane[p0 .. p0+16), zero at and past P, as four little-endian
// words.  vec: the plane is 16-byte aligned and P a multiple of 16, so a run
// starting below P lies inside the plane.
__device__ __forceinline__ void load_run16(const uint8_t *plane, uint32_t p0, uint32_t P, bool vec,
                                           uint32_t x[4]) {
    if (vec) {
        const uint4 v = *reinterpret_cast<const uint4 *>(plane + p0);
        x[0] = v.x;
        x[1] = v.y;
        x[2] = v.z;
        x[3] = v.w;
        return;
    }
    x[0] = x[1] = x[2] = x[3] = 0u;
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j)
        if (p0 + j < P) x[j >> 2] |= (uint32_t)plane[p0 + j] << (8u * (j & 3u));
}

__device__ __forceinline__ bool runs_aligned(const EncodeArgs &a) {
    return ((uintptr_t)a.dense & 15u) == 0 && (a.P & 15u) == 0;
}

// Orders this wave's LDS traffic (a wave works on its own histogram).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kBlock) void csf_enc_bases_kernel(EncodeArgs a) {
    constexpr uint32_t kWaves = kBlock / kWave;
    constexpr uint32_t kRows = 4;  // rows per wave at a time: their dependent chains interleave
    __shared__ __align__(16) uint32_t hist[kWaves][kRows][256];
    const uint32_t wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint32_t W = 1u << a.wbits;
    const uint64_t rows = (uint64_t)a.E * a.R;
    for (uint64_t r0 = ((uint64_t)blockIdx.x * kWaves + wave) * kRows; r0 < rows;
         r0 += (uint64_t)gridDim.x * kWaves * kRows) {
#pragma unroll
        for (uint32_t r = 0; r < kRows; ++r)
            reinterpret_cast<uint4 *>(hist[wave][r])[lane] = make_uint4(0u, 0u, 0u, 0u);
        wave_lds_sync();
        for (uint32_t c = lane; c < a.C; c += kWave) {
            uint32_t v[kRows];
#pragma unroll
            for (uint32_t r = 0; r < kRows; ++r)
                v[r] = r0 + r < rows ? (uint32_t)a.dense[(r0 + r) * a.C + c] : 0x100u;
#pragma unroll
            for (uint32_t r = 0; r < kRows; ++r)
                if (v[r] < 256u) atomicAdd(&hist[wave][r][v[r]], 1u);
        }
        wave_lds_sync();
        // Lane l holds bins 4l .. 4l+3 of each row.  below[i] = values < 4l + i,
        // from the lane's exclusive prefix over the wave plus its own bins.
        uint32_t cnt[kRows][4], incl[kRows], own[kRows];
#pragma unroll
        for (uint32_t r = 0; r < kRows; ++r) {
            const uint4 c4 = reinterpret_cast<const uint4 *>(hist[wave][r])[lane];
            cnt[r][0] = c4.x;
            cnt[r][1] = c4.y;
            cnt[r][2] = c4.z;
            cnt[r][3] = c4.w;
            own[r] = c4.x + c4.y + c4.z + c4.w;
            incl[r] = own[r];
        }
#pragma unroll
        for (uint32_t d = 1; d < kWave; d <<= 1) {
#pragma unroll
            for (uint32_t r = 0; r < kRows; ++r) {
                const uint32_t y = __shfl_up(incl[r], d, kWave);
                if (lane >= d) incl[r] += y;
            }
        }
        // Values in [v, v + W - 1] (bins past 255 empty) = below(v + W) - below(v);
        // v + W = 4(l + q) + r with q, r the same for every lane, and
        // below(256 and up) = C.
        // key = (count in window << 8) | (255 - v) over present values v: the
        // largest key has the largest count, then the smallest v.
        uint32_t best[kRows];
#pragma unroll
        for (uint32_t r = 0; r < kRows; ++r) {
            const uint32_t ex = incl[r] - own[r];
            const uint32_t below[4] = {ex, ex + cnt[r][0], ex + cnt[r][0] + cnt[r][1],
                                       ex + cnt[r][0] + cnt[r][1] + cnt[r][2]};
            best[r] = 0;
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                const uint32_t q = (i + W) >> 2, m = (i + W) & 3u;
                const uint32_t src = lane + q;
                const uint32_t sel = m == 0 ? below[0] : m == 1 ? below[1] : m == 2 ? below[2] : below[3];
                const uint32_t far = __shfl(sel, (int)(src & (kWave - 1u)), kWave);
                const uint32_t top = src < kWave ? far : a.C;
                const uint32_t v = 4u * lane + i;
                if (cnt[r][i] != 0) best[r] = max(best[r], ((top - below[i]) << 8) | (255u - v));
            }
        }
#pragma unroll
        for (uint32_t d = 32; d >= 1; d >>= 1) {
#pragma unroll
            for (uint32_t r = 0; r < kRows; ++r) best[r] = max(best[r], (uint32_t)__shfl_xor(best[r], d, kWave));
        }
        if (lane == 0) {
#pragma unroll
            for (uint32_t r = 0; r < kRows; ++r)
                if (r0 + r < rows) a.bases[r0 + r] = (uint8_t)(255u - (best[r] & 0xffu));
        }
        wave_lds_sync();
    }
}

__global__ __launch_bounds__(kBlock) void csf_enc_pack_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t waves_per_expert = (a.groups + kWave - 1) / kWave;
    const uint64_t total_waves = (uint64_t)a.E * waves_per_expert;
    const uint32_t W = 1u << a.wbits;
    const uint32_t G = 128u / a.wbits;
    const uint32_t F = 8u / a.wbits;
    const uint32_t seg = kIndexTile / G;  // lanes (groups) per index tile: 64 or 16
    const bool vec = runs_aligned(a);
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves;
         wv += (uint64_t)gridDim.x * kBlock / kWave) {
        const uint32_t e = (uint32_t)(wv / waves_per_expert);
        const uint32_t g = (uint32_t)(wv - (uint64_t)e * waves_per_expert) * kWave + lane;
        const uint8_t *plane = a.dense + (uint64_t)e * a.P;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        uint32_t word[4] = {0u, 0u, 0u, 0u};
        uint32_t outside = 0;
        if (g < a.groups) {
            for (uint32_t f = 0; f < F; ++f) {
                const uint32_t p0 = g * G + 16u * f;
                if (p0 >= a.P) break;
                uint32_t x[4];
                load_run16(plane, p0, a.P, vec, x);
                uint32_t r = div_exact(p0, a.rcp_cols);
                uint32_t next = (r + 1u) * a.C;
                uint32_t b = brow[r];
#pragma unroll
                for (uint32_t j = 0; j < 16; ++j) {
                    const uint32_t p = p0 + j;
                    if (p < a.P) {
                        if (p == next) {
                            ++r;
                            next += a.C;
                            b = brow[r];
                        }
                        // unsigned 32-bit difference: the window [b, b + W - 1] does
                        // not wrap past 255, so a value below b is never inside it
                        const uint32_t d = ((x[j >> 2] >> (8u * (j & 3u))) & 0xffu) - b;
                        const bool in = d < W;
                        outside += in ? 0u : 1u;
                        word[j >> 2] |= (in ? d : 0u) << (8u * (j & 3u) + a.wbits * f);
                    }
                }
            }
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.offsets + (uint64_t)e * a.stride + 16u * g);
            dst[0] = word[0];
            dst[1] = word[1];
            dst[2] = word[2];
            dst[3] = word[3];
        }
        // Sum the counts of each index tile's lanes (seg consecutive lanes).
        for (uint32_t d = 1; d < seg; d <<= 1) outside += __shfl_xor(outside, d, kWave);
        const uint32_t tile = g / seg;
        if (lane % seg == 0 && tile < a.index_tiles && g < a.groups)
            a.tile_index[(uint64_t)e * a.index_tiles + tile] = (int32_t)outside;
    }
}

// One workgroup: tile_index[0 .. N) holds per-tile counts; replace them by
// their exclusive prefix, set tile_index[N] = total, prefix[e] =
// tile_index[e * NT] and prefix[E] = total.  The host keeps E * P < 2^31.
__global__ __launch_bounds__(kScanThreads) void csf_enc_scan_kernel(EncodeArgs a) {
    __shared__ uint32_t part[kScanThreads];
    const uint32_t N = a.E * a.index_tiles;
    const uint32_t chunk = (N + kScanThreads - 1) / kScanThreads;
    const uint32_t t = threadIdx.x;
    const uint32_t lo = min(t * chunk, N), hi = min(lo + chunk, N);
    uint32_t sum = 0;
#pragma unroll 8
    for (uint32_t i = lo; i < hi; ++i) sum += (uint32_t)a.tile_index[i];
    part[t] = sum;
    __syncthreads();
    // Hillis-Steele inclusive scan of the partial sums.
    for (uint32_t d = 1; d < kScanThreads; d <<= 1) {
        const uint32_t v = t >= d ? part[t - d] : 0u;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t run = part[t] - sum;  // exclusive
#pragma unroll 8
    for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t c = (uint32_t)a.tile_index[i];
        a.tile_index[i] = (int32_t)run;
        run += c;
    }
    const uint32_t total = part[kScanThreads - 1];
    if (t == 0) {
        a.tile_index[N] = (int32_t)total;
        a.prefix[a.E] = (int32_t)total;
    }
    __syncthreads();  // every thread's tile_index writes are visible in the workgroup
    for (uint32_t e = t; e < a.E; e += kScanThreads)
        a.prefix[e] = a.tile_index[(uint64_t)e * a.index_tiles];
}

// One wave per index tile of kIndexTile positions; lane l takes positions
// 32l .. 32l+31 of the tile, so lane order is position order.
__global__ __launch_bounds__(kBlock) void csf_enc_entries_kernel(EncodeArgs a) {
    constexpr uint32_t kPerLane = kIndexTile / kWave;  // 32
    const uint32_t lane = threadIdx.x % kWave;
    const uint64_t total_waves = (uint64_t)a.E * a.index_tiles;
    const uint32_t W = 1u << a.wbits;
    const bool vec = runs_aligned(a);
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves;
         wv += (uint64_t)gridDim.x * kBlock / kWave) {
        const uint32_t e = (uint32_t)(wv / a.index_tiles);
        const uint32_t it = (uint32_t)(wv - (uint64_t)e * a.index_tiles);
        const uint8_t *plane = a.dense + (uint64_t)e * a.P;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        const uint32_t p0 = it * kIndexTile + lane * kPerLane;
        uint32_t flags = 0;
        if (p0 < a.P) {
            uint32_t x[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            load_run16(plane, p0, a.P, vec, x);
            if (p0 + 16u < a.P) load_run16(plane, p0 + 16u, a.P, vec, x + 4);
            uint32_t r = div_exact(p0, a.rcp_cols);
            uint32_t next = (r + 1u) * a.C;
            uint32_t b = brow[r];
#pragma unroll
            for (uint32_t k = 0; k < kPerLane; ++k) {
                const uint32_t p = p0 + k;
                if (p < a.P) {
                    if (p == next) {
                        ++r;
                        next += a.C;
                        b = brow[r];
                    }
                    const uint32_t byte = (x[k >> 2] >> (8u * (k & 3u))) & 0xffu;
                    if (byte - b >= W) flags |= 1u << k;  // no wrap past 255
                }
            }
        }
        const uint32_t cnt = __popc(flags);
        uint32_t incl = cnt;
#pragma unroll
        for (uint32_t d = 1; d < kWave; d <<= 1) {
            const uint32_t y = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += y;
        }
        uint32_t k_out = (uint32_t)a.tile_index[wv] + (incl - cnt);
        while (flags != 0) {
            const uint32_t k = __ffs(flags) - 1;
            flags &= flags - 1;
            a.exc[k_out++] = ((p0 + k) << 8) | plane[p0 + k];
        }
    }
}

}  // namespace

static uint32_t grid_for(uint64_t waves_needed, uint32_t cus) {
    const uint64_t wgs = (waves_needed + kBlock / kWave - 1) / (kBlock / kWave);
    const uint64_t cap = (uint64_t)cus * 16;
    return (uint32_t)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap);
}

hipError_t launch_encode_streams(const EncodeArgs &a, uint32_t cus, hipStream_t stream) {
    uint32_t grid = grid_for((uint64_t)a.E * a.R, cus);
    hipLaunchKernelGGL(csf_enc_bases_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    grid = grid_for((uint64_t)a.E * ((a.groups + kWave - 1) / kWave), cus);
    hipLaunchKernelGGL(csf_enc_pack_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(csf_enc_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_encode_entries(const EncodeArgs &a, uint32_t cus, hipStream_t stream) {
    const uint32_t grid = grid_for((uint64_t)a.E * a.index_tiles, cus);
    hipLaunchKernelGGL(csf_enc_entries_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csf
