// CSF encoder on gfx950: the preparation step run on the GPU, as the pages'
// preparation does ("Load native FP4 experts with optional lossless CSF
// scales", vLLM PR 964, preparation paragraphs: encoding plus the index on the
// GPU).  Output is byte-identical to the host encoder for every input: the
// base of a row is the row value v with the most row values in
// [v, v + 2^w - 1], ties to the smallest v; offsets, exception entries,
// prefix and tile index follow the layout in include/csf.h.
//
// Four kernels, all byte streams bound by HBM bandwidth:
//   csf_enc_bases_short_kernel  rows of at most 255 columns (every workload
//                           stack): 16 lanes per row, byte-wide bins, window
//                           counts by SWAR arithmetic and DPP (below).
//   csf_enc_bases_kernel    any row: one wave per 4 rows at a time, a 256-bin
//                           histogram per row in LDS (4 bins per lane),
//                           window counts as differences of a wave prefix
//                           over the bins, arg-max by a wave reduction.
//   csf_enc_pack_kernel     one wave per index tile, one 16-byte run of
//                           dense bytes per lane and load: fields packed in
//                           the contiguous-decoding order, a group's runs
//                           combined across lanes; the tile's out-of-window
//                           count reduced across the wave.
//   csf_enc_scan_kernel     one workgroup: exclusive scan of the per-tile
//                           counts, in place, into tile_index and prefix;
//                           each wave reads and writes coalesced lines.
//   csf_enc_entries_kernel  one wave per index tile, one 16-byte run per lane
//                           and load: out-of-window positions ranked by wave
//                           prefixes and written in ascending order at the
//                           tile's index.
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

// Row bases along ascending positions of a plane from p0 on: the base of
// p0's row, then each further row's base read when a position reaches it.
struct RunBases {
    uint32_t r, next, b;
    __device__ __forceinline__ RunBases(const EncodeArgs &a, const uint8_t *brow, uint32_t p0) {
        r = div_exact(p0, a.rcp_cols);
        next = (r + 1u) * a.C;
        b = brow[r];
    }
    // base of position p; calls in ascending p
    __device__ __forceinline__ uint32_t at(const EncodeArgs &a, const uint8_t *brow, uint32_t p) {
        if (p == next) {
            ++r;
            next += a.C;
            b = brow[r];
        }
        return b;
    }
};

// 0xff in the bytes k >= s of a word, 0 below.
__device__ __forceinline__ uint32_t bytes_from(int32_t s) {
    return s <= 0 ? 0xffffffffu : (s >= 4 ? 0u : 0xffffffffu << (8 * s));
}

// Byte-wise x - y modulo 256 (no borrow between bytes).
__device__ __forceinline__ uint32_t byte_sub(uint32_t x, uint32_t y) {
    return ((x | 0x80808080u) - (y & 0x7f7f7f7fu)) ^ ((x ^ ~y) & 0x80808080u);
}

// 0x80 in each byte of x that is zero, else 0.
__device__ __forceinline__ uint32_t zero_bytes(uint32_t x) {
    return ~((((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) | 0x7f7f7f7fu);
}

// The two runs of 16 dense bytes a lane takes in an index tile (runs l and
// l + 64 of the tile for lane l) and, for rows of at least 16 columns, the
// bases of the row each run starts in and of the row after it: a run of 16
// meets at most two rows then.
struct TileRuns {
    uint32_t x[2][4];
    uint32_t b0[2], b1[2];
};

// (Tile numbers fit 32 bits: the host keeps E * P below 2^31.)
__device__ __forceinline__ uint32_t run_start(const EncodeArgs &a, uint64_t wv, uint32_t h, uint32_t lane) {
    const uint32_t it = (uint32_t)wv % a.index_tiles;
    return 16u * (it * (kIndexTile / 16) + h * kWave + lane);
}

__device__ __forceinline__ void fetch_runs(const EncodeArgs &a, uint64_t wv, uint32_t lane, bool vec,
                                           bool long_rows, TileRuns &t) {
    const uint32_t e = (uint32_t)wv / a.index_tiles;
    const uint8_t *plane = a.dense + (uint64_t)e * a.P;
    const uint8_t *brow = a.bases + (uint64_t)e * a.R;
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t p0 = run_start(a, wv, h, lane);
        t.x[h][0] = t.x[h][1] = t.x[h][2] = t.x[h][3] = 0u;
        t.b0[h] = t.b1[h] = 0u;
        if (p0 < a.P) {
            load_run16(plane, p0, a.P, vec, t.x[h]);
            if (long_rows) {
                const uint32_t r = div_exact(p0, a.rcp_cols);
                t.b0[h] = brow[r];
                t.b1[h] = r + 1u < a.R ? brow[r + 1u] : 0u;
            }
        }
    }
}

// Window test of run h of t (positions p0 .. p0 + 15, rows of at least 16
// columns), four bytes at a time: d[j] holds the byte differences (modulo
// 256) to the bases of their rows, valid[j] 0x80 in each byte inside the
// plane, keep[j] 0x80 in each valid byte inside its row's window: a
// difference below W without a borrow (a base may exceed 256 - W, so a byte
// below it can still differ by less than W modulo 256).
__device__ __forceinline__ void window_test16(const EncodeArgs &a, const TileRuns &t, uint32_t h, uint32_t p0,
                                              uint32_t (&d)[4], uint32_t (&keep)[4], uint32_t (&valid)[4]) {
    const uint32_t next = (div_exact(p0, a.rcp_cols) + 1u) * a.C;  // first position of the next row
    const uint32_t B0 = t.b0[h] * 0x01010101u, B1 = t.b1[h] * 0x01010101u;
    const uint32_t hi = (0x100u - (1u << a.wbits)) * 0x01010101u;  // bits that must be 0 in a kept difference
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t pt = p0 + 4u * j;
        const uint32_t x = t.x[h][j];
        const uint32_t in_next = bytes_from((int32_t)(next - pt));
        valid[j] = ~bytes_from((int32_t)(a.P - pt)) & 0x80808080u;
        const uint32_t bv = (B0 & ~in_next) | (B1 & in_next);
        d[j] = byte_sub(x, bv);
        // borrow out of each byte's top bit: the byte is below its base
        const uint32_t below = ((~x & bv) | (~(x ^ bv) & d[j])) & 0x80808080u;
        keep[j] = zero_bytes(d[j] & hi) & ~below & valid[j];
    }
}

// Buffer resource of the byte range [base, base + bytes): loads past it read 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Orders this wave's LDS traffic without waiting for its global memory
// operations: a wave's LDS operations are performed in issue order, so
// waiting for its outstanding ones (lgkmcnt(0) alone; gfx9 s_waitcnt
// encoding, vmcnt and expcnt left at their maxima) is all the ordering
// between this wave's histogram writes and reads needs.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
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

constexpr uint32_t kShortRows = 4;     // rows per wave at a time
constexpr uint32_t kShortWords = 4;    // 32-bit loads per lane per group: 4 * 4 * 64 bytes >= 4 * 255

// ---------------------------------------------------------------------------
// Row bases of rows of at most 255 columns (every count then fits a byte).
//
// A wave takes 4 rows at a time, 16 lanes per row (lane j of the row's
// group owns values 16 j .. 16 j + 15).  The rows' bytes (4 C, contiguous)
// are read as 32-bit words, the next 4 rows' while this group is counted.
// Counting: byte-wide bins in LDS, 4 per 32-bit word, by LDS atomic adds of
// 1 << 8 (v % 4) at word v / 4 of one of four copies (below).  Lane j then
// holds its 16 bins in four words h[0..3]; with SWAR byte arithmetic (no
// carry crosses a byte, as every sum of bins is at most C <= 255):
//   W = 16:  count(16 j + i) = T_j - pre_j(i) + pre_{j+1}(i), T_j the lane's
//            total and pre_j(i) its bins below i, pre_{j+1} taken from the
//            next lane by DPP (0 past the row's last lane: no values above
//            255);
//   W = 2:   count(v) = bin v + bin v + 1, bin 16 j + 16 being the next
//            lane's first.
// Counts of values absent from the row are zeroed; the row maximum M comes
// from packed 16-bit maxima and a 16-lane DPP rotation; the base is the
// smallest value whose count is M (a present value, since M >= 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t next_lane(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x101, 0xf, 0xf, true);  // row_shl:1
}

__device__ __forceinline__ uint32_t row_max16(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));  // row_ror:8
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false));  // row_ror:4
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xf, 0xf, false));  // row_ror:2
    return max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xf, 0xf, false));  // row_ror:1
}

__device__ __forceinline__ uint32_t row_min16(uint32_t x) {
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xf, 0xf, false));
    return min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xf, 0xf, false));
}

// 0xff in each byte of x that is not zero, else 0.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    const uint32_t t = (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
    return (t >> 7) * 0xffu;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                   __builtin_bit_cast(u16x2, b)));
}

// The base of row g of a group whose 4 rows' bytes are the words w (nbytes
// of them, whole words), counted in the wave's LDS bins hw; written by lane
// 0 of the row's 16 for rows below `rows`.
// LDS bins of one wave: 4 rows x 256 byte-wide bins (64 words per row), in
// K copies.  K = 1: row r's bin word d at 64 r + d.  K = 4: lane l counts
// into copy l % 4, so lanes adding to the same bin mostly hit different
// words, at word 16 d + 4 r + c: the 16 words of one d lie in 16 different
// banks, and one 16-byte read returns the four copies of a row's word.
// Four copies pay where most of a row's values fall in a few bins (the
// two-value window of one-bit offsets); elsewhere the extra clearing and
// reading cost more than the conflicts they remove.
template <uint32_t K>
__device__ __forceinline__ uint32_t bin_word(uint32_t d, uint32_t r, uint32_t lane) {
    return K == 1 ? 64u * r + d : 16u * d + 4u * r + lane % K;
}

template <uint32_t WB, uint32_t K, typename AfterCount>
__device__ __forceinline__ void group_bases(const EncodeArgs &a, uint32_t *hw, const uint32_t (&w)[kShortWords],
                                            uint32_t r0, uint32_t nbytes, uint32_t rows, AfterCount after_count) {
    const uint32_t lane = threadIdx.x % kWave, g = lane / 16, j = lane % 16;
    const uint32_t C = a.C;
#pragma unroll
    for (uint32_t t = 0; t < K; ++t)
        reinterpret_cast<uint4 *>(hw)[t * kWave + lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_order();
    // One branch per word (the group holds whole words).  A word's bytes may
    // straddle a row boundary: one when C >= 4, up to three when C < 4.
    if (C >= 4) {
#pragma unroll
        for (uint32_t i = 0; i < kShortWords; ++i) {
            const uint32_t o = 4u * (i * kWave + lane);  // first byte of the word in the group
            if (o < nbytes) {
                const uint32_t row = (o >= C) + (o >= 2 * C) + (o >= 3 * C);
                const uint32_t next = (row + 1) * C;  // first byte of the next row
#pragma unroll
                for (uint32_t k = 0; k < 4; ++k) {
                    const uint32_t v = __builtin_amdgcn_ubfe(w[i], 8 * k, 8);
                    const uint32_t rk = row + (o + k >= next ? 1u : 0u);
                    atomicAdd(&hw[bin_word<K>(v >> 2, rk, lane)], 1u << ((v & 3u) << 3));
                }
            }
        }
    } else {
        // 4 C <= 12 bytes: lanes 0 .. C - 1 hold the group's words
        const uint32_t o = 4u * lane;
        if (o < nbytes) {
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t ob = o + k;
                const uint32_t v = __builtin_amdgcn_ubfe(w[0], 8 * k, 8);
                const uint32_t rk = (ob >= C) + (ob >= 2 * C) + (ob >= 3 * C);
                atomicAdd(&hw[bin_word<K>(v >> 2, rk, lane)], 1u << ((v & 3u) << 3));
            }
        }
    }
    after_count();  // (the words are no longer needed)
    wave_lds_order();
    // row g, bins 16 j .. 16 j + 15: words 4 j .. 4 j + 3, the copies summed
    // (byte-wise: every sum of bins is at most C <= 255)
    uint32_t h[4];
    if constexpr (K == 1) {
        const uint4 hv = reinterpret_cast<const uint4 *>(hw)[lane];
        h[0] = hv.x;
        h[1] = hv.y;
        h[2] = hv.z;
        h[3] = hv.w;
    } else {
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) {
            const uint4 cp = reinterpret_cast<const uint4 *>(hw)[4 * (4 * j + t) + g];
            h[t] = cp.x + cp.y + cp.z + cp.w;
        }
    }
    uint32_t cnt[4];
    if constexpr (WB == 4) {
        uint32_t pre[4], run = 0;
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) {
            pre[t] = h[t] * 0x01010100u + run * 0x01010101u;  // bins of the lane below each byte
            run += (h[t] * 0x01010101u) >> 24;
        }
        const uint32_t total = run * 0x01010101u;
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) cnt[t] = total - pre[t] + next_lane(pre[t]);
    } else {
        const uint32_t nh0 = next_lane(h[0]);
#pragma unroll
        for (uint32_t t = 0; t < 4; ++t) cnt[t] = h[t] + (h[t] >> 8) + ((t < 3 ? h[t < 3 ? t + 1 : 0] : nh0) << 24);
    }
#pragma unroll
    for (uint32_t t = 0; t < 4; ++t) cnt[t] &= nonzero_bytes(h[t]);
    // the row's largest count
    uint32_t m = max_u16x2(max_u16x2(cnt[0] & 0x00ff00ffu, cnt[1] & 0x00ff00ffu),
                           max_u16x2(cnt[2] & 0x00ff00ffu, cnt[3] & 0x00ff00ffu));
    m = max_u16x2(m, max_u16x2(max_u16x2((cnt[0] >> 8) & 0x00ff00ffu, (cnt[1] >> 8) & 0x00ff00ffu),
                               max_u16x2((cnt[2] >> 8) & 0x00ff00ffu, (cnt[3] >> 8) & 0x00ff00ffu)));
    const uint32_t M = row_max16(max(m & 0xffffu, m >> 16));
    // the smallest value with that count
    const uint32_t sm = M * 0x01010101u;
    const uint64_t z01 = (uint64_t)zero_bytes(cnt[0] ^ sm) | ((uint64_t)zero_bytes(cnt[1] ^ sm) << 32);
    const uint64_t z23 = (uint64_t)zero_bytes(cnt[2] ^ sm) | ((uint64_t)zero_bytes(cnt[3] ^ sm) << 32);
    const uint32_t local = z01 ? (uint32_t)__builtin_ctzll(z01) >> 3
                               : (z23 ? 8u + ((uint32_t)__builtin_ctzll(z23) >> 3) : 256u);
    const uint32_t base = row_min16(local < 256u ? 16u * j + local : 256u);
    if (j == 0 && r0 + g < rows) a.bases[r0 + g] = (uint8_t)base;
    wave_lds_order();  // this group's bins read before the next group clears them
}

// The host sends stacks of fewer than 2^31 bytes, a multiple of 4, with
// rows of at most 255 columns; so the 32-bit group offsets below are exact
// and every group is whole words.
template <uint32_t WB, uint32_t K>
__global__ __launch_bounds__(kBlock) void csf_enc_bases_short_kernel(EncodeArgs a) {
    constexpr uint32_t kWaves = kBlock / kWave;
    __shared__ __align__(16) uint32_t hist[kWaves][256 * K];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t C = a.C;
    const uint32_t rows = a.E * a.R;
    const uint32_t groups = (rows + kShortRows - 1) / kShortRows;
    const uint32_t stride = gridDim.x * kWaves;
    uint32_t *hw = hist[wave];

    // The words of group q: bytes [4 q C, min(4 q C + 4 C, rows C)), word d
    // at byte 4 d, loaded through a resource over exactly those bytes.
    auto load_group = [&](uint32_t q, uint32_t (&w)[kShortWords]) {
        // (uniform; said so, so the resource stays in scalar registers)
        const uint32_t first = __builtin_amdgcn_readfirstlane(q * kShortRows * C);
        const uint32_t end = __builtin_amdgcn_readfirstlane(min(first + kShortRows * C, rows * C));
        const rsrc_t r = make_rsrc(a.dense + first, end - first);
#pragma unroll
        for (uint32_t i = 0; i < kShortWords; ++i)
            w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(4u * (i * kWave + lane)), 0, 0);
    };
    auto nbytes_of = [&](uint32_t q) { return (min(q * kShortRows + kShortRows, rows) - q * kShortRows) * C; };

    // The next group's words are loaded once this group's are counted, while
    // its bases are found.
    uint32_t q = blockIdx.x * kWaves + wave;
    uint32_t w[kShortWords];
    if (q < groups) load_group(q, w);
    for (; q < groups; q += stride)
        group_bases<WB, K>(a, hw, w, q * kShortRows, nbytes_of(q), rows, [&] {
            if (q + stride < groups) load_group(q + stride, w);
        });
}

// OR of x over this lane and the s - 1 lanes below it in its 16-lane row
// (s = 1, 2, 4 or 8): the last lane of each aligned group of s holds the
// group's OR.
__device__ __forceinline__ uint32_t or_down(uint32_t x, uint32_t s) {
    if (s > 1) x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    if (s > 2) x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    if (s > 4) x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    return x;
}

// One wave per index tile (kIndexTile positions = 128 runs of 16); lane l
// takes runs l and l + 64 of the tile, so each load instruction of a wave
// reads 1 KiB of contiguous dense bytes.  Run q holds field q % F of group
// q / F (F = 8 / w runs per group): its 16 values' offsets (0 out of the
// window) at bits w (q % F) of the group's 16 bytes.  The F runs of a group
// are F consecutive lanes; an OR down those lanes gives the group to its
// last lane, which stores it.  The tile's out-of-window count is a sum over
// the wave.
__global__ __launch_bounds__(kBlock) void csf_enc_pack_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x % kWave;
    const uint64_t total_waves = (uint64_t)a.E * a.index_tiles;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock / kWave;
    const uint32_t W = 1u << a.wbits;
    const uint32_t F = 8u / a.wbits;
    const bool vec = runs_aligned(a);
    const bool long_rows = a.C >= 16u;
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves; wv += stride) {
        TileRuns cur;
        fetch_runs(a, wv, lane, vec, long_rows, cur);
        const uint32_t e = (uint32_t)wv / a.index_tiles;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        uint32_t outside = 0;
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            const uint32_t q = p0 / 16u;  // run in the plane
            const uint32_t f = q % F;
            uint32_t word[4] = {0u, 0u, 0u, 0u};
            if (p0 < a.P && long_rows) {
                uint32_t d[4], keep[4], valid[4];
                window_test16(a, cur, h, p0, d, keep, valid);
#pragma unroll
                for (uint32_t t = 0; t < 4; ++t) {
                    // a kept difference is below W: its field is its low w bits
                    word[t] = (d[t] & ((keep[t] >> 7) * 0xffu)) << (a.wbits * f);
                    outside += __popc(valid[t] & ~keep[t]);
                }
            } else if (p0 < a.P) {
                RunBases rb(a, brow, p0);
#pragma unroll
                for (uint32_t j = 0; j < 16; ++j) {
                    const uint32_t p = p0 + j;
                    if (p < a.P) {
                        const uint32_t b = rb.at(a, brow, p);
                        // unsigned 32-bit difference: a value below b differs by far more than W
                        const uint32_t d = ((cur.x[h][j >> 2] >> (8u * (j & 3u))) & 0xffu) - b;
                        const bool in = d < W;
                        outside += in ? 0u : 1u;
                        word[j >> 2] |= (in ? d : 0u) << (8u * (j & 3u) + a.wbits * f);
                    }
                }
            }
#pragma unroll
            for (uint32_t t = 0; t < 4; ++t) word[t] = or_down(word[t], F);
            const uint32_t g = q / F;
            if (f == F - 1u && g < a.groups) {
                uint4 *dst = reinterpret_cast<uint4 *>(a.offsets + (uint64_t)e * a.stride + 16u * g);
                *dst = make_uint4(word[0], word[1], word[2], word[3]);
            }
        }
        for (uint32_t d = 1; d < kWave; d <<= 1) outside += __shfl_xor(outside, d, kWave);
        if (lane == 0) a.tile_index[wv] = (int32_t)outside;
    }
}

// Inclusive sum of x over lanes 0 .. lane of the wave: a scan inside each
// 16-lane row by DPP row shifts (lanes shifted in from outside the row add
// 0), then the totals of the rows below added from their last lanes.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    const uint32_t row = (threadIdx.x % kWave) / 16;
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    return x + (row > 0 ? t0 : 0u) + (row > 1 ? t1 : 0u) + (row > 2 ? t2 : 0u);
}

// One workgroup: tile_index[0 .. N) holds per-tile counts; replace them by
// their exclusive prefix, set tile_index[N] = total, prefix[e] =
// tile_index[e * NT] and prefix[E] = total.  The host keeps E * P < 2^31.
// Wave w owns the contiguous segment [w * seg, (w + 1) * seg) of whole
// 64-count lines and reads it kScanBatch lines at a time, each load one
// coalesced line, every load of a batch in flight together; when the
// segment fits one batch its counts stay in registers for the second pass.
__global__ __launch_bounds__(kScanThreads) void csf_enc_scan_kernel(EncodeArgs a) {
    constexpr uint32_t kScanBatch = 32;
    constexpr uint32_t kWaves = kScanThreads / kWave;
    __shared__ uint32_t wave_sums[kWaves];
    const uint32_t N = a.E * a.index_tiles;
    const uint32_t seg = (N + kScanThreads - 1) / kScanThreads * kWave;  // counts per wave
    const uint32_t wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint32_t lo = min(wid * seg, N), hi = min(lo + seg, N);
    int32_t *ti = a.tile_index;
    uint32_t v[kScanBatch];
    uint32_t sum = 0;
    for (uint32_t b = lo; b < hi; b += kScanBatch * kWave) {
#pragma unroll
        for (uint32_t i = 0; i < kScanBatch; ++i) {
            const uint32_t k = b + i * kWave + lane;
            v[i] = k < hi ? (uint32_t)ti[k] : 0u;
        }
#pragma unroll
        for (uint32_t i = 0; i < kScanBatch; ++i) sum += v[i];
    }
    const uint32_t wave_total = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(sum), kWave - 1);
    if (lane == 0) wave_sums[wid] = wave_total;
    __syncthreads();
    uint32_t run = 0, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; ++w) {
        const uint32_t s = wave_sums[w];
        run += w < wid ? s : 0u;
        total += s;
    }
    const bool kept = seg <= kScanBatch * kWave;  // v holds this wave's whole segment
    for (uint32_t b = lo; b < hi; b += kScanBatch * kWave) {
        if (!kept) {
#pragma unroll
            for (uint32_t i = 0; i < kScanBatch; ++i) {
                const uint32_t k = b + i * kWave + lane;
                v[i] = k < hi ? (uint32_t)ti[k] : 0u;
            }
        }
#pragma unroll
        for (uint32_t i = 0; i < kScanBatch; ++i) {
            const uint32_t k = b + i * kWave + lane;
            const uint32_t inc = wave_inclusive_sum(v[i]);
            if (k < hi) ti[k] = (int32_t)(run + inc - v[i]);
            run += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
        }
    }
    if (threadIdx.x == 0) {
        ti[N] = (int32_t)total;
        a.prefix[a.E] = (int32_t)total;
    }
    __syncthreads();  // every thread's tile_index writes are visible in the workgroup
    for (uint32_t e = threadIdx.x; e < a.E; e += kScanThreads) a.prefix[e] = ti[(uint64_t)e * a.index_tiles];
}

// One wave per index tile (128 runs of 16 positions); lane l takes runs l
// and l + 64 of the tile, so each load instruction reads 1 KiB of contiguous
// dense bytes.  Position order is (half, lane, position in run): a wave
// prefix of the out-of-window counts of each half ranks the entries, and
// each lane writes its own in ascending order, bytes taken from the loaded
// registers.
__global__ __launch_bounds__(kBlock) void csf_enc_entries_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x % kWave;
    const uint64_t total_waves = (uint64_t)a.E * a.index_tiles;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock / kWave;
    const uint32_t W = 1u << a.wbits;
    const bool vec = runs_aligned(a);
    const bool long_rows = a.C >= 16u;
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves; wv += stride) {
        TileRuns cur;
        fetch_runs(a, wv, lane, vec, long_rows, cur);
        const uint32_t e = (uint32_t)wv / a.index_tiles;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        uint32_t flags[2] = {0u, 0u};
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            if (p0 < a.P && long_rows) {
                uint32_t d[4], keep[4], valid[4];
                window_test16(a, cur, h, p0, d, keep, valid);
#pragma unroll
                for (uint32_t t = 0; t < 4; ++t) {
                    // gather the 0x80 bits of the word's outside bytes into 4 bits
                    const uint32_t out = valid[t] & ~keep[t];
                    flags[h] |= ((out * 0x00204081u) >> 28) << (4u * t);
                }
            } else if (p0 < a.P) {
                RunBases rb(a, brow, p0);
#pragma unroll
                for (uint32_t j = 0; j < 16; ++j) {
                    const uint32_t p = p0 + j;
                    if (p < a.P) {
                        const uint32_t b = rb.at(a, brow, p);
                        const uint32_t byte = (cur.x[h][j >> 2] >> (8u * (j & 3u))) & 0xffu;
                        if (byte - b >= W) flags[h] |= 1u << j;  // 32-bit difference: below b is outside
                    }
                }
            }
        }
        const uint32_t c0 = __popc(flags[0]), c1 = __popc(flags[1]);
        const uint32_t i0 = wave_inclusive_sum(c0), i1 = wave_inclusive_sum(c1);
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)i0, kWave - 1);
        const uint32_t first = (uint32_t)a.tile_index[wv];
        const uint32_t out0[2] = {first + i0 - c0, first + t0 + i1 - c1};
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            uint32_t fl = flags[h], o = out0[h];
            while (fl != 0u) {
                const uint32_t j = __ffs(fl) - 1u;
                fl &= fl - 1u;
                const uint32_t w = j < 8u ? (j < 4u ? cur.x[h][0] : cur.x[h][1])
                                          : (j < 12u ? cur.x[h][2] : cur.x[h][3]);
                a.exc[o++] = ((p0 + j) << 8) | __builtin_amdgcn_ubfe(w, 8u * (j & 3u), 8u);
            }
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
    uint32_t grid;
    const uint64_t n = (uint64_t)a.E * a.R * a.C;
    if (a.C <= 255 && ((uintptr_t)a.dense & 3u) == 0 && n % 4 == 0 && n < (1ull << 31)) {
        const uint64_t groups = ((uint64_t)a.E * a.R + kShortRows - 1) / kShortRows;
        grid = grid_for(groups, cus);
        if (a.wbits == 4)
            hipLaunchKernelGGL((csf_enc_bases_short_kernel<4, 1>), dim3(grid), dim3(kBlock), 0, stream, a);
        else
            hipLaunchKernelGGL((csf_enc_bases_short_kernel<1, 4>), dim3(grid), dim3(kBlock), 0, stream, a);
    } else {
        grid = grid_for((uint64_t)a.E * a.R, cus);
        hipLaunchKernelGGL(csf_enc_bases_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    grid = grid_for((uint64_t)a.E * a.index_tiles, cus);
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
