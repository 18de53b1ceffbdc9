// CSF encoder on gfx950: the preparation step run on the GPU, as the pages'
// preparation does ("Load native FP4 experts with optional lossless CSF
// scales", vLLM PR 964, preparation paragraphs: encoding plus the index on the
// GPU).  Output is byte-identical to the host encoder for every input: the
// base of a row is the row value v with the most row values in
// [v, v + 2^w - 1], ties to the smallest v; offsets, exception entries,
// prefix and tile index follow the layout in include/csf.h.
//
// The kernels, in launch order:
//   csf_enc_bases_pair_kernel  rows of at most 255 columns in a 16-byte
//                           aligned stack (every workload stack): two lanes
//                           per row, the row's byte-wide bins in LDS, window
//                           counts by SWAR arithmetic (below).
//   csf_enc_bases_kernel    any other stack: one wave per 4 rows, a 256-bin
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

__host__ __device__ inline bool runs_aligned(const EncodeArgs &a) {
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
    const uint32_t c = (uint32_t)min(max(s, 0), 4);
    return (uint32_t)(0xffffffffffffffffull << (8u * c));
}

// 0xff in each byte of x whose bit 7 is set, else 0 (v_perm's sign
// selectors 8-11 read bit 7 of bytes 1, 3, 5, 7 of {x, x << 8}).
__device__ __forceinline__ uint32_t widen80(uint32_t x) { return __builtin_amdgcn_perm(x, x << 8, 0x0b090a08u); }

// Byte b (< 256) in all four bytes.
__device__ __forceinline__ uint32_t splat_byte(uint32_t b) { return __builtin_amdgcn_perm(0u, b, 0u); }

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
// plane (every byte when VEC: the plane is whole runs), keep[j] 0x80 in each
// valid byte inside its row's window: a difference below W, without a
// borrow when HIGH (some base in the wave exceeds 256 - W, so a byte below
// it can still differ from it by less than W modulo 256).
template <bool VEC, bool HIGH>
__device__ __forceinline__ void window_test16(const EncodeArgs &a, const TileRuns &t, uint32_t h, uint32_t p0,
                                              uint32_t (&d)[4], uint32_t (&keep)[4], uint32_t (&valid)[4]) {
    const int32_t to_next = (int32_t)((div_exact(p0, a.rcp_cols) + 1u) * a.C - p0);  // bytes left in p0's row
    const uint32_t B0 = splat_byte(t.b0[h]), B1 = splat_byte(t.b1[h]);
    const uint32_t hi = (0x100u - (1u << a.wbits)) * 0x01010101u;  // bits that must be 0 in a kept difference
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t x = t.x[h][j];
        const uint32_t in_next = bytes_from(to_next - (int32_t)(4u * j));
        valid[j] = VEC ? 0x80808080u : ~bytes_from((int32_t)(a.P - p0 - 4u * j)) & 0x80808080u;
        const uint32_t bv = (B0 & ~in_next) | (B1 & in_next);
        d[j] = byte_sub(x, bv);
        uint32_t k = zero_bytes(d[j] & hi) & valid[j];
        if (HIGH) k &= ~((~x & bv) | (~(x ^ bv) & d[j]));  // borrow out of a byte: below its base
        keep[j] = k;
    }
}

// Buffer resource of the byte range [base, base + bytes): loads past it read 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                   __builtin_bit_cast(u16x2, b)));
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

// ---------------------------------------------------------------------------
// Row bases, two lanes per row (rows of at most 255 columns, a 16-byte
// aligned stack).  A wave takes 32 rows at a time: lanes r and r + 32 share
// row r.  The row's histogram of the 256 byte values lives in LDS, one byte
// per bin (a row's count fits a byte), 64 words plus one of padding, so
// word w of row r sits in bank (r + w) mod 32 and the 32 lanes of a half
// wave never meet in a bank.  Lane half h reads the 16-byte chunks h, h + 2,
// ... that cover the row (buffer loads, the next group of rows in flight
// while this one is counted) and adds each of the row's bytes to its bin.
// Then half h walks bin words 32h .. 32h + 31: byte-wise prefix sums give
// every window count four candidates at a time (the four windows that cross
// into the upper half take the upper lane's first prefixes by one lane
// exchange); the largest key (count << 8 | 255 - v) over the two lanes
// gives the best count and its first v, and the first value present from
// that v on is the base (most values in the window, then the smallest
// present v).  The lanes then clear their bins.  Nothing else crosses
// lanes, so there is no barrier.
// ---------------------------------------------------------------------------
constexpr uint32_t kRowWords = 65;       // 64 bin words + 1 of padding
constexpr uint32_t kPairRows = 32;       // rows per wave at a time
constexpr uint32_t kPairWavesPerCu = 18;  // one-wave workgroups per CU: 18 x 8,320 B of LDS


// Fold the window counts cnt of candidates 4s .. 4s + 3 (s relative to the
// lane's half) into best: two u16 keys per word, count << 8 | 255 - v.  The
// keys interleave cnt's bytes with those of k = (255 - v, 254 - v, 253 - v,
// 252 - v) for v = 4s, one byte permute each.
__device__ __forceinline__ uint32_t fold_keys(uint32_t best, uint32_t cnt, uint32_t s) {
    const uint32_t k = 0xfcfdfeffu - 0x04040404u * s;
    const uint32_t lo = __builtin_amdgcn_perm(cnt, k, 0x06020400u);  // v, v + 2
    const uint32_t hi = __builtin_amdgcn_perm(cnt, k, 0x07030501u);  // v + 1, v + 3
    return max_u16x2(best, max_u16x2(lo, hi));
}

template <uint32_t WB, uint32_t CPL, bool ALIGNED>  // CPL: chunks per lane at most
__global__ __launch_bounds__(kWave) void csf_enc_bases_pair_kernel(EncodeArgs a) {
    __shared__ uint32_t hist[kPairRows * kRowWords];
    const uint32_t lane = threadIdx.x, r = lane % kPairRows, half = lane / kPairRows;
    uint32_t *h = hist + r * kRowWords;
    uint32_t *hh = h + 32u * half;  // this lane's half of the bins
    const uint32_t C = a.C, rows = a.E * a.R;  // rows * C < 2^31
    const uint32_t n = rows * C;
    const uint32_t groups = (rows + kPairRows - 1) / kPairRows;
    // chunks a row can meet: it starts at a multiple of gcd(C, 16) within its chunk
    const uint32_t nch = ALIGNED ? C / 16u : (C + 31u - min(C & (0u - C), 16u)) / 16u;
    const rsrc_t src = make_rsrc(a.dense, n);
#pragma unroll
    for (uint32_t w = 0; w < 32; ++w) hh[w] = 0u;
    // (The buffer's range check zeroes a whole dword that runs past the stack,
    // so the chunk holding the stack's last bytes, when they are not whole
    // dwords, is read byte by byte.)
    auto load = [&](uint32_t g, uint32_t (&x)[CPL][4]) {
        const uint32_t first = ((g * kPairRows + r) * C) & ~15u;
#pragma unroll
        for (uint32_t c = 0; c < CPL; ++c) {
            x[c][0] = x[c][1] = x[c][2] = x[c][3] = 0u;
            const uint32_t i = 2u * c + half;
            const uint32_t off = first + 16u * i;
            if (i < nch) {
                if (off + 16u <= n || off >= n) {
                    const v4u q = __builtin_amdgcn_raw_buffer_load_b128(src, (int)off, 0, 0);
                    x[c][0] = q[0];
                    x[c][1] = q[1];
                    x[c][2] = q[2];
                    x[c][3] = q[3];
                } else {
#pragma unroll
                    for (uint32_t b = 0; b < 16; ++b)
                        if (off + b < n) x[c][b >> 2] |= (uint32_t)a.dense[off + b] << (8u * (b & 3u));
                }
            }
        }
    };
    uint32_t x[CPL][4];
    uint32_t g = blockIdx.x;
    if (g < groups) load(g, x);
    for (; g < groups; g += gridDim.x) {
        uint32_t y[CPL][4];
        if (g + gridDim.x < groups) load(g + gridDim.x, y);
        const uint32_t row = g * kPairRows + r;
        const bool live = row < rows;  // the same for both lanes of a row
        if (live) {
            const uint32_t o = ALIGNED ? 0u : (row * C) & 15u;  // the row's first byte in chunk 0
#pragma unroll
            for (uint32_t c = 0; c < CPL; ++c) {
                const uint32_t i = 2u * c + half;
                if (i < nch) {
#pragma unroll
                    for (uint32_t j = 0; j < 16; ++j) {
                        const uint32_t v = __builtin_amdgcn_ubfe(x[c][j >> 2], 8u * (j & 3u), 8u);
                        uint32_t add = 1u << (8u * (v & 3u));
                        if (!ALIGNED) add = (16u * i + j - o) < C ? add : 0u;  // a byte of this row
                        atomicAdd(&h[v >> 2], add);
                    }
                }
            }
        }
        // Both lanes of a row have added their bytes before either reads the
        // bins: the wave's LDS operations are performed in order (and the
        // compiler keeps them in program order).
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        uint32_t run = 0, best = 0;
        if constexpr (WB == 4) {
            // px[t]: byte k = values of this half below bin 4t + k (t local);
            // the window of v = 4s + k holds px[s + 4] - px[s]; the upper
            // half's first four prefixes, plus the lower half's total, close
            // the lower half's last four windows; the upper half's close on
            // its own total (bins up to 255).
            uint32_t pxq[4], up[4];
#pragma unroll
            for (uint32_t t = 0; t < 32; ++t) {
                const uint32_t hw = live ? hh[t] : 0u;
                const uint32_t px = (hw << 8) + (hw << 16) + (hw << 24) + splat_byte(run);
                run = __builtin_amdgcn_udot4(hw, 0x01010101u, run, false);
                if (t < 4) up[t] = __shfl_xor(px, kPairRows, kWave);
                if (t >= 4) best = fold_keys(best, px - pxq[t % 4], t - 4);
                pxq[t % 4] = px;
            }
            const uint32_t tail = splat_byte(run);
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) best = fold_keys(best, (half ? 0u : up[k]) + tail - pxq[k], 28u + k);
        } else {
            // W = 2: the window of v holds bins v and v + 1; the lower half's
            // last window takes the upper half's first bin.
            uint32_t prev = 0, first = 0;
#pragma unroll
            for (uint32_t t = 0; t < 32; ++t) {
                const uint32_t hw = live ? hh[t] : 0u;
                if (t == 0) first = __shfl_xor(hw, kPairRows, kWave);
                if (t >= 1) best = fold_keys(best, prev + (prev >> 8) + (hw << 24), t - 1);
                prev = hw;
            }
            const uint32_t nxt = half ? 0u : first;
            best = fold_keys(best, prev + (prev >> 8) + (nxt << 24), 31u);
        }
        // keys of the upper half used 255 - (v - 128)
        uint32_t key = max(best & 0xffffu, best >> 16) - (half ? 128u : 0u);
        key = max(key, (uint32_t)__shfl_xor((int)key, kPairRows, kWave));
        if (live && half == 0) {
            // The keys counted every v, present in the row or not.  The first
            // best v, u, has a value in its window; the smallest such value
            // has a window at least as full (it loses only bins below it,
            // which are empty) and no smaller present value has the best
            // count, so it is the base.  It lies in bins u .. u + W - 1.
            const uint32_t u = 255u - (key & 0xffu);
            constexpr uint32_t NW = WB == 4 ? 5u : 2u;  // bin words that can hold it
            uint32_t base = 256u;
#pragma unroll
            for (uint32_t i = NW; i-- > 0;) {
                const uint32_t w = (u >> 2) + i;
                uint32_t z = w < 64u ? h[w] : 0u;
                if (i == 0) z &= 0xffffffffu << (8u * (u & 3u));  // bins below u
                const uint32_t nz = (((z & 0x7f7f7f7fu) + 0x7f7f7f7fu) | z) & 0x80808080u;
                base = nz ? 4u * w + ((uint32_t)__builtin_ctz(nz) >> 3) : base;
            }
            a.bases[row] = (uint8_t)base;
        }
        if (live) {
#pragma unroll
            for (uint32_t t = 0; t < 32; ++t) hh[t] = 0u;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // bins cleared before the next group's adds
#pragma unroll
        for (uint32_t c = 0; c < CPL; ++c)
#pragma unroll
            for (uint32_t j = 0; j < 4; ++j) x[c][j] = y[c][j];
    }
}

// One wave per index tile (kIndexTile positions = 128 runs of 16); lane l
// takes runs l and l + 64 of the tile, so each load instruction of a wave
// reads 1 KiB of contiguous dense bytes.  Run q holds field q % F of group
// q / F (F = 8 / w runs per group): its 16 values' offsets (0 out of the
// window) at bits w (q % F) of the group's 16 bytes.  The F runs of a group
// are F consecutive lanes; an OR down those lanes gives the group to its
// last lane, which stores it.  The tile's out-of-window count is a sum over
// the wave.
// Offset fields of run h of t (rows of at least 16 columns) at bits w f of
// word[0..3]; returns the run's out-of-window count.
template <bool VEC, bool HIGH>
__device__ __forceinline__ uint32_t pack_run(const EncodeArgs &a, const TileRuns &t, uint32_t h, uint32_t p0,
                                             uint32_t f, uint32_t (&word)[4]) {
    uint32_t d[4], keep[4], valid[4], outside = 0;
    window_test16<VEC, HIGH>(a, t, h, p0, d, keep, valid);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
        // a kept difference is below W: its field is its low w bits
        word[j] = (d[j] & widen80(keep[j])) << (a.wbits * f);
        outside += __popc(valid[j] & ~keep[j]);
    }
    return outside;
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void csf_enc_pack_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x % kWave;
    const uint64_t total_waves = (uint64_t)a.E * a.index_tiles;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock / kWave;
    const uint32_t W = 1u << a.wbits;
    const uint32_t F = 8u / a.wbits, fshift = a.wbits == 4 ? 1u : 3u;  // runs per group: 2 or 8
    const bool long_rows = a.C >= 16u;
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves; wv += stride) {
        TileRuns cur;
        fetch_runs(a, wv, lane, VEC, long_rows, cur);
        const uint32_t e = (uint32_t)wv / a.index_tiles;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        // a base above 256 - W anywhere in the wave needs the borrow check
        const bool high = __ballot(max(max(cur.b0[0], cur.b1[0]), max(cur.b0[1], cur.b1[1])) > 256u - W) != 0;
        uint32_t outside = 0;
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            const uint32_t q = p0 / 16u;  // run in the plane
            const uint32_t f = q & (F - 1u);
            uint32_t word[4] = {0u, 0u, 0u, 0u};
            if (p0 < a.P && long_rows) {
                outside += high ? pack_run<VEC, true>(a, cur, h, p0, f, word) : pack_run<VEC, false>(a, cur, h, p0, f, word);
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
            const uint32_t g = q >> fshift;
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
// 0x80 in each byte of run h of t (rows of at least 16 columns) that lies
// outside its row's window, four bytes per word of out.
template <bool VEC, bool HIGH>
__device__ __forceinline__ void outside_run(const EncodeArgs &a, const TileRuns &t, uint32_t h, uint32_t p0,
                                            uint32_t (&out)[4]) {
    uint32_t d[4], keep[4], valid[4];
    window_test16<VEC, HIGH>(a, t, h, p0, d, keep, valid);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) out[j] = valid[j] & ~keep[j];
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void csf_enc_entries_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x % kWave;
    const uint64_t total_waves = (uint64_t)a.E * a.index_tiles;
    const uint64_t stride = (uint64_t)gridDim.x * kBlock / kWave;
    const uint32_t W = 1u << a.wbits;
    const bool long_rows = a.C >= 16u;
    for (uint64_t wv = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; wv < total_waves; wv += stride) {
        TileRuns cur;
        fetch_runs(a, wv, lane, VEC, long_rows, cur);
        const uint32_t e = (uint32_t)wv / a.index_tiles;
        const uint8_t *brow = a.bases + (uint64_t)e * a.R;
        const bool high = __ballot(max(max(cur.b0[0], cur.b1[0]), max(cur.b0[1], cur.b1[1])) > 256u - W) != 0;
        // outside bytes of each run: bit 8 j + 7 of m[h][j / 8] for byte j
        uint64_t m[2][2] = {{0u, 0u}, {0u, 0u}};
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            uint32_t out[4] = {0u, 0u, 0u, 0u};
            if (p0 < a.P && long_rows) {
                if (high)
                    outside_run<VEC, true>(a, cur, h, p0, out);
                else
                    outside_run<VEC, false>(a, cur, h, p0, out);
            } else if (p0 < a.P) {
                RunBases rb(a, brow, p0);
#pragma unroll
                for (uint32_t j = 0; j < 16; ++j) {
                    const uint32_t p = p0 + j;
                    if (p < a.P) {
                        const uint32_t b = rb.at(a, brow, p);
                        const uint32_t byte = (cur.x[h][j >> 2] >> (8u * (j & 3u))) & 0xffu;
                        if (byte - b >= W) out[j >> 2] |= 0x80u << (8u * (j & 3u));  // below b is outside too
                    }
                }
            }
            m[h][0] = (uint64_t)out[0] | ((uint64_t)out[1] << 32);
            m[h][1] = (uint64_t)out[2] | ((uint64_t)out[3] << 32);
        }
        const uint32_t c0 = (uint32_t)(__popcll(m[0][0]) + __popcll(m[0][1]));
        const uint32_t c1 = (uint32_t)(__popcll(m[1][0]) + __popcll(m[1][1]));
        const uint32_t i0 = wave_inclusive_sum(c0), i1 = wave_inclusive_sum(c1);
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)i0, kWave - 1);
        const uint32_t first = (uint32_t)a.tile_index[wv];
        const uint32_t out0[2] = {first + i0 - c0, first + t0 + i1 - c1};
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t p0 = run_start(a, wv, h, lane);
            uint32_t o = out0[h];
#pragma unroll
            for (uint32_t k = 0; k < 2; ++k) {
                uint64_t mk = m[h][k];
                while (mk != 0u) {
                    const uint32_t j = 8u * k + ((uint32_t)__builtin_ctzll(mk) >> 3);
                    mk &= mk - 1u;
                    const uint32_t w = j < 8u ? (j < 4u ? cur.x[h][0] : cur.x[h][1])
                                              : (j < 12u ? cur.x[h][2] : cur.x[h][3]);
                    a.exc[o++] = ((p0 + j) << 8) | __builtin_amdgcn_ubfe(w, 8u * (j & 3u), 8u);
                }
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
    if (a.C <= 255 && ((uintptr_t)a.dense & 15u) == 0 && n < (1ull << 31)) {
        const bool aligned = a.C % 16 == 0;
        const uint32_t low = std::min<uint32_t>(a.C & (0u - a.C), 16u);
        const uint32_t nch = aligned ? a.C / 16 : (a.C + 31 - low) / 16;
        const uint64_t groups = ((uint64_t)a.E * a.R + kPairRows - 1) / kPairRows;
        grid = (uint32_t)std::min<uint64_t>(groups, (uint64_t)cus * kPairWavesPerCu);
#define CSF_PAIR(WB, CPL, AL) \
    hipLaunchKernelGGL((csf_enc_bases_pair_kernel<WB, CPL, AL>), dim3(grid), dim3(kWave), 0, stream, a)
#define CSF_PAIR_CPL(WB, AL)            \
    if (nch <= 4) CSF_PAIR(WB, 2, AL);       \
    else if (nch <= 8) CSF_PAIR(WB, 4, AL);  \
    else if (nch <= 12) CSF_PAIR(WB, 6, AL); \
    else CSF_PAIR(WB, 9, AL);
        if (a.wbits == 4) {
            if (aligned) { CSF_PAIR_CPL(4, true) } else { CSF_PAIR_CPL(4, false) }
        } else {
            if (aligned) { CSF_PAIR_CPL(1, true) } else { CSF_PAIR_CPL(1, false) }
        }
#undef CSF_PAIR_CPL
#undef CSF_PAIR
    } else {
        grid = grid_for((uint64_t)a.E * a.R, cus);
        hipLaunchKernelGGL(csf_enc_bases_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    grid = grid_for((uint64_t)a.E * a.index_tiles, cus);
    if (runs_aligned(a))
        hipLaunchKernelGGL(csf_enc_pack_kernel<true>, dim3(grid), dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL(csf_enc_pack_kernel<false>, dim3(grid), dim3(kBlock), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(csf_enc_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_encode_entries(const EncodeArgs &a, uint32_t cus, hipStream_t stream) {
    const uint32_t grid = grid_for((uint64_t)a.E * a.index_tiles, cus);
    if (runs_aligned(a))
        hipLaunchKernelGGL(csf_enc_entries_kernel<true>, dim3(grid), dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL(csf_enc_entries_kernel<false>, dim3(grid), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csf
