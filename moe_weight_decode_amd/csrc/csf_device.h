// Device helpers shared by the gfx950 kernels of the CSF library (the decoder
// and the W4A16 consumer): byte arithmetic, buffer resources, row-base
// lookup, tile expansion into LDS and the routing maps.  Internal; every
// definition has internal linkage, so each kernel file gets its own copy.
#pragma once

#include "csf_launch.h"

namespace csf {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t int32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kWave = 64;

// Byte-wise sum modulo 256 of four packed bytes: no carry crosses a byte.
__device__ __forceinline__ uint32_t add_bytes(uint32_t a, uint32_t b) {
    const uint32_t s = (a & 0x7f7f7f7fu) + (b & 0x7f7f7f7fu);
    return s ^ ((a ^ b) & 0x80808080u);
}

__device__ __forceinline__ u32x4 add_bytes4(u32x4 a, u32x4 b) {
    return (u32x4){add_bytes(a.x, b.x), add_bytes(a.y, b.y), add_bytes(a.z, b.z),
                   add_bytes(a.w, b.w)};
}

// Buffer resources: a 128-bit descriptor of a byte range [base, base+bytes).
// A buffer load outside the range returns 0 and a buffer store outside it is
// dropped by the hardware, so the tile loop issues every load and store
// unconditionally: the number of memory operations between a load and its
// use is then fixed, and each wait covers exactly the loads it needs (never
// the stores issued after them).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw byte buffer, 32-bit data format (gfx9 family)
constexpr int kNonTemporal = 2;         // cache policy bit NT (streaming access)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// floor(n / d) for n, d < 2^24 with rcp = 1.0 / d.  (n + 0.5) / d lies at least
// 0.5 / d >= 2^-25 away from an integer while the fp64 error stays below 2^-28.
__device__ __forceinline__ uint32_t div_exact(uint32_t n, double rcp) {
    return (uint32_t)(((double)n + 0.5) * rcp);
}

// Mask of the first k bytes of a 32-bit word, k clamped to [0, 4].
__device__ __forceinline__ uint32_t low_bytes_mask(int k) {
    return k >= 4 ? 0xffffffffu : (k <= 0 ? 0u : ((1u << (8 * k)) - 1u));
}

// Row bases of the 16 positions pos .. pos+15 of one plane, packed like the
// output.  lds holds the bases of rows r_lo, r_lo+1, ... of the current tile.
template <int MODE>
__device__ __forceinline__ u32x4 run_bases(const uint8_t *lds, uint32_t pos, uint32_t r_lo,
                                           uint32_t C, double rcp) {
    const uint32_t r0 = div_exact(pos, rcp);
    const uint32_t s0 = (uint32_t)lds[r0 - r_lo] * 0x01010101u;
    if constexpr (MODE == kRowSplat) {
        return (u32x4){s0, s0, s0, s0};
    } else if constexpr (MODE == kRowTwo) {
        // C >= 16: the run ends inside row r0 or r0 + 1.
        const int left = (int)((r0 + 1) * C - pos);
        if (left >= 16) return (u32x4){s0, s0, s0, s0};
        const uint32_t s1 = (uint32_t)lds[r0 + 1 - r_lo] * 0x01010101u;
        u32x4 out;
        uint32_t m;
        m = low_bytes_mask(left);      out.x = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 4);  out.y = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 8);  out.z = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 12); out.w = (s0 & m) | (s1 & ~m);
        return out;
    } else {
        // C < 16: walk the row boundaries byte by byte.
        uint32_t r = r0;
        uint32_t next = (r0 + 1) * C;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (pos + j == next) {
                ++r;
                next += C;
            }
            w[j >> 2] |= (uint32_t)lds[r - r_lo] << (8 * (j & 3));
        }
        return (u32x4){w[0], w[1], w[2], w[3]};
    }
}

// Store bytes first .. nvalid-1 (nvalid clamped to 16) of the 16-byte run v
// at dst.  Whole, 16-byte aligned runs (every run of an aligned plane whose
// size is a multiple of 16) take one 128-bit store; STREAM marks it
// non-temporal (the decoder never reads its output back).
template <bool STREAM>
__device__ __forceinline__ void store_run(uint8_t *dst, u32x4 v, uint32_t first, uint32_t nvalid) {
    if (first == 0 && nvalid >= 16 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
        if constexpr (STREAM)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
        else
            *reinterpret_cast<u32x4 *>(dst) = v;
        return;
    }
    const uint32_t n = nvalid < 16 ? nvalid : 16;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j)
        if (j >= first && j < n) dst[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
}

// flags[e] = 1 iff expert e has routed tokens, expert_start[e + 1] >
// expert_start[e], for e in [first, E) with stride step; the routing tensor is
// int32 or int64 (the grouped routing comes in both widths).
template <typename T>
__device__ __forceinline__ void stage_flags(const T *es, uint32_t E, uint32_t first, uint32_t step,
                                            uint8_t *flags) {
    for (uint32_t i = first; i < E; i += step) flags[i] = es[i + 1] > es[i] ? 1 : 0;
}

// Wave 0 of the workgroup: list the active experts (flags[e] != 0, or all
// when flags is null) in increasing order into act[];
// for each stack s < ns also the exclusive prefix M_s over the listed experts
// of their entry counts (prefix[e+1] - prefix[e], clamped to [0, n_exc]),
// capped at n_exc.  Returns the number of active experts.  A wave-level
// prefix: ballot + popcount for the positions, a shuffle scan for the counts.
__device__ uint32_t build_maps(const uint8_t *flags, uint32_t E, uint16_t *act, uint32_t ns,
                               const int32_t *pfx0, const int32_t *pfx1, uint32_t n0,
                               uint32_t n1, uint32_t *M0, uint32_t *M1) {
    const uint32_t lane = threadIdx.x;
    uint32_t n = 0;
    uint64_t run0 = 0, run1 = 0;
    if (lane == 0 && ns > 0) {
        M0[0] = 0;
        if (ns > 1) M1[0] = 0;
    }
    for (uint32_t base = 0; base < E; base += kWave) {
        const uint32_t e = base + lane;
        const bool on = e < E && (flags == nullptr || flags[e] != 0);
        const uint64_t mask = __ballot(on);
        const uint32_t slot = n + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
        if (on) act[slot] = (uint16_t)e;
        if (ns > 0) {
            int64_t c0 = on ? (int64_t)pfx0[e + 1] - (int64_t)pfx0[e] : 0;
            c0 = c0 < 0 ? 0 : (c0 > (int64_t)n0 ? (int64_t)n0 : c0);
            uint64_t s0 = (uint64_t)c0;
            int64_t c1 = 0;
            if (ns > 1) {
                c1 = on ? (int64_t)pfx1[e + 1] - (int64_t)pfx1[e] : 0;
                c1 = c1 < 0 ? 0 : (c1 > (int64_t)n1 ? (int64_t)n1 : c1);
            }
            uint64_t s1 = (uint64_t)c1;
#pragma unroll
            for (uint32_t d = 1; d < kWave; d <<= 1) {
                const uint64_t y0 = __shfl_up(s0, d, kWave);
                const uint64_t y1 = __shfl_up(s1, d, kWave);
                if (lane >= d) {
                    s0 += y0;
                    s1 += y1;
                }
            }
            if (on) {
                const uint64_t t0 = run0 + s0;
                M0[slot + 1] = (uint32_t)(t0 < n0 ? t0 : n0);
                if (ns > 1) {
                    const uint64_t t1 = run1 + s1;
                    M1[slot + 1] = (uint32_t)(t1 < n1 ? t1 : n1);
                }
            }
            run0 += __shfl(s0, kWave - 1, kWave);
            run1 += __shfl(s1, kWave - 1, kWave);
        }
        n += (uint32_t)__popcll(mask);
    }
    return n;
}

// Expand this lane's runs of one tile: tile positions q0 .. q1-1, lds_bases
// holding rows from r_lo.  FUSED writes the runs into the LDS tile; otherwise
// positions sb .. q1-1 are stored to the plane directly (sb > q0 only in a
// WINDOW launch, whose row window may start inside the tile).
template <int WB, int MODE, bool FUSED, uint32_t RUNS, bool WINDOW>
__device__ __forceinline__ void expand_tile(const StackArgs &st, const u32x4 *v, uint32_t q0,
                                            uint32_t q1, uint32_t sb, const uint8_t *lds_bases,
                                            uint32_t r_lo, uint8_t *tile, uint8_t *plane) {
    constexpr uint32_t MASK = WB == 4 ? 0x0f0f0f0fu : 0x01010101u;
    constexpr uint32_t FMASK = 8 / WB - 1;  // fields per group - 1
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t j = i * kBlock + threadIdx.x;
        const uint32_t pos = q0 + kRunBytes * j;
        if (pos >= q1) break;
        const uint32_t f = (pos >> 4) & FMASK;
        const u32x4 field = (v[i] >> (uint32_t)(WB * f)) & MASK;
        const u32x4 out = add_bytes4(field, run_bases<MODE>(lds_bases, pos, r_lo, st.C, st.rcp_cols));
        if constexpr (FUSED) {
            *reinterpret_cast<u32x4 *>(tile + kRunBytes * j) = out;
        } else {
            if constexpr (WINDOW) {
                if (pos + kRunBytes > sb)
                    store_run<false>(plane + pos, out, sb > pos ? sb - pos : 0u, q1 - pos);
            } else {
                store_run<false>(plane + pos, out, 0u, q1 - pos);
            }
        }
    }
}

template <bool FUSED, uint32_t RUNS, bool WINDOW>
__device__ __forceinline__ void expand_dispatch(const StackArgs &st, const u32x4 *v, uint32_t q0,
                                                uint32_t q1, uint32_t sb, const uint8_t *lds_bases,
                                                uint32_t r_lo, uint8_t *tile, uint8_t *plane) {
    switch ((st.wbits == 4 ? 0u : 3u) + st.row_mode) {
        case 0: expand_tile<4, kRowSplat, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
        case 1: expand_tile<4, kRowTwo, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
        case 2: expand_tile<4, kRowBytes, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
        case 3: expand_tile<1, kRowSplat, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
        case 4: expand_tile<1, kRowTwo, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
        default: expand_tile<1, kRowBytes, FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane); break;
    }
}

}  // namespace
}  // namespace csf
