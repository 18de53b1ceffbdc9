// Device helpers shared by the gfx950 kernels of the CSF library (the decoder
// and the W4A16 consumer): byte arithmetic, buffer resources, row-base
// lookup, tile expansion into LDS and the list of routed experts.  Internal; every
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

// Set bits of m below this lane.
__device__ __forceinline__ uint32_t bits_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr uint32_t kListChunks = 8;  // 64-expert chunks of routing read per round trip

// Wave 0 of the workgroup lists the experts with routed tokens (expert e has
// them iff es[e + 1] > es[e]; every expert when es is null) in increasing
// order into act[] and returns their number.  The routing of CH chunks of 64
// experts is read in one round trip (kListChunks chunks, fewer in a kernel
// whose registers are tight): each lane loads two neighbouring values per
// chunk, at addresses clamped into the tensor; a ballot per chunk gives each
// listed expert its slot.  The routing is int32 or int64 (the grouped routing
// comes in both widths), in global memory or in LDS.
template <uint32_t CH = kListChunks, typename T>
__device__ __forceinline__ uint32_t list_experts(const T *es, uint32_t E, uint16_t *act) {
    const uint32_t lane = threadIdx.x;
    uint32_t n = 0;
    for (uint32_t base = 0; base < E; base += kWave * CH) {
        bool on[CH];
        if (es != nullptr) {
            T lo[CH], hi[CH];
#pragma unroll
            for (uint32_t u = 0; u < CH; ++u) {
                const uint32_t e = min(base + kWave * u + lane, E - 1u);
                lo[u] = es[e];
                hi[u] = es[e + 1];
            }
#pragma unroll
            for (uint32_t u = 0; u < CH; ++u) on[u] = base + kWave * u + lane < E && hi[u] > lo[u];
        } else {
#pragma unroll
            for (uint32_t u = 0; u < CH; ++u) on[u] = base + kWave * u + lane < E;
        }
#pragma unroll
        for (uint32_t u = 0; u < CH; ++u) {
            const uint64_t mask = __ballot(on[u]);
            if (on[u]) act[n + bits_below(mask)] = (uint16_t)(base + kWave * u + lane);
            n += (uint32_t)__popcll(mask);
        }
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
