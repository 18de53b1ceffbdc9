// CSF block-scale decode kernels for gfx950 (CDNA4, wave64).
//
// The decoder on "finegrained-kernels: decode losslessly compressed NVFP4
// scales (CSF)" (kernels-community PR 1236, API paragraph) is a fixed stream
// that writes base + offset for every position plus an exception pass that
// writes the bytes the offsets cannot reach.  With the grouped-routing
// expert_start tensor both skip experts with no routed tokens and never address
// their planes; the routing is read on the device only.  Every launch covers
// one or two stacks (gate/up + down, "NVFP4-CSF: expand_scales() for
// ahead-of-call scale expansion (canonical twin of #477)", b12x PR 478, commit
// messages).
//
// Four kernels:
//   csf_fused_kernel  both parts in one pass: a tile is expanded into LDS, the
//                     tile's exception entries (found through the per-tile
//                     exception index) are patched into LDS, then the tile is
//                     written with full-line stores.  Every dense byte is
//                     written once.
//   csf_routed_kernel the same pass for routed calls, one tile per workgroup,
//                     its routing inputs passed ahead of the argument block.
//   csf_fixed_kernel  the fixed stream alone, stored straight from registers.
//   csf_exc_kernel    the exception pass alone, indexed by a wave-level prefix
//                     over per-expert entry counts (needs no tile index).
//
// The work is a byte expansion bound by HBM bandwidth: no matrix cores, a few
// integer ops per output byte.  Lane l of a workgroup owns the 16-byte output
// runs l, l + 256, ... of a tile, so every store instruction of a wave covers
// 1 KiB of contiguous output.  A tile is 4096, 8192 or 16384 positions (1, 2
// or 4 runs per lane); the host picks one per launch.
#include "csf_device.h"

namespace csf {
namespace {

__device__ __forceinline__ StackArgs pick(const DecodeArgs &a, uint32_t s) {
    return s ? a.st[1] : a.st[0];
}

// Routed mode: the active-expert list in LDS, written by wave 0 straight from
// the routing and shared by a barrier.  Two chunks of 64 experts per round
// trip keep the tile loops' register budgets.
__device__ uint32_t active_experts(const DecodeArgs &a, uint16_t *act) {
    __shared__ uint32_t s_nact;
    if (threadIdx.x < kWave) {
        const uint32_t n = a.es_wide ? list_experts<2>(static_cast<const int64_t *>(a.expert_start), a.E, act)
                                     : list_experts<2>(static_cast<const int32_t *>(a.expert_start), a.E, act);
        if (threadIdx.x == 0) s_nact = n;
    }
    __syncthreads();
    return s_nact;
}

// Work unit u of a launch: stack s, expert e, tile t of e's plane (tiles are
// counted from the plane's start; a decode covers tiles tile0 .. tile0 +
// tiles - 1 of every plane).  Units run over stack 0's active experts'
// tiles, then stack 1's.
struct Unit {
    uint32_t s, e, t;
};

template <bool UNIFORM>
__device__ __forceinline__ Unit locate(const DecodeArgs &a, uint32_t u, uint32_t u0,
                                       const uint16_t *act, bool routed) {
    const uint32_t s = u >= u0 ? 1u : 0u;
    const uint32_t uu = u - (s ? u0 : 0u);
    const uint32_t tiles = s ? a.st[1].tiles : a.st[0].tiles;
    const uint32_t k = uu / tiles;
    uint32_t e = k;
    if (routed) e = UNIFORM ? (uint32_t)__builtin_amdgcn_readfirstlane(act[k]) : (uint32_t)act[k];
    return {s, e, (s ? a.st[1].tile0 : a.st[0].tile0) + uu - k * tiles};
}

// ---------------------------------------------------------------------------
// Serial tile loop (the fixed-stream kernel, and the fused kernel on dense
// exception streams).
//
// Work unit = (stack, active expert, tile of TILE = 4096 * RUNS positions);
// workgroups take units grid-stride, so the units in flight at any moment
// are neighbours in memory.  Per tile the workgroup loads each lane's 16-byte
// offset groups with 128-bit loads (lanes reading fields of the same group
// share one load), the tile's index bounds and then its first EXC * kBlock
// exception entries, and its row bases into LDS; it widens each lane's field
// to 16 bytes and adds the row bases byte-wise.  FUSED then patches the
// tile's entries into the LDS tile and stores the finished tile with
// non-temporal stores; otherwise the runs are stored straight from
// registers.  OFFSET_NT / ENTRY_NT mark the offset / entry loads
// non-temporal.
// ---------------------------------------------------------------------------
template <bool FUSED, uint32_t RUNS, uint32_t EXC, bool OFFSET_NT, bool ENTRY_NT, bool WINDOW>
__device__ __forceinline__ void tile_loop_serial(const DecodeArgs &a, uint8_t *dyn, uint8_t *tile) {
    constexpr uint32_t TILE = tile_positions(RUNS);
    constexpr uint32_t INDEX_PER_TILE = TILE / kIndexTile;
    uint8_t *lds_bases = dyn;
    uint16_t *act = reinterpret_cast<uint16_t *>(dyn + a.bases_stage);

    const bool routed = a.expert_start != nullptr;
    const uint32_t nact = routed ? active_experts(a, act) : a.E;
    const uint32_t u0 = nact * a.st[0].tiles;
    const uint32_t total = u0 + (a.nstacks > 1 ? nact * a.st[1].tiles : 0u);

    for (uint32_t u = blockIdx.x; u < total; u += gridDim.x) {
        const uint32_t s = u >= u0 ? 1u : 0u;
        const StackArgs st = pick(a, s);
        const uint32_t uu = u - (s ? u0 : 0u);
        const uint32_t k = uu / st.tiles;
        const uint32_t t = st.tile0 + uu - k * st.tiles;
        const uint32_t e = routed ? (uint32_t)act[k] : k;
        const uint32_t q0 = t * TILE;
        const uint32_t q1 = min(q0 + TILE, st.pend);
        const uint32_t sb = WINDOW ? max(q0, st.pbeg) : q0;  // first position stored

        // Offset groups: run q (positions 16q .. 16q+15) is field q % F of
        // group q / F, F = 8 / w fields per group.
        const u32x4 *seg = reinterpret_cast<const u32x4 *>(st.offsets + (uint64_t)e * st.stride);
        const uint32_t gshift = st.wbits == 4 ? 1u : 3u;
        u32x4 v[RUNS];
#pragma unroll
        for (uint32_t i = 0; i < RUNS; ++i) {
            const uint32_t pos = q0 + kRunBytes * (i * kBlock + threadIdx.x);
            const u32x4 *src = seg + ((pos >> 4) >> gshift);
            if (pos >= q1)
                v[i] = (u32x4){0u, 0u, 0u, 0u};
            else if constexpr (OFFSET_NT)
                v[i] = __builtin_nontemporal_load(src);
            else
                v[i] = *src;
        }

        // The tile's exception entries, prefetched into registers.
        uint32_t lo = 0, hi = 0;
        uint32_t w[EXC];
        if constexpr (FUSED) {
            const int32_t *ti = st.tile_index + (uint64_t)e * st.index_tiles + t * INDEX_PER_TILE;
            const uint32_t last = min(INDEX_PER_TILE, st.index_tiles - t * INDEX_PER_TILE);
            const int32_t l0 = ti[0], h0 = ti[last];
            hi = h0 < 0 ? 0u : min((uint32_t)h0, st.n_exc);
            lo = l0 < 0 ? 0u : min((uint32_t)l0, hi);
#pragma unroll
            for (uint32_t i = 0; i < EXC; ++i) {
                const uint32_t kk = lo + i * kBlock + threadIdx.x;
                if (kk >= hi)
                    w[i] = 0xffffffffu;  // position 2^24 - 1: never in a tile
                else if constexpr (ENTRY_NT)
                    w[i] = __builtin_nontemporal_load(st.exc + kk);
                else
                    w[i] = st.exc[kk];
            }
        }

        // Row bases of the tile into LDS.
        const uint32_t r_lo = div_exact(q0, st.rcp_cols);
        const uint32_t nrows = div_exact(q1 - 1u, st.rcp_cols) - r_lo + 1u;
        if (!FUSED && u != blockIdx.x) __syncthreads();  // previous tile done with lds_bases
        const uint8_t *brow = st.bases + (uint64_t)e * st.R + r_lo;
        for (uint32_t r = threadIdx.x; r < nrows; r += kBlock) lds_bases[r] = brow[r];
        __syncthreads();

        uint8_t *plane = st.ws + (uint64_t)e * st.P;
        expand_dispatch<FUSED, RUNS, WINDOW>(st, v, q0, q1, sb, lds_bases, r_lo, tile, plane);

        if constexpr (FUSED) {
            __syncthreads();  // tile expanded
#pragma unroll
            for (uint32_t i = 0; i < EXC; ++i) {
                const uint32_t pos = w[i] >> 8;
                if (pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(w[i] & 0xffu);
            }
            for (uint32_t kk = lo + EXC * kBlock + threadIdx.x; kk < hi; kk += kBlock) {
                const uint32_t x = st.exc[kk];
                const uint32_t pos = x >> 8;
                if (pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(x & 0xffu);
            }
            __syncthreads();  // tile patched
#pragma unroll
            for (uint32_t i = 0; i < RUNS; ++i) {
                const uint32_t j = i * kBlock + threadIdx.x;
                const uint32_t pos = q0 + kRunBytes * j;
                if (pos >= q1) break;
                const u32x4 out = *reinterpret_cast<const u32x4 *>(tile + kRunBytes * j);
                if constexpr (WINDOW) {
                    if (pos + kRunBytes > sb)
                        store_run<true>(plane + pos, out, sb > pos ? sb - pos : 0u, q1 - pos);
                } else {
                    store_run<true>(plane + pos, out, 0u, q1 - pos);
                }
            }
            // The next tile's first barrier orders these LDS reads before the
            // next expansion overwrites the tile.
        }
    }
}

// Load schedule of the fused kernel (the host picks one per call).
//   kPipelined      pipelined loop, cached loads (stacks with few exceptions)
//   kStreamEntries  serial loop, non-temporal entry loads (dense exception
//                   streams)
//   kRouted         routed decodes: at most one tile per workgroup, its
//                   loads issued in one round trip after the routing's
//                   (routed_decode); more tiles than workgroups take the
//                   pipelined loop.  Offset and entry loads are
//                   non-temporal: routed planes are read once and are
//                   rarely cache-resident.
// Which loop suits which stream was measured on MI355X: on dense exception
// streams the serial loop with non-temporal entries is the fastest.
enum Sched : uint32_t {
    kPipelined = kSchedPipelined,
    kStreamEntries = kSchedStreamEntries,
    kRouted = kSchedRouted
};

// Everything a tile needs from memory, loaded ahead of its decode: the
// lane's offset groups, two row bases, EXC exception entries (slot i holds
// entry entry_of(first, i)) and the tile's entry range [lo, hi).
template <uint32_t RUNS, uint32_t EXC>
struct TileLoads {
    u32x4 v[RUNS];
    uint32_t w[EXC];
    uint8_t b0, b1;
    uint32_t lo, hi, first;
};

// Stream index of slot i of a lane's prefetched entries: each 16-byte load
// of a workgroup covers 4 * kBlock consecutive entries.
__device__ __forceinline__ uint32_t entry_of(uint32_t first, uint32_t i) {
    return first + 4u * ((i / 4u) * kBlock + threadIdx.x) + (i % 4u);
}

// Issue the loads of unit w (tile positions from q0); its tile index bounds
// are lane j of the batch registers blo/bhi, read only after the offset and
// base loads are issued, so only the entry loads wait for a batch still in
// flight.  Every load is issued, whatever the tile holds: loads past the
// expert's offset segment or bases, or past the tile's entries, read 0.
template <uint32_t RUNS, uint32_t EXC, int POLICY>
__device__ __forceinline__ void issue_loads(const StackArgs &st, const Unit &w, uint32_t q0,
                                            int32_t blo, int32_t bhi, uint32_t j, TileLoads<RUNS, EXC> &L) {
    // Offset groups: run q (positions 16q .. 16q+15) is field q % F of
    // group q / F, F = 8 / w fields per group.
    const rsrc_t seg = make_rsrc(st.offsets + (uint64_t)w.e * st.stride, (uint32_t)st.stride);
    const uint32_t gshift = st.wbits == 4 ? 1u : 3u;
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t run = (q0 >> 4) + i * kBlock + threadIdx.x;
        L.v[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(seg, (int)((run >> gshift) << 4), 0, POLICY));
    }
    // Row bases of the tile's first 2 * kBlock rows; the resource covers the
    // tile's rows only, so lanes past them read nothing from memory.
    const uint32_t r_lo = __builtin_amdgcn_readfirstlane(div_exact(q0, st.rcp_cols));
    const uint32_t r_hi =
        __builtin_amdgcn_readfirstlane(div_exact(min(q0 + tile_positions(RUNS), st.pend) - 1u, st.rcp_cols) + 1u);
    const rsrc_t rb = make_rsrc(st.bases + (uint64_t)w.e * st.R + r_lo, r_hi - r_lo);
    L.b0 = __builtin_amdgcn_raw_buffer_load_b8(rb, (int)threadIdx.x, 0, 0);
    L.b1 = __builtin_amdgcn_raw_buffer_load_b8(rb, (int)(kBlock + threadIdx.x), 0, 0);
    // the unit's tile-index bounds (lane j of the batch): only the entry loads
    // below wait for them
    __builtin_amdgcn_sched_barrier(0);
    const int32_t l0 = __builtin_amdgcn_readlane(blo, j), h0 = __builtin_amdgcn_readlane(bhi, j);
    // Entries from `first` (lo rounded down to a multiple of 4) in 16-byte
    // loads; the resource ends at hi.
    L.hi = h0 < 0 ? 0u : min((uint32_t)h0, st.n_exc);
    L.lo = l0 < 0 ? 0u : min((uint32_t)l0, L.hi);
    L.first = L.lo & ~3u;
    const rsrc_t rx = make_rsrc(st.exc + L.first, 4u * (L.hi - L.first));
#pragma unroll
    for (uint32_t i = 0; i < EXC / 4; ++i) {
        const u32x4 q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(16u * (i * kBlock + threadIdx.x)), 0,
                                                         POLICY));
        L.w[4 * i] = q.x;
        L.w[4 * i + 1] = q.y;
        L.w[4 * i + 2] = q.z;
        L.w[4 * i + 3] = q.w;
    }
}

// Store tile bytes s0 .. n-1 of the LDS tile to plane positions q0 .. q1-1
// (s0 > 0 only where a row window starts inside the tile).  Whole 16-byte
// runs of an aligned tile from the first run boundary at or after s0,
// h .. wend-1, take one non-temporal 128-bit store each, issued for every
// run: the resource starts at h, so runs before it have offsets that wrap
// past the resource and runs past wend lie beyond it; the hardware drops
// both.  A ragged window edge or a misaligned workspace leaves bytes for the
// byte loop.
template <uint32_t RUNS, bool WINDOW>
__device__ __forceinline__ void store_tile(const StackArgs &st, uint8_t *plane, uint32_t q0, uint32_t q1,
                                           const uint8_t *tile) {
    uint8_t *dst = plane + q0;
    const uint32_t n = q1 - q0;
    const uint32_t s0 = WINDOW && st.pbeg > q0 ? st.pbeg - q0 : 0u;
    const bool aligned = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    const uint32_t h = aligned ? (WINDOW ? min((s0 + 15u) & ~15u, n) : 0u) : n;
    const uint32_t wend = max(h, n & ~15u);
    const rsrc_t rw = make_rsrc(dst + h, wend - h);
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t off = kRunBytes * (i * kBlock + threadIdx.x);
        const u32x4 out = *reinterpret_cast<const u32x4 *>(tile + off);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int32x4_t, out), rw, (int)(off - h), 0,
                                               kNonTemporal);
    }
    if (WINDOW || !aligned) [[unlikely]]
        for (uint32_t b = s0 + threadIdx.x; b < h; b += kBlock) dst[b] = tile[b];
    if (wend < n) [[unlikely]]
        for (uint32_t b = wend + threadIdx.x; b < n; b += kBlock) dst[b] = tile[b];
}

// Row bases of a tile's rows into LDS: the first 2 * kBlock from the loaded
// bytes b0 / b1, any further rows from memory.
__device__ __forceinline__ void stage_bases(const StackArgs &st, uint32_t e, uint32_t r_lo, uint32_t nrows,
                                            uint8_t b0, uint8_t b1, uint8_t *lds_bases) {
    if (threadIdx.x < nrows) lds_bases[threadIdx.x] = b0;
    if (threadIdx.x + kBlock < nrows) lds_bases[threadIdx.x + kBlock] = b1;
    const uint8_t *brow = st.bases + (uint64_t)e * st.R + r_lo;
    for (uint32_t r = threadIdx.x + 2u * kBlock; r < nrows; r += kBlock) lds_bases[r] = brow[r];
}

// ---------------------------------------------------------------------------
// Pipelined tile loop of the fused kernel.
//
// Work unit = (stack, active expert, tile of TILE = 4096 * RUNS positions);
// workgroups take units grid-stride, so the units in flight at any moment
// are neighbours in memory.  A tile's loads are its lanes' 16-byte offset
// groups (128-bit loads; lanes reading fields of the same group share one
// load), its row bases and its first EXC * kBlock exception entries.  The
// entry ranges come from the tile index, read for 64 units at a time (lane j
// of every wave holds unit j's range), so no load of a tile waits on another
// load.  Per tile the workgroup stages the row bases in LDS, widens each
// lane's field to 16 bytes and adds the row bases byte-wise into an LDS tile,
// patches the tile's entries into it and stores the finished tile with
// non-temporal stores.  The next tile's loads go out before this tile's
// stores, so no wait on a tile's data also waits for the stores before it.
// POLICY is the cache policy of the offset and entry loads.  Routed launches
// pass their nact active experts in act[] (routed), others every expert.
// ---------------------------------------------------------------------------
template <uint32_t RUNS, uint32_t EXC, int POLICY, bool WINDOW>
__device__ __forceinline__ void tile_loop_pipelined(const DecodeArgs &a, uint8_t *lds_bases, uint8_t *tile,
                                                    uint32_t nact, const uint16_t *act, bool routed) {
    constexpr uint32_t TILE = tile_positions(RUNS);
    constexpr uint32_t INDEX_PER_TILE = TILE / kIndexTile;
    static_assert(EXC % 4 == 0, "entries are prefetched in 16-byte loads");

    const uint32_t u0 = nact * a.st[0].tiles;
    const uint32_t total = u0 + (a.nstacks > 1 ? nact * a.st[1].tiles : 0u);
    if (blockIdx.x >= total) return;
    const uint32_t G = gridDim.x;
    const uint32_t lane = threadIdx.x & (kWave - 1u);

    // Tile index bounds of units ub + j*G, j < 64, in lane j.
    int32_t blo = 0, bhi = 0;
    auto load_batch = [&](uint32_t ub) {
        const uint32_t uj = ub + lane * G;
        if (uj < total) {
            const Unit w = locate<false>(a, uj, u0, act, routed);
            const StackArgs &st = w.s ? a.st[1] : a.st[0];
            const int32_t *ti = st.tile_index + (uint64_t)w.e * st.index_tiles + w.t * INDEX_PER_TILE;
            blo = ti[0];
            bhi = ti[min(INDEX_PER_TILE, st.index_tiles - w.t * INDEX_PER_TILE)];
        }
    };

    uint32_t u = blockIdx.x;
    uint32_t j = 0;
    load_batch(u);
    Unit cur = locate<true>(a, u, u0, act, routed);
    TileLoads<RUNS, EXC> L;
    {
        const StackArgs st = pick(a, cur.s);
        issue_loads<RUNS, EXC, POLICY>(st, cur, cur.t * TILE, blo, bhi, 0u, L);
        // As many stores as a tile's store phase, into an empty range (the
        // hardware drops them): the loop is then entered with the same memory
        // operations in flight from here as from its own end, and its waits
        // need not cover the previous tile's stores.
        const rsrc_t none = make_rsrc(st.ws, 0u);
#pragma unroll
        for (uint32_t i = 0; i < RUNS; ++i)
            __builtin_amdgcn_raw_buffer_store_b128((int32x4_t){0, 0, 0, 0}, none,
                                                   (int)(kRunBytes * (i * kBlock + threadIdx.x)), 0,
                                                   kNonTemporal);
    }
    while (true) {
        const StackArgs st = pick(a, cur.s);
        const uint32_t e = cur.e;
        const uint32_t q0 = cur.t * TILE;
        const uint32_t q1 = min(q0 + TILE, st.pend);
        const uint32_t r_lo = div_exact(q0, st.rcp_cols);
        const uint32_t nrows = div_exact(q1 - 1u, st.rcp_cols) - r_lo + 1u;

        // Row bases into LDS (the barrier also ends the previous tile's LDS reads).
        stage_bases(st, e, r_lo, nrows, L.b0, L.b1, lds_bases);
        __syncthreads();

        uint8_t *plane = st.ws + (uint64_t)e * st.P;
        expand_dispatch<true, RUNS, false>(st, L.v, q0, q1, q0, lds_bases, r_lo, tile, plane);
        __syncthreads();  // tile expanded

#pragma unroll
        for (uint32_t i = 0; i < EXC; ++i) {
            const uint32_t k = entry_of(L.first, i);
            const uint32_t pos = L.w[i] >> 8;
            if (k >= L.lo && k < L.hi && pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(L.w[i] & 0xffu);
        }
        for (uint32_t kk = L.first + EXC * kBlock + threadIdx.x; kk < L.hi; kk += kBlock) {
            const uint32_t x = st.exc[kk];
            const uint32_t pos = x >> 8;
            if (pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(x & 0xffu);
        }
        __syncthreads();  // tile patched

        const uint32_t un = u + G;
        const bool more = un < total;
        if (more) {
            // Each branch reads its bounds itself, so no later wait covers the
            // batch load.
            if (++j == kWave) {
                load_batch(un);
                j = 0;
            }
            cur = locate<true>(a, un, u0, act, routed);
            // The next unit's loads go out before this tile's stores.
            issue_loads<RUNS, EXC, POLICY>(pick(a, cur.s), cur, cur.t * TILE, blo, bhi, j, L);
        }
        store_tile<RUNS, WINDOW>(st, plane, q0, q1, tile);
        // The next tile's first barrier orders these LDS reads before the
        // next expansion overwrites the tile.
        if (!more) break;
        u = un;
    }
}

// ---------------------------------------------------------------------------
// Routed decode (kRouted).
//
// Every wave reads expert_start on its own with 16-byte loads: lane l of
// chunk i holds the V = 16 / sizeof(T) values from 64 V i + V l (and, by one
// more load, the value after them), so the active flags of 64 V experts take
// one load per lane plus one, and V ballots hold them in scalar registers
// (no LDS, no barrier).  When the launch has a workgroup for every unit
// (stack, active expert, tile), workgroup b takes unit b: the workgroup's
// expert is the k-th active one, found from the ballots with per-lane bit
// counts.  Its tile then costs two more round trips: the offset groups, the
// row bases each lane's 16-byte run touches (read into registers) and the
// tile-index bounds, then the tile's exception entries.  More units than
// workgroups, or more experts, take the pipelined loop.  The routing's inputs
// and the grid come as leading kernel arguments that the hardware preloads
// into scalar registers, so the routing read is the first memory access.
// Most workgroups of a routed call are the first on their CU and fetch the
// kernel's code cold, so the common path is kept short and straight: int64
// routing is its own instantiation, and rows of fewer than 16 columns and
// tiles with more entries than the registers prefetch branch off it.
// STAMP records s_memrealtime values per workgroup in a.stamps (phases in
// csf_decode_traced's documentation).
// ---------------------------------------------------------------------------
constexpr uint32_t kFastExperts = 512;

// Position of the k-th set bit (k < popcount) of w.
__device__ __forceinline__ uint32_t nth_set_bit(uint64_t w, uint32_t k) {
    uint32_t pos = 0;
#pragma unroll
    for (uint32_t s = 32; s >= 1; s >>= 1) {
        const uint32_t c = (uint32_t)__popcll(w & ((1ull << s) - 1ull));
        if (k >= c) {
            k -= c;
            w >>= s;
            pos += s;
        }
    }
    return pos;
}

// The routed unit of this workgroup.
struct RoutedUnit {
    uint32_t total;    // units of the launch
    uint32_t s, e, t;  // this workgroup's unit (when blockIdx.x < total <= gridDim.x)
};

// The routing's inputs, passed to the routed kernel as leading scalar
// arguments: the hardware loads those into scalar registers when it launches
// a wave (kernel-argument preloading), so the routing read is issued without
// first waiting for a load of the argument block.
struct RouteHead {
    const void *expert_start;
    uint32_t E;
    uint32_t flags;            // kHeadPair: two stacks
    uint32_t tiles[2], first[2];  // per stack: tiles decoded per plane, first tile
    uint32_t grid;             // workgroups of the launch
};
constexpr uint32_t kHeadPair = 2;

template <typename T>
__device__ __forceinline__ RoutedUnit route_unit(const RouteHead &h, const T *es) {
    constexpr uint32_t V = 16 / sizeof(T);                 // experts per lane per chunk
    constexpr uint32_t CH = kFastExperts / (kWave * V);    // chunks at most
    typedef T tv __attribute__((ext_vector_type(V)));
    const uint32_t E = h.E, lane = threadIdx.x % kWave;
    // Loads are issued unconditionally, at addresses clamped into the tensor,
    // so none waits for another; lanes and chunks past E are masked below.
    // Whole 16-byte loads when they cannot run past the tensor.
    const bool vec = (reinterpret_cast<uintptr_t>(es) & 15u) == 0 && E % V == 0;
    T x[CH][V], nxt[CH];
    if (vec) [[likely]] {
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            const uint32_t b = kWave * V * i + V * lane;  // first expert of this lane
            const tv q = *reinterpret_cast<const tv *>(es + min(b, E - V));
#pragma unroll
            for (uint32_t c = 0; c < V; ++c) x[i][c] = q[c];
            nxt[i] = es[min(b + V, E)];
        }
    } else [[unlikely]] {
#pragma unroll
        for (uint32_t i = 0; i < CH; ++i) {
            const uint32_t b = kWave * V * i + V * lane;
#pragma unroll
            for (uint32_t c = 0; c < V; ++c) x[i][c] = es[min(b + c, E)];
            nxt[i] = es[min(b + V, E)];
        }
    }
    // f[i]: bit c = expert 64 V i + V lane + c has tokens; ballots per c.
    uint32_t f[CH];
    uint64_t m[CH][V];
    uint32_t nact = 0;
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        const uint32_t b = kWave * V * i + V * lane;
        f[i] = 0;
#pragma unroll
        for (uint32_t c = 0; c < V; ++c) {
            const T after = c + 1 < V ? x[i][c + 1 < V ? c + 1 : 0] : nxt[i];
            const bool on = b + c < E && after > x[i][c];
            f[i] |= on ? 1u << c : 0u;
            m[i][c] = __ballot(on);
            nact += (uint32_t)__popcll(m[i][c]);
        }
    }
    RoutedUnit r;
    const uint32_t u0 = nact * h.tiles[0];
    r.total = u0 + ((h.flags & kHeadPair) ? nact * h.tiles[1] : 0u);
    r.s = r.e = r.t = 0;
    const uint32_t u = blockIdx.x;
    if (u >= r.total || r.total > h.grid) return r;
    r.s = u >= u0 ? 1u : 0u;
    const uint32_t tiles = h.tiles[r.s];
    const uint32_t uu = u - (r.s ? u0 : 0u);
    uint32_t k = uu / tiles;
    r.t = h.first[r.s] + uu - k * tiles;
    // The k-th active expert: its chunk, then its lane (the lane whose bits
    // below it in the chunk count at most k), then its bit.
    uint32_t e = 0;
#pragma unroll
    for (uint32_t i = 0; i < CH; ++i) {
        uint32_t cnt = 0, below = 0;
#pragma unroll
        for (uint32_t c = 0; c < V; ++c) {
            cnt += (uint32_t)__popcll(m[i][c]);
            below += bits_below(m[i][c]);
        }
        if (k < cnt) {
            const uint32_t own = (uint32_t)__popc(f[i]);
            const uint64_t hit = __ballot(below <= k && k < below + own);
            const uint32_t L = (uint32_t)__builtin_ctzll(hit);
            const uint32_t fl = __builtin_amdgcn_readlane(f[i], (int)L);
            const uint32_t bl = __builtin_amdgcn_readlane(below, (int)L);
            e = kWave * V * i + V * L + nth_set_bit(fl, k - bl);
            k = ~0u >> 1;  // found: no later chunk matches
        } else {
            k -= cnt;
        }
    }
    r.e = __builtin_amdgcn_readfirstlane(e);
    return r;
}

template <bool STAMP>
struct Clock {
    uint64_t t[kStampsPerGroup];
    __device__ __forceinline__ Clock() {
        if constexpr (STAMP)
            for (uint32_t i = 0; i < kStampsPerGroup; ++i) t[i] = 0;
    }
    __device__ __forceinline__ void mark(uint32_t i) {
        if constexpr (STAMP) t[i] = __builtin_amdgcn_s_memrealtime();
    }
    // Wait for every memory operation of the thread, then mark.
    __device__ __forceinline__ void mark_drained(uint32_t i) {
        if constexpr (STAMP) {
            __builtin_amdgcn_s_waitcnt(0);
            t[i] = __builtin_amdgcn_s_memrealtime();
        }
    }
    __device__ __forceinline__ void write(const DecodeArgs &a, uint64_t tag) {
        if constexpr (STAMP) {
            if (threadIdx.x == 0) {
                t[kStampsPerGroup - 1] = tag;
                uint64_t *dst = a.stamps + (uint64_t)blockIdx.x * kStampsPerGroup;
#pragma unroll
                for (uint32_t i = 0; i < kStampsPerGroup; ++i) dst[i] = t[i];
            }
        }
    }
};

// One lane's run of a routed tile, widened and based from the row bases s0
// (row r0 = pos / C) and s1 (row r0 + 1), both splat over four bytes; w
// offset bits per field (4 or 1).  One code path for both formats and row
// kinds (a run of a stack whose C is a multiple of 16 never crosses a row,
// so the blend below never applies there): the routed kernel keeps its code
// short, since most of its workgroups run it once on a cold instruction cache.
__device__ __forceinline__ u32x4 expand_run(u32x4 v, uint32_t pos, uint32_t r0, uint32_t C, uint32_t s0,
                                            uint32_t s1, uint32_t w) {
    const uint32_t mask = w == 4 ? 0x0f0f0f0fu : 0x01010101u;
    const uint32_t f = (pos >> 4) & (w == 4 ? 1u : 7u);  // field of the run within its group
    const u32x4 field = (v >> (w * f)) & mask;
    u32x4 b = {s0, s0, s0, s0};
    const int left = (int)((r0 + 1) * C - pos);
    if (left < 16) {
        uint32_t m;
        m = low_bytes_mask(left);      b.x = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 4);  b.y = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 8);  b.z = (s0 & m) | (s1 & ~m);
        m = low_bytes_mask(left - 12); b.w = (s0 & m) | (s1 & ~m);
    }
    return add_bytes4(field, b);
}

template <uint32_t RUNS, uint32_t EXC, bool WINDOW, bool STAMP, bool WIDE>
__device__ __forceinline__ void routed_decode(const RouteHead &h, const DecodeArgs &a, uint8_t *dyn,
                                              uint8_t *tile) {
    constexpr uint32_t TILE = tile_positions(RUNS);
    constexpr uint32_t INDEX_PER_TILE = TILE / kIndexTile;
    static_assert(EXC % 4 == 0, "entries are read in 16-byte loads");
    Clock<STAMP> clk;
    clk.mark(0);
    uint8_t *lds_bases = dyn;

    // (route_unit reads only inside the tensor, so it runs before the expert
    // count is checked; its loads need only the preloaded leading arguments.)
    const RoutedUnit ru = route_unit(h, static_cast<const std::conditional_t<WIDE, int64_t, int32_t> *>(h.expert_start));
    const bool fast = h.E <= kFastExperts;
    clk.mark(1);
    if (!fast || ru.total > h.grid) [[unlikely]] {
        uint16_t *act = reinterpret_cast<uint16_t *>(dyn + a.bases_stage);
        const uint32_t nact = active_experts(a, act);
        tile_loop_pipelined<RUNS, EXC, kNonTemporal, WINDOW>(a, lds_bases, tile, nact, act, true);
        clk.write(a, ~0ull);
        return;
    }
    if (blockIdx.x >= ru.total) {
        clk.write(a, 0ull);
        return;
    }

    const uint32_t u = blockIdx.x;
    const uint32_t s = ru.s, e = ru.e, t = ru.t;
    const StackArgs st = pick(a, s);
    const uint32_t q0 = t * TILE;
    const uint32_t q1 = min(q0 + TILE, st.pend);

    // Offset groups of the tile (run q: field q % F of group q / F).
    u32x4 v[RUNS];
    const rsrc_t seg = make_rsrc(st.offsets + (uint64_t)e * st.stride, (uint32_t)st.stride);
    const uint32_t gshift = st.wbits == 4 ? 1u : 3u;
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t run = (q0 >> 4) + i * kBlock + threadIdx.x;
        v[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(seg, (int)((run >> gshift) << 4), 0, kNonTemporal));
    }
    // Row bases: for C >= 16 the two rows each run may touch, into registers;
    // for C < 16 the tile's rows, to be staged in LDS.
    const rsrc_t rb = make_rsrc(st.bases + (uint64_t)e * st.R, st.R);
    const bool direct = __builtin_amdgcn_readfirstlane(st.row_mode) != kRowBytes;  // the same in every lane
    const uint32_t r_lo = div_exact(q0, st.rcp_cols);
    uint32_t rrow[RUNS], bb0[RUNS], bb1[RUNS];
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t pos = q0 + kRunBytes * (i * kBlock + threadIdx.x);
        rrow[i] = direct ? div_exact(min(pos, q1 - 1u), st.rcp_cols) : r_lo + i * kBlock + threadIdx.x;
        bb0[i] = __builtin_amdgcn_raw_buffer_load_b8(rb, (int)rrow[i], 0, 0);
        bb1[i] = direct ? __builtin_amdgcn_raw_buffer_load_b8(rb, (int)(rrow[i] + 1u), 0, 0)
                        : __builtin_amdgcn_raw_buffer_load_b8(rb, (int)(rrow[i] + RUNS * kBlock), 0, 0);
    }
    // (the offset and base loads above are issued before the wait for the
    // index bounds below)
    __builtin_amdgcn_sched_barrier(0);
    // The tile's index bounds, then its first EXC * kBlock entries in 16-byte
    // loads from `first` (lo rounded down to a multiple of 4).
    const int32_t *ti = st.tile_index + (uint64_t)e * st.index_tiles + t * INDEX_PER_TILE;
    const int32_t l0 = ti[0], h0 = ti[min(INDEX_PER_TILE, st.index_tiles - t * INDEX_PER_TILE)];
    const uint32_t hi = h0 < 0 ? 0u : min((uint32_t)h0, st.n_exc);
    const uint32_t lo = l0 < 0 ? 0u : min((uint32_t)l0, hi);
    const uint32_t first = lo & ~3u;
    const rsrc_t rx = make_rsrc(st.exc + first, 4u * (hi - first));
    uint32_t w[EXC];
#pragma unroll
    for (uint32_t i = 0; i < EXC / 4; ++i) {
        const u32x4 q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(16u * (i * kBlock + threadIdx.x)), 0,
                                                         kNonTemporal));
        w[4 * i] = q.x;
        w[4 * i + 1] = q.y;
        w[4 * i + 2] = q.z;
        w[4 * i + 3] = q.w;
    }
    clk.mark_drained(2);

    uint8_t *plane = st.ws + (uint64_t)e * st.P;
    // The prefetched entries, then any beyond them; the tile's stores.
    auto patch_and_store = [&]() {
#pragma unroll
        for (uint32_t i = 0; i < EXC; ++i) {
            const uint32_t kk = entry_of(first, i);
            const uint32_t pos = w[i] >> 8;
            if (kk >= lo && kk < hi && pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(w[i] & 0xffu);
        }
        if (first + EXC * kBlock < hi) [[unlikely]] {
            for (uint32_t kk = first + EXC * kBlock + threadIdx.x; kk < hi; kk += kBlock) {
                const uint32_t x = st.exc[kk];
                const uint32_t pos = x >> 8;
                if (pos >= q0 && pos < q1) tile[pos - q0] = (uint8_t)(x & 0xffu);
            }
        }
        __syncthreads();  // tile patched
        clk.mark(4);
        store_tile<RUNS, WINDOW>(st, plane, q0, q1, tile);
        clk.mark(5);
        clk.mark_drained(6);
        clk.write(a, 1ull + u + ((uint64_t)(hi - first > EXC * kBlock) << 32));
    };
    if (!direct) [[unlikely]] {
        // rows of fewer than 16 columns: the tile's row bases staged in LDS
        const uint32_t nrows = div_exact(q1 - 1u, st.rcp_cols) - r_lo + 1u;
#pragma unroll
        for (uint32_t i = 0; i < RUNS; ++i) {
            const uint32_t r = i * kBlock + threadIdx.x;
            if (r < nrows) lds_bases[r] = (uint8_t)bb0[i];
            if (r + RUNS * kBlock < nrows) lds_bases[r + RUNS * kBlock] = (uint8_t)bb1[i];
        }
        const uint8_t *brow = st.bases + (uint64_t)e * st.R + r_lo;
        for (uint32_t r = threadIdx.x + 2u * RUNS * kBlock; r < nrows; r += kBlock) lds_bases[r] = brow[r];
        __syncthreads();
        expand_dispatch<true, RUNS, false>(st, v, q0, q1, q0, lds_bases, r_lo, tile, plane);
        __syncthreads();  // tile expanded
        clk.mark(3);
        patch_and_store();
        return;
    }
#pragma unroll
    for (uint32_t i = 0; i < RUNS; ++i) {
        const uint32_t j = i * kBlock + threadIdx.x;
        const uint32_t pos = q0 + kRunBytes * j;
        if (pos >= q1) break;
        const uint32_t s0 = bb0[i] * 0x01010101u, s1 = bb1[i] * 0x01010101u;
        *reinterpret_cast<u32x4 *>(tile + kRunBytes * j) = expand_run(v[i], pos, rrow[i], st.C, s0, s1, st.wbits);
    }
    __syncthreads();  // tile expanded
    clk.mark(3);
    patch_and_store();
}

// WINDOW: some stack's row window does not cover its whole plane (csf_decode_rows).
template <uint32_t RUNS, uint32_t EXC, uint32_t SCHED, bool WINDOW>
__global__ __launch_bounds__(kBlock, SCHED == kPipelined ? 6 : 1) void csf_fused_kernel(DecodeArgs a) {
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    __shared__ __align__(16) uint8_t tile[tile_positions(RUNS)];
    if constexpr (SCHED == kStreamEntries)
        tile_loop_serial<true, RUNS, EXC, false, true, WINDOW>(a, dyn_lds, tile);
    else
        tile_loop_pipelined<RUNS, EXC, 0, WINDOW>(a, dyn_lds, tile, a.E, reinterpret_cast<const uint16_t *>(dyn_lds), a.expert_start != nullptr);
}

// The routed schedule (kRouted), its routing inputs ahead of the argument
// block (RouteHead).  STAMP: a traced routed decode (timestamps per workgroup);
// WIDE: int64 expert_start.
template <uint32_t RUNS, uint32_t EXC, bool WINDOW, bool STAMP, bool WIDE>
__global__ __launch_bounds__(kBlock, 1) void csf_routed_kernel(const void *expert_start, uint32_t E, uint32_t flags,
                                                               uint32_t tiles0, uint32_t tiles1, uint32_t first0,
                                                               uint32_t first1, uint32_t grid, DecodeArgs a) {
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    __shared__ __align__(16) uint8_t tile[tile_positions(RUNS)];
    const RouteHead h = {expert_start, E, flags, {tiles0, tiles1}, {first0, first1}, grid};
    routed_decode<RUNS, EXC, WINDOW, STAMP, WIDE>(h, a, dyn_lds, tile);
}

template <uint32_t RUNS, bool WINDOW>
__global__ __launch_bounds__(kBlock) void csf_fixed_kernel(DecodeArgs a) {
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    tile_loop_serial<false, RUNS, 1, false, false, WINDOW>(a, dyn_lds, nullptr);
}

// Largest k in [k, n) with M[k] <= t, given M[k] <= t < M[n]: gallop, then bisect.
__device__ __forceinline__ uint32_t find_expert(const uint32_t *M, uint32_t k, uint32_t n,
                                                uint32_t t) {
    uint32_t lo = k, hi = k + 1, step = 1;
    while (hi < n && M[hi] <= t) {
        lo = hi;
        step <<= 1;
        hi = lo + step;
    }
    if (hi > n) hi = n;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (M[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Exception pass alone.
//
// The entries of all active experts of both stacks form one index space
// [0, N0 + N1), laid out by the prefixes M_s over the listed experts' entry
// counts.  Workgroups take chunks of kBlock*EPL consecutive indices, EPL (1,
// 2, 4 or kExcPerLane entries per lane) the fewest that leave each workgroup
// at most one chunk; lane l handles index t = chunk + l + i*kBlock, so each
// load instruction of a wave reads 64 consecutive entries.  Entry t of stack
// s belongs to the listed expert k with M_s[k] <= t < M_s[k+1]; it is word
// B_s[k] + (t - M_s[k]), B_s[k] being that expert's prefix value.
// ---------------------------------------------------------------------------
constexpr uint32_t kCountChunks = 4; // 64-expert chunks of prefix bounds read per round trip

// Inclusive scan over the wave of counts capped at cap (< 2^31, so a sum of
// two capped values fits in 32 bits): lane l gets min(cap, c_0 + ... + c_l).
__device__ __forceinline__ uint32_t capped_scan(uint32_t c, uint32_t cap) {
    const uint32_t lane = threadIdx.x % kWave;
#pragma unroll
    for (uint32_t d = 1; d < kWave; d <<= 1) {
        const uint32_t y = __shfl_up(c, d, kWave);
        if (lane >= d) c = min(c + y, cap);
    }
    return c;
}

// Wave 0, after list_experts: for the n listed experts of stack s, B_s[k] =
// prefix_s[act[k]] and M_s[k + 1] = min(n_exc_s, entries of listed experts
// 0..k), an expert's entry count being prefix_s[e+1] - prefix_s[e] clamped
// to [0, n_exc_s]; M_s[0] = 0.  The prefix bounds of kCountChunks * 64
// experts are read in one round trip.
__device__ __forceinline__ void count_entries(const DecodeArgs &a, uint32_t ns, const uint16_t *act,
                                              uint32_t n, int32_t *B0, int32_t *B1, uint32_t *M0,
                                              uint32_t *M1) {
    const uint32_t lane = threadIdx.x;
    // With one stack, stack 1's bounds are read from stack 0's prefix (so
    // every load is unconditional) and capped to nothing.
    const int32_t *pf0 = a.st[0].prefix, *pf1 = ns > 1 ? a.st[1].prefix : pf0;
    const uint32_t cap0 = a.st[0].n_exc, cap1 = ns > 1 ? a.st[1].n_exc : 0u;
    if (lane == 0) {
        M0[0] = 0;
        M1[0] = 0;
    }
    uint32_t run0 = 0, run1 = 0;
    for (uint32_t kb = 0; kb < n; kb += kWave * kCountChunks) {
        int32_t lo0[kCountChunks], hi0[kCountChunks], lo1[kCountChunks], hi1[kCountChunks];
#pragma unroll
        for (uint32_t u = 0; u < kCountChunks; ++u) {
            const uint32_t k = kb + kWave * u + lane;
            const uint32_t e = act[min(k, n - 1u)];
            lo0[u] = pf0[e];
            hi0[u] = pf0[e + 1];
            lo1[u] = pf1[e];
            hi1[u] = pf1[e + 1];
        }
#pragma unroll
        for (uint32_t u = 0; u < kCountChunks; ++u) {
            const uint32_t k = kb + kWave * u + lane;
            const bool live = k < n;
            const int64_t d0 = (int64_t)hi0[u] - lo0[u], d1 = (int64_t)hi1[u] - lo1[u];
            const uint32_t c0 = live ? (uint32_t)(d0 < 0 ? 0 : d0 > cap0 ? cap0 : d0) : 0u;
            const uint32_t c1 = live ? (uint32_t)(d1 < 0 ? 0 : d1 > cap1 ? cap1 : d1) : 0u;
            const uint32_t s0 = min(run0 + capped_scan(c0, cap0), cap0);
            const uint32_t s1 = min(run1 + capped_scan(c1, cap1), cap1);
            if (live) {
                B0[k] = lo0[u];
                M0[k + 1] = s0;
                if (ns > 1) {
                    B1[k] = lo1[u];
                    M1[k + 1] = s1;
                }
            }
            run0 = __shfl(s0, kWave - 1, kWave);
            run1 = __shfl(s1, kWave - 1, kWave);
        }
    }
}

__global__ __launch_bounds__(kBlock) void csf_exc_kernel(DecodeArgs a) {
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    __shared__ uint32_t s_nact;

    const uint32_t E = a.E;
    const uint32_t ns = a.nstacks;
    const uint32_t words = (E + 1u + 3u) & ~3u;  // one [E+1] map of 4-byte words, padded to 16 B
    uint16_t *act = reinterpret_cast<uint16_t *>(dyn_lds);
    int32_t *B0 = reinterpret_cast<int32_t *>(dyn_lds + ((2u * E + 15u) & ~15u));
    int32_t *B1 = B0 + words;
    uint32_t *M0 = reinterpret_cast<uint32_t *>(B1 + words);
    uint32_t *M1 = M0 + words;

    if (threadIdx.x < kWave) {
        uint32_t n;
        if (a.expert_start == nullptr)
            n = list_experts(static_cast<const int32_t *>(nullptr), E, act);
        else if (a.es_wide)
            n = list_experts(static_cast<const int64_t *>(a.expert_start), E, act);
        else
            n = list_experts(static_cast<const int32_t *>(a.expert_start), E, act);
        // act was written by other lanes of this wave; LDS accesses of one
        // wave take effect in order.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (n > 0) count_entries(a, ns, act, n, B0, B1, M0, M1);
        if (threadIdx.x == 0) s_nact = n;
    }
    __syncthreads();
    const uint32_t nact = s_nact;
    if (nact == 0) return;
    const uint32_t N0 = M0[nact];
    const uint32_t N = N0 + (ns > 1 ? M1[nact] : 0u);
    // Both stacks' fields as values: the stack is picked per entry, that is
    // per lane, and a field read through an address picked per lane would be
    // a vector load from the argument block, waited for before each entry.
    const uint32_t *const exc0 = a.st[0].exc, *const exc1 = a.st[1].exc;
    uint8_t *const ws0 = a.st[0].ws, *const ws1 = a.st[1].ws;
    const uint32_t nexc0 = a.st[0].n_exc, nexc1 = a.st[1].n_exc;
    const uint32_t P0 = a.st[0].P, P1 = a.st[1].P;
    const uint32_t beg0 = a.st[0].pbeg, beg1 = a.st[1].pbeg;
    const uint32_t end0 = a.st[0].pend, end1 = a.st[1].pend;

    // EPL entries per lane per chunk.
    auto scatter = [&](auto eplc) {
        constexpr uint32_t EPL = decltype(eplc)::value;
        const uint32_t chunk = kBlock * EPL;
        for (uint32_t c0 = blockIdx.x * chunk; c0 < N; c0 += gridDim.x * chunk) {
            uint32_t id[EPL], x[EPL];
            uint8_t *dst[EPL];
            bool hi[EPL], ok[EPL];
            uint32_t k = 0, prev_s = 0;
            // Locate every entry first, then load them all unconditionally, so
            // the loads are in flight together: lanes past N re-read entry
            // N - 1, and an index past its stack's entries (a prefix that
            // overruns them) reads the stack's last entry; neither is stored.
            // A stack that owns a compacted index has at least one entry.
#pragma unroll
            for (uint32_t i = 0; i < EPL; ++i) {
                const uint32_t tl = c0 + threadIdx.x + i * kBlock;
                const uint32_t t = tl < N ? tl : N - 1u;
                const uint32_t s = t >= N0 ? 1u : 0u;
                const uint32_t tt = t - (s ? N0 : 0u);
                if (s != prev_s) {
                    k = 0;
                    prev_s = s;
                }
                const uint32_t *M = s ? M1 : M0;
                k = find_expert(M, k, nact, tt);
                const uint32_t e = act[k];
                const uint32_t j = (uint32_t)(s ? B1 : B0)[k] + (tt - M[k]);
                const uint32_t n = s ? nexc1 : nexc0;
                hi[i] = s != 0;
                ok[i] = tl < N && j < n;
                id[i] = j < n ? j : n - 1u;
                dst[i] = (s ? ws1 : ws0) + (uint64_t)e * (s ? P1 : P0);
            }
#pragma unroll
            for (uint32_t i = 0; i < EPL; ++i) x[i] = (hi[i] ? exc1 : exc0)[id[i]];
#pragma unroll
            for (uint32_t i = 0; i < EPL; ++i) {
                const uint32_t pos = x[i] >> 8;
                if (ok[i] && pos >= (hi[i] ? beg1 : beg0) && pos < (hi[i] ? end1 : end0))
                    dst[i][pos] = (uint8_t)(x[i] & 0xffu);
            }
        }
    };
    // The fewest entries per lane that still give every workgroup at most one
    // chunk: a routed call has few entries for its grid, and smaller chunks
    // spread them over more workgroups, so each lane locates, loads and stores
    // fewer one after another.  The grid-stride loop is correct for any grid.
    const uint32_t per_group = (N + gridDim.x - 1u) / gridDim.x;
    if (per_group <= kBlock)
        scatter(std::integral_constant<uint32_t, 1>{});
    else if (per_group <= 2u * kBlock)
        scatter(std::integral_constant<uint32_t, 2>{});
    else if (per_group <= 4u * kBlock)
        scatter(std::integral_constant<uint32_t, 4>{});
    else
        scatter(std::integral_constant<uint32_t, kExcPerLane>{});
}

// ---------------------------------------------------------------------------
// Per-tile exception index: thread i < E*NT handles tile j = i % NT of expert
// e = i / NT and writes prefix[e] + #{entries of e with position < j*kIndexTile}
// (a binary search over the expert's ascending positions); the last thread
// writes prefix[E].  Prefix values are clamped to [0, n_exc].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void csf_index_kernel(StackArgs s, uint32_t E, int32_t *out) {
    const uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t total = (uint64_t)E * s.index_tiles;
    if (i > total) return;
    auto clampn = [&](int32_t v) -> uint32_t { return v < 0 ? 0u : min((uint32_t)v, s.n_exc); };
    if (i == total) {
        out[i] = (int32_t)clampn(s.prefix[E]);
        return;
    }
    const uint32_t e = (uint32_t)(i / s.index_tiles);
    const uint32_t j = (uint32_t)(i - (uint64_t)e * s.index_tiles);
    uint32_t lo = clampn(s.prefix[e]);
    uint32_t hi = clampn(s.prefix[e + 1]);
    if (hi < lo) hi = lo;
    const uint32_t bound = j * kIndexTile;
    while (lo < hi) {  // first entry with position >= bound
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if ((s.exc[mid] >> 8) < bound) lo = mid + 1; else hi = mid;
    }
    out[i] = (int32_t)lo;
}

}  // namespace

size_t tile_lds_bytes(const DecodeArgs &a) {
    size_t n = a.bases_stage;
    if (a.expert_start != nullptr) n += (2u * a.E + 15u) & ~15u;  // active list
    return n;
}

static size_t exc_lds_bytes(const DecodeArgs &a) {
    const size_t words = (a.E + 1u + 3u) & ~3u;
    return ((2u * a.E + 15u) & ~15u) + 4u * 4u * words;
}

template <bool WINDOW>
hipError_t launch_fixed_t(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    const size_t lds = tile_lds_bytes(a);
    switch (a.runs) {
        case 1: hipLaunchKernelGGL((csf_fixed_kernel<1, WINDOW>), dim3(grid), dim3(kBlock), lds, stream, a); break;
        case 2: hipLaunchKernelGGL((csf_fixed_kernel<2, WINDOW>), dim3(grid), dim3(kBlock), lds, stream, a); break;
        case 4: hipLaunchKernelGGL((csf_fixed_kernel<4, WINDOW>), dim3(grid), dim3(kBlock), lds, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fixed(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    return a.windowed ? launch_fixed_t<true>(a, grid, stream) : launch_fixed_t<false>(a, grid, stream);
}

static uint32_t head_flags(const DecodeArgs &a) {
    return a.nstacks > 1 ? kHeadPair : 0u;
}

template <bool WINDOW>
hipError_t launch_fused_t(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    const size_t lds = tile_lds_bytes(a);
    const dim3 g(grid), b(kBlock);
    // (runs, entries per lane, load schedule) combinations the host plans
    if (a.runs == 1 && a.exc_regs == 4 && a.sched == kSchedRouted)
        hipLaunchKernelGGL((a.es_wide ? csf_routed_kernel<1, 4, WINDOW, false, true>
                                      : csf_routed_kernel<1, 4, WINDOW, false, false>),
                           g, b, lds, stream, a.expert_start, a.E, head_flags(a), a.st[0].tiles, a.st[1].tiles,
                           a.st[0].tile0, a.st[1].tile0, grid, a);
    else if (a.runs == 2 && a.exc_regs == 4 && a.sched == kSchedStreamEntries)
        hipLaunchKernelGGL((csf_fused_kernel<2, 4, kStreamEntries, WINDOW>), g, b, lds, stream, a);
    else if (a.runs == 2 && a.exc_regs == 8 && a.sched == kSchedStreamEntries)
        hipLaunchKernelGGL((csf_fused_kernel<2, 8, kStreamEntries, WINDOW>), g, b, lds, stream, a);
    else if (a.runs == 4 && a.exc_regs == 4 && a.sched == kSchedPipelined)
        hipLaunchKernelGGL((csf_fused_kernel<4, 4, kPipelined, WINDOW>), g, b, lds, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fused(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    return a.windowed ? launch_fused_t<true>(a, grid, stream) : launch_fused_t<false>(a, grid, stream);
}

hipError_t launch_fused_traced(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    const size_t lds = tile_lds_bytes(a);
    const dim3 g(grid), b(kBlock);
    if (a.windowed || a.stamps == nullptr || a.sched != kSchedRouted || a.runs != 1) return hipErrorInvalidValue;
    if (a.exc_regs != 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((a.es_wide ? csf_routed_kernel<1, 4, false, true, true>
                                  : csf_routed_kernel<1, 4, false, true, false>),
                       g, b, lds, stream, a.expert_start, a.E, head_flags(a), a.st[0].tiles, a.st[1].tiles,
                       a.st[0].tile0, a.st[1].tile0, grid, a);
    return hipGetLastError();
}

hipError_t launch_exceptions(const DecodeArgs &a, uint32_t grid, hipStream_t stream) {
    hipLaunchKernelGGL(csf_exc_kernel, dim3(grid), dim3(kBlock), exc_lds_bytes(a), stream, a);
    return hipGetLastError();
}

hipError_t launch_build_index(const StackArgs &s, uint32_t E, int32_t *tile_index,
                              hipStream_t stream) {
    const uint64_t n = (uint64_t)E * s.index_tiles + 1;
    const uint32_t grid = (uint32_t)((n + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(csf_index_kernel, dim3(grid), dim3(kBlock), 0, stream, s, E, tile_index);
    return hipGetLastError();
}

}  // namespace csf
