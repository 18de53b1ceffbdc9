// Internal interface between the C ABI (csf_api.cpp) and the gfx950 kernels
// (csf_kernels.hip).  Not installed; the public ABI is include/csf.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csf {

constexpr uint32_t kBlock = 256;                    // threads per workgroup (4 wave64)
constexpr uint32_t kRunBytes = 16;                  // output bytes per lane per run
constexpr uint32_t kIndexTile = 2048;               // positions per exception-index tile

// Tile = kBlock * kRunBytes * runs positions, runs (per lane) in {1, 2, 4}.
constexpr uint32_t tile_positions(uint32_t runs) { return kBlock * kRunBytes * runs; }
constexpr uint32_t kExcPerLane = 8;                 // entries per lane of an exception-pass chunk, at most (the grid is sized for it)
constexpr uint32_t kBasesSlack = 32;                // rows read past a tile's last row by edge runs
constexpr uint32_t kMaxExperts = 2048;              // experts per stack (the ABI's limit)
constexpr uint32_t kStampsPerGroup = 8;             // timestamps a traced decode records per workgroup

// Load schedules of the fused kernel (csf_kernels.hip describes them).
constexpr uint32_t kSchedPipelined = 0;
constexpr uint32_t kSchedStreamEntries = 1;
constexpr uint32_t kSchedRouted = 2;

// How a 16-byte output run finds its row bases.
enum RowMode : uint32_t {
    kRowSplat = 0,  // C % 16 == 0: a run never crosses a row
    kRowTwo = 1,    // C >= 16: a run spans at most two rows
    kRowBytes = 2   // C < 16: per-byte row walk
};

// One compressed stack plus its dense destination, as the kernels see it.
struct StackArgs {
    const uint8_t *bases;       // [E * R]
    const uint8_t *offsets;     // [E * stride], 16-byte aligned
    const uint32_t *exc;        // [n_exc] (never dereferenced when n_exc == 0)
    const int32_t *prefix;      // [E + 1]
    const int32_t *tile_index;  // [E * index_tiles + 1] or nullptr
    uint8_t *ws;                // [E * P], any alignment
    int64_t stride;             // offset bytes per expert (multiple of 16)
    double rcp_cols;            // 1.0 / C, for exact row = pos / C with pos < 2^24
    uint32_t n_exc;             // total entries (< 2^31)
    uint32_t P;                 // R * C  (< 2^24)
    uint32_t R;
    uint32_t C;
    uint32_t pbeg, pend;        // positions decoded: rows begin .. end-1 (0, P: every row)
    uint32_t tile0;             // first tile decoded: pbeg / tile positions of the launch
    uint32_t tiles;             // tiles decoded per plane: tile0 .. ceil(pend / tile) - 1
    uint32_t index_tiles;       // ceil(P / kIndexTile)
    uint32_t wbits;             // 4 (NVFP4) or 1 (MXFP4)
    uint32_t row_mode;          // RowMode
};

struct DecodeArgs {
    StackArgs st[2];
    const void *expert_start;     // int32 or int64 [E + 1]; nullptr: every expert is active
    uint32_t nstacks;             // 1 or 2
    uint32_t E;                   // experts (same for both stacks)
    uint32_t bases_stage;         // bytes of dynamic LDS for one tile's row bases
    uint32_t runs;                // 16-byte runs per lane per tile (1, 2 or 4)
    uint32_t sched;               // load schedule of the fused kernel (kSched*)
    uint32_t exc_regs;            // entries per lane loaded with the offsets (fused: 4 or 8)
    uint32_t es_wide;             // expert_start holds int64 (else int32)
    uint32_t windowed;            // some stack decodes a row window short of its whole plane
    uint64_t *stamps;             // traced decodes: kStampsPerGroup clock values per workgroup, else nullptr
};

// Dynamic LDS bytes a tile kernel needs for these arguments.
size_t tile_lds_bytes(const DecodeArgs &a);

// Fixed stream alone: every position = base + offset field (a.runs picks the tile).
hipError_t launch_fixed(const DecodeArgs &a, uint32_t grid, hipStream_t stream);
// Exception scatter alone (after the fixed stream): entries overwrite their positions.
hipError_t launch_exceptions(const DecodeArgs &a, uint32_t grid, hipStream_t stream);
// Both in one pass, exceptions patched on chip before the stores (needs tile_index).
hipError_t launch_fused(const DecodeArgs &a, uint32_t grid, hipStream_t stream);
// The same with per-workgroup timestamps written to a.stamps (routed decodes only).
hipError_t launch_fused_traced(const DecodeArgs &a, uint32_t grid, hipStream_t stream);
// Per-tile exception index of one stack from its entries and prefix.
hipError_t launch_build_index(const StackArgs &s, uint32_t E, int32_t *tile_index, hipStream_t stream);

// W4A16 MoE projection consuming the compressed scales (csf_moe.hip).
struct MoeArgs {
    StackArgs st;                  // scale stack: shape, and the CSF streams when dense is nullptr
    const uint8_t *dense;          // dense scales [E][N][C], or nullptr: scales decoded into LDS
    const uint8_t *w;              // E2M1 codes [E][N][K/2], even k in the low nibble
    const uint16_t *x;             // bfloat16 activations [T][K], tokens grouped by expert
    const float *alpha;            // per-expert tensor scale [E]
    const int32_t *expert_start;   // [E + 1]
    float *y;                      // [T][N]
    uint32_t E, N, K, C, T;        // C = K / 16 (NVFP4) or K / 32 (MXFP4)
    uint32_t ntiles;               // ceil(N / 32) work units per routed expert
    uint32_t bases_stage;          // dynamic LDS bytes for one unit's row bases
    uint32_t pad_;
};

size_t moe_lds_bytes(const MoeArgs &a);
hipError_t launch_moe_w4a16(const MoeArgs &a, uint32_t grid, hipStream_t stream);

// Encoder on the device (csf_encode.hip).
struct EncodeArgs {
    const uint8_t *dense;   // [E * P]
    uint8_t *bases;         // [E * R]
    uint8_t *offsets;       // [E * stride]
    uint32_t *exc;          // [n]
    int32_t *prefix;        // [E + 1]
    int32_t *tile_index;    // [E * index_tiles + 1]
    int64_t stride;         // 16 * groups
    double rcp_cols;        // 1.0 / C
    uint32_t E, R, C, P;
    uint32_t groups;        // 16-byte offset groups per expert
    uint32_t index_tiles;   // ceil(P / kIndexTile)
    uint32_t wbits;         // 4 or 1
    uint32_t pad_;
};

// Row bases, offset stream, per-tile entry counts scanned into tile_index
// and prefix.
hipError_t launch_encode_streams(const EncodeArgs &a, uint32_t cus, hipStream_t stream);
// Exception entries (after launch_encode_streams, in stream order).
hipError_t launch_encode_entries(const EncodeArgs &a, uint32_t cus, hipStream_t stream);

}  // namespace csf
