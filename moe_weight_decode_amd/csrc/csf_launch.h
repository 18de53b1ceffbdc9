// Internal interface between the C ABI (csf_api.cpp) and the gfx950 kernels
// (csf_kernels.hip).  Not installed; the public ABI is include/csf.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csf {

constexpr int kBlock = 256;          // threads per workgroup (4 wave64)
constexpr int kFixedMaxSlots = 4;    // offset groups per lane per fixed-stream unit
constexpr int kBasesLds = 4096;      // bytes of row bases staged per fixed-stream unit
constexpr int kBasesLdsSlack = 32;   // rows read past a unit's last row by edge runs
constexpr int kExcPerLane = 8;       // exception entries per lane per exception chunk

// How a 16-byte output run finds its row bases.
enum RowMode : uint32_t {
    kRowSplat = 0,  // C % 16 == 0: a run never crosses a row
    kRowTwo = 1,    // C >= 16: a run spans at most two rows
    kRowBytes = 2   // C < 16: per-byte row walk
};

// One compressed stack plus its dense destination, as the kernels see it.
struct StackArgs {
    const uint8_t *bases;     // [E * R]
    const uint8_t *offsets;   // [E * stride], 16-byte aligned
    const uint32_t *exc;      // [n_exc] (never dereferenced when n_exc == 0)
    const int32_t *prefix;    // [E + 1]
    uint8_t *ws;              // [E * P], any alignment
    int64_t stride;           // offset bytes per expert (multiple of 16)
    double rcp_cols;          // 1.0 / C, for exact row = pos / C with pos < 2^24
    uint32_t n_exc;           // total entries (< 2^31)
    uint32_t P;               // R * C  (< 2^24)
    uint32_t R;
    uint32_t C;
    uint32_t groups;          // 16-byte offset groups per expert: ceil(P / G)
    uint32_t unit_groups;     // groups per fixed-stream unit (<= kBlock * kFixedMaxSlots)
    uint32_t units;           // fixed-stream units per expert: ceil(groups / unit_groups)
    uint32_t wbits;           // 4 (NVFP4) or 1 (MXFP4)
    uint32_t row_mode;        // RowMode
    uint32_t pad_;
};

struct DecodeArgs {
    StackArgs st[2];
    const int32_t *expert_start;  // nullptr: every expert is active
    uint32_t nstacks;             // 1 or 2
    uint32_t E;                   // experts (same for both stacks)
};

// Enqueue the fixed-stream expansion (every position = base + offset field).
hipError_t launch_fixed(const DecodeArgs &a, uint32_t grid, hipStream_t stream);
// Enqueue the exception scatter (entries overwrite their positions).
hipError_t launch_exceptions(const DecodeArgs &a, uint32_t grid, hipStream_t stream);

}  // namespace csf
