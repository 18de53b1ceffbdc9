// C ABI of the CSF decoder: argument checks, launch planning, the host
// encoder and the host-side stream validator.  Declarations and the layout are
// in include/csf.h; the kernels are in csf_kernels.hip.
#include "csf.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "csf_launch.h"

namespace {

using csf::DecodeArgs;
using csf::StackArgs;

constexpr int64_t kMaxPlane = int64_t(1) << 24;  // positions ride in 24 bits of an entry

// Launch plan of the tile kernels (measured on MI355X with HBM-resident
// stacks): NVFP4 stacks with few exceptions stream best in 16384-position
// tiles at 6 workgroups per CU with the pipelined schedule (the next tile's
// loads before this tile's stores, entries read 16 bytes per lane); stacks
// with more exceptions, and MXFP4, in 8192-position tiles at 7 per CU, one
// tile's loads at a time, with non-temporal entry loads; routed decodes of a
// few experts in 4096-position tiles, which spread the little work over more
// CUs, with non-temporal offset and entry loads (their planes are read once
// and rarely cache-resident).  Each lane prefetches 4 of its tile's
// exception entries, 8 when the stack's exception density would average more
// than 3.5 per lane.
#ifndef CSF_SPARSE_RUNS
#define CSF_SPARSE_RUNS 4
#endif
#ifndef CSF_SPARSE_WG_PER_CU
#define CSF_SPARSE_WG_PER_CU 6
#endif
#ifndef CSF_DENSE_RUNS
#define CSF_DENSE_RUNS 2
#endif
#ifndef CSF_DENSE_WG_PER_CU
#define CSF_DENSE_WG_PER_CU 7
#endif
#ifndef CSF_ROUTED_RUNS
#define CSF_ROUTED_RUNS 1
#endif
#ifndef CSF_ROUTED_WG_PER_CU
#define CSF_ROUTED_WG_PER_CU 2
#endif
// "Few exceptions": at most this many entries per million dense positions.
#ifndef CSF_SPARSE_PPM
#define CSF_SPARSE_PPM 50000
#endif
// Mean entries per lane and tile above which a lane loads 8 instead of 4.
#ifndef CSF_EXC_LANE_MILLI
#define CSF_EXC_LANE_MILLI 3500
#endif
#ifndef CSF_EXC_WG_PER_CU
#define CSF_EXC_WG_PER_CU 8
#endif

int offset_bits(int32_t format) {
    if (format == CSF_NVFP4_E4M3) return 4;
    if (format == CSF_MXFP4_UE8M0) return 1;
    return 0;
}

csf_status check_shape(int32_t format, int32_t E, int32_t R, int32_t C) {
    if (offset_bits(format) == 0) return CSF_E_FORMAT;
    if (E <= 0 || R <= 0 || C <= 0) return CSF_E_SHAPE;
    if (int64_t(R) * C >= kMaxPlane) return CSF_E_SHAPE;
    return CSF_OK;
}

int64_t min_stride(int32_t format, int32_t R, int32_t C) {
    const int64_t G = 128 / offset_bits(format);
    return 16 * ((int64_t(R) * C + G - 1) / G);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Everything a decode can check without touching device memory.
csf_status check_stack(const csf_stack *s, const uint8_t *ws) {
    if (s == nullptr || ws == nullptr) return CSF_E_NULL;
    csf_status st = check_shape(s->format, s->num_experts, s->rows, s->cols);
    if (st != CSF_OK) return st;
    if (s->num_experts > CSF_MAX_EXPERTS) return CSF_E_SHAPE;
    if (s->bases == nullptr || s->offsets == nullptr || s->exc_prefix == nullptr) return CSF_E_NULL;
    if (s->num_exceptions < 0 || s->num_exceptions >= (int64_t(1) << 31)) return CSF_E_SIZE;
    if (s->num_exceptions > 0 && s->exceptions == nullptr) return CSF_E_NULL;
    // at least the plane's offset groups, 16-byte steps, and below 2^31 (an
    // expert segment is addressed by 32-bit buffer offsets)
    if (s->offsets_stride < min_stride(s->format, s->rows, s->cols) || s->offsets_stride % 16 != 0 ||
        s->offsets_stride >= (int64_t(1) << 31))
        return CSF_E_SIZE;
    if (!aligned(s->offsets, 16) || !aligned(s->exc_prefix, 4)) return CSF_E_ALIGN;
    if (s->num_exceptions > 0 && !aligned(s->exceptions, 4)) return CSF_E_ALIGN;
    if (s->tile_index != nullptr && !aligned(s->tile_index, 4)) return CSF_E_ALIGN;
    return CSF_OK;
}

int64_t index_tiles(int32_t R, int32_t C) {
    return (int64_t(R) * C + CSF_INDEX_TILE - 1) / CSF_INDEX_TILE;
}

static_assert(CSF_INDEX_TILE == csf::kIndexTile, "index tile of the ABI and the kernels");

// Rows [rb, re) of every plane are decoded (0 <= rb <= re <= R).
void fill_stack(StackArgs &a, const csf_stack &s, uint8_t *ws, uint32_t tile, int32_t rb, int32_t re) {
    const uint32_t P = uint32_t(s.rows) * uint32_t(s.cols);
    const uint32_t C = uint32_t(s.cols);
    a.bases = s.bases;
    a.offsets = s.offsets;
    a.exc = s.exceptions;
    a.prefix = s.exc_prefix;
    a.tile_index = s.tile_index;
    a.ws = ws;
    a.stride = s.offsets_stride;
    a.rcp_cols = 1.0 / double(C);
    a.n_exc = uint32_t(s.num_exceptions);
    a.P = P;
    a.R = uint32_t(s.rows);
    a.C = C;
    a.pbeg = uint32_t(rb) * C;
    a.pend = uint32_t(re) * C;
    a.tile0 = a.pbeg / tile;
    a.tiles = a.pend > a.pbeg ? (a.pend + tile - 1) / tile - a.tile0 : 0u;
    a.index_tiles = uint32_t(index_tiles(s.rows, s.cols));
    a.wbits = uint32_t(offset_bits(s.format));
    a.row_mode = (C % 16 == 0) ? csf::kRowSplat : (C >= 16 ? csf::kRowTwo : csf::kRowBytes);
}

// LDS for one tile's row bases: a tile of `tile` positions touches at most
// (tile - 1) / C + 2 rows; edge runs read up to kBasesSlack rows further.
uint32_t bases_stage_bytes(uint32_t C, uint32_t tile) {
    const uint32_t rows = (tile - 1) / C + 2 + csf::kBasesSlack;
    return (rows + 15u) & ~15u;
}

struct Plan {
    uint32_t runs;
    uint32_t wg_per_cu;
    uint32_t sched;
    uint32_t exc_regs;
};

// Tile size, grid and entry prefetch of the tile kernels for one call, from
// host data only (formats, shapes, entry counts).
Plan plan_tiles(const csf_stack *s0, const csf_stack *s1, bool routed) {
    int64_t entries = s0->num_exceptions, dense = int64_t(s0->num_experts) * s0->rows * s0->cols;
    bool nvfp4 = s0->format == CSF_NVFP4_E4M3;
    if (s1 != nullptr) {
        entries += s1->num_exceptions;
        dense += int64_t(s1->num_experts) * s1->rows * s1->cols;
        nvfp4 = nvfp4 && s1->format == CSF_NVFP4_E4M3;
    }
    Plan p;
    if (routed)
        p = {CSF_ROUTED_RUNS, CSF_ROUTED_WG_PER_CU, csf::kSchedRouted, 4};
    else if (nvfp4 && entries * 1000000 <= dense * int64_t(CSF_SPARSE_PPM))
        p = {CSF_SPARSE_RUNS, CSF_SPARSE_WG_PER_CU, csf::kSchedPipelined, 4};
    else
        p = {CSF_DENSE_RUNS, CSF_DENSE_WG_PER_CU, csf::kSchedStreamEntries, 4};
    // mean entries per lane and tile = density * tile / kBlock
    const int64_t tile = csf::tile_positions(p.runs);
    if (p.runs == 2 && entries * tile * 1000 > dense * int64_t(csf::kBlock) * CSF_EXC_LANE_MILLI)
        p.exc_regs = 8;
    return p;
}

// Compute units of each device, read once per device (the grid of every
// launch is a multiple of it).  A stream's device is remembered per thread
// for the last stream seen: a stale entry (a stream destroyed and its handle
// reused on another device) could only change a grid size, never a result,
// since every kernel is correct for any grid.
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_cus[kMaxDevices];

int stream_device(hipStream_t stream) {
    thread_local hipStream_t last_stream = nullptr;
    thread_local int last_dev = -1;
    int dev = -1;
    if (stream == nullptr) {
        if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    } else if (stream == last_stream && last_dev >= 0) {
        dev = last_dev;
    } else if (hipStreamGetDevice(stream, &dev) == hipSuccess) {
        last_stream = stream;
        last_dev = dev;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        dev = -1;
    }
    (void)hipGetLastError();  // a failed query leaves no error for the launch that follows
    return dev;
}

uint32_t cu_count(hipStream_t stream) {
    const int dev = stream_device(stream);
    if (dev < 0 || dev >= kMaxDevices) return 256;
    uint32_t n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
            (void)hipGetLastError();
            return 256;
        }
        n = uint32_t(v);
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// HIP reports the last error of any runtime call on the thread: one left by
// an earlier call must not be taken for a failure of this call's launches.
void clear_stale_error() { (void)hipGetLastError(); }

// Row window of a stack: rows, or every row when rows is NULL.
bool window(const csf_stack *s, const csf_rows *rows, int32_t &rb, int32_t &re) {
    rb = rows ? rows->begin : 0;
    re = rows ? rows->end : s->rows;
    return 0 <= rb && rb <= re && re <= s->rows;
}

// A traced decode (csf_decode_traced): where the timestamps go.
struct Trace {
    uint64_t *stamps;
    uint64_t capacity;
    uint32_t *groups;
};

csf_status enqueue(const csf_stack *s0, uint8_t *ws0, const csf_rows *rows0, const csf_stack *s1,
                   uint8_t *ws1, const csf_rows *rows1, const void *expert_start, bool es_wide,
                   uint32_t passes, void *hip_stream, const Trace *trace = nullptr) {
    if (passes == 0 || (passes & ~CSF_PASS_ALL) != 0) return CSF_E_SIZE;
    csf_status st = check_stack(s0, ws0);
    if (st != CSF_OK) return st;
    if (s1 != nullptr) {
        st = check_stack(s1, ws1);
        if (st != CSF_OK) return st;
        if (s1->num_experts != s0->num_experts) return CSF_E_MISMATCH;
    }
    const bool routed = expert_start != nullptr;
    if (routed && !aligned(expert_start, es_wide ? 8 : 4)) return CSF_E_ALIGN;
    int32_t rb0 = 0, re0 = 0, rb1 = 0, re1 = 0;
    if (!window(s0, rows0, rb0, re0)) return CSF_E_SHAPE;
    if (s1 != nullptr && !window(s1, rows1, rb1, re1)) return CSF_E_SHAPE;
    // A stack with an empty window is left out of the launch.
    if (s1 != nullptr && rb1 == re1) s1 = nullptr;
    if (rb0 == re0) {
        if (s1 == nullptr) return CSF_OK;
        s0 = s1, ws0 = ws1, rb0 = rb1, re0 = re1;
        s1 = nullptr;
    }

    const Plan plan = plan_tiles(s0, s1, routed);
    const uint32_t tile = csf::tile_positions(plan.runs);
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.expert_start = expert_start;
    a.es_wide = es_wide ? 1u : 0u;
    a.nstacks = s1 ? 2u : 1u;
    a.E = uint32_t(s0->num_experts);
    a.runs = plan.runs;
    a.sched = plan.sched;
    a.exc_regs = plan.exc_regs;
    fill_stack(a.st[0], *s0, ws0, tile, rb0, re0);
    a.bases_stage = bases_stage_bytes(a.st[0].C, tile);
    if (s1) {
        fill_stack(a.st[1], *s1, ws1, tile, rb1, re1);
        a.bases_stage = std::max(a.bases_stage, bases_stage_bytes(a.st[1].C, tile));
    } else {
        a.st[1] = a.st[0];  // never read: nstacks == 1
    }
    a.windowed = (rb0 != 0 || re0 != s0->rows || (s1 && (rb1 != 0 || re1 != s1->rows))) ? 1u : 0u;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const uint32_t cus = cu_count(stream);
    const uint64_t tile_units = uint64_t(a.E) * a.st[0].tiles + (s1 ? uint64_t(a.E) * a.st[1].tiles : 0);
    const uint64_t tile_cap = uint64_t(cus) * plan.wg_per_cu;
    const uint32_t tile_grid = uint32_t(std::max<uint64_t>(1, std::min(tile_units, tile_cap)));

    const bool indexed = s0->tile_index != nullptr && (s1 == nullptr || s1->tile_index != nullptr);
    if (trace != nullptr) {
        if (!indexed || !routed) return CSF_E_NULL;
        if (trace->stamps == nullptr) {
            *trace->groups = tile_grid;
            return CSF_OK;
        }
        if (trace->capacity < uint64_t(csf::kStampsPerGroup) * tile_grid) return CSF_E_SIZE;
        a.stamps = trace->stamps;
        clear_stale_error();
        if (csf::launch_fused_traced(a, tile_grid, stream) != hipSuccess) return CSF_E_HIP;
        *trace->groups = tile_grid;
        return CSF_OK;
    }
    clear_stale_error();
    if (passes == CSF_PASS_ALL && indexed) {
        if (csf::launch_fused(a, tile_grid, stream) != hipSuccess) return CSF_E_HIP;
        return CSF_OK;
    }
    if (passes & CSF_PASS_FIXED) {
        if (csf::launch_fixed(a, tile_grid, stream) != hipSuccess) return CSF_E_HIP;
    }
    if (passes & CSF_PASS_EXCEPTIONS) {
        const uint64_t entries = uint64_t(a.st[0].n_exc) + (s1 ? uint64_t(a.st[1].n_exc) : 0);
        if (entries > 0) {
            const uint64_t per = uint64_t(csf::kBlock) * csf::kExcPerLane;
            const uint64_t chunks = (entries + per - 1) / per;
            const uint64_t cap = uint64_t(cus) * (routed ? CSF_ROUTED_WG_PER_CU : CSF_EXC_WG_PER_CU);
            const uint32_t grid = uint32_t(std::max<uint64_t>(1, std::min(chunks, cap)));
            if (csf::launch_exceptions(a, grid, stream) != hipSuccess) return CSF_E_HIP;
        }
    }
    return CSF_OK;
}

// Workgroups per CU of the W4A16 consumer (8 waves of up to 256 VGPRs: one).
#ifndef CSF_MOE_WG_PER_CU
#define CSF_MOE_WG_PER_CU 1
#endif

csf_status moe_impl(const csf_stack *scales, const uint8_t *dense, const uint8_t *weights,
                    const uint16_t *x, int32_t num_tokens, const float *alpha,
                    const int32_t *expert_start, float *y, void *hip_stream) {
    csf_status st = check_stack(scales, weights);
    if (st != CSF_OK) return st;
    if (scales->format != CSF_NVFP4_E4M3 && scales->format != CSF_MXFP4_UE8M0) return CSF_E_FORMAT;
    const bool mx = scales->format == CSF_MXFP4_UE8M0;
    const int64_t C = scales->cols, K = (mx ? 32 : 16) * C;
    if (K % 32 != 0 || K > 8192) return CSF_E_SHAPE;  // whole 32-wide MFMA lane groups, at most 4 K-tiles
    if (num_tokens < 0) return CSF_E_SIZE;
    if (alpha == nullptr || expert_start == nullptr) return CSF_E_NULL;
    if (num_tokens > 0 && (x == nullptr || y == nullptr)) return CSF_E_NULL;  // no tokens: x, y may be NULL
    if (dense == nullptr && scales->tile_index == nullptr) return CSF_E_NULL;
    // dense NVFP4 scales are read two bytes at a time (C = K/16 is even)
    if (!aligned(weights, 16) || (x && !aligned(x, 4)) || !aligned(alpha, 4) || !aligned(expert_start, 4) ||
        (y && !aligned(y, 4)) || (dense && !mx && !aligned(dense, 2)))
        return CSF_E_ALIGN;
    if (num_tokens == 0) return CSF_OK;

    csf::MoeArgs a;
    std::memset(&a, 0, sizeof(a));
    fill_stack(a.st, *scales, nullptr, csf::kIndexTile, 0, scales->rows);
    a.dense = dense;
    a.w = weights;
    a.x = x;
    a.alpha = alpha;
    a.expert_start = expert_start;
    a.y = y;
    a.E = uint32_t(scales->num_experts);
    a.N = uint32_t(scales->rows);
    a.K = uint32_t(K);
    a.C = uint32_t(C);
    a.T = uint32_t(num_tokens);
    a.ntiles = (a.N + 31u) / 32u;
    a.bases_stage = bases_stage_bytes(a.C, 32u * a.C);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const uint64_t units = uint64_t(a.E) * a.ntiles;
    const uint64_t cap = uint64_t(cu_count(stream)) * CSF_MOE_WG_PER_CU;
    const uint32_t grid = uint32_t(std::max<uint64_t>(1, std::min(units, cap)));
    clear_stale_error();
    if (csf::launch_moe_w4a16(a, grid, stream) != hipSuccess) return CSF_E_HIP;
    return CSF_OK;
}

csf_status build_index_impl(const csf_stack *s, int32_t *tile_index, void *hip_stream) {
    if (tile_index == nullptr) return CSF_E_NULL;
    csf_status st = check_stack(s, reinterpret_cast<const uint8_t *>(tile_index));
    if (st != CSF_OK) return st;
    if (!aligned(tile_index, 4)) return CSF_E_ALIGN;
    StackArgs a;
    fill_stack(a, *s, nullptr, csf::kIndexTile, 0, s->rows);
    if (a.n_exc == 0) a.exc = nullptr;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    clear_stale_error();
    if (csf::launch_build_index(a, uint32_t(s->num_experts), tile_index, stream) != hipSuccess)
        return CSF_E_HIP;
    return CSF_OK;
}

csf_status encode_device_impl(int32_t format, int32_t E, int32_t R, int32_t C, const uint8_t *dense,
                              uint8_t *bases, uint8_t *offsets, uint32_t *exceptions,
                              int32_t *exc_prefix, int32_t *tile_index, uint32_t phase,
                              void *hip_stream) {
    csf_status st = check_shape(format, E, R, C);
    if (st != CSF_OK) return st;
    if (phase != CSF_ENCODE_STREAMS && phase != CSF_ENCODE_ENTRIES) return CSF_E_SIZE;
    if (int64_t(E) * R * C >= (int64_t(1) << 31)) return CSF_E_SIZE;
    if (dense == nullptr || bases == nullptr || tile_index == nullptr) return CSF_E_NULL;
    if (phase == CSF_ENCODE_STREAMS && (offsets == nullptr || exc_prefix == nullptr)) return CSF_E_NULL;
    if (phase == CSF_ENCODE_ENTRIES && exceptions == nullptr) return CSF_E_NULL;
    if (!aligned(tile_index, 4)) return CSF_E_ALIGN;
    if (phase == CSF_ENCODE_STREAMS && (!aligned(offsets, 16) || !aligned(exc_prefix, 4))) return CSF_E_ALIGN;
    if (phase == CSF_ENCODE_ENTRIES && !aligned(exceptions, 4)) return CSF_E_ALIGN;

    csf::EncodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.dense = dense;
    a.bases = bases;
    a.offsets = offsets;
    a.exc = exceptions;
    a.prefix = exc_prefix;
    a.tile_index = tile_index;
    a.stride = min_stride(format, R, C);
    a.rcp_cols = 1.0 / double(C);
    a.E = uint32_t(E);
    a.R = uint32_t(R);
    a.C = uint32_t(C);
    a.P = uint32_t(R) * uint32_t(C);
    a.groups = uint32_t(a.stride / 16);
    a.index_tiles = uint32_t(index_tiles(R, C));
    a.wbits = uint32_t(offset_bits(format));
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const uint32_t cus = cu_count(stream);
    clear_stale_error();
    const hipError_t err = phase == CSF_ENCODE_STREAMS ? csf::launch_encode_streams(a, cus, stream)
                                                       : csf::launch_encode_entries(a, cus, stream);
    return err == hipSuccess ? CSF_OK : CSF_E_HIP;
}

// ---------------------------------------------------------------------------
// Host encoder.  Same definition as the format in csf.h; written as a
// sliding-window base search, a per-position field pass and a group packing
// pass.
// ---------------------------------------------------------------------------
struct EncodeShape {
    int w, W, G, F;
    int64_t R, C, P, S;
};

// Base of each row: slide a W-wide window over the row's 256-bin histogram.
void choose_row_bases(const EncodeShape &sh, const uint8_t *plane, uint8_t *bases) {
    uint32_t hist[256 + 16];
    for (int64_t r = 0; r < sh.R; ++r) {
        std::memset(hist, 0, sizeof(hist));
        const uint8_t *row = plane + r * sh.C;
        for (int64_t c = 0; c < sh.C; ++c) ++hist[row[c]];
        uint32_t win = 0;
        for (int v = 0; v < sh.W; ++v) win += hist[v];
        uint32_t best = 0;
        int best_v = 0;
        for (int v = 0; v < 256; ++v) {
            if (hist[v] != 0 && win > best) {
                best = win;
                best_v = v;
            }
            win += hist[v + sh.W];
            win -= hist[v];
        }
        bases[r] = uint8_t(best_v);
    }
}

int64_t count_outside(const EncodeShape &sh, const uint8_t *plane, const uint8_t *bases) {
    int64_t n = 0;
    for (int64_t r = 0; r < sh.R; ++r) {
        const unsigned b = bases[r];
        const uint8_t *row = plane + r * sh.C;
        for (int64_t c = 0; c < sh.C; ++c) n += (unsigned(row[c]) - b) >= unsigned(sh.W);
    }
    return n;
}

// Offsets and exception words of one expert.
void encode_plane(const EncodeShape &sh, const uint8_t *plane, const uint8_t *bases, uint8_t *seg,
                  uint32_t *exc, std::vector<uint8_t> &field) {
    field.assign(size_t(sh.S / 16) * sh.G, 0);  // one byte per position, padded to whole groups
    int64_t n = 0;
    for (int64_t r = 0; r < sh.R; ++r) {
        const unsigned b = bases[r];
        for (int64_t c = 0; c < sh.C; ++c) {
            const int64_t p = r * sh.C + c;
            const unsigned d = unsigned(plane[p]) - b;
            if (d < unsigned(sh.W)) {
                field[size_t(p)] = uint8_t(d);
            } else {
                exc[n++] = (uint32_t(p) << 8) | plane[p];
            }
        }
    }
    const int64_t groups = sh.S / 16;
    for (int64_t g = 0; g < groups; ++g) {
        const uint8_t *fg = field.data() + g * sh.G;
        for (int j = 0; j < 16; ++j) {
            unsigned byte = 0;
            for (int f = 0; f < sh.F; ++f) byte |= unsigned(fg[16 * f + j]) << (sh.w * f);
            seg[g * 16 + j] = uint8_t(byte);
        }
    }
}

template <class Fn>
void parallel_experts(int32_t E, Fn fn) {
    const unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    const unsigned nt = std::min<unsigned>(hw, unsigned(E));
    if (nt <= 1) {
        for (int32_t e = 0; e < E; ++e) fn(e);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(nt);
    for (unsigned t = 0; t < nt; ++t)
        pool.emplace_back([&, t] {
            for (int32_t e = int32_t(t); e < E; e += int32_t(nt)) fn(e);
        });
    for (auto &th : pool) th.join();
}

// Tile index of one expert: walk its ascending entries once, closing tile j
// at the first entry whose position reaches j * CSF_INDEX_TILE.
void index_expert(const uint32_t *exc, int64_t begin, int64_t end, int64_t NT, int32_t *out) {
    int64_t k = begin;
    for (int64_t j = 0; j < NT; ++j) {
        const int64_t bound = j * CSF_INDEX_TILE;
        while (k < end && int64_t(exc[k] >> 8) < bound) ++k;
        out[j] = int32_t(k);
    }
}

csf_status prepare_impl(int32_t format, int32_t E, int32_t R, int32_t C, const uint8_t *dense,
                        csf_sizes *out, uint8_t *bases, uint8_t *offsets, uint32_t *exceptions,
                        int32_t *exc_prefix, int32_t *tile_index) {
    csf_status st = check_shape(format, E, R, C);
    if (st != CSF_OK) return st;
    if (dense == nullptr || out == nullptr) return CSF_E_NULL;
    const bool query = bases == nullptr && offsets == nullptr && exceptions == nullptr &&
                       exc_prefix == nullptr && tile_index == nullptr;
    if (!query && (bases == nullptr || offsets == nullptr || exc_prefix == nullptr)) return CSF_E_NULL;

    EncodeShape sh;
    sh.w = offset_bits(format);
    sh.W = 1 << sh.w;
    sh.G = 128 / sh.w;
    sh.F = 8 / sh.w;
    sh.R = R;
    sh.C = C;
    sh.P = int64_t(R) * C;
    sh.S = min_stride(format, R, C);

    std::vector<uint8_t> scratch_bases;
    uint8_t *b = bases;
    if (query) {
        scratch_bases.resize(size_t(E) * R);
        b = scratch_bases.data();
    }
    std::vector<int64_t> counts(size_t(E), 0);
    parallel_experts(E, [&](int32_t e) {
        const uint8_t *plane = dense + int64_t(e) * sh.P;
        choose_row_bases(sh, plane, b + int64_t(e) * R);
        counts[size_t(e)] = count_outside(sh, plane, b + int64_t(e) * R);
    });
    int64_t n = 0;
    for (int64_t c : counts) n += c;
    if (n >= (int64_t(1) << 31)) return CSF_E_SIZE;

    out->dense_bytes = int64_t(E) * sh.P;
    out->bases_bytes = int64_t(E) * R;
    out->offsets_stride = sh.S;
    out->offsets_bytes = int64_t(E) * sh.S;
    out->num_exceptions = n;
    out->exceptions_bytes = 4 * n;
    out->prefix_bytes = 4 * (int64_t(E) + 1);
    out->index_tiles = index_tiles(R, C);
    out->index_bytes = 4 * (int64_t(E) * out->index_tiles + 1);
    out->compressed_bytes = out->bases_bytes + out->offsets_bytes + out->exceptions_bytes +
                            out->prefix_bytes + out->index_bytes;
    if (query) return CSF_OK;
    if (n > 0 && exceptions == nullptr) return CSF_E_NULL;

    std::vector<int64_t> start(size_t(E) + 1, 0);
    for (int32_t e = 0; e < E; ++e) start[size_t(e) + 1] = start[size_t(e)] + counts[size_t(e)];
    for (int32_t e = 0; e <= E; ++e) exc_prefix[e] = int32_t(start[size_t(e)]);
    parallel_experts(E, [&](int32_t e) {
        thread_local std::vector<uint8_t> field;
        encode_plane(sh, dense + int64_t(e) * sh.P, b + int64_t(e) * R, offsets + int64_t(e) * sh.S,
                     exceptions + start[size_t(e)], field);
        if (tile_index != nullptr)
            index_expert(exceptions, start[size_t(e)], start[size_t(e) + 1], out->index_tiles,
                         tile_index + int64_t(e) * out->index_tiles);
    });
    if (tile_index != nullptr) tile_index[int64_t(E) * out->index_tiles] = int32_t(n);
    return CSF_OK;
}

csf_status validate_impl(const csf_stack *s) {
    if (s == nullptr) return CSF_E_NULL;
    csf_status st = check_shape(s->format, s->num_experts, s->rows, s->cols);
    if (st != CSF_OK) return st;
    if (s->bases == nullptr || s->offsets == nullptr || s->exc_prefix == nullptr) return CSF_E_NULL;
    if (s->num_exceptions < 0) return CSF_E_SIZE;
    if (s->num_exceptions > 0 && s->exceptions == nullptr) return CSF_E_NULL;
    if (s->offsets_stride < min_stride(s->format, s->rows, s->cols) || s->offsets_stride % 16 != 0 ||
        s->offsets_stride >= (int64_t(1) << 31))
        return CSF_E_SIZE;  // as the decoder's check
    const int w = offset_bits(s->format);
    const unsigned W = 1u << w;
    const int64_t G = 128 / w;
    const int64_t R = s->rows, C = s->cols, P = R * C, S = s->offsets_stride;
    // The whole prefix before any entry: 0, non-decreasing, num_exceptions at
    // the end, so every expert's entry range lies inside the entry array.
    const int32_t *pf = s->exc_prefix;
    if (pf[0] != 0 || pf[s->num_experts] != s->num_exceptions) return CSF_E_CORRUPT;
    for (int32_t e = 0; e < s->num_experts; ++e)
        if (pf[e + 1] < pf[e]) return CSF_E_CORRUPT;
    std::vector<uint8_t> is_exc(static_cast<size_t>(P));
    for (int32_t e = 0; e < s->num_experts; ++e) {
        const uint8_t *base = s->bases + int64_t(e) * R;
        const uint8_t *seg = s->offsets + int64_t(e) * S;
        std::fill(is_exc.begin(), is_exc.end(), 0);
        int64_t prev = -1;
        for (int64_t k = pf[e]; k < pf[e + 1]; ++k) {
            const uint32_t x = s->exceptions[k];
            const int64_t pos = x >> 8;
            if (pos <= prev || pos >= P) return CSF_E_CORRUPT;
            prev = pos;
            if (unsigned(x & 0xffu) - base[pos / C] < W) return CSF_E_CORRUPT;  // fits the window
            is_exc[size_t(pos)] = 1;
        }
        for (int64_t byte = 0; byte < S; ++byte) {
            const int64_t g = byte / 16, j = byte % 16;
            for (int f = 0; f < 8 / w; ++f) {
                const int64_t p = g * G + 16 * f + j;
                const unsigned field = (unsigned(seg[byte]) >> (w * f)) & (W - 1);
                if (field == 0) continue;
                if (p >= P || is_exc[size_t(p)]) return CSF_E_CORRUPT;  // must be zero
                if (base[p / C] + field > 255u) return CSF_E_CORRUPT;    // would wrap
            }
        }
    }
    if (s->tile_index != nullptr) {
        const int64_t NT = index_tiles(s->rows, s->cols);
        std::vector<int32_t> want(static_cast<size_t>(NT));
        for (int32_t e = 0; e < s->num_experts; ++e) {
            index_expert(s->exceptions, pf[e], pf[e + 1], NT, want.data());
            for (int64_t j = 0; j < NT; ++j)
                if (s->tile_index[e * NT + j] != want[size_t(j)]) return CSF_E_CORRUPT;
        }
        if (s->tile_index[int64_t(s->num_experts) * NT] != s->num_exceptions) return CSF_E_CORRUPT;
    }
    return CSF_OK;
}

}  // namespace

extern "C" {

int csf_abi_version(void) { return CSF_ABI_VERSION; }

const char *csf_status_str(csf_status s) {
    switch (s) {
        case CSF_OK: return "ok";
        case CSF_E_NULL: return "a required pointer is NULL";
        case CSF_E_SHAPE: return "bad shape (E, R, C must be positive, R*C < 2^24, E <= CSF_MAX_EXPERTS)";
        case CSF_E_FORMAT: return "unknown format";
        case CSF_E_SIZE: return "stride, exception count or pass selection inconsistent";
        case CSF_E_ALIGN:
            return "misaligned buffer (offsets and weights need 16 bytes; exceptions, prefix, index, x, alpha, y 4; "
                   "expert_start its element size; dense NVFP4 scales 2)";
        case CSF_E_CORRUPT: return "compressed stream breaks the layout";
        case CSF_E_MISMATCH: return "paired stacks have different expert counts";
        case CSF_E_HIP: return "HIP runtime refused the launch";
    }
    return "unknown status";
}

csf_status csf_prepare(int32_t format, int32_t num_experts, int32_t rows, int32_t cols,
                       const uint8_t *dense_host, csf_sizes *out_sizes, uint8_t *bases,
                       uint8_t *offsets, uint32_t *exceptions, int32_t *exc_prefix,
                       int32_t *tile_index) {
    try {
        return prepare_impl(format, num_experts, rows, cols, dense_host, out_sizes, bases, offsets,
                            exceptions, exc_prefix, tile_index);
    } catch (...) {
        return CSF_E_SIZE;  // allocation failure in the host encoder
    }
}

csf_status csf_encode_device(int32_t format, int32_t num_experts, int32_t rows, int32_t cols,
                             const uint8_t *dense, uint8_t *bases, uint8_t *offsets,
                             uint32_t *exceptions, int32_t *exc_prefix, int32_t *tile_index,
                             uint32_t phase, void *hip_stream) {
    try {
        return encode_device_impl(format, num_experts, rows, cols, dense, bases, offsets, exceptions,
                                  exc_prefix, tile_index, phase, hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_build_index(const csf_stack *compressed, int32_t *tile_index, void *hip_stream) {
    try {
        return build_index_impl(compressed, tile_index, hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode(const csf_stack *compressed, uint8_t *workspace, const int32_t *expert_start,
                      void *hip_stream) {
    try {
        return enqueue(compressed, workspace, nullptr, nullptr, nullptr, nullptr, expert_start, false, CSF_PASS_ALL,
                       hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode_paired(const csf_stack *gate_up, uint8_t *ws_gate_up, const csf_stack *down,
                             uint8_t *ws_down, const int32_t *expert_start, void *hip_stream) {
    if (down == nullptr) return CSF_E_NULL;
    try {
        return enqueue(gate_up, ws_gate_up, nullptr, down, ws_down, nullptr, expert_start, false, CSF_PASS_ALL,
                       hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode_passes(const csf_stack *first, uint8_t *ws_first, const csf_stack *second,
                             uint8_t *ws_second, const int32_t *expert_start, uint32_t passes,
                             void *hip_stream) {
    try {
        return enqueue(first, ws_first, nullptr, second, second ? ws_second : nullptr, nullptr, expert_start,
                       false, passes,
                       hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode_i64(const csf_stack *first, uint8_t *ws_first, const csf_stack *second,
                          uint8_t *ws_second, const int64_t *expert_start, void *hip_stream) {
    try {
        return enqueue(first, ws_first, nullptr, second, second ? ws_second : nullptr, nullptr, expert_start,
                       true,
                       CSF_PASS_ALL, hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode_rows(const csf_stack *first, uint8_t *ws_first, const csf_rows *rows_first,
                           const csf_stack *second, uint8_t *ws_second, const csf_rows *rows_second,
                           const int32_t *expert_start, uint32_t passes, void *hip_stream) {
    try {
        return enqueue(first, ws_first, rows_first, second, second ? ws_second : nullptr,
                       second ? rows_second : nullptr, expert_start, false, passes, hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_moe_w4a16(const csf_stack *scales, const uint8_t *dense_scales, const uint8_t *weights,
                         const uint16_t *x, int32_t num_tokens, const float *alpha,
                         const int32_t *expert_start, float *y, void *hip_stream) {
    try {
        return moe_impl(scales, dense_scales, weights, x, num_tokens, alpha, expert_start, y, hip_stream);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_decode_traced(const csf_stack *first, uint8_t *ws_first, const csf_stack *second,
                             uint8_t *ws_second, const int32_t *expert_start, uint64_t *stamps,
                             uint64_t capacity, uint32_t *groups, void *hip_stream) {
    if (expert_start == nullptr || groups == nullptr) return CSF_E_NULL;
    const Trace trace{stamps, capacity, groups};
    try {
        return enqueue(first, ws_first, nullptr, second, second ? ws_second : nullptr, nullptr, expert_start,
                       false, CSF_PASS_ALL, hip_stream, &trace);
    } catch (...) {
        return CSF_E_HIP;
    }
}

csf_status csf_validate(const csf_stack *host_copy) {
    try {
        return validate_impl(host_copy);
    } catch (...) {
        return CSF_E_SIZE;
    }
}

}  // extern "C"
