// W4A16 MoE projection with NVFP4 or MXFP4 weights on gfx950: the consumer
// of the CSF-compressed block scales.
//
// "NVFP4-CSF: expand_scales() for ahead-of-call scale expansion (canonical
// twin of #477)" (b12x PR 478), last commit message: the W4A16 MoE kernel
// reads its experts' E4M3 block scales (one per 16 weights) in compressed
// form; the scales a step of its software pipeline consumes are turned back
// into plain bytes in on-chip shared memory right before use, which spares
// small calls the separate expansion of all routed experts' scales into a
// dense buffer.  "finegrained-kernels: decode
// losslessly compressed NVFP4 scales (CSF)" (kernels-community PR 1236),
// format paragraph: NVFP4 = 4-bit (E2M1) weights and one E4M3 scale per 16
// weights.  The same pages compress MXFP4 scale planes (one UE8M0 scale per 32
// E2M1 weights, OCP Microscaling Formats v1.0) with one-bit offsets; the MXFP4
// instantiation is the same projection on those.
//
// For every expert e with routed tokens t in [expert_start[e], expert_start[e+1]):
//     y[t, n] = alpha[e] * sum_k x[t, k] * e2m1(W[e, n, k]) * e4m3(S[e, n, k / 16])     (NVFP4)
//     y[t, n] = alpha[e] * sum_k x[t, k] * e2m1(W[e, n, k]) * 2^(S[e, n, k / 32] - 127) (MXFP4)
// x bfloat16 [T][K], W two E2M1 codes per byte [E][N][K/2] (even k in the low
// nibble), y float32 [T][N].
//
// Work unit = (routed expert, 32 consecutive weight rows).  A workgroup of
// 8 waves issues every load of the unit at once, in a fixed order: the
// tile-index bounds of the rows' scale span, the expert's alpha, the span's
// offset runs and row bases (or its dense scale bytes), 32 weight bytes per
// lane and the activations of up to 64 tokens; once the index bounds are in,
// it issues the span's exception entries, so their round trip overlaps the
// bulk loads.  The scale bytes are expanded into LDS with the decoder's tile
// code and patched with the entries.  Wave w owns K in [256w, 256w + 256), two
// 128-wide chunks: per 16-row block and chunk a lane turns 32 E2M1 codes of
// one row into bfloat16 weights (NVFP4: hardware E2M1 -> f32 conversion, one
// exact multiply by the E4M3 scale, top halves packed; MXFP4: the hardware
// E2M1 -> bf16 conversion with the UE8M0 scale applied) and issues 4 MFMA 16x16x32
// bf16 steps per 16-token block.  K is permuted consistently in both operands
// (lane group q of step s holds k = chunk + 32q + 8s .. +7), which leaves the sums
// unchanged and makes every operand 16 contiguous bytes.  The operand layout
// puts 16 different tokens on every 16 consecutive lanes, so loading it
// directly splits each load into 16-byte pieces of 16 rows (about 36 GB/s per
// CU against 94 GB/s for quad-contiguous loads); instead each lane quad loads
// 64 contiguous bytes of one token row (the four steps' pieces of one lane
// group), and a 4 x 4 transpose inside the quad across the four step registers
// (two rounds of DPP quad permutes) moves every piece to its operand lane.  The waves' partial
// sums meet in LDS and are added in wave order, so the result does not depend
// on timing.  K above 2048 runs in K-tiles of 1024 (every wave one 128-wide
// chunk of each) and passes of 32 tokens: the unit's whole scale span is
// expanded into LDS once, two register buffers take turns so that K-tile
// kt + 1's codes and activations load while K-tile kt computes, and every
// wave accumulates its chunks of all K-tiles, in K order, before the waves'
// sums meet once per pass.
#include "csf_device.h"

#include <hip/hip_fp16.h>

#include <type_traits>

namespace csf {
namespace {

constexpr uint32_t kMoeRowBlocks = 2;   // 16-row MFMA row blocks per work unit
constexpr uint32_t kMoeRows = 16 * kMoeRowBlocks;
constexpr uint32_t kMoeChunk = 128;     // K per chunk (4 lane groups x 32)
constexpr uint32_t kMoeChunks = 2;      // chunks per wave
constexpr uint32_t kMoeWaveK = kMoeChunk * kMoeChunks;
constexpr uint32_t kMoeWaves = 8;       // waves per workgroup
constexpr uint32_t kMoeThreads = kMoeWaves * kWave;
constexpr uint32_t kMoeBlocks = 4;      // 16-token MFMA column blocks per pass
constexpr uint32_t kMoePass = 16 * kMoeBlocks;
constexpr uint32_t kMoeBlocksM = 2;     // K-tile path: 16-token blocks per pass (two buffers of each)
constexpr uint32_t kMoePassM = 16 * kMoeBlocksM;
constexpr uint32_t kMoeSteps = 4;       // MFMA 16x16x32 steps per 128-wide chunk
constexpr uint32_t kMoeKTile = kMoeWaves * kMoeWaveK;  // K of the single-K-tile path: one 256-wide slice per wave
constexpr uint32_t kMoeKTileM = kMoeWaves * kMoeChunk; // K per K-tile above that: one 128-wide chunk per wave
constexpr uint32_t kMoeMaxCols = 512;   // scale columns per row: K <= 8192
constexpr uint32_t kMoeStage = 4096;    // dense-scale bytes read with the unit's first loads (K <= 2048 NVFP4)
constexpr uint32_t kXcds = 8;           // MI355X: workgroups go round-robin to 8 XCDs

typedef float v2f32 __attribute__((ext_vector_type(2)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));

// E4M3 "E4M3FN" scale byte (bit 7 sign, bits 6..3 exponent with bias 7,
// bits 2..0 mantissa; exponent 0 subnormal; S.1111.111 NaN, no infinities)
// -> its float value, without branches: bits 6..0 placed at half-precision
// bits 13..7 give the value times 2^-8 (subnormals included), which the
// half -> float conversion and a multiply by 2^8 make exact.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    const float v = __half2float(__ushort_as_half((unsigned short)(((b & 0x7fu) << 7) | ((b & 0x80u) << 8)))) * 256.0f;
    return (b & 0x7fu) == 0x7fu ? __uint_as_float(0x7fc00000u) : v;
}

// bfloat16 weights of one MFMA step: the 8 E2M1 codes of a 32-bit word (byte
// j holds codes 2j in the low and 2j + 1 in the high nibble) times the scale.
// The hardware conversion gives each code's exact value (its scale operand,
// 1.0 here, acts through its exponent only, so it cannot carry an E4M3
// scale); code value x scale has at most 6 significant bits and lies in
// bfloat16's range, so the float product is exact and its top 16 bits are
// the bfloat16 weight.
__device__ __forceinline__ uint32_t pack_hi(v2f32 f, float scale) {
    return __builtin_amdgcn_perm(__float_as_uint(f.y * scale), __float_as_uint(f.x * scale), 0x07060302u);
}

__device__ __forceinline__ v8bf16 dequant8(uint32_t codes, float scale) {
    const u32x4 w = {pack_hi(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0), scale),
                     pack_hi(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1), scale),
                     pack_hi(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2), scale),
                     pack_hi(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3), scale)};
    return __builtin_bit_cast(v8bf16, w);
}

// MXFP4: a UE8M0 scale byte b (value 2^(b - 127), 0xFF NaN; OCP Microscaling
// Formats v1.0, E8M0) as the float whose exponent field is b: the hardware
// conversion below reads only that field, so byte 0 (2^-127) is passed as 0.0.
__device__ __forceinline__ float ue8m0_as_scale(uint32_t b) {
    return b == 0xffu ? __uint_as_float(0x7fc00000u) : __uint_as_float(b << 23);
}

// MXFP4 weights of one MFMA step: 8 E2M1 codes times 2^(b - 127) straight to
// bfloat16 pairs by the hardware conversion, whose scale acts through its
// exponent, exactly the UE8M0 scale (code value x power of two is exact while
// it stays in bfloat16's range).
__device__ __forceinline__ v8bf16 dequant8_mx(uint32_t codes, float scale) {
    const u32x4 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3))};
    return __builtin_bit_cast(v8bf16, w);
}

__device__ __forceinline__ uint32_t load_b32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Lane j of every quad reads lane j ^ m of the same quad: quad_perm 0x4E is
// [2, 3, 0, 1] (m = 2), 0xB1 is [1, 0, 3, 2] (m = 1).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// Exchange across one bit m of the quad lane and of the register index:
// a'[j] = hi ? b[j ^ m] : a[j], b'[j] = hi ? b[j] : a[j ^ m], hi = bit m of j.
template <int CTRL>
__device__ __forceinline__ void quad_swap(u32x4 &a, u32x4 &b, bool hi) {
    // each lane sends what its partner (the lane with the other bit) keeps of
    // the pair: a from a set lane, b from a clear one
    u32x4 t = hi ? a : b;
    t = (u32x4){quad_dpp<CTRL>(t.x), quad_dpp<CTRL>(t.y), quad_dpp<CTRL>(t.z), quad_dpp<CTRL>(t.w)};
    a = hi ? t : a;
    b = hi ? b : t;
}
// Register j of quad lane s <- register s of quad lane j (each bit of the
// register index trades places with the same bit of the quad lane).
__device__ __forceinline__ void quad_transpose(u32x4 (&r)[4], bool hi1, bool hi0) {
    quad_swap<0x4E>(r[0], r[2], hi1);
    quad_swap<0x4E>(r[1], r[3], hi1);
    quad_swap<0xB1>(r[0], r[1], hi0);
    quad_swap<0xB1>(r[2], r[3], hi0);
}
__device__ __forceinline__ u32x4 load_b128(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every range used here: reads 0

// MULTI: K > 2048, several K-tiles per unit (a separate instantiation, so the
// single K-tile code keeps its own register allocation).  MX: MXFP4 weights
// with UE8M0 scales per 32 (one-bit CSF offsets) instead of NVFP4 with E4M3
// scales per 16 (four-bit offsets).
template <bool DENSE, bool MULTI, bool MX>
__global__ __launch_bounds__(kMoeThreads) void csf_moe_w4a16_kernel(MoeArgs a) {
    constexpr uint32_t WB = MX ? 1u : 4u;       // CSF offset bits
    constexpr uint32_t GROUP = 128u / WB;       // positions per 16-byte offset group
    constexpr uint32_t BLOCK = MX ? 32u : 16u;  // weights per scale
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    __shared__ __align__(16) uint8_t s_scales[kMoeRows * kMoeMaxCols];
    __shared__ __align__(16) v4f32 s_part[kMoeWaves][kMoeRowBlocks][kMoeBlocks][kWave];
    __shared__ uint32_t s_nact;
    // dynamic LDS: row bases | expert_start copy | active list
    uint8_t *lds_bases = dyn_lds;
    int32_t *s_es = reinterpret_cast<int32_t *>(dyn_lds + a.bases_stage);
    uint16_t *act = reinterpret_cast<uint16_t *>(s_es + ((a.E + 1u + 3u) & ~3u));
    const uint32_t tid = threadIdx.x;

    // Routing: expert_start into LDS (token ranges later cost no round trip),
    // routed experts listed from that copy by wave 0.
    for (uint32_t i = tid; i <= a.E; i += kMoeThreads) s_es[i] = a.expert_start[i];
    __syncthreads();
    if (tid < kWave) {
        const uint32_t n = list_experts(static_cast<const int32_t *>(s_es), a.E, act);
        if (tid == 0) s_nact = n;
    }
    __syncthreads();
    const uint32_t total = s_nact * a.ntiles;

    const uint32_t wave = tid / kWave, lane = tid % kWave;
    const uint32_t row = lane & 15u;  // row within a row block (A) / token within a block (B)
    const uint32_t kq = lane >> 4;    // lane group: k = chunk + 32 * kq ..
    const uint32_t C = a.C, K = a.K, half_k = K / 2;
    uint32_t k0[kMoeChunks];          // this lane's 32 k of each of the wave's chunks, in a K-tile
    bool lvalid[kMoeChunks];          // (first K-tile) K is a multiple of 32: whole lane groups
#pragma unroll
    for (uint32_t c = 0; c < kMoeChunks; ++c) {
        k0[c] = wave * kMoeWaveK + c * kMoeChunk + 32u * kq;
        lvalid[c] = k0[c] < K;
    }
    // lane-constant buffer offsets of the weight and activation loads (past
    // every range where the lane has no k, so those loads read 0: k0[c] < K
    // holds for all four lanes of a quad alike)
    uint32_t woff[kMoeChunks], xraw[kMoeChunks];
    const bool qhi1 = (lane & 2u) != 0, qhi0 = (lane & 1u) != 0;  // quad lane bits
#pragma unroll
    for (uint32_t c = 0; c < kMoeChunks; ++c) {
        woff[c] = lvalid[c] ? row * half_k + k0[c] / 2u : kOutOfRange;
        // activations, load s: quad (lane / 4) % 4 takes token 4 * that + s of
        // the 16-token block, its lane j the 8 k at k0[c] + 8j (64 bytes per
        // quad); after the quad transpose, register s of lane l holds token
        // l % 16 at k0[c] + 8s, the operand layout
        xraw[c] = ((4u * ((lane >> 2) & 3u)) * K + k0[c] + 8u * (lane & 3u)) * 2u;
    }
    // K-tile path: the lane's 32 k of a K-tile, and its lane-constant weight
    // and activation offsets (as above, one chunk per wave)
    const uint32_t kwm = wave * kMoeChunk + 32u * kq;
    const uint32_t woffm = row * half_k + kwm / 2u;
    const uint32_t xrawm = ((4u * ((lane >> 2) & 3u)) * K + kwm + 8u * (lane & 3u)) * 2u;
    const uint32_t nwaves1 = min(kMoeWaves, (K + kMoeWaveK - 1u) / kMoeWaveK);  // waves with some K (one K-tile)
    const uint64_t plane = (uint64_t)a.N * C;

    // Units in XCD order: workgroup b runs on XCD b % 8, so each XCD takes a
    // contiguous range of units (the rows of few experts), and an expert's
    // activations are fetched into few L2 caches.  Any grid size stays
    // correct: without 8 | grid the units go round-robin.
    uint32_t u = blockIdx.x, ustep = gridDim.x, uend = total;
    if ((gridDim.x & (kXcds - 1u)) == 0) {
        const uint32_t per = (total + kXcds - 1u) / kXcds, x = blockIdx.x & (kXcds - 1u);
        u = x * per + blockIdx.x / kXcds;
        ustep = gridDim.x / kXcds;
        uend = min(total, (x + 1u) * per);
    }

    for (; u < uend; u += ustep) {
        const uint32_t kx = u / a.ntiles;
        const uint32_t e = __builtin_amdgcn_readfirstlane(act[kx]);
        const uint32_t n0 = (u - kx * a.ntiles) * kMoeRows;
        const uint32_t nrows = min(kMoeRows, a.N - n0);
        const int32_t s0 = s_es[e], s1 = s_es[e + 1];
        const uint32_t t0 = (uint32_t)min(max(s0, 0), (int32_t)a.T);
        const uint32_t t1 = (uint32_t)min(max(s1, (int32_t)t0), (int32_t)a.T);
        const uint32_t m = t1 - t0;
        const uint32_t q0 = n0 * C, q1 = (n0 + nrows) * C;

        // One unit with NB 16-token blocks in its first pass (more passes
        // only when m > 64, with NB = 4).  Straight-line loads per NB keep
        // every wait exact.
        auto unit = [&](auto nbc) {
            constexpr uint32_t NB = decltype(nbc)::value;
            // ---- loads, in order
            uint32_t l0 = 0, h0 = 0;
            if constexpr (!DENSE) {
                const rsrc_t rt = make_rsrc(a.st.tile_index + (uint64_t)e * a.st.index_tiles,
                                            (a.st.index_tiles + 1u) * 4u);
                l0 = load_b32(rt, 4u * (q0 / kIndexTile));
                h0 = load_b32(rt, 4u * min((q1 + kIndexTile - 1u) / kIndexTile, a.st.index_tiles));
            }
            const float alpha = __uint_as_float(load_b32(make_rsrc(a.alpha + e, 4u), 0u));
            u32x4 runs = {0u, 0u, 0u, 0u};
            // dense scales: 16-bit loads for NVFP4 (C even: every span and its
            // start are even), byte loads for MXFP4 (C = K/32 may be odd);
            // either way kDenseLoads per lane cover a single-K-tile span
            constexpr uint32_t kDenseLoads = kMoeStage / 2u / kMoeThreads;
            constexpr uint32_t DW = MX ? 1u : 2u;
            uint32_t base_byte = 0u, dense2[kDenseLoads] = {};
            if constexpr (DENSE) {
                const rsrc_t rd = make_rsrc(a.dense + (uint64_t)e * plane + q0, q1 - q0);
#pragma unroll
                for (uint32_t i = 0; i < kDenseLoads; ++i) {
                    const int off = (int)(DW * (tid + i * kMoeThreads));
                    dense2[i] = MX ? __builtin_amdgcn_raw_buffer_load_b8(rd, off, 0, 0)
                                   : __builtin_amdgcn_raw_buffer_load_b16(rd, off, 0, 0);
                }
            } else {
                // GROUP positions per 16-byte offset group
                const rsrc_t rs = make_rsrc(a.st.offsets + (uint64_t)e * a.st.stride, ((q1 + GROUP - 1u) / GROUP) * 16u);
                runs = load_b128(rs, ((q0 + kRunBytes * tid) / GROUP) * 16u);
                base_byte = __builtin_amdgcn_raw_buffer_load_b8(
                    make_rsrc(a.st.bases + (uint64_t)e * a.st.R + n0, nrows), (int)tid, 0, 0);
            }
            // One buffer resource per 16-row block and per 16-token block:
            // every load is then a lane-constant offset plus an immediate.
            // 32 codes of row rb*16 + row at k0[c] (rows past the unit's and
            // k past K read 0)
            // single K-tile: chunk c of the wave's slice in wa[.][c], xa[.][c];
            // K-tile path: K-tiles in the two buffers c = 0, 1 (double buffering)
            u32x4 wa[kMoeRowBlocks][kMoeChunks];
            u32x4 xa[NB][kMoeChunks][kMoeSteps];
            auto load_pass = [&](uint32_t tb) {
#pragma unroll
                for (uint32_t b = 0; b < NB; ++b) {
                    const uint32_t t = tb + b * 16u;
                    const uint32_t toks = m > t ? min(16u, m - t) : 0u;
                    const rsrc_t rx = make_rsrc(a.x + (uint64_t)(t0 + t) * K, toks * K * 2u);
#pragma unroll
                    for (uint32_t c = 0; c < kMoeChunks; ++c)
#pragma unroll
                        for (uint32_t s = 0; s < kMoeSteps; ++s) xa[b][c][s] = load_b128(rx, (lvalid[c] ? xraw[c] : kOutOfRange) + 2u * s * K);
                }
            };
            // K-tile path: codes and activations of K-tile kt, pass tb, into buffer CB
            auto load_kt = [&](uint32_t tb, uint32_t kt, auto cbuf) {
                constexpr uint32_t CB = decltype(cbuf)::value;
                const uint32_t kb = kt * kMoeKTileM;
                const bool v = kb + kwm < K;  // alike for the four lanes of a quad
#pragma unroll
                for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb) {
                    const uint32_t rows = nrows > rb * 16u ? min(16u, nrows - rb * 16u) : 0u;
                    const rsrc_t rw = make_rsrc(a.w + ((uint64_t)e * a.N + n0 + rb * 16u) * half_k, rows * half_k);
                    wa[rb][CB] = load_b128(rw, v ? woffm + kb / 2u : kOutOfRange);
                }
#pragma unroll
                for (uint32_t b = 0; b < NB; ++b) {
                    const uint32_t t = tb + b * 16u;
                    const uint32_t toks = m > t ? min(16u, m - t) : 0u;
                    const rsrc_t rx = make_rsrc(a.x + (uint64_t)(t0 + t) * K, toks * K * 2u);
#pragma unroll
                    for (uint32_t s = 0; s < kMoeSteps; ++s)
                        xa[b][CB][s] = load_b128(rx, v ? xrawm + 2u * kb + 2u * s * K : kOutOfRange);
                }
            };
            if constexpr (MULTI) {
                load_kt(0u, 0u, std::integral_constant<uint32_t, 0>{});
            } else {
                // 32 codes of row rb*16 + row at k0[c] (rows past the unit's
                // and k past K read 0), then the first pass's activations
#pragma unroll
                for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb) {
                    const uint32_t rows = nrows > rb * 16u ? min(16u, nrows - rb * 16u) : 0u;
                    const rsrc_t rw = make_rsrc(a.w + ((uint64_t)e * a.N + n0 + rb * 16u) * half_k, rows * half_k);
#pragma unroll
                    for (uint32_t c = 0; c < kMoeChunks; ++c) wa[rb][c] = load_b128(rw, woff[c]);
                }
                load_pass(0);
            }
            // every load above is issued before the first wait below
            __builtin_amdgcn_sched_barrier(0);

            // ---- scale bytes of the unit's rows into LDS
            if constexpr (DENSE) {
#pragma unroll
                for (uint32_t i = 0; i < kDenseLoads; ++i) {
                    const uint32_t off = DW * (tid + i * kMoeThreads);
                    if (off < q1 - q0) {
                        if constexpr (MX)
                            s_scales[off] = (uint8_t)dense2[i];
                        else
                            *reinterpret_cast<uint16_t *>(s_scales + off) = (uint16_t)dense2[i];
                    }
                }
                if constexpr (MULTI) {  // K > 2048: the rest of the span
                    const rsrc_t rd = make_rsrc(a.dense + (uint64_t)e * plane + q0, q1 - q0);
                    for (uint32_t b = kDenseLoads * kMoeThreads + tid; DW * b < q1 - q0; b += kMoeThreads) {
                        if constexpr (MX)
                            s_scales[b] = (uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rd, (int)b, 0, 0);
                        else
                            *reinterpret_cast<uint16_t *>(s_scales + 2u * b) =
                                (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rd, (int)(2u * b), 0, 0);
                    }
                }
            } else {
                // the span's exception entries, once the index bounds are in
                const int32_t l = (int32_t)__builtin_amdgcn_readfirstlane(l0);
                const int32_t h = (int32_t)__builtin_amdgcn_readfirstlane(h0);
                const uint32_t hi = h < 0 ? 0u : min((uint32_t)h, a.st.n_exc);
                const uint32_t lo = l < 0 ? 0u : min((uint32_t)l, hi);
                const uint32_t cnt = hi - lo;
                const uint32_t entry = load_b32(make_rsrc(a.st.exc + lo, min(cnt, kMoeThreads) * 4u), 4u * tid);
                if (tid < nrows) lds_bases[tid] = (uint8_t)base_byte;
                __syncthreads();
                if constexpr (!MULTI) {
                    switch (a.st.row_mode) {
                        case kRowSplat: expand_tile<WB, kRowSplat, true, 1, false>(a.st, &runs, q0, q1, q0, lds_bases, n0, s_scales, nullptr); break;
                        case kRowTwo: expand_tile<WB, kRowTwo, true, 1, false>(a.st, &runs, q0, q1, q0, lds_bases, n0, s_scales, nullptr); break;
                        default: expand_tile<WB, kRowBytes, true, 1, false>(a.st, &runs, q0, q1, q0, lds_bases, n0, s_scales, nullptr); break;
                    }
                } else {
                    // one 16-position run per thread: 8192 positions per round, the
                    // first round's offsets read with the unit's first loads
                    for (uint32_t g = 0; g * kRunBytes * kMoeThreads < q1 - q0; ++g) {
                        const uint32_t qg = q0 + g * kRunBytes * kMoeThreads;
                        if (g > 0) {  // K > 4096
                            const rsrc_t rs = make_rsrc(a.st.offsets + (uint64_t)e * a.st.stride, ((q1 + GROUP - 1u) / GROUP) * 16u);
                            runs = load_b128(rs, ((qg + kRunBytes * tid) / GROUP) * 16u);
                        }
                        uint8_t *dst = s_scales + (qg - q0);
                        switch (a.st.row_mode) {
                            case kRowSplat: expand_tile<WB, kRowSplat, true, 1, false>(a.st, &runs, qg, q1, qg, lds_bases, n0, dst, nullptr); break;
                            case kRowTwo: expand_tile<WB, kRowTwo, true, 1, false>(a.st, &runs, qg, q1, qg, lds_bases, n0, dst, nullptr); break;
                            default: expand_tile<WB, kRowBytes, true, 1, false>(a.st, &runs, qg, q1, qg, lds_bases, n0, dst, nullptr); break;
                        }
                    }
                }
                __syncthreads();
                if (tid < cnt) {
                    const uint32_t p = entry >> 8;
                    if (p >= q0 && p < q1) s_scales[p - q0] = (uint8_t)(entry & 0xffu);
                }
                for (uint32_t k = kMoeThreads + tid; k < cnt; k += kMoeThreads) {  // dense spans only
                    const uint32_t x = a.st.exc[lo + k];
                    const uint32_t p = x >> 8;
                    if (p >= q0 && p < q1) s_scales[p - q0] = (uint8_t)(x & 0xffu);
                }
            }
            __syncthreads();

            if constexpr (!MULTI) {
                // the scales of the lane's codes: blocks k0[c]/16 and k0[c]/16 + 1
                // (0 past the rows or past K, where the codes read 0)
                float sc[kMoeRowBlocks][kMoeChunks][2];
#pragma unroll
                for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb)
#pragma unroll
                    for (uint32_t c = 0; c < kMoeChunks; ++c) {
                        const uint32_t r = rb * 16u + row;
                        const bool valid = lvalid[c] && r < nrows;
                        if constexpr (MX) {  // one scale per 32 weights: the lane's 32
                            sc[rb][c][0] = valid ? ue8m0_as_scale(s_scales[r * C + k0[c] / BLOCK]) : 0.f;
                            sc[rb][c][1] = 0.f;
                        } else {
                            sc[rb][c][0] = valid ? e4m3_value(s_scales[r * C + k0[c] / BLOCK]) : 0.f;
                            sc[rb][c][1] = valid ? e4m3_value(s_scales[r * C + k0[c] / BLOCK + 1u]) : 0.f;
                        }
                    }

                for (uint32_t tb = 0; tb < m; tb += kMoePass) {
                    if (tb > 0) {
                        __syncthreads();  // the previous pass's partial sums are read
                        load_pass(tb);
                    }
                    if (wave < nwaves1) {
#pragma unroll
                        for (uint32_t b = 0; b < NB; ++b)
#pragma unroll
                            for (uint32_t c = 0; c < kMoeChunks; ++c) quad_transpose(xa[b][c], qhi1, qhi0);
#pragma unroll
                        for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb) {
                            v4f32 acc[NB];
#pragma unroll
                            for (uint32_t b = 0; b < NB; ++b) acc[b] = (v4f32){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (uint32_t c = 0; c < kMoeChunks; ++c) {
                                const uint32_t wd[4] = {wa[rb][c].x, wa[rb][c].y, wa[rb][c].z, wa[rb][c].w};
#pragma unroll
                                for (uint32_t s = 0; s < kMoeSteps; ++s) {
                                    // one step at a time: converted ahead, the weights of every
                                    // step would hold their float intermediates at once
                                    const v8bf16 aw = MX ? dequant8_mx(wd[s], sc[rb][c][0]) : dequant8(wd[s], sc[rb][c][s >> 1]);
#pragma unroll
                                    for (uint32_t b = 0; b < NB; ++b)
                                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                            aw, __builtin_bit_cast(v8bf16, xa[b][c][s]), acc[b], 0, 0, 0);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            }
#pragma unroll
                            for (uint32_t b = 0; b < NB; ++b) s_part[wave][rb][b][lane] = acc[b];
                        }
                    }
                    __syncthreads();
                    // Lane l of a wave holds rows 4*(l/16) .. +3 of token l % 16
                    // of its 16 x 16 block: one thread per such 4-row vector adds
                    // the waves' vectors in wave order and writes 4 outputs.
                    if (tid < kMoeRowBlocks * NB * kWave) {
                        const uint32_t l = tid % kWave, b = (tid / kWave) % NB, rb = tid / (kWave * NB);
                        v4f32 r = s_part[0][rb][b][l];
                        for (uint32_t w = 1; w < nwaves1; ++w) r += s_part[w][rb][b][l];
                        const uint32_t t = tb + b * 16u + l % 16u, nn = rb * 16u + 4u * (l / 16u);
                        if (t < m) {
                            float *dst = a.y + (uint64_t)(t0 + t) * a.N + n0 + nn;
                            const float rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                            for (uint32_t c = 0; c < 4; ++c)
                                if (nn + c < nrows) dst[c] = rr[c] * alpha;
                        }
                    }
                }
            } else {
                // K-tiles of kMoeKTileM, double-buffered: K-tile kt + 1 is
                // loaded while K-tile kt computes, and every wave accumulates
                // its chunks of all K-tiles in registers, in K order, so the
                // waves' sums meet once per pass.
                const uint32_t nktm = (K + kMoeKTileM - 1u) / kMoeKTileM;
                for (uint32_t tb = 0; tb < m; tb += kMoePassM) {
                    if (tb > 0) {
                        __syncthreads();  // the previous pass's partial sums are read
                        load_kt(tb, 0u, std::integral_constant<uint32_t, 0>{});
                    }
                    v4f32 acc[kMoeRowBlocks][NB];
#pragma unroll
                    for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb)
#pragma unroll
                        for (uint32_t b = 0; b < NB; ++b) acc[rb][b] = (v4f32){0.f, 0.f, 0.f, 0.f};
                    auto compute = [&](uint32_t kt, auto cbuf) {
                        constexpr uint32_t CB = decltype(cbuf)::value;
                        const uint32_t kb = kt * kMoeKTileM;
                        if (kb + wave * kMoeChunk >= K) return;  // the wave has no K in this K-tile
#pragma unroll
                        for (uint32_t b = 0; b < NB; ++b) quad_transpose(xa[b][CB], qhi1, qhi0);
#pragma unroll
                        for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb) {
                            // the scales of the lane's 32 codes (0 past the rows or
                            // past K, where the codes read 0)
                            const uint32_t r = rb * 16u + row;
                            const bool valid = kb + kwm < K && r < nrows;
                            const uint32_t i = valid ? r * C + (kb + kwm) / BLOCK : 0u;
                            float s0, s1;
                            if constexpr (MX) {
                                s0 = valid ? ue8m0_as_scale(s_scales[i]) : 0.f;
                                s1 = s0;
                            } else {
                                s0 = valid ? e4m3_value(s_scales[i]) : 0.f;
                                s1 = valid ? e4m3_value(s_scales[i + 1u]) : 0.f;
                            }
                            const uint32_t wd[4] = {wa[rb][CB].x, wa[rb][CB].y, wa[rb][CB].z, wa[rb][CB].w};
#pragma unroll
                            for (uint32_t s = 0; s < kMoeSteps; ++s) {
                                const v8bf16 aw = MX ? dequant8_mx(wd[s], s0) : dequant8(wd[s], s < 2u ? s0 : s1);
#pragma unroll
                                for (uint32_t b = 0; b < NB; ++b)
                                    acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        aw, __builtin_bit_cast(v8bf16, xa[b][CB][s]), acc[rb][b], 0, 0, 0);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                    };
                    for (uint32_t kt = 0; kt < nktm; kt += 2u) {
                        if (kt + 1u < nktm) load_kt(tb, kt + 1u, std::integral_constant<uint32_t, 1>{});
                        __builtin_amdgcn_sched_barrier(0);
                        compute(kt, std::integral_constant<uint32_t, 0>{});
                        if (kt + 1u >= nktm) break;
                        if (kt + 2u < nktm) load_kt(tb, kt + 2u, std::integral_constant<uint32_t, 0>{});
                        __builtin_amdgcn_sched_barrier(0);
                        compute(kt + 1u, std::integral_constant<uint32_t, 1>{});
                    }
#pragma unroll
                    for (uint32_t rb = 0; rb < kMoeRowBlocks; ++rb)
#pragma unroll
                        for (uint32_t b = 0; b < NB; ++b) s_part[wave][rb][b][lane] = acc[rb][b];
                    __syncthreads();
                    // Lane l of a wave holds rows 4*(l/16) .. +3 of token l % 16
                    // of its 16 x 16 block: one thread per such 4-row vector adds
                    // the waves' vectors in wave order and writes 4 outputs.
                    if (tid < kMoeRowBlocks * NB * kWave) {
                        const uint32_t l = tid % kWave, b = (tid / kWave) % NB, rb = tid / (kWave * NB);
                        v4f32 r = s_part[0][rb][b][l];
                        for (uint32_t w = 1; w < kMoeWaves; ++w) r += s_part[w][rb][b][l];
                        const uint32_t t = tb + b * 16u + l % 16u, nn = rb * 16u + 4u * (l / 16u);
                        if (t < m) {
                            float *dst = a.y + (uint64_t)(t0 + t) * a.N + n0 + nn;
                            const float rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                            for (uint32_t c = 0; c < 4; ++c)
                                if (nn + c < nrows) dst[c] = rr[c] * alpha;
                        }
                    }
                }
            }
        };
        // The next unit's first LDS writes (row bases, scale bytes) touch
        // nothing the reduction reads, and its partial sums are written only
        // after a barrier every wave passes once its reduction is done.
        if constexpr (MULTI) {
            switch ((m + 15u) / 16u) {
                case 0: break;
                case 1: unit(std::integral_constant<uint32_t, 1>{}); break;
                default: unit(std::integral_constant<uint32_t, kMoeBlocksM>{}); break;
            }
        } else {
            switch ((m + 15u) / 16u) {
                case 0: break;
                case 1: unit(std::integral_constant<uint32_t, 1>{}); break;
                case 2: unit(std::integral_constant<uint32_t, 2>{}); break;
                case 3: unit(std::integral_constant<uint32_t, 3>{}); break;
                default: unit(std::integral_constant<uint32_t, 4>{}); break;
            }
        }
    }
}

}  // namespace

size_t moe_lds_bytes(const MoeArgs &a) {
    return a.bases_stage + 4u * ((a.E + 1u + 3u) & ~3u) + ((2u * a.E + 15u) & ~15u);
}

template <bool DENSE, bool MULTI, bool MX>
static void launch_one(const MoeArgs &a, uint32_t grid, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL((csf_moe_w4a16_kernel<DENSE, MULTI, MX>), dim3(grid), dim3(kMoeThreads), lds, stream, a);
}

hipError_t launch_moe_w4a16(const MoeArgs &a, uint32_t grid, hipStream_t stream) {
    const size_t lds = moe_lds_bytes(a);
    const bool dense = a.dense != nullptr, multi = a.K > kMoeKTile, mx = a.st.wbits == 1;
    switch ((dense ? 4 : 0) + (multi ? 2 : 0) + (mx ? 1 : 0)) {
        case 0: launch_one<false, false, false>(a, grid, lds, stream); break;
        case 1: launch_one<false, false, true>(a, grid, lds, stream); break;
        case 2: launch_one<false, true, false>(a, grid, lds, stream); break;
        case 3: launch_one<false, true, true>(a, grid, lds, stream); break;
        case 4: launch_one<true, false, false>(a, grid, lds, stream); break;
        case 5: launch_one<true, false, true>(a, grid, lds, stream); break;
        case 6: launch_one<true, true, false>(a, grid, lds, stream); break;
        default: launch_one<true, true, true>(a, grid, lds, stream); break;
    }
    return hipGetLastError();
}

}  // namespace csf
