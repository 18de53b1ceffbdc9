// W4A16 MoE projection with NVFP4 weights on gfx950: the consumer of the
// CSF-compressed block scales.
//
// "NVFP4-CSF: expand_scales() for ahead-of-call scale expansion (canonical
// twin of #477)" (b12x PR 478), last commit message: packed W4A16 experts keep
// their E4M3 scales (one per 16 weights) as compressed storage and each
// pipeline stage of the MoE GEMM rebuilds the scales it needs in shared memory
// from that storage, so small calls no longer expand every routed expert's
// scales into a dense scratch before the MoE.  "finegrained-kernels: decode
// losslessly compressed NVFP4 scales (CSF)" (kernels-community PR 1236),
// format paragraph: NVFP4 = 4-bit (E2M1) weights and one E4M3 scale per 16
// weights.
//
// For every expert e with routed tokens t in [expert_start[e], expert_start[e+1]):
//     y[t, n] = alpha[e] * sum_k x[t, k] * e2m1(W[e, n, k]) * e4m3(S[e, n, k / 16])
// x bfloat16 [T][K], W two E2M1 codes per byte [E][N][K/2] (even k in the low
// nibble), y float32 [T][N].
//
// Work unit = (routed expert, 16 consecutive weight rows).  The workgroup
// first brings the 16 x K/16 scale bytes of its rows into LDS: straight from
// the CSF streams (the rows are one contiguous span of scale positions,
// expanded with the decoder's tile code and patched with the span's
// exception entries found through the tile index), or, for comparison, from a
// dense scale workspace.  Its 4 waves then split K in 128-wide chunks: per
// chunk a lane loads 32 E2M1 codes of one row (16 bytes) and the matching 32
// bfloat16 activations of one token (64 bytes), turns the codes into bfloat16
// weights (code value x scale is exact in bfloat16) and issues 8 MFMA
// 16x16x16 bf16 steps per 16-token block.  K is permuted consistently in
// both operands (lane group q of an MFMA step holds k = chunk + 32q + 4s ..
// +3), which leaves the sums unchanged and lets every load be 16 contiguous
// bytes.  The four waves' partial sums meet in LDS and wave 0 writes y.
#include "csf_device.h"

namespace csf {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMoeRows = 16;      // weight rows per work unit (one MFMA row block)
constexpr uint32_t kMoeTokens = 64;    // tokens per pass (four 16-token MFMA column blocks)
constexpr uint32_t kMoeChunk = 128;    // K per wave step (4 lane groups x 32)
constexpr uint32_t kMoeMaxCols = 256;  // scale columns per row (K <= 4096)

// E4M3 ("E4M3FN") byte -> float: sign, 4-bit exponent with bias 7, 3-bit
// mantissa; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t em = b & 0x7fu;
    float mag = em >= 0x08u ? __uint_as_float((((em >> 3) + 120u) << 23) | ((em & 7u) << 20))
                            : (float)em * 0x1p-9f;
    if (em == 0x7fu) mag = __uint_as_float(0x7fc00000u);
    return __uint_as_float(__float_as_uint(mag) | ((b & 0x80u) << 24));
}

// E2M1 code -> float: sign bit 3, 2-bit exponent with bias 1, 1-bit mantissa;
// exponent 0 is subnormal (m * 0.5).  Values 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t mag = c & 7u;
    const float v = mag < 2u ? 0.5f * (float)mag
                             : __uint_as_float((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22));
    return (c & 8u) ? -v : v;
}

// bfloat16 pattern of code * scale (the product has at most 6 significant
// bits and lies in bfloat16's range, so dropping the low 16 bits is exact).
__device__ __forceinline__ uint32_t dequant_bf16(uint32_t code, float scale) {
    return __float_as_uint(e2m1_to_f32(code) * scale) >> 16;
}

// The scale bytes of rows n0 .. n0+nrows-1 of expert e (positions q0 .. q1-1
// of its plane) into LDS, expanded from the CSF streams: one 16-position run
// per lane, row bases staged in LDS, then the span's exception entries.
__device__ void span_scales_from_csf(const StackArgs &st, uint32_t e, uint32_t q0, uint32_t q1,
                                     uint8_t *lds_bases, uint8_t *tile) {
    const u32x4 *seg = reinterpret_cast<const u32x4 *>(st.offsets + (uint64_t)e * st.stride);
    const uint32_t pos = q0 + kRunBytes * threadIdx.x;
    u32x4 v[1];
    v[0] = pos < q1 ? seg[pos >> 5] : (u32x4){0u, 0u, 0u, 0u};  // NVFP4: 32 positions per group
    const uint32_t r_lo = div_exact(q0, st.rcp_cols);
    const uint32_t nrows = div_exact(q1 - 1u, st.rcp_cols) - r_lo + 1u;
    const uint8_t *brow = st.bases + (uint64_t)e * st.R + r_lo;
    for (uint32_t r = threadIdx.x; r < nrows; r += kBlock) lds_bases[r] = brow[r];
    // entry range of the span from the tile index
    const int32_t *ti = st.tile_index + (uint64_t)e * st.index_tiles;
    const uint32_t i1 = min((q1 + kIndexTile - 1u) / kIndexTile, st.index_tiles);
    const int32_t l0 = ti[q0 / kIndexTile], h0 = ti[i1];
    const uint32_t hi = h0 < 0 ? 0u : min((uint32_t)h0, st.n_exc);
    const uint32_t lo = l0 < 0 ? 0u : min((uint32_t)l0, hi);
    __syncthreads();
    expand_dispatch<true, 1, false>(st, v, q0, q1, q0, lds_bases, r_lo, tile, nullptr);
    __syncthreads();
    for (uint32_t k = lo + threadIdx.x; k < hi; k += kBlock) {
        const uint32_t x = st.exc[k];
        const uint32_t p = x >> 8;
        if (p >= q0 && p < q1) tile[p - q0] = (uint8_t)(x & 0xffu);
    }
}

template <bool DENSE>
__global__ __launch_bounds__(kBlock) void csf_moe_w4a16_kernel(MoeArgs a) {
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    __shared__ __align__(16) uint8_t s_scales[kMoeRows * kMoeMaxCols];
    __shared__ __align__(16) v4f32 s_red[3][kMoeTokens / 16][kWave];
    __shared__ uint32_t s_nact;
    uint8_t *lds_bases = dyn_lds;
    uint16_t *act = reinterpret_cast<uint16_t *>(dyn_lds + a.bases_stage);
    uint8_t *flags = dyn_lds + a.bases_stage + ((2u * a.E + 15u) & ~15u);

    // Routed experts, listed in LDS by wave 0.
    stage_flags(a.expert_start, a.E, threadIdx.x, kBlock, flags);
    __syncthreads();
    if (threadIdx.x < kWave) {
        const uint32_t n = build_maps(flags, a.E, act, 0, nullptr, nullptr, 0, 0, nullptr, nullptr);
        if (threadIdx.x == 0) s_nact = n;
    }
    __syncthreads();
    const uint32_t nact = s_nact;
    const uint32_t total = nact * a.ntiles;

    const uint32_t wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint32_t row = lane & 15u;  // weight row within the unit (A) / token within a block (B)
    const uint32_t kq = lane >> 4;    // lane group: k = chunk + 32 * kq ..
    const uint32_t C = a.C, K = a.K, half_k = K / 2;
    const uint32_t nchunks = (K + kMoeChunk - 1) / kMoeChunk;
    const uint64_t plane = (uint64_t)a.N * C;

    for (uint32_t u = blockIdx.x; u < total; u += gridDim.x) {
        const uint32_t kx = u / a.ntiles;
        const uint32_t e = __builtin_amdgcn_readfirstlane(act[kx]);
        const uint32_t n0 = (u - kx * a.ntiles) * kMoeRows;
        const uint32_t nrows = min(kMoeRows, a.N - n0);
        const int32_t s0 = a.expert_start[e], s1 = a.expert_start[e + 1];
        const uint32_t t0 = (uint32_t)min(max(s0, 0), (int32_t)a.T);
        const uint32_t t1 = (uint32_t)min(max(s1, (int32_t)t0), (int32_t)a.T);
        const uint32_t m = t1 - t0;

        // 1. this unit's 16 x C scale bytes into LDS
        const uint32_t q0 = n0 * C, q1 = (n0 + nrows) * C;
        if constexpr (DENSE) {
            const uint8_t *src = a.dense + (uint64_t)e * plane + q0;
            for (uint32_t b = threadIdx.x; b < q1 - q0; b += kBlock) s_scales[b] = src[b];
        } else {
            span_scales_from_csf(a.st, e, q0, q1, lds_bases, s_scales);
        }
        __syncthreads();

        const rsrc_t rw = make_rsrc(a.w + ((uint64_t)e * a.N + n0) * half_k, nrows * half_k);
        const float alpha = a.alpha[e];
        for (uint32_t tb0 = 0; tb0 < m; tb0 += kMoeTokens) {
            const uint32_t mt = min(kMoeTokens, m - tb0);
            const uint32_t nblk = (mt + 15u) / 16u;
            const rsrc_t rx = make_rsrc(a.x + (uint64_t)(t0 + tb0) * K, mt * K * 2u);
            v4f32 acc[kMoeTokens / 16];
#pragma unroll
            for (uint32_t b = 0; b < kMoeTokens / 16; ++b) acc[b] = (v4f32){0.f, 0.f, 0.f, 0.f};

            for (uint32_t ch = wave; ch < nchunks; ch += kBlock / kWave) {
                const uint32_t k0 = ch * kMoeChunk + 32u * kq;
                const bool valid = k0 < K && row < nrows;
                // 32 codes of weight row `row`, k0 .. k0+31, and their two scales
                u32x4 wa = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(row * half_k + k0 / 2u), 0, 0));
                float sc0 = 0.f, sc1 = 0.f;
                if (valid) {
                    sc0 = e4m3_to_f32(s_scales[row * C + k0 / 16u]);
                    sc1 = e4m3_to_f32(s_scales[row * C + k0 / 16u + 1u]);
                } else {
                    wa = (u32x4){0u, 0u, 0u, 0u};
                }
                // bfloat16 weights: step s takes codes 4s .. 4s+3 (bytes 2s, 2s+1)
                v4i16 aw[8];
                const uint32_t wd[4] = {wa.x, wa.y, wa.z, wa.w};
#pragma unroll
                for (uint32_t s = 0; s < 8; ++s) {
                    const uint32_t bits = wd[s >> 1] >> (16u * (s & 1u));  // 4 codes of step s
                    const float sc = s < 4 ? sc0 : sc1;
                    aw[s] = (v4i16){(short)dequant_bf16(bits & 15u, sc), (short)dequant_bf16((bits >> 4) & 15u, sc),
                                    (short)dequant_bf16((bits >> 8) & 15u, sc),
                                    (short)dequant_bf16((bits >> 12) & 15u, sc)};
                }
#pragma unroll
                for (uint32_t b = 0; b < kMoeTokens / 16; ++b) {
                    if (b >= nblk) break;
                    // 32 activations of token b*16 + row, k0 .. k0+31 (64 bytes)
                    const uint32_t off = ((b * 16u + row) * K + k0) * 2u;
                    u32x4 xa[4];
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q) {
                        xa[q] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16u * q), 0, 0));
                        if (!(k0 < K)) xa[q] = (u32x4){0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (uint32_t s = 0; s < 8; ++s) {
                        const u32x4 q = xa[s >> 1];
                        const uint32_t lo = (s & 1u) ? q.z : q.x, hi = (s & 1u) ? q.w : q.y;
                        const v4i16 bx = (v4i16){(short)(lo & 0xffffu), (short)(lo >> 16), (short)(hi & 0xffffu),
                                                 (short)(hi >> 16)};
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aw[s], bx, acc[b], 0, 0, 0);
                    }
                }
            }

            // 2. sum the four waves' partial sums; wave 0 writes y
            if (wave > 0) {
#pragma unroll
                for (uint32_t b = 0; b < kMoeTokens / 16; ++b) s_red[wave - 1][b][lane] = acc[b];
            }
            __syncthreads();
            if (wave == 0) {
                const uint32_t nq = n0 + 4u * kq;  // output rows nq .. nq+3 of token b*16 + row
#pragma unroll
                for (uint32_t b = 0; b < kMoeTokens / 16; ++b) {
                    const uint32_t tok = b * 16u + row;
                    if (tok >= mt) continue;
                    v4f32 r = acc[b] + s_red[0][b][lane] + s_red[1][b][lane] + s_red[2][b][lane];
                    r *= alpha;
                    float *dst = a.y + (uint64_t)(t0 + tb0 + tok) * a.N + nq;
                    if (nq + 4u <= a.N && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
                        *reinterpret_cast<v4f32 *>(dst) = r;
                    } else {
                        const float rr[4] = {r.x, r.y, r.z, r.w};
                        for (uint32_t i = 0; i < 4; ++i)
                            if (nq + i < a.N) dst[i] = rr[i];
                    }
                }
            }
            __syncthreads();  // s_red and s_scales are reused
        }
    }
}

}  // namespace

size_t moe_lds_bytes(const MoeArgs &a) { return a.bases_stage + ((2u * a.E + 15u) & ~15u) + a.E; }

hipError_t launch_moe_w4a16(const MoeArgs &a, uint32_t grid, hipStream_t stream) {
    const size_t lds = moe_lds_bytes(a);
    if (a.dense != nullptr)
        hipLaunchKernelGGL(csf_moe_w4a16_kernel<true>, dim3(grid), dim3(kBlock), lds, stream, a);
    else
        hipLaunchKernelGGL(csf_moe_w4a16_kernel<false>, dim3(grid), dim3(kBlock), lds, stream, a);
    return hipGetLastError();
}

}  // namespace csf
