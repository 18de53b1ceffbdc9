/*
 * csf.h — C ABI of the CSF block-scale decoder for MI355X (gfx950).
 *
 * CSF ("finegrained-kernels: decode losslessly compressed NVFP4 scales (CSF)",
 * kernels-community PR 1236, format paragraph) stores the FP8 block-scale bytes
 * of stacked MoE expert projections as one base byte per row, a resident stream
 * of small offsets from that base, and an exception stream for the values the
 * offsets cannot reach; decoding gives back the original bytes exactly.
 * Offsets are 4 bits wide for NVFP4 (E4M3 scale per 16 weights) and 1 bit for
 * MXFP4 (UE8M0 scale per 32 weights), reordered for contiguous decoding
 * ("NVFP4-CSF: expand_scales() for ahead-of-call scale expansion (canonical
 * twin of #477)", b12x PR 478, commit messages).
 *
 * Layout of one compressed stack (format, E experts, R rows, C scale columns;
 * w = offset bits, G = 128 / w positions per 16-byte group, P = R * C):
 *   bases       u8[E * R]            row-major (expert, row)
 *   offsets     u8[E * stride]       stride >= 16 * ceil(P / G), multiple of 16;
 *                                    position p of expert e is byte
 *                                    e*stride + 16*(p/G) + p%16, bits
 *                                    [w*f, w*f + w) with f = (p % G) / 16
 *   exceptions  u32[n]               (p << 8) | byte, expert-major, ascending p
 *   exc_prefix  i32[E + 1]           exclusive prefix of per-expert entry counts
 *   tile_index  i32[E * NT + 1]      optional; NT = ceil(P / CSF_INDEX_TILE):
 *                                    tile_index[e*NT + j] = exc_prefix[e] +
 *                                    #{entries of e with p < j*CSF_INDEX_TILE},
 *                                    tile_index[E*NT] = n
 *   dense       u8[E][R][C]          plane e at workspace + e * P
 * Fields at exception positions and past the plane are zero.  The tile index
 * is the exception index built at preparation ("Load native FP4 experts with
 * optional lossless CSF scales", vLLM PR 964, preparation paragraphs; PR 478
 * commits on indexed reconstruction with exception lookup); it lets the
 * decoder patch every exception before the dense bytes are stored.
 *
 * Error behaviour: every function returns a csf_status; nothing aborts and no
 * C++ exception crosses this boundary.  Decode functions check their arguments
 * on the host (no device reads, no synchronisation) and launch nothing when a
 * check fails.
 */
#ifndef CSF_H
#define CSF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSF_ABI_VERSION 5

/* Positions per exception-index tile. */
#define CSF_INDEX_TILE 2048

/* Largest expert count a decode accepts (routing maps are kept on chip). */
#define CSF_MAX_EXPERTS 2048

typedef enum csf_format {
    CSF_NVFP4_E4M3 = 0,  /* 4-bit offsets, one scale per 16 weights */
    CSF_MXFP4_UE8M0 = 1  /* 1-bit offsets, one scale per 32 weights */
} csf_format;

typedef enum csf_status {
    CSF_OK = 0,
    CSF_E_NULL = 1,     /* a required pointer is NULL */
    CSF_E_SHAPE = 2,    /* E, R or C <= 0, R*C >= 2^24, or E > CSF_MAX_EXPERTS */
    CSF_E_FORMAT = 3,   /* unknown format */
    CSF_E_SIZE = 4,     /* stride or exception count inconsistent with the shape (stride below
                           16 * ceil(R * C / G), not a multiple of 16, or not below 2^31) */
    CSF_E_ALIGN = 5,    /* a buffer below its alignment: offsets and W4A16 weights 16 bytes;
                           exceptions, prefix, tile index, x, alpha, y 4; expert_start its element
                           size; dense NVFP4 scales of the W4A16 projection 2 */
    CSF_E_CORRUPT = 6,  /* csf_validate: the stream breaks the layout */
    CSF_E_MISMATCH = 7, /* paired stacks have different expert counts */
    CSF_E_HIP = 8       /* the HIP runtime refused a launch */
} csf_status;

/* Buffer sizes of one compressed stack, in bytes unless named otherwise. */
typedef struct csf_sizes {
    int64_t dense_bytes;       /* E * R * C */
    int64_t bases_bytes;       /* E * R */
    int64_t offsets_stride;    /* 16 * ceil(R * C / G) */
    int64_t offsets_bytes;     /* E * offsets_stride */
    int64_t num_exceptions;    /* entries */
    int64_t exceptions_bytes;  /* 4 * num_exceptions */
    int64_t prefix_bytes;      /* 4 * (E + 1) */
    int64_t index_tiles;       /* NT = ceil(R * C / CSF_INDEX_TILE) per expert */
    int64_t index_bytes;       /* 4 * (E * NT + 1) */
    int64_t compressed_bytes;  /* bases + offsets + exceptions + prefix + index */
} csf_sizes;

/*
 * Descriptor of one compressed stack.  The struct itself lives in host memory
 * and is copied into the kernel arguments; the pointers are device pointers.
 * exceptions may be NULL iff num_exceptions == 0.  tile_index may be NULL:
 * the decode then runs the fixed stream and the exception pass as two kernels.
 */
typedef struct csf_stack {
    int32_t format;
    int32_t num_experts;
    int32_t rows;
    int32_t cols;
    int64_t offsets_stride;
    int64_t num_exceptions;
    const uint8_t *bases;
    const uint8_t *offsets;
    const uint32_t *exceptions;
    const int32_t *exc_prefix;
    const int32_t *tile_index;
} csf_stack;

int csf_abi_version(void);
const char *csf_status_str(csf_status status);

/*
 * Encode a dense stack (PR 1236, API paragraph: the preparation helper).
 * dense_host: u8[E][R][C] in host memory.  Two-call pattern: with bases,
 * offsets, exceptions, exc_prefix and tile_index all NULL only *out_sizes is
 * filled; with bases, offsets and exc_prefix non-NULL (host buffers of at least
 * the reported sizes; exceptions may be NULL only when num_exceptions is 0)
 * the stack is encoded, and the tile index too when tile_index is non-NULL.
 * Any other mix returns CSF_E_NULL.  The output is deterministic: the base of a row
 * is the row value v with the most row values in [v, v + 2^w - 1], ties to the
 * smallest v.  Host memory only; the caller copies the buffers to the device.
 * Errors: CSF_E_FORMAT, CSF_E_SHAPE, CSF_E_NULL.
 */
csf_status csf_prepare(int32_t format, int32_t num_experts, int32_t rows, int32_t cols,
                       const uint8_t *dense_host, csf_sizes *out_sizes, uint8_t *bases,
                       uint8_t *offsets, uint32_t *exceptions, int32_t *exc_prefix,
                       int32_t *tile_index);

/* Phases of csf_encode_device. */
#define CSF_ENCODE_STREAMS 1u /* bases, offsets, exc_prefix, tile_index */
#define CSF_ENCODE_ENTRIES 2u /* exceptions */

/*
 * Encode a dense stack that is already in device memory, on the GPU ("Load
 * native FP4 experts with optional lossless CSF scales", vLLM PR 964,
 * preparation paragraphs: encoding and its index built on the GPU).  Same
 * bytes as csf_prepare for every input.  All pointers are device pointers;
 * dense is u8[E][R][C].  Two phases, so the caller can size the exception
 * buffer in between (the library allocates nothing):
 *   CSF_ENCODE_STREAMS writes bases (E*R), offsets (E*stride, 16-byte
 *     aligned, stride = 16*ceil(R*C/G)), exc_prefix (E+1) and tile_index
 *     (E*NT+1); exceptions is ignored.  Once the stream has run it,
 *     exc_prefix[E] is the entry count n.
 *   CSF_ENCODE_ENTRIES then writes the n entries to exceptions (u32[n]),
 *     reading dense, bases and tile_index from the first phase.
 * Both phases are enqueued on hip_stream and return without synchronising.
 * Errors: CSF_E_NULL, CSF_E_FORMAT, CSF_E_SHAPE, CSF_E_SIZE (E*R*C >= 2^31, or
 * a phase other than the two above), CSF_E_ALIGN, CSF_E_HIP.
 */
csf_status csf_encode_device(int32_t format, int32_t num_experts, int32_t rows, int32_t cols,
                             const uint8_t *dense, uint8_t *bases, uint8_t *offsets,
                             uint32_t *exceptions, int32_t *exc_prefix, int32_t *tile_index,
                             uint32_t phase, void *hip_stream);

/*
 * Build the tile index of a stack on the GPU from its exceptions and prefix
 * (device buffers, as in the descriptor; compressed->tile_index is ignored),
 * into device int32[E * NT + 1] at tile_index.  For streams prepared without an
 * index.  Enqueued on hip_stream; allocates nothing.  Errors as csf_decode.
 */
csf_status csf_build_index(const csf_stack *compressed, int32_t *tile_index, void *hip_stream);

/*
 * Expand a compressed stack into the dense workspace (PR 1236, API paragraph).
 * The decode runs on the GPU, into a workspace the caller owns and may reuse:
 * a fixed-stream pass, then an exception pass.  When the device-side token
 * offsets per expert (expert_start) are given, an expert without tokens is
 * skipped by both passes and its plane keeps its previous bytes; the call
 * needs no host read-back and no list of selected experts.  With expert_start
 * NULL every plane is expanded.
 *
 * workspace: device u8[E*R*C], any byte alignment (PR 1236, validation
 *   paragraph: odd-offset workspace).
 * expert_start: NULL, or device int32[E + 1]; expert e is expanded iff
 *   expert_start[e + 1] > expert_start[e].  It is read on the device only.
 * hip_stream: a hipStream_t (NULL = the null stream).  With a tile index the
 *   call enqueues one kernel that writes every dense byte once (exceptions are
 *   patched on chip); without one, the fixed-stream kernel then the exception
 *   kernel.  It returns after enqueueing; it allocates nothing, synchronises
 *   nothing and keeps no state, so it can be captured in a HIP graph.  The
 *   caller orders other users of the workspace.
 * Errors: CSF_E_NULL, CSF_E_FORMAT, CSF_E_SHAPE, CSF_E_SIZE, CSF_E_ALIGN,
 *   CSF_E_HIP (launch refused).
 */
csf_status csf_decode(const csf_stack *compressed, uint8_t *workspace,
                      const int32_t *expert_start, void *hip_stream);

/*
 * Gate/up and down stacks of the same experts in one call: each pass is a
 * single launch covering both stacks (PR 478, commit messages: the gate/up
 * and the down scales of the routed experts are expanded together, with no
 * extra streams, and unrouted experts are skipped).
 * Formats and shapes may differ between the stacks; expert counts must match
 * (CSF_E_MISMATCH).  expert_start is shared and may be NULL.  The single-pass
 * kernel is used when both stacks carry a tile index.  Otherwise as
 * csf_decode.
 */
csf_status csf_decode_paired(const csf_stack *gate_up, uint8_t *ws_gate_up,
                             const csf_stack *down, uint8_t *ws_down,
                             const int32_t *expert_start, void *hip_stream);

/*
 * csf_decode / csf_decode_paired with an int64 expert_start (int64[E + 1],
 * 8-byte aligned): the pages keep the paired decode for both routing integer
 * types (PR 478, commit messages).  second may be NULL for a single stack;
 * expert_start may be NULL (full decode).  Otherwise as csf_decode_paired.
 */
csf_status csf_decode_i64(const csf_stack *first, uint8_t *ws_first, const csf_stack *second,
                          uint8_t *ws_second, const int64_t *expert_start, void *hip_stream);

/* Pass selection for csf_decode_passes. */
#define CSF_PASS_FIXED 1u      /* base + offset expansion of every position */
#define CSF_PASS_EXCEPTIONS 2u /* exception entries overwrite their positions */
#define CSF_PASS_ALL 3u

/*
 * The two passes of the unindexed decode, selectable one at a time so a caller
 * can schedule or time them separately: CSF_PASS_FIXED enqueues the fixed
 * stream alone, CSF_PASS_EXCEPTIONS the exception pass alone (meaningful only
 * after CSF_PASS_FIXED of the same arguments, earlier in stream order; it needs
 * no tile index).  CSF_PASS_ALL is exactly csf_decode / csf_decode_paired.
 * second may be NULL (then ws_second is ignored).  passes must be a non-zero
 * subset of CSF_PASS_ALL (else CSF_E_SIZE).
 */
csf_status csf_decode_passes(const csf_stack *first, uint8_t *ws_first,
                             const csf_stack *second, uint8_t *ws_second,
                             const int32_t *expert_start, uint32_t passes,
                             void *hip_stream);

/* A window of rows [begin, end) of every plane of a stack, 0 <= begin <= end <= rows. */
typedef struct csf_rows {
    int32_t begin;
    int32_t end;
} csf_rows;

/*
 * csf_decode_passes restricted to a window of rows of each stack (PR 478,
 * commit messages: decode only the gate halves a consumer reads).  Rows
 * rows_first->begin .. rows_first->end - 1 of every expanded plane of first
 * (likewise for second) are written, in the usual dense layout; every other
 * workspace byte keeps its value, as the planes of unrouted experts do.  For
 * a gate/up stack whose planes hold the gate rows before the up rows, the
 * gate half is {0, rows / 2}.  rows_first / rows_second may be NULL (every
 * row); an empty window writes nothing for that stack.  expert_start is int32
 * [E + 1] or NULL; passes as csf_decode_passes (CSF_PASS_ALL decodes in one
 * kernel when every stack carries a tile index).
 * Errors: CSF_E_SHAPE for a window outside [0, rows]; otherwise as
 *   csf_decode_passes.
 */
csf_status csf_decode_rows(const csf_stack *first, uint8_t *ws_first, const csf_rows *rows_first,
                           const csf_stack *second, uint8_t *ws_second, const csf_rows *rows_second,
                           const int32_t *expert_start, uint32_t passes, void *hip_stream);

/*
 * W4A16 MoE projection whose block scales stay compressed: the consumer the
 * pages pair with the compressed scales ("NVFP4-CSF: expand_scales() ...",
 * b12x PR 478, last commit message: the MoE kernel keeps the E4M3 block
 * scales, one per 16 weights, compressed and expands only those a pipeline
 * step is about to use, in on-chip shared memory, so a small call needs no
 * separate dense expansion).  The same holds for the MXFP4 stack (the pages'
 * 1-bit layout: one UE8M0 scale per 32 weights).  For every expert e with
 * tokens t in [expert_start[e], expert_start[e+1]):
 *     y[t][n] = alpha[e] * sum_k x[t][k] * e2m1(W[e][n][k]) * scale(S[e][n][k/B])
 * with B = 16 and scale = e4m3 for NVFP4, B = 32 and scale(b) = 2^(b - 127)
 * (b = 255: NaN) for MXFP4.
 *
 * scales: the NVFP4 or MXFP4 stack of the projection's scales (E experts,
 *   rows = N output features, cols = K/B; K a multiple of 32, at most 8192),
 *   device buffers.  With dense_scales NULL each workgroup expands the scales
 *   of its 32 rows straight into LDS from the CSF streams (needs the tile
 *   index); otherwise the scales are read from dense_scales, u8[E][N][K/B]
 *   (for example a csf_decode workspace; 2-byte aligned for NVFP4) and the
 *   CSF streams are not read.
 * weights: u8[E][N][K/2], two E2M1 codes per byte, code k of row n in the low
 *   nibble of byte k/2 for even k, the high nibble for odd k; 16-byte aligned.
 * x: bfloat16 [num_tokens][K], tokens sorted by expert (the grouped routing).
 * alpha: float32 [E].  x, alpha, expert_start and y are 4-byte aligned.
 * expert_start: int32 [E + 1] on the device; token
 *   indices are clamped to [0, num_tokens].  y: float32 [num_tokens][N]; rows
 *   of tokens outside every expert's range are not written.  With num_tokens 0
 *   x and y may be NULL and nothing is enqueued.
 * MXFP4 weights are widened to bfloat16 with their scale applied: exact for
 *   scale bytes 2..252 and 255; with bytes 0, 1 (weights below bfloat16's
 *   normal range) or 253, 254 (weights up to 6 * 2^127, beyond its largest
 *   finite value) the result follows the hardware's conversion.  The E4M3
 *   path widens every weight exactly.  Accumulation is in float32: for
 *   exactly widened weights |y - y_exact| <= (K + 8) 2^-24 |alpha[e]|
 *   sum_k |x[t][k] w[n][k]|.
 * Enqueued on hip_stream; allocates nothing; no host synchronisation.
 * Errors: CSF_E_NULL (a required pointer, or the tile index when dense_scales is
 *   NULL), CSF_E_FORMAT (neither NVFP4 nor MXFP4), CSF_E_SHAPE (K not a
 *   multiple of 32 or above 8192, or the stack's own shape checks),
 *   CSF_E_SIZE (num_tokens < 0), CSF_E_ALIGN, CSF_E_HIP.
 */
csf_status csf_moe_w4a16(const csf_stack *scales, const uint8_t *dense_scales, const uint8_t *weights,
                         const uint16_t *x, int32_t num_tokens, const float *alpha,
                         const int32_t *expert_start, float *y, void *hip_stream);

/*
 * Routed csf_decode_paired with timestamps, to show where the time of a
 * routed call goes (PR 1236, measurements paragraph, times the decode of the
 * routed experts' scales alone).  Decodes exactly as csf_decode_paired with
 * a non-NULL int32 expert_start (second may be NULL for one stack); both
 * stacks need a tile index.  Each workgroup also writes, from the GPU's
 * constant-rate clock (s_memrealtime, 100 MHz on MI355X), eight words to
 * stamps[8 g .. 8 g + 7] (g = workgroup):
 *   0 start;  1 routing read (expert_start loaded, active experts counted);
 *   2 the tile's loads complete (offsets, row bases and tile-index bounds,
 *   then the tile's first 1024 exception entries);  3 tile expanded in LDS;
 *   4 exceptions patched;  5 stores issued;  6 stores complete;  7 a tag:
 *   0 = no tile for this workgroup, 1 + u = tile u (plus 2^32 when the tile
 *   has more entries than those first ones), all ones = more tiles than
 *   workgroups (the pipelined loop ran).  Steps a workgroup does not reach
 *   read 0.
 * The waits before steps 2 and 6 make the traced call a little slower than
 * the untraced one.  Two-call pattern: with stamps NULL, *groups receives the
 * number of workgroups the call launches and nothing is enqueued; otherwise
 * capacity (words) must be at least 8 * that number.
 * Errors: CSF_E_NULL (expert_start, groups, or a tile index missing),
 *   CSF_E_SIZE (capacity), otherwise as csf_decode_paired.
 */
csf_status csf_decode_traced(const csf_stack *first, uint8_t *ws_first, const csf_stack *second,
                             uint8_t *ws_second, const int32_t *expert_start, uint64_t *stamps,
                             uint64_t capacity, uint32_t *groups, void *hip_stream);

/*
 * Full host-side check of a stack whose buffers are in HOST memory: prefix
 * starts at 0, is non-decreasing and ends at num_exceptions; entries ascend
 * strictly within each expert and stay inside the plane; no entry byte lies in
 * its row's offset window; offset fields past the plane and at exception
 * positions are zero, and no field makes base + field exceed 255; the tile
 * index, when present, equals the one the entries define.  The prefix is
 * checked whole before any entry is read, so a corrupt prefix never sends a
 * read past entry num_exceptions - 1.  Returns CSF_E_CORRUPT on a violation.
 * Not called by the decoder, which never reads device memory from the host.
 */
csf_status csf_validate(const csf_stack *host_copy);

#ifdef __cplusplus
}
#endif

#endif /* CSF_H */
