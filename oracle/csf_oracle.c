/*
 * CSF block-scale codec: CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the CSF decoder computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  The product library
 * shares no code, header, table or helper with it, and never calls it.
 *
 * What the method computes (all integer, byte exact):
 *
 *   "finegrained-kernels: decode losslessly compressed NVFP4 scales (CSF)"
 *   (kernels-community PR 1236), paragraph on the format: an NVFP4 tensor has
 *   one 8-bit scale for each group of 16 weights.  The lossless CSF form keeps,
 *   per row, a single base byte; a scale within the 4-bit reach above the base
 *   is kept as its offset, any other scale goes to a separate list of
 *   (position, byte) exceptions; the decoder restores every byte unchanged.
 *
 *   "NVFP4-CSF: expand_scales() for ahead-of-call scale expansion (canonical
 *   twin of #477)" (b12x PR 478), commit messages: offsets are one bit wide for
 *   MXFP4 (UE8M0 scales, one per 32 weights) and four bits for NVFP4, measured
 *   from a row base byte; the resident offsets are reordered for contiguous
 *   decoding.
 *
 *   PR 1236, paragraph on the API: decoding runs a fixed stream and an
 *   exception pass; given the grouped-routing expert_start tensor both skip
 *   experts with no routed tokens and leave their workspace planes untouched;
 *   without it the whole stack is expanded.
 *
 * The pages leave the byte layout, the choice of base, the exception entry
 * format and the offset order open.  This oracle fixes them as follows (the
 * readings are listed with their reasons in the design notes):
 *
 *   w  = offset width in bits: 4 (NVFP4) or 1 (MXFP4);  W = 2^w
 *   P  = R*C positions per expert plane, p = r*C + c (row-major)
 *   G  = 128/w positions per 16-byte offset group
 *   S  = 16*ceil(P/G) offset bytes per expert
 *   base of a row: the row value v with the most row values in [v, v+W-1];
 *                  ties go to the smallest such v
 *   field of p:    x - base if 0 <= x - base < W, else 0 and (p<<8 | x) is an
 *                  exception entry (entries expert-major, ascending p)
 *   offset order:  position p sits in group p/G, byte p%16, bit field
 *                  (p%G)/16 (bits w*f .. w*f+w-1), so shifting one 16-byte
 *                  group right by w*f and masking each byte yields 16
 *                  consecutive positions
 *   exc_prefix:    int32[E+1], exc_prefix[e] = entries of experts < e
 *
 * No precision choices: every step is byte or integer arithmetic, and a byte
 * sum wraps modulo 256 exactly as uint8_t arithmetic does.
 *
 * Parity pins (tests/test_oracle.py): the round trip decode(encode(x)) == x,
 * an exhaustive sweep of all two-column rows against the closed form, brute
 * force base choice over every candidate byte, hand-worked offset bytes,
 * the page-printed stack sizes, and routed decodes against the poison bytes.
 */
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)

/* Offset width per format (b12x PR 478 commit: one-bit MXFP4, four-bit NVFP4). */
static int offset_bits(int fmt)
{
    if (fmt == 0) return 4; /* NVFP4, E4M3 scales */
    if (fmt == 1) return 1; /* MXFP4, UE8M0 scales */
    return 0;
}

static int shape_ok(int fmt, int E, int R, int C)
{
    if (offset_bits(fmt) == 0) return 0;
    if (E <= 0 || R <= 0 || C <= 0) return 0;
    /* An exception entry carries the plane position in 24 bits. */
    if ((int64_t)R * (int64_t)C >= ((int64_t)1 << 24)) return 0;
    return 1;
}

int oracle_offset_bits(int fmt) { return offset_bits(fmt); }

int64_t oracle_segment_bytes(int fmt, int R, int C)
{
    int w = offset_bits(fmt);
    if (w == 0) return -1;
    int64_t P = (int64_t)R * C;
    int64_t G = 128 / w;
    int64_t groups = (P + G - 1) / G;
    return 16 * groups;
}

/*
 * Step 1: one base byte per row (PR 1236, format paragraph).  For every value v
 * present in the row, count the row values in [v, v + W - 1]; the base is the
 * first v (in increasing byte order) with the largest count.
 */
int oracle_choose_bases(int fmt, int E, int R, int C, const uint8_t *x,
                        uint8_t *bases)
{
    if (!shape_ok(fmt, E, R, C)) return ORACLE_BAD_ARGS;
    int W = 1 << offset_bits(fmt);
    for (int64_t row = 0; row < (int64_t)E * R; row++) {
        const uint8_t *xr = x + row * C;
        int64_t hist[256];
        memset(hist, 0, sizeof(hist));
        for (int c = 0; c < C; c++) hist[xr[c]]++;
        int best_v = -1;
        int64_t best_count = -1;
        for (int v = 0; v < 256; v++) {
            if (hist[v] == 0) continue;
            int64_t count = 0;
            for (int u = v; u <= v + W - 1 && u <= 255; u++) count += hist[u];
            if (count > best_count) {
                best_count = count;
                best_v = v;
            }
        }
        bases[row] = (uint8_t)best_v;
    }
    return ORACLE_OK;
}

/* A value is stored as an offset iff it lies in [base, base + W - 1]. */
static int in_window(int value, int base, int W)
{
    int d = value - base;
    return d >= 0 && d < W;
}

/* Number of exception entries the given bases produce. */
int64_t oracle_count_exceptions(int fmt, int E, int R, int C, const uint8_t *x,
                                const uint8_t *bases)
{
    if (!shape_ok(fmt, E, R, C)) return ORACLE_BAD_ARGS;
    int W = 1 << offset_bits(fmt);
    int64_t n = 0;
    for (int64_t row = 0; row < (int64_t)E * R; row++)
        for (int c = 0; c < C; c++)
            if (!in_window(x[row * C + c], bases[row], W)) n++;
    return n;
}

/*
 * Steps 2-3: the resident offset stream and the exception stream for given
 * bases (PR 1236 format paragraph; PR 478 commits on offset width and on the
 * reordering for contiguous decoding).  offsets must hold E*S bytes, exc the
 * count from oracle_count_exceptions, prefix E+1 ints.
 */
int oracle_encode_streams(int fmt, int E, int R, int C, const uint8_t *x,
                          const uint8_t *bases, uint8_t *offsets,
                          uint32_t *exc, int32_t *prefix)
{
    if (!shape_ok(fmt, E, R, C)) return ORACLE_BAD_ARGS;
    int w = offset_bits(fmt);
    int W = 1 << w;
    int64_t G = 128 / w;
    int64_t P = (int64_t)R * C;
    int64_t S = oracle_segment_bytes(fmt, R, C);
    memset(offsets, 0, (size_t)(E * S));
    int64_t n = 0;
    prefix[0] = 0;
    for (int e = 0; e < E; e++) {
        for (int r = 0; r < R; r++) {
            int base = bases[(int64_t)e * R + r];
            for (int c = 0; c < C; c++) {
                int64_t p = (int64_t)r * C + c;
                int value = x[(int64_t)e * P + p];
                int field;
                if (in_window(value, base, W)) {
                    field = value - base;
                } else {
                    field = 0;
                    exc[n++] = ((uint32_t)p << 8) | (uint32_t)value;
                }
                int64_t group = p / G;
                int64_t byte_in_group = p % 16;
                int64_t field_index = (p % G) / 16;
                offsets[(int64_t)e * S + 16 * group + byte_in_group] |=
                    (uint8_t)(field << (w * field_index));
            }
        }
        prefix[e + 1] = (int32_t)n;
    }
    return ORACLE_OK;
}

/* Whole encoder: step 1 then steps 2-3. */
int oracle_encode(int fmt, int E, int R, int C, const uint8_t *x,
                  uint8_t *bases, uint8_t *offsets, uint32_t *exc,
                  int32_t *prefix)
{
    int rc = oracle_choose_bases(fmt, E, R, C, x, bases);
    if (rc != ORACLE_OK) return rc;
    return oracle_encode_streams(fmt, E, R, C, x, bases, offsets, exc, prefix);
}

/*
 * Exception index (PR 964, "Load native FP4 experts with optional lossless CSF
 * scales", paragraphs on preparation: encoding is followed by an index built
 * on the GPU; PR 478 commit messages: indexed reconstruction with exception
 * lookup).  The pages do not give its form; this build's reading: every plane
 * is cut into tiles of 2048 positions, NT = ceil(P / 2048) per expert, and
 *   tile_index[e*NT + j] = prefix[e] + #{entries of expert e with p < 2048*j}
 *   tile_index[E*NT]     = prefix[E]
 * so the entries of tile j of expert e are tile_index[e*NT + j] ..
 * tile_index[e*NT + j + 1] - 1 (the last tile of an expert ends where the next
 * expert's first tile starts).  tile_index holds E*NT + 1 ints.
 */
#define ORACLE_INDEX_TILE 2048

int64_t oracle_index_tiles(int R, int C)
{
    int64_t P = (int64_t)R * C;
    return (P + ORACLE_INDEX_TILE - 1) / ORACLE_INDEX_TILE;
}

int oracle_build_index(int E, int R, int C, const uint32_t *exc,
                       const int32_t *prefix, int32_t *tile_index)
{
    if (E <= 0 || R <= 0 || C <= 0) return ORACLE_BAD_ARGS;
    int64_t NT = oracle_index_tiles(R, C);
    for (int e = 0; e < E; e++) {
        for (int64_t j = 0; j < NT; j++) {
            int64_t below = 0;
            for (int64_t k = prefix[e]; k < prefix[e + 1]; k++)
                if ((int64_t)(exc[k] >> 8) < ORACLE_INDEX_TILE * j) below++;
            tile_index[e * NT + j] = (int32_t)(prefix[e] + below);
        }
    }
    tile_index[(int64_t)E * NT] = prefix[E];
    return ORACLE_OK;
}

/*
 * Decoder (PR 1236, API paragraph).  expert_start may be NULL: then every
 * expert is expanded.  Otherwise expert e is expanded iff
 * expert_start[e+1] > expert_start[e], and the planes of all other experts are
 * not written.  For each expanded expert: the fixed stream gives
 * base[row] + field for every position, then the expert's exception entries
 * overwrite their positions.  Entries whose position is outside the plane are
 * ignored.
 */
int oracle_decode(int fmt, int E, int R, int C, const uint8_t *bases,
                  const uint8_t *offsets, const uint32_t *exc,
                  const int32_t *prefix, const int32_t *expert_start,
                  uint8_t *ws)
{
    if (!shape_ok(fmt, E, R, C)) return ORACLE_BAD_ARGS;
    int w = offset_bits(fmt);
    int W = 1 << w;
    int64_t G = 128 / w;
    int64_t P = (int64_t)R * C;
    int64_t S = oracle_segment_bytes(fmt, R, C);
    for (int e = 0; e < E; e++) {
        if (expert_start != NULL && !(expert_start[e + 1] > expert_start[e]))
            continue;
        /* fixed stream */
        for (int64_t p = 0; p < P; p++) {
            int64_t r = p / C;
            int64_t group = p / G;
            int64_t byte_in_group = p % 16;
            int64_t field_index = (p % G) / 16;
            int byte = offsets[(int64_t)e * S + 16 * group + byte_in_group];
            int field = (byte >> (w * field_index)) & (W - 1);
            ws[(int64_t)e * P + p] = (uint8_t)(bases[(int64_t)e * R + r] + field);
        }
        /* exception pass */
        for (int64_t k = prefix[e]; k < prefix[e + 1]; k++) {
            int64_t pos = exc[k] >> 8;
            if (pos < P) ws[(int64_t)e * P + pos] = (uint8_t)(exc[k] & 0xFF);
        }
    }
    return ORACLE_OK;
}

/*
 * Row-window decoder ("NVFP4-CSF: expand_scales() ..." b12x PR 478, commit
 * messages: decode only the gate halves a consumer reads).  Reading: the
 * consumer reads rows row_begin .. row_end-1 of every plane; exactly those
 * rows of each expanded plane are written, in the usual dense layout, and
 * every other byte of the workspace keeps its value, as the planes of
 * unrouted experts do.  Routing as oracle_decode.  The fixed stream writes
 * base[row] + field for the positions of those rows; an exception entry is
 * applied when its position lies in one of those rows.
 */
int oracle_decode_rows(int fmt, int E, int R, int C, const uint8_t *bases,
                       const uint8_t *offsets, const uint32_t *exc,
                       const int32_t *prefix, const int32_t *expert_start,
                       int row_begin, int row_end, uint8_t *ws)
{
    if (!shape_ok(fmt, E, R, C)) return ORACLE_BAD_ARGS;
    if (row_begin < 0 || row_begin > row_end || row_end > R) return ORACLE_BAD_ARGS;
    int w = offset_bits(fmt);
    int W = 1 << w;
    int64_t G = 128 / w;
    int64_t P = (int64_t)R * C;
    int64_t S = oracle_segment_bytes(fmt, R, C);
    for (int e = 0; e < E; e++) {
        if (expert_start != NULL && !(expert_start[e + 1] > expert_start[e]))
            continue;
        /* fixed stream, rows of the window */
        for (int64_t r = row_begin; r < row_end; r++) {
            for (int64_t c = 0; c < C; c++) {
                int64_t p = r * C + c;
                int64_t group = p / G;
                int64_t byte_in_group = p % 16;
                int64_t field_index = (p % G) / 16;
                int byte = offsets[(int64_t)e * S + 16 * group + byte_in_group];
                int field = (byte >> (w * field_index)) & (W - 1);
                ws[(int64_t)e * P + p] = (uint8_t)(bases[(int64_t)e * R + r] + field);
            }
        }
        /* exception pass, entries of the window's rows */
        for (int64_t k = prefix[e]; k < prefix[e + 1]; k++) {
            int64_t pos = exc[k] >> 8;
            int64_t row = pos / C;
            if (pos < P && row >= row_begin && row < row_end)
                ws[(int64_t)e * P + pos] = (uint8_t)(exc[k] & 0xFF);
        }
    }
    return ORACLE_OK;
}
