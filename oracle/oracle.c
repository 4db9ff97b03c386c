/*
 * CPU oracle for MoE token dispatch and combine -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The product path never calls it and shares no
 * code, header or table with it.
 *
 * It is the plain, slow, obviously-correct definition of what the three
 * host calls of the sglang page "[jit_kernel] Add prepare_moe_input JIT
 * kernels" (section "Changes") compute:
 *
 *   prepare_moe_input   tokens per expert, the prefix sum of expert offsets,
 *                       the optional FP8 block-scale offsets, and the input
 *                       and output permutations (its kernels
 *                       compute_problem_sizes / compute_expert_offsets /
 *                       compute_expert_blockscale_offsets / compute_arg_sorts);
 *   shuffle_rows        a dtype-agnostic row gather;
 *   apply_shuffle_mul_sum  gather, scale by the top-k weight, reduce with
 *                       FP32 accumulation, cast to the output dtype.
 *
 * Readings of points the page leaves open (each is listed with its reason in
 * the design notes):
 *   - picks are flattened row-major, i = t*k + j;
 *   - a pick is valid iff 0 <= id < E; invalid picks are dropped (-1);
 *   - rows of one expert are ordered by ascending flat pick index (stable);
 *   - expert segment e occupies ceil(count_e / A) * A rows (A = row_align);
 *     block-scale offsets are the same running sum with each count rounded
 *     up to B (default 128);
 *   - input_permutation maps a dispatched row to its source token (i / k),
 *     -1 for padding and unused capacity; output_permutation maps a pick to
 *     its dispatched row;
 *   - problem sizes are [E][3] = (count_e, N, K) with N, K given;
 *   - the combine sums j = 0..k-1 in ascending order as
 *     acc = fmaf(y, w, acc) from +0.0f, then rounds to nearest-even.
 *
 * Beyond those three calls it defines, from the TensorRT-LLM page "Enable
 * CuteDSL MoE with Large EP": the in-place output memset (rows of tokens
 * with a permuted index >= 0 become zero), the tile-padded sort over a
 * window of local experts (moe_sort), and the 1 x 128 FP8 e4m3fn input
 * quantization; and the zero-fill of padding rows (padding rows are those
 * with input_permutation < 0 below the padded total).
 *
 * Parity unpinned (the pages do not fix these; each is pinned to its own
 * definition by hand-worked cases and library routines, not to the pages'
 * implementations): the N / K columns of the problem sizes, the 128-row
 * rounding of block-scale offsets, the meaning of moe_sort's tile limit and
 * row maps (TensorRT-LLM's kernel source is not available), and the FP8
 * handling of NaN and infinities.
 *
 * Built with gcc -O2 -ffp-contract=off so the compiler neither fuses nor
 * reorders the float arithmetic written here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types understood by the oracle (its own numbering). */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ---------------------------------------------------------------------- */
/* Number formats, from their definitions.                                 */
/* ---------------------------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32: widening appends 16 zero
 * bits to the significand. */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static float f16_to_f32(uint16_t h) {
    int sign = h >> 15;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    float v;
    if (ex == 0)
        v = ldexpf((float)fr, -24);                 /* zero / subnormal */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + fr), ex - 25);    /* (1.fr) * 2^(ex-15) */
    return sign ? -v : v;
}

/* binary32 -> bfloat16, round to nearest, ties to even.  The two bfloat16
 * candidates are the truncation t (toward zero) and its successor; pick the
 * nearer by comparing the discarded 16 bits against one half ulp. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);   /* quiet NaN */
    uint32_t t = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (t & 1u)))
        t += 1;                  /* magnitude up; carries into the exponent */
    return (uint16_t)t;
}

/* binary32 -> binary16, round to nearest, ties to even (rint uses the
 * default rounding mode, which is nearest-even). */
static uint16_t f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return sign | 0x7e00;
    float a = fabsf(f);
    if (a >= 65520.0f) return sign | 0x7c00;   /* at or past the midpoint 65504..65536 */
    if (a < 0x1p-14f) {                         /* subnormal range: units of 2^-24 */
        float q = rintf(a * 0x1p24f);           /* exact scaling, then round */
        return sign | (uint16_t)q;              /* q == 1024 is the smallest normal */
    }
    int e2;
    frexpf(a, &e2);                             /* a = m * 2^e2, m in [0.5, 1) */
    int ex = e2 - 1;                            /* a in [2^ex, 2^(ex+1)) */
    float q = rintf(ldexpf(a, 10 - ex));        /* significand in units of 2^-10 */
    if (q == 2048.0f) { q = 1024.0f; ex += 1; }
    if (ex > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)q - 1024));
}

static float load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case OR_F32: return ((const float*)base)[idx];
    case OR_F16: return f16_to_f32(((const uint16_t*)base)[idx]);
    default:     return bf16_to_f32(((const uint16_t*)base)[idx]);
    }
}

static void store_elem(void* base, int dtype, int64_t idx, float v) {
    switch (dtype) {
    case OR_F32: ((float*)base)[idx] = v; break;
    case OR_F16: ((uint16_t*)base)[idx] = f32_to_f16(v); break;
    default:     ((uint16_t*)base)[idx] = f32_to_bf16(v); break;
    }
}

/* Exported for the tests that pin the conversions against library routines.
 * Values cross the interface as bit patterns: a float passed through a
 * double (as Python floats are) would have its signalling NaNs quieted
 * before the conversion sees them. */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
uint16_t oracle_f32_to_bf16(uint32_t bits) { return f32_to_bf16(f32_from_bits(bits)); }
uint16_t oracle_f32_to_f16(uint32_t bits) { return f32_to_f16(f32_from_bits(bits)); }
uint32_t oracle_bf16_to_f32(uint16_t h) { return f32_bits(bf16_to_f32(h)); }
uint32_t oracle_f16_to_f32(uint16_t h) { return f32_bits(f16_to_f32(h)); }

/* ---------------------------------------------------------------------- */
/* prepare_moe_input                                                        */
/* ---------------------------------------------------------------------- */

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

static int64_t read_id(const void* ids, int id_bytes, int64_t i) {
    return id_bytes == 8 ? ((const int64_t*)ids)[i] : (int64_t)((const int32_t*)ids)[i];
}

/*
 * Returns 0 on success, -1 on bad arguments, -2 if r_max is smaller than the
 * padded row count, -3 on allocation failure.
 *
 * ids            [T*k] int32 (id_bytes 4) or int64 (id_bytes 8)
 * expert_offsets [E+1] out
 * ps1, ps2       [E*3] out or NULL: (count_e, n, k) per expert
 * input_perm     [r_max] out: dispatched row -> source token, -1 if none
 * output_perm    [T*k] out: pick -> dispatched row, -1 if dropped
 * bs_offsets     [E+1] out or NULL
 */
int oracle_prepare_moe_input(const void* ids, int id_bytes, int64_t T, int32_t k, int32_t E,
                             int32_t g1_n, int32_t g1_k, int32_t g2_n, int32_t g2_k,
                             int32_t row_align, int32_t bs_align,
                             int32_t* expert_offsets, int32_t* ps1, int32_t* ps2,
                             int32_t* input_perm, int64_t r_max, int32_t* output_perm,
                             int32_t* bs_offsets) {
    if ((id_bytes != 4 && id_bytes != 8) || T < 0 || k < 1 || E < 1 ||
        row_align < 1 || bs_align < 1)
        return -1;
    const int64_t n = T * (int64_t)k;

    /* Tokens per expert (compute_problem_sizes). */
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    if (!count || !cursor) { free(count); free(cursor); return -3; }
    for (int64_t i = 0; i < n; ++i) {
        int64_t e = read_id(ids, id_bytes, i);
        if (e >= 0 && e < E) count[e] += 1;
    }

    /* Running sums of the (rounded-up) counts (compute_expert_offsets and
     * compute_expert_blockscale_offsets). */
    int64_t off = 0, bs = 0;
    expert_offsets[0] = 0;
    if (bs_offsets) bs_offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        cursor[e] = off;
        off += round_up(count[e], row_align);
        bs += round_up(count[e], bs_align);
        expert_offsets[e + 1] = (int32_t)off;
        if (bs_offsets) bs_offsets[e + 1] = (int32_t)bs;
        if (ps1) { ps1[3 * e] = (int32_t)count[e]; ps1[3 * e + 1] = g1_n; ps1[3 * e + 2] = g1_k; }
        if (ps2) { ps2[3 * e] = (int32_t)count[e]; ps2[3 * e + 1] = g2_n; ps2[3 * e + 2] = g2_k; }
    }
    if (off > r_max) { free(count); free(cursor); return -2; }

    /* Stable counting-sort scatter (compute_arg_sorts). */
    for (int64_t r = 0; r < r_max; ++r) input_perm[r] = -1;
    for (int64_t i = 0; i < n; ++i) {
        int64_t e = read_id(ids, id_bytes, i);
        if (e >= 0 && e < E) {
            int64_t r = cursor[e]++;
            output_perm[i] = (int32_t)r;
            input_perm[r] = (int32_t)(i / k);
        } else {
            output_perm[i] = -1;
        }
    }
    free(count);
    free(cursor);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* shuffle_rows: dst[r] = src[dst2src[r]] byte for byte; rows whose source   */
/* index is outside [0, n_src) are left untouched.                           */
/* ---------------------------------------------------------------------- */

void oracle_shuffle_rows(const uint8_t* src, int64_t n_src, int64_t row_bytes,
                         const int32_t* dst2src, int64_t n_dst, uint8_t* dst) {
    for (int64_t r = 0; r < n_dst; ++r) {
        int64_t s = dst2src[r];
        if (s < 0 || s >= n_src) continue;
        for (int64_t b = 0; b < row_bytes; ++b)
            dst[r * row_bytes + b] = src[s * row_bytes + b];
    }
}

/* ---------------------------------------------------------------------- */
/* apply_shuffle_mul_sum:                                                   */
/*   out[t][h] = round( sum_j  w[t][j] * y[perm[t*k+j]][h] )                 */
/* with the sum taken in fp32 in ascending j by fused multiply-add from +0,  */
/* picks whose row is outside [0, n_rows) skipped, w = 1 when factors is     */
/* NULL.                                                                    */
/* ---------------------------------------------------------------------- */

void oracle_apply_shuffle_mul_sum(const void* y, int y_dtype, int64_t n_rows,
                                  const int32_t* perm, const void* factors, int f_dtype,
                                  int64_t T, int32_t k, int64_t H,
                                  void* out, int out_dtype) {
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                int64_t r = perm[t * k + j];
                if (r < 0 || r >= n_rows) continue;
                float w = factors ? load_elem(factors, f_dtype, t * k + j) : 1.0f;
                float v = load_elem(y, y_dtype, r * H + h);
                acc = fmaf(v, w, acc);
            }
            store_elem(out, out_dtype, t * H + h, acc);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Zeroing rows in place (the output memset of the TensorRT-LLM page        */
/* "Enable CuteDSL MoE with Large EP", walkthrough and its memset test, and */
/* the zero-filled padding rows for grouped GEMM tiles).                    */
/* ---------------------------------------------------------------------- */

/* Output row t (row_bytes bytes) becomes all zero bytes iff at least one of
 * its k picks has a permuted index >= 0; every other row is left as it is. */
void oracle_output_memset(uint8_t* out, int64_t T, int32_t k, int64_t row_bytes,
                          const int32_t* expanded_to_permuted) {
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int32_t j = 0; j < k; ++j)
            if (expanded_to_permuted[t * k + j] >= 0) any = 1;
        if (any) memset(out + t * row_bytes, 0, (size_t)row_bytes);
    }
}

/* Dispatched row r < limit becomes all zero bytes iff input_perm[r] < 0
 * (a padding row); limit = expert_offsets[E] when expert_offsets is given,
 * else n_rows.  Rows at or past the limit are left as they are. */
void oracle_zero_padding_rows(uint8_t* rows, int64_t n_rows, int64_t row_bytes,
                              const int32_t* input_perm, const int32_t* expert_offsets,
                              int32_t E) {
    int64_t limit = expert_offsets ? expert_offsets[E] : n_rows;
    if (limit > n_rows) limit = n_rows;
    for (int64_t r = 0; r < limit; ++r)
        if (input_perm[r] < 0) memset(rows + r * row_bytes, 0, (size_t)row_bytes);
}

/* ---------------------------------------------------------------------- */
/* Tile-padded sort with a local-expert window (the sort of the TensorRT-LLM */
/* page "Enable CuteDSL MoE with Large EP": its outputs                     */
/* tile_idx_to_group_idx, tile_idx_to_mn_limit, expanded_idx_to_permuted_idx,*/
/* permuted_idx_to_expanded_idx, total_num_padded_tokens,                   */
/* num_non_exiting_tiles, and its num_local_experts / local_expert_offset / */
/* tile_size parameters).                                                   */
/*                                                                          */
/* A pick i = t*k + j is local iff local_offset <= id < local_offset +      */
/* num_local (and id < E); its group is g = id - local_offset.  Local picks */
/* are sorted stably by group; group g takes ceil(count_g / tile) whole     */
/* tiles.  permuted_to_expanded[r] is the pick i of row r, -1 for padding   */
/* and unused rows; the tiles of group g hold g and the row limit           */
/* first_row(g) + count_g; unused tiles hold -1.                            */
/* Returns 0, -1 on bad arguments, -2 when capacity or max_tiles is too     */
/* small, -3 on allocation failure.                                         */
/* ---------------------------------------------------------------------- */

int oracle_moe_sort(const void* ids, int id_bytes, int64_t T, int32_t k, int32_t E,
                    int32_t local_offset, int32_t num_local, int32_t tile,
                    int32_t* expanded_to_permuted, int32_t* permuted_to_expanded,
                    int64_t capacity, int32_t* tile_group, int32_t* tile_limit,
                    int64_t max_tiles, int32_t* total_padded, int32_t* num_tiles) {
    if ((id_bytes != 4 && id_bytes != 8) || T < 0 || k < 1 || E < 1 || local_offset < 0 ||
        num_local < 1 || (int64_t)local_offset + num_local > E || tile < 1)
        return -1;
    const int64_t n = T * (int64_t)k;
    int64_t* count = (int64_t*)calloc((size_t)num_local, sizeof(int64_t));
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * ((size_t)num_local + 1));
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_local);
    if (!count || !first || !next) { free(count); free(first); free(next); return -3; }

    for (int64_t i = 0; i < n; ++i) {
        int64_t g = read_id(ids, id_bytes, i) - local_offset;
        if (g >= 0 && g < num_local) count[g] += 1;
    }
    first[0] = 0;
    for (int32_t g = 0; g < num_local; ++g)
        first[g + 1] = first[g] + (count[g] + tile - 1) / tile * tile;
    const int64_t total = first[num_local];
    if (total > capacity || total / tile > max_tiles) {
        free(count); free(first); free(next);
        return -2;
    }

    for (int64_t r = 0; r < capacity; ++r) permuted_to_expanded[r] = -1;
    for (int64_t q = 0; q < max_tiles; ++q) { tile_group[q] = -1; tile_limit[q] = -1; }
    for (int32_t g = 0; g < num_local; ++g) next[g] = first[g];
    for (int64_t i = 0; i < n; ++i) {
        int64_t g = read_id(ids, id_bytes, i) - local_offset;
        if (g >= 0 && g < num_local) {
            int64_t r = next[g]++;
            expanded_to_permuted[i] = (int32_t)r;
            permuted_to_expanded[r] = (int32_t)i;
        } else {
            expanded_to_permuted[i] = -1;
        }
    }
    for (int32_t g = 0; g < num_local; ++g)
        for (int64_t q = first[g] / tile; q < first[g + 1] / tile; ++q) {
            tile_group[q] = g;
            tile_limit[q] = (int32_t)(first[g] + count[g]);
        }
    *total_padded = (int32_t)total;
    *num_tiles = (int32_t)(total / tile);
    free(count); free(first); free(next);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* FP8 quantization of a row in 1 x block groups (the quantize_input step of */
/* the TensorRT-LLM large-EP page, and the FP8 block-scale layout of the    */
/* sglang page's blockscale offsets).  Reading: per group of `block`         */
/* consecutive elements, amax = max |x|, scale = amax / 448 (1 when amax is */
/* 0), q = e4m3fn(x / scale) rounded to nearest even and saturated at 448;  */
/* all float arithmetic in fp32 (correctly rounded division).               */
/* ---------------------------------------------------------------------- */

/* binary32 -> OCP e4m3fn (1 sign, 4 exponent bits with bias 7, 3 fraction
 * bits; largest finite 448 = 1.75 * 2^8; no infinities), round to nearest
 * even, magnitudes beyond 448 saturate to 448.  NaN maps to 0x7f. */
static uint8_t f32_to_e4m3(float f) {
    uint8_t sign = signbit(f) ? 0x80 : 0;
    if (isnan(f)) return 0x7f;
    float a = fabsf(f);
    if (a >= 448.0f) return sign | 0x7e;
    if (a < 0x1p-6f) {                           /* subnormal range: units of 2^-9 */
        float q = rintf(a * 0x1p9f);             /* 8 becomes the smallest normal  */
        return sign | (uint8_t)q;
    }
    int e2;
    frexpf(a, &e2);
    int ex = e2 - 1;                             /* a in [2^ex, 2^(ex+1)), ex >= -6 */
    float q = rintf(ldexpf(a, 3 - ex));          /* significand in units of 2^-3 */
    if (q == 16.0f) { q = 8.0f; ex += 1; }
    uint8_t code = (uint8_t)(((ex + 7) << 3) | ((int)q - 8));
    return sign | (code > 0x7e ? 0x7e : code);
}

uint8_t oracle_f32_to_e4m3(uint32_t bits) { return f32_to_e4m3(f32_from_bits(bits)); }

/* x [T][H] bf16 -> q [T][H] e4m3fn bytes and scales [T][H / block] fp32;
 * H must be a multiple of block. */
void oracle_quantize_fp8_rows(const uint16_t* x, int64_t T, int64_t H, int32_t block,
                              uint8_t* q, float* scales) {
    const int64_t groups = H / block;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g = 0; g < groups; ++g) {
            const uint16_t* xs = x + t * H + g * block;
            float amax = 0.0f;
            for (int32_t e = 0; e < block; ++e) {
                float v = fabsf(bf16_to_f32(xs[e]));
                if (v > amax) amax = v;
            }
            float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[t * groups + g] = scale;
            for (int32_t e = 0; e < block; ++e)
                q[t * H + g * block + e] = f32_to_e4m3(bf16_to_f32(xs[e]) / scale);
        }
    }
}
