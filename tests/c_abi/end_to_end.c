/*
 * The library driven from plain C, with no Python and no PyTorch: device
 * memory, copies and the stream come from the HIP runtime, every call goes
 * through include/mxmoe.h, and every output is compared byte for byte with
 * the CPU oracle (oracle/oracle.c, linked as test infrastructure).
 *
 * Per case: mx_prepare_moe_input -> mx_dispatch_rows ->
 * mx_apply_shuffle_mul_sum, then mx_prepare_dispatch and
 * mx_prepare_moe_input_noalloc on the same ids.  The cases reach each
 * routing path (one workgroup, one launch per tile, two launches), both id
 * widths, padded and unpadded segments, block-scale offsets, invalid ids,
 * bf16 and fp32 combine output, and an empty batch.
 *
 * Inputs are seeded splitmix64 draws (S. Vigna's published generator); they
 * carry none of the method's arithmetic.
 *
 * Usage: end_to_end              exit status 0 iff every case matches
 *        end_to_end --host-cost  also times each call at the decode shape
 *                                (T = 32, H = 4096, E = 256, top-8): host
 *                                time to enqueue one call, and GPU time per
 *                                call with calls back to back
 */
#define _POSIX_C_SOURCE 199309L  /* clock_gettime */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "mxmoe.h"

/* The oracle's entry points (oracle/oracle.c). */
int oracle_prepare_moe_input(const void* ids, int id_bytes, int64_t T, int32_t k, int32_t E,
                             int32_t g1_n, int32_t g1_k, int32_t g2_n, int32_t g2_k,
                             int32_t row_align, int32_t bs_align, int32_t* expert_offsets,
                             int32_t* ps1, int32_t* ps2, int32_t* input_perm, int64_t r_max,
                             int32_t* output_perm, int32_t* bs_offsets);
void oracle_shuffle_rows(const uint8_t* src, int64_t n_src, int64_t row_bytes,
                         const int32_t* dst2src, int64_t n_dst, uint8_t* dst);
void oracle_apply_shuffle_mul_sum(const void* y, int y_dtype, int64_t n_rows, const int32_t* perm,
                                  const void* factors, int f_dtype, int64_t T, int32_t k,
                                  int64_t H, void* out, int out_dtype);

static uint64_t g_state;

static uint64_t next_u64(void) {
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* A finite bf16 value of magnitude below 4 (exponent field at most 128). */
static uint16_t draw_bf16(void) {
    const uint64_t u = next_u64();
    const uint16_t sign = (uint16_t)((u >> 63) << 15);
    const uint16_t expo = (uint16_t)(100 + (u >> 8) % 29);
    return (uint16_t)(sign | (expo << 7) | (uint16_t)(u & 0x7f));
}

static int g_failures;

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call,              \
                    hipGetErrorString(e_));                                            \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

#define MX_OK_OR_DIE(call)                                                             \
    do {                                                                               \
        mx_status s_ = (call);                                                         \
        if (s_ != MX_OK) {                                                             \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call,              \
                    mx_status_string(s_));                                             \
            exit(3);                                                                   \
        }                                                                              \
    } while (0)

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

static void* host_alloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 16);
    if (!p) {
        fprintf(stderr, "out of host memory\n");
        exit(2);
    }
    return p;
}

/* Copies n bytes of device memory back and compares them with want. */
static void expect_bytes(const char* what, const char* label, const void* dev, const void* want,
                         size_t n, hipStream_t stream) {
    if (n == 0) return;
    uint8_t* got = (uint8_t*)host_alloc(n);
    HIP_OK(hipMemcpyAsync(got, dev, n, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    const uint8_t* w = (const uint8_t*)want;
    for (size_t i = 0; i < n; ++i) {
        if (got[i] != w[i]) {
            fprintf(stderr, "%s: %s differs from the oracle at byte %zu (%u, oracle %u)\n",
                    label, what, i, got[i], w[i]);
            ++g_failures;
            break;
        }
    }
    free(got);
}

typedef struct {
    const char* label;
    int64_t T;
    int32_t k, E, row_align, blockscale;
    int ids64;
    int64_t H;          /* hidden size; rows are bf16 */
    int32_t out_dtype;  /* MX_BF16 or MX_F32 */
    int invalid_per_mille;
} Case;

static void run_case(const Case* c, hipStream_t stream) {
    const int64_t T = c->T, H = c->H, n = T * c->k;
    const int32_t k = c->k, E = c->E, A = c->row_align;
    const int id_bytes = c->ids64 ? 8 : 4;
    const int32_t g1n = 2 * 512, g1k = (int32_t)H, g2n = (int32_t)H, g2k = 512;
    const int32_t bs_align = 128;
    const int64_t cap = mx_dispatch_capacity(T, k, E, A);
    const int64_t row_bytes = H * 2;
    const size_t out_elem = c->out_dtype == MX_F32 ? 4 : 2;

    /* host inputs */
    uint8_t* ids = (uint8_t*)host_alloc((size_t)n * id_bytes);
    for (int64_t i = 0; i < n; ++i) {
        const uint64_t u = next_u64();
        int64_t id = (int64_t)(u % (uint64_t)E);
        if ((int)((u >> 32) % 1000) < c->invalid_per_mille) id = (u >> 40) & 1 ? -1 : E + 3;
        if (c->ids64) memcpy(ids + i * 8, &id, 8);
        else {
            const int32_t v = (int32_t)id;
            memcpy(ids + i * 4, &v, 4);
        }
    }
    uint16_t* x = (uint16_t*)host_alloc((size_t)(T * H) * 2);
    for (int64_t i = 0; i < T * H; ++i) x[i] = draw_bf16();
    uint16_t* y = (uint16_t*)host_alloc((size_t)(cap * H) * 2);
    for (int64_t i = 0; i < cap * H; ++i) y[i] = draw_bf16();
    float* w = (float*)host_alloc((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) w[i] = (float)((next_u64() >> 40) * (1.0 / 16777216.0));

    /* the oracle */
    int32_t* o_eo = (int32_t*)host_alloc((size_t)(E + 1) * 4);
    int32_t* o_bs = (int32_t*)host_alloc((size_t)(E + 1) * 4);
    int32_t* o_ps1 = (int32_t*)host_alloc((size_t)E * 12);
    int32_t* o_ps2 = (int32_t*)host_alloc((size_t)E * 12);
    int32_t* o_inp = (int32_t*)host_alloc((size_t)cap * 4);
    int32_t* o_outp = (int32_t*)host_alloc((size_t)n * 4);
    if (oracle_prepare_moe_input(ids, id_bytes, T, k, E, g1n, g1k, g2n, g2k, A, bs_align, o_eo,
                                 o_ps1, o_ps2, o_inp, cap, o_outp,
                                 c->blockscale ? o_bs : NULL) != 0) {
        fprintf(stderr, "%s: the oracle refused the case\n", c->label);
        exit(4);
    }
    uint8_t* o_xd = (uint8_t*)host_alloc((size_t)(cap * row_bytes));
    memset(o_xd, 0xa5, (size_t)(cap * row_bytes));
    oracle_shuffle_rows((const uint8_t*)x, T, row_bytes, o_inp, cap, o_xd);
    uint8_t* o_out = (uint8_t*)host_alloc((size_t)(T * H) * out_elem);
    oracle_apply_shuffle_mul_sum(y, MX_BF16, cap, o_outp, w, MX_F32, T, k, H, o_out,
                                 c->out_dtype);

    /* device buffers */
    void* d_ids = dev_alloc((size_t)n * id_bytes);
    void* d_x = dev_alloc((size_t)(T * row_bytes));
    void* d_y = dev_alloc((size_t)(cap * row_bytes));
    void* d_w = dev_alloc((size_t)n * 4);
    int32_t* d_eo = (int32_t*)dev_alloc((size_t)(E + 1) * 4);
    int32_t* d_bs = (int32_t*)dev_alloc((size_t)(E + 1) * 4);
    int32_t* d_ps1 = (int32_t*)dev_alloc((size_t)E * 12);
    int32_t* d_ps2 = (int32_t*)dev_alloc((size_t)E * 12);
    int32_t* d_inp = (int32_t*)dev_alloc((size_t)cap * 4);
    int32_t* d_outp = (int32_t*)dev_alloc((size_t)n * 4);
    void* d_xd = dev_alloc((size_t)(cap * row_bytes));
    void* d_out = dev_alloc((size_t)(T * H) * out_elem);
    const size_t ws_bytes = mx_prepare_workspace_size(T, k, E);
    void* d_ws = dev_alloc(ws_bytes);
    HIP_OK(hipMemcpyAsync(d_ids, ids, (size_t)n * id_bytes, hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(d_x, x, (size_t)(T * row_bytes), hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(d_y, y, (size_t)(cap * row_bytes), hipMemcpyHostToDevice, stream));
    HIP_OK(hipMemcpyAsync(d_w, w, (size_t)n * 4, hipMemcpyHostToDevice, stream));
    const int32_t ids_dtype = c->ids64 ? MX_I64 : MX_I32;
    int32_t* bs_arg = c->blockscale ? d_bs : NULL;

    /* three calls */
    HIP_OK(hipMemsetAsync(d_xd, 0xa5, (size_t)(cap * row_bytes), stream));
    MX_OK_OR_DIE(mx_prepare_moe_input(d_ids, ids_dtype, T, k, E, g1n, g1k, g2n, g2k, A, d_eo,
                                      d_ps1, d_ps2, d_inp, cap, d_outp, bs_arg, bs_align, d_ws,
                                      ws_bytes, stream));
    MX_OK_OR_DIE(mx_dispatch_rows(d_x, T, k, row_bytes, d_outp, d_xd, cap, NULL, 0, NULL, stream));
    MX_OK_OR_DIE(mx_apply_shuffle_mul_sum(d_y, MX_BF16, cap, H, d_outp, d_w, MX_F32, T, k, d_out,
                                          c->out_dtype, stream));
    expect_bytes("expert_offsets", c->label, d_eo, o_eo, (size_t)(E + 1) * 4, stream);
    if (c->blockscale)
        expect_bytes("blockscale_offsets", c->label, d_bs, o_bs, (size_t)(E + 1) * 4, stream);
    expect_bytes("problem_sizes1", c->label, d_ps1, o_ps1, (size_t)E * 12, stream);
    expect_bytes("problem_sizes2", c->label, d_ps2, o_ps2, (size_t)E * 12, stream);
    expect_bytes("input_permutation", c->label, d_inp, o_inp, (size_t)cap * 4, stream);
    expect_bytes("output_permutation", c->label, d_outp, o_outp, (size_t)n * 4, stream);
    expect_bytes("dispatched rows", c->label, d_xd, o_xd, (size_t)(cap * row_bytes), stream);
    expect_bytes("combine output", c->label, d_out, o_out, (size_t)(T * H) * out_elem, stream);

    /* routing and dispatch in one call, on cleared outputs */
    HIP_OK(hipMemsetAsync(d_xd, 0xa5, (size_t)(cap * row_bytes), stream));
    HIP_OK(hipMemsetAsync(d_inp, 0, (size_t)cap * 4, stream));
    HIP_OK(hipMemsetAsync(d_outp, 0, (size_t)n * 4, stream));
    HIP_OK(hipMemsetAsync(d_eo, 0, (size_t)(E + 1) * 4, stream));
    MX_OK_OR_DIE(mx_prepare_dispatch(d_ids, ids_dtype, T, k, E, g1n, g1k, g2n, g2k, A, d_eo,
                                     d_ps1, d_ps2, d_inp, cap, d_outp, bs_arg, bs_align, d_ws,
                                     ws_bytes, d_x, row_bytes, d_xd, cap, NULL, 0, NULL, stream));
    expect_bytes("expert_offsets (prepare_dispatch)", c->label, d_eo, o_eo, (size_t)(E + 1) * 4,
                 stream);
    expect_bytes("input_permutation (prepare_dispatch)", c->label, d_inp, o_inp,
                 (size_t)cap * 4, stream);
    expect_bytes("output_permutation (prepare_dispatch)", c->label, d_outp, o_outp,
                 (size_t)n * 4, stream);
    expect_bytes("dispatched rows (prepare_dispatch)", c->label, d_xd, o_xd,
                 (size_t)(cap * row_bytes), stream);

    /* routing without a workspace */
    HIP_OK(hipMemsetAsync(d_inp, 0, (size_t)cap * 4, stream));
    HIP_OK(hipMemsetAsync(d_outp, 0, (size_t)n * 4, stream));
    MX_OK_OR_DIE(mx_prepare_moe_input_noalloc(d_ids, ids_dtype, T, k, E, g1n, g1k, g2n, g2k, A,
                                              d_eo, d_ps1, d_ps2, d_inp, cap, d_outp, bs_arg,
                                              bs_align, stream));
    expect_bytes("input_permutation (noalloc)", c->label, d_inp, o_inp, (size_t)cap * 4, stream);
    expect_bytes("output_permutation (noalloc)", c->label, d_outp, o_outp, (size_t)n * 4,
                 stream);

    HIP_OK(hipStreamSynchronize(stream));
    void* dev_bufs[] = {d_ids, d_x, d_y, d_w, d_eo, d_bs, d_ps1, d_ps2,
                        d_inp, d_outp, d_xd, d_out, d_ws};
    for (size_t i = 0; i < sizeof dev_bufs / sizeof dev_bufs[0]; ++i) HIP_OK(hipFree(dev_bufs[i]));
    void* host_bufs[] = {ids, x, y, w, o_eo, o_bs, o_ps1, o_ps2, o_inp, o_outp, o_xd, o_out};
    for (size_t i = 0; i < sizeof host_bufs / sizeof host_bufs[0]; ++i) free(host_bufs[i]);
    printf("end_to_end: %s: T=%lld k=%d E=%d row_align=%d H=%lld %s ids, %s out: %s\n",
           c->label, (long long)T, k, E, A, (long long)H, c->ids64 ? "int64" : "int32",
           c->out_dtype == MX_F32 ? "fp32" : "bf16", g_failures ? "FAILED so far" : "ok");
    fflush(stdout);
}

static double now_us(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return ts.tv_sec * 1e6 + ts.tv_nsec * 1e-3;
}

/* Host and GPU time per call of each entry point at the decode shape, with
 * `reps` calls enqueued back to back on one stream. */
static void host_cost(hipStream_t stream) {
    const int64_t T = 32, H = 4096, n = T * 8;
    const int32_t k = 8, E = 256, A = 1, reps = 2000;
    const int64_t cap = mx_dispatch_capacity(T, k, E, A), row_bytes = H * 2;
    int64_t* ids = (int64_t*)host_alloc((size_t)n * 8);
    for (int64_t i = 0; i < n; ++i) ids[i] = (int64_t)(next_u64() % (uint64_t)E);
    void* d_ids = dev_alloc((size_t)n * 8);
    HIP_OK(hipMemcpy(d_ids, ids, (size_t)n * 8, hipMemcpyHostToDevice));
    int32_t* d_eo = (int32_t*)dev_alloc((size_t)(E + 1) * 4);
    int32_t* d_inp = (int32_t*)dev_alloc((size_t)cap * 4);
    int32_t* d_outp = (int32_t*)dev_alloc((size_t)n * 4);
    void* d_x = dev_alloc((size_t)(T * row_bytes));
    void* d_xd = dev_alloc((size_t)(cap * row_bytes));
    void* d_w = dev_alloc((size_t)n * 4);
    void* d_out = dev_alloc((size_t)(T * row_bytes));
    HIP_OK(hipMemset(d_x, 0, (size_t)(T * row_bytes)));
    HIP_OK(hipMemset(d_xd, 0, (size_t)(cap * row_bytes)));
    HIP_OK(hipMemset(d_w, 0, (size_t)n * 4));
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    const char* names[] = {"mx_prepare_moe_input", "mx_dispatch_rows", "mx_apply_shuffle_mul_sum",
                           "mx_prepare_dispatch"};
    for (int call = 0; call < 4; ++call) {
        double host = 0.0, host_first = 0.0, drain = 0.0;
        float gpu_ms = 0.0f;
        for (int pass = 0; pass < 2; ++pass) {  /* the first pass warms up */
            HIP_OK(hipStreamSynchronize(stream));
            HIP_OK(hipEventRecord(e0, stream));
            const double t0 = now_us();
            for (int r = 0; r < reps; ++r) {
                mx_status st = MX_OK;
                switch (call) {
                case 0:
                    st = mx_prepare_moe_input(d_ids, MX_I64, T, k, E, 1024, (int32_t)H, (int32_t)H,
                                              512, A, d_eo, NULL, NULL, d_inp, cap, d_outp, NULL,
                                              128, NULL, 0, stream);
                    break;
                case 1:
                    st = mx_dispatch_rows(d_x, T, k, row_bytes, d_outp, d_xd, cap, NULL, 0, NULL,
                                          stream);
                    break;
                case 2:
                    st = mx_apply_shuffle_mul_sum(d_xd, MX_BF16, cap, H, d_outp, d_w, MX_F32, T,
                                                  k, d_out, MX_BF16, stream);
                    break;
                default:
                    st = mx_prepare_dispatch(d_ids, MX_I64, T, k, E, 1024, (int32_t)H,
                                             (int32_t)H, 512, A, d_eo, NULL, NULL, d_inp, cap,
                                             d_outp, NULL, 128, NULL, 0, d_x, row_bytes, d_xd,
                                             cap, NULL, 0, NULL, stream);
                    break;
                }
                if (st != MX_OK) {
                    fprintf(stderr, "%s: %s\n", names[call], mx_status_string(st));
                    exit(3);
                }
                if (r == 99) host_first = (now_us() - t0) / 100;
            }
            const double t1 = now_us();
            host = (t1 - t0) / reps;
            HIP_OK(hipEventRecord(e1, stream));
            HIP_OK(hipEventSynchronize(e1));
            drain = now_us() - t1;
            HIP_OK(hipEventElapsedTime(&gpu_ms, e0, e1));
        }
        printf("host_cost: %s: %.2f us host per call over the first 100 calls, %.2f over %d "
               "(then %.0f us until the GPU finished); %.2f us GPU per call back to back\n",
               names[call], host_first, host, reps, drain, gpu_ms * 1e3 / reps);
    }
    fflush(stdout);
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    void* bufs[] = {d_ids, d_eo, d_inp, d_outp, d_x, d_xd, d_w, d_out};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(ids);
}

int main(int argc, char** argv) {
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    g_state = 20260407u;
    const Case cases[] = {
        /* one workgroup does the routing (and, in prepare_dispatch, the rows) */
        {"decode", 32, 8, 256, 128, 1, 1, 4096, MX_BF16, 0},
        /* one launch per tile: every tile counts every pick */
        {"medium", 700, 8, 64, 16, 1, 0, 1024, MX_BF16, 20},
        /* count and scatter launches, 288 slots, fp32 output */
        {"large", 3000, 8, 288, 1, 0, 0, 7168, MX_F32, 0},
        /* many experts, top-6, padded, invalid ids */
        {"wide", 2500, 6, 1000, 8, 1, 1, 512, MX_F32, 50},
        /* nothing to route */
        {"empty", 0, 8, 256, 128, 1, 1, 4096, MX_BF16, 0},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) run_case(&cases[i], stream);
    if (argc > 1 && strcmp(argv[1], "--host-cost") == 0) host_cost(stream);
    HIP_OK(hipStreamDestroy(stream));
    if (g_failures) {
        fprintf(stderr, "end_to_end: %d comparison(s) failed\n", g_failures);
        return 1;
    }
    printf("end_to_end: every case matches the oracle\n");
    return 0;
}
