/*
 * abi_driver.c -- a plain C program that drives libsb through include/sb.h
 * and the HIP runtime alone (no Python, no torch), for the GPU test that
 * checks the library as a standalone C ABI (tests/test_gpu_abi_driver.py).
 *
 *   abi_driver DIR
 *
 * DIR/head.txt holds "B H V k off_0 ... off_k"; DIR/x.bin the hidden rows
 * (B x H bf16 bit patterns, uint16, row-major) and DIR/w.bin the head weight
 * (H x V, uint16, row-major).  The program puts x at a row stride rounded up
 * to 8 elements and every lane in an allocation of its own at one common row
 * stride, runs every call on one stream, and writes to DIR:
 *   ids_tok.bin, ids_static.bin, ids_lp.bin, ids_r0.bin  int32 [B]
 *   lane_ids.bin int32 [B][k], lane_max.bin float [B][k]
 *   lse.bin, sel.bin float [B], lp.bin float [B][V], logits.bin float [B][V]
 * It also checks that three invalid calls are refused with the documented
 * status before anything is enqueued.  Exit status 0 on success; otherwise
 * the failing step is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sb.h"

#define CHECK_HIP(call)                                                        \
    do {                                                                       \
        hipError_t e_ = (call);                                                \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));  \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

#define CHECK_SB(call)                                                         \
    do {                                                                       \
        sb_status s_ = (call);                                                 \
        if (s_ != SB_OK) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #call, sb_status_string(s_));   \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(1);
    }
    void *p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short read of %s\n", path);
        exit(1);
    }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(1);
    }
    fclose(f);
}

/* Copy a device buffer of `bytes` to DIR/name. */
static void dump(const char *dir, const char *name, const void *dev, size_t bytes)
{
    void *h = malloc(bytes ? bytes : 1);
    if (!h)
        exit(1);
    CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    write_file(dir, name, h, bytes);
    free(h);
}

/* Copy a [rows][ld] fp32 device matrix's first `cols` columns to DIR/name. */
static void dump_rows(const char *dir, const char *name, const float *dev, int rows,
                      int64_t ld, int cols)
{
    float *h = (float *)malloc((size_t)rows * (size_t)cols * sizeof(float) + 1);
    if (!h)
        exit(1);
    CHECK_HIP(hipMemcpy2D(h, (size_t)cols * sizeof(float), dev, (size_t)ld * sizeof(float),
                          (size_t)cols * sizeof(float), (size_t)rows, hipMemcpyDeviceToHost));
    write_file(dir, name, h, (size_t)rows * (size_t)cols * sizeof(float));
    free(h);
}

static void expect(sb_status got, sb_status want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d\n", what, (int)got,
                sb_status_string(got), (int)want);
        exit(1);
    }
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/head.txt", dir);
    FILE *f = fopen(path, "r");
    int B, H, V, k;
    if (!f || fscanf(f, "%d %d %d %d", &B, &H, &V, &k) != 4 || B < 1 || H < 1 || V < 1 ||
        k < 1 || k > SB_MAX_LANES) {
        fprintf(stderr, "bad %s\n", path);
        return 1;
    }
    int32_t off[SB_MAX_LANES + 1];
    for (int i = 0; i <= k; ++i) {
        int o;
        if (fscanf(f, "%d", &o) != 1) {
            fprintf(stderr, "bad lane offsets in %s\n", path);
            return 1;
        }
        off[i] = (int32_t)o;
    }
    fclose(f);

    uint16_t *x = (uint16_t *)read_file(dir, "x.bin", (size_t)B * H * 2);
    uint16_t *w = (uint16_t *)read_file(dir, "w.bin", (size_t)H * V * 2);

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    /* x at a row stride of a multiple of 8 elements */
    const int64_t ldx = (H + 7) / 8 * 8;
    void *dx;
    CHECK_HIP(hipMalloc(&dx, (size_t)B * ldx * 2));
    CHECK_HIP(hipMemset(dx, 0, (size_t)B * ldx * 2));
    CHECK_HIP(hipMemcpy2D(dx, (size_t)ldx * 2, x, (size_t)H * 2, (size_t)H * 2, (size_t)B,
                          hipMemcpyHostToDevice));

    /* every lane in its own allocation, one common row stride */
    int maxw = 0;
    for (int i = 0; i < k; ++i)
        if (off[i + 1] - off[i] > maxw)
            maxw = off[i + 1] - off[i];
    const int64_t ldw = (maxw + 7) / 8 * 8;
    const void *dw[SB_MAX_LANES];
    for (int i = 0; i < k; ++i) {
        void *p;
        const int wi = off[i + 1] - off[i];
        CHECK_HIP(hipMalloc(&p, (size_t)H * ldw * 2));
        CHECK_HIP(hipMemset(p, 0, (size_t)H * ldw * 2));
        CHECK_HIP(hipMemcpy2D(p, (size_t)ldw * 2, w + off[i], (size_t)V * 2, (size_t)wi * 2,
                              (size_t)H, hipMemcpyHostToDevice));
        dw[i] = p;
    }

    sb_head_desc d;
    memset(&d, 0, sizeof d);
    d.B = B;
    d.H = H;
    d.V = V;
    d.k = k;
    d.lane_off = off;
    d.x = dx;
    d.ldx = ldx;
    d.w = dw;
    d.ldw = ldw;

    /* one workspace sized for the largest surface */
    size_t need = 0;
    for (int s = SB_SURF_TOKENS; s <= SB_SURF_FULL_LOGITS; ++s) {
        sb_status st;
        const size_t n = sb_workspace_bytes(&d, s, &st);
        CHECK_SB(st);
        if (n > need)
            need = n;
    }
    void *ws;
    CHECK_HIP(hipMalloc(&ws, need ? need : 16));

    const int64_t ld = (V + 3) / 4 * 4;  /* fp32 outputs: a multiple of 4 */
    int32_t *ids_tok, *ids_static, *ids_lp, *ids_r0, *lane_ids;
    float *lane_max, *lse, *sel, *lp, *logits;
    CHECK_HIP(hipMalloc((void **)&ids_tok, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&ids_static, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&ids_lp, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&ids_r0, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&lane_ids, (size_t)B * k * 4));
    CHECK_HIP(hipMalloc((void **)&lane_max, (size_t)B * k * 4));
    CHECK_HIP(hipMalloc((void **)&lse, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&sel, (size_t)B * 4));
    CHECK_HIP(hipMalloc((void **)&lp, (size_t)B * ld * 4));
    CHECK_HIP(hipMalloc((void **)&logits, (size_t)B * ld * 4));

    /* refused calls: nothing is enqueued, no output touched */
    {
        sb_status st;
        (void)sb_workspace_bytes(&d, 7, &st);
        expect(st, SB_ERR_SHAPE, "sb_workspace_bytes with an unknown surface");
        const size_t tok = sb_workspace_bytes(&d, SB_SURF_TOKENS, &st);
        CHECK_SB(st);
        if (tok > 0)
            expect(sb_project_tokens(&d, ids_tok, ws, tok - 1, stream), SB_ERR_WORKSPACE,
                   "sb_project_tokens with a workspace one byte short");
        expect(sb_project_tokens(&d, NULL, ws, need, stream), SB_ERR_NULL,
               "sb_project_tokens without an ID buffer");
    }

    CHECK_SB(sb_project_tokens(&d, ids_tok, ws, need, stream));
    CHECK_SB(sb_project_tokens_static(&d, ids_static, stream));
    CHECK_SB(sb_project_lane_results(&d, ids_r0, lane_ids, lane_max, ws, need, stream));
    CHECK_SB(sb_project_logprobs(&d, ids_lp, lse, sel, lp, ld, ws, need, stream));
    CHECK_SB(sb_full_logits(&d, logits, ld, ids_r0, ws, need, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    dump(dir, "ids_tok.bin", ids_tok, (size_t)B * 4);
    dump(dir, "ids_static.bin", ids_static, (size_t)B * 4);
    dump(dir, "ids_lp.bin", ids_lp, (size_t)B * 4);
    dump(dir, "ids_r0.bin", ids_r0, (size_t)B * 4);
    dump(dir, "lane_ids.bin", lane_ids, (size_t)B * k * 4);
    dump(dir, "lane_max.bin", lane_max, (size_t)B * k * 4);
    dump(dir, "lse.bin", lse, (size_t)B * 4);
    dump(dir, "sel.bin", sel, (size_t)B * 4);
    dump_rows(dir, "lp.bin", lp, B, ld, V);
    dump_rows(dir, "logits.bin", logits, B, ld, V);

    CHECK_HIP(hipFree(ids_tok));
    CHECK_HIP(hipFree(ids_static));
    CHECK_HIP(hipFree(ids_lp));
    CHECK_HIP(hipFree(ids_r0));
    CHECK_HIP(hipFree(lane_ids));
    CHECK_HIP(hipFree(lane_max));
    CHECK_HIP(hipFree(lse));
    CHECK_HIP(hipFree(sel));
    CHECK_HIP(hipFree(lp));
    CHECK_HIP(hipFree(logits));
    CHECK_HIP(hipFree(ws));
    for (int i = 0; i < k; ++i)
        CHECK_HIP(hipFree((void *)dw[i]));
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipStreamDestroy(stream));
    free(x);
    free(w);
    printf("abi_driver ok: B=%d H=%d V=%d k=%d\n", B, H, V, k);
    return 0;
}
