/*
 * c_abi_path.c -- one decode step through libdsa's C ABI from plain C99.
 *
 * Reads a batch of decode inputs from a file, runs dsa_index_scores -> dsa_topk ->
 * sparse_mla_decode on the GPU with buffers this program allocates, and writes the
 * scores, the indices, the attention output and its lse to a second file.  It also checks
 * that a bad argument is refused with a message and that nothing is launched for it.
 *
 *   c_abi_path IN OUT
 *
 * IN (little endian): int32 B, T, H_I, D_I, H, D_c, D_r, k; int64 max_ctx; float sm_scale,
 * kv_scale; then int64 kv_indptr[B+1], uint16 q_idx[T][H_I][D_I] (bf16), float w[T][H_I],
 * uint8 k_idx[N][D_I] (E4M3), float k_scale[N], uint16 q[T][H][D_c+D_r] (bf16),
 * uint8 kv[N][D_c+D_r] (E4M3), with N = kv_indptr[B].
 * OUT: float scores[T][max_ctx] (entries past a row's visible count undefined),
 * int32 indices[T][k], uint16 out[T][H][D_c] (bf16), float lse[T][H].
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dsa.h"

static void die(const char *what)
{
    fprintf(stderr, "c_abi_path: %s\n", what);
    exit(1);
}

static void hip_ok(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        fprintf(stderr, "c_abi_path: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void dsa_ok(dsa_status st, const char *what)
{
    if (st != DSA_OK) {
        fprintf(stderr, "c_abi_path: %s failed (%d): %s\n", what, (int)st, dsa_last_error());
        exit(1);
    }
}

/* read n bytes from f into a new device buffer */
static void *upload(FILE *f, size_t n)
{
    void *h = malloc(n ? n : 1), *d = NULL;
    if (!h || fread(h, 1, n, f) != n)
        die("short input file");
    hip_ok(hipMalloc(&d, n ? n : 1), "hipMalloc");
    hip_ok(hipMemcpy(d, h, n, hipMemcpyHostToDevice), "upload");
    free(h);
    return d;
}

static void download(FILE *f, const void *d, size_t n)
{
    void *h = malloc(n ? n : 1);
    if (!h)
        die("out of host memory");
    hip_ok(hipMemcpy(h, d, n, hipMemcpyDeviceToHost), "download");
    if (fwrite(h, 1, n, f) != n)
        die("cannot write output");
    free(h);
}

int main(int argc, char **argv)
{
    if (argc != 3)
        die("usage: c_abi_path IN OUT");
    if (dsa_abi_version() != DSA_ABI_VERSION)
        die("library and header disagree on the ABI version");
    FILE *in = fopen(argv[1], "rb");
    if (!in)
        die("cannot open input");
    int32_t hdr[8];
    int64_t max_ctx;
    float sm_scale, kv_scale;
    if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&max_ctx, 8, 1, in) != 1 || fread(&sm_scale, 4, 1, in) != 1 ||
        fread(&kv_scale, 4, 1, in) != 1)
        die("short header");
    const int B = hdr[0], T = hdr[1], H_I = hdr[2], D_I = hdr[3], H = hdr[4], Dc = hdr[5], Dr = hdr[6], k = hdr[7];
    int64_t *kvp = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
    if (!kvp || fread(kvp, sizeof(int64_t), (size_t)(B + 1), in) != (size_t)(B + 1))
        die("short kv_indptr");
    const int64_t N = kvp[B];

    void *d_kvp = NULL;
    hip_ok(hipMalloc(&d_kvp, sizeof(int64_t) * (size_t)(B + 1)), "hipMalloc");
    hip_ok(hipMemcpy(d_kvp, kvp, sizeof(int64_t) * (size_t)(B + 1), hipMemcpyHostToDevice), "upload");
    void *d_qi = upload(in, (size_t)T * H_I * D_I * 2);
    void *d_w = upload(in, (size_t)T * H_I * 4);
    void *d_ki = upload(in, (size_t)N * D_I);
    void *d_ks = upload(in, (size_t)N * 4);
    void *d_q = upload(in, (size_t)T * H * (Dc + Dr) * 2);
    void *d_kv = upload(in, (size_t)N * (Dc + Dr));
    fclose(in);

    dsa_layout L;
    memset(&L, 0, sizeof L);
    L.batch = B;
    L.total_q = T;
    L.max_ctx = max_ctx;
    L.kv_indptr = (const int64_t *)d_kvp;
    L.q_indptr = NULL;   /* decode: one query row per sequence */
    L.block_table = NULL; /* contiguous caches */

    float *d_scores = NULL, *d_lse = NULL;
    int32_t *d_idx = NULL;
    void *d_out = NULL, *d_tws = NULL, *d_mws = NULL;
    hip_ok(hipMalloc((void **)&d_scores, (size_t)T * max_ctx * 4), "hipMalloc");
    hip_ok(hipMalloc((void **)&d_idx, (size_t)T * k * 4), "hipMalloc");
    hip_ok(hipMalloc(&d_out, (size_t)T * H * Dc * 2), "hipMalloc");
    hip_ok(hipMalloc((void **)&d_lse, (size_t)T * H * 4), "hipMalloc");
    const size_t tws = dsa_topk_workspace_size(&L, max_ctx, k);
    const size_t mws = sparse_mla_workspace_size(&L, H, Dc, Dr, k, 1);
    if (tws) {
        hip_ok(hipMalloc(&d_tws, tws), "hipMalloc");
        hip_ok(hipMemset(d_tws, 0, tws), "hipMemset"); /* zero before its first use */
    }
    if (mws)
        hip_ok(hipMalloc(&d_mws, mws), "hipMalloc");

    /* a refused call: k = 0 is outside [1, DSA_TOPK_MAX]; nothing may be written */
    hip_ok(hipMemset(d_idx, 0x7F, (size_t)T * k * 4), "hipMemset");
    if (dsa_topk(&L, d_scores, max_ctx, 0, d_idx, d_tws, tws, NULL) != DSA_ERR_INVALID_ARG ||
        dsa_last_error()[0] == '\0')
        die("k = 0 was not refused with a message");
    hip_ok(hipDeviceSynchronize(), "sync");
    int32_t probe = 0;
    hip_ok(hipMemcpy(&probe, d_idx, 4, hipMemcpyDeviceToHost), "download");
    if (probe != 0x7F7F7F7F)
        die("a refused call wrote its output");
    printf("refused call: %s\n", dsa_last_error());

    dsa_ok(dsa_index_scores(&L, H_I, D_I, DSA_BF16, d_qi, NULL, (const float *)d_w, DSA_FP8_E4M3FN, d_ki, D_I,
                            (const float *)d_ks, 1, d_scores, max_ctx, NULL),
           "dsa_index_scores");
    dsa_ok(dsa_topk(&L, d_scores, max_ctx, k, d_idx, d_tws, tws, NULL), "dsa_topk");
    dsa_ok(sparse_mla_decode(&L, H, Dc, Dr, sm_scale, DSA_BF16, d_q, DSA_FP8_E4M3FN, d_kv, kv_scale, d_idx, k,
                             DSA_BF16, d_out, d_lse, d_mws, mws, NULL),
           "sparse_mla_decode");
    hip_ok(hipDeviceSynchronize(), "sync");

    FILE *out = fopen(argv[2], "wb");
    if (!out)
        die("cannot open output");
    download(out, d_scores, (size_t)T * max_ctx * 4);
    download(out, d_idx, (size_t)T * k * 4);
    download(out, d_out, (size_t)T * H * Dc * 2);
    download(out, d_lse, (size_t)T * H * 4);
    fclose(out);
    printf("decode step of %d rows done\n", T);

    void *bufs[] = {d_kvp, d_qi, d_w, d_ki, d_ks, d_q, d_kv, d_scores, d_idx, d_out, d_lse, d_tws, d_mws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i])
            hip_ok(hipFree(bufs[i]), "hipFree");
    free(kvp);
    return 0;
}
