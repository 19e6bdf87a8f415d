/*
 * A plain C consumer of the library's C ABI (include/bsa.h): it plans a
 * BLOCK_U8 mask and runs the forward pass through bsa_plan / bsa_forward
 * with device buffers it allocates itself, with no Python in the process.
 * Test infrastructure: tests/test_gpu_c_abi.py writes the inputs, runs this
 * program and compares its output with the fp64 oracle.
 *
 * usage: c_abi_forward DIR
 *   DIR/shape.txt  "B H L d block_q block_k"
 *   DIR/mask.u8    uint8 [B][H][ceil(L/block_q)][ceil(L/block_k)]
 *   DIR/q.bf16, DIR/k.bf16, DIR/v.bf16   bf16 bits [B][H][L][d]
 * writes DIR/o.bf16 (bf16 bits [B][H][L][d]) and prints one line with the
 * plan's regime and tile counts. Exit status 0 on success, 1 on a library
 * or HIP error (the message names the failing call), 2 on a usage error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsa.h"

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *buf = malloc(bytes ? bytes : 1);
    const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(buf);
        return NULL;
    }
    return buf;
}

static int hip_ok(hipError_t e, const char *what)
{
    if (e == hipSuccess) return 1;
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
}

static int bsa_ok(int32_t st, const char *what)
{
    if (st == BSA_OK) return 1;
    fprintf(stderr, "%s: %s (%s)\n", what, bsa_status_str(st), bsa_last_error());
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/shape.txt", dir);
    FILE *f = fopen(path, "r");
    long long B, H, L, d, bq, bk;
    if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld", &B, &H, &L, &d, &bq, &bk) != 6) {
        fprintf(stderr, "cannot read %s\n", path);
        if (f) fclose(f);
        return 2;
    }
    fclose(f);
    if (B < 1 || H < 1 || L < 1 || (d != 64 && d != 128) || bq < 1 || bk < 1) {
        fprintf(stderr, "bad shape\n");
        return 2;
    }
    const size_t nqb = (size_t)((L + bq - 1) / bq), nkb = (size_t)((L + bk - 1) / bk);
    const size_t mask_bytes = (size_t)B * H * nqb * nkb;
    const size_t tensor_bytes = (size_t)B * H * L * d * 2;
    uint8_t *mask = read_file(dir, "mask.u8", mask_bytes);
    void *q = read_file(dir, "q.bf16", tensor_bytes);
    void *k = read_file(dir, "k.bf16", tensor_bytes);
    void *v = read_file(dir, "v.bf16", tensor_bytes);
    void *o = malloc(tensor_bytes);
    if (!mask || !q || !k || !v || !o) {
        fprintf(stderr, "cannot read the inputs in %s\n", dir);
        return 2;
    }
    if (bsa_abi_version() != BSA_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header %d\n", bsa_abi_version(), BSA_ABI_VERSION);
        return 1;
    }

    int rc = 1;
    void *dq = NULL, *dk = NULL, *dv = NULL, *dO = NULL;
    bsa_plan_t plan = NULL;
    bsa_mask_desc_t m;
    memset(&m, 0, sizeof m);
    m.kind = BSA_MASK_BLOCK_U8;
    m.data = mask;
    bsa_plan_opts_t opts;
    bsa_plan_opts_default(&opts);
    opts.device = 0;
    if (!hip_ok(hipSetDevice(0), "hipSetDevice")) goto done;
    if (!hip_ok(hipMalloc(&dq, tensor_bytes), "hipMalloc Q") || !hip_ok(hipMalloc(&dk, tensor_bytes), "hipMalloc K") ||
        !hip_ok(hipMalloc(&dv, tensor_bytes), "hipMalloc V") || !hip_ok(hipMalloc(&dO, tensor_bytes), "hipMalloc O"))
        goto done;
    if (!hip_ok(hipMemcpy(dq, q, tensor_bytes, hipMemcpyHostToDevice), "copy Q") ||
        !hip_ok(hipMemcpy(dk, k, tensor_bytes, hipMemcpyHostToDevice), "copy K") ||
        !hip_ok(hipMemcpy(dv, v, tensor_bytes, hipMemcpyHostToDevice), "copy V"))
        goto done;
    /* the mask may be freed once bsa_plan returns: the plan keeps what it needs */
    if (!bsa_ok(bsa_plan(&m, (int32_t)B, (int32_t)H, L, (int32_t)d, (int32_t)bq, (int32_t)bk, &opts, &plan), "bsa_plan"))
        goto done;
    free(mask);
    mask = NULL;
    if (!bsa_ok(bsa_forward(plan, dq, dk, dv, dO, NULL), "bsa_forward")) goto done;
    if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) goto done;
    if (!hip_ok(hipMemcpy(o, dO, tensor_bytes, hipMemcpyDeviceToHost), "copy O")) goto done;
    bsa_plan_info_t info;
    if (!bsa_ok(bsa_plan_info(plan, &info), "bsa_plan_info")) goto done;
    snprintf(path, sizeof path, "%s/o.bf16", dir);
    f = fopen(path, "wb");
    if (!f || fwrite(o, 1, tensor_bytes, f) != tensor_bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        if (f) fclose(f);
        goto done;
    }
    fclose(f);
    printf("regime %d tiles_full %lld tiles_partial %lld\n", info.regime, (long long)info.tiles_full,
           (long long)info.tiles_partial);
    rc = 0;
done:
    bsa_plan_destroy(plan);
    if (dq) (void)hipFree(dq);
    if (dk) (void)hipFree(dk);
    if (dv) (void)hipFree(dv);
    if (dO) (void)hipFree(dO);
    free(mask);
    free(q);
    free(k);
    free(v);
    free(o);
    return rc;
}
