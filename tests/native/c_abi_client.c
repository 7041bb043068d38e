/*
 * A plain C client of the attention library: device memory from the HIP
 * runtime, no torch, no Python.  It reads bf16 Q, K, V (raw little-endian
 * bit patterns) from files, runs one prefill and one decode (with the
 * default split plan and a workspace it sizes through the ABI) on a stream
 * it creates, and writes the two bf16 outputs to files.  The GPU test that
 * builds and runs it compares those outputs with the oracle.
 *
 *   c_abi_client DIR B H_q H_kv T D
 *     DIR/q.bin  [B][H_q][T][D]   DIR/k.bin, DIR/v.bin  [B][H_kv][T][D]
 *     writes DIR/o_prefill.bin (causal prefill, scale 1/sqrt(D))
 *            DIR/o_decode.bin  [B][H_q][1][D]: the last query row of each
 *                              head against all T keys
 *
 * Exit status 0 on success; any failed call prints its status and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "attn.h"

static int fail(const char* what, int status) {
    fprintf(stderr, "%s failed: %s\n", what, attn_status_string(status));
    return 1;
}

static int fail_hip(const char* what, int err) {
    fprintf(stderr, "%s failed: hipError %d\n", what, err);
    return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const int bad = fwrite(p, 1, bytes, f) != bytes;
    fclose(f);
    return bad;
}

int main(int argc, char** argv) {
    if (argc != 7) {
        fprintf(stderr, "usage: %s DIR B H_q H_kv T D\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    const int B = atoi(argv[2]), H_q = atoi(argv[3]), H_kv = atoi(argv[4]), T = atoi(argv[5]), D = atoi(argv[6]);
    if (attn_abi_version() != ATTN_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header %d\n", attn_abi_version(), ATTN_ABI_VERSION);
        return 1;
    }
    const size_t nq = (size_t)B * H_q * T * D * 2, nkv = (size_t)B * H_kv * T * D * 2;
    const size_t nd = (size_t)B * H_q * D * 2;  /* one decode row per head */
    void* hq = read_file(dir, "q.bin", nq);
    void* hk = read_file(dir, "k.bin", nkv);
    void* hv = read_file(dir, "v.bin", nkv);
    if (!hq || !hk || !hv) {
        fprintf(stderr, "cannot read the inputs\n");
        return 1;
    }
    /* the decode query: the last row of every head of Q */
    unsigned char* hqd = (unsigned char*)malloc(nd);
    for (size_t bh = 0; bh < (size_t)B * H_q; ++bh)
        for (size_t e = 0; e < (size_t)D * 2; ++e)
            hqd[bh * D * 2 + e] = ((unsigned char*)hq)[(bh * T + (T - 1)) * D * 2 + e];

    void *q, *k, *v, *o, *qd, *od, *ws = NULL;
    hipStream_t s;
    int e;
    if ((e = hipStreamCreate(&s)) != 0) return fail_hip("hipStreamCreate", e);
    if ((e = hipMalloc(&q, nq)) || (e = hipMalloc(&k, nkv)) || (e = hipMalloc(&v, nkv)) || (e = hipMalloc(&o, nq)) ||
        (e = hipMalloc(&qd, nd)) || (e = hipMalloc(&od, nd)))
        return fail_hip("hipMalloc", e);
    if ((e = hipMemcpy(q, hq, nq, hipMemcpyHostToDevice)) || (e = hipMemcpy(k, hk, nkv, hipMemcpyHostToDevice)) ||
        (e = hipMemcpy(v, hv, nkv, hipMemcpyHostToDevice)) || (e = hipMemcpy(qd, hqd, nd, hipMemcpyHostToDevice)))
        return fail_hip("hipMemcpy", e);

    const float scale = 1.0f / sqrtf((float)D);
    attn_status_t st = attn_fwd_prefill(q, k, v, o, B, H_q, H_kv, T, T, D, 1, scale, ATTN_BF16, s);
    if (st != ATTN_OK) return fail("attn_fwd_prefill", st);

    const size_t wsb = attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T, D, ATTN_BF16, 0);
    if (wsb > 0 && (e = hipMalloc(&ws, wsb))) return fail_hip("hipMalloc(workspace)", e);
    st = attn_fwd_decode(qd, k, v, od, B, H_q, H_kv, 1, T, D, 0, scale, ATTN_BF16, 0, ws, wsb, s);
    if (st != ATTN_OK) return fail("attn_fwd_decode", st);
    if ((e = hipStreamSynchronize(s))) return fail_hip("hipStreamSynchronize", e);

    void* ho = malloc(nq);
    void* hod = malloc(nd);
    if ((e = hipMemcpy(ho, o, nq, hipMemcpyDeviceToHost)) || (e = hipMemcpy(hod, od, nd, hipMemcpyDeviceToHost)))
        return fail_hip("hipMemcpy back", e);
    if (write_file(dir, "o_prefill.bin", ho, nq) || write_file(dir, "o_decode.bin", hod, nd)) {
        fprintf(stderr, "cannot write the outputs\n");
        return 1;
    }
    printf("ok: %d splits\n", attn_fwd_decode_default_splits(B, H_q, H_kv, T, D));
    hipFree(q), hipFree(k), hipFree(v), hipFree(o), hipFree(qd), hipFree(od);
    if (ws) hipFree(ws);
    hipStreamDestroy(s);
    free(hq), free(hk), free(hv), free(hqd), free(ho), free(hod);
    return 0;
}
