/*
 * librax from plain C, with no PyTorch in the process: device memory through the HIP runtime,
 * the calls through include/librax.h.
 *
 * One request holds one stored key. With a single key the softmax weight is exactly 1, so
 * DECODE and EXTEND must both return that key's V row, bit for bit, for every query head of the
 * group (query head h reads kv head h / G). The pool's other slots hold NaN, so a read of any
 * other slot would show. A NULL argument must be refused with RAX_ERR_NULL.
 *
 * Exit status 0 and the line "c-abi ok" on success; 1 on a wrong result; 2 on a HIP error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "librax.h"

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            return 2;                                                              \
        }                                                                          \
    } while (0)

enum { S = 64, HKV = 2, HQ = 8, D = 128, G = HQ / HKV, STRIDE = 4, SLOT = 37 };

/* bf16 bits of a float whose low 16 bits are zero (every value used here is such a float) */
static uint16_t bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int same_as_v(const uint16_t* out, const uint16_t* v, const char* what) {
    for (int h = 0; h < HQ; ++h)
        for (int d = 0; d < D; ++d)
            if (out[h * D + d] != v[(h / G) * D + d]) {
                fprintf(stderr, "%s: head %d element %d is %04x, want %04x\n", what, h, d,
                        out[h * D + d], v[(h / G) * D + d]);
                return 0;
            }
    return 1;
}

int main(void) {
    static uint16_t k_new[HKV * D], v_new[HKV * D], q[HQ * D], out[HQ * D];
    for (int i = 0; i < HKV * D; ++i) {
        k_new[i] = bf16_bits((float)(i % 7 - 3));
        v_new[i] = bf16_bits(0.25f * (float)(i % 11 - 5));
    }
    for (int i = 0; i < HQ * D; ++i) q[i] = bf16_bits(0.5f * (float)(i % 5 - 2));
    const int32_t loc[1] = {SLOT};
    const int32_t table[STRIDE] = {SLOT, -1, -1, -1};
    const int32_t zero[1] = {0}, one[1] = {1};
    const size_t pool_bytes = (size_t)S * HKV * D * 2;

    void *kp, *vp, *kn, *vn, *dq, *dout, *ws;
    int32_t *dloc, *dtab, *dzero, *done;
    HIP_OK(hipMalloc(&kp, pool_bytes));
    HIP_OK(hipMalloc(&vp, pool_bytes));
    HIP_OK(hipMemset(kp, 0xFF, pool_bytes)); /* 0xFFFF: a bf16 NaN in every slot */
    HIP_OK(hipMemset(vp, 0xFF, pool_bytes));
    HIP_OK(hipMalloc(&kn, sizeof k_new));
    HIP_OK(hipMalloc(&vn, sizeof v_new));
    HIP_OK(hipMalloc(&dq, sizeof q));
    HIP_OK(hipMalloc(&dout, sizeof out));
    HIP_OK(hipMalloc((void**)&dloc, sizeof loc));
    HIP_OK(hipMalloc((void**)&dtab, sizeof table));
    HIP_OK(hipMalloc((void**)&dzero, sizeof zero));
    HIP_OK(hipMalloc((void**)&done, sizeof one));
    HIP_OK(hipMemcpy(kn, k_new, sizeof k_new, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(vn, v_new, sizeof v_new, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dloc, loc, sizeof loc, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dtab, table, sizeof table, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dzero, zero, sizeof zero, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(done, one, sizeof one, hipMemcpyHostToDevice));

    const float scale = 0.08838834764831845f;
    int st = rax_kv_store(RAX_BF16, kn, vn, dloc, 1, kp, vp, S, HKV, D, NULL);
    if (st != RAX_OK) { fprintf(stderr, "kv_store: %s\n", rax_status_str(st)); return 1; }

    /* DECODE: the request's only position is the stored key */
    const size_t ws_bytes = rax_decode_workspace_bytes(RAX_BF16, 1, STRIDE, HQ, HKV, D);
    HIP_OK(hipMalloc(&ws, ws_bytes));
    st = rax_decode_attention(RAX_BF16, dq, dout, kp, vp, S, dtab, STRIDE, dzero, done, 1, STRIDE, HQ,
                              HKV, D, scale, ws, ws_bytes, NULL);
    if (st != RAX_OK) { fprintf(stderr, "decode: %s\n", rax_status_str(st)); return 1; }
    HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    if (!same_as_v(out, v_new, "decode")) return 1;

    /* EXTEND: the same key as a one-token suffix on an empty prefix */
    HIP_OK(hipMemset(dout, 0xFF, sizeof out));
    st = rax_extend_attention(RAX_BF16, dq, dout, kp, vp, S, dtab, STRIDE, dzero, dzero, done, dzero, 1,
                              1, 1, 1, HQ, HKV, D, scale, NULL, 0, NULL);
    if (st != RAX_OK) { fprintf(stderr, "extend: %s\n", rax_status_str(st)); return 1; }
    HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
    if (!same_as_v(out, v_new, "extend")) return 1;

    /* a NULL query is refused on the host */
    st = rax_decode_attention(RAX_BF16, NULL, dout, kp, vp, S, dtab, STRIDE, dzero, done, 1, STRIDE, HQ,
                              HKV, D, scale, ws, ws_bytes, NULL);
    if (st != RAX_ERR_NULL || strcmp(rax_status_str(st), "RAX_ERR_NULL") != 0) {
        fprintf(stderr, "NULL q: got %s\n", rax_status_str(st));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    printf("c-abi ok\n");
    return 0;
}
