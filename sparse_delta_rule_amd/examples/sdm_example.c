/*
 * A plain C caller of libsdm (include/sdm.h): device memory and a stream from the
 * HIP runtime, three sdm_decode_step calls on a small bfloat16 bank, one
 * sdm_gather with two operands and a stash, and one call that the library
 * rejects. Prints every result as raw bits, one array per line:
 *     <name> <count> <hex> <hex> ...
 * and "status <name> <code>" for the rejected call.
 *
 * The inputs are closed-form integer patterns (no randomness), so any other
 * program can rebuild them exactly:
 *   bank[i][c]        = bf16 bits of ((i * 7 + c * 3) % 17 - 8) / 16      (i < NS, c < HD)
 *   k_idx[t][s][w]    = s * P + (t * 5 + w * 3 + s) % P                    (P slots per stream)
 *   q_idx[t][s][r]    = s * P + (t * 2 + r * 5 + 1) % P
 *   k_val[t][s][w]    = ((t + 2 * s + w) % 5 - 2) / 4
 *   q_val[t][s][r]    = ((t + s + 3 * r) % 7 - 3) / 8
 *   v[t][s][c]        = ((3 * t + s + c) % 9 - 4) / 8
 *   beta[t][s]        = (1 + (t + s) % 3) / 4
 *   g[t][s][w]        = -((t + s + w) % 4) / 16                           (G = W)
 *   gather: idx0[t][n] = (t * 11 + n * 7) % NS, idx1[t][n] = (t * 3 + n * 13 + 5) % NS,
 *           w0[t][n] = ((t + n) % 5 - 2) / 2, w1[t][n] = ((2 * t + n) % 3 - 1) / 4 (float32),
 *           chunk 4, valid 3, over the bank after the three decode steps.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sdm.h"

enum { S = 3, P = 8, NS = S * P, HD = 8, W = 3, R = 2, T = 3, GT = 8, GW0 = 3, GW1 = 2, CHUNK = 4, VALID = 3 };

static uint16_t bf16_bits(float x) {
    /* every pattern value above is exact in bfloat16: the high half of the float32 */
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(call)                                                                  \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

#define CHECK_SDM(call)                                                                  \
    do {                                                                                 \
        int s_ = (call);                                                                 \
        if (s_ != SDM_OK) {                                                              \
            fprintf(stderr, "%s returned %d: %s\n", #call, s_, sdm_last_error());        \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

static void print_u16(const char* name, const uint16_t* a, int n) {
    printf("%s %d", name, n);
    for (int i = 0; i < n; ++i) printf(" %04x", a[i]);
    printf("\n");
}

static void print_f32(const char* name, const float* a, int n) {
    printf("%s %d", name, n);
    for (int i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &a[i], 4);
        printf(" %08x", u);
    }
    printf("\n");
}

int main(void) {
    if (sdm_abi_version() != SDM_ABI_VERSION) {
        fprintf(stderr, "libsdm ABI %d, header %d\n", sdm_abi_version(), SDM_ABI_VERSION);
        return 1;
    }
    uint16_t bank_h[NS * HD];
    for (int i = 0; i < NS; ++i)
        for (int c = 0; c < HD; ++c) bank_h[i * HD + c] = bf16_bits((float)((i * 7 + c * 3) % 17 - 8) / 16.0f);

    int32_t k_idx[T][S][W], q_idx[T][S][R];
    float k_val[T][S][W], q_val[T][S][R], v[T][S][HD], beta[T][S], g[T][S][W];
    for (int t = 0; t < T; ++t)
        for (int s = 0; s < S; ++s) {
            for (int w = 0; w < W; ++w) {
                k_idx[t][s][w] = s * P + (t * 5 + w * 3 + s) % P;
                k_val[t][s][w] = (float)((t + 2 * s + w) % 5 - 2) / 4.0f;
                g[t][s][w] = -(float)((t + s + w) % 4) / 16.0f;
            }
            for (int r = 0; r < R; ++r) {
                q_idx[t][s][r] = s * P + (t * 2 + r * 5 + 1) % P;
                q_val[t][s][r] = (float)((t + s + 3 * r) % 7 - 3) / 8.0f;
            }
            for (int c = 0; c < HD; ++c) v[t][s][c] = (float)((3 * t + s + c) % 9 - 4) / 8.0f;
            beta[t][s] = (float)(1 + (t + s) % 3) / 4.0f;
        }

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    void *bank, *dk_idx, *dq_idx, *dk_val, *dq_val, *dv, *dbeta, *dg, *dread;
    CHECK_HIP(hipMalloc(&bank, sizeof bank_h));
    CHECK_HIP(hipMalloc(&dk_idx, sizeof k_idx));
    CHECK_HIP(hipMalloc(&dq_idx, sizeof q_idx));
    CHECK_HIP(hipMalloc(&dk_val, sizeof k_val));
    CHECK_HIP(hipMalloc(&dq_val, sizeof q_val));
    CHECK_HIP(hipMalloc(&dv, sizeof v));
    CHECK_HIP(hipMalloc(&dbeta, sizeof beta));
    CHECK_HIP(hipMalloc(&dg, sizeof g));
    CHECK_HIP(hipMalloc(&dread, sizeof(uint16_t) * T * S * HD));
    CHECK_HIP(hipMemcpy(bank, bank_h, sizeof bank_h, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk_idx, k_idx, sizeof k_idx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dq_idx, q_idx, sizeof q_idx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk_val, k_val, sizeof k_val, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dq_val, q_val, sizeof q_val, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dbeta, beta, sizeof beta, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, g, sizeof g, hipMemcpyHostToDevice));

    /* three tokens, one sdm_decode_step call each, in order on the stream */
    for (int t = 0; t < T; ++t)
        CHECK_SDM(sdm_decode_step(bank, SDM_BF16, NS, HD, S, W, R, W,
                                  (char*)dk_idx + t * sizeof k_idx[0], SDM_I32,
                                  (char*)dk_val + t * sizeof k_val[0], (char*)dv + t * sizeof v[0],
                                  (char*)dq_val + t * sizeof q_val[0], SDM_F32,
                                  (const float*)((char*)dbeta + t * sizeof beta[0]),
                                  (const float*)((char*)dg + t * sizeof g[0]),
                                  (char*)dq_idx + t * sizeof q_idx[0], SDM_I32,
                                  (char*)dread + t * sizeof(uint16_t) * S * HD, stream));

    /* the gather over the updated bank */
    int32_t idx0[GT][GW0], idx1[GT][GW1];
    float w0[GT][GW0], w1[GT][GW1];
    for (int t = 0; t < GT; ++t) {
        for (int n = 0; n < GW0; ++n) {
            idx0[t][n] = (t * 11 + n * 7) % NS;
            w0[t][n] = (float)((t + n) % 5 - 2) / 2.0f;
        }
        for (int n = 0; n < GW1; ++n) {
            idx1[t][n] = (t * 3 + n * 13 + 5) % NS;
            w1[t][n] = (float)((2 * t + n) % 3 - 1) / 4.0f;
        }
    }
    void *di0, *di1, *dw0, *dw1, *dout0, *dout1, *dstash;
    CHECK_HIP(hipMalloc(&di0, sizeof idx0));
    CHECK_HIP(hipMalloc(&di1, sizeof idx1));
    CHECK_HIP(hipMalloc(&dw0, sizeof w0));
    CHECK_HIP(hipMalloc(&dw1, sizeof w1));
    CHECK_HIP(hipMalloc(&dout0, sizeof(float) * GT * HD));
    CHECK_HIP(hipMalloc(&dout1, sizeof(float) * GT * HD));
    CHECK_HIP(hipMalloc(&dstash, sizeof(uint16_t) * GT * GW0 * HD));
    CHECK_HIP(hipMemcpyAsync(di0, idx0, sizeof idx0, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(di1, idx1, sizeof idx1, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(dw0, w0, sizeof w0, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(dw1, w1, sizeof w1, hipMemcpyHostToDevice, stream));
    CHECK_SDM(sdm_gather(bank, SDM_BF16, NS, HD, GT, CHUNK, VALID, NULL, SDM_I32, SDM_F32, di0, dw0, GW0,
                         (float*)dout0, dstash, di1, dw1, GW1, (float*)dout1, stream));

    /* a width outside 1..SDM_MAX_WIDTH is rejected before any HIP call */
    const int bad = sdm_decode_step(bank, SDM_BF16, NS, HD, S, SDM_MAX_WIDTH + 1, R, 1, dk_idx, SDM_I32, dk_val,
                                    dv, dq_val, SDM_F32, (const float*)dbeta, (const float*)dg, dq_idx, SDM_I32,
                                    dread, stream);

    CHECK_HIP(hipStreamSynchronize(stream));
    uint16_t read_h[T * S * HD], stash_h[GT * GW0 * HD];
    float out0_h[GT * HD], out1_h[GT * HD];
    CHECK_HIP(hipMemcpy(bank_h, bank, sizeof bank_h, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(read_h, dread, sizeof read_h, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out0_h, dout0, sizeof out0_h, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out1_h, dout1, sizeof out1_h, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(stash_h, dstash, sizeof stash_h, hipMemcpyDeviceToHost));
    print_u16("readings", read_h, T * S * HD);
    print_u16("bank", bank_h, NS * HD);
    print_f32("out0", out0_h, GT * HD);
    print_f32("out1", out1_h, GT * HD);
    print_u16("stash", stash_h, GT * GW0 * HD);
    printf("status width_257 %d\n", bad);

    void* bufs[] = {bank, dk_idx, dq_idx, dk_val, dq_val, dv, dbeta, dg, dread, di0, di1, dw0, dw1, dout0, dout1,
                    dstash};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
    CHECK_HIP(hipStreamDestroy(stream));
    return 0;
}
