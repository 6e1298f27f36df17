/*
 * A consumer of liba2av.so written in plain C: no Python, no torch. It runs
 * the one-call and the three-call a2av on W = 4 ranks with equal splits and
 * checks the result against its closed form (equal splits make the exchange a
 * block transpose: destination d holds chunk d of every source, in source
 * order), then checks that an oversized split is refused with nothing written.
 * Prints "c abi consumer: ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "a2av.h"

#define W 4
#define ROWS 1024          /* rows per rank */
#define RB 40              /* bytes per row: not a multiple of 16 */
#define CHUNK (ROWS / W)   /* rows each rank sends to each rank */

#define HIP_OK(x) do { if ((x) != hipSuccess) { printf("hip error line %d\n", __LINE__); return 1; } } while (0)
#define EXPECT(c) do { if (!(c)) { printf("check failed line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static unsigned char byte_of(int s, int row, int b) { return (unsigned char)(s * 97 + row * 31 + b * 7 + 1); }

static int run(int fused) {
    void *in[W], *out[W];
    int64_t in_rows[W], cap[W], S[W * W];
    int64_t *dS, *dO, *dso, *dro;
    int32_t *dst, hst = -1;
    unsigned char *host = malloc((size_t)ROWS * RB);
    for (int r = 0; r < W; r++) {
        HIP_OK(hipMalloc(&in[r], (size_t)ROWS * RB));
        HIP_OK(hipMalloc(&out[r], (size_t)ROWS * RB));
        HIP_OK(hipMemset(out[r], 0, (size_t)ROWS * RB));
        for (int i = 0; i < ROWS; i++)
            for (int b = 0; b < RB; b++) host[(size_t)i * RB + b] = byte_of(r, i, b);
        HIP_OK(hipMemcpy(in[r], host, (size_t)ROWS * RB, hipMemcpyHostToDevice));
        in_rows[r] = ROWS;
        cap[r] = ROWS;
    }
    for (int i = 0; i < W * W; i++) S[i] = CHUNK;
    HIP_OK(hipMalloc((void **)&dS, sizeof(S)));
    HIP_OK(hipMalloc((void **)&dO, sizeof(S)));
    HIP_OK(hipMalloc((void **)&dso, sizeof(int64_t) * W * (W + 1)));
    HIP_OK(hipMalloc((void **)&dro, sizeof(int64_t) * W * (W + 1)));
    HIP_OK(hipMalloc((void **)&dst, sizeof(int32_t)));
    HIP_OK(hipMemcpy(dS, S, sizeof(S), hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dst, 0, sizeof(int32_t)));
    if (fused) {
        EXPECT(a2av_all_to_all_vdev(W, RB, (const void *const *)in, in_rows, out, cap, dS, dO, dso,
                                    dro, dst, NULL) == A2AV_OK);
    } else {
        EXPECT(a2av_exchange_splits(W, dS, dO, dst, NULL) == A2AV_OK);
        EXPECT(a2av_offsets(W, dS, dO, dso, dro, dst, NULL) == A2AV_OK);
        EXPECT(a2av_copy(W, RB, (const void *const *)in, in_rows, out, cap, dS, dso, dro, dst,
                         NULL) == A2AV_OK);
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(&hst, dst, sizeof(int32_t), hipMemcpyDeviceToHost));
    EXPECT(hst == 0);
    int64_t ro[W * (W + 1)];
    HIP_OK(hipMemcpy(ro, dro, sizeof(ro), hipMemcpyDeviceToHost));
    for (int d = 0; d < W; d++) {
        for (int s = 0; s <= W; s++) EXPECT(ro[d * (W + 1) + s] == (int64_t)s * CHUNK);
        HIP_OK(hipMemcpy(host, out[d], (size_t)ROWS * RB, hipMemcpyDeviceToHost));
        for (int s = 0; s < W; s++)
            for (int i = 0; i < CHUNK; i++)
                for (int b = 0; b < RB; b++)
                    EXPECT(host[((size_t)s * CHUNK + i) * RB + b] == byte_of(s, d * CHUNK + i, b));
    }
    /* an oversized split: the status says so and no output byte changes */
    for (int r = 0; r < W; r++) HIP_OK(hipMemset(out[r], 0x5A, (size_t)ROWS * RB));
    S[1] = (int64_t)1 << 41;
    HIP_OK(hipMemcpy(dS, S, sizeof(S), hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dst, 0, sizeof(int32_t)));
    EXPECT(a2av_all_to_all_vdev(W, RB, (const void *const *)in, in_rows, out, cap, dS, dO, dso, dro,
                                dst, NULL) == A2AV_OK);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(&hst, dst, sizeof(int32_t), hipMemcpyDeviceToHost));
    EXPECT(hst == A2AV_ST_BAD_SPLIT);
    for (int d = 0; d < W; d++) {
        HIP_OK(hipMemcpy(host, out[d], (size_t)ROWS * RB, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < (size_t)ROWS * RB; i++) EXPECT(host[i] == 0x5A);
    }
    for (int r = 0; r < W; r++) {
        HIP_OK(hipFree(in[r]));
        HIP_OK(hipFree(out[r]));
    }
    HIP_OK(hipFree(dS)); HIP_OK(hipFree(dO)); HIP_OK(hipFree(dso)); HIP_OK(hipFree(dro));
    HIP_OK(hipFree(dst));
    free(host);
    return 0;
}

int main(void) {
    EXPECT(a2av_abi_version() == A2AV_ABI_VERSION);
    EXPECT(a2av_exchange_splits(0, NULL, NULL, NULL, NULL) == A2AV_EARG);
    if (run(1) || run(0)) return 1;
    printf("c abi consumer: ok\n");
    return 0;
}
