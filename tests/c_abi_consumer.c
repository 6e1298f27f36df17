/*
 * A consumer of liba2av.so written in plain C: no Python, no torch. It runs
 * the one-call and the three-call a2av on W = 4 ranks with equal splits and
 * checks the result against its closed form (equal splits make the exchange a
 * block transpose: destination d holds chunk d of every source, in source
 * order), then checks that an oversized split is refused with nothing written.
 * Then a one-step MoE trip on two ranks: the pack and the dispatch into
 * expert-major receivers, the un-pack read at the owners (every slot gets its
 * token's bytes back) and the weighted combine read at the owners (weights
 * 1/2 and 1/2 over the same token twice give the token itself, exactly).
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

#define MW 2               /* ranks of the MoE trip */
#define MT 64              /* tokens per rank */
#define MK 2               /* experts per token */
#define ME 4               /* experts (2 per rank) */
#define MH 16              /* bf16 elements per row */

/* a finite normal bf16 per (rank, token, element): halving is exact */
static uint16_t bf16_of(int s, int t, int h) { return (uint16_t)(0x3C00 | ((s * 131 + t * 7 + h) & 0x3FF)); }

static int run_moe(void) {
    const size_t R = MH * 2;
    void *tok[MW], *ids[MW], *perm[MW], *recv[MW], *home[MW], *wts[MW], *comb[MW];
    int64_t cap[MW] = {0, 0};
    int32_t hid[MT * MK];
    uint16_t htok[MT * MH], hbuf[MT * MK * MH];
    float hw[MT * MK];
    for (int q = 0; q < MT * MK; q++) hw[q] = 0.5f;
    for (int s = 0; s < MW; s++) {
        for (int t = 0; t < MT; t++) {
            hid[t * MK] = (t + s) % ME;          /* two distinct experts per token */
            hid[t * MK + 1] = (t + s + 1) % ME;
            for (int h = 0; h < MH; h++) htok[t * MH + h] = bf16_of(s, t, h);
        }
        for (int q = 0; q < MT * MK; q++) cap[hid[q] / (ME / MW)] += 1;
        HIP_OK(hipMalloc(&tok[s], sizeof(htok)));
        HIP_OK(hipMalloc(&ids[s], sizeof(hid)));
        HIP_OK(hipMalloc(&perm[s], sizeof(int64_t) * MT * MK));
        HIP_OK(hipMalloc(&home[s], sizeof(hbuf)));
        HIP_OK(hipMalloc(&wts[s], sizeof(hw)));
        HIP_OK(hipMalloc(&comb[s], sizeof(htok)));
        HIP_OK(hipMemcpy(tok[s], htok, sizeof(htok), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(ids[s], hid, sizeof(hid), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(wts[s], hw, sizeof(hw), hipMemcpyHostToDevice));
    }
    for (int d = 0; d < MW; d++) HIP_OK(hipMalloc(&recv[d], (size_t)cap[d] * R));
    int64_t *dS, *dcnt, *dboff;
    int32_t *dst, hst = -1;
    void *ws1, *ws2, *ws3;
    const size_t n1 = moe_pack_dispatch_workspace_bytes(MW, MT, MK, ME);
    const size_t n2 = moe_unpack_return_workspace_bytes(MW, ME);
    const size_t n3 = moe_combine_return_workspace_bytes(MW, MT, MK, ME);
    EXPECT(n1 > 0 && n2 > 0 && n3 > 0);
    HIP_OK(hipMalloc((void **)&dS, sizeof(int64_t) * MW * MW));
    HIP_OK(hipMalloc((void **)&dcnt, sizeof(int64_t) * MW * ME));
    HIP_OK(hipMalloc((void **)&dboff, sizeof(int64_t) * MW * (ME / MW + 1)));
    HIP_OK(hipMalloc((void **)&dst, sizeof(int32_t)));
    HIP_OK(hipMalloc(&ws1, n1));
    HIP_OK(hipMalloc(&ws2, n2));
    HIP_OK(hipMalloc(&ws3, n3));
    HIP_OK(hipMemset(dst, 0, sizeof(int32_t)));
    EXPECT(moe_pack_dispatch(MW, MT, MK, ME, R, (const void *const *)tok,
                             (const int32_t *const *)ids, recv, cap, (int64_t *const *)perm, dS,
                             dcnt, dboff, 1, ws1, n1, dst, NULL) == A2AV_OK);
    EXPECT(moe_unpack_return(MW, MT, MK, ME, R, dcnt, (const int32_t *const *)ids,
                             (const int64_t *const *)perm, (const void *const *)recv, cap, home,
                             1, ws2, n2, dst, NULL) == A2AV_OK);
    EXPECT(moe_combine_return(MW, MT, MK, ME, MH, dcnt, (const int32_t *const *)ids,
                              (const int64_t *const *)perm, (const void *const *)recv, cap,
                              (const float *const *)wts, comb, 1, ws3, n3, dst, NULL) == A2AV_OK);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(&hst, dst, sizeof(int32_t), hipMemcpyDeviceToHost));
    EXPECT(hst == 0);
    for (int s = 0; s < MW; s++) {
        HIP_OK(hipMemcpy(hbuf, home[s], sizeof(hbuf), hipMemcpyDeviceToHost));
        for (int q = 0; q < MT * MK; q++)
            for (int h = 0; h < MH; h++) EXPECT(hbuf[q * MH + h] == bf16_of(s, q / MK, h));
        HIP_OK(hipMemcpy(htok, comb[s], sizeof(htok), hipMemcpyDeviceToHost));
        for (int t = 0; t < MT; t++)
            for (int h = 0; h < MH; h++) EXPECT(htok[t * MH + h] == bf16_of(s, t, h));
    }
    for (int s = 0; s < MW; s++) {
        HIP_OK(hipFree(tok[s])); HIP_OK(hipFree(ids[s])); HIP_OK(hipFree(perm[s]));
        HIP_OK(hipFree(home[s])); HIP_OK(hipFree(wts[s])); HIP_OK(hipFree(comb[s]));
        HIP_OK(hipFree(recv[s]));
    }
    HIP_OK(hipFree(dS)); HIP_OK(hipFree(dcnt)); HIP_OK(hipFree(dboff)); HIP_OK(hipFree(dst));
    HIP_OK(hipFree(ws1)); HIP_OK(hipFree(ws2)); HIP_OK(hipFree(ws3));
    return 0;
}

int main(void) {
    EXPECT(a2av_abi_version() == A2AV_ABI_VERSION);
    EXPECT(a2av_exchange_splits(0, NULL, NULL, NULL, NULL) == A2AV_EARG);
    if (run(1) || run(0) || run_moe()) return 1;
    printf("c abi consumer: ok\n");
    return 0;
}
