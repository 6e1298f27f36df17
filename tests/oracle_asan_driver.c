/*
 * Drives the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built and run by test_oracle_sanitized.py, host only). Every buffer is
 * allocated at exactly the size the definition allows, so any read or write
 * past a rank's rows, past an output's capacity or past a permutation is
 * reported. Also checks the round trip and the pack/unpack identity.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "a2av_ref.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) {  /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); exit(1); } } while (0)

static void one_exchange(int W, size_t R, int zero_pct) {
    int64_t *S = malloc(sizeof(int64_t) * W * W), *S2 = malloc(sizeof(int64_t) * W * W);
    int64_t *O = malloc(sizeof(int64_t) * W * W);
    int64_t *so = malloc(sizeof(int64_t) * W * (W + 1)), *ro = malloc(sizeof(int64_t) * W * (W + 1));
    int64_t *rows = malloc(sizeof(int64_t) * W), *cap = calloc(W, sizeof(int64_t));
    unsigned char **in = malloc(sizeof(void *) * W), **out = malloc(sizeof(void *) * W), **back = malloc(sizeof(void *) * W);
    for (int i = 0; i < W * W; i++) S[i] = (int)(next_u64() % 100) < zero_pct ? 0 : (int64_t)(next_u64() % 40);
    for (int s = 0; s < W; s++) {
        rows[s] = 0;
        for (int d = 0; d < W; d++) { rows[s] += S[s * W + d]; cap[d] += S[s * W + d]; }
    }
    for (int s = 0; s < W; s++) {
        in[s] = malloc(rows[s] * R + 1);
        for (int64_t b = 0; b < rows[s] * (int64_t)R; b++) in[s][b] = (unsigned char)next_u64();
        out[s] = malloc(cap[s] * R + 1);
        back[s] = malloc(rows[s] * R + 1);
    }
    CHECK(ref_a2av(W, R, (const void *const *)in, rows, (void *const *)out, cap, S, O, so, ro) == 0);
    CHECK(ref_copy(W, R, (const void *const *)in, rows, (void *const *)out, cap, S, so, ro) == 0);
    memcpy(S2, O, sizeof(int64_t) * W * W);
    CHECK(ref_a2av(W, R, (const void *const *)out, cap, (void *const *)back, rows, S2, O, so, ro) == 0);
    for (int s = 0; s < W; s++) CHECK(memcmp(back[s], in[s], rows[s] * R) == 0);
    for (int d = 0; d < W; d++) {
        for (int64_t j = 0; j < cap[d]; j++) {
            int sr; int64_t i;
            CHECK(ref_source_of(W, S, d, j, &sr, &i) == 0);
            CHECK(memcmp(out[d] + j * R, in[sr] + i * R, R) == 0);
        }
        int sr; int64_t i;
        CHECK(ref_source_of(W, S, d, cap[d], &sr, &i) == 1);
    }
    /* one row too many for rank 0 and one row too few room for rank 0 */
    if (rows[0] > 0) {
        rows[0] -= 1;
        CHECK(ref_a2av(W, R, (const void *const *)in, rows, (void *const *)out, cap, S, O, so, ro) == REF_SEND_OVERRUN);
        rows[0] += 1;
    }
    if (cap[0] > 0) {
        cap[0] -= 1;
        CHECK(ref_a2av(W, R, (const void *const *)in, rows, (void *const *)out, cap, S, O, so, ro) == REF_RECV_OVERFLOW);
        cap[0] += 1;
    }
    for (int s = 0; s < W; s++) { free(in[s]); free(out[s]); free(back[s]); }
    free(in); free(out); free(back); free(S); free(S2); free(O); free(so); free(ro); free(rows); free(cap);
}

static void one_pack(int64_t T, int k, int E, int W, size_t R) {
    int64_t Q = T * k;
    unsigned char *tok = malloc(T * R + 1), *send = malloc(Q * R + 1), *out = malloc(Q * R + 1);
    int32_t *ids = malloc(sizeof(int32_t) * (Q + 1));
    int64_t *perm = malloc(sizeof(int64_t) * (Q + 1)), *splits = malloc(sizeof(int64_t) * W);
    int64_t *counts = malloc(sizeof(int64_t) * E);
    for (int64_t b = 0; b < T * (int64_t)R; b++) tok[b] = (unsigned char)next_u64();
    for (int64_t q = 0; q < Q; q++) ids[q] = (int32_t)(next_u64() % E);
    CHECK(ref_moe_pack(T, k, E, W, R, tok, ids, send, perm, splits, counts) == 0);
    CHECK(ref_moe_unpack(T, k, R, send, perm, out) == 0);
    for (int64_t q = 0; q < Q; q++) CHECK(memcmp(out + q * R, tok + (q / k) * R, R) == 0);
    if (Q > 0) {
        ids[Q / 2] = E;
        CHECK(ref_moe_pack(T, k, E, W, R, tok, ids, send, perm, splits, counts) == REF_BAD_EXPERT);
    }
    free(tok); free(send); free(out); free(ids); free(perm); free(splits); free(counts);
}

/* pack on every rank, regroup each rank's received rows to expert-major and
 * back, on buffers of exactly the received size */
static void one_regroup(int W, int E, size_t R) {
    int64_t *counts = malloc(sizeof(int64_t) * W * E);
    const int P = E / W;
    for (int i = 0; i < W * E; i++) counts[i] = (int64_t)(next_u64() % 5);
    for (int d = 0; d < W; d++) {
        int64_t n = 0;
        for (int s = 0; s < W; s++)
            for (int j = 0; j < P; j++) n += counts[s * E + d * P + j];
        unsigned char *in = malloc(n * R + 1), *mid = malloc(n * R + 1), *back = malloc(n * R + 1);
        int64_t *eoff = malloc(sizeof(int64_t) * (P + 1));
        for (int64_t b = 0; b < n * (int64_t)R; b++) in[b] = (unsigned char)next_u64();
        CHECK(ref_moe_regroup(W, E, d, R, counts, in, n, mid, n, eoff, 0) == 0);
        CHECK(eoff[P] == n);
        CHECK(ref_moe_regroup(W, E, d, R, counts, mid, n, back, n, eoff, 1) == 0);
        CHECK(n == 0 || memcmp(in, back, n * R) == 0);
        if (n > 0) {
            CHECK(ref_moe_regroup(W, E, d, R, counts, in, n - 1, mid, n, eoff, 0) == REF_SEND_OVERRUN);
            CHECK(ref_moe_regroup(W, E, d, R, counts, in, n, mid, n - 1, eoff, 0) == REF_RECV_OVERFLOW);
        }
        free(in); free(mid); free(back); free(eoff);
    }
    free(counts);
}

static void one_combine(int64_t T, int k, int64_t H) {
    const int64_t Q = T * k;
    uint16_t *back = malloc(sizeof(uint16_t) * (Q * H + 1)), *out = malloc(sizeof(uint16_t) * (T * H + 1));
    int64_t *perm = malloc(sizeof(int64_t) * (Q + 1));
    float *w = malloc(sizeof(float) * (Q + 1));
    for (int64_t i = 0; i < Q * H; i++) back[i] = (uint16_t)next_u64();  /* any bits, NaNs too */
    for (int64_t q = 0; q < Q; q++) { perm[q] = q; w[q] = (float)(next_u64() % 1000) / 999.0f; }
    for (int64_t q = Q - 1; q > 0; q--) {
        int64_t r = (int64_t)(next_u64() % (uint64_t)(q + 1)), t = perm[q];
        perm[q] = perm[r]; perm[r] = t;
    }
    CHECK(ref_moe_combine(T, k, H, back, perm, w, out) == 0);
    if (Q > 0) {
        perm[Q - 1] = Q;
        CHECK(ref_moe_combine(T, k, H, back, perm, w, out) == REF_BAD_PERM);
    }
    free(back); free(out); free(perm); free(w);
}

static void one_bucketize(int W, int n_tables, int64_t batch) {
    const int64_t nl = (int64_t)n_tables * batch;
    int32_t *len = malloc(sizeof(int32_t) * (nl + 1)), *lo = malloc(sizeof(int32_t) * (nl + 1));
    int64_t n = 0;
    for (int64_t i = 0; i < nl; i++) { len[i] = (int32_t)(next_u64() % 7); n += len[i]; }
    int64_t *keys = malloc(sizeof(int64_t) * (n + 1)), *ko = malloc(sizeof(int64_t) * (n + 1));
    int64_t *sk = malloc(sizeof(int64_t) * W), *sl = malloc(sizeof(int64_t) * W);
    for (int64_t i = 0; i < n; i++) keys[i] = (int64_t)(next_u64() >> 1);
    CHECK(ref_keys_bucketize(W, n_tables, batch, len, keys, n, lo, ko, sk, sl) == 0);
    int64_t tk = 0, tl = 0;
    for (int d = 0; d < W; d++) { tk += sk[d]; tl += sl[d]; }
    CHECK(tk == n && tl == nl);
    if (n > 0) CHECK(ref_keys_bucketize(W, n_tables, batch, len, keys, n - 1, lo, ko, sk, sl) == REF_SEND_OVERRUN);
    free(len); free(lo); free(keys); free(ko); free(sk); free(sl);
}

static void one_keys_exchange(int W, int n_tables, int64_t batch) {
    const int64_t nl = (int64_t)n_tables * batch;
    int32_t **len = malloc(sizeof(int32_t *) * W), **lo = malloc(sizeof(int32_t *) * W);
    int64_t **keys = malloc(sizeof(int64_t *) * W), **ko = malloc(sizeof(int64_t *) * W);
    int64_t *nk = malloc(sizeof(int64_t) * W), *kcap = calloc(W, sizeof(int64_t));
    int64_t *lcap = calloc(W, sizeof(int64_t));
    int64_t *sk = malloc(sizeof(int64_t) * W * W), *sl = malloc(sizeof(int64_t) * W * W);
    int64_t *ro = malloc(sizeof(int64_t) * W * (W + 1));
    for (int s = 0; s < W; s++) {
        len[s] = malloc(sizeof(int32_t) * (nl + 1));
        nk[s] = 0;
        for (int64_t i = 0; i < nl; i++) {
            len[s][i] = (int32_t)(next_u64() % 5);
            nk[s] += len[s][i];
            kcap[(i / (batch > 0 ? batch : 1)) % W] += len[s][i];
        }
        keys[s] = malloc(sizeof(int64_t) * (nk[s] + 1));
        for (int64_t i = 0; i < nk[s]; i++) keys[s][i] = (int64_t)(next_u64() >> 2);
    }
    for (int d = 0; d < W; d++) {
        for (int t = d; t < n_tables; t += W) lcap[d] += (int64_t)W * batch;
        lo[d] = malloc(sizeof(int32_t) * (lcap[d] + 1));
        ko[d] = malloc(sizeof(int64_t) * (kcap[d] + 1));
    }
    CHECK(ref_keys_exchange(W, n_tables, batch, (const int32_t *const *)len,
                            (const int64_t *const *)keys, nk, lo, lcap, ko, kcap, sk, sl, ro) == 0);
    if (kcap[0] > 0) {
        kcap[0] -= 1;
        CHECK(ref_keys_exchange(W, n_tables, batch, (const int32_t *const *)len,
                                (const int64_t *const *)keys, nk, lo, lcap, ko, kcap, sk, sl, ro) ==
              REF_RECV_OVERFLOW);
    }
    for (int s = 0; s < W; s++) { free(len[s]); free(keys[s]); free(lo[s]); free(ko[s]); }
    free(len); free(lo); free(keys); free(ko); free(nk); free(kcap); free(lcap);
    free(sk); free(sl); free(ro);
}

static void one_grouped(int W, int E, size_t R) {
    const int P = E / W;
    int64_t *counts = malloc(sizeof(int64_t) * W * E);
    int64_t *rows = calloc(W, sizeof(int64_t)), *cap = calloc(W, sizeof(int64_t));
    int64_t *eoff = malloc(sizeof(int64_t) * W * (P + 1));
    for (int i = 0; i < W * E; i++) counts[i] = (int64_t)(next_u64() % 4);
    for (int s = 0; s < W; s++)
        for (int e = 0; e < E; e++) { rows[s] += counts[s * E + e]; cap[e / P] += counts[s * E + e]; }
    unsigned char **in = malloc(sizeof(void *) * W), **out = malloc(sizeof(void *) * W);
    unsigned char **back = malloc(sizeof(void *) * W);
    for (int r = 0; r < W; r++) {
        in[r] = malloc(rows[r] * R + 1);
        back[r] = malloc(rows[r] * R + 1);
        out[r] = malloc(cap[r] * R + 1);
        for (int64_t b = 0; b < rows[r] * (int64_t)R; b++) in[r][b] = (unsigned char)next_u64();
    }
    CHECK(ref_moe_dispatch_grouped(W, E, R, counts, (const void *const *)in, rows,
                                   (void *const *)out, cap, eoff, 0) == 0);
    CHECK(ref_moe_dispatch_grouped(W, E, R, counts, (const void *const *)out, cap,
                                   (void *const *)back, rows, eoff, 1) == 0);
    for (int r = 0; r < W; r++) CHECK(rows[r] == 0 || memcmp(in[r], back[r], rows[r] * R) == 0);
    for (int r = 0; r < W; r++) { free(in[r]); free(out[r]); free(back[r]); }
    free(in); free(out); free(back); free(counts); free(rows); free(cap); free(eoff);
}

/* pack, grouped dispatch, then the combine read from the expert side */
static void one_combine_grouped(int W, int64_t T, int k, int E, int64_t H) {
    const int P = E / W;
    const int64_t Q = T * k;
    int64_t *counts = malloc(sizeof(int64_t) * W * E), *exp_rows = calloc(W, sizeof(int64_t));
    int32_t **ids = malloc(sizeof(void *) * W);
    int64_t **perm = malloc(sizeof(void *) * W);
    float **w = malloc(sizeof(void *) * W);
    uint16_t **out = malloc(sizeof(void *) * W), **xs = malloc(sizeof(void *) * W);
    unsigned char *tok = calloc((size_t)T + 1, 1), *send = malloc((size_t)Q + 1);
    int64_t *splits = malloc(sizeof(int64_t) * W);
    for (int s = 0; s < W; s++) {
        ids[s] = malloc(sizeof(int32_t) * (Q + 1));
        perm[s] = malloc(sizeof(int64_t) * (Q + 1));
        w[s] = malloc(sizeof(float) * (Q + 1));
        out[s] = malloc(sizeof(uint16_t) * (T * H + 1));
        for (int64_t q = 0; q < Q; q++) { ids[s][q] = (int32_t)(next_u64() % E); w[s][q] = 0.5f; }
        CHECK(ref_moe_pack(T, k, E, W, 1, tok, ids[s], send, perm[s], splits, counts + (size_t)s * E) == 0);
    }
    for (int s = 0; s < W; s++)
        for (int e = 0; e < E; e++) exp_rows[e / P] += counts[s * E + e];
    for (int d = 0; d < W; d++) {
        xs[d] = malloc(sizeof(uint16_t) * (exp_rows[d] * H + 1));
        for (int64_t i = 0; i < exp_rows[d] * H; i++) xs[d][i] = (uint16_t)(next_u64() & 0x7F7F);
    }
    CHECK(ref_moe_combine_grouped(W, T, k, E, H, counts, (const int32_t *const *)ids,
                                  (const int64_t *const *)perm, (const uint16_t *const *)xs,
                                  exp_rows, (const float *const *)w, out) == 0);
    for (int s = 0; s < W; s++) { free(ids[s]); free(perm[s]); free(w[s]); free(out[s]); free(xs[s]); }
    free(ids); free(perm); free(w); free(out); free(xs); free(counts); free(exp_rows);
    free(tok); free(send); free(splits);
}

/* pack + dispatch in one step and its inverse, both layouts: every slot comes home */
static void one_pack_dispatch(int W, int64_t T, int k, int E, size_t R, int layout) {
    const int P = E / W;
    const int64_t Q = T * k;
    const int G = layout == 0 ? W : P;
    void **tok = malloc(sizeof(void *) * W), **recv = malloc(sizeof(void *) * W);
    void **out = malloc(sizeof(void *) * W);
    int32_t **ids = malloc(sizeof(void *) * W);
    int64_t **perm = malloc(sizeof(void *) * W);
    int64_t *S = malloc(sizeof(int64_t) * W * W), *counts = malloc(sizeof(int64_t) * W * E);
    int64_t *boff = malloc(sizeof(int64_t) * W * (G + 1)), *cap = malloc(sizeof(int64_t) * W);
    int64_t *rows = malloc(sizeof(int64_t) * W);
    for (int s = 0; s < W; s++) {
        tok[s] = malloc((size_t)T * R + 1);
        for (int64_t i = 0; i < T * (int64_t)R; i++) ((unsigned char *)tok[s])[i] = (unsigned char)next_u64();
        ids[s] = malloc(sizeof(int32_t) * (Q + 1));
        perm[s] = malloc(sizeof(int64_t) * (Q + 1));
        out[s] = malloc((size_t)Q * R + 1);
        for (int64_t q = 0; q < Q; q++) ids[s][q] = (int32_t)(next_u64() % E);
    }
    for (int d = 0; d < W; d++) {
        rows[d] = 0;
        for (int s = 0; s < W; s++)
            for (int64_t q = 0; q < Q; q++) rows[d] += ids[s][q] / P == d;
        cap[d] = rows[d];
        recv[d] = malloc((size_t)rows[d] * R + 1);
    }
    CHECK(ref_moe_pack_dispatch(W, T, k, E, R, (const void *const *)tok,
                                (const int32_t *const *)ids, recv, cap, perm, S, counts, boff,
                                layout) == 0);
    CHECK(ref_moe_unpack_return(W, T, k, E, R, counts, (const int32_t *const *)ids,
                                (const int64_t *const *)perm, (const void *const *)recv, rows, out,
                                layout) == 0);
    if (R % 2 == 0) {  /* the same rows as bf16: the weighted combine at the owners */
        const int64_t H = (int64_t)R / 2;
        float **w = malloc(sizeof(void *) * W);
        uint16_t **cout = malloc(sizeof(void *) * W);
        for (int s = 0; s < W; s++) {
            w[s] = malloc(sizeof(float) * (Q + 1));
            for (int64_t q = 0; q < Q; q++) w[s][q] = 0.25f;
            cout[s] = malloc(sizeof(uint16_t) * (T * H + 1));
        }
        CHECK(ref_moe_combine_return(W, T, k, E, H, counts, (const int32_t *const *)ids,
                                     (const int64_t *const *)perm, (const uint16_t *const *)recv,
                                     rows, (const float *const *)w, cout, layout) == 0);
        for (int s = 0; s < W; s++) { free(w[s]); free(cout[s]); }
        free(w); free(cout);
    }
    for (int s = 0; s < W; s++)
        for (int64_t q = 0; q < Q; q++)
            CHECK(memcmp((unsigned char *)out[s] + q * R, (unsigned char *)tok[s] + (q / k) * R, R) == 0);
    for (int s = 0; s < W; s++) { free(tok[s]); free(recv[s]); free(out[s]); free(ids[s]); free(perm[s]); }
    free(tok); free(recv); free(out); free(ids); free(perm); free(S); free(counts); free(boff);
    free(cap); free(rows);
}

int main(void) {
    const size_t widths[] = {1, 3, 8, 16, 100};
    for (int W = 1; W <= 9; W++)
        for (int wi = 0; wi < 5; wi++)
            for (int z = 0; z <= 80; z += 40) one_exchange(W, widths[wi], z);
    one_exchange(64, 4, 50);
    one_exchange(64, 1, 0);
    one_pack(200, 8, 256, 8, 16);
    one_pack(333, 3, 12, 4, 5);
    one_pack(1, 1, 1, 1, 1);
    one_pack(0, 2, 8, 2, 4);
    one_regroup(8, 256, 16);
    one_regroup(3, 12, 7);
    one_regroup(1, 1, 1);
    one_combine(50, 8, 33);
    one_combine(0, 2, 4);
    one_combine(7, 1, 1);
    one_bucketize(8, 26, 64);
    one_bucketize(3, 2, 0);
    one_bucketize(5, 0, 10);
    one_combine_grouped(8, 100, 8, 256, 24);
    one_combine_grouped(3, 17, 2, 6, 5);
    one_combine_grouped(1, 1, 1, 1, 1);
    one_grouped(8, 256, 16);
    one_grouped(3, 12, 5);
    one_grouped(1, 1, 1);
    for (int layout = 0; layout < 2; layout++) {
        one_pack_dispatch(8, 60, 8, 256, 16, layout);
        one_pack_dispatch(3, 17, 2, 6, 5, layout);
        one_pack_dispatch(1, 1, 1, 1, 1, layout);
        one_pack_dispatch(4, 0, 2, 8, 3, layout);
    }
    one_keys_exchange(8, 26, 32);
    one_keys_exchange(3, 2, 5);
    one_keys_exchange(1, 3, 4);
    one_keys_exchange(4, 0, 7);
    printf("oracle sanitized: ok\n");
    return 0;
}
