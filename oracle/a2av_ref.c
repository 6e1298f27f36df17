/*
 * a2av_ref.c — CPU oracle (plain, slow, single-threaded C).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. Shares no code with
 * the HIP library. Each function writes out the definition it follows, step by
 * step, with no blocking, fusion or reordering.
 *
 * Reading of the operation (the pages name nvshmem_all_to_all_vdev in the
 * "Problem" section of "[a2av] Improve tuning for 4 GPUs" but never define
 * it): all-to-all-v with device-held counts.
 *   1. splits must be valid (non-negative, at most REF_MAX_SPLIT rows);
 *   2. output splits O[d][s] = S[s][d];
 *   3. send_off[s][d] = sum_{d' < d} S[s][d'], total at index W;
 *      the total may not exceed the rows rank s holds;
 *   4. recv_off[d][s] = sum_{s' < s} O[d][s'], total at index W;
 *      the total may not exceed the rows rank d can hold;
 *   5. for each d, for each s in ascending order, copy S[s][d] rows from
 *      rank s's input at send_off[s][d] to rank d's output at recv_off[d][s];
 *   6. nothing past a destination's total is touched; on any failure no
 *      payload byte is written.
 */
#include "a2av_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int split_is_valid(int64_t v) { return v >= 0 && v <= REF_MAX_SPLIT; }

/* Host-side argument checks shared by the payload functions of this file. */
static int check_rank_sizes(int W, size_t R, const void *const *bufs,
                            const int64_t *rows) {
    if (W < 1 || W > REF_MAX_W || R == 0 || bufs == NULL || rows == NULL)
        return REF_EARG;
    for (int r = 0; r < W; r++) {
        if (rows[r] < 0) return REF_EARG;
        if ((uint64_t)rows[r] > (uint64_t)INT64_MAX / R) return REF_EARG;
        if (rows[r] > 0 && bufs[r] == NULL) return REF_EARG;
    }
    return 0;
}

int ref_exchange_splits(int W, const int64_t *S, int64_t *O) {
    if (W < 1 || W > REF_MAX_W || S == NULL || O == NULL) return REF_EARG;
    for (int s = 0; s < W; s++)
        for (int d = 0; d < W; d++)
            if (!split_is_valid(S[s * W + d])) return REF_BAD_SPLIT;
    /* Step 2: the receive counts are the transpose of the send counts. */
    for (int d = 0; d < W; d++)
        for (int s = 0; s < W; s++)
            O[d * W + s] = S[s * W + d];
    return 0;
}

int ref_offsets(int W, const int64_t *S, const int64_t *O,
                int64_t *send_off, int64_t *recv_off) {
    if (W < 1 || W > REF_MAX_W || !S || !O || !send_off || !recv_off)
        return REF_EARG;
    for (int i = 0; i < W * W; i++)
        if (!split_is_valid(S[i]) || !split_is_valid(O[i])) return REF_BAD_SPLIT;
    /* Step 3: exclusive scan of each send row; the total lands at index W. */
    for (int s = 0; s < W; s++) {
        int64_t run = 0;
        for (int d = 0; d < W; d++) {
            send_off[s * (W + 1) + d] = run;
            run += S[s * W + d];
        }
        send_off[s * (W + 1) + W] = run;
    }
    /* Step 4: exclusive scan of each receive row. */
    for (int d = 0; d < W; d++) {
        int64_t run = 0;
        for (int s = 0; s < W; s++) {
            recv_off[d * (W + 1) + s] = run;
            run += O[d * W + s];
        }
        recv_off[d * (W + 1) + W] = run;
    }
    return 0;
}

/* Step 5 alone, once every check has passed. */
static void copy_chunks(int W, size_t R, const void *const *in,
                        void *const *out, const int64_t *S,
                        const int64_t *send_off, const int64_t *recv_off) {
    for (int d = 0; d < W; d++) {
        for (int s = 0; s < W; s++) {
            int64_t rows = S[s * W + d];
            if (rows == 0) continue;
            const unsigned char *src =
                (const unsigned char *)in[s] + (size_t)send_off[s * (W + 1) + d] * R;
            unsigned char *dst =
                (unsigned char *)out[d] + (size_t)recv_off[d * (W + 1) + s] * R;
            memcpy(dst, src, (size_t)rows * R);
        }
    }
}

int ref_copy(int W, size_t R,
             const void *const *in, const int64_t *in_rows,
             void *const *out, const int64_t *out_cap_rows,
             const int64_t *S, const int64_t *send_off, const int64_t *recv_off) {
    if (check_rank_sizes(W, R, in, in_rows) || check_rank_sizes(W, R, (const void *const *)out, out_cap_rows))
        return REF_EARG;
    if (!S || !send_off || !recv_off) return REF_EARG;

    int st = 0;
    for (int i = 0; i < W * W; i++)
        if (!split_is_valid(S[i])) st |= REF_BAD_SPLIT;

    /* The given offsets must be the scans of step 3 and 4 (compared modulo
     * 2^64 so that garbage input cannot overflow a signed add). */
    for (int s = 0; s < W; s++) {
        if (send_off[s * (W + 1)] != 0) st |= REF_BAD_OFFSETS;
        for (int d = 0; d < W; d++) {
            uint64_t step = (uint64_t)send_off[s * (W + 1) + d + 1] -
                            (uint64_t)send_off[s * (W + 1) + d];
            if (step != (uint64_t)S[s * W + d]) st |= REF_BAD_OFFSETS;
        }
    }
    for (int d = 0; d < W; d++) {
        if (recv_off[d * (W + 1)] != 0) st |= REF_BAD_OFFSETS;
        for (int s = 0; s < W; s++) {
            uint64_t step = (uint64_t)recv_off[d * (W + 1) + s + 1] -
                            (uint64_t)recv_off[d * (W + 1) + s];
            if (step != (uint64_t)S[s * W + d]) st |= REF_BAD_OFFSETS;
        }
    }
    /* Step 3 and 4 bounds, on the totals as given. */
    for (int s = 0; s < W; s++)
        if (send_off[s * (W + 1) + W] > in_rows[s]) st |= REF_SEND_OVERRUN;
    for (int d = 0; d < W; d++)
        if (recv_off[d * (W + 1) + W] > out_cap_rows[d]) st |= REF_RECV_OVERFLOW;
    if (st) return st;

    copy_chunks(W, R, in, out, S, send_off, recv_off);
    return 0;
}

int ref_a2av(int W, size_t R,
             const void *const *in, const int64_t *in_rows,
             void *const *out, const int64_t *out_cap_rows,
             const int64_t *S, int64_t *O, int64_t *send_off, int64_t *recv_off) {
    if (check_rank_sizes(W, R, in, in_rows) || check_rank_sizes(W, R, (const void *const *)out, out_cap_rows))
        return REF_EARG;
    if (!S || !O || !send_off || !recv_off) return REF_EARG;

    int st = ref_exchange_splits(W, S, O);
    if (st) return st;
    st = ref_offsets(W, S, O, send_off, recv_off);
    if (st) return st;
    for (int s = 0; s < W; s++)
        if (send_off[s * (W + 1) + W] > in_rows[s]) st |= REF_SEND_OVERRUN;
    for (int d = 0; d < W; d++)
        if (recv_off[d * (W + 1) + W] > out_cap_rows[d]) st |= REF_RECV_OVERFLOW;
    if (st) return st;
    copy_chunks(W, R, in, out, S, send_off, recv_off);
    return 0;
}

int ref_source_of(int W, const int64_t *S, int d, int64_t j,
                  int *src_rank, int64_t *src_row) {
    if (W < 1 || W > REF_MAX_W || !S || d < 0 || d >= W || j < 0 ||
        !src_rank || !src_row)
        return REF_EARG;
    for (int i = 0; i < W * W; i++)
        if (!split_is_valid(S[i])) return REF_EARG;
    /* Walk rank d's receive row in source order (step 4) until row j falls
     * inside source s's chunk; then step 3 gives the row inside in[s]. */
    int64_t recv_start = 0;
    for (int s = 0; s < W; s++) {
        int64_t rows = S[s * W + d];
        if (j < recv_start + rows) {
            int64_t send_start = 0;
            for (int dd = 0; dd < d; dd++) send_start += S[s * W + dd];
            *src_rank = s;
            *src_row = send_start + (j - recv_start);
            return 0;
        }
        recv_start += rows;
    }
    return 1;
}

/*
 * MoE dispatch pack of one rank, as a stable counting sort of the T*k routing
 * slots by expert id (tokens routed to experts, then grouped by the rank that
 * owns each expert; the page's "MoE related region" is the message this
 * builds). Experts are owned in contiguous blocks: owner(e) = e / (E / W),
 * so sorting by expert also groups by destination rank.
 */
int ref_moe_pack(int64_t T, int k, int E, int W, size_t R,
                 const void *tokens, const int32_t *ids,
                 void *send, int64_t *perm, int64_t *splits,
                 int64_t *expert_counts) {
    if (T < 0 || k < 1 || E < 1 || W < 1 || W > REF_MAX_W || E % W != 0 || R == 0)
        return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int64_t Q = T * k;
    if (Q > 0 && (!tokens || !ids || !send || !perm)) return REF_EARG;
    if (!splits || !expert_counts) return REF_EARG;

    /* Every id must name an expert before anything is written. */
    for (int64_t q = 0; q < Q; q++)
        if (ids[q] < 0 || ids[q] >= E) return REF_BAD_EXPERT;

    int64_t *count = calloc((size_t)E, sizeof(int64_t));
    int64_t *next = calloc((size_t)E, sizeof(int64_t));
    if (!count || !next) { free(count); free(next); return REF_EARG; }

    /* count[e] = number of slots routed to expert e. */
    for (int64_t q = 0; q < Q; q++) count[ids[q]] += 1;
    /* base[e] = slots of all smaller experts; next[e] starts at base[e]. */
    int64_t run = 0;
    for (int e = 0; e < E; e++) { next[e] = run; run += count[e]; }
    /* perm[q] = base[e(q)] + number of earlier slots with the same expert. */
    for (int64_t q = 0; q < Q; q++) perm[q] = next[ids[q]]++;
    /* send[perm[q]] = the token of slot q. */
    for (int64_t q = 0; q < Q; q++)
        memcpy((unsigned char *)send + (size_t)perm[q] * R,
               (const unsigned char *)tokens + (size_t)(q / k) * R, R);
    /* splits[d] = slots whose expert rank d owns. */
    const int per_rank = E / W;
    for (int d = 0; d < W; d++) splits[d] = 0;
    for (int e = 0; e < E; e++) splits[e / per_rank] += count[e];
    for (int e = 0; e < E; e++) expert_counts[e] = count[e];

    free(count);
    free(next);
    return 0;
}

int ref_moe_unpack(int64_t T, int k, size_t R,
                   const void *back, const int64_t *perm, void *out) {
    if (T < 0 || k < 1 || R == 0) return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int64_t Q = T * k;
    if (Q > 0 && (!back || !perm || !out)) return REF_EARG;
    for (int64_t q = 0; q < Q; q++)
        if (perm[q] < 0 || perm[q] >= Q) return REF_BAD_PERM;
    /* out[q] = back[perm[q]]: the row that slot q was packed to comes home. */
    for (int64_t q = 0; q < Q; q++)
        memcpy((unsigned char *)out + (size_t)q * R,
               (const unsigned char *)back + (size_t)perm[q] * R, R);
    return 0;
}

/*
 * Receive-side expert regroup of one rank: the step after the dispatch, so
 * that each expert's rows sit together for its GEMM. Rank d receives from
 * each source the rows routed to d's experts, ordered by expert; regrouping
 * makes the order (expert, source) instead of (source, expert).
 */
int ref_moe_regroup(int W, int E, int d, size_t R, const int64_t *counts,
                    const void *in, int64_t in_rows, void *out, int64_t out_cap,
                    int64_t *expert_offsets, int direction) {
    if (W < 1 || W > REF_MAX_W || E < 1 || E % W != 0 || d < 0 || d >= W || R == 0 ||
        !counts || !expert_offsets || in_rows < 0 || out_cap < 0 ||
        (direction != 0 && direction != 1))
        return REF_EARG;
    const int P = E / W;
    /* the P owned columns of counts */
    for (int s = 0; s < W; s++)
        for (int j = 0; j < P; j++)
            if (!split_is_valid(counts[s * E + d * P + j])) return REF_BAD_SPLIT;
    int64_t total = 0;
    for (int s = 0; s < W; s++)
        for (int j = 0; j < P; j++) total += counts[s * E + d * P + j];
    int st = 0;
    if (total > in_rows) st |= REF_SEND_OVERRUN;
    if (total > out_cap) st |= REF_RECV_OVERFLOW;
    if (st) return st;
    if (total > 0 && (!in || !out)) return REF_EARG;
    /* expert-major offsets */
    int64_t run = 0;
    for (int j = 0; j < P; j++) {
        expert_offsets[j] = run;
        for (int s = 0; s < W; s++) run += counts[s * E + d * P + j];
    }
    expert_offsets[P] = run;
    /* walk the blocks in source-major order, keeping both positions */
    int64_t src_major = 0;
    for (int s = 0; s < W; s++) {
        for (int j = 0; j < P; j++) {
            const int64_t n = counts[s * E + d * P + j];
            int64_t expert_major = expert_offsets[j];
            for (int s2 = 0; s2 < s; s2++) expert_major += counts[s2 * E + d * P + j];
            const int64_t from = direction == 0 ? src_major : expert_major;
            const int64_t to = direction == 0 ? expert_major : src_major;
            if (n > 0)
                memcpy((unsigned char *)out + (size_t)to * R,
                       (const unsigned char *)in + (size_t)from * R, (size_t)n * R);
            src_major += n;
        }
    }
    return 0;
}

/* bfloat16 is the top half of an IEEE binary32. */
static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary32 to bfloat16, to nearest, ties to even. Every NaN becomes
 * the canonical quiet NaN 0x7FC0: IEEE 754 leaves the sign and payload of a
 * NaN result open, so they are not part of the result. */
static uint16_t float_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return 0x7FC0u;
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

int ref_moe_combine(int64_t T, int k, int64_t H, const uint16_t *back,
                    const int64_t *perm, const float *w, uint16_t *out) {
    if (T < 0 || k < 1 || H < 1) return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int64_t Q = T * k;
    if (Q > 0 && (!back || !perm || !w || !out)) return REF_EARG;
    for (int64_t q = 0; q < Q; q++)
        if (perm[q] < 0 || perm[q] >= Q) return REF_BAD_PERM;
    for (int64_t t = 0; t < T; t++) {
        for (int64_t h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int j = 0; j < k; j++) {
                const int64_t row = perm[t * k + j];
                acc = fmaf(w[t * k + j], bf16_to_float(back[row * H + h]), acc);
            }
            out[t * H + h] = float_to_bf16(acc);
        }
    }
    return 0;
}

/* Embedding keys bucketed by the rank that owns their table, before the key
 * exchange: tables in (owner, table) order, samples in order inside a table. */
int ref_keys_bucketize(int W, int n_tables, int64_t batch, const int32_t *lengths,
                       const int64_t *keys, int64_t n_keys, int32_t *lengths_out,
                       int64_t *keys_out, int64_t *split_keys, int64_t *split_lengths) {
    if (W < 1 || W > REF_MAX_W || n_tables < 0 || batch < 0 || n_keys < 0 || !split_keys ||
        !split_lengths)
        return REF_EARG;
    if (n_tables > 0 && batch > INT64_MAX / n_tables) return REF_EARG;
    const int64_t nl = (int64_t)n_tables * batch;
    if (nl > 0 && (!lengths || !lengths_out)) return REF_EARG;
    for (int64_t i = 0; i < nl; i++)
        if (lengths[i] < 0) return REF_BAD_SPLIT;
    /* keys of each table and where they start in the input */
    int64_t *tk = calloc((size_t)(n_tables > 0 ? n_tables : 1), sizeof(int64_t));
    int64_t *tstart = calloc((size_t)(n_tables > 0 ? n_tables : 1), sizeof(int64_t));
    if (!tk || !tstart) { free(tk); free(tstart); return REF_EARG; }
    int64_t run = 0;
    for (int t = 0; t < n_tables; t++) {
        tstart[t] = run;
        for (int64_t b = 0; b < batch; b++) tk[t] += lengths[(int64_t)t * batch + b];
        run += tk[t];
    }
    if (run > n_keys) { free(tk); free(tstart); return REF_SEND_OVERRUN; }
    if (run > 0 && (!keys || !keys_out)) { free(tk); free(tstart); return REF_EARG; }
    for (int d = 0; d < W; d++) { split_keys[d] = 0; split_lengths[d] = 0; }
    int64_t kpos = 0, lpos = 0;
    for (int d = 0; d < W; d++) {
        for (int t = d; t < n_tables; t += W) {  /* tables owned by d, ascending */
            if (batch > 0)
                memcpy(lengths_out + lpos, lengths + (int64_t)t * batch, (size_t)batch * 4);
            if (tk[t] > 0)
                memcpy(keys_out + kpos, keys + tstart[t], (size_t)tk[t] * 8);
            lpos += batch;
            kpos += tk[t];
            split_keys[d] += tk[t];
            split_lengths[d] += batch;
        }
    }
    free(tk);
    free(tstart);
    return 0;
}

/*
 * The whole embedding-key exchange of one batch, as the plain composition of
 * its two steps: every rank buckets its keys by owner (ref_keys_bucketize),
 * then keys and lengths go out as two all-to-all-v calls whose splits are the
 * bucketing's split rows. Checks in the order the composition meets them:
 * the bucketing of every source first (their bits are the result if any
 * fails), then the receive capacities; payload only when all pass.
 */
int ref_keys_exchange(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                      const int64_t *const *keys, const int64_t *n_keys,
                      int32_t *const *lengths_out, const int64_t *lengths_cap,
                      int64_t *const *keys_out, const int64_t *keys_cap, int64_t *split_keys,
                      int64_t *split_lengths, int64_t *recv_off_keys) {
    if (W < 1 || W > REF_MAX_W || n_tables < 0 || batch < 0 || !lengths || !keys || !n_keys ||
        !lengths_out || !lengths_cap || !keys_out || !keys_cap || !split_keys ||
        !split_lengths || !recv_off_keys)
        return REF_EARG;
    if (n_tables > 0 && batch > INT64_MAX / n_tables) return REF_EARG;
    const int64_t nl = (int64_t)n_tables * batch;
    int st = 0;
    int32_t **lo = calloc((size_t)W, sizeof(int32_t *));
    int64_t **ko = calloc((size_t)W, sizeof(int64_t *));
    int64_t *Sk = calloc((size_t)W * W, sizeof(int64_t));
    int64_t *Sl = calloc((size_t)W * W, sizeof(int64_t));
    if (!lo || !ko || !Sk || !Sl) { st = REF_EARG; goto done; }
    /* step 1: bucketing on every source rank */
    for (int s = 0; s < W; s++) {
        if (n_keys[s] < 0) { st = REF_EARG; goto done; }
        lo[s] = malloc((size_t)(nl > 0 ? nl : 1) * sizeof(int32_t));
        ko[s] = malloc((size_t)(n_keys[s] > 0 ? n_keys[s] : 1) * sizeof(int64_t));
        if (!lo[s] || !ko[s]) { st = REF_EARG; goto done; }
        st |= ref_keys_bucketize(W, n_tables, batch, lengths[s], keys[s], n_keys[s], lo[s], ko[s],
                                 Sk + (size_t)s * W, Sl + (size_t)s * W);
    }
    if (st) goto done;
    /* step 2: what each receiver gets against its capacities */
    for (int d = 0; d < W; d++) {
        int64_t rk = 0, rl = 0;
        for (int s = 0; s < W; s++) { rk += Sk[s * W + d]; rl += Sl[s * W + d]; }
        if (rk > keys_cap[d] || rl > lengths_cap[d]) { st |= REF_RECV_OVERFLOW; continue; }
        /* this receiver's split columns and receive offsets */
        int64_t run = 0;
        for (int s = 0; s < W; s++) {
            split_keys[s * W + d] = Sk[s * W + d];
            split_lengths[s * W + d] = Sl[s * W + d];
            recv_off_keys[d * (W + 1) + s] = run;
            run += Sk[s * W + d];
        }
        recv_off_keys[d * (W + 1) + W] = run;
    }
    if (st) goto done;
    /* step 3: the two exchanges */
    {
        int64_t *rows_k = malloc((size_t)W * sizeof(int64_t));
        int64_t *rows_l = malloc((size_t)W * sizeof(int64_t));
        int64_t *O = malloc((size_t)W * W * sizeof(int64_t));
        int64_t *so = malloc((size_t)W * (W + 1) * sizeof(int64_t));
        int64_t *ro = malloc((size_t)W * (W + 1) * sizeof(int64_t));
        if (!rows_k || !rows_l || !O || !so || !ro) {
            st = REF_EARG;
        } else {
            for (int s = 0; s < W; s++) { rows_k[s] = n_keys[s]; rows_l[s] = nl; }
            st |= ref_a2av(W, 8, (const void *const *)ko, rows_k, (void *const *)keys_out, keys_cap,
                           Sk, O, so, ro);
            if (!st)
                st |= ref_a2av(W, 4, (const void *const *)lo, rows_l, (void *const *)lengths_out,
                               lengths_cap, Sl, O, so, ro);
        }
        free(rows_k); free(rows_l); free(O); free(so); free(ro);
    }
done:
    if (lo) for (int s = 0; s < W; s++) free(lo[s]);
    if (ko) for (int s = 0; s < W; s++) free(ko[s]);
    free(lo); free(ko); free(Sk); free(Sl);
    return st;
}

/*
 * The MoE dispatch with its receive-side regroup in one step, and its
 * inverse. Pack side: rank s's rows in pack order (expert ascending, the
 * counts[s][e] rows of expert e at Σ_{e'<e} counts[s][e']). Expert side:
 * rank d's rows in expert-major order (owned expert j outer, source s inner).
 * Direction 0 moves pack side -> expert side (the dispatch a2av followed by
 * the regroup); direction 1 moves expert side -> pack side (the inverse
 * regroup followed by the return a2av).
 */
int ref_moe_dispatch_grouped(int W, int E, size_t R, const int64_t *counts,
                             const void *const *in, const int64_t *in_rows,
                             void *const *out, const int64_t *out_cap,
                             int64_t *expert_offsets, int direction) {
    if (W < 1 || W > REF_MAX_W || E < 1 || E % W != 0 || R == 0 || !counts || !in || !in_rows ||
        !out || !out_cap || !expert_offsets || (direction != 0 && direction != 1))
        return REF_EARG;
    const int P = E / W;
    for (int64_t i = 0; i < (int64_t)W * E; i++)
        if (!split_is_valid(counts[i])) return REF_BAD_SPLIT;
    /* the expert side: offsets of each owned expert at its owner */
    for (int d = 0; d < W; d++) {
        int64_t run = 0;
        for (int j = 0; j < P; j++) {
            expert_offsets[d * (P + 1) + j] = run;
            for (int s = 0; s < W; s++) run += counts[s * E + d * P + j];
        }
        expert_offsets[d * (P + 1) + P] = run;
    }
    int st = 0;
    for (int r = 0; r < W; r++) {
        int64_t pack_total = 0;
        for (int e = 0; e < E; e++) pack_total += counts[r * E + e];
        const int64_t exp_total = expert_offsets[r * (P + 1) + P];
        const int64_t sent = direction == 0 ? pack_total : exp_total;
        const int64_t received = direction == 0 ? exp_total : pack_total;
        if (sent > in_rows[r]) st |= REF_SEND_OVERRUN;
        if (received > out_cap[r]) st |= REF_RECV_OVERFLOW;
        if ((sent > 0 && !in[r]) || (received > 0 && !out[r])) return REF_EARG;
    }
    if (st) return st;
    for (int s = 0; s < W; s++) {
        int64_t pack_pos = 0;
        for (int e = 0; e < E; e++) {
            const int d = e / P, j = e % P;
            const int64_t n = counts[s * E + e];
            int64_t exp_pos = expert_offsets[d * (P + 1) + j];
            for (int s2 = 0; s2 < s; s2++) exp_pos += counts[s2 * E + e];
            if (n > 0) {
                if (direction == 0)
                    memcpy((unsigned char *)out[d] + (size_t)exp_pos * R,
                           (const unsigned char *)in[s] + (size_t)pack_pos * R, (size_t)n * R);
                else
                    memcpy((unsigned char *)out[s] + (size_t)pack_pos * R,
                           (const unsigned char *)in[d] + (size_t)exp_pos * R, (size_t)n * R);
            }
            pack_pos += n;
        }
    }
    return 0;
}

/*
 * The gate-weighted combine read straight from the expert side: the grouped
 * return (ref_moe_dispatch_grouped, direction 1) followed by ref_moe_combine,
 * written as one step. Slot q = t*k + j of source s names its expert
 * ids[s][q] and its pack-order row perm[s][q]; that row lies in expert e's
 * pack block [Y_s(e), Y_s(e) + counts[s][e]) and sits on the expert side of
 * owner e / P at expert_start(s, e) + (perm[s][q] - Y_s(e)).
 */
int ref_moe_combine_grouped(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                            const int32_t *const *ids, const int64_t *const *perm,
                            const uint16_t *const *expert_side, const int64_t *exp_rows,
                            const float *const *w, uint16_t *const *out) {
    if (W < 1 || W > REF_MAX_W || T < 0 || k < 1 || E < 1 || E % W != 0 || H < 1 || !counts ||
        !ids || !perm || !expert_side || !exp_rows || !w || !out)
        return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int P = E / W;
    const int64_t Q = T * k;
    for (int64_t i = 0; i < (int64_t)W * E; i++)
        if (!split_is_valid(counts[i])) return REF_BAD_SPLIT;
    /* Y[s][e]: pack position of expert e at source s; X[s][e]: its start on the expert side */
    int64_t *Y = malloc(sizeof(int64_t) * (size_t)W * E);
    int64_t *X = malloc(sizeof(int64_t) * (size_t)W * E);
    if (!Y || !X) { free(Y); free(X); return REF_EARG; }
    int st = 0;
    for (int d = 0; d < W; d++) {
        int64_t run = 0;
        for (int j = 0; j < P; j++)
            for (int s = 0; s < W; s++) {
                X[s * E + d * P + j] = run;
                run += counts[s * E + d * P + j];
            }
        if (run > exp_rows[d]) st |= REF_SEND_OVERRUN;
    }
    for (int s = 0; s < W; s++) {
        int64_t run = 0;
        for (int e = 0; e < E; e++) { Y[s * E + e] = run; run += counts[s * E + e]; }
    }
    for (int s = 0; s < W; s++)
        for (int64_t q = 0; q < Q; q++) {
            const int32_t e = ids[s][q];
            const int64_t p = perm[s][q];
            if (e < 0 || e >= E) { st |= REF_BAD_EXPERT; continue; }
            if (p < Y[s * E + e] || p >= Y[s * E + e] + counts[s * E + e]) st |= REF_BAD_PERM;
        }
    if (st) { free(Y); free(X); return st; }
    for (int s = 0; s < W; s++)
        for (int64_t t = 0; t < T; t++)
            for (int64_t h = 0; h < H; h++) {
                float acc = 0.0f;
                for (int j = 0; j < k; j++) {
                    const int64_t q = t * k + j;
                    const int e = ids[s][q];
                    const int64_t row = X[s * E + e] + (perm[s][q] - Y[s * E + e]);
                    acc = fmaf(w[s][q], bf16_to_float(expert_side[e / P][row * H + h]), acc);
                }
                out[s][t * H + h] = float_to_bf16(acc);
            }
    free(Y);
    free(X);
    return 0;
}

/*
 * The MoE pack and its dispatch in one step, for all W ranks: each routing
 * slot's token row goes straight to the receive buffer of its expert's owner
 * (e / P, P = E / W). Owner d's rows are its slots from every source, sorted
 * by the key (source, expert, slot) for layout 0, the order the pack
 * followed by the a2av leaves, or (expert, source, slot) for layout 1, the
 * order the pack followed by the grouped dispatch leaves. Written here as
 * that sort, with perm, the splits and the counts from the pack's own
 * definition.
 */
typedef struct {
    int64_t key[3];
    int src;
    int64_t tok;
} ref_slot_key;

static int cmp_slot_key(const void *a, const void *b) {
    const ref_slot_key *x = a, *y = b;
    for (int i = 0; i < 3; i++)
        if (x->key[i] != y->key[i]) return x->key[i] < y->key[i] ? -1 : 1;
    return 0;
}

int ref_moe_pack_dispatch(int W, int64_t T, int k, int E, size_t R,
                          const void *const *tokens, const int32_t *const *ids,
                          void *const *recv, const int64_t *recv_cap, int64_t *const *perm,
                          int64_t *S, int64_t *expert_counts, int64_t *block_offsets,
                          int layout) {
    if (W < 1 || W > REF_MAX_W || T < 0 || k < 1 || E < 1 || E % W != 0 || R == 0 || !tokens ||
        !ids || !recv || !recv_cap || !perm || !S || !expert_counts || !block_offsets ||
        (layout != 0 && layout != 1))
        return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int P = E / W;
    const int64_t Q = T * k;
    for (int s = 0; s < W; s++) {
        if (Q > 0 && (!tokens[s] || !ids[s] || !perm[s])) return REF_EARG;
        for (int64_t q = 0; q < Q; q++)
            if (ids[s][q] < 0 || ids[s][q] >= E) return REF_BAD_EXPERT;
    }
    /* the pack of every source: counts, perm, splits */
    int64_t *next = malloc(sizeof(int64_t) * (size_t)E);
    if (!next) return REF_EARG;
    for (int s = 0; s < W; s++) {
        int64_t *cnt = expert_counts + (size_t)s * E;
        for (int e = 0; e < E; e++) cnt[e] = 0;
        for (int64_t q = 0; q < Q; q++) cnt[ids[s][q]] += 1;
        int64_t run = 0;
        for (int e = 0; e < E; e++) { next[e] = run; run += cnt[e]; }
        for (int64_t q = 0; q < Q; q++) perm[s][q] = next[ids[s][q]]++;
        for (int d = 0; d < W; d++) {
            S[s * W + d] = 0;
            for (int j = 0; j < P; j++) S[s * W + d] += cnt[d * P + j];
        }
    }
    free(next);
    /* block starts at each receiver: sources (layout 0) or owned experts (layout 1) */
    int st = 0;
    const int G = layout == 0 ? W : P;
    for (int d = 0; d < W; d++) {
        int64_t run = 0;
        for (int g = 0; g < G; g++) {
            block_offsets[d * (G + 1) + g] = run;
            if (layout == 0) run += S[g * W + d];
            else for (int s = 0; s < W; s++) run += expert_counts[(size_t)s * E + d * P + g];
        }
        block_offsets[d * (G + 1) + G] = run;
        if (run > recv_cap[d]) st |= REF_RECV_OVERFLOW;
        if (run > 0 && !recv[d]) return REF_EARG;
    }
    if (st) return st;
    ref_slot_key *keys = malloc(sizeof(ref_slot_key) * (size_t)(W * Q > 0 ? W * Q : 1));
    if (!keys) return REF_EARG;
    for (int d = 0; d < W; d++) {
        int64_t n = 0;
        for (int s = 0; s < W; s++)
            for (int64_t q = 0; q < Q; q++) {
                const int64_t e = ids[s][q];
                if (e / P != d) continue;
                ref_slot_key *x = &keys[n++];
                x->key[0] = layout == 0 ? s : e;
                x->key[1] = layout == 0 ? e : s;
                x->key[2] = q;
                x->src = s;
                x->tok = q / k;
            }
        qsort(keys, (size_t)n, sizeof(ref_slot_key), cmp_slot_key);
        for (int64_t i = 0; i < n; i++)
            memcpy((unsigned char *)recv[d] + (size_t)i * R,
                   (const unsigned char *)tokens[keys[i].src] + (size_t)keys[i].tok * R, R);
    }
    free(keys);
    return 0;
}

/*
 * The inverse of ref_moe_pack_dispatch: every slot's row read back from its
 * owner's receive buffer (the return a2av followed by the un-pack, or the
 * grouped return followed by the un-pack, as one step). Slot q of source s
 * names expert e = ids[s][q] and pack row perm[s][q], which must lie in
 * expert e's pack block [Y_s(e), Y_s(e) + counts[s][e]); the row sits at
 * owner e / P at the start of the (s, e) block in the layout's order plus
 * perm[s][q] - Y_s(e).
 */
int ref_moe_unpack_return(int W, int64_t T, int k, int E, size_t R, const int64_t *counts,
                          const int32_t *const *ids, const int64_t *const *perm,
                          const void *const *recv, const int64_t *recv_rows, void *const *out,
                          int layout) {
    if (W < 1 || W > REF_MAX_W || T < 0 || k < 1 || E < 1 || E % W != 0 || R == 0 || !counts ||
        !ids || !perm || !recv || !recv_rows || !out || (layout != 0 && layout != 1))
        return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int P = E / W;
    const int64_t Q = T * k;
    for (int64_t i = 0; i < (int64_t)W * E; i++)
        if (!split_is_valid(counts[i])) return REF_BAD_SPLIT;
    /* Y[s][e]: pack position of expert e at source s; Z[s][e]: start of the (s, e) block at its owner */
    int64_t *Y = malloc(sizeof(int64_t) * (size_t)W * E);
    int64_t *Z = malloc(sizeof(int64_t) * (size_t)W * E);
    if (!Y || !Z) { free(Y); free(Z); return REF_EARG; }
    int st = 0;
    for (int s = 0; s < W; s++) {
        int64_t run = 0;
        for (int e = 0; e < E; e++) { Y[s * E + e] = run; run += counts[s * E + e]; }
    }
    for (int d = 0; d < W; d++) {
        int64_t run = 0;
        if (layout == 0) {
            for (int s = 0; s < W; s++)
                for (int j = 0; j < P; j++) { Z[s * E + d * P + j] = run; run += counts[s * E + d * P + j]; }
        } else {
            for (int j = 0; j < P; j++)
                for (int s = 0; s < W; s++) { Z[s * E + d * P + j] = run; run += counts[s * E + d * P + j]; }
        }
        if (run > recv_rows[d]) st |= REF_SEND_OVERRUN;
    }
    for (int s = 0; s < W; s++) {
        if (Q > 0 && (!ids[s] || !perm[s] || !out[s])) { free(Y); free(Z); return REF_EARG; }
        for (int64_t q = 0; q < Q; q++) {
            const int32_t e = ids[s][q];
            const int64_t p = perm[s][q];
            if (e < 0 || e >= E) { st |= REF_BAD_EXPERT; continue; }
            if (p < Y[s * E + e] || p >= Y[s * E + e] + counts[s * E + e]) st |= REF_BAD_PERM;
        }
    }
    if (st) { free(Y); free(Z); return st; }
    for (int s = 0; s < W; s++)
        for (int64_t q = 0; q < Q; q++) {
            const int e = ids[s][q];
            const int64_t row = Z[s * E + e] + (perm[s][q] - Y[s * E + e]);
            memcpy((unsigned char *)out[s] + (size_t)q * R,
                   (const unsigned char *)recv[e / P] + (size_t)row * R, R);
        }
    free(Y);
    free(Z);
    return 0;
}

/*
 * The gate-weighted combine read at the owners: ref_moe_unpack_return (the
 * return trip in one step, either layout) followed by ref_moe_combine over
 * the rows it brings home, slot q = t*k + j of token t being row q there.
 * Written as that composition; its status is the inverse's, and nothing is
 * written when it fails.
 */
int ref_moe_combine_return(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                           const int32_t *const *ids, const int64_t *const *perm,
                           const uint16_t *const *recv, const int64_t *recv_rows,
                           const float *const *w, uint16_t *const *out, int layout) {
    if (W < 1 || W > REF_MAX_W || T < 0 || k < 1 || H < 1 || !w || !out) return REF_EARG;
    if (T > INT64_MAX / k) return REF_EARG;
    const int64_t Q = T * k;
    void **home = calloc((size_t)W, sizeof(void *));
    int64_t *ident = malloc(sizeof(int64_t) * (size_t)(Q > 0 ? Q : 1));
    if (!home || !ident) { free(home); free(ident); return REF_EARG; }
    int st = 0;
    for (int s = 0; s < W && !st; s++) {
        home[s] = malloc((size_t)(Q > 0 ? Q : 1) * (size_t)H * 2);
        if (!home[s]) st = REF_EARG;
    }
    if (!st)
        st = ref_moe_unpack_return(W, T, k, E, (size_t)H * 2, counts, ids, perm,
                                   (const void *const *)recv, recv_rows, home, layout);
    for (int64_t q = 0; q < Q; q++) ident[q] = q;
    for (int s = 0; s < W && !st; s++)
        st = ref_moe_combine(T, k, H, (const uint16_t *)home[s], ident, w[s], out[s]);
    for (int s = 0; s < W; s++) free(home[s]);
    free(home);
    free(ident);
    return st;
}
