/*
 * a2av_ref.h — CPU oracle for the device-split all-to-all-v and the MoE
 * pack/unpack around it.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no source, header, table or helper with
 * the HIP library.
 *
 * Every function is plain, single-threaded C over host pointers. Status bits
 * have the same meaning as the device status bits of the HIP library, but the
 * values are defined here again, on purpose, so the two sides share nothing.
 *
 * Source of the operation: the page "[a2av] Improve tuning for 4 GPUs"
 * (pytorch/pytorch pull 154580), section "Problem", names the op
 * nvshmem_all_to_all_vdev and times it; it does not spell out what it
 * computes. The plain reading used here is MPI all-to-all-v with the counts
 * held on the device: rank s sends S[s][d] rows to rank d, the receive counts
 * are the transpose, send and receive displacements are exclusive scans of
 * the counts, and each destination receives its chunks in source-rank order.
 */
#ifndef A2AV_REF_H
#define A2AV_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Returned status bits (OR-ed together); 0 = success. */
#define REF_BAD_SPLIT     1  /* a split is negative or above REF_MAX_SPLIT      */
#define REF_SEND_OVERRUN  2  /* a rank sends more rows than its input holds     */
#define REF_RECV_OVERFLOW 4  /* a rank receives more rows than its output holds */
#define REF_BAD_EXPERT    8  /* an expert id is outside [0, E)                  */
#define REF_BAD_OFFSETS  16  /* given offsets are not the scans of the splits   */
#define REF_BAD_PERM     32  /* a permutation entry is outside its range        */

/* Host argument error (nothing computed, nothing written). */
#define REF_EARG (-1)

#define REF_MAX_SPLIT ((int64_t)1 << 40)
#define REF_MAX_W 64

/* O[d][s] = S[s][d] for a W x W row-major matrix (row s = rank s's splits). */
int ref_exchange_splits(int W, const int64_t *S, int64_t *O);

/* send_off[s][0..W] = exclusive scan of row s of S, with the total at index W;
 * recv_off[d][0..W] = exclusive scan of row d of O, with the total at index W.
 * Both outputs are W x (W+1) row-major. */
int ref_offsets(int W, const int64_t *S, const int64_t *O,
                int64_t *send_off, int64_t *recv_off);

/* Payload step: for every destination d and source s (ascending), copy
 * S[s][d] rows of R bytes from in[s] at row send_off[s][d] to out[d] at row
 * recv_off[d][s]. Checks every condition first; writes nothing on failure. */
int ref_copy(int W, size_t R,
             const void *const *in, const int64_t *in_rows,
             void *const *out, const int64_t *out_cap_rows,
             const int64_t *S, const int64_t *send_off, const int64_t *recv_off);

/* The whole definition from S alone: exchange, offsets, payload. O,
 * send_off and recv_off are written when the splits are valid; the payload
 * only when every check passes. */
int ref_a2av(int W, size_t R,
             const void *const *in, const int64_t *in_rows,
             void *const *out, const int64_t *out_cap_rows,
             const int64_t *S, int64_t *O, int64_t *send_off, int64_t *recv_off);

/* Inverse map for one output row: output row j of rank d came from input row
 * *src_row of rank *src_rank. Returns 0, or 1 when j is past rank d's total,
 * or REF_EARG. Lets a test check sampled rows of a workload too large to run
 * whole. */
int ref_source_of(int W, const int64_t *S, int d, int64_t j,
                  int *src_rank, int64_t *src_row);

/* MoE dispatch pack for ONE rank. T tokens of R bytes, k expert ids each
 * (ids is T x k, slot q = t*k + j), E experts spread over W ranks in
 * contiguous blocks of E/W. Outputs: perm[q] = row of slot q in send (a
 * stable counting sort by expert id), send[perm[q]] = token q/k,
 * splits[d] = slots bound for rank d, expert_counts[e] = slots for expert e. */
int ref_moe_pack(int64_t T, int k, int E, int W, size_t R,
                 const void *tokens, const int32_t *ids,
                 void *send, int64_t *perm, int64_t *splits,
                 int64_t *expert_counts);

/* Inverse of the pack after the return trip, for ONE rank:
 * out[q] = back[perm[q]] for q < T*k (rows of R bytes). */
int ref_moe_unpack(int64_t T, int k, size_t R,
                   const void *back, const int64_t *perm, void *out);

/* Receive-side expert regroup for ONE rank d. counts is the W x E matrix of
 * rows each source s routed to each expert e (row s = source s). The rank
 * owns experts d*P .. d*P+P-1 (P = E/W). Source-major order: for each source
 * s, for each owned expert j, counts[s][d*P+j] rows. Expert-major order: for
 * each owned expert j, for each source s, the same blocks. direction 0 turns
 * source-major `in` into expert-major `out`; direction 1 the reverse.
 * expert_offsets[j] = rows before owned expert j in expert-major order, with
 * the total at index P. */
int ref_moe_regroup(int W, int E, int d, size_t R, const int64_t *counts,
                    const void *in, int64_t in_rows, void *out, int64_t out_cap,
                    int64_t *expert_offsets, int direction);

/* Gate-weighted combine for ONE rank: for token t and element h,
 * acc = +0.0f; for j = 0..k-1: acc = fmaf(w[t][j], float(back[perm[t*k+j]][h]), acc);
 * out[t][h] = acc rounded to bfloat16 (round to nearest even; any NaN is written
 * as the quiet NaN 0x7FC0). back is [T*k][H] bf16, w is [T][k] fp32, out is
 * [T][H] bf16. */
int ref_moe_combine(int64_t T, int k, int64_t H, const uint16_t *back,
                    const int64_t *perm, const float *w, uint16_t *out);

/* Bucketing of ONE rank's jagged embedding keys by owning rank (table t is
 * owned by rank t mod W). lengths is [n_tables][batch] int32 in table order,
 * keys are the keys of table 0, then table 1, ... (n_keys of them). Outputs
 * lengths_out / keys_out hold the tables in (owner, t) order;
 * split_keys[d] / split_lengths[d] = keys / lengths rows bound for rank d. */
int ref_keys_bucketize(int W, int n_tables, int64_t batch, const int32_t *lengths,
                       const int64_t *keys, int64_t n_keys, int32_t *lengths_out,
                       int64_t *keys_out, int64_t *split_keys, int64_t *split_lengths);

/* MoE dispatch plus receive-side regroup in one step, for all W ranks.
 * counts is the W x E matrix of moe_pack's expert counts (row s = source s).
 * Pack side of rank s: its rows in pack order (expert ascending). Expert side
 * of rank d: for each owned expert j (e = d*P + j, P = E/W), for each source
 * s, counts[s][e] rows. direction 0: in = pack side (indexed by source),
 * out = expert side (indexed by owner); direction 1: the reverse.
 * expert_offsets [W][P+1] = rows before owned expert j on the expert side
 * (total at P), written whenever the counts are valid. REF_BAD_SPLIT for a
 * count outside [0, 2^40] (nothing written); else REF_SEND_OVERRUN /
 * REF_RECV_OVERFLOW when a rank's sent / received total exceeds in_rows /
 * out_cap (no payload). */
int ref_moe_dispatch_grouped(int W, int E, size_t R, const int64_t *counts,
                             const void *const *in, const int64_t *in_rows,
                             void *const *out, const int64_t *out_cap,
                             int64_t *expert_offsets, int direction);

/* The gate-weighted combine read straight from the expert side, for all W
 * ranks: what ref_moe_dispatch_grouped (direction 1) followed by
 * ref_moe_combine gives, as one step. ids[s] and perm[s] are moe_pack's
 * inputs and output for source s (T*k slots); expert_side[d] holds
 * exp_rows[d] rows of H bf16 in owner d's expert-major order; w[s] is
 * [T][k] fp32; out[s] is [T][H] bf16. REF_BAD_SPLIT for a count outside
 * [0, 2^40] (first); else the OR of REF_SEND_OVERRUN (an owner's rows exceed
 * exp_rows), REF_BAD_EXPERT (an id outside [0, E)) and REF_BAD_PERM (a perm
 * entry outside its expert's pack block). Nothing is written on failure. */
int ref_moe_combine_grouped(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                            const int32_t *const *ids, const int64_t *const *perm,
                            const uint16_t *const *expert_side, const int64_t *exp_rows,
                            const float *const *w, uint16_t *const *out);

/* The MoE pack and its dispatch in one step, for all W ranks: slot q of
 * source s (expert e = ids[s][q]) sends token row q / k of tokens[s]
 * straight to owner e / P (P = E / W). Owner d's receive rows are its slots
 * from all sources sorted by (source, expert, slot) for layout 0 (what
 * ref_moe_pack followed by ref_a2av leaves) or (expert, source, slot) for
 * layout 1 (what ref_moe_pack followed by ref_moe_dispatch_grouped leaves).
 * perm[s] ([T*k]), S (W x W, row s = source s) and expert_counts (W x E) are
 * ref_moe_pack's outputs; block_offsets[d] ([G+1], G = W for layout 0, E/W
 * for layout 1) = rows before block g (source g, or owned expert g) at
 * receiver d, total at G. REF_BAD_EXPERT for an id outside [0, E) (nothing
 * written); else REF_RECV_OVERFLOW when a receiver's total exceeds recv_cap
 * (perm, S, counts and offsets written; no payload). */
int ref_moe_pack_dispatch(int W, int64_t T, int k, int E, size_t R,
                          const void *const *tokens, const int32_t *const *ids,
                          void *const *recv, const int64_t *recv_cap, int64_t *const *perm,
                          int64_t *S, int64_t *expert_counts, int64_t *block_offsets,
                          int layout);

/* The inverse: out[s][q] = the row of slot q of source s, read from its
 * owner's receive buffer recv[d] (recv_rows[d] rows in the layout's order).
 * counts is the W x E expert-count matrix; ids and perm are the pack's input
 * and output per source. REF_BAD_SPLIT for a count outside [0, 2^40]
 * (first); else the OR of REF_SEND_OVERRUN (an owner's rows exceed
 * recv_rows), REF_BAD_EXPERT and REF_BAD_PERM (a perm entry outside its
 * expert's pack block). Nothing is written on failure. */
int ref_moe_unpack_return(int W, int64_t T, int k, int E, size_t R, const int64_t *counts,
                          const int32_t *const *ids, const int64_t *const *perm,
                          const void *const *recv, const int64_t *recv_rows, void *const *out,
                          int layout);

/* The gate-weighted combine read at the owners, for all W ranks:
 * ref_moe_unpack_return (layout 0 or 1) followed by ref_moe_combine over the
 * rows it brings home (slot t*k + j of token t). recv[d] holds recv_rows[d]
 * bf16 rows of H; w[s] is [T][k] fp32; out[s] is [T][H] bf16. Status and
 * what is written on failure: those of ref_moe_unpack_return. */
int ref_moe_combine_return(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                           const int32_t *const *ids, const int64_t *const *perm,
                           const uint16_t *const *recv, const int64_t *recv_rows,
                           const float *const *w, uint16_t *const *out, int layout);

/* The whole key exchange of one batch for all W ranks: ref_keys_bucketize on
 * every source, then keys (8-byte rows) and lengths (4-byte rows) as two
 * ref_a2av calls with the bucketing's split rows. lengths_cap / keys_cap are
 * the receivers' capacities (entries). Result: the OR of the sources'
 * bucketing bits if any fails (nothing written); else REF_RECV_OVERFLOW if a
 * receiver's totals exceed its capacities (split columns and receive offsets
 * written for the receivers that fit; no payload); else 0 with everything
 * written. split_keys / split_lengths are W x W (row s = source s);
 * recv_off_keys[d][s] = keys before source s's chunk at receiver d, total at
 * index W. */
int ref_keys_exchange(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                      const int64_t *const *keys, const int64_t *n_keys,
                      int32_t *const *lengths_out, const int64_t *lengths_cap,
                      int64_t *const *keys_out, const int64_t *keys_cap, int64_t *split_keys,
                      int64_t *split_lengths, int64_t *recv_off_keys);

#ifdef __cplusplus
}
#endif

#endif /* A2AV_REF_H */
