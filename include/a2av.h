/*
 * a2av.h — C ABI of liba2av.so: device-split all-to-all-v (a2av) and the MoE
 * dispatch pack/unpack around it, for AMD Instinct MI355X (gfx950).
 *
 * What is computed. The page "[a2av] Improve tuning for 4 GPUs" (pytorch
 * pull 154580), section "Problem", times nvshmem_all_to_all_vdev on 4 GPUs
 * with per-rank messages of 0.5..4096 MiB; its section "Change" re-balances
 * the thread blocks of that exchange between the peer dimension and the
 * data-parallel dimension. The page does not spell out the operation; it is
 * read here as MPI all-to-all-v with device-resident counts:
 *   - rank s holds an input buffer and an int64 split vector S[s][0..W-1]
 *     (rows it sends to each rank d);
 *   - the output splits are the transpose O[d][s] = S[s][d];
 *   - send and receive offsets are exclusive scans of S and O rows;
 *   - rank d's output is the concatenation of the chunks sent to it, in
 *     source-rank order.
 * The W ranks are W partitions of one GPU's HBM: rank r is the pair of device
 * buffers (in[r], out[r]) and row r of the split matrices.
 *
 * Conventions for every call:
 *   - Matrices are row-major int64 in device memory: S and O are W x W, offsets
 *     are W x (W+1) with the row total at index W.
 *   - Pointer arrays (in, out, tokens, ...) and row-count arrays (in_rows,
 *     out_cap_rows) are HOST arrays of length W holding device pointers / host
 *     integers; they are read during the call and not kept.
 *   - The caller owns every buffer. Nothing is allocated by the library
 *     except as stated; scratch comes from a caller-provided workspace.
 *   - Every call enqueues its kernels on `stream` and returns without
 *     synchronising. Stream order carries the dependencies between calls.
 *   - Return value (host side): 0 = enqueued; A2AV_EARG = a bad argument
 *     (nothing enqueued); A2AV_EHIP = the HIP runtime refused a launch.
 *   - Device-side failures are reported through `status`, a caller-zeroed
 *     device int32. Kernels OR status bits into it. An op that finds the word
 *     nonzero on entry writes nothing, and an op that detects a failure writes
 *     no payload byte (all-or-nothing); on a capacity failure some ops still
 *     write their splits, counts or offsets, as each call below states. A
 *     failed op poisons the rest of a sequence that shares the word. Read it
 *     after synchronising the stream.
 *   - Calls that overlap in time on buffers they share race; calls on
 *     disjoint buffers may run concurrently on different streams.
 *   - The copy, scatter, gather and combine kernels launch one wave per
 *     piece, row or slot, up to A2AV_MAX_GRID workgroups (environment,
 *     read on every call; default and maximum 2^22); their waves loop over
 *     what a smaller grid leaves. The setting changes only the schedule.
 */
#ifndef A2AV_H
#define A2AV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define A2AV_ABI_VERSION 1
#define A2AV_MAX_W 64                        /* virtual ranks per call        */
#define A2AV_MAX_SPLIT ((int64_t)1 << 40)    /* largest valid split (rows)    */
#define A2AV_MAX_EXPERTS 4096                /* experts per moe_pack call     */
#define A2AV_MAX_TABLES 4096                 /* tables per keys_bucketize call */

/* host return codes */
#define A2AV_OK 0
#define A2AV_EARG (-1)
#define A2AV_EHIP (-2)

/* device status bits */
#define A2AV_ST_BAD_SPLIT 1      /* a split is negative or above A2AV_MAX_SPLIT */
#define A2AV_ST_SEND_OVERRUN 2   /* a rank sends more rows than in_rows        */
#define A2AV_ST_RECV_OVERFLOW 4  /* a rank receives more rows than out_cap_rows */
#define A2AV_ST_BAD_EXPERT 8     /* an expert id is outside [0, E)              */
#define A2AV_ST_BAD_OFFSETS 16   /* offsets are not the exclusive scans of S    */
#define A2AV_ST_BAD_PERM 32      /* a permutation entry is outside [0, T*k)     */

/* ABI version of the loaded library (A2AV_ABI_VERSION it was built with). */
int a2av_abi_version(void);

/* Static text for a host return code or a status bit; never NULL. */
const char *a2av_strerror(int code);

/*
 * Splits exchange, the first step of the exchange timed on the page "[a2av]
 * Improve tuning for 4 GPUs" (section "Problem"), as read above:
 * O[d][s] = S[s][d] (the output split matrix is the transpose of the input
 * splits; row d of O is what rank d receives from each source).
 *   W      1..A2AV_MAX_W
 *   S      device int64 [W][W], row s = rank s's split vector (rows per peer)
 *   O      device int64 [W][W], written
 *   status device int32; sets A2AV_ST_BAD_SPLIT (and writes nothing) if any
 *          split is negative or above A2AV_MAX_SPLIT.
 * One single-workgroup kernel.
 */
int a2av_exchange_splits(int W, const int64_t *S, int64_t *O, int32_t *status,
                         hipStream_t stream);

/*
 * Offsets, the second step of that exchange (same page and section, as read
 * above): send_off[s][d] = sum_{d'<d} S[s][d'] and recv_off[d][s] =
 * sum_{s'<s} O[d][s'] (exclusive scans), with the row totals at index W.
 *   S, O      device int64 [W][W]
 *   send_off  device int64 [W][W+1], written
 *   recv_off  device int64 [W][W+1], written
 *   status    sets A2AV_ST_BAD_SPLIT (writes nothing) for an invalid entry.
 * One single-workgroup kernel; one wave64 prefix scan per row.
 */
int a2av_offsets(int W, const int64_t *S, const int64_t *O, int64_t *send_off,
                 int64_t *recv_off, int32_t *status, hipStream_t stream);

/*
 * Payload, the third step of that exchange (same page, sections "Problem" and
 * "Change", as read above): for every (s, d), rows [send_off[s][d],
 * +S[s][d]) of in[s] are copied to out[d] at row recv_off[d][s]; rows are row_bytes wide and copied
 * bit-for-bit. Output bytes past recv_off[d][W] rows are not touched; input
 * rows past send_off[s][W] are not sent.
 *   row_bytes     >= 1, same for every rank; any alignment is accepted, the
 *                 fast path wants source and destination congruent mod 16
 *   in[W]         host array of device pointers, in[s] holds in_rows[s] rows
 *                 (may be NULL when in_rows[s] == 0)
 *   out[W]        host array of device pointers, out[d] holds out_cap_rows[d]
 *   S, send_off, recv_off  device matrices as produced by
 *                 a2av_exchange_splits + a2av_offsets
 *   status        checked before any byte moves, in every workgroup:
 *                 A2AV_ST_BAD_SPLIT, A2AV_ST_BAD_OFFSETS (offsets are not the
 *                 scans of S and S^T), A2AV_ST_SEND_OVERRUN
 *                 (send_off[s][W] > in_rows[s]), A2AV_ST_RECV_OVERFLOW
 *                 (recv_off[d][W] > out_cap_rows[d]); any of them => no byte
 *                 of any out[d] is written.
 * The destination byte space of all ranks (out[0]'s rows, then out[1]'s, ...)
 * is cut into equal pieces, one per wave, so skewed or zero splits leave no
 * compute unit idle; pieces are copied with 16-byte coalesced non-temporal
 * accesses (realigned in registers when source and destination differ mod
 * 16), and the grid is sized to min(sum in_rows, sum out_cap_rows) *
 * row_bytes. For W <= 8 this is one kernel: every wave reads S and the
 * per-rank arrays through the scalar cache, scans S itself, and checks the
 * given offsets against its scans before its first store. For larger W a
 * single workgroup checks everything first and the copy kernel follows (two
 * launches); its workgroups take the destination totals and one row of
 * recv_off from two scalar bursts shared through LDS, and a wave in another
 * destination loads that destination's row of recv_off.
 * The wave kernels of a2av_copy and a2av_all_to_all_vdev (from 64 MiB per
 * side; above 8 ranks only with 16-byte rows), the plain copy, the block copies
 * (from 64 MiB per side, with 16-byte rows) and the weighted combine (always)
 * reserve LDS they do not use, to run fewer workgroups per CU; a kernel on
 * another stream then finds less LDS free on the CUs they occupy.
 * Tuning (read on every call; defaults are compiled in): A2AV_WAVE_PIECE,
 * A2AV_WAVE_UNROLL (4, 8 or 16), A2AV_WAVE_LDS (bytes of LDS per workgroup
 * the kernel does not use, which limits workgroups per CU) for the wave
 * kernels; A2AV_BLOCK_KERNEL=1 forces the older
 * workgroup kernel (one workgroup per piece, matrices staged in LDS for
 * W <= 16); A2AV_BLOCKS_PER_CU, A2AV_UNROLL, A2AV_NT, A2AV_PIECE,
 * A2AV_MIN_PIECE (workgroup kernel). Every setting gives identical bytes.
 */
int a2av_copy(int W, size_t row_bytes, const void *const *in,
              const int64_t *in_rows, void *const *out,
              const int64_t *out_cap_rows, const int64_t *S,
              const int64_t *send_off, const int64_t *recv_off,
              int32_t *status, hipStream_t stream);

/*
 * The whole a2av in one call, nvshmem_all_to_all_vdev of the page "[a2av]
 * Improve tuning for 4 GPUs" (section "Problem") as read above:
 * a2av_exchange_splits, a2av_offsets and a2av_copy with the same arguments, same outputs and same status bits
 * (BAD_SPLIT alone stops it before O and the offsets are written; SEND_OVERRUN
 * / RECV_OVERFLOW leave O and the offsets written and no payload byte).
 *   S                      device int64 [W][W] (input splits)
 *   O, send_off, recv_off  device outputs as in the separate calls
 * For W <= 8 this is ONE kernel launch: every wave reads S, computes O and
 * both offset matrices in registers (the first one also writes them out),
 * checks them, and copies its piece of the destination space. For larger W,
 * two launches: one workgroup computes, writes and checks O and the offsets,
 * then the wave copy of a2av_copy runs on them. (With A2AV_BLOCK_KERNEL=1:
 * one workgroup-kernel launch for W <= 16, the three calls above that.)
 */
int a2av_all_to_all_vdev(int W, size_t row_bytes, const void *const *in,
                         const int64_t *in_rows, void *const *out,
                         const int64_t *out_cap_rows, const int64_t *S, int64_t *O,
                         int64_t *send_off, int64_t *recv_off, int32_t *status,
                         hipStream_t stream);

/*
 * Workspace bytes moe_pack needs for these sizes (0 for invalid sizes): the
 * scratch of the pack below, the step before the dispatch exchange of the MoE
 * region on the page "[a2av] Improve tuning for 4 GPUs" (section "Change",
 * the sentence under its timing table).
 */
size_t moe_pack_workspace_bytes(int W, int64_t T, int k, int E);

/*
 * MoE dispatch pack: the page "[a2av] Improve tuning for 4 GPUs" (section
 * "Change", the sentence under its timing table) singles out the MoE region
 * of message sizes, where each rank's message is its tokens grouped by
 * destination rank; the pack builds that message. Read here as: for every
 * rank r at once, the T*k routing slots
 * (slot q = t*k + j routes token t to expert ids[r][q]) are ordered by a
 * stable counting sort on the expert id. Experts are owned in contiguous
 * blocks of E/W per rank, so the order is (destination rank, expert, token,
 * slot), the layout a following a2av sends.
 *   T, k, E       tokens per rank, experts per token, experts in total;
 *                 E % W == 0, 1 <= E <= A2AV_MAX_EXPERTS, T*k < 2^31
 *   row_bytes     token row width in bytes (>= 1)
 *   tokens[W]     device [T][row_bytes] per rank
 *   ids[W]        device int32 [T][k] per rank
 *   send[W]       device [T*k][row_bytes] per rank, written: send[perm[q]] =
 *                 tokens[q / k]
 *   perm[W]       device int64 [T*k] per rank, written: row of slot q in send
 *   S             device int64 [W][W], written: S[r][d] = slots of rank r bound
 *                 for rank d (the split matrix of the dispatch a2av)
 *   expert_counts device int64 [W][E], written: slots per (rank, expert)
 *   workspace     device scratch of >= moe_pack_workspace_bytes() bytes
 *   status        A2AV_ST_BAD_EXPERT for an id outside [0, E): nothing but
 *                 the workspace is written.
 * Four kernels: an LDS histogram per slot segment, an expert-major scan of the
 * histograms, a stable in-segment rank (wave ballots), and a token-major row
 * scatter that reads each token once and writes it k times (one wave per
 * token and chunk of at most 8 KiB; the chunks tile the row).
 */
int moe_pack(int W, int64_t T, int k, int E, size_t row_bytes,
             const void *const *tokens, const int32_t *const *ids,
             void *const *send, int64_t *const *perm, int64_t *S,
             int64_t *expert_counts, void *workspace, size_t workspace_bytes,
             int32_t *status, hipStream_t stream);

/*
 * Workspace bytes moe_pack_dispatch needs (0 for invalid sizes).
 */
size_t moe_pack_dispatch_workspace_bytes(int W, int64_t T, int k, int E);

/*
 * moe_pack and the dispatch a2av of its rows as one step, for all W ranks:
 * the MoE region on the page "[a2av] Improve tuning for 4 GPUs" (section
 * "Change") packs tokens by destination rank and expert and then exchanges
 * them; here every slot's token row is written once, straight into the
 * receive buffer of its expert's owner (rank e / (E/W)), and no send buffer
 * exists. Owner d's rows come in one of two orders:
 *   layout 0  (source, expert, token, slot): what moe_pack followed by
 *             a2av_all_to_all_vdev with its splits delivers
 *   layout 1  (expert, source, token, slot): what moe_pack followed by
 *             moe_dispatch_grouped (direction 0) delivers
 *   tokens[W], ids[W]   as moe_pack (k <= 64)
 *   recv[W]             device [recv_cap_rows[d]][row_bytes] per owner (host
 *                       recv_cap_rows); rows past the owner's total untouched
 *   perm[W], S, expert_counts   written as moe_pack writes them (perm = each
 *                       slot's row in the pack order, which the inverse and
 *                       moe_combine_grouped read)
 *   block_offsets       device int64 [W][G+1], written: rows before block g at
 *                       owner d, total at G; blocks are sources (G = W, the
 *                       a2av's receive offsets) for layout 0 and owned experts
 *                       (G = E/W, moe_dispatch_grouped's expert_offsets) for
 *                       layout 1
 *   workspace           device scratch of >= moe_pack_dispatch_workspace_bytes()
 *   status              A2AV_ST_BAD_EXPERT for an id outside [0, E): nothing
 *                       but the workspace is written; A2AV_ST_RECV_OVERFLOW
 *                       when an owner's rows exceed recv_cap_rows: perm, S,
 *                       expert_counts and block_offsets are written (so the
 *                       caller can size the buffers), no payload byte.
 * Five kernels: the three of moe_pack's counting sort, a plan (one workgroup
 * per source; for every (source, expert) the shift from a slot's pack row to
 * its row at the owner) and moe_pack's token-major row scatter with those
 * destinations.
 */
int moe_pack_dispatch(int W, int64_t T, int k, int E, size_t row_bytes,
                      const void *const *tokens, const int32_t *const *ids,
                      void *const *recv, const int64_t *recv_cap_rows, int64_t *const *perm,
                      int64_t *S, int64_t *expert_counts, int64_t *block_offsets, int layout,
                      void *workspace, size_t workspace_bytes, int32_t *status,
                      hipStream_t stream);

/*
 * Workspace bytes moe_unpack_return needs (0 for invalid sizes).
 */
size_t moe_unpack_return_workspace_bytes(int W, int E);

/*
 * The inverse of moe_pack_dispatch: the return trip of the MoE exchange on
 * the page "[a2av] Improve tuning for 4 GPUs" (section "Change") and the
 * un-pack as one step, out[s][q] = the row of slot q of source s, read from
 * the receive buffer of its owner in the given layout. Equal to the return a2av (splits
 * O) followed by moe_unpack for layout 0, and to moe_dispatch_grouped
 * (direction 1) followed by moe_unpack for layout 1, without the returned
 * buffer.
 *   expert_counts    device int64 [W][E] (moe_pack's)
 *   ids[W], perm[W]  device int32 / int64 [T*k] per source
 *   recv[W]          device [recv_rows[d]][row_bytes] per owner (host recv_rows)
 *   out[W]           device [T*k][row_bytes] per source
 *   workspace        device scratch of >= moe_unpack_return_workspace_bytes()
 *   status           A2AV_ST_BAD_SPLIT (a count outside [0, 2^40]); else the
 *                    OR of A2AV_ST_SEND_OVERRUN (an owner's rows exceed
 *                    recv_rows), A2AV_ST_BAD_EXPERT and A2AV_ST_BAD_PERM (a
 *                    perm entry outside its expert's block of the pack order).
 *                    Nothing is written on failure.
 * Three kernels: the plan of moe_pack_dispatch, a check of every slot, and a
 * row gather (one wave per slot row, as moe_unpack).
 */
int moe_unpack_return(int W, int64_t T, int k, int E, size_t row_bytes,
                      const int64_t *expert_counts, const int32_t *const *ids,
                      const int64_t *const *perm, const void *const *recv,
                      const int64_t *recv_rows, void *const *out, int layout, void *workspace,
                      size_t workspace_bytes, int32_t *status, hipStream_t stream);

/*
 * Workspace bytes moe_combine_return needs (0 for invalid sizes).
 */
size_t moe_combine_return_workspace_bytes(int W, int64_t T, int k, int E);

/*
 * The gate-weighted combine (as moe_combine) read at the owners: the return
 * trip of the MoE exchange on the page "[a2av] Improve tuning for 4 GPUs"
 * (section "Change") and the combine in one pass, for rows left by
 * moe_pack_dispatch in either layout. Equal to moe_unpack_return followed by moe_combine over the
 * rows it brings home (slot t*k + j of token t), without writing them; for
 * layout 1 equal to moe_combine_grouped.
 *   expert_counts    device int64 [W][E] (moe_pack's)
 *   ids[W], perm[W]  device int32 / int64 [T*k] per source
 *   recv[W]          device bf16 [recv_rows[d]][H] per owner (host recv_rows)
 *   weights[W]       device fp32 [T][k];  out[W]  device bf16 [T][H]
 *   workspace        device scratch of >= moe_combine_return_workspace_bytes()
 *   status           as moe_unpack_return; nothing is written on failure.
 * Three kernels: the plan of moe_pack_dispatch, a check of every slot that
 * also records its row's address, and the combine of moe_combine reading
 * those rows in place.
 */
int moe_combine_return(int W, int64_t T, int k, int E, int64_t H, const int64_t *expert_counts,
                       const int32_t *const *ids, const int64_t *const *perm,
                       const void *const *recv, const int64_t *recv_rows,
                       const float *const *weights, void *const *out, int layout,
                       void *workspace, size_t workspace_bytes, int32_t *status,
                       hipStream_t stream);

/*
 * MoE un-pack after the return trip of the MoE exchange on the page "[a2av]
 * Improve tuning for 4 GPUs" (section "Change"), the "inverse combine"
 * without weights: out[r][q] = back[r][perm[r][q]] for q < T*k, i.e. every
 * slot gets back the row it was packed to. back is what the return a2av (splits O, the
 * transpose of the dispatch splits) delivered to rank r.
 *   back[W], out[W]  device [T*k][row_bytes] per rank
 *   perm[W]          device int64 [T*k] per rank, from moe_pack
 *   status           A2AV_ST_BAD_PERM if an entry is outside [0, T*k):
 *                    nothing is written.
 * Two kernels: a range check of perm, then a row gather (one wave per row).
 * Tuning: A2AV_MOE_GATHER_UNROLL.
 */
int moe_unpack(int W, int64_t T, int k, size_t row_bytes,
               const void *const *back, const int64_t *const *perm,
               void *const *out, int32_t *status, hipStream_t stream);

/*
 * MoE gate-weighted combine after the return trip, the weighted half of what
 * the MoE region on the page "[a2av] Improve tuning for 4 GPUs" (section
 * "Change", its 32 MB remark) sends back: for every rank r, token t < T and
 * element h < H,
 *   acc = +0.0f; for j = 0..k-1: acc = fmaf(w[r][t][j], back[r][perm[r][t*k+j]][h], acc);
 *   out[r][t][h] = acc rounded to bfloat16 (nearest even); a NaN result is
 *                  written as the quiet NaN 0x7FC0, since IEEE 754 does not
 *                  fix the sign or payload of a NaN.
 * The order of the slots and the single rounding of each fused multiply-add
 * fix every bit of the result; fp32 subnormals are kept, not flushed.
 *   back[W]     device bf16 [T*k][H] per rank (the returned rows, in the
 *               order moe_pack packed them)
 *   perm[W]     device int64 [T*k] per rank, from moe_pack
 *   weights[W]  device fp32 [T][k] per rank (gate weights)
 *   out[W]      device bf16 [T][H] per rank
 *   status      A2AV_ST_BAD_PERM if a perm entry is outside [0, T*k):
 *               nothing is written.
 * Two kernels: a range check of perm, then the sum. When H % 8 == 0 and
 * every base is 16-byte aligned, one wave per (rank, token, 512 elements)
 * loads the token's k rows 8 slots at a time (16 bytes per lane) and
 * accumulates in registers; otherwise one wave per (rank, token) goes one
 * element per lane. Tuning: A2AV_COMBINE_STORE_NT (0/1, non-temporal stores).
 */
int moe_combine(int W, int64_t T, int k, int64_t H, const void *const *back,
                const int64_t *const *perm, const float *const *weights,
                void *const *out, int32_t *status, hipStream_t stream);

/*
 * Workspace bytes moe_regroup needs (0 for invalid sizes).
 */
size_t moe_regroup_workspace_bytes(int W, int E);

/*
 * Receive-side expert regroup, the step after the dispatch a2av of the MoE
 * region on the page "[a2av] Improve tuning for 4 GPUs" (section "Change"):
 * rank d owns experts d*P .. d*P+P-1 (P = E/W) and received, from each source
 * s in turn, the rows s routed to those experts, expert by expert. With
 * counts[s][e] the rows source s routed to expert e (the expert_counts matrix
 * of moe_pack; rank d reads column block d of it, which is the exchange of
 * the counts), rank d's blocks (s, j) of counts[s][d*P+j] rows are
 *   source-major: s = 0..W-1 outer, j = 0..P-1 inner (how the a2av delivers)
 *   expert-major: j outer, s inner (each expert's rows contiguous)
 *   direction 0: in source-major -> out expert-major; 1: the reverse.
 *   counts          device int64 [W][E]
 *   in[W], out[W]   device [rows][row_bytes] per rank; not overlapping
 *   in_rows[W], out_cap_rows[W]  host: rows each buffer holds
 *   expert_offsets  device int64 [W][P+1]: rows before expert j in the
 *                   expert-major order of rank d, the total at index P;
 *                   written for every rank that passes its checks
 *   workspace       device scratch of >= moe_regroup_workspace_bytes() bytes
 *   status          A2AV_ST_BAD_SPLIT (an owned count outside [0, 2^40]),
 *                   A2AV_ST_SEND_OVERRUN (a rank's total > in_rows),
 *                   A2AV_ST_RECV_OVERFLOW (> out_cap_rows): no payload byte
 *                   of any rank is written.
 * Two kernels: a plan (one workgroup per rank: two block scans give every
 * block's source and destination start), then a copy that cuts all ranks'
 * destination bytes into equal pieces, one per wave.
 */
int moe_regroup(int W, int E, size_t row_bytes, const int64_t *counts,
                const void *const *in, const int64_t *in_rows, void *const *out,
                const int64_t *out_cap_rows, int64_t *expert_offsets, int direction,
                void *workspace, size_t workspace_bytes, int32_t *status,
                hipStream_t stream);

/*
 * Workspace bytes moe_dispatch_grouped needs (0 for invalid sizes).
 */
size_t moe_dispatch_grouped_workspace_bytes(int W, int E);

/*
 * The MoE dispatch a2av and the receive-side regroup (moe_regroup) as one
 * copy, and the inverse: the exchange of the MoE region on the page "[a2av]
 * Improve tuning for 4 GPUs" (section "Change") delivered straight into the
 * layout an expert GEMM reads. With counts[s][e] the rows source s routed to
 * expert e (moe_pack's expert_counts) and P = E/W experts per rank:
 *   pack side of rank s    its rows in expert order, as moe_pack wrote them
 *                          (expert e's counts[s][e] rows after those of the
 *                          experts before e)
 *   expert side of rank d  for each owned expert j (e = d*P + j), for each
 *                          source s, counts[s][e] rows
 *   direction 0 (dispatch): in[s] = pack side, out[d] = expert side
 *   direction 1 (return):   in[d] = expert side, out[s] = pack side
 * The result equals a2av_all_to_all_vdev with the owner-grouped splits
 * followed by moe_regroup (direction 0), or moe_regroup direction 1 followed
 * by the return a2av (direction 1), without the intermediate buffers.
 *   counts          device int64 [W][E]
 *   in[W], out[W]   device [rows][row_bytes]; in_rows[W], out_cap_rows[W] host
 *   expert_offsets  device int64 [W][P+1]: rows before owned expert j on the
 *                   expert side of rank d, total at P; written whenever the
 *                   counts are valid
 *   workspace       device scratch of >= moe_dispatch_grouped_workspace_bytes()
 *   status          A2AV_ST_BAD_SPLIT (a count outside [0, 2^40]; nothing
 *                   written), else A2AV_ST_SEND_OVERRUN / A2AV_ST_RECV_OVERFLOW
 *                   (a rank sends more than in_rows / receives more than
 *                   out_cap_rows; no payload byte written).
 * Two kernels: a plan (one workgroup per destination rank; its blocks and,
 * for each, the source rank and row) and the block copy of moe_regroup, each
 * wave reading its piece in place from the source rank's buffer.
 */
int moe_dispatch_grouped(int W, int E, size_t row_bytes, const int64_t *counts,
                         const void *const *in, const int64_t *in_rows, void *const *out,
                         const int64_t *out_cap_rows, int64_t *expert_offsets, int direction,
                         void *workspace, size_t workspace_bytes, int32_t *status,
                         hipStream_t stream);

/*
 * Workspace bytes moe_combine_grouped needs (0 for invalid sizes).
 */
size_t moe_combine_grouped_workspace_bytes(int W, int64_t T, int k, int E);

/*
 * The gate-weighted combine (as moe_combine) read straight from where
 * moe_dispatch_grouped (direction 0) left every row: the return trip and the
 * combine in one pass, for all W ranks at once. Equal to
 * moe_dispatch_grouped(direction 1) into the pack side followed by
 * moe_combine, without writing the pack side. Slot q = t*k + j of source s
 * has expert ids[s][q] and pack row perm[s][q] (moe_pack's input and output);
 * its row on the expert side of owner e / (E/W) is found from the counts.
 *   counts            device int64 [W][E] (moe_pack's expert_counts)
 *   ids[W], perm[W]   device int32 / int64 [T*k] per source
 *   expert_side[W]    device bf16 [exp_rows[d]][H] per owner d (host exp_rows)
 *   weights[W]        device fp32 [T][k];  out[W]  device bf16 [T][H]
 *   workspace         device scratch of >= moe_combine_grouped_workspace_bytes()
 *   status            A2AV_ST_BAD_SPLIT (a count outside [0, 2^40]); else the OR
 *                     of A2AV_ST_SEND_OVERRUN (an owner's rows exceed exp_rows),
 *                     A2AV_ST_BAD_EXPERT (an id outside [0, E)) and
 *                     A2AV_ST_BAD_PERM (a perm entry outside its expert's block
 *                     of the pack order). Nothing is written on failure.
 * The expert side is moe_pack_dispatch's layout 1, so this runs as
 * moe_combine_return with layout 1: a plan, a check that also records every
 * slot's row address, and the combine (one wave per (source, token, 512
 * elements), as moe_combine, 16-byte vectors when H % 8 == 0 and the bases
 * are 16-byte aligned, else one element per lane).
 */
int moe_combine_grouped(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                        const int32_t *const *ids, const int64_t *const *perm,
                        const void *const *expert_side, const int64_t *exp_rows,
                        const float *const *weights, void *const *out, void *workspace,
                        size_t workspace_bytes, int32_t *status, hipStream_t stream);

/*
 * Workspace bytes keys_bucketize needs (0 for invalid sizes).
 */
size_t keys_bucketize_workspace_bytes(int W, int n_tables);

/*
 * Owner-order bucketing of jagged embedding keys before the key exchange,
 * the exchange that the page "Different nccl stream within EmbeddingKey
 * alltoall and EmbeddingValue..." (TorchRec, description) moves to a stream
 * of its own. Table t is owned by rank t mod W. For every rank r:
 *   lengths[r]      device int32 [n_tables][batch]: keys per (table, sample)
 *   keys[r]         device int64 [n_keys[r]]: table 0's keys (sample 0, 1, ..),
 *                   then table 1's, ...
 *   lengths_out[r]  device int32 [n_tables][batch], keys_out[r] device int64
 *                   [n_keys[r]]: the same data with the tables in (owner,
 *                   table) order
 *   split_keys      device int64 [W][W]: keys rank r sends to rank d
 *   split_lengths   device int64 [W][W]: lengths entries r sends to d
 *                   (the two split matrices of the keys and lengths a2av)
 *   n_keys          host int64 [W]
 *   workspace       device scratch of >= keys_bucketize_workspace_bytes()
 *   status          A2AV_ST_BAD_SPLIT (a negative length) or
 *                   A2AV_ST_SEND_OVERRUN (the lengths add up to more than
 *                   n_keys[r]): nothing but the workspace is written, except
 *                   the splits of ranks that passed.
 * Keys past the lengths' total are not read and not written.
 * Three kernels up to W = 32: per-(table, rank) key counts, a per-rank plan,
 * and one block copy of keys and lengths together; above 32 ranks the keys
 * and the lengths are two block copies.
 */
int keys_bucketize(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                   const int64_t *const *keys, const int64_t *n_keys,
                   int32_t *const *lengths_out, int64_t *const *keys_out,
                   int64_t *split_keys, int64_t *split_lengths, void *workspace,
                   size_t workspace_bytes, int32_t *status, hipStream_t stream);

/*
 * Workspace bytes keys_exchange needs (0 for invalid sizes).
 */
size_t keys_exchange_workspace_bytes(int W, int n_tables);

/*
 * The whole embedding-key exchange of one batch in one call: the result of
 * keys_bucketize on every rank followed by the keys a2av (8-byte rows) and
 * the lengths a2av (4-byte rows) on the bucketing's split matrices, without
 * writing the bucketed arrays. This is the exchange the page "Different nccl
 * stream within EmbeddingKey alltoall and EmbeddingValue..." (TorchRec,
 * description) gives a stream of its own. Table t is owned by rank t mod W.
 *   lengths[W], keys[W], n_keys[W]   as for keys_bucketize (table order)
 *   lengths_out[W]  device int32 per receiver d: for s = 0..W-1, the lengths
 *                   rows of the tables d owns (ascending) from source s;
 *                   lengths_cap[d] (host) entries of room
 *   keys_out[W]     device int64 per receiver d: the same order for the
 *                   keys; keys_cap[d] (host) entries of room
 *   split_keys, split_lengths  device int64 [W][W] (row s = source s), the
 *                   splits of the two exchanges
 *   recv_off_keys   device int64 [W][W+1]: keys before source s's chunk at
 *                   receiver d, the total at index W
 *   workspace       device scratch of >= keys_exchange_workspace_bytes()
 *   status          checks in the order the composition meets them: if any
 *                   source fails its bucketing checks (A2AV_ST_BAD_SPLIT for a
 *                   negative length, else A2AV_ST_SEND_OVERRUN when its
 *                   lengths add to more than n_keys), those bits and nothing
 *                   written; else A2AV_ST_RECV_OVERFLOW if a receiver lacks
 *                   room (its split columns and offsets are then not written,
 *                   those of the others are) and no payload; else everything.
 * Three kernels up to W = 32: per-(table, rank) key counts, a per-receiver
 * plan (every source's table scan, then the receiver's blocks in (source,
 * table) order), and one block copy of keys and lengths together that reads
 * each source's arrays in place. Above 32 ranks the keys and the lengths are
 * two block copies.
 */
int keys_exchange(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                  const int64_t *const *keys, const int64_t *n_keys,
                  int32_t *const *lengths_out, const int64_t *lengths_cap,
                  int64_t *const *keys_out, const int64_t *keys_cap, int64_t *split_keys,
                  int64_t *split_lengths, int64_t *recv_off_keys, void *workspace,
                  size_t workspace_bytes, int32_t *status, hipStream_t stream);

/*
 * Scratch bytes per GPU behind keys_exchange_noalloc (1 MiB): room for
 * keys_exchange_workspace_bytes(W, n_tables) up to about 2700 tables at
 * W = 8, or 280 tables at W = 64.
 */
#define A2AV_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

/*
 * keys_exchange for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments without the workspace; the same kernels, outputs and
 * status bits. Its scratch is one fixed array of A2AV_NOALLOC_SCRATCH_BYTES
 * in the library's device code: each GPU the library runs on holds its own
 * copy until the process ends, and its address on a GPU is looked up (with
 * that GPU made current for the lookup) on the first call whose stream runs
 * there, then kept. A call allocates nothing: no hipMalloc, no hipFree, no
 * library routine that allocates.
 *   returns A2AV_EARG (nothing enqueued) for every argument keys_exchange
 *           rejects and when keys_exchange_workspace_bytes(W, n_tables)
 *           exceeds A2AV_NOALLOC_SCRATCH_BYTES; A2AV_EHIP when the array's
 *           address cannot be found on the stream's GPU.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no call needs any of it cleared: each writes what it reads before
 * reading it). Calls that overlap in time on one GPU, from different streams
 * or host threads, therefore race: the caller serialises them.
 */
int keys_exchange_noalloc(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                          const int64_t *const *keys, const int64_t *n_keys,
                          int32_t *const *lengths_out, const int64_t *lengths_cap,
                          int64_t *const *keys_out, const int64_t *keys_cap,
                          int64_t *split_keys, int64_t *split_lengths, int64_t *recv_off_keys,
                          int32_t *status, hipStream_t stream);

/*
 * Plain contiguous device copy of `bytes` bytes (dst and src device pointers,
 * not overlapping), with the same copy loop as a2av_copy. A bandwidth
 * ceiling for the payload kernel and the reference for counter scaling.
 */
int a2av_device_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

/* Words of the sink array a2av_device_read XORs into. */
#define A2AV_SINK_WORDS 4096

/*
 * One-direction bandwidth ceilings, with the pieces, access width and launch
 * shapes of a2av_device_copy moving as many bytes; for measurement, as the
 * ceilings of kernels whose traffic runs mostly one way (the pack's row
 * scatter writes k bytes for each byte it reads). Both want `bytes` a
 * multiple of 16 and a 16-byte-aligned buffer (else A2AV_EARG).
 *   a2av_device_read   reads every byte of src once and writes only the
 *                      device int64 sink[A2AV_SINK_WORDS] (caller-zeroed): each
 *                      wave XORs the 64-bit fold of what it read into one
 *                      sink word, so the XOR of all of them equals, for the
 *                      XOR X of all 16-byte vectors of src taken as four
 *                      32-bit words (x, y, z, w), the word
 *                      ((x ^ z) << 32) | (y ^ w).
 *   a2av_device_fill   writes the 32-bit pattern to every 4-byte word of dst,
 *                      with non-temporal stores when nontemporal != 0.
 */
int a2av_device_read(const void *src, size_t bytes, uint64_t *sink, hipStream_t stream);
int a2av_device_fill(void *dst, size_t bytes, uint32_t pattern, int nontemporal,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* A2AV_H */
