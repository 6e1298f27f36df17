// moe.hip — MoE dispatch pack and un-pack around the a2av (gfx950).
//
// The pack is a stable counting sort of the T*k routing slots of each rank
// by expert id; experts are owned by ranks in contiguous blocks, so sorting by
// expert also groups the send buffer by destination rank, which is the
// message layout of the MoE region the tuning page measures at 32 MiB.
//
//   k_moe_hist    LDS histogram of expert ids per segment of kSeg slots
//   k_moe_scan    expert-major exclusive scan of the histograms (per rank):
//                 base[e][seg] = slots of smaller experts + slots of expert e
//                 in earlier segments; also the expert counts and splits
//   k_moe_rank    stable rank inside a segment from wave64 ballots:
//                 perm[q] = base[e][seg] + earlier slots of e in the segment
//   k_moe_scatter token-major row scatter: read each token once, write it to
//                 its k packed rows
//   k_perm_check + k_moe_gather   the un-pack: out[q] = back[perm[q]]
#include <hip/hip_runtime.h>

#include <cstring>

#include "common.hpp"

namespace a2av {

constexpr int kSeg = 1024;       // routing slots per segment
constexpr int kRankWaves = 4;    // waves in a k_moe_rank block
constexpr int kSlotsPerWave = kSeg / kRankWaves;

struct MoeArgs {
    const unsigned char *tokens[A2AV_MAX_W];
    const int32_t *ids[A2AV_MAX_W];
    unsigned char *send[A2AV_MAX_W];
    int64_t *perm[A2AV_MAX_W];
    int64_t *S;
    int64_t *expert_counts;
    int32_t *hist;   // workspace: [W][E][nseg] int32
    // pack + dispatch in one step: slot rows go to row_addr[s][e] + perm * R
    // (an owner's receive buffer) instead of send[s] + perm * R
    const uint64_t *row_addr;   // [W][E]
    const int32_t *plan_bits;   // the plan's verdict
    int32_t *status;
    uint64_t R;
    int64_t T;
    int64_t Q;       // T * k
    int k;
    int E;
    int W;
    int nseg;
};

// ------------------------------------------------------------------ histogram
constexpr int kHistThreads = 256;

__global__ __launch_bounds__(kHistThreads) void k_moe_hist(const MoeArgs a) {
    extern __shared__ int32_t hist[];
    __shared__ int poisoned;
    const int r = blockIdx.y, seg = blockIdx.x, E = a.E;
    const int32_t *ids = a.ids[r];
    const int64_t q0 = (int64_t)seg * kSeg;
    // the segment's ids, every load in flight together, and then the word
    // (blocks of this launch set it; one read per block keeps its waves in
    // agreement)
    constexpr int kPer = kSeg / kHistThreads;
    int32_t idv[kPer];
    const bool any = q0 < a.Q;  // the same in the whole block
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int64_t q = q0 + threadIdx.x + j * kHistThreads;
        idv[j] = any ? ids[q < a.Q ? q : a.Q - 1] : 0;
    }
    if (threadIdx.x == 0) poisoned = status_poisoned(a.status);
    for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
    __syncthreads();
    if (poisoned) return;
    int bad = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        if (q0 + threadIdx.x + j * kHistThreads < a.Q) {
            const int e = idv[j];
            if ((unsigned)e >= (unsigned)E) bad = 1;
            else atomicAdd(&hist[e], 1);
        }
    }
    bad = __syncthreads_or(bad);
    int32_t *H = a.hist + (size_t)r * E * a.nseg;
    for (int e = threadIdx.x; e < E; e += kHistThreads) H[(size_t)e * a.nseg + seg] = hist[e];
    if (bad && threadIdx.x == 0) atomicOr(a.status, A2AV_ST_BAD_EXPERT);
}

// ------------------------------------------------------------------ scan
// One block per rank, in passes of kScanPass counters: thread t loads
// counters t, t + 1024, ... of the pass (coalesced, all in flight together),
// each wave scans every group of 64 with DPP moves, and one wave scans the
// 256 group totals of the pass, in counter order, through LDS. (A form where
// each thread scanned a contiguous run of 16 counters made every load and
// store instruction touch 64 cache lines: 18.3 us per call against 6.1 us at
// 8 ranks x 256 experts x 64 segments.)
constexpr int kScanPer = 16;                     // counters per thread per pass
constexpr int kScanWaves = 1024 / kWave;         // 16
constexpr int kScanPass = kScanPer * 1024;       // counters per pass
static_assert(kScanPer * kScanWaves == 4 * kWave, "one wave scans the group totals, 4 per lane");

__global__ __launch_bounds__(1024) void k_moe_scan(const MoeArgs a) {
    __shared__ int32_t part[kScanPer * kScanWaves];  // group totals of a pass, counter order
    __shared__ int32_t carry_sh;
    if (status_poisoned(a.status)) return;
    const int r = blockIdx.x;
    const int64_t N = (int64_t)a.E * a.nseg;
    int32_t *H = a.hist + (size_t)r * N;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int32_t carry = 0;  // counters of the passes before
    for (int64_t base = 0; base < N; base += kScanPass) {
        int32_t v[kScanPer], inc[kScanPer];
#pragma unroll
        for (int u = 0; u < kScanPer; u++) {
            const int64_t i = base + (int64_t)u * 1024 + tid;
            v[u] = i < N ? H[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kScanPer; u++) {
            inc[u] = (int32_t)wave_incl_scan_u32((uint32_t)v[u]);
            if (lane == kWave - 1) part[u * kScanWaves + wave] = inc[u];
        }
        __syncthreads();
        if (wave == 0) {
            int32_t t[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                t[j] = part[lane * 4 + j];
                sum += t[j];
            }
            int32_t run = (int32_t)wave_incl_scan_u32((uint32_t)sum) - sum + carry;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                part[lane * 4 + j] = run;
                run += t[j];
            }
            if (lane == kWave - 1) carry_sh = run;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kScanPer; u++) {
            const int64_t i = base + (int64_t)u * 1024 + tid;
            if (i < N) H[i] = part[u * kScanWaves + wave] + inc[u] - v[u];
        }
        carry = carry_sh;
        __syncthreads();  // part and carry_sh are rewritten by the next pass
    }
    // base of expert e = H[e][0]; the count is the gap to the next base
    const int E = a.E, nthr = blockDim.x;
    for (int e = threadIdx.x; e < E; e += nthr) {
        const int64_t b = H[(size_t)e * a.nseg];
        const int64_t nb = e + 1 < E ? (int64_t)H[(size_t)(e + 1) * a.nseg] : a.Q;
        a.expert_counts[(size_t)r * E + e] = nb - b;
    }
    const int per_rank = E / a.W;
    for (int d = threadIdx.x; d < a.W; d += nthr) {
        const int64_t b = H[(size_t)d * per_rank * a.nseg];
        const int64_t nb = d + 1 < a.W ? (int64_t)H[(size_t)(d + 1) * per_rank * a.nseg] : a.Q;
        a.S[(size_t)r * a.W + d] = nb - b;
    }
}

// ------------------------------------------------------------------ stable rank
// Wave w of the block owns slots [w*256, (w+1)*256) of the segment and walks
// them 64 at a time in order. Lanes holding the same expert find each other
// with one ballot per bit of the id; the lowest such lane bumps the wave's LDS
// counter. After a barrier, the counts of earlier waves are added.
__global__ __launch_bounds__(256) void k_moe_rank(const MoeArgs a) {
    extern __shared__ int32_t cnt[];  // [kRankWaves][E]
    const int r = blockIdx.y, seg = blockIdx.x, E = a.E;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    constexpr int kChunks = kSlotsPerWave / kWave;
    const int32_t *ids = a.ids[r];
    const int32_t *H = a.hist + (size_t)r * E * a.nseg;
    const int64_t qbase = (int64_t)seg * kSeg + wave * kSlotsPerWave;
    // the wave's ids, then their experts' bases for this segment (written by
    // the scan), all loaded before any ballot; slots past Q (the launch has
    // Q >= 1) read the last one and count nothing. The word is read beside
    // them: no kernel of this launch writes it, so every thread finds the
    // same value.
    int e_of[kChunks];
    int32_t hb[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
        const int64_t q = qbase + c * kWave + lane;
        e_of[c] = ids[q < a.Q ? q : a.Q - 1];
    }
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
        const int e = (unsigned)e_of[c] < (unsigned)E ? e_of[c] : 0;
        hb[c] = H[(size_t)e * a.nseg + seg];
    }
    if (status_poisoned(a.status)) return;
    for (int i = threadIdx.x; i < kRankWaves * E; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const uint64_t below = (1ull << lane) - 1;
    int32_t *mine = cnt + wave * E;
    int rank_of[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
        const int64_t q = qbase + c * kWave + lane;
        const bool ok = q < a.Q;
        const int e = ok ? e_of[c] : 0;
        uint64_t peers = __ballot(ok);
        for (int b = 0; b < nbits; b++) {
            const int bit = (e >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        rank_of[c] = 0;
        if (ok) {
            const int before = mine[e];
            const int rk = __popcll(peers & below);
            rank_of[c] = before + rk;
            if (rk == 0) mine[e] = before + __popcll(peers);
        }
    }
    __syncthreads();
    int64_t *perm = a.perm[r];
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
        const int64_t q = qbase + c * kWave + lane;
        if (q < a.Q) {
            const int e = e_of[c];
            int32_t pre = 0;
            for (int w = 0; w < wave; w++) pre += cnt[w * E + e];
            perm[q] = (int64_t)hb[c] + pre + rank_of[c];
        }
    }
}

// ------------------------------------------------------------------ scatter
// One wave per (rank, token, chunk of 64 x U vectors): the chunk of the token
// row is read once into registers and stored to the k rows of its slots. The
// host picks the chunk count and U (1..8) so that the chunks tile the row
// with as few idle lanes as it can (a 14 KiB row: two chunks of 7 vectors per
// lane); short waves with few registers keep more stores in flight per CU
// than one wave per row did. Lane j < k holds the address of slot j's row:
// send[r] + perm * R for the pack, or the owner's receive row
// row_addr[r][e] + perm * R when the pack and the dispatch run as one step
// (DIRECT). Rows or bases that are not 16-byte aligned take one wave per
// token and k realigning wave copies of the row (the re-reads hit in L2).
template <int U, bool ALIGNED, bool DIRECT>
__global__ __launch_bounds__(256) void k_moe_scatter(const MoeArgs a, uint64_t nch) {
    if (status_poisoned(a.status)) return;
    if constexpr (DIRECT) {
        // a receiver too small: report once; no wave writes a row
        const int32_t pb = *(const const_i32 *)a.plan_bits;
        if (pb) {
            if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.status, pb);
            return;
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t nwork = (uint64_t)a.W * (uint64_t)a.T * nch;
    const uint64_t R = a.R;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (uint64_t w = (uint64_t)blockIdx.x * wpb + wid; w < nwork; w += (uint64_t)gridDim.x * wpb) {
        const uint64_t tok = w / nch;
        const uint64_t c = w - tok * nch;
        const int r = (int)(tok / (uint64_t)a.T);
        const int64_t t = (int64_t)(tok - (uint64_t)r * (uint64_t)a.T);
        const unsigned char *src = a.tokens[r] + (uint64_t)t * R;
        // the token's k rows, one address per lane, fetched before any store
        // (k <= 64 here; the host routes larger k to the pack's unaligned form)
        uint64_t al = 0;
        bool okl = false;
        if (lane < a.k) {
            const int64_t p = a.perm[r][t * a.k + lane];
            okl = p >= 0 && p < a.Q;
            if constexpr (DIRECT) {
                const int e = a.ids[r][t * a.k + lane];
                okl = okl && (unsigned)e < (unsigned)a.E;
                al = okl ? a.row_addr[(int64_t)r * a.E + e] + (uint64_t)p * R : 0;
            } else {
                al = (uint64_t)(uintptr_t)a.send[r] + (uint64_t)p * R;
            }
        }
        const uint64_t okm = __ballot(okl);
        if constexpr (ALIGNED) {
            const uint64_t nv = R / 16;
            const u32x4 *s16 = (const u32x4 *)src;
            const uint64_t base = c * (uint64_t)kWave * U;
            // indices past the row end are clamped to its last vector (no
            // per-lane branch; the clamped lanes store identical bytes)
            u32x4 v[U];
            uint64_t idx[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t i = base + (uint64_t)u * kWave + lane;
                idx[u] = i < nv ? i : nv - 1;
                v[u] = ld<true>(s16 + idx[u]);
            }
            for (int j = 0; j < a.k; j++) {
                if (!((okm >> j) & 1)) continue;
                u32x4 *d16 = (u32x4 *)(uintptr_t)readlane_u64(al, j);
#pragma unroll
                for (int u = 0; u < U; u++) st<false>(d16 + idx[u], v[u]);
            }
        } else if constexpr (DIRECT) {
            for (int j = 0; j < a.k; j++) {
                if (!((okm >> j) & 1)) continue;
                wave_copy_any<4>((unsigned char *)(uintptr_t)readlane_u64(al, j), src, R, lane);
            }
        } else {
            // any k: slot j's row straight from perm
            for (int j = 0; j < a.k; j++) {
                const int64_t p = a.perm[r][t * a.k + j];
                if (p < 0 || p >= a.Q) continue;
                wave_copy_any<4>(a.send[r] + (uint64_t)p * R, src, R, lane);
            }
        }
    }
}

// ------------------------------------------------------------------ row shifts
// Where slot rows sit at their owners when the pack and the dispatch run as
// one step. Owner d = e / P (P = E / W) keeps its rows in one of two orders:
// layout 0 = (source, expert, slot), as the pack followed by the a2av leaves
// them; layout 1 = (expert, source, slot), as the pack followed by the
// grouped dispatch leaves them. Slot q of source s with expert e and pack row
// p then sits at owner row p + shift(s, e):
//   layout 0: shift = (rows d holds from sources before s) - Y_s(d*P)
//   layout 1: shift = (rows d holds of its experts before e)
//                     + (rows of expert e from sources before s) - Y_s(e)
// where Y_s(e) = rows of source s's smaller experts (its pack position).
struct ShiftArgs {
    const unsigned char *base[A2AV_MAX_W];  // row 0 of each owner's receive buffer
    int64_t limit[A2AV_MAX_W];              // rows each owner's buffer holds
    const int64_t *counts;                  // [W][E]
    uint64_t *row_addr;                     // [W][E] base[d] + shift * R (mod 2^64)
    int64_t *ystart;                        // [W][E] Y_s(e), or null
    int64_t *block_offsets;                 // [W][G + 1] (G = W or P), or null
    int32_t *words;                         // [0] plan bits, [1] cleared for the slot check
    const int32_t *status;
    uint64_t R;
    int W;
    int E;
    int layout;
    int over_bit;      // raised when an owner's rows exceed its limit
    int check_counts;  // counts come from the caller: range-check them
};

__global__ __launch_bounds__(kPlanThreads) void k_shift_plan(const ShiftArgs a) {
    __shared__ ScanLds3 lds;
    __shared__ int64_t gb[A2AV_MAX_W + 1];  // column sums over experts before d*P
    __shared__ int64_t bb[A2AV_MAX_W + 1];  // rows of sources before s, experts before d*P
    __shared__ int64_t yb[A2AV_MAX_W + 1];  // Y_s(d*P)
    __shared__ uint64_t base[A2AV_MAX_W];
    __shared__ int64_t limit[A2AV_MAX_W];
    const int s = blockIdx.x, tid = threadIdx.x;
    const int W = a.W, E = a.E, P = E / W;
    // thread tid: experts tid * kPlanPer + u, every source's count of them,
    // read in groups of 8 sources with all of a group's loads in flight
    // together (entries past W or E read entry 0 and count nothing); with
    // them the owners' bases and limits and the status word. Every count is
    // read by exactly one thread, which also range-checks it.
    constexpr int kGroup = 8;
    int64_t col[kPlanPer], before[kPlanPer], mine[kPlanPer];
    int bad = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) col[u] = before[u] = mine[u] = 0;
    const uint64_t my_base = (uint64_t)(uintptr_t)a.base[tid < W ? tid : 0];
    const int64_t my_limit = a.limit[tid < W ? tid : 0];
    const int poisoned = status_poisoned(a.status);
    auto group = [&](int s0) {
        int64_t c[kPlanPer][kGroup];
#pragma unroll
        for (int u = 0; u < kPlanPer; u++)
#pragma unroll
            for (int j = 0; j < kGroup; j++) {
                const int e = tid * kPlanPer + u, s2 = s0 + j;
                c[u][j] = a.counts[e < E && s2 < W ? (int64_t)s2 * E + e : 0];
            }
#pragma unroll
        for (int u = 0; u < kPlanPer; u++)
#pragma unroll
            for (int j = 0; j < kGroup; j++) {
                const int e = tid * kPlanPer + u, s2 = s0 + j;
                if (e < E && s2 < W) {
                    const int64_t v = c[u][j];
                    bad |= (int)split_invalid(v);
                    col[u] += v;
                    if (s2 < s) before[u] += v;
                    if (s2 == s) mine[u] = v;
                }
            }
    };
    // the first group in line with the loads above, so that no loop head
    // waits for them first; threads past the experts load nothing
    if (tid * kPlanPer < E) {
        group(0);
        for (int s0 = kGroup; s0 < W; s0 += kGroup) group(s0);
    }
    if (tid < W) {
        base[tid] = my_base;
        limit[tid] = my_limit;
    }
    const int flags = __syncthreads_or(poisoned * 2 | (a.check_counts ? bad : 0));
    if (flags & 2) return;
    if (flags & 1) {
        if (s == 0 && tid == 0) {
            a.words[0] = A2AV_ST_BAD_SPLIT;
            a.words[1] = 0;
        }
        return;
    }
    int64_t scol = 0, sbef = 0, smine = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        scol += col[u];
        sbef += before[u];
        smine += mine[u];
    }
    const int64_t sums[3] = {scol, sbef, smine};
    int64_t ex[3], tot[3];
    block_excl_scan3(sums, lds, ex, tot);
    int64_t gx = ex[0], yx = ex[2];
    const int64_t bx = ex[1], gt = tot[0], bt = tot[1], yt = tot[2];
    // the prefixes at every owner's first expert
    {
        int64_t g = gx, b = bx, y = yx;
#pragma unroll
        for (int u = 0; u < kPlanPer; u++) {
            const int e = tid * kPlanPer + u;
            if (e < E && e % P == 0) {
                gb[e / P] = g;
                bb[e / P] = b;
                yb[e / P] = y;
            }
            g += col[u];
            b += before[u];
            y += mine[u];
        }
    }
    if (tid == 0) {
        gb[W] = gt;
        bb[W] = bt;
        yb[W] = yt;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int e = tid * kPlanPer + u;
        if (e < E) {
            const int d = e / P;
            const int64_t shift = a.layout == 0 ? (bb[d + 1] - bb[d]) - yb[d]
                                                : (gx - gb[d]) + before[u] - yx;
            a.row_addr[(int64_t)s * E + e] = base[d] + (uint64_t)shift * a.R;
            if (a.ystart) a.ystart[(int64_t)s * E + e] = yx;
            if (a.block_offsets && a.layout == 1 && s == 0)
                a.block_offsets[(int64_t)d * (P + 1) + (e - d * P)] = gx - gb[d];
        }
        gx += col[u];
        yx += mine[u];
    }
    if (tid < W && a.block_offsets) {
        const int d = tid;
        if (a.layout == 0) {
            a.block_offsets[(int64_t)d * (W + 1) + s] = bb[d + 1] - bb[d];
            if (s == 0) a.block_offsets[(int64_t)d * (W + 1) + W] = gb[d + 1] - gb[d];
        } else if (s == 0) {
            a.block_offsets[(int64_t)d * (P + 1) + P] = gb[d + 1] - gb[d];
        }
    }
    if (s == 0) {
        // every owner's rows against what its buffer holds
        int over = 0;
        if (tid < W) over = gb[tid + 1] - gb[tid] > limit[tid];
        over = __syncthreads_or(over);
        if (tid == 0) {
            a.words[0] = over ? a.over_bit : 0;
            a.words[1] = 0;
        }
    }
}

// ------------------------------------------------------------------ return in one step
// The inverse of the fused pack + dispatch: every slot's row read back from
// its owner's receive buffer, out[s][q] = that row.
struct ReturnArgs {
    unsigned char *out[A2AV_MAX_W];
    const int32_t *ids[A2AV_MAX_W];
    const int64_t *perm[A2AV_MAX_W];
    const int64_t *counts;     // [W][E]
    const uint64_t *row_addr;  // [W][E] (plan)
    const int64_t *ystart;     // [W][E] (plan)
    uint64_t *xaddr;           // [W][T*k] each slot's row address, or null
    int32_t *words;            // [0] plan bits, [1] slot bits
    int32_t *status;
    uint64_t R;
    int64_t Q;
    int E;
    int W;
};

// One thread per (slot, source): its id in range and its pack row inside its
// expert's block, so every row the gather reads lies in the owner's buffer;
// for the combine, also the address of the slot's row.
__global__ __launch_bounds__(256) void k_slot_check(const ReturnArgs a) {
    const int s = blockIdx.y;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // the slot's id and pack row beside the word (the launch has Q >= 1;
    // threads past Q read slot 0 and check nothing), then the entries of its
    // expert together
    const int64_t qc = q < a.Q ? q : 0;
    const int32_t e = a.ids[s][qc];
    const int64_t pq = a.perm[s][qc];
    if (status_poisoned(a.status)) return;
    int bad = 0;
    if (q < a.Q) {
        if (e < 0 || e >= a.E) {
            bad = A2AV_ST_BAD_EXPERT;
        } else {
            const int64_t ys = a.ystart[(int64_t)s * a.E + e];
            const int64_t cn = a.counts[(int64_t)s * a.E + e];
            const uint64_t ra = a.xaddr ? a.row_addr[(int64_t)s * a.E + e] : 0;
            const int64_t p = pq - ys;
            if (p < 0 || p >= cn) bad = A2AV_ST_BAD_PERM;
            else if (a.xaddr) a.xaddr[(int64_t)s * a.Q + q] = ra + (uint64_t)pq * a.R;
        }
    }
    const int be = __ballot(bad & A2AV_ST_BAD_EXPERT) != 0, bp = __ballot(bad & A2AV_ST_BAD_PERM) != 0;
    if ((be || bp) && (threadIdx.x & (kWave - 1)) == 0)
        atomicOr(&a.words[1], (be ? A2AV_ST_BAD_EXPERT : 0) | (bp ? A2AV_ST_BAD_PERM : 0));
}

// One wave per (source, slot): the slot's row copied home. With a verdict
// from the plan or the slot check, the first thread reports it (a bad count
// alone, since the other checks read the counts) and no row moves.
template <int U, bool ALIGNED>
__global__ __launch_bounds__(256) void k_moe_gather_home(const ReturnArgs a) {
    if (status_poisoned(a.status)) return;
    const int32_t pb = *(const const_i32 *)&a.words[0];
    const int32_t cw = *(const const_i32 *)&a.words[1];
    if (pb | cw) {
        if (blockIdx.x == 0 && threadIdx.x == 0)
            atomicOr(a.status, (pb & A2AV_ST_BAD_SPLIT) ? A2AV_ST_BAD_SPLIT : (pb | cw));
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t nwork = (uint64_t)a.W * (uint64_t)a.Q;
    const uint64_t R = a.R;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (uint64_t w = (uint64_t)blockIdx.x * wpb + wid; w < nwork; w += (uint64_t)gridDim.x * wpb) {
        const int r = (int)(w / (uint64_t)a.Q);
        const int64_t q = (int64_t)(w - (uint64_t)r * (uint64_t)a.Q);
        const int e = *(const const_i32 *)(a.ids[r] + q);
        const int64_t p = *(const const_i64 *)(a.perm[r] + q);
        const unsigned char *src =
            (const unsigned char *)(uintptr_t)(a.row_addr[(int64_t)r * a.E + e] + (uint64_t)p * R);
        unsigned char *dst = a.out[r] + (uint64_t)q * R;
        if constexpr (ALIGNED) copy_elems<u32x4, kWave, U, true>((u32x4 *)dst, (const u32x4 *)src, R / 16, lane);
        else wave_copy_any<U>(dst, src, R, lane);
    }
}

// ------------------------------------------------------------------ un-pack
struct UnpackArgs {
    const unsigned char *back[A2AV_MAX_W];
    const int64_t *perm[A2AV_MAX_W];
    unsigned char *out[A2AV_MAX_W];
    int32_t *status;
    uint64_t R;
    int64_t Q;
    int W;
};

__global__ __launch_bounds__(256) void k_perm_check(const UnpackArgs a) {
    if (status_poisoned(a.status)) return;
    const int r = blockIdx.y;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (q < a.Q) {
        const int64_t p = a.perm[r][q];
        bad = p < 0 || p >= a.Q;
    }
    if (__ballot(bad) != 0 && (threadIdx.x & (kWave - 1)) == 0) atomicOr(a.status, A2AV_ST_BAD_PERM);
}

// One wave per (rank, slot): out[q] = back[perm[q]].
template <int U, bool ALIGNED>
__global__ __launch_bounds__(256) void k_moe_gather(const UnpackArgs a) {
    if (status_poisoned(a.status)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t nwork = (uint64_t)a.W * (uint64_t)a.Q;
    const uint64_t R = a.R;
    for (uint64_t w = (uint64_t)blockIdx.x * wpb + threadIdx.x / kWave; w < nwork;
         w += (uint64_t)gridDim.x * wpb) {
        const int r = (int)(w / (uint64_t)a.Q);
        const int64_t q = (int64_t)(w - (uint64_t)r * (uint64_t)a.Q);
        const int64_t p = a.perm[r][q];
        const unsigned char *src = a.back[r] + (uint64_t)p * R;
        unsigned char *dst = a.out[r] + (uint64_t)q * R;
        if constexpr (ALIGNED) copy_elems<u32x4, kWave, U, true>((u32x4 *)dst, (const u32x4 *)src, R / 16, lane);
        else wave_copy_any<U>(dst, src, R, lane);
    }
}

// ------------------------------------------------------------------ combine
// Gate-weighted combine: out[r][t][h] = bf16( fma chain over j = 0..k-1 of
// w[r][t][j] * back[r][perm[r][t*k+j]][h] ), accumulated in fp32 from +0 with
// one fused multiply-add per slot, in slot order, rounded to bfloat16 to
// nearest even at the end. One wave per (rank, token): lane j of the wave
// holds perm and weight of slot j, and every lane owns 8 consecutive elements
// (16 bytes) of the token's row per vector step.
struct CombineArgs {
    const unsigned char *back[A2AV_MAX_W];
    const int64_t *perm[A2AV_MAX_W];
    const float *w[A2AV_MAX_W];
    unsigned char *out[A2AV_MAX_W];
    // read at the owners (HOME): slot rows at xaddr[r][t*k + j], after the
    // verdict in words[0] (plan) and words[1] (slot check)
    const uint64_t *xaddr;
    const int32_t *words;
    int32_t *status;
    int64_t T;
    int64_t H;
    int k;
    int W;
};

// The verdict of the plan and the slot check of a combine read at the owners:
// the first thread reports it (a bad count alone, since the other checks read
// the counts); then no wave writes.
__device__ __forceinline__ bool home_verdict(const CombineArgs &a) {
    const int32_t pb = *(const const_i32 *)&a.words[0];
    const int32_t cw = *(const const_i32 *)&a.words[1];
    if ((pb | cw) == 0) return false;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        atomicOr(a.status, (pb & A2AV_ST_BAD_SPLIT) ? A2AV_ST_BAD_SPLIT : (pb | cw));
    return true;
}


constexpr int kCombineGroup = 8;  // slots whose rows are loaded before their fmas

// Occupancy caps of the combine, as LDS per workgroup that the kernel does not
// use: its 51 registers would allow eight waves per SIMD, and fewer streamed
// HBM better (dispatch workload, same box: 1502 -> 1402 us with 32 KiB for the
// combine over a returned buffer; 1529 -> 1427 us with 52 KiB for the combine
// read at the owners, whose best cap differs).
constexpr unsigned kCombineLds = 32768;
constexpr unsigned kCombineHomeLds = 53248;

// One wave per (rank, token, chunk of 64 vectors = 512 elements). The wave
// index is made uniform so that the token, its perm entries and weights (read
// with scalar loads) and the row bases all live in scalar registers; each
// row load is then a base in scalar registers plus one shared 32-bit lane
// offset. Slots go in groups of 8: the group's 8 row loads are issued before
// any of its fused multiply-adds (a scheduling barrier keeps the compiler from
// interleaving them), and the adds run in slot order. Short-lived waves with
// few registers keep many loads in flight per CU: in measurements this beat
// looping waves, with or without software pipelining.
template <bool SNT, bool HOME>
__global__ __launch_bounds__(256) void k_moe_combine(const CombineArgs a, uint64_t nchunk) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    // earlier kernels' verdict; HOME waves also OR bits in (home_verdict), and
    // every wave of this launch reads the same words and reaches the same one
    if (status_at_entry(a.status)) return;
    if constexpr (HOME) {
        if (home_verdict(a)) return;
    }
    const uint64_t nwork = (uint64_t)a.W * (uint64_t)a.T * nchunk;
    const int k = a.k;
    const uint64_t rowb = (uint64_t)a.H * 2;
    const uint64_t nv = (uint64_t)a.H / 8;  // 16-byte vectors per row
    const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (uint64_t wk = (uint64_t)blockIdx.x * wpb + wid; wk < nwork;
         wk += (uint64_t)gridDim.x * wpb) {
        const uint64_t tok = wk / nchunk;
        const uint64_t c = wk - tok * nchunk;
        const int r = (int)(tok / (uint64_t)a.T);
        const int64_t t = (int64_t)(tok - (uint64_t)r * (uint64_t)a.T);
        const const_i64 *pp = HOME ? (const const_i64 *)(a.xaddr + (uint64_t)r * a.T * k + t * k)
                                   : (const const_i64 *)(a.perm[r] + t * k);
        const const_i32 *wp = (const const_i32 *)(a.w[r] + t * k);
        const unsigned char *bk = a.back[r];
        uint64_t i = c * kWave + lane;
        i = i < nv ? i : nv - 1;  // clamped lanes redo the last vector
        const uint32_t off = (uint32_t)i * 16u;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
            u32x4 v[kCombineGroup];
            float wt[kCombineGroup];
#pragma unroll
            for (int g = 0; g < kCombineGroup; g++) {
                // past the last slot the load repeats slot k-1; its fma is skipped
                const int j = j0 + g < k ? j0 + g : k - 1;
                const unsigned char *row = HOME ? (const unsigned char *)(uintptr_t)(uint64_t)pp[j]
                                                : bk + (uint64_t)pp[j] * rowb;
                v[g] = ld<true>((const u32x4 *)(row + off));
                wt[g] = __int_as_float(wp[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < kCombineGroup; g++) {
                if (j0 + g < k) {
                    acc[0] = __builtin_fmaf(wt[g], bf16_lo(v[g].x), acc[0]);
                    acc[1] = __builtin_fmaf(wt[g], bf16_hi(v[g].x), acc[1]);
                    acc[2] = __builtin_fmaf(wt[g], bf16_lo(v[g].y), acc[2]);
                    acc[3] = __builtin_fmaf(wt[g], bf16_hi(v[g].y), acc[3]);
                    acc[4] = __builtin_fmaf(wt[g], bf16_lo(v[g].z), acc[4]);
                    acc[5] = __builtin_fmaf(wt[g], bf16_hi(v[g].z), acc[5]);
                    acc[6] = __builtin_fmaf(wt[g], bf16_lo(v[g].w), acc[6]);
                    acc[7] = __builtin_fmaf(wt[g], bf16_hi(v[g].w), acc[7]);
                }
            }
        }
        u32x4 o;
        o.x = to_bf16(acc[0]) | (to_bf16(acc[1]) << 16);
        o.y = to_bf16(acc[2]) | (to_bf16(acc[3]) << 16);
        o.z = to_bf16(acc[4]) | (to_bf16(acc[5]) << 16);
        o.w = to_bf16(acc[6]) | (to_bf16(acc[7]) << 16);
        st<SNT>((u32x4 *)(a.out[r] + (uint64_t)t * rowb + off), o);
    }
}

// Any row width or alignment: one element per lane per step.
template <bool HOME>
__global__ __launch_bounds__(256) void k_moe_combine_any(const CombineArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    if (status_at_entry(a.status)) return;
    if constexpr (HOME) {
        if (home_verdict(a)) return;
    }
    const uint64_t nwork = (uint64_t)a.W * (uint64_t)a.T;
    const int k = a.k;
    const uint64_t H = (uint64_t)a.H;
    for (uint64_t wk = (uint64_t)blockIdx.x * wpb + threadIdx.x / kWave; wk < nwork;
         wk += (uint64_t)gridDim.x * wpb) {
        const int r = (int)(wk / (uint64_t)a.T);
        const int64_t t = (int64_t)(wk - (uint64_t)r * (uint64_t)a.T);
        const int64_t *pp = a.perm[r] + t * k;
        const float *wp = a.w[r] + t * k;
        const uint16_t *bk = (const uint16_t *)a.back[r];
        uint16_t *dst = (uint16_t *)a.out[r] + (uint64_t)t * H;
        const uint64_t *xa = HOME ? a.xaddr + (uint64_t)r * a.T * k + t * k : nullptr;
        for (uint64_t h = lane; h < H; h += kWave) {
            float acc = 0.0f;
            for (int j = 0; j < k; j++) {
                const uint16_t *row = HOME ? (const uint16_t *)(uintptr_t)xa[j]
                                           : bk + (uint64_t)pp[j] * H;
                acc = __builtin_fmaf(wp[j], __uint_as_float((uint32_t)row[h] << 16), acc);
            }
            dst[h] = (uint16_t)to_bf16(acc);
        }
    }
}

static int64_t n_segments(int64_t Q) { return (Q + kSeg - 1) / kSeg; }

static bool moe_sizes_ok(int W, int64_t T, int k, int E) {
    if (W < 1 || W > A2AV_MAX_W || T < 0 || k < 1 || E < 1 || E > A2AV_MAX_EXPERTS) return false;
    if (E % W != 0) return false;
    if (T > ((int64_t)1 << 31) / k) return false;
    return T * k < ((int64_t)1 << 31);
}

// The counting sort of the pack for every rank: histograms, their scan (expert
// counts and splits), then the stable rank of every slot (perm).
static void launch_pack_sort(MoeArgs &a, hipStream_t stream) {
    const int W = a.W, E = a.E;
    a.nseg = (int)n_segments(a.Q);
    const int nseg_grid = a.nseg > 0 ? a.nseg : 1;
    if (a.nseg > 0) {
        hipLaunchKernelGGL(k_moe_hist, dim3(a.nseg, W), dim3(kHistThreads), E * sizeof(int32_t), stream, a);
    } else {
        a.nseg = 1;  // no slots: one empty segment so counts and splits come out zero
        hipLaunchKernelGGL(k_moe_hist, dim3(1, W), dim3(kHistThreads), E * sizeof(int32_t), stream, a);
    }
    hipLaunchKernelGGL(k_moe_scan, dim3(W), dim3(1024), 0, stream, a);
    if (a.Q > 0)
        hipLaunchKernelGGL(k_moe_rank, dim3(nseg_grid, W), dim3(kRankWaves * kWave),
                           kRankWaves * E * sizeof(int32_t), stream, a);
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// The row scatter: chunks of at most 512 vectors (8 per lane), as few as
// tile the row, and U = the vectors per lane that cover one chunk.
template <bool DIRECT>
static void launch_scatter(const MoeArgs &a, bool aligned, hipStream_t stream) {
    const uint64_t ntok = (uint64_t)a.W * (uint64_t)a.T;
    if (!aligned || a.k > kWave) {
        uint64_t blocks = (ntok + 3) / 4;
        if (blocks > max_grid()) blocks = max_grid();  // the wave loop strides over the rest
        hipLaunchKernelGGL((k_moe_scatter<4, false, DIRECT>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, a, (uint64_t)1);
        return;
    }
    const uint64_t nv = a.R / 16;
    const uint64_t nch = (nv + 8 * kWave - 1) / (8 * kWave);
    const int U = (int)((nv + nch * kWave - 1) / (nch * kWave));
    uint64_t blocks = (ntok * nch + 3) / 4;
    if (blocks > max_grid()) blocks = max_grid();
    const dim3 g((unsigned)blocks), b(256);
    switch (U) {
    case 1: hipLaunchKernelGGL((k_moe_scatter<1, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 2: hipLaunchKernelGGL((k_moe_scatter<2, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 3: hipLaunchKernelGGL((k_moe_scatter<3, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 4: hipLaunchKernelGGL((k_moe_scatter<4, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 5: hipLaunchKernelGGL((k_moe_scatter<5, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 6: hipLaunchKernelGGL((k_moe_scatter<6, true, DIRECT>), g, b, 0, stream, a, nch); break;
    case 7: hipLaunchKernelGGL((k_moe_scatter<7, true, DIRECT>), g, b, 0, stream, a, nch); break;
    default: hipLaunchKernelGGL((k_moe_scatter<8, true, DIRECT>), g, b, 0, stream, a, nch); break;
    }
}

}  // namespace a2av

using namespace a2av;

A2AV_API size_t moe_pack_workspace_bytes(int W, int64_t T, int k, int E) {
    if (!moe_sizes_ok(W, T, k, E)) return 0;
    const int64_t nseg = n_segments(T * k);
    size_t b = (size_t)W * (size_t)E * (size_t)(nseg > 0 ? nseg : 1) * sizeof(int32_t);
    return (b + 255) & ~(size_t)255;
}

A2AV_API int moe_pack(int W, int64_t T, int k, int E, size_t row_bytes,
                      const void *const *tokens, const int32_t *const *ids, void *const *send,
                      int64_t *const *perm, int64_t *S, int64_t *expert_counts, void *workspace,
                      size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (!moe_sizes_ok(W, T, k, E) || row_bytes == 0 || !tokens || !ids || !send || !perm || !S ||
        !expert_counts || !status)
        return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_pack_workspace_bytes(W, T, k, E)) return A2AV_EARG;
    if ((uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
    MoeArgs a;
    std::memset(&a, 0, sizeof(a));
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!tokens[r] || !ids[r] || !send[r] || !perm[r])) return A2AV_EARG;
        a.tokens[r] = (const unsigned char *)tokens[r];
        a.ids[r] = ids[r];
        a.send[r] = (unsigned char *)send[r];
        a.perm[r] = perm[r];
        aligned = aligned && ((uintptr_t)tokens[r] % 16 == 0) && ((uintptr_t)send[r] % 16 == 0);
    }
    a.S = S;
    a.expert_counts = expert_counts;
    a.hist = (int32_t *)workspace;
    a.status = status;
    a.R = row_bytes;
    a.T = T;
    a.k = k;
    a.Q = T * k;
    a.E = E;
    a.W = W;
    launch_pack_sort(a, stream);
    if (a.Q > 0) launch_scatter<false>(a, aligned, stream);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t moe_pack_dispatch_workspace_bytes(int W, int64_t T, int k, int E) {
    const size_t pack = moe_pack_workspace_bytes(W, T, k, E);
    if (pack == 0) return 0;
    return pack + round256((size_t)W * (size_t)E * 8) + 256;
}

A2AV_API int moe_pack_dispatch(int W, int64_t T, int k, int E, size_t row_bytes,
                               const void *const *tokens, const int32_t *const *ids,
                               void *const *recv, const int64_t *recv_cap_rows,
                               int64_t *const *perm, int64_t *S, int64_t *expert_counts,
                               int64_t *block_offsets, int layout, void *workspace,
                               size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (!moe_sizes_ok(W, T, k, E) || k > kWave || row_bytes == 0 || !tokens || !ids || !recv ||
        !recv_cap_rows || !perm || !S || !expert_counts || !block_offsets || !status ||
        (layout != 0 && layout != 1))
        return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_pack_dispatch_workspace_bytes(W, T, k, E))
        return A2AV_EARG;
    if ((uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
    MoeArgs a;
    ShiftArgs p;
    std::memset(&a, 0, sizeof(a));
    std::memset(&p, 0, sizeof(p));
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!tokens[r] || !ids[r] || !perm[r])) return A2AV_EARG;
        const int64_t cap = recv_cap_rows[r];
        if (cap < 0 || (uint64_t)cap > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
        if (cap > 0 && !recv[r]) return A2AV_EARG;
        a.tokens[r] = (const unsigned char *)tokens[r];
        a.ids[r] = ids[r];
        a.perm[r] = perm[r];
        p.base[r] = (const unsigned char *)recv[r];
        p.limit[r] = cap;
        aligned = aligned && ((uintptr_t)tokens[r] % 16 == 0) && ((uintptr_t)recv[r] % 16 == 0);
    }
    unsigned char *ws = (unsigned char *)workspace;
    const size_t pack_ws = moe_pack_workspace_bytes(W, T, k, E);
    uint64_t *row_addr = (uint64_t *)(ws + pack_ws);
    int32_t *words = (int32_t *)(ws + pack_ws + round256((size_t)W * (size_t)E * 8));
    a.S = S;
    a.expert_counts = expert_counts;
    a.hist = (int32_t *)ws;
    a.row_addr = row_addr;
    a.plan_bits = words;
    a.status = status;
    a.R = row_bytes;
    a.T = T;
    a.k = k;
    a.Q = T * k;
    a.E = E;
    a.W = W;
    launch_pack_sort(a, stream);
    p.counts = expert_counts;
    p.row_addr = row_addr;
    p.block_offsets = block_offsets;
    p.words = words;
    p.status = status;
    p.R = row_bytes;
    p.W = W;
    p.E = E;
    p.layout = layout;
    p.over_bit = A2AV_ST_RECV_OVERFLOW;
    hipLaunchKernelGGL(k_shift_plan, dim3(W), dim3(kPlanThreads), 0, stream, p);
    if (a.Q > 0) launch_scatter<true>(a, aligned, stream);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t moe_unpack_return_workspace_bytes(int W, int E) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0) return 0;
    return 2 * round256((size_t)W * (size_t)E * 8) + 256;
}

A2AV_API int moe_unpack_return(int W, int64_t T, int k, int E, size_t row_bytes,
                               const int64_t *expert_counts, const int32_t *const *ids,
                               const int64_t *const *perm, const void *const *recv,
                               const int64_t *recv_rows, void *const *out, int layout,
                               void *workspace, size_t workspace_bytes, int32_t *status,
                               hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || T < 0 ||
        k < 1 || row_bytes == 0 || !expert_counts || !ids || !perm || !recv || !recv_rows ||
        !out || !status || (layout != 0 && layout != 1))
        return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_unpack_return_workspace_bytes(W, E)) return A2AV_EARG;
    if (T > ((int64_t)1 << 31) / k || (uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / row_bytes)
        return A2AV_EARG;
    ShiftArgs p;
    ReturnArgs c;
    std::memset(&p, 0, sizeof(p));
    std::memset(&c, 0, sizeof(c));
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!ids[r] || !perm[r] || !out[r])) return A2AV_EARG;
        const int64_t rows = recv_rows[r];
        if (rows < 0 || (uint64_t)rows > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
        if (rows > 0 && !recv[r]) return A2AV_EARG;
        p.base[r] = (const unsigned char *)recv[r];
        p.limit[r] = rows;
        c.out[r] = (unsigned char *)out[r];
        c.ids[r] = ids[r];
        c.perm[r] = perm[r];
        aligned = aligned && ((uintptr_t)recv[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    unsigned char *ws = (unsigned char *)workspace;
    const size_t table = round256((size_t)W * (size_t)E * 8);
    uint64_t *row_addr = (uint64_t *)ws;
    int64_t *ystart = (int64_t *)(ws + table);
    int32_t *words = (int32_t *)(ws + 2 * table);
    p.counts = expert_counts;
    p.row_addr = row_addr;
    p.ystart = ystart;
    p.words = words;
    p.status = status;
    p.R = row_bytes;
    p.W = W;
    p.E = E;
    p.layout = layout;
    p.over_bit = A2AV_ST_SEND_OVERRUN;
    p.check_counts = 1;
    c.counts = expert_counts;
    c.row_addr = row_addr;
    c.ystart = ystart;
    c.words = words;
    c.status = status;
    c.R = row_bytes;
    c.Q = T * k;
    c.E = E;
    c.W = W;
    hipLaunchKernelGGL(k_shift_plan, dim3(W), dim3(kPlanThreads), 0, stream, p);
    if (c.Q > 0)
        hipLaunchKernelGGL(k_slot_check, dim3((unsigned)((c.Q + 255) / 256), W), dim3(256), 0,
                           stream, c);
    // at least one wave, so that a verdict of the plan is reported
    uint64_t blocks = ((uint64_t)W * (uint64_t)c.Q + 3) / 4;
    if (blocks < 1) blocks = 1;
    if (blocks > max_grid()) blocks = max_grid();  // the wave loop strides over the rest
    if (aligned)
        hipLaunchKernelGGL((k_moe_gather_home<16, true>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, c);
    else
        hipLaunchKernelGGL((k_moe_gather_home<8, false>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, c);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t moe_combine_return_workspace_bytes(int W, int64_t T, int k, int E) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || T < 0 || k < 1)
        return 0;
    if (T > ((int64_t)1 << 31) / k) return 0;
    return 2 * round256((size_t)W * (size_t)E * 8) + 256 +
           round256((size_t)W * (size_t)(T * k) * 8);
}

A2AV_API int moe_combine_return(int W, int64_t T, int k, int E, int64_t H,
                                const int64_t *expert_counts, const int32_t *const *ids,
                                const int64_t *const *perm, const void *const *recv,
                                const int64_t *recv_rows, const float *const *weights,
                                void *const *out, int layout, void *workspace,
                                size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || T < 0 ||
        k < 1 || H < 1 || !expert_counts || !ids || !perm || !recv || !recv_rows || !weights ||
        !out || !status || (layout != 0 && layout != 1))
        return A2AV_EARG;
    if (T > ((int64_t)1 << 31) / k || (uint64_t)H > (uint64_t)INT64_MAX / 2) return A2AV_EARG;
    const uint64_t row_bytes = 2 * (uint64_t)H;
    if ((uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_combine_return_workspace_bytes(W, T, k, E))
        return A2AV_EARG;
    ShiftArgs p;
    ReturnArgs c;
    CombineArgs m;
    std::memset(&p, 0, sizeof(p));
    std::memset(&c, 0, sizeof(c));
    std::memset(&m, 0, sizeof(m));
    bool aligned = (H % 8) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!ids[r] || !perm[r] || !weights[r] || !out[r])) return A2AV_EARG;
        const int64_t rows = recv_rows[r];
        if (rows < 0 || (uint64_t)rows > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
        if (rows > 0 && !recv[r]) return A2AV_EARG;
        p.base[r] = (const unsigned char *)recv[r];
        p.limit[r] = rows;
        c.ids[r] = ids[r];
        c.perm[r] = perm[r];
        m.w[r] = weights[r];
        m.out[r] = (unsigned char *)out[r];
        aligned = aligned && ((uintptr_t)recv[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    unsigned char *ws = (unsigned char *)workspace;
    const size_t table = round256((size_t)W * (size_t)E * 8);
    uint64_t *row_addr = (uint64_t *)ws;
    int64_t *ystart = (int64_t *)(ws + table);
    int32_t *words = (int32_t *)(ws + 2 * table);
    uint64_t *xaddr = (uint64_t *)(ws + 2 * table + 256);
    p.counts = expert_counts;
    p.row_addr = row_addr;
    p.ystart = ystart;
    p.words = words;
    p.status = status;
    p.R = row_bytes;
    p.W = W;
    p.E = E;
    p.layout = layout;
    p.over_bit = A2AV_ST_SEND_OVERRUN;
    p.check_counts = 1;
    c.counts = expert_counts;
    c.row_addr = row_addr;
    c.ystart = ystart;
    c.xaddr = xaddr;
    c.words = words;
    c.status = status;
    c.R = row_bytes;
    c.Q = T * k;
    c.E = E;
    c.W = W;
    m.xaddr = xaddr;
    m.words = words;
    m.status = status;
    m.T = T;
    m.H = H;
    m.k = k;
    m.W = W;
    hipLaunchKernelGGL(k_shift_plan, dim3(W), dim3(kPlanThreads), 0, stream, p);
    if (c.Q > 0)
        hipLaunchKernelGGL(k_slot_check, dim3((unsigned)((c.Q + 255) / 256), W), dim3(256), 0,
                           stream, c);
    // at least one wave, so that a verdict of the plan is reported; the fast
    // path needs 16-byte vectors and rows under 4 GiB (32-bit lane offsets)
    if (!aligned || row_bytes >= (1ull << 32)) {
        uint64_t blocks = ((uint64_t)W * (uint64_t)T + 3) / 4;
        if (blocks < 1) blocks = 1;
        if (blocks > max_grid()) blocks = max_grid();  // the wave loop strides over the rest
        hipLaunchKernelGGL(k_moe_combine_any<true>, dim3((unsigned)blocks), dim3(256), 0, stream, m);
    } else {
        const uint64_t nchunk = ((uint64_t)H / 8 + kWave - 1) / kWave;
        uint64_t blocks = ((uint64_t)W * (uint64_t)T * nchunk + 3) / 4;
        if (blocks < 1) blocks = 1;
        if (blocks > max_grid()) blocks = max_grid();
        hipLaunchKernelGGL((k_moe_combine<true, true>), dim3((unsigned)blocks), dim3(256),
                           (unsigned)env_long("A2AV_COMBINE_LDS", kCombineHomeLds, 0, 65536),
                           stream, m, nchunk);
    }
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API int moe_unpack(int W, int64_t T, int k, size_t row_bytes, const void *const *back,
                        const int64_t *const *perm, void *const *out, int32_t *status,
                        hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || T < 0 || k < 1 || row_bytes == 0 || !back || !perm || !out ||
        !status)
        return A2AV_EARG;
    if (T > INT64_MAX / k || (uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / row_bytes)
        return A2AV_EARG;
    UnpackArgs a;
    std::memset(&a, 0, sizeof(a));
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!back[r] || !perm[r] || !out[r])) return A2AV_EARG;
        a.back[r] = (const unsigned char *)back[r];
        a.perm[r] = perm[r];
        a.out[r] = (unsigned char *)out[r];
        aligned = aligned && ((uintptr_t)back[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    a.status = status;
    a.R = row_bytes;
    a.Q = T * k;
    a.W = W;
    if (a.Q == 0) return A2AV_OK;
    const int64_t check_blocks = (a.Q + 255) / 256;
    if (check_blocks > INT32_MAX) return A2AV_EARG;
    uint64_t gather_blocks = ((uint64_t)W * (uint64_t)a.Q + 3) / 4;
    if (gather_blocks > max_grid()) gather_blocks = max_grid();  // the wave loop strides over the rest
    hipLaunchKernelGGL(k_perm_check, dim3((unsigned)check_blocks, W), dim3(256), 0, stream, a);
    const int gu = (int)env_long("A2AV_MOE_GATHER_UNROLL", 16, 4, 16);
    if (aligned && gu >= 16)
        hipLaunchKernelGGL((k_moe_gather<16, true>), dim3((unsigned)gather_blocks), dim3(256), 0,
                           stream, a);
    else if (aligned && gu <= 4)
        hipLaunchKernelGGL((k_moe_gather<4, true>), dim3((unsigned)gather_blocks), dim3(256), 0,
                           stream, a);
    else if (aligned)
        hipLaunchKernelGGL((k_moe_gather<8, true>), dim3((unsigned)gather_blocks), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((k_moe_gather<8, false>), dim3((unsigned)gather_blocks), dim3(256), 0,
                           stream, a);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API int moe_combine(int W, int64_t T, int k, int64_t H, const void *const *back,
                         const int64_t *const *perm, const float *const *weights,
                         void *const *out, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || T < 0 || k < 1 || H < 1 || !back || !perm || !weights ||
        !out || !status)
        return A2AV_EARG;
    if (T > INT64_MAX / k || (uint64_t)T * (uint64_t)k > (uint64_t)INT64_MAX / (2 * (uint64_t)H))
        return A2AV_EARG;
    CombineArgs a;
    UnpackArgs c;
    std::memset(&a, 0, sizeof(a));
    std::memset(&c, 0, sizeof(c));
    bool aligned = (H % 8) == 0;
    for (int r = 0; r < W; r++) {
        if (T > 0 && (!back[r] || !perm[r] || !weights[r] || !out[r])) return A2AV_EARG;
        a.back[r] = (const unsigned char *)back[r];
        a.perm[r] = perm[r];
        a.w[r] = weights[r];
        a.out[r] = (unsigned char *)out[r];
        c.perm[r] = perm[r];
        aligned = aligned && ((uintptr_t)back[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    a.status = c.status = status;
    a.T = T;
    a.H = H;
    a.k = k;
    a.W = W;
    c.Q = T * k;
    c.W = W;
    c.R = 1;
    if (T == 0) return A2AV_OK;
    const int64_t check_blocks = (c.Q + 255) / 256;
    if (check_blocks > INT32_MAX) return A2AV_EARG;
    hipLaunchKernelGGL(k_perm_check, dim3((unsigned)check_blocks, W), dim3(256), 0, stream, c);
    // the fast path needs 16-byte vectors and rows under 4 GiB (32-bit lane offsets)
    if (!aligned || (uint64_t)H * 2 >= (1ull << 32)) {
        uint64_t blocks = ((uint64_t)W * (uint64_t)T + 3) / 4;
        if (blocks > max_grid()) blocks = max_grid();  // the wave loop strides over the rest
        hipLaunchKernelGGL(k_moe_combine_any<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    } else {
        const uint64_t nchunk = ((uint64_t)H / 8 + kWave - 1) / kWave;
        uint64_t blocks = ((uint64_t)W * (uint64_t)T * nchunk + 3) / 4;
        if (blocks > max_grid()) blocks = max_grid();  // the wave loop strides over the rest
        // tuning knob: A2AV_COMBINE_STORE_NT (non-temporal stores, 0/1)
        if (env_long("A2AV_COMBINE_STORE_NT", 1, 0, 1))
            hipLaunchKernelGGL((k_moe_combine<true, false>), dim3((unsigned)blocks), dim3(256),
                               (unsigned)env_long("A2AV_COMBINE_LDS", kCombineLds, 0, 65536), stream, a,
                               nchunk);
        else
            hipLaunchKernelGGL((k_moe_combine<false, false>), dim3((unsigned)blocks), dim3(256),
                               (unsigned)env_long("A2AV_COMBINE_LDS", kCombineLds, 0, 65536), stream, a,
                               nchunk);
    }
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}
