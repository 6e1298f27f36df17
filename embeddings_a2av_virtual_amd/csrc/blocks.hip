// blocks.hip — block-permutation copies next to the a2av (gfx950): the
// receive-side expert regroup after the MoE dispatch, the dispatch and the
// regroup as one copy (grouped dispatch), the bucketing of jagged embedding
// keys by owning rank, and the bucketing with both key exchanges in one call.
//
// All of them move whole runs of rows ("blocks"): inside each virtual rank,
// or, with a source rank recorded per block, across ranks. A planning kernel
// writes, per destination rank, the blocks in destination order:
//   dst_start[r][b]  first destination row of block b (exclusive scan, the
//                    rank's total at b = B)
//   src_start[r][b]  first source row of block b
//   bits[r]          the rank's error bits (0 when it passed its checks)
// and k_block_copy moves the bytes. The copy cuts the destination byte space
// of all ranks (rank 0's rows, then rank 1's, ...) into equal pieces, one per
// wave, like the a2av payload kernel; a wave finds the block holding its
// piece with a 64-way search of dst_start (one ballot per level).
//
// Error protocol: a planning kernel never writes the status word (so every
// block of it sees the word as it was when the operation began) and writes
// its bits to the workspace; the copy kernel reads them, one wave ORs them
// into the status word, and no byte moves when any rank failed.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "common.hpp"

namespace a2av {

struct BlockArgs {
    const unsigned char *in[A2AV_MAX_W];
    unsigned char *out[A2AV_MAX_W];
    int64_t in_rows[A2AV_MAX_W];
    int64_t cap[A2AV_MAX_W];
    const int64_t *dst_start;  // [W][B + 1]
    const int64_t *src_start;  // [W][B]
    const int32_t *src_rank;   // [W][B] source rank of each block, or null: the rank itself
    const int32_t *bits;       // [W]
    int32_t *status;
    uint64_t R;
    uint64_t piece;
    int W;
    int B;
    uint32_t Rr[A2AV_MAX_W];   // row bytes per rank (k_block_copy<.., true> only)
};

// Largest i in [0, n) with v[i] <= key, for v non-decreasing with v[0] <= key
// (-1 if v[0] > key, which a valid plan never gives). One ballot per level of
// a 64-way search: two levels cover 4096 entries.
__device__ __forceinline__ int find_last_le(const int64_t *v, int n, uint64_t key, int lane) {
    int lo = 0, len = n;
    while (len > kWave) {
        const int stride = (len + kWave - 1) / kWave;
        const int off = lane * stride;
        const bool ok = off < len && (uint64_t)v[lo + off] <= key;
        const uint64_t m = __ballot(ok);
        if (m == 0) return -1;
        const int h = 63 - __clzll(m);
        lo += h * stride;
        len = stride < len - h * stride ? stride : len - h * stride;
    }
    const uint64_t m = __ballot(lane < len && (uint64_t)v[lo + lane] <= key);
    if (m == 0) return -1;
    return lo + 63 - __clzll(m);
}

// LDS the block copy declares itself: the ranks' rows and row bytes, one
// plan row, the waves' error bits; a multiple of 16 bytes, so that the size
// the launch subtracts from the occupancy cap is the size the kernel is given.
constexpr int kCopyRowMax = kWave - 1;  // plans of up to this many blocks per rank stage a row
struct CopyLds {
    uint64_t rows[A2AV_MAX_W];      // rank r: rows it receives (dst_start[r][B])
    uint64_t row[kCopyRowMax + 1];  // dst_start row of the workgroup's first rank, lane b: entry b
    uint32_t rb[A2AV_MAX_W];        // rank r: row bytes (MIXED)
    int32_t bits[4];                // OR of the planning bits each wave loaded
};
constexpr unsigned kCopyOwnLds = sizeof(CopyLds);
static_assert(kCopyOwnLds % 16 == 0, "LDS rounded to 16 bytes");

// MIXED: every rank has its own row size (Rr), so two exchanges with
// different rows (keys and lengths) run as one launch over 2W ranks.
//
// Before its pieces, the workgroup loads what its waves look up first
// through the scalar cache, in two bursts shared in LDS (a vector load of a
// young wave waits behind the payload traffic older waves keep in flight on
// the CU; a scalar load does not): (1) the status word, and for ranks
// 16k .. 16k + 15 (wave k) the planning bits, the rows each rank receives and
// (MIXED) the row bytes; (2) with at most kCopyRowMax blocks per rank, the
// dst_start row of the rank holding the workgroup's first byte, wave k taking
// entries 16k .. 16k + 16. A piece in that rank searches the row in LDS; any
// other searches the plan in global memory. Every wave reaches both barriers
// before it looks at the status word or the bits.
template <int U, bool ALIGNED, bool MIXED = false>
__global__ __launch_bounds__(256) void k_block_copy(const BlockArgs a) {
    __shared__ CopyLds sh;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t gw = (uint64_t)blockIdx.x * 4 + k;
    const uint64_t TW = (uint64_t)gridDim.x * 4;
    const int W = a.W, B = a.B, B1 = B + 1;
    const const_i64 *dsc = (const const_i64 *)a.dst_start;
    const const_i32 *bic = (const const_i32 *)a.bits;

    const int32_t st0 = status_at_entry(a.status);
    // entries past W repeat rank W - 1 and are not stored
    uint64_t t[16];
    int32_t bb[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int e = 16 * k + i < W ? 16 * k + i : W - 1;
        t[i] = (uint64_t)at_byte(dsc, (uint32_t)(e * B1 + B) * 8u);
        bb[i] = at_byte(bic, (uint32_t)e * 4u);
    }
    uint32_t rr[16];  // MIXED: row bytes of ranks 16k .. 16k + 15 (the array holds 64)
    if constexpr (MIXED) {
#pragma unroll
        for (int i = 0; i < 16; i++) rr[i] = a.Rr[16 * k + i];
        asm volatile("" : A2AV_SREG16_IO(t, 0), A2AV_SREG16_IO(bb, 0), A2AV_SREG16_IO(rr, 0) : "s"(st0));
    } else {
        asm volatile("" : A2AV_SREG16_IO(t, 0), A2AV_SREG16_IO(bb, 0) : "s"(st0));
    }
    int32_t ob = 0;
    uint64_t part = 0;
    uint32_t rpart = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        ob |= 16 * k + i < W ? bb[i] : 0;
        part = writelane_u64(part, t[i], i);
        if constexpr (MIXED) rpart = (uint32_t)amdgcn_writelane((int)rr[i], i, (int)rpart);
    }
    if (lane < 16 && 16 * k + lane < W) sh.rows[16 * k + lane] = part;
    if (MIXED && lane < 16) sh.rb[16 * k + lane] = rpart;
    if (lane == 0) sh.bits[k] = ob;
    __syncthreads();
    // lane r: rank r's rows, row bytes, and bytes
    const uint64_t rows = lane < W ? sh.rows[lane] : 0;
    const uint64_t Rl = MIXED ? (lane < W ? (uint64_t)sh.rb[lane] : 1) : a.R;
    const int32_t bad = sh.bits[0] | sh.bits[1] | sh.bits[2] | sh.bits[3];
    // lane r: bytes of rank r and where they start in the flat space
    const uint64_t bytes = rows * Rl;
    const uint64_t incl = wave_incl_scan_u64(bytes);
    const uint64_t base = incl - bytes;
    const uint64_t total = readlane_u64(incl, kWave - 1);
    const uint64_t piece = a.piece;
    // the rank holding the workgroup's first byte (the same in its four
    // waves: they scan the same rows) and, with few blocks, its plan row
    const bool staged = B <= kCopyRowMax;
    const uint64_t x0 = (uint64_t)blockIdx.x * 4 * piece;
    const uint64_t m0 = __ballot(lane < W && base <= x0);
    const int d0 = __builtin_amdgcn_readfirstlane(m0 ? 63 - (int)__clzll(m0) : 0);
    if (staged) {
        uint64_t u[17];
#pragma unroll
        for (int i = 0; i < 17; i++)
            u[i] = (uint64_t)at_byte(dsc, (uint32_t)(d0 * B1 + (16 * k + i <= B ? 16 * k + i : B)) * 8u);
        asm volatile("" : A2AV_SREG16_IO(u, 0), "+s"(u[16]));
        part = 0;
#pragma unroll
        for (int i = 0; i < 17; i++) part = writelane_u64(part, u[i], i);
        if (lane < 17 && 16 * k + lane <= B) sh.row[16 * k + lane] = part;
        __syncthreads();
    }
    if (st0) return;
    if (bad) {
        if (gw == 0 && lane == 0) atomicOr(a.status, bad);
        return;
    }
    // lane b: entry b of the staged row (b <= B < 64)
    const uint64_t srow = staged && lane <= B ? sh.row[lane] : 0;
    for (uint64_t p = gw; p * piece < total; p += TW) {
        uint64_t x = p * piece;
        uint64_t hi = x + piece < total ? x + piece : total;
        if constexpr (!ALIGNED) {
            // cut where the destination address is 128-byte aligned, so no
            // cache line is split between two waves' partial writes
            x = snap_to_line(x, total, base, lane, W, a.out);
            hi = snap_to_line(hi, total, base, lane, W, a.out);
            if (x >= hi) continue;
        }
        while (x < hi) {
            // last rank starting at or before x: empty ranks share the base of
            // the next one, so the highest match is the one holding x
            const uint64_t md = __ballot(lane < W && base <= x);
            const int d = 63 - __clzll(md);  // md has lane 0 (base 0)
            const uint64_t rbase = readlane_u64(base, d);
            const uint64_t rend = rbase + readlane_u64(bytes, d);
            const uint64_t xr = x - rbase;
            const uint64_t hr = (hi < rend ? hi : rend) - rbase;
            const uint64_t R = MIXED ? readlane_u64(Rl, d) : a.R;
            // d and b are the same in every lane; the block's plan entries
            // (written by the launch before, not during this one) come from
            // the staged row or through the scalar cache
            const int du = __builtin_amdgcn_readfirstlane(d);
            int b;
            uint64_t r0, r1;
            if (staged && du == d0) {
                const uint64_t mb = __ballot(lane < B && srow <= xr / R);
                if (mb == 0) return;  // not a valid plan
                b = __builtin_amdgcn_readfirstlane(63 - (int)__clzll(mb));
                r0 = readlane_u64(srow, b);
                r1 = readlane_u64(srow, b + 1);
            } else {
                const int64_t *ds = a.dst_start + (uint64_t)d * (B + 1);
                b = __builtin_amdgcn_readfirstlane(find_last_le(ds, B, xr / R, lane));
                if (b < 0) return;  // not a valid plan
                const const_i64 *dsu = (const const_i64 *)(a.dst_start + (uint64_t)du * (B + 1));
                r0 = (uint64_t)dsu[b];
                r1 = (uint64_t)dsu[b + 1];
            }
            const uint64_t s0 = (uint64_t)((const const_i64 *)a.src_start)[(uint64_t)du * B + b];
            const int sr = a.src_rank ? ((const const_i32 *)a.src_rank)[(uint64_t)du * B + b] : du;
            const uint64_t e = hr < r1 * R ? hr : r1 * R;
            if (e <= xr || sr < 0 || sr >= W) return;  // not a valid plan
            // a valid plan always passes; the check keeps every access inside
            // the caller's buffers regardless (rows [r0, r1) of the
            // destination and [s0, s0 + r1 - r0) of the source, with no sum
            // that can wrap)
            if (r0 <= r1 && span_fits(r0, r1 - r0, (uint64_t)a.cap[du]) &&
                span_fits(s0, r1 - r0, (uint64_t)a.in_rows[sr])) {
                unsigned char *dst = a.out[du] + xr;
                const unsigned char *src = a.in[sr] + s0 * R + (xr - r0 * R);
                if constexpr (ALIGNED) wave_copy16<U>(dst, src, e - xr, lane);
                else wave_copy_any<U>(dst, src, e - xr, lane);
            }
            x = rbase + e;
        }
    }
}

// ------------------------------------------------------------ expert regroup plan
struct RegroupPlanArgs {
    const int64_t *counts;    // [W][E]
    int64_t *dst_start;       // [W][E + 1]
    int64_t *src_start;       // [W][E]
    int32_t *bits;            // [W]
    int64_t *expert_offsets;  // [W][P + 1]
    const int32_t *status;
    int64_t in_rows[A2AV_MAX_W];
    int64_t cap[A2AV_MAX_W];
    int W;
    int E;
    int direction;  // 0: (source, expert) -> (expert, source); 1: the reverse
};

// Rank d's blocks are the pairs (s, j), s a source rank and j one of the
// P = E / W experts d owns, of counts[s][d*P + j] rows each. Source-major
// order lists them as index s*P + j, expert-major as j*W + s.
__global__ __launch_bounds__(kPlanThreads) void k_regroup_plan(const RegroupPlanArgs a) {
    __shared__ ScanLds lds;
    __shared__ int poisoned;
    const int d = blockIdx.x, tid = threadIdx.x;
    if (tid == 0) poisoned = *a.status != 0;
    __syncthreads();
    if (poisoned) return;
    const int W = a.W, E = a.E, P = E / W;
    const bool to_expert = a.direction == 0;
    int64_t nd[kPlanPer], ns[kPlanPer];  // sizes in destination / source order
    int64_t sd = 0, ss = 0;
    int bad = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int i = tid * kPlanPer + u;
        nd[u] = ns[u] = 0;
        if (i < E) {
            const int sm_s = i / P, sm_j = i - (i / P) * P;  // i read source-major
            const int em_j = i / W, em_s = i - (i / W) * W;  // i read expert-major
            const int64_t c_sm = a.counts[(int64_t)sm_s * E + d * P + sm_j];
            const int64_t c_em = a.counts[(int64_t)em_s * E + d * P + em_j];
            bad |= (int)split_invalid(c_sm);
            nd[u] = to_expert ? c_em : c_sm;
            ns[u] = to_expert ? c_sm : c_em;
        }
        sd += nd[u];
        ss += ns[u];
    }
    if (__syncthreads_or(bad)) {
        if (tid == 0) a.bits[d] = A2AV_ST_BAD_SPLIT;
        return;
    }
    int64_t ed, es, total, total2;
    block_excl_scan2(sd, ss, lds, &ed, &es, &total, &total2);
    int32_t bits = 0;
    if (total > a.in_rows[d]) bits |= A2AV_ST_SEND_OVERRUN;
    if (total > a.cap[d]) bits |= A2AV_ST_RECV_OVERFLOW;
    int64_t *dst = a.dst_start + (int64_t)d * (E + 1);
    int64_t *src = a.src_start + (int64_t)d * E;
    int64_t *eoff = a.expert_offsets + (int64_t)d * (P + 1);
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int i = tid * kPlanPer + u;
        if (i < E) {
            dst[i] = ed;
            // source-order index i is the block (s, j); its destination index
            const int b = to_expert ? (i - (i / P) * P) * W + i / P    // s*P+j -> j*W+s
                                    : (i - (i / W) * W) * P + i / W;   // j*W+s -> s*P+j
            src[b] = es;
            if (bits == 0 && i % W == 0) eoff[i / W] = to_expert ? ed : es;
        }
        ed += nd[u];
        es += ns[u];
    }
    if (tid == 0) {
        dst[E] = total;
        if (bits == 0) eoff[P] = total;
        a.bits[d] = bits;
    }
}

// ------------------------------------------------------------ key bucketing
struct BucketArgs {
    const int32_t *lengths[A2AV_MAX_W];  // [n_tables][batch] per rank
    int64_t n_keys[A2AV_MAX_W];
    int64_t *tk;            // [W][n_tables] keys per table, -1 for a negative length
    int64_t *kdst;          // [W][n_tables + 1] plan of the keys
    int64_t *ksrc;          // [W][n_tables]
    int64_t *ldst;          // [W][n_tables + 1] plan of the lengths
    int64_t *lsrc;          // [W][n_tables]
    int32_t *bits;          // [W] ([2W] when merged)
    int64_t *split_keys;    // [W][W]
    int64_t *split_lengths; // [W][W]
    const int32_t *status;
    int64_t batch;
    int W;
    int n_tables;
    int merged;  // 1: one block copy over 2W ranks moves keys and lengths,
                 // rank r's lengths being rank W + r
};

// One block per (table, rank): the table's key count, or -1 when a length is
// negative.
__global__ __launch_bounds__(256) void k_bucket_sums(const BucketArgs a) {
    __shared__ int64_t part[256 / kWave];
    __shared__ int neg[256 / kWave];
    const int t = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int32_t *L = a.lengths[r] + (int64_t)t * a.batch;
    int64_t s = 0;
    int n = 0;
    if ((a.batch & 3) == 0 && ((uintptr_t)L & 15) == 0 && a.batch > 0) {
        // four lengths per load, eight loads in flight per thread (a batch
        // of 8192: all of the table's); indices past the end load the last
        // vector again and count nothing
        constexpr int kPer = 8;
        static_assert(kPer == 8, "the asm statement below names eight vectors");
        const u32x4 *L4 = (const u32x4 *)L;
        const int64_t n4 = a.batch / 4;
        for (int64_t i0 = tid; i0 < n4; i0 += 256 * kPer) {
            u32x4 v[kPer];
#pragma unroll
            for (int u = 0; u < kPer; u++) {
                const int64_t i = i0 + (int64_t)u * 256;
                v[u] = L4[i < n4 ? i : n4 - 1];
            }
            // every load in flight before the first sum uses one (without
            // this the compiler reused registers and issued the last two
            // after the first results came back)
            asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                         "+v"(v[6]), "+v"(v[7]));
#pragma unroll
            for (int u = 0; u < kPer; u++) {
                if (i0 + (int64_t)u * 256 >= n4) v[u] = u32x4{0, 0, 0, 0};
                s += (int64_t)(int32_t)v[u].x + (int32_t)v[u].y + (int32_t)v[u].z + (int32_t)v[u].w;
                n |= (int32_t)(v[u].x | v[u].y | v[u].z | v[u].w) < 0;
            }
        }
    } else {
        for (int64_t i = tid; i < a.batch; i += 256) {
            const int32_t v = L[i];
            s += v;
            n |= v < 0;
        }
    }
    s = wave_incl_scan(s);
    n = __ballot(n) != 0;
    if ((tid & (kWave - 1)) == kWave - 1) {
        part[tid / kWave] = s;
        neg[tid / kWave] = n;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t tot = 0;
        int ng = 0;
        for (int w = 0; w < 256 / kWave; w++) {
            tot += part[w];
            ng |= neg[w];
        }
        a.tk[(int64_t)r * a.n_tables + t] = ng ? -1 : tot;
    }
}

// One block per rank: table t goes to rank t mod W; destination order is
// owner-major, tables ascending inside an owner, so table t sits at position
// (tables owned by ranks < t mod W) + t / W.
__global__ __launch_bounds__(kPlanThreads) void k_bucket_plan(const BucketArgs a) {
    __shared__ ScanLds lds;
    __shared__ unsigned long long owner_keys[A2AV_MAX_W];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int W = a.W, NT = a.n_tables;
    // the word as the operation found it (no kernel of it has written it
    // yet), loaded beside the key counts (a vector load: a scalar one would
    // hold the counts' address, which waits for every scalar load in
    // flight); it and the counts are judged together at the first barrier
    const int32_t st0 = status_poisoned(a.status);
    if (tid < A2AV_MAX_W) owner_keys[tid] = 0;
    const int64_t *tk = a.tk + (int64_t)r * NT;
    // by position in destination order: the table there, its key count
    int64_t nd[kPlanPer], nt[kPlanPer];
    int64_t sd = 0, st = 0;
    int bad = 0;
    int tpos[kPlanPer];
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int i = tid * kPlanPer + u;
        tpos[u] = 0;
        if (i < NT) {
            // the table at position i: owner o is the largest with first(o) <= i,
            // first(o) = sum over o' < o of ceil((NT - o') / W)
            int o = 0, first = 0;
            while (o + 1 < W) {
                const int cnt = (NT - o + W - 1) / W;
                if (first + cnt > i) break;
                first += cnt;
                o++;
            }
            tpos[u] = o + (i - first) * W;
        }
    }
    if (NT > 0) {
        // every load in flight together: positions past NT read table 0 and
        // count nothing
#pragma unroll
        for (int u = 0; u < kPlanPer; u++) {
            const int i = tid * kPlanPer + u;
            nd[u] = tk[i < NT ? tpos[u] : 0];
            nt[u] = tk[i < NT ? i : 0];  // table order, for the source starts
        }
    }
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        if (NT == 0 || tid * kPlanPer + u >= NT) nd[u] = nt[u] = 0;
        bad |= nt[u] < 0;
        sd += nd[u];
        st += nt[u];
    }
    const int flags = __syncthreads_or((st0 != 0 ? 2 : 0) | bad);
    if (flags & 2) return;
    if (a.merged && tid == 0) a.bits[W + r] = 0;  // the plan's verdict sits in bits[r]
    if (flags & 1) {
        if (tid == 0) a.bits[r] = A2AV_ST_BAD_SPLIT;
        return;
    }
    int64_t ed, et, total, total2;
    block_excl_scan2(sd, st, lds, &ed, &et, &total, &total2);
    const int32_t bits = total > a.n_keys[r] ? A2AV_ST_SEND_OVERRUN : 0;
    int64_t *kdst = a.kdst + (int64_t)r * (NT + 1);
    int64_t *ksrc = a.ksrc + (int64_t)r * NT;
    int64_t *ldst = a.ldst + (int64_t)r * (NT + 1);
    int64_t *lsrc = a.lsrc + (int64_t)r * NT;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int i = tid * kPlanPer + u;
        if (i < NT) {
            kdst[i] = ed;
            ldst[i] = (int64_t)i * a.batch;
            // table i (table order) starts at et in the input; its position
            const int o = i % W;
            int first = 0;
            for (int o2 = 0; o2 < o; o2++) first += (NT - o2 + W - 1) / W;
            const int pos = first + i / W;
            ksrc[pos] = et;
            lsrc[pos] = (int64_t)i * a.batch;
            atomicAdd(&owner_keys[o], (unsigned long long)nt[u]);
        }
        ed += nd[u];
        et += nt[u];
    }
    __syncthreads();
    if (tid == 0) {
        kdst[NT] = total;
        ldst[NT] = (int64_t)NT * a.batch;
        a.bits[r] = bits;
    }
    if (bits == 0 && tid < W) {
        a.split_keys[(int64_t)r * W + tid] = (int64_t)owner_keys[tid];
        a.split_lengths[(int64_t)r * W + tid] = (int64_t)((NT - tid + W - 1) / W) * a.batch;
    }
}

// ------------------------------------------------------------ fused key exchange
// Bucketing and both exchanges in one plan: receiver d's blocks are the pairs
// (source s, i-th table d owns), in that order, B = W * cmax of them per
// receiver (cmax = tables of the owner with the most; blocks past a
// receiver's own count are empty). Each block copies straight from source s's
// table-order keys (or lengths) into d's output, so the bucketed arrays are
// never written.
constexpr int kKxPer = 5;  // blocks per planning thread: up to 5120 per receiver
constexpr int kKxMaxB = A2AV_MAX_TABLES + A2AV_MAX_W;
// the block copy reads plan entries at 32-bit byte offsets
static_assert((uint64_t)A2AV_MAX_W * (kKxMaxB + 1) * 8 < (1ull << 31) &&
                  (uint64_t)A2AV_MAX_W * (A2AV_MAX_EXPERTS + 1) * 8 < (1ull << 31),
              "plan offsets fit 32 bits");

struct KeyxArgs {
    int64_t n_keys[A2AV_MAX_W];
    int64_t key_cap[A2AV_MAX_W];
    int64_t len_cap[A2AV_MAX_W];
    const int64_t *tk;       // [W][NT] keys per (source, table), -1 for a negative length
    int64_t *kdst;           // [W][B + 1] keys plan, per receiver
    int64_t *ksrc;           // [W][B]
    int64_t *ldst;           // [W][B + 1] lengths plan
    int64_t *lsrc;           // [W][B]
    int32_t *rank;           // [W][B] source of each block ([2W][B] when merged)
    int32_t *bits;           // [W] ([2W] when merged)
    int64_t *split_keys;     // [W][W] outputs
    int64_t *split_lengths;  // [W][W]
    int64_t *recv_off;       // [W][W + 1]
    const int32_t *status;
    int64_t batch;
    int W;
    int NT;
    int cmax;
    int B;
    int merged;  // 1: the plan also serves one block copy over 2W ranks,
                 // receiver d's lengths being rank W + d (source s: W + s)
};

__global__ __launch_bounds__(kPlanThreads) void k_keyx_plan(const KeyxArgs a) {
    __shared__ ScanLds lds;
    __shared__ int64_t tst[kKxMaxB];           // start of (s, i) in source s's keys
    __shared__ int64_t tnk[kKxMaxB];           // keys of (s, i)
    __shared__ int64_t sstart[A2AV_MAX_W + 1];  // first key of source s at this receiver
    constexpr int NWV = kPlanThreads / kWave;
    __shared__ int wbits[NWV];                   // the sources' bits, per wave
    __shared__ int32_t st_sh;
    const int d = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int W = a.W, NT = a.NT, cmax = a.cmax, B = a.B;
    // the word as the operation found it (no kernel of it has written it
    // yet), loaded beside the key counts (a vector load: a scalar one would
    // hold the counts' address, which waits for every scalar load in flight);
    // the scan below only writes LDS, so it may run first; the first wave's
    // read decides for the block
    const int32_t st0 = status_poisoned(a.status);
    // every source's table-order scan (one wave per source): where the tables
    // d owns start, and the source's own checks (as its bucketing makes them)
    int wb = 0;
    for (int s = wave; s < W; s += NWV) {
        int64_t run = 0;
        bool neg = false;
        for (int c0 = 0; c0 < NT; c0 += kWave) {
            const int t = c0 + lane;
            int64_t v = t < NT ? a.tk[(int64_t)s * NT + t] : 0;
            neg = neg || __ballot(v < 0) != 0;
            v = v < 0 ? 0 : v;
            const int64_t incl = wave_incl_scan(v);
            if (t < NT && t % W == d) {
                tst[s * cmax + t / W] = run + incl - v;
                tnk[s * cmax + t / W] = v;
            }
            run += (int64_t)readlane_u64((uint64_t)incl, kWave - 1);
        }
        wb |= neg ? A2AV_ST_BAD_SPLIT : run > a.n_keys[s] ? A2AV_ST_SEND_OVERRUN : 0;
    }
    if (lane == 0) wbits[wave] = wb;
    if (tid == 0) st_sh = st0;
    __syncthreads();
    if (st_sh) return;
    if (a.merged && tid == 0) a.bits[W + d] = 0;  // the plan's verdict sits in bits[d]
    int sbits = 0;
#pragma unroll
    for (int w = 0; w < NWV; w++) sbits |= wbits[w];
    if (sbits) {
        if (tid == 0) a.bits[d] = sbits;
        return;
    }
    const int cnt = (NT - d + W - 1) / W;  // tables d owns
    int64_t nk[kKxPer], nl[kKxPer];
    int64_t sk = 0, sl = 0;
#pragma unroll
    for (int u = 0; u < kKxPer; u++) {
        const int b = tid * kKxPer + u;
        nk[u] = nl[u] = 0;
        if (b < B) {
            const int s = b / cmax, i = b - (b / cmax) * cmax;
            if (i < cnt) {
                nk[u] = tnk[s * cmax + i];
                nl[u] = a.batch;
            }
        }
        sk += nk[u];
        sl += nl[u];
    }
    int64_t ek, el, TK, TL;
    block_excl_scan2(sk, sl, lds, &ek, &el, &TK, &TL);
    const int32_t bits = TK > a.key_cap[d] || TL > a.len_cap[d] ? A2AV_ST_RECV_OVERFLOW : 0;
    int64_t *kdst = a.kdst + (int64_t)d * (B + 1);
    int64_t *ldst = a.ldst + (int64_t)d * (B + 1);
#pragma unroll
    for (int u = 0; u < kKxPer; u++) {
        const int b = tid * kKxPer + u;
        if (b < B) {
            const int s = b / cmax, i = b - (b / cmax) * cmax;
            const bool real = i < cnt;
            kdst[b] = ek;
            ldst[b] = el;
            a.ksrc[(int64_t)d * B + b] = real ? tst[s * cmax + i] : 0;
            a.lsrc[(int64_t)d * B + b] = real ? (int64_t)(d + i * W) * a.batch : 0;
            a.rank[(int64_t)d * B + b] = s;
            if (a.merged) a.rank[(int64_t)(W + d) * B + b] = W + s;
            if (i == 0) sstart[s] = ek;
        }
        ek += nk[u];
        el += nl[u];
    }
    if (tid == 0) {
        kdst[B] = TK;
        ldst[B] = TL;
        sstart[W] = TK;
        a.bits[d] = bits;
    }
    __syncthreads();
    if (bits == 0 && tid < W) {
        // with no tables (cmax == 0) every source starts at 0
        const int64_t s0 = cmax > 0 ? sstart[tid] : 0;
        const int64_t s1 = cmax > 0 ? sstart[tid + 1] : 0;
        a.split_keys[(int64_t)tid * W + d] = s1 - s0;
        a.split_lengths[(int64_t)tid * W + d] = (int64_t)cnt * a.batch;
        a.recv_off[(int64_t)d * (W + 1) + tid] = s0;
        if (tid == W - 1) a.recv_off[(int64_t)d * (W + 1) + W] = TK;
    }
}

// ------------------------------------------------------------ grouped MoE dispatch
// The dispatch a2av and the receive-side regroup as one block copy (and the
// inverse). Pack side of rank s: its rows by expert, expert e's counts[s][e]
// rows at Y_s(e) = sum of counts[s][e'] for e' < e. Expert side of rank d:
// owned expert j (e = d*P + j) outer, source s inner. Forward plans run per
// owner d (blocks (j, s) in expert-major order, read from source s's pack
// side); backward plans run per source s (blocks e in pack order, read from
// the owner's expert side).
struct GroupedArgs {
    int64_t in_rows[A2AV_MAX_W];
    int64_t cap[A2AV_MAX_W];
    const int64_t *counts;    // [W][E]
    int64_t *dst;             // [W][E + 1]
    int64_t *src;             // [W][E]
    int32_t *rank;            // [W][E]
    int32_t *bits;            // [W]
    int64_t *expert_offsets;  // [W][P + 1]
    const int32_t *status;
    int W;
    int E;
};

// Every count in range; the caller's workgroup decides together.
__device__ __forceinline__ bool grouped_counts_bad(const GroupedArgs &a) {
    int bad = 0;
    for (int i = threadIdx.x; i < a.W * a.E; i += kPlanThreads) bad |= (int)split_invalid(a.counts[i]);
    return __syncthreads_or(bad) != 0;
}

__global__ __launch_bounds__(kPlanThreads) void k_grouped_plan_fwd(const GroupedArgs a) {
    __shared__ ScanLds lds;
    __shared__ int64_t ypre[A2AV_MAX_EXPERTS];  // Y_s(d*P + j) at j*W + s
    __shared__ int poisoned, sbits;
    const int d = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int NWV = kPlanThreads / kWave;
    const int W = a.W, E = a.E, P = E / W;
    if (tid == 0) {
        poisoned = *a.status != 0;
        sbits = 0;
    }
    __syncthreads();
    if (poisoned) return;
    if (grouped_counts_bad(a)) {
        if (tid == 0) a.bits[d] = A2AV_ST_BAD_SPLIT;
        return;
    }
    // one wave per source: its pack-side prefix over experts, kept for the
    // experts d owns, and its pack total against its rows
    for (int s = wave; s < W; s += NWV) {
        int64_t run = 0;
        for (int c0 = 0; c0 < E; c0 += kWave) {
            const int e = c0 + lane;
            const int64_t v = e < E ? a.counts[(int64_t)s * E + e] : 0;
            const int64_t incl = wave_incl_scan(v);
            if (e >= d * P && e < d * P + P) ypre[(e - d * P) * W + s] = run + incl - v;
            run += (int64_t)readlane_u64((uint64_t)incl, kWave - 1);
        }
        if (lane == 0 && run > a.in_rows[s]) atomicOr(&sbits, A2AV_ST_SEND_OVERRUN);
    }
    __syncthreads();
    int64_t nb[kPlanPer];
    int64_t sum = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int b = tid * kPlanPer + u;  // b = j*W + s
        nb[u] = b < E ? a.counts[(int64_t)(b - (b / W) * W) * E + d * P + b / W] : 0;
        sum += nb[u];
    }
    int64_t ex, ex2, total, total2;
    block_excl_scan2(sum, 0, lds, &ex, &ex2, &total, &total2);
    int64_t *dst = a.dst + (int64_t)d * (E + 1);
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int b = tid * kPlanPer + u;
        if (b < E) {
            dst[b] = ex;
            a.src[(int64_t)d * E + b] = ypre[b];
            a.rank[(int64_t)d * E + b] = b - (b / W) * W;
            if (b % W == 0) a.expert_offsets[(int64_t)d * (P + 1) + b / W] = ex;
        }
        ex += nb[u];
    }
    if (tid == 0) {
        dst[E] = total;
        a.expert_offsets[(int64_t)d * (P + 1) + P] = total;
        a.bits[d] = sbits | (total > a.cap[d] ? A2AV_ST_RECV_OVERFLOW : 0);
    }
}

__global__ __launch_bounds__(kPlanThreads) void k_grouped_plan_bwd(const GroupedArgs a) {
    __shared__ ScanLds lds;
    __shared__ int64_t gpre[A2AV_MAX_EXPERTS + 1];  // exclusive scan of column sums over e
    __shared__ int poisoned, sbits;
    const int s = blockIdx.x, tid = threadIdx.x;
    const int W = a.W, E = a.E, P = E / W;
    if (tid == 0) {
        poisoned = *a.status != 0;
        sbits = 0;
    }
    __syncthreads();
    if (poisoned) return;
    if (grouped_counts_bad(a)) {
        if (tid == 0) a.bits[s] = A2AV_ST_BAD_SPLIT;
        return;
    }
    // per expert: the column sum (rows at its owner) and the rows of the
    // sources before s; per source s: its own counts (pack order)
    int64_t col[kPlanPer], before[kPlanPer], mine[kPlanPer];
    int64_t scol = 0, smine = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int e = tid * kPlanPer + u;
        col[u] = before[u] = mine[u] = 0;
        if (e < E) {
            for (int s2 = 0; s2 < W; s2++) {
                const int64_t c = a.counts[(int64_t)s2 * E + e];
                col[u] += c;
                if (s2 < s) before[u] += c;
            }
            mine[u] = a.counts[(int64_t)s * E + e];
        }
        scol += col[u];
        smine += mine[u];
    }
    int64_t gx, yx, gtot, ytot;
    block_excl_scan2(scol, smine, lds, &gx, &yx, &gtot, &ytot);
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int e = tid * kPlanPer + u;
        if (e < E) gpre[e] = gx;
        gx += col[u];
    }
    if (tid == 0) gpre[E] = gtot;
    __syncthreads();
    int64_t *dst = a.dst + (int64_t)s * (E + 1);
#pragma unroll
    for (int u = 0; u < kPlanPer; u++) {
        const int e = tid * kPlanPer + u;
        if (e < E) {
            const int d = e / P;
            const int64_t at_owner = gpre[e] - gpre[d * P];  // expert_offsets[d][e - d*P]
            dst[e] = yx;
            a.src[(int64_t)s * E + e] = at_owner + before[u];
            a.rank[(int64_t)s * E + e] = d;
            if (s == 0) a.expert_offsets[(int64_t)d * (P + 1) + (e - d * P)] = at_owner;
        }
        yx += mine[u];
    }
    if (tid < W) {
        const int64_t owner_total = gpre[(tid + 1) * P] - gpre[tid * P];
        if (s == 0) a.expert_offsets[(int64_t)tid * (P + 1) + P] = owner_total;
        if (owner_total > a.in_rows[tid]) atomicOr(&sbits, A2AV_ST_SEND_OVERRUN);
    }
    __syncthreads();
    if (tid == 0) {
        dst[E] = ytot;
        a.bits[s] = sbits | (ytot > a.cap[s] ? A2AV_ST_RECV_OVERFLOW : 0);
    }
}

// ------------------------------------------------------------ host side
// Pieces of the block copy. From 64 MiB of traffic up: 4 KiB pieces with 4
// loads in flight per lane, and with 16-byte rows at most a few workgroups per
// CU (32 KiB of LDS per workgroup that the kernel does not use), as for the
// a2av: dispatch workload regroup 2614 -> 2552 us, grouped dispatch 2579 ->
// 2545 us; key workload (8-byte rows, no cap: with it they were slower) fused
// exchange 108.4 -> 106.8 us. Below that, 8 KiB pieces with 8 loads in flight
// (16 with 32 KiB pieces above 512 MiB).
static void piece_policy(uint64_t bmax, bool aligned, int *unroll, uint64_t *piece,
                         unsigned *lds) {
    if (bmax >= (64ull << 20)) {
        *unroll = 4;
        *piece = 4096;
        *lds = aligned ? 32768u : 0u;
        return;
    }
    const bool small = bmax <= (512ull << 20);
    *unroll = small ? 8 : 16;
    *piece = small ? 8192 : 32768;
    *lds = 0;
}

static int copy_grid(uint64_t bmax, uint64_t piece) {
    uint64_t g = (bmax + piece * 4 - 1) / (piece * 4);  // 4 waves per block
    if (g < 1) g = 1;  // one wave always runs, to report the planning bits
    if (g > max_grid()) g = max_grid();  // the piece loop strides over the rest
    return (int)g;
}

// Launch k_block_copy; bmax bounds the bytes any rank can move.
static void launch_block_copy(const BlockArgs &a, uint64_t bmax, bool aligned, hipStream_t st) {
    int unroll;
    uint64_t piece;
    unsigned lds;
    piece_policy(bmax, aligned, &unroll, &piece, &lds);
    // the kernel's own LDS counts against the occupancy cap
    if (lds > kCopyOwnLds) lds -= kCopyOwnLds;
    BlockArgs b = a;
    b.piece = piece;
    const int grid = copy_grid(bmax, piece);
    if (unroll == 16) {
        if (aligned) hipLaunchKernelGGL((k_block_copy<16, true>), dim3(grid), dim3(256), lds, st, b);
        else hipLaunchKernelGGL((k_block_copy<16, false>), dim3(grid), dim3(256), lds, st, b);
    } else if (unroll == 4) {
        if (aligned) hipLaunchKernelGGL((k_block_copy<4, true>), dim3(grid), dim3(256), lds, st, b);
        else hipLaunchKernelGGL((k_block_copy<4, false>), dim3(grid), dim3(256), lds, st, b);
    } else {
        if (aligned) hipLaunchKernelGGL((k_block_copy<8, true>), dim3(grid), dim3(256), lds, st, b);
        else hipLaunchKernelGGL((k_block_copy<8, false>), dim3(grid), dim3(256), lds, st, b);
    }
}

// The same with a row size per rank (a.Rr), any alignment.
static void launch_block_copy_mixed(const BlockArgs &a, uint64_t bmax, hipStream_t st) {
    int unroll;
    uint64_t piece;
    unsigned lds;
    piece_policy(bmax, false, &unroll, &piece, &lds);
    if (lds > kCopyOwnLds) lds -= kCopyOwnLds;
    BlockArgs b = a;
    b.piece = piece;
    const int grid = copy_grid(bmax, piece);
    if (unroll == 16) hipLaunchKernelGGL((k_block_copy<16, false, true>), dim3(grid), dim3(256), lds, st, b);
    else if (unroll == 4) hipLaunchKernelGGL((k_block_copy<4, false, true>), dim3(grid), dim3(256), lds, st, b);
    else hipLaunchKernelGGL((k_block_copy<8, false, true>), dim3(grid), dim3(256), lds, st, b);
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace a2av

using namespace a2av;

A2AV_API size_t moe_regroup_workspace_bytes(int W, int E) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0) return 0;
    return round256((size_t)W * (2 * (size_t)E + 1) * 8) + round256((size_t)W * 4);
}

A2AV_API int moe_regroup(int W, int E, size_t row_bytes, const int64_t *counts,
                         const void *const *in, const int64_t *in_rows, void *const *out,
                         const int64_t *out_cap_rows, int64_t *expert_offsets, int direction,
                         void *workspace, size_t workspace_bytes, int32_t *status,
                         hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || row_bytes == 0 ||
        !counts || !in || !in_rows || !out || !out_cap_rows || !expert_offsets || !status ||
        (direction != 0 && direction != 1))
        return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_regroup_workspace_bytes(W, E)) return A2AV_EARG;
    BlockArgs c;
    RegroupPlanArgs p;
    std::memset(&c, 0, sizeof(c));
    std::memset(&p, 0, sizeof(p));
    uint64_t bmax = 0, cap_bytes = 0;
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (in_rows[r] < 0 || out_cap_rows[r] < 0) return A2AV_EARG;
        if ((uint64_t)in_rows[r] > (uint64_t)INT64_MAX / row_bytes ||
            (uint64_t)out_cap_rows[r] > (uint64_t)INT64_MAX / row_bytes)
            return A2AV_EARG;
        if ((in_rows[r] > 0 && !in[r]) || (out_cap_rows[r] > 0 && !out[r])) return A2AV_EARG;
        c.in[r] = (const unsigned char *)in[r];
        c.out[r] = (unsigned char *)out[r];
        c.in_rows[r] = p.in_rows[r] = in_rows[r];
        c.cap[r] = p.cap[r] = out_cap_rows[r];
        const int64_t m = in_rows[r] < out_cap_rows[r] ? in_rows[r] : out_cap_rows[r];
        bmax += (uint64_t)m * row_bytes;
        cap_bytes += (uint64_t)out_cap_rows[r] * row_bytes;
        if (cap_bytes > ((uint64_t)1 << 62)) return A2AV_EARG;
        aligned = aligned && ((uintptr_t)in[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    unsigned char *ws = (unsigned char *)workspace;
    int64_t *dst = (int64_t *)ws;
    int64_t *src = dst + (size_t)W * (E + 1);
    int32_t *bits = (int32_t *)(ws + round256((size_t)W * (2 * (size_t)E + 1) * 8));
    p.counts = counts;
    p.dst_start = dst;
    p.src_start = src;
    p.bits = bits;
    p.expert_offsets = expert_offsets;
    p.status = status;
    p.W = W;
    p.E = E;
    p.direction = direction;
    hipLaunchKernelGGL(k_regroup_plan, dim3(W), dim3(kPlanThreads), 0, stream, p);
    c.dst_start = dst;
    c.src_start = src;
    c.bits = bits;
    c.status = status;
    c.R = row_bytes;
    c.W = W;
    c.B = E;
    launch_block_copy(c, bmax, aligned, stream);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t keys_bucketize_workspace_bytes(int W, int n_tables) {
    if (W < 1 || W > A2AV_MAX_W || n_tables < 0 || n_tables > A2AV_MAX_TABLES) return 0;
    const size_t nt = (size_t)n_tables;
    return round256((size_t)W * (5 * nt + 2) * 8) + round256(2 * (size_t)W * 4);
}

A2AV_API int keys_bucketize(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                            const int64_t *const *keys, const int64_t *n_keys,
                            int32_t *const *lengths_out, int64_t *const *keys_out,
                            int64_t *split_keys, int64_t *split_lengths, void *workspace,
                            size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || n_tables < 0 || n_tables > A2AV_MAX_TABLES || batch < 0 ||
        !lengths || !keys || !n_keys || !lengths_out || !keys_out || !split_keys ||
        !split_lengths || !status)
        return A2AV_EARG;
    if (!workspace || workspace_bytes < keys_bucketize_workspace_bytes(W, n_tables)) return A2AV_EARG;
    if (n_tables > 0 && batch > ((int64_t)1 << 40) / n_tables) return A2AV_EARG;
    const int64_t nl = (int64_t)n_tables * batch;
    BucketArgs b;
    BlockArgs ck, cl;
    std::memset(&b, 0, sizeof(b));
    std::memset(&ck, 0, sizeof(ck));
    std::memset(&cl, 0, sizeof(cl));
    uint64_t kmax = 0;
    // the 16-byte path needs every block edge on a 16-byte boundary: never
    // true for 8-byte keys in general, true for the lengths when batch % 4 == 0
    const bool kal = false;
    bool lal = (batch % 4) == 0;
    for (int r = 0; r < W; r++) {
        if (n_keys[r] < 0 || n_keys[r] > ((int64_t)1 << 59)) return A2AV_EARG;
        if (nl > 0 && (!lengths[r] || !lengths_out[r])) return A2AV_EARG;
        if (n_keys[r] > 0 && (!keys[r] || !keys_out[r])) return A2AV_EARG;
        b.lengths[r] = lengths[r];
        b.n_keys[r] = n_keys[r];
        ck.in[r] = (const unsigned char *)keys[r];
        ck.out[r] = (unsigned char *)keys_out[r];
        ck.in_rows[r] = ck.cap[r] = n_keys[r];
        cl.in[r] = (const unsigned char *)lengths[r];
        cl.out[r] = (unsigned char *)lengths_out[r];
        cl.in_rows[r] = cl.cap[r] = nl;
        kmax += (uint64_t)n_keys[r] * 8;
        lal = lal && ((uintptr_t)lengths[r] % 16 == 0) && ((uintptr_t)lengths_out[r] % 16 == 0);
    }
    // workspace: tk | kdst | ldst | ksrc | lsrc | bits [2W]. The two plans sit
    // back to back, so that with 2W ranks at most one block copy moves both.
    const size_t nt = (size_t)n_tables;
    const bool merged = 2 * W <= A2AV_MAX_W;
    int64_t *ws = (int64_t *)workspace;
    b.tk = ws;
    b.kdst = b.tk + (size_t)W * nt;
    b.ldst = b.kdst + (size_t)W * (nt + 1);
    b.ksrc = b.ldst + (size_t)W * (nt + 1);
    b.lsrc = b.ksrc + (size_t)W * nt;
    b.bits = (int32_t *)((unsigned char *)workspace + round256((size_t)W * (5 * nt + 2) * 8));
    b.merged = merged ? 1 : 0;
    b.split_keys = split_keys;
    b.split_lengths = split_lengths;
    b.status = status;
    b.batch = batch;
    b.W = W;
    b.n_tables = n_tables;
    if (n_tables > 0)
        hipLaunchKernelGGL(k_bucket_sums, dim3(n_tables, W), dim3(256), 0, stream, b);
    hipLaunchKernelGGL(k_bucket_plan, dim3(W), dim3(kPlanThreads), 0, stream, b);
    ck.dst_start = b.kdst;
    ck.src_start = b.ksrc;
    ck.bits = b.bits;
    ck.status = status;
    ck.R = 8;
    ck.W = W;
    ck.B = n_tables;
    cl.dst_start = b.ldst;
    cl.src_start = b.lsrc;
    cl.bits = b.bits;
    cl.status = status;
    cl.R = 4;
    cl.W = W;
    cl.B = n_tables;
    if (merged) {
        // one launch: ranks 0..W-1 move keys (8-byte rows), ranks W..2W-1
        // lengths (4-byte rows); it also reports the planning bits
        BlockArgs c = ck;
        c.W = 2 * W;
        for (int r = 0; r < W; r++) {
            c.in[W + r] = cl.in[r];
            c.out[W + r] = cl.out[r];
            c.in_rows[W + r] = cl.in_rows[r];
            c.cap[W + r] = cl.cap[r];
            c.Rr[r] = 8;
            c.Rr[W + r] = 4;
        }
        launch_block_copy_mixed(c, kmax + (uint64_t)W * (uint64_t)nl * 4, stream);
    } else if (n_tables > 0) {
        launch_block_copy(ck, kmax, kal, stream);
        launch_block_copy(cl, (uint64_t)W * (uint64_t)nl * 4, lal, stream);
    } else {
        // no tables: nothing to move, but the planning bits still go out
        launch_block_copy(ck, 0, kal, stream);
    }
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t keys_exchange_workspace_bytes(int W, int n_tables) {
    if (W < 1 || W > A2AV_MAX_W || n_tables < 0 || n_tables > A2AV_MAX_TABLES) return 0;
    const size_t cmax = ((size_t)n_tables + W - 1) / W;
    const size_t B = (size_t)W * cmax;
    const size_t i64s = (size_t)W * n_tables + 4 * (size_t)W * B + 2 * (size_t)W;
    return round256(i64s * 8) + round256(2 * (size_t)W * B * 4) + round256(2 * (size_t)W * 4);
}

// ------------------------------------------------------------ fixed scratch
// The scratch of keys_exchange_noalloc: one array in the library's device
// code, which every GPU the library runs on holds a copy of until the process
// ends, so a call allocates nothing. In host code `scratch` names a host-side
// stand-in, not a device address: host code never passes it to a kernel or a
// copy, only the address hipGetSymbolAddress gives on the stream's GPU,
// looked up once per GPU with that GPU current and kept.
static __device__ __align__(256) unsigned char scratch[A2AV_NOALLOC_SCRATCH_BYTES];

namespace a2av {

constexpr int kMaxDevices = 256;

static void *noalloc_scratch(hipStream_t stream) {
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int dev = 0;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

// The body of keys_exchange on a workspace of at least
// keys_exchange_workspace_bytes(W, n_tables) bytes, which the callers check;
// a null workspace means the fixed scratch of the stream's GPU, looked up
// once every argument has passed.
static int keys_exchange_run(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                             const int64_t *const *keys, const int64_t *n_keys,
                             int32_t *const *lengths_out, const int64_t *lengths_cap,
                             int64_t *const *keys_out, const int64_t *keys_cap,
                             int64_t *split_keys, int64_t *split_lengths, int64_t *recv_off_keys,
                             void *workspace, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || n_tables < 0 || n_tables > A2AV_MAX_TABLES || batch < 0 ||
        !lengths || !keys || !n_keys || !lengths_out || !lengths_cap || !keys_out || !keys_cap ||
        !split_keys || !split_lengths || !recv_off_keys || !status)
        return A2AV_EARG;
    if (n_tables > 0 && batch > ((int64_t)1 << 40) / n_tables) return A2AV_EARG;
    const int64_t nl = (int64_t)n_tables * batch;
    const int cmax = (n_tables + W - 1) / W;
    const int B = W * cmax;
    BucketArgs b;
    KeyxArgs x;
    BlockArgs ck, cl;
    std::memset(&b, 0, sizeof(b));
    std::memset(&x, 0, sizeof(x));
    std::memset(&ck, 0, sizeof(ck));
    std::memset(&cl, 0, sizeof(cl));
    uint64_t kin = 0, kout = 0, lout = 0;
    bool lal = (batch % 4) == 0;  // 16-byte path: every block edge on a 16-byte boundary
    for (int r = 0; r < W; r++) {
        if (n_keys[r] < 0 || n_keys[r] > ((int64_t)1 << 59) || keys_cap[r] < 0 ||
            keys_cap[r] > ((int64_t)1 << 59) || lengths_cap[r] < 0 ||
            lengths_cap[r] > ((int64_t)1 << 59))
            return A2AV_EARG;
        if (nl > 0 && !lengths[r]) return A2AV_EARG;
        if (n_keys[r] > 0 && !keys[r]) return A2AV_EARG;
        if ((keys_cap[r] > 0 && !keys_out[r]) || (lengths_cap[r] > 0 && !lengths_out[r]))
            return A2AV_EARG;
        b.lengths[r] = lengths[r];
        x.n_keys[r] = n_keys[r];
        x.key_cap[r] = keys_cap[r];
        x.len_cap[r] = lengths_cap[r];
        ck.in[r] = (const unsigned char *)keys[r];
        ck.out[r] = (unsigned char *)keys_out[r];
        ck.in_rows[r] = n_keys[r];
        ck.cap[r] = keys_cap[r];
        cl.in[r] = (const unsigned char *)lengths[r];
        cl.out[r] = (unsigned char *)lengths_out[r];
        cl.in_rows[r] = nl;
        cl.cap[r] = lengths_cap[r];
        kin += (uint64_t)n_keys[r];
        kout += (uint64_t)keys_cap[r];
        lout += (uint64_t)lengths_cap[r];
        lal = lal && ((uintptr_t)lengths[r] % 16 == 0) && ((uintptr_t)lengths_out[r] % 16 == 0);
    }
    if (workspace == nullptr) {
        workspace = noalloc_scratch(stream);
        if (workspace == nullptr) return A2AV_EHIP;
    }
    // workspace: tk | kdst | ldst | ksrc | lsrc | src rank [2W][B] | bits [2W].
    // The keys and lengths plans sit back to back, so that with 2W ranks at
    // most one block copy moves both: receiver d's lengths are rank W + d.
    int64_t *ws = (int64_t *)workspace;
    const size_t nt = (size_t)n_tables, BB = (size_t)B;
    int64_t *tk = ws;
    int64_t *kdst = tk + (size_t)W * nt;
    int64_t *ldst = kdst + (size_t)W * (BB + 1);
    int64_t *ksrc = ldst + (size_t)W * (BB + 1);
    int64_t *lsrc = ksrc + (size_t)W * BB;
    const size_t i64s = (size_t)W * nt + 4 * (size_t)W * BB + 2 * (size_t)W;
    int32_t *rank = (int32_t *)((unsigned char *)workspace + round256(i64s * 8));
    int32_t *bits = (int32_t *)((unsigned char *)rank + round256(2 * (size_t)W * BB * 4));
    const bool merged = 2 * W <= A2AV_MAX_W;
    b.tk = tk;
    b.batch = batch;
    b.W = W;
    b.n_tables = n_tables;
    x.tk = tk;
    x.kdst = kdst;
    x.ksrc = ksrc;
    x.ldst = ldst;
    x.lsrc = lsrc;
    x.rank = rank;
    x.bits = bits;
    x.split_keys = split_keys;
    x.split_lengths = split_lengths;
    x.recv_off = recv_off_keys;
    x.status = status;
    x.batch = batch;
    x.W = W;
    x.NT = n_tables;
    x.cmax = cmax;
    x.B = B;
    x.merged = merged ? 1 : 0;
    if (n_tables > 0)
        hipLaunchKernelGGL(k_bucket_sums, dim3(n_tables, W), dim3(256), 0, stream, b);
    hipLaunchKernelGGL(k_keyx_plan, dim3(W), dim3(kPlanThreads), 0, stream, x);
    ck.dst_start = kdst;
    ck.src_start = ksrc;
    ck.src_rank = rank;
    ck.bits = bits;
    ck.status = status;
    ck.R = 8;
    ck.W = W;
    ck.B = B;
    cl.dst_start = ldst;
    cl.src_start = lsrc;
    cl.src_rank = rank;
    cl.bits = bits;
    cl.status = status;
    cl.R = 4;
    cl.W = W;
    cl.B = B;
    const uint64_t kmax = (kin < kout ? kin : kout) * 8;
    const uint64_t lin = (uint64_t)W * (uint64_t)nl;
    const uint64_t lmax = (lin < lout ? lin : lout) * 4;
    if (merged) {
        // one launch: ranks 0..W-1 move keys (8-byte rows), ranks W..2W-1
        // lengths (4-byte rows); it also reports the planning bits
        BlockArgs c = ck;
        c.W = 2 * W;
        for (int r = 0; r < W; r++) {
            c.in[W + r] = cl.in[r];
            c.out[W + r] = cl.out[r];
            c.in_rows[W + r] = cl.in_rows[r];
            c.cap[W + r] = cl.cap[r];
            c.Rr[r] = 8;
            c.Rr[W + r] = 4;
        }
        launch_block_copy_mixed(c, kmax + lmax, stream);
    } else {
        launch_block_copy(ck, kmax, false, stream);  // also reports the planning bits
        if (lmax > 0) launch_block_copy(cl, lmax, lal, stream);
    }
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

}  // namespace a2av

A2AV_API int keys_exchange(int W, int n_tables, int64_t batch, const int32_t *const *lengths,
                           const int64_t *const *keys, const int64_t *n_keys,
                           int32_t *const *lengths_out, const int64_t *lengths_cap,
                           int64_t *const *keys_out, const int64_t *keys_cap, int64_t *split_keys,
                           int64_t *split_lengths, int64_t *recv_off_keys, void *workspace,
                           size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    const size_t need = keys_exchange_workspace_bytes(W, n_tables);
    if (need == 0 || !workspace || workspace_bytes < need) return A2AV_EARG;
    return keys_exchange_run(W, n_tables, batch, lengths, keys, n_keys, lengths_out, lengths_cap,
                             keys_out, keys_cap, split_keys, split_lengths, recv_off_keys,
                             workspace, status, stream);
}

A2AV_API int keys_exchange_noalloc(int W, int n_tables, int64_t batch,
                                   const int32_t *const *lengths, const int64_t *const *keys,
                                   const int64_t *n_keys, int32_t *const *lengths_out,
                                   const int64_t *lengths_cap, int64_t *const *keys_out,
                                   const int64_t *keys_cap, int64_t *split_keys,
                                   int64_t *split_lengths, int64_t *recv_off_keys,
                                   int32_t *status, hipStream_t stream) {
    const size_t need = keys_exchange_workspace_bytes(W, n_tables);
    if (need == 0 || need > A2AV_NOALLOC_SCRATCH_BYTES) return A2AV_EARG;
    return keys_exchange_run(W, n_tables, batch, lengths, keys, n_keys, lengths_out, lengths_cap,
                             keys_out, keys_cap, split_keys, split_lengths, recv_off_keys,
                             nullptr, status, stream);
}

A2AV_API size_t moe_dispatch_grouped_workspace_bytes(int W, int E) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0) return 0;
    return round256((size_t)W * (2 * (size_t)E + 1) * 8) + round256((size_t)W * E * 4) +
           round256((size_t)W * 4);
}

A2AV_API int moe_dispatch_grouped(int W, int E, size_t row_bytes, const int64_t *counts,
                                  const void *const *in, const int64_t *in_rows,
                                  void *const *out, const int64_t *out_cap_rows,
                                  int64_t *expert_offsets, int direction, void *workspace,
                                  size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || row_bytes == 0 ||
        !counts || !in || !in_rows || !out || !out_cap_rows || !expert_offsets || !status ||
        (direction != 0 && direction != 1))
        return A2AV_EARG;
    if (!workspace || workspace_bytes < moe_dispatch_grouped_workspace_bytes(W, E)) return A2AV_EARG;
    GroupedArgs g;
    BlockArgs c;
    std::memset(&g, 0, sizeof(g));
    std::memset(&c, 0, sizeof(c));
    uint64_t in_total = 0, cap_total = 0;
    bool aligned = (row_bytes % 16) == 0;
    for (int r = 0; r < W; r++) {
        if (in_rows[r] < 0 || out_cap_rows[r] < 0) return A2AV_EARG;
        if ((uint64_t)in_rows[r] > (uint64_t)INT64_MAX / row_bytes ||
            (uint64_t)out_cap_rows[r] > (uint64_t)INT64_MAX / row_bytes)
            return A2AV_EARG;
        if ((in_rows[r] > 0 && !in[r]) || (out_cap_rows[r] > 0 && !out[r])) return A2AV_EARG;
        g.in_rows[r] = c.in_rows[r] = in_rows[r];
        g.cap[r] = c.cap[r] = out_cap_rows[r];
        c.in[r] = (const unsigned char *)in[r];
        c.out[r] = (unsigned char *)out[r];
        in_total += (uint64_t)in_rows[r];
        cap_total += (uint64_t)out_cap_rows[r];
        if (cap_total * row_bytes > ((uint64_t)1 << 62)) return A2AV_EARG;
        aligned = aligned && ((uintptr_t)in[r] % 16 == 0) && ((uintptr_t)out[r] % 16 == 0);
    }
    unsigned char *ws = (unsigned char *)workspace;
    int64_t *dst = (int64_t *)ws;
    int64_t *src = dst + (size_t)W * (E + 1);
    int32_t *rank = (int32_t *)(ws + round256((size_t)W * (2 * (size_t)E + 1) * 8));
    int32_t *bits = (int32_t *)((unsigned char *)rank + round256((size_t)W * E * 4));
    g.counts = counts;
    g.dst = dst;
    g.src = src;
    g.rank = rank;
    g.bits = bits;
    g.expert_offsets = expert_offsets;
    g.status = status;
    g.W = W;
    g.E = E;
    if (direction == 0)
        hipLaunchKernelGGL(k_grouped_plan_fwd, dim3(W), dim3(kPlanThreads), 0, stream, g);
    else
        hipLaunchKernelGGL(k_grouped_plan_bwd, dim3(W), dim3(kPlanThreads), 0, stream, g);
    c.dst_start = dst;
    c.src_start = src;
    c.src_rank = rank;
    c.bits = bits;
    c.status = status;
    c.R = row_bytes;
    c.W = W;
    c.B = E;
    const uint64_t bmax = (in_total < cap_total ? in_total : cap_total) * row_bytes;
    launch_block_copy(c, bmax, aligned, stream);
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

A2AV_API size_t moe_combine_grouped_workspace_bytes(int W, int64_t T, int k, int E) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || T < 0 || k < 1)
        return 0;
    if (T > ((int64_t)1 << 31) / k) return 0;
    const size_t P = (size_t)E / W;
    return round256((size_t)W * (2 * (size_t)E + 1) * 8) + round256((size_t)W * E * 4) +
           round256((size_t)W * 4) + round256((size_t)W * (P + 1) * 8) + 256 +
           round256((size_t)W * (size_t)(T * k) * 8);
}

A2AV_API int moe_combine_grouped(int W, int64_t T, int k, int E, int64_t H, const int64_t *counts,
                                 const int32_t *const *ids, const int64_t *const *perm,
                                 const void *const *expert_side, const int64_t *exp_rows,
                                 const float *const *weights, void *const *out, void *workspace,
                                 size_t workspace_bytes, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || E < 1 || E > A2AV_MAX_EXPERTS || E % W != 0 || T < 0 || k < 1 ||
        H < 1 || !counts || !ids || !perm || !expert_side || !exp_rows || !weights || !out ||
        !status)
        return A2AV_EARG;
    const size_t need = moe_combine_grouped_workspace_bytes(W, T, k, E);
    if (need == 0 || !workspace || workspace_bytes < need) return A2AV_EARG;
    if ((uint64_t)H * 2 >= (1ull << 32)) return A2AV_EARG;  // 32-bit lane offsets in a row
    // the expert side is moe_pack_dispatch's layout 1: the combine read at the
    // owners in that order (its workspace never exceeds this one's)
    return moe_combine_return(W, T, k, E, H, counts, ids, perm, expert_side, exp_rows, weights,
                              out, 1, workspace, workspace_bytes, status, stream);
}
