// a2av.hip — device-split all-to-all-v over W virtual ranks in one GPU's HBM
// (gfx950): splits exchange, offset scans and the payload copy.
//
// The operation is the one the page "[a2av] Improve tuning for 4 GPUs" times
// in its "Problem" section (nvshmem_all_to_all_vdev), read as all-to-all-v
// with device-held counts. That page's "Change" section keeps the thread-block
// count fixed when the peer count drops and moves blocks into the
// data-parallel dimension; the payload kernel here goes one step further and
// drops the peer dimension from the grid altogether: the destination byte
// space of all ranks is cut into equal contiguous pieces, one per workgroup.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.hpp"
#include "wave_walk.h"

namespace a2av {

// ====================================================================== host helpers
int device_cu_count(hipStream_t stream) {
    static std::mutex mu;
    static int cache[256] = {0};
    int dev = 0;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 256 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev >= 0 && dev < 256) cache[dev] = n;
    return n;
}

long env_long(const char *name, long dflt, long lo, long hi) {
    const char *v = std::getenv(name);
    if (v == nullptr || *v == 0) return dflt;
    char *end = nullptr;
    long x = std::strtol(v, &end, 0);
    if (end == v || x < lo || x > hi) return dflt;
    return x;
}

// Largest grid, in workgroups, of the kernels whose waves loop over their
// work (the loops stride over what the grid does not cover). A2AV_MAX_GRID
// lowers it, so that small inputs run the loops' later passes too.
unsigned max_grid() { return (unsigned)env_long("A2AV_MAX_GRID", 1L << 22, 1, 1L << 22); }

// ====================================================================== exchange
// One block. The status word comes through the scalar cache (this launch's
// one block is its only writer) and S is loaded by every thread before
// anything waits, so the word and the matrix take one memory round trip.
__global__ __launch_bounds__(256) void k_exchange(int W, const int64_t *__restrict__ S,
                                                  int64_t *__restrict__ O, int32_t *status) {
    constexpr int kPer = (A2AV_MAX_W * A2AV_MAX_W + 255) / 256;  // entries per thread at most
    const int n = W * W;
    const int32_t st0 = status_at_entry(status);
    int64_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * 256;
        v[k] = i < n ? S[i] : 0;
    }
    if (st0) return;
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kPer; k++) bad |= split_invalid(v[k]);
    if (__syncthreads_or(bad)) {
        if (threadIdx.x == 0) atomicOr(status, A2AV_ST_BAD_SPLIT);
        return;
    }
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * 256;
        if (i < n) {
            const int s = i / W, d = i - s * W;
            O[d * W + s] = v[k];
        }
    }
}

// ====================================================================== offsets
// Row r < W scans S row r into send_off; row W + r scans O row r into
// recv_off. One wave per row (W <= 64 entries fit one wave64 scan), at most
// 16 waves, each loading all of its rows (and the status word, through the
// scalar cache: one block, the only writer) before anything waits.
__global__ __launch_bounds__(1024) void k_offsets(int W, const int64_t *__restrict__ S,
                                                  const int64_t *__restrict__ O,
                                                  int64_t *__restrict__ send_off,
                                                  int64_t *__restrict__ recv_off,
                                                  int32_t *status) {
    constexpr int kRows = (2 * A2AV_MAX_W + 15) / 16;  // rows per wave at most
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const int32_t st0 = status_at_entry(status);
    int64_t v[kRows];
#pragma unroll
    for (int k = 0; k < kRows; k++) {
        const int row = wave + k * nwaves;
        const int64_t *src = row < W ? S + (size_t)row * W : O + (size_t)(row - W) * W;
        v[k] = row < 2 * W && lane < W ? src[lane] : 0;
    }
    if (st0) return;
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kRows; k++) bad |= split_invalid(v[k]);
    if (__syncthreads_or(bad)) {
        if (threadIdx.x == 0) atomicOr(status, A2AV_ST_BAD_SPLIT);
        return;
    }
#pragma unroll
    for (int k = 0; k < kRows; k++) {
        const int row = wave + k * nwaves;  // the same in every lane of the wave
        if (row < 2 * W) {
            int64_t *dst = row < W ? send_off + (size_t)row * (W + 1) : recv_off + (size_t)(row - W) * (W + 1);
            const int64_t incl = (int64_t)wave_incl_scan_u64((uint64_t)v[k]);
            if (lane < W) dst[lane] = incl - v[k];
            if (lane == W - 1) dst[W] = incl;
        }
    }
}

// ====================================================================== W <= 8
// The same two steps in one wave each (no barrier): lane i < W * W holds
// S[i / W][i % W] for the exchange; for the offsets, the eight lanes of
// group r hold row r of S and row r of O, scanned inside the group.
__global__ __launch_bounds__(64) void k_exchange_w8(int W, const int64_t *__restrict__ S,
                                                    int64_t *__restrict__ O, int32_t *status) {
    const int lane = threadIdx.x, n = W * W;
    const int32_t st0 = status_at_entry(status);
    const int64_t v = lane < n ? S[lane] : 0;
    if (st0) return;
    if (__ballot(split_invalid(v))) {
        if (lane == 0) atomicOr(status, A2AV_ST_BAD_SPLIT);
        return;
    }
    if (lane < n) {
        const int s = lane / W, d = lane - s * W;
        O[d * W + s] = v;
    }
}

__global__ __launch_bounds__(64) void k_offsets_w8(int W, const int64_t *__restrict__ S,
                                                   const int64_t *__restrict__ O,
                                                   int64_t *__restrict__ send_off,
                                                   int64_t *__restrict__ recv_off, int32_t *status) {
    const int lane = threadIdx.x, r = lane / 8, k = lane % 8;
    const bool act = r < W && k < W;
    const int32_t st0 = status_at_entry(status);
    const int64_t vs = act ? S[r * W + k] : 0;
    const int64_t vo = act ? O[r * W + k] : 0;
    if (st0) return;
    if (__ballot(split_invalid(vs) || split_invalid(vo))) {
        if (lane == 0) atomicOr(status, A2AV_ST_BAD_SPLIT);
        return;
    }
    const int64_t is = (int64_t)group_incl_scan<8>((uint64_t)vs, k);
    const int64_t io = (int64_t)group_incl_scan<8>((uint64_t)vo, k);
    if (act) {
        send_off[r * (W + 1) + k] = is - vs;
        recv_off[r * (W + 1) + k] = io - vo;
        if (k == W - 1) {
            send_off[r * (W + 1) + W] = is;
            recv_off[r * (W + 1) + W] = io;
        }
    }
}

// ====================================================================== payload copy
// A block stages the split and offset matrices in LDS when W <= kMetaW (one
// global round trip for all of its metadata); above that it reads them from
// global memory (they are a few KiB and stay in L2).
constexpr int kMetaW = 16;

struct CopyArgs {
    const unsigned char *in[A2AV_MAX_W];
    unsigned char *out[A2AV_MAX_W];
    int64_t in_rows[A2AV_MAX_W];
    int64_t cap[A2AV_MAX_W];
    const int64_t *S;
    const int64_t *send_off;   // copy modes: input; fused mode: unused
    const int64_t *recv_off;
    int64_t *O_out;            // fused mode: outputs written by block 0
    int64_t *send_off_out;
    int64_t *recv_off_out;
    int32_t *status;
    uint64_t R;          // row bytes
    uint64_t min_piece;  // smallest piece of the destination space per block
    uint64_t piece;      // 0: one contiguous piece per block; else fixed piece
                         // size, pieces dealt to blocks round-robin
    int W;
};

template <int MW>
struct MetaLds {
    int64_t S[MW * MW];
    int64_t so[MW * (MW + 1)];
    int64_t ro[MW * (MW + 1)];
    int64_t pre[A2AV_MAX_W + 1];  // rows of destinations before d; [W] = total
    int bits;
    int poisoned;
};

enum PayloadMode {
    kCopyGiven = 0,  // a2av_copy: offsets given (staged in LDS by the block kernel)
    kCopyGlobal = 1,  // a2av_copy, W > kMetaW: metadata read from global
    kFused = 2,       // a2av_all_to_all_vdev, W <= kMetaW: offsets computed here
};

// Consistency of one (s, d) pair of the given offsets with S: the checks the
// payload step makes before any byte moves.
__device__ __forceinline__ int pair_bits(int64_t v, int64_t so0, int64_t so1, int64_t ro0,
                                         int64_t ro1, int s, int d) {
    int bits = 0;
    if (split_invalid(v)) bits |= A2AV_ST_BAD_SPLIT;
    if ((uint64_t)so1 - (uint64_t)so0 != (uint64_t)v) bits |= A2AV_ST_BAD_OFFSETS;
    if ((uint64_t)ro1 - (uint64_t)ro0 != (uint64_t)v) bits |= A2AV_ST_BAD_OFFSETS;
    if (d == 0 && so0 != 0) bits |= A2AV_ST_BAD_OFFSETS;
    if (s == 0 && ro0 != 0) bits |= A2AV_ST_BAD_OFFSETS;
    return bits;
}

// Wave 0: rows before each destination (pre) and the totals against the
// capacities. The capacity arrays are read with a uniform index (scalar
// loads from the kernel arguments).
template <int MW>
__device__ __forceinline__ int totals_and_pre(const CopyArgs &a, MetaLds<MW> &m,
                                              const int64_t *so, const int64_t *ro) {
    const int W = a.W, W1 = W + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = lane < W ? ro[lane * W1 + W] : 0;
    const int64_t incl = wave_incl_scan(t);
    if (lane < W) m.pre[lane] = incl - t;
    if (lane == W - 1) m.pre[W] = incl;
    int bits = 0;
    for (int r = 0; r < W; r++) {
        if (so[r * W1 + W] > a.in_rows[r]) bits |= A2AV_ST_SEND_OVERRUN;
        if (ro[r * W1 + W] > a.cap[r]) bits |= A2AV_ST_RECV_OVERFLOW;
    }
    return bits;
}

template <int BS, int U, bool NT, int MODE>
__global__ __launch_bounds__(BS) void k_a2av_payload(const CopyArgs a) {
    constexpr int MW = MODE == kCopyGlobal ? 1 : kMetaW;
    __shared__ MetaLds<MW> m;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int W = a.W, W1 = W + 1;

    // ---- prologue: the status word and the metadata loads go out together.
    // One thread reads the word and the block decides together: a failing
    // block of this same launch may set it at any moment, and waves of one
    // block must not disagree about it.
    if (tid == 0) {
        m.bits = 0;
        m.poisoned = status_poisoned(a.status);
    }
    if constexpr (MODE != kCopyGlobal) {
        for (int i = tid; i < W * W; i += BS) m.S[i] = a.S[i];
    }
    if constexpr (MODE == kCopyGiven) {
        for (int i = tid; i < W * W1; i += BS) {
            m.so[i] = a.send_off[i];
            m.ro[i] = a.recv_off[i];
        }
    }
    __syncthreads();
    if (m.poisoned) return;

    const int64_t *Sp = MODE == kCopyGlobal ? a.S : m.S;
    const int64_t *sop = MODE == kCopyGlobal ? a.send_off : m.so;
    const int64_t *rop = MODE == kCopyGlobal ? a.recv_off : m.ro;
    int bits = 0;
    if constexpr (MODE == kFused) {
        // splits valid; then send rows (S rows) and receive rows (S columns)
        // scanned, one wave64 scan per row
        for (int i = tid; i < W * W; i += BS)
            if (split_invalid(m.S[i])) bits |= A2AV_ST_BAD_SPLIT;
        for (int r = wave; r < 2 * W; r += BS / kWave) {
            int64_t v = 0;
            if (lane < W) v = r < W ? m.S[r * W + lane] : m.S[lane * W + (r - W)];
            const int64_t incl = wave_incl_scan(v);
            int64_t *dst = r < W ? m.so + r * W1 : m.ro + (r - W) * W1;
            if (lane < W) dst[lane] = incl - v;
            if (lane == W - 1) dst[W] = incl;
        }
        __syncthreads();
    } else {
        for (int i = tid; i < W * W; i += BS) {
            const int s = i / W, d = i - s * W;
            bits |= pair_bits(Sp[i], sop[s * W1 + d], sop[s * W1 + d + 1], rop[d * W1 + s],
                              rop[d * W1 + s + 1], s, d);
        }
    }
    if (wave == 0) bits |= totals_and_pre(a, m, sop, rop);
    if (bits) atomicOr(&m.bits, bits);
    __syncthreads();
    bits = m.bits;
    // fused: invalid splits stop the sequence at the exchange, as three
    // separate calls would, so the totals of bad scans are not reported
    if (MODE == kFused && (bits & A2AV_ST_BAD_SPLIT)) bits = A2AV_ST_BAD_SPLIT;

    if constexpr (MODE == kFused) {
        // block 0 publishes the exchange and offsets (when the splits are valid)
        if (blockIdx.x == 0) {
            if (!(bits & A2AV_ST_BAD_SPLIT)) {
                for (int i = tid; i < W * W; i += BS) {
                    const int s = i / W, d = i - s * W;
                    a.O_out[d * W + s] = m.S[i];
                }
                for (int i = tid; i < W * W1; i += BS) {
                    a.send_off_out[i] = m.so[i];
                    a.recv_off_out[i] = m.ro[i];
                }
            }
            if (bits && tid == 0) atomicOr(a.status, bits);
        }
    } else {
        if (bits && tid == 0) atomicOr(a.status, bits);
    }
    if (bits) return;

    // ---- the destination byte space: out[0] rows, then out[1] rows, ...
    const uint64_t R = a.R;
    const uint64_t B = (uint64_t)m.pre[W] * R;
    const uint64_t G = gridDim.x;
    uint64_t piece = a.piece;
    if (piece == 0) {
        piece = (B + G - 1) / G;
        if (piece < a.min_piece) piece = a.min_piece;
        piece = (piece + 4095) & ~(uint64_t)4095;
    }
    for (uint64_t p = blockIdx.x; p * piece < B; p += G) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < B ? lo + piece : B;
        // last destination whose space starts at or before lo, then the last
        // source chunk inside it that starts at or before lo
        const int64_t pre_l = lane < W ? m.pre[lane] : 0;
        const uint64_t mask_d = __ballot(lane < W && (uint64_t)pre_l * R <= lo);
        if (mask_d == 0) break;  // cannot happen after validation (pre[0] == 0)
        int d = 63 - __clzll(mask_d);
        uint64_t dbase = (uint64_t)m.pre[d] * R;
        const int64_t roff = lane < W ? rop[d * W1 + lane] : 0;
        const uint64_t mask_s = __ballot(lane < W && dbase + (uint64_t)roff * R <= lo);
        if (mask_s == 0) break;  // cannot happen after validation (offsets start at 0)
        int s = 63 - __clzll(mask_s);
        uint64_t x = lo;
        while (x < hi && d < W) {
            const int64_t r0 = rop[d * W1 + s];
            const int64_t n = Sp[s * W + d];
            const uint64_t F = dbase + (uint64_t)r0 * R;
            const uint64_t L = (uint64_t)n * R;
            if (n > 0 && x < F + L) {
                const uint64_t e = hi < F + L ? hi : F + L;
                const uint64_t off = x - F;
                const int64_t so = sop[s * W1 + d];
                // validated metadata always passes; the check keeps every
                // access inside the caller's buffers regardless (no sum that
                // can wrap: a negative value reads as 2^63 or more and fails)
                if (span_fits((uint64_t)r0, (uint64_t)n, (uint64_t)a.cap[d]) &&
                    span_fits((uint64_t)so, (uint64_t)n, (uint64_t)a.in_rows[s]))
                    copy_segment<BS, U, NT>(a.out[d] + (uint64_t)r0 * R + off,
                                            a.in[s] + (uint64_t)so * R + off, e - x, tid);
                x = e;
            }
            if (++s == W) {
                s = 0;
                ++d;
                if (d < W) dbase = (uint64_t)m.pre[d] * R;
            }
        }
    }
}

// ====================================================================== plain copy
template <int BS, int U, bool NT>
__global__ __launch_bounds__(BS) void k_device_copy(unsigned char *dst, const unsigned char *src,
                                                    uint64_t bytes, uint64_t min_piece,
                                                    uint64_t fixed_piece) {
    const uint64_t G = gridDim.x;
    uint64_t piece = fixed_piece;
    if (piece == 0) {
        piece = (bytes + G - 1) / G;
        if (piece < min_piece) piece = min_piece;
        piece = (piece + 4095) & ~(uint64_t)4095;
    }
    for (uint64_t p = blockIdx.x; p * piece < bytes; p += G) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < bytes ? lo + piece : bytes;
        copy_segment<BS, U, NT>(dst + lo, src + lo, hi - lo, threadIdx.x);
    }
}

// ====================================================================== wave-level payload (W <= 8)
// For up to 8 ranks every wave is self-contained. It reads the status word,
// the split matrix and the per-rank rows and capacities through the scalar
// cache (the scalar path does not queue behind the vector stream that older
// waves keep in flight on the same CU, which starves the vector loads of a
// young wave), computes every offset it needs in registers, and copies one
// piece of the destination space. No LDS and no barrier: the grid is sized to
// the traffic so that the hardware dispatcher hands pieces to waves as older
// ones retire, which evens out the unequal bandwidth that waves of different
// age get.
//
// Every wave spends its first instructions on the offsets, so their latency
// is paid once per piece and, at the start of a launch, before any payload
// byte moves. Two layouts of groups of P lanes (P the power of two at or
// above W, so that no group straddles a 16-lane DPP row) keep that short:
//   row layout     lane s*P + d holds the (s, d) entry: S[s][d], send_off[s][d]
//   column layout  lane d*P + s holds the (s, d) entry: recv_off[d][s]
// S enters the row layout by v_writelane from the scalar loads (two
// instructions per entry), scans inside groups are DPP row shifts (no LDS
// round trip), and one ds_bpermute round turns S and send_off into the
// column layout, where the scans give recv_off and the rows before each
// destination. Lane g*P + W-1, the last of group g, holds group g's totals
// and rank g's rows and capacity, so the range checks are vector compares.
constexpr int kWaveMaxW = 8;

// LDS the kernel declares for W > 4: S in the row layout and the four
// per-rank arrays.
constexpr unsigned kWaveOwnLds = (64 + 4 * 8) * sizeof(uint64_t);

template <int W>
constexpr int group_lanes() {
    return W <= 1 ? 1 : W <= 2 ? 2 : W <= 4 ? 4 : 8;
}

// The first five arguments repeat fields of a (S, status, R, piece and the
// grid's wave count) so that the compiler preloads them into scalar
// registers at wave launch (the library is built with
// -amdgpu-kernarg-preload-count=5): the first scalar burst can go out at
// once.
template <int W, int U, bool ALIGNED, int MODE>
__global__ __launch_bounds__(256) void k_a2av_wave(const int64_t *Sp, int32_t *stp, uint64_t R,
                                                   uint64_t piece, uint32_t waves, const CopyArgs a) {
    static_assert(W >= 1 && W <= kWaveMaxW, "one (s, d) entry per lane");
    constexpr int P = group_lanes<W>();
    constexpr int Q = W - 1;  // index in a group of the lane holding the group's totals
    constexpr uint32_t wpb = 256 / kWave;  // the launch's block size
    const int lane = threadIdx.x & (kWave - 1);
    // the wave's index, said to be uniform so that the piece loop runs on the
    // scalar unit
    const uint64_t gw = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const uint64_t TW = waves;
    const int gi = lane / P, gk = lane % P;  // group, index in the group
    const bool act = gi < W && gk < W;       // holds an (s, d) entry
    const bool last = gi < W && gk == Q;     // holds group gi's totals

    // ---- scalar loads into lanes. Every load of a burst is in flight
    // together, forced by an empty asm statement that needs all of its
    // values, and each wave makes one burst: at the start of a launch every
    // line it touches is cold, and each miss costs a memory round trip before
    // any payload byte moves. Afterwards the buffer addresses stay in lanes
    // and the piece walk reads them with v_readlane.
    //   W <= 4: each wave loads the status word, S (16 entries at most) and
    //     the rows, capacities and buffer addresses of every rank.
    //   W > 4: the workgroup's four waves share the work: wave k loads the
    //     status word, rows k and k + 4 of S and the k-th of the four
    //     per-rank arrays (input addresses, output addresses, rows,
    //     capacities), and the waves exchange them through LDS.
    constexpr int N = W * W;
    constexpr bool kOneBurst = W <= 4;
    const const_i64 *Sc = (const const_i64 *)Sp;
    const int32_t st0 = status_at_entry(stp);
    uint64_t v = 0;  // row layout: S[s][d]
    // lane r*P + Q (for W > 4 every lane of group r): in_rows[r], cap[r],
    // in[r], out[r]
    uint64_t lim_in = 0, lim_cap = 0, lane_in = 0, lane_out = 0;
    if constexpr (kOneBurst) {
        uint64_t t[16], ir[4], cp[4], pin[4], pout[4];  // entries past N or W repeat entry 0
#pragma unroll
        for (int i = 0; i < 16; i++) t[i] = (uint64_t)Sc[i < N ? i : 0];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int q = r < W ? r : 0;
            ir[r] = (uint64_t)a.in_rows[q];
            cp[r] = (uint64_t)a.cap[q];
            pin[r] = (uint64_t)(uintptr_t)a.in[q];
            pout[r] = (uint64_t)(uintptr_t)a.out[q];
        }
        asm volatile("" ::A2AV_SREG16(t, 0), "s"(st0), A2AV_SREG4(ir, 0), A2AV_SREG4(cp, 0),
                     A2AV_SREG4(pin, 0), A2AV_SREG4(pout, 0));
#pragma unroll
        for (int i = 0; i < N; i++) v = writelane_u64(v, t[i], i / W * P + i % W);
#pragma unroll
        for (int r = 0; r < W; r++) {
            lim_in = writelane_u64(lim_in, ir[r], r * P + Q);
            lim_cap = writelane_u64(lim_cap, cp[r], r * P + Q);
            lane_in = writelane_u64(lane_in, pin[r], r * P + Q);
            lane_out = writelane_u64(lane_out, pout[r], r * P + Q);
        }
    } else {
        static_assert(P == 8, "rows of S in groups of 8 lanes");
        __shared__ uint64_t sh_s[64];    // S in the row layout
        __shared__ uint64_t sh_a[4][8];  // in[], out[], in_rows[], cap[]
        const int k = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        // the k-th per-rank array: CopyArgs holds in, out, in_rows and cap
        // back to back, 64 entries each (entries past W are not used)
        const const_i64 *arr = (const const_i64 *)&a.in[0] + 64 * k;
        uint64_t ar[8];
#pragma unroll
        for (int r = 0; r < 8; r++) ar[r] = (uint64_t)arr[r];
        // rows k and k + 4 of S (a row past W loads row 0 and is dropped)
        const bool hi_row = k + 4 < W;
        const const_i64 *r0p = Sc + k * W;
        const const_i64 *r1p = Sc + (hi_row ? (k + 4) * W : 0);
        uint64_t t[16];
#pragma unroll
        for (int d = 0; d < 8; d++) {
            t[d] = (uint64_t)r0p[d < W ? d : 0];
            t[8 + d] = (uint64_t)r1p[d < W ? d : 0];
        }
        asm volatile("" ::A2AV_SREG16(t, 0), "s"(st0), A2AV_SREG8(ar, 0));
        uint64_t part = 0, apart = 0;  // lanes 0..7: row k, 8..15: row k + 4
#pragma unroll
        for (int d = 0; d < W; d++) {
            part = writelane_u64(part, t[d], d);
            part = writelane_u64(part, hi_row ? t[8 + d] : 0, 8 + d);
        }
#pragma unroll
        for (int r = 0; r < W; r++) apart = writelane_u64(apart, ar[r], r);
        if (lane < 16) sh_s[8 * k + lane + (lane >= 8 ? 24 : 0)] = part;
        if (lane < 8) sh_a[k][lane] = apart;
        __syncthreads();
        v = sh_s[lane];
        lane_in = sh_a[0][gi];
        lane_out = sh_a[1][gi];
        lim_in = sh_a[2][gi];
        lim_cap = sh_a[3][gi];
    }
    // copy mode: the given send_off[s][d] (row layout) and recv_off[d][s]
    // (column layout) share one index, row gi entry gk of each matrix, and
    // the last lane of a group also takes the row's total
    uint64_t gso = 0, gro = 0, gso_t = 0, gro_t = 0;
    auto load_given = [&]() {
        if (act) {
            gso = (uint64_t)a.send_off[gi * (W + 1) + gk];
            gro = (uint64_t)a.recv_off[gi * (W + 1) + gk];
            if (gk == Q) {
                gso_t = (uint64_t)a.send_off[gi * (W + 1) + W];
                gro_t = (uint64_t)a.recv_off[gi * (W + 1) + W];
            }
        }
    };
    // copy mode: with aligned rows and 8 vectors in flight per lane the
    // offsets are loaded behind the wave's first payload loads (see the gate
    // below); otherwise here. (With 16 in flight the gate's wait for all of
    // them before the first store cost more than it saved: copies of 1 GiB
    // per rank took 4 % longer.)
    constexpr bool kDeferred = MODE == kCopyGiven && ALIGNED && U <= 8;
    if constexpr (MODE == kCopyGiven && !kDeferred) load_given();
    if (st0) return;

    // ---- offsets from S (wrapping arithmetic, as the checks compare modulo
    // 2^64); lanes outside the entries hold zeros, so a group's scan reaches
    // its total at index Q
    const uint64_t inc = group_incl_scan<P>(v, gk);  // row layout: send_off[s][d + 1]
    const uint64_t so = inc - v;                     // row layout: send_off[s][d]
    const int tsrc = gk * P + gi;                    // the row-layout lane of this column-layout lane
    const uint64_t vt = lane_gather(v, tsrc);        // column layout: S[s][d]
    const uint64_t sot = lane_gather(so, tsrc);      // column layout: send_off[s][d]
    const uint64_t inc2 = group_incl_scan<P>(vt, gk);  // column layout: recv_off[d][s + 1]
    const uint64_t ro = inc2 - vt;                     // column layout: recv_off[d][s]
    // lane d*P + Q: rows of the destinations before d, the sum over s of
    // send_off[s][d]
    const uint64_t pre = group_incl_scan<P>(sot, gk);
    const uint64_t total = readlane_u64(pre, Q * P + Q) + readlane_u64(inc2, Q * P + Q);

    // ---- checks, identical in every wave
    int bits = __ballot(act && split_invalid((int64_t)v)) ? A2AV_ST_BAD_SPLIT : 0;
    // copy mode: the given offsets and totals against S and the buffers. When
    // deferred, the offsets are loaded and checked once the wave's first
    // payload loads are in flight (a gate before its first store), so the
    // check costs no round trip of its own; otherwise it runs here.
    auto given_bits = [&]() -> int {
        int b = bits;
        const bool bad_off = act && (gso != so || gro != ro || (gk == Q && (gso_t != inc || gro_t != inc2)));
        if (__ballot(bad_off)) b |= A2AV_ST_BAD_OFFSETS;
        if (__ballot(last && (int64_t)gso_t > (int64_t)lim_in)) b |= A2AV_ST_SEND_OVERRUN;
        if (__ballot(last && (int64_t)gro_t > (int64_t)lim_cap)) b |= A2AV_ST_RECV_OVERFLOW;
        return b;
    };
    bool pending = kDeferred;  // the gate has not run yet
    auto gate = [&]() -> bool {
        if (!pending) return true;
        pending = false;
        load_given();
        const int b = given_bits();
        if (b && gw == 0 && lane == 0) atomicOr(stp, b);
        return b == 0;
    };
    if constexpr (MODE == kCopyGiven) {
        if (kDeferred && bits) load_given();
        if (!kDeferred || bits) bits = given_bits();
    } else {
        if (__ballot(last && (int64_t)inc > (int64_t)lim_in)) bits |= A2AV_ST_SEND_OVERRUN;
        if (__ballot(last && (int64_t)inc2 > (int64_t)lim_cap)) bits |= A2AV_ST_RECV_OVERFLOW;
        // invalid splits stop the sequence at the exchange
        if (bits & A2AV_ST_BAD_SPLIT) bits = A2AV_ST_BAD_SPLIT;
    }
    if (gw == 0) {
        if constexpr (MODE == kFused) {
            if (!(bits & A2AV_ST_BAD_SPLIT) && act) {
                a.O_out[gi * W + gk] = (int64_t)vt;  // O[d][s] = S[s][d]
                a.send_off_out[gi * (W + 1) + gk] = (int64_t)so;
                a.recv_off_out[gi * (W + 1) + gk] = (int64_t)ro;
                if (gk == Q) {
                    a.send_off_out[gi * (W + 1) + W] = (int64_t)inc;
                    a.recv_off_out[gi * (W + 1) + W] = (int64_t)inc2;
                }
            }
        }
        if (bits && lane == 0) atomicOr(stp, bits);
    }
    if (bits) return;

    // ---- pieces of the destination space: out[0] rows, then out[1] rows, ...
    const uint64_t B = total * R;
    for (uint64_t p = gw; p * piece < B; p += TW) {
        uint64_t lo = p * piece;
        uint64_t hi = lo + piece < B ? lo + piece : B;
        if constexpr (!ALIGNED) {
            // rows that are not 16-byte multiples: cut where the destination
            // address is 128-byte aligned, so no cache line is split between
            // two waves' partial writes (neighbouring pieces move the same
            // boundary, so the pieces still tile the space)
            lo = snap_to_line<P, Q>(lo, B, pre * R, lane, W, a.out);
            hi = snap_to_line<P, Q>(hi, B, pre * R, lane, W, a.out);
            if (lo >= hi) continue;
        }
        // last destination starting at or before lo (lane d*P + Q holds its
        // rows before), then the last source chunk inside it starting at or
        // before lo (lane d*P + s holds recv_off[d][s])
        const uint64_t mask_d = __ballot(last && pre * R <= lo);
        if (mask_d == 0) break;  // cannot happen: pre[0] == 0
        int d = (63 - __clzll(mask_d)) / P;
        uint64_t dbase = readlane_u64(pre, d * P + Q) * R;
        const uint64_t mask_s = __ballot(gi == d && gk < W && dbase + ro * R <= lo);
        if (mask_s == 0) break;  // cannot happen: recv_off[d][0] == 0
        int s = (63 - __clzll(mask_s)) % P;
        uint64_t x = lo;
        while (x < hi && d < W) {
            const int lr = s * P + d, lc = d * P + s;  // row and column layout lanes
            const uint64_t n = readlane_u64(v, lr);
            const uint64_t r0 = readlane_u64(ro, lc);
            const uint64_t F = dbase + r0 * R;
            const uint64_t L = n * R;
            if (n > 0 && x < F + L) {
                const uint64_t e = hi < F + L ? hi : F + L;
                const uint64_t off = x - F;
                const uint64_t s0 = readlane_u64(so, lr);
                // d and s are wave-uniform; saying so keeps the argument
                // reads below scalar (a vector read would wait behind the
                // payload traffic of older waves on the CU)
                const int du = __builtin_amdgcn_readfirstlane(d);
                const int su = __builtin_amdgcn_readfirstlane(s);
                // validated offsets always pass; the check keeps every access
                // inside the caller's buffers regardless (no sum that can
                // wrap); the capacities and rows come from the lanes that
                // hold them, and both sides are evaluated (no short cut)
                if (span_fits(r0, n, readlane_u64(lim_cap, du * P + Q)) &
                    span_fits(s0, n, readlane_u64(lim_in, su * P + Q))) {
                    unsigned char *dst =
                        (unsigned char *)(uintptr_t)readlane_u64(lane_out, du * P + Q) + r0 * R + off;
                    const unsigned char *src =
                        (const unsigned char *)(uintptr_t)readlane_u64(lane_in, su * P + Q) + s0 * R + off;
                    if constexpr (kDeferred) {
                        if (!wave_copy16<U>(dst, src, e - x, lane, gate)) return;
                    } else if constexpr (ALIGNED) {
                        wave_copy16<U>(dst, src, e - x, lane);
                    } else {
                        wave_copy_any<U>(dst, src, e - x, lane);
                    }
                }
                x = e;
            }
            if (++s == W) {
                s = 0;
                ++d;
                if (d < W) dbase = readlane_u64(pre, d * P + Q) * R;
            }
        }
    }
    // a wave that copied nothing still reports the verdict from wave 0
    if constexpr (kDeferred) {
        if (pending && gw == 0) gate();
    }
}

// ---------------------------------------------------------------- W > 8
// More ranks than a wave holds (s, d) pairs: one workgroup prepares and
// checks everything first, then waves copy pieces of the flat destination
// space as above, looking the pieces up in the offsets the prep wrote.
//
// k_a2av_prep (one 1024-thread workgroup). Fused mode: checks the splits,
// writes O, send_off and recv_off from S, and checks the totals against the
// caller's rows and capacities. Given mode (a2av_copy): checks the given
// offsets against S and the given totals against rows and capacities. It is
// the only writer of the status word before the copy launch, and it reads
// the word once, at entry.
template <bool FUSED>
__global__ __launch_bounds__(1024) void k_a2av_prep(const CopyArgs a) {
    __shared__ int64_t sl[A2AV_MAX_W * A2AV_MAX_W];
    __shared__ int poisoned, lbits;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int NWV = 1024 / kWave;
    const int W = a.W, W1 = W + 1;
    if (tid == 0) {
        poisoned = status_poisoned(a.status);
        lbits = 0;
    }
    int bad = 0;
    for (int i = tid; i < W * W; i += 1024) {
        sl[i] = a.S[i];
        bad |= (int)split_invalid(sl[i]);
    }
    __syncthreads();
    if (poisoned) return;
    if (FUSED && __syncthreads_or(bad)) {
        // invalid splits stop the sequence at the exchange
        if (tid == 0) atomicOr(a.status, A2AV_ST_BAD_SPLIT);
        return;
    }
    int bits = 0;
    if constexpr (FUSED) {
        // rows r < W: send offsets of rank r; rows W + d: receive offsets of d
        for (int r = wave; r < 2 * W; r += NWV) {
            int64_t v = 0;
            if (lane < W) v = r < W ? sl[r * W + lane] : sl[lane * W + (r - W)];
            const int64_t incl = wave_incl_scan(v);
            int64_t *dst = r < W ? a.send_off_out + r * W1 : a.recv_off_out + (r - W) * W1;
            if (lane < W) dst[lane] = incl - v;
            if (lane == W - 1) {
                dst[W] = incl;
                if (r < W && incl > a.in_rows[r]) bits |= A2AV_ST_SEND_OVERRUN;
                if (r >= W && incl > a.cap[r - W]) bits |= A2AV_ST_RECV_OVERFLOW;
            }
        }
        for (int i = tid; i < W * W; i += 1024) {
            const int s = i / W, d = i - s * W;
            a.O_out[d * W + s] = sl[i];
        }
    } else {
        for (int i = tid; i < W * W; i += 1024) {
            const int s = i / W, d = i - s * W;
            bits |= pair_bits(sl[i], a.send_off[s * W1 + d], a.send_off[s * W1 + d + 1],
                              a.recv_off[d * W1 + s], a.recv_off[d * W1 + s + 1], s, d);
        }
        for (int r = tid; r < W; r += 1024) {
            if (a.send_off[r * W1 + W] > a.in_rows[r]) bits |= A2AV_ST_SEND_OVERRUN;
            if (a.recv_off[r * W1 + W] > a.cap[r]) bits |= A2AV_ST_RECV_OVERFLOW;
        }
    }
    if (bits) atomicOr(&lbits, bits);
    __syncthreads();
    if (tid == 0 && lbits) atomicOr(a.status, lbits);
}

// The GPU's wave for walk_pieces_any (wave_walk.h): one lane per thread,
// cross-lane operations from the hardware, uniform loads through the scalar
// cache (send_off is not written during the copy), the payload moved with the
// wave copies. The destination totals and one receive-offset row come from
// the workgroup's scalar loads (k_a2av_wave_any); any other row is loaded by
// the lanes.
typedef __attribute__((address_space(3))) const uint64_t lds_u64;


template <int U, bool ALIGNED>
struct DeviceWave {
    int ln;
    uint64_t tot;       // lane d < W: recv_off[d][W]
    int d_row;          // the destination whose row is in row_lds
    const lds_u64 *row_lds;  // recv_off[d_row][0..W]
    __device__ int lane() const { return ln; }
    __device__ int64_t load_uniform(const int64_t *p) const {
        // the address taken from the first lane, so that the load is a
        // scalar one whatever the compiler could prove about it
        const uint64_t x = (uint64_t)(uintptr_t)p;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
        return *(const const_i64 *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    }
    __device__ void copy(unsigned char *d, const unsigned char *s, uint64_t n) const {
        if constexpr (ALIGNED) wave_copy16<U>(d, s, n, ln);
        else wave_copy_any<U>(d, s, n, ln);
    }
    __device__ uint64_t ballot(int, bool b) const { return __ballot(b); }
    __device__ uint64_t readlane(int, uint64_t v, int l) const { return readlane_u64(v, l); }
    __device__ int uniform(int, int x) const { return __builtin_amdgcn_readfirstlane(x); }
    __device__ uint64_t incl_scan(int, uint64_t v) const { return wave_incl_scan_u64(v); }
    __device__ uint64_t dest_totals(int, const CopyArgs &) const { return tot; }
    __device__ void row(int, const CopyArgs &a, int d, uint64_t &ro, uint64_t &n) const {
        const int W = a.W;
        if (d == d_row) {
            ro = ln < W ? row_lds[ln] : 0;
            n = ln < W ? row_lds[ln + 1] - ro : 0;
        } else {
            const int64_t *rrow = a.recv_off + (uint64_t)d * (W + 1);
            ro = ln < W ? (uint64_t)rrow[ln] : 0;
            n = ln < W ? (uint64_t)rrow[ln + 1] - ro : 0;
        }
    }
};

// LDS the W > 8 wave kernel declares itself: the destination totals and one
// receive-offset row, in one array whose size is a multiple of 16 bytes (so
// that the size the launch subtracts from the occupancy cap is the size the
// kernel is given).
constexpr int kAnyLdsWords = 2 * A2AV_MAX_W + 2;
constexpr unsigned kAnyOwnLds = kAnyLdsWords * 8;
static_assert(kAnyOwnLds % 16 == 0, "LDS rounded to 16 bytes");

// The copy after k_a2av_prep, one piece per wave (walk_pieces_any). Before
// the walk, the workgroup loads what its waves look up first, through the
// scalar cache in two bursts (a vector load of a young wave waits behind the
// payload traffic older waves keep in flight on the CU; a scalar load does
// not), and shares it through LDS:
//   1. the status word and the destination totals recv_off[d][W], wave k
//      taking d = 16k .. 16k + 15;
//   2. the receive-offset row of the destination holding the workgroup's
//      first byte (its four waves' pieces are neighbours, so they nearly
//      always start in it), wave k taking entries 16k .. 16k + 16.
// Every wave reaches both barriers before it looks at the status word.
template <int U, bool ALIGNED>
__global__ __launch_bounds__(256) void k_a2av_wave_any(const CopyArgs a) {
    __shared__ uint64_t sh_meta[kAnyLdsWords];
    uint64_t *const sh_tot = sh_meta;               // [A2AV_MAX_W]
    uint64_t *const sh_row = sh_meta + A2AV_MAX_W;  // [A2AV_MAX_W + 1]
    const int lane = threadIdx.x & (kWave - 1);
    const int k = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t gw = (uint64_t)blockIdx.x * 4 + k;
    const uint64_t TW = (uint64_t)gridDim.x * 4;
    const int W = a.W, W1 = W + 1;
    const const_i64 *rc = (const const_i64 *)a.recv_off;
    const int32_t st0 = status_at_entry(a.status);
    // entries past the matrix repeat its last one and are not stored; each
    // load takes the matrix address and a 32-bit byte offset (the matrix is
    // at most 64 x 65 entries), so the burst needs one address, not sixteen
    uint64_t t[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int e = 16 * k + i < W ? 16 * k + i : W - 1;
        t[i] = (uint64_t)at_byte(rc, (uint32_t)(e * W1 + W) * 8u);
    }
    asm volatile("" : A2AV_SREG16_IO(t, 0) : "s"(st0));
    uint64_t part = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) part = writelane_u64(part, t[i], i);
    if (lane < 16 && 16 * k + lane < W) sh_tot[16 * k + lane] = part;
    __syncthreads();
    const uint64_t tot = lane < W ? sh_tot[lane] : 0;
    const uint64_t incl = wave_incl_scan_u64(tot);
    const uint64_t pre = incl - tot;
    // the last destination starting at or before the workgroup's first byte
    // (the same in its four waves: they scan the same totals)
    const uint64_t lo0 = (uint64_t)blockIdx.x * 4 * a.piece;
    const uint64_t mask = __ballot(lane < W && pre * a.R <= lo0);
    const int dw = __builtin_amdgcn_readfirstlane(mask ? 63 - (int)__clzll(mask) : 0);
    uint64_t u[17];
#pragma unroll
    for (int i = 0; i < 17; i++)
        u[i] = (uint64_t)at_byte(rc, (uint32_t)(dw * W1 + (16 * k + i <= W ? 16 * k + i : W)) * 8u);
    asm volatile("" : A2AV_SREG16_IO(u, 0), "+s"(u[16]));
    part = 0;
#pragma unroll
    for (int i = 0; i < 17; i++) part = writelane_u64(part, u[i], i);
    if (lane < 17 && 16 * k + lane <= W) sh_row[16 * k + lane] = part;
    __syncthreads();
    if (st0) return;  // final: the prep launch wrote it
    DeviceWave<U, ALIGNED> wv{lane, tot, dw, (const lds_u64 *)sh_row};
    walk_pieces_any(wv, a, gw, TW);
}

// Plain copy with the same one-piece-per-wave structure.
template <int U, bool ALIGNED>
__global__ __launch_bounds__(256) void k_device_copy_wave(unsigned char *dst, const unsigned char *src,
                                                          uint64_t bytes, uint64_t piece) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t TW = (uint64_t)gridDim.x * wpb;
    for (uint64_t p = (uint64_t)blockIdx.x * wpb + threadIdx.x / kWave; p * piece < bytes; p += TW) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < bytes ? lo + piece : bytes;
        if constexpr (ALIGNED) wave_copy16<U>(dst + lo, src + lo, hi - lo, lane);
        else wave_copy_any<U>(dst + lo, src + lo, hi - lo, lane);
    }
}

// ====================================================================== one-direction ceilings
// Streams that only read or only write, with the piece structure of the
// plain copy (one piece per wave, 16-byte accesses, U of them in flight per
// lane): the HBM ceilings for kernels whose traffic runs mostly one way,
// such as the pack's row scatter, which writes k bytes for every byte it
// reads.
constexpr int kSinkWords = 4096;

// Every 16-byte vector of src is read once. Each wave XOR-folds what it read
// into one 64-bit word and XORs that into sink[wave mod kSinkWords] (one
// atomic per wave, spread over 32 KiB), so the XOR of all sink words is the
// fold of the XOR of every vector: the loads cannot be dropped and a test can
// check that each was made.
template <int U>
__global__ __launch_bounds__(256) void k_device_read_wave(const unsigned char *src, uint64_t bytes,
                                                          uint64_t piece, uint64_t *sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t gw = (uint64_t)blockIdx.x * wpb + threadIdx.x / kWave;
    const uint64_t TW = (uint64_t)gridDim.x * wpb;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t p = gw; p * piece < bytes; p += TW) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < bytes ? lo + piece : bytes;
        const u32x4 *s = (const u32x4 *)(src + lo);
        const uint64_t nv = (hi - lo) / 16;
        for (uint64_t base = 0; base < nv; base += (uint64_t)kWave * U) {
            u32x4 r[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t i = base + (uint64_t)u * kWave + lane;
                r[u] = ld<true>(s + (i < nv ? i : nv - 1));
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                // a clamped index re-read the last vector: it is not counted
                const uint32_t m = base + (uint64_t)u * kWave + lane < nv ? ~0u : 0u;
                acc.x ^= r[u].x & m;
                acc.y ^= r[u].y & m;
                acc.z ^= r[u].z & m;
                acc.w ^= r[u].w & m;
            }
        }
    }
    uint64_t x = ((uint64_t)(acc.x ^ acc.z) << 32) | (uint64_t)(acc.y ^ acc.w);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) x ^= (uint64_t)__shfl_xor((long long)x, o, kWave);
    if (lane == 0 && x != 0) atomicXor((unsigned long long *)&sink[gw % kSinkWords], x);
}

// Every 16-byte vector of dst is written once with the pattern.
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_device_fill_wave(unsigned char *dst, uint64_t bytes,
                                                          uint64_t piece, uint32_t pattern) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wpb = blockDim.x / kWave;
    const uint64_t TW = (uint64_t)gridDim.x * wpb;
    const u32x4 v = {pattern, pattern, pattern, pattern};
    for (uint64_t p = (uint64_t)blockIdx.x * wpb + threadIdx.x / kWave; p * piece < bytes; p += TW) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < bytes ? lo + piece : bytes;
        u32x4 *d = (u32x4 *)(dst + lo);
        const uint64_t nv = (hi - lo) / 16;
        for (uint64_t base = 0; base < nv; base += (uint64_t)kWave * U) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t i = base + (uint64_t)u * kWave + lane;
                st<NT>(d + (i < nv ? i : nv - 1), v);
            }
        }
    }
}

// ====================================================================== launch config
struct CopyTuning {
    int blocks_per_cu;
    int unroll;
    int nontemporal;
    long min_piece;
    long piece;
    int block_kernel;  // 1: use the workgroup (LDS) kernel for W <= 8 too
};

static CopyTuning copy_tuning() {
    CopyTuning t;
    t.blocks_per_cu = (int)env_long("A2AV_BLOCKS_PER_CU", 16, 1, 64);
    t.unroll = (int)env_long("A2AV_UNROLL", 4, 1, 8);
    t.nontemporal = (int)env_long("A2AV_NT", 1, 0, 1);
    t.min_piece = env_long("A2AV_MIN_PIECE", 16384, 4096, 1L << 30);
    t.piece = env_long("A2AV_PIECE", 0, 0, 1L << 34);
    if (t.piece != 0) t.piece = (t.piece + 4095) & ~4095L;
    t.block_kernel = (int)env_long("A2AV_BLOCK_KERNEL", 0, 0, 1);
    return t;
}

template <int BS, int U, int MODE>
static void launch_payload_u(const CopyArgs &a, int grid, bool nt, hipStream_t st) {
    if (nt) hipLaunchKernelGGL((k_a2av_payload<BS, U, true, MODE>), dim3(grid), dim3(BS), 0, st, a);
    else hipLaunchKernelGGL((k_a2av_payload<BS, U, false, MODE>), dim3(grid), dim3(BS), 0, st, a);
}

template <int MODE>
static void launch_payload(const CopyArgs &a, int grid, const CopyTuning &t, hipStream_t st) {
    const bool nt = t.nontemporal != 0;
    switch (t.unroll) {
    case 1: launch_payload_u<256, 1, MODE>(a, grid, nt, st); break;
    case 2: launch_payload_u<256, 2, MODE>(a, grid, nt, st); break;
    case 8: launch_payload_u<256, 8, MODE>(a, grid, nt, st); break;
    default: launch_payload_u<256, 4, MODE>(a, grid, nt, st); break;
    }
}

template <int BS, int U>
static void launch_dcopy_u(unsigned char *d, const unsigned char *s, uint64_t n, const CopyTuning &t,
                           int grid, hipStream_t st) {
    if (t.nontemporal)
        hipLaunchKernelGGL((k_device_copy<BS, U, true>), dim3(grid), dim3(BS), 0, st, d, s, n,
                           (uint64_t)t.min_piece, (uint64_t)t.piece);
    else
        hipLaunchKernelGGL((k_device_copy<BS, U, false>), dim3(grid), dim3(BS), 0, st, d, s, n,
                           (uint64_t)t.min_piece, (uint64_t)t.piece);
}

// Wave kernel: traffic up to kSmallTraffic moves in 8 KiB pieces with 8
// loads in flight per lane; larger traffic in 32 KiB pieces with 16.
//
// W <= 8 with 16-byte rows from kShortTraffic up: 4 KiB pieces with 4 loads
// in flight per lane, and for the one-call kernel (and the plain copy) at most
// a few workgroups per CU, enforced with 32 KiB of LDS per workgroup that the
// kernel does not use. Fewer, shorter-lived waves per CU stream HBM better
// here: at W = 4 / 8 x 32 MiB per rank the one-call kernel went 46.6 -> 45.2 /
// 89.7 -> 85.8 us and the copy-only kernel 47.3 -> 44.8 / 91.1 -> 87.4 us;
// at 1 GiB per rank 1434 -> 1409 / 2887 -> 2826 us and 1451 -> 1414 /
// 2990 -> 2867 us. The copy-only kernel's own registers already keep it to
// five waves per SIMD there; the LDS cap made it slower. Below 64 MiB per
// side the shapes above stay, and rows that are not 16-byte multiples get no
// cap.
constexpr uint64_t kSmallTraffic = 512ull << 20;
constexpr uint64_t kShortTraffic = 64ull << 20;
constexpr unsigned kCapLds = 32768;

struct WaveTuning {
    int unroll;
    uint64_t piece;
    unsigned lds;  // dynamic LDS per workgroup (occupancy cap), 0: none
};

static WaveTuning wave_tuning(uint64_t bmax, bool short_pieces = false, bool cap = false) {
    WaveTuning t;
    const bool small = bmax <= kSmallTraffic;
    const int u0 = short_pieces ? 4 : small ? 8 : 16;
    const long p0 = short_pieces ? 4096 : small ? 8192 : 32768;
    t.unroll = (int)env_long("A2AV_WAVE_UNROLL", u0, 4, 16);
    if (t.unroll != 4 && t.unroll != 8 && t.unroll != 16) t.unroll = 8;
    t.piece = (uint64_t)env_long("A2AV_WAVE_PIECE", p0, 4096, 1L << 30);
    t.piece = (t.piece + 4095) & ~(uint64_t)4095;
    t.lds = (unsigned)env_long("A2AV_WAVE_LDS", short_pieces && cap ? kCapLds : 0, 0, 65536);
    return t;
}

// The tuning of the W <= 8 wave kernel, the one-call kernel and a2av_copy
// alike, rows of any width: from kShortTraffic up, short pieces and the
// occupancy cap. (Measured on the current prologue: the copy-only kernel
// W = 4 x 32 MiB 44.76 -> 43.47 us, x 256 MiB 345.7 -> 335.7 us, same-process
// A/B; the keys a2av, 8-byte rows, 87.5 -> 86.2 us, where with the older
// prologue the cap had made both slower.)
static WaveTuning wave_tuning_w8(uint64_t bmax) {
    const bool short_pieces = bmax >= kShortTraffic;
    return wave_tuning(bmax, short_pieces, true);
}

// The tuning of the more-than-8-ranks wave kernel: short pieces and the cap
// in both entries (W = 16 / 64 x 32 MiB per rank: one-call 186.4 -> 178.3 /
// 798.3 -> 763.0 us, copy-only 184.3 -> 175.0 / 789.4 -> 753.1 us).
static WaveTuning wave_tuning_any(uint64_t bmax, bool aligned) {
    return wave_tuning(bmax, aligned && bmax >= kShortTraffic, true);
}

static int wave_grid(uint64_t bmax, uint64_t piece) {
    const uint64_t per_block = piece * 4;  // 4 waves per 256-thread block
    uint64_t g = (bmax + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > max_grid()) g = max_grid();  // the piece loop strides over the rest
    return (int)g;
}

template <int W, int MODE>
static void launch_wave_w(const CopyArgs &a, bool aligned, const WaveTuning &wt, int grid,
                          hipStream_t st) {
    // the LDS the kernel declares itself (W > 4) counts against the
    // occupancy cap
    constexpr unsigned own = W > 4 ? kWaveOwnLds : 0;
    const unsigned lds = wt.lds > own ? wt.lds - own : wt.lds;
    const uint32_t waves = (uint32_t)grid * (256 / kWave);
    if (wt.unroll == 16) {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave<W, 16, true, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
        else hipLaunchKernelGGL((k_a2av_wave<W, 16, false, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
    } else if (wt.unroll == 4) {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave<W, 4, true, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
        else hipLaunchKernelGGL((k_a2av_wave<W, 4, false, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
    } else {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave<W, 8, true, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
        else hipLaunchKernelGGL((k_a2av_wave<W, 8, false, MODE>), dim3(grid), dim3(256), lds, st, a.S,
                                     a.status, a.R, a.piece, waves, a);
    }
}

template <int MODE>
static void launch_wave(const CopyArgs &a, bool aligned, const WaveTuning &wt, int grid,
                        hipStream_t st) {
    switch (a.W) {
    case 1: launch_wave_w<1, MODE>(a, aligned, wt, grid, st); break;
    case 2: launch_wave_w<2, MODE>(a, aligned, wt, grid, st); break;
    case 3: launch_wave_w<3, MODE>(a, aligned, wt, grid, st); break;
    case 4: launch_wave_w<4, MODE>(a, aligned, wt, grid, st); break;
    case 5: launch_wave_w<5, MODE>(a, aligned, wt, grid, st); break;
    case 6: launch_wave_w<6, MODE>(a, aligned, wt, grid, st); break;
    case 7: launch_wave_w<7, MODE>(a, aligned, wt, grid, st); break;
    default: launch_wave_w<8, MODE>(a, aligned, wt, grid, st); break;
    }
}

// W > kWaveMaxW: the prep workgroup, then the wave copy on the offsets it
// checked (fused: the offsets it wrote).
template <bool FUSED>
static void launch_wave_any(CopyArgs a, bool aligned, const WaveTuning &wt, int grid,
                            hipStream_t st) {
    hipLaunchKernelGGL((k_a2av_prep<FUSED>), dim3(1), dim3(1024), 0, st, a);
    if (FUSED) {
        a.send_off = a.send_off_out;
        a.recv_off = a.recv_off_out;
    }
    // the kernel's own LDS counts against the occupancy cap
    const unsigned lds = wt.lds > kAnyOwnLds ? wt.lds - kAnyOwnLds : wt.lds;
    if (wt.unroll == 16) {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave_any<16, true>), dim3(grid), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((k_a2av_wave_any<16, false>), dim3(grid), dim3(256), lds, st, a);
    } else if (wt.unroll == 4) {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave_any<4, true>), dim3(grid), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((k_a2av_wave_any<4, false>), dim3(grid), dim3(256), lds, st, a);
    } else {
        if (aligned) hipLaunchKernelGGL((k_a2av_wave_any<8, true>), dim3(grid), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((k_a2av_wave_any<8, false>), dim3(grid), dim3(256), lds, st, a);
    }
}

// Largest possible traffic in bytes (what either side can hold) and whether
// every base and row allows the 16-byte path.
static void traffic_bound(const CopyArgs &a, uint64_t *bmax, bool *aligned) {
    uint64_t in_total = 0, out_total = 0;
    bool al = (a.R % 16) == 0;
    for (int r = 0; r < a.W; r++) {
        in_total += (uint64_t)a.in_rows[r];
        out_total += (uint64_t)a.cap[r];
        al = al && ((uintptr_t)a.in[r] % 16 == 0) && ((uintptr_t)a.out[r] % 16 == 0);
    }
    *bmax = (in_total < out_total ? in_total : out_total) * a.R;
    *aligned = al;
}

static int launch_status() {
    return hipGetLastError() == hipSuccess ? A2AV_OK : A2AV_EHIP;
}

// Host checks shared by a2av_copy and a2av_all_to_all_vdev; fills the buffer
// part of the kernel arguments.
static int fill_buffers(CopyArgs &a, int W, size_t row_bytes, const void *const *in,
                        const int64_t *in_rows, void *const *out, const int64_t *out_cap_rows) {
    std::memset(&a, 0, sizeof(a));
    uint64_t cap_bytes = 0;  // the flat destination space must fit 62 bits
    for (int r = 0; r < W; r++) {
        if (in_rows[r] < 0 || out_cap_rows[r] < 0) return A2AV_EARG;
        if ((uint64_t)in_rows[r] > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
        if ((uint64_t)out_cap_rows[r] > (uint64_t)INT64_MAX / row_bytes) return A2AV_EARG;
        if (in_rows[r] > 0 && in[r] == nullptr) return A2AV_EARG;
        if (out_cap_rows[r] > 0 && out[r] == nullptr) return A2AV_EARG;
        a.in[r] = (const unsigned char *)in[r];
        a.out[r] = (unsigned char *)out[r];
        a.in_rows[r] = in_rows[r];
        a.cap[r] = out_cap_rows[r];
        cap_bytes += (uint64_t)out_cap_rows[r] * row_bytes;
        if (cap_bytes > ((uint64_t)1 << 62)) return A2AV_EARG;
    }
    a.R = row_bytes;
    a.W = W;
    return A2AV_OK;
}

static int payload_grid(const CopyTuning &t, hipStream_t stream) {
    return device_cu_count(stream) * t.blocks_per_cu;
}

}  // namespace a2av

using namespace a2av;

// ====================================================================== C ABI
A2AV_API int a2av_abi_version(void) { return A2AV_ABI_VERSION; }

A2AV_API const char *a2av_strerror(int code) {
    switch (code) {
    case A2AV_OK: return "ok";
    case A2AV_EARG: return "invalid argument (nothing enqueued)";
    case A2AV_EHIP: return "HIP runtime refused a launch";
    case A2AV_ST_BAD_SPLIT: return "a split is negative or too large";
    case A2AV_ST_SEND_OVERRUN: return "a rank sends more rows than its input holds";
    case A2AV_ST_RECV_OVERFLOW: return "a rank receives more rows than its output holds";
    case A2AV_ST_BAD_EXPERT: return "an expert id is out of range";
    case A2AV_ST_BAD_OFFSETS: return "offsets are not the exclusive scans of the splits";
    case A2AV_ST_BAD_PERM: return "a permutation entry is out of range";
    default: return "unknown code";
    }
}

A2AV_API int a2av_exchange_splits(int W, const int64_t *S, int64_t *O, int32_t *status,
                                  hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || !S || !O || !status) return A2AV_EARG;
    if (W <= kWaveMaxW) hipLaunchKernelGGL(k_exchange_w8, dim3(1), dim3(kWave), 0, stream, W, S, O, status);
    else hipLaunchKernelGGL(k_exchange, dim3(1), dim3(256), 0, stream, W, S, O, status);
    return launch_status();
}

A2AV_API int a2av_offsets(int W, const int64_t *S, const int64_t *O, int64_t *send_off,
                          int64_t *recv_off, int32_t *status, hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || !S || !O || !send_off || !recv_off || !status) return A2AV_EARG;
    if (W <= kWaveMaxW) {
        hipLaunchKernelGGL(k_offsets_w8, dim3(1), dim3(kWave), 0, stream, W, S, O, send_off, recv_off,
                           status);
        return launch_status();
    }
    const int threads = 2 * W * kWave < 1024 ? 2 * W * kWave : 1024;
    hipLaunchKernelGGL(k_offsets, dim3(1), dim3(threads), 0, stream, W, S, O, send_off, recv_off,
                       status);
    return launch_status();
}

A2AV_API int a2av_copy(int W, size_t row_bytes, const void *const *in, const int64_t *in_rows,
                       void *const *out, const int64_t *out_cap_rows, const int64_t *S,
                       const int64_t *send_off, const int64_t *recv_off, int32_t *status,
                       hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || row_bytes == 0 || !in || !in_rows || !out || !out_cap_rows ||
        !S || !send_off || !recv_off || !status)
        return A2AV_EARG;
    CopyArgs a;
    const int rc = fill_buffers(a, W, row_bytes, in, in_rows, out, out_cap_rows);
    if (rc != A2AV_OK) return rc;
    a.S = S;
    a.send_off = send_off;
    a.recv_off = recv_off;
    a.status = status;
    const CopyTuning t = copy_tuning();
    a.min_piece = (uint64_t)t.min_piece;
    a.piece = (uint64_t)t.piece;
    if (!t.block_kernel) {
        uint64_t bmax;
        bool aligned;
        traffic_bound(a, &bmax, &aligned);
        const WaveTuning wt = W <= kWaveMaxW ? wave_tuning_w8(bmax)
                                             : wave_tuning_any(bmax, aligned);
        a.piece = wt.piece;
        if (W <= kWaveMaxW) launch_wave<kCopyGiven>(a, aligned, wt, wave_grid(bmax, wt.piece), stream);
        else launch_wave_any<false>(a, aligned, wt, wave_grid(bmax, wt.piece), stream);
        return launch_status();
    }
    const int grid = payload_grid(t, stream);
    if (W <= kMetaW) launch_payload<kCopyGiven>(a, grid, t, stream);
    else launch_payload<kCopyGlobal>(a, grid, t, stream);
    return launch_status();
}

A2AV_API int a2av_all_to_all_vdev(int W, size_t row_bytes, const void *const *in,
                                  const int64_t *in_rows, void *const *out,
                                  const int64_t *out_cap_rows, const int64_t *S, int64_t *O,
                                  int64_t *send_off, int64_t *recv_off, int32_t *status,
                                  hipStream_t stream) {
    if (W < 1 || W > A2AV_MAX_W || row_bytes == 0 || !in || !in_rows || !out || !out_cap_rows ||
        !S || !O || !send_off || !recv_off || !status)
        return A2AV_EARG;
    CopyArgs a;
    const int rc = fill_buffers(a, W, row_bytes, in, in_rows, out, out_cap_rows);
    if (rc != A2AV_OK) return rc;
    const CopyTuning t = copy_tuning();
    if (W > kWaveMaxW && !t.block_kernel) {
        a.S = S;
        a.O_out = O;
        a.send_off_out = send_off;
        a.recv_off_out = recv_off;
        a.status = status;
        uint64_t bmax;
        bool aligned;
        traffic_bound(a, &bmax, &aligned);
        const WaveTuning wt = wave_tuning_any(bmax, aligned);
        a.piece = wt.piece;
        launch_wave_any<true>(a, aligned, wt, wave_grid(bmax, wt.piece), stream);
        return launch_status();
    }
    if (W > kMetaW) {
        // the three steps as separate launches, in stream order
        int r = a2av_exchange_splits(W, S, O, status, stream);
        if (r == A2AV_OK) r = a2av_offsets(W, S, O, send_off, recv_off, status, stream);
        if (r == A2AV_OK)
            r = a2av_copy(W, row_bytes, in, in_rows, out, out_cap_rows, S, send_off, recv_off,
                          status, stream);
        return r;
    }
    a.S = S;
    a.O_out = O;
    a.send_off_out = send_off;
    a.recv_off_out = recv_off;
    a.status = status;
    a.min_piece = (uint64_t)t.min_piece;
    a.piece = (uint64_t)t.piece;
    if (W <= kWaveMaxW && !t.block_kernel) {
        uint64_t bmax;
        bool aligned;
        traffic_bound(a, &bmax, &aligned);
        const WaveTuning wt = wave_tuning_w8(bmax);
        a.piece = wt.piece;
        launch_wave<kFused>(a, aligned, wt, wave_grid(bmax, wt.piece), stream);
        return launch_status();
    }
    launch_payload<kFused>(a, payload_grid(t, stream), t, stream);
    return launch_status();
}

A2AV_API int a2av_device_read(const void *src, size_t bytes, uint64_t *sink, hipStream_t stream) {
    if (bytes == 0) return A2AV_OK;
    if (!src || !sink || bytes % 16 != 0 || (uintptr_t)src % 16 != 0) return A2AV_EARG;
    // the shapes of the plain copy moving as many bytes (read + write)
    const WaveTuning wt = wave_tuning(2 * (uint64_t)bytes, bytes >= kShortTraffic, true);
    const int grid = wave_grid(bytes, wt.piece);
    const unsigned char *s = (const unsigned char *)src;
    if (wt.unroll == 16)
        hipLaunchKernelGGL((k_device_read_wave<16>), dim3(grid), dim3(256), wt.lds, stream, s,
                           (uint64_t)bytes, wt.piece, sink);
    else if (wt.unroll == 4)
        hipLaunchKernelGGL((k_device_read_wave<4>), dim3(grid), dim3(256), wt.lds, stream, s,
                           (uint64_t)bytes, wt.piece, sink);
    else
        hipLaunchKernelGGL((k_device_read_wave<8>), dim3(grid), dim3(256), wt.lds, stream, s,
                           (uint64_t)bytes, wt.piece, sink);
    return launch_status();
}

A2AV_API int a2av_device_fill(void *dst, size_t bytes, uint32_t pattern, int nontemporal,
                              hipStream_t stream) {
    if (bytes == 0) return A2AV_OK;
    if (!dst || bytes % 16 != 0 || (uintptr_t)dst % 16 != 0) return A2AV_EARG;
    const WaveTuning wt = wave_tuning(2 * (uint64_t)bytes, bytes >= kShortTraffic, true);
    const int grid = wave_grid(bytes, wt.piece);
    unsigned char *d = (unsigned char *)dst;
#define A2AV_FILL(U)                                                                            \
    if (nontemporal)                                                                            \
        hipLaunchKernelGGL((k_device_fill_wave<U, true>), dim3(grid), dim3(256), wt.lds, stream, \
                           d, (uint64_t)bytes, wt.piece, pattern);                              \
    else                                                                                        \
        hipLaunchKernelGGL((k_device_fill_wave<U, false>), dim3(grid), dim3(256), wt.lds,        \
                           stream, d, (uint64_t)bytes, wt.piece, pattern);
    if (wt.unroll == 16) {
        A2AV_FILL(16)
    } else if (wt.unroll == 4) {
        A2AV_FILL(4)
    } else {
        A2AV_FILL(8)
    }
#undef A2AV_FILL
    return launch_status();
}

A2AV_API int a2av_device_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return A2AV_OK;
    if (!dst || !src) return A2AV_EARG;
    const CopyTuning t = copy_tuning();
    if (!t.block_kernel) {
        const bool aligned = ((uintptr_t)dst % 16 == 0) && ((uintptr_t)src % 16 == 0) && bytes % 16 == 0;
        // the same shapes as the one-call a2av moving as many bytes
        const WaveTuning wt = wave_tuning(2 * (uint64_t)bytes, aligned && bytes >= kShortTraffic, true);
        const int grid = wave_grid(bytes, wt.piece);
        unsigned char *d = (unsigned char *)dst;
        const unsigned char *s = (const unsigned char *)src;
        if (!aligned)
            hipLaunchKernelGGL((k_device_copy_wave<8, false>), dim3(grid), dim3(256), 0, stream, d, s,
                               (uint64_t)bytes, wt.piece);
        else if (wt.unroll == 16)
            hipLaunchKernelGGL((k_device_copy_wave<16, true>), dim3(grid), dim3(256), wt.lds, stream,
                               d, s, (uint64_t)bytes, wt.piece);
        else if (wt.unroll == 4)
            hipLaunchKernelGGL((k_device_copy_wave<4, true>), dim3(grid), dim3(256), wt.lds, stream,
                               d, s, (uint64_t)bytes, wt.piece);
        else
            hipLaunchKernelGGL((k_device_copy_wave<8, true>), dim3(grid), dim3(256), wt.lds, stream,
                               d, s, (uint64_t)bytes, wt.piece);
        return launch_status();
    }
    const int grid = payload_grid(t, stream);
    unsigned char *d = (unsigned char *)dst;
    const unsigned char *s = (const unsigned char *)src;
    switch (t.unroll) {
    case 1: launch_dcopy_u<256, 1>(d, s, bytes, t, grid, stream); break;
    case 2: launch_dcopy_u<256, 2>(d, s, bytes, t, grid, stream); break;
    case 8: launch_dcopy_u<256, 8>(d, s, bytes, t, grid, stream); break;
    default: launch_dcopy_u<256, 4>(d, s, bytes, t, grid, stream); break;
    }
    return launch_status();
}
