// common.hpp — device helpers shared by the a2av and MoE kernels (gfx950).
//
// Wave64 scans and the cooperative contiguous byte copy that every payload
// kernel uses. Written for CDNA wavefronts of 64 lanes: one 16-byte access per
// lane gives a fully coalesced 1 KiB per wave instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/a2av.h"
#include "bounds.h"

#define A2AV_API extern "C" __attribute__((visibility("default")))

namespace a2av {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------ status word
// The word is read once at kernel entry; a nonzero value means an earlier op
// on the same word failed and this one must not write anything.
__device__ __forceinline__ int status_poisoned(const int32_t *status) {
    return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ bool split_invalid(int64_t v) {
    return v < 0 || v > A2AV_MAX_SPLIT;
}

// ------------------------------------------------------------ loads / stores
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V *p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// A check run once by copy_elems between the loads and the stores of its
// first step (see below); the default lets every store through.
struct NoGate {
    __device__ __forceinline__ bool operator()() const { return true; }
};

// Cooperative copy of nv elements of V by BS threads: thread `tid` moves
// elements tid, tid + BS, ...; each step issues U loads before their U
// stores, so every lane keeps U accesses in flight. Full steps carry no
// per-lane guard. The last, partial step clamps the index to nv - 1 instead
// of branching: a lane past the end re-copies the last element, and every
// such lane writes the same bytes to the same place. (Guards in this loop
// make the compiler wait for each load before the next one.)
//
// With a gate, the first step's loads are issued before the gate runs and
// nothing is stored unless it returns true (then the copy returns false);
// a check that waits on loads of its own thus overlaps the first payload
// loads. Every thread must get the same verdict.
template <typename V, int BS, int U, bool NT, typename Gate = NoGate>
__device__ __forceinline__ bool copy_elems(V *__restrict__ d, const V *__restrict__ s,
                                           uint64_t nv, int tid, Gate gate = Gate()) {
    constexpr bool kGated = !std::is_same<Gate, NoGate>::value;
    constexpr uint64_t step = (uint64_t)BS * U;
    bool first = kGated;
    uint64_t base = 0;
    for (; base + step <= nv; base += step) {
        V r[U];
#pragma unroll
        for (int u = 0; u < U; u++) r[u] = ld<NT>(s + base + (uint64_t)u * BS + tid);
        if constexpr (kGated) {
            if (first) {
                __builtin_amdgcn_sched_barrier(0);
                first = false;
                if (!gate()) return false;
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) st<NT>(d + base + (uint64_t)u * BS + tid, r[u]);
    }
    if (base < nv) {
        V r[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t i = base + (uint64_t)u * BS + tid;
            r[u] = ld<NT>(s + (i < nv ? i : nv - 1));
        }
        if constexpr (kGated) {
            if (first) {
                __builtin_amdgcn_sched_barrier(0);
                first = false;
                if (!gate()) return false;
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t i = base + (uint64_t)u * BS + tid;
            st<NT>(d + (i < nv ? i : nv - 1), r[u]);
        }
    }
    if constexpr (kGated) {
        if (first) return gate();  // nothing to copy: the verdict still counts
    }
    return true;
}

// Block-cooperative copy of n bytes between non-overlapping device ranges.
// The widest width w in {16, 8, 4, 2, 1} with src == dst (mod w) is used for
// the body; a head of < w bytes brings dst to a multiple of w and a tail of
// < w bytes finishes. All threads of the block must call it with the same
// arguments.
template <int BS, int U, bool NT>
__device__ __forceinline__ void copy_segment(unsigned char *dst, const unsigned char *src,
                                             uint64_t n, int tid) {
    const uintptr_t mis = (uintptr_t)dst ^ (uintptr_t)src;
    const uint64_t w = (mis & 15) == 0 ? 16 : (mis & 7) == 0 ? 8 : (mis & 3) == 0 ? 4
                     : (mis & 1) == 0 ? 2 : 1;
    uint64_t head = (w - ((uintptr_t)dst & (w - 1))) & (w - 1);
    if (head > n) head = n;
    if ((uint64_t)tid < head) dst[tid] = src[tid];
    dst += head;
    src += head;
    n -= head;
    const uint64_t nv = n / w;
    switch (w) {
    case 16: copy_elems<u32x4, BS, U, NT>((u32x4 *)dst, (const u32x4 *)src, nv, tid); break;
    case 8: copy_elems<u32x2, BS, U, NT>((u32x2 *)dst, (const u32x2 *)src, nv, tid); break;
    case 4: copy_elems<uint32_t, BS, U, NT>((uint32_t *)dst, (const uint32_t *)src, nv, tid); break;
    case 2: copy_elems<uint16_t, BS, U, NT>((uint16_t *)dst, (const uint16_t *)src, nv, tid); break;
    default: copy_elems<uint8_t, BS, U, NT>(dst, src, nv, tid); break;
    }
    const uint64_t done = nv * w;
    if ((uint64_t)tid < n - done) dst[done + tid] = src[done + tid];
}

// Funnel 16 bytes out of the 32-byte pair (a, b) starting at byte `delta`
// (1..15): dword j of the result is bytes [delta + 4j, delta + 4j + 4).
__device__ __forceinline__ u32x4 funnel16(const u32x4 &a, const u32x4 &b, uint32_t delta) {
    const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint32_t q = delta >> 2, sh = delta & 3;
    u32x4 o;
    // q and sh are the same in every lane, so the branches do not diverge
#define A2AV_FUNNEL(Q)                                                                       \
    if (sh == 0) {                                                                         \
        o.x = c[Q]; o.y = c[Q + 1]; o.z = c[Q + 2]; o.w = c[Q + 3];                       \
    } else {                                                                               \
        o.x = __builtin_amdgcn_alignbyte(c[Q + 1], c[Q], sh);                              \
        o.y = __builtin_amdgcn_alignbyte(c[Q + 2], c[Q + 1], sh);                          \
        o.z = __builtin_amdgcn_alignbyte(c[Q + 3], c[Q + 2], sh);                          \
        o.w = __builtin_amdgcn_alignbyte(c[Q + 4], c[Q + 3], sh);                          \
    }
    switch (q) {
    case 0: A2AV_FUNNEL(0) break;
    case 1: A2AV_FUNNEL(1) break;
    case 2: A2AV_FUNNEL(2) break;
    default: A2AV_FUNNEL(3) break;
    }
#undef A2AV_FUNNEL
    return o;
}

// A 16-byte vector that is only known to be 4-byte aligned. Global loads of
// it are still single 16-byte loads (gfx950 needs dword alignment for them).
typedef unsigned int u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// copy_elems with the loads at a source that is 4-byte but not 16-byte
// aligned: one 16-byte load per 16-byte aligned store, reading exactly the
// source range.
template <int U>
__device__ __forceinline__ void copy_elems_dw(u32x4 *__restrict__ d, const u32x4_a4 *__restrict__ s,
                                              uint64_t nv, int lane) {
    constexpr uint64_t step = (uint64_t)kWave * U;
    for (uint64_t base = 0; base < nv; base += step) {
        u32x4_a4 r[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            uint64_t i = base + (uint64_t)u * kWave + lane;
            i = i < nv ? i : nv - 1;
            // the builtin on the 4-byte-aligned type itself: through ld<>
            // the type would decay to the 16-byte-aligned vector
            r[u] = __builtin_nontemporal_load(s + i);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            uint64_t i = base + (uint64_t)u * kWave + lane;
            i = i < nv ? i : nv - 1;
            st<true>(d + i, (u32x4)r[u]);
        }
    }
}

// Wave-cooperative copy of n bytes at any alignment (64 lanes, all calling
// with the same arguments). A head of < 16 bytes brings the destination to a
// 16-byte boundary; then every lane stores one aligned 16-byte block per
// step. Its source bytes come from one 16-byte load at their own address when
// that address is 4-byte aligned (as fast as an aligned copy; the two-load
// form below costs about 8 % of bandwidth); otherwise they are cut out of the
// two aligned 16-byte source blocks that hold them (the second one is the
// block its right neighbour loads, so it comes from cache). Every source
// block read holds at least one byte of the source range, so no read leaves
// the pages the range lives on. The last step clamps its index like
// copy_elems; the tail of < 16 bytes goes byte by byte.
template <int U>
__device__ __forceinline__ void wave_copy_any(unsigned char *dst, const unsigned char *src,
                                              uint64_t n, int lane) {
    uint64_t head = (16 - ((uintptr_t)dst & 15)) & 15;
    if (head > n) head = n;
    if ((uint64_t)lane < head) dst[lane] = src[lane];
    dst += head;
    src += head;
    n -= head;
    const uint64_t nv = n / 16;
    const uint32_t delta = (uint32_t)((uintptr_t)src & 15);
    u32x4 *d16 = (u32x4 *)dst;
    if (delta == 0) {
        copy_elems<u32x4, kWave, U, true>(d16, (const u32x4 *)src, nv, lane);
    } else if ((delta & 3) == 0) {
        copy_elems_dw<U>(d16, (const u32x4_a4 *)src, nv, lane);
    } else if (nv > 0) {
        const u32x4 *sa = (const u32x4 *)(src - delta);
        for (uint64_t base = 0; base < nv; base += (uint64_t)kWave * U) {
            u32x4 lo[U], hi[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                uint64_t i = base + (uint64_t)u * kWave + lane;
                i = i < nv ? i : nv - 1;
                lo[u] = ld<true>(sa + i);
                hi[u] = ld<true>(sa + i + 1);  // block nv still holds source bytes
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                uint64_t i = base + (uint64_t)u * kWave + lane;
                i = i < nv ? i : nv - 1;
                st<true>(d16 + i, funnel16(lo[u], hi[u], delta));
            }
        }
    }
    const uint64_t done = nv * 16;
    if ((uint64_t)lane < n - done) dst[done + lane] = src[done + lane];
}

// Wave-cooperative copy of n bytes, n a multiple of 16, both ends 16-aligned.
// With a gate, as copy_elems: false (and nothing stored) when it refuses.
template <int U, typename Gate = NoGate>
__device__ __forceinline__ bool wave_copy16(unsigned char *dst, const unsigned char *src,
                                            uint64_t n, int lane, Gate gate = Gate()) {
    return copy_elems<u32x4, kWave, U, true>((u32x4 *)dst, (const u32x4 *)src, n / 16, lane, gate);
}

// ------------------------------------------------------------ wave-uniform values
// Pointers into the constant address space: loads through them that the
// compiler can prove uniform become scalar loads, which do not queue behind
// the wave's vector memory traffic.
typedef __attribute__((address_space(4))) const int64_t const_i64;
typedef __attribute__((address_space(4))) const int32_t const_i32;

// The entry off bytes past p, through the scalar cache: a scalar load with a
// register offset, so that a burst of loads from one array at computed
// offsets needs one address pair, not one per load.
__device__ __forceinline__ int64_t at_byte(const const_i64 *p, uint32_t off) {
    typedef __attribute__((address_space(4))) const char const_c;
    return *(const const_i64 *)((const const_c *)p + off);
}
__device__ __forceinline__ int32_t at_byte(const const_i32 *p, uint32_t off) {
    typedef __attribute__((address_space(4))) const char const_c;
    return *(const const_i32 *)((const const_c *)p + off);
}

// The status word as a wave finds it at entry, read once through the scalar
// cache (a uniform load that does not queue behind the vector traffic older
// waves keep in flight on the CU). The constant address space tells the
// compiler the word does not change during the kernel, which is not so:
// waves of the same launch may OR failure bits into it. The read is still
// exact for its one use, an early return before the wave writes anything:
// whatever the compiler does with a single-use load, the value it yields is
// what earlier kernels left (their writes are visible at kernel start),
// possibly with bits a wave of this launch has set since. The kernels that
// call this have every wave make those checks itself and reach the same
// verdict, so returning early on such bits changes nothing. A kernel whose
// waves could disagree reads the word with status_poisoned instead.
__device__ __forceinline__ int32_t status_at_entry(const int32_t *status) {
    return *(const const_i32 *)status;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}


// ------------------------------------------------------------ lanes, DPP and bursts
// x of the lane O below in the same 16-lane row (0 for the first O lanes of
// a row); every lane must be active.
template <int O>
__device__ __forceinline__ uint64_t dpp_row_shr(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, 0x110 + O, 0xf, 0xf, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), 0x110 + O, 0xf, 0xf, true);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan inside aligned groups of P lanes (P = 1, 2, 4, 8 or 16); k
// is the lane's index in its group. A lane adds the value O lanes below only
// when that lane is in its own group, which is then in its own DPP row.
template <int P>
__device__ __forceinline__ uint64_t group_incl_scan(uint64_t x, int k) {
    static_assert(P == 1 || P == 2 || P == 4 || P == 8 || P == 16, "groups inside a DPP row");
    if constexpr (P > 1) {
        const uint64_t t = dpp_row_shr<1>(x);
        if (k >= 1) x += t;
    }
    if constexpr (P > 2) {
        const uint64_t t = dpp_row_shr<2>(x);
        if (k >= 2) x += t;
    }
    if constexpr (P > 4) {
        const uint64_t t = dpp_row_shr<4>(x);
        if (k >= 4) x += t;
    }
    if constexpr (P > 8) {
        const uint64_t t = dpp_row_shr<8>(x);
        if (k >= 8) x += t;
    }
    return x;
}

// x of the last lane of the row before (DPP row_bcast: lane 15 into row 1
// and lane 47 into row 3 for ROWS = 0xa; lane 31 into rows 2 and 3 for
// ROWS = 0xc), 0 in the other rows; every lane must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_row_bcast(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, ROWS, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan over the 64 lanes: inside each 16-lane row, then the rows'
// totals carried forward (lane 15 into row 1, lane 31 into rows 2 and 3,
// lane 47 into row 3); DPP moves only, no LDS round trip. Every lane must be
// active.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
    const int lane = threadIdx.x & (kWave - 1);
    x = group_incl_scan<16>(x, lane & 15);
    x += dpp_row_bcast<0x142, 0xa>(x);
    x += dpp_row_bcast<0x143, 0xc>(x);
    return x;
}

// The same for signed values (the sum modulo 2^64 is the same bits).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
    return (int64_t)wave_incl_scan_u64((uint64_t)v);
}

// The same for 32-bit values.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    const int k = threadIdx.x & 15;
    uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    if (k >= 1) x += t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    if (k >= 2) x += t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    if (k >= 4) x += t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
    if (k >= 8) x += t;
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
    return x;
}

// x of lane src (any lane; every lane must be active).
__device__ __forceinline__ uint64_t lane_gather(uint64_t x, int src) {
    const int addr = src << 2;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// v_writelane_b32 (this compiler has no builtin for it): old with lane l set
// to the uniform value val.
__device__ int amdgcn_writelane(int val, int l, int old) __asm("llvm.amdgcn.writelane.i32");

// Sixteen 64-bit values of array t from index o, as scalar-register operands
// of an asm statement.
#define A2AV_SREG16(t, o)                                                                        \
    "s"(t[o + 0]), "s"(t[o + 1]), "s"(t[o + 2]), "s"(t[o + 3]), "s"(t[o + 4]), "s"(t[o + 5]),       \
        "s"(t[o + 6]), "s"(t[o + 7]), "s"(t[o + 8]), "s"(t[o + 9]), "s"(t[o + 10]), "s"(t[o + 11]), \
        "s"(t[o + 12]), "s"(t[o + 13]), "s"(t[o + 14]), "s"(t[o + 15])

// The same as operands the asm statement reads and writes: what uses the
// values afterwards cannot be scheduled before the statement, so no use of
// an early value splits the burst with a wait for the loads issued so far.
#define A2AV_SREG16_IO(t, o)                                                                     \
    "+s"(t[o + 0]), "+s"(t[o + 1]), "+s"(t[o + 2]), "+s"(t[o + 3]), "+s"(t[o + 4]),                \
        "+s"(t[o + 5]), "+s"(t[o + 6]), "+s"(t[o + 7]), "+s"(t[o + 8]), "+s"(t[o + 9]),            \
        "+s"(t[o + 10]), "+s"(t[o + 11]), "+s"(t[o + 12]), "+s"(t[o + 13]), "+s"(t[o + 14]),       \
        "+s"(t[o + 15])

#define A2AV_SREG4(t, o) "s"(t[o + 0]), "s"(t[o + 1]), "s"(t[o + 2]), "s"(t[o + 3])
#define A2AV_SREG8(t, o)                                                                        \
    "s"(t[o + 0]), "s"(t[o + 1]), "s"(t[o + 2]), "s"(t[o + 3]), "s"(t[o + 4]), "s"(t[o + 5]),       \
        "s"(t[o + 6]), "s"(t[o + 7])

// v with lane l (a constant) set to the uniform value x.
__device__ __forceinline__ uint64_t writelane_u64(uint64_t v, uint64_t x, int l) {
    const uint32_t lo = (uint32_t)amdgcn_writelane((int)(uint32_t)x, l, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)amdgcn_writelane((int)(uint32_t)(x >> 32), l, (int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------ bfloat16
// The two bf16 halves of a 32-bit word as fp32 (bf16 is the top half of an
// IEEE binary32).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// float -> bfloat16 bits, round to nearest even; every NaN becomes 0x7FC0
// (the sign and payload of a NaN result are not fixed by IEEE 754 and differ
// between processors).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------ piece boundaries
// A flat position of the destination space (destination d's bytes start at
// start_d, held by lane d*P + Q) moved up to the next 128-byte boundary of its
// destination's address, or to that destination's end; 0 and B stay put.
template <int P = 1, int Q = 0>
__device__ __forceinline__ uint64_t snap_to_line(uint64_t x, uint64_t B, uint64_t start_d,
                                                 int lane, int W, unsigned char *const *out) {
    if (x == 0 || x >= B) return x < B ? x : B;
    const uint64_t md = __ballot(lane % P == Q && lane / P < W && start_d <= x);
    const int d = (63 - __clzll(md)) / P;
    const uint64_t db = readlane_u64(start_d, d * P + Q);
    const uint64_t de = d + 1 < W ? readlane_u64(start_d, (d + 1) * P + Q) : B;
    const uint64_t addr = (uint64_t)(uintptr_t)out[d] + (x - db);
    const uint64_t up = ((addr + 127) & ~(uint64_t)127) - addr;
    return x + up < de ? x + up : de;
}

// ------------------------------------------------------------ block scans
// Plans run one 1024-thread workgroup per rank, each thread owning up to
// kPlanPer consecutive entries (4096 per rank at most).
constexpr int kPlanThreads = 1024;
constexpr int kPlanPer = 4;

// Two exclusive scans over the workgroup at once, with both totals.
struct ScanLds {
    int64_t a[kPlanThreads / kWave];
    int64_t b[kPlanThreads / kWave];
};

__device__ __forceinline__ void block_excl_scan2(int64_t va, int64_t vb, ScanLds &l,
                                                 int64_t *ea, int64_t *eb, int64_t *ta, int64_t *tb) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NW = kPlanThreads / kWave;
    const int64_t ia = wave_incl_scan(va), ib = wave_incl_scan(vb);
    if (lane == kWave - 1) {
        l.a[wv] = ia;
        l.b[wv] = ib;
    }
    __syncthreads();
    int64_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        const int64_t xa = l.a[w], xb = l.b[w];
        if (w < wv) {
            pa += xa;
            pb += xb;
        }
        sa += xa;
        sb += xb;
    }
    __syncthreads();  // the arrays may be reused by the caller
    *ea = pa + ia - va;
    *eb = pb + ib - vb;
    *ta = sa;
    *tb = sb;
}

// Three exclusive scans over the workgroup at once, with their totals.
struct ScanLds3 {
    int64_t v[3][kPlanThreads / kWave];
};

__device__ __forceinline__ void block_excl_scan3(const int64_t (&v)[3], ScanLds3 &l,
                                                 int64_t (&ex)[3], int64_t (&tot)[3]) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int NW = kPlanThreads / kWave;
    int64_t inc[3];
#pragma unroll
    for (int i = 0; i < 3; i++) {
        inc[i] = wave_incl_scan(v[i]);
        if (lane == kWave - 1) l.v[i][wv] = inc[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 3; i++) {
        int64_t pre = 0, sum = 0;
#pragma unroll 4
        for (int w = 0; w < NW; w++) {
            const int64_t x = l.v[i][w];
            pre += w < wv ? x : 0;
            sum += x;
        }
        ex[i] = pre + inc[i] - v[i];
        tot[i] = sum;
    }
    __syncthreads();  // the arrays may be reused by the caller
}

// ------------------------------------------------------------ host helpers
int device_cu_count(hipStream_t stream);
long env_long(const char *name, long dflt, long lo, long hi);
unsigned max_grid();

}  // namespace a2av
