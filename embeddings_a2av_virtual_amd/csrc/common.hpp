// common.hpp — device helpers shared by the a2av and MoE kernels (gfx950).
//
// Wave64 scans and the cooperative contiguous byte copy that every payload
// kernel uses. Written for CDNA wavefronts of 64 lanes: one 16-byte access per
// lane gives a fully coalesced 1 KiB per wave instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/a2av.h"

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

// ------------------------------------------------------------ wave64 scans
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int64_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ int32_t wave_incl_scan32(int32_t v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int32_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
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

// Block-cooperative copy of nv elements of V: thread `tid` of BS moves
// elements tid, tid + BS, ...; U loads are issued before their U stores so
// each lane keeps U accesses in flight.
template <typename V, int BS, int U, bool NT>
__device__ __forceinline__ void copy_elems(V *__restrict__ d, const V *__restrict__ s,
                                           uint64_t nv, int tid) {
    uint64_t i = (uint64_t)tid;
    constexpr uint64_t step = (uint64_t)BS * U;
    for (; i + (uint64_t)(U - 1) * BS < nv; i += step) {
        V r[U];
#pragma unroll
        for (int u = 0; u < U; u++) r[u] = ld<NT>(s + i + (uint64_t)u * BS);
#pragma unroll
        for (int u = 0; u < U; u++) st<NT>(d + i + (uint64_t)u * BS, r[u]);
    }
    for (; i < nv; i += BS) st<NT>(d + i, ld<NT>(s + i));
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

// ------------------------------------------------------------ host helpers
int device_cu_count(hipStream_t stream);
long env_long(const char *name, long dflt, long lo, long hi);

}  // namespace a2av
