// mk_device.h -- gfx950 device primitives for the MoE megakernel: agent-scope event
// counters, wave64 exchanges, bf16 helpers and the bf16 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_common.h"

namespace mk {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round to nearest even (finite values; NaN keeps a NaN pattern).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// ---------------------------------------------------------------------------- atomics
// Event counters and every value one task publishes to another live in device memory
// shared by the 8 XCDs, whose L2 caches are not coherent with each other.  Published
// values are therefore written with agent-scope stores (coherent across XCDs: the
// same instruction the compiler uses for a relaxed agent-scope atomic store), so a
// notification needs no L2 write-back: each wave waits for its stores to complete
// (vmcnt 0), the workgroup synchronises, then one thread updates the counter.  A wait
// polls the counter with agent-scope loads and ends with an agent-scope acquire fence,
// which invalidates the CU's L1 and the XCD's non-coherent L2 lines.  (An agent-scope
// release fence would write back the whole L2 on every notification; measured on
// MI355X it costs several microseconds per task, the acquire a fraction of one.)

__device__ __forceinline__ int ld_relaxed(const MK_G int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(MK_G int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_relaxed(MK_G int *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same without a reply: the wave goes on without waiting for the atomic to be performed.
__device__ __forceinline__ void add_relaxed_noret(MK_G int *p, int v) {
    (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Wait until this wave's outstanding vector memory operations (stores included) completed.
__device__ __forceinline__ void wave_drain_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); /* vmcnt(0) */ }

// Publishing stores (agent scope).
__device__ __forceinline__ void pub(MK_G int *p, int v) { st_relaxed(p, v); }
__device__ __forceinline__ void pub(MK_G float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub(MK_G uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long ld_relaxed64(const MK_G unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed64(MK_G unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_error(MK_G int *ctl, int bits) {
    __hip_atomic_fetch_or(ctl + CTL_ERR, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Spin (one thread) until *p == target.  Returns false when the error word is set or the
// watchdog expires (which also sets the error word), so callers never hang.
__device__ __forceinline__ bool spin_until(const MK_G int *p, int target, MK_G int *ctl, long long watchdog) {
    if (ld_relaxed(p) == target) return true;
    const unsigned long long t0 = now_ticks();
    for (unsigned it = 1;; ++it) {
        // back off after a while: hundreds of idle workgroups polling one counter would
        // otherwise crowd the memory channel it lives on
        if (it < 64)
            __builtin_amdgcn_s_sleep(1);
        else
            __builtin_amdgcn_s_sleep(8);
        if (ld_relaxed(p) == target) return true;
        if ((it & 31u) == 0) {
            if (ld_relaxed(ctl + CTL_ERR) != 0) return false;
            if ((long long)(now_ticks() - t0) > watchdog) {
                set_error(ctl, 1 /* MOE_MK_ERR_WATCHDOG */);
                return false;
            }
        }
    }
}

// ---------------------------------------------------------------------------- wave64
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
// A value every lane of the wave holds alike, made visibly wave-uniform for the compiler
// (arguments of out-of-line functions arrive in vector registers; branching on them
// would otherwise be compiled as divergent, with accumulators copied at every join).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// wave index within the workgroup, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
        unsigned olo = (unsigned)__shfl_xor((int)lo, m, 64);
        unsigned ohi = (unsigned)__shfl_xor((int)hi, m, 64);
        unsigned long long o = ((unsigned long long)ohi << 32) | olo;
        v = o > v ? o : v;
    }
    return v;
}

// Order-preserving map of a float (with -0 folded onto +0 beforehand) to uint32.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace mk
