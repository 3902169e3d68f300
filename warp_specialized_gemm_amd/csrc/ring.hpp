// ring.hpp - the full/empty LDS ring protocol shared by the staged copy and
// the GEMM kernels (device code, gfx950).
//
// Protocol (three web pages on warp specialization):
//   * a ring of S LDS slots; tile t uses slot t mod S ("Producer-Consumer
//     Warp Specialization for TMA Operations" enumerates tiles 0, 1, 2, 3 over
//     buffers 0, 1, 0, 1; the pwwt.cn article, section 3.4, writes
//     tile % stages);
//   * every slot has a "full" flag (data landed) and an "empty" flag (data
//     drained); one flag per slot is not enough (pwwt.cn section 3.4);
//   * a flag counts arrivals against an expected number and, on the last
//     one, completes a phase (pwwt.cn section 2.2, the mbarrier as a counter);
//   * wait(p) proceeds once the phase of parity p has completed, i.e. once the
//     phase bit differs from p; consumers of tile t wait "full" with
//     p = (t / S) & 1 (the same post, phase-bit paragraphs);
//   * producers wait "empty" for the release of tile t - S, i.e. with parity
//     ((t / S) & 1) ^ 1, which passes at once on the first lap.
//
// gfx950 has neither TMA nor mbarrier: a flag is one 32-bit LDS word.
//   bits [15:0]  arrivals in the current phase
//   bits [31:16] completed phases (mod 2^16); bit 16 is the phase bit.
// The last arrival adds (1 << 16) - expected, which clears the count and
// flips the phase bit in one add. Waves of one workgroup are co-resident, so
// spinning on an LDS word is safe; every wait is bounded and records a
// timeout in a device status word instead of hanging.
//
// Flag accesses are inline assembly with their own lgkmcnt wait. The
// compiler treats any LDS access that follows an LDS-DMA load as possibly
// aliasing it and puts a vmcnt(0) in front, which would drain the producer's
// loads in flight; the assembly keeps those loads outstanding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

constexpr uint32_t kFlagCountMask = 0xFFFFu;
constexpr uint32_t kPhaseOne = 1u << 16;
constexpr uint32_t kSpinLimit = 1u << 25;  // about a second of polling
constexpr int kFlagBytes = 256;            // LDS bytes reserved for flags at offset 0
constexpr int kMaxStages = 32;             // full[32] + empty[32] words fit in kFlagBytes

// device status word bits
constexpr unsigned kStatusTimeout = 1u;
constexpr unsigned kStatusCopy = 2u;
constexpr unsigned kStatusGemm = 4u;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}

__device__ __forceinline__ uint32_t flag_load(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// full[s] at 4*s, empty[s] at 128 + 4*s
__device__ __forceinline__ uint32_t full_flag(uint32_t base, int s) { return base + 4u * (uint32_t)s; }
__device__ __forceinline__ uint32_t empty_flag(uint32_t base, int s) { return base + 128u + 4u * (uint32_t)s; }

// Proceed once the phase bit of the flag differs from `parity`. Returns false
// (after recording the timeout) when the wait gives up.
__device__ __forceinline__ bool flag_wait(uint32_t addr, uint32_t parity, unsigned *status, unsigned who) {
    uint32_t spins = 0;
    while (true) {
        uint32_t v = __builtin_amdgcn_readfirstlane(flag_load(addr));
        if (((v >> 16) & 1u) != parity) return true;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
            if ((threadIdx.x & 63) == 0) atomicOr(status, kStatusTimeout | who);
            return false;
        }
    }
}

// One arrival of the calling wave (lane 0 does the atomic). The caller has
// already waited for the wave's own LDS writes or reads of the slot.
__device__ __forceinline__ void flag_arrive(uint32_t addr, uint32_t expected) {
    if ((threadIdx.x & 63) != 0) return;
    if (expected == 1) {
        asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(kPhaseOne) : "memory");
        return;
    }
    uint32_t old;
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(old)
                 : "v"(addr), "v"(1u)
                 : "memory");
    if ((old & kFlagCountMask) == expected - 1) {
        asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(kPhaseOne - expected)
                     : "memory");
    }
}

// All of this wave's LDS operations done. The builtin (not inline assembly)
// lets the compiler's own wait insertion see it, so later uses of registers
// loaded before it need no further wait.
__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt(0), vmcnt and expcnt unconstrained
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt needs an immediate; dispatch a wave-uniform count.
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    if constexpr (N >= 63) {
        wait_vmcnt<63>();
    } else {
        if (n <= N) {
            wait_vmcnt<N>();
        } else {
            wait_vmcnt_dyn<N + 1>(n);
        }
    }
}

// Buffer resource over [base, base + num_records) bytes. Loads at offsets
// past num_records return zeros without touching memory (used for masking).
// Word 3 is the raw-buffer format for gfx9-family devices.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_records, 0x00020000);
}

constexpr uint32_t kOobOffset = 0x80000000u;  // above any num_records the library builds

// 16 bytes per lane, global -> LDS without passing through VGPRs. Lane l's
// data lands at lds_wave_base + 16 * l (lds_wave_base is wave-uniform).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, void *lds_wave_base, uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds_wave_base, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace wsg
