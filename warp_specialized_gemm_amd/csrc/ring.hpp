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
// gfx950 has neither TMA nor mbarrier: a flag is one 32-bit LDS word that
// counts arrivals. Expected arrival counts are powers of two (E = 1, 2, 4, 8
// waves), so E arrivals complete a phase exactly when bit log2(E) of the
// counter flips: that bit is the phase bit. An arrival is then a single
// LDS add with no return value and nothing to wait for. Waves of one
// workgroup are co-resident, so spinning on an LDS word is safe; every wait
// is bounded and records a timeout in a device status word instead of
// hanging.
//
// Producer-side flag accesses are inline assembly with their own lgkmcnt
// wait: the compiler treats any LDS access that follows an LDS-DMA load as
// possibly aliasing it and puts a vmcnt(0) in front, which would drain the
// loads in flight. Consumers, which issue no LDS-DMA, may also read a flag
// ahead of time with an ordinary atomic load and test it later.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

constexpr uint32_t kSpinLimit = 1u << 25;  // about a second of polling
constexpr int kFlagBytes = 256;            // LDS bytes reserved for flags at offset 0
constexpr int kMaxStages = 32;             // full[32] + empty[32] words fit in kFlagBytes

// wait statistics layout (unsigned long long[16]): each block of three is
// {waits, waits that found the flag unflipped, polls}
constexpr int kStatGemmConsumer = 0;  // full waits of GEMM consumers (early flag reads count as waits)
constexpr int kStatGemmProducer = 3;  // empty waits of GEMM producers
constexpr int kStatCopyConsumer = 6;
constexpr int kStatCopyProducer = 9;
constexpr int kStatAttnConsumer = 12;  // full waits of attention consumers
constexpr int kStatWords = 16;

// device status word bits
constexpr unsigned kStatusTimeout = 1u;
constexpr unsigned kStatusCopy = 2u;
constexpr unsigned kStatusGemm = 4u;
constexpr unsigned kStatusAttention = 8u;

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

template <int E>
constexpr int log2_arrivals() {
    static_assert(E == 1 || E == 2 || E == 4 || E == 8 || E == 16, "expected arrivals must be a power of two");
    return E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : E == 8 ? 3 : 4;
}

// Phase bit of a flag word whose phases complete every E arrivals.
template <int E>
__device__ __forceinline__ uint32_t phase_of(uint32_t word) {
    return (word >> log2_arrivals<E>()) & 1u;
}

// Per-wave count of flag waits, kept in registers: how many waits there
// were, how many found the flag not yet flipped, and how many polls those
// took. Written out only when the host asks for wait statistics.
struct WaitTally {
    uint32_t waits = 0, blocked = 0, polls = 0;
};

// Proceed once the phase bit differs from `parity`, i.e. once the phase of
// that parity has completed. Returns false (after recording the timeout)
// when the wait gives up.
// `poll` returns the flag word (wave-uniform).
// RECORD = false leaves the status word to the caller, which records the
// timeout once outside its loop (so the loop keeps no registers for it).
template <int E, bool RECORD = true, typename Poll>
__device__ __forceinline__ bool flag_wait_with(Poll poll, uint32_t parity, unsigned *status, unsigned who,
                                               WaitTally &tally) {
    uint32_t spins = 0;
    ++tally.waits;
    while (true) {
        const uint32_t v = poll();
        if (phase_of<E>(v) != parity) {
            tally.blocked += spins != 0;
            tally.polls += spins;
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
            if constexpr (RECORD) atomicOr(status, kStatusTimeout | who);  // every lane: keeps the loop uniform
            return false;
        }
    }
}

template <int E, bool RECORD = true>
__device__ __forceinline__ bool flag_wait(uint32_t addr, uint32_t parity, unsigned *status, unsigned who,
                                          WaitTally &tally) {
    return flag_wait_with<E, RECORD>([&] { return __builtin_amdgcn_readfirstlane(flag_load(addr)); }, parity, status,
                                     who, tally);
}

// Add a wave's tally to stats[0..2] (once per wave, at its end).
__device__ __forceinline__ void publish_tally(unsigned long long *stats, const WaitTally &t) {
    if (!stats || (threadIdx.x & 63) != 0) return;
    atomicAdd(stats + 0, (unsigned long long)t.waits);
    atomicAdd(stats + 1, (unsigned long long)t.blocked);
    atomicAdd(stats + 2, (unsigned long long)t.polls);
}

// One arrival of the calling wave: lane 0 adds n (1 unless a wave stands in
// for missing ones, so that the count per phase stays a power of two, e.g. 7
// consumer waves of which one adds 2). The caller has already
// waited for the wave's own LDS writes or reads of the slot; LDS operations
// of one wave execute in order, so nothing here needs waiting for. The add
// runs with exec narrowed to lane 0 inside the assembly rather than under a
// lane test, so the code around it stays wave-uniform and the ring counters
// stay in scalar registers.
__device__ __forceinline__ void flag_arrive(uint32_t addr, uint32_t n = 1u) {
    uint64_t saved;
    asm volatile(
        "s_mov_b64 %0, exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "ds_add_u32 %1, %2\n\t"
        "s_mov_b64 exec, %0"
        : "=&s"(saved)
        : "v"(addr), "v"(n)
        : "memory");
}

// An arrival of n (1 unless a wave stands in for missing ones, as in
// flag_arrive) on a flag with E expected arrivals per phase (wave-uniform LDS
// address), returning the arrivals of the current phase that preceded it
// (0 .. E - 1). The add returns a value, so its wait is inside the assembly.
template <int E>
__device__ __forceinline__ uint32_t flag_arrive_rank(uint32_t addr, uint32_t n = 1u) {
    uint64_t saved;
    uint32_t va, vn, old;
    asm volatile(
        "s_mov_b64 %0, exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "v_mov_b32 %1, %4\n\t"
        "v_mov_b32 %2, %5\n\t"
        "ds_add_rtn_u32 %3, %1, %2\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b64 exec, %0"
        : "=&s"(saved), "=&v"(va), "=&v"(vn), "=&v"(old)
        : "s"(addr), "s"(n)
        : "memory");
    return __builtin_amdgcn_readfirstlane(old) & (uint32_t)(E - 1);
}

// ---------------------------------------------------------------------------
// The ring's flag words as the kernels use them: full[s] and empty[s] in the
// first kFlagBytes of the workgroup's LDS, one ds_* instruction per flag
// operation.
// ---------------------------------------------------------------------------
struct LdsFlags {
    uint32_t fb;            // LDS address of the flag area
    const uint32_t *words;  // the same area as a generic pointer, for early reads
    __device__ void arrive_full(int s) const { flag_arrive(full_flag(fb, s)); }
    __device__ void arrive_empty(int s, uint32_t n = 1u) const { flag_arrive(empty_flag(fb, s), n); }
    template <int E, bool RECORD = true>
    __device__ bool wait_full(int s, uint32_t parity, unsigned *status, unsigned who, WaitTally &t) const {
        return flag_wait<E, RECORD>(full_flag(fb, s), parity, status, who, t);
    }
    template <int E>
    __device__ uint32_t arrive_empty_rank(int s, uint32_t n = 1u) const {
        return flag_arrive_rank<E>(__builtin_amdgcn_readfirstlane(empty_flag(fb, s)), n);
    }
    template <int E, bool RECORD = true>
    __device__ bool wait_empty(int s, uint32_t parity, unsigned *status, unsigned who, WaitTally &t) const {
        return flag_wait<E, RECORD>(empty_flag(fb, s), parity, status, who, t);
    }
    // early read of full[s] by a consumer (which has no LDS-DMA in flight);
    // the compiler waits for it where the value is used
    __device__ uint32_t peek_full(int s) const {
        return __hip_atomic_load(words + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
};

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

constexpr int kAuxNontemporal = 2;  // cache-policy bits of a buffer load: nt (streaming)

// 16 bytes per lane, global -> LDS without passing through VGPRs. Lane l's
// data lands at lds_wave_base + 16 * l (lds_wave_base is wave-uniform).
template <int AUX = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, void *lds_wave_base, uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds_wave_base, 16, voffset, 0, 0, AUX);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace wsg
