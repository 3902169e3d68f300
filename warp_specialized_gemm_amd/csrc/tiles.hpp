// tiles.hpp - pieces shared by the kernels that stream tiles through the LDS
// ring: fragment vector types, the ring's prologue, the slot swizzles and the
// LDS-DMA tile loaders (global -> LDS, 16 bytes per lane, out-of-range chunks
// load zeros).
#pragma once

#include "internal.hpp"
#include "ring.hpp"

namespace wsg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2. Logical index of workgroup bid when every XCD takes a contiguous run of
// the `total` logical indices instead.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_linear(int bid, int total) {
    const int x = bid % kXcds, i = bid / kXcds;
    const int q = total / kXcds, r = total % kXcds;
    return x * q + min(x, r) + i;
}

// Kernel prologue for the ring's flags: zero the LDS flag words, then the
// workgroup's first (and the specialized kernels' only) barrier.
__device__ __forceinline__ LdsFlags init_flags(unsigned char *lds) {
    if (threadIdx.x < kFlagBytes / 4) reinterpret_cast<uint32_t *>(lds)[threadIdx.x] = 0u;
    __syncthreads();
    return LdsFlags{lds_addr(lds), reinterpret_cast<const uint32_t *>(lds)};
}

// XOR applied to the chunk index of row m (QPR chunks of 16 bytes per row),
// chosen so that the 16 consecutive rows one 16-lane read pass covers land on
// 16 distinct 16-byte positions of a 256-byte bank span. A span holds 16 / QPR
// rows, so rows that share their position within the span are 16 / QPR apart,
// and the XOR must differ between them: (m / (16 / QPR)) mod QPR. 4 chunks
// (64-byte rows): (m / 4) mod 4; 8 chunks (128-byte rows): (m / 2) mod 8;
// 16 chunks (256-byte rows): m mod 16. With m mod 8 for 8 and 16 chunks, rows
// 8 apart collided: bf16 GEMM consumers spent 37% and attention consumers 31%
// of their LDS cycles on bank conflicts (rocprofv3 SQ_LDS_BANK_CONFLICT
// against SQ_LDS_IDX_ACTIVE); with (m / 2) mod 4 for 4 chunks, rows 8 apart
// collided too (bf16 256 x 256 x 32: 34%).
template <int QPR>
__device__ __forceinline__ int row_swizzle(int m) {
    if constexpr (QPR == 4) return (m >> 2) & 3;
    else if constexpr (QPR == 8) return (m >> 1) & 7;
    else return m & 15;
}

// Slot position of logical 16-byte chunk q of row m, through a per-row
// parameter. Rows of a power-of-two chunk count: XOR with row_swizzle. Rows of
// 6 chunks (a 48-deep bf16 k tile): rotation by (m / 8) mod 6, which puts the
// 16 consecutive rows one read pass covers on 16 distinct 16-byte positions
// of a 256-byte bank span (96-byte rows repeat their bank offset every 8 rows).
template <int QPR>
__device__ __forceinline__ int chunk_param(int m) {
    if constexpr (QPR == 6) return (m >> 3) % 6;
    else return row_swizzle<QPR>(m);
}
template <int QPR>
__device__ __forceinline__ int chunk_at(int q, int param) {  // logical -> slot
    if constexpr (QPR == 6) {
        const int s = q + param;
        return s >= 6 ? s - 6 : s;
    } else {
        return q ^ param;
    }
}
template <int QPR>
__device__ __forceinline__ int chunk_of(int pq, int param) {  // slot -> logical
    if constexpr (QPR == 6) {
        const int s = pq - param;
        return s < 0 ? s + 6 : s;
    } else {
        return pq ^ param;
    }
}

// XOR applied to the chunk index of row k of a B slot (CPR chunks per row).
// fp32 (CPR >= 16): the four k rows 4 apart that one b32 fragment read spans
// land in different 64-byte bank groups. bf16: one transpose read has two
// 16-lane groups (two column halves, 2 chunks each) over the same 4 rows;
// XOR with 2r + 8(r & 1) (r = k mod 4) puts those 8 (row, chunk) pairs on 8
// distinct 16-byte positions of a 128-byte span and all 16 pairs of both
// groups on distinct positions of a 256-byte span. Rows of 8 chunks only get
// the first part.
template <int ES, int CPR>
__device__ __forceinline__ int b_swizzle(int k) {
    if constexpr (ES == 4) return ((k >> 2) & 3) << 2;
    else if constexpr (CPR >= 16) return ((k & 3) << 1) | ((k & 1) << 3);
    else return (k & 3) << 1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ----------------------------------------------------------------------------
// A by LDS-DMA: BM rows x BK elements of ES bytes, QPR chunks per row.
// ----------------------------------------------------------------------------
template <int BM, int BK, int ES, int P>
struct ADma {
    static constexpr int EPC = 16 / ES;  // elements per chunk
    static constexpr int QPR = BK / EPC;
    static constexpr int CHUNKS = BM * QPR;
    static constexpr int NL = CHUNKS / (64 * P);
    static_assert(CHUNKS % (64 * P) == 0, "A chunks split evenly over producer waves");
    uint32_t off[NL];
    int kq[NL];
    bool ok[NL];

    __device__ __forceinline__ void init(int wave, int lane, int64_t K, int rows_valid) {
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const int p = (r * P + wave) * 64 + lane;
            const int m = p / QPR;
            const int q = chunk_of<QPR>(p % QPR, chunk_param<QPR>(m));
            off[r] = (uint32_t)m * (uint32_t)K * ES + (uint32_t)q * 16u;
            kq[r] = q * EPC;
            ok[r] = m < rows_valid;
        }
    }
    __device__ __forceinline__ void issue(unsigned char *slot, int wave, const unsigned char *A_rows, int rows_valid,
                                          int64_t K, int64_t k0) const {
        const int64_t rec = ((int64_t)rows_valid * K - k0) * ES;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A_rows + (size_t)k0 * ES, (uint32_t)min(rec, (int64_t)0x7FFFFFFF));
#pragma unroll
        for (int r = 0; r < NL; ++r)
            lds_dma16(rs, slot + (r * P + wave) * 1024, (ok[r] && k0 + kq[r] < K) ? off[r] : kOobOffset);
    }
};

// ----------------------------------------------------------------------------
// B by LDS-DMA: BK rows x BN elements of ES bytes, chunks swizzled by k.
// ----------------------------------------------------------------------------
template <int BN, int BK, int ES, int P>
struct BDma {
    static constexpr int EPC = 16 / ES;
    static constexpr int CPR = BN / EPC;  // chunks per row
    static constexpr int CHUNKS = BK * CPR;
    static constexpr int NL = CHUNKS / (64 * P);
    static_assert(CHUNKS % (64 * P) == 0 && CPR >= (ES == 4 ? 16 : 8), "B chunks");
    uint32_t off[NL];
    int kk[NL];
    bool ok[NL];

    __device__ __forceinline__ void init(int wave, int lane, int64_t N, int64_t n0) {
#pragma unroll
        for (int r = 0; r < NL; ++r) {
            const int p = (r * P + wave) * 64 + lane;
            const int k = p / CPR;
            const int c = (p % CPR) ^ b_swizzle<ES, CPR>(k);
            off[r] = (uint32_t)k * (uint32_t)N * ES + (uint32_t)c * 16u;
            kk[r] = k;
            ok[r] = n0 + EPC * c < N;
        }
    }
    __device__ __forceinline__ void issue(unsigned char *slotB, int wave, const unsigned char *B, int64_t N, int64_t K,
                                          int64_t n0, int64_t k0) const {
        const int64_t rec = (K * N - k0 * N - n0) * ES;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(B + (size_t)(k0 * N + n0) * ES, (uint32_t)min(rec, (int64_t)0x7FFFFFFF));
#pragma unroll
        for (int r = 0; r < NL; ++r)
            lds_dma16(rs, slotB + (r * P + wave) * 1024, (ok[r] && k0 + kk[r] < K) ? off[r] : kOobOffset);
    }
};

}  // namespace wsg
