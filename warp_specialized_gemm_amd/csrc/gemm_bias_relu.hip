// gemm_bias_relu.hip - C = relu(A @ B + bias) as a wave-specialized GEMM.
//
// The operator is the SGEMM with a bias + ReLU epilogue of the pwwt.cn
// article on intra-kernel pipelining (section 4.1). Its K loop is split
// between roles as in aicassindra's "GPU warp specialization" ("The
// architecture: every piece explained", "End-to-end flow"): each workgroup
// owns one BM x BN tile of C; producer waves stream BK-deep tiles of A and B
// through an S-slot LDS ring; consumer waves wait for a full slot, multiply on
// the matrix cores into register accumulators, and hand the slot back.
// Slot = t mod S, full-wait parity = (t / S) & 1, empty-wait parity =
// ((t / S) & 1) ^ 1 (ring.hpp).
//
// Producers (one implementation for both dtypes)
//   A and B go global -> LDS by 16-byte LDS-DMA loads through buffer
//   resources (no VGPRs; completion by vmcnt), the analogue of an
//   asynchronous bulk copy. Chunks past M, N or K get an out-of-range offset,
//   which loads zeros, so consumers never mask. Up to D = min(S - 1, ...)
//   tiles stay in flight, and the oldest is published before each wait for a
//   free slot. This needs 16-byte aligned rows; other shapes use a
//   register-staged producer with per-element masks and the same slot layout.
//
// Slot layout: A as BM rows of BK elements, 16-byte chunks XOR-swizzled
// within a row (rotated, for the 6-chunk rows of a 48-deep bf16 tile) so that
// consecutive rows reading the same chunk index hit distinct banks; B as BK
// rows of BN elements (its natural layout), chunks XOR-swizzled by k.
//
// Consumers (one wave per SIMD in the default tiles: 2 x 2 waves of 128 x 64)
//   fp32: v_mfma_f32_16x16x4_f32. Over a 16-deep k group, lane group q
//   (lanes 16q..16q+15) supplies k = 16g + 4q + j at step j = 0..3, so each
//   lane's four A values are one 16-byte chunk of its row.
//   bf16: v_mfma_f32_32x32x16_bf16; lane half h supplies k = 16g + 8h + e.
//   A comes as one 16-byte chunk of its row; B, which is n-contiguous in the
//   slot, comes through two LDS transpose reads (ds_read_b64_tr_b16): in each
//   16-lane group, lane i' points at 4 consecutive n of row k0 + i'/4, and
//   lane i receives rows k0..k0+3 of column n0 + i.
//   The fragments of the next k group are read while the MFMAs of the current
//   one run, and a slot is released as soon as its last group is in
//   registers.
//   On gfx950, while a wave streams fp32 MFMAs, LDS reads issued by the other
//   waves on its SIMD wait until the stream pauses. Two fp32 consumers on a
//   SIMD would hold back each other's fragment reads, so the fp32 default puts
//   one consumer (a 128 x 64 wave tile) on each SIMD; the producer's flag polls
//   still wait behind its SIMD's consumer.
//
// The homogeneous kernel (no producer waves; sync_loop below) runs the same
// consumer fragments and MFMA order with workgroup barriers instead of roles,
// as the baseline the specialization is measured against.
#include <utility>

#include "internal.hpp"
#include "ring.hpp"
#include "tiles.hpp"

namespace wsg {

struct GemmArgs {
    const unsigned char *A;
    const unsigned char *B;
    const unsigned char *bias;
    float *C;
    int64_t M, N, K;
    int S;
    int tiles_m, tiles_n;
    unsigned *status;
    unsigned long long *stats;  // wait statistics, or null
    // stream-K launches only (kernels built with SK): see sk_unit
    int dp_tiles, sk_tiles, workers;
    float *part;      // one partial tile (BM x BN fp32) per worker
    unsigned *cnt;    // per stream-K tile and consumer wave: contributor pieces done
};

// Each XCD takes a contiguous run of logical tiles (xcd_linear), walked in
// groups of a few tile rows so the tiles resident on one XCD at a time share
// rows of A and columns of B. kGroupRows tile rows per group: 8 for square
// tiles; for tall tiles fewer rows (and so more columns) keep the A and B
// bytes a group touches balanced.

template <int kGroupRows>
__device__ __forceinline__ void swizzle_tile(int L, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per_group = kGroupRows * tiles_n;
    const int grp = L / per_group;
    const int first_m = grp * kGroupRows;
    const int gm = min(tiles_m - first_m, kGroupRows);
    const int rem = L - grp * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
}

// Grouped launches: the experts of a mixture-of-experts layer, each applying
// its own weights and biases to the token rows routed to it (rows sorted by
// expert). Expert e owns rows row0[e] .. row0[e + 1] - 1 of A and C, the e-th
// K x N block of B, the e-th N biases, and the launch's logical tiles
// tile0[e] .. tile0[e + 1] - 1 (empty experts own none); entries past the
// last expert repeat the totals. The table travels in the kernel arguments.
struct GroupTable {
    int n;
    int tile0[WSG_MAX_GROUPS + 1];
    int64_t row0[WSG_MAX_GROUPS + 1];
};

// Kernel arguments of a grouped launch: the GEMM's (with the whole launch's
// pointers) plus the expert table. Ordinary launches pass GemmArgs alone, so
// their kernels are compiled exactly as without grouping.
struct GroupedArgs {
    GemmArgs a;
    GroupTable gt;
};
template <bool GR>
struct KernelArgs {
    using type = GemmArgs;
};
template <>
struct KernelArgs<true> {
    using type = GroupedArgs;
};
__device__ __forceinline__ GemmArgs &gemm_args(GemmArgs &p) { return p; }
__device__ __forceinline__ GemmArgs &gemm_args(GroupedArgs &p) { return p.a; }

template <int kGroupRows>
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    swizzle_tile<kGroupRows>(xcd_linear(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// Workgroup -> (tile row, tile column). For a grouped launch it also points
// the GEMM arguments at the expert's operands and row count; the XCD step
// runs over the whole launch, so each XCD's run of tiles stays contiguous
// across experts.
template <int kGroupRows, int BM, int ES>
__device__ __forceinline__ void resolve_tile(GemmArgs &a, int &tm, int &tn) {
    tile_coords<kGroupRows>(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
}
template <int kGroupRows, int BM, int ES>
__device__ __forceinline__ void resolve_tile(GroupedArgs &p, int &tm, int &tn) {
    GemmArgs &a = p.a;
    const GroupTable &gt = p.gt;
    const int L = xcd_linear(blockIdx.x, gt.tile0[WSG_MAX_GROUPS]);
    // tile0 is nondecreasing (entries past the last expert hold the totals):
    // the expert is the last entry at or below L, its end the first above.
    // Constant indices only, so the table is read with scalar loads rather
    // than copied to scratch memory for a dynamic index.
    int e = 0, t0 = 0;
    int64_t r0 = 0, r1 = 0;
    bool above = false;
#pragma unroll
    for (int i = 1; i <= WSG_MAX_GROUPS; ++i) {
        const int ti = gt.tile0[i];
        if (ti <= L) {
            e = i;
            t0 = ti;
            r0 = gt.row0[i];
        } else if (!above) {
            r1 = gt.row0[i];
            above = true;
        }
    }
    a.M = r1 - r0;
    a.tiles_m = (int)((a.M + BM - 1) / BM);
    a.A += (size_t)r0 * (size_t)a.K * ES;
    a.B += (size_t)e * (size_t)a.K * (size_t)a.N * ES;
    a.bias += (size_t)e * (size_t)a.N * ES;  // the bias has the operands' element type
    a.C += r0 * a.N;
    swizzle_tile<kGroupRows>(L - t0, a.tiles_m, a.tiles_n, tm, tn);
}

__device__ __forceinline__ float relu_f32(float v) { return (v > 0.0f || v != v) ? v : 0.0f; }

// ----------------------------------------------------------------------------
// Register-staged loads with per-element masks, same slot layouts.
// ----------------------------------------------------------------------------
template <int BM, int BK, int ES, int P>
__device__ __forceinline__ void a_general(unsigned char *slotA, int wave, int lane, const unsigned char *A, int64_t m0,
                                          int rows_valid, int64_t K, int64_t k0) {
    constexpr int EPC = 16 / ES, QPR = BK / EPC, NL = BM * QPR / (64 * P);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int p = (r * P + wave) * 64 + lane;
        const int m = p / QPR;
        const int q = chunk_of<QPR>(p % QPR, chunk_param<QPR>(m));
        u32x4 v;
        if constexpr (ES == 4) {
            const float *Af = reinterpret_cast<const float *>(A);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t k = k0 + 4 * q + e;
                v[e] = (m < rows_valid && k < K) ? __float_as_uint(Af[(m0 + m) * K + k]) : 0u;
            }
        } else {
            const uint16_t *Ah = reinterpret_cast<const uint16_t *>(A);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t k = k0 + 8 * q + 2 * e;
                const uint32_t lo = (m < rows_valid && k < K) ? Ah[(m0 + m) * K + k] : 0u;
                const uint32_t hi = (m < rows_valid && k + 1 < K) ? Ah[(m0 + m) * K + k + 1] : 0u;
                v[e] = lo | (hi << 16);
            }
        }
        *reinterpret_cast<u32x4 *>(slotA + (size_t)p * 16u) = v;
    }
}

template <int BN, int BK, int ES, int P>
__device__ __forceinline__ void b_general(unsigned char *slotB, int wave, int lane, const unsigned char *B, int64_t N,
                                          int64_t K, int64_t n0, int64_t k0) {
    constexpr int EPC = 16 / ES, CPR = BN / EPC, NL = BK * CPR / (64 * P);
#pragma unroll
    for (int r = 0; r < NL; ++r) {
        const int p = (r * P + wave) * 64 + lane;
        const int k = p / CPR;
        const int c = (p % CPR) ^ b_swizzle<ES, CPR>(k);
        u32x4 v;
        if constexpr (ES == 4) {
            const float *Bf = reinterpret_cast<const float *>(B);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t n = n0 + 4 * c + e;
                v[e] = (k0 + k < K && n < N) ? __float_as_uint(Bf[(k0 + k) * N + n]) : 0u;
            }
        } else {
            const uint16_t *Bh = reinterpret_cast<const uint16_t *>(B);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t n = n0 + 8 * c + 2 * e;
                const uint32_t lo = (k0 + k < K && n < N) ? Bh[(k0 + k) * N + n] : 0u;
                const uint32_t hi = (k0 + k < K && n + 1 < N) ? Bh[(k0 + k) * N + n + 1] : 0u;
                v[e] = lo | (hi << 16);
            }
        }
        *reinterpret_cast<u32x4 *>(slotB + (size_t)p * 16u) = v;
    }
}

// ----------------------------------------------------------------------------
// Producer waves, shared by both kernels.
// ----------------------------------------------------------------------------
template <int BM, int BN, int BK, int ES, int P, int NCW, bool DMA, typename Flags>
__device__ __forceinline__ void produce(const GemmArgs &a, unsigned char *ring, const Flags &fl, int wave, int lane,
                                        int64_t m0, int64_t n0, int T) {
    constexpr int A_BYTES = BM * BK * ES, SLOT = A_BYTES + BK * BN * ES;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int S = a.S;
    const int rows_valid = (int)min((int64_t)BM, M - m0);
    const unsigned char *A_rows = a.A + (size_t)m0 * (size_t)K * ES;
    int s = 0;
    uint32_t lap = 0;
    WaitTally tally;
    if constexpr (DMA) {
        using AD = ADma<BM, BK, ES, P>;
        using BD = BDma<BN, BK, ES, P>;
        constexpr int NL = AD::NL + BD::NL;
        static_assert(NL <= 63, "one tile's loads must fit vmcnt");
        AD ad;
        BD bd;
        ad.init(wave, lane, K, rows_valid);
        bd.init(wave, lane, N, n0);
        // Up to D tiles in flight. The oldest is completed and published
        // before the wait for the next free slot, so a full signal never
        // waits on an empty one (the producer spends the steady state of a
        // compute-bound kernel blocked on empty slots).
        // The 12-wave bf16 kernels with a ring of 4 (or more, even) slots and an
        // even tile count: each producer step takes two slots, issuing each
        // slot's loads as soon as that slot is free, then publishes each slot
        // as its loads land, so the per-step bookkeeping comes once per two
        // tiles; with 4 slots, one pair loads while the consumers read the
        // other (measured on MI355X, bf16 8192^3 at S = 4, interleaved runs,
        // bit-identical: +2% to +5% with both slots waited for, loaded and
        // published together, 1056-1116 -> 1110-1136 TFLOP/s; +1.2% more with
        // each published as it lands; +2.6% to +4.6% more, 1118-1137 ->
        // 1167-1169, with each loaded once free). An odd tile count takes the
        // one-slot loop below, which keeps the in-flight load counts exact.
        if constexpr (NCW == 8 && ES == 2 && 2 * NL <= 63) {
            if (S >= 4 && (S & 1) == 0 && (T & 1) == 0) {
                const int D2 = max(1, min(S / 2 - 1, 63 / (2 * NL)));  // pairs in flight
                int inflight = 0, ps = 0;
                for (int t = 0; t < T; t += 2) {
                    if (inflight == D2) {
                        wait_vmcnt_dyn((D2 - 1) * 2 * NL + NL);  // the pair's first slot has landed
                        fl.arrive_full(ps);
                        wait_vmcnt_dyn((D2 - 1) * 2 * NL);
                        fl.arrive_full(ps + 1);
                        ps = ps + 2 == S ? 0 : ps + 2;
                        --inflight;
                    }
                    if (!fl.template wait_empty<NCW>(s, (lap & 1u) ^ 1u, a.status, kStatusGemm, tally)) return;
                    unsigned char *slot = ring + (size_t)s * SLOT;
                    const int64_t k0 = (int64_t)t * BK;
                    ad.issue(slot, wave, A_rows, rows_valid, K, k0);
                    bd.issue(slot + A_BYTES, wave, a.B, N, K, n0, k0);
                    if (!fl.template wait_empty<NCW>(s + 1, (lap & 1u) ^ 1u, a.status, kStatusGemm, tally)) return;
                    ad.issue(slot + SLOT, wave, A_rows, rows_valid, K, k0 + BK);
                    bd.issue(slot + SLOT + A_BYTES, wave, a.B, N, K, n0, k0 + BK);
                    ++inflight;
                    s += 2;
                    if (s == S) {
                        s = 0;
                        ++lap;
                    }
                }
                while (inflight > 0) {
                    wait_vmcnt_dyn((inflight - 1) * 2 * NL + NL);
                    fl.arrive_full(ps);
                    wait_vmcnt_dyn((inflight - 1) * 2 * NL);
                    fl.arrive_full(ps + 1);
                    ps = ps + 2 == S ? 0 : ps + 2;
                    --inflight;
                }
                publish_tally(a.stats ? a.stats + kStatGemmProducer : nullptr, tally);
                return;
            }
        }
        const int D = max(1, min(S - 1, 63 / NL));
        int inflight = 0, ps = 0;  // tiles issued but not published; slot of the oldest
        for (int t = 0; t < T; ++t) {
            if (inflight == D) {
                wait_vmcnt_dyn((D - 1) * NL);
                fl.arrive_full(ps);
                if (++ps == S) ps = 0;
                --inflight;
            }
            if (!fl.template wait_empty<NCW>(s, (lap & 1u) ^ 1u, a.status, kStatusGemm, tally)) return;
            const int64_t k0 = (int64_t)t * BK;
            unsigned char *slot = ring + (size_t)s * SLOT;
            ad.issue(slot, wave, A_rows, rows_valid, K, k0);
            bd.issue(slot + A_BYTES, wave, a.B, N, K, n0, k0);
            ++inflight;
            if (++s == S) {
                s = 0;
                ++lap;
            }
        }
        while (inflight > 0) {
            wait_vmcnt_dyn((inflight - 1) * NL);
            fl.arrive_full(ps);
            if (++ps == S) ps = 0;
            --inflight;
        }
    } else {
        for (int t = 0; t < T; ++t) {
            if (!fl.template wait_empty<NCW>(s, (lap & 1u) ^ 1u, a.status, kStatusGemm, tally)) return;
            const int64_t k0 = (int64_t)t * BK;
            unsigned char *slot = ring + (size_t)s * SLOT;
            a_general<BM, BK, ES, P>(slot, wave, lane, a.A, m0, rows_valid, K, k0);
            b_general<BN, BK, ES, P>(slot + A_BYTES, wave, lane, a.B, N, K, n0, k0);
            wait_lgkm0();
            fl.arrive_full(s);
            if (++s == S) {
                s = 0;
                ++lap;
            }
        }
    }
    publish_tally(a.stats ? a.stats + kStatGemmProducer : nullptr, tally);
}

// ----------------------------------------------------------------------------
// Stream-K tail (fp32 kernels built with SK). When the output tiles do not
// fill a whole number of rounds of the persistent grid (`workers` workgroups,
// as many as the device holds at once), the last, partial round would leave
// CUs idle: 480 tiles of 256 x 128 on 256 CUs run as a full round and a round
// of 224. Instead, each worker w first computes data-parallel tiles w,
// w + workers, ... (dp_tiles of them in all, whole rounds only), then an equal
// contiguous share of the remaining sk_tiles x T k-tile steps (tile-major, k
// ascending). A share is at most one tile long, so it holds at most two
// pieces: the end of one tile and the start of the next, each stored in a
// partial slot of its own (2 w and 2 w + 1). Every piece of a split tile is
// stored, then counted on the tile's counter (per consumer wave); the wave
// whose count completes the tile reads all of its pieces back in piece order
// (so the sum order is fixed whoever finishes last) and runs the epilogue.
// No workgroup ever waits for another, so the launch needs no co-residency.
// The ring flags carry on across a worker's units: producers stream them back
// to back.
// ----------------------------------------------------------------------------
// Cache policy of the partial-sum stores and loads: sc1, device scope.
constexpr int kScopeDevice = 16;
// Fewest k steps per worker for which a launch with fewer tiles than workers
// is split by stream-K by default.
constexpr int64_t kStreamKMinSteps = 16;

struct SkUnit {
    int tile;      // logical tile index (before the tile-row swizzle)
    int kb, ke;    // k-tile range [kb, ke)
    int sk_tile;   // index among the stream-K tiles (split tiles only)
    int first, npieces;  // worker of the tile's first piece, pieces of the tile (1: whole)
    int slot;      // partial slot of this piece
    int first_slot;  // partial slot of the tile's first piece (the others': 2 (first + p))
};

// Worker whose share of the Z stream-K steps holds step i: shares are
// [w Z / G, (w + 1) Z / G), so it is the largest w with w Z / G <= i.
__device__ __forceinline__ int sk_worker_of(int64_t i, int64_t Z, int G) { return (int)(((i + 1) * G - 1) / Z); }

// Unit u of worker w (wave-uniform); false past the last one.
__device__ __forceinline__ bool sk_unit(const GemmArgs &a, int T, int w, int u, SkUnit &out) {
    const int G = a.workers;
    const int rounds = a.dp_tiles / G;
    if (u < rounds) {
        out = SkUnit{u * G + w, 0, T, -1, w, 1, -1, -1};
        return true;
    }
    int idx = u - rounds;
    // with fewer steps than workers only the first Z workers take one each:
    // every share is then non-empty, so the workers between a tile's first
    // and last piece all hold a piece of it; a piece other than a tile's
    // first starts its worker's share, so it sits in that worker's slot 0
    const int64_t Z = (int64_t)a.sk_tiles * T;
    const int Gs = (int)min((int64_t)G, Z);
    if (w >= Gs) return false;
    int64_t i = (int64_t)w * Z / Gs;
    const int64_t e = (int64_t)(w + 1) * Z / Gs;
    for (int piece = 0; i < e; ++piece) {
        const int64_t tau = i / T;
        const int kb = (int)(i - tau * T);
        const int ke = (int)min((int64_t)T, e - tau * T);
        if (idx == 0) {
            const int wf = sk_worker_of(tau * T, Z, Gs), wl = sk_worker_of(tau * T + T - 1, Z, Gs);
            out.tile = a.dp_tiles + (int)tau;
            out.kb = kb;
            out.ke = ke;
            out.sk_tile = (int)tau;
            out.first = wf;
            out.npieces = wl - wf + 1;
            out.slot = 2 * w + piece;
            out.first_slot = 2 * wf + ((int64_t)wf * Z / Gs == tau * T ? 0 : 1);
            return true;
        }
        --idx;
        i = tau * T + ke;
    }
    return false;
}

// Producer of a stream-K worker: the LDS-DMA producer above, run over every
// k-tile of the worker's units in order, with one in-flight window across
// them.
template <int BM, int BN, int BK, int ES, int P, int NCW, int kGroupRows, typename Flags>
__device__ __forceinline__ void produce_sk(const GemmArgs &a, unsigned char *ring, const Flags &fl, int wave, int lane,
                                           int T, int w) {
    constexpr int A_BYTES = BM * BK * ES, SLOT = A_BYTES + BK * BN * ES;
    using AD = ADma<BM, BK, ES, P>;
    using BD = BDma<BN, BK, ES, P>;
    constexpr int NL = AD::NL + BD::NL;
    static_assert(NL <= 63, "one tile's loads must fit vmcnt");
    const int64_t M = a.M, N = a.N, K = a.K;
    const int S = a.S;
    const int D = max(1, min(S - 1, 63 / NL));
    int s = 0, inflight = 0, ps = 0;
    uint32_t lap = 0;
    WaitTally tally;
    SkUnit un;
    for (int u = 0; sk_unit(a, T, w, u, un); ++u) {
        int tm, tn;
        swizzle_tile<kGroupRows>(un.tile, a.tiles_m, a.tiles_n, tm, tn);
        const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
        const int rows_valid = (int)min((int64_t)BM, M - m0);
        const unsigned char *A_rows = a.A + (size_t)m0 * (size_t)K * ES;
        AD ad;
        BD bd;
        ad.init(wave, lane, K, rows_valid);
        bd.init(wave, lane, N, n0);
        for (int t = un.kb; t < un.ke; ++t) {
            if (inflight == D) {
                wait_vmcnt_dyn((D - 1) * NL);
                fl.arrive_full(ps);
                if (++ps == S) ps = 0;
                --inflight;
            }
            if (!fl.template wait_empty<NCW>(s, (lap & 1u) ^ 1u, a.status, kStatusGemm, tally)) return;
            const int64_t k0 = (int64_t)t * BK;
            unsigned char *slot = ring + (size_t)s * SLOT;
            ad.issue(slot, wave, A_rows, rows_valid, K, k0);
            bd.issue(slot + A_BYTES, wave, a.B, N, K, n0, k0);
            ++inflight;
            if (++s == S) {
                s = 0;
                ++lap;
            }
        }
    }
    while (inflight > 0) {
        wait_vmcnt_dyn((inflight - 1) * NL);
        fl.arrive_full(ps);
        if (++ps == S) ps = 0;
        --inflight;
    }
    publish_tally(a.stats ? a.stats + kStatGemmProducer : nullptr, tally);
}

// Ring position of a consumer between units: the slot and lap of the next
// tile it reads.
struct RingPos {
    int s = 0;
    uint32_t lap = 0;
};

// ----------------------------------------------------------------------------
// Consumer walk over the ring, a group at a time (the fp32 kernels, whose
// 256-register consumers spill under the per-tile walk below). The K loop is
// cut into U = T * KG groups of 16 k; the fragments of group u + 1 are read
// while the MFMAs of group u run. A slot is released (one arrival on its
// empty flag) once the reads of its last group have completed. The full flag
// of the next tile is read early, together with the last group's fragments,
// and only if that early value shows the tile unpublished does the wave spin
// on it.
// Returns false if a wait gave up.
// ----------------------------------------------------------------------------
// IL > 0: the next group's fragment reads and the current group's MFMAs form
// one straight-line block (on the last step the reads repeat the current
// group, harmlessly), and the scheduler is asked to alternate them, IL pairs
// of one MFMA and one LDS read, so the reads issue in the shadow of the MFMAs
// instead of in a burst between them (measured on MI355X: +1.7% for the fp32
// 4096^3 default, +2.6 to +5.5% for the bf16 configurations).
template <int KG, int P, typename Frag, int IL = 0, typename Flags, typename Read, typename Mma>
__device__ __forceinline__ bool consume_ring(int T, int S, unsigned char *ring, int slot_bytes, const Flags &fl,
                                             unsigned *status, WaitTally &tally, Read read, Mma mma,
                                             RingPos &pos) {
    const int U = T * KG;
    if (U == 0) return true;
    Frag f0, f1;
    int rs = pos.s, rg = 0;  // slot and group of the latest read
    uint32_t rlap = pos.lap;
    int cs = pos.s;          // slot being consumed
    uint32_t peek = 0;       // early value of the next tile's full flag
    if (!fl.template wait_full<P>(pos.s, pos.lap & 1u, status, kStatusGemm, tally)) return false;
    read(f0, ring + (size_t)pos.s * slot_bytes, 0);
    if (KG == 1 && U > 1) peek = fl.peek_full(pos.s + 1 == S ? 0 : pos.s + 1);
    bool alive = true;
    auto step = [&](int u, Frag &cur, Frag &nxt) {
        wait_lgkm0();  // the reads of group u (and the early flag value) have landed
        const uint32_t pk = __builtin_amdgcn_readfirstlane(peek);
        if (u % KG == KG - 1) {
            fl.arrive_empty(cs);
            if (++cs == S) cs = 0;
        }
        if constexpr (IL == 0) {
            if (u + 1 < U) {
                if (++rg == KG) {
                    rg = 0;
                    if (++rs == S) {
                        rs = 0;
                        ++rlap;
                    }
                    if (phase_of<P>(pk) == (rlap & 1u)) {
                        if (!fl.template wait_full<P>(rs, rlap & 1u, status, kStatusGemm, tally)) {
                            alive = false;
                            return;
                        }
                    } else {
                        ++tally.waits;  // satisfied by the early read
                    }
                    asm volatile("" ::: "memory");
                }
                read(nxt, ring + (size_t)rs * slot_bytes, rg);
                if (rg == KG - 1 && u + 1 + KG < U) peek = fl.peek_full(rs + 1 == S ? 0 : rs + 1);
            }
            mma(cur);
        } else {
            if (u + 1 < U && ++rg == KG) {
                rg = 0;
                if (++rs == S) {
                    rs = 0;
                    ++rlap;
                }
                if (phase_of<P>(pk) == (rlap & 1u)) {
                    if (!fl.template wait_full<P>(rs, rlap & 1u, status, kStatusGemm, tally)) {
                        alive = false;
                        return;
                    }
                } else {
                    ++tally.waits;  // satisfied by the early read
                }
                asm volatile("" ::: "memory");
            }
            const uint32_t pv = fl.peek_full(rs + 1 == S ? 0 : rs + 1);
            read(nxt, ring + (size_t)rs * slot_bytes, rg);
            mma(cur);
            peek = (rg == KG - 1 && u + 1 + KG < U) ? pv : peek;
#pragma unroll
            for (int i = 0; i < IL; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
        }
    };
    for (int u = 0; alive && u < U; u += 2) {
        step(u, f0, f1);
        if (alive && u + 1 < U) step(u + 1, f1, f0);
    }
    // the next tile after the last one read
    pos.s = rs + 1 == S ? 0 : rs + 1;
    pos.lap = pos.s == 0 ? rlap + 1 : rlap;
    return alive;
}

// Ask the scheduler to alternate IL pairs of one MFMA and one LDS read in the
// current straight-line block.
template <int IL>
__device__ __forceinline__ void interleave_mfma_reads() {
#pragma unroll
    for (int i = 0; i < IL; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}
template <int I, typename F>
__device__ __forceinline__ F &pick(F &x0, F &x1) {
    if constexpr (I == 0) return x0;
    else return x1;
}
// f(integral_constant<0>) && f(integral_constant<1>) && ... (stops at the first false)
template <typename F, int... Is>
__device__ __forceinline__ bool for_each_group(F &&f, std::integer_sequence<int, Is...>) {
    return (f(std::integral_constant<int, Is>{}) && ...);
}
// ----------------------------------------------------------------------------
// Consumer walk over the ring, one tile at a time (the bf16 kernels). The KG
// fragment groups of a tile are unrolled: group g's MFMAs run while group
// g + 1's fragments are read, in one straight-line block with no flag access
// and no branch. Only the last group of a tile touches the ring: once its
// reads have landed the slot is released (one arrival on its empty flag), and
// the next tile's full flag, read early together with the fragments of the
// tile's last group (KG >= 2) or of the previous tile's (KG == 1), decides
// whether the wave must spin before it reads the next tile's first group.
// Fragment buffers f0 / f1 alternate by group; with an odd KG the buffer of a
// tile's first group alternates too, so tiles are unrolled in pairs. An early
// flag read is issued only where its value is used: a load whose result is
// dead lets the register allocator reuse its destination while the load is in
// flight, which forces a full LDS drain in the middle of the MFMA block.
// Against the group-at-a-time walk above (measured on MI355X, bf16 8192^3,
// bit-identical): +8% for 256x128x64 tiles at S = 3, +15% with k groups of 16.
// Returns false if a wait gave up.
// ----------------------------------------------------------------------------
template <int KG, int P, typename Frag, int IL, typename Flags, typename Read, typename Mma>
__device__ __forceinline__ bool consume_tiles(int T, int S, unsigned char *ring, int slot_bytes, const Flags &fl,
                                              unsigned *status, WaitTally &tally, Read read, Mma mma) {
    if (T == 0) return true;
    Frag f0, f1;
    if (!fl.template wait_full<P>(0, 0u, status, kStatusGemm, tally)) return false;
    read(f0, ring, 0);
    uint32_t peek = KG == 1 ? fl.peek_full(S > 1 ? 1 : 0) : 0u;  // early value of tile 1's full flag
    int cs = 0;        // slot of the tile being consumed
    uint32_t lap = 0;  // its lap, t / S
    auto tile = [&](int t, auto first) __attribute__((always_inline)) -> bool {
        constexpr int b0 = decltype(first)::value;  // buffer holding this tile's group 0
        const int ns = cs + 1 == S ? 0 : cs + 1;
        const uint32_t nlap = ns == 0 ? lap + 1 : lap;
        unsigned char *slot = ring + (size_t)cs * slot_bytes;
        auto group = [&](auto G) __attribute__((always_inline)) -> bool {
            constexpr int g = decltype(G)::value;
            Frag &cur = pick<(b0 + g) & 1>(f0, f1);
            Frag &nxt = pick<(b0 + g + 1) & 1>(f0, f1);
            wait_lgkm0();  // group g's fragments (and the early flag value) have landed
            if constexpr (g < KG - 1) {
                const uint32_t pv = g == KG - 2 ? fl.peek_full(ns) : 0u;
                read(nxt, slot, g + 1);
                mma(cur);
                if (g == KG - 2) peek = pv;
                interleave_mfma_reads<IL>();
                return true;
            } else {
                fl.arrive_empty(cs);  // every read of this tile has landed
                if (t + 1 < T) {
                    if (phase_of<P>(__builtin_amdgcn_readfirstlane(peek)) == (nlap & 1u)) {
                        if (!fl.template wait_full<P>(ns, nlap & 1u, status, kStatusGemm, tally)) return false;
                    } else {
                        ++tally.waits;  // satisfied by the early read
                    }
                }
                asm volatile("" ::: "memory");
                // After the last tile this reads a slot no producer writes any
                // more; the values are never used. One code path keeps the
                // MFMAs accumulating in place.
                const uint32_t pv = KG == 1 ? fl.peek_full(ns + 1 == S ? 0 : ns + 1) : 0u;
                read(nxt, ring + (size_t)ns * slot_bytes, 0);
                mma(cur);
                if (KG == 1) peek = pv;
                interleave_mfma_reads<IL>();
                return true;
            }
        };
        if (!for_each_group(group, std::make_integer_sequence<int, KG>{})) return false;
        cs = ns;
        lap = nlap;
        return true;
    };
    if constexpr (KG % 2 == 0) {
        for (int t = 0; t < T; ++t)
            if (!tile(t, std::integral_constant<int, 0>{})) return false;
    } else {
        for (int t = 0; t < T; t += 2) {
            if (!tile(t, std::integral_constant<int, 0>{})) return false;
            if (t + 1 < T && !tile(t + 1, std::integral_constant<int, 1>{})) return false;
        }
    }
    return true;
}

// ----------------------------------------------------------------------------
// Consumer walk for workgroups of more than 8 waves (three waves share a SIMD,
// so each has at most 168 registers: a 128 x 64 bf16 wave tile's 128
// accumulators leave room for one set of fragments, not two). The wave keeps
// ONE fragment set. `step(next_slot, next_k, mid)` runs the current k step's
// MFMAs and re-reads each fragment piece for the next k step as soon as the
// last MFMA of this step that uses it has issued, so the next step's LDS
// reads still fly under this step's MFMAs; the second consumer on the SIMD
// covers what remains. `mid()` runs after the step's first column block of
// MFMAs has issued and before its first re-read. KS k steps of 16 per tile
// (KS >= 2). Flags only at tile boundaries: the next tile's full flag is read
// early with the reads of the tile's last step. In the last step, `mid`
// waits for every read of the slot (the last of them fed the MFMAs just
// issued, so nothing is left to wait for in the steady state), releases the
// slot and waits for the next tile's full flag; the step's re-reads then come
// from the next slot (after the last tile: a slot no producer writes any
// more, values unused).
// The loop keeps its scalar work small: with two consumers and a producer on
// each SIMD, the scalar unit issued an instruction on about two thirds of a
// CU's cycles (11 per MFMA), so the ring position advances once per tile, the
// next k step comes from a mask, and a wait that gives up ends the loop
// through its counter rather than a second exit (measured on MI355X, bf16
// 8192^3 at S = 4: +3.5%, bit-identical).
// Returns false if a wait gave up.
// ----------------------------------------------------------------------------
template <int KS, int P, int C, typename Flags, typename Prime, typename Step>
__device__ __forceinline__ bool consume_lean(int T, int S, unsigned char *ring, int slot_bytes, const Flags &fl,
                                             unsigned *status, WaitTally &tally, Prime prime, Step step) {
    static_assert(KS >= 2, "the lean walk reads the next tile's flag one k step early");
    if (T == 0) return true;
    if (!fl.template wait_full<P>(0, 0u, status, kStatusGemm, tally)) return false;
    prime(ring, 0);
    // Nothing in flight when the loop starts (the kernel's scalar loads share
    // the LDS counter and return out of order): without this the compiler
    // drains the counter at the top of every step instead of waiting only for
    // the fragments the step's first MFMAs use.
    wait_lgkm0();
    // One k step per iteration: each fragment piece re-read in the body is the
    // loop-carried value of the piece it replaces, so the register allocator
    // gives both the same registers (unrolled steps rotated through half as
    // many again and spilled accumulators).
    static_assert((KS & (KS - 1)) == 0, "k steps per tile: a power of two");
    uint32_t peek = 0;  // the next tile's full flag as read one step earlier
    // ring position of the tile being read and of the next one, advanced once
    // per tile; the next tile's full flag word as an LDS address, for its
    // early reads
    int cs = 0, ns = S > 1 ? 1 : 0, ks = 0;
    uint32_t lap = 0, nlap = ns == 0 ? 1u : 0u;
    unsigned char *cur = ring, *nxt = ring + (size_t)ns * slot_bytes;
    const uint32_t *peek_at = fl.words + ns;
    bool ok = true;
    for (int u = T * KS; u > 0; --u) {
        const int nk = (ks + 1) & (KS - 1);  // the k step the re-reads are for
        const bool last = nk == 0;
        step(last ? nxt : cur, nk, [&]() {
            if (last) {
                wait_lgkm0();  // every read of this tile (and the early flag value) has landed
                // Two consumers share each SIMD's matrix unit, which issues
                // the older wave's MFMAs first, so one consumer drifted up to
                // a tile ahead of its sibling and the slot the laggard still
                // held took the producers' lead (traced on MI355X: the 8
                // consumers released a tile 2500-3800 cycles apart). The
                // consumers that release a slot in the later half raise their
                // wave priority for the next tile, the earlier half lower it.
                if (fl.template arrive_empty_rank<C>(cs) >= (uint32_t)(C / 2))
                    __builtin_amdgcn_s_setprio(1);
                else
                    __builtin_amdgcn_s_setprio(0);
                if (u > 1) {
                    if (phase_of<P>(__builtin_amdgcn_readfirstlane(peek)) == (nlap & 1u)) {
                        ok = fl.template wait_full<P, false>(ns, nlap & 1u, status, kStatusGemm, tally);
                    } else {
                        ++tally.waits;  // satisfied by the early read
                    }
                }
                asm volatile("" ::: "memory");
            }
            // the next tile's full flag, for the tile's last step (read in
            // every step; in the last step it is overwritten before use)
            peek = __hip_atomic_load(peek_at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        });
        ks = nk;
        if (last) {
            if (!ok) u = 1;  // a wait gave up: the loop ends here
            cs = ns;
            lap = nlap;
            cur = nxt;
            ns = ns + 1 == S ? 0 : ns + 1;
            nlap = ns == 0 ? lap + 1 : lap;
            nxt = ring + (size_t)ns * slot_bytes;
            peek_at = fl.words + ns;
        }
    }
    if (!ok) atomicOr(status, kStatusTimeout | kStatusGemm);  // the wait in the loop gave up
    return ok;
}

// A consumer wave whose part of the output tile lies wholly past M or N (the
// last row tile of an expert in a grouped launch, ragged shapes) has nothing
// to compute, but the producers count on its release of every slot. It waits
// for each tile to be published before it releases it, so its arrival falls
// in the same phase of the empty flag as its siblings'. Its SIMD's other
// consumer meanwhile has the matrix unit to itself (measured on MI355X, the
// bf16 expert layer of 8 experts, 8192 routed rows, K 4096, N 14336, where 4
// experts end in a row tile of at most 128 rows: +2%, bit-identical).
template <int P, typename Flags>
__device__ __forceinline__ bool release_only(int T, int S, const Flags &fl, unsigned *status, WaitTally &tally) {
    int cs = 0;
    uint32_t lap = 0;
    for (int t = 0; t < T; ++t) {
        if (!fl.template wait_full<P>(cs, lap & 1u, status, kStatusGemm, tally)) return false;
        fl.arrive_empty(cs);
        if (++cs == S) {
            cs = 0;
            ++lap;
        }
    }
    return true;
}

// ----------------------------------------------------------------------------
// Homogeneous K loop, the baseline that specialization is measured against
// (pwwt.cn article, section 1.1: every thread loads the next tile into shared
// memory, a block barrier, every thread computes, a second barrier before the
// buffer is overwritten). No wave has a role: all NW waves issue their share
// of each tile's LDS-DMA loads (the same loads and slot layout as the
// producers above) and all of them compute.
//   S == 1: that loop as written: load t, wait, barrier, compute t, barrier.
//   S >= 2: prefetched: tile t + S - 1 goes into the slot of tile t - 1, which
//           every wave finished reading before the barrier that opened tile t,
//           so one barrier per tile suffices. A tile's fragments are all read
//           before the next loads are issued (the compiler orders LDS reads
//           after outstanding LDS-DMA writes), then its MFMAs run while those
//           loads fly.
// ----------------------------------------------------------------------------
__device__ __forceinline__ void workgroup_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int BM, int BN, int BK, int ES, int NW, int KG, typename Frag, typename Read, typename Mma>
__device__ __forceinline__ void sync_loop(const GemmArgs &a, unsigned char *ring, int wave, int lane, int64_t m0,
                                          int64_t n0, int T, Read read, Mma mma) {
    constexpr int A_BYTES = BM * BK * ES, SLOT = A_BYTES + BK * BN * ES;
    using AD = ADma<BM, BK, ES, NW>;
    using BD = BDma<BN, BK, ES, NW>;
    constexpr int NL = AD::NL + BD::NL;
    static_assert(NL <= 63, "one tile's loads must fit vmcnt");
    const int64_t N = a.N, K = a.K;
    const int S = a.S;
    const int rows_valid = (int)min((int64_t)BM, a.M - m0);
    const unsigned char *A_rows = a.A + (size_t)m0 * (size_t)K * ES;
    AD ad;
    BD bd;
    ad.init(wave, lane, K, rows_valid);
    bd.init(wave, lane, N, n0);
    // tiles loaded ahead of the one being computed
    const int ahead = S == 1 ? 1 : min(S - 1, 1 + 63 / NL);
    int is = 0;  // slot of the next tile to issue
    auto issue = [&](int t) {
        unsigned char *slot = ring + (size_t)is * SLOT;
        ad.issue(slot, wave, A_rows, rows_valid, K, (int64_t)t * BK);
        bd.issue(slot + A_BYTES, wave, a.B, N, K, n0, (int64_t)t * BK);
        if (++is == S) is = 0;
    };
    for (int t = 0; t < min(ahead, T); ++t) issue(t);
    Frag f[KG];
    int cs = 0;  // slot of tile t
    for (int t = 0; t < T; ++t) {
        wait_vmcnt_dyn(min(ahead - 1, T - 1 - t) * NL);  // this wave's part of tile t has landed
        workgroup_barrier();                              // ... and every other wave's
        const unsigned char *slot = ring + (size_t)cs * SLOT;
#pragma unroll
        for (int g = 0; g < KG; ++g) read(f[g], slot, g);
        wait_lgkm0();
        if (S > 1 && t + ahead < T) issue(t + ahead);
#pragma unroll
        for (int g = 0; g < KG; ++g) mma(f[g]);
        if (S == 1) {
            workgroup_barrier();  // every wave is done with the only slot
            if (t + 1 < T) issue(t + 1);
        }
        if (++cs == S) cs = 0;
    }
}

// ----------------------------------------------------------------------------
// fp32 kernel
// ----------------------------------------------------------------------------
template <int BM, int BN, int BK, int P, int CWM, int CWN, bool DMA, bool GR, bool SK = false>
__global__ void __launch_bounds__((P + CWM * CWN) * 64) gemm_f32_kernel(typename KernelArgs<GR>::type ka) {
    static_assert(!SK || (P > 0 && DMA && !GR), "stream-K: specialized LDS-DMA kernels, ordinary launches");
    GemmArgs &a = gemm_args(ka);
    constexpr int NCW = CWM * CWN;
    constexpr int WTM = BM / CWM, WTN = BN / CWN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int QPR = BK / 4;
    constexpr int A_BYTES = BM * BK * 4, B_BYTES = BK * BN * 4, SLOT = A_BYTES + B_BYTES;
    constexpr int KG = BK / 16;
    static_assert(BK % 16 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds + kFlagBytes;
    const int wave = wave_id();
    const int lane = lane_id();

    const LdsFlags fl = init_flags(lds);

    constexpr int kGroupRows = 8 * BN / BM > 0 ? 8 * BN / BM : 1;
    int tm = 0, tn = 0, w = 0;  // tile (ordinary launches) or stream-K worker
    if constexpr (SK) w = xcd_linear(blockIdx.x, a.workers);
    else resolve_tile<kGroupRows, BM, 4>(ka, tm, tn);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int T = (int)((K + BK - 1) / BK);
    const int S = a.S;

    if constexpr (P > 0) {
        if (wave < P) {
            if constexpr (SK) produce_sk<BM, BN, BK, 4, P, NCW, kGroupRows>(a, ring, fl, wave, lane, T, w);
            else produce<BM, BN, BK, 4, P, NCW, DMA>(a, ring, fl, wave, lane, m0, n0, T);
            return;
        }
    }

    // ================= consumer =================
    const int cw = wave - P;
    const int wr = cw / CWN, wc = cw % CWN;
    const int li = lane & 15, q = lane >> 4;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    int a_off[FM], a_swz[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wr * WTM + 16 * i + li;
        a_off[i] = row * QPR * 16;
        a_swz[i] = row_swizzle<QPR>(row);
    }
    int b_chunk[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_chunk[j] = (wc * WTN + 16 * j + li) >> 2;
    const int b_sub = (li & 3) * 4;

    struct Frag {
        f32x4 a[FM];
        float b[FN][4];
    };
    auto read = [&](Frag &f, const unsigned char *slot, int g) {
        const unsigned char *slotB = slot + A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = *reinterpret_cast<const f32x4 *>(slot + a_off[i] + (((4 * g + q) ^ a_swz[i]) << 4));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int k = 16 * g + 4 * q + jj;
            const unsigned char *row = slotB + k * BN * 4 + b_sub;
            const int sw = b_swizzle<4, BN / 4>(k);
#pragma unroll
            for (int j = 0; j < FN; ++j) f.b[j][jj] = *reinterpret_cast<const float *>(row + ((b_chunk[j] ^ sw) << 4));
        }
    };
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[i][jj], f.b[j][jj], acc[i][j], 0, 0, 0);
    };

    // epilogue: C = relu(acc + bias[n]); lane (li, q) holds column li and rows
    // 4q + r of each 16x16 block
    auto epilogue = [&](int64_t m0, int64_t n0) {
        const float *bias = reinterpret_cast<const float *>(a.bias) + n0;
        float *ctile = a.C + m0 * N + n0;
        const int rbase = wr * WTM + 4 * q, cbase = wc * WTN + li;
        const int rows_valid = (int)min((int64_t)BM, M - m0), cols_valid = (int)min((int64_t)BN, N - n0);
        // all bias loads first: stores count in the same counter, so a bias load
        // waited for between stores would also wait for every store before it
        float bv[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = cbase + 16 * j < cols_valid ? bias[cbase + 16 * j] : 0.0f;
        if (rows_valid == BM && cols_valid == BN) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = cbase + 16 * j;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ctile[(int64_t)(rbase + 16 * i + r) * N + col] = relu_f32(acc[i][j][r] + bv[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = cbase + 16 * j;
                if (col >= cols_valid) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = rbase + 16 * i + r;
                        if (row < rows_valid) ctile[(int64_t)row * N + col] = relu_f32(acc[i][j][r] + bv[j]);
                    }
            }
        }
    };

    if constexpr (SK) {
        // stream-K worker: every unit's k range through the same ring, then
        // its epilogue, partial store or fixup
        constexpr int ACC = FM * FN * 4;  // accumulators per lane
        WaitTally tally;
        RingPos pos;
        SkUnit un;
        bool ok = true;
        for (int u = 0; ok && sk_unit(a, T, w, u, un); ++u) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            ok = consume_ring<KG, P, Frag, FM + 4 * FN>(un.ke - un.kb, S, ring, SLOT, fl, a.status, tally, read, mma,
                                                         pos);
            if (!ok) break;
            int utm, utn;
            swizzle_tile<kGroupRows>(un.tile, a.tiles_m, a.tiles_n, utm, utn);
            // The lane index through an empty asm: addresses derived from it
            // are formed here, not hoisted out of the unit loop where they
            // would stay live (and spill) through the K loop.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            if (un.npieces > 1) {
                // a piece: store it in its partial slot, fragment-major
                // (fragment q of lane l as 16 bytes at (q * 64 + l) * 16), at
                // device scope (written through to memory, not left in this
                // XCD's L2); once the stores have completed, count it on the
                // tile. The wave whose count completes the tile adds every
                // piece back in piece order, reading at device scope, and
                // runs the epilogue; the others go on to their next unit.
                const __amdgpu_buffer_rsrc_t rp =
                    make_rsrc(a.part + ((size_t)un.slot * NCW + cw) * (64 * ACC), 64 * ACC * 4);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rp, 16 * ln,
                                                               (i * FN + j) * 1024, kScopeDevice);
                wait_vmcnt<0>();
                unsigned *cnt = a.cnt + (size_t)un.sk_tile * NCW + cw;
                uint32_t before = 0;
                if (ln == 0) before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (__builtin_amdgcn_readfirstlane(before) + 1 != (uint32_t)un.npieces) continue;
                asm volatile("" ::: "memory");  // no load of a piece moves above the count
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                for (int p = 0; p < un.npieces; ++p) {
                    const int slot = p == 0 ? un.first_slot : 2 * (un.first + p);
                    const __amdgpu_buffer_rsrc_t rq =
                        make_rsrc(a.part + ((size_t)slot * NCW + cw) * (64 * ACC), 64 * ACC * 4);
                    // NB fragments in flight at a time: all loads of a batch
                    // issue before its adds
                    constexpr int NQ = FM * FN, NB = NQ < 8 ? NQ : 8;
                    static_assert(NQ % NB == 0, "fragments per batch");
#pragma unroll
                    for (int q0 = 0; q0 < NQ; q0 += NB) {
                        u32x4 t[NB];
#pragma unroll
                        for (int q = 0; q < NB; ++q)
                            t[q] = __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * ln, (q0 + q) * 1024, kScopeDevice);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < NB; ++q)
                            acc[(q0 + q) / FN][(q0 + q) % FN] += __builtin_bit_cast(f32x4, t[q]);
                    }
                }
            }
            // epilogue through a buffer resource at the tile's origin (as in
            // the single-fragment bf16 kernels): one lane offset, each store's
            // row and column block added into a temporary; rows past M fall
            // outside the range (which covers the VGPR offset), columns past
            // N are masked per lane
            const int64_t um0 = (int64_t)utm * BM, un0 = (int64_t)utn * BN;
            const int rbase = wr * WTM + 4 * (ln >> 4), cbase = wc * WTN + (ln & 15);
            const int rows_valid = (int)min((int64_t)BM, M - um0), cols_valid = (int)min((int64_t)BN, N - un0);
            const float *bias = reinterpret_cast<const float *>(a.bias) + un0;
            float bv[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) bv[j] = cbase + 16 * j < cols_valid ? bias[cbase + 16 * j] : 0.0f;
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc(a.C + um0 * N + un0, (uint32_t)(((int64_t)(rows_valid - 1) * N + cols_valid) * 4));
            const uint32_t voff = (uint32_t)(rbase * (int)N + cbase) * 4u;
            const uint32_t row4 = (uint32_t)N * 4u;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if (cbase + 16 * j >= cols_valid) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_uint(relu_f32(acc[i][j][r] + bv[j])), rc,
                            voff + (uint32_t)(16 * i + r) * row4 + 64u * j, 0, 0);
            }
        }
        if (!ok) {
            atomicOr(a.status, kStatusTimeout | kStatusGemm);
            return;
        }
        publish_tally(a.stats ? a.stats + kStatGemmConsumer : nullptr, tally);
        return;
    }

    if constexpr (P == 0) {
        static_assert(DMA, "the homogeneous loop loads by LDS-DMA");
        sync_loop<BM, BN, BK, 4, NCW, KG, Frag>(a, ring, cw, lane, m0, n0, T, read, mma);
    } else {
        WaitTally tally;
        RingPos pos;
        if (!consume_ring<KG, P, Frag, FM + 4 * FN>(T, S, ring, SLOT, fl, a.status, tally, read, mma, pos)) return;
        publish_tally(a.stats ? a.stats + kStatGemmConsumer : nullptr, tally);
    }

    epilogue(m0, n0);
}

// ----------------------------------------------------------------------------
// bf16 kernel
// ----------------------------------------------------------------------------
// GK: k per fragment group (16 or 32). A deeper group gives each consumer
// step more MFMA work to hide the next group's LDS reads behind.
template <int BM, int BN, int BK, int P, int CWM, int CWN, bool DMA, int GK, bool GR>
__global__ void __launch_bounds__((P + CWM * CWN) * 64) gemm_bf16_kernel(typename KernelArgs<GR>::type ka) {
    GemmArgs &a = gemm_args(ka);
    constexpr int NCW = CWM * CWN;
    constexpr int WTM = BM / CWM, WTN = BN / CWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int QPR = BK / 8;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2, SLOT = A_BYTES + B_BYTES;
    constexpr int GS = GK / 16;  // 16-deep MFMA steps per group
    constexpr int KG = BK / GK;
    static_assert(BK % GK == 0 && (GK == 16 || GK == 32) && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds + kFlagBytes;
    const int wave = wave_id();
    const int lane = lane_id();

    const LdsFlags fl = init_flags(lds);

    int tm, tn;
    resolve_tile<(8 * BN / BM > 0 ? 8 * BN / BM : 1), BM, 2>(ka, tm, tn);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int T = (int)((K + BK - 1) / BK);
    const int S = a.S;

    if constexpr (P > 0) {
        if (wave < P) {
            produce<BM, BN, BK, 2, P, NCW, DMA>(a, ring, fl, wave, lane, m0, n0, T);
            return;
        }
    }

    // ================= consumer =================
    const int cw = wave - P;
    const int wr = cw / CWN, wc = cw % CWN;
    const int li = lane & 31, h = lane >> 5;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    int a_off[FM], a_swz[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wr * WTM + 32 * i + li;
        a_off[i] = row * QPR * 16;
        a_swz[i] = chunk_param<QPR>(row);
    }
    // B: in 16-lane group g16 = lane / 16 (k half h = g16 / 2, column half
    // g16 % 2), lane i' = lane % 16 points at columns 4 * (i' % 4) .. + 3 of k
    // row 16 g + 8 h + 4 r + i' / 4 (r = 0, 1: the two halves of the lane's 8
    // k values); the transpose read hands lane i' its column's 4 rows.
    const int ip = lane & 15;
    const int b_row = (8 * h + (ip >> 2)) * BN * 2;
    const int b_sw = b_swizzle<2, BN / 8>(ip >> 2);  // k = 16g + 8h + 4r + ip/4, so k mod 4 = ip/4
    int b_col[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = wc * WTN + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (ip & 3);
        b_col[j] = (((n >> 3) ^ b_sw) << 4) + 8 * (ip & 1);
    }
    // The two halves of a B fragment stay separate until the MFMA that uses
    // them, so joining them (if the register allocator needs a copy) happens
    // after the reads have landed, not while they are in flight.
    struct Frag {
        bf16x8 a[GS][FM];
        v4i16 b_lo[GS][FN], b_hi[GS][FN];
    };
    auto read = [&](Frag &f, const unsigned char *slot, int g) {
#pragma unroll
        for (int ks = 0; ks < GS; ++ks) {
            const int step = g * GS + ks;
            const int c = 2 * step + h;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                f.a[ks][i] = *reinterpret_cast<const bf16x8 *>(slot + a_off[i] + (chunk_at<QPR>(c, a_swz[i]) << 4));
            const unsigned char *slotB = slot + A_BYTES + b_row + 16 * step * BN * 2;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                f.b_lo[ks][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(slotB + b_col[j]));
                f.b_hi[ks][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(slotB + 4 * BN * 2 + b_col[j]));
            }
        }
    };
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int ks = 0; ks < GS; ++ks)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(f.b_lo[ks][j], f.b_hi[ks][j], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], b, acc[i][j], 0, 0, 0);
            }
    };

    // More than 8 waves: three share a SIMD (168 registers each), so the
    // consumers keep a single fragment set (consume_lean).
    constexpr bool LEAN = P > 0 && P + NCW > 8;
    if constexpr (P == 0) {
        static_assert(DMA, "the homogeneous loop loads by LDS-DMA");
        sync_loop<BM, BN, BK, 2, NCW, KG, Frag>(a, ring, cw, lane, m0, n0, T, read, mma);
    } else if constexpr (LEAN) {
        if (wr * WTM >= M - m0 || wc * WTN >= N - n0) {  // nothing of this wave's part is in C
            WaitTally tally;
            if (release_only<P>(T, S, fl, a.status, tally))
                publish_tally(a.stats ? a.stats + kStatGemmConsumer : nullptr, tally);
            return;
        }
        constexpr int KS = BK / 16;
        struct LeanFrag {
            bf16x8 a[FM];
            v4i16 lo[FN], hi[FN];
        };
        LeanFrag lf;
        // One lane register per operand. A: row blocks 32 rows apart share the
        // row swizzle for 4 or 8 chunks per row (it depends on the row mod 16),
        // 2 * step + h = (2 * step) ^ h, and a row's start is a multiple of its
        // QPR * 16 bytes while the chunk offset is below that, so
        // address = slot + 32 i QPR 16 + (a_lane ^ 32 step). B: column blocks
        // 32 apart move the chunk index by 4 j, a bit the within-wave column
        // bits never set, so b_col[j] = b_col[0] ^ 64 j; the row offset is a
        // multiple of the row's BN * 2 bytes, above every column offset.
        static_assert(QPR == 4 || QPR == 8, "lean walk: k tiles of 32 or 64");
        const uint32_t a_lane = (uint32_t)a_off[0] | (uint32_t)((h ^ a_swz[0]) << 4);
        const uint32_t b_lane = (uint32_t)b_row | (uint32_t)b_col[0];
        auto rd_a = [&](int i, const unsigned char *slot, int step) {
            lf.a[i] = *reinterpret_cast<const bf16x8 *>(slot + i * 32 * QPR * 16 + (a_lane ^ (uint32_t)(32 * step)));
        };
        auto rd_b = [&](int j, const unsigned char *slot, int step) {
            const unsigned char *p = slot + A_BYTES + 16 * step * BN * 2 + (b_lane ^ (uint32_t)(64 * j));
            lf.lo[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
            lf.hi[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * BN * 2));
        };
        auto prime = [&](const unsigned char *slot, int step) {
#pragma unroll
            for (int j = 0; j < FN; ++j) rd_b(j, slot, step);
#pragma unroll
            for (int i = 0; i < FM; ++i) rd_a(i, slot, step);
        };
        // One k step: column block j's MFMAs over every row block i; B[j] is
        // re-read once its FM MFMAs have issued, and in the last column block
        // each A[i] right after its MFMA. The order is pinned (no instruction
        // crosses a sched_barrier(0)), so every re-read follows the last use
        // of the registers it overwrites and the two never need to coexist.
        auto step = [&](const unsigned char *nslot, int nstep, auto mid) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const bf16x8 b =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lf.lo[j], lf.hi[j], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf.a[i], b, acc[i][j], 0, 0, 0);
                    if (j == FN - 1) {
                        __builtin_amdgcn_sched_barrier(0);
                        rd_a(i, nslot, nstep);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (j == 0) mid();
                rd_b(j, nslot, nstep);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        WaitTally tally;
        if (!consume_lean<KS, P, NCW>(T, S, ring, SLOT, fl, a.status, tally, prime, step)) return;
        publish_tally(a.stats ? a.stats + kStatGemmConsumer : nullptr, tally);
    } else {
        WaitTally tally;
        if (!consume_tiles<KG, P, Frag, GS * FM * FN>(T, S, ring, SLOT, fl, a.status, tally, read, mma)) return;
        publish_tally(a.stats ? a.stats + kStatGemmConsumer : nullptr, tally);
    }

    // epilogue: lane (li, h) holds column li of each 32x32 block and rows
    // 8*(r/4) + 4*h + (r%4) of its 16 registers
    const uint16_t *bias = reinterpret_cast<const uint16_t *>(a.bias) + n0;
    float *ctile = a.C + m0 * N + n0;
    const int rbase = wr * WTM + 4 * h, cbase = wc * WTN + li;
    const int rows_valid = (int)min((int64_t)BM, M - m0), cols_valid = (int)min((int64_t)BN, N - n0);
    float bv[FN];  // all bias loads before the first store, as in the fp32 epilogue
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = cbase + 32 * j < cols_valid ? bf16_to_f32(bias[cbase + 32 * j]) : 0.0f;
    if constexpr (LEAN) {
        // Buffer stores through a resource at the tile's origin: each lane
        // keeps one 32-bit offset (its row and column) and adds the store's
        // row and column block (a scalar) into a temporary per store. The
        // resource's range ends after the last valid element, so rows past M
        // are dropped by the range check, which covers the VGPR offset (the
        // scalar-offset operand stays 0); columns past N (which would land in
        // the next row) are masked per lane. 64-bit addresses per store took
        // registers the 128 accumulators do not leave. The planner picks
        // these kernels only when BM rows of C span less than 2^31 bytes.
        const uint32_t nbytes = (uint32_t)(((int64_t)(rows_valid - 1) * N + cols_valid) * 4);
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(ctile, nbytes);
        const uint32_t voff = (uint32_t)(rbase * (int)N + cbase) * 4u;
        const uint32_t row4 = (uint32_t)N * 4u;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if (cbase + 32 * j >= cols_valid) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t soff = (uint32_t)(32 * i + 8 * (r >> 2) + (r & 3)) * row4 + 128u * j;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(relu_f32(acc[i][j][r] + bv[j])), rc,
                                                          voff + soff, 0, 0);
                }
        }
        return;
    }
    if (rows_valid == BM && cols_valid == BN) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = cbase + 32 * j;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    ctile[(int64_t)(rbase + 32 * i + 8 * (r >> 2) + (r & 3)) * N + col] =
                        relu_f32(acc[i][j][r] + bv[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = cbase + 32 * j;
            if (col >= cols_valid) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rbase + 32 * i + 8 * (r >> 2) + (r & 3);
                    if (row < rows_valid) ctile[(int64_t)row * N + col] = relu_f32(acc[i][j][r] + bv[j]);
                }
        }
    }
}

namespace {

// The stream-K instantiation of an fp32 variant: built for the specialized
// LDS-DMA kernels only.
template <int BM, int BN, int BK, int P, int CWM, int CWN, bool DMA>
constexpr const void *f32_sk_kernel() {
    if constexpr (P > 0 && DMA) return reinterpret_cast<const void *>(&gemm_f32_kernel<BM, BN, BK, P, CWM, CWN, DMA,
                                                                                        false, true>);
    else return nullptr;
}

#define WSG_F32(BM, BN, BK, P, CWM, CWN, DMA)                                                              \
    {WSG_FP32, BM, BN, BK, P, CWM, CWN, DMA, 16,                                                           \
     reinterpret_cast<const void *>(&gemm_f32_kernel<BM, BN, BK, P, CWM, CWN, DMA, false>),                \
     reinterpret_cast<const void *>(&gemm_f32_kernel<BM, BN, BK, P, CWM, CWN, DMA, true>),                 \
     f32_sk_kernel<BM, BN, BK, P, CWM, CWN, DMA>()}
#define WSG_BF(BM, BN, BK, P, CWM, CWN, DMA, GK)                                                           \
    {WSG_BF16, BM, BN, BK, P, CWM, CWN, DMA, GK,                                                           \
     reinterpret_cast<const void *>(&gemm_bf16_kernel<BM, BN, BK, P, CWM, CWN, DMA, GK, false>),           \
     reinterpret_cast<const void *>(&gemm_bf16_kernel<BM, BN, BK, P, CWM, CWN, DMA, GK, true>), nullptr}

// When the caller leaves fields at 0, the first variant (in this order) whose
// tile matches the size class and whose ring fits in LDS wins.
const GemmVariant kGemmVariants[] = {
    // fp32, wave-specialized, LDS-DMA producer. One consumer wave per SIMD
    // first (a second one would stall the first one's LDS reads while it
    // streams fp32 MFMAs), with one producer wave per SIMD: a producer shares
    // its SIMD with a consumer's MFMA stream, which slows its LDS-DMA issue.
    WSG_F32(256, 128, 32, 4, 2, 2, true),  WSG_F32(256, 128, 16, 4, 2, 2, true),
    WSG_F32(256, 128, 32, 2, 2, 2, true),  WSG_F32(256, 128, 16, 2, 2, 2, true),
    WSG_F32(128, 128, 32, 2, 2, 2, true),  WSG_F32(128, 128, 16, 1, 2, 2, true),
    WSG_F32(128, 128, 16, 2, 2, 2, true),
    // 64 x 64 tiles (small problems, where each k tile's load latency is
    // the critical path): four producer waves issue a tile's eight loads two
    // each (measured on MI355X, 10 launches between events: 256^3 2.50 ->
    // 2.80 TFLOP/s and 512^3 11.1 -> 12.6 against one producer issuing all
    // eight; bit-identical)
    WSG_F32(64, 64, 16, 4, 2, 2, true),    WSG_F32(64, 64, 16, 2, 2, 2, true),
    WSG_F32(64, 64, 16, 1, 2, 2, true),
    WSG_F32(256, 128, 32, 1, 2, 2, true),  WSG_F32(256, 128, 32, 2, 4, 2, true),
    WSG_F32(256, 128, 16, 2, 4, 2, true),  WSG_F32(256, 128, 32, 1, 4, 2, true),
    WSG_F32(256, 128, 16, 1, 4, 2, true),  WSG_F32(256, 128, 32, 4, 4, 2, true),
    WSG_F32(128, 256, 16, 2, 2, 4, true),
    // fp32, register-staged producer (any shape)
    WSG_F32(256, 128, 16, 2, 4, 2, false), WSG_F32(128, 128, 16, 1, 2, 2, false),
    WSG_F32(64, 64, 16, 1, 2, 2, false),
    // fp32, homogeneous (no producer waves)
    WSG_F32(256, 128, 32, 0, 2, 2, true),  WSG_F32(256, 128, 16, 0, 2, 2, true),
    WSG_F32(256, 128, 32, 0, 4, 2, true),  WSG_F32(256, 128, 16, 0, 4, 2, true),
    WSG_F32(128, 128, 32, 0, 2, 2, true),
    WSG_F32(64, 64, 16, 0, 2, 2, true),
    // bf16, wave-specialized. Four producer waves first (one per SIMD): with
    // consumers walking the ring a tile at a time, 8192^3 measured 934 / 822
    // TFLOP/s for 4 / 2 producers at S = 2, 1019 / 1007 at S = 3 and 846 / 840
    // at S = 4 (k = 32 tiles); with one producer, consumers found the next
    // tile unpublished at 41% of their waits.
    WSG_BF(256, 128, 64, 4, 2, 2, true, 32),  WSG_BF(256, 128, 48, 4, 2, 2, true, 16),
    WSG_BF(256, 128, 48, 2, 2, 2, true, 16),  WSG_BF(256, 128, 32, 4, 2, 2, true, 32),
    WSG_BF(256, 128, 64, 2, 2, 2, true, 32),  WSG_BF(256, 128, 64, 2, 2, 2, true, 16),
    WSG_BF(256, 128, 32, 2, 2, 2, true, 32),  WSG_BF(256, 128, 64, 1, 2, 2, true, 32),
    WSG_BF(256, 128, 32, 1, 2, 2, true, 32),  WSG_BF(256, 128, 32, 1, 2, 2, true, 16),
    WSG_BF(256, 128, 64, 4, 2, 2, true, 16),
    WSG_BF(256, 128, 32, 4, 2, 2, true, 16),  WSG_BF(256, 128, 32, 2, 2, 2, true, 16),
    WSG_BF(128, 128, 64, 1, 2, 2, true, 32),  WSG_BF(128, 128, 32, 1, 2, 2, true, 16),
    // 64 x 64: four producers, as for fp32 (measured on MI355X: 256^3 5.02 ->
    // 5.41 TFLOP/s, 512^3 26.0 -> 28.4 against one producer; bit-identical)
    WSG_BF(64, 64, 32, 4, 2, 2, true, 16),    WSG_BF(64, 64, 32, 2, 2, 2, true, 16),
    WSG_BF(64, 64, 32, 1, 2, 2, true, 16),    WSG_BF(256, 128, 32, 1, 2, 2, false, 32),
    WSG_BF(128, 128, 32, 1, 2, 2, false, 16), WSG_BF(64, 64, 32, 1, 2, 2, false, 16),
    // bf16, 256 x 256 tiles: 8 consumer waves of 128 x 64 and 4 producers,
    // three waves per SIMD, consumers on the single-fragment walk
    WSG_BF(256, 256, 64, 4, 2, 4, true, 16),  WSG_BF(256, 256, 32, 4, 2, 4, true, 16),
    // bf16, homogeneous
    WSG_BF(256, 128, 64, 0, 2, 2, true, 32),  WSG_BF(256, 128, 64, 0, 4, 2, true, 32),
    WSG_BF(256, 128, 48, 0, 2, 2, true, 16),
    WSG_BF(256, 256, 32, 0, 2, 4, true, 16),
    WSG_BF(256, 128, 32, 0, 2, 2, true, 32),  WSG_BF(128, 128, 32, 0, 2, 2, true, 16),
    WSG_BF(64, 64, 32, 0, 2, 2, true, 16),
};

}  // namespace

int plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B, int stages,
              const wsg_config *cfg, const DeviceInfo &dev, GemmPlan *plan, std::string *err) {
    if (stages < 1) {
        *err = "stages must be >= 1";
        return WSG_EINVAL;
    }
    if (stages > kMaxStages) {
        *err = "stages above the flag area's limit of " + std::to_string(kMaxStages);
        return WSG_EUNSUPPORTED;
    }
    const int esz = dtype == WSG_FP32 ? 4 : 2;
    int BM = cfg && cfg->BM ? cfg->BM : 0, BN = cfg && cfg->BN ? cfg->BN : 0, BK = cfg && cfg->BK ? cfg->BK : 0;
    int P = cfg && cfg->producer_waves ? cfg->producer_waves : 0;
    int CW = cfg && cfg->consumer_waves ? cfg->consumer_waves : 0;
    int GK = cfg && cfg->group_k ? cfg->group_k : 0;
    const bool force_general = cfg && (cfg->flags & WSG_FLAG_GENERAL_PRODUCER);
    const bool homogeneous = cfg && (cfg->flags & WSG_FLAG_HOMOGENEOUS);
    if (homogeneous && (P || force_general)) {
        *err = "the homogeneous kernel has no producer waves and loads by LDS-DMA: leave producer_waves 0 and "
               "WSG_FLAG_GENERAL_PRODUCER clear";
        return WSG_EINVAL;
    }
    // the DMA producer needs 16-byte aligned rows and offsets within 31 bits
    const int align_elems = 16 / esz;
    const bool aligned = K % align_elems == 0 && N % align_elems == 0 && ((uintptr_t)A % 16) == 0 &&
                         ((uintptr_t)B % 16) == 0;
    const bool default_tile = !BM && !BN && !BK;
    if (default_tile) {
        // default tile by problem size: small problems need more workgroups
        const int64_t big = (M + 255) / 256 * ((N + 127) / 128);
        const int64_t mid = (M + 127) / 128 * ((N + 127) / 128);
        // fp32 with fewer 256 x 128 tiles than CUs but a deep K: keep the big
        // tile and let a stream-K launch split the k steps over every CU, if
        // 128 x 128 tiles would leave CUs idle or K is very deep (measured on
        // MI355X, TFLOP/s, stream-K 256 x 128 against the smaller default:
        // 1024 x 1024 x 16384 117 / 40; 1024 x 2048 x 2048 91 / 58;
        // 2048 x 2048 x 8192 130 / 117; but 2048 x 2048 x 1024 98 / 105 and
        // 2048^3 115 / 113, where 256 tiles of 128 x 128 fill the chip)
        const int64_t steps_per_cu = big * ((K + 31) / 32) / dev.cu_count;
        const bool deep_k = dtype == WSG_FP32 && !homogeneous && !force_general && aligned &&
                            !(cfg && (cfg->flags & WSG_FLAG_NO_STREAM_K)) && steps_per_cu >= kStreamKMinSteps &&
                            (mid < (int64_t)dev.cu_count || steps_per_cu >= 4 * kStreamKMinSteps);
        if (big >= (int64_t)dev.cu_count || deep_k) {
            BM = 256;
            BN = 128;
        } else if (mid >= (int64_t)dev.cu_count / 2) {
            BM = 128;
            BN = 128;
        } else {
            BM = 64;
            BN = 64;
        }
    }
    if (homogeneous && !aligned) {
        *err = "the homogeneous kernel loads by LDS-DMA: K and N must be multiples of " + std::to_string(align_elems) +
               " and A and B 16-byte aligned";
        return WSG_EUNSUPPORTED;
    }
    bool lds_short = false;
    auto search = [&](int qBM, int qBN) -> const GemmVariant * {
        for (int pass = 0; pass < 2; ++pass) {
            const bool want_dma = pass == 0;
            if (want_dma && (force_general || !aligned)) continue;
            for (const GemmVariant &v : kGemmVariants) {
                if (v.dtype != dtype || v.dma != want_dma || (v.P == 0) != homogeneous) continue;
                if ((qBM && v.BM != qBM) || (qBN && v.BN != qBN) || (BK && v.BK != BK)) continue;
                if ((P && v.P != P) || (CW && v.CWM * v.CWN != CW) || (GK && v.GK != GK)) continue;
                if (want_dma && ((int64_t)v.BM * K * esz >= 0x7FFFFFFF || (int64_t)v.BK * N * esz >= 0x7FFFFFFF))
                    continue;
                // more than 8 waves: the buffer-store epilogue addresses BM rows of C with 32-bit offsets
                if (v.P + v.CWM * v.CWN > 8 && (int64_t)v.BM * N * 4 >= 0x7FFFFFFF) continue;
                const size_t need = (size_t)kFlagBytes + (size_t)stages * (size_t)(v.BM * v.BK + v.BK * v.BN) * esz;
                if (need > dev.max_lds) {
                    lds_short = true;  // a smaller BK of the same tile may still fit
                    continue;
                }
                return &v;
            }
        }
        return nullptr;
    };
    // bf16 defaults on large problems: 256 x 256 tiles (8 consumer and 4
    // producer waves) where their ring fits, 64 deep for up to 2 stages and
    // 32 deep for 4; at 3 stages the 256 x 128 x 64 tile is faster (measured
    // on MI355X, 8192^3 in one interleaved run: 256 x 256 x 32 at S = 4 1016
    // TFLOP/s against 910 for 256 x 128 x 48; at S = 3, 1023 against 1073
    // for 256 x 128 x 64; at S = 2, 1102 for 256 x 256 x 64).
    const GemmVariant *pick = nullptr;
    if (default_tile && dtype == WSG_BF16 && !homogeneous && !P && !CW && !GK && stages != 3 && BM == 256 &&
        (M + 255) / 256 * ((N + 255) / 256) >= (int64_t)dev.cu_count)
        pick = search(256, 256);
    if (!pick) {
        lds_short = false;
        pick = search(BM, BN);
    }
    if (!pick && lds_short) {
        *err = "no built " + std::to_string(BM) + "x" + std::to_string(BN) + " tile fits a " + std::to_string(stages) +
               "-stage ring in the " + std::to_string(dev.max_lds) + " bytes of LDS a workgroup may use";
        return WSG_EUNSUPPORTED;
    }
    if (!pick) {
        *err = "no GEMM kernel built for tile " + std::to_string(BM) + "x" + std::to_string(BN) + "x" +
               std::to_string(BK) + " with " + std::to_string(P) + " producer and " + std::to_string(CW) +
               " consumer waves";
        return WSG_EUNSUPPORTED;
    }
    const size_t slot = (size_t)(pick->BM * pick->BK + pick->BK * pick->BN) * esz;
    const size_t lds = (size_t)kFlagBytes + (size_t)stages * slot;
    if (lds > dev.max_lds) {
        *err = "ring needs " + std::to_string(lds) + " bytes of LDS, the device allows " +
               std::to_string(dev.max_lds) + " per workgroup";
        return WSG_EUNSUPPORTED;
    }
    const int64_t tiles_m = (M + pick->BM - 1) / pick->BM, tiles_n = (N + pick->BN - 1) / pick->BN;
    if (tiles_m * tiles_n > 0x7FFFFFFF) {
        *err = "too many output tiles";
        return WSG_EUNSUPPORTED;
    }
    plan->v = pick;
    plan->stages = stages;
    plan->tiles_m = tiles_m;
    plan->tiles_n = tiles_n;
    plan->lds_bytes = lds;
    return WSG_OK;
}

namespace {

void fill_common(const LaunchCtx &ctx, const GemmPlan &plan, GemmArgs &args) {
    args.S = plan.stages;
    args.tiles_n = (int)plan.tiles_n;
    args.status = ctx.dev.status;
    args.stats = ctx.wait_stats ? ctx.dev.stats : nullptr;
}

int launch_with(const LaunchCtx &ctx, const GemmPlan &plan, const void *kernel, void *kernel_args, int64_t grid,
                std::string *err) {
    const int threads = (plan.v->P + plan.v->CWM * plan.v->CWN) * 64;
    const int rc = prepare_kernel(kernel, ctx.dev, err);
    if (rc != WSG_OK) return rc;
    void *kargs[] = {kernel_args};
    hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(threads), kargs, plan.lds_bytes, ctx.stream);
    if (e != hipSuccess) {
        *err = std::string("gemm launch: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    return WSG_OK;
}

GemmArgs make_args(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias, float *C) {
    GemmArgs args;
    args.A = static_cast<const unsigned char *>(A);
    args.B = static_cast<const unsigned char *>(B);
    args.bias = static_cast<const unsigned char *>(bias);
    args.C = C;
    args.M = M;
    args.N = N;
    args.K = K;
    return args;
}

}  // namespace

// Zero the stream-K counters before a launch (a kernel, not a memset, so that
// the two launches can be captured in a graph).
__global__ void sk_clear_kernel(unsigned *cnt, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) cnt[i] = 0u;
}

SkShape plan_stream_k(const GemmPlan &plan, int64_t M, int64_t N, int64_t K, int flags, const DeviceInfo &dev) {
    SkShape sk;
    const GemmVariant &v = *plan.v;
    if (!v.sk_kernel || (flags & WSG_FLAG_NO_STREAM_K) || M == 0 || N == 0 || K == 0) return sk;
    // the buffer-store epilogue and partial slots use 32-bit offsets
    if ((int64_t)v.BM * N * 4 >= 0x7FFFFFFF) return sk;
    const int threads = (v.P + v.CWM * v.CWN) * 64;
    const int64_t workers = (int64_t)dev.cu_count * blocks_per_cu(v.sk_kernel, dev, threads, plan.lds_bytes);
    const int64_t tiles = plan.tiles_m * plan.tiles_n;
    const int64_t rounds = tiles / workers, rem = tiles % workers;
    if (!(flags & WSG_FLAG_STREAM_K)) {
        // a tail worth spreading: a last round at most 90% full (480 tiles on
        // 256 CUs: 224 in the last round) after at least one whole round, or
        // fewer 256 x 128 (or larger) tiles than workers but enough k steps
        // to give each worker kStreamKMinSteps of them; smaller tiles were
        // chosen to fill the chip (split 128 x 128 tiles ran slower than
        // whole ones: 88 against 105 TFLOP/s on 2048 x 2048 x 1024)
        const int64_t steps = tiles * ((K + v.BK - 1) / v.BK);
        const bool tail = rounds >= 1 && rem > 0 && rem * 10 <= workers * 9;
        const bool deep = rounds == 0 && v.BM * v.BN >= 256 * 128 && steps >= kStreamKMinSteps * workers;
        if (!tail && !deep) return sk;
    }
    if (2 * workers * (int64_t)v.BM * v.BN * 4 >= 0x7FFFFFFF) return sk;
    sk.use = true;
    sk.workers = (int)workers;
    sk.dp_tiles = rem == 0 ? (rounds - 1) * workers : rounds * workers;  // forced with no tail: split the last round
    sk.sk_tiles = tiles - sk.dp_tiles;
    sk.part_bytes = (size_t)2 * workers * v.BM * v.BN * 4;  // two pieces per worker
    sk.cnt_bytes = ((size_t)sk.sk_tiles * v.CWM * v.CWN * 4 + 255) / 256 * 256;
    return sk;
}

int launch_gemm(const LaunchCtx &ctx, const GemmPlan &plan, int64_t M, int64_t N, int64_t K, const void *A,
                const void *B, const void *bias, float *C, const SkShape *sk, void *ws, std::string *err) {
    if (M == 0 || N == 0) return WSG_OK;
    GemmArgs args = make_args(M, N, K, A, B, bias, C);
    fill_common(ctx, plan, args);
    args.tiles_m = (int)plan.tiles_m;
    args.dp_tiles = args.sk_tiles = args.workers = 0;
    args.part = nullptr;
    args.cnt = nullptr;
    if (!sk || !sk->use) return launch_with(ctx, plan, plan.v->kernel, &args, plan.tiles_m * plan.tiles_n, err);
    args.dp_tiles = (int)sk->dp_tiles;
    args.sk_tiles = (int)sk->sk_tiles;
    args.workers = sk->workers;
    args.part = static_cast<float *>(ws);
    args.cnt = reinterpret_cast<unsigned *>(static_cast<unsigned char *>(ws) + sk->part_bytes);
    const int ncnt = (int)(sk->sk_tiles * plan.v->CWM * plan.v->CWN);
    unsigned *cnt = args.cnt;
    void *cargs[] = {&cnt, (void *)&ncnt};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&sk_clear_kernel), dim3((ncnt + 255) / 256),
                                   dim3(256), cargs, 0, ctx.stream);
    if (e != hipSuccess) {
        *err = std::string("stream-K counter clear: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    return launch_with(ctx, plan, plan.v->sk_kernel, &args, sk->workers, err);
}

int launch_grouped_gemm(const LaunchCtx &ctx, const GemmPlan &plan, int groups, const int64_t *group_rows, int64_t N,
                        int64_t K, const void *A, const void *B, const void *bias, float *C, std::string *err) {
    if (groups < 1 || groups > WSG_MAX_GROUPS) {
        *err = "groups must be in 1.." + std::to_string(WSG_MAX_GROUPS);
        return WSG_EUNSUPPORTED;
    }
    if (N == 0) return WSG_OK;
    GroupedArgs ga;
    GroupTable &gt = ga.gt;
    gt.n = groups;
    gt.row0[0] = 0;
    gt.tile0[0] = 0;
    int64_t tiles = 0;
    for (int e = 0; e < groups; ++e) {
        gt.row0[e + 1] = gt.row0[e] + group_rows[e];
        tiles += (group_rows[e] + plan.v->BM - 1) / plan.v->BM * plan.tiles_n;
        if (tiles > 0x7FFFFFFF) {
            *err = "too many output tiles";
            return WSG_EUNSUPPORTED;
        }
        gt.tile0[e + 1] = (int)tiles;
    }
    for (int e = groups + 1; e <= WSG_MAX_GROUPS; ++e) {
        gt.row0[e] = gt.row0[groups];
        gt.tile0[e] = gt.tile0[groups];
    }
    if (tiles == 0) return WSG_OK;
    ga.a = make_args(gt.row0[groups], N, K, A, B, bias, C);
    fill_common(ctx, plan, ga.a);
    ga.a.tiles_m = 0;  // per expert, set on the device
    return launch_with(ctx, plan, plan.v->grouped_kernel, &ga, tiles, err);
}

}  // namespace wsg
