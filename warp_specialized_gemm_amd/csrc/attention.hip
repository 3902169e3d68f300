// attention.hip - scaled dot-product attention forward, the second consumer
// type ("GPU warp specialization", aicassindra.com, names attention beside
// GEMM among the kernels built on producer and consumer warps):
//   O = softmax(scale * Q K^T [causal mask]) V   per (batch, head),
// bf16 Q, K, V, fp32 softmax statistics and accumulation, fp32 O.
//
// Same ring as the GEMM: producer waves stream 64-key tiles of K and V into
// S LDS slots by LDS-DMA (K in the GEMM's A layout, rows of D; V in its B
// layout, rows of D columns; keys past Skv load as zeros and are masked);
// consumer waves wait for a full slot, compute on it and release it.
//
// A workgroup owns 32 queries of one head per consumer wave (4 or 7 waves),
// with their Q rows in registers for the whole kernel. A consumer needs over
// 200 registers, so a SIMD holds two waves and a CU one workgroup: with 4
// consumers each SIMD runs one of them and its softmax leaves the matrix unit
// idle; with 7 (one producer, eight waves) three SIMDs run two consumers whose
// softmax and MFMAs can overlap. Per key
// tile a consumer computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K
// rows from LDS, B = Q^T from registers), so a lane's accumulators hold the
// scores of ONE query (lane l: query l mod 32) for 32 of the 64 keys; lane l
// and lane l ^ 32 share a query. Online softmax per query (running max m and
// sum l, base-2 exponentials of pre-scaled scores), then O^T += V^T P^T with
// A = V^T (LDS transpose reads of the V tile) and B = P^T taken from the
// score accumulators in place, rounded to bf16. The MFMA's k order is the
// key order the score accumulators happen to hold (lane half h has keys
// 4h..4h+3 and 8+4h..8+4h+3 of each 16), and the V^T reads follow the same
// permutation, so no data moves between lanes. O^T keeps each lane on one
// query as well, so the rescale by exp2(m_old - m_new) is one multiply per
// register. At the end O = O^T / l (zero rows for a query that sees no key).
#include "internal.hpp"
#include "ring.hpp"
#include "tiles.hpp"

namespace wsg {

struct AttnArgs {
    const unsigned char *Q, *K, *V;  // bf16 bits; Q (BH, Sq, D), K and V (BH, Skv, D), row-major
    float *O;                        // (BH, Sq, D)
    int64_t Sq, Skv;
    int q_tiles;        // ceil(Sq / queries per workgroup)
    int tiles;          // BH * q_tiles
    float scale_log2e;  // scale * log2(e): scores go to base 2
    int causal;         // query i sees keys j <= i + (Skv - Sq)
    int S;              // ring slots
    unsigned *status;
    unsigned long long *stats;
};

// per workgroup: 32 queries per consumer wave
constexpr int kAttnKeys = 64;      // per ring slot
constexpr int kKAhead = 4;         // K fragment reads in flight ahead of the score MFMAs

// The two lanes of a query, l and l ^ 32, exchange values with one
// v_permlane32_swap (no LDS round trip): with both operands x, the pair it
// returns holds x[l] and x[l ^ 32] in every lane l. The softmax is bound by
// VALU issue (two consumer waves share each SIMD's vector unit); this and the
// select-free exponent in the consumer loop gained 5.6% non-causal and 3.8%
// causal (measured on MI355X, batch 4 x 32 heads x 4096^2, bit-identical).
__device__ __forceinline__ float lane_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Expected arrivals on an empty flag: the consumer count rounded up to a
// power of two; the last consumer wave adds the difference.
constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

template <int D, int P, int NCW>
__global__ void __launch_bounds__((P + NCW) * 64) attention_kernel(AttnArgs a) {
    constexpr int BKV = kAttnKeys;
    constexpr int BQ = 32 * NCW;                // queries per workgroup
    constexpr int NE = pow2_at_least(NCW);      // arrivals per empty phase
    constexpr int QPR = D / 8;                  // 16-byte chunks per row
    constexpr int K_BYTES = BKV * D * 2, SLOT = 2 * K_BYTES;
    constexpr int KB = BKV / 32;                // 32-key blocks of S^T
    constexpr int DS = D / 16;                  // 16-deep steps over d
    constexpr int DB = D / 32;                  // 32-row blocks of O^T
    constexpr int KS = BKV / 16;                // 16-key steps of O^T
    static_assert(D == 64 || D == 128, "head dimension");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds + kFlagBytes;
    const int wave = wave_id();
    const int lane = lane_id();
    const LdsFlags fl = init_flags(lds);

    // consecutive logical tiles (one XCD) are the query tiles of one head,
    // so that head's K and V stay in that XCD's L2; with the causal mask the
    // last query tiles see the most keys, so they go first
    const int L = xcd_linear(blockIdx.x, a.tiles);
    const int64_t bh = L / a.q_tiles;
    const int qt = L % a.q_tiles;
    const int64_t q0 = (int64_t)(a.causal ? a.q_tiles - 1 - qt : qt) * BQ;
    const int64_t Sq = a.Sq, Skv = a.Skv;
    int64_t kv_end = Skv;
    if (a.causal) kv_end = max((int64_t)0, min(Skv, min(q0 + BQ, Sq) + (Skv - Sq)));
    const int T = (int)((kv_end + BKV - 1) / BKV);
    const int S = a.S;
    const unsigned char *Kh = a.K + (size_t)bh * (size_t)Skv * D * 2;
    const unsigned char *Vh = a.V + (size_t)bh * (size_t)Skv * D * 2;

    if (wave < P) {
        // ---------------- producer ----------------
        using KD = ADma<BKV, D, 2, P>;
        using VD = BDma<D, BKV, 2, P>;
        constexpr int NL = KD::NL + VD::NL;
        static_assert(NL <= 63, "one tile's loads must fit vmcnt");
        KD kd;
        VD vd;
        kd.init(wave, lane, D, BKV);  // rows past Skv: the buffer range loads zeros
        vd.init(wave, lane, D, 0);
        const int Dinf = max(1, min(S - 1, 63 / NL));
        int s = 0, ps = 0, inflight = 0;
        uint32_t lap = 0;
        WaitTally tally;
        for (int t = 0; t < T; ++t) {
            if (inflight == Dinf) {
                wait_vmcnt_dyn((Dinf - 1) * NL);
                fl.arrive_full(ps);
                if (++ps == S) ps = 0;
                --inflight;
            }
            if (!fl.template wait_empty<NE>(s, (lap & 1u) ^ 1u, a.status, kStatusAttention, tally)) return;
            const int64_t k0 = (int64_t)t * BKV;
            const int rows = (int)min((int64_t)BKV, Skv - k0);
            unsigned char *slot = ring + (size_t)s * SLOT;
            kd.issue(slot, wave, Kh + (size_t)k0 * D * 2, rows, D, 0);
            vd.issue(slot + K_BYTES, wave, Vh, D, Skv, 0, k0);
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
        return;
    }

    // ---------------- consumer ----------------
    const int cw = wave - P;
    const int li = lane & 31, h = lane >> 5, ip = lane & 15;
    const int64_t qrow = q0 + 32 * cw + li;
    const bool qvalid = qrow < Sq;
    const int64_t last_key = qrow + (Skv - Sq);              // causal: the last key this query sees
    const int64_t wave_last_key = q0 + 32 * cw + (Skv - Sq);  // the same for the wave's first query

    // Q^T as the B operand: lane (li, h) holds d = 16 s + 8 h .. + 7 of its query
    bf16x8 qf[DS];
    {
        const unsigned char *qr = a.Q + ((size_t)bh * (size_t)Sq + (size_t)(qvalid ? qrow : 0)) * D * 2;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qr + (16 * s + 8 * h) * 2);
            qf[s] = __builtin_bit_cast(bf16x8, qvalid ? v : u32x4{0u, 0u, 0u, 0u});
        }
    }
    // K rows (A operand of S^T): key 32 b + li of the tile, chunk 2 s + h
    int k_off[KB], k_swz[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const int row = 32 * b + li;
        k_off[b] = row * QPR * 16;
        k_swz[b] = row_swizzle<QPR>(row);
    }
    // V^T (A operand of O^T) through transpose reads of the V tile (B layout):
    // lane i' of a 16-lane group points at 4 consecutive d of key row
    // 16 ks + 4 h + i'/4 (and 8 rows further for the second half) and receives
    // its own d column's 4 keys
    const int v_row = (4 * h + (ip >> 2)) * D * 2;
    const int v_sw = b_swizzle<2, D / 8>(ip >> 2);  // key mod 4 = ip / 4 on every row read
    int v_col[DB];
#pragma unroll
    for (int c = 0; c < DB; ++c) {
        const int n = 32 * c + 16 * ((lane >> 4) & 1) + 4 * (ip & 3);
        v_col[c] = (((n >> 3) ^ v_sw) << 4) + 8 * (ip & 1);
    }

    f32x16 acc_o[DB];
#pragma unroll
    for (int c = 0; c < DB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[c][r] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;
    const float sl2 = a.scale_log2e;

    // Key tiles this wave computes: none when all of its queries lie past Sq
    // (the last query tile of a head), and with the causal mask only those up
    // to its last query's limit. Every key of a later tile is hidden from all
    // of the wave's queries, so its scores would all be -inf and the tile
    // would leave m, l and O^T as they are: the wave only takes part in the
    // ring (waits for the slot and releases it). Its SIMD's other consumer
    // then runs alone (measured on MI355X, batch 4 x 32 heads x 4096^2: +6%
    // causal, non-causal unchanged, bit-identical).
    int T_wave = q0 + 32 * cw >= Sq ? 0 : T;
    if (a.causal) T_wave = (int)min((int64_t)T_wave, max((int64_t)0, (wave_last_key + 31 + BKV) / BKV));

    WaitTally tally;
    int cs = 0;
    uint32_t lap = 0;
    for (int t = 0; t < T; ++t) {
        if (!fl.template wait_full<P>(cs, lap & 1u, a.status, kStatusAttention, tally)) return;
        asm volatile("" ::: "memory");
        if (t < T_wave) {
            const unsigned char *slot = ring + (size_t)cs * SLOT;
            const unsigned char *slotV = slot + K_BYTES;
            const int64_t k0 = (int64_t)t * BKV;

            // S^T = K Q^T for the tile's 64 keys
            f32x16 sc[KB];
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) sc[b][r] = 0.0f;
            // K fragments are read kKAhead MFMAs ahead of their use: left to
            // itself the scheduler keeps two in flight, and each pair of MFMAs
            // waited a whole LDS round trip (measured on MI355X: +2.4% non-causal,
            // +3.2% causal with 4 ahead; 6 or 8 gained no more).
            {
                bf16x8 kf[DS][KB];
#pragma unroll
                for (int s = 0; s < DS; ++s)
#pragma unroll
                    for (int b = 0; b < KB; ++b)
                        kf[s][b] = *reinterpret_cast<const bf16x8 *>(slot + k_off[b] + (((2 * s + h) ^ k_swz[b]) << 4));
#pragma unroll
                for (int s = 0; s < DS; ++s)
#pragma unroll
                    for (int b = 0; b < KB; ++b)
                        sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][b], qf[s], sc[b], 0, 0, 0);
                constexpr int NK = DS * KB, AH = kKAhead < NK ? kKAhead : NK;
                __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // AH LDS reads first
#pragma unroll
                for (int i = 0; i < NK - AH; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // then one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // and one read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);  // the last AH MFMAs
            }
            // online softmax over this tile's keys, in base 2 (scores times
            // scale * log2 e); masked keys are -inf. Only tiles that reach past
            // Skv or past the causal limit of the wave's first query need the
            // mask (a wave-uniform test), so interior tiles skip it.
            const bool edge = k0 + BKV > Skv || (a.causal && k0 + BKV - 1 > wave_last_key);
            if (edge) {
#pragma unroll
                for (int b = 0; b < KB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t key = k0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool vis = key < Skv && (!a.causal || key <= last_key);
                        sc[b][r] = vis ? sc[b][r] : -__builtin_inff();
                    }
            }
            float mt = -__builtin_inff();
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[b][r]);
            mt = lane_max(mt) * sl2;
            const float m_new = fmaxf(m_run, mt);
            const bool none = m_new == -__builtin_inff();  // no visible key so far
            const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            // with no visible key so far every score is -inf, and -inf * sl2 -
            // m_use (sl2 > 0, m_use finite) gives exp2(-inf) = 0 without a
            // select per score
            const float m_use = none ? 0.0f : m_new;
            float rs = 0.0f;
            bf16x8 pf[KS];
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][r], sl2, -m_use));
                    rs += p;
                    pf[2 * b + (r >> 3)][r & 7] = (__bf16)p;
                }
            rs = lane_sum(rs);
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int c = 0; c < DB; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[c][r] *= alpha;

            // O^T += V^T P^T, V^T fragments read one key step at a time
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 vf[DB];
#pragma unroll
                for (int c = 0; c < DB; ++c) {
                    const unsigned char *p = slotV + v_row + 16 * ks * D * 2 + v_col[c];
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 8 * D * 2));
                    vf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int c = 0; c < DB; ++c)
                    acc_o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c], pf[ks], acc_o[c], 0, 0, 0);
            }
        }
        wait_lgkm0();  // every read of the slot has landed
        // Consumers sharing a SIMD drift apart (its matrix unit issues the
        // older wave's MFMAs first): the ones releasing a slot in the later
        // half raise their wave priority for the next tile (measured on
        // MI355X, batch 4 x 32 heads x 4096^2: +3.6% non-causal, +3.5%
        // causal, bit-identical).
        if (fl.template arrive_empty_rank<NE>(cs, cw == NCW - 1 ? NE - NCW + 1 : 1) >= (uint32_t)(NE / 2))
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        if (++cs == S) {
            cs = 0;
            ++lap;
        }
    }
    publish_tally(a.stats ? a.stats + kStatAttnConsumer : nullptr, tally);

    // O[query][d]: lane (li, h) holds its query's d = 32 c + 8 (r / 4) + 4 h + (r % 4)
    if (qvalid) {
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        float *orow = a.O + ((size_t)bh * (size_t)Sq + (size_t)qrow) * D;
#pragma unroll
        for (int c = 0; c < DB; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) orow[32 * c + 8 * (r >> 2) + 4 * h + (r & 3)] = acc_o[c][r] * inv;
    }
}

namespace {

struct AttnVariant {
    int D, P, NCW;
    const void *kernel;
};

#define WSG_ATTN(D, P, NCW) {D, P, NCW, reinterpret_cast<const void *>(&attention_kernel<D, P, NCW>)}

// First match per head dimension is the default. D = 128: 7 consumer waves
// first (measured on MI355X, batch 4 x 32 heads x 4096^2, S = 3, bit-identical
// to 4 consumers: 862 against 810 TFLOP/s non-causal, 749 against 710 causal).
const AttnVariant kAttnVariants[] = {
    WSG_ATTN(128, 1, 7), WSG_ATTN(128, 1, 4), WSG_ATTN(128, 2, 4), WSG_ATTN(128, 4, 4),
    WSG_ATTN(64, 1, 4),  WSG_ATTN(64, 2, 4),
};

}  // namespace

int launch_attention(const LaunchCtx &ctx, int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const void *Q,
                     const void *K, const void *V, float *O, float scale, int causal, int stages, int producers,
                     int consumers, std::string *err) {
    const AttnVariant *pick = nullptr;
    for (const AttnVariant &v : kAttnVariants) {
        if (v.D != D || (producers && v.P != producers) || (consumers && v.NCW != consumers)) continue;
        pick = &v;
        break;
    }
    if (!pick) {
        *err = "no attention kernel built for head dimension " + std::to_string(D) + " with " +
               std::to_string(producers) + " producer and " + std::to_string(consumers) +
               " consumer waves (built: D = 64 or 128; 1, 2 or 4 producers with 4 consumers; for D = 128 also 1 "
               "producer with 7 consumers)";
        return WSG_EUNSUPPORTED;
    }
    if (stages < 1 || stages > kMaxStages) {
        *err = "stages must be in 1.." + std::to_string(kMaxStages);
        return stages < 1 ? WSG_EINVAL : WSG_EUNSUPPORTED;
    }
    const size_t lds = (size_t)kFlagBytes + (size_t)stages * 2 * kAttnKeys * (size_t)D * 2;
    if (lds > ctx.dev.max_lds) {
        *err = "ring needs " + std::to_string(lds) + " bytes of LDS, the device allows " +
               std::to_string(ctx.dev.max_lds) + " per workgroup";
        return WSG_EUNSUPPORTED;
    }
    if (BH == 0 || Sq == 0) return WSG_OK;
    const int64_t BQ = 32 * pick->NCW;
    const int64_t q_tiles = (Sq + BQ - 1) / BQ;
    if (BH * q_tiles > 0x7FFFFFFF) {
        *err = "too many query tiles";
        return WSG_EUNSUPPORTED;
    }
    AttnArgs args;
    args.Q = static_cast<const unsigned char *>(Q);
    args.K = static_cast<const unsigned char *>(K);
    args.V = static_cast<const unsigned char *>(V);
    args.O = O;
    args.Sq = Sq;
    args.Skv = Skv;
    args.q_tiles = (int)q_tiles;
    args.tiles = (int)(BH * q_tiles);
    args.scale_log2e = scale * 1.4426950408889634f;
    args.causal = causal ? 1 : 0;
    args.S = stages;
    args.status = ctx.dev.status;
    args.stats = ctx.wait_stats ? ctx.dev.stats : nullptr;
    const int rc = prepare_kernel(pick->kernel, ctx.dev, err);
    if (rc != WSG_OK) return rc;
    void *kargs[] = {&args};
    hipError_t e = hipLaunchKernel(pick->kernel, dim3((unsigned)args.tiles), dim3((pick->P + pick->NCW) * 64), kargs, lds,
                                   ctx.stream);
    if (e != hipSuccess) {
        *err = std::string("attention launch: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    return WSG_OK;
}

}  // namespace wsg
