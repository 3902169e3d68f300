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
// Producers (two builds):
//   DMA      16-byte LDS-DMA loads through buffer resources (the analogue of
//            an asynchronous bulk copy: no VGPRs, completion by vmcnt). Chunks
//            past M, N or K get an out-of-range offset, which loads zeros, so
//            consumers never mask. Up to S - 1 tiles stay in flight. Needs
//            16-byte aligned rows (K, N multiples of 4 for fp32).
//   general  per-element masked loads into VGPRs, then 16-byte LDS writes in
//            the same slot layout; any shape and 4-byte alignment.
//
// Slot layout (fp32): A as BM rows of BK floats, 16-byte chunks XOR-swizzled
// within a row so that 8 consecutive rows read the same chunk index from
// distinct banks; B as BK rows of BN floats.
//
// Consumers run v_mfma_f32_32x32x2_f32. Over one 16-deep k group a lane of
// half h (lanes 32h..32h+31) supplies k = 16g + 8h + j at step j = 0..7, so
// its eight A values are two consecutive 16-byte chunks of one row; B values
// are single floats of one column. The slot is released as soon as the
// fragments are in registers, before the MFMAs run.
#include "internal.hpp"
#include "ring.hpp"

namespace wsg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
    const unsigned char *A;
    const unsigned char *B;
    const unsigned char *bias;
    float *C;
    int64_t M, N, K;
    int S;
    int tiles_m, tiles_n;
    unsigned *status;
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Give each XCD a contiguous run of logical tiles, then walk those in
// groups of kGroupRows tile rows so the tiles resident on one XCD share rows
// of A and columns of B.
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int G = tiles_m * tiles_n;
    const int x = bid % kXcds, i = bid / kXcds;
    const int q = G / kXcds, r = G % kXcds;
    const int L = x * q + min(x, r) + i;
    const int per_group = kGroupRows * tiles_n;
    const int grp = L / per_group;
    const int first_m = grp * kGroupRows;
    const int gm = min(tiles_m - first_m, kGroupRows);
    const int rem = L - grp * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
}

__device__ __forceinline__ float relu_f32(float v) { return (v > 0.0f || v != v) ? v : 0.0f; }

template <int QPR>
__device__ __forceinline__ int a_swizzle(int m) {
    // chunk index XOR so that 8 consecutive rows hit 8 distinct 16-byte bank groups
    if constexpr (QPR == 4) return (m >> 1) & 3;
    else return m & 7;
}

template <int BM, int BN, int BK, int P, int CWM, int CWN, bool DMA>
__global__ void __launch_bounds__((P + CWM * CWN) * 64) gemm_f32_kernel(GemmArgs a) {
    constexpr int NCW = CWM * CWN;
    constexpr int WTM = BM / CWM, WTN = BN / CWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int QPR = BK / 4;
    constexpr int A_BYTES = BM * BK * 4, B_BYTES = BK * BN * 4, SLOT = A_BYTES + B_BYTES;
    constexpr int A_CHUNKS = BM * QPR, B_CHUNKS = BK * BN / 4;
    constexpr int NLA = A_CHUNKS / (64 * P), NLB = B_CHUNKS / (64 * P);
    constexpr int NL = NLA + NLB;
    constexpr int KG = BK / 16;
    static_assert(BK % 16 == 0 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
    static_assert(A_CHUNKS % (64 * P) == 0 && B_CHUNKS % (64 * P) == 0, "chunks split evenly over producer waves");
    static_assert(NL <= 63, "one tile's loads must fit vmcnt");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds + kFlagBytes;
    const uint32_t fb = lds_addr(lds);
    const int wave = wave_id();
    const int lane = lane_id();

    if (threadIdx.x < kFlagBytes / 4) reinterpret_cast<uint32_t *>(lds)[threadIdx.x] = 0u;
    __syncthreads();  // the only workgroup barrier

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int T = (int)((K + BK - 1) / BK);
    const int S = a.S;

    if (wave < P) {
        // ================= producer =================
        const int rows_valid = (int)min((int64_t)BM, M - m0);
        if constexpr (DMA) {
            uint32_t a_off[NLA];
            int a_q[NLA];
            bool a_ok[NLA];
#pragma unroll
            for (int r = 0; r < NLA; ++r) {
                const int p = (r * P + wave) * 64 + lane;
                const int m = p / QPR;
                const int q = (p % QPR) ^ a_swizzle<QPR>(m);
                a_off[r] = (uint32_t)m * (uint32_t)K * 4u + (uint32_t)q * 16u;
                a_q[r] = q;
                a_ok[r] = m < rows_valid;
            }
            uint32_t b_off[NLB];
            int b_k[NLB];
            bool b_ok[NLB];
#pragma unroll
            for (int r = 0; r < NLB; ++r) {
                const int p = (r * P + wave) * 64 + lane;
                const int k = p / (BN / 4);
                const int c = p % (BN / 4);
                b_off[r] = (uint32_t)k * (uint32_t)N * 4u + (uint32_t)c * 16u;
                b_k[r] = k;
                b_ok[r] = n0 + 4 * c < N;
            }
            const unsigned char *Abase = a.A + (size_t)m0 * (size_t)K * 4u;
            const int D = min(S - 1, 63 / NL);
            int s = 0;
            uint32_t lap = 0;
            for (int t = 0; t < T; ++t) {
                if (!flag_wait(empty_flag(fb, s), (lap & 1u) ^ 1u, a.status, kStatusGemm)) return;
                const int64_t k0 = (int64_t)t * BK;
                unsigned char *slot = ring + (size_t)s * SLOT;
                const int64_t a_rec = ((int64_t)rows_valid * K - k0) * 4;
                const __amdgpu_buffer_rsrc_t ra =
                    make_rsrc(Abase + (size_t)k0 * 4u, (uint32_t)min(a_rec, (int64_t)0x7FFFFFFF));
#pragma unroll
                for (int r = 0; r < NLA; ++r) {
                    const bool ok = a_ok[r] && (k0 + 4 * a_q[r] < K);
                    lds_dma16(ra, slot + (r * P + wave) * 1024, ok ? a_off[r] : kOobOffset);
                }
                const int64_t b_rec = (K * N - k0 * N - n0) * 4;
                const __amdgpu_buffer_rsrc_t rb =
                    make_rsrc(a.B + (size_t)(k0 * N + n0) * 4u, (uint32_t)min(b_rec, (int64_t)0x7FFFFFFF));
#pragma unroll
                for (int r = 0; r < NLB; ++r) {
                    const bool ok = b_ok[r] && (k0 + b_k[r] < K);
                    lds_dma16(rb, slot + A_BYTES + (r * P + wave) * 1024, ok ? b_off[r] : kOobOffset);
                }
                if (t >= D) {
                    wait_vmcnt_dyn(D * NL);
                    flag_arrive(full_flag(fb, (t - D) % S), P);
                }
                if (++s == S) {
                    s = 0;
                    ++lap;
                }
            }
            for (int t = max(0, T - D); t < T; ++t) {
                wait_vmcnt_dyn((T - 1 - t) * NL);
                flag_arrive(full_flag(fb, t % S), P);
            }
        } else {
            const float *A = reinterpret_cast<const float *>(a.A);
            const float *B = reinterpret_cast<const float *>(a.B);
            int s = 0;
            uint32_t lap = 0;
            for (int t = 0; t < T; ++t) {
                if (!flag_wait(empty_flag(fb, s), (lap & 1u) ^ 1u, a.status, kStatusGemm)) return;
                const int64_t k0 = (int64_t)t * BK;
                unsigned char *slot = ring + (size_t)s * SLOT;
#pragma unroll
                for (int r = 0; r < NLA; ++r) {
                    const int p = (r * P + wave) * 64 + lane;
                    const int m = p / QPR;
                    const int q = (p % QPR) ^ a_swizzle<QPR>(m);
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t k = k0 + 4 * q + e;
                        v[e] = (m < rows_valid && k < K) ? A[(m0 + m) * K + k] : 0.0f;
                    }
                    *reinterpret_cast<f32x4 *>(slot + (size_t)p * 16u) = v;
                }
#pragma unroll
                for (int r = 0; r < NLB; ++r) {
                    const int p = (r * P + wave) * 64 + lane;
                    const int k = p / (BN / 4);
                    const int c = p % (BN / 4);
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t n = n0 + 4 * c + e;
                        v[e] = (k0 + k < K && n < N) ? B[(k0 + k) * N + n] : 0.0f;
                    }
                    *reinterpret_cast<f32x4 *>(slot + A_BYTES + (size_t)p * 16u) = v;
                }
                wait_lgkm0();
                flag_arrive(full_flag(fb, s), P);
                if (++s == S) {
                    s = 0;
                    ++lap;
                }
            }
        }
        return;
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

    int a_row_off[FM], a_swz[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wr * WTM + 32 * i + li;
        a_row_off[i] = row * QPR * 16;
        a_swz[i] = a_swizzle<QPR>(row);
    }
    int b_col[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_col[j] = wc * WTN + 32 * j + li;

    int s = 0;
    uint32_t lap = 0;
    for (int t = 0; t < T; ++t) {
        if (!flag_wait(full_flag(fb, s), lap & 1u, a.status, kStatusGemm)) return;
        const unsigned char *slotA = ring + (size_t)s * SLOT;
        const float *slotB = reinterpret_cast<const float *>(slotA + A_BYTES);
        f32x4 af[KG][FM][2];
        float bf[KG][FN][8];
#pragma unroll
        for (int g = 0; g < KG; ++g) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int q0 = 4 * g + 2 * h;
                af[g][i][0] = *reinterpret_cast<const f32x4 *>(slotA + a_row_off[i] + ((q0 ^ a_swz[i]) << 4));
                af[g][i][1] = *reinterpret_cast<const f32x4 *>(slotA + a_row_off[i] + (((q0 + 1) ^ a_swz[i]) << 4));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) bf[g][j][kk] = slotB[(16 * g + 8 * h + kk) * BN + b_col[j]];
        }
        wait_lgkm0();
        flag_arrive(empty_flag(fb, s), NCW);
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[g][i][kk >> 2][kk & 3], bf[g][j][kk],
                                                                          acc[i][j], 0, 0, 0);
        if (++s == S) {
            s = 0;
            ++lap;
        }
    }

    // epilogue: C = relu(acc + bias[n]); lane (li, h) holds column li of each
    // 32x32 block and rows 8*(r/4) + 4*h + (r%4) of its 16 registers
    const float *bias = reinterpret_cast<const float *>(a.bias);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + b_col[j];
        const float bv = col < N ? bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wr * WTM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M && col < N) a.C[row * N + col] = relu_f32(acc[i][j][r] + bv);
            }
        }
    }
}

namespace {

#define WSG_F32(BM, BN, BK, P, CWM, CWN, DMA)                                                              \
    {WSG_FP32, BM, BN, BK, P, CWM, CWN, DMA,                                                               \
     reinterpret_cast<const void *>(&gemm_f32_kernel<BM, BN, BK, P, CWM, CWN, DMA>)}

const GemmVariant kGemmVariants[] = {
    WSG_F32(128, 128, 16, 1, 2, 2, true),  WSG_F32(128, 128, 16, 2, 2, 2, true),
    WSG_F32(256, 128, 16, 2, 4, 2, true),  WSG_F32(128, 256, 16, 2, 2, 4, true),
    WSG_F32(128, 128, 32, 2, 2, 2, true),  WSG_F32(64, 64, 16, 1, 2, 2, true),
    WSG_F32(128, 128, 16, 1, 2, 2, false), WSG_F32(64, 64, 16, 1, 2, 2, false),
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
    if (dtype != WSG_FP32) {
        *err = "dtype not built";
        return WSG_EUNSUPPORTED;
    }
    const int esz = 4;
    int BM = cfg && cfg->BM ? cfg->BM : 0, BN = cfg && cfg->BN ? cfg->BN : 0, BK = cfg && cfg->BK ? cfg->BK : 0;
    int P = cfg && cfg->producer_waves ? cfg->producer_waves : 0;
    int CW = cfg && cfg->consumer_waves ? cfg->consumer_waves : 0;
    bool force_general = cfg && (cfg->flags & WSG_FLAG_GENERAL_PRODUCER);
    if (!BM && !BN && !BK) {
        // default tile by problem size: small problems need more workgroups
        if ((M + 127) / 128 * ((N + 127) / 128) >= (int64_t)dev.cu_count) {
            BM = 128;
            BN = 128;
        } else {
            BM = 64;
            BN = 64;
        }
        BK = 16;
    }
    // the DMA producer needs 16-byte aligned rows and offsets within 31 bits
    const bool aligned = (K * esz) % 16 == 0 && (N * esz) % 16 == 0 && ((uintptr_t)A % 16) == 0 &&
                         ((uintptr_t)B % 16) == 0;
    const GemmVariant *pick = nullptr;
    for (int pass = 0; pass < 2 && !pick; ++pass) {
        const bool want_dma = pass == 0;
        if (want_dma && (force_general || !aligned)) continue;
        if (want_dma && ((int64_t)(BM ? BM : 256) * K * esz >= 0x7FFFFFFF ||
                         (int64_t)(BK ? BK : 64) * N * esz >= 0x7FFFFFFF))
            continue;
        for (const GemmVariant &v : kGemmVariants) {
            if (v.dtype != dtype || v.dma != want_dma) continue;
            if ((BM && v.BM != BM) || (BN && v.BN != BN) || (BK && v.BK != BK)) continue;
            if ((P && v.P != P) || (CW && v.CWM * v.CWN != CW)) continue;
            pick = &v;
            break;
        }
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

int launch_gemm(const LaunchCtx &ctx, const GemmPlan &plan, int64_t M, int64_t N, int64_t K, const void *A,
                const void *B, const void *bias, float *C, std::string *err) {
    if (M == 0 || N == 0) return WSG_OK;
    GemmArgs args;
    args.A = static_cast<const unsigned char *>(A);
    args.B = static_cast<const unsigned char *>(B);
    args.bias = static_cast<const unsigned char *>(bias);
    args.C = C;
    args.M = M;
    args.N = N;
    args.K = K;
    args.S = plan.stages;
    args.tiles_m = (int)plan.tiles_m;
    args.tiles_n = (int)plan.tiles_n;
    args.status = ctx.dev.status;
    const int threads = (plan.v->P + plan.v->CWM * plan.v->CWN) * 64;
    hipError_t e =
        hipFuncSetAttribute(plan.v->kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds_bytes);
    if (e != hipSuccess) {
        *err = std::string("hipFuncSetAttribute: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    void *kargs[] = {&args};
    e = hipLaunchKernel(plan.v->kernel, dim3((unsigned)(plan.tiles_m * plan.tiles_n)), dim3(threads), kargs,
                        plan.lds_bytes, ctx.stream);
    if (e != hipSuccess) {
        *err = std::string("gemm launch: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    return WSG_OK;
}

}  // namespace wsg
