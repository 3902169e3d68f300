// staged_copy.hip - HBM -> LDS ring -> HBM copy with producer and consumer
// waves ("Producer-Consumer Warp Specialization for TMA Operations": a
// double-buffered load into shared memory and a store back out, where the
// full flag trips as data flows into a buffer and the empty flag as it flows
// out).
//
// Work split: a persistent grid of G workgroups (one per CU: two 64 KiB slots
// take most of the 160 KiB of LDS); workgroup g copies tiles g, g + G, ...,
// and its j-th tile uses slot j mod S with wait parity (j / S) & 1.
//
// Producer waves issue 16-byte LDS-DMA loads (global -> LDS, no VGPRs) for a
// tile and keep up to S - 1 further tiles in flight before they mark a tile
// full (vmcnt counts loads in issue order). Consumer waves wait full, read
// the slot into VGPRs, release it as soon as those reads completed, then
// store to dst. Data moves as raw bits throughout.
#include "internal.hpp"
#include "ring.hpp"

namespace wsg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NT: stream both directions past the caches (non-temporal loads into LDS
// and non-temporal stores), since each byte is touched exactly once.
template <int P, int C, int TILE, bool NT>
__global__ void __launch_bounds__((P + C) * 64)
    staged_copy_kernel(const unsigned char *__restrict__ src, unsigned char *__restrict__ dst, uint64_t bytes,
                       uint64_t ntiles, int S, unsigned *status, unsigned long long *stats) {
    static_assert(TILE % (P * 1024) == 0 && TILE % (C * 1024) == 0, "tile must split into 1 KiB wave chunks");
    constexpr int NL = TILE / (P * 1024);  // LDS-DMA loads per producer wave per tile
    constexpr int NC = TILE / (C * 1024);  // 16-byte reads per consumer lane per tile
    static_assert(NL <= 63, "a tile's loads must fit the vmcnt counter");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds + kFlagBytes;
    const uint32_t fb = lds_addr(lds);
    const int wave = wave_id();
    const int lane = lane_id();

    if (threadIdx.x < kFlagBytes / 4) reinterpret_cast<uint32_t *>(lds)[threadIdx.x] = 0u;
    __syncthreads();  // the only workgroup barrier: flags start at phase 0

    const uint64_t G = gridDim.x;
    const uint64_t g = blockIdx.x;
    if (g >= ntiles) return;
    const int64_t nloc = (int64_t)((ntiles - g + G - 1) / G);  // tiles of this workgroup

    WaitTally tally;
    if (wave < P) {
        // ---------------- producer ----------------
        // Up to D tiles in flight; the oldest is completed and published
        // before the wait for the next free slot, so a full signal never
        // waits on an empty one.
        const int D = max(1, min(S - 1, 63 / NL));
        auto finish = [&](int64_t j) {
            const int s = (int)(j % S);
            const uint64_t base = (g + (uint64_t)j * G) * (uint64_t)TILE;
            const uint64_t valid = min((uint64_t)TILE, bytes - base);
            const uint64_t v16 = valid & ~(uint64_t)15;
            // The partial 16-byte chunk at v16 lies past the buffer range, so
            // an LDS-DMA load of this tile has already written zeros over it:
            // the one issued by the wave that owns v16's 1 KiB block, (v16 /
            // 1024) mod P. That wave alone writes the tail bytes, after the
            // vmcnt wait that completed its own loads of the tile, so its
            // ds_write lands after those zeros (one wave's LDS writes are
            // ordered). Another wave could not know when the zeros land.
            if ((valid & 15u) && wave == (int)((v16 >> 10) % (uint64_t)P)) {
                // bytes past the last whole 16-byte chunk: byte loads into the slot
                if ((uint64_t)lane < (valid - v16)) {
                    unsigned char b = src[base + v16 + lane];
                    ring[(size_t)s * TILE + v16 + lane] = b;
                }
                wait_vmcnt<0>();
                wait_lgkm0();
            }
            flag_arrive(full_flag(fb, s));
        };
        int s = 0;
        uint32_t lap = 0;
        int inflight = 0;
        for (int64_t j = 0; j < nloc; ++j) {
            if (inflight == D) {
                wait_vmcnt_dyn((D - 1) * NL);
                finish(j - D);
                --inflight;
            }
            if (!flag_wait<C>(empty_flag(fb, s), (lap & 1u) ^ 1u, status, kStatusCopy, tally)) return;
            const uint64_t base = (g + (uint64_t)j * G) * (uint64_t)TILE;
            const uint64_t valid = min((uint64_t)TILE, bytes - base);
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + base, (uint32_t)(valid & ~(uint64_t)15));
            unsigned char *slot = ring + (size_t)s * TILE;
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                const uint32_t off = (uint32_t)(r * P + wave) * 1024u;
                lds_dma16<NT ? kAuxNontemporal : 0>(rs, slot + off, off + 16u * lane);
            }
            ++inflight;
            if (++s == S) {
                s = 0;
                ++lap;
            }
        }
        for (int64_t j = nloc - inflight; j < nloc; ++j) {
            wait_vmcnt_dyn((int)(nloc - 1 - j) * NL);
            finish(j);
        }
        publish_tally(stats ? stats + kStatCopyProducer : nullptr, tally);
    } else {
        // ---------------- consumer ----------------
        const int cw = wave - P;
        int s = 0;
        uint32_t lap = 0;
        for (int64_t j = 0; j < nloc; ++j) {
            if (!flag_wait<P>(full_flag(fb, s), lap & 1u, status, kStatusCopy, tally)) return;
            const unsigned char *slot = ring + (size_t)s * TILE;
            uint4 v[NC];
#pragma unroll
            for (int r = 0; r < NC; ++r)
                v[r] = *reinterpret_cast<const uint4 *>(slot + (size_t)(r * C + cw) * 1024u + 16u * lane);
            wait_lgkm0();
            flag_arrive(empty_flag(fb, s));
            const uint64_t base = (g + (uint64_t)j * G) * (uint64_t)TILE;
            const uint64_t valid = min((uint64_t)TILE, bytes - base);
            unsigned char *out = dst + base;
            if (valid == (uint64_t)TILE) {
#pragma unroll
                for (int r = 0; r < NC; ++r) {
                    unsigned char *o = out + (size_t)(r * C + cw) * 1024u + 16u * lane;
                    if constexpr (NT)
                        __builtin_nontemporal_store(u32x4{v[r].x, v[r].y, v[r].z, v[r].w}, reinterpret_cast<u32x4 *>(o));
                    else
                        *reinterpret_cast<uint4 *>(o) = v[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < NC; ++r) {
                    const uint64_t off = (uint64_t)(r * C + cw) * 1024u + 16u * lane;
                    if (off + 16 <= valid) {
                        *reinterpret_cast<uint4 *>(out + off) = v[r];
                    } else if (off < valid) {
                        const uint32_t words[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
                        const uint32_t n = (uint32_t)(valid - off);
#pragma unroll
                        for (uint32_t i = 0; i < 16; ++i)
                            if (i < n) out[off + i] = (unsigned char)(words[i >> 2] >> (8 * (i & 3)));
                    }
                }
            }
            if (++s == S) {
                s = 0;
                ++lap;
            }
        }
        publish_tally(stats ? stats + kStatCopyConsumer : nullptr, tally);
    }
}

// The copy without staging or roles, the baseline the staged copy is measured
// against: every lane moves 16-byte chunks src -> VGPRs -> dst in a
// grid-stride loop, U chunks in flight per lane (consecutive lanes, consecutive
// chunks), then the bytes past the last whole chunk. No LDS and no flags.
template <int U, bool NT>
__global__ void __launch_bounds__(256) direct_copy_kernel(const unsigned char *__restrict__ src,
                                                          unsigned char *__restrict__ dst, uint64_t bytes) {
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
    u32x4 *d = reinterpret_cast<u32x4 *>(dst);
    const uint64_t chunks = bytes >> 4;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < chunks; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(s + i + u * stride) : s[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (NT) __builtin_nontemporal_store(v[u], d + i + u * stride);
            else d[i + u * stride] = v[u];
        }
    }
    for (; i < chunks; i += stride) d[i] = s[i];
    const uint64_t tail = bytes & 15u;
    if (blockIdx.x == 0 && threadIdx.x < tail) dst[(chunks << 4) + threadIdx.x] = src[(chunks << 4) + threadIdx.x];
}

namespace {

constexpr int kDirectUnroll = 4;  // chunks in flight per lane

struct CopyVariant {
    int P, C, tile;
    bool nt;
    const void *kernel;
};

#define WSG_COPY_VARIANT(P, C, T, NT) {P, C, T, NT, reinterpret_cast<const void *>(&staged_copy_kernel<P, C, T, NT>)}

// First match per (tile, nt) is the default wave split for that tile.
const CopyVariant kCopyVariants[] = {
    WSG_COPY_VARIANT(8, 8, 65536, true),   WSG_COPY_VARIANT(4, 4, 65536, true),  WSG_COPY_VARIANT(2, 2, 32768, true),
    WSG_COPY_VARIANT(2, 2, 16384, true),   WSG_COPY_VARIANT(1, 1, 16384, true),  WSG_COPY_VARIANT(1, 1, 8192, true),
    WSG_COPY_VARIANT(4, 4, 65536, false),  WSG_COPY_VARIANT(2, 2, 65536, false), WSG_COPY_VARIANT(8, 8, 65536, false),
    WSG_COPY_VARIANT(4, 8, 65536, false),  WSG_COPY_VARIANT(4, 4, 32768, false), WSG_COPY_VARIANT(2, 2, 32768, false),
    WSG_COPY_VARIANT(2, 2, 16384, false),  WSG_COPY_VARIANT(1, 1, 16384, false), WSG_COPY_VARIANT(1, 1, 8192, false),
    WSG_COPY_VARIANT(1, 1, 4096, false),   WSG_COPY_VARIANT(1, 1, 4096, true),
};

}  // namespace

int plan_copy(size_t bytes, int stages, const wsg_config *cfg, const DeviceInfo &dev, CopyPlan *plan,
              std::string *err) {
    (void)bytes;
    int tile = (cfg && cfg->copy_tile_bytes) ? cfg->copy_tile_bytes : 0;
    int P = (cfg && cfg->producer_waves) ? cfg->producer_waves : 0;
    int C = (cfg && cfg->consumer_waves) ? cfg->consumer_waves : 0;
    bool nt = cfg && (cfg->flags & WSG_FLAG_NONTEMPORAL);
    const int workgroups = cfg ? cfg->copy_workgroups : 0;
    if (workgroups < 0) {
        *err = "copy_workgroups must be >= 0";
        return WSG_EINVAL;
    }
    if (stages < 1) {
        *err = "stages must be >= 1";
        return WSG_EINVAL;
    }
    if (cfg && (cfg->flags & WSG_FLAG_DIRECT_COPY)) {
        // the unstaged baseline: no ring, no roles (stages is not used)
        plan->direct = true;
        plan->P = plan->C = 0;
        plan->tile = 16;
        plan->stages = stages;
        plan->kernel = nt ? reinterpret_cast<const void *>(&direct_copy_kernel<kDirectUnroll, true>)
                          : reinterpret_cast<const void *>(&direct_copy_kernel<kDirectUnroll, false>);
        plan->lds_bytes = 0;
        plan->workgroups = workgroups;
        return WSG_OK;
    }
    if (!cfg) {
        // defaults: the largest slot that lets `stages` slots share 128 KiB of
        // LDS, streamed past the caches (the fastest measured settings)
        nt = true;
        tile = 65536;
        while (tile > 8192 && (size_t)stages * (size_t)tile > 131072) tile /= 2;
    } else if (!tile) {
        tile = 65536;
    }
    if (stages > kMaxStages) {
        *err = "stages above the flag area's limit of " + std::to_string(kMaxStages);
        return WSG_EUNSUPPORTED;
    }
    const CopyVariant *pick = nullptr;
    for (const CopyVariant &v : kCopyVariants) {
        if (v.tile != tile || v.nt != nt) continue;
        if (P && v.P != P) continue;
        if (C && v.C != C) continue;
        pick = &v;
        break;
    }
    if (!pick) {
        *err = "no staged-copy kernel built for tile " + std::to_string(tile) + " bytes, " + std::to_string(P) +
               " producer and " + std::to_string(C) + " consumer waves";
        return WSG_EUNSUPPORTED;
    }
    size_t lds = (size_t)kFlagBytes + (size_t)stages * (size_t)tile;
    if (lds > dev.max_lds) {
        *err = "ring needs " + std::to_string(lds) + " bytes of LDS, the device allows " +
               std::to_string(dev.max_lds) + " per workgroup";
        return WSG_EUNSUPPORTED;
    }
    plan->P = pick->P;
    plan->C = pick->C;
    plan->tile = pick->tile;
    plan->stages = stages;
    plan->kernel = pick->kernel;
    plan->lds_bytes = lds;
    plan->workgroups = workgroups;
    return WSG_OK;
}

int launch_copy(const LaunchCtx &ctx, const CopyPlan &plan, const void *src, void *dst, size_t bytes,
                std::string *err) {
    if (bytes == 0) return WSG_OK;
    if (plan.direct) {
        // one 4-wave workgroup per CU by default (measured on MI355X: the
        // fastest plain-copy launch shape, 256 workgroups x 4 waves with 4
        // loads in flight per lane)
        const uint64_t lanes_needed = (bytes / 16 + 255) / 256;
        uint64_t grid = plan.workgroups > 0 ? (uint64_t)plan.workgroups : (uint64_t)ctx.dev.cu_count;
        if (grid > lanes_needed) grid = lanes_needed;
        if (grid < 1) grid = 1;
        const unsigned char *s = static_cast<const unsigned char *>(src);
        unsigned char *d = static_cast<unsigned char *>(dst);
        uint64_t nb = bytes;
        void *args[] = {&s, &d, &nb};
        hipError_t e = hipLaunchKernel(plan.kernel, dim3((unsigned)grid), dim3(256), args, 0, ctx.stream);
        if (e != hipSuccess) {
            *err = std::string("direct copy launch: ") + hipGetErrorString(e);
            return WSG_ELAUNCH;
        }
        return WSG_OK;
    }
    const uint64_t ntiles = (bytes + (uint64_t)plan.tile - 1) / (uint64_t)plan.tile;
    const int threads = (plan.P + plan.C) * 64;
    const int rc = prepare_kernel(plan.kernel, ctx.dev, err);
    if (rc != WSG_OK) return rc;
    const int per_cu = blocks_per_cu(plan.kernel, ctx.dev, threads, plan.lds_bytes);
    // Persistent grid: by default 3/4 of the resident workgroups for 64 KiB
    // slots, 15/16 for smaller ones (a 1 GiB copy measured on MI355X, 64 KiB
    // slots: 6.0 TB/s at 192 of 256 workgroups, 5.5 TB/s at 256; 16 KiB slots
    // in an 8-deep ring: best at 240).
    const uint64_t resident = (uint64_t)ctx.dev.cu_count * (uint64_t)per_cu;
    uint64_t grid = plan.workgroups > 0 ? (uint64_t)plan.workgroups
                                        : (plan.tile >= 65536 ? resident * 3 / 4 : resident * 15 / 16);
    if (grid < 1) grid = 1;
    if (grid > ntiles) grid = ntiles;
    const unsigned char *s = static_cast<const unsigned char *>(src);
    unsigned char *d = static_cast<unsigned char *>(dst);
    uint64_t nb = bytes;
    int S = plan.stages;
    unsigned *status = ctx.dev.status;
    unsigned long long *stats = ctx.wait_stats ? ctx.dev.stats : nullptr;
    void *args[] = {&s, &d, &nb, (void *)&ntiles, &S, &status, &stats};
    hipError_t e = hipLaunchKernel(plan.kernel, dim3((unsigned)grid), dim3(threads), args, plan.lds_bytes, ctx.stream);
    if (e != hipSuccess) {
        *err = std::string("staged_copy launch: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    return WSG_OK;
}

}  // namespace wsg
