// internal.hpp - host-side declarations shared by the library's translation
// units (not part of the public ABI; see include/wsg.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/wsg.h"

namespace wsg {

struct DeviceInfo {
    int device = -1;
    int cu_count = 0;
    size_t max_lds = 0;  // bytes of LDS one workgroup may allocate
    unsigned *status = nullptr;  // device address of the status word
    unsigned long long *stats = nullptr;  // device address of the wait statistics
    void *scratch = nullptr;  // device address of this device's allocation-free scratch array
};

struct LaunchCtx {
    hipStream_t stream = nullptr;
    DeviceInfo dev;
    bool wait_stats = false;  // pass dev.stats to the kernels
};

// One compiled GEMM variant.
struct GemmVariant {
    int dtype;    // WSG_FP32 / WSG_BF16
    int BM, BN, BK;
    int P;        // producer waves
    int CWM, CWN; // consumer wave grid
    bool dma;     // LDS-DMA producer (aligned shapes) or register-staged producer (any shape)
    int GK;       // consumer k per fragment group
    const void *kernel;          // ordinary launch
    const void *grouped_kernel;  // the same kernel for a grouped (mixture-of-experts) launch
    const void *sk_kernel;       // the same kernel as a stream-K persistent grid, or null if not built
};

struct GemmPlan {
    const GemmVariant *v = nullptr;
    int stages = 0;
    int64_t tiles_m = 0, tiles_n = 0;
    size_t lds_bytes = 0;
};

struct CopyPlan {
    int P = 0, C = 0, tile = 0, stages = 0;
    int workgroups = 0;  // persistent grid size requested (0: the default policy)
    bool direct = false;  // the unstaged baseline (WSG_FLAG_DIRECT_COPY)
    const void *kernel = nullptr;
    size_t lds_bytes = 0;
};

// The text wsg_check_device_status reports for a status word.
std::string timeout_message(unsigned word);

// Once per (device, kernel): raise the kernel's dynamic-LDS limit to the
// device maximum, so that launches need no attribute call of their own.
int prepare_kernel(const void *kernel, const DeviceInfo &dev, std::string *err);

// Workgroups of `threads` threads and `lds` bytes of LDS one CU holds (at
// least 1), cached per (device, kernel, threads, lds).
int blocks_per_cu(const void *kernel, const DeviceInfo &dev, int threads, size_t lds);

// Fill `plan` for the arguments; returns WSG_OK or an error code with `err` set.
int plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B, int stages,
              const wsg_config *cfg, const DeviceInfo &dev, GemmPlan *plan, std::string *err);
// Stream-K tail of an ordinary launch (fp32 specialized LDS-DMA kernels): a
// persistent grid of `workers` workgroups computes dp_tiles whole tiles (whole
// rounds) and splits the sk_tiles left over evenly along K. Its workspace:
// part_bytes of partial tiles (one per worker), then cnt_bytes of counters.
struct SkShape {
    bool use = false;
    int workers = 0;
    int64_t dp_tiles = 0, sk_tiles = 0;
    size_t part_bytes = 0, cnt_bytes = 0;
    size_t bytes() const { return part_bytes + cnt_bytes; }
};
// Decide whether the launch `plan` runs with a stream-K tail and size it.
// flags: WSG_FLAG_STREAM_K forces it, WSG_FLAG_NO_STREAM_K forbids it; by
// default it is used when the last round of tiles would be at most 90% full.
SkShape plan_stream_k(const GemmPlan &plan, int64_t M, int64_t N, int64_t K, int flags, const DeviceInfo &dev);
// `sk` null or unused: one workgroup per tile. Otherwise `ws` is a device
// workspace of at least sk->bytes() bytes, 256-byte aligned.
int launch_gemm(const LaunchCtx &ctx, const GemmPlan &plan, int64_t M, int64_t N, int64_t K, const void *A,
                const void *B, const void *bias, float *C, const SkShape *sk, void *ws, std::string *err);
// One launch over the tiles of `groups` experts (rows sorted by expert,
// group_rows[e] rows each; B and bias hold one block per expert); `plan` was
// made for the total row count.
int launch_grouped_gemm(const LaunchCtx &ctx, const GemmPlan &plan, int groups, const int64_t *group_rows, int64_t N,
                        int64_t K, const void *A, const void *B, const void *bias, float *C, std::string *err);

// Scaled dot-product attention forward over BH = batch * heads independent
// heads (Q: BH x Sq x D, K and V: BH x Skv x D, bf16 bits; O fp32).
// producers = 0 / consumers = 0 pick the default wave counts.
int launch_attention(const LaunchCtx &ctx, int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const void *Q,
                     const void *K, const void *V, float *O, float scale, int causal, int stages, int producers,
                     int consumers, std::string *err);

int plan_copy(size_t bytes, int stages, const wsg_config *cfg, const DeviceInfo &dev, CopyPlan *plan,
              std::string *err);
int launch_copy(const LaunchCtx &ctx, const CopyPlan &plan, const void *src, void *dst, size_t bytes,
                std::string *err);

}  // namespace wsg
