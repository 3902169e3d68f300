// abi.hip - the extern "C" entry points declared in include/wsg.h: argument
// validation, per-device state, the calling thread's stream and last error.
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.hpp"
#include "ring.hpp"

// Device status word; each GPU holds its own copy. Kernels get its device
// address (looked up per device with hipGetSymbolAddress) as an argument.
__device__ unsigned wsg_status_word;

// Wait statistics (see wsg_read_wait_stats); each GPU holds its own copy.
__device__ unsigned long long wsg_wait_stats[wsg::kStatWords];

// Stream-K workspace of gemm_bias_relu_ex_noalloc; each GPU holds its own
// copy until the process ends. Host code never names it in a launch or copy:
// it uses the device address looked up per device in device_info.
static __device__ __align__(256) unsigned char scratch[WSG_NOALLOC_SCRATCH_BYTES];

static_assert(wsg::kStatusTimeout == WSG_STATUS_TIMEOUT && wsg::kStatusCopy == WSG_STATUS_COPY &&
                  wsg::kStatusGemm == WSG_STATUS_GEMM && wsg::kStatusAttention == WSG_STATUS_ATTENTION,
              "status bits of the kernels and of the public header");

namespace {

thread_local hipStream_t tl_stream = nullptr;
thread_local std::string tl_err;
thread_local bool tl_wait_stats = false;

std::mutex g_mu;
std::vector<wsg::DeviceInfo> g_devs;

int fail(int code, const std::string &msg) {
    tl_err = msg;
    return code;
}

int ok() {
    tl_err.clear();
    return WSG_OK;
}

int device_info(wsg::DeviceInfo *out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_mu);
    if ((int)g_devs.size() <= dev) g_devs.resize(dev + 1);
    wsg::DeviceInfo &d = g_devs[dev];
    if (d.device < 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
        if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
            return fail(WSG_EUNSUPPORTED, std::string("libwsg is built for gfx950 only; device is ") + prop.gcnArchName);
        int lds = 0;
        e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(wsg_status_word));
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        void *st = nullptr;
        e = hipGetSymbolAddress(&st, HIP_SYMBOL(wsg_wait_stats));
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        void *sc = nullptr;
        e = hipGetSymbolAddress(&sc, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        d.cu_count = prop.multiProcessorCount;
        d.max_lds = (size_t)lds;
        d.status = static_cast<unsigned *>(p);
        d.stats = static_cast<unsigned long long *>(st);
        d.scratch = sc;
        d.device = dev;
    }
    *out = d;
    return WSG_OK;
}

// Stream-K workspaces, allocated on first need and grown as needed, one per
// (device, stream): launches on one stream run in order, so they may share
// it; launches on different streams may overlap, so they may not.
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, std::pair<void *, size_t>> g_ws;

int sk_workspace(int dev, hipStream_t stream, size_t bytes, void **out) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto &w = g_ws[{dev, stream}];
    if (w.second < bytes) {
        if (w.first) {
            // the previous workspace may still be in use by queued launches
            hipError_t e = hipStreamSynchronize(stream);
            if (e == hipSuccess) e = hipFree(w.first);
            if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("stream-K workspace release: ") + hipGetErrorString(e));
            w = {nullptr, 0};
        }
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, bytes);
        if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("stream-K workspace: hipMalloc: ") + hipGetErrorString(e));
        w = {p, bytes};
    }
    *out = w.first;
    return WSG_OK;
}

std::mutex g_kernel_mu;
std::map<std::pair<int, const void *>, bool> g_prepared;
std::map<std::tuple<int, const void *, int, size_t>, int> g_occupancy;

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!an || !bn) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

constexpr int64_t kMaxDim = 0x7FFFFFFF;
constexpr uint64_t kMaxElems = 1ull << 56;  // per operand: keeps every byte count well inside size_t

// `blocks` B and bias blocks (the experts of a grouped launch; 1 otherwise)
int validate_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias,
                  const float *C, int stages, int64_t blocks = 1) {
    if (dtype != WSG_FP32 && dtype != WSG_BF16) return fail(WSG_EINVAL, "dtype must be WSG_FP32 or WSG_BF16");
    if (M < 0 || N < 0 || K < 0) return fail(WSG_EINVAL, "negative dimension");
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(WSG_EUNSUPPORTED, "dimension above 2^31 - 1");
    if (stages < 1) return fail(WSG_EINVAL, "stages must be >= 1");
    if (M == 0 || N == 0) return WSG_OK;
    if ((uint64_t)M * (uint64_t)K > kMaxElems || (uint64_t)K * (uint64_t)N > kMaxElems / (uint64_t)blocks ||
        (uint64_t)M * (uint64_t)N > kMaxElems)
        return fail(WSG_EUNSUPPORTED, "operand larger than 2^56 elements");
    const size_t esz = dtype == WSG_FP32 ? 4 : 2;
    if (K > 0 && (!A || !B)) return fail(WSG_EINVAL, "null A or B with a nonzero size");
    if (!bias || !C) return fail(WSG_EINVAL, "null bias or C with a nonzero size");
    if (((uintptr_t)A % esz) || ((uintptr_t)B % esz) || ((uintptr_t)bias % esz))
        return fail(WSG_EINVAL, "A, B and bias must be aligned to their element size");
    if ((uintptr_t)C % 4) return fail(WSG_EINVAL, "C must be 4-byte aligned");
    const size_t cbytes = (size_t)M * (size_t)N * 4;
    if (overlaps(C, cbytes, A, (size_t)M * (size_t)K * esz) ||
        overlaps(C, cbytes, B, (size_t)blocks * (size_t)K * (size_t)N * esz) ||
        overlaps(C, cbytes, bias, (size_t)blocks * (size_t)N * esz))
        return fail(WSG_EINVAL, "C overlaps an input");
    return WSG_OK;
}

// noalloc: the stream-K workspace is the device's scratch array, never a
// library allocation; a launch that needs more is rejected
int gemm_impl(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias, float *C,
              int stages, const wsg_config *cfg, bool noalloc = false) {
    int rc = validate_gemm(dtype, M, N, K, A, B, bias, C, stages);
    if (rc != WSG_OK) return rc;
    if (M == 0 || N == 0) return ok();
    wsg::LaunchCtx ctx;
    rc = device_info(&ctx.dev);
    if (rc != WSG_OK) return rc;
    ctx.stream = tl_stream;
    ctx.wait_stats = tl_wait_stats;
    wsg::GemmPlan plan;
    std::string err;
    rc = wsg::plan_gemm(dtype, M, N, K, A, B, stages, cfg, ctx.dev, &plan, &err);
    if (rc != WSG_OK) return fail(rc, err);
    const wsg::SkShape sk = wsg::plan_stream_k(plan, M, N, K, cfg ? cfg->flags : 0, ctx.dev);
    void *ws = nullptr;
    if (sk.use && noalloc) {
        if (sk.bytes() > (size_t)WSG_NOALLOC_SCRATCH_BYTES)
            return fail(WSG_EUNSUPPORTED, "stream-K workspace of " + std::to_string(sk.bytes()) +
                                              " bytes exceeds the " + std::to_string(WSG_NOALLOC_SCRATCH_BYTES) +
                                              "-byte scratch of gemm_bias_relu_ex_noalloc (WSG_FLAG_NO_STREAM_K "
                                              "avoids the workspace)");
        ws = ctx.dev.scratch;
    } else if (sk.use) {
        rc = sk_workspace(ctx.dev.device, ctx.stream, sk.bytes(), &ws);
        if (rc != WSG_OK) return rc;
    }
    rc = wsg::launch_gemm(ctx, plan, M, N, K, A, B, bias, C, &sk, ws, &err);
    if (rc != WSG_OK) return fail(rc, err);
    return ok();
}

int grouped_impl(int dtype, int groups, const int64_t *group_rows, int64_t N, int64_t K, const void *A, const void *B,
                 const void *bias, float *C, int stages, const wsg_config *cfg) {
    if (groups < 1) return fail(WSG_EINVAL, "groups must be >= 1");
    if (groups > WSG_MAX_GROUPS) return fail(WSG_EUNSUPPORTED, "more than WSG_MAX_GROUPS experts");
    if (!group_rows) return fail(WSG_EINVAL, "null group_rows");
    int64_t rows = 0;
    for (int e = 0; e < groups; ++e) {
        if (group_rows[e] < 0) return fail(WSG_EINVAL, "negative row count for an expert");
        if (group_rows[e] > kMaxDim - rows) return fail(WSG_EUNSUPPORTED, "total rows above 2^31 - 1");
        rows += group_rows[e];
    }
    int rc = validate_gemm(dtype, rows, N, K, A, B, bias, C, stages, groups);
    if (rc != WSG_OK) return rc;
    if (rows == 0 || N == 0) return ok();
    wsg::LaunchCtx ctx;
    rc = device_info(&ctx.dev);
    if (rc != WSG_OK) return rc;
    ctx.stream = tl_stream;
    ctx.wait_stats = tl_wait_stats;
    wsg::GemmPlan plan;
    std::string err;
    rc = wsg::plan_gemm(dtype, rows, N, K, A, B, stages, cfg, ctx.dev, &plan, &err);
    if (rc != WSG_OK) return fail(rc, err);
    rc = wsg::launch_grouped_gemm(ctx, plan, groups, group_rows, N, K, A, B, bias, C, &err);
    if (rc != WSG_OK) return fail(rc, err);
    return ok();
}

int attention_impl(int64_t batch, int64_t heads, int64_t Sq, int64_t Skv, int64_t D, const uint16_t *Q,
                   const uint16_t *K, const uint16_t *V, float *O, float scale, int causal, int stages,
                   const wsg_config *cfg) {
    if (batch < 0 || heads < 0 || Sq < 0 || Skv < 0 || D < 0) return fail(WSG_EINVAL, "negative dimension");
    if (stages < 1) return fail(WSG_EINVAL, "stages must be >= 1");
    // the kernel takes each row's maximum before scaling and marks hidden
    // keys with -inf, so the scale must be positive; at least 2^-126 so that
    // scale * log2(e) is a normal float, never flushed to zero
    if (!(scale >= 0x1p-126f) || scale == __builtin_inff())
        return fail(WSG_EINVAL, "scale must be finite and at least 2^-126");
    if (D != 64 && D != 128) return fail(WSG_EUNSUPPORTED, "head dimension must be 64 or 128");
    if (batch > kMaxDim || heads > kMaxDim || Sq > kMaxDim || Skv > kMaxDim)
        return fail(WSG_EUNSUPPORTED, "dimension above 2^31 - 1");
    const uint64_t BH = (uint64_t)batch * (uint64_t)heads;
    if (BH > (uint64_t)kMaxDim) return fail(WSG_EUNSUPPORTED, "batch * heads above 2^31 - 1");
    if (BH == 0 || Sq == 0) return ok();
    if (BH * (uint64_t)Sq > kMaxElems / (uint64_t)D || BH * (uint64_t)Skv > kMaxElems / (uint64_t)D)
        return fail(WSG_EUNSUPPORTED, "operand larger than 2^56 elements");
    if (!Q || !O || (Skv > 0 && (!K || !V))) return fail(WSG_EINVAL, "null operand with a nonzero size");
    if (((uintptr_t)Q % 16) || ((uintptr_t)K % 16) || ((uintptr_t)V % 16))
        return fail(WSG_EINVAL, "Q, K and V must be 16-byte aligned");
    if ((uintptr_t)O % 4) return fail(WSG_EINVAL, "O must be 4-byte aligned");
    const size_t obytes = (size_t)(BH * (uint64_t)Sq * (uint64_t)D) * 4;
    const size_t qbytes = (size_t)(BH * (uint64_t)Sq * (uint64_t)D) * 2;
    const size_t kvbytes = (size_t)(BH * (uint64_t)Skv * (uint64_t)D) * 2;
    if (overlaps(O, obytes, Q, qbytes) || overlaps(O, obytes, K, kvbytes) || overlaps(O, obytes, V, kvbytes))
        return fail(WSG_EINVAL, "O overlaps an input");
    wsg::LaunchCtx ctx;
    int rc = device_info(&ctx.dev);
    if (rc != WSG_OK) return rc;
    ctx.stream = tl_stream;
    ctx.wait_stats = tl_wait_stats;
    std::string err;
    rc = wsg::launch_attention(ctx, (int64_t)BH, Sq, Skv, D, Q, K, V, O, scale, causal, stages,
                               cfg ? cfg->producer_waves : 0, cfg ? cfg->consumer_waves : 0, &err);
    if (rc != WSG_OK) return fail(rc, err);
    return ok();
}

int copy_impl(const void *src, void *dst, size_t bytes, int stages, const wsg_config *cfg) {
    if (stages < 1) return fail(WSG_EINVAL, "stages must be >= 1");
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(WSG_EINVAL, "null src or dst with a nonzero size");
    if (((uintptr_t)src % 16) || ((uintptr_t)dst % 16)) return fail(WSG_EINVAL, "src and dst must be 16-byte aligned");
    if (overlaps(src, bytes, dst, bytes)) return fail(WSG_EINVAL, "src and dst overlap");
    wsg::LaunchCtx ctx;
    int rc = device_info(&ctx.dev);
    if (rc != WSG_OK) return rc;
    ctx.stream = tl_stream;
    ctx.wait_stats = tl_wait_stats;
    wsg::CopyPlan plan;
    std::string err;
    rc = wsg::plan_copy(bytes, stages, cfg, ctx.dev, &plan, &err);
    if (rc != WSG_OK) return fail(rc, err);
    rc = wsg::launch_copy(ctx, plan, src, dst, bytes, &err);
    if (rc != WSG_OK) return fail(rc, err);
    return ok();
}

}  // namespace

namespace wsg {

std::string timeout_message(unsigned word) {
    if (!(word & kStatusTimeout)) return "no ring flag wait gave up";
    std::string who;
    const std::pair<unsigned, const char *> kernels[] = {
        {kStatusCopy, "staged_copy"}, {kStatusGemm, "gemm"}, {kStatusAttention, "attention"}};
    for (const auto &k : kernels) {
        if (!(word & k.first)) continue;
        if (!who.empty()) who += " and ";
        who += k.second;
    }
    if (who.empty()) who = "an unnamed kernel";
    return "a ring flag wait gave up in " + who + " (protocol fault)";
}

int prepare_kernel(const void *kernel, const DeviceInfo &dev, std::string *err) {
    std::lock_guard<std::mutex> lock(g_kernel_mu);
    bool &done = g_prepared[{dev.device, kernel}];
    if (done) return WSG_OK;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
    if (e != hipSuccess) {
        *err = std::string("hipFuncSetAttribute: ") + hipGetErrorString(e);
        return WSG_ELAUNCH;
    }
    done = true;
    return WSG_OK;
}

int blocks_per_cu(const void *kernel, const DeviceInfo &dev, int threads, size_t lds) {
    std::lock_guard<std::mutex> lock(g_kernel_mu);
    const auto key = std::make_tuple(dev.device, kernel, threads, lds);
    auto it = g_occupancy.find(key);
    if (it != g_occupancy.end()) return it->second;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
    if (e != hipSuccess || per_cu < 1) per_cu = 1;
    g_occupancy[key] = per_cu;
    return per_cu;
}

}  // namespace wsg

extern "C" {

int gemm_bias_relu(int64_t M, int64_t N, int64_t K, const float *A, const float *B, const float *bias, float *C,
                   int stages) {
    return gemm_impl(WSG_FP32, M, N, K, A, B, bias, C, stages, nullptr);
}

int gemm_bias_relu_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                        float *C, int stages) {
    return gemm_impl(WSG_BF16, M, N, K, A, B, bias, C, stages, nullptr);
}

int gemm_bias_relu_ex(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias,
                      float *C, int stages, const wsg_config *cfg) {
    return gemm_impl(dtype, M, N, K, A, B, bias, C, stages, cfg);
}

int gemm_bias_relu_ex_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                              const void *bias, float *C, int stages, const wsg_config *cfg) {
    return gemm_impl(dtype, M, N, K, A, B, bias, C, stages, cfg, true);
}

int grouped_gemm_bias_relu_ex(int dtype, int groups, const int64_t *group_rows, int64_t N, int64_t K, const void *A,
                              const void *B, const void *bias, float *C, int stages, const wsg_config *cfg) {
    return grouped_impl(dtype, groups, group_rows, N, K, A, B, bias, C, stages, cfg);
}

int attention_fwd(int64_t batch, int64_t heads, int64_t Sq, int64_t Skv, int64_t D, const uint16_t *Q,
                  const uint16_t *K, const uint16_t *V, float *O, float scale, int causal, int stages,
                  const wsg_config *cfg) {
    return attention_impl(batch, heads, Sq, Skv, D, Q, K, V, O, scale, causal, stages, cfg);
}

int wsg_gemm_resolve_config(int dtype, int64_t M, int64_t N, int64_t K, int stages, const wsg_config *cfg,
                            wsg_config *out) {
    if (!out) return fail(WSG_EINVAL, "null output config");
    if (dtype != WSG_FP32 && dtype != WSG_BF16) return fail(WSG_EINVAL, "dtype must be WSG_FP32 or WSG_BF16");
    if (M < 0 || N < 0 || K < 0) return fail(WSG_EINVAL, "negative dimension");
    if (stages < 1) return fail(WSG_EINVAL, "stages must be >= 1");
    wsg::DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != WSG_OK) return rc;
    wsg::GemmPlan plan;
    std::string err;
    // 16-byte aligned operands are assumed, as from any device allocator
    rc = wsg::plan_gemm(dtype, M, N, K, nullptr, nullptr, stages, cfg, dev, &plan, &err);
    if (rc != WSG_OK) return fail(rc, err);
    out->BM = plan.v->BM;
    out->BN = plan.v->BN;
    out->BK = plan.v->BK;
    out->producer_waves = plan.v->P;
    out->consumer_waves = plan.v->CWM * plan.v->CWN;
    out->copy_tile_bytes = 0;
    out->flags = (plan.v->dma ? 0 : WSG_FLAG_GENERAL_PRODUCER) | (plan.v->P == 0 ? WSG_FLAG_HOMOGENEOUS : 0) |
                 (wsg::plan_stream_k(plan, M, N, K, cfg ? cfg->flags : 0, dev).use ? WSG_FLAG_STREAM_K : 0);
    out->group_k = plan.v->GK;
    return ok();
}

int staged_copy(const void *src, void *dst, size_t bytes, int stages) {
    return copy_impl(src, dst, bytes, stages, nullptr);
}

int staged_copy_ex(const void *src, void *dst, size_t bytes, int stages, const wsg_config *cfg) {
    return copy_impl(src, dst, bytes, stages, cfg);
}

int wsg_set_stream(void *hip_stream) {
    tl_stream = static_cast<hipStream_t>(hip_stream);
    return ok();
}

void *wsg_get_stream(void) { return tl_stream; }

const char *wsg_last_error(void) { return tl_err.c_str(); }

int wsg_check_device_status(void) {
    wsg::DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != WSG_OK) return rc;
    hipError_t e = hipStreamSynchronize(tl_stream);
    if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    unsigned word = 0, zero = 0;
    e = hipMemcpy(&word, dev.status, sizeof word, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(dev.status, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("status word copy: ") + hipGetErrorString(e));
    if (word & wsg::kStatusTimeout) return fail(WSG_ETIMEOUT, wsg::timeout_message(word));
    return ok();
}

const char *wsg_status_message(unsigned word) {
    thread_local std::string msg;
    msg = wsg::timeout_message(word);
    return msg.c_str();
}

int wsg_set_wait_stats(int enable) {
    tl_wait_stats = enable != 0;
    return ok();
}

int wsg_read_wait_stats(uint64_t *out) {
    if (!out) return fail(WSG_EINVAL, "null output array");
    wsg::DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != WSG_OK) return rc;
    hipError_t e = hipStreamSynchronize(tl_stream);
    if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    unsigned long long buf[wsg::kStatWords] = {};
    e = hipMemcpy(buf, dev.stats, sizeof buf, hipMemcpyDeviceToHost);
    const unsigned long long zero[wsg::kStatWords] = {};
    if (e == hipSuccess) e = hipMemcpy(dev.stats, zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(WSG_ELAUNCH, std::string("wait statistics copy: ") + hipGetErrorString(e));
    for (int i = 0; i < wsg::kStatWords; ++i) out[i] = buf[i];
    return ok();
}

const char *wsg_version(void) { return "wsg 0.1 (gfx950)"; }

}  // extern "C"
