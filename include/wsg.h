/*
 * wsg.h - C ABI of libwsg.so: a wave-specialized GEMM with a fused bias + ReLU
 * epilogue and an LDS-staged copy, for AMD MI355X (gfx950).
 *
 * Sources (three web pages on warp specialization):
 *   [KP] pwwt.cn/news/4436243, Chinese article on intra-kernel pipelining
 *        with TMA and mbarrier; section 4.1 defines the operator: float
 *        A[M,K], B[K,N], C[M,N] = A*B + bias followed by a ReLU; sections
 *        3.2-3.4 describe producer and consumer warps joined by a ring of
 *        shared-memory stages with a full and an empty barrier per stage.
 *   [WS] aicassindra.com, "GPU warp specialization"; "End-to-end flow": one
 *        output tile per block, K-dimension tiles of A and B streamed through
 *        an N-stage ring by producer warps while consumer warps accumulate.
 *   [PC] willy-chan.github.io, "Producer-Consumer Warp Specialization for
 *        TMA Operations": a double-buffered load into shared memory and store
 *        back out to global memory, tile i in buffer i mod 2, waits on the
 *        parity of i / 2.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     allocates no memory for them and keeps no pointer after returning.
 *   - Launches are asynchronous on the calling thread's stream (see
 *     wsg_set_stream); the caller keeps buffers alive and synchronizes before
 *     reading results, as with any stream API.
 *   - Matrices are dense row-major: A[m*K + k], B[k*N + n], C[m*N + n];
 *     bias has N entries, one per output column.
 *   - Return codes: WSG_OK, or a negative WSG_E* code; wsg_last_error()
 *     then returns a description (thread-local).
 */
#ifndef WSG_H
#define WSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WSG_OK 0
#define WSG_EINVAL (-1)       /* invalid argument: negative size, null or misaligned pointer, overlap, stages < 1 */
#define WSG_EUNSUPPORTED (-2) /* configuration the device cannot run: LDS over the per-workgroup limit, tile or wave
                                 combination not built, sizes beyond the 32-bit offsets of a tile */
#define WSG_ELAUNCH (-3)      /* HIP runtime error while launching; see wsg_last_error() */
#define WSG_ETIMEOUT (-4)     /* a bounded flag wait on the device gave up (reported by wsg_check_device_status) */

/* dtype codes for gemm_bias_relu_ex, grouped_gemm_bias_relu_ex and wsg_gemm_resolve_config */
#define WSG_FP32 0
#define WSG_BF16 1

/* flags for wsg_config.flags */
#define WSG_FLAG_GENERAL_PRODUCER 1 /* GEMM: force the register-staged producer (any shape) over the LDS-DMA one */
#define WSG_FLAG_NONTEMPORAL 2      /* staged copy: streaming (non-temporal) loads and stores */
#define WSG_FLAG_HOMOGENEOUS 4      /* GEMM: the baseline without roles (see below); producer_waves must be 0 */
#define WSG_FLAG_DIRECT_COPY 8      /* staged copy: the baseline without staging (see staged_copy_ex) */
#define WSG_FLAG_STREAM_K 16        /* fp32 GEMM: always give the last round of tiles a stream-K split (see below) */
#define WSG_FLAG_NO_STREAM_K 32     /* fp32 GEMM: never split tiles along K: one workgroup per output tile */

/*
 * Launch configuration. A zero field means "choose the default". The
 * workgroup runs producer_waves + consumer_waves wavefronts of 64 lanes.
 */
typedef struct wsg_config {
    int BM, BN, BK;       /* GEMM workgroup tile: rows of C, columns of C, k per ring slot */
    int producer_waves;   /* waves that fill the ring */
    int consumer_waves;   /* waves that drain it (GEMM: run the MFMAs; copy: store to dst) */
    int copy_tile_bytes;  /* staged copy: bytes per ring slot (default 65536) */
    int flags;            /* WSG_FLAG_* */
    int group_k;          /* GEMM consumers: k per fragment group read ahead of the MFMAs (16 or 32) */
    int copy_workgroups;  /* staged copy: workgroups in the persistent grid (default: see staged_copy) */
} wsg_config;

/*
 * C = relu(A @ B + bias), fp32 operands and output, fp32 MFMA with fp32
 * accumulation ([KP] section 4.1). The K loop runs through an LDS ring of
 * `stages` slots: producer waves load K-tiles of A and B into slot t mod S
 * and mark it full; consumer waves wait for it with parity (t / S) & 1,
 * multiply, and mark it empty ([WS] "End-to-end flow"; [PC]).
 *   M, N, K  >= 0. M == 0 or N == 0: nothing written. K == 0: C = relu(bias).
 *   A        M x K, B K x N, bias N, C M x N; 4-byte aligned; C must not
 *            overlap A, B or bias.
 *   stages   ring depth S >= 1; S beyond what fits in LDS -> WSG_EUNSUPPORTED.
 *            The default tiles run fastest at S = 2 on MI355X: a deeper ring
 *            leaves LDS only for shallower k tiles (bf16 256 x 256 tiles take
 *            k = 64 at S = 2 but k = 32 at S = 4, about 12% slower at 8192^3).
 * relu(x) is x for x > 0, NaN for NaN, +0 otherwise. Any M, N, K are
 * accepted; out-of-range rows, columns and k are zero-filled by the producer.
 */
int gemm_bias_relu(int64_t M, int64_t N, int64_t K, const float *A, const float *B, const float *bias,
                   float *C, int stages);

/*
 * The same operator with bf16 operands and bias (raw bf16 bit patterns,
 * 2-byte aligned), bf16 MFMA with fp32 accumulation, fp32 output C.
 */
int gemm_bias_relu_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                        const uint16_t *bias, float *C, int stages);

/*
 * Either GEMM with an explicit launch configuration (cfg may be NULL).
 * dtype is WSG_FP32 (A, B, bias are float*) or WSG_BF16 (uint16_t* bits).
 */
int gemm_bias_relu_ex(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                      const void *bias, float *C, int stages, const wsg_config *cfg);

/* Bytes of the per-device scratch array of gemm_bias_relu_ex_noalloc: 72 MiB. */
#define WSG_NOALLOC_SCRATCH_BYTES 75497472

/*
 * gemm_bias_relu_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same kernels and results as gemm_bias_relu_ex (bit for bit,
 * same arguments and configuration), but the stream-K workspace is a static
 * device array of WSG_NOALLOC_SCRATCH_BYTES that every GPU the library runs
 * on holds until the process ends; no call allocates or frees. A launch whose
 * stream-K workspace would exceed it returns WSG_EUNSUPPORTED (on a 256-CU
 * device the built tile shapes need 64 MiB of partial sums, two tiles' fp32
 * accumulators per resident workgroup, and a few KiB of counters;
 * WSG_FLAG_NO_STREAM_K needs none). The array keeps the last call's contents;
 * each launch clears the counters it uses, with a kernel. All calls on one
 * GPU share the array: calls that may overlap on that GPU (on different
 * streams, or from different threads without ordering) race and must be
 * serialized by the caller.
 */
int gemm_bias_relu_ex_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                              const void *bias, float *C, int stages, const wsg_config *cfg);

/* Largest number of experts one grouped launch takes. */
#define WSG_MAX_GROUPS 64

/*
 * Grouped GEMM + bias + ReLU for the expert layer of a mixture-of-experts
 * model, the operator [KP] section 1.1 was tuning when it met the
 * load-barrier-compute loop. The token rows of A are sorted by expert;
 * expert e owns the next group_rows[e] rows and applies its own weights and
 * biases:
 *   C[r_e + i, :] = relu(A[r_e + i, :] @ B[e] + bias[e]),  0 <= i < group_rows[e],
 *   r_e = group_rows[0] + ... + group_rows[e - 1].
 *   groups      1 .. WSG_MAX_GROUPS (< 1: WSG_EINVAL; above: WSG_EUNSUPPORTED).
 *   group_rows  HOST array of `groups` row counts >= 0 (0: an expert with no
 *               tokens); read during the call, not kept. Their sum is A's and
 *               C's row count.
 *   A           rows x K;  B  `groups` blocks of K x N, B[e*K*N + k*N + n];
 *   bias        groups x N;  C  rows x N (fp32).
 *   dtype, stages, cfg, alignment and overlap rules as gemm_bias_relu_ex, with
 *   B and bias at their full sizes. The default tile is chosen for the total
 *   row count.
 * One launch covers every expert's tiles (each expert's rows are tiled on
 * their own, so its last tile row is ragged); every expert's rows equal what
 * gemm_bias_relu_ex returns for that expert's slice with the same explicit
 * configuration and WSG_FLAG_NO_STREAM_K (grouped launches take no stream-K
 * tail).
 */
int grouped_gemm_bias_relu_ex(int dtype, int groups, const int64_t *group_rows, int64_t N, int64_t K,
                              const void *A, const void *B, const void *bias, float *C, int stages,
                              const wsg_config *cfg);

/*
 * WSG_FLAG_HOMOGENEOUS selects the kernel the wave-specialized one is measured
 * against ([KP] section 1.1): the same tiles, slot layout and consumer
 * fragments, but no producer waves. Every wave loads its share of each K-tile,
 * a workgroup barrier publishes the tile, and every wave computes on it.
 * stages == 1 is that loop as written (load, barrier, compute, barrier);
 * stages >= 2 loads tile t + S - 1 while tile t is computed, with one barrier
 * per tile. It needs the LDS-DMA alignment (K and N multiples of 16 bytes,
 * 16-byte aligned A and B; else WSG_EUNSUPPORTED).
 *
 * Stream-K tail (fp32, wave-specialized LDS-DMA kernels; not from the pages,
 * which launch one workgroup per output tile): when the tiles fill at least
 * one round of the device's resident workgroups and the last round is at most
 * 90% full, or when there are fewer tiles of 256 x 128 or more than resident
 * workgroups but at least 16 k steps of BK per workgroup, the launch is a
 * persistent grid of one round. With the default tile, such a deep-K problem
 * keeps the 256 x 128 tile rather than a smaller one when 128 x 128 tiles
 * would leave CUs idle or there are at least 64 k steps per CU. Each workgroup takes
 * its whole-tile rounds, then an equal share of the remaining tiles' K steps;
 * a tile split between workgroups is summed in a fixed order (its pieces by
 * increasing k, added by whichever workgroup finishes the last piece; no
 * workgroup waits for another), so results do not depend on timing but differ
 * in rounding from the one-workgroup-per-tile launch.
 * WSG_FLAG_STREAM_K forces the split (with no ragged round, the last full
 * round is split); WSG_FLAG_NO_STREAM_K forbids it. The partial sums and
 * counters live in a device workspace the library allocates on first need
 * per (device, stream) and keeps until the process ends; growing it waits
 * for that stream, so a launch that would need to allocate or grow it cannot
 * be captured in a HIP graph (gemm_bias_relu_ex_noalloc can).
 */

/*
 * Scaled dot-product attention forward, the second consumer type: [WS] names
 * attention beside GEMM among the kernels built on producer and consumer warps.
 *   O[b, h, i, :] = sum_j P[i, j] V[b, h, j, :],
 *   P[i, :] = softmax_j(scale * Q[b, h, i, :] . K[b, h, j, :])
 * over the keys j the query may see: all of them, or with causal != 0 those
 * with j <= i + (Skv - Sq) (the last query and the last key are aligned). A
 * query that sees no key gets a row of zeros.
 *   Q       batch x heads x Sq x D, K and V batch x heads x Skv x D: bf16 bit
 *           patterns, dense row-major, 16-byte aligned.
 *   O       batch x heads x Sq x D fp32, 4-byte aligned, not overlapping the
 *           inputs.
 *   D       64 or 128 (else WSG_EUNSUPPORTED); sizes >= 0.
 *   scale   finite and at least 2^-126 (positive and normal), else
 *           WSG_EINVAL: each row's maximum is taken before scaling.
 *   stages  ring slots of 64 keys (K and V tiles, 32 KiB per slot for
 *           D = 128): 1 .. 4 for D = 128, 1 .. 9 for D = 64.
 *   cfg     may be NULL; cfg->producer_waves (1, 2 or 4; 0 = default) and
 *           cfg->consumer_waves (4, or 7 with one producer for D = 128;
 *           0 = default). Other combinations: WSG_EUNSUPPORTED.
 * Producer waves stream K and V tiles through the LDS ring; each consumer wave
 * keeps 32 queries' rows in registers and runs an online softmax (running max
 * and sum) with MFMAs for Q K^T and P V. Scores, softmax and accumulation are
 * fp32; P is rounded to bf16 for the P V products.
 */
int attention_fwd(int64_t batch, int64_t heads, int64_t Sq, int64_t Skv, int64_t D, const uint16_t *Q,
                  const uint16_t *K, const uint16_t *V, float *O, float scale, int causal, int stages,
                  const wsg_config *cfg);

/*
 * The configuration gemm_bias_relu_ex would launch for these arguments,
 * written to *out, after the same validation (returns its error code).
 * Writes the resolved tile and wave counts; no device work. flags reports
 * WSG_FLAG_GENERAL_PRODUCER, WSG_FLAG_HOMOGENEOUS and WSG_FLAG_STREAM_K for
 * the kernel that would run.
 */
int wsg_gemm_resolve_config(int dtype, int64_t M, int64_t N, int64_t K, int stages, const wsg_config *cfg,
                            wsg_config *out);

/*
 * dst[0:bytes] = src[0:bytes], staged through a ring of `stages` LDS slots
 * ([PC]): producer waves load a tile into slot j mod S and mark it full;
 * consumer waves wait on its parity, copy it out to dst and mark it empty.
 *   src, dst  device pointers, 16-byte aligned, non-overlapping (else
 *             WSG_EINVAL); any byte count, bytes == 0 is a no-op.
 *   stages    S >= 1; S * tile bytes must fit in LDS (else WSG_EUNSUPPORTED,
 *             e.g. 3 x 64 KiB).
 * Bits move as integers: NaN payloads and -0 are preserved.
 */
int staged_copy(const void *src, void *dst, size_t bytes, int stages);

/*
 * staged_copy with an explicit configuration (copy_tile_bytes, wave counts,
 * copy_workgroups; cfg may be NULL). The grid is persistent: workgroup g
 * copies tiles g, g + G, ... By default G is 3/4 of the workgroups the device
 * holds at once for 64 KiB slots and 15/16 for smaller slots (measured on
 * MI355X: fewer concurrent streams of large tiles keep HBM busier; a
 * 1 GiB copy with 64 KiB slots runs at 6.0 TB/s with 192 workgroups and
 * 5.5 TB/s with 256). copy_workgroups > 0 sets G (capped at the tile count).
 *
 * WSG_FLAG_DIRECT_COPY selects the copy the staged one is measured against:
 * no LDS ring and no roles, every lane moving 16-byte chunks src -> registers
 * -> dst in a grid-stride loop with 4 chunks in flight (one 4-wave workgroup
 * per CU unless copy_workgroups says otherwise; WSG_FLAG_NONTEMPORAL applies;
 * stages is validated but not used). Same arguments, same result.
 */
int staged_copy_ex(const void *src, void *dst, size_t bytes, int stages, const wsg_config *cfg);

/*
 * Stream used by this thread's later launches (a hipStream_t; NULL = the
 * default stream). Thread-local. Returns WSG_OK.
 */
int wsg_set_stream(void *hip_stream);

/* The calling thread's current stream (as set by wsg_set_stream). */
void *wsg_get_stream(void);

/* Text describing the calling thread's last nonzero return code ("" if none). */
const char *wsg_last_error(void);

/*
 * Synchronizes the calling thread's stream, then reads and clears the
 * current device's status word. Every flag wait in the kernels gives up after
 * a bounded number of polls (so a protocol fault ends the kernel instead of
 * hanging the GPU) and records it there. Returns WSG_OK, WSG_ETIMEOUT, or
 * WSG_ELAUNCH if synchronization failed.
 */
int wsg_check_device_status(void);

/*
 * Status-word bits, as wsg_check_device_status reads them: WSG_STATUS_TIMEOUT
 * is set when a wait gave up, together with the bit of the kernel it was in.
 */
#define WSG_STATUS_TIMEOUT 1u
#define WSG_STATUS_COPY 2u
#define WSG_STATUS_GEMM 4u
#define WSG_STATUS_ATTENTION 8u

/*
 * The message wsg_check_device_status reports for a status word `word`
 * (naming every kernel whose bit is set). Host-only, no device access; the
 * returned text is thread-local and valid until the thread's next call.
 */
const char *wsg_status_message(unsigned word);

/*
 * Wait statistics, a diagnostic of the ring handshake: with wsg_set_wait_stats(1)
 * the calling thread's later launches count, per role, every flag wait, the
 * waits that found the flag not yet flipped, and the polls those took (each
 * wave keeps the counts in registers and adds them once at its end). The
 * pages' steady state, consumers never waiting for data and producers
 * blocked on free slots, reads directly off these numbers.
 * wsg_read_wait_stats synchronizes the calling thread's stream, copies the
 * current device's 16 counters to out[16] and clears them:
 *   out[0..2]   GEMM consumers, full waits   {waits, blocked, polls}
 *               (a wait settled by an early read of the flag counts as unblocked)
 *   out[3..5]   GEMM producers, empty waits  {waits, blocked, polls}
 *   out[6..8]   copy consumers, full waits
 *   out[9..11]  copy producers, empty waits
 *   out[12..14] attention consumers, full waits
 *   out[15]     zero
 * Counts accumulate over launches and across streams of one device until read.
 */
int wsg_set_wait_stats(int enable);
int wsg_read_wait_stats(uint64_t *out);

/* Library version string. */
const char *wsg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WSG_H */
