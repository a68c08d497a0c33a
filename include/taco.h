/*
 * libtaco -- the TACO fused FP8 compression operator for AMD Instinct MI355X
 * (gfx950), as a C ABI.
 *
 * The operator is the one described on the page "TACO: Efficient Communication
 * Compression of Intermediate Tensors for Scalable Tensor-Parallel LLM
 * Training" (cited below as [TACO]):
 *
 *   sender   (section 4.2.2 Eq. 5-8, section 4.3 Eq. 9-10, Algorithm 1, sender
 *             side): split the flattened tensor into contiguous blocks of B
 *             elements; per block compute the RMS amplitude
 *             sigma = sqrt(mean(G^2) + eps) and alpha = tau / sigma; rotate the
 *             rescaled block with the orthonormal Walsh-Hadamard transform,
 *             Z = H_B (alpha G) / sqrt(B); take s = max|Z| / Q_max and emit the
 *             E4M3 codes of Z / s.
 *   receiver (section 4.3 Eq. 11-13, Algorithm 1, receiver side):
 *             G' = H_B (decode(q) * s) / sqrt(B) / alpha.
 *   reduce   (section 4.4.2: the reduce-scatter phase of the two-shot
 *             all-reduce ends in one local reduction of the received
 *             payloads): acc += G' per payload, or for several payloads in
 *             one pass, or reduced and compressed again (the owner step).
 *
 * Beside the operator: the interleaved wire layout of section 4.4.2
 * (*_packed), the E5M2 and INT8 code formats (*_fmt, taco_format), and a
 * fidelity study of the ablation variants (taco_roundtrip).
 *
 * Conventions shared by every call below
 *   - All tensor pointers are DEVICE pointers (any device allocation, e.g. a
 *     torch tensor's data pointer), owned by the caller; the library
 *     allocates nothing and keeps no state between calls (except the fixed
 *     per-GPU working array of taco_roundtrip_noalloc, described there).
 *   - A [tokens, hidden] tensor is row-major and is processed as its
 *     flattened vector of N = tokens * hidden elements; block k covers
 *     elements [k*B, (k+1)*B).  N must be a multiple of B; blocks may cross
 *     rows.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Calls are asynchronous on `stream` (NULL = the null stream).  The
 *     returned status covers argument validation and the kernel launch only.
 *     On any error nothing is launched and nothing is written.
 *   - N == 0 is a no-op that returns TACO_OK (pointers may then be NULL).
 *   - Checks run in this order, and the first that fails decides the status:
 *     format (FORMAT); tokens, hidden and N (SHAPE); block (BLOCK); N % block
 *     (SHAPE); target energy, payload count, variant (PARAM); N == 0 (TACO_OK,
 *     nothing else checked); required pointers (NULL); alignment (ALIGN);
 *     overlaps (ALIAS); the launch (HIP).
 *   - Inputs must be finite.  Blocks whose RMS exceeds ~2^126 / target_energy
 *     get a subnormal float32 alpha (less precise); non-finite inputs give
 *     unspecified codes and scalars (but never out-of-bounds accesses).
 *   - Thread-safe: apart from taco_roundtrip_noalloc's per-GPU working
 *     array, the library has no mutable state.  Calls on different
 *     streams may overlap if their buffers do not.
 */
#ifndef TACO_H
#define TACO_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest finite OCP E4M3 ("E4M3FN") value: Q_max of [TACO] Eq. 9. */
#define TACO_QMAX 448.0f

/* epsilon of [TACO] Eq. 6, inside the square root (the page describes it
 * only as a small stabilising constant for near-zero blocks and gives no
 * value).  Far below the energy of any realistic block, yet it keeps alpha
 * finite (tau * 1e10) for an all-zero block. */
#define TACO_EPS 1e-20f

/* Supported block sizes B.  [TACO] Table 2 sweeps 32..512; 256 is its best. */
#define TACO_MIN_BLOCK 32
#define TACO_MAX_BLOCK 512

/* Largest accepted target energy tau: keeps alpha = tau / sigma finite for
 * an all-zero block (sigma = sqrt(eps)). */
#define TACO_MAX_TARGET_ENERGY 1e20f

/* Most received payloads one taco_reduce_compress or
 * taco_decompress_accumulate_n call sums (tensor parallelism up to 9 ranks). */
#define TACO_MAX_PAYLOADS 8

/* Code formats of Eq. 10-11.  E4M3 is the operator's; the other two keep
 * Eq. 5-13 and change only the code and Q_max ([TACO] section 5.3.2 compares
 * the three formats; section 6 describes the INT8 variant for hardware
 * without FP8):
 *   TACO_FORMAT_E4M3  OCP E4M3FN, Q_max = 448 (TACO_QMAX).
 *   TACO_FORMAT_E5M2  OCP E5M2 (bias 15, with infinities), Q_max = 57344.
 *   TACO_FORMAT_INT8  the uniform quantiser of [TACO] section 2.3 / Eq. 1 with
 *                     the dual scale s as its step: q = round(Z / s), to
 *                     nearest with ties to even, in [-127, 127], stored as a
 *                     two's complement byte; Q_max = 127.
 * Every format rounds the float32 value Z / s (as E4M3 does), and exact
 * zeros encode as 0x00. */
typedef enum {
    TACO_FORMAT_E4M3 = 0,
    TACO_FORMAT_E5M2 = 1,
    TACO_FORMAT_INT8 = 2
} taco_format;

#define TACO_E5M2_MAX 57344.0f
#define TACO_INT8_MAX 127.0f

typedef enum {
    TACO_OK = 0,
    TACO_ERR_NULL = 1,   /* a required pointer is NULL                          */
    TACO_ERR_SHAPE = 2,  /* tokens < 0, hidden <= 0, N > 2^60, N % block != 0    */
    TACO_ERR_BLOCK = 3,  /* block is not one of 32, 64, 128, 256, 512            */
    TACO_ERR_PARAM = 4,  /* target_energy not finite or outside (0, 1e20], a
                            payload count outside 0..TACO_MAX_PAYLOADS, or an
                            unknown taco_variant                               */
    TACO_ERR_ALIGN = 5,  /* a tensor is not 16-byte aligned, or alpha / scale
                            not 4-byte aligned                                  */
    TACO_ERR_ALIAS = 6,  /* an output buffer overlaps an input or another output */
    TACO_ERR_HIP = 7,    /* the HIP runtime refused the launch                  */
    TACO_ERR_FORMAT = 8  /* format is not one of the taco_format values         */
} taco_status;

/* Number of blocks M = tokens * hidden / block, or -1 if the shape or block
 * is invalid (same rules as the calls below). */
int64_t taco_num_blocks(int64_t tokens, int64_t hidden, int32_t block);

/*
 * Compress ([TACO] Eq. 5-10, Algorithm 1, sender side).
 *   x_bf16      [tokens*hidden] bf16 input, 16-byte aligned.
 *   block       B in {32, 64, 128, 256, 512}.
 *   target_energy  tau of Eq. 7 (the codes do not depend on it; alpha and s
 *               scale with it).
 *   codes_e4m3  [tokens*hidden] output: E4M3 code of element i, same order
 *               as x; 16-byte aligned.  Exact zeros of Z encode as 0x00.
 *   alpha       [M] float32 output: alpha_k of Eq. 7.
 *   scale       [M] float32 output: s_k of Eq. 9 (0 for an all-zero block).
 * Outputs must not overlap x or each other.
 */
taco_status taco_compress(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                          int32_t block, float target_energy, uint8_t *codes_e4m3,
                          float *alpha, float *scale, hipStream_t stream);

/*
 * Decompress ([TACO] Eq. 11-13, Algorithm 1, receiver side): y = bf16(G'),
 * rounded to nearest even.  codes / alpha / scale as produced by
 * taco_compress for the same shape and block; y_bf16 [tokens*hidden] is
 * 16-byte aligned and must not overlap the inputs.
 */
taco_status taco_decompress(const uint8_t *codes_e4m3, const float *alpha,
                            const float *scale, int64_t tokens, int64_t hidden,
                            int32_t block, uint16_t *y_bf16, hipStream_t stream);

/*
 * Decompress and accumulate ([TACO] Eq. 11-13 followed by the local
 * reduction of section 4.4.2): acc_f32 += G' (G' in float32, one float32
 * addition per element).  acc_f32 [tokens*hidden] is read and written,
 * 16-byte aligned, and must not overlap the inputs.  Several payloads are
 * summed by calling it once per payload on the same stream.
 */
taco_status taco_decompress_accumulate(const uint8_t *codes_e4m3, const float *alpha,
                                       const float *scale, int64_t tokens,
                                       int64_t hidden, int32_t block, float *acc_f32,
                                       hipStream_t stream);

/*
 * Several payloads at once ([TACO] section 4.4.2: the owner of a segment
 * reduces the payloads it receives): acc_f32 += sum_p G'_p over npayloads
 * (0..TACO_MAX_PAYLOADS) payloads, in one pass.  The payloads are summed in
 * the rotated domain (H G'_p = sqrt(B) (s_p / alpha_p) decode(q_p)) and
 * transformed back once, so the accumulator is read and written once instead
 * of once per payload.  codes_e4m3, alpha, scale: HOST arrays of npayloads
 * DEVICE pointers, each payload as produced by taco_compress with the same
 * shape and block.  acc_f32 as in taco_decompress_accumulate (16-byte aligned,
 * must not overlap any payload).  npayloads == 0 is a no-op.  Rounding
 * differs from npayloads separate taco_decompress_accumulate calls only by
 * float32 evaluation order.
 */
taco_status taco_decompress_accumulate_n(int32_t npayloads, const uint8_t *const *codes_e4m3,
                                         const float *const *alpha, const float *const *scale,
                                         int64_t tokens, int64_t hidden, int32_t block,
                                         float *acc_f32, hipStream_t stream);

/*
 * Owner step of the two-shot all-reduce ([TACO] section 4.4.2: the
 * reduce-scatter phase is one compressed all-to-all followed by a single
 * local reduction, and the reduced segment is compressed again for the
 * all-gather).  Computes the codes, alpha and s ([TACO] Eq. 5-10) of
 *     X = own + sum_p G'_p,     G'_p = the reconstruction (Eq. 11-13) of payload p,
 * in one pass and without materialising X or any G'_p.
 *   own_bf16     [tokens*hidden] bf16, 16-byte aligned, or NULL (X = sum of
 *                the payloads).
 *   npayloads    0..TACO_MAX_PAYLOADS (0 needs own_bf16).
 *   codes_e4m3, alpha, scale
 *                HOST arrays of npayloads DEVICE pointers: payload p is
 *                (codes_e4m3[p] [tokens*hidden], alpha[p] [M], scale[p] [M])
 *                as produced by taco_compress with the same shape and block.
 *   out_codes, out_alpha, out_scale
 *                outputs as in taco_compress; they must not overlap any input
 *                or each other.
 * Rounding differs from decompressing, summing and compressing separately
 * only by float32 evaluation order.
 */
taco_status taco_reduce_compress(const uint16_t *own_bf16, int32_t npayloads,
                                 const uint8_t *const *codes_e4m3, const float *const *alpha,
                                 const float *const *scale, int64_t tokens, int64_t hidden,
                                 int32_t block, float target_energy, uint8_t *out_codes,
                                 float *out_alpha, float *out_scale, hipStream_t stream);

/*
 * Interleaved wire layout ([TACO] section 4.4.2: alpha_k and s_k are stored
 * contiguously with block k's FP8 payload, so a single message carries the
 * whole compressed tensor and a receiver finds the scalars by pointer
 * arithmetic).  A payload is M records of block + 8 bytes: record k holds
 * block k's block codes (same element order as x), then alpha_k and s_k as
 * float32 (little-endian).  Payload buffers are 16-byte aligned.  The calls
 * below compute exactly what their side-buffer counterparts compute; only the
 * placement of codes, alpha and s differs.
 *
 * taco_packed_bytes: payload size M * (block + 8), or -1 for an invalid shape
 * or block (same rules as taco_num_blocks).
 */
int64_t taco_packed_bytes(int64_t tokens, int64_t hidden, int32_t block);

/* taco_compress writing one interleaved payload (must not overlap x). */
taco_status taco_compress_packed(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                 int32_t block, float target_energy, uint8_t *payload,
                                 hipStream_t stream);

/* taco_decompress reading one interleaved payload. */
taco_status taco_decompress_packed(const uint8_t *payload, int64_t tokens, int64_t hidden,
                                   int32_t block, uint16_t *y_bf16, hipStream_t stream);

/* taco_decompress_accumulate reading one interleaved payload. */
taco_status taco_decompress_accumulate_packed(const uint8_t *payload, int64_t tokens,
                                              int64_t hidden, int32_t block, float *acc_f32,
                                              hipStream_t stream);

/* taco_reduce_compress with interleaved payloads: payloads is a HOST array of
 * npayloads DEVICE pointers to payloads; the result is one interleaved
 * payload (must not overlap own or any input payload). */
taco_status taco_reduce_compress_packed(const uint16_t *own_bf16, int32_t npayloads,
                                        const uint8_t *const *payloads, int64_t tokens,
                                        int64_t hidden, int32_t block, float target_energy,
                                        uint8_t *out_payload, hipStream_t stream);

/*
 * The calls above with a code format (taco_format): the same operations,
 * validation and layouts, with codes of that format and its Q_max.  The
 * format is checked first (TACO_ERR_FORMAT, also for N == 0).  Payloads of
 * one format must be decoded, accumulated and reduced with the same format.
 * The calls without a format are these with TACO_FORMAT_E4M3.
 */
taco_status taco_compress_fmt(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                              int32_t block, float target_energy, taco_format format,
                              uint8_t *codes, float *alpha, float *scale, hipStream_t stream);
taco_status taco_decompress_fmt(const uint8_t *codes, const float *alpha, const float *scale,
                                int64_t tokens, int64_t hidden, int32_t block, taco_format format,
                                uint16_t *y_bf16, hipStream_t stream);
taco_status taco_decompress_accumulate_fmt(const uint8_t *codes, const float *alpha,
                                           const float *scale, int64_t tokens, int64_t hidden,
                                           int32_t block, taco_format format, float *acc_f32,
                                           hipStream_t stream);
taco_status taco_reduce_compress_fmt(const uint16_t *own_bf16, int32_t npayloads,
                                     const uint8_t *const *codes, const float *const *alpha,
                                     const float *const *scale, int64_t tokens, int64_t hidden,
                                     int32_t block, float target_energy, taco_format format,
                                     uint8_t *out_codes, float *out_alpha, float *out_scale,
                                     hipStream_t stream);
taco_status taco_compress_packed_fmt(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                     int32_t block, float target_energy, taco_format format,
                                     uint8_t *payload, hipStream_t stream);
taco_status taco_decompress_packed_fmt(const uint8_t *payload, int64_t tokens, int64_t hidden,
                                       int32_t block, taco_format format, uint16_t *y_bf16,
                                       hipStream_t stream);
taco_status taco_decompress_accumulate_packed_fmt(const uint8_t *payload, int64_t tokens,
                                                  int64_t hidden, int32_t block,
                                                  taco_format format, float *acc_f32,
                                                  hipStream_t stream);
taco_status taco_decompress_accumulate_n_fmt(int32_t npayloads, const uint8_t *const *codes,
                                             const float *const *alpha, const float *const *scale,
                                             int64_t tokens, int64_t hidden, int32_t block,
                                             taco_format format, float *acc_f32,
                                             hipStream_t stream);
/* taco_decompress_accumulate_n with interleaved payloads (HOST array of
 * npayloads DEVICE pointers to payloads). */
taco_status taco_decompress_accumulate_n_packed(int32_t npayloads, const uint8_t *const *payloads,
                                                int64_t tokens, int64_t hidden, int32_t block,
                                                float *acc_f32, hipStream_t stream);
taco_status taco_decompress_accumulate_n_packed_fmt(int32_t npayloads,
                                                    const uint8_t *const *payloads, int64_t tokens,
                                                    int64_t hidden, int32_t block,
                                                    taco_format format, float *acc_f32,
                                                    hipStream_t stream);
taco_status taco_reduce_compress_packed_fmt(const uint16_t *own_bf16, int32_t npayloads,
                                            const uint8_t *const *payloads, int64_t tokens,
                                            int64_t hidden, int32_t block, float target_energy,
                                            taco_format format, uint8_t *out_payload,
                                            hipStream_t stream);

/*
 * Fidelity study: round trips of the operator and of the variants [TACO]
 * compares it with, measured against the input.
 *   TACO_VARIANT_TACO      the operator: ASH + DS, Eq. 5-13 (compress, then
 *                          decompress, in one pass; codes stay in registers).
 *   TACO_VARIANT_DIRECT    direct cast of x to codes, no scaling (section
 *                          4.2.1 direct FP8 quantization; the NVFP8 arm of
 *                          section 5.2.2); saturating at +-Q_max.
 *   TACO_VARIANT_DS        dual scale alone: per block s = max|x| / Q_max,
 *                          no rotation (section 5.2.2, DS in isolation).
 *   TACO_VARIANT_ASH       Eq. 6-8 without the post-rotation scale: codes of
 *                          Z itself, saturating (section 5.2.2, ASH alone).
 *   TACO_VARIANT_HADAMARD  the standard rotation alone, Z = H x / sqrt(B),
 *                          saturating (sections 4.2.1 and 5.3.1).
 *   TACO_VARIANT_TENSOR    one scale for the whole tensor, max|x| / Q_max (the
 *                          quantiser of section 2.3 / Eq. 1 with INT8 codes).
 * Every variant uses the code format given (and its Q_max).
 */
typedef enum {
    TACO_VARIANT_TACO = 0,
    TACO_VARIANT_DIRECT = 1,
    TACO_VARIANT_DS = 2,
    TACO_VARIANT_ASH = 3,
    TACO_VARIANT_HADAMARD = 4,
    TACO_VARIANT_TENSOR = 5
} taco_variant;

/* Sums a round trip accumulates, in device memory (8-byte aligned; the
 * caller allocates sizeof(taco_fidelity_sums) bytes).  With n elements, x
 * the input and x' the float32 reconstruction (before any output rounding),
 * the metrics of the GIFT page's Eq. 21 ("GIFT: Geometry-Informed
 * Low-precision Gradient Communication for LLM Pretraining") are
 * RelL2 = sqrt(sum_sq_err / sum_sq_ref),
 * Cos = sum_dot / sqrt(sum_sq_ref * sum_sq_out), MaxErr = max_abs_err and
 * MSE = sum_sq_err / n.  Per-block partial sums are float32; work-groups add
 * them in double, with atomics, into TACO_FIDELITY_SLOTS slots (so the last
 * bits of a total vary between runs); the totals are the slots' sum. */
#define TACO_FIDELITY_SLOTS 64
typedef struct {
    double sum_sq_err;    /* sum (x' - x)^2 */
    double sum_sq_ref;    /* sum x^2 */
    double sum_sq_out;    /* sum x'^2 */
    double sum_dot;       /* sum x' x */
    float max_abs_err;    /* max |x' - x| */
    float tensor_absmax;  /* max |x| (TACO_VARIANT_TENSOR only; else 0) */
    /* Written by the library before the totals above (contents unspecified
     * for the caller). */
    double slot_sum[4][TACO_FIDELITY_SLOTS];
    uint32_t slot_max_err[TACO_FIDELITY_SLOTS];
    uint32_t slot_absmax[TACO_FIDELITY_SLOTS];
} taco_fidelity_sums;

/*
 * One round trip of a variant over a bf16 tensor (shape, block and
 * target_energy as in taco_compress; target_energy is used by the TACO and
 * ASH variants).  sums (required, device) is overwritten with this call's
 * sums; y_bf16 (optional, NULL for none) receives x' rounded to bf16.
 * sums must not overlap x or y.  A bad variant is TACO_ERR_PARAM.  As
 * everywhere, N == 0 is a no-op (sums is then not written).
 */
taco_status taco_roundtrip(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                           int32_t block, float target_energy, taco_format format,
                           taco_variant variant, uint16_t *y_bf16, taco_fidelity_sums *sums,
                           hipStream_t stream);

/* The totals of taco_fidelity_sums alone: the same six fields, in the same
 * order and at the same offsets as its first members (40 bytes). */
typedef struct {
    double sum_sq_err;
    double sum_sq_ref;
    double sum_sq_out;
    double sum_dot;
    float max_abs_err;
    float tensor_absmax;
} taco_fidelity_totals;

/*
 * taco_roundtrip for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It computes exactly what taco_roundtrip computes (same kernels, same
 * validation; a bad variant is TACO_ERR_PARAM), but the working memory that
 * taco_roundtrip keeps in the caller's taco_fidelity_sums (the per-slot
 * partial sums) lives in a fixed array inside the library, one per GPU
 * (TACO_ROUNDTRIP_SCRATCH_BYTES, held until the process ends); the caller
 * passes only the outputs.
 *   totals   (required, device, 8-byte aligned) overwritten with this call's
 *            totals; must not overlap x or y.
 *   y_bf16   as in taco_roundtrip (optional).
 * The working memory does not grow with the tensor: every accepted shape
 * fits it, so no size is refused for lack of it.  The first call on a
 * device looks up that device's copy of the array (the current device,
 * which must be the device of `stream`, one of the first 64 devices; a
 * failed lookup is TACO_ERR_HIP and launches nothing): make that first call
 * before capturing a graph.  No call allocates or frees memory.  Every call on one
 * GPU shares that GPU's array, and each call clears it first (with a
 * kernel, on `stream`): calls on one GPU must therefore not overlap in time
 * (calls on different streams race, and their totals are then undefined);
 * calls on one stream are ordered and safe.  N == 0 is a no-op (totals not
 * written).
 */
#define TACO_ROUNDTRIP_SCRATCH_BYTES 4096
taco_status taco_roundtrip_noalloc(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                   int32_t block, float target_energy, taco_format format,
                                   taco_variant variant, uint16_t *y_bf16,
                                   taco_fidelity_totals *totals, hipStream_t stream);

/*
 * The E4M3 conversions the kernels above use (Cvt_FP8 of [TACO] Eq. 10 and
 * Cvt_FP32 of Eq. 11), exposed element-wise so that they can be checked
 * exhaustively.  encode: round to nearest even, OCP E4M3FN; inputs of
 * magnitude 464 or more are outside its contract (the operator never
 * produces them).  decode: exact.  n >= 0 elements; x / out 16-byte aligned,
 * codes 16-byte aligned; outputs must not overlap inputs.
 */
taco_status taco_e4m3_encode(const float *x, int64_t n, uint8_t *codes, hipStream_t stream);
taco_status taco_e4m3_decode(const uint8_t *codes, int64_t n, float *out, hipStream_t stream);

/* The same for any format (taco_e4m3_* are these with TACO_FORMAT_E4M3).
 * Encode contracts: |x| < 464 (E4M3), |x| < 61440 (E5M2), |x| < 127.5
 * (INT8); larger inputs give unspecified codes. */
taco_status taco_encode(taco_format format, const float *x, int64_t n, uint8_t *codes,
                        hipStream_t stream);
taco_status taco_decode(taco_format format, const uint8_t *codes, int64_t n, float *out,
                        hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *taco_status_string(taco_status status);

#ifdef __cplusplus
}
#endif

#endif /* TACO_H */
