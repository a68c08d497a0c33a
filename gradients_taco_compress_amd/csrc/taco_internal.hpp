// Declarations shared by the translation units of libtaco: the per-format
// kernel sets (taco_e4m3.hip, taco_e5m2.hip, taco_int8.hip, each compiling
// taco_kernels.hpp for one format) and the C ABI (taco_abi.hip).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "taco.h"

namespace taco_internal {

// Code format of Eq. 10-11: E4M3 (the operator's), E5M2 and INT8.
enum class Fmt { kE4M3, kE5M2, kInt8 };

// Side buffers (codes, alpha, scale) or interleaved records of B + 8 bytes.
enum class Layout { kSide, kPacked };

// Decompress output: bf16 tensor, or float32 accumulator (acc += G').
enum class Out { kBf16, kAccumulate };

// Round-trip variants of the fidelity study (taco_variant of taco.h).
enum class Variant { kTaco, kDirect, kDs, kAsh, kHadamard, kTensor };

// Device pointers of the owner step's received payloads, passed by value to
// the kernel.  For the interleaved layout, alpha[p] / scale[p] point at the
// scalars of payload p's record 0.
struct Payloads {
    const uint8_t *codes[TACO_MAX_PAYLOADS];
    const float *alpha[TACO_MAX_PAYLOADS];
    const float *scale[TACO_MAX_PAYLOADS];
};

// Kernel launches for one code format.  Arguments are validated by the
// caller; nblocks >= 1; block is one of the supported sizes.  For the
// interleaved layout, codes points at record 0 and alpha / scale at record
// 0's scalars.
template <Fmt F>
struct Ops {
    static taco_status compress(Layout layout, int32_t block, const uint16_t *x, int64_t nblocks,
                                float tau, uint8_t *codes, float *alpha, float *scale,
                                hipStream_t stream);
    static taco_status decompress(Layout layout, Out mode, int32_t block, const uint8_t *codes,
                                  const float *alpha, const float *scale, int64_t nblocks,
                                  uint16_t *y, float *acc, hipStream_t stream);
    static taco_status reduce_compress(Layout layout, int32_t block, int npay,
                                       const uint16_t *own, const Payloads &pay, int64_t nblocks,
                                       float tau, uint8_t *codes, float *alpha, float *scale,
                                       hipStream_t stream);
    // acc += the sum of npay (1..8) payloads' reconstructions.
    static taco_status accumulate_n(Layout layout, int32_t block, int npay, const Payloads &pay,
                                    int64_t nblocks, float *acc, hipStream_t stream);
    // Clears *sums, then (kTensor) finds max|x|, then runs the round trip,
    // then writes the totals of the slots of *sums to *totals (which may be
    // the front of *sums).
    static taco_status roundtrip(Variant variant, int32_t block, const uint16_t *x,
                                 int64_t nblocks, float tau, uint16_t *y,
                                 taco_fidelity_sums *sums, taco_fidelity_totals *totals,
                                 hipStream_t stream);
    static taco_status encode(const float *x, int64_t n, uint8_t *codes, hipStream_t stream);
    static taco_status decode(const uint8_t *codes, int64_t n, float *out, hipStream_t stream);
};

extern template struct Ops<Fmt::kE4M3>;
extern template struct Ops<Fmt::kE5M2>;
extern template struct Ops<Fmt::kInt8>;

}  // namespace taco_internal
