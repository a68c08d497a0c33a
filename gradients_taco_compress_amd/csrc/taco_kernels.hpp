// libtaco kernels: the TACO compression operator as hand-written HIP for
// gfx950, templated on the code format.  Each taco_<format>.hip includes this
// file and instantiates Ops<format>; the C ABI (taco_abi.hip) calls those.
//
// Operator: [TACO] = the page "TACO: Efficient Communication Compression of
// Intermediate Tensors for Scalable Tensor-Parallel LLM Training", section
// 4.2.2 (Eq. 5-8), section 4.3 (Eq. 9-13), Algorithm 1 and section 4.4.1
// (one fused kernel per direction).  The C ABI is documented in taco.h.
//
// Design (gfx950, wave64, no MFMA: the path streams HBM and does O(B log B)
// adds per block, nothing here is a dense contraction; the transform needs no
// LDS, which serves only as a wave-private staging area that makes the
// memory traffic contiguous, and for the fidelity sums):
//
//  * Lane layout.  A block of B elements is owned by LPB = 8 lanes of one
//    wavefront (4 lanes when B = 32, 16 when B = 512).  Lane t of a block
//    holds the 16-byte chunks k = 0..B/(8*LPB)-1 at element offset
//    8*LPB*k + 8*t, so each load instruction of the wave reads whole
//    128-byte lines.  Within a block the element index is
//    e = 8*LPB*k + 8*t + j:  bits of j (register) and k (register) are
//    butterflied in registers, bits of t across lanes.
//  * Lane bits of t are lane-id bits 0, 1 and 3, the three that gfx9 DPP
//    reaches in one instruction (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
//    row_ror:8); lane-id bits 2, 4, 5 select one of the 8 blocks a wave
//    handles per step.  At B = 512 (16 lanes, 32 values each instead of 64,
//    which would take 146-190 VGPRs) t also takes lane-id bit 2, whose stage
//    goes through ds_swizzle; bits 4 and 5 select one of 4 blocks.
//  * Cross-lane butterfly in one instruction per element:
//    v <- v + sgn * v@partner  (v_fmac_f32_dpp, sgn = -1 on the upper lane).
//    The upper lane then holds the negated butterfly output; partners always
//    carry the same accumulated sign, so after all stages lane t holds
//    (-1)^popcount(t) * (H x).  That sign is folded into the per-lane
//    quantisation factor (compress) or output factor (decompress), so it
//    costs nothing per element.
//  * Fused single pass ([TACO] section 4.4.1 fuses the energy reduction and
//    the post-rotation max into the one kernel): since Z = alpha H x / sqrt(B)
//    and s = max|Z| / Q, the code argument is Z / s = Q * (H x) / max|H x|, so
//    the kernel rotates the raw block R = H x, reduces sum x^2 and max |R|,
//    and quantises v = R * (Q / max|R|).  alpha and s are computed once per
//    block from the two reductions.
//  * Stores: 8 codes per lane per chunk, gathered per wave-step in LDS and
//    written as contiguous 16-byte pieces; alpha / s as float32.  E4M3 and E5M2
//    use the hardware conversions (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32, OCP
//    formats on gfx950, round to nearest even); INT8 rounds with one float
//    addition (see Codec<Fmt::kInt8>).  Decompress decodes, rotates and
//    rounds to bf16 with v_cvt_pk_bf16_f32.
//  * Grid-stride loop over wave-steps (one step per wave by default, so a
//    large tensor launches tens of thousands of work-groups); when a wave
//    has several steps, the next step's loads are issued before the current
//    step is processed.  Every byte is streamed once; the cache policy of
//    each access (non-temporal or not) is chosen by measurement below.
//  * Beyond the operator's two directions: the owner step of the two-shot
//    all-reduce (reduce_compress_kernel) and the multi-payload accumulate
//    (accumulate_n_kernel) add payloads in the rotated domain, since
//    H H = B I; the fidelity round trip (roundtrip_kernel) runs the operator
//    and its ablation variants with the codes kept in registers.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "taco.h"
#include "taco_internal.hpp"

namespace taco_internal {
namespace {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

#ifndef TACO_WAVES_PER_GROUP
#define TACO_WAVES_PER_GROUP 4
#endif
constexpr int kWave = 64;
constexpr int kWavesPerGroup = TACO_WAVES_PER_GROUP;
constexpr int kGroup = kWave * kWavesPerGroup;

// Lanes per block for each block size (4 or 8; 4 halves the per-block
// scalar work per element but doubles the registers per lane).
#ifndef TACO_LPB_32
#define TACO_LPB_32 4
#endif
#ifndef TACO_LPB_64
#define TACO_LPB_64 8
#endif
#ifndef TACO_LPB_128
#define TACO_LPB_128 8
#endif
#ifndef TACO_LPB_256
#define TACO_LPB_256 8
#endif
#ifndef TACO_LPB_512
#define TACO_LPB_512 16
#endif
// Cache policy of the global accesses (1 = non-temporal, "streaming").
// Measured on MI355X with inputs streamed from HBM: the 8-byte code loads
// are 4-7 % faster as ordinary (temporal) loads (a wave reads each 128-byte
// line of codes in two halves, and the second half then hits in L2); the
// 16-byte bf16 and float32 loads and every store are faster non-temporal.
#ifndef TACO_NT_TENSOR_LOADS
#define TACO_NT_TENSOR_LOADS 1
#endif
#ifndef TACO_NT_CODE_LOADS
#define TACO_NT_CODE_LOADS 0
#endif
#ifndef TACO_NT_ACC_LOADS
#define TACO_NT_ACC_LOADS 1
#endif
#ifndef TACO_NT_STORES
#define TACO_NT_STORES 1
#endif
// Block energy from packed bf16 pairs with v_dot2_f32_bf16 (else from
// float32 squares).
#ifndef TACO_DOT2_ENERGY
#define TACO_DOT2_ENERGY 1
#endif
// Wave-steps (BPW blocks each) that one wave processes; the grid is sized
// so that every wave gets this many (the last ones fewer).
#ifndef TACO_STEPS_PER_WAVE
#define TACO_STEPS_PER_WAVE 1
#endif
// Wave-steps per unit: a wave of compress_kernel / decompress_kernel issues
// the loads of P consecutive wave-steps together, then processes them one
// after the other.  With B <= 64 a wave-step moves only 1 KiB of bf16 (512
// bytes of codes), and on large tensors P = 2 is 6-9 % faster (measured at
// 40 and 112 MiB); on small ones the fewer, longer waves lengthen the tail
// (10 % slower at 4 MiB), and at B >= 128 it gains at most 1 %.  So the
// launchers take P = 2 for B <= 64 from kPairMinSteps wave-steps up (twice
// the waves the GPU holds at once), else P = 1.
constexpr int64_t kPairMinSteps = 16384;
template <int B>
constexpr bool pairs_steps() { return B <= 64; }

constexpr int lanes_per_block(int b) {
    return b == 32    ? TACO_LPB_32
           : b == 64  ? TACO_LPB_64
           : b == 128 ? TACO_LPB_128
           : b == 256 ? TACO_LPB_256
                      : TACO_LPB_512;
}

template <int B>
struct Geo {
    static constexpr int LPB = lanes_per_block(B);  // lanes per block
    static constexpr int EPL = B / LPB;            // elements per lane
    static constexpr int CH = EPL / 8;             // 16-byte bf16 chunks per lane
    static constexpr int BPW = kWave / LPB;        // blocks per wave-step
    static constexpr int SPAN = LPB * 8;           // element stride between chunks
    static_assert(B >= 32 && B <= 512 && (B & (B - 1)) == 0, "block size");
    static_assert((LPB == 4 || LPB == 8 || LPB == 16) && EPL >= 8, "lane layout");
};

// Where block k's codes, alpha and s live (Layout):
//  kSide:   codes[k*B .. k*B+B), alpha[k], scale[k] (three buffers).
//  kPacked: one record of B + 8 bytes per block ([TACO] section 4.4.2, the
//           zero-copy metadata layout): the block's codes, then alpha_k and
//           s_k as float32; `alpha` and `scale` point at record 0's
//           scalars, so block k's are alpha[k * kScalarStride].
template <int B, Layout L>
struct Wire {
    static constexpr int64_t kRecord = (L == Layout::kPacked) ? B + 8 : B;     // bytes
    static constexpr int64_t kScalarStride = (L == Layout::kPacked) ? (B + 8) / 4 : 1;  // floats
};

// ---------------------------------------------------------------- lanes ----

template <int LPB>
__device__ __forceinline__ int lane_sub(int lane) {   // t: position inside the block
    return (LPB == 16) ? (lane & 15)
           : (LPB == 8) ? ((lane & 3) | ((lane >> 1) & 4)) : (lane & 3);
}
template <int LPB>
__device__ __forceinline__ int lane_slot(int lane) {  // which block of the wave-step
    return (LPB == 16) ? (lane >> 4)
           : (LPB == 8) ? (((lane >> 2) & 1) | ((lane >> 3) & 6)) : (lane >> 2);
}

// DPP controls (gfx9 encoding) for the three lane-id bits of t.
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppXor8 = 0x128;  // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Lane-id bit 2 (the fourth bit of t when 16 lanes own a block): no single
// gfx9 DPP control swaps lanes i and i ^ 4, so this stage reads the partner
// through ds_swizzle in bit-mask mode (source lane = lane ^ 4 inside each
// 32-lane half; and-mask 0x1f, or-mask 0, xor-mask 4).  Every lane of the
// wave must be active.
constexpr int kSwizzleXor4 = 0x1F | (4 << 10);
__device__ __forceinline__ float swz_xor4(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor4));
}

template <int LPB>
__device__ __forceinline__ float block_sum(float v) {
    // Butterfly order: partners add the same two values, so every lane of
    // the block ends with the same bits.
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    if (LPB == 16) v += swz_xor4(v);
    if (LPB >= 8) v += dpp<kDppXor8>(v);
    return v;
}
// Maximum over the block's lanes of a non-negative float.  Non-negative
// floats order like their bit patterns, so the reduction runs on unsigned
// integers (which need no NaN quieting and fuse with the DPP move).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int LPB>
__device__ __forceinline__ float block_max(float f) {
    uint32_t v = __float_as_uint(f);
    v = max(v, dpp_u<kDppXor1>(v));
    v = max(v, dpp_u<kDppXor2>(v));
    if (LPB == 16) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, kSwizzleXor4));
    if (LPB >= 8) v = max(v, dpp_u<kDppXor8>(v));
    return __uint_as_float(v);
}

// v[i] <- v[i] + sgn * v[i]@partner for 8 registers, partner given by the
// DPP control.  The leading s_nop covers the gfx9 requirement of two wait
// states between a VALU write of a VGPR and a DPP read of it; inside the
// group every register read was written before the group started.
#define TACO_FMAC_DPP8(CTRL, v, o, sgn)                                         \
    asm volatile("s_nop 1\n\t"                                                  \
                 "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"      \
                 : "+v"(v[o + 0]), "+v"(v[o + 1]), "+v"(v[o + 2]), "+v"(v[o + 3]),   \
                   "+v"(v[o + 4]), "+v"(v[o + 5]), "+v"(v[o + 6]), "+v"(v[o + 7])    \
                 : "v"(sgn))

// Unnormalised Walsh-Hadamard transform of the block held by LPB lanes
// (EPL registers each), Sylvester order over e = 8*LPB*k + 8*t + j.  Must
// run with every lane of the wave active.  On return lane t holds
// (-1)^popcount(t) times its outputs.  The stages commute, so any order
// gives H x (float32 rounding aside).
template <int LPB, int EPL>
__device__ __forceinline__ void fwht_block(float (&v)[EPL], float sg1, float sg2, float sg8) {
    constexpr int CH = EPL / 8;
    // Bits of j: h = 1, 2, 4 inside each 8-element chunk.
#pragma unroll
    for (int h = 1; h < 8; h *= 2) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
    // Bits of k: chunk pairs (c, c + hc).
#pragma unroll
    for (int hc = 1; hc < CH; hc *= 2) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if ((c & hc) == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float a = v[8 * c + j], b = v[8 * (c + hc) + j];
                    v[8 * c + j] = a + b;
                    v[8 * (c + hc) + j] = a - b;
                }
            }
        }
    }
    // Bits of t: across lanes.
#pragma unroll
    for (int o = 0; o < EPL; o += 8) TACO_FMAC_DPP8("quad_perm:[1,0,3,2]", v, o, sg1);
#pragma unroll
    for (int o = 0; o < EPL; o += 8) TACO_FMAC_DPP8("quad_perm:[2,3,0,1]", v, o, sg2);
    if (LPB >= 8) {
#pragma unroll
        for (int o = 0; o < EPL; o += 8) TACO_FMAC_DPP8("row_ror:8", v, o, sg8);
    }
    if (LPB == 16) {
        // Lane-id bit 2 through ds_swizzle: v <- v + sgn * v@(lane ^ 4), one
        // rounding as in the DPP stages.
        const float sg4 = (__lane_id() & 4) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[i] = __builtin_fmaf(sg4, swz_xor4(v[i]), v[i]);
    }
}

// Global memory access (each byte is touched once; cache policy above).
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

template <bool NT, typename V>
__device__ __forceinline__ V load_as(const void *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
    else return *reinterpret_cast<const V *>(p);
}
template <bool NT, typename V>
__device__ __forceinline__ void store_as(void *p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
    else *reinterpret_cast<V *>(p) = v;
}
// Inputs: bf16 tensors (16 bytes) and codes (8 bytes).
__device__ __forceinline__ u4v ld16(const void *p) {
    return load_as<TACO_NT_TENSOR_LOADS != 0, u4v>(p);
}
__device__ __forceinline__ u2v ld8(const void *p) {
    return load_as<TACO_NT_CODE_LOADS != 0, u2v>(p);
}
// The float32 accumulator, read once and written back.
__device__ __forceinline__ u4v ld16_acc(const void *p) {
    return load_as<TACO_NT_ACC_LOADS != 0, u4v>(p);
}
__device__ __forceinline__ void st16(void *p, u4v v) { store_as<TACO_NT_STORES != 0>(p, v); }
__device__ __forceinline__ void st8(void *p, u2v v) { store_as<TACO_NT_STORES != 0>(p, v); }

// Sum of squares of packed bf16 pairs accumulated in float32
// (v_dot2_f32_bf16: c + a*a + b*b).  Only the block energy uses it; its
// rounding of the sum need not match a float32 addition, as alpha's
// tolerance (1e-6 relative) is far above the few ulps at stake.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_acc(uint32_t w, float c) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
}

// Empty asm that forces each value to exist in a VGPR at this point of the
// program (it emits no instruction).
template <int N>
__device__ __forceinline__ void pin_values(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const u4v w, float *v) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// Block energy from packed bf16: four accumulator chains of dot2 (so the
// rounding depth is CH + 2 in-lane, plus log2(LPB) across lanes).
template <int CH>
__device__ __forceinline__ float energy_packed(const u4v (&buf)[CH]) {
    float e[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = dot2_acc(buf[k][i], e[i]);
    return (e[0] + e[1]) + (e[2] + e[3]);
}

// Sum of squares of EPL values by a pairwise tree: each x^2 of a bf16 value
// is exact in float32, every partial sum is rounded once, and the depth is
// log2(EPL) (plus log2(LPB) across lanes), which bounds the relative error
// of the block energy by about 9 * 2^-24.
template <int EPL>
__device__ __forceinline__ float sum_squares(const float (&v)[EPL]) {
    float p[EPL / 2];
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) p[i] = fmaf(v[2 * i], v[2 * i], v[2 * i + 1] * v[2 * i + 1]);
#pragma unroll
    for (int w = EPL / 4; w >= 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) p[i] = p[i] + p[i + w];
    }
    return p[0];
}

// max |v| over EPL values with v_max3_f32 and |.| source modifiers, two
// values per instruction.  (fmaxf would first quiet each operand, which
// costs an extra instruction per element; NaN handling is not needed here.)
template <int EPL>
__device__ __forceinline__ float max_abs(const float (&v)[EPL]) {
    static_assert(EPL >= 8 && EPL % 2 == 0, "max_abs layout");
    float m0, m1;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m0) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m1) : "v"(v[3]), "v"(v[4]), "v"(v[5]));
#pragma unroll
    for (int i = 6; i < EPL; i += 2) {
        if ((i / 2) & 1)
            asm("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(m0) : "v"(v[i]), "v"(v[i + 1]));
        else
            asm("v_max3_f32 %0, %0, |%1|, |%2|" : "+v"(m1) : "v"(v[i]), "v"(v[i + 1]));
    }
    asm("v_max_f32 %0, %0, %1" : "+v"(m0) : "v"(m1));
    return m0;
}

// Q / m as an unevaluated sum hi + lo (|lo| <= ulp(hi)): the hardware
// reciprocal refined by one Newton step gives hi, and the exact residual
// Q - m hi (one fma) divided by m gives lo.  m must be a positive normal.
struct Quot { float hi, lo; };
__device__ __forceinline__ Quot quotient(float q, float m) {
    const float rc = __builtin_amdgcn_rcpf(m);
    const float q0 = q * rc;
    const float hi = fmaf(fmaf(-m, q0, q), rc, q0);
    const float lo = fmaf(-m, hi, q) * rc;
    return {hi, lo};
}

// Code formats: Q_max of Eq. 9 and the conversions of Eq. 10 (pack8: the
// codes of 8 float32 values) and Eq. 11 (decode8: the values of 8 codes).
// Codes are little-endian, element j in byte j.  encode8 gives the codes of
// v * Q / m for 8 values, given Q / m as hi + lo: the argument of the
// conversion is v * (hi + lo) with a single final rounding, i.e. float32 of
// v * Q / m almost always correctly rounded; the +0 addend of the inner fma
// maps an exact zero of either sign to +0.  In pack8 each word takes two
// conversions: the second overwrites the half the first one keeps, so the
// first is seeded with any register (its own argument) rather than zero.
template <Fmt F>
struct Codec;

template <Fmt F>
__device__ __forceinline__ u2v encode8(const float *v, Quot r) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = fmaf(v[j], r.hi, fmaf(v[j], r.lo, 0.0f));
    return Codec<F>::pack8(q);
}

// OCP E4M3 ("E4M3FN"), the operator's format ([TACO] section 4.3).
template <>
struct Codec<Fmt::kE4M3> {
    static constexpr float kQmax = TACO_QMAX;
    static __device__ __forceinline__ u2v pack8(const float *q) {
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __float_as_int(q[0]), false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], __float_as_int(q[4]), false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
        return (u2v){(uint32_t)lo, (uint32_t)hi};
    }
    static __device__ __forceinline__ void decode8(const u2v c, float *v) {
        f2v a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
        f2v b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
        f2v d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
        f2v e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
        v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
        v[4] = d.x; v[5] = d.y; v[6] = e.x; v[7] = e.y;
    }
};

// OCP E5M2 ([TACO] section 5.3.2 format ablation; section 2.3 / Figure 3).
template <>
struct Codec<Fmt::kE5M2> {
    static constexpr float kQmax = TACO_E5M2_MAX;
    static __device__ __forceinline__ u2v pack8(const float *q) {
        int lo = __builtin_amdgcn_cvt_pk_bf8_f32(q[0], q[1], __float_as_int(q[0]), false);
        lo = __builtin_amdgcn_cvt_pk_bf8_f32(q[2], q[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_bf8_f32(q[4], q[5], __float_as_int(q[4]), false);
        hi = __builtin_amdgcn_cvt_pk_bf8_f32(q[6], q[7], hi, true);
        return (u2v){(uint32_t)lo, (uint32_t)hi};
    }
    static __device__ __forceinline__ void decode8(const u2v c, float *v) {
        f2v a = __builtin_amdgcn_cvt_pk_f32_bf8((int)c.x, false);
        f2v b = __builtin_amdgcn_cvt_pk_f32_bf8((int)c.x, true);
        f2v d = __builtin_amdgcn_cvt_pk_f32_bf8((int)c.y, false);
        f2v e = __builtin_amdgcn_cvt_pk_f32_bf8((int)c.y, true);
        v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
        v[4] = d.x; v[5] = d.y; v[6] = e.x; v[7] = e.y;
    }
};

// Symmetric INT8 with the dual scale as its step ([TACO] section 6 fallback;
// quantiser of section 2.3 / Eq. 1): q = round(Z / s) in [-127, 127] as a
// two's complement byte.  For |q| < 2^22, float32 q + 1.5 * 2^23 rounds q to
// the nearest integer, ties to even, in one addition, and the low byte of
// the sum's bit pattern is that integer's two's complement byte.  Arguments
// never exceed 127 in magnitude (Z / s <= Q_max), so no clamp is needed.
template <>
struct Codec<Fmt::kInt8> {
    static constexpr float kQmax = TACO_INT8_MAX;
    static __device__ __forceinline__ u2v pack8(const float *q) {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = __float_as_uint(q[j] + 0x1.8p23f);
        // v_perm_b32 byte selectors: 0-3 pick bytes of the second operand,
        // 4-7 bytes of the first, 0x0c gives a zero byte.
        const uint32_t lo = __builtin_amdgcn_perm(w[1], w[0], 0x0c0c0400u) |
                            __builtin_amdgcn_perm(w[3], w[2], 0x04000c0cu);
        const uint32_t hi = __builtin_amdgcn_perm(w[5], w[4], 0x0c0c0400u) |
                            __builtin_amdgcn_perm(w[7], w[6], 0x04000c0cu);
        return (u2v){lo, hi};
    }
    static __device__ __forceinline__ void decode8(const u2v c, float *v) {
        // (the bit-field extract builtin returns its sign-extended field as
        // an unsigned value: convert it as a signed one)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = (float)(int32_t)__builtin_amdgcn_sbfe(c.x, 8 * j, 8);
            v[4 + j] = (float)(int32_t)__builtin_amdgcn_sbfe(c.y, 8 * j, 8);
        }
    }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf2v r = __builtin_convertvector((f2v){a, b}, bf2v);   // round to nearest even
    return __builtin_bit_cast(uint32_t, r);
}

// 1 / sqrt(B) for the supported block sizes (double literals, rounded once
// to float where used).
constexpr double inv_sqrt(int b) {
    return b == 32    ? 0.17677669529663688110
           : b == 64  ? 0.125
           : b == 128 ? 0.08838834764831844055
           : b == 256 ? 0.0625
                      : 0.04419417382415922028;
}

// Blocks whose energy reaches this are rescaled by 2^-80 before squaring so
// that sum x^2 stays finite for every bf16 input: sum (x 2^-80)^2 <=
// 512 (2^128 2^-80)^2 = 2^105.  (kBigMax: the same for a block maximum,
// before a plain rotation.)
constexpr float kBigEnergy = 0x1p100f;
constexpr float kBigMax = 0x1p100f;
constexpr float kBigShift = 0x1p-80f;
constexpr float kBigShiftInv = 0x1p80f;
constexpr float kBigUnshift = 0x1p-80f;   // alpha of the original block = alpha' * 2^-80
// Blocks with max|R| below this get R and max|R| scaled by 2^64 before
// Q / max|R| is formed, so that the quotient cannot overflow.
constexpr float kTinyMax = 0x1p-96f;
constexpr float kTinyShift = 0x1p64f;
// Output factors below this are applied in two steps (see decompress).
constexpr float kTinyOut = 0x1p-100f;
constexpr float kOutShift = 0x1p64f;
constexpr float kOutUnshift = 0x1p-64f;

// ------------------------------------------------- staged code traffic ----

// A lane's codes of a block are 8-byte runs 8 * LPB bytes apart, so direct
// 8-byte stores or loads move 512 bytes per instruction in 64-byte pieces.
// Staged through a wave-private LDS region (the wave-step's BPW * B code
// bytes in element order), every instruction moves 1 KiB of contiguous
// codes.  Measured: compress 1-3 % faster from 112 MiB up, even at 40 MiB,
// 0.06 us slower on a 4 MiB tensor; the owner step 1-2 % faster; decompress
// 2-3 % faster for B >= 256 and slower for B = 128, so the receive side
// stages only from B = 256 up.  Side-buffer layout only.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store the wave-step's codes c (lane's runs) to cb, the step's first code
// byte; only the first nvalid bytes (whole blocks) are written.
template <int B>
__device__ __forceinline__ void codes_store_staged(uint8_t *stg, uint8_t *__restrict__ cb,
                                                   int nvalid, const u2v (&c)[Geo<B>::CH],
                                                   int g, int t, int lane) {
    using G = Geo<B>;
    wave_lds_sync();                   // earlier readers of the stage are done
#pragma unroll
    for (int k = 0; k < G::CH; ++k)
        *reinterpret_cast<u2v *>(stg + g * B + k * G::SPAN + 8 * t) = c[k];
    wave_lds_sync();
#pragma unroll
    for (int i0 = 0; i0 < G::BPW * B; i0 += 16 * kWave) {
        const int i = i0 + 16 * lane;
        if (i < nvalid) st16(cb + i, *reinterpret_cast<const u4v *>(stg + i));
    }
}

// The interleaved layout's records of one wave-step (BPW * (B + 8) bytes,
// a multiple of 64) assembled in LDS from the lanes' code runs and each
// block's alpha and s (written by lane t = 0), then stored 16 bytes per lane
// (first nvalid bytes only): direct 8-byte stores of B + 8-byte records
// straddle lines (measured: the owner step ~15 % slower than on side
// buffers).  rb is the step's first record.
template <int B>
__device__ __forceinline__ void records_store_staged(uint8_t *stg, uint8_t *__restrict__ rb,
                                                     int nvalid, const u2v (&c)[Geo<B>::CH],
                                                     float a, float s, int g, int t, int lane) {
    using G = Geo<B>;
    constexpr int kRec = B + 8;
    wave_lds_sync();
    uint8_t *rec = stg + g * kRec;
#pragma unroll
    for (int k = 0; k < G::CH; ++k) *reinterpret_cast<u2v *>(rec + k * G::SPAN + 8 * t) = c[k];
    if (t == 0) {
        *reinterpret_cast<float *>(rec + B) = a;
        *reinterpret_cast<float *>(rec + B + 4) = s;
    }
    wave_lds_sync();
    // nvalid is a multiple of 8 (whole records) but not always of 16: the
    // last piece may be an 8-byte one.
#pragma unroll
    for (int i0 = 0; i0 < G::BPW * kRec; i0 += 16 * kWave) {
        const int i = i0 + 16 * lane;
        if (i + 16 <= nvalid)
            st16(rb + i, *reinterpret_cast<const u4v *>(stg + i));
        else if (i < nvalid)
            st8(rb + i, *reinterpret_cast<const u2v *>(stg + i));
    }
}

// The receive side in two halves: issue the contiguous loads (bytes past
// nvalid read as zero), and later hand each lane its runs through LDS.
template <int B>
struct CodesLoad {
    static constexpr int kBytes = Geo<B>::BPW * B;
    static constexpr int kPieces = (kBytes + 16 * kWave - 1) / (16 * kWave);
};
template <int B>
__device__ __forceinline__ void codes_load_issue(const uint8_t *__restrict__ cb, int nvalid,
                                                 u4v (&raw)[CodesLoad<B>::kPieces], int lane) {
#pragma unroll
    for (int c = 0; c < CodesLoad<B>::kPieces; ++c) {
        const int i = c * 16 * kWave + 16 * lane;
        raw[c] = (i < nvalid) ? ld16(cb + i) : (u4v){0u, 0u, 0u, 0u};
    }
}
template <int B>
__device__ __forceinline__ void codes_load_finish(uint8_t *stg,
                                                  const u4v (&raw)[CodesLoad<B>::kPieces],
                                                  u2v (&c)[Geo<B>::CH], int g, int t, int lane) {
    using G = Geo<B>;
    wave_lds_sync();
#pragma unroll
    for (int p = 0; p < CodesLoad<B>::kPieces; ++p) {
        const int i = p * 16 * kWave + 16 * lane;
        if (i < CodesLoad<B>::kBytes) *reinterpret_cast<u4v *>(stg + i) = raw[p];
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < G::CH; ++k)
        c[k] = *reinterpret_cast<const u2v *>(stg + g * B + k * G::SPAN + 8 * t);
}

// ----------------------------------------------------------- compress -----

// Side buffers: codes[N], alpha[M], scale[M].  (The interleaved layout has
// its own kernel, compress_packed_kernel, below.)  A wave works on units of
// P consecutive wave-steps (see kPairMinSteps): the unit's loads are issued
// together, then its wave-steps are processed one after the other.
template <int B, Fmt F, int P>
__global__ __launch_bounds__(kGroup) void compress_kernel(
    const uint16_t *__restrict__ x, int64_t nblocks, float tau,
    uint8_t *__restrict__ codes, float *__restrict__ alpha, float *__restrict__ scale) {
    using G = Geo<B>;
    static_assert(P == 1 || (P == 2 && pairs_steps<B>()), "wave-steps per unit");
    // The unit's codes leave through this wave's LDS region.
    __shared__ __align__(16) uint8_t stage_all[kWavesPerGroup][P * G::BPW * B];
    uint8_t *stage = stage_all[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
    const int lane = threadIdx.x & (kWave - 1);
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    using C = Codec<F>;
    // 1 / (sqrt(B) * Q_max), rounded once.
    constexpr float kScaleFactor = (float)(inv_sqrt(B) / (double)C::kQmax);
    constexpr float kInvB = 1.0f / (float)B;

    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t nunits = (nsteps + P - 1) / P;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerGroup +
                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    // Every address is a wave-uniform base (the wave-step's first block)
    // plus a 32-bit byte offset of the lane, so the memory instructions take
    // the base in scalar registers and the offset in one vector register.
    const char *const xb = reinterpret_cast<const char *>(x);
    const uint32_t lane_scalar = (uint32_t)(g * 4);
    constexpr int64_t kStepX = G::BPW * B * 2;                        // bytes of x
    constexpr int64_t kStepCodes = G::BPW * B;
    constexpr int64_t kStepScalars = G::BPW * 4;

    // Index of the last block slot of a wave-step that holds a block (BPW - 1
    // except in the final wave-step).  Slots past it re-read that block, so
    // every load is in bounds and no lane needs zero-filling; their results
    // are never stored.
    auto last_slot = [&](int64_t step) -> int {
        const int64_t left = nblocks - step * G::BPW;          // wave-uniform
        return (int)(left < G::BPW ? left : G::BPW) - 1;
    };
    auto lane_offset = [&](int last) -> uint32_t {
        const int gl = g < last ? g : last;
        return (uint32_t)(gl * (2 * B) + 16 * t);
    };
    u4v buf[P][G::CH];
    // A unit's wave-steps past the last one re-read the last wave-step (in
    // bounds; nothing of theirs is stored).
    auto load = [&](int64_t unit) {
#pragma unroll
        for (int h = 0; h < P; ++h) {
            int64_t step = unit * P + h;
            step = step < nsteps ? step : nsteps - 1;
            const char *p = xb + step * kStepX + lane_offset(last_slot(step));
#pragma unroll
            for (int k = 0; k < G::CH; ++k) buf[h][k] = ld16(p + k * G::SPAN * 2);
        }
    };

    if (wave0 < nunits) load(wave0);
    for (int64_t unit = wave0; unit < nunits; unit += nwaves) {
        float v[P][G::EPL];
        float energy[P];
#pragma unroll
        for (int h = 0; h < P; ++h) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) unpack8(buf[h][k], &v[h][8 * k]);
            // [TACO] Eq. 6: block energy (raw second moment), this lane's part.
#if TACO_DOT2_ENERGY
            energy[h] = energy_packed<G::CH>(buf[h]);
#else
            energy[h] = sum_squares<G::EPL>(v[h]);
#endif
            // Materialise these values here, so that the prefetch below can
            // reuse buf's registers instead of copying them.
            pin_values(v[h]);
            asm volatile("" : "+v"(energy[h]));
        }
        if (unit + nwaves < nunits) load(unit + nwaves);

#pragma unroll
        for (int h = 0; h < P; ++h) {
            const int64_t step = unit * P + h;
            if (step >= nsteps) break;                               // wave-uniform
            const int last = last_slot(step);
            const bool active = g <= last;

            float e = block_sum<G::LPB>(energy[h]);
            float unshift = 1.0f;
            if (__builtin_expect(e >= kBigEnergy, 0)) {
                // Huge block (sum x^2 near or past float32 range): reload it and
                // work on x * 2^-80 (exact), undoing the factor in alpha.
                const char *p = xb + step * kStepX + lane_offset(last);
#pragma unroll
                for (int k = 0; k < G::CH; ++k) unpack8(ld16(p + k * G::SPAN * 2), &v[h][8 * k]);
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[h][i] *= kBigShift;
                e = block_sum<G::LPB>(sum_squares<G::EPL>(v[h]));
                unshift = kBigUnshift;
            }
            // [TACO] Eq. 6-7: alpha = tau / sqrt(mean(x^2) + eps).
            const float a = tau * __builtin_amdgcn_rsqf(e * kInvB + TACO_EPS);

            // [TACO] Eq. 8 without its constant factors: R = H x.
            fwht_block<G::LPB, G::EPL>(v[h], sg1, sg2, sg8);

            // [TACO] Eq. 9: max|Z| = alpha max|R| / sqrt(B).
            float m = block_max<G::LPB>(max_abs<G::EPL>(v[h]));
            const float s = a * m * kScaleFactor;
            if (__builtin_expect(m < kTinyMax && m > 0.0f, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[h][i] *= kTinyShift;
                m *= kTinyShift;
            }
            // [TACO] Eq. 10: Z / s = Q * R / max|R|.
            Quot r = quotient(C::kQmax, m);
            r.hi = (m > 0.0f) ? r.hi * lane_sign : 0.0f;
            r.lo = (m > 0.0f) ? r.lo * lane_sign : 0.0f;

            u2v c[G::CH];
#pragma unroll
            for (int k = 0; k < G::CH; ++k) c[k] = encode8<F>(&v[h][8 * k], r);
            codes_store_staged<B>(stage + h * kStepCodes, codes + step * kStepCodes,
                                  (last + 1) * B, c, g, t, lane);
            if (active && t == 0) {
                const int64_t sb = step * kStepScalars;
                *reinterpret_cast<float *>(reinterpret_cast<char *>(alpha) + sb + lane_scalar) =
                    a * unshift;
                *reinterpret_cast<float *>(reinterpret_cast<char *>(scale) + sb + lane_scalar) = s;
            }
        }
    }
}

// Compress into the interleaved layout, staged through LDS.  A record is
// B + 8 bytes, so a wave-step's 8 records are not a whole number of 128-byte
// lines and its code stores would straddle lines.  Here each wave assembles
// R = 16 consecutive records (16 (B + 8) bytes: always a multiple of 128,
// since B / 8 + 1 is odd) in its own LDS region and writes them with
// 16-byte stores, each store instruction covering whole lines.  The
// arithmetic is compress_kernel's, step for step.
template <int B, Fmt F>
__global__ __launch_bounds__(kGroup) void compress_packed_kernel(
    const uint16_t *__restrict__ x, int64_t nblocks, float tau, uint8_t *__restrict__ payload) {
    using G = Geo<B>;
    using C = Codec<F>;
    constexpr int kRec = B + 8;                 // bytes per record
    constexpr int R = 16;                       // records per unit
    constexpr int S = R / G::BPW;               // wave-steps per unit (1, 2 or 4)
    constexpr int kUnit = R * kRec;             // bytes per unit
    static_assert(kUnit % 128 == 0 && R % G::BPW == 0, "unit layout");
    __shared__ __align__(16) uint8_t stage_all[kWavesPerGroup][kUnit];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    constexpr float kScaleFactor = (float)(inv_sqrt(B) / (double)C::kQmax);
    constexpr float kInvB = 1.0f / (float)B;
    uint8_t *stage = stage_all[wave];

    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t nunits = (nblocks + R - 1) / R;
    const int64_t unit0 = (int64_t)blockIdx.x * kWavesPerGroup + wave;
    const int64_t nunits_grid = (int64_t)gridDim.x * kWavesPerGroup;

    // As in compress_kernel: slots past the last block re-read it.
    auto lane_offset = [&](int64_t step) -> uint32_t {
        const int64_t left = nblocks - step * G::BPW;
        const int gl = (left >= G::BPW || g < left) ? g : (int)left - 1;
        return (uint32_t)(gl * B + 8 * t);
    };
    u4v buf[G::CH];
    auto load = [&](int64_t step) {
        const uint16_t *p = x + step * (G::BPW * B) + lane_offset(step);
#pragma unroll
        for (int k = 0; k < G::CH; ++k) buf[k] = ld16(p + k * G::SPAN);
    };

    for (int64_t unit = unit0; unit < nunits; unit += nunits_grid) {
        const int64_t step0 = unit * S;
        load(step0);
#pragma unroll
        for (int h = 0; h < S; ++h) {
            const int64_t step = step0 + h;
            if (step >= nsteps) break;                       // wave-uniform
            float v[G::EPL];
#pragma unroll
            for (int k = 0; k < G::CH; ++k) unpack8(buf[k], &v[8 * k]);
#if TACO_DOT2_ENERGY
            float energy = energy_packed<G::CH>(buf);
#else
            float energy = sum_squares<G::EPL>(v);
#endif
            pin_values(v);
            asm volatile("" : "+v"(energy));
            if (h + 1 < S && step + 1 < nsteps) load(step + 1);

            const int64_t blk = step * G::BPW + g;
            energy = block_sum<G::LPB>(energy);
            float unshift = 1.0f;
            if (__builtin_expect(energy >= kBigEnergy, 0)) {
                const uint16_t *p = x + step * (G::BPW * B) + lane_offset(step);
#pragma unroll
                for (int k = 0; k < G::CH; ++k) unpack8(ld16(p + k * G::SPAN), &v[8 * k]);
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kBigShift;
                energy = block_sum<G::LPB>(sum_squares<G::EPL>(v));
                unshift = kBigUnshift;
            }
            const float a = tau * __builtin_amdgcn_rsqf(energy * kInvB + TACO_EPS);
            fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
            float m = block_max<G::LPB>(max_abs<G::EPL>(v));
            const float s = a * m * kScaleFactor;
            if (__builtin_expect(m < kTinyMax && m > 0.0f, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kTinyShift;
                m *= kTinyShift;
            }
            Quot r = quotient(C::kQmax, m);
            r.hi = (m > 0.0f) ? r.hi * lane_sign : 0.0f;
            r.lo = (m > 0.0f) ? r.lo * lane_sign : 0.0f;

            if (blk < nblocks) {
                uint8_t *rec = stage + (h * G::BPW + g) * kRec;
#pragma unroll
                for (int k = 0; k < G::CH; ++k)
                    *reinterpret_cast<u2v *>(rec + 8 * t + k * G::SPAN) = encode8<F>(&v[8 * k], r);
                if (t == 0) {
                    const f2v as = {a * unshift, s};
                    *reinterpret_cast<f2v *>(rec + B) = as;
                }
            }
        }
        // The unit's records are in LDS: write its valid bytes out.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t left = nblocks - unit * R;
        const int bytes = (int)(left < R ? left : R) * kRec;      // a multiple of 8
        uint8_t *dst = payload + unit * kUnit;
        for (int off = 16 * lane; off < bytes; off += 16 * kWave) {
            if (off + 16 <= bytes)
                st16(dst + off, *reinterpret_cast<const u4v *>(stage + off));
            else
                st8(dst + off, *reinterpret_cast<const u2v *>(stage + off));
        }
        // Every lane has read its part of the stage before it is rewritten.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ------------------------------------------------ float32 accumulator -----

// The accumulator update acc += G' of one wave-step, staged through LDS.  A
// lane holds its block's values as runs of 8 elements, 8 * LPB elements
// apart, so direct 16-byte read-modify-writes would cover only half of
// every 32-byte sector per instruction (measured: ~5 % more HBM writes and
// ~3 % more reads than the accumulator's bytes).  Instead the wave writes
// its G' to a wave-private LDS region in element order, then updates the
// accumulator in contiguous 16-byte pieces, 1 KiB per instruction.  A pass
// stages at most 2048 floats (8 KiB per wave), so B = 512 takes two passes.
template <int B>
struct AccStage {
    static constexpr int kBpw = Geo<B>::BPW;
    static constexpr int kBlocks = (kBpw * B <= 2048) ? kBpw : 2048 / B;  // blocks per pass
    static constexpr int kElems = kBlocks * B;                             // floats per wave
    static constexpr int kPasses = kBpw / kBlocks;
    static_assert(kPasses * kBlocks == kBpw && kElems % (4 * kWave) == 0, "stage layout");
};

// acc[step's elements] += v (the lane's G' values, final float32 products);
// slots past the last block (g beyond it) are not written.  stg: this
// wave's AccStage<B>::kElems floats of LDS.
template <int B>
__device__ __forceinline__ void acc_update_staged(float *stg, float *__restrict__ acc,
                                                  int64_t step, int64_t nblocks,
                                                  const float (&v)[Geo<B>::EPL], int g, int t,
                                                  int lane) {
    using G = Geo<B>;
    using S = AccStage<B>;
    const int64_t left = nblocks - step * G::BPW;                       // wave-uniform
    const int nvalid = (int)(left < G::BPW ? left : G::BPW) * B;        // elements
    float *ab = acc + step * (int64_t)(G::BPW * B);
#pragma unroll
    for (int pass = 0; pass < S::kPasses; ++pass) {
        // Every lane has read the previous contents before they are rewritten.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int gl = g - pass * S::kBlocks;
        if (S::kPasses == 1 || (gl >= 0 && gl < S::kBlocks)) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) {
                float *sp = stg + gl * B + k * G::SPAN + 8 * t;
                const float *w = &v[8 * k];
                *reinterpret_cast<u4v *>(sp) = (u4v){__float_as_uint(w[0]), __float_as_uint(w[1]),
                                                     __float_as_uint(w[2]), __float_as_uint(w[3])};
                *reinterpret_cast<u4v *>(sp + 4) =
                    (u4v){__float_as_uint(w[4]), __float_as_uint(w[5]), __float_as_uint(w[6]),
                          __float_as_uint(w[7])};
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int base = pass * S::kElems;
#pragma unroll
        for (int i0 = 0; i0 < S::kElems; i0 += 4 * kWave) {
            const int i = i0 + 4 * lane;
            if (base + i < nvalid) {
                float *pa = ab + base + i;
                const u4v p = ld16_acc(pa);
                const u4v q = *reinterpret_cast<const u4v *>(stg + i);
                u4v o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = __float_as_uint(__uint_as_float(p[j]) + __uint_as_float(q[j]));
                st16(pa, o);
            }
        }
    }
}

// --------------------------------------------------------- decompress -----

template <int B, Fmt F, Out MODE, Layout L, int P>
__global__ __launch_bounds__(kGroup) void decompress_kernel(
    const uint8_t *__restrict__ codes, const float *__restrict__ alpha,
    const float *__restrict__ scale, int64_t nblocks, uint16_t *__restrict__ y,
    float *__restrict__ acc) {
    using G = Geo<B>;
    using W = Wire<B, L>;
    constexpr bool kAcc = MODE == Out::kAccumulate;
    constexpr bool kCodes = L == Layout::kSide && B >= 256;   // staged code loads
    static_assert(P == 1 || (P == 2 && pairs_steps<B>() && !kCodes), "wave-steps per unit");
    // One LDS region per wave serves both stages (codes first, then G').
    constexpr int kAccBytes = kAcc ? AccStage<B>::kElems * 4 : 0;
    constexpr int kCodeBytes = kCodes ? CodesLoad<B>::kBytes : 0;
    constexpr int kStageBytes = kAccBytes > kCodeBytes ? kAccBytes : kCodeBytes;
    constexpr bool kAny = kStageBytes > 0;
    __shared__ __align__(16) uint8_t stage_all[kAny ? kWavesPerGroup : 1][kAny ? kStageBytes : 16];
    uint8_t *stage_b = stage_all[kAny ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0];
    float *stage = reinterpret_cast<float *>(stage_b);
    const int lane = threadIdx.x & (kWave - 1);
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    using C = Codec<F>;
    // 1 / sqrt(B), rounded once.
    constexpr float kInvSqrtB = (float)inv_sqrt(B);

    // Units of P consecutive wave-steps (see kPairMinSteps).
    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t nunits = (nsteps + P - 1) / P;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;

    // Slots past the last block (and wave-steps past the last one) re-read
    // the last block; nothing of theirs is stored.  (With staged code loads
    // those slots decode zeros.)
    u2v buf[P][G::CH];
    u4v raw[kCodes ? CodesLoad<B>::kPieces : 1];
    float a_buf[P], s_buf[P];
    auto load = [&](int64_t unit) {
#pragma unroll
        for (int h = 0; h < P; ++h) {
            const int64_t step = unit * P + h;
            int64_t blk = step * G::BPW + g;
            blk = blk < nblocks ? blk : nblocks - 1;
            if constexpr (kCodes) {
                const int64_t left = nblocks - step * G::BPW;
                codes_load_issue<B>(codes + step * (int64_t)(G::BPW * B),
                                    (int)(left < G::BPW ? left : G::BPW) * B, raw, lane);
            } else {
                const uint8_t *p = codes + blk * W::kRecord + 8 * t;
#pragma unroll
                for (int k = 0; k < G::CH; ++k) buf[h][k] = ld8(p + k * G::SPAN);
            }
            a_buf[h] = alpha[blk * W::kScalarStride];
            s_buf[h] = scale[blk * W::kScalarStride];
        }
    };

    if (wave0 < nunits) load(wave0);
    for (int64_t unit = wave0; unit < nunits; unit += nwaves) {
        if constexpr (kCodes) codes_load_finish<B>(stage_b, raw, buf[0], g, t, lane);
        float v[P][G::EPL];
        float a[P], s[P];
#pragma unroll
        for (int h = 0; h < P; ++h) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) C::decode8(buf[h][k], &v[h][8 * k]);   // Eq. 11 (before * s)
            a[h] = a_buf[h];
            s[h] = s_buf[h];
            pin_values(v[h]);
            asm volatile("" : "+v"(a[h]), "+v"(s[h]));
        }
        if (unit + nwaves < nunits) load(unit + nwaves);

#pragma unroll
        for (int h = 0; h < P; ++h) {
            const int64_t step = unit * P + h;
            if (step >= nsteps) break;                               // wave-uniform
            const int64_t blk = step * G::BPW + g;
            const bool active = blk < nblocks;

            fwht_block<G::LPB, G::EPL>(v[h], sg1, sg2, sg8);          // Eq. 12 (unnormalised)
            // Eq. 11-13 constant factors: s / sqrt(B) / alpha, with the lane sign.
            const float f = ((s[h] * kInvSqrtB) / a[h]) * lane_sign;
            if (__builtin_expect(s[h] > 0.0f && fabsf(f) < kTinyOut, 0)) {
                // The factor would lose bits as a float32 subnormal: apply it as
                // (2^64 f) then 2^-64, so that only the final product rounds.
                const float fs = (((s[h] * kOutShift) * kInvSqrtB) / a[h]) * lane_sign;
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[h][i] = (v[h][i] * fs) * kOutUnshift;
            } else {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[h][i] *= f;
            }

            if constexpr (kAcc) {
                acc_update_staged<B>(stage, acc, step, nblocks, v[h], g, t, lane);
            } else if (active) {
                const int64_t e0 = blk * B + 8 * t;
#pragma unroll
                for (int k = 0; k < G::CH; ++k) {
                    const float *w = &v[h][8 * k];
                    const u4v o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                   pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
                    st16(y + e0 + k * G::SPAN, o);
                }
            }
        }
    }
}

// ------------------------------------------------------ owner step -------

// Owner step of the two-shot all-reduce ([TACO] section 4.4.2): compress
// X = own + sum_p G'_p without materialising X.  With H H = B I,
// H G'_p = sqrt(B) (s_p / alpha_p) decode(q_p), so
//     H X = H own + sum_p sqrt(B) (s_p / alpha_p) decode(q_p):
// one transform (of own) plus one multiply-add per payload element, all in
// the rotated domain.  The block energy follows from Parseval,
// sum X^2 = sum (H X)^2 / B, and Eq. 6-10 proceed as in compress_kernel.
template <int B, Fmt F, int P, Layout L>
__global__ __launch_bounds__(kGroup) void reduce_compress_kernel(
    const uint16_t *__restrict__ own, Payloads pay, int64_t nblocks, float tau,
    uint8_t *__restrict__ codes, float *__restrict__ alpha, float *__restrict__ scale) {
    using G = Geo<B>;
    using W = Wire<B, L>;
    // Codes (side buffers) or whole records (interleaved) leave through LDS.
    __shared__ __align__(16) uint8_t stage_all[kWavesPerGroup][G::BPW * W::kRecord];
    uint8_t *stage = stage_all[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
    const int lane = threadIdx.x & (kWave - 1);
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    using C = Codec<F>;
    constexpr float kScaleFactor = (float)(inv_sqrt(B) / (double)C::kQmax);
    // sqrt(B) = kSqrtBHi + kSqrtBLo to about 2^-48.
    constexpr float kSqrtBHi = (float)(1.0 / inv_sqrt(B));
    constexpr float kSqrtBLo = (float)(1.0 / inv_sqrt(B) - (double)kSqrtBHi);
    // mean(X^2) = sum over the block of (H X)^2 / B^2.
    constexpr float kInvB2 = 1.0f / ((float)B * (float)B);
    const bool has_own = own != nullptr;

    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerGroup +
                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const uint32_t lane_elem = (uint32_t)(g * B + 8 * t);

    for (int64_t step = wave0; step < nsteps; step += nwaves) {
        // Slots past the last block re-read the last block and store nothing.
        const int64_t left = nblocks - step * G::BPW;
        const uint32_t off = left >= G::BPW ? lane_elem
                                            : (uint32_t)((g < left ? g : (int)left - 1) * B + 8 * t);
        const int64_t base = step * (G::BPW * B);
        const int64_t lblk = (base + off) / B;
        const uint32_t coff = (uint32_t)(lblk - step * G::BPW) * (uint32_t)W::kRecord + 8 * t;
        const int64_t cbase = step * G::BPW * W::kRecord;

        // Loads: own (bf16) and every payload's codes and scalars.
        u4v xo[G::CH];
        if (has_own) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) xo[k] = ld16(own + base + off + k * G::SPAN);
        }
        u2v qc[P > 0 ? P : 1][G::CH];
        float wa[P > 0 ? P : 1], ws[P > 0 ? P : 1];
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) qc[p][k] = ld8(pay.codes[p] + cbase + coff + k * G::SPAN);
            wa[p] = pay.alpha[p][lblk * W::kScalarStride];
            ws[p] = pay.scale[p][lblk * W::kScalarStride];
        }

        float v[G::EPL];
        if (has_own) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) unpack8(xo[k], &v[8 * k]);
            fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);          // H own (lane-signed)
        } else {
#pragma unroll
            for (int i = 0; i < G::EPL; ++i) v[i] = 0.0f;
        }
        // v += sum_p c_p decode(q_p), c_p = sqrt(B) s_p / alpha_p times
        // `shift` (with the lane sign of the stored layout) as hi + lo,
        // added high part first: each fma then rounds relative to the
        // running sum, so a payload that nearly cancels own keeps the
        // precision of the result.
        auto add_payloads = [&](const u2v (&qp)[P > 0 ? P : 1][G::CH], float shift) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                // (shift s_p) / alpha_p: the shift is applied before the
                // division, so that the quotient is not a float32 subnormal
                // for tiny blocks; a subnormal alpha would overflow the
                // reciprocal, so it takes a plain division.
                Quot sa = {0.0f, 0.0f};
                const float sp = ws[p] * shift;
                if (ws[p] > 0.0f)
                    sa = wa[p] >= 0x1p-120f ? quotient(sp, wa[p]) : Quot{sp / wa[p], 0.0f};
                const float ch = kSqrtBHi * sa.hi;
                const float cl = fmaf(kSqrtBHi, sa.hi, -ch) +
                                 fmaf(kSqrtBHi, sa.lo, kSqrtBLo * sa.hi);
                const float chs = ch * lane_sign, cls = cl * lane_sign;
                float d[G::EPL];
#pragma unroll
                for (int k = 0; k < G::CH; ++k) C::decode8(qp[p][k], &d[8 * k]);
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] = fmaf(d[i], cls, fmaf(d[i], chs, v[i]));
            }
        };
        auto energy_of_v = [&]() {
            float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
            for (int i = 0; i < G::EPL; i += 2) {
                e0 = fmaf(v[i], v[i], e0);
                e1 = fmaf(v[i + 1], v[i + 1], e1);
            }
            return block_sum<G::LPB>(e0 + e1);
        };
        add_payloads(qc, 1.0f);

        // Eq. 6 via Parseval.
        float energy = energy_of_v();
        float unshift = 1.0f;
        if (__builtin_expect(!(energy < kBigEnergy), 0)) {
            // Huge block (its energy, or H X itself, may have left float32
            // range): rebuild H X from the inputs scaled by 2^-80 (exact),
            // undoing the factor in alpha.
            if (has_own) {
#pragma unroll
                for (int k = 0; k < G::CH; ++k)
                    unpack8(ld16(own + base + off + k * G::SPAN), &v[8 * k]);
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kBigShift;
                fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
            } else {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] = 0.0f;
            }
            u2v qr[P > 0 ? P : 1][G::CH];
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int k = 0; k < G::CH; ++k) qr[p][k] = ld8(pay.codes[p] + cbase + coff + k * G::SPAN);
            add_payloads(qr, kBigShift);
            energy = energy_of_v();
            unshift = kBigUnshift;
        }
        // Eq. 7.
        const float a = tau * __builtin_amdgcn_rsqf(energy * kInvB2 + TACO_EPS);
        // Eq. 9-10 as in compress_kernel.
        float m = block_max<G::LPB>(max_abs<G::EPL>(v));
        float s = a * m * kScaleFactor;
        if (__builtin_expect(m < kTinyMax && m > 0.0f, 0)) {
            // Tiny block: its rotated values (and payload factors) are
            // float32 subnormals, with too few bits for the codes.  Rebuild
            // H X from the inputs scaled by 2^64 (exact).
            if (has_own) {
#pragma unroll
                for (int k = 0; k < G::CH; ++k)
                    unpack8(ld16(own + base + off + k * G::SPAN), &v[8 * k]);
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kTinyShift;
                fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
            } else {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] = 0.0f;
            }
            u2v qr[P > 0 ? P : 1][G::CH];
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int k = 0; k < G::CH; ++k) qr[p][k] = ld8(pay.codes[p] + cbase + coff + k * G::SPAN);
            add_payloads(qr, kTinyShift);
            m = block_max<G::LPB>(max_abs<G::EPL>(v));                // 2^64 max|H X|
            s = (a * m * kScaleFactor) * kOutUnshift;
        }
        // As in compress_kernel, v holds lane_sign * (H X), so r carries the
        // lane sign too.
        Quot r = quotient(C::kQmax, m);
        r.hi = (m > 0.0f) ? r.hi * lane_sign : 0.0f;
        r.lo = (m > 0.0f) ? r.lo * lane_sign : 0.0f;

        const int64_t blk = step * G::BPW + g;
        u2v c[G::CH];
#pragma unroll
        for (int k = 0; k < G::CH; ++k) c[k] = encode8<F>(&v[8 * k], r);
        const int nvalid = (int)(left < G::BPW ? left : G::BPW);            // blocks
        uint8_t *rb = codes + step * (int64_t)(G::BPW * W::kRecord);
        if constexpr (L == Layout::kSide) {
            codes_store_staged<B>(stage, rb, nvalid * B, c, g, t, lane);
            if (blk < nblocks && t == 0) {
                alpha[blk] = a * unshift;
                scale[blk] = s;
            }
        } else {
            records_store_staged<B>(stage, rb, nvalid * (int)W::kRecord, c, a * unshift, s, g, t,
                                    lane);
        }
    }
}

// Several payloads into one float32 accumulator in one pass (the local
// reduction of [TACO] section 4.4.2 over P received payloads): acc += sum_p
// G'_p.  With H H = B I, sum_p G'_p = H (sum_p sqrt(B) (s_p / alpha_p)
// decode(q_p)) / B: the payloads are summed in the rotated domain and
// transformed back once, so each element costs P decodes and one inverse
// transform, and the accumulator is read and written once.
template <int B, Fmt F, int P, Layout L>
__global__ __launch_bounds__(kGroup) void accumulate_n_kernel(Payloads pay, int64_t nblocks,
                                                              float *__restrict__ acc) {
    using G = Geo<B>;
    using W = Wire<B, L>;
    using C = Codec<F>;
    __shared__ __align__(16) float stage_all[kWavesPerGroup][AccStage<B>::kElems];
    float *stage = stage_all[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
    const int lane = threadIdx.x & (kWave - 1);
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    constexpr float kSqrtBHi = (float)(1.0 / inv_sqrt(B));
    constexpr float kSqrtBLo = (float)(1.0 / inv_sqrt(B) - (double)kSqrtBHi);
    constexpr float kInvB = 1.0f / (float)B;                  // exact

    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerGroup +
                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const uint32_t lane_elem = (uint32_t)(g * B + 8 * t);

    for (int64_t step = wave0; step < nsteps; step += nwaves) {
        // Slots past the last block re-read the last block and store nothing.
        const int64_t left = nblocks - step * G::BPW;
        const uint32_t off = left >= G::BPW ? lane_elem
                                            : (uint32_t)((g < left ? g : (int)left - 1) * B + 8 * t);
        const int64_t lblk = (step * (G::BPW * B) + off) / B;
        const uint32_t coff = (uint32_t)(lblk - step * G::BPW) * (uint32_t)W::kRecord + 8 * t;
        const int64_t cbase = step * G::BPW * W::kRecord;

        u2v qc[P][G::CH];
        float wa[P], ws[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) qc[p][k] = ld8(pay.codes[p] + cbase + coff + k * G::SPAN);
            wa[p] = pay.alpha[p][lblk * W::kScalarStride];
            ws[p] = pay.scale[p][lblk * W::kScalarStride];
        }

        // r_p = s_p / alpha_p as hi + lo; a power-of-two shift keeps
        // sqrt(B) r_p decode(q_p) and the rotated sum inside float32 range
        // (near the bf16 maximum) and out of the subnormals (tiny blocks).
        // The shift is chosen from a plain estimate of the largest r_p and
        // applied to s_p before the precise quotient, so that no r_p is a
        // float32 subnormal.
        float rmax = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) rmax = fmaxf(rmax, ws[p] > 0.0f ? ws[p] / wa[p] : 0.0f);
        const float shift = rmax >= kBigMax ? kBigShift
                            : (rmax > 0.0f && rmax < kTinyMax) ? kTinyShift : 1.0f;
        Quot r[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float sp = ws[p] * shift;
            r[p] = Quot{0.0f, 0.0f};
            if (ws[p] > 0.0f)   // (a subnormal alpha would overflow the reciprocal)
                r[p] = wa[p] >= 0x1p-120f ? quotient(sp, wa[p]) : Quot{sp / wa[p], 0.0f};
        }
        const float sh = kSqrtBHi, sl = kSqrtBLo;

        float v[G::EPL];
#pragma unroll
        for (int i = 0; i < G::EPL; ++i) v[i] = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float ch = sh * r[p].hi;
            const float cl = fmaf(sh, r[p].hi, -ch) + fmaf(sh, r[p].lo, sl * r[p].hi);
            float d[G::EPL];
#pragma unroll
            for (int k = 0; k < G::CH; ++k) C::decode8(qc[p][k], &d[8 * k]);
#pragma unroll
            for (int i = 0; i < G::EPL; ++i) v[i] = fmaf(d[i], cl, fmaf(d[i], ch, v[i]));
        }
        fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);          // lane-signed H (sum)
        // Undo the shift and divide by B (both powers of two: one rounding,
        // in the final product).
        const float fo = (kInvB / shift) * lane_sign;
#pragma unroll
        for (int i = 0; i < G::EPL; ++i) v[i] *= fo;
        acc_update_staged<B>(stage, acc, step, nblocks, v, g, t, lane);
    }
}

// ---------------------------------------------------- fidelity study -----

// Saturating codes of 8 values (the ablation variants without a scale can
// exceed Q_max): clamp to +-Q_max, map -0 to +0 (as encode8 does), convert.
template <Fmt F>
__device__ __forceinline__ u2v encode8_sat(const float *v, float factor) {
    constexpr float Q = Codec<F>::kQmax;
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(fmaf(v[j], factor, 0.0f), -Q), Q);
    return Codec<F>::pack8(q);
}

// Wave-level sum of a double (butterfly over the 64 lanes).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

// Clears the sums (one work-group).
__global__ __launch_bounds__(kGroup) void fidelity_clear_kernel(taco_fidelity_sums *sums) {
    const int i = threadIdx.x;
    if (i < 4 * TACO_FIDELITY_SLOTS) (&sums->slot_sum[0][0])[i] = 0.0;
    if (i < TACO_FIDELITY_SLOTS) {
        sums->slot_max_err[i] = 0u;
        sums->slot_absmax[i] = 0u;
    }
    if (i == 0) {
        sums->sum_sq_err = 0.0;
        sums->sum_sq_ref = 0.0;
        sums->sum_sq_out = 0.0;
        sums->sum_dot = 0.0;
        sums->max_abs_err = 0.0f;
        sums->tensor_absmax = 0.0f;
    }
}

// max |x| of a bf16 tensor into the absmax slots (n a multiple of 8, 16-byte
// aligned).  |bf16| as an integer orders like the value; the result is kept
// as float32 bits.
__global__ __launch_bounds__(kGroup) void absmax_kernel(const uint16_t *__restrict__ x,
                                                        int64_t nchunks,
                                                        taco_fidelity_sums *sums) {
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks; i += stride) {
        const u4v w = ld16(x + 8 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    m = wave_max_u(m);
    __shared__ uint32_t part[kWavesPerGroup];
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t mm = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) mm = max(mm, part[w]);
        atomicMax(&sums->slot_absmax[blockIdx.x % TACO_FIDELITY_SLOTS], mm << 16);
    }
}

// max over the absmax slots (every thread of the caller reads all slots).
__device__ __forceinline__ float tensor_absmax_of(const taco_fidelity_sums *sums) {
    uint32_t m = 0;
    for (int i = 0; i < TACO_FIDELITY_SLOTS; ++i) m = max(m, sums->slot_absmax[i]);
    return __uint_as_float(m);
}

// Totals from the slots of `sums` (one wave; slot i in lane i, a fixed
// order), written to `out`: the totals at the front of `sums` itself, or a
// separate taco_fidelity_totals.
__global__ __launch_bounds__(kGroup) void fidelity_finish_kernel(const taco_fidelity_sums *sums,
                                                                 taco_fidelity_totals *out) {
    const int lane = threadIdx.x;
    if (lane >= kWave) return;
    double t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = wave_sum(sums->slot_sum[q][lane]);
    const uint32_t me = wave_max_u(sums->slot_max_err[lane]);
    const uint32_t ma = wave_max_u(sums->slot_absmax[lane]);
    if (lane == 0) {
        out->sum_sq_err = t[0];
        out->sum_sq_ref = t[1];
        out->sum_sq_out = t[2];
        out->sum_dot = t[3];
        out->max_abs_err = __uint_as_float(me);
        out->tensor_absmax = __uint_as_float(ma);
    }
}

// One round trip of variant V per block, with the reconstruction error sums
// (see taco_fidelity_sums).  Same lane layout as compress_kernel; the codes
// of each chunk stay in registers.  The TACO variant repeats compress_kernel
// and decompress_kernel operation for operation, so its output equals
// decompress(compress(x)).  Grid-stride over wave-steps; each work-group
// adds its sums with one atomic per quantity.
template <int B, Fmt F, Variant V>
__global__ __launch_bounds__(kGroup) void roundtrip_kernel(
    const uint16_t *__restrict__ x, int64_t nblocks, float tau, uint16_t *__restrict__ y,
    taco_fidelity_sums *sums) {
    using G = Geo<B>;
    using C = Codec<F>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int t = lane_sub<G::LPB>(lane);
    const int g = lane_slot<G::LPB>(lane);
    const float sg1 = (lane & 1) ? -1.0f : 1.0f;
    const float sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg8 = (lane & 8) ? -1.0f : 1.0f;
    const float lane_sign = (__popc(t) & 1) ? -1.0f : 1.0f;
    constexpr float kScaleFactor = (float)(inv_sqrt(B) / (double)C::kQmax);
    constexpr float kInvSqrtB = (float)inv_sqrt(B);
    constexpr float kInvB = 1.0f / (float)B;

    // The whole tensor's max |x| (TENSOR variant; from absmax_kernel).
    const float tmax = (V == Variant::kTensor) ? tensor_absmax_of(sums) : 0.0f;

    double acc_e = 0.0, acc_r = 0.0, acc_o = 0.0, acc_d = 0.0;
    uint32_t max_e = 0;

    const int64_t nsteps = (nblocks + G::BPW - 1) / G::BPW;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    for (int64_t step = (int64_t)blockIdx.x * kWavesPerGroup + wave; step < nsteps;
         step += nwaves) {
        // Slots past the last block re-read the last block; nothing of them
        // is stored or summed.
        const int64_t left = nblocks - step * G::BPW;
        const int gl = (left >= G::BPW || g < left) ? g : (int)left - 1;
        const uint16_t *p = x + step * (G::BPW * B) + (uint32_t)(gl * B + 8 * t);
        const int64_t blk = step * G::BPW + g;
        const bool active = blk < nblocks;
        u4v buf[G::CH];
#pragma unroll
        for (int k = 0; k < G::CH; ++k) buf[k] = ld16(p + k * G::SPAN);
        float xin[G::EPL], v[G::EPL];
#pragma unroll
        for (int k = 0; k < G::CH; ++k) unpack8(buf[k], &xin[8 * k]);
#pragma unroll
        for (int i = 0; i < G::EPL; ++i) v[i] = xin[i];

        u2v q[G::CH];
        float f = 1.0f;            // output factor applied after decoding
        bool rotate_back = false;  // inverse transform after decoding
        bool two_step = false;     // TACO: apply (2^64 f) then 2^-64, as decompress does
        float fs = 0.0f;

        if (V == Variant::kTaco || V == Variant::kAsh) {
            // Eq. 6-7 as in compress_kernel (including its huge-block path).
#if TACO_DOT2_ENERGY
            float energy = energy_packed<G::CH>(buf);
#else
            float energy = sum_squares<G::EPL>(v);
#endif
            energy = block_sum<G::LPB>(energy);
            float unshift = 1.0f;
            if (__builtin_expect(energy >= kBigEnergy, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kBigShift;
                energy = block_sum<G::LPB>(sum_squares<G::EPL>(v));
                unshift = kBigUnshift;
            }
            const float a = tau * __builtin_amdgcn_rsqf(energy * kInvB + TACO_EPS);
            fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
            rotate_back = true;
            if (V == Variant::kTaco) {
                float m = block_max<G::LPB>(max_abs<G::EPL>(v));
                const float s = a * m * kScaleFactor;
                if (__builtin_expect(m < kTinyMax && m > 0.0f, 0)) {
#pragma unroll
                    for (int i = 0; i < G::EPL; ++i) v[i] *= kTinyShift;
                    m *= kTinyShift;
                }
                Quot r = quotient(C::kQmax, m);
                r.hi = (m > 0.0f) ? r.hi * lane_sign : 0.0f;
                r.lo = (m > 0.0f) ? r.lo * lane_sign : 0.0f;
#pragma unroll
                for (int k = 0; k < G::CH; ++k) q[k] = encode8<F>(&v[8 * k], r);
                // decompress_kernel's output factor from the stored alpha, s.
                const float at = a * unshift;
                f = ((s * kInvSqrtB) / at) * lane_sign;
                if (__builtin_expect(s > 0.0f && fabsf(f) < kTinyOut, 0)) {
                    two_step = true;
                    fs = (((s * kOutShift) * kInvSqrtB) / at) * lane_sign;
                }
            } else {
                // Z = alpha R / sqrt(B) with R = H x (lane-signed), codes of Z.
                const float za = a * kInvSqrtB * lane_sign;
#pragma unroll
                for (int k = 0; k < G::CH; ++k) q[k] = encode8_sat<F>(&v[8 * k], za);
                f = (kInvSqrtB / (a * unshift)) * lane_sign;
            }
        } else if (V == Variant::kHadamard) {
            // Blocks whose rotated values could overflow float32 are rotated
            // as x 2^-80 (exact); the codes of Z = 2^80 R' / sqrt(B) then
            // saturate as Z's would.
            float zf = kInvSqrtB * lane_sign;
            if (__builtin_expect(block_max<G::LPB>(max_abs<G::EPL>(v)) >= kBigMax, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kBigShift;
                zf *= kBigShiftInv;
            }
            fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
            rotate_back = true;
#pragma unroll
            for (int k = 0; k < G::CH; ++k) q[k] = encode8_sat<F>(&v[8 * k], zf);
            f = kInvSqrtB * lane_sign;
        } else if (V == Variant::kDirect) {
#pragma unroll
            for (int k = 0; k < G::CH; ++k) q[k] = encode8_sat<F>(&v[8 * k], 1.0f);
        } else {
            // DS (block max) or TENSOR (tensor max): codes of x Q / m, x' = decode * (m / Q).
            float m = (V == Variant::kDs) ? block_max<G::LPB>(max_abs<G::EPL>(v)) : tmax;
            const float s = m / C::kQmax;
            // quotient() needs Q / m and 1 / m in the normal range.
            if (__builtin_expect(m >= kBigMax, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kBigShift;
                m *= kBigShift;
            }
            if (__builtin_expect(m < kTinyMax && m > 0.0f, 0)) {
#pragma unroll
                for (int i = 0; i < G::EPL; ++i) v[i] *= kTinyShift;
                m *= kTinyShift;
            }
            Quot r = quotient(C::kQmax, m);
            r.hi = (m > 0.0f) ? r.hi : 0.0f;
            r.lo = (m > 0.0f) ? r.lo : 0.0f;
#pragma unroll
            for (int k = 0; k < G::CH; ++k) q[k] = encode8<F>(&v[8 * k], r);
            f = s;
        }

        // Receiver side: decode, rotate back, scale.
#pragma unroll
        for (int k = 0; k < G::CH; ++k) C::decode8(q[k], &v[8 * k]);
        if (rotate_back) fwht_block<G::LPB, G::EPL>(v, sg1, sg2, sg8);
        if (V == Variant::kTaco && two_step) {
#pragma unroll
            for (int i = 0; i < G::EPL; ++i) v[i] = (v[i] * fs) * kOutUnshift;
        } else if (V != Variant::kDirect) {
#pragma unroll
            for (int i = 0; i < G::EPL; ++i) v[i] *= f;
        }

        if (active) {
            if (y) {
                const int64_t e0 = blk * B + 8 * t;
#pragma unroll
                for (int k = 0; k < G::CH; ++k) {
                    const float *w = &v[8 * k];
                    const u4v o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                                   pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
                    st16(y + e0 + k * G::SPAN, o);
                }
            }
            float se = 0.0f, sr = 0.0f, so = 0.0f, sd = 0.0f, me = 0.0f;
#pragma unroll
            for (int i = 0; i < G::EPL; ++i) {
                const float d = v[i] - xin[i];
                se = fmaf(d, d, se);
                sr = fmaf(xin[i], xin[i], sr);
                so = fmaf(v[i], v[i], so);
                sd = fmaf(v[i], xin[i], sd);
                me = fmaxf(me, fabsf(d));
            }
            acc_e += (double)se;
            acc_r += (double)sr;
            acc_o += (double)so;
            acc_d += (double)sd;
            max_e = max(max_e, __float_as_uint(me));
        }
    }

    // Work-group totals: waves reduce, wave 0 adds them with atomics.
    __shared__ double part[kWavesPerGroup][4];
    __shared__ uint32_t part_max[kWavesPerGroup];
    acc_e = wave_sum(acc_e);
    acc_r = wave_sum(acc_r);
    acc_o = wave_sum(acc_o);
    acc_d = wave_sum(acc_d);
    max_e = wave_max_u(max_e);
    if (lane == 0) {
        part[wave][0] = acc_e;
        part[wave][1] = acc_r;
        part[wave][2] = acc_o;
        part[wave][3] = acc_d;
        part_max[wave] = max_e;
    }
    __syncthreads();
    const int slot = blockIdx.x % TACO_FIDELITY_SLOTS;
    if (wave == 0 && lane < 5) {
        if (lane < 4) {
            double tsum = 0.0;
#pragma unroll
            for (int w = 0; w < kWavesPerGroup; ++w) tsum += part[w][lane];
            atomicAdd(&sums->slot_sum[lane][slot], tsum);
        } else {
            uint32_t mm = 0;
#pragma unroll
            for (int w = 0; w < kWavesPerGroup; ++w) mm = max(mm, part_max[w]);
            atomicMax(&sums->slot_max_err[slot], mm);
        }
    }
}

// ------------------------------------------------------------- codec ------

// Element-wise conversions through the same pack8 / decode8 the operator
// uses (the operator's own scaling, and with it the mapping of -0 to +0,
// is not part of the conversion).
template <Fmt F>
__global__ __launch_bounds__(kGroup) void encode_kernel(const float *__restrict__ x, int64_t n,
                                                        uint8_t *__restrict__ codes) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i * 8 < n; i += stride) {
        const int64_t e = i * 8;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (e + j < n) ? x[e + j] : 0.0f;
        const u2v w = Codec<F>::pack8(q);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e + j < n) codes[e + j] = (uint8_t)(w[j / 4] >> (8 * (j % 4)));
    }
}

template <Fmt F>
__global__ __launch_bounds__(kGroup) void decode_kernel(const uint8_t *__restrict__ codes,
                                                        int64_t n, float *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i * 8 < n; i += stride) {
        const int64_t e = i * 8;
        u2v w = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e + j < n) w[j / 4] |= (uint32_t)codes[e + j] << (8 * (j % 4));
        float r[8];
        Codec<F>::decode8(w, r);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e + j < n) out[e + j] = r[j];
    }
}

// -------------------------------------------------------------- host ------

// Grid: each wave takes TACO_STEPS_PER_WAVE wave-steps (grid-stride), so
// large tensors launch many work-groups, which keeps every compute unit
// busy up to the tail.
unsigned grid_for(int64_t nsteps) {
    constexpr int64_t per_group = (int64_t)kWavesPerGroup * TACO_STEPS_PER_WAVE;
    int64_t g = (nsteps + per_group - 1) / per_group;
    // A dispatch counts its work-items in 32 bits: at most 2^32 - 1 threads.
    // Larger tensors take several wave-steps per wave (grid-stride loops).
#ifdef TACO_MAX_GROUPS
    const int64_t cap = TACO_MAX_GROUPS;
#else
    const int64_t cap = (INT64_C(0xFFFFFFFF) / kGroup);
#endif
    g = g < cap ? g : cap;
    return (unsigned)(g > 0 ? g : 1);
}

template <typename... Args>
taco_status launch(const void *fn, unsigned grid, hipStream_t stream, Args... args) {
    void *ptrs[] = {static_cast<void *>(&args)...};
    const hipError_t err = hipLaunchKernel(fn, dim3(grid), dim3(kGroup), ptrs, 0, stream);
    return err == hipSuccess ? TACO_OK : TACO_ERR_HIP;
}

// Calls f.template run<B>() for the runtime block size (validated before).
template <typename F>
taco_status for_block(int32_t block, F &&f) {
    switch (block) {
        case 32: return f.template run<32>();
        case 64: return f.template run<64>();
        case 128: return f.template run<128>();
        case 256: return f.template run<256>();
        default: return f.template run<512>();
    }
}

template <int B>
int64_t steps_of(int64_t nblocks) { return (nblocks + Geo<B>::BPW - 1) / Geo<B>::BPW; }

template <Fmt F>
struct CompressLaunch {
    const uint16_t *x; int64_t m; float tau; uint8_t *codes; float *alpha; float *scale;
    hipStream_t stream;
    template <int B> taco_status run() const {
        const int64_t steps = steps_of<B>(m);
        if constexpr (pairs_steps<B>()) {
            if (steps >= kPairMinSteps)
                return launch(reinterpret_cast<const void *>(&compress_kernel<B, F, 2>),
                              grid_for((steps + 1) / 2), stream, x, m, tau, codes, alpha, scale);
        }
        return launch(reinterpret_cast<const void *>(&compress_kernel<B, F, 1>),
                      grid_for(steps), stream, x, m, tau, codes, alpha, scale);
    }
};

template <Fmt F, Out MODE, Layout L>
struct DecompressLaunch {
    const uint8_t *codes; const float *alpha; const float *scale; int64_t m; uint16_t *y;
    float *acc; hipStream_t stream;
    template <int B> taco_status run() const {
        const int64_t steps = steps_of<B>(m);
        if constexpr (pairs_steps<B>()) {
            if (steps >= kPairMinSteps)
                return launch(reinterpret_cast<const void *>(&decompress_kernel<B, F, MODE, L, 2>),
                              grid_for((steps + 1) / 2), stream, codes, alpha, scale, m, y, acc);
        }
        return launch(reinterpret_cast<const void *>(&decompress_kernel<B, F, MODE, L, 1>),
                      grid_for(steps), stream, codes, alpha, scale, m, y, acc);
    }
};

template <Fmt F, Layout L>
struct ReduceLaunch {
    int npay; const uint16_t *own; Payloads pay; int64_t m; float tau; uint8_t *codes;
    float *alpha; float *scale; hipStream_t stream;
    template <int B, int P> taco_status go() const {
        return launch(reinterpret_cast<const void *>(&reduce_compress_kernel<B, F, P, L>),
                      grid_for(steps_of<B>(m)), stream, own, pay, m, tau, codes, alpha, scale);
    }
    template <int B> taco_status run() const {
        switch (npay) {
            case 0: return go<B, 0>();
            case 1: return go<B, 1>();
            case 2: return go<B, 2>();
            case 3: return go<B, 3>();
            case 4: return go<B, 4>();
            case 5: return go<B, 5>();
            case 6: return go<B, 6>();
            case 7: return go<B, 7>();
            default: return go<B, 8>();
        }
    }
};

unsigned codec_grid(int64_t n) {
    const int64_t items = (n + 7) / 8;
    const int64_t need = (items + kGroup - 1) / kGroup;
    return (unsigned)(need < 65536 ? need : 65536);
}

}  // namespace

// ------------------------------------------------- per-format entry -------

template <Fmt F>
struct CompressPackedLaunch {
    const uint16_t *x; int64_t m; float tau; uint8_t *payload; hipStream_t stream;
    template <int B> taco_status run() const {
        // One unit of 16 records per wave.
        const int64_t nunits = (m + 15) / 16;
        return launch(reinterpret_cast<const void *>(&compress_packed_kernel<B, F>),
                      grid_for(nunits), stream, x, m, tau, payload);
    }
};

template <Fmt F>
taco_status Ops<F>::compress(Layout layout, int32_t block, const uint16_t *x, int64_t nblocks,
                             float tau, uint8_t *codes, float *alpha, float *scale,
                             hipStream_t stream) {
    if (layout == Layout::kPacked)   // codes = the payload; alpha / scale point into it
        return for_block(block, CompressPackedLaunch<F>{x, nblocks, tau, codes, stream});
    return for_block(block, CompressLaunch<F>{x, nblocks, tau, codes, alpha, scale,
                                                              stream});
}

template <Fmt F>
taco_status Ops<F>::decompress(Layout layout, Out mode, int32_t block, const uint8_t *codes,
                               const float *alpha, const float *scale, int64_t nblocks,
                               uint16_t *y, float *acc, hipStream_t stream) {
    if (layout == Layout::kPacked) {
        if (mode == Out::kAccumulate)
            return for_block(block, DecompressLaunch<F, Out::kAccumulate, Layout::kPacked>{
                                        codes, alpha, scale, nblocks, y, acc, stream});
        return for_block(block, DecompressLaunch<F, Out::kBf16, Layout::kPacked>{
                                    codes, alpha, scale, nblocks, y, acc, stream});
    }
    if (mode == Out::kAccumulate)
        return for_block(block, DecompressLaunch<F, Out::kAccumulate, Layout::kSide>{
                                    codes, alpha, scale, nblocks, y, acc, stream});
    return for_block(block, DecompressLaunch<F, Out::kBf16, Layout::kSide>{
                                codes, alpha, scale, nblocks, y, acc, stream});
}

template <Fmt F>
taco_status Ops<F>::reduce_compress(Layout layout, int32_t block, int npay, const uint16_t *own,
                                    const Payloads &pay, int64_t nblocks, float tau,
                                    uint8_t *codes, float *alpha, float *scale,
                                    hipStream_t stream) {
    if (layout == Layout::kPacked)
        return for_block(block, ReduceLaunch<F, Layout::kPacked>{npay, own, pay, nblocks, tau,
                                                                  codes, alpha, scale, stream});
    return for_block(block, ReduceLaunch<F, Layout::kSide>{npay, own, pay, nblocks, tau, codes,
                                                            alpha, scale, stream});
}

template <Fmt F, Variant V>
struct RoundtripLaunch {
    const uint16_t *x; int64_t m; float tau; uint16_t *y; taco_fidelity_sums *sums;
    hipStream_t stream;
    template <int B> taco_status run() const {
        // Capped grid: 2048 groups of 4 waves fill every wave slot, and each
        // group adds its totals with one atomic per quantity into one of
        // the 64 slots (32 groups per slot).
        unsigned grid = grid_for(steps_of<B>(m));
        grid = grid < 2048u ? grid : 2048u;
        return launch(reinterpret_cast<const void *>(&roundtrip_kernel<B, F, V>), grid, stream,
                      x, m, tau, y, sums);
    }
};

template <Fmt F>
taco_status roundtrip_variant(Variant variant, int32_t block, const uint16_t *x, int64_t nblocks,
                              float tau, uint16_t *y, taco_fidelity_sums *sums,
                              hipStream_t stream) {
    switch (variant) {
        case Variant::kTaco:
            return for_block(block, RoundtripLaunch<F, Variant::kTaco>{x, nblocks, tau, y, sums, stream});
        case Variant::kDirect:
            return for_block(block, RoundtripLaunch<F, Variant::kDirect>{x, nblocks, tau, y, sums, stream});
        case Variant::kDs:
            return for_block(block, RoundtripLaunch<F, Variant::kDs>{x, nblocks, tau, y, sums, stream});
        case Variant::kAsh:
            return for_block(block, RoundtripLaunch<F, Variant::kAsh>{x, nblocks, tau, y, sums, stream});
        case Variant::kHadamard:
            return for_block(block, RoundtripLaunch<F, Variant::kHadamard>{x, nblocks, tau, y, sums, stream});
        case Variant::kTensor:
            return for_block(block, RoundtripLaunch<F, Variant::kTensor>{x, nblocks, tau, y, sums, stream});
    }
    return TACO_ERR_PARAM;
}

template <Fmt F>
taco_status Ops<F>::roundtrip(Variant variant, int32_t block, const uint16_t *x, int64_t nblocks,
                              float tau, uint16_t *y, taco_fidelity_sums *sums,
                              taco_fidelity_totals *totals, hipStream_t stream) {
    taco_status st = launch(reinterpret_cast<const void *>(&fidelity_clear_kernel), 1u, stream,
                            sums);
    if (st != TACO_OK || nblocks == 0) return st;
    if (variant == Variant::kTensor) {
        const int64_t nchunks = nblocks * block / 8;
        const int64_t need = (nchunks + kGroup - 1) / kGroup;
        const unsigned grid = (unsigned)(need < 1024 ? need : 1024);
        st = launch(reinterpret_cast<const void *>(&absmax_kernel), grid, stream, x, nchunks, sums);
        if (st != TACO_OK) return st;
    }
    st = roundtrip_variant<F>(variant, block, x, nblocks, tau, y, sums, stream);
    if (st != TACO_OK) return st;
    return launch(reinterpret_cast<const void *>(&fidelity_finish_kernel), 1u, stream,
                  static_cast<const taco_fidelity_sums *>(sums), totals);
}

template <Fmt F, Layout L>
struct AccumulateNLaunch {
    int npay; Payloads pay; int64_t m; float *acc; hipStream_t stream;
    template <int B, int P> taco_status go() const {
        return launch(reinterpret_cast<const void *>(&accumulate_n_kernel<B, F, P, L>),
                      grid_for(steps_of<B>(m)), stream, pay, m, acc);
    }
    template <int B> taco_status run() const {
        switch (npay) {
            case 1: return go<B, 1>();
            case 2: return go<B, 2>();
            case 3: return go<B, 3>();
            case 4: return go<B, 4>();
            case 5: return go<B, 5>();
            case 6: return go<B, 6>();
            case 7: return go<B, 7>();
            default: return go<B, 8>();
        }
    }
};

template <Fmt F>
taco_status Ops<F>::accumulate_n(Layout layout, int32_t block, int npay, const Payloads &pay,
                                 int64_t nblocks, float *acc, hipStream_t stream) {
    if (layout == Layout::kPacked)
        return for_block(block, AccumulateNLaunch<F, Layout::kPacked>{npay, pay, nblocks, acc, stream});
    return for_block(block, AccumulateNLaunch<F, Layout::kSide>{npay, pay, nblocks, acc, stream});
}

template <Fmt F>
taco_status Ops<F>::encode(const float *x, int64_t n, uint8_t *codes, hipStream_t stream) {
    return launch(reinterpret_cast<const void *>(&encode_kernel<F>), codec_grid(n), stream, x, n,
                  codes);
}

template <Fmt F>
taco_status Ops<F>::decode(const uint8_t *codes, int64_t n, float *out, hipStream_t stream) {
    return launch(reinterpret_cast<const void *>(&decode_kernel<F>), codec_grid(n), stream, codes,
                  n, out);
}

}  // namespace taco_internal
