// libtaco C ABI (declared in include/taco.h): argument validation and
// dispatch to the per-format kernel sets (Ops<format>, one translation unit
// each).  Every check runs on the host before anything is launched.  The
// only device memory of the library itself is the fixed working array of
// taco_roundtrip_noalloc below.

#include <stdint.h>
#include <stddef.h>
#include <atomic>
#include <mutex>
#include <hip/hip_runtime.h>

#include "taco.h"
#include "taco_internal.hpp"

using namespace taco_internal;

// Working memory of taco_roundtrip_noalloc: the slots of a
// taco_fidelity_sums, in a fixed device array instead of the caller's
// buffer.  Each GPU holds its own copy; host code reaches it only through
// the address that hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[TACO_ROUNDTRIP_SCRATCH_BYTES];
static_assert(sizeof(taco_fidelity_sums) <= TACO_ROUNDTRIP_SCRATCH_BYTES,
              "the round trip's working sums must fit the fixed array");

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool valid_block(int32_t block) {
    return block == 32 || block == 64 || block == 128 || block == 256 || block == 512;
}

// N = tokens * hidden, or -1 on a bad shape (negative, zero hidden, overflow).
int64_t numel(int64_t tokens, int64_t hidden) {
    if (tokens < 0 || hidden <= 0) return -1;
    if (tokens > 0 && hidden > (INT64_C(1) << 60) / tokens) return -1;
    return tokens * hidden;
}

// Shape, block and element count checks shared by every entry point.
taco_status check_shape(int64_t tokens, int64_t hidden, int32_t block, int64_t *n_out) {
    const int64_t n = numel(tokens, hidden);
    if (n < 0) return TACO_ERR_SHAPE;
    if (!valid_block(block)) return TACO_ERR_BLOCK;
    if (n % block) return TACO_ERR_SHAPE;
    *n_out = n;
    return TACO_OK;
}

bool valid_tau(float tau) { return tau > 0.0f && tau <= TACO_MAX_TARGET_ENERGY; }

// Shared validation of the decompress-side calls (side-buffer layout).
taco_status check_receiver(const uint8_t *codes, const float *alpha, const float *scale,
                           int64_t tokens, int64_t hidden, int32_t block, const void *out,
                           size_t out_elem, int64_t *nblocks_out) {
    int64_t n = 0;
    const taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    *nblocks_out = n / block;
    if (n == 0) return TACO_OK;
    if (!codes || !alpha || !scale || !out) return TACO_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
        return TACO_ERR_ALIGN;
    const size_t nb = (size_t)(n / block) * sizeof(float);
    const size_t no = (size_t)n * out_elem;
    if (overlap(out, no, codes, (size_t)n) || overlap(out, no, alpha, nb) || overlap(out, no, scale, nb))
        return TACO_ERR_ALIAS;
    return TACO_OK;
}

// Shared validation of the decompress-side calls (interleaved layout).
taco_status check_receiver_packed(const uint8_t *payload, int64_t tokens, int64_t hidden,
                                  int32_t block, const void *out, size_t out_elem,
                                  int64_t *nblocks_out) {
    int64_t n = 0;
    const taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    *nblocks_out = n / block;
    if (n == 0) return TACO_OK;
    if (!payload || !out) return TACO_ERR_NULL;
    if (!aligned(payload, 16) || !aligned(out, 16)) return TACO_ERR_ALIGN;
    if (overlap(out, (size_t)n * out_elem, payload, (size_t)(n / block) * (size_t)(block + 8)))
        return TACO_ERR_ALIAS;
    return TACO_OK;
}

// Validation of the owner step's payloads; fills pay.  `bytes` is the size
// of one payload (codes + scalars as laid out), `packed` selects how the
// scalar pointers are derived.
taco_status check_payloads(int npay, const uint8_t *const *codes, const float *const *alpha,
                           const float *const *scale, int64_t n, int32_t block, bool packed,
                           const void *const *outs, const size_t *out_len, int nouts,
                           Payloads *pay) {
    const size_t nc = (size_t)n, nb = (size_t)(n / block) * sizeof(float);
    for (int p = 0; p < npay; ++p) {
        const uint8_t *c = codes[p];
        const float *a = packed ? (c ? reinterpret_cast<const float *>(c + block) : nullptr) : alpha[p];
        const float *sc = packed ? (c ? reinterpret_cast<const float *>(c + block + 4) : nullptr) : scale[p];
        if (!c || !a || !sc) return TACO_ERR_NULL;
        if (!aligned(c, 16) || !aligned(a, 4) || !aligned(sc, 4)) return TACO_ERR_ALIGN;
        const void *ins[3] = {c, a, sc};
        const size_t lens[3] = {packed ? (size_t)(n / block) * (size_t)(block + 8) : nc,
                                packed ? 0 : nb, packed ? 0 : nb};
        for (int i = 0; i < 3; ++i)
            for (int o = 0; o < nouts; ++o)
                if (overlap(outs[o], out_len[o], ins[i], lens[i])) return TACO_ERR_ALIAS;
        pay->codes[p] = c;
        pay->alpha[p] = a;
        pay->scale[p] = sc;
    }
    return TACO_OK;
}

// Calls fn(Ops<F>{}) for the runtime format, or reports a bad format.
template <typename Fn>
taco_status with_format(taco_format format, Fn &&fn) {
    switch (format) {
        case TACO_FORMAT_E4M3: return fn(Ops<Fmt::kE4M3>{});
        case TACO_FORMAT_E5M2: return fn(Ops<Fmt::kE5M2>{});
        case TACO_FORMAT_INT8: return fn(Ops<Fmt::kInt8>{});
    }
    return TACO_ERR_FORMAT;
}

bool valid_format(taco_format format) {
    return format == TACO_FORMAT_E4M3 || format == TACO_FORMAT_E5M2 || format == TACO_FORMAT_INT8;
}

taco_status compress_side(const uint16_t *x, int64_t tokens, int64_t hidden, int32_t block,
                          float tau, taco_format format, uint8_t *codes, float *alpha,
                          float *scale, hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    const taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (!valid_tau(tau)) return TACO_ERR_PARAM;
    if (n == 0) return TACO_OK;
    if (!x || !codes || !alpha || !scale) return TACO_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
        return TACO_ERR_ALIGN;
    const int64_t m = n / block;
    const size_t nx = (size_t)n * 2, nc = (size_t)n, nb = (size_t)m * sizeof(float);
    if (overlap(codes, nc, x, nx) || overlap(alpha, nb, x, nx) || overlap(scale, nb, x, nx) ||
        overlap(codes, nc, alpha, nb) || overlap(codes, nc, scale, nb) ||
        overlap(alpha, nb, scale, nb))
        return TACO_ERR_ALIAS;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::compress(Layout::kSide, block, x, m, tau, codes, alpha, scale, stream);
    });
}

taco_status compress_packed(const uint16_t *x, int64_t tokens, int64_t hidden, int32_t block,
                            float tau, taco_format format, uint8_t *payload, hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    const taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (!valid_tau(tau)) return TACO_ERR_PARAM;
    if (n == 0) return TACO_OK;
    if (!x || !payload) return TACO_ERR_NULL;
    if (!aligned(x, 16) || !aligned(payload, 16)) return TACO_ERR_ALIGN;
    const int64_t m = n / block;
    if (overlap(payload, (size_t)m * (size_t)(block + 8), x, (size_t)n * 2)) return TACO_ERR_ALIAS;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::compress(Layout::kPacked, block, x, m, tau, payload,
                                       reinterpret_cast<float *>(payload + block),
                                       reinterpret_cast<float *>(payload + block + 4), stream);
    });
}

taco_status decompress_side(const uint8_t *codes, const float *alpha, const float *scale,
                            int64_t tokens, int64_t hidden, int32_t block, taco_format format,
                            Out mode, void *out, hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    const size_t elem = mode == Out::kBf16 ? 2 : 4;
    int64_t m = 0;
    const taco_status st = check_receiver(codes, alpha, scale, tokens, hidden, block, out, elem, &m);
    if (st != TACO_OK || m == 0) return st;
    uint16_t *y = mode == Out::kBf16 ? static_cast<uint16_t *>(out) : nullptr;
    float *acc = mode == Out::kAccumulate ? static_cast<float *>(out) : nullptr;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::decompress(Layout::kSide, mode, block, codes, alpha, scale, m, y, acc,
                                         stream);
    });
}

taco_status decompress_packed(const uint8_t *payload, int64_t tokens, int64_t hidden,
                              int32_t block, taco_format format, Out mode, void *out,
                              hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    const size_t elem = mode == Out::kBf16 ? 2 : 4;
    int64_t m = 0;
    const taco_status st = check_receiver_packed(payload, tokens, hidden, block, out, elem, &m);
    if (st != TACO_OK || m == 0) return st;
    uint16_t *y = mode == Out::kBf16 ? static_cast<uint16_t *>(out) : nullptr;
    float *acc = mode == Out::kAccumulate ? static_cast<float *>(out) : nullptr;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::decompress(Layout::kPacked, mode, block, payload,
                                         reinterpret_cast<const float *>(payload + block),
                                         reinterpret_cast<const float *>(payload + block + 4), m,
                                         y, acc, stream);
    });
}

taco_status reduce_side(const uint16_t *own, int32_t npayloads, const uint8_t *const *codes,
                        const float *const *alpha, const float *const *scale, int64_t tokens,
                        int64_t hidden, int32_t block, float tau, taco_format format,
                        uint8_t *out_codes, float *out_alpha, float *out_scale,
                        hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (!valid_tau(tau)) return TACO_ERR_PARAM;
    if (npayloads < 0 || npayloads > TACO_MAX_PAYLOADS) return TACO_ERR_PARAM;
    if (npayloads == 0 && !own) return TACO_ERR_PARAM;
    if (n == 0) return TACO_OK;
    if (!out_codes || !out_alpha || !out_scale) return TACO_ERR_NULL;
    if (npayloads > 0 && (!codes || !alpha || !scale)) return TACO_ERR_NULL;
    const int64_t m = n / block;
    const size_t nc = (size_t)n, nb = (size_t)m * sizeof(float);
    if (!aligned(out_codes, 16) || !aligned(out_alpha, 4) || !aligned(out_scale, 4))
        return TACO_ERR_ALIGN;
    if (overlap(out_codes, nc, out_alpha, nb) || overlap(out_codes, nc, out_scale, nb) ||
        overlap(out_alpha, nb, out_scale, nb))
        return TACO_ERR_ALIAS;
    const void *outs[3] = {out_codes, out_alpha, out_scale};
    const size_t out_len[3] = {nc, nb, nb};
    if (own) {
        if (!aligned(own, 16)) return TACO_ERR_ALIGN;
        for (int o = 0; o < 3; ++o)
            if (overlap(outs[o], out_len[o], own, (size_t)n * 2)) return TACO_ERR_ALIAS;
    }
    Payloads pay = {};
    st = check_payloads(npayloads, codes, alpha, scale, n, block, false, outs, out_len, 3, &pay);
    if (st != TACO_OK) return st;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::reduce_compress(Layout::kSide, block, npayloads, own, pay, m, tau,
                                              out_codes, out_alpha, out_scale, stream);
    });
}

taco_status reduce_packed(const uint16_t *own, int32_t npayloads, const uint8_t *const *payloads,
                          int64_t tokens, int64_t hidden, int32_t block, float tau,
                          taco_format format, uint8_t *out_payload, hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (!valid_tau(tau)) return TACO_ERR_PARAM;
    if (npayloads < 0 || npayloads > TACO_MAX_PAYLOADS) return TACO_ERR_PARAM;
    if (npayloads == 0 && !own) return TACO_ERR_PARAM;
    if (n == 0) return TACO_OK;
    if (!out_payload) return TACO_ERR_NULL;
    if (npayloads > 0 && !payloads) return TACO_ERR_NULL;
    const int64_t m = n / block;
    if (!aligned(out_payload, 16)) return TACO_ERR_ALIGN;
    const void *outs[1] = {out_payload};
    const size_t out_len[1] = {(size_t)m * (size_t)(block + 8)};
    if (own) {
        if (!aligned(own, 16)) return TACO_ERR_ALIGN;
        if (overlap(out_payload, out_len[0], own, (size_t)n * 2)) return TACO_ERR_ALIAS;
    }
    Payloads pay = {};
    st = check_payloads(npayloads, payloads, nullptr, nullptr, n, block, true, outs, out_len, 1,
                        &pay);
    if (st != TACO_OK) return st;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::reduce_compress(
            Layout::kPacked, block, npayloads, own, pay, m, tau, out_payload,
            reinterpret_cast<float *>(out_payload + block),
            reinterpret_cast<float *>(out_payload + block + 4), stream);
    });
}

taco_status accumulate_n_any(int32_t npayloads, const uint8_t *const *codes,
                             const float *const *alpha, const float *const *scale, bool packed,
                             int64_t tokens, int64_t hidden, int32_t block, taco_format format,
                             float *acc, hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (npayloads < 0 || npayloads > TACO_MAX_PAYLOADS) return TACO_ERR_PARAM;
    if (n == 0 || npayloads == 0) return TACO_OK;
    if (!acc) return TACO_ERR_NULL;
    if (!codes || (!packed && (!alpha || !scale))) return TACO_ERR_NULL;
    if (!aligned(acc, 16)) return TACO_ERR_ALIGN;
    const void *outs[1] = {acc};
    const size_t out_len[1] = {(size_t)n * sizeof(float)};
    Payloads pay = {};
    st = check_payloads(npayloads, codes, alpha, scale, n, block, packed, outs, out_len, 1, &pay);
    if (st != TACO_OK) return st;
    const Layout layout = packed ? Layout::kPacked : Layout::kSide;
    return with_format(format, [&](auto ops) {
        return decltype(ops)::accumulate_n(layout, block, npayloads, pay, n / block, acc, stream);
    });
}

taco_status encode_any(taco_format format, const float *x, int64_t n, uint8_t *codes,
                       hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    if (n < 0) return TACO_ERR_SHAPE;
    if (n == 0) return TACO_OK;
    if (!x || !codes) return TACO_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16)) return TACO_ERR_ALIGN;
    if (overlap(codes, (size_t)n, x, (size_t)n * 4)) return TACO_ERR_ALIAS;
    return with_format(format, [&](auto ops) { return decltype(ops)::encode(x, n, codes, stream); });
}

taco_status decode_any(taco_format format, const uint8_t *codes, int64_t n, float *out,
                       hipStream_t stream) {
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    if (n < 0) return TACO_ERR_SHAPE;
    if (n == 0) return TACO_OK;
    if (!codes || !out) return TACO_ERR_NULL;
    if (!aligned(out, 16) || !aligned(codes, 16)) return TACO_ERR_ALIGN;
    if (overlap(out, (size_t)n * 4, codes, (size_t)n)) return TACO_ERR_ALIAS;
    return with_format(format, [&](auto ops) { return decltype(ops)::decode(codes, n, out, stream); });
}

// The totals of taco_fidelity_sums sit at its front with the layout of
// taco_fidelity_totals, so the finish kernel can write either.
static_assert(offsetof(taco_fidelity_sums, sum_sq_err) == offsetof(taco_fidelity_totals, sum_sq_err) &&
                  offsetof(taco_fidelity_sums, sum_sq_ref) == offsetof(taco_fidelity_totals, sum_sq_ref) &&
                  offsetof(taco_fidelity_sums, sum_sq_out) == offsetof(taco_fidelity_totals, sum_sq_out) &&
                  offsetof(taco_fidelity_sums, sum_dot) == offsetof(taco_fidelity_totals, sum_dot) &&
                  offsetof(taco_fidelity_sums, max_abs_err) == offsetof(taco_fidelity_totals, max_abs_err) &&
                  offsetof(taco_fidelity_sums, tensor_absmax) ==
                      offsetof(taco_fidelity_totals, tensor_absmax) &&
                  sizeof(taco_fidelity_totals) == 40,
              "taco_fidelity_totals must match the front of taco_fidelity_sums");

// Validation of a round trip.  out / out_bytes: the caller's sums or totals
// (8-byte aligned, must not overlap x or y).  On TACO_OK with *n_out > 0
// the caller launches.
taco_status check_roundtrip(const uint16_t *x, int64_t tokens, int64_t hidden, int32_t block,
                            float tau, taco_format format, taco_variant variant,
                            const uint16_t *y, const void *out, size_t out_bytes,
                            int64_t *n_out) {
    *n_out = 0;
    if (!valid_format(format)) return TACO_ERR_FORMAT;
    int64_t n = 0;
    const taco_status st = check_shape(tokens, hidden, block, &n);
    if (st != TACO_OK) return st;
    if (!valid_tau(tau)) return TACO_ERR_PARAM;
    if (variant < TACO_VARIANT_TACO || variant > TACO_VARIANT_TENSOR) return TACO_ERR_PARAM;
    if (n == 0) return TACO_OK;
    if (!out || !x) return TACO_ERR_NULL;
    if (!aligned(out, 8)) return TACO_ERR_ALIGN;
    if (!aligned(x, 16) || (y && !aligned(y, 16))) return TACO_ERR_ALIGN;
    if (overlap(out, out_bytes, x, (size_t)n * 2) ||
        (y && overlap(out, out_bytes, y, (size_t)n * 2)) ||
        (y && overlap(y, (size_t)n * 2, x, (size_t)n * 2)))
        return TACO_ERR_ALIAS;
    *n_out = n;
    return TACO_OK;
}

// Launches a validated round trip of n > 0 elements: working sums in *sums,
// totals to *totals.
taco_status launch_roundtrip(const uint16_t *x, int64_t n, int32_t block, float tau,
                             taco_format format, taco_variant variant, uint16_t *y,
                             taco_fidelity_sums *sums, taco_fidelity_totals *totals,
                             hipStream_t stream) {
    const Variant v = static_cast<Variant>(static_cast<int>(variant));
    return with_format(format, [&](auto ops) {
        return decltype(ops)::roundtrip(v, block, x, n / block, tau, y, sums, totals, stream);
    });
}

// ---------------------------------------------- working array, one per GPU ---

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch`, looked up on
// the first call per device (once; later calls read the cached address).
// The stream must belong to the current device.
taco_status scratch_address(hipStream_t stream, void **addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TACO_ERR_HIP;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return TACO_ERR_HIP;
    }
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return TACO_ERR_HIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return TACO_OK;
}

}  // namespace

// ---------------------------------------------------------------- C ABI ---

extern "C" {

int64_t taco_num_blocks(int64_t tokens, int64_t hidden, int32_t block) {
    int64_t n = 0;
    if (check_shape(tokens, hidden, block, &n) != TACO_OK) return -1;
    return n / block;
}

int64_t taco_packed_bytes(int64_t tokens, int64_t hidden, int32_t block) {
    int64_t n = 0;
    if (check_shape(tokens, hidden, block, &n) != TACO_OK) return -1;
    return (n / block) * (block + 8);
}

taco_status taco_compress(const uint16_t *x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                          float target_energy, uint8_t *codes_e4m3, float *alpha, float *scale,
                          hipStream_t stream) {
    return compress_side(x_bf16, tokens, hidden, block, target_energy, TACO_FORMAT_E4M3,
                         codes_e4m3, alpha, scale, stream);
}

taco_status taco_compress_fmt(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                              int32_t block, float target_energy, taco_format format,
                              uint8_t *codes, float *alpha, float *scale, hipStream_t stream) {
    return compress_side(x_bf16, tokens, hidden, block, target_energy, format, codes, alpha, scale,
                         stream);
}

taco_status taco_compress_packed(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                 int32_t block, float target_energy, uint8_t *payload,
                                 hipStream_t stream) {
    return compress_packed(x_bf16, tokens, hidden, block, target_energy, TACO_FORMAT_E4M3, payload,
                           stream);
}

taco_status taco_compress_packed_fmt(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                     int32_t block, float target_energy, taco_format format,
                                     uint8_t *payload, hipStream_t stream) {
    return compress_packed(x_bf16, tokens, hidden, block, target_energy, format, payload, stream);
}

taco_status taco_decompress(const uint8_t *codes_e4m3, const float *alpha, const float *scale,
                            int64_t tokens, int64_t hidden, int32_t block, uint16_t *y_bf16,
                            hipStream_t stream) {
    return decompress_side(codes_e4m3, alpha, scale, tokens, hidden, block, TACO_FORMAT_E4M3,
                           Out::kBf16, y_bf16, stream);
}

taco_status taco_decompress_fmt(const uint8_t *codes, const float *alpha, const float *scale,
                                int64_t tokens, int64_t hidden, int32_t block, taco_format format,
                                uint16_t *y_bf16, hipStream_t stream) {
    return decompress_side(codes, alpha, scale, tokens, hidden, block, format, Out::kBf16, y_bf16,
                           stream);
}

taco_status taco_decompress_packed(const uint8_t *payload, int64_t tokens, int64_t hidden,
                                   int32_t block, uint16_t *y_bf16, hipStream_t stream) {
    return decompress_packed(payload, tokens, hidden, block, TACO_FORMAT_E4M3, Out::kBf16, y_bf16,
                             stream);
}

taco_status taco_decompress_packed_fmt(const uint8_t *payload, int64_t tokens, int64_t hidden,
                                       int32_t block, taco_format format, uint16_t *y_bf16,
                                       hipStream_t stream) {
    return decompress_packed(payload, tokens, hidden, block, format, Out::kBf16, y_bf16, stream);
}

taco_status taco_decompress_accumulate(const uint8_t *codes_e4m3, const float *alpha,
                                       const float *scale, int64_t tokens, int64_t hidden,
                                       int32_t block, float *acc_f32, hipStream_t stream) {
    return decompress_side(codes_e4m3, alpha, scale, tokens, hidden, block, TACO_FORMAT_E4M3,
                           Out::kAccumulate, acc_f32, stream);
}

taco_status taco_decompress_accumulate_fmt(const uint8_t *codes, const float *alpha,
                                           const float *scale, int64_t tokens, int64_t hidden,
                                           int32_t block, taco_format format, float *acc_f32,
                                           hipStream_t stream) {
    return decompress_side(codes, alpha, scale, tokens, hidden, block, format, Out::kAccumulate,
                           acc_f32, stream);
}

taco_status taco_decompress_accumulate_packed(const uint8_t *payload, int64_t tokens,
                                              int64_t hidden, int32_t block, float *acc_f32,
                                              hipStream_t stream) {
    return decompress_packed(payload, tokens, hidden, block, TACO_FORMAT_E4M3, Out::kAccumulate,
                             acc_f32, stream);
}

taco_status taco_decompress_accumulate_packed_fmt(const uint8_t *payload, int64_t tokens,
                                                  int64_t hidden, int32_t block,
                                                  taco_format format, float *acc_f32,
                                                  hipStream_t stream) {
    return decompress_packed(payload, tokens, hidden, block, format, Out::kAccumulate, acc_f32,
                             stream);
}

taco_status taco_reduce_compress(const uint16_t *own_bf16, int32_t npayloads,
                                 const uint8_t *const *codes_e4m3, const float *const *alpha,
                                 const float *const *scale, int64_t tokens, int64_t hidden,
                                 int32_t block, float target_energy, uint8_t *out_codes,
                                 float *out_alpha, float *out_scale, hipStream_t stream) {
    return reduce_side(own_bf16, npayloads, codes_e4m3, alpha, scale, tokens, hidden, block,
                       target_energy, TACO_FORMAT_E4M3, out_codes, out_alpha, out_scale, stream);
}

taco_status taco_reduce_compress_fmt(const uint16_t *own_bf16, int32_t npayloads,
                                     const uint8_t *const *codes, const float *const *alpha,
                                     const float *const *scale, int64_t tokens, int64_t hidden,
                                     int32_t block, float target_energy, taco_format format,
                                     uint8_t *out_codes, float *out_alpha, float *out_scale,
                                     hipStream_t stream) {
    return reduce_side(own_bf16, npayloads, codes, alpha, scale, tokens, hidden, block,
                       target_energy, format, out_codes, out_alpha, out_scale, stream);
}

taco_status taco_reduce_compress_packed(const uint16_t *own_bf16, int32_t npayloads,
                                        const uint8_t *const *payloads, int64_t tokens,
                                        int64_t hidden, int32_t block, float target_energy,
                                        uint8_t *out_payload, hipStream_t stream) {
    return reduce_packed(own_bf16, npayloads, payloads, tokens, hidden, block, target_energy,
                         TACO_FORMAT_E4M3, out_payload, stream);
}

taco_status taco_reduce_compress_packed_fmt(const uint16_t *own_bf16, int32_t npayloads,
                                            const uint8_t *const *payloads, int64_t tokens,
                                            int64_t hidden, int32_t block, float target_energy,
                                            taco_format format, uint8_t *out_payload,
                                            hipStream_t stream) {
    return reduce_packed(own_bf16, npayloads, payloads, tokens, hidden, block, target_energy,
                         format, out_payload, stream);
}

taco_status taco_decompress_accumulate_n(int32_t npayloads, const uint8_t *const *codes_e4m3,
                                         const float *const *alpha, const float *const *scale,
                                         int64_t tokens, int64_t hidden, int32_t block,
                                         float *acc_f32, hipStream_t stream) {
    return accumulate_n_any(npayloads, codes_e4m3, alpha, scale, false, tokens, hidden, block,
                            TACO_FORMAT_E4M3, acc_f32, stream);
}

taco_status taco_decompress_accumulate_n_fmt(int32_t npayloads, const uint8_t *const *codes,
                                             const float *const *alpha, const float *const *scale,
                                             int64_t tokens, int64_t hidden, int32_t block,
                                             taco_format format, float *acc_f32,
                                             hipStream_t stream) {
    return accumulate_n_any(npayloads, codes, alpha, scale, false, tokens, hidden, block, format,
                            acc_f32, stream);
}

taco_status taco_decompress_accumulate_n_packed(int32_t npayloads, const uint8_t *const *payloads,
                                                int64_t tokens, int64_t hidden, int32_t block,
                                                float *acc_f32, hipStream_t stream) {
    return accumulate_n_any(npayloads, payloads, nullptr, nullptr, true, tokens, hidden, block,
                            TACO_FORMAT_E4M3, acc_f32, stream);
}

taco_status taco_decompress_accumulate_n_packed_fmt(int32_t npayloads,
                                                    const uint8_t *const *payloads, int64_t tokens,
                                                    int64_t hidden, int32_t block,
                                                    taco_format format, float *acc_f32,
                                                    hipStream_t stream) {
    return accumulate_n_any(npayloads, payloads, nullptr, nullptr, true, tokens, hidden, block,
                            format, acc_f32, stream);
}

taco_status taco_e4m3_encode(const float *x, int64_t n, uint8_t *codes, hipStream_t stream) {
    return encode_any(TACO_FORMAT_E4M3, x, n, codes, stream);
}

taco_status taco_e4m3_decode(const uint8_t *codes, int64_t n, float *out, hipStream_t stream) {
    return decode_any(TACO_FORMAT_E4M3, codes, n, out, stream);
}

taco_status taco_encode(taco_format format, const float *x, int64_t n, uint8_t *codes,
                        hipStream_t stream) {
    return encode_any(format, x, n, codes, stream);
}

taco_status taco_decode(taco_format format, const uint8_t *codes, int64_t n, float *out,
                        hipStream_t stream) {
    return decode_any(format, codes, n, out, stream);
}

taco_status taco_roundtrip(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                           int32_t block, float target_energy, taco_format format,
                           taco_variant variant, uint16_t *y_bf16, taco_fidelity_sums *sums,
                           hipStream_t stream) {
    int64_t n = 0;
    const taco_status st = check_roundtrip(x_bf16, tokens, hidden, block, target_energy, format,
                                           variant, y_bf16, sums, sizeof(taco_fidelity_sums), &n);
    if (st != TACO_OK || n == 0) return st;
    return launch_roundtrip(x_bf16, n, block, target_energy, format, variant, y_bf16, sums,
                            reinterpret_cast<taco_fidelity_totals *>(sums), stream);
}

taco_status taco_roundtrip_noalloc(const uint16_t *x_bf16, int64_t tokens, int64_t hidden,
                                   int32_t block, float target_energy, taco_format format,
                                   taco_variant variant, uint16_t *y_bf16,
                                   taco_fidelity_totals *totals, hipStream_t stream) {
    int64_t n = 0;
    taco_status st = check_roundtrip(x_bf16, tokens, hidden, block, target_energy, format,
                                     variant, y_bf16, totals, sizeof(taco_fidelity_totals), &n);
    if (st != TACO_OK || n == 0) return st;
    void *work = nullptr;
    st = scratch_address(stream, &work);
    if (st != TACO_OK) return st;
    return launch_roundtrip(x_bf16, n, block, target_energy, format, variant, y_bf16,
                            static_cast<taco_fidelity_sums *>(work), totals, stream);
}

const char *taco_status_string(taco_status status) {
    switch (status) {
        case TACO_OK: return "ok";
        case TACO_ERR_NULL: return "a required pointer is NULL";
        case TACO_ERR_SHAPE: return "bad shape: tokens < 0, hidden <= 0, or N not a multiple of the block";
        case TACO_ERR_BLOCK: return "block size must be 32, 64, 128, 256 or 512";
        case TACO_ERR_PARAM: return "target energy must be finite and in (0, 1e20], the payload count in 0..8 (0 only with own data), and the variant a taco_variant value";
        case TACO_ERR_ALIGN: return "tensors must be 16-byte aligned, alpha and scale 4-byte aligned";
        case TACO_ERR_ALIAS: return "an output buffer overlaps an input or another output";
        case TACO_ERR_HIP: return "the HIP runtime refused the kernel launch";
        case TACO_ERR_FORMAT: return "code format must be TACO_FORMAT_E4M3, TACO_FORMAT_E5M2 or TACO_FORMAT_INT8";
    }
    return "unknown status";
}

}  // extern "C"
