// libtaco_probe (declared in include/taco_probe.h): an empty kernel and
// plain streaming kernels with the byte mixes of libtaco's kernels, for
// measuring the launch floor and the streaming ceiling at each tensor size.
// Not part of the operator; built as its own library.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "taco_probe.h"

namespace {

constexpr int kGroup = TACO_PROBE_GROUP;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = kGroup / kWave;
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGroup) void probe_empty_kernel() {}

// Wavefront w moves LD KiB in and ST KiB out: lane l reads the 16 bytes at
// 1024 i + 16 l of its KiB i (one contiguous KiB per instruction) and
// writes likewise.  All loads are issued before the first store.  Between
// them each lane issues `valu` (a multiple of 4) dependent float32 adds on
// the loaded bits, standing in for a kernel's arithmetic (WORK: a separate
// instantiation, so that traces tell the two streams apart).
template <int LD, int ST, bool WORK>
__global__ __launch_bounds__(kGroup) void probe_stream_kernel(const u4v *__restrict__ src,
                                                              u4v *__restrict__ dst,
                                                              int64_t waves, int valu) {
    const int64_t w = (int64_t)blockIdx.x * kWavesPerGroup +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= waves) return;
    const int lane = threadIdx.x & (kWave - 1);
    const u4v *s = src + w * (LD * kWave) + lane;
    u4v v[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) v[i] = __builtin_nontemporal_load(s + i * kWave);
    u4v acc = v[0];
#pragma unroll
    for (int i = 1; i < LD; ++i) acc ^= v[i];
    if (WORK) {
        float f0 = __uint_as_float(acc.x), f1 = __uint_as_float(acc.y);
        float f2 = __uint_as_float(acc.z), f3 = __uint_as_float(acc.w);
        for (int k = 0; k < valu; k += 4) {
            // A chain the compiler cannot fold or reorder: each add needs the
            // previous one's result.
            asm volatile("v_add_f32 %0, %0, %1" : "+v"(f0) : "v"(f1));
            asm volatile("v_add_f32 %0, %0, %1" : "+v"(f1) : "v"(f2));
            asm volatile("v_add_f32 %0, %0, %1" : "+v"(f2) : "v"(f3));
            asm volatile("v_add_f32 %0, %0, %1" : "+v"(f3) : "v"(f0));
        }
        acc = (u4v){__float_as_uint(f0), __float_as_uint(f1), __float_as_uint(f2),
                    __float_as_uint(f3)};
    }
    u4v *d = dst + w * (ST * kWave) + lane;
#pragma unroll
    for (int j = 0; j < ST; ++j) __builtin_nontemporal_store(acc + (unsigned)j, d + j * kWave);
}

// Launches fn on `groups` work-groups with the given arguments; the status
// is the launch's own (not an earlier error left in the runtime).
template <typename... Args>
int launch(const void *fn, int64_t groups, hipStream_t stream, Args... args) {
    void *ptrs[] = {static_cast<void *>(&args)...};
    const hipError_t err =
        hipLaunchKernel(fn, dim3((unsigned)groups), dim3(kGroup), ptrs, 0, stream);
    return err == hipSuccess ? TACO_PROBE_OK : TACO_PROBE_ERR_HIP;
}

template <int LD, int ST>
int launch_stream(const void *src, void *dst, int64_t waves, int valu, hipStream_t stream) {
    const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    const u4v *s = static_cast<const u4v *>(src);
    u4v *d = static_cast<u4v *>(dst);
    if (valu > 0)
        return launch(reinterpret_cast<const void *>(&probe_stream_kernel<LD, ST, true>), groups,
                      stream, s, d, waves, valu);
    return launch(reinterpret_cast<const void *>(&probe_stream_kernel<LD, ST, false>), groups,
                  stream, s, d, waves, 0);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// A dispatch counts its work-items in 32 bits.
constexpr int64_t kMaxGroups = INT64_C(0xFFFFFFFF) / kGroup;

extern "C" {

int taco_probe_empty(int64_t groups, hipStream_t stream) {
    if (groups < 1 || groups > kMaxGroups) return TACO_PROBE_ERR_ARGS;
    return launch(reinterpret_cast<const void *>(&probe_empty_kernel), groups, stream);
}

int taco_probe_stream(int32_t loads, int32_t stores, int32_t valu, const void *src, void *dst,
                      int64_t waves, hipStream_t stream) {
    if (waves < 1 || (waves + kWavesPerGroup - 1) / kWavesPerGroup > kMaxGroups)
        return TACO_PROBE_ERR_ARGS;
    if (valu < 0 || valu > 65536 || (valu & 3)) return TACO_PROBE_ERR_ARGS;
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return TACO_PROBE_ERR_ARGS;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t ns = (uintptr_t)waves * (uintptr_t)(loads > 0 ? loads : 0) * 1024u;
    const uintptr_t nd = (uintptr_t)waves * (uintptr_t)(stores > 0 ? stores : 0) * 1024u;
    if (s0 < d0 + nd && d0 < s0 + ns) return TACO_PROBE_ERR_ARGS;
    if (loads == 2 && stores == 1) return launch_stream<2, 1>(src, dst, waves, valu, stream);
    if (loads == 1 && stores == 2) return launch_stream<1, 2>(src, dst, waves, valu, stream);
    if (loads == 5 && stores == 4) return launch_stream<5, 4>(src, dst, waves, valu, stream);
    if (loads == 1 && stores == 1) return launch_stream<1, 1>(src, dst, waves, valu, stream);
    return TACO_PROBE_ERR_ARGS;
}

}  // extern "C"
