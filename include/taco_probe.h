/*
 * libtaco_probe -- measurement kernels that sit beside libtaco (they are
 * not part of the operator): an empty kernel and plain streaming kernels
 * with the byte mixes of the operator's kernels.  Timed with the same
 * launch shape and buffer rotation as the operator, they measure what any
 * single-launch kernel pays at a given tensor size: the launch floor (an
 * empty kernel on the same grid) and the streaming ceiling (loads and
 * stores of the same bytes, no arithmetic).
 *
 * Conventions: device pointers owned by the caller, calls asynchronous on
 * `stream`, 0 on success, TACO_PROBE_ERR_ARGS for bad arguments (nothing
 * launched), TACO_PROBE_ERR_HIP when the runtime refuses the launch.
 */
#ifndef TACO_PROBE_H
#define TACO_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TACO_PROBE_OK 0
#define TACO_PROBE_ERR_ARGS 1
#define TACO_PROBE_ERR_HIP 2

/* Threads per work-group of every probe kernel (four wavefronts), as in
 * libtaco's kernels. */
#define TACO_PROBE_GROUP 256

/* An empty kernel on `groups` work-groups of TACO_PROBE_GROUP threads
 * (1 <= groups <= 2^31 - 1). */
int taco_probe_empty(int64_t groups, hipStream_t stream);

/*
 * A plain stream over `waves` wavefronts (four per work-group): wavefront w
 * reads `loads` KiB from src starting at byte w * loads * 1024 and writes
 * `stores` KiB to dst starting at byte w * stores * 1024, 1 KiB per
 * instruction (16 bytes per lane, non-temporal, like the operator's bulk
 * traffic).  Between its loads and its stores each wavefront issues `valu`
 * dependent float32 vector instructions (0 <= valu <= 65536, a multiple of
 * 4), standing in for the arithmetic of a kernel with that many VALU
 * instructions per wavefront.  Supported (loads, stores): (2, 1), the compress mix at B = 128
 * (2 bytes of bf16 in, 1 byte of code out per element); (1, 2), the
 * decompress mix; (5, 4), the accumulate mix (1 + 4 bytes in, 4 out per
 * element); (1, 1), a copy.  src holds waves * loads KiB and dst
 * waves * stores KiB, both 16-byte aligned and not overlapping.  The bytes
 * written are a function of the bytes read (their XOR), so nothing is
 * optimised away.
 */
int taco_probe_stream(int32_t loads, int32_t stores, int32_t valu, const void *src, void *dst,
                      int64_t waves, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TACO_PROBE_H */
