// Host-side helpers of libqi4: argument checks, the device check, launch errors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qi4.h"

namespace qi4 {

// True when [a, a+na) and [b, b+nb) (bytes) overlap.
inline bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

inline bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// The group size a call means: 0 stands for one group per row (K).
inline int64_t effective_group(int group_size, int64_t K) { return group_size == 0 ? K : group_size; }

// K of the packed 4-bit matrix that holds an N x K matrix: an 8-bit matrix is
// stored as two 4-bit planes, one 128-wide block of each per block of K.
inline int64_t packed_k(int64_t K, int flags) { return (flags & QI4_INT8) ? 2 * K : K; }

// Bytes of the canonical codes of an N x K matrix.
inline int64_t code_bytes(int64_t N, int64_t K, int flags) {
    return (flags & QI4_INT8) ? N * K : N * K / 2;
}

// Shape checks common to every call on a packed matrix.
inline int check_matrix(int64_t N, int64_t K, int group_size, int flags) {
    // 64, or a multiple of 128 dividing K (0 or K: one group per row)
    const int64_t gs = effective_group(group_size, K);
    if (group_size < 0 || (gs != 64 && (gs < 128 || gs % 128 != 0))) return QI4_ERR_GROUP;
    if (gs > 64 && K % gs != 0) return QI4_ERR_SHAPE;
    if (flags & ~(QI4_PACK_GATEUP | QI4_INT8)) return QI4_ERR_UNSUPPORTED;
    if (N < 1 || K < 128 || (K % 128) != 0) return QI4_ERR_SHAPE;
    if ((flags & QI4_PACK_GATEUP) && (N % 2) != 0) return QI4_ERR_SHAPE;
    if (N > (int64_t(1) << 31) || K > (int64_t(1) << 30)) return QI4_ERR_SHAPE;
    return QI4_OK;
}

// QI4_OK when the current device is gfx950 (cached per device), else
// QI4_ERR_UNSUPPORTED, or QI4_ERR_HIP when no device can be queried.
int check_device();

// Map the launch status of the last kernel to a return code.
inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QI4_OK : QI4_ERR_HIP;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace qi4
