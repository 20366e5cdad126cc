// Measurement probes: what the chip delivers on the two resources the kernels
// of this library are bound by, measured on the same machine as the kernels.
//  * qi4_probe_stream_read: every byte of a large buffer read once with
//    16-byte non-temporal loads, eight in flight per lane, one contiguous span
//    per workgroup; the achieved bytes per second is the practical HBM read
//    ceiling.
//  * qi4_probe_mfma: independent chains of fp16 16x16x32 MFMAs on every SIMD
//    (eight accumulators per wave), no memory traffic; the achieved flops per
//    second is the practical dense fp16/bf16 matrix-core ceiling.
// Both write a value derived from their work to `sink` so nothing is removed
// by the compiler.
#include "../../include/qi4_probe.h"
#include "qi4_dev.h"
#include "qi4_host.h"

namespace qi4 {
namespace {

constexpr int kReadThreads = 256;

// A 16-byte load with the non-temporal hint (each byte is read once): on
// MI355X this reads 6.8-6.9 TB/s against 6.0 TB/s with ordinary loads.
__device__ inline uint4 load_nt(const uint4 *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}
constexpr int kReadUnroll = 8;
constexpr int kReadBlocks = QI4_PROBE_READ_SINK_WORDS / (kReadThreads / 64);

// Each workgroup reads one contiguous span (its share of the buffer, a
// multiple of kReadThreads * 16 * kReadUnroll bytes except in the last
// workgroup), kReadUnroll 16-byte loads per lane in flight, consecutive lanes
// on consecutive 16-byte chunks: the access pattern of the weight streams.
__global__ void __launch_bounds__(kReadThreads)
stream_read_kernel(const uint4 *__restrict__ buf, int64_t n16, uint32_t *__restrict__ sink) {
    constexpr int64_t step = (int64_t)kReadThreads * kReadUnroll;   // 16-byte chunks per round
    const int64_t rounds = (n16 + step - 1) / step;
    const int64_t per = (rounds + gridDim.x - 1) / gridDim.x;      // rounds per workgroup
    const int64_t beg = (int64_t)blockIdx.x * per * step;
    int64_t end = beg + per * step;
    if (end > n16) end = n16;
    uint32_t acc = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + (kReadUnroll - 1) * kReadThreads < end; i += step) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = load_nt(buf + i + u * kReadThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += kReadThreads) {
        const uint4 v = load_nt(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one value per wave, the xor of its lanes, so the loads stay
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

constexpr int kMfmaChains = 8;

__global__ void __launch_bounds__(256)
mfma_probe_kernel(int64_t iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(0.001f * (float)((lane + e) & 7));
        b[e] = (_Float16)(0.002f * (float)((lane * 3 + e) & 7));
    }
    f32x4 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // each accumulator tied to its own registers: with the builtin the register
    // allocator rotated the eight chains through moves every iteration
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c)
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (s == 12345.678f) sink[0] = s;   // practically never; keeps the MFMAs live
}

}  // namespace
}  // namespace qi4

using namespace qi4;

extern "C" int qi4_probe_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                                     void *stream) {
    if (!buf || !sink) return QI4_ERR_NULL;
    if (bytes < 16 || bytes % 16 || !aligned(buf, 16)) return QI4_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    // 8 workgroups per CU on 256 CUs; sink holds one word per wave
    stream_read_kernel<<<kReadBlocks, kReadThreads, 0, as_stream(stream)>>>(
        static_cast<const uint4 *>(buf), bytes / 16, sink);
    return launch_status();
}

extern "C" int64_t qi4_probe_mfma_flops(int64_t iters, int64_t workgroups) {
    if (iters < 1 || workgroups < 1) return QI4_ERR_SHAPE;
    // 4 waves per workgroup, kMfmaChains MFMAs per iteration, 2 * 16 * 16 * 32 flop each
    return workgroups * 4 * iters * kMfmaChains * (2 * 16 * 16 * 32);
}

extern "C" int qi4_probe_mfma(int64_t iters, int64_t workgroups, float *sink, void *stream) {
    if (!sink) return QI4_ERR_NULL;
    if (iters < 1 || workgroups < 1 || workgroups > 0x7fffffff) return QI4_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    mfma_probe_kernel<<<(unsigned)workgroups, 256, 0, as_stream(stream)>>>(iters, sink);
    return launch_status();
}
