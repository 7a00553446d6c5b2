// Measurement support, not on the product path: a plain streaming read of a device buffer,
// the achievable HBM read rate the weight stream is compared against.  The MARLIN paper
// bounds the layer by weight loading (sec. 3.4, "Bound By Weight Loading"), so the fraction
// of a measured read rate says how close the multiply comes to that bound on this chip,
// beside the fraction of the nominal 8 TB/s.
//
// Access pattern: each workgroup streams one contiguous chunk of the buffer, its 256 lanes
// reading 4 KiB per step with 128-bit non-temporal loads, eight steps in flight.  Among the
// patterns measured on MI355X this one reads fastest (6.80-6.85 TB/s over 4 GiB in every
// recorded run, against 6.0-6.8 TB/s for grid-stride loops), so it serves as the achievable
// read rate.
//
// The second probe times the matrix cores on operands that change from one instruction to
// the next: each wave cycles eight independent fp32 accumulators through pairs of 16 operand
// fragments loaded from a buffer of random fp16 values, so the multipliers see data like a
// GEMM's (the sustained rate with random data is well below the rate with constant data: the
// chip lowers its clock under the higher power).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "w4a16.h"
#include "device.h"
#include "kernel_common.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeWGs = 2048;
constexpr int kProbeDepth = 8;              // 16-byte loads per lane in flight
constexpr uint32_t kMagic = 0x9e3779b9u;   // the checksum that would trigger a store

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u4 *__restrict__ src,
                                                                   uint64_t n16,
                                                                   uint32_t *__restrict__ out)
{
    const uint64_t per = n16 / gridDim.x;                    // whole chunks per workgroup
    const u4 *p = src + per * blockIdx.x;
    uint32_t x = 0;
    uint64_t i = threadIdx.x;
    for (; i + (kProbeDepth - 1) * kProbeThreads < per; i += kProbeDepth * kProbeThreads) {
        u4 e = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d)
            e ^= __builtin_nontemporal_load(p + i + d * kProbeThreads);
        x ^= e[0] ^ e[1] ^ e[2] ^ e[3];
    }
    for (; i < per; i += kProbeThreads) {
        const u4 a = __builtin_nontemporal_load(p + i);
        x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    // the chunks past gridDim.x * per, one per workgroup
    const uint64_t tail = per * gridDim.x + static_cast<uint64_t>(blockIdx.x) * kProbeThreads +
                          threadIdx.x;
    if (tail < n16) {
        const u4 a = __builtin_nontemporal_load(src + tail);
        x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    // every load feeds x; the store happens only for one checksum value in 2^32
    if (x == kMagic)
        out[blockIdx.x] = x;
}

typedef float f16v __attribute__((ext_vector_type(16)));

// shape 0: 16x16x32 (acc 4 floats), 1: 32x32x16 (acc 16 floats).  Fragment f of lane l of
// global wave w is 16-byte chunk ((w * 64 + l) * 16 + f) mod n16 of src.
template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const u4 *__restrict__ src,
                                                                   uint32_t n16, int iters,
                                                                   float *__restrict__ out)
{
    const uint32_t gl = blockIdx.x * kProbeThreads + threadIdx.x;     // global lane
    h8 a[8], b[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        a[f] = __builtin_bit_cast(h8, src[(gl * 16u + f) % n16]);
        b[f] = __builtin_bit_cast(h8, src[(gl * 16u + 8 + f) % n16]);
    }
    using Acc = std::conditional_t<SHAPE == 0, f4, f16v>;
    Acc acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = Acc{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (SHAPE == 0)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[(i + j) & 7], acc[i],
                                                                    0, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[(i + j) & 7], acc[i],
                                                                    0, 0, 0);
            }
    }
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < (SHAPE == 0 ? 4 : 16); ++e)
            x += acc[i][e];
    out[gl] = x;
}

}  // namespace

extern "C" int w4a16_mfma_probe(const void *src, size_t src_bytes, int shape, int workgroups,
                                int iters, float *out, void *stream)
{
    if (!src || !out || src_bytes == 0 || src_bytes % 16 || (src_bytes >> 4) > 0xffffffffu ||
        (reinterpret_cast<uintptr_t>(src) & 15) || workgroups <= 0 || iters <= 0 ||
        (shape != 0 && shape != 1))
        return W4A16_EINVAL;
    w4a16_detail::DeviceInfo d;
    const int rc = w4a16_detail::current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    const uint32_t n16 = static_cast<uint32_t>(src_bytes >> 4);
    if (shape == 0)
        hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(workgroups), dim3(kProbeThreads), 0,
                           static_cast<hipStream_t>(stream), static_cast<const u4 *>(src), n16,
                           iters, out);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(workgroups), dim3(kProbeThreads), 0,
                           static_cast<hipStream_t>(stream), static_cast<const u4 *>(src), n16,
                           iters, out);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

extern "C" int w4a16_read_probe(const void *src, size_t bytes, uint32_t *out, void *stream)
{
    if (!src || !out || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15))
        return W4A16_EINVAL;
    w4a16_detail::DeviceInfo d;
    const int rc = w4a16_detail::current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeWGs), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u4 *>(src),
                       static_cast<uint64_t>(bytes / 16), out);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_EHIP;
}
