// Load-time conversion, on the GPU, of checkpoint-style packed 4-bit weights with their scales
// and zero points into the layout w4a16_gemm streams (w4a16_pack / w4a16_pack_zp's output).
//
// Marlin deep-dive page "Marlin 完全拆解": section "直接生成 MMA 所需的寄存器 fragment" (a
// checkpoint's packed tensor cannot be handed to the kernel as it is; it is converted into the
// kernel's layout while the weights are loaded), and the deployment section on checkpoint
// formats (formats labelled the same INT4 / group 128 differ in nibble order, scale arrangement
// and zero-point convention; the conversion only moves codes, it never changes one).
//
// The two source arrangements taken here are the two ways 8 codes can share a 32-bit word:
// eight consecutive rows of one column (packed along K) or eight consecutive columns of one
// row (packed along N, in a caller-given nibble order).  Zero points come packed along N.
//
// Every kernel is a pure bit move, bound by HBM: it reads K*N/2 bytes of codes and writes
// K*N/2, plus the scale and zero-point bytes.  Writes are whole 16-byte lane chunks of the
// output's 1 KiB blocks; reads are whole rows of a workgroup's tile.

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "w4a16.h"
#include "device.h"

namespace {

constexpr int kThreads = 256;

// Nibble of an output word that holds code i (rows 8r + i): 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ constexpr int out_nibble(int i) { return (i >> 1) + 4 * (i & 1); }

// Output word from eight codes, code i taken from nibble `pos` of v[i].
__device__ __forceinline__ uint32_t gather8(const uint32_t (&v)[8], int pos)
{
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o |= ((v[i] >> (4 * pos)) & 15u) << (4 * out_nibble(i));
    return o;
}

// Output word from one word holding rows 8r..8r+7 of a column (row 8r + i in nibble i).
__device__ __forceinline__ uint32_t reorder_rows(uint32_t v)
{
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o |= ((v >> (4 * i)) & 15u) << (4 * out_nibble(i));
    return o;
}

// Packed along K: source word (r, n) at r * N + n.  Output block (j, g) -- columns 16j..16j+15,
// rows 128g..128g+127 -- is 256 words at (j * G + g) * 256; lane l of the wave that writes it
// stores words 4l..4l+3: column 16j + l % 16, rows 128g + 32t + 8(l / 16) + 0..7 for t = 0..3,
// each one source word with its nibbles reordered.  A workgroup covers four adjacent slabs
// (one per wave) of one group, so every source row it reads is 256 contiguous bytes.
__global__ __launch_bounds__(kThreads) void repack_along_k_kernel(const uint32_t *__restrict__ src,
                                                                  uint32_t *__restrict__ out,
                                                                  int N, int G, int nj4)
{
    const int g = blockIdx.x / nj4;
    const int j = (blockIdx.x % nj4) * 4 + static_cast<int>(threadIdx.x) / 64;
    if (j >= N / 16)
        return;
    const int l = threadIdx.x % 64;
    const size_t n = 16 * static_cast<size_t>(j) + l % 16;
    uint4 w;
    uint32_t *wp = reinterpret_cast<uint32_t *>(&w);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const size_t r = 16 * static_cast<size_t>(g) + 4 * t + l / 16;     // 8-row block
        wp[t] = reorder_rows(src[r * N + n]);
    }
    reinterpret_cast<uint4 *>(out)[(static_cast<size_t>(j) * G + g) * 64 + l] = w;
}

// Packed along N: source word (k, c) at k * (N / 8) + c holds columns 8c..8c+7 of row k, the
// one at offset e in nibble pos(e) = (pos_of >> 4e) & 7.  An output word needs one nibble from
// each of 8 rows, so a workgroup takes a 128-row group by 256 columns (16 slabs): it reads the
// 128 x 32-word source tile row by row (128 contiguous bytes a row) and stores it in LDS
// transposed, one 128-word column per source word column, so that the 8 rows an output word
// needs are two 16-byte LDS reads.  Each wave then writes four of the 16 output blocks.
constexpr int kTileRows = 128;
constexpr int kTileWords = 32;                       // source words per tile row (256 columns)
constexpr int kLdsStride = kTileRows + 4;            // words per LDS column (16-byte aligned)

__global__ __launch_bounds__(kThreads) void repack_along_n_kernel(const uint32_t *__restrict__ src,
                                                                  uint32_t *__restrict__ out,
                                                                  int N, int G, int nj16,
                                                                  uint32_t pos_of)
{
    __shared__ __attribute__((aligned(16))) uint32_t tile[kTileWords * kLdsStride];
    const int g = blockIdx.x / nj16;
    const int tcol = blockIdx.x % nj16;              // 256-column tile
    const size_t NW = static_cast<size_t>(N) / 8;    // source words per row
    const size_t c0 = static_cast<size_t>(tcol) * kTileWords;
    const int tid = threadIdx.x;

    // 128 rows x 8 quads of 4 words: four passes of 256 quads.
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int q = pass * kThreads + tid;
        const int row = q / 8, cq = (q % 8) * 4;
        const size_t base = (static_cast<size_t>(kTileRows) * g + row) * NW + c0 + cq;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = c0 + cq + k < NW ? src[base + k] : 0u;
            tile[(cq + k) * kLdsStride + row] = v;
        }
    }
    __syncthreads();

    const int wave = tid / 64, l = tid % 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int jj = wave * 4 + s;                  // slab within the tile
        const int j = tcol * 16 + jj;
        if (j >= N / 16)
            break;                                    // whole wave; no barrier follows
        const int nl = 16 * jj + l % 16;              // column within the tile
        const int c = nl / 8;
        const int pos = static_cast<int>((pos_of >> (4 * (nl % 8))) & 7u);
        uint4 w;
        uint32_t *wp = reinterpret_cast<uint32_t *>(&w);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 *r = reinterpret_cast<const uint4 *>(tile + c * kLdsStride + 32 * t +
                                                             8 * (l / 16));
            const uint4 a = r[0], b = r[1];
            const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            wp[t] = gather8(v, pos);
        }
        reinterpret_cast<uint4 *>(out)[(static_cast<size_t>(j) * G + g) * 64 + l] = w;
    }
}

// Scales, and with zero points the zero terms 0x6400 | z, in the order the multiply reads
// them.  One thread per output half.  Without zero points half i is the scale of
// (slab group u, scale group g, column c, slab b) with i = ((u * Gs + g) * 16 + c) * Q + b;
// with them each (u, g, c) holds its Q scales and then its Q zero terms.  Column
// n = 16(uQ + b) + c.  Zero points: word (g, n / 8) of qzeros, nibble pos(n % 8).
__global__ __launch_bounds__(kThreads) void repack_params_kernel(
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros,
    uint16_t *__restrict__ out, int N, int Gs, int Q, uint32_t pos_of, size_t total)
{
    const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= total)
        return;
    const int per = qzeros ? 2 * Q : Q;
    const int h = static_cast<int>(i % per);
    size_t rest = i / per;
    const int c = static_cast<int>(rest % 16);
    rest /= 16;
    const int g = static_cast<int>(rest % Gs);
    const size_t u = rest / Gs;
    const size_t n = 16 * (u * Q + h % Q) + c;
    uint16_t v;
    if (h < Q) {
        v = scales[static_cast<size_t>(g) * N + n];
    } else {
        const uint32_t w = qzeros[static_cast<size_t>(g) * (N / 8) + n / 8];
        const int pos = static_cast<int>((pos_of >> (4 * (n % 8))) & 7u);
        v = static_cast<uint16_t>(0x6400u | ((w >> (4 * pos)) & 15u));
    }
    out[i] = v;
}

int slabs_per_scale_group(int N) { return N % 256 == 0 ? 4 : (N % 128 == 0 ? 2 : 1); }

}  // namespace

extern "C" int w4a16_repack(const uint32_t *qweight, int src_layout, const uint8_t *order,
                            const uint16_t *scales, const uint32_t *qzeros, int K, int N,
                            int group, uint32_t *packed_out, uint16_t *params_out, void *stream)
{
    if (!qweight || !scales || !packed_out || !params_out || K < 0 || N < 0)
        return W4A16_EINVAL;
    if (src_layout != W4A16_PACKED_ALONG_K && src_layout != W4A16_PACKED_ALONG_N)
        return W4A16_EINVAL;
    if ((reinterpret_cast<uintptr_t>(packed_out) & 15) ||
        (reinterpret_cast<uintptr_t>(qweight) & 3) || (reinterpret_cast<uintptr_t>(scales) & 1) ||
        (reinterpret_cast<uintptr_t>(params_out) & 1) ||
        (qzeros && (reinterpret_cast<uintptr_t>(qzeros) & 3)))
        return W4A16_EINVAL;
    // pos_of nibble e = the nibble that holds column offset e
    uint32_t pos_of = 0x76543210u;
    if (order) {
        pos_of = 0;
        unsigned seen = 0;
        for (int i = 0; i < 8; ++i) {
            if (order[i] > 7 || (seen >> order[i]) & 1u)
                return W4A16_EINVAL;
            seen |= 1u << order[i];
            pos_of |= static_cast<uint32_t>(i) << (4 * order[i]);
        }
    }
    if (K == 0 || N == 0 || K % W4A16_GROUP || N % 16 || (group != W4A16_GROUP && group != K))
        return W4A16_ESHAPE;
    const int G = K / W4A16_GROUP, Gs = K / group, Q = slabs_per_scale_group(N);
    const long long nj4 = (N / 16 + 3) / 4, nj16 = (N / 16 + 15) / 16;
    const long long blocks_w = static_cast<long long>(G) * (src_layout == W4A16_PACKED_ALONG_K ? nj4 : nj16);
    const size_t params = static_cast<size_t>(Gs) * N * (qzeros ? 2 : 1);
    const long long blocks_p = static_cast<long long>((params + kThreads - 1) / kThreads);
    if (blocks_w > INT_MAX || blocks_p > INT_MAX)
        return W4A16_ESHAPE;

    w4a16_detail::DeviceInfo d;
    const int rc = w4a16_detail::current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (src_layout == W4A16_PACKED_ALONG_K)
        repack_along_k_kernel<<<static_cast<int>(blocks_w), kThreads, 0, s>>>(
            qweight, packed_out, N, G, static_cast<int>(nj4));
    else
        repack_along_n_kernel<<<static_cast<int>(blocks_w), kThreads, 0, s>>>(
            qweight, packed_out, N, G, static_cast<int>(nj16), pos_of);
    if (hipGetLastError() != hipSuccess)
        return W4A16_EHIP;
    repack_params_kernel<<<static_cast<int>(blocks_p), kThreads, 0, s>>>(
        scales, qzeros, params_out, N, Gs, Q, pos_of, params);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_EHIP;
}
