// FP16 x INT4 (group-128) linear layer for CDNA4 (gfx950): C = A * Bhat,
// Bhat[k][n] = s[k/128][n] * (q[k][n] - 8), fp32 accumulation, fp16 output.
//
// Design (the pages' Ampere kernel is prior art; what carries over is kept, the rest is
// rebuilt for 64-lane waves, MFMA, LDS and a 256-CU chip):
//
// * Weight stream.  The packed codes (layout in w4a16.h) are read with one 128-bit
//   non-temporal load per lane per 128x16 block -- 1 KiB contiguous per wave -- straight into
//   the registers that feed the matrix cores; no fp16 copy of the weights exists anywhere.
//   Pages: MARLIN paper sec. 3.4 "Maximizing Loading Bandwidth" (widest loads, full lines,
//   weights read once with an evict-first hint).
// * Activations.  The A tile of each 128-row K step is loaded once per workgroup (one
//   16-byte chunk per thread per 16 rows) and staged in a three-stage LDS ring, XOR-swizzled
//   so stores and the 16-lane fragment reads are bank-conflict-free; all four waves read
//   their MFMA fragments from it.  A is re-read from L2 once per column slice, so wide
//   slices keep its traffic below the weight stream's (MARLIN paper sec. 3.4 "Bound By
//   Weight Loading", Eq. (1); "Shared Memory Layouts"; "Memory Load Pipelining").
// * Dequantisation.  One 32-bit word holds 8 codes; mask-and-OR into the fp16 exponent
//   0x6400 gives 1024 + q (low nibbles) or 1024 + 16q (high nibbles), and one packed fp16
//   add or FMA per pair returns q - 8 exactly.  Deep-dive page "Marlin 完全拆解", section
//   "INT4 只是存储类型，不是这条路径的计算类型".
// * Scales.  The MFMA sums A * (q - 8) over one 128-row group in fp32 (exact products);
//   that partial is multiplied by the group's scale and added to the running fp32 sum.
//   This is the grouped sum C = sum_g s_g sum_{k in g} A (q - 8) written out on the deep-dive
//   page (section "scale 为什么有时在内环乘，有时在末尾乘"); it costs 4 FMAs per 16x16
//   output tile per group instead of one fp16 multiply per weight.
// * Contraction: v_mfma_f32_16x16x32_f16, tokens as the 16 rows, output columns as the 16
//   columns; k-step loop outermost so independent accumulators separate dependent MFMAs
//   (MARLIN paper sec. 3.2 "Tensor Core Level").
// * Scheduling.  Tiles are 128 (K) x Nt (N) x Mt (M rows).  Tile order: column slice, then
//   64-row M sub-problem, then K (weights of a slice are re-read from cache for the next M
//   sub-problem: the pages' "virtual replication" of the weight grid for large M).  Each
//   workgroup takes one contiguous run of floor/ceil(T/W) tiles (a stripe), so every CU gets
//   the same work and only stripe ends split a slice.  Pages: deep-dive page sections
//   "为什么规则二维网格会浪费最后一波 SM" and "大 M 时虚拟复制权重网格"; MARLIN README
//   page, striped partitioning.  Workgroup ids are remapped so consecutive stripes sit on
//   the same XCD (the hardware deals workgroups round-robin over the 8 XCDs).
// * Cross-workgroup reduction.  Only the first and last slice of a stripe can be shared
//   with a neighbouring stripe.  At such a slice's end the workgroup writes its fp32 partial
//   tile to its own workspace slot with device-scope stores and streams on without
//   waiting.  After its last tile it waits once for its stores and bumps each shared
//   slice's counter; the contributor that draws the last count reads the partials back
//   with device-scope loads, adds them in stripe order (a fixed order, so results are
//   bitwise repeatable), writes C and resets the counter.  No cache-wide writeback or
//   invalidate is issued, and no workgroup ever waits for another.  The pages sum such partials serially with locks and stage them
//   in fp16 in the output (deep-dive page section "为什么归约串行，却不一定慢"); fp32
//   partials and a last-arriver sum keep the same "no big temporary" property, keep full
//   precision, and never spin, so no co-residency assumption is needed.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <algorithm>
#include <mutex>

#include "w4a16.h"

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                 // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kGroup = 128;                   // K rows per tile = one scale group
constexpr size_t kCounterBytes = 4096;        // fixed counter area at the workspace start
constexpr int kMaxWGs = static_cast<int>(kCounterBytes / sizeof(int));

struct Params {
    const uint16_t *A;        // fp16 [M][K]
    const u4 *packed;         // 16-byte quads, 64 per 128x16 block
    const uint16_t *scales;   // fp16 bits, 16 per block
    uint16_t *C;              // fp16 [M][N]
    int *counters;            // kMaxWGs ints, zero between calls
    float *partials;          // 2 * W slots of Mt*Nt floats
    int M, K, N;
    int G;                    // K / 128: tiles per slice
    int P;                    // M sub-problems of Mt rows
    int W;                    // workgroups = stripes
    long long T;              // total tiles = (N / Nt) * P * G
};

// (a & m) | o in one VALU op.  gfx9 VOP3 encodings take no literal and read at most one
// SGPR, so left to itself the compiler splits this into v_and + v_or; the "v" constraints
// keep both constants in (loop-invariant) VGPRs instead.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// 8 codes -> 8 fp16 values q - 8, in MFMA B-operand order (see pack.cpp for the nibbles).
// 9 VALU ops per 8 weights: 4 mask-and-OR, 1 shift, 2 packed adds, 2 packed FMAs.
__device__ __forceinline__ h8 dequant8(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic)
{
    const uint32_t w8 = w >> 8;
    const uint32_t x0 = and_or(w, mlo, magic);     // k0, k1: fp16 1024 + q
    const uint32_t x1 = and_or(w, mhi, magic);     // k2, k3: fp16 1024 + 16 q
    const uint32_t x2 = and_or(w8, mlo, magic);    // k4, k5
    const uint32_t x3 = and_or(w8, mhi, magic);    // k6, k7
    const h2 sub = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 mul = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const h2 add = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
    const h2 y0 = __builtin_bit_cast(h2, x0) - sub;                                // q - 8
    const h2 y1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x1), mul, add); // q - 8
    const h2 y2 = __builtin_bit_cast(h2, x2) - sub;
    const h2 y3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, x3), mul, add);
    h8 r;
    r[0] = y0[0]; r[1] = y0[1]; r[2] = y1[0]; r[3] = y1[1];
    r[4] = y2[0]; r[5] = y2[1]; r[6] = y3[0]; r[7] = y3[1];
    return r;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x)
{
    // v_cvt_f16_f32: one rounding, nearest-even in the default mode
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// First tile of stripe r, and the stripe that owns tile t (stripes are [r*T/W, (r+1)*T/W)).
__device__ __forceinline__ long long stripe_begin(long long r, long long T, int W)
{
    return r * T / W;
}
__device__ __forceinline__ int stripe_owner(long long t, long long T, int W)
{
    return static_cast<int>(((t + 1) * W - 1) / T);
}

template <int MB, int NBW>
struct Tile {
    static constexpr int Mt = 16 * MB;                 // rows per M sub-problem
    static constexpr int Nt = 16 * NBW * kWaves;       // columns per slice
    static constexpr int kStageQuads = MB * 256;       // 16-byte LDS chunks per A stage
    static constexpr int kStages = 3;                  // A ring depth (see the kernel loop)
    static constexpr int kSlotFloats = Mt * Nt;
};

// Raw buffer resources: base, size in bytes, gfx9 dword-access flags.  Loads past `bytes`
// return zero, which masks the rows of A beyond M for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr int kNonTemporal = 2;    // cache policy: streaming, evict first (weights, read once)
constexpr int kDeviceScope = 16;   // cache policy sc1: write through / read past the XCD's L2

// Where the next tile's loads come from.  Tiles run in (slice, M sub-problem, K) order;
// inside a slice only the K step changes and every offset moves by a constant.
struct LoadCursor {
    int g, pm, s;
    uint32_t wblk;      // block index of this wave's first slab at K step g (uniform)
    uint32_t a_soff;    // byte offset of K step g in an A row (uniform)
};

template <int MB, int NBW>
__device__ __forceinline__ void load_cursor_set(const Params &p, int wave, LoadCursor &c)
{
    c.wblk = (static_cast<uint32_t>(c.s) * (kWaves * NBW) + wave * NBW) * p.G + c.g;
    c.a_soff = static_cast<uint32_t>(c.g) * (kGroup * 2);
}

// The A tile of one K step (Mt rows x 128 k) is loaded by the whole workgroup, one 16-byte
// chunk per thread per 16-row sub-tile: thread `tid` takes row tid/16 and chunk tid%16
// (k = 8 * chunk .. +7).  Its byte offset in A for sub-problem row `arow`:
template <int MB>
__device__ __forceinline__ void a_thread_offsets(const Params &p, int tid, int arow,
                                                 uint32_t (&voff)[MB])
{
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        voff[mb] = (static_cast<uint32_t>(arow + 16 * mb + (tid >> 4)) * p.K + 8 * (tid & 15)) * 2;
}

// Global -> registers.  Rows at or past M fall outside the buffer and read as zero.
template <int MB>
__device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t rA, const uint32_t (&voff)[MB],
                                       uint32_t soff_in, u4 (&ar)[MB])
{
    const uint32_t soff = __builtin_amdgcn_readfirstlane(soff_in);   // uniform: keep in SGPR
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        ar[mb] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rA, voff[mb], soff, 0));
}

// Registers -> LDS stage, XOR-swizzled: chunk c of row i goes to position c ^ (i mod 16), so
// the 16 lanes that read one k-chunk of 16 different rows hit 16 different bank groups
// (MARLIN paper sec. 3.4 "Shared Memory Layouts": (i, j) -> (i, i XOR j)).  The stores are
// conflict-free too: the 16 threads of a row write a permutation of its 16 chunks.
template <int MB>
__device__ __forceinline__ void store_a(u4 *stage, int tid, const u4 (&ar)[MB])
{
    const int r = tid >> 4, c = tid & 15;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        stage[(16 * mb + r) * 16 + (c ^ r)] = ar[mb];
}

// This wave's packed weight quads (1 KiB contiguous per slab) and scales.  With 16-row
// tiles every weight byte is used once, so it is streamed non-temporally (evict first, the
// pages' evict_first hint).  Larger tiles re-read a slice's weights for the next 64-row
// sub-problem right away, and measure faster with the weights left in the cache.
template <int MB, int NBW>
__device__ __forceinline__ void load_w(__amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rS,
                                       int G, int lane, uint32_t wblk, u4 (&wq)[NBW],
                                       uint32_t (&sc)[NBW])
{
    constexpr int policy = MB == 1 ? kNonTemporal : 0;
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const uint32_t blk = __builtin_amdgcn_readfirstlane(wblk + static_cast<uint32_t>(b * G));
        wq[b] = __builtin_bit_cast(
            u4, __builtin_amdgcn_raw_buffer_load_b128(rW, lane * 16, blk * 1024u, policy));
        // the aligned dword holding this column's scale and its neighbour's (a 16-bit load
        // result would be re-copied across the loop back-edge)
        sc[b] = __builtin_amdgcn_raw_buffer_load_b32(rS, (lane & 14) * 2, blk * 32u, 0);
    }
}

// Where the group scale is applied.  Small tiles (MB <= 2) keep (q - 8) exact: the MFMA
// sums A * (q - 8) over the group in fp32 and the fp32 partial is scaled once per output
// (4 FMAs per 16x16 tile per group).  With 64 or more rows the per-tile FMAs and the partial
// registers cost more than scaling the weights: each dequantised pair is multiplied by the
// column's scale in fp16 (one packed multiply per two weights, the pages' own order:
// dequantise, scale, then MMA) and the MFMA accumulates straight into the output sum.  The
// rounding of s * (q - 8) to fp16 is below 2^-11 relative per weight.
template <int MB>
struct ScaleMode {
    static constexpr bool kWeights = MB >= 4;
};

template <int MB, int NBW>
__device__ __forceinline__ void compute_tile(const u4 *stage, int lane, const u4 (&wq)[NBW],
                                             const uint32_t (&sc)[NBW], f4 (&acc)[MB][NBW],
                                             uint32_t mlo, uint32_t mhi, uint32_t magic)
{
    // Scales first: converting them here ends the loaded registers' live range before the
    // next tile's loads reuse them (the empty asm keeps the conversion from being sunk).
    const int sshift = (lane & 1) * 16;               // odd columns: high half of the dword
    float sf[NBW];
    h8 s8[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        if constexpr (ScaleMode<MB>::kWeights) {
            const _Float16 sh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sc[b] >> sshift));
            s8[b] = h8{sh, sh, sh, sh, sh, sh, sh, sh};
            asm volatile("" : "+v"(s8[b]));
        } else {
            sf[b] = half_bits_to_float(static_cast<uint16_t>(sc[b] >> sshift));
            asm volatile("" : "+v"(sf[b]));
        }
    }
    // A fragments from LDS: row lane%16 of each sub-tile, k = 32t + 8(lane/16) .. +7.
    const int row = lane & 15, quad = lane >> 4;
    h8 a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            a[mb][t] = __builtin_bit_cast(h8, stage[(16 * mb + row) * 16 + ((4 * t + quad) ^ row)]);

    if constexpr (ScaleMode<MB>::kWeights) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const h8 bw = dequant8(wq[b][t], mlo, mhi, magic) * s8[b];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb][t], bw, acc[mb][b],
                                                                        0, 0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                asm volatile("" : "+v"(acc[mb][b]));    // finish the update here
        return;
    }

    f4 part[MB][NBW];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            const h8 bw = dequant8(wq[b][t], mlo, mhi, magic);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const f4 cin = (t == 0) ? f4{0.f, 0.f, 0.f, 0.f} : part[mb][b];
                part[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb][t], bw, cin, 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[mb][b][r] = __builtin_fmaf(sf[b], part[mb][b][r], acc[mb][b][r]);
            asm volatile("" : "+v"(acc[mb][b]));        // finish the update here
        }
}

// acc[mb][b][r] is C[row0 + 16mb + 4(lane/16) + r][col0 + 16b + lane%16].
template <int MB, int NBW>
__device__ __forceinline__ void write_c(const Params &p, int wave, int lane, long long sigma,
                                        const f4 (&acc)[MB][NBW])
{
    const long long s = sigma / p.P;
    const int pm = static_cast<int>(sigma - s * p.P);
    const int row0 = pm * 16 * MB + 4 * (lane >> 4);
    const size_t col0 = static_cast<size_t>(s) * Tile<MB, NBW>::Nt + wave * NBW * 16 + (lane & 15);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 16 * mb + r;
                if (row < p.M)
                    p.C[static_cast<size_t>(row) * p.N + col0 + 16 * b] =
                        float_to_half_bits(acc[mb][b][r]);
            }
}

// Byte offset of this lane's 16-byte piece of sub-tile (mb, b) in partial slot `slot` of
// stripe `stripe`.
template <int MB, int NBW>
__device__ __forceinline__ uint32_t slot_offset(int stripe, int slot, int wave, int mb, int b,
                                                int lane)
{
    return ((static_cast<uint32_t>(stripe) * 2 + slot) * Tile<MB, NBW>::kSlotFloats +
            ((wave * MB + mb) * NBW + b) * 256 + lane * 4) * 4;
}

// Partial tile of a split slice -> this stripe's workspace slot, with device-scope
// (write-through) stores.  Nothing waits here: the stores complete while streaming goes on.
template <int MB, int NBW>
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t rP, int stripe, int slot,
                                              int wave, int lane, const f4 (&acc)[MB][NBW])
{
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u4, acc[mb][b]), rP,
                slot_offset<MB, NBW>(stripe, slot, wave, mb, b, lane), 0, kDeviceScope);
}

// Sum the partials of split slice sigma in stripe order (a fixed order: results repeat bit
// for bit) and write C.  Partials are read past the L2 with device-scope loads.
template <int MB, int NBW>
__device__ __forceinline__ void reduce_slice(const Params &p, __amdgpu_buffer_rsrc_t rP,
                                             long long sigma, int w_lo, int w_hi, int wave,
                                             int lane)
{
    f4 sum[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
            sum[mb][b] = f4{0.f, 0.f, 0.f, 0.f};
    for (int w = w_lo; w <= w_hi; ++w) {
        const int slot = (sigma == stripe_begin(w, p.T, p.W) / p.G) ? 0 : 1;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int b = 0; b < NBW; ++b)
                sum[mb][b] += __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                    rP, slot_offset<MB, NBW>(w, slot, wave, mb, b, lane), 0, kDeviceScope));
    }
    write_c<MB, NBW>(p, wave, lane, sigma, sum);
}

// After the stripe's last tile: settle the (at most two) split slices it touched -- the
// first, which it may have entered part-way (slot 0), and the last, which it may have left
// part-way (slot 1).  part0 / part1 are those slices as recorded when their partials were
// stored, or -1.  Every wave waits for its own stores, the workgroup synchronises, and
// thread 0 counts this stripe in for each split slice with a device-scope atomic.  The
// stripe that draws the last count of a slice sums all its partials and writes C.  Nobody
// ever waits for another workgroup, so no co-residency is assumed.
//
// Visibility without cache-wide fences.  The XCDs' L2s are not coherent with each other,
// and a workgroup's XCD is not known in advance.  Partial slots are therefore only ever
// written with device-scope stores and read with device-scope loads -- the cache-policy
// encodings the compiler itself uses for device-scope atomic stores and loads, which must be
// coherent across XCDs.  A writer's stores have completed (s_waitcnt vmcnt(0)) before its
// counter increment is issued, and a reader issues its loads only after its own increment
// has returned the final count.  Each slot is written once per call and read once, after its
// write, and a slot owns whole cache lines, so no XCD can hold a stale copy made during the
// call; copies from earlier work do not survive the cache invalidation at kernel start.
// A release/acquire fence pair would add an L2 writeback and invalidate per workgroup;
// measured, that costs about a sixth of the runtime at M <= 16.
template <int MB, int NBW>
__device__ __forceinline__ void settle_split_slices(const Params &p, __amdgpu_buffer_rsrc_t rP,
                                                    long long part0, long long part1, int tid,
                                                    int *flag)
{
    if (part0 < 0 && part1 < 0)
        return;
    const int wave = tid >> 6, lane = tid & 63;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's partial stores are done
    __syncthreads();
    if (tid == 0) {
        if (part0 >= 0)
            flag[0] = __hip_atomic_fetch_add(p.counters + stripe_owner(part0 * p.G, p.T, p.W), 1,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (part1 >= 0)
            flag[1] = __hip_atomic_fetch_add(p.counters + stripe_owner(part1 * p.G, p.T, p.W), 1,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const long long sigma = i == 0 ? part0 : part1;
        if (sigma < 0)
            continue;
        const int w_lo = stripe_owner(sigma * p.G, p.T, p.W);
        const int w_hi = stripe_owner(sigma * p.G + p.G - 1, p.T, p.W);
        if (flag[i] != w_hi - w_lo)
            continue;               // another contributor is still running; it will finish
        reduce_slice<MB, NBW>(p, rP, sigma, w_lo, w_hi, wave, lane);
        if (tid == 0)
            __hip_atomic_store(p.counters + w_lo, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MB, int NBW>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(Params p)
{
    using TL = Tile<MB, NBW>;
    __shared__ u4 lds[TL::kStages * TL::kStageQuads];
    __shared__ int flag[2];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;

    // XCD-aware stripe id: hardware workgroup b runs on XCD b % 8; give each XCD a
    // contiguous block of stripes.
    int stripe = blockIdx.x;
    if ((p.W & 7) == 0)
        stripe = (blockIdx.x & 7) * (p.W >> 3) + (blockIdx.x >> 3);

    const long long t0 = stripe_begin(stripe, p.T, p.W);
    const long long t1 = stripe_begin(stripe + 1, p.T, p.W);
    if (t0 >= t1)
        return;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.K) * 2u);
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(p.packed, static_cast<uint32_t>(static_cast<size_t>(p.K) * p.N / 2));
    const __amdgpu_buffer_rsrc_t rS =
        make_rsrc(p.scales, static_cast<uint32_t>(static_cast<size_t>(p.G) * p.N * 2));
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(p.partials, static_cast<uint32_t>(2u * p.W * TL::kSlotFloats * 4u));

    // dequant constants in VGPRs for v_and_or_b32
    const uint32_t mlo = 0x000f000fu, mhi = 0x00f000f0u, magic = 0x64006400u;

    f4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
            acc[mb][b] = f4{0.f, 0.f, 0.f, 0.f};

    // Compute position: tile t, its K step g and slice sigma.
    long long t = t0;
    const long long sigma0 = t0 / p.G;           // the stripe's first slice
    long long sigma = sigma0;
    int g = static_cast<int>(t0 - sigma * p.G);
    long long part0 = -1, part1 = -1;            // split slices whose partials were stored

    // Load position, clamped to the stripe's last tile so every load is unconditional (a
    // re-read of the last tile is a cache hit).  A loads run two tiles ahead of the compute;
    // each A load is issued before the weight load of the same tile (see the schedule below).
    LoadCursor lc;
    lc.g = g;
    lc.s = static_cast<int>(sigma / p.P);
    lc.pm = static_cast<int>(sigma - static_cast<long long>(lc.s) * p.P);
    load_cursor_set<MB, NBW>(p, wave, lc);
    uint32_t a_voff[MB];
    a_thread_offsets<MB>(p, tid, lc.pm * 16 * MB, a_voff);
    long long lt = t0;                 // tile lc points at

    auto step_load = [&]() {
        if (lt + 1 < t1) {
            ++lt;
            ++lc.g;
            ++lc.wblk;
            lc.a_soff += kGroup * 2;
            if (lc.g == p.G) {         // next slice (uniform, rare)
                lc.g = 0;
                if (++lc.pm == p.P) {
                    lc.pm = 0;
                    ++lc.s;
                }
                load_cursor_set<MB, NBW>(p, wave, lc);
                a_thread_offsets<MB>(p, tid, lc.pm * 16 * MB, a_voff);
            }
        }
    };

    // Registers: weights double-buffered (tile i in buffer i % 2); A staged through `ar`
    // into a three-stage LDS ring (tile i in stage i % 3).  Per tile i the order is
    //   store A(i+1) -> stage (i+1) % 3, load A(i+2) -> ar, barrier, compute(i), load W(i+2).
    // Ring safety: the stage written at tile i was last read by compute(i-2), and no wave
    // passes barrier(i-1) before every wave has finished compute(i-2); the data stored at
    // tile i is visible to compute(i+1) through barrier(i).  (With two stages a fast wave
    // could overwrite the stage a slow wave is still reading.)
    // The vector-memory counter completes in order, and every A load is issued before the
    // weight load of the same tile, so waiting for A(i+1) never waits for a weight tile that
    // is not needed yet: each weight tile has one whole tile of compute to arrive in.
    u4 ar[MB];
    u4 wq0[NBW], wq1[NBW];
    uint32_t sc0[NBW], sc1[NBW];
    int st_cp = 0, st_st = 1;             // ring stages being computed from / stored to
    auto next_stage = [](int x) { return x == TL::kStages - 1 ? 0 : x + 1; };

    load_a<MB>(rA, a_voff, lc.a_soff, ar);                   // A(t0)
    load_w<MB, NBW>(rW, rS, p.G, lane, lc.wblk, wq0, sc0);        // W(t0)
    store_a<MB>(lds, tid, ar);                                // stage 0
    step_load();
    load_a<MB>(rA, a_voff, lc.a_soff, ar);                   // A(t0+1)
    load_w<MB, NBW>(rW, rS, p.G, lane, lc.wblk, wq1, sc1);        // W(t0+1)
    step_load();                                              // lc -> t0+2

    // End of a tile: at a slice's end, write C if this stripe owns the whole slice, else
    // leave its partial in the workspace for settle_split_slices.
    auto end_of_tile = [&]() {
        if (g == p.G - 1 || t + 1 == t1) {
            const long long s0 = sigma * p.G;
            if (t0 <= s0 && t == s0 + p.G - 1) {
                write_c<MB, NBW>(p, wave, lane, sigma, acc);
            } else if (sigma == sigma0) {
                store_partial<MB, NBW>(rP, stripe, 0, wave, lane, acc);
                part0 = sigma;
            } else {
                store_partial<MB, NBW>(rP, stripe, 1, wave, lane, acc);
                part1 = sigma;
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    acc[mb][b] = f4{0.f, 0.f, 0.f, 0.f};
        }
        ++t;
        if (++g == p.G) {
            g = 0;
            ++sigma;
        }
    };

    // Whole pairs of tiles per iteration; a single trailing tile is finished after the
    // loop.  Exiting only at the end of a pair keeps the control flow simple enough for the
    // compiler to wait for exactly one tile's loads.  A slice's end is handled before the
    // next weight tile is requested.  The asm/scheduling barriers keep each tile's loads
    // after the last use of the registers they overwrite.
    while (t + 1 < t1) {
        store_a<MB>(lds + st_st * TL::kStageQuads, tid, ar);  // A(t+1)
        load_a<MB>(rA, a_voff, lc.a_soff, ar);                // A(t+2)
        __syncthreads();
        compute_tile<MB, NBW>(lds + st_cp * TL::kStageQuads, lane, wq0, sc0, acc, mlo, mhi, magic);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        end_of_tile();
        load_w<MB, NBW>(rW, rS, p.G, lane, lc.wblk, wq0, sc0);    // W(t+2)
        step_load();
        st_cp = st_st;
        st_st = next_stage(st_st);

        store_a<MB>(lds + st_st * TL::kStageQuads, tid, ar);  // A(t+1)
        load_a<MB>(rA, a_voff, lc.a_soff, ar);                // A(t+2)
        __syncthreads();
        compute_tile<MB, NBW>(lds + st_cp * TL::kStageQuads, lane, wq1, sc1, acc, mlo, mhi, magic);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        end_of_tile();
        load_w<MB, NBW>(rW, rS, p.G, lane, lc.wblk, wq1, sc1);    // W(t+2)
        step_load();
        st_cp = st_st;
        st_st = next_stage(st_st);
    }
    if (t < t1) {
        __syncthreads();
        compute_tile<MB, NBW>(lds + st_cp * TL::kStageQuads, lane, wq0, sc0, acc, mlo, mhi, magic);
        end_of_tile();
    }
    settle_split_slices<MB, NBW>(p, rP, part0, part1, tid, flag);
}

// ------------------------------------------------------------------------------- host side

struct DeviceInfo {
    bool queried = false;
    bool gfx950 = false;
    int cus = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

int current_device(DeviceInfo *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return W4A16_EHIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.queried) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return W4A16_EHIP;
        const char *a = prop.gcnArchName;
        d.gfx950 = a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                   a[5] == '0' && (a[6] == '\0' || a[6] == ':');
        d.cus = prop.multiProcessorCount;
        d.queried = true;
    }
    *out = d;
    return d.gfx950 ? W4A16_OK : W4A16_EUNSUPPORTED;
}

struct Config {
    int MB, NBW;     // M sub-tiles of 16 rows; 16-column slabs per wave
    int P, S, G, W;
    long long T;
};

int check_gemm_shape(int M, int K, int N)
{
    if (M < 0 || K < 0 || N < 0)
        return W4A16_EINVAL;
    if (K == 0 || K % kGroup || N == 0 || N % W4A16_N_ALIGN)
        return W4A16_ESHAPE;
    // Buffer resources address at most 4 GiB; A offsets run up to 64 rows past M.
    const uint64_t lim = uint64_t(1) << 32;
    if ((static_cast<uint64_t>(M) + 64) * static_cast<uint64_t>(K) * 2 >= lim ||
        static_cast<uint64_t>(K) * static_cast<uint64_t>(N) / 2 >= lim)
        return W4A16_ESHAPE;
    return W4A16_OK;
}

// Number of stripes: a whole number of workgroups per CU, so every CU streams the same
// amount (a fractional count leaves some CUs with one workgroup more than others).  Two per
// CU measured best for every tile size.
int choose_stripes(long long T, int cus)
{
    long long w = static_cast<long long>(cus) * 2;
    if (w > kMaxWGs)
        w = kMaxWGs;
    if (w > T)
        w = T;
    return static_cast<int>(w);
}

Config choose_config(int M, int K, int N, int cus)
{
    Config c{};
    c.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const int Mt = 16 * c.MB;
    c.P = (M + Mt - 1) / Mt;
    c.G = K / kGroup;
    // widest slice (4 slabs per wave) that divides N
    c.NBW = 1;
    for (int nbw = 4; nbw >= 1; nbw >>= 1)
        if (N % (16 * kWaves * nbw) == 0) {
            c.NBW = nbw;
            break;
        }
    c.S = N / (16 * kWaves * c.NBW);
    c.T = static_cast<long long>(c.S) * c.P * c.G;
    c.W = choose_stripes(c.T, cus);
    return c;
}

size_t workspace_for(const Config &c)
{
    const size_t slot = static_cast<size_t>(16 * c.MB) * (16 * kWaves * c.NBW) * sizeof(float);
    return kCounterBytes + 2 * static_cast<size_t>(c.W) * slot;
}

template <int MB, int NBW>
hipError_t launch(const Params &p, hipStream_t stream)
{
    hipLaunchKernelGGL((w4a16_gemm_kernel<MB, NBW>), dim3(p.W), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

extern "C" int w4a16_workspace_size(int M, int K, int N, size_t *bytes)
{
    if (!bytes)
        return W4A16_EINVAL;
    int rc = check_gemm_shape(M, K, N);
    if (rc != W4A16_OK)
        return rc;
    DeviceInfo d;
    rc = current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    *bytes = M == 0 ? kCounterBytes : workspace_for(choose_config(M, K, N, d.cus));
    return W4A16_OK;
}

extern "C" int w4a16_gemm(const void *A, const uint32_t *packed, const uint16_t *scales, void *C,
                          int M, int K, int N, void *workspace, void *stream)
{
    if (!A || !packed || !scales || !C || !workspace)
        return W4A16_EINVAL;
    int rc = check_gemm_shape(M, K, N);
    if (rc != W4A16_OK)
        return rc;
    DeviceInfo d;
    rc = current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    if (M == 0)
        return W4A16_OK;

    const Config c = choose_config(M, K, N, d.cus);
    Params p;
    p.A = static_cast<const uint16_t *>(A);
    p.packed = reinterpret_cast<const u4 *>(packed);
    p.scales = scales;
    p.C = static_cast<uint16_t *>(C);
    p.counters = static_cast<int *>(workspace);
    p.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    p.M = M;
    p.K = K;
    p.N = N;
    p.G = c.G;
    p.P = c.P;
    p.W = c.W;
    p.T = c.T;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (c.MB * 10 + c.NBW) {
    case 11: e = launch<1, 1>(p, s); break;
    case 12: e = launch<1, 2>(p, s); break;
    case 14: e = launch<1, 4>(p, s); break;
    case 21: e = launch<2, 1>(p, s); break;
    case 22: e = launch<2, 2>(p, s); break;
    case 24: e = launch<2, 4>(p, s); break;
    case 41: e = launch<4, 1>(p, s); break;
    case 42: e = launch<4, 2>(p, s); break;
    case 44: e = launch<4, 4>(p, s); break;
    default: return W4A16_EHIP;
    }
    return e == hipSuccess ? W4A16_OK : W4A16_EHIP;
}
