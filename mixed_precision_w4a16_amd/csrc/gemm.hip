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
// * Scales.  With 16- and 32-row tiles the MFMA sums A * (q - 8) over one 128-row group in
//   fp32 (exact products) and that partial is multiplied by the group's scale and added to
//   the running fp32 sum: the grouped sum C = sum_g s_g sum_{k in g} A (q - 8) written out on
//   the deep-dive page (section "scale 为什么有时在内环乘，有时在末尾乘"), 4 FMAs per 16x16 output
//   tile per group.  With 64 or more rows a decoded fragment feeds enough MFMAs that scaling
//   the weights in fp16 (the pages' own order) is cheaper.
// * Contraction: v_mfma_f32_16x16x32_f16, tokens as the 16 rows, output columns as the 16
//   columns; k-step loop outermost so independent accumulators separate dependent MFMAs
//   (MARLIN paper sec. 3.2 "Tensor Core Level").
// * Scheduling.  Tiles are 128 (K) x Nt (N) x Mt (M rows).  Tile order: M sub-problem, then
//   column slice, then K (with several M sub-problems the weight grid is walked once per
//   sub-problem: the pages' "virtual replication" of the weight grid for large M).  Each
//   workgroup takes one contiguous run of floor/ceil(T/W) tiles (a stripe), so every CU gets
//   the same work and only stripe ends split a slice.  Pages: deep-dive page sections
//   "为什么规则二维网格会浪费最后一波 SM" and "大 M 时虚拟复制权重网格"; MARLIN README
//   page, striped partitioning.  Workgroup ids are remapped so consecutive stripes sit on
//   the same XCD (the hardware deals workgroups round-robin over the 8 XCDs), so each XCD
//   works on few M sub-problems at a time and their rows of A stay in its L2, while the
//   weights, read once per sub-problem, come from HBM or the memory-side cache (sub-problem
//   outermost measured 5-7% faster than slice outermost at M = 256..1024, which re-read all
//   of A per slice).
// * Cross-workgroup reduction.  Only the first and last slice of a stripe can be shared
//   with a neighbouring stripe.  A stripe that entered a slice part-way writes its fp32 piece
//   to its own workspace slot with device-scope stores and streams on without waiting; the
//   stripe holding the slice's first tiles (its owner, usually the last to finish it) keeps
//   its piece in registers.  After its last tile each stripe counts in once per shared slice;
//   exactly one contributor -- the owner if it arrives last -- sums the pieces in stripe order
//   (a fixed order, so results are bitwise repeatable), writes C and resets the counter.  No
//   cache-wide writeback or invalidate is issued, and no workgroup ever waits for another.
//   The pages sum such partials serially with locks and stage them in fp16 in the output
//   (deep-dive page section "为什么归约串行，却不一定慢"); fp32 partials and a last-arriver sum
//   keep the same "no big temporary" property, keep full precision, and never spin, so no
//   co-residency assumption is needed.
// * M > 64 runs a second kernel with 128-row tiles (w4a16_gemm_wide_kernel, further down):
//   every weight tile meets a whole 128-row block of A, A is brought into LDS by DMA.
// * M <= 16 runs a third kernel (w4a16_gemm_skinny_kernel, further down) on most shapes, and
//   M = 17..128 on weights of up to 7 (4 above 32 rows) slabs per CU: a workgroup owns a few 16-column slabs over
//   all of K (or over one of a few K splits) and its four waves split that range.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "w4a16.h"
#include "device.h"
#include "kernel_common.h"

namespace {

// Measurement-only builds, never the shipped library (build.py --ablation): the pages'
// Figure 12 ablations as they map onto these kernels.
//   W4A16_ABLATE_CACHED_WEIGHTS  weights loaded with the default cache policy, not streamed
//                                (the pages' evict_first off)
//   W4A16_ABLATE_SHALLOW         load pipelines one step shallower: the whole-K kernels keep
//                                one tile of registers instead of two, the stripe kernel's A
//                                ring has two stages instead of three (a second barrier per
//                                tile keeps it safe) (the pages' pipeline depth 4 -> 2)
//   W4A16_ABLATE_NO_SWIZZLE      A stored in LDS row-major, without the XOR swizzle
#ifdef W4A16_ABLATE_CACHED_WEIGHTS
constexpr int kWeightPolicy = 0;
#else
constexpr int kWeightPolicy = kNonTemporal;
#endif
#ifdef W4A16_ABLATE_SHALLOW
constexpr int kLoadDepth = 1;             // whole-K kernels: tiles of registers in flight
constexpr int kStripeStages = 2;          // stripe kernel: A ring stages
#else
constexpr int kLoadDepth = 2;
constexpr int kStripeStages = 3;
#endif
// LDS position of 16-byte chunk c of A row r
__device__ __forceinline__ int swz(int c, int r)
{
#ifdef W4A16_ABLATE_NO_SWIZZLE
    (void)r;
    return c;
#else
    return c ^ (r & 15);
#endif
}

constexpr size_t kCounterBytes = 4096;        // fixed counter area at the workspace start
constexpr int kMaxWGs = static_cast<int>(kCounterBytes / sizeof(int));

struct Params {
    const uint16_t *A;        // fp16 [M][K]
    const u4 *packed;         // 16-byte quads, 64 per 128x16 block
    const uint16_t *scales;   // fp16 bits: scales (and zero terms) in w4a16_pack(_zp) order
    uint16_t *C;              // fp16 [M][N]
    int *counters;            // kMaxWGs ints, zero between calls
    float *partials;          // 2 * W slots of Mt*Nt floats
    int M, K, N;
    int G;                    // K / 128: tiles per slice
    int Gs;                   // scale groups per column: G, or 1 for one scale per column
    int P;                    // M sub-problems of Mt rows
    int S;                    // column slices of Nt columns
    int gens;                 // workgroups resident per CU (1..3), for wave priorities
    int KS;                   // whole-K kernel: workgroups sharing one slab group's K range
    int Kq, Kr;               // ... and G = KS * Kq + Kr: split k gets Kq (+1 if k < Kr) tiles
    int SP;                   // whole-K kernel: row sub-problems of 16 * MB rows (grid z)
    int W;                    // workgroups = stripes
    long long T;              // total tiles = (N / Nt) * P * G
};

// Packed format: zero points (per group and column, else the fixed 8), where the scale
// sits (per 128-row group, or one per column applied once at the end), and whether the
// weights are 2:4-sparse along K (w4a16_pack_24: group-128 scales, z = 8).
template <bool ZP_, bool COL_, bool SP_ = false>
struct Fmt {
    static_assert(!SP_ || (!ZP_ && !COL_), "2:4-sparse weights have group scales and z = 8");
    static constexpr bool ZP = ZP_;
    static constexpr bool COL = COL_;
    static constexpr bool SP = SP_;
    // the K loop needs per-tile parameters unless the scale is per column and z is fixed
    static constexpr bool kTileParams = ZP_ || !COL_;
    // bytes of one 128 x 16 weight block and of one lane's share of it
    static constexpr uint32_t kBlockBytes = SP_ ? 768u : 1024u;
};
using FmtSym = Fmt<false, false>;
using FmtSp = Fmt<false, false, true>;

// Wave priority by dispatch order.  With several workgroups resident per CU, instruction
// arbitration favours the oldest waves, so a CU's workgroups run one after the other in
// effect and the last one streams alone at the end; giving later-dispatched workgroups a
// higher priority measured 3-6% faster on the whole-K kernels (72k x 18k: 110.0 -> 107.0 us
// at M = 1, 125.7 -> 117.0 us at M = 16).  Workgroup b of a grid dispatched in order is in
// dispatch round b * gens / W.
__device__ __forceinline__ void priority_by_dispatch_round(int gens)
{
    if (gens <= 1)
        return;
    const int round = static_cast<int>(blockIdx.x * static_cast<uint32_t>(gens) / gridDim.x);
    if (round == 1)
        __builtin_amdgcn_s_setprio(1);
    else if (round >= 2)
        __builtin_amdgcn_s_setprio(2);
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

template <int MB, int NBW, int WAVES = kWaves>
struct Tile {
    static constexpr int Mt = 16 * MB;                 // rows per M sub-problem
    static constexpr int Nt = 16 * NBW * WAVES;        // columns per slice
    static constexpr int kStageQuads = MB * 256;       // 16-byte LDS chunks per A stage
    static constexpr int kStages = kStripeStages;      // A ring depth (see the kernel loop)
    static constexpr int kSlotFloats = Mt * Nt;
};


// Where the next tile's loads come from.  Tiles run in (M sub-problem, slice, K) order;
// inside a slice only the K step changes and every offset moves by a constant.
struct LoadCursor {
    int g, pm, s;
    uint32_t wblk;      // block index of this wave's first slab at K step g (uniform)
    uint32_t sblk;      // index of this wave's scale group at K step g (uniform)
    uint32_t a_soff;    // byte offset of K step g in an A row (uniform)
};

template <int MB, int NBW, int WAVES = kWaves>
__device__ __forceinline__ void load_cursor_set(const Params &p, int wave, LoadCursor &c)
{
    c.wblk = (static_cast<uint32_t>(c.s) * (WAVES * NBW) + wave * NBW) * p.G + c.g;
    // with one scale per column (Gs = 1) the parameters stay at group 0 for the whole slice
    c.sblk = (static_cast<uint32_t>(c.s) * WAVES + wave) * p.Gs + (p.Gs == 1 ? 0 : c.g);
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
        stage[(16 * mb + r) * 16 + swz(c, r)] = ar[mb];
}

// Per-column parameters of a wave's NBW slabs at one K step (its "scale group" sblk):
// w4a16_pack stores the NBW scales of a column side by side, w4a16_pack_zp the NBW scales then
// the NBW zero terms (ZP), so one load per lane brings what a step needs: 2 NBW or 4 NBW bytes
// per column.  The symmetric format with NBW = 1 loads the aligned dword holding its column's
// scale and its neighbour's.  (A 16-bit load result would be re-copied across the loop
// back-edge.)  With one scale per column and zero points the K loop needs only the zero terms
// and the epilogue only the scales, so those loads bring just that part: a dword of a load
// whose value is never read would be handed to the next instruction that needs a register,
// and writing a register a load has not yet filled waits for every load in flight.
enum class Part { Scales, Both, Zeros };

template <int NBW, bool ZP, Part PT>
struct PRegs {
    static constexpr int n = PT == Part::Both ? NBW : (NBW >= 2 ? NBW / 2 : 1);
};

// What the K loop loads per step for format F (nothing, if kTileParams is false).
template <class F>
constexpr Part tile_part()
{
    return F::ZP ? (F::COL ? Part::Zeros : Part::Both) : Part::Scales;
}

template <int NBW, class F>
using TileRegs = PRegs<NBW, F::ZP, tile_part<F>()>;

template <int NBW, bool ZP, Part PT>
__device__ __forceinline__ void load_params(__amdgpu_buffer_rsrc_t rS, int lane, uint32_t sblk,
                                            uint32_t (&pr)[PRegs<NBW, ZP, PT>::n])
{
    static_assert(ZP || PT == Part::Scales, "the stream without zero points holds scales only");
    constexpr uint32_t per_group = 16u * 2u * (ZP ? 2 * NBW : (NBW >= 2 ? NBW : 1));
    const uint32_t so = __builtin_amdgcn_readfirstlane(sblk * per_group);
    constexpr int n = PRegs<NBW, ZP, PT>::n;                       // dwords per lane
    uint32_t off;
    if constexpr (ZP)      // column c at 4 NBW c bytes; its zero terms 2 NBW bytes further
        off = (lane & 15) * (4 * NBW) + (PT == Part::Zeros && NBW >= 2 ? 2 * NBW : 0);
    else if constexpr (NBW >= 2)
        off = (lane & 15) * (2 * NBW);
    else
        off = (lane & 14) * 2;
    if constexpr (n == 4) {
        const auto v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rS, off, so, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pr[i] = v[i];
    } else if constexpr (n == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rS, off, so, 0);
        pr[0] = v[0];
        pr[1] = v[1];
    } else {
        pr[0] = __builtin_amdgcn_raw_buffer_load_b32(rS, off, so, 0);
    }
}

// fp16 bits of slab b's scale for this lane's column (the scales come first in a load).
template <int NBW, bool ZP, Part PT>
__device__ __forceinline__ uint16_t scale_bits(const uint32_t (&pr)[PRegs<NBW, ZP, PT>::n],
                                               int b, int lane)
{
    static_assert(PT != Part::Zeros, "no scales in this load");
    if constexpr (ZP || NBW >= 2)
        return static_cast<uint16_t>(pr[b >> 1] >> ((b & 1) * 16));
    else
        return static_cast<uint16_t>(pr[0] >> ((lane & 1) * 16));
}

// Decode constants of slab b: (1024 + z, -(64 + z)) from the stored zero term, or those of
// z = 8.  The zero term is half NBW + b of a load of both parts, half b of a zero-term load
// (NBW >= 2), the upper half of the scale-and-zero dword (NBW = 1).
template <int NBW, bool ZP, Part PT>
__device__ __forceinline__ void zero_consts(const uint32_t (&pr)[PRegs<NBW, ZP, PT>::n], int b,
                                            h2 &zsub, h2 &zadd)
{
    if constexpr (ZP) {
        const int i = PT == Part::Both ? NBW + b : (NBW >= 2 ? b : 1);
        const _Float16 zt =
            __builtin_bit_cast(_Float16, static_cast<uint16_t>(pr[i >> 1] >> ((i & 1) * 16)));
        zsub = h2{zt, zt};
        const h2 k960 = {static_cast<_Float16>(960.0f), static_cast<_Float16>(960.0f)};
        zadd = k960 - zsub;
    } else {
        zsub = sym_zsub();
        zadd = sym_zadd();
    }
}

// This wave's packed weight quads (1 KiB contiguous per slab) and, if the format needs them
// per K step, its parameters.  ONCE: the call has one row sub-problem, so every weight byte
// is used once and is streamed non-temporally (evict first, the pages' evict_first hint),
// leaving the caches to A (72k x 18k weight: 4% faster at M = 64, 3% at M = 128).  With
// several row sub-problems a slice's weights are re-read right away and measure faster left
// in the cache (8192 x 28672 at M = 1024: 5% faster).
// A lane's share of one weight block: 16 bytes (8 codes of each of 4 32-k steps), or for
// 2:4-sparse weights 12 (the kept codes of the block's two 64-k steps and their positions).
template <class F>
using WQuad = std::conditional_t<F::SP, u3, u4>;

template <int MB, int NBW, class F, bool ONCE>
__device__ __forceinline__ void load_w(__amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rS,
                                       int G, int lane, uint32_t wblk, uint32_t sblk,
                                       WQuad<F> (&wq)[NBW], uint32_t (&pr)[TileRegs<NBW, F>::n])
{
    constexpr int policy = ONCE ? kWeightPolicy : 0;
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const uint32_t blk = __builtin_amdgcn_readfirstlane(wblk + static_cast<uint32_t>(b * G));
        if constexpr (F::SP)
            wq[b] = __builtin_bit_cast(
                u3, __builtin_amdgcn_raw_buffer_load_b96(rW, lane * 12, blk * F::kBlockBytes,
                                                         policy));
        else
            wq[b] = __builtin_bit_cast(
                u4, __builtin_amdgcn_raw_buffer_load_b128(rW, lane * 16, blk * F::kBlockBytes,
                                                          policy));
    }
    if constexpr (F::kTileParams)
        load_params<NBW, F::ZP, tile_part<F>()>(rS, lane, sblk, pr);
}

// Where the scale is applied.  One scale per column: not in the K loop at all; the fp32 sum
// of A * (q - z) over the whole K range is scaled once at the slice's end (slice_end), the
// pages' AB = (AQ) diag(s).  Per group, small tiles (MB <= 2) keep (q - z) exact: the MFMA
// sums A * (q - z) over the group in fp32 and the fp32 partial is scaled once per output
// (4 FMAs per 16x16 tile per group).  With 64 or more rows the per-tile FMAs and the partial
// registers cost more than scaling the weights: each decoded pair is multiplied by the
// column's scale in fp16 (one packed multiply per two weights, the pages' own order:
// dequantise, scale, then MMA) and the MFMA accumulates straight into the output sum.  The
// rounding of s * (q - z) to fp16 is below 2^-11 relative per weight.
template <int MB, class F>
struct ScaleMode {
    static constexpr bool kWeights = !F::COL && (MB >= 4 || F::SP);
    static constexpr bool kPartial = !F::COL && MB < 4 && !F::SP;
    // raw decode (raw8: no per-weight arithmetic) for the symmetric formats on 16- and 32-row
    // tiles: the tile's sums of A * raw codes and of A * offsets are formed by two chains in
    // the same order and subtracted, then scaled (per group) or added (one scale per column)
    static constexpr bool kRaw = !F::ZP && !F::SP && MB <= 2;
};

template <int MB, int NBW, class F>
__device__ __forceinline__ void compute_tile(const u4 *stage, int lane, const WQuad<F> (&wq)[NBW],
                                             const uint32_t (&pr)[TileRegs<NBW, F>::n],
                                             f4 (&acc)[MB][NBW], uint32_t mlo, uint32_t mhi,
                                             uint32_t magic, uint32_t magic_hi)
{
    // Parameters first: converting them here ends the loaded registers' live range before
    // the next tile's loads reuse them (the empty asm keeps the conversion from being sunk).
    float sf[NBW];
    h2 s2[NBW], zsub[NBW], zadd[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        if constexpr (ScaleMode<MB, F>::kWeights) {
            const _Float16 sh =
                __builtin_bit_cast(_Float16, scale_bits<NBW, F::ZP, tile_part<F>()>(pr, b, lane));
            s2[b] = h2{sh, sh};
            asm volatile("" : "+v"(s2[b]));
        } else if constexpr (ScaleMode<MB, F>::kPartial) {
            sf[b] = half_bits_to_float(scale_bits<NBW, F::ZP, tile_part<F>()>(pr, b, lane));
            asm volatile("" : "+v"(sf[b]));
        }
        zero_consts<NBW, F::ZP, tile_part<F>()>(pr, b, zsub[b], zadd[b]);
        if constexpr (F::ZP) {
            asm volatile("" : "+v"(zsub[b]));
            asm volatile("" : "+v"(zadd[b]));
        }
    }
    // A fragments from LDS: row lane%16 of each sub-tile, k = 32t + 8(lane/16) .. +7.
    const int row = lane & 15, quad = lane >> 4;
    h8 a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            a[mb][t] = __builtin_bit_cast(h8, stage[(16 * mb + row) * 16 + swz(4 * t + quad, row)]);

    if constexpr (ScaleMode<MB, F>::kRaw) {
        const h8 off = raw_offsets();
        f4 P[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                P[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    a[mb][t], off, t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : P[mb], 0, 0, 0);
        f4 D[MB][NBW];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const h8 x = raw8(wq[b][t], mlo, mhi, magic, magic_hi);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    D[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a[mb][t], x, t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : D[mb][b], 0, 0, 0);
            }
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const f4 part = D[mb][b] - P[mb];
                if constexpr (F::COL)
                    acc[mb][b] += part;
                else
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[mb][b][r] = __builtin_fmaf(sf[b], part[r], acc[mb][b][r]);
                asm volatile("" : "+v"(acc[mb][b]));    // finish the update here
            }
        return;
    } else if constexpr (F::SP) {
        // The transposed product on the sparse instruction (see the 2:4 kernel below): the
        // lane's decoded weights are the sparse operand (row = the lane's column), A fragments
        // 2h and 2h + 1 together are the dense operand of 64-k step h.
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            const h8 x0 = dequant8_scaled(wq[b][0], s2[b], mlo, mhi, magic, zsub[b], zadd[b]);
            const h8 x1 = dequant8_scaled(wq[b][1], s2[b], mlo, mhi, magic, zsub[b], zadd[b]);
            const int idx0 = static_cast<int>(wq[b][2]);
            const int idx1 = static_cast<int>(wq[b][2] >> 16);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const h16 d0 = __builtin_shufflevector(a[mb][0], a[mb][1], 0, 1, 2, 3, 4, 5, 6,
                                                       7, 8, 9, 10, 11, 12, 13, 14, 15);
                const h16 d1 = __builtin_shufflevector(a[mb][2], a[mb][3], 0, 1, 2, 3, 4, 5, 6,
                                                       7, 8, 9, 10, 11, 12, 13, 14, 15);
                acc[mb][b] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(x0, d0, acc[mb][b], idx0,
                                                                      0, 0);
                acc[mb][b] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(x1, d1, acc[mb][b], idx1,
                                                                      0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                asm volatile("" : "+v"(acc[mb][b]));    // finish the update here
        return;
    } else if constexpr (!ScaleMode<MB, F>::kPartial) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                h8 bw;
                if constexpr (ScaleMode<MB, F>::kWeights)
                    bw = dequant8_scaled(wq[b][t], s2[b], mlo, mhi, magic, zsub[b], zadd[b]);
                else
                    bw = dequant8(wq[b][t], mlo, mhi, magic, zsub[b], zadd[b]);
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
    } else {
        f4 part[MB][NBW];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const h8 bw = dequant8(wq[b][t], mlo, mhi, magic, zsub[b], zadd[b]);
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
                asm volatile("" : "+v"(acc[mb][b]));    // finish the update here
            }
    }
}


// acc[mb][b][r] is C[row0 + 16mb + 4(lane/16) + r][col0 + 16b + lane%16].  C is written
// through a buffer resource of exactly M * N * 2 bytes: stores to rows at or past M fall
// outside it and are dropped by the hardware, so no per-row test is needed.  The lane's own
// offset is one VGPR; the tile's position and the (mb, r) row are a running scalar offset and
// 16b columns an immediate.  TR: the transposed product of the 2:4-sparse weights, where
// acc[mb][b][r] is C[row0 + 16mb + lane%16][col0 + 16b + 4(lane/16) + r], 8 bytes a lane.
template <int MB, int NBW, int WAVES = kWaves, bool TR = false>
__device__ __forceinline__ void write_c(const Params &p, __amdgpu_buffer_rsrc_t rC, int wave,
                                        int lane, long long sigma, const f4 (&acc)[MB][NBW])
{
    const int pm = static_cast<int>(sigma / p.S);
    const long long s = sigma - static_cast<long long>(pm) * p.S;
    const uint32_t rowN = opaque(static_cast<uint32_t>(p.N) * 2);
    if constexpr (TR) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const uint32_t voff = ((lane & 15) * static_cast<uint32_t>(p.N) + wave * NBW * 16 +
                               4 * (lane >> 4)) * 2;
        uint32_t srow = __builtin_amdgcn_readfirstlane(
            (static_cast<uint32_t>(pm * 16 * MB) * static_cast<uint32_t>(p.N) +
             static_cast<uint32_t>(s) * Tile<MB, NBW, WAVES>::Nt) * 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const f4 v = acc[mb][b];
                const uint32_t lo = static_cast<uint32_t>(float_to_half_bits(v[0])) |
                                    (static_cast<uint32_t>(float_to_half_bits(v[1])) << 16);
                const uint32_t hi = static_cast<uint32_t>(float_to_half_bits(v[2])) |
                                    (static_cast<uint32_t>(float_to_half_bits(v[3])) << 16);
                __builtin_amdgcn_raw_buffer_store_b64(u2{lo, hi}, rC, voff + 32 * b, srow, 0);
            }
            srow += 16 * rowN;
        }
        return;
    }
    const uint32_t voff = ((4 * (lane >> 4)) * static_cast<uint32_t>(p.N) + wave * NBW * 16 +
                           (lane & 15)) * 2;
    uint32_t srow = __builtin_amdgcn_readfirstlane(
        (static_cast<uint32_t>(pm * 16 * MB) * static_cast<uint32_t>(p.N) +
         static_cast<uint32_t>(s) * Tile<MB, NBW, WAVES>::Nt) * 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int b = 0; b < NBW; ++b)
                __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(acc[mb][b][r]), rC,
                                                      voff + 32 * b, srow, 0);
            srow += rowN;
        }
        srow += 12 * rowN;             // the other three lane groups' rows of this 16-row block
    }
}

// Partial slot layout: slot `slot` of stripe `stripe` holds the workgroup's Mt x Nt fp32 tile
// as 16-byte pieces, piece (wave, mb, b, lane) at 16 * (((wave * MB + mb) * NBW + b) * 64 + lane).
// The 128-row tiles keep only the lane part in a vector register and compute the rest as a
// scalar offset where it is used (their vector registers are all taken by the accumulators);
// the smaller tiles keep whole offsets in vector registers, which measures faster there.
template <int MB, int NBW, int WAVES>
__device__ __forceinline__ uint32_t slot_base(int stripe, int slot, int wave, int mb, int b)
{
    return ((static_cast<uint32_t>(stripe) * 2 + slot) * Tile<MB, NBW, WAVES>::kSlotFloats +
            ((wave * MB + mb) * NBW + b) * 256) * 4;
}

template <int MB, int NBW, int WAVES>
__device__ __forceinline__ void slot_store(__amdgpu_buffer_rsrc_t rP, uint32_t sbase, int stripe,
                                           int slot, int wave, int mb, int b, int lane, f4 v)
{
    if constexpr (MB >= 8)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), rP, lane * 16,
                                               sbase + (mb * NBW + b) * 1024, kDeviceScope);
    else
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u4, v), rP,
            slot_base<MB, NBW, WAVES>(stripe, slot, wave, mb, b) + lane * 16, 0, kDeviceScope);
}

template <int MB, int NBW, int WAVES>
__device__ __forceinline__ f4 slot_load(__amdgpu_buffer_rsrc_t rP, uint32_t sbase, int stripe,
                                        int slot, int wave, int mb, int b, int lane)
{
    if constexpr (MB >= 8)
        return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rP, lane * 16, sbase + (mb * NBW + b) * 1024,
                                          kDeviceScope));
    else
        return __builtin_bit_cast(
            f4, __builtin_amdgcn_raw_buffer_load_b128(
                    rP, slot_base<MB, NBW, WAVES>(stripe, slot, wave, mb, b) + lane * 16, 0,
                    kDeviceScope));
}

// Scalar base of a wave's pieces in a slot (used by the 128-row tiles).
template <int MB, int NBW, int WAVES>
__device__ __forceinline__ uint32_t slot_sbase(int stripe, int slot, int wave)
{
    return opaque(__builtin_amdgcn_readfirstlane(slot_base<MB, NBW, WAVES>(stripe, slot, wave, 0, 0)));
}

// Partial tile of a split slice -> this stripe's workspace slot, with device-scope
// (write-through) stores.  Nothing waits here: the stores complete while streaming goes on.
template <int MB, int NBW, int WAVES = kWaves>
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t rP, int stripe, int slot,
                                              int wave, int lane, const f4 (&acc)[MB][NBW])
{
    const uint32_t sbase = MB >= 8 ? slot_sbase<MB, NBW, WAVES>(stripe, slot, wave) : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
            slot_store<MB, NBW, WAVES>(rP, sbase, stripe, slot, wave, mb, b, lane, acc[mb][b]);
}

// The partial slot stripe w used for split slice sigma: 0 if sigma is the slice the stripe
// starts in, else 1 (the slice it ends in).
__device__ __forceinline__ int slot_of(const Params &p, long long sigma, int w)
{
    return sigma == stripe_begin(w, p.T, p.W) / p.G ? 0 : 1;
}

// Sum the pieces of split slice sigma in stripe order w_lo .. w_hi (a fixed order: results
// repeat bit for bit) and write C.  The sum is formed in `acc`, which on entry either holds the
// first piece (the owner's own, kept in registers) or is free, and then gets the first piece
// from its slot like the others: either way the additions are the same.  Partials are read
// past the L2 with device-scope loads, half a tile at a time so that the loads in flight fit
// in the registers next to the sum (spilling would serialise them).
template <int MB, int NBW, int WAVES = kWaves, bool TR = false>
__device__ __forceinline__ void reduce_slice(const Params &p, __amdgpu_buffer_rsrc_t rP,
                                             __amdgpu_buffer_rsrc_t rC, long long sigma,
                                             int w_lo, int w_hi, int wave, int lane,
                                             bool first_in_regs, f4 (&acc)[MB][NBW])
{
    constexpr int H = MB >= 8 ? MB / 4 : (MB >= 2 ? MB / 2 : 1);   // row blocks per load round
    if (!first_in_regs) {
        const int slot = slot_of(p, sigma, w_lo);
        const uint32_t sbase = MB >= 8 ? slot_sbase<MB, NBW, WAVES>(w_lo, slot, wave) : 0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int b = 0; b < NBW; ++b)
                acc[mb][b] = slot_load<MB, NBW, WAVES>(rP, sbase, w_lo, slot, wave, mb, b, lane);
    }
    for (int w = w_lo + 1; w <= w_hi; ++w) {
        const int slot = slot_of(p, sigma, w);
        const uint32_t sbase = MB >= 8 ? slot_sbase<MB, NBW, WAVES>(w, slot, wave) : 0;
#pragma unroll
        for (int h = 0; h < MB; h += H) {
            f4 x[H][NBW];
#pragma unroll
            for (int mb = 0; mb < H; ++mb)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    x[mb][b] = slot_load<MB, NBW, WAVES>(rP, sbase, w, slot, wave, h + mb, b, lane);
#pragma unroll
            for (int mb = 0; mb < H; ++mb)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    acc[h + mb][b] += x[mb][b];
        }
    }
    write_c<MB, NBW, WAVES, TR>(p, rC, wave, lane, sigma, acc);
}

// End of a slice (or of the stripe) for the running accumulators.  With one scale per
// column the accumulators hold the sum of A * (q - z) over the stripe's K range; they are
// scaled here, once per output (pieces of a split slice are scaled before they are summed:
// the scale is the same for all of them).  Then three cases:
//  * the stripe computed the whole slice: write C;
//  * the stripe entered the slice part-way (so it is the slice it started in): store the
//    piece to slot 0 and record it in `nonown`;
//  * the stripe holds the slice's first tile but not its last (so this is its last tile):
//    it is the slice's owner and keeps its piece in the accumulators for settle().
template <int MB, int NBW, class F, int WAVES = kWaves>
__device__ __forceinline__ void slice_end(const Params &p, __amdgpu_buffer_rsrc_t rP,
                                          __amdgpu_buffer_rsrc_t rC, __amdgpu_buffer_rsrc_t rS,
                                          int stripe, long long t0, long long t, long long sigma,
                                          int wave, int lane, f4 (&acc)[MB][NBW],
                                          long long &nonown, long long &own)
{
    if constexpr (F::COL) {
        const long long sl = sigma % p.S;
        uint32_t pr[PRegs<NBW, F::ZP, Part::Scales>::n];
        load_params<NBW, F::ZP, Part::Scales>(rS, lane, static_cast<uint32_t>(sl) * WAVES + wave,
                                              pr);
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            const float sc =
                half_bits_to_float(scale_bits<NBW, F::ZP, Part::Scales>(pr, b, lane));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb][b] *= sc;
        }
    }
    const long long s0 = sigma * p.G;
    if (t0 <= s0 && t == s0 + p.G - 1) {
        write_c<MB, NBW, WAVES, F::SP>(p, rC, wave, lane, sigma, acc);
    } else if (t0 <= s0) {
        own = sigma;
    } else {
        store_partial<MB, NBW, WAVES>(rP, stripe, 0, wave, lane, acc);
        // The caller zeroes the accumulators next.  A 128-bit store reads its data registers
        // after it issues, and the compiler put the reset of the last stored fragment's first
        // register right behind its store with no wait states in between (seen in the ISA of
        // the 128-row kernel: element 0 of row block 7 then went out as zero now and then).
        // Wait states here keep the reset behind the stores' register reads.
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        nonown = sigma;
    }
}

// After the stripe's last tile: settle the (at most two) split slices it touched.  A split
// slice is shared by stripes w_lo .. w_hi; its owner w_lo holds the slice's first tiles, which
// come at the very end of w_lo's stripe, while the others entered the slice part-way and (all
// but the middle ones) finished their pieces early.  The owner is therefore usually the last
// to arrive, and it then sums the others' stored pieces with its own, which it never stores.
//
// Each slice has a counter (at counters[w_lo]): every other contributor adds 1 once its piece
// is stored; the owner adds kArrived when it arrives.  The owner sums at once if the other
// c - 1 pieces are all in; otherwise it stores its piece too and adds 1, and whoever brings
// the low count to c (owner or not) sums everything from the slots.  Exactly one contributor
// sums, it resets the counter, and nobody waits for another workgroup, so no co-residency is
// assumed.  Thread 0 does the counting; the result is broadcast through LDS.
//
// Visibility without cache-wide fences.  The XCDs' L2s are not coherent with each other,
// and a workgroup's XCD is not known in advance.  Partial slots are therefore only ever
// written with device-scope stores and read with device-scope loads -- the cache-policy
// encodings the compiler itself uses for device-scope atomic stores and loads, which must be
// coherent across XCDs.  A writer's stores have completed (s_waitcnt vmcnt(0)) before its
// counter increment is issued, and a reader issues its loads only after its own counter
// access has returned a value that includes every writer's increment.  Each slot is written
// at most once per call and read once, after its write, and a slot owns whole cache lines, so
// no XCD can hold a stale copy made during the call; copies from earlier work do not survive
// the cache invalidation at kernel start.  A release/acquire fence pair would add an L2
// writeback and invalidate per workgroup; measured, that costs about a sixth of the runtime
// at M <= 16.
constexpr int kArrived = 1 << 16;
constexpr int kCountMask = kArrived - 1;

template <int MB, int NBW, int WAVES = kWaves, bool TR = false>
__device__ __forceinline__ void settle(const Params &p, __amdgpu_buffer_rsrc_t rP,
                                       __amdgpu_buffer_rsrc_t rC, int stripe, long long nonown,
                                       long long own, int tid, f4 (&acc)[MB][NBW], int *flag)
{
    if (nonown < 0 && own < 0)
        return;
    const int wave = tid >> 6, lane = tid & 63;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's stores are done
    __syncthreads();
    if (tid == 0) {
        if (nonown >= 0)
            flag[0] = __hip_atomic_fetch_add(p.counters + stripe_owner(nonown * p.G, p.T, p.W), 1,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (own >= 0)
            flag[1] = __hip_atomic_fetch_add(p.counters + stripe, kArrived, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // The owned slice first: its piece is still in the accumulators, which are dead after.
    if (own >= 0) {
        const int w_hi = stripe_owner(own * p.G + p.G - 1, p.T, p.W);
        const int c = w_hi - stripe + 1;
        if ((flag[1] & kCountMask) == c - 1) {
            reduce_slice<MB, NBW, WAVES, TR>(p, rP, rC, own, stripe, w_hi, wave, lane, true, acc);
            if (tid == 0)
                __hip_atomic_store(p.counters + stripe, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            store_partial<MB, NBW, WAVES>(rP, stripe, slot_of(p, own, stripe), wave, lane, acc);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
                flag[1] = __hip_atomic_fetch_add(p.counters + stripe, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (((flag[1] + 1) & kCountMask) == c) {
                reduce_slice<MB, NBW, WAVES, TR>(p, rP, rC, own, stripe, w_hi, wave, lane, false, acc);
                if (tid == 0)
                    __hip_atomic_store(p.counters + stripe, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (nonown >= 0) {
        const int w_lo = stripe_owner(nonown * p.G, p.T, p.W);
        const int w_hi = stripe_owner(nonown * p.G + p.G - 1, p.T, p.W);
        const int v = flag[0] + 1;
        if ((v & kArrived) && (v & kCountMask) == w_hi - w_lo + 1) {
            reduce_slice<MB, NBW, WAVES, TR>(p, rP, rC, nonown, w_lo, w_hi, wave, lane, false, acc);
            if (tid == 0)
                __hip_atomic_store(p.counters + w_lo, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int MB, int NBW, class F, bool ONCE>
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
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(
        p.packed, static_cast<uint32_t>(static_cast<size_t>(p.K) * p.N * (F::SP ? 3 : 4) / 8));
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(
        p.scales, static_cast<uint32_t>(static_cast<size_t>(p.Gs) * p.N * (F::ZP ? 4 : 2)));
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(p.partials, static_cast<uint32_t>(2u * p.W * TL::kSlotFloats * 4u));
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.C, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.N) * 2u);

    // dequant constants in VGPRs for v_and_or_b32
    const uint32_t mlo = in_vgpr(0x000f000fu), mhi = in_vgpr(0x00f000f0u);
    const uint32_t magic = in_vgpr(0x64006400u);
    const uint32_t magic_hi = in_vgpr(0x54005400u);   // raw decode of the high nibbles

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
    long long nonown = -1, own = -1;             // split slices (see slice_end / settle)

    // Load position, clamped to the stripe's last tile so every load is unconditional (a
    // re-read of the last tile is a cache hit).  A loads run two tiles ahead of the compute;
    // each A load is issued before the weight load of the same tile (see the schedule below).
    LoadCursor lc;
    lc.g = g;
    lc.pm = static_cast<int>(sigma / p.S);
    lc.s = static_cast<int>(sigma - static_cast<long long>(lc.pm) * p.S);
    load_cursor_set<MB, NBW>(p, wave, lc);
    uint32_t a_voff[MB];
    a_thread_offsets<MB>(p, tid, lc.pm * 16 * MB, a_voff);
    long long lt = t0;                 // tile lc points at

    auto step_load = [&]() {
        if (lt + 1 < t1) {
            ++lt;
            ++lc.g;
            ++lc.wblk;
            if constexpr (!F::COL)
                ++lc.sblk;
            lc.a_soff += kGroup * 2;
            if (lc.g == p.G) {         // next slice (uniform, rare)
                lc.g = 0;
                if (++lc.s == p.S) {
                    lc.s = 0;
                    ++lc.pm;
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
    WQuad<F> wq0[NBW], wq1[NBW];
    uint32_t sc0[TileRegs<NBW, F>::n], sc1[TileRegs<NBW, F>::n];
    int st_cp = 0, st_st = 1;             // ring stages being computed from / stored to
    auto next_stage = [](int x) { return x == TL::kStages - 1 ? 0 : x + 1; };

    load_a<MB>(rA, a_voff, lc.a_soff, ar);                   // A(t0)
    load_w<MB, NBW, F, ONCE>(rW, rS, p.G, lane, lc.wblk, lc.sblk, wq0, sc0);        // W(t0)
    store_a<MB>(lds, tid, ar);                                // stage 0
    step_load();
    load_a<MB>(rA, a_voff, lc.a_soff, ar);                   // A(t0+1)
    load_w<MB, NBW, F, ONCE>(rW, rS, p.G, lane, lc.wblk, lc.sblk, wq1, sc1);        // W(t0+1)
    step_load();                                              // lc -> t0+2

    // End of a tile: at a slice's end, hand the accumulators to slice_end.  The stripe's last
    // piece is finished after the loop (it may be kept in the accumulators for settle).
    auto end_of_tile = [&]() {
        if (t + 1 == t1) {
            ++t;
            return;
        }
        if (g == p.G - 1) {
            slice_end<MB, NBW, F>(p, rP, rC, rS, stripe, t0, t, sigma, wave, lane, acc, nonown,
                                  own);
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
        if constexpr (TL::kStages == 2)
            __syncthreads();           // two stages: every wave is done with the one refilled
        store_a<MB>(lds + st_st * TL::kStageQuads, tid, ar);  // A(t+1)
        load_a<MB>(rA, a_voff, lc.a_soff, ar);                // A(t+2)
        __syncthreads();
        compute_tile<MB, NBW, F>(lds + st_cp * TL::kStageQuads, lane, wq0, sc0, acc, mlo, mhi, magic,
                                 magic_hi);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        end_of_tile();
        load_w<MB, NBW, F, ONCE>(rW, rS, p.G, lane, lc.wblk, lc.sblk, wq0, sc0);    // W(t+2)
        step_load();
        st_cp = st_st;
        st_st = next_stage(st_st);

        if constexpr (TL::kStages == 2)
            __syncthreads();
        store_a<MB>(lds + st_st * TL::kStageQuads, tid, ar);  // A(t+1)
        load_a<MB>(rA, a_voff, lc.a_soff, ar);                // A(t+2)
        __syncthreads();
        compute_tile<MB, NBW, F>(lds + st_cp * TL::kStageQuads, lane, wq1, sc1, acc, mlo, mhi, magic,
                                 magic_hi);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        end_of_tile();
        load_w<MB, NBW, F, ONCE>(rW, rS, p.G, lane, lc.wblk, lc.sblk, wq1, sc1);    // W(t+2)
        step_load();
        st_cp = st_st;
        st_st = next_stage(st_st);
    }
    if (t < t1) {
        __syncthreads();
        compute_tile<MB, NBW, F>(lds + st_cp * TL::kStageQuads, lane, wq0, sc0, acc, mlo, mhi, magic,
                                 magic_hi);
        end_of_tile();
    }
    slice_end<MB, NBW, F>(p, rP, rC, rS, stripe, t0, t1 - 1, sigma, wave, lane, acc, nonown, own);
    settle<MB, NBW, kWaves, F::SP>(p, rP, rC, stripe, nonown, own, tid, acc, flag);
}

// ------------------------------------------------------------------- wide tile, M >= 128
//
// Once every 128-row block of A meets a weight tile, the product is bound by the matrix
// cores, not by the weight stream (MARLIN paper sec. 3.2 and its Eq. (1): arithmetic
// intensity grows with the batch).  The cost to keep under the MFMA time is the dequantisation:
// 13 VALU ops (9 to decode, 4 to scale) per 8 weights of one B fragment.  That fragment feeds
// one 16x16x32 MFMA per 16 rows the wave covers, so each wave takes all 128 rows of the tile
// and 64 columns (8 x 4 accumulator tiles, 128 VGPRs): decode work is about 40% of the MFMA
// time and overlaps it.  The weights of a 128-row K step are still one 1 KiB load per slab per
// wave, straight into registers.
//
// A arrives by DMA: buffer loads that write LDS directly (no staging registers, no LDS store
// instructions), into a ring of 32 KiB stages (128 rows x 128 k).  A DMA writes 64 consecutive
// 16-byte LDS chunks, so the XOR swizzle of the ring is applied on the global side: the lane
// that fills LDS position p of row r fetches chunk p ^ (r mod 16) of that row.
//
// Four waves side by side in N make a 128 x 256 workgroup tile; two workgroups share a CU
// (2 x 64 KiB of LDS for a two-stage ring, at most 256 VGPRs per lane), so one workgroup's
// barrier and load waits are covered by the other's MFMAs.  A and the weights are fetched one
// tile ahead.  The kernel is written for any wave count and ring depth: an eight-wave,
// 128 x 512, three-stage variant (loads two tiles ahead, half the A traffic per FLOP) measured
// no faster, its extra weight buffers pushing the register allocator into spills.
//
// Measured (hardware counters, ablations): with the loads and the barrier removed the loop
// keeps the matrix cores about 80% busy; the loads cost the rest.  Neither the LDS reads, the
// dequantisation nor spreading the loads over the tile changes that.

constexpr int kWideMB = 8;
constexpr int kWideNBW = 4;

// A stage is filled by 32 DMAs of 4 rows each; wave w issues DMAs ND * w .. ND * w + ND - 1
// (ND = 32 / WAVES), DMA j filling stage rows 4j .. 4j + 3.  Lane l of DMA j fetches row
// r = 4j + l / 16 of the tile, chunk c = (l mod 16) ^ (r mod 16).  Since ND is a multiple of 4,
// r mod 16 = 4 (d mod 4) + l / 16 for the wave's d-th DMA: the lane-dependent part of the
// offset, l / 16 rows plus 16 c bytes, takes four values (d mod 4); the rest, the tile's first
// row, 4 (ND w + d) rows and the K step, is uniform.
// This wave's DMAs for one A stage: `rowoff` is the byte offset of the wave's first row (tile
// row + 4 ND w) plus the K step.  The four lane offsets are recomputed here from an opaque copy of the lane
// index (a few VALU ops): kept live across the main loop instead, they are the first values
// the register allocator spills, and every reload then waits for all outstanding loads.
template <int WAVES>
__device__ __forceinline__ void wide_dma_a(const Params &p, __amdgpu_buffer_rsrc_t rA, u4 *stage,
                                           int wave, int lane_in, uint32_t rowoff)
{
    constexpr int ND = 32 / WAVES;
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    uint32_t lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = swz(lane & 15, 4 * j + (lane >> 4));
        lo[j] = (static_cast<uint32_t>(lane >> 4) * p.K + 8 * c) * 2;
    }
    const uint32_t row4 = static_cast<uint32_t>(p.K) * 8;         // 4 rows, in bytes
#pragma unroll
    for (int d = 0; d < ND; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void *)(stage + (ND * wave + d) * 64), 16,
            lo[d & 3], __builtin_amdgcn_readfirstlane(rowoff + d * row4), 0, 0);
}

// One 128-row K step of the wave's 128 x 64 output block.  Per 32-k MFMA step the four B
// fragments are decoded (and, with per-group scales, scaled) first; then each A fragment
// (row block mb) is read from LDS once and used by four MFMAs.
template <class F>
__device__ __forceinline__ void wide_compute(const u4 *stage, int lane,
                                             const u4 (&wq)[kWideNBW],
                                             const uint32_t (&pr)[TileRegs<kWideNBW, F>::n],
                                             f4 (&acc)[kWideMB][kWideNBW], uint32_t mlo,
                                             uint32_t mhi, uint32_t magic)
{
    h2 s2[kWideNBW], zsub[kWideNBW], zadd[kWideNBW];
#pragma unroll
    for (int b = 0; b < kWideNBW; ++b) {
        if constexpr (!F::COL) {
            const _Float16 sh =
                __builtin_bit_cast(_Float16,
                                   scale_bits<kWideNBW, F::ZP, tile_part<F>()>(pr, b, lane));
            s2[b] = h2{sh, sh};
            asm volatile("" : "+v"(s2[b]));
        }
        zero_consts<kWideNBW, F::ZP, tile_part<F>()>(pr, b, zsub[b], zadd[b]);
        if constexpr (F::ZP) {
            asm volatile("" : "+v"(zsub[b]));
            asm volatile("" : "+v"(zadd[b]));
        }
    }
    const int row = lane & 15, quad = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        h8 bw[kWideNBW];
#pragma unroll
        for (int b = 0; b < kWideNBW; ++b) {
            if constexpr (F::COL)
                bw[b] = dequant8(wq[b][t], mlo, mhi, magic, zsub[b], zadd[b]);
            else
                bw[b] = dequant8_scaled(wq[b][t], s2[b], mlo, mhi, magic, zsub[b], zadd[b]);
        }
#pragma unroll
        for (int mb = 0; mb < kWideMB; ++mb) {
            const h8 a = __builtin_bit_cast(h8, stage[(16 * mb + row) * 16 + swz(4 * t + quad, row)]);
#pragma unroll
            for (int b = 0; b < kWideNBW; ++b)
                acc[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[b], acc[mb][b], 0, 0, 0);
        }
    }
}

// s_waitcnt immediate for "vmcnt(n)" alone (lgkmcnt and expcnt left at their maxima).
constexpr int vmcnt_imm(int n)
{
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

template <int WAVES, int STAGES, class F, bool ONCE>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void w4a16_gemm_wide_kernel(Params p)
{
    using TL = Tile<kWideMB, kWideNBW, WAVES>;
    constexpr int MB = kWideMB, NBW = kWideNBW;
    constexpr int ND = 32 / WAVES;             // A DMAs per wave per tile
    constexpr int NW = NBW + (F::kTileParams ? 1 : 0);   // weight + parameter loads per tile
    // The stages are separate arrays: with distinct objects the compiler can tell that the
    // reads of one stage do not depend on a DMA into another (it waits for pending LDS DMA
    // before any LDS read that may alias it).
    __shared__ u4 st0[TL::kStageQuads];
    __shared__ u4 st1[TL::kStageQuads];
    __shared__ u4 st2[STAGES > 2 ? TL::kStageQuads : 1];
    __shared__ int flag[2];
    auto stage = [&](auto k) __attribute__((always_inline)) -> u4 * {
        if constexpr (decltype(k)::value == 0) return st0;
        else if constexpr (decltype(k)::value == 1) return st1;
        else return st2;
    };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;

    int stripe = blockIdx.x;
    if ((p.W & 7) == 0)
        stripe = (blockIdx.x & 7) * (p.W >> 3) + (blockIdx.x >> 3);
    const long long t0 = stripe_begin(stripe, p.T, p.W);
    const long long t1 = stripe_begin(stripe + 1, p.T, p.W);
    if (t0 >= t1)
        return;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.K) * 2u);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(
        p.packed, static_cast<uint32_t>(static_cast<size_t>(p.K) * p.N * (F::SP ? 3 : 4) / 8));
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(
        p.scales, static_cast<uint32_t>(static_cast<size_t>(p.Gs) * p.N * (F::ZP ? 4 : 2)));
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(p.partials, static_cast<uint32_t>(2u * p.W * TL::kSlotFloats * 4u));
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.C, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.N) * 2u);
    const uint32_t mlo = in_vgpr(0x000f000fu), mhi = in_vgpr(0x00f000f0u);
    const uint32_t magic = in_vgpr(0x64006400u);

    f4 acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
            acc[mb][b] = f4{0.f, 0.f, 0.f, 0.f};

    long long t = t0;
    long long sigma = t0 / p.G;
    int g = static_cast<int>(t0 - sigma * p.G);
    long long nonown = -1, own = -1;

    // Load position, clamped to the stripe's last tile so that every tile issues the same
    // loads (the last tiles re-read their own data into idle buffers).  A branch around the
    // loads would leave the compiler's waits at the join assuming no loads were issued,
    // i.e. waiting for everything.
    LoadCursor lc;
    lc.g = g;
    lc.pm = static_cast<int>(sigma / p.S);
    lc.s = static_cast<int>(sigma - static_cast<long long>(lc.pm) * p.S);
    load_cursor_set<MB, NBW, WAVES>(p, wave, lc);
    // byte offset of the wave's first A row at the load position's K step (uniform)
    auto a_rowoff = [&]() __attribute__((always_inline)) {
        return (static_cast<uint32_t>(lc.pm * TL::Mt + 4 * ND * wave) * p.K) * 2 + lc.a_soff;
    };
    long long lt = t0;

    auto advance = [&]() __attribute__((always_inline)) {
        if (lt + 1 < t1) {
            ++lt;
            ++lc.g;
            ++lc.wblk;
            if constexpr (!F::COL)
                ++lc.sblk;
            lc.a_soff += kGroup * 2;
            if (lc.g == p.G) {
                lc.g = 0;
                if (++lc.s == p.S) {
                    lc.s = 0;
                    ++lc.pm;
                }
                load_cursor_set<MB, NBW, WAVES>(p, wave, lc);
            }
        }
    };

    // Weight buffers, one per stage: tile i uses stage and buffer i % STAGES.
    u4 wq[STAGES][NBW];
    uint32_t sc[STAGES][TileRegs<NBW, F>::n];

    // Issue the loads of the tile at the load position into stage / buffer k, the DMAs first
    // (the asm and scheduling barriers keep that order), and move the cursor on.
    auto issue = [&](auto k) __attribute__((always_inline)) {
        constexpr int K = decltype(k)::value;
        wide_dma_a<WAVES>(p, rA, stage(k), wave, lane, a_rowoff());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_w<MB, NBW, F, ONCE>(rW, rS, p.G, lane, lc.wblk, lc.sblk, wq[K], sc[K]);
        advance();
    };

    auto end_of_tile = [&]() __attribute__((always_inline)) {
        if (t + 1 == t1) {
            ++t;
            return;
        }
        if (g == p.G - 1) {
            slice_end<MB, NBW, F, WAVES>(p, rP, rC, rS, stripe, t0, t, sigma, wave, lane, acc,
                                         nonown, own);
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

    // Tile i (phase k = i % STAGES): wait until A(i) has landed, barrier, issue the loads of
    // tile i + STAGES - 1 into the stage / buffer that tile i - 1 used, compute tile i.
    // A(i) was issued STAGES - 1 tiles ago; every tile issues ND DMAs then NW weight loads,
    // and the vector-memory counter completes in order, so A(i) has landed once at most
    // NW + (STAGES - 2) * (ND + NW) operations are outstanding (stores issued since only make
    // the wait stricter).  The barrier then makes A(i) visible to every wave, and the stage
    // about to be refilled was last read by compute(i - 1), which every wave has finished
    // before it reaches the barrier.
    constexpr int kWaitA = NW + (STAGES - 2) * (ND + NW);
    auto tile = [&](auto k) __attribute__((always_inline)) {
        constexpr int K = decltype(k)::value;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitA));
        __syncthreads();
        issue(std::integral_constant<int, (K + STAGES - 1) % STAGES>{});
        wide_compute<F>(stage(k), lane, wq[K], sc[K], acc, mlo, mhi, magic);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        end_of_tile();
    };

    issue(std::integral_constant<int, 0>{});
    if constexpr (STAGES > 2)
        issue(std::integral_constant<int, 1>{});

    // Whole rounds of STAGES tiles (phases 0 .. STAGES-1), then up to STAGES - 1 more.
    while (t + STAGES - 1 < t1) {
        tile(std::integral_constant<int, 0>{});
        tile(std::integral_constant<int, 1>{});
        if constexpr (STAGES > 2)
            tile(std::integral_constant<int, 2>{});
    }
    if (t < t1)
        tile(std::integral_constant<int, 0>{});
    if constexpr (STAGES > 2)
        if (t < t1)
            tile(std::integral_constant<int, 1>{});
    // The last tiles' re-read DMAs may still be writing LDS: let them land before the
    // workgroup's LDS can be handed to another workgroup.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    slice_end<MB, NBW, F, WAVES>(p, rP, rC, rS, stripe, t0, t1 - 1, sigma, wave, lane, acc, nonown,
                                 own);
    settle<MB, NBW, WAVES>(p, rP, rC, stripe, nonown, own, tid, acc, flag);
}

// ------------------------------------------------------------------------- skinny kernel
//
// `w4a16_gemm_skinny_kernel<MB, NS, F>`, MB 16-row blocks (M <= 16; M = 17..32 on weights of
// up to seven slabs per CU and M = 33..128 on weights of up to four, as two 64-row
// sub-problems above 64 rows (grid z), where one workgroup per CU leaves registers to spare), N
// a multiple of 256.  Each decoded weight fragment feeds MB
// matrix instructions.  The weight stream bounds
// the product, and the stripe scheme's split slices cost a store, a counter and a read at the
// very end, when every stripe finishes at once (on small weights that chain is most of the
// time).  Here a workgroup owns NS consecutive 16-column slabs over the whole K range, so no
// output is shared between workgroups.  Its four waves split the K tiles into four contiguous
// runs; each streams all NS slabs over its run (NS KiB of weights per tile in two register
// buffers; three at M <= 8 on small weights, one in the 32-row form at two workgroups per CU),
// and the four fp32 partial sums meet in LDS at the end in a fixed order (the in-block
// reduction of warp partial sums the deep-dive page describes in "让多个 warp 计算同一个输出
// tile 的部分和").  A needs no LDS: each wave loads its A fragments (16 bytes per lane per 32-k
// step) straight into the MFMA operand registers, rows at or past M falling outside the buffer
// (zero, no memory access).  No per-tile barrier.
//
// Split K (p.KS > 1), for weights with too few slab groups to give every CU work: the grid's
// second dimension is the split (the third, above 64 rows, the 64-row sub-problem), and the
// KS workgroups (x, 0 .. KS - 1, z) share slab group x of sub-problem z, each taking a
// contiguous 1/KS of the K tiles.  Each stores its fp32 sums as one piece (device-scope
// stores, a 1 KiB slot per slab and row block), counts in on the group's counter, and the
// last to arrive sums the KS pieces in split order -- a fixed
// order, so results repeat bit for bit -- scales, writes C and resets the counter, the
// protocol of the stripe kernel's split slices (see settle()).  Nobody waits for another
// workgroup.
//
// Parameters: with N a multiple of 256 the parameter stream groups four slabs, so per K step a
// column holds 4 scales (and 4 zero terms) of a group in 8 (16) contiguous bytes.  A
// workgroup's NS slabs start at j0 and touch at most (NS + 6) / 4 groups; one load per group
// brings the lane's column, and the halves of slabs j0 .. j0 + NS - 1 are picked out by two
// uniform selects per dword (j0 % 4 is the same for the whole workgroup).
//
// The tiles after a wave's run are still "loaded" (every iteration issues the same loads),
// from an offset outside every buffer (kOutside): no memory traffic, and the compiler never meets a join
// where it would have to wait for everything.

constexpr int kSkinnyMaxKS = 8;            // split-K pieces summed in one load round
constexpr int kTrRowBlock = 16 * 17;       // 16-byte LDS chunks of one transposed row block

template <int NS>
struct SkinnyGroups {
    static constexpr int n = (NS + 6) / 4;   // parameter groups NS slabs can touch
    static constexpr int nh = (NS + 1) / 2;  // dwords holding NS halves
};

template <int MB, int NS, class F, bool DM = false>
struct SkinnyBuf {
    u4 w[NS];                                // weight quads, one per slab
    h8 a[DM ? 1 : MB][DM ? 1 : 4];           // A of the 4 32-k steps per row block (not DM)
    uint32_t p[F::COL ? 1 : SkinnyGroups<NS>::n][F::ZP ? 4 : 2];   // per-group parameters
};

// TWO: 32 rows at two workgroups per CU (weights of more than seven slabs per CU, symmetric
// formats): the raw-decode chains are then formed one slab at a time, so that only one slab's
// sums are live beside the running ones and the registers fit 256 per lane.
template <int MB, int NS, class F, bool TWO = false, int DEPTH = kLoadDepth, bool FL = false,
          bool DM = false>
__global__ __launch_bounds__(kThreads, (MB == 1 || TWO) ? 2 : 1) void w4a16_gemm_skinny_kernel(
    Params p)
{
    using SG = SkinnyGroups<NS>;
    using Buf = SkinnyBuf<MB, NS, F, DM>;
    constexpr int NG = SG::n, NH = SG::nh;
    constexpr uint32_t PB = F::ZP ? 16 : 8;              // bytes per column, group and K step
    static_assert(!DM || FL, "the DMA form loads whole lines");
    // DM: each wave's A tiles arrive by DMA into its own LDS buffers (DEPTH of them, one per
    // register buffer), which the partial sums (red) reuse after the K loop
    constexpr int kRed = kWaves * NS * 64, kDma = DM ? kWaves * DEPTH * MB * 256 : 0;
    __shared__ u4 smem[kRed > kDma ? kRed : kDma];
    f4 *red = reinterpret_cast<f4 *>(smem);
    __shared__ u4 atr[(FL && !DM) ? kWaves * MB * kTrRowBlock : 1];   // per-wave A transposes
    priority_by_dispatch_round(p.gens);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15;
    const int S = p.N >> 4;                              // slabs
    const int U = S >> 2;                                // parameter groups
    const int KS = p.KS;
    const int jg = blockIdx.x;                           // slab group
    const int ks = blockIdx.y;                           // its K split
    const int row0 = static_cast<int>(blockIdx.z) * 16 * MB;   // its row sub-problem
    const int grp = static_cast<int>(blockIdx.z * gridDim.x + blockIdx.x);  // counter, pieces
    const int j0 = jg * NS;                              // the workgroup's first slab
    const int u0 = j0 >> 2, r = j0 & 3;
    const int gk0 = ks * p.Kq + (ks < p.Kr ? ks : p.Kr);            // the split's K tiles
    const int gk1 = gk0 + p.Kq + (ks < p.Kr ? 1 : 0);
    const int g0 = gk0 + (gk1 - gk0) * wave / kWaves;    // this wave's run of them
    const int g1 = gk0 + (gk1 - gk0) * (wave + 1) / kWaves;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.K) * 2u);
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(p.packed, static_cast<uint32_t>(static_cast<size_t>(p.K) * p.N / 2));
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(
        p.scales, static_cast<uint32_t>(static_cast<size_t>(p.Gs) * p.N * (F::ZP ? 4 : 2)));
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.C, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.N) * 2u);

    const uint32_t mlo = in_vgpr(0x000f000fu), mhi = in_vgpr(0x00f000f0u);
    const uint32_t magic = in_vgpr(0x64006400u);
    const uint32_t magic_hi = in_vgpr(0x54005400u);   // raw decode of the high nibbles

    // byte offset of parameter block (group u, scale group gs); the lane's column adds c * PB
    auto par_soff = [&](int u, int gs) __attribute__((always_inline)) {
        return (static_cast<uint32_t>(u) * p.Gs + gs) * (16u * PB);
    };
    const uint32_t v_par = static_cast<uint32_t>(c) * PB;
    // A operand of row block mb: row 16 mb + c, k = 8 * (lane / 16) of each 32-k step.  FL:
    // the load of step t brings rows 4t .. 4t + 3 of the block instead, 16 lanes a row, 16
    // bytes each: whole 128-byte lines (the fragment layout touches 16 rows of 64 bytes, half
    // of 16 lines, per load, and the vector L1 is the bottleneck of those loads once A has
    // real rows: its address path stalls for more than half of its busy cycles at M = 16 and
    // 32); the wave puts them in fragment order through its own LDS region (compute).  DM:
    // the same lines by DMA straight into the wave's LDS buffer of the tile, no registers in
    // flight and no LDS stores (the nine-slab 32-row form and four row blocks, where the
    // registers are the limit).
    uint32_t v_a[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        v_a[mb] = FL ? (static_cast<uint32_t>(row0 + 16 * mb + (lane >> 4)) * p.K + 8 * c) * 2
                     : (static_cast<uint32_t>(row0 + 16 * mb + c) * p.K + 8 * (lane >> 4)) * 2;
    const uint32_t rows4 = static_cast<uint32_t>(p.K) * 8;      // 4 rows of A, in bytes
    auto slab = [&](int i) __attribute__((always_inline)) {
        const int j = j0 + i;
        return j < S ? j : S - 1;          // slabs past N re-read the last one; never stored
    };

    // DM: lane (rq, p) of the load of step t fetches chunk p ^ r of row r = 4t + rq of the
    // block (the XOR swizzle applied on the global side: a DMA writes 64 consecutive chunks),
    // so the 16 rows read at one chunk lie in 16 bank groups
    const uint32_t cx16 = static_cast<uint32_t>(c ^ (lane >> 4)) * 16;
    u4 *const dma_base = smem + wave * (DEPTH * MB * 256);
    auto load = [&](Buf &b, int g, int d) __attribute__((always_inline)) {
        const bool live = g < g1;
        const uint32_t vw = live ? static_cast<uint32_t>(lane) * 16 : kOutside;
        const uint32_t vp = live ? v_par : kOutside;
        const int gg = live ? g : g1 - 1;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if constexpr (DM) {
                uint32_t va = v_a[mb];
                asm volatile("" : "+v"(va));
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rA,
                        (__attribute__((address_space(3))) void *)(dma_base +
                                                                   (d * MB + mb) * 256 + t * 64),
                        16,
                        live ? va + static_cast<uint32_t>(t) * rows4 + (cx16 ^ (64u * t)) - 16u * c
                             : kOutside,
                        static_cast<uint32_t>(gg * kGroup) * 2, 0, 0);
            } else if constexpr (FL) {
                // the row in the vector offset (rows past M fall outside the buffer: zeros);
                // one base per row block, the four steps' offsets added at each load
                uint32_t va = v_a[mb];
                asm volatile("" : "+v"(va));
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    b.a[mb][t] = __builtin_bit_cast(
                        h8, __builtin_amdgcn_raw_buffer_load_b128(
                                rA, live ? va + static_cast<uint32_t>(t) * rows4 : kOutside,
                                static_cast<uint32_t>(gg * kGroup) * 2, 0));
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    b.a[mb][t] = __builtin_bit_cast(
                        h8, __builtin_amdgcn_raw_buffer_load_b128(
                                rA, live ? v_a[mb] : kOutside,
                                static_cast<uint32_t>(gg * kGroup + 32 * t) * 2, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < NS; ++i)
            b.w[i] = __builtin_bit_cast(
                u4, __builtin_amdgcn_raw_buffer_load_b128(
                        rW, vw, (static_cast<uint32_t>(slab(i)) * p.G + gg) * 1024u, kWeightPolicy));
        if constexpr (!F::COL) {
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                const int u = u0 + k < U ? u0 + k : U - 1;
                if constexpr (F::ZP) {
                    const u4 v = __builtin_bit_cast(
                        u4, __builtin_amdgcn_raw_buffer_load_b128(rS, vp, par_soff(u, gg), 0));
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        b.p[k][d] = v[d];
                } else {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rS, vp, par_soff(u, gg), 0);
                    b.p[k][0] = v[0];
                    b.p[k][1] = v[1];
                }
            }
        }
    };

    // Halves r .. r + NS - 1 of the concatenated groups (part 0: scales, 1: zero terms), two
    // per dword: dword m of the result holds slabs 2m and 2m + 1.
    const bool sel_dw = (r & 2) != 0, sel_half = (r & 1) != 0;     // uniform
    auto pick = [&](const uint32_t (&pg)[NG][F::ZP ? 4 : 2], int part, uint32_t (&out)[NH])
        __attribute__((always_inline)) {
        auto D = [&](int m) __attribute__((always_inline)) {
            m = m < 2 * NG ? m : 2 * NG - 1;           // past the last half needed
            return pg[m >> 1][2 * part + (m & 1)];
        };
        uint32_t e[NH + 1];
#pragma unroll
        for (int m = 0; m <= NH; ++m)
            e[m] = sel_dw ? D(m + 1) : D(m);
#pragma unroll
        for (int m = 0; m < NH; ++m)
            out[m] = sel_half ? __builtin_amdgcn_alignbit(e[m + 1], e[m], 16) : e[m];
    };

    // One scale per column: the half of slab j at group 0 (part 1: its zero term), and its
    // position in the dword that holds it.
    auto col_param = [&](int j, int part) __attribute__((always_inline)) {
        const uint32_t half = (static_cast<uint32_t>(j >> 2) * 16u + c) * (PB / 2) + 4u * part +
                              static_cast<uint32_t>(j & 3);
        const uint32_t dw = __builtin_amdgcn_raw_buffer_load_b32(rS, (half >> 1) * 4, 0, 0);
        return static_cast<uint16_t>(dw >> (16 * (half & 1)));
    };

    // With one scale per column and zero points the zero terms are the same for every tile.
    uint16_t zcol[(F::ZP && F::COL) ? NS : 1];
    if constexpr (F::ZP && F::COL) {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            zcol[i] = col_param(slab(i), 1);
    }

    f4 acc[MB][NS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < NS; ++i)
            acc[mb][i] = f4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](Buf &b, int d, bool tail) __attribute__((always_inline)) {
        h8 af[DM ? MB : 1][DM ? 4 : 1];
        if constexpr (DM) {
            // This tile's DMA has landed once at most the DEPTH - 1 load calls issued after
            // its own are outstanding (in the loop; the tail waits for all): the vector
            // memory counter completes in order
            constexpr int kPerLoad = 4 * MB + NS + (F::COL ? 0 : NG);
            static_assert((DEPTH - 1) * kPerLoad <= 63, "vmcnt range");
            if (tail)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_imm((DEPTH - 1) * kPerLoad));
            asm volatile("" ::: "memory");
            const u4 *src = dma_base + d * (MB * 256);
            const int q = lane >> 4;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    af[mb][t] = __builtin_bit_cast(
                        h8, src[(mb * 4 + (c >> 2)) * 64 + (c & 3) * 16 + ((4 * t + q) ^ c)]);
        } else if constexpr (FL) {
            // rows 4t .. 4t + 3 of step t -> the wave's LDS region (rows of 17 chunks, so
            // that the 16 rows read at one chunk lie in 16 different bank groups) -> back in
            // fragment order, in place.  One wave writes and reads its own region: LDS
            // operations of a wave complete in order, no barrier.
            u4 *reg = atr + wave * (MB * kTrRowBlock);
            const int rq = lane >> 4;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    reg[(16 * mb + 4 * t + rq) * 17 + c] = __builtin_bit_cast(u4, b.a[mb][t]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    b.a[mb][t] = __builtin_bit_cast(h8, reg[(16 * mb + c) * 17 + 4 * t + rq]);
        }
        auto av = [&](int mb, int t) __attribute__((always_inline)) -> const h8 & {
            if constexpr (DM)
                return af[mb][t];
            else
                return b.a[mb][t];
        };
        float sf[NS];
        h2 zsub[NS], zadd[NS];
        uint32_t sh[NH], zh[NH];
        if constexpr (!F::COL) {
            pick(b.p, 0, sh);
            if constexpr (F::ZP)
                pick(b.p, 1, zh);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if constexpr (!F::COL && !TWO) {
                sf[i] = half_bits_to_float(static_cast<uint16_t>(sh[i >> 1] >> (16 * (i & 1))));
                asm volatile("" : "+v"(sf[i]));
            }
            if constexpr (F::ZP) {
                uint16_t zb;
                if constexpr (F::COL)
                    zb = zcol[i];
                else
                    zb = static_cast<uint16_t>(zh[i >> 1] >> (16 * (i & 1)));
                const _Float16 zt = __builtin_bit_cast(_Float16, zb);
                zsub[i] = h2{zt, zt};
                const h2 k960 = {static_cast<_Float16>(960.0f), static_cast<_Float16>(960.0f)};
                zadd[i] = k960 - zsub[i];
                asm volatile("" : "+v"(zsub[i]));
                asm volatile("" : "+v"(zadd[i]));
            } else {
                zsub[i] = sym_zsub();
                zadd[i] = sym_zadd();
            }
        }
        if constexpr (!F::ZP) {
            // Symmetric formats, raw decode: per row block the chain P sums A * offsets over
            // the tile's four 32-k steps, per slab the chain D sums A * raw codes in the same
            // order, and D - P is the tile's sum of A * (q - 8) (exactly 0 when every code is 8:
            // the two chains then see the same values).  Per group it is scaled into the
            // running sums; with one scale per column it is added, the scale coming at the end.
            const h8 off = raw_offsets();
            f4 P[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    P[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        av(mb, t), off, t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : P[mb], 0, 0, 0);
            if constexpr (TWO) {
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    f4 D[MB];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const h8 x = raw8(b.w[i][t], mlo, mhi, magic, magic_hi);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            D[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                av(mb, t), x, t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : D[mb], 0, 0, 0);
                    }
                    // (the scale converted here, where it is used: no nine live at once)
                    float sfi = 1.0f;
                    if constexpr (!F::COL)
                        sfi = half_bits_to_float(
                            static_cast<uint16_t>(sh[i >> 1] >> (16 * (i & 1))));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const f4 part = D[mb] - P[mb];
                        if constexpr (F::COL)
                            acc[mb][i] += part;
                        else
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                acc[mb][i][q] = __builtin_fmaf(sfi, part[q], acc[mb][i][q]);
                        asm volatile("" : "+v"(acc[mb][i]));
                    }
                }
                return;
            }
            f4 D[MB][NS];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const h8 x = raw8(b.w[i][t], mlo, mhi, magic, magic_hi);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        D[mb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            av(mb, t), x, t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : D[mb][i], 0, 0, 0);
                }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const f4 part = D[mb][i] - P[mb];
                    if constexpr (F::COL)
                        acc[mb][i] += part;
                    else
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mb][i][q] = __builtin_fmaf(sf[i], part[q], acc[mb][i][q]);
                    asm volatile("" : "+v"(acc[mb][i]));
                }
        } else if constexpr (F::COL) {
            // one scale per column: sum A * (q - z) over the whole K range, scale at the end
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const h8 x = dequant8(b.w[i][t], mlo, mhi, magic, zsub[i], zadd[i]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av(mb, t), x,
                                                                            acc[mb][i], 0, 0, 0);
                }
        } else {
            // per group: the exact sum of A * (q - z) over the group, then one scale per output
            f4 part[MB][NS];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const h8 x = dequant8(b.w[i][t], mlo, mhi, magic, zsub[i], zadd[i]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const f4 cin = t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : part[mb][i];
                        part[mb][i] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(av(mb, t), x, cin, 0, 0, 0);
                    }
                }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < NS; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[mb][i][q] = __builtin_fmaf(sf[i], part[mb][i][q], acc[mb][i][q]);
                    asm volatile("" : "+v"(acc[mb][i]));
                }
        }
    };

    if (g0 < g1) {
        // D buffers, tile i in buffer i % D, so D - 1 tiles of weights are in flight while one
        // is computed.  Whole rounds of D tiles run in a
        // loop with one exit (a loop the compiler can leave from several places gets an edge on
        // which the last loads issued are the buffer about to be used, and then waits for every
        // load in flight); the remaining tiles follow.  The empty asm statements fence memory,
        // so each buffer's loads are issued right after the compute that frees it and are not
        // sunk toward their use.
        constexpr int D = DEPTH;
        Buf b[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(b[d], g0 + d, d);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        const int rounds = (g1 - g0) / D;
        int g = g0;
        for (int it = 0; it < rounds; ++it) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute(b[d], d, false);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                load(b[d], g + d + D, d);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
            g += D;
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (g + d < g1)
                compute(b[d], d, true);
        // the loads past the run touch no memory, but their registers (and, DM, the waves'
        // LDS buffers) are still written
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (DM)
        __syncthreads();                       // every wave is done with its A buffers (red)

    // The four waves' partial sums meet in LDS, one row block at a time; wave w then
    // finishes slabs w, w + 4, ...
    const uint32_t v_c = (static_cast<uint32_t>(4 * (lane >> 4)) * p.N + c) * 2;
    const uint32_t rowN = opaque(static_cast<uint32_t>(p.N) * 2);
    auto write_slab = [&](int mb, int i, f4 v) __attribute__((always_inline)) {
        if constexpr (F::COL)
            v *= half_bits_to_float(col_param(j0 + i, 0));
        uint32_t srow =
            static_cast<uint32_t>(j0 + i) * 32 + static_cast<uint32_t>(row0 + 16 * mb) * rowN;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_raw_buffer_store_b16(float_to_half_bits(v[q]), rC, v_c, srow, 0);
            srow += rowN;
        }
    };
    // Split K: the piece of row block mb of slab j0 + i from split k goes to slot
    // ((grp * KS + k) * NS + i) * MB + mb, grp = the slab group within its row sub-problem.
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(p.partials, static_cast<uint32_t>(gridDim.x * gridDim.z) * KS * NS * MB * 1024u);
    auto slot = [&](int k, int i, int mb) __attribute__((always_inline)) {
        return (((static_cast<uint32_t>(grp) * KS + k) * NS + i) * MB + mb) * 1024u;
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (mb > 0)
            __syncthreads();                   // the previous block's sums have been read
#pragma unroll
        for (int i = 0; i < NS; ++i)
            red[(wave * NS + i) * 64 + lane] = acc[mb][i];
        __syncthreads();
#pragma unroll
        for (int i0 = 0; i0 < NS; i0 += kWaves) {
            const int i = i0 + wave;
            if (i < NS && j0 + i < S) {
                f4 v = red[(0 * NS + i) * 64 + lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
                    v += red[(w * NS + i) * 64 + lane];
                if (KS == 1)
                    write_slab(mb, i, v);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), rP,
                                                           lane * 16, slot(ks, i, mb),
                                                           kDeviceScope);
            }
        }
    }
    if (KS == 1)
        return;

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's pieces are stored
    __shared__ int arrived;
    __syncthreads();
    if (tid == 0)
        arrived = __hip_atomic_fetch_add(p.counters + grp, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != KS - 1)
        return;
    // the last to arrive: every piece is stored; sum them in split order
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i0 = 0; i0 < NS; i0 += kWaves) {
            const int i = i0 + wave;
            if (i < NS && j0 + i < S) {
                f4 x[kSkinnyMaxKS];
#pragma unroll
                for (int k = 0; k < kSkinnyMaxKS; ++k) {
                    // splits past KS: a lane offset outside the buffer (reads zero, no access)
                    const uint32_t vo = k < KS ? slot(k, i, mb) + lane * 16 : kOutside;
                    x[k] = __builtin_bit_cast(
                        f4, __builtin_amdgcn_raw_buffer_load_b128(rP, vo, 0, kDeviceScope));
                }
                f4 v = x[0];
#pragma unroll
                for (int k = 1; k < kSkinnyMaxKS; ++k)
                    if (k < KS)
                        v += x[k];
                write_slab(mb, i, v);
            }
        }
    if (tid == 0)
        __hip_atomic_store(p.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ 2:4-sparse weights
//
// `w4a16_gemm_sparse_kernel<MB, NS>`: the product with weights that keep 2 of every 4 along K
// (w4a16_pack_24; group-128 scales, zero point 8), on gfx950's structured-sparse matrix
// instruction v_smfmac_f32_16x16x64_f16.  Its first operand is the sparse one (16 rows x 64 k
// held as the 32 kept values with a 2-bit position each), so the product is computed
// transposed, C^T = Bhat^T A^T, as Sparse-MARLIN rewrites AB as (B^T A^T)^T for the same
// reason (deep-dive page, Sparse-MARLIN section): output columns are the instruction's rows,
// tokens its columns.  Operand layout, measured on the hardware: sparse-operand lane l holds
// row l % 16 and the kept values of the four groups of four in k = 16(l/16) .. +15 (value e
// of group e/2, its position in bits 2e..2e+1 of the index register); dense-operand lane l
// holds column l % 16 with k = 8(l/16) + 0..7 in halves 0..7 and 32 + 8(l/16) + 0..7 in halves
// 8..15 -- the A fragments of two consecutive 32-k steps of the dense kernels; result lane l
// holds rows 4(l/16) + 0..3 of column l % 16.
//
// Structure as the whole-K kernel above: a workgroup owns NS slabs over all of K, its four
// waves split the K tiles, partial sums meet in LDS in a fixed order.  A lane's 12 bytes per
// 128 x 16 block are one 96-bit load: the kept codes of the block's two 64-k steps (8 per
// word, decoded by the dense kernels' mask-and-OR) and their positions.  The decoded values are
// scaled in fp16 (the lane's sparse-operand row is an output column, so its own column scale
// applies; one rounding of s * (q - 8), as in the 64- and 128-row dense tiles).  MB blocks of
// 16 rows per launch; the host runs larger M as several launches.
template <int MB, int NS>
struct SparseBuf {
    uint32_t w[NS][3];                       // kept codes of the two 64-k steps, positions
    h8 a[MB][4];                             // A fragments of each 16-row block
    uint32_t p[SkinnyGroups<NS>::n][2];      // four scales of the lane's column per group
};

template <int MB, int NS, bool FL = false>
__global__ __launch_bounds__(kThreads, 2) void w4a16_gemm_sparse_kernel(Params p)
{
    using SG = SkinnyGroups<NS>;
    constexpr int NG = SG::n, NH = SG::nh;
    __shared__ f4 red[kWaves * MB * NS * 64];
    __shared__ u4 atr[FL ? kWaves * MB * kTrRowBlock : 1];   // per-wave A transposes (FL)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15;
    const int S = p.N >> 4;                              // slabs
    const int U = S >> 2;                                // parameter groups
    const int j0 = blockIdx.x * NS;
    const int u0 = j0 >> 2, r = j0 & 3;
    const int g0 = p.G * wave / kWaves;
    const int g1 = p.G * (wave + 1) / kWaves;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.K) * 2u);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(
        p.packed, static_cast<uint32_t>(static_cast<size_t>(p.K) * p.N * 3 / 8));
    const __amdgpu_buffer_rsrc_t rS =
        make_rsrc(p.scales, static_cast<uint32_t>(static_cast<size_t>(p.G) * p.N * 2));
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.C, static_cast<uint32_t>(p.M) * static_cast<uint32_t>(p.N) * 2u);

    const uint32_t mlo = in_vgpr(0x000f000fu), mhi = in_vgpr(0x00f000f0u);
    const uint32_t magic = in_vgpr(0x64006400u);
    const uint32_t v_par = static_cast<uint32_t>(c) * 8;
    // A operand of row block mb: row 16 mb + c, k = 8 * (lane / 16) of each 32-k step; FL:
    // whole-line loads of rows 4t .. 4t + 3 per step and a transpose in the wave's LDS
    // region, as the dense whole-K kernel
    uint32_t v_a[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        v_a[mb] = FL ? (static_cast<uint32_t>(16 * mb + (lane >> 4)) * p.K + 8 * c) * 2
                     : (static_cast<uint32_t>(16 * mb + c) * p.K + 8 * (lane >> 4)) * 2;
    const uint32_t rows4 = static_cast<uint32_t>(p.K) * 8;      // 4 rows of A, in bytes
    auto slab = [&](int i) __attribute__((always_inline)) {
        const int j = j0 + i;
        return j < S ? j : S - 1;          // slabs past N re-read the last one; never stored
    };

    auto load = [&](SparseBuf<MB, NS> &b, int g) __attribute__((always_inline)) {
        const bool live = g < g1;
        const uint32_t vw = live ? static_cast<uint32_t>(lane) * 12 : kOutside;
        const uint32_t vp = live ? v_par : kOutside;
        const int gg = live ? g : g1 - 1;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            uint32_t va = v_a[mb];
            if constexpr (FL)
                asm volatile("" : "+v"(va));
#pragma unroll
            for (int t = 0; t < 4; ++t)
                b.a[mb][t] = __builtin_bit_cast(
                    h8, __builtin_amdgcn_raw_buffer_load_b128(
                            rA,
                            live ? (FL ? va + static_cast<uint32_t>(t) * rows4 : va) : kOutside,
                            static_cast<uint32_t>(gg * kGroup + (FL ? 0 : 32 * t)) * 2, 0));
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b96(
                rW, vw, (static_cast<uint32_t>(slab(i)) * p.G + gg) * 768u, kNonTemporal);
            b.w[i][0] = v[0];
            b.w[i][1] = v[1];
            b.w[i][2] = v[2];
        }
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int u = u0 + k < U ? u0 + k : U - 1;
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(
                rS, vp, (static_cast<uint32_t>(u) * p.G + gg) * 128u, 0);
            b.p[k][0] = v[0];
            b.p[k][1] = v[1];
        }
    };

    // scale halves of slabs j0 .. j0 + NS - 1 (two per dword), as in the whole-K kernel
    const bool sel_dw = (r & 2) != 0, sel_half = (r & 1) != 0;
    auto pick = [&](const uint32_t (&pg)[NG][2], uint32_t (&out)[NH]) __attribute__((always_inline)) {
        auto D = [&](int m) __attribute__((always_inline)) {
            m = m < 2 * NG ? m : 2 * NG - 1;
            return pg[m >> 1][m & 1];
        };
        uint32_t e[NH + 1];
#pragma unroll
        for (int m = 0; m <= NH; ++m)
            e[m] = sel_dw ? D(m + 1) : D(m);
#pragma unroll
        for (int m = 0; m < NH; ++m)
            out[m] = sel_half ? __builtin_amdgcn_alignbit(e[m + 1], e[m], 16) : e[m];
    };

    f4 acc[MB][NS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < NS; ++i)
            acc[mb][i] = f4{0.f, 0.f, 0.f, 0.f};

    // The decoded weights are scaled in fp16 and the sparse instruction accumulates straight
    // into the running sums, which are read only after the last tile.  (Per-tile sums started
    // from zero in the accumulator and read right behind the instruction gave wrong results on
    // gfx950: unlike the dense instruction, whose zero accumulator is an inline constant, the
    // sparse one's accumulator is its destination register, written by a move just before.)
    auto compute = [&](SparseBuf<MB, NS> &b) __attribute__((always_inline)) {
        if constexpr (FL) {
            u4 *reg = atr + wave * (MB * kTrRowBlock);
            const int rq = lane >> 4;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    reg[(16 * mb + 4 * t + rq) * 17 + c] = __builtin_bit_cast(u4, b.a[mb][t]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    b.a[mb][t] = __builtin_bit_cast(h8, reg[(16 * mb + c) * 17 + 4 * t + rq]);
        }
        uint32_t sh[NH];
        pick(b.p, sh);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const _Float16 sv = __builtin_bit_cast(
                _Float16, static_cast<uint16_t>(sh[i >> 1] >> (16 * (i & 1))));
            const h2 s2 = {sv, sv};
            const h8 x0 = dequant8_scaled(b.w[i][0], s2, mlo, mhi, magic, sym_zsub(), sym_zadd());
            const h8 x1 = dequant8_scaled(b.w[i][1], s2, mlo, mhi, magic, sym_zsub(), sym_zadd());
            const int idx0 = static_cast<int>(b.w[i][2]);
            const int idx1 = static_cast<int>(b.w[i][2] >> 16);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const h16 d0 = __builtin_shufflevector(b.a[mb][0], b.a[mb][1], 0, 1, 2, 3, 4, 5,
                                                       6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                const h16 d1 = __builtin_shufflevector(b.a[mb][2], b.a[mb][3], 0, 1, 2, 3, 4, 5,
                                                       6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                acc[mb][i] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(x0, d0, acc[mb][i], idx0,
                                                                      0, 0);
                acc[mb][i] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(x1, d1, acc[mb][i], idx1,
                                                                      0, 0);
            }
        }
    };

    if (g0 < g1) {
        // two buffers, one exit, memory fences: as the whole-K kernel (see there)
        SparseBuf<MB, NS> b[2];
        load(b[0], g0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load(b[1], g0 + 1);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int rounds = (g1 - g0) >> 1;
        int g = g0;
        for (int it = 0; it < rounds; ++it) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                compute(b[d]);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                load(b[d], g + d + 2);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
            g += 2;
        }
        if (g < g1)
            compute(b[0]);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // The four waves' partial sums meet in LDS; wave w finishes slabs w, w + 4, ...  Result
    // lane l holds output columns 16j + 4(l/16) + 0..3 of row 16 mb + l % 16: 8 bytes of C.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < NS; ++i)
            red[((wave * MB + mb) * NS + i) * 64 + lane] = acc[mb][i];
    __syncthreads();
#pragma unroll
    for (int i0 = 0; i0 < NS; i0 += kWaves) {
        const int i = i0 + wave;
        if (i < NS && j0 + i < S) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                f4 v = red[((0 * MB + mb) * NS + i) * 64 + lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
                    v += red[((w * MB + mb) * NS + i) * 64 + lane];
                const uint32_t lo = static_cast<uint32_t>(float_to_half_bits(v[0])) |
                                    (static_cast<uint32_t>(float_to_half_bits(v[1])) << 16);
                const uint32_t hi = static_cast<uint32_t>(float_to_half_bits(v[2])) |
                                    (static_cast<uint32_t>(float_to_half_bits(v[3])) << 16);
                typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                const uint32_t voff = (static_cast<uint32_t>(16 * mb + c) * p.N + 16 * (j0 + i) +
                                       4 * (lane >> 4)) * 2;
                __builtin_amdgcn_raw_buffer_store_b64(u2{lo, hi}, rC, voff, 0, 0);
            }
        }
    }
}

// ------------------------------------------------------------------------------- host side

struct Config {
    int MB, NBW;     // M sub-tiles of 16 rows; 16-column slabs per wave
    int waves;       // waves per workgroup
    int P, S, G, W;
    long long T;
    int NS;          // > 0: the skinny kernel, NS slabs per workgroup (W workgroups)
    int KS;          // the skinny kernel's K splits per slab group (1: none)
    int SMB;         // the skinny kernel's 16-row blocks (1, 2 or 4)
    int SP;          // the skinny kernel's row sub-problems (2 for M = 65..128)
    bool TWO;        // the skinny kernel's 32-row form at two workgroups per CU
    bool DEEP;       // the skinny kernel with one more tile of registers in flight
    bool FL;         // the skinny kernel's whole-line A loads (M > 8)
};

constexpr int kSkinnyMaxNS = 10;
constexpr int kSkinnyOneMaxNS = 7;        // one workgroup per CU up to this many slabs
constexpr int kSkinnyTwoMaxNS = 9;        // 32 rows at two per CU, symmetric formats
constexpr int kSkinnyTwoMinNS = 7;
constexpr int kSkinnyDeepNS = 3;          // one more buffer at M <= 8 up to this many slabs

// Skinny kernel (M <= 128, N a multiple of 256; 17..128 rows only in the one-per-CU regime
// below, two 64-row sub-problems above 64 rows).  Weights of up to 7 slabs per CU (N up to
// 28672 on 256 CUs) take the fewest slabs that leave at most one workgroup per CU: measured
// on K 4096..8192, N 7168..28672 this beats two or three per CU by 1.1-1.5x (8192 x 10240 at
// M = 16: 13.6 us with 3 slabs, 20.7 with 2; 8192 x 28672: 23.8 us with 7, 29.5 with 4); a
// CU running two workgroups of a short weight takes twice as long, it does not overlap them.
// Larger weights: NS = the fewest slabs per workgroup that keep
// the workgroups within two per CU, so every workgroup streams as many bytes as possible at
// once.  At M <= 8 (A mostly rows past M, read as zero without memory traffic) three per CU
// measure faster where that leaves 2 to 7 slabs (7 still fits three workgroups' registers):
// 72k x 18k 110.5 vs 113.2 us at M = 1; at M = 16 the extra A re-reads make it slower (128.9
// vs 124.4 us).  With one slab per workgroup four of a wave's six loads per tile are A fragments;
// there the stripe kernel measures faster once K runs long (28672 x 8192: 31 vs 33 us at
// M = 1) unless K is split (choose_config), while on every shorter or wider weight measured
// the skinny kernel is faster (1.1x to 4x).  Its dead loads point 2 GiB past the buffer
// starts, so the weights and A must lie below that.
int skinny_slabs(int M, int K, int N, int cus, bool zp, bool *two)
{
    *two = false;
    if (M > 128 || N % 256)
        return 0;
    const long long S = N / 16;
    const long long P = M > 64 ? 2 : 1;   // 64-row sub-problems side by side
    long long ns = (S + 2LL * cus - 1) / (2LL * cus);
    const long long ns1 = (P * S + cus - 1) / cus;
    // four row blocks: up to 7 slabs per 64-row sub-problem (one workgroup per CU, so the
    // accumulators may spill into the AGPRs), measured against the stripe and 128-row kernels:
    // 4096 x 22016 at M = 64, 6 slabs, 29.3 -> 25.7 us; 8192 x 28672, 7 slabs, 53.6 -> 49.4;
    // two sub-problems, 4096 x 12288 at M = 128, 6 slabs, 27.7 -> 24.8; 8192 x 10240, 5,
    // 41.7 -> 38.6
    if (M > 32 && ns1 > kSkinnyOneMaxNS)
        return 0;
    if (ns1 <= kSkinnyOneMaxNS) {
        ns = ns1;
    } else if (M > 16) {
        // 32 rows on a larger weight: two workgroups per CU of seven to nine slabs, symmetric
        // formats only (their raw decode leaves the registers for it).  Against the 32-row
        // stripe tiles, measured in the same runs: 72k x 18k 142 vs 161 us at M = 17, 144 vs
        // 155 at M = 24, a tie at 32; 8192 x 57344 52 vs 57 at M = 24.  With fewer slabs a
        // wave's tiles are too light (8192 x 32768, four slabs: 47 vs 38 us at M = 32).
        if (zp || ns > kSkinnyTwoMaxNS || ns < kSkinnyTwoMinNS)
            return 0;
        *two = true;
    } else if (M <= 8) {
        const long long ns3 = (S + 3LL * cus - 1) / (3LL * cus);
        if (ns3 >= 2 && ns3 <= 7)
            ns = ns3;
    }
    if (ns > kSkinnyMaxNS ||
        static_cast<uint64_t>(K) * static_cast<uint64_t>(N) / 2 >= kOutside ||
        static_cast<uint64_t>(64) * static_cast<uint64_t>(K) * 2 >= kOutside) {
        *two = false;
        return 0;
    }
    return static_cast<int>(ns);
}

// Slabs and K splits for the skinny kernel once it runs at most one workgroup per CU.  There
// its time follows the K tiles each wave walks one after the other: about 2.5 us, plus per tile
// a + b * NS (a = 0.27, b = 0.075 us at M <= 8; a = 0.45, b = 0.06 at M = 16), plus ~2.1 us for
// the split's store, count and reload when K is split; with two row blocks (M = 17..32)
// 1.9 us + (0.90 + 0.057 NS) per tile + 3.4 us per split, with four (M = 33..64) 4.9 us +
// (1.60 + 0.079 NS) per tile + 3.4 us per split (fitted to timings of K 1024..28672,
// N 256..10240, NS 1..4, KS 1..8 on MI355X; past four slabs the model is too optimistic).  The
// search keeps at most one workgroup per CU and kSkinnyMaxKS splits (summed in one load
// round), never below two tiles per wave, and leaves the one-per-CU choice only for a
// predicted gain of 15%.  Up to 4 slabs, and where A has real rows (M = 9..16: 8 slabs;
// M = 17..32: 5, the registers of two row blocks) more, but then only with at least 8 K tiles
// a wave: more slabs per A fragment pay once the A loads carry data, short runs do not (at
// M = 1 the 28672 x 8192 weight's 8 slabs x 4 splits ran 3% slower, and 11008 x 4096 at
// M = 16 with 8 x 8, 2.7 tiles a wave, 11% slower).  Measured: 8192 x 1280 at M = 16 10.3 -> 6.5-6.8 us,
// 11008 x 4096 13.4 -> 9.6 us, 14336 x 2048 16.5 -> 8.4 us, 28672 x 1024 22 -> 10 us; past
// four slabs 28672 x 8192 at M = 12 / 16 25.7 -> 23.4 / 27.7 -> 23.9 us (8 slabs, 4 splits),
// 8192 x 10240 at M = 16 / 24 / 32 13.4 -> 12.9 / 18.0 -> 16.3 / 20.4 -> 17.4 us (5, 2), the
// other Llama-2 layer and rank shapes unchanged within 3%.  The counters bound the slab
// groups.
double skinny_model_us(int G, int NS, int KS, int M)
{
    // fixed time, per-tile time a + b * NS, split cost; fitted per row range
    const double c0 = M <= 16 ? 2.5 : (M <= 32 ? 1.93 : 4.89);
    const double a = M <= 8 ? 0.27 : (M <= 16 ? 0.45 : (M <= 32 ? 0.90 : 1.60));
    const double b = M <= 8 ? 0.075 : (M <= 16 ? 0.06 : (M <= 32 ? 0.057 : 0.079));
    const double cs = M <= 16 ? 2.1 : (M <= 32 ? 3.44 : 3.39);
    return c0 + static_cast<double>(G) / (kWaves * KS) * (a + b * NS) + (KS > 1 ? cs : 0.0);
}

void skinny_split(int S, int G, int M, int P, int cus, int &ns, int &ks)
{
    ks = 1;
    if (P * ((S + ns - 1) / ns) > cus)
        return;                                   // more than one workgroup per CU
    const double base = skinny_model_us(G, ns, 1, M);
    double best = 0.85 * base;
    const int ns0 = ns;
    const int nmax = M <= 8 ? 4 : (M <= 16 ? 8 : (M <= 32 ? 5 : 4));
    for (int n = ns0; n <= nmax; n = n < 2 ? 2 : n + 2) {
        const int wn = (S + n - 1) / n;
        if (P * wn > kMaxWGs)
            continue;
        // past four slabs only with at least 8 K tiles a wave (short runs of wide tiles
        // measure slower than the model says)
        const int kmax = std::min({kSkinnyMaxKS, cus / (P * wn), G / (2 * kWaves),
                                   n > 4 ? std::max(1, G / (8 * kWaves)) : kSkinnyMaxKS});
        for (int k = 2; k <= kmax; ++k) {
            const double t = skinny_model_us(G, n, k, M);
            if (t < best) {
                best = t;
                ns = n;
                ks = k;
            }
        }
    }
}

int check_gemm_shape(int M, int K, int N)
{
    if (M < 0 || K < 0 || N < 0)
        return W4A16_EINVAL;
    if (K == 0 || K % kGroup || N == 0 || N % W4A16_N_ALIGN)
        return W4A16_ESHAPE;
    // Buffer resources address at most 4 GiB; A and C offsets run up to 128 rows past M.
    const uint64_t lim = uint64_t(1) << 32;
    if ((static_cast<uint64_t>(M) + 128) * static_cast<uint64_t>(K) * 2 >= lim ||
        (static_cast<uint64_t>(M) + 128) * static_cast<uint64_t>(N) * 2 >= lim ||
        static_cast<uint64_t>(K) * static_cast<uint64_t>(N) / 2 >= lim)
        return W4A16_ESHAPE;
    return W4A16_OK;
}

// Number of stripes W, from a cost model of the stripe kernel fitted to timings on gfx950
// (K 4096 .. 28672, N 4096 .. 73728, M 24 .. 128).  A stripe's tiles stream one after the
// other, each taking the longer of a latency floor (loads run two tiles ahead: about 1.1 us
// with 16- and 32-row tiles, 1.3 us with more rows) and its share of HBM bandwidth with W
// tiles in flight (6 TB/s); a slice split into n pieces
// is summed by one workgroup at about 0.8 us a piece.  Many stripes buy bandwidth, few buy
// short sums: a 4096 x 4096 weight at M = 24 takes 27 us with 512 one-tile stripes (32 pieces
// a slice) and 12 us with 128.  W is two per CU or at most one per CU, so that every CU
// streams the same amount (an uneven count leaves some CUs with twice the work of others).
int choose_stripes(long long T, int G, int MB, double tile_bytes, int cus)
{
    const long long wmax = std::min<long long>({2LL * cus, kMaxWGs, T});
    const double floor_us = MB <= 2 ? 1.1 : 1.3;
    auto cost = [&](long long W) {
        const long long tps = (T + W - 1) / W;               // tiles of the longest stripe
        const double per_tile =
            std::max(floor_us, static_cast<double>(W) * tile_bytes / 6.0e6);
        // stripes sharing a slice: one more where stripe and slice ends do not line up
        const double per = static_cast<double>(T) / static_cast<double>(W);
        const bool aligned = T % W == 0 && (G % tps == 0 || tps % G == 0);
        const double pieces = std::ceil(G / per) + (aligned ? 0.0 : 1.0);
        return static_cast<double>(tps) * per_tile + 0.8 * pieces;
    };
    // fewer stripes than two per CU only for a clear gain: where both are bandwidth-bound
    // the model ties them, and two workgroups per CU hide latency better
    long long best = wmax;
    double tb = 0.95 * cost(wmax);
    for (long long W = std::min<long long>(cus, wmax); W >= 1; --W) {
        const double t = cost(W);
        if (t < tb) {
            tb = t;
            best = W;
        }
    }
    return static_cast<int>(best);
}

// HBM bytes of one stripe-kernel tile: Nt columns x 128 rows of codes (4 bits, or 3 per
// weight for 2:4-sparse blocks), the Mt x 128 A tile, one fp16 parameter per column.
double tile_bytes(int MB, int NBW, bool sparse)
{
    const double nt = 16.0 * kWaves * NBW;
    return nt * kGroup * (sparse ? 0.375 : 0.5) + 16.0 * MB * kGroup * 2 + nt * 2;
}

Config choose_config(int M, int K, int N, int cus, bool zp)
{
    Config c{};
    c.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    c.waves = kWaves;
    c.G = K / kGroup;
    const int per_cu = 2;                        // two workgroups per CU measured best
    if (M > 64 && N % (16 * kWideNBW * kWaves) == 0) {
        // Wide tiles (all rows of a 128-row block per wave) unless the output has so few of
        // them that each would be split between more than four stripes: the split pieces are
        // then summed serially by one workgroup, and 64-row tiles (twice as many, half the
        // partial size) measure faster.
        const long long tiles = static_cast<long long>(N / (16 * kWideNBW * kWaves)) *
                                ((M + 16 * kWideMB - 1) / (16 * kWideMB));
        const long long stripes = std::min<long long>(static_cast<long long>(cus) * per_cu,
                                                      tiles * c.G);
        if (4 * tiles >= stripes)
            c.MB = kWideMB;
    }
    const int Mt = 16 * c.MB;
    c.P = (M + Mt - 1) / Mt;
    // widest slice (4 slabs per wave) that divides N
    c.NBW = 1;
    for (int nbw = 4; nbw >= 1; nbw >>= 1)
        if (N % (16 * c.waves * nbw) == 0) {
            c.NBW = nbw;
            break;
        }
    c.S = N / (16 * c.waves * c.NBW);
    c.T = static_cast<long long>(c.S) * c.P * c.G;
    c.W = choose_stripes(c.T, c.G, c.MB, tile_bytes(c.MB, c.NBW, false), cus);
    c.NS = skinny_slabs(M, K, N, cus, zp, &c.TWO);
    c.KS = 1;
    c.SMB = M > 32 ? 4 : (M > 16 ? 2 : 1);
    c.SP = M > 64 ? 2 : 1;
    if (c.NS > 0 && c.TWO) {
        c.W = (N / 16 + c.NS - 1) / c.NS;          // two per CU, no K split
    } else if (c.NS > 0) {
        skinny_split(N / 16, c.G, M, c.SP, cus, c.NS, c.KS);
        const int wn = (N / 16 + c.NS - 1) / c.NS;
        if (c.NS == 1 && c.KS == 1 && c.G > 128)
            c.NS = 0;                  // one slab a workgroup over a long K: the stripe kernel
        else if (M > 16 && c.G > (M > 32 ? 16 : 32) * kWaves * c.KS)
            c.NS = 0;                  // 32 rows over more than 32 tiles a wave, 64 over more
                                       // than 16: the stripe kernel (28672 x 8192 at M = 64,
                                       // 28 tiles: 48.6 vs 51.1 us).  With A as whole lines
                                       // (by DMA for four row blocks) shorter walks favour
                                       // the whole-K kernel: 8192 x 10240 at M = 64, 16
                                       // tiles, 24.6 vs 31.7 us; 28672 x 8192 at M = 32, 28
                                       // tiles, 34.0 vs 36.1
        else
            c.W = wn * c.KS * c.SP;
    }
    // At M <= 8 most A rows lie past M and read as zero without memory traffic, so with up
    // to three slabs a wave's tile is little more than its weights: a third buffer, two weight
    // tiles in flight instead of one, measured 2-8% faster there (M = 1 / 8: 4096 x 4096 5.5
    // -> 5.2 / 6.0 -> 5.5 us, 8192 x 8192 9.5 -> 8.9 / 10.1 -> 10.0, 4096 x 12288 7.7 -> 7.5)
    // and no faster with more slabs or real A rows (M = 16: up to 4% slower), nor where a
    // wave walks only a few K tiles (1024 x 8192, two: 3.45 -> 3.7 us).
    c.DEEP = c.NS > 0 && !c.TWO && c.SMB == 1 && M <= 8 && c.NS <= kSkinnyDeepNS &&
             c.G >= 6 * kWaves * c.KS;
    // Whole-line A loads once A has real rows past the first few: measured 2-19% faster at
    // M = 17..64 (3584 x 8192 at M = 32 10.1 -> 8.2 us, 8192 x 57344 57.1 -> 50.4 us) and at
    // M = 9..16 where a wave walks at least 8 K tiles (8192 x 8192 12.1 -> 10.1 us, 8192 x
    // 7168 11.9 -> 10.1 us); not at M <= 8, where the loads of dead rows cost nothing (3-6%
    // slower with the LDS round trip), nor at M = 9..16 over fewer tiles (1024 x 8192 and
    // 3584 x 8192 at M = 16: 4% slower).  (The nine-slab 32-row form takes its whole lines by
    // DMA, see dispatch_skinny.)
    c.FL = c.NS > 0 && (M > 16 || (M > 8 && c.G >= 8 * kWaves * c.KS));
    return c;
}

// 2:4-sparse weights on the stripe kernel: 16-, 32- and 64-row tiles over 256-column slices
// (N a multiple of 256), as for dense weights but never the 128-row tiles.
Config choose_config_24(int M, int K, int N, int cus)
{
    Config c{};
    c.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    c.NBW = 4;
    c.waves = kWaves;
    c.G = K / kGroup;
    c.P = (M + 16 * c.MB - 1) / (16 * c.MB);
    c.S = N / (16 * c.waves * c.NBW);
    c.T = static_cast<long long>(c.S) * c.P * c.G;
    c.W = choose_stripes(c.T, c.G, c.MB, tile_bytes(c.MB, c.NBW, true), cus);
    c.NS = 0;
    c.KS = 1;
    return c;
}

size_t workspace_for(const Config &c)
{
    if (c.NS > 0)       // the skinny kernel: one 1 KiB piece per slab and row block when split
        return kCounterBytes +
               (c.KS > 1 ? static_cast<size_t>(c.W) * c.NS * c.SMB * 1024 : 0);
    const size_t slot = static_cast<size_t>(16 * c.MB) * (16 * c.waves * c.NBW) * sizeof(float);
    return kCounterBytes + 2 * static_cast<size_t>(c.W) * slot;
}

// ONCE (weights streamed, not cached) whenever the call has one row sub-problem; with 16- and
// 32-row tiles that is every call.
template <int MB, int NBW, class F>
hipError_t launch(const Params &p, hipStream_t stream)
{
    if constexpr (MB > 2) {
        if (p.P > 1) {
            hipLaunchKernelGGL((w4a16_gemm_kernel<MB, NBW, F, false>), dim3(p.W), dim3(kThreads),
                               0, stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((w4a16_gemm_kernel<MB, NBW, F, true>), dim3(p.W), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

template <int WAVES, int STAGES, class F>
hipError_t launch_wide(const Params &p, hipStream_t stream)
{
    if (p.P == 1) {
        hipLaunchKernelGGL((w4a16_gemm_wide_kernel<WAVES, STAGES, F, true>), dim3(p.W),
                           dim3(64 * WAVES), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((w4a16_gemm_wide_kernel<WAVES, STAGES, F, false>), dim3(p.W), dim3(64 * WAVES), 0,
                       stream, p);
    return hipGetLastError();
}

template <int MB, int NS, class F, bool TWO = false, int DEPTH = kLoadDepth, bool FL = false,
          bool DM = false>
hipError_t launch_skinny(const Params &p, hipStream_t stream)
{
    hipLaunchKernelGGL((w4a16_gemm_skinny_kernel<MB, NS, F, TWO, DEPTH, FL, DM>),
                       dim3(p.W / (p.KS * p.SP), p.KS, p.SP), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <class F>
hipError_t dispatch_skinny(int mb, int ns, bool two, bool deep, bool fl, const Params &p,
                           hipStream_t s)
{
    constexpr int D = kLoadDepth;
    if (deep) {
        if (mb == 1) {
            switch (ns) {
            case 1: return launch_skinny<1, 1, F, false, D + 1>(p, s);
            case 2: return launch_skinny<1, 2, F, false, D + 1>(p, s);
            case 3: return launch_skinny<1, 3, F, false, D + 1>(p, s);
            default: break;
            }
        }
        return hipErrorInvalidValue;
    }
    if (two) {
        if constexpr (!F::ZP) {
            if (mb == 2) {
                // One register buffer: the CU's other seven waves hide each wave's loads.
                // Against two buffers, alternated in one process (8192 x 57344, seven slabs, at
                // M = 24 / 32: 0.93-0.96x the time in two runs, even in a third; 72k x 18k,
                // nine slabs: 0.98-1.0x).  The form with one row block keeps two buffers: there
                // a single one measured anywhere from 3% faster to 6% slower.
                switch (ns) {
                case 7: return launch_skinny<2, 7, F, true, 1, true>(p, s);
                case 8: return launch_skinny<2, 8, F, true, 1, true>(p, s);
                case 9: return launch_skinny<2, 9, F, true, 1, true, true>(p, s);
                default: break;
                }
            }
        }
        return hipErrorInvalidValue;
    }
    // 17 rows and more: always the whole-line A loads; with four row blocks by DMA (their
    // registers are full; 10-15% faster than through registers at M = 64 and 128, while with
    // one row block the DMA form measured up to 14% slower at M = 16)
    if (mb == 4) {
        switch (ns) {
        case 1: return launch_skinny<4, 1, F, false, D, true, true>(p, s);
        case 2: return launch_skinny<4, 2, F, false, D, true, true>(p, s);
        case 3: return launch_skinny<4, 3, F, false, D, true, true>(p, s);
        case 4: return launch_skinny<4, 4, F, false, D, true, true>(p, s);
        case 5: return launch_skinny<4, 5, F, false, D, true, true>(p, s);
        case 6: return launch_skinny<4, 6, F, false, D, true, true>(p, s);
        case 7: return launch_skinny<4, 7, F, false, D, true, true>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (mb == 2) {
        switch (ns) {
        case 1: return launch_skinny<2, 1, F, false, D, true>(p, s);
        case 2: return launch_skinny<2, 2, F, false, D, true>(p, s);
        case 3: return launch_skinny<2, 3, F, false, D, true>(p, s);
        case 4: return launch_skinny<2, 4, F, false, D, true>(p, s);
        case 5: return launch_skinny<2, 5, F, false, D, true>(p, s);
        case 6: return launch_skinny<2, 6, F, false, D, true>(p, s);
        case 7: return launch_skinny<2, 7, F, false, D, true>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (fl) {
        switch (ns) {
        case 1: return launch_skinny<1, 1, F, false, D, true>(p, s);
        case 2: return launch_skinny<1, 2, F, false, D, true>(p, s);
        case 3: return launch_skinny<1, 3, F, false, D, true>(p, s);
        case 4: return launch_skinny<1, 4, F, false, D, true>(p, s);
        case 5: return launch_skinny<1, 5, F, false, D, true>(p, s);
        case 6: return launch_skinny<1, 6, F, false, D, true>(p, s);
        case 7: return launch_skinny<1, 7, F, false, D, true>(p, s);
        case 8: return launch_skinny<1, 8, F, false, D, true>(p, s);
        case 9: return launch_skinny<1, 9, F, false, D, true>(p, s);
        case 10: return launch_skinny<1, 10, F, false, D, true>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (ns) {
    case 1: return launch_skinny<1, 1, F>(p, s);
    case 2: return launch_skinny<1, 2, F>(p, s);
    case 3: return launch_skinny<1, 3, F>(p, s);
    case 4: return launch_skinny<1, 4, F>(p, s);
    case 5: return launch_skinny<1, 5, F>(p, s);
    case 6: return launch_skinny<1, 6, F>(p, s);
    case 7: return launch_skinny<1, 7, F>(p, s);
    case 8: return launch_skinny<1, 8, F>(p, s);
    case 9: return launch_skinny<1, 9, F>(p, s);
    case 10: return launch_skinny<1, 10, F>(p, s);
    default: return hipErrorInvalidValue;
    }
}

// The kernel for this configuration and format.
template <class F>
int dispatch(const Config &c, const Params &p, hipStream_t s)
{
    hipError_t e;
    if (c.NS > 0) {
        e = dispatch_skinny<F>(c.SMB, c.NS, c.TWO, c.DEEP, c.FL, p, s);
        return e == hipSuccess ? W4A16_OK : W4A16_EHIP;
    }
    switch (c.MB * 10 + c.NBW) {
    case 11: e = launch<1, 1, F>(p, s); break;
    case 12: e = launch<1, 2, F>(p, s); break;
    case 14: e = launch<1, 4, F>(p, s); break;
    case 21: e = launch<2, 1, F>(p, s); break;
    case 22: e = launch<2, 2, F>(p, s); break;
    case 24: e = launch<2, 4, F>(p, s); break;
    case 41: e = launch<4, 1, F>(p, s); break;
    case 42: e = launch<4, 2, F>(p, s); break;
    case 44: e = launch<4, 4, F>(p, s); break;
    case kWideMB * 10 + kWideNBW: e = launch_wide<kWaves, 2, F>(p, s); break;
    default: return W4A16_EHIP;
    }
    return e == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

}  // namespace

namespace w4a16_detail {

namespace {
std::mutex g_dev_mu;
DeviceInfo g_dev[64];
}  // namespace

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

}  // namespace w4a16_detail

using w4a16_detail::current_device;
using w4a16_detail::DeviceInfo;

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
    // the most any format's choice of kernel needs
    size_t b = kCounterBytes;
    if (M > 0) {
        b = std::max(workspace_for(choose_config(M, K, N, d.cus, false)),
                     workspace_for(choose_config(M, K, N, d.cus, true)));
        if (N % 256 == 0)
            b = std::max(b, workspace_for(choose_config_24(M, K, N, d.cus)));
    }
    *bytes = b;
    return W4A16_OK;
}

namespace {

// Arguments of w4a16_gemm_ex other than the workspace, checked; the current device in *d.
int check_gemm_args(const void *A, const uint32_t *packed, const uint16_t *params, void *C,
                    int M, int K, int N, int group, int zero_points, DeviceInfo *d)
{
    if (!A || !packed || !params || !C || (zero_points != 0 && zero_points != 1))
        return W4A16_EINVAL;
    int rc = check_gemm_shape(M, K, N);
    if (rc != W4A16_OK)
        return rc;
    if (group != kGroup && group != K)
        return W4A16_ESHAPE;
    return current_device(d);
}

// The product with checked arguments, configuration c and a workspace of workspace_for(c)
// bytes whose counter area is zero.
int gemm_run(const Config &c, const void *A, const uint32_t *packed, const uint16_t *params,
             void *C, int M, int K, int N, int group, int zero_points, void *workspace,
             const DeviceInfo &d, void *stream)
{
    // K = 128 makes the two scale granularities the same thing; take the grouped path
    const bool col = group != kGroup;
    Params p{};
    p.A = static_cast<const uint16_t *>(A);
    p.packed = reinterpret_cast<const u4 *>(packed);
    p.scales = params;
    p.C = static_cast<uint16_t *>(C);
    p.counters = static_cast<int *>(workspace);
    p.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    p.M = M;
    p.K = K;
    p.N = N;
    p.G = c.G;
    p.Gs = col ? 1 : c.G;
    p.P = c.P;
    p.S = c.S;
    p.W = c.W;
    p.T = c.T;
    p.gens = std::min(3, (c.W + d.cus - 1) / d.cus);
    p.KS = c.KS;
    p.SP = c.NS > 0 ? c.SP : 1;
    p.Kq = c.G / c.KS;
    p.Kr = c.G % c.KS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (zero_points)
        return col ? dispatch<Fmt<true, true>>(c, p, s) : dispatch<Fmt<true, false>>(c, p, s);
    return col ? dispatch<Fmt<false, true>>(c, p, s) : dispatch<FmtSym>(c, p, s);
}

}  // namespace

extern "C" int w4a16_gemm_ex(const void *A, const uint32_t *packed, const uint16_t *params,
                             void *C, int M, int K, int N, int group, int zero_points,
                             void *workspace, void *stream)
{
    if (!workspace)
        return W4A16_EINVAL;
    DeviceInfo d;
    const int rc = check_gemm_args(A, packed, params, C, M, K, N, group, zero_points, &d);
    if (rc != W4A16_OK || M == 0)
        return rc;
    return gemm_run(choose_config(M, K, N, d.cus, zero_points != 0), A, packed, params, C, M, K,
                    N, group, zero_points, workspace, d, stream);
}

namespace {

template <int MB, int NS, bool FL = false>
hipError_t launch_sparse(const Params &p, hipStream_t stream)
{
    hipLaunchKernelGGL((w4a16_gemm_sparse_kernel<MB, NS, FL>), dim3(p.W), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

// Most slabs per workgroup each row-block count allows without spilling (1, 2, 4 blocks of
// 16 rows hold 4, 8, 16 A registers per 32-k step and buffer).
constexpr int kSparseMaxNS[3] = {10, 6, 3};
constexpr int kSparseWholeKRows = 16;   // more rows: the stripe kernel

hipError_t dispatch_sparse(int mb, int ns, bool fl, const Params &p, hipStream_t s)
{
    if (fl) {
        switch (mb * 16 + ns) {
        case 17: return launch_sparse<1, 1, true>(p, s);
        case 18: return launch_sparse<1, 2, true>(p, s);
        case 19: return launch_sparse<1, 3, true>(p, s);
        case 20: return launch_sparse<1, 4, true>(p, s);
        case 21: return launch_sparse<1, 5, true>(p, s);
        case 22: return launch_sparse<1, 6, true>(p, s);
        case 23: return launch_sparse<1, 7, true>(p, s);
        case 24: return launch_sparse<1, 8, true>(p, s);
        case 25: return launch_sparse<1, 9, true>(p, s);
        case 26: return launch_sparse<1, 10, true>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (mb * 16 + ns) {
    case 17: return launch_sparse<1, 1>(p, s);
    case 18: return launch_sparse<1, 2>(p, s);
    case 19: return launch_sparse<1, 3>(p, s);
    case 20: return launch_sparse<1, 4>(p, s);
    case 21: return launch_sparse<1, 5>(p, s);
    case 22: return launch_sparse<1, 6>(p, s);
    case 23: return launch_sparse<1, 7>(p, s);
    case 24: return launch_sparse<1, 8>(p, s);
    case 25: return launch_sparse<1, 9>(p, s);
    case 26: return launch_sparse<1, 10>(p, s);
    case 33: return launch_sparse<2, 1>(p, s);
    case 34: return launch_sparse<2, 2>(p, s);
    case 35: return launch_sparse<2, 3>(p, s);
    case 36: return launch_sparse<2, 4>(p, s);
    case 37: return launch_sparse<2, 5>(p, s);
    case 38: return launch_sparse<2, 6>(p, s);
    case 65: return launch_sparse<4, 1>(p, s);
    case 66: return launch_sparse<4, 2>(p, s);
    case 67: return launch_sparse<4, 3>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" int w4a16_gemm_24(const void *A, const uint32_t *packed, const uint16_t *scales,
                             void *C, int M, int K, int N, void *workspace, void *stream)
{
    if (!A || !packed || !scales || !C || !workspace || M < 0 || K < 0 || N < 0)
        return W4A16_EINVAL;
    int rc = check_gemm_shape(M, K, N);
    if (rc != W4A16_OK)
        return rc;
    // 256-column parameter groups; the whole-K kernel's dead loads point 2 GiB past the
    // buffer starts
    if (N % 256 || static_cast<uint64_t>(K) * static_cast<uint64_t>(N) * 3 / 8 >= kOutside ||
        static_cast<uint64_t>(64) * static_cast<uint64_t>(K) * 2 >= kOutside)
        return W4A16_ESHAPE;
    DeviceInfo d;
    rc = current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    if (M == 0)
        return W4A16_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Params p{};
    p.A = static_cast<const uint16_t *>(A);
    p.packed = reinterpret_cast<const u4 *>(packed);
    p.scales = scales;
    p.C = static_cast<uint16_t *>(C);
    p.counters = static_cast<int *>(workspace);
    p.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    p.M = M;
    p.K = K;
    p.N = N;
    p.G = K / kGroup;
    p.Gs = p.G;
    if (M <= kSparseWholeKRows) {
        // whole-K workgroups of NS slabs, two per CU
        const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        const int S = N / 16;
        const int per = 2 * d.cus;
        const int ns = std::min((S + per - 1) / per, kSparseMaxNS[mb == 1 ? 0 : (mb == 2 ? 1 : 2)]);
        p.P = 1;
        p.W = (S + ns - 1) / ns;
        p.gens = std::min(3, (p.W + d.cus - 1) / d.cus);
        // whole-line A loads above 8 rows over at least 8 K tiles a wave (as the dense kernel)
        const bool fl = mb == 1 && M > 8 && p.G >= 8 * kWaves;
        return dispatch_sparse(mb, ns, fl, p, s) == hipSuccess ? W4A16_OK : W4A16_EHIP;
    }
    const Config c = choose_config_24(M, K, N, d.cus);
    p.P = c.P;
    p.S = c.S;
    p.W = c.W;
    p.T = c.T;
    p.gens = std::min(3, (c.W + d.cus - 1) / d.cus);
    const hipError_t e = c.MB == 1   ? launch<1, 4, FmtSp>(p, s)
                         : c.MB == 2 ? launch<2, 4, FmtSp>(p, s)
                                     : launch<4, 4, FmtSp>(p, s);
    return e == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

extern "C" int w4a16_gemm(const void *A, const uint32_t *packed, const uint16_t *scales, void *C,
                          int M, int K, int N, void *workspace, void *stream)
{
    return w4a16_gemm_ex(A, packed, scales, C, M, K, N, kGroup, 0, workspace, stream);
}

// ------------------------------------------------------- entry point that allocates nothing
//
// w4a16_gemm_noalloc is w4a16_gemm_ex with the workspace taken from a file-scope device array
// (one per GPU, held until the process ends), for callers that cannot allocate.  In host code
// the array's name stands for a host-side shadow, not a device address: each device's address
// is fetched once with hipGetSymbolAddress, with that device current, and only that address
// is ever handed to a kernel.  The counter area starts at zero (a device global without an
// initialiser is zero-filled when the code object loads, and the first call on a device
// clears it again on the caller's stream with a small kernel, not a memset); every call
// leaves it zero.  The partial slots need no clearing.
constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == kCounterBytes + (size_t(128) << 20), "counters + 128 MiB");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch[64];           // per device: the array's device address, once fetched

__global__ void zero_words_kernel(uint32_t *p, int n)
{
    const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

// This device's scratch address (fetching it, and clearing the counters on `stream`, on the
// first call per device).
int scratch_for_device(hipStream_t stream, void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return W4A16_EHIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return W4A16_EHIP;
        constexpr int words = static_cast<int>(kCounterBytes / 4);
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t *>(ptr), words);
        if (hipGetLastError() != hipSuccess)
            return W4A16_EHIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return W4A16_OK;
}

}  // namespace

extern "C" int w4a16_gemm_noalloc(const void *A, const uint32_t *packed, const uint16_t *params,
                                  void *C, int M, int K, int N, int group, int zero_points,
                                  void *stream)
{
    DeviceInfo d;
    const int rc = check_gemm_args(A, packed, params, C, M, K, N, group, zero_points, &d);
    if (rc != W4A16_OK || M == 0)
        return rc;
    const Config c = choose_config(M, K, N, d.cus, zero_points != 0);
    if (workspace_for(c) > kScratchBytes)
        return W4A16_ESHAPE;
    void *ws = nullptr;
    const int rs = scratch_for_device(static_cast<hipStream_t>(stream), &ws);
    if (rs != W4A16_OK)
        return rs;
    return gemm_run(c, A, packed, params, C, M, K, N, group, zero_points, ws, d, stream);
}
