// Grouped W4A16 product of a mixture-of-experts layer on gfx950: every token row meets the
// weights of the experts its router picked, each expert with its own number of rows.
//
// The pages (deep-dive page, section on where the format stops paying off, items 1 and 4):
// an MoE layer regroups the tokens by expert, so each expert's GEMM sees its own M, not the
// batch's, and the grouped product is scheduled differently from a dense layer.  Here:
//
// * w4a16_moe_align: the regrouping.  The assignments a = t * topk + j (token t, its j-th
//   expert) are sorted by expert with a stable counting sort, so expert e's rows are
//   sorted_ids[offsets[e] .. offsets[e + 1]) in increasing a.  One workgroup; ranks inside
//   a wave come from ballots, so the order is deterministic.
// * w4a16_moe_gemm: one launch for all experts.  Workgroup (e, s) owns NS 16-column slabs
//   of expert e over the whole K range (the whole-K scheme of the dense kernel for few
//   rows: four waves split K, partial sums meet in LDS, no output shared between
//   workgroups); an expert's weights are read only if a token uses it.  With no more
//   assignments than experts the launch holds min(E, T * topk) rows of workgroups; each
//   workgroup counts the rows of every expert and takes a slab group of the (blockIdx / WE)-th
//   expert in use, so the workgroups of the experts in use are dispatched first whichever
//   experts they are.  Otherwise workgroup row e serves expert e, idle ones return at once.  Each lane gathers its own A row (row a / topk of A)
//   and scatters its outputs to rows a of C, so no permuted copy of A or C is made.
//   An expert's rows go through in passes of up to MBX 16-row blocks, each pass streaming
//   the workgroup's slab weights once for all its blocks; the launch sizes MBX for the
//   busiest expert expected, and each expert takes the fewest passes that cover its rows.
// * fp16 activations: the dense kernels' exact decode (q - z in fp16 by mask-and-OR into
//   the exponent 0x6400 and one packed add or FMA per pair), fp32 sums over each 128-row
//   group, one scale FMA per output and group.
// * bf16 activations (and bf16 scales): gfx950 has bf16 matrix instructions but no packed
//   bf16 add or multiply, so the codes are fed as they come: mask-and-OR into the bf16
//   exponent 0x4300 gives 128 + q exactly (7 VALU ops per 8 weights), the MFMA sums
//   A * (128 + q) over the group, and (128 + z) * sum_k A is subtracted per row and group
//   before the scale: sum_k A (q - z) = sum_k A (128 + q) - (128 + z) sum_k A.  The row sums
//   come from the same MFMA against a ones operand (4 extra instructions per 16 rows and
//   group, shared by every slab).  The fp32 error this adds is near 2^-24 * 136 relative to
//   the group's sum of |A|, far below bf16's 2^-9.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "w4a16.h"
#include "device.h"
#include "kernel_common.h"

namespace {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// ----------------------------------------------------------------------------- regrouping

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ uint64_t ballot(bool p)
{
    return __builtin_amdgcn_ballot_w64(p);
}

// Lanes below this one.
__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(kAlignThreads) void moe_align_kernel(const int32_t *__restrict__ ids,
                                                                  int R, int E,
                                                                  int32_t *__restrict__ sorted,
                                                                  int32_t *__restrict__ offsets)
{
    __shared__ int cnt[kAlignWaves][kMaxExperts];   // per round: wave w's rows of expert e
    __shared__ int base[kMaxExperts];               // next free position of expert e
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    for (int e = tid; e < E; e += kAlignThreads) {
        base[e] = 0;
#pragma unroll
        for (int w = 0; w < kAlignWaves; ++w)
            cnt[w][e] = 0;
    }
    __syncthreads();
    // totals (order-free: LDS atomics)
    for (int a = tid; a < R; a += kAlignThreads) {
        const int e = ids[a];
        if (e >= 0 && e < E)
            atomicAdd(&base[e], 1);
    }
    __syncthreads();
    // Exclusive scan of the totals, by one wave: lane j adds up experts [jc, (j+1)c) with
    // c = ceil(E / 64), the 64 lane sums are scanned across the wave, and each lane hands out
    // its experts' bases.
    if (wave == 0) {
        const int c = (E + 63) / 64;
        const int e0 = lane * c, e1 = e0 + c < E ? e0 + c : E;
        int sum = 0;
        for (int x = e0; x < e1; ++x)
            sum += base[x];
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += y;
        }
        int run = incl - sum;
        for (int x = e0; x < e1; ++x) {
            const int v = base[x];
            base[x] = run;
            offsets[x] = run;
            run += v;
        }
        if (lane == 63)
            offsets[E] = incl;
    }
    __syncthreads();

    // Stable scatter, kAlignThreads assignments per round.  In each wave, lanes holding the
    // same expert find each other with ballots (one pass per distinct expert in the wave);
    // a lane's position is its expert's base, plus that expert's rows in lower waves of the
    // round, plus its rank among the lower lanes of its own wave.
    for (int a0 = 0; a0 < R; a0 += kAlignThreads) {
        const int a = a0 + tid;
        const int e = a < R ? ids[a] : -1;
        const bool valid = e >= 0 && e < E;
        int rank = 0;
        uint64_t todo = ballot(valid);
        while (todo) {
            const int leader = __builtin_ctzll(todo);
            const int v = __builtin_amdgcn_readlane(e, leader);
            const uint64_t same = ballot(valid && e == v);
            if (valid && e == v)
                rank = __builtin_popcountll(same & lanes_below(lane));
            if (lane == leader)
                cnt[wave][v] = __builtin_popcountll(same);
            todo &= ~same;
        }
        __syncthreads();
        if (valid) {
            int pos = base[e] + rank;
            for (int w = 0; w < wave; ++w)
                pos += cnt[w][e];
            sorted[pos] = a;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kAlignThreads) {
            int t = 0;
#pragma unroll
            for (int w = 0; w < kAlignWaves; ++w) {
                t += cnt[w][x];
                cnt[w][x] = 0;
            }
            base[x] += t;
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------------------- grouped GEMM

struct MoeParams {
    const uint16_t *A;          // [T][K], fp16 or bf16
    const u4 *packed;           // E experts, K * N / 8 words each (w4a16_pack layout)
    const uint16_t *params;     // E experts, G * N halves each (2 G N with zero points)
    const int32_t *sorted;      // assignments grouped by expert (presorted entry)
    const int32_t *offsets;     // [E + 1] (presorted entry)
    const int32_t *topk_ids;    // [T * topk] (routing entry)
    const float *row_scale;     // [T * topk] or null
    uint16_t *C;                // [T * topk][N]
    int T, topk, E, K, N, G;
    int WE;                     // workgroups per expert
    int compact;                // 1: workgroups go to the experts in use only (see the kernel)
};

// Parameter groups a workgroup's NS slabs can touch, and dwords holding NS halves.
template <int NS>
struct MoeGroups {
    static constexpr int n = (NS + 6) / 4;
    static constexpr int nh = (NS + 1) / 2;
};

template <int MB, int NS, bool ZP, bool BF>
struct MoeBuf {
    u4 w[NS];                                 // weight quads, one per slab
    u4 a[MB][4];                              // A fragments, 4 32-k steps per 16-row block
    uint32_t p[MoeGroups<NS>::n][ZP ? 4 : 2]; // per-group parameters of the lane's column
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b)
{
    return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float x)
{
    // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Routing inside the product (w4a16_moe_gemm_topk): the workgroup lists expert e's
// assignments itself.  Wave w scans a contiguous quarter of topk_ids, 64 ids per ballot, all
// its loads issued before the first ballot; the waves' counts meet in LDS, and each wave
// writes its matches at its offset.  The list comes out in increasing order, as
// w4a16_moe_align's, so both entries put the same rows in the same blocks.
constexpr int kRouteMax = 2048;                          // assignments the routing entry takes
constexpr int kTrRows = 16 * 17;                         // LDS chunks of one transposed block

__device__ __forceinline__ int route_rows(const int32_t *__restrict__ ids, int R, int e, int wave,
                                          int lane, int *rlist, int *wcnt)
{
    constexpr int kChunks = kRouteMax / (64 * kWaves);
    const int per = (R + 64 * kWaves - 1) / (64 * kWaves) * 64;    // ids per wave
    const int a0 = wave * per;
    int ev[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int a = a0 + 64 * i + lane;
        ev[i] = (64 * i < per && a < R) ? ids[a] : -1;
    }
    uint64_t m[kChunks];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        m[i] = ballot(ev[i] == e);
        cnt += __builtin_popcountll(m[i]);
    }
    if (lane == 0)
        wcnt[wave] = cnt;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = wcnt[w];
        base += w < wave ? c : 0;
        total += c;
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        if (ev[i] == e)
            rlist[base + __builtin_popcountll(m[i] & lanes_below(lane))] = a0 + 64 * i + lane;
        base += __builtin_popcountll(m[i]);
    }
    __syncthreads();
    return total;
}

// The k-th expert (in expert order) that has rows, from the row counts in LDS, or -1 if fewer
// than k + 1 experts have rows.  Wave 0 counts the experts with rows in each lane's run of
// ceil(E / 64) experts, scans the counts across the wave, and the lane whose run holds the
// k-th walks it.  Every thread gets the answer (through LDS).
__device__ __forceinline__ int kth_active_expert(const int *cnt, int E, int k, int wave,
                                                 int lane, int *out)
{
    if (wave == 0) {
        const int c = (E + 63) / 64;
        const int e0 = lane * c, e1 = e0 + c < E ? e0 + c : E;
        int n = 0;
        for (int x = e0; x < e1; ++x)
            n += cnt[x] > 0 ? 1 : 0;
        int incl = n;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += y;
        }
        int r = incl - n;
        if (k >= r && k < incl) {
            for (int x = e0; x < e1; ++x)
                if (cnt[x] > 0) {
                    if (r == k)
                        *out = x;
                    ++r;
                }
        }
        if (lane == 63 && k >= incl)
            *out = -1;
    }
    __syncthreads();
    return *out;
}

template <int MBX, int NS, bool ZP, bool BF, bool RT, int DEPTH = 2>
__global__ __launch_bounds__(kThreads, 2) void w4a16_moe_kernel(MoeParams p)
{
    using MG = MoeGroups<NS>;
    constexpr int NG = MG::n, NH = MG::nh;
    constexpr uint32_t PB = ZP ? 16 : 8;                 // parameter bytes per column and group
    // partial sums after the K loop; during it, the waves' A transposes (FL passes)
    __shared__ u4 red_q[std::max(kWaves * MBX * NS * 64, kWaves * std::min(MBX, 2) * kTrRows)];
    f4 *red = reinterpret_cast<f4 *>(red_q);
    __shared__ int rlist[RT ? kRouteMax : 1];            // expert e's assignments (RT)
    __shared__ int wcnt[kWaves];
    __shared__ int ecnt[kMaxExperts];                    // rows per expert
    __shared__ int picked;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    // compact: workgroup b takes slab group b % WE of the (b / WE)-th expert that has rows,
    // so the experts in use fill the lowest workgroup ids and the rest return at once (when
    // most experts are idle).  Otherwise expert b / WE, and workgroups of idle experts return.
    int e = static_cast<int>(blockIdx.x) / p.WE;
    if (p.compact) {
        if constexpr (RT) {
            for (int x = tid; x < p.E; x += kThreads)
                ecnt[x] = 0;
            __syncthreads();
            const int R = p.T * p.topk;
            for (int a = tid; a < R; a += kThreads) {
                const int x = p.topk_ids[a];
                if (x >= 0 && x < p.E)
                    atomicAdd(&ecnt[x], 1);
            }
        } else {
            for (int x = tid; x < p.E; x += kThreads)
                ecnt[x] = p.offsets[x + 1] - p.offsets[x];
        }
        __syncthreads();
        e = kth_active_expert(ecnt, p.E, e, wave, lane, &picked);
        if (e < 0)
            return;
    }
    const int j0 = (static_cast<int>(blockIdx.x) % p.WE) * NS;   // first slab of the workgroup
    int row0 = 0, rows;
    if constexpr (RT) {
        rows = route_rows(p.topk_ids, p.T * p.topk, e, wave, lane, rlist, wcnt);
    } else {
        row0 = p.offsets[e];
        rows = p.offsets[e + 1] - row0;
    }
    if (rows <= 0)
        return;
    // assignment of the expert's i-th row
    auto row_of = [&](int i) __attribute__((always_inline)) {
        if constexpr (RT)
            return rlist[i];
        else
            return p.sorted[row0 + i];
    };
    const int c = lane & 15, quad = lane >> 4;
    const int S = p.N >> 4;
    const int U = S >> 2;
    const int u0 = j0 >> 2, r = j0 & 3;
    const int g0 = p.G * wave / kWaves;
    const int g1 = p.G * (wave + 1) / kWaves;

    const size_t ew = static_cast<size_t>(p.K) * p.N / 2;               // weight bytes / expert
    const size_t ep = static_cast<size_t>(p.G) * p.N * (ZP ? 2 : 1);    // params / expert
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A, static_cast<uint32_t>(p.T) * static_cast<uint32_t>(p.K) * 2u);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(
        reinterpret_cast<const char *>(p.packed) + static_cast<size_t>(e) * ew,
        static_cast<uint32_t>(ew));
    const __amdgpu_buffer_rsrc_t rS =
        make_rsrc(p.params + static_cast<size_t>(e) * ep, static_cast<uint32_t>(ep * 2));
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(
        p.C, static_cast<uint32_t>(p.T) * static_cast<uint32_t>(p.topk) *
                 static_cast<uint32_t>(p.N) * 2u);

    const uint32_t mlo = in_vgpr(0x000f000fu), mhi = in_vgpr(0x00f000f0u);
    const uint32_t magic = in_vgpr(BF ? 0x43004300u : 0x64006400u);
    const uint32_t magic_hi = in_vgpr(0x54005400u);   // fp16 raw decode of the high nibbles
    const uint32_t v_par = static_cast<uint32_t>(c) * PB;
    auto slab = [&](int i) __attribute__((always_inline)) {
        const int j = j0 + i;
        return j < S ? j : S - 1;          // slabs past N re-read the last one; never stored
    };
    const bool sel_dw = (r & 2) != 0, sel_half = (r & 1) != 0;     // uniform
    // halves r .. r + NS - 1 of the concatenated groups (part 0: scales, 1: zero terms)
    auto pick = [&](const uint32_t (&pg)[NG][ZP ? 4 : 2], int part, uint32_t (&out)[NH])
        __attribute__((always_inline)) {
        auto D = [&](int m) __attribute__((always_inline)) {
            m = m < 2 * NG ? m : 2 * NG - 1;
            return pg[m >> 1][2 * part + (m & 1)];
        };
        uint32_t x[NH + 1];
#pragma unroll
        for (int m = 0; m <= NH; ++m)
            x[m] = sel_dw ? D(m + 1) : D(m);
#pragma unroll
        for (int m = 0; m < NH; ++m)
            out[m] = sel_half ? __builtin_amdgcn_alignbit(x[m + 1], x[m], 16) : x[m];
    };

    // One pass over the K tiles for the row blocks [rb, rb + 16 MB): each weight tile loaded
    // feeds every row block of the pass.
    auto pass = [&](auto mb_count, auto fl_flag, int rb) __attribute__((always_inline)) {
        constexpr int MB = decltype(mb_count)::value;
        // FL (passes of one block with more than 8 rows, or of two, over at least 8 K tiles a
        // wave): the load of step t brings rows 4t .. 4t + 3 of a block, 16 lanes a row, as
        // whole 128-byte lines, and the wave puts them in fragment order through its LDS
        // region (compute), as the dense whole-K kernel does.  With up to 8 rows the fragment
        // layout's loads of rows past the expert's touch no memory, and over few K tiles the
        // LDS round trip's latency shows: there it would only cost (64 experts, K = 1408 and
        // 2048: 1-4% slower); with four blocks the registers are full.
        constexpr bool FL = decltype(fl_flag)::value;
        static_assert(!FL || MB <= 2, "registers");
        constexpr int NA = FL ? 4 : 1;
        // the lane's A row (token a / topk of assignment a) per block (and step, FL)
        uint32_t v_a[MB][NA];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < NA; ++t) {
                const int i = rb + 16 * mb + (FL ? 4 * t + quad : c);
                v_a[mb][t] = kOutside;
                if (i < rows) {
                    const int a = row_of(i);
                    v_a[mb][t] = (static_cast<uint32_t>(a / p.topk) * p.K + 8 * (FL ? c : quad)) * 2;
                }
            }

        auto load = [&](MoeBuf<MB, NS, ZP, BF> &b, int g) __attribute__((always_inline)) {
            const bool live = g < g1;
            const uint32_t vw = live ? static_cast<uint32_t>(lane) * 16 : kOutside;
            const uint32_t vp = live ? v_par : kOutside;
            const int gg = live ? g : g1 - 1;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    b.a[mb][t] = __builtin_bit_cast(
                        u4, __builtin_amdgcn_raw_buffer_load_b128(
                                rA, live ? v_a[mb][FL ? t : 0] : kOutside,
                                static_cast<uint32_t>(gg * kGroup + (FL ? 0 : 32 * t)) * 2, 0));
#pragma unroll
            for (int i = 0; i < NS; ++i)
                b.w[i] = __builtin_bit_cast(
                    u4, __builtin_amdgcn_raw_buffer_load_b128(
                            rW, vw, (static_cast<uint32_t>(slab(i)) * p.G + gg) * 1024u,
                            kNonTemporal));
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                const int u = u0 + k < U ? u0 + k : U - 1;
                const uint32_t so = (static_cast<uint32_t>(u) * p.G + gg) * (16u * PB);
                if constexpr (ZP) {
                    const u4 v = __builtin_bit_cast(
                        u4, __builtin_amdgcn_raw_buffer_load_b128(rS, vp, so, 0));
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        b.p[k][d] = v[d];
                } else {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rS, vp, so, 0);
                    b.p[k][0] = v[0];
                    b.p[k][1] = v[1];
                }
            }
        };

        f4 acc[MB][NS];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < NS; ++i)
                acc[mb][i] = f4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](MoeBuf<MB, NS, ZP, BF> &b) __attribute__((always_inline)) {
            if constexpr (FL) {
                // rows 4t .. 4t + 3 of step t -> the wave's region (rows of 17 chunks: the 16
                // rows read at one chunk fall in 16 bank groups) -> fragment order, in place;
                // a wave's LDS operations complete in order
                u4 *reg = red_q + wave * (MB * kTrRows);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        reg[(16 * mb + 4 * t + quad) * 17 + c] = b.a[mb][t];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        b.a[mb][t] = reg[(16 * mb + c) * 17 + 4 * t + quad];
            }
            uint32_t sh[NH], zh[NH];
            pick(b.p, 0, sh);
            if constexpr (ZP)
                pick(b.p, 1, zh);
            float sf[NS];
            uint32_t zb[NS];
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const uint32_t sb = (sh[i >> 1] >> (16 * (i & 1))) & 0xffffu;
                sf[i] = BF ? bf16_bits_to_float(sb) : half_bits_to_float(static_cast<uint16_t>(sb));
                asm volatile("" : "+v"(sf[i]));
                zb[i] = ZP ? (zh[i >> 1] >> (16 * (i & 1))) & 0xffffu : 0x6408u;
            }
            if constexpr (BF) {
                // A * (128 + q) per group, minus (128 + z) times the group's row sums of A
                const u4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
                f4 rs[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    rs[mb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        rs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(b8, b.a[mb][t]), __builtin_bit_cast(b8, ones),
                            rs[mb], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    f4 part[MB];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t w = b.w[i][t];
                        const u4 x = {and_or(w, mlo, magic), and_or(w >> 4, mlo, magic),
                                      and_or(w >> 8, mlo, magic), and_or(w >> 12, mlo, magic)};
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            const f4 cin = t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : part[mb];
                            part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(b8, b.a[mb][t]), __builtin_bit_cast(b8, x),
                                cin, 0, 0, 0);
                        }
                    }
                    const float nz = -static_cast<float>(128 + (zb[i] & 15u));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mb][i][q] = __builtin_fmaf(
                                sf[i], __builtin_fmaf(nz, rs[mb][q], part[mb][q]), acc[mb][i][q]);
                        asm volatile("" : "+v"(acc[mb][i]));
                    }
                }
            } else if constexpr (!ZP) {
                // symmetric: the dense whole-K kernel's raw decode, the same arithmetic in the
                // same order (per row block the chain of A * offsets, per slab the chain of
                // A * raw codes, their difference scaled into the sums), so a row equals the
                // dense product's bit for bit
                const h8 off = raw_offsets();
                f4 P[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        P[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(h8, b.a[mb][t]), off,
                            t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : P[mb], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    f4 D[MB];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const h8 x = raw8(b.w[i][t], mlo, mhi, magic, magic_hi);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            D[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(h8, b.a[mb][t]), x,
                                t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : D[mb], 0, 0, 0);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const f4 part = D[mb] - P[mb];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mb][i][q] = __builtin_fmaf(sf[i], part[q], acc[mb][i][q]);
                        asm volatile("" : "+v"(acc[mb][i]));
                    }
                }
            } else {
                // exact q - z per group in fp16, one scale FMA per output
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const _Float16 zt = __builtin_bit_cast(_Float16, static_cast<uint16_t>(zb[i]));
                    const h2 zsub = {zt, zt};
                    const h2 k960 = {static_cast<_Float16>(960.0f), static_cast<_Float16>(960.0f)};
                    const h2 zadd = k960 - zsub;
                    f4 part[MB];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const h8 x = dequant8(b.w[i][t], mlo, mhi, magic, zsub, zadd);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            const f4 cin = t == 0 ? f4{0.f, 0.f, 0.f, 0.f} : part[mb];
                            part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(h8, b.a[mb][t]), x, cin, 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mb][i][q] = __builtin_fmaf(sf[i], part[mb][q], acc[mb][i][q]);
                        asm volatile("" : "+v"(acc[mb][i]));
                    }
                }
            }
        };

        if (g0 < g1) {
            // DEPTH buffers (D - 1 tiles of weights in flight while one is computed), one loop
            // exit, memory fences: as the dense whole-K kernel
            constexpr int D = DEPTH;
            MoeBuf<MB, NS, ZP, BF> b[D];
#pragma unroll
            for (int d = 0; d < D; ++d) {
                load(b[d], g0 + d);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
            const int rounds = (g1 - g0) / D;
            int g = g0;
            for (int it = 0; it < rounds; ++it) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    compute(b[d]);
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                    load(b[d], g + d + D);
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                }
                g += D;
            }
#pragma unroll
            for (int d = 0; d < D - 1; ++d)
                if (g + d < g1)
                    compute(b[d]);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        if constexpr (FL)
            __syncthreads();                // every wave is done with its transposes (red_q)

        // Partial sums meet in LDS; wave w finishes slabs w, w + 4, ...  Result lane l holds
        // rows 16 mb + 4(l/16) + 0..3 of the block, column 16j + l % 16.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < NS; ++i)
                red[((wave * MB + mb) * NS + i) * 64 + lane] = acc[mb][i];
        __syncthreads();
        int orow[MB][4];                    // output row (assignment) of each result, or -1
        float osc[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = rb + 16 * mb + 4 * quad + q;
                orow[mb][q] = i < rows ? row_of(i) : -1;
                osc[mb][q] = (p.row_scale && orow[mb][q] >= 0) ? p.row_scale[orow[mb][q]] : 1.0f;
            }
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
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float y = v[q] * osc[mb][q];
                        const uint16_t h = BF ? float_to_bf16_bits(y) : float_to_half_bits(y);
                        const uint32_t off =
                            orow[mb][q] >= 0
                                ? (static_cast<uint32_t>(orow[mb][q]) * p.N + 16 * (j0 + i) + c) * 2
                                : kOutside;
                        __builtin_amdgcn_raw_buffer_store_b16(h, rC, off, 0, 0);
                    }
                }
            }
        }
        __syncthreads();                    // red is reused by the next pass
    };

    // Passes of MBX, MBX / 2 or one row block: while more rows are left than half the largest
    // pass holds, the largest (so 17..32 rows take one pass of two blocks, 33..64 one of four,
    // its blocks past the rows reading no memory), then the smallest that covers the rest.
    using yes = std::true_type;
    using no = std::false_type;
    const bool fl_ok = p.G >= 8 * kWaves;             // at least 8 K tiles a wave
    for (int rb = 0; rb < rows;) {
        const int left = rows - rb;
        if constexpr (MBX >= 4) {
            if (left > 32) {
                pass(std::integral_constant<int, 4>{}, no{}, rb);
                rb += 64;
                continue;
            }
        }
        if constexpr (MBX >= 2) {
            if (left > 16) {
                if (fl_ok)
                    pass(std::integral_constant<int, 2>{}, yes{}, rb);
                else
                    pass(std::integral_constant<int, 2>{}, no{}, rb);
                rb += 32;
                continue;
            }
        }
        if (left > 8 && fl_ok)
            pass(std::integral_constant<int, 1>{}, yes{}, rb);
        else
            pass(std::integral_constant<int, 1>{}, no{}, rb);
        rb += 16;
    }
}

template <int MB, int NS, bool ZP, bool BF, bool RT, int DEPTH = 2>
hipError_t launch_moe(const MoeParams &p, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL((w4a16_moe_kernel<MB, NS, ZP, BF, RT, DEPTH>), dim3(blocks), dim3(kThreads),
                       0, s, p);
    return hipGetLastError();
}

template <bool ZP, bool BF, bool RT>
hipError_t dispatch_moe(int mb, int ns, bool deep, const MoeParams &p, int blocks, hipStream_t s)
{
    if (deep) {
        switch (mb * 16 + ns) {
        case 17: return launch_moe<1, 1, ZP, BF, RT, 3>(p, blocks, s);
        case 18: return launch_moe<1, 2, ZP, BF, RT, 3>(p, blocks, s);
        case 20: return launch_moe<1, 4, ZP, BF, RT, 3>(p, blocks, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (mb * 16 + ns) {
    case 17: return launch_moe<1, 1, ZP, BF, RT>(p, blocks, s);
    case 18: return launch_moe<1, 2, ZP, BF, RT>(p, blocks, s);
    case 20: return launch_moe<1, 4, ZP, BF, RT>(p, blocks, s);
    case 33: return launch_moe<2, 1, ZP, BF, RT>(p, blocks, s);
    case 34: return launch_moe<2, 2, ZP, BF, RT>(p, blocks, s);
    case 36: return launch_moe<2, 4, ZP, BF, RT>(p, blocks, s);
    case 38: return launch_moe<2, 6, ZP, BF, RT>(p, blocks, s);
    case 65: return launch_moe<4, 1, ZP, BF, RT>(p, blocks, s);
    case 66: return launch_moe<4, 2, ZP, BF, RT>(p, blocks, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool RT>
hipError_t dispatch_moe_fmt(bool zp, bool bf, int mb, int ns, bool deep, const MoeParams &p,
                            int blocks, hipStream_t s)
{
    if (zp)
        return bf ? dispatch_moe<true, true, RT>(mb, ns, deep, p, blocks, s)
                  : dispatch_moe<true, false, RT>(mb, ns, deep, p, blocks, s);
    return bf ? dispatch_moe<false, true, RT>(mb, ns, deep, p, blocks, s)
              : dispatch_moe<false, false, RT>(mb, ns, deep, p, blocks, s);
}

// Checks shared by both entries, the launch shape, and the launch.  `routed`: the product
// lists each expert's rows itself from p.topk_ids.
int moe_run(MoeParams &p, int zero_points, int act_dtype, bool routed, void *stream)
{
    const int T = p.T, topk = p.topk, E = p.E, K = p.K, N = p.N;
    if (!p.A || !p.packed || !p.params || !p.C || T < 0 || topk < 1 || E < 1 || K < 0 ||
        N < 0 || (zero_points != 0 && zero_points != 1) ||
        (act_dtype != W4A16_ACT_F16 && act_dtype != W4A16_ACT_BF16))
        return W4A16_EINVAL;
    if (K == 0 || K % kGroup || N == 0 || N % 256 || E > kMaxExperts)
        return W4A16_ESHAPE;
    // 32-bit buffer offsets, and the dead loads' offset above every buffer
    const uint64_t R = static_cast<uint64_t>(T) * static_cast<uint64_t>(topk);
    if (static_cast<uint64_t>(K) * static_cast<uint64_t>(N) / 2 >= kOutside ||
        static_cast<uint64_t>(T) * static_cast<uint64_t>(K) * 2 >= kOutside ||
        R * static_cast<uint64_t>(N) * 2 >= kOutside ||
        static_cast<uint64_t>(K / kGroup) * static_cast<uint64_t>(N) * 4 >= kOutside ||
        (routed && R > static_cast<uint64_t>(kRouteMax)))
        return W4A16_ESHAPE;
    w4a16_detail::DeviceInfo d;
    const int rc = w4a16_detail::current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    if (T == 0)
        return W4A16_OK;

    // Most row blocks per pass (mb): enough for the busiest expert expected, so that its
    // weights are streamed once.  Under even routing the largest of E binomial counts of mean
    // m lies near m + sqrt(2 m ln E); half that spread again allows for routers that favour
    // some experts.  Each expert takes the fewest passes that cover its own rows (one 16-row
    // pass for 16 rows or fewer, whatever mb is), but mb sets the kernel's registers: one
    // block per pass leaves room for more workgroups per CU.  Four slabs per workgroup (as
    // many weight loads per K step as A loads with 16-row blocks), two with 64-row passes
    // (registers), fewer only while the experts in use -- at most min(E, T * topk) -- would
    // not give every CU a workgroup.
    const double mean_rows = static_cast<double>(R) / E;
    const double busiest =
        mean_rows + 1.5 * std::sqrt(2.0 * std::log(static_cast<double>(E)) * mean_rows);
    const int mb = busiest <= 16.0 ? 1 : (busiest <= 32.0 ? 2 : 4);
    const long long S = N / 16;
    const long long active = std::min<long long>(E, static_cast<long long>(R));
    int ns = mb == 4 ? 2 : 4;
    // Passes of two blocks over many workgroups (at least two rounds of two per CU): six
    // slabs, more weight bytes per A fragment, measured 9% faster (8 experts x 28672 wide at
    // T = 64: 111 -> 101 us; 64 experts x 2816: 46.6 -> 42.3 us); with fewer workgroups six
    // slabs leave CUs idle (8 experts x 4096 wide: 73 -> 81 us).
    if (mb == 2 && active * ((S + 5) / 6) >= 4LL * d.cus)
        ns = 6;
    while (ns > 1 && active * ((S + ns - 1) / ns) < d.cus)
        ns /= 2;
    p.G = K / kGroup;
    p.WE = static_cast<int>((S + ns - 1) / ns);
    // With no more assignments than experts, many experts are idle: the launch holds one row
    // of workgroups per expert that can have rows (min(E, T * topk)), given to the experts in
    // use in order (64 experts, top 6, T = 1: 11.5 -> 9.0 us; 8 experts, top 2, T = 4: 32.1 ->
    // 24.0 us).  With more, counting every expert's rows first costs 1-2 us a workgroup
    // (64 experts, T = 64: 25.4 -> 27.7 us) and every expert gets a row of workgroups.
    p.compact = static_cast<long long>(R) <= E ? 1 : 0;
    const long long blocks = static_cast<long long>(p.WE) * (p.compact ? active : E);
    if (blocks > INT_MAX)
        return W4A16_ESHAPE;
    // One pass of one block, at most a workgroup per CU and a long K (at least 16 K tiles a
    // wave): the waves' weight streams are latency-bound, and a third buffer (two tiles in
    // flight) measured 10% faster (8 experts x 14336 x 4096 at T = 1: 20.2 -> 18.2 us); with
    // more workgroups or passes it measured slower (its registers spill with two blocks).
    const bool deep = mb == 1 && blocks <= d.cus && p.G >= 16 * kWaves;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = act_dtype == W4A16_ACT_BF16;
    const int nb = static_cast<int>(blocks);
    const hipError_t e =
        routed ? dispatch_moe_fmt<true>(zero_points != 0, bf, mb, ns, deep, p, nb, s)
               : dispatch_moe_fmt<false>(zero_points != 0, bf, mb, ns, deep, p, nb, s);
    return e == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

}  // namespace

extern "C" int w4a16_moe_align(const int32_t *topk_ids, int T, int topk, int E,
                               int32_t *sorted_ids, int32_t *expert_offsets, void *stream)
{
    if (!topk_ids || !sorted_ids || !expert_offsets || T < 0 || topk < 1 || E < 1)
        return W4A16_EINVAL;
    if (E > kMaxExperts || static_cast<long long>(T) * topk > INT_MAX)
        return W4A16_ESHAPE;
    w4a16_detail::DeviceInfo d;
    const int rc = w4a16_detail::current_device(&d);
    if (rc != W4A16_OK)
        return rc;
    hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(kAlignThreads), 0,
                       static_cast<hipStream_t>(stream), topk_ids, T * topk, E, sorted_ids,
                       expert_offsets);
    return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

extern "C" int w4a16_moe_gemm(const void *A, const uint32_t *packed, const uint16_t *params,
                              const int32_t *sorted_ids, const int32_t *expert_offsets,
                              const float *row_scale, void *C, int T, int topk, int E, int K,
                              int N, int zero_points, int act_dtype, void *stream)
{
    if (!sorted_ids || !expert_offsets)
        return W4A16_EINVAL;
    MoeParams p{};
    p.A = static_cast<const uint16_t *>(A);
    p.packed = reinterpret_cast<const u4 *>(packed);
    p.params = params;
    p.sorted = sorted_ids;
    p.offsets = expert_offsets;
    p.row_scale = row_scale;
    p.C = static_cast<uint16_t *>(C);
    p.T = T;
    p.topk = topk;
    p.E = E;
    p.K = K;
    p.N = N;
    return moe_run(p, zero_points, act_dtype, false, stream);
}

extern "C" int w4a16_moe_gemm_topk(const void *A, const uint32_t *packed, const uint16_t *params,
                                   const int32_t *topk_ids, const float *row_scale, void *C,
                                   int T, int topk, int E, int K, int N, int zero_points,
                                   int act_dtype, void *stream)
{
    if (!topk_ids)
        return W4A16_EINVAL;
    MoeParams p{};
    p.A = static_cast<const uint16_t *>(A);
    p.packed = reinterpret_cast<const u4 *>(packed);
    p.params = params;
    p.topk_ids = topk_ids;
    p.row_scale = row_scale;
    p.C = static_cast<uint16_t *>(C);
    p.T = T;
    p.topk = topk;
    p.E = E;
    p.K = K;
    p.N = N;
    return moe_run(p, zero_points, act_dtype, true, stream);
}
