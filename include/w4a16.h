/*
 * w4a16.h -- C ABI of libw4a16: the FP16 x INT4 (group-128) linear layer on one MI355X (gfx950).
 *
 *   C[M x N] = A[M x K] * Bhat[K x N],   Bhat[k][n] = s[k / 128][n] * (q[k][n] - 8)
 *
 * A and C are fp16, q are 4-bit codes 0..15, s are fp16 scales, one per 128 consecutive rows
 * of each column; products are accumulated in fp32 and C is rounded to fp16 once
 * (round-to-nearest-even).
 *   Problem statement: MARLIN paper (arXiv 2408.11743) sec. 3.4 "Kernel Design" (A fp16,
 *   B symmetrically quantised to INT4 with one FP16 scale per G consecutive weights of a
 *   column); Marlin deep-dive page "Marlin 完全拆解", section "Marlin 要解决的精确问题"
 *   (dequantisation s_{g,n}(q_{k,n} - z) with the symmetric zero point folded to 8).
 *   Interface shape: Marlin README page, usage section (an offline pack step that reorders
 *   weights and scales, then a multiply call on pre-packed data).
 *
 * Two further formats (w4a16_pack / w4a16_pack_zp with w4a16_gemm_ex): one scale per column
 * (group = K: deep-dive page, section "scale 为什么有时在内环乘，有时在末尾乘", AB = (AQ) diag(s),
 * the scale applied once per output), and a zero point per group and column,
 * Bhat[k][n] = s[g][n] * (q[k][n] - z[g][n]) with z a code 0..15 (the page's general affine
 * form s_{g,n}(q_{k,n} - z_{g,n}), section "Marlin 要解决的精确问题").
 *
 * Conventions for every entry point:
 *   - fp16 values travel as their IEEE binary16 bit patterns (uint16_t on the host side).
 *   - Matrices are dense row-major with no padding: A is M x K, C is M x N, codes K x N,
 *     scales and zero points (K/group) x N.
 *   - Sizes are int; a negative size is W4A16_EINVAL.  All arguments are checked before
 *     anything runs; on an error nothing is written.
 *   - The library never takes ownership of a pointer and never allocates device memory.
 *   - Errors are return codes; nothing is thrown or aborted across this boundary.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_GROUP 128           /* rows per scale group; group = K (one per column) also works */
#define W4A16_N_ALIGN 64          /* N must be a multiple of this */

/* Activation types of w4a16_moe_gemm (A, C and the scales share it). */
#define W4A16_ACT_F16 0           /* IEEE binary16 */
#define W4A16_ACT_BF16 1          /* bfloat16: the upper 16 bits of an IEEE binary32 */

/* Source arrangements for w4a16_repack (8 codes per 32-bit word). */
#define W4A16_PACKED_ALONG_K 0    /* word (r, n) of [K/8][N]: rows 8r..8r+7 of column n */
#define W4A16_PACKED_ALONG_N 1    /* word (k, c) of [K][N/8]: columns 8c..8c+7 of row k */

typedef enum {
    W4A16_OK = 0,
    W4A16_EINVAL = -1,            /* null pointer, negative size, a code or zero point
                                     above 15, zero_points not 0 or 1 */
    W4A16_ESHAPE = -2,            /* group not 128 or K, K not a positive multiple of 128,
                                     N not a multiple of 16 (pack) or 64 (gemm), or a
                                     size limit of w4a16_gemm exceeded */
    W4A16_EUNSUPPORTED = -3,      /* the current HIP device is not a gfx950 GPU */
    W4A16_EHIP = -4               /* a HIP runtime call or the kernel launch failed */
} w4a16_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *w4a16_status_string(int status);

/*
 * Offline reorder of codes and scales into the layout w4a16_gemm streams.
 * Host memory, synchronous, no GPU needed.  Follows the pages' one-time load step that
 * permutes weights and scales so the kernel's loads land directly in its operand registers
 * (deep-dive page, sections "直接生成 MMA 所需的寄存器 fragment" and "全局内存布局";
 * MARLIN paper sec. 3.4 "Maximizing Loading Bandwidth": weights are static, so tiles are
 * reshuffled offline to be contiguous).
 *
 *   codes      [in]  uint8 [K*N], row-major (k, n), one code 0..15 per byte
 *   scales     [in]  fp16 bits [(K/group)*N], row-major (g, n)
 *   group      [in]  128, or K for one scale per column
 *   packed_out [out] uint32 [K*N/8]
 *   scales_out [out] fp16 bits [(K/group)*N]
 *
 * Packed layout (the part of this ABI a caller may rely on; 4.125 bits per weight):
 *   The weight matrix is cut into blocks of 128 rows (one scale group) x 16 columns.  Block
 *   (j, g) -- columns 16j..16j+15, rows 128g..128g+127 -- is 256 consecutive uint32 words
 *   starting at word (j*(K/128) + g)*256, so the blocks of one 16-column slab follow each
 *   other down K.  Word 4*l + t of a block (l = 0..63, t = 0..3) holds the 8 codes of
 *   column 16j + (l mod 16), rows 128g + 32t + 8*(l div 16) + i for i = 0..7, code i in
 *   nibble p(i) (bits 4p..4p+3) with p = {0, 4, 1, 5, 2, 6, 3, 7}.
 *   Scales are grouped by Q consecutive slabs, Q = 4 if N is a multiple of 256, else 2 if N
 *   is a multiple of 128, else 1 (the slabs one wave of w4a16_gemm works on); with
 *   Gs = K/group scale groups per column:
 *   scales_out[(((j div Q)*Gs + g)*16 + c)*Q + (j mod Q)] = scales[g][16j + c],
 *   c = 0..15, so the Q scales of one column at one group are adjacent.
 *
 * Returns W4A16_OK, W4A16_EINVAL (null pointer, negative size, a code > 15) or
 * W4A16_ESHAPE (group not 128 or K, K not a positive multiple of 128, N not a positive
 * multiple of 16).
 */
int w4a16_pack(const uint8_t *codes, const uint16_t *scales, int K, int N, int group,
               uint32_t *packed_out, uint16_t *scales_out);

/*
 * Exact inverse of w4a16_pack (host, synchronous).  For tests and tooling; not on the
 * multiply path: the layout check the deep-dive page lists among its validation levels
 * (section "适用边界与工程陷阱", level "布局": unpacking what was packed or repacked must give
 * back the same codes, scales and zero points).  Same arguments and errors as w4a16_pack with
 * inputs and outputs swapped.
 */
int w4a16_unpack(const uint32_t *packed, const uint16_t *scales_packed, int K, int N, int group,
                 uint8_t *codes_out, uint16_t *scales_out);

/*
 * w4a16_pack with a zero point per group and column (host, synchronous): the deep-dive
 * page's general dequantisation s_{g,n}(q_{k,n} - z_{g,n}) (section "Marlin 要解决的精确问题").
 *
 *   zeros      [in]  uint8 [(K/group)*N], row-major (g, n), one code 0..15 per byte
 *   params_out [out] fp16 bits [2*(K/group)*N]: per column and group its scale and its zero
 *                    term, the fp16 value 1024 + z (bits 0x6400 | z) that the kernel's decode
 *                    subtracts.  Layout: the Q scales of a column at one group, then its Q
 *                    zero terms: params_out[i] = scales[g][16j + c] and
 *                    params_out[i + Q] = 0x6400 | zeros[g][16j + c] with
 *                    i = (((j div Q)*Gs + g)*16 + c)*2Q + (j mod Q).
 * Other arguments, the code layout and the errors as w4a16_pack (a zero point above 15 is
 * W4A16_EINVAL).
 */
int w4a16_pack_zp(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, int K,
                  int N, int group, uint32_t *packed_out, uint16_t *params_out);

/*
 * Exact inverse of w4a16_pack_zp (host, synchronous; tests and tooling).  W4A16_EINVAL also
 * if a zero term is not of the form 0x6400 | z.
 */
int w4a16_unpack_zp(const uint32_t *packed, const uint16_t *params, int K, int N, int group,
                    uint8_t *codes_out, uint16_t *scales_out, uint8_t *zeros_out);

/*
 * Bytes of device workspace w4a16_gemm, w4a16_gemm_ex and w4a16_gemm_24 need for this shape
 * on the current device (a fixed 4 KiB counter area plus room for fp32 partial output
 * tiles), written to *bytes.
 * A workspace sized for one shape may be reused for any shape whose requirement is not
 * larger.  Returns W4A16_OK, W4A16_EINVAL (bytes == NULL, negative size), W4A16_ESHAPE
 * (as w4a16_gemm), W4A16_EUNSUPPORTED (current device is not gfx950) or W4A16_EHIP.
 */
int w4a16_workspace_size(int M, int K, int N, size_t *bytes);

/*
 * A bound on w4a16_workspace_size(M, K, N) that needs no device: never smaller than what any
 * device of at most 512 compute units asks for (MI355X has 256), for any of the multiply
 * entry points that take a workspace.  For sizing a workspace before a GPU is chosen or
 * where the exact call cannot be made (the pages allocate and zero the workspace once, when
 * the layer is loaded: deep-dive page, "可复现的调用链与实现伪代码").  Sizes as w4a16_gemm;
 * returns 0 for a negative size or K not a positive multiple of 128.
 *
 * Terms: the 4 KiB counter area, plus the larger of
 *   - the stripe kernels' fp32 partial tiles: two Mt x Nt tiles per stripe, at most 1024
 *     stripes and at most one stripe per 128 x Nt x Mt tile, Mt = 16, 32, 64 or 128 rows as M
 *     is at most 16, 32, 64 or larger, Nt = 256 columns (N if smaller);
 *   - the whole-K kernels' split-K pieces: 1 KiB per 16 x 16 output block per K split, at
 *     most 64 pieces per 16-column slab (M <= 128 only), and at most 40 MiB.
 */
static inline size_t w4a16_workspace_bound(int M, int K, int N)
{
    if (M < 0 || K <= 0 || N < 0 || K % 128)
        return 0;
    const size_t mt = M <= 16 ? 16 : (M <= 32 ? 32 : (M <= 64 ? 64 : 128));
    const size_t nt = N < 256 ? (size_t)N : 256;
    const size_t mcov = M <= 64 ? mt : 128 * (((size_t)M + 127) / 128);
    size_t stripes = 2 * 1024 * mt * nt * 4;
    const size_t by_tiles = 8 * (size_t)N * ((size_t)K / 128) * mcov;
    if (by_tiles < stripes)
        stripes = by_tiles;
    size_t pieces = 0;
    if (M <= 128) {
        pieces = ((size_t)N / 16 + 9) * 64 * 1024;
        if (pieces > ((size_t)40 << 20))
            pieces = (size_t)40 << 20;
    }
    return 4096 + (stripes > pieces ? stripes : pieces);
}

/*
 * C = A * Bhat on the current HIP device, enqueued on `stream` (a hipStream_t passed as
 * void*; NULL means the null stream).  Asynchronous: returns once the work is enqueued.
 *
 *   A          [in]  device, fp16 [M*K] row-major
 *   packed     [in]  device, uint32 [K*N/8] from w4a16_pack
 *   scales     [in]  device, fp16 bits [(K/128)*N] from w4a16_pack (scales_out)
 *   C          [out] device, fp16 [M*N] row-major, every element overwritten
 *   workspace  [in/out] device, at least w4a16_workspace_size(M, K, N) bytes.  Its first
 *                  4 KiB must be zero before the first call (zero it once after allocation);
 *                  every call leaves them zero again.  One workspace must not be used by
 *                  two calls that can run at the same time.
 *
 * The weight matrix is split into column slices and each slice's K range into 128-row
 * tiles; workgroups take equal runs of consecutive tiles ("stripes", deep-dive page
 * section "Split-K 与全局归约"; MARLIN README page, striped partitioning).  For M <= 16,
 * and up to M = 128 on narrower weights, workgroups instead own a few 16-column slabs over
 * all of K or over one of a few equal K splits.  Output shared by several workgroups is
 * summed in fp32 in a fixed order, so results are identical from run to run.
 *
 * Alignment: A, packed and scales must be 16-byte aligned (any hipMalloc pointer is).
 * Limits: (M + 128) * K * 2, (M + 128) * N * 2 and K * N / 2 must each be below 2^32 bytes
 * (the kernels address A, C and the packed weights through 32-bit buffer offsets).
 *
 * M == 0 is a no-op returning W4A16_OK.  Errors: W4A16_EINVAL (null pointer, negative
 * size), W4A16_ESHAPE (K not a positive multiple of 128, N not a positive multiple of 64,
 * a limit above exceeded), W4A16_EUNSUPPORTED (current device is not gfx950),
 * W4A16_EHIP (launch failure).
 */
int w4a16_gemm(const void *A, const uint32_t *packed, const uint16_t *scales, void *C,
               int M, int K, int N, void *workspace, void *stream);

/*
 * w4a16_gemm for every packed format (device, asynchronous on `stream`):
 *   group        128, or K for one scale per column: the fp32 sum over all of K is
 *                scaled once per output before C is written (deep-dive page, section
 *                "scale 为什么有时在内环乘，有时在末尾乘": AB = (AQ) diag(s)).
 *   zero_points  0: `params` are the scales from w4a16_pack, z = 8;
 *                1: `params` are from w4a16_pack_zp (scale and zero term per column and
 *                   group), Bhat = s (q - z).
 * w4a16_gemm(...) is w4a16_gemm_ex(..., 128, 0, ...).  The workspace size does not depend on
 * the format.  Other arguments, limits and errors as w4a16_gemm; a group other than 128 or K
 * is W4A16_ESHAPE, zero_points other than 0 or 1 W4A16_EINVAL.
 */
int w4a16_gemm_ex(const void *A, const uint32_t *packed, const uint16_t *params, void *C,
                  int M, int K, int N, int group, int zero_points, void *workspace,
                  void *stream);

/*
 * w4a16_gemm_ex with no workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * library keeps one scratch area per GPU in a device array of W4A16_NOALLOC_SCRATCH_BYTES
 * (128 MiB + 4 KiB, reserved on each GPU the library runs on until the process ends); it
 * covers every shape w4a16_gemm_ex accepts on MI355X.  Nothing is allocated: no hipMalloc,
 * hipFree or allocating library call.  The first call on a GPU clears the scratch's counter
 * area with a small kernel on `stream`; every call leaves it clear.
 * All calls on one GPU share that GPU's scratch: calls that can overlap in time (two streams,
 * two threads) race and give wrong results -- serialise them, or use w4a16_gemm_ex with a
 * workspace each.  Other arguments, results (bit for bit the same as w4a16_gemm_ex's for the
 * same inputs) and errors as w4a16_gemm_ex; a shape whose workspace would exceed the scratch
 * (w4a16_workspace_size above W4A16_NOALLOC_SCRATCH_BYTES) is W4A16_ESHAPE.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (((size_t)128 << 20) + 4096)
int w4a16_gemm_noalloc(const void *A, const uint32_t *packed, const uint16_t *params, void *C,
                       int M, int K, int N, int group, int zero_points, void *stream);

/*
 * 2:4-sparse weights (Sparse-MARLIN: MARLIN paper sec. 1 "Contribution" and sec. 2.1.1, the
 * 2:4 format of two non-zeros in every 4 consecutive weights with their positions as
 * metadata; deep-dive page, Sparse-MARLIN section: 4-bit non-zeros plus 2-bit positions, the
 * product computed as (B^T A^T)^T).  Group-128 scales, zero point 8: a weight is zero when its
 * code is 8, and every aligned group of 4 rows of a column may hold at most 2 other codes.
 *
 * w4a16_pack_24 (host, synchronous): codes uint8 [K*N] (row-major (k, n), 0..15, 2:4 along K
 * as above), scales fp16 bits [(K/128)*N] -> packed_out uint32 [K*N*3/32], scales_out fp16
 * bits [(K/128)*N] (the layout of w4a16_pack's scales_out).
 * Packed layout: blocks of 128 rows x 16 columns, block (j, g) -- columns 16j..16j+15, rows
 * 128g..128g+127 -- is 192 consecutive words starting at word (j*(K/128) + g)*192.  Lane
 * l = 0..63 owns words 3l, 3l+1, 3l+2: column 16j + (l mod 16); word 3l + s (s = 0, 1) holds
 * the two kept codes of each group of four rows 128g + 64s + 16*(l div 16) + 4p + 0..3,
 * p = 0..3, in row order -- kept code e = 2p + i (i = 0, 1) in nibble q(e), q = {0, 4, 1, 5,
 * 2, 6, 3, 7} -- and word 3l + 2 holds their positions in the group (0..3), code e of word
 * 3l + s in bits 16s + 2e .. 16s + 2e + 1.  Kept positions are the non-zero weights, completed
 * by the lowest other positions (which then hold code 8).  3.125 bits per weight with scales.
 * Returns W4A16_OK, W4A16_EINVAL (null pointer, negative size, a code above 15, a group with
 * more than 2 codes other than 8) or W4A16_ESHAPE (as w4a16_pack with group 128).
 */
int w4a16_pack_24(const uint8_t *codes, const uint16_t *scales, int K, int N,
                  uint32_t *packed_out, uint16_t *scales_out);

/*
 * Exact inverse of w4a16_pack_24 (host, synchronous; tests and tooling): codes at pruned
 * positions come back as 8.  W4A16_EINVAL also if a group's two positions are not increasing.
 */
int w4a16_unpack_24(const uint32_t *packed, const uint16_t *scales_packed, int K, int N,
                    uint8_t *codes_out, uint16_t *scales_out);

/*
 * C = A * Bhat with 2:4-sparse Bhat from w4a16_pack_24 (device, asynchronous on `stream`),
 * on the structured-sparse matrix instruction, computed transposed as C^T = Bhat^T A^T
 * (Sparse-MARLIN section of the deep-dive page).  A, C, workspace (at least
 * w4a16_workspace_size(M, K, N) bytes, first 4 KiB zero, one call at a time), alignment and
 * the size limits as w4a16_gemm; packed and scales as w4a16_pack_24 wrote them (device
 * copies).  N must be a multiple of 256, and K*N*3/8 and 128*K below 2^31 bytes.  Sums are
 * formed in a fixed order: results repeat bit for bit.  M == 0 is a no-op.  Errors:
 * W4A16_EINVAL (null pointer, negative size), W4A16_ESHAPE (shape or limit),
 * W4A16_EUNSUPPORTED (not gfx950), W4A16_EHIP (launch failure).
 */
int w4a16_gemm_24(const void *A, const uint32_t *packed, const uint16_t *scales, void *C,
                  int M, int K, int N, void *workspace, void *stream);

/*
 * Device-side load-time conversion of checkpoint-style packed tensors into the layouts of
 * w4a16_pack (qzeros NULL) or w4a16_pack_zp (device, asynchronous on `stream`).  The pages'
 * load step that turns a GPTQ/AWQ-style checkpoint into the kernel's layout: it only moves
 * codes, it never changes one (deep-dive page, section "直接生成 MMA 所需的寄存器 fragment", and
 * the deployment section on checkpoint formats, which differ in nibble order, scale
 * arrangement and zero-point convention).
 *
 *   qweight    [in]  device uint32, the codes, 8 per word:
 *                    W4A16_PACKED_ALONG_K: [K/8][N], word (r, n) holds rows 8r..8r+7 of
 *                      column n, row 8r + i in bits 4i..4i+3;
 *                    W4A16_PACKED_ALONG_N: [K][N/8], word (k, c) holds columns 8c..8c+7 of
 *                      row k, column 8c + order[i] in bits 4i..4i+3.
 *   src_layout [in]  W4A16_PACKED_ALONG_K or W4A16_PACKED_ALONG_N
 *   order      [in]  host uint8[8], a permutation of 0..7, or NULL for 0, 1, ..., 7: the
 *                    column offset that nibble i holds in every word packed along N
 *                    (qweight with W4A16_PACKED_ALONG_N, and qzeros)
 *   scales     [in]  device fp16 bits [(K/group)][N], row-major (g, n)
 *   qzeros     [in]  device uint32 [(K/group)][N/8] packed along N (word (g, c): zero points
 *                    z of columns 8c..8c+7 at group g, each a code 0..15 taken as stored),
 *                    or NULL for the symmetric format (z = 8)
 *   group      [in]  128, or K for one scale per column
 *   packed_out [out] device uint32 [K*N/8]: exactly w4a16_pack's packed_out for these codes
 *   params_out [out] device fp16 bits: qzeros NULL: [(K/group)*N], w4a16_pack's scales_out;
 *                    else [2*(K/group)*N], w4a16_pack_zp's params_out
 * Then call w4a16_gemm_ex with the same group and zero_points = (qzeros != NULL).
 *
 * Outputs must not overlap the inputs.  Alignment: packed_out 16 bytes, qweight and qzeros
 * 4, scales and params_out 2 (any hipMalloc pointer is aligned).
 * Errors: W4A16_EINVAL (null pointer other than order / qzeros, negative size, unknown
 * src_layout, order not a permutation of 0..7, misaligned pointer), W4A16_ESHAPE (as
 * w4a16_pack: group not 128 or K, K not a positive multiple of 128, N not a positive multiple
 * of 16; or a grid too large to launch), W4A16_EUNSUPPORTED (current device is not gfx950),
 * W4A16_EHIP (launch failure).  Arguments are checked before any device call.
 */
int w4a16_repack(const uint32_t *qweight, int src_layout, const uint8_t *order,
                 const uint16_t *scales, const uint32_t *qzeros, int K, int N, int group,
                 uint32_t *packed_out, uint16_t *params_out, void *stream);

/*
 * Regrouping of a mixture-of-experts layer's token assignments by expert (device,
 * asynchronous on `stream`).  The pages' observation that an MoE layer regroups tokens by
 * expert, so that each expert's product sees its own M (deep-dive page, section on where the
 * format pays off, item 1; item 4 on grouped GEMM).
 *
 *   topk_ids       [in]  device int32 [T*topk]: entry a = t*topk + j is the j-th expert of
 *                        token t.  Entries outside 0..E-1 are left out (their rows of C are
 *                        then not written by w4a16_moe_gemm).
 *   sorted_ids     [out] device int32 [T*topk]: the assignments a with a valid expert,
 *                        grouped by expert (expert 0 first), increasing a within an expert;
 *                        entries past expert_offsets[E] are not written.
 *   expert_offsets [out] device int32 [E+1]: expert e's assignments are
 *                        sorted_ids[expert_offsets[e] .. expert_offsets[e+1]).
 * Deterministic (a stable counting sort in one workgroup).  E at most 1024.  Errors:
 * W4A16_EINVAL (null pointer, T < 0, topk < 1, E < 1), W4A16_ESHAPE (E > 1024 or
 * T*topk >= 2^31), W4A16_EUNSUPPORTED, W4A16_EHIP.
 */
int w4a16_moe_align(const int32_t *topk_ids, int T, int topk, int E, int32_t *sorted_ids,
                    int32_t *expert_offsets, void *stream);

/*
 * Grouped W4A16 product of an MoE layer (device, asynchronous on `stream`), one launch for
 * all experts:
 *   C[a][n] = row_scale[a] * sum_k A[a / topk][k] * Bhat_e[k][n],  e = expert of assignment a,
 * for every assignment a listed in sorted_ids, with Bhat_e = s_e (q_e - z_e) as in
 * w4a16_gemm_ex (group 128; z = 8, or per group and column with zero_points = 1).  Each
 * token row is read where it lies in A and each result written to its own row of C: no
 * permuted copy is made.  Experts without rows cost nothing but early exits; with no more
 * assignments than experts (T*topk <= E) the launch holds only min(E, T*topk) rows of
 * workgroups and the experts in use take the lowest workgroup ids.
 *
 *   A              [in]  device [T*K] row-major, fp16 or bf16 (act_dtype)
 *   packed         [in]  device uint32 [E][K*N/8]: expert e's w4a16_pack / w4a16_pack_zp
 *                        output (group 128) at word e*K*N/8
 *   params         [in]  device 16-bit [E][(K/128)*N] (scales_out of w4a16_pack), or
 *                        [E][2*(K/128)*N] with zero_points = 1 (params_out of w4a16_pack_zp);
 *                        the scales are of type act_dtype (w4a16_pack moves their bits only)
 *   sorted_ids, expert_offsets  [in] device, as w4a16_moe_align writes them
 *   row_scale      [in]  device float [T*topk] indexed by assignment, or NULL for 1 (the
 *                        router weight of a down projection)
 *   C              [out] device [T*topk][N] of act_dtype; rows not listed are not written
 *   zero_points    0 or 1;  act_dtype  W4A16_ACT_F16 or W4A16_ACT_BF16
 * fp32 sums, one rounding of C to nearest-even.  fp16: the dense path's exact decode, so a
 * row equals w4a16_gemm's result for that token and expert bit for bit when w4a16_gemm
 * takes its whole-K kernel without a K split (M <= 16).  bf16: codes enter the matrix unit as 128 + q and
 * (128 + z) * sum_k A is subtracted per row and group before the scale.
 * Results do not depend on how the rows are grouped.  Limits: K a multiple of 128, N a
 * multiple of 256, E at most 1024, and K*N/2, T*K*2, T*topk*N*2 and (K/128)*N*4 below 2^31
 * bytes.  T == 0
 * is a no-op.  Errors: W4A16_EINVAL (null pointer other than row_scale, negative size,
 * topk or E below 1, zero_points or act_dtype out of range), W4A16_ESHAPE (shape or
 * limit), W4A16_EUNSUPPORTED (not gfx950), W4A16_EHIP (launch failure).
 */
int w4a16_moe_gemm(const void *A, const uint32_t *packed, const uint16_t *params,
                   const int32_t *sorted_ids, const int32_t *expert_offsets,
                   const float *row_scale, void *C, int T, int topk, int E, int K, int N,
                   int zero_points, int act_dtype, void *stream);

/*
 * w4a16_moe_gemm with the regrouping done inside the product (device, asynchronous on
 * `stream`): for decode-sized batches, where a separate w4a16_moe_align launch would cost as
 * much as the product of a few experts.  Every workgroup lists its expert's assignments from
 * topk_ids itself (same order as w4a16_moe_align, so the results equal w4a16_moe_gemm's bit
 * for bit).  topk_ids as for w4a16_moe_align ([T*topk] int32, entries outside 0..E-1 left
 * out, their rows of C not written); everything else as w4a16_moe_gemm.  T*topk at most
 * 2048, else W4A16_ESHAPE (use w4a16_moe_align + w4a16_moe_gemm).
 */
int w4a16_moe_gemm_topk(const void *A, const uint32_t *packed, const uint16_t *params,
                        const int32_t *topk_ids, const float *row_scale, void *C, int T,
                        int topk, int E, int K, int N, int zero_points, int act_dtype,
                        void *stream);

/*
 * Measurement support, not part of the multiply: streams `bytes` from device buffer `src`
 * (each workgroup one contiguous chunk, 128-bit non-temporal loads, the fastest read pattern
 * measured) and discards the data, for a measured HBM read rate to compare the multiply against
 * (MARLIN paper sec. 3.4: the layer is bound by weight loading).  `out`: device uint32[2048],
 * written only in the rare case a checksum equals a fixed value (the writes keep the loads
 * alive).  Device, asynchronous on `stream`.  Errors: W4A16_EINVAL (null pointer, bytes 0
 * or not a multiple of 16, src not 16-byte aligned), W4A16_EUNSUPPORTED, W4A16_EHIP.
 */
int w4a16_read_probe(const void *src, size_t bytes, uint32_t *out, void *stream);

/*
 * Measurement support, not part of the multiply: the matrix cores' sustained fp16 rate on
 * operands that change from one instruction to the next, for a measured peak to set the
 * compute-bound sweep against beside the nominal 2.5 PFLOP/s (deep-dive page, "适用边界与工程陷阱",
 * validation level "Kernel": record the matrix units' utilisation beside HBM bandwidth).
 * `workgroups` workgroups of 4 waves each run `iters` rounds of 64 fp16 matrix instructions
 * (8 independent fp32 accumulators), each wave on 16 operand fragments of its own taken from
 * `src` (random fp16 values give the power draw of real data; constant ones run faster).
 *   shape      0: v_mfma_f32_16x16x32_f16 (16384 flops each), 1: v_mfma_f32_32x32x16_f16
 *              (32768 flops each)
 *   src        device, src_bytes bytes (a multiple of 16, at least 16), 16-byte aligned
 *   out        device float [workgroups * 256]: one sum of accumulators per lane (keeps the
 *              work alive)
 * Flops = workgroups * 4 * iters * 64 * (16384 or 32768).  Device, asynchronous on `stream`.
 * Errors: W4A16_EINVAL (null pointer, src_bytes not a positive multiple of 16, misaligned
 * src, workgroups or iters not positive, shape not 0 or 1), W4A16_EUNSUPPORTED, W4A16_EHIP.
 */
int w4a16_mfma_probe(const void *src, size_t src_bytes, int shape, int workgroups, int iters,
                     float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
