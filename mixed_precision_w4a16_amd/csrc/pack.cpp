// Offline weight/scale reorder for the gfx950 W4A16 kernel (host code, no GPU needed).
//
// The pages reorder the quantised weights once at load time so that every thread's wide
// load delivers exactly the codes its matrix-core operand needs, with the nibbles of a word
// in an order that a short mask-and-OR sequence turns into fp16 pairs (Marlin deep-dive page
// "Marlin 完全拆解", sections "直接生成 MMA 所需的寄存器 fragment" and "全局内存布局";
// MARLIN paper sec. 3.4 "Maximizing Loading Bandwidth").  The layout here is built for the
// CDNA4 16x16x32 fp16 MFMA on 64-lane waves instead of Ampere's mma.sync fragments:
//
//   block (j, g) = rows 128g..128g+127 (one scale group) x columns 16j..16j+15, 1 KiB;
//   lane l of a wave loads the block's 16-byte word quad l (one 128-bit load per lane,
//   1 KiB contiguous per wave); word t of that quad feeds MFMA k-step t and holds column
//   16j + l%16, rows 128g + 32t + 8(l/16) + i (i = 0..7), code i in nibble kNibble[i].
//   Nibble pairs (0,4), (1,5), (2,6), (3,7) then become the fp16 pairs (k0,k1), (k2,k3),
//   (k4,k5), (k6,k7) of the MFMA B operand.
//
// Blocks of a 16-column slab are consecutive down K, so a workgroup walking down K streams
// contiguous memory.  Scales are grouped for the same walk: a wave works on Q consecutive
// slabs (Q = 4, 2 or 1: the widest that divides N / 64, as the kernel chooses), and the Q
// scales of one column of those slabs at one group are adjacent, so one 2Q-byte load per
// lane brings all the scales a wave needs for a K step.
#include "w4a16.h"

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kNibble[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// Slabs per scale group: the widest of 4, 2, 1 such that N is a multiple of 64 * Q (N a
// multiple of 16 only: 1).
size_t slabs_per_scale_group(size_t N)
{
    return N % 256 == 0 ? 4 : (N % 128 == 0 ? 2 : 1);
}

// Position in scales_out of scale (g, column 16j + c); G = scale groups per column.
size_t scale_index(size_t j, size_t g, size_t c, size_t G, size_t Q)
{
    return (((j / Q) * G + g) * 16 + c) * Q + j % Q;
}

// Position in params_out (w4a16_pack_zp) of scale (g, column 16j + c); its zero term follows
// Q places later: each column's Q scales, then its Q zero terms.
size_t param_index(size_t j, size_t g, size_t c, size_t G, size_t Q)
{
    return (((j / Q) * G + g) * 16 + c) * 2 * Q + j % Q;
}

int check_shape(const void *a, const void *b, const void *c, const void *d, int K, int N,
                int group)
{
    if (!a || !b || !c || !d || K < 0 || N < 0)
        return W4A16_EINVAL;
    if (K == 0 || N == 0 || K % W4A16_GROUP || N % 16 || (group != W4A16_GROUP && group != K))
        return W4A16_ESHAPE;
    return W4A16_OK;
}

// Reorder the codes into the block layout (shared by both pack calls).
void pack_codes(const uint8_t *codes, size_t nk, size_t nn, uint32_t *packed_out)
{
    const size_t G = nk / W4A16_GROUP;
    const size_t slabs = nn / 16;
    for (size_t j = 0; j < slabs; ++j) {
        for (size_t g = 0; g < G; ++g) {
            uint32_t *blk = packed_out + (j * G + g) * 256;
            for (int l = 0; l < 64; ++l) {
                const size_t n = j * 16 + (l & 15);
                for (int t = 0; t < 4; ++t) {
                    const size_t k0 = g * W4A16_GROUP + 32 * t + 8 * (l >> 4);
                    uint32_t w = 0;
                    for (int i = 0; i < 8; ++i)
                        w |= static_cast<uint32_t>(codes[(k0 + i) * nn + n]) << (4 * kNibble[i]);
                    blk[4 * l + t] = w;
                }
            }
        }
    }
}

void unpack_codes(const uint32_t *packed, size_t nk, size_t nn, uint8_t *codes_out)
{
    const size_t G = nk / W4A16_GROUP;
    const size_t slabs = nn / 16;
    for (size_t j = 0; j < slabs; ++j) {
        for (size_t g = 0; g < G; ++g) {
            const uint32_t *blk = packed + (j * G + g) * 256;
            for (int l = 0; l < 64; ++l) {
                const size_t n = j * 16 + (l & 15);
                for (int t = 0; t < 4; ++t) {
                    const size_t k0 = g * W4A16_GROUP + 32 * t + 8 * (l >> 4);
                    const uint32_t w = blk[4 * l + t];
                    for (int i = 0; i < 8; ++i)
                        codes_out[(k0 + i) * nn + n] =
                            static_cast<uint8_t>((w >> (4 * kNibble[i])) & 0xF);
                }
            }
        }
    }
}

bool codes_valid(const uint8_t *v, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (v[i] > 15)
            return false;
    return true;
}

// fp16 bits of 1024 + z (exact: the spacing of fp16 at 1024 is 1).
uint16_t zero_term(uint8_t z)
{
    return static_cast<uint16_t>(0x6400 | z);
}

// 2:4-sparse layout (w4a16_pack_24): per 128 x 16 block, lane l (0..63) owns 3 words at
// 3l: column 16j + l % 16; word 3l + s (s = 0, 1) holds the 8 kept codes of rows
// 128g + 64s + 16(l / 16) + 0..15 (two per group of four rows, in row order: kept code e of
// group e / 2, in nibble kNibble[e]); word 3l + 2 holds their positions in the group, 2 bits
// each, code e of step s at bits 16s + 2e.
constexpr size_t kSparseBlockWords = 192;

// Kept positions of the group of four codes c[0..3]: the nonzero weights (code != 8) in row
// order, completed by the lowest other positions.  False if more than two are nonzero.
bool kept_pair(const uint8_t (&c)[4], int (&pos)[2])
{
    int n = 0;
    for (int i = 0; i < 4; ++i)
        if (c[i] != 8) {
            if (n == 2)
                return false;
            pos[n++] = i;
        }
    for (int i = 0; i < 4 && n < 2; ++i)      // lowest positions not yet taken
        if (n == 0 || pos[0] != i)
            pos[n++] = i;
    if (pos[0] > pos[1]) {
        const int t = pos[0];
        pos[0] = pos[1];
        pos[1] = t;
    }
    return true;
}

bool pack_codes_24(const uint8_t *codes, size_t nk, size_t nn, uint32_t *packed_out)
{
    const size_t G = nk / W4A16_GROUP;
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < G; ++g) {
            uint32_t *blk = packed_out + (j * G + g) * kSparseBlockWords;
            for (int l = 0; l < 64; ++l) {
                const size_t n = j * 16 + (l & 15);
                uint32_t idx = 0;
                for (int s = 0; s < 2; ++s) {
                    uint32_t w = 0;
                    for (int p = 0; p < 4; ++p) {
                        const size_t k4 = g * W4A16_GROUP + 64 * s + 16 * (l >> 4) + 4 * p;
                        uint8_t c[4];
                        for (int i = 0; i < 4; ++i)
                            c[i] = codes[(k4 + i) * nn + n];
                        int pos[2];
                        if (!kept_pair(c, pos))
                            return false;
                        for (int i = 0; i < 2; ++i) {
                            const int e = 2 * p + i;
                            w |= static_cast<uint32_t>(c[pos[i]]) << (4 * kNibble[e]);
                            idx |= static_cast<uint32_t>(pos[i]) << (16 * s + 2 * e);
                        }
                    }
                    blk[3 * l + s] = w;
                }
                blk[3 * l + 2] = idx;
            }
        }
    return true;
}

bool unpack_codes_24(const uint32_t *packed, size_t nk, size_t nn, uint8_t *codes_out)
{
    const size_t G = nk / W4A16_GROUP;
    for (size_t i = 0; i < nk * nn; ++i)
        codes_out[i] = 8;
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < G; ++g) {
            const uint32_t *blk = packed + (j * G + g) * kSparseBlockWords;
            for (int l = 0; l < 64; ++l) {
                const size_t n = j * 16 + (l & 15);
                const uint32_t idx = blk[3 * l + 2];
                for (int s = 0; s < 2; ++s)
                    for (int p = 0; p < 4; ++p) {
                        const size_t k4 = g * W4A16_GROUP + 64 * s + 16 * (l >> 4) + 4 * p;
                        const int e0 = 2 * p;
                        const uint32_t p0 = (idx >> (16 * s + 2 * e0)) & 3;
                        const uint32_t p1 = (idx >> (16 * s + 2 * e0 + 2)) & 3;
                        if (p0 >= p1)
                            return false;      // not written by w4a16_pack_24
                        codes_out[(k4 + p0) * nn + n] = static_cast<uint8_t>(
                            (blk[3 * l + s] >> (4 * kNibble[e0])) & 0xF);
                        codes_out[(k4 + p1) * nn + n] = static_cast<uint8_t>(
                            (blk[3 * l + s] >> (4 * kNibble[e0 + 1])) & 0xF);
                    }
            }
        }
    return true;
}

}  // namespace

extern "C" int w4a16_pack(const uint8_t *codes, const uint16_t *scales, int K, int N, int group,
                          uint32_t *packed_out, uint16_t *scales_out)
{
    int rc = check_shape(codes, scales, packed_out, scales_out, K, N, group);
    if (rc != W4A16_OK)
        return rc;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    if (!codes_valid(codes, nk * nn))
        return W4A16_EINVAL;
    pack_codes(codes, nk, nn, packed_out);
    const size_t Gs = nk / static_cast<size_t>(group);
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < Gs; ++g)
            for (size_t c = 0; c < 16; ++c)
                scales_out[scale_index(j, g, c, Gs, Q)] = scales[g * nn + j * 16 + c];
    return W4A16_OK;
}

extern "C" int w4a16_pack_zp(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                             int K, int N, int group, uint32_t *packed_out, uint16_t *params_out)
{
    int rc = check_shape(codes, scales, packed_out, params_out, K, N, group);
    if (rc != W4A16_OK)
        return rc;
    if (!zeros)
        return W4A16_EINVAL;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    const size_t Gs = nk / static_cast<size_t>(group);
    if (!codes_valid(codes, nk * nn) || !codes_valid(zeros, Gs * nn))
        return W4A16_EINVAL;
    pack_codes(codes, nk, nn, packed_out);
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < Gs; ++g)
            for (size_t c = 0; c < 16; ++c) {
                const size_t i = param_index(j, g, c, Gs, Q);
                params_out[i] = scales[g * nn + j * 16 + c];
                params_out[i + Q] = zero_term(zeros[g * nn + j * 16 + c]);
            }
    return W4A16_OK;
}

extern "C" int w4a16_unpack(const uint32_t *packed, const uint16_t *scales_packed, int K, int N,
                            int group, uint8_t *codes_out, uint16_t *scales_out)
{
    int rc = check_shape(packed, scales_packed, codes_out, scales_out, K, N, group);
    if (rc != W4A16_OK)
        return rc;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    unpack_codes(packed, nk, nn, codes_out);
    const size_t Gs = nk / static_cast<size_t>(group);
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < Gs; ++g)
            for (size_t c = 0; c < 16; ++c)
                scales_out[g * nn + j * 16 + c] = scales_packed[scale_index(j, g, c, Gs, Q)];
    return W4A16_OK;
}

extern "C" int w4a16_unpack_zp(const uint32_t *packed, const uint16_t *params, int K, int N,
                               int group, uint8_t *codes_out, uint16_t *scales_out,
                               uint8_t *zeros_out)
{
    int rc = check_shape(packed, params, codes_out, scales_out, K, N, group);
    if (rc != W4A16_OK)
        return rc;
    if (!zeros_out)
        return W4A16_EINVAL;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    const size_t Gs = nk / static_cast<size_t>(group);
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < Gs; ++g)
            for (size_t c = 0; c < 16; ++c)
                if ((params[param_index(j, g, c, Gs, Q) + Q] & 0xFFF0) != 0x6400)
                    return W4A16_EINVAL;          // not a zero term written by w4a16_pack_zp
    unpack_codes(packed, nk, nn, codes_out);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < Gs; ++g)
            for (size_t c = 0; c < 16; ++c) {
                const size_t i = param_index(j, g, c, Gs, Q);
                scales_out[g * nn + j * 16 + c] = params[i];
                zeros_out[g * nn + j * 16 + c] = static_cast<uint8_t>(params[i + Q] & 0xF);
            }
    return W4A16_OK;
}

extern "C" int w4a16_pack_24(const uint8_t *codes, const uint16_t *scales, int K, int N,
                             uint32_t *packed_out, uint16_t *scales_out)
{
    int rc = check_shape(codes, scales, packed_out, scales_out, K, N, W4A16_GROUP);
    if (rc != W4A16_OK)
        return rc;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    if (!codes_valid(codes, nk * nn) || !pack_codes_24(codes, nk, nn, packed_out))
        return W4A16_EINVAL;
    const size_t G = nk / W4A16_GROUP;
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < G; ++g)
            for (size_t c = 0; c < 16; ++c)
                scales_out[scale_index(j, g, c, G, Q)] = scales[g * nn + j * 16 + c];
    return W4A16_OK;
}

extern "C" int w4a16_unpack_24(const uint32_t *packed, const uint16_t *scales_packed, int K,
                               int N, uint8_t *codes_out, uint16_t *scales_out)
{
    int rc = check_shape(packed, scales_packed, codes_out, scales_out, K, N, W4A16_GROUP);
    if (rc != W4A16_OK)
        return rc;
    const size_t nk = static_cast<size_t>(K), nn = static_cast<size_t>(N);
    if (!unpack_codes_24(packed, nk, nn, codes_out))
        return W4A16_EINVAL;
    const size_t G = nk / W4A16_GROUP;
    const size_t Q = slabs_per_scale_group(nn);
    for (size_t j = 0; j < nn / 16; ++j)
        for (size_t g = 0; g < G; ++g)
            for (size_t c = 0; c < 16; ++c)
                scales_out[g * nn + j * 16 + c] = scales_packed[scale_index(j, g, c, G, Q)];
    return W4A16_OK;
}

extern "C" const char *w4a16_status_string(int status)
{
    switch (status) {
    case W4A16_OK:
        return "ok";
    case W4A16_EINVAL:
        return "invalid argument (null pointer, negative size, code or zero point above 15, or "
               "more than 2 non-zero weights in a group of 4 for the 2:4-sparse format)";
    case W4A16_ESHAPE:
        return "unsupported shape (group must be 128 or K, K a positive multiple of 128, "
               "N a positive multiple of 64)";
    case W4A16_EUNSUPPORTED:
        return "current HIP device is not a gfx950 GPU";
    case W4A16_EHIP:
        return "HIP runtime error";
    default:
        return "unknown status";
    }
}
