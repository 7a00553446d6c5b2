"""Test-side encoders of documented layouts (no library or oracle code).

* layout_reference / params_layout_reference: the packed weight and parameter layouts exactly
  as include/w4a16.h states them, written with numpy indexing.
* encode_along_k / encode_along_n: checkpoint-style words built one nibble at a time, the
  inputs of the load-time repack.
"""
import numpy as np

NIBBLE = [0, 4, 1, 5, 2, 6, 3, 7]    # nibble of a packed word that holds code i


def slabs_per_group(N):
    return 4 if N % 256 == 0 else (2 if N % 128 == 0 else 1)


def layout_reference(codes, scales):
    """(packed words, permuted scale bits) as w4a16_pack documents them; scales [Gs, N] with
    Gs = K/128 or 1."""
    K, N = codes.shape
    G = K // 128
    packed = np.zeros((N // 16, G, 64, 4), dtype=np.uint32)
    l = np.arange(64)
    for t in range(4):
        for i in range(8):
            k = (np.arange(G)[:, None] * 128 + 32 * t + 8 * (l[None, :] // 16) + i)   # [G, 64]
            for j in range(N // 16):
                n = 16 * j + (l % 16)
                packed[j, :, :, t] |= codes[k, n[None, :]].astype(np.uint32) << np.uint32(4 * NIBBLE[i])
    Q = slabs_per_group(N)
    Gs = scales.shape[0]
    # [g][slab group u][slab b in group][c] -> [u][g][c][b]
    sp = np.asarray(scales).reshape(Gs, N // (16 * Q), Q, 16).transpose(1, 0, 3, 2).reshape(-1)
    return packed.reshape(-1), sp


def params_layout_reference(scales, zeros):
    """w4a16_pack_zp's params as the header states it: per column and group its scale, then
    its zero term 0x6400 | z, grouped by Q slabs (fp16 bits)."""
    Gs, N = scales.shape
    Q = slabs_per_group(N)
    s = scales.view(np.uint16).reshape(Gs, N // (16 * Q), Q, 16).transpose(1, 0, 3, 2)  # [u][g][c][b]
    z = (0x6400 | zeros.astype(np.uint16)).reshape(Gs, N // (16 * Q), Q, 16).transpose(1, 0, 3, 2)
    return np.concatenate([s, z], axis=3).reshape(-1)


def encode_along_k(codes):
    """Words [K/8, N]: word (r, n) gets code (8r + i, n) in bits 4i..4i+3."""
    K, N = codes.shape
    c = np.asarray(codes, dtype=np.uint32).reshape(K // 8, 8, N)
    w = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        w |= c[:, i, :] << np.uint32(4 * i)
    return w


def encode_along_n(codes, order=None):
    """Words [rows, N/8]: word (k, c) gets code (k, 8c + order[i]) in bits 4i..4i+3."""
    order = list(range(8)) if order is None else list(order)
    rows, N = codes.shape
    c = np.asarray(codes).reshape(rows, N // 8, 8)
    w = np.zeros((rows, N // 8), dtype=np.uint32)
    for i in range(8):
        w |= c[:, :, order[i]].astype(np.uint32) << np.uint32(4 * i)
    return w


def layout_reference_24(codes):
    """w4a16_pack_24's words as the header states them: per 128 x 16 block, lane l's three
    words -- kept codes of the two 64-row halves, then their positions."""
    K, N = codes.shape
    G = K // 128
    out = np.zeros((N // 16, G, 64, 3), dtype=np.uint32)
    for j in range(N // 16):
        for g in range(G):
            for l in range(64):
                n = 16 * j + l % 16
                for s in range(2):
                    w = 0
                    for p in range(4):
                        k4 = 128 * g + 64 * s + 16 * (l // 16) + 4 * p
                        grp = [int(codes[k4 + i, n]) for i in range(4)]
                        keep = [i for i in range(4) if grp[i] != 8]
                        keep += [i for i in range(4) if i not in keep][:2 - len(keep)]
                        keep.sort()
                        for i, pos in enumerate(keep):
                            e = 2 * p + i
                            w |= grp[pos] << (4 * NIBBLE[e])
                            out[j, g, l, 2] |= np.uint32(pos << (16 * s + 2 * e))
                    out[j, g, l, s] = w
    return out.reshape(-1)
