"""Independent readers for the two packed weight images.

These follow the byte-level format described below and are written without
reference to the library's packer, so a mistake in either shows up as a
mismatch.  The format itself is the library's own choice: the pages say only
that each 64x128 block is stored with its own bitwidth next to its metadata
(ScaleBITS explainer, section 3.2, block-wise memory layout) and that MixLLM
pre-packs its weights so nothing is permuted at run time (MixLLM page,
section 3.3).

Block image ("GBB1")
--------------------
header (64 B, little endian): u32 magic 0x31424247, u32 version 1, u32 N,
u32 K, u32 N/64, u32 K/128, u64 offset of bits, u64 offset of block offsets,
u64 offset of scale/zero, u64 offset of codes, u64 code bytes.  Sections start
on 256-byte boundaries (bits at 256).

bits   u8 per block, block index = block_row * (K/128) + block_col.
offs   u32 per block + 1: start of each block in the code section in KiB.
sz     per block 64 u32; entry 4 r + t belongs to row 16 t + r of the block
       (r < 16, t < 4): low half fp16 s, high half fp16 z (an integer
       0 .. 2^b - 1).
codes  block i occupies 1024 * b_i bytes, split into planes of width
       1 (b=1), 2 (b=2), 2+1 (b=3), 4 (b=4), 4+2 (b=6), 4+4 (b=8); the first
       plane holds the low bits.  A plane of width w is w KiB; its dword
       (t, lane, c) at 1024 t + 16 lane + 4 c is the lane's dword d = 4 t + c.
       Each dword holds 16/w code pairs; pair slot i keeps code A in bits
       [w i, w i + w) and code B in bits [16 + w i, 16 + w i + w).  With
       P = d * 16/w + i, u = P // 4, p = P % 4, rt = u // 4, kt = u % 4:
       row = 16 rt + lane % 16, column A = 32 kt + 8 (lane // 16) + 2 p,
       column B = column A + 1 (row and column inside the block).

Version 2: 64x64 blocks (the ScaleBITS explainer's other GPU block size)
-------------------------------------------------------------------------
Same header, magic and sections with version 2, K/64 block columns and
groups of 64 columns.  offs counts 512-byte units.  Block i occupies 512 * b_i
bytes of codes in the same planes; a plane of width w is w half-slots of
512 bytes.  In half-slot j, lane l's 8 bytes at 8 l are two little-endian
words d = 0, 1; each 16-bit half holds 16/w fields of width w, field f of
the low half of word d being the code of row 16 rt + l % 16, column
32 kt + 8 (l // 16) + 2 c and the same field of the high half column + 1,
with c = 2 d + f // (8/w), i = f % (8/w), 4 kt + rt = j (8/w) + i (kt = 0, 1).

W4/W8 image ("GW48")
--------------------
header (first 72 B): u32 magic 0x38345747, u32 version 1, u32 N, u32 K,
u32 n8, u32 n4, u32 T8 = ceil(n8/16), u32 T4 = ceil(n4/16), u64 offsets of
rows, s, z, codes8, codes4 (each 256-byte aligned, rows at 256).
rows   i32 [16 (T8 + T4)]: original output row of each packed row (8-bit rows
       first, then 4-bit rows, each ascending); -1 for padding rows.
s      fp16 [T8 + T4][K/128][16]: scale of packed row 16 t + r in group g.
z      u8 [T4][K/128][16]: zero point (0..15) of the 4-bit rows.
codes8 int8, per (tile t, k-tile kt of 64) a 1 KiB fragment at
       (t * K/64 + kt) * 1024; lane l's 16 bytes at 16 l hold
       q[16 t + l % 16][64 kt + 16 (l // 16) + e], e = 0..15.
codes4 per (t, kt) a 512-byte fragment; lane l's two dwords at 8 l; in dword
       j byte i holds element e = 8 j + i in its low nibble and e = 8 j + i + 4
       in its high nibble (same row/column rule as codes8).
"""
from __future__ import annotations

import numpy as np

GBB_MAGIC = 0x31424247
GW48_MAGIC = 0x38345747
PLANES = {1: (1,), 2: (2,), 3: (2, 1), 4: (4,), 6: (4, 2), 8: (4, 4)}


def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def block_image_size(bits: np.ndarray, block_cols: int = 128) -> int:
    """Byte size of a block image: header, bits, offsets, 256 B of scale/zero
    per block and 64 * block_cols * b / 8 bytes of codes per block (1024 b for
    64x128 blocks, 512 b for 64x64), sections 256-aligned."""
    bits = np.asarray(bits)
    nblk = bits.size
    off = 256
    off = _align256(off + nblk)              # after bits
    off = _align256(off + 4 * (nblk + 1))    # after offsets
    off = off + 256 * nblk                   # after scale/zero
    return off + 8 * block_cols * int(bits.astype(np.int64).sum())


def _plane_codes(plane: np.ndarray, w: int) -> np.ndarray:
    """Decode one plane for many blocks.

    plane: uint8 [nb][w*1024].  Slot j (1 KiB) holds, for lane l, four little-
    endian words c = 0..3; bit field i (width w) of the low half of word c is
    the code of row 16*rt + l%16, column 32*kt + 8*(l//16) + 2*c, the same
    field of the high half that of the next column, with j*(16//w) + i =
    4*kt + rt.  Returns uint8 [nb][64][128] (row, column)."""
    nb = plane.shape[0]
    words = plane.view("<u4").reshape(nb, w, 64, 4)          # [blk][slot][lane][c]
    npair = 16 // w
    mask = (1 << w) - 1
    out = np.empty((nb, 64, 128), np.uint8)
    lane = np.arange(64)
    for j in range(w):
        for c in range(4):
            word = words[:, j, :, c].astype(np.uint64)
            for i in range(npair):
                kt, rt = divmod(j * npair + i, 4)
                row = 16 * rt + lane % 16
                col = 32 * kt + 8 * (lane // 16) + 2 * c
                out[:, row, col] = ((word >> np.uint64(w * i)) & np.uint64(mask)).astype(np.uint8)
                out[:, row, col + 1] = ((word >> np.uint64(16 + w * i)) & np.uint64(mask)).astype(np.uint8)
    return out


def _half_plane_codes(plane: np.ndarray, w: int) -> np.ndarray:
    """Decode one plane of 64x64 blocks (version 2).

    plane: uint8 [nb][w*512]; half-slot j holds, for lane l, two words d;
    field f of the low half of word d is the code of row 16*rt + l%16, column
    32*kt + 8*(l//16) + 2*c with c = 2*d + f//(8//w), j*(8//w) + f%(8//w) =
    4*kt + rt; the high half holds column + 1.  Returns uint8 [nb][64][64]."""
    nb = plane.shape[0]
    words = plane.view("<u4").reshape(nb, w, 64, 2)          # [blk][half-slot][lane][d]
    per = 8 // w
    mask = (1 << w) - 1
    out = np.empty((nb, 64, 64), np.uint8)
    lane = np.arange(64)
    for j in range(w):
        for d in range(2):
            word = words[:, j, :, d].astype(np.uint64)
            for f in range(16 // w):
                c, i = 2 * d + f // per, f % per
                kt, rt = divmod(j * per + i, 4)
                row = 16 * rt + lane % 16
                col = 32 * kt + 8 * (lane // 16) + 2 * c
                out[:, row, col] = ((word >> np.uint64(w * f)) & np.uint64(mask)).astype(np.uint8)
                out[:, row, col + 1] = ((word >> np.uint64(16 + w * f)) & np.uint64(mask)).astype(np.uint8)
    return out


def read_block_image(buf) -> dict:
    """Decode a block image into N, K, bits [N/64][K/128], q uint8 [N][K],
    s16 / z16 float16 [N][K/128]."""
    b = np.frombuffer(bytes(buf) if not isinstance(buf, np.ndarray) else buf.tobytes(), np.uint8)
    magic, ver, N, K, nbr, nbc = (int(v) for v in b[:24].view("<u4"))
    if magic != GBB_MAGIC or ver not in (1, 2):
        raise ValueError("not a version-1 or version-2 block image")
    bcols = 128 if ver == 1 else 64           # block columns (= group size)
    unit = 8 * bcols                          # bytes of codes per bit of width per block
    if nbr * 64 != N or nbc * bcols != K:
        raise ValueError("inconsistent header")
    bits_off, offs_off, sz_off, codes_off, codes_bytes = (int(v) for v in b[24:64].view("<u8"))
    nblk = nbr * nbc
    bits = b[bits_off:bits_off + nblk].copy()
    if not np.isin(bits, list(PLANES)).all():
        raise ValueError("bad bitwidth")
    offs = b[offs_off:offs_off + 4 * (nblk + 1)].view("<u4").astype(np.int64)
    if offs[0] != 0 or not np.array_equal(np.diff(offs), bits.astype(np.int64)):
        raise ValueError("block offsets disagree with bitwidths")
    if offs[-1] * unit != codes_bytes or b.size < codes_off + codes_bytes:
        raise ValueError("code section size")
    sz = b[sz_off:sz_off + 256 * nblk].view("<u2").reshape(nbr, nbc, 16, 4, 2)
    sz = sz.transpose(0, 1, 3, 2, 4).reshape(nbr, nbc, 64, 2)        # row 16 t + r
    s16 = sz[..., 0].copy().view(np.float16).transpose(0, 2, 1).reshape(N, nbc)
    z16 = sz[..., 1].copy().view(np.float16).transpose(0, 2, 1).reshape(N, nbc)

    q = np.empty((nbr, nbc, 64, bcols), np.uint8)
    flat_bits = bits.reshape(-1)
    decode = _plane_codes if ver == 1 else _half_plane_codes
    for bw, widths in PLANES.items():
        idx = np.nonzero(flat_bits == bw)[0]
        if idx.size == 0:
            continue
        starts = codes_off + unit * offs[idx]
        raw = np.stack([b[s:s + unit * bw] for s in starts])      # [nb][unit*bw]
        acc = np.zeros((idx.size, 64, bcols), np.uint16)
        pos, shift = 0, 0
        for w in widths:
            acc |= decode(np.ascontiguousarray(raw[:, pos:pos + unit * w]), w).astype(np.uint16) << shift
            pos += unit * w
            shift += w
        q.reshape(-1, 64, bcols)[idx] = acc.astype(np.uint8)
    q = q.transpose(0, 2, 1, 3).reshape(N, K)
    return dict(N=N, K=K, bits=bits.reshape(nbr, nbc), q=q, s16=s16, z16=z16, block_cols=bcols,
                codes_bytes=codes_bytes, size=codes_off + codes_bytes)


def w48_image_size(N: int, K: int, n8: int) -> int:
    n4 = N - n8
    T8, T4 = (n8 + 15) // 16, (n4 + 15) // 16
    G = K // 128
    off = 256
    off = _align256(off + 4 * 16 * (T8 + T4))     # rows
    off = _align256(off + 2 * (T8 + T4) * G * 16)  # s
    off = _align256(off + T4 * G * 16)            # z
    off = _align256(off + T8 * (K // 64) * 1024)  # codes8
    return off + T4 * (K // 64) * 512


def read_w48_image(buf) -> dict:
    """Decode a W4/W8 image: rows8, rows4 (original indices), q8 int8 [n8][K],
    s8 fp16 [n8][G], q4 uint8 [n4][K], s4 fp16 [n4][G], z4 uint8 [n4][G]."""
    b = np.frombuffer(bytes(buf) if not isinstance(buf, np.ndarray) else buf.tobytes(), np.uint8)
    magic, ver, N, K, n8, n4, T8, T4 = (int(v) for v in b[:32].view("<u4"))
    if magic != GW48_MAGIC or ver != 1 or n8 + n4 != N:
        raise ValueError("not a version-1 W4/W8 image")
    rows_off, s_off, z_off, c8_off, c4_off = (int(v) for v in b[32:72].view("<u8"))
    G, KT = K // 128, K // 64
    rows = b[rows_off:rows_off + 4 * 16 * (T8 + T4)].view("<i4")
    s = b[s_off:s_off + 2 * (T8 + T4) * G * 16].view("<u2").reshape(T8 + T4, G, 16)
    s = s.transpose(0, 2, 1).reshape(16 * (T8 + T4), G).view(np.float16)
    z = b[z_off:z_off + T4 * G * 16].reshape(T4, G, 16).transpose(0, 2, 1).reshape(16 * T4, G)

    lane = np.arange(64)
    c8 = b[c8_off:c8_off + T8 * KT * 1024].view(np.int8).reshape(T8, KT, 64, 16)
    q8 = np.zeros((16 * T8, K), np.int8)
    for e in range(16):
        rr = (np.arange(T8)[:, None] * 16 + lane % 16)            # [T8][64]
        cc = (np.arange(KT)[:, None] * 64 + 16 * (lane // 16) + e)  # [KT][64]
        q8[rr[:, None, :], cc[None, :, :]] = c8[:, :, :, e]
    c4 = b[c4_off:c4_off + T4 * KT * 512].view("<u4").reshape(T4, KT, 64, 2)
    q4 = np.zeros((16 * T4, K), np.uint8)
    for j in range(2):
        for i in range(4):
            byte = (c4[:, :, :, j] >> np.uint32(8 * i)) & np.uint32(0xFF)
            for hi in range(2):
                e = 8 * j + i + 4 * hi
                rr = (np.arange(T4)[:, None] * 16 + lane % 16)
                cc = (np.arange(KT)[:, None] * 64 + 16 * (lane // 16) + e)
                q4[rr[:, None, :], cc[None, :, :]] = ((byte >> np.uint32(4 * hi)) & np.uint32(0xF)).astype(np.uint8)
    rows8 = rows[:n8].copy()
    rows4 = rows[16 * T8:16 * T8 + n4].copy()
    return dict(N=N, K=K, n8=n8, n4=n4, rows8=rows8, rows4=rows4,
                rows_pad=rows.copy(),
                q8=q8[:n8], s8=s[:n8], q4=q4[:n4], s4=s[16 * T8:16 * T8 + n4],
                z4=z[:n4].copy(), q8_pad=q8[n8:], q4_pad=q4[n4:],
                s_pad8=s[n8:16 * T8], s_pad4=s[16 * T8 + n4:], z_pad=z[n4:])
