// Byte layout of the two packed weight images (host and device code).
//
// The pages fix only the ingredients: 64x128 blocks with one bitwidth each,
// stored block by block next to a small bitwidth record (ScaleBITS explainer
// page, section 3.2), and a weight layout pre-packed so that nothing is
// permuted at run time (MixLLM page, section 3.3).  The concrete layout below
// is chosen for gfx950: every 1 KiB of codes is one fully coalesced 16-byte
// load per lane of a 64-lane wavefront, and the codes a lane loads are exactly
// the weights it feeds to the matrix cores (the A/B operand of
// v_mfma_f32_16x16x32_f16 or v_mfma_i32_16x16x64_i8).
#pragma once
#include <cstddef>
#include <cstdint>

namespace gbb {

constexpr uint32_t kMagicBlocks = 0x31424247u;  // "GBB1"
constexpr uint32_t kMagicW48 = 0x38345747u;     // "GW48"
constexpr uint32_t kVersion = 1;     // 64x128 blocks
constexpr uint32_t kVersion64 = 2;   // 64x64 blocks
constexpr int kBlockRows = 64;
constexpr int kGroup = 128;

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Block image: 64-byte header, then 256-byte aligned sections
//   bits  u8 [nblk]            block index = block_row * (K/128) + block_col
//   offs  u32 [nblk + 1]       start of each block's codes, in KiB
//   sz    u32 [nblk][16][4]    entry [r][t] is row 16 t + r of the block:
//                              fp16 s (low half), fp16 z (high half)
//   codes 1024 * b bytes per block, planes of width 1|2|4 (low bits first).
//         A plane of width w is w slots of 1 KiB; lane l's 16 bytes of slot j
//         are four u32 words c = 0..3 whose bit field i (width w) of the low
//         half holds the code of row 16 rt + l % 16, column
//         32 kt + 8 (l / 16) + 2 c, and of the high half the next column, for
//         4 kt + rt = j (16 / w) + i.  So the four words of a slot at one field
//         are one v_mfma_f32_16x16x32_f16 B operand (tile rt, kt).
//
// Version 2 (64x64 blocks, groups of 64 columns): the same sections with
// K/64 block columns; offs counts 512-byte units and a block holds 512 * b
// bytes.  A plane of width w is w half-slots of 512 bytes; lane l's 8 bytes
// of half-slot j are two u32 words d = 0, 1 whose bit field f (width w) of
// the low half holds the code of row 16 rt + l % 16, column 32 kt +
// 8 (l / 16) + 2 c, and of the high half the next column, for
// c = 2 d + f / (8 / w) and 4 kt + rt = j (8 / w) + f % (8 / w), kt = 0, 1.
// So the two words, each read at two field positions, give the four words
// of one MFMA B operand.
struct BlockLayout {
  size_t nblk, bits_off, offs_off, sz_off, codes_off;
};

inline BlockLayout block_layout(int N, int K, int bc = kGroup) {
  BlockLayout l;
  l.nblk = size_t(N / kBlockRows) * size_t(K / bc);
  l.bits_off = 256;
  l.offs_off = align256(l.bits_off + l.nblk);
  l.sz_off = align256(l.offs_off + 4 * (l.nblk + 1));
  l.codes_off = l.sz_off + 256 * l.nblk;
  return l;
}

struct BlockHeader {
  uint32_t magic, version, N, K, nbr, nbc;
  uint64_t bits_off, offs_off, sz_off, codes_off, codes_bytes;
};
static_assert(sizeof(BlockHeader) == 64, "header is 64 bytes");

// Plane split of a bitwidth: widths (low plane first) and the shift of the
// second plane.  b = 1, 2, 4 are one plane; 3 = 2 + 1, 6 = 4 + 2, 8 = 4 + 4.
inline bool valid_bits(int b) { return b == 1 || b == 2 || b == 3 || b == 4 || b == 6 || b == 8; }
inline int plane0_width(int b) { return b == 3 ? 2 : (b >= 4 ? 4 : b); }
inline int plane1_width(int b) { return b == 3 ? 1 : (b == 6 ? 2 : (b == 8 ? 4 : 0)); }

// W4/W8 image: 64-byte header, then 256-byte aligned sections
//   rows   i32 [16 (T8 + T4)]     original row of each packed row, -1 = padding
//   s      fp16 [T8 + T4][K/128][16]
//   z      u8 [T4][K/128][16]
//   codes8 int8 fragments, 1 KiB per (16-row tile, 64-column k tile)
//   codes4 nibble fragments, 512 B per (16-row tile, 64-column k tile)
struct W48Layout {
  int T8, T4;
  size_t rows_off, s_off, z_off, c8_off, c4_off, total;
};

inline W48Layout w48_layout(int N, int K, int n8) {
  W48Layout l;
  const int n4 = N - n8;
  l.T8 = (n8 + 15) / 16;
  l.T4 = (n4 + 15) / 16;
  const size_t G = size_t(K / kGroup), KT = size_t(K / 64);
  l.rows_off = 256;
  l.s_off = align256(l.rows_off + 4 * 16 * size_t(l.T8 + l.T4));
  l.z_off = align256(l.s_off + 2 * size_t(l.T8 + l.T4) * G * 16);
  l.c8_off = align256(l.z_off + size_t(l.T4) * G * 16);
  l.c4_off = align256(l.c8_off + size_t(l.T8) * KT * 1024);
  l.total = l.c4_off + size_t(l.T4) * KT * 512;
  return l;
}

struct W48Header {
  uint32_t magic, version, N, K, n8, n4, T8, T4;
  uint64_t rows_off, s_off, z_off, c8_off, c4_off;
  uint64_t reserved[3];
};
static_assert(sizeof(W48Header) == 96, "w48 header");

}  // namespace gbb
