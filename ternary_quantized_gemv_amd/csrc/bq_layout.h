// bq_layout.h -- internal to libbq: device layout of packed weights, error
// reporting helpers.  Not part of the public ABI (include/bq.h).
//
// Device layout (written by bq_pack, read by the kernels):
//
//   rows are grouped in tiles of 64 (one wavefront: lane i owns row 64t+i);
//   the last tile is padded with zero rows.
//
//   payload plane, u32 words:  [tile][block][lane 0..63][word 0..3]
//     word j of a block is the canonical little-endian payload word j rotated
//     left by 2 bits.  In a canonical word the eight 4-bit nibbles are the
//     eight lane groups (Q1_0: the 4 sign bits of weights 4L..4L+3 of
//     sub-block j; Q2_0: two 2-bit codes).  After the rotation, nibble 2m
//     sits in bits 2..5 of byte m, and nibble 2m+1 does so after a further
//     right rotation by 4, so that masking a byte with 0x3C yields
//     nibble * 4, a byte offset into a table of 16 floats.
//     One wavefront reads one block of its 64 rows as 1 KiB contiguous.
//     Q2_0 only: after every eight tiles the plane leaves a gap of
//     kGroupGap blocks, so tile t starts at block t * nb + 7 * (t / 8)
//     (tile_block0).  Wavefronts that walk neighbouring tiles' rows in step
//     then request different low address bits in each group of eight tiles
//     (measured: the Q2_0 token sweep 2.7% faster; the Q1_0 sweep, slower
//     with every such shift tried, has no gaps).  The gaps are zero and
//     never read.
//
//   scale plane, u16 (f16 bit patterns): [tile][block / 8][lane][block % 8]
//     blocks padded to a multiple of 8 with zero scales; one 16-byte load per
//     lane fetches the scales of 8 consecutive blocks.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace bq {

constexpr int kTileRows = 64;
constexpr int kBlockBytes = 18;
constexpr int kPayloadBytes = 16;
constexpr int kScalesPerGroup = 8;
// The kernels address a 64-row tile's payload (nb * 1 KiB) and its scales
// through one buffer resource with 32-bit offsets, so a tile's payload may
// not exceed this many bytes (cols up to 268,435,328 for Q1_0, 134,217,664
// for Q2_0); rows and cols stay below 2^31.
constexpr int64_t kMaxTileBytes = 0x7FFFFFF0;
constexpr int64_t kMaxDim = int64_t(1) << 31;  // rows and cols must be below this
inline bool tile_fits(int64_t nb) { return nb * kTileRows * kPayloadBytes <= kMaxTileBytes; }

inline int block_len(int fmt) { return fmt == 1 ? 128 : fmt == 2 ? 64 : 0; }
inline int64_t tiles_of(int64_t rows) { return (rows + kTileRows - 1) / kTileRows; }
inline int64_t groups_of(int64_t nb) { return (nb + kScalesPerGroup - 1) / kScalesPerGroup; }

// First block of tile t in the payload plane, and the plane's length in
// blocks for `tiles` tiles.
constexpr int64_t kGroupGap = 7;
constexpr int64_t tile_block0(int fmt, int64_t t, int64_t nb) { return t * nb + (fmt == 2 ? kGroupGap * (t >> 3) : 0); }
inline int64_t payload_blocks(int fmt, int64_t tiles, int64_t nb) { return tile_block0(fmt, tiles - 1, nb) + nb; }

inline uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }
inline uint32_t rotr32(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

// Error reporting: a thread-local message naming the failing call.
int set_error(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace bq

#define BQ_EXPORT extern "C" __attribute__((visibility("default")))
