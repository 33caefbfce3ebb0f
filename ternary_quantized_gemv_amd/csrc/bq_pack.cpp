// bq_pack.cpp -- host side of libbq: error text, ABI version, and the one-time
// repacking of canonical weight blocks into the device layout described in
// bq_layout.h.  bankML's GPU page ("gpu/ -- the video-card component",
// section "kernels.rs") repacks weights once and activations per call, with
// the numbers unchanged; here the 18 bytes of every block are kept (the f16
// scales are not widened) and only re-ordered so that a wavefront reads its
// 64 rows' block as one contiguous 1 KiB (Q2_0 tiles in groups of eight
// with a gap after each group: tile_block0).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bq.h"
#include "bq_layout.h"

namespace bq {

static thread_local char g_err[512];

int set_error(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

static int check_shape(const char *fn, int32_t fmt, int64_t rows, int64_t cols)
{
    int qk = block_len(fmt);
    if (qk == 0)
        return set_error(BQ_EARG, "%s: fmt %d is not BQ_Q1_0 or BQ_Q2_0", fn, (int)fmt);
    if (rows < 1 || cols < 1)
        return set_error(BQ_EARG, "%s: rows (%lld) and cols (%lld) must be >= 1", fn, (long long)rows,
                         (long long)cols);
    if (cols % qk)
        return set_error(BQ_EARG, "%s: cols (%lld) is not a multiple of the block length %d", fn,
                         (long long)cols, qk);
    if (rows >= kMaxDim || cols >= kMaxDim)
        return set_error(BQ_EARG, "%s: rows and cols must be below 2^31", fn);
    if (!tile_fits(cols / qk))
        return set_error(BQ_EARG, "%s: cols %lld: a 64-row tile's payload would exceed %lld bytes", fn,
                         (long long)cols, (long long)kMaxTileBytes);
    return BQ_OK;
}

}  // namespace bq

using namespace bq;

BQ_EXPORT int bq_abi_version(void) { return BQ_ABI_VERSION; }

BQ_EXPORT const char *bq_last_error(void) { return g_err; }

BQ_EXPORT int bq_packed_bytes(int32_t fmt, int64_t rows, int64_t cols, size_t *bits_bytes,
                              size_t *scale_bytes)
{
    int rc = check_shape("bq_packed_bytes", fmt, rows, cols);
    if (rc)
        return rc;
    if (!bits_bytes || !scale_bytes)
        return set_error(BQ_EARG, "bq_packed_bytes: null output pointer");
    int64_t nb = cols / block_len(fmt);
    int64_t tiles = tiles_of(rows);
    *bits_bytes = (size_t)(payload_blocks(fmt, tiles, nb) * kTileRows * kPayloadBytes);
    *scale_bytes = (size_t)(tiles * groups_of(nb) * kTileRows * kScalesPerGroup * 2);
    return BQ_OK;
}

BQ_EXPORT int bq_pack(int32_t fmt, const uint8_t *canon, int64_t rows, int64_t cols, void *bits_out,
                      uint16_t *scales_out)
{
    int rc = check_shape("bq_pack", fmt, rows, cols);
    if (rc)
        return rc;
    if (!canon || !bits_out || !scales_out)
        return set_error(BQ_EARG, "bq_pack: null pointer");
    const int64_t nb = cols / block_len(fmt);
    const int64_t tiles = tiles_of(rows);
    const int64_t ng = groups_of(nb);
    uint32_t *words = static_cast<uint32_t *>(bits_out);
    memset(words, 0, (size_t)(payload_blocks(fmt, tiles, nb) * kTileRows * kPayloadBytes));
    memset(scales_out, 0, (size_t)(tiles * ng * kTileRows * kScalesPerGroup * 2));
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = r / kTileRows, lane = r % kTileRows;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = canon + (r * nb + b) * kBlockBytes;
            uint16_t sc = (uint16_t)(blk[0] | (blk[1] << 8));
            scales_out[((t * ng + b / kScalesPerGroup) * kTileRows + lane) * kScalesPerGroup +
                       b % kScalesPerGroup] = sc;
            uint32_t *dst = words + ((tile_block0(fmt, t, nb) + b) * kTileRows + lane) * 4;
            for (int j = 0; j < 4; ++j) {
                const uint8_t *p = blk + 2 + 4 * j;
                uint32_t w = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                             ((uint32_t)p[3] << 24);
                dst[j] = rotl32(w, 2);
            }
        }
    }
    return BQ_OK;
}

BQ_EXPORT int bq_unpack(int32_t fmt, const void *bits, const uint16_t *scales, int64_t rows, int64_t cols,
                        uint8_t *canon_out)
{
    int rc = check_shape("bq_unpack", fmt, rows, cols);
    if (rc)
        return rc;
    if (!bits || !scales || !canon_out)
        return set_error(BQ_EARG, "bq_unpack: null pointer");
    const int64_t nb = cols / block_len(fmt);
    const int64_t ng = groups_of(nb);
    const uint32_t *words = static_cast<const uint32_t *>(bits);
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = r / kTileRows, lane = r % kTileRows;
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *blk = canon_out + (r * nb + b) * kBlockBytes;
            uint16_t sc = scales[((t * ng + b / kScalesPerGroup) * kTileRows + lane) * kScalesPerGroup +
                                 b % kScalesPerGroup];
            blk[0] = (uint8_t)(sc & 0xFF);
            blk[1] = (uint8_t)(sc >> 8);
            const uint32_t *src = words + ((tile_block0(fmt, t, nb) + b) * kTileRows + lane) * 4;
            for (int j = 0; j < 4; ++j) {
                uint32_t w = rotr32(src[j], 2);
                for (int i = 0; i < 4; ++i)
                    blk[2 + 4 * j + i] = (uint8_t)(w >> (8 * i));
            }
        }
    }
    return BQ_OK;
}
