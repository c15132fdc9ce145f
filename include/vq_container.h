/*
 * vq_container.h - on-disk container of VQ3R / VQ4P expert records (libvq).
 *
 * [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".
 * Its §4 describes the conversion path this container serves:
 *   - the per-layer codebooks are stored with the container (as a codebooks
 *     file that the engine keeps resident in memory);
 *   - each expert is stored as the encoder's winning indices;
 *   - a verifier dequantizes the container and compares it, record by record,
 *     with the source weights, to confirm that the stored data reproduces the
 *     measured precision.
 * §1 streams experts from disk on demand, so a record must be cheap to move
 * into device memory; §5 makes VQ4P a separate, explicitly chosen record
 * format. The page points to a format specification that it does not
 * reproduce: the byte layout below is this library's own.
 *
 * One container holds n_records records of one shape [rows x cols] and one
 * codebook set (for example the w1 matrices of all experts of one layer).
 *
 * Layout: little-endian; every section and every record starts at a multiple
 * of 4096 bytes, so a record can be read into a page-aligned pinned buffer and
 * copied to device memory as it is.
 *
 *   offset 0: header, 4096 bytes
 *       0  char[4]  magic "VQC1"
 *       4  u32      version = 1
 *       8  u32      format (vq_format)
 *      12  u32      stages (3 or 4)
 *      16  u32      entries per codebook (256 or 64)
 *      20  u32      0
 *      24  u64      rows per record
 *      32  u64      cols per record (a multiple of 8)
 *      40  u64      n_records
 *      48  u64      codebooks offset (= 4096)
 *      56  u64      codebooks bytes (= stages * entries * 8 * 4)
 *      64  u64      table offset
 *      72  u64      table bytes (= n_records * 64)
 *      80  u64      records offset
 *      88  u64      record stride
 *      96  u64      scales bytes per record (= rows * 2)
 *     104  u64      index offset inside a record (scales bytes rounded up to 256)
 *     112  u64      index bytes per record (= rows * cols / 8 * 3)
 *     120  u32      CRC-32 of the codebook bytes
 *     124  u32      CRC-32 of header bytes [0, 124)
 *     128  zero up to 4096
 *   codebooks: fp32 [stages][entries][8]
 *   record table: n_records entries of 64 bytes
 *       0  u64      offset of the record in the file
 *       8  u32      CRC-32 of the record's scale bytes followed by its index bytes
 *      12  u32      flags: bit 0 = the record has been written
 *      16  f64[4]   stored relative Frobenius error after stages 1..4 (NaN = none)
 *      48  zero up to 64
 *   records: record r at (records offset + r * record stride)
 *       fp16 scale bits [rows], zero up to the index offset,
 *       index bytes [rows][cols/8][3] exactly as vq_encode writes them,
 *       zero up to the stride (a multiple of 4096).
 *
 * CRC-32 is the IEEE 802.3 polynomial (reflected form 0xEDB88320, initial value
 * and final xor 0xFFFFFFFF), the checksum of zlib and PNG.
 *
 * All functions are host functions and are not thread-safe for concurrent
 * writers of one file. Paths are NUL-terminated. Return values are vq_status
 * codes (vq.h); VQ_EIO reports a failed or short open/read/write, VQ_EFORMAT a
 * file that is not a container of this version, a checksum mismatch, a record
 * that was never written, or a shape that does not match.
 */
#ifndef VQ_CONTAINER_H
#define VQ_CONTAINER_H

#include <stddef.h>
#include <stdint.h>

#include "vq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of a container of n_records records of [rows x cols] in
 * `format`; 0 for invalid sizes (cols % 8, rows < 1, n_records < 0, or a record
 * beyond the per-call limits of vq.h). Each out-parameter may be NULL. */
uint64_t vqc_layout(int format, int64_t rows, int64_t cols, int64_t n_records, uint64_t* table_offset,
                    uint64_t* records_offset, uint64_t* record_stride);

/* CRC-32 (see above) of n host bytes, continuing from `crc` (0 to start). */
uint32_t vqc_crc32(uint32_t crc, const void* data, size_t n);

/* Creates or truncates `path` and writes the header, the codebooks (host fp32
 * [stages][entries][8]) and an empty record table, and extends the file to its
 * full size. Records are then written with vqc_write_records. */
int vqc_create(const char* path, int format, int64_t rows, int64_t cols, int64_t n_records, const float* codebooks);

/* Writes records [first, first + count) from host buffers: scales fp16 bits
 * [count][rows], idx [count][rows][cols/8][3], and optionally rel_err f64
 * [count][4] (the measured relative error after each stage; NULL stores NaN).
 * Each record's table entry gets its CRC-32 and the written flag. */
int vqc_write_records(const char* path, int64_t first, int64_t count, const uint16_t* scales, const uint8_t* idx,
                      const double* rel_err);

/* Reads and validates the header (magic, version, header CRC, file size).
 * Each out-parameter may be NULL. */
int vqc_info(const char* path, int* format, int64_t* rows, int64_t* cols, int64_t* n_records);

/* Reads the codebooks (host fp32 [stages][entries][8]) and checks their CRC. */
int vqc_read_codebooks(const char* path, float* codebooks);

/* Reads records [first, first + count) into host buffers (layouts as in
 * vqc_write_records; rel_err may be NULL). Every record must have been written
 * and must match its CRC, else VQ_EFORMAT and the outputs are unspecified. */
int vqc_read_records(const char* path, int64_t first, int64_t count, uint16_t* scales, uint8_t* idx,
                     double* rel_err);

/* Streams records [first, first + count) into DEVICE buffers scales_dev fp16
 * [count][rows] and idx_dev [count][rows][cols/8][3] through a caller-owned
 * host staging buffer (pinned with hipHostMalloc for asynchronous copies;
 * 4096-byte aligned; at least 2 * record stride bytes). The file is read into
 * the two halves of the staging buffer in turn; each record's CRC is checked
 * on the host before its copy to the device is enqueued on `stream`, so reading
 * the next records overlaps the copies of the previous ones. Returns after
 * every copy has completed. rel_err (host f64 [count][4]) may be NULL. On an
 * error the device buffers may be partly written. */
int vqc_load_records(const char* path, int64_t first, int64_t count, uint16_t* scales_dev, uint8_t* idx_dev,
                     double* rel_err, void* staging, size_t staging_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_CONTAINER_H */
