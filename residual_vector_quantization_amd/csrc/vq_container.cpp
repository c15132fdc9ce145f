// Container of VQ3R / VQ4P expert records (byte layout in vq_container.h):
// a header, the codebooks, a record table with per-record CRC-32 and stored
// errors, and 4096-aligned records that hold the encoder's output unchanged.
// [VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验":
// §1 experts streamed from disk on demand (vqc_load_records moves records
// into device memory through a pinned staging buffer, reading the next
// records while the previous ones are copied), §4 codebooks stored with the
// container and record-by-record verification against the source weights
// (the stored per-stage errors and CRCs), §5 VQ4P records.
#include <errno.h>
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "../../include/vq_container.h"

namespace {

constexpr uint64_t kAlign = 4096, kHeaderBytes = 4096, kEntryBytes = 64;
constexpr uint32_t kFileVersion = 1;
constexpr char kMagic[4] = {'V', 'Q', 'C', '1'};

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct Layout {
  uint32_t format, stages, entries;
  uint64_t rows, cols, n;
  uint64_t cb_off, cb_bytes, table_off, table_bytes, rec_off, stride, sc_bytes, idx_off, idx_bytes, total;
};

bool make_layout(int format, int64_t rows, int64_t cols, int64_t n, Layout& L) {
  if (format != VQ_FMT_VQ3R && format != VQ_FMT_VQ4P) return false;
  if (rows < 1 || cols < 8 || cols % 8 != 0 || cols > (1 << 20) || n < 0 || n > (int64_t(1) << 31)) return false;
  if ((uint64_t)rows * (uint64_t)(cols / 8) >= (uint64_t(1) << 32)) return false;
  L.format = (uint32_t)format;
  L.stages = format == VQ_FMT_VQ3R ? 3 : 4;
  L.entries = format == VQ_FMT_VQ3R ? 256 : 64;
  L.rows = (uint64_t)rows;
  L.cols = (uint64_t)cols;
  L.n = (uint64_t)n;
  L.cb_off = kHeaderBytes;
  L.cb_bytes = (uint64_t)L.stages * L.entries * 8 * 4;
  L.table_off = round_up(L.cb_off + L.cb_bytes, kAlign);
  L.table_bytes = L.n * kEntryBytes;
  L.rec_off = round_up(L.table_off + L.table_bytes, kAlign);
  L.sc_bytes = L.rows * 2;
  L.idx_off = round_up(L.sc_bytes, 256);
  L.idx_bytes = L.rows * (L.cols / 8) * 3;
  L.stride = round_up(L.idx_off + L.idx_bytes, kAlign);
  L.total = L.rec_off + L.n * L.stride;
  return true;
}

// ---------------------------------------------------------------- CRC-32
// Reflected IEEE polynomial 0xEDB88320, eight bytes per step with eight
// derived tables (the slicing-by-8 method of Kounavis and Berry): table k maps
// a byte to the CRC of that byte followed by k zero bytes.
struct CrcTables {
  uint32_t t[8][256];
  CrcTables() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? (c >> 1) ^ 0xEDB88320u : (c >> 1);
      t[0][i] = c;
    }
    for (int k = 1; k < 8; ++k)
      for (uint32_t i = 0; i < 256; ++i) t[k][i] = (t[k - 1][i] >> 8) ^ t[0][t[k - 1][i] & 0xFFu];
  }
};

const CrcTables& crc_tables() {
  static const CrcTables tables;
  return tables;
}

uint32_t crc32_update(uint32_t crc, const uint8_t* p, size_t n) {
  const CrcTables& T = crc_tables();
  uint32_t c = ~crc;
  while (n >= 8) {
    uint32_t lo, hi;
    memcpy(&lo, p, 4);
    memcpy(&hi, p + 4, 4);
    lo ^= c;
    c = T.t[7][lo & 0xFF] ^ T.t[6][(lo >> 8) & 0xFF] ^ T.t[5][(lo >> 16) & 0xFF] ^ T.t[4][lo >> 24] ^
        T.t[3][hi & 0xFF] ^ T.t[2][(hi >> 8) & 0xFF] ^ T.t[1][(hi >> 16) & 0xFF] ^ T.t[0][hi >> 24];
    p += 8;
    n -= 8;
  }
  while (n--) c = (c >> 8) ^ T.t[0][(c ^ *p++) & 0xFF];
  return ~c;
}

// ---------------------------------------------------------------- file helpers
struct Fd {
  int fd = -1;
  ~Fd() {
    if (fd >= 0) close(fd);
  }
};

bool pread_all(int fd, void* buf, uint64_t n, uint64_t off) {
  uint8_t* p = static_cast<uint8_t*>(buf);
  while (n > 0) {
    const ssize_t r = pread(fd, p, n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (uint64_t)r;
    off += (uint64_t)r;
  }
  return true;
}

bool pwrite_all(int fd, const void* buf, uint64_t n, uint64_t off) {
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  while (n > 0) {
    const ssize_t r = pwrite(fd, p, n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (uint64_t)r;
    off += (uint64_t)r;
  }
  return true;
}

template <class T>
void put(uint8_t* h, size_t off, T v) {
  memcpy(h + off, &v, sizeof(T));
}
template <class T>
T get(const uint8_t* h, size_t off) {
  T v;
  memcpy(&v, h + off, sizeof(T));
  return v;
}

void make_header(const Layout& L, uint32_t cb_crc, uint8_t* h) {
  memset(h, 0, kHeaderBytes);
  memcpy(h, kMagic, 4);
  put<uint32_t>(h, 4, kFileVersion);
  put<uint32_t>(h, 8, L.format);
  put<uint32_t>(h, 12, L.stages);
  put<uint32_t>(h, 16, L.entries);
  put<uint64_t>(h, 24, L.rows);
  put<uint64_t>(h, 32, L.cols);
  put<uint64_t>(h, 40, L.n);
  put<uint64_t>(h, 48, L.cb_off);
  put<uint64_t>(h, 56, L.cb_bytes);
  put<uint64_t>(h, 64, L.table_off);
  put<uint64_t>(h, 72, L.table_bytes);
  put<uint64_t>(h, 80, L.rec_off);
  put<uint64_t>(h, 88, L.stride);
  put<uint64_t>(h, 96, L.sc_bytes);
  put<uint64_t>(h, 104, L.idx_off);
  put<uint64_t>(h, 112, L.idx_bytes);
  put<uint32_t>(h, 120, cb_crc);
  put<uint32_t>(h, 124, crc32_update(0, h, 124));
}

// Opens `path` and checks its header against a layout rebuilt from the stored
// format and shape; on success fills L and the codebook CRC.
int open_container(const char* path, int flags, Fd& f, Layout& L, uint32_t& cb_crc) {
  if (!path) return VQ_EINVAL;
  f.fd = open(path, flags | O_CLOEXEC);
  if (f.fd < 0) return VQ_EIO;
  uint8_t h[kHeaderBytes];
  if (!pread_all(f.fd, h, kHeaderBytes, 0)) return VQ_EFORMAT;  // shorter than a header
  if (memcmp(h, kMagic, 4) != 0 || get<uint32_t>(h, 4) != kFileVersion) return VQ_EFORMAT;
  if (get<uint32_t>(h, 124) != crc32_update(0, h, 124)) return VQ_EFORMAT;
  const uint64_t rows = get<uint64_t>(h, 24), cols = get<uint64_t>(h, 32), n = get<uint64_t>(h, 40);
  if (rows > (uint64_t(1) << 40) || cols > (uint64_t(1) << 40) || n > (uint64_t(1) << 40)) return VQ_EFORMAT;
  if (!make_layout((int)get<uint32_t>(h, 8), (int64_t)rows, (int64_t)cols, (int64_t)n, L)) return VQ_EFORMAT;
  cb_crc = get<uint32_t>(h, 120);
  uint8_t expect[kHeaderBytes];
  make_header(L, cb_crc, expect);
  if (memcmp(h, expect, kHeaderBytes) != 0) return VQ_EFORMAT;
  struct stat st;
  if (fstat(f.fd, &st) != 0) return VQ_EIO;
  if ((uint64_t)st.st_size < L.total) return VQ_EFORMAT;  // truncated
  return VQ_OK;
}

struct Entry {
  uint64_t offset;
  uint32_t crc, flags;
  double rel_err[4];
};

void encode_entry(const Entry& e, uint8_t* b) {
  memset(b, 0, kEntryBytes);
  put<uint64_t>(b, 0, e.offset);
  put<uint32_t>(b, 8, e.crc);
  put<uint32_t>(b, 12, e.flags);
  for (int s = 0; s < 4; ++s) put<double>(b, 16 + 8 * s, e.rel_err[s]);
}

Entry decode_entry(const uint8_t* b) {
  Entry e;
  e.offset = get<uint64_t>(b, 0);
  e.crc = get<uint32_t>(b, 8);
  e.flags = get<uint32_t>(b, 12);
  for (int s = 0; s < 4; ++s) e.rel_err[s] = get<double>(b, 16 + 8 * s);
  return e;
}

int read_entries(int fd, const Layout& L, int64_t first, int64_t count, std::vector<Entry>& out) {
  std::vector<uint8_t> raw((size_t)count * kEntryBytes);
  if (count > 0 && !pread_all(fd, raw.data(), raw.size(), L.table_off + (uint64_t)first * kEntryBytes))
    return VQ_EIO;
  out.resize((size_t)count);
  for (int64_t r = 0; r < count; ++r) {
    out[(size_t)r] = decode_entry(raw.data() + r * kEntryBytes);
    if (out[(size_t)r].offset != L.rec_off + (uint64_t)(first + r) * L.stride) return VQ_EFORMAT;
    if (!(out[(size_t)r].flags & 1u)) return VQ_EFORMAT;  // never written
  }
  return VQ_OK;
}

uint32_t record_crc(const Layout& L, const uint8_t* rec) {
  return crc32_update(crc32_update(0, rec, L.sc_bytes), rec + L.idx_off, L.idx_bytes);
}

// Reads k consecutive records into a buffer and checks their CRCs, the
// records spread over a few host threads (each thread reads and checks its
// own records, so page-cache copies and checksums run in parallel).
// Returns VQ_OK, VQ_EIO or VQ_EFORMAT.
int read_check_records(int fd, const Layout& L, uint8_t* buf, const Entry* e, int64_t k) {
  const unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  const int64_t nth = (L.stride * (uint64_t)k < (uint64_t(8) << 20)) ? 1 : std::min<int64_t>(k, (int64_t)hw);
  std::vector<int> st((size_t)k, VQ_OK);
  auto work = [&](int64_t t) {
    for (int64_t r = t; r < k; r += nth) {
      uint8_t* rec = buf + r * L.stride;
      if (!pread_all(fd, rec, L.stride, e[r].offset)) st[(size_t)r] = VQ_EIO;
      else if (record_crc(L, rec) != e[r].crc) st[(size_t)r] = VQ_EFORMAT;
    }
  };
  std::vector<std::thread> th;
  for (int64_t t = 1; t < nth; ++t) th.emplace_back(work, t);
  work(0);
  for (auto& x : th) x.join();
  for (int64_t r = 0; r < k; ++r)
    if (st[(size_t)r] != VQ_OK) return st[(size_t)r];
  return VQ_OK;
}

bool range_ok(const Layout& L, int64_t first, int64_t count) {
  return first >= 0 && count >= 0 && (uint64_t)first + (uint64_t)count <= L.n;
}

}  // namespace

extern "C" {

uint64_t vqc_layout(int format, int64_t rows, int64_t cols, int64_t n_records, uint64_t* table_offset,
                    uint64_t* records_offset, uint64_t* record_stride) {
  Layout L;
  if (!make_layout(format, rows, cols, n_records, L)) return 0;
  if (table_offset) *table_offset = L.table_off;
  if (records_offset) *records_offset = L.rec_off;
  if (record_stride) *record_stride = L.stride;
  return L.total;
}

uint32_t vqc_crc32(uint32_t crc, const void* data, size_t n) {
  if (!data && n) return crc;
  return crc32_update(crc, static_cast<const uint8_t*>(data), n);
}

int vqc_create(const char* path, int format, int64_t rows, int64_t cols, int64_t n_records, const float* codebooks) {
  Layout L;
  if (!path || !codebooks || !make_layout(format, rows, cols, n_records, L)) return VQ_EINVAL;
  Fd f;
  f.fd = open(path, O_CREAT | O_TRUNC | O_RDWR | O_CLOEXEC, 0644);
  if (f.fd < 0) return VQ_EIO;
  const uint32_t cb_crc = crc32_update(0, reinterpret_cast<const uint8_t*>(codebooks), L.cb_bytes);
  std::vector<uint8_t> h(kHeaderBytes);
  make_header(L, cb_crc, h.data());
  if (!pwrite_all(f.fd, h.data(), kHeaderBytes, 0)) return VQ_EIO;
  if (!pwrite_all(f.fd, codebooks, L.cb_bytes, L.cb_off)) return VQ_EIO;
  std::vector<uint8_t> table((size_t)L.table_bytes);
  for (uint64_t r = 0; r < L.n; ++r) {
    Entry e;
    e.offset = L.rec_off + r * L.stride;
    e.crc = 0;
    e.flags = 0;
    for (int s = 0; s < 4; ++s) e.rel_err[s] = NAN;
    encode_entry(e, table.data() + r * kEntryBytes);
  }
  if (L.n && !pwrite_all(f.fd, table.data(), table.size(), L.table_off)) return VQ_EIO;
  if (ftruncate(f.fd, (off_t)L.total) != 0) return VQ_EIO;
  return VQ_OK;
}

int vqc_write_records(const char* path, int64_t first, int64_t count, const uint16_t* scales, const uint8_t* idx,
                      const double* rel_err) {
  if (count > 0 && (!scales || !idx)) return VQ_EINVAL;
  Fd f;
  Layout L;
  uint32_t cb_crc;
  int st = open_container(path, O_RDWR, f, L, cb_crc);
  if (st != VQ_OK) return st;
  if (!range_ok(L, first, count)) return VQ_EINVAL;
  std::vector<uint8_t> rec((size_t)L.stride), ent(kEntryBytes);
  for (int64_t r = 0; r < count; ++r) {
    std::fill(rec.begin(), rec.end(), 0);
    memcpy(rec.data(), scales + (uint64_t)r * L.rows, L.sc_bytes);
    memcpy(rec.data() + L.idx_off, idx + (uint64_t)r * L.idx_bytes, L.idx_bytes);
    Entry e;
    e.offset = L.rec_off + (uint64_t)(first + r) * L.stride;
    e.crc = record_crc(L, rec.data());
    e.flags = 1u;
    for (int s = 0; s < 4; ++s) e.rel_err[s] = (rel_err && s < (int)L.stages) ? rel_err[r * 4 + s] : NAN;
    encode_entry(e, ent.data());
    if (!pwrite_all(f.fd, rec.data(), L.stride, e.offset)) return VQ_EIO;
    if (!pwrite_all(f.fd, ent.data(), kEntryBytes, L.table_off + (uint64_t)(first + r) * kEntryBytes)) return VQ_EIO;
  }
  return VQ_OK;
}

int vqc_info(const char* path, int* format, int64_t* rows, int64_t* cols, int64_t* n_records) {
  Fd f;
  Layout L;
  uint32_t cb_crc;
  const int st = open_container(path, O_RDONLY, f, L, cb_crc);
  if (st != VQ_OK) return st;
  if (format) *format = (int)L.format;
  if (rows) *rows = (int64_t)L.rows;
  if (cols) *cols = (int64_t)L.cols;
  if (n_records) *n_records = (int64_t)L.n;
  return VQ_OK;
}

int vqc_read_codebooks(const char* path, float* codebooks) {
  if (!codebooks) return VQ_EINVAL;
  Fd f;
  Layout L;
  uint32_t cb_crc;
  const int st = open_container(path, O_RDONLY, f, L, cb_crc);
  if (st != VQ_OK) return st;
  if (!pread_all(f.fd, codebooks, L.cb_bytes, L.cb_off)) return VQ_EIO;
  if (crc32_update(0, reinterpret_cast<const uint8_t*>(codebooks), L.cb_bytes) != cb_crc) return VQ_EFORMAT;
  return VQ_OK;
}

int vqc_read_records(const char* path, int64_t first, int64_t count, uint16_t* scales, uint8_t* idx,
                     double* rel_err) {
  if (count > 0 && (!scales || !idx)) return VQ_EINVAL;
  Fd f;
  Layout L;
  uint32_t cb_crc;
  int st = open_container(path, O_RDONLY, f, L, cb_crc);
  if (st != VQ_OK) return st;
  if (!range_ok(L, first, count)) return VQ_EINVAL;
  std::vector<Entry> ents;
  if ((st = read_entries(f.fd, L, first, count, ents)) != VQ_OK) return st;
  std::vector<uint8_t> rec((size_t)L.stride);
  for (int64_t r = 0; r < count; ++r) {
    if (!pread_all(f.fd, rec.data(), L.stride, ents[(size_t)r].offset)) return VQ_EIO;
    if (record_crc(L, rec.data()) != ents[(size_t)r].crc) return VQ_EFORMAT;
    memcpy(scales + (uint64_t)r * L.rows, rec.data(), L.sc_bytes);
    memcpy(idx + (uint64_t)r * L.idx_bytes, rec.data() + L.idx_off, L.idx_bytes);
    if (rel_err)
      for (int s = 0; s < 4; ++s) rel_err[r * 4 + s] = ents[(size_t)r].rel_err[s];
  }
  return VQ_OK;
}

int vqc_load_records(const char* path, int64_t first, int64_t count, uint16_t* scales_dev, uint8_t* idx_dev,
                     double* rel_err, void* staging, size_t staging_bytes, void* stream) {
  if (count > 0 && (!scales_dev || !idx_dev)) return VQ_EINVAL;
  Fd f;
  Layout L;
  uint32_t cb_crc;
  int st = open_container(path, O_RDONLY, f, L, cb_crc);
  if (st != VQ_OK) return st;
  if (!range_ok(L, first, count)) return VQ_EINVAL;
  if (count == 0) return VQ_OK;
  if (!staging || (reinterpret_cast<uintptr_t>(staging) & (kAlign - 1)) != 0 || staging_bytes < 2 * L.stride)
    return VQ_EWORKSPACE;
  std::vector<Entry> ents;
  if ((st = read_entries(f.fd, L, first, count, ents)) != VQ_OK) return st;
  if (rel_err)
    for (int64_t r = 0; r < count; ++r)
      for (int s = 0; s < 4; ++s) rel_err[r * 4 + s] = ents[(size_t)r].rel_err[s];
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint64_t half = (staging_bytes / 2) / kAlign * kAlign;
  const int64_t per = (int64_t)(half / L.stride);  // >= 1 records per half
  uint8_t* buf[2] = {static_cast<uint8_t*>(staging), static_cast<uint8_t*>(staging) + half};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  for (int h = 0; h < 2; ++h)
    if (hipEventCreateWithFlags(&ev[h], hipEventDisableTiming) != hipSuccess) st = VQ_EDEVICE;
  for (int64_t r0 = 0, batch = 0; st == VQ_OK && r0 < count; r0 += per, ++batch) {
    const int h = (int)(batch & 1);
    const int64_t k = std::min(per, count - r0);
    // the copies out of this half (two batches ago) must be done before it is refilled
    if (pending[h] && hipEventSynchronize(ev[h]) != hipSuccess) {
      st = VQ_EDEVICE;
      break;
    }
    pending[h] = false;
    if ((st = read_check_records(f.fd, L, buf[h], &ents[(size_t)r0], k)) != VQ_OK) break;
    for (int64_t r = 0; r < k && st == VQ_OK; ++r) {
      const uint8_t* rec = buf[h] + r * L.stride;
      if (hipMemcpyAsync(scales_dev + (uint64_t)(r0 + r) * L.rows, rec, L.sc_bytes, hipMemcpyHostToDevice, s) !=
              hipSuccess ||
          hipMemcpyAsync(idx_dev + (uint64_t)(r0 + r) * L.idx_bytes, rec + L.idx_off, L.idx_bytes,
                         hipMemcpyHostToDevice, s) != hipSuccess)
        st = VQ_EDEVICE;
    }
    if (st == VQ_OK && hipEventRecord(ev[h], s) != hipSuccess) st = VQ_EDEVICE;
    pending[h] = st == VQ_OK;
  }
  // every copy that was enqueued reads the staging buffer: wait for all of them
  if (hipStreamSynchronize(s) != hipSuccess && st == VQ_OK) st = VQ_EDEVICE;
  for (int h = 0; h < 2; ++h)
    if (ev[h]) (void)hipEventDestroy(ev[h]);
  return st;
}

}  // extern "C"
