// lbf_api.cpp — the C ABI of liblbf.so: argument and descriptor checks, the
// host part of encoding (choice of the 15 coded exponents), and dispatch to
// the gfx950 kernels.  Declarations and conventions: include/lbf.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "lbf.h"
#include "lbf_internal.h"

static_assert(sizeof(lbf_desc) == 96, "descriptor must be 96 bytes");
static_assert(offsetof(lbf_desc, lut) == 72, "descriptor layout");
static_assert(offsetof(lbf_desc, n_codes) == 88, "descriptor layout");
static_assert(offsetof(lbf_desc, desc_crc) == 92, "descriptor layout");
static_assert(sizeof(lbf_hdesc) == 128, "K15H descriptor must be 128 bytes");
static_assert(offsetof(lbf_hdesc, lut) == 88, "K15H descriptor layout");
static_assert(offsetof(lbf_hdesc, n_codes) == 104, "K15H descriptor layout");
static_assert(offsetof(lbf_hdesc, len) == 108, "K15H descriptor layout");
static_assert(offsetof(lbf_hdesc, desc_crc) == 124, "K15H descriptor layout");

namespace lbf {

Layout layout_of(uint64_t rows, uint64_t cols, uint64_t n_esc) {
  auto up = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
  Layout L;
  L.n = rows * cols;
  L.n_tiles = (L.n + LBF_TILE - 1) / LBF_TILE;
  L.n_esc = n_esc;
  L.off_raw = LBF_HEADER_BYTES;
  L.off_nib = up(L.off_raw + L.n_tiles * LBF_TILE);
  L.off_idx = up(L.off_nib + L.n_tiles * (LBF_TILE / 2));
  L.off_esc = up(L.off_idx + 4 * (L.n_tiles + 1));
  L.blob_bytes = up(L.off_esc + n_esc);
  return L;
}

// Launch facts per device.  One lock guards the three tables; every entry is
// computed at most once per device (per kernel and block size), so the lock
// is taken on the host side of a launch only, never while a kernel waits.
namespace {
std::mutex g_facts_mu;
std::map<int, int> g_cus;                                    // device -> CUs
std::map<std::tuple<const void*, int, int>, int> g_per_cu;   // (kernel, device, block) -> blocks a CU
std::map<std::pair<const void*, int>, int> g_lds;            // (kernel, device) -> dynamic LDS opened
}  // namespace

hipError_t device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_facts_mu);
  auto it = g_cus.find(dev);
  if (it == g_cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return hipErrorUnknown;
    it = g_cus.emplace(dev, n).first;
  }
  *cus = it->second;
  return hipSuccess;
}

hipError_t blocks_per_cu(const void* fn, int block, int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_facts_mu);
  const auto key = std::make_tuple(fn, dev, block);
  auto it = g_per_cu.find(key);
  if (it == g_per_cu.end()) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, block, 0) != hipSuccess || v < 1) v = 1;
    it = g_per_cu.emplace(key, v).first;
  }
  *n = it->second;
  return hipSuccess;
}

hipError_t open_dynamic_lds(const void* fn, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_facts_mu);
  int& have = g_lds[std::make_pair(fn, dev)];
  if (have >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  have = bytes;
  return hipSuccess;
}

// CRC-32 (IEEE 802.3), table driven.
uint32_t crc32(const void* data, size_t len) {
  struct Table {
    uint32_t t[256];
    Table() {
      for (uint32_t i = 0; i < 256; i++) {
        uint32_t c = i;
        for (int k = 0; k < 8; k++) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
        t[i] = c;
      }
    }
  };
  static const Table table;  // built once; C++ makes the first use thread-safe
  const uint8_t* p = static_cast<const uint8_t*>(data);
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < len; i++) c = table.t[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
  return c ^ 0xFFFFFFFFu;
}

KLut klut_from(const uint8_t lut[16], int n_codes) {
  KLut k;
  for (int q = 0; q < 4; q++)
    k.t[q] = lut[4 * q] | (lut[4 * q + 1] << 8) | (lut[4 * q + 2] << 16) | ((uint32_t)lut[4 * q + 3] << 24);
  k.base4 = lut[0] * 0x01010101u;
  k.contiguous = n_codes > 0;
  for (int c = 0; c < n_codes; c++)
    if (lut[c] != lut[0] + c) k.contiguous = 0;
  // codes >= n_codes never occur, so lut[0] + c only has to be right below n_codes;
  // the byte-wise add must not carry: lut[0] + 15 <= 255
  if (lut[0] > 240) k.contiguous = 0;
  return k;
}

KLut klut_of(const lbf_desc& d) { return klut_from(d.lut, d.n_codes); }

static bool shape_ok(uint64_t rows, uint64_t cols) {
  if (cols != 0 && rows > UINT64_MAX / cols) return false;
  return rows * cols < (uint64_t(1) << 32);
}

static int check(const lbf_desc* d) {
  if (!d) return LBF_E_INVAL;
  if (d->magic != LBF_MAGIC || d->version != LBF_VERSION || d->tile_log2 != LBF_TILE_LOG2) return LBF_E_DESC;
  if (crc32(d, offsetof(lbf_desc, desc_crc)) != d->desc_crc) return LBF_E_DESC;
  if (!shape_ok(d->rows, d->cols)) return LBF_E_DESC;
  const Layout L = layout_of(d->rows, d->cols, d->n_esc);
  if (d->n_esc > L.n) return LBF_E_DESC;
  if (d->off_raw != L.off_raw || d->off_nib != L.off_nib || d->off_idx != L.off_idx || d->off_esc != L.off_esc ||
      d->blob_bytes != L.blob_bytes)
    return LBF_E_DESC;
  if (d->n_codes > 15) return LBF_E_DESC;
  for (int c = 1; c < d->n_codes; c++)
    if (d->lut[c] <= d->lut[c - 1]) return LBF_E_DESC;
  for (int c = d->n_codes; c < 16; c++)
    if (d->lut[c] != 0) return LBF_E_DESC;
  if (d->reserved[0] | d->reserved[1] | d->reserved[2]) return LBF_E_DESC;
  // fewer than 15 coded exponents means every exponent present got a code
  if (d->n_codes < 15 && d->n_esc != 0) return LBF_E_DESC;
  if (L.n > 0 && d->n_codes == 0) return LBF_E_DESC;
  return LBF_OK;
}

// Code table rules shared by both descriptors.
static bool table_ok(const uint8_t lut[16], int n_codes, uint64_t n, uint64_t n_esc) {
  if (n_codes > 15) return false;
  for (int c = 1; c < n_codes; c++)
    if (lut[c] <= lut[c - 1]) return false;
  for (int c = n_codes; c < 16; c++)
    if (lut[c] != 0) return false;
  // fewer than 15 coded exponents means every exponent present got a code
  if (n_codes < 15 && n_esc != 0) return false;
  if (n > 0 && n_codes == 0) return false;
  return true;
}

static int hcheck(const lbf_hdesc* h) {
  if (!h) return LBF_E_INVAL;
  if (h->magic != LBF_HMAGIC || h->version != LBF_HVERSION || h->tile_log2 != LBF_TILE_LOG2) return LBF_E_DESC;
  if (crc32(h, offsetof(lbf_hdesc, desc_crc)) != h->desc_crc) return LBF_E_DESC;
  if (!shape_ok(h->rows, h->cols)) return LBF_E_DESC;
  const HLayout L = hlayout_of(h->rows, h->cols, h->n_esc, h->stream_words);
  // every tile holds at least one code bit, so at least one word
  if (h->n_esc > L.n || h->stream_words > L.n_tiles * LBF_HMAX_TILE_WORDS || h->stream_words < L.n_tiles)
    return LBF_E_DESC;
  if (h->off_raw != L.off_raw || h->off_bits != L.off_bits || h->off_woff != L.off_woff ||
      h->off_idx != L.off_idx || h->off_esc != L.off_esc || h->blob_bytes != L.blob_bytes)
    return LBF_E_DESC;
  if (!table_ok(h->lut, h->n_codes, L.n, h->n_esc) || h->reserved[0] | h->reserved[1]) return LBF_E_DESC;
  // lengths: exactly the codes that occur (the table's, and 15 when there are
  // escapes) have one, forming a complete prefix code (one code: length 1)
  uint32_t kraft = 0, used = 0, max_len = 0;
  for (int c = 0; c < 16; c++) {
    const bool occurs = c < h->n_codes || (c == 15 && h->n_esc > 0);
    if (h->len[c] > 15 || (h->len[c] != 0) != occurs) return LBF_E_DESC;
    if (!h->len[c]) continue;
    used++;
    kraft += 1u << (15 - h->len[c]);
    max_len = std::max<uint32_t>(max_len, h->len[c]);
  }
  if (h->max_len != max_len) return LBF_E_DESC;
  if (used >= 2 && kraft != (1u << 15)) return LBF_E_DESC;
  if (used == 1 && max_len != 1) return LBF_E_DESC;
  if (used == 0 && (L.n != 0 || h->stream_words != 0)) return LBF_E_DESC;
  return LBF_OK;
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Choose the coded exponents from the histogram: sort by count descending,
// ties to the smaller exponent, keep the first 15 present ones, then hand
// codes out in ascending exponent order.
static void fill_desc(const uint32_t hist[256], uint64_t rows, uint64_t cols, lbf_desc* d) {
  std::vector<int> order;
  for (int e = 0; e < 256; e++)
    if (hist[e]) order.push_back(e);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return hist[a] > hist[b]; });
  if (order.size() > 15) order.resize(15);
  std::sort(order.begin(), order.end());
  uint64_t coded = 0;
  for (int e : order) coded += hist[e];

  std::memset(d, 0, sizeof(*d));
  d->magic = LBF_MAGIC;
  d->version = LBF_VERSION;
  d->tile_log2 = LBF_TILE_LOG2;
  d->rows = rows;
  d->cols = cols;
  d->n_esc = rows * cols - coded;
  const Layout L = layout_of(rows, cols, d->n_esc);
  d->off_raw = L.off_raw;
  d->off_nib = L.off_nib;
  d->off_idx = L.off_idx;
  d->off_esc = L.off_esc;
  d->blob_bytes = L.blob_bytes;
  for (size_t c = 0; c < order.size(); c++) d->lut[c] = (uint8_t)order[c];
  d->n_codes = (uint8_t)order.size();
  d->desc_crc = crc32(d, offsetof(lbf_desc, desc_crc));
}

// Per-group kernel records for the product calls; checks every group.
static int build_groups(const lbf_desc* descs, const void* const* d_blobs, int n_groups, const void* const* d_x,
                        void* const* d_y, std::vector<GroupArg>& out) {
  if (!descs || !d_blobs || !d_x || !d_y || n_groups < 1) return LBF_E_INVAL;
  out.resize((size_t)n_groups);
  for (int g = 0; g < n_groups; g++) {
    const lbf_desc& d = descs[g];
    const int rc = check(&d);
    if (rc) return rc;
    if (!d_blobs[g] || !d_x[g] || !d_y[g]) return LBF_E_INVAL;
    if (!aligned(d_blobs[g], 256) || !aligned(d_x[g], 16) || !aligned(d_y[g], 4)) return LBF_E_ALIGN;
    if (d.rows == 0 || d.cols == 0 || d.cols % LBF_TILE != 0) return LBF_E_SHAPE;
    GroupArg& G = out[(size_t)g];
    G.blob = static_cast<const uint8_t*>(d_blobs[g]);
    G.x = static_cast<const uint16_t*>(d_x[g]);
    G.y = d_y[g];
    G.rows = (uint32_t)d.rows;
    G.tiles = (uint32_t)(d.cols / LBF_TILE);
    G.n_esc = (uint32_t)d.n_esc;
    G.aux = klut_of(d).contiguous ? kAuxContig : 0u;
  }
  return LBF_OK;
}

}  // namespace lbf

using namespace lbf;

extern "C" {

const char* lbf_strerror(int status) {
  switch (status) {
    case LBF_OK: return "ok";
    case LBF_E_INVAL: return "invalid argument";
    case LBF_E_SHAPE: return "unsupported or mismatched shape";
    case LBF_E_ALIGN: return "misaligned device pointer";
    case LBF_E_DESC: return "descriptor failed validation";
    case LBF_E_CAPACITY: return "buffer too small";
    case LBF_E_HIP: return "HIP runtime error";
    case LBF_E_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

uint64_t lbf_encode_work_bytes(uint64_t rows, uint64_t cols) {
  if (!shape_ok(rows, cols)) return 0;
  const Layout L = layout_of(rows, cols, 0);
  return kWorkHistBytes + ((4 * L.n_tiles + 255) & ~uint64_t(255));
}

int lbf_desc_check(const lbf_desc* desc) { return check(desc); }

static int encode(const void* d_w, uint64_t rows, uint64_t cols, void* d_work, uint64_t work_bytes, void* d_blob,
                  uint64_t blob_cap, lbf_desc* desc, hipStream_t s) {
  if (!desc || !d_work) return LBF_E_INVAL;
  if (!shape_ok(rows, cols)) return LBF_E_SHAPE;
  const uint64_t n = rows * cols;
  if (n && !d_w) return LBF_E_INVAL;
  if (!aligned(d_w, 16) || !aligned(d_work, 256)) return LBF_E_ALIGN;
  if (work_bytes < lbf_encode_work_bytes(rows, cols)) return LBF_E_CAPACITY;
  uint32_t* hist = static_cast<uint32_t*>(d_work);
  uint32_t* tile_cnt = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(d_work) + kWorkHistBytes);
  if (!d_blob) {  // phase 1
    uint32_t h[256];
    if (n) {
      if (launch_hist(static_cast<const uint16_t*>(d_w), n, hist, s) != hipSuccess) return LBF_E_HIP;
      if (hipMemcpyAsync(h, hist, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return LBF_E_HIP;
      if (hipStreamSynchronize(s) != hipSuccess) return LBF_E_HIP;
    } else {
      std::memset(h, 0, sizeof h);
    }
    uint64_t total = 0;
    for (int e = 0; e < 256; e++) total += h[e];
    if (total != n) return LBF_E_HIP;  // the histogram must account for every weight
    fill_desc(h, rows, cols, desc);
    return LBF_OK;
  }
  // phase 2
  const int rc = check(desc);
  if (rc) return rc;
  if (desc->rows != rows || desc->cols != cols) return LBF_E_SHAPE;
  if (!aligned(d_blob, 256)) return LBF_E_ALIGN;
  if (blob_cap < desc->blob_bytes) return LBF_E_CAPACITY;
  if (launch_pack(static_cast<const uint16_t*>(d_w), *desc, static_cast<uint8_t*>(d_blob), tile_cnt, s) != hipSuccess)
    return LBF_E_HIP;
  return LBF_OK;
}

int lbf_encode(const void* d_w, uint64_t rows, uint64_t cols, void* d_work, uint64_t work_bytes, void* d_blob,
               uint64_t blob_cap, lbf_desc* desc, hipStream_t s) {
  return encode(d_w, rows, cols, d_work, work_bytes, d_blob, blob_cap, desc, s);
}

int lbf_encode_noalloc(const void* d_w, uint64_t rows, uint64_t cols, void* d_blob, uint64_t blob_cap, lbf_desc* desc,
                       hipStream_t s) {
  if (!desc) return LBF_E_INVAL;
  if (!shape_ok(rows, cols)) return LBF_E_SHAPE;
  if (lbf_encode_work_bytes(rows, cols) > LBF_NOALLOC_SCRATCH_BYTES) return LBF_E_CAPACITY;
  void* work = nullptr;
  if (encode_scratch(&work) != hipSuccess) return LBF_E_HIP;
  return encode(d_w, rows, cols, work, LBF_NOALLOC_SCRATCH_BYTES, d_blob, blob_cap, desc, s);
}

int lbf_hdesc_check(const lbf_hdesc* hdesc) { return hcheck(hdesc); }

static uint64_t up256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

uint64_t lbf_hencode_work_bytes(const lbf_desc* desc) {
  if (check(desc)) return 0;
  const Layout L = layout_of(desc->rows, desc->cols, desc->n_esc);
  return 256 + up256(4 * L.n_tiles) + up256(4 * (L.n_tiles + 1));
}

int lbf_hencode(const lbf_desc* desc, const void* d_blob, void* d_work, uint64_t work_bytes, void* d_hblob,
                uint64_t hblob_cap, lbf_hdesc* hdesc, hipStream_t s) {
  const int rc = check(desc);
  if (rc) return rc;
  if (!hdesc || !d_work || !d_blob) return LBF_E_INVAL;
  if (!aligned(d_blob, 256) || !aligned(d_work, 256)) return LBF_E_ALIGN;
  if (work_bytes < lbf_hencode_work_bytes(desc)) return LBF_E_CAPACITY;
  const Layout V = layout_of(desc->rows, desc->cols, desc->n_esc);
  const uint8_t* blob = static_cast<const uint8_t*>(d_blob);
  uint8_t* work = static_cast<uint8_t*>(d_work);
  uint32_t* counts = reinterpret_cast<uint32_t*>(work);
  uint32_t* words = reinterpret_cast<uint32_t*>(work + 256);
  uint32_t* woff = reinterpret_cast<uint32_t*>(work + 256 + up256(4 * V.n_tiles));
  if (!d_hblob) {  // phase 1
    uint32_t cnt[16] = {0};
    if (V.n) {
      if (launch_hcount(*desc, blob, counts, s) != hipSuccess) return LBF_E_HIP;
      if (hipMemcpyAsync(cnt, counts, sizeof cnt, hipMemcpyDeviceToHost, s) != hipSuccess) return LBF_E_HIP;
      if (hipStreamSynchronize(s) != hipSuccess) return LBF_E_HIP;
    }
    uint64_t total = 0, c64[16];
    for (int c = 0; c < 16; c++) total += c64[c] = cnt[c];
    if (total != V.n) return LBF_E_HIP;  // the counts must account for every weight
    if (cnt[15] != desc->n_esc) return LBF_E_DESC;
    for (int c = desc->n_codes; c < 15; c++)
      if (cnt[c]) return LBF_E_DESC;  // an unused code: not a valid v1 blob
    uint8_t len[16];
    huffman_lengths(c64, len);
    uint32_t stream_words = 0;
    if (launch_hwoff(*desc, blob, len, words, woff, s) != hipSuccess) return LBF_E_HIP;
    if (hipMemcpyAsync(&stream_words, woff + V.n_tiles, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return LBF_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return LBF_E_HIP;
    const HLayout H = hlayout_of(desc->rows, desc->cols, desc->n_esc, stream_words);
    std::memset(hdesc, 0, sizeof(*hdesc));
    hdesc->magic = LBF_HMAGIC;
    hdesc->version = LBF_HVERSION;
    hdesc->tile_log2 = LBF_TILE_LOG2;
    hdesc->rows = desc->rows;
    hdesc->cols = desc->cols;
    hdesc->n_esc = desc->n_esc;
    hdesc->off_raw = H.off_raw;
    hdesc->off_bits = H.off_bits;
    hdesc->off_woff = H.off_woff;
    hdesc->off_idx = H.off_idx;
    hdesc->off_esc = H.off_esc;
    hdesc->blob_bytes = H.blob_bytes;
    hdesc->stream_words = stream_words;
    std::memcpy(hdesc->lut, desc->lut, 16);
    hdesc->n_codes = desc->n_codes;
    for (int c = 0; c < 16; c++) {
      hdesc->len[c] = len[c];
      hdesc->max_len = std::max(hdesc->max_len, len[c]);
    }
    hdesc->desc_crc = crc32(hdesc, offsetof(lbf_hdesc, desc_crc));
    return LBF_OK;
  }
  // phase 2
  const int hrc = hcheck(hdesc);
  if (hrc) return hrc;
  if (hdesc->rows != desc->rows || hdesc->cols != desc->cols || hdesc->n_esc != desc->n_esc ||
      hdesc->n_codes != desc->n_codes || std::memcmp(hdesc->lut, desc->lut, 16) != 0)
    return LBF_E_DESC;
  if (!aligned(d_hblob, 256)) return LBF_E_ALIGN;
  if (hblob_cap < hdesc->blob_bytes) return LBF_E_CAPACITY;
  const HLayout H = hlayout_of(hdesc->rows, hdesc->cols, hdesc->n_esc, hdesc->stream_words);
  uint8_t* out = static_cast<uint8_t*>(d_hblob);
  uint32_t* out_woff = reinterpret_cast<uint32_t*>(out + H.off_woff);
  if (launch_hfill(*hdesc, out, s) != hipSuccess) return LBF_E_HIP;
  if (hipMemcpyAsync(out + H.off_raw, blob + V.off_raw, V.n_tiles * LBF_TILE, hipMemcpyDeviceToDevice, s) !=
          hipSuccess ||
      hipMemcpyAsync(out + H.off_idx, blob + V.off_idx, 4 * (V.n_tiles + 1), hipMemcpyDeviceToDevice, s) !=
          hipSuccess)
    return LBF_E_HIP;
  if (V.n_esc &&
      hipMemcpyAsync(out + H.off_esc, blob + V.off_esc, V.n_esc, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LBF_E_HIP;
  if (launch_hwoff(*desc, blob, hdesc->len, words, out_woff, s) != hipSuccess) return LBF_E_HIP;
  if (launch_hpack(*desc, blob, hcode_of(hdesc->len), out_woff, reinterpret_cast<uint32_t*>(out + H.off_bits),
                   hdesc->stream_words, s) != hipSuccess)
    return LBF_E_HIP;
  return LBF_OK;
}

int lbf_hdecode(const lbf_hdesc* hdesc, const void* d_hblob, void* d_w_out, hipStream_t s) {
  const int rc = hcheck(hdesc);
  if (rc) return rc;
  if (hdesc->rows * hdesc->cols == 0) return LBF_OK;
  if (!d_hblob || !d_w_out) return LBF_E_INVAL;
  if (!aligned(d_hblob, 256) || !aligned(d_w_out, 16)) return LBF_E_ALIGN;
  if (launch_hdecode(*hdesc, hcode_of(hdesc->len), static_cast<const uint8_t*>(d_hblob),
                     static_cast<uint16_t*>(d_w_out), s) != hipSuccess)
    return LBF_E_HIP;
  return LBF_OK;
}

int lbf_decode(const lbf_desc* desc, const void* d_blob, void* d_w_out, hipStream_t s) {
  const int rc = check(desc);
  if (rc) return rc;
  const uint64_t n = desc->rows * desc->cols;
  if (n == 0) return LBF_OK;
  if (!d_blob || !d_w_out) return LBF_E_INVAL;
  if (!aligned(d_blob, 256) || !aligned(d_w_out, 16)) return LBF_E_ALIGN;
  if (launch_decode(*desc, static_cast<const uint8_t*>(d_blob), static_cast<uint16_t*>(d_w_out), s) != hipSuccess)
    return LBF_E_HIP;
  return LBF_OK;
}

int lbf_verify(const lbf_desc* desc, const void* d_blob, uint32_t* d_flags, hipStream_t s) {
  const int rc = check(desc);
  if (rc) return rc;
  if (!d_blob || !d_flags) return LBF_E_INVAL;
  if (!aligned(d_blob, 256) || !aligned(d_flags, 4)) return LBF_E_ALIGN;
  if (launch_verify(*desc, static_cast<const uint8_t*>(d_blob), d_flags, s) != hipSuccess) return LBF_E_HIP;
  return LBF_OK;
}

int lbf_crc32(const void* d_data, uint64_t n, uint32_t* d_crc, hipStream_t s) {
  if ((n && !d_data) || !d_crc) return LBF_E_INVAL;
  if (!aligned(d_data, 16) || !aligned(d_crc, 4)) return LBF_E_ALIGN;
  if (launch_crc32(static_cast<const uint8_t*>(d_data), n, d_crc, s) != hipSuccess) return LBF_E_HIP;
  return LBF_OK;
}

static int product(bool mfma, const lbf_desc* descs, const void* const* d_blobs, int n_groups,
                   const void* const* d_x, int batch, void* const* d_y, int y_dtype, hipStream_t s) {
  if (y_dtype != LBF_F32 && y_dtype != LBF_BF16) return LBF_E_INVAL;
  if (mfma ? (batch < 9 || batch > 256) : (batch < 1 || batch > 8)) return LBF_E_INVAL;
  std::vector<GroupArg> groups;
  const int rc = build_groups(descs, d_blobs, n_groups, d_x, d_y, groups);
  if (rc) return rc;
  if (mfma)
    for (const GroupArg& G : groups)
      if (G.tiles > kGemmMaxTiles) return LBF_E_UNSUPPORTED;
  for (int g0 = 0; g0 < n_groups; g0 += LBF_MAX_GROUPS) {
    const int cnt = std::min(LBF_MAX_GROUPS, n_groups - g0);
    const hipError_t e = mfma ? launch_gemm(groups.data() + g0, cnt, batch, y_dtype, s)
                              : launch_gemv(groups.data() + g0, cnt, batch, y_dtype, s);
    if (e != hipSuccess) return LBF_E_HIP;
  }
  return LBF_OK;
}

int lbf_gemv_swiglu(const lbf_desc* gate_desc, const void* d_gate_blob, const lbf_desc* up_desc,
                    const void* d_up_blob, const void* d_x, int batch, void* d_h, int h_dtype, hipStream_t s) {
  if (h_dtype != LBF_F32 && h_dtype != LBF_BF16) return LBF_E_INVAL;
  if (batch < 1 || batch > 8 || !gate_desc || !up_desc) return LBF_E_INVAL;
  const lbf_desc descs[2] = {*gate_desc, *up_desc};
  const void* blobs[2] = {d_gate_blob, d_up_blob};
  const void* xs[2] = {d_x, d_x};
  void* hs[2] = {d_h, d_h};
  std::vector<GroupArg> groups;
  const int rc = build_groups(descs, blobs, 2, xs, hs, groups);
  if (rc) return rc;
  if (gate_desc->rows != up_desc->rows || gate_desc->cols != up_desc->cols) return LBF_E_SHAPE;
  if ((uint64_t)batch * gate_desc->cols * 2 > kGatedMaxXBytes) return LBF_E_UNSUPPORTED;
  if (launch_gemv_gated(groups[0], groups[1], batch, d_h, h_dtype, s) != hipSuccess) return LBF_E_HIP;
  return LBF_OK;
}

int lbf_gemv(const lbf_desc* descs, const void* const* d_blobs, int n_groups, const void* const* d_x, int batch,
             void* const* d_y, int y_dtype, hipStream_t s) {
  return product(false, descs, d_blobs, n_groups, d_x, batch, d_y, y_dtype, s);
}

int lbf_gemm(const lbf_desc* descs, const void* const* d_blobs, int n_groups, const void* const* d_x, int batch,
             void* const* d_y, int y_dtype, hipStream_t s) {
  return product(true, descs, d_blobs, n_groups, d_x, batch, d_y, y_dtype, s);
}

}  // extern "C"
