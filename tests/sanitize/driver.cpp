// CPU sanitizer driver: the oracle (oracle/lbf_oracle.c) and the library's
// host-side logic (descriptor and argument checks, group records, the
// K15H host helpers), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer and driven over valid, corrupted, truncated and random inputs.
// Device calls go to stand-ins that report no device (hip_stubs.cpp), so
// every library entry point runs its checks and stops at its first device
// step.  A sanitizer report or a failed expectation ends the run with a
// non-zero status.  Test infrastructure only.
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lbf.h"
#include "lbf_internal.h"

extern "C" {
uint32_t lbfo_crc32(const uint8_t* data, uint64_t len);
int lbfo_plan(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t lut[16], uint8_t* n_codes, uint64_t* n_esc,
              uint64_t* blob_bytes);
int lbfo_encode(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* blob, uint64_t blob_cap);
int lbfo_read_header(const uint8_t* blob, uint64_t blob_len, uint64_t* rows, uint64_t* cols, uint64_t* n_esc,
                     uint8_t lut[16], uint8_t* n_codes);
int lbfo_decode(const uint8_t* blob, uint64_t blob_len, uint16_t* out, uint64_t out_len);
unsigned lbfo_verify(const uint8_t* blob, uint64_t blob_len, const uint8_t desc96[96]);
void lbfo_matvec(const uint16_t* W, uint64_t rows, uint64_t cols, const uint16_t* x, uint64_t batch, double* y,
                 double* a);
double lbfo_entropy16(const uint16_t* w, uint64_t n);
double lbfo_entropy_exponent(const uint16_t* w, uint64_t n);
void lbfo_huffman_lengths(const uint64_t count[16], uint8_t len[16]);
void lbfo_canonical_codes(const uint8_t len[16], uint16_t code[16]);
int lbfo_hplan(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t code_count[16], uint8_t len[16],
               uint64_t* stream_words, uint64_t* blob_bytes);
int lbfo_hencode(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* blob, uint64_t blob_cap);
int lbfo_hdecode(const uint8_t* blob, uint64_t blob_len, uint16_t* out, uint64_t out_len);
void lbfo_swiglu(const uint16_t* G, const uint16_t* U, uint64_t rows, uint64_t cols, const uint16_t* x,
                 uint64_t batch, double* h, double* g, double* u, double* ag, double* au);
}

#define EXPECT(c)                                                         \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Weights shaped like a trained tensor: random sign and mantissa, exponents
// around 2^-6 with a few far outliers (escapes), some zeros.
static std::vector<uint16_t> weights(uint64_t n, int kind) {
  std::vector<uint16_t> w(n);
  for (uint64_t i = 0; i < n; i++) {
    const uint64_t r = next_u64();
    if (kind == 1) {
      w[i] = (uint16_t)i;  // every bit pattern in turn
      continue;
    }
    uint32_t e = 121u + (uint32_t)(r % 7u);
    if ((r >> 8) % 1000u < 3u) e = 127u + (uint32_t)((r >> 20) % 8u);  // outliers
    if ((r >> 32) % 4096u == 0) e = 0;                                   // zeros and denormals
    w[i] = (uint16_t)(((r >> 40) & 1u) << 15 | e << 7 | ((r >> 48) & 0x7Fu));
  }
  return w;
}

static void oracle_round_trips(uint64_t rows, uint64_t cols, int kind, std::vector<std::vector<uint8_t>>& blobs,
                               std::vector<std::vector<uint8_t>>& hblobs) {
  const uint64_t n = rows * cols;
  const std::vector<uint16_t> w = weights(n, kind);
  uint8_t lut[16], n_codes;
  uint64_t n_esc = 0, bytes = 0;
  EXPECT(lbfo_plan(w.data(), rows, cols, lut, &n_codes, &n_esc, &bytes) == 0);
  std::vector<uint8_t> blob(bytes);  // exactly the blob: any write past it is caught
  EXPECT(lbfo_encode(w.data(), rows, cols, blob.data(), blob.size()) == 0);
  std::vector<uint16_t> out(n);
  EXPECT(lbfo_decode(blob.data(), blob.size(), out.data(), out.size()) == 0);
  EXPECT(out == w);
  EXPECT(lbfo_verify(blob.data(), blob.size(), blob.data()) == 0);
  EXPECT(lbfo_encode(w.data(), rows, cols, blob.data(), blob.size() - 1) != 0);  // too small: refused
  // truncated and corrupted blobs: any status, no access outside the buffers
  for (uint64_t len : {(uint64_t)0, (uint64_t)95, (uint64_t)255, (uint64_t)256, blob.size() / 2, blob.size() - 1}) {
    std::vector<uint8_t> t(blob.begin(), blob.begin() + (std::ptrdiff_t)len);
    (void)lbfo_decode(t.data(), t.size(), out.data(), out.size());
    (void)lbfo_verify(t.data(), t.size(), blob.data());
  }
  for (int k = 0; k < 300; k++) {
    std::vector<uint8_t> c = blob;
    const uint64_t at = k < 100 ? next_u64() % 96u : next_u64() % c.size();
    c[at] ^= (uint8_t)(1u << (next_u64() % 8u));
    if (k % 3 == 0 && c.size() > 256) c[256 + next_u64() % (c.size() - 256)] = (uint8_t)next_u64();
    (void)lbfo_decode(c.data(), c.size(), out.data(), out.size());
    (void)lbfo_verify(c.data(), c.size(), blob.data());
    uint64_t r, cc, e;
    uint8_t l[16], nc;
    (void)lbfo_read_header(c.data(), c.size(), &r, &cc, &e, l, &nc);
  }
  // K15H
  uint64_t counts[16], words = 0, hbytes = 0;
  uint8_t len[16];
  EXPECT(lbfo_hplan(w.data(), rows, cols, counts, len, &words, &hbytes) == 0);
  std::vector<uint8_t> hblob(hbytes);
  EXPECT(lbfo_hencode(w.data(), rows, cols, hblob.data(), hblob.size()) == 0);
  std::fill(out.begin(), out.end(), (uint16_t)0);
  EXPECT(lbfo_hdecode(hblob.data(), hblob.size(), out.data(), out.size()) == 0);
  EXPECT(out == w);
  for (int k = 0; k < 200; k++) {
    std::vector<uint8_t> c = hblob;
    c[next_u64() % c.size()] ^= (uint8_t)(1u << (next_u64() % 8u));
    (void)lbfo_hdecode(c.data(), c.size(), out.data(), out.size());
  }
  // products and statistics over the same tensor
  if (kind == 0 && rows <= 64 && cols <= 4096) {
    const uint64_t batch = 2;
    const std::vector<uint16_t> x = weights(batch * cols, 0);
    std::vector<double> y(batch * rows), a(batch * rows), h(batch * rows), g(batch * rows), u(batch * rows),
        ag(batch * rows), au(batch * rows);
    lbfo_matvec(w.data(), rows, cols, x.data(), batch, y.data(), a.data());
    lbfo_swiglu(w.data(), w.data(), rows, cols, x.data(), batch, h.data(), g.data(), u.data(), ag.data(), au.data());
  }
  (void)lbfo_entropy16(w.data(), n);
  (void)lbfo_entropy_exponent(w.data(), n);
  blobs.push_back(blob);
  hblobs.push_back(hblob);
}

// The oracle's and the library's Huffman code lengths (written apart: the
// library's host helper, lbf_host.cpp) agree on random counts, and both
// builders, with the library's canonical codes and layouts, stay clean.
static void huffman_cases() {
  for (int k = 0; k < 2000; k++) {
    uint64_t count[16];
    for (int s = 0; s < 16; s++) {
      const uint64_t r = next_u64();
      count[s] = r % 4u == 0 ? 0 : (r >> 8) % (k % 2 ? 1000u : 1u << 30);
    }
    uint8_t len[16], len_lib[16];
    uint16_t code[16];
    lbfo_huffman_lengths(count, len);
    lbfo_canonical_codes(len, code);
    lbf::huffman_lengths(count, len_lib);
    EXPECT(std::memcmp(len, len_lib, 16) == 0);
    (void)lbf::hcode_of(len_lib);
    (void)lbf::hlayout_of(next_u64() >> 34, next_u64() >> 34, next_u64() >> 34, next_u64() >> 34);
    (void)lbf::layout_of(next_u64() >> 34, next_u64() >> 34, next_u64() >> 34);
  }
}

static void library_checks(const std::vector<std::vector<uint8_t>>& blobs,
                           const std::vector<std::vector<uint8_t>>& hblobs) {
  for (int st = -40; st <= 40; st++) EXPECT(lbf_strerror(st) != nullptr);
  for (int k = 0; k < 1000; k++) (void)lbf_encode_work_bytes(next_u64() >> (next_u64() % 64u), next_u64() >> (next_u64() % 64u));
  void* const dev = reinterpret_cast<void*>(uintptr_t(1) << 20);  // a device address: never dereferenced on the host
  void* const odd = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);
  for (const auto& b : blobs) {
    lbf_desc d;
    std::memcpy(&d, b.data(), sizeof d);
    EXPECT(lbf_desc_check(&d) == LBF_OK);
    for (int bit = 0; bit < 96 * 8; bit++) {  // every single-bit change is refused
      lbf_desc c = d;
      reinterpret_cast<uint8_t*>(&c)[bit / 8] ^= (uint8_t)(1u << (bit % 8));
      EXPECT(lbf_desc_check(&c) == LBF_E_DESC);
      (void)lbf_decode(&c, dev, dev, nullptr);
    }
    // valid descriptor: every entry point runs its checks, then meets no device
    const lbf_desc ds[2] = {d, d};
    const void* bl[2] = {dev, dev};
    const void* xs[2] = {dev, dev};
    void* ys[2] = {dev, dev};
    (void)lbf_decode(&d, dev, dev, nullptr);
    (void)lbf_decode(&d, odd, dev, nullptr);
    (void)lbf_decode(&d, nullptr, dev, nullptr);
    (void)lbf_verify(&d, dev, static_cast<uint32_t*>(dev), nullptr);
    (void)lbf_hencode_work_bytes(&d);
    lbf_hdesc hd;
    (void)lbf_hencode(&d, dev, dev, 1u << 20, dev, 1u << 30, &hd, nullptr);
    for (int batch : {-1, 0, 1, 4, 8, 9, 16, 64, 65, 256, 257}) {
      for (int dt : {(int)LBF_F32, (int)LBF_BF16, 7}) {
        for (int ng : {-1, 0, 1, 2}) {
          (void)lbf_gemv(ds, bl, ng, xs, batch, ys, dt, nullptr);
          (void)lbf_gemm(ds, bl, ng, xs, batch, ys, dt, nullptr);
        }
      }
      (void)lbf_gemv_swiglu(&d, dev, &d, dev, dev, batch, dev, LBF_BF16, nullptr);
    }
    const void* bad_bl[2] = {odd, dev};
    (void)lbf_gemv(ds, bad_bl, 2, xs, 1, ys, LBF_F32, nullptr);
    (void)lbf_gemv(ds, nullptr, 2, xs, 1, ys, LBF_F32, nullptr);
    (void)lbf_gemv(nullptr, bl, 2, xs, 1, ys, LBF_F32, nullptr);
    (void)lbf_gemm(ds, bl, 2, nullptr, 16, ys, LBF_F32, nullptr);
  }
  for (const auto& hb : hblobs) {
    lbf_hdesc h;
    std::memcpy(&h, hb.data(), sizeof h);
    EXPECT(lbf_hdesc_check(&h) == LBF_OK);
    for (int bit = 0; bit < (int)sizeof h * 8; bit++) {
      lbf_hdesc c = h;
      reinterpret_cast<uint8_t*>(&c)[bit / 8] ^= (uint8_t)(1u << (bit % 8));
      EXPECT(lbf_hdesc_check(&c) != LBF_OK);
      (void)lbf_hdecode(&c, dev, dev, nullptr);
    }
    (void)lbf_hdecode(&h, dev, dev, nullptr);
  }
  // random descriptors of both kinds
  for (int k = 0; k < 20000; k++) {
    uint8_t raw[sizeof(lbf_hdesc)];
    for (auto& v : raw) v = (uint8_t)next_u64();
    if (k % 2) {  // plausible magic and version, so the deeper checks run
      const uint32_t m = k % 4 == 1 ? LBF_MAGIC : LBF_HMAGIC;
      std::memcpy(raw, &m, 4);
      raw[4] = 1;
      raw[5] = 0;
      raw[6] = 10;
      raw[7] = 0;
    }
    lbf_desc d;
    lbf_hdesc h;
    std::memcpy(&d, raw, sizeof d);
    std::memcpy(&h, raw, sizeof h);
    (void)lbf_desc_check(&d);
    (void)lbf_hdesc_check(&h);
    (void)lbf_decode(&d, dev, dev, nullptr);
    (void)lbf_hdecode(&h, dev, dev, nullptr);
  }
  // encode arguments: shapes past the limits, missing buffers, every size
  lbf_desc out;
  for (int k = 0; k < 2000; k++) {
    const uint64_t rows = next_u64() >> (next_u64() % 64u), cols = next_u64() >> (next_u64() % 64u);
    (void)lbf_encode(dev, rows, cols, dev, next_u64() >> (next_u64() % 64u), dev, next_u64() >> (next_u64() % 64u),
                     &out, nullptr);
    (void)lbf_encode_noalloc(dev, rows, cols, dev, next_u64() >> (next_u64() % 64u), &out, nullptr);
  }
  (void)lbf_encode(nullptr, 3, 5, dev, 1u << 20, dev, 1u << 20, &out, nullptr);
  (void)lbf_encode(dev, 3, 5, dev, 1u << 20, dev, 1u << 20, nullptr, nullptr);
  (void)lbf_crc32(dev, 1000, static_cast<uint32_t*>(dev), nullptr);
  (void)lbf_crc32(nullptr, 0, static_cast<uint32_t*>(dev), nullptr);
}

int main() {
  std::vector<std::vector<uint8_t>> blobs, hblobs;
  const struct {
    uint64_t rows, cols;
    int kind;
  } shapes[] = {{3, 5, 0}, {1, 1024, 0}, {2, 1500, 0}, {7, 2048, 0}, {33, 300, 0}, {64, 1024, 1}, {5, 4096, 0},
                {1, 1, 0}, {16, 1024, 1}};
  for (const auto& s : shapes) oracle_round_trips(s.rows, s.cols, s.kind, blobs, hblobs);
  huffman_cases();
  library_checks(blobs, hblobs);
  std::printf("sanitizer driver: %zu tensors, oracle and library host checks clean\n", blobs.size());
  return 0;
}
