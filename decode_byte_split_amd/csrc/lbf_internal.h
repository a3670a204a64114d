// lbf_internal.h — host-side declarations shared by the library's sources.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "lbf.h"

namespace lbf {

// Byte layout of a format-v1 blob for a [rows, cols] tensor with n_esc escapes.
struct Layout {
  uint64_t n, n_tiles, n_esc;
  uint64_t off_raw, off_nib, off_idx, off_esc, blob_bytes;
};
Layout layout_of(uint64_t rows, uint64_t cols, uint64_t n_esc);

uint32_t crc32(const void* data, size_t len);

// Code table as handed to kernels.
struct KLut {
  uint32_t t[4];   // lut bytes, little-endian words
  uint32_t base4;  // lut[0] * 0x01010101
  int contiguous;  // lut[c] == lut[0] + c for every c < n_codes
};
KLut klut_of(const lbf_desc& d);
KLut klut_from(const uint8_t lut[16], int n_codes);

// Launchers (defined next to their kernels).  All enqueue on `s` and return
// the launch status.
hipError_t launch_decode(const lbf_desc& d, const uint8_t* blob, uint16_t* out, hipStream_t s);
hipError_t launch_verify(const lbf_desc& d, const uint8_t* blob, uint32_t* flags, hipStream_t s);
hipError_t launch_crc32(const uint8_t* data, uint64_t n, uint32_t* crc, hipStream_t s);

hipError_t launch_hist(const uint16_t* w, uint64_t n, uint32_t* hist, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, const lbf_desc& d, uint8_t* blob, uint32_t* tile_cnt, hipStream_t s);

// Per-tensor record of a product launch (40 bytes, 64 per launch): the three
// pointers and one 16-byte word of geometry taken from the host-checked
// descriptor, so every bound a kernel uses comes from a validated source.
// The code table is not here: each kernel reads it from the blob's own
// header copy (bytes 72..87), where a corrupt value can only give wrong
// weights, never an access outside the blob.
struct GroupArg {
  const uint8_t* blob;
  const uint16_t* x;
  void* y;
  uint32_t rows;
  uint32_t tiles;  // cols / 1024
  uint32_t n_esc;
  uint32_t aux;    // bit 0: contiguous table (lut[c] = lut[0] + c); the rest is launcher-specific
};
static_assert(sizeof(GroupArg) == 40, "group record");
constexpr uint32_t kAuxContig = 1u;

hipError_t launch_gemv(const GroupArg* groups, int n_groups, int batch, int y_dtype, hipStream_t s);
hipError_t launch_gemm(const GroupArg* groups, int n_groups, int batch, int y_dtype, hipStream_t s);
// h = silu(gate x) * (up x), one launch; x (batch * cols bf16) must fit the
// ring kernel's LDS x area.
constexpr uint64_t kGatedMaxXBytes = 131072;
hipError_t launch_gemv_gated(const GroupArg& gate, const GroupArg& up, int batch, void* h, int h_dtype,
                             hipStream_t s);

// K15H (entropy-coded variant): layout, code, and launchers (lbf_huff.hip).
struct HLayout {
  uint64_t n, n_tiles, n_esc, stream_words;
  uint64_t off_raw, off_bits, off_woff, off_idx, off_esc, blob_bytes;
};
HLayout hlayout_of(uint64_t rows, uint64_t cols, uint64_t n_esc, uint64_t stream_words);
void huffman_lengths(const uint64_t count[16], uint8_t len[16]);
struct HCode {
  uint32_t sym[16];  // code c: its canonical value bit-reversed << 4 | its length (0: unused)
};
HCode hcode_of(const uint8_t len[16]);
hipError_t launch_hcount(const lbf_desc& d, const uint8_t* blob, uint32_t* counts, hipStream_t s);
hipError_t launch_hwoff(const lbf_desc& d, const uint8_t* blob, const uint8_t len[16], uint32_t* words,
                        uint32_t* woff, hipStream_t s);
hipError_t launch_hpack(const lbf_desc& d, const uint8_t* blob, const HCode& code, const uint32_t* woff,
                        uint32_t* bits, uint64_t stream_words, hipStream_t s);
hipError_t launch_hfill(const lbf_hdesc& h, uint8_t* blob, hipStream_t s);
hipError_t launch_hdecode(const lbf_hdesc& h, const HCode& code, const uint8_t* blob, uint16_t* out, hipStream_t s);

// lbf_gemm keeps the byte offsets of 16 rows (or x rows) of a tensor in 32
// bits; rows longer than this many tiles (16,777,216 columns) are not supported.
constexpr uint32_t kGemmMaxTiles = 16384;

// Workspace layout of lbf_encode: hist[256] u32, then tile counts u32[n_tiles].
constexpr uint64_t kWorkHistBytes = 1024;
// Device address, on the current device, of the library's own encoder
// workspace (LBF_NOALLOC_SCRATCH_BYTES, lbf_encode.hip).
hipError_t encode_scratch(void** ptr);

// Launch facts of the current device, looked up once per device and kept for
// the process (thread-safe; lbf_api.cpp).
// Compute units of the current device.
hipError_t device_cus(int* cus);
// Resident workgroups per CU of kernel `fn` at `block` threads and no dynamic
// LDS on the current device (at least 1).
hipError_t blocks_per_cu(const void* fn, int block, int* n);
// Lets kernel `fn` take `bytes` of dynamic LDS on the current device: the
// attribute only grows, so concurrent callers that need different sizes
// never lower it under one another.
hipError_t open_dynamic_lds(const void* fn, int bytes);

}  // namespace lbf
