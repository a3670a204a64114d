// lbf_encode.hip — GPU encoder: exponent histogram, plane packing, escape
// index (prefix sum of per-tile counts) and escape stream compaction.
//
// Method ("Lossless LLM Weight Compression vs 8-bit GGUF", section "What did
// the GLM-5.2 experiment actually prove?"): frequent exponents get a fixed
// 4-bit code, the rest are written verbatim, in element order, to an escape
// stream.  The histogram drives the choice of the 15 coded exponents (made on
// the host between the two encode phases).
//
// Kernels, in stream order for phase 2:
//   k_pack     one wave per 1024-weight tile: raw and nibble planes, per-tile
//              escape count, and (block 0) the 256-byte header
//   k_scan     one workgroup: idx[t+1] = idx[t] + count[t]; zeroes the
//              alignment gaps after the index and the escape stream
//   k_escapes  one wave per tile with escapes: writes the tile's escape bytes
//              at idx[t] + (rank among the tile's escapes), so the stream is in
//              element order without atomics; positions at or past the
//              descriptor's escape count are dropped, so weights that no longer
//              match phase 1 can never write past the blob (the index then
//              disagrees with the header and lbf_verify reports it)
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kEncWaves = 4;

__global__ void k_zero_u32(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Exponent histogram: per-wave LDS bins (integer atomics, so the result does
// not depend on ordering), summed into the global 256-bin histogram.
__global__ __launch_bounds__(256) void k_hist(const uint16_t* __restrict__ w, uint64_t n, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[4][256];
  for (int i = threadIdx.x; i < 4 * 256; i += blockDim.x) (&h[0][0])[i] = 0u;
  __syncthreads();
  uint32_t* mine = h[threadIdx.x >> 6];
  const uint64_t n8 = n / 8;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const u32x4* w8 = reinterpret_cast<const u32x4*>(w);
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const u32x4 v = load_nt(w8 + i);
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      atomicAdd(&mine[(words[q] >> 7) & 0xFFu], 1u);
      atomicAdd(&mine[(words[q] >> 23) & 0xFFu], 1u);
    }
  }
  for (uint64_t i = n8 * 8 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    atomicAdd(&mine[(w[i] >> 7) & 0xFFu], 1u);
  __syncthreads();
  for (int e = threadIdx.x; e < 256; e += blockDim.x) {
    const uint32_t s = h[0][e] + h[1][e] + h[2][e] + h[3][e];
    if (s) atomicAdd(&hist[e], s);
  }
}

hipError_t launch_hist(const uint16_t* w, uint64_t n, uint32_t* hist, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(256), 0, s, hist, 256u);
  const uint64_t n8 = n / 8;
  uint64_t blocks = (n8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_hist, dim3((unsigned)blocks), dim3(256), 0, s, w, n, hist);
  return hipGetLastError();
}

struct PackArgs {
  const uint16_t* w;
  uint8_t* blob;
  uint8_t* raw;
  uint8_t* nib;
  uint32_t* tile_cnt;
  uint32_t n, n_tiles;
  uint32_t inv[64];     // inv[e] = code of exponent e (15 = escape), 4 per word
  uint32_t header[24];  // the 96 descriptor bytes
};

// Raw byte, code and escape flag of each of a lane's 16 weights.
__device__ __forceinline__ void lane_fields(const uint16_t* __restrict__ w, uint64_t e0, uint32_t n,
                                            const uint8_t* inv, uint32_t raw[4], uint32_t code[2],
                                            uint32_t& esc_mask) {
  uint32_t h[8];
  if (e0 + 16 <= n) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w + e0);
    const u32x4 a = load_nt(p), b = load_nt(p + 1);
    h[0] = a.x; h[1] = a.y; h[2] = a.z; h[3] = a.w;
    h[4] = b.x; h[5] = b.y; h[6] = b.z; h[7] = b.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const uint32_t lo = (e0 + 2 * q < n) ? w[e0 + 2 * q] : 0u;
      const uint32_t hi = (e0 + 2 * q + 1 < n) ? w[e0 + 2 * q + 1] : 0u;
      h[q] = lo | (hi << 16);
    }
  }
  // raw byte of weight i: mantissa_i << 1 | sign of partner i ^ 1;
  // code of weight i: nibble word i >> 3, byte i & 3, high nibble if bit 2 of i
  raw[0] = raw[1] = raw[2] = raw[3] = 0u;
  code[0] = code[1] = 0u;
  esc_mask = 0u;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const uint32_t v = (h[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const uint32_t partner = (h[i >> 1] >> (16 * ((i & 1) ^ 1))) & 0xFFFFu;
    const bool valid = e0 + (uint64_t)i < n;
    const uint32_t r = ((v & 0x7Fu) << 1) | (partner >> 15);
    const uint32_t c = valid ? (uint32_t)inv[(v >> 7) & 0xFFu] : 0u;
    raw[i >> 2] |= r << (8 * (i & 3));
    code[i >> 3] |= c << (8 * (i & 3) + 4 * ((i >> 2) & 1));
    if (c == 15u) esc_mask |= 1u << i;
  }
}

__global__ __launch_bounds__(kEncWaves * kWave) void k_pack(PackArgs a) {
  __shared__ uint8_t inv[256];
  if (threadIdx.x < 64) reinterpret_cast<uint32_t*>(inv)[threadIdx.x] = a.inv[threadIdx.x];
  if (blockIdx.x == 0 && threadIdx.x < 64)
    reinterpret_cast<uint32_t*>(a.blob)[threadIdx.x] = threadIdx.x < 24 ? a.header[threadIdx.x] : 0u;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t t = uniform(blockIdx.x * kEncWaves + (uint32_t)wave);
  if (t >= a.n_tiles) return;
  const uint64_t e0 = (uint64_t)t * kTile + (uint64_t)lane * 16;
  uint32_t raw[4], code[2], esc_mask;
  lane_fields(a.w, e0, a.n, inv, raw, code, esc_mask);
  __builtin_nontemporal_store((u32x4){raw[0], raw[1], raw[2], raw[3]},
                              reinterpret_cast<u32x4*>(a.raw + (size_t)t * kTile) + lane);
  __builtin_nontemporal_store((u32x2){code[0], code[1]}, reinterpret_cast<u32x2*>(a.nib + (size_t)t * (kTile / 2)) + lane);
  // tile escape count = sum over lanes of popcount(esc_mask), bit by bit
  const uint32_t k = (uint32_t)__builtin_popcount(esc_mask);
  uint32_t total = 0;
#pragma unroll
  for (int b = 0; b < 5; b++) total += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(((k >> b) & 1u) != 0)) << b;
  if (lane == 0) a.tile_cnt[t] = total;
}

// Single workgroup: exclusive prefix sum of the per-tile counts into idx[],
// 1024 tiles per round, plus zeroing of the blob's alignment gaps.
__global__ __launch_bounds__(1024) void k_scan(const uint32_t* __restrict__ cnt, uint32_t n_tiles, uint32_t* idx,
                                               uint8_t* gap_a, uint32_t gap_a_len, uint8_t* gap_b, uint32_t gap_b_len) {
  __shared__ uint32_t s[1024];
  __shared__ uint32_t carry;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    carry = 0;
    idx[0] = 0;
  }
  for (uint32_t i = tid; i < gap_a_len; i += 1024) gap_a[i] = 0;
  for (uint32_t i = tid; i < gap_b_len; i += 1024) gap_b[i] = 0;
  __syncthreads();
  for (uint32_t base = 0; base < n_tiles; base += 1024) {
    const uint32_t v = (base + tid < n_tiles) ? cnt[base + tid] : 0u;
    s[tid] = v;
    __syncthreads();
    for (uint32_t d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
      const uint32_t add = tid >= d ? s[tid - d] : 0u;
      __syncthreads();
      s[tid] += add;
      __syncthreads();
    }
    if (base + tid < n_tiles) idx[base + tid + 1] = carry + s[tid];
    __syncthreads();
    if (tid == 1023) carry += s[1023];
    __syncthreads();
  }
}

struct EscArgs {
  const uint16_t* w;
  const uint32_t* idx;
  uint8_t* esc;
  uint32_t n, n_tiles;
  uint32_t n_esc;  // escape bytes the blob holds (from the phase-1 descriptor)
  uint32_t inv[64];
};

__global__ __launch_bounds__(kEncWaves * kWave) void k_escapes(EscArgs a) {
  __shared__ uint8_t inv[256];
  if (threadIdx.x < 64) reinterpret_cast<uint32_t*>(inv)[threadIdx.x] = a.inv[threadIdx.x];
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t t = uniform(blockIdx.x * kEncWaves + (uint32_t)wave);
  if (t >= a.n_tiles) return;
  const uint32_t first = a.idx[t];
  if (a.idx[t + 1] == first) return;
  const uint64_t e0 = (uint64_t)t * kTile + (uint64_t)lane * 16;
  uint32_t raw[4], code[2], esc_mask;
  lane_fields(a.w, e0, a.n, inv, raw, code, esc_mask);
  uint32_t j = first + wave_excl_scan_small((uint32_t)__builtin_popcount(esc_mask));
  while (esc_mask) {
    const uint32_t i = (uint32_t)__builtin_ctz(esc_mask);
    if (j < a.n_esc) a.esc[j] = (uint8_t)((a.w[e0 + i] >> 7) & 0xFFu);
    j++;
    esc_mask &= esc_mask - 1;
  }
}

// ---- Encoder workspace held by the library (lbf_encode_noalloc) ------------
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid it) get the encoder's workspace from
// this file-scope device array instead of an argument.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is only a stand-in, never a device address: its address on the
// current device comes from hipGetSymbolAddress, looked up once per device
// (with that device current) and kept.
static __device__ __align__(256) uint8_t scratch[LBF_NOALLOC_SCRATCH_BYTES];

hipError_t encode_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> per_device;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = per_device.find(dev);
  if (it == per_device.end()) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess) return r;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = per_device.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

hipError_t launch_pack(const uint16_t* w, const lbf_desc& d, uint8_t* blob, uint32_t* tile_cnt, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  uint8_t inv8[256];
  for (int e = 0; e < 256; e++) inv8[e] = 15;
  for (int c = 0; c < d.n_codes; c++) inv8[d.lut[c]] = (uint8_t)c;

  PackArgs p;
  p.w = w;
  p.blob = blob;
  p.raw = blob + L.off_raw;
  p.nib = blob + L.off_nib;
  p.tile_cnt = tile_cnt;
  p.n = (uint32_t)L.n;
  p.n_tiles = (uint32_t)L.n_tiles;
  for (int q = 0; q < 64; q++)
    p.inv[q] = inv8[4 * q] | (inv8[4 * q + 1] << 8) | (inv8[4 * q + 2] << 16) | ((uint32_t)inv8[4 * q + 3] << 24);
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(&d);
  for (int q = 0; q < 24; q++)
    p.header[q] = hb[4 * q] | (hb[4 * q + 1] << 8) | (hb[4 * q + 2] << 16) | ((uint32_t)hb[4 * q + 3] << 24);
  const unsigned grid = (unsigned)((L.n_tiles + kEncWaves - 1) / kEncWaves);
  // block 0 writes the header even for an empty tensor
  hipLaunchKernelGGL(k_pack, dim3(grid ? grid : 1), dim3(kEncWaves * kWave), 0, s, p);

  uint32_t* idx = reinterpret_cast<uint32_t*>(blob + L.off_idx);
  uint8_t* gap_a = blob + L.off_idx + 4 * (L.n_tiles + 1);
  const uint32_t gap_a_len = (uint32_t)(L.off_esc - (L.off_idx + 4 * (L.n_tiles + 1)));
  uint8_t* gap_b = blob + L.off_esc + L.n_esc;
  const uint32_t gap_b_len = (uint32_t)(L.blob_bytes - (L.off_esc + L.n_esc));
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, tile_cnt, (uint32_t)L.n_tiles, idx, gap_a, gap_a_len, gap_b,
                     gap_b_len);
  if (d.n_esc && grid) {
    EscArgs e;
    e.w = w;
    e.idx = idx;
    e.esc = blob + L.off_esc;
    e.n = (uint32_t)L.n;
    e.n_tiles = (uint32_t)L.n_tiles;
    e.n_esc = (uint32_t)L.n_esc;
    for (int q = 0; q < 64; q++) e.inv[q] = p.inv[q];
    hipLaunchKernelGGL(k_escapes, dim3(grid), dim3(kEncWaves * kWave), 0, s, e);
  }
  return hipGetLastError();
}

}  // namespace lbf
