// lbf_decode.hip — standalone bit-exact decode of a blob back to BF16.
//
// Rebuilds the source tensor exactly (the round trip that makes the coding
// lossless: "Lossless LLM Weight Compression vs 8-bit GGUF", section "What does
// 'lossless' mean for LLM weights?").  One wave decodes one 1024-weight tile:
// 16 weights per lane from a 16-byte raw load and an 8-byte nibble load, both
// coalesced across the wave (1 KiB and 512 B contiguous); output is two 16-byte
// stores per lane.  HBM traffic per weight: 1 + 0.5 bytes read, 2 written, plus
// 4 bytes of index per tile and one byte per escape.
#include <hip/hip_runtime.h>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kDecodeWaves = 4;  // waves per workgroup

struct DecodeArgs {
  const uint8_t* raw;
  const uint8_t* nib;
  const uint32_t* idx;
  const uint8_t* esc;
  uint16_t* out;
  uint32_t n, n_tiles, n_esc;
  Lut lut;
  uint32_t base4;
};

template <bool CONTIG>
__global__ __launch_bounds__(kDecodeWaves * kWave) void k_decode(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t esc_lds[kDecodeWaves][kEscSlot];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint32_t t = uniform(blockIdx.x * kDecodeWaves + (uint32_t)wave);
  if (t >= a.n_tiles) return;

  const u32x4 raw = load_nt(reinterpret_cast<const u32x4*>(a.raw + (size_t)t * kTile) + lane);
  const u32x2 nib = load_nt(reinterpret_cast<const u32x2*>(a.nib + (size_t)t * (kTile / 2)) + lane);
  uint32_t first, cnt;
  tile_escape_range(a.idx, t, a.n_esc, first, cnt);

  uint32_t E[4];
  exponents16<CONTIG>(nib, a.lut, a.base4, E);
  if (cnt) place_escapes(nib, a.esc, first, cnt, esc_lds[wave], E);
  uint32_t w[8];
  assemble16(raw, E, w);

  const uint64_t e0 = (uint64_t)t * kTile + (uint64_t)lane * 16;
  if (e0 + 16 <= a.n) {
    u32x4* o = reinterpret_cast<u32x4*>(a.out + e0);
    __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, o);
    __builtin_nontemporal_store((u32x4){w[4], w[5], w[6], w[7]}, o + 1);
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (e0 + i < a.n) a.out[e0 + i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    }
  }
}

hipError_t launch_decode(const lbf_desc& d, const uint8_t* blob, uint16_t* out, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  if (L.n_tiles == 0) return hipSuccess;
  const KLut k = klut_of(d);
  DecodeArgs a;
  a.raw = blob + L.off_raw;
  a.nib = blob + L.off_nib;
  a.idx = reinterpret_cast<const uint32_t*>(blob + L.off_idx);
  a.esc = blob + L.off_esc;
  a.out = out;
  a.n = (uint32_t)L.n;
  a.n_tiles = (uint32_t)L.n_tiles;
  a.n_esc = (uint32_t)L.n_esc;
  a.lut = Lut{k.t[0], k.t[1], k.t[2], k.t[3]};
  a.base4 = k.base4;
  const unsigned grid = (unsigned)((L.n_tiles + kDecodeWaves - 1) / kDecodeWaves);
  if (k.contiguous)
    hipLaunchKernelGGL(k_decode<true>, dim3(grid), dim3(kDecodeWaves * kWave), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3(grid), dim3(kDecodeWaves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace lbf
