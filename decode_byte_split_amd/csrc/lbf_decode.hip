// lbf_decode.hip — standalone bit-exact decode of a blob back to BF16.
//
// Rebuilds the source tensor exactly (the round trip that makes the coding
// lossless: "Lossless LLM Weight Compression vs 8-bit GGUF", section "What does
// 'lossless' mean for LLM weights?").  One wave decodes one 1024-weight tile,
// lane l the weights 8l..8l+7 of each half (16 in all): two 8-byte raw loads
// and two 4-byte nibble loads, each coalesced across the wave (512 and 256 B
// contiguous), and two 16-byte stores, each writing one contiguous KiB of the
// output.  (With the lane's 16 weights contiguous instead, each store
// instruction wrote half of every 32 bytes of a 2 KiB span and the other
// store the rest: 152 against 136 us for the 8B-shaped layer.)  HBM traffic
// per weight: 1 + 0.5 bytes read, 2 written, plus 4 bytes of index per tile
// and one byte per escape.
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

// Escapes of the tile, when it has any: the slice esc[first, first + cnt)
// is copied into the wave's LDS slot by five 4-byte buffer loads per lane
// that write straight into LDS (one wait); escapes are numbered in element
// order, so those of the first halves (weights 0..511, lane by lane) come
// before those of the second halves.
__device__ __forceinline__ void patch_halves(u32x2 nib, const uint8_t* __restrict__ esc, uint32_t first, uint32_t cnt,
                                             uint8_t* slot, uint32_t E[4]) {
  const uint32_t lane = (uint32_t)lane_id();
  const uint32_t a0 = first & ~3u, nb = first + cnt - a0;
  // one range over the slice, rounded up to whole dwords (the escape plane
  // starts on a 256-byte boundary and the blob is a multiple of 256 bytes);
  // loads past it read as zeros
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(esc + a0), (short)0,
                                                                     (int)((nb + 3u) & ~3u), 0x00020000);
  uint32_t vo = 4 * lane;
  asm volatile("" : "+v"(vo));
  static_assert(kEscSlot == 5 * 256, "five loads of 256 bytes");
#pragma unroll
  for (uint32_t i = 0; i < 5; i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(slot + 256 * i), 4,
                                             vo + 256 * i, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the slice is in LDS
  wave_lds_sync();
  const uint64_t m0 = escape_mask8(nib.x), m1 = escape_mask8(nib.y);
  const uint32_t k0 = (uint32_t)__builtin_popcountll(m0), k1 = (uint32_t)__builtin_popcountll(m1);
  const uint32_t j0 = wave_excl_scan_small(k0);
  const uint32_t total0 = (uint32_t)__builtin_amdgcn_readlane((int)(j0 + k0), 63);
  const uint32_t j1 = total0 + wave_excl_scan_small(k1);
  const uint8_t* src = slot + (first & 3u);
  patch_escapes(src, j0, cnt, m0, 0, E);  // weights 0..7 of E: the first half
  patch_escapes(src, j1, cnt, 0, m1, E);  // weights 8..15: the second half
  wave_lds_sync();  // the slot is rewritten for the next tile
}

template <bool CONTIG>
__global__ __launch_bounds__(kDecodeWaves * kWave) void k_decode(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t esc_lds[kDecodeWaves][kEscSlot];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint32_t t = uniform(blockIdx.x * kDecodeWaves + (uint32_t)wave);
  if (t >= a.n_tiles) return;

  // the planes are whole tiles (padding included), so every load is in range
  const uint8_t* raw_t = a.raw + (size_t)t * kTile;
  const uint8_t* nib_t = a.nib + (size_t)t * (kTile / 2);
  const u32x2 ra = load_nt(reinterpret_cast<const u32x2*>(raw_t) + lane);
  const u32x2 rb = load_nt(reinterpret_cast<const u32x2*>(raw_t + kTile / 2) + lane);
  const uint32_t na = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(nib_t) + lane);
  const uint32_t nb = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(nib_t + kTile / 4) + lane);
  uint32_t first, cnt;
  tile_escape_range(a.idx, t, a.n_esc, first, cnt);

  // E[0..1] and w[0..3]: weights 8 lane .. 8 lane + 7; E[2..3] and w[4..7]:
  // weights 512 + 8 lane .. 512 + 8 lane + 7
  const u32x2 nib = u32x2{na, nb};
  uint32_t E[4];
  exponents16<CONTIG>(nib, a.lut, a.base4, E);
  if (cnt) patch_halves(nib, a.esc, first, cnt, esc_lds[wave], E);
  uint32_t w[8];
  assemble16(u32x4{ra.x, ra.y, rb.x, rb.y}, E, w);

  const uint64_t t0 = (uint64_t)t * kTile;
  const uint32_t n_real = (uint32_t)min((uint64_t)kTile, (uint64_t)a.n - t0);
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t i0 = (uint32_t)h * (kTile / 2) + 8u * (uint32_t)lane;  // first weight of this half in the tile
    const uint32_t* wh = w + 4 * h;
    if (i0 + 8 <= n_real) {
      __builtin_nontemporal_store((u32x4){wh[0], wh[1], wh[2], wh[3]}, reinterpret_cast<u32x4*>(a.out + t0 + i0));
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 8; i++)
        if (i0 + i < n_real) a.out[t0 + i0 + i] = (uint16_t)(wh[i >> 1] >> (16 * (i & 1)));
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
