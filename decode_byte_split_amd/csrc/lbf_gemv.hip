// lbf_gemv.hip — fused decode + matrix-vector product for batch 1..8.
//
// y[b, r] = sum_k W[r, k] x[b, k]: each coded weight is rebuilt, exactly, in
// registers and consumed at once by v_dot2_f32_bf16 (two bf16 products added
// to an fp32 accumulator); the decoded matrix never exists in memory.  This is
// the in-VRAM use of lossless coding described on "Lossless LLM Weight
// Compression vs 8-bit GGUF", section "What does 'lossless' mean for LLM
// weights?".  Weight bandwidth is the bound (same page, section "Lossless
// compression or Q8 GGUF: which should you deploy?", on weight-bandwidth-bound
// fleets), so the kernel is shaped for HBM streaming:
//
//  * work unit = (weight tensor, block of rows); one 256-thread workgroup per
//    unit, several tensors ("groups") per launch;
//  * K-stationary waves: within a unit each wave owns a fixed slice of whole
//    1024-weight tiles of every row it handles, keeps the matching x values
//    in VGPRs (B x tiles x 8 registers) and walks rows; the tensor's 4 waves
//    split K into 1, 2 or 4 slices and the rows between them;
//  * per tile and lane: one 16-byte raw load and one 8-byte nibble load, both
//    non-temporal and coalesced; the escape index is read with scalar loads
//    and the escape path runs only for tiles that hold escapes;
//  * each row's lane partials are summed across the wave with DPP and lane
//    reads in a fixed order, slices are combined in LDS in slice order: no
//    floating-point atomics, bitwise-reproducible output.
#include <hip/hip_runtime.h>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kGemvWaves = 4;
constexpr int kMaxUnitRows = 64;
constexpr int kUnitTiles = 128;  // target tiles of weights per work unit

struct GemvLaunch {
  GemvGroup g[LBF_MAX_GROUPS];
  int n_groups;
  int y_bf16;
};

// Sum of v over the 64 lanes, the same value in every lane, in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  // every lane of each 16-lane row now holds its row's sum
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN, sign kept
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int B>
__device__ __forceinline__ void dot16(const uint32_t w[8], const uint32_t (*xr)[8], float acc[B][2]) {
#pragma unroll
  for (int b = 0; b < B; b++) {
#pragma unroll
    for (int j = 0; j < 8; j++)
      acc[b][j & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]),
                                                      __builtin_bit_cast(bf16x2, xr[b][j]), acc[b][j & 1], false);
  }
}

template <int B, int SMAX>
__global__ __launch_bounds__(kGemvWaves * kWave) void k_gemv(GemvLaunch L) {
  __shared__ float part[kGemvWaves][kMaxUnitRows][B];
  __shared__ uint8_t esc_lds[kGemvWaves][kTile];

  const uint32_t u = blockIdx.x;
  int gi = 0;
  while (gi + 1 < L.n_groups && L.g[gi + 1].unit_begin <= u) gi++;
  const GemvGroup& G = L.g[gi];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t T = G.cols >> 10;  // tiles per row
  const uint32_t rb = G.geom & 0xFFFFu;
  const uint32_t nks = (G.geom >> 16) & 0xFu;
  const uint32_t phases = (G.geom >> 20) & 0xFu;
  const uint32_t r0 = (u - G.unit_begin) * rb;
  const uint32_t nr = min(rb, G.rows - r0);
  const uint32_t slice = (uint32_t)wave % nks, phase = (uint32_t)wave / nks;

  const uint64_t n_tiles = (uint64_t)G.rows * T;
  const uint8_t* raw_p = G.blob + LBF_HEADER_BYTES;
  const uint8_t* nib_p = raw_p + n_tiles * kTile;
  const uint32_t* idx_p = reinterpret_cast<const uint32_t*>(nib_p + n_tiles * (kTile / 2));
  const uint8_t* esc_p = G.blob + ((LBF_HEADER_BYTES + n_tiles * (kTile + kTile / 2) + 4 * (n_tiles + 1) + 255) & ~uint64_t(255));
  const Lut lut{G.lut[0], G.lut[1], G.lut[2], G.lut[3]};
  const bool contig = G.flags & 1u;

  for (uint32_t c0 = 0; c0 < T; c0 += nks * SMAX) {
    const uint32_t tb = c0 + slice * SMAX;
    const uint32_t S = tb < T ? min((uint32_t)SMAX, T - tb) : 0u;
    uint32_t xr[SMAX][B][8];
#pragma unroll
    for (int j = 0; j < SMAX; j++) {
      if ((uint32_t)j < S) {
#pragma unroll
        for (int b = 0; b < B; b++) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(G.x + (size_t)b * G.cols + (size_t)(tb + j) * kTile) + lane * 2;
          const u32x4 a0 = xp[0], a1 = xp[1];
          xr[j][b][0] = a0.x; xr[j][b][1] = a0.y; xr[j][b][2] = a0.z; xr[j][b][3] = a0.w;
          xr[j][b][4] = a1.x; xr[j][b][5] = a1.y; xr[j][b][6] = a1.z; xr[j][b][7] = a1.w;
        }
      }
    }
    for (uint32_t rl = phase; rl < nr; rl += phases) {
      const uint64_t t0 = (uint64_t)(r0 + rl) * T + tb;
      u32x4 raw[SMAX];
      u32x2 nib[SMAX];
#pragma unroll
      for (int j = 0; j < SMAX; j++) {
        if ((uint32_t)j < S) {
          raw[j] = load_nt(reinterpret_cast<const u32x4*>(raw_p + (t0 + j) * kTile) + lane);
          nib[j] = load_nt(reinterpret_cast<const u32x2*>(nib_p + (t0 + j) * (kTile / 2)) + lane);
        }
      }
      float acc[B][2];
#pragma unroll
      for (int b = 0; b < B; b++) acc[b][0] = acc[b][1] = 0.f;
#pragma unroll
      for (int j = 0; j < SMAX; j++) {
        if ((uint32_t)j < S) {
          uint32_t first, cnt;
          tile_escape_range(idx_p, (uint32_t)(t0 + j), G.n_esc, first, cnt);
          uint32_t E[4];
          if (contig)
            exponents16<true>(nib[j], lut, G.base4, E);
          else
            exponents16<false>(nib[j], lut, G.base4, E);
          if (cnt) place_escapes(nib[j], esc_p, first, cnt, esc_lds[wave], E);
          uint32_t w[8];
          assemble16(raw[j], E, w);
          dot16<B>(w, xr[j], acc);
        }
      }
#pragma unroll
      for (int b = 0; b < B; b++) {
        const float s = wave_sum(acc[b][0] + acc[b][1]);
        if (lane == 0) part[slice][rl][b] = (c0 == 0 ? 0.f : part[slice][rl][b]) + s;
      }
    }
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nr * B; i += kGemvWaves * kWave) {
    const uint32_t b = i / nr, rl = i % nr;
    float v = part[0][rl][b];
    for (uint32_t s = 1; s < nks; s++) v += part[s][rl][b];
    const size_t o = (size_t)b * G.rows + r0 + rl;
    if (L.y_bf16)
      static_cast<uint16_t*>(G.y)[o] = f32_to_bf16_rne(v);
    else
      static_cast<float*>(G.y)[o] = v;
  }
}

template <int B, int SMAX>
static hipError_t run(GemvLaunch& L, uint32_t units, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv<B, SMAX>), dim3(units), dim3(kGemvWaves * kWave), 0, s, L);
  return hipGetLastError();
}

// Unit geometry of one group for a given SMAX: K slices (1, 2 or 4), row
// phases (waves per slice) and rows per unit (a multiple of the phases, about
// kUnitTiles tiles of weights in total, at most kMaxUnitRows).
static uint32_t geometry(uint32_t rows, uint32_t T, uint32_t smax) {
  uint32_t nks = 1;
  while (nks < 4 && (T + nks - 1) / nks > smax) nks *= 2;
  const uint32_t phases = kGemvWaves / nks;
  uint32_t rb = kUnitTiles / T;
  rb = rb / phases * phases;
  if (rb < phases) rb = phases;
  if (rb > kMaxUnitRows) rb = kMaxUnitRows;
  if (rb > rows) rb = (rows + phases - 1) / phases * phases;
  if (rb > kMaxUnitRows) rb = kMaxUnitRows;
  return rb | (nks << 16) | (phases << 20);
}

hipError_t launch_gemv(const GemvGroup* groups, int n_groups, int batch, int y_dtype, hipStream_t s) {
  static const int smax_of[9] = {0, 8, 4, 2, 2, 1, 1, 1, 1};
  const int smax = smax_of[batch];
  GemvLaunch L;
  L.n_groups = n_groups;
  L.y_bf16 = y_dtype == LBF_BF16;
  uint32_t units = 0;
  for (int g = 0; g < n_groups; g++) {
    L.g[g] = groups[g];
    const uint32_t geom = geometry(groups[g].rows, groups[g].cols >> 10, (uint32_t)smax);
    L.g[g].geom = geom;
    L.g[g].unit_begin = units;
    const uint32_t rb = geom & 0xFFFFu;
    units += (groups[g].rows + rb - 1) / rb;
  }
  switch (batch) {
    case 1: return run<1, 8>(L, units, s);
    case 2: return run<2, 4>(L, units, s);
    case 3: return run<3, 2>(L, units, s);
    case 4: return run<4, 2>(L, units, s);
    case 5: return run<5, 1>(L, units, s);
    case 6: return run<6, 1>(L, units, s);
    case 7: return run<7, 1>(L, units, s);
    default: return run<8, 1>(L, units, s);
  }
}

}  // namespace lbf
