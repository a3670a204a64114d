// lbf_gemv.hip — fused decode + matrix-vector product for batch 1..8.
//
// y[b, r] = sum_k W[r, k] x[b, k]: each coded weight is rebuilt, exactly, in
// registers and consumed at once by v_dot2_f32_bf16 (two bf16 products added
// to an fp32 accumulator); the decoded matrix never exists in memory.  This is
// the in-VRAM use of lossless coding described on "Lossless LLM Weight
// Compression vs 8-bit GGUF", section "What does 'lossless' mean for LLM
// weights?".  Weight bandwidth is the bound (same page, section "Lossless
// compression or Q8 GGUF: which should you deploy?", on fleets whose
// bottleneck is weight bandwidth), so the kernel is built for HBM streaming:
//
//  * persistent workgroups (as many as fit on the chip), each taking one
//    contiguous, cost-balanced range of work units across the launch's
//    weight tensors ("groups"); a unit is `phases` consecutive rows of one
//    tensor, all K;
//  * K-stationary waves: each of the 4 waves owns a fixed slice of whole
//    1024-weight tiles (1, 2 or 4 slices per row) and one row of every unit
//    (the row phase), keeps the matching x values in VGPRs and walks rows;
//  * per tile and lane one 16-byte raw load and one 8-byte nibble load, both
//    non-temporal and coalesced; the loads for the next row are issued before
//    the current row is decoded (two row buffers, ping-pong);
//  * the escape bytes of a workgroup's whole range of one tensor are one
//    contiguous slice of the escape stream: they are preloaded into LDS once,
//    so a tile with escapes costs no extra memory round trip; the tile index
//    is read with scalar loads;
//  * each row's lane partials are summed across the wave with DPP and lane
//    reads in a fixed order, K slices are combined in LDS in slice order: no
//    floating-point atomics, bitwise-reproducible output.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kGemvWaves = 4;
constexpr int kSubUnits = 64;     // units whose partial sums share one LDS batch
constexpr int kEscShared = 8192;  // escape bytes a workgroup preloads per tensor range

struct GemvLaunch {
  GemvGroup g[LBF_MAX_GROUPS];
  uint64_t total_cost;
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

// One row's coded data for one wave's K slice.  The tile index travels with
// the data as a vector load (lane j holds idx[t0 + j]), so that waiting for
// it never waits on LDS traffic (scalar loads share LDS's wait counter).
template <int SMAX>
struct RowBuf {
  u32x4 raw[SMAX];
  u32x2 nib[SMAX];
  uint32_t ixv;
};

// Loads are never conditional: a tile past the slice end (S < SMAX) reloads
// the slice's last tile, and the prefetch after a wave's last row reloads
// that row.  The redundant requests hit cache; in exchange the compiler can
// count outstanding loads exactly and keeps the next row in flight while the
// current one is decoded.
template <int SMAX>
__device__ __forceinline__ void load_row(RowBuf<SMAX>& R, const uint8_t* raw_p, const uint8_t* nib_p,
                                         const uint32_t* idx_p, uint64_t t0, uint32_t S, int lane) {
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    const uint64_t t = t0 + min((uint32_t)j, S - 1);
    R.raw[j] = load_nt(reinterpret_cast<const u32x4*>(raw_p + t * kTile) + lane);
    R.nib[j] = load_nt(reinterpret_cast<const u32x2*>(nib_p + t * (kTile / 2)) + lane);
  }
  R.ixv = idx_p[t0 + min((uint32_t)lane, S)];
}

struct SegCtx {
  const uint8_t* esc_p;  // escape stream of the tensor
  const uint8_t* esc_sh; // LDS copy of escapes [e_lo, e_hi) when preloaded
  uint8_t* esc_wave;     // this wave's 1 KiB staging slot otherwise
  uint32_t e_lo, e_hi;   // escape range of the workgroup's rows (clamped)
  Lut lut;
  uint32_t base4;
};

// PRELOAD: the segment's escapes sit in LDS (the common case).  Otherwise
// (dense escapes) each tile's slice is staged from memory when needed.
template <int B, int SMAX, bool CONTIG, bool PRELOAD>
__device__ __forceinline__ void row_dot(const RowBuf<SMAX>& R, uint32_t S, const uint32_t (*xr)[B][8],
                                        const SegCtx& C, float acc[B][2]) {
#pragma unroll
  for (int b = 0; b < B; b++) acc[b][0] = acc[b][1] = 0.f;
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    if ((uint32_t)j < S) {
      uint32_t E[4];
      exponents16<CONTIG>(R.nib[j], C.lut, C.base4, E);
      // clamp the index into the range this workgroup knows, so a corrupt
      // blob can only give wrong values, never an out-of-range access
      const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)R.ixv, j);
      const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)R.ixv, j + 1);
      const uint32_t a = min(max(ia, C.e_lo), C.e_hi);
      const uint32_t e = min(max(ib, a), C.e_hi);
      const uint32_t cnt = min(e - a, (uint32_t)kTile);
      if (cnt) {
        if (PRELOAD) {
          uint64_t m0, m1;
          const uint32_t r = escape_rank(R.nib[j], m0, m1);
          patch_escapes(C.esc_sh + (a - C.e_lo), r, cnt, m0, m1, E);
        } else {
          place_escapes(R.nib[j], C.esc_p, a, cnt, C.esc_wave, E);
        }
      }
      uint32_t w[8];
      assemble16(R.raw[j], E, w);
      dot16<B>(w, xr[j], acc);
    }
  }
}

// The rows of one pass (one K chunk of one batch of units) for one wave.
template <int B, int SMAX, bool CONTIG, bool PRELOAD>
__device__ __forceinline__ void run_rows(RowBuf<SMAX>& A, const uint8_t* raw_p, const uint8_t* nib_p,
                                         const uint32_t* idx_p, uint64_t row_tile0, uint64_t row_stride,
                                         uint32_t n_mine, uint32_t S, const uint32_t (*xr)[B][8], const SegCtx& C,
                                         float (*part)[kGemvWaves][B], uint32_t wave, bool accumulate, int lane) {
  RowBuf<SMAX> Bf;
  auto finish = [&](uint32_t ul, float acc[B][2]) {
#pragma unroll
    for (int b = 0; b < B; b++) {
      const float s = wave_sum(acc[b][0] + acc[b][1]);
      if (lane == 0) part[ul][wave][b] = (accumulate ? part[ul][wave][b] : 0.f) + s;
    }
  };
  const uint32_t last = n_mine - 1;
  for (uint32_t ul = 0;; ul += 2) {
    float acc[B][2];
    load_row<SMAX>(Bf, raw_p, nib_p, idx_p, row_tile0 + (uint64_t)min(ul + 1, last) * row_stride, S, lane);
    row_dot<B, SMAX, CONTIG, PRELOAD>(A, S, xr, C, acc);
    finish(ul, acc);
    if (ul + 1 > last) break;
    load_row<SMAX>(A, raw_p, nib_p, idx_p, row_tile0 + (uint64_t)min(ul + 2, last) * row_stride, S, lane);
    row_dot<B, SMAX, CONTIG, PRELOAD>(Bf, S, xr, C, acc);
    finish(ul + 1, acc);
    if (ul + 2 > last) break;
  }
}

// One workgroup's units [u_lo, u_hi) of group G.
template <int B, int SMAX, bool CONTIG>
__device__ __forceinline__ void run_segment(const GemvGroup& G, uint32_t u_lo, uint32_t u_hi, bool y_bf16,
                                            float (*part)[kGemvWaves][B], uint8_t* esc_sh, uint8_t* esc_wave,
                                            uint32_t wave, int lane) {
  const uint32_t T = G.cols >> 10;
  const uint32_t nks = G.geom & 0xFu, phases = (G.geom >> 4) & 0xFu;
  const uint32_t slice = wave % nks, phase = wave / nks;
  const uint64_t n_tiles = (uint64_t)G.rows * T;
  const uint8_t* raw_p = G.blob + LBF_HEADER_BYTES;
  const uint8_t* nib_p = raw_p + n_tiles * kTile;
  const uint32_t* idx_p = reinterpret_cast<const uint32_t*>(nib_p + n_tiles * (kTile / 2));
  const uint8_t* esc_p =
      G.blob + ((LBF_HEADER_BYTES + n_tiles * (kTile + kTile / 2) + 4 * (n_tiles + 1) + 255) & ~uint64_t(255));
  const uint32_t r_lo = u_lo * phases, r_hi = min(G.rows, u_hi * phases);

  SegCtx C;
  C.esc_p = esc_p;
  C.esc_sh = esc_sh;
  C.esc_wave = esc_wave;
  C.lut = Lut{G.lut[0], G.lut[1], G.lut[2], G.lut[3]};
  C.base4 = G.base4;
  // escape range of the whole segment (scalar loads, waited for only after
  // the first row's loads are on their way)
  const uint32_t seg_hi = idx_p[(uint64_t)r_hi * T];
  const uint32_t seg_lo = idx_p[(uint64_t)r_lo * T];
  __syncthreads();  // the previous segment is done with esc_sh and part

  bool first = true, preload = true;
  for (uint32_t sub = u_lo; sub < u_hi; sub += kSubUnits) {
    const uint32_t nsub = min((uint32_t)kSubUnits, u_hi - sub);
    for (uint32_t c0 = 0; c0 < T; c0 += nks * SMAX) {
      // this wave's K slice: tiles [tb, tb + S) of each row (S = 0: the
      // slice is past the row's end; loads then use the row's last tile)
      const uint32_t tb = c0 + slice * SMAX;
      const uint32_t S = tb < T ? min((uint32_t)SMAX, T - tb) : 0u;
      const uint32_t tl = tb < T ? tb : T - 1;
      const uint32_t SL = S ? S : 1u;
      // this wave's rows: r(ul) = (sub + ul) * phases + phase, ul < n_mine
      uint32_t n_mine = 0;
      while (n_mine < nsub && (sub + n_mine) * phases + phase < G.rows) n_mine++;
      const uint64_t row_tile0 = (uint64_t)(sub * phases + phase) * T + tl;
      const uint64_t row_stride = (uint64_t)phases * T;
      RowBuf<SMAX> A;
      if (n_mine) load_row<SMAX>(A, raw_p, nib_p, idx_p, row_tile0, SL, lane);
      uint32_t xr[SMAX][B][8];
#pragma unroll
      for (int j = 0; j < SMAX; j++) {
        const uint32_t tj = tl + min((uint32_t)j, SL - 1);
#pragma unroll
        for (int b = 0; b < B; b++) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(G.x + (size_t)b * G.cols + (size_t)tj * kTile) + lane * 2;
          const u32x4 a0 = xp[0], a1 = xp[1];
          xr[j][b][0] = a0.x; xr[j][b][1] = a0.y; xr[j][b][2] = a0.z; xr[j][b][3] = a0.w;
          xr[j][b][4] = a1.x; xr[j][b][5] = a1.y; xr[j][b][6] = a1.z; xr[j][b][7] = a1.w;
        }
      }
      if (first) {  // uniform across the workgroup: preload the segment's escapes
        first = false;
        C.e_hi = min(seg_hi, G.n_esc);
        C.e_lo = min(seg_lo, C.e_hi);
        preload = C.e_hi - C.e_lo <= (uint32_t)kEscShared;
        if (!preload) {  // dense escapes: per-tile staging, bounded by the stream itself
          C.e_lo = 0;
          C.e_hi = G.n_esc;
        } else {
          for (uint32_t p = threadIdx.x; p < C.e_hi - C.e_lo; p += kGemvWaves * kWave) esc_sh[p] = esc_p[C.e_lo + p];
        }
        __syncthreads();
      }
      if (n_mine) {
        if (preload)
          run_rows<B, SMAX, CONTIG, true>(A, raw_p, nib_p, idx_p, row_tile0, row_stride, n_mine, S, xr, C, part, wave,
                                          c0 != 0, lane);
        else
          run_rows<B, SMAX, CONTIG, false>(A, raw_p, nib_p, idx_p, row_tile0, row_stride, n_mine, S, xr, C, part,
                                           wave, c0 != 0, lane);
      }
    }
    __syncthreads();
    const uint32_t nrow = min(nsub * phases, G.rows - sub * phases);
    for (uint32_t i = threadIdx.x; i < nrow * B; i += kGemvWaves * kWave) {
      const uint32_t b = i / nrow, rl = i % nrow;
      const uint32_t ul = rl / phases, ph = rl % phases;
      float v = part[ul][ph * nks][b];
      for (uint32_t s = 1; s < nks; s++) v += part[ul][ph * nks + s][b];
      const size_t o = (size_t)b * G.rows + (size_t)sub * phases + rl;
      if (y_bf16)
        static_cast<uint16_t*>(G.y)[o] = f32_to_bf16_rne(v);
      else
        static_cast<float*>(G.y)[o] = v;
    }
    __syncthreads();
  }
}

template <int B, int SMAX>
__global__ __launch_bounds__(kGemvWaves * kWave) void k_gemv(GemvLaunch L) {
  __shared__ float part[kSubUnits][kGemvWaves][B];
  __shared__ uint8_t esc_sh[kEscShared];
  __shared__ uint8_t esc_wave[kGemvWaves][kTile];
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const int lane = lane_id();
  // this workgroup's share of the total cost: units whose start cost is in [c_lo, c_hi)
  const uint64_t c_lo = L.total_cost * blockIdx.x / gridDim.x;
  const uint64_t c_hi = L.total_cost * (blockIdx.x + 1) / gridDim.x;
  for (int gi = 0; gi < L.n_groups; gi++) {
    const GemvGroup& G = L.g[gi];
    const uint64_t g_lo = G.cost_begin, g_hi = G.cost_begin + (uint64_t)G.n_units * G.unit_cost;
    if (g_hi <= c_lo) continue;
    if (g_lo >= c_hi) break;
    const uint32_t u_lo = c_lo > g_lo ? (uint32_t)((c_lo - g_lo + G.unit_cost - 1) / G.unit_cost) : 0u;
    const uint32_t u_hi = (uint32_t)min((uint64_t)G.n_units, (c_hi - g_lo + G.unit_cost - 1) / G.unit_cost);
    if (u_lo >= u_hi) continue;
    if (G.flags & 1u)
      run_segment<B, SMAX, true>(G, u_lo, u_hi, L.y_bf16, part, esc_sh, esc_wave[wave], wave, lane);
    else
      run_segment<B, SMAX, false>(G, u_lo, u_hi, L.y_bf16, part, esc_sh, esc_wave[wave], wave, lane);
  }
}

// Unit geometry of one group: K slices (1, 2 or 4 per row, each at most
// smax tiles per pass) and row phases (waves per slice, 4 / slices).
static uint32_t geometry(uint32_t T, uint32_t smax) {
  uint32_t nks = 1;
  while (nks < (uint32_t)kGemvWaves && (T + nks - 1) / nks > smax) nks *= 2;
  return nks | ((kGemvWaves / nks) << 4);
}

template <int B, int SMAX>
static hipError_t run(GemvLaunch& L, hipStream_t s) {
  static int per_cu = 0, cus = 0;
  if (!per_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return hipErrorUnknown;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gemv<B, SMAX>, kGemvWaves * kWave, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  uint64_t units = 0;
  for (int g = 0; g < L.n_groups; g++) units += L.g[g].n_units;
  const uint64_t grid = std::min<uint64_t>((uint64_t)per_cu * cus, units);
  hipLaunchKernelGGL((k_gemv<B, SMAX>), dim3((unsigned)grid), dim3(kGemvWaves * kWave), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvGroup* groups, int n_groups, int batch, int y_dtype, hipStream_t s) {
  static const int smax_of[9] = {0, 4, 4, 2, 2, 1, 1, 1, 1};
  const uint32_t smax = (uint32_t)smax_of[batch];
  GemvLaunch L;
  L.n_groups = n_groups;
  L.y_bf16 = y_dtype == LBF_BF16;
  uint64_t cost = 0;
  for (int g = 0; g < n_groups; g++) {
    GemvGroup G = groups[g];
    const uint32_t T = G.cols >> 10;
    G.geom = geometry(T, smax);
    const uint32_t phases = (G.geom >> 4) & 0xFu;
    G.n_units = (G.rows + phases - 1) / phases;
    // cost of a tile in 1/16 units: 16 plus the escape work, ~1/8 per escape
    const uint64_t n_tiles = (uint64_t)G.rows * T;
    const uint32_t esc_per_tile = (uint32_t)std::min<uint64_t>(1024, (G.n_esc + n_tiles - 1) / n_tiles);
    G.unit_cost = phases * T * (16u + esc_per_tile / 8u);
    G.cost_begin = cost;
    cost += (uint64_t)G.n_units * G.unit_cost;
    L.g[g] = G;
  }
  L.total_cost = cost;
  switch (batch) {
    case 1: return run<1, 4>(L, s);
    case 2: return run<2, 4>(L, s);
    case 3: return run<3, 2>(L, s);
    case 4: return run<4, 2>(L, s);
    case 5: return run<5, 1>(L, s);
    case 6: return run<6, 1>(L, s);
    case 7: return run<7, 1>(L, s);
    default: return run<8, 1>(L, s);
  }
}

}  // namespace lbf
