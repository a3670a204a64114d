// lbf_gemv.hip — fused decode + matrix-vector product for batch 1..8.
//
// y[b, r] = sum_k W[r, k] x[b, k]: each coded weight is rebuilt, exactly, in
// registers and consumed at once by v_dot2_f32_bf16 (two bf16 products added
// to an fp32 accumulator); the decoded matrix never exists in memory.  This is
// the in-VRAM use of lossless coding described on "Lossless LLM Weight
// Compression vs 8-bit GGUF", section "What does 'lossless' mean for LLM
// weights?".  Weight bandwidth is the bound (same page, section "Lossless
// compression or Q8 GGUF: which should you deploy?", on fleets whose
// bottleneck is weight bandwidth), so both kernels here are HBM streams:
//
//  * k_gemv_ring (x of each tensor fits in 128 KiB of LDS): one workgroup
//    per CU (16 waves); the tensors are cut into teams whose x fits in LDS
//    together (one team when all of it does), each team gets CUs in
//    proportion to its coded bytes, its rows are dealt to those CUs, and
//    waves take rows from an LDS counter and stream them through a
//    three-slot register ring (details at the kernel);
//  * k_gemv (everything else): persistent workgroups, each taking one
//    contiguous, cost-balanced range of work units across the launch's
//    tensors; a unit is `phases` consecutive rows of one tensor, all K; each
//    of the 4 waves owns a fixed slice of whole tiles (1, 2 or 4 slices per
//    row), keeps the matching x in VGPRs and walks rows, loads for the next
//    row in flight (two row buffers); the escape bytes of a workgroup's range
//    of one tensor are one contiguous slice, preloaded into LDS once.
//
// Both read every tile with one 16-byte raw load and one 8-byte nibble load
// per lane (non-temporal, coalesced), sum each row's lane partials across the
// wave with DPP and lane reads in a fixed order and combine K slices in LDS in
// slice order: no floating-point atomics, bitwise-reproducible output.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kGemvWaves = 4;
constexpr int kSubUnits = 64;     // units whose partial sums share one LDS batch
constexpr int kEscShared = 8192;  // escape bytes a workgroup preloads per tensor range

struct GemvLaunch {
  GroupArg g[LBF_MAX_GROUPS];
  uint64_t total_cost;  // sum over groups of n_units * unit_cost (unit_info)
  int n_groups;
  int y_bf16;
};
static_assert(sizeof(GemvLaunch) <= 3072, "kernel arguments stay well inside the 4 KiB limit");

// Work units of one group in the static kernel: K slices (1, 2 or 4 per row,
// each at most smax tiles per pass), row phases (waves per slice, 4 /
// slices), units (phases consecutive rows, all K) and the cost of a unit in
// 1/16 tiles: 16 per tile plus the escape work, ~1/8 per escape.  The
// launcher puts log2(slices) and the per-tile cost factor into the record's
// aux word (bits 16..17 and 8..15), from which host and device derive the
// rest the same way.
struct UnitInfo {
  uint32_t nks, phases, n_units, unit_cost;
};
static uint32_t static_aux(const GroupArg& G, uint32_t smax) {
  uint32_t lg = 0;
  while ((1u << lg) < (uint32_t)kGemvWaves && (G.tiles + (1u << lg) - 1) >> lg > smax) lg++;
  const uint64_t n_tiles = (uint64_t)G.rows * G.tiles;
  const uint64_t ept = (G.n_esc + n_tiles - 1) / n_tiles;
  const uint32_t f = 16u + (uint32_t)(ept < 1024 ? ept : 1024) / 8u;  // <= 144
  return (G.aux & kAuxContig) | (f << 8) | (lg << 16);
}
__host__ __device__ inline UnitInfo unit_info(const GroupArg& G) {
  UnitInfo u;
  const uint32_t lg = (G.aux >> 16) & 3u;
  u.nks = 1u << lg;
  u.phases = (uint32_t)kGemvWaves >> lg;
  u.n_units = (G.rows + u.phases - 1) >> (2u - lg);
  u.unit_cost = u.phases * G.tiles * ((G.aux >> 8) & 0xFFu);
  return u;
}


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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// v from lane i ^ 32 (H = 32) or i ^ 16 (H = 16), by the gfx950 lane swaps:
// swapping a register with itself leaves each lane's partner value in one
// of the two results.
template <int H>
__device__ __forceinline__ float lane_xor(float v, bool upper) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = H == 32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

// out[b] = sum over the wave of in[b], b < B, uniform (B <= 8), in a fixed
// order.  Instead of B separate reductions, B values are folded together:
// at each of up to three lane bits (3, then 5, then 4) the lanes on one side
// keep the lower half of their values and the others the upper half, each
// adding its partner's copy of what it kept; one value a lane remains, which
// is summed over the remaining lane bits and read from one lane per b.
template <int B>
__device__ __forceinline__ void wave_sums(const float (&in)[B], float (&out)[B], int lane) {
  if constexpr (B == 1) {
    out[0] = wave_sum(in[0]);
  } else {
    constexpr int P = B <= 2 ? 2 : (B <= 4 ? 4 : 8);
    float v[P];
#pragma unroll
    for (int i = 0; i < P; i++) v[i] = i < B ? in[i] : 0.f;
    auto fold = [&](int n, bool upper, auto partner) {
#pragma unroll
      for (int i = 0; i < n / 2; i++) {
        const float keep = upper ? v[n / 2 + i] : v[i], give = upper ? v[i] : v[n / 2 + i];
        v[i] = keep + partner(give);
      }
    };
    fold(P, (lane & 8) != 0, [](float g) { return dpp_f<0x128>(g); });  // row_ror:8 = lane ^ 8 in a row
    if constexpr (P >= 4) fold(P / 2, (lane & 32) != 0, [&](float g) { return lane_xor<32>(g, (lane & 32) != 0); });
    if constexpr (P >= 8) fold(P / 4, (lane & 16) != 0, [&](float g) { return lane_xor<16>(g, (lane & 16) != 0); });
    float t = v[0];
    t += dpp_f<0xB1>(t);   // lane ^ 1
    t += dpp_f<0x4E>(t);   // lane ^ 2
    t += dpp_f<0x141>(t);  // 7 - lane within 8: the other quad
    if constexpr (P <= 4) t += lane_xor<16>(t, (lane & 16) != 0);
    if constexpr (P <= 2) t += lane_xor<32>(t, (lane & 32) != 0);
    // value index = bit 3 (P / 2) + bit 5 (P / 4) + bit 4 (P / 8) of the lane
#pragma unroll
    for (int b = 0; b < B; b++) {
      const int l = P == 8 ? ((b >> 2) << 3) | (((b >> 1) & 1) << 5) | ((b & 1) << 4)
                           : (P == 4 ? ((b >> 1) << 3) | ((b & 1) << 5) : b << 3);
      out[b] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), l));
    }
  }
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

// Row loads are raw buffer loads: a descriptor per plane and row (built in
// scalar registers), a per-lane offset fixed for the whole kernel and the
// tile as an immediate offset.  They are never conditional (a tile past the
// slice end lies outside the descriptor's range and reads as zeros without a
// memory access) and need no per-row vector address arithmetic, so the
// compiler counts outstanding loads exactly and keeps the next row in flight
// while the current one is decoded.
template <int SMAX>
__device__ __forceinline__ void load_row(RowBuf<SMAX>& R, const uint8_t* raw_p, const uint8_t* nib_p,
                                         const uint32_t* idx_p, uint64_t t0, uint32_t S, int lane) {
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(raw_p + t0 * kTile, S * kTile);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(nib_p + t0 * (kTile / 2), S * (kTile / 2));
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx_p + t0, (S + 1) * 4);
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    R.raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)lane * 16 + j * kTile, 0, kNonTemporal);
    R.nib[j] = __builtin_amdgcn_raw_buffer_load_b64(rn, (uint32_t)lane * 8 + j * (kTile / 2), 0, kNonTemporal);
  }
  R.ixv = __builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)lane * 4, 0, 0);
}

struct SegCtx {
  const uint8_t* esc_p;  // escape stream of the tensor
  const uint8_t* esc_sh; // LDS copy of escapes [e_lo, e_hi) when preloaded
  uint8_t* esc_wave;     // this wave's staging slot (kEscSlot bytes) otherwise
  uint32_t e_lo, e_hi;   // escape range of the workgroup's rows (clamped)
  Lut lut;
  uint32_t base4;
};

// Escape information of the S tiles held in one row buffer: where each
// tile's escapes start in the stream, how many there are, and (preloaded
// case, one or two escapes) their exponent bytes.  The index values are
// clamped into the range this workgroup knows, so a corrupt blob can only
// give wrong values, never an out-of-range access.
template <int SMAX, bool PRELOAD>
__device__ __forceinline__ void chunk_escapes(uint32_t ixv, uint32_t S, const SegCtx& C, uint32_t first[SMAX],
                                              uint32_t cnt[SMAX], uint32_t e1[SMAX], uint32_t e2[SMAX]) {
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)ixv, j);
    const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)ixv, j + 1);
    first[j] = min(max(ia, C.e_lo), C.e_hi);
    cnt[j] = min(min(max(ib, first[j]), C.e_hi) - first[j], (uint32_t)kTile);
    e1[j] = e2[j] = 0;
    if (PRELOAD && (uint32_t)j < S && cnt[j] != 0 && cnt[j] <= 2) {
      const uint32_t o = first[j] - C.e_lo;
      e1[j] = uniform(C.esc_sh[o]);
      e2[j] = cnt[j] == 2 ? uniform(C.esc_sh[o + 1]) : e1[j];
    }
  }
}

// Exponent bytes of one tile (PRELOAD: the segment's escapes sit in LDS, the
// common case; otherwise, dense escapes, each tile's slice is staged from
// memory when needed).
//
// A tile whose escapes all carry the same exponent (in practice: most tiles
// with one or two escapes) needs no per-weight placement: that exponent
// becomes the table entry of code 15 and the tile is decoded through the
// table like any other.  Only the remaining tiles take the rank-and-patch
// path.
template <bool CONTIG, bool PRELOAD>
__device__ __forceinline__ void tile_exponents(u32x2 nib, uint32_t first, uint32_t cnt, uint32_t e1, uint32_t e2,
                                               const SegCtx& C, uint32_t E[4]) {
  if (cnt == 0) {
    exponents16<CONTIG>(nib, C.lut, C.base4, E);
  } else if (PRELOAD && cnt <= 2 && e1 == e2) {
    const Lut L{C.lut.t0, C.lut.t1, C.lut.t2, (C.lut.t3 & 0x00FFFFFFu) | (e1 << 24)};
    exponents16<false>(nib, L, C.base4, E);
  } else {
    exponents16<CONTIG>(nib, C.lut, C.base4, E);
    if (PRELOAD) {
      uint64_t m0, m1;
      const uint32_t r = escape_rank(nib, m0, m1);
      patch_escapes(C.esc_sh + (first - C.e_lo), r, cnt, m0, m1, E);
    } else {
      place_escapes(nib, C.esc_p, first, cnt, C.esc_wave, E);
    }
  }
}

template <int B, int SMAX, bool CONTIG, bool PRELOAD>
__device__ __forceinline__ void row_dot(const RowBuf<SMAX>& R, uint32_t S, const uint32_t (*xr)[B][8],
                                        const SegCtx& C, float acc[B][2]) {
#pragma unroll
  for (int b = 0; b < B; b++) acc[b][0] = acc[b][1] = 0.f;
  uint32_t first[SMAX], cnt[SMAX], e1[SMAX], e2[SMAX];
  chunk_escapes<SMAX, PRELOAD>(R.ixv, S, C, first, cnt, e1, e2);
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    if ((uint32_t)j < S) {
      uint32_t E[4];
      tile_exponents<CONTIG, PRELOAD>(R.nib[j], first[j], cnt[j], e1[j], e2[j], C, E);
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
    float in[B], sum[B];
#pragma unroll
    for (int b = 0; b < B; b++) in[b] = acc[b][0] + acc[b][1];
    wave_sums<B>(in, sum, lane);
#pragma unroll
    for (int b = 0; b < B; b++)
      if (lane == 0) part[ul][wave][b] = (accumulate ? part[ul][wave][b] : 0.f) + sum[b];
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
__device__ __forceinline__ void run_segment(const GroupArg& G, const UnitInfo& U, uint32_t u_lo, uint32_t u_hi,
                                            bool y_bf16, float (*part)[kGemvWaves][B], uint8_t* esc_sh,
                                            uint8_t* esc_wave, uint32_t wave, int lane) {
  const uint32_t T = G.tiles;
  const uint32_t cols = T << 10;
  const uint32_t nks = U.nks, phases = U.phases;
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
  C.lut = header_lut(G.blob);
  C.base4 = (C.lut.t0 & 0xFFu) * 0x01010101u;
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
      if (n_mine) load_row<SMAX>(A, raw_p, nib_p, idx_p, row_tile0, S, lane);
      uint32_t xr[SMAX][B][8];
#pragma unroll
      for (int j = 0; j < SMAX; j++) {
        const uint32_t tj = tl + min((uint32_t)j, SL - 1);
#pragma unroll
        for (int b = 0; b < B; b++) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(G.x + (size_t)b * cols + (size_t)tj * kTile) + lane * 2;
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

// Batch 5..8 (one tile a K slice) is held to 128 VGPRs, four waves per SIMD:
// batch 8 would take 129 and drop to three (the layer at batch 8: 119 -> 110 us).
template <int B, int SMAX>
__global__ __launch_bounds__(kGemvWaves * kWave) __attribute__((amdgpu_waves_per_eu(B >= 5 ? 4 : 1)))
void k_gemv(GemvLaunch L) {
  __shared__ float part[kSubUnits][kGemvWaves][B];
  __shared__ uint8_t esc_sh[kEscShared];
  __shared__ __attribute__((aligned(16))) uint8_t esc_wave[kGemvWaves][kEscSlot];
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const int lane = lane_id();
  // this workgroup's share of the total cost: units whose start cost is in [c_lo, c_hi)
  const uint64_t c_lo = L.total_cost * blockIdx.x / gridDim.x;
  const uint64_t c_hi = L.total_cost * (blockIdx.x + 1) / gridDim.x;
  uint64_t g_lo = 0;  // cost of all earlier groups' units
  for (int gi = 0; gi < L.n_groups; gi++) {
    const GroupArg& G = L.g[gi];
    const UnitInfo U = unit_info(G);
    const uint64_t g_hi = g_lo + (uint64_t)U.n_units * U.unit_cost;
    if (g_lo >= c_hi) break;
    if (g_hi > c_lo) {
      const uint32_t u_lo = c_lo > g_lo ? (uint32_t)((c_lo - g_lo + U.unit_cost - 1) / U.unit_cost) : 0u;
      const uint32_t u_hi = (uint32_t)min((uint64_t)U.n_units, (c_hi - g_lo + U.unit_cost - 1) / U.unit_cost);
      if (u_lo < u_hi) {
        if (G.aux & kAuxContig)
          run_segment<B, SMAX, true>(G, U, u_lo, u_hi, L.y_bf16, part, esc_sh, esc_wave[wave], wave, lane);
        else
          run_segment<B, SMAX, false>(G, U, u_lo, u_hi, L.y_bf16, part, esc_sh, esc_wave[wave], wave, lane);
      }
    }
    g_lo = g_hi;
  }
}

template <int B, int SMAX>
static hipError_t run(GemvLaunch& L, hipStream_t s) {
  int per_cu = 0, cus = 0;
  hipError_t e = device_cus(&cus);
  if (e == hipSuccess)
    e = blocks_per_cu(reinterpret_cast<const void*>(&k_gemv<B, SMAX>), kGemvWaves * kWave, &per_cu);
  if (e != hipSuccess) return e;
  uint64_t units = 0;
  for (int g = 0; g < L.n_groups; g++) units += unit_info(L.g[g]).n_units;
  const uint64_t grid = std::min<uint64_t>((uint64_t)per_cu * cus, units);
  hipLaunchKernelGGL((k_gemv<B, SMAX>), dim3((unsigned)grid), dim3(kGemvWaves * kWave), 0, s, L);
  return hipGetLastError();
}

// ---- Ring GEMV (x of every tensor fits in LDS) ------------------------------
//
// The fastest form, used for batch 1..8 when x of every tensor of the call
// fits in LDS.  One 1024-thread workgroup per CU.  The unit of work is one
// row; rows of all tensors are dealt to the CUs cyclically (CU w takes rows
// w, w + #CUs, ...), so every CU gets the same mix, and inside a CU the 16
// waves take rows from a counter in LDS, so they finish together whatever
// their scheduling priority.  Waves share nothing but x (staged once in
// LDS) and never wait for each other.  Each wave streams its rows in chunks
// of up to 4 tiles through a ring of three chunk slots: while chunk i is
// decoded, the coded planes and the escape bytes of chunk i + 1 and the tile
// index of chunk i + 2 are in flight (the escape bytes need the index, the
// index needs nothing).  Every memory operation is issued unconditionally
// (a disabled one gets a zero-length buffer range) and the ring is unrolled
// by three, so the compiler counts outstanding loads exactly.
constexpr int kRingWaves = 16;  // waves per workgroup (4 per SIMD), every batch
// Ring geometry: tiles a chunk (the last of a row may be shorter) and chunks
// in the ring (N - 2 have their planes in flight while one is decoded).  Two
// tiles with four or five slots, or one tile with eight, measured slower:
// the per-chunk scalar work grows faster than the extra loads in flight help.
constexpr int kRingTiles = 4;
constexpr int kRingSlots = 3;
constexpr uint32_t kStageWaves = 8;  // batch 1: waves that stage x (the first two of each SIMD)
constexpr uint32_t kTailRows = 4;  // batch-1 tail: rows per wave rank a SIMD left to the earlier waves
constexpr uint32_t kRingXMax = 131072;  // x area; with the wave slots 144 KiB of the 160 KiB LDS

// Ring launch: the group records, rows dealt in record order (the launcher
// puts the longest rows first).  Team t is groups [team_g0[t],
// team_g0[t + 1]) and workgroups [wg_begin[t], wg_begin[t + 1]); its rows
// are a contiguous range of the launch's row space, dealt over its
// workgroups only, and each of its workgroups stages the x of its groups
// alone.  In each record's aux word, bit 1 marks the team's first group of
// each distinct x array (staged once) and bits 8..31 hold the LDS byte
// offset of the group's x (a multiple of 1024).
constexpr uint32_t kAuxStageX = 2u;
struct RingLaunch {
  GroupArg g[LBF_MAX_GROUPS];
  uint32_t gtab[LBF_MAX_GROUPS];  // group table entry of each group (group_entry)
  void* h;                        // gated product (g[0] = gate, g[1] = up): h[b, r] = silu(gate) * up
  uint32_t n_rows;
  int n_groups, n_teams, y_bf16;
  uint32_t wg_begin[LBF_MAX_GROUPS + 1];
  uint32_t team_g0[LBF_MAX_GROUPS + 1];
};
static_assert(sizeof(RingLaunch) <= 3584, "kernel arguments stay inside the 4 KiB limit");
static_assert(LBF_MAX_GROUPS <= 64, "the ring kernel keeps one group per lane");

template <int C>
struct Slot {
  u32x4 raw[C];
  u32x2 nib[C];
  uint32_t idxv;  // lane j: idx[t0 + j], j <= S
  uint32_t escv;  // lane p: escape p of the chunk's slice, p < 64
};

// Position of a chunk: tiles [c, c + S) of row r of group g (T tiles a row).
struct Pos {
  uint32_t g, r, c, S, T;
  bool valid;
};

__device__ __forceinline__ Planes ptrs_of(const GroupArg& G) {
  return planes_of(G.blob, (uint64_t)G.rows * G.tiles);
}

// Group table in one VGPR, lane g for group g (loaded once per kernel): the
// group's first global row (the launcher's prefix sum of the groups' rows)
// in bits 6..31 and its tiles per row minus one in bits 0..5; all ones past
// the last group.  The ring launcher guarantees tiles <= 64 (x fits in LDS)
// and fewer than 2^26 rows.
constexpr uint32_t kRingMaxRows = 1u << 26;
constexpr uint32_t group_entry(uint32_t first_row, uint32_t tiles) { return (first_row << 6) | (tiles - 1u); }

__device__ __forceinline__ uint32_t group_regs(const RingLaunch& L, int lane) {
  return lane < L.n_groups ? L.gtab[lane] : ~0u;
}

// Unit q of the launch: a row of one group, or (GATED) row q of the gate
// tensor followed by row q of the up tensor.  The group is the last one whose
// first row is at or before q (a ballot over the group table, no memory).
template <bool GATED, int C>
__device__ __forceinline__ Pos row_pos(const RingLaunch& L, uint32_t GR, uint32_t q) {
  Pos p;
  p.valid = q < L.n_rows;
  const uint32_t qq = p.valid ? q : L.n_rows - 1;
  const uint32_t g = GATED ? 0u : (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((GR >> 6) <= qq)) - 1u;
  const uint32_t e = GATED ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)GR, (int)g);
  p.g = g;
  p.r = GATED ? qq : qq - (e >> 6);
  p.T = GATED ? L.g[0].tiles : (e & 63u) + 1u;
  p.c = 0;
  p.S = p.valid ? min((uint32_t)C, p.T) : 0u;
  return p;
}

__device__ __forceinline__ uint64_t tile_of(const Pos& p) { return (uint64_t)p.r * p.T + p.c; }

template <int C>
__device__ __forceinline__ void load_idx(Slot<C>& s, const RingLaunch& L, const Pos& p, int lane) {
  const Planes P = ptrs_of(L.g[p.g]);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(P.idx + tile_of(p), p.valid ? (p.S + 1) * 4 : 0u);
  s.idxv = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)lane * 4, 0, 0);
}

// Escape slice of the chunk, from its index (already loaded).
template <int C>
__device__ __forceinline__ void load_esc(Slot<C>& s, const RingLaunch& L, const Pos& p, uint32_t& e_first,
                                         uint32_t& e_cnt, int lane) {
  const GroupArg& G = L.g[p.g];
  const Planes P = ptrs_of(G);
  const uint32_t hi = min((uint32_t)__builtin_amdgcn_readlane((int)s.idxv, (int)p.S), G.n_esc);
  e_first = min((uint32_t)__builtin_amdgcn_readlane((int)s.idxv, 0), hi);
  e_cnt = p.valid ? hi - e_first : 0u;
  const __amdgpu_buffer_rsrc_t re = make_rsrc(P.esc + e_first, min(e_cnt, 64u));
  s.escv = __builtin_amdgcn_raw_buffer_load_b8(re, (uint32_t)lane, 0, 0);
}

// Raw and nibble planes of the chunk (2 C loads; they need no index).
template <int C>
__device__ __forceinline__ void load_planes(Slot<C>& s, const RingLaunch& L, const Pos& p, int lane) {
  const Planes P = ptrs_of(L.g[p.g]);
  const uint64_t t0 = tile_of(p);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(P.raw + t0 * kTile, p.S * kTile);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(P.nib + t0 * (kTile / 2), p.S * (kTile / 2));
#pragma unroll
  for (int j = 0; j < C; j++) {
    s.raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)lane * 16 + j * kTile, 0, kNonTemporal);
    s.nib[j] = __builtin_amdgcn_raw_buffer_load_b64(rn, (uint32_t)lane * 8 + j * (kTile / 2), 0, kNonTemporal);
  }
}

template <int C>
__device__ __forceinline__ void load_data(Slot<C>& s, const RingLaunch& L, const Pos& p, uint32_t& e_first,
                                          uint32_t& e_cnt, int lane) {
  load_esc(s, L, p, e_first, e_cnt, lane);
  load_planes(s, L, p, lane);
}

// x of every group of [g_lo, g_hi) whose aux word says so, from memory
// straight into LDS (buffer loads to LDS: no registers, one wait before the
// barrier), at the LDS offset in its aux word.  In a group's x area, element
// (b, t, lane, half) is at ((b T + t) 2 + half) 1024 + 16 lane: 1 KiB block
// jj = (b T + t) 2 + half is one load instruction of a wave, lane l bringing
// the 16 bytes at x + b cols + t 1024 + 16 l + 8 half (bf16 elements).  The
// blocks of the range's x arrays, counted one after the other, go to the
// waves in turn.
template <int B, int W>
__device__ __forceinline__ void stage_x(const RingLaunch& L, uint8_t* smem, uint32_t g_lo, uint32_t g_hi,
                                        uint32_t wave, int lane) {
  uint32_t base = 0;  // blocks of the arrays before this one
  for (uint32_t g = g_lo; g < g_hi; g++) {
    const GroupArg& G = L.g[g];
    if (!(G.aux & kAuxStageX)) continue;  // uniform
    const uint32_t nb = (uint32_t)B * G.tiles * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(G.x, nb * (uint32_t)kTile);
    uint8_t* const dst = smem + (G.aux >> 8);
    for (uint32_t jj = (wave + W - base % W) % W; jj < nb; jj += W)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dst + (size_t)jj * kTile),
                                               16, (uint32_t)lane * 32u + (jj & 1u) * 16u, (jj >> 1) * 2048u, 0, 0);
    base += nb;
  }
}

// Exponent bytes of tile j of a chunk; the chunk's escapes are in escv (and,
// for the patch path, in the wave's LDS slot) unless the chunk holds more
// than 64 of them (dense: each tile's slice is staged from memory).
__device__ __forceinline__ void ring_exponents(u32x2 nib, const Lut& lut, uint32_t base4, bool contig, uint32_t n_esc,
                                               uint32_t ia, uint32_t ib, uint32_t escv, uint32_t e_first,
                                               uint32_t e_cnt, const uint8_t* esc_p, uint8_t* slot, uint32_t E[4]) {
  const bool dense = e_cnt > 64u;
  const uint32_t lo = dense ? 0u : e_first, hi = dense ? n_esc : e_first + e_cnt;
  const uint32_t first = min(max(ia, lo), hi);
  const uint32_t cnt = min(min(max(ib, first), hi) - first, (uint32_t)kTile);
  if (cnt == 0) {
    if (contig)
      exponents16<true>(nib, lut, base4, E);
    else
      exponents16<false>(nib, lut, base4, E);
    return;
  }
  if (!dense) {
    const uint32_t o = first - e_first;  // < 64 here
    const uint32_t e1 = (uint32_t)__builtin_amdgcn_readlane((int)escv, (int)o);
    const uint32_t e2 = cnt == 2 ? (uint32_t)__builtin_amdgcn_readlane((int)escv, (int)min(o + 1, 63u)) : e1;
    if (cnt <= 2 && e1 == e2) {
      const Lut L2{lut.t0, lut.t1, lut.t2, (lut.t3 & 0x00FFFFFFu) | (e1 << 24)};
      exponents16<false>(nib, L2, base4, E);
      return;
    }
  }
  if (contig)
    exponents16<true>(nib, lut, base4, E);
  else
    exponents16<false>(nib, lut, base4, E);
  if (!dense) {
    uint64_t m0, m1;
    const uint32_t rk = escape_rank(nib, m0, m1);
    patch_escapes(slot + (first - e_first), rk, cnt, m0, m1, E);
  } else {
    place_escapes(nib, esc_p, first, cnt, slot, E);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// One round of a ring of N slots: step(integral_constant<K>) for K = 0..N-1,
// stopping at the first that reports no further chunk.
template <int K, int N, class F>
__device__ __forceinline__ bool ring_round(F& f) {
  if constexpr (K == N) {
    return true;
  } else {
    if (!f(std::integral_constant<int, K>{})) return false;
    return ring_round<K + 1, N>(f);
  }
}

template <int B, int W, bool GATED, int C, int N, bool TEAMS>
__global__ __launch_bounds__(W * kWave) void k_gemv_ring(RingLaunch L) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const int lane = lane_id();
  uint8_t* slot_lds = smem + kRingXMax + wave * kEscSlot;
  uint32_t* lctr = reinterpret_cast<uint32_t*>(smem + kRingXMax + W * kEscSlot);
  // TEAMS: this workgroup's team, its groups, workgroups and rows (teams
  // ending at or before this workgroup counted by a ballot: a search loop
  // here costs the main loop registers).  Otherwise one team: every group,
  // every workgroup, every row.
  uint32_t g_lo = 0, g_hi = (uint32_t)L.n_groups, q0 = 0, n_wg = gridDim.x, row_hi = L.n_rows;
  if constexpr (TEAMS) {
    const uint32_t WB = lane < L.n_teams ? L.wg_begin[lane + 1] : ~0u;
    const uint32_t t = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(WB <= blockIdx.x));
    g_lo = L.team_g0[t];
    g_hi = L.team_g0[t + 1];
    const uint32_t wg0 = L.wg_begin[t];
    n_wg = L.wg_begin[t + 1] - wg0;
    row_hi = g_hi >= (uint32_t)L.n_groups ? L.n_rows : L.gtab[g_hi] >> 6;
    q0 = (L.gtab[g_lo] >> 6) + blockIdx.x - wg0;
  }
  // Start-up order.  Batch 1 (kChunkFirst): the group table, then the first
  // chunk's index words and planes, the first two escape slices as soon as
  // the index words are in, then x, so the planes stream while x is staged
  // and the first decode waits for nothing else (8B layer: 55.2 -> 54.6 us,
  // escape slices before x another 0.1 us, gate_proj 0.2 us; a single
  // tensor needs no table load).  Larger batches: x first, the group table
  // load after it and waited for with it (the first order costs gate_proj
  // at batch 4 half a microsecond, and the single-tensor shortcut pushes
  // those kernels past their registers).
  constexpr bool kChunkFirst = B == 1;
  if constexpr (!kChunkFirst) {
    stage_x<B, W>(L, smem, g_lo, g_hi, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t GR = GATED ? 0u  // the gated launch has one row space
                      : (kChunkFirst && L.n_groups == 1) ? (lane == 0 ? group_entry(0u, L.g[0].tiles) : ~0u)
                                                         : group_regs(L, lane);

  // rows of this CU: the team's row_lo + b + k * n_wg (b: the workgroup
  // within the team); the wave's first two come from k = wave, wave + 16,
  // the rest from the LDS counter (starts at 32)
  uint32_t k_static = 0;
  // Tail (batch 1, one team).  The four waves of a SIMD are served by the
  // memory pipeline in the order they issue: the first wave of each SIMD
  // gets its chunks back soonest and the fourth last (on the 8B layer they
  // decode about 17 against 10 chunks a launch, and the fourth ends 2-3 us
  // after the first).  So the waves after the first of their SIMD stop
  // taking rows kTailRows rows per rank before this CU's last row (a soft
  // limit: a row taken from the counter is always decoded), and the last
  // rows go to the waves that return them soonest (8B layer 54.4 -> 53.9 us,
  // gate_proj 18.9 -> 18.7 us, fused SwiGLU 32.5 -> 31.7 us).  Not with
  // teams, whose last rows can be the costliest (escape-dense tensors; 64
  // experts at batch 1: 110 -> 116 us), and not above batch 1, where the
  // extra registers spill.
  constexpr bool kTail = B == 1 && !TEAMS;
  uint32_t kcap = ~0u;
  if constexpr (kTail) {
    const uint32_t b = blockIdx.x, per = gridDim.x >> 3;
    const uint32_t cu = (gridDim.x & 7u) ? b : (b & 7u) * per + (b >> 3);
    const uint32_t n_k = row_hi > cu ? (row_hi - cu + gridDim.x - 1) / gridDim.x : 0u;  // rows k of this CU: k < n_k
    // the first wave of each SIMD takes rows until the counter runs out, so
    // every row is taken whatever the limits of the others
    kcap = (wave >> 2) == 0 ? ~0u : n_k - min(n_k, kTailRows * (wave >> 2));
  }
  auto next_row = [&]() -> Pos {
    uint32_t k;
    if (k_static < 2) {
      k = wave + W * k_static++;
    } else if constexpr (kTail) {
      uint32_t v = ~0u;
      if (lane == 0 && __hip_atomic_load(lctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kcap)
        v = atomicAdd(lctr, 1u);
      k = uniform(v);
      if (k == ~0u) return row_pos<GATED, C>(L, GR, L.n_rows);  // past this wave's limit: it stops
    } else {
      uint32_t v = 0;
      if (lane == 0) v = atomicAdd(lctr, 1u);
      k = uniform(v);
    }
    uint64_t q;
    if constexpr (TEAMS) {
      q = q0 + (uint64_t)k * n_wg;
    } else {
      // workgroups go round-robin over the 8 XCDs: give each XCD a contiguous
      // block of gridDim.x / 8 consecutive rows per round
      const uint32_t b = blockIdx.x, per = gridDim.x >> 3;
      const uint32_t cu = (gridDim.x & 7u) ? b : (b & 7u) * per + (b >> 3);
      q = cu + (uint64_t)k * gridDim.x;
    }
    return row_pos<GATED, C>(L, GR, q < row_hi ? (uint32_t)q : L.n_rows);
  };
  auto advance = [&](const Pos& p) -> Pos {
    if (p.valid && p.c + C < p.T) {
      Pos n = p;
      n.c = p.c + C;
      n.S = min((uint32_t)C, p.T - n.c);
      return n;
    }
    if (!p.valid) return p;
    if (GATED && p.g == 0) {  // the gate row is done: the same row of the up tensor
      Pos n = p;
      n.g = 1;
      n.c = 0;
      n.S = min((uint32_t)C, p.T);
      return n;
    }
    return next_row();
  };

  // ring of N slots: the chunk decoded at rotation K is in slot K; then the
  // planes and escapes of the next N - 2 chunks are in flight and the index
  // of the one after them
  Slot<C> sl[N];
  Pos pp[N];
  uint32_t ef[N], en[N];  // escape slice (first, count) of each slot's chunk
  static_assert(N == 3, "the start-up below fills a ring of three slots");
  // Start-up.  x is what every wave waits for first, and all CUs start at
  // once: requested together with the planes, x would queue behind the whole
  // chip's plane traffic (6-9 us).  So x (issued above, before the group
  // table) is awaited alone; then the index words and planes of the first
  // chunks go out together, and the escape slices once the index words are
  // in.  At batch 1 two chunks per wave are filled; larger batches have no
  // registers for a second one, which comes with the first step.
  constexpr int F = B == 1 ? 2 : 1;  // chunks filled at start-up
  pp[0] = next_row();  // the group table load is waited for here
  pp[1] = advance(pp[0]);
  if constexpr (kChunkFirst) {
    __builtin_amdgcn_sched_barrier(0);
    load_idx(sl[0], L, pp[0], lane);
    load_idx(sl[1], L, pp[1], lane);
    load_planes(sl[0], L, pp[0], lane);
    __builtin_amdgcn_sched_barrier(0);
    // the escape slices go out as soon as the index words are in (loads
    // complete in order: they were issued first) and before x, so that the
    // wait for x covers them: requested after x, they would queue behind
    // the whole chip's plane traffic and hold up the first decode
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * C));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < F; i++) load_esc(sl[i], L, pp[i], ef[i], en[i], lane);
    __builtin_amdgcn_sched_barrier(0);
    // x is staged by the first two waves of each SIMD only (the ones the
    // memory pipeline serves first); the others pass the barrier below
    // without waiting for their own first chunk, which the first decode
    // waits for (gate_proj 18.6 -> 18.25 us, 64 experts 110.2 -> 109.4 us)
    if (wave < kStageWaves) {
      stage_x<B, kStageWaves>(L, smem, g_lo, g_hi, wave, lane);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's x, the first chunk and the escapes are in
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's x is in LDS
    __builtin_amdgcn_sched_barrier(0);
    load_idx(sl[0], L, pp[0], lane);
    load_idx(sl[1], L, pp[1], lane);
    load_planes(sl[0], L, pp[0], lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (threadIdx.x == 0) *lctr = 2u * W;
  __syncthreads();
  if constexpr (!kChunkFirst) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * C));  // the index words are in
    __builtin_amdgcn_sched_barrier(0);
    // escapes before the second chunk's planes: loads complete in order, and
    // the first step needs only chunk 0
#pragma unroll
    for (int i = 0; i < F; i++) load_esc(sl[i], L, pp[i], ef[i], en[i], lane);
  }
  if constexpr (F == 2) load_planes(sl[1], L, pp[1], lane);

  float acc[B][2];
  float gsum[B];  // GATED: the finished gate sums of the current row
#pragma unroll
  for (int bb = 0; bb < B; bb++) acc[bb][0] = acc[bb][1] = gsum[bb] = 0.f;

  // one step: chunk p0 in `cur` is decoded; the next chunk p1 (index in
  // already) gets its escapes and planes (unless the start-up issued them);
  // the one after, p2, its index
  auto step = [&](auto rot, auto started) -> bool {
    constexpr int K = decltype(rot)::value, I1 = (K + N - 1) % N, I2 = (K + N - 2) % N;
    pp[I1] = advance(pp[I2]);
    load_idx(sl[I1], L, pp[I1], lane);
    if constexpr (!decltype(started)::value) load_data(sl[I2], L, pp[I2], ef[I2], en[I2], lane);
    Slot<C>& cur = sl[K];
    const Pos& p0 = pp[K];
    const uint32_t f0 = ef[K], n0 = en[K];
    const GroupArg& G = L.g[p0.g];
    const Planes P = ptrs_of(G);
    const uint8_t* x_g = smem + (G.aux >> 8);
    const Lut lut = header_lut(G.blob);
    const uint32_t base4 = (lut.t0 & 0xFFu) * 0x01010101u;
    slot_lds[lane] = (uint8_t)cur.escv;  // the chunk's escapes, for the patch path
    wave_lds_sync();
    // bit j: the index gives tile j escapes (lane j compares idx[t0 + j] with
    // idx[t0 + j + 1], fetched from lane j + 1 by a row shift); tiles without
    // escapes decode with no per-tile scalar work
    const uint32_t idx_up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cur.idxv, 0x101, 0xF, 0xF, false);
    const uint64_t esc_tiles = __builtin_amdgcn_ballot_w64((uint32_t)lane < p0.S && idx_up != cur.idxv);
    const bool contig = G.aux & kAuxContig;
#pragma unroll
    for (int j = 0; j < C; j++) {
      if ((uint32_t)j < p0.S) {
        // batch rows 0..kEarly-1: x read before the decode (hides the LDS
        // latency); the rest one row at a time after it (fewer live registers)
        constexpr int kEarly = B <= 4 ? B : 2;
        auto xload = [&](int bb, uint32_t* xv) {
          const uint8_t* xs = x_g + (size_t)((bb * p0.T + p0.c + j) * 2) * kTile + lane * 16;
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(xs);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(xs + kTile);
          xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
          xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
        };
        uint32_t xr[kEarly][8];
#pragma unroll
        for (int bb = 0; bb < kEarly; bb++) xload(bb, xr[bb]);
        uint32_t E[4];
        if ((esc_tiles >> j) & 1u) {
          const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)cur.idxv, j);
          const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)cur.idxv, j + 1);
          ring_exponents(cur.nib[j], lut, base4, contig, G.n_esc, ia, ib, cur.escv, f0, n0, P.esc, slot_lds, E);
        } else if (contig) {
          exponents16<true>(cur.nib[j], lut, base4, E);
        } else {
          exponents16<false>(cur.nib[j], lut, base4, E);
        }
        uint32_t w[8];
        assemble16(cur.raw[j], E, w);
#pragma unroll
        for (int bb = 0; bb < B; bb++) {
          uint32_t xl[8];
          if (bb < kEarly) {
#pragma unroll
            for (int q = 0; q < 8; q++) xl[q] = xr[bb < kEarly ? bb : 0][q];
          } else {
            xload(bb, xl);
          }
#pragma unroll
          for (int q = 0; q < 8; q++)
            acc[bb][q & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[q]),
                                                             __builtin_bit_cast(bf16x2, xl[q]), acc[bb][q & 1], false);
        }
      }
    }
    // row end: the sums of row p0.r are stored by lane 0 (range 0 otherwise)
    const bool row_end = p0.valid && p0.c + C >= p0.T;
    float v[B];
#pragma unroll
    for (int bb = 0; bb < B; bb++) v[bb] = 0.f;
    if (row_end) {
      float in[B];
#pragma unroll
      for (int bb = 0; bb < B; bb++) {
        in[bb] = acc[bb][0] + acc[bb][1];
        acc[bb][0] = acc[bb][1] = 0.f;
      }
      wave_sums<B>(in, v, lane);
    }
    // GATED: the gate row's sums wait in gsum; the up row's end stores
    // silu(gate) * up into h
    bool store = row_end;
    void* out = G.y;
    if (GATED) {
      if (row_end && p0.g == 0) {
#pragma unroll
        for (int bb = 0; bb < B; bb++) gsum[bb] = v[bb];
      }
      store = row_end && p0.g == 1;
      out = L.h;
#pragma unroll
      for (int bb = 0; bb < B; bb++) v[bb] = store ? silu(gsum[bb]) * v[bb] : 0.f;
    }
#pragma unroll
    for (int bb = 0; bb < B; bb++) {
      if (L.y_bf16) {
        const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<uint16_t*>(out) + (size_t)bb * G.rows + p0.r, store ? 2u : 0u);
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v[bb]), yr, (uint32_t)lane * 2, 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<float*>(out) + (size_t)bb * G.rows + p0.r, store ? 4u : 0u);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[bb]), yr, (uint32_t)lane * 4, 0, 0);
      }
    }
    wave_lds_sync();  // the slot is rewritten by the next chunk
    return pp[(K + 1) % N].valid;
  };
  auto steady = [&](auto rot) -> bool { return step(rot, std::false_type{}); };
  if constexpr (F == 2) {
    if (pp[0].valid && step(std::integral_constant<int, 0>{}, std::true_type{}) && ring_round<1, N>(steady))
      while (ring_round<0, N>(steady)) {
      }
  } else {
    if (pp[0].valid)
      while (ring_round<0, N>(steady)) {
      }
  }
}

// 16 waves a workgroup (4 per SIMD, <= 128 VGPRs each) for every batch:
// above batch 4 only two batch rows of x are read before a tile's decode and
// the others one at a time after it, which keeps batch 8 within 128 VGPRs.
template <int B, bool GATED = false, bool TEAMS = false>
static hipError_t run_ring_kernel(RingLaunch& L, hipStream_t s) {
  constexpr int W = kRingWaves, C = kRingTiles, N = kRingSlots;
  const uint32_t lds = kRingXMax + W * kEscSlot + 16;
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e == hipSuccess) e = open_dynamic_lds(reinterpret_cast<const void*>(&k_gemv_ring<B, W, GATED, C, N, TEAMS>), (int)lds);
  if (e != hipSuccess) return e;
  if (L.n_teams == 0) {  // one team: every group, one workgroup per CU
    L.n_teams = 1;
    L.team_g0[0] = 0;
    L.team_g0[1] = (uint32_t)L.n_groups;
    L.wg_begin[0] = 0;
    L.wg_begin[1] = (uint32_t)std::min<uint64_t>((uint64_t)cus, L.n_rows);
  }
  const uint32_t grid = L.wg_begin[L.n_teams];
  hipLaunchKernelGGL((k_gemv_ring<B, W, GATED, C, N, TEAMS>), dim3(grid), dim3(W * kWave), lds, s, L);
  return hipGetLastError();
}

hipError_t launch_gemv_gated(const GroupArg& gate, const GroupArg& up, int batch, void* h, int h_dtype,
                             hipStream_t s) {
  static_assert(kGatedMaxXBytes == kRingXMax, "the gated launch stages x in the ring kernel's LDS area");
  if ((uint64_t)batch * gate.tiles * kTile * 2 > kRingXMax) return hipErrorInvalidValue;  // x must fit in LDS
  RingLaunch L;
  L.g[0] = gate;
  L.g[1] = up;
  L.g[0].aux = (gate.aux & kAuxContig) | kAuxStageX;  // one x for both, at LDS offset 0
  L.g[1].aux = up.aux & kAuxContig;
  L.gtab[0] = L.gtab[1] = 0u;  // one row space (unused)
  L.n_rows = gate.rows;
  L.n_groups = 2;
  L.n_teams = 0;
  L.y_bf16 = h_dtype == LBF_BF16;
  L.h = h;
  switch (batch) {
    case 1: return run_ring_kernel<1, true>(L, s);
    case 2: return run_ring_kernel<2, true>(L, s);
    case 3: return run_ring_kernel<3, true>(L, s);
    case 4: return run_ring_kernel<4, true>(L, s);
    case 5: return run_ring_kernel<5, true>(L, s);
    case 6: return run_ring_kernel<6, true>(L, s);
    case 7: return run_ring_kernel<7, true>(L, s);
    default: return run_ring_kernel<8, true>(L, s);
  }
}

// Ring path if x of each group fits in LDS.  Groups, longest rows first,
// are cut into teams whose distinct x arrays fit in LDS together (one team
// when all of them do; as few as possible otherwise: a team's time is set
// by its workgroup count, and one workgroup more or less matters less the
// more a team has).  Each team gets workgroups in proportion to its cost
// (coded bytes, each escape counted as four: it is read, staged, ranked and
// placed; weights of 2 / 3 / 4 / 6 put the 64 escape-stress experts at
// batch 4 at 131 / 126 / 126 / 131 us and at batch 1 at 114 / 111 / 110 /
// 108 us), at least one and at most one a row; one workgroup per CU in all.
static hipError_t launch_ring(const GroupArg* groups, int n_groups, int batch, int y_dtype, bool& used,
                              hipStream_t s) {
  used = false;
  RingLaunch L;
  uint64_t rows = 0;
  // longest rows first: rows are handed out in this order, so the coarsest
  // units are taken early and the last ones are the shortest
  int order[LBF_MAX_GROUPS];
  for (int g = 0; g < n_groups; g++) order[g] = g;
  std::stable_sort(order, order + n_groups, [&](int a, int b) { return groups[a].tiles > groups[b].tiles; });
  int cus = 0;
  if (const hipError_t e = device_cus(&cus); e != hipSuccess) return e;
  int n_teams = 0;
  uint64_t x_bytes = 0;  // 64-bit: batch * cols * 2 can pass 2^32 for one very wide row
  uint64_t team_work[LBF_MAX_GROUPS] = {}, team_rows[LBF_MAX_GROUPS] = {};
  for (int g = 0; g < n_groups; g++) {
    const GroupArg& G = groups[order[g]];
    const uint64_t xb = (uint64_t)batch * G.tiles * kTile * 2;
    if (xb > kRingXMax) return hipSuccess;  // this x alone does not fit
    int same = -1;  // an earlier group of the current team with the same x array (pointer and width)
    for (int k = n_teams ? L.team_g0[n_teams - 1] : 0; k < g && same < 0; k++)
      if ((L.g[k].aux & kAuxStageX) && L.g[k].x == G.x && L.g[k].tiles == G.tiles) same = k;
    if (n_teams == 0 || (same < 0 && x_bytes + xb > kRingXMax)) {  // a new team
      L.team_g0[n_teams++] = (uint32_t)g;
      x_bytes = 0;
      same = -1;
    }
    L.g[g] = G;
    L.g[g].aux = G.aux & kAuxContig;
    if (same >= 0) {
      L.g[g].aux |= L.g[same].aux & ~0xFFu;
    } else {
      L.g[g].aux |= kAuxStageX | (uint32_t)(x_bytes << 8);
      x_bytes += xb;
    }
    if (rows + G.rows >= kRingMaxRows) return hipSuccess;
    L.gtab[g] = group_entry((uint32_t)rows, G.tiles);
    rows += G.rows;
    team_work[n_teams - 1] += (uint64_t)G.rows * G.tiles * (kTile + kTile / 2) + 4ull * G.n_esc;
    team_rows[n_teams - 1] += G.rows;
  }
  if (rows >= kRingMaxRows || rows == 0) return hipSuccess;
  L.team_g0[n_teams] = (uint32_t)n_groups;
  L.n_teams = n_teams;
  // workgroups: the CUs shared by cost, each team at least one and at most
  // one a row; what rounding leaves goes to the largest remainders
  uint64_t total = 0;
  for (int t = 0; t < n_teams; t++) total += team_work[t];
  uint32_t n_wg[LBF_MAX_GROUPS];
  uint64_t rem[LBF_MAX_GROUPS];
  uint64_t given = 0;
  for (int t = 0; t < n_teams; t++) {
    const uint64_t share = (uint64_t)cus * team_work[t];
    n_wg[t] = (uint32_t)std::min<uint64_t>(team_rows[t], std::max<uint64_t>(1, share / total));
    rem[t] = share % total;
    given += n_wg[t];
  }
  while (given < (uint64_t)cus) {
    int best = -1;
    for (int t = 0; t < n_teams; t++)
      if (n_wg[t] < team_rows[t] && (best < 0 || rem[t] > rem[best])) best = t;
    if (best < 0) break;
    n_wg[best]++;
    rem[best] = 0;
    given++;
  }
  uint32_t wg = 0;
  for (int t = 0; t < n_teams; t++) {
    L.wg_begin[t] = wg;
    wg += n_wg[t];
  }
  L.wg_begin[n_teams] = wg;
  L.n_rows = (uint32_t)rows;
  L.n_groups = n_groups;
  L.y_bf16 = y_dtype == LBF_BF16;
  L.h = nullptr;
  used = true;
  if (n_teams > 1) {
    switch (batch) {
      case 1: return run_ring_kernel<1, false, true>(L, s);
      case 2: return run_ring_kernel<2, false, true>(L, s);
      case 3: return run_ring_kernel<3, false, true>(L, s);
      case 4: return run_ring_kernel<4, false, true>(L, s);
      case 5: return run_ring_kernel<5, false, true>(L, s);
      case 6: return run_ring_kernel<6, false, true>(L, s);
      case 7: return run_ring_kernel<7, false, true>(L, s);
      default: return run_ring_kernel<8, false, true>(L, s);
    }
  }
  // one team: every workgroup deals every row (the kernel without teams)
  L.n_teams = 0;
  switch (batch) {
    case 1: return run_ring_kernel<1>(L, s);
    case 2: return run_ring_kernel<2>(L, s);
    case 3: return run_ring_kernel<3>(L, s);
    case 4: return run_ring_kernel<4>(L, s);
    case 5: return run_ring_kernel<5>(L, s);
    case 6: return run_ring_kernel<6>(L, s);
    case 7: return run_ring_kernel<7>(L, s);
    default: return run_ring_kernel<8>(L, s);
  }
}

hipError_t launch_gemv(const GroupArg* groups, int n_groups, int batch, int y_dtype, hipStream_t s) {
  // batch 8 is faster on the MFMA kernel (gate_proj 14336 x 4096: 25.8 against
  // 27.5 us; batch 5 and 6 are faster here), unless escapes are dense (its
  // escape path reads them one at a time) or a row is too wide for it
  if (batch == 8) {
    uint64_t n = 0, esc = 0;
    bool fits = true;
    for (int g = 0; g < n_groups; g++) {
      n += (uint64_t)groups[g].rows * groups[g].tiles * kTile;
      esc += groups[g].n_esc;
      fits = fits && groups[g].tiles <= kGemmMaxTiles;
    }
    if (fits && esc * 100 <= n) return launch_gemm(groups, n_groups, batch, y_dtype, s);
  }
  bool used = false;
  const hipError_t e = launch_ring(groups, n_groups, batch, y_dtype, used, s);
  if (used || e != hipSuccess) return e;
  // tiles a wave's K slice holds per pass: x of the slice sits in registers
  // (smax * batch * 8 VGPRs), so fewer tiles means more waves per SIMD (batch
  // 1: two tiles, 92 instead of 147 VGPRs, 64 experts 176 -> 146 us); at
  // batch 4, one tile when no row is wider than 4 tiles (64 experts of 4096
  // columns: 187 -> 168 us at five waves per SIMD instead of three), two
  // otherwise (a 14-tile down_proj is faster with two)
  static const int smax_of[9] = {0, 2, 2, 2, 2, 1, 1, 1, 1};
  uint32_t t_max = 0;
  for (int g = 0; g < n_groups; g++) t_max = std::max(t_max, groups[g].tiles);
  const uint32_t smax = batch == 4 && t_max <= 4 ? 1u : (uint32_t)smax_of[batch];
  GemvLaunch L;
  L.n_groups = n_groups;
  L.y_bf16 = y_dtype == LBF_BF16;
  uint64_t cost = 0;
  for (int g = 0; g < n_groups; g++) {
    L.g[g] = groups[g];
    L.g[g].aux = static_aux(groups[g], smax);
    const UnitInfo U = unit_info(L.g[g]);
    cost += (uint64_t)U.n_units * U.unit_cost;
  }
  L.total_cost = cost;
  switch (batch) {
    case 1: return run<1, 2>(L, s);
    case 2: return run<2, 2>(L, s);
    case 3: return run<3, 2>(L, s);
    case 4: return smax == 1 ? run<4, 1>(L, s) : run<4, 2>(L, s);
    case 5: return run<5, 1>(L, s);
    case 6: return run<6, 1>(L, s);
    case 7: return run<7, 1>(L, s);
    default: return run<8, 1>(L, s);
  }
}

}  // namespace lbf
