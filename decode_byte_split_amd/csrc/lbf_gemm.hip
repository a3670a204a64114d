// lbf_gemm.hip — fused decode + matrix product on bf16 MFMA for batch 9..256.
//
// Y[b, r] = sum_k W[r, k] X[b, k] with W decoded straight into the A operand
// of v_mfma_f32_16x16x32_bf16 (fp32 accumulation); nothing decoded touches
// memory.  (Coded weights stay in GPU memory and are rebuilt exactly in
// registers right before the multiply: "Lossless LLM Weight Compression vs
// 8-bit GGUF", section "What does 'lossless' mean for LLM weights?"; a fused
// decompression-GEMM is the prior art named in "How does this compare with
// prior lossless systems?".)
//
// At these batch sizes the product is still bound by reading the coded
// weights (2B flops per ~1.5 bytes), so the kernel is laid out like a stream:
//  - a workgroup is 4 waves; each wave owns one block of 16 rows for the
//    whole K and keeps the batch (up to 64 columns, 4 blocks of 16) in fp32
//    accumulators;
//  - MFMA operand layout (16x16x32): lane l holds A[l % 16][8 (l / 16) + s]
//    and B[8 (l / 16) + s][l % 16], s = 0..7, and D[4 (l / 16) + s][l % 16],
//    s = 0..3.  The sum over k does not care which physical column sits in
//    which k slot, so each lane loads the coded chunk it needs directly: lane
//    (i, q) = (l % 16, l / 16) of step k takes the 16-weight chunk
//    16 (k % 4) + 4 j + q (j = 0..3) of tile k / 4 of row i — per load
//    instruction 64 contiguous raw bytes of each of the 16 rows — and the x
//    operand is read from LDS with the same column order;
//  - a wave's 16 rows are 16 T consecutive tiles, so its tile index words and
//    its whole escape slice are contiguous: both are staged in LDS once, and
//    every tile's escape count and first escape come from there.  A tile
//    whose escapes all carry one exponent (0, 1, or 2 equal ones: nearly all
//    of them for trained weights) puts that exponent into the lane's own LUT
//    slot 15 and needs no ranking; otherwise the lane ranks its escapes
//    across the 4 lanes of its row with ds_bpermute and patches them from LDS;
//  - x is staged per step (256 columns of every batch row) in LDS, loaded
//    straight into it (buffer_load_dwordx4 ... lds: no registers): with 16
//    columns and K in two parts, every step's x at once before the loop when
//    it fits (a 4096-column tensor: 128 KB), and no barrier after; otherwise
//    up to 32 columns two steps at a time into four buffers, a barrier every
//    second step; above, one step ahead into two buffers, a barrier every
//    step (LDS holds no more at the occupancy the kernel runs at); each
//    row's 16-byte column chunks sit in slots XOR-swizzled by the row so the
//    operand reads are at most two-way bank conflicted; the coded chunks run
//    through a ring of four register slots (two steps in flight), which
//    keeps every column count at two waves per SIMD; every coded load is
//    issued unconditionally (invalid ones go out of the buffer range and
//    return 0).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kGemmWaves = 4;
constexpr int kGemmRows = 16 * kGemmWaves;     // rows per workgroup
constexpr int kGemmBatch = 64;                 // batch columns per launch
constexpr int kStepK = 256;                    // columns per pipeline step
constexpr int kXStride = kStepK * 2;           // LDS bytes per staged x row (16-byte chunks swizzled)
constexpr uint32_t kEscCap = 2048;             // escape bytes per wave held in LDS
constexpr uint32_t kOOB = 0x80000000u;         // a buffer offset past every range used here (all < 2^31)
constexpr uint32_t kFullXLds = 160 * 1024;     // LDS of one workgroup a CU

struct GemmLaunch {
  GroupArg g[LBF_MAX_GROUPS];
  uint32_t wg_begin[LBF_MAX_GROUPS + 1];  // first workgroup of each group
  uint32_t idx_bytes;                     // LDS bytes per wave for index words
  uint32_t x_steps;                       // XB == 0: x buffers (steps) staged up front
  int n_groups, batch, y_bf16;
};
static_assert(sizeof(GemmLaunch) <= 3072, "kernel arguments stay well inside the 4 KiB limit");

struct GSlot {
  u32x4 raw[4];
  u32x2 nib[4];
};

template <int NB, int S, int XB>
__global__ __launch_bounds__(kGemmWaves * S * kWave) void k_gemm(GemmLaunch L) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t rb = wave & 3u;  // row block of this wave
  const uint32_t kh = wave >> 2;  // its share of K: tiles kh, kh + S, kh + 2 S, ...
  const int lane = lane_id();
  const uint32_t li = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;

  uint32_t g = 0;
  while (g + 1 < (uint32_t)L.n_groups && L.wg_begin[g + 1] <= blockIdx.x) g++;
  const GroupArg& G = L.g[g];
  const uint32_t T = G.tiles;
  const uint32_t cols = T << 10;
  const Lut hl = header_lut(G.blob);  // the code table, from the blob's header copy
  const uint32_t lut0 = hl.t0, lut1 = hl.t1, lut2 = hl.t2, lut3 = hl.t3;
  const uint64_t n_tiles = (uint64_t)G.rows * T;
  const Planes P = planes_of(G.blob, n_tiles);
  const uint32_t r0 = (blockIdx.x - L.wg_begin[g]) * kGemmRows + rb * 16u;
  const uint32_t rows_here = r0 < G.rows ? min(16u, G.rows - r0) : 0u;
  const uint32_t tiles_here = rows_here * T;
  const uint64_t t_first = (uint64_t)r0 * T;

  constexpr uint32_t kXBuf = NB * 16 * kXStride;  // one K part's x of one step
  uint8_t* xs = smem;                             // [XB buffers][S parts][NB * 16 rows][kXStride]
  const uint32_t n_xbuf = XB ? (uint32_t)XB : L.x_steps;
  uint8_t* wl = smem + n_xbuf * S * kXBuf + rb * (L.idx_bytes + kEscCap);  // shared by the row block's waves
  uint32_t* idx_l = reinterpret_cast<uint32_t*>(wl);
  uint8_t* esc_l = wl + L.idx_bytes;

  // step k: round k / 4 (tiles (k / 4) S .. (k / 4) S + S - 1, one per K
  // part), columns 256 (k % 4) .. + 256 of each of them
  const uint32_t n_steps = 4 * ((T + S - 1) / S);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(P.raw + t_first * kTile, tiles_here * kTile);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(P.nib + t_first * (kTile / 2), tiles_here * (kTile / 2));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(G.x, (uint32_t)L.batch * cols * 2);

  // coded chunks of step k: lane (li, lq), chunk j -> tile c = (k / 4) S + kh
  // of row li, 16-weight chunk 16 (k % 4) + 4 j + lq.  The lane part of the
  // offset is fixed, the step part is uniform (scalar offset) and j goes in
  // the instruction's immediate; a step past the end gets a lane offset past
  // the range, and so do rows past the tensor, so every such load returns 0
  // whether or not the range check counts the scalar offset.
  const uint32_t vo_raw = li * T * kTile + lq * 16u;
  const uint32_t vo_nib = li * T * (kTile / 2) + lq * 8u;
  auto load_step = [&](GSlot& Sl, uint32_t k) {
    const uint32_t c = (k >> 2) * S + kh;
    const bool ok = k < n_steps && c < T;  // uniform
    const uint32_t vr = ok ? vo_raw : kOOB, vn = ok ? vo_nib : kOOB;
    const uint32_t sr = ok ? c * kTile + (k & 3u) * 256u : 0u;
    const uint32_t sn = ok ? c * (kTile / 2) + (k & 3u) * 128u : 0u;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      // default cache policy: a row's 128-byte lines are read by two or four
      // consecutive load instructions
      Sl.raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rr, vr + 64u * j, sr, 0);
      Sl.nib[j] = __builtin_amdgcn_raw_buffer_load_b64(rn, vn + 32u * j, sn, 0);
    }
  };
  // x of step k for every K part, loaded straight into LDS (no registers):
  // chunk P = 256 S m + threadIdx.x (16 bytes) is part h = P / (512 NB),
  // batch row (P / 32) % (16 NB) and slot s = P % 32 of that row, which holds
  // column chunk s ^ (row & 15) of the step's 256 columns; one instruction
  // fills 64 consecutive slots.  A part past the row's tiles gets zeros.
  auto dma_x = [&](uint32_t k, uint32_t buf) {
#pragma unroll
    for (int m = 0; m < NB * 2; m++) {
      const uint32_t p0 = 256u * S * m + uniform(threadIdx.x & ~63u);  // the wave's first chunk
      const uint32_t p = p0 + (uint32_t)lane;
      const uint32_t h = p0 / (512u * NB), pp = p % (512u * NB), row = pp >> 5, slot = pp & 31u;
      const uint32_t c = (k >> 2) * S + h;
      uint8_t* dst = xs + (buf * S + h) * kXBuf + (p0 % (512u * NB)) * 16u;
      if (c < T) {
        const uint32_t vo = row * cols * 2 + (slot ^ (row & 15u)) * 16u;
        const uint32_t so = (c * kTile + (k & 3u) * kStepK) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)dst, 16, vo, so, 0, 0);
      } else {
        *reinterpret_cast<u32x4*>(dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // issue order (loads retire in order): x of step 0, coded data 2 steps ahead
  GSlot s0, s1, s2, s3;
  if (XB == 0) {  // every step's x, once
    for (uint32_t k = 0; k < n_steps; k++) dma_x(k, k);
  } else {
    dma_x(0, 0);
    if (XB == 4 && 1 < n_steps) dma_x(1, 1);
  }
  load_step(s0, 0);
  load_step(s1, 1);

  // the row block's index words idx[t_first .. t_first + tiles_here] and
  // escape bytes (staged by its first wave), clamped to the stream so a
  // corrupt index stays in bounds
  uint32_t e_lo = 0, e_hi = 0, a0 = 0;
  bool dense = false;
  if (rows_here && kh == 0) {
    for (uint32_t w = (uint32_t)lane; w <= tiles_here; w += kWave) idx_l[w] = min(P.idx[t_first + w], G.n_esc);
    wave_lds_sync();
    e_lo = idx_l[0];
    e_hi = max(idx_l[tiles_here], e_lo);
    a0 = e_lo & ~3u;
    if (e_hi - a0 <= kEscCap) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(P.esc + a0);
      const uint32_t nw = (e_hi - a0 + 3) >> 2;
      for (uint32_t w = (uint32_t)lane; w < nw; w += kWave) reinterpret_cast<uint32_t*>(esc_l)[w] = src[w];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // x of step 0 is in LDS (every load of this wave done)
  __syncthreads();
  if (rows_here) {
    e_lo = idx_l[0];
    e_hi = max(idx_l[tiles_here], e_lo);
    a0 = e_lo & ~3u;
    dense = e_hi - a0 > kEscCap;
  }

  // slot of column chunk 8 j + 2 lq + h in row nb 16 + li: (8 j + 2 lq + h) ^ li
  // = 8 (j ^ (li >> 3)) + ((2 lq + h) ^ (li & 7)); byte offset 128 j + xsw[j & 1][h]
  const uint32_t sw_lo0 = ((2u * lq) ^ (li & 7u)) * 16u, sw_lo1 = ((2u * lq + 1u) ^ (li & 7u)) * 16u;
  const uint32_t flip = (li >> 3) * 128u;  // rows 8..15 of a block swap 128-byte groups 2i and 2i + 1
  const uint32_t xsw[2][2] = {{sw_lo0 + flip, sw_lo1 + flip}, {sw_lo0 - flip, sw_lo1 - flip}};
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per tile: first escape (absolute), count, the lane's LUT word 3 and
  // whether any row of the wave needs ranked escapes
  uint32_t t_ia = 0, t_cnt = 0, t3 = lut3, run = 0;
  bool any_slow = false, fast = true;
  // The main loop, instantiated twice: waves whose escape slice fits in LDS
  // read escapes there only; the rest ("dense" slices) read them from
  // memory.  Keeping the two apart leaves the common loop free of loads
  // whose completion the compiler cannot count.  Both run the same barriers.
  auto main_loop = [&](auto dense_tag) {
    constexpr bool DENSE = decltype(dense_tag)::value;
    auto esc_at = [&](uint32_t pos) -> uint32_t {  // pos absolute, in [e_lo, e_hi)
      if constexpr (DENSE)
        return (uint32_t)P.esc[pos];
      else
        return (uint32_t)esc_l[pos - a0];
    };

    // step k: x of step k + 2 and coded data of step k + 2 are issued, step k
    // is computed from slot `cur` and x buffer k % 2, and x of step k + 1
    // (issued a step earlier) goes to x buffer (k + 1) % 2.  A tile starts
    // every 4 steps (TILE_START).
    auto step = [&](GSlot& cur, GSlot& nx2, uint32_t k, auto tile_start) {
      // XB == 2: x of step k + 1 into the other buffer (read last in step
      // k - 1, before the barrier that ended it).  XB == 4: at even steps, x
      // of steps k + 2 and k + 3 into the buffers read in steps k - 2 and
      // k - 1; barriers only after odd steps.  Then coded data of step k + 2.
      const bool more = k + 1 < n_steps;
      if constexpr (XB == 0) {
      } else if constexpr (XB == 2) {
        if (more) dma_x(k + 1, (k + 1) & 1u);
      } else {
        if ((k & 1u) == 0) {
          if (k + 2 < n_steps) dma_x(k + 2, (k + 2) & 3u);
          if (k + 3 < n_steps) dma_x(k + 3, (k + 3) & 3u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_step(nx2, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(tile_start)::value) {
        const uint32_t c = (k >> 2) * S + kh;
        uint32_t ia = e_lo, ib = e_lo;
        if (li < rows_here && c < T) {
          ia = min(max(idx_l[li * T + c], e_lo), e_hi);
          ib = min(max(idx_l[li * T + c + 1], ia), e_hi);
        }
        t_ia = ia;
        t_cnt = ib - ia;
        const uint32_t e1 = t_cnt ? esc_at(ia) : 0u;
        const uint32_t e2 = t_cnt > 1 ? esc_at(ia + 1) : e1;
        fast = t_cnt == 0 || (t_cnt <= 2 && e1 == e2);
        t3 = fast ? ((lut3 & 0x00FFFFFFu) | (e1 << 24)) : lut3;
        any_slow = __builtin_amdgcn_ballot_w64(!fast) != 0;
        run = 0;
      }
      const Lut lut{lut0, lut1, lut2, t3};
      const uint8_t* xb = xs + ((XB ? k % (XB ? XB : 1) : k) * S + kh) * kXBuf + li * kXStride;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint32_t E[4];
        exponents16<false>(cur.nib[j], lut, 0u, E);
        if (any_slow) {
          uint64_t m0 = fast ? 0 : escape_mask8(cur.nib[j].x);
          uint64_t m1 = fast ? 0 : escape_mask8(cur.nib[j].y);
          const uint32_t cl = (uint32_t)(__builtin_popcountll(m0) + __builtin_popcountll(m1));
          // most chunks of a ranked tile hold none of its escapes
          if (__builtin_amdgcn_ballot_w64(cl != 0) != 0) {
            uint32_t pre = 0, tot = 0;
#pragma unroll
            for (uint32_t q = 0; q < 4; q++) {
              const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((li + 16u * q) * 4u), (int)cl);
              pre += q < lq ? v : 0u;
              tot += v;
            }
            uint32_t pos = run + pre;
            run += tot;
            while (m0) {
              const uint32_t w = (uint32_t)__builtin_ctzll(m0) >> 3;
              patch_exponent(E, w, pos < t_cnt ? esc_at(t_ia + pos) : 0u);
              m0 &= m0 - 1;
              pos++;
            }
            while (m1) {
              const uint32_t w = 8u + ((uint32_t)__builtin_ctzll(m1) >> 3);
              patch_exponent(E, w, pos < t_cnt ? esc_at(t_ia + pos) : 0u);
              m1 &= m1 - 1;
              pos++;
            }
          }
        }
        uint32_t w[8];
        assemble16(cur.raw[j], E, w);
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]});
#pragma unroll
          for (int nb = 0; nb < NB; nb++) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xb + nb * 16 * kXStride + j * 128 + xsw[j & 1][h]);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, xv), acc[nb], 0, 0, 0);
          }
        }
      }
      // this wave's x of step k + 1 has landed (only the 8 coded loads of
      // step k + 2 are younger); the barrier makes every wave's visible
      if constexpr (XB == 0) {
        (void)more;
      } else if constexpr (XB == 2) {
        if (more) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
        __syncthreads();
      } else if (k & 1u) {
        // x of steps k + 1, k + 2 issued at step k - 1, before the coded
        // loads of steps k + 1 and k + 2 (16 younger loads)
        if (more) __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
        __syncthreads();
      }
    };

    // n_steps is a multiple of 4: one iteration is one tile
    for (uint32_t k = 0; k < n_steps; k += 4) {
      step(s0, s2, k, std::true_type{});
      step(s1, s3, k + 1, std::false_type{});
      step(s2, s0, k + 2, std::false_type{});
      step(s3, s1, k + 3, std::false_type{});
    }
  };
  if (dense)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  // K parts: the row block's later waves hand their sums to its first wave
  // through LDS (the x buffers are free after the last barrier), which adds
  // them in part order
  if constexpr (S > 1) {
    if constexpr (XB == 0) __syncthreads();  // no wave still reads the x buffers the sums go into
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    if (kh > 0) {
#pragma unroll
      for (int nb = 0; nb < NB; nb++) red[(((kh - 1) * 4 + rb) * NB + nb) * kWave + lane] = acc[nb];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (uint32_t h = 1; h < (uint32_t)S; h++)
#pragma unroll
      for (int nb = 0; nb < NB; nb++) acc[nb] += red[(((h - 1) * 4 + rb) * NB + nb) * kWave + lane];
  }

  // lane (li, lq) of block nb holds Y[nb*16 + li][r0 + 4 lq + s], s = 0..3;
  // values and offsets are formed first, the stores follow in straight-line
  // code (one branch on the output type, outside the loops)
  const uint32_t eb = L.y_bf16 ? 2u : 4u;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(G.y, (uint32_t)L.batch * G.rows * eb);
  uint32_t off[NB][4], val[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const uint32_t b = nb * 16u + li;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t r = r0 + 4u * lq + s;
      off[nb][s] = (b < (uint32_t)L.batch && r < G.rows) ? (b * G.rows + r) * eb : kOOB;
      const float v = acc[nb][s];  // element copy first: a bit_cast of acc[nb][s] itself reads element 0
      val[nb][s] = __builtin_bit_cast(uint32_t, v);
    }
  }
  if (L.y_bf16) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int s = 0; s < 4; s++)
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(__builtin_bit_cast(float, val[nb][s])), ry, off[nb][s], 0, 0);
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int s = 0; s < 4; s++) __builtin_amdgcn_raw_buffer_store_b32(val[nb][s], ry, off[nb][s], 0, 0);
  }
}

template <int NB, int S, int XB = (NB <= 2 ? 4 : 2)>
static hipError_t run_gemm(const GemmLaunch& L, uint32_t grid, hipStream_t s) {
  const int n_xbuf = XB ? XB : (int)L.x_steps;
  const int lds = n_xbuf * S * NB * 16 * kXStride + kGemmWaves * (int)(L.idx_bytes + kEscCap);
  const hipError_t e = open_dynamic_lds(reinterpret_cast<const void*>(&k_gemm<NB, S, XB>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm<NB, S, XB>), dim3(grid), dim3(kGemmWaves * S * kWave), lds, s, L);
  return hipGetLastError();
}

// Batch columns go in slabs of up to 64 (each slab re-reads the coded
// weights); a slab of m columns runs ceil(m / 16) MFMA column blocks.
hipError_t launch_gemm(const GroupArg* groups, int n_groups, int batch, int y_dtype, hipStream_t s) {
  const uint32_t eb = y_dtype == LBF_BF16 ? 2u : 4u;
  for (int b0 = 0; b0 < batch; b0 += kGemmBatch) {
    const int nb = std::min(kGemmBatch, batch - b0);
    GemmLaunch L;
    L.n_groups = n_groups;
    L.batch = nb;
    L.y_bf16 = y_dtype == LBF_BF16;
    uint32_t wg = 0, t_max = 1, t_min = kGemmMaxTiles;
    for (int g = 0; g < n_groups; g++) {
      GroupArg G = groups[g];
      if (G.tiles > kGemmMaxTiles) return hipErrorNotSupported;
      G.x += (size_t)b0 * G.tiles * kTile;
      G.y = static_cast<uint8_t*>(G.y) + (size_t)b0 * G.rows * eb;
      L.g[g] = G;
      L.wg_begin[g] = wg;
      wg += (G.rows + kGemmRows - 1) / kGemmRows;
      t_max = std::max(t_max, G.tiles);
      t_min = std::min(t_min, G.tiles);
    }
    L.wg_begin[n_groups] = wg;
    L.idx_bytes = (4 * (16 * t_max + 1) + 15) & ~15u;
    // rows of two or more tiles split K over two waves per row block (8
    // waves a workgroup, two per SIMD): a gate-sized tensor has too few
    // 16-row blocks to fill the chip otherwise (at 64 columns the split
    // takes gate_proj from 46 to 37 us)
    const bool split = t_min >= 2;
    L.x_steps = 0;
    const bool full_x = 4u * ((t_max + 1) / 2) * 2 * 16 * kXStride + kGemmWaves * (L.idx_bytes + kEscCap) <= kFullXLds;
    hipError_t e;
    switch ((nb + 15) / 16) {
      case 1:
        // 16 columns, K split in two: every step's x staged once when it fits
        // beside the escape staging (4096 columns: 128 KB), no barriers after
        if (split && full_x) {
          L.x_steps = 4 * ((t_max + 1) / 2);
          e = run_gemm<1, 2, 0>(L, wg, s);
        } else {
          e = split ? run_gemm<1, 2>(L, wg, s) : run_gemm<1, 1>(L, wg, s);
        }
        break;
      case 2: e = split ? run_gemm<2, 2>(L, wg, s) : run_gemm<2, 1>(L, wg, s); break;
      case 3: e = split ? run_gemm<3, 2>(L, wg, s) : run_gemm<3, 1>(L, wg, s); break;
      default: e = split ? run_gemm<4, 2>(L, wg, s) : run_gemm<4, 1>(L, wg, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lbf
