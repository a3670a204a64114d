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
// weights (2B flops per ~1.5 bytes), so the kernel is a stream with no
// synchronisation inside it:
//  - a workgroup covers up to 64 rows (four MFMA row blocks of 16) of one
//    tensor with 8 waves; the host sizes the row share so that a
//    single-tensor launch has one workgroup per compute unit where it can
//    (14336 rows: 256 workgroups of 56).  With one block of 16 batch
//    columns the registers allow four waves a SIMD: a workgroup then covers
//    up to 32 rows (two row blocks) and each compute unit holds two
//    (14336 rows: 512 workgroups of 28); more waves a SIMD hide more of the
//    memory latency (gate_proj at batch 8: 25.5 -> 23.2 us).  Wave w owns the half-tiles w,
//    w + 8, ... of K (columns [512 h, 512 h + 512) of every row), so the
//    waves share nothing until the end, where their partial sums are added
//    through LDS in wave order (a fixed order: bitwise reproducible);
//  - MFMA operand layout (16x16x32): lane l holds A[l % 16][8 (l / 16) + s]
//    and B[8 (l / 16) + s][l % 16], s = 0..7, and D[4 (l / 16) + s][l % 16],
//    s = 0..3.  The sum over k does not care which physical column sits in
//    which k slot, so a step is 128 columns and lane (i, q) = (l % 16, l / 16)
//    takes 32 consecutive columns 32 q .. 32 q + 31 of row i of every row
//    block: two 16-byte raw loads and one 16-byte nibble load, i.e. each
//    row's whole 128-byte raw line and half its nibble line in one step.
//    MFMA h (0..3) of a row block takes the lane's weights 8 h .. 8 h + 7;
//  - x of a step goes through the wave's own LDS slot: buffer-to-LDS loads
//    in which each lane quad reads 64 contiguous bytes of one x row (lanes
//    in the MFMA layout would each read 16 bytes of a different row, about
//    four times the address work for the same bytes), placed so that the
//    B-operand reads hit 16 different bank groups.  At the start of a step
//    the wave copies its x into registers, and the slot takes the next
//    step's x at once, a whole step before it is needed.  Each wave reads
//    only the x of its own columns: nothing is shared, no barrier;
//  - escapes: per row and half-tile, one lane a row loads the tile's index
//    words and its first four escape bytes ahead of time.  A tile whose
//    escapes all carry one exponent (none, or up to four equal ones: nearly
//    all tiles of trained weights) puts it into the row's LUT slot 15;
//    otherwise the escapes of a step are ranked across the row's four lanes
//    (ds_bpermute) and taken from those four bytes, or, past them, from the
//    escape stream.  The rank needs the tile's escapes before the step: the
//    first half-tile walks forward and counts them; the second walks
//    backward, counting those after the step, and takes the rest from the
//    tile's total, so no wave needs another's count;
//  - the coded data runs through a ring of D register sets (D = 2 up to 48
//    batch columns, 1 at 64 for lack of registers): a row block is decoded,
//    its registers take its chunks of step k + D, and then it is
//    multiplied, so D steps are in flight.  Only those coded loads follow a
//    step's x loads, which fixes the count the step's wait for x uses.
//    Loads past the wave's last step get an offset past their range and
//    return 0 without a memory access.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kGemmWaves = 8;                       // waves per workgroup, one share of the half-tiles each
constexpr uint32_t kGemmMinRows = 16;               // rows per workgroup at least (unless the tensor is smaller)
constexpr int kGemmBatch = 64;                      // batch columns per launch
constexpr uint32_t kGemmStep = 128;                 // columns per step
constexpr uint32_t kHalfSteps = kTile / 2 / kGemmStep;  // steps per half-tile (4)
constexpr uint32_t kOOB = 0x80000000u;              // a buffer offset past every range used here (all < 2^31)
constexpr uint32_t kAuxRowsShift = 8;               // GroupArg::aux >> 8: rows per workgroup

struct GemmLaunch {
  GroupArg g[LBF_MAX_GROUPS];
  uint32_t wg_begin[LBF_MAX_GROUPS + 1];  // first workgroup of each group
  int n_groups, batch, y_bf16;
};
static_assert(sizeof(GemmLaunch) <= 3072, "kernel arguments stay well inside the 4 KiB limit");

// One step's coded chunks for one lane: per row block, weights 0..15 and
// 16..31 of its 32 columns (raw) and their 32 codes (nibbles).
template <int RB>
struct Coded {
  u32x4 raw0[RB], raw1[RB], nib[RB];
};

// 16 bytes a lane from a buffer straight into LDS: lane l's bytes land at
// LDS byte address lds + 16 l.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voffset,
                                              uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voffset,
                                           soffset, 0, 0);
}

// RB row blocks of 16 a wave: RB = 4 with two waves a SIMD (one workgroup
// a compute unit), RB = 2 with four (two workgroups a compute unit, more
// waves to cover memory latency; used for one block of batch columns, where
// the registers allow it).
template <int NB, int D, int RB>
__global__ __launch_bounds__(kGemmWaves * kWave) __attribute__((amdgpu_waves_per_eu(RB == 2 ? 4 : 1)))
void k_gemm(GemmLaunch L) {
  constexpr int kGemmRB = RB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // the waves' partial sums
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const int lane = lane_id();
  const uint32_t li = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;

  uint32_t g = 0;
  while (g + 1 < (uint32_t)L.n_groups && L.wg_begin[g + 1] <= blockIdx.x) g++;
  const GroupArg& G = L.g[g];
  const uint32_t T = G.tiles, cols = T << 10;
  const Planes P = planes_of(G.blob, (uint64_t)G.rows * T);
  const Lut lut = header_lut(G.blob);
  const uint32_t rpw = G.aux >> kAuxRowsShift;
  const uint32_t r0 = (blockIdx.x - L.wg_begin[g]) * rpw;
  const uint32_t rows_here = min(rpw, G.rows - r0);  // >= 1
  const uint32_t n_rb = (rows_here + 15u) >> 4;

  // Buffer ranges: the coded rows of each row block and the x rows of each
  // block of 16 batch columns.  The lane's part of every offset (row,
  // column chunk, x row) is in the vector offset and lies past the range
  // for rows and batch columns that do not exist, so those loads return 0
  // whether or not the range check counts the step's scalar offset.
  __amdgpu_buffer_rsrc_t rr[kGemmRB], rn[kGemmRB], rx[NB];
#pragma unroll
  for (int rb = 0; rb < kGemmRB; rb++) {
    const uint32_t lo = min(16u * rb, rows_here), n = min(16u, rows_here - lo);
    rr[rb] = make_rsrc(P.raw + ((uint64_t)r0 + lo) * T * kTile, n * T * kTile);
    rn[rb] = make_rsrc(P.nib + ((uint64_t)r0 + lo) * T * (kTile / 2), n * T * (kTile / 2));
  }
#pragma unroll
  for (int cb = 0; cb < NB; cb++) {
    const uint32_t lo = min(16u * cb, (uint32_t)L.batch), n = min(16u, (uint32_t)L.batch - lo);
    rx[cb] = make_rsrc(G.x + (size_t)lo * cols, n * cols * 2u);
  }
  const uint32_t vo_raw = li * T * kTile + lq * 32u, vo_nib = li * T * (kTile / 2) + lq * 16u;

  // This wave's steps: half-tiles ht = wave + 8 j (tile ht / 2, half ht % 2),
  // four steps each; the second half of a tile is walked backward.
  const uint32_t n_half = 2u * T;
  const uint32_t n_mine = wave < n_half ? (n_half - wave + kGemmWaves - 1) / kGemmWaves : 0u;
  const uint32_t n_steps = n_mine * kHalfSteps;
  auto col0_of = [&](uint32_t k) -> uint32_t {  // first column of step k
    const uint32_t ht = wave + kGemmWaves * (k / kHalfSteps), s = k % kHalfSteps;
    const uint32_t half = ht & 1u;
    return (ht >> 1) * kTile + half * (kTile / 2) + (half ? kHalfSteps - 1 - s : s) * kGemmStep;
  };
  auto load_block = [&](Coded<RB>& C, int rb, uint32_t k) {
    const bool ok = k < n_steps;  // uniform
    const uint32_t c0 = ok ? col0_of(k) : 0u;
    const uint32_t vr = ok ? vo_raw : kOOB, vn = ok ? vo_nib : kOOB;
    C.raw0[rb] = __builtin_amdgcn_raw_buffer_load_b128(rr[rb], vr, c0, 0);
    C.raw1[rb] = __builtin_amdgcn_raw_buffer_load_b128(rr[rb], vr + 16u, c0, 0);
    C.nib[rb] = __builtin_amdgcn_raw_buffer_load_b128(rn[rb], vn, c0 / 2u, 0);
  };
  // x of a step goes through this wave's LDS slot: per block of 16 batch
  // columns, four buffer-to-LDS loads (no registers), each lane quad reading
  // 64 contiguous bytes of one x row (a quarter of the 128 columns).  Load i
  // lane (a, h) = (l / 4, l % 4) takes the 16 bytes of columns 32 (a / 4) +
  // 8 h of x row 4 (a % 4) + i; load i lands at i * 1040 bytes into the
  // block's 4160-byte area.  The B operand of MFMA h for lane (n, q) is then
  // at (n % 4) * 1040 + 64 (4 q + n / 4) + 16 h: the 16 lanes of a row of
  // the wave read 16 different 16-byte bank groups.
  constexpr uint32_t kXLoad = 1040, kXBlock = 4 * kXLoad;
  uint8_t* const xw = smem + wave * (NB * kXBlock);
  const uint32_t vo_xd = (4u * ((uint32_t)lane >> 2 & 3u)) * cols * 2u + 64u * ((uint32_t)lane >> 4) + 16u * ((uint32_t)lane & 3u);
  const uint32_t rd_x = (li & 3u) * kXLoad + 64u * (4u * lq + (li >> 2));
  auto dma_x = [&](uint32_t k) {
    const uint32_t c0 = col0_of(k), vx = vo_xd;
    // the slot address is formed here from one register rather than kept
    // for every load in scalar registers across the loop
    uint32_t xb = (uint32_t)(uintptr_t)xw;
    asm volatile("" : "+s"(xb));
#pragma unroll
    for (int cb = 0; cb < NB; cb++)
#pragma unroll
      for (uint32_t i = 0; i < 4; i++)
        load16_to_lds(rx[cb], xb + cb * kXBlock + i * kXLoad, vx + i * cols * 2u, c0 * 2u);
  };

  // Escape facts, loaded ahead in every step (the same loads each step, so
  // no register is loaded on one path only).  Lane l < rows_here owns row
  // r0 + l.  After step k's loads, nx_a / nx_b are the index words of the
  // tile of half-tile hb(k + 2) (hb(j): the half-tile of step j) and
  // e_first / e_cnt / e_byte the first escape, count and first four escape
  // bytes of hb(k + 1)'s tile; cur_* are those of the current half-tile.
  const __amdgpu_buffer_rsrc_t ridx = make_rsrc(P.idx + (uint64_t)r0 * T, (rows_here * T + 1u) * 4u);
  const __amdgpu_buffer_rsrc_t resc = make_rsrc(P.esc, G.n_esc);
  uint32_t nx_a = 0, nx_b = 0, e_first = 0, e_cnt = 0, cur_first = 0, cur_cnt = 0, cur_e = 0;
  uint32_t e_byte[4] = {0, 0, 0, 0};
  uint32_t t3[kGemmRB], run[kGemmRB];
  uint32_t fastm = 0, slow_rb = 0;  // bit rb: the lane's row of block rb is on the LUT path / some row of rb is not
  auto meta_idx = [&](uint32_t k) {  // index words of hb(k)
    const uint32_t ht = wave + kGemmWaves * (k / kHalfSteps);
    const uint32_t vi = (ht < n_half && (uint32_t)lane < rows_here) ? ((uint32_t)lane * T + (ht >> 1)) * 4u : kOOB;
    nx_a = __builtin_amdgcn_raw_buffer_load_b32(ridx, vi, 0, 0);
    nx_b = __builtin_amdgcn_raw_buffer_load_b32(ridx, vi + 4u, 0, 0);
  };
  auto meta_esc = [&]() {  // escape facts from nx_a / nx_b
    // clamped so that a corrupt index reads nothing outside the stream
    const uint32_t b = min(nx_b, G.n_esc), a = min(nx_a, b);
    const uint32_t cnt = min(b - a, (uint32_t)kTile);
    // four separate bytes, combined only when taken: nothing waits for them here
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) e_byte[j] = __builtin_amdgcn_raw_buffer_load_b8(resc, j < cnt ? a + j : kOOB, 0, 0);
    e_first = a;
    e_cnt = cnt;
  };
  auto meta_take = [&]() {
    cur_first = e_first;
    cur_cnt = e_cnt;
    cur_e = e_byte[0] | e_byte[1] << 8 | e_byte[2] << 16 | e_byte[3] << 24;
    // from here on these are plain register values: their loads are waited
    // for once, here, and no later use (in loops, at joins) waits for the
    // memory pipeline again
    asm volatile("" : "+v"(cur_first), "+v"(cur_cnt), "+v"(cur_e));
    const uint32_t e0 = cur_e & 0xFFu;
    const uint32_t mask = cur_cnt >= 4 ? ~0u : (1u << (8 * cur_cnt)) - 1u;
    const bool fast = cur_cnt == 0 || (cur_cnt <= 4 && ((cur_e ^ (e0 * 0x01010101u)) & mask) == 0);
    const uint32_t word = e0 | (fast ? 0x100u : 0u);
    fastm = 0;
    slow_rb = 0;
#pragma unroll
    for (int rb = 0; rb < kGemmRB; rb++) {
      const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((16u * rb + li) * 4u), (int)word);
      const bool f = (v & 0x100u) != 0;
      t3[rb] = f ? ((lut.t3 & 0x00FFFFFFu) | ((v & 0xFFu) << 24)) : lut.t3;
      fastm |= f ? 1u << rb : 0u;
      slow_rb |= __builtin_amdgcn_ballot_w64(!f) != 0 ? 1u << rb : 0u;
      run[rb] = 0;
    }
  };

  f32x4 acc[kGemmRB][NB];
#pragma unroll
  for (int rb = 0; rb < kGemmRB; rb++)
#pragma unroll
    for (int cb = 0; cb < NB; cb++) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step: the escape facts ahead, this step's x into registers (the
  // slot then takes the next step's x at once), then per row block: decode,
  // reload the block's registers for step k + D, multiply.
  auto step = [&](Coded<RB>& C, uint32_t k) {
    const bool backward = ((wave + kGemmWaves * (k / kHalfSteps)) & 1u) != 0;
    if (k % kHalfSteps == 0) meta_take();  // a new half-tile: its escape facts
    // only the 3 * kGemmRB coded loads of the last step were issued after
    // x of step k (b128 / b128 / b128 per block: the compiler cannot merge
    // them), so x and everything older has landed once at most that many
    // are outstanding
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kGemmRB));
    wave_lds_sync();
    u32x4 X[NB][4];
#pragma unroll
    for (int cb = 0; cb < NB; cb++)
#pragma unroll
      for (int h = 0; h < 4; h++) X[cb][h] = *reinterpret_cast<const u32x4*>(xw + cb * kXBlock + rd_x + 16u * h);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): x is in registers, the slot is free
    __builtin_amdgcn_sched_barrier(0);
    // escape facts ahead, then the next step's x: both older than the coded
    // loads of this step
    meta_esc();
    meta_idx(k + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (k + 1 < n_steps) dma_x(k + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < kGemmRB; rb++) {
      uint32_t w[16];
      const bool live = rb == 0 || (uint32_t)rb < n_rb;  // uniform
      if (live) {
        const Lut lr{lut.t0, lut.t1, lut.t2, t3[rb]};
        uint32_t E0[4], E1[4];
        exponents16<false>(u32x2{C.nib[rb].x, C.nib[rb].y}, lr, 0u, E0);
        exponents16<false>(u32x2{C.nib[rb].z, C.nib[rb].w}, lr, 0u, E1);
        if ((slow_rb >> rb) & 1u) {
          // ranked escapes; lanes of rows on the LUT path count none
          const int src = (int)((16u * rb + li) * 4u);
          const uint32_t cnt = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)cur_cnt);
          const uint32_t e4 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)cur_e);
          const uint32_t first = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)cur_first);
          const bool f = (fastm >> rb) & 1u;
          uint64_t m[4];
          m[0] = f ? 0 : escape_mask8(C.nib[rb].x);
          m[1] = f ? 0 : escape_mask8(C.nib[rb].y);
          m[2] = f ? 0 : escape_mask8(C.nib[rb].z);
          m[3] = f ? 0 : escape_mask8(C.nib[rb].w);
          const uint32_t cl = (uint32_t)(__builtin_popcountll(m[0]) + __builtin_popcountll(m[1]) +
                                         __builtin_popcountll(m[2]) + __builtin_popcountll(m[3]));
          uint32_t pre = 0, tot = 0;
#pragma unroll
          for (uint32_t q = 0; q < 4; q++) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((li + 16u * q) * 4u), (int)cl);
            pre += q < lq ? v : 0u;
            tot += v;
          }
          // escapes of the tile before this step: counted so far (forward),
          // or the tile's total less those at and after it (backward)
          const uint32_t before = backward ? cnt - min(run[rb] + tot, cnt) : run[rb];
          run[rb] += tot;
          uint32_t pos = before + pre;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            while (m[i]) {
              const uint32_t wi = 8u * (i & 1) + ((uint32_t)__builtin_ctzll(m[i]) >> 3);
              // the first four escapes of the tile are in registers; only
              // past them is the stream read (and only that path waits)
              if (pos < min(cnt, 4u)) {
                patch_exponent(i < 2 ? E0 : E1, wi, (e4 >> (8 * pos)) & 0xFFu);
              } else {
                const uint32_t e = pos < cnt ? (uint32_t)P.esc[first + pos] : 0u;
                patch_exponent(i < 2 ? E0 : E1, wi, e);
              }
              m[i] &= m[i] - 1;
              pos++;
            }
          }
        }
        assemble16(C.raw0[rb], E0, w);
        assemble16(C.raw1[rb], E1, w + 8);
      }
      // this block's registers take its chunks of step k + D (issued for
      // every block, so that the count of younger loads stays fixed)
      __builtin_amdgcn_sched_barrier(0);
      load_block(C, rb, k + D);
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
#pragma unroll
        for (int h = 0; h < 4; h++) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]});
#pragma unroll
          for (int cb = 0; cb < NB; cb++)
            acc[rb][cb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, X[cb][h]), acc[rb][cb], 0, 0, 0);
        }
      }
    }
  };

  if (n_steps) {
    // x of step 0 goes before the coded loads, so that at least 3 * kGemmRB
    // loads follow it before step 0 waits for it.  With four row blocks
    // every coded load of the ring goes out before the escape facts wait for
    // their index words; with two (four waves a SIMD, whose loads queue
    // longer) only step 0's do, so that the escape facts and the next index
    // words queue behind one step instead of the whole ring
    constexpr int kFirst = RB == 2 ? 1 : D;
    meta_idx(0);
    dma_x(0);
    Coded<RB> C[D];
#pragma unroll
    for (int d = 0; d < kFirst; d++)
#pragma unroll
      for (int rb = 0; rb < kGemmRB; rb++) load_block(C[d], rb, d);
    meta_esc();
    meta_idx(1);
#pragma unroll
    for (int d = kFirst; d < D; d++)
#pragma unroll
      for (int rb = 0; rb < kGemmRB; rb++) load_block(C[d], rb, d);
    // n_steps is a multiple of 4, and D divides 4
    for (uint32_t k = 0; k < n_steps; k += D) {
#pragma unroll
      for (int d = 0; d < D; d++) step(C[d], k + d);
    }
  }
  // the slot takes this wave's partial sums next: nothing may still be
  // landing in it
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // partial sums through LDS, [wave][row block][column block][lane]; each
  // thread then adds entries over the waves in wave order and stores them
  // (each wave's partial sums go into its own x slot: no wave reads another's
  // slot before the barrier)
  constexpr uint32_t kEnt = kGemmRB * NB * kWave;
  constexpr uint32_t kSlot = NB * kXBlock / 16;  // f32x4 per wave slot
  static_assert(kEnt <= kSlot, "partial sums fit the x slot");
  f32x4* red = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int rb = 0; rb < kGemmRB; rb++)
#pragma unroll
    for (int cb = 0; cb < NB; cb++) red[wave * kSlot + (rb * NB + cb) * kWave + lane] = acc[rb][cb];
  __syncthreads();
  for (uint32_t e = threadIdx.x; e < kEnt; e += kGemmWaves * kWave) {
    f32x4 s = red[e];
#pragma unroll
    for (uint32_t w = 1; w < (uint32_t)kGemmWaves; w++) s += red[w * kSlot + e];
    // entry (rb, cb, lane (i, q)) holds Y[16 cb + i][r0 + 16 rb + 4 q + j], j = 0..3
    const uint32_t rb = e / (NB * kWave), cb = (e / kWave) % NB, ln = e % kWave;
    const uint32_t b = 16u * cb + (ln & 15u), rr0 = 16u * rb + 4u * (ln >> 4);
    if (b >= (uint32_t)L.batch) continue;
    const size_t base = (size_t)b * G.rows + r0;
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) {
      if (rr0 + j >= rows_here) break;
      if (L.y_bf16)
        static_cast<uint16_t*>(G.y)[base + rr0 + j] = f32_to_bf16_rne(s[j]);
      else
        static_cast<float*>(G.y)[base + rr0 + j] = s[j];
    }
  }
}

template <int NB, int D, int RB>
static hipError_t run_gemm(const GemmLaunch& L, uint32_t grid, hipStream_t s) {
  constexpr int lds = kGemmWaves * NB * 4 * 1040;
  const hipError_t e = open_dynamic_lds(reinterpret_cast<const void*>(&k_gemm<NB, D, RB>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm<NB, D, RB>), dim3(grid), dim3(kGemmWaves * kWave), lds, s, L);
  return hipGetLastError();
}

// Rows per workgroup of each group: a single tensor gets one workgroup per
// slot (slots = workgroups the compute units hold at once) where 16 ..
// max_rows rows a workgroup allow it; in a grouped launch each tensor gets
// its share of the slots by coded size.
static void gemm_rows_per_wg(GroupArg* g, int n_groups, uint64_t slots, uint32_t max_rows) {
  uint64_t total = 0;
  for (int i = 0; i < n_groups; i++) total += (uint64_t)g[i].rows * g[i].tiles;
  for (int i = 0; i < n_groups; i++) {
    const uint64_t rows = g[i].rows;
    const uint64_t lo = (rows + max_rows - 1) / max_rows, hi = (rows + kGemmMinRows - 1) / kGemmMinRows;
    const uint64_t want = total ? (slots * rows * g[i].tiles + total - 1) / total : 1;
    const uint64_t n_wg = std::max<uint64_t>(1, std::min(std::max(want, lo), hi));
    const uint32_t rpw = (uint32_t)((rows + n_wg - 1) / n_wg);
    g[i].aux = (g[i].aux & ((1u << kAuxRowsShift) - 1)) | (rpw << kAuxRowsShift);
  }
}

// One launch layout: rows per workgroup for waves of RB row blocks, the
// groups reordered so that the workgroups of the costliest come first
// (blocks are dispatched in order, so the longest ones do not start last;
// cost of one workgroup: its coded bytes, escapes weighted for the ranked
// path), and each group's first workgroup.  perm[g] is the caller's index
// of launch group g.
struct GemmLayout {
  GemmLaunch L;
  int perm[LBF_MAX_GROUPS];
  uint64_t wg;
};

static void gemm_layout(GemmLayout& Y, const GroupArg* groups, int n_groups, int cus, int rb, int y_bf16) {
  GemmLaunch& L = Y.L;
  L.n_groups = n_groups;
  L.y_bf16 = y_bf16;
  for (int g = 0; g < n_groups; g++) L.g[g] = groups[g];
  gemm_rows_per_wg(L.g, n_groups, (uint64_t)cus * (rb == 2 ? 2 : 1), 16u * rb);
  uint64_t wcost[LBF_MAX_GROUPS];
  for (int g = 0; g < n_groups; g++) {
    Y.perm[g] = g;
    const uint64_t rpw = L.g[g].aux >> kAuxRowsShift, rows = std::max<uint64_t>(1, L.g[g].rows);
    wcost[g] = rpw * L.g[g].tiles * (kTile + kTile / 2) + 64ull * L.g[g].n_esc * rpw / rows;
  }
  std::stable_sort(Y.perm, Y.perm + n_groups, [&](int a, int b) { return wcost[a] > wcost[b]; });
  GroupArg tmp[LBF_MAX_GROUPS];
  for (int g = 0; g < n_groups; g++) tmp[g] = L.g[Y.perm[g]];
  for (int g = 0; g < n_groups; g++) L.g[g] = tmp[g];
  uint64_t wg = 0;
  for (int g = 0; g < n_groups; g++) {
    const uint32_t rpw = L.g[g].aux >> kAuxRowsShift;
    L.wg_begin[g] = (uint32_t)wg;
    wg += L.g[g].rows ? (L.g[g].rows + rpw - 1) / rpw : 0;
  }
  L.wg_begin[n_groups] = (uint32_t)std::min<uint64_t>(wg, 0xFFFFFFFFu);
  Y.wg = wg;
}

// Batch columns go in slabs of up to 64 (each slab reads the coded weights
// again); a slab of m columns runs ceil(m / 16) MFMA column blocks, a slab
// of one block with waves of two row blocks.
hipError_t launch_gemm(const GroupArg* groups, int n_groups, int batch, int y_dtype, hipStream_t s) {
  int cus = 0;
  if (const hipError_t e = device_cus(&cus); e != hipSuccess) return e;
  const uint32_t eb = y_dtype == LBF_BF16 ? 2u : 4u;
  for (int g = 0; g < n_groups; g++)
    if (groups[g].tiles > kGemmMaxTiles) return hipErrorNotSupported;
  GemmLayout Y[2];  // [0]: four row blocks a wave, [1]: two
  bool made[2] = {false, false};
  for (int b0 = 0; b0 < batch; b0 += kGemmBatch) {
    const int nb = std::min(kGemmBatch, batch - b0);
    const int nblk = (nb + 15) / 16, which = nblk == 1 ? 1 : 0;
    GemmLayout& y = Y[which];
    if (!made[which]) {
      gemm_layout(y, groups, n_groups, cus, which ? 2 : 4, y_dtype == LBF_BF16);
      made[which] = true;
    }
    if (y.wg == 0) return hipSuccess;
    if (y.wg > 0x7FFFFFFFu) return hipErrorNotSupported;
    GemmLaunch& L = y.L;
    L.batch = nb;
    for (int g = 0; g < n_groups; g++) {
      const GroupArg& o = groups[y.perm[g]];
      L.g[g].x = o.x + (size_t)b0 * o.tiles * kTile;
      L.g[g].y = static_cast<uint8_t*>(o.y) + (size_t)b0 * o.rows * eb;
    }
    hipError_t e;
    switch (nblk) {
      case 1: e = run_gemm<1, 2, 2>(L, (uint32_t)y.wg, s); break;
      case 2: e = run_gemm<2, 2, 4>(L, (uint32_t)y.wg, s); break;
      case 3: e = run_gemm<3, 2, 4>(L, (uint32_t)y.wg, s); break;
      default: e = run_gemm<4, 1, 4>(L, (uint32_t)y.wg, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lbf
