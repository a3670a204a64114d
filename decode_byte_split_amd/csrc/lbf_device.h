// lbf_device.h — device-side building blocks shared by the gfx950 kernels:
// nibble-code expansion, exponent lookup, BF16 reassembly, escape placement
// and wave-level integer prefix sums.
//
// Format (see include/lbf.h): per weight one raw byte (mantissa << 1 | sign
// of the pair partner) and one 4-bit code; code c < 15 stands for exponent lut[c], code 15 takes
// the next byte of the tile's escape slice.  The pages this follows:
// "Lossless LLM Weight Compression vs 8-bit GGUF" (wavect.io), sections
// "What does 'lossless' mean for LLM weights?" (exact rebuild in registers
// right before the multiply) and "What did the GLM-5.2 experiment actually
// prove?" (fixed short codes for frequent exponents, exact escape stream).
//
// Lane work unit: 16 consecutive weights of a 1024-weight tile, i.e. one
// 16-byte raw load (4 words: weights 4q .. 4q+3 in word q) and one 8-byte
// nibble load (word 0: weights 0..7, word 1: weights 8..15; in each word,
// byte j holds weight j in its low nibble and weight 4 + j in its high one).
// The raw byte of weight i is mantissa_i << 1 | sign of its partner i ^ 1.
// Decoded weights leave as 8 packed bf16 pairs, pair p = weights (2p, 2p+1),
// low half first: the operand layout of v_dot2_f32_bf16 and of memory.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbf {

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kTile = 1024;
constexpr int kWave = 64;

// Code table as four little-endian words: t[q] bytes = lut[4q .. 4q+3].
struct Lut {
  uint32_t t0, t1, t2, t3;
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four code bytes (each 0..15) -> four exponent bytes, lut[c] per byte.
// v_perm_b32 looks bytes up in an 8-byte table; codes 0..7 use lut[0..7],
// codes 8..15 use lut[8..15] with the selector's bit 3 cleared, and a
// per-byte mask built from bit 3 (selector 4 -> 0xFF byte, 12 -> 0x00)
// picks between the two lookups.
__device__ __forceinline__ uint32_t lut_lookup(uint32_t c, const Lut& L) {
  uint32_t c7 = c & 0x07070707u;
  uint32_t lo = perm(L.t1, L.t0, c7);
  uint32_t hi = perm(L.t3, L.t2, c7);
  uint32_t sel = (c & 0x08080808u) | 0x04040404u;
  uint32_t keep_lo = perm(0xFFFFFFFFu, 0u, sel);
  return (lo & keep_lo) | (hi & ~keep_lo);
}

// Exponent bytes of a lane's 16 weights from its two nibble words:
// E[q] byte j = exponent of weight 4q + j.
// CONTIG: the table is lut[c] = lut[0] + c (the common case for trained
// weights), so a byte-wise add replaces the lookup; `base4` = lut[0] * 0x01010101.
template <bool CONTIG>
__device__ __forceinline__ void exponents16(u32x2 nib, const Lut& L, uint32_t base4, uint32_t E[4]) {
  uint32_t c[4];
  c[0] = nib.x & 0x0F0F0F0Fu;
  c[1] = (nib.x >> 4) & 0x0F0F0F0Fu;
  c[2] = nib.y & 0x0F0F0F0Fu;
  c[3] = (nib.y >> 4) & 0x0F0F0F0Fu;
#pragma unroll
  for (int q = 0; q < 4; q++) E[q] = CONTIG ? c[q] + base4 : lut_lookup(c[q], L);
}

// Rebuild 8 bf16 pairs.  For weights a = 2p, b = 2p + 1 one v_perm_b32 forms
// the word [raw_a, e_a, raw_b, e_b] (low byte first); rotating it right by
// one bit puts mantissa_a in bits 0..6, e_a in 7..14, sign_a (bit 0 of
// raw_b) in bit 15, mantissa_b in 16..22, e_b in 23..30 and sign_b (bit 0 of
// raw_a) in bit 31: exactly the two bf16 values.
__device__ __forceinline__ void assemble16(u32x4 raw, const uint32_t E[4], uint32_t w[8]) {
  const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int p = 0; p < 8; p++) {
    const uint32_t v = perm(E[p >> 1], rw[p >> 1], (p & 1) ? 0x07030602u : 0x05010400u);
    w[p] = __builtin_amdgcn_alignbit(v, v, 1u);
  }
}

// Escape flags of the 8 weights of one nibble word, in weight order: bit 8i
// is set iff weight i's code is 15.
__device__ __forceinline__ uint64_t escape_mask8(uint32_t n) {
  uint32_t t = n & (n >> 2);
  t &= t >> 1;  // bit 4k: all four bits of nibble k are set
  const uint32_t lo = t & 0x01010101u, hi = (t >> 4) & 0x01010101u;
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of a wave-wide ballot in lanes below this one.
__device__ __forceinline__ uint32_t ballot_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the wave of v (0 <= v < 32), bit by bit:
// sum_b 2^b * #{lower lanes with bit b of v set}.
__device__ __forceinline__ uint32_t wave_excl_scan_small(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 5; b++) r += ballot_rank(__builtin_amdgcn_ballot_w64(((v >> b) & 1u) != 0)) << b;
  return r;
}

// Overwrite the exponent byte of weight i (0..15) in the E[] layout above.
__device__ __forceinline__ void patch_exponent(uint32_t E[4], uint32_t i, uint32_t e) {
  const uint32_t word = i >> 2;
  const uint32_t sh = (i & 3u) * 8u;
  const uint32_t m = 0xFFu << sh, v = e << sh;
#pragma unroll
  for (uint32_t q = 0; q < 4; q++) E[q] = (word == q) ? ((E[q] & ~m) | v) : E[q];
}

// Escapes of one tile, one wave (all 64 lanes must call): which of the lane's
// 16 weights escape (bit 8i of m0 / m1 for weight i / 8 + i) and how many
// escapes of the tile precede the lane's first one.  When no lane holds more
// than one escape a single ballot gives the rank.
__device__ __forceinline__ uint32_t escape_rank(u32x2 nib, uint64_t& m0, uint64_t& m1) {
  m0 = escape_mask8(nib.x);
  m1 = escape_mask8(nib.y);
  const uint32_t k = (uint32_t)(__builtin_popcountll(m0) + __builtin_popcountll(m1));
  if (__builtin_amdgcn_ballot_w64(k > 1u) == 0) return ballot_rank(__builtin_amdgcn_ballot_w64(k != 0u));
  return wave_excl_scan_small(k);
}

// Patch the lane's escaped exponents, in element order, from src[j ...],
// a byte array in LDS holding the tile's escapes; reads at or past cnt (a
// corrupt blob) yield exponent 0 and touch nothing outside src[0, cnt).
__device__ __forceinline__ void patch_escapes(const uint8_t* src, uint32_t j, uint32_t cnt, uint64_t m0, uint64_t m1,
                                              uint32_t E[4]) {
  while (m0) {
    const uint32_t i = (uint32_t)__builtin_ctzll(m0) >> 3;
    patch_exponent(E, i, j < cnt ? src[j] : 0u);
    m0 &= m0 - 1;
    j++;
  }
  while (m1) {
    const uint32_t i = 8u + ((uint32_t)__builtin_ctzll(m1) >> 3);
    patch_exponent(E, i, j < cnt ? src[j] : 0u);
    m1 &= m1 - 1;
    j++;
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS bytes of a wave's escape staging slot: a tile's slice (<= 1024 bytes)
// from its 4-byte aligned start, in five 256-byte loads.
constexpr uint32_t kEscSlot = 1280;

// Escape placement for one tile held by one wave (called by all 64 lanes,
// only when the tile has escapes).  The tile's escape slice esc[first,
// first + cnt) (cnt <= 1024) is copied into this wave's LDS slot (kEscSlot
// bytes, 4-byte aligned) by five 4-byte buffer loads per lane that write
// straight into LDS, all issued before a single wait; the slice then starts
// at slot[first & 3] (bytes past it read as zeros, with no memory access).
// Each lane patches its exponent bytes in element order.
__device__ __forceinline__ void place_escapes(u32x2 nib, const uint8_t* __restrict__ esc, uint32_t first,
                                              uint32_t cnt, uint8_t* slot, uint32_t E[4]) {
  const uint32_t lane = (uint32_t)lane_id();
  const uint32_t a0 = first & ~3u, nb = first + cnt - a0;  // bytes from the aligned start
  // one range over the slice, rounded up to whole dwords (the range check is
  // per dword; the escape plane starts on a 256-byte boundary and the blob's
  // size is a multiple of 256, so that dword is inside the blob); loads past
  // it read as zeros.  Load i takes the 256 bytes from a0 + 256 i into slot +
  // 256 i.  The lane offset is made opaque here so that the five offsets are
  // formed on this (rare) path instead of being kept in registers for the
  // whole kernel.
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
  uint64_t m0, m1;
  const uint32_t j = escape_rank(nib, m0, m1);
  patch_escapes(slot + (first & 3u), j, cnt, m0, m1, E);
  wave_lds_sync();  // the slot is rewritten for the next tile
}

// Escape range of tile t from the index plane, clamped so that a corrupt
// index can neither read past the escape stream nor overflow an LDS slot.
__device__ __forceinline__ void tile_escape_range(const uint32_t* __restrict__ idx, uint32_t t, uint32_t n_esc,
                                                  uint32_t& first, uint32_t& cnt) {
  uint32_t a = idx[t], b = idx[t + 1];
  if (b > n_esc) b = n_esc;
  if (a > b) a = b;
  first = a;
  cnt = b - a;
  if (cnt > (uint32_t)kTile) cnt = kTile;
}

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 load_nt(const u32x2* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// s_waitcnt operand that limits only the vector-memory count to n (0..63):
// gfx9 encoding, vmcnt in bits 3..0 and 15..14, expcnt (6..4) and lgkmcnt
// (11..8) left at their maxima so nothing else is waited for.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(waitcnt_vm(8) == 0x0F78 && waitcnt_vm(16) == 0x4F70, "vmcnt encoding");

// Plane addresses of a format-v1 blob with n_tiles tiles (header 256 bytes,
// raw and nibble planes back to back, index, escapes at the next 256 boundary).
struct Planes {
  const uint8_t *raw, *nib, *esc;
  const uint32_t* idx;
};
__device__ __forceinline__ Planes planes_of(const uint8_t* blob, uint64_t n_tiles) {
  Planes P;
  P.raw = blob + 256;
  P.nib = P.raw + n_tiles * kTile;
  P.idx = reinterpret_cast<const uint32_t*>(P.nib + n_tiles * (kTile / 2));
  P.esc = blob + ((256 + n_tiles * (kTile + kTile / 2) + 4 * (n_tiles + 1) + 255) & ~uint64_t(255));
  return P;
}

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return 0 and stores there are dropped, without touching memory.
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access on gfx9
constexpr int kNonTemporal = 2;         // cache policy: streaming
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// The code table of a blob, from its header copy (lut[16] at byte 72).  The
// header does not change while a kernel runs, so it is read through the
// constant address space: with a uniform blob pointer, one scalar load into
// SGPRs and no vector registers.
typedef __attribute__((address_space(4))) const u32x4 ConstU32x4;
__device__ __forceinline__ Lut header_lut(const uint8_t* blob) {
  const u32x4 h = *reinterpret_cast<ConstU32x4*>(reinterpret_cast<uintptr_t>(blob + 72));
  return Lut{h.x, h.y, h.z, h.w};
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet, sign kept).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace lbf
