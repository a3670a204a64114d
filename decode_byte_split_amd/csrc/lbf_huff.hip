// lbf_huff.hip — K15H, the entropy-coded variant: format v1's 4-bit codes
// Huffman-coded tile by tile, and their GPU decoder.  The English page's
// larger K15 reduction is for an entropy-coded form of the split ("Lossless
// LLM Weight Compression vs 8-bit GGUF", opening section); DFloat11 codes the
// exponent this way and keeps sign and mantissa raw ("你的 bf16 模型,有 5 個
// bit 是廢的", section 二).  The format is declared in include/lbf.h.
//
// Re-coding a v1 blob (all reads of its codes are coalesced 8-byte loads):
//   k_hcount        code counts over the real weights
//   k_htile_words   32-bit words of every tile's stream
//   k_hscan         one workgroup: woff[t] = words of tiles before t
//   k_hpack         one wave per tile: each lane's codes are OR-ed into the
//                   tile's words in LDS at the lane's prefix bit offset, then
//                   the words are written out coalesced
//
// Decoding (k_hdecode, one wave per tile, persistent grid): the only side
// information is each tile's first word, so lanes cannot know where their
// codes start.  The tile's stream is staged in LDS and cut into 64 equal bit
// windows; lane l decodes the codes that start inside window l, starting
// first at the window's first bit (a guess for every lane but lane 0).  A
// prefix code decoded from a wrong bit position typically falls back into
// step with the true code boundaries within a few codes, so most guessed
// lanes already end where the truth ends.  The wave then repeats: every lane
// takes the end position of the lane before it as its start; lanes whose
// start changed decode again; this stops when no start changes (lane l is
// exact after at most l rounds, typically one or two).  A prefix sum of the
// lanes' code counts places every code at its weight index in LDS, and the
// rest is format v1's decode: the table exponents, the escapes of the tile
// and the raw bytes assembled into BF16.  Codes of up to 12 bits are found
// with one lookup in a 4096-entry LDS table indexed by the next 12 stream
// bits; longer ones (rare: escapes and outlier exponents) by comparing the
// next 15 bits against each symbol's code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr int kHWaves = 4;                               // encode kernels
constexpr int kHDecWaves = 8;                            // decoder
constexpr uint32_t kHTableBits = 12;                     // primary decode table
constexpr uint32_t kHMaxWords = LBF_HMAX_TILE_WORDS;     // words of one tile's stream
constexpr uint32_t kHWordsLds = kHMaxWords + 4;          // + zero guard words

// Code of weight 16 lane + q from the lane's two split-half nibble words.
__device__ __forceinline__ uint32_t code_at(u32x2 nib, int q) {
  const uint32_t word = (q < 8) ? nib.x : nib.y;
  return (word >> (8 * (q & 3) + 4 * ((q >> 2) & 1))) & 15u;
}

__global__ void k_hzero(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Code counts: per-wave LDS bins, then one global add per bin and block.
__global__ __launch_bounds__(kHWaves * kWave) void k_hcount(const uint8_t* __restrict__ nib, uint64_t n,
                                                            uint64_t n_tiles, uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[kHWaves][16];
  const uint32_t wave = threadIdx.x >> 6;
  if (threadIdx.x < kHWaves * 16) (&h[0][0])[threadIdx.x] = 0u;
  __syncthreads();
  const uint64_t groups = n_tiles * kWave;  // 16 weights (8 nibble bytes) each
  for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (uint64_t)gridDim.x * blockDim.x) {
    const u32x2 v = load_nt(reinterpret_cast<const u32x2*>(nib) + g);
    const uint64_t w0 = g * 16;
#pragma unroll
    for (int q = 0; q < 16; q++)
      if (w0 + q < n) atomicAdd(&h[wave][code_at(v, q)], 1u);
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    uint32_t s = 0;
    for (int w = 0; w < kHWaves; w++) s += h[w][threadIdx.x];
    if (s) atomicAdd(&counts[threadIdx.x], s);
  }
}

// Length of code c from the 16 lengths packed 4 bits each into two words.
__device__ __forceinline__ uint32_t packed_len(uint32_t c, uint32_t len_lo, uint32_t len_hi) {
  return ((c < 8 ? len_lo : len_hi) >> (4 * (c & 7u))) & 15u;
}

__global__ __launch_bounds__(kHWaves * kWave) void k_htile_words(const uint8_t* __restrict__ nib, uint64_t n,
                                                                 uint64_t n_tiles, uint32_t len_lo, uint32_t len_hi,
                                                                 uint32_t* __restrict__ words) {
  const int lane = lane_id();
  const uint64_t t = (uint64_t)blockIdx.x * kHWaves + (threadIdx.x >> 6);
  if (t >= n_tiles) return;
  const u32x2 v = load_nt(reinterpret_cast<const u32x2*>(nib + t * (kTile / 2)) + lane);
  const uint64_t w0 = t * kTile + (uint64_t)lane * 16;
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 16; q++)
    if (w0 + q < n) bits += packed_len(code_at(v, q), len_lo, len_hi);
  for (int o = 32; o >= 1; o >>= 1) bits += (uint32_t)__shfl_xor((int)bits, o, kWave);
  if (lane == 0) words[t] = (bits + 31) / 32;
}

// woff[0] = 0, woff[t + 1] = woff[t] + words[t]; one workgroup of 1024.
__global__ __launch_bounds__(1024) void k_hscan(const uint32_t* __restrict__ words, uint64_t n_tiles,
                                                uint32_t* __restrict__ woff) {
  __shared__ uint32_t part[1024];
  __shared__ uint32_t carry;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    carry = 0;
    woff[0] = 0;
  }
  __syncthreads();
  for (uint64_t base = 0; base < n_tiles; base += 1024) {
    part[tid] = (base + tid < n_tiles) ? words[base + tid] : 0u;
    __syncthreads();
    for (uint32_t d = 1; d < 1024; d <<= 1) {  // inclusive scan
      const uint32_t add = tid >= d ? part[tid - d] : 0u;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (base + tid < n_tiles) woff[base + tid + 1] = carry + part[tid];
    __syncthreads();
    if (tid == 0) carry += part[1023];
    __syncthreads();
  }
}

struct HPackArgs {
  const uint8_t* nib;
  const uint32_t* woff;
  uint32_t* bits;
  uint64_t n, n_tiles, stream_words;
  uint32_t sym[16];  // reversed code << 4 | length
};

__global__ __launch_bounds__(kHWaves * kWave) void k_hpack(HPackArgs a) {
  __shared__ uint32_t buf[kHWaves][kHWordsLds];
  __shared__ uint32_t symtab[16];
  const uint32_t wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (threadIdx.x < 16) symtab[threadIdx.x] = a.sym[threadIdx.x];
  __syncthreads();
  const uint64_t t = (uint64_t)blockIdx.x * kHWaves + wave;
  if (t >= a.n_tiles) return;
  uint32_t* tb = buf[wave];
  for (uint32_t i = (uint32_t)lane; i < kHWordsLds; i += kWave) tb[i] = 0u;
  const u32x2 v = load_nt(reinterpret_cast<const u32x2*>(a.nib + t * (kTile / 2)) + lane);
  const uint64_t w0 = t * kTile + (uint64_t)lane * 16;
  uint32_t nbits = 0;
#pragma unroll
  for (int q = 0; q < 16; q++)
    if (w0 + q < a.n) nbits += symtab[code_at(v, q)] & 15u;
  // exclusive prefix of the lanes' bit counts (each < 256), bit by bit
  uint32_t pos = 0;
#pragma unroll
  for (int b = 0; b < 8; b++) pos += ballot_rank(__builtin_amdgcn_ballot_w64((nbits >> b) & 1u)) << b;
  wave_lds_sync();
  uint32_t wi = pos >> 5, nacc = pos & 31u;
  uint64_t acc = 0;  // pending bits of word wi, from bit 0 (bits below pos belong to earlier lanes)
#pragma unroll
  for (int q = 0; q < 16; q++) {
    if (w0 + q < a.n) {
      const uint32_t e = symtab[code_at(v, q)];
      acc |= (uint64_t)(e >> 4) << nacc;
      nacc += e & 15u;
      if (nacc >= 32) {
        if (wi < kHMaxWords) atomicOr(&tb[wi], (uint32_t)acc);
        acc >>= 32;
        nacc -= 32;
        wi++;
      }
    }
  }
  if (nacc && wi < kHMaxWords) atomicOr(&tb[wi], (uint32_t)acc);
  wave_lds_sync();
  const uint64_t base = a.woff[t];
  uint64_t nw = a.woff[t + 1] - base;
  if (a.woff[t + 1] < base) nw = 0;
  if (nw > kHMaxWords) nw = kHMaxWords;
  for (uint32_t i = (uint32_t)lane; i < nw; i += kWave)
    if (base + i < a.stream_words) a.bits[base + i] = tb[i];
}

// ---- decoder ---------------------------------------------------------------------

struct HDecArgs {
  const uint8_t* raw;
  const uint32_t* bits;
  const uint32_t* woff;
  const uint32_t* idx;
  const uint8_t* esc;
  uint16_t* out;
  uint32_t n, n_tiles, n_esc, stream_words;
  uint32_t esc_last;  // last readable byte of `esc` (clamp for unconditional loads)
  uint32_t waves;     // waves in the grid
  Lut lut;
  uint32_t base4;
  uint32_t sym[16];  // reversed code << 4 | length
};

// Decode table entry for the next 12 stream bits: up to four whole codes.
//   bits 0..3    total length of those codes (0: the first code is longer
//                than 12 bits and is found by hdec_long instead)
//   bits 4..14   bit j - 1 set if a code starts at offset j (1 <= j <= 11);
//                a code always starts at offset 0
//   bits 16..31  the symbols, 4 bits each, first code lowest
__device__ __forceinline__ uint32_t entry_len(uint32_t e) { return e & 15u; }
__device__ __forceinline__ uint32_t entry_starts(uint32_t e) { return 1u | ((e >> 3) & 0xFFEu); }

// The single code longer than the table at the low bits of v (at least 15
// valid): symbol << 4 | length; no match (a corrupt stream) gives symbol 0
// and length 1, so decoding always moves on.
__device__ __forceinline__ uint32_t hdec_long(const uint32_t* symtab, uint32_t v) {
  uint32_t e = 1u;
#pragma nounroll
  for (int s = 0; s < 16; s++) {
    const uint32_t d = symtab[s], L = d & 15u;
    if (L > kHTableBits && (v & ((1u << L) - 1)) == (d >> 4)) e = ((uint32_t)s << 4) | L;
  }
  return e;
}

// One decode step at the low bits of v: the codes it covers (`starts`, bit j
// = a code starting j bits on), its length `len`, and its symbols.  Codes
// starting at or after `room` bits belong to the next lane: they are cut off,
// and `len` then ends at the first of them.
struct Step {
  uint32_t starts, len, syms;
};

__device__ __forceinline__ Step hstep(const uint32_t* table, const uint32_t* symtab, uint32_t v, uint32_t room) {
  Step st;
  const uint32_t e = table[v & ((1u << kHTableBits) - 1)];
  if (entry_len(e)) {
    st.len = entry_len(e);
    st.starts = entry_starts(e);
    st.syms = e >> 16;
  } else {
    const uint32_t d = hdec_long(symtab, v);
    st.len = d & 15u;
    st.starts = 1u;
    st.syms = d >> 4;
  }
  if (st.len > room) {  // room >= 1: the first code is always the lane's
    const uint32_t rest = (st.starts | (1u << st.len)) >> room;
    st.starts &= (1u << room) - 1;
    st.len = room + (uint32_t)__builtin_ctz(rest);
  }
  return st;
}

// The tile's stream bits from a position on, least significant first, in a
// 64-bit register with at least 32 valid bits; the next word is read from
// LDS one refill ahead, so a decode step waits only for its table lookup.
struct BitReader {
  uint64_t buf;
  uint32_t have, next, ahead;
};

__device__ __forceinline__ void br_init(BitReader& r, const uint32_t* W, uint32_t pos) {
  const uint32_t i = pos >> 5;
  r.buf = (((uint64_t)W[i + 1] << 32) | W[i]) >> (pos & 31u);
  r.have = 64 - (pos & 31u);
  r.next = i + 2;
  r.ahead = W[min(r.next, kHWordsLds - 1)];
}

__device__ __forceinline__ void br_skip(BitReader& r, const uint32_t* W, uint32_t L) {
  r.buf >>= L;
  r.have -= L;
  if (r.have < 32) {
    r.buf |= (uint64_t)r.ahead << r.have;
    r.have += 32;
    r.next++;
    r.ahead = W[min(r.next, kHWordsLds - 1)];
  }
}

// What a tile needs from memory, loaded one tile ahead of its decode: the
// words of its stream (word lane + 64 j in bits[j]), its raw bytes, and the
// first 64 bytes of its escape slice.  Every load is issued unconditionally
// from a clamped, in-bounds address (unused results are replaced), so the
// compiler's in-order load counting stays exact across loop iterations.
constexpr int kHBitRegs = (kHMaxWords + kWave - 1) / kWave;

struct HTile {
  uint32_t w0, nw, first, n_esc;  // wave-uniform
  u32x4 raw;
  uint32_t bits[kHBitRegs];
  uint32_t escv;
};

// Index words of tile t (woff and idx pairs) into lanes 0 and 1.
__device__ __forceinline__ void htile_index(const HDecArgs& a, uint32_t t, int lane, uint32_t& wv, uint32_t& iv) {
  const uint32_t j = min(t + (uint32_t)(lane & 1), a.n_tiles);
  wv = a.woff[j];
  iv = a.idx[j];
}

__device__ __forceinline__ void htile_load(const HDecArgs& a, uint32_t t, int lane, uint32_t wv, uint32_t iv,
                                           HTile& T) {
  const uint32_t wa = (uint32_t)__builtin_amdgcn_readlane((int)wv, 0);
  const uint32_t wb = (uint32_t)__builtin_amdgcn_readlane((int)wv, 1);
  T.w0 = min(wa, a.stream_words);
  T.nw = min(min(max(wb, T.w0), a.stream_words) - T.w0, kHMaxWords);
  uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)iv, 0);
  uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)iv, 1);
  ib = min(ib, a.n_esc);  // as tile_escape_range
  ia = min(ia, ib);
  T.first = ia;
  T.n_esc = min(ib - ia, (uint32_t)kTile);
  const uint32_t tc = min(t, a.n_tiles - 1);
  T.raw = load_nt(reinterpret_cast<const u32x4*>(a.raw + (size_t)tc * kTile) + lane);
#pragma unroll
  for (int j = 0; j < kHBitRegs; j++) {
    const uint32_t i = (uint32_t)lane + kWave * j;
    const uint32_t v = a.bits[min(T.w0 + i, a.stream_words - 1)];
    T.bits[j] = i < T.nw ? v : 0u;
  }
  const uint32_t ev = a.esc[min(T.first + (uint32_t)lane, a.esc_last)];
  T.escv = (uint32_t)lane < T.n_esc ? ev : 0u;
}

template <bool CONTIG>
__global__ __launch_bounds__(kHDecWaves * kWave) void k_hdecode(HDecArgs a) {
  __shared__ uint32_t table[1u << kHTableBits];
  __shared__ uint32_t symtab[16];
  __shared__ uint32_t words[kHDecWaves][kHWordsLds];
  __shared__ __align__(16) uint8_t codes[kHDecWaves][kTile];
  __shared__ uint8_t esc_lds[kHDecWaves][kTile];
  const uint32_t wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (threadIdx.x < 16) symtab[threadIdx.x] = a.sym[threadIdx.x];
  __syncthreads();
  // single-code table first (symbol << 4 | length, 0 for codes over 12 bits),
  // in the codes buffer, then the multi-code entries by chaining it
  uint8_t* single = &codes[0][0];
  for (uint32_t i = threadIdx.x; i < (1u << kHTableBits); i += blockDim.x) {
    uint32_t e = 0;
    for (int s = 0; s < 16; s++) {
      const uint32_t d = symtab[s], L = d & 15u;
      if (L && L <= kHTableBits && (i & ((1u << L) - 1)) == (d >> 4)) e = ((uint32_t)s << 4) | L;
    }
    single[i] = (uint8_t)e;
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < (1u << kHTableBits); i += blockDim.x) {
    uint32_t pos = 0, starts = 0, syms = 0, n = 0;
    while (n < 4 && pos < kHTableBits) {
      const uint32_t d = single[i >> pos], L = d & 15u;
      if (!L || L > kHTableBits - pos) break;  // no whole code left in the 12 bits
      starts |= 1u << pos;
      syms |= (d >> 4) << (4 * n);
      n++;
      pos += L;
    }
    table[i] = n ? (pos | ((starts >> 1) << 4) | (syms << 16)) : 0u;
  }
  __syncthreads();
  uint32_t* W = words[wave];
  uint8_t* C = codes[wave];
  uint8_t* X = esc_lds[wave];

  uint32_t t = blockIdx.x * kHDecWaves + wave;
  if (t >= a.n_tiles) return;
  // two-deep pipeline: index words two tiles ahead, tile data one tile ahead
  uint32_t wv, iv, wv_next, iv_next;
  htile_index(a, t, lane, wv, iv);
  htile_index(a, t + a.waves, lane, wv_next, iv_next);
  HTile cur;
  htile_load(a, t, lane, wv, iv, cur);

  for (; t < a.n_tiles; t += a.waves) {
    HTile nxt;
    htile_load(a, t + a.waves, lane, wv_next, iv_next, nxt);
    uint32_t wv_nn, iv_nn;
    htile_index(a, t + 2 * a.waves, lane, wv_nn, iv_nn);

#pragma unroll
    for (int j = 0; j < kHBitRegs; j++) {
      const uint32_t i = (uint32_t)lane + kWave * j;
      if (i < kHWordsLds) W[i] = cur.bits[j];  // zeros from nw on: the guard words
    }
    reinterpret_cast<u32x4*>(C)[lane] = u32x4{0, 0, 0, 0};
    if ((uint32_t)lane < cur.n_esc) X[lane] = (uint8_t)cur.escv;
    for (uint32_t p = kWave + (uint32_t)lane; p < cur.n_esc; p += kWave) X[p] = a.esc[cur.first + p];  // rare
    wave_lds_sync();

    // lane windows of `win` bits; a first pass from every window's first bit
    // records the code starts it meets (bit p - lo of `seen`, windows of at
    // most 64 bits), so a later pass from the true start can stop at the
    // first recorded start it lands on: from there both passes agree.
    const uint32_t nbits = 32 * cur.nw, win = (nbits + 63) >> 6;
    const uint32_t lo = min((uint32_t)lane * win, nbits), hi = min(lo + win, nbits);
    const bool track = win <= 64;
    uint64_t seen = 0;
    uint32_t s = lo, e, cnt = 0;
    {
      BitReader r;
      br_init(r, W, lo);
      uint32_t pos = lo;
      while (pos < hi) {
        const Step st = hstep(table, symtab, (uint32_t)r.buf, hi - pos);
        if (track) seen |= (uint64_t)st.starts << (pos - lo);
        cnt += (uint32_t)__builtin_popcount(st.starts);
        br_skip(r, W, st.len);
        pos += st.len;
      }
      e = pos;
    }
    const uint32_t first_end = e;
    for (int round = 0; round < kWave; round++) {
      uint32_t ns = (uint32_t)__shfl_up((int)e, 1, kWave);
      if (lane == 0) ns = 0;
      const bool moved = ns != s;
      if (__builtin_amdgcn_ballot_w64(moved) == 0) break;
      if (moved) {
        s = ns;
        BitReader r;
        br_init(r, W, s);
        uint32_t pos = s, c = 0;
        while (pos < hi) {
          const Step st = hstep(table, symtab, (uint32_t)r.buf, hi - pos);
          const uint32_t hit = track ? (uint32_t)(seen >> (pos - lo)) & st.starts : 0u;
          if (hit) {  // a code start the first pass also met: from there both agree
            const uint32_t j = (uint32_t)__builtin_ctz(hit);
            c += (uint32_t)__builtin_popcount(st.starts & ((1u << j) - 1));
            c += (uint32_t)__builtin_popcountll(seen >> (pos + j - lo));
            pos = first_end;
            break;
          }
          c += (uint32_t)__builtin_popcount(st.starts);
          br_skip(r, W, st.len);
          pos += st.len;
        }
        e = pos;
        cnt = c;
      }
    }
    // first weight index of the lane's codes: exclusive prefix of the counts (< 256)
    uint32_t k = 0;
#pragma unroll
    for (int b = 0; b < 8; b++) k += ballot_rank(__builtin_amdgcn_ballot_w64((cnt >> b) & 1u)) << b;
    const uint64_t tile0 = (uint64_t)t * kTile;
    const uint32_t n_real = (uint32_t)min<uint64_t>(kTile, a.n - tile0);
    {
      BitReader r;
      br_init(r, W, s);
      for (uint32_t pos = s; pos < hi;) {
        const Step st = hstep(table, symtab, (uint32_t)r.buf, hi - pos);
        const uint32_t n = (uint32_t)__builtin_popcount(st.starts);
#pragma unroll
        for (uint32_t m = 0; m < 4; m++)
          if (m < n && k + m < n_real) C[k + m] = (uint8_t)((st.syms >> (4 * m)) & 15u);
        k += n;
        br_skip(r, W, st.len);
        pos += st.len;
      }
    }
    wave_lds_sync();

    // format v1's decode from here: codes -> exponents, escapes, raw bytes
    const u32x4 c4 = reinterpret_cast<const u32x4*>(C)[lane];
    const u32x2 nib = u32x2{c4.x | (c4.y << 4), c4.z | (c4.w << 4)};
    uint32_t E[4];
    exponents16<CONTIG>(nib, a.lut, a.base4, E);
    if (cur.n_esc) {
      uint64_t m0, m1;
      const uint32_t j = escape_rank(nib, m0, m1);
      patch_escapes(X, j, cur.n_esc, m0, m1, E);
    }
    uint32_t w[8];
    assemble16(cur.raw, E, w);
    const uint64_t e0 = tile0 + (uint64_t)lane * 16;
    if (e0 + 16 <= a.n) {
      u32x4* o = reinterpret_cast<u32x4*>(a.out + e0);
      __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, o);
      __builtin_nontemporal_store((u32x4){w[4], w[5], w[6], w[7]}, o + 1);
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (e0 + i < a.n) a.out[e0 + i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    }
    wave_lds_sync();  // the words, codes and escapes are rewritten for the next tile
    cur = nxt;
    wv_next = wv_nn;
    iv_next = iv_nn;
  }
}

// ---- host side ---------------------------------------------------------------------

// Code lengths, canonical codes and the blob layout: lbf_host.cpp.

static void pack_lengths(const uint8_t len[16], uint32_t& lo, uint32_t& hi) {
  lo = hi = 0;
  for (int c = 0; c < 8; c++) {
    lo |= (uint32_t)len[c] << (4 * c);
    hi |= (uint32_t)len[8 + c] << (4 * c);
  }
}

hipError_t launch_hcount(const lbf_desc& d, const uint8_t* blob, uint32_t* counts, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  hipLaunchKernelGGL(k_hzero, dim3(1), dim3(64), 0, s, counts, 16u);
  if (L.n_tiles) {
    const uint64_t groups = L.n_tiles * kWave;
    const unsigned grid = (unsigned)std::min<uint64_t>(4096, (groups + kHWaves * kWave - 1) / (kHWaves * kWave));
    hipLaunchKernelGGL(k_hcount, dim3(grid), dim3(kHWaves * kWave), 0, s, blob + L.off_nib, L.n, L.n_tiles, counts);
  }
  return hipGetLastError();
}

hipError_t launch_hwoff(const lbf_desc& d, const uint8_t* blob, const uint8_t len[16], uint32_t* words,
                        uint32_t* woff, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  uint32_t lo, hi;
  pack_lengths(len, lo, hi);
  if (L.n_tiles) {
    const unsigned grid = (unsigned)((L.n_tiles + kHWaves - 1) / kHWaves);
    hipLaunchKernelGGL(k_htile_words, dim3(grid), dim3(kHWaves * kWave), 0, s, blob + L.off_nib, L.n, L.n_tiles, lo,
                       hi, words);
  }
  hipLaunchKernelGGL(k_hscan, dim3(1), dim3(1024), 0, s, words, L.n_tiles, woff);
  return hipGetLastError();
}

hipError_t launch_hpack(const lbf_desc& d, const uint8_t* blob, const HCode& code, const uint32_t* woff,
                        uint32_t* bits, uint64_t stream_words, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  if (!L.n_tiles) return hipSuccess;
  HPackArgs a;
  a.nib = blob + L.off_nib;
  a.woff = woff;
  a.bits = bits;
  a.n = L.n;
  a.n_tiles = L.n_tiles;
  a.stream_words = stream_words;
  for (int c = 0; c < 16; c++) a.sym[c] = code.sym[c];
  const unsigned grid = (unsigned)((L.n_tiles + kHWaves - 1) / kHWaves);
  hipLaunchKernelGGL(k_hpack, dim3(grid), dim3(kHWaves * kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_hdecode(const lbf_hdesc& h, const HCode& code, const uint8_t* blob, uint16_t* out, hipStream_t s) {
  const HLayout L = hlayout_of(h.rows, h.cols, h.n_esc, h.stream_words);
  if (!L.n_tiles) return hipSuccess;
  int cus = 0;
  if (const hipError_t e = device_cus(&cus); e != hipSuccess) return e;
  const KLut k = klut_from(h.lut, h.n_codes);
  HDecArgs a;
  a.raw = blob + L.off_raw;
  a.bits = reinterpret_cast<const uint32_t*>(blob + L.off_bits);
  a.woff = reinterpret_cast<const uint32_t*>(blob + L.off_woff);
  a.idx = reinterpret_cast<const uint32_t*>(blob + L.off_idx);
  // with no escapes the escape plane is empty: point its (unused) loads at the index
  a.esc = L.n_esc ? blob + L.off_esc : blob + L.off_idx;
  a.esc_last = L.n_esc ? (uint32_t)(L.n_esc - 1) : 0u;
  a.out = out;
  a.n = (uint32_t)L.n;
  a.n_tiles = (uint32_t)L.n_tiles;
  a.n_esc = (uint32_t)L.n_esc;
  a.stream_words = (uint32_t)L.stream_words;
  a.lut = Lut{k.t[0], k.t[1], k.t[2], k.t[3]};
  a.base4 = k.base4;
  for (int c = 0; c < 16; c++) a.sym[c] = code.sym[c];
  // a persistent grid: exactly the workgroups that can be resident at once
  int per_cu = 0;
  const void* fn = k.contiguous ? reinterpret_cast<const void*>(&k_hdecode<true>)
                                : reinterpret_cast<const void*>(&k_hdecode<false>);
  if (const hipError_t occ = blocks_per_cu(fn, kHDecWaves * kWave, &per_cu); occ != hipSuccess) return occ;
  const uint64_t blocks = std::min<uint64_t>((L.n_tiles + kHDecWaves - 1) / kHDecWaves,
                                             (uint64_t)std::max(cus, 1) * (uint64_t)std::max(per_cu, 1));
  a.waves = (uint32_t)(blocks * kHDecWaves);
  if (k.contiguous)
    hipLaunchKernelGGL(k_hdecode<true>, dim3((unsigned)blocks), dim3(kHDecWaves * kWave), 0, s, a);
  else
    hipLaunchKernelGGL(k_hdecode<false>, dim3((unsigned)blocks), dim3(kHDecWaves * kWave), 0, s, a);
  return hipGetLastError();
}

// The header (128 descriptor bytes, then zeros) and every gap the format pads.
struct HFillArgs {
  uint8_t* blob;
  uint32_t head[32];
  uint64_t gap_at[4], gap_len[4];
};

__global__ __launch_bounds__(256) void k_hfill(HFillArgs a) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  if (tid < LBF_HEADER_BYTES / 4)
    reinterpret_cast<uint32_t*>(a.blob)[tid] = tid < 32 ? a.head[tid] : 0u;
  for (int g = 0; g < 4; g++)
    for (uint64_t i = tid; i < a.gap_len[g]; i += stride) a.blob[a.gap_at[g] + i] = 0;
}

hipError_t launch_hfill(const lbf_hdesc& h, uint8_t* blob, hipStream_t s) {
  const HLayout L = hlayout_of(h.rows, h.cols, h.n_esc, h.stream_words);
  HFillArgs a;
  a.blob = blob;
  std::memcpy(a.head, &h, sizeof a.head);
  a.gap_at[0] = L.off_bits + 4 * L.stream_words;
  a.gap_len[0] = L.off_woff - a.gap_at[0];
  a.gap_at[1] = L.off_woff + 4 * (L.n_tiles + 1);
  a.gap_len[1] = L.off_idx - a.gap_at[1];
  a.gap_at[2] = L.off_idx + 4 * (L.n_tiles + 1);
  a.gap_len[2] = L.off_esc - a.gap_at[2];
  a.gap_at[3] = L.off_esc + L.n_esc;
  a.gap_len[3] = L.blob_bytes - a.gap_at[3];
  hipLaunchKernelGGL(k_hfill, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lbf
