// lbf_verify.hip — integrity checks of coded blobs on the GPU: a structural
// verification against the trusted host descriptor, and CRC-32 of device
// memory (so a stored hash of a whole blob can be checked without a host
// copy).  Corrupt weights must be detected and refused rather than decoded
// into wrong values ("Lossless LLM Weight Compression vs 8-bit GGUF",
// sections "Is the GLM-5.2 result production-ready?" and "Questions to ask a
// vendor or research team").
//
// Verification needs no decode: every code-15 nibble of a tile must be
// matched by one index entry, codes n_codes..14 are never written, an escape
// byte is never one of the coded exponents, and everything the format pads
// is zero.  The raw sign/mantissa bytes of real weights carry no redundancy;
// the CRC covers them.  Whole tiles are checked eight per wave step with
// byte-parallel nibble arithmetic; the partial last tile and the byte-sized
// regions (header, index ends, escapes, gaps) take a plain per-element path.
//
// CRC-32 here is zlib's (IEEE 802.3 polynomial, reflected, initial value and
// final xor all ones).  With S(c, M) the CRC register after message M from
// register c, S is linear over GF(2): S(c, M) = c * x^(8|M|) + S(0, M), and
// S(0, M) is the XOR of the contributions of M's bytes, byte b at distance d
// from the end contributing T0[b] * x^(8d) (T0 the one-byte table).  The
// message is cut into 1 KiB lines; lane l of a wave owns bytes [16 l, 16 l +
// 16) of every line, and the W waves of the launch take the lines in turn, so
// every load is a coalesced 16-byte load.  A lane's register jumps over the
// bytes other lanes own with four lookup tables (byte k of the register
// times x^(8 (1024 W - 1 - k))), then takes its 16 new bytes from sixteen
// tables (byte b followed by 15 - k zero bytes).  Lines are counted so that
// the last step of every wave ends at the message end; missing lines are
// taken as leading zero lines, which leave a zero register unchanged.  At the
// end each lane's register is moved to the message end by one multiply with
// a constant of its lane and one of its wave, and the moved registers are
// XOR-ed together (atomically; XOR is order-free, so the result is exact and
// deterministic).  The host precomputes every power of x the kernel needs.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lbf_device.h"
#include "lbf_internal.h"

namespace lbf {

constexpr uint32_t kCrcPoly = 0xEDB88320u;  // reflected IEEE 802.3
constexpr uint32_t kCrcOne = 0x80000000u;   // the polynomial 1 (bit 31 holds x^0)
constexpr uint32_t kCrcX = 0x40000000u;     // the polynomial x
constexpr uint32_t kCrcLine = 1024;         // bytes per wave step: 64 lanes x 16
constexpr int kCrcWaves = 4;
constexpr int kCrcPowBits = 16;             // a launch has fewer than 2^16 waves
constexpr int kVerifyWaves = 4;
constexpr int kVerifyGroup = 8;             // whole tiles per wave step: 4 loads of 2 tiles

// a * b modulo the CRC polynomial, both in the reflected representation: add
// b for every set bit of a (bit 31 first, x^0), multiplying b by x after each.
__host__ __device__ inline uint32_t crc_mul(uint32_t a, uint32_t b) {
  uint32_t p = 0;
  for (int i = 0; i < 32; i++) {
    p ^= b & (0u - ((a >> (31 - i)) & 1u));
    b = (b >> 1) ^ (kCrcPoly & (0u - (b & 1u)));
  }
  return p;
}

// ---- structural verification ---------------------------------------------------

struct VerifyArgs {
  const uint8_t* blob;
  uint32_t* flags;
  uint32_t desc[24];  // the 96 trusted header bytes
  uint32_t coded[8];  // bit e set: exponent e has a code
  uint64_t n, n_tiles, n_full, n_esc, off_raw, off_nib, off_idx, off_esc, blob_bytes;
  uint32_t n_codes, waves;
};

__global__ void k_word_set(uint32_t* p, uint32_t v) { *p = v; }

__device__ __forceinline__ void report(uint32_t* flags, uint32_t f) {
  if (f) atomicOr(flags, f);
}

// One 32-bit nibble word (eight codes, all of weights below n): count the
// code-15 nibbles and mark codes n_codes..14.  Each nibble is widened to a
// byte, so adding (16 - n_codes) sets bit 4 exactly for codes >= n_codes and
// adding 1 sets it exactly for code 15; no byte overflows into the next.
__device__ __forceinline__ void nibble_word(uint32_t w, uint32_t k_ge, uint32_t& fifteens, uint32_t& bad) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t e_lo = (lo + 0x01010101u) & 0x10101010u;
  const uint32_t e_hi = (hi + 0x01010101u) & 0x10101010u;
  fifteens += (uint32_t)__builtin_popcount(e_lo | (e_hi >> 1));
  bad |= (((lo + k_ge) & ~e_lo) | ((hi + k_ge) & ~e_hi)) & 0x10101010u;
}

// The index checks of one tile from its two index words and its code-15 count.
__device__ __forceinline__ uint32_t index_flags(uint32_t ia, uint32_t ib, uint32_t total) {
  uint32_t f = 0;
  if (ib < ia) f |= LBF_VERIFY_INDEX;
  if ((ib < ia && total != 0) || (ib >= ia && total != ib - ia)) f |= LBF_VERIFY_COUNT;
  return f;
}

// The partial last tile t, one wave, element by element: codes, count, index,
// and the padding past n in the nibble and raw planes.
__device__ void verify_last_tile(const VerifyArgs& a, uint64_t t, int lane, uint32_t& f) {
  const uint32_t* idx = reinterpret_cast<const uint32_t*>(a.blob + a.off_idx);
  const u32x2 nib = reinterpret_cast<const u32x2*>(a.blob + a.off_nib + t * (kTile / 2))[lane];
  const uint64_t w0 = t * kTile + (uint64_t)lane * 16;  // weight of the lane's first nibble
  uint32_t fifteens = 0;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    // weight 16 lane + q: word q / 8, byte q % 4, high nibble if bit 2 of q
    const uint32_t word = (q < 8) ? nib.x : nib.y;
    const uint32_t c = (word >> (8 * (q & 3) + 4 * ((q >> 2) & 1))) & 15u;
    if (w0 + q >= a.n) {
      if (c) f |= LBF_VERIFY_PADDING;
    } else if (c == 15u) {
      fifteens++;
    } else if (c >= a.n_codes) {
      f |= LBF_VERIFY_CODE;
    }
  }
  uint32_t total = 0;  // wave sum of the lane counts (each < 32), bit by bit
#pragma unroll
  for (int b = 0; b < 5; b++) total += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((fifteens >> b) & 1u)) << b;
  if (lane == 0) f |= index_flags(idx[t], idx[t + 1], total);
  const u32x4 r = reinterpret_cast<const u32x4*>(a.blob + a.off_raw + t * kTile)[lane];
  const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const uint64_t i = w0 + q;
    const uint32_t byte = (rw[q >> 2] >> (8 * (q & 3))) & 0xFFu;
    const uint32_t allowed = (i == a.n && (a.n & 1u)) ? 1u : 0u;  // byte n carries the sign of weight n - 1
    if (i >= a.n && (byte & ~allowed)) f |= LBF_VERIFY_PADDING;
  }
}

__global__ __launch_bounds__(kVerifyWaves * kWave) void k_verify(VerifyArgs a) {
  const int lane = lane_id();
  const uint32_t w = blockIdx.x * kVerifyWaves + (threadIdx.x >> 6);
  const uint32_t* idx = reinterpret_cast<const uint32_t*>(a.blob + a.off_idx);
  const uint32_t k_ge = (16u - min(a.n_codes, 16u)) * 0x01010101u;
  uint32_t f = 0;
  // whole tiles, eight per step: load i covers tile t0 + 2i (lanes 0-31) and
  // t0 + 2i + 1 (lanes 32-63), 16 bytes = 32 codes per lane
  for (uint64_t t0 = (uint64_t)w * kVerifyGroup; t0 < a.n_full; t0 += (uint64_t)a.waves * kVerifyGroup) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint64_t t = t0 + 2 * i + (lane >> 5);
      v[i] = t < a.n_full ? *reinterpret_cast<const u32x4*>(a.blob + a.off_nib + t * (kTile / 2) + (lane & 31) * 16)
                          : u32x4{0, 0, 0, 0};
    }
    const uint32_t iv = (lane <= kVerifyGroup && t0 + lane <= a.n_tiles) ? idx[t0 + lane] : 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t fifteens = 0, bad = 0;
      nibble_word(v[i].x, k_ge, fifteens, bad);
      nibble_word(v[i].y, k_ge, fifteens, bad);
      nibble_word(v[i].z, k_ge, fifteens, bad);
      nibble_word(v[i].w, k_ge, fifteens, bad);
      const uint64_t ta = t0 + 2 * i;
      if (ta + (lane >> 5) >= a.n_full) fifteens = bad = 0;
      if (bad) f |= LBF_VERIFY_CODE;
      uint32_t tot_a = 0, tot_b = 0;  // half-wave sums of the lane counts (each <= 32)
#pragma unroll
      for (int b = 0; b < 6; b++) {
        const uint64_t m = __builtin_amdgcn_ballot_w64((fifteens >> b) & 1u);
        tot_a += (uint32_t)__builtin_popcount((uint32_t)m) << b;
        tot_b += (uint32_t)__builtin_popcount((uint32_t)(m >> 32)) << b;
      }
      const uint32_t i0 = (uint32_t)__builtin_amdgcn_readlane((int)iv, 2 * i);
      const uint32_t i1 = (uint32_t)__builtin_amdgcn_readlane((int)iv, 2 * i + 1);
      const uint32_t i2 = (uint32_t)__builtin_amdgcn_readlane((int)iv, 2 * i + 2);
      if (lane == 0) {
        if (ta < a.n_full) f |= index_flags(i0, i1, tot_a);
        if (ta + 1 < a.n_full) f |= index_flags(i1, i2, tot_b);
      }
    }
  }
  if (w == a.waves - 1 && a.n_full < a.n_tiles) verify_last_tile(a, a.n_full, lane, f);

  // byte-sized regions, grid-stride over single bytes
  const uint64_t stride = (uint64_t)a.waves * kWave;
  const uint64_t tid = (uint64_t)w * kWave + lane;
  if (tid < LBF_HEADER_BYTES) {
    const uint32_t want = tid < 96 ? (a.desc[tid >> 2] >> (8 * (tid & 3))) & 0xFFu : 0u;
    if (a.blob[tid] != want) f |= LBF_VERIFY_HEADER;
  }
  if (tid == 0 && (idx[0] != 0 || idx[a.n_tiles] != a.n_esc)) f |= LBF_VERIFY_INDEX;
  for (uint64_t j = tid; j < a.n_esc; j += stride) {
    const uint32_t e = a.blob[a.off_esc + j];
    if ((a.coded[e >> 5] >> (e & 31u)) & 1u) f |= LBF_VERIFY_ESCAPE;
  }
  const uint64_t gap0 = a.off_idx + 4 * (a.n_tiles + 1);
  for (uint64_t j = gap0 + tid; j < a.off_esc; j += stride)
    if (a.blob[j]) f |= LBF_VERIFY_PADDING;
  for (uint64_t j = a.off_esc + a.n_esc + tid; j < a.blob_bytes; j += stride)
    if (a.blob[j]) f |= LBF_VERIFY_PADDING;
  report(a.flags, f);
}

// Waves for a launch: about `per` units of work each, at most 16 per CU, a
// whole number of workgroups.
static uint32_t launch_waves(uint64_t units, uint64_t per, int cus, int per_block) {
  const uint64_t want = (units + per - 1) / per;
  const uint64_t cap = std::min<uint64_t>((uint64_t)std::max(cus, 1) * 16, (1u << kCrcPowBits) - per_block);
  const uint64_t w = std::max<uint64_t>(1, std::min(want, cap));
  return (uint32_t)((w + per_block - 1) / per_block * per_block);
}

hipError_t launch_verify(const lbf_desc& d, const uint8_t* blob, uint32_t* flags, hipStream_t s) {
  const Layout L = layout_of(d.rows, d.cols, d.n_esc);
  VerifyArgs a;
  a.blob = blob;
  a.flags = flags;
  const uint8_t* db = reinterpret_cast<const uint8_t*>(&d);
  for (int i = 0; i < 24; i++)
    a.desc[i] = (uint32_t)db[4 * i] | (uint32_t)db[4 * i + 1] << 8 | (uint32_t)db[4 * i + 2] << 16 |
                (uint32_t)db[4 * i + 3] << 24;
  for (int i = 0; i < 8; i++) a.coded[i] = 0;
  for (int c = 0; c < d.n_codes; c++) a.coded[d.lut[c] >> 5] |= 1u << (d.lut[c] & 31u);
  a.n = L.n;
  a.n_tiles = L.n_tiles;
  a.n_full = L.n / kTile;
  a.n_esc = L.n_esc;
  a.off_raw = L.off_raw;
  a.off_nib = L.off_nib;
  a.off_idx = L.off_idx;
  a.off_esc = L.off_esc;
  a.blob_bytes = L.blob_bytes;
  a.n_codes = d.n_codes;
  int cus = 0;
  if (device_cus(&cus) != hipSuccess) return hipErrorUnknown;
  // two steps of whole tiles per wave, or enough threads for the byte regions
  const uint64_t groups = (a.n_full + kVerifyGroup - 1) / kVerifyGroup;
  const uint64_t bytes = std::max<uint64_t>(LBF_HEADER_BYTES, L.n_esc + (L.blob_bytes - L.off_idx));
  a.waves = std::max(launch_waves(groups, 2, cus, kVerifyWaves), launch_waves(bytes, 16 * kWave, cus, kVerifyWaves));
  hipLaunchKernelGGL(k_word_set, dim3(1), dim3(1), 0, s, flags, 0u);
  hipLaunchKernelGGL(k_verify, dim3(a.waves / kVerifyWaves), dim3(kVerifyWaves * kWave), 0, s, a);
  return hipGetLastError();
}

// ---- CRC-32 ------------------------------------------------------------------

struct CrcArgs {
  const uint8_t* data;
  uint32_t* out;
  uint64_t lines;                  // whole 1 KiB lines
  uint64_t steps;                  // lines per wave, rounded up
  uint32_t tail;                   // bytes after the last whole line (< 1024)
  uint32_t waves;                  // W
  uint32_t pad;                    // steps * W - lines leading zero lines
  uint32_t jump[4];                // x^(8 (1024 W - 1 - k)): byte k of a register carried W lines on
  uint32_t lane_end[kWave];        // x^(8 (1024 - 16 (l + 1) + tail)): lane l's last segment to the end
  uint32_t tail_end[kWave];        // x^(8 (tail - 16 (l + 1))): lane l's whole tail segment to the end
  uint32_t wave_pow[kCrcPowBits];  // X^(2^k), X = x^(8 * 1024)
};

// S(0, d) of 16 bytes: byte k (memory order) followed by 15 - k more bytes.
__device__ __forceinline__ uint32_t crc_seg16(const uint32_t (*tab)[256], u32x4 d) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int b = 0; b < 4; b++) r ^= tab[15 - 4 * j - b][(w[j] >> (8 * b)) & 0xFFu];
  return r;
}

// The register c carried over W lines (1024 W bytes), the last 16 of them d.
__device__ __forceinline__ uint32_t crc_step(const uint32_t (*tab)[256], uint32_t c, u32x4 d) {
  return tab[16][c & 0xFFu] ^ tab[17][(c >> 8) & 0xFFu] ^ tab[18][(c >> 16) & 0xFFu] ^ tab[19][c >> 24] ^
         crc_seg16(tab, d);
}

__global__ __launch_bounds__(kCrcWaves * kWave) void k_crc32(CrcArgs a) {
  // tab[k], k < 16: register after byte b and k zero bytes, from 0;
  // tab[16 + k]: after byte b and 1024 W - 1 - k zero bytes
  __shared__ uint32_t tab[20][256];
  const uint32_t tid = threadIdx.x;
  uint32_t t0 = tid;
  for (int k = 0; k < 8; k++) t0 = (t0 >> 1) ^ (kCrcPoly & (0u - (t0 & 1u)));
  tab[0][tid] = t0;
#pragma unroll
  for (int k = 0; k < 4; k++) tab[16 + k][tid] = crc_mul(t0, a.jump[k]);
  __syncthreads();
  uint32_t v = t0;
  for (int k = 1; k < 16; k++) {
    v = (v >> 8) ^ tab[0][v & 0xFFu];
    tab[k][tid] = v;
  }
  __syncthreads();

  const uint32_t lane = tid & 63u;
  const uint32_t w = blockIdx.x * kCrcWaves + (tid >> 6);
  // step q of wave w takes padded line q W + w, real line q W + w - pad
  uint64_t q = w < a.pad ? 1 : 0;
  const uint64_t stride = (uint64_t)a.waves * kCrcLine;
  const uint8_t* p = a.data + (q * a.waves + w - a.pad) * kCrcLine + 16u * lane;
  uint32_t c = 0;
  for (; q + 4 <= a.steps; q += 4, p += 4 * stride) {
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 d1 = *reinterpret_cast<const u32x4*>(p + stride);
    const u32x4 d2 = *reinterpret_cast<const u32x4*>(p + 2 * stride);
    const u32x4 d3 = *reinterpret_cast<const u32x4*>(p + 3 * stride);
    c = crc_step(tab, c, d0);
    c = crc_step(tab, c, d1);
    c = crc_step(tab, c, d2);
    c = crc_step(tab, c, d3);
  }
  for (; q < a.steps; q++, p += stride) c = crc_step(tab, c, *reinterpret_cast<const u32x4*>(p));

  // move every lane's register to the message end and XOR them over the wave
  uint32_t u = crc_mul(c, a.lane_end[lane]);
  const uint32_t e = a.waves - 1 - w;  // X^e moves the wave's last line to the last line
  uint32_t f = (lane < (uint32_t)kCrcPowBits && ((e >> lane) & 1u)) ? a.wave_pow[lane] : kCrcOne;
  for (int o = 1; o < kCrcPowBits; o <<= 1) f = crc_mul(f, (uint32_t)__shfl_xor((int)f, o, kWave));
  for (int o = 32; o >= 1; o >>= 1) u ^= (uint32_t)__shfl_xor((int)u, o, kWave);
  uint32_t total = crc_mul(u, (uint32_t)__shfl((int)f, 0, kWave));

  if (w == a.waves - 1 && a.tail) {  // the bytes after the last whole line
    const uint32_t s0 = 16u * lane;
    uint32_t t = 0;
    if (s0 < a.tail) {
      const uint8_t* tp = a.data + a.lines * kCrcLine + s0;
      if (s0 + 16 <= a.tail) {
        t = crc_mul(crc_seg16(tab, *reinterpret_cast<const u32x4*>(tp)), a.tail_end[lane]);
      } else {
        for (uint32_t i = 0; s0 + i < a.tail; i++) t = tab[0][(t ^ tp[i]) & 0xFFu] ^ (t >> 8);
      }
    }
    for (int o = 32; o >= 1; o >>= 1) t ^= (uint32_t)__shfl_xor((int)t, o, kWave);
    total ^= t;
  }
  if (lane == 0 && total) atomicXor(a.out, total);
}

// x^(8 m) modulo the polynomial, by square and multiply.
static uint32_t crc_xpow8(uint64_t m) {
  uint32_t r = kCrcOne, b = kCrcX;
  for (uint64_t e = m << 3; e; e >>= 1) {
    if (e & 1u) r = crc_mul(r, b);
    b = crc_mul(b, b);
  }
  return r;
}

hipError_t launch_crc32(const uint8_t* data, uint64_t n, uint32_t* crc, hipStream_t s) {
  // zlib's CRC is S(~0, M) ^ ~0 = ~0 * x^(8 n) + S(0, M) + ~0: the constant
  // part is written first, the kernel XORs S(0, M) into it
  hipLaunchKernelGGL(k_word_set, dim3(1), dim3(1), 0, s, crc, crc_mul(0xFFFFFFFFu, crc_xpow8(n)) ^ 0xFFFFFFFFu);
  if (!n) return hipGetLastError();
  int cus = 0;
  if (device_cus(&cus) != hipSuccess) return hipErrorUnknown;
  CrcArgs a;
  a.data = data;
  a.out = crc;
  a.lines = n / kCrcLine;
  a.tail = (uint32_t)(n % kCrcLine);
  a.waves = launch_waves(a.lines, 16, cus, kCrcWaves);
  a.steps = (a.lines + a.waves - 1) / a.waves;
  a.pad = (uint32_t)(a.steps * a.waves - a.lines);
  const uint32_t x8 = crc_xpow8(1), z16 = crc_xpow8(16);
  a.jump[3] = crc_xpow8((uint64_t)kCrcLine * a.waves - 4);
  for (int k = 2; k >= 0; k--) a.jump[k] = crc_mul(a.jump[k + 1], x8);
  uint32_t m = crc_xpow8(a.tail);
  for (int l = kWave - 1; l >= 0; l--, m = crc_mul(m, z16)) a.lane_end[l] = m;
  for (int l = 0; l < kWave; l++) a.tail_end[l] = kCrcOne;
  m = crc_xpow8(a.tail % 16);
  for (int l = (int)(a.tail / 16) - 1; l >= 0; l--, m = crc_mul(m, z16)) a.tail_end[l] = m;
  m = crc_xpow8(kCrcLine);
  for (int k = 0; k < kCrcPowBits; k++, m = crc_mul(m, m)) a.wave_pow[k] = m;
  hipLaunchKernelGGL(k_crc32, dim3(a.waves / kCrcWaves), dim3(kCrcWaves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace lbf
