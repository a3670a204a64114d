/*
 * lbf_oracle.c — CPU oracle for lossless byte-split BF16 weight coding.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, calls or includes anything from this directory, and this file shares
 * no code, header or table with it.  Everything here is plain, scalar,
 * single-threaded C99 written to be checked against the method by eye.
 *
 * What the method computes (sources are the pages this project follows):
 *  - "Lossless LLM Weight Compression vs 8-bit GGUF" (wavect.io, English),
 *    section "What does 'lossless' mean for LLM weights?": the coded form must
 *    rebuild every bit of the source BF16 tensor; decoding is a round trip.
 *  - same page, section "What did the GLM-5.2 experiment actually prove?":
 *    a BF16 weight splits into sign (1 bit), exponent (8) and mantissa (7);
 *    since trained tensors concentrate on few exponent values, the frequent
 *    ones are given fixed-width short codes and the infrequent ones are stored
 *    verbatim in a separate escape stream.
 *  - same page, opening section ("The short answer"): the byte-split
 *    representation, rebuilt bit-for-bit; "K15" names a 15-symbol alphabet.
 *  - "你的 bf16 模型,有 5 個 bit 是廢的" (meowlab), section 一: the field
 *    table (sign 1, exponent 8, mantissa 7) and the order-0 entropy used as a
 *    lower bound for any code that stores each weight independently.
 *
 * Readings taken where the pages are silent:
 *  - only the 8-bit exponent is coded; sign and mantissa stay in the raw
 *    plane, one byte per weight: weight i's byte holds its mantissa in bits
 *    7..1 and, in bit 0, the sign of its pair partner i ^ 1 (weights pair up
 *    as 2j, 2j+1; a missing partner past the end counts as +0.0);
 *  - the alphabet is the 15 most frequent exponents (count descending, ties to
 *    the smaller exponent); codes 0..n_codes-1 go to them in ascending
 *    exponent order; code 15 means "escape";
 *  - an escape stores the full 8-bit exponent as one byte, in flat element
 *    order; tiles are 1024 consecutive weights and a uint32 prefix-sum index
 *    idx[t] gives where tile t's escapes start (idx[n_t] = number of escapes);
 *  - codes go in groups of 8 weights, one 4-byte word per group: weight
 *    8g + j (j = 0..3) has the low nibble and weight 8g + 4 + j the high
 *    nibble of nibble-plane byte 4g + j.
 *
 * Blob layout (format v1), all integers little-endian:
 *   [0,256)             header (see put_header)
 *   [off_raw, ...)      raw plane: n bytes, padded to n_t*1024 (padding weights
 *                       are +0.0 with code 0; byte n carries sign n-1 if n is odd)
 *   [off_nib, ...)      nibble plane: n_t*512 bytes (codes of padding are 0)
 *   [off_idx, ...)      idx plane: uint32[n_t + 1]
 *   [off_esc, ...)      escape stream: n_esc bytes
 * Every plane starts at a multiple of 256 and blob_bytes is a multiple of 256.
 *
 * The header's 96 meaningful bytes:
 *   0 u32 magic 0x3146424C ("LBF1") | 4 u16 version 1 | 6 u16 tile_log2 10
 *   8 u64 rows | 16 u64 cols | 24 u64 n_esc | 32 u64 off_raw | 40 u64 off_nib
 *   48 u64 off_idx | 56 u64 off_esc | 64 u64 blob_bytes | 72 u8 lut[16]
 *   88 u8 n_codes | 89..91 zero | 92 u32 CRC-32 of bytes [0,92); rest zero.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define TILE 1024u
#define HEADER 256u

/* ---- small helpers --------------------------------------------------- */

static uint64_t round_up_256(uint64_t v) { return (v + 255u) / 256u * 256u; }

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 3; i >= 0; i--) v = (v << 8) | p[i];
  return v;
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
  return v;
}

/* CRC-32 (IEEE 802.3, reflected polynomial 0xEDB88320), bit by bit. */
uint32_t lbfo_crc32(const uint8_t* data, uint64_t len) {
  uint32_t crc = 0xFFFFFFFFu;
  for (uint64_t i = 0; i < len; i++) {
    crc ^= data[i];
    for (int b = 0; b < 8; b++) crc = (crc & 1u) ? (crc >> 1) ^ 0xEDB88320u : crc >> 1;
  }
  return ~crc;
}

/* ---- the three BF16 fields (meowlab page, section 一, field table) ---- */

static unsigned sign_of(uint16_t w) { return (w >> 15) & 1u; }
static unsigned exponent_of(uint16_t w) { return (w >> 7) & 0xFFu; }
static unsigned mantissa_of(uint16_t w) { return w & 0x7Fu; }

/* ---- step 1: exponent histogram -------------------------------------- */

void lbfo_histogram(const uint16_t* w, uint64_t n, uint64_t hist[256]) {
  for (int e = 0; e < 256; e++) hist[e] = 0;
  for (uint64_t i = 0; i < n; i++) hist[exponent_of(w[i])]++;
}

/* ---- step 2: the code table (frequent exponents get 4-bit codes) ------
 * Pick up to 15 exponents: repeatedly take the most frequent exponent not yet
 * taken; a tie goes to the smaller exponent (the scan runs upward and only a
 * strictly larger count replaces the current best).  Exponents that never
 * occur are never taken.  Codes are then handed out in ascending exponent
 * order.  Unused table slots, and slot 15 (escape), hold 0.
 */
void lbfo_code_table(const uint64_t hist[256], uint8_t lut[16], uint8_t* n_codes) {
  int taken[256] = {0};
  int chosen = 0;
  for (int round = 0; round < 15; round++) {
    int best = -1;
    for (int e = 0; e < 256; e++) {
      if (taken[e] || hist[e] == 0) continue;
      if (best < 0 || hist[e] > hist[best]) best = e;
    }
    if (best < 0) break;
    taken[best] = 1;
    chosen++;
  }
  for (int c = 0; c < 16; c++) lut[c] = 0;
  int c = 0;
  for (int e = 0; e < 256; e++)
    if (taken[e]) lut[c++] = (uint8_t)e;
  *n_codes = (uint8_t)chosen;
}

/* where weight i's 4-bit code lives: byte of the nibble plane and shift */
static uint64_t code_byte(uint64_t i) { return (i / 8) * 4 + (i % 4); }
static unsigned code_shift(uint64_t i) { return (unsigned)((i % 8) / 4) * 4u; }

/* the code an exponent gets: its slot in the table, or 15 (escape) */
static unsigned code_of(unsigned e, const uint8_t lut[16], unsigned n_codes) {
  for (unsigned c = 0; c < n_codes; c++)
    if (lut[c] == e) return c;
  return 15u;
}

/* ---- sizes ----------------------------------------------------------- */

typedef struct {
  uint64_t n, n_tiles, n_esc;
  uint64_t off_raw, off_nib, off_idx, off_esc, blob_bytes;
} layout_t;

static layout_t layout_for(uint64_t rows, uint64_t cols, uint64_t n_esc) {
  layout_t L;
  L.n = rows * cols;
  L.n_tiles = (L.n + TILE - 1) / TILE;
  L.n_esc = n_esc;
  L.off_raw = HEADER;
  L.off_nib = round_up_256(L.off_raw + L.n_tiles * TILE);
  L.off_idx = round_up_256(L.off_nib + L.n_tiles * (TILE / 2));
  L.off_esc = round_up_256(L.off_idx + 4u * (L.n_tiles + 1));
  L.blob_bytes = round_up_256(L.off_esc + n_esc);
  return L;
}

/* Escape count: weights whose exponent did not get a code. */
static uint64_t escape_count(const uint64_t hist[256], const uint8_t lut[16], unsigned n_codes) {
  uint64_t n = 0;
  for (int e = 0; e < 256; e++)
    if (code_of((unsigned)e, lut, n_codes) == 15u) n += hist[e];
  return n;
}

/* Everything the encoder decides before writing: table, escape count, size. */
int lbfo_plan(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t lut[16], uint8_t* n_codes,
              uint64_t* n_esc, uint64_t* blob_bytes) {
  uint64_t hist[256];
  if (cols != 0 && rows > UINT64_MAX / cols) return -1;
  uint64_t n = rows * cols;
  if (n >= (1ull << 32)) return -1; /* uint32 escape index */
  lbfo_histogram(w, n, hist);
  lbfo_code_table(hist, lut, n_codes);
  *n_esc = escape_count(hist, lut, *n_codes);
  *blob_bytes = layout_for(rows, cols, *n_esc).blob_bytes;
  return 0;
}

/* ---- step 3: write the blob ------------------------------------------ */

static void put_header(uint8_t* blob, uint64_t rows, uint64_t cols, const layout_t* L,
                       const uint8_t lut[16], uint8_t n_codes) {
  memset(blob, 0, HEADER);
  put_u32(blob + 0, 0x3146424Cu);
  put_u16(blob + 4, 1);
  put_u16(blob + 6, 10);
  put_u64(blob + 8, rows);
  put_u64(blob + 16, cols);
  put_u64(blob + 24, L->n_esc);
  put_u64(blob + 32, L->off_raw);
  put_u64(blob + 40, L->off_nib);
  put_u64(blob + 48, L->off_idx);
  put_u64(blob + 56, L->off_esc);
  put_u64(blob + 64, L->blob_bytes);
  memcpy(blob + 72, lut, 16);
  blob[88] = n_codes;
  put_u32(blob + 92, lbfo_crc32(blob, 92));
}

int lbfo_encode(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* blob, uint64_t blob_cap) {
  uint8_t lut[16], n_codes;
  uint64_t n_esc, blob_bytes;
  if (lbfo_plan(w, rows, cols, lut, &n_codes, &n_esc, &blob_bytes) != 0) return -1;
  if (blob_cap < blob_bytes) return -2;
  layout_t L = layout_for(rows, cols, n_esc);
  memset(blob, 0, blob_bytes);
  put_header(blob, rows, cols, &L, lut, n_codes);

  uint8_t* raw = blob + L.off_raw;
  uint8_t* nib = blob + L.off_nib;
  uint8_t* idx = blob + L.off_idx;
  uint8_t* esc = blob + L.off_esc;
  uint64_t* tile_escapes = (uint64_t*)calloc(L.n_tiles + 1, sizeof(uint64_t));
  if (!tile_escapes) return -3;

  uint64_t written = 0;
  for (uint64_t i = 0; i < L.n; i++) {
    unsigned s = sign_of(w[i]), e = exponent_of(w[i]), m = mantissa_of(w[i]);
    raw[i] |= (uint8_t)(m << 1);
    raw[i ^ 1u] |= (uint8_t)s; /* the partner's byte carries this sign */
    unsigned code = code_of(e, lut, n_codes);
    nib[code_byte(i)] |= (uint8_t)(code << code_shift(i));
    if (code == 15u) {
      esc[written++] = (uint8_t)e; /* flat element order */
      tile_escapes[i / TILE]++;
    }
  }
  /* prefix-sum index: idx[0] = 0, idx[t+1] = idx[t] + escapes in tile t */
  uint64_t run = 0;
  put_u32(idx, 0);
  for (uint64_t t = 0; t < L.n_tiles; t++) {
    run += tile_escapes[t];
    put_u32(idx + 4u * (t + 1), (uint32_t)run);
  }
  free(tile_escapes);
  return (written == n_esc && run == n_esc) ? 0 : -4;
}

/* ---- header reading (used by decode) ---------------------------------- */

int lbfo_read_header(const uint8_t* blob, uint64_t blob_len, uint64_t* rows, uint64_t* cols,
                     uint64_t* n_esc, uint8_t lut[16], uint8_t* n_codes) {
  if (blob_len < HEADER) return -1;
  if (get_u32(blob) != 0x3146424Cu) return -1;
  if (blob[4] != 1 || blob[5] != 0 || blob[6] != 10 || blob[7] != 0) return -1;
  if (get_u32(blob + 92) != lbfo_crc32(blob, 92)) return -1;
  *rows = get_u64(blob + 8);
  *cols = get_u64(blob + 16);
  *n_esc = get_u64(blob + 24);
  memcpy(lut, blob + 72, 16);
  *n_codes = blob[88];
  if (*n_codes > 15) return -1;
  if (*cols != 0 && *rows > UINT64_MAX / *cols) return -1;
  if (*rows * *cols >= (1ull << 32)) return -1;
  layout_t L = layout_for(*rows, *cols, *n_esc);
  if (get_u64(blob + 32) != L.off_raw || get_u64(blob + 40) != L.off_nib ||
      get_u64(blob + 48) != L.off_idx || get_u64(blob + 56) != L.off_esc ||
      get_u64(blob + 64) != L.blob_bytes || blob_len < L.blob_bytes)
    return -1;
  return 0;
}

/* ---- decode: rebuild each weight from its raw byte and its exponent ---- */

int lbfo_decode(const uint8_t* blob, uint64_t blob_len, uint16_t* out, uint64_t out_len) {
  uint64_t rows, cols, n_esc;
  uint8_t lut[16], n_codes;
  if (lbfo_read_header(blob, blob_len, &rows, &cols, &n_esc, lut, &n_codes) != 0) return -1;
  layout_t L = layout_for(rows, cols, n_esc);
  if (out_len < L.n) return -2;
  const uint8_t* raw = blob + L.off_raw;
  const uint8_t* nib = blob + L.off_nib;
  const uint8_t* idx = blob + L.off_idx;
  const uint8_t* esc = blob + L.off_esc;
  if (get_u32(idx) != 0 || get_u32(idx + 4u * L.n_tiles) != n_esc) return -3;

  for (uint64_t t = 0; t < L.n_tiles; t++) {
    uint64_t first = get_u32(idx + 4u * t), last = get_u32(idx + 4u * (t + 1));
    if (last < first || last > n_esc) return -3;
    uint64_t seen = 0; /* escapes met so far inside this tile */
    uint64_t end = (t + 1) * TILE < L.n ? (t + 1) * TILE : L.n;
    for (uint64_t i = t * TILE; i < end; i++) {
      unsigned code = (nib[code_byte(i)] >> code_shift(i)) & 15u;
      unsigned e;
      if (code == 15u) {
        if (first + seen >= last) return -3;
        e = esc[first + seen];
        seen++;
      } else {
        if (code >= n_codes) return -3;
        e = lut[code];
      }
      unsigned s = raw[i ^ 1u] & 1u, m = raw[i] >> 1;
      out[i] = (uint16_t)((s << 15) | (e << 7) | m);
    }
    if (first + seen != last) return -3;
  }
  return 0;
}

/* ---- verification without decoding -------------------------------------
 * Checks a blob against the 96 descriptor bytes the caller trusts (corruption
 * must be detected and refused: "Lossless LLM Weight Compression vs 8-bit
 * GGUF", sections "Is the GLM-5.2 result production-ready?" and "Questions to
 * ask a vendor or research team").  Each failed check sets one bit:
 *    1  header: bytes [0,96) differ from desc96, or [96,256) are not zero
 *    2  index: idx[0] != 0, idx decreases, or idx[n_t] != n_esc
 *    4  count: a tile holds a number of code-15 nibbles other than
 *       idx[t+1] - idx[t]
 *    8  code: a nibble of a real weight holds an unused code (n_codes..14)
 *   16  escape: an escape byte equals a coded exponent (escapes are, by
 *       definition, the exponents outside the table)
 *   32  padding: a byte the format defines as zero is not (raw and code bits of
 *       padding weights past n; the gap after the index; bytes after the
 *       escape stream up to blob_bytes)
 * The raw sign/mantissa bytes of real weights carry no redundancy: only a
 * hash of the blob (lbfo_crc32) catches changes there.
 * desc96 must describe a layout that fits blob_len (else the result is 1).
 */
unsigned lbfo_verify(const uint8_t* blob, uint64_t blob_len, const uint8_t desc96[96]) {
  unsigned bad = 0;
  uint64_t rows = get_u64(desc96 + 8), cols = get_u64(desc96 + 16), n_esc = get_u64(desc96 + 24);
  unsigned n_codes = desc96[88];
  const uint8_t* lut = desc96 + 72;
  if (n_codes > 15 || (cols != 0 && rows > UINT64_MAX / cols) || rows * cols >= (1ull << 32)) return 1;
  layout_t L = layout_for(rows, cols, n_esc);
  if (blob_len < L.blob_bytes) return 1;

  if (memcmp(blob, desc96, 96) != 0) bad |= 1u;
  for (uint64_t i = 96; i < HEADER; i++)
    if (blob[i] != 0) bad |= 1u;

  const uint8_t* raw = blob + L.off_raw;
  const uint8_t* nib = blob + L.off_nib;
  const uint8_t* idx = blob + L.off_idx;
  const uint8_t* esc = blob + L.off_esc;
  if (get_u32(idx) != 0 || get_u32(idx + 4u * L.n_tiles) != n_esc) bad |= 2u;
  for (uint64_t t = 0; t < L.n_tiles; t++) {
    uint32_t a = get_u32(idx + 4u * t), b = get_u32(idx + 4u * (t + 1));
    if (b < a) bad |= 2u;
    uint64_t fifteens = 0;
    for (uint64_t i = t * TILE; i < (t + 1) * TILE; i++) {
      unsigned code = (nib[code_byte(i)] >> code_shift(i)) & 15u;
      if (i >= L.n) {
        if (code != 0) bad |= 32u;
        continue;
      }
      if (code == 15u)
        fifteens++;
      else if (code >= n_codes)
        bad |= 8u;
    }
    if (b >= a && fifteens != (uint64_t)(b - a)) bad |= 4u;
    if (b < a && fifteens != 0) bad |= 4u;
  }
  /* padding weights: mantissa bits 0; the sign bit of byte i is weight i^1's,
     so byte n (n odd) may carry the sign of weight n - 1 */
  for (uint64_t i = L.n; i < L.n_tiles * TILE; i++) {
    uint8_t allowed = (i == L.n && (L.n & 1u)) ? 1u : 0u;
    if (raw[i] & (uint8_t)~allowed) bad |= 32u;
  }
  for (uint64_t j = 0; j < n_esc; j++)
    if (code_of(esc[j], lut, n_codes) != 15u) bad |= 16u;
  for (uint64_t i = L.off_idx + 4u * (L.n_tiles + 1); i < L.off_esc; i++)
    if (blob[i] != 0) bad |= 32u;
  for (uint64_t i = L.off_esc + n_esc; i < L.blob_bytes; i++)
    if (blob[i] != 0) bad |= 32u;
  return bad;
}

/* ---- y = W x in float64 ------------------------------------------------
 * y[b*rows + r] = sum_k W[r,k] * x[b,k], summed in k order in double;
 * a[b*rows + r] = sum_k |W[r,k]| * |x[b,k]|, the scale the error bound uses.
 * W is row-major [rows x cols]; x is row-major [batch x cols]; both bf16.
 */
static double bf16_to_double(uint16_t v) {
  uint32_t bits = (uint32_t)v << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

void lbfo_matvec(const uint16_t* W, uint64_t rows, uint64_t cols, const uint16_t* x, uint64_t batch,
                 double* y, double* a) {
  for (uint64_t b = 0; b < batch; b++) {
    for (uint64_t r = 0; r < rows; r++) {
      double sum = 0.0, mag = 0.0;
      for (uint64_t k = 0; k < cols; k++) {
        double wv = bf16_to_double(W[r * cols + k]);
        double xv = bf16_to_double(x[b * cols + k]);
        sum += wv * xv;
        mag += fabs(wv) * fabs(xv);
      }
      y[b * rows + r] = sum;
      if (a) a[b * rows + r] = mag;
    }
  }
}

/* Same product, rows [r0, r1) only (lets a caller sample rows of a big W). */
void lbfo_matvec_rows(const uint16_t* W, uint64_t rows, uint64_t cols, uint64_t r0, uint64_t r1,
                      const uint16_t* x, uint64_t batch, double* y, double* a) {
  for (uint64_t b = 0; b < batch; b++) {
    for (uint64_t r = r0; r < r1 && r < rows; r++) {
      double sum = 0.0, mag = 0.0;
      for (uint64_t k = 0; k < cols; k++) {
        double wv = bf16_to_double(W[r * cols + k]);
        double xv = bf16_to_double(x[b * cols + k]);
        sum += wv * xv;
        mag += fabs(wv) * fabs(xv);
      }
      y[b * (r1 - r0) + (r - r0)] = sum;
      if (a) a[b * (r1 - r0) + (r - r0)] = mag;
    }
  }
}

/* ---- order-0 entropy of the 16-bit values, in bits per weight ----------
 * (meowlab page, section 二: the lower bound for any code that stores each
 * weight on its own)  H0 = -sum_v p_v log2 p_v over the 65,536 patterns.
 */
double lbfo_entropy16(const uint16_t* w, uint64_t n) {
  if (n == 0) return 0.0;
  uint64_t* count = (uint64_t*)calloc(65536, sizeof(uint64_t));
  if (!count) return -1.0;
  for (uint64_t i = 0; i < n; i++) count[w[i]]++;
  double h = 0.0;
  for (int v = 0; v < 65536; v++) {
    if (count[v] == 0) continue;
    double p = (double)count[v] / (double)n;
    h -= p * log2(p);
  }
  free(count);
  return h;
}

/* Order-0 entropy of the exponent field alone (same page, section 一 table). */
double lbfo_entropy_exponent(const uint16_t* w, uint64_t n) {
  if (n == 0) return 0.0;
  uint64_t hist[256];
  lbfo_histogram(w, n, hist);
  double h = 0.0;
  for (int e = 0; e < 256; e++) {
    if (hist[e] == 0) continue;
    double p = (double)hist[e] / (double)n;
    h -= p * log2(p);
  }
  return h;
}

/* ---- the entropy-coded variant (K15H) ----------------------------------
 * The English page's larger "K15" reduction belongs to an entropy-coded form
 * of the same split (opening section), and DFloat11 entropy-codes the
 * exponent while sign and mantissa stay raw (meowlab page, section 二).  Here
 * the 4-bit K15 code of every weight (codes 0..14 for the table's exponents,
 * 15 for an escape, exactly as above) is Huffman-coded; the raw plane, the
 * escape index and the escape stream are those of format v1.
 * Readings taken where the pages are silent:
 *  - symbol counts are over the n real weights (not the tile padding);
 *  - code lengths come from Huffman's procedure run with two queues: the used
 *    symbols sorted by count, then by symbol, and the merged nodes in the
 *    order they are made; each step merges the two lightest queue fronts, the
 *    leaf queue winning a tie.  A lone used symbol gets length 1.  With at
 *    most 16 symbols no length exceeds 15;
 *  - codes are canonical as RFC 1951 section 3.2.2 defines them: shorter
 *    codes first, equal lengths in symbol order, consecutive values;
 *  - a code is written most significant bit first into a bit stream whose
 *    bit k is bit k % 32 of 32-bit word k / 32 (little-endian words);
 *  - each 1024-weight tile is its own stream of whole words, its codes in
 *    element order, unused bits zero; woff[t] is the first word of tile t,
 *    woff[n_t] the total word count.
 * Blob layout (K15H), every plane starting at a multiple of 256:
 *   [0,256)      header, 128 meaningful bytes, then zeros:
 *                0 u32 magic 0x4846424C ("LBFH") | 4 u16 version 1 |
 *                6 u16 tile_log2 10 | 8 u64 rows | 16 u64 cols | 24 u64 n_esc |
 *                32 u64 off_raw | 40 u64 off_bits | 48 u64 off_woff |
 *                56 u64 off_idx | 64 u64 off_esc | 72 u64 blob_bytes |
 *                80 u64 stream_words | 88 u8 lut[16] | 104 u8 n_codes |
 *                105 u8 max_len | 106..107 zero | 108 u8 len[16] |
 *                124 u32 CRC-32 of bytes [0,124)
 *   off_raw      raw plane, as format v1 (n_t * 1024 bytes)
 *   off_bits     code stream, stream_words 32-bit words
 *   off_woff     uint32 woff[n_t + 1]
 *   off_idx      uint32 idx[n_t + 1], as format v1
 *   off_esc      escape stream, as format v1
 */

/* Huffman code lengths of 16 symbols from their counts (two-queue form). */
void lbfo_huffman_lengths(const uint64_t count[16], uint8_t len[16]) {
  int leaf_sym[16], m = 0;
  uint64_t weight[31];
  int parent[31];
  memset(len, 0, 16);
  for (int s = 0; s < 16; s++)
    if (count[s] > 0) leaf_sym[m++] = s;
  if (m == 0) return;
  if (m == 1) {
    len[leaf_sym[0]] = 1;
    return;
  }
  /* leaves sorted by (count, symbol): insertion sort, stable on symbol */
  for (int i = 1; i < m; i++) {
    int s = leaf_sym[i], j = i - 1;
    while (j >= 0 && count[leaf_sym[j]] > count[s]) {
      leaf_sym[j + 1] = leaf_sym[j];
      j--;
    }
    leaf_sym[j + 1] = s;
  }
  for (int i = 0; i < m; i++) {
    weight[i] = count[leaf_sym[i]];
    parent[i] = -1;
  }
  int next_leaf = 0, next_node = m, made = m;
  for (int step = 0; step < m - 1; step++) {
    int pick[2];
    for (int k = 0; k < 2; k++) {
      int leaf_ok = next_leaf < m, node_ok = next_node < made;
      if (leaf_ok && (!node_ok || weight[next_leaf] <= weight[next_node]))
        pick[k] = next_leaf++;
      else
        pick[k] = next_node++;
    }
    weight[made] = weight[pick[0]] + weight[pick[1]];
    parent[made] = -1;
    parent[pick[0]] = parent[pick[1]] = made;
    made++;
  }
  for (int i = 0; i < m; i++) {
    int depth = 0;
    for (int k = i; parent[k] >= 0; k = parent[k]) depth++;
    len[leaf_sym[i]] = (uint8_t)depth;
  }
}

/* Canonical code values from lengths (RFC 1951, section 3.2.2). */
void lbfo_canonical_codes(const uint8_t len[16], uint16_t code[16]) {
  unsigned bl_count[16] = {0}, next_code[16] = {0};
  for (int s = 0; s < 16; s++)
    if (len[s]) bl_count[len[s]]++;
  unsigned c = 0;
  for (int bits = 1; bits < 16; bits++) {
    c = (c + bl_count[bits - 1]) << 1;
    next_code[bits] = c;
  }
  for (int s = 0; s < 16; s++) code[s] = len[s] ? (uint16_t)next_code[len[s]]++ : 0;
}

typedef struct {
  uint64_t n, n_tiles, n_esc, stream_words;
  uint64_t off_raw, off_bits, off_woff, off_idx, off_esc, blob_bytes;
} hlayout_t;

static hlayout_t hlayout_for(uint64_t rows, uint64_t cols, uint64_t n_esc, uint64_t stream_words) {
  hlayout_t L;
  L.n = rows * cols;
  L.n_tiles = (L.n + TILE - 1) / TILE;
  L.n_esc = n_esc;
  L.stream_words = stream_words;
  L.off_raw = HEADER;
  L.off_bits = round_up_256(L.off_raw + L.n_tiles * TILE);
  L.off_woff = round_up_256(L.off_bits + 4u * stream_words);
  L.off_idx = round_up_256(L.off_woff + 4u * (L.n_tiles + 1));
  L.off_esc = round_up_256(L.off_idx + 4u * (L.n_tiles + 1));
  L.blob_bytes = round_up_256(L.off_esc + n_esc);
  return L;
}

/* The K15 code of every real weight, read from a format-v1 blob. */
static unsigned v1_code(const uint8_t* nib, uint64_t i) { return (nib[code_byte(i)] >> code_shift(i)) & 15u; }

/* Everything the K15H encoder decides before writing: the v1 plan, the code
 * counts, the code lengths, the stream size and the blob size. */
int lbfo_hplan(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t code_count[16], uint8_t len[16],
               uint64_t* stream_words, uint64_t* blob_bytes) {
  uint8_t lut[16], n_codes;
  uint64_t n_esc, v1_bytes;
  if (lbfo_plan(w, rows, cols, lut, &n_codes, &n_esc, &v1_bytes) != 0) return -1;
  uint64_t n = rows * cols;
  memset(code_count, 0, 16 * sizeof(uint64_t));
  for (uint64_t i = 0; i < n; i++) code_count[code_of(exponent_of(w[i]), lut, n_codes)]++;
  lbfo_huffman_lengths(code_count, len);
  uint64_t words = 0;
  for (uint64_t t = 0; t * TILE < n; t++) {
    uint64_t bits = 0, end = (t + 1) * TILE < n ? (t + 1) * TILE : n;
    for (uint64_t i = t * TILE; i < end; i++) bits += len[code_of(exponent_of(w[i]), lut, n_codes)];
    words += (bits + 31) / 32;
  }
  *stream_words = words;
  *blob_bytes = hlayout_for(rows, cols, n_esc, words).blob_bytes;
  return 0;
}

/* Write the K15H blob of w: the v1 blob first (raw plane, codes, index,
 * escapes), then its codes re-written as Huffman codes tile by tile. */
int lbfo_hencode(const uint16_t* w, uint64_t rows, uint64_t cols, uint8_t* blob, uint64_t blob_cap) {
  uint64_t code_count[16], words, bytes, v1_bytes, n_esc;
  uint8_t len[16], lut[16], n_codes;
  uint16_t code[16];
  if (lbfo_hplan(w, rows, cols, code_count, len, &words, &bytes) != 0) return -1;
  if (blob_cap < bytes) return -2;
  if (lbfo_plan(w, rows, cols, lut, &n_codes, &n_esc, &v1_bytes) != 0) return -1;
  uint8_t* v1 = (uint8_t*)malloc(v1_bytes);
  if (!v1) return -3;
  if (lbfo_encode(w, rows, cols, v1, v1_bytes) != 0) {
    free(v1);
    return -4;
  }
  layout_t V = layout_for(rows, cols, n_esc);
  hlayout_t L = hlayout_for(rows, cols, n_esc, words);
  lbfo_canonical_codes(len, code);
  unsigned max_len = 0;
  for (int s = 0; s < 16; s++)
    if (len[s] > max_len) max_len = len[s];

  memset(blob, 0, bytes);
  put_u32(blob + 0, 0x4846424Cu);
  put_u16(blob + 4, 1);
  put_u16(blob + 6, 10);
  put_u64(blob + 8, rows);
  put_u64(blob + 16, cols);
  put_u64(blob + 24, n_esc);
  put_u64(blob + 32, L.off_raw);
  put_u64(blob + 40, L.off_bits);
  put_u64(blob + 48, L.off_woff);
  put_u64(blob + 56, L.off_idx);
  put_u64(blob + 64, L.off_esc);
  put_u64(blob + 72, L.blob_bytes);
  put_u64(blob + 80, words);
  memcpy(blob + 88, lut, 16);
  blob[104] = n_codes;
  blob[105] = (uint8_t)max_len;
  memcpy(blob + 108, len, 16);
  put_u32(blob + 124, lbfo_crc32(blob, 124));

  memcpy(blob + L.off_raw, v1 + V.off_raw, L.n_tiles * TILE);
  memcpy(blob + L.off_idx, v1 + V.off_idx, 4u * (L.n_tiles + 1));
  memcpy(blob + L.off_esc, v1 + V.off_esc, n_esc);

  uint8_t* bits = blob + L.off_bits;
  uint8_t* woff = blob + L.off_woff;
  uint64_t word = 0; /* first word of the current tile */
  for (uint64_t t = 0; t < L.n_tiles; t++) {
    put_u32(woff + 4u * t, (uint32_t)word);
    uint64_t k = 0; /* bit position inside the tile's stream */
    uint64_t end = (t + 1) * TILE < L.n ? (t + 1) * TILE : L.n;
    for (uint64_t i = t * TILE; i < end; i++) {
      unsigned s = v1_code(v1 + V.off_nib, i);
      for (int b = len[s] - 1; b >= 0; b--, k++) { /* most significant bit first */
        if ((code[s] >> b) & 1u) {
          uint64_t at = 4u * (word + k / 32) + (k % 32) / 8; /* byte of the little-endian word */
          bits[at] |= (uint8_t)(1u << (k % 8));
        }
      }
    }
    word += (k + 31) / 32;
  }
  put_u32(woff + 4u * L.n_tiles, (uint32_t)word);
  free(v1);
  return word == words ? 0 : -5;
}

/* Read and check a K15H header: magic, version, CRC, shape, table, lengths
 * (a complete prefix code when two or more symbols are used) and layout. */
int lbfo_hread_header(const uint8_t* blob, uint64_t blob_len, uint64_t* rows, uint64_t* cols, uint64_t* n_esc,
                      uint64_t* stream_words, uint8_t lut[16], uint8_t* n_codes, uint8_t len[16]) {
  if (blob_len < HEADER) return -1;
  if (get_u32(blob) != 0x4846424Cu) return -1;
  if (blob[4] != 1 || blob[5] != 0 || blob[6] != 10 || blob[7] != 0) return -1;
  if (get_u32(blob + 124) != lbfo_crc32(blob, 124)) return -1;
  *rows = get_u64(blob + 8);
  *cols = get_u64(blob + 16);
  *n_esc = get_u64(blob + 24);
  *stream_words = get_u64(blob + 80);
  memcpy(lut, blob + 88, 16);
  *n_codes = blob[104];
  memcpy(len, blob + 108, 16);
  if (*n_codes > 15) return -1;
  if (*cols != 0 && *rows > UINT64_MAX / *cols) return -1;
  if (*rows * *cols >= (1ull << 32)) return -1;
  unsigned used = 0, max_len = 0;
  double kraft = 0.0;
  for (int s = 0; s < 16; s++) {
    if (len[s] > 15) return -1;
    if (!len[s]) continue;
    used++;
    kraft += ldexp(1.0, -(int)len[s]);
    if (len[s] > max_len) max_len = len[s];
  }
  if (blob[105] != max_len) return -1;
  if (used >= 2 && kraft != 1.0) return -1;
  if (used == 1 && max_len != 1) return -1;
  hlayout_t L = hlayout_for(*rows, *cols, *n_esc, *stream_words);
  if (get_u64(blob + 32) != L.off_raw || get_u64(blob + 40) != L.off_bits || get_u64(blob + 48) != L.off_woff ||
      get_u64(blob + 56) != L.off_idx || get_u64(blob + 64) != L.off_esc || get_u64(blob + 72) != L.blob_bytes ||
      blob_len < L.blob_bytes)
    return -1;
  return 0;
}

/* Decode a K15H blob: per tile, read codes bit by bit (a code is complete
 * when its value and length match a symbol's canonical code), then rebuild
 * each weight from its raw byte and its exponent as format v1 does. */
int lbfo_hdecode(const uint8_t* blob, uint64_t blob_len, uint16_t* out, uint64_t out_len) {
  uint64_t rows, cols, n_esc, words;
  uint8_t lut[16], n_codes, len[16];
  uint16_t code[16];
  if (lbfo_hread_header(blob, blob_len, &rows, &cols, &n_esc, &words, lut, &n_codes, len) != 0) return -1;
  hlayout_t L = hlayout_for(rows, cols, n_esc, words);
  if (out_len < L.n) return -2;
  lbfo_canonical_codes(len, code);
  const uint8_t* raw = blob + L.off_raw;
  const uint8_t* bits = blob + L.off_bits;
  const uint8_t* woff = blob + L.off_woff;
  const uint8_t* idx = blob + L.off_idx;
  const uint8_t* esc = blob + L.off_esc;
  if (get_u32(woff) != 0 || get_u32(woff + 4u * L.n_tiles) != words) return -3;
  if (get_u32(idx) != 0 || get_u32(idx + 4u * L.n_tiles) != n_esc) return -3;

  for (uint64_t t = 0; t < L.n_tiles; t++) {
    uint64_t w0 = get_u32(woff + 4u * t), w1 = get_u32(woff + 4u * (t + 1));
    uint64_t first = get_u32(idx + 4u * t), last = get_u32(idx + 4u * (t + 1));
    if (w1 < w0 || w1 > words || last < first || last > n_esc) return -3;
    uint64_t k = 0, limit = 32u * (w1 - w0), seen = 0;
    uint64_t end = (t + 1) * TILE < L.n ? (t + 1) * TILE : L.n;
    for (uint64_t i = t * TILE; i < end; i++) {
      unsigned value = 0, s = 16;
      for (unsigned l = 1; l <= 15 && s == 16; l++) {
        if (k >= limit) return -3;
        uint64_t at = 4u * (w0 + k / 32) + (k % 32) / 8;
        value = (value << 1) | ((bits[at] >> (k % 8)) & 1u);
        k++;
        for (unsigned c = 0; c < 16; c++)
          if (len[c] == l && code[c] == value) s = c;
      }
      if (s == 16) return -3;
      unsigned e;
      if (s == 15u) {
        if (first + seen >= last) return -3;
        e = esc[first + seen++];
      } else {
        if (s >= n_codes) return -3;
        e = lut[s];
      }
      unsigned sg = raw[i ^ 1u] & 1u, m = raw[i] >> 1;
      out[i] = (uint16_t)((sg << 15) | (e << 7) | m);
    }
    if (first + seen != last) return -3;
    for (; k < limit; k++) { /* bits after the tile's last code are zero */
      uint64_t at = 4u * (w0 + k / 32) + (k % 32) / 8;
      if ((bits[at] >> (k % 8)) & 1u) return -3;
    }
  }
  return 0;
}

/* ---- the gated MLP product of the layer ---------------------------------
 * h[b*rows + r] = silu(g) * u with g = sum_k G[r,k] x[b,k], u = sum_k U[r,k]
 * x[b,k] (both as lbfo_matvec, float64) and silu(z) = z / (1 + e^-z): the
 * gate_proj / up_proj pair of the 8B-shaped layer's MLP, whose product feeds
 * down_proj.  Also returns ag, au (sum |G||x|, sum |U||x|) and g, u for the
 * error bound.  Reading: the MLP of the 8B-shaped decoder layer is SwiGLU
 * (the pages name the layer's tensors, not its activation).
 */
double lbfo_silu(double z) { return z / (1.0 + exp(-z)); }

void lbfo_swiglu(const uint16_t* G, const uint16_t* U, uint64_t rows, uint64_t cols, const uint16_t* x,
                 uint64_t batch, double* h, double* g, double* u, double* ag, double* au) {
  lbfo_matvec(G, rows, cols, x, batch, g, ag);
  lbfo_matvec(U, rows, cols, x, batch, u, au);
  for (uint64_t i = 0; i < batch * rows; i++) h[i] = lbfo_silu(g[i]) * u[i];
}
