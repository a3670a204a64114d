/*
 * lbf.h — C ABI of liblbf.so: lossless byte-split BF16 weights decoded on an
 * MI355X (gfx950) straight into the matrix-vector or matrix product.
 *
 * The method (pages this library follows):
 *  - "Lossless LLM Weight Compression vs 8-bit GGUF" (wavect.io, English),
 *    section "What does 'lossless' mean for LLM weights?": coded weights may
 *    stay in GPU memory and be rebuilt, exactly, in registers or shared
 *    memory right before the multiply; the round trip decides losslessness.
 *  - same page, section "What did the GLM-5.2 experiment actually prove?":
 *    BF16 is sign (1) + exponent (8) + mantissa (7) bits; the frequent
 *    exponents get short fixed-width codes and the others go, verbatim, to an
 *    escape stream.
 *  - same page, opening section: the byte-split representation; "K15", read
 *    here as an alphabet of 15 coded symbols plus one escape code.
 *
 * Format v1 (one "blob" per weight tensor, one contiguous device buffer):
 *   [0, 256)        header: the 96-byte lbf_desc below, then zeros
 *   off_raw = 256   raw plane, one byte per weight: mantissa_i << 1 | sign of
 *                   weight i ^ 1 (weights pair up as 2j, 2j + 1; padding
 *                   weights count as +0.0), padded to n_tiles * 1024 bytes
 *   off_nib         nibble plane, one 32-bit word per 8 weights: byte j of
 *                   word g holds the code of weight 8g + j in its low nibble
 *                   and of weight 8g + 4 + j in its high nibble; code c < 15
 *                   means exponent lut[c], code 15 means "next escape byte";
 *                   n_tiles * 512 bytes (padding codes are 0)
 *   off_idx         uint32 idx[n_tiles + 1]: idx[0] = 0 and idx[t + 1] - idx[t]
 *                   is the number of escapes in tile t (1024 weights)
 *   off_esc         escape stream: one exponent byte per escaped weight, in
 *                   flat element order; tile t's escapes are [idx[t], idx[t+1])
 * Each plane starts at a multiple of 256; blob_bytes is a multiple of 256.
 * n = rows * cols, n_tiles = ceil(n / 1024); W is row-major [rows, cols]
 * (rows = out_features, cols = in_features: the nn.Linear layout).
 *
 * Code table: the (up to) 15 most frequent exponents of the tensor, count
 * descending, ties to the smaller exponent; codes are given in ascending
 * exponent order.  Unused lut slots and lut[15] are 0.
 *
 * Conventions for every call:
 *  - d_* arguments are device pointers (or host arrays of device pointers
 *    where the type says so); the caller allocates and owns all memory.  The
 *    library allocates no device memory and keeps no mutable global state
 *    beyond per-device launch facts (CU count, resident workgroups, each
 *    kernel's dynamic LDS limit), looked up once per device under a lock:
 *    calls may be made from several threads and on several devices at once.
 *  - every call checks its arguments and descriptors on the host before it
 *    launches anything and returns a negative LBF_E_* status, with no side
 *    effect, when a check fails.  A failed launch returns LBF_E_HIP.
 *  - every call except encode phase 1 only enqueues work on the stream `s`
 *    (a hipStream_t; NULL is the null stream) and returns.
 *  - identical inputs give bitwise-identical outputs (no floating-point
 *    atomics; fixed reduction order).
 */
#ifndef LBF_H
#define LBF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBF_MAGIC 0x3146424Cu /* "LBF1" little-endian */
#define LBF_VERSION 1
#define LBF_TILE_LOG2 10
#define LBF_TILE 1024
#define LBF_HEADER_BYTES 256
#define LBF_MAX_GROUPS 64 /* groups per kernel launch; larger calls are split */

/* Host copy of a blob's header; byte-for-byte the first 96 bytes of the blob. */
typedef struct lbf_desc {
  uint32_t magic;      /* LBF_MAGIC */
  uint16_t version;    /* LBF_VERSION */
  uint16_t tile_log2;  /* LBF_TILE_LOG2 */
  uint64_t rows, cols; /* W is [rows, cols], row-major; rows * cols < 2^32 */
  uint64_t n_esc;      /* number of escaped weights */
  uint64_t off_raw, off_nib, off_idx, off_esc, blob_bytes;
  uint8_t lut[16];     /* lut[c] = exponent of code c, c < n_codes */
  uint8_t n_codes;     /* 0..15 */
  uint8_t reserved[3]; /* zero */
  uint32_t desc_crc;   /* CRC-32 (IEEE) of the 92 bytes before this field */
} lbf_desc;

enum {
  LBF_OK = 0,
  LBF_E_INVAL = -1,       /* null pointer, bad enum, batch out of range */
  LBF_E_SHAPE = -2,       /* shape not supported by this call, or mismatched */
  LBF_E_ALIGN = -3,       /* a device pointer is not aligned as required */
  LBF_E_DESC = -4,        /* descriptor fails validation (corrupt or foreign) */
  LBF_E_CAPACITY = -5,    /* destination or workspace buffer too small */
  LBF_E_HIP = -6,         /* a HIP runtime call or launch failed */
  LBF_E_UNSUPPORTED = -7  /* valid request the library does not handle */
};

enum { LBF_F32 = 0, LBF_BF16 = 1 }; /* output element types */

/* Human-readable text for a status code (static storage). */
const char* lbf_strerror(int status);

/* Bytes of device workspace lbf_encode needs for a [rows, cols] tensor. */
uint64_t lbf_encode_work_bytes(uint64_t rows, uint64_t cols);

/* Host-only check of a descriptor (magic, version, CRC, offsets, table).
 * Returns LBF_OK or LBF_E_DESC.  Needs no GPU. */
int lbf_desc_check(const lbf_desc* desc);

/*
 * lbf_encode — code a BF16 tensor into a blob (two phases).
 * The coding step of "Lossless LLM Weight Compression vs 8-bit GGUF", section
 * "What did the GLM-5.2 experiment actually prove?": a histogram of the
 * exponent field picks the symbols that get short fixed-width codes (here
 * the 15 most frequent exponents, 4 bits each); every other exponent is sent
 * verbatim through the escape stream, while sign and mantissa stay raw.
 *   d_w        device, bf16 bit patterns [rows, cols], row-major, 16-byte aligned
 *   d_work     device workspace of at least lbf_encode_work_bytes(rows, cols)
 *              bytes, 256-byte aligned; its contents on entry do not matter
 *   desc       host; phase 1 writes it, phase 2 reads it
 * Phase 1 (d_blob == NULL): exponent histogram on the GPU, then the code table,
 *   escape count and plane offsets on the host; fills *desc.  This call waits
 *   for the stream (the only synchronising call in the library).
 * Phase 2 (d_blob != NULL): writes the whole blob (header included) on `s`;
 *   desc must be the unchanged phase-1 result for the same d_w.  d_blob must
 *   be 256-byte aligned and blob_cap >= desc->blob_bytes (else
 *   LBF_E_CAPACITY).  Phase 2 never writes outside [d_blob, d_blob +
 *   desc->blob_bytes): if d_w changed between the phases (more or fewer
 *   escapes than desc->n_esc), the escape bytes past desc->n_esc are dropped
 *   and the blob is not a valid coding — its index disagrees with the header,
 *   which lbf_verify reports (LBF_VERIFY_INDEX).
 * Shapes: any rows, cols with rows * cols < 2^32 (LBF_E_SHAPE otherwise).
 */
int lbf_encode(const void* d_w, uint64_t rows, uint64_t cols, void* d_work, uint64_t work_bytes,
               void* d_blob, uint64_t blob_cap, lbf_desc* desc, hipStream_t s);

/*
 * lbf_encode_noalloc — lbf_encode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same two phases, arguments and results as
 * lbf_encode, but the workspace is the library's own device array of
 * LBF_NOALLOC_SCRATCH_BYTES, one per GPU, kept until the process ends.
 * The call allocates nothing.
 *  - tensors whose lbf_encode_work_bytes(rows, cols) exceeds
 *    LBF_NOALLOC_SCRATCH_BYTES (more than 261,888 tiles, about 268 million
 *    weights) are refused with LBF_E_CAPACITY before anything runs;
 *  - every call on one GPU shares that GPU's array, and each call clears
 *    what it needs cleared (the histogram) itself: calls that overlap on one
 *    GPU (other streams or threads, or a phase 1 enqueued before another
 *    call's phase 2 has run) race and may write a wrong blob.  Serialize
 *    them, or use lbf_encode with a workspace per caller.
 */
#define LBF_NOALLOC_SCRATCH_BYTES (1u << 20)
int lbf_encode_noalloc(const void* d_w, uint64_t rows, uint64_t cols, void* d_blob, uint64_t blob_cap,
                       lbf_desc* desc, hipStream_t s);

/*
 * lbf_decode — rebuild the exact BF16 tensor from a blob.
 * Lossless means the decoded bits equal the source bits, and that is what
 * this call delivers ("Lossless LLM Weight Compression vs 8-bit GGUF",
 * section "What does 'lossless' mean for LLM weights?"): per weight, the
 * exponent is lut[code] or, for code 15, the tile's next escape byte, and
 * sign and mantissa come back from the raw byte.
 *   desc       host copy of the blob's header (checked with lbf_desc_check)
 *   d_blob     device, 256-byte aligned, desc->blob_bytes long
 *   d_w_out    device, bf16 [rows, cols], 16-byte aligned; fully overwritten
 * Bit-exact: NaN payloads, signed zeros, infinities and denormals survive.
 */
int lbf_decode(const lbf_desc* desc, const void* d_blob, void* d_w_out, hipStream_t s);

/*
 * lbf_gemv — y[g][b, r] = sum_k W_g[r, k] * x[g][b, k] for each group g, with
 * each W_g decoded in registers only, products accumulated in fp32.
 * (Fused decode and multiply: same page, section "What does 'lossless' mean
 * for LLM weights?".)
 *   descs      host array [n_groups] of descriptors, one per weight tensor
 *   d_blobs    host array [n_groups] of device blob pointers (256-B aligned)
 *   d_x        host array [n_groups] of device pointers to bf16 x_g
 *              [batch, cols_g], row-major, 16-byte aligned
 *   batch      1..8
 *   d_y        host array [n_groups] of device pointers to y_g [batch, rows_g]
 *              (row-major, the F.linear output layout), 4-byte aligned,
 *              element type y_dtype (LBF_F32, or LBF_BF16 rounded to nearest
 *              even from the fp32 sum); fully overwritten
 * Requires cols_g % 1024 == 0 (LBF_E_SHAPE otherwise).  n_groups >= 1; calls
 * with more than LBF_MAX_GROUPS groups are issued as several launches.
 * Every group runs in the same launch when n_groups <= LBF_MAX_GROUPS.
 * A launch passes each kernel 40 bytes per group (blob, x and y pointers and
 * the checked rows, tiles and escape count); every workgroup takes the code
 * table from the blob's own header copy, so the device header must equal
 * descs[g] (as lbf_encode writes it; lbf_verify checks it).  A device header
 * that differs can give wrong outputs but no access outside the buffers.
 * A batch-8 call whose escapes are at most 1 % of its weights runs on the
 * MFMA kernel of lbf_gemm (faster there); its fp32 sums then add in that
 * kernel's fixed order, a different one from the other batches'.
 */
int lbf_gemv(const lbf_desc* descs, const void* const* d_blobs, int n_groups, const void* const* d_x,
             int batch, void* const* d_y, int y_dtype, hipStream_t s);

/*
 * lbf_gemv_swiglu — the gated MLP product of a decoder layer in one launch:
 *   h[b, r] = silu(g[b, r]) * u[b, r],  g = W_gate x,  u = W_up x,
 * sums in fp32 as lbf_gemv, silu(z) = z / (1 + e^-z) in fp32.  One wave
 * decodes gate row r and then up row r, so g and u never leave registers and
 * the two products and the activation cost one launch and one write of h.
 * Decoding pays only where it hides under weight traffic and serving is bound
 * by weight bandwidth ("Verlustfreie LLM-Gewichtskompression vs. 8-bit GGUF",
 * opening section: a Split12 serving test ran slower than BF16; "Lossless
 * LLM Weight Compression vs 8-bit GGUF", section "Lossless compression or Q8
 * GGUF: which should you deploy?"), so the layer's small epilogues are fused.
 *   gate_desc, d_gate_blob, up_desc, d_up_blob   the two tensors: same
 *              [rows, cols] (LBF_E_SHAPE otherwise), blobs 256-byte aligned
 *   d_x        device bf16 [batch, cols], 16-byte aligned; batch 1..8
 *   d_h        device [batch, rows], 4-byte aligned, element type h_dtype
 *              (LBF_F32, or LBF_BF16 rounded to nearest even); overwritten
 * Requires cols % 1024 == 0 (LBF_E_SHAPE) and batch * cols * 2 <= 131072 (x is
 * staged once in LDS; LBF_E_UNSUPPORTED otherwise).
 */
int lbf_gemv_swiglu(const lbf_desc* gate_desc, const void* d_gate_blob, const lbf_desc* up_desc,
                    const void* d_up_blob, const void* d_x, int batch, void* d_h, int h_dtype, hipStream_t s);

/*
 * lbf_gemm — the same product for batch >= 9, on bf16 MFMA (matrix cores)
 * with fp32 accumulation; the decoded weights go straight into the MFMA
 * operand registers and are never written to memory.  (Same page, section
 * "How does this compare with prior lossless systems?": a fused
 * decompression-GEMM.)  Arguments and layouts as lbf_gemv; batch 9..256
 * (LBF_E_INVAL otherwise).  Requires cols_g % 1024 == 0 (LBF_E_SHAPE) and
 * cols_g <= 16777216 (LBF_E_UNSUPPORTED).  Batches above 64 run as several
 * launches of up to 64 columns, each reading the coded weights once.
 */
int lbf_gemm(const lbf_desc* descs, const void* const* d_blobs, int n_groups, const void* const* d_x,
             int batch, void* const* d_y, int y_dtype, hipStream_t s);

/* Checks of lbf_verify; its result is the OR of the failed ones (0: all pass). */
enum {
  LBF_VERIFY_HEADER = 1,  /* device bytes [0,96) differ from *desc, or [96,256) are not zero */
  LBF_VERIFY_INDEX = 2,   /* idx[0] != 0, idx decreases, or idx[n_tiles] != n_esc */
  LBF_VERIFY_COUNT = 4,   /* a tile holds a number of code-15 nibbles other than idx[t+1] - idx[t] */
  LBF_VERIFY_CODE = 8,    /* a real weight holds an unused code (n_codes .. 14) */
  LBF_VERIFY_ESCAPE = 16, /* an escape byte is one of the coded exponents */
  LBF_VERIFY_PADDING = 32 /* a byte the format pads with zero is not zero */
};

/*
 * lbf_verify — structural check of a device blob against the host descriptor
 * the caller trusts, on the GPU, without decoding.  Corrupt weights must be
 * detected and refused (same page, sections "Is the GLM-5.2 result
 * production-ready?" and "Questions to ask a vendor or research team").
 *   desc      host descriptor (checked with lbf_desc_check: LBF_E_DESC)
 *   d_blob    device, 256-byte aligned, desc->blob_bytes long
 *   d_flags   device uint32, 4-byte aligned: overwritten with the OR of the
 *             failed LBF_VERIFY_* checks once the stream reaches it
 * Not covered: the sign and mantissa bits of real weights and escaped
 * exponents changed into other uncoded ones carry no redundancy; compare
 * lbf_crc32 of the blob with a stored hash to cover every byte.
 */
int lbf_verify(const lbf_desc* desc, const void* d_blob, uint32_t* d_flags, hipStream_t s);

/*
 * lbf_crc32 — CRC-32 of n bytes of device memory (IEEE 802.3 polynomial,
 * reflected, initial value and final xor 0xFFFFFFFF: zlib's crc32), on the
 * GPU.  Lets a stored hash of a blob be checked where the blob lives.
 *   d_data    device, 16-byte aligned (any n, including 0)
 *   d_crc     device uint32, 4-byte aligned: overwritten with the CRC once the
 *             stream reaches it
 */
int lbf_crc32(const void* d_data, uint64_t n, uint32_t* d_crc, hipStream_t s);

/*
 * ---- K15H: the entropy-coded variant ----------------------------------------
 * The English page's larger K15 reduction belongs to an entropy-coded form of
 * the byte split ("Lossless LLM Weight Compression vs 8-bit GGUF", opening
 * section), and DFloat11 entropy-codes the exponent while sign and mantissa
 * stay raw ("你的 bf16 模型,有 5 個 bit 是廢的", section 二).  K15H keeps format
 * v1's symbols (the 4-bit code of every weight: 0..14 for the table's
 * exponents, 15 for an escape) and codes them with a Huffman code:
 *  - code lengths from Huffman's procedure over the codes' counts among the
 *    n real weights, run with two queues (used symbols sorted by count, then
 *    symbol; merged nodes in creation order; a leaf wins a tie); a lone used
 *    symbol gets length 1; no length exceeds 15;
 *  - canonical code values (RFC 1951, section 3.2.2), written most
 *    significant bit first into a bit stream whose bit k is bit k % 32 of
 *    32-bit word k / 32;
 *  - each 1024-weight tile is a stream of whole words (its codes in element
 *    order, unused bits zero); woff[t] is tile t's first word.
 * Blob layout (every plane at a multiple of 256; blob_bytes too):
 *   [0, 256)   header: the 128-byte lbf_hdesc, then zeros
 *   off_raw    raw plane, exactly format v1's (n_tiles * 1024 bytes)
 *   off_bits   code stream, stream_words 32-bit words
 *   off_woff   uint32 woff[n_tiles + 1] (woff[n_tiles] = stream_words)
 *   off_idx    uint32 idx[n_tiles + 1], format v1's escape index
 *   off_esc    escape stream, format v1's
 */
#define LBF_HMAGIC 0x4846424Cu /* "LBFH" little-endian */
#define LBF_HVERSION 1
#define LBF_HMAX_TILE_WORDS 480 /* 1024 codes of at most 15 bits */

/* Host copy of a K15H blob's header; byte-for-byte its first 128 bytes. */
typedef struct lbf_hdesc {
  uint32_t magic;      /* LBF_HMAGIC */
  uint16_t version;    /* LBF_HVERSION */
  uint16_t tile_log2;  /* LBF_TILE_LOG2 */
  uint64_t rows, cols, n_esc;
  uint64_t off_raw, off_bits, off_woff, off_idx, off_esc, blob_bytes;
  uint64_t stream_words;
  uint8_t lut[16];     /* as lbf_desc */
  uint8_t n_codes;     /* as lbf_desc */
  uint8_t max_len;     /* largest len[] */
  uint8_t reserved[2]; /* zero */
  uint8_t len[16];     /* Huffman code length of code c (0: c never occurs) */
  uint32_t desc_crc;   /* CRC-32 (IEEE) of the 124 bytes before this field */
} lbf_hdesc;

/* Host-only check of a K15H descriptor: magic, version, CRC, layout, table,
 * and code lengths (a complete prefix code when two or more codes are used).
 * Returns LBF_OK or LBF_E_DESC (LBF_E_INVAL for NULL). */
int lbf_hdesc_check(const lbf_hdesc* hdesc);

/* Bytes of device workspace lbf_hencode needs for the tensor of `desc`
 * (0 if desc fails lbf_desc_check). */
uint64_t lbf_hencode_work_bytes(const lbf_desc* desc);

/*
 * lbf_hencode — re-code a format-v1 blob as a K15H blob (two phases, as
 * lbf_encode).  The source must be a valid v1 blob (lbf_verify passes): its
 * codes are read, not checked.
 *   desc, d_blob  the v1 blob (256-byte aligned) and its descriptor
 *   d_work        device workspace, 256-byte aligned, at least
 *                 lbf_hencode_work_bytes(desc) bytes; contents on entry
 *                 do not matter
 *   hdesc         host; phase 1 writes it, phase 2 reads it
 * Phase 1 (d_hblob == NULL): counts the codes and sizes every tile's stream
 *   on the GPU, builds the code on the host, fills *hdesc.  Waits for the
 *   stream.
 * Phase 2 (d_hblob != NULL): writes the whole K15H blob on `s`; hdesc must be
 *   the unchanged phase-1 result for the same v1 blob; d_hblob 256-byte
 *   aligned, hblob_cap >= hdesc->blob_bytes (else LBF_E_CAPACITY).
 */
int lbf_hencode(const lbf_desc* desc, const void* d_blob, void* d_work, uint64_t work_bytes, void* d_hblob,
                uint64_t hblob_cap, lbf_hdesc* hdesc, hipStream_t s);

/*
 * lbf_hdecode — rebuild the exact BF16 tensor from a K15H blob.
 *   hdesc      host copy of the blob's header (checked with lbf_hdesc_check)
 *   d_hblob    device, 256-byte aligned, hdesc->blob_bytes long
 *   d_w_out    device, bf16 [rows, cols], 16-byte aligned; fully overwritten
 * Bit-exact as lbf_decode.  A corrupt stream or index decodes to wrong
 * values but never reads or writes outside the blob and the output.
 */
int lbf_hdecode(const lbf_hdesc* hdesc, const void* d_hblob, void* d_w_out, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* LBF_H */
