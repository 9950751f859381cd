/*
 * splitzip_oracle.c -- plain, slow, scalar CPU oracle of the SplitZip exponent
 * codec (stream format "SZ1").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls it, and the two share no code, headers or tables.
 *
 * Every element is handled one at a time, in the order the method states the
 * steps.  Codebook membership is a linear search over the 16 entries (the
 * definition), not a lookup table.
 *
 * Sources: the pages on "SplitZip: Ultra Fast Lossless KV Compression for
 * Disaggregated LLM Serving" (arXiv 2605.01708v2), cited as
 *   [TS] the Spanish technical summary (gist.science), "section / bullet";
 *   [EX] the English explainer (gist.science), numbered section;
 *   [AB] the authors' abstract (fugumt.com listing).
 *
 * What the pages fix:
 *   - BF16 = 1 sign, 8 exponent, 7 mantissa bits; the exponent is split from
 *     the sign and mantissa  ([EX] "1. The 'Note' Structure";
 *     [TS] Metodologia / Informacion Clave).
 *   - An offline-calibrated top-16 exponent codebook maps frequent exponents
 *     to fixed 4-bit codes, two codes per byte
 *     ([TS] Metodologia / Codificacion de Longitud Fija; [AB]).
 *   - Exponents outside the codebook become escapes: a 16-bit element
 *     position plus the 8-bit raw exponent, in a sparse stream
 *     ([TS] Metodologia / Flujo de Escape; [EX] "3. The SplitZip Strategy").
 *   - Sign and mantissa are kept losslessly as a raw 8-bit stream
 *     ([TS] Metodologia / Preservacion de Signo/Mantisa).
 *   - Decode maps the 4-bit codes through a lookup table, rebuilds the values
 *     densely, then overwrites the escaped exponents with their raw values
 *     ([TS] Estrategia de Decodificacion / Paralelismo, Correccion).
 *   - The same scheme applies to FP8 E5M2 (5-bit exponent)
 *     ([TS] Contribuciones Clave 4; [AB]).
 *
 * What the pages leave open, and the reading taken here (each one is listed
 * in the design notes):
 *   R1 sign|mantissa byte: sign in bit 7, mantissa in bits 6..0.
 *   R2 nibble order: the even element goes to the low nibble.
 *   R3 code k is the k-th most frequent exponent; equal counts go to the
 *      lower exponent; exponents never seen fill the remaining slots in
 *      ascending order.
 *   R4 an escaped element's nibble is 0.
 *   R5 escape position is relative to its 65536-element chunk (16 bits).
 *   R6 escapes are stored in element order, as 3-byte records
 *      [pos lo, pos hi, value].
 *   R7 E5M2 sign|mantissa is 3 bits (sign<<2 | mantissa), packed 8 elements
 *      per 3 little-endian bytes, element j of a group at bits 3j..3j+2.
 *   R8 stream header, per-chunk escape offsets, 256-byte section alignment,
 *      zero padding: see the layout below.
 *
 * Stream layout (little-endian; A(x) = x rounded up to a multiple of 256;
 * C = ceil(n / 65536); K codebooks; E escapes):
 *   0   u32 magic 0x00315A53 ("SZ1\0")   4  u16 version = 1
 *   6   u8  dtype (1 BF16, 2 E5M2)        7  u8  log2 chunk = 16
 *   8   u64 n        16 u64 E        24 u64 total bytes S
 *   32  u32 C        36 u32 K        40 u64 segment elements (n if K == 1)
 *   48  16 bytes zero
 *   64          K x 16 bytes codebooks (entry k = exponent of code k)
 *   64 + 16K    (C + 1) x u64 exclusive escape offsets per chunk
 *   N0 = A(64 + 16K + 8(C + 1))   nibbles, ceil(n/2) bytes
 *   N1 = N0 + A(ceil(n/2))         sign|mantissa: n bytes (BF16) or
 *                                  3 ceil(n/8) bytes (E5M2)
 *   P  = N1 + A(sm bytes)          E escape records of 3 bytes
 *   S  = P + 3E
 *   Every byte between sections is zero.  Chunk c uses codebook 0 when K == 1,
 *   else codebook floor(65536 c / segment).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

#define SZO_OK 0
#define SZO_E_INVALID (-1)
#define SZO_E_CAPACITY (-2)
#define SZO_E_CODEBOOK (-3)
#define SZO_E_CORRUPT (-4)

#define SZO_BF16 1
#define SZO_E5M2 2

#define SZO_CHUNK 65536ull
#define SZO_MAX_K 65535u
#define SZO_MAX_N (1ull << 40)

static uint64_t align256(uint64_t x) { return (x + 255ull) / 256ull * 256ull; }
static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

static int dtype_ok(int dtype) { return dtype == SZO_BF16 || dtype == SZO_E5M2; }

/* Number of exponent values the dtype has: 8 bits for BF16, 5 for E5M2. */
static unsigned exponent_values(int dtype) { return dtype == SZO_BF16 ? 256u : 32u; }

/* Field split of one element ([EX] "1. The 'Note' Structure"; [TS] Informacion
 * Clave).  BF16: bit 15 sign, bits 14..7 exponent, bits 6..0 mantissa.
 * E5M2: bit 7 sign, bits 6..2 exponent, bits 1..0 mantissa. */
static unsigned get_exponent(int dtype, const void *data, uint64_t i) {
  if (dtype == SZO_BF16) {
    uint16_t x = ((const uint16_t *)data)[i];
    return (x >> 7) & 0xFFu;
  } else {
    uint8_t b = ((const uint8_t *)data)[i];
    return (b >> 2) & 0x1Fu;
  }
}

/* Sign|mantissa of one element: BF16 -> 8 bits (sign at bit 7, R1);
 * E5M2 -> 3 bits (sign at bit 2, R7). */
static unsigned get_signmant(int dtype, const void *data, uint64_t i) {
  if (dtype == SZO_BF16) {
    uint16_t x = ((const uint16_t *)data)[i];
    unsigned sign = (x >> 15) & 1u;
    unsigned mant = x & 0x7Fu;
    return (sign << 7) | mant;
  } else {
    uint8_t b = ((const uint8_t *)data)[i];
    unsigned sign = (b >> 7) & 1u;
    unsigned mant = b & 0x3u;
    return (sign << 2) | mant;
  }
}

/* Inverse of the split: put sign, exponent and mantissa back together. */
static void put_element(int dtype, void *data, uint64_t i, unsigned exponent, unsigned signmant) {
  if (dtype == SZO_BF16) {
    unsigned sign = (signmant >> 7) & 1u;
    unsigned mant = signmant & 0x7Fu;
    ((uint16_t *)data)[i] = (uint16_t)((sign << 15) | ((exponent & 0xFFu) << 7) | mant);
  } else {
    unsigned sign = (signmant >> 2) & 1u;
    unsigned mant = signmant & 0x3u;
    ((uint8_t *)data)[i] = (uint8_t)((sign << 7) | ((exponent & 0x1Fu) << 2) | mant);
  }
}

static void put_u16(uint8_t *p, uint64_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint64_t v) { for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int k = 0; k < 8; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static uint64_t get_u16(const uint8_t *p) { return (uint64_t)p[0] | ((uint64_t)p[1] << 8); }
static uint64_t get_u32(const uint8_t *p) {
  uint64_t v = 0;
  for (int k = 3; k >= 0; --k) v = (v << 8) | p[k];
  return v;
}
static uint64_t get_u64(const uint8_t *p) {
  uint64_t v = 0;
  for (int k = 7; k >= 0; --k) v = (v << 8) | p[k];
  return v;
}

/* Bytes of the sign|mantissa section before padding (R7 for E5M2). */
static uint64_t signmant_bytes(int dtype, uint64_t n) {
  return dtype == SZO_BF16 ? n : 3ull * ceil_div(n, 8);
}

typedef struct {
  uint64_t C, N0, N1, P;
} szo_layout;

static szo_layout layout_of(int dtype, uint64_t n, uint64_t K) {
  szo_layout L;
  L.C = ceil_div(n, SZO_CHUNK);
  L.N0 = align256(64 + 16 * K + 8 * (L.C + 1));
  L.N1 = L.N0 + align256(ceil_div(n, 2));
  L.P = L.N1 + align256(signmant_bytes(dtype, n));
  return L;
}

/* Size of a stream with E escapes: the closed form
 * S = A(64 + 16K + 8(C+1)) + A(ceil(n/2)) + A(sm bytes) + 3E. */
uint64_t szo_stream_size(int dtype, uint64_t n, uint32_t K, uint64_t E) {
  if (!dtype_ok(dtype)) return 0;
  szo_layout L = layout_of(dtype, n, K);
  return L.P + 3ull * E;
}

/* Section offsets of a stream: out[0] = C, out[1] = offset table, out[2] =
 * nibbles N0, out[3] = sign|mantissa N1, out[4] = escape records P. */
int szo_sections(int dtype, uint64_t n, uint32_t K, uint64_t out[5]) {
  if (!dtype_ok(dtype) || out == NULL) return SZO_E_INVALID;
  szo_layout L = layout_of(dtype, n, K);
  out[0] = L.C;
  out[1] = 64 + 16ull * K;
  out[2] = L.N0;
  out[3] = L.N1;
  out[4] = L.P;
  return SZO_OK;
}

/* Worst case (every element escapes). */
uint64_t szo_max_size(int dtype, uint64_t n, uint32_t K) { return szo_stream_size(dtype, n, K, n); }

/* ---- Calibration ([TS] Codificacion de Longitud Fija, Optimizacion; [TS]
 * Resultados / Calibracion; [AB]): histogram of exponents over the samples,
 * then the 16 most frequent values, equal counts to the lower exponent (R3). */
int szo_calibrate(int dtype, const void *samples, uint64_t n, uint8_t codebook_out[16]) {
  if (!dtype_ok(dtype) || codebook_out == NULL || (samples == NULL && n > 0)) return SZO_E_INVALID;
  unsigned V = exponent_values(dtype);
  uint64_t hist[256];
  for (unsigned v = 0; v < 256; ++v) hist[v] = 0;
  for (uint64_t i = 0; i < n; ++i) hist[get_exponent(dtype, samples, i)] += 1;
  /* Selection by repeated maximum: pick the value with the largest count not
   * yet chosen; on equal counts the lower value wins because the scan is
   * ascending and only a strictly larger count replaces the candidate. */
  int chosen[256];
  for (unsigned v = 0; v < 256; ++v) chosen[v] = 0;
  for (unsigned k = 0; k < 16; ++k) {
    int best = -1;
    for (unsigned v = 0; v < V; ++v) {
      if (chosen[v]) continue;
      if (best < 0 || hist[v] > hist[best]) best = (int)v;
    }
    chosen[best] = 1;
    codebook_out[k] = (uint8_t)best;
  }
  return SZO_OK;
}

/* A codebook is usable when its 16 entries are distinct exponent values. */
static int codebook_valid(int dtype, const uint8_t *cb) {
  unsigned V = exponent_values(dtype);
  for (int a = 0; a < 16; ++a) {
    if (cb[a] >= V) return 0;
    for (int b = 0; b < a; ++b)
      if (cb[a] == cb[b]) return 0;
  }
  return 1;
}

/* Which codebook chunk c uses. */
static uint64_t chunk_codebook(uint64_t c, uint64_t K, uint64_t seg) {
  if (K == 1) return 0;
  return (c * SZO_CHUNK) / seg;
}

/* Code of exponent e in a codebook, or -1 if e is not one of its entries. */
static int code_of(const uint8_t *cb, unsigned e) {
  for (int k = 0; k < 16; ++k)
    if (cb[k] == e) return k;
  return -1;
}

static int compress_args_ok(int dtype, const void *in, uint64_t n, const uint8_t *cbs, uint32_t K, uint64_t seg) {
  if (!dtype_ok(dtype)) return SZO_E_INVALID;
  if (in == NULL && n > 0) return SZO_E_INVALID;
  if (n > SZO_MAX_N) return SZO_E_INVALID;
  if (cbs == NULL || K == 0 || K > SZO_MAX_K) return SZO_E_INVALID;
  if (K > 1) {
    if (seg == 0 || seg % SZO_CHUNK != 0) return SZO_E_INVALID;
    if (seg < ceil_div(n, K)) return SZO_E_INVALID; /* K * seg must cover n */
  }
  for (uint32_t k = 0; k < K; ++k)
    if (!codebook_valid(dtype, cbs + 16ull * k)) return SZO_E_CODEBOOK;
  return SZO_OK;
}

/* ---- Encode ([TS] Estrategia de Codificacion; [EX] "3. The SplitZip
 * Strategy"; [AB]).  Chunk by chunk, element by element: split, look the
 * exponent up in the chunk's codebook, write its 4-bit code (or 0 and an
 * escape record), write the sign|mantissa bits. */
int szo_compress(int dtype, const void *in, uint64_t n, const uint8_t *cbs, uint32_t K, uint64_t seg,
                 uint8_t *out, uint64_t capacity, uint64_t *out_bytes) {
  int rc = compress_args_ok(dtype, in, n, cbs, K, seg);
  if (rc != SZO_OK) return rc;
  if (out == NULL) return SZO_E_INVALID;
  if (capacity < szo_max_size(dtype, n, K)) return SZO_E_CAPACITY;
  szo_layout L = layout_of(dtype, n, K);
  uint64_t seg_stored = (K == 1) ? n : seg;

  /* Everything not written below is zero padding. */
  memset(out, 0, L.P);

  uint8_t *nib = out + L.N0;
  uint8_t *sm = out + L.N1;
  uint8_t *esc = out + L.P;
  uint8_t *off = out + 64 + 16ull * K;
  uint64_t E = 0;

  for (uint64_t c = 0; c < L.C; ++c) {
    const uint8_t *cb = cbs + 16ull * chunk_codebook(c, K, seg);
    uint64_t first = c * SZO_CHUNK;
    uint64_t last = first + SZO_CHUNK < n ? first + SZO_CHUNK : n;
    put_u64(off + 8 * c, E);
    for (uint64_t i = first; i < last; ++i) {
      unsigned e = get_exponent(dtype, in, i);
      int code = code_of(cb, e);
      unsigned nibble;
      if (code >= 0) {
        nibble = (unsigned)code;
      } else {
        nibble = 0; /* R4 */
        uint64_t pos = i - first;  /* R5 */
        put_u16(esc + 3 * E, pos); /* R6 */
        esc[3 * E + 2] = (uint8_t)e;
        E += 1;
      }
      /* R2: even element in the low nibble. */
      if (i % 2 == 0)
        nib[i / 2] = (uint8_t)(nib[i / 2] | nibble);
      else
        nib[i / 2] = (uint8_t)(nib[i / 2] | (nibble << 4));

      unsigned s = get_signmant(dtype, in, i);
      if (dtype == SZO_BF16) {
        sm[i] = (uint8_t)s;
      } else {
        /* R7: group q = i / 8 occupies bytes 3q..3q+2 as one 24-bit
         * little-endian value; element j of the group sits at bits 3j. */
        uint64_t q = i / 8, j = i % 8;
        uint64_t g = sm[3 * q] | ((uint64_t)sm[3 * q + 1] << 8) | ((uint64_t)sm[3 * q + 2] << 16);
        g |= (uint64_t)s << (3 * j);
        sm[3 * q] = (uint8_t)g;
        sm[3 * q + 1] = (uint8_t)(g >> 8);
        sm[3 * q + 2] = (uint8_t)(g >> 16);
      }
    }
  }
  put_u64(off + 8 * L.C, E);

  put_u32(out + 0, 0x00315A53u);
  put_u16(out + 4, 1);
  out[6] = (uint8_t)dtype;
  out[7] = 16;
  put_u64(out + 8, n);
  put_u64(out + 16, E);
  put_u64(out + 24, L.P + 3 * E);
  put_u32(out + 32, L.C);
  put_u32(out + 36, K);
  put_u64(out + 40, seg_stored);
  memcpy(out + 64, cbs, 16ull * K);
  if (out_bytes) *out_bytes = L.P + 3 * E;
  return SZO_OK;
}

/* ---- Stream validation: every field and every escape record is checked
 * before any element is written, so a corrupt stream is reported, never
 * half-decoded. */
static int parse_header(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n, uint64_t *K_out,
                        uint64_t *seg_out, uint64_t *E_out, szo_layout *L_out) {
  if (in_bytes < 64) return SZO_E_CORRUPT;
  if (get_u32(in) != 0x00315A53u) return SZO_E_CORRUPT;
  if (get_u16(in + 4) != 1) return SZO_E_CORRUPT;
  if (in[6] != dtype) return SZO_E_CORRUPT;
  if (in[7] != 16) return SZO_E_CORRUPT;
  if (get_u64(in + 8) != n) return SZO_E_CORRUPT;
  for (int k = 48; k < 64; ++k)
    if (in[k] != 0) return SZO_E_CORRUPT;
  uint64_t E = get_u64(in + 16);
  uint64_t S = get_u64(in + 24);
  uint64_t C = get_u32(in + 32);
  uint64_t K = get_u32(in + 36);
  uint64_t seg = get_u64(in + 40);
  if (C != ceil_div(n, SZO_CHUNK)) return SZO_E_CORRUPT;
  if (K == 0 || K > SZO_MAX_K) return SZO_E_CORRUPT;
  if (K == 1) {
    if (seg != n) return SZO_E_CORRUPT;
  } else {
    if (seg == 0 || seg % SZO_CHUNK != 0 || seg < ceil_div(n, K)) return SZO_E_CORRUPT;
  }
  if (E > n) return SZO_E_CORRUPT;
  szo_layout L = layout_of(dtype, n, K);
  if (S != L.P + 3 * E) return SZO_E_CORRUPT;
  if (S > in_bytes) return SZO_E_CORRUPT;
  *K_out = K;
  *seg_out = seg;
  *E_out = E;
  *L_out = L;
  return SZO_OK;
}

/* Full check of a stream: header, codebooks, offsets, escape positions. */
int szo_validate(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n) {
  if (!dtype_ok(dtype) || in == NULL) return SZO_E_INVALID;
  uint64_t K, seg, E;
  szo_layout L;
  int rc = parse_header(in, in_bytes, dtype, n, &K, &seg, &E, &L);
  if (rc != SZO_OK) return rc;
  for (uint64_t k = 0; k < K; ++k)
    if (!codebook_valid(dtype, in + 64 + 16 * k)) return SZO_E_CORRUPT;
  const uint8_t *off = in + 64 + 16 * K;
  const uint8_t *esc = in + L.P;
  if (get_u64(off) != 0 || get_u64(off + 8 * L.C) != E) return SZO_E_CORRUPT;
  for (uint64_t c = 0; c < L.C; ++c) {
    uint64_t lo = get_u64(off + 8 * c), hi = get_u64(off + 8 * (c + 1));
    if (lo > hi || hi > E) return SZO_E_CORRUPT;
    uint64_t len = (c + 1) * SZO_CHUNK <= n ? SZO_CHUNK : n - c * SZO_CHUNK;
    for (uint64_t r = lo; r < hi; ++r) {
      uint64_t pos = get_u16(esc + 3 * r);
      if (pos >= len) return SZO_E_CORRUPT;
      if (r > lo && pos <= get_u16(esc + 3 * (r - 1))) return SZO_E_CORRUPT;
      if (esc[3 * r + 2] >= exponent_values(dtype)) return SZO_E_CORRUPT;
    }
  }
  return SZO_OK;
}

/* ---- Decode ([TS] Estrategia de Decodificacion / Paralelismo, Correccion;
 * [EX] "4. Why It's Fast").  Dense pass: code -> exponent through the
 * chunk's codebook, recombined with sign|mantissa.  Then the escape pass
 * overwrites the exponent of every escaped element. */
int szo_decompress(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n, void *out) {
  if (!dtype_ok(dtype) || in == NULL || (out == NULL && n > 0)) return SZO_E_INVALID;
  int rc = szo_validate(in, in_bytes, dtype, n);
  if (rc != SZO_OK) return rc;
  uint64_t K = get_u32(in + 36);
  uint64_t seg = get_u64(in + 40);
  szo_layout L = layout_of(dtype, n, K);
  const uint8_t *nib = in + L.N0;
  const uint8_t *sm = in + L.N1;
  const uint8_t *esc = in + L.P;
  const uint8_t *off = in + 64 + 16 * K;

  for (uint64_t c = 0; c < L.C; ++c) {
    const uint8_t *cb = in + 64 + 16 * chunk_codebook(c, K, seg);
    uint64_t first = c * SZO_CHUNK;
    uint64_t last = first + SZO_CHUNK < n ? first + SZO_CHUNK : n;
    for (uint64_t i = first; i < last; ++i) {
      unsigned nibble = (i % 2 == 0) ? (nib[i / 2] & 0xFu) : (nib[i / 2] >> 4);
      unsigned s;
      if (dtype == SZO_BF16) {
        s = sm[i];
      } else {
        uint64_t q = i / 8, j = i % 8;
        uint64_t g = sm[3 * q] | ((uint64_t)sm[3 * q + 1] << 8) | ((uint64_t)sm[3 * q + 2] << 16);
        s = (unsigned)((g >> (3 * j)) & 0x7u);
      }
      put_element(dtype, out, i, cb[nibble], s);
    }
  }
  for (uint64_t c = 0; c < L.C; ++c) {
    uint64_t lo = get_u64(off + 8 * c), hi = get_u64(off + 8 * (c + 1));
    for (uint64_t r = lo; r < hi; ++r) {
      uint64_t i = c * SZO_CHUNK + get_u16(esc + 3 * r);
      unsigned v = esc[3 * r + 2];
      unsigned s = get_signmant(dtype, out, i); /* sign|mantissa already in place */
      put_element(dtype, out, i, v, s);
    }
  }
  return SZO_OK;
}

/* Escape count a stream would have, without building it. */
uint64_t szo_count_escapes(int dtype, const void *in, uint64_t n, const uint8_t *cbs, uint32_t K, uint64_t seg) {
  if (compress_args_ok(dtype, in, n, cbs, K, seg) != SZO_OK) return UINT64_MAX;
  uint64_t E = 0;
  for (uint64_t i = 0; i < n; ++i) {
    const uint8_t *cb = cbs + 16ull * chunk_codebook(i / SZO_CHUNK, K, seg);
    if (code_of(cb, get_exponent(dtype, in, i)) < 0) E += 1;
  }
  return E;
}

/* ---- Ablation variants (BF16), the two designs the pages compare against
 * the top-16 codec ([TS] Metodologia / Decision de Diseno and Resultados):
 *
 *   variant 1, top-15 + sentinel: codes 0..14 are the 15 most frequent
 *     exponents (codebook entries 0..14) and code 15 marks an escape.  The
 *     escape stream holds only the raw exponents, in element order; an
 *     escape's position is where its sentinel sits.  The pages say this
 *     saves metadata but makes decoding irregular (3.5x slower).
 *   variant 2, top-8: 3-bit codes for the 8 most frequent exponents
 *     (entries 0..7); the pages report 92% coverage instead of 99.8% and a
 *     3x slower decode.
 *
 * What the pages leave open, and the reading taken here:
 *   V1 layout: the main layout with the variant id in header byte 48; the
 *      per-chunk escape offsets are kept in both (a chunk-parallel decoder
 *      needs them; 8 bytes per 65536 elements).
 *   V2 top-15: an escaped element's nibble is 15; the escape section is E
 *      bytes of raw exponents (no positions).
 *   V3 top-8: codes are packed 8 per 3 little-endian bytes, element j of a
 *      group at bits 3j (as the E5M2 triples, R7); an escaped element's code
 *      is 0 and its escape is a 3-byte record as in R6.
 *   V4 codebooks: 16 distinct entries are stored per segment as in the main
 *      format; the variant uses the first 15 or 8.
 *   Sections (A = round up to 256): N0 = A(64 + 16K + 8(C+1)); codes;
 *   N1 = N0 + A(code bytes); sign|mantissa n bytes; P = N1 + A(n);
 *   S = P + E (top-15) or P + 3E (top-8). */
#define SZO_V_SENTINEL 1
#define SZO_V_TOP8 2

static int variant_ok(int v) { return v == SZO_V_SENTINEL || v == SZO_V_TOP8; }
static uint64_t variant_code_bytes(int v, uint64_t n) { return v == SZO_V_TOP8 ? 3ull * ceil_div(n, 8) : ceil_div(n, 2); }
static uint64_t variant_record_bytes(int v) { return v == SZO_V_SENTINEL ? 1ull : 3ull; }
static unsigned variant_codes(int v) { return v == SZO_V_SENTINEL ? 15u : 8u; }

static szo_layout variant_layout(int v, uint64_t n, uint64_t K) {
  szo_layout L;
  L.C = ceil_div(n, SZO_CHUNK);
  L.N0 = align256(64 + 16 * K + 8 * (L.C + 1));
  L.N1 = L.N0 + align256(variant_code_bytes(v, n));
  L.P = L.N1 + align256(n);
  return L;
}

uint64_t szo_variant_stream_size(int v, uint64_t n, uint32_t K, uint64_t E) {
  if (!variant_ok(v)) return 0;
  return variant_layout(v, n, K).P + variant_record_bytes(v) * E;
}

uint64_t szo_variant_max_size(int v, uint64_t n, uint32_t K) { return szo_variant_stream_size(v, n, K, n); }

/* Code of exponent e among the variant's first entries, or -1. */
static int variant_code_of(int v, const uint8_t *cb, unsigned e) {
  for (unsigned k = 0; k < variant_codes(v); ++k)
    if (cb[k] == e) return (int)k;
  return -1;
}

/* Code of element i in the code section. */
static unsigned variant_get_code(int v, const uint8_t *codes, uint64_t i) {
  if (v == SZO_V_SENTINEL) return (i % 2 == 0) ? (codes[i / 2] & 0xFu) : (codes[i / 2] >> 4);
  uint64_t q = i / 8, j = i % 8;
  uint64_t g = codes[3 * q] | ((uint64_t)codes[3 * q + 1] << 8) | ((uint64_t)codes[3 * q + 2] << 16);
  return (unsigned)((g >> (3 * j)) & 0x7u);
}

static void variant_put_code(int v, uint8_t *codes, uint64_t i, unsigned code) {
  if (v == SZO_V_SENTINEL) {
    if (i % 2 == 0)
      codes[i / 2] = (uint8_t)(codes[i / 2] | code);
    else
      codes[i / 2] = (uint8_t)(codes[i / 2] | (code << 4));
    return;
  }
  uint64_t q = i / 8, j = i % 8;
  uint64_t g = codes[3 * q] | ((uint64_t)codes[3 * q + 1] << 8) | ((uint64_t)codes[3 * q + 2] << 16);
  g |= (uint64_t)code << (3 * j);
  codes[3 * q] = (uint8_t)g;
  codes[3 * q + 1] = (uint8_t)(g >> 8);
  codes[3 * q + 2] = (uint8_t)(g >> 16);
}

int szo_variant_compress(int v, const void *in, uint64_t n, const uint8_t *cbs, uint32_t K, uint64_t seg,
                         uint8_t *out, uint64_t capacity, uint64_t *out_bytes) {
  if (!variant_ok(v)) return SZO_E_INVALID;
  int rc = compress_args_ok(SZO_BF16, in, n, cbs, K, seg);
  if (rc != SZO_OK) return rc;
  if (out == NULL) return SZO_E_INVALID;
  if (capacity < szo_variant_max_size(v, n, K)) return SZO_E_CAPACITY;
  szo_layout L = variant_layout(v, n, K);
  memset(out, 0, L.P);
  uint8_t *codes = out + L.N0;
  uint8_t *sm = out + L.N1;
  uint8_t *esc = out + L.P;
  uint8_t *off = out + 64 + 16ull * K;
  uint64_t E = 0;
  for (uint64_t c = 0; c < L.C; ++c) {
    const uint8_t *cb = cbs + 16ull * chunk_codebook(c, K, seg);
    uint64_t first = c * SZO_CHUNK;
    uint64_t last = first + SZO_CHUNK < n ? first + SZO_CHUNK : n;
    put_u64(off + 8 * c, E);
    for (uint64_t i = first; i < last; ++i) {
      unsigned e = get_exponent(SZO_BF16, in, i);
      int code = variant_code_of(v, cb, e);
      unsigned written;
      if (code >= 0) {
        written = (unsigned)code;
      } else if (v == SZO_V_SENTINEL) {
        written = 15; /* V2 */
        esc[E] = (uint8_t)e;
        E += 1;
      } else {
        written = 0; /* V3 */
        put_u16(esc + 3 * E, i - first);
        esc[3 * E + 2] = (uint8_t)e;
        E += 1;
      }
      variant_put_code(v, codes, i, written);
      sm[i] = (uint8_t)get_signmant(SZO_BF16, in, i);
    }
  }
  put_u64(off + 8 * L.C, E);
  uint64_t S = L.P + variant_record_bytes(v) * E;
  put_u32(out + 0, 0x00315A53u);
  put_u16(out + 4, 1);
  out[6] = (uint8_t)SZO_BF16;
  out[7] = 16;
  put_u64(out + 8, n);
  put_u64(out + 16, E);
  put_u64(out + 24, S);
  put_u32(out + 32, L.C);
  put_u32(out + 36, K);
  put_u64(out + 40, K == 1 ? n : seg);
  out[48] = (uint8_t)v; /* V1 */
  memcpy(out + 64, cbs, 16ull * K);
  if (out_bytes) *out_bytes = S;
  return SZO_OK;
}

int szo_variant_decompress(int v, const uint8_t *in, uint64_t in_bytes, uint64_t n, void *out) {
  if (!variant_ok(v) || in == NULL || (out == NULL && n > 0)) return SZO_E_INVALID;
  /* header */
  if (in_bytes < 64 || get_u32(in) != 0x00315A53u || get_u16(in + 4) != 1 || in[6] != SZO_BF16 || in[7] != 16 ||
      get_u64(in + 8) != n || in[48] != v)
    return SZO_E_CORRUPT;
  for (int k = 49; k < 64; ++k)
    if (in[k] != 0) return SZO_E_CORRUPT;
  uint64_t E = get_u64(in + 16), S = get_u64(in + 24), C = get_u32(in + 32), K = get_u32(in + 36);
  uint64_t seg = get_u64(in + 40);
  if (C != ceil_div(n, SZO_CHUNK) || K == 0 || K > SZO_MAX_K) return SZO_E_CORRUPT;
  if (K == 1 ? seg != n : (seg == 0 || seg % SZO_CHUNK != 0 || seg < ceil_div(n, K))) return SZO_E_CORRUPT;
  if (E > n) return SZO_E_CORRUPT;
  szo_layout L = variant_layout(v, n, K);
  if (S != L.P + variant_record_bytes(v) * E || S > in_bytes) return SZO_E_CORRUPT;
  for (uint64_t k = 0; k < K; ++k)
    if (!codebook_valid(SZO_BF16, in + 64 + 16 * k)) return SZO_E_CORRUPT;
  const uint8_t *off = in + 64 + 16 * K;
  const uint8_t *codes = in + L.N0;
  const uint8_t *sm = in + L.N1;
  const uint8_t *esc = in + L.P;
  if (get_u64(off) != 0 || get_u64(off + 8 * C) != E) return SZO_E_CORRUPT;
  for (uint64_t c = 0; c < C; ++c) {
    uint64_t lo = get_u64(off + 8 * c), hi = get_u64(off + 8 * (c + 1));
    if (lo > hi || hi > E) return SZO_E_CORRUPT;
    uint64_t first = c * SZO_CHUNK;
    uint64_t last = first + SZO_CHUNK < n ? first + SZO_CHUNK : n;
    if (v == SZO_V_SENTINEL) {
      uint64_t sentinels = 0;
      for (uint64_t i = first; i < last; ++i) sentinels += variant_get_code(v, codes, i) == 15;
      if (sentinels != hi - lo) return SZO_E_CORRUPT;
    } else {
      for (uint64_t r = lo; r < hi; ++r) {
        uint64_t pos = get_u16(esc + 3 * r);
        if (pos >= last - first) return SZO_E_CORRUPT;
        if (r > lo && pos <= get_u16(esc + 3 * (r - 1))) return SZO_E_CORRUPT;
      }
    }
  }
  /* dense pass, then (top-8) the escape overwrite */
  for (uint64_t c = 0; c < C; ++c) {
    const uint8_t *cb = in + 64 + 16 * chunk_codebook(c, K, seg);
    uint64_t first = c * SZO_CHUNK;
    uint64_t last = first + SZO_CHUNK < n ? first + SZO_CHUNK : n;
    uint64_t r = get_u64(off + 8 * c);
    for (uint64_t i = first; i < last; ++i) {
      unsigned code = variant_get_code(v, codes, i);
      unsigned e;
      if (v == SZO_V_SENTINEL && code == 15) {
        e = esc[r]; /* the r-th escape of the stream belongs to the r-th sentinel */
        r += 1;
      } else {
        e = cb[code];
      }
      put_element(SZO_BF16, out, i, e, sm[i]);
    }
  }
  if (v == SZO_V_TOP8) {
    for (uint64_t c = 0; c < C; ++c) {
      uint64_t lo = get_u64(off + 8 * c), hi = get_u64(off + 8 * (c + 1));
      for (uint64_t r = lo; r < hi; ++r) {
        uint64_t i = c * SZO_CHUNK + get_u16(esc + 3 * r);
        put_element(SZO_BF16, out, i, esc[3 * r + 2], get_signmant(SZO_BF16, out, i));
      }
    }
  }
  return SZO_OK;
}
