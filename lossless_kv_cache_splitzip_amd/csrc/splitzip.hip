// libsplitzip -- SplitZip exponent codec for MI355X (gfx950), hand-written HIP.
//
// Method: "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
// Serving" (arXiv 2605.01708v2).  The pages fix the arithmetic (Spanish
// technical summary, "Metodologia"): a BF16 value is split into its 8-bit
// exponent and an 8-bit sign|mantissa byte; the exponent is mapped through an
// offline top-16 codebook to a 4-bit code, two codes per byte; exponents
// outside the codebook go to a sparse escape stream of (16-bit position,
// 8-bit raw exponent); decode maps codes back through a lookup table,
// recombines, and overwrites the escaped exponents.  The stream layout (SZ1)
// is stated in include/splitzip.h.
//
// GPU design (ours):
//   prep          header, codebooks and the zero padding between sections:
//                 one extra workgroup of a later launch when the codebooks
//                 fit the kernel arguments, else launches of their own.
//   encode_dense  one workgroup per tile (8192 BF16 or 16384 E5M2 elements):
//                 16-byte loads issued before the codebook tables are built
//                 in LDS, then codes, nibbles and sign|mantissa bytes with
//                 byte permutes (E5M2: one OR of four per-byte-position
//                 exponent-table words per input word, the sign|mantissa
//                 triples by shifts and masks), non-temporal lane-contiguous
//                 stores, element-order escape ranks (wave64 DPP scan +
//                 LDS), escape records staged per tile in the workspace
//                 (input read once with non-temporal loads; the exponents
//                 of groups with escapes kept in LDS).
//   encode_sums   escape count of each block of 64 tiles.
//   encode_place  per range of 8 to 64 tiles: base (lower super-blocks,
//                 blocks and tiles), tile scan, chunk offsets, staged records
//                 moved to their place four at a time as whole words; tiles
//                 whose records overflowed their slot are encoded again and
//                 written through an LDS window.
//   encode_single splitzip_compress_static up to 512 tiles, one launch:
//                 each workgroup encodes its tile, publishes its escape
//                 count in the library's static array, adds up the lower
//                 tiles' counts (computing any that do not arrive in time)
//                 and writes its own records.
//   decode        one workgroup per tile inside one chunk (8192 BF16 or
//                 16384 E5M2 elements).  A short chunk's escape records (in
//                 groups of four, as words), then the dense data, are loaded
//                 first; the tile's escapes are staged in LDS (bitmap +
//                 values), after a 64-way wave search for a long chunk's
//                 records; codes go through an LDS table
//                 indexed by a whole nibble byte, and escapes are patched in
//                 registers before non-temporal stores.
//   *_sentinel_*, *_top8_*  the pages' two alternative designs (top-15 codes
//                 with a sentinel; 3-bit top-8 codes), for comparison.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "splitzip.h"

namespace {

constexpr uint64_t kChunk = 65536;
constexpr int kThreads = 256;
constexpr uint64_t kEncTileBf16 = 8192;   // elements per encode workgroup
constexpr uint64_t kEncTileE5m2 = 16384;
constexpr uint32_t kDecTileBf16 = 8192;   // elements per decode workgroup (measured best: BF16 8192,
constexpr uint32_t kDecTileE5m2 = 16384;  // E5M2 16384; larger tiles cost occupancy, smaller ones overhead)
constexpr uint32_t kMagic = 0x00315A53u;
constexpr uint32_t kMaxK = 65535;
constexpr uint64_t kMaxN = 1ull << 36;  // every grid then stays below 2^32 work-items
constexpr int kCbPerPrep = 128;
constexpr uint8_t kEsc = 0x10;  // table entry of an exponent outside the codebook

// Stream variants: the codec, and the two designs the pages compare it with
// (BF16 only): top-15 codes with code 15 as an escape sentinel and escapes
// stored as raw exponents only, and top-8 3-bit codes with the codec's
// position records.  Header byte 48 holds the variant (0 in the codec).
constexpr int kMain = 0, kSentinel = 1, kTop8 = 2;

__host__ __device__ inline uint64_t round256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
__host__ __device__ inline uint64_t divup(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Codebook of chunk c when a segment spans seg_chunks > 0 chunks, in 32-bit
// arithmetic (c < 2^20 since n <= 2^36); a 64-bit division would cost every
// wave a long emulation.
__device__ inline uint32_t codebook_of_chunk(uint64_t c, uint64_t seg_chunks) {
  return seg_chunks > 0xFFFFFFFFull ? 0u : (uint32_t)c / (uint32_t)seg_chunks;
}

struct Sections {
  uint64_t chunks, offsets, nib, sm, esc, sm_bytes, rec;  // nib: the code section; rec: bytes per escape
};

__host__ __device__ inline Sections sections_of(int dtype, uint64_t n, uint64_t k, int variant = kMain) {
  Sections s;
  s.chunks = divup(n, kChunk);
  s.offsets = 64 + 16 * k;
  s.nib = round256(s.offsets + 8 * (s.chunks + 1));
  s.sm_bytes = dtype == SPLITZIP_BF16 ? n : 3 * divup(n, 8);
  s.sm = s.nib + round256(variant == kTop8 ? 3 * divup(n, 8) : divup(n, 2));
  s.esc = s.sm + round256(s.sm_bytes);
  s.rec = variant == kSentinel ? 1 : 3;
  return s;
}

// Staged escape records per tile in the encoder workspace: enough for the
// codec's workloads (at most a few percent escapes); the top-8 variant, whose
// codes miss about 7% of exponents on the same data, gets twice as many.
__host__ __device__ constexpr uint32_t stage_slot(int variant) { return variant == kTop8 ? 1024u : 512u; }

// Encoder workspace, after the largest possible stream: u64 escapes per
// block of 64 tiles and per super-block of 64 blocks, u32 escapes per tile,
// then per tile a staging slot of stage_slot(variant) u32 records.
__host__ __device__ inline uint64_t workspace_offset(int dtype, uint64_t n, uint64_t k, int variant) {
  const Sections s = sections_of(dtype, n, k, variant);
  return round256(s.esc + s.rec * n);
}

struct Workspace {
  uint64_t* block_sum;
  uint64_t* super_sum;  // per 64 blocks
  uint32_t* tile_count;
  uint32_t* stage;
  uint64_t end;  // bytes from the stream start
};

// Byte offsets of the workspace parts from the stream start.
struct WorkspaceLayout {
  uint64_t block_sum, super_sum, tile_count, stage, end;
};

__host__ inline WorkspaceLayout workspace_layout(int dtype, uint64_t n, uint64_t k, int variant = kMain) {
  const uint64_t tiles = divup(n, 8192), blocks = divup(tiles, 64);
  WorkspaceLayout l;
  l.block_sum = workspace_offset(dtype, n, k, variant);
  l.super_sum = l.block_sum + 8 * blocks;
  l.tile_count = round256(l.block_sum + 8 * (blocks + divup(blocks, 64)));  // 16-byte loads in encode_sums
  l.stage = round256(l.tile_count + 4 * tiles);
  l.end = round256(l.stage + 4ull * stage_slot(variant) * tiles);
  return l;
}

__host__ inline Workspace workspace_of(uint8_t* out, int dtype, uint64_t n, uint64_t k, int variant = kMain) {
  const WorkspaceLayout l = workspace_layout(dtype, n, k, variant);
  Workspace w;
  w.block_sum = reinterpret_cast<uint64_t*>(out + l.block_sum);
  w.super_sum = reinterpret_cast<uint64_t*>(out + l.super_sum);
  w.tile_count = reinterpret_cast<uint32_t*>(out + l.tile_count);
  w.stage = reinterpret_cast<uint32_t*>(out + l.stage);
  w.end = l.end;
  return w;
}

// ----------------------------------------------------------------- helpers
// Streaming stores of the dense outputs: the codec never reads them back, so
// they are written non-temporally.  Used where a wave's store instruction
// covers contiguous memory (lane-contiguous words); for half-density
// patterns non-temporal stores measured slower than plain ones.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline void store_stream(void* p, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p)); }
__device__ inline void store_stream(void* p, uint2 v) {
  const u32x2_t t = {v.x, v.y};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
}
__device__ inline void store_stream(void* p, uint4 v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Inclusive prefix sum across a wave64: DPP row shifts inside each 16-lane
// row, then the row totals are carried with readlane.  All 64 lanes active.
__device__ inline uint32_t wave_inclusive_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
  const uint32_t row = __lane_id() >> 4;
  uint32_t carry = 0;
  carry += row >= 1 ? r0 : 0u;
  carry += row >= 2 ? r1 : 0u;
  carry += row >= 3 ? r2 : 0u;
  return v + carry;
}

// 4 table entries (code | escape flag << 4), one per byte, for BF16 word pair.
__device__ inline uint32_t gather4(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  return t0 | (t1 << 8) | (t2 << 16) | (t3 << 24);
}

// Register-array reads with a run-time index, as selects (no scratch memory).
__device__ inline uint32_t pick4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t i) {
  return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}

// Element-order bit mask of the escape flags (bit 4 of each byte) of a word
// of four table entries: flag of byte k -> bit k.
__device__ inline uint32_t flag_mask4(uint32_t codes) {
  const uint32_t t = (codes >> 4) & 0x01010101u;
  return ((t * 0x01020408u) >> 24) & 0xFu;
}

// Byte mask of four flag bits: bit k of f (k < 4) -> 0xFF in byte k.  The
// product moves bit k to bit 8k (the shifted copies never collide below
// bit 25), and perm selector 12 / 13 yields 0x00 / 0xFF.
__device__ inline uint32_t byte_mask4(uint32_t f) {
  return perm(0u, 0u, ((f * 0x00204081u) & 0x01010101u) | 0x0C0C0C0Cu);
}

__device__ inline uint32_t keep_low_bytes(uint32_t nbytes) {
  return nbytes >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nbytes)) - 1u);
}

// Codebook lookup of four 4-bit codes (one per byte of s; bits above 3 of
// each byte are ignored) through the 16-entry LUT held in l0..l3.
__device__ inline uint32_t lut4(uint32_t s, uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3) {
  const uint32_t idx = s & 0x07070707u;
  const uint32_t lo = perm(l1, l0, idx);
  const uint32_t hi = perm(l3, l2, idx);
  // selector 12 yields 0x00, 13 yields 0xFF: a byte mask from code bit 3
  const uint32_t m = perm(0u, 0u, ((s >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  return (hi & m) | (lo & ~m);
}

// ------------------------------------------------------------- prep kernel
struct PrepArgs {
  uint8_t* out;
  uint64_t n, seg_stored, nib, sm, esc, sm_bytes, offsets, chunks, code_bytes;
  uint64_t* out_bytes;
  uint32_t k, dtype, cb_first, cb_count, main, variant;
  uint8_t cbs[kCbPerPrep * 16];
};

__device__ inline void put_le(uint8_t* p, uint64_t v, int bytes) {
  for (int i = 0; i < bytes; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

// Header, codebooks and zero padding, by workgroup wg of n_wg.  Header bytes
// 16..31 (E and S) are written here only for n == 0; otherwise the placement
// pass writes them, possibly in the same launch.
__device__ void prep_work(const PrepArgs& a, uint32_t wg, uint32_t n_wg) {
  const uint64_t gtid = (uint64_t)wg * kThreads + threadIdx.x;
  const uint64_t gsize = (uint64_t)n_wg * kThreads;
  for (uint64_t i = gtid; i < (uint64_t)a.cb_count * 16; i += gsize)
    a.out[64 + 16 * (uint64_t)a.cb_first + i] = a.cbs[i];
  if (!a.main || wg != 0) return;
  const uint32_t t = threadIdx.x;
  // zero padding after the offsets, the nibbles and the sign|mantissa bytes
  const uint64_t ends[3] = {a.offsets + 8 * (a.chunks + 1), a.nib + a.code_bytes, a.sm + a.sm_bytes};
  const uint64_t stops[3] = {a.nib, a.sm, a.esc};
  for (int r = 0; r < 3; ++r)
    if (ends[r] + t < stops[r]) a.out[ends[r] + t] = 0;
  if (t < 64) {
    // byte t of the 64-byte header; E and S are final here only when n == 0
    uint64_t v = 0;
    int off = 0;
    if (t < 4) { v = kMagic; off = t; }
    else if (t < 6) { v = 1; off = t - 4; }
    else if (t == 6) { v = a.dtype; }
    else if (t == 7) { v = 16; }
    else if (t < 16) { v = a.n; off = t - 8; }
    else if (t < 32) { if (a.n != 0) return; v = t >= 24 ? a.esc : 0; off = t & 7; }
    else if (t < 36) { v = a.chunks; off = t - 32; }
    else if (t < 40) { v = a.k; off = t - 36; }
    else if (t < 48) { v = a.seg_stored; off = t - 40; }
    else if (t == 48) { v = a.variant; }
    a.out[t] = (uint8_t)(v >> (8 * off));
  }
  if (a.n == 0 && t == 0) {
    put_le(a.out + a.offsets, 0, 8);
    if (a.out_bytes) *a.out_bytes = a.esc;
  }
}

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) { prep_work(a, blockIdx.x, gridDim.x); }

// ---------------------------------------------------------- encode kernels
//
// Three launches (two with at most 64 blocks: no encode_sums); no workgroup
// waits on another, so no launch needs co-residency:
//   encode_dense  one workgroup per tile (8192 BF16 or 16384 E5M2
//                 elements): dense encode (codes,
//                 sign|mantissa) and element-order escape ranks.  The tile's
//                 escape count goes to the workspace; when it holds at most
//                 stage_slot escapes its records go to the tile's staging
//                 slot.
//   encode_sums   one thread per block of kBlockTiles tiles: the block's
//                 escape count.
//   encode_place  one workgroup per range of 8 to 64 tiles (about 2048
//                 workgroups): the range's base (sum of the lower blocks and
//                 tiles), scan of its tiles' counts, chunk offsets (E and S
//                 for the last range), staged records moved to their place
//                 four at a time as whole words; a tile whose escapes
//                 overflowed its slot is encoded again and its records go
//                 through an LDS window, also as whole words.
struct EncArgs {
  const uint8_t* in;
  uint8_t* out;
  uint64_t n, n_tiles, n_blocks, offsets, nib, sm, esc, chunks;
  uint64_t seg_chunks;    // chunks per codebook segment, 0 when one codebook
  uint32_t* tile_count;   // per tile: escapes in it
  uint32_t* stage;        // per tile: stage_slot(variant) records (position | exponent << 16)
  uint64_t* block_sum;    // per block of kBlockTiles tiles: escapes in it
  uint64_t* super_sum;    // per 64 blocks: escapes in them
  uint64_t* out_bytes;
  uint32_t place_tiles;   // tiles per encode_place workgroup: 8, 16, 32 or 64
  uint32_t cb_args;       // codebooks read from prep.cbs (all of them fit), else from the stream
  uint32_t prep_in;       // header, codebooks and padding written by: 0 prep_kernel, 1 encode_sums, 2 encode_place
  uint32_t sums_in_place; // at most 64 blocks: encode_place sums the lower tiles itself, encode_sums is not launched
  uint32_t* single;       // encode_single: arrival counter and per-tile count words (static array)
  uint32_t wait_polls;    // encode_single: polls for a lower tile's count before it is computed here
  PrepArgs prep;          // the header work folded into a later launch (prep_in 1, 2 or 3)
};

constexpr uint32_t kBlockTiles = 64;  // tiles per block of the escape-count sums (a placement range lies inside one)

struct EncShared {
  uint8_t table[256];
  // E5M2: words 32j + e, for the exponent e of the element at byte position
  // j of a 4-element word: code << 4j | escaped << (28 + j).  Indexed by the
  // 5-bit exponent, lanes holding the same exponent read one address
  // (broadcast) and different exponents fall in different banks.  After the
  // tile's rank scan the array holds the tile's staged escape records.
  uint32_t pos4[4 * 256];
  uint32_t wave[8];
  uint64_t red[16];
  alignas(16) uint32_t s3[4 * 96];  // E5M2: a wave's 64 x 6 sign|mantissa bytes, gathered for aligned stores
};

static_assert(stage_slot(kMain) <= 4 * 256 && stage_slot(kTop8) <= 4 * 256,
              "staged records reuse the E5M2 table space");

constexpr uint32_t kPlaceRecs = 2048;  // escape records per LDS window of place_range
constexpr uint32_t kPlaceWgs = 2048;   // encode_place aims at this many workgroups


// Exclusive prefix over the workgroup's threads (thread order) of per-thread
// u32 values whose sum over the workgroup fits 32 bits; *total gets the sum.
template <int kWaves>
__device__ inline uint32_t block_exclusive_sum(uint64_t* red, uint32_t v, uint32_t* total) {
  const uint32_t inc = wave_inclusive_sum(v);
  const uint32_t wave = threadIdx.x >> 6;
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 63) red[wave] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (uint32_t w = 0; w < kWaves; ++w) {
    pre += w < wave ? (uint32_t)red[w] : 0u;
    tot += (uint32_t)red[w];
  }
  *total = tot;
  return pre + inc - v;
}

// Exponent -> code table of codebook cbi: the first `codes` entries get their
// code, every other exponent the escape entry (kEsc; with the sentinel
// variant kEsc | 15, so an escape's nibble is the sentinel).
template <int kVariant = kMain>
__device__ inline void build_table(const EncArgs& a, EncShared& sh, uint64_t cbi, uint32_t entries,
                                   uint32_t tid = threadIdx.x) {
  constexpr uint32_t kCodes = kVariant == kSentinel ? 15 : kVariant == kTop8 ? 8 : 16;
  constexpr uint8_t kEscEntry = kVariant == kSentinel ? (kEsc | 15) : kEsc;
  if (tid < entries) sh.table[tid] = kEscEntry;
  __syncthreads();
  if (tid < kCodes) sh.table[a.cb_args ? a.prep.cbs[16 * cbi + tid] : a.out[64 + 16 * cbi + tid]] = (uint8_t)tid;
  __syncthreads();
  if (entries == 32) {  // E5M2 per-position words, from the exponent table
    if (tid < 128) {
      const uint32_t j = tid >> 5, c = sh.table[tid & 31u];
      sh.pos4[tid] = ((c & 0xFu) << (4 * j)) | ((c >> 4) << (28 + j));  // kEsc: code 0, escaped
    }
    __syncthreads();
  }
}

// Per-thread escape bookkeeping of one tile: element-order rank of the
// thread's first escape in each group, and the escape masks.
struct TileEsc {
  uint32_t agg;      // escapes in the tile
  uint32_t rank[4];  // per group (4 groups: BF16 8 elements per thread, E5M2 16)
  uint32_t mask[4];  // escaped elements of each group, bit j = element j
  uint32_t g01, g23; // escapes of groups 0 and 1, 2 and 3 (16-bit fields; the same in every thread)
};

__device__ inline void wave_totals_to_lds(EncShared& sh, uint32_t i01, uint32_t i23, uint32_t tid) {
  const uint32_t wave = tid >> 6;
  if ((tid & 63) == 63) {
    sh.wave[wave] = i01;
    sh.wave[4 + wave] = i23;
  }
  __syncthreads();
}

// Element-order ranks of a tile of four groups: groups are ordered (g,
// thread), so the four per-thread counts are scanned as 16-bit fields (a
// group holds at most 4096 escapes).
__device__ inline void tile_ranks4(EncShared& sh, const uint32_t cnt[4], TileEsc& r, uint32_t tid) {
  const uint32_t wave = tid >> 6;
  const uint32_t p01 = cnt[0] | (cnt[1] << 16), p23 = cnt[2] | (cnt[3] << 16);
  const uint32_t i01 = wave_inclusive_sum(p01), i23 = wave_inclusive_sum(p23);
  wave_totals_to_lds(sh, i01, i23, tid);
  uint32_t pre01 = 0, pre23 = 0, tot01 = 0, tot23 = 0;
#pragma unroll
  for (uint32_t v = 0; v < 4; ++v) {
    const uint32_t x = sh.wave[v], y = sh.wave[4 + v];
    pre01 += v < wave ? x : 0u;
    pre23 += v < wave ? y : 0u;
    tot01 += x;
    tot23 += y;
  }
  const uint32_t g0 = tot01 & 0xFFFF, g1 = tot01 >> 16, g2 = tot23 & 0xFFFF, g3 = tot23 >> 16;
  r.agg = g0 + g1 + g2 + g3;
  r.g01 = tot01;
  r.g23 = tot23;
  const uint32_t x01 = pre01 + i01 - p01, x23 = pre23 + i23 - p23;
  r.rank[0] = x01 & 0xFFFF;
  r.rank[1] = g0 + (x01 >> 16);
  r.rank[2] = g0 + g1 + (x23 & 0xFFFF);
  r.rank[3] = g0 + g1 + g2 + (x23 >> 16);
}

// BF16 tile: 8192 elements = 4 groups of 2048; thread t owns elements
// 8t..8t+7 of each group (16-byte loads, coalesced per wave).
// Input of one BF16 tile in registers (loaded ahead of its encode).
struct TileIn {
  uint4 w[4];
};

__device__ inline uint32_t valid_in_group(uint64_t n, uint64_t e0, uint32_t width) {
  return e0 >= n ? 0u : (uint32_t)std::min<uint64_t>(width, n - e0);
}

__device__ inline TileIn load_tile_bf16(const EncArgs& a, uint64_t tile, uint32_t tid = threadIdx.x) {
  const uint64_t first = tile * kEncTileBf16;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(a.in) + first;
  TileIn in;
  uint4* w = in.w;
  if (first + kEncTileBf16 <= a.n) {  // same in every thread
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // read once: non-temporal
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + g * 2048 + 8 * tid));
      w[g] = make_uint4(v.x, v.y, v.z, v.w);
    }
    return in;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t local = g * 2048 + 8 * tid;
    const uint32_t valid = valid_in_group(a.n, first + local, 8);
    uint32_t v0 = 0, v1 = 0, v2 = 0, v3 = 0;
    for (uint32_t j = 0; j < valid; ++j) {
      const uint32_t x = (uint32_t)src[local + j] << (16 * (j & 1));
      if (j < 2) v0 |= x;
      else if (j < 4) v1 |= x;
      else if (j < 6) v2 |= x;
      else v3 |= x;
    }
    w[g] = make_uint4(v0, v1, v2, v3);
  }
  return in;
}

// Codes of one word of four table entries (code | escape << 4 per byte) and
// the next word, as 8 nibbles (even element low): per byte, the code and the
// next byte's code moved to the high nibble, then the even bytes.
__device__ inline uint32_t pack_codes8(uint32_t c_lo, uint32_t c_hi) {
  const uint32_t u = (c_lo & 0x0F0F0F0Fu) | ((c_lo >> 4) & 0xF0F0F0F0u);
  const uint32_t v = (c_hi & 0x0F0F0F0Fu) | ((c_hi >> 4) & 0xF0F0F0F0u);
  return perm(v, u, 0x06040200u);
}

// Four table bytes (code in bits 0..2 of each) -> 12 bits, code k at bit 3k.
__device__ inline uint32_t codes12(uint32_t w) {
  const uint32_t t = w & 0x07070707u;
  const uint32_t v = t | (t >> 5);  // bits 0..5: c0 | c1 << 3; bits 16..21: c2 | c3 << 3
  return (v & 0x3Fu) | ((v >> 10) & 0xFC0u);
}

// With `exps` (the dense kernel), every thread of a wave in which any thread
// holds an escape in a group writes that group's 8 exponent bytes to
// exps[element]: the escape pass reads them there, so the input is read
// once, with non-temporal loads (re-reading an escape's exponent from the
// input would then miss the cache).  Groups without escapes in the wave skip
// the writes.

template <int kVariant = kMain>
__device__ TileEsc encode_tile_bf16(const EncArgs& a, EncShared& sh, uint64_t tile, const TileIn& in, bool store,
                                   uint32_t tid = threadIdx.x, uint8_t* exps = nullptr) {
  const uint32_t lane = tid & 63, wave = tid >> 6;
  const uint64_t first = tile * kEncTileBf16;
  const bool tile_full = first + kEncTileBf16 <= a.n;  // same in every thread
  const uint4* w = in.w;
  TileEsc r;
  uint32_t cnt[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t local = g * 2048 + 8 * tid;
    const uint4 x = w[g];
    const uint8_t* tb = sh.table;
    uint32_t lo = gather4(tb[(x.x >> 7) & 0xFF], tb[(x.x >> 23) & 0xFF], tb[(x.y >> 7) & 0xFF], tb[(x.y >> 23) & 0xFF]);
    uint32_t hi = gather4(tb[(x.z >> 7) & 0xFF], tb[(x.z >> 23) & 0xFF], tb[(x.w >> 7) & 0xFF], tb[(x.w >> 23) & 0xFF]);
    uint32_t valid = 8;
    if (!tile_full) {  // elements past n: no code, no escape
      valid = valid_in_group(a.n, first + local, 8);
      lo &= keep_low_bytes(valid);
      hi &= valid > 4 ? keep_low_bytes(valid - 4) : 0u;
    }
    // escape flags, element k of lo at bit 8k and element 4 + k at bit 8k + 1
    const uint32_t f = ((lo >> 4) & 0x01010101u) | ((hi >> 3) & 0x02020202u);
    r.mask[g] = f;
    cnt[g] = __builtin_popcount(f);
    if (exps && __ballot(f != 0)) {  // same in the wave
      const uint32_t e03 = perm((x.y >> 7) & 0x00FF00FFu, (x.x >> 7) & 0x00FF00FFu, 0x06040200u);
      const uint32_t e47 = perm((x.w >> 7) & 0x00FF00FFu, (x.z >> 7) & 0x00FF00FFu, 0x06040200u);
      *reinterpret_cast<uint2*>(exps + local) = make_uint2(e03, e47);
    }
    if (store) {
      // sign|mantissa: high bytes and low bytes of the four BF16 pairs
      const uint32_t h01 = perm(x.y, x.x, 0x07050301u), l01 = perm(x.y, x.x, 0x06040200u);
      const uint32_t h23 = perm(x.w, x.z, 0x07050301u), l23 = perm(x.w, x.z, 0x06040200u);
      const uint32_t sm0 = (h01 & 0x80808080u) | (l01 & 0x7F7F7F7Fu);
      const uint32_t sm1 = (h23 & 0x80808080u) | (l23 & 0x7F7F7F7Fu);
      if (kVariant == kTop8) {
        // 8 codes of 3 bits, element j at bit 3j: 3 bytes per thread, gathered
        // per wave in LDS for 12 aligned 16-byte stores (in-order LDS within
        // a wave: only the compiler needs a barrier)
        const uint32_t c24 = codes12(lo) | (codes12(hi) << 12);
        if (tile_full) {
          uint8_t* buf = reinterpret_cast<uint8_t*>(sh.s3 + wave * 96);
          buf[3 * lane] = (uint8_t)c24;
          buf[3 * lane + 1] = (uint8_t)(c24 >> 8);
          buf[3 * lane + 2] = (uint8_t)(c24 >> 16);
          asm volatile("" ::: "memory");
          if (lane < 12)
            store_stream(a.out + a.nib + 3 * ((first + g * 2048 + 512 * wave) / 8) + 16 * lane,
                         *reinterpret_cast<const uint4*>(sh.s3 + wave * 96 + 4 * lane));
          asm volatile("" ::: "memory");
        } else if (valid > 0) {
          const uint64_t e0 = first + local;
          for (uint32_t b = 0; b < 3 * ((valid + 7) / 8); ++b) a.out[a.nib + 3 * (e0 / 8) + b] = (uint8_t)(c24 >> (8 * b));
        }
      } else {
        const uint32_t nib = pack_codes8(lo, hi);
        if (tile_full) {
          store_stream(a.out + a.nib + first / 2 + local / 2, nib);
        } else if (valid > 0) {
          const uint64_t e0 = first + local;
          for (uint32_t b = 0; b < (valid + 1) / 2; ++b) a.out[a.nib + e0 / 2 + b] = (uint8_t)(nib >> (8 * b));
        }
      }
      if (tile_full) {
        store_stream(a.out + a.sm + first + local, make_uint2(sm0, sm1));
      } else if (valid > 0) {
        const uint64_t e0 = first + local;
        for (uint32_t j = 0; j < valid; ++j) a.out[a.sm + e0 + j] = (uint8_t)((j < 4 ? sm0 : sm1) >> (8 * (j & 3)));
      }
    }
  }
  tile_ranks4(sh, cnt, r, tid);
  return r;
}

// The escapes of one BF16 tile: position in chunk and raw exponent, handed
// to `put(rank, pos, exponent)` in element order (a thread's escapes of one
// group have consecutive ranks).  Dense kernel: the exponents come from
// `exps` (every group with an escape in the thread's wave was written there).
template <typename Put>
__device__ inline void dense_escapes_bf16(uint64_t tile, const TileEsc& r, const uint8_t* exps, Put put) {
  const uint32_t tid = threadIdx.x;
  const uint32_t in_chunk = (uint32_t)(tile & 7) * (uint32_t)kEncTileBf16;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t f = r.mask[g];  // element k at bit 8k, element 4 + k at bit 8k + 1
    if (!f) continue;
    uint32_t m = flag_mask4(f << 4) | (flag_mask4(f << 3) << 4), k = r.rank[g];  // element order
    const uint32_t local = g * 2048 + 8 * tid;
    const uint2 e = *reinterpret_cast<const uint2*>(exps + local);
    while (m) {
      const uint32_t j = __builtin_ctz(m);
      m &= m - 1;
      put(k++, in_chunk + local + j, ((j < 4 ? e.x : e.y) >> (8 * (j & 3))) & 0xFF);
    }
  }
}

// Re-encode of a tile that overflowed its slot: exponents from the tile's
// registers, and only ranks in [w0, w0 + wlen) are wanted (groups whose
// ranks all miss the window are skipped).
__device__ inline bool ranks_miss(uint32_t k, uint32_t count, uint32_t w0, uint32_t wlen) {
  return k + count <= w0 || (k >= w0 && k - w0 >= wlen);
}

// Words of group g of a tile's registers, by selects (no scratch memory).
__device__ inline uint4 pick_group(const TileIn& in, uint32_t g) {
  return make_uint4(pick4(in.w[0].x, in.w[1].x, in.w[2].x, in.w[3].x, g), pick4(in.w[0].y, in.w[1].y, in.w[2].y, in.w[3].y, g),
                    pick4(in.w[0].z, in.w[1].z, in.w[2].z, in.w[3].z, g), pick4(in.w[0].w, in.w[1].w, in.w[2].w, in.w[3].w, g));
}

// The records of group g of an escape-dense BF16 tile, handed to
// put(index within the group, position, exponent): each element of the
// thread is tried in turn (unrolled, so its word is a fixed register) and,
// if escaped, put at its rank in the group; no per-escape loop.
template <typename Put>
__device__ inline void group_escapes_bf16(uint64_t tile, const TileEsc& r, const TileIn& in, uint32_t g,
                                          uint32_t g_first, uint32_t tid, Put put) {
  const uint32_t in_chunk = (uint32_t)(tile & 7) * (uint32_t)kEncTileBf16;
  const uint32_t f = pick4(r.mask[0], r.mask[1], r.mask[2], r.mask[3], g);
  if (!f) return;
  const uint32_t m = flag_mask4(f << 4) | (flag_mask4(f << 3) << 4);  // element j at bit j
  const uint32_t k0 = pick4(r.rank[0], r.rank[1], r.rank[2], r.rank[3], g) - g_first;
  const uint4 w = pick_group(in, g);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  const uint32_t p0 = in_chunk + g * 2048 + 8 * tid;
#pragma unroll
  for (uint32_t j = 0; j < 8; ++j) {
    if ((m >> j) & 1u) put(k0 + __builtin_popcount(m & ((1u << j) - 1u)), p0 + j, (wd[j >> 1] >> (16 * (j & 1) + 7)) & 0xFF);
  }
}

// E5M2 tile: 16384 elements = 4 groups of 4096; thread t owns elements
// 16t..16t+15 of each group: 16 input bytes, 8 nibble bytes and 6
// sign|mantissa bytes, all lane-contiguous across a wave.
__device__ inline TileIn load_tile_e5m2(const EncArgs& a, uint64_t tile, uint32_t tid = threadIdx.x) {
  TileIn in;
  const uint64_t first = tile * kEncTileE5m2;
  const uint8_t* src = a.in + first;
  if (first + kEncTileE5m2 <= a.n) {  // same in every thread
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + g * 4096 + 16 * tid));
      in.w[g] = make_uint4(v.x, v.y, v.z, v.w);
    }
    return in;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t local = g * 4096 + 16 * tid;
    const uint32_t valid = valid_in_group(a.n, first + local, 16);
    uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      for (uint32_t b = 0; b < 4 && 4 * k + b < valid; ++b) v[k] |= (uint32_t)src[local + 4 * k + b] << (8 * b);
    in.w[g] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  return in;
}

// Per-position table words of the exponents of the four bytes of x, OR-ed:
// nibble codes of the four elements in bits 0..15, escape flags in bits
// 28..31.
__device__ inline uint32_t e5m2_pos_word(const uint32_t* pos4, uint32_t x) {
  return pos4[(x >> 2) & 0x1Fu] | pos4[32 + ((x >> 10) & 0x1Fu)] | pos4[64 + ((x >> 18) & 0x1Fu)] |
         pos4[96 + ((x >> 26) & 0x1Fu)];
}

// Sign|mantissa triples (sign << 2 | mantissa) of the four bytes of x, the
// element at byte j in bits 3j..3j+2: the triples land in bytes, then pairs
// of bytes are merged and the two halves joined.
__device__ inline uint32_t e5m2_tri12(uint32_t x) {
  const uint32_t t = ((x >> 5) & 0x04040404u) | (x & 0x03030303u);
  const uint32_t v = t | (t >> 5);  // bits 0..5: t0 | t1 << 3; bits 16..21: t2 | t3 << 3
  return (v & 0x3Fu) | ((v >> 10) & 0xFC0u);
}

constexpr uint32_t kEscSlots = 16;  // per wave and group: input words of lanes with escapes kept in LDS

__device__ inline uint32_t lane_slot(uint64_t bal) {  // lanes below this one in bal
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

__device__ TileEsc encode_tile_e5m2(const EncArgs& a, EncShared& sh, uint64_t tile, const TileIn& in, bool store,
                                   uint32_t tid = threadIdx.x, uint4* escw = nullptr) {
  const uint32_t lane = tid & 63, wave = tid >> 6;
  const uint64_t first = tile * kEncTileE5m2;
  const bool tile_full = first + kEncTileE5m2 <= a.n;  // same in every thread
  TileEsc r;
  uint32_t cnt[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t local = g * 4096 + 16 * tid;
    const uint32_t r0 = e5m2_pos_word(sh.pos4, in.w[g].x), r1 = e5m2_pos_word(sh.pos4, in.w[g].y);
    const uint32_t r2 = e5m2_pos_word(sh.pos4, in.w[g].z), r3 = e5m2_pos_word(sh.pos4, in.w[g].w);
    // escape flags in element order, nibbles, 16 triples = 48 bits (element i at bit 3i)
    uint32_t f = (r0 >> 28) | ((r1 >> 24) & 0xF0u) | ((r2 >> 20) & 0xF00u) | ((r3 >> 16) & 0xF000u);
    uint2 nib = make_uint2(perm(r1, r0, 0x05040100u), perm(r3, r2, 0x05040100u));
    const uint32_t t2 = e5m2_tri12(in.w[g].z);
    uint32_t lo = e5m2_tri12(in.w[g].x) | (e5m2_tri12(in.w[g].y) << 12) | (t2 << 24);
    uint32_t hi = (t2 >> 8) | (e5m2_tri12(in.w[g].w) << 4);
    uint32_t valid = 16;
    if (!tile_full) {  // elements past n: no code, no triple, no escape
      valid = valid_in_group(a.n, first + local, 16);
      const uint64_t k48 = (1ull << (3 * valid)) - 1, k64 = valid >= 16 ? ~0ull : (1ull << (4 * valid)) - 1;
      f &= (1u << valid) - 1u;
      nib.x &= (uint32_t)k64;
      nib.y &= (uint32_t)(k64 >> 32);
      lo &= (uint32_t)k48;
      hi &= (uint32_t)(k48 >> 32);
    }
    r.mask[g] = f;
    cnt[g] = __builtin_popcount(f);
    if (escw) {
      const uint64_t bal = __ballot(f != 0);
      if (bal) {  // same in the wave
        const uint32_t slot = lane_slot(bal);
        if (f && slot < kEscSlots) escw[(wave * 4 + g) * kEscSlots + slot] = in.w[g];
      }
    }
    if (!store) continue;
    if (tile_full) {
      store_stream(a.out + a.nib + (first + local) / 2, nib);
      // the wave's 64 x 6 sign|mantissa bytes go through its own LDS slice
      // to 24 aligned 16-byte stores.  A wave's LDS operations complete in
      // issue order, so only the compiler needs a barrier here.
      uint16_t* buf = reinterpret_cast<uint16_t*>(sh.s3 + wave * 96);
      buf[3 * lane] = (uint16_t)lo;
      buf[3 * lane + 1] = (uint16_t)(lo >> 16);
      buf[3 * lane + 2] = (uint16_t)hi;
      asm volatile("" ::: "memory");
      if (lane < 24) {
        const uint64_t wave_smo = a.sm + 6 * ((first + g * 4096 + 1024 * wave) / 16);
        store_stream(a.out + wave_smo + 16 * lane, *reinterpret_cast<const uint4*>(sh.s3 + wave * 96 + 4 * lane));
      }
      asm volatile("" ::: "memory");
    } else if (valid > 0) {
      const uint64_t e0 = first + local;
      const uint64_t smo = a.sm + 6 * (e0 / 16);
      for (uint32_t b = 0; b < (valid + 1) / 2; ++b)
        a.out[a.nib + e0 / 2 + b] = (uint8_t)((b < 4 ? nib.x : nib.y) >> (8 * (b & 3)));
      for (uint32_t b = 0; b < 3 * ((valid + 7) / 8); ++b)
        a.out[smo + b] = (uint8_t)((b < 4 ? lo : hi) >> (8 * (b & 3)));
    }
  }
  tile_ranks4(sh, cnt, r, tid);
  return r;
}

// The escapes of one E5M2 tile, handed to `put` as for BF16.  Dense kernel:
// the input is read once (non-temporal loads); during the encode pass each
// lane holding escapes in a group stored its 16-byte input word in its wave's
// LDS slots for that group (the lane's rank among such lanes), so the
// exponents come from LDS; a lane ranked beyond the kEscSlots slots (more
// than 16 lanes of a wave with escapes in one group) reads its word again
// from the input.
template <typename Put>
__device__ inline void dense_escapes_e5m2(const EncArgs& a, uint64_t tile, const TileEsc& r, const uint4* escw,
                                          Put put) {
  const uint32_t tid = threadIdx.x, wave = tid >> 6;
  const uint8_t* in8 = a.in + tile * kEncTileE5m2;
  const uint32_t in_chunk = (uint32_t)(tile & 3) * (uint32_t)kEncTileE5m2;
  uint32_t slot[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) slot[g] = lane_slot(__ballot(r.mask[g] != 0));
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t m = r.mask[g], k = r.rank[g];
    if (!m) continue;
    const uint32_t local = g * 4096 + 16 * tid;
    uint4 w;
    if (slot[g] < kEscSlots) {
      w = escw[(wave * 4 + g) * kEscSlots + slot[g]];
    } else {  // more lanes with escapes than slots: the input again
      w = *reinterpret_cast<const uint4*>(in8 + local);
    }
    while (m) {
      const uint32_t j = __builtin_ctz(m);
      m &= m - 1;
      const uint32_t x = pick4(w.x, w.y, w.z, w.w, j >> 2) >> (8 * (j & 3));
      put(k++, in_chunk + local + j, (x >> 2) & 0x1F);
    }
  }
}

template <typename Put>
__device__ inline void window_escapes_e5m2(uint64_t tile, const TileEsc& r, const TileIn& in, uint32_t w0,
                                           uint32_t wlen, uint32_t tid, Put put) {
  const uint32_t in_chunk = (uint32_t)(tile & 3) * (uint32_t)kEncTileE5m2;
#pragma unroll 1
  for (uint32_t g = 0; g < 4; ++g) {
    const uint32_t m = pick4(r.mask[0], r.mask[1], r.mask[2], r.mask[3], g);  // element j at bit j
    const uint32_t k0 = pick4(r.rank[0], r.rank[1], r.rank[2], r.rank[3], g);
    if (ranks_miss(k0, __builtin_popcount(m), w0, wlen)) continue;
    const uint4 w = pick_group(in, g);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const uint32_t p0 = in_chunk + g * 4096 + 16 * tid;
#pragma unroll
    for (uint32_t j = 0; j < 16; ++j) {
      if ((m >> j) & 1u) put(k0 + __builtin_popcount(m & ((1u << j) - 1u)), p0 + j, (wd[j >> 2] >> (8 * (j & 3) + 2)) & 0x1F);
    }
  }
}

template <int kVariant = kMain>
__device__ inline void put_record(const EncArgs& a, uint64_t index, uint32_t pos, uint32_t val) {
  if (index >= a.n) return;  // never taken for a correct scan; keeps stores inside the stream
  if (kVariant == kSentinel) {  // the raw exponent only
    a.out[a.esc + index] = (uint8_t)val;
    return;
  }
  uint8_t* d = a.out + a.esc + 3 * index;
  d[0] = (uint8_t)pos;
  d[1] = (uint8_t)(pos >> 8);
  d[2] = (uint8_t)val;
}

// Records idx .. idx+3 (idx a multiple of 4, each position | exponent << 16):
// whole 4-byte words of the escape section, which is 256-aligned -- 3 words
// of [pos lo, pos hi, exponent] records, or 1 word of exponent bytes with the
// sentinel variant.
template <int kVariant = kMain>
__device__ inline void put_record_group(const EncArgs& a, uint64_t idx, uint32_t r0, uint32_t r1, uint32_t r2,
                                        uint32_t r3) {
  if (idx + 4 > a.n) return;  // never taken for a correct scan; keeps stores inside the stream
  if (kVariant == kSentinel) {
    *reinterpret_cast<uint32_t*>(a.out + a.esc + idx) =
        (r0 >> 16) | ((r1 >> 8) & 0xFF00u) | (r2 & 0xFF0000u) | ((r3 << 8) & 0xFF000000u);
    return;
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(a.out + a.esc + 3 * idx);
  d[0] = (r0 & 0xFFFFFFu) | (r1 << 24);
  d[1] = ((r1 >> 8) & 0xFFFFu) | (r2 << 16);
  d[2] = ((r2 >> 16) & 0xFFu) | (r3 << 8);
}

// LDS of a dense tile encode beside EncShared: BF16, the exponent bytes by
// element; E5M2, the input words of lanes with escapes.
template <bool kBf16>
struct DenseLds {
  alignas(16) uint8_t exps[kBf16 ? kEncTileBf16 : 16 * 16 * kEscSlots];
};

// Tile t: dense encode, its escape count to the workspace and, when they fit
// its slot, its escape records staged there.
template <bool kBf16, int kVariant = kMain>
__device__ void dense_tile(const EncArgs& a, EncShared& sh, DenseLds<kBf16>& dl, uint64_t t) {
  uint8_t* exps = dl.exps;
  const TileIn in = kBf16 ? load_tile_bf16(a, t) : load_tile_e5m2(a, t);  // in flight during the table build
  build_table<kVariant>(a, sh, a.seg_chunks ? codebook_of_chunk(t >> (kBf16 ? 3 : 2), a.seg_chunks) : 0,
                        kBf16 ? 256u : 32u);
  uint4* escw = reinterpret_cast<uint4*>(exps);
  const TileEsc r = kBf16 ? encode_tile_bf16<kVariant>(a, sh, t, in, true, threadIdx.x, exps)
                          : encode_tile_e5m2(a, sh, t, in, true, threadIdx.x, escw);
  if (threadIdx.x == 0) a.tile_count[t] = r.agg;
  constexpr uint32_t kSlot = stage_slot(kVariant);
  if (r.agg <= kSlot) {  // uniform
    // records gathered in LDS first (the E5M2 tables are dead after the
    // rank scan's barrier), then written to the slot with contiguous
    // stores instead of scattered 4-byte ones
    uint32_t* rec = sh.pos4;
    auto stage = [&](uint32_t k, uint32_t pos, uint32_t val) { rec[k] = pos | (val << 16); };
    if (kBf16) dense_escapes_bf16(t, r, exps, stage);
    else dense_escapes_e5m2(a, t, r, escw, stage);
    __syncthreads();
    uint32_t* slot = a.stage + t * kSlot;
    for (uint32_t i = threadIdx.x; i < r.agg; i += kThreads) slot[i] = rec[i];
  }
}

template <bool kBf16, int kVariant = kMain>
__device__ void encode_dense(const EncArgs& a) {
  __shared__ EncShared sh;
  __shared__ DenseLds<kBf16> dl;
  dense_tile<kBf16, kVariant>(a, sh, dl, blockIdx.x);
}

__global__ __launch_bounds__(kThreads) void encode_dense_bf16_kernel(EncArgs a) { encode_dense<true>(a); }
__global__ __launch_bounds__(kThreads) void encode_dense_e5m2_kernel(EncArgs a) { encode_dense<false>(a); }
__global__ __launch_bounds__(kThreads) void encode_dense_sentinel_kernel(EncArgs a) { encode_dense<true, kSentinel>(a); }
__global__ __launch_bounds__(kThreads) void encode_dense_top8_kernel(EncArgs a) { encode_dense<true, kTop8>(a); }

// One thread per block of 64 tiles, one wave per 64 blocks (a super-block):
// block sums, and each wave's total as its super-block sum.
__global__ __launch_bounds__(kThreads) void encode_sums_kernel(EncArgs a) {
  if (a.prep_in == 1 && blockIdx.x == gridDim.x - 1) {  // the launch's extra workgroup
    prep_work(a.prep, 0, 1);
    return;
  }
  const uint64_t blk = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint64_t t0 = blk * kBlockTiles, t1 = std::min<uint64_t>(t0 + kBlockTiles, a.n_tiles);
  uint64_t sum = 0;
  if (blk >= a.n_blocks) {
    // past the last block: contributes 0 to its wave's total
  } else if (t1 - t0 == kBlockTiles) {  // 16 x 16-byte loads, issued together
    const uint4* c = reinterpret_cast<const uint4*>(a.tile_count + t0);
    uint4 v[kBlockTiles / 4];
#pragma unroll
    for (uint32_t i = 0; i < kBlockTiles / 4; ++i) v[i] = c[i];
#pragma unroll
    for (uint32_t i = 0; i < kBlockTiles / 4; ++i) sum += (uint64_t)v[i].x + v[i].y + v[i].z + v[i].w;
  } else {
    for (uint64_t t = t0; t < t1; ++t) sum += a.tile_count[t];
  }
  if (blk < a.n_blocks) a.block_sum[blk] = sum;
  uint64_t v = sum;  // wave total, all 64 lanes active
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  if ((threadIdx.x & 63) == 0 && blk < a.n_blocks) a.super_sum[blk >> 6] = v;
}

constexpr uint32_t kPlaceBatch = 8;  // staged records per thread and step (loads issued together)

// Records rec[0, m) (LDS, position | exponent << 16) to escape indices
// [d0, d0 + m) of the stream.  Records whose index is a multiple of 4 start
// on a 4-byte boundary (the escape section is 256-aligned), so every 4
// records fill 3 whole words (1 with the sentinel variant) and are written
// with word stores; the records before the first such index and after the
// last group are written byte by byte.  Other workgroups may write the
// neighbouring bytes of the first and last words: stores carry byte masks.
template <int kVariant = kMain>
__device__ void write_records(const EncArgs& a, const uint32_t* rec, uint64_t d0, uint32_t m, uint32_t tid = threadIdx.x) {
  const uint32_t head = std::min<uint32_t>(m, (uint32_t)(-d0 & 3));
  const uint32_t groups = (m - head) / 4, tail = head + 4 * groups;
  if (tid < head) put_record<kVariant>(a, d0 + tid, rec[tid] & 0xFFFF, rec[tid] >> 16);
  if (tid < m - tail) put_record<kVariant>(a, d0 + tail + tid, rec[tail + tid] & 0xFFFF, rec[tail + tid] >> 16);
  for (uint32_t g = tid; g < groups; g += kThreads) {
    const uint32_t* r = rec + head + 4 * g;
    put_record_group<kVariant>(a, d0 + head + 4 * (uint64_t)g, r[0], r[1], r[2], r[3]);
  }
}

// Tile tt, whose n_i escapes take stream indices [dest, dest + n_i), encoded
// again without stores, its records written in element order through the
// LDS window rec (kPlaceRecs records) as whole words.  The exponent table is
// built for the tile's codebook unless table_cb already names it.
template <bool kBf16, int kVariant>
__device__ inline void reencode_records(const EncArgs& a, uint32_t* rec, EncShared& esh, uint64_t tt, uint32_t n_i,
                                        uint64_t dest, uint64_t& table_cb, uint32_t tid) {
  const uint64_t cbi = a.seg_chunks ? codebook_of_chunk(tt >> (kBf16 ? 3 : 2), a.seg_chunks) : 0;
  const TileIn in = kBf16 ? load_tile_bf16(a, tt, tid) : load_tile_e5m2(a, tt, tid);
  if (cbi != table_cb) {
    build_table<kVariant>(a, esh, cbi, kBf16 ? 256u : 32u, tid);
    table_cb = cbi;
  }
  const TileEsc r = kBf16 ? encode_tile_bf16<kVariant>(a, esh, tt, in, false, tid)
                          : encode_tile_e5m2(a, esh, tt, in, false, tid);
  if (kBf16) {
    // one window per group: a group of 2048 elements holds at most
    // kPlaceRecs records, and its records follow the lower groups'
#pragma unroll 1
    for (uint32_t g = 0, g_first = 0; g < 4; ++g) {
      const uint32_t cnt = ((g < 2 ? r.g01 : r.g23) >> (16 * (g & 1))) & 0xFFFFu;  // the same in every thread
      if (cnt) {
        group_escapes_bf16(tt, r, in, g, g_first, tid,
                           [&](uint32_t k, uint32_t pos, uint32_t val) { rec[k] = pos | (val << 16); });
        __syncthreads();
        write_records<kVariant>(a, rec, dest + g_first, cnt, tid);
        __syncthreads();  // rec is reused
      }
      g_first += cnt;
    }
  } else {
    for (uint32_t w0 = 0; w0 < n_i; w0 += kPlaceRecs) {  // one window per 2048 records
      auto stage = [&](uint32_t k, uint32_t pos, uint32_t val) {
        if (k - w0 < kPlaceRecs) rec[k - w0] = pos | (val << 16);
      };
      window_escapes_e5m2(tt, r, in, w0, kPlaceRecs, tid, stage);
      __syncthreads();
      write_records<kVariant>(a, rec, dest + w0, std::min<uint32_t>(kPlaceRecs, n_i - w0), tid);
      __syncthreads();  // rec and esh are reused
    }
  }
}

// LDS of place_range for ranges of up to kMax tiles.
template <uint32_t kMax>
struct PlaceLds {
  uint64_t red[16];
  uint32_t pre_all[kMax + 1];     // escapes before each tile of the range
  uint32_t pre_staged[kMax + 1];  // staged records before each tile of the range
  alignas(16) uint32_t rec[kPlaceRecs];  // re-encoded tile's records (position | exponent << 16) in escape order
};

// The tiles [t0, t0 + tiles) (tiles <= kMax <= 4 * kThreads), whose first
// escape has stream index `base`: the scan of
// their counts (kMax / kThreads consecutive tiles per thread, so the thread
// order is the tile order), their chunk offsets (E, S and the stream size
// when the last tile of the stream is among them), their staged records
// moved to their place, and the tiles whose escapes overflowed their slot
// encoded again.
template <bool kBf16, int kVariant, uint32_t kMax>
__device__ void place_range(const EncArgs& a, PlaceLds<kMax>& sh, EncShared& esh, uint64_t t0, uint32_t tiles,
                            uint64_t base) {
  constexpr uint64_t kRec = kVariant == kSentinel ? 1 : 3;  // stream bytes per escape
  constexpr uint32_t kPer = (kMax + kThreads - 1) / kThreads;  // tiles per thread
  constexpr uint32_t kSlot = stage_slot(kVariant);
  const uint32_t tid = threadIdx.x;
  uint32_t cnt[kPer], sum = 0, ssum = 0;
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k) {
    const uint32_t i = tid * kPer + k;
    cnt[k] = i < tiles ? a.tile_count[t0 + i] : 0u;
    sum += cnt[k];
    ssum += cnt[k] > kSlot ? 0u : cnt[k];
  }
  uint32_t total, staged_total;
  uint32_t pre = block_exclusive_sum<kThreads / 64>(sh.red, sum, &total);
  uint32_t spre = block_exclusive_sum<kThreads / 64>(sh.red, ssum, &staged_total);
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k) {
    const uint32_t i = tid * kPer + k;
    if (i <= kMax) {
      sh.pre_all[i] = pre;
      sh.pre_staged[i] = spre;
    }
    pre += cnt[k];
    spre += cnt[k] > kSlot ? 0u : cnt[k];
  }
  if (tid == 0 && kPer * kThreads <= kMax) {  // entry kMax, past every thread's tiles
    sh.pre_all[kMax] = total;
    sh.pre_staged[kMax] = staged_total;
  }
  const bool any_over = staged_total != total;  // uniform
  __syncthreads();
  constexpr uint32_t kTpcLog2 = kBf16 ? 3 : 2;  // tiles per chunk: 8 BF16, 4 E5M2
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k) {
    const uint32_t i = tid * kPer + k;
    if (i >= tiles) continue;
    const uint64_t t = t0 + i;
    if ((t & ((1u << kTpcLog2) - 1)) == 0) put_le(a.out + a.offsets + 8 * (t >> kTpcLog2), base + sh.pre_all[i], 8);
    if (t == a.n_tiles - 1) {
      const uint64_t e = std::min<uint64_t>(base + sh.pre_all[i] + cnt[k], a.n);
      const uint64_t s = a.esc + kRec * e;
      put_le(a.out + a.offsets + 8 * a.chunks, e, 8);
      put_le(a.out + 16, e, 8);
      put_le(a.out + 24, s, 8);
      if (a.out_bytes) *a.out_bytes = s;
    }
  }

  // staged records of the range, flattened: record j belongs to the tile i
  // with pre_staged[i] <= j < pre_staged[i + 1]
  auto tile_of = [&](uint32_t j) {
    uint32_t lo = 0, hi = tiles;  // last i with pre_staged[i] <= j
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (sh.pre_staged[mid] <= j) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  if (!any_over) {  // uniform
    // the records fill escape indices [base, base + total): a thread takes
    // 4 of them from an index that is a multiple of 4, which fill whole
    // words (3, or 1 with the sentinel variant); the few records before the
    // first and after the last such group are written byte by byte
    const uint32_t head = std::min<uint32_t>(total, (uint32_t)(-base & 3));
    const uint32_t groups = (total - head) / 4, tail0 = head + 4 * groups;
    const uint32_t j_odd = tid < head ? tid : tail0 + (tid - head);  // head then tail records, one per thread
    if (j_odd < total && (tid < head || tid - head < total - tail0)) {
      const uint32_t i = tile_of(j_odd);
      const uint32_t v = a.stage[(t0 + i) * kSlot + (j_odd - sh.pre_staged[i])];
      put_record<kVariant>(a, base + j_odd, v & 0xFFFF, v >> 16);
    }
    for (uint32_t g = tid; g < groups; g += kThreads) {
      const uint32_t j = head + 4 * g;
      uint32_t i = tile_of(j);
      uint32_t v[4];
#pragma unroll
      for (uint32_t k = 0; k < 4; ++k) {
        if (i + 1 < tiles && sh.pre_staged[i + 1] <= j + k) i = tile_of(j + k);  // record j + k is in a later tile
        v[k] = a.stage[(t0 + i) * kSlot + (j + k - sh.pre_staged[i])];
      }
      put_record_group<kVariant>(a, base + j, v[0], v[1], v[2], v[3]);
    }
    return;
  }
  for (uint32_t j0 = 0; j0 < staged_total; j0 += kThreads * kPlaceBatch) {
    uint32_t v[kPlaceBatch];
    uint64_t dst[kPlaceBatch];
#pragma unroll
    for (uint32_t u = 0; u < kPlaceBatch; ++u) {
      const uint32_t j = j0 + u * kThreads + tid;
      dst[u] = ~0ull;
      if (j < staged_total) {
        const uint32_t lo = tile_of(j);
        const uint32_t r = j - sh.pre_staged[lo];
        v[u] = a.stage[(t0 + lo) * kSlot + r];
        dst[u] = base + sh.pre_all[lo] + r;
      }
    }
#pragma unroll
    for (uint32_t u = 0; u < kPlaceBatch; ++u)
      if (dst[u] != ~0ull) put_record<kVariant>(a, dst[u], v[u] & 0xFFFF, v[u] >> 16);
  }

  // tiles whose escapes overflowed their slot: encoded again, records in
  // element order through LDS windows to word stores.  The thread index is
  // passed through an empty asm statement in each iteration, so the compiler
  // cannot hoist the per-thread address arithmetic of the loop body out of
  // the loop (holding it live across iterations costs the kernel about 40
  // registers, which the common path pays in occupancy).
  uint64_t table_cb = ~0ull;
  for (uint32_t i = 0; i < tiles; ++i) {
    const uint32_t n_i = sh.pre_all[i + 1] - sh.pre_all[i];
    if (n_i <= kSlot) continue;  // uniform
    uint32_t tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    reencode_records<kBf16, kVariant>(a, sh.rec, esh, t0 + i, n_i, base + sh.pre_all[i], table_cb, tid_i);
  }
}

// One workgroup per range of place_tiles tiles (a power of two up to
// kBlockTiles, so a range lies inside one block): the range's base (escapes
// of the lower super-blocks, of the lower blocks of its super-block and of
// the lower tiles of its block), then place_range.
template <bool kBf16, int kVariant = kMain>
__device__ void encode_place(const EncArgs& a) {
  __shared__ PlaceLds<kBlockTiles> sh;
  __shared__ EncShared esh;
  if (a.prep_in == 2 && blockIdx.x == gridDim.x - 1) {  // the launch's extra workgroup
    prep_work(a.prep, 0, 1);
    return;
  }
  const uint32_t tid = threadIdx.x;
  const uint64_t t0 = (uint64_t)blockIdx.x * a.place_tiles;
  const uint32_t tiles = (uint32_t)std::min<uint64_t>(a.place_tiles, a.n_tiles - t0);
  const uint64_t blk = t0 / kBlockTiles;
  const uint32_t below = (uint32_t)(t0 % kBlockTiles);  // tiles of the block before the range

  // base: the first wave adds the lower blocks of the super-block, the
  // second the lower tiles of the block, all waves the lower super-blocks;
  // with at most 64 blocks (no block sums) all waves add the lower tiles
  uint64_t lower = 0;
  if (a.sums_in_place) {
    for (uint32_t i = tid; i < (uint32_t)t0; i += kThreads) lower += a.tile_count[i];
  } else {
    for (uint64_t i = tid; i < (blk >> 6); i += kThreads) lower += a.super_sum[i];
    if (tid < (blk & 63)) lower += a.block_sum[(blk & ~63ull) + tid];
    if (tid >= 64 && tid - 64 < below) lower += a.tile_count[blk * kBlockTiles + (tid - 64)];
  }
  {
    // wave sum of u64 through two u32 halves; one lane per wave stores it
    uint64_t v = lower;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
      v += ((uint64_t)hi << 32) | lo;
    }
    if ((tid & 63) == 0) sh.red[8 + (tid >> 6)] = v;
  }
  __syncthreads();
  const uint64_t base = sh.red[8] + sh.red[9] + sh.red[10] + sh.red[11];
  place_range<kBf16, kVariant, kBlockTiles>(a, sh, esh, t0, tiles, base);
}

__global__ __launch_bounds__(kThreads) void encode_place_bf16_kernel(EncArgs a) { encode_place<true>(a); }
__global__ __launch_bounds__(kThreads) void encode_place_e5m2_kernel(EncArgs a) { encode_place<false>(a); }
__global__ __launch_bounds__(kThreads) void encode_place_sentinel_kernel(EncArgs a) { encode_place<true, kSentinel>(a); }
__global__ __launch_bounds__(kThreads) void encode_place_top8_kernel(EncArgs a) { encode_place<true, kTop8>(a); }

// ------------------------------------------------- static-scratch workspace
//
// splitzip_compress_static runs the same launches as splitzip_compress, with
// the encoder's workspace (tile counts and staging slots; inputs of at most
// kStaticMaxTiles tiles need no block sums) in the library's own device
// array instead of the tail of the caller's buffer.  Every word a call reads
// there it wrote first (counts of all its tiles, the slots of the tiles it
// staged), so nothing needs clearing between calls; calls that overlap on
// one GPU share the array, so they race.
constexpr uint32_t kStaticMaxTiles = 2048;  // 16M BF16 or 32M E5M2 elements (32 MiB)
constexpr uint32_t kStaticStageAt = kStaticMaxTiles;  // words: tile counts, then staging slots
constexpr uint32_t kSingleMaxTiles = 512;   // one launch up to 4M BF16 or 8M E5M2 elements (8 MiB)
constexpr uint64_t kSingleAt = kStaticStageAt + (uint64_t)kStaticMaxTiles * stage_slot(kMain);
constexpr uint32_t kSingleCounts = 64;      // encode_single's words: the arrival counter, then (a cache line on) the count words
constexpr uint64_t kStaticWords = kSingleAt + kSingleCounts + kSingleMaxTiles;

static_assert(kStaticMaxTiles <= 64 * kBlockTiles, "inputs within the limit take the path without block sums");

// The encoder workspace of splitzip_compress_static, one copy per GPU (about
// 4 MiB).  Host code reaches it only through the address hipGetSymbolAddress
// returns with that GPU current.
static __device__ __align__(256) uint32_t scratch[kStaticWords];

// ------------------------------------------------- one-launch static encode
//
// Inputs of at most kSingleMaxTiles tiles take one launch in
// splitzip_compress_static: each workgroup encodes its tile, publishes the
// tile's escape count in the static array, adds up the counts of the lower
// tiles and writes its own records at their place.  No escape record crosses
// workgroups, only the count words, which are written and read with relaxed
// device-scope atomics (coherent across the XCDs' L2 caches).  A count word
// is valid | epoch << 16 | count.  The epoch is what a call-wide counter A
// (static array) held when the workgroup started; every workgroup adds 1 to A
// after publishing.  Calls on one stream run one after another, so every
// workgroup of a call reads A at or above the value the previous call's
// last workgroup left, which exceeds every epoch that call used (by less
// than 2^15, the epoch's width): a word left by the previous call never
// passes for this one.  A call also zeroes the count words of the tiles it
// does not have, so no word outlives the call after the one that wrote it.
// Nothing decides a "last" workgroup, so overlapping calls (which race, as
// documented) leave no state that could mislead later calls.
// A workgroup polls for a lower tile's count at most wait_polls times; a
// count still missing then (its workgroup has not run yet, or started after
// others of the call had finished and so read another epoch) is computed
// from that tile's input, encoded again without stores.  No result depends
// on the order the workgroups run in, and no wave waits without bound.
constexpr uint32_t kCountValid = 1u << 31, kEpochShift = 16, kEpochMask = 0x7FFFu, kCountMask = 0xFFFFu;

__device__ inline uint32_t load_agent(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct SingleLds {
  alignas(16) uint32_t rec[kPlaceRecs];       // the tile's records (position | exponent << 16) in element order
  uint32_t missing[kSingleMaxTiles / 32];     // lower tiles whose count did not arrive in time
  uint32_t epoch;
};

template <bool kBf16>
__device__ void encode_single(const EncArgs& a) {
  __shared__ EncShared sh;
  __shared__ DenseLds<kBf16> dl;
  __shared__ SingleLds ss;
  const uint64_t n_tiles = a.n_tiles;
  if (blockIdx.x == n_tiles) {  // the launch's extra workgroup: header, codebooks, padding
    prep_work(a.prep, 0, 1);
    return;
  }
  constexpr uint32_t kTpcLog2 = kBf16 ? 3 : 2;  // tiles per chunk: 8 BF16, 4 E5M2
  constexpr uint32_t kPer = kSingleMaxTiles / kThreads;
  const uint32_t tid = threadIdx.x;
  const uint64_t t = blockIdx.x;
  uint32_t* arrivals = a.single;  // A: workgroups that published, over all calls
  uint32_t* counts = a.single + kSingleCounts;
  if (tid == 0) ss.epoch = load_agent(arrivals) & kEpochMask;
  if (tid < kSingleMaxTiles / 32) ss.missing[tid] = 0;
  const TileIn in = kBf16 ? load_tile_bf16(a, t) : load_tile_e5m2(a, t);
  build_table<kMain>(a, sh, a.seg_chunks ? codebook_of_chunk(t >> kTpcLog2, a.seg_chunks) : 0, kBf16 ? 256u : 32u);
  uint4* escw = reinterpret_cast<uint4*>(dl.exps);
  const TileEsc r = kBf16 ? encode_tile_bf16<kMain>(a, sh, t, in, true, tid, dl.exps)
                          : encode_tile_e5m2(a, sh, t, in, true, tid, escw);
  // publish (ss.epoch is visible: the table build and the rank scan hold barriers)
  const uint32_t tag = kCountValid | (ss.epoch << kEpochShift);
  if (tid == 0) {
    store_agent(counts + t, tag | r.agg);
    __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const bool staged = r.agg <= kPlaceRecs;  // uniform
  if (staged) {
    auto stage = [&](uint32_t k, uint32_t pos, uint32_t val) { ss.rec[k] = pos | (val << 16); };
    if (kBf16) dense_escapes_bf16(t, r, dl.exps, stage);
    else dense_escapes_e5m2(a, t, r, escw, stage);
  }

  // counts of the lower tiles: thread i awaits tiles i, i + 256, ...
  uint32_t lower = 0, want = 0;
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k)
    if (tid + k * kThreads < t) want |= 1u << k;
  for (uint32_t p = 0;; ++p) {
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
      if (!((want >> k) & 1u)) continue;
      const uint32_t w = load_agent(counts + tid + k * kThreads);
      if ((w & ~kCountMask) == tag) {
        lower += w & kCountMask;
        want &= ~(1u << k);
      }
    }
    if (!__syncthreads_or(want != 0) || p >= a.wait_polls) break;  // uniform
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k) {
    const uint32_t j = tid + k * kThreads;
    if ((want >> k) & 1u) atomicOr(&ss.missing[j >> 5], 1u << (j & 31));
  }
  if (__syncthreads_or(want != 0)) {  // uniform: counts that never arrived, from the tiles' input
    uint64_t table_cb = ~0ull;
    for (uint32_t j = 0; j < (uint32_t)t; ++j) {
      if (!((ss.missing[j >> 5] >> (j & 31)) & 1u)) continue;  // uniform
      const uint64_t cbi = a.seg_chunks ? codebook_of_chunk(j >> kTpcLog2, a.seg_chunks) : 0;
      const TileIn inj = kBf16 ? load_tile_bf16(a, j) : load_tile_e5m2(a, j);
      if (cbi != table_cb) {
        build_table<kMain>(a, sh, cbi, kBf16 ? 256u : 32u);
        table_cb = cbi;
      }
      const TileEsc rj = kBf16 ? encode_tile_bf16<kMain>(a, sh, j, inj, false) : encode_tile_e5m2(a, sh, j, inj, false);
      if (tid == 0) lower += rj.agg;
    }
  }
  uint32_t base32 = 0;
  block_exclusive_sum<kThreads / 64>(sh.red, lower, &base32);  // the total over the workgroup
  const uint64_t base = base32;

  if (tid == 0) {
    if ((t & ((1u << kTpcLog2) - 1)) == 0) put_le(a.out + a.offsets + 8 * (t >> kTpcLog2), base, 8);
    if (t == n_tiles - 1) {
      const uint64_t e = base + r.agg, sz = a.esc + 3 * e;
      put_le(a.out + a.offsets + 8 * a.chunks, e, 8);
      put_le(a.out + 16, e, 8);
      put_le(a.out + 24, sz, 8);
      if (a.out_bytes) *a.out_bytes = sz;
    }
  }
  if (staged) {
    write_records<kMain>(a, ss.rec, base, r.agg);  // ss.rec is complete: the sums above hold barriers
  } else {
    uint64_t table_cb = ~0ull;  // the table may hold a lower tile's codebook
    reencode_records<kBf16, kMain>(a, ss.rec, sh, t, r.agg, base, table_cb, tid);
  }
  // count words past this call's tiles, for the calls that follow
  for (uint64_t j = n_tiles + t * kThreads + tid; j < kSingleMaxTiles; j += n_tiles * kThreads) store_agent(counts + j, 0);
}

__global__ __launch_bounds__(kThreads) void encode_single_bf16_kernel(EncArgs a) { encode_single<true>(a); }
__global__ __launch_bounds__(kThreads) void encode_single_e5m2_kernel(EncArgs a) { encode_single<false>(a); }

// ---------------------------------------------------------- decode kernels
struct DecArgs {
  const uint8_t* in;
  uint64_t in_bytes;
  uint8_t* out;
  uint64_t n;
  int32_t* status;
  int dtype;
  int variant;  // header byte 48
};

struct Header {
  uint64_t k, seg, e, chunks;
  Sections s;
};

__device__ inline uint64_t ld64(const uint8_t* p) { return *reinterpret_cast<const uint64_t*>(p); }
__device__ inline uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
// A load through the vector memory path even where the address is the same
// in every lane: the zero offset is opaque to the compiler, which therefore
// cannot turn the load into a scalar-cache load.  Used for the chunk offsets
// that every decoder waits on first; as scalar loads their latency (and the
// lgkmcnt waits they share with the LDS traffic of escape staging) cost the
// top-8 decoder 19% and the BF16 decoder 3%.
__device__ inline uint64_t vld64(const uint8_t* p) {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return *reinterpret_cast<const uint64_t*>(p + z);
}

// Header checks shared by every workgroup (all reads inside the first 64
// bytes; in_bytes >= 64 is checked on the host).
__device__ bool read_header(const DecArgs& a, Header& h) {
  const uint8_t* in = a.in;
  const uint32_t w0 = ld32(in), w1 = ld32(in + 4);
  if (w0 != kMagic) return false;
  if ((w1 & 0xFFFF) != 1 || ((w1 >> 16) & 0xFF) != (uint32_t)a.dtype || (w1 >> 24) != 16) return false;
  if (ld64(in + 8) != a.n) return false;
  if (ld64(in + 48) != (uint64_t)a.variant || ld64(in + 56) != 0) return false;  // variant byte, then zeros
  h.e = ld64(in + 16);
  const uint64_t total = ld64(in + 24);
  h.chunks = ld32(in + 32);
  h.k = ld32(in + 36);
  h.seg = ld64(in + 40);
  if (h.chunks != divup(a.n, kChunk)) return false;
  if (h.k == 0 || h.k > kMaxK) return false;
  if (h.k == 1) {
    if (h.seg != a.n) return false;
  } else if (h.seg == 0 || (h.seg % kChunk) != 0 || (h.seg < a.n && h.seg * h.k < a.n)) {  // seg >= ceil(n / k); k < 2^16
    return false;
  }
  if (h.e > a.n) return false;
  h.s = sections_of(a.dtype, a.n, h.k, a.variant);
  if (total != h.s.esc + h.s.rec * h.e || total > a.in_bytes) return false;
  return true;
}

__device__ inline void report_corrupt(int32_t* status) {
  if (status) __hip_atomic_store(status, (int32_t)SPLITZIP_E_CORRUPT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether v equals the value of another lane of its 16-lane row: the 15
// row rotations (DPP row_ror 1..15) of v, compared with v.
template <int kRot = 1>
__device__ inline bool row_has_duplicate(uint32_t v) {
  if constexpr (kRot == 16) {
    return false;
  } else {
    const bool same = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + kRot, 0xf, 0xf, false) == v;
    return same | row_has_duplicate<kRot + 1>(v);
  }
}

// Every codebook of the stream must hold 16 distinct entries, each below
// vmax (32 for E5M2; any byte for BF16), as a stream the encoder writes
// does.  The K codebooks are spread over the launch's workgroups, four per
// pass of one full wave: lane l holds entry l & 15 of codebook 4q + (l >> 4)
// and compares it with the 15 other entries of its 16-lane row through DPP
// row rotations.  Reports a bad stream through the status word.
__device__ inline void check_codebooks(const DecArgs& a, uint64_t k, uint32_t vmax) {
  const uint32_t lane = __lane_id();
  bool bad = false;
  const uint32_t quads = (uint32_t)(k + 3) / 4;  // k <= 65535 (header check)
  for (uint32_t q = blockIdx.x; q < quads; q += gridDim.x) {  // same in the wave
    const uint32_t cb = 4 * q + (lane >> 4);
    const bool live = cb < k;  // same in each 16-lane row
    const uint32_t v = live ? a.in[64 + 16 * cb + (lane & 15)] : 0u;
    bad |= live && (row_has_duplicate(v) || v >= vmax);
  }
  if (__ballot(bad) != 0 && lane == 0) report_corrupt(a.status);
}

__device__ inline uint32_t record_pos(const uint8_t* rec) { return rec[0] | ((uint32_t)rec[1] << 8); }

// Smallest index i in [lo, hi] with i == hi or position(i) >= key (positions
// ascend in a valid stream; a corrupt order is caught by the caller).  Run by
// one full wave as a 64-way search: each round probes 64 evenly spaced
// records at once and keeps the bucket holding the first hit, so a range of
// L records takes ceil(log64(L + 1)) dependent loads instead of log2(L).
// Ranges of 1024 records or more start with a round around the index that
// key / key_span interpolates (key_span: the chunk's length): escapes spread
// evenly put the answer within that round's 64 probes, leaving one more
// round (256 MiB of uniform bits: 191 -> 183 us; top-8 ablation 359 -> 334 us).
__device__ uint64_t wave_lower_bound(const uint8_t* esc, uint64_t lo, uint64_t hi, uint32_t key, uint32_t key_span) {
  const uint64_t lane = __lane_id();
  constexpr uint64_t kGap = 16;  // records between the interpolation round's probes
  if (hi - lo >= 64 * kGap) {
    // first round around the interpolated index (positions spread evenly put
    // the answer near it): 64 probes kGap apart, strictly increasing inside
    // [lo, hi); the first hit brackets the answer as in the rounds below
    const uint64_t g = lo + (hi - lo) * std::min<uint32_t>(key, key_span) / key_span;
    const uint64_t start = std::min<uint64_t>(std::max<uint64_t>(g >= 32 * kGap ? g - 32 * kGap : 0, lo), hi - 1 - 63 * kGap);
    const uint64_t q = start + lane * kGap;
    const bool hit = record_pos(esc + 3 * q) >= key;
    const uint64_t bal = __ballot(hit);
    const uint32_t i = bal ? (uint32_t)__builtin_ctzll(bal) : 64u;  // probe start + i kGap is the first hit
    if (i < 64) hi = start + (uint64_t)i * kGap;
    if (i > 0) lo = start + (uint64_t)(i - 1) * kGap + 1;
  }
  while (hi - lo > 63) {
    const uint64_t step = (hi - lo + 63) / 64;  // 64 * step >= hi - lo: probe 64 hits hi
    const uint64_t p = lo + (lane + 1) * step;
    const bool hit = p >= hi || record_pos(esc + 3 * p) >= key;
    const uint32_t i = (uint32_t)__builtin_ctzll(__ballot(hit));  // probe lo + (i + 1) step is the first hit
    const uint64_t new_hi = std::min<uint64_t>(lo + (uint64_t)(i + 1) * step, hi);
    lo = i == 0 ? lo : lo + (uint64_t)i * step + 1;                 // probe lo + i step missed
    hi = new_hi;
  }
  const uint64_t p = lo + lane;  // hi - lo <= 63: lane hi - lo sees p == hi
  const bool hit = p >= hi || record_pos(esc + 3 * p) >= key;
  return lo + (uint64_t)__builtin_ctzll(__ballot(hit));
}

// Four records of the escape section: records 4q .. 4q+3 fill its words
// 3q .. 3q+2 exactly (the section is 256-aligned), and bytes 1 and 2 of word
// 3q-1 hold the position of record 4q-1.  One group is read with word
// loads and unpacked with fixed shifts, the inverse of the encoder's packing.
struct RecGroup {
  uint32_t pos[4], val[4];
  uint32_t prev_pos;  // position of record 4q-1 (0 for q == 0)
};

struct RecWords {  // words 3q-1 .. 3q+2 as loaded (w0 = 0 for q == 0)
  uint32_t w0, w1, w2, w3;
};

__device__ inline RecWords load_rec_words(const DecArgs& a, uint64_t esc, uint64_t q) {
  const uint64_t b = esc + 12 * q;
  uint32_t w0 = 0, w1, w2, w3;
  if (b + 12 <= a.in_bytes) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(a.in + b);
    if (q > 0) w0 = p[-1];
    w1 = p[0];
    w2 = p[1];
    w3 = p[2];
  } else {  // the stream's last bytes: nothing past in_bytes is read
    uint32_t w[3] = {0, 0, 0};
    for (uint32_t i = 0; i < 12 && b + i < a.in_bytes; ++i) w[i >> 2] |= (uint32_t)a.in[b + i] << (8 * (i & 3));
    if (q > 0) w0 = *reinterpret_cast<const uint32_t*>(a.in + b - 4);
    w1 = w[0];
    w2 = w[1];
    w3 = w[2];
  }
  return RecWords{w0, w1, w2, w3};
}

__device__ inline RecGroup unpack_rec_group(const RecWords& w) {
  const uint32_t w0 = w.w0, w1 = w.w1, w2 = w.w2, w3 = w.w3;
  RecGroup g;
  g.pos[0] = w1 & 0xFFFFu;
  g.val[0] = (w1 >> 16) & 0xFFu;
  g.pos[1] = (w1 >> 24) | ((w2 & 0xFFu) << 8);
  g.val[1] = (w2 >> 8) & 0xFFu;
  g.pos[2] = w2 >> 16;
  g.val[2] = w3 & 0xFFu;
  g.pos[3] = (w3 >> 8) & 0xFFFFu;
  g.val[3] = w3 >> 24;
  g.prev_pos = (w0 >> 8) & 0xFFFFu;
  return g;
}

__device__ inline RecGroup load_rec_group(const DecArgs& a, uint64_t esc, uint64_t q) {
  return unpack_rec_group(load_rec_words(a, esc, q));
}

constexpr uint32_t kScanGroups = 1;   // record groups per thread and step of a long chunk (more cost occupancy)
constexpr uint32_t kShortGroups = 2;  // record groups per thread of a short chunk

// The tile's chunk's record range and, for a short chunk (at most
// kShortGroups * kThreads record groups, 2048 records), this thread's
// groups: loaded before the tile's dense loads are issued, so that waiting
// for the records does not mean waiting for the dense data queued behind
// them (loads complete in issue order).  The words are kept as loaded and
// unpacked by stage_escapes, after the dense loads have been issued.
struct EscFetch {
  uint64_t lo, hi;           // the chunk's records (offsets table)
  RecWords W[kShortGroups];  // groups lo / 4 + k * kThreads + thread index, short chunk only
};

template <uint32_t kDecTile>
__device__ inline EscFetch fetch_escapes(const DecArgs& a, const Header& h, uint64_t tile) {
  EscFetch f;
  const uint64_t chunk = tile / (kChunk / kDecTile);
  const uint8_t* offs = a.in + h.s.offsets;
  f.lo = vld64(offs + 8 * chunk);
  f.hi = vld64(offs + 8 * (chunk + 1));
  const uint64_t g_lo = f.lo / 4, g_hi = (f.hi + 3) / 4;
  const uint64_t g = g_lo + threadIdx.x;
  // an inconsistent range is rejected by stage_escapes; nothing is read for it
  if (f.lo <= f.hi && f.hi <= h.e && g_hi - g_lo <= kShortGroups * kThreads) {
#pragma unroll
    for (uint32_t k = 0; k < kShortGroups; ++k)
      if (g + k * kThreads < g_hi) f.W[k] = load_rec_words(a, h.s.esc, g + k * kThreads);
  }
  return f;
}

// Stage this tile's escapes in LDS: a bitmap over the tile's elements and
// the raw exponents.  Every record of the chunk is checked by exactly one of
// the chunk's tiles (in window, strictly increasing, valid value).  Returns
// false (the same in every thread) if the stream is invalid.
template <uint32_t kDecTile>
__device__ bool stage_escapes(const DecArgs& a, const Header& h, uint64_t tile, const EscFetch& f, uint32_t* bitmap,
                              uint8_t* vals, uint32_t* s_range, int* s_err) {
  const uint32_t tid = threadIdx.x;
  const uint64_t chunk = tile / (kChunk / kDecTile);
  const uint32_t q = (uint32_t)(tile % (kChunk / kDecTile));
  const uint64_t chunk_len = std::min<uint64_t>(kChunk, a.n - chunk * kChunk);
  const uint32_t win_lo = q * (uint32_t)kDecTile;
  const uint32_t win_len = (uint32_t)std::min<uint64_t>(kDecTile, chunk_len - win_lo);
  const bool last_in_chunk = win_lo + win_len == chunk_len;
  const uint64_t lo = f.lo, hi = f.hi;
  // at most one record per element of the chunk (this also bounds the
  // record ranges kept as 32-bit counts below)
  bool ok = lo <= hi && hi <= h.e && hi - lo <= chunk_len;
  if (chunk == 0 && lo != 0) ok = false;
  if (chunk == h.chunks - 1 && hi != h.e) ok = false;
  if (!ok) return false;  // uniform: every thread read the same words
  const uint32_t vmax = a.dtype == SPLITZIP_BF16 ? 256u : 32u;

  // records [ra, rb) of group g: each must lie in [p_lo, p_lo + p_len) and
  // follow its predecessor in the range; in-window ones are staged
  auto check_group = [&](uint64_t g, uint64_t ra, uint64_t rb, uint32_t p_lo, uint32_t p_len, const RecGroup& G,
                         bool& bad) {
    const uint64_t r0 = 4 * g;  // record j of the group is r0 + j
    const uint32_t j_lo = ra > r0 ? (uint32_t)(ra - r0) : 0u;  // < 4 for a group that meets the range
    const uint32_t j_hi = (uint32_t)std::min<uint64_t>(4, rb - r0);
    const bool first = ra >= r0;  // the range's first record is in this group (at j_lo)
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
      if (j < j_lo || j >= j_hi) continue;
      const uint32_t pos = G.pos[j], val = G.val[j];
      const uint32_t prev1 = (first && j == j_lo) ? 0u : (j == 0 ? G.prev_pos : G.pos[j > 0 ? j - 1 : 0]) + 1;
      if (pos - p_lo >= p_len || val >= vmax || prev1 > pos) {  // pos - p_lo wraps for pos < p_lo
        bad = true;
        continue;
      }
      const uint32_t local = pos - win_lo;  // wraps for pos < win_lo
      if (local < win_len) {
        vals[local] = (uint8_t)val;
        atomicOr(&bitmap[local >> 5], 1u << (local & 31));
      }
    }
  };

  const uint64_t g_lo = lo / 4, g_hi = (hi + 3) / 4;  // record groups of the chunk
  if (g_hi - g_lo <= kShortGroups * kThreads) {  // uniform
    // short chunk (up to 2048 records): every tile of the chunk has loaded
    // all of its records, two groups per thread (no search, whose dependent
    // loads would lengthen the tile's critical path); it checks all of them
    // and stages those in its window
    const uint64_t g = g_lo + tid;
    for (uint32_t i = tid; i < kDecTile / 32; i += kThreads) bitmap[i] = 0;
    if (tid == 0) *s_err = 0;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (uint32_t k = 0; k < kShortGroups; ++k)
      if (g + k * kThreads < g_hi)
        check_group(g + k * kThreads, lo, hi, 0, (uint32_t)chunk_len, unpack_rec_group(f.W[k]), bad);
    if (bad) *s_err = 1;
    __syncthreads();
    return *s_err == 0;
  }

  for (uint32_t i = tid; i < kDecTile / 32; i += kThreads) bitmap[i] = 0;
  if (tid == 0) *s_err = 0;
  // long chunk: wave 0 finds the tile's first record, wave 1 its end
  if (tid < 64) {
    const uint64_t r = q == 0 ? lo : wave_lower_bound(a.in + h.s.esc, lo, hi, win_lo, (uint32_t)chunk_len);
    if (tid == 0) s_range[0] = (uint32_t)(r - lo);
  } else if (tid < 128) {
    const uint64_t r = last_in_chunk ? hi : wave_lower_bound(a.in + h.s.esc, lo, hi, win_lo + win_len, (uint32_t)chunk_len);
    if (tid == 64) s_range[1] = (uint32_t)(r - lo);
  }
  __syncthreads();
  const uint64_t ra = lo + s_range[0], rb = lo + s_range[1];
  bool bad = false;
  // the tile's records, a group per thread per step
  for (uint64_t g0 = ra / 4; g0 < (rb + 3) / 4; g0 += (uint64_t)kScanGroups * kThreads) {
    RecGroup G[kScanGroups];
#pragma unroll
    for (uint32_t k = 0; k < kScanGroups; ++k) {
      const uint64_t g = g0 + k * kThreads + tid;
      if (g < (rb + 3) / 4) G[k] = load_rec_group(a, h.s.esc, g);
    }
#pragma unroll
    for (uint32_t k = 0; k < kScanGroups; ++k) {
      const uint64_t g = g0 + k * kThreads + tid;
      if (g < (rb + 3) / 4) check_group(g, ra, rb, win_lo, win_len, G[k], bad);
    }
  }
  if (bad) *s_err = 1;
  __syncthreads();
  return *s_err == 0;
}

// BF16 decode of 8 elements: the 8 codes (4 nibble bytes) through the
// code-pair table (entry = exponent of the low code << 7 | exponent of the
// high code << 23, i.e. the exponent fields of two output values) and the 8
// sign|mantissa bytes: mantissa bits to bits 0..6 and the sign to bit 15 of
// each value, by one byte permutation of the masked bytes.
__device__ inline uint4 bf16_decode8(const uint32_t* tab2, uint32_t nib, uint2 sm) {
  const uint32_t m0 = sm.x & 0x7F7F7F7Fu, s0 = sm.x & 0x80808080u;
  const uint32_t m1 = sm.y & 0x7F7F7F7Fu, s1 = sm.y & 0x80808080u;
  return make_uint4(perm(s0, m0, 0x05010400u) | tab2[nib & 0xFFu], perm(s0, m0, 0x07030602u) | tab2[(nib >> 8) & 0xFFu],
                    perm(s1, m1, 0x05010400u) | tab2[(nib >> 16) & 0xFFu], perm(s1, m1, 0x07030602u) | tab2[nib >> 24]);
}

// Raw exponents of escaped elements replace the looked-up ones in the value
// pair w (elements 2k, 2k+1): esc2 holds their flags, v2 their staged bytes
// in bytes 0 and 1.
__device__ inline uint32_t bf16_patch2(uint32_t w, uint32_t esc2, uint32_t v2) {
  const uint32_t m = ((esc2 & 1u) ? 0x00007F80u : 0u) | ((esc2 & 2u) ? 0x7F800000u : 0u);
  const uint32_t e = perm(0u, v2, 0x0C010C00u) << 7;  // byte 0 -> bits 7..14, byte 1 -> bits 23..30
  return (w & ~m) | (e & m);
}

__device__ inline void bf16_patch8(uint4& o, uint32_t esc8, uint2 v) {
  o.x = bf16_patch2(o.x, esc8 & 3u, v.x);
  o.y = bf16_patch2(o.y, (esc8 >> 2) & 3u, v.x >> 16);
  o.z = bf16_patch2(o.z, (esc8 >> 4) & 3u, v.y);
  o.w = bf16_patch2(o.w, (esc8 >> 6) & 3u, v.y >> 16);
}

// BF16 decode tile: 8192 elements = 4 groups of 2048; thread t owns elements
// 8t..8t+7 of each group (4 nibble bytes, 8 sign|mantissa bytes, 16 output
// bytes; lane-contiguous across a wave).  A whole tile takes the fast path
// (no bounds checks); the last, partial tile goes element by element.
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecArgs a) {
  constexpr uint32_t kDecTile = kDecTileBf16, kGroups = kDecTile / 2048;
  __shared__ uint32_t bitmap[kDecTile / 32];
  __shared__ alignas(16) uint8_t vals[kDecTile];
  __shared__ uint32_t tab2[256];
  __shared__ uint32_t s_range[2];
  __shared__ int s_err;
  Header h;
  if (!read_header(a, h)) {
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  if (a.n == 0) {  // header-only stream: off[0] must be 0
    if (threadIdx.x == 0 && ld64(a.in + h.s.offsets) != 0) report_corrupt(a.status);
    if (threadIdx.x < 64) check_codebooks(a, h.k, a.dtype == SPLITZIP_BF16 ? 256u : 32u);
    return;
  }
  const uint64_t tile = blockIdx.x;
  const uint64_t chunk = tile / (kChunk / kDecTile);
  const uint64_t cbi = h.k == 1 ? 0 : codebook_of_chunk(chunk, h.seg / kChunk);
  const uint8_t* cb = a.in + 64 + 16 * cbi;
  const uint32_t tid = threadIdx.x;
  const uint64_t first = tile * kDecTile;
  const bool fast = first + kDecTile <= a.n;  // same in every thread
  const uint8_t* nib_t = a.in + h.s.nib + first / 2;
  const uint8_t* sm_t = a.in + h.s.sm + first;
  const EscFetch fe = fetch_escapes<kDecTile>(a, h, tile);
  // then the tile's dense loads: the escape staging overlaps them
  uint32_t nibs[kGroups];
  uint2 sms[kGroups];
  if (fast) {
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      // read once: non-temporal.  Plain loads allocate in the memory-side
      // cache; after a write-heavy kernel that cache holds dirty lines, and
      // the decode then paid for writing them back (1 GiB: 300 -> 369 us
      // after a 512 MiB fill; 302 us with these loads).
      nibs[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(nib_t + g * 1024 + 4 * tid));
      const u32x2_t s2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(sm_t + g * 2048 + 8 * tid));
      sms[g] = make_uint2(s2.x, s2.y);
    }
  }
  {  // code-pair table entry tid: codes tid & 15 (even element) and tid >> 4
    const uint32_t l0 = ld32(cb), l1 = ld32(cb + 4), l2 = ld32(cb + 8), l3 = ld32(cb + 12);
    const uint32_t c = tid & 0xFFu;
    const uint32_t pair = lut4((c & 0xFu) | ((c >> 4) << 8), l0, l1, l2, l3);  // bytes 0, 1: the two exponents
    tab2[c] = ((pair & 0xFFu) << 7) | (((pair >> 8) & 0xFFu) << 23);
  }
  if (!stage_escapes<kDecTile>(a, h, tile, fe, bitmap, vals, s_range, &s_err)) {  // its barriers publish tab2
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  const uint8_t* bm8 = reinterpret_cast<const uint8_t*>(bitmap);
  if (fast) {
    uint8_t* out_t = a.out + 2 * first;
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      const uint32_t local = g * 2048 + 8 * tid;
      uint4 o = bf16_decode8(tab2, nibs[g], sms[g]);
      const uint32_t esc8 = bm8[local >> 3];
      if (esc8) bf16_patch8(o, esc8, *reinterpret_cast<const uint2*>(vals + local));
      store_stream(out_t + 2 * local, o);
    }
    if (tid < 64) check_codebooks(a, h.k, 256u);
    return;
  }
  // last tile: byte-wise loads and stores
  uint16_t* out16 = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll 1
  for (uint32_t g = 0; g < kGroups; ++g) {
    const uint32_t local = g * 2048 + 8 * tid;
    const uint64_t e0 = first + local;
    if (e0 >= a.n) break;
    const uint32_t valid = (uint32_t)std::min<uint64_t>(8, a.n - e0);
    uint32_t tn = 0, t0 = 0, t1 = 0;
    for (uint32_t b = 0; b < (valid + 1) / 2; ++b) tn |= (uint32_t)nib_t[local / 2 + b] << (8 * b);
    for (uint32_t j = 0; j < valid; ++j) {
      const uint32_t x = (uint32_t)sm_t[local + j] << (8 * (j & 3));
      if (j < 4) t0 |= x;
      else t1 |= x;
    }
    uint4 o = bf16_decode8(tab2, tn, make_uint2(t0, t1));
    const uint32_t esc8 = bm8[local >> 3];
    if (esc8) bf16_patch8(o, esc8, *reinterpret_cast<const uint2*>(vals + local));
    for (uint32_t j = 0; j < valid; ++j) out16[e0 + j] = (uint16_t)(pick4(o.x, o.y, o.z, o.w, j >> 1) >> (16 * (j & 1)));
  }
  if (tid < 64) check_codebooks(a, h.k, 256u);
}

// E5M2 decode of 16 elements: the 16 codes (8 nibble bytes) through the
// code-pair table (entry = exponent of the low code << 2 | exponent of the
// high code << 10, i.e. two output bytes' exponent fields), and the 16
// sign|mantissa triples (bits 0..47 of lo:hi, element j at bit 3j).  The
// triples of word k (elements 4k..4k+3) are spread to one per byte in two
// steps (pairs to 16-bit halves, then triples to bytes); t + (t << 5) keeps
// the mantissa in bits 0..1 and moves the sign to bit 7 (no carries: t < 8).
__device__ inline uint32_t e5m2_spread(uint32_t y) {  // y: pairs at bits 0..5, 16..21
  const uint32_t z = (y & 0x00070007u) | ((y << 5) & 0x07000700u);
  return (z + (z << 5)) & 0x83838383u;
}

__device__ inline uint4 e5m2_decode16(const uint16_t* tab2, uint2 nib, uint32_t lo, uint32_t hi) {
  const uint32_t e0 = tab2[nib.x & 0xFF] | ((uint32_t)tab2[(nib.x >> 8) & 0xFF] << 16);
  const uint32_t e1 = tab2[(nib.x >> 16) & 0xFF] | ((uint32_t)tab2[nib.x >> 24] << 16);
  const uint32_t e2 = tab2[nib.y & 0xFF] | ((uint32_t)tab2[(nib.y >> 8) & 0xFF] << 16);
  const uint32_t e3 = tab2[(nib.y >> 16) & 0xFF] | ((uint32_t)tab2[nib.y >> 24] << 16);
  const uint32_t y0 = (lo & 0x3Fu) | ((lo << 10) & 0x3F0000u);
  const uint32_t y1 = ((lo >> 12) & 0x3Fu) | ((lo >> 2) & 0x3F0000u);
  const uint32_t y2 = ((lo >> 24) & 0x3Fu) | (__builtin_amdgcn_alignbit(hi, lo, 14) & 0x3F0000u);
  const uint32_t y3 = ((hi >> 4) & 0x3Fu) | ((hi << 6) & 0x3F0000u);
  return make_uint4(e5m2_spread(y0) | e0, e5m2_spread(y1) | e1, e5m2_spread(y2) | e2, e5m2_spread(y3) | e3);
}

// Raw exponents of escaped elements replace the looked-up ones: esc16 holds
// one flag per element, v the 16 staged bytes (bytes of elements without an
// escape are never used).
__device__ inline uint32_t e5m2_patch4(uint32_t w, uint32_t esc4, uint32_t v) {
  const uint32_t m = byte_mask4(esc4);
  return (w & ~(m & 0x7C7C7C7Cu)) | ((v & m) << 2);
}

__device__ inline void e5m2_patch16(uint4& o, uint32_t esc16, uint4 v) {
  o.x = e5m2_patch4(o.x, esc16 & 0xFu, v.x);
  o.y = e5m2_patch4(o.y, (esc16 >> 4) & 0xFu, v.y);
  o.z = e5m2_patch4(o.z, (esc16 >> 8) & 0xFu, v.z);
  o.w = e5m2_patch4(o.w, esc16 >> 12, v.w);
}

// E5M2 decode tile: 16384 elements = 4 groups of 4096; thread t owns
// elements 16t..16t+15 of each group (8 nibble bytes, 6 sign|mantissa bytes,
// 16 output bytes; lane-contiguous across a wave).  A whole tile takes the
// fast path: no bounds checks, and each thread's two aligned sign|mantissa
// dwords stay inside the tile's bytes (6t mod 4 is 0 or 2, and the last
// thread is odd).
__global__ __launch_bounds__(kThreads) void decode_e5m2_kernel(DecArgs a) {
  constexpr uint32_t kDecTile = kDecTileE5m2, kGroups = kDecTile / 4096;
  __shared__ uint32_t bitmap[kDecTile / 32];
  __shared__ alignas(16) uint8_t vals[kDecTile];
  __shared__ uint16_t tab2[256];
  __shared__ uint32_t s_range[2];
  __shared__ int s_err;
  Header h;
  if (!read_header(a, h)) {
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  if (a.n == 0) {  // header-only stream: off[0] must be 0
    if (threadIdx.x == 0 && ld64(a.in + h.s.offsets) != 0) report_corrupt(a.status);
    if (threadIdx.x < 64) check_codebooks(a, h.k, a.dtype == SPLITZIP_BF16 ? 256u : 32u);
    return;
  }
  const uint64_t tile = blockIdx.x;
  const uint64_t chunk = tile / (kChunk / kDecTile);
  const uint64_t cbi = h.k == 1 ? 0 : codebook_of_chunk(chunk, h.seg / kChunk);
  const uint8_t* cb = a.in + 64 + 16 * cbi;
  const uint32_t tid = threadIdx.x;
  const uint64_t first = tile * kDecTile;
  const bool fast = first + kDecTile <= a.n;  // same in every thread
  const uint8_t* nib_t = a.in + h.s.nib + first / 2;
  const uint8_t* sm_t = a.in + h.s.sm + 3 * (first / 8);
  const EscFetch fe = fetch_escapes<kDecTile>(a, h, tile);
  // then the tile's dense loads: the escape staging overlaps them
  uint2 pn[kGroups];
  uint32_t p0[kGroups], p1[kGroups];
  if (fast) {
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      // read once: non-temporal (as the BF16 decoder: 2.5 GiB after a 512 MiB
      // fill 900 -> 833 us)
      const u32x2_t n2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(nib_t + g * 2048 + 8 * tid));
      pn[g] = make_uint2(n2.x, n2.y);
      const uint8_t* s = sm_t + g * 1536 + ((6 * tid) & ~3u);
      p0[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(s));
      p1[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(s + 4));
    }
  }
  const uint32_t l0 = ld32(cb), l1 = ld32(cb + 4), l2 = ld32(cb + 8), l3 = ld32(cb + 12);
  if (((l0 | l1 | l2 | l3) & 0xE0E0E0E0u) != 0) {  // E5M2 exponents are 5 bits
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  {  // code-pair table entry tid: codes tid & 15 (even element) and tid >> 4
    const uint32_t c = tid & 0xFFu;
    const uint32_t pair = lut4((c & 0xFu) | ((c >> 4) << 8), l0, l1, l2, l3);  // bytes 0, 1: the two exponents
    tab2[c] = (uint16_t)((pair & 0xFFu) << 2 | ((pair >> 8) & 0xFFu) << 10);
  }
  if (!stage_escapes<kDecTile>(a, h, tile, fe, bitmap, vals, s_range, &s_err)) {  // its barriers publish tab2
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  if (fast) {
    uint8_t* out_t = a.out + first;
    const uint32_t sh = (tid & 1u) * 16;  // 6t mod 4 = 2 (t & 1)
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      const uint32_t local = g * 4096 + 16 * tid;
      uint4 o = e5m2_decode16(tab2, pn[g], __builtin_amdgcn_alignbit(p1[g], p0[g], sh), p1[g] >> sh);
      const uint32_t esc16 = (bitmap[local >> 5] >> (local & 31)) & 0xFFFFu;
      if (esc16) e5m2_patch16(o, esc16, *reinterpret_cast<const uint4*>(vals + local));
      store_stream(out_t + local, o);
    }
    if (tid < 64) check_codebooks(a, h.k, 32u);
    return;
  }
  // last tile: byte-wise loads and stores
#pragma unroll 1
  for (uint32_t g = 0; g < kGroups; ++g) {
    const uint32_t local = g * 4096 + 16 * tid;
    const uint64_t e0 = first + local;
    if (e0 >= a.n) break;
    const uint32_t valid = (uint32_t)std::min<uint64_t>(16, a.n - e0);
    uint32_t n0 = 0, n1 = 0;
    for (uint32_t k = 0; k < (valid + 1) / 2; ++k) {
      const uint32_t x = (uint32_t)nib_t[local / 2 + k] << (8 * (k & 3));
      if (k < 4) n0 |= x;
      else n1 |= x;
    }
    uint64_t v48 = 0;
    const uint8_t* s = sm_t + 6 * (local / 16);
    for (uint32_t k = 0; k < 3 * ((valid + 7) / 8); ++k) v48 |= (uint64_t)s[k] << (8 * k);
    uint4 o = e5m2_decode16(tab2, make_uint2(n0, n1), (uint32_t)v48, (uint32_t)(v48 >> 32));
    const uint32_t esc16 = (bitmap[local >> 5] >> (local & 31)) & 0xFFFFu;
    if (esc16) e5m2_patch16(o, esc16, *reinterpret_cast<const uint4*>(vals + local));
    for (uint32_t j = 0; j < valid; ++j) a.out[e0 + j] = (uint8_t)(pick4(o.x, o.y, o.z, o.w, j >> 2) >> (8 * (j & 3)));
  }
  if (tid < 64) check_codebooks(a, h.k, 32u);
}

// ---------------------------------------------- ablation decoders (BF16)
// Top-8: 3-bit codes, 8 per 3 bytes, element j of a group at bit 3j; the
// rest as the BF16 decode (8192-element tiles, 4 groups of 2048, 8 elements
// per thread, escapes staged from the position records).
__device__ inline uint32_t top8_spread4(uint32_t c12) {  // 4 codes of 3 bits -> one per byte
  const uint32_t y = (c12 & 0x3Fu) | ((c12 << 10) & 0x3F0000u);
  return (y & 0x00070007u) | ((y << 5) & 0x07000700u);
}

__device__ inline uint4 top8_decode8(uint32_t l0, uint32_t l1, uint32_t c24, uint2 sm) {
  const uint32_t e_lo = perm(l1, l0, top8_spread4(c24 & 0xFFFu));  // exponents of elements 0..3
  const uint32_t e_hi = perm(l1, l0, top8_spread4((c24 >> 12) & 0xFFFu));
  const uint32_t m0 = sm.x & 0x7F7F7F7Fu, s0 = sm.x & 0x80808080u;
  const uint32_t m1 = sm.y & 0x7F7F7F7Fu, s1 = sm.y & 0x80808080u;
  // value pair (2k, 2k+1): mantissas and signs by one permute, exponents e << 7 and e << 23
  return make_uint4(perm(s0, m0, 0x05010400u) | (perm(0u, e_lo, 0x0C010C00u) << 7),
                    perm(s0, m0, 0x07030602u) | (perm(0u, e_lo, 0x0C030C02u) << 7),
                    perm(s1, m1, 0x05010400u) | (perm(0u, e_hi, 0x0C010C00u) << 7),
                    perm(s1, m1, 0x07030602u) | (perm(0u, e_hi, 0x0C030C02u) << 7));
}

__global__ __launch_bounds__(kThreads) void decode_top8_kernel(DecArgs a) {
  constexpr uint32_t kDecTile = 8192, kGroups = 4;
  __shared__ uint32_t bitmap[kDecTile / 32];
  __shared__ alignas(16) uint8_t vals[kDecTile];
  __shared__ uint32_t s_range[2];
  __shared__ int s_err;
  Header h;
  if (!read_header(a, h)) {
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  if (a.n == 0) {
    if (threadIdx.x == 0 && ld64(a.in + h.s.offsets) != 0) report_corrupt(a.status);
    if (threadIdx.x < 64) check_codebooks(a, h.k, 256u);
    return;
  }
  const uint64_t tile = blockIdx.x;
  const uint64_t chunk = tile / (kChunk / kDecTile);
  const uint64_t cbi = h.k == 1 ? 0 : codebook_of_chunk(chunk, h.seg / kChunk);
  const uint8_t* cb = a.in + 64 + 16 * cbi;
  const uint32_t tid = threadIdx.x;
  const uint64_t first = tile * kDecTile;
  const bool fast = first + kDecTile <= a.n;  // same in every thread
  const uint8_t* code_t = a.in + h.s.nib + 3 * (first / 8);
  const uint8_t* sm_t = a.in + h.s.sm + first;
  const EscFetch fe = fetch_escapes<kDecTile>(a, h, tile);
  // the 3 code bytes of a thread lie in two aligned dwords; the last
  // thread's second dword reaches 4 bytes past the tile's codes, still
  // inside the stream (the sign|mantissa section follows)
  uint32_t p0[kGroups], p1[kGroups];
  uint2 sms[kGroups];
  if (fast) {
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      const uint8_t* c = code_t + g * 768 + ((3 * tid) & ~3u);
      p0[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c));  // read once, as the codec's decoder
      p1[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c + 4));
      const u32x2_t s2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(sm_t + g * 2048 + 8 * tid));
      sms[g] = make_uint2(s2.x, s2.y);
    }
  }
  const uint32_t l0 = ld32(cb), l1 = ld32(cb + 4);
  if (!stage_escapes<kDecTile>(a, h, tile, fe, bitmap, vals, s_range, &s_err)) {
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  const uint8_t* bm8 = reinterpret_cast<const uint8_t*>(bitmap);
  if (fast) {
    uint8_t* out_t = a.out + 2 * first;
    const uint32_t sh = 8 * ((3 * tid) & 3u);
#pragma unroll
    for (uint32_t g = 0; g < kGroups; ++g) {
      const uint32_t local = g * 2048 + 8 * tid;
      const uint32_t c24 = (uint32_t)(((((uint64_t)p1[g]) << 32) | p0[g]) >> sh) & 0xFFFFFFu;
      uint4 o = top8_decode8(l0, l1, c24, sms[g]);
      const uint32_t esc8 = bm8[local >> 3];
      if (esc8) bf16_patch8(o, esc8, *reinterpret_cast<const uint2*>(vals + local));
      store_stream(out_t + 2 * local, o);
    }
    if (tid < 64) check_codebooks(a, h.k, 256u);
    return;
  }
  uint16_t* out16 = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll 1
  for (uint32_t g = 0; g < kGroups; ++g) {
    const uint32_t local = g * 2048 + 8 * tid;
    const uint64_t e0 = first + local;
    if (e0 >= a.n) break;
    const uint32_t valid = (uint32_t)std::min<uint64_t>(8, a.n - e0);
    uint32_t c24 = 0, t0 = 0, t1 = 0;
    for (uint32_t b = 0; b < 3; ++b) c24 |= (uint32_t)code_t[3 * (local / 8) + b] << (8 * b);
    for (uint32_t j = 0; j < valid; ++j) {
      const uint32_t x = (uint32_t)sm_t[local + j] << (8 * (j & 3));
      if (j < 4) t0 |= x;
      else t1 |= x;
    }
    uint4 o = top8_decode8(l0, l1, c24, make_uint2(t0, t1));
    const uint32_t esc8 = bm8[local >> 3];
    if (esc8) bf16_patch8(o, esc8, *reinterpret_cast<const uint2*>(vals + local));
    for (uint32_t j = 0; j < valid; ++j) out16[e0 + j] = (uint16_t)(pick4(o.x, o.y, o.z, o.w, j >> 1) >> (16 * (j & 1)));
  }
  if (tid < 64) check_codebooks(a, h.k, 256u);
}

// Sets the exponent field of value j (0..7) of a decoded group to v.
__device__ inline void bf16_set_exponent(uint4& o, uint32_t j, uint32_t v) {
  const uint32_t sh = (j & 1u) ? 23u : 7u;
  const uint32_t m = 0xFFu << sh, x = v << sh;
  switch (j >> 1) {
    case 0: o.x = (o.x & ~m) | x; break;
    case 1: o.y = (o.y & ~m) | x; break;
    case 2: o.z = (o.z & ~m) | x; break;
    default: o.w = (o.w & ~m) | x; break;
  }
}

// Top-15 + sentinel: one workgroup per chunk.  A sentinel's raw exponent is
// the next unread value of the chunk's list, so an element's value index is
// the number of sentinels before it in the chunk: the chunk is decoded in 8
// passes of 8192 elements, each with a workgroup scan of the threads'
// sentinel counts, carried into the next pass.  This serial dependence is
// what the pages avoid by storing positions.
__global__ __launch_bounds__(kThreads) void decode_sentinel_kernel(DecArgs a) {
  __shared__ uint32_t tab2[256];
  __shared__ uint32_t wsum[2][8];
  __shared__ int s_bad;
  Header h;
  if (!read_header(a, h)) {
    if (threadIdx.x == 0) report_corrupt(a.status);
    return;
  }
  if (a.n == 0) {
    if (threadIdx.x == 0 && ld64(a.in + h.s.offsets) != 0) report_corrupt(a.status);
    if (threadIdx.x < 64) check_codebooks(a, h.k, 256u);
    return;
  }
  const uint32_t tid = threadIdx.x, wave = tid >> 6;
  const uint64_t chunk = blockIdx.x;
  const uint64_t chunk_first = chunk * kChunk;
  const uint32_t chunk_len = (uint32_t)std::min<uint64_t>(kChunk, a.n - chunk_first);
  const uint64_t cbi = h.k == 1 ? 0 : codebook_of_chunk(chunk, h.seg / kChunk);
  const uint8_t* cb = a.in + 64 + 16 * cbi;
  const uint8_t* offs = a.in + h.s.offsets;
  const uint64_t lo = ld64(offs + 8 * chunk), hi = ld64(offs + 8 * (chunk + 1));
  bool ok = lo <= hi && hi <= h.e;
  if (chunk == 0 && lo != 0) ok = false;
  if (chunk == h.chunks - 1 && hi != h.e) ok = false;
  if (!ok) {  // uniform
    if (tid == 0) report_corrupt(a.status);
    return;
  }
  {
    const uint32_t l0 = ld32(cb), l1 = ld32(cb + 4), l2 = ld32(cb + 8), l3 = ld32(cb + 12);
    const uint32_t pair = lut4((tid & 0xFu) | ((tid >> 4) << 8), l0, l1, l2, l3);
    tab2[tid] = ((pair & 0xFFu) << 7) | (((pair >> 8) & 0xFFu) << 23);
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const uint8_t* nib_c = a.in + h.s.nib + chunk_first / 2;
  const uint8_t* sm_c = a.in + h.s.sm + chunk_first;
  const uint8_t* esc = a.in + h.s.esc;
  uint16_t* out_c = reinterpret_cast<uint16_t*>(a.out) + chunk_first;
  uint64_t run = lo;  // value index of the pass's first sentinel, same in every thread
  bool bad = false;
  for (uint32_t pass = 0; pass < kChunk / 8192; ++pass) {
    const uint32_t pfirst = pass * 8192;
    if (pfirst >= chunk_len) break;  // uniform
    const bool full = pfirst + 8192 <= chunk_len;
    uint32_t nibs[4], mk[4], cnt[4];
    uint2 sms[4];
#pragma unroll
    for (uint32_t g = 0; g < 4; ++g) {
      const uint32_t local = pfirst + g * 2048 + 8 * tid;
      if (full) {
        nibs[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(nib_c + local / 2));
        const u32x2_t s2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(sm_c + local));  // read once
        sms[g] = make_uint2(s2.x, s2.y);
      } else {
        const uint32_t valid = local < chunk_len ? std::min<uint32_t>(8, chunk_len - local) : 0u;
        uint32_t tn = 0, t0 = 0, t1 = 0;
        for (uint32_t j = 0; j < valid; ++j) {
          const uint32_t nb = (nib_c[(local + j) / 2] >> (4 * (j & 1))) & 0xFu;  // missing elements: code 0
          tn |= nb << (4 * j);
          const uint32_t x = (uint32_t)sm_c[local + j] << (8 * (j & 3));
          if (j < 4) t0 |= x;
          else t1 |= x;
        }
        nibs[g] = tn;
        sms[g] = make_uint2(t0, t1);
      }
      const uint32_t w = nibs[g];
      mk[g] = w & (w >> 1) & (w >> 2) & (w >> 3) & 0x11111111u;  // nibble j == 15 -> bit 4j
      cnt[g] = __builtin_popcount(mk[g]);
    }
    // element-order ranks within the pass: groups in order, threads in order
    const uint32_t p01 = cnt[0] | (cnt[1] << 16), p23 = cnt[2] | (cnt[3] << 16);
    const uint32_t i01 = wave_inclusive_sum(p01), i23 = wave_inclusive_sum(p23);
    uint32_t* ws = wsum[pass & 1];
    if ((tid & 63) == 63) {
      ws[wave] = i01;
      ws[4 + wave] = i23;
    }
    __syncthreads();
    uint32_t pre01 = 0, pre23 = 0, tot01 = 0, tot23 = 0;
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) {
      pre01 += v < wave ? ws[v] : 0u;
      pre23 += v < wave ? ws[4 + v] : 0u;
      tot01 += ws[v];
      tot23 += ws[4 + v];
    }
    const uint32_t g0 = tot01 & 0xFFFF, g1 = tot01 >> 16, g2 = tot23 & 0xFFFF, g3 = tot23 >> 16;
    const uint32_t x01 = pre01 + i01 - p01, x23 = pre23 + i23 - p23;
    const uint32_t rank[4] = {x01 & 0xFFFF, g0 + (x01 >> 16), g0 + g1 + (x23 & 0xFFFF), g0 + g1 + g2 + (x23 >> 16)};
#pragma unroll
    for (uint32_t g = 0; g < 4; ++g) {
      const uint32_t local = pfirst + g * 2048 + 8 * tid;
      uint4 o = bf16_decode8(tab2, nibs[g], sms[g]);
      uint32_t m = mk[g];
      uint64_t idx = run + rank[g];
      while (m) {  // sentinels: their raw exponents, in order
        const uint32_t j = __builtin_ctz(m) >> 2;
        m &= m - 1;
        if (idx >= hi) {
          bad = true;
          break;
        }
        bf16_set_exponent(o, j, esc[idx]);
        ++idx;
      }
      if (full) {
        store_stream(out_c + local, o);
      } else if (local < chunk_len) {
        const uint32_t valid = std::min<uint32_t>(8, chunk_len - local);
        for (uint32_t j = 0; j < valid; ++j) out_c[local + j] = (uint16_t)(pick4(o.x, o.y, o.z, o.w, j >> 1) >> (16 * (j & 1)));
      }
    }
    run += g0 + g1 + g2 + g3;
  }
  if (bad) s_bad = 1;
  __syncthreads();
  if (tid == 0 && (s_bad || run != hi)) report_corrupt(a.status);
  if (tid < 64) check_codebooks(a, h.k, 256u);
}

// ------------------------------------------------------------ host helpers
bool dtype_valid(int dtype) { return dtype == SPLITZIP_BF16 || dtype == SPLITZIP_FP8_E5M2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint32_t exponent_of(int dtype, const void* data, size_t i) {
  if (dtype == SPLITZIP_BF16) return (static_cast<const uint16_t*>(data)[i] >> 7) & 0xFFu;
  return (static_cast<const uint8_t*>(data)[i] >> 2) & 0x1Fu;
}

int codebooks_valid(int dtype, const uint8_t* cbs, uint32_t k) {
  const uint32_t limit = dtype == SPLITZIP_BF16 ? 256u : 32u;
  for (uint32_t c = 0; c < k; ++c) {
    uint32_t seen[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < 16; ++i) {
      const uint32_t v = cbs[16 * c + i];
      if (v >= limit || (seen[v >> 5] >> (v & 31)) & 1u) return 0;
      seen[v >> 5] |= 1u << (v & 31);
    }
  }
  return 1;
}

// Worst-case stream plus encoder workspace.
size_t max_size_of(int dtype, int variant, size_t n_elems, uint32_t n_codebooks) {
  if (!dtype_valid(dtype) || n_codebooks == 0 || n_codebooks > kMaxK || n_elems > kMaxN) return 0;
  return workspace_layout(dtype, n_elems, n_codebooks, variant).end;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

int splitzip_calibrate(int dtype, const void* host_samples, size_t n_elems, uint8_t codebook_out[16]) {
  if (!dtype_valid(dtype) || codebook_out == nullptr || (host_samples == nullptr && n_elems > 0))
    return SPLITZIP_E_INVALID;
  const uint32_t values = dtype == SPLITZIP_BF16 ? 256u : 32u;
  uint64_t count[256] = {};
  for (size_t i = 0; i < n_elems; ++i) ++count[exponent_of(dtype, host_samples, i)];
  uint32_t order[256];
  for (uint32_t v = 0; v < values; ++v) order[v] = v;
  std::stable_sort(order, order + values, [&](uint32_t x, uint32_t y) { return count[x] > count[y]; });
  for (int k = 0; k < 16; ++k) codebook_out[k] = static_cast<uint8_t>(order[k]);
  return SPLITZIP_OK;
}

size_t splitzip_max_compressed_size(int dtype, size_t n_elems, uint32_t n_codebooks) {
  if (!dtype_valid(dtype) || n_codebooks == 0 || n_codebooks > kMaxK || n_elems > kMaxN) return 0;
  return max_size_of(dtype, kMain, n_elems, n_codebooks);
}

}  // extern "C"

namespace {

// Polls encode_single makes for a lower tile's count before computing it
// itself: SPLITZIP_STATIC_WAIT_POLLS if set (0 makes every count that has not
// arrived at the first poll be computed, which tests use), else 64 (about a
// tenth of a millisecond; co-resident workgroups need one or two).
uint32_t static_wait_polls() {
  constexpr uint32_t kDefault = 64;
  const char* v = getenv("SPLITZIP_STATIC_WAIT_POLLS");
  if (v == nullptr || *v == 0) return kDefault;
  char* end = nullptr;
  const unsigned long x = strtoul(v, &end, 10);
  return (end && *end == 0 && x <= 0xFFFFFFFFul) ? (uint32_t)x : kDefault;
}

// Host half of the compress entry points.  static_ws: the current device's
// one-launch scratch (splitzip_compress_static), else nullptr (the workspace
// is the tail of d_out).
int compress_impl(int dtype, int variant, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                  uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity, uint64_t* d_out_bytes,
                  hipStream_t stream, uint32_t* static_ws = nullptr) {
  if (!dtype_valid(dtype) || n_elems > kMaxN || h_codebooks == nullptr || n_codebooks == 0 || n_codebooks > kMaxK)
    return SPLITZIP_E_INVALID;
  if ((d_in == nullptr && n_elems > 0) || d_out == nullptr || !aligned(d_in, 16) || !aligned(d_out, 16) ||
      !aligned(d_out_bytes, 8))
    return SPLITZIP_E_INVALID;
  if (n_codebooks > 1 && (segment_elems == 0 || segment_elems % kChunk != 0 || segment_elems < divup(n_elems, n_codebooks)))
    return SPLITZIP_E_INVALID;
  if (!codebooks_valid(dtype, h_codebooks, n_codebooks)) return SPLITZIP_E_CODEBOOK;
  const uint64_t need = static_ws ? workspace_offset(dtype, n_elems, n_codebooks, variant)
                                  : max_size_of(dtype, variant, n_elems, n_codebooks);
  if (out_capacity < need) return SPLITZIP_E_CAPACITY;

  const uint64_t n = n_elems;
  const Sections s = sections_of(dtype, n, n_codebooks, variant);
  const uint64_t n_tiles = divup(n, dtype == SPLITZIP_BF16 ? kEncTileBf16 : kEncTileE5m2);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  Workspace w = workspace_of(out, dtype, n, n_codebooks, variant);
  if (static_ws) {
    w.tile_count = static_ws;
    w.stage = static_ws + kStaticStageAt;
    w.block_sum = w.super_sum = nullptr;  // at most 64 blocks: never read
  }

  // header, codebooks and padding: a launch of their own when the stream is
  // empty or the codebooks do not fit the kernel arguments; otherwise folded
  // into a later launch as one extra workgroup
  auto prep_args = [&](PrepArgs& p, uint32_t first) {
    memset(&p, 0, sizeof(p));
    p.out = out;
    p.n = n;
    p.seg_stored = n_codebooks == 1 ? n : segment_elems;
    p.nib = s.nib;
    p.sm = s.sm;
    p.esc = s.esc;
    p.sm_bytes = s.sm_bytes;
    p.code_bytes = variant == kTop8 ? 3 * divup(n, 8) : divup(n, 2);
    p.offsets = s.offsets;
    p.chunks = s.chunks;
    p.out_bytes = d_out_bytes;
    p.k = n_codebooks;
    p.dtype = (uint32_t)dtype;
    p.variant = (uint32_t)variant;
    p.cb_first = first;
    p.cb_count = std::min<uint32_t>(kCbPerPrep, n_codebooks - first);
    p.main = first == 0;
    memcpy(p.cbs, h_codebooks + 16ull * first, 16ull * p.cb_count);
  };
  const bool cb_args = n > 0 && n_codebooks <= (uint32_t)kCbPerPrep;
  if (!cb_args) {
    for (uint32_t first = 0; first < n_codebooks; first += kCbPerPrep) {
      PrepArgs p;
      prep_args(p, first);
      const uint32_t blocks = (uint32_t)std::max<uint64_t>(1, divup(16ull * p.cb_count, kThreads));
      prep_kernel<<<blocks, kThreads, 0, stream>>>(p);
      if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
    }
  }
  if (n == 0) return SPLITZIP_OK;

  EncArgs e;
  e.in = static_cast<const uint8_t*>(d_in);
  e.out = out;
  e.n = n;
  e.n_tiles = n_tiles;
  e.offsets = s.offsets;
  e.nib = s.nib;
  e.sm = s.sm;
  e.esc = s.esc;
  e.chunks = s.chunks;
  e.seg_chunks = n_codebooks == 1 ? 0 : segment_elems / kChunk;
  e.tile_count = w.tile_count;
  e.stage = w.stage;
  e.block_sum = w.block_sum;
  e.super_sum = w.super_sum;
  e.out_bytes = d_out_bytes;
  const uint32_t tiles = (uint32_t)n_tiles;  // n <= 2^36 -> at most 2^23 tiles
  const uint64_t blocks = divup(n_tiles, kBlockTiles);
  e.n_blocks = blocks;
  // tiles per encode_place workgroup: the power of two from 8 to 64 that
  // gives about kPlaceWgs workgroups
  e.place_tiles = 8;
  while (e.place_tiles < kBlockTiles && (uint64_t)e.place_tiles * kPlaceWgs < n_tiles) e.place_tiles *= 2;
  e.cb_args = cb_args;
  e.sums_in_place = blocks <= 64;
  e.prep_in = cb_args ? (e.sums_in_place ? 2 : 1) : 0;
  e.single = nullptr;
  e.wait_polls = 0;
  if (cb_args) prep_args(e.prep, 0);
  else memset(&e.prep, 0, sizeof(e.prep));
  if (static_ws && variant == kMain && n_tiles <= kSingleMaxTiles) {
    // one launch (encode_single), the header work as its extra workgroup
    e.single = static_ws + kSingleAt;
    e.wait_polls = static_wait_polls();
    e.prep_in = cb_args ? 3 : 0;
    const uint32_t wgs = tiles + (cb_args ? 1u : 0u);
    if (dtype == SPLITZIP_FP8_E5M2) encode_single_e5m2_kernel<<<wgs, kThreads, 0, stream>>>(e);
    else encode_single_bf16_kernel<<<wgs, kThreads, 0, stream>>>(e);
    return hipGetLastError() == hipSuccess ? SPLITZIP_OK : SPLITZIP_E_HIP;
  }
  if (dtype == SPLITZIP_FP8_E5M2) encode_dense_e5m2_kernel<<<tiles, kThreads, 0, stream>>>(e);
  else if (variant == kSentinel) encode_dense_sentinel_kernel<<<tiles, kThreads, 0, stream>>>(e);
  else if (variant == kTop8) encode_dense_top8_kernel<<<tiles, kThreads, 0, stream>>>(e);
  else encode_dense_bf16_kernel<<<tiles, kThreads, 0, stream>>>(e);
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  if (!e.sums_in_place) {
    encode_sums_kernel<<<(uint32_t)divup(blocks, kThreads) + (e.prep_in == 1), kThreads, 0, stream>>>(e);
    if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  }
  const uint32_t place_wgs = (uint32_t)divup(n_tiles, e.place_tiles) + (e.prep_in == 2);
  if (dtype == SPLITZIP_FP8_E5M2) encode_place_e5m2_kernel<<<place_wgs, kThreads, 0, stream>>>(e);
  else if (variant == kSentinel) encode_place_sentinel_kernel<<<place_wgs, kThreads, 0, stream>>>(e);
  else if (variant == kTop8) encode_place_top8_kernel<<<place_wgs, kThreads, 0, stream>>>(e);
  else encode_place_bf16_kernel<<<place_wgs, kThreads, 0, stream>>>(e);
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  return SPLITZIP_OK;
}

}  // namespace

extern "C" {

int splitzip_compress(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks, uint32_t n_codebooks,
                      size_t segment_elems, void* d_out, size_t out_capacity, uint64_t* d_out_bytes,
                      hipStream_t stream) {
  return compress_impl(dtype, kMain, d_in, n_elems, h_codebooks, n_codebooks, segment_elems, d_out, out_capacity,
                       d_out_bytes, stream);
}

}  // extern "C"

namespace {

// Per device: the address of `scratch` (hipGetSymbolAddress with the device
// current), looked up at the device's first splitzip_compress_static call.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
uint32_t* g_scratch[kMaxDevices] = {};

// The current device's scratch address.
int static_scratch(uint32_t** ws) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPLITZIP_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SPLITZIP_E_HIP;
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *ws = g_scratch[dev];
  return SPLITZIP_OK;
}

}  // namespace

extern "C" {

int splitzip_compress_static(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                             uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity,
                             uint64_t* d_out_bytes, hipStream_t stream) {
  if (!dtype_valid(dtype)) return SPLITZIP_E_INVALID;
  const uint64_t tile = dtype == SPLITZIP_BF16 ? kEncTileBf16 : kEncTileE5m2;
  if (n_elems > kStaticMaxTiles * tile) return SPLITZIP_E_TOO_LARGE;
  if (n_elems == 0)  // header only: no workspace
    return compress_impl(dtype, kMain, d_in, 0, h_codebooks, n_codebooks, segment_elems, d_out, out_capacity,
                         d_out_bytes, stream);
  uint32_t* ws = nullptr;
  const int rc = static_scratch(&ws);
  if (rc != SPLITZIP_OK) return rc;
  return compress_impl(dtype, kMain, d_in, n_elems, h_codebooks, n_codebooks, segment_elems, d_out, out_capacity,
                       d_out_bytes, stream, ws);
}

size_t splitzip_variant_max_compressed_size(int variant, size_t n_elems, uint32_t n_codebooks) {
  if (variant != kSentinel && variant != kTop8) return 0;
  return max_size_of(SPLITZIP_BF16, variant, n_elems, n_codebooks);
}

int splitzip_variant_compress(int variant, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                              uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity,
                              uint64_t* d_out_bytes, hipStream_t stream) {
  if (variant != kSentinel && variant != kTop8) return SPLITZIP_E_INVALID;
  return compress_impl(SPLITZIP_BF16, variant, d_in, n_elems, h_codebooks, n_codebooks, segment_elems, d_out,
                       out_capacity, d_out_bytes, stream);
}

int splitzip_decompress(const void* d_in, size_t in_bytes, int dtype, size_t n_elems, void* d_out, int32_t* d_status,
                        hipStream_t stream) {
  if (!dtype_valid(dtype) || n_elems > kMaxN || d_in == nullptr || in_bytes < 64 || !aligned(d_in, 16) ||
      (d_out == nullptr && n_elems > 0) || !aligned(d_out, 16) || !aligned(d_status, 4))
    return SPLITZIP_E_INVALID;
  DecArgs a;
  a.in = static_cast<const uint8_t*>(d_in);
  a.in_bytes = in_bytes;
  a.out = static_cast<uint8_t*>(d_out);
  a.n = n_elems;
  a.status = d_status;
  a.dtype = dtype;
  a.variant = kMain;
  // one workgroup per tile; a header-only stream (n == 0) still gets one
  // workgroup, which only validates
  if (dtype == SPLITZIP_BF16) {
    decode_bf16_kernel<<<(uint32_t)std::max<uint64_t>(1, divup(n_elems, kDecTileBf16)), kThreads, 0, stream>>>(a);
  } else {
    decode_e5m2_kernel<<<(uint32_t)std::max<uint64_t>(1, divup(n_elems, kDecTileE5m2)), kThreads, 0, stream>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  return SPLITZIP_OK;
}

int splitzip_variant_decompress(int variant, const void* d_in, size_t in_bytes, size_t n_elems, void* d_out,
                                int32_t* d_status, hipStream_t stream) {
  if ((variant != kSentinel && variant != kTop8) || n_elems > kMaxN || d_in == nullptr || in_bytes < 64 ||
      !aligned(d_in, 16) || (d_out == nullptr && n_elems > 0) || !aligned(d_out, 16) || !aligned(d_status, 4))
    return SPLITZIP_E_INVALID;
  DecArgs a;
  a.in = static_cast<const uint8_t*>(d_in);
  a.in_bytes = in_bytes;
  a.out = static_cast<uint8_t*>(d_out);
  a.n = n_elems;
  a.status = d_status;
  a.dtype = SPLITZIP_BF16;
  a.variant = variant;
  if (variant == kTop8) {
    decode_top8_kernel<<<(uint32_t)std::max<uint64_t>(1, divup(n_elems, 8192)), kThreads, 0, stream>>>(a);
  } else {
    decode_sentinel_kernel<<<(uint32_t)std::max<uint64_t>(1, divup(n_elems, kChunk)), kThreads, 0, stream>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  return SPLITZIP_OK;
}

const char* splitzip_status_string(int status) {
  switch (status) {
    case SPLITZIP_OK: return "ok";
    case SPLITZIP_E_INVALID: return "invalid argument";
    case SPLITZIP_E_CAPACITY: return "output capacity too small";
    case SPLITZIP_E_CODEBOOK: return "invalid codebook";
    case SPLITZIP_E_CORRUPT: return "corrupt stream";
    case SPLITZIP_E_HIP: return "HIP launch failure";
    case SPLITZIP_E_TOO_LARGE: return "input larger than splitzip_compress_static's workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
