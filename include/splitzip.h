/*
 * splitzip.h -- C ABI of libsplitzip, a lossless exponent codec for BF16 and
 * FP8 E5M2 KV-cache tensors on AMD Instinct MI355X (gfx950).
 *
 * The method is SplitZip ("SplitZip: Ultra Fast Lossless KV Compression for
 * Disaggregated LLM Serving", arXiv 2605.01708v2).  Its pages state the
 * problem this ABI serves: KV tensors must reach the decode side bit for bit,
 * and the codec must plug into a serving stack without touching model
 * execution (authors' abstract; Spanish technical summary, "Metodologia").
 *
 * Conventions for every call:
 *   - extern "C", never throws, returns an int status (SPLITZIP_OK = 0 or a
 *     negative SPLITZIP_E_* code); sizes are element or byte counts.
 *   - "d_" pointers are device memory (hipMalloc'd, or any memory the GPU
 *     can address); "h_" pointers are host memory.  The caller owns every
 *     buffer.  No call allocates device or host memory (the pipelined
 *     transfer creates HIP events for the duration of its call).
 *   - GPU work is enqueued on `stream` (NULL = the default stream) and is not
 *     waited for.  Host-detectable argument errors return at once and enqueue
 *     nothing.  A failed kernel launch returns SPLITZIP_E_HIP.
 *   - Calls on different streams may run concurrently when their buffers are
 *     disjoint; the library keeps no mutable global state, except the device
 *     array behind splitzip_compress_static (whose calls must not overlap on
 *     one GPU; see there).
 *   - The device calls (compress, decompress and their variants, the device
 *     calibration) only launch kernels on `stream`: no allocation, memset or
 *     synchronization, so they can be captured in a HIP graph and replayed.
 *     Decompress takes in_bytes as an upper bound (the buffer's size), so a
 *     captured decompress serves streams of any size S <= in_bytes.
 *
 * Stream format "SZ1" (little-endian; A(x) = x rounded up to a multiple of
 * 256; n elements, C = ceil(n / 65536) chunks, K codebooks, E escapes):
 *   0    u32 magic 0x00315A53        4  u16 version 1
 *   6    u8  dtype                    7  u8  log2 chunk size = 16
 *   8    u64 n                        16 u64 E
 *   24   u64 total stream bytes S     32 u32 C      36 u32 K
 *   40   u64 elements per segment (n when K == 1)
 *   48   16 zero bytes
 *   64          K codebooks of 16 bytes (byte k = exponent of 4-bit code k)
 *   64 + 16K    C + 1 u64: escapes before chunk c (off[C] = E)
 *   N0 = A(64 + 16K + 8(C + 1)): 4-bit codes, two per byte, even element in
 *        the low nibble; an escaped element has code 0        (ceil(n/2) B)
 *   N1 = N0 + A(ceil(n/2)): sign|mantissa
 *        BF16: one byte per element, sign at bit 7, mantissa bits 6..0 (n B)
 *        E5M2: 3 bits per element (sign << 2 | mantissa), 8 elements per 3
 *              little-endian bytes, element j of a group at bits 3j  (3 ceil(n/8) B)
 *   P  = N1 + A(sign|mantissa bytes): E escape records of 3 bytes
 *        [position in chunk, low byte][high byte][raw exponent], in element order
 *   S  = P + 3E.  All bytes between sections are zero.
 * Chunk c is coded with codebook 0 when K == 1, else with codebook
 * floor(65536 c / segment_elems).
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  BF16: 1 sign, 8 exponent, 7 mantissa bits (English
 * explainer, "1. The 'Note' Structure").  FP8 E5M2: 1 sign, 5 exponent,
 * 2 mantissa bits (technical summary, "Contribuciones Clave" 4). */
typedef enum { SPLITZIP_BF16 = 1, SPLITZIP_FP8_E5M2 = 2 } splitzip_dtype;

enum {
  SPLITZIP_OK = 0,
  SPLITZIP_E_INVALID = -1,  /* bad argument: null/misaligned pointer, dtype, sizes, segments */
  SPLITZIP_E_CAPACITY = -2, /* output buffer smaller than splitzip_max_compressed_size() */
  SPLITZIP_E_CODEBOOK = -3, /* codebook entries repeated or out of range for the dtype */
  SPLITZIP_E_CORRUPT = -4,  /* stream fails validation (reported through d_status) */
  SPLITZIP_E_HIP = -5,      /* a HIP launch failed */
  SPLITZIP_E_TOO_LARGE = -6 /* input beyond splitzip_compress_static's limit */
};

/* Offline calibration (technical summary, "Metodologia / Codificacion de
 * Longitud Fija" and "Optimizacion"; "Resultados / Calibracion"; abstract):
 * histogram the exponents of n_elems host samples and return the 16 most
 * frequent exponent values in codebook_out[0..15], most frequent first;
 * equal counts go to the lower exponent; values never seen fill the
 * remaining slots in ascending order, so the 16 entries are always distinct.
 * host_samples: n_elems BF16 (uint16 bit patterns) or E5M2 (uint8) values in
 * host memory; may be NULL only when n_elems == 0.  Synchronous, host only.
 * Returns SPLITZIP_OK or SPLITZIP_E_INVALID. */
int splitzip_calibrate(int dtype, const void* host_samples, size_t n_elems, uint8_t codebook_out[16]);

/* Bytes the caller must provide as d_out of splitzip_compress for n_elems
 * elements and n_codebooks codebooks: the largest possible stream (every
 * element escaped) rounded up to 256, plus the encoder's workspace: per
 * 8192-element tile 2052 bytes (a count and a staging slot for up to 512
 * escape records), per 64 tiles 8 bytes and per 4096 tiles 8 bytes, with
 * 256-byte alignment.  Returns 0 for an invalid dtype,
 * n_codebooks == 0 or n_elems > 2^36 (the largest n any call accepts: every
 * kernel grid then stays below 2^32 work-items; 2^36 BF16 elements are
 * 128 GiB). */
size_t splitzip_max_compressed_size(int dtype, size_t n_elems, uint32_t n_codebooks);

/* Encode (technical summary, "Estrategia de Codificacion"; abstract; English
 * explainer, "3. The SplitZip Strategy"): split every element into exponent
 * and sign|mantissa, map the exponent through its chunk's codebook to a 4-bit
 * code, and route exponents outside the codebook to the escape records.
 *   d_in          n_elems elements (BF16 as uint16, E5M2 as uint8), 16-byte aligned.
 *   h_codebooks   n_codebooks x 16 bytes, host memory, read before return.
 *   segment_elems elements per codebook; ignored when n_codebooks == 1,
 *                 else a non-zero multiple of 65536 with
 *                 n_codebooks * segment_elems >= n_elems.
 *   d_out         out_capacity bytes, 16-byte aligned; the stream is written
 *                 at its start; bytes after the stream are the encoder's
 *                 workspace and are overwritten.
 *   d_out_bytes   optional (may be NULL): receives the stream size S, written
 *                 by the GPU when the encode completes (device or pinned host
 *                 memory, 8-byte aligned).
 * The stream is byte-for-byte deterministic for given inputs.  d_in is not
 * modified.  Returns SPLITZIP_OK, SPLITZIP_E_INVALID, SPLITZIP_E_CODEBOOK,
 * SPLITZIP_E_CAPACITY or SPLITZIP_E_HIP. */
int splitzip_compress(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                      uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity,
                      uint64_t* d_out_bytes, hipStream_t stream);

/* Decode (technical summary, "Estrategia de Decodificacion / Paralelismo"
 * and "Correccion"; English explainer, "4. Why It's Fast"): map every 4-bit
 * code through its codebook, recombine with the sign|mantissa bits, then
 * overwrite the exponent of every escaped element with its raw value.  One
 * kernel launch.
 *   d_in      the stream (in_bytes >= its size S, 16-byte aligned).
 *   dtype, n_elems must match the stream header.
 *   d_out     n_elems elements, 16-byte aligned.
 *   d_status  optional (may be NULL), device int32, sticky: the caller sets
 *             it to SPLITZIP_OK (0) beforehand; the GPU writes
 *             SPLITZIP_E_CORRUPT into it if it finds the stream invalid and
 *             never clears it, so one word can watch many calls.  d_out is
 *             then unspecified.  Invalid means: bad magic, version, dtype, n,
 *             non-zero reserved header bytes, chunk count, codebook count
 *             or segment size; E > n or
 *             S != P + 3E or S > in_bytes; any of the K codebooks (used by a
 *             chunk or not) with a repeated entry or, for E5M2, an entry of
 *             32 or more; chunk offsets not starting at 0, decreasing, above
 *             E, not ending at E, or giving a chunk more records than
 *             elements; an escape position outside its chunk or not above
 *             the previous one of the chunk; an escape value of 32 or more
 *             (E5M2).  Every stream the encoder writes passes these checks,
 *             and they are the oracle's.  Every read stays inside in_bytes.
 * Returns SPLITZIP_OK, SPLITZIP_E_INVALID or SPLITZIP_E_HIP. */
int splitzip_decompress(const void* d_in, size_t in_bytes, int dtype, size_t n_elems, void* d_out,
                        int32_t* d_status, hipStream_t stream);

/* Static text for a status code. */
const char* splitzip_status_string(int status);

/* splitzip_compress for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The encoder's workspace (per-tile escape counts and record
 * staging slots) is the library's own device array (about 4 MiB per GPU,
 * kept until the process ends) instead of the tail of d_out.  Inputs of at
 * most 512 tiles (4M BF16 or 8M E5M2 elements) take one launch whose
 * workgroups exchange their tiles' escape counts through that array (a wait
 * for a count is bounded: SPLITZIP_STATIC_WAIT_POLLS polls, 64 if unset,
 * after which the count is computed from the input); larger ones take the
 * launches of splitzip_compress.  d_out only needs room for the largest
 * stream:
 *   out_capacity >= A(P + 3 n_elems), P as in the layout above with
 *   n_elems escapes (splitzip_max_compressed_size minus the workspace).
 * Limit: n_elems <= 2048 * 8192 (BF16) or 2048 * 16384 (E5M2), 32 MiB of
 * input, else SPLITZIP_E_TOO_LARGE.  Other arguments, errors and the stream
 * are those of splitzip_compress: the stream is byte for byte the one
 * splitzip_compress writes.  No hipMalloc, hipFree, memset or host
 * synchronization, so it can be captured in a HIP graph.  Every call on one
 * GPU shares that GPU's workspace: calls that overlap on one GPU (two
 * streams, two host threads) race and may write wrong streams; serialize
 * them.  Calls that follow a race are not affected by it.  The stream
 * passed must belong to the current device.
 * Returns SPLITZIP_OK, SPLITZIP_E_INVALID, SPLITZIP_E_CODEBOOK,
 * SPLITZIP_E_CAPACITY, SPLITZIP_E_TOO_LARGE or SPLITZIP_E_HIP. */
int splitzip_compress_static(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                             uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity,
                             uint64_t* d_out_bytes, hipStream_t stream);

/* ---- Ablation variants (BF16) ---------------------------------------------
 * The two designs the pages measure against the top-16 codec (technical
 * summary, "Metodologia / Decision de Diseno" and "Resultados"), as streams
 * of their own, to compare decode speed and size on this GPU:
 *   SPLITZIP_VARIANT_TOP15_SENTINEL  codebook entries 0..14 get codes 0..14;
 *     code 15 marks an escape, whose raw exponent is the next byte of the
 *     escape section (no positions: the pages' design with less side data).
 *   SPLITZIP_VARIANT_TOP8            codebook entries 0..7 get 3-bit codes,
 *     8 codes per 3 little-endian bytes (element j at bit 3j); escapes are the
 *     codec's 3-byte position records.
 * Layout: the SZ1 layout with header byte 48 = the variant, the code section
 * of ceil(n/2) (top-15) or 3 ceil(n/8) (top-8) bytes, and E escape bytes
 * (top-15) or 3E (top-8) at the end.  Codebooks are 16 distinct entries per
 * segment as for splitzip_compress; the variant uses the first 15 or 8.
 * The arguments, alignment, workspace and status conventions are those of
 * splitzip_max_compressed_size, splitzip_compress and splitzip_decompress,
 * except that the top-8 workspace stages up to 1024 escape records per
 * 8192-element tile (4 KiB per tile, against 2 KiB for the codec's 512);
 * dtype is BF16.  An invalid variant returns 0 / SPLITZIP_E_INVALID. */
typedef enum { SPLITZIP_VARIANT_TOP15_SENTINEL = 1, SPLITZIP_VARIANT_TOP8 = 2 } splitzip_variant;

size_t splitzip_variant_max_compressed_size(int variant, size_t n_elems, uint32_t n_codebooks);

int splitzip_variant_compress(int variant, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                              uint32_t n_codebooks, size_t segment_elems, void* d_out, size_t out_capacity,
                              uint64_t* d_out_bytes, hipStream_t stream);

/* Top-8: one workgroup per 8192-element tile, as splitzip_decompress.
 * Top-15 + sentinel: one workgroup per chunk, which counts the sentinels
 * before every element to find its value (the irregular step the pages
 * attribute the design's slower decode to). */
int splitzip_variant_decompress(int variant, const void* d_in, size_t in_bytes, size_t n_elems, void* d_out,
                                int32_t* d_status, hipStream_t stream);

/* ---- On-device calibration ------------------------------------------------
 * The pages calibrate offline, so that no histogram is built on the critical
 * path (technical summary, "Optimizacion" and "Resultados / Calibracion";
 * abstract).  splitzip_calibrate_device builds that histogram on the GPU, to
 * measure what calibrating online would cost and to calibrate per tensor or
 * per layer at run time.  The codebooks equal splitzip_calibrate's on the same
 * samples: the 16 most frequent exponents, most frequent first, equal counts
 * to the lower exponent, unseen exponents filling up in ascending order.
 *
 * splitzip_calibrate_device_work_bytes: bytes of d_work for n_codebooks
 * segments (8 per histogram bin: 256 bins BF16, 32 E5M2), 0 for an invalid
 * dtype or n_codebooks outside 1..65535. */
size_t splitzip_calibrate_device_work_bytes(int dtype, uint32_t n_codebooks);

/* splitzip_calibrate_device: one codebook per segment of d_samples.
 *   d_samples       n_elems elements on the device (BF16 as uint16, E5M2 as
 *                   uint8), 16-byte aligned.
 *   segment_elems   elements per segment, ignored when n_codebooks == 1
 *                   (one segment: the whole tensor); else segment k covers
 *                   [k * segment_elems, min((k + 1) * segment_elems, n)) and
 *                   n_codebooks * segment_elems >= n_elems.  A segment with no
 *                   elements gets the codebook 0, 1, ..., 15.
 *   d_codebooks_out n_codebooks x 16 bytes, device memory, written by the GPU.
 *   d_work          work_bytes of device memory, 8-byte aligned, overwritten.
 * Stream-ordered, three launches, no host synchronization.  Returns
 * SPLITZIP_OK, SPLITZIP_E_INVALID, SPLITZIP_E_CAPACITY or SPLITZIP_E_HIP. */
int splitzip_calibrate_device(int dtype, const void* d_samples, size_t n_elems, size_t segment_elems,
                              uint32_t n_codebooks, uint8_t* d_codebooks_out, void* d_work, size_t work_bytes,
                              hipStream_t stream);

/* ---- Chunk-pipelined transfer through a host link -------------------------
 * The pages' setting is a KV cache moving from a prefill node to a decode
 * node over a 50-100 GB/s link, where the codec shrinks the transferred bytes
 * and pays for itself (technical summary, "Planteamiento del Problema" and
 * "Resultados": 1.22-1.32x faster transfers).  On one GPU the link is the
 * PCIe path to pinned host memory: each group of group_elems elements is
 * compressed (splitzip_compress), copied to host memory and back by the copy
 * engines, and decompressed (splitzip_decompress) into d_out, with up to
 * `depth` groups in flight.  A compressed group's size exists only on the
 * device: the encoder writes it into the link buffer, and the host, one group
 * behind the encoder, polls it before queuing that group's copies.
 *
 * Each group is a complete SZ1 stream of its own elements.  group_elems is a
 * non-zero multiple of 65536; with n_codebooks > 1, group_elems is a multiple
 * of segment_elems or divides it, so a group uses the codebooks of the
 * segments it covers.  depth is 2..32.
 *
 * splitzip_pipeline_sizes: bytes of the device work area (2 * depth slots)
 * and of the pinned host link buffer (depth slots, then one u64 per group:
 * the bytes it sent).  Returns SPLITZIP_OK or SPLITZIP_E_INVALID. */
int splitzip_pipeline_sizes(int dtype, size_t n_elems, uint32_t n_codebooks, size_t segment_elems,
                            size_t group_elems, uint32_t depth, size_t* d_work_bytes, size_t* h_link_bytes);

/* splitzip_pipeline_transfer: d_in (n_elems, device, 16-byte aligned) ->
 * d_out (device, 16-byte aligned).
 *   compress      1: groups travel compressed; 0: the raw groups travel the
 *                 same pipeline (the uncompressed baseline).
 *   d_work        device memory of d_work_bytes, 256-byte aligned.
 *   h_link        pinned host memory (hipHostMalloc with hipHostMallocCoherent,
 *                 so the encoder's size words reach the host at once) of
 *                 h_link_bytes, 256-byte aligned.
 *   d_status      optional device int32, as in splitzip_decompress.
 *   h_group_bytes optional host array of ceil(n / group_elems) entries: the
 *                 bytes each group sent over the link.
 *   streams       four distinct streams: encode, device-to-host copies,
 *                 host-to-device copies, decode.
 * Blocking: the calling thread drives the pipeline and returns after all four
 * streams are synchronized.  When no step can be queued it polls for 40 us,
 * then naps 20 us between polls; if no step can proceed for 60 s it returns
 * SPLITZIP_E_HIP.  The call creates 4 * depth HIP events (no timing) and
 * destroys them before it returns; it allocates no device or host buffer.
 * On an error return, work already queued may still run; synchronize the
 * streams before reusing the buffers.  Returns SPLITZIP_OK,
 * SPLITZIP_E_INVALID, SPLITZIP_E_CAPACITY, SPLITZIP_E_CODEBOOK or
 * SPLITZIP_E_HIP. */
int splitzip_pipeline_transfer(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                               uint32_t n_codebooks, size_t segment_elems, size_t group_elems, uint32_t depth,
                               int compress, void* d_work, size_t d_work_bytes, void* h_link, size_t h_link_bytes,
                               void* d_out, int32_t* d_status, uint64_t* h_group_bytes,
                               const hipStream_t streams[4]);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
