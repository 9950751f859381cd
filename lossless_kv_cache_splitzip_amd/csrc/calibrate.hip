// On-device calibration: exponent histograms and the top-16 codebook of each
// segment of a device tensor, the step the pages run offline ([TS]
// "Optimizacion": a codebook calibrated in advance avoids histogramming on
// the critical path; [TS] "Resultados" / "Calibracion"; [AB]).  Here it is
// measured on the GPU, and serves dynamic or per-tensor calibration.
//
// Three launches on the caller's stream:
//   calib_zero     clears the K x bins u64 histograms in the work area (a
//                  kernel, not a memset, so the sequence can be captured)
//   calib_hist     grid (blocks per segment, K): each workgroup counts its
//                  share of one segment into LDS histograms (one copy per
//                  lane slot, so lanes of a wave rarely hit one address) and
//                  adds its non-zero bins to the segment's histogram with
//                  relaxed device-scope atomics
//   calib_select   one workgroup per segment: rank of every exponent by
//                  (count descending, exponent ascending); ranks 0..15 form
//                  the codebook, so unseen exponents fill up in ascending
//                  order (the same order as splitzip_calibrate on the host)
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "splitzip.h"

namespace {

constexpr int kHistThreads = 512;
constexpr uint64_t kElemsPerRange = 65536;  // elements per calib_hist step
constexpr uint32_t kMaxBlocksPerSeg = 8192;  // workgroups per segment; more ranges loop
// ranges per workgroup (grid-stride): fewer workgroups clear, reduce and add
// their histograms (1 -> 4 measured -4% BF16, -7% E5M2 on the 1 and 2.5 GiB caches)
constexpr uint64_t kRangesPerBlock = 4;
// ... but at least about this many workgroups in all (down to one range
// each) when there are few segments: one 4 MiB layer 26.7 -> 17.2 us
constexpr uint64_t kTargetWgs = 1024;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

uint64_t divup_u64(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(256) void calib_zero_kernel(uint64_t* hist, uint32_t words) {
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) hist[i] = 0;
}

// BF16: 256 bins x 32 copies (lane & 31); E5M2: 32 bins x 64 copies (lane).
template <bool kBf16>
__global__ __launch_bounds__(kHistThreads) void calib_hist_kernel(const uint8_t* in, uint64_t n, uint64_t seg,
                                                                  uint64_t* hist) {
  constexpr uint32_t kBins = kBf16 ? 256 : 32, kCopies = kBf16 ? 32 : 64;
  __shared__ uint32_t h[kBins * kCopies];
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < kBins * kCopies; i += kHistThreads) h[i] = 0;
  __syncthreads();
  const uint64_t k = blockIdx.y;
  const uint64_t seg_lo = k * seg, seg_hi = std::min<uint64_t>(n, seg_lo + seg);
  const uint32_t copy = tid & (kCopies - 1);
  for (uint64_t lo = seg_lo + (uint64_t)blockIdx.x * kElemsPerRange; lo < seg_hi;
       lo += (uint64_t)gridDim.x * kElemsPerRange) {
    const uint64_t hi = std::min<uint64_t>(seg_hi, lo + kElemsPerRange);
    // 16-byte loads where the whole word is inside [lo, hi), else elements
    constexpr uint32_t kPer = kBf16 ? 8 : 16;  // elements per 16 bytes
    const uint64_t first_word = (lo + kPer - 1) / kPer, last_word = hi / kPer;
    for (uint64_t e = lo + tid; e < std::min<uint64_t>(hi, first_word * kPer); e += kHistThreads) {
      const uint32_t x = kBf16 ? (uint32_t)reinterpret_cast<const uint16_t*>(in)[e] >> 7 : (uint32_t)in[e] >> 2;
      atomicAdd(&h[((x & (kBins - 1)) * kCopies) | copy], 1u);
    }
    const uint4* w = reinterpret_cast<const uint4*>(in);
    for (uint64_t i = first_word + tid; i < last_word; i += kHistThreads) {
      // read once: non-temporal (1 GiB, 32 segments: 192 -> 171 us; inputs that
      // fit the memory-side cache lose its reuse between back-to-back calls)
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w + i));
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kBf16) {
          atomicAdd(&h[(((q[j] >> 7) & 0xFFu) * kCopies) | copy], 1u);
          atomicAdd(&h[(((q[j] >> 23) & 0xFFu) * kCopies) | copy], 1u);
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) atomicAdd(&h[(((q[j] >> (8 * b + 2)) & 0x1Fu) * kCopies) | copy], 1u);
        }
      }
    }
    for (uint64_t e = std::max<uint64_t>(last_word * kPer, first_word * kPer) + tid; e < hi; e += kHistThreads) {
      const uint32_t x = kBf16 ? (uint32_t)reinterpret_cast<const uint16_t*>(in)[e] >> 7 : (uint32_t)in[e] >> 2;
      atomicAdd(&h[((x & (kBins - 1)) * kCopies) | copy], 1u);
    }
  }
  __syncthreads();
  if (tid < kBins) {
    uint32_t c = 0;
    for (uint32_t j = 0; j < kCopies; ++j) c += h[tid * kCopies + ((j + tid) & (kCopies - 1))];
    if (c) __hip_atomic_fetch_add(&hist[k * kBins + tid], (uint64_t)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(256) void calib_select_kernel(const uint64_t* hist, uint32_t bins, uint8_t* codebooks) {
  __shared__ uint64_t cnt[256];
  const uint32_t t = threadIdx.x;
  const uint64_t k = blockIdx.x;
  if (t < bins) cnt[t] = __hip_atomic_load(&hist[k * bins + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (t >= bins) return;
  const uint64_t c = cnt[t];
  uint32_t rank = 0;
  for (uint32_t u = 0; u < bins; ++u) rank += (cnt[u] > c || (cnt[u] == c && u < t)) ? 1u : 0u;
  if (rank < 16) codebooks[16 * k + rank] = (uint8_t)t;
}

}  // namespace

extern "C" {

size_t splitzip_calibrate_device_work_bytes(int dtype, uint32_t n_codebooks) {
  if ((dtype != SPLITZIP_BF16 && dtype != SPLITZIP_FP8_E5M2) || n_codebooks == 0 || n_codebooks > 65535) return 0;
  return (size_t)n_codebooks * (dtype == SPLITZIP_BF16 ? 256 : 32) * 8;
}

int splitzip_calibrate_device(int dtype, const void* d_samples, size_t n_elems, size_t segment_elems,
                              uint32_t n_codebooks, uint8_t* d_codebooks_out, void* d_work, size_t work_bytes,
                              hipStream_t stream) {
  const size_t need = splitzip_calibrate_device_work_bytes(dtype, n_codebooks);
  if (need == 0 || n_elems > (1ull << 36) || (d_samples == nullptr && n_elems > 0) || d_codebooks_out == nullptr ||
      d_work == nullptr || (reinterpret_cast<uintptr_t>(d_samples) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(d_work) & 7) != 0)
    return SPLITZIP_E_INVALID;
  const uint64_t seg = n_codebooks == 1 ? std::max<uint64_t>(n_elems, 1) : segment_elems;
  if (seg == 0 || (uint64_t)n_codebooks * seg < n_elems) return SPLITZIP_E_INVALID;
  const uint64_t ranges = divup_u64(seg, kElemsPerRange);
  const uint64_t blocks = std::min<uint64_t>(
      kMaxBlocksPerSeg, std::min<uint64_t>(ranges, std::max<uint64_t>(divup_u64(ranges, kRangesPerBlock),
                                                                       divup_u64(kTargetWgs, n_codebooks))));
  if (work_bytes < need) return SPLITZIP_E_CAPACITY;
  const uint32_t bins = dtype == SPLITZIP_BF16 ? 256 : 32;
  uint64_t* hist = static_cast<uint64_t*>(d_work);
  const uint32_t words = n_codebooks * bins;
  calib_zero_kernel<<<(words + 255) / 256, 256, 0, stream>>>(hist, words);
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  if (n_elems > 0) {
    const dim3 grid((uint32_t)blocks, n_codebooks);
    const uint8_t* in = static_cast<const uint8_t*>(d_samples);
    if (dtype == SPLITZIP_BF16) calib_hist_kernel<true><<<grid, kHistThreads, 0, stream>>>(in, n_elems, seg, hist);
    else calib_hist_kernel<false><<<grid, kHistThreads, 0, stream>>>(in, n_elems, seg, hist);
    if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  }
  calib_select_kernel<<<n_codebooks, 256, 0, stream>>>(hist, bins, d_codebooks_out);
  if (hipGetLastError() != hipSuccess) return SPLITZIP_E_HIP;
  return SPLITZIP_OK;
}

}  // extern "C"
