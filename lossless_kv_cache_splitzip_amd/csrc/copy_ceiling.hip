// Measurement kernels for the benchmark's bandwidth ceiling: a plain device
// copy and a read-only pass with the same access shape as the codec's
// streaming kernels at their best (one 16-byte access per lane, consecutive
// lanes on consecutive 16 bytes, non-temporal, 256-thread workgroups).  They
// carry no codec arithmetic; the benchmark times them next to the codec to
// give "fraction of what this GPU's HBM delivers to such a kernel", and the
// counter runs use the copy's known byte count to scale the L2-to-memory
// request counters into bytes.
//
// Built into its own library (libszceiling.so), loaded only by bench.py.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// One 16-byte word per thread; the last workgroup may be partial.
__global__ __launch_bounds__(kThreads) void copy16_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                          uint64_t words) {
  const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < words) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read-only: every word is loaded; a word that equals the key (never, for
// the benchmark's data) is counted, so the loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void read16_kernel(const u32x4_t* __restrict__ src, uint64_t words,
                                                          uint32_t* __restrict__ hits, uint32_t key) {
  const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= words) return;
  const u32x4_t v = __builtin_nontemporal_load(src + i);
  if ((v.x ^ v.y ^ v.z ^ v.w) == key && v.x == key) atomicAdd(hits, 1u);
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) from src
// to dst on `stream`.  Returns 0, -1 for bad arguments, -5 for a failed
// launch.  At most 2^32 - 1 workgroups (64 TiB).
int szceiling_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15) ||
      (bytes > 0 && (src == nullptr || dst == nullptr)))
    return -1;
  const uint64_t words = bytes / 16, groups = (words + kThreads - 1) / kThreads;
  if (groups == 0) return 0;
  if (groups > 0xFFFFFFFFull) return -1;
  copy16_kernel<<<(uint32_t)groups, kThreads, 0, stream>>>(static_cast<const u32x4_t*>(src),
                                                           static_cast<u32x4_t*>(dst), words);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) on `stream`; *hits (a
// device word, 4-byte aligned) counts words whose first lane equals the XOR
// of all four and equals `key`.
int szceiling_read(const void* src, size_t bytes, uint32_t* hits, uint32_t key, hipStream_t stream) {
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) || hits == nullptr ||
      (reinterpret_cast<uintptr_t>(hits) & 3) || (bytes > 0 && src == nullptr))
    return -1;
  const uint64_t words = bytes / 16, groups = (words + kThreads - 1) / kThreads;
  if (groups == 0) return 0;
  if (groups > 0xFFFFFFFFull) return -1;
  read16_kernel<<<(uint32_t)groups, kThreads, 0, stream>>>(static_cast<const u32x4_t*>(src), words, hits, key);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
