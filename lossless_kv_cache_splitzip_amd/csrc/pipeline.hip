// Chunk-pipelined transfer of a tensor through a host "link": the tensor is
// cut into groups of whole chunks; each group is compressed on the GPU,
// copied to pinned host memory and back by the copy engines, and
// decompressed, with up to `depth` groups in flight.  This is the single-GPU
// stand-in for the pages' prefill-to-decode transfer: the codec shrinks the
// bytes that cross a 50-100 GB/s link ([TS] "Planteamiento del Problema";
// [TS] "Resultados": 1.22-1.32x faster transfers, codec about 7% of the
// transfer time at 64K tokens).  compress = 0 sends the raw groups through
// the same pipeline, the baseline of that comparison.
//
// The calling thread drives the pipeline as a state machine: it queues each
// step of a group once the host has seen, by querying events, that the
// step's inputs are complete and its ring slot is free, so no stream ever
// waits on another (cross-stream event waits cost up to a millisecond each
// between copy-engine queues on this system).  When no step can be queued,
// the thread polls for a short while (the next step is often moments away)
// and then naps between polls, so it does not hold a host core for the
// whole transfer (waiting in hipEventSynchronize, even on blocking-sync
// events, kept a core busy).  A compressed group's size exists only on the
// device: the encoder writes it into the pinned link buffer, where the host
// reads it before queuing the group's copies.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <chrono>
#include <thread>
#include <vector>

#include "splitzip.h"

namespace {

constexpr uint64_t kChunkElems = 65536;

uint64_t round_up256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct Plan {
  uint64_t groups = 0, slot = 0;  // group count, bytes per ring slot
  uint32_t cb_per_group = 1;      // codebooks a full group carries
};

// Groups hold whole chunks; with K > 1 codebooks a group holds whole segments
// or lies inside one segment, so each group is a valid stream of its own.
int plan_of(int dtype, size_t n, uint32_t k, size_t seg, size_t group, uint32_t depth, Plan* p) {
  if ((dtype != SPLITZIP_BF16 && dtype != SPLITZIP_FP8_E5M2) || k == 0 || depth < 2 || depth > 32 || group == 0 ||
      group % kChunkElems != 0)
    return SPLITZIP_E_INVALID;
  if (k > 1) {
    if (seg == 0 || seg % kChunkElems != 0 || (seg % group != 0 && group % seg != 0)) return SPLITZIP_E_INVALID;
    if ((uint64_t)k * seg < n) return SPLITZIP_E_INVALID;
    p->cb_per_group = group % seg == 0 ? (uint32_t)(group / seg) : 1u;
  }
  const size_t elem = dtype == SPLITZIP_BF16 ? 2 : 1;
  const size_t stream = splitzip_max_compressed_size(dtype, group, p->cb_per_group);
  if (stream == 0) return SPLITZIP_E_INVALID;
  p->groups = (n + group - 1) / group;
  p->slot = round_up256(std::max<size_t>(stream, group * elem));
  return SPLITZIP_OK;
}

struct Events {
  std::vector<hipEvent_t> e;
  ~Events() {
    for (hipEvent_t x : e)
      if (x) (void)hipEventDestroy(x);
  }
};

}  // namespace

extern "C" {

int splitzip_pipeline_sizes(int dtype, size_t n_elems, uint32_t n_codebooks, size_t segment_elems,
                            size_t group_elems, uint32_t depth, size_t* d_work_bytes, size_t* h_link_bytes) {
  Plan p;
  const int rc = plan_of(dtype, n_elems, n_codebooks, segment_elems, group_elems, depth, &p);
  if (rc != SPLITZIP_OK) return rc;
  if (d_work_bytes) *d_work_bytes = 2 * (size_t)depth * p.slot;
  if (h_link_bytes) *h_link_bytes = (size_t)depth * p.slot + round_up256(8 * p.groups);
  return SPLITZIP_OK;
}

int splitzip_pipeline_transfer(int dtype, const void* d_in, size_t n_elems, const uint8_t* h_codebooks,
                               uint32_t n_codebooks, size_t segment_elems, size_t group_elems, uint32_t depth,
                               int compress, void* d_work, size_t d_work_bytes, void* h_link, size_t h_link_bytes,
                               void* d_out, int32_t* d_status, uint64_t* h_group_bytes,
                               const hipStream_t streams[4]) {
  Plan p;
  int rc = plan_of(dtype, n_elems, n_codebooks, segment_elems, group_elems, depth, &p);
  if (rc != SPLITZIP_OK) return rc;
  if (streams == nullptr || h_link == nullptr || d_work == nullptr || h_codebooks == nullptr ||
      (n_elems > 0 && (d_in == nullptr || d_out == nullptr)) || (reinterpret_cast<uintptr_t>(d_in) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(d_out) & 15) != 0 || (reinterpret_cast<uintptr_t>(h_link) & 255) != 0 ||
      (reinterpret_cast<uintptr_t>(d_work) & 255) != 0)
    return SPLITZIP_E_INVALID;
  if (d_work_bytes < 2 * (size_t)depth * p.slot || h_link_bytes < (size_t)depth * p.slot + round_up256(8 * p.groups))
    return SPLITZIP_E_CAPACITY;
  if (n_elems == 0) return SPLITZIP_OK;

  const hipStream_t s_enc = streams[0], s_d2h = streams[1], s_h2d = streams[2], s_dec = streams[3];
  const size_t elem = dtype == SPLITZIP_BF16 ? 2 : 1;
  uint8_t* send = static_cast<uint8_t*>(d_work);
  uint8_t* recv = send + depth * p.slot;
  uint8_t* host = static_cast<uint8_t*>(h_link);
  // bytes each group sends; the encoder writes compressed sizes here
  volatile uint64_t* sizes = reinterpret_cast<volatile uint64_t*>(host + depth * p.slot);
  const uint8_t* in = static_cast<const uint8_t*>(d_in);
  uint8_t* out = static_cast<uint8_t*>(d_out);

  // ring events: [0] compressed, [1] copied to host, [2] copied back, [3] decoded
  Events ev;
  ev.e.assign(4 * (size_t)depth, nullptr);
  for (hipEvent_t& x : ev.e)
    if (hipEventCreateWithFlags(&x, hipEventDisableTiming) != hipSuccess) return SPLITZIP_E_HIP;
  auto E = [&](int kind, uint64_t g) { return ev.e[4 * (g % depth) + kind]; };
  auto record = [&](int kind, uint64_t g, hipStream_t st) { return hipEventRecord(E(kind, g), st) == hipSuccess; };
  hipError_t qerr = hipSuccess;
  auto done = [&](int kind, uint64_t g) {  // step `kind` of group g has completed
    const hipError_t q = hipEventQuery(E(kind, g));
    if (q != hipSuccess && q != hipErrorNotReady) qerr = q;
    return q == hipSuccess;
  };

  auto group_n = [&](uint64_t g) { return std::min<uint64_t>(group_elems, n_elems - g * group_elems); };
  auto codebooks_of = [&](uint64_t g, const uint8_t** cb, uint32_t* k, size_t* seg) {
    const uint64_t first = g * group_elems;
    if (n_codebooks == 1) {
      *cb = h_codebooks, *k = 1, *seg = 0;
    } else if (group_elems % segment_elems == 0) {  // whole segments
      *cb = h_codebooks + 16 * (first / segment_elems);
      *k = (uint32_t)((group_n(g) + segment_elems - 1) / segment_elems);
      *seg = *k > 1 ? segment_elems : 0;
    } else {  // inside one segment
      *cb = h_codebooks + 16 * (first / segment_elems), *k = 1, *seg = 0;
    }
  };
  std::vector<uint64_t> moved(p.groups, 0);  // bytes each group's copies move

  // next group to take each step: compress, copy out, copy back, decode
  uint64_t nc = 0, nd = 0, nh = 0, nx = 0;
  const uint64_t G = p.groups;
  // after a step was queued, poll this long before napping between polls
  constexpr auto kPoll = std::chrono::microseconds(40);
  constexpr auto kNap = std::chrono::microseconds(20);
  // a step that makes no progress for this long means the device stopped
  // answering: give up rather than wait forever
  constexpr auto kStall = std::chrono::seconds(60);
  auto last_progress = std::chrono::steady_clock::now();
  while (compress ? nx < G : nh < G) {
    bool progress = false;
    // compress g: its send slot is free once group g - depth was copied out
    if (nc < G && (nc < depth || nd > nc - depth) && (nc < depth || done(1, nc - depth))) {
      const uint64_t g = nc, slot = g % depth;
      if (compress) {
        sizes[g] = 0;
        const uint8_t* cb;
        uint32_t k;
        size_t seg;
        codebooks_of(g, &cb, &k, &seg);
        rc = splitzip_compress(dtype, in + g * group_elems * elem, group_n(g), cb, k, seg, send + slot * p.slot,
                               p.slot, const_cast<uint64_t*>(sizes + g), s_enc);
        if (rc != SPLITZIP_OK) return rc;
      } else {
        sizes[g] = group_n(g) * elem;
      }
      if (!record(0, g, s_enc)) return SPLITZIP_E_HIP;
      ++nc, progress = true;
    }
    // copy g to host: once compressed, and once group g - depth has been
    // copied back out of the host slot
    if (nd < nc && (nd < depth || nh > nd - depth) && done(0, nd) && (nd < depth || done(2, nd - depth))) {
      const uint64_t g = nd, slot = g % depth;
      const uint64_t bytes = sizes[g];
      if (bytes == 0 || bytes > p.slot) return SPLITZIP_E_HIP;
      // whole 256-byte blocks (the slots have room): sizes that are not a
      // multiple of 4 sent the copy engines down a much slower path
      moved[g] = compress ? round_up256(bytes) : bytes;
      if (h_group_bytes) h_group_bytes[g] = bytes;
      const void* src = compress ? static_cast<const void*>(send + slot * p.slot) : in + g * group_elems * elem;
      if (hipMemcpyAsync(host + slot * p.slot, src, moved[g], hipMemcpyDeviceToHost, s_d2h) != hipSuccess ||
          !record(1, g, s_d2h))
        return SPLITZIP_E_HIP;
      ++nd, progress = true;
    }
    // copy g back: once on the host, and once group g - depth has been decoded
    // out of the receive slot
    if (nh < nd && done(1, nh) && (!compress || nh < depth || (nx > nh - depth && done(3, nh - depth)))) {
      const uint64_t g = nh, slot = g % depth;
      void* dst = compress ? static_cast<void*>(recv + slot * p.slot) : out + g * group_elems * elem;
      if (hipMemcpyAsync(dst, host + slot * p.slot, moved[g], hipMemcpyHostToDevice, s_h2d) != hipSuccess ||
          !record(2, g, s_h2d))
        return SPLITZIP_E_HIP;
      ++nh, progress = true;
    }
    // decode g: once copied back
    if (compress && nx < nh && done(2, nx)) {
      const uint64_t g = nx, slot = g % depth;
      rc = splitzip_decompress(recv + slot * p.slot, moved[g], dtype, group_n(g), out + g * group_elems * elem,
                               d_status, s_dec);
      if (rc != SPLITZIP_OK) return rc;
      if (!record(3, g, s_dec)) return SPLITZIP_E_HIP;
      ++nx, progress = true;
    }
    if (qerr != hipSuccess) return SPLITZIP_E_HIP;
    if (progress) {
      last_progress = std::chrono::steady_clock::now();
    } else {
      const auto idle = std::chrono::steady_clock::now() - last_progress;
      if (idle > kStall) return SPLITZIP_E_HIP;
      if (idle < kPoll) std::this_thread::yield();
      else std::this_thread::sleep_for(kNap);
    }
  }
  for (int i = 0; i < 4; ++i)
    if (hipStreamSynchronize(streams[i]) != hipSuccess) return SPLITZIP_E_HIP;
  return SPLITZIP_OK;
}

}  // extern "C"
