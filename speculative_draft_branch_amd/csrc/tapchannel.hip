// Tap mailbox on one GPU: slots allocated in advance by the caller, each with
// a sequence stamp; one-way writes and reads ordered by that stamp (rcap.io
// explainer, the TapChannel paragraph and its per-microbatch write /
// wait_and_read pseudo-code; evolve.pub review, "Frequently asked questions",
// what TapChannel is).
//
// Every write and read is three kernels in stream order. A single-thread
// decide kernel reads the slot header, takes the protocol decision and, when
// the call is accepted, claims the slot for that stamp (a field of the
// header); the copy kernel moves the payload only if the claim is in place;
// a single-thread commit kernel then publishes the stamp (write) or marks it
// consumed (read) and drops the claim. Kernel boundaries order the payload
// before the stamp. The decision is taken once, so a reader that marks a
// stamp consumed on another stream between a write's decision and its commit
// cannot make the commit publish a payload that was never copied; and a
// writer can claim the slot only after the reader has marked the current
// stamp consumed, which its commit kernel does after its copy.
//
// Header fields are written with ordinary (vector) global stores.
#include <algorithm>
#include <string>

#include "launch.hpp"
#include "tapchannel.h"

namespace ba {
namespace {

constexpr uint32_t kTapMagic = 0x54415031u;  // "TAP1"
constexpr size_t kTapHeaderBytes = 256;

struct TapHeader {
  uint64_t stamp;          // last committed stamp (0 = none)
  uint64_t consumed;       // last stamp the reader consumed
  uint64_t nbytes;         // bytes of the committed tap
  uint64_t capacity;       // payload bytes of the slot
  uint64_t write_claim;    // stamp of the write in flight (0 = none)
  uint64_t write_nbytes;   // its size
  uint64_t read_claim;     // stamp of the read in flight (0 = none)
  uint32_t magic;
  uint32_t pad;
};
static_assert(sizeof(TapHeader) <= kTapHeaderBytes, "header fits its 256 bytes");

__host__ __device__ inline int32_t write_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t stamp,
                                                  uint64_t nbytes, uint64_t capacity) {
  if (stamp <= slot_stamp) return BA_TAP_STALE;
  if (consumed < slot_stamp) return BA_TAP_BUSY;
  if (nbytes > capacity) return BA_TAP_TOO_BIG;
  return BA_TAP_OK;
}

__host__ __device__ inline int32_t read_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t expected,
                                                 uint64_t nbytes, uint64_t dst_bytes) {
  if (slot_stamp < expected) return BA_TAP_NOT_READY;
  if (slot_stamp > expected) return BA_TAP_SKIPPED;
  if (consumed >= expected) return BA_TAP_DUPLICATE;
  if (nbytes > dst_bytes) return BA_TAP_TOO_BIG;
  return BA_TAP_OK;
}

// Header loads that must see the latest value written by an earlier kernel.
__device__ __forceinline__ uint64_t ld(const uint64_t *p) { return __atomic_load_n(p, __ATOMIC_RELAXED); }

__global__ void tap_init_kernel(TapHeader *h, uint64_t capacity) {
  if (threadIdx.x != 0) return;
  h->stamp = 0;
  h->consumed = 0;
  h->nbytes = 0;
  h->capacity = capacity;
  h->write_claim = 0;
  h->write_nbytes = 0;
  h->read_claim = 0;
  h->magic = kTapMagic;
  h->pad = 0;
}

__global__ void tap_write_decide_kernel(TapHeader *h, uint64_t stamp, uint64_t nbytes, uint64_t capacity,
                                        int32_t *status) {
  if (threadIdx.x != 0) return;
  const uint64_t cap = min(capacity, ld(&h->capacity));
  int32_t st = write_decision(ld(&h->stamp), ld(&h->consumed), stamp, nbytes, cap);
  if (h->magic != kTapMagic) st = BA_TAP_NOT_READY;  // never initialised: refuse
  h->write_nbytes = st == BA_TAP_OK ? nbytes : 0;
  h->write_claim = st == BA_TAP_OK ? stamp : 0;
  *status = st;
}

__global__ void tap_write_commit_kernel(TapHeader *h, uint64_t stamp) {
  if (threadIdx.x != 0) return;
  if (ld(&h->write_claim) != stamp) return;
  h->nbytes = ld(&h->write_nbytes);
  h->stamp = stamp;
  h->write_claim = 0;
}

__global__ void tap_read_decide_kernel(TapHeader *h, uint64_t expected, uint64_t dst_bytes, int32_t *status,
                                       uint64_t *nbytes_out) {
  if (threadIdx.x != 0) return;
  const uint64_t n = ld(&h->nbytes);
  int32_t st = read_decision(ld(&h->stamp), ld(&h->consumed), expected, n, dst_bytes);
  if (h->magic != kTapMagic) st = BA_TAP_NOT_READY;
  h->read_claim = st == BA_TAP_OK ? expected : 0;
  *status = st;
  if (nbytes_out && st == BA_TAP_OK) *nbytes_out = n;
}

__global__ void tap_read_commit_kernel(TapHeader *h, uint64_t expected) {
  if (threadIdx.x != 0) return;
  if (ld(&h->read_claim) != expected) return;
  h->consumed = expected;
  h->read_claim = 0;
}

// Payload copy, only while the claim field holds `stamp`; the byte count comes
// from the header (at most `bound`). 16-byte chunks over a grid-stride loop,
// the last partial chunk byte by byte.
__global__ __launch_bounds__(256) void tap_copy_kernel(const TapHeader *h, int reading, uint64_t stamp,
                                                       const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                       uint64_t bound) {
  const uint64_t claim = reading ? ld(&h->read_claim) : ld(&h->write_claim);
  if (claim != stamp) return;
  const uint64_t n = min(reading ? ld(&h->nbytes) : ld(&h->write_nbytes), bound);
  const uint64_t chunks = n / 16;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
  uint4 *d4 = reinterpret_cast<uint4 *>(dst);
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride) d4[i] = s4[i];
  if (blockIdx.x == 0 && threadIdx.x < n % 16) dst[chunks * 16 + threadIdx.x] = src[chunks * 16 + threadIdx.x];
}

unsigned copy_grid(uint64_t bytes) {
  const uint64_t chunks = (bytes + 15) / 16;
  const uint64_t blocks = (chunks + 256 * 4 - 1) / (256 * 4);
  return (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(blocks, 4096));
}

ba_status_t tap_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return BA_OK;
  return set_error(BA_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

ba_status_t check_slot(const void *slot, size_t capacity) {
  if (!slot) return set_error(BA_EINVAL, "tap slot is NULL");
  if (reinterpret_cast<uintptr_t>(slot) % 256 != 0) return set_error(BA_EINVAL, "tap slot must be 256-byte aligned");
  if (capacity > ((uint64_t)1 << 46)) return set_error(BA_EINVAL, "tap capacity out of range");
  return BA_OK;
}

ba_status_t check_buf(const void *p, size_t bytes, const char *name) {
  if (bytes == 0) return BA_OK;
  if (!p) return set_error(BA_EINVAL, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return set_error(BA_EINVAL, std::string(name) + " is not 16-byte aligned");
  return BA_OK;
}

ba_status_t check_status_ptr(const int32_t *status) {
  if (!status) return set_error(BA_EINVAL, "status is NULL");
  if (reinterpret_cast<uintptr_t>(status) % 4 != 0) return set_error(BA_EINVAL, "status is not 4-byte aligned");
  return BA_OK;
}

}  // namespace
}  // namespace ba

using namespace ba;

extern "C" {

size_t ba_tap_slot_bytes(size_t capacity) { return kTapHeaderBytes + align_up(capacity, 256); }

ba_status_t ba_tap_slot_init(void *slot, size_t capacity, void *stream) {
  ba_status_t s = check_slot(slot, capacity);
  if (s != BA_OK) return s;
  tap_init_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(static_cast<TapHeader *>(slot), capacity);
  return tap_hip(hipGetLastError(), "tap slot init");
}

ba_status_t ba_tap_write(void *slot, size_t capacity, const void *src, size_t nbytes, uint64_t stamp, int32_t *status,
                         void *done_event, void *stream) {
  ba_status_t s = check_slot(slot, capacity);
  if (s == BA_OK) s = check_buf(src, nbytes, "tap source");
  if (s == BA_OK) s = check_status_ptr(status);
  if (s != BA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TapHeader *h = static_cast<TapHeader *>(slot);
  uint8_t *payload = static_cast<uint8_t *>(slot) + kTapHeaderBytes;
  tap_write_decide_kernel<<<1, 64, 0, st>>>(h, stamp, nbytes, capacity, status);
  s = tap_hip(hipGetLastError(), "tap write (decide)");
  if (s != BA_OK) return s;
  if (nbytes > 0 && nbytes <= capacity) {
    tap_copy_kernel<<<copy_grid(nbytes), 256, 0, st>>>(h, 0, stamp, static_cast<const uint8_t *>(src), payload, nbytes);
    s = tap_hip(hipGetLastError(), "tap write (copy)");
    if (s != BA_OK) return s;
  }
  tap_write_commit_kernel<<<1, 64, 0, st>>>(h, stamp);
  s = tap_hip(hipGetLastError(), "tap write (commit)");
  if (s != BA_OK || !done_event) return s;
  return tap_hip(hipEventRecord(static_cast<hipEvent_t>(done_event), st), "tap write (event record)");
}

ba_status_t ba_tap_read(void *slot, size_t capacity, void *dst, size_t dst_bytes, uint64_t expected, int32_t *status,
                        uint64_t *nbytes, void *stream) {
  ba_status_t s = check_slot(slot, capacity);
  if (s == BA_OK) s = check_buf(dst, dst_bytes, "tap destination");
  if (s == BA_OK) s = check_status_ptr(status);
  if (s == BA_OK && nbytes && reinterpret_cast<uintptr_t>(nbytes) % 8 != 0)
    s = set_error(BA_EINVAL, "nbytes is not 8-byte aligned");
  if (s != BA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TapHeader *h = static_cast<TapHeader *>(slot);
  const uint8_t *payload = static_cast<const uint8_t *>(slot) + kTapHeaderBytes;
  tap_read_decide_kernel<<<1, 64, 0, st>>>(h, expected, dst_bytes, status, nbytes);
  s = tap_hip(hipGetLastError(), "tap read (decide)");
  if (s != BA_OK) return s;
  const uint64_t bound = std::min<uint64_t>(dst_bytes, capacity);
  if (bound > 0) {
    tap_copy_kernel<<<copy_grid(bound), 256, 0, st>>>(h, 1, expected, payload, static_cast<uint8_t *>(dst), bound);
    s = tap_hip(hipGetLastError(), "tap read (copy)");
    if (s != BA_OK) return s;
  }
  tap_read_commit_kernel<<<1, 64, 0, st>>>(h, expected);
  return tap_hip(hipGetLastError(), "tap read (commit)");
}

ba_status_t ba_tap_wait_and_read(void *slot, size_t capacity, void *dst, size_t dst_bytes, uint64_t expected,
                                 int32_t *status, uint64_t *nbytes, void *written_event, void *stream) {
  if (!written_event) return set_error(BA_EINVAL, "written_event is NULL");
  ba_status_t s = check_slot(slot, capacity);
  if (s != BA_OK) return s;
  s = tap_hip(hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(written_event), 0),
              "tap wait (stream wait event)");
  if (s != BA_OK) return s;
  return ba_tap_read(slot, capacity, dst, dst_bytes, expected, status, nbytes, stream);
}

int32_t ba_tap_write_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t stamp, size_t nbytes,
                              size_t capacity) {
  return write_decision(slot_stamp, consumed, stamp, nbytes, capacity);
}

int32_t ba_tap_read_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t expected, uint64_t nbytes,
                             size_t dst_bytes) {
  return read_decision(slot_stamp, consumed, expected, nbytes, dst_bytes);
}

}  // extern "C"
