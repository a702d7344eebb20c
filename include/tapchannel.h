/*
 * tapchannel.h -- one-GPU part of the tap mailbox (C ABI, libbranch_attn.so).
 *
 * A draft model co-trained beside a pipelined target reads "taps", the
 * target's intermediate hidden states, from every pipeline stage. Each source
 * stage owns a mailbox slot that is allocated in advance in the draft stage's
 * memory; after its forward pass of a microbatch the source writes that
 * microbatch's tap into the slot, and the draft stage reads it before its own
 * forward. The data flows one way (no gradient comes back), and a sequence
 * stamp orders writes and reads (rcap.io explainer, the TapChannel paragraph
 * and the per-microbatch write / wait_and_read pseudo-code; evolve.pub review,
 * "Frequently asked questions", what TapChannel is). The transport between
 * GPUs (IPC mappings, RDMA) is not part of this library: here the slot, the
 * source buffer and the destination buffer are device memory of one GPU, and
 * producer and consumer are streams ordered by events.
 *
 * Protocol (the reading this library implements). A slot holds the stamp of
 * its last committed tap (0 = none yet) and the last stamp its reader
 * consumed. Stamps of one slot increase strictly; the first is >= 1.
 *   write(stamp): accepted iff stamp > the slot's stamp, the slot's stamp has
 *     been consumed (the writer never overwrites an unread tap), and the tap
 *     fits. Then the payload is copied and, after it, the stamp committed.
 *     A stamp above the slot's stamp + 1 is accepted: the reader sees the gap.
 *   read(expected): accepted iff the slot's stamp equals expected and that
 *     stamp has not been consumed yet, and the destination is large enough;
 *     then the payload is copied out and, after it, the stamp is marked
 *     consumed. Otherwise the status says why: NOT_READY (the slot still holds
 *     an older stamp), SKIPPED (it holds a newer one: the expected tap was
 *     never written), DUPLICATE (the expected stamp was already consumed).
 * A rejected call changes neither the slot nor the destination.
 * A slot that was never initialised (ba_tap_slot_init) refuses every write and
 * read with NOT_READY.
 *
 * Each call enqueues three small kernels on the caller's stream (decide,
 * copy, commit); statuses are decided on the device when the work runs and
 * are written to the caller's int32 status word. One writer and one reader per
 * slot; the writer's and reader's streams are ordered through events (see
 * ba_tap_wait_and_read). Slots, payloads and status words are ordinary
 * (coarse-grained) device memory owned by the caller; the library allocates
 * nothing. All device pointers must be 16-byte aligned; slots 256-byte aligned.
 */
#ifndef TAPCHANNEL_H
#define TAPCHANNEL_H

#include <stddef.h>
#include <stdint.h>

#include "branch_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_TAP_OK = 0,
  BA_TAP_NOT_READY = 1,  /* read: the slot holds an older stamp than expected */
  BA_TAP_SKIPPED = 2,    /* read: the slot holds a newer stamp; the expected one never arrived */
  BA_TAP_DUPLICATE = 3,  /* read: the expected stamp was already consumed */
  BA_TAP_STALE = 4,      /* write: the stamp does not exceed the slot's stamp */
  BA_TAP_BUSY = 5,       /* write: the slot's current tap has not been consumed */
  BA_TAP_TOO_BIG = 6     /* write: more bytes than the slot holds; read: more than the destination holds */
} ba_tap_status_t;

/* Bytes of device memory a slot of `capacity` payload bytes occupies: a
 * 256-byte header plus the payload rounded up to 256 bytes. */
size_t ba_tap_slot_bytes(size_t capacity);

/* Enqueue the initialisation of a slot (stamp 0, nothing consumed). The slot
 * must not be in use by other work. BA_EINVAL for a NULL or misaligned slot. */
ba_status_t ba_tap_slot_init(void *slot, size_t capacity, void *stream);

/* Enqueue a write of `nbytes` bytes from `src` (device) into the slot under
 * `stamp`; *status (device int32) receives the ba_tap_status_t. If
 * `done_event` is not NULL it is recorded on the stream after the commit, so
 * a reader's stream can wait for it (a hipEvent_t). */
ba_status_t ba_tap_write(void *slot, size_t capacity, const void *src, size_t nbytes, uint64_t stamp,
                         int32_t *status, void *done_event, void *stream);

/* Enqueue a read of the tap stamped `expected` into `dst` (device, dst_bytes
 * large); *status (device int32) receives the ba_tap_status_t and *nbytes
 * (device uint64, may be NULL) the tap's size on success. */
ba_status_t ba_tap_read(void *slot, size_t capacity, void *dst, size_t dst_bytes, uint64_t expected,
                        int32_t *status, uint64_t *nbytes, void *stream);

/* The rendezvous of the draft side: make `stream` wait for `written_event`
 * (recorded after the producer's ba_tap_write, on the producer's stream), then
 * enqueue ba_tap_read. No kernel spins: the wait is a stream dependency. */
ba_status_t ba_tap_wait_and_read(void *slot, size_t capacity, void *dst, size_t dst_bytes, uint64_t expected,
                                 int32_t *status, uint64_t *nbytes, void *written_event, void *stream);

/* The protocol's decisions as host functions (the kernels make the same ones):
 * the status a write or read would get against a slot whose last committed
 * stamp is slot_stamp and whose last consumed stamp is consumed. */
int32_t ba_tap_write_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t stamp, size_t nbytes,
                              size_t capacity);
int32_t ba_tap_read_decision(uint64_t slot_stamp, uint64_t consumed, uint64_t expected, uint64_t nbytes,
                             size_t dst_bytes);

#ifdef __cplusplus
}
#endif
#endif /* TAPCHANNEL_H */
