// rcs_internal.h -- calls shared between the library's own source files; not
// part of the C ABI.
#ifndef RCS_INTERNAL_H
#define RCS_INTERNAL_H

// Drops the events ckpt_pack_async keeps for a snapshot buffer of device dev
// (call before freeing the buffer; no copy out of it may still be pending).
void rcs_snapshot_forget(int dev, const void *snapshot);

#endif
