// The Dvec workspace of the allocating backward entry points: a small per-device cache of
// device buffers, reused across calls so that a call in steady state neither allocates nor
// makes the host wait for the GPU.
//
// Why not stream-ordered allocation: with this HIP runtime, hipFreeAsync of a block that
// hipMallocAsync has just recycled from a free still pending on the stream blocks the host
// until the stream reaches that free, i.e. until the previous call's kernels have finished, for
// the default pool and for private pools whatever their release threshold.  A backward that
// allocated per call that way held the host for the whole GPU step.
//
// Reuse is ordered on the GPU: each buffer carries an event recorded after the last kernel
// that read it; a call that takes a buffer whose event has not completed first makes its
// stream wait for that event (hipStreamWaitEvent, no host wait), so no call reads a buffer
// another call may still use, whichever streams and host threads are involved.  A call
// prefers a buffer that is idle or last used on its own stream, so one stream in a loop keeps
// reusing one buffer.  Under stream capture the lease falls back to stream-ordered allocation,
// which a graph records as allocation nodes.
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>

namespace fa {

// Buffers kept per device until the process ends; a request that finds none idle or last used
// on its stream, and no slot left, reuses the buffer whose last use is oldest (after a GPU-side
// wait), or replaces the smallest one (after a host wait: growth only) when none is large
// enough.
constexpr int kWorkspaceSlots = 4;
// Buffer sizes are rounded up to this many bytes, so nearby request sizes share a buffer.
constexpr size_t kWorkspaceGranule = size_t(1) << 20;

// One call's use of a workspace buffer.  acquire() holds the device's cache lock until
// release() (or the destructor), so take it after validation, release it right after the last
// kernel that reads the buffer has been enqueued, and enqueue nothing else in between.
class WorkspaceLease {
  public:
    WorkspaceLease() = default;
    WorkspaceLease(const WorkspaceLease&) = delete;
    WorkspaceLease& operator=(const WorkspaceLease&) = delete;
    ~WorkspaceLease() { (void)release(); }

    // A buffer of at least `bytes` bytes (bytes > 0) on the current device, usable by work
    // enqueued on `stream` after this returns.  On error nothing is held.
    hipError_t acquire(size_t bytes, hipStream_t stream);
    // Marks the buffer free once the work enqueued on the stream so far has finished.
    hipError_t release();
    float* ptr() const { return ptr_; }

  private:
    float* ptr_ = nullptr;
    hipStream_t stream_ = nullptr;
    int dev_ = -1;
    int slot_ = -1;        // cache slot, or -1 for a stream-ordered allocation
    bool held_ = false;
};

}  // namespace fa
