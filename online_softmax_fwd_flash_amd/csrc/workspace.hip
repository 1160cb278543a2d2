// Per-device cache of backward workspace buffers; the rules are stated in workspace.h.
#include <mutex>

#include "kernels.h"
#include "workspace.h"

namespace fa {

namespace {

struct Slot {
    float* ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;   // recorded after the last kernel that read the buffer
    hipStream_t last_stream = nullptr;
    unsigned long long last_use = 0;
};

struct DeviceCache {
    std::mutex mu;
    Slot slot[kWorkspaceSlots];
    unsigned long long uses = 0;
};

DeviceCache g_cache[kMaxDeviceSlots];

size_t round_up(size_t bytes) {
    return (bytes + kWorkspaceGranule - 1) / kWorkspaceGranule * kWorkspaceGranule;
}

// Fills an empty slot with a new buffer and its event.
hipError_t fill(Slot& s, size_t bytes) {
    const size_t want = round_up(bytes);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, want);
    if (e != hipSuccess) return e;
    hipEvent_t ev = nullptr;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return e;
    }
    s.ptr = static_cast<float*>(p);
    s.bytes = want;
    s.done = ev;
    return hipSuccess;
}

// Frees a slot's buffer once its last use has finished (host wait: only on growth).
hipError_t empty(Slot& s) {
    hipError_t e = hipEventSynchronize(s.done);
    if (e != hipSuccess) return e;
    e = hipFree(s.ptr);
    const hipError_t e2 = hipEventDestroy(s.done);
    s = Slot();
    return e != hipSuccess ? e : e2;
}

}  // namespace

hipError_t WorkspaceLease::acquire(size_t bytes, hipStream_t stream) {
    if (held_) return hipErrorInvalidValue;
    if (bytes == 0) return hipErrorInvalidValue;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        // a graph records this pair as allocation nodes; nothing runs now
        void* p = nullptr;
        e = hipMallocAsync(&p, bytes, stream);
        if (e != hipSuccess) return e;
        ptr_ = static_cast<float*>(p);
        stream_ = stream;
        slot_ = -1;
        held_ = true;
        return hipSuccess;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDeviceSlots) return hipErrorInvalidDevice;
    DeviceCache& c = g_cache[dev];
    c.mu.lock();
    // 1. a large enough buffer whose last use has finished: no wait at all
    // 2. a large enough buffer last used on this stream: the wait is already in stream order
    //    (it is still enqueued, in case the handle now names another stream)
    // 3. an empty slot: a new buffer
    // 4. the large enough buffer used longest ago: the stream waits for it on the GPU
    // 5. otherwise the smallest buffer is replaced by a larger one
    int pick = -1, same_stream = -1, empty_slot = -1, oldest_fit = -1, smallest = -1;
    for (int i = 0; i < kWorkspaceSlots && pick < 0; ++i) {
        Slot& s = c.slot[i];
        if (s.ptr == nullptr) {
            if (empty_slot < 0) empty_slot = i;
            continue;
        }
        if (smallest < 0 || s.bytes < c.slot[smallest].bytes) smallest = i;
        if (s.bytes < bytes) continue;
        const hipError_t q = hipEventQuery(s.done);
        if (q == hipSuccess) {
            pick = i;
        } else if (q == hipErrorNotReady) {
            if (s.last_stream == stream && same_stream < 0) same_stream = i;
            if (oldest_fit < 0 || s.last_use < c.slot[oldest_fit].last_use) oldest_fit = i;
        } else {
            c.mu.unlock();
            return q;
        }
    }
    bool wait = false;
    if (pick < 0 && same_stream >= 0) {
        pick = same_stream;
        wait = true;
    } else if (pick < 0 && empty_slot >= 0) {
        e = fill(c.slot[empty_slot], bytes);
        pick = empty_slot;
    } else if (pick < 0 && oldest_fit >= 0) {
        pick = oldest_fit;
        wait = true;
    } else if (pick < 0) {
        e = empty(c.slot[smallest]);
        if (e == hipSuccess) e = fill(c.slot[smallest], bytes);
        pick = smallest;
    }
    if (e == hipSuccess && wait) e = hipStreamWaitEvent(stream, c.slot[pick].done, 0);
    if (e != hipSuccess) {
        c.mu.unlock();
        return e;
    }
    ptr_ = c.slot[pick].ptr;
    stream_ = stream;
    dev_ = dev;
    slot_ = pick;
    held_ = true;
    return hipSuccess;
}

hipError_t WorkspaceLease::release() {
    if (!held_) return hipSuccess;
    held_ = false;
    if (slot_ < 0) {
        const hipError_t e = hipFreeAsync(ptr_, stream_);
        ptr_ = nullptr;
        return e;
    }
    DeviceCache& c = g_cache[dev_];
    Slot& s = c.slot[slot_];
    hipError_t e = hipEventRecord(s.done, stream_);
    if (e != hipSuccess) {
        // the event no longer marks the buffer's last use: wait for the stream, so the buffer
        // is idle before anyone else takes it
        (void)hipStreamSynchronize(stream_);
    }
    s.last_stream = stream_;
    s.last_use = ++c.uses;
    ptr_ = nullptr;
    c.mu.unlock();
    return e;
}

}  // namespace fa
