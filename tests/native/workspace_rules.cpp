// Host-only check of the backward's workspace cache (csrc/workspace.hip): the HIP runtime
// calls it makes are replaced by stand-ins defined here, whose events stay pending until the
// test says their stream has finished, so every rule of the cache is taken deterministically:
// an idle buffer, a buffer last used on the caller's stream, a new slot, the oldest pending
// buffer behind a GPU-side wait, replacement of the smallest buffer (the only host wait), the
// capture fallback and the error paths.  Prints "workspace-rules ok" on success.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <set>
#include <thread>
#include <vector>

#include "workspace.h"

namespace {

struct FakeEvent {
    bool pending = false;
    hipStream_t stream = nullptr;
};

int g_device = 0;
hipStream_t g_capturing = nullptr;   // the stream under capture, if any
bool g_fail_malloc = false, g_fail_record = false;
int g_mallocs = 0, g_frees = 0, g_async_mallocs = 0, g_async_frees = 0, g_host_waits = 0,
    g_stream_syncs = 0;
std::set<void*> g_live;
std::vector<std::pair<hipStream_t, FakeEvent*>> g_waits;   // hipStreamWaitEvent log
std::vector<FakeEvent*> g_events;
std::mutex g_mu;   // the stand-ins may be called from two threads in the lock test

hipStream_t stream(int i) { return reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(0x1000 + 16 * i)); }

// the GPU reached the end of everything enqueued on s so far
void finish(hipStream_t s) {
    std::lock_guard<std::mutex> l(g_mu);
    for (FakeEvent* e : g_events)
        if (e->stream == s) e->pending = false;
}

int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::printf("CHECK failed line %d: %s\n", __LINE__, #c);    \
            ++failures;                                                  \
        }                                                                \
    } while (0)

}  // namespace

extern "C" {

hipError_t hipGetDevice(int* d) {
    *d = g_device;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t s, hipStreamCaptureStatus* st) {
    *st = (g_capturing != nullptr && s == g_capturing) ? hipStreamCaptureStatusActive
                                                       : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t bytes) {
    std::lock_guard<std::mutex> l(g_mu);
    if (g_fail_malloc) return hipErrorOutOfMemory;
    *p = std::malloc(bytes);
    g_live.insert(*p);
    ++g_mallocs;
    return hipSuccess;
}
hipError_t hipFree(void* p) {
    std::lock_guard<std::mutex> l(g_mu);
    if (!g_live.erase(p)) return hipErrorInvalidValue;
    std::free(p);
    ++g_frees;
    return hipSuccess;
}
hipError_t hipMallocAsync(void** p, size_t bytes, hipStream_t) {
    *p = std::malloc(bytes);
    ++g_async_mallocs;
    return hipSuccess;
}
hipError_t hipFreeAsync(void* p, hipStream_t) {
    std::free(p);
    ++g_async_frees;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    std::lock_guard<std::mutex> l(g_mu);
    FakeEvent* f = new FakeEvent;
    g_events.push_back(f);
    *e = reinterpret_cast<hipEvent_t>(f);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    std::lock_guard<std::mutex> l(g_mu);
    FakeEvent* f = reinterpret_cast<FakeEvent*>(e);
    for (auto it = g_events.begin(); it != g_events.end(); ++it)
        if (*it == f) {
            g_events.erase(it);
            delete f;
            return hipSuccess;
        }
    return hipErrorInvalidValue;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
    std::lock_guard<std::mutex> l(g_mu);
    if (g_fail_record) return hipErrorUnknown;
    FakeEvent* f = reinterpret_cast<FakeEvent*>(e);
    f->pending = true;
    f->stream = s;
    return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t e) {
    std::lock_guard<std::mutex> l(g_mu);
    return reinterpret_cast<FakeEvent*>(e)->pending ? hipErrorNotReady : hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
    std::lock_guard<std::mutex> l(g_mu);
    reinterpret_cast<FakeEvent*>(e)->pending = false;
    ++g_host_waits;
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int) {
    std::lock_guard<std::mutex> l(g_mu);
    g_waits.emplace_back(s, reinterpret_cast<FakeEvent*>(e));
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t s) {
    ++g_stream_syncs;
    for (FakeEvent* f : g_events)
        if (f->stream == s) f->pending = false;
    return hipSuccess;
}

}  // extern "C"

namespace {

constexpr size_t MiB = size_t(1) << 20;

// one call: take a buffer of `bytes` on stream s, release it (its reader enqueued)
float* call(hipStream_t s, size_t bytes, hipError_t* err = nullptr) {
    fa::WorkspaceLease lease;
    const hipError_t e = lease.acquire(bytes, s);
    if (err) *err = e;
    if (e != hipSuccess) return nullptr;
    float* p = lease.ptr();
    CHECK(lease.release() == hipSuccess || g_fail_record);
    return p;
}

}  // namespace

int main() {
    static_assert(fa::kWorkspaceSlots == 4, "the scenario below fills four slots");
    const hipStream_t A = stream(0), B = stream(1), C = stream(2), Dst = stream(3), E = stream(4);

    // 3: the first call allocates (rounded up to the granule); nothing to wait for
    float* a0 = call(A, 1);
    CHECK(a0 != nullptr && g_mallocs == 1 && g_waits.empty() && g_host_waits == 0);
    // 2: the same stream again while its last use is pending: same buffer, a GPU-side wait on
    //    its event, no allocation
    float* a1 = call(A, MiB);
    CHECK(a1 == a0 && g_mallocs == 1 && g_waits.size() == 1 && g_waits[0].first == A);
    // 3: another stream while A's use is pending: a second buffer, no wait
    float* b0 = call(B, MiB);
    CHECK(b0 != a0 && g_mallocs == 2 && g_waits.size() == 1);
    // 1: A has finished: the idle buffer, no wait, no allocation
    finish(A);
    float* c0 = call(C, MiB);
    CHECK(c0 == a0 && g_mallocs == 2 && g_waits.size() == 1);
    // fill the last two slots (C's and B's buffers are pending)
    float* d0 = call(Dst, MiB);
    float* e0 = call(E, MiB);
    CHECK(d0 != a0 && d0 != b0 && e0 != a0 && e0 != b0 && e0 != d0 && g_mallocs == 4);
    // 4: all four pending on other streams: the one used longest ago (B's), behind a wait
    const hipStream_t F = stream(5);
    float* f0 = call(F, MiB);
    CHECK(f0 == b0 && g_mallocs == 4 && g_waits.size() == 2 && g_waits[1].first == F);
    CHECK(g_host_waits == 0);
    // 5: a larger request with no buffer large enough: the smallest is replaced, after the
    //    only host wait of the cache
    float* g0 = call(stream(6), 3 * MiB);
    CHECK(g0 != nullptr && g_mallocs == 5 && g_frees == 1 && g_host_waits == 1);
    // the large buffer now serves small requests on its stream too (same stream, pending)
    float* g1 = call(stream(6), MiB);
    CHECK(g1 == g0 && g_mallocs == 5);

    // capture: stream-ordered allocation, the cache untouched
    g_capturing = stream(7);
    const int m = g_mallocs;
    float* cap = call(stream(7), MiB);
    CHECK(cap != nullptr && g_async_mallocs == 1 && g_async_frees == 1 && g_mallocs == m);
    g_capturing = nullptr;

    // errors: a failed allocation holds nothing (the next call proceeds); a failed event
    // record synchronises the stream so the buffer is idle before anyone takes it
    for (int i = 0; i < 8; ++i) finish(stream(i));
    g_fail_malloc = true;
    hipError_t err = hipSuccess;
    float* big = call(stream(8), 64 * MiB, &err);   // needs a new buffer: fails
    CHECK(big == nullptr && err == hipErrorOutOfMemory);
    g_fail_malloc = false;
    float* ok = call(stream(8), MiB, &err);          // an idle buffer: works, lock released
    CHECK(ok != nullptr && err == hipSuccess);
    g_fail_record = true;
    const int syncs = g_stream_syncs;
    {
        fa::WorkspaceLease lease;
        CHECK(lease.acquire(MiB, stream(9)) == hipSuccess);
        CHECK(lease.release() == hipErrorUnknown && g_stream_syncs == syncs + 1);
    }
    g_fail_record = false;
    // a device index beyond the cache's table
    g_device = 1000;
    {
        fa::WorkspaceLease lease;
        CHECK(lease.acquire(MiB, A) == hipErrorInvalidDevice && lease.ptr() == nullptr);
    }
    g_device = 0;
    // a zero-byte request is refused
    {
        fa::WorkspaceLease lease;
        CHECK(lease.acquire(0, A) == hipErrorInvalidValue);
    }
    // the destructor releases a lease that was not released explicitly
    {
        fa::WorkspaceLease lease;
        CHECK(lease.acquire(MiB, A) == hipSuccess);
    }
    float* after = call(B, MiB);
    CHECK(after != nullptr);

    // two host threads: a lease holds the device's cache lock, so the second acquire waits
    // for the first release and the two never hold one buffer at the same time
    {
        for (int i = 0; i < 12; ++i) finish(stream(i));
        fa::WorkspaceLease first;
        CHECK(first.acquire(MiB, stream(10)) == hipSuccess);
        float* p1 = first.ptr();
        float* p2 = nullptr;
        std::chrono::steady_clock::time_point t_acq;
        std::thread t([&] {
            fa::WorkspaceLease second;
            if (second.acquire(MiB, stream(11)) == hipSuccess) {
                t_acq = std::chrono::steady_clock::now();
                p2 = second.ptr();
                (void)second.release();
            }
        });
        std::this_thread::sleep_for(std::chrono::milliseconds(100));
        const auto t_rel = std::chrono::steady_clock::now();
        CHECK(first.release() == hipSuccess);
        t.join();
        CHECK(p2 != nullptr && t_acq >= t_rel);
        CHECK(p1 != nullptr);
    }

    if (failures == 0) std::printf("workspace-rules ok\n");
    return failures == 0 ? 0 : 1;
}
