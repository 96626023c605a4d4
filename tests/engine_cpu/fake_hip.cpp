// Host-only implementation of the HIP runtime subset in
// fake_hip/hip/hip_runtime_api.h (test infrastructure for tests/engine_cpu).
//
// Ordering model, the one the GPU runtime guarantees and nothing more:
//  - a stream is a FIFO of operations run by its own worker thread, one at a
//    time, in enqueue order;
//  - work enqueued by a host thread happens after that thread's earlier
//    actions (the queue's mutex carries the edge);
//  - hipEventRecord(e, s) enqueues a marker; e is complete once every record
//    of it issued so far has run (the marker's completion is published under
//    the event's mutex);
//  - hipStreamWaitEvent(s, e) enqueues a wait for the records of e issued
//    before the call; hipEventSynchronize / hipStreamSynchronize block the
//    host the same way; hipEventQuery reports completion without blocking.
// No lock is held while an operation runs, so two operations that the rules
// above leave unordered really are concurrent: ThreadSanitizer reports their
// conflicting accesses, and random delays (FAKE_HIP_JITTER_US) vary which
// finishes first.  Memory: "device" buffers are ordinary host memory;
// hipHostMalloc registers its ranges as pinned for hipPointerGetAttributes.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <functional>
#include <map>
#include <mutex>
#include <random>
#include <thread>

struct FakeEvent {
  std::mutex mu;
  std::condition_variable cv;
  uint64_t recorded = 0;   // records issued
  uint64_t completed = 0;  // highest record that has run
  double time_ms = 0.0;    // when it ran
};

struct FakeStream {
  std::mutex mu;
  std::condition_variable cv;
  std::deque<std::function<void()>> q;
  uint64_t enqueued = 0, done = 0;
  bool stop = false;
  std::thread worker;
  std::mt19937 rng;
  int jitter_us = 0;

  explicit FakeStream(unsigned seed) : rng(seed) {
    if (const char* j = std::getenv("FAKE_HIP_JITTER_US")) jitter_us = std::atoi(j);
    worker = std::thread([this] { run(); });
  }
  void run() {
    for (;;) {
      std::function<void()> op;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || !q.empty(); });
        if (q.empty()) return;
        op = std::move(q.front());
        q.pop_front();
      }
      if (jitter_us > 0) {
        const int d = static_cast<int>(rng() % static_cast<unsigned>(jitter_us + 1));
        if (d > 0) std::this_thread::sleep_for(std::chrono::microseconds(d));
      }
      op();
      {
        std::lock_guard<std::mutex> lk(mu);
        ++done;
      }
      cv.notify_all();
    }
  }
  void push(std::function<void()> op) {
    {
      std::lock_guard<std::mutex> lk(mu);
      q.push_back(std::move(op));
      ++enqueued;
    }
    cv.notify_all();
  }
  void drain() {
    std::unique_lock<std::mutex> lk(mu);
    const uint64_t target = enqueued;
    cv.wait(lk, [&] { return done >= target; });
  }
  ~FakeStream() {
    drain();
    {
      std::lock_guard<std::mutex> lk(mu);
      stop = true;
    }
    cv.notify_all();
    worker.join();
  }
};

namespace {

std::atomic<unsigned> g_seed{12345};
std::mutex g_default_mu;
FakeStream* g_default = nullptr;
std::mutex g_pinned_mu;
std::map<uintptr_t, size_t> g_pinned;  // start -> bytes

FakeStream* resolve(hipStream_t s) {
  if (s) return s;
  std::lock_guard<std::mutex> lk(g_default_mu);
  if (!g_default) {
    if (const char* sd = std::getenv("FAKE_HIP_SEED")) g_seed = static_cast<unsigned>(std::atoi(sd)) * 7919u;
    g_default = new FakeStream(g_seed++);
  }
  return g_default;
}

double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

}  // namespace

hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  if (d) *d = 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) {
  switch (e) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    case hipErrorOutOfMemory: return "hipErrorOutOfMemory";
    case hipErrorNotReady: return "hipErrorNotReady";
    default: return "hipErrorUnknown";
  }
}
hipError_t hipGetLastError(void) { return hipSuccess; }

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  if (!s) return hipErrorInvalidValue;
  if (const char* sd = std::getenv("FAKE_HIP_SEED")) {
    static std::once_flag once;
    std::call_once(once, [&] { g_seed = static_cast<unsigned>(std::atoi(sd)) * 7919u; });
  }
  *s = new FakeStream(g_seed++);
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  delete s;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t s) {
  resolve(s)->drain();
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int) {
  if (!e) return hipErrorInvalidValue;
  uint64_t target;
  {
    std::lock_guard<std::mutex> lk(e->mu);
    target = e->recorded;
  }
  if (target == 0) return hipSuccess;  // never recorded: nothing to wait for
  resolve(s)->push([e, target] {
    std::unique_lock<std::mutex> lk(e->mu);
    e->cv.wait(lk, [&] { return e->completed >= target; });
  });
  return hipSuccess;
}

hipError_t hipEventCreate(hipEvent_t* e) {
  if (!e) return hipErrorInvalidValue;
  *e = new FakeEvent();
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned int) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  if (!e) return hipErrorInvalidValue;
  uint64_t seq;
  {
    std::lock_guard<std::mutex> lk(e->mu);
    seq = ++e->recorded;
  }
  resolve(s)->push([e, seq] {
    {
      std::lock_guard<std::mutex> lk(e->mu);
      if (seq > e->completed) {
        e->completed = seq;
        e->time_ms = now_ms();
      }
    }
    e->cv.notify_all();
  });
  return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t e) {
  if (!e) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(e->mu);
  return e->completed >= e->recorded ? hipSuccess : hipErrorNotReady;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
  if (!e) return hipErrorInvalidValue;
  std::unique_lock<std::mutex> lk(e->mu);
  const uint64_t target = e->recorded;
  e->cv.wait(lk, [&] { return e->completed >= target; });
  return hipSuccess;
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  if (!ms || !a || !b) return hipErrorInvalidValue;
  double ta, tb;
  {
    std::lock_guard<std::mutex> lk(a->mu);
    if (a->completed < a->recorded || a->recorded == 0) return hipErrorNotReady;
    ta = a->time_ms;
  }
  {
    std::lock_guard<std::mutex> lk(b->mu);
    if (b->completed < b->recorded || b->recorded == 0) return hipErrorNotReady;
    tb = b->time_ms;
  }
  *ms = static_cast<float>(tb - ta);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (!dst || !src) return hipErrorInvalidValue;
  resolve(s)->push([dst, src, bytes] { std::memcpy(dst, src, bytes); });
  return hipSuccess;
}

hipError_t hipHostMalloc(void** p, size_t bytes, unsigned int) {
  if (!p) return hipErrorInvalidValue;
  const size_t n = (bytes + 255) / 256 * 256;
  *p = std::aligned_alloc(256, n ? n : 256);
  if (!*p) return hipErrorOutOfMemory;
  std::lock_guard<std::mutex> lk(g_pinned_mu);
  g_pinned[reinterpret_cast<uintptr_t>(*p)] = n ? n : 256;
  return hipSuccess;
}
hipError_t hipHostFree(void* p) {
  if (!p) return hipSuccess;
  {
    std::lock_guard<std::mutex> lk(g_pinned_mu);
    g_pinned.erase(reinterpret_cast<uintptr_t>(p));
  }
  std::free(p);
  return hipSuccess;
}
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* p) {
  if (!attr) return hipErrorInvalidValue;
  std::memset(attr, 0, sizeof *attr);
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  std::lock_guard<std::mutex> lk(g_pinned_mu);
  auto it = g_pinned.upper_bound(u);
  if (it != g_pinned.begin()) {
    --it;
    if (u < it->first + it->second) {
      attr->type = hipMemoryTypeHost;
      attr->hostPointer = const_cast<void*>(p);
      return hipSuccess;
    }
  }
  return hipErrorInvalidValue;  // pageable memory
}

// Waits for every stream of the process (the harness calls it before
// comparing results and at exit).
void fake_hip_drain_default() {
  FakeStream* s = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_default_mu);
    s = g_default;
  }
  if (s) s->drain();
}

// Enqueues a host function as a stream operation (the fake kernels' launch).
void fake_enqueue(hipStream_t s, std::function<void()> f) { resolve(s)->push(std::move(f)); }
