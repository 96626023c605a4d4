// The layer-sliding engine: one training iteration over L decoder layers
// with only `window` layers' parameters and gradients resident on the device.
//
// What the pages describe (de §2A "Leichtgewichtige asynchrone Engine",
// es §2A "Arquitectura de Deslizamiento de Capas", fr §2A; de/es/fr §2B):
//  - the device holds a small active window of layers, the rest live in host
//    memory; a layer is the unit of transfer and update;
//  - a fixed queue of pre-allocated device cache units, each sized for one
//    layer's parameters and gradients (fixed footprint, no reallocation);
//  - in the backward, layer L_i's gradients go to host memory asynchronously
//    and host threads run Adam on L_i while the device computes L_{i-1} and
//    the parameters of L_{i-2} are prefetched;
//  - a thread-based design with dedicated streams and CPU threads;
//  - gradient buffers on the host are shared by all layers.
//
// Realisation here.  HIP streams: compute (the caller's), H2D (layer
// prefetch), D2H (gradients) and the context's side stream, which besides
// the layer backward's weight-gradient GEMMs carries the LM head's update and
// the uploads Adam queues; all at default priority and ordered only through
// events, so host-link copies in both directions overlap kernels.  Four
// streams in all: the device has four hardware queues by default, and a
// stream beyond them shares a queue, where its work waits behind everything
// queued before it on the other streams of that queue.  Unit u = layer mod window; each unit has
// separate "parameters free" and "gradients free" events, so a unit's
// parameter slot can be refilled for L_{i-window+1} as soon as the backward
// of L_i is done while its gradient slot is still draining.  A dispatcher
// thread waits for each gradient copy and runs Adam on a worker pool, then
// releases the shared host gradient slot.  Adam of layer i uses this
// iteration's gradients and only affects the next iteration, so the result
// equals plain synchronous training.
//
// Gradients leave in ranges of at most an eighth of a layer (>= 1 MiB), and
// Adam of a range starts as soon as its copy lands, so copy and update of
// one layer overlap.  The backward ends with layers W-1 .. 0, which are
// also the first the next forward needs: their updated ranges go straight
// back into their units, each upload overlapping the Adam of the next range,
// and the next step's forward starts without waiting for them.
//
// Embedding and LM head (resident in HBM): by default a device Adam updates
// them (fp32 master and moments in HBM), the LM head and final norm on the
// side stream once the last layer's MLP weight gradients are final, the
// embedding from its sparse gradient (distinct rows and a row map) at the
// end of the backward.  With SF_ENGINE_HEAD_HOST_ADAM
// they take the host path like a layer: the LM-head and final-norm gradients
// leave right after the head and are applied (and their parameters uploaded
// again) while the layer backward runs; the embedding gradient leaves sparse
// -- only the rows of ids present in the batch are nonzero -- and its dense
// Adam (every row: moments decay) is pipelined with the upload of the
// updated rows.
//
// Sliding activation checkpointing (de/es/fr §2B, SF_ENGINE_CKPT): layer
// inputs leave for pinned host memory on the D2H stream as soon as they are
// produced and the forward cycles through a ring of three input buffers; in
// the backward the input of layer i-1 comes back into one of two slots while
// layer i runs, and each layer first recomputes its forward (same kernels,
// same inputs: the same bits) into a scratch output and saved set.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "adam.h"
#include "internal.h"
#include "rowops.h"

namespace sf {

namespace {

// A fixed pool of worker threads running index-parallel loops.  Adam jobs
// arrive back to back (one per gradient range), so idle workers spin for a
// short while before sleeping: waking a sleeping thread costs tens of
// microseconds per job.
class Pool {
 public:
  explicit Pool(int n) {
    for (int i = 0; i < n; ++i) th_.emplace_back([this] { loop(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_.store(true);
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  // Run fn(0 .. n-1) on the pool and the calling thread; returns when done
  // and no worker still refers to this call.
  void run(size_t n, const std::function<void(size_t)>& fn) {
    if (n == 0) return;
    Task t;
    t.fn = &fn;
    t.n = n;
    {
      std::lock_guard<std::mutex> lk(mu_);
      cur_ = &t;
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    work(t);
    {
      // no new worker may pick the task up from here on
      std::lock_guard<std::mutex> lk(mu_);
      cur_ = nullptr;
    }
    auto finished = [&] { return t.done.load(std::memory_order_acquire) == n && active_.load() == 0; };
    for (int spin = 0; !finished(); ++spin) {
      if (spin < (1 << 16)) {
        cpu_relax();
      } else {
        std::unique_lock<std::mutex> lk(mu_);
        cv_done_.wait(lk, finished);
      }
    }
  }

 private:
  struct Task {
    const std::function<void(size_t)>* fn = nullptr;
    size_t n = 0;
    std::atomic<size_t> next{0}, done{0};
  };
  static void cpu_relax() { __builtin_ia32_pause(); }
  static void work(Task& t) {
    for (;;) {
      const size_t i = t.next.fetch_add(1);
      if (i >= t.n) break;
      (*t.fn)(i);
      t.done.fetch_add(1, std::memory_order_acq_rel);
    }
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      // spin about 100 us for the next task, then sleep
      for (int spin = 0; spin < 20000 && gen_.load(std::memory_order_acquire) == seen && !stop_.load(); ++spin)
        cpu_relax();
      Task* t = nullptr;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
        if (stop_.load()) return;
        seen = gen_.load();
        t = cur_;
        if (t) active_.fetch_add(1);
      }
      if (!t) continue;
      work(*t);
      {
        std::lock_guard<std::mutex> lk(mu_);
        active_.fetch_sub(1);
      }
      cv_done_.notify_all();
    }
  }
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_, cv_done_;
  Task* cur_ = nullptr;
  std::atomic<int> active_{0};
  std::atomic<uint64_t> gen_{0};
  std::atomic<bool> stop_{false};
};

enum JobKind { kLayer = 0, kHeadLm = 1, kEmbed = 2 };

struct Job {
  int kind;
  int layer;  // kLayer
  int slot;   // host gradient slot (kLayer)
  hipEvent_t ready;
  size_t lo = 0, hi = 0;  // kLayer: byte range of the layer's fp32 gradients
  hipEvent_t verdict = nullptr;  // loss scaling: the layer's gradients have been checked
  bool first = false;     // kLayer: the layer's first range
  bool last = false;      // kLayer: the layer's final range (frees the slot)
  int64_t step = 0;       // the iteration whose gradients these are
  AdamCoef coef{};        // that iteration's Adam coefficients
};

struct Interval {
  hipEvent_t a, b;
  int kind;  // 0 compute, 1 H2D, 2 D2H
  double bytes;
  int64_t seq;  // issue order (the oldest live interval is waited for first)
};

// Streams whose timed intervals complete in issue order: the compute
// stream, the H2D stream, the D2H stream and the context's side stream
// (head update and the uploads Adam queues).
enum { kStComp = 0, kStH2d = 1, kStD2h = 2, kStSide = 3, kNumStreams = 4 };

// One row of the step trace: what, when (ms after the step's first device
// event), and its bytes (copies) or layer (Adam jobs).
struct TraceRow {
  double kind, start, end, info;
};

double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

bool is_pinned(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

// Sparse embedding-gradient block inside the first V*H floats of the head
// gradient region: [count | pad | ids (T) | pad | rows (T x H) | scratch (2T)],
// offsets in 4-byte words.
struct SparseLayout {
  size_t ids, rows, scratch, copy_words, total;
};
SparseLayout sparse_layout(int64_t T, int H) {
  SparseLayout s;
  s.ids = 64;
  s.rows = (s.ids + T + 63) / 64 * 64;
  s.scratch = s.rows + static_cast<size_t>(T) * H;
  s.copy_words = s.scratch;
  s.total = s.scratch + 2 * static_cast<size_t>(T);
  return s;
}

}  // namespace

}  // namespace sf

using namespace sf;

struct sf_engine {
  sf_ctx* ctx = nullptr;
  sf_engine_cfg cfg{};
  Dims d;
  sf_layout L{};
  int nl = 0, W = 0;
  size_t unit_bytes = 0, x_bytes = 0;
  size_t chunk_bytes = 0;  // gradient D2H / Adam / re-upload granularity
  bool preloaded = false;  // units 0..W-1 hold this step's layers 0..W-1 already
  hipStream_t s_comp = nullptr, s_h2d = nullptr, s_d2h = nullptr, s_head = nullptr;
  // uploads of updated ranges that Adam queues (layers below the window):
  // never behind the forward's prefetches or the gradient copies.  The device
  // has few hardware queues (4 by default) and streams beyond them share one,
  // where work waits for everything queued before it on any of its streams:
  // a stream of their own shared a queue with the gradient copies.  So the
  // uploads and the head's update (s_head) go on the context's side stream,
  // which is idle at the end of the backward, where these uploads come, and
  // the engine adds only the H2D and D2H streams to the caller's and the
  // context's.
  hipStream_t s_up = nullptr;
  bool own_head = false;  // s_head created here (the context has no side stream)
  std::vector<char*> uparam, ugrad, x, saved;
  char* dbuf = nullptr;
  // activation checkpointing: layer inputs ring (3), checkpoint slots for the
  // backward (2), recompute output scratch, saved sets (0: scratch, 1: last
  // layer's, kept from the forward)
  bool ckpt = false;
  char* xr[3] = {nullptr, nullptr, nullptr};
  char* cs[2] = {nullptr, nullptr};
  char* ys = nullptr;
  char* sv[2] = {nullptr, nullptr};
  hipEvent_t ev_xfree[3] = {nullptr, nullptr, nullptr}, ev_cready[2] = {nullptr, nullptr},
             ev_cfree[2] = {nullptr, nullptr}, ev_ckpt_out = nullptr;
  float* d_loss = nullptr;
  // the loss as the host reads it: one pinned word written by a kernel on
  // the compute stream (a synchronous read-back would queue behind the
  // uploads in flight on the copy engines and return milliseconds late)
  float* h_loss = nullptr;
  std::vector<hipEvent_t> ev_param_ready, ev_param_free, ev_grad_free;
  // the gradient region of a unit as a second parameter slot in the forward
  std::vector<hipEvent_t> ev_gslot_ready, ev_gslot_free;
  // Timing events: a fixed pool created with the engine.  An interval's two
  // events go back to the pool once its end event has completed and its
  // times (ms after the window's origin) are in `rows`; when the pool is
  // empty, the host waits for the oldest live interval.  Shared with the
  // dispatcher thread (under tmu).
  std::mutex tmu;
  std::vector<hipEvent_t> tev_all, tev_free;
  std::deque<Interval> live[kNumStreams];
  std::vector<TraceRow> rows;  // completed intervals of the measurement window
  int64_t seq = 0;
  int64_t blocked_waits = 0;
  // markers inside a layer's backward (MLP weight gradients final, Wd's
  // final), one pair per unit, re-recorded for every layer of the unit
  std::vector<hipEvent_t> ev_ffn, ev_wd;
  // test hook: the Adam job with this index (counted from engine creation)
  // reports a failure instead of running (environment SF_FAULT_ADAM_JOB)
  int64_t fault_adam_job = -1, adam_jobs_seen = 0;
  // Dynamic loss scaling (SF_F16 storage).  d_ovf: running OR of non-finite
  // gradients of the step's backward (device, in the activation region's
  // tail); d_ovf_head: its value right after the head (the head's device
  // Adam reads it); h_ovf: pinned verdicts [2 steps by parity][n_layers + 2]
  // (layer i, n_layers: head, n_layers + 1: whole step) that the compute
  // stream publishes; ev_verdict[i]: layer i's verdict is published.
  bool lscale = false;
  float scale = 1.f;
  int32_t scale_window = 2000;
  int64_t good_steps = 0;
  int32_t* d_ovf = nullptr;
  int32_t* d_ovf_head = nullptr;
  int32_t* h_ovf = nullptr;
  std::vector<hipEvent_t> ev_verdict;
  // Adam steps applied so far per layer, LM head and embedding (a skipped
  // update does not count) and this step's coefficients from them
  std::vector<int64_t> adam_t;
  int64_t head_t = 0, embed_t = 0;
  std::vector<AdamCoef> lcoef;
  AdamCoef hcoef{}, ecoef{};
  float last_scale = 1.f;
  int32_t last_skipped = 0;
  int fault_nonfinite_layer = -1;  // test hook (environment SF_FAULT_NONFINITE_LAYER)
  int64_t step = 0;
  bool failed = false;
  // embedding sparse gradients
  SparseLayout sp{};
  std::vector<int32_t> slot_of_row;
  std::vector<float> zero_row;
  // Adam machinery
  std::unique_ptr<Pool> pool;
  std::thread dispatcher;
  std::mutex mu;
  std::condition_variable cv;
  std::deque<Job> jobs;
  std::vector<bool> slot_free;
  int next_slot = 0;
  int pending = 0;
  bool stop = false;
  std::string job_error;
  AdamCoef coef{};
  int n_threads = 1;  // Adam threads: the pool plus the dispatcher
  double adam_ms = 0;
  // Cross-step pipelining (SF_ENGINE_PIPELINE): a step returns with its Adam
  // jobs still running; adam_done[l] is the last step whose Adam of layer l
  // is complete (its updated parameters written and, for layers below the
  // window, their uploads queued), and the next forward waits on it per layer.
  bool pipe = false;
  std::vector<int64_t> adam_done;
  hipEvent_t ev_head_done = nullptr;  // device Adam of the LM head and final gain
  // Measurement window: one step (synchronous) or every step since the last
  // sf_engine_sync (pipelined).
  bool window_open = false;
  hipEvent_t ev_origin = nullptr;  // recorded when a window opens (timing)
  hipEvent_t ev_start = nullptr;   // each later step's start (side streams wait on it)
  sf_step_stats last_stats{};
  double host_t0 = 0;                 // host clock at the window's first device event
  std::vector<TraceRow> adam_rows;    // host Adam jobs of the current step (under mu)
  std::vector<TraceRow> trace;        // the last completed step
};

namespace sf {
namespace {

// Move every completed interval at the head of a stream's queue into
// `rows` and its events back to the pool; returns how many.  Under tmu.
size_t reclaim_locked(sf_engine* e) {
  size_t n = 0;
  for (auto& q : e->live) {
    while (!q.empty() && hipEventQuery(q.front().b) == hipSuccess) {
      const Interval& x = q.front();
      float a = 0, b = 0;
      (void)hipEventElapsedTime(&a, e->ev_origin, x.a);
      (void)hipEventElapsedTime(&b, e->ev_origin, x.b);
      e->rows.push_back({static_cast<double>(x.kind), a, b, x.bytes});
      e->tev_free.push_back(x.a);
      e->tev_free.push_back(x.b);
      q.pop_front();
      ++n;
    }
  }
  return n;
}

// A free timing event from the pool; waits for the oldest live interval
// when none is free.  nullptr only if the pool is empty with nothing live.
hipEvent_t timing_event(sf_engine* e) {
  std::unique_lock<std::mutex> lk(e->tmu);
  for (;;) {
    if (!e->tev_free.empty()) {
      hipEvent_t ev = e->tev_free.back();
      e->tev_free.pop_back();
      return ev;
    }
    if (reclaim_locked(e) > 0) continue;
    const Interval* oldest = nullptr;
    for (auto& q : e->live)
      if (!q.empty() && (!oldest || q.front().seq < oldest->seq)) oldest = &q.front();
    if (!oldest) return nullptr;
    hipEvent_t wait = oldest->b;
    ++e->blocked_waits;
    lk.unlock();
    (void)hipEventSynchronize(wait);
    lk.lock();
  }
}

sf_status record_interval(sf_engine* e, hipEvent_t a, hipEvent_t b, int kind, double bytes, int stream) {
  if (!a || !b) return fail(SF_ERR_HIP, "event pool exhausted");
  std::lock_guard<std::mutex> lk(e->tmu);
  e->live[stream].push_back({a, b, kind, bytes, e->seq++});
  return SF_OK;
}

// One H2D copy on stream s (the H2D stream or the side stream) with a timed interval.
sf_status timed_h2d(sf_engine* e, void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipEvent_t a = timing_event(e), b = timing_event(e);
  if (!a || !b) return fail(SF_ERR_HIP, "event pool exhausted");
  SF_HIP(hipEventRecord(a, s));
  SF_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s));
  SF_HIP(hipEventRecord(b, s));
  return record_interval(e, a, b, 1, static_cast<double>(bytes), s == e->s_h2d ? kStH2d : kStSide);
}

// Adam over segments (fp32 offset in master/m/v/grad, count, element offset
// of the storage-dtype copy), chunked across the pool.
struct Seg {
  size_t off, n, out_off;
};

void run_adam(sf_engine* e, const AdamCoef& c, float* p, float* m, float* v, const float* g, void* out,
              bool out_is_master, const std::vector<Seg>& segs) {
  // about four tasks per thread, each 16K .. 256K elements
  size_t total = 0;
  for (const Seg& s : segs) total += s.n;
  const size_t per = total / (4 * static_cast<size_t>(e->n_threads)) / 64 * 64;
  const size_t chunk = std::min<size_t>(1 << 18, std::max<size_t>(1 << 14, per));
  std::vector<Seg> tasks;
  for (const Seg& s : segs)
    for (size_t b = 0; b < s.n; b += chunk) tasks.push_back({s.off + b, std::min(chunk, s.n - b), s.out_off + b});
  const bool half = e->d.dtype != SF_F32;
  const int out16 = e->d.dtype == SF_F16 ? 2 : 1;
  e->pool->run(tasks.size(), [&](size_t i) {
    const Seg& t = tasks[i];
    if (half) {
      adam_range(p + t.off, m + t.off, v + t.off, g + t.off, static_cast<uint16_t*>(out) + t.out_off, t.n, c, out16);
    } else {
      adam_range(p + t.off, m + t.off, v + t.off, g + t.off, nullptr, t.n, c);
      if (!out_is_master) std::memcpy(static_cast<float*>(out) + t.out_off, p + t.off, t.n * 4);
    }
  });
}

// Embedding: dense Adam over every row (rows without a gradient this step
// take g = 0, exactly as a dense zero gradient would), in groups of rows;
// each group's updated storage-dtype rows are uploaded on the head stream
// while the next group is updated.
sf_status run_embed_adam(sf_engine* e, const AdamCoef& cf) {
  const sf_engine_cfg& c = e->cfg;
  const int H = e->d.H, V = e->d.V;
  const float* hg = c.h_head_grads;
  const int32_t count = reinterpret_cast<const int32_t*>(hg)[0];
  const int32_t* ids = reinterpret_cast<const int32_t*>(hg) + e->sp.ids;
  const float* rows = hg + e->sp.rows;
  if (count < 0 || count > e->d.T) return fail(SF_ERR_HIP, "corrupt sparse embedding gradient count %d", count);
  for (int s = 0; s < count; ++s) {
    const int id = ids[s];
    if (id < 0 || id >= V) return fail(SF_ERR_HIP, "corrupt sparse embedding gradient id %d", id);
    e->slot_of_row[id] = s;
  }
  const bool bf = e->d.dtype != SF_F32;
  const int out16 = e->d.dtype == SF_F16 ? 2 : 1;
  const bool out_is_master = c.h_head_params == static_cast<void*>(c.h_head_master);
  const int rows_per_task = std::max(1, (1 << 17) / H);
  const int groups = 8;
  const int rows_per_group = (V + groups - 1) / groups;
  sf_status rc = SF_OK;
  for (int g0 = 0; g0 < V && rc == SF_OK; g0 += rows_per_group) {
    const int g1 = std::min(V, g0 + rows_per_group);
    const size_t ntask = (g1 - g0 + rows_per_task - 1) / rows_per_task;
    e->pool->run(ntask, [&](size_t ti) {
      const int r0 = g0 + static_cast<int>(ti) * rows_per_task, r1 = std::min(g1, r0 + rows_per_task);
      for (int r = r0; r < r1; ++r) {
        const int s = e->slot_of_row[r];
        const float* gr = s >= 0 ? rows + static_cast<size_t>(s) * H : e->zero_row.data();
        const size_t o = static_cast<size_t>(r) * H;
        if (bf) {
          adam_range(c.h_head_master + o, c.h_head_m + o, c.h_head_v + o, gr,
                     static_cast<uint16_t*>(c.h_head_params) + o, H, cf, out16);
        } else {
          adam_range(c.h_head_master + o, c.h_head_m + o, c.h_head_v + o, gr, nullptr, H, cf);
          if (!out_is_master) std::memcpy(static_cast<float*>(c.h_head_params) + o, c.h_head_master + o, H * 4);
        }
      }
    });
    const size_t off = static_cast<size_t>(g0) * H * e->d.e;
    rc = timed_h2d(e, static_cast<char*>(c.d_E) + off, static_cast<const char*>(c.h_head_params) + off,
                   static_cast<size_t>(g1 - g0) * H * e->d.e, e->s_head);
  }
  for (int s = 0; s < count; ++s) e->slot_of_row[ids[s]] = -1;
  return rc;
}

// Adam segments and the parameter byte range [plo, phi) that belong to the
// gradient bytes [lo, hi) of a layer (the range may span tensors; padding
// between tensors is skipped).
struct ChunkMap {
  std::vector<Seg> segs;
  size_t plo = SIZE_MAX, phi = 0;
};
ChunkMap chunk_map(const sf_layout& L, int eb, size_t lo, size_t hi) {
  ChunkMap cm;
  for (int t = 0; t < SF_NTENSORS; ++t) {
    const size_t a = std::max(lo, L.grad_off[t]), b = std::min(hi, L.grad_off[t] + L.grad_bytes_t[t]);
    if (a >= b) continue;
    const size_t i0 = (a - L.grad_off[t]) / 4, i1 = (b - L.grad_off[t]) / 4;
    cm.segs.push_back({a / 4, i1 - i0, L.off[t] / eb + i0});
    cm.plo = std::min(cm.plo, L.off[t] + i0 * eb);
    cm.phi = std::max(cm.phi, L.off[t] + i1 * eb);
  }
  return cm;
}

sf_status run_job(sf_engine* e, const Job& j) {
  const sf_engine_cfg& c = e->cfg;
  const size_t VH = static_cast<size_t>(e->d.V) * e->d.H;
  if (j.kind == kLayer) {
    const ChunkMap cm = chunk_map(e->L, e->d.e, j.lo, j.hi);
    // loss scaling: a non-finite gradient in this layer or before it in the
    // backward leaves the layer as it is (its unit still holds it)
    const bool skip = e->lscale && e->h_ovf[(j.step & 1) * (e->nl + 2) + j.layer] != 0;
    if (!skip)
      run_adam(e, j.coef, c.h_master[j.layer], c.h_m[j.layer], c.h_v[j.layer], c.h_grad_slots[j.slot],
               c.h_params[j.layer], c.h_params[j.layer] == static_cast<void*>(c.h_master[j.layer]), cm.segs);
    // Layers 0 .. W-1 open the next step's forward and finish their backward
    // last: upload each updated range into the layer's unit right away, so
    // the upload of one range overlaps the Adam of the next.
    if (j.layer < e->W) {
      const int u = j.layer;
      if (j.first) SF_HIP(hipStreamWaitEvent(e->s_up, e->ev_param_free[u], 0));
      if (!skip && cm.phi > cm.plo) {
        if (sf_status rc = timed_h2d(e, e->uparam[u] + cm.plo, static_cast<const char*>(c.h_params[j.layer]) + cm.plo,
                                     cm.phi - cm.plo, e->s_up))
          return rc;
      }
      if (j.last) SF_HIP(hipEventRecord(e->ev_param_ready[u], e->s_up));
    }
    return SF_OK;
  }
  if (j.kind == kHeadLm) {
    // final-norm gain and LM head: [VH, VH + H) and [VH + H, 2 VH + H)
    run_adam(e, j.coef, c.h_head_master, c.h_head_m, c.h_head_v, c.h_head_grads, c.h_head_params,
             c.h_head_params == static_cast<void*>(c.h_head_master), {{VH, VH + e->d.H, VH}});
    const char* hp = static_cast<const char*>(c.h_head_params);
    sf_status rc = timed_h2d(e, c.d_gf, hp + VH * e->d.e, e->d.H * e->d.e, e->s_head);
    if (rc) return rc;
    return timed_h2d(e, c.d_wlm, hp + (VH + e->d.H) * e->d.e, VH * e->d.e, e->s_head);
  }
  return run_embed_adam(e, j.coef);
}

void dispatcher_loop(sf_engine* e) {
  (void)hipSetDevice(e->ctx->device);
  for (;;) {
    Job j;
    {
      std::unique_lock<std::mutex> lk(e->mu);
      e->cv.wait(lk, [&] { return e->stop || !e->jobs.empty(); });
      if (e->jobs.empty()) return;  // stop requested and nothing left
      // Among the ranges whose copies have landed (ranges of one layer in
      // order): first the layers above the window in the order they arrived
      // (highest first), since a layer frees its gradient slot, which a later
      // layer's copies wait for, only when all its ranges are done; then the
      // window's layers lowest first, as the next forward needs layer 0 first
      // and layer 0's gradients arrive last.  A layer's last range (its gains,
      // a few KB) goes before all others.  With none landed, the oldest range
      // (its copy was queued first).
      size_t pick = 0;
      int best = INT32_MAX;
      for (size_t q = 0; q < e->jobs.size(); ++q) {
        const Job& cand = e->jobs[q];
        const int key = cand.kind != kLayer ? -1
                        : cand.last         ? -2
                        : cand.layer >= e->W ? e->nl - cand.layer
                                             : e->nl + cand.layer;
        if (key >= best) continue;
        bool earlier_same = false;  // keep a layer's ranges in order
        for (size_t r = 0; r < q && !earlier_same; ++r)
          earlier_same = e->jobs[r].kind == cand.kind && e->jobs[r].layer == cand.layer;
        if (earlier_same) continue;
        if (hipEventQuery(cand.ready) != hipSuccess) continue;
        best = key;
        pick = q;
      }
      j = e->jobs[pick];
      e->jobs.erase(e->jobs.begin() + static_cast<std::ptrdiff_t>(pick));
    }
    std::string err;
    hipError_t he = hipEventSynchronize(j.ready);
    if (he == hipSuccess && j.verdict) he = hipEventSynchronize(j.verdict);
    const double t0 = now_ms();
    const bool fault = e->fault_adam_job >= 0 && e->adam_jobs_seen++ == e->fault_adam_job;
    if (he != hipSuccess) {
      err = std::string("gradient copy failed: ") + hipGetErrorString(he);
    } else if (fault) {
      err = "injected failure of Adam job " + std::to_string(e->fault_adam_job) + " (SF_FAULT_ADAM_JOB)";
    } else {
      const sf_status rc = run_job(e, j);
      if (rc != SF_OK) err = sf_last_error();
    }
    const double t1 = now_ms();
    std::lock_guard<std::mutex> lk(e->mu);
    if (!err.empty() && e->job_error.empty()) e->job_error = err;
    e->adam_ms += t1 - t0;
    e->adam_rows.push_back({3.0 + j.kind, t0 - e->host_t0, t1 - e->host_t0, static_cast<double>(j.layer)});
    if (j.kind == kLayer && j.last) {
      e->slot_free[j.slot] = true;
      if (err.empty()) e->adam_done[j.layer] = j.step;
    }
    --e->pending;
    e->cv.notify_all();
  }
}

// H2D of layer j's parameters into unit j % W.
sf_status prefetch(sf_engine* e, int j) {
  const int u = j % e->W;
  SF_HIP(hipStreamWaitEvent(e->s_h2d, e->ev_param_free[u], 0));
  if (sf_status rc = timed_h2d(e, e->uparam[u], e->cfg.h_params[j], e->L.param_bytes, e->s_h2d)) return rc;
  SF_HIP(hipEventRecord(e->ev_param_ready[u], e->s_h2d));
  return SF_OK;
}

double union_ms(std::vector<std::pair<double, double>> v) {
  std::sort(v.begin(), v.end());
  double tot = 0, cs = -1e300, ce = -1e300;
  for (auto& p : v) {
    if (p.first > ce) {
      if (ce > cs) tot += ce - cs;
      cs = p.first;
      ce = p.second;
    } else {
      ce = std::max(ce, p.second);
    }
  }
  if (ce > cs) tot += ce - cs;
  return tot;
}

sf_status fill_stats(sf_engine* e, sf_step_stats* st) {
  std::vector<std::pair<double, double>> comp, copy, h2d, d2h;
  double lo = 1e300, hi = -1e300, hb = 0, db = 0;
  {
    // every stream has been synchronised: all live intervals are complete
    std::lock_guard<std::mutex> lk(e->tmu);
    reclaim_locked(e);
    for (auto& q : e->live)
      if (!q.empty()) return fail(SF_ERR_HIP, "a timed interval did not complete");
  }
  e->trace.clear();
  for (const TraceRow& x : e->rows) {
    const double a = x.start, b = x.end;
    const int kind = static_cast<int>(x.kind);
    e->trace.push_back(x);
    lo = std::min(lo, a);
    hi = std::max(hi, b);
    if (kind == 0) comp.push_back({a, b});
    else copy.push_back({a, b});
    if (kind == 1) { h2d.push_back({a, b}); hb += x.info; }
    if (kind == 2) { d2h.push_back({a, b}); db += x.info; }
  }
  st->compute_ms = union_ms(comp);
  st->copy_ms = union_ms(copy);
  st->h2d_ms = union_ms(h2d);
  st->d2h_ms = union_ms(d2h);
  st->span_ms = hi > lo ? hi - lo : 0;
  std::vector<std::pair<double, double>> all(comp);
  all.insert(all.end(), copy.begin(), copy.end());
  st->busy_ms = union_ms(all);
  // time both a kernel and a copy are in flight = comp + copy - (comp U copy)
  const double both = st->compute_ms + st->copy_ms - st->busy_ms;
  const double mn = std::min(st->compute_ms, st->copy_ms);
  st->overlap_pct = mn > 0 ? 100.0 * both / mn : 0.0;
  st->h2d_bytes = hb;
  st->d2h_bytes = db;
  st->h2d_gbps = st->h2d_ms > 0 ? hb / (st->h2d_ms * 1e6) : 0;
  st->d2h_gbps = st->d2h_ms > 0 ? db / (st->d2h_ms * 1e6) : 0;
  return SF_OK;
}

sf_status wait_slot(sf_engine* e, int* slot) {
  std::unique_lock<std::mutex> lk(e->mu);
  const int k = e->next_slot;
  e->next_slot = (k + 1) % e->cfg.n_grad_slots;
  e->cv.wait(lk, [&] { return e->slot_free[k]; });
  if (e->cfg.flags & SF_ENGINE_ADAM) e->slot_free[k] = false;
  *slot = k;
  return SF_OK;
}

void push_job(sf_engine* e, Job j) {
  j.step = e->step;
  j.coef = j.kind == kLayer ? e->lcoef[j.layer] : e->coef;
  std::lock_guard<std::mutex> lk(e->mu);
  e->jobs.push_back(j);
  ++e->pending;
  e->cv.notify_all();
}

void drain(sf_engine* e) {
  std::unique_lock<std::mutex> lk(e->mu);
  e->cv.wait(lk, [&] { return e->pending == 0; });
}

// D2H copy on the gradient stream after `after` (an event on the compute
// stream); returns the copy's end event in *done.
sf_status timed_d2h(sf_engine* e, void* dst, const void* src, size_t bytes, hipEvent_t after, hipEvent_t* done) {
  hipEvent_t b0 = timing_event(e), b1 = timing_event(e);
  if (!b0 || !b1) return fail(SF_ERR_HIP, "event pool exhausted");
  SF_HIP(hipStreamWaitEvent(e->s_d2h, after, 0));
  SF_HIP(hipEventRecord(b0, e->s_d2h));
  SF_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, e->s_d2h));
  SF_HIP(hipEventRecord(b1, e->s_d2h));
  *done = b1;
  return record_interval(e, b0, b1, 2, static_cast<double>(bytes), kStD2h);
}

// Wait for every copy, kernel and Adam job, then measure the window (one
// step, or all pipelined steps since the window opened) into *st.
sf_status close_window(sf_engine* e, sf_step_stats* st) {
  SF_HIP(hipStreamSynchronize(e->s_comp));
  SF_HIP(hipStreamSynchronize(e->s_d2h));
  drain(e);  // Adam jobs; they queue the re-upload of layers 0 .. W-1
  SF_HIP(hipStreamSynchronize(e->s_h2d));
  SF_HIP(hipStreamSynchronize(e->s_up));
  SF_HIP(hipStreamSynchronize(e->s_head));
  {
    std::lock_guard<std::mutex> lk(e->mu);
    if (!e->job_error.empty()) return fail(SF_ERR_HIP, "%s", e->job_error.c_str());
  }
  sf_step_stats local{};
  if (!e->window_open) {
    if (st) *st = e->last_stats;
    return SF_OK;
  }
  if (sf_status rc = fill_stats(e, &local)) return rc;
  std::lock_guard<std::mutex> lk(e->mu);
  local.adam_ms = e->adam_ms;
  // the loss scale and skips of the window's last step
  local.loss_scale = e->last_scale;
  local.skipped = e->last_skipped;
  e->trace.insert(e->trace.end(), e->adam_rows.begin(), e->adam_rows.end());
  e->window_open = false;
  e->last_stats = local;
  if (st) *st = local;
  return SF_OK;
}

sf_status step_impl(sf_engine* e, const void* d_in, const void* d_dy, sf_step_stats* st) {
  const Dims& d = e->d;
  const sf_engine_cfg& c = e->cfg;
  const bool head = (c.flags & SF_ENGINE_HEAD) != 0;
  const bool adam = (c.flags & SF_ENGINE_ADAM) != 0;
  const bool head_host = (c.flags & SF_ENGINE_HEAD_HOST_ADAM) != 0;
  const int nl = e->nl, W = e->W;
  sf_ctx* ctx = e->ctx;
  {
    // a failed Adam job of an earlier (pipelined) step
    std::lock_guard<std::mutex> lk(e->mu);
    if (!e->job_error.empty()) return fail(SF_ERR_HIP, "%s", e->job_error.c_str());
  }
  // a new measurement window: no Adam job is running (synchronous steps end
  // with none; a pipelined window opens after sf_engine_sync drained them)
  const bool new_window = !e->window_open;
  if (new_window) {
    std::lock_guard<std::mutex> lk(e->tmu);
    e->rows.clear();
  }
  e->step += 1;
  // Adam coefficients of this step: the step number of each tensor counts
  // its applied updates (all of them without loss scaling); gradients enter
  // times 1 / S
  const float gscale = 1.0f / e->scale;
  e->coef = adam_coef(e->step, c.lr, c.b1, c.b2, c.eps);
  e->coef.gscale = gscale;
  for (int l = 0; l < nl; ++l) {
    e->lcoef[l] = adam_coef(e->adam_t[l] + 1, c.lr, c.b1, c.b2, c.eps);
    e->lcoef[l].gscale = gscale;
  }
  e->hcoef = adam_coef(e->head_t + 1, c.lr, c.b1, c.b2, c.eps);
  e->ecoef = adam_coef(e->embed_t + 1, c.lr, c.b1, c.b2, c.eps);
  e->hcoef.gscale = e->ecoef.gscale = gscale;
  // this step's verdicts (the slots of step - 2, long complete)
  int32_t* hv = e->lscale ? e->h_ovf + (e->step & 1) * (nl + 2) : nullptr;
  if (hv)
    for (int k = 0; k < nl + 2; ++k) hv[k] = 0;

  hipEvent_t ev0 = new_window ? e->ev_origin : e->ev_start;
  SF_HIP(hipEventRecord(ev0, e->s_comp));
  if (e->lscale) SF_HIP(set_word(e->d_ovf, 0, e->s_comp));
  if (new_window) {
    e->host_t0 = now_ms();
    e->window_open = true;
    std::lock_guard<std::mutex> lk(e->mu);
    e->adam_ms = 0;
    e->adam_rows.clear();
  }
  // The side streams start after everything the caller queued before this call.
  SF_HIP(hipStreamWaitEvent(e->s_h2d, ev0, 0));
  SF_HIP(hipStreamWaitEvent(e->s_up, ev0, 0));
  SF_HIP(hipStreamWaitEvent(e->s_d2h, ev0, 0));
  SF_HIP(hipStreamWaitEvent(e->s_head, ev0, 0));

  auto comp_begin = [&](hipEvent_t* a) -> sf_status {
    *a = timing_event(e);
    if (!*a) return fail(SF_ERR_HIP, "event pool exhausted");
    SF_HIP(hipEventRecord(*a, e->s_comp));
    return SF_OK;
  };
  auto comp_end = [&](hipEvent_t a, hipEvent_t* b_out) -> sf_status {
    hipEvent_t b = timing_event(e);
    if (!b) return fail(SF_ERR_HIP, "event pool exhausted");
    SF_HIP(hipEventRecord(b, e->s_comp));
    if (b_out) *b_out = b;
    return record_interval(e, a, b, 0, 0, kStComp);
  };
  sf_status rc;
  hipEvent_t a, b;

  std::vector<const void*> xin(nl + 1);
  const int32_t* ids = static_cast<const int32_t*>(d_in);
  const bool ck = e->ckpt;
  // layer inputs: all resident, or (checkpointing) a ring of three
  auto xslot = [&](int i) -> char* { return ck ? e->xr[i % 3] : e->x[i]; };
  if (head) {
    if ((rc = comp_begin(&a))) return rc;
    if ((rc = sf_embed_fwd(ctx, c.d_E, ids, xslot(0), e->s_comp))) return rc;
    if ((rc = comp_end(a, &b))) return rc;
    xin[0] = xslot(0);
  } else {
    xin[0] = d_in;
    b = ev0;
  }
  for (int i = 1; i <= nl; ++i) xin[i] = xslot(i);
  // checkpointing: x_i leaves for host memory as soon as it exists (layers
  // 0 .. nl-2; the last layer keeps its saved activations)
  char* hck = static_cast<char*>(c.h_ckpt);
  // (without a head, x_0 is the caller's input and stays where it is)
  auto ckpt_out = [&](int i, hipEvent_t ready) -> sf_status {
    if (!ck || i > nl - 2 || (i == 0 && !head)) return SF_OK;
    hipEvent_t done;
    if (sf_status r = timed_d2h(e, hck + static_cast<size_t>(i) * e->x_bytes, xin[i], e->x_bytes, ready, &done))
      return r;
    SF_HIP(hipEventRecord(e->ev_xfree[i % 3], e->s_d2h));
    return SF_OK;
  };
  if ((rc = ckpt_out(0, b))) return rc;

  // ---------------- forward: layer i in unit i % W, prefetch i + 1
  // (layers below W were uploaded at the end of the previous step, right
  // after their Adam, when that step ran Adam).  Pipelined, the previous
  // step's Adam of layer j may still be running: wait for it before its
  // parameters are read (host copy) or its upload is waited on (units).
  auto await_adam = [&](int j) -> sf_status {
    if (!adam || !e->pipe) return SF_OK;
    std::unique_lock<std::mutex> lk(e->mu);
    e->cv.wait(lk, [&] { return e->adam_done[j] >= e->step - 1 || !e->job_error.empty(); });
    if (!e->job_error.empty()) return fail(SF_ERR_HIP, "%s", e->job_error.c_str());
    return SF_OK;
  };
  // Forward buffers.  A unit's gradient region is idle in the forward once
  // the previous backward's gradients have left, so it holds a layer's
  // parameters too.  By default layer i runs from unit i % W: from its
  // parameter region when i mod 2W < W, from its gradient region otherwise,
  // so an upload waits for the forward of the layer 2W back instead of W
  // back.  Of the last W layers, which stay for the backward, those in a
  // gradient region move to their unit's parameter region by a device copy
  // after their forward.  Without Adam
  // after a preloaded start (params_first) the previous step's last
  // gradients are still leaving the gradient regions as the forward begins:
  // in pages of W layers, pages 0 (the preloaded layers) and 1 then both run
  // from parameter regions (page 1 behind the forward of the layer W back),
  // gradient and parameter regions alternate after that, and layer k of a
  // gradient page takes unit W-1-k, the order in which the previous
  // backward's gradients leave the regions.
  const bool params_first = e->preloaded && !adam;
  auto in_gslot = [&](int i) { return params_first ? (i >= 2 * W && (i / W) % 2 == 0) : (i % (2 * W) >= W); };
  auto gunit = [&](int i) { return params_first ? W - 1 - i % W : i % W; };
  // the layer whose forward an upload of layer j waits for (the buffer's
  // previous user in this step; negative: none)
  auto dep = [&](int j) { return params_first && j < 2 * W ? j - W : j - 2 * W; };
  auto fetch = [&](int j) -> sf_status {
    if (e->preloaded && j < W) return SF_OK;
    if (sf_status r = await_adam(j)) return r;
    if (!in_gslot(j)) return prefetch(e, j);
    const int u = gunit(j);
    // The region's last gradients must be out.  The host waits for that
    // copy rather than the H2D stream: an H2D queue waiting on the D2H
    // queue's event while later gradient copies are still queued sent those
    // copies into a ~13 GB/s mode on the MI355X machine (pipelined steps without
    // Adam, whose last copies run into the next forward).  In synchronous
    // steps and with Adam the copy is long done here.
    SF_HIP(hipEventSynchronize(e->ev_grad_free[u]));
    SF_HIP(hipStreamWaitEvent(e->s_h2d, e->ev_gslot_free[u], 0));  // layer dep(j)'s forward
    if (sf_status r = timed_h2d(e, e->ugrad[u], c.h_params[j], e->L.param_bytes, e->s_h2d)) return r;
    SF_HIP(hipEventRecord(e->ev_gslot_ready[u], e->s_h2d));
    return SF_OK;
  };
  auto adam_ready = [&](int j) {
    if (!adam || !e->pipe) return true;
    std::lock_guard<std::mutex> lk(e->mu);
    return e->adam_done[j] >= e->step - 1;
  };
  // Default order: uploads are queued in layer order as far ahead as the
  // buffers allow (2W - 1 layers); pipelined, one whose update is still
  // running waits for a later turn unless the next forward needs it.  The
  // exception is the first window of layers that run from gradient regions
  // (W .. 2W-1) after a preloaded start (with Adam): those
  // regions are freed by the previous backward from unit W-1 down to unit 0,
  // so each of these layers is queued, highest first, as soon as its update
  // is done rather than behind a lower one still waiting for its region.
  // While the host can wait (the forward of a preloaded layer awaits its
  // update), a first-window upload is queued only once its region is free on
  // the device as well: queued earlier, its wait for the gradients to leave
  // would hold up the work behind it on a hardware queue that the upload
  // stream may share with the streams of Adam's uploads.
  std::vector<char> fetched(nl, 0);
  int next_fetch = 0;  // every layer below it is fetched (or preloaded)
  auto region_free = [&](int j) {
    return !(e->preloaded && j >= W && j < 2 * W) || hipEventQuery(e->ev_grad_free[j % W]) == hipSuccess;
  };
  auto issue_ready = [&](int i, int lim, bool can_wait) -> sf_status {
    if (e->preloaded) {
      for (int j = std::min(lim, 2 * W) - 1; j >= W; --j) {
        if (fetched[j] || (j > i && (!adam_ready(j) || (can_wait && !region_free(j))))) continue;
        if (sf_status r = fetch(j)) return r;
        fetched[j] = 1;
      }
    }
    for (; next_fetch < lim; ++next_fetch) {
      const int j = next_fetch;
      if (fetched[j] || (e->preloaded && j < W)) continue;
      if (j > i && (!adam_ready(j) || (can_wait && !region_free(j)))) break;
      if (sf_status r = fetch(j)) return r;
      fetched[j] = 1;
    }
    return SF_OK;
  };
  // Before the forward of layer i: queue the uploads of the next layers whose
  // update is done.  While the update of a preloaded layer i (re-uploaded by
  // its own Adam) is still running, wait for Adam progress and queue each
  // later layer's upload as soon as its update finishes, so the copies run
  // meanwhile instead of after it.
  auto advance = [&](int i) -> sf_status {
    // an upload may be queued once the forward it waits for (the layer 2W
    // back) has been: its stream wait takes that event's latest record
    const int lim = std::min(nl, i + 2 * W);
    const bool wait_i = adam && e->pipe && e->preloaded && i < W;
    for (;;) {
      if (sf_status r = issue_ready(i, lim, wait_i)) return r;
      if (!wait_i) return SF_OK;
      // a first-window upload held back for its region: poll the device
      bool held = false;
      for (int j = next_fetch; j < lim && !held; ++j) held = j >= W && j < 2 * W && !fetched[j];
      std::unique_lock<std::mutex> lk(e->mu);
      if (!e->job_error.empty()) return fail(SF_ERR_HIP, "%s", e->job_error.c_str());
      const int64_t want = e->step - 1;
      if (e->adam_done[i] >= want) return SF_OK;
      const int nf = next_fetch;
      auto progress = [&] {
        if (e->adam_done[i] >= want || !e->job_error.empty()) return true;
        for (int j = nf; j < lim; ++j)
          if (!fetched[j] && !(e->preloaded && j < W) && e->adam_done[j] >= want && !(j >= W && j < 2 * W))
            return true;
        return false;
      };
      if (held) e->cv.wait_for(lk, std::chrono::microseconds(50), progress);
      else e->cv.wait(lk, progress);
    }
  };
  // params_first: uploads are queued in layer order once the forward they
  // wait for is queued.  While the next one still waits for its region to
  // drain, a later one that does not is queued whenever the H2D queue has
  // run dry, and the forward of layer i goes ahead unless it needs that
  // upload (the host polls the device meanwhile).
  hipEvent_t last_up = nullptr;
  auto done = [&](hipEvent_t ev, bool* yes) -> sf_status {
    const hipError_t q = ev ? hipEventQuery(ev) : hipSuccess;
    if (q != hipSuccess && q != hipErrorNotReady) return fail(SF_ERR_HIP, "%s", hipGetErrorString(q));
    *yes = q == hipSuccess;
    return SF_OK;
  };
  auto advance_pf = [&](int i) -> sf_status {
    const int lim = std::min(nl, i + 2 * W);
    for (;;) {
      int j0 = -1;
      for (int j = W; j < lim && j0 < 0; ++j)
        if (!fetched[j] && dep(j) < i) j0 = j;
      if (j0 < 0) return SF_OK;
      auto ready = [&](int j, bool* yes) -> sf_status {
        *yes = true;
        return in_gslot(j) ? done(e->ev_grad_free[gunit(j)], yes) : SF_OK;
      };
      int pick = -1;
      bool yes = false;
      if (sf_status r = ready(j0, &yes)) return r;
      if (yes) {
        pick = j0;
      } else {
        bool idle = false;
        if (sf_status r = done(last_up, &idle)) return r;
        for (int j = j0 + 1; idle && j < lim && pick < 0; ++j) {
          if (fetched[j] || dep(j) >= i) continue;
          if (sf_status r = ready(j, &yes)) return r;
          if (yes) pick = j;
        }
      }
      if (pick >= 0) {
        if (sf_status r = fetch(pick)) return r;
        fetched[pick] = 1;
        last_up = in_gslot(pick) ? e->ev_gslot_ready[gunit(pick)] : e->ev_param_ready[pick % W];
        continue;
      }
      if (j0 > i) return SF_OK;
      std::this_thread::sleep_for(std::chrono::microseconds(20));
    }
  };
  for (int i = 0; i < nl; ++i) {
    const int u = i % W;
    const bool gs = in_gslot(i);
    const int ug = gunit(i);
    if ((rc = params_first ? advance_pf(i) : advance(i))) return rc;
    if (e->preloaded && i < W && (rc = await_adam(i))) return rc;
    SF_HIP(hipStreamWaitEvent(e->s_comp, gs ? e->ev_gslot_ready[ug] : e->ev_param_ready[u], 0));
    // the output slot held x_{i-2}: its copy to the host must be done
    if (ck && i >= 2) SF_HIP(hipStreamWaitEvent(e->s_comp, e->ev_xfree[(i + 1) % 3], 0));
    if ((rc = comp_begin(&a))) return rc;
    void* sv = ck ? e->sv[i == nl - 1 ? 1 : 0] : e->saved[i];
    if ((rc = sf_layer_fwd(ctx, gs ? e->ugrad[ug] : e->uparam[u], xin[i], xslot(i + 1), sv, e->s_comp))) return rc;
    if (gs && i >= nl - W)  // stays for the backward: into the parameter region (layer i - W is done with it)
      SF_HIP(hipMemcpyAsync(e->uparam[u], e->ugrad[ug], e->L.param_bytes, hipMemcpyDeviceToDevice, e->s_comp));
    if ((rc = comp_end(a, &b))) return rc;
    SF_HIP(hipEventRecord(gs ? e->ev_gslot_free[ug] : e->ev_param_free[u], e->s_comp));
    if ((rc = ckpt_out(i + 1, b))) return rc;
  }
  if (ck && nl >= 2) SF_HIP(hipEventRecord(e->ev_ckpt_out, e->s_d2h));
  // checkpoint of layer i back into slot i % 2 (after every checkpoint left
  // and after the backward that last used the slot)
  auto ckpt_in = [&](int i) -> sf_status {
    if (!ck || i < 0 || i > nl - 2 || (i == 0 && !head)) return SF_OK;
    SF_HIP(hipStreamWaitEvent(e->s_h2d, e->ev_ckpt_out, 0));
    SF_HIP(hipStreamWaitEvent(e->s_h2d, e->ev_cfree[i % 2], 0));
    if (sf_status r = timed_h2d(e, e->cs[i % 2], hck + static_cast<size_t>(i) * e->x_bytes, e->x_bytes, e->s_h2d))
      return r;
    SF_HIP(hipEventRecord(e->ev_cready[i % 2], e->s_h2d));
    return SF_OK;
  };

  // ---------------- head: loss, dx_L, dg_f, dW_lm; their Adam starts now
  const void* dy = d_dy;
  float* hg = c.d_head_grads;
  const size_t VH = static_cast<size_t>(d.V) * d.H;
  // device Adam of a resident head tensor: master/m/v at element offset `off`
  // of d_head_state's three regions, gradient at the same offset of hg
  const size_t NH = 2 * VH + d.H;
  auto dev_adam = [&](size_t off, size_t n, void* out, hipStream_t st_, const AdamCoef& k,
                      const int32_t* skip) -> sf_status {
    float* st = c.d_head_state;
    SF_HIP(adam_device(d.dtype, st + off, st + NH + off, st + 2 * NH + off, hg + off, out, static_cast<int64_t>(n),
                       k.b1, k.b2, k.one_b1, k.one_b2, k.inv_bc1, k.inv_bc2, k.lr, k.eps, st_, k.gscale, skip));
    return SF_OK;
  };
  // With the device Adam of the LM head, the head's last W_lm gradient GEMM
  // and that Adam run on the head stream once the last layer's MLP weight
  // gradients are final: nothing in the step reads them, and beside the
  // start of the backward they would delay the first gradient range, which
  // host Adam waits for.
  const bool head_dev_adam = head && adam && !head_host;
  // with loss scaling the head computes its whole W_lm gradient itself, so
  // that it is checked before any layer's
  const bool defer_dw = head_dev_adam && !e->lscale;
  hipEvent_t head_end = nullptr;
  auto head_update = [&](hipEvent_t mlp_done) -> sf_status {
    hipEvent_t ha = timing_event(e), hb = timing_event(e);
    if (!ha || !hb) return fail(SF_ERR_HIP, "event pool exhausted");
    SF_HIP(hipStreamWaitEvent(e->s_head, head_end, 0));
    SF_HIP(hipStreamWaitEvent(e->s_head, mlp_done, 0));
    SF_HIP(hipEventRecord(ha, e->s_head));
    if (defer_dw)
      if (sf_status r = head_last_dw(ctx, hg + VH + d.H, e->s_head)) return r;
    const int32_t* skip = e->lscale ? e->d_ovf_head : nullptr;
    if (sf_status r = dev_adam(VH, d.H, c.d_gf, e->s_head, e->hcoef, skip)) return r;
    if (sf_status r = dev_adam(VH + d.H, VH, c.d_wlm, e->s_head, e->hcoef, skip)) return r;
    SF_HIP(hipEventRecord(hb, e->s_head));
    SF_HIP(hipEventRecord(e->ev_head_done, e->s_head));
    return record_interval(e, ha, hb, 0, 0, kStSide);
  };
  if (head) {
    // the previous step's device Adam of the LM head (head stream) reads hg
    // and writes d_gf / d_wlm
    SF_HIP(hipStreamWaitEvent(e->s_comp, e->ev_head_done, 0));
    if ((rc = comp_begin(&a))) return rc;
    if ((rc = head_fwd_bwd(ctx, c.d_gf, c.d_wlm, xin[nl], ids, e->d_loss, e->dbuf, hg + VH, hg + VH + d.H,
                           e->s_comp, defer_dw, e->scale)))
      return rc;
    SF_HIP(copy_f32(e->h_loss, e->d_loss, 1, e->s_comp));
    if (e->lscale) {
      // the head's gradients (final gain and LM head, contiguous) decide its
      // own update and are the first part of every layer's verdict
      SF_HIP(nonfinite_flag(hg + VH, static_cast<int64_t>(VH) + d.H, e->d_ovf, e->s_comp));
      SF_HIP(copy_words(reinterpret_cast<uint32_t*>(e->d_ovf_head), reinterpret_cast<const uint32_t*>(e->d_ovf), 1,
                        e->s_comp));
      SF_HIP(copy_words(reinterpret_cast<uint32_t*>(hv + nl), reinterpret_cast<const uint32_t*>(e->d_ovf), 1,
                        e->s_comp));
    }
    if ((rc = comp_end(a, &b))) return rc;
    head_end = b;
    if (head_host) {
      hipEvent_t done;
      if ((rc = timed_d2h(e, c.h_head_grads + VH, hg + VH, (VH + d.H) * 4, b, &done))) return rc;
      if (adam) {
        // the head-upload stream may overwrite d_gf / d_wlm only after the head read them
        SF_HIP(hipStreamWaitEvent(e->s_head, b, 0));
        push_job(e, Job{kHeadLm, -1, -1, done});
      }
    }
    dy = e->dbuf;
  } else if (e->lscale) {
    // the caller's upstream gradient times S seeds the backward
    SF_HIP(scale_storage(d.dtype, d_dy, e->dbuf, static_cast<int64_t>(d.T) * d.H, e->scale, e->s_comp));
    dy = e->dbuf;
  }
  // loss scaling: each layer's fp32 gradient tensors (not the padding
  // between them) are checked after its backward
  FloatSegs gsegs{};
  for (int t = 0; t < SF_NTENSORS; ++t) {
    gsegs.off[t] = static_cast<int64_t>(e->L.grad_off[t] / 4);
    gsegs.n[t] = static_cast<int64_t>(e->L.grad_bytes_t[t] / 4);
  }
  gsegs.count = SF_NTENSORS;

  // ---------------- backward: layer i in unit i % W, prefetch i - W + 1
  // (checkpointing: the input of layer i - 1 comes back meanwhile, and every
  // layer but the last recomputes its forward before its backward)
  for (int i = nl - 1; i >= 0; --i) {
    const int u = i % W;
    const int j = i - W + 1;
    if (j >= 0 && j < nl - W && (rc = prefetch(e, j))) return rc;
    // the slot of layer i - 1 was last read by the backward of layer i + 1
    if ((rc = ckpt_in(i - 1))) return rc;
    SF_HIP(hipStreamWaitEvent(e->s_comp, e->ev_param_ready[u], 0));
    SF_HIP(hipStreamWaitEvent(e->s_comp, e->ev_grad_free[u], 0));
    if ((rc = comp_begin(&a))) return rc;
    const void* xi = xin[i];
    void* sv = ck ? e->sv[1] : e->saved[i];
    if (ck && i < nl - 1) {
      if (i > 0 || head) {
        SF_HIP(hipStreamWaitEvent(e->s_comp, e->ev_cready[i % 2], 0));
        xi = e->cs[i % 2];
      }
      sv = e->sv[0];
      if ((rc = sf_layer_fwd(ctx, e->uparam[u], xi, e->ys, sv, e->s_comp))) return rc;
    }
    hipEvent_t ffn = e->ev_ffn[u], wd = e->ev_wd[u];
    if ((rc = layer_bwd(ctx, e->uparam[u], xi, sv, dy, e->dbuf, reinterpret_cast<float*>(e->ugrad[u]), e->s_comp,
                        ffn, wd)))
      return rc;
    if (head_dev_adam && i == nl - 1 && (rc = head_update(ffn))) return rc;
    if (e->lscale) {
      if (i == e->fault_nonfinite_layer) SF_HIP(set_word(e->d_ovf, 1, e->s_comp));
      SF_HIP(nonfinite_flag_segs(reinterpret_cast<const float*>(e->ugrad[u]), gsegs, e->d_ovf, e->s_comp));
      SF_HIP(copy_words(reinterpret_cast<uint32_t*>(hv + i), reinterpret_cast<const uint32_t*>(e->d_ovf), 1,
                        e->s_comp));
      SF_HIP(hipEventRecord(e->ev_verdict[i], e->s_comp));
    }
    if (ck && i < nl - 1) SF_HIP(hipEventRecord(e->ev_cfree[i % 2], e->s_comp));
    if ((rc = comp_end(a, &b))) return rc;
    dy = e->dbuf;
    SF_HIP(hipEventRecord(e->ev_param_free[u], e->s_comp));
    int k = 0;
    if ((rc = wait_slot(e, &k))) return rc;
    // Gradients leave in ranges and Adam of a range starts as soon as it
    // lands; the MLP weights' gradients (most of a layer) go first: Wd's
    // right after the backward's first weight-gradient GEMM, Wg and Wu's
    // after the MLP half of the backward.
    const size_t gb = e->L.grad_bytes;
    const size_t f0 = e->L.grad_off[SF_WG], fd = e->L.grad_off[SF_WD];
    const size_t f1 = fd + e->L.grad_bytes_t[SF_WD];
    const struct {
      size_t lo, hi;
      hipEvent_t after;
    } parts[4] = {{fd, f1, wd}, {f0, fd, ffn}, {0, f0, b}, {f1, gb, b}};
    std::vector<Job> rj;
    for (const auto& pt : parts) {
      for (size_t lo = pt.lo; lo < pt.hi; lo += e->chunk_bytes) {
        Job jb{kLayer, i, k, nullptr};
        jb.verdict = e->lscale ? e->ev_verdict[i] : nullptr;
        jb.lo = lo;
        jb.hi = std::min(pt.hi, lo + e->chunk_bytes);
        if ((rc = timed_d2h(e, reinterpret_cast<char*>(c.h_grad_slots[k]) + lo, e->ugrad[u] + lo, jb.hi - lo,
                            pt.after, &jb.ready)))
          return rc;
        rj.push_back(jb);
      }
    }
    if (adam) {
      rj.front().first = true;
      rj.back().last = true;
      for (const Job& jb : rj) push_job(e, jb);
    }
    SF_HIP(hipEventRecord(e->ev_grad_free[u], e->s_d2h));
  }

  // ---------------- embedding backward (+ its device Adam)
  // With Adam, the gradient stays sparse: the summed rows of the ids present
  // (embed_bwd_sparse, in the dense gradient's region, which is then unused)
  // and a row map feed the device Adam, which gives rows no token touched a
  // zero gradient -- the same bits as Adam over the dense gradient, without
  // clearing, scattering and re-reading V x H fp32 values.
  const bool sparse_embed = adam && e->sp.total + static_cast<size_t>(d.V) <= VH;
  // loss scaling: the embedding's gradient rows are sums of dx_0, so dx_0
  // decides; the whole step's verdict is then final
  if (e->lscale) {
    if (head) SF_HIP(nonfinite_storage(d.dtype, e->dbuf, static_cast<int64_t>(d.T) * d.H, e->d_ovf, e->s_comp));
    SF_HIP(copy_words(reinterpret_cast<uint32_t*>(hv + nl + 1), reinterpret_cast<const uint32_t*>(e->d_ovf), 1,
                      e->s_comp));
  }
  const int32_t* embed_skip = e->lscale ? e->d_ovf : nullptr;
  if (head && !head_host) {
    if ((rc = comp_begin(&a))) return rc;
    if (sparse_embed) {
      int32_t* hgi = reinterpret_cast<int32_t*>(hg);
      SF_HIP(embed_bwd_sparse(d.dtype, e->dbuf, ids, hgi + e->sp.ids, hg + e->sp.rows, hgi, hgi + e->sp.scratch,
                              static_cast<int>(d.T), d.H, d.V, e->s_comp));
      float* st = c.d_head_state;
      const AdamCoef& k = e->ecoef;
      SF_HIP(embed_adam_sparse(d.dtype, st, st + NH, st + 2 * NH, hg + e->sp.rows, hgi + e->sp.ids, hgi,
                               hgi + e->sp.total, static_cast<int>(d.T), c.d_E, d.V, d.H, k.b1, k.b2, k.one_b1,
                               k.one_b2, k.inv_bc1, k.inv_bc2, k.lr, k.eps, e->s_comp, k.gscale, embed_skip));
    } else {
      if ((rc = sf_embed_bwd(ctx, e->dbuf, ids, hg, e->s_comp))) return rc;
      if (adam && (rc = dev_adam(0, VH, c.d_E, e->s_comp, e->ecoef, embed_skip))) return rc;
    }
    if ((rc = comp_end(a, nullptr))) return rc;
  }
  // ---------------- embedding backward on the host path: sparse rows of the ids present
  if (head && head_host) {
    int32_t* hgi = reinterpret_cast<int32_t*>(hg);
    if ((rc = comp_begin(&a))) return rc;
    SF_HIP(embed_bwd_sparse(d.dtype, e->dbuf, ids, hgi + e->sp.ids, hg + e->sp.rows, hgi, hgi + e->sp.scratch,
                            static_cast<int>(d.T), d.H, d.V, e->s_comp));
    if ((rc = comp_end(a, &b))) return rc;
    hipEvent_t done;
    if ((rc = timed_d2h(e, c.h_head_grads, hg, e->sp.copy_words * 4, b, &done))) return rc;
    if (adam) {
      // the embedding upload must not overtake this step's gather
      SF_HIP(hipStreamWaitEvent(e->s_head, b, 0));
      push_job(e, Job{kEmbed, -1, -1, done});
    }
  }

  SF_HIP(hipStreamSynchronize(e->s_comp));
  // The verdicts are published: count the updates each tensor applied (all
  // of them without loss scaling) and move the loss scale for the next step.
  e->last_scale = e->scale;
  e->last_skipped = 0;
  if (adam) {
    for (int l = 0; l < nl; ++l) {
      const bool skip = hv && hv[l] != 0;
      e->adam_t[l] += skip ? 0 : 1;
      e->last_skipped += skip ? 1 : 0;
    }
    if (head) {
      const bool hs = hv && hv[nl] != 0, es = hv && hv[nl + 1] != 0;
      e->head_t += hs ? 0 : 1;
      e->embed_t += es ? 0 : 1;
      e->last_skipped += (hs ? 1 : 0) + (es ? 1 : 0);
    }
  }
  if (hv) {
    if (hv[nl + 1] != 0) {
      e->scale = std::max(1.0f, e->scale * 0.5f);
      e->good_steps = 0;
    } else if (++e->good_steps >= e->scale_window) {
      if (std::isfinite(e->scale * 2.0f)) e->scale *= 2.0f;
      e->good_steps = 0;
    }
  }
  // the units of layers 0 .. W-1 hold what the next forward reads first:
  // their updated parameters (Adam re-uploads them) or, with the
  // parameters fixed between steps, the ones the backward just used
  e->preloaded = adam || (c.flags & SF_ENGINE_KEEP_TURNAROUND) != 0;
  if (e->pipe) {
    // Adam jobs (and the uploads they queue) go on; the next step waits for
    // them layer by layer, sf_engine_sync for all of them
    std::lock_guard<std::mutex> lk(e->mu);
    if (!e->job_error.empty()) return fail(SF_ERR_HIP, "%s", e->job_error.c_str());
    return SF_OK;
  }
  return close_window(e, st);
}

}  // namespace
}  // namespace sf

extern "C" {

sf_status sf_engine_act_bytes_flags(const sf_shape* shape, int32_t n_layers, int32_t flags, size_t* out) {
  Dims d;
  if (sf_status st = check_shape(shape, &d)) return st;
  if (n_layers < 1 || !out) return fail(SF_ERR_ARG, "n_layers must be >= 1 and out non-NULL");
  const size_t xb = align256(static_cast<size_t>(d.T) * d.H * d.e);
  const size_t sb = saved_layout(d).total;
  if (flags & SF_ENGINE_CKPT)  // input ring 3, checkpoint slots 2, recompute output, 2 saved sets
    *out = 6 * xb + 2 * sb + xb + 256;
  else
    *out = (n_layers + 1) * xb + n_layers * sb + xb + 256;
  return SF_OK;
}

sf_status sf_engine_act_bytes(const sf_shape* shape, int32_t n_layers, size_t* out) {
  return sf_engine_act_bytes_flags(shape, n_layers, 0, out);
}

sf_status sf_engine_create(sf_ctx* ctx, const sf_engine_cfg* cfg, sf_engine** out) {
  if (!ctx || !cfg || !out) return fail(SF_ERR_ARG, "NULL argument");
  *out = nullptr;
  const sf_engine_cfg& c = *cfg;
  const Dims& d = ctx->dims;
  const bool head = (c.flags & SF_ENGINE_HEAD) != 0;
  const bool adam = (c.flags & SF_ENGINE_ADAM) != 0;
  if (c.n_layers < 1) return fail(SF_ERR_ARG, "n_layers must be >= 1");
  if (c.window < 2) return fail(SF_ERR_ARG, "window must be >= 2");
  if (c.n_grad_slots < 2) return fail(SF_ERR_ARG, "n_grad_slots must be >= 2");
  if (head && d.V <= 0) return fail(SF_ERR_ARG, "SF_ENGINE_HEAD needs a context with vocab > 0");
  if (!c.d_pool || !c.d_act || !c.h_params || !c.h_grad_slots)
    return fail(SF_ERR_ARG, "d_pool, d_act, h_params and h_grad_slots are required");
  if ((reinterpret_cast<uintptr_t>(c.d_pool) | reinterpret_cast<uintptr_t>(c.d_act)) & 255u)
    return fail(SF_ERR_ALIGN, "d_pool and d_act must be 256-byte aligned");
  const sf_layout& L = ctx->layout;
  const int W = std::min(c.window, c.n_layers);
  const size_t unit = align256(L.param_bytes) + align256(L.grad_bytes);
  if (c.pool_bytes < static_cast<size_t>(W) * unit)
    return fail(SF_ERR_POOL, "pool has %zu bytes, %d units need %zu", c.pool_bytes, W, W * unit);
  sf_shape shp{};
  shp.hidden = d.H; shp.n_heads = d.nh; shp.n_kv_heads = d.nkv; shp.head_dim = d.d; shp.ffn = d.F;
  shp.vocab = d.V; shp.batch = d.B; shp.seq = d.S; shp.rms_eps = d.eps; shp.rope_base = d.rope_base;
  shp.dtype = d.dtype;
  size_t act = 0;
  if (sf_status st = sf_engine_act_bytes_flags(&shp, c.n_layers, c.flags, &act)) return st;
  const bool ckpt = (c.flags & SF_ENGINE_CKPT) != 0;
  if (ckpt && c.n_layers >= 2) {
    if (!c.h_ckpt) return fail(SF_ERR_ARG, "SF_ENGINE_CKPT needs h_ckpt");
    if (!is_pinned(c.h_ckpt)) return fail(SF_ERR_NOT_PINNED, "h_ckpt is not pinned host memory");
  }
  if (c.act_bytes < act) return fail(SF_ERR_POOL, "activation region has %zu bytes, needs %zu", c.act_bytes, act);
  for (int l = 0; l < c.n_layers; ++l) {
    if (!c.h_params[l]) return fail(SF_ERR_ARG, "h_params[%d] is NULL", l);
    if (!is_pinned(c.h_params[l])) return fail(SF_ERR_NOT_PINNED, "h_params[%d] is not pinned host memory", l);
    if (adam && (!c.h_master || !c.h_m || !c.h_v || !c.h_master[l] || !c.h_m[l] || !c.h_v[l]))
      return fail(SF_ERR_ARG, "SF_ENGINE_ADAM needs h_master/h_m/h_v for layer %d", l);
  }
  for (int k = 0; k < c.n_grad_slots; ++k)
    if (!c.h_grad_slots[k] || !is_pinned(c.h_grad_slots[k]))
      return fail(SF_ERR_NOT_PINNED, "h_grad_slots[%d] is not pinned host memory", k);
  const SparseLayout sp = sparse_layout(d.T, d.H);
  const bool head_host = (c.flags & SF_ENGINE_HEAD_HOST_ADAM) != 0;
  if (head) {
    if (!c.d_E || !c.d_gf || !c.d_wlm || !c.d_head_grads)
      return fail(SF_ERR_ARG, "SF_ENGINE_HEAD needs d_E, d_gf, d_wlm and d_head_grads");
    if (adam && !head_host && !c.d_head_state)
      return fail(SF_ERR_ARG, "SF_ENGINE_HEAD with SF_ENGINE_ADAM needs d_head_state (device Adam of the head)");
  }
  const bool pipe = (c.flags & SF_ENGINE_PIPELINE) != 0;
  if (pipe && head && head_host)
    return fail(SF_ERR_UNSUPPORTED, "SF_ENGINE_PIPELINE does not combine with SF_ENGINE_HEAD_HOST_ADAM");
  const bool lscale = d.dtype == SF_F16;
  if (lscale && head && head_host)
    return fail(SF_ERR_UNSUPPORTED, "SF_F16 loss scaling does not combine with SF_ENGINE_HEAD_HOST_ADAM");
  if (lscale && !(c.loss_scale >= 0.f && std::isfinite(c.loss_scale)))
    return fail(SF_ERR_ARG, "loss_scale must be finite and >= 0 (0: the default)");
  if (lscale && c.scale_window < 0) return fail(SF_ERR_ARG, "scale_window must be >= 0 (0: the default)");
  if (head && head_host) {
    if (!c.h_head_grads) return fail(SF_ERR_ARG, "SF_ENGINE_HEAD_HOST_ADAM needs h_head_grads");
    if (!is_pinned(c.h_head_grads)) return fail(SF_ERR_NOT_PINNED, "h_head_grads is not pinned");
    if (sp.total > static_cast<size_t>(d.V) * d.H)
      return fail(SF_ERR_UNSUPPORTED, "batch*seq too large for the sparse embedding gradient block");
    if (adam) {
      if (!c.h_head_params || !c.h_head_master || !c.h_head_m || !c.h_head_v)
        return fail(SF_ERR_ARG, "SF_ENGINE_HEAD with ADAM needs h_head_params/master/m/v");
      if (!is_pinned(c.h_head_params)) return fail(SF_ERR_NOT_PINNED, "h_head_params is not pinned");
    }
  }

  sf_engine* e = new sf_engine();
  e->ctx = ctx;
  e->cfg = c;
  e->d = d;
  e->L = L;
  e->nl = c.n_layers;
  e->W = W;
  e->pipe = pipe;
  e->adam_done.assign(c.n_layers, 0);
  e->unit_bytes = unit;
  e->x_bytes = align256(static_cast<size_t>(d.T) * d.H * d.e);
  {
    // at most 8 ranges per layer, none under 1 MiB
    const size_t n = std::max<size_t>(1, std::min<size_t>(8, L.grad_bytes >> 20));
    e->chunk_bytes = align256((L.grad_bytes + n - 1) / n);
  }
  e->sp = sp;
  if (head) {
    e->slot_of_row.assign(d.V, -1);
    e->zero_row.assign(d.H, 0.0f);
  }
  e->s_comp = static_cast<hipStream_t>(c.compute_stream);
  auto cleanup = [&](sf_status st) {
    sf_engine_destroy(e);
    return st;
  };
  if (hipStreamCreateWithFlags(&e->s_h2d, hipStreamNonBlocking) != hipSuccess ||
      hipStreamCreateWithFlags(&e->s_d2h, hipStreamNonBlocking) != hipSuccess)
    return cleanup(fail(SF_ERR_HIP, "stream creation failed"));
  if (ctx->side) {
    e->s_head = ctx->side;
  } else {
    if (hipStreamCreateWithFlags(&e->s_head, hipStreamNonBlocking) != hipSuccess)
      return cleanup(fail(SF_ERR_HIP, "stream creation failed"));
    e->own_head = true;
  }
  e->s_up = e->s_head;
  char* pool = static_cast<char*>(c.d_pool);
  for (int u = 0; u < W; ++u) {
    e->uparam.push_back(pool + u * unit);
    e->ugrad.push_back(pool + u * unit + align256(L.param_bytes));
  }
  char* act_p = static_cast<char*>(c.d_act);
  const size_t sb = ctx->saved.total;
  e->ckpt = ckpt;
  if (ckpt) {
    for (int k = 0; k < 3; ++k) e->xr[k] = act_p + k * e->x_bytes;
    for (int k = 0; k < 2; ++k) e->cs[k] = act_p + (3 + k) * e->x_bytes;
    e->ys = act_p + 5 * e->x_bytes;
    act_p += 6 * e->x_bytes;
    for (int k = 0; k < 2; ++k) e->sv[k] = act_p + k * sb;
    act_p += 2 * sb;
  } else {
    for (int i = 0; i <= e->nl; ++i) e->x.push_back(act_p + i * e->x_bytes);
    act_p += (e->nl + 1) * e->x_bytes;
    for (int i = 0; i < e->nl; ++i) e->saved.push_back(act_p + i * sb);
    act_p += e->nl * sb;
  }
  e->dbuf = act_p;
  e->d_loss = reinterpret_cast<float*>(act_p + e->x_bytes);
  // the loss word's 256-byte tail also holds the loss-scaling flags
  e->d_ovf = reinterpret_cast<int32_t*>(act_p + e->x_bytes + 64);
  e->d_ovf_head = reinterpret_cast<int32_t*>(act_p + e->x_bytes + 128);
  e->lscale = lscale;
  e->scale = lscale ? (c.loss_scale > 0.f ? c.loss_scale : 65536.0f) : 1.0f;
  e->scale_window = lscale && c.scale_window > 0 ? c.scale_window : 2000;
  e->last_scale = e->scale;
  e->adam_t.assign(c.n_layers, 0);
  e->lcoef.assign(c.n_layers, AdamCoef{});
  if (lscale) {
    if (hipHostMalloc(reinterpret_cast<void**>(&e->h_ovf), 2 * (c.n_layers + 2) * sizeof(int32_t),
                      hipHostMallocDefault) != hipSuccess)
      return cleanup(fail(SF_ERR_HIP, "pinned loss-scaling flags allocation failed"));
    std::memset(e->h_ovf, 0, 2 * (c.n_layers + 2) * sizeof(int32_t));
    for (int l = 0; l < c.n_layers; ++l) {
      hipEvent_t ev;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
        return cleanup(fail(SF_ERR_HIP, "event creation failed"));
      e->ev_verdict.push_back(ev);
    }
    if (const char* f = std::getenv("SF_FAULT_NONFINITE_LAYER")) e->fault_nonfinite_layer = std::atoi(f);
  }
  if (hipHostMalloc(reinterpret_cast<void**>(&e->h_loss), 256, hipHostMallocDefault) != hipSuccess)
    return cleanup(fail(SF_ERR_HIP, "pinned loss word allocation failed"));
  *e->h_loss = 0.f;
  auto mk = [&](std::vector<hipEvent_t>& v) {
    for (int u = 0; u < W; ++u) {
      hipEvent_t ev;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return false;
      v.push_back(ev);
    }
    return true;
  };
  if (!mk(e->ev_param_ready) || !mk(e->ev_param_free) || !mk(e->ev_grad_free) || !mk(e->ev_gslot_ready) ||
      !mk(e->ev_gslot_free) || !mk(e->ev_ffn) || !mk(e->ev_wd) ||
      hipEventCreateWithFlags(&e->ev_head_done, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&e->ev_start, hipEventDisableTiming) != hipSuccess ||
      hipEventCreate(&e->ev_origin) != hipSuccess)
    return cleanup(fail(SF_ERR_HIP, "event creation failed"));
  if (ckpt) {
    std::vector<hipEvent_t*> evs = {&e->ev_xfree[0], &e->ev_xfree[1], &e->ev_xfree[2], &e->ev_cready[0],
                                    &e->ev_cready[1], &e->ev_cfree[0], &e->ev_cfree[1], &e->ev_ckpt_out};
    for (hipEvent_t* ev : evs)
      if (hipEventCreateWithFlags(ev, hipEventDisableTiming) != hipSuccess)
        return cleanup(fail(SF_ERR_HIP, "event creation failed"));
  }
  // about two steps' worth of timed intervals (a step records at most ~14
  // per layer, two events each): pipelined steps then rarely wait for one
  for (int i = 0; i < 64 * e->nl + 128; ++i) {
    hipEvent_t ev;
    if (hipEventCreate(&ev) != hipSuccess) return cleanup(fail(SF_ERR_HIP, "event creation failed"));
    e->tev_all.push_back(ev);
  }
  e->tev_free = e->tev_all;
  e->rows.reserve(e->tev_all.size());
  if (const char* f = std::getenv("SF_FAULT_ADAM_JOB")) e->fault_adam_job = std::atoll(f);
  e->slot_free.assign(c.n_grad_slots, true);
  // default: every available core but two (the thread that queues device
  // work and the HIP runtime's own), so a preempted Adam worker does not
  // stall a whole gradient range
  const int nt = c.adam_threads > 0 ? c.adam_threads : std::max(1, default_threads() - 2);
  e->n_threads = std::max(1, nt);
  e->pool.reset(new Pool(e->n_threads - 1));
  e->dispatcher = std::thread(dispatcher_loop, e);
  *out = e;
  return SF_OK;
}

sf_status sf_slide_step(sf_engine* e, const void* d_in, const void* d_dy, float* h_loss, sf_step_stats* stats) {
  if (!e) return fail(SF_ERR_ARG, "engine is NULL");
  if (e->failed) return fail(SF_ERR_STATE, "engine is in an error state after an earlier failure");
  const bool head = (e->cfg.flags & SF_ENGINE_HEAD) != 0;
  if (!d_in || (!head && !d_dy)) return fail(SF_ERR_ARG, "d_in (and d_dy without a head) are required");
  if (!aligned16(d_in) || (d_dy && !aligned16(d_dy))) return fail(SF_ERR_ALIGN, "inputs must be 16-byte aligned");
  const double t0 = now_ms();
  sf_status rc = step_impl(e, d_in, d_dy, stats);
  if (rc != SF_OK) {
    // Leave no work in flight: finish the streams and any queued Adam jobs.
    const std::string msg = sf_last_error();
    (void)hipStreamSynchronize(e->s_comp);
    (void)hipStreamSynchronize(e->s_d2h);
    drain(e);
    (void)hipStreamSynchronize(e->s_h2d);
    (void)hipStreamSynchronize(e->s_up);
    (void)hipStreamSynchronize(e->s_head);
    e->failed = true;
    return fail(rc, "%s", msg.c_str());
  }
  float loss = 0.f;
  if (head) {
    // written on the compute stream, which the step has synchronised
    loss = *static_cast<volatile float*>(e->h_loss);
    if (h_loss) *h_loss = loss;
  }
  if (stats) {
    stats->wall_ms = now_ms() - t0;
    stats->loss = loss;
    stats->loss_scale = e->last_scale;
    stats->skipped = e->last_skipped;
  }
  return SF_OK;
}

sf_status sf_engine_sync(sf_engine* e, sf_step_stats* stats) {
  if (!e) return fail(SF_ERR_ARG, "engine is NULL");
  if (e->failed) return fail(SF_ERR_STATE, "engine is in an error state after an earlier failure");
  if (sf_status rc = close_window(e, stats)) {
    e->failed = true;
    return rc;
  }
  return SF_OK;
}

sf_status sf_engine_layer_input(sf_engine* e, int32_t layer, void** d_x) {
  if (!e || !d_x || layer < 0 || layer > e->nl) return fail(SF_ERR_ARG, "bad argument");
  if (e->ckpt) {
    // only the last layer's input and output stay on the device
    if (layer < e->nl - 1) return fail(SF_ERR_UNSUPPORTED, "layer %d's input lives in host memory (checkpointing)", layer);
    *d_x = e->xr[layer % 3];
    return SF_OK;
  }
  *d_x = e->x[layer];
  return SF_OK;
}

sf_status sf_engine_dx0(sf_engine* e, void** d_dx0) {
  if (!e || !d_dx0) return fail(SF_ERR_ARG, "bad argument");
  *d_dx0 = e->dbuf;
  return SF_OK;
}

sf_status sf_engine_trace(sf_engine* e, double* out, int32_t capacity, int32_t* n_rows) {
  if (!e || !n_rows || capacity < 0 || (capacity > 0 && !out)) return fail(SF_ERR_ARG, "bad argument");
  const size_t n = e->trace.size();
  *n_rows = static_cast<int32_t>(n);
  const size_t m = std::min(n, static_cast<size_t>(capacity));
  for (size_t i = 0; i < m; ++i) {
    const TraceRow& r = e->trace[i];
    out[4 * i + 0] = r.kind;
    out[4 * i + 1] = r.start;
    out[4 * i + 2] = r.end;
    out[4 * i + 3] = r.info;
  }
  return SF_OK;
}

sf_status sf_engine_counters(sf_engine* e, int64_t* out, int32_t n) {
  if (!e || !out || n < 0) return fail(SF_ERR_ARG, "bad argument");
  int64_t v[5];
  {
    std::lock_guard<std::mutex> lk(e->tmu);
    size_t live = 0;
    for (auto& q : e->live) live += q.size();
    v[0] = static_cast<int64_t>(e->tev_all.size());
    v[1] = static_cast<int64_t>(e->tev_free.size());
    v[2] = static_cast<int64_t>(live);
    v[3] = static_cast<int64_t>(e->rows.size());
    v[4] = e->blocked_waits;
  }
  for (int32_t i = 0; i < n && i < 5; ++i) out[i] = v[i];
  return SF_OK;
}

sf_status sf_engine_destroy(sf_engine* e) {
  if (!e) return SF_OK;
  if (e->dispatcher.joinable()) {
    {
      std::lock_guard<std::mutex> lk(e->mu);
      e->stop = true;
    }
    e->cv.notify_all();
    e->dispatcher.join();
  }
  e->pool.reset();
  for (hipStream_t s : {e->s_h2d, e->s_d2h, e->s_head})
    if (s) (void)hipStreamSynchronize(s);
  for (auto* v : {&e->ev_param_ready, &e->ev_param_free, &e->ev_grad_free, &e->ev_gslot_ready, &e->ev_gslot_free,
                  &e->ev_ffn, &e->ev_wd, &e->tev_all, &e->ev_verdict})
    for (hipEvent_t ev : *v) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : {e->ev_xfree[0], e->ev_xfree[1], e->ev_xfree[2], e->ev_cready[0], e->ev_cready[1],
                        e->ev_cfree[0], e->ev_cfree[1], e->ev_ckpt_out, e->ev_head_done, e->ev_start, e->ev_origin})
    if (ev) (void)hipEventDestroy(ev);
  for (hipStream_t s : {e->s_h2d, e->s_d2h, e->own_head ? e->s_head : nullptr})
    if (s) (void)hipStreamDestroy(s);
  if (e->h_loss || e->h_ovf) {
    if (e->s_comp) (void)hipStreamSynchronize(e->s_comp);
    if (e->h_loss) (void)hipHostFree(e->h_loss);
    if (e->h_ovf) (void)hipHostFree(e->h_ovf);
  }
  delete e;
  return SF_OK;
}

}  // extern "C"
