// hc_ctx.hip — host side of the C ABI declared in include/hc.h.
//
// The CPU only manages resources and lifetimes; every per-selection decision
// (ranking, lookup, replacement, transfer) is made by the kernels (page "From
// 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading", section
// "Decision three: let the GPU manage the hot cache directly").  Long-lived
// buffers are sized exactly (section "Ten sessions exposed a
// physical-allocation problem"): the device workspace is one caller-owned
// block whose exact size hc_workspace_bytes reports, and the host row store
// is one exact-size pinned allocation per (session, layer).  Creation is
// all-or-nothing and destruction first waits for every enqueued step (the
// page "Making KV offload correct", sections "A grouped allocation is a
// transaction" and "Response completion is not copy completion").
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "hc_internal.h"
#ifdef HC_TEST_HOOKS
#include "hc_test.h"
#endif

using namespace hc;

namespace {

constexpr uint64_t kAlign = 256;

struct Layout {
  uint64_t pos2slot, slot2pos, last_use, oq, qlive, cnt, seg, cand, sel_slot, miss_pos,
      victim, miss_idx, miss_old, host_tab, hot, ring, refbits, total;
};

// Score-scan segments per selection unit: enough for the longest history in
// chunks of 2,048 positions, at most kMaxSegs (longer histories use longer
// segments).
uint64_t max_segs_of(uint64_t hcap) {
  const uint64_t n = (hcap + 2047) / 2048;
  return n < (uint64_t)kMaxSegs ? n : (uint64_t)kMaxSegs;
}

// Sizes of hc_config before the recent-ring fields and before `queries` were
// added; both are accepted (no ring, one query).
constexpr uint32_t kConfigSizeNoRing = offsetof(hc_config, ring_rows);
constexpr uint32_t kConfigSizeOneQuery = offsetof(hc_config, queries);

// A full-size copy of the caller's config (missing fields zero); false if the
// struct size is none of the known forms.
bool normalize(const hc_config* in, hc_config* out) {
  if (!in) return false;
  const uint32_t n = in->struct_size;
  if (n != sizeof(hc_config) && n != kConfigSizeNoRing && n != kConfigSizeOneQuery) return false;
  *out = hc_config{};
  std::memcpy(out, in, n);
  out->struct_size = sizeof(hc_config);
  if (out->queries == 0) out->queries = 1;
  return true;
}

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_config(const hc_config* c) {
  if (!c || c->struct_size != sizeof(hc_config)) return false;
  if (c->ring_rows == 0 ? c->copyback_rows != 0
                        : (c->ring_rows > HC_MAX_RING_ROWS || c->copyback_rows < 1 ||
                           c->copyback_rows > c->ring_rows))
    return false;
  if (c->n_sessions < 1 || c->n_sessions > (uint32_t)kMaxSessions) return false;
  if (c->n_layers < 1 || c->layers_per_select < 1) return false;
  if (c->top_k < 1 || c->top_k > HC_MAX_TOPK) return false;
  if (c->queries < 1 || c->queries > HC_MAX_QUERIES) return false;
  const uint64_t qk = (uint64_t)c->queries * c->top_k;
  if (qk > HC_MAX_ROUND_ROWS) return false;
  if (c->cache_slots < qk || c->cache_slots > HC_MAX_SLOTS) return false;
  // positions < 2^31 - 2^19 keep -(C + 1 + position) inside int32
  if (c->max_positions < c->top_k || c->max_positions > (1ull << 31) - (1ull << 19)) return false;
  if (c->flags != 0) return false;
  if (c->replacement > HC_REPLACE_CLOCK) return false;
  const uint64_t layers = (uint64_t)c->n_sessions * c->n_layers;
  if (layers * c->queries > 60000) return false;  // one gather grid row per layer and query
  // in 64 bits: L + R - 1 can pass 2^32
  const uint64_t G = ((uint64_t)c->n_layers + c->layers_per_select - 1) / c->layers_per_select;
  if ((uint64_t)c->n_sessions * G > (uint64_t)kMaxUnits) return false;
  return true;
}

uint64_t queue_cap(uint64_t C) { return (2 * C + 3) / 4 * 4; }
// Words of a unit's live-entry bitmap: a bit per queue entry, in 64-bit groups.
uint64_t qlive_words(uint64_t C) { return (queue_cap(C) + 63) / 64 * 2; }

Layout layout_of(const hc_config* c) {
  const uint64_t S = c->n_sessions, L = c->n_layers;
  const uint64_t G = (L + c->layers_per_select - 1) / c->layers_per_select;
  const uint64_t U = S * G, C = c->cache_slots, K = c->top_k, hcap = c->max_positions;
  const uint64_t Q = c->queries, SU = U * Q;  // selection units: one per query row
  Layout lo{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = align_up(off);
    off = o + bytes;
    return o;
  };
  lo.pos2slot = take(U * hcap * 4);
  lo.slot2pos = take(U * C * 4);
  lo.last_use = take(U * C * 4);
  lo.oq = take(U * 2 * queue_cap(C) * 8);
  lo.qlive = take(U * qlive_words(C) * 4);
  lo.cnt = take(SU * kCntStride * 4);
  lo.seg = take(SU * max_segs_of(hcap) * 8);
  lo.cand = take(SU * hcap * sizeof(Ent));
  lo.sel_slot = take(SU * K * 4);
  lo.miss_pos = take(SU * K * 4);
  lo.victim = take(SU * K * 4);
  lo.miss_idx = take(SU * K * 4);
  lo.miss_old = take(SU * K * 4);
  lo.host_tab = take(S * L * 8);
  lo.hot = take(S * L * C * kSlotStride);
  lo.ring = take(S * L * (uint64_t)c->ring_rows * kRow);
  lo.refbits = take(U * ((C + 31) / 32) * 4);
  lo.total = align_up(off);
  return lo;
}

// Restores the calling thread's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
    // the launchers read hipGetLastError(): leave no error of this call (or of
    // the caller's earlier HIP calls) behind for them to take as their own
    (void)hipGetLastError();
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

__global__ void k_init(DevState d, int64_t n_pos, int64_t n_slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < n_pos; i += stride) d.pos2slot[i] = -1;
  for (int64_t i = i0; i < n_slots; i += stride) {
    d.slot2pos[i] = -1;
    d.last_use[i] = -1;
  }
  const int64_t sel_units = (int64_t)d.S * d.G * d.Q;
  for (int64_t i = i0; i < sel_units * d.K; i += stride) d.sel_slot[i] = 0;
  for (int64_t i = i0; i < sel_units * kCntStride; i += stride) {
    const int64_t f = i % kCntStride;
    // no window, no compaction prepared; empty LRU queues
    d.cnt[i] = f == kCntWinLo || f == kCntWinHi || f == kCntCntStep ? -1 : 0;
  }
  // the first step's cut histograms (see launch_cold_cut)
  if (d.hcap >= kColdMinPositions)
    for (int64_t i = i0; i < sel_units * kBins1; i += stride)
      reinterpret_cast<uint32_t*>(d.cand + (i / kBins1) * d.hcap)[i % kBins1] = 0u;
  const int64_t ref_words = (int64_t)d.S * d.G * ((d.C + 31) / 32);
  for (int64_t i = i0; i < ref_words; i += stride) d.refbits[i] = 0;
}

// Scratch of hc_attend_cached_noalloc: the attention's split partials, for
// callers that cannot allocate.  Each GPU the library runs on holds its own
// copy for the life of the process.  In host code `scratch` only names the
// symbol; its device address, per device, comes from hipGetSymbolAddress at
// context creation and is the only form passed to kernels.
static __device__ __align__(256) uint8_t scratch[HC_ATTEND_STATIC_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once set

// Looks up the current device's address of `scratch` once; false on failure.
bool init_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev]) return true;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return false;
  g_scratch_ptr[dev] = p;
  return true;
}

void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[dev];
}

}  // namespace

namespace hc {
hipError_t launch_init(const DevState& d, hipStream_t st) {
  const int64_t units = (int64_t)d.S * d.G;
  hipLaunchKernelGGL(k_init, dim3(1024), dim3(256), 0, st, d, units * d.hcap, units * d.C);
  return hipGetLastError();
}
}  // namespace hc

struct hc_ctx {
  hc_config cfg;
  DevState dev;
  Layout lo;
  uint8_t* ws = nullptr;
  std::vector<uint8_t*> host_rows;   // S*L pinned buffers
  uint64_t t = 0;                    // steps issued
  std::vector<uint64_t> last_len;    // previous hist_len per session
  // recent ring, per session: appended positions [first, end), of which
  // [first, copied) have a copyback enqueued; first = -1 before any append
  std::vector<int64_t> first, end, copied;
  uint64_t* host_count = nullptr;    // pinned [S], written by the device after copybacks
  uint64_t* host_count_dev = nullptr;
  uint32_t* err = nullptr;           // pinned [kErrKinds]: set by kernels on inconsistent state
  uint32_t* err_dev = nullptr;
  bool poisoned = false;
  bool enqueued = false;
  bool appended_since_step = false;  // an hc_append after the last hc_step
  hipStream_t last_stream = nullptr; // stream of the last enqueued work
  hipEvent_t done = nullptr;         // recorded after all enqueued work; device-scope only
  hipEvent_t host_done = nullptr;    // system-scope: the host's waits (host_wait)
  hipStream_t sync_stream = nullptr; // private, non-blocking: where host_done is recorded
#ifdef HC_TEST_HOOKS
  bool test_fail_launch = false;     // the next hc_step fails before its first launch
  bool test_poison = false;          // sentinel over victim slots before each gather
#endif
  // profiling: a (start, stop) event pair per stage and step, attached to the
  // stage's first and last kernel dispatch
  std::vector<hipEvent_t> prof;
  uint32_t prof_cap = 0, prof_used = 0;
};

namespace {

// Pinned host memory the library holds (all contexts), for the tests of
// all-or-nothing creation.
std::atomic<uint64_t> g_pinned_bytes{0};
#ifdef HC_TEST_HOOKS
std::atomic<int64_t> g_fail_pinned{-1};   // pinned allocations to grant before one fails
#endif

// Mapped pinned host memory of `bytes`, or nullptr.
void* pinned_alloc(uint64_t bytes) {
#ifdef HC_TEST_HOOKS
  if (g_fail_pinned.load() >= 0 && g_fail_pinned.fetch_sub(1) == 0) return nullptr;
#endif
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes, hipHostMallocMapped) != hipSuccess || !p) return nullptr;
  g_pinned_bytes += bytes;
  return p;
}

void pinned_free(void* p, uint64_t bytes) {
  if (!p) return;
  (void)hipHostFree(p);
  g_pinned_bytes -= bytes;
}

void free_host(hc_ctx* c) {
  const uint64_t row_bytes = c->cfg.max_positions * (uint64_t)kRow;
  for (uint8_t* p : c->host_rows) pinned_free(p, row_bytes);
  c->host_rows.clear();
  pinned_free(c->host_count, c->cfg.n_sessions * sizeof(uint64_t));
  c->host_count = c->host_count_dev = nullptr;
  pinned_free(c->err, kErrKinds * sizeof(uint32_t));
  c->err = c->err_dev = nullptr;
}

// Orders work enqueued on `st` after everything the context enqueued on
// another stream before (entry points may be called on different streams).
hipError_t order_after_last(hc_ctx* c, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (c->enqueued && st != c->last_stream) e = hipStreamWaitEvent(st, c->done, 0);
  c->last_stream = st;
  return e;
}

// Waits on the host until everything the context enqueued has completed, its
// writes to device memory visible to the host.  `done`, recorded after every
// call to order the context's streams, has no system-scope fence (with one,
// each record cost about 2 us of device time per step), so the system-scope
// event is recorded here, on a private stream that waits for `done` first.
hipError_t host_wait(hc_ctx* c) {
  hipError_t e = hipStreamWaitEvent(c->sync_stream, c->done, 0);
  if (e == hipSuccess) e = hipEventRecord(c->host_done, c->sync_stream);
  if (e == hipSuccess) e = hipEventSynchronize(c->host_done);
  return e;
}

void destroy_sync(hc_ctx* c) {
  if (c->done) (void)hipEventDestroy(c->done);
  if (c->host_done) (void)hipEventDestroy(c->host_done);
  if (c->sync_stream) (void)hipStreamDestroy(c->sync_stream);
  c->done = c->host_done = nullptr;
  c->sync_stream = nullptr;
}

void free_prof(hc_ctx* c) {
  for (hipEvent_t e : c->prof)
    if (e) (void)hipEventDestroy(e);
  c->prof.clear();
  c->prof_cap = c->prof_used = 0;
}

hc_status fail_hip(hc_ctx* c) {
  c->poisoned = true;
  return HC_E_HIP;
}

// A kernel reported an inconsistent device state (every kernel that has
// completed has written its report by now): the context is poisoned.
bool device_error(hc_ctx* c) {
  const volatile uint32_t* e = c->err;
  bool any = false;
  for (int k = 0; k < kErrKinds; ++k) any |= e[k] != 0;
  if (any) c->poisoned = true;
  return any;
}

// Enqueues the copyback of every session with at least `min_pending` appended
// rows not yet in host RAM (plus the count update) and marks them copied.
hipError_t copy_back(hc_ctx* c, hipStream_t st, int64_t min_pending) {
  CopybackArgs a{};
  for (uint32_t s = 0; s < c->cfg.n_sessions; ++s) {
    const int64_t pending = c->end[s] - c->copied[s];
    if (c->first[s] < 0 || pending == 0 || pending < min_pending) continue;
    a.lo[s] = (uint32_t)c->copied[s];
    a.hi[s] = (uint32_t)c->end[s];
    a.max_rows = std::max(a.max_rows, a.hi[s] - a.lo[s]);
  }
  hipError_t e = launch_copyback(c->dev, a, c->host_count_dev, st);
  if (e == hipSuccess)
    for (uint32_t s = 0; s < c->cfg.n_sessions; ++s)
      if (a.hi[s] > a.lo[s]) c->copied[s] = a.hi[s];
  return e;
}

}  // namespace

extern "C" {

hc_status hc_workspace_bytes(const hc_config* cfg_in, uint64_t* bytes) {
  hc_config full;
  const hc_config* cfg = &full;
  if (!normalize(cfg_in, &full) || !valid_config(cfg) || !bytes) return HC_E_INVAL;
  *bytes = layout_of(cfg).total;
  return HC_OK;
}

hc_status hc_create(const hc_config* cfg_in, void* dev_workspace, uint64_t ws_bytes,
                    hc_ctx** out) {
  if (out) *out = nullptr;
  hc_config full;
  const hc_config* cfg = &full;
  if (!normalize(cfg_in, &full) || !valid_config(cfg) || !out || !dev_workspace)
    return HC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(dev_workspace) % kAlign) return HC_E_INVAL;
  const Layout lo = layout_of(cfg);
  if (ws_bytes < lo.total) return HC_E_NOMEM;
  DeviceGuard dg(cfg->device);
  if (!dg.ok) return HC_E_INVAL;
  // the no-allocation attention's scratch address on this device (once per device)
  if (!init_scratch(cfg->device)) return HC_E_HIP;

  hc_ctx* c = new (std::nothrow) hc_ctx();
  if (!c) return HC_E_NOMEM;
  c->cfg = *cfg;
  c->lo = lo;
  c->ws = static_cast<uint8_t*>(dev_workspace);
  const uint32_t S = cfg->n_sessions, L = cfg->n_layers, R = cfg->layers_per_select;
  const uint32_t G = (uint32_t)(((uint64_t)L + R - 1) / R);   // <= HC_MAX_UNITS, checked
  c->last_len.assign(S, 0);
  c->first.assign(S, -1);
  c->end.assign(S, 0);
  c->copied.assign(S, 0);

  // pinned, mapped host rows: one exact-size buffer per (session, layer)
  const uint64_t row_bytes = cfg->max_positions * (uint64_t)kRow;
  std::vector<const uint8_t*> dev_ptrs(S * (size_t)L);
  c->host_rows.assign(S * (size_t)L, nullptr);
  hc_status st = HC_OK;
  for (size_t i = 0; i < c->host_rows.size() && st == HC_OK; ++i) {
    void* p = pinned_alloc(row_bytes);
    if (!p) {
      st = HC_E_NOMEM;
      break;
    }
    c->host_rows[i] = static_cast<uint8_t*>(p);
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess || !dp) st = HC_E_HIP;
    dev_ptrs[i] = static_cast<const uint8_t*>(dp);
  }
  if (st == HC_OK && cfg->ring_rows) {
    void* p = pinned_alloc(S * sizeof(uint64_t));
    if (!p) {
      st = HC_E_NOMEM;
    } else {
      c->host_count = static_cast<uint64_t*>(p);
      std::memset(c->host_count, 0, S * sizeof(uint64_t));
      void* dp = nullptr;
      if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess || !dp) st = HC_E_HIP;
      c->host_count_dev = static_cast<uint64_t*>(dp);
    }
  }
  if (st == HC_OK) {
    void* p = pinned_alloc(kErrKinds * sizeof(uint32_t));
    if (!p) {
      st = HC_E_NOMEM;
    } else {
      c->err = static_cast<uint32_t*>(p);
      std::memset(c->err, 0, kErrKinds * sizeof(uint32_t));
      void* dp = nullptr;
      if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess || !dp) st = HC_E_HIP;
      c->err_dev = static_cast<uint32_t*>(dp);
    }
  }
  if (st == HC_OK &&
      hipEventCreateWithFlags(&c->done, hipEventDisableTiming | hipEventDisableSystemFence) !=
          hipSuccess)
    st = HC_E_HIP;
  if (st == HC_OK && hipEventCreateWithFlags(&c->host_done, hipEventDisableTiming) != hipSuccess)
    st = HC_E_HIP;
  if (st == HC_OK && hipStreamCreateWithFlags(&c->sync_stream, hipStreamNonBlocking) != hipSuccess)
    st = HC_E_HIP;

  DevState& d = c->dev;
  d.S = (int32_t)S;
  d.L = (int32_t)L;
  d.R = (int32_t)R;
  d.G = (int32_t)G;
  d.K = (int32_t)cfg->top_k;
  d.C = (int32_t)cfg->cache_slots;
  d.Q = (int32_t)cfg->queries;
  d.hcap = (int64_t)cfg->max_positions;
  uint8_t* w = c->ws;
  d.pos2slot = reinterpret_cast<int32_t*>(w + lo.pos2slot);
  d.slot2pos = reinterpret_cast<int32_t*>(w + lo.slot2pos);
  d.last_use = reinterpret_cast<int32_t*>(w + lo.last_use);
  d.oq = reinterpret_cast<int2*>(w + lo.oq);
  d.qcap = (int32_t)queue_cap(cfg->cache_slots);
  d.qlive = reinterpret_cast<uint32_t*>(w + lo.qlive);
  d.qlive_words = (int32_t)qlive_words(cfg->cache_slots);
  d.cnt = reinterpret_cast<int32_t*>(w + lo.cnt);
  d.seg = reinterpret_cast<int2*>(w + lo.seg);
  d.max_segs = (int32_t)max_segs_of(cfg->max_positions);
  d.err = c->err_dev;
  d.cand = reinterpret_cast<Ent*>(w + lo.cand);
  d.sel_slot = reinterpret_cast<int32_t*>(w + lo.sel_slot);
  d.miss_pos = reinterpret_cast<int32_t*>(w + lo.miss_pos);
  d.victim = reinterpret_cast<int32_t*>(w + lo.victim);
  d.miss_idx = reinterpret_cast<int32_t*>(w + lo.miss_idx);
  d.miss_old = reinterpret_cast<int32_t*>(w + lo.miss_old);
  d.host = reinterpret_cast<const uint8_t* const*>(w + lo.host_tab);
  d.hot = w + lo.hot;
  d.ring = w + lo.ring;
  d.ring_rows = (int32_t)cfg->ring_rows;
  d.policy = (int32_t)cfg->replacement;
  d.refbits = reinterpret_cast<uint32_t*>(w + lo.refbits);

  if (st == HC_OK &&
      hipMemcpy(w + lo.host_tab, dev_ptrs.data(), dev_ptrs.size() * sizeof(void*),
                hipMemcpyHostToDevice) != hipSuccess)
    st = HC_E_HIP;
  // initialise on the null stream and wait for that work alone (not for every
  // stream of the device)
  if (st == HC_OK && launch_init(d, nullptr) != hipSuccess) st = HC_E_HIP;
  if (st == HC_OK && hipEventRecord(c->host_done, nullptr) != hipSuccess) st = HC_E_HIP;
  if (st == HC_OK && hipEventSynchronize(c->host_done) != hipSuccess) st = HC_E_HIP;
  if (st != HC_OK) {
    free_host(c);
    destroy_sync(c);
    delete c;
    return st;
  }
  *out = c;
  return HC_OK;
}

uint8_t* hc_host_rows(hc_ctx* c, uint32_t session, uint32_t layer) {
  if (!c || session >= c->cfg.n_sessions || layer >= c->cfg.n_layers) return nullptr;
  return c->host_rows[(size_t)session * c->cfg.n_layers + layer];
}

hc_status hc_step(hc_ctx* c, void* stream, const float* d_scores, uint64_t score_stride,
                  const uint64_t* hist_len, uint16_t* d_out, int32_t* d_sel, int32_t* d_trace) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  if (device_error(c)) return HC_E_DEVICE;   // reported by an earlier step that has completed
  if (!d_scores || !hist_len || !d_sel) return HC_E_INVAL;   // d_out may be NULL
  const uint32_t S = c->cfg.n_sessions;
  uint64_t max_len = 0;
  for (uint32_t s = 0; s < S; ++s) {
    const uint64_t h = hist_len[s];
    if (h < c->cfg.top_k || h > c->cfg.max_positions || h < c->last_len[s]) return HC_E_INVAL;
    if (c->first[s] >= 0 && h > (uint64_t)c->end[s]) return HC_E_INVAL;  // rows not appended yet
    max_len = std::max(max_len, h);
  }
  if (score_stride < max_len) return HC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(d_out) % 16) return HC_E_INVAL;
  if (c->t >= 0x7FFFFFFFull) return HC_E_INVAL;  // last-use stamps are int32

  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  StepArgs a;
  a.t = (int32_t)c->t;
  for (uint32_t s = 0; s < (uint32_t)kMaxSessions; ++s) {
    a.hist_len[s] = s < S ? (uint32_t)hist_len[s] : 0u;
    a.ring_lo[s] = kNoRing;
    // the ring holds the session's last ring_rows appended positions
    if (s < S && c->first[s] >= 0)
      a.ring_lo[s] = (uint32_t)std::max(c->first[s], c->end[s] - (int64_t)c->cfg.ring_rows);
  }
  const bool vec4 =
      (reinterpret_cast<uintptr_t>(d_scores) % 16 == 0) && (score_stride % 4 == 0);

  const bool prof = c->prof_used < c->prof_cap;
  StageEv ev[HC_NUM_STAGES];
  if (prof)
    for (int i = 0; i < HC_NUM_STAGES; ++i) {
      ev[i].start = c->prof[((size_t)c->prof_used * HC_NUM_STAGES + i) * 2];
      ev[i].stop = c->prof[((size_t)c->prof_used * HC_NUM_STAGES + i) * 2 + 1];
    }
  const StageEv ev_scan = ev[HC_STAGE_TOPK_SCAN], ev_sel = ev[HC_STAGE_SELECT];
  DevState d = c->dev;

  hipError_t e = order_after_last(c, st);
#ifdef HC_TEST_HOOKS
  if (c->test_fail_launch && e == hipSuccess) e = hipErrorLaunchFailure;   // as if a launch failed
  c->test_fail_launch = false;
#endif
  const bool cold = c->t == 0 && d.hcap >= kColdMinPositions;
  if (cold && e == hipSuccess)
    e = launch_cold_cut(d, a, d_scores, score_stride, (int64_t)max_len, st,
                        StageEv{ev_scan.start, nullptr});
  if (e == hipSuccess)
    e = launch_topk_scan(d, a, d_scores, score_stride, (int64_t)max_len, vec4, st,
                         StageEv{cold ? nullptr : ev_scan.start, ev_scan.stop});
  if (e == hipSuccess)
    e = launch_select(d, a, d_scores, score_stride, (int64_t)max_len, d_sel, d_trace, st,
                      StageEv{ev_sel.start, d.Q > 1 ? nullptr : ev_sel.stop});
  if (e == hipSuccess && d.Q > 1)
    e = launch_round(d, a, d_sel, d_trace, st, StageEv{nullptr, ev_sel.stop});
#ifdef HC_TEST_HOOKS
  if (e == hipSuccess && c->test_poison) e = launch_poison(d, st);
#endif
  if (e == hipSuccess) e = launch_gather(d, d_out, a.t, d_trace, st, ev[HC_STAGE_GATHER]);
  if (e == hipSuccess) e = hipEventRecord(c->done, st);
  c->enqueued = true;
#ifdef HC_TEST_HOOKS
  c->dev.test_force = 0;   // a forced report concerns one step
#endif
  if (e != hipSuccess) return fail_hip(c);
  if (prof) ++c->prof_used;
  for (uint32_t s = 0; s < S; ++s) c->last_len[s] = hist_len[s];
  ++c->t;
  c->appended_since_step = false;
  return HC_OK;
}

hc_status hc_append(hc_ctx* c, void* stream, const uint8_t* d_rows, const uint64_t* pos) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  if (device_error(c)) return HC_E_DEVICE;
  if (!c->cfg.ring_rows || !d_rows || !pos) return HC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(d_rows) % 16) return HC_E_INVAL;
  const uint32_t S = c->cfg.n_sessions;
  AppendArgs a{};
  for (uint32_t s = 0; s < (uint32_t)kMaxSessions; ++s) a.entry[s] = kNoRing;
  for (uint32_t s = 0; s < S; ++s) {
    const uint64_t p = pos[s];
    if (p == HC_NO_APPEND) continue;
    if (p >= c->cfg.max_positions) return HC_E_INVAL;
    if (c->first[s] < 0 ? p < c->last_len[s] : p != (uint64_t)c->end[s]) return HC_E_INVAL;
    a.entry[s] = (uint32_t)(p % c->cfg.ring_rows);
  }
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the entry being overwritten left the ring copyback_rows <= ring_rows
  // appends ago, so its copyback is already enqueued ahead of this launch
  hipError_t e = order_after_last(c, st);
  if (e == hipSuccess) e = launch_append(c->dev, a, d_rows, st);
  c->enqueued = true;
  c->appended_since_step = true;
  if (e == hipSuccess) {
    for (uint32_t s = 0; s < S; ++s) {
      if (pos[s] == HC_NO_APPEND) continue;
      if (c->first[s] < 0) c->first[s] = c->copied[s] = (int64_t)pos[s];
      c->end[s] = (int64_t)pos[s] + 1;
    }
    const int64_t batch = c->cfg.copyback_rows;
    e = copy_back(c, st, batch);
  }
  if (e == hipSuccess) e = hipEventRecord(c->done, st);
  return e == hipSuccess ? HC_OK : fail_hip(c);
}

hc_status hc_flush(hc_ctx* c, void* stream, uint64_t* host_count) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t S = c->cfg.n_sessions;
  if (c->cfg.ring_rows) {
    hipError_t e = order_after_last(c, st);
    if (e == hipSuccess) e = copy_back(c, st, 1);
    if (e == hipSuccess) e = hipEventRecord(c->done, st);
    c->enqueued = true;
    if (e != hipSuccess) return fail_hip(c);
  }
  // wait for the copy itself, not for its submission
  if (c->enqueued && host_wait(c) != hipSuccess) return fail_hip(c);
  if (hipStreamSynchronize(st) != hipSuccess) return fail_hip(c);
  if (device_error(c)) return HC_E_DEVICE;
  hc_status r = HC_OK;
  for (uint32_t s = 0; s < S; ++s) {
    const uint64_t n = c->host_count ? reinterpret_cast<volatile uint64_t*>(c->host_count)[s] : 0;
    if (host_count) host_count[s] = c->first[s] >= 0 ? n : 0;
    if (c->first[s] >= 0 && n != (uint64_t)c->end[s]) r = HC_E_CONSISTENCY;
  }
  return r;
}

hc_status hc_attend_workspace_bytes(const hc_ctx* c, uint32_t heads, uint64_t* bytes) {
  if (!c || !bytes || heads == 0 || heads % 64 || heads > 4096) return HC_E_INVAL;
  *bytes = attend_work_bytes(c->dev, (int)heads);
  return HC_OK;
}

namespace {

hc_status attend(hc_ctx* c, void* stream, bool from_slots, const uint16_t* d_q, uint32_t heads,
                 float scale, const uint16_t* d_rows, void* d_work, uint64_t work_bytes,
                 float* d_out) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  if (!d_q || !d_work || !d_out || (!from_slots && !d_rows)) return HC_E_INVAL;
  if (heads == 0 || heads % 64 || heads > 4096) return HC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(d_q) % 16 || (d_rows && reinterpret_cast<uintptr_t>(d_rows) % 16) ||
      reinterpret_cast<uintptr_t>(d_work) % 16 || reinterpret_cast<uintptr_t>(d_out) % 16)
    return HC_E_INVAL;
  if (work_bytes < attend_work_bytes(c->dev, (int)heads)) return HC_E_NOMEM;
  if (c->t == 0) return HC_E_INVAL;   // no step has selected rows yet
  // an append since the last step may have overwritten a ring entry that step
  // selected: the ring no longer holds the step's rows
  if (from_slots && c->cfg.ring_rows && c->appended_since_step) return HC_E_INVAL;
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = order_after_last(c, st);
  if (e == hipSuccess)
    e = launch_attend(c->dev, from_slots, d_q, (int)heads, scale, d_rows, d_work, d_out, st);
  if (e == hipSuccess) e = hipEventRecord(c->done, st);
  c->enqueued = true;
  return e == hipSuccess ? HC_OK : fail_hip(c);
}

}  // namespace

hc_status hc_attend(hc_ctx* c, void* stream, const uint16_t* d_q, uint32_t heads, float scale,
                    const uint16_t* d_rows, void* d_work, uint64_t work_bytes, float* d_out) {
  return attend(c, stream, false, d_q, heads, scale, d_rows, d_work, work_bytes, d_out);
}

hc_status hc_attend_cached(hc_ctx* c, void* stream, const uint16_t* d_q, uint32_t heads,
                           float scale, void* d_work, uint64_t work_bytes, float* d_out) {
  return attend(c, stream, true, d_q, heads, scale, nullptr, d_work, work_bytes, d_out);
}

hc_status hc_attend_cached_noalloc(hc_ctx* c, void* stream, const uint16_t* d_q, uint32_t heads,
                                   float scale, float* d_out) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  if (heads == 0 || heads % 64 || heads > 4096) return HC_E_INVAL;
  if (attend_work_bytes(c->dev, (int)heads) > HC_ATTEND_STATIC_BYTES) return HC_E_NOMEM;
  void* work = scratch_of(c->cfg.device);   // set by hc_create on this device
  if (!work) return HC_E_STATE;
  return attend(c, stream, true, d_q, heads, scale, nullptr, work, HC_ATTEND_STATIC_BYTES, d_out);
}

hc_status hc_export_state(hc_ctx* c, uint32_t session, uint32_t layer, int32_t* slot2pos,
                          int32_t* last_use, int32_t* pos2slot, uint8_t* hot_rows) {
  if (!c || !slot2pos || !last_use) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  if (session >= c->cfg.n_sessions || layer >= c->cfg.n_layers) return HC_E_INVAL;
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  if (c->enqueued && host_wait(c) != hipSuccess) return fail_hip(c);
  if (device_error(c)) return HC_E_DEVICE;
  const DevState& d = c->dev;
  const size_t u = (size_t)session * d.G + layer / d.R;
  const size_t sl = (size_t)session * d.L + layer;
  const size_t C = (size_t)d.C;
  bool ok = hipMemcpy(slot2pos, d.slot2pos + u * C, C * 4, hipMemcpyDeviceToHost) == hipSuccess &&
            hipMemcpy(last_use, d.last_use + u * C, C * 4, hipMemcpyDeviceToHost) == hipSuccess;
  if (ok && pos2slot)
    ok = hipMemcpy(pos2slot, d.pos2slot + u * (size_t)d.hcap, (size_t)d.hcap * 4,
                   hipMemcpyDeviceToHost) == hipSuccess;
  if (ok && hot_rows)
    ok = hipMemcpy2D(hot_rows, kRow, d.hot + sl * C * kSlotStride, kSlotStride, kRow, C,
                     hipMemcpyDeviceToHost) == hipSuccess;
  return ok ? HC_OK : fail_hip(c);
}

hc_status hc_profile_enable(hc_ctx* c, uint32_t max_steps) {
  if (!c) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  if (c->enqueued && host_wait(c) != hipSuccess) return fail_hip(c);
  free_prof(c);
  if (max_steps == 0) return HC_OK;
  c->prof.assign((size_t)max_steps * HC_NUM_STAGES * 2, nullptr);
  for (hipEvent_t& e : c->prof) {
    if (hipEventCreate(&e) != hipSuccess) {
      free_prof(c);
      return HC_E_NOMEM;
    }
  }
  c->prof_cap = max_steps;
  return HC_OK;
}

hc_status hc_profile_read(hc_ctx* c, double* stage_ms, double* per_step, uint64_t per_step_cap,
                          uint64_t* n_steps) {
  if (!c || !stage_ms || !n_steps) return HC_E_INVAL;
  if (c->poisoned) return HC_E_STATE;
  DeviceGuard dg(c->cfg.device);
  if (!dg.ok) return HC_E_INVAL;
  for (int i = 0; i < HC_NUM_STAGES; ++i) stage_ms[i] = 0.0;
  for (uint32_t k = 0; k < c->prof_used; ++k) {
    hipEvent_t* ev = &c->prof[(size_t)k * HC_NUM_STAGES * 2];
    if (hipEventSynchronize(ev[HC_NUM_STAGES * 2 - 1]) != hipSuccess) return fail_hip(c);
    for (int i = 0; i < HC_NUM_STAGES; ++i) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) return fail_hip(c);
      stage_ms[i] += ms;
      if (per_step && k < per_step_cap) per_step[(size_t)k * HC_NUM_STAGES + i] = ms;
    }
  }
  *n_steps = c->prof_used;
  return HC_OK;
}

hc_status hc_steps_done(const hc_ctx* c, uint64_t* n) {
  if (!c || !n) return HC_E_INVAL;
  *n = c->t;
  return HC_OK;
}

hc_status hc_destroy(hc_ctx* c) {
  if (!c) return HC_OK;
  hc_status st = HC_OK;
  {
    DeviceGuard dg(c->cfg.device);
    if (c->enqueued && c->done && host_wait(c) != hipSuccess) st = HC_E_HIP;
    free_prof(c);
    destroy_sync(c);
    free_host(c);
  }
  delete c;
  return st;
}

#ifdef HC_TEST_HOOKS
hc_status hc_test_hook(hc_ctx* c, int kind, int64_t arg, uint64_t* out) {
  switch (kind) {
    case HC_TEST_FAIL_LAUNCH:
      if (!c) return HC_E_INVAL;
      c->test_fail_launch = true;
      return HC_OK;
    case HC_TEST_FORCE_SELECT:
      if (!c) return HC_E_INVAL;
      c->dev.test_force = 1;
      return HC_OK;
    case HC_TEST_CORRUPT_LRU: {
      if (!c) return HC_E_INVAL;
      DeviceGuard dg(c->cfg.device);
      if (c->enqueued && host_wait(c) != hipSuccess) return fail_hip(c);
      // every slot claimed used, an empty queue: the next step that misses
      // finds no victim
      const size_t U = (size_t)c->dev.S * c->dev.G;
      for (size_t u = 0; u < U; ++u) {
        int32_t* line = c->dev.cnt + u * c->dev.Q * kCntStride;
        const int32_t zero = 0, full = c->dev.C;
        if (hipMemcpy(line + kCntQHead, &zero, 4, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(line + kCntQTail, &zero, 4, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(line + kCntFill, &full, 4, hipMemcpyHostToDevice) != hipSuccess)
          return fail_hip(c);
      }
      return HC_OK;
    }
    case HC_TEST_POISON_VICTIMS:
      if (!c) return HC_E_INVAL;
      c->test_poison = arg != 0;
      return HC_OK;
    case HC_TEST_FAIL_PINNED:
      g_fail_pinned = arg;
      return HC_OK;
    case HC_TEST_PINNED_BYTES:
      if (!out) return HC_E_INVAL;
      *out = g_pinned_bytes.load();
      return HC_OK;
  }
  return HC_E_INVAL;
}
#endif

const char* hc_status_str(hc_status s) {
  switch (s) {
    case HC_OK: return "ok";
    case HC_E_INVAL: return "invalid argument";
    case HC_E_NOMEM: return "out of memory or workspace too small";
    case HC_E_HIP: return "HIP error (context poisoned)";
    case HC_E_STATE: return "context poisoned by an earlier HIP error";
    case HC_E_CONSISTENCY: return "host row count differs from the logical row count";
    case HC_E_DEVICE: return "a kernel found the context's device state inconsistent (context poisoned)";
  }
  return "unknown status";
}

}  // extern "C"
