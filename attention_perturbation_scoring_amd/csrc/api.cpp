// libdropkv host side: argument checks, scratch ownership, launch sequencing,
// the device error latch and optional per-kernel event timing.  The C ABI is
// declared (and documented) in include/dropkv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dropkv.h"
#include "common.h"

using namespace dropkv;

// Scratch of dropkv_score_noalloc, for callers that cannot allocate: one copy
// per device, resident while the library is loaded.  Host code never uses the
// array's name as an address: its device address is read once per device with
// hipGetSymbolAddress (at dropkv_create) and used from then on.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
};

struct dropkv_ctx {
  int device = 0;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  // selection scratch (see carve_select): [0] per-head selection, [1] the
  // layer-wide one, kept apart so that alternating calls do not re-zero them
  struct SelBuf {
    void* p = nullptr;
    size_t bytes = 0;
    int hkv = 0;                   // head count the zeroed prefix was laid out for
    uint32_t epoch = 0;            // single-launch selections since the prefix was zeroed
  } sel[2];
  int64_t sel_wait = kSelectWait;  // team-barrier polls before a selection workgroup goes alone
  void* noalloc_scratch = nullptr; // device address of this device's `scratch` array
  int score_hv = 0, score_splits = 0, score_dp = 0, score_xh = 0;   // layout of `scratch` (counters zeroed for it)
  uint32_t* latch = nullptr;       // device word
  uint32_t* latch_host = nullptr;  // pinned read-back
  bool prof = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> free_events;
  hipEvent_t pending_start = nullptr;
};

namespace {

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipEvent_t get_event(dropkv_ctx* c) {
  if (!c->free_events.empty()) {
    hipEvent_t e = c->free_events.back();
    c->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Device address of the no-allocation scratch array on `device` (the current
// device), looked up once per device.
void* noalloc_scratch_ptr(int device) {
  static std::mutex mu;
  static void* ptr[64];
  static bool known[64];
  if (device < 0 || device >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!known[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[device] = p;
    known[device] = true;
  }
  return ptr[device];
}

// The layout (virtual heads, splits, padded width, helpers) that the
// no-allocation scratch's counters on `device` were last zeroed for.  The
// merge's arrival counters and head flags move with the layout (onto bytes
// another layout used for partial sums), and every call leaves them zeroed, so
// they are zeroed again only when the layout changes or a call failed part-way.
struct NoAllocLayout {
  int hv = -1, splits = 0, dp = 0, xh = 0;
};
std::mutex noalloc_mu;
NoAllocLayout noalloc_layout[64];
bool noalloc_needs_zero(int device, int hv, int splits, int dp, int xh) {
  if (device < 0 || device >= 64) return true;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  NoAllocLayout& l = noalloc_layout[device];
  if (l.hv == hv && l.splits == splits && l.dp == dp && l.xh == xh) return false;
  l.hv = hv; l.splits = splits; l.dp = dp; l.xh = xh;
  return true;
}
void noalloc_forget(int device) {
  if (device < 0 || device >= 64) return;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  noalloc_layout[device].hv = -1;
}

int to_status(hipError_t e) {
  if (e == hipSuccess) return DROPKV_OK;
  if (e == hipErrorOutOfMemory) return DROPKV_ENOMEM;
  return DROPKV_EDEVICE;
}

}  // namespace

namespace dropkv {
void prof_begin(void* ctx, const char* name, hipStream_t s) {
  (void)name;
  auto* c = static_cast<dropkv_ctx*>(ctx);
  if (!c || !c->prof) return;
  c->pending_start = get_event(c);
  if (c->pending_start) (void)hipEventRecord(c->pending_start, s);
}
void prof_end(void* ctx, const char* name, hipStream_t s) {
  auto* c = static_cast<dropkv_ctx*>(ctx);
  if (!c || !c->prof || !c->pending_start) return;
  hipEvent_t stop = get_event(c);
  if (!stop) return;
  (void)hipEventRecord(stop, s);
  c->recs.push_back(ProfRec{name, c->pending_start, stop});
  c->pending_start = nullptr;
}
}  // namespace dropkv

extern "C" {

int dropkv_create(dropkv_ctx** out, int device) {
  if (!out) return DROPKV_EINVAL;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) return DROPKV_EINVAL;
  DeviceGuard guard(device);
  if (!guard.ok) return DROPKV_EDEVICE;
  auto* c = new dropkv_ctx();
  c->device = device;
  hipError_t e = hipMalloc(&c->latch, 256);
  if (e == hipSuccess) e = hipMemset(c->latch, 0, 256);
  // complete before any call, whatever stream it uses
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipHostMalloc(&c->latch_host, 2 * sizeof(uint32_t));
  if (e == hipSuccess) {
    c->noalloc_scratch = noalloc_scratch_ptr(device);
    if (!c->noalloc_scratch) e = hipErrorInvalidSymbol;
  }
  if (e != hipSuccess) {
    if (c->latch) (void)hipFree(c->latch);
    if (c->latch_host) (void)hipHostFree(c->latch_host);
    delete c;
    return to_status(e);
  }
  *out = c;
  return DROPKV_OK;
}

int dropkv_destroy(dropkv_ctx* c) {
  if (!c) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  (void)hipDeviceSynchronize();
  for (auto& r : c->recs) { (void)hipEventDestroy(r.start); (void)hipEventDestroy(r.stop); }
  for (auto e : c->free_events) (void)hipEventDestroy(e);
  if (c->scratch) (void)hipFree(c->scratch);
  for (auto& b : c->sel)
    if (b.p) (void)hipFree(b.p);
  if (c->latch) (void)hipFree(c->latch);
  if (c->latch_host) (void)hipHostFree(c->latch_host);
  delete c;
  return DROPKV_OK;
}

int dropkv_scratch_bytes(int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                         int64_t* score_bytes, int64_t* select_bytes) {
  if (!score_bytes || !select_bytes) return DROPKV_EINVAL;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n < 1 || n >= (int64_t(1) << 31) || w < 1 || w > n ||
      d < 8 || d % 8 != 0 || d > 256)
    return DROPKV_EINVAL;
  const int M = (Hq / Hkv) * w;
  if ((int64_t)M > (int64_t)kRows * kMaxRowGroups) return DROPKV_EINVAL;
  const int DP = (d + 31) / 32 * 32, R = (M + kRows - 1) / kRows;
  int64_t len = 0;
  const int splits = plan_splits(n, Hkv * R, &len, kTargetWG1);
  const int xh = plan_helpers(n, Hkv * R, splits);
  *score_bytes = (int64_t)score_scratch_bytes(Hkv * R, splits, DP, xh);
  *select_bytes = (int64_t)select_scratch_bytes(Hkv, n);
  return DROPKV_OK;
}

int dropkv_plan_splits(int64_t n, int32_t Hkv, int32_t* splits) {
  if (!splits || n < 1 || Hkv < 1) return DROPKV_EINVAL;
  int64_t len = 0;
  *splits = plan_splits(n, Hkv, &len);
  return DROPKV_OK;
}

namespace {

// Shared by the scoring entry points: checks, launch geometry, scratch (the
// context's, grown on demand, or -- noalloc -- the static per-device array, with
// no allocation and no profiling events).
int score_common(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                 const uint16_t* v_cache, bool attention_only, int64_t n, int32_t w, int32_t Hq,
                 int32_t Hkv, int32_t d, int32_t pool, float* scores, float* out_a,
                 float* out_lse, void* stream, bool noalloc = false, int64_t cap = 0,
                 uint32_t* hist1 = nullptr) {
  if (!c) return DROPKV_EINVAL;
  if (!aligned16(q_win) || !aligned16(k_cache) || !aligned16(scores)) return DROPKV_EINVAL;
  if ((out_a && !aligned16(out_a)) || (out_lse && !aligned16(out_lse))) return DROPKV_EINVAL;
  if (!attention_only && !aligned16(v_cache)) return DROPKV_EINVAL;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return DROPKV_EINVAL;
  if (n < 1 || n >= (int64_t(1) << 31)) return DROPKV_EINVAL;
  if (w < 1 || w > n) return DROPKV_EINVAL;
  if (pool < 1 || pool % 2 == 0 || pool > 129) return DROPKV_EINVAL;
  if (d < 8 || d % 8 != 0 || d > 256) return DROPKV_EINVAL;
  const int G = Hq / Hkv;
  if ((int64_t)G * w > (int64_t)kRows * kMaxRowGroups) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  ScoreArgs a{};
  a.q = q_win; a.k = k_cache; a.v = v_cache; a.scores = scores;
  a.n = n; a.w = w; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.G = G; a.M = G * w; a.pool = pool;
  a.hs = (cap > 0 ? cap : n) * (int64_t)d;   // a resident cache keeps cap rows per head
  a.DP = (d + 31) / 32 * 32;
  a.R = (a.M + kRows - 1) / kRows;
  if (!attention_only && !score_fits(a.DP, a.R)) return DROPKV_EINVAL;
  // the first pass runs per (KV head, row group): plan its splits over all of them
  a.splits = plan_splits(n, Hkv * a.R, &a.split_len, attention_only ? kTargetWGAttn : kTargetWG1);
  a.chunks2 = plan_chunks2(n, Hkv, &a.chunk2_len, attention_only ? kTargetWGAttnB : kTargetWG2);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  a.latch = c->latch;
  a.out_a = out_a;
  a.out_lse = out_lse;
  a.xh = plan_helpers(n, Hkv * a.R, a.splits);
  if (hist1 && !attention_only) {   // score + select: the selection's first digit, built in pass 2
    a.hist1 = hist1;
    a.hist1_stride = fused_bins();
  }
  const size_t need = score_scratch_bytes(Hkv * a.R, a.splits, a.DP, a.xh);
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return DROPKV_ESCRATCH;
    if (!c->noalloc_scratch) return DROPKV_EDEVICE;
    carve_scratch(c->noalloc_scratch, Hkv * a.R, a.splits, a.DP, a.xh, &a.part, &a.rs, &a.ex);
    if (!attention_only && noalloc_needs_zero(c->device, Hkv * a.R, a.splits, a.DP, a.xh)) {
      // (a zero-fill kernel, not a memset: callers may capture the call in a graph)
      const hipError_t e = launch_zero(a.ex.cnt, (size_t)(a.ex.head + Hkv * a.R) - (size_t)a.ex.cnt, s);
      if (e != hipSuccess) { noalloc_forget(c->device); return to_status(e); }
    }
    const int rc = to_status(launch_score(nullptr, a, s));
    if (rc != DROPKV_OK) noalloc_forget(c->device);
    return rc;
  }
  // a layout change moves the merge's arrival counters: zero them (in stream
  // order) whenever the scratch or its layout changes; every call leaves them zeroed
  const bool relayout = need > c->scratch_bytes || Hkv * a.R != c->score_hv ||
                        a.splits != c->score_splits || a.DP != c->score_dp || a.xh != c->score_xh;
  if (need > c->scratch_bytes) {
    if (c->scratch) {
      (void)hipStreamSynchronize(s);
      (void)hipDeviceSynchronize();
      (void)hipFree(c->scratch);
      c->scratch = nullptr;
      c->scratch_bytes = 0;
    }
    hipError_t e = hipMalloc(&c->scratch, need);
    if (e != hipSuccess) { c->scratch = nullptr; return DROPKV_ENOMEM; }
    c->scratch_bytes = need;
    c->score_hv = -1;   // fresh memory: the next scoring call zeroes its counters
  }
  carve_scratch(c->scratch, Hkv * a.R, a.splits, a.DP, a.xh, &a.part, &a.rs, &a.ex);
  if (!attention_only && relayout) {
    // the merge's arrival counters and head flags (adjacent in the carve)
    const hipError_t e = launch_zero(a.ex.cnt, (size_t)(a.ex.head + Hkv * a.R) - (size_t)a.ex.cnt, s);
    if (e != hipSuccess) return to_status(e);
    c->score_hv = Hkv * a.R; c->score_splits = a.splits; c->score_dp = a.DP; c->score_xh = a.xh;
  }
  const int rc = to_status(attention_only ? launch_score_attention(c, a, s) : launch_score(c, a, s));
  // a call that failed part-way may leave counters set: zero them next time
  if (rc != DROPKV_OK && !attention_only) c->score_hv = -1;
  return rc;
}

}  // namespace

int dropkv_score(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                 const uint16_t* v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                 int32_t pool, float* scores, void* stream) {
  return score_common(c, q_win, k_cache, v_cache, false, n, w, Hq, Hkv, d, pool, scores, nullptr,
                      nullptr, stream);
}

int dropkv_score_ex(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                    const uint16_t* v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                    int32_t d, int32_t pool, float* scores, float* out_a, float* out_lse,
                    void* stream) {
  return score_common(c, q_win, k_cache, v_cache, false, n, w, Hq, Hkv, d, pool, scores, out_a,
                      out_lse, stream);
}

int dropkv_score_noalloc(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                         int32_t d, int32_t pool, float* scores, void* stream) {
  return score_common(c, q_win, k_cache, v_cache, false, n, w, Hq, Hkv, d, pool, scores, nullptr,
                      nullptr, stream, true);
}

int64_t dropkv_noalloc_scratch_bytes(void) { return (int64_t)kNoAllocScratchBytes; }

int dropkv_score_attention(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                           int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool,
                           float* scores, void* stream) {
  return score_common(c, q_win, k_cache, nullptr, true, n, w, Hq, Hkv, d, pool, scores, nullptr,
                      nullptr, stream);
}

namespace {

// Selection scratch for Hkv heads of n tokens in buffer `b`: (re)allocated on
// growth; its zeroed prefix is (re)laid out when the head count changes (and
// the single-launch call count restarts), and every selection leaves what the
// next one reads zeroed: the multi-launch path its own words, the single-launch
// path the set of the next call's parity.
int sel_prepare(dropkv_ctx* c, dropkv_ctx::SelBuf& b, int Hkv, int64_t n, hipStream_t s,
                SelScratch* sc) {
  const size_t need = select_scratch_bytes(Hkv, n);
  if (need > b.bytes || Hkv != b.hkv) {
    if (b.p) {
      (void)hipStreamSynchronize(s);
      (void)hipDeviceSynchronize();
      if (need > b.bytes) {
        (void)hipFree(b.p);
        b.p = nullptr;
        b.bytes = 0;
      }
    }
    if (!b.p) {
      hipError_t e = hipMalloc(&b.p, need);
      if (e != hipSuccess) { b.p = nullptr; return DROPKV_ENOMEM; }
      b.bytes = need;
    }
    // stream-ordered (a null-stream memset would not order with a
    // non-blocking stream's kernels)
    hipError_t e = launch_zero(b.p, select_zero_prefix_bytes(Hkv), s);
    if (e != hipSuccess) return to_status(e);
    b.hkv = Hkv;
    b.epoch = 0;
  }
  carve_select(b.p, Hkv, n, sc);
  sc->par = (int)(b.epoch & 1u);
  return DROPKV_OK;
}

}  // namespace

int dropkv_select(dropkv_ctx* c, const float* scores, int32_t Hkv, int64_t n, int64_t budget,
                  int32_t* keep, void* stream) {
  if (!c || !aligned16(scores)) return DROPKV_EINVAL;
  if (Hkv < 1 || n < 1 || n >= (int64_t(1) << 31) || budget < 0 || budget > n) return DROPKV_EINVAL;
  if (budget == 0) return DROPKV_OK;  // nothing to write
  if (!aligned16(keep)) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SelScratch sc{};
  const int rc = sel_prepare(c, c->sel[0], Hkv, n, s, &sc);
  if (rc != DROPKV_OK) return rc;
  return to_status(
      launch_select(c, scores, Hkv, n, budget, keep, c->latch, sc, c->sel_wait, s, &c->sel[0].epoch));
}

namespace {

// Scoring (K/V head stride cap * d when cap > 0, else n * d) and selection in
// one call: the second pass also counts the selection's first radix digit when
// the selection runs as one launch.
int score_select_impl(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                      const uint16_t* v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                      int32_t d, int32_t pool, int64_t budget, float* scores, int32_t* keep,
                      void* stream, int64_t cap) {
  if (!c) return DROPKV_EINVAL;
  if (Hkv < 1 || n < 1 || budget < 0 || budget > n) return DROPKV_EINVAL;
  if (budget > 0 && !aligned16(keep)) return DROPKV_EINVAL;
  const int G = (Hkv > 0 && Hq % Hkv == 0) ? Hq / Hkv : 1;
  const int DP = (d + 31) / 32 * 32, R = (G * w + kRows - 1) / kRows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hist1 = nullptr;
  SelScratch sc{};
  const bool pre1 = d >= 8 && d <= 256 && w >= 1 && select_prebuilt_applies(Hkv, n, budget) &&
                    score_hist_fits(DP, R);
  if (pre1) {
    DeviceGuard guard(c->device);
    if (!guard.ok) return DROPKV_EDEVICE;
    // the selection scratch first: its histogram must be zeroed before pass 2 adds
    const int rc = sel_prepare(c, c->sel[0], Hkv, n, s, &sc);
    if (rc != DROPKV_OK) return rc;
    hist1 = sc.fh + (size_t)sc.par * Hkv * fused_bins();   // this call's parity
  }
  int rc = score_common(c, q_win, k_cache, v_cache, false, n, w, Hq, Hkv, d, pool, scores, nullptr,
                        nullptr, stream, false, cap, hist1);
  if (rc != DROPKV_OK) {
    if (pre1) {   // pass 2 may have added part of a histogram: the scratch is stale
      c->sel[0].hkv = -1;
    }
    return rc;
  }
  if (budget == 0) return DROPKV_OK;
  if (!pre1) return dropkv_select(c, scores, Hkv, n, budget, keep, stream);
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  return to_status(launch_select(c, scores, Hkv, n, budget, keep, c->latch, sc, c->sel_wait, s,
                                 &c->sel[0].epoch, true));
}

}  // namespace

int dropkv_score_select(dropkv_ctx* c, const uint16_t* q_win, const uint16_t* k_cache,
                        const uint16_t* v_cache, int64_t n, int32_t w, int32_t Hq, int32_t Hkv,
                        int32_t d, int32_t pool, int64_t budget, float* scores, int32_t* keep,
                        void* stream) {
  return score_select_impl(c, q_win, k_cache, v_cache, n, w, Hq, Hkv, d, pool, budget, scores,
                           keep, stream, 0);
}

int dropkv_select_layer(dropkv_ctx* c, const float* scores, int32_t Hkv, int64_t n,
                        int64_t budget, int32_t* keep, int32_t* counts, void* stream) {
  if (!c || !aligned16(scores) || !aligned16(counts)) return DROPKV_EINVAL;
  if (Hkv < 1 || n < 1) return DROPKV_EINVAL;
  const int64_t total = (int64_t)Hkv * n;
  if (total >= (int64_t(1) << 31) || budget < 0 || budget > total) return DROPKV_EINVAL;
  if (budget > 0 && !aligned16(keep)) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (budget > 0) {
    // the [Hkv][n] scores are one sequence in (head, index) order
    SelScratch sc{};
    const int rc = sel_prepare(c, c->sel[1], 1, total, s, &sc);
    if (rc != DROPKV_OK) return rc;
    const hipError_t e = launch_select(c, scores, 1, total, budget, keep, c->latch, sc, c->sel_wait, s,
                                       &c->sel[1].epoch);
    if (e != hipSuccess) return to_status(e);
  }
  return to_status(launch_layer_counts(c, keep, budget, n, Hkv, counts, c->latch, s));
}

int dropkv_compact(dropkv_ctx* c, const uint16_t* k, const uint16_t* v, int32_t Hkv, int64_t n,
                   int32_t d, const int32_t* keep, int64_t budget, uint16_t* k_out,
                   uint16_t* v_out, void* stream) {
  if (!c) return DROPKV_EINVAL;
  if (Hkv < 1 || n < 1 || n >= (int64_t(1) << 31) || d < 8 || d % 8 != 0 || d > 256)
    return DROPKV_EINVAL;
  if (budget < 0 || budget > n) return DROPKV_EINVAL;
  if (budget == 0) return DROPKV_OK;  // nothing to write
  if (!aligned16(k) || !aligned16(v) || !aligned16(keep) || !aligned16(k_out) || !aligned16(v_out))
    return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  return to_status(launch_compact(c, k, v, Hkv, n, d, keep, budget, k_out, v_out, c->latch,
                                  static_cast<hipStream_t>(stream)));
}

int dropkv_compact_inplace(dropkv_ctx* c, uint16_t* k_cache, uint16_t* v_cache, int32_t Hkv,
                           int64_t cap, int64_t n_valid, int32_t d, const int32_t* keep,
                           int64_t budget, void* stream) {
  if (!c) return DROPKV_EINVAL;
  if (Hkv < 1 || cap < 1 || cap >= (int64_t(1) << 31) || n_valid < 1 || n_valid > cap || d < 8 ||
      d % 8 != 0 || d > 256)
    return DROPKV_EINVAL;
  if (budget < 0 || budget > n_valid) return DROPKV_EINVAL;
  if (budget == 0) return DROPKV_OK;  // nothing moves
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(keep)) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  return to_status(launch_compact_inplace(c, k_cache, v_cache, Hkv, cap * (int64_t)d, d, n_valid, keep,
                                          budget, c->latch, static_cast<hipStream_t>(stream)));
}

int dropkv_rescore(dropkv_ctx* c, const uint16_t* q_win, uint16_t* k_cache, uint16_t* v_cache,
                   int64_t cap, int64_t n_valid, int32_t w, int32_t Hq, int32_t Hkv, int32_t d,
                   int32_t pool, int64_t budget, float* scores, int32_t* keep, void* stream) {
  if (!c) return DROPKV_EINVAL;
  if (cap < 1 || cap >= (int64_t(1) << 31) || n_valid < 1 || n_valid > cap) return DROPKV_EINVAL;
  if (budget < 0 || budget > n_valid) return DROPKV_EINVAL;
  if (budget > 0 && !aligned16(keep)) return DROPKV_EINVAL;
  int rc = score_select_impl(c, q_win, k_cache, v_cache, n_valid, w, Hq, Hkv, d, pool, budget,
                             scores, keep, stream, cap);
  if (rc != DROPKV_OK || budget == 0) return rc;
  return dropkv_compact_inplace(c, k_cache, v_cache, Hkv, cap, n_valid, d, keep, budget, stream);
}

int dropkv_stream_read(dropkv_ctx* c, const void* p, int64_t bytes, void* stream) {
  if (!c || bytes <= 0 || bytes % 16 != 0 || !aligned16(p)) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  // the sink is the spare tail of the latch block (words 32..39 of 64)
  return to_status(launch_stream_read(c, p, bytes, c->latch + 32, static_cast<hipStream_t>(stream)));
}

int dropkv_sync(dropkv_ctx* c, void* stream) {
  if (!c) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  if (!guard.ok) return DROPKV_EDEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // word 0: scoring, selection and packing; word 1: the in-place compaction's checks
  hipError_t e = hipMemcpyAsync(c->latch_host, c->latch, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return to_status(e);
  const uint32_t bits = c->latch_host[0] | c->latch_host[1];
  if (bits) {
    e = hipMemsetAsync(c->latch, 0, 2 * sizeof(uint32_t), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return to_status(e);
  }
  if (bits & LATCH_NONFINITE) return DROPKV_ENONFINITE;
  if (bits & LATCH_INPUT_RANGE) return DROPKV_ERANGE;
  if (bits & LATCH_SINGULAR) return DROPKV_ESINGULAR;
  if (bits & (LATCH_RANGE | LATCH_OVERFLOW)) return DROPKV_ERANGE;
  return DROPKV_OK;
}

const char* dropkv_strerror(int code) {
  switch (code) {
    case DROPKV_OK: return "ok";
    case DROPKV_EINVAL: return "invalid argument";
    case DROPKV_ESINGULAR: return "a window query puts probability that rounds to 1 on one key";
    case DROPKV_ENONFINITE: return "non-finite input";
    case DROPKV_ERANGE: return "value out of range";
    case DROPKV_EDEVICE: return "HIP runtime error";
    case DROPKV_ENOMEM: return "out of device memory";
    case DROPKV_ESCRATCH: return "needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int dropkv_set_select_wait(dropkv_ctx* c, int64_t polls) {
  if (!c) return DROPKV_EINVAL;
  c->sel_wait = polls < 0 ? -1 : polls;
  return DROPKV_OK;
}

int dropkv_profile_enable(dropkv_ctx* c, int on) {
  if (!c) return DROPKV_EINVAL;
  c->prof = on != 0;
  return DROPKV_OK;
}

int dropkv_profile_reset(dropkv_ctx* c) {
  if (!c) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  for (auto& r : c->recs) {
    (void)hipEventSynchronize(r.stop);
    c->free_events.push_back(r.start);
    c->free_events.push_back(r.stop);
  }
  c->recs.clear();
  return DROPKV_OK;
}

int dropkv_profile_read(dropkv_ctx* c, const char* name, double* total_ms, int64_t* launches) {
  if (!c || !name || !total_ms || !launches) return DROPKV_EINVAL;
  DeviceGuard guard(c->device);
  double tot = 0.0;
  int64_t cnt = 0;
  for (auto& r : c->recs) {
    if (r.name != name) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return to_status(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return to_status(e);
    tot += ms;
    ++cnt;
  }
  *total_ms = tot;
  *launches = cnt;
  return DROPKV_OK;
}

}  // extern "C"
