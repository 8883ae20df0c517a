// C ABI of libgdn: argument validation, the split planner, workspace carving and
// the launch sequence.  Declarations and the full contract are in include/gdn.h.
//
// Planner (FlashQLA talk transcript, tokendh.com, auto-CP section): the number of
// splits per sequence is not fixed by the hardware the way inter-card parallelism
// is; with L chunks per segment and N chunks per sequence the one-wave model is
// T = lambda1 L + lambda2 N / L (the chunk-serial passes scale with L, the
// recurrence over segments with N / L).  On a GPU with 256 CUs and one fused
// workgroup per CU the first term is really the makespan of the fused pass: its
// units (sequence, segment, head, column block) run in dispatch order on the
// earliest free CU of their XCD, and with packed sequences of different lengths the
// tail of that schedule, not the average, decides.  So the planner simulates that
// schedule for a ladder of candidate lengths (pass3_makespan) and takes
// argmin lambda1 * makespan(L) + lambda2 * (N_longest / L - 1), with "no split"
// competing as one more candidate.  lambda1, lambda2 and the model's start-up and
// lookback costs are MI355X measurements; the choice is a performance decision only
// (every plan computes the same result within rounding).
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <queue>
#include <vector>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

using gdn::kChunk;
using gdn::kWindowMaxCap;

constexpr size_t kAlign = 256;
// Per-kernel cost model of one call, in microseconds, fitted on MI355X to the five
// workloads and to forced segment lengths on them (bench stage times):
//   forward   kFwdFixedUs + step(busy) * makespan, the makespan in chunk steps from the
//             simulated schedule (pass3_makespan: a unit's chunks, its start-up
//             kStartSteps, kLookbackSteps for a segment after the first).  One-pass
//             step(busy) = kStepBaseUs + kStepPerBusyUs * busy workgroups (HBM and L2
//             contention: 2.7 us at 64 busy, 3.7 us at 256); two-kernel path: λ1.
//   K1        two-kernel path only: kK1FixedUs + kK1PerChunkHeadUs per chunk-head.
//   split     kSplitFixedUs (one-pass: kSplitFixedWyUs) + kSplitPerChunkHeadUs per
//             chunk-head: the gate sums, the gate scan and the launches of the
//             correction stages (on a window-only problem they read the gate scan's
//             count and return at once); packed input adds the table launch,
//             kPackedTablesUs.
//   corrected heads (a segment start without a window), per call: pass 1
//             (kPass1FixedUs + kPass1StepUs * L per round of workgroups; one-pass
//             plans form T inside pass 1, two-kernel plans read K1's) and the merge
//             (short chain: kMergeFixedUs + λ2 per step; tree: kTreeFixedUs +
//             kTreeSqrtUs * sqrt(steps)), which take the place of kCorrReplacesUs of
//             the empty correction launches.
// λ1 and λ2 are the per-call overrides gdn_opts.lambda1_us / lambda2_us.
constexpr float kLambda1Us = 3.8f;
constexpr float kLambda2Us = 0.75f;
constexpr double kStartSteps = 2.2;
constexpr double kLookbackSteps = 1.0;
constexpr double kFwdFixedUs = 4.5;
constexpr double kStepBaseUs = 2.33, kStepPerBusyUs = 0.0055;
constexpr double kStepF32Us = 5.5;               // two-kernel step on fp32 inputs
constexpr double kK1FixedUs = 10.0, kK1PerChunkHeadUs = 0.004;
constexpr double kSplitFixedUs = 17.5, kSplitFixedWyUs = 12.5, kSplitPerChunkHeadUs = 0.0, kPackedTablesUs = 4.0;
constexpr double kCorrReplacesUs = 8.0;
constexpr double kPass1FixedUs = 3.0, kPass1StepUs = 2.0;
constexpr double kMergeFixedUs = 7.0, kTreeFixedUs = 35.4, kTreeSqrtUs = 3.18;
constexpr int kMinSegmentChunks = 8;
constexpr int64_t kPlanModelMaxUnits = 1 << 16;   // larger plans use the closed form
constexpr float kWindowMargin = 1e-3f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

// Scratch of the allocation-free entry point (gdn_chunk_fwd_noalloc): a file-scope
// device array, one copy per GPU the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host that name is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress returns,
// taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of this device's `scratch` (nullptr if the query fails).  The first
// call on a device makes the query; later calls return the cached address.
void* scratch_address() {
  static std::atomic<void*> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  cache[dev].store(q, std::memory_order_release);   // same value from any racing thread
  return q;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, queried once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The caller's timing events of a stage, handed to its launcher, which records them
// from the dispatch of the stage's first (start) and last (stop) kernel; null entries
// are skipped.
gdn::KernelEvents stage_events(const gdn_opts* o, int stage) {
  gdn::KernelEvents e;
  if (o && o->stage_events) {
    e.start = o->stage_events[2 * stage];
    e.stop = o->stage_events[2 * stage + 1];
  }
  return e;
}


int validate_shape(const gdn_shape* s) {
  if (!s) return GDN_ERR_ARG;
  if (s->B < 1 || s->T < 0 || s->H < 1 || s->N < 0) return GDN_ERR_ARG;
  if (s->T > INT_MAX / 2 || s->H > 65535 || s->B * s->H > INT_MAX / 2) return GDN_ERR_ARG;
  if ((s->dk != 64 && s->dk != 128) || (s->dv != 64 && s->dv != 128)) return GDN_ERR_UNSUPPORTED;
  if ((s->qkv_dtype != GDN_BF16 && s->qkv_dtype != GDN_F32) ||
      (s->beta_dtype != GDN_BF16 && s->beta_dtype != GDN_F32))
    return GDN_ERR_UNSUPPORTED;
  if (s->cu_seqlens_host) {
    if (s->B != 1 || s->N < 1 || s->N * s->H > INT_MAX / 2) return GDN_ERR_ARG;
    const int32_t* cu = s->cu_seqlens_host;
    if (cu[0] != 0 || cu[s->N] != s->T) return GDN_ERR_ARG;
    for (int64_t n = 0; n < s->N; ++n)
      if (cu[n + 1] < cu[n]) return GDN_ERR_ARG;
  } else if (s->N != s->B) {
    return GDN_ERR_ARG;
  }
  return GDN_OK;
}

int validate_opts(const gdn_opts* o) {
  if (!o) return GDN_OK;
  if (o->value_block != 0 && o->value_block != 64 && o->value_block != 128) return GDN_ERR_ARG;
  if (o->one_pass < -1 || o->one_pass > 1) return GDN_ERR_ARG;
  if (o->force_segment_chunks < 0 || o->window_max_chunks < 0 ||
      o->window_max_chunks > kWindowMaxCap)
    return GDN_ERR_ARG;
  if (!std::isfinite(o->window_log_eps) || o->window_log_eps > 0.f) return GDN_ERR_ARG;
  if (!(o->lambda1_us >= 0.f) || !(o->lambda2_us >= 0.f)) return GDN_ERR_ARG;
  return GDN_OK;
}

int64_t seq_chunks(const gdn_shape* s, int64_t n) {
  const int64_t len = s->cu_seqlens_host ? s->cu_seqlens_host[n + 1] - s->cu_seqlens_host[n] : s->T;
  return (len + kChunk - 1) / kChunk;
}

struct Plan {
  int64_t total_chunks = 0, max_chunks = 0;
  int seg_chunks = INT_MAX / 2;
  bool split = false;
  int64_t total_segs = 0;
  int value_block = 128;
  int pass1_block = 64;
  // one-pass kernel (fused_wy.hip, bf16): the chunk inverse is formed inside the forward
  // pass; K1 and the T buffer are needed only when a split plan runs pass 1
  bool wy = false;
  int wmax = kWindowMaxCap;
  float log_eps = 0.f;
};

// Pass-3 makespan, in chunk steps, of segment length L: the kernel's units (segment,
// head, column block) in dispatch order, dealt to the 8 XCDs round robin (workgroup
// id mod 8), each XCD placing a unit on its earliest free CU (one workgroup per CU).
// The segment order is the kernel's: packed input (split, at most kSegOrderMaxSeqs
// sequences) takes full segments first and then the last segments longest first;
// otherwise sequence order.  A unit costs its chunks, plus the lookback for segments
// after the first, plus the start-up.  Plans too large to simulate cheaply use the
// closed form max(average work per CU, longest unit).
double pass3_makespan(const gdn_shape* s, int64_t L, int64_t cus, int ncb) {
  const int64_t per_xcd = std::max<int64_t>(1, cus / 8);
  std::vector<double> full, last;
  for (int64_t n = 0; n < s->N; ++n) {
    const int64_t nch = seq_chunks(s, n);
    const int64_t segs = std::max<int64_t>(1, (nch + L - 1) / L);
    for (int64_t j = 0; j < segs; ++j) {
      const double c = (double)std::min(L, std::max<int64_t>(0, nch - j * L)) +
                       (j > 0 ? kLookbackSteps : 0.0) + kStartSteps;
      (j + 1 < segs ? full : last).push_back(c);
    }
  }
  const int64_t per_seg = s->H * ncb;
  const int64_t units = (int64_t)(full.size() + last.size()) * per_seg;
  double work = 0, longest = 0;
  for (double c : full) work += c, longest = std::max(longest, c);
  for (double c : last) work += c, longest = std::max(longest, c);
  work *= (double)per_seg;
  if (units > kPlanModelMaxUnits) return std::max(work / (double)cus, longest);
  std::vector<double> order;
  const bool lpt = s->cu_seqlens_host && s->N <= gdn::kSegOrderMaxSeqs && !full.empty();
  if (lpt) {
    order = full;
    std::stable_sort(last.begin(), last.end(), std::greater<double>());
    order.insert(order.end(), last.begin(), last.end());
  } else {
    // sequence order: rebuild it (full and last were separated above)
    for (int64_t n = 0; n < s->N; ++n) {
      const int64_t nch = seq_chunks(s, n);
      const int64_t segs = std::max<int64_t>(1, (nch + L - 1) / L);
      for (int64_t j = 0; j < segs; ++j)
        order.push_back((double)std::min(L, std::max<int64_t>(0, nch - j * L)) +
                        (j > 0 ? kLookbackSteps : 0.0) + kStartSteps);
    }
  }
  std::vector<std::priority_queue<double, std::vector<double>, std::greater<double>>> xcd(8);
  for (auto& q : xcd)
    for (int64_t i = 0; i < per_xcd; ++i) q.push(0.0);
  int64_t u = 0;
  for (double c : order) {
    for (int64_t k = 0; k < per_seg; ++k, ++u) {
      auto& q = xcd[u % 8];
      const double t = q.top();
      q.pop();
      q.push(t + c);
    }
  }
  double m = 0;   // latest finishing CU: the last element left in each min-heap
  for (auto& q : xcd) {
    while (q.size() > 1) q.pop();
    m = std::max(m, q.top());
  }
  return m;
}

// The modelled time of one call (see the constants above) with segment length L
// (L >= the longest sequence's chunks: no split) and a fraction `corr` of the
// (sequence, head) pairs that take the correction (a segment start without a window).
double call_us(const gdn_shape* s, const Plan& P, const gdn_opts* o, int64_t L, int64_t cus,
               double corr) {
  const bool split = L < P.max_chunks;
  const int ncb = (int)(s->dv / P.value_block);
  int64_t segs = 0, longest_steps = 0;
  for (int64_t n = 0; n < s->N; ++n) {
    const int64_t nch = seq_chunks(s, n);
    const int64_t sg = split ? std::max<int64_t>(1, (nch + L - 1) / L) : 1;
    segs += sg;
    longest_steps = std::max(longest_steps, sg - 1);
  }
  const double units = (double)segs * s->H * ncb;
  const double busy = std::min<double>(units, (double)cus);
  const double l1 = (o && o->lambda1_us > 0.f) ? o->lambda1_us : -1.0;
  const double l2 = (o && o->lambda2_us > 0.f) ? o->lambda2_us : kLambda2Us;
  double step = P.wy ? kStepBaseUs + kStepPerBusyUs * busy
                     : (s->qkv_dtype == GDN_BF16 ? kLambda1Us : kStepF32Us);
  if (l1 > 0) step = l1;
  double t = kFwdFixedUs + step * pass3_makespan(s, split ? L : INT_MAX / 2, cus, ncb);
  const double chunk_heads = (double)P.total_chunks * s->H;
  if (!P.wy) t += kK1FixedUs + kK1PerChunkHeadUs * chunk_heads;
  if (s->cu_seqlens_host) t += kPackedTablesUs;
  if (!split) return t;
  t += (P.wy ? kSplitFixedWyUs : kSplitFixedUs) + kSplitPerChunkHeadUs * chunk_heads;
  if (corr > 0 && longest_steps > 0) {
    t -= kCorrReplacesUs;
    // pass 1's column blocks: dv wide in the one-pass kernel, pass1_block in the other
    const int p1_block = P.wy ? s->dv : P.pass1_block;
    const double p1_wgs = corr * (double)(segs - s->N) * s->H * ((s->dv + s->dk) / p1_block);
    const double rounds = std::max(1.0, std::ceil(p1_wgs / (double)cus));
    t += kPass1FixedUs + kPass1StepUs * (double)L * rounds;
    t += longest_steps > gdn::kMergeTreeMinSteps ? kTreeFixedUs + kTreeSqrtUs * std::sqrt((double)longest_steps)
                                                 : kMergeFixedUs + l2 * (double)longest_steps;
  }
  return t;
}

Plan plan_uncached(const gdn_shape* s, const gdn_opts* o) {
  Plan P;
  for (int64_t n = 0; n < s->N; ++n) {
    const int64_t c = seq_chunks(s, n);
    P.total_chunks += c;
    P.max_chunks = std::max(P.max_chunks, c);
  }
  const int vb_req = o ? o->value_block : 0;
  const int one_pass = o ? o->one_pass : 0;
  P.wy = s->qkv_dtype == GDN_BF16 && (one_pass == 1 || (one_pass == 0 && vb_req == 0));
  P.value_block = P.wy ? (int)s->dv : (s->qkv_dtype == GDN_BF16 && s->dv % 128 == 0 && vb_req != 64) ? 128 : 64;
  P.pass1_block = vb_req == 128 ? 128 : 64;
  P.wmax = (o && o->window_max_chunks > 0) ? o->window_max_chunks : kWindowMaxCap;
  // default window tolerance: 2^-16 for bf16 storage (256 times below its unit
  // roundoff 2^-8), 2^-24 for fp32 (its unit roundoff)
  P.log_eps = (o && o->window_log_eps != 0.f) ? o->window_log_eps
             : (float)std::log(s->qkv_dtype == GDN_BF16 ? 0x1p-16 : 0x1p-24);
  int64_t L = INT_MAX / 2;
  if (!(o && o->no_split) && P.max_chunks > 1) {
    if (o && o->force_segment_chunks > 0) {
      L = o->force_segment_chunks;
    } else {
      // T auto-CP: the split length minimises the modelled call (call_us above, every
      // head assumed to take a lookback window unless the correction is forced: the
      // gates are on the device); no split (L = max_chunks) competes too.  The
      // makespan is simulated (see pass3_makespan), so unequal sequence lengths are
      // scheduled as they will run.
      const int64_t cus = device_cus();
      const double corr = (o && o->force_correction) ? 1.0 : 0.0;
      auto cost = [&](int64_t cand) { return call_us(s, P, o, cand, cus, corr); };
      // candidates: a ladder of round lengths (ratio about 1.25 to 1.5) and the lengths
      // that cut the longest sequence into 2..8 equal segments
      std::vector<int64_t> cands;
      for (int64_t c = kMinSegmentChunks; c < P.max_chunks;) {
        cands.push_back(c);
        c = c < 16 ? c + 4 : (c < 32 ? c + 8 : (c < 64 ? c + 16 : c + c / 2));
      }
      for (int64_t k = 2; k <= 8; ++k) {
        const int64_t c = (P.max_chunks + k - 1) / k;
        if (c >= kMinSegmentChunks && c < P.max_chunks) cands.push_back(c);
      }
      double best = cost(P.max_chunks);
      for (int64_t cand : cands) {
        const double c = cost(cand);
        if (c < best || (c == best && cand > L && L < INT_MAX / 2)) {
          best = c;
          L = cand;
        }
      }
    }
  }
  P.split = L < P.max_chunks;
  // An unsplit plan carries the one-segment value even when a segment length was
  // forced: the kernels' decode without segment tables derives segments per sequence
  // from it (packed input has none; its T spans all sequences).
  P.seg_chunks = P.split ? (int)L : INT_MAX / 2;
  if (P.split) {
    for (int64_t n = 0; n < s->N; ++n)  // an empty sequence still owns one unit (its final state)
      P.total_segs += std::max<int64_t>(1, (seq_chunks(s, n) + L - 1) / L);
  } else {
    P.total_segs = s->N;
  }
  return P;
}

// Plans are memoised per thread: a model calls the library with the same shapes
// layer after layer (and the binding asks for the workspace size before every call),
// while simulating the candidate schedules costs 0.05-0.3 ms of host time.  The key
// holds every input the plan depends on, the packed lengths included, and the CU
// count of the current device; a few entries are kept, replaced round robin.
struct PlanKey {
  int64_t dims[6] = {0, 0, 0, 0, 0, 0};
  int32_t dtypes[2] = {0, 0};
  int32_t no_split = 0, force_segment_chunks = 0, window_max_chunks = 0, value_block = 0, one_pass = 0;
  float window_log_eps = 0.f, lambda1_us = 0.f, lambda2_us = 0.f;
  int cus = 0;
  bool packed = false;
  std::vector<int32_t> cu;

  void set(const gdn_shape* s, const gdn_opts* o, int cus_) {
    const int64_t d[6] = {s->B, s->T, s->H, s->dk, s->dv, s->N};
    std::memcpy(dims, d, sizeof(dims));
    dtypes[0] = s->qkv_dtype;
    dtypes[1] = s->beta_dtype;
    const gdn_opts z{};
    const gdn_opts& r = o ? *o : z;
    no_split = r.no_split;
    force_segment_chunks = r.force_segment_chunks;
    window_max_chunks = r.window_max_chunks;
    value_block = r.value_block;
    one_pass = r.one_pass;
    window_log_eps = r.window_log_eps;
    lambda1_us = r.lambda1_us;
    lambda2_us = r.lambda2_us;
    cus = cus_;
    packed = s->cu_seqlens_host != nullptr;
    if (packed) cu.assign(s->cu_seqlens_host, s->cu_seqlens_host + s->N + 1);
    else cu.clear();
  }
  bool same(const PlanKey& k) const {
    return std::memcmp(dims, k.dims, sizeof(dims)) == 0 && dtypes[0] == k.dtypes[0] &&
           dtypes[1] == k.dtypes[1] && no_split == k.no_split &&
           force_segment_chunks == k.force_segment_chunks &&
           window_max_chunks == k.window_max_chunks && value_block == k.value_block &&
           one_pass == k.one_pass &&
           window_log_eps == k.window_log_eps && lambda1_us == k.lambda1_us &&
           lambda2_us == k.lambda2_us && cus == k.cus && packed == k.packed && cu == k.cu;
  }
};

constexpr int kPlanCacheEntries = 4;
struct PlanCache {
  PlanKey key[kPlanCacheEntries];
  Plan plan[kPlanCacheEntries];
  bool valid[kPlanCacheEntries] = {false, false, false, false};
  int next = 0;
};

Plan make_plan(const gdn_shape* s, const gdn_opts* o) {
  thread_local PlanCache cache;
  thread_local PlanKey probe;
  probe.set(s, o, device_cus());
  for (int i = 0; i < kPlanCacheEntries; ++i)
    if (cache.valid[i] && cache.key[i].same(probe)) return cache.plan[i];
  const Plan P = plan_uncached(s, o);
  const int i = cache.next;
  cache.next = (i + 1) % kPlanCacheEntries;
  cache.key[i] = probe;
  cache.plan[i] = P;
  cache.valid[i] = true;
  return P;
}

// Whether the chunk-inverse kernel runs: on the two-pass path only (the one-pass
// kernel forms the inverses itself, in pass 3 and in pass 1).
bool runs_k1(const Plan& P) { return !P.wy; }

struct Layout {
  size_t tmat = 0, chunk_off = 0, seg_off = 0, seg_order = 0, csum = 0, sstar = 0, mcorr = 0, hstart = 0;
  size_t gmat = 0, gvec = 0, ncorr = 0, seg_win = 0, p1_slots = 0;
  bool has_seg_order = false;
  size_t total = 0;
};

Layout layout(const gdn_shape* s, const Plan& P) {
  Layout L;
  const size_t esz = s->qkv_dtype == GDN_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  L.tmat = take(runs_k1(P) ? (size_t)P.total_chunks * s->H * kChunk * kChunk * esz : 0);
  L.chunk_off = take((size_t)(s->N + 1) * sizeof(int32_t));
  L.seg_off = take((size_t)(s->N + 1) * sizeof(int32_t));
  if (s->cu_seqlens_host && P.split && s->N <= gdn::kSegOrderMaxSeqs) {
    L.seg_order = take((size_t)P.total_segs * sizeof(int32_t));
    L.has_seg_order = true;
  }
  if (P.split) {
    L.ncorr = take(2 * sizeof(uint32_t));
    L.seg_win = take((size_t)P.total_segs * s->H * sizeof(int32_t));
    L.p1_slots = take((size_t)(P.total_segs - s->N) * s->H * sizeof(int32_t));
    L.csum = take((size_t)P.total_chunks * s->H * sizeof(float));
    const size_t slots = (size_t)P.total_segs * s->H;
    L.sstar = take(slots * s->dk * s->dv * sizeof(float));
    L.mcorr = take(slots * 2 * s->dk * s->dk * sizeof(uint16_t));   // bf16 hi + lo
    L.hstart = take(slots * s->dk * s->dv * sizeof(float));
    const int64_t max_steps = (P.max_chunks + P.seg_chunks - 1) / P.seg_chunks - 1;
    if (max_steps > gdn::kMergeTreeMinSteps) {   // group maps of the tree merge
      L.gmat = take(slots * 2 * s->dk * s->dk * sizeof(uint16_t));
      L.gvec = take(slots * s->dk * s->dv * sizeof(float));
    }
  }
  L.total = off;
  return L;
}

gdn::Problem make_problem(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* h0, const int32_t* cu, float scale,
                          void* o, float* hT, const gdn_shape* s, int64_t total_chunks) {
  gdn::Problem p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.cu = cu;
  p.chunk_off = nullptr; p.o = o; p.hT = hT;
  p.T = s->T;
  p.total_chunks = total_chunks;
  p.N = (int)s->N; p.H = (int)s->H; p.dk = (int)s->dk; p.dv = (int)s->dv;
  p.qkv_bf16 = s->qkv_dtype == GDN_BF16;
  p.beta_bf16 = s->beta_dtype == GDN_BF16;
  p.scale = scale;
  return p;
}

int check_inputs(const void* k, const float* g, const void* beta, const int32_t* cu,
                 const gdn_shape* s) {
  if ((cu == nullptr) != (s->cu_seqlens_host == nullptr)) return GDN_ERR_ARG;
  if (s->T > 0 && (!k || !g || !beta)) return GDN_ERR_ARG;
  if (k && !aligned(k, 16)) return GDN_ERR_ARG;
  if (g && !aligned(g, 4)) return GDN_ERR_ARG;
  if (beta && !aligned(beta, s->beta_dtype == GDN_BF16 ? 2 : 4)) return GDN_ERR_ARG;
  if (cu && !aligned(cu, 4)) return GDN_ERR_ARG;
  return GDN_OK;
}


// Every launch of the plan fits the dispatch limits: an AQL dispatch counts work-items
// per grid dimension in 32 bits, so a grid beyond 2^32 - 1 work-items would wrap and
// silently drop work.  Each bound below is the launch's own grid (pass 1 and pass 3
// run 4 threads per value column in either block shape).
bool grids_fit(const gdn_shape* s, const Plan& P) {
  auto fits = [](int64_t groups, int64_t items_each) {
    return groups >= 0 && (items_each == 0 || groups <= gdn::kMaxDispatchItems / items_each);
  };
  const int64_t H = s->H, nh = s->N * s->H;
  if (!fits(P.total_chunks * ((H + 3) / 4), 256)) return false;                  // K1
  const int64_t unit_groups = (P.total_segs * H + 7) / 8;
  if (!fits(unit_groups * 8, s->dv * 4)) return false;                           // pass 3
  if (P.wy && !fits(unit_groups * 8, 512)) return false;                          // one pass
  if (!P.split) return true;
  if (!fits(nh, P.max_chunks > 512 ? 1024 : 256)) return false;                   // gate scan
  if (!fits(unit_groups * 8, (s->dv + s->dk) * 4)) return false;                  // pass 1
  const int64_t merge_threads = s->dk / 16 * 64;
  const int64_t steps = (P.max_chunks + P.seg_chunks - 1) / P.seg_chunks - 1;
  int64_t G = 1;
  while (G * G < steps) ++G;
  const int64_t maxg = steps > gdn::kMergeTreeMinSteps ? (steps + G - 1) / G : 1;
  return fits((nh * maxg + 7) / 8 * 8, (s->dk + s->dv) / 16 * merge_threads);   // merge
}

// Runs stages [first, last] of the forward pass (GDN_STAGE_*, launch order) on one
// workspace; gdn_chunk_fwd is all of them.  Every call validates all arguments and
// plans the same way, so a caller that runs the stages one by one, in order, on one
// stream and workspace, gets the result of gdn_chunk_fwd bit for bit.  Stages the
// plan does not need (the split stages of an unsplit plan, the gate scan when the
// correction is forced) enqueue nothing.
int run_stages(int first, int last, const void* q, const void* k, const void* v, const float* g,
               const void* beta, const float* initial_state, const int32_t* cu_seqlens,
               float scale, void* o, float* final_state, const gdn_shape* shape,
               const gdn_opts* opts, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  auto runs = [&](int st) { return first <= st && st <= last; };
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc == GDN_OK) rc = check_inputs(k, g, beta, cu_seqlens, shape);
  if (rc != GDN_OK) return rc;
  if (shape->T > 0 && (!q || !v || !o)) return GDN_ERR_ARG;
  if ((q && !aligned(q, 16)) || (v && !aligned(v, 16)) || (o && !aligned(o, 16)) ||
      (initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return GDN_ERR_ARG;
  if (!std::isfinite(scale)) return GDN_ERR_ARG;
  const Plan P = make_plan(shape, opts);
  if (!grids_fit(shape, P)) return GDN_ERR_UNSUPPORTED;
  const Layout L = layout(shape, P);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace) || !aligned(workspace, kAlign))
    return GDN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  gdn::Problem p = make_problem(q, k, v, g, beta, initial_state, cu_seqlens, scale, o,
                                final_state, shape, P.total_chunks);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
  int32_t* seg_off = reinterpret_cast<int32_t*>(ws + L.seg_off);
  int32_t* seg_order = reinterpret_cast<int32_t*>(ws + L.seg_order);
  // the packed-sequence tables live in the workspace and are rebuilt by every call (a
  // single stage too), so no kernel indexes by workspace contents it did not write
  if (cu_seqlens) {
    if (gdn::launch_plan_tables(cu_seqlens, p.N, P.seg_chunks, chunk_off,
                                P.split ? seg_off : nullptr, L.has_seg_order ? seg_order : nullptr,
                                stream) != hipSuccess)
      return GDN_ERR_HIP;
  }
  if (cu_seqlens) p.chunk_off = chunk_off;

  void* tmat = ws + L.tmat;
  float* csum = P.split ? reinterpret_cast<float*>(ws + L.csum) : nullptr;
  const bool forced = opts && opts->force_correction;
  // One-pass plans read no T (the one-pass kernel forms it, in pass 3 and in pass 1):
  // the inverse stage of a split one forms the chunk gate sums alone, for the scan.
  const bool listed = P.wy && P.split && !forced;
  // counts of the heads without a window and of pass 1's units (one-pass split plans):
  // zeroed with the gate sums, added to by the gate scan, read first by every
  // correction launch
  uint32_t* ncorr = listed ? reinterpret_cast<uint32_t*>(ws + L.ncorr) : nullptr;
  if (runs(GDN_STAGE_INVERSE)) {
    const gdn::KernelEvents ev = stage_events(opts, GDN_STAGE_INVERSE);
    hipError_t e = hipSuccess;
    if (listed) e = gdn::launch_chunk_gate_sums(p, csum, stream, ev, ncorr);
    else if (!runs_k1(P)) ev.record_empty(stream);
    else e = gdn::launch_chunk_inverse(p, tmat, csum, false, stream, ev);
    if (e != hipSuccess) return GDN_ERR_HIP;
  }

  gdn::FwdPlan plan;
  plan.Tmat = tmat;
  plan.seg_chunks = P.seg_chunks;
  plan.seg_off = (cu_seqlens && P.split) ? seg_off : nullptr;
  plan.seg_order = (cu_seqlens && L.has_seg_order) ? seg_order : nullptr;
  plan.units = P.total_segs * p.H;
  plan.value_block = P.value_block;
  plan.pass1_block = P.pass1_block;
  plan.mode = gdn::kPass3;
  plan.cp = gdn::CpBuffers{};
  plan.ckpt = nullptr;
  plan.bwd_maps = 0;
  if (P.split) {
    plan.cp.force_correction = forced ? 1 : 0;
    plan.cp.sstar = reinterpret_cast<float*>(ws + L.sstar);
    plan.cp.mcorr = ws + L.mcorr;
    plan.cp.hstart = reinterpret_cast<float*>(ws + L.hstart);
    plan.cp.gmat = L.gmat ? ws + L.gmat : nullptr;
    plan.cp.gvec = L.gvec ? reinterpret_cast<float*>(ws + L.gvec) : nullptr;
    plan.cp.ncorr = ncorr;
    int32_t* seg_win = reinterpret_cast<int32_t*>(ws + L.seg_win);
    plan.cp.seg_win = seg_win;
    int32_t* p1_slots = ncorr ? reinterpret_cast<int32_t*>(ws + L.p1_slots) : nullptr;
    plan.cp.p1_slots = p1_slots;
    if (!plan.cp.force_correction && runs(GDN_STAGE_GATE_SCAN)) {
      if (gdn::launch_gate_scan(p, csum, P.max_chunks, P.wmax, nullptr, stream,
                                stage_events(opts, GDN_STAGE_GATE_SCAN), P.log_eps - kWindowMargin, ncorr,
                                P.seg_chunks,
                                cu_seqlens ? seg_off : nullptr, seg_win, p1_slots,
                                (P.total_segs - p.N) * p.H) != hipSuccess)
        return GDN_ERR_HIP;
    }
    if (runs(GDN_STAGE_CP_PASS1)) {
      gdn::FwdPlan p1 = plan;
      p1.mode = gdn::kPass1;
      if (p1_slots) p1.units = (P.total_segs - p.N) * p.H;   // the list's capacity
      const gdn::KernelEvents ev = stage_events(opts, GDN_STAGE_CP_PASS1);
      if ((P.wy ? gdn::launch_fused_wy(p, p1, stream, ev) : gdn::launch_fused_forward(p, p1, stream, ev)) !=
          hipSuccess)
        return GDN_ERR_HIP;
    }
    if (runs(GDN_STAGE_CP_MERGE)) {
      const int max_steps = (int)((P.max_chunks + P.seg_chunks - 1) / P.seg_chunks - 1);
      if (gdn::launch_cp_merge(p, plan, max_steps, stream, stage_events(opts, GDN_STAGE_CP_MERGE)) !=
          hipSuccess)
        return GDN_ERR_HIP;
    }
  }
  if (runs(GDN_STAGE_FORWARD)) {
    const gdn::KernelEvents ev = stage_events(opts, GDN_STAGE_FORWARD);
    if ((P.wy ? gdn::launch_fused_wy(p, plan, stream, ev) : gdn::launch_fused_forward(p, plan, stream, ev)) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int64_t gdn_total_chunks(const gdn_shape* shape) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  int64_t c = 0;
  for (int64_t n = 0; n < shape->N; ++n) c += seq_chunks(shape, n);
  return c;
}

int64_t gdn_plan_segment_chunks(const gdn_shape* shape, const gdn_opts* opts) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  return make_plan(shape, opts).seg_chunks;
}

int gdn_plan_predict_us(const gdn_shape* shape, const gdn_opts* opts, double corrected_fraction,
                        double* us) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  if (!us || !(corrected_fraction >= 0.0 && corrected_fraction <= 1.0)) return GDN_ERR_ARG;
  const Plan P = make_plan(shape, opts);
  const double corr = (opts && opts->force_correction) ? 1.0 : corrected_fraction;
  *us = call_us(shape, P, opts, P.split ? P.seg_chunks : std::max<int64_t>(P.max_chunks, 1), device_cus(), corr);
  return GDN_OK;
}

int gdn_plan_one_pass(const gdn_shape* shape, const gdn_opts* opts) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  return make_plan(shape, opts).wy ? 1 : 0;
}

int gdn_chunk_fwd_workspace_bytes(const gdn_shape* shape, const gdn_opts* opts, size_t* bytes) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  if (!bytes) return GDN_ERR_ARG;
  *bytes = layout(shape, make_plan(shape, opts)).total;
  return GDN_OK;
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, float scale, void* o,
                  float* final_state, const gdn_shape* shape, const gdn_opts* opts,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_stages(0, GDN_NUM_STAGES - 1, q, k, v, g, beta, initial_state, cu_seqlens, scale, o,
                    final_state, shape, opts, workspace, workspace_bytes, stream);
}

int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* initial_state,
                          const int32_t* cu_seqlens, float scale, void* o, float* final_state,
                          const gdn_shape* shape, const gdn_opts* opts, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  const size_t need = layout(shape, make_plan(shape, opts)).total;
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return GDN_ERR_HIP;
  return run_stages(0, GDN_NUM_STAGES - 1, q, k, v, g, beta, initial_state, cu_seqlens, scale, o,
                    final_state, shape, opts, ws, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}

int gdn_chunk_fwd_stage(int stage, const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                        float scale, void* o, float* final_state, const gdn_shape* shape,
                        const gdn_opts* opts, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (stage < 0 || stage >= GDN_NUM_STAGES) return GDN_ERR_ARG;
  return run_stages(stage, stage, q, k, v, g, beta, initial_state, cu_seqlens, scale, o,
                    final_state, shape, opts, workspace, workspace_bytes, stream);
}

int gdn_chunk_fwd_workspace_region(const gdn_shape* shape, const gdn_opts* opts, int region,
                                   size_t* offset, size_t* bytes) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  if (!offset || !bytes || region < 0 || region >= GDN_NUM_REGIONS) return GDN_ERR_ARG;
  const Plan P = make_plan(shape, opts);
  const Layout L = layout(shape, P);
  const size_t esz = shape->qkv_dtype == GDN_BF16 ? 2 : 4;
  const size_t slots = (size_t)P.total_segs * shape->H;
  *offset = 0;
  *bytes = 0;
  switch (region) {
    case GDN_REGION_CHUNK_INVERSE:
      *offset = L.tmat;
      *bytes = runs_k1(P) ? (size_t)P.total_chunks * shape->H * kChunk * kChunk * esz : 0;
      break;
    case GDN_REGION_SEGMENT_WINDOWS:
      if (P.split) {
        *offset = L.seg_win;
        *bytes = slots * sizeof(int32_t);
      }
      break;
    case GDN_REGION_SEGMENT_MAPS:
      if (P.split) {
        *offset = L.sstar;
        *bytes = L.mcorr - L.sstar + slots * 2 * shape->dk * shape->dk * sizeof(uint16_t);
      }
      break;
    default:   // GDN_REGION_SEGMENT_STARTS
      if (P.split) {
        *offset = L.hstart;
        *bytes = slots * shape->dk * shape->dv * sizeof(float);
      }
      break;
  }
  return GDN_OK;
}

int gdn_chunk_inverse(const void* k, const float* g, const void* beta, const int32_t* cu_seqlens,
                      const gdn_shape* shape, void* t_out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  rc = check_inputs(k, g, beta, cu_seqlens, shape);
  if (rc != GDN_OK) return rc;
  const int64_t nch = gdn_total_chunks(shape);
  if (nch > 0 && (!t_out || !aligned(t_out, 16))) return GDN_ERR_ARG;
  if (nch * ((shape->H + 3) / 4) > gdn::kMaxDispatchItems / 256) return GDN_ERR_UNSUPPORTED;
  gdn::Problem p = make_problem(nullptr, k, nullptr, g, beta, nullptr, cu_seqlens, 1.f, nullptr,
                                nullptr, shape, nch);
  if (cu_seqlens) {
    const size_t need = align_up((size_t)(shape->N + 1) * sizeof(int32_t));
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return GDN_ERR_WORKSPACE;
    p.chunk_off = static_cast<int32_t*>(workspace);
    if (gdn::launch_chunk_offsets(cu_seqlens, p.N, static_cast<int32_t*>(workspace), stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  if (gdn::launch_chunk_inverse(p, t_out, nullptr, true, stream) != hipSuccess) return GDN_ERR_HIP;
  return GDN_OK;
}

int gdn_gate_scan_workspace_bytes(const gdn_shape* shape, size_t* bytes) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  if (!bytes) return GDN_ERR_ARG;
  int64_t chunks = 0;
  for (int64_t n = 0; n < shape->N; ++n) chunks += seq_chunks(shape, n);
  *bytes = align_up((size_t)(shape->N + 1) * sizeof(int32_t)) +
           align_up((size_t)shape->N * shape->H * kWindowMaxCap * sizeof(uint32_t)) +
           align_up((size_t)chunks * shape->H * sizeof(float));
  return GDN_OK;
}

int gdn_gate_scan(const float* g, const int32_t* cu_seqlens, const gdn_shape* shape,
                  const gdn_opts* opts, int32_t* window_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  if ((cu_seqlens == nullptr) != (shape->cu_seqlens_host == nullptr)) return GDN_ERR_ARG;
  if ((shape->T > 0 && !g) || (g && !aligned(g, 4)) || !window_out || !aligned(window_out, 4))
    return GDN_ERR_ARG;
  size_t need = 0;
  gdn_gate_scan_workspace_bytes(shape, &need);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return GDN_ERR_WORKSPACE;
  const Plan P = make_plan(shape, opts);
  // chunk gate sums (256 threads per 4 heads of a chunk), the scan (256 or 1024 per
  // sequence-head) and the finalisation (one thread per sequence-head) must fit a dispatch
  if (P.total_chunks * ((shape->H + 3) / 4) > gdn::kMaxDispatchItems / 256 ||
      shape->N * shape->H > gdn::kMaxDispatchItems / 1024)
    return GDN_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  const size_t off_best = align_up((size_t)(shape->N + 1) * sizeof(int32_t));
  const size_t off_csum = off_best + align_up((size_t)shape->N * shape->H * kWindowMaxCap *
                                              sizeof(uint32_t));
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws);
  uint32_t* best = reinterpret_cast<uint32_t*>(ws + off_best);
  float* csum = reinterpret_cast<float*>(ws + off_csum);
  gdn::Problem p = make_problem(nullptr, nullptr, nullptr, g, nullptr, nullptr, cu_seqlens, 1.f,
                                nullptr, nullptr, shape, P.total_chunks);
  if (cu_seqlens &&
      gdn::launch_plan_tables(cu_seqlens, p.N, 1, chunk_off, nullptr, nullptr, stream) != hipSuccess)
    return GDN_ERR_HIP;
  if (cu_seqlens) p.chunk_off = chunk_off;
  if (gdn::launch_chunk_gate_sums(p, csum, stream) != hipSuccess) return GDN_ERR_HIP;
  if (gdn::launch_gate_scan(p, csum, P.max_chunks, P.wmax, best, stream) != hipSuccess)
    return GDN_ERR_HIP;
  if (gdn::launch_gate_finalize(p, best, P.wmax, P.log_eps - kWindowMargin, window_out, stream) !=
      hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

// The backward's split of the reverse sweep (the state-gradient chain is serial per
// sequence like the forward's state chain, so a (sequence, head, 32 value columns)
// workgroup per CU leaves most of the chip idle when there are few of them): segments
// of L chunks, each run from the true state gradient at its end, which a merge over
// the segments' maps finds.  A pass costs each segment twice its chunks (pass 1 and
// the full pass), so it pays once there are enough segments per sequence: at least
// kBwdMinSegments, L at least kBwdMinSegChunks, and as many segments as keep every CU
// busy.  no_split and force_segment_chunks as for the forward.
constexpr int kBwdMinSegments = 4, kBwdMinSegChunks = 8;
static int64_t bwd_segment_chunks(const gdn_shape* s, const gdn_opts* o, int64_t max_chunks) {
  if (max_chunks <= 1 || (o && o->no_split)) return std::max<int64_t>(1, max_chunks);
  if (o && o->force_segment_chunks > 0) return std::min<int64_t>(o->force_segment_chunks, max_chunks);
  const int64_t units = s->N * s->H * (s->dv / gdn::kBwdColumnBlock);
  const int64_t segs = device_cus() / std::max<int64_t>(1, units);
  if (segs < kBwdMinSegments || max_chunks < kBwdMinSegments * kBwdMinSegChunks) return max_chunks;
  return std::max<int64_t>(kBwdMinSegChunks, (max_chunks + segs - 1) / segs);
}

// Backward workspace: packed chunk offsets, the chunk inverses and chunk-start states
// of the checkpoint pass, the workgroups' fp32 shares of dq, dk, dbeta and dg, and
// with a split the segment offsets, the segments' transposed maps, offsets and end
// state gradients (and the merge's group maps for long chains).
struct BwdLayout {
  size_t chunk_off = 0, tmat = 0, hchk = 0, dhchk = 0, gnh = 0, dq_p = 0, dk_p = 0, dbeta_p = 0, dg_p = 0, total = 0;
  size_t seg_off = 0, seg_b = 0, seg_m = 0, seg_g = 0, gmat = 0, gvec = 0;
  int max_chunks = 0;
  int64_t seg_chunks = 0, total_segs = 0, max_steps = 0;
  bool split = false;
  bool mfma = false;   // bf16 q / k / v: the MFMA chain and per-chunk kernels
};
static BwdLayout bwd_layout(const gdn_shape* s, const gdn_opts* o) {
  BwdLayout L;
  int64_t chunks = 0;
  for (int64_t n = 0; n < s->N; ++n) {
    chunks += seq_chunks(s, n);
    L.max_chunks = std::max(L.max_chunks, (int)seq_chunks(s, n));
  }
  L.seg_chunks = bwd_segment_chunks(s, o, L.max_chunks);
  L.split = L.seg_chunks < L.max_chunks;
  for (int64_t n = 0; n < s->N; ++n) {
    const int64_t sg = L.split ? std::max<int64_t>(1, (seq_chunks(s, n) + L.seg_chunks - 1) / L.seg_chunks) : 1;
    L.total_segs += sg;
    L.max_steps = std::max(L.max_steps, sg - 1);
  }
  const int64_t tot = s->B * s->T, nblk = s->dv / gdn::kBwdColumnBlock;
  const size_t esz = s->qkv_dtype == GDN_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  L.chunk_off = take(s->cu_seqlens_host ? (size_t)(s->N + 1) * sizeof(int32_t) : 0);
  L.tmat = take((size_t)chunks * s->H * kChunk * kChunk * esz);
  L.hchk = take((size_t)chunks * s->H * s->dk * s->dv * sizeof(float));
  L.mfma = s->qkv_dtype == GDN_BF16;
  if (L.mfma) {
    L.dhchk = take((size_t)chunks * s->H * 2 * s->dk * s->dv * sizeof(uint16_t));
    L.gnh = take((size_t)chunks * s->H * nblk * sizeof(float));
  } else {
    L.dq_p = take((size_t)nblk * tot * s->H * s->dk * sizeof(float));
    L.dk_p = take((size_t)nblk * tot * s->H * s->dk * sizeof(float));
    L.dbeta_p = take((size_t)nblk * tot * s->H * sizeof(float));
    L.dg_p = take((size_t)nblk * tot * s->H * sizeof(float));
  }
  if (L.split) {
    const size_t slots = (size_t)L.total_segs * s->H;
    L.seg_off = take(s->cu_seqlens_host ? (size_t)(s->N + 1) * sizeof(int32_t) : 0);
    L.seg_b = take(slots * s->dk * s->dv * sizeof(float));
    L.seg_m = take(slots * 2 * s->dk * s->dk * sizeof(uint16_t));
    L.seg_g = take(slots * s->dk * s->dv * sizeof(float));
    if (L.max_steps > gdn::kMergeTreeMinSteps) {
      L.gmat = take(slots * 2 * s->dk * s->dk * sizeof(uint16_t));
      L.gvec = take(slots * s->dk * s->dv * sizeof(float));
    }
  }
  L.total = off;
  return L;
}

int gdn_chunk_bwd_workspace_bytes(const gdn_shape* shape, const gdn_opts* opts, size_t* bytes) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc != GDN_OK) return rc;
  if (!bytes) return GDN_ERR_ARG;
  *bytes = bwd_layout(shape, opts).total;
  return GDN_OK;
}

int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, float scale,
                  const void* d_o, const float* d_final_state, void* dq, void* dk, void* dv,
                  float* dg, void* dbeta, float* d_initial_state, const gdn_shape* shape,
                  const gdn_opts* opts, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc == GDN_OK) rc = validate_opts(opts);
  if (rc == GDN_OK) rc = check_inputs(k, g, beta, cu_seqlens, shape);
  if (rc != GDN_OK) return rc;
  if (!std::isfinite(scale)) return GDN_ERR_ARG;
  if (shape->T > 0 && (!q || !v || !d_o || !dq || !dk || !dv || !dg || !dbeta)) return GDN_ERR_ARG;
  const int eb = shape->beta_dtype == GDN_BF16 ? 2 : 4;
  if ((q && !aligned(q, 16)) || (v && !aligned(v, 16)) || (d_o && !aligned(d_o, 16)) ||
      (dq && !aligned(dq, 16)) || (dk && !aligned(dk, 16)) || (dv && !aligned(dv, 16)) ||
      (dg && !aligned(dg, 4)) || (dbeta && !aligned(dbeta, eb)) ||
      (initial_state && !aligned(initial_state, 16)) || (d_final_state && !aligned(d_final_state, 16)) ||
      (d_initial_state && !aligned(d_initial_state, 16)))
    return GDN_ERR_ARG;
  const BwdLayout L = bwd_layout(shape, opts);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace) || !aligned(workspace, kAlign))
    return GDN_ERR_WORKSPACE;
  const int64_t nblk = shape->dv / gdn::kBwdColumnBlock;
  if (L.total_segs * shape->H * nblk > gdn::kMaxDispatchItems / 1024) return GDN_ERR_UNSUPPORTED;
  const int64_t total_chunks = gdn_total_chunks(shape);
  if (L.mfma && total_chunks * shape->H > gdn::kMaxDispatchItems / 512) return GDN_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  gdn::Problem p = make_problem(q, k, v, g, beta, initial_state, cu_seqlens, scale, nullptr, nullptr,
                                shape, total_chunks);
  int32_t* seg_off = L.split && cu_seqlens ? reinterpret_cast<int32_t*>(ws + L.seg_off) : nullptr;
  if (cu_seqlens) {
    int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    if (gdn::launch_plan_tables(cu_seqlens, p.N, (int)L.seg_chunks, chunk_off, seg_off, nullptr, stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
    p.chunk_off = chunk_off;
  }
  gdn::BwdArgs a;
  a.d_o = d_o;
  a.dhT = d_final_state;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.dh0 = d_initial_state;
  a.hchk = reinterpret_cast<float*>(ws + L.hchk);
  a.dq_p = reinterpret_cast<float*>(ws + L.dq_p);
  a.dk_p = reinterpret_cast<float*>(ws + L.dk_p);
  a.dbeta_p = reinterpret_cast<float*>(ws + L.dbeta_p);
  a.dg_p = reinterpret_cast<float*>(ws + L.dg_p);
  a.total_tokens = shape->B * shape->T;
  a.seg_chunks = L.split ? (int)L.seg_chunks : 0;
  a.seg_off = seg_off;
  a.units = (L.split ? L.total_segs : shape->N) * shape->H;
  a.mode = gdn::kBwdFull;
  a.seg_b = L.split ? reinterpret_cast<float*>(ws + L.seg_b) : nullptr;
  a.seg_g = L.split ? reinterpret_cast<const float*>(ws + L.seg_g) : nullptr;
  void* tmat = ws + L.tmat;
  a.tmat = tmat;
  a.dhchk = L.mfma ? ws + L.dhchk : nullptr;
  a.gnh = L.mfma ? reinterpret_cast<float*>(ws + L.gnh) : nullptr;
  if (total_chunks > 0) {
    // the state at every chunk start, by the forward's own recurrence: the chunk
    // inverses (whole, for the MFMA backward's transposed reads), then the checkpoint
    // pass over whole sequences (one segment each)
    if (gdn::launch_chunk_inverse(p, tmat, nullptr, L.mfma, stream) != hipSuccess) return GDN_ERR_HIP;
    gdn::FwdPlan ck;
    ck.Tmat = tmat;
    ck.seg_chunks = std::max(1, L.max_chunks);
    ck.seg_off = nullptr;
    ck.seg_order = nullptr;
    ck.units = p.N * (int64_t)p.H;
    ck.value_block = 64;
    ck.pass1_block = 64;
    ck.mode = gdn::kCkpt;
    ck.cp = gdn::CpBuffers{};
    ck.ckpt = a.hchk;
    ck.bwd_maps = 0;
    if (gdn::launch_fused_forward(p, ck, stream) != hipSuccess) return GDN_ERR_HIP;
  }
  if (L.split) {
    // the state gradient at every segment's end: the transposed segment maps (the
    // forward's pass 1 on the identity columns), the offsets (the backward from a zero
    // gradient at each segment's end), and the merge over the segments last to first
    // from dhT
    gdn::FwdPlan mp;
    mp.Tmat = tmat;
    mp.seg_chunks = (int)L.seg_chunks;
    mp.seg_off = seg_off;
    mp.seg_order = nullptr;
    mp.units = L.total_segs * shape->H;
    mp.value_block = 64;
    mp.pass1_block = 64;
    mp.mode = gdn::kPass1;
    mp.cp = gdn::CpBuffers{};
    mp.cp.force_correction = 1;
    mp.cp.mcorr = ws + L.seg_m;
    mp.cp.sstar = a.seg_b;
    mp.cp.hstart = reinterpret_cast<float*>(ws + L.seg_g);
    mp.cp.gmat = L.gmat ? ws + L.gmat : nullptr;
    mp.cp.gvec = L.gvec ? reinterpret_cast<float*>(ws + L.gvec) : nullptr;
    mp.ckpt = nullptr;
    mp.bwd_maps = 1;
    if (gdn::launch_fused_forward(p, mp, stream) != hipSuccess) return GDN_ERR_HIP;
    gdn::BwdArgs ch = a;
    ch.mode = gdn::kBwdChain;
    if ((L.mfma ? gdn::launch_bwd_dh(p, ch, stream) : gdn::launch_chunk_bwd(p, ch, stream)) != hipSuccess)
      return GDN_ERR_HIP;
    gdn::Problem pm = p;
    pm.h0 = d_final_state;   // the merge's chain starts from the gradient of the final state
    mp.bwd_maps = 0;
    if (gdn::launch_cp_merge(pm, mp, (int)L.max_steps, stream) != hipSuccess) return GDN_ERR_HIP;
  }
  if (L.mfma) {
    if (gdn::launch_bwd_dh(p, a, stream) != hipSuccess) return GDN_ERR_HIP;
    if (gdn::launch_bwd_grads(p, a, stream) != hipSuccess) return GDN_ERR_HIP;
  } else if (gdn::launch_chunk_bwd(p, a, stream) != hipSuccess) {
    return GDN_ERR_HIP;
  }
  return GDN_OK;
}

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP launch failed";
    case GDN_ERR_SCRATCH: return "problem needs more than the built-in scratch of gdn_chunk_fwd_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
