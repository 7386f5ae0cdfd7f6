// Eviction selection and cache compaction for gfx950.
//
// Selection (DropKV implementation notes, "Algorithm 1": the smallest scores are
// evicted): per KV head, evict the k = n - budget smallest scores by the total
// order (score, index) and list the survivors in ascending index order.  Scores
// map to order-preserving 32-bit keys; an exact MSB-first radix select (a
// 12-bit digit, then two 10-bit digits over the candidates of the threshold
// bin) finds the k-th smallest key T and how many of the keys equal to T must
// go; an ordered pass with block-wide scans then emits the survivors.
//
// Compaction (Section 2.2: eviction removes tokens from the resident cache):
// 16-byte row-chunk gathers k_out[g][r] = k[g][keep[g][r]], v likewise.
#include <float.h>

#include "common.h"

namespace dropkv {

// Selection is exact integer arithmetic on order-preserving keys.  A head of
// at most 16384 tokens is one workgroup (select_solo): the three radix rounds,
// the ties and the ordered emission all stay in LDS.  When a larger head's
// team of ceil(n / 16384) workgroups fits on the device at once, one
// kernel does everything with each workgroup's keys held in registers: a 12-bit
// histogram round over the team (device-scope adds, then a per-head barrier)
// finds the bin holding the k-th smallest key; the team then exchanges that
// bin's keys and each member's count of keys above it, after which every
// member finds T, its own output offset and its evicted ties without further
// waiting, and emits its survivors.  (If the bin holds more than 8192 keys, two
// more histogram rounds and an exchange of per-member counts replace the
// candidate exchange.)  Otherwise selection runs as four wide kernels over
// blocks of kSelBlock tokens:
//   s1  12-bit histogram of the keys' top bits (per-block LDS, then global adds)
//   find1  per head, the bin b1 holding the k-th smallest key
//   s2  count keys above b1 per block and collect the keys of bin b1 (with
//       their indices) as candidates
//   s3  per head: the exact k-th smallest key T from the candidates (two more
//       10-bit digits), how many keys equal to T are evicted, and each block's
//       output offset and number of evicted ties
//   s4  ordered emission of the survivors, and clean-up of the shared scratch
constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kSelBlock = kSelThreads * kSelPer;   // 4096 tokens per block
constexpr int kCandCap = 8192;
constexpr int kS3Threads = 1024;

// Exclusive block scan of one uint per thread (NW waves); returns the total too.
// `sh` holds at least NW words; the block may reuse it once this returns.
template <int NW>
__device__ __forceinline__ uint32_t block_exscan(uint32_t x, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sh[w];
    tot += t;
    before += w < wid ? t : 0u;
  }
  *total = tot;
  __syncthreads();
  return before + incl - x;
}

struct SelArgs {
  const float* scores;
  int32_t* keep;
  int64_t n, budget;
  int nblk;                 // blocks of kSelBlock tokens per head
  const uint32_t* latch;
  SelScratch sc;
  int64_t wait;             // single-launch path: polls at a team barrier before a
                            // workgroup finishes its share alone (< 0: at once)
  int pre1;                 // single-launch path: the first-digit histogram of the
                            // head's scores is already in sc.fh (built by the second
                            // pass, without the padding slots)
};

// Word 0 of the latch holds the errors of scoring, selection and packing; word 1
// those found by the in-place compaction's own checks (kept apart so that one
// head's failed check does not stop the moves of the call's other heads).
__device__ __forceinline__ bool latched(const uint32_t* latch) {
  return (__atomic_load_n(latch, __ATOMIC_RELAXED) | __atomic_load_n(latch + 1, __ATOMIC_RELAXED)) != 0u;
}

__global__ __launch_bounds__(kSelThreads) void select_s1(SelArgs a) {
  __shared__ uint32_t h[kBins1];
  const bool stop = latched(a.latch);   // tested once the scores are requested
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)b * kSelBlock;
  const bool full = base + kSelBlock <= a.n;
  float x[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    x[i] = (j < a.n) ? sg[j] : 0.f;
  }
  if (stop) return;
  for (int i = tid; i < kBins1; i += kSelThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    const uint32_t bin = order_key(x[i]) >> 20;
    if (full) {
      // a wave whose 64 keys share one bin adds once (heavy ties)
      const uint32_t b0 = __shfl(bin, 0);
      if (__all(bin == b0)) {
        if ((tid & 63) == 0) atomicAdd(&h[b0], 64u);
        continue;
      }
    }
    if (j < a.n) atomicAdd(&h[bin], 1u);
  }
  __syncthreads();
  uint32_t* hg = a.sc.hist1 + (size_t)g * kBins1;
  for (int i = tid; i < kBins1; i += kSelThreads)
    if (h[i]) atomicAdd(&hg[i], h[i]);
}

// Bin holding the krem-th smallest key among hist[0..nbins): returns the bin and
// the count of keys in lower bins.  Whole block participates.
template <int NW>
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t krem, uint32_t* s_bin,
                         uint32_t* s_below, uint32_t* sh) {
  const int per = (nbins + NW * 64 - 1) / (NW * 64);
  const int t = threadIdx.x;
  uint32_t loc = 0u;
  for (int i = 0; i < per; ++i) {
    const int bb = t * per + i;
    if (bb < nbins) loc += hist[bb];
  }
  uint32_t tot;
  const uint32_t excl = block_exscan<NW>(loc, &tot, sh);
  if (excl < krem && excl + loc >= krem) {
    uint32_t c = excl;
    for (int i = 0; i < per; ++i) {
      const int bb = t * per + i;
      const uint32_t hb = (bb < nbins) ? hist[bb] : 0u;
      if (c + hb >= krem) { *s_bin = (uint32_t)bb; *s_below = c; break; }
      c += hb;
    }
  }
  __syncthreads();
}

// Once per head: the 12-bit bin holding the k-th smallest key, and the rank
// left within it (so that s2's blocks read two words, not the histogram).
__global__ __launch_bounds__(kSelThreads) void select_find1(SelArgs a) {
  __shared__ uint32_t sh[2 * (kSelThreads / 64) + 1];
  __shared__ uint32_t s_bin, s_below;
  if (latched(a.latch)) return;
  const int g = blockIdx.x;
  const uint32_t kev = (uint32_t)(a.n - a.budget);
  find_bin<kSelThreads / 64>(a.sc.hist1 + (size_t)g * kBins1, kBins1, kev, &s_bin, &s_below, sh);
  if (threadIdx.x == 0) {
    a.sc.b1[g] = s_bin;
    a.sc.krem1[g] = kev - s_below;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_s2(SelArgs a) {
  __shared__ uint32_t sh[2 * (kSelThreads / 64) + 1];
  __shared__ uint32_t s_cnt, s_base;
  __shared__ uint32_t lk[kSelBlock];
  __shared__ int32_t li[kSelBlock];
  // every read (latch, this block's scores, the head's threshold bin) is
  // requested before any is used: one memory round trip
  const bool stop = latched(a.latch);
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)b * kSelBlock;
  float x[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    x[i] = (j < a.n) ? sg[j] : 0.f;
  }
  const uint32_t b1 = a.sc.b1[g];
  if (stop) return;
  if (tid == 0) s_cnt = 0u;
  __syncthreads();
  uint32_t above = 0u;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    if (j < a.n) {
      const uint32_t key = order_key(x[i]);
      const uint32_t bin = key >> 20;
      if (bin > b1) ++above;
      if (bin == b1) {
        const uint32_t slot = atomicAdd(&s_cnt, 1u);
        lk[slot] = key;
        li[slot] = (int32_t)j;
      }
    }
  }
  uint32_t tot;
  (void)block_exscan<kSelThreads / 64>(above, &tot, sh);
  if (tid == 0) {
    a.sc.blk_above[(size_t)g * a.nblk + b] = tot;
    s_base = s_cnt ? atomicAdd(&a.sc.cand_cnt[g], s_cnt) : 0u;
  }
  __syncthreads();
  for (uint32_t i = tid; i < s_cnt; i += kSelThreads) {
    const uint32_t slot = s_base + i;
    if (slot < (uint32_t)kCandCap) {
      a.sc.cand_key[(size_t)g * kCandCap + slot] = lk[i];
      a.sc.cand_idx[(size_t)g * kCandCap + slot] = li[i];
    }
  }
}

__global__ __launch_bounds__(kS3Threads) void select_s3(SelArgs a) {
  constexpr int NW = kS3Threads / 64;
  __shared__ uint32_t sh[2 * NW + 1];
  __shared__ uint32_t h[1024];
  __shared__ uint32_t s_bin, s_below;
  __shared__ uint32_t ck[kCandCap];
  if (latched(a.latch)) return;
  const int g = blockIdx.x, tid = threadIdx.x;
  const uint32_t b1 = a.sc.b1[g];
  uint32_t krem = a.sc.krem1[g];
  const uint32_t cnt = a.sc.cand_cnt[g];
  const bool inlds = cnt <= (uint32_t)kCandCap;
  const float* sg = a.scores + (size_t)g * a.n;
  if (inlds)
    for (uint32_t i = tid; i < cnt; i += kS3Threads) ck[i] = a.sc.cand_key[(size_t)g * kCandCap + i];
  // two 10-bit digits below the 12-bit bin; the candidates live in LDS unless
  // they overflowed the buffer, then the head's scores are re-read
  uint32_t prefix = b1 << 20, mask = 0xfff00000u;
  for (int shift = 10; shift >= 0; shift -= 10) {
    for (int i = tid; i < 1024; i += kS3Threads) h[i] = 0u;
    __syncthreads();
    if (inlds) {
      for (uint32_t i = tid; i < cnt; i += kS3Threads) {
        const uint32_t key = ck[i];
        if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 1023u], 1u);
      }
    } else {
      for (int64_t j = tid; j < a.n; j += kS3Threads) {
        const uint32_t key = order_key(sg[j]);
        if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 1023u], 1u);
      }
    }
    __syncthreads();
    find_bin<NW>(h, 1024, krem, &s_bin, &s_below, sh);
    prefix |= s_bin << shift;
    mask |= 1023u << shift;
    krem -= s_below;
    __syncthreads();
  }
  const uint32_t T = prefix, need = krem;
  // per-block counts of bin-b1 keys above T and of ties (== T)
  uint32_t* above_in = a.sc.blk_above_in + (size_t)g * a.nblk;
  uint32_t* ties = a.sc.blk_ties + (size_t)g * a.nblk;
  for (int i = tid; i < a.nblk; i += kS3Threads) { above_in[i] = 0u; ties[i] = 0u; }
  __syncthreads();
  if (inlds) {
    for (uint32_t i = tid; i < cnt; i += kS3Threads) {
      const uint32_t key = ck[i];
      const int blk = a.sc.cand_idx[(size_t)g * kCandCap + i] / kSelBlock;
      if (key > T) atomicAdd(&above_in[blk], 1u);
      else if (key == T) atomicAdd(&ties[blk], 1u);
    }
  } else {
    for (int64_t j = tid; j < a.n; j += kS3Threads) {
      const uint32_t key = order_key(sg[j]);
      if ((key >> 20) != b1) continue;
      const int blk = (int)(j / kSelBlock);
      if (key > T) atomicAdd(&above_in[blk], 1u);
      else if (key == T) atomicAdd(&ties[blk], 1u);
    }
  }
  __syncthreads();
  // offsets: keep count of block = above b1 + above T within b1 + kept ties;
  // evicted ties are the oldest `need` ones, so they fill blocks in order
  uint32_t run_keep = 0u, run_ties = 0u;
  uint32_t* off = a.sc.blk_off + (size_t)g * a.nblk;
  uint32_t* evt = a.sc.blk_evt + (size_t)g * a.nblk;
  for (int c0 = 0; c0 < a.nblk; c0 += kS3Threads) {
    const int bb = c0 + tid;
    const uint32_t tb = (bb < a.nblk) ? ties[bb] : 0u;
    uint32_t ttot;
    const uint32_t tpre = run_ties + block_exscan<NW>(tb, &ttot, sh);
    const uint32_t ev = (need > tpre) ? min(tb, need - tpre) : 0u;
    const uint32_t kc = (bb < a.nblk) ? a.sc.blk_above[(size_t)g * a.nblk + bb] + above_in[bb] + (tb - ev) : 0u;
    uint32_t ktot;
    const uint32_t kpre = run_keep + block_exscan<NW>(kc, &ktot, sh);
    if (bb < a.nblk) { off[bb] = kpre; evt[bb] = ev; }
    run_ties += ttot;
    run_keep += ktot;
  }
  if (tid == 0) a.sc.T[g] = T;
}

__global__ __launch_bounds__(kSelThreads) void select_s4(SelArgs a) {
  __shared__ uint32_t sh[2 * (kSelThreads / 64) + 1];
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  // every read (latch, block parameters, this thread's scores) is requested
  // before any is used: one memory round trip
  const bool skip = latched(a.latch);
  const uint32_t T = a.sc.T[g];
  const uint32_t off = a.sc.blk_off[(size_t)g * a.nblk + b];
  const uint32_t ev = a.sc.blk_evt[(size_t)g * a.nblk + b];
  const float* sg = a.scores + (size_t)g * a.n;
  // thread owns kSelPer consecutive tokens so that index order = (thread, i)
  const int64_t base = (int64_t)b * kSelBlock + (int64_t)tid * kSelPer;
  uint32_t keys[kSelPer];
  if (base + kSelPer <= a.n && (((size_t)g * a.n + base) & 3) == 0) {   // 16-byte aligned run
    float4 x[kSelPer / 4];
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) x[q] = *reinterpret_cast<const float4*>(sg + base + 4 * q);
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
      keys[4 * q + 0] = order_key(x[q].x);
      keys[4 * q + 1] = order_key(x[q].y);
      keys[4 * q + 2] = order_key(x[q].z);
      keys[4 * q + 3] = order_key(x[q].w);
    }
  } else {
    float x[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) x[i] = (base + i < a.n) ? sg[base + i] : 0.f;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) keys[i] = (base + i < a.n) ? order_key(x[i]) : 0u;
  }
  if (!skip) {
    int32_t* kg = a.keep + (size_t)g * a.budget;
    uint32_t nt = 0u;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i)
      if (base + i < a.n && keys[i] == T) ++nt;
    uint32_t ttot;
    uint32_t rank = block_exscan<kSelThreads / 64>(nt, &ttot, sh);
    uint32_t kc = 0u, keepbits = 0u;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int64_t j = base + i;
      if (j >= a.n) continue;
      bool keepit = keys[i] > T;
      if (keys[i] == T) { keepit = rank >= ev; ++rank; }
      if (keepit) { keepbits |= 1u << i; ++kc; }
    }
    uint32_t ktot;
    uint32_t pos = off + block_exscan<kSelThreads / 64>(kc, &ktot, sh);
#pragma unroll
    for (int i = 0; i < kSelPer; ++i)
      if ((keepbits >> i) & 1u) {
        if (pos < (uint32_t)a.budget) kg[pos] = (int32_t)(base + i);
        ++pos;
      }
  }
  // leave the shared scratch zeroed for the next call
  const int slice = (kBins1 + a.nblk - 1) / a.nblk;
  uint32_t* hg = a.sc.hist1 + (size_t)g * kBins1;
  for (int i = b * slice + tid; i < min(kBins1, (b + 1) * slice); i += kSelThreads) hg[i] = 0u;
  if (b == 0 && tid == 0) a.sc.cand_cnt[g] = 0u;
}

// ------------------------------------------------ single-launch selection --
// A team of ceil(n / kFusedBlock) workgroups per head, kFusedThreads threads
// each holding kFusedPer consecutive keys in registers.  Large workgroups keep
// the device-scope histogram adds and reads shallow (at most a team's worth of
// adds land on one bin); 16 keys per thread (8 workgroups per head at 128K
// tokens) load the keys sooner than 32 and measured fastest on MI355X
// (23 vs 28 us over 8 heads of 128K tokens; 8 or 12 keys: 25 us).
// The launch is an ordinary one: a cooperative launch (guaranteed
// co-residency) measured 16 us slower per call on MI355X.  A team member that
// waits too long at a team barrier (its teammates not resident, e.g. on a
// device shared with other work) does not fail: it finishes its share alone
// from the scores in memory (select_alone), which gives the same keep entries.
#ifndef DROPKV_SEL_THREADS
#define DROPKV_SEL_THREADS 1024
#endif
#ifndef DROPKV_SEL_PER
#define DROPKV_SEL_PER 16
#endif
constexpr int kFusedThreads = DROPKV_SEL_THREADS;
constexpr int kFusedPer = DROPKV_SEL_PER;
constexpr int kFusedBlock = kFusedThreads * kFusedPer;   // tokens per workgroup (16384 by default)
static_assert(kFusedBlock < 65536, "per-member counts are scanned packed in 16 bits");
static_assert(kFusedThreads >= 256 && kFusedThreads <= 1024 && kFusedPer % 4 == 0, "team shape");
constexpr int kFusedBins = kBins1 + 2 * 1024;            // per-head histograms of the three rounds
constexpr int kFusedCand = 8192;                         // threshold-bin keys a team exchanges

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive at the head's barrier and wait for `target` arrivals in total (the
// counter only grows during one call).  Everything the team exchanges goes
// through device-scope accesses (atomics, and agent-scope stores and loads that
// bypass the non-coherent L2), so no cache maintenance is needed: the barrier
// below first waits for every wave's accesses to complete, then arrives.
// Returns false, for every thread of the workgroup, if the wait gave up after
// `wait` polls.
__device__ bool team_barrier(uint32_t* bar, uint32_t target, int64_t wait, int* s_ok) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t o = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(o) : "memory");
    int64_t spins = 0;
    int ok = 1;
    while (load_agent(bar) < target) {
      if (++spins > wait) { ok = 0; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Like find_bin, over a histogram whose bins t * PER .. t * PER + PER - 1 this
// thread holds in hv.
template <int NW, int PER>
__device__ void find_bin_regs(const uint32_t (&hv)[PER], uint32_t krem, uint32_t* s_bin,
                              uint32_t* s_below, uint32_t* s_count, uint32_t* sh) {
  const int t = threadIdx.x;
  uint32_t loc = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) loc += hv[i];
  uint32_t tot;
  const uint32_t excl = block_exscan<NW>(loc, &tot, sh);
  if (excl < krem && excl + loc >= krem) {
    uint32_t c = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (c < krem && c + hv[i] >= krem) {
        *s_bin = (uint32_t)(t * PER + i);
        *s_below = c;
        *s_count = hv[i];
      }
      c += hv[i];
    }
  }
  __syncthreads();
}

// Like find_bin, over a histogram the team built with device-scope adds.
template <int NW, int NB>
__device__ void find_bin_agent(const uint32_t* hist, uint32_t krem, uint32_t* s_bin,
                               uint32_t* s_below, uint32_t* s_count, uint32_t* sh) {
  constexpr int PER = NB / (NW * 64);
  uint32_t hv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) hv[i] = load_agent(hist + threadIdx.x * PER + i);
  find_bin_regs<NW, PER>(hv, krem, s_bin, s_below, s_count, sh);
}

// One radix round: add this workgroup's keys matching (prefix, mask) to the
// head's histogram of digit (key >> shift) & (NB - 1), wait for the rest of the
// team, then narrow the prefix to the bin holding the krem-th smallest key.
// In the first round every key matches (mask = 0).
template <int NB, bool FIRST>
__device__ bool radix_round(const uint32_t (&key)[kFusedPer], int shift, uint32_t* h,
                            uint32_t* gh, uint32_t* bar, uint32_t target, int64_t wait,
                            uint32_t& prefix, uint32_t& mask, uint32_t& krem, uint32_t* sh,
                            uint32_t* s_bin, uint32_t* s_below, uint32_t* s_count, int* s_ok) {
  constexpr int NW = kFusedThreads / 64;
  constexpr int PER = NB / kFusedThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) h[i * kFusedThreads + tid] = 0u;
  __syncthreads();
  if (FIRST) {
    // consecutive tokens often share a bin (pooling makes plateaus): one add per run
    uint32_t run = 0u;
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i) {
      const uint32_t bin = (key[i] >> shift) & (NB - 1);
      ++run;
      const bool last = i == kFusedPer - 1 || ((key[i + (i < kFusedPer - 1)] >> shift) & (NB - 1)) != bin;
      if (last) atomicAdd(&h[bin], run);
      run = last ? 0u : run;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i)
      if ((key[i] & mask) == prefix) atomicAdd(&h[(key[i] >> shift) & (NB - 1)], 1u);
  }
  __syncthreads();
  // issue every device-scope add, then wait once for all of them
  uint32_t hv[PER], old[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) hv[i] = h[i * kFusedThreads + tid];
#pragma unroll
  for (int i = 0; i < PER; ++i)
    old[i] = hv[i] ? __hip_atomic_fetch_add(&gh[i * kFusedThreads + tid], hv[i], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                   : 0u;
  uint32_t sink = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) sink |= old[i];
  asm volatile("s_waitcnt vmcnt(0)" ::"v"(sink) : "memory");
  if (!team_barrier(bar, target, wait, s_ok)) return false;
  find_bin_agent<NW, NB>(gh, krem, s_bin, s_below, s_count, sh);
  prefix |= *s_bin << shift;
  mask |= (uint32_t)(NB - 1) << shift;
  krem -= *s_below;
  __syncthreads();
  return true;
}

__device__ __forceinline__ uint64_t load_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A team member that stopped waiting for its team: the head's threshold key T
// and the number `need` of keys equal to T that are evicted, from every score
// of the head (three radix rounds over the keys in memory, histograms in LDS),
// and the counts of keys above T and equal to T in the tokens before this
// member.  Exactly what the team computes together, so the member's keep
// entries are the same either way.  Whole workgroup.
__device__ void select_alone(const SelArgs& a, int g, int b, uint32_t* h, uint32_t* sh,
                             uint32_t* s_bin, uint32_t* s_below, uint32_t& T, uint32_t& need,
                             uint32_t& gt_before, uint32_t& ties_before) {
  constexpr int NW = kFusedThreads / 64;
  const int tid = threadIdx.x;
  const float* sg = a.scores + (size_t)g * a.n;
  uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)(a.n - a.budget);
  for (int r = 0; r < 3; ++r) {
    const int shift = r == 0 ? 20 : (r == 1 ? 10 : 0);
    const int nb = r == 0 ? kBins1 : 1024;
    for (int i = tid; i < nb; i += kFusedThreads) h[i] = 0u;
    __syncthreads();
    for (int64_t j = tid; j < a.n; j += kFusedThreads) {
      const uint32_t k = order_key(sg[j]);
      if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    find_bin<NW>(h, nb, krem, s_bin, s_below, sh);
    prefix |= *s_bin << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem -= *s_below;
    __syncthreads();
  }
  T = prefix;
  need = krem;
  const int64_t before = min(a.n, (int64_t)b * kFusedBlock);
  uint32_t gt = 0u, nt = 0u;
  for (int64_t j = tid; j < before; j += kFusedThreads) {
    const uint32_t k = order_key(sg[j]);
    gt += k > T ? 1u : 0u;
    nt += k == T ? 1u : 0u;
  }
  uint32_t tg, tt;   // (a member's 16384 tokens fit 16 bits, a head's prefix may not)
  (void)block_exscan<NW>(gt, &tg, sh);
  (void)block_exscan<NW>(nt, &tt, sh);
  gt_before = tg;
  ties_before = tt;
}

// Slots past the end of the head hold key 0, below every key a float maps to
// (-inf maps to 0x007fffff): they rank first, the rank sought moves up by their
// number, and they are never kept.
__global__ __launch_bounds__(kFusedThreads) void select_fused(SelArgs a) {
  constexpr int NW = kFusedThreads / 64;
  __shared__ uint32_t h[kBins1];
  __shared__ uint32_t ck[kFusedCand];            // candidate keys of the threshold bin
  __shared__ uint16_t cw[kFusedCand];            // ... and the team member each came from
  __shared__ uint32_t gtc[kFusedThreads];        // per team member: keys above T
  __shared__ uint32_t tiec[kFusedThreads];       // per team member: keys equal to T
  __shared__ uint32_t sh[NW];
  __shared__ uint32_t s_bin, s_below, s_count, s_base;
  __shared__ int s_ok;
  // a latched device error withholds the keep list; the latch is read first and
  // tested once the keys have been requested, so the reads overlap
  const bool stop = latched(a.latch);
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  const uint32_t nblk = (uint32_t)a.nblk;
  const size_t heads = gridDim.x / nblk, cur = (size_t)a.sc.par * heads + g,
               oth = (size_t)(a.sc.par ^ 1) * heads + g;
  uint32_t* bar = a.sc.bar + cur;
  uint32_t* fh = a.sc.fh + cur * kFusedBins;
  uint32_t* fcnt = a.sc.fcnt + cur;
  uint32_t* blk_gt = a.sc.blk_above + (size_t)g * nblk;
  uint32_t* blk_tie = a.sc.blk_ties + (size_t)g * nblk;

  // A histogram the second pass built (a previous kernel: ordinary loads see it)
  // is requested first, to land with the keys; otherwise these words are unused.
  constexpr int HPER = kBins1 / kFusedThreads;
  static_assert(HPER % 4 == 0, "16-byte loads of the prebuilt histogram");
  uint32_t hpre[HPER];
#pragma unroll
  for (int q = 0; q < HPER / 4; ++q) {
    const uint4 x = *reinterpret_cast<const uint4*>(fh + HPER * tid + 4 * q);
    hpre[4 * q] = x.x; hpre[4 * q + 1] = x.y; hpre[4 * q + 2] = x.z; hpre[4 * q + 3] = x.w;
  }
  // taken as used at the end of both key branches below, so that the load is
  // issued ahead of them (not sunk to its first use, one round trip later)
  auto pin_hist = [&]() {
#pragma unroll
    for (int i = 0; i < HPER; ++i) asm volatile("" ::"v"(hpre[i]));
  };
  // this thread's kFusedPer consecutive tokens, as order keys
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)b * kFusedBlock + (int64_t)tid * kFusedPer;
  const int nv = (int)max((int64_t)0, min((int64_t)kFusedPer, a.n - base));
  uint32_t key[kFusedPer];
  if (nv == kFusedPer && (((size_t)g * a.n + base) & 3) == 0) {   // 16-byte aligned run
#pragma unroll
    for (int q = 0; q < kFusedPer / 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(sg + base + 4 * q);
      key[4 * q + 0] = order_key(x.x);
      key[4 * q + 1] = order_key(x.y);
      key[4 * q + 2] = order_key(x.z);
      key[4 * q + 3] = order_key(x.w);
    }
    pin_hist();
  } else {
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i) key[i] = i < nv ? order_key(sg[base + i]) : 0u;
    pin_hist();
  }
  const uint32_t pad = nblk * (uint32_t)kFusedBlock - (uint32_t)a.n;
  // The other parity's histograms and counters (the previous call's, which has
  // ended) are cleared for the next call, each member its share; this call's
  // are cleared by the next one, whatever way this one ends.
  {
    uint32_t* fo = a.sc.fh + oth * kFusedBins;
    const int per = (kFusedBins + (int)nblk - 1) / (int)nblk;
    const int lo = b * per, hi = min(kFusedBins, lo + per);
    for (int i = lo + tid; i < hi; i += kFusedThreads) fo[i] = 0u;
    if (b == 0 && tid == 0) {
      a.sc.bar[oth] = 0u;
      a.sc.fcnt[oth] = 0u;
    }
  }
  if (stop) return;   // nothing has been written

  // T is the k-th smallest key; `need` (>= 1) of the keys equal to T are
  // evicted; the members before b hold gt_before keys above T and ties_before
  // keys equal to T
  uint32_t T = 0u, need = 0u, gt_before = 0u, ties_before = 0u;
  bool alone = a.wait < 0;
  // round 1: the 12-bit bin b1 holding the k-th smallest key, and its size.
  // A histogram the second pass built counts the head's real keys only (no
  // padding slots), and needs no team barrier: it is complete when this
  // launch starts.  `bar0` is the barrier arrivals before the exchange.
  uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)(a.n - a.budget) + (a.pre1 ? 0u : pad);
  const uint32_t bar0 = a.pre1 ? 0u : nblk;
  if (!alone) {
    if (a.pre1) {
      find_bin_regs<NW, HPER>(hpre, krem, &s_bin, &s_below, &s_count, sh);
      prefix |= s_bin << 20;
      mask |= (uint32_t)(kBins1 - 1) << 20;
      krem -= s_below;
      __syncthreads();
    } else {
      alone = !radix_round<kBins1, true>(key, 20, h, fh, bar, nblk, a.wait, prefix, mask, krem, sh,
                                         &s_bin, &s_below, &s_count, &s_ok);
    }
  }
  if (!alone) {
    const uint32_t c1 = s_count;   // the same in every member: read from one histogram
    const uint32_t b1 = prefix >> 20;
    if (c1 <= (uint32_t)kFusedCand) {
      // Exchange the bin's keys (tagged with the member) and each member's count
      // of keys above the bin; then every member finishes alone.
      uint32_t mine = 0u, gt1 = 0u;
#pragma unroll
      for (int i = 0; i < kFusedPer; ++i) {
        const uint32_t bin = key[i] >> 20;
        mine += bin == b1 ? 1u : 0u;
        gt1 += bin > b1 ? 1u : 0u;
      }
      uint32_t tot;   // both counts are below 2^16 per member: scan them packed
      const uint32_t off = block_exscan<NW>(mine | (gt1 << 16), &tot, sh) & 0xffffu;
      if (tid == 0) {
        const uint32_t o = __hip_atomic_exchange(blk_gt + b, tot >> 16, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t mt = tot & 0xffffu;
        s_base = mt ? __hip_atomic_fetch_add(fcnt, mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0u;
        asm volatile("s_waitcnt vmcnt(0)" ::"v"(o) : "memory");
      }
      __syncthreads();
      uint64_t* cand = a.sc.fcand + (size_t)g * kFusedCand;
      uint32_t pos = s_base + off;
      // agent-scope stores (written through to the coherence point, unlike a
      // read-modify-write atomic per key, which would serialise at the memory
      // side); the teammates read them with agent-scope loads after the barrier
#pragma unroll
      for (int i = 0; i < kFusedPer; ++i)
        if ((key[i] >> 20) == b1) {
          if (pos < (uint32_t)kFusedCand)
            __hip_atomic_store(cand + pos, (uint64_t)key[i] | ((uint64_t)b << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          ++pos;
        }
      alone = !team_barrier(bar, bar0 + nblk, a.wait, &s_ok);
      if (!alone) {
        // every candidate and count load in flight at once (c1 <= kFusedCand)
        constexpr int CU = kFusedCand / kFusedThreads;
        uint64_t cv[CU];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const uint32_t i = (uint32_t)tid + (uint32_t)(u * kFusedThreads);
          cv[u] = i < c1 ? load_agent64(cand + i) : 0u;
        }
        const uint32_t gv = (uint32_t)tid < nblk ? load_agent(blk_gt + tid) : 0u;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const uint32_t i = (uint32_t)tid + (uint32_t)(u * kFusedThreads);
          if (i < c1) {
            ck[i] = (uint32_t)cv[u];
            cw[i] = (uint16_t)(cv[u] >> 32);
          }
        }
        if ((uint32_t)tid < nblk) {
          gtc[tid] = gv;
          tiec[tid] = 0u;
        }
        __syncthreads();
        // the exact k-th smallest key: two 10-bit digits below the bin, in LDS
        for (int shift = 10; shift >= 0; shift -= 10) {
          for (int i = tid; i < 1024; i += kFusedThreads) h[i] = 0u;
          __syncthreads();
          for (uint32_t i = tid; i < c1; i += kFusedThreads) {
            const uint32_t k = ck[i];
            if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & 1023u], 1u);
          }
          __syncthreads();
          find_bin<NW>(h, 1024, krem, &s_bin, &s_below, sh);
          prefix |= s_bin << shift;
          mask |= 1023u << shift;
          krem -= s_below;
          __syncthreads();
        }
        T = prefix;
        need = krem;
        for (uint32_t i = tid; i < c1; i += kFusedThreads) {
          const uint32_t k = ck[i];
          if (k > T) atomicAdd(&gtc[cw[i]], 1u);
          else if (k == T) atomicAdd(&tiec[cw[i]], 1u);
        }
        __syncthreads();
      }
    } else {
      // Too many keys share the bin: two more histogram rounds over the team,
      // then an exchange of each member's counts above and equal to T.
      bool ok = radix_round<1024, false>(key, 10, h, fh + kBins1, bar, bar0 + nblk, a.wait, prefix,
                                         mask, krem, sh, &s_bin, &s_below, &s_count, &s_ok);
      ok = ok && radix_round<1024, false>(key, 0, h, fh + kBins1 + 1024, bar, bar0 + 2 * nblk, a.wait,
                                          prefix, mask, krem, sh, &s_bin, &s_below, &s_count,
                                          &s_ok);
      if (ok) {
        T = prefix;
        need = krem;
        uint32_t gt = 0u, nt = 0u;
#pragma unroll
        for (int i = 0; i < kFusedPer; ++i) {
          gt += key[i] > T ? 1u : 0u;
          nt += key[i] == T ? 1u : 0u;
        }
        uint32_t tot;
        (void)block_exscan<NW>(gt | (nt << 16), &tot, sh);
        if (tid == 0) {
          const uint32_t o1 = __hip_atomic_exchange(blk_gt + b, tot & 0xffffu, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t o2 = __hip_atomic_exchange(blk_tie + b, tot >> 16, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          asm volatile("s_waitcnt vmcnt(0)" ::"v"(o1), "v"(o2) : "memory");
        }
        ok = team_barrier(bar, bar0 + 3 * nblk, a.wait, &s_ok);
        if (ok) {
          for (uint32_t i = tid; i < nblk; i += kFusedThreads) {
            gtc[i] = load_agent(blk_gt + i);
            tiec[i] = load_agent(blk_tie + i);
          }
          __syncthreads();
        }
      }
      alone = !ok;
    }
    if (!alone)
      for (int bb = 0; bb < b; ++bb) {
        gt_before += gtc[bb];
        ties_before += tiec[bb];
      }
  }
  if (alone)   // the teammates did not all arrive in time: the same answer alone
    select_alone(a, g, b, h, sh, &s_bin, &s_below, T, need, gt_before, ties_before);

  // Evicted ties are the oldest, so the members before b evict min(need, their
  // ties) of them and b evicts what remains of `need`, up to its own ties.
  uint32_t gt = 0u, nt = 0u;
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    gt += key[i] > T ? 1u : 0u;
    nt += key[i] == T ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_exscan<NW>(gt | (nt << 16), &tot, sh);
  const uint32_t ev_before = min(need, ties_before);
  const uint32_t ev = min(tot >> 16, need - ev_before);
  const uint32_t keep_before = gt_before + ties_before - ev_before;

  // ordered emission (thread order is index order within the member): the
  // threads before this one hold gt_pre keys above T and tie_pre ties, of which
  // the first `ev` of the member are evicted
  const uint32_t gt_pre = pre & 0xffffu, tie_pre = pre >> 16;
  uint32_t rank = tie_pre, keepbits = 0u;
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    const bool tie = key[i] == T;
    const bool keepit = key[i] > T || (tie && rank >= ev);
    rank += tie ? 1u : 0u;
    keepbits |= keepit ? 1u << i : 0u;
  }
  uint32_t pos = keep_before + gt_pre + (tie_pre > ev ? tie_pre - ev : 0u);
  int32_t* kg = a.keep + (size_t)g * a.budget;
  while (keepbits) {   // one store per kept token, in index order
    const int i = __builtin_ctz(keepbits);
    keepbits &= keepbits - 1u;
    if (pos < (uint32_t)a.budget) kg[pos] = (int32_t)(base + i);
    ++pos;
  }
}

// A head that fits one workgroup (n <= kFusedBlock): select_fused's steps for a
// team of one, with every histogram in LDS, so no device-scope traffic, no
// barrier beyond the workgroup's and no shared scratch (the fused kernel's
// counters are left as they are).
__global__ __launch_bounds__(kFusedThreads) void select_solo(SelArgs a) {
  constexpr int NW = kFusedThreads / 64;
  __shared__ uint32_t h[kBins1];
  __shared__ uint32_t sh[NW];
  __shared__ uint32_t s_bin, s_below;
  const bool stop = latched(a.latch);   // tested once the keys have been requested
  const int g = blockIdx.x, tid = threadIdx.x;

  // this thread's kFusedPer consecutive tokens, as order keys (0 past the end)
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)tid * kFusedPer;
  const int nv = (int)max((int64_t)0, min((int64_t)kFusedPer, a.n - base));
  uint32_t key[kFusedPer];
  if (nv == kFusedPer && (((size_t)g * a.n + base) & 3) == 0) {   // 16-byte aligned run
#pragma unroll
    for (int q = 0; q < kFusedPer / 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(sg + base + 4 * q);
      key[4 * q + 0] = order_key(x.x);
      key[4 * q + 1] = order_key(x.y);
      key[4 * q + 2] = order_key(x.z);
      key[4 * q + 3] = order_key(x.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i) key[i] = i < nv ? order_key(sg[base + i]) : 0u;
  }
  if (stop) return;   // nothing has been written yet

  // the k-th smallest key T, digits of 12, 10 and 10 bits; the slots past the
  // end hold key 0 and rank first, so the rank sought moves up by their number
  const uint32_t pad = (uint32_t)kFusedBlock - (uint32_t)a.n;
  uint32_t prefix = 0u, mask = 0u;
  uint32_t krem = (uint32_t)(a.n - a.budget) + pad;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int shift = r == 0 ? 20 : (r == 1 ? 10 : 0);
    const int nb = r == 0 ? kBins1 : 1024;
    for (int i = tid; i < nb; i += kFusedThreads) h[i] = 0u;
    __syncthreads();
    // the slots past the end count once, while the prefix still admits key 0;
    // real keys add once per run of one bin (pooling makes plateaus), so
    // neither piles same-address LDS atomics onto one bin
    if (tid == 0 && prefix == 0u && pad) atomicAdd(&h[0], pad);
    uint32_t run = 0u, rbin = 0u;
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i) {
      const uint32_t bin = (key[i] >> shift) & (uint32_t)(nb - 1);
      const bool in = i < nv && (key[i] & mask) == prefix;
      if (in && run && bin == rbin) {
        ++run;
      } else if (in) {
        if (run) atomicAdd(&h[rbin], run);
        rbin = bin;
        run = 1u;
      }
    }
    if (run) atomicAdd(&h[rbin], run);
    __syncthreads();
    find_bin<NW>(h, nb, krem, &s_bin, &s_below, sh);
    prefix |= s_bin << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem -= s_below;
    __syncthreads();
  }
  const uint32_t T = prefix, need = krem;   // need >= 1 of the keys equal to T are evicted

  // ordered emission (thread order is index order): the first `need` ties go
  uint32_t gt = 0u, nt = 0u;
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    gt += key[i] > T ? 1u : 0u;
    nt += key[i] == T ? 1u : 0u;
  }
  uint32_t tot;   // both counts are below 2^16 per head: scan them packed
  const uint32_t pre = block_exscan<NW>(gt | (nt << 16), &tot, sh);
  const uint32_t gt_pre = pre & 0xffffu, tie_pre = pre >> 16;
  uint32_t rank = tie_pre, keepbits = 0u;
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    const bool tie = key[i] == T;
    const bool keepit = key[i] > T || (tie && rank >= need);
    rank += tie ? 1u : 0u;
    keepbits |= keepit ? 1u << i : 0u;
  }
  uint32_t pos = gt_pre + (tie_pre > need ? tie_pre - need : 0u);
  int32_t* kg = a.keep + (size_t)g * a.budget;
  while (keepbits) {   // one store per kept token, in index order
    const int i = __builtin_ctz(keepbits);
    keepbits &= keepbits - 1u;
    if (pos < (uint32_t)a.budget) kg[pos] = (int32_t)(base + i);
    ++pos;
  }
}

__global__ __launch_bounds__(256) void select_all_kernel(int32_t* keep, int64_t n, int64_t total,
                                                         const uint32_t* latch) {
  if (latched(latch)) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    keep[i] = (int32_t)(i % n);
}

size_t select_scratch_bytes(int Hkv, int64_t n) {
  const int64_t nblk = (n + kSelBlock - 1) / kSelBlock;
  const size_t per_head = (size_t)kBins1 * 4 + 2 * (size_t)kFusedBins * 4 + (size_t)kCandCap * 8 +
                          (size_t)kFusedCand * 8 + 12 * 4 + (size_t)nblk * 5 * 4;
  return (size_t)Hkv * per_head + 64 * 256;
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

void carve_select(void* base, int Hkv, int64_t n, SelScratch* sc) {
  char* c = static_cast<char*>(base);
  const int64_t nblk = (n + kSelBlock - 1) / kSelBlock;
  auto take = [&](size_t bytes) { char* x = c; c += al256(bytes); return x; };
  sc->hist1 = (uint32_t*)take((size_t)Hkv * kBins1 * 4);
  sc->cand_cnt = (uint32_t*)take((size_t)Hkv * 4);
  sc->fh = (uint32_t*)take(2 * (size_t)Hkv * kFusedBins * 4);
  sc->bar = (uint32_t*)take(2 * (size_t)Hkv * 4);
  sc->fcnt = (uint32_t*)take(2 * (size_t)Hkv * 4);
  sc->fcand = (uint64_t*)take((size_t)Hkv * kFusedCand * 8);
  sc->cand_key = (uint32_t*)take((size_t)Hkv * kCandCap * 4);
  sc->cand_idx = (int32_t*)take((size_t)Hkv * kCandCap * 4);
  sc->b1 = (uint32_t*)take((size_t)Hkv * 4);
  sc->krem1 = (uint32_t*)take((size_t)Hkv * 4);
  sc->T = (uint32_t*)take((size_t)Hkv * 4);
  sc->blk_above = (uint32_t*)take((size_t)Hkv * nblk * 4);
  sc->blk_above_in = (uint32_t*)take((size_t)Hkv * nblk * 4);
  sc->blk_ties = (uint32_t*)take((size_t)Hkv * nblk * 4);
  sc->blk_off = (uint32_t*)take((size_t)Hkv * nblk * 4);
  sc->blk_evt = (uint32_t*)take((size_t)Hkv * nblk * 4);
}

// Bytes of select scratch that must start zeroed (hist1, cand_cnt and both
// parities of fh, bar and fcnt lead the carve).
size_t select_zero_prefix_bytes(int Hkv) {
  return al256((size_t)Hkv * kBins1 * 4) + al256((size_t)Hkv * 4) +
         al256(2 * (size_t)Hkv * kFusedBins * 4) + 2 * al256(2 * (size_t)Hkv * 4);
}

// Zero-fill of a scratch prefix (a multiple of 4 bytes), ordered on the caller's
// stream: a kernel rather than a null-stream memset, which streams created
// non-blocking do not wait for.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// Row copies, optionally non-temporal.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
  if constexpr (kNTCompactLd) return __builtin_nontemporal_load(p);
  return *p;
}
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 x) {
  if constexpr (kNTCompactSt) __builtin_nontemporal_store(x, p);
  else *p = x;
}

__global__ __launch_bounds__(256) void compact_kernel(const u16* __restrict__ k,
                                                      const u16* __restrict__ v, int64_t n, int d,
                                                      const int32_t* __restrict__ keep,
                                                      int64_t budget, int64_t rows,
                                                      u16* __restrict__ k_out,
                                                      u16* __restrict__ v_out, uint32_t* latch) {
  const int per_row = d / 8;
  const int64_t total = rows * per_row;
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int c = (int)(i - row * per_row);
    const int64_t g = row / budget;
    const int32_t j = keep[row];
    u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (j >= 0 && j < n) {
      const size_t src = ((size_t)g * n + j) * d + (size_t)c * 8;
      kx = ld_stream(reinterpret_cast<const u32x4*>(k + src));
      vx = ld_stream(reinterpret_cast<const u32x4*>(v + src));
    } else {
      bad = 1;
    }
    const size_t dst = (size_t)row * d + (size_t)c * 8;
    st_stream(reinterpret_cast<u32x4*>(k_out + dst), kx);
    st_stream(reinterpret_cast<u32x4*>(v_out + dst), vx);
  }
  if (bad) atomicOr(latch, LATCH_RANGE);
}

// ------------------------------------------------------- in-place compaction --
// Rows keep[g][0..budget) of a resident cache [Hkv][cap][d] move to rows
// 0..budget-1 of the same buffer.  keep is strictly ascending, so keep[j] >= j:
// every row moves toward the front or stays.  A plain parallel gather would
// race (row i may be written while another row still has to read it), so a
// workgroup owns one 16-byte column chunk of K or of V of one KV head, for all
// its rows, and walks the destinations in order, kIpRows at a time: every load
// of a batch completes before any of its stores issues (wait for the loads,
// then a barrier across the waves), and a later batch reads only rows at or
// past its own destinations, which lie past every row an earlier batch writes.
// Workgroups touch disjoint bytes, so no order between them is needed and none
// waits for another.  The eight chunks of one 128-byte line of a row go to
// workgroups whose indices agree modulo 8 -- the same XCD under the hardware's
// round-robin placement -- so that XCD's L2 serves all eight from one fetch of
// the line.  Before moving anything each workgroup checks its head's whole keep
// list (strictly ascending, inside [0, n_valid)); the workgroups of a head read
// the same list, so either all of them move or none does.
constexpr int kIpThreads = 1024;
constexpr int kIpU = 2;                          // rows per thread per batch
constexpr int kIpB = kIpThreads * kIpU;          // rows per batch
constexpr int kIpRows = 8192;                    // keep entries staged in LDS at a time
static_assert(kIpRows % kIpB == 0, "whole batches per staged block");

template <int N>
__device__ __forceinline__ void ip_wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(kIpThreads) void compact_inplace_kernel(u16* k, u16* v, int64_t hs, int d,
                                                                    int64_t n_valid,
                                                                    const int32_t* __restrict__ keep,
                                                                    int64_t budget, int Hkv,
                                                                    int nlines, int units8,
                                                                    uint32_t* latch) {
  __shared__ int32_t idx[kIpRows];
  const int tid = threadIdx.x;
  // blockIdx = sub * units8 + unit: unit = (head, K or V, 128-byte line), sub =
  // the 16-byte chunk within the line
  const int unit = blockIdx.x % units8, sub = blockIdx.x / units8;
  const int line = unit % nlines, kv = (unit / nlines) & 1, g = unit / (2 * nlines);
  const int col = 64 * line + 8 * sub;   // first of the 8 columns this workgroup moves
  if (g >= Hkv || col >= d) return;   // padding workgroups (whole workgroup: g and col are uniform)
  // an error latched by scoring or selection withholds the keep list: move
  // nothing (decided for the whole workgroup at once)
  if (__syncthreads_or(__atomic_load_n(latch, __ATOMIC_RELAXED) != 0u)) return;
  const int32_t* kp = keep + (size_t)g * budget;
  u16* base = (kv ? v : k) + (size_t)g * hs + col;
  // loads of one batch (rows b0 .. b0 + kIpB of the staged block).  Every lane
  // loads (past the block's end, row 0), so each call issues exactly kIpU load
  // instructions per wave -- the counter waits below rely on that count -- and
  // indices are clamped into [0, n_valid), so even an unchecked list reads in
  // bounds.
  auto load = [&](int b0, int ni, u32x4 (&x)[kIpU]) {
#pragma unroll
    for (int u = 0; u < kIpU; ++u) {
      const int i = b0 + u * kIpThreads + tid;
      int64_t j = i < ni ? (int64_t)idx[i] : 0;
      j = j < 0 ? 0 : (j >= n_valid ? n_valid - 1 : j);
      x[u] = *reinterpret_cast<const u32x4*>(base + (size_t)j * d);
    }
  };
  auto store = [&](int64_t i0, int b0, int ni, const u32x4 (&x)[kIpU]) {
#pragma unroll
    for (int u = 0; u < kIpU; ++u) {
      const int i = b0 + u * kIpThreads + tid;
      const int64_t dst = i0 + i;
      if (i < ni && (int64_t)idx[i] != dst)   // a row already in place is not rewritten
        *reinterpret_cast<u32x4*>(base + (size_t)dst * d) = x[u];
    }
  };
  // The whole list is checked before any row moves.  A list that fits one
  // staged block is checked in LDS while the first batch's loads fly (loads
  // only read; the check gates the stores); a longer one first in memory.
  const bool one_block = budget <= kIpRows;
  int bad = 0;
  if (!one_block) {
    for (int64_t j = tid; j < budget; j += kIpThreads) {
      const int32_t x = kp[j], prev = j > 0 ? kp[j - 1] : -1;
      if (x < 0 || (int64_t)x >= n_valid || x <= prev) bad = 1;
    }
    if (__syncthreads_or(bad)) {
      if (tid == 0) atomicOr(latch + 1, (uint32_t)LATCH_RANGE);
      return;
    }
  }
  for (int64_t i0 = 0; i0 < budget; i0 += kIpRows) {
    const int ni = (int)min((int64_t)kIpRows, budget - i0);
    __syncthreads();   // the previous block of entries is no longer read
    for (int i = tid; i < ni; i += kIpThreads) idx[i] = kp[i0 + i];
    __syncthreads();
    const int nb = (ni + kIpB - 1) / kIpB;
    u32x4 xa[kIpU], xb[kIpU];
    load(0, ni, xa);
    if (one_block) {
      for (int i = tid; i < ni; i += kIpThreads) {
        const int32_t x = idx[i], prev = i > 0 ? idx[i - 1] : -1;
        if (x < 0 || (int64_t)x >= n_valid || x <= prev) bad = 1;
      }
      if (__syncthreads_or(bad)) {
        if (tid == 0) atomicOr(latch + 1, (uint32_t)LATCH_RANGE);
        return;
      }
    }
    // batch b's stores issue once every wave's loads of batches <= b are done
    // (vmcnt(kIpU) right after batch b+1's kIpU loads: everything older --
    // batch b's loads, earlier stores -- has completed; then the barrier);
    // batch b+1's loads are issued before those stores (they read rows past
    // every row batch b writes), so the two overlap
    for (int b = 0; b < nb; b += 2) {
      if (b + 1 < nb) { load((b + 1) * kIpB, ni, xb); ip_wait_vmem<kIpU>(); }
      else ip_wait_vmem<0>();
      __syncthreads();
      store(i0, b * kIpB, ni, xa);
      if (b + 1 >= nb) break;
      if (b + 2 < nb) { load((b + 2) * kIpB, ni, xa); ip_wait_vmem<kIpU>(); }
      else ip_wait_vmem<0>();
      __syncthreads();
      store(i0, (b + 1) * kIpB, ni, xb);
    }
  }
}

// Workgroups of select_fused that can be resident at once on the current device
// (0 if the device cannot launch cooperatively).
static int64_t fused_capacity() {
  static int64_t cap[64];
  static bool known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!known[dev]) {
    int coop = 0, cus = 0, per_cu = 0;
    int64_t c = 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        coop &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, select_fused, kFusedThreads, 0) ==
            hipSuccess)
      c = (int64_t)cus * per_cu;
    cap[dev] = c;
    known[dev] = true;
  }
  return cap[dev];
}

bool select_prebuilt_applies(int Hkv, int64_t n, int64_t budget) {
  const int64_t team = (n + kFusedBlock - 1) / kFusedBlock;
  return budget > 0 && budget < n && team > 1 && team <= kFusedThreads &&
         (int64_t)Hkv * team <= fused_capacity();
}
int64_t fused_bins() { return kFusedBins; }

hipError_t launch_select(void* ctx, const float* scores, int Hkv, int64_t n, int64_t budget,
                         int32_t* keep, uint32_t* latch, const SelScratch& sc, int64_t wait,
                         hipStream_t s, uint32_t* epoch, bool pre1) {
  // this call's histograms (the prebuilt one included)
  uint32_t* fh_cur = sc.fh + (size_t)sc.par * Hkv * kFusedBins;
  if (pre1 && !select_prebuilt_applies(Hkv, n, budget)) {   // (callers ask first; kept safe)
    const hipError_t e = launch_zero(fh_cur, (size_t)Hkv * kFusedBins * 4, s);
    if (e != hipSuccess) return e;
    pre1 = false;
  }
  if (budget == n) {
    const int64_t total = (int64_t)Hkv * n;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    prof_begin(ctx, "select", s);
    hipLaunchKernelGGL(select_all_kernel, dim3((unsigned)blocks), dim3(256), 0, s, keep, n, total,
                       (const uint32_t*)latch);
    prof_end(ctx, "select", s);
    return hipGetLastError();
  }
  SelArgs a{};
  a.scores = scores; a.keep = keep; a.n = n; a.budget = budget;
  a.nblk = (int)((n + kSelBlock - 1) / kSelBlock);
  a.latch = latch;
  a.sc = sc;
  a.wait = wait;
  prof_begin(ctx, "select", s);
  const int64_t team = (n + kFusedBlock - 1) / kFusedBlock;
  if (team == 1) {   // one workgroup per head: no team, no co-residency needed
    hipLaunchKernelGGL(select_solo, dim3(Hkv), dim3(kFusedThreads), 0, s, a);
    prof_end(ctx, "select", s);
    return hipGetLastError();
  }
  if (team <= kFusedThreads && (int64_t)Hkv * team <= fused_capacity()) {
    SelArgs f = a;
    f.nblk = (int)team;
    f.pre1 = pre1 ? 1 : 0;
    void* args[] = {&f};
    const dim3 fgrid((unsigned)((int64_t)Hkv * team)), fblock(kFusedThreads);
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(select_fused), fgrid, fblock, args, 0, s);
    if (e == hipSuccess) {
      ++*epoch;   // the kernel clears the other parity for the next call
      prof_end(ctx, "select", s);
      return hipSuccess;
    }
    (void)hipGetLastError();   // did not fit after all: take the multi-launch path
  }
  if (pre1) {   // the prebuilt histogram is not used: leave this parity zeroed
    const hipError_t e = launch_zero(fh_cur, (size_t)Hkv * kFusedBins * 4, s);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)((int64_t)Hkv * a.nblk);
  hipLaunchKernelGGL(select_s1, dim3(grid), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_find1, dim3(Hkv), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_s2, dim3(grid), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_s3, dim3(Hkv), dim3(kS3Threads), 0, s, a);
  hipLaunchKernelGGL(select_s4, dim3(grid), dim3(kSelThreads), 0, s, a);
  prof_end(ctx, "select", s);
  return hipGetLastError();
}

// Per-head counts of a layer-wide keep list (flat indices g*n + j, ascending):
// head g owns the entries in [g*n, (g+1)*n).  One wave per head finds both
// ends by two 64-way searches run in lockstep (each round trip probes 64
// positions and narrows the range 64-fold) rather than binary searches of one
// dependent load per step.
__global__ __launch_bounds__(256) void layer_counts_kernel(const int32_t* keep, int64_t budget,
                                                           int64_t n, int Hkv, int32_t* counts,
                                                           const uint32_t* latch) {
  const bool stop = latched(latch);
  const int g = blockIdx.x * 4 + (int)(threadIdx.x >> 6);   // wave-uniform
  const int lane = threadIdx.x & 63;
  if (stop || g >= Hkv) return;
  // first index i with keep[i] >= x[s], for the two bounds s = 0, 1
  const int64_t x[2] = {(int64_t)g * n, (int64_t)(g + 1) * n};
  int64_t lo[2] = {0, 0}, hi[2] = {budget, budget};
  while (lo[0] < hi[0] || lo[1] < hi[1]) {
    bool p[2];
    int64_t step[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      step[k] = (hi[k] - lo[k] + 63) / 64;
      const int64_t idx = lo[k] + (int64_t)lane * step[k];
      p[k] = lo[k] < hi[k] && idx < hi[k] && keep[idx] < x[k];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (lo[k] >= hi[k]) continue;
      // the predicate holds on a prefix of the probes: lanes 0 .. c-1
      const int c = __popcll(__ballot(p[k]));
      if (c == 0) {
        hi[k] = lo[k];
      } else {
        const int64_t l0 = lo[k];
        lo[k] = l0 + (int64_t)(c - 1) * step[k] + 1;
        hi[k] = min(hi[k], l0 + (int64_t)c * step[k]);
      }
    }
  }
  if (lane == 0) counts[g] = (int32_t)(lo[1] - lo[0]);
}

hipError_t launch_layer_counts(void* ctx, const int32_t* keep, int64_t budget, int64_t n, int Hkv,
                               int32_t* counts, uint32_t* latch, hipStream_t s) {
  prof_begin(ctx, "select", s);
  hipLaunchKernelGGL(layer_counts_kernel, dim3((unsigned)((Hkv + 3) / 4)), dim3(256), 0, s,
                     keep, budget, n, Hkv, counts, (const uint32_t*)latch);
  prof_end(ctx, "select", s);
  return hipGetLastError();
}

hipError_t launch_compact_inplace(void* ctx, u16* k, u16* v, int Hkv, int64_t hs, int d,
                                  int64_t n_valid, const int32_t* keep, int64_t budget,
                                  uint32_t* latch, hipStream_t s) {
  if (budget == 0) return hipSuccess;
  const int nlines = (d + 63) / 64;                 // 128-byte lines of a row
  const int64_t units = (int64_t)Hkv * 2 * nlines;  // (head, K or V, line)
  const int64_t units8 = (units + 7) / 8 * 8;
  prof_begin(ctx, "compact_inplace", s);
  hipLaunchKernelGGL(compact_inplace_kernel, dim3((unsigned)(8 * units8)), dim3(kIpThreads), 0, s, k,
                     v, hs, d, n_valid, keep, budget, Hkv, nlines, (int)units8, latch);
  prof_end(ctx, "compact_inplace", s);
  return hipGetLastError();
}

hipError_t launch_compact(void* ctx, const u16* k, const u16* v, int Hkv, int64_t n, int d,
                          const int32_t* keep, int64_t budget, u16* k_out, u16* v_out,
                          uint32_t* latch, hipStream_t s) {
  const int64_t rows = (int64_t)Hkv * budget;
  if (rows == 0) return hipSuccess;
  const int64_t total = rows * (d / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  prof_begin(ctx, "compact", s);
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, s, k, v, n, d, keep,
                     budget, rows, k_out, v_out, latch);
  prof_end(ctx, "compact", s);
  return hipGetLastError();
}

}  // namespace dropkv
