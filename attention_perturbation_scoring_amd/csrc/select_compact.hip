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

// Selection runs as four wide kernels over blocks of kSelBlock consecutive
// tokens of one head (all integer arithmetic, so the result is exact):
//   s1  12-bit histogram of the keys' top bits (per-block LDS, then global adds)
//   s2  find the bin b1 holding the k-th smallest key; count keys above b1 per
//       block and collect the keys of bin b1 (with their indices) as candidates
//   s3  per head: the exact k-th smallest key T from the candidates (two more
//       10-bit digits), how many keys equal to T are evicted, and each block's
//       output offset and number of evicted ties
//   s4  ordered emission of the survivors, and clean-up of the shared scratch
constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kSelBlock = kSelThreads * kSelPer;   // 4096 tokens per block
constexpr int kBins1 = 4096;
constexpr int kCandCap = 8192;
constexpr int kS3Threads = 1024;

// Floats -> uint32 keys whose unsigned order is the float order; -0 == +0;
// every NaN maps above +inf.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block scan of one uint per thread (NW waves); returns the total too.
template <int NW>
__device__ __forceinline__ uint32_t block_exscan(uint32_t x, uint32_t* total, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const uint32_t t = (lane < NW) ? sh[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const uint32_t y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    if (lane < NW) sh[NW + lane] = ti - t;
    if (lane == NW - 1) sh[2 * NW] = ti;
  }
  __syncthreads();
  const uint32_t res = sh[NW + wid] + incl - x;
  *total = sh[2 * NW];
  __syncthreads();
  return res;
}

struct SelArgs {
  const float* scores;
  int32_t* keep;
  int64_t n, budget;
  int nblk;                 // blocks of kSelBlock tokens per head
  const uint32_t* latch;
  SelScratch sc;
};

__device__ __forceinline__ bool latched(const uint32_t* latch) {
  return __atomic_load_n(latch, __ATOMIC_RELAXED) != 0u;
}

__global__ __launch_bounds__(kSelThreads) void select_s1(SelArgs a) {
  __shared__ uint32_t h[kBins1];
  if (latched(a.latch)) return;
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins1; i += kSelThreads) h[i] = 0u;
  __syncthreads();
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)b * kSelBlock;
  const bool full = base + kSelBlock <= a.n;
  float x[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    x[i] = (j < a.n) ? sg[j] : 0.f;
  }
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

__global__ __launch_bounds__(kSelThreads) void select_s2(SelArgs a) {
  __shared__ uint32_t sh[2 * (kSelThreads / 64) + 1];
  __shared__ uint32_t s_bin, s_below, s_cnt, s_base;
  __shared__ uint32_t lk[kSelBlock];
  __shared__ int32_t li[kSelBlock];
  if (latched(a.latch)) return;
  const int g = blockIdx.x / a.nblk, b = blockIdx.x % a.nblk;
  const int tid = threadIdx.x;
  const uint32_t kev = (uint32_t)(a.n - a.budget);
  find_bin<kSelThreads / 64>(a.sc.hist1 + (size_t)g * kBins1, kBins1, kev, &s_bin, &s_below, sh);
  const uint32_t b1 = s_bin;
  if (tid == 0) {
    s_cnt = 0u;
    if (b == 0) { a.sc.b1[g] = b1; a.sc.krem1[g] = kev - s_below; }
  }
  __syncthreads();
  const float* sg = a.scores + (size_t)g * a.n;
  const int64_t base = (int64_t)b * kSelBlock;
  uint32_t above = 0u;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int64_t j = base + i * kSelThreads + tid;
    if (j < a.n) {
      const uint32_t key = order_key(sg[j]);
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
  const bool skip = latched(a.latch);
  if (!skip) {
    const uint32_t T = a.sc.T[g];
    const uint32_t off = a.sc.blk_off[(size_t)g * a.nblk + b];
    const uint32_t ev = a.sc.blk_evt[(size_t)g * a.nblk + b];
    const float* sg = a.scores + (size_t)g * a.n;
    int32_t* kg = a.keep + (size_t)g * a.budget;
    // thread owns kSelPer consecutive tokens so that index order = (thread, i)
    const int64_t base = (int64_t)b * kSelBlock + (int64_t)tid * kSelPer;
    uint32_t keys[kSelPer];
    uint32_t nt = 0u;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int64_t j = base + i;
      keys[i] = (j < a.n) ? order_key(sg[j]) : 0u;
      if (j < a.n && keys[i] == T) ++nt;
    }
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

__global__ __launch_bounds__(256) void select_all_kernel(int32_t* keep, int64_t n, int64_t total,
                                                         const uint32_t* latch) {
  if (latched(latch)) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    keep[i] = (int32_t)(i % n);
}

size_t select_scratch_bytes(int Hkv, int64_t n) {
  const int64_t nblk = (n + kSelBlock - 1) / kSelBlock;
  const size_t per_head = (size_t)kBins1 * 4 + (size_t)kCandCap * 8 + 5 * 4 * 4 + (size_t)nblk * 5 * 4;
  return (size_t)Hkv * per_head + 64 * 256;
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

void carve_select(void* base, int Hkv, int64_t n, SelScratch* sc) {
  char* c = static_cast<char*>(base);
  const int64_t nblk = (n + kSelBlock - 1) / kSelBlock;
  auto take = [&](size_t bytes) { char* x = c; c += al256(bytes); return x; };
  sc->hist1 = (uint32_t*)take((size_t)Hkv * kBins1 * 4);
  sc->cand_cnt = (uint32_t*)take((size_t)Hkv * 4);
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

// Bytes of select scratch that must start zeroed (hist1 and cand_cnt lead the carve).
size_t select_zero_prefix_bytes(int Hkv) {
  return al256((size_t)Hkv * kBins1 * 4) + al256((size_t)Hkv * 4);
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
      kx = *reinterpret_cast<const u32x4*>(k + src);
      vx = *reinterpret_cast<const u32x4*>(v + src);
    } else {
      bad = 1;
    }
    const size_t dst = (size_t)row * d + (size_t)c * 8;
    *reinterpret_cast<u32x4*>(k_out + dst) = kx;
    *reinterpret_cast<u32x4*>(v_out + dst) = vx;
  }
  if (bad) atomicOr(latch, LATCH_RANGE);
}

hipError_t launch_select(void* ctx, const float* scores, int Hkv, int64_t n, int64_t budget,
                         int32_t* keep, uint32_t* latch, const SelScratch& sc, hipStream_t s) {
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
  const unsigned grid = (unsigned)((int64_t)Hkv * a.nblk);
  prof_begin(ctx, "select", s);
  hipLaunchKernelGGL(select_s1, dim3(grid), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_s2, dim3(grid), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_s3, dim3(Hkv), dim3(kS3Threads), 0, s, a);
  hipLaunchKernelGGL(select_s4, dim3(grid), dim3(kSelThreads), 0, s, a);
  prof_end(ctx, "select", s);
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
