// Eviction selection and cache compaction for gfx950.
//
// Selection (DropKV implementation notes, "Algorithm 1": the smallest scores are
// evicted): per KV head, evict the k = n - budget smallest scores by the total
// order (score, index) and list the survivors in ascending index order.  Scores
// map to order-preserving 32-bit keys; an exact MSB-first radix select (four
// 8-bit digits, LDS histograms) finds the k-th smallest key T and how many of
// the keys equal to T must go; one ordered pass with block-wide scans then
// emits the survivors.  Integer work only, so the result is exact.
//
// Compaction (Section 2.2: eviction removes tokens from the resident cache):
// 16-byte row-chunk gathers k_out[g][r] = k[g][keep[g][r]], v likewise.
#include <float.h>

#include "common.h"

namespace dropkv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Floats -> uint32 keys whose unsigned order is the float order; -0 == +0;
// every NaN maps above +inf.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one uint per thread across the block; also returns the total.
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
    uint32_t t = (lane < kSelWaves) ? sh[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      const uint32_t y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    if (lane < kSelWaves) sh[kSelWaves + lane] = ti - t;  // exclusive wave offsets
    if (lane == kSelWaves - 1) sh[2 * kSelWaves] = ti;
  }
  __syncthreads();
  const uint32_t res = sh[kSelWaves + wid] + incl - x;
  *total = sh[2 * kSelWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             int64_t n, int64_t budget,
                                                             int32_t* __restrict__ keep,
                                                             const uint32_t* latch) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2 * kSelWaves + 1];
  __shared__ uint32_t s_bin, s_below;
  if (__atomic_load_n(latch, __ATOMIC_RELAXED) != 0u) return;  // a latched error: no keep list
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = blockIdx.x;
  const float* sg = scores + (size_t)g * n;
  int32_t* kg = keep + (size_t)g * budget;
  const int64_t kev = n - budget;
  if (budget == 0) return;
  if (kev == 0) {
    for (int64_t j = tid; j < n; j += kSelThreads) kg[j] = (int32_t)j;
    return;
  }
  // ---- exact k-th smallest key, MSB-first, 8 bits per pass ----
  uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)kev;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t j = tid; j < n; j += kSelThreads) {
      const uint32_t key = order_key(sg[j]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      // lane owns bins 4*lane .. 4*lane+3
      uint32_t h[4], loc = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) { h[i] = hist[4 * lane + i]; loc += h[i]; }
      uint32_t incl = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const uint32_t excl = incl - loc;
      const bool mine = excl < krem && incl >= krem;
      if (mine) {
        uint32_t c = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (c + h[i] >= krem) { s_bin = 4 * lane + i; s_below = c; break; }
          c += h[i];
        }
      }
    }
    __syncthreads();
    prefix |= s_bin << shift;
    mask |= 255u << shift;
    krem -= s_below;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need = krem;  // keys equal to T that are evicted (the oldest ones)

  // ---- ordered emission: 4 consecutive tokens per thread per round ----
  uint32_t tie_base = 0u, keep_base = 0u;
  for (int64_t base = 0; base < n; base += 4 * kSelThreads) {
    uint32_t eqc = 0u, eqbits = 0u, lessbits = 0u, okbits = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t j = base + 4 * tid + e;
      if (j < n) {
        const uint32_t key = order_key(sg[j]);
        okbits |= 1u << e;
        if (key == T) { eqbits |= 1u << e; ++eqc; }
        if (key < T) lessbits |= 1u << e;
      }
    }
    uint32_t eq_total;
    const uint32_t eq_before = block_exscan(eqc, &eq_total, sh);
    uint32_t rank = tie_base + eq_before, kc = 0u, keepbits = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!((okbits >> e) & 1u)) continue;
      bool evict = (lessbits >> e) & 1u;
      if ((eqbits >> e) & 1u) { evict = rank < need; ++rank; }
      if (!evict) { keepbits |= 1u << e; ++kc; }
    }
    uint32_t keep_total;
    uint32_t pos = keep_base + block_exscan(kc, &keep_total, sh);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((keepbits >> e) & 1u) {
        if (pos < (uint32_t)budget) kg[pos] = (int32_t)(base + 4 * tid + e);
        ++pos;
      }
    tie_base += eq_total;
    keep_base += keep_total;
  }
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
                         int32_t* keep, uint32_t* latch, hipStream_t s) {
  prof_begin(ctx, "select", s);
  hipLaunchKernelGGL(select_kernel, dim3(Hkv), dim3(kSelThreads), 0, s, scores, n, budget, keep,
                     (const uint32_t*)latch);
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
