// Internal declarations shared by libdropkv's translation units (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dropkv {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------ wave-level DPP helpers --
// Inclusive scan / reduction over the 64 lanes of a wave with DPP moves: row
// shifts combine within each row of 16 lanes, then two row broadcasts carry
// row totals forward (lane 15 into row 1 and row 3, lane 31 into rows 2 and 3).
// Lanes whose source is out of range take `ident`, the operation's identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t x, uint32_t ident, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}

// Inclusive prefix sum of a uint over the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  return wave_incl_u32(x, 0u, [](uint32_t p, uint32_t q) { return p + q; });
}

// Sum of a float over the wave, in every lane (fixed combination order).
__device__ __forceinline__ float wave_sum_dpp(float x) {
  const uint32_t r = wave_incl_u32(__float_as_uint(x), 0u, [](uint32_t p, uint32_t q) {
    return __float_as_uint(__uint_as_float(p) + __uint_as_float(q));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}

// Bitwise OR of a uint over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_or_dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_incl_u32(x, 0u, [](uint32_t p, uint32_t q) { return p | q; }), 63);
}

template <int CTRL, int RMASK>
__device__ __forceinline__ uint64_t max_u64_dpp_step(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, RMASK, 0xf, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, RMASK, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return v > o ? v : o;
}

// Maximum of a uint64 over the wave, in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max_u64_dpp_step<0x111, 0xf>(x);
  x = max_u64_dpp_step<0x112, 0xf>(x);
  x = max_u64_dpp_step<0x114, 0xf>(x);
  x = max_u64_dpp_step<0x118, 0xf>(x);
  x = max_u64_dpp_step<0x142, 0xa>(x);
  x = max_u64_dpp_step<0x143, 0xc>(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Device error latch bits (OR-ed by kernels, decoded by dropkv_sync in the
// order NONFINITE, INPUT_RANGE, SINGULAR, then RANGE / OVERFLOW).
enum : uint32_t {
  LATCH_NONFINITE = 1u,     // an input element is not finite (the first pass's scan)
  LATCH_SINGULAR = 2u,
  LATCH_RANGE = 4u,         // a keep index out of range, or a score beyond FLT_MAX
  LATCH_INPUT_RANGE = 8u,   // an input element of magnitude >= 2^48 (the first pass's scan)
  LATCH_OVERFLOW = 16u,     // an fp32 intermediate overflowed (only outside the input contract)
};
// Input contract: every Q, K and V element is finite and of magnitude below
// 2^48, i.e. its bf16 bits with the sign cleared are below this.  Then no
// logit (|q.k| <= d 2^96), no ||a||^2, ||v||^2, a.v or distance (<= 4 d 2^96)
// and no score (odds^2 <= 1 off the arg-max, whose term is formed exactly)
// comes near FLT_MAX.
constexpr uint32_t kInputRangeBits = 0x5780u;   // 2^48 in bf16

// Polls a workgroup of the single-launch selection makes at a team barrier
// before it finishes its share alone (about 10-20 ms on MI355X).
constexpr int64_t kSelectWait = 16384;

constexpr int kRows = 32;        // window-query rows of one row group (one MFMA tile)
constexpr int kMaxRowGroups = 4; // G*w <= 128 rows per KV head
constexpr int kTile = 32;        // tokens per MFMA tile
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
// Launch shape of the two K/V passes (d <= 128): waves per SIMD the register
// budget is cut for, and whether a wave starts its next tile's loads before
// finishing the current tile (tuning knobs; the defaults are the measured best).
#ifndef DROPKV_P1_WAVES
#define DROPKV_P1_WAVES 2
#endif
#ifndef DROPKV_P2_WAVES
#define DROPKV_P2_WAVES 2
#endif
#ifndef DROPKV_P1_OVERLAP
#define DROPKV_P1_OVERLAP 0
#endif
#ifndef DROPKV_P2_OVERLAP
#define DROPKV_P2_OVERLAP 0
#endif
#ifndef DROPKV_ATTN_TILES
#define DROPKV_ATTN_TILES 1
#endif
constexpr int kAttnTiles = DROPKV_ATTN_TILES;   // K tiles loaded per iteration (attention-only mode)
// Non-temporal loads/stores per site (bit mask).  On MI355X a 1 GiB streaming
// read whose every load instruction covers whole 128-byte lines reaches
// ~6.9 TB/s with non-temporal loads against ~6.1 TB/s with ordinary ones; loads
// that cover a line in several instructions (the K/V tiles in MFMA operand
// layout) run far slower non-temporal, since the line is not kept between them.
// Bits: 1 pass-1 V tile (whole rows per 16 lanes) and pass-2 V rows, 2 K/V
// tiles in MFMA operand layout, 4 compaction loads, 8 compaction stores, 16
// the streaming-read reference, 32 pass-2 K rows ORDINARY (their lines then
// stay in the Infinity Cache, where the compaction that follows finds the
// kept rows: ~1 us faster at the headline size, pass 2 unchanged).
#ifndef DROPKV_NT
#define DROPKV_NT 57
#endif
constexpr bool kNTV1 = (DROPKV_NT & 1) != 0;
constexpr bool kNTMfma = (DROPKV_NT & 2) != 0;
constexpr bool kNTCompactLd = (DROPKV_NT & 4) != 0;
constexpr bool kNTCompactSt = (DROPKV_NT & 8) != 0;
constexpr bool kNTStream = (DROPKV_NT & 16) != 0;
constexpr bool kNTP2K = (DROPKV_NT & 32) == 0;
#ifndef DROPKV_P2_VLDS
#define DROPKV_P2_VLDS 2
#endif
// pass 2: V tile (1) or K and V tiles (2) through LDS (whole-line loads)
constexpr bool kP2VLds = DROPKV_P2_VLDS != 0;
constexpr bool kP2KLds = DROPKV_P2_VLDS >= 2;
#ifndef DROPKV_P1_XCDSWZ
#define DROPKV_P1_XCDSWZ 1
#endif
constexpr bool kP1XcdSwz = DROPKV_P1_XCDSWZ != 0;   // pass 1: XCD-aware split deal
#ifndef DROPKV_P1_WG_WAVES
#define DROPKV_P1_WG_WAVES 4
#endif
constexpr int kP1Waves = DROPKV_P1_WAVES;
constexpr int kP2Waves = DROPKV_P2_WAVES;
// pass 1 prefetch of the next tile: 1 K and V, 2 V only, 3 K only
constexpr bool kP1PreK = DROPKV_P1_OVERLAP == 1 || DROPKV_P1_OVERLAP == 3;
constexpr bool kP1PreV = DROPKV_P1_OVERLAP == 1 || DROPKV_P1_OVERLAP == 2;
constexpr bool kP2Overlap = DROPKV_P2_OVERLAP != 0;
#ifndef DROPKV_P1_GRANULE
#define DROPKV_P1_GRANULE 1
#endif
constexpr int kP1Granule = DROPKV_P1_GRANULE;   // first-pass split interleave granule (tiles; 0 = contiguous)
constexpr int kChunk2 = 2048;                // most tokens per pass-2 workgroup (before the pooling halo)
// Pass 1 runs kP1WgWaves waves per workgroup: four by default, two
// workgroups per CU at two waves per SIMD (4 * kP1Waves = 8 makes one
// workgroup fill the CU; measured no faster).  Head dimensions above 128 need
// more than 256 VGPRs, one wave per SIMD: their workgroups keep four waves.
constexpr int kP1WgWaves = DROPKV_P1_WG_WAVES;
constexpr int p1_waves(int DP) { return DP <= 128 ? kP1WgWaves : 4; }
#ifndef DROPKV_P1_SPLIT_MULT
#define DROPKV_P1_SPLIT_MULT 1
#endif
constexpr int kTargetWG1 =   // pass-1 workgroups aimed for
    DROPKV_P1_SPLIT_MULT * 256 * 4 * kP1Waves / kP1WgWaves;
#ifndef DROPKV_P2_TARGET
#define DROPKV_P2_TARGET (256 * DROPKV_P2_WAVES)
#endif
constexpr int kTargetWG2 = DROPKV_P2_TARGET;   // pass-2 workgroups aimed for over all heads

// A first-pass split whose S_excl is below this (its arg-max holds more than
// ~0.94 of its mass) is flagged; a row whose winning split is flagged takes
// its arg-max term and a - v_j* from the exact sum without the arg-max, which
// the merge's helper workgroups recompute over that split's tokens.
constexpr float kFixupThreshold = 0.0625f;
constexpr int kMaxHelpers = 8;    // merge helper workgroups per (KV head, row group)

// Pass 2 takes ||a - v||^2 from the expansion ||a||^2 - 2 a.v + ||v||^2 unless
// that value is below this fraction of ||a||^2 + ||v||^2: there the expansion's
// rounding (a split into two bf16 parts, fp32 sums: about 3e-5 of ||a||^2 +
// ||v||^2 at worst) could exceed 1e-3 of the result, and the distance is summed
// directly instead, as ||(a - v_j*) + (v_j* - v)||^2.
constexpr float kCancelFrac = 0.0625f;

// Per-row (window query) state produced by the merge, consumed by pass 2.
struct RowState {
  float* m2;      // [Hkv][32] running max of the logits, log2 units
  float* lse2;    // [Hkv][32] log2 of the softmax normaliser
  float* S;       // [Hkv][32] normaliser in units of the max
  float* an2;     // [Hkv][32] ||a||^2
  float* cstar;   // [Hkv][32] arg-max token's contribution ||Delta_j*||^2
  int* jstar;     // [Hkv][32] arg-max token index (lowest on ties)
  int* fix;       // [Hkv][32] 1 if the arg-max term needs the exclusion kernel
  u16* a_hi;      // [Hkv][32][DP] bf16 high part of a
  u16* a_lo;      // [Hkv][32][DP] bf16 remainder a - a_hi
  float* ares;    // [Hkv][32][DP] a - v_j* in fp32: from the exact exclusion sum for
                  // rows whose arg-max holds p* > ~0.94, else from a (zero past d)
};

struct Partials {
  float* m2;      // [Hkv][splits][32]
  float* S;       // [Hkv][splits][32]
  float* Sx;      // [Hkv][splits][32]
  int* jstar;     // [Hkv][splits][32]
  int* bad;       // [Hkv][splits][32]
  float* a;       // [Hkv][splits][32][DP] un-normalised output
};

// Scratch of the exact exclusion sums (see the merge): per virtual head, each
// helper's partial sums over its share of the winning split's tokens, the row
// workgroup's sum over the other splits, and per-row arrival counters (zero
// between calls: the last arrival resets them).
struct ExclScratch {
  float* part;     // [Hv][xh][32][DP]  helper h: sum of e_j v_j over its tokens, j != j*
  float* sx;       // [Hv][xh][32]      helper h: sum of e_j over the same tokens
  float* ao;       // [Hv][32][DP]      sum over the other splits of f_s a_s
  float* meta;     // [Hv][32][4]       S, S_excl, S over the other splits, j* (bits)
  uint32_t* cnt;   // [Hv][32]          arrivals (xh helpers + the row's workgroup)
  uint32_t* head;  // [Hv]              some split of the virtual head is flagged (set by
                   //                   the first pass, cleared by the second)
};

struct ScoreArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  float* scores;
  int64_t n;
  int64_t hs;           // elements from one KV head's K (and V) rows to the next: n * d, or cap * d
                        // for a resident cache of capacity cap
  int w, Hq, Hkv, d, G, M, pool, DP;
  int R;                // 32-row groups per KV head: ceil(M / 32), at most kMaxRowGroups
  int splits;
  int64_t split_len;
  int chunks2;          // pass-2 workgroups per head
  int64_t chunk2_len;   // tokens per pass-2 workgroup (multiple of the tile, <= kChunk2)
  float scale_log2;   // log2(e) / sqrt(d)
  Partials part;
  RowState rs;
  uint32_t* latch;
  float* out_a;     // optional [Hq][w][d] fp32: each window query's attention output
  float* out_lse;   // optional [Hq][w]: natural-log log-sum-exp of its visible logits
  int xh;           // merge helper workgroups per virtual head
  ExclScratch ex;
  // With the score + select entry point: the selection's first-digit histogram
  // of every head's final scores (12-bit digit key >> 20, kBins1 entries per
  // head at stride hist1_stride), added to by the second pass; nullptr: none.
  uint32_t* hist1;
  int64_t hist1_stride;
};

constexpr int kBins1 = 4096;   // the selection's first radix digit: the key's top 12 bits

// Floats -> uint32 keys whose unsigned order is the float order; -0 == +0;
// every NaN maps above +inf.  The selection ranks scores by these keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scratch of the selection kernels (owned by the context; hist1 and cand_cnt
// must be zero between calls -- the last selection kernel leaves them zeroed).
struct SelScratch {
  uint32_t* hist1;         // [Hkv][4096]
  uint32_t* cand_cnt;      // [Hkv]
  // The single-launch path's histograms and counters come in two sets, used by
  // calls of alternating parity: each call clears the other set (the previous
  // call's) for the next one, so no workgroup has to learn that it finished last.
  uint32_t* fh;            // [2][Hkv][4096 + 1024 + 1024] histograms of the single-launch path
  uint32_t* bar;           // [2][Hkv] arrival counters of the single-launch path
  uint32_t* fcnt;          // [2][Hkv] threshold-bin candidate counters of the single-launch path
  int par;                 // parity of the next single-launch call (0 or 1)
  uint64_t* fcand;         // [Hkv][8192] (key, member) candidates of the single-launch path
  uint32_t* cand_key;      // [Hkv][8192]
  int32_t* cand_idx;       // [Hkv][8192]
  uint32_t* b1;            // [Hkv]
  uint32_t* krem1;         // [Hkv]
  uint32_t* T;             // [Hkv]
  uint32_t* blk_above;     // [Hkv][nblk]
  uint32_t* blk_above_in;  // [Hkv][nblk]
  uint32_t* blk_ties;      // [Hkv][nblk]
  uint32_t* blk_off;       // [Hkv][nblk]
  uint32_t* blk_evt;       // [Hkv][nblk]
};
size_t select_scratch_bytes(int Hkv, int64_t n);
void carve_select(void* base, int Hkv, int64_t n, SelScratch* sc);
size_t select_zero_prefix_bytes(int Hkv);
// Zeroes `bytes` (a multiple of 4) at device address p, ordered on stream s.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Profiling hooks implemented by the host library (no-ops unless enabled).
struct ProfScope;
void prof_begin(void* ctx, const char* name, hipStream_t s);
void prof_end(void* ctx, const char* name, hipStream_t s);

hipError_t launch_score(void* ctx, const ScoreArgs& a, hipStream_t s);
// pre1: the second pass has built the first-digit histogram into sc.fh (only
// when select_prebuilt_applies said so)
// `epoch` counts the single-launch calls on this scratch (advanced after each);
// sc.par must be its parity.
hipError_t launch_select(void* ctx, const float* scores, int Hkv, int64_t n, int64_t budget,
                         int32_t* keep, uint32_t* latch, const SelScratch& sc, int64_t wait,
                         hipStream_t s, uint32_t* epoch, bool pre1 = false);
// Whether selection of these sizes runs the single-launch team path, which can
// start from a histogram the second pass built (sc.fh, stride fused_bins()).
bool select_prebuilt_applies(int Hkv, int64_t n, int64_t budget);
int64_t fused_bins();
// Whether the second pass has LDS for its chunk's histogram (head dim / row groups).
bool score_hist_fits(int DP, int R);
hipError_t launch_layer_counts(void* ctx, const int32_t* keep, int64_t budget, int64_t n, int Hkv,
                               int32_t* counts, uint32_t* latch, hipStream_t s);
// In place: rows keep[g][0..budget) of the [Hkv][hs / d][d] K and V caches move to
// rows 0..budget-1 (keep strictly ascending inside [0, n_valid), checked on the
// device; a head whose list fails is left untouched and LATCH_RANGE goes to
// latch word 1).
hipError_t launch_compact_inplace(void* ctx, u16* k, u16* v, int Hkv, int64_t hs, int d,
                                  int64_t n_valid, const int32_t* keep, int64_t budget,
                                  uint32_t* latch, hipStream_t s);
hipError_t launch_compact(void* ctx, const u16* k, const u16* v, int Hkv, int64_t n, int d,
                          const int32_t* keep, int64_t budget, u16* k_out, u16* v_out,
                          uint32_t* latch, hipStream_t s);

// Bytes of scratch the scoring pass needs for these sizes (Hkv counts virtual
// heads: KV heads times row groups; xh merge helpers per virtual head).
size_t score_scratch_bytes(int Hkv, int splits, int DP, int xh);
void carve_scratch(void* base, int Hkv, int splits, int DP, int xh, Partials* p, RowState* rs,
                   ExclScratch* ex);
// Merge helpers per virtual head: enough to cut the winning split's tokens into
// pieces of about eight tiles, at most kMaxHelpers and about 1024 over the call.
int plan_helpers(int64_t n, int Hv, int splits);
int plan_splits(int64_t n, int Hkv, int64_t* split_len, int target = kTargetWG1);
hipError_t launch_score_attention(void* ctx, const ScoreArgs& a, hipStream_t s);
bool score_fits(int DP, int R);
// sink: device memory of at least 8 words, written only in the
// practically impossible case that the buffer's XOR equals a fixed constant
hipError_t launch_stream_read(void* ctx, const void* p, int64_t bytes, uint32_t* sink,
                              hipStream_t s);
constexpr int kAttnWaves = kAttnTiles > 1 ? 3 : 4;   // attention-only passes: waves per SIMD (d <= 128)
// attention-only pass A: 512 workgroups (64 splits per head at 8 heads) beat
// one per wave slot (1024): pass B then merges half the split states per row
#ifndef DROPKV_ATTN_A_TARGET
#define DROPKV_ATTN_A_TARGET 512
#endif
constexpr int kTargetWGAttn = DROPKV_ATTN_A_TARGET;
#ifndef DROPKV_ATTN_B_TARGET
#define DROPKV_ATTN_B_TARGET 512
#endif
constexpr int kTargetWGAttnB = DROPKV_ATTN_B_TARGET;   // attention-only pass B: two chunks of up to 2048 tokens per CU
int plan_chunks2(int64_t n, int Hkv, int64_t* chunk_len, int target = kTargetWG2);

}  // namespace dropkv
