// DropKV scoring kernels for gfx950 (MI355X, CDNA4).
//
// What is computed (DropKV, arXiv 2610.22130: Section 3.1 / Appendix C.2 for the
// single-token perturbation Delta_j = p_j/(1-p_j) (a - v_j); Section 3.3 and the
// implementation notes' "Core equation" for the window sum of ||Delta_j||^2; the
// notes' "Algorithm 1" for head averaging, MaxPool1D, +inf protection and the
// rejection of probabilities that round to 1):
//
//   pass1  : per (KV head, sequence split) stream K and V once.  For the G*w = M
//            window-query rows of the group: logits S^T = K Q^T on bf16 MFMA, an
//            online softmax (running max, normaliser S, and S_excl = mass off the
//            running arg-max, kept without cancellation) and the un-normalised
//            output a^T += V^T P^T on MFMA with P split into bf16 hi + lo parts.
//   merge  : per row, combine the split partials: final max, S, S_excl, arg-max
//            j*, a = a_un / S, ||a||^2, a as bf16 hi + lo, the arg-max token's
//            own term from a, and the singular / non-finite decisions.
//            Rows whose arg-max holds probability above ~0.94 recompute the
//            output over the other tokens exactly and take the arg-max term as
//            p*^2 ||abar - v_j*||^2, which stays accurate as p* -> 1.
//   pass2  : per (KV head, chunk of up to 2048 tokens + pooling halo) stream K and V again:
//            logits Q K^T and A V^T (a as hi + lo) on MFMA, then per element
//            p = 2^(l - lse), odds = p/(1-p), ||a - v||^2 = ||a||^2 - 2 a.v + ||v||^2,
//            contribution odds^2 ||a - v||^2, summed over the M rows, divided by
//            G; then max-pool over the chunk, +inf on the last w positions.
//
// Nothing of size O(n) besides the caller's score buffer is ever written.
#include <float.h>
#include <limits.h>

#include "common.h"

namespace dropkv {

// 16 bytes of K or V, optionally non-temporal.
template <bool NT>
__device__ __forceinline__ u32x4 stream16(const u16* p) {
  const u32x4* a = reinterpret_cast<const u32x4*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(a);
  return *a;
}
__device__ __forceinline__ bf16x8 load8(const u16* p) {
  return __builtin_bit_cast(bf16x8, stream16<kNTMfma>(p));
}
__device__ __forceinline__ bf16x8 zero8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_or_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o);
  return x;
}

// The input check: a running maximum of the magnitude bits (sign cleared) of
// every bf16 element a workgroup loads, two elements per operation
// (v_pk_max_u16); only the largest is needed to decide the contract.
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ us2 mag_max(us2 m, uint32_t x) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(us2, x & 0x7FFF7FFFu));
}
__device__ __forceinline__ us2 mag_max4(us2 m, u32x4 x) {
  m = mag_max(m, x[0]);
  m = mag_max(m, x[1]);
  m = mag_max(m, x[2]);
  return mag_max(m, x[3]);
}
// After the loads: NONFINITE if some element was inf or NaN, INPUT_RANGE if
// one was of magnitude >= 2^48 (wave-reduced, one atomic per offending wave).
__device__ __forceinline__ void latch_inputs(uint32_t* latch, us2 m) {
  const uint32_t b = max((uint32_t)m.x, (uint32_t)m.y);
  int f = b >= 0x7F80u ? (int)LATCH_NONFINITE : (b >= kInputRangeBits ? (int)LATCH_INPUT_RANGE : 0);
  f = wave_or_i(f);
  if (f && (threadIdx.x & 63) == 0) atomicOr(latch, (uint32_t)f);
}

// ---------------------------------------------------------------- pass 1 --
// Lane layout of the 32x32x16 bf16 MFMA (checked on gfx950): A[i][k] sits in
// lane i + 32*(k/8), element k%8; B[k][j] in lane j + 32*(k/8), element k%8;
// D[i][j] in lane j + 32*h, register v, with i = 8*(v/4) + 4*h + v%4.
//
// Pass 1 computes S^T = K Q^T (tokens x rows), so lane l owns query row l%32
// and 16 of the tile's 32 tokens; the softmax statistics of a row stay within
// the lane pair (l, l^32).  For PV it computes a^T = V^T P^T: P^T's operand is
// taken straight from S^T's registers by ordering the MFMA's reduction slots as
// token(kc, h, e) = 16*kc + 8*(e/4) + 4*h + e%4, and V^T's operand is gathered
// from a per-wave LDS copy of the V tile in that same order.

// LDS rows that MFMA operands are read from: a row of DP bf16 is CH = DP/8
// 16-byte chunks, chunk c stored at position c ^ (row & MASK) of a row of CHP
// (CH rounded up to a power of two) chunks.  Lanes reading the same chunk of 16
// consecutive rows, or 64 bytes of two rows four apart, then hit distinct banks.
template <int DP>
struct RowLayout {
  static constexpr int CH = DP / 8;
  static constexpr int CHP = CH <= 4 ? 4 : CH <= 8 ? 8 : CH <= 16 ? 16 : 32;
  static constexpr int ROWB = CHP * 16;
  static constexpr int MASK = CHP < 16 ? CHP - 1 : 15;
  __device__ __forceinline__ static int off(int row, int chunk) {
    return row * ROWB + ((chunk ^ (row & MASK)) << 4);
  }
};

template <int DP>
__device__ __forceinline__ bf16x8 lds8(const unsigned char* base, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + RowLayout<DP>::off(row, chunk)));
}

// Stage rows [0, 32) of a row-major bf16 matrix (rows >= nrows and columns >= d
// are zero) into LDS with the swizzled layout.  Whole workgroup.
// A load phase and a store phase with compile-time trip counts, so that a
// workgroup's staging loads (several blocks of rows) are all in flight at once
// rather than one memory round trip per chunk per block.
template <int DP, int NT = kThreads>
struct RowStage {
  static constexpr int IT = (kRows * RowLayout<DP>::CH + NT - 1) / NT;
  u32x4 x[IT];
  __device__ __forceinline__ void load(const u16* src, int nrows, int ld, int d) {
    using L = RowLayout<DP>;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = (int)threadIdx.x + k * NT;
      const int row = i / L::CH, ch = i % L::CH;
      x[k] = u32x4{0u, 0u, 0u, 0u};
      if (i < kRows * L::CH && row < nrows && ch * 8 < d)
        x[k] = *reinterpret_cast<const u32x4*>(src + (size_t)row * ld + ch * 8);
    }
  }
  __device__ __forceinline__ void store(unsigned char* dst) const {
    using L = RowLayout<DP>;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = (int)threadIdx.x + k * NT;
      if (i < kRows * L::CH) *reinterpret_cast<u32x4*>(dst + L::off(i / L::CH, i % L::CH)) = x[k];
    }
  }
};
template <int DP, int NT = kThreads>
__device__ __forceinline__ void stage_rows(unsigned char* dst, const u16* src, int nrows, int ld, int d) {
  RowStage<DP, NT> st;
  st.load(src, nrows, ld, d);
  st.store(dst);
}

// One 32-token K/V tile in MFMA operand layout: lane l holds 8 consecutive d
// values (16 bytes) of token l%32.  Interior tiles load unconditionally; only a
// ragged tile (tokens past the range end) or a head dimension below the padded
// width masks lanes to zero.
template <int NC, bool FULLD>
__device__ __forceinline__ void load_kv_tile(const u16* kg, const u16* vg, int64_t tok, bool tok_ok,
                                             bool ragged, int hh, int d, bf16x8 (&kk)[NC],
                                             bf16x8 (&vv)[NC]) {
  if (FULLD && !ragged) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = 16 * c + 8 * hh;
      kk[c] = load8(kg + tok * d + col);
      vv[c] = load8(vg + tok * d + col);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = 16 * c + 8 * hh;
      const bool ok = tok_ok && (FULLD || col < d);
      kk[c] = ok ? load8(kg + tok * d + col) : zero8();
      vv[c] = ok ? load8(vg + tok * d + col) : zero8();
    }
  }
}

template <int DP>
constexpr size_t pass1_lds_bytes() {
  // Q rows, then one V slot per wave
  return (size_t)kRows * RowLayout<DP>::ROWB * (1 + p1_waves(DP));
}

// K tile into registers (operand layout as load_kv_tile).
template <int NC, bool FULLD>
__device__ __forceinline__ void load_k_tile(const u16* kg, int64_t tok, bool tok_ok, bool ragged, int hh,
                                            int d, bf16x8 (&kk)[NC]) {
  if (FULLD && !ragged) {
#pragma unroll
    for (int c = 0; c < NC; ++c) kk[c] = load8(kg + tok * d + 16 * c + 8 * hh);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = 16 * c + 8 * hh;
      kk[c] = (tok_ok && (FULLD || col < d)) ? load8(kg + tok * d + col) : zero8();
    }
  }
}

// One direct global->LDS load of 16 bytes per lane from a wave-uniform base
// address (scalar registers) plus a 32-bit per-lane byte offset: lane l's
// bytes land at LDS address `lds` + 16 l.  Issued from inline assembly so that
// the compiler does not order every later LDS access after it; the caller waits
// explicitly (vector-memory counter) before reading the destination.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  // the base is wave-uniform by contract; reading it from the first lane lets
  // the compiler keep it in scalar registers whatever it can prove.  M0 is
  // written here without a clobber (the compiler reserves it and rejects one);
  // no compiler-generated code in these kernels reads M0.
  // (readfirstlane returns int: each half goes through uint32_t, never sign-extended)
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(u)), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS layout of a V tile: row-major rows of CHP 16-byte chunks, the chunk
// index XOR-ed with 4 * (row % 4) (kept inside the row): the four rows one
// transposed read gathers from land in distinct 64-byte bank ranges.
template <int DP>
struct VLayout {
  static constexpr int CHP = RowLayout<DP>::CHP;
  static constexpr int ROWB = RowLayout<DP>::ROWB;
  __device__ __forceinline__ static int sw(int row) { return ((row & 3) << 2) & (CHP - 1); }
  __device__ __forceinline__ static int off(int row, int chunk) {
    return row * ROWB + ((chunk ^ sw(row)) << 4);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (checked on gfx950): within each group of 16 lanes, lane i
// receives, as element e (e < 4), the 16-bit element i % 4 of the 8 bytes that
// lane 4e + i / 4 of its group addresses.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) unsigned char*)p));
}

// V tile of tokens [t0, t0+32) into registers, already in the order of its
// LDS slot (VLayout): register i of lane l is the 16 bytes the lane later
// stores at byte 1024 i + 16 l of the slot.  Padding chunks (column >= d) and
// tokens past `end` read some in-range row of the tile instead; they are
// multiplied by p = 0 or never used.
// With ROWL the registers are in RowLayout order instead (the layout MFMA
// operands are read from with lds8): a K tile loaded this way and stored with
// store_v_tile is read back in operand layout.  Either way each load
// instruction covers whole rows (CHP lanes per row), i.e. whole cache lines.
// With ZPAD, chunks past the head dimension are zero instead.  NT selects
// non-temporal loads.
template <int DP, bool ROWL = false, bool ZPAD = false, bool NT = kNTV1>
__device__ __forceinline__ void load_v_tile(const u16* vg, int64_t t0, int64_t end, int d, int lane,
                                            u32x4 (&vr)[VLayout<DP>::CHP / 2]) {
  using L = VLayout<DP>;
  constexpr int RPI = 64 / L::CHP;   // token rows one register covers
  const int row0 = lane / L::CHP, pc = lane % L::CHP;
  const int nrow = (int)min((int64_t)kTile, end - t0);
#pragma unroll
  for (int i = 0; i < L::CHP / 2; ++i) {
    const int row = RPI * i + row0;
    int c = ROWL ? pc ^ (row & RowLayout<DP>::MASK) : pc ^ L::sw(row);
    const bool pad = c * 8 >= d;
    if (pad) c = 0;
    const int rr = row < nrow ? row : 0;
    vr[i] = stream16<NT>(vg + (t0 + rr) * d + c * 8);
    if (ZPAD && pad) vr[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int DP>
__device__ __forceinline__ void store_v_tile(unsigned char* slot, int lane,
                                             const u32x4 (&vr)[VLayout<DP>::CHP / 2]) {
#pragma unroll
  for (int i = 0; i < VLayout<DP>::CHP / 2; ++i)
    *reinterpret_cast<u32x4*>(slot + 1024 * i + 16 * lane) = vr[i];
}

// V tile of tokens [t0, t0+32) straight into an LDS slot (no registers), in
// VLayout order: instruction i fills bytes [1024 i, 1024 i + 1024) of the slot,
// lane l the 16 bytes at 1024 i + 16 l.  Padding chunks (column >= d) and
// tokens past `end` read some in-range row of the tile instead; they are
// multiplied by p = 0 or never used.  Issues RowLayout<DP>::CHP / 2 loads.
template <int DP>
__device__ __forceinline__ void dma_v_tile(const u16* vg, int64_t t0, int64_t end, int d,
                                           unsigned char* slot, int lane) {
  using L = VLayout<DP>;
  constexpr int RPI = 64 / L::CHP;   // token rows one instruction fills
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)((__attribute__((address_space(3))) unsigned char*)slot));
  const int row0 = lane / L::CHP, pc = lane % L::CHP;
  if (t0 + kTile <= end) {
    // whole tile: the row offset of instruction i goes into the scalar base
#pragma unroll
    for (int i = 0; i < L::CHP / 2; ++i) {
      int c = pc ^ L::sw(RPI * i + row0);
      if (c * 8 >= d) c = 0;
      dma16s(vg + (t0 + RPI * i) * d, (uint32_t)(row0 * d + c * 8) * 2u, lds0 + 1024u * i);
    }
  } else {
    const int nrow = (int)(end - t0);
#pragma unroll
    for (int i = 0; i < L::CHP / 2; ++i) {
      const int row = RPI * i + row0;
      int c = pc ^ L::sw(row);
      if (c * 8 >= d) c = 0;
      const int rr = row < nrow ? row : 0;
      dma16s(vg + t0 * d, (uint32_t)(rr * d + c * 8) * 2u, lds0 + 1024u * i);
    }
  }
}


// Split dealt to a first-pass workgroup.  Workgroups are spread over the 8 XCDs
// by index modulo 8, so with the identity map the workgroups of one XCD would
// all read tiles of one residue modulo 8; with kP1XcdSwz (and a split count
// that is a multiple of 8) split s takes the deal of (s % 8) * (splits / 8) +
// s / 8, so every XCD reads every residue (measured: pass 1 ~1.3 us faster at
// 8 x 128K tokens).  A bijection: the split states and their fixed-order merge
// are unchanged in kind.
__device__ __forceinline__ int split_deal(int s, int splits) {
  if (!kP1XcdSwz || (splits & 7) != 0) return s;
  return (s & 7) * (splits >> 3) + (s >> 3);
}

// The tiles of one first-pass split.  With kP1Granule = 0 a split is one
// contiguous run of split_len tokens; otherwise the head's tiles are cut into
// granules of kP1Granule consecutive tiles dealt round robin to the splits
// (split s takes granules s, s + splits, ...), so every workgroup's reads
// spread over the whole head (measured: 3-4 % faster than contiguous runs at
// 128K tokens).  Either way a split's tiles ascend in token order, and jend
// bounds every tile of the split.
struct SplitTiles {
  static constexpr int GR = kP1Granule, GRD = GR > 0 ? GR : 1;
  int64_t jbeg, jend;
  int ntiles, s, splits;
  __device__ SplitTiles(int64_t n, int s_, int splits_, int64_t split_len) : s(s_), splits(splits_) {
    jbeg = GR ? 0 : (int64_t)s * split_len;
    jend = GR ? n : min(n, jbeg + split_len);
    if (GR) {
      const int64_t ttot = (n + kTile - 1) / kTile;
      const int64_t ngran = (ttot + GRD - 1) / GRD;
      const int64_t nk = s < ngran ? (ngran - 1 - s) / splits + 1 : 0;
      int64_t nt = nk * GRD;
      if (nk > 0 && s + (int64_t)splits * (nk - 1) == ngran - 1) nt -= ngran * GRD - ttot;
      ntiles = (int)nt;
    } else {
      ntiles = (int)((jend - jbeg + kTile - 1) / kTile);
    }
  }
  // first token of the split's t-th tile
  __device__ int64_t start(int t) const {
    if (!GR) return jbeg + (int64_t)t * kTile;
    const int64_t k = t / GRD, o = t % GRD;
    return (((int64_t)s + (int64_t)splits * k) * GRD + o) * kTile;
  }
};

template <int DP, bool FULLD>
__global__ __launch_bounds__(64 * p1_waves(DP), (DP <= 128 ? kP1Waves : 1)) void pass1_kernel(
    ScoreArgs a) {
  using L = RowLayout<DP>;
  constexpr int NC = DP / 16;
  constexpr int DB = DP / 32;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int NWV = p1_waves(DP), NT = 64 * NWV;
  __shared__ float sm_m[NWV][kRows], sm_S[NWV][kRows], sm_Sx[NWV][kRows];
  __shared__ int sm_j[NWV][kRows], sm_bad[NWV][kRows];

  const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  // a virtual head is one 32-row group of one KV head
  const int hv = blockIdx.x / a.splits, s = split_deal(blockIdx.x % a.splits, a.splits);
  const int g = hv / a.R, row0 = kRows * (hv % a.R);
  const SplitTiles sp(a.n, s, a.splits, a.split_len);
  const int64_t jend = sp.jend;
  const int ntiles = sp.ntiles;
  const int d = FULLD ? DP : a.d;   // a compile-time constant in the full-width instance
  const u16* kg = a.k + (size_t)g * a.hs;
  const u16* vg = a.v + (size_t)g * a.hs;
  const bool row_ok = row0 + r < a.M;
  const int64_t causal = row_ok ? a.n - a.w + ((row0 + r) % a.w) : -1;
  const int64_t all_see = a.n - a.w;   // every window query sees keys 0..n-w
  unsigned char* qs = smem_raw;                                  // Q rows of the group
  unsigned char* vs = smem_raw + (size_t)kRows * L::ROWB * (1 + wid);   // this wave's V tile

  // largest magnitude bits of the Q and V elements loaded here (K is checked by
  // the second pass, which reads every key too: checking it here would keep a
  // tile's K registers alive across the next tile's prefetch)
  us2 mg = {0, 0};
  {
    RowStage<DP, NT> qst;
    qst.load(a.q + ((size_t)g * a.M + row0) * d, min(kRows, a.M - row0), d, d);
#pragma unroll
    for (int k = 0; k < RowStage<DP, NT>::IT; ++k) mg = mag_max4(mg, qst.x[k]);
    qst.store(qs);
  }
  __syncthreads();

  float m = -INFINITY, S = 0.f, Sx = 0.f, chk = 0.f;
  int jst = INT_MAX, bad = 0;
  bool has = false;
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;

  // Each wave walks its tiles in order.  K and V of a tile come straight into
  // registers; V then goes through the wave's LDS slot, from which the PV
  // product gathers it transposed.  With the overlap option the next tile's K
  // is loaded into the same registers as soon as the logits have consumed
  // them, and its V as soon as this tile's V is in LDS, so those loads fly
  // during this tile's softmax and PV.  The second workgroup on the CU covers
  // the rest of the latency.
  // Head dimensions above 128 have no registers to spare for V: it goes from
  // memory straight into the LDS slot (direct loads), without prefetch.
  constexpr bool kVRegs = DP <= 128;
  constexpr bool kPreK = kP1PreK && kVRegs, kPreV = kP1PreV && kVRegs;
  bf16x8 kk[NC];
  u32x4 vr[kVRegs ? L::CHP / 2 : 1];
  if (wid < ntiles) {
    const int64_t f0 = sp.start(wid);
    if constexpr (kPreK) load_k_tile<NC, FULLD>(kg, f0 + r, f0 + r < jend, f0 + kTile > jend, hh, d, kk);
    if constexpr (kPreV) load_v_tile<DP>(vg, f0, jend, d, lane, vr);
  }
  for (int t = wid; t < ntiles; t += NWV) {
    const int64_t j0 = sp.start(t);
    // lane-derived addresses are recomputed every tile (two or three integer
    // operations each) instead of being held in registers across the loop
    int lx = lane;
    asm volatile("" : "+v"(lx));
    const int rx = lx & 31, hx = lx >> 5;
    if constexpr (!kPreK) load_k_tile<NC, FULLD>(kg, j0 + rx, j0 + rx < jend, j0 + kTile > jend, hx, d, kk);
    if constexpr (!kVRegs) dma_v_tile<DP>(vg, j0, jend, d, vs, lx);
    else if constexpr (!kPreV) load_v_tile<DP>(vg, j0, jend, d, lx, vr);
    f32x16 st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      st = mfma32(kk[c], lds8<DP>(qs, rx, 2 * c + hx), st);
    }
    const bool more = t + NWV < ntiles;
    const int64_t n0 = sp.start(t + NWV);
    if (kPreK && more)
      load_k_tile<NC, FULLD>(kg, n0 + rx, n0 + rx < jend, n0 + kTile > jend, hx, d, kk);

    // logits in log2 units, in place; masks only on tiles that reach past the
    // split end or into the window (rows >= M have zero queries and are never
    // read).  Token offsets within the tile are small integers: register v of
    // lane (r, hh) holds offset 8 (v / 4) + 4 hh + v % 4.
    const bool interior = (j0 + kTile <= jend) && (j0 + kTile - 1 <= all_see);
    float lm = -INFINITY;
    if (interior) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        chk = fmaf(st[v], 0.f, chk);          // becomes NaN on any inf / NaN logit
        st[v] *= a.scale_log2;
        lm = fmaxf(lm, st[v]);
      }
    } else {
      // last valid offset of this row in this tile (-1: none)
      const int64_t lim64 = min(min(jend - j0 - 1, causal - j0), (int64_t)kTile);
      const int lim = (int)max(lim64, (int64_t)-1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool valid = 8 * (v >> 2) + 4 * hx + (v & 3) <= lim;
        if (valid) chk = fmaf(st[v], 0.f, chk);
        st[v] = valid ? st[v] * a.scale_log2 : -INFINITY;
        lm = fmaxf(lm, st[v]);
      }
    }
    lm = fmaxf(lm, __shfl_xor(lm, 32));
    const bool newmax = lm > m;
    if (__any(newmax)) {
      // some row's running maximum moves: find the tile arg-max (lowest index)
      // and rescale; the old arg-max's unit mass joins S_excl
      int lj = INT_MAX;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 8 * (v >> 2) + 4 * hx + (v & 3);
        if (st[v] == lm && lm > -INFINITY) lj = min(lj, off);
      }
      lj = min(lj, __shfl_xor(lj, 32));
      const float mn = newmax ? lm : m;
      const bool live = mn > -INFINITY;
      const float alpha = live ? ex2(m - mn) : 1.f;
      float ts = 0.f, tx = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 8 * (v >> 2) + 4 * hx + (v & 3);
        st[v] = live ? ex2(st[v] - mn) : 0.f;
        ts += st[v];
        tx += (off == lj) ? 0.f : st[v];
      }
      ts += __shfl_xor(ts, 32);
      tx += __shfl_xor(tx, 32);
      if (newmax) {
        Sx = (Sx + (has ? 1.f : 0.f)) * alpha + tx;
        jst = (int)j0 + lj;
        has = true;
      } else {
        Sx = Sx + ts;
      }
      S = S * alpha + ts;
      m = mn;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] *= alpha;
    } else {
      // no maximum moved: every token of the tile joins S and S_excl
      const float mref = (m > -INFINITY) ? m : 0.f;
      float ts = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        st[v] = ex2(st[v] - mref);
        ts += st[v];
      }
      ts += __shfl_xor(ts, 32);
      S += ts;
      Sx += ts;
    }

    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = st[8 * kc + e];
        const __bf16 hi = (__bf16)x;
        ph[kc][e] = hi;
        pl[kc][e] = (__bf16)(x - (float)hi);
      }
    // this tile's V has landed once at most the loads issued above are pending
    if constexpr (kVRegs) {
#pragma unroll
      for (int i = 0; i < L::CHP / 2; ++i) mg = mag_max4(mg, vr[i]);
      store_v_tile<DP>(vs, lx, vr);
      if (kPreV && more) load_v_tile<DP>(vg, n0, jend, d, lx, vr);
    } else {
      wait_vmem_below<0>();   // this tile's V has landed in the slot
    }
    wave_sync_lds();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // V^T operand of lane (r, hh): column 32 b + r, tokens 16 kc + 8 (e/4) +
      // 4 hh + e%4.  Two transposed reads per block: lane 4e' + q of each
      // 16-lane group addresses token row 16 kc + 8 half + 4 hh + e' and the
      // 8 bytes holding columns 32 b + 16 (group % 2) + 4 q .. + 3.
      const int gsub = (lx >> 4) & 1, e4 = (lx >> 2) & 3, q = lx & 3;
      bf16x8 va[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        s16x4 part[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int row = 16 * kc + 8 * half + 4 * hx + e4;
          const int chunk = 4 * b + 2 * gsub + (q >> 1);
          part[half] = lds_read_tr16(vs + VLayout<DP>::off(row, chunk) + 8 * (q & 1));
        }
        va[b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3,
                                                                   4, 5, 6, 7));
        if constexpr (!kVRegs) {   // V came straight to LDS: check it as it is read
          const u32x4 vx = __builtin_bit_cast(u32x4, va[b]);
          mg = mag_max4(mg, vx);
        }
      }
      // the DB accumulators are independent: issue them back to back
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] = mfma32(va[b], ph[kc], acc[b]);
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] = mfma32(va[b], pl[kc], acc[b]);
    }
    wave_sync_lds();
  }
  if (!(chk == 0.f)) bad = 1;
  latch_inputs(a.latch, mg);

  // ---- combine the waves' states for each row (fixed order) ----
  bad |= __shfl_xor(bad, 32);
  if (hh == 0) {
    sm_m[wid][r] = m;
    sm_S[wid][r] = S;
    sm_Sx[wid][r] = Sx;
    sm_j[wid][r] = has ? jst : INT_MAX;
    sm_bad[wid][r] = bad;
  }
  __syncthreads();
  float Mf = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) Mf = fmaxf(Mf, sm_m[w][r]);
  int wstar = -1, jbest = INT_MAX, badf = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if (Mf > -INFINITY && sm_m[w][r] == Mf && sm_j[w][r] < jbest) {
      jbest = sm_j[w][r];
      wstar = w;
    }
    badf |= sm_bad[w][r];
  }
  float Sf = 0.f, Sxf = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const float f = (sm_m[w][r] > -INFINITY) ? ex2(sm_m[w][r] - Mf) : 0.f;
    Sf += sm_S[w][r] * f;
    Sxf += (w == wstar) ? sm_Sx[w][r] * f : sm_S[w][r] * f;
  }
  const float myf = (m > -INFINITY) ? ex2(m - Mf) : 0.f;
  __syncthreads();  // every wave is done with its V tile; reuse LDS as float slabs
  // each wave stores its scaled accumulators in a slab of its own (row stride
  // DP + 1 floats, so the 32 rows a store touches fall in distinct banks); one
  // barrier; then the slabs are summed in wave order straight into the partials
  constexpr int SP = DP + 1;
  float* slab = reinterpret_cast<float*>(smem_raw) + (size_t)wid * kRows * SP;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int dd = 32 * b + 8 * (v >> 2) + 4 * hh + (v & 3);
      slab[r * SP + dd] = acc[b][v] * myf;
    }
  __syncthreads();
  const size_t pb = ((size_t)hv * a.splits + s) * kRows;
  if (tid < kRows) {
    a.part.m2[pb + r] = Mf;
    a.part.S[pb + r] = Sf;
    a.part.Sx[pb + r] = Sxf;
    a.part.jstar[pb + r] = jbest;
    // bit 1: the split's arg-max holds all but S_excl / S < kFixupThreshold of its mass
    const bool flagged = Mf > -INFINITY && Sxf < kFixupThreshold;
    a.part.bad[pb + r] = badf | (flagged ? 2 : 0);
    if (__any(flagged) && tid == 0) atomicOr(a.ex.head + hv, 1u);   // rare
  }
  const float* slabs = reinterpret_cast<const float*>(smem_raw);
  for (int i = tid; i < kRows * DP; i += NT) {   // the group's 32 rows (padding rows are ignored later)
    const int rr = i / DP, dd = i - rr * DP;
    float x = slabs[rr * SP + dd];
#pragma unroll
    for (int w = 1; w < NWV; ++w) x += slabs[(size_t)w * kRows * SP + rr * SP + dd];
    a.part.a[pb * DP + i] = x;
  }
}

// ----------------------------------------------------------------- merge --
// One workgroup per (KV head, window row).  Every split's statistics and the first
// partial sums of a are fetched in one round trip; the maximum and its split
// come from one packed reduction; every reduction has a fixed order (bitwise
// reproducible); a is summed by float4 column group with the splits
// partitioned over SG thread groups.
//
// Rows whose winning split is flagged (its arg-max holds more than ~0.94 of the
// split's mass) take the arg-max term from the exact output over the other
// tokens, abar = sum_{j != j*} e_j v_j / S_excl.  Every split but the winning
// one already sums only tokens other than j* (the first pass partitions the
// tokens), so only the winning split's tokens are summed again, j* left out.
// That work is spread over xh helper workgroups per (KV head, row group): each
// takes a slice of the winning split's tokens for every flagged row of the
// group.  The row's workgroup and its helpers each count themselves in on a
// per-row counter after writing their part; whichever arrives last adds the
// parts in a fixed order and writes the arg-max term (no workgroup ever waits
// for another).  The helpers take the lowest workgroup indices, so that in the
// rare call that needs them their first loads reach memory ahead of the row
// workgroups' (measured: peaked merge ~27 us against ~29 us with helpers
// last); in the common call they read one flag and exit.
constexpr int kMaxSplits = 1024;

__device__ __forceinline__ float block_sum256(float x, float* red) {
  x = wave_sum(x);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Order-preserving uint32 image of a float for max-reductions; NaN and -0 map
// like -inf and +0 (fmaxf ignores NaN).
__device__ __forceinline__ uint32_t max_key(float f) {
  if (!(f == f)) f = -INFINITY;
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_max_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// (max key of m2, ~arg-max token): the largest m2, the lowest token on ties
__device__ __forceinline__ uint64_t split_key(float m2, int j) {
  return ((uint64_t)max_key(m2) << 32) | (uint32_t)~(uint32_t)j;
}

__device__ __forceinline__ uint32_t load_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// After this workgroup's writes: count it in on `cnt` (release, agent scope);
// true, for every thread, if it was the last of `total` arrivals -- its
// caller then reads the others' writes (acquire already done here).
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, uint32_t total, int* s_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == total - 1u;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

// The last arrival for flagged rows rows[0..nl) (arg-max tokens js[0..nl)):
// abar from the other splits' sum and the helpers' parts (added in helper
// order), then a - v_j* = (S_excl / S)(abar - v_j*) and the arg-max term
// p*^2 ||abar - v_j*||^2.  Every load is issued before the first result is
// used, and every sum has a fixed order, so the result does not depend on which
// workgroup arrived last.  Whole workgroup; dsq holds nl * DP / 4 floats, sxs
// and rmeta nl entries; resets the rows' counters.
template <int DP>
__device__ void exclusion_combine(const ScoreArgs& a, int hv, const int* rows, const int* js, int nl,
                                  float* dsq, float* sxs, float4* rmeta) {
  constexpr int CG = DP / 4;   // float4 column groups of a row
  // (row, column group) pairs per thread whose loads fly together: all of a
  // 32-row group's at DP <= 128
  constexpr int U = DP <= 128 ? (kRows * CG + kThreads - 1) / kThreads : 2;
  constexpr bool kOneBatch = U * kThreads >= kRows * CG;
  static_assert(CG % 8 == 0, "eight lanes share a row's distance");
  const int tid = threadIdx.x;
  const int g = hv / a.R;
  // uniform bases; the per-lane offsets below fit 32 bits
  const float* aob = a.ex.ao + (size_t)hv * kRows * DP;
  const float* pbase = a.ex.part + (size_t)hv * a.xh * kRows * DP;   // helper h, row r: (h * 32 + r) * DP
  const float* sxb = a.ex.sx + (size_t)hv * a.xh * kRows;
  float* aresb = a.rs.ares + (size_t)hv * kRows * DP;
  const u16* vb = a.v + (size_t)g * a.hs;
  // the rows' scalars (threads below nl) in the same round trip as the first pairs
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  float sxp[kMaxHelpers];
#pragma unroll
  for (int h = 0; h < kMaxHelpers; ++h) sxp[h] = 0.f;
  if (tid < nl) {
    const int row = rows[tid];
    m = *reinterpret_cast<const float4*>(a.ex.meta + ((size_t)hv * kRows + row) * 4);   // S, S_excl, S other, -
#pragma unroll
    for (int h = 0; h < kMaxHelpers; ++h)
      if (h < a.xh) sxp[h] = sxb[(uint32_t)(h * kRows + row)];
  }
  const int np = nl * CG;
  float4 ao[U], pv[U][kMaxHelpers];
  uint2 vv[U];
  auto load_pairs = [&](int p0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * kThreads;
      const bool in = p < np;
      const int i = in ? p / CG : 0, cg = in ? p - (p / CG) * CG : 0, row = rows[i];
      const bool col = in && 4 * cg < a.d;
      const uint32_t off = (uint32_t)(row * DP + 4 * cg);
      ao[u] = col ? *reinterpret_cast<const float4*>(aob + off) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int h = 0; h < kMaxHelpers; ++h)
        pv[u][h] = (col && h < a.xh)
                       ? *reinterpret_cast<const float4*>(pbase + (uint32_t)(h * kRows * DP) + off)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      const int jst = js[i];   // checked in range before a row is flagged; kept so here
      vv[u] = (col && jst >= 0 && jst < a.n)
                  ? *reinterpret_cast<const uint2*>(vb + (size_t)jst * a.d + 4 * cg)
                  : make_uint2(0u, 0u);
    }
  };
  auto publish_rows = [&]() {
    if (tid < nl) {
      float x = m.z;
#pragma unroll
      for (int h = 0; h < kMaxHelpers; ++h) x += sxp[h];
      sxs[tid] = x;
      rmeta[tid] = m;
    }
    __syncthreads();
  };
  auto finish_pairs = [&](int p0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * kThreads;
      if (p >= np) continue;
      const int i = p / CG, cg = p - i * CG;
      float4 t = ao[u];
#pragma unroll
      for (int h = 0; h < kMaxHelpers; ++h) {
        t.x += pv[u][h].x; t.y += pv[u][h].y; t.z += pv[u][h].z; t.w += pv[u][h].w;
      }
      const float sx = sxs[i];
      const bool in = 4 * cg < a.d;   // columns past d are zero
      const float d0 = in ? t.x / sx - __uint_as_float(vv[u].x << 16) : 0.f;
      const float d1 = in ? t.y / sx - __uint_as_float(vv[u].x & 0xffff0000u) : 0.f;
      const float d2 = in ? t.z / sx - __uint_as_float(vv[u].y << 16) : 0.f;
      const float d3 = in ? t.w / sx - __uint_as_float(vv[u].y & 0xffff0000u) : 0.f;
      const float k = rmeta[i].y / rmeta[i].x;   // S_excl / S
      *reinterpret_cast<float4*>(aresb + (uint32_t)(rows[i] * DP + 4 * cg)) =
          make_float4(k * d0, k * d1, k * d2, k * d3);
      dsq[p] = (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
  };
  if constexpr (kOneBatch) {
    load_pairs(tid);
    publish_rows();
    finish_pairs(tid);
  } else {
    const int nb = (np + U * kThreads - 1) / (U * kThreads);
    for (int bt = 0; bt < nb; ++bt) {
      load_pairs(bt * U * kThreads + tid);
      if (bt == 0) publish_rows();
      finish_pairs(bt * U * kThreads + tid);
    }
  }
  __syncthreads();
  // a row's squared distance: eight lanes over consecutive column groups, then a
  // butterfly; lane 0 of the eight holds the fixed-order total
  {
    const int i = tid >> 3, k = tid & 7;
    float x = 0.f;
    if (i < nl)
#pragma unroll
      for (int c = 0; c < CG / 8; ++c) x += dsq[i * CG + k * (CG / 8) + c];
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 1);
    if (k == 0 && i < nl) {
      const size_t ro = (size_t)hv * kRows + rows[i];
      const float pstar = 1.f / rmeta[i].x;
      a.rs.cstar[ro] = pstar * pstar * x;
      __hip_atomic_store(a.ex.cnt + ro, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
}

template <int DP>
struct MergeRowLds {
  float m2[kMaxSplits], S[kMaxSplits], Sx[kMaxSplits], f[kMaxSplits];
  int j[kMaxSplits], bad[kMaxSplits];
  float4 red4[kThreads];
};
// V tiles in flight per helper wave: two at DP <= 128, one above
template <int DP>
constexpr int help_tb() { return DP <= 128 ? 2 : 1; }
template <int DP>
struct MergeHelpLds {
  // the group's Q rows, then help_tb V tile slots per wave (VLayout, as in the
  // first pass); after the tiles, the slots hold two slabs of sums
  unsigned char buf[(1 + kWaves * help_tb<DP>()) * kRows * RowLayout<DP>::ROWB];
  float m2[kRows];
  int js[kRows], sst[kRows], lim[kRows];
  int act[kRows];                            // row flagged and in the split being summed
  float sxw[kWaves][kRows];
  int nlist, list[kRows];                    // distinct winning splits of flagged rows
  static_assert(2 * (size_t)kRows * DP * 4 <= (size_t)kWaves * kRows * RowLayout<DP>::ROWB,
                "two slabs fit the tile slots");
  static_assert((size_t)kRows * DP <= sizeof(buf), "the combine's squares fit the tiles");
};
template <int DP>
struct MergeCombineLds {
  float dsq[kRows * DP / 4];
};

// A helper: the flagged rows of virtual head hv (from the same order-free
// maximum as their row workgroups), then for each distinct winning split its
// slice of the split's tokens, summed for every flagged row of that split.
// The dependent steps are kept few: statistics and Q rows in one round trip,
// a wave's tile loads (two tiles at DP <= 128: K into registers, V straight
// into LDS) in the next, one arrival round trip for all rows, and two for the
// combine.
template <int DP>
__device__ void merge_helper(const ScoreArgs& a, int hv, int h, MergeHelpLds<DP>& L, float* dsq,
                             int* crows, int* cjs, float* csxs, float4* cmeta, int* s_flag) {
  using RL = RowLayout<DP>;
  const int tid = threadIdx.x;
  const int g = hv / a.R, row0 = kRows * (hv % a.R);
  const int S = a.splits;
  const size_t base = (size_t)hv * S * kRows;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 31;
  // no split of this virtual head is flagged (the common case): nothing to do
  if (load_agent_u32(a.ex.head + hv) == 0u) return;
  // the group's query rows (zero past d and past M), loaded with the statistics
  RowStage<DP> qst;
  qst.load(a.q + ((size_t)g * a.M + row0) * a.d, min(kRows, a.M - row0), a.d, a.d);
  // rows: 8 threads each, splits strided by 8; a batch of SB splits per thread
  // loaded at once, and the winner found in registers
  {
    constexpr int SB = 8;
    const int row = tid >> 3, k = tid & 7;
    const bool rok = row0 + row < a.M;
    const float* m2b = a.part.m2 + base;   // uniform bases, 32-bit offsets
    const int* jb = a.part.jstar + base;
    const int* bb = a.part.bad + base;
    uint64_t best = 0u;
    int bs = -1, bflag = 0;
#pragma unroll 1
    for (int s0 = k; s0 < S; s0 += 8 * SB) {
      float mv[SB];
      int jv[SB], bv[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int sp_ = s0 + 8 * u;
        const bool ok = rok && sp_ < S;
        const uint32_t o = (uint32_t)((ok ? sp_ : 0) * kRows + row);
        mv[u] = ok ? m2b[o] : -INFINITY;
        jv[u] = ok ? jb[o] : INT_MAX;
        bv[u] = ok ? bb[o] : 0;
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const uint64_t key = split_key(mv[u], jv[u]);
        if (s0 + 8 * u < S && key > best) { best = key; bs = s0 + 8 * u; bflag = bv[u]; }
      }
    }
    uint64_t gbest = best;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)gbest, o);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(gbest >> 32), o);
      const uint64_t ob = ((uint64_t)hi << 32) | lo;
      gbest = gbest > ob ? gbest : ob;
    }
    const float M = from_max_key((uint32_t)(gbest >> 32));
    const int jst = (int)~(uint32_t)gbest;
    if (k == 0) {
      L.sst[row] = -1;
      L.m2[row] = M;
      L.js[row] = jst;
      L.act[row] = 0;
      L.lim[row] = rok ? (int)(a.n - a.w + ((row0 + row) % a.w)) : -1;
    }
    __syncthreads();
    // the lane holding the winning split (keys are distinct: tokens differ)
    if (rok && M > -INFINITY && best == gbest && bs >= 0)
      L.sst[row] = ((bflag & 2) && jst >= 0 && jst < a.n) ? bs : -1;
    __syncthreads();
  }
  // the distinct winning splits of the flagged rows (any order: a row belongs
  // to exactly one of them)
  if (wid == 0) {
    const int s = lane < kRows ? L.sst[lane] : -1;
    bool first = s >= 0;
#pragma unroll 1
    for (int o = 0; o < kRows; ++o) {
      const int so = __builtin_amdgcn_readlane(s, o);   // (a register read, no LDS round trip)
      if (o < lane && so == s) first = false;
    }
    const uint64_t fm = __ballot(first);
    if (first) L.list[__popcll(fm & ((1ull << lane) - 1ull))] = s;
    if (lane == 0) L.nlist = __popcll(fm);
  }
  __syncthreads();
  if (L.nlist == 0) return;   // no flagged row: nothing to sum, nobody to meet

  constexpr int NC = DP / 16, DB = DP / 32;
  constexpr int TB = help_tb<DP>(), VI = VLayout<DP>::CHP / 2;   // VI: loads per V tile
  unsigned char* qs = L.buf;
  qst.store(qs);
  unsigned char* vs0 = L.buf + (size_t)kRows * RL::ROWB * (1 + TB * wid);   // this wave's V slots
  const u16* kg = a.k + (size_t)g * a.hs;
  const u16* vg = a.v + (size_t)g * a.hs;
  __syncthreads();
  for (int li = 0; li < L.nlist; ++li) {
    const int s0 = __builtin_amdgcn_readfirstlane(L.list[li]);
    if (tid < kRows) L.act[tid] = L.sst[tid] == s0 ? 1 : 0;
    __syncthreads();
    const bool ract = L.act[r] != 0;
    const float rm2 = L.m2[r];
    const int rjs = L.js[r], rlim = L.lim[r];
    const SplitTiles sp(a.n, s0, a.splits, a.split_len);
    const int tph = (sp.ntiles + a.xh - 1) / a.xh;   // tiles per helper
    const int t0 = h * tph, t1 = min(sp.ntiles, t0 + tph);
    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
    float sx = 0.f;
    // each wave walks its tiles as in the first pass, TB at a time with every
    // load issued first (K tiles into registers, then V tiles straight into
    // the wave's slots); e_j = 2^(l_j - m2) with the row's own maximum, zero
    // for the arg-max, for keys past the row's causal limit and past the
    // split, and for rows not summed here
    for (int tb = t0 + wid; tb < t1; tb += TB * kWaves) {
      const int nu = (TB > 1 && tb + kWaves < t1) ? 2 : 1;   // tiles this pass (wave-uniform)
      // lane-derived addresses are recomputed every tile from an opaque copy of
      // the lane index (as in the first pass), not held in registers across the loop
      int lx = lane;
      asm volatile("" : "+v"(lx));
      const int rx = lx & 31, hx = lx >> 5;
      // every load first: K tiles into registers (the second into kB), then the
      // V tiles straight into the wave's slots
      bf16x8 kA[NC], kB[NC];
      {
        const int64_t j0 = sp.start(tb);
        load_k_tile<NC, false>(kg, j0 + rx, j0 + rx < sp.jend, j0 + kTile > sp.jend, hx, a.d, kA);
      }
      if (nu > 1) {
        const int64_t j1 = sp.start(tb + kWaves);
        load_k_tile<NC, false>(kg, j1 + rx, j1 + rx < sp.jend, j1 + kTile > sp.jend, hx, a.d, kB);
      }
      dma_v_tile<DP>(vg, sp.start(tb), sp.jend, a.d, vs0, lx);
      if (nu > 1) dma_v_tile<DP>(vg, sp.start(tb + kWaves), sp.jend, a.d, vs0 + kRows * RL::ROWB, lx);
      // one copy of the tile's code, run nu times (the helper path runs once per
      // call: its code is cold in the instruction cache, so it is kept short)
#pragma unroll 1
      for (int u = 0; u < nu; ++u) {
        const int64_t j0 = sp.start(tb + u * kWaves);
        unsigned char* vs = vs0 + (size_t)u * kRows * RL::ROWB;
        int ly = lane;
        asm volatile("" : "+v"(ly));
        const int ry = ly & 31, hy = ly >> 5;
        f32x16 st;
#pragma unroll
        for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) st = mfma32(kA[c], lds8<DP>(qs, ry, 2 * c + hy), st);
        // offsets within the tile: valid below `end` (the split's end and the
        // row's causal limit), and not the arg-max's (`skip`, -1 when elsewhere)
        const int end = ract ? (int)max(min(min(sp.jend - j0, (int64_t)rlim - j0 + 1), (int64_t)kTile),
                                        (int64_t)0)
                             : 0;
        const int skip = (rjs >= j0 && rjs < j0 + kTile) ? (int)(rjs - j0) : -1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 8 * (v >> 2) + 4 * hy + (v & 3);
          const bool ok = off < end && off != skip;
          st[v] = ok ? ex2(st[v] * a.scale_log2 - rm2) : 0.f;
          sx += st[v];
        }
        bf16x8 ph[2], pl[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = st[8 * kc + e];
            const __bf16 hi = (__bf16)x;
            ph[kc][e] = hi;
            pl[kc][e] = (__bf16)(x - (float)hi);
          }
        // this tile's V has landed once at most the next tile's V loads are pending
        if (u + 1 < nu) wait_vmem_below<VI>();
        else wait_vmem_below<0>();
        wave_sync_lds();
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int gsub = (ly >> 4) & 1, e4 = (ly >> 2) & 3, q = ly & 3;
          bf16x8 va[DB];
#pragma unroll
          for (int b = 0; b < DB; ++b) {
            s16x4 part[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int row = 16 * kc + 8 * half + 4 * hy + e4;
              const int chunk = 4 * b + 2 * gsub + (q >> 1);
              part[half] = lds_read_tr16(vs + VLayout<DP>::off(row, chunk) + 8 * (q & 1));
            }
            va[b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3,
                                                                       4, 5, 6, 7));
          }
#pragma unroll
          for (int b = 0; b < DB; ++b) acc[b] = mfma32(va[b], ph[kc], acc[b]);
#pragma unroll
          for (int b = 0; b < DB; ++b) acc[b] = mfma32(va[b], pl[kc], acc[b]);
        }
        wave_sync_lds();
        if (u + 1 < nu) {
#pragma unroll
          for (int c = 0; c < NC; ++c) kA[c] = kB[c];
        }
      }
    }
    sx += __shfl_xor(sx, 32);
    // the waves' sums over the tile slots: waves 0 and 1 store slabs 0 and 1,
    // waves 2 and 3 add into them, then slab 0 + slab 1: a fixed order.  Rows are padded to DP + 1 floats where two such slabs fit
    // the slots (the 32 rows one store touches then fall in distinct banks, and
    // every store is a constant offset from the row); otherwise columns are
    // XOR-ed with the row within their 32-column block.
    constexpr bool kPadSlab = 2 * kRows * (DP + 1) * 4 <= TB * kWaves * kRows * RL::ROWB;
    constexpr int SP = kPadSlab ? DP + 1 : DP;
    static_assert(2 * kRows * SP * 4 <= TB * kWaves * kRows * RL::ROWB, "two slabs fit the slots");
    __syncthreads();   // every wave is done with its slots
    int lz = lane;
    asm volatile("" : "+v"(lz));
    const int rz = lz & 31, hz = lz >> 5;
    float* slab = reinterpret_cast<float*>(L.buf + (size_t)kRows * RL::ROWB);
    float* mine = slab + (size_t)(wid & 1) * kRows * SP + rz * SP;
    if (hz == 0) L.sxw[wid][rz] = sx;
    if (wid < 2) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * b + 8 * (v >> 2) + 4 * hz + (v & 3);
          mine[kPadSlab ? c : (c ^ rz)] = acc[b][v];
        }
    }
    __syncthreads();
    if (wid >= 2) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * b + 8 * (v >> 2) + 4 * hz + (v & 3);
          mine[kPadSlab ? c : (c ^ rz)] += acc[b][v];
        }
    }
    __syncthreads();
    // this helper's part for the split's rows, four columns per store
    const size_t hb = ((size_t)hv * a.xh + h) * kRows;
    static_assert((kRows * DP / 4) % kThreads == 0, "whole passes over the part");
#pragma unroll
    for (int i4 = tid; i4 < kRows * DP / 4; i4 += kThreads) {
      const int row = (4 * i4) / DP, dd = 4 * i4 - row * DP;
      float4 x;
      float* xs = reinterpret_cast<float*>(&x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int o = row * SP + (kPadSlab ? dd + e : ((dd + e) ^ (row & 31)));
        xs[e] = slab[o] + slab[kRows * SP + o];
      }
      if (L.act[row]) *reinterpret_cast<float4*>(a.ex.part + (hb + row) * DP + dd) = x;
    }
    if (tid < kRows && L.act[tid]) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) x += L.sxw[w][tid];
      a.ex.sx[hb + tid] = x;
    }
    __syncthreads();
  }
  // count in on every flagged row at once (one lane per row), then combine
  // those this helper finished last
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    bool last = false;
    if (lane < kRows && L.sst[lane] >= 0) {
      const uint32_t old = __hip_atomic_fetch_add(a.ex.cnt + (size_t)hv * kRows + lane, 1u,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = old == (uint32_t)a.xh;   // xh helpers + the row's workgroup
    }
    const uint64_t lm = __ballot(last);
    if (lm) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (last) {
      const int at = __popcll(lm & ((1ull << lane) - 1ull));
      crows[at] = lane;
      cjs[at] = L.js[lane];
    }
    if (lane == 0) *s_flag = __popcll(lm);
  }
  __syncthreads();
  const int nl = *s_flag;
  if (nl) exclusion_combine<DP>(a, hv, crows, cjs, nl, dsq, csxs, cmeta);   // dsq overlays the slots
}

template <int DP>
__global__ __launch_bounds__(kThreads, (DP <= 128 ? 2 : 1)) void merge_kernel(ScoreArgs a) {
  constexpr int CG = DP / 4;              // float4 column groups of a row of a
  constexpr int SG = kThreads / CG;       // split groups summing a
  constexpr int PF = 8;                   // a loads per thread issued before the weights exist
  // one LDS region for the role of the workgroup; the combine's squares reuse
  // it once the row workgroup's arrays or the helper's tiles are done with
  __shared__ __align__(16) union {
    MergeRowLds<DP> r;
    MergeHelpLds<DP> h;
    MergeCombineLds<DP> c;
  } lds;
  __shared__ int crows[kRows], cjs[kRows];
  __shared__ float csxs[kRows];
  __shared__ float4 cmeta[kRows];
  __shared__ uint64_t rk[kWaves];
  __shared__ int s_star, s_flag;
  __shared__ float rf[3][kWaves];
  __shared__ uint32_t ro_[2][kWaves];
  __shared__ float tmp[kWaves];
  float* sm_m2 = lds.r.m2;
  float* sm_S = lds.r.S;
  float* sm_Sx = lds.r.Sx;
  float* sm_f = lds.r.f;
  int* sm_j = lds.r.j;
  int* sm_bad = lds.r.bad;
  float4* red4 = lds.r.red4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // virtual head hv = (KV head g, row group); r is the row within the group and
  // rg_row the window query row within the KV head.  A group has RB =
  // min(32, M) workgroups: with fewer than 32 window rows per KV head, the
  // workgroup of row r also zeroes the padded rows r + RB, r + 2 RB, ... of
  // its group, which have no window row to merge.  The helpers come first.
  const int RB = min(kRows, a.M);
  const int nhelp = a.Hkv * a.R * a.xh;
  if ((int)blockIdx.x < nhelp) {
    const int hb = blockIdx.x;
    merge_helper<DP>(a, hb / a.xh, hb % a.xh, lds.h, lds.c.dsq, crows, cjs, csxs, cmeta, &s_flag);
    return;
  }
  const int bx = blockIdx.x - nhelp;
  const int hv = bx / RB, r = bx % RB;
  const int g = hv / a.R, rg_row = kRows * (hv % a.R) + r;
  const size_t ro = (size_t)hv * kRows + r;
  auto zero_row = [&](size_t rz) {   // padded rows: zero operands so pass 2's MFMA rows stay inert
    for (int dd = tid; dd < DP; dd += kThreads) {
      a.rs.a_hi[rz * DP + dd] = 0;
      a.rs.a_lo[rz * DP + dd] = 0;
      a.rs.ares[rz * DP + dd] = 0.f;
    }
    if (tid == 0) {
      a.rs.m2[rz] = 0.f; a.rs.lse2[rz] = INFINITY; a.rs.S[rz] = 1.f; a.rs.an2[rz] = 0.f;
      a.rs.cstar[rz] = 0.f; a.rs.jstar[rz] = -1; a.rs.fix[rz] = 0;
    }
  };
  for (int rp = r + RB; rp < kRows; rp += RB) zero_row((size_t)hv * kRows + rp);
  if (rg_row >= a.M) {   // the last group's rows past M (M > 32 only)
    zero_row(ro);
    return;
  }
  const int S = a.splits;
  const size_t base = (size_t)hv * S * kRows;

  // Issue the first PF partial-a loads of this thread (they need no weights yet)
  // together with every split's statistics: one memory round trip.
  const int cg = tid % CG, sg = tid / CG;
  const bool sum_lane = sg < SG;
  const float* pa = a.part.a + (base + r) * DP + cg * 4;
  float4 av[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int s = sg + SG * k;
    av[k] = (sum_lane && s < S) ? *reinterpret_cast<const float4*>(pa + (size_t)s * kRows * DP)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  uint64_t best = 0u;
  uint32_t badl = 0u;
  for (int s = tid; s < S; s += kThreads) {
    const size_t o = base + (size_t)s * kRows + r;
    const float ms = a.part.m2[o];
    sm_m2[s] = ms;
    sm_S[s] = a.part.S[o];
    sm_Sx[s] = a.part.Sx[o];
    sm_j[s] = a.part.jstar[o];
    const int bd = a.part.bad[o];
    sm_bad[s] = bd;
    badl |= (bd & 1) ? 1u : 0u;
    const uint64_t k = split_key(ms, sm_j[s]);
    best = best > k ? best : k;
  }
  best = wave_max_u64(best);
  if (lane == 0) rk[wid] = best;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) best = best > rk[w] ? best : rk[w];
  const float M = from_max_key((uint32_t)(best >> 32));
  const bool have = M > -INFINITY;
  // the split holding the winning token (tokens are distinct across splits),
  // and whether it is flagged
  if (tid == 0) { s_star = -1; s_flag = 0; }
  __syncthreads();
  if (have)
    for (int s = tid; s < S; s += kThreads)
      if (sm_m2[s] > -INFINITY && split_key(sm_m2[s], sm_j[s]) == best) {
        s_star = s;
        s_flag = (sm_bad[s] & 2) ? 1 : 0;
      }
  __syncthreads();
  const int sstar = have ? s_star : -1;
  int jst = (sstar >= 0) ? sm_j[sstar] : -1;
  uint32_t bad = 0u;
  if (jst < 0 || jst >= a.n) { jst = -1; bad = 1u; }
  // the row takes the exact arg-max term (helpers sum the winning split again);
  // decided exactly as the helpers decide it
  const bool fix = sstar >= 0 && jst >= 0 && s_flag != 0;
  // the arg-max token's value row, needed at the end
  const float vstar = (tid < a.d && jst >= 0) ? bf2f(a.v[(size_t)g * a.hs + (size_t)jst * a.d + tid]) : 0.f;

  // split weights f_s = 2^(m2_s - M) and the normaliser with and without the
  // arg-max split (fixed-order sums)
  float Sf = 0.f, Sxo = 0.f;
  for (int s = tid; s < S; s += kThreads) {
    const float ms = sm_m2[s];
    const float f = (ms > -INFINITY) ? ex2(ms - M) : 0.f;
    sm_f[s] = f;
    Sf += sm_S[s] * f;
    if (s != sstar) Sxo += sm_S[s] * f;
  }
  Sf = wave_sum_dpp(Sf);
  Sxo = wave_sum_dpp(Sxo);
  badl = wave_or_dpp(badl);
  if (lane == 0) { rf[0][wid] = Sf; rf[1][wid] = Sxo; ro_[0][wid] = badl; }
  __syncthreads();
  Sf = 0.f; Sxo = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) { Sf += rf[0][w]; Sxo += rf[1][w]; bad |= ro_[0][w]; }
  const float Sx = have ? sm_Sx[sstar] + Sxo : 0.f;

  // a = sum_s f_s a_s / S, and for a flagged row also the sum without the
  // arg-max's split: each thread sums its column group over its splits
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acx = acc;
  if (sum_lane) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int s = sg + SG * k;
      const float f = s < S ? sm_f[s] : 0.f;
      const float fx = s != sstar ? f : 0.f;
      acc.x += av[k].x * f; acc.y += av[k].y * f; acc.z += av[k].z * f; acc.w += av[k].w * f;
      acx.x += av[k].x * fx; acx.y += av[k].y * fx; acx.z += av[k].z * fx; acx.w += av[k].w * fx;
    }
    for (int s = sg + SG * PF; s < S; s += SG) {
      const float4 x = *reinterpret_cast<const float4*>(pa + (size_t)s * kRows * DP);
      const float f = sm_f[s];
      const float fx = s != sstar ? f : 0.f;
      acc.x += x.x * f; acc.y += x.y * f; acc.z += x.z * f; acc.w += x.w * f;
      acx.x += x.x * fx; acx.y += x.y * fx; acx.z += x.z * fx; acx.w += x.w * fx;
    }
    red4[sg * CG + cg] = acc;
  }
  __syncthreads();
  const float invS = 1.f / Sf;
  float an2 = 0.f, dist = 0.f;
  uint32_t nonfin = 0u;
  if (tid < DP) {
    const float* rr = reinterpret_cast<const float*>(red4);
    float tt = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) tt += rr[k * DP + tid];
    // columns >= d hold products with padding rows of V: they are zero by definition
    const float avv = tid < a.d ? tt * invS : 0.f;
    if (!(fabsf(avv) <= FLT_MAX)) nonfin = 1u;
    an2 = avv * avv;
    const __bf16 hi = (__bf16)avv;
    const __bf16 lo = (__bf16)(avv - (float)hi);
    a.rs.a_hi[ro * DP + tid] = __builtin_bit_cast(u16, hi);
    a.rs.a_lo[ro * DP + tid] = __builtin_bit_cast(u16, lo);
    // a - v_j* (zero past d); a flagged row's comes from the exact sum instead
    if (!fix) a.rs.ares[ro * DP + tid] = avv - vstar;
    // row r of head g is window query (g * G + r / w, r % w): [Hq][w][d] order
    if (a.out_a && tid < a.d) a.out_a[((size_t)g * a.M + rg_row) * a.d + tid] = avv;
    if (tid < a.d && jst >= 0) {
      const float df = avv - vstar;
      dist = df * df;
    }
  }
  an2 = wave_sum_dpp(an2);
  dist = wave_sum_dpp(dist);
  nonfin = wave_or_dpp(nonfin);
  if (lane == 0) { rf[2][wid] = an2; tmp[wid] = dist; ro_[1][wid] = nonfin; }
  __syncthreads();
  an2 = 0.f; dist = 0.f; nonfin = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) { an2 += rf[2][w]; dist += tmp[w]; nonfin |= ro_[1][w]; }
  nonfin |= bad | (!(Sf <= FLT_MAX) ? 1u : 0u) | (!have ? 1u : 0u);
  const bool singular = !nonfin && !(Sx > 0x1p-53f);
  if (tid == 0) {
    a.rs.m2[ro] = M;
    a.rs.S[ro] = Sf;
    a.rs.lse2[ro] = M + log2f(Sf);
    if (a.out_lse) a.out_lse[(size_t)g * a.M + rg_row] = (M + log2f(Sf)) * 0.6931471805599453f;
    a.rs.an2[ro] = an2;
    a.rs.jstar[ro] = jst;
    a.rs.fix[ro] = fix ? 1 : 0;
    if (!fix) a.rs.cstar[ro] = (nonfin || singular) ? 0.f : dist / (Sx * Sx);
    // a non-finite intermediate with finite inputs inside the contract cannot
    // occur: it is an overflow (the first pass latched any input out of range)
    const uint32_t bits = (nonfin ? LATCH_OVERFLOW : 0u) | (singular ? LATCH_SINGULAR : 0u);
    if (bits) atomicOr(a.latch, bits);
  }
  if (!fix) return;
  // the other splits' part of the exact sum, then count in with the helpers
  __syncthreads();   // red4 is reused
  if (sum_lane) red4[sg * CG + cg] = acx;
  __syncthreads();
  if (tid < DP) {
    const float* rr = reinterpret_cast<const float*>(red4);
    float ao = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) ao += rr[k * DP + tid];
    a.ex.ao[ro * DP + tid] = ao;
  }
  if (tid == 0) {
    float* meta = a.ex.meta + ro * 4;
    meta[0] = Sf; meta[1] = Sx; meta[2] = Sxo; meta[3] = __int_as_float(jst);
  }
  if (arrive_last(a.ex.cnt + ro, (uint32_t)a.xh + 1u, &s_flag)) {
    if (tid == 0) { crows[0] = r; cjs[0] = jst; }
    __syncthreads();
    exclusion_combine<DP>(a, hv, crows, cjs, 1, lds.c.dsq, csxs, cmeta);
  }
}

// ----------------------------------------------------------------- pass 2 --
// S = Q K^T and A V^T (rows x tokens): lane l owns token l%32 and 16 rows; the
// sum over rows stays within the lane pair.  Raw scores of the chunk and its
// pooling halo go to LDS, then the workgroup pools and protects them.
constexpr int kMaxRadius = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS of pass 2 for R row groups: per group the Q, a_hi and a_lo rows, then per
// group and row lse, ||a||^2, the arg-max token and its term, then the chunk's
// raw scores with the pooling halo.
template <int DP>
constexpr size_t pass2_group_bytes() {
  return (size_t)3 * kRows * RowLayout<DP>::ROWB;
}
template <int DP>
constexpr bool pass2_vlds() { return kP2VLds && DP <= 128 && !kP2Overlap; }
template <int DP>
constexpr size_t pass2_lds_base(int R) {
  return (size_t)R * pass2_group_bytes<DP>() + (size_t)R * 4 * kRows * 4 +
         (size_t)(kChunk2 + 2 * kMaxRadius + kTile) * 4;
}
// ... and, with V through LDS, one V tile slot per wave
template <int DP>
constexpr size_t pass2_lds_bytes(int R) {
  return pass2_lds_base<DP>(R) + (pass2_vlds<DP>() ? (size_t)kWaves * kRows * RowLayout<DP>::ROWB : 0);
}

// ||a - v||^2 summed directly for one (row, token): the row's a is held as its
// arg-max token's value row c = v_j* (bf16, from the cache) plus the fp32
// difference ares = a - v_j*, so a - v = ares + (c - v), where c - v of two bf16
// values is exact in fp32.  Used where the expansion could have cancelled
// (value rows near a, e.g. copies of a dominant token's value row): a rare
// path.  `vchunk(c)` gives the token's value columns 8c .. 8c + 7; ares and c
// come from the row state and the cache (L2-resident), four chunks' loads in
// flight at a time.
template <int DP, typename VChunk>
__device__ __forceinline__ float direct_dist(const float* __restrict__ ares,
                                             const u16* __restrict__ crow, int d, VChunk vchunk) {
  constexpr int CH = DP / 8, U = 4;
  float s = 0.f;
#pragma unroll 1
  for (int c0 = 0; c0 < CH; c0 += U) {
    u32x4 cx[U];
    float4 r0[U], r1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u, CH - 1);
      cx[u] = *reinterpret_cast<const u32x4*>(crow + 8 * min(c, d / 8 - 1));
      r0[u] = *reinterpret_cast<const float4*>(ares + 8 * c);
      r1[u] = *reinterpret_cast<const float4*>(ares + 8 * c + 4);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      if (c >= CH || 8 * c >= d) break;
      const bf16x8 vx = vchunk(c);
      const u32x4 cw = cx[u];
      const float rv[8] = {r0[u].x, r0[u].y, r0[u].z, r0[u].w, r1[u].x, r1[u].y, r1[u].z, r1[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = cw[e >> 1];
        const float ce = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
        const float x = rv[e] + (ce - (float)vx[e]);
        s = fmaf(x, x, s);
      }
    }
  }
  return s;
}

// NB8: 8-row blocks of the row group that can hold window rows (rows >= M have
// p = 0 and are skipped in the per-row vector work): 4 in general, 1 for an
// instance launched only when G * w <= 8 (multi-head attention with w <= 8).
template <int DP, bool FULLD, int NB8 = 4>
__global__ __launch_bounds__(kThreads, (DP <= 128 ? kP2Waves : 1)) void pass2_kernel(ScoreArgs a) {
  using L = RowLayout<DP>;
  constexpr int NC = DP / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int R = a.R;
  float* lse_s = reinterpret_cast<float*>(smem_raw + (size_t)R * pass2_group_bytes<DP>());
  float* an2_s = lse_s + R * kRows;
  int* js_s = reinterpret_cast<int*>(an2_s + R * kRows);   // arg-max token per row
  float* cs_s = reinterpret_cast<float*>(js_s + R * kRows);  // and its precomputed term
  float* rawbuf = cs_s + R * kRows;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int64_t n = a.n;
  const int g = blockIdx.x / a.chunks2, ch = blockIdx.x % a.chunks2;
  const int64_t c0 = (int64_t)ch * a.chunk2_len, c1 = min(n, c0 + a.chunk2_len);
  const int rad = (a.pool - 1) / 2;
  const int64_t e0 = max((int64_t)0, c0 - rad), e1 = min(n, c1 + rad);
  const int next = (int)((e1 - e0 + kTile - 1) / kTile);
  const int d = FULLD ? DP : a.d;   // a compile-time constant in the full-width instance
  const u16* kg = a.k + (size_t)g * a.hs;
  const u16* vg = a.v + (size_t)g * a.hs;
  const int64_t all_see = n - a.w;

  for (int rg = 0; rg < R; ++rg) {
    unsigned char* qs = smem_raw + (size_t)rg * pass2_group_bytes<DP>();
    const size_t ro0 = ((size_t)g * R + rg) * kRows;   // this group's row state
    const int row0 = kRows * rg;
    // Q, a_hi, a_lo and the row state: every load issued before any store
    RowStage<DP> sq, sh, sl;
    sq.load(a.q + ((size_t)g * a.M + row0) * d, min(kRows, a.M - row0), d, d);
    sh.load(a.rs.a_hi + ro0 * DP, kRows, DP, DP);
    sl.load(a.rs.a_lo + ro0 * DP, kRows, DP, DP);
    // rows >= M carry lse = +inf (set by the merge): their p and contribution are 0
    float lse = 0.f, an2 = 0.f, cst = 0.f;
    int jsv = 0;
    if (tid < kRows) {
      lse = a.rs.lse2[ro0 + tid];
      an2 = a.rs.an2[ro0 + tid];
      jsv = a.rs.jstar[ro0 + tid];
      cst = a.rs.cstar[ro0 + tid];
    }
    sq.store(qs);
    sh.store(qs + kRows * L::ROWB);
    sl.store(qs + 2 * kRows * L::ROWB);
    if (tid < kRows) {
      lse_s[rg * kRows + tid] = lse;
      an2_s[rg * kRows + tid] = an2;
      js_s[rg * kRows + tid] = jsv;
      cs_s[rg * kRows + tid] = cst;
    }
  }
  const float invG = 1.f / (float)a.G;
  uint32_t flags = 0;
  // the merge has read this KV head's flags: clear them for the next call
  if (ch == 0 && tid < R) a.ex.head[(size_t)g * R + tid] = 0u;
  __syncthreads();   // the staged rows and their state, for every wave

  auto issue = [&](int t, bf16x8 (&kk)[NC], bf16x8 (&vv)[NC]) {
    const int64_t t0 = e0 + (int64_t)t * kTile;
    load_kv_tile<NC, FULLD>(kg, vg, t0 + r, t0 + r < e1, t0 + kTile > e1, hh, d, kk, vv);
  };
  // Each wave walks its tiles in order.  By default (d <= 128) a tile's K and V
  // rows arrive in whole-line non-temporal loads and pass through the wave's
  // LDS slot into operand layout; the other waves of the CU (two workgroups)
  // cover the latency.  With the overlap option (register operands loaded
  // directly) the next tile's K and V are loaded into the same registers as
  // soon as the matrix products have consumed them.  Every row group of the
  // head uses the same K/V tile.
  bf16x8 kB[NC], vB[NC];
  us2 mg = {0, 0};   // largest magnitude bits of the keys read here (the input check)
  if (kP2Overlap && wid < next) issue(wid, kB, vB);
  for (int t = wid; t < next; t += kWaves) {
    const int64_t j0 = e0 + (int64_t)t * kTile;
    const int64_t tok = j0 + r;
    const bool tok_ok = tok < e1;
    if constexpr (pass2_vlds<DP>()) {
      // V in whole-line loads, through this wave's slot into operand layout
      unsigned char* vslot = smem_raw + pass2_lds_base<DP>(R) + (size_t)wid * kRows * L::ROWB;
      u32x4 vr[L::CHP / 2];
      if constexpr (kP2KLds) {
        // K the same way first, through the same slot
        u32x4 kr[L::CHP / 2];
        load_v_tile<DP, true, !FULLD, kNTP2K>(kg, j0, e1, d, lane, kr);
        load_v_tile<DP, true, !FULLD>(vg, j0, e1, d, lane, vr);
        store_v_tile<DP>(vslot, lane, kr);
        wave_sync_lds();
#pragma unroll
        for (int c = 0; c < NC; ++c) kB[c] = lds8<DP>(vslot, r, 2 * c + hh);
        wave_sync_lds();
      } else {
        load_k_tile<NC, FULLD>(kg, tok, tok_ok, j0 + kTile > e1, hh, d, kB);
        load_v_tile<DP, true, !FULLD>(vg, j0, e1, d, lane, vr);
      }
      store_v_tile<DP>(vslot, lane, vr);
      wave_sync_lds();
#pragma unroll
      for (int c = 0; c < NC; ++c) vB[c] = lds8<DP>(vslot, r, 2 * c + hh);
      wave_sync_lds();
    } else if (!kP2Overlap) {
      issue(t, kB, vB);
    }
    float vn2 = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      mg = mag_max4(mg, __builtin_bit_cast(u32x4, kB[c]));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 x2 = {vB[c][2 * e], vB[c][2 * e + 1]};
        vn2 = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, vn2, false);
      }
    }
    vn2 += __shfl_xor(vn2, 32);
    const bool interior = (j0 + kTile <= e1) && (j0 + kTile - 1 <= all_see);
    float tsum = 0.f;   // this token's sum over every row of the head
#pragma unroll 1
    for (int rg = 0; rg < R; ++rg) {
      const unsigned char* qs = smem_raw + (size_t)rg * pass2_group_bytes<DP>();
      const unsigned char* hs = qs + kRows * L::ROWB;
      const unsigned char* ls = hs + kRows * L::ROWB;
      // four independent accumulation chains (logits split in two, a.v split
      // into its hi and lo parts) keep the matrix core busy
      f32x16 sacc, sacc1, av, av1;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; sacc1[v] = 0.f; av[v] = 0.f; av1[v] = 0.f; }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c & 1) sacc1 = mfma32(lds8<DP>(qs, r, 2 * c + hh), kB[c], sacc1);
        else sacc = mfma32(lds8<DP>(qs, r, 2 * c + hh), kB[c], sacc);
        av = mfma32(lds8<DP>(hs, r, 2 * c + hh), vB[c], av);
        av1 = mfma32(lds8<DP>(ls, r, 2 * c + hh), vB[c], av1);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] += sacc1[v]; av[v] += av1[v]; }
      float cc[16];
#pragma unroll
      for (int v = 4 * NB8; v < 16; ++v) cc[v] = 0.f;
      float ovf = 0.f;   // becomes NaN if an expansion term overflowed fp32
      uint32_t near = 0u;   // elements whose distance is summed directly (bit v)
#pragma unroll
      for (int q4 = 0; q4 < NB8; ++q4) {
        // this lane's rows 8*q4 + 4*hh + 0..3 of the group
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + rg * kRows + 8 * q4 + 4 * hh);
        const float4 n4 = *reinterpret_cast<const float4*>(an2_s + rg * kRows + 8 * q4 + 4 * hh);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float nv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * q4 + i;
          const float p = ex2(sacc[v] * a.scale_log2 - lv[i]);
          const float odds = p * __builtin_amdgcn_rcpf(1.f - p);
          const float o2 = odds * odds;
          const float d0 = nv[i] - 2.f * av[v] + vn2;
          ovf = fmaf(d0, 0.f, ovf);
          // the expansion is kept where it cannot have cancelled (or where the
          // contribution is zero anyway); the rest get o2 now, the distance later
          const bool cancel = o2 > 0.f && d0 < kCancelFrac * (nv[i] + vn2);
          near |= cancel ? 1u << v : 0u;
          cc[v] = cancel ? o2 : o2 * fmaxf(d0, 0.f);
        }
      }
      if (tok_ok && !(ovf == 0.f)) flags |= LATCH_RANGE;
      if (!interior) {
        const int itok = (int)tok;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rv = kRows * rg + 8 * (v >> 2) + 4 * hh + (v & 3);   // row within the head
          const int lim = rv < a.M ? (int)(n - a.w + (rv % a.w)) : -1;
          const bool ok = tok_ok && itok <= lim;
          cc[v] = ok ? cc[v] : 0.f;
          near &= ok ? ~0u : ~(1u << v);
        }
      }
      // the arg-max token of a row takes the value computed by the merge instead
      const int jsl = (lane < kRows) ? js_s[rg * kRows + lane] : -1;
      const bool hit = (jsl >= j0) && (jsl < j0 + kTile);
      uint64_t bal = __ballot(hit);
      while (bal) {
        const int rr = __ffsll((unsigned long long)bal) - 1;
        bal &= bal - 1;
        const int js = js_s[rg * kRows + rr];
        const float cs = cs_s[rg * kRows + rr];
        const int Ln = (int)(js - j0) + 32 * ((rr >> 2) & 1);
        const int vr = 4 * (rr >> 3) + (rr & 3);
        if (lane == Ln && tok_ok) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (v == vr) cc[v] = cs;
          near &= ~(1u << vr);
        }
      }
      if (__builtin_expect(__any(near != 0u), 0)) {
        // value rows close to a (other than the arg-max's own): the exact
        // distance for each such element
        const size_t ro0 = ((size_t)g * R + rg) * kRows;
        while (near) {
          const int v = __builtin_ctz(near);
          near &= near - 1u;
          const int rho = 8 * (v >> 2) + 4 * hh + (v & 3);   // row within the group
          const int js = js_s[rg * kRows + rho];
          // (a row without an arg-max is a rejected input: nothing to read)
          float dist = 0.f;
          if (js >= 0) {
            const float* ar = a.rs.ares + (ro0 + rho) * DP;
            const u16* cr = vg + (size_t)js * d;
            if constexpr (pass2_vlds<DP>()) {
              // this token's value row is still in the wave's LDS slot
              const unsigned char* vslot =
                  smem_raw + pass2_lds_base<DP>(R) + (size_t)wid * kRows * L::ROWB;
              dist = direct_dist<DP>(ar, cr, d, [&](int c) { return lds8<DP>(vslot, r, c); });
            } else {
              const u16* vrow = vg + (size_t)tok * d;
              dist = direct_dist<DP>(ar, cr, d, [&](int c) {
                return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow + 8 * c));
              });
            }
          }
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (u == v) cc[u] *= dist;
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) sum += cc[v];
      sum += __shfl_xor(sum, 32);
      tsum += sum;
    }
    if (kP2Overlap && t + kWaves < next) issue(t + kWaves, kB, vB);
    const float raw = tsum * invG;
    // inputs were checked finite by pass 1 / merge, so an inf or NaN here is an
    // fp32 overflow of a score or of its terms
    if (tok_ok && !(raw <= FLT_MAX)) flags |= LATCH_RANGE;
    if (hh == 0 && tok_ok) rawbuf[tok - e0] = raw;
  }
  __syncthreads();
  if (a.hist1) {
    // score + select: the chunk's final scores also go into the selection's
    // first-digit histogram -- 16-bit counts, two per word, in the staging
    // region (free after the tiles), then one device-scope add per non-empty bin
    uint32_t* h32 = reinterpret_cast<uint32_t*>(smem_raw);
    for (int i = tid; i < kBins1 / 2; i += kThreads) h32[i] = 0u;
    __syncthreads();
    for (int64_t j = c0 + tid; j < c1; j += kThreads) {
      const int64_t lo = max((int64_t)0, j - rad), hi = min(n - 1, j + rad);
      float mx = rawbuf[lo - e0];
      for (int64_t i = lo + 1; i <= hi; ++i) mx = fmaxf(mx, rawbuf[i - e0]);
      const float sv = (j >= n - a.w) ? INFINITY : mx + 0.f;
      a.scores[(size_t)g * n + j] = sv;
      const uint32_t bin = order_key(sv) >> 20;
      atomicAdd(h32 + (bin >> 1), (bin & 1u) ? 0x10000u : 1u);
    }
    __syncthreads();
    uint32_t* gh = a.hist1 + (size_t)g * a.hist1_stride;
    for (int i = tid; i < kBins1 / 2; i += kThreads) {
      const uint32_t c2 = h32[i];
      if (c2 & 0xffffu) atomicAdd(gh + 2 * i, c2 & 0xffffu);
      if (c2 >> 16) atomicAdd(gh + 2 * i + 1, c2 >> 16);
    }
  } else {
    for (int64_t j = c0 + tid; j < c1; j += kThreads) {
      const int64_t lo = max((int64_t)0, j - rad), hi = min(n - 1, j + rad);
      float mx = rawbuf[lo - e0];
      for (int64_t i = lo + 1; i <= hi; ++i) mx = fmaxf(mx, rawbuf[i - e0]);
      a.scores[(size_t)g * n + j] = (j >= n - a.w) ? INFINITY : mx + 0.f;
    }
  }
  if (flags) atomicOr(a.latch, flags);
  latch_inputs(a.latch, mg);
}

// -------------------------------------------------------- attention-only --
// Attention-only scores, the pages' SnapKV comparison ("paper tables",
// Table 14: MaxPool over the window-summed attention weights; "paper digest",
// App. B: same observation window and pooling as DropKV).  Pass A is pass 1
// without V: per (head, split) the running maximum and normaliser of every row.
// Pass B turns the split states into each row's log-sum-exp (fixed order),
// recomputes the logits, adds p over the rows of each token, divides by G and
// pools / protects like pass 2.  Only K is read, twice.
template <int DP, bool FULLD>
__global__ __launch_bounds__(kThreads, (DP <= 128 ? kAttnWaves : 2)) void attn_pass1_kernel(ScoreArgs a) {
  constexpr int NC = DP / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ float sm_m[kWaves][kRows], sm_S[kWaves][kRows];
  __shared__ int sm_bad[kWaves][kRows];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int hv = blockIdx.x / a.splits, s = split_deal(blockIdx.x % a.splits, a.splits);   // (KV head, row group)
  const int g = hv / a.R, row0 = kRows * (hv % a.R);
  const SplitTiles sp(a.n, s, a.splits, a.split_len);
  const int64_t jend = sp.jend;
  const int ntiles = sp.ntiles;
  const int d = FULLD ? DP : a.d;   // a compile-time constant in the full-width instance
  const u16* kg = a.k + (size_t)g * a.hs;
  const bool row_ok = row0 + r < a.M;
  const int64_t causal = row_ok ? a.n - a.w + ((row0 + r) % a.w) : -1;
  const int64_t all_see = a.n - a.w;
  unsigned char* qs = smem_raw;
  us2 mg = {0, 0};   // largest magnitude bits of the Q and K elements loaded here
  {
    RowStage<DP> qst;
    qst.load(a.q + ((size_t)g * a.M + row0) * d, min(kRows, a.M - row0), d, d);
#pragma unroll
    for (int k = 0; k < RowStage<DP>::IT; ++k) mg = mag_max4(mg, qst.x[k]);
    qst.store(qs);
  }
  __syncthreads();

  // S^T = K Q^T as in pass 1: lane l owns row l%32 and 16 of the tile's tokens
  float m = -INFINITY, S = 0.f, chk = 0.f;
  // kAttnTiles tiles per iteration: all their loads are issued before the first
  // is consumed (more bytes in flight per wave); the tiles are still visited in
  // the order t, t + 4, t + 8, ... so the result does not depend on it
  for (int t0 = wid; t0 < ntiles; t0 += kWaves * kAttnTiles) {
    bf16x8 kk[kAttnTiles][NC];
#pragma unroll
    for (int u = 0; u < kAttnTiles; ++u) {
      const int t = t0 + u * kWaves;
      const int64_t j0 = sp.start(t);
      if (t < ntiles) load_k_tile<NC, FULLD>(kg, j0 + r, j0 + r < jend, j0 + kTile > jend, hh, d, kk[u]);
    }
#pragma unroll
    for (int u = 0; u < kAttnTiles; ++u) {
    const int t = t0 + u * kWaves;
    if (t >= ntiles) break;
    const int64_t j0 = sp.start(t);
    f32x16 st, st1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { st[v] = 0.f; st1[v] = 0.f; }
#pragma unroll
    for (int c = 0; c < NC; c += 2) {
      st = mfma32(kk[u][c], lds8<DP>(qs, r, 2 * c + hh), st);
      if (c + 1 < NC) st1 = mfma32(kk[u][c + 1], lds8<DP>(qs, r, 2 * c + 2 + hh), st1);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) mg = mag_max4(mg, __builtin_bit_cast(u32x4, kk[u][c]));
    const bool interior = (j0 + kTile <= jend) && (j0 + kTile - 1 <= all_see);
    float s2[16];
    float lm = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x = st[v] + st1[v];
      const int64_t tv = j0 + 8 * (v >> 2) + 4 * hh + (v & 3);
      const bool valid = interior || (row_ok && tv < jend && tv <= causal);
      if (valid) chk = fmaf(x, 0.f, chk);   // becomes NaN on any inf / NaN logit
      s2[v] = valid ? x * a.scale_log2 : -INFINITY;
      lm = fmaxf(lm, s2[v]);
    }
    lm = fmaxf(lm, __shfl_xor(lm, 32));
    const float mn = fmaxf(m, lm);
    if (mn > -INFINITY) {
      const float alpha = ex2(m - mn);   // 0 while nothing was seen (S = 0 then)
      float ts = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) ts += ex2(s2[v] - mn);
      ts += __shfl_xor(ts, 32);
      S = S * alpha + ts;
      m = mn;
    }
    }
  }
  int bad = (chk == 0.f) ? 0 : 1;
  bad |= __shfl_xor(bad, 32);
  latch_inputs(a.latch, mg);
  if (hh == 0) {
    sm_m[wid][r] = m;
    sm_S[wid][r] = S;
    sm_bad[wid][r] = bad;
  }
  __syncthreads();
  if (tid < kRows) {   // combine the waves' states of row tid (fixed order)
    float Mf = -INFINITY;
    int badf = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { Mf = fmaxf(Mf, sm_m[w][tid]); badf |= sm_bad[w][tid]; }
    float Sf = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      Sf += (sm_m[w][tid] > -INFINITY) ? sm_S[w][tid] * ex2(sm_m[w][tid] - Mf) : 0.f;
    const size_t pb = ((size_t)hv * a.splits + s) * kRows + tid;
    a.part.m2[pb] = Mf;
    a.part.S[pb] = Sf;
    a.part.bad[pb] = badf;
  }
}

template <int DP>
constexpr size_t attn_pass2_base(int R) {
  return (size_t)R * kRows * RowLayout<DP>::ROWB + (size_t)(kChunk2 + 2 * kMaxRadius + kTile) * 4;
}
template <int DP>
constexpr size_t attn_pass2_lds_bytes(int R) {
  return attn_pass2_base<DP>(R);
}

template <int DP, bool FULLD, int NB8 = 4>   // NB8 as in pass2_kernel
__global__ __launch_bounds__(kThreads, (DP <= 128 ? kAttnWaves : 2)) void attn_pass2_kernel(ScoreArgs a) {
  constexpr int NC = DP / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ float lse_s[kMaxRowGroups * kRows];
  const int R = a.R;
  float* rawbuf = reinterpret_cast<float*>(smem_raw + (size_t)R * kRows * RowLayout<DP>::ROWB);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int64_t n = a.n;
  const int g = blockIdx.x / a.chunks2, ch = blockIdx.x % a.chunks2;
  const int64_t c0 = (int64_t)ch * a.chunk2_len, c1 = min(n, c0 + a.chunk2_len);
  const int rad = (a.pool - 1) / 2;
  const int64_t e0 = max((int64_t)0, c0 - rad), e1 = min(n, c1 + rad);
  const int next = (int)((e1 - e0 + kTile - 1) / kTile);
  const int d = FULLD ? DP : a.d;   // a compile-time constant in the full-width instance
  const u16* kg = a.k + (size_t)g * a.hs;
  const int64_t all_see = n - a.w;

  for (int rg = 0; rg < R; ++rg)
    stage_rows<DP>(smem_raw + (size_t)rg * kRows * RowLayout<DP>::ROWB,
                   a.q + ((size_t)g * a.M + kRows * rg) * d, min(kRows, a.M - kRows * rg), d, d);
  for (int rg = 0; rg < R; ++rg) {   // each row's log2-sum-exp from the split states: 8 threads per row take
      // every 8th split (online max/sum), then a fixed shuffle tree combines them
    const int row = tid >> 3, part = tid & 7;
    const size_t base = ((size_t)g * R + rg) * a.splits * kRows + row;
    float M = -INFINITY, Ssum = 0.f;
    int bad = 0;
    // batches of eight splits: all their loads requested, then combined in
    // split order (one memory round trip per batch, not per split)
    constexpr int SB = 8;
    for (int sp0 = part; sp0 < a.splits; sp0 += 8 * SB) {
      float msv[SB], ssv[SB];
      int bv[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int sp = sp0 + 8 * u;
        const bool ok = sp < a.splits;
        const size_t o = base + (size_t)(ok ? sp : 0) * kRows;   // split 0 always exists
        msv[u] = a.part.m2[o];
        ssv[u] = a.part.S[o];
        bv[u] = a.part.bad[o];
        if (!ok) { msv[u] = -INFINITY; ssv[u] = 0.f; bv[u] = 0; }
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const float ms = msv[u], ss = ssv[u];
        bad |= bv[u];
        if (ms > M) {
          Ssum = Ssum * ex2(M - ms) + ss;
          M = ms;
        } else if (ms > -INFINITY) {
          Ssum += ss * ex2(ms - M);
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float Mo = __shfl_xor(M, o), So = __shfl_xor(Ssum, o);
      bad |= __shfl_xor(bad, o);
      const float Mn = fmaxf(M, Mo);
      const float x = (M > -INFINITY) ? Ssum * ex2(M - Mn) : 0.f;
      const float y = (Mo > -INFINITY) ? So * ex2(Mo - Mn) : 0.f;
      // the lower lane of the pair adds first, so both lanes hold the same sum
      Ssum = ((tid & o) == 0) ? x + y : y + x;
      M = Mn;
    }
    const int hrow = kRows * rg + row;   // row within the head
    if (part == 0) {
      // rows >= M have no query: lse = +inf makes every p of theirs 0
      lse_s[hrow] = (hrow < a.M && M > -INFINITY) ? M + log2f(Ssum) : INFINITY;
      if (hrow < a.M && (bad || !(M > -INFINITY) || !(Ssum <= FLT_MAX)) && ch == 0)
        atomicOr(a.latch, LATCH_OVERFLOW);   // an overflow: inputs were checked by pass A
    }
  }
  __syncthreads();
  const float invG = 1.f / (float)a.G;

  // S = Q K^T as in pass 2: lane l owns token l%32 and 16 rows; kAttnTiles
  // tiles' loads are issued before the first is consumed
  for (int t0 = wid; t0 < next; t0 += kWaves * kAttnTiles) {
    bf16x8 kB[kAttnTiles][NC];
#pragma unroll
    for (int u = 0; u < kAttnTiles; ++u) {
      const int t = t0 + u * kWaves;
      const int64_t j0 = e0 + (int64_t)t * kTile;
      if (t < next) load_k_tile<NC, FULLD>(kg, j0 + r, j0 + r < e1, j0 + kTile > e1, hh, d, kB[u]);
    }
#pragma unroll
    for (int u = 0; u < kAttnTiles; ++u) {
    const int t = t0 + u * kWaves;
    if (t >= next) break;
    const int64_t j0 = e0 + (int64_t)t * kTile;
    const int64_t tok = j0 + r;
    const bool tok_ok = tok < e1;
    const bool interior = (j0 + kTile <= e1) && (j0 + kTile - 1 <= all_see);
    float sum = 0.f;
#pragma unroll 1
    for (int rg = 0; rg < R; ++rg) {
      const unsigned char* qs = smem_raw + (size_t)rg * kRows * RowLayout<DP>::ROWB;
      f32x16 sacc, sacc1;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; sacc1[v] = 0.f; }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c & 1) sacc1 = mfma32(lds8<DP>(qs, r, 2 * c + hh), kB[u][c], sacc1);
        else sacc = mfma32(lds8<DP>(qs, r, 2 * c + hh), kB[u][c], sacc);
      }
#pragma unroll
      for (int q4 = 0; q4 < NB8; ++q4) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + kRows * rg + 8 * q4 + 4 * hh);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * q4 + i;
          float p = ex2((sacc[v] + sacc1[v]) * a.scale_log2 - lv[i]);
          if (!interior) {
            const int rv = kRows * rg + 8 * q4 + 4 * hh + i;   // row within the head
            const int64_t lim = rv < a.M ? n - a.w + (rv % a.w) : -1;
            p = (tok_ok && tok <= lim) ? p : 0.f;
          }
          sum += p;
        }
      }
    }
    sum += __shfl_xor(sum, 32);
    if (hh == 0 && tok_ok) rawbuf[tok - e0] = sum * invG;
    }
  }
  __syncthreads();
  for (int64_t j = c0 + tid; j < c1; j += kThreads) {
    const int64_t lo = max((int64_t)0, j - rad), hi = min(n - 1, j + rad);
    float mx = rawbuf[lo - e0];
    for (int64_t i = lo + 1; i <= hi; ++i) mx = fmaxf(mx, rawbuf[i - e0]);
    a.scores[(size_t)g * n + j] = (j >= n - a.w) ? INFINITY : mx + 0.f;
  }
}

// Dynamic LDS above the 64 KB default is granted per kernel, raised as needed.
template <auto KERN>
static hipError_t grant_lds(size_t bytes) {
  static size_t granted = 65536;
  if (bytes <= granted) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) granted = bytes;
  return e;
}

// The second pass's instance: one 8-row block when G * w <= 8 (d <= 128).
template <int DP, bool FULLD, template <int, bool, int> class K>
static hipError_t launch_second(const ScoreArgs& a, size_t lds, hipStream_t s) {
  if constexpr (DP <= 128) {
    if (a.M <= 8) {
      hipError_t e = grant_lds<K<DP, FULLD, 1>::fn>(lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((K<DP, FULLD, 1>::fn), dim3((unsigned)a.Hkv * a.chunks2), dim3(kThreads), lds, s, a);
      return hipGetLastError();
    }
  }
  hipError_t e = grant_lds<K<DP, FULLD, 4>::fn>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((K<DP, FULLD, 4>::fn), dim3((unsigned)a.Hkv * a.chunks2), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}
template <int DP, bool FULLD, int NB8>
struct Pass2K { static constexpr auto fn = pass2_kernel<DP, FULLD, NB8>; };
template <int DP, bool FULLD, int NB8>
struct AttnPass2K { static constexpr auto fn = attn_pass2_kernel<DP, FULLD, NB8>; };

template <int DP, bool FULLD>
static hipError_t launch_attn_dp(void* ctx, const ScoreArgs& a, hipStream_t s) {
  const size_t lds1 = (size_t)kRows * RowLayout<DP>::ROWB;
  const size_t lds2 = attn_pass2_lds_bytes<DP>(a.R);
  prof_begin(ctx, "attn_pass1", s);
  hipLaunchKernelGGL((attn_pass1_kernel<DP, FULLD>), dim3(a.Hkv * a.R * a.splits), dim3(kThreads),
                     lds1, s, a);
  prof_end(ctx, "attn_pass1", s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(ctx, "attn_pass2", s);
  e = launch_second<DP, FULLD, AttnPass2K>(a, lds2, s);
  prof_end(ctx, "attn_pass2", s);
  return e;
}

template <int DP>
static hipError_t launch_attn_d(void* ctx, const ScoreArgs& a, hipStream_t s) {
  return a.d == DP ? launch_attn_dp<DP, true>(ctx, a, s) : launch_attn_dp<DP, false>(ctx, a, s);
}

bool score_hist_fits(int DP, int R) {
  // the histogram overlays the row groups' staging (Q, a_hi, a_lo rows)
  size_t gb = 0;
  switch (DP) {
    case 32: gb = pass2_group_bytes<32>(); break;
    case 64: gb = pass2_group_bytes<64>(); break;
    case 96: gb = pass2_group_bytes<96>(); break;
    case 128: gb = pass2_group_bytes<128>(); break;
    case 160: gb = pass2_group_bytes<160>(); break;
    case 192: gb = pass2_group_bytes<192>(); break;
    case 224: gb = pass2_group_bytes<224>(); break;
    case 256: gb = pass2_group_bytes<256>(); break;
    default: return false;
  }
  return (size_t)R * gb >= (size_t)kBins1 / 2 * 4;
}

// Whether pass 2's LDS (the row groups' Q / a rows and the chunk buffer) fits a
// workgroup for this padded head dimension and number of row groups.
bool score_fits(int DP, int R) {
  constexpr size_t kLdsMax = 160 * 1024;
  switch (DP) {
    case 32: return pass2_lds_bytes<32>(R) <= kLdsMax;
    case 64: return pass2_lds_bytes<64>(R) <= kLdsMax;
    case 96: return pass2_lds_bytes<96>(R) <= kLdsMax;
    case 128: return pass2_lds_bytes<128>(R) <= kLdsMax;
    case 160: return pass2_lds_bytes<160>(R) <= kLdsMax;
    case 192: return pass2_lds_bytes<192>(R) <= kLdsMax;
    case 224: return pass2_lds_bytes<224>(R) <= kLdsMax;
    case 256: return pass2_lds_bytes<256>(R) <= kLdsMax;
    default: return false;
  }
}

hipError_t launch_score_attention(void* ctx, const ScoreArgs& a, hipStream_t s) {
  switch (a.DP) {
    case 32: return launch_attn_d<32>(ctx, a, s);
    case 64: return launch_attn_d<64>(ctx, a, s);
    case 96: return launch_attn_d<96>(ctx, a, s);
    case 128: return launch_attn_d<128>(ctx, a, s);
    case 160: return launch_attn_d<160>(ctx, a, s);
    case 192: return launch_attn_d<192>(ctx, a, s);
    case 224: return launch_attn_d<224>(ctx, a, s);
    case 256: return launch_attn_d<256>(ctx, a, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------- host side --
int plan_splits(int64_t n, int Hkv, int64_t* split_len, int target) {
  // about `target` workgroups over the chip, at least 256 tokens each.
  int64_t want = (target + Hkv - 1) / Hkv;
  const int64_t max_by_len = (n + 255) / 256;
  if (want > max_by_len) want = max_by_len;
  if (want > kMaxSplits) want = kMaxSplits;
  if (want < 1) want = 1;
  int64_t len = (n + want - 1) / want;
  len = (len + kTile - 1) / kTile * kTile;
  *split_len = len;
  return (int)((n + len - 1) / len);
}

int plan_chunks2(int64_t n, int Hkv, int64_t* chunk_len, int target) {
  // about `target` workgroups over the chip, whole tiles, at most kChunk2 tokens
  int64_t want = (target + Hkv - 1) / Hkv;
  if (want < 1) want = 1;
  int64_t len = (n + want - 1) / want;
  len = (len + kTile - 1) / kTile * kTile;
  if (len < 256) len = 256;
  if (len > kChunk2) len = kChunk2;
  *chunk_len = len;
  return (int)((n + len - 1) / len);
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t score_scratch_bytes(int Hkv, int splits, int DP, int xh) {
  const size_t prow = (size_t)Hkv * splits * kRows;
  const size_t rrow = (size_t)Hkv * kRows;
  return align256(prow * 4) * 5 + align256(prow * DP * 4) + align256(rrow * 4) * 7 +
         align256(rrow * DP * 2) * 2 + align256(rrow * DP * 4) +
         align256(rrow * xh * DP * 4) + align256(rrow * xh * 4) + align256(rrow * DP * 4) +
         align256(rrow * 4 * 4) + align256(rrow * 4) + align256((size_t)Hkv * 4);
}

void carve_scratch(void* base, int Hkv, int splits, int DP, int xh, Partials* p, RowState* rs,
                   ExclScratch* ex) {
  char* c = static_cast<char*>(base);
  const size_t prow = (size_t)Hkv * splits * kRows;
  const size_t rrow = (size_t)Hkv * kRows;
  auto take = [&](size_t bytes) { char* x = c; c += align256(bytes); return x; };
  p->m2 = (float*)take(prow * 4);
  p->S = (float*)take(prow * 4);
  p->Sx = (float*)take(prow * 4);
  p->jstar = (int*)take(prow * 4);
  p->bad = (int*)take(prow * 4);
  p->a = (float*)take(prow * DP * 4);
  rs->m2 = (float*)take(rrow * 4);
  rs->lse2 = (float*)take(rrow * 4);
  rs->S = (float*)take(rrow * 4);
  rs->an2 = (float*)take(rrow * 4);
  rs->cstar = (float*)take(rrow * 4);
  rs->jstar = (int*)take(rrow * 4);
  rs->fix = (int*)take(rrow * 4);
  rs->a_hi = (u16*)take(rrow * DP * 2);
  rs->a_lo = (u16*)take(rrow * DP * 2);
  rs->ares = (float*)take(rrow * DP * 4);
  ex->part = (float*)take(rrow * xh * DP * 4);
  ex->sx = (float*)take(rrow * xh * 4);
  ex->ao = (float*)take(rrow * DP * 4);
  ex->meta = (float*)take(rrow * 4 * 4);
  ex->cnt = (uint32_t*)take(rrow * 4);
  ex->head = (uint32_t*)take((size_t)Hkv * 4);   // right after cnt: one zeroed range
}

int plan_helpers(int64_t n, int Hv, int splits) {
  const int64_t tiles = ((n + kTile - 1) / kTile + splits - 1) / splits;   // per split
  int64_t xh = (tiles + 7) / 8;   // two tiles per wave of a helper
  const int64_t cap = 1024 / Hv;
  if (xh > cap) xh = cap;
  if (xh > kMaxHelpers) xh = kMaxHelpers;
  if (xh < 1) xh = 1;
  return (int)xh;
}

template <int DP, bool FULLD>
static hipError_t launch_score_dp(void* ctx, const ScoreArgs& a, hipStream_t s) {
  const size_t red = (size_t)p1_waves(DP) * kRows * (DP + 1) * 4;   // the combine's slabs
  const size_t lds1 = pass1_lds_bytes<DP>() > red ? pass1_lds_bytes<DP>() : red;
  const size_t lds2 = pass2_lds_bytes<DP>(a.R);
  hipError_t e = grant_lds<pass1_kernel<DP, FULLD>>(lds1);
  if (e != hipSuccess) return e;
  prof_begin(ctx, "pass1", s);
  hipLaunchKernelGGL((pass1_kernel<DP, FULLD>), dim3(a.Hkv * a.R * a.splits), dim3(64 * p1_waves(DP)),
                     lds1, s, a);
  prof_end(ctx, "pass1", s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(ctx, "merge", s);
  // xh helpers per (KV head, row group), then the row workgroups
  hipLaunchKernelGGL(merge_kernel<DP>,
                     dim3(a.Hkv * a.R * ((a.M < kRows ? a.M : kRows) + a.xh)), dim3(kThreads), 0, s,
                     a);
  prof_end(ctx, "merge", s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(ctx, "pass2", s);
  e = launch_second<DP, FULLD, Pass2K>(a, lds2, s);
  prof_end(ctx, "pass2", s);
  return e;
}

template <int DP>
static hipError_t launch_score_d(void* ctx, const ScoreArgs& a, hipStream_t s) {
  return a.d == DP ? launch_score_dp<DP, true>(ctx, a, s) : launch_score_dp<DP, false>(ctx, a, s);
}

hipError_t launch_score(void* ctx, const ScoreArgs& a, hipStream_t s) {
  switch (a.DP) {
    case 32: return launch_score_d<32>(ctx, a, s);
    case 64: return launch_score_d<64>(ctx, a, s);
    case 96: return launch_score_d<96>(ctx, a, s);
    case 128: return launch_score_d<128>(ctx, a, s);
    case 160: return launch_score_d<160>(ctx, a, s);
    case 192: return launch_score_d<192>(ctx, a, s);
    case 224: return launch_score_d<224>(ctx, a, s);
    case 256: return launch_score_d<256>(ctx, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dropkv
