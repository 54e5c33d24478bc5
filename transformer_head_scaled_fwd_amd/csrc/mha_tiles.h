// mha_tiles.h -- device building blocks shared by the attention kernels for
// gfx950: buffer resources, the lane-pair reductions, LDS swizzles, the K/V
// tile ring filled by buffer->LDS direct loads, and the per-wave phases of
// one key block (scores on MFMA, mask, distance bias, weights, PV on MFMA).
//
// Layout conventions (see the kernels for the full picture): a wave owns 32
// query rows; score tiles are S^T (keys on the MFMA M axis, queries on N), so
// lane l holds query row l % 32 and keys {8g + 4(l/32) + r} of a 32-key tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mha {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 32;
constexpr int BC = 64;  // keys per block
// The running max used for exp2 is raised only when a row's max exceeds it
// by more than TAU (log2 units), so right after a raise the unnormalised
// weights stay below 2^TAU.  (The forward kernel forms the block max only
// when a weight could exceed 2^16; see its key walk.)
constexpr float TAU = 8.0f;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the kernels' result stores (the aux operand of the buffer
// store builtins): sc0 | sc1, written through to memory instead of being
// held dirty in the XCD's L2 until the kernel ends.  Results are read by the
// next kernel or the host, not by this one.  It pays when a launch's
// results fit the L2s (8 x 4 MB): held there, they are written back at the
// end of the kernel, after its last workgroup, which lengthens short
// launches by several microseconds.  Results well beyond the L2s leave it
// during the kernel anyway, and writing them through costs more than it
// saves (measured on the weights pass, with the non-temporal bit as well:
// 17-34 MB of output 7-11% faster, 67-134 MB 3-5% slower).  The
// non-temporal bit (nt) would make the short launches a little faster
// still, but the kernel that reads the results next then finds them further
// away (the multi-head layer's output projection after the core: the layer
// 3% slower instead of 3% faster).
constexpr int kStoreOut = 1 | 16;
constexpr int64_t kStreamOutMaxBytes = (int64_t)48 << 20;

#define MHA_INLINE __device__ static inline __attribute__((always_inline))
#define MHA_MEMBER __device__ inline __attribute__((always_inline))

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// A result store at byte offset off of r: written through (kStoreOut) or
// with the default policy.
__device__ inline void store_result(u32x4 v, __amdgpu_buffer_rsrc_t r, int off, bool stream) {
  if (stream) __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreOut);
  else __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ inline void store_result(u32x2 v, __amdgpu_buffer_rsrc_t r, int off, bool stream) {
  if (stream) __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStoreOut);
  else __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ inline void store_result(uint32_t v, __amdgpu_buffer_rsrc_t r, int off, bool stream) {
  if (stream) __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStoreOut);
  else __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ inline void store_result(uint16_t v, __amdgpu_buffer_rsrc_t r, int off, bool stream) {
  if (stream) __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kStoreOut);
  else __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// max / sum of x over lanes l and l^32 (the two lanes that share a query
// row).  v_permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second; called with (x, x) each lane receives
// both its own value and its partner's, in an order that depends on the
// half, so only symmetric combinations are formed from the pair.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// LDS swizzles of 16-byte chunks for a row of D elements of type T.
template <typename T, int D>
struct Swz {
  static constexpr bool BF16 = sizeof(T) == 2;
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // chunks per row: 8, 16 or 32
  // K is read by rows j = 0..31 of one 16-byte column chunk per MFMA
  // operand: make the chunk position differ across 16 consecutive rows.
  __device__ static inline int k(int r) { return CPR == 8 ? ((r >> 1) & 7) : (r & 15); }
  // V, bf16: the transpose read touches rows 4h..4h+3 x 4 chunks per 32 lanes;
  // fp32: 32 consecutive elements of rows j and j+4.
  __device__ static inline int v(int r) {
    if constexpr (BF16) return CPR == 8 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
    else return 8 * ((r >> 2) & 1);
  }
};

// Tile geometry and LDS ring.  ES: element bytes; NW: waves per workgroup;
// KS: key groups per workgroup (the waves form NW / KS row groups of 32
// query rows, and key group g of a row group takes the g-th of every KS
// consecutive key blocks, so one ring stage holds KS blocks).
template <typename T, int D, int NW, int KS = 1>
struct Geo {
  using S = Swz<T, D>;
  static constexpr int ES = sizeof(T);
  static constexpr bool BF16 = (ES == 2);
  static constexpr int RG = NW / KS;            // row groups
  static constexpr int BR = kRowsPerWave * RG;  // query rows per workgroup
  static constexpr int ROWB = D * ES;           // bytes per K or V row in LDS
  static constexpr int CPR = ROWB / 16;         // chunks per row
  static constexpr int TILE = KS * BC * ROWB;   // KS K or V blocks (one ring stage)
  static_assert(NW % KS == 0, "waves must split evenly into key groups");
  // Two stages: a block is loaded one block ahead of its use.  (A third
  // stage, loading two blocks ahead, measured slower: the loads already land
  // within one block's compute, and the ring index costs more.)
  static constexpr int NSTAGE = 2;
  static constexpr int DIST = NSTAGE - 1;              // how many blocks ahead loads run
  static constexpr int LDS_BYTES = NSTAGE * 2 * TILE;  // K ring, then V ring
  // direct-load instructions per wave for one tile (each moves 1 KiB)
  static constexpr int LOADS = TILE / 1024 / NW;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads per wave");

  // Direct loads of one ring stage of keys or values (rows KS * BC * kb
  // onwards, rows at or beyond `bytes` read as 0) into the tile at LDS
  // address `tile`.  Load u of a wave fills bytes [1 KiB * (u * NW + wave),
  // +1 KiB) of the tile; lane t writes the 16 bytes at +16t, i.e. chunk
  // position pc of row r, which holds global chunk pc ^ swizzle(r).  The
  // swizzles repeat every 16 rows, so each BC-row block of a stage is laid
  // out as a stand-alone tile would be.
  //
  // The stage's first row goes into the buffer resource (base advanced,
  // record count shortened, so rows past `bytes` still read as 0): base,
  // bytes and kb are uniform, so this is scalar work, and each lane's
  // offset is the same for every stage, computed once.
  //
  // The loads are issued from inline assembly (M0 set in the same statement)
  // so that the compiler's wait-count pass does not treat every later LDS
  // read as a possible reader of this tile and wait for the loads there;
  // the kernel waits for them explicitly before the barrier that publishes
  // the tile.
  //
  // STREAM marks the loads non-temporal (nt), for rows that no other
  // workgroup reads again: a decode step's cache rows.
  template <bool IS_K, bool STREAM = false>
  __device__ static inline void stage(uint32_t tile, const T* base, uint32_t bytes, int kb,
                                      int wave, int lane) {
    // (readfirstlane states the uniformity, so that the resource is built
    // in scalar registers, as the instruction requires.)
    const uint32_t start = (uint32_t)kb * (uint32_t)TILE;
    const uint64_t addr = (uint64_t)(uintptr_t)base + start;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    // bytes and start stay below 2^31 (a head is under 2 GiB): a signed
    // difference clamped at 0, which the scalar unit has instructions for.
    const int rest = (int)bytes - (int)start;
    const uint32_t left = __builtin_amdgcn_readfirstlane((uint32_t)(rest > 0 ? rest : 0));
    const auto rs = make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), left);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int slot = (u * NW + wave) * 64;  // first chunk of this load
      const int q = slot + lane;
      const int r = q / CPR, pc = q % CPR;
      const uint32_t off = ((uint32_t)r * D) * ES + (pc ^ (IS_K ? S::k(r) : S::v(r))) * 16;
      if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :: "s"(tile + slot * 16), "v"(off), "s"(rs) : "memory");
      else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(tile + slot * 16), "v"(off), "s"(rs) : "memory");
    }
  }

  // Wait until at most `n` direct loads of this thread are in flight.
  template <int n>
  __device__ static inline void wait_loads() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(n) : "memory");
  }
};

// The phases of one key block for one wave (32 query rows).
template <typename T, int D>
struct Phase {
  using S = Swz<T, D>;
  static constexpr bool BF16 = sizeof(T) == 2;
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int NS = BC / 32;                 // 32-key score tiles per block
  static constexpr int NQF = BF16 ? D / 16 : D / 8;  // 16-byte Q fragments per lane
  // P as the PV MFMA consumes it: bf16 slices of 16 keys, or fp32 tiles.
  using PFrag = std::conditional_t<BF16, bf16x8[BC / 16], f32x16[NS]>;

  // Q fragments of this lane's query row, the B operand of S^T = K Q^T.
  // bf16: slice s covers features 16s..16s+15, lane holds 8 of them.
  // fp32: step s pairs feature s (lanes 0-31) with feature D/2 + s (lanes 32-63).
  // The loads are completed here: otherwise the in-order memory counter
  // makes every later wait for a prefetch also wait for them.
  MHA_INLINE void load_q(u32x4 (&qf)[NQF], __amdgpu_buffer_rsrc_t rq, int row, int hi) {
    issue_q(qf, rq, row, hi);
    pin_q(qf);
  }
  // The two halves of load_q, for a caller that issues other loads between
  // them: the Q loads, then an empty use that makes the compiler wait for them.
  MHA_INLINE void issue_q(u32x4 (&qf)[NQF], __amdgpu_buffer_rsrc_t rq, int row, int hi) {
    constexpr int ES = (int)sizeof(T);
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      const uint32_t col = BF16 ? (16 * s + 8 * hi) : (4 * s + (D / 2) * hi);
      qf[s] = load16(rq, ((uint32_t)row * D + col) * ES);
    }
  }
  MHA_INLINE void pin_q(const u32x4 (&qf)[NQF]) {
#pragma unroll
    for (int s = 0; s < NQF; ++s) asm volatile("" : : "v"(qf[s]));
  }

  // S^T[j][i] for the BC keys of the tile at kt.
  MHA_INLINE void scores(f32x16 (&s)[NS], const char* kt, const u32x4 (&qf)[NQF], int li, int hi) {
#pragma unroll
    for (int jt = 0; jt < NS; ++jt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[jt][e] = 0.0f;
      const int j = jt * 32 + li;
      const char* krow = kt + j * ROWB;
      const int sw = S::k(j);
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(krow + ((2 * ks + hi) ^ sw) * 16);
          s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ks]), s[jt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < D / 8; ++q4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(krow + ((q4 + (D / 8) * hi) ^ sw) * 16);
          const f32x4 bq = __builtin_bit_cast(f32x4, qf[q4]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], bq[e], s[jt], 0, 0, 0);
        }
      }
    }
  }

  // The score MFMAs with the lane's K operand offsets precomputed: ko[ks] is
  // the byte offset, within a 64-key tile, of this lane's 16-byte chunk of
  // feature slice ks (row li, swizzled); rows 32jt + li add 32jt rows.  The
  // empty asm makes each offset opaque, so that the compiler keeps the sums
  // in registers instead of re-adding their two parts in every block.
  static constexpr int NKO = BF16 ? D / 16 : D / 8;
  MHA_INLINE void k_offsets(uint32_t (&ko)[NKO], int li, int hi) {
    const int sw = S::k(li);
#pragma unroll
    for (int ks = 0; ks < NKO; ++ks) {
      ko[ks] = (uint32_t)(li * ROWB + ((BF16 ? (2 * ks + hi) : (ks + (D / 8) * hi)) ^ sw) * 16);
      asm volatile("" : "+v"(ko[ks]));
    }
  }
  // With INIT every tile's accumulators start from *c0 instead of 0 (the
  // MFMA adds its accumulator input, so a per-element term costs no vector
  // ALU).
  template <bool INIT = false>
  MHA_INLINE void scores_ko(f32x16 (&s)[NS], const char* kt, const u32x4 (&qf)[NQF],
                            const uint32_t (&ko)[NKO], const f32x16* c0 = nullptr) {
    static_assert(BF16, "precomputed K offsets: bf16 tiles");
#pragma unroll
    for (int jt = 0; jt < NS; ++jt) {
      if constexpr (INIT) {
        s[jt] = *c0;
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[jt][e] = 0.0f;
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt + jt * 32 * ROWB + ko[ks]);
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ks]), s[jt], 0, 0, 0);
      }
    }
  }

  // Schedule of the score MFMAs: keep the K operand reads four MFMAs ahead
  // of their use (the compiler's own schedule issues them about two ahead,
  // which leaves the MFMAs waiting on LDS latency).
  MHA_INLINE void prefetch_k() {
    if constexpr (BF16) {
      constexpr int NM = NS * (D / 16);  // score MFMAs = K operand reads
      constexpr int AHEAD = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }

  // -inf where the key is invalid.  The lane holds keys
  // 32jt + 8g + 4hi + r of the block; `lim` is the first invalid key of the
  // row minus the block's first key minus 4hi.
  //
  // Two spellings of the same selects, which the compiler lowers
  // differently: the conditional store becomes 32 compares into separate
  // lane masks joined by a chain of scalar ORs, then 32 selects; the select
  // expression becomes compare / wait / select triples on VCC.  The second
  // measured 1-3% faster on the d = 64 launches (three waves per SIMD) and
  // 1-2% slower on the four-wave d = 128 causal ones (two waves per SIMD,
  // where the scalar ORs run beside the other wave's vector work); the
  // results are the same bits.
  MHA_INLINE void mask(f32x16 (&s)[NS], int lim) {
#pragma unroll
    for (int jt = 0; jt < NS; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool out = 32 * jt + 8 * g + r >= lim;
          if constexpr (D == 64) s[jt][4 * g + r] = out ? -__builtin_inff() : s[jt][4 * g + r];
          else if (out) s[jt][4 * g + r] = -__builtin_inff();
        }
  }

  // Linear distance bias (ALiBi, "第2章：完整的 Transformer 架构" §5.3): the
  // scaled score of (i, j) loses slope * |p_i - j|.  Scores here are raw
  // dot products (the scale is applied with log2 e in the exponent), so the
  // raw score loses sr * |p_i - j| with sr = slope / scale.  `base` is
  // p_i - (first key of the block) - 4hi; the lane's key offsets within the
  // block are the constants 32jt + 8g + r, so every distance is exact.
  MHA_INLINE void bias(f32x16 (&s)[NS], float base, float sr) {
#pragma unroll
    for (int jt = 0; jt < NS; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dist = __builtin_fabsf(base - (float)(32 * jt + 8 * g + r));
          s[jt][4 * g + r] = __builtin_fmaf(-sr, dist, s[jt][4 * g + r]);
        }
  }

  // This lane's maximum over its keys of the block (before the pair exchange).
  MHA_INLINE float lane_max(const f32x16 (&s)[NS]) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < NS; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jt][e]);
    return mx;
  }
  // The same over the lane's keys of one 32-key tile.
  MHA_INLINE float tile_max(const f32x16& s) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
    return mx;
  }

  // p = 2^(s * scale * log2e - msub[jt]) for the keys of score tile jt,
  // rounded to the PV operand type; the lane's share of the row sum
  // accumulates the rounded values.
  //
  // bf16: slice k (16 keys, k = 0..3) takes tile jt = k/2, groups
  // g = 2(k%2) and 2(k%2)+1: lane half hi holds keys 16k + 4hi + r (k-slots
  // 8hi + r) and 16k + 8 + 4hi + r (k-slots 8hi + 4 + r), r = 0..3.
  MHA_INLINE void weights(PFrag& pf, const f32x16 (&s)[NS], float sl2, const float (&msub)[NS],
                          float& l) {
    if constexpr (BF16) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int k = 0; k < BC / 16; ++k) {
        const int jt = k / 2, g0 = 2 * (k % 2);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int g = g0 + e / 4, r = e % 4;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r], sl2, -msub[jt]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r + 1], sl2, -msub[jt]));
          const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
          l = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l, false);
          pf[k][e] = pk[0];
          pf[k][e + 1] = pk[1];
        }
      }
    } else {
#pragma unroll
      for (int jt = 0; jt < NS; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][e], sl2, -msub[jt]));
          pf[jt][e] = p;
          l += p;
        }
    }
  }
  // The same subtrahend for every tile.
  MHA_INLINE void weights(PFrag& pf, const f32x16 (&s)[NS], float sl2, float msub, float& l) {
    float ms[NS];
#pragma unroll
    for (int jt = 0; jt < NS; ++jt) ms[jt] = msub;
    weights(pf, s, sl2, ms, l);
  }

  // O^T += V^T P^T for the value tile at vt.
  MHA_INLINE void pv(f32x16 (&o)[D / 32], const char* vt, const PFrag& pf, int lane) {
    const int li = lane % 32, hi = lane / 32;
    if constexpr (BF16) {
      // V^T operand through the LDS transpose read: in each 16-lane group
      // lanes 4k'..4k'+3 read 16 consecutive features of key row k', and
      // lane t receives feature t of the four rows.  Group gi = lane/16
      // covers features 16(gi%2)..+15 of the 32-feature tile and keys of
      // lane half gi/2 (= hi).
      const int gi = lane / 16, t16 = lane % 16, kr = t16 / 4, qq = t16 % 4;
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        const int cc = ct * 4 + 2 * (gi % 2) + qq / 2;  // 16-byte chunk of the 4 features
#pragma unroll
        for (int k = 0; k < BC / 16; ++k) {
          bf16x8 a;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int row = 16 * k + 8 * half + 4 * hi + kr;
            const char* p = vt + row * ROWB + ((cc ^ S::v(row)) * 16) + (qq % 2) * 8;
            const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(p));
            const bf16x4 b4 = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * half + e] = b4[e];
          }
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[k], o[ct], 0, 0, 0);
        }
      }
    } else {
      // fp32: one MFMA per accumulator element; k-slot hi of the step
      // (jt, g, r) is key 32jt + 8g + 4hi + r, read as a single element of
      // the row-major V tile.
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        const int c = ct * 32 + li;
#pragma unroll
        for (int jt = 0; jt < NS; ++jt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 32 * jt + 8 * g + 4 * hi + r;
              const float a = *reinterpret_cast<const float*>(
                  vt + row * ROWB + (((c / 4) ^ S::v(row)) * 16) + (c % 4) * 4);
              o[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf[jt][4 * g + r], o[ct], 0, 0, 0);
            }
      }
    }
  }

  // An empty use of the weights: the compiler must produce them here, which
  // keeps their computation in the same basic block as the PV MFMAs instead
  // of sinking it past the rescale branch.
  MHA_INLINE void pin(const PFrag& pf) {
    if constexpr (BF16) {
#pragma unroll
      for (int k = 0; k < BC / 16; ++k) asm volatile("" : : "v"(pf[k]));
    } else {
#pragma unroll
      for (int jt = 0; jt < NS; ++jt) asm volatile("" : : "v"(pf[jt]));
    }
  }
};

}  // namespace mha
