// mha_fwd_kernel.hip -- fused attention forward for gfx950 (MI355X).
//
// One workgroup computes BR = 32 * NW query rows of one (batch, head): NW
// wave64s, each owning 32 rows.  It walks the key axis in blocks of BC = 64
// keys.  Per block:
//
//   stage    K and V blocks -> LDS, row-major, by buffer->LDS direct loads
//            (no register staging), in a ring of NSTAGE stages so that a
//            block streams in one or two blocks ahead of its use; one
//            barrier per block;
//   scores   S^T = K Q^T on MFMA (32x32 tiles, fp32 accumulate), Q held in
//            registers for the whole walk;
//   mask     -inf where j >= L_b or (causal and j > i)
//            ("Transformer: 详解" §3.4, §5.3);
//   softmax  online: running row max and sum in fp32, exp2 with the scale
//            and log2(e) folded into one FMA, rescale of the output only when
//            the row max grew by more than 2^TAU ("Transformer" wiki page:
//            mixed precision needs the blockwise, online softmax);
//   PV       O^T += V^T P^T on MFMA with P rounded to the input dtype; the V
//            operand comes straight from the row-major tile through the
//            LDS transpose read (ds_read_b64_tr_b16).
//
// The n x m score matrix exists only as register tiles and never reaches
// memory ("Transformer: 详解" §8.2: the n^2 score/weight matrices are what
// limits long contexts).  The epilogue divides by the row sum (0 for rows
// with no valid key) and stores O once.
//
// Computing S^T and O^T (keys / features on the MFMA M axis, queries on N)
// puts one query row in each lane: in the 32x32 accumulator lane l holds
// column l % 32 and rows {8g + 4(l/32) + r}.  Row max and row sum are then
// in-lane reductions plus one exchange between lane halves, the P^T
// accumulator feeds the PV MFMA as its B operand without leaving registers,
// and the rescale factor of a row is a per-lane scalar.
//
// The key walk is software-pipelined by one block: iteration kb issues the
// score MFMAs of block kb+1, then the PV MFMAs of block kb while the vector
// ALU computes the max, rescale factor and weights of block kb+1.
//
// LDS tiles are stored in 16-byte chunks with the chunk index XOR-ed by a
// function of the row ("swizzle"), chosen per read pattern so that the lanes
// of one LDS read cycle hit distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mha_launch.h"

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
// by more than TAU (log2 units), so unnormalised weights stay below 2^TAU.
constexpr float TAU = 8.0f;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

#define MHA_INLINE __device__ static inline __attribute__((always_inline))
#define MHA_MEMBER __device__ inline __attribute__((always_inline))

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
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

// Tile geometry and LDS ring.  ES: element bytes; NW: waves per workgroup.
template <typename T, int D, int NW>
struct Geo {
  using S = Swz<T, D>;
  static constexpr int ES = sizeof(T);
  static constexpr bool BF16 = (ES == 2);
  static constexpr int BR = kRowsPerWave * NW;  // query rows per workgroup
  static constexpr int ROWB = D * ES;           // bytes per K or V row in LDS
  static constexpr int CPR = ROWB / 16;         // chunks per row
  static constexpr int TILE = BC * ROWB;        // one K or one V block
  // Two stages: a block is loaded one block ahead of its use.  (A third
  // stage, loading two blocks ahead, measured slower: the loads already land
  // within one block's compute, and the ring index costs more.)
  static constexpr int NSTAGE = 2;
  static constexpr int DIST = NSTAGE - 1;              // how many blocks ahead loads run
  static constexpr int LDS_BYTES = NSTAGE * 2 * TILE;  // K ring, then V ring
  // direct-load instructions per wave for one tile (each moves 1 KiB)
  static constexpr int LOADS = TILE / 1024 / NW;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads per wave");

  // Direct loads of one key or value block (block kb, rows at or beyond
  // `bytes` read as 0) into the tile at LDS address `tile`.  Load u of a
  // wave fills bytes [1 KiB * (u * NW + wave), +1 KiB) of the tile; lane t
  // writes the 16 bytes at +16t, i.e. chunk position pc of row r, which
  // holds global chunk pc ^ swizzle(r).
  //
  // The loads are issued from inline assembly (M0 set in the same statement)
  // so that the compiler's wait-count pass does not treat every later LDS
  // read as a possible reader of this tile and wait for the loads there;
  // the kernel waits for them explicitly before the barrier that publishes
  // the tile.
  template <bool IS_K>
  __device__ static inline void stage(uint32_t tile, const T* base, uint32_t bytes, int kb,
                                      int wave, int lane) {
    const auto rs = make_rsrc(base, bytes);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int slot = (u * NW + wave) * 64;  // first chunk of this load
      const int q = slot + lane;
      const int r = q / CPR, pc = q % CPR;
      const uint32_t off =
          ((uint32_t)(kb * BC + r) * D) * ES + (pc ^ (IS_K ? S::k(r) : S::v(r))) * 16;
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
  MHA_INLINE void mask(f32x16 (&s)[NS], int lim) {
#pragma unroll
    for (int jt = 0; jt < NS; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * jt + 8 * g + r >= lim) s[jt][4 * g + r] = -__builtin_inff();
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

  // p = 2^(s * scale * log2e - msub), rounded to the PV operand type; the
  // lane's share of the row sum accumulates the rounded values.
  //
  // bf16: slice k (16 keys, k = 0..3) takes tile jt = k/2, groups
  // g = 2(k%2) and 2(k%2)+1: lane half hi holds keys 16k + 4hi + r (k-slots
  // 8hi + r) and 16k + 8 + 4hi + r (k-slots 8hi + 4 + r), r = 0..3.
  MHA_INLINE void weights(PFrag& pf, const f32x16 (&s)[NS], float sl2, float msub, float& l) {
    if constexpr (BF16) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int k = 0; k < BC / 16; ++k) {
        const int jt = k / 2, g0 = 2 * (k % 2);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int g = g0 + e / 4, r = e % 4;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r], sl2, -msub));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r + 1], sl2, -msub));
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
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][e], sl2, -msub));
          pf[jt][e] = p;
          l += p;
        }
    }
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

// Per-wave state of the key walk: 32 query rows, one per lane pair.
template <typename T, int D, int NW, bool CAUSAL>
struct Walk {
  using G = Geo<T, D, NW>;
  using P = Phase<T, D>;
  static constexpr int NS = P::NS;

  const char* ktiles;  // LDS: K ring, NSTAGE tiles
  const char* vtiles;  // LDS: V ring, NSTAGE tiles
  int lane, li, hi;
  int row_w;           // first query row of the wave
  int row_lim;         // first invalid key of this lane's row
  int L;               // valid keys of the sequence
  int wave_nkb;        // key blocks this wave reads
  float sl2;           // scale * log2(e)
  u32x4 qf[P::NQF];    // Q fragments
  f32x16 o[D / 32];    // O^T accumulator
  float m_run;         // running max of scale*log2(e)*s (per row)
  float l_run;         // this lane's share of the row sum

  MHA_MEMBER bool needs_mask(int kb) const {
    return (kb * BC + BC > L) || (CAUSAL && kb * BC + BC - 1 > row_w);
  }
  MHA_MEMBER const char* k_tile(int kb) const { return ktiles + (kb % G::NSTAGE) * G::TILE; }
  MHA_MEMBER const char* v_tile(int kb) const { return vtiles + (kb % G::NSTAGE) * G::TILE; }

  // Softmax bookkeeping for a block whose raw row max is mx: the running
  // max is raised only when the block max exceeds it by more than TAU.
  // Returns the factor alpha by which earlier sums and outputs must be
  // multiplied (1 when the max stays); the sum is rescaled here, the output
  // by the caller once the PV MFMAs that still add to it have been issued.
  MHA_MEMBER float raise_max(float mx, bool& grew) {
    const float mx2 = mx * sl2;  // -inf stays -inf (sl2 > 0)
    grew = mx2 > m_run + TAU;
    const float m_new = grew ? mx2 : m_run;
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    return alpha;
  }
  MHA_MEMBER void rescale_output(float alpha, bool grew) {
    if (__any(grew)) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
    }
  }
  MHA_MEMBER float msub() const { return (m_run == -__builtin_inff()) ? 0.0f : m_run; }

  // Scores, mask, running max and weights of the first block (prologue).
  MHA_MEMBER void first_block(typename P::PFrag& pf) {
    f32x16 s[NS];
    P::scores(s, k_tile(0), qf, li, hi);
    if (needs_mask(0)) P::mask(s, row_lim - 4 * hi);
    bool grew;
    raise_max(pair_max(P::lane_max(s)), grew);  // nothing accumulated yet
    P::weights(pf, s, sl2, msub(), l_run);
  }

  // PV of block kb (weights in pf_cur) and, when this wave reads block
  // kb+1, its scores, mask, running max and weights into pf_nxt.
  MHA_MEMBER void step(int kb, const typename P::PFrag& pf_cur, typename P::PFrag& pf_nxt) {
    if (kb + 1 < wave_nkb) {
      f32x16 s[NS];
      P::scores(s, k_tile(kb + 1), qf, li, hi);
      P::prefetch_k();
      if (needs_mask(kb + 1)) P::mask(s, row_lim - (kb + 1) * BC - 4 * hi);
      P::pv(o, v_tile(kb), pf_cur, lane);
      bool grew;
      const float alpha = raise_max(pair_max(P::lane_max(s)), grew);
      P::weights(pf_nxt, s, sl2, msub(), l_run);
      P::pin(pf_nxt);
      rescale_output(alpha, grew);
    } else {
      P::pv(o, v_tile(kb), pf_cur, lane);
    }
  }
};

template <typename T, int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW, 2)
attn_fwd_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp,
                const T* __restrict__ Vp, const int32_t* __restrict__ key_lens,
                T* __restrict__ Op, int H, int n, int m, int nqb, float scale_log2) {
  using G = Geo<T, D, NW>;
  using W = Walk<T, D, NW, CAUSAL>;
  using P = typename W::P;
  constexpr int ES = G::ES;
  constexpr bool BF16 = G::BF16;
  constexpr int BR = G::BR;
  constexpr int DIST = G::DIST;
  constexpr int LOADS = G::LOADS;
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES];
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);
  const uint32_t lds_k = lds_base;                        // K ring
  const uint32_t lds_v = lds_base + G::NSTAGE * G::TILE;  // V ring

  W w;
  w.ktiles = smem;
  w.vtiles = smem + G::NSTAGE * G::TILE;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  w.lane = tid % 64;
  w.li = w.lane % 32;  // query row within the wave's 32 (MFMA column)
  w.hi = w.lane / 32;  // which half of the k / row groups this lane holds
  const int lane = w.lane, li = w.li, hi = w.hi;

  // Heaviest query blocks first for causal attention: the work of a block
  // grows with its index, so launching them in reverse evens out the tail.
  const int BH = gridDim.x / nqb;
  const int bid = blockIdx.x;
  const int qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
  const int bh = bid % BH;
  const int b = bh / H;
  const int q0 = qb * BR;

  int L = m;
  if (key_lens != nullptr) {
    L = key_lens[b];
    L = L < 0 ? 0 : (L > m ? m : L);
  }
  w.L = L;
  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkb = (kend + BC - 1) / BC;
  w.row_w = q0 + wave * kRowsPerWave;
  const int my_row = w.row_w + li;
  // Key blocks any row of this wave can see.
  w.wave_nkb = CAUSAL ? min(nkb, (w.row_w + kRowsPerWave + BC - 1) / BC) : nkb;
  w.row_lim = CAUSAL ? min(L, my_row + 1) : L;
  w.sl2 = scale_log2;

  // Buffer resources: out-of-range loads read 0 (also into LDS) and
  // out-of-range stores are dropped, so rows >= n (queries) and >= L (keys,
  // values) need no branch and padded keys are never read from memory.
  const size_t head_q = (size_t)bh * (size_t)n * D;
  const size_t head_k = (size_t)bh * (size_t)m * D;
  const auto rq = make_rsrc(Qp + head_q, (uint32_t)n * D * ES);
  const uint32_t kv_bytes = (uint32_t)L * D * ES;  // rows >= L read as 0
  const auto ro = make_rsrc(Op + head_q, (uint32_t)n * D * ES);
  const T* kbase = Kp + head_k;
  const T* vbase = Vp + head_k;

  // Loads of key block j and value block j into their ring slots.
  auto load_k = [&](int j) {
    G::template stage<true>(lds_k + (j % G::NSTAGE) * G::TILE, kbase, kv_bytes, j, wave, lane);
  };
  auto load_v = [&](int j) {
    G::template stage<false>(lds_v + (j % G::NSTAGE) * G::TILE, vbase, kv_bytes, j, wave, lane);
  };

  // The first key/value blocks are requested before Q so that their memory
  // latency overlaps the Q loads.
  if (nkb > 0) {
    for (int j = 0; j <= DIST && j < nkb; ++j) load_k(j);
    for (int j = 0; j < DIST && j < nkb; ++j) load_v(j);
  }

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), kept in registers ----
  // bf16: slice s covers features 16s..16s+15, lane holds 8 of them.
  // fp32: step s pairs feature s (lanes 0-31) with feature D/2 + s (lanes 32-63).
#pragma unroll
  for (int s = 0; s < P::NQF; ++s) {
    uint32_t col = BF16 ? (16 * s + 8 * hi) : (4 * s + (D / 2) * hi);
    w.qf[s] = load16(rq, ((uint32_t)my_row * D + col) * ES);
  }
  // Complete the Q loads here: otherwise the in-order memory counter makes
  // every iteration of the key loop wait for its own prefetch as well.
#pragma unroll
  for (int s = 0; s < P::NQF; ++s) asm volatile("" : : "v"(w.qf[s]));

#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) w.o[t][e] = 0.0f;
  w.m_run = -__builtin_inff();
  w.l_run = 0.0f;

  // Pipeline: iteration kb reads K(kb+1) and V(kb).  It issues the loads of
  // K(kb+1+DIST) and V(kb+DIST), which go to the ring slots of K(kb) and
  // V(kb-1), both last read before the barrier that ended iteration kb-1.
  // Before its own barrier it waits for the loads issued DIST-1 iterations
  // earlier, i.e. for K(kb+2) and V(kb+1).  Two weight buffers alternate,
  // unrolled by two.
  typename P::PFrag pa, pb;
  if (nkb > 0) {
    G::template wait_loads<0>();
    __syncthreads();
    if (0 < w.wave_nkb) w.first_block(pa);
    __syncthreads();  // K(0) is consumed before its slot is refilled
  }

  // Issue this iteration's loads; returns how many tiles were issued.
  auto issue = [&](int kb) -> int {
    int issued = 0;
    if (kb + DIST < nkb) {
      load_v(kb + DIST);
      issued = 1;
      if (kb + 1 + DIST < nkb) {
        load_k(kb + 1 + DIST);
        issued = 2;
      }
    }
    return issued;
  };
  // Wait for the loads of DIST-1 iterations ago (leaving this iteration's in
  // flight when DIST is 2) and publish them with a barrier.
  auto publish = [&](int issued) {
    if constexpr (DIST == 1) {
      G::template wait_loads<0>();
    } else {
      if (issued == 2) G::template wait_loads<2 * LOADS>();
      else if (issued == 1) G::template wait_loads<LOADS>();
      else G::template wait_loads<0>();
    }
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    int issued = issue(kb);
    if (kb < w.wave_nkb) w.step(kb, pa, pb);
    publish(issued);
    if (kb + 1 >= nkb) break;
    issued = issue(kb + 1);
    if (kb + 1 < w.wave_nkb) w.step(kb + 1, pb, pa);
    publish(issued);
  }

  // ---- epilogue: divide by the row sum (0 when no key was valid), store
  const float l_tot = pair_sum(w.l_run);
  const float inv = (l_tot > 0.0f) ? (1.0f / l_tot) : 0.0f;
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = ((uint32_t)my_row * D + ct * 32 + 8 * g + 4 * hi) * ES;
      if constexpr (BF16) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(w.o[ct][4 * g + r] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), ro, (int)off, 0, 0);
      } else {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = w.o[ct][4 * g + r] * inv;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, (int)off, 0, 0);
      }
    }
}

template <typename T, int D, int NW, bool CAUSAL>
static hipError_t launch_one(const LaunchArgs& a) {
  constexpr int BR = Geo<T, D, NW>::BR;
  const int nqb = (int)((a.n + BR - 1) / BR);
  const int64_t blocks = (int64_t)nqb * a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, NW, CAUSAL>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                     (hipStream_t)a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V, a.key_lens,
                     (T*)a.O, (int)a.H, (int)a.n, (int)a.m, nqb, a.scale_log2);
  return hipGetLastError();
}

// Workgroup size: 8 waves (256 query rows, one workgroup per CU) for bf16
// with d = 128 when the query axis gives every CU several workgroups;
// otherwise 4 waves (128 rows, two workgroups per CU).
template <typename T, int D>
static hipError_t launch_d(const LaunchArgs& a) {
  if constexpr (D == 128 && sizeof(T) == 2) {
    const int64_t big_blocks = ((a.n + 255) / 256) * a.B * a.H;
    if (big_blocks >= 4 * 256)
      return a.causal ? launch_one<T, D, 8, true>(a) : launch_one<T, D, 8, false>(a);
  }
  return a.causal ? launch_one<T, D, 4, true>(a) : launch_one<T, D, 4, false>(a);
}

template <typename T>
static hipError_t launch_t(const LaunchArgs& a) {
  return a.d == 64 ? launch_d<T, 64>(a) : launch_d<T, 128>(a);
}

hipError_t launch_attention(const LaunchArgs& a) {
  return a.bf16 ? launch_t<__bf16>(a) : launch_t<float>(a);
}

}  // namespace mha
