// mha_fwd_kernel.hip -- fused attention forward for gfx950 (MI355X).
//
// One workgroup computes BR = 128 query rows of one (batch, head): four
// wave64s, each owning 32 rows.  It walks the key axis in blocks of BC = 64
// keys.  Per block:
//
//   stage    K and V blocks -> LDS, row-major, by buffer->LDS direct loads
//            (no register staging), double-buffered: block kb+1 streams in
//            while block kb is computed, one barrier per block;
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
// LDS tiles are stored in 16-byte chunks with the chunk index XOR-ed by a
// function of the row ("swizzle"), chosen per read pattern so that the lanes
// of one LDS read cycle hit distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int BR = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int BC = 64;                     // keys per block
// The running max used for exp2 is raised only when a row's max exceeds it
// by more than TAU (log2 units), so unnormalised weights stay below 2^TAU.
constexpr float TAU = 8.0f;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

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

// Tile geometry and LDS swizzles.  ES: element bytes; CPR: 16-byte chunks
// per row of D elements.
template <typename T, int D>
struct Geo {
  static constexpr int ES = sizeof(T);
  static constexpr bool BF16 = (ES == 2);
  static constexpr int ROWB = D * ES;          // bytes per K or V row in LDS
  static constexpr int CPR = ROWB / 16;        // chunks per row: 8, 16 or 32
  static constexpr int TILE = BC * ROWB;       // one K or one V block
  static constexpr int STAGE = 2 * TILE;       // K + V
  static constexpr int LDS_BYTES = 2 * STAGE;  // double-buffered
  // direct-load instructions per wave for one tile (each moves 1 KiB)
  static constexpr int LOADS = TILE / 1024 / kWaves;
  static_assert(TILE % (1024 * kWaves) == 0, "tile must split into 1 KiB loads per wave");

  // K is read by rows j = 0..31 of one 16-byte column chunk per MFMA
  // operand: make the chunk position differ across 16 consecutive rows.
  __device__ static inline int swz_k(int r) { return CPR == 8 ? ((r >> 1) & 7) : (r & 15); }
  // V, bf16: the transpose read touches rows 4h..4h+3 x 4 chunks per 32 lanes;
  // fp32: 32 consecutive elements of rows j and j+4.
  __device__ static inline int swz_v(int r) {
    if constexpr (BF16) return CPR == 8 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
    else return 8 * ((r >> 2) & 1);
  }

  // Direct loads of key/value block kb into LDS stage st.  Load u of a wave
  // fills LDS bytes [1 KiB * (u * kWaves + wave), +1 KiB) of each tile; lane
  // t writes the 16 bytes at +16t, i.e. chunk position pc of row r, which
  // holds global chunk pc ^ swizzle(r).  Rows at or beyond `bytes` read as 0.
  //
  // The loads are issued from inline assembly (M0 set in the same statement)
  // so that the compiler's wait-count pass does not treat every later LDS
  // read as a possible reader of this stage and wait for the loads there;
  // the kernel waits for them explicitly before the barrier that publishes
  // the stage.
  __device__ static inline void stage(uint32_t lds_base, const T* kbase, const T* vbase,
                                      uint32_t bytes, int kb, int st, int wave, int lane) {
    const auto rk = make_rsrc(kbase, bytes);
    const auto rv = make_rsrc(vbase, bytes);
    const uint32_t kt = lds_base + st * STAGE;
    const uint32_t vt = kt + TILE;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int slot = (u * kWaves + wave) * 64;  // first chunk of this load
      const int q = slot + lane;
      const int r = q / CPR, pc = q % CPR;
      const uint32_t row_off = ((uint32_t)(kb * BC + r) * D) * ES;
      const uint32_t koff = row_off + (pc ^ swz_k(r)) * 16;
      const uint32_t voff = row_off + (pc ^ swz_v(r)) * 16;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(kt + slot * 16), "v"(koff), "s"(rk) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(vt + slot * 16), "v"(voff), "s"(rv) : "memory");
    }
  }
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp,
                const T* __restrict__ Vp, const int32_t* __restrict__ key_lens,
                T* __restrict__ Op, int H, int n, int m, int nqb, float scale_log2) {
  using G = Geo<T, D>;
  constexpr int ES = G::ES;
  constexpr bool BF16 = G::BF16;
  __shared__ __attribute__((aligned(1024))) char smem[G::LDS_BYTES];
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int li = lane % 32;  // query row within the wave's 32 (MFMA column)
  const int hi = lane / 32;  // which half of the k / row groups this lane holds

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
  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkb = (kend + BC - 1) / BC;
  const int row_w = q0 + wave * kRowsPerWave;  // first row of this wave
  const int my_row = row_w + li;
  // Last key block any row of this wave can see.
  const int wave_nkb = CAUSAL ? min(nkb, (row_w + kRowsPerWave + BC - 1) / BC) : nkb;

  // Buffer resources: out-of-range loads read 0 (also into LDS) and
  // out-of-range stores are dropped, so rows >= n (queries) and >= L (keys,
  // values) need no branch and padded keys are never read from memory.
  const size_t head_q = (size_t)bh * (size_t)n * D;
  const size_t head_k = (size_t)bh * (size_t)m * D;
  const auto rq = make_rsrc(Qp + head_q, (uint32_t)n * D * ES);
  const uint32_t kv_bytes = (uint32_t)L * D * ES;  // rows >= L read as 0
  const auto ro = make_rsrc(Op + head_q, (uint32_t)n * D * ES);

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), kept in registers ----
  // bf16: slice s covers features 16s..16s+15, lane holds 8 of them.
  // fp32: step s pairs feature s (lanes 0-31) with feature D/2 + s (lanes 32-63).
  constexpr int NQF = BF16 ? D / 16 : D / 8;  // 16-byte loads per lane
  u32x4 qf[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) {
    uint32_t col = BF16 ? (16 * s + 8 * hi) : (4 * s + (D / 2) * hi);
    qf[s] = load16(rq, ((uint32_t)my_row * D + col) * ES);
  }
  // Complete the Q loads here: otherwise the in-order memory counter makes
  // every iteration of the key loop wait for its own prefetch as well.
#pragma unroll
  for (int s = 0; s < NQF; ++s) asm volatile("" : : "v"(qf[s]));

  // ---- running state: one query row per lane ----
  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.0f;
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s
  float l_run = 0.0f;               // this lane's share of the row sum

  if (nkb > 0) G::stage(lds_base, Kp + head_k, Vp + head_k, kv_bytes, 0, 0, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    // Block kb+1 goes to the other stage, which every wave finished reading
    // before the barrier that ended the previous iteration.
    if (kb + 1 < nkb) G::stage(lds_base, Kp + head_k, Vp + head_k, kv_bytes, kb + 1, st ^ 1, wave, lane);
    const char* kt = smem + st * G::STAGE;
    const char* vt = kt + G::TILE;

    if (kb < wave_nkb) {
      // ---- scores: S^T[j][i] for the 64 keys of this block, two 32-key tiles
      f32x16 s[BC / 32];
#pragma unroll
      for (int jt = 0; jt < BC / 32; ++jt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[jt][e] = 0.0f;
        const int j = jt * 32 + li;
        const char* krow = kt + j * G::ROWB;
        const int sw = G::swz_k(j);
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
            const f32x4 a =
                *reinterpret_cast<const f32x4*>(krow + ((q4 + (D / 8) * hi) ^ sw) * 16);
            const f32x4 bq = __builtin_bit_cast(f32x4, qf[q4]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], bq[e], s[jt], 0, 0, 0);
          }
        }
      }

      // ---- mask: lane holds keys j = kb*BC + 32jt + 8g + 4hi + r of row my_row
      const int jblk = kb * BC;
      const bool need_mask = (jblk + BC > L) || (CAUSAL && jblk + BC - 1 > row_w);
      if (need_mask) {
        // valid iff j < key_limit; key offsets within the block are constants
        const int lim = (CAUSAL ? min(L, my_row + 1) : L) - jblk - 4 * hi;
#pragma unroll
        for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (32 * jt + 8 * g + r >= lim) s[jt][4 * g + r] = -__builtin_inff();
      }

      // ---- online softmax: block row max, conditional rescale
      float mx = -__builtin_inff();
#pragma unroll
      for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jt][e]);
      mx = pair_max(mx);
      const float mx2 = mx * scale_log2;  // -inf stays -inf (scale_log2 > 0)
      const bool grow = mx2 > m_run + TAU;
      if (__any(grow)) {
        const float m_new = fmaxf(m_run, mx2);
        const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
        m_run = m_new;
      }
      const float msub = (m_run == -__builtin_inff()) ? 0.0f : m_run;

      // ---- weights p = 2^(s*scale*log2e - m), rounded to T, and PV
      if constexpr (BF16) {
        // Slice k (16 keys, k = 0..3) of this block takes accumulator tile
        // jt = k/2, groups g = 2(k%2) and 2(k%2)+1: lane half hi holds keys
        // 16k + 4hi + r (k-slots 8hi + r) and 16k + 8 + 4hi + r (k-slots
        // 8hi + 4 + r), r = 0..3.
        bf16x8 pf[BC / 16];
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int k = 0; k < BC / 16; ++k) {
          const int jt = k / 2, g0 = 2 * (k % 2);
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int g = g0 + e / 4, r = e % 4;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r], scale_log2, -msub));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][4 * g + r + 1], scale_log2, -msub));
            const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_run, false);
            pf[k][e] = pk[0];
            pf[k][e + 1] = pk[1];
          }
        }
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
              const char* p = vt + row * G::ROWB + ((cc ^ G::swz_v(row)) * 16) + (qq % 2) * 8;
              const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
              const bf16x4 b4 = __builtin_bit_cast(bf16x4, v4);
              a[4 * half + 0] = b4[0];
              a[4 * half + 1] = b4[1];
              a[4 * half + 2] = b4[2];
              a[4 * half + 3] = b4[3];
            }
            o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[k], o[ct], 0, 0, 0);
          }
        }
      } else {
        // fp32: one MFMA per accumulator element; k-slot hi of the step
        // (jt, g, r) is key 32jt + 8g + 4hi + r, read as a single element of
        // the row-major V tile.
#pragma unroll
        for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][e], scale_log2, -msub));
            s[jt][e] = p;
            l_run += p;
          }
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const int c = ct * 32 + li;
#pragma unroll
          for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int row = 32 * jt + 8 * g + 4 * hi + r;
                const float a = *reinterpret_cast<const float*>(
                    vt + row * G::ROWB + (((c / 4) ^ G::swz_v(row)) * 16) + (c % 4) * 4);
                o[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[jt][4 * g + r], o[ct], 0, 0, 0);
              }
        }
      }
    }

    // This thread's direct loads of block kb+1 have landed; after the
    // barrier every wave's have, and every wave is done with stage st.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: divide by the row sum (0 when no key was valid), store
  const float l_tot = pair_sum(l_run);
  const float inv = (l_tot > 0.0f) ? (1.0f / l_tot) : 0.0f;
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = ((uint32_t)my_row * D + ct * 32 + 8 * g + 4 * hi) * ES;
      if constexpr (BF16) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[ct][4 * g + r] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), ro, (int)off, 0, 0);
      } else {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = o[ct][4 * g + r] * inv;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, (int)off, 0, 0);
      }
    }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_one(const LaunchArgs& a) {
  const int nqb = (int)((a.n + BR - 1) / BR);
  const int64_t blocks = (int64_t)nqb * a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V, a.key_lens,
                     (T*)a.O, (int)a.H, (int)a.n, (int)a.m, nqb, a.scale_log2);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const LaunchArgs& a) {
  return a.causal ? launch_one<T, D, true>(a) : launch_one<T, D, false>(a);
}

template <typename T>
static hipError_t launch_t(const LaunchArgs& a) {
  return a.d == 64 ? launch_d<T, 64>(a) : launch_d<T, 128>(a);
}

hipError_t launch_attention(const LaunchArgs& a) {
  return a.bf16 ? launch_t<__bf16>(a) : launch_t<float>(a);
}

int query_rows_per_block() { return BR; }
int keys_per_block() { return BC; }

}  // namespace mha
