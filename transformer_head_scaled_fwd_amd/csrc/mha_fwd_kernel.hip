// mha_fwd_kernel.hip -- fused attention forward for gfx950 (MI355X).
//
// One workgroup computes BR = 128 query rows of one (batch, head): four
// wave64s, each owning 32 rows.  It walks the key axis in blocks of BC = 64
// keys.  Per block:
//
//   stage    K block -> LDS (row-major) and V block -> LDS (transposed),
//            from 16-byte buffer loads issued one block ahead;
//   scores   S^T = K Q^T on MFMA (32x32 tiles, fp32 accumulate), Q held in
//            registers for the whole walk;
//   mask     -inf where j >= L_b or (causal and j > i)
//            ("Transformer: 详解" §3.4, §5.3);
//   softmax  online: running row max and sum in fp32, exp2 with the scale
//            and log2(e) folded into one FMA, rescale of the output only when
//            the row max grew by more than 2^TAU ("Transformer" wiki page:
//            mixed precision needs the blockwise, online softmax);
//   PV       O^T += V^T P^T on MFMA with P rounded to the input dtype.
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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mha_launch.h"

namespace mha {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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

// Value of the lane 32 positions away (lanes l and l^32 share a query row).
__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

template <typename T>
struct Elem;

// bf16 operands: v_mfma_f32_32x32x16_bf16.  A (32x16): lane l supplies row
// l%32, k = 8(l/32)..+7; B (16x32): column l%32, same k.
template <>
struct Elem<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr int kK = 16;  // contraction depth of one MFMA
};

// fp32 operands: v_mfma_f32_32x32x2_f32.  A: lane l supplies row l%32,
// k = l/32; B: column l%32, k = l/32.
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  static constexpr int kK = 2;
};

// Position of key u (0..15 within a group of 16) in the transposed bf16 V
// tile: bits 2 and 3 swapped, so that the 8 keys a lane feeds to one PV MFMA
// are contiguous (see the P packing in the main loop).
__device__ inline int vt_pos16(int j) {
  return (j & ~15) | ((j & 4) << 1) | ((j & 8) >> 1) | (j & 3);
}

template <typename T, int D, bool CAUSAL>
struct Tile {
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int KROW = D * ES + 16;   // K tile row stride (bytes), padded
  static constexpr int VROW = BC * ES + 16;  // transposed V tile row stride, padded
  static constexpr int K_BYTES = BC * KROW;
  static constexpr int V_BYTES = D * VROW;
  static constexpr int LDS_BYTES = K_BYTES + V_BYTES;
  static constexpr int CPR = D * ES / 16;            // 16-byte chunks per row
  static constexpr int K_CHUNKS = BC * CPR / kThreads;  // per thread
  // V staging: each thread owns VR consecutive rows x one 16-byte chunk.
  static constexpr int V_ITEMS = BC * CPR;             // (row, chunk) pairs
  static constexpr int VR = V_ITEMS / kThreads;        // rows per thread (>= 1)
  static constexpr int VR_TOTAL = VR;                  // loads per thread
  static_assert(BC * CPR % kThreads == 0, "K staging must tile the workgroup");
  static_assert(VR == 2 || VR == 4 || VR == 8, "V staging needs 2, 4 or 8 rows per thread");
};

// Which (row group, chunk) a thread stages for the transposed V tile.
template <typename T, int D>
__device__ inline void v_item(int tid, int& row0, int& chunk) {
  constexpr int CPR = D * Elem<T>::kBytes / 16;
  constexpr int VR = (BC * CPR) / kThreads;
  chunk = tid % CPR;
  row0 = (tid / CPR) * VR;
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp,
                const T* __restrict__ Vp, const int32_t* __restrict__ key_lens,
                T* __restrict__ Op, int H, int n, int m, int nqb, float scale_log2) {
  using TL = Tile<T, D, CAUSAL>;
  constexpr int ES = TL::ES;
  constexpr bool BF16 = (ES == 2);
  __shared__ __attribute__((aligned(16))) char smem[TL::LDS_BYTES];
  char* Ks = smem;
  char* Vt = smem + TL::K_BYTES;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
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

  // Buffer resources: out-of-range loads read 0 and out-of-range stores are
  // dropped, so rows >= n (queries) and >= L (keys, values) need no branch.
  const size_t head_q = (size_t)bh * (size_t)n * D;
  const size_t head_k = (size_t)bh * (size_t)m * D;
  const auto rq = make_rsrc(Qp + head_q, (uint32_t)n * D * ES);
  const auto rk = make_rsrc(Kp + head_k, (uint32_t)L * D * ES);
  const auto rv = make_rsrc(Vp + head_k, (uint32_t)L * D * ES);
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

  // ---- staging of one K/V block into registers, then into LDS ----
  u32x4 kreg[TL::K_CHUNKS];
  u32x4 vreg[TL::VR_TOTAL];
  int v_row0, v_chunk;
  v_item<T, D>(tid, v_row0, v_chunk);

  auto fetch = [&](int kb) {
    const uint32_t base = (uint32_t)kb * BC;
#pragma unroll
    for (int u = 0; u < TL::K_CHUNKS; ++u) {
      const int id = u * kThreads + tid;
      const int r = id / TL::CPR, c = id % TL::CPR;
      kreg[u] = load16(rk, ((base + r) * D) * ES + c * 16);
    }
#pragma unroll
    for (int r = 0; r < TL::VR; ++r)
      vreg[r] = load16(rv, ((base + v_row0 + r) * D) * ES + v_chunk * 16);
  };

  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < TL::K_CHUNKS; ++u) {
      const int id = u * kThreads + tid;
      const int r = id / TL::CPR, c = id % TL::CPR;
      *reinterpret_cast<u32x4*>(Ks + r * TL::KROW + c * 16) = kreg[u];
    }
    if constexpr (BF16) {
      // Transpose: element (row j, feature c) goes to Vt[c][vt_pos16(j)].
      // Each dword of a loaded chunk holds features 2w (low half) and 2w+1.
      const int pos = vt_pos16(v_row0);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t sel = p ? 0x07060302u : 0x05040100u;
          const int c = v_chunk * 8 + 2 * w + p;
          char* dst = Vt + c * TL::VROW + pos * 2;
          if constexpr (TL::VR == 2) {
            *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
          } else {
            u32x2 val;
            val[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
            val[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
            *reinterpret_cast<u32x2*>(dst) = val;
          }
        }
      }
    } else {
      // fp32: element (row j, feature c) goes to Vt[c][j]; 4 rows per store.
#pragma unroll
      for (int g = 0; g < TL::VR / 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = v_chunk * 4 + e;
          u32x4 val;
          val[0] = vreg[4 * g + 0][e];
          val[1] = vreg[4 * g + 1][e];
          val[2] = vreg[4 * g + 2][e];
          val[3] = vreg[4 * g + 3][e];
          *reinterpret_cast<u32x4*>(Vt + c * TL::VROW + (v_row0 + 4 * g) * 4) = val;
        }
      }
    }
  };

  // ---- running state: one query row per lane ----
  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.0f;
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s
  float l_run = 0.0f;               // this lane's share of the row sum

  if (nkb > 0) {
    fetch(0);
    stash();
  }
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) fetch(kb + 1);

    if (kb < wave_nkb) {
      // ---- scores: S^T[j][i] for the 64 keys of this block, two 32-key tiles
      f32x16 s[BC / 32];
#pragma unroll
      for (int jt = 0; jt < BC / 32; ++jt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[jt][e] = 0.0f;
        const char* krow = Ks + (jt * 32 + li) * TL::KROW;
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(krow + (16 * ks + 8 * hi) * 2);
            s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ks]), s[jt], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int q4 = 0; q4 < D / 8; ++q4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(krow + (4 * q4 + (D / 2) * hi) * 4);
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
#pragma unroll
        for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = jblk + 32 * jt + 8 * g + 4 * hi + r;
              const bool ok = (j < L) && (!CAUSAL || j <= my_row);
              if (!ok) s[jt][4 * g + r] = -__builtin_inff();
            }
      }

      // ---- online softmax: block row max, conditional rescale
      float mx = -__builtin_inff();
#pragma unroll
      for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jt][e]);
      mx = fmaxf(mx, other_half(mx));
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
        // jt = k/2, groups g = 2(k%2) and 2(k%2)+1: lane half hi then holds
        // keys 16k + {4hi + r, 8 + 4hi + r}, r = 0..3, as k-slots 8hi..8hi+7,
        // which is why the V tile is stored with bits 2 and 3 of the key
        // index swapped.
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
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const char* vrow = Vt + (ct * 32 + li) * TL::VROW;
#pragma unroll
          for (int k = 0; k < BC / 16; ++k) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vrow + (16 * k + 8 * hi) * 2);
            o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[k], o[ct], 0, 0, 0);
          }
        }
      } else {
        // fp32: one MFMA per accumulator element; k-slot hi of the step
        // (jt, g, r) is key 32jt + 8g + 4hi + r, read from the natural-order
        // transposed V tile.
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
          const char* vrow = Vt + (ct * 32 + li) * TL::VROW;
#pragma unroll
          for (int jt = 0; jt < BC / 32; ++jt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 a = *reinterpret_cast<const f32x4*>(vrow + (32 * jt + 8 * g + 4 * hi) * 4);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                o[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[r], s[jt][4 * g + r], o[ct], 0, 0, 0);
            }
        }
      }
    }

    __syncthreads();
    if (kb + 1 < nkb) stash();
    __syncthreads();
  }

  // ---- epilogue: divide by the row sum (0 when no key was valid), store
  const float l_tot = l_run + other_half(l_run);
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
