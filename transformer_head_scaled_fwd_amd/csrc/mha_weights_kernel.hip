// mha_weights_kernel.hip -- the attention weights A as an output, for gfx950.
//
// A[b,t,i,j] = exp(scale * q_i.k_j + bias_ij - lse_i) for a valid pair and 0
// otherwise: the softmax weights that the pages' attention function returns
// next to its output ("序列建模架构的演进与变革（二）" §4.9, which returns the
// weight matrix; "Transformer: 详解" §4.1).  lse_i is the row's log-sum-exp,
// stored by the forward kernel, so one extra pass of score MFMAs rebuilds
// the normalised weights without a second reduction.
//
// Unlike the forward pass this materialises B*H*n*m elements; it is the
// optional, memory-bound companion of the forward kernel, not part of it.
//
// One workgroup (4 waves, 128 query rows) of one (batch, head) walks one
// chunk of consecutive key blocks: blocks that hold a visible key get
// S^T = K Q^T on MFMA (K staged through the direct-load ring, one block
// ahead), the distance bias, the mask and the exponent; blocks past the last
// visible key are written as zeros without reading K.  The weights of
// different key blocks are independent, so the key axis is cut into as many
// chunks (workgroups) as it takes to give every CU several workgroups; no
// result is combined across chunks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mha_launch.h"
#include "mha_tiles.h"

namespace mha {

struct WeightParams {
  int H, group;          // query heads, query heads per K/V head
  int n, m;              // query rows, key rows per head
  int nqb;               // query blocks per head
  int nkb_all;           // key blocks covering m
  int kchunk;            // key blocks per workgroup (one chunk)
  int bottom_right;      // causal alignment: 0 top-left, 1 bottom-right
  int vec;               // 1 when m % 4 == 0: four keys per store
  int vec8;              // 1 when m % 8 == 0: rows staged through LDS, 16-byte stores
  float scale;           // the caller's scale
  float scale_log2;      // scale * log2(e)
  int stream_out;        // A written through to memory (kStoreOut)
  int BH, H_kv;          // batch x query heads, K/V heads
  // Divisors of the block-index decode, fixed at launch (FastDiv).
  FastDiv div_bh, div_nqb, div_h, div_group;
};

// Resident workgroups per CU: two, except fp32 with d = 128, whose K ring and
// staging take 98 KiB of LDS.
template <typename T, int D>
constexpr int weights_wg_per_cu() {
  return (sizeof(T) == 4 && D == 128) ? 1 : 2;
}

template <typename T, int D, bool CAUSAL, bool ALIBI>
__global__ void __launch_bounds__(256, (weights_wg_per_cu<T, D>()))
attn_weights_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp,
                    const int32_t* __restrict__ key_lens, const float* __restrict__ alibi_slopes,
                    const float* __restrict__ lse, T* __restrict__ Ap, WeightParams prm) {
  constexpr int NW = 4;
  using G = Geo<T, D, NW>;
  using P = Phase<T, D>;
  constexpr int ES = G::ES;
  constexpr bool BF16 = G::BF16;
  constexpr int BR = G::BR;
  constexpr int NS = P::NS;
  // Staging of one 64-key block of the wave's 32 rows, padded by 16 bytes
  // per row so that the lanes writing one row each land in distinct banks.
  constexpr int SROW = BC * ES + 16;
  constexpr int SWAVE = kRowsPerWave * SROW;
  __shared__ __attribute__((aligned(1024))) char smem[G::NSTAGE * G::TILE + NW * SWAVE];
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, li = lane % 32, hi = lane / 32;
  const int n = prm.n, m = prm.m;
  // Workgroup index: (chunk, query block, batch * head), the last fastest;
  // the divisions are by launch constants (div_by).
  const uint32_t bid = blockIdx.x;
  const uint32_t r1 = div_by(bid, prm.div_bh);             // chunk * nqb + query block
  const int bh = (int)(bid - r1 * (uint32_t)prm.BH);
  const uint32_t kcu = div_by(r1, prm.div_nqb);
  const int qb = (int)(r1 - kcu * (uint32_t)prm.nqb);
  const int kc = (int)kcu;
  const int kb0 = kc * prm.kchunk;                      // this chunk's key blocks
  const int kb1 = min(prm.nkb_all, kb0 + prm.kchunk);   // [kb0, kb1)
  const int b = (int)div_by((uint32_t)bh, prm.div_h);
  const int t = bh - b * prm.H;
  const int bkv = b * prm.H_kv + (int)div_by((uint32_t)t, prm.div_group);
  const int q0 = qb * BR;

  int L = m;
  if (key_lens != nullptr) {
    L = key_lens[b];
    L = L < 0 ? 0 : (L > m ? m : L);
  }
  const int off = (CAUSAL && prm.bottom_right) ? L - n : 0;
  const int kend = CAUSAL ? max(0, min(L, q0 + off + BR)) : L;
  const int nkb = (kend + BC - 1) / BC;  // blocks with a visible key for some row
  const int kvis = min(nkb, kb1);        // this chunk's visible blocks end here
  const int row_w = q0 + wave * kRowsPerWave;
  const int prow_w = row_w + off;
  const int wave_nkb = CAUSAL ? max(0, min(nkb, (prow_w + kRowsPerWave + BC - 1) / BC)) : nkb;
  const int my_row = row_w + li;
  const int prow = my_row + off;
  const int row_lim = CAUSAL ? min(L, prow + 1) : L;
  const float sr = ALIBI ? alibi_slopes[t] / prm.scale : 0.0f;

  const auto rq = make_rsrc(Qp + (size_t)bh * n * D, (uint32_t)n * D * ES);
  const T* kbase = Kp + (size_t)bkv * m * D;
  const uint32_t kv_bytes = (uint32_t)L * D * ES;
  // A of this head: rows >= n fall outside the resource and are dropped.
  const auto ra = make_rsrc(Ap + (size_t)bh * n * m, (uint32_t)((size_t)n * m * ES));

  // log2-domain row constant; a row with no valid key has lse = -inf and
  // every score masked, so its exponent must not become -inf - -inf.
  float lse2 = 0.0f;
  if (my_row < n) {
    const float v = lse[(size_t)bh * n + my_row];
    lse2 = (v == -__builtin_inff()) ? 0.0f : v * 1.4426950408889634f;
  }

  auto load_k = [&](int j) {
    G::template stage<true>(lds_k + (j % G::NSTAGE) * G::TILE, kbase, kv_bytes, j, wave, lane);
  };
  if (kb0 < kvis) load_k(kb0);

  u32x4 qf[P::NQF];
  P::load_q(qf, rq, my_row, hi);

  // Store the 16 values of score tile jt of block kb (keys
  // kb*BC + 32jt + 8g + 4hi + r, r = 0..3) for this lane's row.
  auto store_tile = [&](const f32x16& p, int kb, int jt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int key = kb * BC + 32 * jt + 8 * g + 4 * hi;
      const uint32_t off_el = (uint32_t)my_row * (uint32_t)m + (uint32_t)key;
      if (prm.vec) {
        if (key < m) {
          if constexpr (BF16) {
            bf16x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (__bf16)p[4 * g + r];
            store_result(__builtin_bit_cast(u32x2, v), ra, (int)(off_el * ES), prm.stream_out);
          } else {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = p[4 * g + r];
            store_result(__builtin_bit_cast(u32x4, v), ra, (int)(off_el * ES), prm.stream_out);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (key + r < m) {
            if constexpr (BF16) {
              const __bf16 h = (__bf16)p[4 * g + r];
              store_result(__builtin_bit_cast(uint16_t, h), ra, (int)((off_el + r) * ES),
                           prm.stream_out);
            } else {
              // (the element is copied out first: a bit cast taken straight
              // from a vector element reads element 0 of the group here)
              const float x = p[4 * g + r];
              store_result(__builtin_bit_cast(uint32_t, x), ra, (int)((off_el + r) * ES),
                           prm.stream_out);
            }
          }
        }
      }
    }
  };

  // Rows staged through LDS, then stored 16 bytes per lane: each store
  // instruction writes whole 128-byte row segments (bf16: 8 rows of 64 keys;
  // fp32: 4 rows) instead of 16 scattered bytes per row.
  char* stage_w = smem + G::NSTAGE * G::TILE + wave * SWAVE;
  constexpr int CPRW = BC * ES / 16;    // 16-byte chunks per staged row: 8 (bf16), 16 (fp32)
  constexpr int RPI = 64 / CPRW;        // rows per store instruction
  auto store_chunks = [&](int kb, auto&& chunk_of) {
#pragma unroll
    for (int rep = 0; rep < kRowsPerWave / RPI; ++rep) {
      const int rr = rep * RPI + lane / CPRW, c = lane % CPRW;
      const int key = kb * BC + c * (16 / ES);
      if (key < m) {
        const uint32_t off_el = (uint32_t)(row_w + rr) * (uint32_t)m + (uint32_t)key;
        store_result(chunk_of(rr, c), ra, (int)(off_el * ES), prm.stream_out);
      }
    }
  };
  auto store_block = [&](const f32x16 (&p)[NS], int kb) {
#pragma unroll
    for (int jt = 0; jt < NS; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        char* dst = stage_w + li * SROW + (32 * jt + 8 * g + 4 * hi) * ES;
        if constexpr (BF16) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)p[jt][4 * g + r];
          *reinterpret_cast<bf16x4*>(dst) = v;
        } else {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = p[jt][4 * g + r];
          *reinterpret_cast<f32x4*>(dst) = v;
        }
      }
    // The staging area belongs to this wave alone: order its writes before
    // the reads below (LDS operations of a wave complete in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    store_chunks(kb, [&](int rr, int c) {
      return *reinterpret_cast<const u32x4*>(stage_w + rr * SROW + c * 16);
    });
    // The next block's writes must not overtake these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto store_zero_block = [&](int kb) {
    store_chunks(kb, [&](int, int) { return u32x4{0u, 0u, 0u, 0u}; });
  };

  f32x16 zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.0f;

  for (int kb = kb0; kb < kb1; ++kb) {
    if (kb < kvis) {
      // K(kb) was requested one block ago; request K(kb+1) into the other
      // slot (last read before the barrier that ended block kb-1), then wait
      // for K(kb) only.
      if (kb + 1 < kvis) {
        load_k(kb + 1);
        G::template wait_loads<G::LOADS>();
      } else {
        G::template wait_loads<0>();
      }
      __syncthreads();
      if (kb < wave_nkb) {
        f32x16 s[NS];
        P::scores(s, smem + (kb % G::NSTAGE) * G::TILE, qf, li, hi);
        if constexpr (ALIBI) P::bias(s, (float)(prow - kb * BC - 4 * hi), sr);
        if ((kb * BC + BC > L) || (CAUSAL && kb * BC + BC - 1 > prow_w))
          P::mask(s, row_lim - kb * BC - 4 * hi);
#pragma unroll
        for (int jt = 0; jt < NS; ++jt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            s[jt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jt][e], prm.scale_log2, -lse2));
        if (prm.vec8) {
          store_block(s, kb);
        } else {
#pragma unroll
          for (int jt = 0; jt < NS; ++jt) store_tile(s[jt], kb, jt);
        }
      } else if (prm.vec8) {
        store_zero_block(kb);
      } else {
#pragma unroll
        for (int jt = 0; jt < NS; ++jt) store_tile(zero, kb, jt);
      }
      __syncthreads();  // K(kb) is consumed before its slot is refilled
    } else if (prm.vec8) {
      store_zero_block(kb);
    } else {
#pragma unroll
      for (int jt = 0; jt < NS; ++jt) store_tile(zero, kb, jt);
    }
  }
}

template <typename T, int D, bool CAUSAL, bool ALIBI>
static hipError_t launch_w(const WeightsArgs& a) {
  constexpr int BR = Geo<T, D, 4>::BR;
  WeightParams prm;
  prm.H = (int)a.H;
  prm.group = (int)(a.H / a.H_kv);
  prm.n = (int)a.n;
  prm.m = (int)a.m;
  prm.nqb = (int)((a.n + BR - 1) / BR);
  prm.nkb_all = (int)((a.m + BC - 1) / BC);
  // Key chunks (whole blocks; a workgroup walks its chunk's blocks serially,
  // one wave per SIMD each): without a mask, enough workgroups to fill the
  // CUs once (B8 H8 n = m = 512 9.10 -> 8.58 us against four per CU,
  // B2 H8 n = 256 m = 2048 d = 128 8.92 -> 7.16 us); causal, about four per
  // CU, whose chunks of unequal work then balance over the CUs.
  const int64_t units = (int64_t)((a.n + BR - 1) / BR) * a.B * a.H;
  const int64_t per_cu = a.mode == 0 ? weights_wg_per_cu<T, D>() : 4;
  const int64_t want = (per_cu * 256 + units - 1) / units;
  const int64_t nkc0 = want < 1 ? 1 : (want > prm.nkb_all ? prm.nkb_all : want);
  prm.kchunk = prm.nkb_all > 0 ? (int)((prm.nkb_all + nkc0 - 1) / nkc0) : 1;
  const int64_t nkc = prm.nkb_all > 0 ? (prm.nkb_all + prm.kchunk - 1) / prm.kchunk : 1;
  prm.bottom_right = a.mode == 2;
  prm.vec = (a.m % 4) == 0;
  prm.vec8 = (a.m % 8) == 0;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale_log2;
  // A written through to memory when it fits the L2s (kStoreOut).
  prm.stream_out = a.B * a.H * a.n * a.m * (int64_t)sizeof(T) <= kStreamOutMaxBytes;
  prm.BH = (int)(a.B * a.H);
  prm.H_kv = (int)a.H_kv;
  prm.div_bh = fast_div((uint32_t)prm.BH);
  prm.div_nqb = fast_div((uint32_t)prm.nqb);
  prm.div_h = fast_div((uint32_t)prm.H);
  prm.div_group = fast_div((uint32_t)prm.group);
  const int64_t blocks = units * nkc;
  hipLaunchKernelGGL((attn_weights_kernel<T, D, CAUSAL, ALIBI>), dim3((unsigned)blocks), dim3(256),
                     0, (hipStream_t)a.stream, (const T*)a.Q, (const T*)a.K, a.key_lens,
                     a.alibi_slopes, a.lse, (T*)a.A, prm);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_wd(const WeightsArgs& a) {
  const bool causal = a.mode != 0;
  if (a.alibi_slopes != nullptr)
    return causal ? launch_w<T, D, true, true>(a) : launch_w<T, D, false, true>(a);
  return causal ? launch_w<T, D, true, false>(a) : launch_w<T, D, false, false>(a);
}

hipError_t launch_weights(const WeightsArgs& a) {
  if (a.bf16) return a.d == 64 ? launch_wd<__bf16, 64>(a) : launch_wd<__bf16, 128>(a);
  return a.d == 64 ? launch_wd<float, 64>(a) : launch_wd<float, 128>(a);
}

}  // namespace mha
