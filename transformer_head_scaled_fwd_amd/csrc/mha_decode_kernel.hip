// mha_decode_kernel.hip -- attention of a few new queries against a long
// key/value cache, for gfx950.
//
// Incremental decoding keeps the keys and values of every earlier token in a
// cache allocated at its maximum length and computes only the new tokens'
// K and V at each step (hugogu wiki "Transformer", KV-cache section;
// "序列建模架构的演进与变革（二）" §3.4 and §3.8).  The n new queries of
// sequence b are the last n of its L_b filled keys, so query i sits at
// position p_i = i + L_b - n and sees keys j <= p_i (bottom-right causal
// alignment); the result is the same as mha_forward_ex with
// MHA_MASK_CAUSAL_BOTTOM_RIGHT.
//
// The work is a stream over the cache: each cached K/V row is read once for
// all the query rows that use its head (the group of query heads sharing a
// K/V head, times the n new tokens: R = group * n rows, up to 32 per wave).
// The key axis is cut two ways to fill the chip:
//
//   - across the waves of a workgroup: wave w takes key blocks w, w+NW, ...
//     of the workgroup's range, staging each K and V block into its own LDS
//     tiles (buffer->LDS direct loads, one block in flight per tile) and
//     running the same score / mask / bias / online-softmax / PV phases as
//     the forward kernel on its 32 rows;
//   - across workgroups ("splits"): when the (batch, K/V head) pairs alone
//     cannot fill the chip, the range is cut into splits whose partial
//     results (running max m, row sum l, unnormalised O) go to a workspace
//     and a second, small kernel merges them.
//
// Partial results merge by the same rescaling the online softmax uses:
// with M = max_s m_s, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mha_launch.h"
#include "mha_tiles.h"

namespace mha {

struct DecParams {
  int H, group;          // query heads, query heads per K/V head
  int n, m;              // new queries per sequence, cache capacity
  int R;                 // query rows per (batch, K/V head): group * n
  int nrs;               // row sets of 32 rows: ceil(R / 32)
  int nsplit;            // workgroups along the key axis
  int split_blocks;      // key blocks per split (a multiple of the wave count)
  float scale, scale_log2;
  int H_kv;              // K/V heads
  // Divisors of the block-index decode and of a lane's row, fixed at
  // launch (FastDiv): nsplit, nrs, H_kv and n.
  FastDiv div_split, div_nrs, div_hkv, div_n;
};

template <typename T, int D, int NW>
struct DecGeo {
  using G1 = Geo<T, D, 1>;  // one wave stages a whole tile
  static constexpr int TILE = G1::TILE;
  static constexpr int TILES_BYTES = NW * 2 * TILE;                 // K and V tile per wave
  static constexpr int MERGE_BYTES = NW * kRowsPerWave * (D + 2) * 4;  // O, m, l per wave
  static constexpr int LDS_BYTES = TILES_BYTES > MERGE_BYTES ? TILES_BYTES : MERGE_BYTES;
};

template <typename T, int D, int NW, bool ALIBI>
__global__ void __launch_bounds__(64 * NW, 1)
attn_decode_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
                   const int32_t* __restrict__ cache_lens, const float* __restrict__ alibi_slopes,
                   T* __restrict__ Op, float* __restrict__ lse, float* __restrict__ part_o,
                   float* __restrict__ part_ml, DecParams prm) {
  using DG = DecGeo<T, D, NW>;
  using G1 = typename DG::G1;
  using P = Phase<T, D>;
  constexpr int ES = G1::ES;
  constexpr int NS = P::NS;
  constexpr int LOADS = G1::LOADS;  // direct loads per tile
  __shared__ __attribute__((aligned(1024))) char smem[DG::LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, li = lane % 32, hi = lane / 32;
  const int n = prm.n, m = prm.m;

  // grid: ((b * Hkv + g) * nrs + rs) * nsplit + s; the divisions are by
  // launch constants (div_by)
  const uint32_t bid0 = blockIdx.x;
  const uint32_t bid1 = div_by(bid0, prm.div_split);
  const int s = (int)(bid0 - bid1 * (uint32_t)prm.nsplit);
  const uint32_t bid2 = div_by(bid1, prm.div_nrs);
  const int rs = (int)(bid1 - bid2 * (uint32_t)prm.nrs);
  const int Hkv = prm.H_kv;
  const int b = (int)div_by(bid2, prm.div_hkv);
  const int g = (int)bid2 - b * Hkv;

  int L = m;
  if (cache_lens != nullptr) {
    L = cache_lens[b];
    L = L < 0 ? 0 : (L > m ? m : L);
  }

  // This lane's query row: r = rs*32 + li -> head t = g*group + r / n,
  // token i = r % n.  Lanes past R compute a dummy row that is never stored.
  const int r = rs * kRowsPerWave + li;
  const bool real = r < prm.R;
  const int rt = (int)div_by((uint32_t)r, prm.div_n);  // r / n
  const int t = g * prm.group + (real ? rt : 0);
  const int i = real ? r - rt * n : 0;
  const int qrow = real ? t * n + i : prm.H * n;  // row within batch b; dummy reads 0
  const int prow = i + L - n;                     // position of the query
  const int row_lim = real ? min(L, prow + 1) : L;
  const int lim_min = L - n + 1;                  // smallest limit of a real row (i = 0)

  const auto rq = make_rsrc(Qp + (size_t)b * prm.H * n * D, (uint32_t)prm.H * n * D * ES);
  const size_t head_k = ((size_t)b * Hkv + g) * (size_t)m * D;
  const T* kbase = Kp + head_k;
  const T* vbase = Vp + head_k;
  const uint32_t kv_bytes = (uint32_t)L * D * ES;  // rows >= L read as 0
  const float sl2 = prm.scale_log2;
  const float sr = ALIBI ? alibi_slopes[t] / prm.scale : 0.0f;

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);
  const uint32_t kt_lds = lds_base + wave * 2 * DG::TILE;
  const uint32_t vt_lds = kt_lds + DG::TILE;
  const char* ktile = smem + wave * 2 * DG::TILE;
  const char* vtile = ktile + DG::TILE;

  // Key blocks of this wave: kb = kb0 + wave + NW * k, below kb_end.
  const int nkb_all = (L + BC - 1) / BC;
  const int kb0 = s * prm.split_blocks;
  const int kb_end = min(nkb_all, kb0 + prm.split_blocks);

  f32x16 o[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[ct][e] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;

  int kb = kb0 + wave;
  if (kb < kb_end) {
    G1::template stage<true, true>(kt_lds, kbase, kv_bytes, kb, 0, lane);
    G1::template stage<false, true>(vt_lds, vbase, kv_bytes, kb, 0, lane);
  }
  u32x4 qf[P::NQF];
  P::load_q(qf, rq, qrow, hi);

  for (; kb < kb_end; kb += NW) {
    const bool more = kb + NW < kb_end;
    // K(kb) then V(kb) were issued; wait for K only.
    G1::template wait_loads<LOADS>();
    f32x16 sc[NS];
    P::scores(sc, ktile, qf, li, hi);
    // The K tile is free once the score MFMAs have their operands: wait for
    // this wave's LDS reads before the direct loads overwrite the tile.
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      G1::template stage<true, true>(kt_lds, kbase, kv_bytes, kb + NW, 0, lane);
    }
    if constexpr (ALIBI) P::bias(sc, (float)(prow - kb * BC - 4 * hi), sr);
    if (kb * BC + BC > lim_min) P::mask(sc, row_lim - kb * BC - 4 * hi);
    // Online softmax with the max formed on demand, as in the forward
    // kernel: the weights are taken against the running max as it stands;
    // only when a lane's block sum passes 2^16 (or a row meets its first
    // valid key) does the wave form the block max, raise the running max
    // (when the block max exceeds it by more than TAU), recompute the
    // weights and rescale.  With a distance bias the row max rises block
    // after block, so the max is formed every block.  Most blocks thus
    // leave the output accumulators alone, for the MFMAs only.
    typename P::PFrag pf;
    float lb = 0.0f;
    auto exact = [&]() {
      const float mx = pair_max(P::lane_max(sc)) * sl2;
      const bool grew = mx > m_run + TAU;
      const float m_new = grew ? mx : m_run;
      const float alpha =
          (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      lb = 0.0f;
      P::weights(pf, sc, sl2, (m_run == -__builtin_inff()) ? 0.0f : m_run, lb);
      P::pin(pf);
      if (__any(grew)) {
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[ct][e] *= alpha;
      }
    };
    if constexpr (ALIBI) {
      exact();
    } else {
      P::weights(pf, sc, sl2, (m_run == -__builtin_inff()) ? 0.0f : m_run, lb);
      P::pin(pf);
      // A row with no running max yet takes the exact path at its first
      // block with a valid key (keys below row_lim), whatever its weights
      // against 0 summed to: they may all have underflowed to 0.
      const bool slow = (lb > 65536.0f) || (m_run == -__builtin_inff() && kb * BC < row_lim);
      if (__any(slow)) exact();
    }
    l_run += lb;
    // V(kb) was issued before K(kb+NW).
    if (more) G1::template wait_loads<LOADS>();
    else G1::template wait_loads<0>();
    P::pv(o, vtile, pf, lane);
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      G1::template stage<false, true>(vt_lds, vbase, kv_bytes, kb + NW, 0, lane);
    }
  }
  G1::template wait_loads<0>();

  // ---- merge the waves' partial results through LDS ----
  // Only the row set's real rows (R - 32 rs of them, at most 32) are merged:
  // a single decoded token over one K/V head (R = 1) leaves 31 lanes idle.
  const float l_tot = pair_sum(l_run);
  const int rows_here = min(kRowsPerWave, prm.R - rs * kRowsPerWave);
  __syncthreads();  // every wave is done with its tiles
  float* mo = reinterpret_cast<float*>(smem);  // [NW][32][D]
  float* mm = mo + NW * kRowsPerWave * D;      // [NW][32]
  float* ml = mm + NW * kRowsPerWave;          // [NW][32]
  if (li < rows_here) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = o[ct][4 * gg + q];
        *reinterpret_cast<f32x4*>(mo + (wave * kRowsPerWave + li) * D + ct * 32 + 8 * gg + 4 * hi) = v;
      }
  }
  if (hi == 0) {
    mm[wave * kRowsPerWave + li] = m_run;
    ml[wave * kRowsPerWave + li] = l_tot;
  }
  __syncthreads();

  const bool direct = prm.nsplit == 1;
  const size_t q_batch = (size_t)b * prm.H * n;  // first query row of batch b
  for (int e = tid; e < rows_here * D; e += 64 * NW) {
    const int row = e / D, c = e % D;
    const int rr = rs * kRowsPerWave + row;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[w * kRowsPerWave + row]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = mm[w * kRowsPerWave + row];
      const float f = (mw == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      acc += f * mo[(w * kRowsPerWave + row) * D + c];
      lsum += f * ml[w * kRowsPerWave + row];
    }
    const int tt = g * prm.group + rr / n, ii = rr % n;
    const size_t orow = q_batch + (size_t)tt * n + ii;  // query row in [B, H, n]
    if (direct) {
      const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
      Op[orow * D + c] = (T)(acc * inv);
      if (c == 0 && lse != nullptr)
        lse[orow] = (lsum > 0.0f) ? 0.6931471805599453f * (M + __builtin_amdgcn_logf(lsum))
                                  : -__builtin_inff();
    } else {
      const size_t prow_ws = orow * prm.nsplit + s;
      part_o[prow_ws * D + c] = acc;
      if (c == 0) {
        part_ml[2 * prow_ws] = M;
        part_ml[2 * prow_ws + 1] = lsum;
      }
    }
  }
}

// Merge of the splits: CW waves per query row (a 256-thread workgroup holds
// 4 / CW rows).  Every wave forms the row's max M over all splits (lane s
// holds split s's running max, 64 splits at a time, then a wave reduction);
// wave w of a row then sums the splits of its own share, [w * per,
// (w + 1) * per), weighted by 2^(m_s - M): lanes over the features, eight
// splits' loads in flight at a time.  With CW > 1 the waves' sums meet in LDS
// and the row's first wave adds them in wave order, so the result does not
// depend on timing.  Many splits (a long cache over few rows) take CW = 4:
// the shares shorten the chain of dependent loads a row needs.  Up to
// kOneWaveSplits splits take one wave per row that issues all of the row's
// loads at once.
constexpr int kOneWaveSplits = 16;  // most splits a row merges with one wave (CW = 1)
template <typename T, int D, int CW>
__global__ void __launch_bounds__(256)
attn_decode_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                           T* __restrict__ Op, float* __restrict__ lse, int rows, int nsplit) {
  constexpr int FL = D / 64;  // features per lane
  constexpr int RPW = 4 / CW;  // rows per workgroup
  __shared__ float acc_w[CW > 1 ? CW : 1][CW > 1 ? D : 1];
  __shared__ float lsum_w[CW];
  const int w4 = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int row = blockIdx.x * RPW + w4 / CW;
  const int wave = w4 % CW;
  const int lane = threadIdx.x % 64;
  if (CW == 1 && row >= rows) return;
  const float* ml = part_ml + (size_t)row * nsplit * 2;
  const float* po = part_o + (size_t)row * nsplit * D;
  float M = -__builtin_inff();
  float lsum = 0.0f;
  float acc[FL];
#pragma unroll
  for (int u = 0; u < FL; ++u) acc[u] = 0.0f;
  if constexpr (CW == 1) {
    // At most kOneWaveSplits splits: every load of the row is issued at
    // once (split q >= nsplit reads split nsplit - 1 again, weighted 0), so
    // the row waits for one round trip to memory instead of three.
    float mv = -__builtin_inff(), lv = 0.0f;
    if (lane < nsplit) {
      mv = ml[2 * lane];
      lv = ml[2 * lane + 1];
    }
    float v[kOneWaveSplits][FL];
#pragma unroll
    for (int q = 0; q < kOneWaveSplits; ++q)
#pragma unroll
      for (int u = 0; u < FL; ++u) v[q][u] = po[(size_t)min(q, nsplit - 1) * D + lane + 64 * u];
    M = mv;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    const float f = (mv == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
    lsum = f * lv;
#pragma unroll
    for (int q = 0; q < kOneWaveSplits; ++q) {
      const float fq =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), q));
#pragma unroll
      for (int u = 0; u < FL; ++u) acc[u] += fq * v[q][u];
    }
  } else {
    for (int s0 = 0; s0 < nsplit; s0 += 64)
      if (s0 + lane < nsplit) M = fmaxf(M, ml[2 * (s0 + lane)]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    const int per = (nsplit + CW - 1) / CW;
    const int sb = wave * per, se = min(nsplit, sb + per);
    for (int s0 = sb; s0 < se; s0 += 64) {
      // This lane's split: its weight 2^(m_s - M) (0 for a split with no key).
      float f = 0.0f;
      if (s0 + lane < se) {
        const float ms = ml[2 * (s0 + lane)];
        f = (ms == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
        lsum += f * ml[2 * (s0 + lane) + 1];
      }
      const int cnt = min(64, se - s0);
      int j = 0;
      for (; j + 8 <= cnt; j += 8) {
        float v[8][FL];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int u = 0; u < FL; ++u) v[q][u] = po[(size_t)(s0 + j + q) * D + lane + 64 * u];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float fq = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j + q));
#pragma unroll
          for (int u = 0; u < FL; ++u) acc[u] += fq * v[q][u];
        }
      }
      for (; j < cnt; ++j) {
        const float fq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
#pragma unroll
        for (int u = 0; u < FL; ++u) acc[u] += fq * po[(size_t)(s0 + j) * D + lane + 64 * u];
      }
    }
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) lsum += __shfl_xor(lsum, x);
  float total = lsum;
  float sum[FL];
#pragma unroll
  for (int u = 0; u < FL; ++u) sum[u] = acc[u];
  if constexpr (CW > 1) {
#pragma unroll
    for (int u = 0; u < FL; ++u) acc_w[wave][lane + 64 * u] = acc[u];
    if (lane == 0) lsum_w[wave] = lsum;
    __syncthreads();
    if (wave != 0) return;
    total = 0.0f;
#pragma unroll
    for (int u = 0; u < FL; ++u) sum[u] = 0.0f;
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      total += lsum_w[w];
#pragma unroll
      for (int u = 0; u < FL; ++u) sum[u] += acc_w[w][lane + 64 * u];
    }
  }
  const float inv = (total > 0.0f) ? 1.0f / total : 0.0f;
#pragma unroll
  for (int u = 0; u < FL; ++u) Op[(size_t)row * D + lane + 64 * u] = (T)(sum[u] * inv);
  if (lane == 0 && lse != nullptr)
    lse[row] = (total > 0.0f) ? 0.6931471805599453f * (M + __builtin_amdgcn_logf(total))
                              : -__builtin_inff();
}

// Waves per workgroup: four, except fp32 with d = 128, whose tiles allow two.
template <typename T, int D>
constexpr int dec_waves() {
  return (sizeof(T) == 4 && D == 128) ? 2 : 4;
}

template <typename T, int D, bool ALIBI>
static hipError_t launch_dec(const DecodeArgs& a, const DecodePlan& p) {
  constexpr int NW = dec_waves<T, D>();
  DecParams prm;
  prm.H = (int)a.H;
  prm.group = (int)(a.H / a.H_kv);
  prm.n = (int)a.n;
  prm.m = (int)a.m;
  prm.R = (int)(prm.group * a.n);
  prm.nrs = (int)p.nrs;
  prm.nsplit = (int)p.nsplit;
  prm.split_blocks = (int)p.split_blocks;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale_log2;
  prm.H_kv = (int)a.H_kv;
  prm.div_split = fast_div((uint32_t)prm.nsplit);
  prm.div_nrs = fast_div((uint32_t)prm.nrs);
  prm.div_hkv = fast_div((uint32_t)prm.H_kv);
  prm.div_n = fast_div((uint32_t)prm.n);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (p.nsplit > 1) {
    part_o = (float*)a.workspace;
    part_ml = part_o + (size_t)a.B * a.H * a.n * p.nsplit * D;
  }
  const int64_t blocks = a.B * a.H_kv * p.nrs * p.nsplit;
  hipLaunchKernelGGL((attn_decode_kernel<T, D, NW, ALIBI>), dim3((unsigned)blocks), dim3(64 * NW),
                     0, (hipStream_t)a.stream, (const T*)a.Q, (const T*)a.K, (const T*)a.V,
                     a.cache_lens, a.alibi_slopes, (T*)a.O, a.lse, part_o, part_ml, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const int64_t rows = a.B * a.H * a.n;
  if (p.nsplit > kOneWaveSplits)
    hipLaunchKernelGGL((attn_decode_combine_kernel<T, D, 4>), dim3((unsigned)rows), dim3(256), 0,
                       (hipStream_t)a.stream, part_o, part_ml, (T*)a.O, a.lse, (int)rows,
                       (int)p.nsplit);
  else
    hipLaunchKernelGGL((attn_decode_combine_kernel<T, D, 1>), dim3((unsigned)((rows + 3) / 4)),
                       dim3(256), 0, (hipStream_t)a.stream, part_o, part_ml, (T*)a.O, a.lse,
                       (int)rows, (int)p.nsplit);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dec_d(const DecodeArgs& a, const DecodePlan& p) {
  return a.alibi_slopes ? launch_dec<T, D, true>(a, p) : launch_dec<T, D, false>(a, p);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p) {
  if (a.bf16) return a.d == 64 ? launch_dec_d<__bf16, 64>(a, p) : launch_dec_d<__bf16, 128>(a, p);
  return a.d == 64 ? launch_dec_d<float, 64>(a, p) : launch_dec_d<float, 128>(a, p);
}

// ---- the decode scratch of the allocation-free entry point ----
//
// A fixed array in device memory, one per GPU the library runs on, held
// until the process ends, for callers that cannot allocate (code under HIP
// graph capture, serving loops, harnesses that forbid allocation).  It
// holds the split partial results in place of a caller's workspace.  The
// array's name in host code is only a stand-in for the symbol: its device
// address is taken once per device with hipGetSymbolAddress (with that
// device current) and that address is what kernels receive.
static __device__ __align__(256) char decode_scratch[kDecodeScratchBytes];

hipError_t decode_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex lock;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace mha
