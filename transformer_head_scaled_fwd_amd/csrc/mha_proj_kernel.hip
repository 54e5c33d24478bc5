// mha_proj_kernel.hip -- the linear projections around the attention core,
// for gfx950: C = A W^T + bias with A [M, K], W [N, K] (nn.Linear's
// [out, in] layout), fp32 accumulation on MFMA.
//
// Multi-head attention projects the inputs to Q, K and V, splits the model
// width into H heads of d_k, runs attention per head, concatenates the heads
// and projects once more ("序列建模架构的演进与变革（二）" §4.9; "Transformer:
// 详解" §4.2; "第2章：完整的 Transformer 架构" §2.2).  The head split and
// the concatenation are pure layout changes, so they are folded into the
// GEMMs' memory access instead of running as separate passes:
//
//   C_HEADS  the epilogue writes row (b, i), column (t, c) of the [B*L, H*d_k]
//            result straight to [B, H, L, d_k] (split);
//   A_HEADS  the loads read row (b, i), column (t, c) of the [B*L, H*d_k]
//            operand straight from [B, H, L, d_k] (concat).
//
// Tiles: a workgroup of 4 waves computes 128 x 128 outputs, each wave 64 x 64
// as 2 x 2 MFMA tiles (32 x 32).  K advances 128 bytes per step (64 bf16 or
// 32 fp32); both operands are K-contiguous and go global -> LDS by direct
// loads into a two-stage ring, XOR-swizzled by 16-byte chunk so that the 32
// rows one MFMA operand read touches land in distinct banks.  As in the
// attention kernel, the tile is computed transposed (W rows on the MFMA M
// axis), so each lane ends up holding one output row and four consecutive
// output columns, stored as one 8- or 16-byte write.  Up to three problems
// (Q, K and V projections) share one launch, one grid row each.
//
// Tile order: workgroups go to the 8 XCDs round-robin in index order and
// each XCD has its own L2, so XCD x is given a contiguous band of tile rows
// with all their column tiles.  A row band is then read by one XCD only,
// and the workgroups running together on it share A and W tiles in L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mha_launch.h"
#include "mha_tiles.h"

namespace mha {

namespace proj {

constexpr int BM = 128;       // output rows per workgroup
constexpr int BN = 128;       // output columns per workgroup
constexpr int ROWB = 128;     // bytes of one row of a K step
constexpr int CPR = ROWB / 16;
constexpr int TILE = BM * ROWB;  // 16 KiB: one operand tile of one K step
constexpr int NSTAGE = 2;
constexpr int NWAVE = 4;
constexpr int LOADS = TILE / 1024 / NWAVE;  // direct loads per wave per operand tile

__device__ inline int swz(int r) { return (r >> 1) & 7; }

}  // namespace proj

template <typename T, bool A_HEADS, bool C_HEADS>
__global__ void __launch_bounds__(256, 2) proj_gemm_kernel(ProjBatch batch) {
  using namespace proj;
  constexpr int ES = sizeof(T);
  constexpr bool BF16 = ES == 2;
  constexpr int BK = ROWB / ES;  // K elements per step
  constexpr int EPC = 16 / ES;   // elements per 16-byte chunk
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * 2 * TILE];

  const ProjProblem pb = blockIdx.y == 0 ? batch.p[0] : (blockIdx.y == 1 ? batch.p[1] : batch.p[2]);
  const int tiles_m = (pb.M + BM - 1) / BM, tiles_n = (pb.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (t >= total) return;  // the whole workgroup leaves
  if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
  const int tn = t % tiles_n, tm = t / tiles_n;
  const int row0 = tm * BM, col0 = tn * BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, li = lane % 32, hi = lane / 32;
  const int K = pb.K;
  const int dk_shift = pb.dk == 64 ? 6 : 7;

  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  // Buffer resources: A's rows past M and W's rows past N read as 0.
  const auto ra = make_rsrc(pb.A, (uint32_t)pb.a_bytes);
  const auto rw = make_rsrc(pb.W, (uint32_t)((size_t)pb.N * K * ES));

  // Per load u of this wave: the tile row r and the swizzled chunk it
  // fetches; the row's base offset in A does not change along K.
  uint32_t a_row_base[LOADS], w_row_base[LOADS];
  int chunk_of[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int q = (u * NWAVE + wave) * 64 + lane;
    const int r = q / CPR, pc = q % CPR;
    chunk_of[u] = pc ^ swz(r);
    const int row = row0 + r;
    if constexpr (A_HEADS) {
      // row (b, i) of the concatenated heads: element (t, c) lives at
      // ((b*H + t)*L + i)*d_k + c of [B, H, L, d_k]; rows past M land past
      // the end of the tensor and read 0.
      const int b = row / pb.L, i = row % pb.L;
      a_row_base[u] = (uint32_t)(((size_t)b * pb.H * pb.L + i) * pb.dk);
    } else {
      a_row_base[u] = (uint32_t)((size_t)row * K);
    }
    w_row_base[u] = (uint32_t)((size_t)(col0 + r) * K);
  }

  auto load = [&](int kt, int stage) {
    const uint32_t ta = lds + stage * 2 * TILE, tw = ta + TILE;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int slot = (u * NWAVE + wave) * 64;
      const int k = kt * BK + chunk_of[u] * EPC;
      uint32_t aoff;
      if constexpr (A_HEADS) {
        const int t = k >> dk_shift, c = k & (pb.dk - 1);
        aoff = (a_row_base[u] + (uint32_t)t * pb.L * pb.dk + c) * ES;
      } else {
        aoff = (a_row_base[u] + k) * ES;
      }
      const uint32_t woff = (w_row_base[u] + k) * ES;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(ta + slot * 16), "v"(aoff), "s"(ra) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(tw + slot * 16), "v"(woff), "s"(rw) : "memory");
    }
  };

  // Wave tile: output rows 64*wr.., columns 64*wc..
  const int wr = wave / 2, wc = wave % 2;
  f32x16 acc[2][2];  // [column tile jn][row tile im], transposed tiles
#pragma unroll
  for (int jn = 0; jn < 2; ++jn)
#pragma unroll
    for (int im = 0; im < 2; ++im)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[jn][im][e] = 0.0f;

  // Bias of this lane's 32 output columns (see the epilogue), requested
  // before the K loop so that its latency hides behind the first tile's:
  // element loads through a buffer resource, so no bias (0 records) and
  // columns past N read 0 without a branch.
  float bv[2][4][4];
  {
    const auto rb = make_rsrc(pb.bias, pb.bias != nullptr ? (uint32_t)pb.N * ES : 0u);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = (col0 + 64 * wc + 32 * jn + 8 * g + 4 * hi + r) * ES;
          if constexpr (BF16) {
            const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0);
            bv[jn][g][r] = (float)__builtin_bit_cast(__bf16, h);
          } else {
            bv[jn][g][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0));
          }
        }
  }

  const int nkt = K / BK;
  // Two stages: step kt's barrier, after the wait for its own tile, also
  // retires every read of step kt-1, whose slot then receives step kt+1.
  load(0, 0);
  for (int kt = 0; kt < nkt; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nkt) load(kt + 1, (kt + 1) & 1);
    const char* ta = smem + (kt & 1) * 2 * TILE;
    const char* tw = ta + TILE;
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        u32x4 wf[2], af[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rw_ = 64 * wc + 32 * j + li;
          wf[j] = *reinterpret_cast<const u32x4*>(tw + rw_ * ROWB + ((2 * ks + hi) ^ swz(rw_)) * 16);
          const int ra_ = 64 * wr + 32 * j + li;
          af[j] = *reinterpret_cast<const u32x4*>(ta + ra_ * ROWB + ((2 * ks + hi) ^ swz(ra_)) * 16);
        }
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
          for (int im = 0; im < 2; ++im)
            acc[jn][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wf[jn]), __builtin_bit_cast(bf16x8, af[im]),
                acc[jn][im], 0, 0, 0);
      }
    } else {
      // fp32: lane half hi covers chunks 4hi..4hi+3; each chunk holds four k.
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 wf[2], af[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rw_ = 64 * wc + 32 * j + li;
          wf[j] = *reinterpret_cast<const f32x4*>(tw + rw_ * ROWB + ((q4 + 4 * hi) ^ swz(rw_)) * 16);
          const int ra_ = 64 * wr + 32 * j + li;
          af[j] = *reinterpret_cast<const f32x4*>(ta + ra_ * ROWB + ((q4 + 4 * hi) ^ swz(ra_)) * 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int im = 0; im < 2; ++im)
              acc[jn][im] = __builtin_amdgcn_mfma_f32_32x32x2f32(wf[jn][e], af[im][e],
                                                                  acc[jn][im], 0, 0, 0);
      }
    }
  }

  // Epilogue: lane holds output row row0 + 64wr + 32im + li and columns
  // col0 + 64wc + 32jn + 8g + 4hi + {0..3}.  Buffer stores with 32-bit
  // offsets (C stays under 2 GiB): rows past M land past the end of C and
  // are dropped; columns past N would land in other rows, so they branch
  // (N is a multiple of 64, so a wave's 64 columns are all in or all out).
  const auto rc = make_rsrc(pb.C, (uint32_t)((size_t)pb.M * pb.N * ES));
  auto c_off = [&](uint32_t row, uint32_t col) -> uint32_t {
    if (row >= (uint32_t)pb.M) return (uint32_t)pb.M * (uint32_t)pb.N;  // the end of C: dropped
    if constexpr (C_HEADS) {
      const uint32_t b = row / (uint32_t)pb.L, i = row % (uint32_t)pb.L;
      const uint32_t t = col >> dk_shift, c = col & (uint32_t)(pb.dk - 1);
      return ((b * (uint32_t)pb.H + t) * (uint32_t)pb.L + i) * (uint32_t)pb.dk + c;
    } else {
      return row * (uint32_t)pb.N + col;
    }
  };
  if constexpr (BF16) {
    // bf16: the wave's 64 x 64 tile is staged in LDS (the ring is free once
    // every wave has passed this barrier), rows padded by 16 bytes, and
    // stored 16 bytes per lane: each instruction writes 8 whole 128-byte
    // row segments instead of 16 scattered bytes per row.
    constexpr int SR = 64 * 2 + 16;
    static_assert(NWAVE * 64 * SR <= NSTAGE * 2 * TILE, "staging must fit the ring");
    __syncthreads();
    char* st = smem + wave * 64 * SR;
#pragma unroll
    for (int im = 0; im < 2; ++im)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(acc[jn][im][4 * g + r] + bv[jn][g][r]);
          *reinterpret_cast<bf16x4*>(st + (32 * im + li) * SR + (32 * jn + 8 * g + 4 * hi) * 2) = o4;
        }
    // The staging area belongs to this wave: order its writes before the
    // reads (LDS operations of a wave complete in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (col0 + 64 * wc < pb.N) {
#pragma unroll
      for (int rep = 0; rep < 8; ++rep) {
        const int rr = rep * 8 + lane / 8, c = lane % 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + rr * SR + c * 16);
        const uint32_t off = c_off((uint32_t)(row0 + 64 * wr + rr), (uint32_t)(col0 + 64 * wc + 8 * c));
        store_result(v, rc, (int)(off * ES), batch.stream_out);
      }
    }
  } else {
#pragma unroll
    for (int im = 0; im < 2; ++im) {
      const uint32_t row = (uint32_t)(row0 + 64 * wr + 32 * im + li);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col0 + 64 * wc + 32 * jn + 8 * g + 4 * hi;
          if (col >= pb.N) continue;
          const uint32_t off = c_off(row, (uint32_t)col);
          f32x4 o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = acc[jn][im][4 * g + r] + bv[jn][g][r];
          store_result(__builtin_bit_cast(u32x4, o4), rc, (int)(off * ES), batch.stream_out);
        }
    }
  }
}

template <typename T, bool A_HEADS, bool C_HEADS>
static hipError_t launch_proj_t(const ProjBatch& b_in, int count, void* stream) {
  ProjBatch b = b_in;
  int64_t out_bytes = 0;
  for (int i = 0; i < count; ++i) out_bytes += (int64_t)b.p[i].M * b.p[i].N * (int64_t)sizeof(T);
  b.stream_out = out_bytes <= kStreamOutMaxBytes;
  int tiles = 0;
  for (int i = 0; i < count; ++i) {
    const int t = ((b.p[i].M + proj::BM - 1) / proj::BM) * ((b.p[i].N + proj::BN - 1) / proj::BN);
    tiles = t > tiles ? t : tiles;
  }
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((proj_gemm_kernel<T, A_HEADS, C_HEADS>), dim3(tiles, count), dim3(256), 0,
                     (hipStream_t)stream, b);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjBatch& b, int count, bool bf16, bool a_heads, bool c_heads,
                       void* stream) {
  if (bf16) {
    if (a_heads) return launch_proj_t<__bf16, true, false>(b, count, stream);
    return c_heads ? launch_proj_t<__bf16, false, true>(b, count, stream)
                   : launch_proj_t<__bf16, false, false>(b, count, stream);
  }
  if (a_heads) return launch_proj_t<float, true, false>(b, count, stream);
  return c_heads ? launch_proj_t<float, false, true>(b, count, stream)
                 : launch_proj_t<float, false, false>(b, count, stream);
}

}  // namespace mha
