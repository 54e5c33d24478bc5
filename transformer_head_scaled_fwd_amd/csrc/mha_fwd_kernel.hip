// mha_fwd_kernel.hip -- fused attention forward for gfx950 (MI355X).
//
// One workgroup computes BR query rows of one (batch, head) with NW wave64s,
// each owning 32 rows.  It walks the key axis in blocks of BC = 64 keys.
// Usually every wave has rows of its own (BR = 32 NW); on grids too small
// to give each SIMD more than one wave, the waves form two key groups over
// the same BR = 16 NW rows, each walking every other key block, and merge
// their partial softmax sums at the end.  Per block:
//
//   stage    K and V blocks -> LDS, row-major, by buffer->LDS direct loads
//            (no register staging), in a ring of NSTAGE stages so that a
//            block streams in one or two blocks ahead of its use; one
//            barrier per block;
//   scores   S^T = K Q^T on MFMA (32x32 tiles, fp32 accumulate), Q held in
//            registers for the whole walk;
//   bias     optional: minus slope_t * |p_i - j| (ALiBi, "第2章：完整的
//            Transformer 架构" §5.3);
//   mask     -inf where j >= L_b or (causal and j > p_i)
//            ("Transformer: 详解" §3.4, §5.3), where the query's position
//            p_i is i (top-left alignment) or i + L_b - n (bottom-right: the
//            n queries are the last tokens of a sequence of L_b, as in
//            decoding against a key/value cache);
//   softmax  online: running row max and sum in fp32, exp2 with the scale
//            and log2(e) folded into one FMA ("Transformer" wiki page: mixed
//            precision needs the blockwise, online softmax).  A block's
//            weights are taken against the running max as it stands; only
//            when one of them could exceed 2^16 (its lane's block sum does)
//            is the block max formed, the running max raised and the output
//            rescaled.  A distance bias raises a row's max block after block
//            towards the diagonal: causal rows therefore walk their keys
//            backwards, from the diagonal down, and keep the weights-first
//            path; without a mask the block max is formed every block;
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
//
// Grouped K/V heads (GQA / MQA: hugogu wiki "Transformer", table of
// attention optimisations; "序列建模架构的演进与变革（二）" §3.8): query head
// t reads K/V head t / group.  On request the epilogue also stores each
// row's log-sum-exp of its scaled, biased, valid scores, from which a second
// pass can rebuild the weights.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mha_launch.h"
#include "mha_tiles.h"

namespace mha {

// Per-wave state of the key walk: 32 query rows, one per lane pair.  With
// KS key groups the wave reads key blocks kg, kg + KS, kg + 2 KS, ...: its
// j-th block is block j KS + kg, held in ring stage j.
template <typename T, int D, int NW, int KS, bool CAUSAL, bool ALIBI>
struct Walk {
  using G = Geo<T, D, NW, KS>;
  using P = Phase<T, D>;
  static constexpr int NS = P::NS;
  // Causal attention with a distance bias walks its keys backwards, from
  // the diagonal down to key 0.  The bias is then largest in the first
  // blocks a row sees, so its running max is set there and later blocks
  // can keep it (the weights-first softmax below); walked forwards, the max
  // rises block after block towards the diagonal.
  static constexpr bool REV = CAUSAL && ALIBI;
  // With REV, bf16 takes the part of the bias that varies within a 32-key
  // tile, sr * (key offset within the tile), as the initial value of the
  // score MFMAs (the accumulator input, the same for every tile), so that
  // only a per-row shift per tile is left for the vector ALU.
  static constexpr bool BIAS_MFMA = REV && G::BF16;

  const char* ktiles;  // LDS: K ring, NSTAGE stages
  const char* vtiles;  // LDS: V ring, NSTAGE stages
  int lane, li, hi;
  int kg;              // key group of the wave
  int prow_w;          // position of the first query row of the wave
  int prow;            // position of this lane's query row
  int row_lim;         // first invalid key of this lane's row
  int L;               // valid keys of the sequence
  int wave_nkb;        // key blocks this wave reads (its own, every KS-th)
  int nst;             // ring stages the workgroup walks
  int j0;              // first step of this wave's walk: 0, or past the end if empty
  int j1;              // one past its last step
  float sl2;           // scale * log2(e)
  float sr;            // ALiBi slope / scale (raw-score units)
  u32x4 qf[P::NQF];    // Q fragments
  uint32_t ko[P::NKO]; // K operand offsets within a tile (bf16)
  f32x16 o[D / 32];    // O^T accumulator
  float m_run;         // running max of scale*log2(e)*s (per row)
  float m_sub;         // what the weights subtract: m_run, or 0 while it is -inf
  float l_run;         // this lane's share of the row sum
  f32x16 cb;           // BIAS_MFMA: sr * (key offset within the 32-key tile)

  // Ring stage (of KS blocks) that step j walks.
  MHA_MEMBER int stage_of(int j) const { return REV ? nst - 1 - j : j; }
  // Key block of this wave at step j.
  MHA_MEMBER int block_of(int j) const { return stage_of(j) * KS + kg; }

  // gb: key block index (keys gb * BC onwards)
  MHA_MEMBER bool needs_mask(int gb) const {
    return (gb * BC + BC > L) || (CAUSAL && gb * BC + BC - 1 > prow_w);
  }
  // the wave's j-th block: ring stage j % NSTAGE, block kg within the stage
  MHA_MEMBER const char* k_tile(int j) const {
    return ktiles + (j % G::NSTAGE) * G::TILE + kg * (BC * G::ROWB);
  }
  MHA_MEMBER const char* v_tile(int j) const {
    return vtiles + (j % G::NSTAGE) * G::TILE + kg * (BC * G::ROWB);
  }

  // Softmax bookkeeping for a block whose raw row max is mx (the first
  // block, and blocks whose weights against the running max grew too
  // large): the running max is raised only when the block max exceeds it by
  // more than TAU.
  // Returns the factor alpha by which earlier sums and outputs must be
  // multiplied (1 when the max stays); the sum is rescaled here, the output
  // by the caller once the PV MFMAs that still add to it have been issued.
  MHA_MEMBER float raise_max(float mx, bool& grew) {
    const float mx2 = mx * sl2;  // -inf stays -inf (sl2 > 0)
    grew = mx2 > m_run + TAU;
    const float m_new = grew ? mx2 : m_run;
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    m_sub = (m_new == -__builtin_inff()) ? 0.0f : m_new;
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
  MHA_MEMBER float msub() const { return m_sub; }

  // What the wave's scores of tile jt at step j exceed their biased values
  // by, in raw score units: with BIAS_MFMA the scores carry sr * (key
  // offset within the tile) but not the rest of the bias,
  // -sr * (p_i - first key of the tile - 4hi), which is the same for all of
  // a lane's keys of the tile (every key a causal row sees lies at or before
  // it, so the distance is p_i - j).
  MHA_MEMBER float shift(int j, int jt) const {
    if constexpr (BIAS_MFMA) return sr * (float)(prow - block_of(j) * BC - 32 * jt - 4 * hi);
    else return 0.0f;
  }
  // Raw block max of the lane's biased scores at step j.
  MHA_MEMBER float block_max(const f32x16 (&s)[NS], int j) const {
    if constexpr (BIAS_MFMA) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int jt = 0; jt < NS; ++jt) mx = fmaxf(mx, P::tile_max(s[jt]) - shift(j, jt));
      return mx;
    } else {
      return P::lane_max(s);
    }
  }
  // Weights of the scores of step j against the running max m_sub (with
  // BIAS_MFMA, plus each tile's shift).
  MHA_MEMBER void weights_at(typename P::PFrag& pf, const f32x16 (&s)[NS], int j, float& l) const {
    if constexpr (BIAS_MFMA) {
      float ms[NS];
#pragma unroll
      for (int jt = 0; jt < NS; ++jt) ms[jt] = __builtin_fmaf(sl2, shift(j, jt), m_sub);
      P::weights(pf, s, sl2, ms, l);
    } else {
      P::weights(pf, s, sl2, m_sub, l);
    }
  }

  // Scores of the tile at kt (with BIAS_MFMA, started from cb).
  MHA_MEMBER void scores_at(f32x16 (&s)[NS], const char* kt) const {
    if constexpr (BIAS_MFMA) P::template scores_ko<true>(s, kt, qf, ko, &cb);
    else if constexpr (G::BF16) P::scores_ko(s, kt, qf, ko);
    else P::scores(s, kt, qf, li, hi);
  }

  // Distance bias and mask of the scores of the wave's step j.
  MHA_MEMBER void bias_and_mask(f32x16 (&s)[NS], int j) const {
    const int gb = block_of(j);
    if constexpr (ALIBI && !BIAS_MFMA) P::bias(s, (float)(prow - gb * BC - 4 * hi), sr);
    if (needs_mask(gb)) P::mask(s, row_lim - gb * BC - 4 * hi);
  }

  // Scores, mask, running max and weights of the wave's first block, at
  // step j.
  MHA_MEMBER void first_block(typename P::PFrag& pf, int j) {
    f32x16 s[NS];
    if constexpr (BIAS_MFMA) scores_at(s, k_tile(j));
    else P::scores(s, k_tile(j), qf, li, hi);
    bias_and_mask(s, j);
    bool grew;
    raise_max(pair_max(block_max(s, j)), grew);  // nothing accumulated yet
    weights_at(pf, s, j, l_run);
  }

  // PV of the wave's block kb (weights in pf_cur) and, when the wave reads
  // a block kb+1, its scores, mask, running max and weights into pf_nxt.
  //
  // ST = kb % NSTAGE, a constant in the loop (unrolled by the ring depth), so
  // that with the precomputed K offsets every tile read is a register plus
  // an immediate offset.
  template <int ST>
  MHA_MEMBER void step(int kb, const typename P::PFrag& pf_cur, typename P::PFrag& pf_nxt) {
    const int kgo = KS == 1 ? 0 : kg * (BC * G::ROWB);
    const char* kt_next = ktiles + ((ST + 1) % G::NSTAGE) * G::TILE + kgo;
    const char* vt_cur = vtiles + ST * G::TILE + kgo;
    if (kb + 1 < j1) {
      f32x16 s[NS];
      scores_at(s, kt_next);
      P::prefetch_k();
      bias_and_mask(s, kb + 1);
      P::pv(o, vt_cur, pf_cur, lane);
      if constexpr (ALIBI && !REV) {
        // A distance bias raises the row max block after block on the way
        // to the diagonal: form the block max every block.
        bool grew;
        const float alpha = raise_max(pair_max(P::lane_max(s)), grew);
        P::weights(pf_nxt, s, sl2, msub(), l_run);
        P::pin(pf_nxt);
        rescale_output(alpha, grew);
        return;
      }
      // Weights against the running max as it stands.  Every weight is at
      // most the lane's block sum, so while no lane's sum exceeds 2^16 the
      // running max can stay; otherwise the whole wave takes the exact path:
      // raise the max, recompute the weights, rescale.
      //
      // Walked backwards, a row whose first blocks lie past its diagonal
      // meets its first valid key later, with no running max: its weights
      // are then taken against 0 and may all have underflowed to 0, so their
      // sum cannot flag it; its valid keys are those below row_lim, so a
      // block holding one of them takes the exact path too.  Walked
      // forwards, the first block holds key 0 and leaves every row with a
      // valid key with a max.
      float lb = 0.0f;
      weights_at(pf_nxt, s, kb + 1, lb);
      P::pin(pf_nxt);
      bool slow = lb > 65536.0f;
      if constexpr (REV)
        slow = slow || (m_run == -__builtin_inff() && block_of(kb + 1) * BC < row_lim);
      if (__any(slow)) {
        bool grew;
        const float alpha = raise_max(pair_max(block_max(s, kb + 1)), grew);
        lb = 0.0f;
        weights_at(pf_nxt, s, kb + 1, lb);
        P::pin(pf_nxt);
        rescale_output(alpha, grew);
      }
      l_run += lb;
    } else {
      P::pv(o, vt_cur, pf_cur, lane);
    }
  }
};

// Arguments of the forward kernel beyond the tensors.
struct FwdParams {
  int H;              // query heads
  int H_kv;           // K/V heads
  int group;          // query heads per K/V head (H / H_kv)
  int BH;             // batch x query heads
  int n, m;           // query rows, key rows per head
  int nqb;            // query blocks per head
  int bottom_right;   // causal alignment: 0 top-left, 1 bottom-right
  int units_per_xcd;  // K/V heads (batch x H_kv) per XCD, or 0: plain order
  int unit_group;     // K/V heads one XCD works on at a time
  float scale;        // the caller's scale
  float scale_log2;   // scale * log2(e)
  int stream_out;     // results written through to memory (kStoreOut)
  // Divisors of the block-index decode, fixed at launch: BH, H and group
  // (plain order); group * nqb * unit_group, group * unit_group and H_kv
  // (pinned order).
  FastDiv div_bh, div_h, div_group, div_gw, div_pg, div_hkv;
};

// Resident workgroups per CU: one for 8 waves, or when the fp32 d = 128
// tiles take 128 KiB of LDS; otherwise two.
template <typename T, int D, int NW>
constexpr int fwd_wg_per_cu() {
  return (NW == 8 || (sizeof(T) == 4 && D == 128)) ? 1 : 2;
}

template <typename T, int D, int NW, int KS, bool CAUSAL, bool ALIBI>
__global__ void __launch_bounds__(64 * NW, (fwd_wg_per_cu<T, D, NW>()))
attn_fwd_kernel(const T* __restrict__ Qp, const T* __restrict__ Kp,
                const T* __restrict__ Vp, const int32_t* __restrict__ key_lens,
                const float* __restrict__ alibi_slopes, T* __restrict__ Op,
                float* __restrict__ lse, FwdParams prm) {
  using G = Geo<T, D, NW, KS>;
  using W = Walk<T, D, NW, KS, CAUSAL, ALIBI>;
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
  const int rg = wave % G::RG;  // row group: query rows 32 rg .. 32 rg + 31
  w.kg = wave / G::RG;          // key group
  w.lane = tid % 64;
  w.li = w.lane % 32;  // query row within the wave's 32 (MFMA column)
  w.hi = w.lane / 32;  // which half of the k / row groups this lane holds
  const int lane = w.lane, li = w.li, hi = w.hi;

  const int n = prm.n, m = prm.m, nqb = prm.nqb;
  const uint32_t bid = blockIdx.x;
  // Query-block rank (0 = first launched), batch, query head and K/V head of
  // the workgroup.  The divisions are by launch constants (div_by), so the
  // loads below wait on a few scalar instructions instead of division
  // sequences.
  int qbr, b, t, bkv;
  if (prm.units_per_xcd > 0) {
    // Workgroups go to the 8 XCDs round-robin in index order, and each XCD
    // has its own L2.  Pin every K/V head (a "unit": its group of query heads
    // times all their query blocks) to one XCD, x = unit % 8, and let the XCD
    // work through its units unit_group at a time, query-block rank first
    // within the group, so that the workgroups running together on an XCD
    // read the same K/V rows.
    const uint32_t x = bid % 8, r = bid / 8;
    const uint32_t k = div_by(r, prm.div_gw);       // unit group
    const uint32_t w_in = r - k * prm.div_gw.d;   // workgroup within it
    qbr = (int)div_by(w_in, prm.div_pg);
    const uint32_t rest = w_in - (uint32_t)qbr * prm.div_pg.d;  // query head within the group
    const uint32_t uq = div_by(rest, prm.div_group);
    const uint32_t u = x + 8 * (k * prm.unit_group + uq);       // K/V head: batch * H_kv + g
    const uint32_t bb = div_by(u, prm.div_hkv);
    b = (int)bb;
    t = (int)((u - bb * prm.H_kv) * prm.group + (rest - uq * prm.group));
    bkv = (int)u;
  } else {
    qbr = (int)div_by(bid, prm.div_bh);
    const uint32_t bh = bid - (uint32_t)qbr * prm.BH;
    b = (int)div_by(bh, prm.div_h);
    t = (int)(bh - (uint32_t)b * prm.H);
    bkv = b * prm.H_kv + (int)div_by(t, prm.div_group);
  }
  const int bh = b * prm.H + t;
  // Heaviest query blocks first for causal attention: the work of a block
  // grows with its index, so launching them in reverse evens out the tail.
  const int qb = CAUSAL ? (nqb - 1 - qbr) : qbr;
  const int q0 = qb * BR;
  const int row_w = q0 + rg * kRowsPerWave;
  const int my_row = row_w + li;

  // Q fragments (MFMA B operand of S^T = K Q^T), kept in registers.  Their
  // loads go out first: they do not depend on the sequence length, so their
  // latency overlaps that of the length read the K/V loads wait for.
  const size_t head_q = (size_t)bh * (size_t)n * D;
  const auto rq = make_rsrc(Qp + head_q, (uint32_t)n * D * ES);
  P::issue_q(w.qf, rq, my_row, hi);

  int L = m;
  if (key_lens != nullptr) {
    L = key_lens[b];
    L = L < 0 ? 0 : (L > m ? m : L);
  }
  w.L = L;
  // Position of query row i: i + off.
  const int off = (CAUSAL && prm.bottom_right) ? L - n : 0;
  const int kend = CAUSAL ? max(0, min(L, q0 + off + BR)) : L;
  const int nkb = (kend + BC - 1) / BC;  // key blocks of the workgroup
  const int nst = (nkb + KS - 1) / KS;    // ring stages it walks
  w.prow_w = row_w + off;
  w.prow = my_row + off;
  // Key blocks any row of this wave's row group can see, then those of
  // them that belong to the wave's key group.
  const int vis = CAUSAL ? max(0, min(nkb, (w.prow_w + kRowsPerWave + BC - 1) / BC)) : nkb;
  w.wave_nkb = vis > w.kg ? (vis - w.kg + KS - 1) / KS : 0;
  // Steps of the wave: the first wave_nkb forwards.  Backwards (REV) every
  // wave with a key to see walks all the workgroup's stages from the
  // diagonal down: the first one or two stages lie past the last key of a
  // wave whose rows end before them and are masked out whole for it, which
  // costs their MFMAs but keeps the first block out of the loop (and the
  // registers of a second first-block path with it).  An empty walk starts
  // past the end.
  w.nst = nst;
  w.j0 = W::REV ? (w.wave_nkb > 0 ? 0 : nst + 1) : 0;
  w.j1 = W::REV ? nst : w.wave_nkb;
  w.row_lim = CAUSAL ? min(L, my_row + off + 1) : L;
  w.sl2 = prm.scale_log2;
  w.sr = ALIBI ? alibi_slopes[t] / prm.scale : 0.0f;

  // Buffer resources: out-of-range loads read 0 (also into LDS) and
  // out-of-range stores are dropped, so rows >= n (queries) and >= L (keys,
  // values) need no branch and padded keys are never read from memory.
  const size_t head_k = (size_t)bkv * (size_t)m * D;
  const uint32_t kv_bytes = (uint32_t)L * D * ES;  // rows >= L read as 0
  const auto ro = make_rsrc(Op + head_q, (uint32_t)n * D * ES);
  const T* kbase = Kp + head_k;
  const T* vbase = Vp + head_k;

  // Loads of ring stage j of the keys and of the values into their slots.
  auto load_k = [&](int j) {
    G::template stage<true>(lds_k + (j % G::NSTAGE) * G::TILE, kbase, kv_bytes, w.stage_of(j),
                            wave, lane);
  };
  auto load_v = [&](int j) {
    G::template stage<false>(lds_v + (j % G::NSTAGE) * G::TILE, vbase, kv_bytes, w.stage_of(j),
                             wave, lane);
  };

  // The first key/value blocks, then the wait for Q; the wait before the
  // first barrier below covers the key/value loads.
  if (nst > 0) {
    for (int j = 0; j <= DIST && j < nst; ++j) load_k(j);
    for (int j = 0; j < DIST && j < nst; ++j) load_v(j);
  }
  P::pin_q(w.qf);

#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) w.o[t][e] = 0.0f;
  w.m_run = -__builtin_inff();
  w.m_sub = 0.0f;
  w.l_run = 0.0f;
  if constexpr (BF16) P::k_offsets(w.ko, li, hi);
  if constexpr (W::BIAS_MFMA) {
#pragma unroll
    for (int e = 0; e < 16; ++e) w.cb[e] = w.sr * (float)(8 * (e / 4) + e % 4);
  }

  // Pipeline: iteration kb reads K(kb+1) and V(kb).  It issues the loads of
  // K(kb+1+DIST) and V(kb+DIST), which go to the ring slots of K(kb) and
  // V(kb-1), both last read before the barrier that ended iteration kb-1.
  // Before its own barrier it waits for the loads issued DIST-1 iterations
  // earlier, i.e. for K(kb+2) and V(kb+1).  Two weight buffers alternate,
  // unrolled by two.
  typename P::PFrag pa, pb;
  if (nst > 0) {
    G::template wait_loads<0>();
    __syncthreads();
    if (W::REV ? (w.j0 == 0) : (0 < w.wave_nkb)) w.first_block(pa, 0);
    // K(0) is consumed before its slot is refilled, by the load of stage
    // 1 + NSTAGE - 1 in the first iteration; a walk of at most NSTAGE
    // stages never refills it.
    if (nst > G::NSTAGE) __syncthreads();
  }

  // Issue this iteration's loads; returns how many tiles were issued.
  auto issue = [&](int kb) -> int {
    int issued = 0;
    if (kb + DIST < nst) {
      load_v(kb + DIST);
      issued = 1;
      if (kb + 1 + DIST < nst) {
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
  for (int kb = 0; kb < nst; kb += 2) {
    int issued = issue(kb);
    static_assert(G::NSTAGE == 2, "the loop alternates two ring stages");
    if constexpr (W::REV) {
      if (kb >= w.j0) w.template step<0>(kb, pa, pb);
    } else if (kb < w.wave_nkb) {
      w.template step<0>(kb, pa, pb);
    }
    publish(issued);
    if (kb + 1 >= nst) break;
    issued = issue(kb + 1);
    if constexpr (W::REV) {
      if (kb + 1 >= w.j0) w.template step<1>(kb + 1, pb, pa);
    } else if (kb + 1 < w.wave_nkb) {
      w.template step<1>(kb + 1, pb, pa);
    }
    publish(issued);
  }

  // ---- two key groups: key group 1 hands its running max, row-sum share
  // and unnormalised output to key group 0 through LDS (the ring is idle:
  // every wave has passed the loop's last barrier, and with no stage walked
  // nothing was ever staged there).  Both halves are exact partial softmax
  // sums against their own reference max m_g, so the row's sums are
  // sum_g 2^(m_g - M) l_g and sum_g 2^(m_g - M) O_g with M = max_g m_g; a
  // group that saw no valid key has m_g = -inf and contributes 0.
  constexpr int MERGE_BYTES = KS == 2 ? (2 + (D / 32) * 16) * G::RG * 64 * 4 : 0;
  if constexpr (KS == 2) {
    float* mg = reinterpret_cast<float*>(smem);
    // element e of this lane, row group rg: consecutive lanes, consecutive words
    auto at = [&](int e) -> float& { return mg[(e * G::RG + rg) * 64 + lane]; };
    if (w.kg == 1) {
      at(0) = w.m_run;
      at(1) = w.l_run;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) at(2 + 16 * t + e) = w.o[t][e];
    }
    __syncthreads();
    if (w.kg == 1) return;
    const float m1 = at(0), l1 = at(1);
    const float mx = fmaxf(w.m_run, m1);
    const float f0 = (w.m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(w.m_run - mx);
    const float f1 = (m1 == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
    w.l_run = w.l_run * f0 + l1 * f1;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) w.o[t][e] = w.o[t][e] * f0 + at(2 + 16 * t + e) * f1;
    w.m_run = mx;
  }

  // ---- epilogue: divide by the row sum (0 when no key was valid), store
  const float l_tot = pair_sum(w.l_run);
  const float inv = (l_tot > 0.0f) ? (1.0f / l_tot) : 0.0f;
  if (lse != nullptr && hi == 0) {
    // ln(sum_j exp(scaled score)) = ln 2 * (m_run + log2(l)), m_run in log2 units.
    const float v = (l_tot > 0.0f) ? 0.6931471805599453f * (w.m_run + __builtin_amdgcn_logf(l_tot))
                                   : -__builtin_inff();
    const auto rl = make_rsrc(lse + (size_t)bh * n, (uint32_t)n * 4);
    store_result(__builtin_bit_cast(uint32_t, v), rl, (int)((uint32_t)my_row * 4),
                 prm.stream_out);
  }
  // O rows staged in LDS when they fit the (now idle) K/V ring, past the
  // merge area, rows padded by 16 bytes, then stored 16 bytes per lane:
  // each store instruction writes whole row segments (bf16: 4 rows of
  // d = 128 or 8 of d = 64) instead of 16 scattered bytes per row.  Every
  // wave has passed the block loop's last barrier, so no wave still reads
  // the ring (and with no key block nothing was ever staged there).
  constexpr int OSR = D * ES + 16;
  if constexpr (MERGE_BYTES + G::RG * kRowsPerWave * OSR <= G::LDS_BYTES) {
    char* st = smem + MERGE_BYTES + rg * kRowsPerWave * OSR;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        char* dst = st + li * OSR + (ct * 32 + 8 * g + 4 * hi) * ES;
        if constexpr (BF16) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(w.o[ct][4 * g + r] * inv);
          *reinterpret_cast<bf16x4*>(dst) = v;
        } else {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = w.o[ct][4 * g + r] * inv;
          *reinterpret_cast<f32x4*>(dst) = v;
        }
      }
    // The staging area belongs to this wave: order its writes before the
    // reads (LDS operations of a wave complete in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int CPRO = D * ES / 16;  // 16-byte chunks per row
    constexpr int RPI = 64 / CPRO;     // rows per store instruction
#pragma unroll
    for (int rep = 0; rep < kRowsPerWave / RPI; ++rep) {
      const int rr = rep * RPI + lane / CPRO, c = lane % CPRO;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + rr * OSR + c * 16);
      // rows >= n fall outside the O resource and are dropped
      const uint32_t off = ((uint32_t)(row_w + rr) * D) * ES + c * 16;
      store_result(v, ro, (int)off, prm.stream_out);
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t off = ((uint32_t)my_row * D + ct * 32 + 8 * g + 4 * hi) * ES;
        if constexpr (BF16) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(w.o[ct][4 * g + r] * inv);
          store_result(__builtin_bit_cast(u32x2, v), ro, (int)off, prm.stream_out);
        } else {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = w.o[ct][4 * g + r] * inv;
          store_result(__builtin_bit_cast(u32x4, v), ro, (int)off, prm.stream_out);
        }
      }
  }
}

template <typename T, int D, int NW, int KS, bool CAUSAL, bool ALIBI>
static hipError_t launch_one(const LaunchArgs& a) {
  constexpr int BR = Geo<T, D, NW, KS>::BR;
  FwdParams prm;
  prm.H = (int)a.H;
  prm.H_kv = (int)a.H_kv;
  prm.group = (int)(a.H / a.H_kv);
  prm.BH = (int)(a.B * a.H);
  prm.n = (int)a.n;
  prm.m = (int)a.m;
  prm.nqb = (int)((a.n + BR - 1) / BR);
  prm.bottom_right = a.mode == 2;
  // XCD pinning of K/V heads (see the kernel) when they split evenly over
  // the 8 XCDs.  unit_group: enough K/V heads per XCD to fill its 32 CUs;
  // causal, further up to the most heads whose K/V rows stay within twice
  // an XCD's 4 MB L2: the XCD then runs heaviest first across more heads,
  // which balances query blocks of unequal work over its CUs, while their
  // K/V rows still mostly hit in L2.
  const int64_t units = a.B * a.H_kv;
  prm.units_per_xcd = 0;
  prm.unit_group = 1;
  // The plain order already keeps a head's query blocks together on one XCD
  // when one head's blocks fill it; pinning pays when they do not, or when
  // several query heads share a K/V head.
  const int64_t slots = 32 * fwd_wg_per_cu<T, D, NW>();  // resident workgroups per XCD
  const int64_t per_unit = (int64_t)prm.nqb * (a.H / a.H_kv);
  if (units % 8 == 0 && (a.H != a.H_kv || per_unit < slots)) {
    prm.units_per_xcd = (int)(units / 8);
    while ((int64_t)prm.unit_group * per_unit < slots && prm.units_per_xcd % (2 * prm.unit_group) == 0)
      prm.unit_group *= 2;
    if (a.mode != 0) {
      const int64_t unit_bytes = a.m * a.d * 2 * (int64_t)sizeof(T);  // K and V rows of a head
      while (prm.units_per_xcd % (2 * prm.unit_group) == 0 &&
             2 * prm.unit_group * unit_bytes <= ((int64_t)8 << 20))
        prm.unit_group *= 2;
    }
  }
  prm.scale = a.scale;
  prm.scale_log2 = a.scale_log2;
  prm.div_bh = fast_div((uint32_t)prm.BH);
  prm.div_h = fast_div((uint32_t)prm.H);
  prm.div_group = fast_div((uint32_t)prm.group);
  prm.div_gw = fast_div((uint32_t)(prm.unit_group * prm.group * prm.nqb));
  prm.div_pg = fast_div((uint32_t)(prm.unit_group * prm.group));
  prm.div_hkv = fast_div((uint32_t)prm.H_kv);
  const int64_t blocks = (int64_t)prm.nqb * a.B * a.H;
  // Results written through to memory when they fit the L2s (kStoreOut).
  prm.stream_out = a.B * a.H * a.n * a.d * (int64_t)sizeof(T) <= kStreamOutMaxBytes;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, NW, KS, CAUSAL, ALIBI>), dim3((unsigned)blocks),
                     dim3(64 * NW), 0, (hipStream_t)a.stream, (const T*)a.Q, (const T*)a.K,
                     (const T*)a.V, a.key_lens, a.alibi_slopes, (T*)a.O, a.lse, prm);
  return hipGetLastError();
}

template <typename T, int D, int NW, int KS>
static hipError_t launch_variant(const LaunchArgs& a) {
  const bool causal = a.mode != 0;
  if (a.alibi_slopes != nullptr)
    return causal ? launch_one<T, D, NW, KS, true, true>(a) : launch_one<T, D, NW, KS, false, true>(a);
  return causal ? launch_one<T, D, NW, KS, true, false>(a) : launch_one<T, D, NW, KS, false, false>(a);
}

// Workgroup shape as forward_variant (mha_host.cpp) chooses it.
template <typename T, int D>
static hipError_t launch_d(const LaunchArgs& a) {
  const FwdVariant v = forward_variant(sizeof(T) == 2, D, a.B, a.H, a.n, a.m, a.mode);
  if constexpr (sizeof(T) == 2) {
    if (v.nw == 8 && v.ks == 1) {
      if constexpr (D == 128) return launch_variant<T, D, 8, 1>(a);
    }
    if (v.nw == 8 && v.ks == 2) return launch_variant<T, D, 8, 2>(a);
  }
  return launch_variant<T, D, 4, 1>(a);
}

template <typename T>
static hipError_t launch_t(const LaunchArgs& a) {
  return a.d == 64 ? launch_d<T, 64>(a) : launch_d<T, 128>(a);
}

hipError_t launch_attention(const LaunchArgs& a) {
  return a.bf16 ? launch_t<__bf16>(a) : launch_t<float>(a);
}

}  // namespace mha
