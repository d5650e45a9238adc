// attn_fwd.hip -- forward attention kernel for gfx950.
//
// Computes, per query head h and query row i with allowed key set A_i,
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j   and   LSE_i = ln sum_j exp(scale * q_i . k_j),
// the standard softmax attention whose quadratic cost the LongCA-bench pages
// start from (section 1), under a compiled mask.  A row with no allowed key
// gets O = 0, LSE = -inf.
//
// Work decomposition: one work item per (query head, 128-row query tile),
// run by one workgroup of four wave64s of 32 rows each (two workgroups per
// CU at head dim 128, three at 64 and one at 256).  With a caller workspace
// the workgroups claim their items from per-XCD queues (claim_item);
// without one, workgroup b runs item b.  The workgroup walks the query
// tile's list of non-EMPTY 64-key tiles.  K and V tiles reach LDS by direct
// global->LDS loads into a double buffer: the loads of tile t+1 are issued
// right after the barrier that opens tile t, so they overlap tile t's
// arithmetic and no registers are spent on staging.  Per key tile each wave
//   1. forms S^T = K Q^T (keys x queries) with bf16 MFMA; each lane then holds
//      one query row, so the row max and row sum stay in the lane (plus one
//      permlane32 swap with the other half-wave);
//   2. masks PARTIAL tiles (and the ragged last key tile) with -inf;
//   3. updates the online softmax in the exp2 domain against a lagging
//      reference max: P is formed first, and the block's max is taken (the
//      reference moved, the accumulator rescaled and P formed again) only
//      when a lane's block sum of P exceeds 2^8 or a row has no reference;
//   4. accumulates O^T += V^T P^T with P^T taken straight from registers as
//      the MFMA B operand and V^T read transposed from LDS.
#include "kernel_common.hpp"

namespace mad {

// NB: 32-row query blocks per wave (the workgroup's 128 rows are spread over
// 4 / NB waves).
#ifndef FWD_PRE_B
#define FWD_PRE_B 1
#endif
#ifndef FWD_PRE_C
#define FWD_PRE_C 3
#endif
// HM: the head-major item order (MHA masks whose tiles carry even work).
template <int D, int NB, bool HM>
__global__ __launch_bounds__(256 / NB, D == 64 ? 3 : 1) void fwd_kernel(const AttnParams P) {
  // Score steps of the next key block issued before a block's softmax starts
  // (stage B) and P V steps issued before the next block's softmax (stage C).
  constexpr int PRE_B = FWD_PRE_B < D / 16 - 1 ? FWD_PRE_B : D / 16 - 1;
  constexpr int PRE_C = FWD_PRE_C < D / 16 - 1 ? FWD_PRE_C : D / 16 - 1;
  constexpr int BM = BM0, BN = BN0, NKS = D / 16, NDB = D / 32, NW = 4 / NB;
  constexpr int KRS = tile_rs<D, TILE_ROWS>(), KT = tile_elems<D, TILE_ROWS>();
  constexpr int VRS = tile_rs<D, TILE_TR>(), VT = tile_elems<D, TILE_TR>();
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (KT + VT)];  // K0 V0 K1 V1

  // Work item -> (KV head g, query head e of its group, query tile of rank
  // `rank` in the longest-first order), arranged so that the workgroups
  // resident on an XCD share K / V tiles in its L2.  With a GQA group, eight
  // consecutive items (the group's query heads at one rank) share an XCD
  // (xcd_remap), so each XCD serves one KV head.  Masks without a group
  // (MHA) whose tiles carry even work (block-sparse masks, or every list of
  // one length as under FULL) run head by head instead (the HM variant),
  // ranks in turn over the XCDs: every XCD then works on the same one or two
  // heads at a time (ranks outermost put eight heads' K / V on each XCD; the
  // forward fetched 95 GB at 32K, b = 64, s = 0.8).  Masks with uneven tiles
  // keep ranks outermost, where the longest-first order balances the CUs.
  constexpr bool mha = HM;  // launched only for P.R == 1
  // With a workspace the item is claimed from the per-XCD queues (claim_item;
  // the grid holds more workgroups than items, and those that find every
  // queue empty exit); without one, workgroup b takes item b.
  __shared__ int claimed;
  if (threadIdx.x == 0) claimed = P.queue ? claim_item(P.queue, P.n_items) : (int)blockIdx.x;
  __syncthreads();
  const int item = __builtin_amdgcn_readfirstlane(claimed);  // uniform: in scalar registers
  if (item < 0) return;
  const int L = mha ? item : xcd_remap(item, P.n_items);
  const int e = mha ? 0 : L % P.R, t_ = mha ? L : L / P.R;
  const int g = mha ? t_ / P.t.nmajor : t_ % P.Hkv, rank = mha ? t_ % P.t.nmajor : t_ / P.Hkv;
  const int h = g * P.R + e;
  const int qt = sld(P.t.order + rank);
  const int mg = h / P.grp_div;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform
  const int row_base = qt * BM + w * 32 * NB;
  // Block-sparse masks: the keep bitmap rows of this lane's query blocks.
  const bool blocks = P.m.mode == MODE_BLOCKS;
  const uint64_t* krow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    krow[b] = blocks ? P.m.keep + ((size_t)mg * P.m.n_qb + P.m.row_qb[min(row_base + b * 32 + li, P.Tq - 1)]) *
                                      P.m.nw
                     : nullptr;

  const int32_t* ptr = P.t.ptr + (int64_t)mg * (P.t.nmajor + 1);
  const int beg = sld(ptr + qt), end = sld(ptr + qt + 1);
  const bf16* kg = P.k + (int64_t)g * P.k_head;
  const bf16* vg = P.v + (int64_t)g * P.v_head;
  const uint32_t smem_lds = lds_addr(smem);
  TileLoader<D, TILE_ROWS, NW, true> kload;
  TileLoader<D, TILE_TR, NW, false> vload;
  kload.init(P.k_tok, w, lane);
  vload.init(P.v_tok, w, lane);
  auto issue = [&](int kt, int buf) {
    const uint32_t kl = smem_lds + buf * (KT + VT) * 2;
    kload.issue(kl, kg, P.k_tok, kt * BN, P.Tk, w, lane);
    vload.issue(kl + KT * 2, vg, P.v_tok, kt * BN, P.Tk, w, lane);
  };
  if (beg < end) issue(sld(P.t.ent + beg) & 0x7fffffff, 0);

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16ks + 8hh .. +8].
  bf16x8 qf[NB][NKS];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = row_base + b * 32 + li;
    const bf16* src = P.q + (int64_t)min(row, P.Tq - 1) * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[b][ks] = ld16(src + 16 * ks);
  }

  f32x16 acc[NDB][NB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[db][b] = f32x16{};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  float muse[2] = {0.f, 0.f};  // the reference P is formed against (0 while mrow is -inf)

  for (int it = beg; it < end; ++it) {
    const int buf = (it - beg) & 1;
    const uint32_t ent = (uint32_t)sld(P.t.ent + it);
    const int kt = (int)(ent & 0x7fffffffu);
    const bool partial = (ent & ENT_PARTIAL) != 0;
    wait_vmem();
    __syncthreads();

    // Allowed-key masks of this lane's two rows (PARTIAL and ragged tiles
    // only), evaluated before the next tile's loads are issued so that the
    // mask table reads never wait behind them.
    // A block-sparse PARTIAL tile whose four wave strips are each FULL or
    // EMPTY carries the FULL strips as bits in aux: those waves run it as a
    // FULL tile and the others skip it, with no mask arithmetic.
    const bool ragged = (kt + 1) * BN > P.Tk;
    const int aux = partial ? sld(P.t.ent_aux + it) : -1;
    const bool parts = partial && !ragged && P.m.mode == MODE_BLOCKS && aux >= 0;
    const bool masked = (partial && !parts) || ragged;
    uint32_t mbits[2][2];
    if (masked) {
      if (blocks && partial) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint64_t kbits = keymask64_blocks(P.m, krow[b], row_base + b * 32 + li, kt * BN);
          mbits[b][0] = (uint32_t)kbits;
          mbits[b][1] = (uint32_t)(kbits >> 32);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            mbits[b][kb] = keymask32(P.m, aux, mg, partial, row_base + b * 32 + li, kt * BN + kb * 32, row_base,
                                     row_base + 32 * NB - 1);
      }
      wait_vmem();
    }
    if (it + 1 < end) issue(sld(P.t.ent + it + 1) & 0x7fffffff, buf ^ 1);
    if (parts && !((aux >> w) & 1)) continue;
    if (masked) {
      // A wave none of whose rows sees a key of this tile skips it (blocks
      // smaller than the tile leave whole waves masked): it only takes part
      // in the loads and barriers.
      uint32_t any = 0u;
#pragma unroll
      for (int b = 0; b < NB; ++b) any |= mbits[b][0] | mbits[b][1];
      if (__ballot(any != 0u) == 0ull) continue;
    }
    const bf16* Ks = smem + buf * (KT + VT);
    const bf16* Vs = Ks + KT;
    __builtin_amdgcn_sched_barrier(0);

    // Register r of s[kb][b] holds key kb*32 + 16(r/8) + 8hh + r%8 of row
    // b*32 + li.  Each key block's first product starts from an inline zero
    // (no register initialisation); masked (row, key) pairs are set to -inf
    // once the block's products are in, just before its max is taken.
    f32x16 s[2][NB];
    auto apply_mask = [&](int kb) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((mbits[b][kb] >> (16 * (r >> 3) + 8 * hh + (r & 7))) & 1u)) s[kb][b][r] = -INFINITY;
    };

    // LDS operand rings, read two MFMA steps ahead.  Phase-1 step st = (kb,
    // ks): the K row operand; phase-2 step st = (kb, t2, db): the V^T operand.
    bf16x8 kr[3], vr[3];
    auto ldk = [&](int st) {
      const int kb = st / NKS, ks = st % NKS;
      kr[st % 3] = ld16(Ks + (kb * 32 + li) * KRS + (16 * ks + 8 * hh));
    };
    auto ldv = [&](int st) {
      const int kb = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
      const int vrow = kb * 32 + 16 * t2 + 8 * hh + tr_row(lane), vcol = db * 32 + tr_col(lane);
      vr[st % 3] = ld_tr8(Vs + vrow * VRS + vcol, Vs + (vrow + 4) * VRS + vcol);
    };
    auto s_step = [&](int st) {  // S^T of key block st / NKS, k-step st % NKS, both query blocks
      const int kb = st / NKS, ks = st % NKS;
#pragma unroll
      for (int b = 0; b < NB; ++b) s[kb][b] = mfma32(kr[st % 3], qf[b][ks], ks == 0 ? f32x16{} : s[kb][b]);
    };
    bf16x8 pb[2][2][NB];  // P^T operands [kb][t2][b]
    auto pv_step = [&](int st) {  // O^T += V^T P^T for (kb, t2, db), both query blocks
      const int kb = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[db][b] = mfma32(vr[st % 3], pb[kb][t2][b], acc[db][b]);
    };
    // Online softmax in the exp2 domain against a lagging reference max per
    // row: p = exp2(s c - m_ref) is formed against the current reference
    // first.  Only when some lane's sum of its block's p exceeds SUM_LIMIT =
    // 2^8 (so that some p may), or some row of the wave has no reference yet
    // (mrow = -inf: p was formed against 0 and may have underflowed), does
    // the wave take the block's max: m_ref moves to it if larger, O and l are
    // rescaled by exp2(m_old - m_new) and the block's p are formed again.
    // Otherwise every p is at most 2^8 and no max is taken at all.  The
    // result is exact: O and l share the reference and LSE = m_ref + log2 l.
    constexpr float SUM_LIMIT = 256.f;
    constexpr int NE = 16 * NB;  // softmax elements per key block and lane
    float tsum[2][NB];           // per-lane sums of the block's p
    // P = exp2(s c - m) for elements e, e + 1 of key block kb (e = 16 b + r),
    // summed into tsum and written as bf16 into the P^T operand.
    auto softmax2 = [&](int kb, int e) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int b = (e + x) >> 4, r = (e + x) & 15;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][b][r], P.scale_log2, -muse[b]));
        tsum[kb][b] = r == 0 ? pv : tsum[kb][b] + pv;
        pb[kb][r >> 3][b][r & 7] = (bf16)pv;
      }
    };
    auto needs_max = [&](int kb) {
      bool need = false;
#pragma unroll
      for (int b = 0; b < NB; ++b) need |= !(tsum[kb][b] <= SUM_LIMIT) || mrow[b] == -INFINITY;
      return __ballot(need) != 0ull;
    };
    // The rare path: take block kb's max, move the reference, rescale O (all
    // products so far) and l, and form the block's p again.
    auto move_reference = [&](int kb) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][b][r]);
        const float mnew = fmaxf(mrow[b], pair_max(mx) * P.scale_log2);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrow[b] - mnew);
        mrow[b] = mnew;
        muse[b] = (mnew == -INFINITY) ? 0.f : mnew;
        lrow[b] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][b][r] *= alpha;
      }
#pragma unroll
      for (int e = 0; e < NE; e += 2) softmax2(kb, e);
    };

    ldk(0);
    ldk(1);
    __builtin_amdgcn_sched_barrier(0);
    // Stage A: scores of key block 0.
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      ldk(st + 2);
      s_step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Stage B: scores of key block 1 under the softmax of block 0.  Its first
    // PRE_B steps are issued before block 0's softmax starts, so the matrix
    // cores stay busy while the vector unit waits for block 0's last
    // products.
#pragma unroll
    for (int st = NKS; st < NKS + PRE_B; ++st) {
      if (st + 2 < 2 * NKS) ldk(st + 2);
      else ldv(st + 2 - 2 * NKS);
      s_step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(masked, 0)) apply_mask(0);
    constexpr int RB = NKS - PRE_B;                      // remaining stage-B steps
    constexpr int EB = 2 * ((NE / 2 + RB - 1) / RB);     // block-0 elements per remaining stage-B step (even)
#pragma unroll
    for (int st = NKS + PRE_B; st < 2 * NKS; ++st) {
      if (st + 2 < 2 * NKS) ldk(st + 2);
      else ldv(st + 2 - 2 * NKS);
      s_step(st);
#pragma unroll
      for (int e = (st - NKS - PRE_B) * EB; e < (st - NKS - PRE_B + 1) * EB && e < NE; e += 2) softmax2(0, e);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(needs_max(0), 0)) move_reference(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) lrow[b] += tsum[0][b];
    __builtin_amdgcn_sched_barrier(0);
    // Stage C: O^T += V^T P^T for key block 0 under the softmax of block 1
    // (whose reference check, and any rescale of the accumulator, waits until
    // block 0's products are in).  The wave runs it, up to block 1's check,
    // at raised issue priority: its exponentials then go ahead of the other
    // wave on the SIMD, whose stage A or D is matrix work alone.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < PRE_C; ++st) {
      ldv(st + 2);
      pv_step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(masked, 0)) apply_mask(1);
    constexpr int RC = 2 * NDB - PRE_C;                  // remaining stage-C steps
    constexpr int EC = 2 * ((NE / 2 + RC - 1) / RC);     // block-1 elements per remaining stage-C step (even)
#pragma unroll
    for (int st = PRE_C; st < 2 * NDB; ++st) {
      ldv(st + 2);
      pv_step(st);
#pragma unroll
      for (int e = (st - PRE_C) * EC; e < (st - PRE_C + 1) * EC && e < NE; e += 2) softmax2(1, e);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(needs_max(1), 0)) move_reference(1);
#pragma unroll
    for (int b = 0; b < NB; ++b) lrow[b] += tsum[1][b];
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // Stage D: O^T += V^T P^T for key block 1.
#pragma unroll
    for (int st = 2 * NDB; st < 4 * NDB; ++st) {
      if (st + 2 < 4 * NDB) ldv(st + 2);
      pv_step(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float lt = pair_sum(lrow[b]);
    const int row = row_base + b * 32 + li;
    if (row >= P.Tq) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    bf16* dst = P.o + ((int64_t)row * P.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v4;
#pragma unroll
        for (int x = 0; x < 4; ++x) v4[x] = (bf16)(acc[db][b][4 * rg + x] * inv);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * rg + 4 * hh) = v4;
      }
    if (hh == 0) P.lse[(int64_t)h * P.Tq + row] = lt > 0.f ? (mrow[b] + __log2f(lt)) * LN2 : -INFINITY;
  }
}

// 4 waves of 32 rows: 237 registers at D = 128, two waves per SIMD (one at
// D = 256, whose K / V double buffer also fills 141 KB of LDS).
constexpr int FWD_NB = 1;

hipError_t launch_fwd(AttnParams P, int D, int n_items, hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  P.n_items = n_items;
  if (P.queue) hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, stream, P.queue);
  const dim3 grid(P.queue ? claim_grid(n_items) : n_items);
  auto run = [&](auto k, int nb) { hipLaunchKernelGGL(k, grid, dim3(256 / nb), 0, stream, P); };
  if (P.R == 1 && (P.m.mode == MODE_BLOCKS || P.t.uniform)) {
    if (D == 128) run(fwd_kernel<128, FWD_NB, true>, FWD_NB);
    else if (D == 256) run(fwd_kernel<256, 1, true>, 1);
    else run(fwd_kernel<64, FWD_NB, true>, FWD_NB);
  } else {
    if (D == 128) run(fwd_kernel<128, FWD_NB, false>, FWD_NB);
    else if (D == 256) run(fwd_kernel<256, 1, false>, 1);
    else run(fwd_kernel<64, FWD_NB, false>, FWD_NB);
  }
  return hipGetLastError();
}

}  // namespace mad
