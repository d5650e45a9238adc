// attn_dkdv.hpp -- dK / dV kernel for gfx950, head dims 64 and 128 (device
// code, included by attn_dkdv.hip; attn_dkdv256.hip shares its item walk).
//
// For every key j of a KV head and every query head h of its GQA group
// (LongCA-bench section 3.2 names the backward pass as the bottleneck):
//   P_ij  = exp(scale q_i.k_j - LSE_i)          (0 where (i, j) is masked)
//   dS_ij = P_ij (dO_i.v_j - D_i)
//   dV_j  = sum_h sum_i P_ij dO_i,   dK_j = scale sum_h sum_i dS_ij q_i
//
// Work decomposition: one workgroup per (KV head, 128-key tile), four waves
// of 32 keys (per 64-key tile, two waves, for block-sparse plans of smaller
// key blocks).
// K and V of the wave's keys stay in registers as MFMA operands.
// The workgroup walks, for each query head of the group, the key tile's list
// of non-EMPTY 64-row query tiles; the Q / dO tiles and their -LSE/scale and
// -D rows come in by direct global->LDS loads into a double buffer.
//
// One item (64 query rows x the wave's 32 keys) runs in four stages, as two
// 32-row blocks b0 / b1, arranged so that the matrix cores always have work
// while the vector unit computes P and dS:
//   A  S0 = Q0 K^T, dP0 = dO0 V^T       (MFMA)
//   B  S1, dP1 (MFMA)        +  P0, dS0 (VALU)
//   C  dV += P0^T dO0, dK += dS0^T Q0 (MFMA)  +  P1, dS1 (VALU)
//   D  dV += P1^T dO1, dK += dS1^T Q1 (MFMA)
// The score and dP accumulators start from -LSE/scale and -D (read from LDS
// straight into the accumulator registers), so S holds q.k - LSE/scale and
// dP holds dO.v - D when the products finish.  LDS operands are read two
// MFMA steps ahead of their use through a three-slot register ring; every
// step ends in a scheduling fence so that the compiler keeps that distance.
#pragma once

#include <algorithm>

#include "kernel_common.hpp"

namespace mad {

// The items one dK/dV workgroup visits: (query head e of its KV group g,
// position `it` in that head's visit list for key tile kt), as two cursors --
// the item being computed and the next one, whose tiles are prefetched.  When
// every query head of the group uses the same mask group (hence the same
// list), the list is walked from its end with the heads innermost: all
// workgroups then start at the last query tile and move down through the same
// tiles at the same pace, so the workgroups running together read the same
// Q / dO tiles and share them in L2 (walking up from each key tile's first
// tile would spread them apart).  Otherwise each head's list is walked in
// turn.  With S = kv_splits > 1 the column's items are cut into S contiguous
// chunks, one per workgroup (a few very long columns -- key tiles every query
// sees, as under GLOBAL_SLIDING -- would otherwise set the kernel's length on
// their own); the chunks' partial dK / dV are summed in fp32.
struct KvCursor {
  int e, it, end;  // shared list: `it` runs down to `end` (the list start)
  int left;        // items of this workgroup's chunk still to visit
  bool ok;
};

struct KvWalk {
  const AttnParams& P;
  int kt, h0, S, seg;
  bool shared;
  int n0, n1;  // this workgroup's chunk of the column's items

  __device__ __forceinline__ KvWalk(const AttnParams& P_, int g, int kt_, int S_, int seg_)
      : P(P_), kt(kt_), h0(g * P_.R), S(S_), seg(seg_), n0(0), n1(0) {
    shared = (h0 / P.grp_div) == ((h0 + P.R - 1) / P.grp_div);
  }
  __device__ __forceinline__ void head_list(int e, KvCursor& cu) const {
    const int32_t* ptr = P.t.ptr + (int64_t)((h0 + e) / P.grp_div) * (P.t.nmajor + 1);
    cu.e = e;
    cu.it = sld(ptr + kt);
    cu.end = sld(ptr + kt + 1);
  }
  __device__ __forceinline__ void settle(KvCursor& cu) const {  // move past exhausted heads
    while (cu.it >= cu.end && cu.e + 1 < P.R) head_list(cu.e + 1, cu);
  }
  __device__ __forceinline__ KvCursor first() {
    KvCursor cu;
    head_list(0, cu);
    int ncol;
    if (shared) {
      ncol = P.R * (cu.end - cu.it);
    } else {
      ncol = 0;
      for (int e = 0; e < P.R; ++e) {
        KvCursor x;
        head_list(e, x);
        ncol += x.end - x.it;
      }
    }
    n0 = (int)((int64_t)seg * ncol / S);
    n1 = (int)((int64_t)(seg + 1) * ncol / S);
    cu.left = n1 - n0;
    if (shared) {
      const int list_begin = cu.it;
      cu.e = n0 % P.R;
      cu.it = cu.end - 1 - n0 / P.R;
      cu.end = list_begin;
    } else {
      int skip = n0;
      settle(cu);
      while (skip > 0) {
        const int len = cu.end - cu.it;
        if (len <= 0) break;  // lists exhausted (not reached: n0 < the column's item count)
        if (skip < len) {
          cu.it += skip;
          skip = 0;
        } else {
          skip -= len;
          cu.it = cu.end;
          settle(cu);
        }
      }
    }
    cu.ok = cu.left > 0 && (shared || cu.it < cu.end);
    return cu;
  }
  __device__ __forceinline__ KvCursor advance(KvCursor cu) const {
    if (--cu.left <= 0) {
      cu.ok = false;
      return cu;
    }
    if (shared) {
      if (cu.e + 1 < P.R) {
        ++cu.e;
      } else {
        cu.e = 0;
        --cu.it;
      }
      cu.ok = true;
    } else {
      ++cu.it;
      settle(cu);
      cu.ok = cu.it < cu.end;
    }
    return cu;
  }
};

// NW waves of 32 keys: a 128-key tile (NW = 4, one workgroup per CU) or,
// for block-sparse plans of smaller key blocks (64-token or variable), a
// 64-key tile (NW = 2, two workgroups per CU).
// HM: the head-major item order (MHA masks whose columns carry even work).
template <int D, int NW, bool HM>
__global__ __launch_bounds__(64 * NW) void dkdv_kernel(const AttnParams P) {
  static_assert(D == 64 || D == 128, "head dim 256 has a kernel of its own");
  constexpr int BM = BM1, BN = 32 * NW, NKS = D / 16, NDB = D / 32;
  // D = 128: unpadded swizzled Q / dO tiles; D = 64: padded rows.
  constexpr int KIND = D == 128 ? TILE_SWZ : TILE_MIXED;
  constexpr int TILE = tile_elems<D, KIND>(), RS = tile_rs<D, KIND>();
  constexpr int S1 = 2 * NKS;   // phase-1 steps (block, k-step)
  constexpr int S2 = 4 * NDB;   // phase-2 steps (block, t2, d-block)
  // LDS operands are read RA steps ahead through rings of RA + 1 slots.
  constexpr int RA = 2, NR = RA + 1;
  constexpr int EB = 16 / NKS >= 2 ? 16 / NKS : 2;  // P / dS elements per stage-B step (the first 16 / EB steps)
  constexpr int EC = 16 / (2 * NDB);  // P / dS elements per stage-C step
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];   // Q0 dO0 Q1 dO1
  __shared__ __attribute__((aligned(256))) float rowv[2][2 * BM];  // per buffer: -LSE/scale[64], -D[64]

  // Workgroup -> (KV head g, key tile kt of the longest-first order, chunk
  // seg of that column's items).  Consecutive workgroups share g's XCD.
  // Workgroups go to the XCDs in turn.  Consecutive workgroups take
  // consecutive KV heads (with 8 KV heads each XCD serves one head and its
  // group's Q / dO tiles).  Masks without a GQA group (MHA) whose columns
  // carry even work (block-sparse masks, or every column of one length) run
  // head by head instead (the HM variant), so that every
  // XCD works on the same head's Q / dO tiles at a time rather than on eight
  // heads'; masks with uneven columns keep the longest-first order across
  // heads, which balances the CUs.
  const int L = blockIdx.x, S = P.kv_splits;
  constexpr bool mha = HM;  // launched only for P.R == 1
  const int per_head = P.t.nmajor * S;  // workgroups per KV head
  const int g = mha ? L / per_head : L % P.Hkv, rest = mha ? L % per_head : L / P.Hkv;
  const int kt = sld(P.t.order + rest / S), seg = rest % S;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform
  const int key = kt * BN + w * 32 + li;
  const int kc = min(key, P.Tk - 1);
  const float c = P.scale_log2;

  // K, V of this lane's key as B operands: lane holds K[key][16ks + 8hh .. +8].
  bf16x8 kf[NKS], vf[NKS];
  {
    const bf16* ks_ = P.k + (int64_t)kc * P.k_tok + (int64_t)g * P.k_head + 8 * hh;
    const bf16* vs_ = P.v + (int64_t)kc * P.v_tok + (int64_t)g * P.v_head + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = ld16(ks_ + 16 * ks);
      vf[ks] = ld16(vs_ + 16 * ks);
    }
  }
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  KvWalk walk(P, g, kt, S, seg);
  const uint32_t smem_lds = lds_addr(smem), rowv_lds = lds_addr(&rowv[0][0]);
  TileLoader<D, KIND, NW, false> qload, dload;
  SwzRows srow;
  SwzTr str;
  if constexpr (KIND == TILE_SWZ) {
    srow.init(li, hh);
    str.init(lane);
  }
  qload.init(P.q_tok, w, lane);
  dload.init((int64_t)P.Hq * D, w, lane);
  auto issue = [&](const KvCursor& cu, int buf) {
    const int hx = g * P.R + cu.e;
    const int q0 = (sld(P.t.ent + cu.it) & 0x7fffffff) * BM;
    qload.issue(smem_lds + (2 * buf) * TILE * 2, P.q + (int64_t)hx * P.q_head, P.q_tok, q0, P.Tq, w, lane);
    dload.issue(smem_lds + (2 * buf + 1) * TILE * 2, P.d_o + (int64_t)hx * D, (int64_t)P.Hq * D, q0, P.Tq, w,
                lane);
    if (w == 0 && lane < 32) {
      const float* src = (lane < 16 ? P.nlse : P.ndelta) + (int64_t)hx * P.Tq_pad + q0 + 4 * (lane & 15);
      g2lds16(src, rowv_lds + buf * 2 * BM * 4);
    }
  };
  // The K / V register loads complete before the first tiles are requested:
  // the loop's waits count the direct loads, which the compiler does not track.
  wait_vmem();
  KvCursor cur = walk.first();
  if (cur.ok) issue(cur, 0);

  for (int n = 0; cur.ok; ++n) {
    const int buf = n & 1;
    const int h = g * P.R + cur.e;
    const int mg = h / P.grp_div;
    const uint32_t ent = (uint32_t)sld(P.t.ent + cur.it);
    const bool partial = (ent & ENT_PARTIAL) != 0;
    const int q0 = (int)(ent & 0x7fffffffu) * BM;
    const KvCursor nxt = walk.advance(cur);
    wait_vmem();
    __syncthreads();
    // Rows of the tile this lane's key may see (PARTIAL tiles), evaluated
    // before the next tiles' loads are issued so that the mask table reads
    // never wait behind them.
    // Block-sparse PARTIAL tiles whose four key strips are each FULL or EMPTY
    // carry the FULL strips as bits in aux: those waves run the item as a
    // FULL one, the others skip it.
    const int aux = partial ? sld(P.t.ent_aux + cur.it) : -1;
    const bool parts = partial && P.m.mode == MODE_BLOCKS && aux >= 0;
    const bool masked = partial && !parts;
    uint32_t mw[2] = {0u, 0u};
    if (masked) {
      const int k_lo = kt * BN + w * 32;  // the wave's keys, wave-uniform
      const uint64_t rows = rowmask64(P.m, aux, mg, key, q0, k_lo, k_lo + 31);
      mw[0] = (uint32_t)(rows >> (4 * hh));
      mw[1] = (uint32_t)(rows >> (32 + 4 * hh));
      wait_vmem();
    }
    if (nxt.ok) issue(nxt, buf ^ 1);
    const bf16* Qs = smem + (2 * buf) * TILE;
    const bf16* Ds = smem + (2 * buf + 1) * TILE;
    const float* nl_s = &rowv[buf][0];
    const float* nd_s = &rowv[buf][BM];

    // A wave none of whose keys is seen by a row of this tile skips it; it
    // only takes part in the loads and barriers.
    if (parts ? ((aux >> w) & 1) != 0 : (!masked || __ballot((mw[0] | mw[1]) != 0u) != 0ull)) {
      // Register r of block b holds query row b*32 + 8(r/4) + 4hh + r%4.  A
      // masked row starts its score at -inf, so its P (and dS) is exactly 0
      // after the products: the mask costs nothing past the initialisation.
      f32x16 sc[2], dp[2];
      auto init = [&](int b) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int rr = b * 32 + 8 * rg + 4 * hh;
          const float4 l4 = *reinterpret_cast<const float4*>(nl_s + rr);
          const float4 d4 = *reinterpret_cast<const float4*>(nd_s + rr);
          sc[b][4 * rg + 0] = l4.x; sc[b][4 * rg + 1] = l4.y; sc[b][4 * rg + 2] = l4.z; sc[b][4 * rg + 3] = l4.w;
          dp[b][4 * rg + 0] = d4.x; dp[b][4 * rg + 1] = d4.y; dp[b][4 * rg + 2] = d4.z; dp[b][4 * rg + 3] = d4.w;
        }
        if (masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((mw[b] >> (8 * (r >> 2) + (r & 3))) & 1u)) sc[b][r] = -INFINITY;
        }
      };
      // Phase-1 operands of step st: Q and dO rows b*32 + li, columns 16ks + 8hh.
      bf16x8 opq[NR], opd[NR];
      auto ld1 = [&](int st) {
        const int b = st / NKS, ks = st % NKS;
        if constexpr (KIND == TILE_SWZ) {
          const uint32_t off = srow.o[ks] + b * 32 * 256;
          opq[st % NR] = ld16((const bf16*)((const char*)Qs + off));
          opd[st % NR] = ld16((const bf16*)((const char*)Ds + off));
        } else {
          const int off = (b * 32 + li) * RS + 16 * ks + 8 * hh;
          opq[st % NR] = ld16(Qs + off);
          opd[st % NR] = ld16(Ds + off);
        }
      };
      // Phase-2 operands of step st: dO and Q read transposed; contraction
      // element e of half-wave hh is query row b*32 + 16 t2 + 8(e/4) + 4hh + e%4.
      bf16x8 trd[NR], trq[NR];
      auto ld2 = [&](int st) {
        const int b = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
        if constexpr (KIND == TILE_SWZ) {
          const uint32_t rb = (b * 32 + 16 * t2) * 256;
          const char *dc = (const char*)Ds, *qc = (const char*)Qs;
          trd[st % NR] = ld_tr8((const bf16*)(dc + rb + str.o0[db]), (const bf16*)(dc + rb + str.o1[db]));
          trq[st % NR] = ld_tr8((const bf16*)(qc + rb + str.o0[db]), (const bf16*)(qc + rb + str.o1[db]));
        } else {
          const int qrow = b * 32 + 16 * t2 + 4 * hh + tr_row(lane), col = db * 32 + tr_col(lane);
          trd[st % NR] = ld_tr8(Ds + qrow * RS + col, Ds + (qrow + 8) * RS + col);
          trq[st % NR] = ld_tr8(Qs + qrow * RS + col, Qs + (qrow + 8) * RS + col);
        }
      };
      // P = exp2(c S) and dS = P dP for registers r, r + 1 of block b,
      // written as bf16 straight into the phase-2 A operands: register r
      // feeds element r % 8 of k-step t2 = r / 8.
      bf16x8 pa[2][2], sa[2][2];  // [block][t2]
      auto pds = [&](int b, int r) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const float pv = __builtin_amdgcn_exp2f(sc[b][r + x] * c);
          pa[b][(r + x) >> 3][(r + x) & 7] = (bf16)pv;
          sa[b][(r + x) >> 3][(r + x) & 7] = (bf16)(pv * dp[b][r + x]);
        }
      };

      init(0);
#pragma unroll
      for (int st = 0; st < RA; ++st) ld1(st);
      init(1);
      __builtin_amdgcn_sched_barrier(0);
      // Stage A.
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        ld1(st + RA);
        sc[0] = mfma32(opq[st % NR], kf[st], sc[0]);
        dp[0] = mfma32(opd[st % NR], vf[st], dp[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Stage B.
#pragma unroll
      for (int st = NKS; st < S1; ++st) {
        if (st + RA < S1) ld1(st + RA);
        else ld2(st + RA - S1);
        sc[1] = mfma32(opq[st % NR], kf[st - NKS], sc[1]);
        dp[1] = mfma32(opd[st % NR], vf[st - NKS], dp[1]);
#pragma unroll
        for (int x = 0; x < EB; x += 2)
          if ((st - NKS) * EB + x < 16) pds(0, (st - NKS) * EB + x);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Stages C and D.
#pragma unroll
      for (int st = 0; st < S2; ++st) {
        if (st + RA < S2) ld2(st + RA);
        const int b = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
        dva[db] = mfma32(pa[b][t2], trd[st % NR], dva[db]);
        dka[db] = mfma32(sa[b][t2], trq[st % NR], dka[db]);
        if (st < 2 * NDB) {
#pragma unroll
          for (int x = 0; x < EC; x += 2) pds(1, st * EC + x);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
  }

  // dK, dV: lane holds column d = db*32 + li of key rows 8(r/4) + 4hh + r%4 of the wave's 32 keys.
  if (S > 1) {
    if (walk.n1 > walk.n0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kt * BN + w * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (kk < P.Tk) {
            const int64_t off = ((int64_t)kk * P.Hkv + g) * D + db * 32 + li;
            unsafeAtomicAdd(P.dk_acc + off, dka[db][r] * P.scale);
            unsafeAtomicAdd(P.dv_acc + off, dva[db][r]);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kt * BN + w * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kk < P.Tk) {
        const int64_t off = ((int64_t)kk * P.Hkv + g) * D + db * 32 + li;
        P.dk[off] = (bf16)(dka[db][r] * P.scale);
        P.dv[off] = (bf16)dva[db][r];
      }
    }
}

}  // namespace mad
