// attn_bwd.hip -- backward attention kernels for gfx950.
//
// Gradients of the forward in attn_fwd.hip for upstream gradient dO, given
// the forward's O and LSE (or merged ones for a ring step):
//   P_ij  = exp(scale * q_i.k_j - LSE_i) on allowed (i, j), else 0
//   D_i   = dO_i . O_i                              (delta pre-pass)
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale * sum_j dS_ij k_j                 (dQ kernel)
//   dK_j  = scale * sum_{h in group} sum_i dS_ij q_i,  dV_j = sum_{h in group} sum_i P_ij dO_i   (dK/dV kernel)
// The pages single out the backward pass as the common bottleneck (section
// 3.2, the notes' key findings).  Here it is split into three launches with
// no atomic adds into the gradients (but for dK/dV columns cut between
// workgroups, below): a streaming delta pre-pass, a dK/dV kernel that owns a
// key tile and walks the query tiles of its per-key-tile list for every query
// head of its GQA group, and a dQ kernel that owns a query tile and walks its
// key-tile list (the forward's tiling).  Both recompute P from LSE.
//
// Workspace (fp32, rows padded to a multiple of 128 per head):
//   ndelta[h][i] = -D_i and nlse[h][i] = -LSE_i / scale, with nlse = -inf for
//   rows that have no allowed key or lie past Tq -- so their P is exactly 0.
// Both are stored negated so that the dK/dV kernel can start its score and
// dP accumulators from them: P = exp2(scale log2e (q.k + nlse)) and
// dS = P (dP + ndelta).  The last 256 bytes of the required workspace size
// hold the dQ launch's per-XCD work-claim counters (cleared by a kernel
// before it).
#include "kernel_common.hpp"

namespace mad {

// ---------------------------------------------------------------------------
// Delta pre-pass.  One group of D/8 lanes per (row, head); O and dO packed
// [Tq, Hq, D].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const AttnParams P) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t nrows = (int64_t)P.Tq_pad * P.Hq;
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  const int64_t i = r / P.Hq, h = r % P.Hq;
  const bool in = r < nrows && i < P.Tq;
  float acc = 0.f;
  if (in) {
    const bf16x8 a = ld16(P.o_in + r * D + 8 * sub);
    const bf16x8 b = ld16(P.d_o + r * D + 8 * sub);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (r < nrows && sub == 0) {
    float nl = -INFINITY;
    if (in) {
      const float l = P.lse_in[h * P.Tq + i];
      if (l != -INFINITY) nl = -l / P.scale;
    }
    P.ndelta[h * P.Tq_pad + i] = -acc;
    P.nlse[h * P.Tq_pad + i] = nl;
  }
}

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup per (query head, 128-row query tile), four waves
// of 32 rows, walking the forward tiling's key-tile list.  K and V tiles come
// in by direct loads into a double buffer (both stored with the swap23 row
// order).  Per key block kb of 32 keys:
//   S^T = K Q^T, dP^T = V dO^T       (keys x queries; lane = query row)
//   P^T = exp2((S^T scale - LSE) log2e), dS^T = P^T (dP^T - D)
//   dQ^T += K^T dS^T                 (K^T read transposed from LDS)
// The two key blocks of a 64-key tile run one after the other (S^T / dP^T,
// P / dS, dQ^T), which keeps one block's scores live at a time: the kernel
// fits 256 registers and runs two waves per SIMD, so one wave's vector work
// overlaps the other wave's matrix products.  (Staging block 1's products
// under block 0's vector work inside one wave needs both blocks live and
// one wave per SIMD; measured 25.7 ms against 21.7 ms for this form at
// CAUSAL 32K GQA 64:8.)  LDS operands are read two MFMA steps ahead through
// three-slot register rings, each step closed by a scheduling fence.  Masked
// scores start at -inf, so their P is exactly 0 with no per-element test.
// ---------------------------------------------------------------------------
// Two workgroups per CU at D = 64 / 128; one at D = 256, where the Q / dO
// operands and the dQ accumulator take 256 registers per lane (421 in all).
// HM: the head-major item order (MHA masks whose tiles carry even work).
template <int D, bool HM>
__global__ __launch_bounds__(256, D == 256 ? 1 : D == 64 ? 3 : 2) void dq_kernel(const AttnParams P) {
  constexpr int BM = BM0, BN = BN0, NKS = D / 16, NDB = D / 32;
  constexpr int KRS = tile_rs<D, TILE_MIXED>(), KT = tile_elems<D, TILE_MIXED>();
  constexpr int VRS = tile_rs<D, TILE_ROWS>(), VT = tile_elems<D, TILE_ROWS>();
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
  // The item is claimed from the per-XCD queues (claim_item); the grid holds
  // more workgroups than items, and those that find every queue empty exit.
  __shared__ int claimed;
  if (threadIdx.x == 0) claimed = claim_item(P.queue, P.n_items);
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
  const int row = qt * BM + w * 32 + li;  // this lane's query row
  const float c = P.scale_log2;

  const int32_t* ptr = P.t.ptr + (int64_t)mg * (P.t.nmajor + 1);
  const int beg = sld(ptr + qt), end = sld(ptr + qt + 1);
  const bf16* kg = P.k + (int64_t)g * P.k_head;
  const bf16* vg = P.v + (int64_t)g * P.v_head;
  const uint32_t smem_lds = lds_addr(smem);
  TileLoader<D, TILE_MIXED, 4, true> kload;
  TileLoader<D, TILE_ROWS, 4, true> vload;
  kload.init(P.k_tok, w, lane);
  vload.init(P.v_tok, w, lane);
  auto issue = [&](int kt, int buf) {
    const uint32_t kl = smem_lds + buf * (KT + VT) * 2;
    kload.issue(kl, kg, P.k_tok, kt * BN, P.Tk, w, lane);
    vload.issue(kl + KT * 2, vg, P.v_tok, kt * BN, P.Tk, w, lane);
  };

  // Q and dO of this lane's row as B operands: lane holds Q[row][16ks + 8hh .. +8].
  bf16x8 qf[NKS], df[NKS];
  float ml2, ndl;
  {
    const int rc = min(row, P.Tq - 1);
    const bf16* qs = P.q + (int64_t)rc * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
    const bf16* ds = P.d_o + ((int64_t)rc * P.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = ld16(qs + 16 * ks);
      df[ks] = ld16(ds + 16 * ks);
    }
    ml2 = P.nlse[(int64_t)h * P.Tq_pad + row] * c;  // -LSE log2(e); -inf past Tq
    ndl = P.ndelta[(int64_t)h * P.Tq_pad + row];
  }
  // The register loads complete before the first tiles are requested: the
  // loop's waits count the direct loads, which the compiler does not track.
  wait_vmem();
  if (beg < end) issue(sld(P.t.ent + beg) & 0x7fffffff, 0);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  for (int it = beg; it < end; ++it) {
    const int buf = (it - beg) & 1;
    const uint32_t ent = (uint32_t)sld(P.t.ent + it);
    const int kt = (int)(ent & 0x7fffffffu);
    const bool partial = (ent & ENT_PARTIAL) != 0;
    // Block-sparse PARTIAL tiles whose wave strips are each FULL or EMPTY
    // (FULL strips as bits in aux) run as FULL tiles on the FULL strips.
    const bool ragged = (kt + 1) * BN > P.Tk;
    const int aux = partial ? sld(P.t.ent_aux + it) : -1;
    const bool parts = partial && !ragged && P.m.mode == MODE_BLOCKS && aux >= 0;
    const bool masked = (partial && !parts) || ragged;
    wait_vmem();
    __syncthreads();
    // Allowed-key masks (PARTIAL and ragged tiles), evaluated before the next
    // tile's loads are issued so that the mask table reads never wait behind them.
    uint32_t mbits[2] = {0xffffffffu, 0xffffffffu};
    if (masked) {
      const int r_lo = qt * BM + w * 32;  // the wave's rows, wave-uniform
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mbits[kb] = keymask32(P.m, aux, mg, partial, row, kt * BN + kb * 32, r_lo, r_lo + 31);
      wait_vmem();
    }
    if (it + 1 < end) issue(sld(P.t.ent + it + 1) & 0x7fffffff, buf ^ 1);
    // A wave none of whose rows sees a key of this tile skips it; it only
    // takes part in the loads and barriers.
    if (parts && !((aux >> w) & 1)) continue;
    if (masked && __ballot((mbits[0] | mbits[1]) != 0u) == 0ull) continue;
    const bf16* Ks = smem + buf * (KT + VT);
    const bf16* Vs = Ks + KT;

    // Register r of key block kb holds key kb*32 + 16(r/8) + 8hh + r%8.  A
    // block's first products start from an inline zero; masked (row, key)
    // pairs get -inf once its scores are in, before P and dS are formed.
    f32x16 sc[2], dp[2];
    auto apply_mask = [&](int kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!((mbits[kb] >> (16 * (r >> 3) + 8 * hh + (r & 7))) & 1u)) sc[kb][r] = -INFINITY;
    };
    bf16x8 opk[3], opv[3];
    auto ld1 = [&](int st) {
      const int kb = st / NKS, ks = st % NKS;
      opk[st % 3] = ld16(Ks + (kb * 32 + li) * KRS + 16 * ks + 8 * hh);
      opv[st % 3] = ld16(Vs + (kb * 32 + li) * VRS + 16 * ks + 8 * hh);
    };
    // dQ^T step (kb, t2, db): keys 16 t2 + 8 hh + 0..3 of block kb live in LDS
    // rows 16 t2 + 4 hh + 0..3, keys +4..7 in rows +8.
    bf16x8 trk[3];
    auto ld2 = [&](int st) {
      const int kb = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
      const int krow = kb * 32 + 16 * t2 + 4 * hh + tr_row(lane), kcol = db * 32 + tr_col(lane);
      trk[st % 3] = ld_tr8(Ks + krow * KRS + kcol, Ks + (krow + 8) * KRS + kcol);
    };
    bf16x8 sb[2][2];  // dS^T as B operands, [kb][t2]
    auto pds = [&](int kb, int r) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r + x], c, ml2));
        sb[kb][(r + x) >> 3][(r + x) & 7] = (bf16)(pv * (dp[kb][r + x] + ndl));
      }
    };

    // Key blocks one after the other: S^T / dP^T, then P / dS, then dQ^T.
    // LDS operands are read two steps ahead across the whole sequence.
    constexpr int SPB = NKS + 2 * NDB;  // steps per key block
    auto load = [&](int u) {
      const int kb = u / SPB, v = u % SPB;
      if (v < NKS) ld1(kb * NKS + v);
      else ld2(kb * 2 * NDB + (v - NKS));
    };
    load(0);
    load(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2 * SPB; ++u) {
      if (u + 2 < 2 * SPB) load(u + 2);
      const int kb = u / SPB, v = u % SPB;
      if (v < NKS) {
        const int p1 = kb * NKS + v;
        sc[kb] = mfma32(opk[p1 % 3], qf[v], v == 0 ? f32x16{} : sc[kb]);
        dp[kb] = mfma32(opv[p1 % 3], df[v], v == 0 ? f32x16{} : dp[kb]);
      } else {
        const int j = v - NKS, p2 = kb * 2 * NDB + j;
        acc[j % NDB] = mfma32(trk[p2 % 3], sb[kb][j / NDB], acc[j % NDB]);
      }
      if (v == NKS - 1) {
        __builtin_amdgcn_sched_barrier(0);
        if (__builtin_expect(masked, 0)) apply_mask(kb);
#pragma unroll
        for (int r = 0; r < 16; r += 2) pds(kb, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // dQ^T: lane holds query row `row`, column d = db*32 + 8(r/4) + 4hh + r%4.
  if (row < P.Tq && P.dq_acc) {
    // Accumulating form (one call per key chunk): each element has one owner lane.
    float* dst = P.dq_acc + ((int64_t)row * P.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float4* p4 = reinterpret_cast<float4*>(dst + db * 32 + 8 * rg + 4 * hh);
        float4 v4 = *p4;
        v4.x += acc[db][4 * rg + 0] * P.scale;
        v4.y += acc[db][4 * rg + 1] * P.scale;
        v4.z += acc[db][4 * rg + 2] * P.scale;
        v4.w += acc[db][4 * rg + 3] * P.scale;
        *p4 = v4;
      }
  } else if (row < P.Tq) {
    bf16* dst = P.dq + ((int64_t)row * P.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v4;
#pragma unroll
        for (int x = 0; x < 4; ++x) v4[x] = (bf16)(acc[db][4 * rg + x] * P.scale);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * rg + 4 * hh) = v4;
      }
  }
}

hipError_t launch_dkdv(const AttnParams& P, int D, int n_items, hipStream_t stream);

hipError_t launch_bwd(AttnParams Pq, const AttnParams& Pkv, int D, int nq_items, int nkv_items,
                      uint32_t phases, hipStream_t stream) {
  const int64_t nrows = (int64_t)Pq.Tq_pad * Pq.Hq;
  if ((phases & MAD_BWD_DELTA) && nrows > 0) {
    const int64_t threads = nrows * (D / 8);
    const int nb = (int)((threads + 255) / 256);
    if (D == 128) hipLaunchKernelGGL(delta_kernel<128>, dim3(nb), dim3(256), 0, stream, Pq);
    else if (D == 256) hipLaunchKernelGGL(delta_kernel<256>, dim3(nb), dim3(256), 0, stream, Pq);
    else hipLaunchKernelGGL(delta_kernel<64>, dim3(nb), dim3(256), 0, stream, Pq);
  }
  const bool kv = (phases & MAD_BWD_DKDV) && nkv_items > 0, dq = (phases & MAD_BWD_DQ) && nq_items > 0;
  if (dq) hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, stream, Pq.queue);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (kv) {
    err = launch_dkdv(Pkv, D, nkv_items, stream);
    if (err != hipSuccess) return err;
  }
  if (dq) {
    Pq.n_items = nq_items;
    auto run = [&](auto k) { hipLaunchKernelGGL(k, dim3(claim_grid(nq_items)), dim3(256), 0, stream, Pq); };
    if (Pq.R == 1 && (Pq.m.mode == MODE_BLOCKS || Pq.t.uniform)) {
      if (D == 128) run(dq_kernel<128, true>);
      else if (D == 256) run(dq_kernel<256, true>);
      else run(dq_kernel<64, true>);
    } else {
      if (D == 128) run(dq_kernel<128, false>);
      else if (D == 256) run(dq_kernel<256, false>);
      else run(dq_kernel<64, false>);
    }
  }
  return hipGetLastError();
}

}  // namespace mad
