// attn_fwd.hip -- forward attention kernel for gfx950.
//
// Computes, per query head h and query row i with allowed key set A_i,
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j   and   LSE_i = ln sum_j exp(scale * q_i . k_j),
// the standard softmax attention whose quadratic cost the LongCA-bench pages
// start from (section 1), under a compiled mask.  A row with no allowed key
// gets O = 0, LSE = -inf.
//
// Work decomposition: one workgroup per (query head, 128-row query tile), two
// wave64s of 64 rows each.  The workgroup walks the query tile's list of
// non-EMPTY 64-key tiles.  K and V tiles reach LDS by direct global->LDS
// loads into a double buffer: the loads of tile t+1 are issued right after
// the barrier that opens tile t, so they overlap tile t's arithmetic and no
// registers are spent on staging.  Per key tile each wave
//   1. forms S^T = K Q^T (keys x queries) with bf16 MFMA; each lane then holds
//      one query row, so the row max and row sum stay in the lane (plus one
//      permlane32 swap with the other half-wave);
//   2. masks PARTIAL tiles (and the ragged last key tile) with -inf;
//   3. updates the online softmax in the exp2 domain against a lagging
//      reference max that moves (with a rescale of the accumulator) only when
//      a row's max grows by more than 2^8;
//   4. accumulates O^T += V^T P^T with P^T taken straight from registers as
//      the MFMA B operand and V^T read transposed from LDS.
#include "kernel_common.hpp"

namespace mad {

template <int D>
__global__ __launch_bounds__(128) void fwd_kernel(const AttnParams P) {
  constexpr int BM = BM0, BN = BN0, NKS = D / 16, NDB = D / 32;
  constexpr int KRS = tile_rs<D, TILE_ROWS>(), KT = tile_elems<D, TILE_ROWS>();
  constexpr int VRS = tile_rs<D, TILE_TR>(), VT = tile_elems<D, TILE_TR>();
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (KT + VT)];  // K0 V0 K1 V1

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int e = L % P.R, t_ = L / P.R;
  const int g = t_ % P.Hkv, rank = t_ / P.Hkv;
  const int h = g * P.R + e;
  const int qt = sld(P.t.order + rank);
  const int mg = h / P.grp_div;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform
  const int row_base = qt * BM + w * 64;

  const int32_t* ptr = P.t.ptr + (int64_t)mg * (P.t.nmajor + 1);
  const int beg = sld(ptr + qt), end = sld(ptr + qt + 1);
  const bf16* kg = P.k + (int64_t)g * P.k_head;
  const bf16* vg = P.v + (int64_t)g * P.v_head;
  const uint32_t smem_lds = lds_addr(smem);
  TileLoader<D, TILE_ROWS, 2, true> kload;
  TileLoader<D, TILE_TR, 2, false> vload;
  kload.init(P.k_tok, w, lane);
  vload.init(P.v_tok, w, lane);
  auto issue = [&](int kt, int buf) {
    const uint32_t kl = smem_lds + buf * (KT + VT) * 2;
    kload.issue(kl, kg, P.k_tok, kt * BN, P.Tk, w, lane);
    vload.issue(kl + KT * 2, vg, P.v_tok, kt * BN, P.Tk, w, lane);
  };
  if (beg < end) issue(sld(P.t.ent + beg) & 0x7fffffff, 0);

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16ks + 8hh .. +8].
  bf16x8 qf[2][NKS];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int row = row_base + b * 32 + li;
    const bf16* src = P.q + (int64_t)min(row, P.Tq - 1) * P.q_tok + (int64_t)h * P.q_head + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[b][ks] = ld16(src + 16 * ks);
  }

  f32x16 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[db][b] = f32x16{};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

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
    const bool masked = partial || (kt + 1) * BN > P.Tk;
    uint32_t mbits[2][2];
    if (masked) {
      const int aux = partial ? sld(P.t.ent_aux + it) : -1;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mbits[b][kb] = keymask32(P.m, aux, mg, partial, row_base + b * 32 + li, kt * BN + kb * 32, row_base,
                                   row_base + 63);
      wait_vmem();
    }
    if (it + 1 < end) issue(sld(P.t.ent + it + 1) & 0x7fffffff, buf ^ 1);
    const bf16* Ks = smem + buf * (KT + VT);
    const bf16* Vs = Ks + KT;
    __builtin_amdgcn_sched_barrier(0);

    // 1. S^T for 2 key blocks x 2 query blocks.
    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int b = 0; b < 2; ++b) s[kb][b] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = ld16(Ks + (kb * 32 + li) * KRS + (16 * ks + 8 * hh));
#pragma unroll
        for (int b = 0; b < 2; ++b) s[kb][b] = mfma32(a, qf[b][ks], s[kb][b]);
      }

    // 2. Mask (a real branch: FULL tiles must not pay for it).
    if (__builtin_expect(masked, 0)) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 16 * (r >> 3) + 8 * hh + (r & 7);
            if (!((mbits[b][kb] >> off) & 1u)) s[kb][b][r] = -INFINITY;
          }
    }

    // 3. Online softmax (exp2 domain) with a lagging reference max: each row
    // keeps a reference m_ref and forms p = exp2(s*c - m_ref).  m_ref moves up
    // (and the accumulator and sum are rescaled by exp2(m_old - m_new)) only
    // when the tile's max exceeds m_ref by more than RESCALE_SLACK, so p stays
    // below 2^RESCALE_SLACK and the rescale is rare.  The result is exact: O
    // and l share the same reference, and LSE = m_ref + log2(l).
    constexpr float RESCALE_SLACK = 8.f;
    float tmax[2];
    bool need = false;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][b][r]);
      tmax[b] = pair_max(mx) * P.scale_log2;
      need |= tmax[b] > mrow[b] + RESCALE_SLACK;
    }
    if (__ballot(need)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float mnew = fmaxf(mrow[b], tmax[b]);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrow[b] - mnew);
        mrow[b] = mnew;
        lrow[b] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][b][r] *= alpha;
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float muse = (mrow[b] == -INFINITY) ? 0.f : mrow[b];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][b][r], P.scale_log2, -muse));
          s[kb][b][r] = pv;
          ls += pv;
        }
      lrow[b] += ls;
    }

    __builtin_amdgcn_sched_barrier(0);
    // 4. O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        bf16x8 pb[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) pb[b] = to_bf16x8(s[kb][b], 8 * t2);
        const int vrow = kb * 32 + 16 * t2 + 8 * hh + tr_row(lane);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int vcol = db * 32 + tr_col(lane);
          const bf16x8 a = ld_tr8(Vs + vrow * VRS + vcol, Vs + (vrow + 4) * VRS + vcol);
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[db][b] = mfma32(a, pb[b], acc[db][b]);
        }
      }
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
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

hipError_t launch_fwd(const AttnParams& P, int D, int n_items, hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (D == 128) hipLaunchKernelGGL(fwd_kernel<128>, dim3(n_items), dim3(128), 0, stream, P);
  else hipLaunchKernelGGL(fwd_kernel<64>, dim3(n_items), dim3(128), 0, stream, P);
  return hipGetLastError();
}

}  // namespace mad
