// attn_dkdv256.hip -- dK / dV kernel for head dim 256 (gfx950).
//
// The quantities are those of attn_dkdv.hpp (LongCA-bench section 3.2): for
// key j of a KV head and every query row i of its GQA group's heads,
//   P_ij = exp(scale q_i.k_j - LSE_i),  dS_ij = P_ij (dO_i.v_j - D_i),
//   dV_j = sum P_ij dO_i,  dK_j = scale sum dS_ij q_i.
//
// At D = 256 one wave cannot hold a 32-key strip's K, V and both full 32 x 256
// accumulators (384 of a lane's 512 registers before any operand).  Here a
// strip belongs to a pair of waves, and each wave accumulates one 128-column
// half of dK and dV.  The scores and dP are not recomputed per half: of an
// item's two 32-row query blocks, wave 0 of the pair takes S of block 0 and
// dP of block 1, wave 1 takes S of block 1 and dP of block 0.  Each wave
// exponentiates its own S while the matrix cores run its dP products, the
// pair swaps P through LDS, each wave forms dS of its dP block and the pair
// swaps dS.  Every pair of (query row, key) then costs 8d MFMA FLOPs, as at
// the other head dims.
//
// Workgroup: four waves = two 32-key strips x two waves, covering 64 keys of
// a key tile (blockIdx.y selects the half of a 128-key tile; a 64-key tile
// has one).  The walk over the tile's query tiles, the double-buffered Q / dO
// tiles and their -LSE/scale and -D rows are those of the other head dims.
// One item (64 query rows) runs in three parts separated by workgroup
// barriers (every wave passes all of them, whether or not its strip has work
// in the item):
//   1  S_own = Q_own K^T, dP_oth = dO_oth V^T (MFMA)  +  P_own (VALU); P_own to LDS
//   2  dV_half += P^T dO (MFMA, own block, then the other block's P read
//      from LDS)  +  dS_oth = P_oth dP_oth (VALU); dS_oth to LDS
//   3  dK_half += dS^T Q (MFMA, dS_oth, then dS_own read from LDS)
// P and dS cross between the waves as bf16, the precision both products take
// them in; dS is formed from the bf16 P.
#include "attn_dkdv.hpp"

namespace mad {

// LDS wait and workgroup barrier that leave the direct tile loads in flight
// (a barrier with a memory fence would wait for them): the P / dS exchange
// only needs this wave's LDS writes done before the others pass.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool HM>
__global__ __launch_bounds__(256) void dkdv256_kernel(const AttnParams P) {
  constexpr int D = 256, BM = BM1, NKS = D / 16, NDB = 4;  // NDB: 32-column blocks per wave (128 columns)
  constexpr int KIND = TILE_MIXED;
  constexpr int TILE = tile_elems<D, KIND>(), RS = tile_rs<D, KIND>();
  constexpr int S1 = 2 * NKS;  // part-1 steps: NKS for S_own, NKS for dP_oth
  constexpr int S2 = 4 * NDB;  // part-2 / part-3 steps: (block, k-step t2, column block)
  constexpr int RA = 3, NR = RA + 1;  // LDS operands read RA steps ahead through an NR-slot ring
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];   // Q0 dO0 Q1 dO1
  __shared__ __attribute__((aligned(256))) float rowv[2][2 * BM];  // per buffer: -LSE/scale[64], -D[64]
  // P / dS exchange, per strip: four 1 KB chunks (block b, k-step t2) of 64
  // lanes x 8 bf16, lane-contiguous so that each access is conflict-free.
  __shared__ __attribute__((aligned(16))) bf16 xch[2][4 * 64 * 8];

  // Workgroup -> (KV head g, key tile kt, chunk seg of its items): the order
  // of the other head dims (heads across XCDs, or head-major for HM).
  const int L = blockIdx.x, S = P.kv_splits;
  const int per_head = P.t.nmajor * S;
  const int g = HM ? L / per_head : L % P.Hkv, rest = HM ? L % per_head : L / P.Hkv;
  const int kt = sld(P.t.order + rest / S), seg = rest % S;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, li = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sp = w >> 1;                        // strip of this workgroup
  const int own = w & 1, oth = own ^ 1;         // own: this wave's S block; oth: its dP block
  const int strip = (int)blockIdx.y * 2 + sp;   // 32-key strip within the key tile
  const int kbase = kt * P.t.BN + strip * 32;
  const int key = kbase + li;
  const int kc = min(key, P.Tk - 1);
  const int c0 = own * 128;                     // first dK / dV column of this wave
  const float c = P.scale_log2;

  // K and V of the lane's key as B operands: lane holds row key, elements 16ks + 8hh .. +8.
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
  TileLoader<D, KIND, 4, false> qload, dload;
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
  bf16* xs = &xch[sp][0];
  bf16* const x_own = xs + own * 2 * 512 + lane * 8;  // chunks of block `own` (t2 = 0 at +0, 1 at +512)
  bf16* const x_oth = xs + oth * 2 * 512 + lane * 8;
  // Per-lane operand offsets (elements) inside a tile: row reads for part 1,
  // transposed reads for parts 2 and 3 (rows 4hh + tr_row and + 8 of a
  // 16-row k-step, columns c0 + 32 db + tr_col).
  const int r1_own = (own * 32 + li) * RS + 8 * hh, r1_oth = (oth * 32 + li) * RS + 8 * hh;
  const int t_row = 4 * hh + tr_row(lane);
  const int r2_own = (own * 32 + t_row) * RS + c0 + tr_col(lane);
  const int r2_oth = (oth * 32 + t_row) * RS + c0 + tr_col(lane);

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
    // before the next tiles' loads are issued; block-sparse PARTIAL tiles
    // whose strips are each FULL or EMPTY carry the FULL strips as bits in
    // aux.  Both waves of a strip take the same decision.
    const int aux = partial ? sld(P.t.ent_aux + cur.it) : -1;
    const bool parts = partial && P.m.mode == MODE_BLOCKS && aux >= 0;
    const bool masked = partial && !parts;
    uint32_t mw[2] = {0u, 0u};
    if (masked) {
      const uint64_t rows = rowmask64(P.m, aux, mg, key, q0, kbase, kbase + 31);
      mw[0] = (uint32_t)(rows >> (4 * hh));
      mw[1] = (uint32_t)(rows >> (32 + 4 * hh));
      wait_vmem();
    }
    if (nxt.ok) issue(nxt, buf ^ 1);
    const bf16* Qs = smem + (2 * buf) * TILE;
    const bf16* Ds = smem + (2 * buf + 1) * TILE;
    const bool act = parts ? ((aux >> strip) & 1) != 0 : (!masked || __ballot((mw[0] | mw[1]) != 0u) != 0ull);

    // Register r of a 32-row block holds query row 8(r/4) + 4hh + r%4 of it;
    // bf16 operand [t2][e] of a block holds its register 8 t2 + e.
    f32x16 s_acc, p_acc;              // S of block own, dP of block oth
    bf16x8 pa_own[2], pa_oth[2];      // P
    bf16x8 sa_own[2], sa_oth[2];      // dS
    // Operand ring, indexed by the item's step count over all three parts
    // (part 1: 0 .. S1-1, part 2: S1 .. S1+S2-1, part 3 after).
    bf16x8 op[NR];
    // Part-1 operand of step st: Q row (own block) for st < NKS, dO row (oth block) after.
    auto ld1 = [&](int st) {
      op[st % NR] = st < NKS ? ld16(Qs + r1_own + 16 * st) : ld16(Ds + r1_oth + 16 * (st - NKS));
    };
    // Operand of step st of part 2 or 3 (ring slot gs): X transposed over
    // (block first / second, k-step t2, column block db), rows 16 t2 + ... of
    // the block, columns c0 + 32 db + ...
    auto ld_t = [&](const bf16* X, int first_off, int second_off, int st, int gs) {
      const int b2 = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
      const int off = (b2 == 0 ? first_off : second_off) + 16 * t2 * RS + 32 * db;
      op[gs % NR] = ld_tr8(X + off, X + off + 8 * RS);
    };

    if (act) {
      const float* nl_s = &rowv[buf][own * 32];
      const float* nd_s = &rowv[buf][BM + oth * 32];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 l4 = *reinterpret_cast<const float4*>(nl_s + 8 * rg + 4 * hh);
        const float4 d4 = *reinterpret_cast<const float4*>(nd_s + 8 * rg + 4 * hh);
        s_acc[4 * rg + 0] = l4.x; s_acc[4 * rg + 1] = l4.y; s_acc[4 * rg + 2] = l4.z; s_acc[4 * rg + 3] = l4.w;
        p_acc[4 * rg + 0] = d4.x; p_acc[4 * rg + 1] = d4.y; p_acc[4 * rg + 2] = d4.z; p_acc[4 * rg + 3] = d4.w;
      }
      if (masked) {
        // A masked pair starts its score at -inf, so its P and dS are exactly 0.
        const uint32_t m = own ? mw[1] : mw[0];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((m >> (8 * (r >> 2) + (r & 3))) & 1u)) s_acc[r] = -INFINITY;
      }
#pragma unroll
      for (int st = 0; st < RA; ++st) ld1(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        ld1(st + RA);
        s_acc = mfma32(op[st % NR], kf[st], s_acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // dP products, with P_own = exp2(c S) one register per step.
#pragma unroll
      for (int st = NKS; st < S1; ++st) {
        if (st + RA < S1) ld1(st + RA);
        else ld_t(Ds, r2_own, r2_oth, st + RA - S1, st + RA);
        p_acc = mfma32(op[st % NR], vf[st - NKS], p_acc);
        const int r = st - NKS;
        pa_own[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(s_acc[r] * c);
        __builtin_amdgcn_sched_barrier(0);
      }
      *reinterpret_cast<bf16x8*>(x_own) = pa_own[0];
      *reinterpret_cast<bf16x8*>(x_own + 512) = pa_own[1];
    }
    lds_barrier();  // P_own of both waves in LDS
    if (act) {
      pa_oth[0] = *reinterpret_cast<const bf16x8*>(x_oth);
      pa_oth[1] = *reinterpret_cast<const bf16x8*>(x_oth + 512);
      // dV: own block first (P in registers), then the other block's P.
#pragma unroll
      for (int st = 0; st < S2; ++st) {
        if (st + RA < S2) ld_t(Ds, r2_own, r2_oth, st + RA, S1 + st + RA);
        else ld_t(Qs, r2_oth, r2_own, st + RA - S2, S1 + st + RA);
        const int b2 = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
        dva[db] = mfma32(b2 == 0 ? pa_own[t2] : pa_oth[t2], op[(S1 + st) % NR], dva[db]);
        // dS_oth = P_oth dP_oth, two registers per step over the first half.
        if (st >= 2 && st < 2 + 8) {
          const int r = 2 * (st - 2);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float pv = (float)pa_oth[(r + x) >> 3][(r + x) & 7];
            sa_oth[(r + x) >> 3][(r + x) & 7] = (bf16)(pv * p_acc[r + x]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      *reinterpret_cast<bf16x8*>(x_oth) = sa_oth[0];
      *reinterpret_cast<bf16x8*>(x_oth + 512) = sa_oth[1];
    }
    lds_barrier();  // dS_oth of both waves in LDS
    if (act) {
      sa_own[0] = *reinterpret_cast<const bf16x8*>(x_own);
      sa_own[1] = *reinterpret_cast<const bf16x8*>(x_own + 512);
      // dK: the other block first (dS in registers), then the own block's dS.
#pragma unroll
      for (int st = 0; st < S2; ++st) {
        if (st + RA < S2) ld_t(Qs, r2_oth, r2_own, st + RA, S1 + S2 + st + RA);
        const int b2 = st / (2 * NDB), t2 = (st / NDB) % 2, db = st % NDB;
        dka[db] = mfma32(b2 == 0 ? sa_oth[t2] : sa_own[t2], op[(S1 + S2 + st) % NR], dka[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
  }

  // dK, dV: lane holds column c0 + 32 db + li of key rows 8(r/4) + 4hh + r%4 of the strip.
  if (S > 1) {
    if (walk.n1 > walk.n0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kbase + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (kk < P.Tk) {
            const int64_t off = ((int64_t)kk * P.Hkv + g) * D + c0 + db * 32 + li;
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
      const int kk = kbase + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kk < P.Tk) {
        const int64_t off = ((int64_t)kk * P.Hkv + g) * D + c0 + db * 32 + li;
        P.dk[off] = (bf16)(dka[db][r] * P.scale);
        P.dv[off] = (bf16)dva[db][r];
      }
    }
}

// grid: (items x splits, key-tile width / 64).
hipError_t launch_dkdv_d256(const AttnParams& P, int n_items, bool hm, hipStream_t stream) {
  const dim3 grid(n_items * P.kv_splits, P.t.BN / 64);
  if (hm) hipLaunchKernelGGL(dkdv256_kernel<true>, grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL(dkdv256_kernel<false>, grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace mad
