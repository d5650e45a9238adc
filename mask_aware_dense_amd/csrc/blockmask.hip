// blockmask.hip -- dynamic block-sparse masks generated on the GPU.
//
// The coarse stage of a block-sparse method (LongCA-bench appendix A.3, VSA:
// mean pooling of the QK scores over block pairs) followed by the top-k
// selection of appendix A.2: for mask group g, query block qb and key block kb
//   score[g][qb][kb] = scale * mean over i in qb, j in kb, h in g of q_i,h . k_j,kv(h)
//                    = scale * qbar[g][qb] . kbar[kv(g)][kb]
// (the mean of the dot products equals the dot product of the means), where
// qbar averages Q over the block's rows and the group's query heads and kbar
// averages K over the block's rows.  Each (g, qb) keeps its k = n_kb -
// floor(pct * n_kb / 100) (at least 1) highest-scoring key blocks; equal
// scores are taken in ascending key-block order.  A group's query heads must
// share one KV head (GQA groups, or one group per query head).
//
// Kernels: two pooling passes (HBM-bound: they read Q and K once), then one
// workgroup per (g, qb) that forms the row of n_kb scores in registers, finds
// the k-th largest by a bitwise radix select over order-preserving integer
// keys, and writes the keep bitmap row with wave ballots.  The score matrix
// is never stored unless the caller asks for it.
#include <algorithm>
#include <string>

#include <type_traits>

#include "kernel_common.hpp"

namespace mad {

// out[grp][blk][:] = mean over rows [edges[blk], edges[blk+1]) and heads
// grp*HG .. grp*HG+HG-1 of x[row][head][:].
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const bf16* x, int64_t tok, int64_t head, const int32_t* edges,
                                                   int32_t nblk, int32_t HG, int32_t T, float* out) {
  constexpr int CH = D / 8, NSLOT = 256 / CH;
  __shared__ float part[NSLOT][D];
  const int grp = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int c8 = threadIdx.x % CH, slot = threadIdx.x / CH;
  // Edges are clamped to [0, T] so that no edge array can send a read out of bounds.
  const int r0 = min(max(sld(edges + blk), 0), T), r1 = min(max(sld(edges + blk + 1), r0), T);
  const int64_t n = (int64_t)(r1 - r0) * HG;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t it = slot; it < n; it += NSLOT) {
    const int64_t r = r0 + it / HG, hd = (int64_t)grp * HG + it % HG;
    const bf16x8 v = ld16(x + r * tok + hd * head + 8 * c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[slot][8 * c8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int k = 0; k < NSLOT; ++k) s += part[k][threadIdx.x];
    out[((int64_t)grp * nblk + blk) * D + threadIdx.x] = n > 0 ? s / (float)n : 0.f;
  }
}

// Order-preserving integer key of a float (larger float <-> larger key); -0 is
// first turned into +0 so that equal scores have equal keys.
__device__ __forceinline__ uint32_t sort_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TOPK_E = 32;  // key blocks per thread: n_kb <= 256 * 32

// One workgroup per (g, qb): scores of the row, top-k, keep bitmap row.
template <int D>
__global__ __launch_bounds__(256) void score_topk_kernel(const float* qp, const float* kp, int32_t nqb, int32_t nkb,
                                                         int32_t grp_per_kv, int32_t kkeep, float scale,
                                                         uint64_t* keep, int32_t nw, float* scores_out) {
  __shared__ float qs[D];
  __shared__ uint32_t red[8];
  const int row = blockIdx.x, g = row / nqb;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* kb0 = kp + (int64_t)(g / grp_per_kv) * nkb * D;
  if (tid < D) qs[tid] = qp[(int64_t)row * D + tid];
  __syncthreads();

  uint32_t key[TOPK_E];
  const int E = (nkb + 255) / 256;
#pragma unroll
  for (int e = 0; e < TOPK_E; ++e) {
    key[e] = 0u;  // below every real key (real keys of finite scores are never 0)
    const int j = e * 256 + tid;
    if (e < E && j < nkb) {
      const float4* kr = reinterpret_cast<const float4*>(kb0 + (int64_t)j * D);
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < D / 4; ++c) {
        const float4 v = kr[c];
        s += qs[4 * c] * v.x + qs[4 * c + 1] * v.y + qs[4 * c + 2] * v.z + qs[4 * c + 3] * v.w;
      }
      s *= scale;
      if (scores_out) scores_out[(int64_t)row * nkb + j] = s;
      key[e] = sort_key(s);
    }
  }
  // Block-wide count of keys >= c.
  auto count_ge = [&](uint32_t c) {
    uint32_t n = 0;
#pragma unroll
    for (int e = 0; e < TOPK_E; ++e) n += (e < E && key[e] >= c) ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
    __syncthreads();
    if (lane == 0) red[wv] = n;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
  };
  // The k-th largest key K: the largest value with count(key >= K) >= k.
  uint32_t K = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = K | (1u << bit);
    if (count_ge(c) >= (uint32_t)kkeep) K = c;
  }
  // Keep every key > K, then keys == K in ascending index order up to k.
  const uint32_t above = count_ge(K + 1u);  // K < 0xffffffff: no finite score reaches it
  const uint32_t room = (uint32_t)kkeep - above;
  uint32_t seen = 0;
  uint64_t* out = keep + (int64_t)row * nw;
#pragma unroll
  for (int e = 0; e < TOPK_E; ++e) {
    if (e < E) {  // uniform
      const int j = e * 256 + tid;
      const bool tie = j < nkb && key[e] == K;
      const uint64_t tb = __ballot(tie);
      __syncthreads();
      if (lane == 0) red[4 + wv] = (uint32_t)__popcll(tb);
      __syncthreads();
      uint32_t before = seen + (uint32_t)__popcll(tb & ((1ull << lane) - 1ull));
      for (int x = 0; x < wv; ++x) before += red[4 + x];
      const bool kept = j < nkb && (key[e] > K || (tie && before < room));
      const uint64_t word = __ballot(kept);
      if (lane == 0 && 4 * e + wv < nw) out[4 * e + wv] = word;  // keys 256e + 64wv + lane
      seen += red[4] + red[5] + red[6] + red[7];
    }
  }
}

namespace {
mad_status hipf(const char* where, hipError_t e) {
  return fail(MAD_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}
}  // namespace
}  // namespace mad

using namespace mad;

extern "C" mad_status mad_block_mask_workspace_bytes(int32_t n_groups, int32_t Hkv, int32_t n_qb, int32_t n_kb,
                                                     int32_t d, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(MAD_ERR_INVALID, "mad_block_mask_workspace_bytes: bytes is NULL");
  if (n_groups <= 0 || Hkv <= 0 || n_qb <= 0 || n_kb <= 0) return fail(MAD_ERR_INVALID, "mad_block_mask_workspace_bytes: bad sizes");
  if (d != 64 && d != 128 && d != 256)
    return fail(MAD_ERR_UNSUPPORTED, "mad_block_mask_workspace_bytes: head dim must be 64, 128 or 256");
  const size_t a = ((size_t)n_groups * n_qb * d * 4 + 255) / 256 * 256;
  *bytes = a + (size_t)Hkv * n_kb * d * 4;
  return MAD_OK;
}

extern "C" mad_status mad_block_mask(const void* q, const void* k, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv,
                                     int32_t d, int32_t n_groups, const int32_t* q_edges, int32_t n_qb,
                                     const int32_t* k_edges, int32_t n_kb, int32_t sparsity_pct, float scale,
                                     void* workspace, size_t ws_bytes, uint64_t* keep, float* scores,
                                     hipStream_t stream) {
  clear_error();
  const std::string f = "mad_block_mask";
  if (Tq <= 0 || Tk <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return fail(MAD_ERR_INVALID, f + ": bad sizes");
  if (d != 64 && d != 128 && d != 256) return fail(MAD_ERR_UNSUPPORTED, f + ": head dim must be 64, 128 or 256");
  if (n_groups <= 0 || Hq % n_groups || n_groups % Hkv)
    return fail(MAD_ERR_INVALID, f + ": n_groups must divide Hq and be a multiple of Hkv (a group's heads share one KV head)");
  if (n_qb <= 0 || n_kb <= 0 || n_qb > Tq || n_kb > Tk) return fail(MAD_ERR_INVALID, f + ": bad block counts");
  if (n_kb > 256 * TOPK_E) return fail(MAD_ERR_UNSUPPORTED, f + ": at most " + std::to_string(256 * TOPK_E) + " key blocks");
  if (sparsity_pct < 0 || sparsity_pct > 100) return fail(MAD_ERR_INVALID, f + ": sparsity_pct must be in 0..100");
  if (!(scale == scale)) return fail(MAD_ERR_INVALID, f + ": scale is NaN");
  if (!q || !k || !q_edges || !k_edges || !keep || !workspace) return fail(MAD_ERR_INVALID, f + ": NULL pointer");
  if (((uintptr_t)q & 15u) || ((uintptr_t)k & 15u) || ((uintptr_t)workspace & 255u) || ((uintptr_t)keep & 7u) ||
      ((uintptr_t)q_edges & 3u) || ((uintptr_t)k_edges & 3u) || ((uintptr_t)scores & 3u))
    return fail(MAD_ERR_UNSUPPORTED, f + ": q/k 16-byte, workspace 256-byte, keep 8-byte, edges/scores 4-byte alignment");
  size_t need = 0;
  mad_block_mask_workspace_bytes(n_groups, Hkv, n_qb, n_kb, d, &need);
  if (ws_bytes < need) return fail(MAD_ERR_INVALID, f + ": workspace must hold " + std::to_string(need) + " bytes");
  float* qp = (float*)workspace;
  float* kp = (float*)((char*)workspace + ((size_t)n_groups * n_qb * d * 4 + 255) / 256 * 256);
  const int kkeep = std::max(1, n_kb - (int)(((int64_t)sparsity_pct * n_kb) / 100));
  const int nw = (n_kb + 63) / 64;
  const int64_t q_tok = (int64_t)Hq * d, k_tok = (int64_t)Hkv * d;
  auto run = [&](auto dtag) {
    constexpr int DD = decltype(dtag)::value;
    hipLaunchKernelGGL(pool_kernel<DD>, dim3(n_groups * n_qb), dim3(256), 0, stream, (const bf16*)q, q_tok, (int64_t)d,
                       q_edges, n_qb, Hq / n_groups, Tq, qp);
    hipLaunchKernelGGL(pool_kernel<DD>, dim3(Hkv * n_kb), dim3(256), 0, stream, (const bf16*)k, k_tok, (int64_t)d,
                       k_edges, n_kb, 1, Tk, kp);
    hipLaunchKernelGGL(score_topk_kernel<DD>, dim3(n_groups * n_qb), dim3(256), 0, stream, qp, kp, n_qb, n_kb,
                       n_groups / Hkv, kkeep, scale, keep, nw, scores);
  };
  if (d == 128) run(std::integral_constant<int, 128>{});
  else if (d == 256) run(std::integral_constant<int, 256>{});
  else run(std::integral_constant<int, 64>{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hipf("mad_block_mask: launch", e);
  return MAD_OK;
}
