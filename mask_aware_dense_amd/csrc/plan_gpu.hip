// plan_gpu.hip -- block-sparse plans compiled on the GPU from a keep bitmap
// that is already in device memory.
//
// A dynamic block-sparse mask (LongCA-bench appendix A.2 and the VSA coarse
// stage of appendix A.3) changes every step: its keep bitmap is produced on
// the GPU (mad_block_mask), and compiling it on the host costs a copy of the
// bitmap, a synchronisation and a host pass over every tile of both tilings
// (tens of milliseconds at 128K).  Here the same compilation runs as GPU
// kernels; the result is bit-identical to mad_sparse_plan's over the same
// edges and bits:
//   1. classify every tile of both tilings (EMPTY / FULL / PARTIAL from the
//      keep bits of the blocks it covers) and count each visit list's
//      entries, one wave per (mask group, major tile);
//   2. turn the counts into list offsets (one workgroup scan per tiling) and
//      count the unmasked pairs per group;
//   3. read back the offsets and counts (the one synchronisation: the plan's
//      device block is sized from them);
//   4. fill the lists (entry = minor tile | PARTIAL bit, aux = the FULL
//      strips of a PARTIAL tile whose strips are all FULL or EMPTY, else -1)
//      and the longest-first orders of the major tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "plan.hpp"

namespace mad {
namespace {

struct BlockSrc {
  const int32_t* row_qb;  // [Tq] query block of each row
  const int32_t* col_kb;  // [Tk] key block of each key
  const uint64_t* keep;   // [G][n_qb][nw]
  int32_t n_qb, nw, G, Tq, Tk;
};

__device__ __forceinline__ bool keep_bit(const BlockSrc& s, int g, int qb, int kb) {
  return (s.keep[((size_t)g * s.n_qb + qb) * s.nw + (kb >> 6)] >> (kb & 63)) & 1ull;
}

// Class of rows [r0, r1) x keys [c0, c1) (non-empty, in range) for group g.
__device__ uint8_t rect_class(const BlockSrc& s, int g, int r0, int r1, int c0, int c1) {
  const int qa = s.row_qb[r0], qz = s.row_qb[r1 - 1];
  const int ka = s.col_kb[c0], kz = s.col_kb[c1 - 1];
  bool any = false, all = true;
  for (int qb = qa; qb <= qz; ++qb)
    for (int kb = ka; kb <= kz; ++kb) {
      const bool k = keep_bit(s, g, qb, kb);
      any |= k;
      all &= k;
    }
  return !any ? CLS_EMPTY : (all ? CLS_FULL : CLS_PARTIAL);
}

// The FULL strips (bit w) of a PARTIAL tile whose four wave strips (32 rows
// for tiling 0, 32 keys for tiling 1) are each FULL or EMPTY; -1 otherwise.
__device__ int32_t strip_classes(const BlockSrc& s, int g, bool rows_split, int r0, int r1, int c0, int c1) {
  int32_t full = 0;
  for (int w = 0; w < 4; ++w) {
    int a0 = r0, a1 = r1, b0 = c0, b1 = c1;
    if (rows_split) {
      a0 = r0 + 32 * w;
      a1 = min(r1, a0 + 32);
    } else {
      b0 = c0 + 32 * w;
      b1 = min(c1, b0 + 32);
    }
    if (a0 >= a1 || b0 >= b1) continue;
    const uint8_t c = rect_class(s, g, a0, a1, b0, b1);
    if (c == CLS_PARTIAL) return -1;
    if (c == CLS_FULL) full |= 1 << w;
  }
  return full;
}

struct TileGeom {
  int BM, BN, nqt, nkt;
  bool csc;  // lists per key tile (tiling 1) instead of per query tile
};

__device__ __forceinline__ uint8_t tile_class(const BlockSrc& s, const TileGeom& t, int g, int M, int m, int& r0,
                                              int& r1, int& c0, int& c1) {
  const int qt = t.csc ? m : M, kt = t.csc ? M : m;
  r0 = qt * t.BM;
  r1 = min(s.Tq, r0 + t.BM);
  c0 = kt * t.BN;
  c1 = min(s.Tk, c0 + t.BN);
  return rect_class(s, g, r0, r1, c0, c1);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Step 1: entries of each (group, major tile) list and the tile class counts.
// One wave per list; wave index g * nmaj + M, the order of the list offsets.
__global__ __launch_bounds__(256) void count_kernel(BlockSrc s, TileGeom t, int32_t* cnt,
                                                    unsigned long long* ncls) {
  const int nmaj = t.csc ? t.nkt : t.nqt, nmin = t.csc ? t.nqt : t.nkt;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= (int64_t)s.G * nmaj) return;  // the whole wave leaves together
  const int g = (int)(wave / nmaj), M = (int)(wave % nmaj);
  int n = 0, nf = 0, np = 0;
  for (int m = lane; m < nmin; m += 64) {
    int r0, r1, c0, c1;
    const uint8_t c = tile_class(s, t, g, M, m, r0, r1, c0, c1);
    n += c != CLS_EMPTY;
    nf += c == CLS_FULL;
    np += c == CLS_PARTIAL;
  }
  n = wave_sum(n);
  nf = wave_sum(nf);
  np = wave_sum(np);
  if (lane == 0) {
    cnt[wave] = n;
    atomicAdd(&ncls[CLS_EMPTY], (unsigned long long)(nmin - n));
    atomicAdd(&ncls[CLS_FULL], (unsigned long long)nf);
    atomicAdd(&ncls[CLS_PARTIAL], (unsigned long long)np);
  }
}

// Step 2a: list offsets.  ptr[g * (nmaj + 1) + M] = entries before list
// (g, M); ptr[g * (nmaj + 1) + nmaj] = entries up to the end of group g.
// One workgroup of 1024 threads, each owning a contiguous run of lists.
// total receives the entry count (int64, checked on the host).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* cnt, int G, int nmaj, int32_t* ptr,
                                                    long long* total) {
  __shared__ long long part[1024];
  const int64_t N = (int64_t)G * nmaj;
  const int64_t per = (N + 1023) / 1024;
  const int tid = threadIdx.x;
  const int64_t a = min(N, tid * per), b = min(N, a + per);
  long long sum = 0;
  for (int64_t x = a; x < b; ++x) sum += cnt[x];
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 1024 partial sums (Hillis-Steele)
  for (int o = 1; o < 1024; o <<= 1) {
    const long long v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  long long run = part[tid] - sum;  // exclusive prefix of this thread's run
  for (int64_t x = a; x < b; ++x) {
    const int g = (int)(x / nmaj), M = (int)(x % nmaj);
    ptr[(int64_t)g * (nmaj + 1) + M] = (int32_t)run;
    run += cnt[x];
    if (M == nmaj - 1) ptr[(int64_t)g * (nmaj + 1) + nmaj] = (int32_t)run;
  }
  if (tid == 1023) *total = part[1023];
}

// Step 2b: unmasked pairs per group (sum of the kept blocks' areas).
__global__ __launch_bounds__(256) void pairs_kernel(BlockSrc s, const int32_t* q_edges, const int32_t* k_edges,
                                                    int n_kb, unsigned long long* pairs) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (int64_t)s.G * s.n_qb) return;
  const int g = (int)(x / s.n_qb), qb = (int)(x % s.n_qb);
  const uint64_t* row = s.keep + ((size_t)g * s.n_qb + qb) * s.nw;
  unsigned long long keys = 0;
  for (int wd = 0; wd < s.nw; ++wd) {
    uint64_t bits = row[wd];
    if (wd == s.nw - 1 && (n_kb & 63)) bits &= (1ull << (n_kb & 63)) - 1ull;
    while (bits) {
      const int kb = wd * 64 + __builtin_ctzll(bits);
      bits &= bits - 1ull;
      keys += (unsigned long long)(k_edges[kb + 1] - k_edges[kb]);
    }
  }
  if (keys) atomicAdd(&pairs[g], keys * (unsigned long long)(q_edges[qb + 1] - q_edges[qb]));
}

// Step 4a: the lists.  Same traversal as count_kernel; lanes that hold a
// non-EMPTY tile take consecutive slots in minor-tile order.
__global__ __launch_bounds__(256) void fill_kernel(BlockSrc s, TileGeom t, const int32_t* ptr, int32_t* ent,
                                                   int32_t* ent_aux) {
  const int nmaj = t.csc ? t.nkt : t.nqt, nmin = t.csc ? t.nqt : t.nkt;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= (int64_t)s.G * nmaj) return;
  const int g = (int)(wave / nmaj), M = (int)(wave % nmaj);
  int base = ptr[(int64_t)g * (nmaj + 1) + M];
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
  for (int m0 = 0; m0 < nmin; m0 += 64) {
    const int m = m0 + lane;
    uint8_t c = CLS_EMPTY;
    int r0 = 0, r1 = 0, c0 = 0, c1 = 0;
    if (m < nmin) c = tile_class(s, t, g, M, m, r0, r1, c0, c1);
    const uint64_t mask = __ballot(c != CLS_EMPTY);
    if (c != CLS_EMPTY) {
      const int pos = base + __popcll(mask & below);
      ent[pos] = (int32_t)((uint32_t)m | (c == CLS_PARTIAL ? ENT_PARTIAL : 0u));
      ent_aux[pos] = c == CLS_PARTIAL ? strip_classes(s, g, !t.csc, r0, r1, c0, c1) : -1;
    }
    base += __popcll(mask);
  }
}

// Step 4b: work per major tile summed over groups, then its rank in
// descending work (ties by index, as a stable sort): order[rank] = M.
__global__ __launch_bounds__(256) void work_kernel(const int32_t* cnt, int G, int nmaj, long long* work) {
  const int M = blockIdx.x * 256 + threadIdx.x;
  if (M >= nmaj) return;
  long long w = 0;
  for (int g = 0; g < G; ++g) w += cnt[(int64_t)g * nmaj + M];
  work[M] = w;
}
__global__ __launch_bounds__(256) void order_kernel(const long long* work, int nmaj, int32_t* order) {
  const int M = blockIdx.x * 256 + threadIdx.x;
  if (M >= nmaj) return;
  const long long w = work[M];
  int rank = 0;
  for (int x = 0; x < nmaj; ++x) {
    const long long v = work[x];
    rank += (v > w) || (v == w && x < M);
  }
  order[rank] = M;
}

__global__ __launch_bounds__(256) void zero_u64_kernel(unsigned long long* p, int n) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x < n) p[x] = 0ull;
}

// Copy of the keep bitmap with the bits past n_kb cleared (as the host
// compile stores it).
__global__ __launch_bounds__(256) void keep_copy_kernel(const uint64_t* src, uint64_t* dst, int64_t rows, int nw,
                                                        int n_kb) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= rows * nw) return;
  uint64_t v = src[x];
  if ((int)(x % nw) == nw - 1 && (n_kb & 63)) v &= (1ull << (n_kb & 63)) - 1ull;
  dst[x] = v;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

mad_status hip_err(const char* what, hipError_t e) {
  return fail(MAD_ERR_HIP, std::string("mad_sparse_plan_device: ") + what + ": " + hipGetErrorString(e));
}

}  // namespace
}  // namespace mad

using namespace mad;

extern "C" mad_status mad_sparse_plan_device(int32_t n_groups, const int32_t* q_edges, int32_t n_qb,
                                             const int32_t* k_edges, int32_t n_kb, const uint64_t* keep,
                                             hipStream_t stream, mad_plan** out) {
  clear_error();
  if (!out) return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: out is NULL");
  *out = nullptr;
  if (!q_edges || !k_edges || !keep) return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: NULL pointer");
  if (n_groups <= 0 || n_qb <= 0 || n_kb <= 0) return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: sizes must be > 0");
  if (q_edges[0] != 0 || k_edges[0] != 0) return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: edges must start at 0");
  for (int32_t x = 0; x < n_qb; ++x)
    if (q_edges[x + 1] <= q_edges[x])
      return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: q_edges not strictly increasing");
  for (int32_t x = 0; x < n_kb; ++x)
    if (k_edges[x + 1] <= k_edges[x])
      return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: k_edges not strictly increasing");
  if ((uintptr_t)keep % 8) return fail(MAD_ERR_INVALID, "mad_sparse_plan_device: keep must be 8-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_err("hipGetDevice", e);

  mad_plan* p = new (std::nothrow) mad_plan();
  if (!p) return fail(MAD_ERR_NOMEM, "mad_sparse_plan_device: out of host memory");
  void* tmp = nullptr;
  void* mem = nullptr;
  auto bail = [&](mad_status st) {
    if (tmp) (void)hipFree(tmp);
    if (mem) (void)hipFree(mem);
    delete p;
    return st;
  };
  std::vector<int32_t> row_qb, col_kb;
  try {
    p->Tq = q_edges[n_qb];
    p->Tk = k_edges[n_kb];
    p->G = n_groups;
    p->mode = MODE_BLOCKS;
    p->n_qb = n_qb;
    p->n_kb = n_kb;
    p->nw = (n_kb + 63) / 64;
    p->q_edges.assign(q_edges, q_edges + n_qb + 1);
    p->k_edges.assign(k_edges, k_edges + n_kb + 1);
    row_qb.resize(p->Tq);
    col_kb.resize(p->Tk);
    for (int32_t b = 0; b < n_qb; ++b)
      for (int32_t i = q_edges[b]; i < q_edges[b + 1]; ++i) row_qb[i] = b;
    for (int32_t b = 0; b < n_kb; ++b)
      for (int32_t j = k_edges[b]; j < k_edges[b + 1]; ++j) col_kb[j] = b;
  } catch (const std::bad_alloc&) {
    return bail(fail(MAD_ERR_NOMEM, "mad_sparse_plan_device: out of host memory"));
  }
  const int G = n_groups;
  TileGeom geo[2];
  for (int w = 0; w < 2; ++w) {
    TilingHost& t = p->tiling[w];
    t.BM = w == 0 ? BM0 : BM1;
    t.BN = w == 0 ? BN0 : dkdv_tile_keys(k_edges, n_kb);
    t.nqt = (p->Tq + t.BM - 1) / t.BM;
    t.nkt = (p->Tk + t.BN - 1) / t.BN;
    geo[w] = TileGeom{t.BM, t.BN, t.nqt, t.nkt, w == 1};
  }
  const int nmaj[2] = {p->tiling[0].nqt, p->tiling[1].nkt};

  // Scratch: row/col block maps and edges (the builder's view of the mask),
  // per-list counts and offsets, work per major tile, the scalar results.
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_rq = take((size_t)p->Tq * 4), o_ck = take((size_t)p->Tk * 4);
  const size_t o_qe = take((size_t)(n_qb + 1) * 4), o_ke = take((size_t)(n_kb + 1) * 4);
  size_t o_cnt[2], o_ptr[2], o_work[2];
  for (int w = 0; w < 2; ++w) {
    o_cnt[w] = take((size_t)G * nmaj[w] * 4);
    o_ptr[w] = take((size_t)G * (nmaj[w] + 1) * 4);
    o_work[w] = take((size_t)nmaj[w] * 8);
  }
  const int n_scalar = 2 + 6 + G;  // totals[2], class counts[2][3], pairs[G]
  const size_t o_sc = take((size_t)n_scalar * 8);
  e = hipMalloc(&tmp, off);
  if (e != hipSuccess) return bail(fail(MAD_ERR_NOMEM, std::string("mad_sparse_plan_device: hipMalloc: ") + hipGetErrorString(e)));
  char* T = (char*)tmp;
  if ((e = hipMemcpyAsync(T + o_rq, row_qb.data(), (size_t)p->Tq * 4, hipMemcpyHostToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(T + o_ck, col_kb.data(), (size_t)p->Tk * 4, hipMemcpyHostToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(T + o_qe, q_edges, (size_t)(n_qb + 1) * 4, hipMemcpyHostToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(T + o_ke, k_edges, (size_t)(n_kb + 1) * 4, hipMemcpyHostToDevice, stream)) != hipSuccess)
    return bail(hip_err("hipMemcpyAsync", e));
  unsigned long long* sc = (unsigned long long*)(T + o_sc);
  BlockSrc src{(const int32_t*)(T + o_rq), (const int32_t*)(T + o_ck), keep, n_qb, p->nw, G, p->Tq, p->Tk};

  hipLaunchKernelGGL(zero_u64_kernel, dim3((n_scalar + 255) / 256), dim3(256), 0, stream, sc, n_scalar);
  for (int w = 0; w < 2; ++w) {
    const int64_t waves = (int64_t)G * nmaj[w];
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, src, geo[w],
                       (int32_t*)(T + o_cnt[w]), sc + 2 + 3 * w);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, (const int32_t*)(T + o_cnt[w]), G, nmaj[w],
                       (int32_t*)(T + o_ptr[w]), (long long*)(sc + w));
    hipLaunchKernelGGL(work_kernel, dim3((nmaj[w] + 255) / 256), dim3(256), 0, stream,
                       (const int32_t*)(T + o_cnt[w]), G, nmaj[w], (long long*)(T + o_work[w]));
  }
  const int64_t nqrows = (int64_t)G * n_qb;
  hipLaunchKernelGGL(pairs_kernel, dim3((unsigned)((nqrows + 255) / 256)), dim3(256), 0, stream, src,
                     (const int32_t*)(T + o_qe), (const int32_t*)(T + o_ke), n_kb, sc + 8);
  if ((e = hipGetLastError()) != hipSuccess) return bail(hip_err("launch", e));

  // The one synchronisation: list sizes, class counts, pairs and offsets.
  std::vector<unsigned long long> scal(n_scalar);
  try {
    for (int w = 0; w < 2; ++w) p->tiling[w].ptr.resize((size_t)G * (nmaj[w] + 1));
    p->pairs.resize(G);
  } catch (const std::bad_alloc&) {
    return bail(fail(MAD_ERR_NOMEM, "mad_sparse_plan_device: out of host memory"));
  }
  if ((e = hipMemcpyAsync(scal.data(), sc, (size_t)n_scalar * 8, hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return bail(hip_err("hipMemcpyAsync", e));
  for (int w = 0; w < 2; ++w)
    if ((e = hipMemcpyAsync(p->tiling[w].ptr.data(), T + o_ptr[w], (size_t)G * (nmaj[w] + 1) * 4,
                            hipMemcpyDeviceToHost, stream)) != hipSuccess)
      return bail(hip_err("hipMemcpyAsync", e));
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return bail(hip_err("hipStreamSynchronize", e));
  for (int w = 0; w < 2; ++w) {
    if (scal[w] > (unsigned long long)INT32_MAX)
      return bail(fail(MAD_ERR_NOMEM, "mad_sparse_plan_device: visit lists exceed 2^31 entries"));
    for (int c = 0; c < 3; ++c) p->tiling[w].n_class[c] = (int64_t)scal[2 + 3 * w + c];
  }
  for (int g = 0; g < G; ++g) p->pairs[g] = (int64_t)scal[8 + g];

  // The plan's device block, laid out as mad_plan_upload lays out a host plan.
  const size_t nkeep = (size_t)G * n_qb * p->nw;
  size_t total = 0;
  auto add = [&](size_t bytes) {
    const size_t o = total;
    total += align256(bytes);
    return o;
  };
  size_t f_ptr[2], f_ent[2], f_aux[2], f_ord[2];
  for (int w = 0; w < 2; ++w) {
    f_ptr[w] = add((size_t)G * (nmaj[w] + 1) * 4);
    f_ent[w] = add((size_t)scal[w] * 4);
    f_aux[w] = add((size_t)scal[w] * 4);
    f_ord[w] = add((size_t)nmaj[w] * 4);
  }
  const size_t f_sl = add(0), f_ts = add(0);
  const size_t f_rq = add((size_t)p->Tq * 4), f_ck = add((size_t)p->Tk * 4);
  const size_t f_ke = add((size_t)(n_kb + 1) * 4), f_qe = add((size_t)(n_qb + 1) * 4);
  const size_t f_kp = add(nkeep * 8);
  e = hipMalloc(&mem, total);
  if (e != hipSuccess) return bail(fail(MAD_ERR_NOMEM, std::string("mad_sparse_plan_device: hipMalloc: ") + hipGetErrorString(e)));
  char* B = (char*)mem;
  for (int w = 0; w < 2; ++w)
    if ((e = hipMemcpyAsync(B + f_ptr[w], T + o_ptr[w], (size_t)G * (nmaj[w] + 1) * 4, hipMemcpyDeviceToDevice,
                            stream)) != hipSuccess)
      return bail(hip_err("hipMemcpyAsync", e));
  if ((e = hipMemcpyAsync(B + f_rq, T + o_rq, (size_t)p->Tq * 4, hipMemcpyDeviceToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(B + f_ck, T + o_ck, (size_t)p->Tk * 4, hipMemcpyDeviceToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(B + f_ke, T + o_ke, (size_t)(n_kb + 1) * 4, hipMemcpyDeviceToDevice, stream)) != hipSuccess ||
      (e = hipMemcpyAsync(B + f_qe, T + o_qe, (size_t)(n_qb + 1) * 4, hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return bail(hip_err("hipMemcpyAsync", e));
  const int64_t rows = (int64_t)G * n_qb;
  hipLaunchKernelGGL(keep_copy_kernel, dim3((unsigned)((rows * p->nw + 255) / 256)), dim3(256), 0, stream, keep,
                     (uint64_t*)(B + f_kp), rows, p->nw, n_kb);
  for (int w = 0; w < 2; ++w) {
    const int64_t waves = (int64_t)G * nmaj[w];
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, src, geo[w],
                       (const int32_t*)(T + o_ptr[w]), (int32_t*)(B + f_ent[w]), (int32_t*)(B + f_aux[w]));
    hipLaunchKernelGGL(order_kernel, dim3((nmaj[w] + 255) / 256), dim3(256), 0, stream,
                       (const long long*)(T + o_work[w]), nmaj[w], (int32_t*)(B + f_ord[w]));
  }
  if ((e = hipGetLastError()) != hipSuccess) return bail(hip_err("launch", e));

  for (int w = 0; w < 2; ++w) {
    TilingDev& d = p->tdev[w];
    d.ptr = (const int32_t*)(B + f_ptr[w]);
    d.ent = (const int32_t*)(B + f_ent[w]);
    d.ent_aux = (const int32_t*)(B + f_aux[w]);
    d.order = (const int32_t*)(B + f_ord[w]);
    d.nmajor = nmaj[w];
    d.nminor = w == 0 ? p->tiling[0].nkt : p->tiling[1].nqt;
    d.BN = p->tiling[w].BN;
    d.uniform = 0;  // block-sparse: the head-major kernels are chosen by the mask mode
  }
  MaskDev& m = p->mdev;
  m.mode = MODE_BLOCKS;
  m.Tq = p->Tq;
  m.Tk = p->Tk;
  m.slices = (const mad_slice*)(B + f_sl);
  m.tile_slices = (const int32_t*)(B + f_ts);
  m.row_qb = (const int32_t*)(B + f_rq);
  m.col_kb = (const int32_t*)(B + f_ck);
  m.k_edges = (const int32_t*)(B + f_ke);
  m.q_edges = (const int32_t*)(B + f_qe);
  m.keep = (const uint64_t*)(B + f_kp);
  m.n_qb = n_qb;
  m.n_kb = n_kb;
  m.nw = p->nw;
  p->dev_mem = mem;
  p->dev_bytes = total;
  p->dev_id = dev;
  p->dev_tmp = tmp;  // read by the kernels still queued on stream; freed with the plan
  p->on_device = true;
  *out = p;
  return MAD_OK;
}
