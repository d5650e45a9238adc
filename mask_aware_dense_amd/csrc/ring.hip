// ring.hip -- LSE merge of partial attention results, and one rank's share of
// ring context-parallel attention run on one GPU (LongCA-bench section 2.3;
// the notes' key designs 3 and 4).
//
// The merge is an HBM-bound elementwise pass: for every (row, head) it reads
// the parts' LSE values and d-wide output rows once and writes one merged row,
// D/8 lanes per (row, head), 16 bytes per lane and part.
//
// The ring object replays, on one GPU, what rank `rank` of an n-rank ring
// computes: step i receives the K/V chunk of rank (rank - i) mod n.  Here the
// "receive" is a device-to-device copy from a global K/V into one of two
// staging buffers on a copy stream, so that the copy for step i + 1 overlaps
// the kernels of step i, as the transfer would overlap compute on a real ring.
#include <algorithm>
#include <string>
#include <vector>

#include "kernel_common.hpp"

namespace mad {

mad_status attn_bwd_impl(const mad_plan* p, const void* q, const void* k, const void* v, const void* o,
                         const void* d_o, const float* lse, void* dq, float* dq_acc, void* dk, void* dv,
                         void* workspace, size_t ws_bytes, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d,
                         const int64_t* strides, float scale, uint32_t phases, hipStream_t stream);

constexpr int MAX_PARTS = 32;

struct MergeArgs {
  const bf16* o[MAX_PARTS];
  const float* lse[MAX_PARTS];
  bf16* out;
  float* lse_out;
  int32_t n, Tq, Hq;
};

// LSE = m + ln sum_t exp(LSE_t - m) with m = max_t LSE_t; O = sum_t w_t O_t
// with w_t = exp(LSE_t - m) / sum_s exp(LSE_s - m).
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs A) {
  constexpr int LPR = D / 8;  // lanes per (row, head)
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;  // row * Hq + head
  const int sub = threadIdx.x % LPR;
  if (r >= (int64_t)A.Tq * A.Hq) return;
  const int64_t i = r / A.Hq, h = r % A.Hq;
  const int64_t li = h * A.Tq + i;
  float m = -INFINITY;
  for (int t = 0; t < A.n; ++t) m = fmaxf(m, A.lse[t][li]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.f;
    for (int t = 0; t < A.n; ++t) {
      const float l = A.lse[t][li];
      if (l == -INFINITY) continue;
      const float wt = __expf(l - m);
      s += wt;
      const bf16x8 x = ld16(A.o[t] + r * D + 8 * sub);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wt * (float)x[e];
    }
    const float inv = 1.f / s;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = m + __logf(s);
  }
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (bf16)acc[e];
  *reinterpret_cast<bf16x8*>(A.out + r * D + 8 * sub) = y;
  if (sub == 0) A.lse_out[li] = lse;
}

// Zero n16 16-byte words.
__global__ __launch_bounds__(256) void zero_kernel(u32x4* p, int64_t n16) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n16; x += (int64_t)gridDim.x * 256)
    p[x] = u32x4{0u, 0u, 0u, 0u};
}

// fp32 -> bf16 (round to nearest even), 8 values per lane; n8 = count / 8.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* src, bf16* dst, int64_t n8) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n8; x += (int64_t)gridDim.x * 256) {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * x];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * x + 1];
    bf16x8 y;
    y[0] = (bf16)a.x; y[1] = (bf16)a.y; y[2] = (bf16)a.z; y[3] = (bf16)a.w;
    y[4] = (bf16)b.x; y[5] = (bf16)b.y; y[6] = (bf16)b.z; y[7] = (bf16)b.w;
    reinterpret_cast<bf16x8*>(dst)[x] = y;
  }
}

namespace {

mad_status hipf(const char* where, hipError_t e) {
  return fail(MAD_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int grid_for(int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 4096); }

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(bytes / 16)), dim3(256), 0, s, (u32x4*)p, bytes / 16);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& A, int d, hipStream_t s) {
  const int64_t threads = (int64_t)A.Tq * A.Hq * (d / 8);
  if (threads == 0) return hipSuccess;
  const int nb = (int)((threads + 255) / 256);
  if (d == 128) hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(nb), dim3(256), 0, s, A);
  else if (d == 256) hipLaunchKernelGGL(lse_merge_kernel<256>, dim3(nb), dim3(256), 0, s, A);
  else hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(nb), dim3(256), 0, s, A);
  return hipGetLastError();
}

}  // namespace
}  // namespace mad

using namespace mad;

extern "C" mad_status mad_lse_merge(int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                                    void* o, float* lse, int32_t Tq, int32_t Hq, int32_t d, hipStream_t stream) {
  clear_error();
  if (n_parts < 1 || n_parts > MAX_PARTS)
    return fail(MAD_ERR_INVALID, "mad_lse_merge: n_parts must be in 1.." + std::to_string(MAX_PARTS));
  if (Tq < 0 || Hq <= 0) return fail(MAD_ERR_INVALID, "mad_lse_merge: sizes must be Tq >= 0 and Hq > 0");
  if (d != 64 && d != 128 && d != 256) return fail(MAD_ERR_UNSUPPORTED, "mad_lse_merge: head dim must be 64, 128 or 256");
  if (!o_parts || !lse_parts) return fail(MAD_ERR_INVALID, "mad_lse_merge: part arrays must not be NULL");
  if (Tq == 0) return MAD_OK;
  if (!o || !lse) return fail(MAD_ERR_INVALID, "mad_lse_merge: o/lse must not be NULL");
  if (!al16(o) || ((uintptr_t)lse & 3u)) return fail(MAD_ERR_UNSUPPORTED, "mad_lse_merge: o must be 16-byte and lse 4-byte aligned");
  MergeArgs A{};
  for (int t = 0; t < n_parts; ++t) {
    if (!o_parts[t] || !lse_parts[t]) return fail(MAD_ERR_INVALID, "mad_lse_merge: a part pointer is NULL");
    if (!al16(o_parts[t]) || ((uintptr_t)lse_parts[t] & 3u))
      return fail(MAD_ERR_UNSUPPORTED, "mad_lse_merge: parts must be 16-byte (o) and 4-byte (lse) aligned");
    A.o[t] = (const bf16*)o_parts[t];
    A.lse[t] = lse_parts[t];
  }
  A.out = (bf16*)o;
  A.lse_out = lse;
  A.n = n_parts;
  A.Tq = Tq;
  A.Hq = Hq;
  hipError_t e = launch_merge(A, d, stream);
  if (e != hipSuccess) return hipf("mad_lse_merge: launch", e);
  return MAD_OK;
}

// ---------------------------------------------------------------------------
// Ring object
// ---------------------------------------------------------------------------
struct mad_ring {
  int32_t layout = 0, N = 0, C = 0, rank = 0, Hq = 0, Hkv = 0, d = 0;
  struct Step {
    int32_t source;
    mad_plan* plan;
    int64_t pairs;
  };
  std::vector<Step> steps;         // non-empty steps in ring order
  std::vector<int32_t> untouched;  // sources whose chunk no step reads
  int dev = -1;
  void* mem = nullptr;
  size_t bytes = 0;
  bf16* kst[2] = {nullptr, nullptr};
  bf16* vst[2] = {nullptr, nullptr};
  bf16* opart = nullptr;  // [n_steps][C, Hq, d]
  float* lpart = nullptr; // [n_steps][Hq, C]
  float* dq_acc = nullptr;
  bf16* dkst = nullptr;   // head-tail: a step's dK / dV before they go to their two global halves
  bf16* dvst = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t copy = nullptr;
  hipEvent_t ev_in = nullptr, ev_copied[2] = {nullptr, nullptr}, ev_done[2] = {nullptr, nullptr};

  int64_t chunk_elems() const { return (int64_t)C * Hkv * d; }  // one K (or V) chunk
  // Global K/V token row where piece `piece` (the chunk itself, or a head-tail half) of source `src` starts.
  int64_t piece_row(int32_t src, int piece) const {
    if (layout == 0) return (int64_t)src * C;
    const int64_t half = C / 2;
    return piece == 0 ? (int64_t)src * half : (int64_t)(2 * N - 1 - src) * half;
  }
  int pieces() const { return layout == 0 ? 1 : 2; }
  int64_t piece_rows() const { return layout == 0 ? C : C / 2; }
};

namespace {

void ring_free(mad_ring* r) {
  for (auto& s : r->steps) mad_plan_destroy(s.plan);
  r->steps.clear();
  if (r->mem) (void)hipFree(r->mem);
  if (r->copy) (void)hipStreamDestroy(r->copy);
  if (r->ev_in) (void)hipEventDestroy(r->ev_in);
  for (int x = 0; x < 2; ++x) {
    if (r->ev_copied[x]) (void)hipEventDestroy(r->ev_copied[x]);
    if (r->ev_done[x]) (void)hipEventDestroy(r->ev_done[x]);
  }
  delete r;
}

// Copy source src's K and V chunk (one or two pieces) into staging slot `slot` on the copy stream.
hipError_t stage(mad_ring* r, const bf16* k, const bf16* v, int32_t src, int slot) {
  const int64_t row = (int64_t)r->Hkv * r->d, n = r->piece_rows() * row * 2;
  for (int pc = 0; pc < r->pieces(); ++pc) {
    const int64_t g = r->piece_row(src, pc) * row, l = pc * r->piece_rows() * row;
    hipError_t e = hipMemcpyAsync(r->kst[slot] + l, k + g, n, hipMemcpyDeviceToDevice, r->copy);
    if (e != hipSuccess) return e;
    e = hipMemcpyAsync(r->vst[slot] + l, v + g, n, hipMemcpyDeviceToDevice, r->copy);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

mad_status ring_check(const char* fn, const mad_ring* r, std::initializer_list<const void*> ptrs, float scale) {
  const std::string f(fn);
  if (!r) return fail(MAD_ERR_INVALID, f + ": ring is NULL");
  for (const void* p : ptrs) {
    if (!p) return fail(MAD_ERR_INVALID, f + ": a tensor pointer is NULL");
    if (!al16(p)) return fail(MAD_ERR_UNSUPPORTED, f + ": tensors must be 16-byte aligned");
  }
  if (!(scale == scale)) return fail(MAD_ERR_INVALID, f + ": scale is NaN");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hipf(fn, e);
  if (dev != r->dev) return fail(MAD_ERR_INVALID, f + ": ring was created on another device");
  return MAD_OK;
}

}  // namespace

extern "C" mad_status mad_ring_create(int32_t layout, int32_t n_ranks, int32_t chunk, int32_t rank, int32_t Hq,
                                      int32_t Hkv, int32_t d, mad_ring** out) {
  clear_error();
  if (!out) return fail(MAD_ERR_INVALID, "mad_ring_create: out is NULL");
  *out = nullptr;
  if (layout != 0 && layout != 1) return fail(MAD_ERR_INVALID, "mad_ring_create: layout must be 0 or 1");
  if (n_ranks < 1 || n_ranks > MAX_PARTS)
    return fail(MAD_ERR_INVALID, "mad_ring_create: n_ranks must be in 1.." + std::to_string(MAX_PARTS));
  if (chunk <= 0 || (layout == 1 && chunk % 2)) return fail(MAD_ERR_INVALID, "mad_ring_create: bad chunk");
  if ((int64_t)chunk * n_ranks > INT32_MAX) return fail(MAD_ERR_UNSUPPORTED, "mad_ring_create: sequence too long");
  if (rank < 0 || rank >= n_ranks) return fail(MAD_ERR_INVALID, "mad_ring_create: rank out of range");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return fail(MAD_ERR_INVALID, "mad_ring_create: Hq must be a positive multiple of Hkv");
  if (d != 64 && d != 128 && d != 256)
    return fail(MAD_ERR_UNSUPPORTED, "mad_ring_create: head dim must be 64, 128 or 256");
  mad_ring* r = new mad_ring();
  r->layout = layout;
  r->N = n_ranks;
  r->C = chunk;
  r->rank = rank;
  r->Hq = Hq;
  r->Hkv = Hkv;
  r->d = d;
  hipError_t e = hipGetDevice(&r->dev);
  if (e != hipSuccess) {
    ring_free(r);
    return hipf("mad_ring_create", e);
  }
  // One plan per step with a non-empty mask, in ring order.
  for (int32_t i = 0; i < n_ranks; ++i) {
    const int32_t src = ((rank - i) % n_ranks + n_ranks) % n_ranks;
    int64_t n = 0;
    mad_status s = mad_ring_step_slices(layout, n_ranks, chunk, rank, src, nullptr, 0, &n);
    std::vector<mad_slice> sl(n > 0 ? n : 1);
    if (s == MAD_OK && n > 0) s = mad_ring_step_slices(layout, n_ranks, chunk, rank, src, sl.data(), n, &n);
    mad_plan* plan = nullptr;
    if (s == MAD_OK && n > 0) s = mad_mask_compile(sl.data(), n, chunk, chunk, &plan);
    int64_t pairs = 0;
    if (s == MAD_OK && plan) s = mad_plan_stats(plan, 0, &pairs, nullptr, nullptr, nullptr);
    if (s == MAD_OK && plan && pairs > 0) s = mad_plan_upload(plan, nullptr);
    if (s != MAD_OK) {
      if (plan) mad_plan_destroy(plan);
      ring_free(r);
      return s;
    }
    if (plan && pairs > 0) {
      r->steps.push_back({src, plan, pairs});
    } else {
      if (plan) mad_plan_destroy(plan);
      r->untouched.push_back(src);
    }
  }
  // Device buffers, one allocation.
  const int64_t S = (int64_t)r->steps.size();
  const int64_t qe = (int64_t)chunk * Hq * d;
  size_t ws = 0;  // the largest workspace any step's backward needs
  for (const auto& st : r->steps) {
    size_t w = 0;
    mad_bwd_workspace_bytes(st.plan, chunk, chunk, Hq, Hkv, d, &w);
    ws = std::max(ws, w);
  }
  size_t total = 0;
  auto take = [&](size_t b) {
    const size_t off = total;
    total += (b + 255) & ~(size_t)255;
    return off;
  };
  size_t o_k[2], o_v[2];
  for (int x = 0; x < 2; ++x) {
    o_k[x] = take(r->chunk_elems() * 2);
    o_v[x] = take(r->chunk_elems() * 2);
  }
  const size_t o_op = take((size_t)S * qe * 2), o_lp = take((size_t)S * Hq * chunk * 4);
  const size_t o_dq = take((size_t)qe * 4), o_dk = take(r->chunk_elems() * 2), o_dv = take(r->chunk_elems() * 2);
  const size_t o_ws = take(ws);
  e = hipMalloc(&r->mem, total);
  if (e != hipSuccess) {
    r->mem = nullptr;
    ring_free(r);
    return fail(MAD_ERR_NOMEM, std::string("mad_ring_create: hipMalloc: ") + hipGetErrorString(e));
  }
  char* base = (char*)r->mem;
  r->bytes = total;
  for (int x = 0; x < 2; ++x) {
    r->kst[x] = (bf16*)(base + o_k[x]);
    r->vst[x] = (bf16*)(base + o_v[x]);
  }
  r->opart = (bf16*)(base + o_op);
  r->lpart = (float*)(base + o_lp);
  r->dq_acc = (float*)(base + o_dq);
  r->dkst = (bf16*)(base + o_dk);
  r->dvst = (bf16*)(base + o_dv);
  r->ws = base + o_ws;
  r->ws_bytes = ws;
  e = hipStreamCreateWithFlags(&r->copy, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_in, hipEventDisableTiming);
  for (int x = 0; x < 2 && e == hipSuccess; ++x) {
    e = hipEventCreateWithFlags(&r->ev_copied[x], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_done[x], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    ring_free(r);
    return hipf("mad_ring_create: stream/event", e);
  }
  *out = r;
  return MAD_OK;
}

extern "C" mad_status mad_ring_info(const mad_ring* r, int32_t* n_steps, int64_t* pairs_per_head,
                                    size_t* device_bytes) {
  clear_error();
  if (!r) return fail(MAD_ERR_INVALID, "mad_ring_info: ring is NULL");
  int64_t p = 0;
  for (const auto& s : r->steps) p += s.pairs;
  if (n_steps) *n_steps = (int32_t)r->steps.size();
  if (pairs_per_head) *pairs_per_head = p;
  if (device_bytes) *device_bytes = r->bytes;
  return MAD_OK;
}

extern "C" void mad_ring_destroy(mad_ring* r) {
  if (!r) return;
  const int dev = r->dev;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != dev) (void)hipSetDevice(dev);
  (void)hipDeviceSynchronize();  // no launch of this object may still use its buffers
  ring_free(r);
  if (cur != dev && cur >= 0) (void)hipSetDevice(cur);
}

extern "C" mad_status mad_ring_fwd(mad_ring* r, const void* q, const void* k, const void* v, void* o, float* lse,
                                   float scale, hipStream_t stream) {
  clear_error();
  mad_status s = ring_check("mad_ring_fwd", r, {q, k, v, o}, scale);
  if (s != MAD_OK) return s;
  if (!lse || ((uintptr_t)lse & 3u)) return fail(MAD_ERR_INVALID, "mad_ring_fwd: lse must be a 4-byte aligned pointer");
  const int64_t qe = (int64_t)r->C * r->Hq * r->d, le = (int64_t)r->Hq * r->C;
  hipError_t e = hipEventRecord(r->ev_in, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(r->copy, r->ev_in, 0);
  if (e != hipSuccess) return hipf("mad_ring_fwd: order", e);
  MergeArgs A{};
  for (size_t i = 0; i < r->steps.size(); ++i) {
    const int slot = (int)(i & 1);
    if (i >= 2) e = hipStreamWaitEvent(r->copy, r->ev_done[slot], 0);  // step i-2 has left the slot
    if (e == hipSuccess) e = stage(r, (const bf16*)k, (const bf16*)v, r->steps[i].source, slot);
    if (e == hipSuccess) e = hipEventRecord(r->ev_copied[slot], r->copy);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, r->ev_copied[slot], 0);
    if (e != hipSuccess) return hipf("mad_ring_fwd: staging", e);
    bf16* op = r->opart + (int64_t)i * qe;
    float* lp = r->lpart + (int64_t)i * le;
    // the backward's workspace is idle during the forward and holds the
    // forward kernel's item-claim counters (each step's forward runs on
    // `stream` after the previous one)
    s = mad_attn_fwd(r->steps[i].plan, q, r->kst[slot], r->vst[slot], op, lp, r->C, r->C, r->Hq, r->Hkv, r->d,
                     nullptr, scale, r->ws, r->ws_bytes, stream);
    if (s != MAD_OK) return s;
    e = hipEventRecord(r->ev_done[slot], stream);
    if (e != hipSuccess) return hipf("mad_ring_fwd: order", e);
    A.o[i] = op;
    A.lse[i] = lp;
  }
  if (r->steps.empty()) return fail(MAD_ERR_INVALID, "mad_ring_fwd: this rank has no non-empty step");
  A.out = (bf16*)o;
  A.lse_out = lse;
  A.n = (int32_t)r->steps.size();
  A.Tq = r->C;
  A.Hq = r->Hq;
  e = launch_merge(A, r->d, stream);
  if (e != hipSuccess) return hipf("mad_ring_fwd: merge", e);
  return MAD_OK;
}

extern "C" mad_status mad_ring_bwd(mad_ring* r, const void* q, const void* k, const void* v, const void* o,
                                   const void* d_o, const float* lse, void* dq, void* dk, void* dv, float scale,
                                   hipStream_t stream) {
  clear_error();
  mad_status s = ring_check("mad_ring_bwd", r, {q, k, v, o, d_o, dq, dk, dv}, scale);
  if (s != MAD_OK) return s;
  if (!lse || ((uintptr_t)lse & 3u)) return fail(MAD_ERR_INVALID, "mad_ring_bwd: lse must be a 4-byte aligned pointer");
  if (r->steps.empty()) return fail(MAD_ERR_INVALID, "mad_ring_bwd: this rank has no non-empty step");
  const int64_t qe = (int64_t)r->C * r->Hq * r->d, row = (int64_t)r->Hkv * r->d;
  // The row vectors (-D, -LSE/scale) depend on the merged O / LSE only: once.
  s = attn_bwd_impl(r->steps[0].plan, q, r->kst[0], r->vst[0], o, d_o, lse, nullptr, r->dq_acc, r->dkst, r->dvst,
                    r->ws, r->ws_bytes, r->C, r->C, r->Hq, r->Hkv, r->d, nullptr, scale, MAD_BWD_DELTA, stream);
  if (s != MAD_OK) return s;
  hipError_t e = launch_zero(r->dq_acc, qe * 4, stream);
  for (int32_t src : r->untouched)
    for (int pc = 0; pc < r->pieces() && e == hipSuccess; ++pc) {
      const int64_t g = r->piece_row(src, pc) * row;
      e = launch_zero((bf16*)dk + g, r->piece_rows() * row * 2, stream);
      if (e == hipSuccess) e = launch_zero((bf16*)dv + g, r->piece_rows() * row * 2, stream);
    }
  if (e == hipSuccess) e = hipEventRecord(r->ev_in, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(r->copy, r->ev_in, 0);
  if (e != hipSuccess) return hipf("mad_ring_bwd: setup", e);
  for (size_t i = 0; i < r->steps.size(); ++i) {
    const int slot = (int)(i & 1);
    const int32_t src = r->steps[i].source;
    if (i >= 2) e = hipStreamWaitEvent(r->copy, r->ev_done[slot], 0);
    if (e == hipSuccess) e = stage(r, (const bf16*)k, (const bf16*)v, src, slot);
    if (e == hipSuccess) e = hipEventRecord(r->ev_copied[slot], r->copy);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, r->ev_copied[slot], 0);
    if (e != hipSuccess) return hipf("mad_ring_bwd: staging", e);
    bf16* dkd = r->layout == 0 ? (bf16*)dk + (int64_t)src * r->C * row : r->dkst;
    bf16* dvd = r->layout == 0 ? (bf16*)dv + (int64_t)src * r->C * row : r->dvst;
    s = attn_bwd_impl(r->steps[i].plan, q, r->kst[slot], r->vst[slot], o, d_o, lse, nullptr, r->dq_acc, dkd, dvd,
                      r->ws, r->ws_bytes, r->C, r->C, r->Hq, r->Hkv, r->d, nullptr, scale,
                      MAD_BWD_DKDV | MAD_BWD_DQ, stream);
    if (s != MAD_OK) return s;
    if (r->layout == 1)
      for (int pc = 0; pc < 2 && e == hipSuccess; ++pc) {
        const int64_t g = r->piece_row(src, pc) * row, l = pc * r->piece_rows() * row, n = r->piece_rows() * row * 2;
        e = hipMemcpyAsync((bf16*)dk + g, r->dkst + l, n, hipMemcpyDeviceToDevice, stream);
        if (e == hipSuccess) e = hipMemcpyAsync((bf16*)dv + g, r->dvst + l, n, hipMemcpyDeviceToDevice, stream);
      }
    if (e == hipSuccess) e = hipEventRecord(r->ev_done[slot], stream);
    if (e != hipSuccess) return hipf("mad_ring_bwd: step", e);
  }
  hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_for(qe / 8)), dim3(256), 0, stream, r->dq_acc, (bf16*)dq, qe / 8);
  e = hipGetLastError();
  if (e != hipSuccess) return hipf("mad_ring_bwd: dq", e);
  return MAD_OK;
}
