// api.hip -- C ABI entry points for attention, plan upload and error reporting.
//
// Every entry point validates all arguments before it launches or writes
// anything, returns a mad_status, and records a message for mad_last_error()
// on the calling thread.  Kernels run on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>

#include "kernel_common.hpp"

namespace mad {

static thread_local std::string g_err;

mad_status fail(mad_status s, const std::string& msg) {
  g_err = msg;
  return s;
}
void clear_error() { g_err.clear(); }

hipError_t launch_fwd(AttnParams P, int D, int n_items, hipStream_t stream);
hipError_t launch_bwd(AttnParams Pq, const AttnParams& Pkv, int D, int nq_items, int nkv_items,
                      uint32_t phases, hipStream_t stream);

namespace {

mad_status hip_fail(const char* where, hipError_t e) {
  return fail(MAD_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Strides {
  int64_t q_tok, q_head, k_tok, k_head, v_tok, v_head;
};

// Shared validation of the attention calls.
mad_status check_common(const char* fn, const mad_plan* p, const void* q, const void* k, const void* v, int32_t Tq,
                        int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d, const int64_t* strides, Strides& st) {
  const std::string f(fn);
  if (!p) return fail(MAD_ERR_INVALID, f + ": plan is NULL");
  if (Tq < 0 || Tk < 0 || Hq <= 0 || Hkv <= 0) return fail(MAD_ERR_INVALID, f + ": sizes must be Tq,Tk >= 0 and Hq,Hkv > 0");
  if (Hq % Hkv) return fail(MAD_ERR_INVALID, f + ": Hq must be a multiple of Hkv");
  if (d != 64 && d != 128 && d != 256) return fail(MAD_ERR_UNSUPPORTED, f + ": head dim must be 64, 128 or 256");
  if (p->Tq != Tq || p->Tk != Tk)
    return fail(MAD_ERR_INVALID, f + ": plan was compiled for Tq=" + std::to_string(p->Tq) + ", Tk=" +
                                     std::to_string(p->Tk));
  if (Hq % p->G) return fail(MAD_ERR_INVALID, f + ": plan mask groups must divide Hq");
  if (!p->dev_mem) return fail(MAD_ERR_INVALID, f + ": plan not uploaded (call mad_plan_upload)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev != p->dev_id) return fail(MAD_ERR_INVALID, f + ": plan was uploaded to another device");
  if (strides) {
    st = Strides{strides[0], strides[1], strides[2], strides[3], strides[4], strides[5]};
  } else {
    st = Strides{(int64_t)Hq * d, d, (int64_t)Hkv * d, d, (int64_t)Hkv * d, d};
  }
  const int64_t all[6] = {st.q_tok, st.q_head, st.k_tok, st.k_head, st.v_tok, st.v_head};
  for (int x = 0; x < 6; ++x)
    if (all[x] < 0 || all[x] % 8) return fail(MAD_ERR_UNSUPPORTED, f + ": strides must be >= 0 and multiples of 8 elements");
  if (Tq > 0 && Tk > 0 && (!q || !k || !v)) return fail(MAD_ERR_INVALID, f + ": q/k/v must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(MAD_ERR_UNSUPPORTED, f + ": q/k/v must be 16-byte aligned");
  return MAD_OK;
}

// Compute units of the current device (cached per device); 256, the MI355X
// count, when no device is visible (host-only use of the queries).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workspace bytes of the dQ kernel's item-claim counters (64 used).
constexpr size_t kQueueBytes = 256;

// Workgroups per key-tile column of the dK/dV kernel.  The kernel runs one
// workgroup per CU; when its longest column holds more than half of one CU's
// average share of the items, that column alone would set the kernel's
// length, so every column is cut into S chunks with the longest chunk at
// most that half-share (S capped at 8).  Balanced masks keep S = 1 (CAUSAL
// 32K GQA: the longest column is a quarter of the average share).
int dkdv_splits(const mad_plan* p, int32_t Hq, int32_t Hkv) {
  const TilingHost& t = p->tiling[1];
  const int R = Hq / Hkv, grp_div = Hq / p->G, nk = t.nkt;
  if (nk == 0 || t.ptr.empty()) return 1;
  int64_t total = 0, mx = 0;
  for (int g = 0; g < Hkv; ++g)
    for (int kt = 0; kt < nk; ++kt) {
      int64_t n = 0;
      for (int e = 0; e < R; ++e) {
        const int mg = (g * R + e) / grp_div;
        n += t.ptr[(size_t)mg * (nk + 1) + kt + 1] - t.ptr[(size_t)mg * (nk + 1) + kt];
      }
      total += n;
      mx = std::max(mx, n);
    }
  if (total == 0) return 1;
  const int64_t cus = device_cus();
  return (int)std::min<int64_t>(8, std::max<int64_t>(1, (mx * 2 * cus + total - 1) / total));
}

AttnParams base_params(const mad_plan* p, int which, const void* q, const void* k, const void* v, int32_t Tq,
                       int32_t Tk, int32_t Hq, int32_t Hkv, const Strides& st, float scale) {
  AttnParams P;
  std::memset(&P, 0, sizeof(P));
  P.q = (const bf16*)q;
  P.k = (const bf16*)k;
  P.v = (const bf16*)v;
  P.q_tok = st.q_tok;
  P.q_head = st.q_head;
  P.k_tok = st.k_tok;
  P.k_head = st.k_head;
  P.v_tok = st.v_tok;
  P.v_head = st.v_head;
  P.Tq = Tq;
  P.Tk = Tk;
  P.Hq = Hq;
  P.Hkv = Hkv;
  P.R = Hq / Hkv;
  P.grp_div = Hq / p->G;
  P.scale = scale;
  P.scale_log2 = scale * LOG2E;
  P.t = p->tdev[which];
  P.m = p->mdev;
  return P;
}

}  // namespace
}  // namespace mad

using namespace mad;

extern "C" const char* mad_last_error(void) { return g_err.c_str(); }

extern "C" const char* mad_version(void) { return "mask_aware_dense_amd 0.1 (gfx950)"; }

extern "C" mad_status mad_plan_upload(mad_plan* p, hipStream_t stream) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_plan_upload: plan is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("mad_plan_upload", e);
  if (p->dev_mem) {
    if (dev == p->dev_id) return MAD_OK;
    return fail(MAD_ERR_UNSUPPORTED, "mad_plan_upload: plan already uploaded to another device");
  }
  // Lay out every array in one allocation, 256-byte aligned pieces.
  struct Piece {
    const void* src;
    size_t bytes;
    size_t off;
  };
  std::vector<Piece> pieces;
  size_t total = 0;
  auto add = [&](const void* src, size_t bytes) -> size_t {
    const size_t off = total;
    pieces.push_back({src, bytes, off});
    total += (bytes + 255) & ~(size_t)255;
    return off;
  };
  size_t off_t[2][4];
  for (int w = 0; w < 2; ++w) {
    const TilingHost& t = p->tiling[w];
    off_t[w][0] = add(t.ptr.data(), t.ptr.size() * 4);
    off_t[w][1] = add(t.ent.data(), t.ent.size() * 4);
    off_t[w][2] = add(t.ent_aux.data(), t.ent_aux.size() * 4);
    off_t[w][3] = add(t.order.data(), t.order.size() * 4);
  }
  const size_t off_sl = add(p->slices.data(), p->slices.size() * sizeof(mad_slice));
  const size_t off_ts = add(p->tile_slices.data(), p->tile_slices.size() * 4);
  const size_t off_rq = add(p->row_qb.data(), p->row_qb.size() * 4);
  const size_t off_ck = add(p->col_kb.data(), p->col_kb.size() * 4);
  const size_t off_ke = add(p->k_edges.data(), p->k_edges.size() * 4);
  const size_t off_qe = add(p->q_edges.data(), p->q_edges.size() * 4);
  const size_t off_kp = add(p->keep.data(), p->keep.size() * 8);
  if (total == 0) total = 256;
  void* mem = nullptr;
  e = hipMalloc(&mem, total);
  if (e != hipSuccess) return fail(MAD_ERR_NOMEM, std::string("mad_plan_upload: hipMalloc: ") + hipGetErrorString(e));
  for (const Piece& pc : pieces) {
    if (!pc.bytes) continue;
    e = hipMemcpyAsync((char*)mem + pc.off, pc.src, pc.bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) {
      (void)hipFree(mem);
      return hip_fail("mad_plan_upload: hipMemcpyAsync", e);
    }
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return hip_fail("mad_plan_upload: hipStreamSynchronize", e);
  }
  char* base = (char*)mem;
  for (int w = 0; w < 2; ++w) {
    const TilingHost& t = p->tiling[w];
    TilingDev& d = p->tdev[w];
    d.ptr = (const int32_t*)(base + off_t[w][0]);
    d.ent = (const int32_t*)(base + off_t[w][1]);
    d.ent_aux = (const int32_t*)(base + off_t[w][2]);
    d.order = (const int32_t*)(base + off_t[w][3]);
    d.nmajor = w == 0 ? t.nqt : t.nkt;
    d.nminor = w == 0 ? t.nkt : t.nqt;
    d.BN = t.BN;
    d.uniform = t.uniform;
  }
  MaskDev& m = p->mdev;
  m.mode = p->mode;
  m.Tq = p->Tq;
  m.Tk = p->Tk;
  m.slices = (const mad_slice*)(base + off_sl);
  m.tile_slices = (const int32_t*)(base + off_ts);
  m.row_qb = (const int32_t*)(base + off_rq);
  m.col_kb = (const int32_t*)(base + off_ck);
  m.k_edges = (const int32_t*)(base + off_ke);
  m.q_edges = (const int32_t*)(base + off_qe);
  m.keep = (const uint64_t*)(base + off_kp);
  m.n_qb = p->n_qb;
  m.n_kb = p->n_kb;
  m.nw = p->nw;
  p->dev_mem = mem;
  p->dev_bytes = total;
  p->dev_id = dev;
  return MAD_OK;
}

extern "C" mad_status mad_plan_device_bytes(const mad_plan* p, size_t* bytes) {
  clear_error();
  if (!p || !bytes) return fail(MAD_ERR_INVALID, "mad_plan_device_bytes: NULL argument");
  *bytes = p->dev_mem ? p->dev_bytes : 0;
  return MAD_OK;
}

extern "C" void mad_plan_destroy(mad_plan* p) {
  if (!p) return;
  if (p->dev_mem) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p->dev_id) (void)hipSetDevice(p->dev_id);
    (void)hipFree(p->dev_mem);
    if (p->dev_tmp) (void)hipFree(p->dev_tmp);
    if (cur != p->dev_id && cur >= 0) (void)hipSetDevice(cur);
  }
  delete p;
}

extern "C" mad_status mad_attn_fwd(const mad_plan* p, const void* q, const void* k, const void* v, void* o, float* lse,
                                   int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d, const int64_t* strides,
                                   float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  Strides st;
  mad_status s = check_common("mad_attn_fwd", p, q, k, v, Tq, Tk, Hq, Hkv, d, strides, st);
  if (s != MAD_OK) return s;
  if (Tq > 0 && (!o || !lse)) return fail(MAD_ERR_INVALID, "mad_attn_fwd: o/lse must not be NULL");
  if (!aligned16(o) || ((uintptr_t)lse & 3u)) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_fwd: o must be 16-byte and lse 4-byte aligned");
  if (!(scale == scale)) return fail(MAD_ERR_INVALID, "mad_attn_fwd: scale is NaN");
  if (workspace && workspace_bytes < MAD_FWD_WORKSPACE_BYTES)
    return fail(MAD_ERR_INVALID, "mad_attn_fwd: workspace must hold " + std::to_string(MAD_FWD_WORKSPACE_BYTES) + " bytes");
  if ((uintptr_t)workspace & 255u) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_fwd: workspace must be 256-byte aligned");
  if (Tq == 0) return MAD_OK;
  AttnParams P = base_params(p, 0, q, k, v, Tq, Tk, Hq, Hkv, st, scale);
  P.o = (bf16*)o;
  P.lse = lse;
  P.queue = (int32_t*)workspace;  // item-claim counters, or NULL: one fixed item per workgroup
  const int64_t n_items = (int64_t)p->tiling[0].nqt * Hq;
  if (n_items > INT32_MAX) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_fwd: too many work items");
  hipError_t e = launch_fwd(P, d, (int)n_items, stream);
  if (e != hipSuccess) return hip_fail("mad_attn_fwd: launch", e);
  return MAD_OK;
}

extern "C" mad_status mad_bwd_workspace_bytes(const mad_plan* p, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv,
                                              int32_t d, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(MAD_ERR_INVALID, "mad_bwd_workspace_bytes: bytes is NULL");
  if (!p) return fail(MAD_ERR_INVALID, "mad_bwd_workspace_bytes: plan is NULL");
  if (Tq < 0 || Tk < 0 || Hq <= 0 || Hkv <= 0) return fail(MAD_ERR_INVALID, "mad_bwd_workspace_bytes: bad sizes");
  if (d != 64 && d != 128 && d != 256)
    return fail(MAD_ERR_UNSUPPORTED, "mad_bwd_workspace_bytes: head dim must be 64, 128 or 256");
  // -delta and -LSE/scale rows, each [Hq][Tq rounded up to 128] fp32; with
  // split dK/dV columns, fp32 dK and dV sums [Tk][Hkv][d] after them; last,
  // 256 bytes for the dQ kernel's item-claim counters
  const size_t tq_pad = ((size_t)Tq + 127) / 128 * 128;
  *bytes = (2 * (size_t)Hq * tq_pad * 4 + 255) / 256 * 256;
  if (Hq % Hkv == 0 && Hq % p->G == 0 && dkdv_splits(p, Hq, Hkv) > 1) *bytes += 2 * (size_t)Tk * Hkv * d * 4;
  *bytes += kQueueBytes;
  return MAD_OK;
}

extern "C" mad_status mad_bwd_kv_splits(const mad_plan* p, int32_t Hq, int32_t Hkv, int32_t* splits) {
  clear_error();
  if (!p || !splits) return fail(MAD_ERR_INVALID, "mad_bwd_kv_splits: NULL argument");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return fail(MAD_ERR_INVALID, "mad_bwd_kv_splits: Hq must be a positive multiple of Hkv");
  if (Hq % p->G) return fail(MAD_ERR_INVALID, "mad_bwd_kv_splits: plan mask groups must divide Hq");
  *splits = dkdv_splits(p, Hq, Hkv);
  return MAD_OK;
}

namespace mad {
// The backward with an optional fp32 dQ accumulator (dq_acc, [Tq, Hq, d]):
// when it is given, the dQ kernel adds its result there and dq is not used.
mad_status attn_bwd_impl(const mad_plan* p, const void* q, const void* k, const void* v, const void* o,
                         const void* d_o, const float* lse, void* dq, float* dq_acc, void* dk, void* dv,
                         void* workspace, size_t ws_bytes, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d,
                         const int64_t* strides, float scale, uint32_t phases, hipStream_t stream) {
  if (phases == 0 || (phases & ~(uint32_t)MAD_BWD_ALL)) return fail(MAD_ERR_INVALID, "mad_attn_bwd: bad phase set");
  Strides st;
  mad_status s = check_common("mad_attn_bwd", p, q, k, v, Tq, Tk, Hq, Hkv, d, strides, st);
  if (s != MAD_OK) return s;
  if (Tq > 0 && (!o || !d_o || !lse || (!dq && !dq_acc)))
    return fail(MAD_ERR_INVALID, "mad_attn_bwd: o/d_o/lse/dq must not be NULL");
  if ((uintptr_t)dq_acc & 15u) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd: dq accumulator must be 16-byte aligned");
  if (Tk > 0 && (!dk || !dv)) return fail(MAD_ERR_INVALID, "mad_attn_bwd: dk/dv must not be NULL");
  if (!aligned16(o) || !aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u))
    return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd: o/d_o/dq/dk/dv must be 16-byte and lse 4-byte aligned");
  size_t need = 0;
  mad_bwd_workspace_bytes(p, Tq, Tk, Hq, Hkv, d, &need);
  if (Tq > 0 && (!workspace || ws_bytes < need))
    return fail(MAD_ERR_INVALID, "mad_attn_bwd: workspace must hold " + std::to_string(need) + " bytes");
  if ((uintptr_t)workspace & 255u) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd: workspace must be 256-byte aligned");
  if (!(scale == scale)) return fail(MAD_ERR_INVALID, "mad_attn_bwd: scale is NaN");
  if (Tq == 0 && Tk == 0) return MAD_OK;
  AttnParams Pq = base_params(p, 0, q, k, v, Tq, Tk, Hq, Hkv, st, scale);
  Pq.o_in = (const bf16*)o;
  Pq.d_o = (const bf16*)d_o;
  Pq.lse_in = lse;
  Pq.Tq_pad = (int32_t)(((int64_t)Tq + 127) / 128 * 128);
  Pq.ndelta = (float*)workspace;
  Pq.nlse = (float*)workspace + (size_t)Hq * Pq.Tq_pad;
  Pq.dq = (bf16*)dq;
  Pq.dq_acc = dq_acc;
  Pq.dk = (bf16*)dk;
  Pq.dv = (bf16*)dv;
  AttnParams Pkv = Pq;
  Pkv.t = p->tdev[1];
  Pkv.kv_splits = dkdv_splits(p, Hq, Hkv);
  if (Pkv.kv_splits > 1) {
    char* acc = (char*)workspace + (2 * (size_t)Hq * Pq.Tq_pad * 4 + 255) / 256 * 256;
    Pkv.dk_acc = (float*)acc;
    Pkv.dv_acc = (float*)acc + (size_t)Tk * Hkv * d;
  }
  Pq.kv_splits = 1;
  // the dQ kernel's item-claim counters: the last kQueueBytes of the workspace
  Pq.queue = Tq > 0 ? (int32_t*)((char*)workspace + need - kQueueBytes) : nullptr;
  const int64_t nq = Tq > 0 ? (int64_t)p->tiling[0].nqt * Hq : 0;
  const int64_t nkv = Tk > 0 ? (int64_t)p->tiling[1].nkt * Hkv : 0;
  if (nq > INT32_MAX || nkv > INT32_MAX) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd: too many work items");
  hipError_t e = launch_bwd(Pq, Pkv, d, (int)nq, (int)nkv, phases, stream);
  if (e != hipSuccess) return hip_fail("mad_attn_bwd: launch", e);
  return MAD_OK;
}
}  // namespace mad

extern "C" mad_status mad_attn_bwd_phases(const mad_plan* p, const void* q, const void* k, const void* v,
                                          const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                                          void* dv, void* workspace, size_t ws_bytes, int32_t Tq, int32_t Tk,
                                          int32_t Hq, int32_t Hkv, int32_t d, const int64_t* strides, float scale,
                                          uint32_t phases, hipStream_t stream) {
  clear_error();
  return attn_bwd_impl(p, q, k, v, o, d_o, lse, dq, nullptr, dk, dv, workspace, ws_bytes, Tq, Tk, Hq, Hkv, d, strides,
                       scale, phases, stream);
}

extern "C" mad_status mad_attn_bwd(const mad_plan* p, const void* q, const void* k, const void* v, const void* o,
                                   const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                   size_t ws_bytes, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d,
                                   const int64_t* strides, float scale, hipStream_t stream) {
  return mad_attn_bwd_phases(p, q, k, v, o, d_o, lse, dq, dk, dv, workspace, ws_bytes, Tq, Tk, Hq, Hkv, d, strides,
                             scale, MAD_BWD_ALL, stream);
}

// ---------------------------------------------------------------------------
// The backward without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts that
// forbid allocation in the step).  Its workspace is this file-scope device
// array: each GPU the library runs on holds one copy, at its own address, from
// the code object's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the device
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept in scratch_dev.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MAD_STATIC_WORKSPACE_BYTES];

namespace mad {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device (null: not looked up yet)

mad_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd_static: device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(MAD_ERR_HIP, std::string("mad_attn_bwd_static: hipGetSymbolAddress: ") + hipGetErrorString(e));
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MAD_OK;
}
}  // namespace
}  // namespace mad

extern "C" mad_status mad_attn_bwd_static(const mad_plan* p, const void* q, const void* k, const void* v,
                                          const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                                          void* dv, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d,
                                          const int64_t* strides, float scale, hipStream_t stream) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_attn_bwd_static: plan is NULL");
  if (!p->dev_mem) return fail(MAD_ERR_INVALID, "mad_attn_bwd_static: plan not uploaded (call mad_plan_upload)");
  size_t need = 0;
  mad_status s = mad_bwd_workspace_bytes(p, Tq, Tk, Hq, Hkv, d, &need);
  if (s != MAD_OK) return s;
  if (need > MAD_STATIC_WORKSPACE_BYTES)
    return fail(MAD_ERR_UNSUPPORTED, "mad_attn_bwd_static: this call needs " + std::to_string(need) +
                                         " bytes of workspace, more than the " +
                                         std::to_string((size_t)MAD_STATIC_WORKSPACE_BYTES) +
                                         "-byte static workspace; use mad_attn_bwd with a caller workspace");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("mad_attn_bwd_static", e);
  void* ws = nullptr;
  s = scratch_address(dev, &ws);
  if (s != MAD_OK) return s;
  return attn_bwd_impl(p, q, k, v, o, d_o, lse, dq, nullptr, dk, dv, ws, MAD_STATIC_WORKSPACE_BYTES, Tq, Tk, Hq, Hkv,
                       d, strides, scale, MAD_BWD_ALL, stream);
}
