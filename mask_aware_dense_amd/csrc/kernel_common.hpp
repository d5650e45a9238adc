// kernel_common.hpp -- device helpers shared by the attention kernels (gfx950).
//
// Matrix products use the CDNA4 bf16 MFMA v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation.  Its lane layout (wave64, l = lane, h = l / 32):
//   A (32 x 16): lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32): lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32): lane l, register r holds C[8(r/4) + 4h + (r%4)][l % 32]
// The transposed LDS read ds_read_b64_tr_b16 lets 16-lane groups fetch an
// operand whose contraction index runs along LDS rows: when lane 16G + i
// points at row k0 + i/4, column n0 + 16(G%2) + 4(i%4), lane l receives the
// four elements X[k0 + e][n0 + l % 32], e = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace mad {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Everything a kernel needs about one attention call.
struct AttnParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const bf16* o_in;   // backward: forward output
  const bf16* d_o;    // backward: upstream gradient (packed [Tq, Hq, D])
  const float* lse_in;
  float* ndelta;      // backward: -rowsum(dO * O), [Hq, Tq_pad]
  float* nlse;        // backward: -LSE / scale, -inf for empty / padded rows, [Hq, Tq_pad]
  int32_t Tq_pad;     // Tq rounded up to a multiple of 128
  bf16* dq;
  float* dq_acc;      // backward: if set, dQ is added into this fp32 [Tq, Hq, D] buffer instead of written to dq
  bf16* dk;
  bf16* dv;
  float* dk_acc;      // dK/dV kernel with kv_splits > 1: fp32 [Tk, Hkv, D] sums of the column chunks
  float* dv_acc;
  int32_t kv_splits;  // dK/dV kernel: workgroups per key-tile column (1: each column in one workgroup)
  int32_t* queue;     // forward / dQ kernels: item-claim counters (claim_item, 64 bytes), zero at launch; or NULL
  int32_t n_items;    // forward / dQ kernels: work items of the launch
  int64_t q_tok, q_head, k_tok, k_head, v_tok, v_head;
  int32_t Tq, Tk, Hq, Hkv;
  int32_t R;        // Hq / Hkv
  int32_t grp_div;  // Hq / n_groups (mask group of head h = h / grp_div)
  float scale;      // softmax scale
  float scale_log2; // scale * log2(e)
  TilingDev t;
  MaskDev m;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Two transposed 4-element reads stacked into one 8-element MFMA operand.
// row0 / row1 address the LDS rows of elements 0..3 and 4..7.
__device__ __forceinline__ bf16x8 ld_tr8(const bf16* row0, const bf16* row1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(row0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(row1));
  u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  u32x4 r = {ua[0], ua[1], ub[0], ub[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// Lane offsets of the transposed read inside a 16-lane group: row within
// the 4-row group and column within the 32-column block.
__device__ __forceinline__ int tr_row(int lane) { return (lane & 15) >> 2; }
__device__ __forceinline__ int tr_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

// Eight fp32 values to an 8 x bf16 MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)s[base + e];
  return r;
}

// max / sum of x over lanes l and l ^ 32 (the two half-waves hold the same
// query row in the transposed score layout).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swap bits 2 and 3 of a row index inside a 32-row block.  K (and V) tiles
// are stored in LDS with row p holding key swap23(p): the score MFMA then
// leaves keys 16(r/8) + 8h + (r%8) in register r of lane half h, so each
// half-wave holds 8 consecutive keys per 8 registers -- the layout of the
// next MFMA's contraction operand.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS tiles are [64 rows][D] bf16 images with padded rows.  The row stride
// RS (elements) depends on how a tile is read, because the two read kinds
// want different bank spreads on the 64-bank LDS (measured with the
// SQ_LDS_BANK_CONFLICT counter):
//   ROWS  - 16-byte row reads (MFMA operand rows): 8 lanes per pass read the
//           same column of 8 consecutive rows; conflict-free when the stride
//           is 4 mod 8 dwords (528 B for D=256, 272 B for D=128, 144 B for
//           D=64).
//   TR    - transposed reads (ds_read_b64_tr_b16): 32 lanes per pass read
//           64 bytes of each of 4 consecutive rows; conflict-free when the
//           stride is 16 mod 32 dwords (576 B for D=256, 320 B for D=128,
//           192 B for D=64).
//   MIXED - both; 560 B (D=256), 304 B (D=128), 144 B (D=64) keep row reads
//           conflict-free.
//           A pure-read probe shows two-way conflicts on transposed reads at
//           this stride, but in the kernels' access order (a wave's 32 lanes
//           reading 4 rows of one 64-byte column block) the counter stays at
//           zero once the direct-load writes are taken away.
//   SWZ   - both, D=128 only, unpadded 256-byte rows: storage row p keeps
//           16-byte chunk c at chunk c ^ swz(p), swz(p) = (p%4)*4 + (p/4)%4.
//           A row-read pass (16 rows, one chunk) then meets 16 distinct
//           chunks, and a transposed pass (4 rows x one aligned 64-byte
//           window) meets 4 distinct windows: both are conflict-free, and the
//           direct loads carry no pad bytes (they cost LDS time per byte
//           written).  Addresses are affine only per chunk, so readers keep a
//           few per-lane offsets (SwzRows, SwzTr).
// Padding keeps every address affine in the row and column, so operand reads
// use immediate offsets from one per-lane base.
enum TileKind { TILE_ROWS = 0, TILE_TR = 1, TILE_MIXED = 2, TILE_SWZ = 3 };
template <int D, int KIND>
constexpr int tile_rs() {
  static_assert(D == 64 || D == 128 || D == 256, "head dim 64, 128 or 256");
  static_assert(KIND != TILE_SWZ || D == 128, "the swizzled tile is for D = 128");
  return D == 256   ? (KIND == TILE_ROWS ? 264 : KIND == TILE_TR ? 288 : 280)
         : D == 128 ? (KIND == TILE_ROWS ? 136 : KIND == TILE_TR ? 160 : KIND == TILE_SWZ ? 128 : 152)
                    : (KIND == TILE_TR ? 96 : 72);
}
// Chunk permutation of storage row p of a SWZ tile.
__device__ __forceinline__ int swz_row(int p) { return ((p & 3) << 2) | ((p >> 2) & 3); }

// Byte offsets of one lane's 16-byte row reads in a SWZ tile: storage row
// li (+ multiples of 16 rows, added by the caller), elements 16 ks + 8 hh.
struct SwzRows {
  uint32_t o[8];
  __device__ __forceinline__ void init(int li, int hh) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) o[ks] = (uint32_t)(li * 256 + 16 * ((2 * ks + hh) ^ swz_row(li)));
  }
};
// Byte offsets of one lane's transposed reads (ld_tr8) in a SWZ tile: rows
// r = 4 hh + tr_row(lane) and r + 8 (+ multiples of 16 rows), columns
// 32 db + tr_col(lane).
struct SwzTr {
  uint32_t o0[4], o1[4];
  __device__ __forceinline__ void init(int lane) {
    const int hh = lane >> 5, r = 4 * hh + tr_row(lane);
    const int ch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1), half = 8 * (lane & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      o0[db] = (uint32_t)(r * 256 + 16 * ((4 * db + ch) ^ swz_row(r)) + half);
      o1[db] = (uint32_t)((r + 8) * 256 + 16 * ((4 * db + ch) ^ swz_row(r + 8)) + half);
    }
  }
};
template <int D, int KIND>
constexpr int tile_elems() { return 64 * tile_rs<D, KIND>(); }

// Direct global -> LDS copies of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane l of the wave writes LDS bytes
// [lds + 16 l, +16); the LDS base goes in M0 and must be wave-uniform.
//
// They are issued from inline assembly on purpose.  The compiler treats a
// direct LDS load it issued itself as a pending LDS write that may alias
// every later LDS read, and so waits for all outstanding vector-memory
// operations (vmcnt 0) before the first LDS read that follows -- which
// turns a prefetch of the next tile into a serial load.  Here the kernels
// own that ordering: they wait for a buffer's loads explicitly
// (wait_vmem / wait_vmem_le) and then pass a workgroup barrier before any
// wave reads it.  M0 is saved and restored around the copy.
// The LDS address and the source base are wave-uniform by contract; the
// readfirstlane only tells the compiler so (it folds away for values already
// in scalar registers).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// Source = base (wave-uniform) + voff (per lane, bytes); destination = LDS
// byte address lds (wave-uniform).
__device__ __forceinline__ void g2lds16(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
// Source = per-lane 64-bit address.
__device__ __forceinline__ void g2lds16(const void* g, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
// Wait until this wave's outstanding vector-memory operations (including
// direct LDS loads) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of them are outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Scalar load of a wave-uniform read-only value (tile lists, plan tables):
// through the constant address space the load goes to the scalar unit
// instead of a vector load plus readfirstlane, and it does not share the
// vector-memory counter with the direct LDS loads in flight.
template <typename T>
__device__ __forceinline__ T sld(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Storage row p of a tile holds tensor row tile_row(p): p itself, or swap23
// within 32-row blocks for tiles read as the score MFMA's A operand.
__device__ __forceinline__ int tile_row(int p, bool perm) { return perm ? ((p & 32) | swap23(p & 31)) : p; }

// Direct loads of a 64-row tile.  A direct load writes 64 consecutive
// 16-byte slots of LDS per wave instruction, so the padded tile image
// (RS / 8 slots per row, 64 rows) takes RS / 8 instructions; slot s holds
// chunk s % (RS/8) of storage row s / (RS/8), and the pad slots of a row
// repeat its first chunk (never read).  Storage row p receives tensor row
// r0 + tile_row(p).  The NW waves of a workgroup take instructions
// w, w + NW, ...  Each lane's source offset within a tile is the same for
// every tile, so it is computed once (init) and a tile then costs one
// wave-uniform base per instruction (issue).  A tile reaching past row T
// (the ragged last tile) clamps its rows to T - 1; callers mask those rows,
// so their values only need to be finite.
template <int D, int KIND, int NW, bool PERM>
struct TileLoader {
  static constexpr int SPR = tile_rs<D, KIND>() / 8, CPR = D / 8, NI = (SPR + NW - 1) / NW;
  // Byte offset of this lane's source chunk from the tile's first row, per
  // instruction: kept in registers for up to 9 instructions per wave, else
  // (two waves loading 512-byte rows) recomputed at each issue, where 18
  // registers per tile would not fit beside the kernel's operands.
  static constexpr bool KEEP = NI <= 9;
  uint32_t off[KEEP ? NI : 1];

  // Tensor chunk held by storage slot (row p, chunk c); pad slots repeat chunk 0.
  static __device__ __forceinline__ int src_chunk(int p, int c) {
    return c >= CPR ? 0 : (KIND == TILE_SWZ ? c ^ swz_row(p) : c);
  }

  static __device__ __forceinline__ uint32_t offset(int i, int64_t tok, int w, int lane) {
    const int s = (i * NW + w) * 64 + lane;
    const int p = s / SPR, c = s % SPR;
    return (uint32_t)(((int64_t)tile_row(p, PERM) * tok + src_chunk(p, c) * 8) * 2);
  }
  __device__ __forceinline__ void init(int64_t tok, int w, int lane) {
    if constexpr (KEEP) {
#pragma unroll
      for (int i = 0; i < NI; ++i) off[i] = offset(i, tok, w, lane);
    }
  }
  // lds: LDS byte address of the tile image; g: the tensor's head; tok: its
  // token stride (elements); w: the wave index, wave-uniform (only the last
  // round of instructions may leave some waves idle, and that test is scalar).
  __device__ __forceinline__ void issue(uint32_t lds, const bf16* g, int64_t tok, int r0, int T, int w,
                                        int lane) const {
    if (r0 + 64 <= T) {
      const char* base = reinterpret_cast<const char*>(g + (int64_t)r0 * tok);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ii = i * NW + w;
        if ((i + 1) * NW <= SPR || ii < SPR) {
          if constexpr (KEEP) g2lds16(base, off[i], lds + ii * 1024);
          else {
            int ln = lane;
            asm volatile("" : "+v"(ln));  // recomputed here, not hoisted out of the caller's loop
            g2lds16(base, offset(i, tok, w, ln), lds + ii * 1024);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ii = i * NW + w;
        if ((i + 1) * NW <= SPR || ii < SPR) {
          const int s = ii * 64 + lane;
          const int p = s / SPR, c = s % SPR;
          const int row = min(r0 + tile_row(p, PERM), T - 1);
          g2lds16(g + (int64_t)row * tok + src_chunk(p, c) * 8, lds + ii * 1024);
        }
      }
    }
  }
};

// Work-item claim of the forward and dQ kernels.  Items are numbered as in a
// grid of one workgroup per item, where the hardware runs workgroup b on XCD
// b % 8; queue x holds the items b < n with b % 8 == x, in increasing
// (longest-first) order, so that each XCD keeps the items (and the L2
// sharing) it would have had.  A workgroup takes the next item from the front
// of its home queue (its own XCD's, blockIdx.x % 8) and, once that is empty,
// from the back of the other queues in turn: their shortest items.  The XCDs
// finish identical shares of work at times that differ by 3-7% (measured per
// workgroup on the real-time clock), so with a fixed share per XCD the faster
// ones sit idle at the end; with the queues and a grid larger than the item
// count (claim_grid) they take over the slower ones' last items: dQ 20.8 ->
// 20.3 ms at CAUSAL 32K GQA 64:8.  (The dK/dV kernel gained nothing from
// either end; its items, whole key-tile columns, are long.)  Each queue is
// one 64-bit counter, front count low and back count high; a claim succeeds
// while front + back < the queue's length, so each item goes out once.
// Called by one lane; the caller broadcasts the result.  Returns the item, or
// -1 when every queue is empty.
__device__ __forceinline__ int claim_item(int32_t* queue, int n) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(queue);
  const int home = (int)(blockIdx.x & 7u);
  for (int k = 0; k < 8; ++k) {
    const int x = (home + k) & 7;
    const int len = (n - x + 7) >> 3;  // items x + 8p < n
    if (len <= 0) continue;
    if (k == 0) {  // own queue: from the front (longest first)
      const unsigned long long old = atomicAdd(q + x, 1ull);
      const int f = (int)(uint32_t)old, b = (int)(old >> 32);
      if (f + b < len) return x + 8 * f;
    } else {       // another XCD's: from the back (its shortest items); read first, so that empty ones cost no atomic
      const unsigned long long cur = __hip_atomic_load(q + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)(uint32_t)cur + (int)(cur >> 32) >= len) continue;
      const unsigned long long old = atomicAdd(q + x, 1ull << 32);
      const int f = (int)(uint32_t)old, b = (int)(old >> 32);
      if (f + b < len) return x + 8 * (len - 1 - b);
    }
  }
  return -1;
}

// Workgroups of a launch whose n items are claimed (claim_item): one per item
// plus an eighth more, so that an XCD running up to 12.5% faster than its
// share finds workgroups to take over the slower XCDs' last items; the
// workgroups left over find every queue empty and exit at once.
// (Clamped to the int range: any grid of at least n workgroups still runs
// every item.)
inline int claim_grid(int n) {
  const int64_t g = (int64_t)n + n / 8 + 8;
  return g > INT32_MAX ? INT32_MAX : (int)g;
}

// A kernel's item-claim counters (64 bytes) start at zero (a kernel rather than a
// memset, so that the launches can be captured in a graph).  Static: each
// source file that launches it has its own copy.
static __global__ __launch_bounds__(64) void queue_reset_kernel(int32_t* q) {
  if (threadIdx.x < 16) q[threadIdx.x] = 0;  // 8 queues x (front, back)
}

// Block index remap so that 8 consecutive logical work items (the query
// heads of one GQA group at one tile) land on the same XCD: workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int full = n - n % 64;
  if (b >= full) return b;
  const int loc = b & 63;
  return (b - loc) + (loc & 7) * 8 + (loc >> 3);
}

__device__ __forceinline__ uint32_t range_bits(int a, int b) {
  a = max(a, 0);
  b = min(b, 32);
  if (a >= b) return 0u;
  const uint32_t hi = (b == 32) ? 0xffffffffu : ((1u << b) - 1u);
  return hi & ~((1u << a) - 1u);
}

// Allowed keys of query row i among keys [key0, key0 + 32) of a visited tile,
// as a bitmask (bit j <-> key key0 + j).  FULL tiles allow every in-range
// key; PARTIAL tiles evaluate the mask source: the tile's slice list (SLICES)
// or the block keep bitmap (BLOCKS).  Keys >= Tk and rows >= Tq are never
// allowed.  [row_lo, row_hi] is the wave-uniform row range of the calling
// wave (it contains i): the query / key blocks it meets, their edges and
// their keep bits are the same for every lane, so they are read with scalar
// loads and each lane only compares its row against the block edges.
__device__ __forceinline__ uint32_t keymask32(const MaskDev& m, int32_t aux, int32_t grp, bool partial, int i,
                                              int key0, int row_lo, int row_hi) {
  uint32_t bits;
  if (!partial) {
    bits = 0xffffffffu;
  } else if (m.mode == MODE_SLICES) {
    bits = 0u;
    const int32_t* lst = m.tile_slices + aux;
    const int n = sld(lst);
    for (int x = 0; x < n; ++x) {
      const int32_t* sp = &m.slices[sld(lst + 1 + x)].q0;  // q0 q1 k0 k1 type window
      const int q0 = sld(sp), q1 = sld(sp + 1), k0 = sld(sp + 2), k1 = sld(sp + 3);
      const int type = sld(sp + 4), window = sld(sp + 5);
      if (i < q0 || i >= q1) continue;
      int lo = k0, hi = k1;
      if (type == MAD_SLICE_CAUSAL) {
        const int off = i - q0;
        hi = min(hi, k0 + off + 1);
        if (window > 0) lo = max(lo, k0 + off - window + 1);
      }
      bits |= range_bits(lo - key0, hi - key0);
    }
  } else {
    bits = 0u;
    const int kend = min(key0 + 32, m.Tk) - 1, rhi = min(row_hi, m.Tq - 1);
    if (key0 <= kend && row_lo <= rhi) {
      const int qa = sld(m.row_qb + row_lo), qz = sld(m.row_qb + rhi);
      const int ka = sld(m.col_kb + key0), kz = sld(m.col_kb + kend);
      if (qz - qa <= 1 && kz - ka <= 1) {
        // At most two query blocks and two key blocks (always, for blocks of
        // 32 or more): every keep word and edge is loaded in one batch.
        const uint64_t* ra = m.keep + ((size_t)grp * m.n_qb + qa) * m.nw;
        const uint64_t* rz = m.keep + ((size_t)grp * m.n_qb + qz) * m.nw;
        const uint64_t waa = sld(ra + (ka >> 6)), waz = sld(ra + (kz >> 6));
        const uint64_t wza = sld(rz + (ka >> 6)), wzz = sld(rz + (kz >> 6));
        const int e0 = sld(m.k_edges + ka), e1 = sld(m.k_edges + ka + 1), e2 = sld(m.k_edges + kz + 1);
        const int qsplit = sld(m.q_edges + qa + 1);  // first row of block qa + 1
        const bool in_a = i < qsplit;                 // this lane's row is in block qa (else in qz)
        const uint64_t w0 = in_a ? waa : wza, w1 = in_a ? waz : wzz;
        if ((w0 >> (ka & 63)) & 1ull) bits |= range_bits(e0 - key0, e1 - key0);
        if (kz > ka && ((w1 >> (kz & 63)) & 1ull)) bits |= range_bits(e1 - key0, e2 - key0);
      } else
      for (int qb = qa; qb <= qz; ++qb) {
        const uint64_t* krow = m.keep + ((size_t)grp * m.n_qb + qb) * m.nw;
        uint32_t kbits = 0u;  // kept keys of query block qb in this 32-key range
        for (int kb = ka; kb <= kz; ++kb)
          if ((sld(krow + (kb >> 6)) >> (kb & 63)) & 1ull)
            kbits |= range_bits(sld(m.k_edges + kb) - key0, sld(m.k_edges + kb + 1) - key0);
        if (i >= sld(m.q_edges + qb) && i < sld(m.q_edges + qb + 1)) bits = kbits;
      }
    }
  }
  const int nvalid = m.Tk - key0;
  if (nvalid < 32) bits &= (nvalid <= 0) ? 0u : ((1u << nvalid) - 1u);
  if (i >= m.Tq) bits = 0u;
  return bits;
}

__device__ __forceinline__ uint64_t range_bits64(int a, int b) {
  a = max(a, 0);
  b = min(b, 64);
  if (a >= b) return 0ull;
  const uint64_t hi = (b == 64) ? ~0ull : ((1ull << b) - 1ull);
  return hi & ~((1ull << a) - 1ull);
}

// Block-sparse mask of a kernel whose lanes keep their query row for the
// whole workgroup (the forward): keys [key0, key0 + 64) that row i may see,
// the same predicate as keymask32 in MODE_BLOCKS.  krow = the keep bitmap
// row of row i's query block in the mask group (any valid row when
// i >= Tq), looked up once per workgroup; only the key blocks are walked,
// four at a time with their loads issued together (edges as scalar loads,
// the lane's keep words as vector loads), instead of keymask32's scalar
// walk over every (query block, key block) pair of the wave's rows.
__device__ __forceinline__ uint64_t keymask64_blocks(const MaskDev& m, const uint64_t* krow, int i, int key0) {
  const int kend = min(key0 + 64, m.Tk) - 1;
  uint64_t bits = 0ull;
  if (i >= m.Tq || key0 > kend) return 0ull;
  const int ka = sld(m.col_kb + key0), kz = sld(m.col_kb + kend);
  // 64 keys span at most 64 key blocks, so their keep bits lie in at most
  // two consecutive words of the row.
  const uint64_t w0 = krow[ka >> 6], w1 = krow[kz >> 6];
  for (int k0 = ka; k0 <= kz; k0 += 4) {
    int e[5];
#pragma unroll
    for (int x = 0; x < 5; ++x) e[x] = sld(m.k_edges + min(k0 + x, m.n_kb));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int kb = k0 + x;
      const uint64_t wd = ((kb >> 6) == (ka >> 6)) ? w0 : w1;
      if (kb <= kz && ((wd >> (kb & 63)) & 1ull)) bits |= range_bits64(e[x] - key0, e[x + 1] - key0);
    }
  }
  return bits;
}
// Allowed query rows among [row0, row0 + 64) for key j of a visited PARTIAL
// tile of the dK/dV tiling, as a bitmask (bit r <-> row row0 + r): the same
// predicate as keymask32, read along the key's column.  Rows >= Tq and keys
// >= Tk are never allowed.  [key_lo, key_hi] is the wave-uniform key range
// of the calling wave (it contains j); as in keymask32 the block structure
// is read with scalar loads.
__device__ __forceinline__ uint64_t rowmask64(const MaskDev& m, int32_t aux, int32_t grp, int j, int row0,
                                              int key_lo, int key_hi) {
  uint64_t bits = 0ull;
  if (j < m.Tk) {
    if (m.mode == MODE_SLICES) {
      const int32_t* lst = m.tile_slices + aux;
      const int n = sld(lst);
      for (int x = 0; x < n; ++x) {
        const int32_t* sp = &m.slices[sld(lst + 1 + x)].q0;  // q0 q1 k0 k1 type window
        const int q0 = sld(sp), q1 = sld(sp + 1), k0 = sld(sp + 2), k1 = sld(sp + 3);
        const int type = sld(sp + 4), window = sld(sp + 5);
        if (j < k0 || j >= k1) continue;
        int lo = q0, hi = q1;
        if (type == MAD_SLICE_CAUSAL) {
          const int off = j - k0;  // row i is allowed from i - q0 = off on ...
          lo = max(lo, q0 + off);
          if (window > 0) hi = min(hi, q0 + off + window);  // ... until i - q0 - off reaches the window
        }
        bits |= range_bits64(lo - row0, hi - row0);
      }
    } else {
      const int rlast = min(row0 + 63, m.Tq - 1), khi = min(key_hi, m.Tk - 1);
      if (row0 <= rlast && key_lo <= khi) {
        const int qa = sld(m.row_qb + row0), qz = sld(m.row_qb + rlast);
        const int ka = sld(m.col_kb + key_lo), kz = sld(m.col_kb + khi);
        for (int kb = ka; kb <= kz; ++kb) {
          uint64_t rbits = 0ull;  // rows of the query blocks that keep key block kb
          for (int qb = qa; qb <= qz; ++qb) {
            const uint64_t* krow = m.keep + ((size_t)grp * m.n_qb + qb) * m.nw;
            if ((sld(krow + (kb >> 6)) >> (kb & 63)) & 1ull)
              rbits |= range_bits64(sld(m.q_edges + qb) - row0, sld(m.q_edges + qb + 1) - row0);
          }
          if (j >= sld(m.k_edges + kb) && j < sld(m.k_edges + kb + 1)) bits = rbits;
        }
      }
    }
  }
  const int nvalid = m.Tq - row0;
  if (nvalid < 64) bits &= (nvalid <= 0) ? 0ull : ((1ull << nvalid) - 1ull);
  return bits;
}

}  // namespace mad
