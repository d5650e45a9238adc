// plan.hpp -- host-side compiled mask ("plan") and the device view handed to kernels.
//
// A plan describes one mask over a Tq x Tk attention matrix, compiled for the
// two kernel tilings of this library:
//   tiling 0 (forward and dQ kernels): BM0 query rows x BN0 keys, visited as
//            per-query-tile lists of key tiles (CSR);
//   tiling 1 (dK/dV kernel):           BM1 query rows x BN1 keys (BN1_FINE
//            for block-sparse masks of smaller key blocks), visited as
//            per-key-tile lists of query tiles (CSC).
// Every tile is EMPTY (never visited), FULL (no mask arithmetic) or PARTIAL
// (per-element mask), judged on its in-range elements only.  The O(#tiles)
// description follows from LongCA-bench's observation that a dense O(S^2)
// block mask dominates memory for long sequences (appendix A.3
// FlexAttention, appendix A.5.2).
//
// Two mask sources:
//   SLICES - a union of (q_range, k_range, full | causal[, window]) slices,
//            the unified mask format; a PARTIAL tile carries the list of
//            slices that touch it.
//   BLOCKS - a block-sparse keep bitmap per mask group over query / key
//            block edges (appendix A.2); a PARTIAL tile is evaluated from
//            the bitmap.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mad.h"

namespace mad {

// Tile shapes of the two tilings; the kernels are instantiated for exactly
// these.
constexpr int BM0 = 128, BN0 = 64;   // forward / dQ
constexpr int BM1 = 64, BN1 = 128;   // dK / dV
// dK / dV key tile of block-sparse plans whose interior key-block edges are
// not all multiples of 128 (64-token blocks, variable block sizes): a
// 128-key tile would keep only part of its keys in most visited tiles and
// leave waves without work (with 64-token blocks, one of its two blocks);
// the 64-key tile's workgroup has two waves, and two workgroups share a CU.
constexpr int BN1_FINE = 64;
// The dK / dV key-tile width for a block-sparse plan with these key edges.
inline int dkdv_tile_keys(const int32_t* k_edges, int32_t n_kb) {
  bool all128 = true;
  for (int32_t b = 1; b < n_kb; ++b) all128 &= k_edges[b] % 128 == 0;  // interior edges (the last one is Tk)
  return (n_kb > 1 && !all128) ? BN1_FINE : BN1;
}

enum MaskMode : int32_t { MODE_SLICES = 0, MODE_BLOCKS = 1 };
enum TileClass : uint8_t { CLS_EMPTY = 0, CLS_FULL = 1, CLS_PARTIAL = 2 };

// Entry of a visit list: the minor tile index in bits 0..30, bit 31 set for
// PARTIAL tiles.
constexpr uint32_t ENT_PARTIAL = 0x80000000u;

struct TilingHost {
  int BM = 0, BN = 0, nqt = 0, nkt = 0;
  // per group, row-major [nqt][nkt] class map
  std::vector<std::vector<uint8_t>> cls;
  // per group, SLICES mode: offset into tile_slices for PARTIAL tiles, -1 otherwise
  std::vector<std::vector<int32_t>> aux;
  // visit lists in the kernel's direction (CSR for tiling 0, CSC for tiling 1),
  // concatenated over groups: ptr has G * (nmajor + 1) entries (absolute offsets)
  std::vector<int32_t> ptr, ent, ent_aux;
  // longest-first order of the major tiles (work summed over groups)
  std::vector<int32_t> order;
  int64_t n_class[3] = {0, 0, 0};
  // every major tile's list (in every group) has the same length: the
  // tiles carry even work, whatever their order
  bool uniform = false;
};

// Device view of one tiling, passed to kernels by value.
struct TilingDev {
  const int32_t* ptr;      // [G][nmajor + 1]
  const int32_t* ent;      // visit-list entries
  const int32_t* ent_aux;  // SLICES: per entry offset into tile_slices (or -1)
  const int32_t* order;    // [nmajor] longest-first major tile order
  int32_t nmajor, nminor;
  int32_t BN;              // key-tile width (tiling 1: BN1 or BN1_FINE)
  int32_t uniform;         // every list has the same length (even work per tile)
};

// Device view of the mask source, passed to kernels by value.
struct MaskDev {
  int32_t mode;
  int32_t Tq, Tk;
  // SLICES
  const mad_slice* slices;
  const int32_t* tile_slices;  // per PARTIAL tile: count, then slice indices
  // BLOCKS
  const int32_t* row_qb;       // [Tq] query block of each row
  const int32_t* col_kb;       // [Tk] key block of each key
  const int32_t* k_edges;      // [n_kb + 1]
  const int32_t* q_edges;      // [n_qb + 1]
  const uint64_t* keep;        // [G][n_qb][nw]
  int32_t n_qb, n_kb, nw;
};

}  // namespace mad

struct mad_plan {
  int32_t Tq = 0, Tk = 0, G = 1;
  int32_t mode = mad::MODE_SLICES;
  std::vector<mad_slice> slices;
  std::vector<int32_t> tile_slices;
  std::vector<int32_t> q_edges, k_edges, row_qb, col_kb;
  std::vector<uint64_t> keep;
  int32_t n_qb = 0, n_kb = 0, nw = 0;
  mad::TilingHost tiling[2];
  std::vector<int64_t> pairs;  // per group
  // device copy (one allocation) and views into it
  void* dev_mem = nullptr;
  int dev_id = -1;
  size_t dev_bytes = 0;
  // plans compiled on the GPU (mad_sparse_plan_device): the builder's scratch,
  // freed with the plan, and no host copy of the tile classes or list entries
  // (host ptr arrays, class counts and pairs are kept)
  void* dev_tmp = nullptr;
  bool on_device = false;
  mad::TilingDev tdev[2] = {};
  mad::MaskDev mdev = {};
};

namespace mad {
// Thread-local error message helpers (api.hip).
mad_status fail(mad_status s, const std::string& msg);
void clear_error();
// Host compilation (mask_host.cpp).
mad_status compile_slices(mad_plan* p);
mad_status compile_blocks(mad_plan* p);
}  // namespace mad
