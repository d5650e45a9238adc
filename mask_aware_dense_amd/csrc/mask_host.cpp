// mask_host.cpp -- host side of the mask path: static patterns to slices,
// ring-step slices, block top-k, and the mask compiler (tile classes and
// visit lists).  Pure C++; no HIP calls.
//
// Pattern definitions follow LongCA-bench section 2.1.1 ("Input mask
// patterns") and the notes' key design 1, with the parameters of the
// benchmark's workloads (sliding window 4K, Prefix LM 25%, one question seen
// by 4 answers, 256 global tokens plus a 2K window, causal blockwise 2K,
// Block Causal Document 1024 from appendix A.4.1).  Readings where the pages
// are silent: a sliding window of W keys includes the key itself; the
// prefix is bidirectional; answers split the rest equally and the last one
// takes the remainder; Block Causal Document blocks start at each document's
// first token; the sixth heterogeneous mask is Prefix LM per document with a
// prefix of floor(L/4).
#include <algorithm>
#include <cstring>
#include <numeric>
#include <thread>

#include "plan.hpp"

namespace mad {
namespace {

struct SliceSink {
  mad_slice* out;
  int64_t cap;
  int64_t n = 0;
  void add(int32_t q0, int32_t q1, int32_t k0, int32_t k1, int32_t type, int32_t window = 0) {
    if (q0 >= q1 || k0 >= k1) return;  // empty slices are dropped
    if (out && n < cap) out[n] = mad_slice{q0, q1, k0, k1, type, window};
    ++n;
  }
};

// Per-row key interval [lo, hi) that slice s allows for query row i (i inside
// [q0, q1)); may be empty (lo >= hi).
inline void slice_row_interval(const mad_slice& s, int64_t i, int64_t& lo, int64_t& hi) {
  lo = s.k0;
  hi = s.k1;
  if (s.type == MAD_SLICE_CAUSAL) {
    int64_t off = i - s.q0;
    hi = std::min<int64_t>(hi, (int64_t)s.k0 + off + 1);
    if (s.window > 0) lo = std::max<int64_t>(lo, (int64_t)s.k0 + off - s.window + 1);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Tile classification for SLICES mode, one tiling.
// ---------------------------------------------------------------------------
static mad_status classify_slices(mad_plan* p, TilingHost& t) {
  const int BM = t.BM, BN = t.BN;
  const int64_t Tq = p->Tq, Tk = p->Tk;
  t.nqt = (int)((Tq + BM - 1) / BM);
  t.nkt = (int)((Tk + BN - 1) / BN);
  const int64_t ntiles = (int64_t)t.nqt * t.nkt;
  t.cls.assign(1, std::vector<uint8_t>(ntiles, CLS_EMPTY));
  t.aux.assign(1, std::vector<int32_t>(ntiles, -1));
  auto& cls = t.cls[0];
  auto& aux = t.aux[0];

  // 1. (tile, slice) records for every tile the slice's allowed band may touch.
  std::vector<std::pair<int64_t, int32_t>> rec;
  for (size_t si = 0; si < p->slices.size(); ++si) {
    const mad_slice& s = p->slices[si];
    if (s.q0 >= s.q1 || s.k0 >= s.k1) continue;
    for (int64_t qt = s.q0 / BM; qt <= (int64_t)(s.q1 - 1) / BM; ++qt) {
      int64_t r0 = std::max<int64_t>(s.q0, qt * BM);
      int64_t r1 = std::min<int64_t>({(int64_t)s.q1, (qt + 1) * BM, Tq});
      if (r0 >= r1) continue;
      int64_t lo0, hi0, lo1, hi1;
      slice_row_interval(s, r0, lo0, hi0);
      slice_row_interval(s, r1 - 1, lo1, hi1);
      // lo and hi are non-decreasing in i, so [lo(r0), hi(r1-1)) covers every row.
      int64_t lo = std::max<int64_t>(lo0, 0), hi = std::min<int64_t>(hi1, Tk);
      if (lo >= hi) continue;
      for (int64_t kt = lo / BN; kt <= (hi - 1) / BN; ++kt) rec.emplace_back(qt * t.nkt + kt, (int32_t)si);
    }
  }
  std::sort(rec.begin(), rec.end());

  // 2. Per touched tile: exact count of allowed in-range elements (union of slices).
  std::vector<std::pair<int64_t, int64_t>> iv;
  std::vector<int32_t> used;
  std::vector<uint8_t> touched;
  int64_t pairs = 0;
  for (size_t a = 0; a < rec.size();) {
    size_t b = a;
    while (b < rec.size() && rec[b].first == rec[a].first) ++b;
    const int64_t tile = rec[a].first;
    const int64_t qt = tile / t.nkt, kt = tile % t.nkt;
    const int64_t r0 = qt * BM, r1 = std::min<int64_t>(Tq, r0 + BM);
    const int64_t c0 = kt * BN, c1 = std::min<int64_t>(Tk, c0 + BN);
    const int64_t area = (r1 - r0) * (c1 - c0);
    int64_t count = -1;
    // fast path: one slice covers the whole in-range tile
    for (size_t x = a; x < b && count < 0; ++x) {
      const mad_slice& s = p->slices[rec[x].second];
      if (s.q0 > r0 || s.q1 < r1 || s.k0 > c0 || s.k1 < c1) continue;
      int64_t lo0, hi0, lo1, hi1;
      slice_row_interval(s, r0, lo0, hi0);
      slice_row_interval(s, r1 - 1, lo1, hi1);
      if (hi0 >= c1 && lo1 <= c0) count = area;
    }
    used.assign(b - a, 0);
    if (count < 0) {
      count = 0;
      for (int64_t i = r0; i < r1; ++i) {
        iv.clear();
        for (size_t x = a; x < b; ++x) {
          const mad_slice& s = p->slices[rec[x].second];
          if (i < s.q0 || i >= s.q1) continue;
          int64_t lo, hi;
          slice_row_interval(s, i, lo, hi);
          lo = std::max(lo, c0);
          hi = std::min(hi, c1);
          if (lo < hi) {
            iv.emplace_back(lo, hi);
            used[x - a] = 1;
          }
        }
        if (iv.empty()) continue;
        std::sort(iv.begin(), iv.end());
        int64_t cl = iv[0].first, ch = iv[0].second;
        for (size_t y = 1; y < iv.size(); ++y) {
          if (iv[y].first > ch) {
            count += ch - cl;
            cl = iv[y].first;
            ch = iv[y].second;
          } else {
            ch = std::max(ch, iv[y].second);
          }
        }
        count += ch - cl;
      }
    }
    pairs += count;
    if (count == 0) {
      cls[tile] = CLS_EMPTY;
    } else if (count == area) {
      cls[tile] = CLS_FULL;
    } else {
      cls[tile] = CLS_PARTIAL;
      int64_t off = (int64_t)p->tile_slices.size();
      if (off > INT32_MAX - 1024) return fail(MAD_ERR_NOMEM, "mask plan: partial-tile slice lists exceed 2^31 entries");
      aux[tile] = (int32_t)off;
      p->tile_slices.push_back(0);
      int32_t n = 0;
      for (size_t x = a; x < b; ++x)
        if (used[x - a]) {
          p->tile_slices.push_back(rec[x].second);
          ++n;
        }
      p->tile_slices[off] = n;
    }
    a = b;
  }
  if (p->pairs.empty()) p->pairs.assign(1, pairs);
  return MAD_OK;
}

// ---------------------------------------------------------------------------
// Tile classification for BLOCKS mode, one tiling, every group.
// ---------------------------------------------------------------------------
static bool keep_bit(const mad_plan* p, int g, int qb, int kb) {
  return (p->keep[((size_t)g * p->n_qb + qb) * p->nw + (kb >> 6)] >> (kb & 63)) & 1u;
}

// Class of the block-mask rectangle rows [r0, r1) x keys [c0, c1) (in range,
// non-empty) for group g.
static uint8_t rect_class(const mad_plan* p, int g, int64_t r0, int64_t r1, int64_t c0, int64_t c1) {
  const int qa = p->row_qb[r0], qz = p->row_qb[r1 - 1];
  const int ka = p->col_kb[c0], kz = p->col_kb[c1 - 1];
  bool any = false, all = true;
  for (int qb = qa; qb <= qz; ++qb)
    for (int kb = ka; kb <= kz; ++kb) {
      const bool k = keep_bit(p, g, qb, kb);
      any |= k;
      all &= k;
    }
  return !any ? CLS_EMPTY : (all ? CLS_FULL : CLS_PARTIAL);
}

// A PARTIAL tile is also split into the four parts its kernel hands to its
// four waves (tiling 0: 32-row strips; tiling 1: 32-key strips).  When every
// part is FULL or EMPTY -- blocks aligned to the strips, e.g. 64- or 128-token
// blocks -- the tile's aux entry records which parts are FULL (bit w for wave
// w), and each wave then runs its part without mask arithmetic or skips it;
// otherwise aux stays -1 and the waves evaluate the keep bitmap.
static int32_t wave_parts(const mad_plan* p, int g, bool rows_split, int64_t r0, int64_t r1, int64_t c0,
                          int64_t c1) {
  int32_t full = 0;
  for (int w = 0; w < 4; ++w) {
    int64_t a0 = r0, a1 = r1, b0 = c0, b1 = c1;
    if (rows_split) {
      a0 = r0 + 32 * w;
      a1 = std::min<int64_t>(r1, a0 + 32);
    } else {
      b0 = c0 + 32 * w;
      b1 = std::min<int64_t>(c1, b0 + 32);
    }
    if (a0 >= a1 || b0 >= b1) continue;  // nothing in range: EMPTY
    const uint8_t c = rect_class(p, g, a0, a1, b0, b1);
    if (c == CLS_PARTIAL) return -1;
    if (c == CLS_FULL) full |= 1 << w;
  }
  return full;
}

static void classify_blocks(mad_plan* p, TilingHost& t) {
  const int BM = t.BM, BN = t.BN;
  const int64_t Tq = p->Tq, Tk = p->Tk;
  const bool rows_split = BM == BM0;  // tiling 0 gives each wave 32 rows; tiling 1 gives each 32 keys
  t.nqt = (int)((Tq + BM - 1) / BM);
  t.nkt = (int)((Tk + BN - 1) / BN);
  const int64_t ntiles = (int64_t)t.nqt * t.nkt;
  t.cls.assign(p->G, std::vector<uint8_t>());
  t.aux.assign(p->G, std::vector<int32_t>());
  auto work = [&](int g) {
    auto& cls = t.cls[g];
    auto& aux = t.aux[g];
    cls.assign(ntiles, CLS_EMPTY);
    aux.assign(ntiles, -1);
    for (int qt = 0; qt < t.nqt; ++qt) {
      const int64_t r0 = (int64_t)qt * BM, r1 = std::min<int64_t>(Tq, r0 + BM);
      for (int kt = 0; kt < t.nkt; ++kt) {
        const int64_t c0 = (int64_t)kt * BN, c1 = std::min<int64_t>(Tk, c0 + BN);
        const uint8_t c = rect_class(p, g, r0, r1, c0, c1);
        cls[(int64_t)qt * t.nkt + kt] = c;
        if (c == CLS_PARTIAL) aux[(int64_t)qt * t.nkt + kt] = wave_parts(p, g, rows_split, r0, r1, c0, c1);
      }
    }
  };
  unsigned nth = std::max(1u, std::min<unsigned>(std::thread::hardware_concurrency(), 16u));
  nth = std::min<unsigned>(nth, (unsigned)p->G);
  std::vector<std::thread> th;
  for (unsigned w = 0; w < nth; ++w)
    th.emplace_back([&, w] {
      for (int g = (int)w; g < p->G; g += (int)nth) work(g);
    });
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------------------
// Visit lists and longest-first order for one tiling.
// ---------------------------------------------------------------------------
static mad_status build_lists(mad_plan* p, TilingHost& t, bool csc) {
  const int nmaj = csc ? t.nkt : t.nqt, nmin = csc ? t.nqt : t.nkt;
  t.ptr.assign((size_t)p->G * (nmaj + 1), 0);
  t.ent.clear();
  t.ent_aux.clear();
  std::vector<int64_t> work(nmaj, 0);
  for (int c = 0; c < 3; ++c) t.n_class[c] = 0;
  for (int g = 0; g < p->G; ++g) {
    const auto& cls = t.cls[g];
    const bool have_aux = !t.aux[g].empty();
    for (int M = 0; M < nmaj; ++M) {
      if (t.ent.size() > (size_t)INT32_MAX - (size_t)nmin)
        return fail(MAD_ERR_NOMEM, "mask plan: visit lists exceed 2^31 entries");
      t.ptr[(size_t)g * (nmaj + 1) + M] = (int32_t)t.ent.size();
      for (int m = 0; m < nmin; ++m) {
        const int64_t tile = csc ? (int64_t)m * t.nkt + M : (int64_t)M * t.nkt + m;
        const uint8_t c = cls[tile];
        t.n_class[c]++;
        if (c == CLS_EMPTY) continue;
        t.ent.push_back((int32_t)((uint32_t)m | (c == CLS_PARTIAL ? ENT_PARTIAL : 0u)));
        t.ent_aux.push_back(have_aux ? t.aux[g][tile] : -1);
        work[M] += 1;
      }
    }
    t.ptr[(size_t)g * (nmaj + 1) + nmaj] = (int32_t)t.ent.size();
  }
  t.order.resize(nmaj);
  std::iota(t.order.begin(), t.order.end(), 0);
  std::stable_sort(t.order.begin(), t.order.end(), [&](int a, int b) { return work[a] > work[b]; });
  t.uniform = true;
  for (int g = 0; g < p->G && t.uniform; ++g)
    for (int M = 0; M < nmaj; ++M) {
      const size_t b = (size_t)g * (nmaj + 1);
      if (t.ptr[b + M + 1] - t.ptr[b + M] != t.ptr[b + 1] - t.ptr[b]) {
        t.uniform = false;
        break;
      }
    }
  return MAD_OK;
}

mad_status compile_slices(mad_plan* p) {
  p->tiling[0].BM = BM0;
  p->tiling[0].BN = BN0;
  p->tiling[1].BM = BM1;
  p->tiling[1].BN = BN1;
  p->pairs.clear();
  for (int w = 0; w < 2; ++w) {
    mad_status s = classify_slices(p, p->tiling[w]);
    if (s != MAD_OK) return s;
    s = build_lists(p, p->tiling[w], w == 1);
    if (s != MAD_OK) return s;
  }
  return MAD_OK;
}

mad_status compile_blocks(mad_plan* p) {
  p->tiling[0].BM = BM0;
  p->tiling[0].BN = BN0;
  p->tiling[1].BM = BM1;
  p->tiling[1].BN = dkdv_tile_keys(p->k_edges.data(), p->n_kb);
  p->pairs.assign(p->G, 0);
  for (int g = 0; g < p->G; ++g) {
    int64_t n = 0;
    for (int qb = 0; qb < p->n_qb; ++qb) {
      const int64_t lq = p->q_edges[qb + 1] - p->q_edges[qb];
      for (int kb = 0; kb < p->n_kb; ++kb)
        if (keep_bit(p, g, qb, kb)) n += lq * (p->k_edges[kb + 1] - p->k_edges[kb]);
    }
    p->pairs[g] = n;
  }
  for (int w = 0; w < 2; ++w) {
    classify_blocks(p, p->tiling[w]);
    mad_status s = build_lists(p, p->tiling[w], w == 1);
    if (s != MAD_OK) return s;
  }
  return MAD_OK;
}

}  // namespace mad

using namespace mad;

// ===========================================================================
// C ABI: mask generation
// ===========================================================================
extern "C" mad_status mad_mask_slices(int32_t pattern, int32_t T, const mad_mask_params* prm,
                                      mad_slice* out, int64_t cap, int64_t* n_out) {
  clear_error();
  if (!n_out) return fail(MAD_ERR_INVALID, "mad_mask_slices: n_out is NULL");
  if (T < 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: T < 0");
  if (out && cap < 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: cap < 0");
  mad_mask_params d{};
  d.window = 4096;
  d.prefix = -1;
  d.question = 2048;
  d.n_answers = 4;
  d.global_len = 256;
  d.block = 1024;
  const mad_mask_params& P = prm ? *prm : d;
  const bool doc = pattern == MAD_MASK_FULL_DOCUMENT || pattern == MAD_MASK_CAUSAL_DOCUMENT ||
                   pattern == MAD_MASK_SLIDING_WINDOW_CAUSAL_DOCUMENT ||
                   pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT || pattern == MAD_MASK_PREFIX_LM_DOCUMENT ||
                   pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT_GLOBAL;
  if (doc) {
    if (!P.doc_lens || P.n_docs < 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: document pattern needs doc_lens");
    int64_t sum = 0;
    for (int32_t x = 0; x < P.n_docs; ++x) {
      if (P.doc_lens[x] < 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: negative document length");
      sum += P.doc_lens[x];
    }
    if (sum != T) return fail(MAD_ERR_INVALID, "mad_mask_slices: document lengths do not sum to T");
  }
  const bool windowed = pattern == MAD_MASK_SLIDING_WINDOW || pattern == MAD_MASK_SLIDING_WINDOW_CAUSAL_DOCUMENT ||
                        pattern == MAD_MASK_GLOBAL_SLIDING;
  if (windowed && P.window <= 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: window must be > 0");
  const bool blocked = pattern == MAD_MASK_CAUSAL_BLOCKWISE || pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT ||
                       pattern == MAD_MASK_CAUSAL_BLOCKWISE_LAST || pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT_GLOBAL;
  if (blocked && P.block <= 0)
    return fail(MAD_ERR_INVALID, "mad_mask_slices: block must be > 0");
  // SHARED_QUESTION: answers split the rest equally, or take the lengths given in doc_lens
  const bool sq_lens = pattern == MAD_MASK_SHARED_QUESTION && P.doc_lens && P.n_docs > 0;
  if (pattern == MAD_MASK_SHARED_QUESTION && (P.question < 0 || (!sq_lens && P.n_answers <= 0)))
    return fail(MAD_ERR_INVALID, "mad_mask_slices: question >= 0 and n_answers > 0 required");
  if (sq_lens) {
    int64_t sum = 0;
    for (int32_t x = 0; x < P.n_docs; ++x) {
      if (P.doc_lens[x] < 0) return fail(MAD_ERR_INVALID, "mad_mask_slices: negative answer length");
      sum += P.doc_lens[x];
    }
    if (sum != T - std::min(P.question, T))
      return fail(MAD_ERR_INVALID, "mad_mask_slices: answer lengths do not sum to T - question");
  }
  if (pattern == MAD_MASK_GLOBAL_SLIDING && P.global_len < 0)
    return fail(MAD_ERR_INVALID, "mad_mask_slices: global_len must be >= 0");

  SliceSink S{out, cap};
  const int32_t F = MAD_SLICE_FULL, C = MAD_SLICE_CAUSAL;
  switch (pattern) {
    case MAD_MASK_FULL: S.add(0, T, 0, T, F); break;
    case MAD_MASK_CAUSAL: S.add(0, T, 0, T, C); break;
    case MAD_MASK_SLIDING_WINDOW: S.add(0, T, 0, T, C, P.window); break;
    case MAD_MASK_FULL_DOCUMENT:
    case MAD_MASK_CAUSAL_DOCUMENT:
    case MAD_MASK_SLIDING_WINDOW_CAUSAL_DOCUMENT:
    case MAD_MASK_BLOCK_CAUSAL_DOCUMENT:
    case MAD_MASK_BLOCK_CAUSAL_DOCUMENT_GLOBAL:
    case MAD_MASK_PREFIX_LM_DOCUMENT: {
      int32_t s0 = 0;
      for (int32_t x = 0; x < P.n_docs; ++x) {
        const int32_t L = P.doc_lens[x], e = s0 + L;
        if (pattern == MAD_MASK_FULL_DOCUMENT) {
          S.add(s0, e, s0, e, F);
        } else if (pattern == MAD_MASK_CAUSAL_DOCUMENT) {
          S.add(s0, e, s0, e, C);
        } else if (pattern == MAD_MASK_SLIDING_WINDOW_CAUSAL_DOCUMENT) {
          S.add(s0, e, s0, e, C, P.window);
        } else if (pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT) {
          // block b of the document (from its start) sees blocks 0..b in full
          for (int32_t b0 = s0; b0 < e; b0 += P.block) {
            const int32_t b1 = std::min(e, b0 + P.block);
            S.add(b0, b1, s0, b1, F);
          }
        } else if (pattern == MAD_MASK_BLOCK_CAUSAL_DOCUMENT_GLOBAL) {
          // the document's rows in global block [g0, g0 + B) see its keys up to that block's end
          for (int64_t g0 = (int64_t)s0 / P.block * P.block; g0 < e; g0 += P.block) {
            const int32_t r0 = (int32_t)std::max<int64_t>(s0, g0), r1 = (int32_t)std::min<int64_t>(e, g0 + P.block);
            S.add(r0, r1, s0, r1, F);
          }
        } else {
          const int32_t pd = L / 4;
          S.add(s0, e, s0, s0 + pd, F);
          S.add(s0 + pd, e, s0 + pd, e, C);
        }
        s0 = e;
      }
      break;
    }
    case MAD_MASK_PREFIX_LM: {
      int32_t Pp = P.prefix < 0 ? T / 4 : std::min(P.prefix, T);
      S.add(0, T, 0, Pp, F);
      S.add(Pp, T, Pp, T, C);
      break;
    }
    case MAD_MASK_SHARED_QUESTION: {
      const int32_t Q = std::min(P.question, T);
      S.add(0, Q, 0, Q, C);
      const int32_t rest = T - Q, na = sq_lens ? P.n_docs : P.n_answers, base = rest / na;
      int32_t a0 = Q;
      for (int32_t a = 0; a < na; ++a) {
        const int32_t a1 = sq_lens ? a0 + P.doc_lens[a] : (a == na - 1) ? T : a0 + base;
        if (a1 > a0) {
          S.add(a0, a1, 0, Q, F);
          S.add(a0, a1, a0, a1, C);
        }
        a0 = a1;
      }
      break;
    }
    case MAD_MASK_GLOBAL_SLIDING: {
      S.add(0, T, 0, T, C, P.window);
      // keys below G that fell out of the window: j < G and j <= i - W
      if (P.window < T) S.add(P.window, T, 0, std::min(P.global_len, T), C);
      break;
    }
    case MAD_MASK_CAUSAL_BLOCKWISE: {
      for (int32_t b0 = 0; b0 < T; b0 += P.block) {
        const int32_t b1 = std::min(T, b0 + P.block);
        S.add(b0, b1, b0, b1, C);
        S.add(b0, b1, 0, b0, F);
      }
      break;
    }
    case MAD_MASK_CAUSAL_BLOCKWISE_LAST: {
      int32_t last = 0;  // start of the last block
      for (int64_t b0 = 0; b0 < T; b0 += P.block) {
        const int32_t b1 = (int32_t)std::min<int64_t>(T, b0 + P.block);
        S.add((int32_t)b0, b1, (int32_t)b0, b1, C);
        last = (int32_t)b0;
      }
      S.add(last, T, 0, last, F);
      break;
    }
    default: return fail(MAD_ERR_INVALID, "mad_mask_slices: unknown pattern " + std::to_string(pattern));
  }
  *n_out = S.n;
  if (out && S.n > cap) return fail(MAD_ERR_INVALID, "mad_mask_slices: cap too small");
  return MAD_OK;
}

extern "C" mad_status mad_varlen_slices(const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int32_t causal,
                                        int32_t window, int32_t bottom_right, mad_slice* out, int64_t cap,
                                        int64_t* n_out) {
  clear_error();
  if (!n_out) return fail(MAD_ERR_INVALID, "mad_varlen_slices: n_out is NULL");
  if (batch < 0 || (batch > 0 && (!cu_q || !cu_k))) return fail(MAD_ERR_INVALID, "mad_varlen_slices: bad batch / offsets");
  if (out && cap < 0) return fail(MAD_ERR_INVALID, "mad_varlen_slices: cap < 0");
  if (window < 0 || (window > 0 && !causal)) return fail(MAD_ERR_INVALID, "mad_varlen_slices: window needs causal");
  if (batch > 0 && (cu_q[0] != 0 || cu_k[0] != 0)) return fail(MAD_ERR_INVALID, "mad_varlen_slices: offsets must start at 0");
  for (int32_t b = 0; b < batch; ++b) {
    if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b])
      return fail(MAD_ERR_INVALID, "mad_varlen_slices: offsets must be non-decreasing");
    if (causal && bottom_right && window > 0 && cu_k[b + 1] - cu_k[b] > cu_q[b + 1] - cu_q[b])
      return fail(MAD_ERR_UNSUPPORTED, "mad_varlen_slices: a window with bottom-right alignment needs Lk <= Lq");
  }
  SliceSink S{out, cap};
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
    if (q0 == q1 || k0 == k1) continue;
    if (!causal) {
      S.add(q0, q1, k0, k1, MAD_SLICE_FULL);
    } else if (!bottom_right) {
      S.add(q0, q1, k0, k1, MAD_SLICE_CAUSAL, window);
    } else {
      const int32_t off = (k1 - k0) - (q1 - q0);  // key c is allowed from row c - off on
      if (off >= 0) {
        if (off > 0) S.add(q0, q1, k0, k0 + off, MAD_SLICE_FULL);  // keys every row sees
        S.add(q0, q1, k0 + off, k1, MAD_SLICE_CAUSAL, window);  // window > 0 only when off == 0
      } else {
        S.add(q0 - off, q1, k0, k1, MAD_SLICE_CAUSAL, window);  // the first -off rows see nothing
      }
    }
  }
  *n_out = S.n;
  if (out && S.n > cap) return fail(MAD_ERR_INVALID, "mad_varlen_slices: cap too small");
  return MAD_OK;
}

extern "C" mad_status mad_ring_step_slices(int32_t layout, int32_t n_ranks, int32_t chunk, int32_t rank,
                                           int32_t source, mad_slice* out, int64_t cap, int64_t* n_out) {
  clear_error();
  if (!n_out) return fail(MAD_ERR_INVALID, "mad_ring_step_slices: n_out is NULL");
  if (layout != 0 && layout != 1) return fail(MAD_ERR_INVALID, "mad_ring_step_slices: layout must be 0 or 1");
  if (n_ranks <= 0 || chunk <= 0 || rank < 0 || rank >= n_ranks || source < 0 || source >= n_ranks)
    return fail(MAD_ERR_INVALID, "mad_ring_step_slices: bad n_ranks/chunk/rank/source");
  if (layout == 1 && chunk % 2) return fail(MAD_ERR_INVALID, "mad_ring_step_slices: head-tail needs an even chunk");
  SliceSink S{out, cap};
  // Pieces: (global piece index, local offset, length) for the query rank and the key rank.
  struct Piece { int64_t gidx; int32_t off, len; };
  Piece qp[2], kp[2];
  int np;
  if (layout == 0) {
    np = 1;
    qp[0] = {rank, 0, chunk};
    kp[0] = {source, 0, chunk};
  } else {
    np = 2;
    const int32_t h = chunk / 2;
    qp[0] = {rank, 0, h};
    qp[1] = {2 * (int64_t)n_ranks - 1 - rank, h, h};
    kp[0] = {source, 0, h};
    kp[1] = {2 * (int64_t)n_ranks - 1 - source, h, h};
  }
  // Pieces have equal length, so global causality between two pieces is
  // FULL (key piece earlier), CAUSAL (same piece) or nothing (key piece later).
  for (int a = 0; a < np; ++a)
    for (int b = 0; b < np; ++b) {
      if (kp[b].gidx < qp[a].gidx)
        S.add(qp[a].off, qp[a].off + qp[a].len, kp[b].off, kp[b].off + kp[b].len, MAD_SLICE_FULL);
      else if (kp[b].gidx == qp[a].gidx)
        S.add(qp[a].off, qp[a].off + qp[a].len, kp[b].off, kp[b].off + kp[b].len, MAD_SLICE_CAUSAL);
    }
  *n_out = S.n;
  if (out && S.n > cap) return fail(MAD_ERR_INVALID, "mad_ring_step_slices: cap too small");
  return MAD_OK;
}

extern "C" mad_status mad_block_topk(const float* scores, int32_t n_groups, int32_t n_qb, int32_t n_kb,
                                     int32_t sparsity_pct, uint64_t* keep) {
  clear_error();
  if (!scores || !keep) return fail(MAD_ERR_INVALID, "mad_block_topk: NULL pointer");
  if (n_groups <= 0 || n_qb <= 0 || n_kb <= 0) return fail(MAD_ERR_INVALID, "mad_block_topk: sizes must be > 0");
  if (sparsity_pct < 0 || sparsity_pct > 100) return fail(MAD_ERR_INVALID, "mad_block_topk: sparsity_pct out of [0,100]");
  const int64_t total = (int64_t)n_groups * n_qb * n_kb;
  for (int64_t x = 0; x < total; ++x)
    if (scores[x] != scores[x]) return fail(MAD_ERR_INVALID, "mad_block_topk: NaN score");
  const int nw = (n_kb + 63) / 64;
  const int k = std::max(1, n_kb - (int)(((int64_t)sparsity_pct * n_kb) / 100));
  const int64_t rows = (int64_t)n_groups * n_qb;
  auto work = [&](int64_t r0, int64_t r1) {
    std::vector<int32_t> idx(n_kb);
    for (int64_t r = r0; r < r1; ++r) {
      const float* s = scores + r * n_kb;
      std::iota(idx.begin(), idx.end(), 0);
      auto better = [s](int32_t a, int32_t b) { return s[a] > s[b] || (s[a] == s[b] && a < b); };
      std::nth_element(idx.begin(), idx.begin() + (k - 1), idx.end(), better);
      uint64_t* w = keep + r * nw;
      std::memset(w, 0, sizeof(uint64_t) * nw);
      for (int x = 0; x < k; ++x) w[idx[x] >> 6] |= 1ull << (idx[x] & 63);
    }
  };
  unsigned nth = std::max(1u, std::min<unsigned>(std::thread::hardware_concurrency(), 16u));
  if (rows < 64) nth = 1;
  std::vector<std::thread> th;
  for (unsigned w = 0; w < nth; ++w) th.emplace_back(work, rows * w / nth, rows * (w + 1) / nth);
  for (auto& x : th) x.join();
  return MAD_OK;
}

// ===========================================================================
// C ABI: compile, inspect, destroy
// ===========================================================================
extern "C" mad_status mad_mask_compile(const mad_slice* slices, int64_t n, int32_t Tq, int32_t Tk, mad_plan** out) {
  clear_error();
  if (!out) return fail(MAD_ERR_INVALID, "mad_mask_compile: out is NULL");
  *out = nullptr;
  if (n < 0 || (n > 0 && !slices)) return fail(MAD_ERR_INVALID, "mad_mask_compile: bad slice array");
  if (Tq < 0 || Tk < 0) return fail(MAD_ERR_INVALID, "mad_mask_compile: Tq, Tk must be >= 0");
  if (n > INT32_MAX) return fail(MAD_ERR_INVALID, "mad_mask_compile: too many slices");
  for (int64_t x = 0; x < n; ++x) {
    const mad_slice& s = slices[x];
    if (s.q0 < 0 || s.q0 > s.q1 || s.q1 > Tq || s.k0 < 0 || s.k0 > s.k1 || s.k1 > Tk)
      return fail(MAD_ERR_INVALID, "mad_mask_compile: slice " + std::to_string(x) + " out of range");
    if (s.type != MAD_SLICE_FULL && s.type != MAD_SLICE_CAUSAL)
      return fail(MAD_ERR_INVALID, "mad_mask_compile: slice " + std::to_string(x) + " has unknown type");
    if (s.window < 0 || (s.window > 0 && s.type != MAD_SLICE_CAUSAL))
      return fail(MAD_ERR_INVALID, "mad_mask_compile: slice " + std::to_string(x) + " has a bad window");
  }
  mad_plan* p = new (std::nothrow) mad_plan();
  if (!p) return fail(MAD_ERR_NOMEM, "mad_mask_compile: out of host memory");
  try {
    p->Tq = Tq;
    p->Tk = Tk;
    p->G = 1;
    p->mode = MODE_SLICES;
    p->slices.assign(slices, slices + n);
    mad_status s = compile_slices(p);
    if (s != MAD_OK) {
      delete p;
      return s;
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MAD_ERR_NOMEM, "mad_mask_compile: out of host memory");
  }
  *out = p;
  return MAD_OK;
}

extern "C" mad_status mad_sparse_plan(int32_t n_groups, const int32_t* q_edges, int32_t n_qb, const int32_t* k_edges,
                                      int32_t n_kb, const uint64_t* keep, mad_plan** out) {
  clear_error();
  if (!out) return fail(MAD_ERR_INVALID, "mad_sparse_plan: out is NULL");
  *out = nullptr;
  if (!q_edges || !k_edges || !keep) return fail(MAD_ERR_INVALID, "mad_sparse_plan: NULL pointer");
  if (n_groups <= 0 || n_qb <= 0 || n_kb <= 0) return fail(MAD_ERR_INVALID, "mad_sparse_plan: sizes must be > 0");
  if (q_edges[0] != 0 || k_edges[0] != 0) return fail(MAD_ERR_INVALID, "mad_sparse_plan: edges must start at 0");
  for (int32_t x = 0; x < n_qb; ++x)
    if (q_edges[x + 1] <= q_edges[x]) return fail(MAD_ERR_INVALID, "mad_sparse_plan: q_edges not strictly increasing");
  for (int32_t x = 0; x < n_kb; ++x)
    if (k_edges[x + 1] <= k_edges[x]) return fail(MAD_ERR_INVALID, "mad_sparse_plan: k_edges not strictly increasing");
  mad_plan* p = new (std::nothrow) mad_plan();
  if (!p) return fail(MAD_ERR_NOMEM, "mad_sparse_plan: out of host memory");
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
    p->keep.assign(keep, keep + (size_t)n_groups * n_qb * p->nw);
    // bits past n_kb in the last word are ignored
    if (n_kb % 64) {
      const uint64_t m = (1ull << (n_kb % 64)) - 1;
      for (size_t r = 0; r < (size_t)n_groups * n_qb; ++r) p->keep[r * p->nw + p->nw - 1] &= m;
    }
    p->row_qb.resize(p->Tq);
    p->col_kb.resize(p->Tk);
    for (int32_t b = 0; b < n_qb; ++b)
      for (int32_t i = q_edges[b]; i < q_edges[b + 1]; ++i) p->row_qb[i] = b;
    for (int32_t b = 0; b < n_kb; ++b)
      for (int32_t j = k_edges[b]; j < k_edges[b + 1]; ++j) p->col_kb[j] = b;
    mad_status s = compile_blocks(p);
    if (s != MAD_OK) {
      delete p;
      return s;
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MAD_ERR_NOMEM, "mad_sparse_plan: out of host memory");
  }
  *out = p;
  return MAD_OK;
}

extern "C" mad_status mad_plan_stats(const mad_plan* p, int32_t which, int64_t* pairs, int64_t* n_full,
                                     int64_t* n_partial, int64_t* n_empty) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_plan_stats: plan is NULL");
  if (which != 0 && which != 1) return fail(MAD_ERR_INVALID, "mad_plan_stats: which must be 0 or 1");
  if (pairs)
    for (int g = 0; g < p->G; ++g) pairs[g] = p->pairs[g];
  const TilingHost& t = p->tiling[which];
  if (n_empty) *n_empty = t.n_class[CLS_EMPTY];
  if (n_full) *n_full = t.n_class[CLS_FULL];
  if (n_partial) *n_partial = t.n_class[CLS_PARTIAL];
  return MAD_OK;
}

extern "C" mad_status mad_plan_lists(const mad_plan* p, int32_t which, int64_t* n_ptr, int64_t* n_ent,
                                     int64_t* n_order, int32_t* ptr, int32_t* ent, int32_t* ent_aux, int32_t* order) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_plan_lists: plan is NULL");
  if (which != 0 && which != 1) return fail(MAD_ERR_INVALID, "mad_plan_lists: which must be 0 or 1");
  const TilingHost& t = p->tiling[which];
  const int64_t np = (int64_t)t.ptr.size(), ne = t.ptr.empty() ? 0 : t.ptr.back();
  const int64_t no = which == 0 ? t.nqt : t.nkt;
  if (n_ptr) *n_ptr = np;
  if (n_ent) *n_ent = ne;
  if (n_order) *n_order = no;
  if (ptr && np) std::memcpy(ptr, t.ptr.data(), (size_t)np * 4);
  if (!p->on_device) {
    if (ent && ne) std::memcpy(ent, t.ent.data(), (size_t)ne * 4);
    if (ent_aux && ne) std::memcpy(ent_aux, t.ent_aux.data(), (size_t)ne * 4);
    if (order && no) std::memcpy(order, t.order.data(), (size_t)no * 4);
    return MAD_OK;
  }
  const TilingDev& d = p->tdev[which];
  hipError_t e = hipSuccess;
  if (ent && ne && e == hipSuccess) e = hipMemcpy(ent, d.ent, (size_t)ne * 4, hipMemcpyDeviceToHost);
  if (ent_aux && ne && e == hipSuccess) e = hipMemcpy(ent_aux, d.ent_aux, (size_t)ne * 4, hipMemcpyDeviceToHost);
  if (order && no && e == hipSuccess) e = hipMemcpy(order, d.order, (size_t)no * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MAD_ERR_HIP, std::string("mad_plan_lists: hipMemcpy: ") + hipGetErrorString(e));
  return MAD_OK;
}

extern "C" mad_status mad_plan_info(const mad_plan* p, int32_t which, int32_t* Tq, int32_t* Tk, int32_t* n_groups,
                                    int32_t* BM, int32_t* BN, int32_t* n_qt, int32_t* n_kt) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_plan_info: plan is NULL");
  if (which != 0 && which != 1) return fail(MAD_ERR_INVALID, "mad_plan_info: which must be 0 or 1");
  const TilingHost& t = p->tiling[which];
  if (Tq) *Tq = p->Tq;
  if (Tk) *Tk = p->Tk;
  if (n_groups) *n_groups = p->G;
  if (BM) *BM = t.BM;
  if (BN) *BN = t.BN;
  if (n_qt) *n_qt = t.nqt;
  if (n_kt) *n_kt = t.nkt;
  return MAD_OK;
}

extern "C" mad_status mad_plan_export(const mad_plan* p, int32_t which, int32_t group, uint8_t* classes,
                                      int64_t* csr_ptr, int32_t* csr_idx, int64_t* csc_ptr, int32_t* csc_idx) {
  clear_error();
  if (!p) return fail(MAD_ERR_INVALID, "mad_plan_export: plan is NULL");
  if (which != 0 && which != 1) return fail(MAD_ERR_INVALID, "mad_plan_export: which must be 0 or 1");
  if (group < 0 || group >= p->G) return fail(MAD_ERR_INVALID, "mad_plan_export: group out of range");
  const TilingHost& t = p->tiling[which];
  std::vector<uint8_t> dev_cls;
  if (p->on_device) {
    // classes rebuilt from the group's visit lists, copied back from the device
    const int nmaj = which == 0 ? t.nqt : t.nkt;
    const int32_t* gp = t.ptr.data() + (size_t)group * (nmaj + 1);
    const int64_t n = gp[nmaj] - gp[0];
    std::vector<int32_t> ent(n);
    if (n > 0) {
      hipError_t e = hipMemcpy(ent.data(), p->tdev[which].ent + gp[0], (size_t)n * 4, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return fail(MAD_ERR_HIP, std::string("mad_plan_export: hipMemcpy: ") + hipGetErrorString(e));
    }
    dev_cls.assign((size_t)t.nqt * t.nkt, CLS_EMPTY);
    for (int M = 0; M < nmaj; ++M)
      for (int32_t x = gp[M]; x < gp[M + 1]; ++x) {
        const uint32_t en = (uint32_t)ent[x - gp[0]];
        const int m = (int)(en & 0x7fffffffu);
        const int64_t tile = which == 0 ? (int64_t)M * t.nkt + m : (int64_t)m * t.nkt + M;
        dev_cls[tile] = (en & ENT_PARTIAL) ? CLS_PARTIAL : CLS_FULL;
      }
  }
  const auto& cls = p->on_device ? dev_cls : t.cls[group];
  if (classes) std::memcpy(classes, cls.data(), cls.size());
  if (csr_ptr || csr_idx) {
    int64_t n = 0;
    for (int qt = 0; qt < t.nqt; ++qt) {
      if (csr_ptr) csr_ptr[qt] = n;
      for (int kt = 0; kt < t.nkt; ++kt)
        if (cls[(int64_t)qt * t.nkt + kt] != CLS_EMPTY) {
          if (csr_idx) csr_idx[n] = kt;
          ++n;
        }
    }
    if (csr_ptr) csr_ptr[t.nqt] = n;
  }
  if (csc_ptr || csc_idx) {
    int64_t n = 0;
    for (int kt = 0; kt < t.nkt; ++kt) {
      if (csc_ptr) csc_ptr[kt] = n;
      for (int qt = 0; qt < t.nqt; ++qt)
        if (cls[(int64_t)qt * t.nkt + kt] != CLS_EMPTY) {
          if (csc_idx) csc_idx[n] = qt;
          ++n;
        }
    }
    if (csc_ptr) csc_ptr[t.nkt] = n;
  }
  return MAD_OK;
}
