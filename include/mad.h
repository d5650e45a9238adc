/*
 * mad.h -- C ABI of the mask-aware dense attention library for MI355X (gfx950).
 *
 * The library computes single-GPU softmax attention forward and backward
 * (bf16 Q/K/V, fp32 accumulation, output plus log-sum-exp) under the mask
 * patterns catalogued by "Long-Context Attention Benchmark: From Kernel
 * Efficiency to Distributed Context Parallelism" (LongCA-bench): 12 static
 * patterns and 2 dynamic block-sparse patterns (section 2.1.1 "Input mask
 * patterns"; the notes' key design 1).  Its input follows the benchmark's
 * unified input representation (section 2.1 "Data preparation", section 2.2
 * "Attention kernel"): variable-length sequences packed along one token axis,
 * MHA/GQA head mapping, and a mask described as a list of
 * (q_range, k_range, full | causal) slices.
 *
 * Conventions shared by every entry point
 *   - Token layout is packed, batch 1: Q is [Tq, Hq, d], K and V are
 *     [Tk, Hkv, d], with d contiguous.  Query head h reads KV head
 *     h / (Hq / Hkv) (contiguous GQA groups; Hkv == Hq is MHA).
 *   - Device pointers come from the caller (for example PyTorch tensors);
 *     the library never frees them.  Host pointers are read during the call
 *     only.  Kernels run on the caller's hipStream_t; a call returns after
 *     enqueueing, so results are ready when the stream is.
 *   - Every call validates its arguments before it writes or launches
 *     anything.  On failure it returns a non-zero mad_status, writes and
 *     launches nothing, and mad_last_error() returns a message for the
 *     calling thread.  Faults inside a kernel surface at the caller's next
 *     synchronisation of the stream.
 *   - Floating point: inputs and O/dQ/dK/dV are bf16 (round to nearest
 *     even on output); LSE and the delta workspace are fp32; LSE is the
 *     natural log of the sum of exp(scale * q.k) over allowed keys.  A query
 *     row with no allowed key gets O = 0 and LSE = -inf.
 */
#ifndef MAD_H_
#define MAD_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAD_OK = 0,
  MAD_ERR_INVALID = 1,     /* bad argument: null pointer, size, range, plan/shape mismatch */
  MAD_ERR_UNSUPPORTED = 2, /* valid but not built: head dim other than 64/128/256, alignment */
  MAD_ERR_HIP = 3,         /* a HIP runtime call failed (message holds the HIP error) */
  MAD_ERR_NOMEM = 4        /* host or device allocation for plan metadata failed */
} mad_status;

/* ---------------------------------------------------------------------------
 * Mask slices -- the unified mask description.
 *
 * A slice allows the pairs (i, j) with q0 <= i < q1 and k0 <= j < k1, and
 *   FULL   : every pair of the rectangle;
 *   CAUSAL : pairs with (j - k0) <= (i - q0), i.e. causal aligned at the
 *            slice's top-left corner, and if window > 0 additionally
 *            (i - q0) - (j - k0) < window (a causal sliding window that
 *            counts the key itself).
 * The mask is the union of all slices; slices may overlap.  Indices are
 * global token positions in the packed Q (i) and K (j) streams.
 * ------------------------------------------------------------------------- */
enum { MAD_SLICE_FULL = 0, MAD_SLICE_CAUSAL = 1 };

typedef struct {
  int32_t q0, q1; /* half-open query range */
  int32_t k0, k1; /* half-open key range */
  int32_t type;   /* MAD_SLICE_FULL or MAD_SLICE_CAUSAL */
  int32_t window; /* CAUSAL only: 0 = unbounded, W > 0 = W-key causal window */
} mad_slice;

/* ---------------------------------------------------------------------------
 * Static mask patterns (LongCA-bench section 2.1.1; the notes' key design 1:
 * six regular patterns -- FULL, CAUSAL, sliding window and the document
 * variants -- and six heterogeneous ones -- Shared Question, Global Sliding,
 * Causal Blockwise, Prefix LM, Block Causal Document and a sixth one the
 * pages do not name, read here as Prefix LM applied per packed document).
 * ------------------------------------------------------------------------- */
typedef enum {
  MAD_MASK_FULL = 0,
  MAD_MASK_CAUSAL = 1,
  MAD_MASK_SLIDING_WINDOW = 2,                 /* i - W < j <= i */
  MAD_MASK_FULL_DOCUMENT = 3,                  /* same document */
  MAD_MASK_CAUSAL_DOCUMENT = 4,                /* same document and j <= i */
  MAD_MASK_SLIDING_WINDOW_CAUSAL_DOCUMENT = 5, /* same document and i - W < j <= i */
  MAD_MASK_PREFIX_LM = 6,                      /* j <= max(i, P - 1) */
  MAD_MASK_SHARED_QUESTION = 7,                /* causal; answers see the question and themselves */
  MAD_MASK_GLOBAL_SLIDING = 8,                 /* j <= i and (j < G or i - j < W) */
  MAD_MASK_CAUSAL_BLOCKWISE = 9,               /* causal in a block, full to earlier blocks */
  MAD_MASK_BLOCK_CAUSAL_DOCUMENT = 10,         /* same document, block-causal from the doc start */
  MAD_MASK_PREFIX_LM_DOCUMENT = 11,            /* prefix LM inside each document, p = L/4 */
  /* Alternative readings of two heterogeneous patterns (the pages name them
   * without a formula; the readings above are the ones the workloads use):   */
  MAD_MASK_CAUSAL_BLOCKWISE_LAST = 12,         /* causal inside each block of B; only the last
                                                  block also sees every earlier block in full
                                                  (the in-context-learning layout: independent
                                                  demonstrations, one query block over all) */
  MAD_MASK_BLOCK_CAUSAL_DOCUMENT_GLOBAL = 13   /* same document and floor(j/B) <= floor(i/B):
                                                  block edges at multiples of B from token 0 */
} mad_mask_pattern;

typedef struct {
  int32_t window;          /* SLIDING_WINDOW*, GLOBAL_SLIDING: W (> 0) */
  int32_t prefix;          /* PREFIX_LM: P; < 0 selects floor(T/4) */
  int32_t question;        /* SHARED_QUESTION: question length */
  int32_t n_answers;       /* SHARED_QUESTION: answers split the rest equally, the last takes the remainder */
  int32_t global_len;      /* GLOBAL_SLIDING: G */
  int32_t block;           /* CAUSAL_BLOCKWISE*, BLOCK_CAUSAL_DOCUMENT* block size (> 0) */
  const int32_t* doc_lens; /* *_DOCUMENT: host array of n_docs lengths summing to T;
                              SHARED_QUESTION: optional n_docs answer lengths summing to
                              T - question, used instead of the equal split (the sampled
                              answer lengths of LongCA-bench appendix A.4) */
  int32_t n_docs;
} mad_mask_params;

/* Build the slice list of a static pattern over a square T x T mask.
 * out may be NULL to query the count; otherwise it must hold cap slices.
 * *n_out receives the number of slices.  Host only; launches nothing. */
mad_status mad_mask_slices(int32_t pattern, int32_t T, const mad_mask_params* params,
                           mad_slice* out, int64_t cap, int64_t* n_out);

/* Slices of a batch of packed variable-length sequences (the varlen layout
 * of LongCA-bench section 2.1.1: sequences of different lengths packed into
 * one token stream), given cumulative offsets cu_q[0..batch] and
 * cu_k[0..batch] (cu_q[0] = cu_k[0] = 0, non-decreasing): query tokens
 * [cu_q[b], cu_q[b+1]) attend keys [cu_k[b], cu_k[b+1]) of the same
 * sequence only.  causal = 0: every key of the sequence.  causal = 1: with
 * local offsets r = i - cu_q[b], c = j - cu_k[b] and lengths Lq, Lk, the key
 * is allowed when c <= r (bottom_right = 0, top-left alignment, the slices'
 * own convention) or c <= r + Lk - Lq (bottom_right = 1: the last query sees
 * the last key, the usual convention for a query chunk that continues a
 * longer key stream).  window W > 0 (causal only) further requires
 * r - c < W (top-left) or r + Lk - Lq - c < W (bottom-right; rejected when
 * some sequence has Lk > Lq, a shape the slice vocabulary cannot express).
 * Tq = cu_q[batch], Tk = cu_k[batch] are the sizes to compile with.
 * out / cap / n_out as in mad_mask_slices.  Host only. */
mad_status mad_varlen_slices(const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int32_t causal,
                             int32_t window, int32_t bottom_right, mad_slice* out, int64_t cap, int64_t* n_out);

/* One GPU's share of a context-parallel ring step (LongCA-bench section 2.3
 * and the notes' key design 3).  The causal sequence of n_ranks * chunk tokens
 * is split over n_ranks ranks; layout 0 = contiguous (rank r holds chunk r),
 * layout 1 = head-tail (2 * n_ranks halves; rank r holds halves r and
 * 2 * n_ranks - 1 - r, which balances causal work).  The slices describe which
 * local queries of `rank` see which local keys received from rank `source`,
 * in the two ranks' local coordinates.  chunk must be even for head-tail. */
mad_status mad_ring_step_slices(int32_t layout, int32_t n_ranks, int32_t chunk, int32_t rank,
                                int32_t source, mad_slice* out, int64_t cap, int64_t* n_out);

/* Dynamic block-sparse masks (LongCA-bench appendix A.2: block partition,
 * block scores, top-k key blocks per query block).  scores is a host array
 * [n_groups][n_qb][n_kb] of fp32 block scores; for each (group, query block)
 * the k = n_kb - floor(sparsity_pct * n_kb / 100) (at least 1) highest
 * scoring key blocks are kept, equal scores preferring the lower block index.
 * keep receives a host bitmap [n_groups][n_qb][ceil(n_kb / 64)] of uint64
 * words, bit (kb % 64) of word kb / 64.  sparsity_pct is in [0, 100]. */
mad_status mad_block_topk(const float* scores, int32_t n_groups, int32_t n_qb, int32_t n_kb,
                          int32_t sparsity_pct, uint64_t* keep);

/* ---------------------------------------------------------------------------
 * Plans.  A plan is the compiled mask: for each kernel tiling it sorts every
 * Q x K tile into EMPTY (skipped), FULL (no mask arithmetic) or PARTIAL
 * (per-element mask), and holds per-query-tile lists of key tiles (used by
 * the forward and dQ kernels) and per-key-tile lists of query tiles (used by
 * the dK/dV kernel).  A tile is judged on its in-range elements only.  Plans
 * are immutable after mad_plan_upload and may be shared across streams.
 * ------------------------------------------------------------------------- */
typedef struct mad_plan mad_plan;

/* Compile n slices for a Tq x Tk mask (LongCA-bench section 2.1 "Data
 * preparation": one interface for every mask pattern and for packed
 * variable-length sequences; section 2.2 "Attention kernel": each kernel's
 * inputs come from one unified representation; appendix A.3, FlexAttention:
 * a block mask that compiles into a dense O(S^2) array costs most of the
 * memory, so this plan is O(tiles + slices)).
 *   slices: host array of n mad_slice (n = 0 gives an all-EMPTY mask); each
 *     must satisfy 0 <= q0 <= q1 <= Tq, 0 <= k0 <= k1 <= Tk, a known type,
 *     window >= 0, and window == 0 on FULL slices.
 *   out: receives a plan owned by the caller (release with mad_plan_destroy).
 * Host only: call mad_plan_upload before attention calls.  Errors:
 * MAD_ERR_INVALID for a bad slice or size (nothing is allocated),
 * MAD_ERR_NOMEM if host memory runs out. */
mad_status mad_mask_compile(const mad_slice* slices, int64_t n, int32_t Tq, int32_t Tk,
                            mad_plan** out);

/* Compile a block-sparse mask (LongCA-bench appendix A.2 "Block-sparse
 * mask generation": the attention map cut into a grid of query and key
 * blocks, uniform or of variable sizes, a top-k key-block set per query
 * block, one set per head under MHA and per KV-head group under GQA;
 * appendix A.3 and A.5.2: FlashInfer's per-element metadata and
 * FlexAttention's O(S^2) block mask run out of memory at long sequences and
 * small blocks, so the plan holds the bitmap and per-tile lists only).
 *   q_edges (n_qb + 1 entries), k_edges (n_kb + 1): host int32, strictly
 *     increasing block boundaries from 0 to Tq and Tk.
 *   keep: host uint64 bitmap of mad_block_topk, [n_groups][n_qb][ceil(n_kb/64)].
 * Query head h uses mask group h / (Hq / n_groups), so n_groups = Hkv shares
 * one keep set per GQA group and n_groups = Hq (MHA) gives one per head.
 * Host only; the plan is owned by the caller.  Errors: MAD_ERR_INVALID for
 * bad edges or sizes, MAD_ERR_NOMEM if host memory runs out. */
mad_status mad_sparse_plan(int32_t n_groups, const int32_t* q_edges, int32_t n_qb,
                           const int32_t* k_edges, int32_t n_kb, const uint64_t* keep,
                           mad_plan** out);

/* The same compilation on the GPU, for a keep bitmap already in device
 * memory (mad_block_mask's output: a dynamic mask of LongCA-bench appendix
 * A.2 / A.3 that changes every step), so the bitmap never travels to the
 * host.  The plan is identical to mad_sparse_plan's over the same edges and
 * bits (visit lists, aux words, longest-first orders, pair and tile counts)
 * and is already uploaded to the current device (mad_plan_upload is a
 * no-op for it).
 *   q_edges / k_edges: host int32, as for mad_sparse_plan.
 *   keep: device uint64 [n_groups][n_qb][ceil(n_kb / 64)], 8-byte aligned;
 *     read by kernels queued on `stream` (bits past n_kb are ignored).
 * Runs its kernels on `stream` and synchronises it once (the plan's device
 * block is sized from the list lengths), then queues the list fill: the
 * caller uses the plan on the same stream, or synchronises first.  The
 * plan owns its device memory (two allocations) until mad_plan_destroy.
 * mad_plan_export works on it (it copies the group's lists back).
 * Invalid arguments return an error before anything is launched. */
mad_status mad_sparse_plan_device(int32_t n_groups, const int32_t* q_edges, int32_t n_qb,
                                  const int32_t* k_edges, int32_t n_kb, const uint64_t* keep,
                                  hipStream_t stream, mad_plan** out);

/* Measurement aid: n_workgroups workgroups of 4 waves each issue 4 * iters
 * back-to-back bf16 MFMAs (v_mfma_f32_32x32x16_bf16, 32768 FLOP each) on
 * register operands, with no memory traffic, so timing the launch gives the
 * matrix cores' sustained rate at the clock they hold under that load.
 * sink: device float [n_workgroups], written (one value per workgroup). */
mad_status mad_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream);

/* The raw visit lists of tiling `which` as the kernels read them (for
 * inspection and tests): ptr [n_ptr = n_groups * (n_major + 1)] absolute
 * offsets, ent / ent_aux [n_ent] (entry = minor tile | 1 << 31 for PARTIAL;
 * aux = slice-list offset (slice masks) or FULL-strip bits / -1 (block
 * masks)), order [n_order = n_major] longest first.  Any output may be NULL;
 * n_* receive the sizes.  Host buffers; a GPU-compiled plan is copied back
 * from the device (synchronously). */
mad_status mad_plan_lists(const mad_plan* plan, int32_t which, int64_t* n_ptr, int64_t* n_ent,
                          int64_t* n_order, int32_t* ptr, int32_t* ent, int32_t* ent_aux, int32_t* order);

/* Copy the plan's metadata to the current device (allocates device memory
 * owned by the plan; synchronises `stream`).  Idempotent. */
mad_status mad_plan_upload(mad_plan* plan, hipStream_t stream);

/* Plan statistics (LongCA-bench appendix A.4: throughput is reported in
 * FLOPS; the effective count takes only the unmasked (query, key) pairs, so
 * it needs the exact pair count of the mask).
 *   pairs_per_group: host int64 [n_groups] (may be NULL), the exact number of
 *     allowed (i, j) pairs of each mask group;
 *   n_full / n_partial / n_empty: host int64 (each may be NULL), the tile-class
 *     counts of tiling `which` (0 = forward/dQ tiling, 1 = dK/dV tiling) summed
 *     over groups.
 * Reads host metadata only (a GPU-compiled plan keeps its counts on the host).
 * Errors: MAD_ERR_INVALID for a NULL plan or a tiling other than 0 / 1. */
mad_status mad_plan_stats(const mad_plan* plan, int32_t which, int64_t* pairs_per_group,
                          int64_t* n_full, int64_t* n_partial, int64_t* n_empty);

/* Device bytes the plan holds after mad_plan_upload (0 before): the only
 * device memory the attention calls use beyond the caller's tensors and
 * workspace (LongCA-bench appendix A.4.2 and A.5.2 report peak memory; the
 * mask representation is where FlexAttention spends most of it). */
mad_status mad_plan_device_bytes(const mad_plan* plan, size_t* bytes);

/* Plan shape: Tq, Tk, number of mask groups, and tile sizes (BM query rows x
 * BN keys) with tile-grid size of tiling `which`: 128 x 64 for tiling 0
 * (forward, dQ); 64 x 128 for tiling 1 (dK/dV), or 64 x 64 for block-sparse
 * plans whose interior key-block edges are not all multiples of 128 (64-token
 * or variable blocks).  Any out pointer may be NULL. */
mad_status mad_plan_info(const mad_plan* plan, int32_t which, int32_t* Tq, int32_t* Tk,
                         int32_t* n_groups, int32_t* BM, int32_t* BN, int32_t* n_qt,
                         int32_t* n_kt);

/* Export tiling `which` for mask group `group` to host arrays, for
 * inspection and tests (LongCA-bench section 2.2: one representation the
 * kernel inputs come from; section 3.1: a column-wise mask representation
 * such as FlashMask's cannot express every pattern, which per-tile classes
 * and visit lists do):
 *   classes [n_qt * n_kt] (0 EMPTY, 1 FULL, 2 PARTIAL, row-major by query tile),
 *   csr_ptr [n_qt + 1] / csr_idx [entries] (ascending key tiles per query tile),
 *   csc_ptr [n_kt + 1] / csc_idx [entries] (ascending query tiles per key tile).
 * Any output may be NULL; list lengths equal the number of non-EMPTY tiles
 * (size the arrays with mad_plan_info and a first call for the ptr arrays).
 * Errors: MAD_ERR_INVALID for a NULL plan, a bad tiling or group; a
 * GPU-compiled plan is copied back synchronously (MAD_ERR_HIP on failure). */
mad_status mad_plan_export(const mad_plan* plan, int32_t which, int32_t group, uint8_t* classes,
                           int64_t* csr_ptr, int32_t* csr_idx, int64_t* csc_ptr, int32_t* csc_idx);

void mad_plan_destroy(mad_plan* plan);

/* ---------------------------------------------------------------------------
 * Attention.  strides (may be NULL = packed) gives, in elements, the token
 * and head strides of q, k and v: {q_tok, q_head, k_tok, k_head, v_tok,
 * v_head}; the head dimension must be contiguous and every row 16-byte
 * aligned.  o, d_o, dq are packed [Tq, Hq, d]; dk, dv packed [Tk, Hkv, d];
 * lse is [Hq, Tq].  d must be 64, 128 or 256; Hq % Hkv == 0; the plan must have
 * been compiled for (Tq, Tk), uploaded, and have n_groups dividing Hq.
 * ------------------------------------------------------------------------- */

/* Device workspace of mad_attn_fwd (optional): the counters through which
 * the kernel's workgroups claim their work items (64 bytes used). */
#define MAD_FWD_WORKSPACE_BYTES 256

/* Forward: O = softmax(scale * Q K^T + mask) V and LSE (LongCA-bench
 * section 1: standard softmax attention).  Tiled with an online softmax;
 * only non-EMPTY tiles are visited and only PARTIAL tiles evaluate the mask.
 *   q, k, v: device bf16, [Tq, Hq, d] and [Tk, Hkv, d] with the strides
 *     above; o: device bf16 [Tq, Hq, d] packed; lse: device fp32 [Hq, Tq]
 *     (natural log; -inf, with O = 0, for rows that see no key).
 *   workspace: NULL, or device memory of at least MAD_FWD_WORKSPACE_BYTES,
 *     256-byte aligned, owned by the caller, contents on entry irrelevant.
 *     With it, workgroups claim work items from per-XCD queues and the
 *     faster XCDs take over the slower ones' last items (the XCDs run at
 *     different speeds); without it each workgroup takes a fixed item.  The
 *     result is the same either way.  Calls that may overlap on the GPU
 *     (other streams) must not share a workspace.
 * Errors: MAD_ERR_INVALID for a NULL plan, mismatched shapes, NULL o / lse
 * (Tq > 0), a NaN scale or a short workspace; MAD_ERR_UNSUPPORTED for
 * misaligned pointers or strides or an unsupported head dim; MAD_ERR_HIP for
 * a failed launch. */
mad_status mad_attn_fwd(const mad_plan* plan, const void* q, const void* k, const void* v,
                        void* o, float* lse, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv,
                        int32_t d, const int64_t* strides, float scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace mad_attn_bwd needs (LongCA-bench section 3.2:
 * the backward is the harder pass and only some kernels have one; appendix
 * A.4.2: peak memory is a metric of its own, and this workspace is all the
 * backward uses beyond its inputs and outputs): two fp32 [Hq][Tq rounded up
 * to 128] arrays holding -D (D = rowsum(dO * O)) and -LSE / scale per row
 * (-inf for rows with no allowed key and for padding rows), and, when the
 * plan's key-tile columns are uneven enough that the dK/dV kernel cuts the
 * longest ones between several workgroups (mad_bwd_kv_splits > 1), two fp32
 * [Tk][Hkv][d] sums for dK and dV; last, 256 bytes of counters through
 * which the dQ kernel's workgroups claim their work items (the XCDs run at
 * different speeds, and the faster ones take over the slower ones' last
 * items; the counters are cleared on the stream before each use).  Depends
 * on the plan and on the compute
 * units of the current device, so query it per plan.  Host only; launches
 * nothing.  Errors: MAD_ERR_INVALID for NULL arguments or bad sizes,
 * MAD_ERR_UNSUPPORTED for a head dim other than 64 / 128 / 256. */
mad_status mad_bwd_workspace_bytes(const mad_plan* plan, int32_t Tq, int32_t Tk, int32_t Hq,
                                   int32_t Hkv, int32_t d, size_t* bytes);

/* Workgroups per key-tile column that the backward's dK/dV kernel uses for
 * this plan and head layout (LongCA-bench section 3.2, the backward).  1: each
 * key tile's dK / dV is accumulated by one workgroup and stored as bf16
 * directly (bit-reproducible).  S > 1 (at most 8): the columns are cut into S
 * chunks whose fp32 partial sums are added atomically into the workspace and
 * rounded by a second kernel; chosen when the longest column holds more than
 * half of one compute unit's average share of the items, read against the
 * current device's compute-unit count (256 on MI355X, also the value used
 * when no device is visible).  Host only; launches nothing.
 *   splits: receives S.
 * Errors: MAD_ERR_INVALID for NULL arguments, Hq % Hkv != 0 or mask groups
 * that do not divide Hq. */
mad_status mad_bwd_kv_splits(const mad_plan* plan, int32_t Hq, int32_t Hkv, int32_t* splits);

/* Backward of the forward above (LongCA-bench section 3.2: the backward pass
 * is the common bottleneck and several sparse kernels have none; section
 * 2.3: a ring step's backward takes the merged O and LSE) for upstream
 * gradient d_o, given o and lse (normally the forward's; for a ring step the
 * merged global ones, so the step's share of the global gradient is
 * produced).  Runs the delta pre-pass D = rowsum(d_o * o) (and LSE / scale)
 * into the workspace, then the dK/dV kernel and the dQ kernel.
 *   q, k, v: as for mad_attn_fwd (strided views allowed).
 *   o, d_o, dq: device bf16 [Tq, Hq, d] packed; dk, dv: device bf16
 *     [Tk, Hkv, d] packed; lse: device fp32 [Hq, Tq].  All 16-byte aligned
 *     (lse 4-byte).  dq, dk, dv are overwritten; dK / dV rows of keys no
 *     query sees are set to 0.
 *   workspace: device, 256-byte aligned, at least mad_bwd_workspace_bytes
 *     long, owned by the caller; its contents on entry do not matter.
 * q/k/v/o/d_o/lse are not modified.  Results are bit-reproducible, except
 * dk/dv of plans whose columns are cut (mad_bwd_kv_splits > 1: their fp32
 * partial sums are added in arrival order).  Errors as for mad_attn_fwd, plus
 * MAD_ERR_INVALID for a missing or undersized workspace. */
mad_status mad_attn_bwd(const mad_plan* plan, const void* q, const void* k, const void* v,
                        const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                        void* dv, void* workspace, size_t workspace_bytes, int32_t Tq,
                        int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d, const int64_t* strides,
                        float scale, hipStream_t stream);

/* The same backward with no workspace argument and no allocation of any kind,
 * for callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The workspace is a static device array of MAD_STATIC_WORKSPACE_BYTES
 * (64 MiB) built into the library: every GPU the library runs on holds its own
 * copy from the library's first use on that device until the process ends.
 * Calls that need more workspace than that (mad_bwd_workspace_bytes: about
 * 8 bytes per query row and head, plus the fp32 dK / dV sums of cut columns)
 * return MAD_ERR_UNSUPPORTED before anything is launched.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents (the
 * kernels rewrite or zero every byte they read, so stale contents do not
 * matter): calls that overlap on one GPU -- on different streams, or from
 * different threads -- race on it and must be serialised by the caller.
 * Arguments, outputs and errors as for mad_attn_bwd; the first call on a
 * device looks up the array's device address (MAD_ERR_HIP on failure). */
#define MAD_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
mad_status mad_attn_bwd_static(const mad_plan* plan, const void* q, const void* k, const void* v,
                               const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                               void* dv, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d,
                               const int64_t* strides, float scale, hipStream_t stream);

/* The same backward, restricted to a subset of its three launches:
 * phases is a bit set of MAD_BWD_DELTA (the delta pre-pass), MAD_BWD_DKDV and
 * MAD_BWD_DQ (which read the workspace's delta rows).  Calling the three
 * phases in that order on one stream is equivalent to mad_attn_bwd; single
 * phases let a caller time each kernel on its own. */
enum { MAD_BWD_DELTA = 1, MAD_BWD_DKDV = 2, MAD_BWD_DQ = 4, MAD_BWD_ALL = 7 };
mad_status mad_attn_bwd_phases(const mad_plan* plan, const void* q, const void* k, const void* v,
                               const void* o, const void* d_o, const float* lse, void* dq, void* dk,
                               void* dv, void* workspace, size_t workspace_bytes, int32_t Tq,
                               int32_t Tk, int32_t Hq, int32_t Hkv, int32_t d, const int64_t* strides,
                               float scale, uint32_t phases, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dynamic block-sparse masks computed on the GPU from Q and K: the coarse
 * stage of a block-sparse method (LongCA-bench appendix A.3: VSA mean-pools
 * the QK scores over blocks) followed by appendix A.2's top-k key blocks per
 * query block.  For mask group g (n_groups groups of Hq / n_groups query
 * heads; a group's heads must share one KV head, so n_groups must be a
 * multiple of Hkv), query block qb and key block kb:
 *   score = scale * (mean of Q over qb's rows and g's heads) . (mean of K over kb's rows)
 * which equals scale times the mean of q_i . k_j over the block pair and the
 * group's heads.  Each (g, qb) keeps its k = n_kb - floor(sparsity_pct * n_kb
 * / 100) (at least 1) highest-scoring key blocks, equal scores in ascending
 * key-block order (the order mad_block_topk uses).
 *   q [Tq, Hq, d], k [Tk, Hkv, d]: device bf16, packed, 16-byte aligned.
 *   q_edges (n_qb + 1) / k_edges (n_kb + 1): device int32, strictly increasing
 *     from 0 to Tq / Tk (as for mad_sparse_plan); n_kb <= 8192.
 *   workspace: device, mad_block_mask_workspace_bytes bytes, 256-byte aligned.
 *   keep: device uint64 [n_groups][n_qb][ceil(n_kb / 64)], fully written; the
 *     host copy of it is what mad_sparse_plan takes.
 *   scores: optional device fp32 [n_groups][n_qb][n_kb] (NULL: not written).
 * Runs on `stream`, allocates nothing; invalid arguments return an error
 * before anything is launched.
 * ------------------------------------------------------------------------- */
mad_status mad_block_mask_workspace_bytes(int32_t n_groups, int32_t Hkv, int32_t n_qb, int32_t n_kb,
                                          int32_t d, size_t* bytes);

mad_status mad_block_mask(const void* q, const void* k, int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv,
                          int32_t d, int32_t n_groups, const int32_t* q_edges, int32_t n_qb,
                          const int32_t* k_edges, int32_t n_kb, int32_t sparsity_pct, float scale,
                          void* workspace, size_t workspace_bytes, uint64_t* keep, float* scores,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Log-sum-exp merge of partial attention results (LongCA-bench section 2.3
 * and the notes' key design 3: ring context parallelism combines, per query
 * row, the outputs that one rank's queries get from each key chunk).  With
 * the keys of a row split into disjoint parts t, each giving O_t and LSE_t
 * over its own keys:
 *   LSE = ln sum_t exp(LSE_t),   O = sum_t exp(LSE_t - LSE) O_t.
 * Parts with LSE_t = -inf weigh zero; a row whose parts are all -inf gets
 * O = 0 and LSE = -inf.
 *   n_parts    1..32.
 *   o_parts    host array of n_parts device pointers, each bf16 [Tq, Hq, d]
 *              packed, 16-byte aligned.
 *   lse_parts  host array of n_parts device pointers, each fp32 [Hq, Tq].
 *   o, lse     outputs in the same layouts; o may alias o_parts[t] and lse
 *              may alias lse_parts[t] (every element is read before it is
 *              written by the same thread).
 *   d          64, 128 or 256.
 * Arithmetic in fp32, O rounded to bf16.  Runs on `stream`; allocates
 * nothing.  Invalid arguments return MAD_ERR_INVALID / MAD_ERR_UNSUPPORTED
 * before anything is launched.
 * ------------------------------------------------------------------------- */
mad_status mad_lse_merge(int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                         void* o, float* lse, int32_t Tq, int32_t Hq, int32_t d, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One rank's share of ring context-parallel attention, run on one GPU
 * (LongCA-bench section 2.3, the notes' key designs 3 and 4).  The causal
 * sequence of n_ranks * chunk tokens is split over n_ranks ranks in the given
 * layout (as in mad_ring_step_slices); this object computes what rank `rank`
 * computes over the n_ranks ring steps, with the K/V chunks that would arrive
 * from the other ranks taken from a global K/V held on this GPU:
 *   forward: for each step with a non-empty mask, the source's K/V chunk is
 *     staged into one of two buffers on a copy stream (the copy of step i+1
 *     overlaps the kernels of step i), the forward kernel gives (O_t, LSE_t)
 *     for the local queries, and one LSE merge gives the rank's O and LSE;
 *   backward: with the merged O / LSE (the pages' rule for ring backward),
 *     the delta pre-pass runs once, then per step the dK/dV and dQ kernels;
 *     dQ is accumulated in fp32 over the steps and rounded once, and each
 *     step's dK / dV (this rank's contribution to the source's keys) is
 *     written at the source chunk's global position.
 * Creation compiles one mask plan per step, uploads them to the current
 * device and allocates every device buffer (K/V staging, per-step partial
 * outputs, the dQ accumulator, the backward workspace); the fwd / bwd calls
 * allocate nothing.
 *   layout     0 = contiguous, 1 = head-tail (chunk even).
 *   Hq, Hkv, d GQA heads (Hq % Hkv == 0) and head dim (64, 128 or 256).
 * Tensors (device, bf16, packed, 16-byte aligned): q, o, d_o, dq [chunk, Hq, d]
 * (the rank's local rows: contiguous -> global rows [rank*chunk, +chunk);
 * head-tail -> halves rank and 2*n_ranks-1-rank of chunk/2 rows each);
 * k, v, dk, dv [n_ranks*chunk, Hkv, d] in global order; lse fp32 [Hq, chunk].
 * dk / dv rows of chunks no step of this rank reads are set to 0.  The
 * object's buffers are reused by every call: calls on one object must not
 * overlap.
 * ------------------------------------------------------------------------- */
typedef struct mad_ring mad_ring;

mad_status mad_ring_create(int32_t layout, int32_t n_ranks, int32_t chunk, int32_t rank, int32_t Hq,
                           int32_t Hkv, int32_t d, mad_ring** out);

/* Number of non-empty steps, unmasked (query, key) pairs per head summed over
 * them, and the device bytes the object holds. */
mad_status mad_ring_info(const mad_ring* ring, int32_t* n_steps, int64_t* pairs_per_head,
                         size_t* device_bytes);

mad_status mad_ring_fwd(mad_ring* ring, const void* q, const void* k, const void* v, void* o, float* lse,
                        float scale, hipStream_t stream);

mad_status mad_ring_bwd(mad_ring* ring, const void* q, const void* k, const void* v, const void* o,
                        const void* d_o, const float* lse, void* dq, void* dk, void* dv, float scale,
                        hipStream_t stream);

void mad_ring_destroy(mad_ring* ring);

/* Message describing the last failure on the calling thread ("" if none). */
const char* mad_last_error(void);

/* Library version string. */
const char* mad_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAD_H_ */
