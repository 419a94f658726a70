/*
 * csa.h -- C ABI of the MI355X (gfx950) library for one layer of hybrid
 * compressed attention: CSA (compressed sparse attention) and HCA (heavily
 * compressed attention), decode and prefill.
 *
 * Sources (web pages summarising the DeepSeek-V4 technical report):
 *   [W1] "DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *        Intelligence" (awesome-system-papers.pages.dev), "核心方法 / Hybrid
 *        CSA + HCA Attention", "关键观察" observation 1.
 *   [W2] "DeepSeek-V4 深读" (ricardokevins.github.io), spec table "模型全貌",
 *        "CSA：4× 压缩之后再 top-k" with the compression equation and Fig. 2,
 *        "HCA：128× 压缩后保留 dense 全局视野", the stability-details paragraph,
 *        "FP4 QAT、可恢复 rollout".
 *   [W3] "AI深一度 第15期|DeepSeek V4" (yeyulingfeng.com), sections 一 and 二.
 *   [W4] "DeepSeek-V4 论文解读" (researchpapers.dev), section "注意力栈".
 *   [W5] "拆解 DeepSeekv4" (daixd5520.github.io), sections CSA, HCA, 细节.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains them.  Strides are in BYTES.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the device or copies to the host.
 *   - Arguments are validated on the host before any launch; on a validation
 *     failure nothing is launched and a negative status is returned.
 *   - Status: CSA_OK (0); CSA_EINVAL (-1) null pointer, misaligned pointer or
 *     inconsistent shape; CSA_EUNSUPPORTED (-2) a shape or format combination
 *     this library has no kernel for; CSA_EHIP (-3) a launch error reported by
 *     the HIP runtime; CSA_EWORKSPACE (-4) workspace missing or too small;
 *     CSA_ESCRATCH (-5) a problem too large for csa_index_topk_noalloc.
 *   - Deterministic: for a fixed input and shape the results are bitwise
 *     reproducible; no kernel uses order-dependent floating-point atomics.
 *   - Thread-safe: the library's only mutable global state is the table of
 *     per-device scratch addresses of csa_index_topk_noalloc, filled once per
 *     device under a lock.  Calls that share a workspace (or, for the
 *     allocation-free entry point, a GPU) must be ordered on one stream by
 *     the caller.
 *   - Positions are absolute token positions (int64).  Token p of a
 *     sequence is the p-th token of its context, starting at 0.
 *
 * Formats (CSA_FMT_*)
 *   F32        every element fp32 (the precision-check mode).
 *   FP8_BF16   main KV entry of d dims: dims [0, d - d_rope) as OCP FP8 E4M3FN
 *              (round-to-nearest-even, saturating, no scale) in the `nope`
 *              array, the last d_rope dims as BF16 in the `rope` array [W2
 *              stability paragraph; W3 section 二].  With d = 512, d_rope = 64
 *              an entry is 448 + 128 = 576 bytes; a packed cache row places
 *              `rope` at byte 448 of a 576-byte row (stride 576 for both).
 *   MXFP4      OCP MX v1.0 FP4: per row, d/2 bytes of E2M1 codes (element 2j
 *              in the low nibble of byte j) and d/32 E8M0 scale bytes, one per
 *              block of 32 elements [W2 "FP4 QAT" section: the indexer QK path
 *              runs in FP4].  Scale = 2^(floor(log2(amax)) - 2); elements
 *              round-to-nearest-even and clamp to +-6.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 3

enum {
  CSA_OK = 0,
  CSA_EINVAL = -1,
  CSA_EUNSUPPORTED = -2,
  CSA_EHIP = -3,
  CSA_EWORKSPACE = -4,
  CSA_ESCRATCH = -5
};

/* Device bytes of the scratch array behind csa_index_topk_noalloc (per GPU). */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum { CSA_FMT_F32 = 0, CSA_FMT_FP8_BF16 = 1, CSA_FMT_MXFP4 = 2 };
enum { CSA_DT_F32 = 0, CSA_DT_BF16 = 1 };
enum { CSA_OP_COMPRESS = 0, CSA_OP_INDEX_TOPK = 1, CSA_OP_ATTEND = 2, CSA_OP_HCA_ATTEND = 3 };

/* Attention flags. */
enum {
  CSA_ATTEND_NORM_Q = 1,      /* RMS-normalise every query head first (weight 1, eps 1e-6) */
  CSA_ATTEND_NO_INV_ROPE = 2, /* skip the inverse output rotation (test hook) */
  /* Batch-invariant mode ["DeepSeek-V4 深读", 系统基础设施, batch invariance:
   * a token's result must not depend on its position in, or the size of,
   * the batch].  The key/value list of every query is split into pieces of a
   * fixed length (CSA_INVARIANT_SPLIT_ROWS rows), whatever B and n_q are, so
   * a query's output and LSE are bitwise the same alone, inside any batch and
   * as one row of a prefill chunk.  Without it the split count follows B and
   * n_q (to fill the GPU), and calls with several queries and a multiple of
   * 128 heads run a kernel that serves 128 heads per workgroup; both change
   * the order of the fp32 sums. */
  CSA_ATTEND_BATCH_INVARIANT = 4,
  /* The window buffer is a per-request ring (the state cache of the paged
   * layout below): position p sits at row p % win_len, and the ring holds
   * positions win_pos0[b] .. win_pos0[b] + win_len - 1 (older rows have been
   * overwritten); with win_pos0 NULL a query at position t finds positions
   * max(0, t - win_len + 1) .. t there (decode: the newest token's row has
   * just been stored).  Without the flag position p sits at row
   * p - win_pos0[b]. */
  CSA_ATTEND_WIN_RING = 8
};
#define CSA_INVARIANT_SPLIT_ROWS 1024

/* Index flags. */
enum {
  /* Batch-invariant mode: every call scores with the exact per-head form
   * (see csa_index_topk), whatever n_q is, so a query's scores and selection
   * are bitwise the same in a decode call, inside any batch and as one row
   * of a prefill chunk.  Costs speed at prefill. */
  CSA_INDEX_BATCH_INVARIANT = 1,
  /* BF16 index scores ["DeepSeek-V4 深读", FP4 QAT section: index scores
   * kept in BF16 instead of FP32 make the top-k selector about twice as fast
   * and keep 99.7% of the selected entries].  Every score is rounded to BF16
   * (nearest even) before it is stored and selected on; selection then
   * follows the same rule on the rounded scores (ties, now more frequent,
   * go to the lower index).  out_score, when given, receives the BF16 codes
   * (2 bytes per score, same [B][n_q][n_cap] layout). */
  CSA_INDEX_BF16_SCORES = 2
};

/*
 * ---------------------------------------------------------------- paged layout
 * Heterogeneous KV cache [W1 "关键观察" observation 3 and "训练与推理基础设施"
 * (异构 KV); W2 "异构 KV cache 与磁盘前缀复用" and Fig. 5]: the layers' caches
 * grow at different rates (one CSA entry and one indexer key per 4 tokens,
 * one HCA entry per 128, window rows per token), so one block size in tokens
 * cannot serve them all.  Compressed entries live in a classical block cache
 * whose blocks cover lcm(4, 128) = 128 raw tokens each: 32 CSA main entries,
 * 32 indexer keys or 1 HCA entry per block of a layer's pool; the sliding
 * window and the not-yet-compressed tail of every request live in a
 * fixed-size per-request state cache (rings).
 *
 * Block tables.  An op that takes `block_table` (int32 [B][bt_stride], device)
 * reads or writes entry i of sequence b in physical block
 * blk = block_table[b * bt_stride + i / block_rows], at row i % block_rows of
 * that block: byte offset (blk * block_rows + i % block_rows) * row_stride
 * from the base pointer of each array (the pool), for every array of the
 * call with its own row stride; the per-sequence stride is then unused.
 * bt_stride * block_rows must cover the op's entry capacity (n_cap).  A
 * block id outside [0, pool_blocks) marks an unallocated block: attention
 * skips its entries, the indexer reads its keys as zero, compression skips
 * its stores.  Block tables must not change while a call that reads them
 * runs.
 *
 * Rings.  csa_compress reads its inputs from rings of `in_ring` rows
 * (position p at row p % in_ring) and the attention reads the window from a
 * ring with CSA_ATTEND_WIN_RING: the state cache.
 */

/*
 * ---------------------------------------------------------------- csa_compress
 * Softmax-gated, position-biased pooling of every m tokens into one entry
 * [W2 compression equation; W3 section 一; W4 注意力栈]:
 *
 *   C_i[c] = sum_{j=mi}^{mi+m-1} S_j[c] C^a_j[c] + sum_{j=m(i-1)}^{mi-1} S_j[c] C^b_j[c]
 *
 * where S is, for every channel c separately, the softmax over all the
 * candidates of entry i of the logits Z^a_j[c] + B^a[j-mi][c] (a-branch) and
 * Z^b_j[c] + B^b[j-m(i-1)][c] (b-branch).  The b-branch exists only with
 * `overlap` (CSA, m = 4) and only for i >= 1; HCA (m = 128) has no overlap
 * [W2 HCA section].  Then, per entry: optional RMSNorm over the d channels
 * (weight 1, `rms_eps`) [W2 stability paragraph], optional RoPE of the last
 * d_rope channels at position m*i (pairs (2u, 2u+1), angle
 * m*i * theta^(-2u/d_rope)) [W1; W2 spec table], and storage in `out_fmt`.
 *
 * Row r of every input holds the token at absolute position pos0 + r for all
 * B sequences (pos0 a multiple of m).  The call writes exactly the entries
 * i in [i_first, i_end):
 *     i_first = pos0/m + (overlap && pos0 > 0 ? 1 : 0),  i_end = (pos0 + n_rows)/m
 * i.e. every complete block whose candidates are all present; with overlap
 * and pos0 > 0 the first m rows only feed the b-branch.  Entry i lands at
 * byte offset (i - out_row0) * out_stride (+ b * out_seq_stride) of each
 * output array: out_row0 = 0 lets the outputs point at the base of a
 * caller-owned cache; a window buffer that starts at position p0 passes
 * out_row0 = p0 (i_first >= out_row0 is required).
 *
 * m = 1 with NULL gates and biases is the raw-window store: every row
 * becomes entry pos0 + r after norm / rotation / storage.
 *
 *   in_dtype   CSA_DT_F32 or CSA_DT_BF16 for kv_* and gate_*.
 *   kv_a/gate_a, kv_b/gate_b  [B][n_rows][d] at in_row_stride / in_seq_stride
 *              bytes; gate_* NULL means logit 0; kv_b/gate_b must be NULL
 *              without overlap and kv_b non-NULL with it.
 *   bias_a, bias_b  fp32 [m][d] contiguous, or NULL (bias 0).
 *   out_fmt F32:      out0 = fp32 [d] per entry.
 *   out_fmt FP8_BF16: out0 = E4M3FN bytes [d - d_rope], out1 = BF16 [d_rope].
 *   out_fmt MXFP4:    out0 = E2M1 codes [d/2], out1 = E8M0 scales [d/32]
 *                     (d % 32 == 0, d_rope == 0, do_norm == 0 expected).
 * Constraints: 1 <= m <= 1024, 1 <= d <= 1024, d % 8 == 0, d_rope even and
 * <= d, n_rows >= 0, B >= 1.  n_rows = 0 or no complete block is a no-op.
 *
 * State cache and paged outputs (ABI 3; see "paged layout" above):
 *   in_ring > 0     the inputs are rings: the token at position p is at row
 *                   p % in_ring (the rows of positions pos0 .. pos0 + n_rows - 1
 *                   must be present, so n_rows <= in_ring); in_seq_stride
 *                   separates the sequences' rings.
 *   out_block_table entry i of sequence b is stored in block
 *                   out_block_table[b * out_bt_stride + i / out_block_rows] of
 *                   each output pool, at row i % out_block_rows (out_row0 must
 *                   be 0; the out*_seq_stride are unused); block ids outside
 *                   [0, out_pool_blocks) skip the store.
 *   out_ring > 0    entry i is stored at output row i % out_ring (a window
 *                   ring; out_row0 must be 0, no block table).
 *   seq_pos         per-sequence decode mode: sequence b's newest token is at
 *                   position seq_pos[b] (its rows already in the rings, so
 *                   in_ring > 0 is required: in_ring >= 2m with overlap, >= m
 *                   without); the call stores the one entry that token
 *                   completes, entry (seq_pos[b] + 1)/m - 1 when
 *                   (seq_pos[b] + 1) % m == 0, and nothing for that sequence
 *                   otherwise.  pos0 and n_rows are ignored.  With m = 1 every
 *                   token is an entry: the window-row store.
 * Decode appends one token per step to the rings and compresses a block when
 * it completes: incremental compression, bitwise equal to compressing the
 * whole sequence at once (same kernels, same order of every sum).
 */
typedef struct CsaCompressArgs {
  int32_t B;
  int32_t n_rows;
  int64_t pos0;
  int32_t m;
  int32_t overlap;
  int32_t d;
  int32_t d_rope;
  int32_t in_dtype;
  int32_t out_fmt;
  int32_t do_norm;
  float rms_eps;
  double rope_theta;
  const void* kv_a;
  const void* gate_a;
  const void* kv_b;
  const void* gate_b;
  int64_t in_row_stride;
  int64_t in_seq_stride;
  const float* bias_a;
  const float* bias_b;
  void* out0;
  void* out1;
  int64_t out_row0;
  int64_t out0_stride;
  int64_t out0_seq_stride;
  int64_t out1_stride;
  int64_t out1_seq_stride;
  /* ABI 3: state-cache rings and paged outputs */
  int32_t in_ring;                  /* 0: row r = position pos0 + r; > 0: position p at row p % in_ring */
  int32_t out_block_rows;           /* entries per block of out_block_table */
  const int32_t* out_block_table;   /* NULL: contiguous outputs; else [B][out_bt_stride] block ids */
  int64_t out_bt_stride;            /* int32 elements per sequence in out_block_table */
  int32_t out_pool_blocks;          /* blocks in the output pools */
  int32_t out_ring;                 /* > 0: entry i at output row i % out_ring (no block table) */
  const int64_t* seq_pos;           /* NULL, or device int64 [B]: per-sequence decode mode */
} CsaCompressArgs;

/*
 * ---------------------------------------------------------------- csa_index_topk
 * Lightning indexer and top-k selection [W2 CSA section and Fig. 2; W5 CSA
 * step 2].  For query r of sequence b at position t = q_pos[b][r]:
 *
 *   n_vis = min(floor(t / m), n_entries[b])      (a query never selects the
 *           block that contains it [W1 observation 1; W5 细节])
 *   I_i   = sum_h w[b][r][h] * ReLU(q_I[b][r][h] . k_I[b][i])   for i < n_vis
 *
 * and out_idx[b][r][0 .. top_k) receives the indices of the top_k largest
 * I_i, ties broken toward the lower index, written in ascending index order;
 * with n_vis <= top_k every visible index is written and the rest is -1.
 * Scores are accumulated in fp32 (E2M1 x E2M1 products and 32-element block
 * sums are exact in fp32).  With MXFP4, two or more queries per call and H_I a
 * multiple of 32, the call evaluates w ReLU(s) as (w/2)|s| + (w/2)s and takes
 * the second term, summed over heads, from a 6-component FP8 E4M3 split of
 * u = sum_h (w_h/2) q_h (per 32-dim block, each component carries 4 more
 * bits): such scores (out_score included) differ from the exact ones by at
 * most about 2^-24 sum_blocks max|u| sum|k|, the order of fp32 rounding.
 * One query per call (decode), and every call with CSA_INDEX_BATCH_INVARIANT,
 * uses the exact form.
 *
 *   fmt F32:   q0 = fp32 [B][n_q][H_I][d_I]; k0 = fp32 [B][n_cap][d_I].
 *   fmt MXFP4: q0 = codes [B][n_q][H_I][d_I/2], q1 = scales [B][n_q][H_I][d_I/32];
 *              k0 = codes [B][n_cap][d_I/2],    k1 = scales [B][n_cap][d_I/32].
 *   All four arrays are contiguous in the order shown.
 *   q_pos      device int64 [B][n_q].
 *   n_entries  device int32 [B] entries present per sequence (NULL = n_cap).
 *   w          device fp32 [B][n_q][H_I] head weights (any sign).
 *   out_idx    device int32 [B][n_q][top_k].
 *   out_score  optional device fp32 [B][n_q][n_cap] (BF16 codes with
 *              CSA_INDEX_BF16_SCORES): I_i for i < n_vis, -inf beyond.
 * Constraints: MXFP4 needs d_I == 128 and H_I a multiple of 16 up to 64
 * (the matrix-core path); F32 needs d_I <= 1024; top_k >= 1; n_cap >= 1;
 * m >= 1.
 * Workspace: csa_workspace_bytes(CSA_OP_INDEX_TOPK, &args) bytes of device
 * memory, 256-byte aligned, used by this op only.  It must be zero-filled
 * before its first use; every call leaves its counters and histogram zeroed
 * again, so later calls need no refill (refill after a failed launch).  The
 * call runs its queries in blocks of csa_index_query_block(&args) queries
 * per sequence, so the workspace stays below about 3 GiB at any n_q (with
 * or without out_score).
 * Constraint: n_cap <= 4194304.
 * Paged keys (ABI 3): with block_table, k0 and k1 are the pools' bases and key
 * i of sequence b is row i % block_rows of block block_table[b * bt_stride +
 * i / block_rows] (64-byte code rows and 4-byte scale words with MXFP4,
 * d_I floats with F32); MXFP4 needs block_rows == 32 and pool_blocks <= 2^20.
 * Scores and selections equal those of the contiguous layout bitwise.
 * Timing hook: ev_start / ev_stop, when not NULL, are HIP events the call
 * records on `stream` around its scoring kernel (with several internal query
 * blocks, before the first block's and after the last block's).
 */
typedef struct CsaIndexArgs {
  int32_t B;
  int32_t n_q;
  int32_t m;
  int32_t n_cap;
  int32_t H_I;
  int32_t d_I;
  int32_t fmt;
  int32_t top_k;
  int32_t flags;     /* CSA_INDEX_* */
  int32_t _pad0;
  const int64_t* q_pos;
  const int32_t* n_entries;
  const void* q0;
  const void* q1;
  const float* w;
  const void* k0;
  const void* k1;
  int32_t* out_idx;
  void* out_score;   /* fp32, or BF16 codes with CSA_INDEX_BF16_SCORES */
  void* ev_start;   /* optional hipEvent_t recorded just before the scoring kernel */
  void* ev_stop;    /* optional hipEvent_t recorded just after it (NULL = none) */
  /* ABI 3: paged keys (see "paged layout"); NULL block_table = contiguous */
  const int32_t* block_table;   /* [B][bt_stride] block ids */
  int32_t bt_stride;
  int32_t block_rows;           /* keys per block: 32 with MXFP4 */
  int32_t pool_blocks;          /* blocks in the k0 / k1 pools */
  int32_t _pad1;
} CsaIndexArgs;

/*
 * ---------------------------------------------------------------- csa_attend / hca_attend
 * Shared-KV multi-query attention with a per-head sink [W2 CSA/HCA intro and
 * stability paragraph; W5 细节].  Every entry is both key and value.  For
 * query r of sequence b at t = q_pos[b][r] and head h:
 *
 *   q'   = RoPE_t(RMSNorm(q_h))            (RMSNorm only with CSA_ATTEND_NORM_Q)
 *   KV   = CSA: the compressed entries idx[b][r][*] that are >= 0 and
 *              < n_vis = min(floor(t/m), n_entries[b])   (csa_attend)
 *          HCA: every compressed entry i < n_vis         (hca_attend, idx NULL)
 *          followed by the raw window tokens of positions
 *          max(0, t-n_win+1) .. t that the window buffer holds [W1 sliding
 *          window; W2 Fig. 2 caption: top-k entries concatenated with the window]
 *   s_j  = softmax_scale * q' . kv_j        (softmax_scale 0 => 1/sqrt(d))
 *   o_h  = sum_j e^{s_j} kv_j / (e^{sink[h]} + sum_j e^{s_j})
 *   out  = o_h with its last d_rope dims rotated by -t (skipped with
 *          CSA_ATTEND_NO_INV_ROPE)   [W2: inverse rotation of the output]
 *   lse  = log sum_j e^{s_j} (the sink excluded; -inf with no KV rows)
 *
 *   fmt F32:      q, out fp32; entries / window fp32 rows in kv0 / win0.
 *   fmt FP8_BF16: q, out BF16; entries / window in storage form (nope bytes
 *                 in kv0 / win0, BF16 rope dims in kv1 / win1).
 *   q, out       [B][n_q][H][d] contiguous.
 *   kv*          row i of sequence b at kv*_base + b*kv_seq_stride + i*kv_stride.
 *   win*         position p of sequence b at row p - win_pos0[b] of the window
 *                buffer (rows 0 .. win_len-1, same addressing with win_stride
 *                and win_seq_stride); positions the buffer does not hold are
 *                skipped.
 *   idx          int32 [B][n_q][top_k] (csa_attend); must be NULL for hca_attend.
 *   sink         fp32 [H].
 *   out_lse      optional fp32 [B][n_q][H].
 * Constraints: FP8_BF16 needs d == 512, d_rope == 64, H % 16 == 0 and row
 * strides (kv_stride, win_stride) below 2^31 bytes (CSA_EUNSUPPORTED otherwise);
 * F32 needs d <= 512 and H <= 128.  1 <= n_win, win_len >= 0.
 * Workspace: csa_workspace_bytes(CSA_OP_ATTEND / CSA_OP_HCA_ATTEND, &args).
 * Paged entries (ABI 3): with block_table, kv0 / kv1 are the pools' bases
 * and entry i of sequence b is row i % block_rows of block block_table[b *
 * bt_stride + i / block_rows] (kv_seq_stride unused); entries in blocks
 * outside [0, pool_blocks) are skipped.  With CSA_ATTEND_WIN_RING the window
 * buffer is a ring (see the flag).  Outputs equal those of the contiguous
 * layout bitwise.
 * Timing hook: ev_start / ev_stop, when not NULL, are HIP events the call
 * records on `stream` around its attention kernel.
 */
typedef struct CsaAttendArgs {
  int32_t B;
  int32_t n_q;
  int32_t H;
  int32_t d;
  int32_t d_rope;
  int32_t m;
  int32_t fmt;
  int32_t flags;
  double rope_theta;
  float softmax_scale;
  int32_t top_k;
  int32_t n_cap;
  int32_t n_win;
  int32_t win_len;
  int32_t _pad0;
  const int64_t* q_pos;
  const void* q;
  const void* kv0;
  const void* kv1;
  int64_t kv_stride;
  int64_t kv_seq_stride;
  const int32_t* n_entries;
  const int32_t* idx;
  const void* win0;
  const void* win1;
  int64_t win_stride;
  int64_t win_seq_stride;
  const int64_t* win_pos0;
  const float* sink;
  void* out;
  float* out_lse;
  void* ev_start;   /* optional hipEvent_t recorded just before the attention kernel */
  void* ev_stop;    /* optional hipEvent_t recorded just after it (NULL = none) */
  /* ABI 3: paged entries (see "paged layout"); NULL block_table = contiguous */
  const int32_t* block_table;   /* [B][bt_stride] block ids */
  int32_t bt_stride;
  int32_t block_rows;           /* entries per block: 32 for CSA, 1 for HCA */
  int32_t pool_blocks;          /* blocks in the kv0 / kv1 pools */
  int32_t _pad1;
} CsaAttendArgs;

/* ABI version of the loaded library (CSA_ABI_VERSION). */
int csa_abi_version(void);

/* Static text for a status code. */
const char* csa_strerror(int status);

/* sizeof the argument struct of `op` as compiled into the library, so a
 * binding can check its own mirror of the layout. */
size_t csa_args_size(int op);

/* Device workspace in bytes that `op` needs for `args` (0 = none).  Returns
 * (size_t)-1 for invalid arguments. */
size_t csa_workspace_bytes(int op, const void* args);

int csa_compress(const CsaCompressArgs* args, void* stream);

/* n_jobs independent csa_compress calls in as few launches as possible (one
 * launch per run of up to four jobs that share in_dtype): e.g. the newest
 * main-KV entry, the newest indexer key and the new raw window row of one
 * decode step.  Every job is validated before anything is launched; the
 * status is that of the first invalid job, else of the launches.  Jobs must
 * not write to overlapping outputs. */
int csa_compress_batch(const CsaCompressArgs* jobs, int n_jobs, void* stream);

/* The same batch with a workspace, so that long blocks (m >= 16, the HCA
 * compression) are pooled over many workgroups instead of one per entry: the
 * candidates of an entry are folded in groups of 16 by separate workgroups
 * into per-channel partial (max, sum, weighted sum) states, which a second
 * launch merges before the norm, rotation and storage of the entry.  The
 * result equals csa_compress_batch's up to the order of the fp32 sums.
 *
 * csa_compress_workspace_bytes: device bytes the batch needs (0 when no job
 * has long blocks with a complete entry; (size_t)-1 when a job is invalid).
 * Workspace: at least that many bytes, 256-byte aligned, caller-owned, no
 * initial contents required; its contents after the call are unspecified.
 * Returns CSA_EWORKSPACE when it is too small or misaligned (nothing is
 * launched), otherwise as csa_compress_batch.  Calls that share a workspace
 * must be ordered on one stream. */
size_t csa_compress_workspace_bytes(const CsaCompressArgs* jobs, int n_jobs);
int csa_compress_batch_ws(const CsaCompressArgs* jobs, int n_jobs, void* workspace, size_t workspace_bytes,
                          void* stream);
int csa_index_topk(const CsaIndexArgs* args, void* workspace, size_t workspace_bytes, void* stream);

/* csa_index_topk without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc).  Same arguments, results and
 * determinism as csa_index_topk; no allocation of any kind.
 *
 * Workspace: a library-owned device array of CSA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held until the process ends; the call runs its queries
 * in blocks that fit it (fewer queries per block than csa_index_topk uses,
 * so large prefill chunks take more launches).  A call whose single query
 * (B sequences of it) does not fit (about B * n_cap * 8 bytes + B * 17 KiB
 * > 64 MiB; n_cap = 262144 allows B <= 30) returns CSA_ESCRATCH and
 * launches nothing.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind; the call itself clears what must start at
 * zero.  Calls that overlap in time on one GPU (different streams or host
 * threads without ordering) race on the array: order them on one stream.
 * `stream` must belong to the current device. */
int csa_index_topk_noalloc(const CsaIndexArgs* args, void* stream);

/* Queries per sequence that csa_index_topk scores and selects per internal
 * block for `args` (its workspace holds one block); a negative status for
 * invalid arguments.  Calls whose visible-entry count changes at a block
 * boundary are where the blocks meet. */
int csa_index_query_block(const CsaIndexArgs* args);
int csa_attend(const CsaAttendArgs* args, void* workspace, size_t workspace_bytes, void* stream);
int hca_attend(const CsaAttendArgs* args, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
