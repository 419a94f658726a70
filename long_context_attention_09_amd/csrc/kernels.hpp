// Launch descriptors passed by value from the validated host API to the
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct CompressLaunch {
  int32_t B, d, d_rope, m, in_dtype, out_fmt, do_norm, n_entries;
  float rms_eps;
  double log_theta;
  int64_t pos0, i_first, out_row0;
  const void* kv_a;
  const void* gate_a;
  const void* kv_b;
  const void* gate_b;
  int64_t in_row_stride, in_seq_stride;
  const float* bias_a;
  const float* bias_b;
  void* out0;
  void* out1;
  int64_t out0_stride, out0_seq_stride, out1_stride, out1_seq_stride;
  float* part;               // NULL, or [B][n_entries][n_parts][3][d] pooled candidate groups
  int32_t n_parts;           // candidate groups of kPartCands per entry (with part)
  int32_t in_ring;           // > 0: inputs are rings, position p at row p % in_ring
  const int32_t* out_bt;     // NULL, or [B][out_bt_stride] output block ids
  int64_t out_bt_stride;
  int32_t out_block_rows, out_pool_blocks;
  int32_t out_ring;          // > 0: entry i at output row i % out_ring
  const int64_t* seq_pos;    // NULL, or [B]: per-sequence decode mode (one entry per sequence at most)
};

// Entry of sequence b that this launch's entry slot e stands for; -1: none.
// Per-sequence decode mode: the entry that token seq_pos[b] completes.
__device__ __forceinline__ int64_t compress_entry(const CompressLaunch& a, int b, int e) {
  if (!a.seq_pos) return a.i_first + e;
  const int64_t p1 = a.seq_pos[b] + 1;
  return (p1 >= a.m && p1 % a.m == 0) ? p1 / a.m - 1 : -1;
}

// Row of position-relative input row `row` (position pos0 + row).
__device__ __forceinline__ int64_t compress_in_row(const CompressLaunch& a, int64_t row) {
  return a.in_ring > 0 ? (row + a.pos0) % a.in_ring : row;
}

// Byte offset of entry i of sequence b in an output array (row stride
// `stride`, sequence stride `seq`); -1 when its block is unallocated.
__device__ __forceinline__ int64_t compress_out_off(const CompressLaunch& a, int b, int64_t i, int64_t stride,
                                                    int64_t seq) {
  if (a.out_ring > 0) return (int64_t)b * seq + (i % a.out_ring) * stride;
  if (!a.out_bt) return (int64_t)b * seq + (i - a.out_row0) * stride;
  if (i / a.out_block_rows >= a.out_bt_stride) return -1;
  const int blk = a.out_bt[(int64_t)b * a.out_bt_stride + i / a.out_block_rows];
  if (blk < 0 || blk >= a.out_pool_blocks) return -1;
  return ((int64_t)blk * a.out_block_rows + i % a.out_block_rows) * stride;
}

// Candidates per workgroup when long blocks are pooled in groups.
constexpr int kPartCands = 16;

// Per-query top-k state kept in the workspace.
struct TopkState {
  uint32_t b1;        // 12-bit bucket (key >> 20) holding the k-th largest key
  int32_t k_rem;      // how many to take inside bucket b1 (-1: every visible entry)
  int32_t n_vis;      // visible entries of the query
  uint32_t T;         // the k-th largest key (query blocks: set by the threshold pass)
  int32_t k_eq;       // keys equal to T to take, lowest indices first (same)
  int32_t pad[3];
};

struct IndexLaunch {
  int32_t B, n_q, m, n_cap, H_I, d_I, fmt, top_k;
  int32_t flags;             // CSA_INDEX_*
  int32_t n_chunks;          // 4096-score chunks per query
  int32_t q_first;           // first query of this query block
  int32_t n_qb;              // queries in this block
  const int64_t* q_pos;
  const int32_t* n_entries;
  const void* q0;
  const void* q1;
  const float* w;
  const void* k0;
  const void* k1;
  int32_t* out_idx;
  float* out_score;          // full [B][n_q][n_cap] output (optional)
  // workspace views (per query of the block: q_local = b * n_qb + r)
  float* scores;             // score rows: row (b, r) at (b * score_seq_rows + score_row0 + r) * n_cap
  int32_t score_seq_rows;    // n_qb for the workspace, n_q for the caller's out_score
  int32_t score_row0;        // 0 for the workspace, q_first for the caller's out_score
  uint32_t* hist;            // [B * n_qb][4096]            zeroed after use
  TopkState* state;          // [B * n_qb]
  uint32_t* cand_key;        // [B * n_qb][n_cap]: chunk c's candidates at [c * 4096, ...)
  int32_t* chunk_cand;       // [B * n_qb][n_chunks] candidates per chunk
  int32_t* chunk_above;      // [B * n_qb][n_chunks] scores above the first-digit bucket
  int32_t* chunk_sel;        // [B * n_qb][n_chunks] query blocks: output start of the chunk's selection
  int32_t* chunk_eqb;        // [B * n_qb][n_chunks] query blocks: keys equal to T before the chunk
  int32_t list_mode;         // collect leaves the chunk's selected-index lists in its score region
  uint8_t* lin;              // [B * n_qb][kIndexLinBytes]: FP8 split of the weighted query sum (query blocks)
  hipEvent_t ev_start, ev_stop;  // recorded around the scoring kernel (may be null)
  const int32_t* bt;         // NULL, or [B][bt_stride] key block ids (k0 / k1 are the pools)
  int32_t bt_stride, block_rows, pool_blocks;
};

// Longest split of a CSA selection list the FP8 attention kernel stages in LDS.
constexpr int kAttendIdxMax = 2048;
constexpr int kIndexLinBytes = 1024;  // per query of a block: the FP8 split of the weighted query sum

struct AttendLaunch {
  int32_t B, n_q, H, d, d_rope, m, fmt, flags;
  double log_theta;
  float scale_log2;          // softmax_scale * log2(e)
  int32_t top_k, n_cap, n_win, win_len;
  int32_t n_splits, list_len, split_len;
  const int64_t* q_pos;
  const void* q;
  const void* kv0;
  const void* kv1;
  int64_t kv_stride, kv_seq_stride;
  const int32_t* n_entries;
  const int32_t* idx;        // NULL: dense (HCA)
  const void* win0;
  const void* win1;
  int64_t win_stride, win_seq_stride;
  const int64_t* win_pos0;
  const float* sink;
  void* out;
  float* out_lse;
  _Float16* part_o;          // [units][n_splits][64][d] partial outputs (normalised)
  float* part_ml;            // [units][n_splits][64][2]  (running max, sum)
  hipEvent_t ev_start, ev_stop;  // recorded around the attention kernel (may be null)
  const int32_t* bt;         // NULL, or [B][bt_stride] entry block ids (kv0 / kv1 are the pools)
  int32_t bt_stride, block_rows, pool_blocks;
};

constexpr int kMaxJobs = 4;
struct CompressBatch {
  CompressLaunch job[kMaxJobs];
  int32_t n_jobs;
};

hipError_t launch_compress(const CompressBatch& b, hipStream_t s);
hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s);
hipError_t launch_attend(const AttendLaunch& a, hipStream_t s);
// The 128-heads-per-workgroup attention for calls with several queries
// (attend_mh.hip): whether it serves `a`, and its launch (no combine).
bool attend_mh_applies(const AttendLaunch& a);
hipError_t launch_attend_mh(const AttendLaunch& a, hipStream_t s);

}  // namespace csa
