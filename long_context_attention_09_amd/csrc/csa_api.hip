// Host side of the C ABI declared in include/csa.h: argument validation,
// workspace sizing and kernel launches.  No allocation and no
// synchronisation; the only global state is the per-device address of the
// allocation-free entry point's scratch array, looked up once per device.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "csa.h"
#include "kernels.hpp"
#include "api_internal.hpp"

#define CSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;
constexpr int kIdxChunk = 4096;       // scores per workgroup in the radix passes
constexpr int64_t kMaxIndexCap = int64_t(1024) * 4096;  // entries per sequence the top-k handles

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ------------------------------------------------------------------ compress

int check_compress(const CsaCompressArgs* a) {
  if (!a) return CSA_EINVAL;
  if (a->B < 1 || a->n_rows < 0 || a->m < 1 || a->m > 1024 || a->d < 1 || a->d > 1024) return CSA_EINVAL;
  if (a->d % 8 || a->d_rope < 0 || a->d_rope > a->d || (a->d_rope & 1)) return CSA_EINVAL;
  if (a->pos0 < 0 || a->pos0 % a->m) return CSA_EINVAL;
  if (a->in_dtype != CSA_DT_F32 && a->in_dtype != CSA_DT_BF16) return CSA_EINVAL;
  if (a->out_fmt != CSA_FMT_F32 && a->out_fmt != CSA_FMT_FP8_BF16 && a->out_fmt != CSA_FMT_MXFP4)
    return CSA_EINVAL;
  if (a->overlap != 0 && a->overlap != 1) return CSA_EINVAL;
  if (!a->kv_a || !a->out0) return CSA_EINVAL;
  if (a->overlap && !a->kv_b) return CSA_EINVAL;
  if (!a->overlap && (a->kv_b || a->gate_b || a->bias_b)) return CSA_EINVAL;
  if (a->out_fmt != CSA_FMT_F32 && !a->out1) return CSA_EINVAL;
  if (!(a->rms_eps >= 0.0f) || (a->d_rope > 0 && !(a->rope_theta > 0.0))) return CSA_EINVAL;
  const size_t es = a->in_dtype == CSA_DT_F32 ? 4 : 2;
  if (a->in_row_stride < (int64_t)(a->d * es) || a->in_row_stride % es || a->in_seq_stride < 0 ||
      a->in_seq_stride % es)
    return CSA_EINVAL;
  const void* ins[4] = {a->kv_a, a->gate_a, a->kv_b, a->gate_b};
  for (const void* p : ins)
    if (p && !aligned(p, es)) return CSA_EINVAL;
  if (a->bias_a && !aligned(a->bias_a, 4)) return CSA_EINVAL;
  if (a->bias_b && !aligned(a->bias_b, 4)) return CSA_EINVAL;
  if (a->out0_stride <= 0 || a->out0_seq_stride < 0) return CSA_EINVAL;
  if (a->out_fmt == CSA_FMT_F32) {
    if (!aligned(a->out0, 4) || a->out0_stride % 4 || a->out0_seq_stride % 4 ||
        a->out0_stride < (int64_t)a->d * 4)
      return CSA_EINVAL;
  } else if (a->out_fmt == CSA_FMT_FP8_BF16) {
    if (a->out1_stride <= 0 || a->out1_seq_stride < 0 || !aligned(a->out1, 2) || a->out1_stride % 2 ||
        a->out1_seq_stride % 2)
      return CSA_EINVAL;
  } else {
    if (a->d % 32 || a->d_rope != 0) return CSA_EUNSUPPORTED;
    if (a->out1_stride <= 0 || a->out1_seq_stride < 0) return CSA_EINVAL;
  }
  if (a->in_ring < 0 || (a->in_ring > 0 && !a->seq_pos && a->n_rows > a->in_ring)) return CSA_EINVAL;
  if (a->out_block_table) {
    if (!aligned(a->out_block_table, 4) || a->out_block_rows < 1 || a->out_bt_stride < 1 ||
        a->out_pool_blocks < 1 || a->out_row0 != 0)
      return CSA_EINVAL;
  }
  if (a->out_ring < 0 || (a->out_ring > 0 && (a->out_block_table || a->out_row0 != 0))) return CSA_EINVAL;
  if (a->seq_pos) {
    if (!aligned(a->seq_pos, 8) || a->in_ring < (a->overlap ? 2 * a->m : a->m)) return CSA_EINVAL;
  }
  return CSA_OK;
}

// Entries [first, end) the job stores (the per-sequence decode mode: one slot,
// resolved per sequence on the device).
void job_entries(const CsaCompressArgs* a, int64_t* first, int64_t* end) {
  if (a->seq_pos) {
    *first = 0;
    *end = 1;
    return;
  }
  *first = a->pos0 / a->m + ((a->overlap && a->pos0 > 0) ? 1 : 0);
  *end = (a->pos0 + a->n_rows) / a->m;
}

}  // namespace

// ------------------------------------------------------------------ index / top-k

namespace csa {
namespace api {

int check_index(const CsaIndexArgs* a) {
  if (!a) return CSA_EINVAL;
  if (a->B < 1 || a->n_q < 1 || a->m < 1 || a->n_cap < 1 || a->H_I < 1 || a->d_I < 1 || a->top_k < 1)
    return CSA_EINVAL;
  if (a->n_cap > kMaxIndexCap) return CSA_EUNSUPPORTED;
  if (a->flags & ~(CSA_INDEX_BATCH_INVARIANT | CSA_INDEX_BF16_SCORES)) return CSA_EINVAL;
  if (!a->q_pos || !a->q0 || !a->w || !a->k0 || !a->out_idx) return CSA_EINVAL;
  if (!aligned(a->q_pos, 8) || !aligned(a->w, 4) || !aligned(a->out_idx, 4)) return CSA_EINVAL;
  if (a->n_entries && !aligned(a->n_entries, 4)) return CSA_EINVAL;
  if (a->out_score && !aligned(a->out_score, (a->flags & CSA_INDEX_BF16_SCORES) ? 2 : 4)) return CSA_EINVAL;
  if (a->fmt == CSA_FMT_MXFP4) {
    if (!a->q1 || !a->k1) return CSA_EINVAL;
    if (a->d_I != 128 || a->H_I % 16 || a->H_I > 64) return CSA_EUNSUPPORTED;
    if (!aligned(a->q0, 16) || !aligned(a->k0, 16) || !aligned(a->k1, 4)) return CSA_EINVAL;
  } else if (a->fmt == CSA_FMT_F32) {
    if (a->d_I > 1024) return CSA_EUNSUPPORTED;
    if (!aligned(a->q0, 4) || !aligned(a->k0, 4)) return CSA_EINVAL;
  } else {
    return CSA_EINVAL;
  }
  if (a->block_table) {
    if (!aligned(a->block_table, 4) || a->block_rows < 1 || a->bt_stride < 1 || a->pool_blocks < 1)
      return CSA_EINVAL;
    if ((int64_t)a->bt_stride * a->block_rows < a->n_cap) return CSA_EINVAL;
    if (a->fmt == CSA_FMT_MXFP4 && (a->block_rows != 32 || a->pool_blocks >= (1 << 20)))
      return CSA_EUNSUPPORTED;
  }
  return CSA_OK;
}


// Workspace layout for query blocks of n_qb queries per sequence.
IndexPlan index_layout(const CsaIndexArgs* a, int n_qb) {
  IndexPlan p;
  p.n_chunks = (a->n_cap + kIdxChunk - 1) / kIdxChunk;
  p.n_qb = n_qb;
  const size_t nq = (size_t)a->B * n_qb;
  size_t off = 0;
  p.off_scores = off;
  const size_t es = (a->flags & CSA_INDEX_BF16_SCORES) ? 2 : 4;   // bytes per score
  if (!a->out_score) off += align_up(nq * (size_t)a->n_cap * es);
  p.off_hist = off;   off += align_up(nq * 4096 * 4);
  p.off_state = off;  off += align_up(nq * sizeof(csa::TopkState));
  p.off_ckey = off;   off += align_up(nq * (size_t)a->n_cap * 4);
  p.off_ccnt = off;   off += align_up(nq * (size_t)p.n_chunks * 4);
  p.off_above = off;  off += align_up(nq * (size_t)p.n_chunks * 4);
  p.off_csel = off;   off += align_up(nq * (size_t)p.n_chunks * 4);
  p.off_ceqb = off;   off += align_up(nq * (size_t)p.n_chunks * 4);
  p.off_lin = off;    off += align_up(nq * (size_t)csa::kIndexLinBytes);
  p.total = off;
  return p;
}

// The largest query block (a multiple of 4 from 4 queries on) whose
// workspace fits `budget` bytes; n_qb = 0 when one query does not fit.
IndexPlan plan_index(const CsaIndexArgs* a, int64_t budget) {
  const int64_t n_chunks = (a->n_cap + kIdxChunk - 1) / kIdxChunk;
  const int64_t es = (a->flags & CSA_INDEX_BF16_SCORES) ? 2 : 4;
  const int64_t per_q = (int64_t)a->B * ((a->out_score ? 0 : (int64_t)a->n_cap * es) + (int64_t)a->n_cap * 4 +
                                         4096 * 4 + (int64_t)sizeof(csa::TopkState) + 4 * n_chunks * 4 +
                                         csa::kIndexLinBytes);
  int64_t n = budget / (per_q > 0 ? per_q : 1);
  if (n > a->n_q) n = a->n_q;
  if (n >= 4) n -= n % 4;
  if (n < 1) n = 1;
  IndexPlan p = index_layout(a, (int)n);
  while (p.total > (size_t)budget && n > 1) {   // alignment padding
    n = n > 4 ? n - 4 : n - 1;
    p = index_layout(a, (int)n);
  }
  if (p.total > (size_t)budget) p.n_qb = 0;
  return p;
}

}  // namespace api
}  // namespace csa

namespace {

using csa::api::IndexPlan;
using csa::api::kWorkspaceBudget;
using csa::api::check_index;
using csa::api::plan_index;

// ------------------------------------------------------------------ attention

int check_attend(const CsaAttendArgs* a, bool dense) {
  if (!a) return CSA_EINVAL;
  if (a->B < 1 || a->n_q < 1 || a->H < 1 || a->d < 1 || a->m < 1 || a->n_win < 1 || a->win_len < 0 ||
      a->n_cap < 0)
    return CSA_EINVAL;
  if (a->d_rope < 0 || a->d_rope > a->d || (a->d_rope & 1)) return CSA_EINVAL;
  if (a->d_rope > 0 && !(a->rope_theta > 0.0)) return CSA_EINVAL;
  if (!(a->softmax_scale >= 0.0f)) return CSA_EINVAL;
  if (!a->q_pos || !a->q || !a->sink || !a->out) return CSA_EINVAL;
  if (!a->win_pos0 && !(a->flags & CSA_ATTEND_WIN_RING)) return CSA_EINVAL;
  if (a->n_cap > 0 && !a->kv0) return CSA_EINVAL;
  if (a->win_len > 0 && !a->win0) return CSA_EINVAL;
  if (dense ? a->idx != nullptr : (a->idx == nullptr || a->top_k < 1)) return CSA_EINVAL;
  if (!aligned(a->q_pos, 8) || (a->win_pos0 && !aligned(a->win_pos0, 8)) || !aligned(a->sink, 4))
    return CSA_EINVAL;
  if (a->idx && !aligned(a->idx, 4)) return CSA_EINVAL;
  if (a->n_entries && !aligned(a->n_entries, 4)) return CSA_EINVAL;
  if (a->out_lse && !aligned(a->out_lse, 4)) return CSA_EINVAL;
  if (a->kv_stride < 0 || a->kv_seq_stride < 0 || a->win_stride < 0 || a->win_seq_stride < 0)
    return CSA_EINVAL;
  if (a->flags & ~(CSA_ATTEND_NORM_Q | CSA_ATTEND_NO_INV_ROPE | CSA_ATTEND_BATCH_INVARIANT | CSA_ATTEND_WIN_RING))
    return CSA_EINVAL;
  if (a->block_table) {
    if (!aligned(a->block_table, 4) || a->block_rows < 1 || a->bt_stride < 1 || a->pool_blocks < 1)
      return CSA_EINVAL;
    if ((int64_t)a->bt_stride * a->block_rows < a->n_cap) return CSA_EINVAL;
    if ((int64_t)a->pool_blocks * a->block_rows > INT32_MAX) return CSA_EUNSUPPORTED;
  }
  if (a->fmt == CSA_FMT_FP8_BF16) {
    if (a->d != 512 || a->d_rope != 64 || a->H % 16) return CSA_EUNSUPPORTED;
    if (a->n_cap > 0 && !a->kv1) return CSA_EINVAL;
    if (a->win_len > 0 && !a->win1) return CSA_EINVAL;
    const void* ps[5] = {a->q, a->kv0, a->kv1, a->win0, a->win1};
    for (const void* p : ps)
      if (p && !aligned(p, 16)) return CSA_EINVAL;
    if (!aligned(a->out, 8)) return CSA_EINVAL;
    if (a->kv_stride % 16 || a->kv_seq_stride % 16 || a->win_stride % 16 || a->win_seq_stride % 16)
      return CSA_EINVAL;
    if (a->kv_stride >= ((int64_t)1 << 31) || a->win_stride >= ((int64_t)1 << 31)) return CSA_EUNSUPPORTED;
  } else if (a->fmt == CSA_FMT_F32) {
    if (a->d > 512 || (a->d & 1) || a->H > 65535) return CSA_EUNSUPPORTED;
    const void* ps[3] = {a->q, a->kv0, a->win0};
    for (const void* p : ps)
      if (p && !aligned(p, 4)) return CSA_EINVAL;
    if (!aligned(a->out, 4)) return CSA_EINVAL;
    if (a->kv_stride % 4 || a->kv_seq_stride % 4 || a->win_stride % 4 || a->win_seq_stride % 4)
      return CSA_EINVAL;
  } else {
    return CSA_EINVAL;
  }
  return CSA_OK;
}

struct AttendPlan {
  int n_splits, split_len, list_len;
  size_t off_o, off_ml, total;
};

AttendPlan plan_attend(const CsaAttendArgs* a, bool dense) {
  AttendPlan p{};
  const int64_t comp = dense ? a->n_cap : a->top_k;
  int64_t list = comp + a->n_win;
  if (list < 1) list = 1;
  p.list_len = (int)list;
  if (a->fmt == CSA_FMT_F32) {
    p.n_splits = 1;
    p.split_len = p.list_len;
    p.total = 0;
    return p;
  }
  const int64_t units = (int64_t)a->B * a->n_q * ((a->H + 63) / 64);
  // Splits take the list's 32-entry tiles round-robin (split s: tiles s,
  // s + n_splits, ...).
  const int64_t tiles = (list + 31) / 32;
  if (a->flags & CSA_ATTEND_BATCH_INVARIANT) {
    // a split count fixed by the list length alone: every query of any batch
    // sums its rows in the same order
    const int64_t per_inv = CSA_INVARIANT_SPLIT_ROWS / 32;
    p.n_splits = (int)((tiles + per_inv - 1) / per_inv);
    p.split_len = CSA_INVARIANT_SPLIT_ROWS;
    if (p.n_splits > 1) {
      const size_t rows = (size_t)units * p.n_splits * 64;
      p.off_o = 0;
      p.off_ml = align_up(rows * 512 * 2);
      p.total = p.off_ml + align_up(rows * 2 * 4);
    }
    return p;
  }
  int64_t s = (256 + units - 1) / units;          // one workgroup per compute unit
  int64_t s_max = (tiles + 2) / 3;                // at least three tiles per split
  if (s > s_max) s = s_max;
  const int64_t per_max = csa::kAttendIdxMax / 32;    // a split's gathered rows fit the kernel's stage
  const bool staged = !dense || a->block_table != nullptr;
  if (staged) {
    const int64_t s_min = (tiles + per_max - 1) / per_max;
    if (s < s_min) s = s_min;
  }
  if (s < 1) s = 1;
  int64_t per = (tiles + s - 1) / s;
  // The kernel runs n_tiles + 2 pipeline steps in rounds of two: splits of
  // an even number of tiles waste no step, so an odd count grows by one
  // (fewer splits for the combine, same kernel time).
  per += per & 1;
  if (staged && per > per_max) per = per_max;
  s = (tiles + per - 1) / per;
  const int64_t len = per * 32;
  p.n_splits = (int)s;
  p.split_len = (int)len;
  if (s > 1) {
    const size_t rows = (size_t)units * s * 64;
    p.off_o = 0;
    p.off_ml = align_up(rows * 512 * 2);
    p.total = p.off_ml + align_up(rows * 2 * 4);
  } else {
    p.total = 0;
  }
  return p;
}

int run_attend(const CsaAttendArgs* a, void* ws, size_t ws_bytes, void* stream, bool dense) {
  int st = check_attend(a, dense);
  if (st) return st;
  const AttendPlan p = plan_attend(a, dense);
  if (p.total > 0 && (!ws || ws_bytes < p.total || !aligned(ws, kAlign))) return CSA_EWORKSPACE;
  csa::AttendLaunch L{};
  L.B = a->B; L.n_q = a->n_q; L.H = a->H; L.d = a->d; L.d_rope = a->d_rope; L.m = a->m;
  L.fmt = a->fmt; L.flags = a->flags;
  L.log_theta = a->d_rope > 0 ? log(a->rope_theta) : 0.0;
  const float scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf((float)a->d);
  L.scale_log2 = scale * 1.4426950408889634f;
  L.top_k = dense ? 0 : a->top_k;
  L.n_cap = a->n_cap; L.n_win = a->n_win; L.win_len = a->win_len;
  L.n_splits = p.n_splits; L.list_len = p.list_len; L.split_len = p.split_len;
  L.q_pos = a->q_pos; L.q = a->q; L.kv0 = a->kv0;
  L.kv1 = a->kv1;
  L.kv_stride = a->kv_stride; L.kv_seq_stride = a->block_table ? 0 : a->kv_seq_stride;
  L.bt = a->block_table; L.bt_stride = a->bt_stride; L.block_rows = a->block_rows;
  L.pool_blocks = a->pool_blocks;
  L.n_entries = a->n_entries; L.idx = dense ? nullptr : a->idx;
  L.win0 = a->win0; L.win1 = a->win1; L.win_stride = a->win_stride; L.win_seq_stride = a->win_seq_stride;
  L.win_pos0 = a->win_pos0; L.sink = a->sink; L.out = a->out; L.out_lse = a->out_lse;
  L.ev_start = (hipEvent_t)a->ev_start; L.ev_stop = (hipEvent_t)a->ev_stop;
  if (p.total > 0) {
    L.part_o = (_Float16*)((char*)ws + p.off_o);
    L.part_ml = (float*)((char*)ws + p.off_ml);
  }
  if (csa::launch_attend(L, (hipStream_t)stream) != hipSuccess) return CSA_EHIP;
  return CSA_OK;
}

}  // namespace

CSA_EXPORT int csa_abi_version(void) { return CSA_ABI_VERSION; }

CSA_EXPORT const char* csa_strerror(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_EINVAL: return "invalid argument (null or misaligned pointer, or inconsistent shape)";
    case CSA_EUNSUPPORTED: return "unsupported shape or format combination";
    case CSA_EHIP: return "HIP runtime reported a launch error";
    case CSA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case CSA_ESCRATCH:
      return "problem too large for the allocation-free entry point's scratch (CSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

CSA_EXPORT size_t csa_args_size(int op) {
  switch (op) {
    case CSA_OP_COMPRESS: return sizeof(CsaCompressArgs);
    case CSA_OP_INDEX_TOPK: return sizeof(CsaIndexArgs);
    case CSA_OP_ATTEND:
    case CSA_OP_HCA_ATTEND: return sizeof(CsaAttendArgs);
    default: return 0;
  }
}

CSA_EXPORT size_t csa_workspace_bytes(int op, const void* args) {
  switch (op) {
    case CSA_OP_COMPRESS:
      return check_compress((const CsaCompressArgs*)args) ? (size_t)-1 : 0;
    case CSA_OP_INDEX_TOPK: {
      const CsaIndexArgs* a = (const CsaIndexArgs*)args;
      if (check_index(a)) return (size_t)-1;
      const IndexPlan p = plan_index(a, kWorkspaceBudget);
      return p.n_qb < 1 ? (size_t)-1 : p.total;
    }
    case CSA_OP_ATTEND:
    case CSA_OP_HCA_ATTEND: {
      const CsaAttendArgs* a = (const CsaAttendArgs*)args;
      const bool dense = op == CSA_OP_HCA_ATTEND;
      if (check_attend(a, dense)) return (size_t)-1;
      return plan_attend(a, dense).total;
    }
    default: return (size_t)-1;
  }
}

namespace {

// Fill the launch descriptor of one validated job; false when it has no entry.
bool compress_job(const CsaCompressArgs* a, csa::CompressLaunch* L) {
  int64_t first, end;
  job_entries(a, &first, &end);
  if (end <= first) return false;
  *L = csa::CompressLaunch{};
  L->B = a->B; L->d = a->d; L->d_rope = a->d_rope; L->m = a->m; L->in_dtype = a->in_dtype;
  L->out_fmt = a->out_fmt; L->do_norm = a->do_norm; L->n_entries = (int32_t)(end - first);
  L->rms_eps = a->rms_eps; L->log_theta = a->d_rope > 0 ? log(a->rope_theta) : 0.0;
  L->pos0 = a->seq_pos ? 0 : a->pos0; L->i_first = first; L->out_row0 = a->out_row0;
  L->kv_a = a->kv_a; L->gate_a = a->gate_a; L->kv_b = a->kv_b; L->gate_b = a->gate_b;
  L->in_row_stride = a->in_row_stride;
  L->in_seq_stride = a->in_seq_stride;
  L->bias_a = a->bias_a; L->bias_b = a->bias_b;
  L->out0 = a->out0; L->out1 = a->out1;
  L->out0_stride = a->out0_stride; L->out0_seq_stride = a->out0_seq_stride;
  L->out1_stride = a->out1_stride; L->out1_seq_stride = a->out1_seq_stride;
  L->in_ring = a->in_ring;
  L->out_bt = a->out_block_table; L->out_bt_stride = a->out_bt_stride;
  L->out_block_rows = a->out_block_rows; L->out_pool_blocks = a->out_pool_blocks;
  L->out_ring = a->out_ring; L->seq_pos = a->seq_pos;
  return true;
}

int check_compress_entries(const CsaCompressArgs* a) {
  if (a->seq_pos) return CSA_OK;     // checked per sequence on the device (block ids against the pool)
  int64_t first, end;
  job_entries(a, &first, &end);
  if (end <= first) return CSA_OK;
  if (first < a->out_row0) return CSA_EINVAL;
  if (end - first > INT32_MAX / 4) return CSA_EUNSUPPORTED;
  if (a->out_block_table && (end - 1) / a->out_block_rows >= a->out_bt_stride) return CSA_EINVAL;
  return CSA_OK;
}

}  // namespace

namespace {

// Candidate groups per entry when a job's long blocks (m >= 16) are pooled
// over several workgroups; 0 for short blocks.
int compress_parts(const CsaCompressArgs* a) {
  if (a->m < 16) return 0;
  const int n_cand = a->overlap ? 2 * a->m : a->m;
  return (n_cand + csa::kPartCands - 1) / csa::kPartCands;
}

size_t compress_part_bytes(const CsaCompressArgs* a) {
  const int P = compress_parts(a);
  int64_t first, end;
  job_entries(a, &first, &end);
  if (P == 0 || end <= first) return 0;
  return align_up((size_t)a->B * (size_t)(end - first) * (size_t)P * 3 * (size_t)a->d * sizeof(float));
}

int check_compress_jobs(const CsaCompressArgs* jobs, int n_jobs) {
  if (!jobs || n_jobs < 0) return CSA_EINVAL;
  for (int j = 0; j < n_jobs; ++j) {
    int st = check_compress(&jobs[j]);
    if (!st) st = check_compress_entries(&jobs[j]);
    if (st) return st;
  }
  return CSA_OK;
}

// One launch (two with grouped long blocks) per run of up to kMaxJobs jobs of
// the same input dtype; ws NULL keeps every block in one workgroup.
int run_compress_batch(const CsaCompressArgs* jobs, int n_jobs, char* ws, void* stream) {
  size_t off = 0;
  for (int dt = CSA_DT_F32; dt <= CSA_DT_BF16; ++dt) {
    csa::CompressBatch bt{};
    for (int j = 0; j < n_jobs; ++j) {
      if (jobs[j].in_dtype != dt) continue;
      if (!compress_job(&jobs[j], &bt.job[bt.n_jobs])) continue;
      const size_t pb = ws ? compress_part_bytes(&jobs[j]) : 0;
      if (pb > 0) {
        bt.job[bt.n_jobs].part = (float*)(ws + off);
        bt.job[bt.n_jobs].n_parts = compress_parts(&jobs[j]);
        off += pb;
      }
      if (++bt.n_jobs == csa::kMaxJobs) {
        if (csa::launch_compress(bt, (hipStream_t)stream) != hipSuccess) return CSA_EHIP;
        bt.n_jobs = 0;
      }
    }
    if (bt.n_jobs > 0 && csa::launch_compress(bt, (hipStream_t)stream) != hipSuccess) return CSA_EHIP;
  }
  return CSA_OK;
}

}  // namespace

CSA_EXPORT int csa_compress_batch(const CsaCompressArgs* jobs, int n_jobs, void* stream) {
  const int st = check_compress_jobs(jobs, n_jobs);
  if (st) return st;
  return run_compress_batch(jobs, n_jobs, nullptr, stream);
}

CSA_EXPORT size_t csa_compress_workspace_bytes(const CsaCompressArgs* jobs, int n_jobs) {
  if (check_compress_jobs(jobs, n_jobs)) return (size_t)-1;
  size_t total = 0;
  for (int j = 0; j < n_jobs; ++j) total += compress_part_bytes(&jobs[j]);
  return total;
}

CSA_EXPORT int csa_compress_batch_ws(const CsaCompressArgs* jobs, int n_jobs, void* ws, size_t ws_bytes,
                                     void* stream) {
  const int st = check_compress_jobs(jobs, n_jobs);
  if (st) return st;
  size_t need = 0;
  for (int j = 0; j < n_jobs; ++j) need += compress_part_bytes(&jobs[j]);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, kAlign))) return CSA_EWORKSPACE;
  return run_compress_batch(jobs, n_jobs, need > 0 ? (char*)ws : nullptr, stream);
}

CSA_EXPORT int csa_compress(const CsaCompressArgs* a, void* stream) {
  if (!a) return CSA_EINVAL;
  return csa_compress_batch(a, 1, stream);
}

namespace csa {
namespace api {

// Query blocks of p.n_qb queries, each through the workspace laid out by p.
int run_index(const CsaIndexArgs* a, const IndexPlan& p, char* ws, void* stream) {
  for (int q0 = 0; q0 < a->n_q; q0 += p.n_qb) {
    csa::IndexLaunch L{};
    L.B = a->B; L.n_q = a->n_q; L.m = a->m; L.n_cap = a->n_cap; L.H_I = a->H_I; L.d_I = a->d_I;
    L.fmt = a->fmt; L.top_k = a->top_k; L.n_chunks = p.n_chunks; L.flags = a->flags;
    L.q_first = q0;
    L.n_qb = a->n_q - q0 < p.n_qb ? a->n_q - q0 : p.n_qb;
    L.q_pos = a->q_pos; L.n_entries = a->n_entries;
    L.q0 = a->q0; L.q1 = a->q1; L.w = a->w; L.k0 = a->k0; L.k1 = a->k1;
    L.out_idx = a->out_idx; L.out_score = (float*)a->out_score;
    if (a->out_score) {
      // the caller's [B][n_q][n_cap] array: block rows start at q0 within each sequence
      L.scores = (float*)a->out_score;
      L.score_seq_rows = a->n_q;
      L.score_row0 = q0;
    } else {
      L.scores = (float*)(ws + p.off_scores);
      L.score_seq_rows = L.n_qb;
      L.score_row0 = 0;
    }
    L.hist = (uint32_t*)(ws + p.off_hist);
    L.state = (csa::TopkState*)(ws + p.off_state);
    L.cand_key = (uint32_t*)(ws + p.off_ckey);
    L.chunk_cand = (int32_t*)(ws + p.off_ccnt);
    L.chunk_above = (int32_t*)(ws + p.off_above);
    L.chunk_sel = (int32_t*)(ws + p.off_csel);
    L.chunk_eqb = (int32_t*)(ws + p.off_ceqb);
    L.lin = (uint8_t*)(ws + p.off_lin);
    L.bt = a->block_table; L.bt_stride = a->bt_stride; L.block_rows = a->block_rows;
    L.pool_blocks = a->pool_blocks;
    L.ev_start = q0 == 0 ? (hipEvent_t)a->ev_start : nullptr;
    L.ev_stop = q0 + p.n_qb >= a->n_q ? (hipEvent_t)a->ev_stop : nullptr;
    if (csa::launch_index_topk(L, (hipStream_t)stream) != hipSuccess) return CSA_EHIP;
  }
  return CSA_OK;
}

}  // namespace api
}  // namespace csa

using csa::api::run_index;

CSA_EXPORT int csa_index_query_block(const CsaIndexArgs* a) {
  const int st = check_index(a);
  if (st) return st;
  return plan_index(a, kWorkspaceBudget).n_qb;
}

CSA_EXPORT int csa_index_topk(const CsaIndexArgs* a, void* ws, size_t ws_bytes, void* stream) {
  int st = check_index(a);
  if (st) return st;
  const IndexPlan p = plan_index(a, kWorkspaceBudget);
  if (p.n_qb < 1) return CSA_EWORKSPACE;
  if (!ws || ws_bytes < p.total || !aligned(ws, kAlign)) return CSA_EWORKSPACE;
  return run_index(a, p, (char*)ws, stream);
}

CSA_EXPORT int csa_attend(const CsaAttendArgs* a, void* ws, size_t ws_bytes, void* stream) {
  return run_attend(a, ws, ws_bytes, stream, false);
}

CSA_EXPORT int hca_attend(const CsaAttendArgs* a, void* ws, size_t ws_bytes, void* stream) {
  return run_attend(a, ws, ws_bytes, stream, true);
}
