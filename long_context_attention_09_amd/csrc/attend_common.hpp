// Pieces shared by the attention kernels (attend.hip: one query and 64 heads
// per workgroup; attend_mh.hip: one query and 128 heads per workgroup): the
// entry layout, a query's list (compressed entries, then its raw window), row
// addressing through block tables and window rings, and small helpers.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kD = 512;
constexpr int kDR = 64;
constexpr int kDN = kD - kDR;         // 448
constexpr int kTile = 32;             // entries per LDS tile
constexpr int kChunksPerRow = kDN / 16 + (kDR * 2) / 16;  // 28 + 8 = 36 sixteen-byte chunks
constexpr int kChunksPerTile = kTile * kChunksPerRow;     // 1152

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

struct ListInfo {
  int n_comp;     // compressed part of the list (top_k for CSA, n_vis for HCA)
  int n_vis;      // visible compressed entries
  int win_lo;     // window buffer row of the first window position in the list
  int n_w;        // window rows present
  int win_wrap;   // rows of the ring (window row win_lo + w wraps there); large without a ring
  int64_t t;
};

__device__ __forceinline__ ListInfo list_info(const AttendLaunch& a, int b, int r) {
  ListInfo L;
  const int64_t t = a.q_pos[(int64_t)b * a.n_q + r];
  L.t = t;
  int64_t nv = t >= 0 ? t / a.m : 0;
  const int64_t ne = a.n_entries ? (int64_t)a.n_entries[b] : (int64_t)a.n_cap;
  nv = nv < ne ? nv : ne;
  nv = nv < a.n_cap ? nv : a.n_cap;
  L.n_vis = (int)(nv < 0 ? 0 : nv);
  L.n_comp = a.idx ? a.top_k : L.n_vis;
  int64_t wp0;
  if (a.win_pos0) {
    wp0 = a.win_pos0[b];
  } else {                       // a ring that ends at the query's own position
    wp0 = t - a.win_len + 1;
    wp0 = wp0 > 0 ? wp0 : 0;
  }
  int64_t lo = t - a.n_win + 1;
  lo = lo > 0 ? lo : 0;
  lo = lo > wp0 ? lo : wp0;
  int64_t hi = t < wp0 + a.win_len - 1 ? t : wp0 + a.win_len - 1;
  const bool ring = (a.flags & CSA_ATTEND_WIN_RING) && a.win_len > 0;
  L.win_lo = ring ? (int)(lo % a.win_len) : (int)(lo - wp0);
  L.win_wrap = ring ? a.win_len : 0x7fffffff;
  L.n_w = hi >= lo ? (int)(hi - lo + 1) : 0;
  return L;
}

// Window buffer row of the list's window position w.
__device__ __forceinline__ int window_row(const ListInfo& L, int w) {
  const int row = L.win_lo + w;
  return row >= L.win_wrap ? row - L.win_wrap : row;
}

// Row of entry e (0 <= e < n_vis) of sequence b in the kv arrays: e itself,
// or with a block table its row in the pool; -1 when its block is unallocated.
__device__ __forceinline__ int entry_row(const AttendLaunch& a, int b, int e) {
  if (!a.bt) return e;
  const int blk = a.bt[(int64_t)b * a.bt_stride + e / a.block_rows];
  return blk >= 0 && blk < a.pool_blocks ? blk * a.block_rows + e % a.block_rows : -1;
}

// Splits of a query's list.  Normally the launch's split count (chosen to fill
// the GPU); in the batch-invariant mode a count fixed by the query's own list
// length (pieces of CSA_INVARIANT_SPLIT_ROWS rows), so the order of every sum
// depends on nothing but the query.
__device__ __forceinline__ int query_splits(const AttendLaunch& a, const ListInfo& L) {
  if (!(a.flags & CSA_ATTEND_BATCH_INVARIANT)) return a.n_splits;
  const int tiles = (L.n_comp + L.n_w + kTile - 1) / kTile;
  constexpr int per = CSA_INVARIANT_SPLIT_ROWS / kTile;
  const int n = (tiles + per - 1) / per;
  return n < 1 ? 1 : n;
}

// Resolve list position p to (nope row pointer, rope row pointer); false when masked.
__device__ __forceinline__ bool list_row(const AttendLaunch& a, int b, int r, const ListInfo& L, int p,
                                         const uint8_t** pn, const uint8_t** pr) {
  if (p < L.n_comp) {
    int e = p;
    if (a.idx) {
      e = a.idx[((int64_t)b * a.n_q + r) * a.top_k + p];
      if (e < 0 || e >= L.n_vis) return false;
    }
    e = entry_row(a, b, e);
    if (e < 0) return false;
    const int64_t off = (int64_t)b * a.kv_seq_stride + (int64_t)e * a.kv_stride;
    *pn = (const uint8_t*)a.kv0 + off;
    *pr = (const uint8_t*)a.kv1 + off;
    return true;
  }
  const int w = p - L.n_comp;
  if (w >= L.n_w) return false;
  const int64_t off = (int64_t)b * a.win_seq_stride + (int64_t)window_row(L, w) * a.win_stride;
  *pn = (const uint8_t*)a.win0 + off;
  *pr = (const uint8_t*)a.win1 + off;
  return true;
}

typedef __attribute__((address_space(1))) const i32x4 gbl_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kRescaleSlack = 8.0f;   // log2 units a running max may lag the true max

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + [15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Workgroup barrier that waits for this wave's LDS traffic only: the row
// loads in flight into registers stay in flight (a __syncthreads fence would
// drain them).
#define ATTEND_BARRIER(waitimm)                  \
  do {                                           \
    __builtin_amdgcn_s_waitcnt(waitimm);         \
    __asm__ __volatile__("" ::: "memory");       \
    __builtin_amdgcn_s_barrier();                \
    __asm__ __volatile__("" ::: "memory");       \
  } while (0)

// eight E4M3FN bytes (two dwords, low byte first) -> eight BF16 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const i32x4 w = {__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
  return __builtin_bit_cast(bf16x8, w);
}

// Where a lane's entry rows come from (one query, one split).  Addresses are
// formed without branches: a base, a row and a stride are selected per lane
// (row strides are below 2^31 bytes, checked on the host).
struct RowSource {
  uint64_t kvb0, kvb1, wb0, wb1, dummy;   // entry / window bases of the sequence
  uint32_t kvs, wns;                      // row strides
  int p1, n_comp, n_vis, n_w;             // list end, list layout
  int wlo, wrap;                          // window row of the first window position; ring rows
  bool gather;                            // entries through staged rows (CSA, or a block table)
};
struct RowPtrs {
  uint64_t pn, pr;                        // FP8 bytes, RoPE bytes of the row
  uint32_t live;                          // the tile's live-entry mask
};

// Row pointers of list position p (sel: its staged row when gathering,
// already checked against the visible entries; -1 = masked).
template <bool kRope>
__device__ __forceinline__ RowPtrs row_ptrs(const RowSource rs, int p, int sel) {
  const bool in = p < rs.p1;
  const bool comp = p < rs.n_comp;
  const int e = rs.gather ? sel : p;
  const int w = p - rs.n_comp;
  const bool ok_c = in && comp && e >= 0 && (rs.gather || e < rs.n_vis);
  const bool ok_w = in && !comp && w < rs.n_w;
  int wr = rs.wlo + w;
  wr = wr >= rs.wrap ? wr - rs.wrap : wr;
  const uint32_t row = ok_c ? (uint32_t)e : ok_w ? (uint32_t)wr : 0u;
  const uint32_t stride = ok_c ? rs.kvs : rs.wns;
  const uint64_t off = (uint64_t)row * stride;
  RowPtrs r;
  r.pn = (ok_c ? rs.kvb0 : ok_w ? rs.wb0 : rs.dummy) + off;
  r.pr = kRope ? (ok_c ? rs.kvb1 : ok_w ? rs.wb1 : rs.dummy) + off : 0;
  r.live = (uint32_t)__ballot(ok_c || ok_w);
  return r;
}

// Row pointers of the tile whose lane 0 has list position p0 (uniform over
// the wave); lane r32 takes position p0 + r32.  A tile wholly inside the
// visible entries of a list that is not gathered takes one multiply-add per
// pointer; any other tile (gathered rows, the window, the list's end) the
// general form above.  The same pointers either way.
template <bool kRope>
__device__ __forceinline__ RowPtrs row_ptrs_tile(const RowSource rs, int p0, int r32, int sel) {
  if (!rs.gather && p0 + kTile <= rs.n_comp && p0 + kTile <= rs.n_vis && p0 + kTile <= rs.p1) {
    const uint64_t off = (uint64_t)(uint32_t)(p0 + r32) * rs.kvs;
    RowPtrs r;
    r.pn = rs.kvb0 + off;
    r.pr = kRope ? rs.kvb1 + off : 0;
    r.live = 0xffffffffu;
    return r;
  }
  return row_ptrs<kRope>(rs, p0 + r32, sel);
}

}  // namespace csa
