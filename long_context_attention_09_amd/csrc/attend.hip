// Shared-KV multi-query attention with a per-head sink: CSA (gathered top-k
// entries + raw window) and HCA (every visible entry + raw window).
//
// What is computed ("DeepSeek-V4 深读", ricardokevins.github.io, CSA/HCA
// section and its stability paragraph; "拆解 DeepSeekv4", daixd5520.github.io,
// section 细节): all query heads read one shared 512-d vector per entry that
// serves as key and value; the last 64 dims of the query carry RoPE at the
// query position and the output's last 64 dims are rotated back; exp(sink_h)
// joins every head's softmax denominator.
//
// FP8_BF16 kernel (gfx950 matrix cores).  A workgroup owns one query, 64
// heads and one contiguous split of the query's KV list.  KV rows stream
// through LDS in tiles of 32 entries: every thread fetches its share of the
// 576-byte rows (448 E4M3FN bytes + 64 BF16 values) with 16-byte loads into
// registers three tiles ahead, then widens FP8 to BF16 (exact, hardware
// converter) into a row-major LDS tile whose 16-byte chunks are swizzled per
// row.  Per tile the eight wavefronts first form the scores
//   S^T[32 entries x 64 heads] = K Q^T       (V_MFMA_F32_32X32X16_BF16)
// split as 2 head halves x 4 dim quarters, with the normalised, rotated
// query held in registers as the B operand; the dim-quarter partials are
// summed through LDS by the wave that runs the online softmax (log2 domain,
// lazy rescale) of 8 heads, which leaves P in LDS as BF16.  Then
//   O^T[512 dims x 64 heads] += V^T P^T
// is split by dims only (64 per wave), with V^T read once through
// ds_read_b64_tr_b16 transposing reads.
//
// A split that covers the whole list finalises in place (sink, normalisation,
// inverse RoPE, BF16 store); otherwise (running max, sum, normalised output) partials
// go to the workspace and combine_kernel merges them.
#include <hip/hip_ext.h>

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

struct ListInfo {
  int n_comp;     // compressed part of the list (top_k for CSA, n_vis for HCA)
  int n_vis;      // visible compressed entries
  int win_lo;     // first window buffer row
  int n_w;        // window rows present
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
  const int64_t wp0 = a.win_pos0[b];
  int64_t lo = t - a.n_win + 1;
  lo = lo > 0 ? lo : 0;
  lo = lo > wp0 ? lo : wp0;
  int64_t hi = t < wp0 + a.win_len - 1 ? t : wp0 + a.win_len - 1;
  L.win_lo = (int)(lo - wp0);
  L.n_w = hi >= lo ? (int)(hi - lo + 1) : 0;
  return L;
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
    const int64_t off = (int64_t)b * a.kv_seq_stride + (int64_t)e * a.kv_stride;
    *pn = (const uint8_t*)a.kv0 + off;
    *pr = (const uint8_t*)a.kv1 + off;
    return true;
  }
  const int w = p - L.n_comp;
  if (w >= L.n_w) return false;
  const int64_t off = (int64_t)b * a.win_seq_stride + (int64_t)(L.win_lo + w) * a.win_stride;
  *pn = (const uint8_t*)a.win0 + off;
  *pr = (const uint8_t*)a.win1 + off;
  return true;
}

typedef __attribute__((address_space(1))) const i32x4 gbl_i32x4;

constexpr float kRescaleSlack = 8.0f;   // log2 units a running max may lag the true max

// Workgroup of 8 wavefronts with two roles per 32-entry tile:
//  * scores: wave w forms S^T = K Q^T for the 32 heads 32 (w >> 2) .. +31 over
//    the 128 dims 128 (w & 3) .. +127 (V_MFMA_F32_32X32X16_BF16, 8 per tile);
//    the four partial blocks of a head half meet in LDS, and wave w sums the
//    8 heads 32 (w >> 2) + 8 (w & 3) .. +7 and runs their online softmax,
//    leaving P (BF16) and each head's rescale factor in LDS;
//  * output: wave w accumulates O^T += V^T P^T for the 64 dims 64 w .. +63 of
//    all 64 heads, so every V element leaves LDS once per workgroup, through
//    ds_read_b64_tr_b16 transposing reads.
// The output product of tile t-1 runs in the same phase as the softmax of
// tile t (matrix cores and vector ALUs overlap); three tile buffers keep
// tile t-1 readable while tile t+1 is being widened.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = kD * 2 + 16;                    // BF16 row in LDS + 16-byte pad
constexpr int kTileBytes = kTile * kRowBytes;             // 32.5 KiB
constexpr int kTileBufs = 3;
constexpr int kXsWave = 32 * 128;                         // one wave's partial scores (bytes)
constexpr int kPRow = 80;                                 // bytes per head in P: 32 BF16 + pad
constexpr int kPBytes = 64 * kPRow;

// Row loads: thread t owns the sixteen-byte chunks t, t + 512 (and threads
// 128 .. 255 also t + 896) of a tile (chunk c = row c / 36, part c % 36:
// parts 0..27 hold FP8 dims, 28..35 BF16 RoPE dims) and keeps kStages tiles of
// them in flight in registers.
constexpr int kChunkSlots = (kChunksPerTile + kThreads - 1) / kThreads;   // 3
constexpr int kStages = 2;
constexpr int kAddrSlots = 8;                             // row-address ring (tiles)
constexpr int kIdxMax = kAttendIdxMax;                    // selected indices staged per split

// Entry slot k (0..31) of a tile lives in LDS row 16 (k / 16) + 2 h + u + 4 q,
// where k % 16 = 8 h + 4 u + q.  Slot order is the order the matrix cores sum
// over (the score MFMA's rows, P's columns, the output MFMA's K index); the
// row placement makes each 32-lane half of a transposing read (4 rows x 64
// bytes) and each 16-lane row read fall on distinct banks with rows padded
// to 1040 bytes, so every fragment address is one register plus immediates.
__device__ __forceinline__ int slot_row(int k) {
  return 16 * (k >> 4) + 2 * ((k >> 3) & 1) + ((k >> 2) & 1) + 4 * (k & 3);
}

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

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;


__global__ void __launch_bounds__(kThreads, 1) attend_fp8_kernel(AttendLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kTileBufs * kTileBytes];  // BF16 rows
  __shared__ __attribute__((aligned(16))) uint8_t xs[kWaves * kXsWave];           // partial scores
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * kPBytes];              // P, two buffers
  __shared__ float alpha_s[2 * 64];                                               // rescale factors
  __shared__ float ml_s[2 * 64];                                                  // final (max, sum)
  __shared__ uint64_t rowa[kAddrSlots * 2 * kTile];                               // [slot][nope|rope][row]
  __shared__ uint32_t rowmask[kAddrSlots];                                        // live rows per tile
  __shared__ float rope_cs[64];                                                   // cos, sin at t
  __shared__ int lidx[kIdxMax];                                                   // staged indices (CSA)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = wave >> 2, dq = wave & 3;
  const int split = blockIdx.x, hg = blockIdx.y;
  const int br = blockIdx.z;
  const int b = br / a.n_q, r = br % a.n_q;
  const ListInfo L = list_info(a, b, r);
  const int list_len = L.n_comp + L.n_w;
  const int p0 = split * a.split_len;
  int p1 = p0 + a.split_len;
  p1 = p1 < list_len ? p1 : list_len;
  const int n_tiles = p1 > p0 ? (p1 - p0 + kTile - 1) / kTile : 0;

  // Prologue, ordered so the query's and the first tiles' loads are in flight
  // while the RoPE table, the row addresses and the query's norm are formed.
  // The query operand of the score role: head 32 hh + (lane % 32), dims
  // 128 dq + 16 s + 8 (lane / 32) + j; RMSNorm over all 512 dims (the four
  // dim quarters add their sums of squares through LDS), RoPE at t, BF16.
  const int head_q = hg * 64 + 32 * hh + (lane & 31);
  const bool q_ok = head_q < a.H;
  i32x4 qraw[8];
  bf16x8 qv[8];                              // formed once the row fetches are issued
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.n_q + r) * a.H + (q_ok ? head_q : 0)) * kD +
                           128 * dq + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) qraw[s] = *(gbl_i32x4*)(qrow + 16 * s);
  }
  // RoPE table at the query position, one pair per thread
  if (tid < kDR / 2) {
    float cs, sn;
    rope_cos_sin((double)L.t, tid, kDR, a.log_theta, &cs, &sn);
    rope_cs[tid] = cs;
    rope_cs[32 + tid] = sn;
  }
  // the split's selected indices (CSA), staged once
  if (a.idx) {
    const int* src = a.idx + ((int64_t)b * a.n_q + r) * a.top_k;
    const int n_sel = (p1 < L.n_comp ? p1 : L.n_comp) - p0;
    for (int i = tid; i < n_sel; i += kThreads) lidx[i] = src[p0 + i];
  }
  ATTEND_BARRIER(kWaitLgkm0);

  // Row addresses of tile t (list positions p0 + 32t ...): 0 marks a masked row.
  auto tile_addrs = [&](int t) {
    if (tid < kTile) {
      const int p = p0 + t * kTile + tid;
      uint64_t an = 0, ar = 0;
      if (p < p1) {
        if (p < L.n_comp) {
          const int e = a.idx ? lidx[p - p0] : p;
          if (!a.idx || (e >= 0 && e < L.n_vis)) {
            const int64_t off = (int64_t)b * a.kv_seq_stride + (int64_t)e * a.kv_stride;
            an = (uint64_t)((const uint8_t*)a.kv0 + off);
            ar = (uint64_t)((const uint8_t*)a.kv1 + off);
          }
        } else {
          const int w = p - L.n_comp;
          if (w < L.n_w) {
            const int64_t off = (int64_t)b * a.win_seq_stride + (int64_t)(L.win_lo + w) * a.win_stride;
            an = (uint64_t)((const uint8_t*)a.win0 + off);
            ar = (uint64_t)((const uint8_t*)a.win1 + off);
          }
        }
      }
      // list position p0 + 32 t + tid fills entry slot tid, i.e. LDS row slot_row(tid)
      uint64_t* slot = rowa + (t % kAddrSlots) * 2 * kTile;
      slot[slot_row(tid)] = an;
      slot[kTile + slot_row(tid)] = ar;
      const uint64_t live = __ballot(an != 0);      // bit k: entry slot k is a real row
      if (tid == 0) rowmask[t % kAddrSlots] = (uint32_t)live;
    }
  };
#pragma unroll
  for (int t = 0; t < kStages + 2; ++t) tile_addrs(t);
  ATTEND_BARRIER(kWaitLgkm0);

  // this thread's chunks of a tile
  int ch_slot[kChunkSlots], ch_src[kChunkSlots], ch_dst[kChunkSlots];
  bool ch_ok[kChunkSlots], ch_rope[kChunkSlots];
#pragma unroll
  for (int k = 0; k < kChunkSlots; ++k) {
    // chunks 0 .. 1023 to every thread twice, 1024 .. 1151 to waves 2 and 3
    // (wave 0 also builds the row addresses)
    const int c = k < 2 ? tid + kThreads * k : 2 * kThreads + tid - 128;
    ch_ok[k] = k < 2 || (tid >= 128 && tid < 128 + kChunksPerTile - 2 * kThreads);
    const int cc = ch_ok[k] ? c : 0;
    const int part = cc % kChunksPerRow;
    const int row = cc / kChunksPerRow;
    ch_rope[k] = part >= 28;
    ch_slot[k] = (ch_rope[k] ? kTile : 0) + row;
    ch_src[k] = part < 28 ? part * 16 : (part - 28) * 16;
    ch_dst[k] = row * kRowBytes + (part < 28 ? part * 32 : kDN * 2 + (part - 28) * 16);
  }
  // Request tile t's chunks into registers.  Every load is issued (a masked
  // row or a missing chunk reads harmless bytes: the query) so the count of
  // loads in flight is the same on every path; bit k of the result says
  // whether chunk k is real data.
  const uint64_t dummy = (uint64_t)a.q;      // any readable bytes (q holds >= 16 KiB)
  auto fetch = [&](int t, i32x4 (&v)[kChunkSlots]) {
    const uint64_t* slot_a = rowa + (t % kAddrSlots) * 2 * kTile;
    uint64_t base[kChunkSlots];
#pragma unroll
    for (int k = 0; k < kChunkSlots; ++k) base[k] = slot_a[ch_slot[k]];   // all requested at once
    int live = 0;
#pragma unroll
    for (int k = 0; k < kChunkSlots; ++k) {
      const uint64_t bk = ch_ok[k] ? base[k] : 0;
      live |= (bk != 0) << k;
      v[k] = *(gbl_i32x4*)((bk ? bk : dummy) + (uint64_t)ch_src[k]);
    }
    return live;
  };
  // Widen tile t's chunks to BF16 rows in buffer t % 3 (FP8 dims exactly;
  // zeros for masked rows).
  auto commit = [&](int t, const i32x4 (&vin)[kChunkSlots], int live) {
    uint8_t* tile = tiles + (t % kTileBufs) * kTileBytes;
#pragma unroll
    for (int k = 0; k < kChunkSlots; ++k) {
      if (!ch_ok[k]) continue;
      const i32x4 zero = {0, 0, 0, 0};
      const i32x4 vk = (live >> k) & 1 ? vin[k] : zero;
      const i32x4 v[1] = {vk};
      if (!ch_rope[k]) {
        // two E4M3 bytes -> two BF16 per instruction (scale 1: exact)
        i32x4 lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int w0 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[0][j], 1.0f, false));
          const int w1 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[0][j], 1.0f, true));
          if (j < 2) { lo[2 * j] = w0; lo[2 * j + 1] = w1; }
          else { hi[2 * (j - 2)] = w0; hi[2 * (j - 2) + 1] = w1; }
        }
        *(i32x4*)(tile + ch_dst[k]) = lo;
        *(i32x4*)(tile + ch_dst[k] + 16) = hi;
      } else {
        *(i32x4*)(tile + ch_dst[k]) = v[0];
      }
    }
  };

  // ---- score role: partial S^T of tile t over this wave's dims, into xs
  struct KIn {
    bf16x8 kf[8];
  };
  auto scores_load = [&](int t) {
    KIn in;
    const uint8_t* tile = tiles + (t % kTileBufs) * kTileBytes;
    const uint8_t* krow = tile + slot_row(lane & 31) * kRowBytes + 2 * (128 * dq + 8 * (lane >> 5));
#pragma unroll
    for (int s = 0; s < 8; ++s) in.kf[s] = *(const bf16x8*)(krow + 32 * s);
    return in;
  };
  auto scores_mma = [&](const KIn& in) {
    f32x16 s0 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(in.kf[s], qv[s], s0, 0, 0, 0);
    // lane holds head (lane % 32), entry slots 8 jb + 4 (lane / 32) + i, i.e.
    // the 16-byte group k = 2 jb + lane / 32 of that head's 32 scores
    uint8_t* xw = xs + wave * kXsWave + (lane & 31) * 128;
    const int sw = ((lane & 31) >> 1) & 7;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      *(f32x4*)(xw + 16 * ((2 * jb + (lane >> 5)) ^ sw)) =
          (f32x4){s0[4 * jb], s0[4 * jb + 1], s0[4 * jb + 2], s0[4 * jb + 3]};
  };

  // ---- softmax role: head sm_head of the group, entries 4 sm_k .. +3
  const int sm_hloc = 8 * dq + (lane >> 3);                 // head within the head half
  const int sm_head = 32 * hh + sm_hloc;                    // head within the group
  const int sm_k = lane & 7;
  float m_run = -INFINITY;     // log2-domain reference max (lags the true max by < the slack)
  float l_part = 0.f;          // this lane's share of the running denominator
  // part 1: the four partial score blocks of the head and the live-row mask
  struct SmIn {
    f32x4 x[4];
    uint32_t live;
  };
  auto sm_load = [&](int t) {
    SmIn in;
    const int swr = (sm_hloc >> 1) & 7;
#pragma unroll
    for (int src = 0; src < 4; ++src)
      in.x[src] = *(const f32x4*)(xs + (hh * 4 + src) * kXsWave + sm_hloc * 128 + 16 * (sm_k ^ swr));
    in.live = rowmask[t % kAddrSlots];
    return in;
  };
  // part 2: online softmax, P and the rescale factor to LDS
  auto sm_compute = [&](int t, const SmIn& in) {
    const f32x4 sc = ((in.x[0] + in.x[1]) + in.x[2]) + in.x[3];
    float v[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (in.live >> (4 * sm_k + i)) & 1 ? sc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, v[i]);
    }
    mx = fmaxf(mx, dpp_f32<0xB1>(mx));     // lane ^ 1
    mx = fmaxf(mx, dpp_f32<0x4E>(mx));     // lane ^ 2
    mx = fmaxf(mx, dpp_f32<0x141>(mx));    // lane 7 - i of each 8: the other quad
    // the reference max moves only when the tile max overtakes it by the slack,
    // so O rescales are rare; probabilities stay below 2^slack
    const float m_new = mx > m_run + kRescaleSlack ? mx : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);   // argument <= 0, or -inf
    float p[4], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(v[i] - m_use);
      psum += p[i];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    const bf16x4 pk = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};   // nearest even
    *(bf16x4*)(pbuf + (t & 1) * kPBytes + sm_head * kPRow + 8 * sm_k) = pk;
    if (sm_k == 0) alpha_s[(t & 1) * 64 + sm_head] = alpha;
  };

  // ---- output role: O^T (dims 64 wave + 32 db + ..., heads 32 hb + ...) += V^T P^T
  f32x16 acc_o[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) acc_o[db][hb] = (f32x16){};
  struct PvIn {
    i16x4 vlo[2][2], vhi[2][2];   // [rs][db]
    bf16x8 pf[2][2];              // [rs][hb]
    float al0, al1;
  };
  // part 1: V^T fragments (transposing reads), P^T fragments, rescale factors
  auto pv_load = [&](int tbuf, int pidx) {
    PvIn in;
    const uint8_t* tile = tiles + tbuf * kTileBytes;
    const uint8_t* pb = pbuf + pidx * kPBytes;
    // transposing reads: lane j of 16-lane group G supplies entry slot
    // 16 rs + 8 (G / 2) + 4 u + j / 4 (u = 0, 1 for the two reads) at the 4
    // dims 64 wave + 32 db + 16 (G % 2) + 4 (j % 4) ..; lane j of the group
    // receives dim j's values of the four slots
    const int G = lane >> 4, j = lane & 15;
    const uint8_t* vb = tile + slot_row(8 * (G >> 1) + (j >> 2)) * kRowBytes +
                        2 * (64 * wave + 16 * (G & 1) + 4 * (j & 3));
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint8_t* v0 = vb + 16 * rs * kRowBytes + 64 * db;
        in.vlo[rs][db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)v0);
        in.vhi[rs][db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + kRowBytes));   // u = 1: next row
      }
    // P^T: lane supplies head 32 hb + lane % 32, entries 16 rs + 8 (lane / 32) .. +7
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        in.pf[rs][hb] = *(const bf16x8*)(pb + (32 * hb + (lane & 31)) * kPRow + 2 * (16 * rs + 8 * (lane >> 5)));
    in.al0 = alpha_s[pidx * 64 + (lane & 31)];
    in.al1 = alpha_s[pidx * 64 + 32 + (lane & 31)];
    return in;
  };
  // part 2: rescale when a running max moved, then 8 MFMAs
  auto pv_mma = [&](const PvIn& in) {
    if (__any(in.al0 != 1.0f || in.al1 != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        acc_o[db][0] *= in.al0;
        acc_o[db][1] *= in.al1;
      }
    }
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        bf16x8 vt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vt[i] = u16_as_bf16((uint16_t)in.vlo[rs][db][i]);
          vt[4 + i] = u16_as_bf16((uint16_t)in.vhi[rs][db][i]);
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          acc_o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, in.pf[rs][hb], acc_o[db][hb], 0, 0, 0);
      }
  };

  // One pipeline step.  Phase 1: every LDS read of the step's matrix work
  // goes out at once (K of tile t; V, P and the rescale factors of tile t-1,
  // whose P was written in the previous step), then O += V P for tile t-1 and
  // the scores of tile t run on the matrix cores while tile t+1 (fetched
  // kStages steps ago) is widened into its buffer and tile t + 1 + kStages is
  // requested into the freed registers.  Barrier.  Phase 2: the softmax of
  // tile t.  Barrier.  The body is the same on every step: tile -1 is an
  // all-zero tile with P = 0 and rescale factors 1, and tiles past the list
  // are masked (scores -inf: P = 0, the running max and sum unchanged).
  auto step = [&](int t, i32x4 (&cur)[kChunkSlots], int& cur_live) {
    const PvIn pin = pv_load((t + 2) % kTileBufs, (t + 1) & 1);   // tile t - 1
    const KIn kin = scores_load(t);
    pv_mma(pin);
    scores_mma(kin);
    commit(t + 1, cur, cur_live);
    tile_addrs(t + kStages + 2);
    cur_live = fetch(t + 1 + kStages, cur);
    ATTEND_BARRIER(kWaitLgkm0);
    sm_compute(t, sm_load(t));
    ATTEND_BARRIER(kWaitLgkm0);
  };

  // Prologue (continued): tiles 0 .. kStages requested, the query operand
  // formed meanwhile, tile 0 widened into buffer 0.  Register slot j carries
  // tiles j, j + kStages, ... (the step loop is unrolled by kStages so every
  // slot is a fixed set of registers).
  static_assert(kStages == 2, "the step loop below is unrolled for two register stages");
  i32x4 st0[kChunkSlots], st1[kChunkSlots];
  int lv0, lv1;
  i32x4 first[kChunkSlots];
  const int lf = fetch(0, first);
  lv1 = fetch(1, st1);
  lv0 = fetch(2, st0);
  {
    float x[8][8];
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      i32x4 v = qraw[s];
      if (!q_ok) v = (i32x4){0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[s][2 * j] = __uint_as_float(((uint32_t)v[j]) << 16);
        x[s][2 * j + 1] = __uint_as_float(((uint32_t)v[j]) & 0xffff0000u);
        ss += x[s][2 * j] * x[s][2 * j] + x[s][2 * j + 1] * x[s][2 * j + 1];
      }
    }
    ss += __shfl_xor(ss, 32, 64);
    float* ssx = (float*)xs;                 // [hh][dq][32], before the tile loop uses xs
    if (lane < 32) ssx[(hh * 4 + dq) * 32 + lane] = ss;
    ATTEND_BARRIER(kWaitLgkm0);
    ss = ((ssx[(hh * 4 + 0) * 32 + (lane & 31)] + ssx[(hh * 4 + 1) * 32 + (lane & 31)]) +
          ssx[(hh * 4 + 2) * 32 + (lane & 31)]) + ssx[(hh * 4 + 3) * 32 + (lane & 31)];
    const float rs = (a.flags & CSA_ATTEND_NORM_Q) ? 1.0f / sqrtf(ss / (float)kD + 1e-6f) : 1.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[s][j] *= rs;
    if (dq == 3) {                           // dims 448 .. 511 carry RoPE
#pragma unroll
      for (int s = 4; s < 8; ++s) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int u = (128 * 3 + 16 * s + 8 * (lane >> 5) + j - kDN) >> 1;
          const float cs = rope_cs[u], sn = rope_cs[32 + u];
          const float xe = x[s][j], xo = x[s][j + 1];
          x[s][j] = xe * cs - xo * sn;
          x[s][j + 1] = xe * sn + xo * cs;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[s][j] = u16_as_bf16(f32_to_bf16(x[s][j]));
  }
  ATTEND_BARRIER(kWaitLgkm0);               // every wave has read the sums before xs is reused
  commit(0, first, lf);
  // tile -1 of the first step's output product: zero rows, P = 0, factors 1
  for (int i = tid; i < kTileBytes / 16; i += kThreads)
    *(i32x4*)(tiles + 2 * kTileBytes + 16 * i) = (i32x4){0, 0, 0, 0};
  for (int i = tid; i < kPBytes / 16; i += kThreads) *(i32x4*)(pbuf + kPBytes + 16 * i) = (i32x4){0, 0, 0, 0};
  if (tid < 64) alpha_s[64 + tid] = 1.0f;
  ATTEND_BARRIER(kWaitLgkm0);
  // Whole rounds of kStages steps (n_tiles + 1 steps are needed: the last one
  // only accumulates the final tile), so every path issues the same loads and
  // the compiler's count of loads in flight stays exact.
  for (int t = 0; t <= n_tiles; t += kStages) {
    step(t, st1, lv1);               // widens t+1 (slot 1), then fetches t+3 into it
    step(t + 1, st0, lv0);
  }

  // the trailing fetches (past the list) must land before the wave ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- epilogue: the softmax role publishes each head's (max, sum)
  {
    float l_run = l_part;
    l_run += __shfl_xor(l_run, 1, 64);
    l_run += __shfl_xor(l_run, 2, 64);
    l_run += __shfl_xor(l_run, 4, 64);
    if (sm_k == 0) {
      ml_s[2 * sm_head] = m_run;
      ml_s[2 * sm_head + 1] = l_run;
    }
  }
  __syncthreads();
  const int64_t unit = (int64_t)br * gridDim.y + hg;
  const bool inv_rope = !(a.flags & CSA_ATTEND_NO_INV_ROPE);
  const bool single = a.n_splits == 1;
  // The normalised output (BF16 with the sink and inverse RoPE when the split
  // covers the whole list, else the fp16 partial) is staged in LDS as
  // [64 heads][512 dims] rows of 1040 bytes (the tile buffers are free now),
  // so the global stores are contiguous 16-byte chunks.
  uint8_t* stage = tiles;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hl = 32 * hb + (lane & 31);
    const int head = hg * 64 + hl;
    const float m_h = ml_s[2 * hl], l_h = ml_s[2 * hl + 1];
    float scale;
    if (single) {
      const float z2 = head < a.H ? a.sink[head] * kLog2e : 0.f;
      const float top = fmaxf(m_h, z2);
      const float den = l_h * exp2f(m_h - top) + exp2f(z2 - top);
      scale = exp2f(m_h - top) / den;                 // 0 when no row was seen
    } else {
      scale = l_h > 0.f ? 1.0f / l_h : 0.f;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int d0 = 64 * wave + 32 * db + 8 * jb + 4 * (lane >> 5);
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc_o[db][hb][4 * jb + i] * scale;
        uint32_t w0, w1;
        if (single) {
          if (d0 >= kDN && inv_rope) {
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const int u = (d0 + i - kDN) >> 1;
              const float cs = rope_cs[u], sn = -rope_cs[32 + u];   // rotation by -t
              const float xe = o[i], xo = o[i + 1];
              o[i] = xe * cs - xo * sn;
              o[i + 1] = xe * sn + xo * cs;
            }
          }
          w0 = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
          w1 = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        } else {
          typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
          w0 = __builtin_bit_cast(uint32_t, (f16x2){(_Float16)o[0], (_Float16)o[1]});
          w1 = __builtin_bit_cast(uint32_t, (f16x2){(_Float16)o[2], (_Float16)o[3]});
        }
        *(u32x2*)(stage + hl * kRowBytes + 2 * d0) = (u32x2){w0, w1};
      }
    if (dq == 0 && (lane >> 5) == 0 && hh == 0 && head < a.H) {   // wave 0, one lane per head
      if (single) {
        if (a.out_lse)
          a.out_lse[((int64_t)b * a.n_q + r) * a.H + head] =
              l_h > 0.f ? (m_h + log2f(l_h)) * 0.6931471805599453f : -INFINITY;
      } else {
        const int64_t ps = (unit * a.n_splits + split) * 64 + hl;
        a.part_ml[ps * 2] = m_h;
        a.part_ml[ps * 2 + 1] = l_h;
      }
    }
  }
  ATTEND_BARRIER(kWaitLgkm0);
  // 64 rows x 64 chunks of 16 bytes, 8 per thread, consecutive threads on
  // consecutive chunks of a row
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = tid + kThreads * k;
    const int hl = c >> 6, ch = c & 63;
    const int head = hg * 64 + hl;
    if (head >= a.H) continue;
    const i32x4 v = *(const i32x4*)(stage + hl * kRowBytes + 16 * ch);
    if (single) {
      uint16_t* orow = (uint16_t*)a.out + (((int64_t)b * a.n_q + r) * a.H + head) * kD;
      *(i32x4*)(orow + 8 * ch) = v;
    } else {
      _Float16* po = a.part_o + ((unit * a.n_splits + split) * 64 + hl) * kD;
      *(i32x4*)(po + 8 * ch) = v;
    }
  }
}

// Merge the split partials: workgroup (unit, head quad), 64 threads per head,
// 8 dims each.
__global__ void __launch_bounds__(256) combine_kernel(AttendLaunch a, int n_hg) {
  __shared__ float rope_cs[64];
  const int unit = blockIdx.x;                 // br * n_hg + hg
  const int br = unit / n_hg, hg = unit % n_hg;
  const int b = br / a.n_q, r = br % a.n_q;
  const int hl = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  const int head = hg * 64 + hl;
  const int64_t t = a.q_pos[(int64_t)b * a.n_q + r];
  if (threadIdx.x < 32) {
    float cs, sn;
    rope_cos_sin(-(double)t, threadIdx.x, kDR, a.log_theta, &cs, &sn);
    rope_cs[threadIdx.x] = cs;
    rope_cs[32 + threadIdx.x] = sn;
  }
  __syncthreads();
  if (head >= a.H) return;
  const int64_t base = (int64_t)unit * a.n_splits * 64 + hl;
  // Splits are merged eight at a time, every load of a group in flight
  // together, against a running maximum: M over the sink logit and the
  // splits' maxima (output and denominator), Mx over the splits only (LSE).
  typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
  constexpr int kGroup = 8;
  const float z2 = a.sink[head] * kLog2e;
  float M = z2, den = 1.0f;                 // den = exp2(z2 - M) + sum l_s exp2(m_s - M)
  float Mx = -INFINITY, lsum = 0.f;         // lsum = sum l_s exp2(m_s - Mx)
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.n_splits; s0 += kGroup) {
    float ms[kGroup], ls[kGroup];
    f16x8 v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int sj = s0 + j < a.n_splits ? s0 + j : s0;
      const int64_t rj = base + (int64_t)sj * 64;
      ms[j] = a.part_ml[rj * 2];
      ls[j] = a.part_ml[rj * 2 + 1];
      v[j] = *(const f16x8*)(a.part_o + rj * kD + d0);
    }
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (s0 + j >= a.n_splits) ms[j] = -INFINITY;
      cm = fmaxf(cm, ms[j]);
    }
    if (cm == -INFINITY) continue;          // no split of the group saw a row
    const float nM = fmaxf(M, cm);
    const float sc = exp2f(M - nM);
    const float nMx = fmaxf(Mx, cm);
    const float scx = Mx == -INFINITY ? 0.f : exp2f(Mx - nMx);
    den *= sc;
    lsum *= scx;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= sc;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (ms[j] == -INFINITY) continue;
      // the partial is normalised: its numerator is o * l
      const float f = ls[j] * exp2f(ms[j] - nM);
      den += f;
      lsum += ls[j] * exp2f(ms[j] - nMx);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] += (float)v[j][i] * f;
    }
    M = nM;
    Mx = nMx;
  }
  const float mmax = Mx;
  const float inv = 1.0f / den;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= inv;
  if (d0 >= kDN && !(a.flags & CSA_ATTEND_NO_INV_ROPE)) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int u = (d0 + i - kDN) >> 1;
      const float cs = rope_cs[u], sn = rope_cs[32 + u];
      const float xe = o[i], xo = o[i + 1];
      o[i] = xe * cs - xo * sn;
      o[i + 1] = xe * sn + xo * cs;
    }
  }
  uint16_t* orow = (uint16_t*)a.out + (((int64_t)b * a.n_q + r) * a.H + head) * kD + d0;
  i32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (int)((uint32_t)f32_to_bf16(o[2 * j]) | ((uint32_t)f32_to_bf16(o[2 * j + 1]) << 16));
  *(i32x4*)orow = w;
  if (a.out_lse && (threadIdx.x & 63) == 0)
    a.out_lse[((int64_t)b * a.n_q + r) * a.H + head] =
        lsum > 0.f ? (mmax + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
}

// ------------------------------------------------------------------ fp32 precision mode

// One workgroup per (query, head); rows in chunks of 256 with an online softmax.
__global__ void __launch_bounds__(256) attend_f32_kernel(AttendLaunch a) {
  __shared__ float qs[kD];
  __shared__ float ps[256];
  __shared__ float red[8];
  __shared__ const float* rowp[256];
  const int br = blockIdx.x, head = blockIdx.y;
  const int b = br / a.n_q, r = br % a.n_q;
  const int tid = threadIdx.x;
  const int d = a.d, d0 = a.d - a.d_rope;
  const ListInfo L = list_info(a, b, r);
  const float* q = (const float*)a.q + (((int64_t)b * a.n_q + r) * a.H + head) * d;
  auto block_sum = [&](float v) {
    v = wave_sum(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
  };
  auto block_max = [&](float v) {
    v = wave_max(v);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  };
  float ss = 0.f;
  for (int c = tid; c < d; c += 256) ss += q[c] * q[c];
  ss = block_sum(ss);
  const float rs = (a.flags & CSA_ATTEND_NORM_Q) ? 1.0f / sqrtf(ss / (float)d + 1e-6f) : 1.0f;
  for (int c = tid; c < d; c += 256) {
    float v = q[c] * rs;
    if (c >= d0) {
      const int pc = c ^ 1;
      const float w = q[pc] * rs;
      float cs, sn;
      rope_cos_sin((double)L.t, (c - d0) >> 1, a.d_rope, a.log_theta, &cs, &sn);
      v = (c & 1) == 0 ? v * cs - w * sn : w * sn + v * cs;
    }
    qs[c] = v;
  }
  __syncthreads();
  const int list_len = L.n_comp + L.n_w;
  float m_run = -INFINITY, l_run = 0.f;
  float o0 = 0.f, o1 = 0.f;     // dims tid and tid + 256
  for (int c0 = 0; c0 < list_len; c0 += 256) {
    const int p = c0 + tid;
    float s = -INFINITY;
    const uint8_t *pn = nullptr, *pr = nullptr;
    if (p < list_len && list_row(a, b, r, L, p, &pn, &pr)) {
      const float* row = (const float*)pn;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(qs[c], row[c], dot);
      s = dot * a.scale_log2;
      rowp[tid] = row;
    } else {
      rowp[tid] = nullptr;
    }
    const float mx = block_max(s);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float p_ = exp2f(s - m_use);
    ps[tid] = p_;
    const float psum = block_sum(p_);
    const float alpha = exp2f(m_run - m_use);
    l_run = l_run * alpha + psum;
    o0 *= alpha;
    o1 *= alpha;
    m_run = m_new;
    __syncthreads();
    const int n = list_len - c0 < 256 ? list_len - c0 : 256;
    for (int j = 0; j < n; ++j) {
      const float* row = rowp[j];
      if (!row) continue;
      const float pj = ps[j];
      if (tid < d) o0 = fmaf(pj, row[tid], o0);
      if (tid + 256 < d) o1 = fmaf(pj, row[tid + 256], o1);
    }
    __syncthreads();
  }
  const float z2 = a.sink[head] * kLog2e;
  const float top = fmaxf(m_run, z2);
  const float den = l_run * exp2f(m_run - top) + exp2f(z2 - top);
  const float inv = exp2f(m_run - top) / den;
  __shared__ float os[kD];
  if (tid < d) os[tid] = o0 * inv;
  if (tid + 256 < d) os[tid + 256] = o1 * inv;
  __syncthreads();
  float* orow = (float*)a.out + (((int64_t)b * a.n_q + r) * a.H + head) * d;
  for (int c = tid; c < d; c += 256) {
    float v = os[c];
    if (c >= d0 && !(a.flags & CSA_ATTEND_NO_INV_ROPE)) {
      const float w = os[c ^ 1];
      float cs, sn;
      rope_cos_sin(-(double)L.t, (c - d0) >> 1, a.d_rope, a.log_theta, &cs, &sn);
      v = (c & 1) == 0 ? v * cs - w * sn : w * sn + v * cs;
    }
    orow[c] = v;
  }
  if (a.out_lse && tid == 0)
    a.out_lse[((int64_t)b * a.n_q + r) * a.H + head] =
        l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_attend(const AttendLaunch& a, hipStream_t s) {
  if (a.fmt == CSA_FMT_F32) {
    dim3 grid(a.B * a.n_q, a.H);
    hipExtLaunchKernelGGL(attend_f32_kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
    return hipGetLastError();
  }
  const int n_hg = (a.H + 63) / 64;
  dim3 grid(a.n_splits, n_hg, a.B * a.n_q);
  hipExtLaunchKernelGGL(attend_fp8_kernel, grid, dim3(kThreads), 0, s, a.ev_start, a.ev_stop, 0, a);
  if (a.n_splits > 1) combine_kernel<<<dim3(a.B * a.n_q * n_hg, 16), 256, 0, s>>>(a, n_hg);
  return hipGetLastError();
}

}  // namespace csa
