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
// heads (16 per wavefront) and one contiguous split of the query's KV list.
// KV rows stream through LDS in tiles of 32 entries: the loader threads fetch
// the 576-byte rows (448 E4M3FN bytes + 64 BF16 values) with 16-byte loads
// into registers while the previous tile is being used, then widen FP8 to
// BF16 (exact) into a row-major LDS tile.  Each wavefront then computes
//   S^T[32 entries x 16 heads] = K Q^T     (V_MFMA_F32_16X16X32_BF16, 32 per tile)
// with its query heads held in registers as the B operand, runs the online
// softmax in the log2 domain, and accumulates
//   O^T[512 dims x 16 heads] += V^T P^T    (32 MFMAs per tile)
// where the B operand P^T is the S^T accumulator itself (the summation order
// over the 32 entries is permuted to match the accumulator layout) and the A
// operand V^T comes from the LDS tile through ds_read_b64_tr_b16 transposing
// reads.  The O^T accumulator keeps one head per lane, so rescaling is a
// per-lane multiply, done only when a running maximum grows.
//
// A split that covers the whole list finalises in place (sink, normalisation,
// inverse RoPE, BF16 store); otherwise (running max, sum, numerator) partials
// go to the workspace and combine_kernel merges them.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kD = 512;
constexpr int kDR = 64;
constexpr int kDN = kD - kDR;         // 448
constexpr int kTile = 32;             // entries per LDS tile
constexpr int kRowBytes = kD * 2 + 16;  // bf16 row + 16 B pad (conflict-free 16-byte row reads)
constexpr int kChunksPerRow = kDN / 16 + (kDR * 2) / 16;  // 28 + 8 = 36 sixteen-byte chunks
constexpr int kChunksPerTile = kTile * kChunksPerRow;     // 1152
constexpr int kLoadsPerThread = (kChunksPerTile + 255) / 256;  // 5 (the last one partial)

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

__device__ __forceinline__ uint32_t pack_hi16(float f0, float f1) {
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

typedef __attribute__((address_space(1))) const i32x4 gbl_i32x4;

constexpr float kRescaleSlack = 8.0f;   // log2 units a running max may lag the true max

// Workgroup of 8 wavefronts: wave w owns 16 heads (w & 3) and one half of the
// 512 dims (w >> 2).  The two waves of a head group each form the scores over
// their half of the dims and swap the partial sums through LDS, so both hold
// the full scores, run the same online softmax, and accumulate the output for
// their own 256 dims.  Two wavefronts per SIMD hide each other's LDS latency.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kDHalf = kD / 2;
constexpr int kTileBytes = kTile * kRowBytes;             // one BF16 tile in LDS

// Row loads: thread t owns the sixteen-byte chunks t, t + 512, t + 1024 of a
// tile (chunk c = row c / 36, part c % 36: parts 0..27 hold FP8 dims, 28..35
// BF16 RoPE dims) and keeps kStages tiles of them in flight in registers.
constexpr int kChunkSlots = (kChunksPerTile + kThreads - 1) / kThreads;   // 3
constexpr int kStages = 3;
constexpr int kAddrSlots = 8;                             // row-address ring (tiles)
constexpr int kIdxMax = kAttendIdxMax;                    // selected indices staged per split

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

__global__ void __launch_bounds__(kThreads, 1) attend_fp8_kernel(AttendLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2 * kTileBytes];  // BF16 rows, two buffers
  __shared__ __attribute__((aligned(16))) float xch[kWaves * 64 * 8];    // score halves
  __shared__ uint64_t rowa[kAddrSlots * 2 * kTile];                      // [slot][nope|rope][row]
  __shared__ float rope_cs[64];                                          // cos, sin at t
  __shared__ int lidx[kIdxMax];                                          // staged indices (CSA)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = wave & 3, dh = wave >> 2;
  const int g = lane >> 4, col = lane & 15;
  const int split = blockIdx.x, hg = blockIdx.y;
  const int br = blockIdx.z;
  const int b = br / a.n_q, r = br % a.n_q;
  const int head = hg * 64 + hq * 16 + col;
  const bool head_ok = head < a.H;
  const ListInfo L = list_info(a, b, r);
  const int list_len = L.n_comp + L.n_w;
  const int p0 = split * a.split_len;
  int p1 = p0 + a.split_len;
  p1 = p1 < list_len ? p1 : list_len;
  const int n_tiles = p1 > p0 ? (p1 - p0 + kTile - 1) / kTile : 0;

  // RoPE table at the query position (fp64 angle), one pair per thread
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
  __syncthreads();

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
      uint64_t* slot = rowa + (t % kAddrSlots) * 2 * kTile;
      slot[tid] = an;
      slot[kTile + tid] = ar;
    }
  };
#pragma unroll
  for (int t = 0; t < kStages + 2; ++t) tile_addrs(t);
  __syncthreads();

  // this thread's chunks of a tile
  int ch_row[kChunkSlots], ch_src[kChunkSlots], ch_dst[kChunkSlots];
  bool ch_ok[kChunkSlots], ch_rope[kChunkSlots];
#pragma unroll
  for (int k = 0; k < kChunkSlots; ++k) {
    const int c = tid + kThreads * k;
    ch_ok[k] = c < kChunksPerTile;
    const int cc = ch_ok[k] ? c : 0;
    const int part = cc % kChunksPerRow;
    ch_row[k] = cc / kChunksPerRow;
    ch_rope[k] = part >= 28;
    ch_src[k] = part < 28 ? part * 16 : (part - 28) * 16;
    ch_dst[k] = ch_row[k] * kRowBytes + (part < 28 ? part * 32 : kDN * 2 + (part - 28) * 16);
  }
  // Request tile t's chunks into registers.  Every load is issued (a masked
  // row or a missing chunk reads harmless bytes: the query) so the count of
  // loads in flight is the same on every path; bit k of the result says
  // whether chunk k is real data.
  const uint64_t dummy = (uint64_t)a.q;      // any readable bytes (q holds >= 16 KiB)
  auto fetch = [&](int t, i32x4 (&v)[kChunkSlots]) {
    const uint64_t* slot_a = rowa + (t % kAddrSlots) * 2 * kTile;
    int live = 0;
#pragma unroll
    for (int k = 0; k < kChunkSlots; ++k) {
      const uint64_t base = ch_ok[k] ? slot_a[(ch_rope[k] ? kTile : 0) + ch_row[k]] : 0;
      live |= (base != 0) << k;
      v[k] = *(gbl_i32x4*)((base ? base : dummy) + (uint64_t)ch_src[k]);
    }
    return live;
  };
  // Widen tile t's chunks to BF16 rows in buffer t % 2 (FP8 dims exactly;
  // zeros for masked rows).
  auto commit = [&](int t, const i32x4 (&vin)[kChunkSlots], int live) {
    uint8_t* tile = tiles + (t & 1) * kTileBytes;
#pragma unroll
    for (int k = 0; k < kChunkSlots; ++k) {
      if (!ch_ok[k]) continue;
      const i32x4 zero = {0, 0, 0, 0};
      const i32x4 vk = (live >> k) & 1 ? vin[k] : zero;
      const i32x4 v[1] = {vk};
      uint8_t* dst = tile + ch_dst[k];
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
        *(i32x4*)dst = lo;
        *(i32x4*)(dst + 16) = hi;
      } else {
        *(i32x4*)dst = v[0];
      }
    }
  };

  // ---- query operand: head `head`, dims 256 dh + 32 kb + 8 g + j, RMSNorm, RoPE at t, BF16
  bf16x8 qv[8];
  {
    const int hq_ = head_ok ? head : 0;
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.n_q + r) * a.H + hq_) * kD;
    float x[8][8];
    float ss = 0.f;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const i32x4 v = *(gbl_i32x4*)(qrow + kDHalf * dh + 32 * kb + 8 * g);
      const i32x4 o = *(gbl_i32x4*)(qrow + kDHalf * (1 - dh) + 32 * kb + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[kb][2 * j] = __uint_as_float(((uint32_t)v[j]) << 16);
        x[kb][2 * j + 1] = __uint_as_float(((uint32_t)v[j]) & 0xffff0000u);
        const float y0 = __uint_as_float(((uint32_t)o[j]) << 16);
        const float y1 = __uint_as_float(((uint32_t)o[j]) & 0xffff0000u);
        ss += x[kb][2 * j] * x[kb][2 * j] + x[kb][2 * j + 1] * x[kb][2 * j + 1] + y0 * y0 + y1 * y1;
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float rs = (a.flags & CSA_ATTEND_NORM_Q) ? 1.0f / sqrtf(ss / (float)kD + 1e-6f) : 1.0f;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[kb][j] *= rs;
    if (dh == 1) {
#pragma unroll
      for (int kb = 6; kb < 8; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int u = (kDHalf + 32 * kb + 8 * g + j - kDN) >> 1;
          const float cs = rope_cs[u], sn = rope_cs[32 + u];
          const float xe = x[kb][j], xo = x[kb][j + 1];
          x[kb][j] = xe * cs - xo * sn;
          x[kb][j + 1] = xe * sn + xo * cs;
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[kb][j] = u16_as_bf16(f32_to_bf16(x[kb][j]));
  }

  f32x4 acc_o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc_o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;     // log2-domain reference max of head `col` (lags the true max by < 8)
  float l_part = 0.f;          // this lane's share of the running denominator
  float* xmine = xch + (wave * 64 + lane) * 8;
  const float* xpart = xch + ((wave ^ 4) * 64 + lane) * 8;

  // One tile of work.  Barriers:
  //   A: tile t's BF16 rows are written (by every wave) and buffer (t+1) % 2
  //      is free again;
  //   B: the score halves are exchanged.
  // Between A and B the scores of tile t are formed and tile t+1 (fetched
  // kStages - 1 tiles ago) is widened into the other buffer; its register
  // slot then fetches tile t + 1 + kStages.  After B: softmax and O += V P.
  auto step = [&](int t, i32x4 (&cur)[kChunkSlots], int& cur_live, bool active) {
    ATTEND_BARRIER(kWaitLgkm0);
    const uint8_t* tile = tiles + (t & 1) * kTileBytes;
    const uint64_t* vrow = rowa + (t % kAddrSlots) * 2 * kTile;   // masked rows have address 0

    // partial S^T = K Q^T over this wave's 256 dims: every K fragment is
    // requested first, then two 16-entry blocks over two accumulators each
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (active) {
      bf16x8 kf[2][8];
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const uint8_t* krow = tile + (eb * 16 + col) * kRowBytes + kDHalf * 2 * dh + 16 * g;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) kf[eb][kb] = *(const bf16x8*)(krow + 64 * kb);
      }
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 8; kb += 2) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[eb][kb], qv[kb], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[eb][kb + 1], qv[kb + 1], s1, 0, 0, 0);
        }
        s[eb] = s0 + s1;
      }
    }
    // swap halves with the partner wave (same heads, other dims)
    *(f32x4*)xmine = s[0];
    *(f32x4*)(xmine + 4) = s[1];
    // widen tile t+1 while the matrix cores work, then reuse its registers
    // (past the list the tiles are all masked and widen to zeros)
    commit(t + 1, cur, cur_live);
    tile_addrs(t + kStages + 2);
    cur_live = fetch(t + 1 + kStages, cur);
    ATTEND_BARRIER(kWaitLgkm0);
    if (!active) return;
    {
      const f32x4 o0 = *(const f32x4*)xpart, o1 = *(const f32x4*)(xpart + 4);
      // the same sum in both waves (a + b == b + a), so both run the same softmax
      s[0] = dh == 0 ? s[0] + o0 : o0 + s[0];
      s[1] = dh == 0 ? s[1] + o1 : o1 + s[1];
    }
    // online softmax (log2 domain); lane holds entries eb*16 + 4g + i of head `col`
    float mx = -INFINITY;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = vrow[eb * 16 + 4 * g + i] ? s[eb][i] * a.scale_log2 : -INFINITY;
        s[eb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // the reference max moves only when the tile max overtakes it by the slack,
    // so the O rescale below is rare; probabilities stay below 2^slack
    const float m_new = mx > m_run + kRescaleSlack ? mx : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // arguments are at most the slack (8), or -inf for masked rows
    const float alpha = fast_exp2(m_run - m_use);
    bf16x8 pv;
    float psum = 0.f;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(s[eb][i] - m_use);
        psum += p;
        pv[eb * 4 + i] = (__bf16)p;          // round to nearest even
      }
    if (__any(alpha != 1.0f)) {
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 16; ++db) acc_o[db] *= alpha;
    }
    l_part += psum;
    m_run = m_new;
    // O^T += V^T P^T over this wave's dims; lane (g, col) supplies row
    // 4g + col/4 (+16) at dims 256 dh + 16 db + 4 (col % 4); the transposed
    // reads go out eight blocks at a time ahead of their MFMAs
    const uint8_t* vbase = tile + (4 * g + (col >> 2)) * kRowBytes + kDHalf * 2 * dh + 8 * (col & 3);
#pragma unroll
    for (int d0 = 0; d0 < 16; d0 += 8) {
      i16x4 lo[8], hi[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lo[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 32 * (d0 + u)));
        hi[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 16 * kRowBytes + 32 * (d0 + u)));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        bf16x8 vt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vt[j] = u16_as_bf16((uint16_t)lo[u][j]);
          vt[4 + j] = u16_as_bf16((uint16_t)hi[u][j]);
        }
        acc_o[d0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pv, acc_o[d0 + u], 0, 0, 0);
      }
    }
  };

  // Prologue: tiles 0 .. kStages in flight, tile 0 widened into buffer 0.
  // Register slot j carries tiles j, j + kStages, ... (the step loop is
  // unrolled by kStages so every slot is a fixed set of registers).
  i32x4 st0[kChunkSlots], st1[kChunkSlots], st2[kChunkSlots];
  int lv0, lv1, lv2;
  {
    i32x4 first[kChunkSlots];
    const int lf = fetch(0, first);
    lv1 = fetch(1, st1);
    lv2 = fetch(2, st2);
    lv0 = fetch(3, st0);
    commit(0, first, lf);
  }
  // Whole rounds of kStages steps, so every path issues the same loads and
  // the compiler's count of loads in flight stays exact; steps past the list
  // only keep the barriers and the ring in step.
  for (int t = 0; t < n_tiles; t += kStages) {
    step(t, st1, lv1, true);               // widens t+1 (slot 1), then fetches t+4 into it
    step(t + 1, st2, lv2, t + 1 < n_tiles);
    step(t + 2, st0, lv0, t + 2 < n_tiles);
  }

  // the trailing fetches (past the list) must land before the wave ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- epilogue: this wave's 256 dims of its 16 heads
  float l_run = l_part + __shfl_xor(l_part, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!head_ok) return;
  const int64_t unit = (int64_t)br * gridDim.y + hg;
  if (a.n_splits == 1) {
    const float z2 = a.sink[head] * kLog2e;
    const float top = fmaxf(m_run, z2);
    const float den = l_run * exp2f(m_run - top) + exp2f(z2 - top);
    const float inv = exp2f(m_run - top) / den;      // 0 when no row was seen
    uint16_t* orow = (uint16_t*)a.out + (((int64_t)b * a.n_q + r) * a.H + head) * kD + kDHalf * dh;
    const bool inv_rope = !(a.flags & CSA_ATTEND_NO_INV_ROPE);
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc_o[db][i] * inv;
      if (dh == 1 && db >= 12 && inv_rope) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int u = (kDHalf + 16 * db + 4 * g + i - kDN) >> 1;
          const float cs = rope_cs[u], sn = -rope_cs[32 + u];   // rotation by -t
          const float xe = o[i], xo = o[i + 1];
          o[i] = xe * cs - xo * sn;
          o[i + 1] = xe * sn + xo * cs;
        }
      }
      const uint32_t w0 = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
      *(i32x2*)(orow + 16 * db + 4 * g) = (i32x2){(int)w0, (int)w1};
    }
    if (a.out_lse && g == 0 && dh == 0)
      a.out_lse[((int64_t)b * a.n_q + r) * a.H + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  } else {
    // partial output normalised by its own denominator, in fp16 (|o| is
    // bounded by the largest |kv| element, far inside the fp16 range; the
    // fp16 step is 4x finer than the BF16 output's)
    const int64_t ps = (unit * a.n_splits + split) * 64 + hq * 16 + col;
    _Float16* po = a.part_o + ps * kD + kDHalf * dh;
    const float inv_l = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
      const f16x4 h = {(_Float16)(acc_o[db][0] * inv_l), (_Float16)(acc_o[db][1] * inv_l),
                       (_Float16)(acc_o[db][2] * inv_l), (_Float16)(acc_o[db][3] * inv_l)};
      *(f16x4*)(po + 16 * db + 4 * g) = h;
    }
    if (g == 0 && dh == 0) {
      a.part_ml[ps * 2] = m_run;
      a.part_ml[ps * 2 + 1] = l_run;
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
  const float z2 = a.sink[head] * kLog2e;
  float top = z2, mmax = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = a.part_ml[(base + s * 64) * 2];
    top = fmaxf(top, ms);
    mmax = fmaxf(mmax, ms);
  }
  float den = exp2f(z2 - top), lsum = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = a.part_ml[(base + s * 64) * 2];
    if (ms == -INFINITY) continue;
    const float ls = a.part_ml[(base + s * 64) * 2 + 1];
    const float wgt = exp2f(ms - top);
    den += ls * wgt;
    lsum += ls * exp2f(ms - mmax);
    // the partial is normalised: its numerator is o * l
    const float f = ls * wgt;
    typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
    const f16x8 v = *(const f16x8*)(a.part_o + (base + s * 64) * kD + d0);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += (float)v[i] * f;
  }
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
