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
// heads and one split of the query's KV list (the list's 32-entry tiles dealt
// round-robin to the splits).  Eight wavefronts, two per SIMD: wave q + 4 h
// owns dim quarter q and head half h.  Each lane loads 16-byte pieces of one
// entry row straight into registers two tiles ahead; the FP8 bytes are
// widened to BF16 in registers for the score product
//   S^T[32 entries x 32 heads] (partial over the quarter) = K Q^T
// (V_MFMA_F32_32X32X16_BF16, normalised and rotated query as the B operand),
// and the raw bytes go to the quarter's slice of an LDS tile.  The four
// quarters' partial scores meet in LDS, where each wave runs the online
// softmax (log2 domain, lazy rescale) of 8 heads and leaves P as BF16; then
//   O^T[quarter's 128 dims x 32 heads] += V^T P^T
// with V^T read back from the slice by transposing LDS reads.  Scores of tile
// t, softmax of tile t-1 and the output product of tile t-2 share one step
// and one barrier.
//
// A split that covers the whole list finalises in place (sink, normalisation,
// inverse RoPE, BF16 store); otherwise (running max, sum, normalised output) partials
// go to the workspace and combine_kernel merges them.
#include <hip/hip_ext.h>

#include "attend_common.hpp"

namespace csa {

// Workgroup of 8 wavefronts, two per SIMD.  Wave w = q + 4 h owns dim
// quarter q of the 512 dims (FP8 dims 128 q .. +127 for q < 3; FP8 dims
// 384 .. 447 plus the 64 BF16 RoPE dims for q = 3) and head half h (heads
// 32 h .. +31); the two waves of a quarter load the same row pieces.  Per
// 32-entry tile:
//  * scores: every lane loads 16-byte pieces of one entry row straight from
//    HBM into registers (two tiles ahead); they are widened FP8 -> BF16 in
//    registers and used as the A operand of
//      S^T[32 entries x 32 heads] (partial over the quarter's dims) = K Q^T
//    (V_MFMA_F32_32X32X16_BF16, 8 per tile) with the normalised, rotated,
//    pre-scaled query as the B operand; the same raw bytes go to the
//    quarter's slice of an LDS tile, where the output product reads them
//    back transposed;
//  * softmax: the four partial score blocks of a head half meet in LDS; wave
//    w runs the online softmax (log2 domain, lazy rescale) of heads 8 w ..
//    +7, eight lanes per head, and leaves P (BF16) and the rescale factors in
//    LDS;
//  * output: O^T[quarter's 128 dims x 32 heads] += V^T P^T (8 MFMAs per
//    tile), V^T read from the slice by ds_read_b64_tr_b8 (FP8, widened in
//    registers) or ds_read_b64_tr_b16 (RoPE dims).
// Two waves per SIMD let one wave's vector work run while the other waits
// on its matrix instructions or memory.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kVRow = 208;                      // bytes per entry in a quarter's slice (192 used)
constexpr int kVQuarter = kTile * kVRow;        // one quarter's slice of a tile
constexpr int kVBuf = 4 * kVQuarter;            // one tile
constexpr int kXsRow = 144;                     // one head's 32 partial scores (fp32) + pad
constexpr int kXsWave = 32 * kXsRow;            // a wave's partial scores (32 heads)
constexpr int kPRow = 80;                       // bytes per head in P: 32 BF16 + pad
constexpr int kPBytes = 64 * kPRow;
constexpr int kStageRow = kD * 2 + 16;          // output staging: one head's row
constexpr int kStages = 2;                      // tiles in flight in registers
constexpr int kXsBuf = kWaves * kXsWave;        // one tile's partial scores
constexpr int kOffXs = 2 * kVBuf;               // slices, partial scores and P are double-buffered
constexpr int kOffP = kOffXs + 2 * kXsBuf;
constexpr int kSmemBytes = kOffP + 2 * kPBytes;
static_assert(64 * kStageRow <= kOffP, "output staging reuses the tile and score regions");
constexpr int kIdxMax = kAttendIdxMax;          // selected indices staged per split

struct AttendShared {
  uint8_t* sm;       // [2 tiles][4 quarters][32 entries][kVRow] | xs[2] | P[2]
  float* alpha;      // [2][64] rescale factors per head
  float* ml;         // [64][2] final (max, sum)
  float* rope;       // cos, sin at the query position
  float* ssx;        // [4 quarters][64 heads] query sums of squares
  int* lidx;         // staged selected indices (CSA)
};

// Chunk c of a lane's row pieces: FP8 bytes wdim + 32 c + 16 g (the RoPE
// quarter: chunks 0, 1 at 384 + ..., chunks 2..5 the RoPE bytes 32 (c - 2) + 16 g).
template <bool kRope>
__device__ __forceinline__ i32x4 load_chunk(int c, const RowPtrs rp, int wdim, int g) {
  if (kRope && c >= 2) return *(gbl_i32x4*)(rp.pr + 32 * (c - 2) + 16 * g);
  return *(gbl_i32x4*)(rp.pn + wdim + 32 * c + 16 * g);
}

template <bool kRopeWave>
__device__ __forceinline__ void attend_wave(const AttendLaunch a, const AttendShared S, const int wave) {
  constexpr int NL = kRopeWave ? 6 : 4;     // 16-byte row pieces per lane per tile
  constexpr int NDT8 = kRopeWave ? 2 : 4;   // 32-dim output tiles read as FP8
  uint8_t* const sm = S.sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5, r32 = lane & 31;
  const int dq = wave & 3, hh = wave >> 2;  // dim quarter, head half
  const int split = blockIdx.x, hg = blockIdx.y;
  const int br = blockIdx.z;
  const int b = br / a.n_q, r = br % a.n_q;
  // (batch-invariant mode: the split count follows the query's list, so the
  // layout comes first; otherwise its loads overlap the first index reads)
  const bool inv = (a.flags & CSA_ATTEND_BATCH_INVARIANT) != 0;
  ListInfo L{};
  if (inv) L = list_info(a, b, r);
  const int n_sp = inv ? query_splits(a, L) : a.n_splits;
  if (split >= n_sp) return;                 // (invariant mode: a shorter list than the launch's longest)
  // Splits take the list's 32-entry tiles round-robin: local tile t of this
  // split is tile t n_sp + split of the list, so the workgroups of a query
  // stream one contiguous front of the cache (HBM serves that faster than
  // one private stream per workgroup).  List position of lane r32's entry:
#define ATTEND_POS(t) (((t) * n_sp + split) * kTile + r32)
  const int wdim = 128 * dq;                // first dim of the quarter (quarter 3: 384)
  const int hq = 32 * hh + r32;             // this lane's head (within the group) in the products

  // The 8 dims of k-step s held by lane half g (A and B operands alike).
  auto kdim = [&](int s) {
    return (kRopeWave && s >= 4) ? kDN + 16 * (s - 4) + 8 * g : wdim + 32 * (s >> 1) + 16 * g + 8 * (s & 1);
  };

  // Prologue.  Loads that do not depend on the list layout go first, so
  // their latencies overlap: the query, the sink logit and (CSA) the first
  // tiles' selected indices; then the layout (query position, visible
  // entries, window start) and the first tiles' row loads.
  const int head_q = hg * 64 + hq;
  const bool q_ok = head_q < a.H;
  const float sink_raw = a.sink[q_ok ? head_q : 0];   // used by the epilogue
  i32x4 qraw[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.n_q + r) * a.H + (q_ok ? head_q : 0)) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qraw[s] = *(gbl_i32x4*)(qrow + kdim(s));
  }
  const int* const idx_row = a.idx ? a.idx + ((int64_t)b * a.n_q + r) * a.top_k : nullptr;
  int sel0[kStages];                         // first tiles' selected indices (a harmless read for HCA)
#pragma unroll
  for (int u = 0; u < kStages; ++u) {
    const int pos = ATTEND_POS(u);
    sel0[u] = a.idx ? idx_row[pos < a.top_k ? pos : 0] : pos;
  }
  if (!inv) L = list_info(a, b, r);
  // Entries are gathered through staged rows for CSA and with a block table:
  // entry index -> row of the kv arrays, -1 for an invisible or unallocated one.
  const bool gather = a.idx != nullptr || a.bt != nullptr;
  auto stage_row = [&](int e) { return e >= 0 && e < L.n_vis ? entry_row(a, b, e) : -1; };
  if (gather) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) sel0[u] = stage_row(sel0[u]);
  }
  const int list_len = L.n_comp + L.n_w;
  const int list_tiles = (list_len + kTile - 1) / kTile;
  const int n_tiles = list_tiles > split ? (list_tiles - split + n_sp - 1) / n_sp : 0;

  // Row pieces of local tile t for this lane's entry (list position
  // ATTEND_POS(t)).  Every load is issued (a masked entry reads harmless bytes:
  // the query) so the count of loads in flight is the same on every path.
  RowSource rsrc;
  rsrc.dummy = (uint64_t)a.q;                // >= 1 KiB of readable bytes
  rsrc.kvb0 = (uint64_t)a.kv0 + (uint64_t)((int64_t)b * a.kv_seq_stride);
  rsrc.kvb1 = (uint64_t)a.kv1 + (uint64_t)((int64_t)b * a.kv_seq_stride);
  rsrc.wb0 = (uint64_t)a.win0 + (uint64_t)((int64_t)b * a.win_seq_stride);
  rsrc.wb1 = (uint64_t)a.win1 + (uint64_t)((int64_t)b * a.win_seq_stride);
  rsrc.wlo = L.win_lo;
  rsrc.wrap = L.win_wrap;
  rsrc.kvs = (uint32_t)a.kv_stride;
  rsrc.wns = (uint32_t)a.win_stride;
  rsrc.p1 = list_len;
  rsrc.n_comp = L.n_comp;
  rsrc.n_vis = L.n_vis;
  rsrc.n_w = L.n_w;
  rsrc.gather = gather;
  // index of tile t's entry for this lane (tiles from kStages on: staged in LDS)
#define ATTEND_SEL(t) S.lidx[(t) * kTile + r32 < kIdxMax ? (t) * kTile + r32 : kIdxMax - 1]
  i32x4 kst[kStages][NL];
  uint32_t kmask[kStages];
#pragma unroll
  for (int u = 0; u < kStages; ++u) {
    const RowPtrs rp = row_ptrs_tile<kRopeWave>(rsrc, ATTEND_POS(u) - r32, r32, sel0[u]);
    kmask[u] = rp.live;
#pragma unroll
    for (int c = 0; c < NL; ++c) kst[u][c] = load_chunk<kRopeWave>(c, rp, wdim, g);
  }
  if (tid < kDR / 2) {
    float cs, sn;
    rope_cos_sin((double)L.t, tid, kDR, a.log_theta, &cs, &sn);
    S.rope[tid] = cs;
    S.rope[32 + tid] = sn;
  }
  if (gather) {
    const int n_loc = n_tiles * kTile < kIdxMax ? n_tiles * kTile : kIdxMax;
    for (int i = tid; i < n_loc; i += kThreads) {
      const int pos = ((i / kTile) * n_sp + split) * kTile + (i % kTile);
      if (pos < L.n_comp) S.lidx[i] = stage_row(idx_row ? idx_row[pos] : pos);
    }
  }
  // tile -1's slices (buffer 1) and tile -2's P (buffer 0) are zero, its factors 1
  for (int i = tid; i < kVBuf / 16; i += kThreads) *(i32x4*)(sm + kVBuf + 16 * i) = (i32x4){0, 0, 0, 0};
  for (int i = tid; i < kPBytes / 16; i += kThreads) *(i32x4*)(sm + kOffP + 16 * i) = (i32x4){0, 0, 0, 0};
  if (tid < 64) S.alpha[tid] = 1.0f;
  ATTEND_BARRIER(kWaitLgkm0);

  // The query operand: head hq, dims kdim(s) .. +7; RMSNorm over all 512
  // dims (the four quarters add their sums of squares through LDS), the
  // softmax scale (log2 units), RoPE at the query position, BF16.
  bf16x8 qv[8];
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = q_ok ? (uint32_t)qraw[s][j] : 0u;
        const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
        ss += lo * lo + hi * hi;
      }
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) S.ssx[dq * 64 + hq] = ss;
    ATTEND_BARRIER(kWaitLgkm0);
    const float tot = ((S.ssx[hq] + S.ssx[64 + hq]) + S.ssx[128 + hq]) + S.ssx[192 + hq];
    // RMSNorm and the softmax scale (log2 units) in one factor; RoPE is linear
    const float rs = ((a.flags & CSA_ATTEND_NORM_Q) ? 1.0f / sqrtf(tot / (float)kD + 1e-6f) : 1.0f) * a.scale_log2;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = q_ok ? (uint32_t)qraw[s][j] : 0u;
        x[2 * j] = __uint_as_float(w << 16) * rs;
        x[2 * j + 1] = __uint_as_float(w & 0xffff0000u) * rs;
      }
      if (kRopeWave && s >= 4) {              // dims 448 .. 511 carry RoPE
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int u = (16 * (s - 4) + 8 * g + j) >> 1;
          const float cs = S.rope[u], sn = S.rope[32 + u];
          const float xe = x[j], xo = x[j + 1];
          x[j] = xe * cs - xo * sn;
          x[j + 1] = xe * sn + xo * cs;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[s][j] = (__bf16)x[j];   // nearest even
    }
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc_o[dt] = (f32x16){};
  // softmax heads of the wave: 8 wave .. +7, eight lanes per head, four
  // entries per lane
  const int hsl = 8 * dq + (lane >> 3);     // head within the half
  const int hs = 32 * hh + hsl;             // head within the group
  const int q8 = lane & 7;                  // its entries 4 q8 .. +3
  float m_run = -INFINITY;   // log2-domain reference max (lags the true max by < the slack)
  float l_part = 0.f;        // this lane's share of the running denominator
  const int G = lane >> 4, j16 = lane & 15;
  // V^T operands of the tile whose output product runs next (zero for tile -2)
  i32x2 vt8[NDT8][2];
  i16x4 vt16[2][2][2];
#pragma unroll
  for (int dt = 0; dt < NDT8; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vt8[dt][ks] = (i32x2){0, 0};
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) vt16[dt][ks][u] = (i16x4){0, 0, 0, 0};
  uint32_t live_prev = 0;    // live-entry mask of tile t-1 (tile -1: none)

  // Software pipeline, one barrier per step: step t forms the scores of
  // tile t, the online softmax of tile t-1 and the output product of tile
  // t-2, so the matrix cores have work on both sides of the softmax.
  // Slices, partial scores, P and the rescale factors are double-buffered
  // and row pieces sit in two register stages: tile t uses buffer and stage
  // t % 2.  Tiles -2 and -1 are empty (zero V, P = 0, factors 1); tiles past
  // the list are masked (scores -inf: P = 0, the running max and sum
  // unchanged).  n_tiles + 2 steps, in rounds of two.
  for (int t0 = 0; t0 <= n_tiles + 1; t0 += kStages) {
#pragma unroll
    for (int buf = 0; buf < kStages; ++buf) {
      const int t = t0 + buf;
      i32x4 (&kr)[NL] = kst[buf];
      uint32_t& km = kmask[buf];
      // masked entries of tile t read zeros (rare: a list's last tile, unused selections)
      const uint32_t live_t = km;
      if (__builtin_expect(live_t != 0xffffffffu, 0)) {
        const bool mine = (live_t >> r32) & 1;
#pragma unroll
        for (int c = 0; c < NL; ++c) kr[c] = mine ? kr[c] : (i32x4){0, 0, 0, 0};
      }
      // LDS reads of the step: P^T and the rescale factors of tile t-2, the
      // partial scores of tile t-1 (head hs, entries 4 q8 .. +3), the staged
      // index of tile t+2's entry
      const uint8_t* pb = sm + kOffP + buf * kPBytes;
      bf16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[ks] = *(const bf16x8*)(pb + hq * kPRow + 16 * (2 * ks + g));
      const float al = S.alpha[buf * 64 + hq];
      const uint8_t* xr = sm + kOffXs + (buf ^ 1) * kXsBuf + (4 * hh) * kXsWave + hsl * kXsRow + 16 * q8;
      f32x4 x[4];
#pragma unroll
      for (int src = 0; src < 4; ++src) x[src] = *(const f32x4*)(xr + src * kXsWave);
      const int sel = ATTEND_SEL(t + kStages);

      // tile t's raw bytes into the quarter's slice (both waves of the
      // quarter write the same bytes)
      uint8_t* vs = sm + buf * kVBuf + dq * kVQuarter + r32 * kVRow;
      if constexpr (!kRopeWave) {
#pragma unroll
        for (int c = 0; c < 4; ++c) *(i32x4*)(vs + 32 * c + 16 * g) = kr[c];
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) *(i32x4*)(vs + 32 * c + 16 * g) = kr[c];
#pragma unroll
        for (int c = 0; c < 4; ++c) *(i32x4*)(vs + 64 + 32 * c + 16 * g) = kr[2 + c];
      }
      // partial scores of tile t; each chunk's registers take tile t+2's chunk
      // once its k-steps are issued
      const RowPtrs rp = row_ptrs_tile<kRopeWave>(rsrc, ATTEND_POS(t + kStages) - r32, r32, sel);
      km = rp.live;
      f32x16 sc = {};
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        if (kRopeWave && c >= 2) {
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[c]), qv[c + 2], sc, 0, 0, 0);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bf16x8 kop = fp8x8_to_bf16((uint32_t)kr[c][2 * h], (uint32_t)kr[c][2 * h + 1]);
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qv[2 * c + h], sc, 0, 0, 0);
          }
        }
        kr[c] = load_chunk<kRopeWave>(c, rp, wdim, g);
      }

      // O rescaled before tile t-2 joins it, when a running max moved (in
      // place in the accumulation registers)
      if (__any(al != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float e = acc_o[dt][i], tmp;
            __asm__ __volatile__(
                "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                : "+a"(e), "=&v"(tmp)
                : "v"(al));
            acc_o[dt][i] = e;
          }
        __asm__ __volatile__("s_nop 4");      // vector writes before the next matrix read
      }

      // tile t's partial scores: lane holds head 32 hh + lane % 32, entries
      // 8 jb + 4 (lane / 32) + i, i.e. the 16-byte group 2 jb + lane / 32
      uint8_t* xw = sm + kOffXs + buf * kXsBuf + wave * kXsWave + r32 * kXsRow;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        *(f32x4*)(xw + 16 * (2 * jb + g)) = (f32x4){sc[4 * jb], sc[4 * jb + 1], sc[4 * jb + 2], sc[4 * jb + 3]};

      // O^T += V^T P^T for tile t-2
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 vop;
          if (dt < NDT8) {
            const int d8 = dt < NDT8 ? dt : 0;
            vop = fp8x8_to_bf16((uint32_t)vt8[d8][ks][0], (uint32_t)vt8[d8][ks][1]);
          } else {
            const int d2 = dt - NDT8 < 0 ? 0 : dt - NDT8;
            vop = bf16x8_of(vt16[d2][ks][0], vt16[d2][ks][1]);
          }
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf[ks], acc_o[dt], 0, 0, 0);
        }

      // online softmax of tile t-1 for head hs
      {
        const f32x4 s4 = ((x[0] + x[1]) + x[2]) + x[3];
        float v[4] = {s4[0], s4[1], s4[2], s4[3]};
        if (__builtin_expect(live_prev != 0xffffffffu, 0)) {   // masked entries: -inf
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (live_prev >> (4 * q8 + i)) & 1 ? v[i] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        mx = fmaxf(mx, dpp_f32<0xB1>(mx));     // lane ^ 1
        mx = fmaxf(mx, dpp_f32<0x4E>(mx));     // lane ^ 2
        mx = fmaxf(mx, dpp_f32<0x141>(mx));    // lane 7 - i of each 8: the other quad
        // the reference max moves only when the tile max overtakes it by the
        // slack, so O rescales are rare; probabilities stay below 2^slack
        const float m_new = mx > m_run + kRescaleSlack ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);   // argument <= 0, or -inf
        float psum = 0.f;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(v[i] - m_use);
          psum += pv[i];
        }
        // nearest even, two per conversion
        const bf16x4 pk = __builtin_bit_cast(bf16x4, (u32x2){pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])});
        l_part = l_part * alpha + psum;
        m_run = m_new;
        *(bf16x4*)(sm + kOffP + (buf ^ 1) * kPBytes + hs * kPRow + 8 * q8) = pk;
        if (q8 == 0) S.alpha[(buf ^ 1) * 64 + hs] = alpha;
      }
      live_prev = live_t;

      // V^T of tile t-1 from the quarter's slice, for the next step's output product
      const uint8_t* vw = sm + (buf ^ 1) * kVBuf + dq * kVQuarter;
#pragma unroll
      for (int dt = 0; dt < NDT8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // lanes 2i, 2i+1 of a 16-lane group supply entry 16 ks + 8 (G / 2) + i,
          // bytes 32 dt + 16 (G % 2) + 8 (j % 2); lane j receives byte j of the 8 entries
          const int row = 16 * ks + 8 * (G >> 1) + (j16 >> 1);
          vt8[dt][ks] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(vw + row * kVRow + 32 * dt + 16 * (G & 1) + 8 * (j16 & 1)));
        }
      if constexpr (kRopeWave) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              // lane j supplies entry 16 ks + 8 (G / 2) + 4 u + j / 4 at the 4 RoPE
              // dims 32 dt + 16 (G % 2) + 4 (j % 4); receives dim j's 4 entries
              const int row = 16 * ks + 8 * (G >> 1) + 4 * u + (j16 >> 2);
              vt16[dt][ks][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)(vw + row * kVRow + 64 + 2 * (32 * dt + 16 * (G & 1) + 4 * (j16 & 3))));
            }
      }
      ATTEND_BARRIER(kWaitLgkm0);
    }
  }
  // the trailing fetches (past the list) must land before the wave ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- epilogue: each head's (max, sum) from its softmax lanes
  {
    float l_run = l_part;
    l_run += dpp_f32<0xB1>(l_run);
    l_run += dpp_f32<0x4E>(l_run);
    l_run += dpp_f32<0x141>(l_run);
    if (q8 == 0) {
      S.ml[2 * hs] = m_run;
      S.ml[2 * hs + 1] = l_run;
    }
  }
  __syncthreads();
  const int64_t unit = (int64_t)br * gridDim.y + hg;
  const bool inv_rope = !(a.flags & CSA_ATTEND_NO_INV_ROPE);
  const bool single = n_sp == 1;
  // The normalised output (BF16 with the sink and inverse RoPE when the split
  // covers the whole list, else the fp16 partial) is staged in LDS as
  // [64 heads][512 dims] rows, so the global stores are contiguous 16-byte chunks.
  uint8_t* stage = sm;
  const float m_h = S.ml[2 * hq], l_h = S.ml[2 * hq + 1];
  float scale;
  if (single) {
    const float z2 = q_ok ? sink_raw * kLog2e : 0.f;
    const float top = fmaxf(m_h, z2);
    const float e_m = exp2f(m_h - top);
    scale = e_m / (l_h * e_m + exp2f(z2 - top));   // 0 when no row was seen
  } else {
    scale = l_h > 0.f ? 1.0f / l_h : 0.f;
  }
  // lane holds dims wdim + 32 dt + 8 jb + 4 (lane / 32) + i of head hq
  uint8_t* const srow = stage + hq * kStageRow;
  if (single) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int d0 = wdim + 32 * dt + 8 * jb + 4 * g;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc_o[dt][4 * jb + i] * scale;
        if (kRopeWave && dt >= NDT8 && inv_rope) {
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const int u = (d0 + i - kDN) >> 1;
            const float cs = S.rope[u], sn = -S.rope[32 + u];   // rotation by -t
            const float xe = o[i], xo = o[i + 1];
            o[i] = xe * cs - xo * sn;
            o[i + 1] = xe * sn + xo * cs;
          }
        }
        const bf16x4 w = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};   // nearest even
        *(bf16x4*)(srow + 2 * d0) = w;
      }
  } else {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const int d0 = wdim + 32 * dt + 8 * jb + 4 * g;
        f16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (_Float16)(acc_o[dt][4 * jb + i] * scale);
        *(f16x4*)(srow + 2 * d0) = w;
      }
  }
  if (dq == 0 && g == 0 && q_ok) {           // one lane per head
    if (single) {
      if (a.out_lse)
        a.out_lse[((int64_t)b * a.n_q + r) * a.H + head_q] =
            l_h > 0.f ? (m_h + log2f(l_h)) * 0.6931471805599453f : -INFINITY;
    } else {
      const int64_t ps = (unit * a.n_splits + split) * 64 + hq;
      a.part_ml[ps * 2] = m_h;
      a.part_ml[ps * 2 + 1] = l_h;
    }
  }
  ATTEND_BARRIER(kWaitLgkm0);
  // 64 rows x 64 chunks of 16 bytes: a row per wave and pass
  uint8_t* const obase = single ? (uint8_t*)a.out + (((int64_t)b * a.n_q + r) * a.H + hg * 64) * (kD * 2)
                                : (uint8_t*)(a.part_o + (unit * a.n_splits + split) * 64 * kD);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int hl = 8 * k + wave;
    if (hg * 64 + hl >= a.H) break;
    const i32x4 v = *(const i32x4*)(stage + hl * kStageRow + 16 * lane);
    *(i32x4*)(obase + (int64_t)hl * (kD * 2) + 16 * lane) = v;
  }
}

__global__ void __launch_bounds__(kThreads, 1) attend_fp8_kernel(AttendLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kSmemBytes];
  __shared__ float alpha_s[2 * 64];
  __shared__ float ml_s[2 * 64];
  __shared__ float rope_cs[64];
  __shared__ float ssx[4 * 64];
  __shared__ int lidx[kIdxMax];
  const AttendShared S{sm, alpha_s, ml_s, rope_cs, ssx, lidx};
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((wave & 3) == 3) attend_wave<true>(a, S, wave);
  else attend_wave<false>(a, S, wave);
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
  // splits this query's partials came from (the attention kernel finalised a
  // query with a single split itself)
  const int n_sp = (a.flags & CSA_ATTEND_BATCH_INVARIANT) ? query_splits(a, list_info(a, b, r)) : a.n_splits;
  if (n_sp == 1) return;
  if (threadIdx.x < 32) {
    float cs, sn;
    rope_cos_sin(-(double)t, threadIdx.x, kDR, a.log_theta, &cs, &sn);
    rope_cs[threadIdx.x] = cs;
    rope_cs[32 + threadIdx.x] = sn;
  }
  __syncthreads();
  if (head >= a.H) return;
  const int64_t base = (int64_t)unit * a.n_splits * 64 + hl;
  // Splits are merged sixteen at a time, every load of a group in flight
  // together, against a running maximum: M over the sink logit and the
  // splits' maxima (output and denominator), Mx over the splits only (LSE).
  typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
  constexpr int kGroup = 16;
  const float z2 = a.sink[head] * kLog2e;
  float M = z2, den = 1.0f;                 // den = exp2(z2 - M) + sum l_s exp2(m_s - M)
  float Mx = -INFINITY, lsum = 0.f;         // lsum = sum l_s exp2(m_s - Mx)
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_sp; s0 += kGroup) {
    float ms[kGroup], ls[kGroup];
    f16x8 v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int sj = s0 + j < n_sp ? s0 + j : s0;
      const int64_t rj = base + (int64_t)sj * 64;
      ms[j] = a.part_ml[rj * 2];
      ls[j] = a.part_ml[rj * 2 + 1];
      v[j] = *(const f16x8*)(a.part_o + rj * kD + d0);
    }
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (s0 + j >= n_sp) ms[j] = -INFINITY;
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
  if (attend_mh_applies(a)) {
    if (launch_attend_mh(a, s) != hipSuccess) return hipGetLastError();
  } else {
    dim3 grid(a.n_splits, n_hg, a.B * a.n_q);
    hipExtLaunchKernelGGL(attend_fp8_kernel, grid, dim3(kThreads), 0, s, a.ev_start, a.ev_stop, 0, a);
  }
  if (a.n_splits > 1) combine_kernel<<<dim3(a.B * a.n_q * n_hg, 16), 256, 0, s>>>(a, n_hg);
  return hipGetLastError();
}

}  // namespace csa
