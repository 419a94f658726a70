// Shared-KV attention with a per-head sink for calls with several queries
// (prefill chunks) of a model with 128 query heads: one query and 128 heads
// per workgroup.
//
// What is computed is what attend.hip computes ("DeepSeek-V4 深读",
// ricardokevins.github.io, CSA/HCA section and its stability paragraph;
// "拆解 DeepSeekv4", daixd5520.github.io, section 细节): every head of a query
// reads one shared 512-d vector per entry as key and value, the query's last
// 64 dims carry RoPE at its position and the output's last 64 dims are
// rotated back, and exp(sink_h) joins each head's softmax denominator.
//
// Design.  Because all heads read the same entry vector, one LDS copy of a
// 32-entry tile serves all 128 heads of the workgroup (the 64-head decode
// kernel serves half of them per copy).  Four wavefronts, one per SIMD; wave
// w owns heads 32 w .. +31 across all 512 dims, so
//   S^T[32 entries x 32 heads] = K Q^T
// (the 448 FP8 dims: 14 V_MFMA_SCALE_F32_32X32X64_F8F6F4 with the entry bytes
// as they are against a two-component E4M3 split of the query; the 64 RoPE
// dims: 4 V_MFMA_F32_32X32X16_BF16)
// is complete inside the wave: the online softmax works on registers (lane l
// holds head l % 32 and 16 of the tile's entries, lane l ^ 32 the other 16),
// two 32-lane swaps per 16 entries turn P^T from the result layout into the
// B-operand layout of
//   O^T[512 dims x 32 heads] += V^T P^T          (32 MFMAs, 256 accumulators)
// and a lane's accumulators all belong to its own head, so a rescale is one
// factor per lane.  K comes from the LDS tile as 16-byte reads used as they
// are (the RoPE dims as BF16), V^T by transposing LDS reads widened FP8 ->
// BF16 in registers.
//
// The tile is stored as [36 sixteen-byte chunks][32 entries]: each 1 KiB
// direct-to-LDS load of a wave brings chunks 2i and 2i+1 of all 32 entries,
// so every lane loads from its own entry's row.  Three tiles live in LDS:
// tile t is computed while t+1 and t+2 are in flight, one barrier per tile.
// A split that covers the whole list finalises in place (sink, normalisation,
// inverse RoPE, BF16); otherwise the normalised fp16 output and (max, sum) go
// to the workspace in the decode kernel's layout and combine_kernel merges.
#include <hip/hip_ext.h>

#include "attend_common.hpp"

namespace csa {
namespace {

constexpr int kMhWaves = 4;
constexpr int kMhThreads = kMhWaves * 64;
constexpr int kMhHeads = 128;                          // heads per workgroup
constexpr int kMhTileBytes = kChunksPerTile * 16;      // 18432
constexpr int kMhLoads = kMhTileBytes / 1024;          // 18 one-KiB wave loads per tile
constexpr int kMhBufs = 3;
constexpr int kMhStageRow = kD * 2 + 16;               // output staging: one head's row
constexpr int kMhSmem = kMhBufs * kMhTileBytes > 64 * kMhStageRow ? kMhBufs * kMhTileBytes : 64 * kMhStageRow;
constexpr int kMhIdxMax = kAttendIdxMax;
static_assert(kMhLoads == 18, "wave w issues loads w, w + 4, ... (five for waves 0 and 1, four for 2 and 3)");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at LDS byte lds_off + 16 l.  Written as inline assembly so that the
// compiler, which cannot tell which LDS bytes such a load writes, does not
// drain every load in flight before each LDS read; the kernel waits for
// these loads itself (they count in vmcnt, in order with other loads, so the
// compiler's own waits for its loads can only wait longer than needed).
__device__ __forceinline__ void lds_dma16(uint64_t gaddr, uint32_t lds_off) {
  __asm__ __volatile__("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :
                       : "v"(gaddr), "s"(lds_off)
                       : "memory", "m0");
}

// Scaled 32x32x64 product of FP8 entry bytes (scale 2^0) and an FP8 query
// component whose E8M0 scale is byte SEL of scw.
template <int SEL>
__device__ __forceinline__ f32x16 mfma_q8(const i32x8& k, const i32x8& q, const f32x16& c, uint32_t scw) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k, q, c, 0, 0, 0, 127, SEL, (int)scw);
}
__device__ __forceinline__ f32x16 mfma_q8_byte(int sel, const i32x8& k, const i32x8& q, const f32x16& c,
                                               uint32_t scw) {
  switch (sel) {
    case 0: return mfma_q8<0>(k, q, c, scw);
    case 1: return mfma_q8<1>(k, q, c, scw);
    case 2: return mfma_q8<2>(k, q, c, scw);
    default: return mfma_q8<3>(k, q, c, scw);
  }
}

}  // namespace

__global__ void __launch_bounds__(kMhThreads, 1) attend_mh_kernel(AttendLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kMhSmem];
  __shared__ int lidx[kMhIdxMax];
  __shared__ float rope_cs[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int G = lane >> 4, j16 = lane & 15;
  const int split = blockIdx.x, hg = blockIdx.y;
  const int br = blockIdx.z;
  const int b = br / a.n_q, r = br % a.n_q;
  const int n_sp = a.n_splits;
  const int head = hg * kMhHeads + 32 * wave + r32;    // this lane's head (column of S^T and O^T)

  // ---- prologue: the query, the sink, the list layout and (gathering) the
  // split's staged entry rows
  const float sink_raw = a.sink[head];
  // BF16 query: the FP8-stored dims in the layout of the scaled 32x32x64
  // operand (K-step s: dims 64 s + 16 g .. +15 and 64 s + 32 + 16 g .. +15),
  // the RoPE dims in the layout of the BF16 32x32x16 operand (dims
  // kDN + 16 u + 8 g .. +7)
  i32x4 qfr[kDN / 64][4];
  i32x4 qrr[kDR / 16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.n_q + r) * a.H + head) * kD;
#pragma unroll
    for (int s = 0; s < kDN / 64; ++s)
#pragma unroll
      for (int p = 0; p < 4; ++p) qfr[s][p] = *(gbl_i32x4*)(qrow + 64 * s + 32 * (p >> 1) + 16 * g + 8 * (p & 1));
#pragma unroll
    for (int u = 0; u < kDR / 16; ++u) qrr[u] = *(gbl_i32x4*)(qrow + kDN + 16 * u + 8 * g);
  }
  const ListInfo L = list_info(a, b, r);
  const bool gather = a.idx != nullptr || a.bt != nullptr;
  const int list_len = L.n_comp + L.n_w;
  const int list_tiles = (list_len + kTile - 1) / kTile;
  const int n_tiles = list_tiles > split ? (list_tiles - split + n_sp - 1) / n_sp : 0;
  // Splits take the list's tiles round-robin: local tile t is list tile
  // t n_sp + split.  List position of lane r32's entry in local tile t:
#define MH_POS(t) (((t) * n_sp + split) * kTile + r32)
  if (gather) {
    const int* const idx_row = a.idx ? a.idx + ((int64_t)b * a.n_q + r) * a.top_k : nullptr;
    const int n_loc = n_tiles * kTile < kMhIdxMax ? n_tiles * kTile : kMhIdxMax;
    for (int i = tid; i < n_loc; i += kMhThreads) {
      const int pos = ((i / kTile) * n_sp + split) * kTile + (i % kTile);
      if (pos < L.n_comp) {
        const int e = idx_row ? idx_row[pos] : pos;
        lidx[i] = e >= 0 && e < L.n_vis ? entry_row(a, b, e) : -1;
      }
    }
  }
  if (tid < kDR / 2) {
    float cs, sn;
    rope_cos_sin((double)L.t, tid, kDR, a.log_theta, &cs, &sn);
    rope_cs[tid] = cs;
    rope_cs[32 + tid] = sn;
  }
  RowSource rsrc;
  rsrc.dummy = (uint64_t)a.q;                          // >= 1 KiB of readable bytes
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
  __syncthreads();

  // Tile t into LDS buffer bi: wave load i brings chunks 2i, 2i+1 of the 32
  // entries (lane l: chunk 2i + l / 32 of entry l % 32, i.e. the 16 bytes at
  // 1024 i + 16 l).  A masked entry reads harmless bytes (the query) and is
  // zeroed in LDS before use.  Returns the tile's live-entry mask.
  auto issue_tile = [&](int t, int bi) -> uint32_t {
    const int li = t * kTile + r32;
    const int sel = gather ? lidx[li < kMhIdxMax ? li : kMhIdxMax - 1] : 0;
    const RowPtrs rp = row_ptrs_tile<true>(rsrc, MH_POS(t) - r32, r32, sel);
    const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)sm + (uint32_t)(bi * kMhTileBytes);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int i = wave + 4 * k;
      if (i < kMhLoads) {
        const int c = 2 * i + g;
        const uint64_t src = c < kDN / 16 ? rp.pn + 16 * c : rp.pr + 16 * (c - kDN / 16);
        lds_dma16(src, (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + 1024u * (uint32_t)i)));
      }
    }
    return rp.live;
  };
  uint32_t live0 = issue_tile(0, 0);
  uint32_t live1 = issue_tile(1, 1);

  // The query operand: RMSNorm over the 512 dims (lane l ^ 32 holds the
  // other half), the softmax scale in log2 units, then
  //  * the FP8-stored dims as two E4M3 components per 32-dim block, each with
  //    its own E8M0 scale that puts the block's largest magnitude in
  //    [128, 256): q = 2^e1 c1 + 2^e2 c2 + r with |r| below 2^-8 of the block
  //    maximum (the precision of BF16), so the score product reads the FP8
  //    entry bytes as they are (scaled 32x32x64 products, no widening);
  //  * RoPE on dims 448 .. 511, BF16 (nearest even).
  // Lane half g supplies the scales of blocks 2 s + g (the operand's rule);
  // component c of K-step s has its scale in byte (7 c + s) % 4 of word
  // (7 c + s) / 4.
  i32x8 qf[2][kDN / 64];
  uint32_t qsc[4] = {0u, 0u, 0u, 0u};
  bf16x8 qv[kDR / 16];
  {
    float ss = 0.f;
    auto acc_ss = [&](const i32x4& w4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)w4[j];
        const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
        ss += lo * lo + hi * hi;
      }
    };
#pragma unroll
    for (int s = 0; s < kDN / 64; ++s)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc_ss(qfr[s][p]);
#pragma unroll
    for (int u = 0; u < kDR / 16; ++u) acc_ss(qrr[u]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
    const float tot = g == 0 ? ss + __uint_as_float(sw[1]) : __uint_as_float(sw[0]) + ss;
    const float rs = ((a.flags & CSA_ATTEND_NORM_Q) ? 1.0f / sqrtf(tot / (float)kD + 1e-6f) : 1.0f) * a.scale_log2;
    // E8M0 exponent that puts a block maximum m in [128, 256) (-127: an all-zero block)
    auto block_exp = [](float m) {
      int e = -127;
      if (m > 0.0f) {
        int ex;
        frexpf(m, &ex);
        e = ex - 8;
      }
      return e < -127 ? -127 : (e > 127 ? 127 : e);
    };
#pragma unroll
    for (int s = 0; s < kDN / 64; ++s) {
      uint32_t wc[2][8];                       // packed codes of both components
      int e_lane[2] = {0, 0};                  // this lane's scales (block 2 s + g)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {         // block 2 s + hb: dims 64 s + 32 hb .. +31
        float x[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = (uint32_t)qfr[s][2 * hb + (j >> 2)][j & 3];
          x[2 * j] = __uint_as_float(w << 16) * rs;
          x[2 * j + 1] = __uint_as_float(w & 0xffff0000u) * rs;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(x[j]));
          const auto mw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(m, __uint_as_float(g == 0 ? mw[1] : mw[0]));   // the block's maximum (both lane halves)
          const int e = block_exp(m);
          const float down = ldexpf(1.0f, -e), up = ldexpf(1.0f, e);
#pragma unroll
          for (int j = 0; j < 16; j += 4) {
            // E4M3 codes by the hardware converter (nearest even; the scaled
            // values lie below 256, inside the format's range)
            int wv = __builtin_amdgcn_cvt_pk_fp8_f32(x[j] * down, x[j + 1] * down, 0, false);
            wv = __builtin_amdgcn_cvt_pk_fp8_f32(x[j + 2] * down, x[j + 3] * down, wv, true);
            // what the next component carries
            x[j] -= __builtin_amdgcn_cvt_f32_fp8(wv, 0) * up;
            x[j + 1] -= __builtin_amdgcn_cvt_f32_fp8(wv, 1) * up;
            x[j + 2] -= __builtin_amdgcn_cvt_f32_fp8(wv, 2) * up;
            x[j + 3] -= __builtin_amdgcn_cvt_f32_fp8(wv, 3) * up;
            wc[c][4 * hb + j / 4] = (uint32_t)wv;
          }
          if (hb == 0) e_lane[c] = e;
          else if (g == 1) e_lane[c] = e;
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        qf[c][s] = (i32x8){(int)wc[c][0], (int)wc[c][1], (int)wc[c][2], (int)wc[c][3],
                           (int)wc[c][4], (int)wc[c][5], (int)wc[c][6], (int)wc[c][7]};
        const int idx = 7 * c + s;
        qsc[idx / 4] |= (uint32_t)(e_lane[c] + 127) << (8 * (idx % 4));
      }
    }
#pragma unroll
    for (int u = 0; u < kDR / 16; ++u) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)qrr[u][j];
        x[2 * j] = __uint_as_float(w << 16) * rs;
        x[2 * j + 1] = __uint_as_float(w & 0xffff0000u) * rs;
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int v = (16 * u + 8 * g + j) >> 1;
        const float cs = rope_cs[v], sn = rope_cs[32 + v];
        const float xe = x[j], xo = x[j + 1];
        x[j] = xe * cs - xo * sn;
        x[j + 1] = xe * sn + xo * cs;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[u][j] = (__bf16)x[j];
    }
  }

  // O^T accumulators: blocks 0..14 in AGPRs (the compiler's choice for the
  // matrix instructions), block 15 (dims 480 .. 511) in VGPRs through inline
  // assembly, so that the score accumulator also finds AGPRs (all 256 would
  // otherwise hold O and the compiler would shuttle blocks in and out)
  f32x16 acc_o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc_o[dt] = (f32x16){};
  float m_run = -INFINITY;   // log2-domain reference max of the head (lags the true max by < the slack)
  float l_part = 0.f;        // this lane's share of the running denominator

  for (int t = 0; t < n_tiles; ++t) {
    // tile t has landed (this wave's loads of tile t+1 may still be in
    // flight); after the barrier every wave's loads of tile t are in LDS and
    // every wave is done with tile t-1, whose buffer takes tile t+2
    if (wave < 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
    ATTEND_BARRIER(kWaitLgkm0);
    const int bi = t % kMhBufs;
    const uint32_t live2 = issue_tile(t + 2, (t + 2) % kMhBufs);
    const uint32_t live_t = live0;
    live0 = live1;
    live1 = live2;
    uint8_t* const tb = sm + bi * kMhTileBytes;
    if (live_t != 0xffffffffu) {
      // masked entries (a list's last tile, unused selections) read zeros, or
      // the output product would multiply P = 0 by whatever bytes they hold
      for (int i = tid; i < kChunksPerTile; i += kMhThreads)
        if (!((live_t >> (i & 31)) & 1u)) *(i32x4*)(tb + 16 * i) = (i32x4){0, 0, 0, 0};
      ATTEND_BARRIER(kWaitLgkm0);
    }

    // scores: lane holds head r32, entries 8 j + 4 g + i (i < 4) in sc[4 j + i]
    f32x16 sc = {};
    // FP8 dims: the entry bytes as the A operand of the scaled 32x32x64
    // product (scale 2^0) against both query components
#pragma unroll
    for (int s = 0; s < kDN / 64; ++s) {
      const i32x4 lo = *(const i32x4*)(tb + (4 * s + g) * 512 + 16 * r32);
      const i32x4 hi = *(const i32x4*)(tb + (4 * s + 2 + g) * 512 + 16 * r32);
      const i32x8 kop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sc = mfma_q8_byte(s % 4, kop, qf[0][s], sc, qsc[s / 4]);
      sc = mfma_q8_byte((7 + s) % 4, kop, qf[1][s], sc, qsc[(7 + s) / 4]);
    }
    // RoPE dims: BF16 products
#pragma unroll
    for (int u = 0; u < kDR / 16; ++u) {
      const bf16x8 kop = *(const bf16x8*)(tb + (kDN / 16 + 2 * u + g) * 512 + 16 * r32);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qv[u], sc, 0, 0, 0);
    }

    // online softmax of the head over the tile
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = sc[e];
    if (__builtin_expect(live_t != 0xffffffffu, 0)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[4 * j + i] = (live_t >> (8 * j + 4 * g + i)) & 1u ? v[4 * j + i] : -INFINITY;
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[e]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(mx, __uint_as_float(g == 0 ? sw[1] : sw[0]));
    }
    // the reference max moves only when the tile max overtakes it by the
    // slack, so rescales are rare; probabilities stay below 2^slack
    const float m_new = mx > m_run + kRescaleSlack ? mx : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);       // argument <= 0, or -inf
    float psum = 0.f;
    uint32_t pw[4][2];                                  // P of entries 8 j + 4 g + i as BF16 pairs
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float p0 = fast_exp2(v[4 * j + 2 * h] - m_use);
        const float p1 = fast_exp2(v[4 * j + 2 * h + 1] - m_use);
        psum += p0 + p1;
        pw[j][h] = pack_bf16x2(p0, p1);                 // nearest even
      }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
      // in place in the accumulation registers (AGPRs: the vector unit
      // reaches them only through copies)
      acc_o[15] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 15; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e = acc_o[dt][i], tmp;
          __asm__ __volatile__(
              "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
              : "+a"(e), "=&v"(tmp)
              : "v"(alpha));
          acc_o[dt][i] = e;
        }
      __asm__ __volatile__("s_nop 4");      // vector writes before the next matrix read
    }
    // P^T as the B operand of k-step ks (entries 16 ks .. +15; lane half g
    // holds entries 16 ks + 8 g .. +7): lanes 0-31 keep their entries
    // 16 ks + 0..3 and take 16 ks + 4..7 from lane + 32; lanes 32-63 take
    // 16 ks + 8..11 from lane - 32 and keep 16 ks + 12..15.
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pw[2 * ks][0], pw[2 * ks + 1][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pw[2 * ks][1], pw[2 * ks + 1][1], false, false);
      const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // O^T += V^T P^T: dims 32 dt + lane % 32 of entries 16 ks + 8 g .. +7
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vop;
        if (dt < kDN / 32) {
          // lanes 2i, 2i+1 of a 16-lane group supply entry 16 ks + 8 (G / 2) + i,
          // bytes 32 dt + 16 (G % 2) + 8 (j % 2); lane j receives byte j of the 8 entries
          const int row = 16 * ks + 8 * (G >> 1) + (j16 >> 1);
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(tb + (2 * dt + (G & 1)) * 512 + 16 * row + 8 * (j16 & 1)));
          vop = fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
        } else {
          i16x4 h[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // lane j supplies entry 16 ks + 8 (G / 2) + 4 u + j / 4 at the 4 RoPE
            // dims 32 d2 + 16 (G % 2) + 4 (j % 4); receives dim j's 4 entries
            const int row = 16 * ks + 8 * (G >> 1) + 4 * u + (j16 >> 2);
            const int byte = 64 * (dt - kDN / 32) + 32 * (G & 1) + 8 * (j16 & 3);   // in the RoPE bytes
            h[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(tb + (kDN / 16 + (byte >> 4)) * 512 + 16 * row + (byte & 15)));
          }
          vop = bf16x8_of(h[0], h[1]);
        }
        if (dt < 15) {
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[ks], acc_o[dt], 0, 0, 0);
        } else {
          // wait states: vector writes of the operands before the matrix
          // read; the matrix result before any later vector access
          __asm__ __volatile__(
              "s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
              : "+v"(acc_o[15])
              : "v"(vop), "v"(pb[ks]));
        }
      }
  }
#undef MH_POS
  // the trailing loads (tiles past the list) land before LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  ATTEND_BARRIER(kWaitLgkm0);

  // ---- epilogue
  float l_run;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
    l_run = l_part + __uint_as_float(g == 0 ? sw[1] : sw[0]);
  }
  const bool single = n_sp == 1;
  const bool inv_rope = !(a.flags & CSA_ATTEND_NO_INV_ROPE);
  float scale;
  if (single) {
    const float z2 = sink_raw * kLog2e;
    const float top = fmaxf(m_run, z2);
    const float e_m = exp2f(m_run - top);
    scale = e_m / (l_run * e_m + exp2f(z2 - top));   // 0 when no entry was seen
    if (a.out_lse && g == 0)
      a.out_lse[((int64_t)b * a.n_q + r) * a.H + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  } else {
    scale = l_run > 0.f ? 1.0f / l_run : 0.f;
  }
  const int n_hg64 = a.H / 64;
  // two passes of 64 heads (waves 2p, 2p + 1) staged in LDS as [64][512]
  // rows, then stored as contiguous 16-byte chunks
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int unit = br * n_hg64 + hg * 2 + pass;      // the decode kernel's 64-head unit
    if ((wave >> 1) == pass) {
      const int hl = 32 * (wave & 1) + r32;             // head within the 64
      uint8_t* const srow = sm + hl * kMhStageRow;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const int d0 = 32 * dt + 8 * jb + 4 * g;
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = acc_o[dt][4 * jb + i] * scale;
          if (single) {
            if (dt >= kDN / 32 && inv_rope) {
#pragma unroll
              for (int i = 0; i < 4; i += 2) {
                const int u = (d0 + i - kDN) >> 1;
                const float cs = rope_cs[u], sn = -rope_cs[32 + u];   // rotation by -t
                const float xe = o[i], xo = o[i + 1];
                o[i] = xe * cs - xo * sn;
                o[i + 1] = xe * sn + xo * cs;
              }
            }
            const bf16x4 w = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};   // nearest even
            *(bf16x4*)(srow + 2 * d0) = w;
          } else {
            typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
            const f16x4 w = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
            *(f16x4*)(srow + 2 * d0) = w;
          }
        }
      if (!single && g == 0) {
        const int64_t ps = ((int64_t)unit * a.n_splits + split) * 64 + hl;
        a.part_ml[ps * 2] = m_run;
        a.part_ml[ps * 2 + 1] = l_run;
      }
    }
    ATTEND_BARRIER(kWaitLgkm0);
    uint8_t* const obase = single ? (uint8_t*)a.out + (((int64_t)b * a.n_q + r) * a.H + hg * kMhHeads + 64 * pass) * (kD * 2)
                                  : (uint8_t*)(a.part_o + ((int64_t)unit * a.n_splits + split) * 64 * kD);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int idx = 256 * k + tid;                     // 64 rows x 64 chunks of 16 bytes
      const int row = idx >> 6, ch = idx & 63;
      const i32x4 v = *(const i32x4*)(sm + row * kMhStageRow + 16 * ch);
      *(i32x4*)(obase + (int64_t)row * (kD * 2) + 16 * ch) = v;
    }
    ATTEND_BARRIER(kWaitLgkm0);
  }
}

// Calls with several queries and a multiple of 128 heads (not the
// batch-invariant mode, whose kernel must not depend on the call's shape).
bool attend_mh_applies(const AttendLaunch& a) {
  return a.fmt == CSA_FMT_FP8_BF16 && a.n_q > 1 && a.H % kMhHeads == 0 &&
         !(a.flags & CSA_ATTEND_BATCH_INVARIANT);
}

hipError_t launch_attend_mh(const AttendLaunch& a, hipStream_t s) {
  dim3 grid(a.n_splits, a.H / kMhHeads, a.B * a.n_q);
  hipExtLaunchKernelGGL(attend_mh_kernel, grid, dim3(kMhThreads), 0, s, a.ev_start, a.ev_stop, 0, a);
  return hipGetLastError();
}

}  // namespace csa
