// Lightning indexer (MXFP4 on the matrix cores) and radix top-k selection.
//
// Score of compressed entry i for a query (indexer of "DeepSeek-V4 深读",
// ricardokevins.github.io, section "CSA：4× 压缩之后再 top-k"; "拆解 DeepSeekv4",
// daixd5520.github.io, section CSA step 2):
//     I_i = sum_h w_h * ReLU(q_h . k_i)
// with query heads and keys in MXFP4 (the FP4 indexer QK path of the FP4 QAT
// section of "DeepSeek-V4 深读").  Only entries of blocks that end before the
// query's own block are visible.
//
// Indexer kernel: the heads form the M side of V_MFMA_SCALE_F32_16X16X128_F8F6F4
// (one instruction covers the whole 128-wide dot product of 16 heads x 16
// keys, with the E8M0 block scales applied by the matrix core), the keys the N
// side.  A 16-key tile is one contiguous 1 KiB read (64 B of codes per key);
// each lane loads 16 bytes straight into its operand registers, so keys
// stream from HBM exactly once.  ReLU and the head weights are applied to the
// 4 accumulator rows a lane holds, and cross-lane swaps over four tiles at a
// time finish the head sum.  The kernel also builds the histogram of the top
// 12 bits of every score's order key for the first radix-select pass.
//
// Query blocks (two or more queries per call, H_I a multiple of 32; a prefill
// chunk) use index_mxfp4_mq_kernel instead: the 32x32x64 form of the scaled
// MFMA and a split of w ReLU(s) into (w/2)|s| + (w/2)s whose second term comes
// from an FP8 split of the weighted query sum (see that kernel).
//
// Top-k over the 32-bit order keys of the scores.  The scoring kernel builds a
// histogram of the top 12 key bits, then two kernels follow, one workgroup
// per 4096-score chunk and query:
//   collect finds (in every workgroup) the bucket holding the k-th key, counts
//           the chunk's keys above that bucket and copies the keys inside it
//           to the chunk's region of the candidate list;
//   select  (every workgroup again) radix-selects the k-th key T among the
//           query's candidates (10 + 10 more bits), derives from the
//           per-chunk counts where its chunk's selection starts in the
//           output, and emits the chunk's selected indices in index order,
//           so the output is ascending; among keys equal to T the lowest
//           indices are taken.
// With 64 or more queries per call the radix search runs once per query
// instead (topk_bucket_kernel, topk_threshold_kernel; see there).
// Histograms use integer atomics only and candidate lists are compacted per
// chunk by block scans, so the result does not depend on any ordering and is
// deterministic.  The histogram is left zeroed by every call.  Kernel
// boundaries order the stages: on a multi-XCD part a device-wide fence or a
// contended device-scope atomic inside a kernel costs more than a launch.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.hpp"

#include "kernels.hpp"

namespace csa {

constexpr int kTilesPerWave = 32;                    // 16 keys per tile: 512 keys per wave
constexpr int kRing = 8;                             // tiles of keys in flight per wave
constexpr int kWaveKeys = kTilesPerWave * 16;        // 512
constexpr int kKeysPerWG = 4 * kWaveKeys;            // 2048
constexpr int kChunk = 4096;                         // scores per workgroup in collect / write
constexpr int kBins1 = 4096;                         // 12-bit first digit
constexpr int kShift1 = 20;
constexpr int kMaxChunks = 1024;                     // per query (n_cap <= 4M)
// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format, the value the ROCm libraries use for untyped buffer loads).
constexpr int kBufferWord3 = 0x00020000;

// max(x, 0) as one integer max on the bit pattern: negative floats (sign bit
// set) are negative integers and map to +0; non-negative floats are unchanged.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Score row of query r of sequence b in this query block: the workspace holds
// the block's rows [B][n_qb]; a caller's score array holds all [B][n_q] rows.
// Scores are fp32, or BF16 codes (2 bytes) with CSA_INDEX_BF16_SCORES.
__device__ __forceinline__ bool bf16_scores(const IndexLaunch& a) { return (a.flags & CSA_INDEX_BF16_SCORES) != 0; }
__device__ __forceinline__ float* score_row(const IndexLaunch& a, int b, int r) {
  const int64_t row = (int64_t)b * a.score_seq_rows + a.score_row0 + r;
  return (float*)((char*)a.scores + row * a.n_cap * (bf16_scores(a) ? 2 : 4));
}
// score i of a row (BF16 codes widen exactly)
__device__ __forceinline__ float load_score(const IndexLaunch& a, const float* row, int64_t i) {
  if (bf16_scores(a)) return bf16_to_f32(((const uint16_t*)row)[i]);
  return row[i];
}
__device__ __forceinline__ void store_score(const IndexLaunch& a, float* row, int64_t i, float v) {
  if (bf16_scores(a)) ((uint16_t*)row)[i] = f32_to_bf16(v);
  else row[i] = v;
}
// the value a score is stored as (BF16 rounds to nearest even)
__device__ __forceinline__ float stored_score(const IndexLaunch& a, float v) {
  return bf16_scores(a) ? bf16_to_f32(f32_to_bf16(v)) : v;
}
// scores i .. i+3 of a row (i + 3 < n_cap), one vector load when aligned
__device__ __forceinline__ void load_score4(const IndexLaunch& a, const float* row, int64_t i, float* out) {
  if (bf16_scores(a)) {
    const uint16_t* r16 = (const uint16_t*)row;
    if ((((uintptr_t)(r16 + i)) & 7) == 0) {
      const u32x2 x = *(const u32x2*)(r16 + i);
      out[0] = __uint_as_float(x[0] << 16); out[1] = __uint_as_float(x[0] & 0xffff0000u);
      out[2] = __uint_as_float(x[1] << 16); out[3] = __uint_as_float(x[1] & 0xffff0000u);
    } else {
      for (int u = 0; u < 4; ++u) out[u] = bf16_to_f32(r16[i + u]);
    }
    return;
  }
  if ((((uintptr_t)(row + i)) & 15) == 0) {
    const f32x4 x = *(const f32x4*)(row + i);
    out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
  } else {
    for (int u = 0; u < 4; ++u) out[u] = row[i + u];
  }
}

__device__ __forceinline__ int query_n_vis(const IndexLaunch& a, int b, int r) {
  const int64_t t = a.q_pos[(int64_t)b * a.n_q + a.q_first + r];
  int64_t v = t >= 0 ? t / a.m : 0;
  const int64_t ne = a.n_entries ? (int64_t)a.n_entries[b] : (int64_t)a.n_cap;
  v = v < ne ? v : ne;
  v = v < a.n_cap ? v : a.n_cap;
  return (int)(v < 0 ? 0 : v);
}

// Flush a block-local histogram into the global one (nonzero bins only).
__device__ __forceinline__ void flush_hist(const uint32_t* lh, uint32_t* gh, int bins) {
  for (int i = threadIdx.x; i < bins; i += blockDim.x) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Bucket search: the bucket holding the k-th largest element and k's rank
// inside it.  Thread t of the 256-thread block holds the counts of buckets
// hi-1, hi-2, ..., hi-PER (hi = 256 PER - PER t) in v[0..PER), i.e. the
// buckets in descending order are spread over the threads in thread order.
// A wave-level scan and one exchange of wave totals find the owner thread,
// which writes the bucket to *digit and the rank to *k_in (shared memory,
// set by the caller for the case where no thread matches).  Two barriers.
template <int PER>
__device__ void bucket_search(const uint32_t (&v)[PER], uint32_t k, uint32_t* digit, uint32_t* k_in) {
  __shared__ uint32_t wtot[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t my = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) my += v[j];
  uint32_t incl = my;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  uint32_t before = incl - my;
  for (int w = 0; w < wv; ++w) before += wtot[w];
  if (before < k && k <= before + my) {
    const int hi = PER * 256 - PER * (int)threadIdx.x;
    uint32_t acc = before;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (acc < k && k <= acc + v[j]) {
        *digit = (uint32_t)(hi - 1 - j);
        *k_in = k - acc;
      }
      acc += v[j];
    }
  }
  __syncthreads();
}

// The PER counts of this thread's buckets (see bucket_search) from a bin array.
template <int PER>
__device__ __forceinline__ void my_buckets(const uint32_t* cnt, uint32_t (&v)[PER]) {
  const int lo = PER * 256 - PER * ((int)threadIdx.x + 1);   // lowest bucket of the thread
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const u32x4 w = *(const u32x4*)(cnt + lo + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[PER - 1 - (j + i)] = w[i];
  }
}

// ------------------------------------------------------------------ MXFP4 indexer

template <int QT, int NHG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 3 : 1)))
index_mxfp4_kernel(IndexLaunch a) {
  __shared__ uint32_t lhist[QT][kBins1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;       // k-group of the operand / row group of the result
  const int col = lane & 15;
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * QT;
  constexpr int nhg = NHG;       // head groups of 16 (H_I / 16)

  for (int i = threadIdx.x; i < QT * kBins1; i += 256) (&lhist[0][0])[i] = 0;
  __syncthreads();

  // Key groups of 64 (four 16-key tiles) are dealt to the waves of the
  // sequence round-robin: wave W scores groups W, W + NW, W + 2 NW, ... so
  // the waves of the grid stream one contiguous front of the key cache
  // (HBM serves that faster than one private stream per wave).
  const int NW = 4 * (int)gridDim.x;                         // waves per sequence
  const int W = (int)blockIdx.x * 4 + wave;
  constexpr int kGroups = kTilesPerWave / 4;                 // groups per wave
  // Paged keys: k0 / k1 are the pools and the wave's 2 kGroups blocks (two
  // per 64-key group) are looked up once, lane l holding slot l; contiguous
  // keys start at the sequence's row 0.
  const bool paged = a.bt != nullptr;
  const uint8_t* kc = (const uint8_t*)a.k0 + (paged ? 0 : (int64_t)b * a.n_cap * 64);
  const uint32_t* ks = (const uint32_t*)a.k1 + (paged ? 0 : (int64_t)b * a.n_cap);

  // Waves with a key of the capacity request their first ring of keys before
  // the visible counts arrive (the counts only set the loop's trip count and
  // which scores are kept); a wave with no key of the capacity has nothing to
  // write.
  if (W < (a.n_cap + 63) / 64) {
    int blk_v = -1;
    if (paged && lane < 2 * kGroups) {
      const int lb = 2 * (W + (lane >> 1) * NW) + (lane & 1);
      if (lb * 32 < a.n_cap) blk_v = a.bt[(int64_t)b * a.bt_stride + lb];
    }
    // query operands: head (16 hg + col), bytes 16g .. 16g+15 of its 64-byte row
    i32x4 qa[QT][4];
    int qs[QT][4];
    float wv[QT][4][4];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const int r = (r0 + qi < a.n_qb) ? r0 + qi : r0;
      const int64_t qrow = ((int64_t)b * a.n_q + a.q_first + r) * a.H_I;
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        if (hg < nhg) {
          const int64_t h = qrow + hg * 16 + col;
          qa[qi][hg] = *(const i32x4*)((const uint8_t*)a.q0 + h * 64 + g * 16);
          qs[qi][hg] = ((const uint8_t*)a.q1)[h * 4 + g];
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[qi][hg][i] = a.w[qrow + hg * 16 + 4 * g + i];
        }
      }
    }
    // Keys and scores go through buffer resources over the sequence (only
    // visible keys for the loads): the hardware range check returns zeros
    // for loads past the end and drops stores past it, so no memory
    // instruction in the loop is conditional.  That keeps the compiler's
    // count of loads in flight exact across iterations, and the ring stays
    // full instead of draining once per round.  (Byte offsets fit 32 bits:
    // n_cap <= 4M keys.)
    const uint32_t n_rec = paged ? (uint32_t)a.pool_blocks * 32u : (uint32_t)a.n_cap;   // key rows in range
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kc, 0, (int)(n_rec * 64u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ks, 0, (int)(n_rec * 4u), kBufferWord3);
    __amdgpu_buffer_rsrc_t rsc[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const bool live = r0 + qi < a.n_qb;
      float* srow = score_row(a, b, live ? r0 + qi : r0);
      rsc[qi] = __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0,
                                                  live ? (int)((uint32_t)a.n_cap * (bf16_scores(a) ? 2u : 4u)) : 0,
                                                  kBufferWord3);
    }
    const uint32_t gs_c = (uint32_t)NW * 4096u, gs_s = (uint32_t)NW * 256u;   // group strides: codes, words
    const uint32_t off_c = (uint32_t)W * 4096u + (uint32_t)col * 64u + (uint32_t)g * 16u;
    // Every lane loads the scale word of its key (16 t + col) with the codes
    // (the byte of its k-group g is the operand's block scale).  Scores move
    // four tiles (64 keys) at a time, as one 256-byte store per wave: lane
    // (g, col) keeps the score of tile g of the group.
    // Scale words: lane l loads the word of key l of a 64-key group with the
    // group's first tile (one 4-byte load per lane and group, against one per
    // lane and tile when every lane fetched its own key's word: four lanes
    // share each word), and the words of the four tiles' keys reach the lanes
    // that use them by lane permutes.
    const uint32_t off_o = (uint32_t)W * 256u + (uint32_t)lane * 4u;
    // ring of kRing tiles in flight (16 B of codes per lane and tile, a scale
    // word per lane and group); tile t + kRing is requested as soon as tile t
    // is scored (tiles past the wave's keys read as zeros without touching
    // memory)
    static_assert(kRing % 4 == 0, "tiles move in groups of four");
    i32x4 kbuf[kRing];
    uint32_t kscg[kRing / 4];
    // tile t of the wave (t % 4 == u % 4): tile t % 4 of its group t / 4
    auto fetch = [&](int t, int u) {
      const uint32_t j = (uint32_t)t >> 2, q = (uint32_t)u & 3u;
      uint32_t oc = off_c + j * gs_c + q * 1024u, os = off_o + j * gs_s;
      if (paged) {
        // tile q of group j: rows 16 (q % 2) .. +15 of the group's block q / 2;
        // an unallocated block (or a tile past the wave's) reads zeros
        const int sl = 2 * (int)j + (int)(q >> 1);
        const int blk = sl < 2 * kGroups ? __builtin_amdgcn_readlane(blk_v, sl) : -1;
        const bool ok = blk >= 0 && blk < a.pool_blocks;
        const uint32_t row = 16u * (q & 1u) + (uint32_t)col;
        oc = ok ? (uint32_t)blk * 2048u + row * 64u + (uint32_t)g * 16u : 0xffffff00u;
        if (q == 0) {
          // key l of the group: row l % 32 of the group's block l / 32
          const int s0 = 2 * (int)j;
          const int b0 = s0 < 2 * kGroups ? __builtin_amdgcn_readlane(blk_v, s0) : -1;
          const int b1 = s0 + 1 < 2 * kGroups ? __builtin_amdgcn_readlane(blk_v, s0 + 1) : -1;
          const int bl = lane < 32 ? b0 : b1;
          os = bl >= 0 && bl < a.pool_blocks ? (uint32_t)bl * 128u + (uint32_t)(lane & 31) * 4u : 0xffffff00u;
        }
      }
      kbuf[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 0));
      if (q == 0) kscg[u >> 2] = __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
    };
    // issue the first round in ring order (the loop consumes it in that order)
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      fetch(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    int nvis[QT];
    int nvis_max = 0;
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      // the counts are uniform over the workgroup: keep them in scalar registers
      nvis[qi] = __builtin_amdgcn_readfirstlane((r0 + qi < a.n_qb) ? query_n_vis(a, b, r0 + qi) : 0);
      nvis_max = nvis[qi] > nvis_max ? nvis[qi] : nvis_max;
    }
    // (the maximum may be formed with a vector instruction: make it a scalar
    // again, or the loop bound below turns into a per-lane one)
    nvis_max = __builtin_amdgcn_readfirstlane(nvis_max);
    const int ngv = (nvis_max + 63) / 64;                    // groups with a visible key
    // rounds over the wave's groups that hold a visible key
    int vgroups = W < ngv ? (ngv - W + NW - 1) / NW : 0;
    vgroups = vgroups < kGroups ? vgroups : kGroups;
    const int n_rounds = (vgroups * 4 + kRing - 1) / kRing;
    for (int t0 = 0; t0 < n_rounds * kRing; t0 += kRing) {
      float part[QT][4];      // lane partials of the group's four tiles
      uint32_t ksw[4];        // scale words of the keys of the group's four tiles (this lane's column)
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
        const int t = t0 + u;
        if (u % 4 == 0) {
          // the group's words, before the slot takes the next group's
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) ksw[qq] = (uint32_t)__shfl((int)kscg[u >> 2], 16 * qq + col, 64);
        }
        const i32x8 kb = {kbuf[u][0], kbuf[u][1], kbuf[u][2], kbuf[u][3], 0, 0, 0, 0};
        const int ksc = (int)((ksw[u % 4] >> (8 * g)) & 0xffu);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
          // w . ReLU over the lane's 4 heads of every head group, in two
          // chains (head groups 0-1 and 2-3)
          float hpart[2] = {0.f, 0.f};
#pragma unroll
          for (int hg = 0; hg < nhg; ++hg) {
            i32x8 qv = {qa[qi][hg][0], qa[qi][hg][1], qa[qi][hg][2], qa[qi][hg][3], 0, 0, 0, 0};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qv, kb, acc, 4, 4, 0,
                                                                   qs[qi][hg], 0, ksc);
            float hp = (hg & 1) ? hpart[hg >> 1] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              hp = ((hg & 1) == 0 && i == 0) ? wv[qi][hg][0] * relu(acc[0]) : fmaf(wv[qi][hg][i], relu(acc[i]), hp);
            hpart[hg >> 1] = hp;
          }
          part[qi][u % 4] = nhg > 2 ? hpart[0] + hpart[1] : hpart[0];
          if (u % 4 == 3) {
            // Sum the four row groups of each of the group's four tiles and
            // leave tile g's sum in row group g: swaps 32 lanes apart pair
            // tiles 0/2 and 1/3 (lanes 0-31 then hold tiles 0 and 1, lanes
            // 32-63 tiles 2 and 3), a swap 16 lanes apart splits the pairs.
            const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qi][0]),
                                                              __float_as_uint(part[qi][2]), false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qi][1]),
                                                              __float_as_uint(part[qi][3]), false, false);
            const float b0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
            const float b1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
            const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b0), __float_as_uint(b1), false, false);
            const float tot = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
            const uint32_t j = (uint32_t)t >> 2;          // the group
            const int key = (W + (int)j * NW) * 64 + lane;
            const bool vis = key < nvis[qi];
            const float sc = vis ? tot : -INFINITY;
            if (bf16_scores(a)) {
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(sc), rsc[qi], (off_o + j * gs_s) >> 1, 0, 0);
              if (vis) atomicAdd(&lhist[qi][order_key(bf16_to_f32(f32_to_bf16(sc))) >> kShift1], 1u);
            } else {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc[qi], off_o + j * gs_s, 0, 0);
              if (vis) atomicAdd(&lhist[qi][order_key(sc) >> kShift1], 1u);
            }
          }
        }
        fetch(t + kRing, u);
      }
    }
    // groups of this wave that the rounds did not reach get -inf
#pragma unroll
    for (int qi = 0; qi < QT; ++qi)
      for (uint32_t j = (uint32_t)(n_rounds * kRing / 4); j < (uint32_t)kGroups; ++j) {
        if (bf16_scores(a))
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0xff80u, rsc[qi], (off_o + j * gs_s) >> 1, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), rsc[qi], off_o + j * gs_s, 0, 0);
      }
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < QT; ++qi)
    if (r0 + qi < a.n_qb) flush_hist(lhist[qi], a.hist + ((int64_t)b * a.n_qb + r0 + qi) * kBins1, kBins1);
}

// ------------------------------------------------------------------ MXFP4 indexer, query blocks

// Many queries per call (a prefill chunk) make the scoring compute-bound, and
// there the ReLU and head weighting cost more vector instructions than the
// matrix cores spend on the dot products.  This path therefore
//  * uses V_MFMA_SCALE_F32_32X32X64_F8F6F4, which runs MXFP4 at twice the
//    rate of the 16x16x128 form: 32 heads x 32 keys per pair of instructions
//    (two 64-wide halves of the 128-wide dot product);
//  * writes w ReLU(s) = (w/2)|s| + (w/2)s.  The first term is one fused
//    multiply-add per head and key with the absolute value taken as an operand
//    modifier; the second, summed over heads, is u . k with
//    u = sum_h (w_h/2) q_h, a single dot product per query and key that the
//    matrix cores take from index_linear_kernel's FP8 split of u (six E4M3
//    components, each with its own E8M0 block scales, so u is carried to
//    about 24 significant bits of its block maximum: the score differs from
//    the exact one by at most about 2^-24 sum_blocks max|u| sum |k|, the
//    order of fp32 rounding).  The linear operand's 32 rows hold
//    component 4 (row / 8) + row % 4 of query (row / 4) % 2, so a lane's
//    result elements 0-5 are the six components of the query of its lane half.
// Every lane of the result holds 16 heads of one key; the two lane halves are
// summed by one 32-lane swap that also leaves query 0 in lanes 0-31 and
// query 1 in lanes 32-63.  The products are software-pipelined one head group
// ahead (the matrix cores work on group g + 1 while the vector unit weighs
// group g, and on the next tile's first group during a tile's epilogue); the
// score dtype and paging are template arguments, so a round of tiles is one
// basic block the scheduler can interleave.
//
// Operand layouts of the 32x32x64 form (per lane l, K-step s of 64 dims):
//   MXFP4 (keys, query heads): row/column l % 32, dims 64 s + 32 (l / 32) .. +31
//     = 16 bytes at byte 32 s + 16 (l / 32) of the 64-byte row, E8M0 scale of
//     block 2 s + l / 32;
//   FP8: bytes 0-15 hold dims 64 s + 16 (l / 32) .. +15, bytes 16-31 dims
//     64 s + 32 + 16 (l / 32) .. +15, E8M0 scale of block 2 s + l / 32;
//   result element 4 j + i: row 8 j + 4 (l / 32) + i, column l % 32.
constexpr int kLinComps = 6;
constexpr int kLinScaleOff = kLinComps * 128;   // per query: FP8 codes [6][128], then E8M0 scales [6][4]
constexpr int kLinBytes = kIndexLinBytes;
static_assert(kLinScaleOff + kLinComps * 4 <= kLinBytes, "linear split fits its slot");
constexpr int kMqQT = 2;             // queries per workgroup
constexpr int kMqTiles = 256;        // 32-key tiles per wave
constexpr int kMqRing = 4;           // tiles of keys in flight per wave

// u = sum_h (w_h / 2) q_h for query (b, r) of the block, in fp32 over
// ascending h, then its six FP8 components: c_1 = RNE(u / s_1),
// c_2 = RNE((u - s_1 c_1) / s_2), ...; each E8M0 scale s puts its 32-dim
// block's largest magnitude in [128, 256), inside the E4M3 range.  Every
// stage leaves at most 2^-4 of the block's largest magnitude (relative
// rounding 2^-4 for normal codes, 2^-10 absolute below them), so after six
// the residual of every element is below 2^-24 max_block |u|: the split
// carries u as far as fp32 does.
__global__ void __launch_bounds__(128) index_linear_kernel(IndexLaunch a) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int k = threadIdx.x;                  // dim (d_I = 128)
  const int64_t qrow = ((int64_t)b * a.n_q + a.q_first + r) * a.H_I;
  const uint8_t* qc = (const uint8_t*)a.q0;
  const uint8_t* qsc = (const uint8_t*)a.q1;
  float u = 0.f;
#pragma unroll 8
  for (int hh = 0; hh < a.H_I; ++hh) {
    const uint32_t byte = qc[(qrow + hh) * 64 + (k >> 1)];
    const float v = e2m1_to_f32((byte >> (4 * (k & 1))) & 15u) *
                    ldexpf(1.0f, (int)qsc[(qrow + hh) * 4 + (k >> 5)] - 127);
    u = fmaf(0.5f * a.w[qrow + hh], v, u);
  }
  uint8_t* out = a.lin + ((int64_t)b * a.n_qb + r) * kLinBytes;
  float res = u;
  for (int c = 0; c < kLinComps; ++c) {
    float m = fabsf(res);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
    int e = -127;
    if (m > 0.0f) {
      int ex;
      frexpf(m, &ex);
      e = ex - 8;                              // m / 2^e in [128, 256)
    }
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const uint32_t code = f32_to_e4m3(res * ldexpf(1.0f, -e));
    out[c * 128 + k] = (uint8_t)code;
    if ((k & 31) == 0) out[kLinScaleOff + c * 4 + (k >> 5)] = (uint8_t)(e + 127);
    res -= e4m3_to_f32(code) * ldexpf(1.0f, e);
  }
}

// Tiles of wave W (of NW per sequence, TPW at most) that hold a visible key.
__device__ __forceinline__ int vt_all(int ntv, int W, int NW, int TPW) {
  const int v = (ntv - W + NW - 1) / NW;
  return v < TPW ? v : TPW;
}

template <int NH32, bool BF16, bool PAGED>
__global__ void __launch_bounds__(256) index_mxfp4_mq_kernel(IndexLaunch a) {
  constexpr int QT = kMqQT, R = kMqRing, TPW = kMqTiles;
  // one spare bin per query takes the adds of invisible keys, so the add needs no branch
  __shared__ uint32_t lhist[QT][kBins1 + 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;        // operand dim half / result row half; after the swap: the query
  const int col = lane & 31;      // key of the tile; row of the query operands
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * QT;
  const int live_q = a.n_qb - r0 < QT ? a.n_qb - r0 : QT;

  for (int i = threadIdx.x; i < QT * (kBins1 + 4); i += 256) (&lhist[0][0])[i] = 0;
  int nvis[QT];
  int nvis_max = 0;
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    nvis[qi] = __builtin_amdgcn_readfirstlane(qi < live_q ? query_n_vis(a, b, r0 + qi) : 0);
    nvis_max = nvis[qi] > nvis_max ? nvis[qi] : nvis_max;
  }
  nvis_max = __builtin_amdgcn_readfirstlane(nvis_max);
  __syncthreads();

  // 32-key tiles are dealt to the waves of the sequence round-robin
  const int NW = 4 * (int)gridDim.x;
  const int W = (int)blockIdx.x * 4 + wave;
  const int ntv = (nvis_max + 31) / 32;        // tiles with a visible key
  // paged keys: k0 / k1 are the pools, a 32-key tile is one block
  constexpr bool paged = PAGED;
  const uint8_t* kc = (const uint8_t*)a.k0 + (paged ? 0 : (int64_t)b * a.n_cap * 64);
  const uint32_t* ks = (const uint32_t*)a.k1 + (paged ? 0 : (int64_t)b * a.n_cap);
  // both query rows of the block's scores through one resource: rows past
  // the live queries are outside it, so their stores are dropped
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)score_row(a, b, r0), 0,
      (int)((uint32_t)live_q * (uint32_t)a.n_cap * (BF16 ? 2u : 4u)), kBufferWord3);
  const int my_nvis = h ? nvis[1] : nvis[0];
  // byte offset of this lane's score for key `key`; keys past the row map
  // outside the resource (their stores are dropped instead of landing in the
  // next query's row)
  constexpr uint32_t es = BF16 ? 2u : 4u;
  auto score_off = [&](int key) {
    return key < a.n_cap ? ((uint32_t)h * (uint32_t)a.n_cap + (uint32_t)key) * es : 0xfffffff0u;
  };
  auto store_sc = [&](float v, uint32_t off) {
    if constexpr (BF16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rsc, off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsc, off, 0, 0);
  };

  if (W < ntv) {
    i32x4 qa[QT][NH32][2];
    int qs[QT][NH32][2];
    float w2[QT][NH32][16];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const int r = qi < live_q ? r0 + qi : r0;
      const int64_t qrow = ((int64_t)b * a.n_q + a.q_first + r) * a.H_I;
#pragma unroll
      for (int hg = 0; hg < NH32; ++hg) {
        const int64_t head = qrow + hg * 32 + col;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          qa[qi][hg][s] = *(const i32x4*)((const uint8_t*)a.q0 + head * 64 + 32 * s + 16 * h);
          qs[qi][hg][s] = ((const uint8_t*)a.q1)[head * 4 + 2 * s + h];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
          w2[qi][hg][e] = 0.5f * a.w[qrow + hg * 32 + 8 * (e >> 2) + 4 * h + (e & 3)];
      }
    }
    // linear operand: row col = component 4 (col / 8) + col % 4 (components
    // 6, 7 of the 8-row groups are zero) of query (col / 4) % 2
    const int lc = 4 * (col >> 3) + (col & 3);
    const int lq = ((col >> 2) & 1) < live_q ? ((col >> 2) & 1) : 0;
    const uint8_t* lin = a.lin + ((int64_t)b * a.n_qb + r0 + lq) * kLinBytes;
    i32x8 la[2];
    int ls[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const i32x4 lo = lc < kLinComps ? *(const i32x4*)(lin + lc * 128 + 64 * s + 16 * h) : (i32x4){0, 0, 0, 0};
      const i32x4 hi = lc < kLinComps ? *(const i32x4*)(lin + lc * 128 + 64 * s + 32 + 16 * h) : (i32x4){0, 0, 0, 0};
      la[s] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      ls[s] = lc < kLinComps ? (int)lin[kLinScaleOff + lc * 4 + 2 * s + h] : 127;
    }
    const uint32_t n_rec = paged ? (uint32_t)a.pool_blocks * 32u : (uint32_t)a.n_cap;   // key rows in range
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kc, 0, (int)(n_rec * 64u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ks, 0, (int)(n_rec * 4u), kBufferWord3);
    const uint32_t off_c = (uint32_t)W * 2048u + (uint32_t)col * 64u + (uint32_t)h * 16u;
    const uint32_t off_s = (uint32_t)W * 128u + (uint32_t)col * 4u;
    const uint32_t st_c = (uint32_t)NW * 2048u, st_s = (uint32_t)NW * 128u;
    // paged: the block of the wave's tile 64 r + l in register r of lane l
    int blk_v[TPW / 64];
#pragma unroll
    for (int r = 0; r < TPW / 64; ++r) {
      const int T = W + (64 * r + lane) * NW;
      blk_v[r] = paged && 64 * r + lane < vt_all(ntv, W, NW, TPW) ? a.bt[(int64_t)b * a.bt_stride + T] : -1;
    }
    i32x4 kb[R][2];
    uint32_t kw[R];
    auto fetch = [&](int j, int u) {
      uint32_t oc = off_c + (uint32_t)j * st_c, os = off_s + (uint32_t)j * st_s;
      if constexpr (PAGED) {
        const int r = j >> 6;
        const int v = r == 0 ? blk_v[0] : r == 1 ? blk_v[1] : r == 2 ? blk_v[2] : blk_v[3];
        const int blk = j < TPW ? __builtin_amdgcn_readlane(v, j & 63) : -1;
        const bool ok = blk >= 0 && blk < a.pool_blocks;
        oc = ok ? (uint32_t)blk * 2048u + (uint32_t)col * 64u + (uint32_t)h * 16u : 0xffffff00u;
        os = ok ? (uint32_t)blk * 128u + (uint32_t)col * 4u : 0xffffff00u;
      }
      kb[u][0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 0));
      kb[u][1] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc + 32u, 0, 0));
      kw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
    };
#pragma unroll
    for (int u = 0; u < R; ++u) {
      fetch(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    int vt = (ntv - W + NW - 1) / NW;
    vt = vt < TPW ? vt : TPW;
    const int n_rounds = (vt + R - 1) / R;
    // key operands of ring slot u
    auto kop = [&](int u, int s) {
      return (i32x8){kb[u][s][0], kb[u][s][1], kb[u][s][2], kb[u][s][3], 0, 0, 0, 0};
    };
    // the keys' scale words shifted so that the matrix instruction's byte
    // select picks block 2 s + h as byte 2 s
    auto ksw = [&](int u) { return (int)(kw[u] >> (8 * h)); };
    // the head group g = qi * NH32 + hg against the keys of ring slot u
    auto head_pair = [&](int g, int u) {
      const int qi = g / NH32, hg = g % NH32;
      const i32x8 a0 = {qa[qi][hg][0][0], qa[qi][hg][0][1], qa[qi][hg][0][2], qa[qi][hg][0][3], 0, 0, 0, 0};
      const i32x8 a1 = {qa[qi][hg][1][0], qa[qi][hg][1][1], qa[qi][hg][1][2], qa[qi][hg][1][3], 0, 0, 0, 0};
      f32x16 acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, kop(u, 0), acc, 4, 4, 0, qs[qi][hg][0], 0, ksw(u));
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, kop(u, 1), acc, 4, 4, 0, qs[qi][hg][1], 2, ksw(u));
      return acc;
    };
    constexpr int G = QT * NH32;
    // the linear product of the keys of ring slot u
    auto lin_pair = [&](int u) {
      f32x16 acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(la[0], kop(u, 0), acc, 0, 4, 0, ls[0], 0, ksw(u));
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(la[1], kop(u, 1), acc, 0, 4, 0, ls[1], 2, ksw(u));
      return acc;
    };
    // software pipeline: the first head group and the linear product of a
    // tile are multiplied while the previous tile's epilogue runs, every
    // later head group while the previous group's weights are applied
    f32x16 acc_cur = head_pair(0, 0);
    for (int j0 = 0; j0 < n_rounds * R; j0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int j = j0 + u;
        const int un = (u + 1) % R;
        const f32x16 accl = lin_pair(u);
        float pp[QT] = {};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          f32x16 nxt;
          if (g + 1 < G) {
            nxt = head_pair(g + 1, u);
          } else {
            nxt = head_pair(0, un);
          }
          const int qi = g / NH32, hg = g % NH32;
#pragma unroll
          for (int e = 0; e < 16; ++e) pp[qi] = fmaf(w2[qi][hg][e], fabsf(acc_cur[e]), pp[qi]);
          acc_cur = nxt;
        }
        float part[QT];
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) part[qi] = pp[qi];
        // lanes 0-31: query 0, lanes 32-63: query 1, summed over both row halves
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
        // the linear term of this lane half's query, smallest components first
        const float lin = ((((accl[5] + accl[4]) + accl[3]) + accl[2]) + accl[1]) + accl[0];
        const float tot = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) + lin;
        const int key = (W + j * NW) * 32 + col;
        const bool vis = key < my_nvis;
        const float sc = vis ? tot : -INFINITY;
        store_sc(sc, score_off(key));
        const float kept = BF16 ? bf16_to_f32(f32_to_bf16(sc)) : sc;
        atomicAdd(&lhist[h][vis ? (int)(order_key(kept) >> kShift1) : kBins1], 1u);
        fetch(j + R, u);
      }
    }
    // tiles of this wave that the rounds did not reach get -inf
    for (int j = n_rounds * R; j < TPW; ++j) {
      store_sc(-INFINITY, score_off((W + j * NW) * 32 + col));
    }
  } else {
    // no query sees any key of this wave
    for (int j = 0; j < TPW; ++j) {
      const int64_t key = (int64_t)(W + j * NW) * 32 + col;
      if (h < live_q && key < a.n_cap) store_score(a, score_row(a, b, r0 + h), key, -INFINITY);
    }
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < QT; ++qi)
    if (qi < live_q) flush_hist(lhist[qi], a.hist + ((int64_t)b * a.n_qb + r0 + qi) * kBins1, kBins1);
}

// ------------------------------------------------------------------ fp32 indexer (precision mode)

__global__ void __launch_bounds__(256) index_f32_kernel(IndexLaunch a) {
  __shared__ uint32_t lhist[kBins1];
  const int b = blockIdx.z, r = blockIdx.y;
  for (int i = threadIdx.x; i < kBins1; i += 256) lhist[i] = 0;
  __syncthreads();
  const int nvis = query_n_vis(a, b, r);
  const int64_t key = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t qrow = ((int64_t)b * a.n_q + a.q_first + r) * a.H_I;
  if (key < a.n_cap) {
    float s = -INFINITY;
    if (key < nvis) {
      int64_t row = (int64_t)b * a.n_cap + key;
      if (a.bt) {                    // paged: row key % block_rows of its block (none: a zero key)
        const int blk = a.bt[(int64_t)b * a.bt_stride + key / a.block_rows];
        row = blk >= 0 && blk < a.pool_blocks ? (int64_t)blk * a.block_rows + key % a.block_rows : -1;
      }
      const float* k = (const float*)a.k0 + (row < 0 ? 0 : row) * a.d_I;
      s = 0.f;
      for (int h = 0; h < a.H_I; ++h) {
        const float* q = (const float*)a.q0 + (qrow + h) * a.d_I;
        float dot = 0.f;
        if (row >= 0)
          for (int c = 0; c < a.d_I; ++c) dot = fmaf(q[c], k[c], dot);
        s += a.w[qrow + h] * fmaxf(dot, 0.f);
      }
      atomicAdd(&lhist[order_key(stored_score(a, s)) >> kShift1], 1u);
    }
    store_score(a, score_row(a, b, r), key, s);
  }
  __syncthreads();
  flush_hist(lhist, a.hist + ((int64_t)b * a.n_qb + r) * kBins1, kBins1);
}

// ------------------------------------------------------------------ collect / refine / write

__device__ __forceinline__ int block_sum_int(int v, int* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Exclusive scan over the block (256 threads) in thread order; *total gets
// the block sum when given.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total = nullptr) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wv; ++w) off += wsum[w];
  if (total) *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return off + incl - v;
}



// Query blocks: the first-digit bucket of the k-th largest score and the rank
// inside it, once per query (the list form of collect reads it from the
// state instead of every chunk workgroup searching the histogram).
__global__ void __launch_bounds__(256) topk_bucket_kernel(IndexLaunch a) {
  const int q = blockIdx.x;
  const int b = q / a.n_qb, r = q % a.n_qb;
  const int n_vis = query_n_vis(a, b, r);
  TopkState st = {};
  st.n_vis = n_vis;
  if (n_vis <= a.top_k) {                       // every visible entry is taken
    st.k_rem = -1;
  } else {
    __shared__ uint32_t s_digit, s_kin;
    if (threadIdx.x == 0) { s_digit = 0; s_kin = 0; }
    uint32_t v[kBins1 / 256];
    my_buckets(a.hist + (int64_t)q * kBins1, v);
    bucket_search(v, (uint32_t)a.top_k, &s_digit, &s_kin);
    st.b1 = s_digit;
    st.k_rem = (int)s_kin;
  }
  if (threadIdx.x == 0) a.state[q] = st;
}

// Per chunk: keys above the first-digit bucket are counted, keys inside it go
// to the chunk's own region of the query's candidate list (no global atomics).
// LIST: the chunk's indices above the bucket and its candidates' indices are
// also written, in index order, over the chunk's scores.
template <bool LIST>
__global__ void __launch_bounds__(256) topk_collect_kernel(IndexLaunch a) {
  const int q = blockIdx.y;
  const int b = q / a.n_qb, r = q % a.n_qb;
  const int n_vis = query_n_vis(a, b, r);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (n_vis <= a.top_k) {                       // every visible entry is taken
    if (!LIST && blockIdx.x == 0 && threadIdx.x == 0) {
      TopkState st = {};
      st.n_vis = n_vis;
      st.k_rem = -1;
      a.state[q] = st;
    }
    return;
  }
  if (c0 >= n_vis) return;
  if constexpr (!LIST) {
    // this chunk's scores are requested first: they do not depend on the search
    const float* sc = score_row(a, q / a.n_qb, q % a.n_qb);
    float sv[kChunk / 256];
#pragma unroll
    for (int j = 0; j < kChunk / 256; ++j) {
      const int64_t i = c0 + j * 256 + threadIdx.x;
      sv[j] = i < n_vis ? load_score(a, sc, i) : 0.f;
    }
    // every workgroup finds the first-digit bucket of the k-th largest score
    __shared__ uint32_t s_digit, s_kin;
    if (threadIdx.x == 0) { s_digit = 0; s_kin = 0; }
    {
      uint32_t v[kBins1 / 256];
      my_buckets(a.hist + (int64_t)q * kBins1, v);
      bucket_search(v, (uint32_t)a.top_k, &s_digit, &s_kin);
    }
    TopkState st = {};
    st.n_vis = n_vis;
    st.b1 = s_digit;
    st.k_rem = (int)s_kin;
    if (blockIdx.x == 0 && threadIdx.x == 0) a.state[q] = st;
    uint32_t* ck = a.cand_key + (int64_t)q * a.n_cap + c0;
    int above = 0;
    uint32_t want = 0;
    uint32_t keys[kChunk / 256];
#pragma unroll
    for (int j = 0; j < kChunk / 256; ++j) {
      const int64_t i = c0 + j * 256 + threadIdx.x;
      const bool in = i < st.n_vis;
      keys[j] = in ? order_key(sv[j]) : 0u;
      const uint32_t d1 = keys[j] >> kShift1;
      above += (in && d1 > st.b1) ? 1 : 0;
      want |= (uint32_t)(in && d1 == st.b1) << j;
    }
    __shared__ int red[4];
    int n_here;
    int slot = block_excl_scan(__popc(want), red, &n_here);
#pragma unroll
    for (int j = 0; j < kChunk / 256; ++j)
      if (want >> j & 1u) ck[slot++] = keys[j];
    above = block_sum_int(above, red);
    if (threadIdx.x == 0) {
      a.chunk_above[(int64_t)q * a.n_chunks + blockIdx.x] = above;
      a.chunk_cand[(int64_t)q * a.n_chunks + blockIdx.x] = n_here;
    }
  } else {
    // Lists of indices in index order: thread t holds the 16 consecutive
    // entries c0 + 16 t + j, so the scans in thread order give index order.
    float* const sc = score_row(a, q / a.n_qb, q % a.n_qb);
    constexpr int PT = kChunk / 256;
    static_assert(PT == 16, "thread t takes entries c0 + 16 t .. +15");
    // thread t loads its 16 consecutive entries (four 16-byte loads of fp32
    // scores, two of BF16 codes) when they lie inside the visible range and
    // the row is 16-byte aligned (a caller's row length may be odd), entry
    // by entry otherwise
    const int64_t e0 = c0 + 16 * (int64_t)threadIdx.x;
    const bool row_aligned = (((uintptr_t)sc) & 15) == 0;
    float sv[PT];
    if (e0 + PT <= n_vis && row_aligned) {
      if (bf16_scores(a)) {
        const uint16_t* r16 = (const uint16_t*)sc + e0;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const i32x4 w = *(const i32x4*)(r16 + 8 * v);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[8 * v + 2 * i] = __uint_as_float((uint32_t)w[i] << 16);
            sv[8 * v + 2 * i + 1] = __uint_as_float((uint32_t)w[i] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const f32x4 w = *(const f32x4*)(sc + e0 + 4 * v);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[4 * v + i] = w[i];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PT; ++j) sv[j] = e0 + j < n_vis ? load_score(a, sc, e0 + j) : 0.f;
    }
    // the bucket of the k-th key, found once per query by topk_bucket_kernel
    const TopkState st = a.state[q];
    uint32_t keys[PT];
    uint32_t want = 0, above = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const bool in = e0 + j < st.n_vis;
      keys[j] = in ? order_key(sv[j]) : 0u;
      const uint32_t d1 = keys[j] >> kShift1;
      above |= (uint32_t)(in && d1 > st.b1) << j;
      want |= (uint32_t)(in && d1 == st.b1) << j;
    }
    __shared__ int red[2][4];
    int n_here, n_above;
    int slot = block_excl_scan(__popc(want), red[0], &n_here);
    int aslot = block_excl_scan(__popc(above), red[1], &n_above);
    uint32_t* ck = a.cand_key + (int64_t)q * a.n_cap + c0;
    // the chunk's own score region (read in full above) takes the indices
    // above the bucket, then the candidates' indices: 32-bit indices over
    // fp32 scores, 16-bit offsets in the chunk over BF16 scores (a chunk's
    // 4096 two-byte slots hold any of its lists)
    const bool b16 = bf16_scores(a);
    uint32_t* const lst = (uint32_t*)sc + c0;
    uint16_t* const lst16 = (uint16_t*)sc + c0;
    auto put = [&](int at, int e_off) {
      if (b16) lst16[at] = (uint16_t)e_off;
      else lst[at] = (uint32_t)(c0 + e_off);
    };
    const int o0 = 16 * (int)threadIdx.x;        // e0 - c0
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (want >> j & 1u) {
        ck[slot] = keys[j];
        put(n_above + slot, o0 + j);
        ++slot;
      }
      if (above >> j & 1u) put(aslot++, o0 + j);
    }
    if (threadIdx.x == 0) {
      a.chunk_above[(int64_t)q * a.n_chunks + blockIdx.x] = n_above;
      a.chunk_cand[(int64_t)q * a.n_chunks + blockIdx.x] = n_here;
    }
  }
}

// Selection, one workgroup per (chunk, query).  Every workgroup of a query
// repeats the same small computation over the query's candidates (the keys in
// the first-digit bucket, a few hundred in practice): radix-select the
// k_rem-th largest of them (bits 19..10, then 9..0) to get the k-th largest
// key T and how many keys equal to T are taken (lowest indices first), count
// per chunk the candidates above and at T, and from those counts and the
// chunks' counts above the bucket derive where this chunk's selection starts
// in the output.  It then emits its selected indices in index order.
//
// The candidates are read in one round trip with everything else: the first
// 4096 / n_chunks slots of every chunk's region are loaded before the counts
// are known (16 per thread) and masked by the counts afterwards;
// only a chunk holding more candidates than that needs a second pass over
// its region.
constexpr int kOptSlots = 4096;                 // candidate slots loaded up front per workgroup
__global__ void __launch_bounds__(256) topk_select_kernel(IndexLaunch a) {
  const int q = blockIdx.y;
  const int b = q / a.n_qb, r = q % a.n_qb;
  const int chunk = blockIdx.x;
  const int64_t c0 = (int64_t)chunk * kChunk;
  const int n_chunks_cap = a.n_chunks;          // chunks of the capacity (>= active chunks)
  // slots per chunk of the up-front load: an equal share of the kOptSlots
  // (4 .. 4096; n_chunks_cap <= kMaxChunks).  Not rounded to a power of two:
  // a capacity one block past 2^k chunks would otherwise halve every chunk's
  // share and send full chunks down the slow overflow path.
  const int slots = kOptSlots / n_chunks_cap;
  // virtual slot v = slot + chunk * slots (an exact integer quotient: slots is uniform)
  auto slot_chunk = [&](int v) { return (int)((uint32_t)v / (uint32_t)slots); };
  // ---- one round trip: this thread's 16 scores, the state, every chunk's
  // counts and the leading candidate slots
  const float* sc = score_row(a, q / a.n_qb, q % a.n_qb);
  const int64_t e0 = c0 + threadIdx.x * 16;
  float sv[16];
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    const int64_t i = e0 + j;
    if (i + 3 < a.n_cap) {
      load_score4(a, sc, i, sv + j);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) sv[j + u] = i + u < a.n_cap ? load_score(a, sc, i + u) : -INFINITY;
    }
  }
  const TopkState st = a.state[q];
  constexpr int kCPT = kMaxChunks / 256;       // chunks per thread
  int ccnt[kCPT], cabv[kCPT];
  {
    const int* cc = a.chunk_cand + (int64_t)q * a.n_chunks;
    const int* ca = a.chunk_above + (int64_t)q * a.n_chunks;
#pragma unroll
    for (int j = 0; j < kCPT; ++j) {
      const int c = threadIdx.x + 256 * j;
      ccnt[j] = c < a.n_chunks ? cc[c] : 0;
      cabv[j] = c < a.n_chunks ? ca[c] : 0;
    }
  }
  const uint32_t* ck = a.cand_key + (int64_t)q * a.n_cap;
  constexpr int kOptPT = kOptSlots / 256;       // up-front slots per thread
  uint32_t okey[kOptPT];
#pragma unroll
  for (int j = 0; j < kOptPT; ++j) {
    const int v = (int)threadIdx.x + 256 * j;   // virtual slot: chunk v / slots, slot v % slots
    const int vc = slot_chunk(v);
    const int64_t e = (int64_t)vc * kChunk + (v - vc * slots);
    okey[j] = e < a.n_cap ? ck[e] : 0u;          // (a chunk's candidates never pass the capacity)
  }
  // leave the first-digit histogram zeroed for the next call (collect, its
  // only reader, has finished)
  {
    uint32_t* gh = a.hist + (int64_t)q * kBins1;
    for (int i = chunk * 256 + threadIdx.x; i < kBins1; i += a.n_chunks * 256) gh[i] = 0;
  }
  int32_t* out = a.out_idx + ((int64_t)b * a.n_q + a.q_first + r) * a.top_k;
  if (st.k_rem < 0) {
    // every visible entry, in order; chunk 0 also writes the padding
    for (int64_t i = c0 + threadIdx.x; i < c0 + kChunk && i < st.n_vis; i += 256) out[i] = (int32_t)i;
    if (chunk == 0)
      for (int i = st.n_vis + threadIdx.x; i < a.top_k; i += 256) out[i] = -1;
    return;
  }
  if (c0 >= st.n_vis) return;

  __shared__ __attribute__((aligned(16))) uint32_t bins[2][1024];
  __shared__ int lcnt[kMaxChunks], cgt[kMaxChunks], ceq[kMaxChunks];
  __shared__ uint32_t s_digit[2], s_kin[2];
  __shared__ int s_over;
  __shared__ int red[4][4];
  const int n_act = (st.n_vis + kChunk - 1) / kChunk;
  for (int i = threadIdx.x; i < 2 * 1024; i += 256) (&bins[0][0])[i] = 0;
  if (threadIdx.x < 2) { s_digit[threadIdx.x] = 0; s_kin[threadIdx.x] = 0; }
  if (threadIdx.x == 0) s_over = 0;
  __syncthreads();
  int over = 0;
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < kMaxChunks) {
      const int n = c < n_act ? ccnt[j] : 0;
      lcnt[c] = n;
      cgt[c] = 0;
      ceq[c] = 0;
      over |= n > slots;
    }
  }
  if (over) s_over = 1;
  __syncthreads();
  const bool overflow = s_over != 0;            // some chunk holds more than `slots` candidates
  // candidate v of the up-front load is real when its slot is below its chunk's count
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kOptPT; ++j) {
    const int v = (int)threadIdx.x + 256 * j;
    const int c = slot_chunk(v);
    valid |= (uint32_t)(c < n_act && (v - c * slots) < lcnt[c < kMaxChunks ? c : 0]) << j;
  }
  // every candidate goes through `visit(key, chunk)`: the up-front ones from
  // registers, the rest of an over-full chunk from its region
  auto for_each = [&](auto&& visit) {
#pragma unroll
    for (int j = 0; j < kOptPT; ++j)
      if (valid >> j & 1u) visit(okey[j], slot_chunk((int)threadIdx.x + 256 * j));
    if (overflow) {
      for (int c = 0; c < n_act; ++c) {
        const int n = lcnt[c];
        for (int i = slots + (int)threadIdx.x; i < n; i += 256) visit(ck[(int64_t)c * kChunk + i], c);
      }
    }
  };
  // radix select of the k_rem-th largest candidate: bits 19..10, then 9..0
  uint32_t prefix = st.b1 << kShift1, mask = 0xfff00000u;
  uint32_t k = (uint32_t)st.k_rem;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    for_each([&](uint32_t key, int) {
      if ((key & mask) == prefix) atomicAdd(&bins[pass][(key >> shift) & 1023u], 1u);
    });
    __syncthreads();
    uint32_t v[4];
    my_buckets(bins[pass], v);
    bucket_search(v, k, &s_digit[pass], &s_kin[pass]);
    prefix |= s_digit[pass] << shift;
    mask |= 1023u << shift;
    k = s_kin[pass];
    // BF16 scores: the bits of an order key below bit 16 are all zero (a
    // score >= 0, top key bit set) or all one (a negative score, whose key is
    // the complement of its bits), so bits 19..10 already fix the k-th key
    // (the last pass would put every candidate into one bin)
    if (bf16_scores(a)) {
      if ((prefix >> 31) == 0) prefix |= 1023u;
      break;
    }
  }
  const uint32_t T = prefix;          // the k-th largest key; k = how many keys == T to take
  for_each([&](uint32_t key, int c) {
    if (key > T) atomicAdd(&cgt[c], 1);
    else if (key == T) atomicAdd(&ceq[c], 1);
  });
  __syncthreads();
  // this chunk's output start: the selection of every earlier chunk (above
  // the bucket, above T, and its share of the keys equal to T)
  int sel_before = 0, eq_before = 0;
  {
    int eq_acc = 0, sel_part = 0;
#pragma unroll
    for (int j = 0; j < kCPT; ++j) {
      if (256 * j >= n_act) break;
      const int c = threadIdx.x + 256 * j;
      const bool in = c < n_act;
      const int neq = in ? ceq[c] : 0;
      int eq_sum;
      const int eq_ex = eq_acc + block_excl_scan(neq, red[1], &eq_sum);
      int take = (int)k - eq_ex;
      take = take < 0 ? 0 : (take > neq ? neq : take);
      if (c < chunk) sel_part += cabv[j] + cgt[c] + take;
      if (c == chunk) eq_before = eq_ex;
      eq_acc += eq_sum;
    }
    __shared__ int s_eqb;
    if (chunk % 256 == threadIdx.x) s_eqb = eq_before;
    sel_before = block_sum_int(sel_part, red[2]);
    eq_before = s_eqb;
  }
  uint32_t gtmask = 0, eqmask = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (e0 + j < st.n_vis) {
      const uint32_t key = order_key(sv[j]);
      gtmask |= (uint32_t)(key > T) << j;
      eqmask |= (uint32_t)(key == T) << j;
    }
  }
  const int eq_excl = eq_before + block_excl_scan(__popc(eqmask), red[3]);
  int can = (int)k - eq_excl;                 // equal keys this thread may still take
  uint32_t selmask = gtmask;
  for (int j = 0; j < 16 && can > 0; ++j)
    if (eqmask >> j & 1u) { selmask |= 1u << j; --can; }
  int pos = sel_before + block_excl_scan(__popc(selmask), red[0]);
  for (int j = 0; j < 16; ++j)
    if ((selmask >> j & 1u) && pos < a.top_k) out[pos++] = (int32_t)(e0 + j);
}

// Query blocks (many queries per call) replace select by two kernels, so
// the radix search over a query's candidates runs once per query instead of
// once per chunk workgroup:
//   threshold (one workgroup per query) finds the k-th key T among the
//             candidates of every chunk and, per chunk, where the chunk's
//             selection starts in the output and how many keys equal to T
//             come before it; the counts go back over chunk_cand /
//             chunk_above, T and the number of equal keys to take into the
//             query's state;
//   emit      (one workgroup per chunk and query) writes the chunk's indices.
// The result is the one select gives.
constexpr int kThrCache = 16;                  // candidates per thread held in registers
constexpr int kSplitSelectQueries = 64;        // queries per call from which threshold + emit replace select
constexpr int kFusedTopK = 2048;               // largest top_k the threshold pass emits itself (list mode)
__global__ void __launch_bounds__(256) topk_threshold_kernel(IndexLaunch a) {
  const int q = blockIdx.x;
  const TopkState st = a.state[q];
  int32_t* const out = a.out_idx + ((int64_t)(q / a.n_qb) * a.n_q + a.q_first + q % a.n_qb) * a.top_k;
  if (a.list_mode) {
    // this pass also writes the output: leave the histogram zeroed here
    uint32_t* gh = a.hist + (int64_t)q * kBins1;
    for (int i = threadIdx.x; i < kBins1; i += 256) gh[i] = 0;
  }
  if (st.k_rem < 0) {
    if (a.list_mode) {
      for (int i = threadIdx.x; i < a.top_k; i += 256) out[i] = i < st.n_vis ? i : -1;
    }
    return;
  }
  constexpr int kCPT = kMaxChunks / 256;
  const int n_act = (st.n_vis + kChunk - 1) / kChunk;
  __shared__ int pre[kMaxChunks + 1];
  __shared__ int cgt[kMaxChunks], ceq[kMaxChunks];
  __shared__ __attribute__((aligned(16))) uint32_t bins[2][1024];
  __shared__ uint32_t s_digit[2], s_kin[2];
  __shared__ int red[4][4];
  __shared__ int apre[kMaxChunks + 1];          // list mode: above-bucket indices before chunk c
  __shared__ uint32_t fa[kFusedTopK], fs[kFusedTopK];
  int* const ccnt_g = a.chunk_cand + (int64_t)q * a.n_chunks;
  int* const cabv_g = a.chunk_above + (int64_t)q * a.n_chunks;
  // chunk c's candidates are flat indices pre[c] .. pre[c+1]-1; thread t
  // holds chunks 4t .. 4t+3 for the scans
  int cnt[kCPT], abv[kCPT];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int c = kCPT * (int)threadIdx.x + j;
    cnt[j] = c < n_act ? ccnt_g[c] : 0;
    abv[j] = c < n_act ? cabv_g[c] : 0;
    mine += cnt[j];
  }
  int n_cand, n_ab;
  int run = block_excl_scan(mine, red[0], &n_cand);
  int arun = block_excl_scan(abv[0] + abv[1] + abv[2] + abv[3], red[1], &n_ab);
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int c = kCPT * (int)threadIdx.x + j;
    pre[c] = run;
    run += cnt[j];
    apre[c] = arun;
    arun += abv[j];
    cgt[c] = 0;
    ceq[c] = 0;
  }
  if (threadIdx.x == 0) { pre[kMaxChunks] = n_cand; apre[kMaxChunks] = n_ab; }
  for (int i = threadIdx.x; i < 2 * 1024; i += 256) (&bins[0][0])[i] = 0;
  if (threadIdx.x < 2) { s_digit[threadIdx.x] = 0; s_kin[threadIdx.x] = 0; }
  __syncthreads();
  const uint32_t* ck = a.cand_key + (int64_t)q * a.n_cap;
  // flat candidate i: its chunk (last c with pre[c] <= i) and key
  auto chunk_of = [&](int i) {
    int lo = 0, hi = n_act;                      // pre[lo] <= i < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
  };
  uint32_t key_c[kThrCache];
  int chk_c[kThrCache];
#pragma unroll
  for (int j = 0; j < kThrCache; ++j) {
    const int i = (int)threadIdx.x + 256 * j;
    chk_c[j] = i < n_cand ? chunk_of(i) : 0;
    key_c[j] = i < n_cand ? ck[(int64_t)chk_c[j] * kChunk + (i - pre[chk_c[j]])] : 0u;
  }
  auto for_each = [&](auto&& visit) {
#pragma unroll
    for (int j = 0; j < kThrCache; ++j)
      if ((int)threadIdx.x + 256 * j < n_cand) visit(key_c[j], chk_c[j]);
    for (int i = (int)threadIdx.x + 256 * kThrCache; i < n_cand; i += 256) {
      const int c = chunk_of(i);
      visit(ck[(int64_t)c * kChunk + (i - pre[c])], c);
    }
  };
  // radix select of the k_rem-th largest candidate: bits 19..10, then 9..0
  uint32_t prefix = st.b1 << kShift1, mask = 0xfff00000u;
  uint32_t k = (uint32_t)st.k_rem;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    uint32_t* const bp = bins[pass];
    const uint32_t mk = mask, px = prefix;
    for_each([bp, mk, px, shift](uint32_t key, int) {
      if ((key & mk) == px) atomicAdd(&bp[(key >> shift) & 1023u], 1u);
    });
    __syncthreads();
    uint32_t v[4];
    my_buckets(bins[pass], v);
    bucket_search(v, k, &s_digit[pass], &s_kin[pass]);
    prefix |= s_digit[pass] << shift;
    mask |= 1023u << shift;
    k = s_kin[pass];
    // BF16 scores: the bits of an order key below bit 16 are all zero (a
    // score >= 0, top key bit set) or all one (a negative score, whose key is
    // the complement of its bits), so bits 19..10 already fix the k-th key
    // (the last pass would put every candidate into one bin)
    if (bf16_scores(a)) {
      if ((prefix >> 31) == 0) prefix |= 1023u;
      break;
    }
  }
  const uint32_t T = prefix;
  for_each([T](uint32_t key, int c) {
    if (key > T) atomicAdd(&cgt[c], 1);
    else if (key == T) atomicAdd(&ceq[c], 1);
  });
  __syncthreads();
  // per chunk: keys equal to T before it, and the start of its selection
  int eq_mine = 0;
#pragma unroll
  for (int j = 0; j < kCPT; ++j) eq_mine += ceq[kCPT * (int)threadIdx.x + j];
  int eq_run = block_excl_scan(eq_mine, red[1]);
  int sel[kCPT], eqb[kCPT];
  int sel_mine = 0;
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int c = kCPT * (int)threadIdx.x + j;
    const int neq = c < n_act ? ceq[c] : 0;
    int take = (int)k - eq_run;
    take = take < 0 ? 0 : (take > neq ? neq : take);
    eqb[j] = eq_run;
    sel[j] = c < n_act ? abv[j] + cgt[c] + take : 0;
    sel_mine += sel[j];
    eq_run += neq;
  }
  int sel_run = block_excl_scan(sel_mine, red[2]);
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int c = kCPT * (int)threadIdx.x + j;
    if (c < n_act) {
      a.chunk_sel[(int64_t)q * a.n_chunks + c] = sel_run;
      a.chunk_eqb[(int64_t)q * a.n_chunks + c] = eqb[j];
    }
    sel_run += sel[j];
  }
  if (threadIdx.x == 0) {
    a.state[q].T = T;
    a.state[q].k_eq = (int32_t)k;
  }
  if (!a.list_mode) return;
  // List mode (collect left, in each chunk's score region, the indices above
  // the bucket and then the candidates' indices, both ascending): the
  // selection is the above-bucket indices of every chunk (fa) merged with the
  // candidates above T and the first k of those equal to T (fs), all in index
  // order; chunks are ascending index ranges, so flat order is index order.
  const uint32_t* const lst = (const uint32_t*)(score_row(a, q / a.n_qb, q % a.n_qb));
  const uint16_t* const lst16 = (const uint16_t*)lst;
  const bool b16 = bf16_scores(a);
  // entry `at` of chunk c's list: an index (fp32 scores) or an offset in the
  // chunk (BF16 scores)
  auto list_at = [&](int c, int at) -> uint32_t {
    const int64_t o = (int64_t)c * kChunk + at;
    return b16 ? (uint32_t)c * (uint32_t)kChunk + lst16[o] : lst[o];
  };
  auto chunk_in = [&](const int* pf, int i) {   // last c with pf[c] <= i
    int lo = 0, hi = n_act;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pf[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
  };
  int n_s = 0, eq_seen = 0;
  for (int j0 = 0; j0 < n_cand; j0 += 256) {
    const int i = j0 + (int)threadIdx.x;
    const bool live = i < n_cand;
    const int c = live ? chunk_of(i) : 0;
    const uint32_t key = live ? ck[(int64_t)c * kChunk + (i - pre[c])] : 0u;
    const bool gt = live && key > T, eq = live && key == T;
    int eq_tot, take_tot;
    const int er = eq_seen + block_excl_scan(eq ? 1 : 0, red[2], &eq_tot);
    const bool take = gt || (eq && er < (int)k);
    const int p = n_s + block_excl_scan(take ? 1 : 0, red[3], &take_tot);
    if (take && p < kFusedTopK) fs[p] = list_at(c, (apre[c + 1] - apre[c]) + (i - pre[c]));
    n_s += take_tot;
    eq_seen += eq_tot;
  }
  for (int i = threadIdx.x; i < n_ab && i < kFusedTopK; i += 256) {
    const int c = chunk_in(apre, i);
    fa[i] = list_at(c, i - apre[c]);
  }
  __syncthreads();
  auto below = [](const uint32_t* v, int n, uint32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (v[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  // output rank = rank in its own list + elements of the other list below it
  for (int i = threadIdx.x; i < n_ab; i += 256) {
    const int pos = i + below(fs, n_s, fa[i]);
    if (pos < a.top_k) out[pos] = (int32_t)fa[i];
  }
  for (int i = threadIdx.x; i < n_s; i += 256) {
    const int pos = i + below(fa, n_ab, fs[i]);
    if (pos < a.top_k) out[pos] = (int32_t)fs[i];
  }
}

// Emit from the scores: one workgroup per chunk (the caller's score array).
__global__ void __launch_bounds__(256) topk_emit_kernel(IndexLaunch a) {
  const int q = blockIdx.y;
  const int b = q / a.n_qb, r = q % a.n_qb;
  const int chunk = blockIdx.x;
  const int64_t c0 = (int64_t)chunk * kChunk;
  const TopkState st = a.state[q];
  {
    uint32_t* gh = a.hist + (int64_t)q * kBins1;
    for (int i = chunk * 256 + threadIdx.x; i < kBins1; i += a.n_chunks * 256) gh[i] = 0;
  }
  int32_t* out = a.out_idx + ((int64_t)b * a.n_q + a.q_first + r) * a.top_k;
  if (st.k_rem < 0) {
    for (int64_t i = c0 + threadIdx.x; i < c0 + kChunk && i < st.n_vis; i += 256) out[i] = (int32_t)i;
    if (chunk == 0)
      for (int i = st.n_vis + threadIdx.x; i < a.top_k; i += 256) out[i] = -1;
    return;
  }
  if (c0 >= st.n_vis) return;
  const int sel_before = a.chunk_sel[(int64_t)q * a.n_chunks + chunk];
  const int eq_before = a.chunk_eqb[(int64_t)q * a.n_chunks + chunk];
  const uint32_t T = st.T;
  const float* sc = score_row(a, q / a.n_qb, q % a.n_qb);
  const int64_t e0 = c0 + threadIdx.x * 16;
  float sv[16];
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    const int64_t i = e0 + j;
    if (i + 3 < a.n_cap) {
      load_score4(a, sc, i, sv + j);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) sv[j + u] = i + u < a.n_cap ? load_score(a, sc, i + u) : -INFINITY;
    }
  }
  __shared__ int red[2][4];
  uint32_t gtmask = 0, eqmask = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (e0 + j < st.n_vis) {
      const uint32_t key = order_key(sv[j]);
      gtmask |= (uint32_t)(key > T) << j;
      eqmask |= (uint32_t)(key == T) << j;
    }
  }
  const int eq_excl = eq_before + block_excl_scan(__popc(eqmask), red[1]);
  int can = st.k_eq - eq_excl;
  uint32_t selmask = gtmask;
  for (int j = 0; j < 16 && can > 0; ++j)
    if (eqmask >> j & 1u) { selmask |= 1u << j; --can; }
  int pos = sel_before + block_excl_scan(__popc(selmask), red[0]);
  for (int j = 0; j < 16; ++j)
    if ((selmask >> j & 1u) && pos < a.top_k) out[pos++] = (int32_t)(e0 + j);
}


hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s) {
  const int nq = a.B * a.n_qb;
  if (a.fmt == CSA_FMT_MXFP4 && a.n_qb >= kMqQT && a.H_I % 32 == 0 && !(a.flags & CSA_INDEX_BATCH_INVARIANT)) {
    index_linear_kernel<<<dim3(a.n_qb, a.B), 128, 0, s>>>(a);
    const int per_wg = 4 * kMqTiles * 32;
    dim3 grid((a.n_cap + per_wg - 1) / per_wg, (a.n_qb + kMqQT - 1) / kMqQT, a.B);
    // score dtype and paging are template arguments, so the tile loop has no branch
    const bool bf = (a.flags & CSA_INDEX_BF16_SCORES) != 0, pg = a.bt != nullptr;
    auto go = [&](auto nh) {
      constexpr int NH = decltype(nh)::value;
      auto* k = bf ? (pg ? index_mxfp4_mq_kernel<NH, true, true> : index_mxfp4_mq_kernel<NH, true, false>)
                   : (pg ? index_mxfp4_mq_kernel<NH, false, true> : index_mxfp4_mq_kernel<NH, false, false>);
      hipExtLaunchKernelGGL(k, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
    };
    if (a.H_I == 64) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 1>{});
  } else if (a.fmt == CSA_FMT_MXFP4) {
    const int kchunks = (a.n_cap + kKeysPerWG - 1) / kKeysPerWG;
    const int nhg = a.H_I / 16;
    auto go = [&](auto qt, auto hg) {
      constexpr int QT = decltype(qt)::value, HG = decltype(hg)::value;
      dim3 grid(kchunks, (a.n_qb + QT - 1) / QT, a.B);
      hipExtLaunchKernelGGL(index_mxfp4_kernel<QT, HG>, grid, dim3(256), 0, s, a.ev_start,
                            a.ev_stop, 0, a);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    if (a.n_qb >= 4) {
      if (nhg == 4) go(I4{}, I4{}); else if (nhg == 3) go(I4{}, I3{});
      else if (nhg == 2) go(I4{}, I2{}); else go(I4{}, I1{});
    } else {
      if (nhg == 4) go(I1{}, I4{}); else if (nhg == 3) go(I1{}, I3{});
      else if (nhg == 2) go(I1{}, I2{}); else go(I1{}, I1{});
    }
  } else {
    dim3 grid((a.n_cap + 255) / 256, a.n_qb, a.B);
    hipExtLaunchKernelGGL(index_f32_kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
  }
  dim3 g2(a.n_chunks, nq);
  IndexLaunch t = a;
  // with many queries and the scores in the workspace, collect leaves the
  // selected-index lists in place of the scores (16-bit offsets in the chunk
  // over BF16 scores) and the threshold pass writes the output from them (no
  // emit launch)
  t.list_mode = nq >= kSplitSelectQueries && !a.out_score && a.top_k <= kFusedTopK;
  if (t.list_mode) {
    topk_bucket_kernel<<<nq, 256, 0, s>>>(t);
    topk_collect_kernel<true><<<g2, 256, 0, s>>>(t);
  } else {
    topk_collect_kernel<false><<<g2, 256, 0, s>>>(t);
  }
  if (nq >= kSplitSelectQueries) {
    topk_threshold_kernel<<<nq, 256, 0, s>>>(t);
    if (!t.list_mode) topk_emit_kernel<<<g2, 256, 0, s>>>(t);
  } else {
    topk_select_kernel<<<g2, 256, 0, s>>>(t);
  }
  return hipGetLastError();
}

}  // namespace csa
