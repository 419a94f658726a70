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
// 4 accumulator rows a lane holds, and two cross-lane adds finish the head
// sum.  The kernel also builds the histogram of the top 11 bits of every
// score's order key for the first radix-select pass.
//
// Top-k: a three-pass radix select on the 32-bit order key (11 + 11 + 10 bits),
// each pass a multi-workgroup histogram of the still-undecided bucket followed
// by a one-workgroup bucket search; then a count pass and a write pass that
// emit the selected indices in ascending order.  Elements equal to the k-th
// key are taken lowest index first.  Histograms use integer atomics only, so
// the result is deterministic.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kTilesPerWave = 16;                    // 16 keys per tile
constexpr int kKeysPerWG = 4 * kTilesPerWave * 16;   // 1024
constexpr int kChunk = 4096;                         // scores per workgroup in the radix passes
constexpr int kBins1 = 2048;

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

// ------------------------------------------------------------------ MXFP4 indexer

template <int QT>
__global__ void __launch_bounds__(256) index_mxfp4_kernel(IndexLaunch a) {
  __shared__ uint32_t lhist[QT][kBins1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;       // k-group of the operand / row group of the result
  const int col = lane & 15;
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * QT;
  const int nhg = a.H_I >> 4;    // head groups of 16

  for (int i = threadIdx.x; i < QT * kBins1; i += 256) (&lhist[0][0])[i] = 0;

  int nvis[QT];
  int nvis_max = 0;
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    nvis[qi] = (r0 + qi < a.n_qb) ? query_n_vis(a, b, r0 + qi) : 0;
    nvis_max = nvis[qi] > nvis_max ? nvis[qi] : nvis_max;
  }
  __syncthreads();

  const int64_t key_base = (int64_t)blockIdx.x * kKeysPerWG + wave * (kTilesPerWave * 16);
  const uint8_t* kc = (const uint8_t*)a.k0 + (int64_t)b * a.n_cap * 64;
  const uint32_t* ks = (const uint32_t*)a.k1 + (int64_t)b * a.n_cap;

  if (key_base < nvis_max) {
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
    // issue every tile's loads first (16 B of codes + the scale word per lane and
    // tile), so a wave keeps 4 KiB of keys in flight, then score them
    i32x4 kbuf[kTilesPerWave];
    uint32_t kscw[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int64_t key = key_base + t * 16 + col;
      kbuf[t] = (i32x4){0, 0, 0, 0};
      kscw[t] = 0x7f7f7f7fu;
      if (key < nvis_max && key < a.n_cap) {
        kbuf[t] = *(const i32x4*)(kc + key * 64 + g * 16);
        kscw[t] = ks[key];
      }
    }
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int64_t key0 = key_base + t * 16;
      if (key0 >= nvis_max) break;
      const int64_t key = key0 + col;
      const bool in_cap = key < a.n_cap;
      const i32x8 kb = {kbuf[t][0], kbuf[t][1], kbuf[t][2], kbuf[t][3], 0, 0, 0, 0};
      const int ksc = (int)((kscw[t] >> (8 * g)) & 0xffu);
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        float part = 0.f;
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) {
          if (hg < nhg) {
            i32x8 qv = {qa[qi][hg][0], qa[qi][hg][1], qa[qi][hg][2], qa[qi][hg][3], 0, 0, 0, 0};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qv, kb, acc, 4, 4, 0, qs[qi][hg],
                                                                   0, ksc);
#pragma unroll
            for (int i = 0; i < 4; ++i) part += wv[qi][hg][i] * fmaxf(acc[i], 0.f);
          }
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if (g == 0 && r0 + qi < a.n_qb && in_cap) {
          const bool vis = key < nvis[qi];
          const float s = vis ? part : -INFINITY;
          a.scores[((int64_t)b * a.n_qb + r0 + qi) * a.n_cap + key] = s;
          if (vis) atomicAdd(&lhist[qi][order_key(s) >> 21], 1u);
        }
      }
    }
  }
  // keys in tiles past every query's visible range still get -inf
  {
    const int64_t wave_end = key_base + kTilesPerWave * 16;
    int64_t start = key_base;
    if (nvis_max > key_base) start = key_base + (((int64_t)nvis_max - key_base + 15) / 16) * 16;
    for (int qi = 0; qi < QT; ++qi) {
      if (r0 + qi >= a.n_qb) break;
      float* row = a.scores + ((int64_t)b * a.n_qb + r0 + qi) * a.n_cap;
      for (int64_t k = start + lane; k < wave_end && k < a.n_cap; k += 64) row[k] = -INFINITY;
    }
  }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < QT; ++qi)
    if (r0 + qi < a.n_qb) flush_hist(lhist[qi], a.hist + ((int64_t)b * a.n_qb + r0 + qi) * kBins1, kBins1);
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
      const float* k = (const float*)a.k0 + ((int64_t)b * a.n_cap + key) * a.d_I;
      s = 0.f;
      for (int h = 0; h < a.H_I; ++h) {
        const float* q = (const float*)a.q0 + (qrow + h) * a.d_I;
        float dot = 0.f;
        for (int c = 0; c < a.d_I; ++c) dot = fmaf(q[c], k[c], dot);
        s += a.w[qrow + h] * fmaxf(dot, 0.f);
      }
      atomicAdd(&lhist[order_key(s) >> 21], 1u);
    }
    a.scores[((int64_t)b * a.n_qb + r) * a.n_cap + key] = s;
  }
  __syncthreads();
  flush_hist(lhist, a.hist + ((int64_t)b * a.n_qb + r) * kBins1, kBins1);
}

// ------------------------------------------------------------------ radix select

// Bucket search over one histogram: pass 0 (bits 31..21), 1 (20..10), 2 (9..0).
// Pass 0 also initialises the state.  Clears the histogram for the next pass.
__global__ void __launch_bounds__(256) topk_select_kernel(IndexLaunch a, int pass) {
  const int q = blockIdx.x;                      // b * n_qb + r
  const int b = q / a.n_qb, r = q % a.n_qb;
  TopkState* st = a.state + q;
  uint32_t* hist = a.hist + (int64_t)q * kBins1;
  __shared__ uint32_t tot[256];
  __shared__ TopkState s0;
  if (threadIdx.x == 0) {
    if (pass == 0) {
      s0.prefix = 0; s0.mask = 0;
      s0.n_vis = query_n_vis(a, b, r);
      s0.k_rem = s0.n_vis <= a.top_k ? -1 : a.top_k;   // -1: every visible entry is taken
    } else {
      s0 = *st;
    }
  }
  __syncthreads();
  const int bins = pass == 2 ? 1024 : 2048;
  const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  const int per = bins / 256;                    // bins per thread, top bins first
  const int hi = bins - per * threadIdx.x;       // thread t owns bins [hi - per, hi)
  uint32_t cnt[8];
  uint32_t my = 0;
  for (int j = 0; j < per; ++j) { cnt[j] = hist[hi - 1 - j]; my += cnt[j]; }
  tot[threadIdx.x] = my;
  __syncthreads();
  // inclusive scan over threads (thread 0 = highest bins)
  for (int o = 1; o < 256; o <<= 1) {
    uint32_t v = threadIdx.x >= o ? tot[threadIdx.x - o] : 0;
    __syncthreads();
    tot[threadIdx.x] += v;
    __syncthreads();
  }
  const int k_rem = s0.k_rem;
  __shared__ TopkState ns;
  if (threadIdx.x == 0) ns = s0;
  __syncthreads();
  if (k_rem > 0) {
    const uint32_t before = threadIdx.x ? tot[threadIdx.x - 1] : 0;
    if (before < (uint32_t)k_rem && (uint32_t)k_rem <= before + my) {
      uint32_t acc = before;
      for (int j = 0; j < per; ++j) {
        if ((uint32_t)k_rem <= acc + cnt[j]) {
          const uint32_t digit = (uint32_t)(hi - 1 - j);
          ns.prefix = s0.prefix | (digit << shift);
          ns.mask = s0.mask | ((uint32_t)(bins - 1) << shift);
          ns.k_rem = k_rem - (int)acc;
          break;
        }
        acc += cnt[j];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *st = ns;
  __syncthreads();
  for (int j = threadIdx.x; j < kBins1; j += 256) hist[j] = 0;
}

// Histogram of the next digit among the elements inside the current bucket.
__global__ void __launch_bounds__(256) topk_hist_kernel(IndexLaunch a, int pass) {
  __shared__ uint32_t lh[kBins1];
  const int q = blockIdx.y;
  const TopkState st = a.state[q];
  if (st.k_rem <= 0) return;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (c0 >= st.n_vis) return;
  for (int i = threadIdx.x; i < kBins1; i += 256) lh[i] = 0;
  __syncthreads();
  const int shift = pass == 1 ? 10 : 0;
  const uint32_t dmask = pass == 1 ? 2047u : 1023u;
  const float* sc = a.scores + (int64_t)q * a.n_cap;
  const int64_t end = c0 + kChunk < st.n_vis ? c0 + kChunk : st.n_vis;
  for (int64_t i = c0 + threadIdx.x; i < end; i += 256) {
    const uint32_t k = order_key(sc[i]);
    if ((k & st.mask) == st.prefix) atomicAdd(&lh[(k >> shift) & dmask], 1u);
  }
  __syncthreads();
  flush_hist(lh, a.hist + (int64_t)q * kBins1, pass == 1 ? 2048 : 1024);
}

// Per chunk: how many visible elements beat the k-th key, and how many equal it.
__global__ void __launch_bounds__(256) topk_count_kernel(IndexLaunch a) {
  const int q = blockIdx.y;
  const TopkState st = a.state[q];
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  int gt = 0, eq = 0;
  if (st.k_rem > 0 && c0 < st.n_vis) {
    const float* sc = a.scores + (int64_t)q * a.n_cap;
    const int64_t end = c0 + kChunk < st.n_vis ? c0 + kChunk : st.n_vis;
    for (int64_t i = c0 + threadIdx.x; i < end; i += 256) {
      const uint32_t k = order_key(sc[i]);
      gt += k > st.prefix;
      eq += k == st.prefix;
    }
  }
  __shared__ int sgt[4], seq[4];
  for (int o = 32; o >= 1; o >>= 1) { gt += __shfl_xor(gt, o, 64); eq += __shfl_xor(eq, o, 64); }
  if ((threadIdx.x & 63) == 0) { sgt[threadIdx.x >> 6] = gt; seq[threadIdx.x >> 6] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int* c = a.counts + ((int64_t)q * a.n_chunks + blockIdx.x) * 2;
    c[0] = sgt[0] + sgt[1] + sgt[2] + sgt[3];
    c[1] = seq[0] + seq[1] + seq[2] + seq[3];
  }
}

// Emit the selected indices of one chunk at their rank among all selected
// indices (ascending index order), and the -1 padding.
__global__ void __launch_bounds__(256) topk_write_kernel(IndexLaunch a) {
  const int q = blockIdx.y;
  const int b = q / a.n_qb, r = q % a.n_qb;
  const TopkState st = a.state[q];
  int32_t* out = a.out_idx + ((int64_t)b * a.n_q + a.q_first + r) * a.top_k;
  const int chunk = blockIdx.x;
  const int64_t c0 = (int64_t)chunk * kChunk;
  const bool all = st.k_rem < 0;
  if (all) {
    // every visible entry, in order; chunk 0 also writes the padding
    for (int64_t i = c0 + threadIdx.x; i < c0 + kChunk && i < st.n_vis; i += 256) out[i] = (int32_t)i;
    if (chunk == 0)
      for (int i = st.n_vis + threadIdx.x; i < a.top_k; i += 256) out[i] = -1;
    return;
  }
  if (c0 >= st.n_vis) return;
  // selected before this chunk
  __shared__ int s_red[2][4];
  int sel_before = 0, eq_before = 0;
  {
    // pass over previous chunks: eq_before is a prefix sum, so do it serially
    // per 64-chunk window with a wave scan
    const int* cnt = a.counts + (int64_t)q * a.n_chunks * 2;
    int acc_sel = 0, acc_eq = 0;
    if (threadIdx.x < 64) {
      for (int base = 0; base < chunk; base += 64) {
        const int c = base + threadIdx.x;
        const int ngt = c < chunk ? cnt[2 * c] : 0;
        const int neq = c < chunk ? cnt[2 * c + 1] : 0;
        // exclusive scan of neq within the wave
        int incl = neq;
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(incl, o, 64);
          if ((int)threadIdx.x >= o) incl += v;
        }
        const int excl = incl - neq + acc_eq;
        int take = st.k_rem - excl;
        take = take < 0 ? 0 : (take > neq ? neq : take);
        int s = ngt + take;
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
        acc_sel += s;
        acc_eq += __shfl(incl, 63, 64);
      }
      if (threadIdx.x == 0) { s_red[0][0] = acc_sel; s_red[1][0] = acc_eq; }
    }
    __syncthreads();
    sel_before = s_red[0][0];
    eq_before = s_red[1][0];
  }
  // each thread owns 16 consecutive elements of the chunk
  const float* sc = a.scores + (int64_t)q * a.n_cap;
  const int64_t e0 = c0 + threadIdx.x * 16;
  uint32_t gtmask = 0, eqmask = 0;
  for (int j = 0; j < 16; ++j) {
    const int64_t i = e0 + j;
    if (i < st.n_vis) {
      const uint32_t k = order_key(sc[i]);
      gtmask |= (uint32_t)(k > st.prefix) << j;
      eqmask |= (uint32_t)(k == st.prefix) << j;
    }
  }
  // block exclusive scans of the eq counts, then of the selected counts
  __shared__ int wsum[4];
  auto block_excl_scan = [&](int v) -> int {
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
    return off + incl - v;
  };
  const int eq_excl = eq_before + block_excl_scan(__popc(eqmask));
  // take the first (k_rem - eq_excl) equal elements of this thread
  int can = st.k_rem - eq_excl;
  uint32_t selmask = gtmask;
  for (int j = 0; j < 16 && can > 0; ++j)
    if (eqmask >> j & 1u) { selmask |= 1u << j; --can; }
  int pos = sel_before + block_excl_scan(__popc(selmask));
  for (int j = 0; j < 16; ++j)
    if ((selmask >> j & 1u) && pos < a.top_k) out[pos++] = (int32_t)(e0 + j);
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s) {
  const int nq = a.B * a.n_qb;
  {
    const int64_t n = (int64_t)nq * kBins1;
    int blocks = (int)((n + 255) / 256);
    blocks = blocks > 4096 ? 4096 : blocks;
    zero_u32_kernel<<<blocks, 256, 0, s>>>(a.hist, n);
  }
  if (a.fmt == CSA_FMT_MXFP4) {
    const int kchunks = (a.n_cap + kKeysPerWG - 1) / kKeysPerWG;
    if (a.n_qb >= 4) {
      dim3 grid(kchunks, (a.n_qb + 3) / 4, a.B);
      hipExtLaunchKernelGGL(index_mxfp4_kernel<4>, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
    } else {
      dim3 grid(kchunks, a.n_qb, a.B);
      hipExtLaunchKernelGGL(index_mxfp4_kernel<1>, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
    }
  } else {
    dim3 grid((a.n_cap + 255) / 256, a.n_qb, a.B);
    hipExtLaunchKernelGGL(index_f32_kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, a);
  }
  dim3 g2(a.n_chunks, nq);
  topk_select_kernel<<<nq, 256, 0, s>>>(a, 0);
  topk_hist_kernel<<<g2, 256, 0, s>>>(a, 1);
  topk_select_kernel<<<nq, 256, 0, s>>>(a, 1);
  topk_hist_kernel<<<g2, 256, 0, s>>>(a, 2);
  topk_select_kernel<<<nq, 256, 0, s>>>(a, 2);
  topk_count_kernel<<<g2, 256, 0, s>>>(a);
  topk_write_kernel<<<g2, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace csa
