// Compressor: softmax-gated, position-biased pooling of m tokens into one entry,
// then RMSNorm, partial RoPE and storage (FP8/BF16, MXFP4 or fp32).
//
// The pooling is the compression equation of "DeepSeek-V4 深读"
// (ricardokevins.github.io), section "CSA：4× 压缩之后再 top-k": per channel, a
// softmax over the candidates' gate logits plus a learned position bias, then
// a weighted sum; CSA adds the previous block through its b-branch, HCA
// ("HCA：128× 压缩后保留 dense 全局视野") has one branch.
//
// One wavefront owns one entry; each lane owns CPT consecutive channels, so a
// row of d channels is one coalesced read of d * sizeof(elem) bytes per wave.
// The candidates are folded into a running (max, sum, weighted sum) per
// channel, so every raw row is read exactly once.  HBM-bound.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// CPT consecutive channels of one row starting at channel c0 (0 beyond d).
// VEC: the row and every lane's slice are aligned to the slice size and d is
// a multiple of CPT (d % 8 == 0, CPT <= 8), so a lane's slice is either wholly
// inside the row or wholly past it; it is fetched with the widest loads and no
// branch (a lane past the row re-reads channel 0 and zeroes it).
template <typename T, int CPT, bool VEC>
__device__ __forceinline__ void load_row(const T* row, int c0, int d, float* v) {
  constexpr int kBytes = CPT * (int)sizeof(T);
  if constexpr (VEC && kBytes >= 4 && CPT <= 8) {
    const bool in = c0 < d;
    constexpr int kWords = kBytes / 4;
    uint32_t w[kWords];
    const char* src = (const char*)(row + (in ? c0 : 0));
    if constexpr (kWords % 4 == 0) {
#pragma unroll
      for (int k = 0; k < kWords; k += 4) {
        const u32x4 x = *(const u32x4*)(src + 4 * k);
        w[k] = x[0]; w[k + 1] = x[1]; w[k + 2] = x[2]; w[k + 3] = x[3];
      }
    } else if constexpr (kWords == 2) {
      const u32x2 x = *(const u32x2*)src;
      w[0] = x[0]; w[1] = x[1];
    } else {
#pragma unroll
      for (int k = 0; k < kWords; ++k) w[k] = ((const uint32_t*)src)[k];
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float x;
      if constexpr (sizeof(T) == 2) x = bf16_to_f32((uint16_t)((w[k >> 1] >> (16 * (k & 1))) & 0xffffu));
      else x = __uint_as_float(w[k]);
      v[k] = in ? x : 0.0f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = (c0 + k < d) ? load_elem<T>(row + c0 + k) : 0.0f;
  }
}

// Raw 32-bit words of a lane's slice (the VEC case of load_row, split in two so
// a batch of candidates can have all its loads in flight before any is used).
template <int KW>
__device__ __forceinline__ void raw_words(const char* src, uint32_t (&w)[KW]) {
  if constexpr (KW % 4 == 0) {
#pragma unroll
    for (int k = 0; k < KW; k += 4) {
      const u32x4 x = *(const u32x4*)(src + 4 * k);
      w[k] = x[0]; w[k + 1] = x[1]; w[k + 2] = x[2]; w[k + 3] = x[3];
    }
  } else if constexpr (KW == 2) {
    const u32x2 x = *(const u32x2*)src;
    w[0] = x[0]; w[1] = x[1];
  } else {
#pragma unroll
    for (int k = 0; k < KW; ++k) w[k] = ((const uint32_t*)src)[k];
  }
}

template <typename T, int CPT, int KW>
__device__ __forceinline__ void unpack_words(const uint32_t (&w)[KW], bool in, float* v) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    float x;
    if constexpr (sizeof(T) == 2) x = bf16_to_f32((uint16_t)((w[k >> 1] >> (16 * (k & 1))) & 0xffffu));
    else x = __uint_as_float(w[k]);
    v[k] = in ? x : 0.0f;
  }
}

// WIDE: one 512-thread workgroup per entry, its eight wavefronts fold
// interleaved candidates and merge their running (max, sum, weighted sum)
// through LDS (the 128-token HCA blocks); otherwise one wavefront per entry
// (in a wide launch too, for the jobs of short blocks, eight to a workgroup).
// blockIdx.z selects one of up to kMaxJobs independent jobs of one launch.
// Merge another running (max, sum, weighted sum) state into this one, channel
// by channel, without branches: where both maxima are -inf the scale factors
// are exp2(-inf) = 0 and the state stays empty.
template <int CPT>
__device__ __forceinline__ void merge_state(float (&mx)[CPT], float (&sm)[CPT], float (&acc)[CPT],
                                            const float* om, const float* os, const float* oa) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const float nm = fmaxf(mx[k], om[k]);
    const float base = nm == -INFINITY ? 0.f : nm;
    const float r0 = fast_exp2(mx[k] - base), r1 = fast_exp2(om[k] - base);
    sm[k] = sm[k] * r0 + os[k] * r1;
    acc[k] = acc[k] * r0 + oa[k] * r1;
    mx[k] = nm;
  }
}

// Cross-wave state exchange through LDS: wave w > 0 stores its state at slot
// w - 1 of red ([slots][3][64 * CPT], 16-byte aligned) with 16-byte stores.
template <int CPT>
__device__ __forceinline__ void put_state(float* red, int slot, int c0, const float* mx, const float* sm,
                                          const float* acc) {
  float* r = red + slot * 3 * 64 * CPT + c0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) { r[k] = mx[k]; r[64 * CPT + k] = sm[k]; r[128 * CPT + k] = acc[k]; }
}

template <int CPT>
__device__ __forceinline__ void get_state(const float* red, int slot, int c0, float* om, float* os, float* oa) {
  const float* r = red + slot * 3 * 64 * CPT + c0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) { om[k] = r[k]; os[k] = r[64 * CPT + k]; oa[k] = r[128 * CPT + k]; }
}

// This lane's CPT channels of a pooled candidate group [3][d] (max, sum,
// weighted sum): 16-byte loads when the lane's slice lies inside the row.
template <int CPT>
__device__ __forceinline__ void part_state(const float* q, int c0, int d, float* pm, float* ps, float* pa) {
  if constexpr (CPT % 4 == 0) {
    if (c0 + CPT <= d) {
      uint32_t wm[CPT], ws[CPT], wa[CPT];
      raw_words<CPT>((const char*)(q + c0), wm);
      raw_words<CPT>((const char*)(q + d + c0), ws);
      raw_words<CPT>((const char*)(q + 2 * d + c0), wa);
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        pm[k] = __uint_as_float(wm[k]);
        ps[k] = __uint_as_float(ws[k]);
        pa[k] = __uint_as_float(wa[k]);
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const bool ok = c0 + k < d;
    pm[k] = ok ? q[c0 + k] : -INFINITY;
    ps[k] = ok ? q[d + c0 + k] : 0.f;
    pa[k] = ok ? q[2 * d + c0 + k] : 0.f;
  }
}

// Fold candidates c_first, c_first + c_step, ... (below c_end) of entry i of
// sequence b into the running per-channel (max, sum, weighted sum) of this
// lane's CPT channels; softmax in base 2.  Candidate c < m is token m*i + c of
// the a-branch (bias row c); m <= c < 2m is token m*(i-1) + c - m of the
// b-branch (bias row c - m).
template <typename T, int CPT, bool VEC, int kBatch>
__device__ __forceinline__ void fold_candidates(const CompressLaunch& a, int b, int64_t i, int lane, int c_first,
                                                int c_step, int c_end, float (&mx)[CPT], float (&sm)[CPT],
                                                float (&acc)[CPT]) {
  const int c0 = lane * CPT;
  const int d = a.d;
  const int m = a.m;
  const char* base_ka = (const char*)a.kv_a + (int64_t)b * a.in_seq_stride;
  const char* base_ga = a.gate_a ? (const char*)a.gate_a + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_kb = a.kv_b ? (const char*)a.kv_b + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_gb = a.gate_b ? (const char*)a.gate_b + (int64_t)b * a.in_seq_stride : nullptr;
  const float* bias_a = a.bias_a;
  const float* bias_b = a.bias_b;
  // Branch-free batches: a dead slot re-reads candidate 0 and gets logit -inf.
  for (int cb = c_first; cb < c_end; cb += kBatch * c_step) {
    constexpr bool kSplitLoads = VEC && CPT * (int)sizeof(T) >= 4 && CPT <= 8;
    if constexpr (kSplitLoads) {
      // Every load of the batch is issued before any is used (kv rows, then
      // under uniform branches the gate and bias rows); the fold below then
      // reads each channel straight from the raw words.
      constexpr int KW = CPT * (int)sizeof(T) / 4, KWB = CPT;
      const bool in = c0 < d;
      const int coff = in ? c0 : 0;
      uint32_t wk[kBatch][KW], wg[kBatch][KW], wb[kBatch][KWB];
      bool live[kBatch], g_ok[kBatch], b_ok[kBatch];
      const char* gp[kBatch];
      const float* bp[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        int c = cb + u * c_step;
        live[u] = c < c_end;
        c = live[u] ? c : 0;
        const bool a_side = c < m;
        const int64_t row = compress_in_row(a, a_side ? m * i + c - a.pos0 : m * (i - 1) + (c - m) - a.pos0);
        const char* kp = (a_side ? base_ka : base_kb) + row * a.in_row_stride + (int64_t)coff * (int64_t)sizeof(T);
        const char* g = a_side ? base_ga : base_gb;
        g_ok[u] = in && g != nullptr;
        gp[u] = g ? g + row * a.in_row_stride + (int64_t)coff * (int64_t)sizeof(T) : kp;
        const float* bb = a_side ? bias_a : bias_b;
        b_ok[u] = in && bb != nullptr;
        bp[u] = bb ? bb + (int64_t)(a_side ? c : c - m) * d + coff : bias_a + coff;
        raw_words<KW>(kp, wk[u]);
      }
      if (base_ga) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) raw_words<KW>(gp[u], wg[u]);
      }
      if (bias_a) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) raw_words<KWB>((const char*)bp[u], wb[u]);
      }
      auto word_f = [&](const uint32_t* w, int k) -> float {
        if constexpr (sizeof(T) == 2) return bf16_to_f32((uint16_t)((w[k >> 1] >> (16 * (k & 1))) & 0xffffu));
        else return __uint_as_float(w[k]);
      };
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float lg[kBatch];
        float bm = mx[k];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float zz = (base_ga && g_ok[u]) ? word_f(wg[u], k) : 0.f;
          const float bz = (bias_a && b_ok[u]) ? __uint_as_float(wb[u][k]) : 0.f;
          lg[u] = live[u] ? (zz + bz) * kLog2e : -INFINITY;
          bm = fmaxf(bm, lg[u]);
        }
        const float base = bm == -INFINITY ? 0.f : bm;
        const float r = fast_exp2(mx[k] - base);       // 0 while nothing was folded
        float sum = sm[k] * r, num = acc[k] * r;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float e = fast_exp2(lg[u] - base);
          const float vv = in ? word_f(wk[u], k) : 0.f;
          sum += e;
          num = fmaf(e, vv, num);
        }
        sm[k] = sum;
        acc[k] = num;
        mx[k] = bm;
      }
    } else {
    float v[kBatch][CPT], z[kBatch][CPT], bias[kBatch][CPT];
    bool live[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int c = cb + u * c_step;
      live[u] = c < c_end;
      c = live[u] ? c : 0;
      const bool a_side = c < m;
      const int64_t row = compress_in_row(a, a_side ? m * i + c - a.pos0 : m * (i - 1) + (c - m) - a.pos0);
      const char* kbase = a_side ? base_ka : base_kb;
      const char* gbase = a_side ? base_ga : base_gb;
      const float* bb = a_side ? a.bias_a : a.bias_b;
      const int brow = a_side ? c : c - m;
      load_row<T, CPT, VEC>((const T*)(kbase + row * a.in_row_stride), c0, d, v[u]);
      if (gbase) {
        load_row<T, CPT, VEC>((const T*)(gbase + row * a.in_row_stride), c0, d, z[u]);
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) z[u][k] = 0.f;
      }
      if (bb) {
        load_row<float, CPT, VEC>(bb + (int64_t)brow * d, c0, d, bias[u]);
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) bias[u][k] = 0.f;
      }
    }
    // Softmax in base 2, folded one batch at a time: the batch's largest
    // logit per channel is found first, so the running state is rescaled once
    // per batch and every candidate costs one exp2.  Dead slots have logit
    // -inf and weight exp2(-inf) = 0.
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float lg[kBatch];
      float bm = mx[k];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        lg[u] = live[u] ? (z[u][k] + bias[u][k]) * kLog2e : -INFINITY;
        bm = fmaxf(bm, lg[u]);
      }
      const float base = bm == -INFINITY ? 0.f : bm;
      const float r = fast_exp2(mx[k] - base);       // 0 while nothing was folded
      float sum = sm[k] * r, num = acc[k] * r;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float e = fast_exp2(lg[u] - base);
        sum += e;
        num = fmaf(e, v[u][k], num);
      }
      sm[k] = sum;
      acc[k] = num;
      mx[k] = bm;
    }
    }
  }
}

template <typename T, int CPT, bool WIDE, bool VEC>
__global__ void __launch_bounds__(WIDE ? 512 : 256, WIDE ? 1 : 2) compress_kernel(CompressBatch batch) {
  const CompressLaunch& a = batch.job[blockIdx.z];
  constexpr int kWaves = WIDE ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // a job of short blocks (m < 16) takes one entry per wave, also when a
  // long-block job of the same batch makes the launch wide (the raw window
  // rows of a prefill chunk beside its long blocks); uniform per workgroup
  const bool per_wave = !WIDE || a.m < 16;
  const int entry_local = per_wave ? (int)blockIdx.x * kWaves + wave : (int)blockIdx.x;
  const int b = blockIdx.y;
  if (b >= a.B || entry_local >= a.n_entries) return;
  const int64_t i = compress_entry(a, b, entry_local);  // absolute entry index
  if (i < 0) return;
  const int c0 = lane * CPT;
  const int d = a.d;
  const int m = a.m;
  // entry 0 has no b-branch
  const int n_cand = (a.kv_b && i >= 1) ? 2 * m : m;

  float mx[CPT], sm[CPT], acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { mx[k] = -INFINITY; sm[k] = 0.f; acc[k] = 0.f; }

  if (a.part) {
    // candidates pooled in n_parts groups by compress_part_kernel: wave w
    // merges the groups' (max, sum, weighted sum) states w, w + kWaves, ...
    const float* pp = a.part + ((int64_t)b * a.n_entries + entry_local) * a.n_parts * 3 * d;
    const int g_first = per_wave ? 0 : wave, g_step = per_wave ? 1 : kWaves;
    for (int g = g_first; g < a.n_parts; g += g_step) {
      const float* q = pp + (int64_t)g * 3 * d;
      float pm[CPT], ps[CPT], pa[CPT];
      part_state<CPT>(q, c0, d, pm, ps, pa);
      merge_state<CPT>(mx, sm, acc, pm, ps, pa);
    }
  } else {
    constexpr int kBatch = CPT >= 16 ? 4 : 8;   // candidates whose loads are in flight together
    fold_candidates<T, CPT, VEC, kBatch>(a, b, i, lane, per_wave ? 0 : wave, per_wave ? 1 : kWaves, n_cand, mx, sm,
                                         acc);
  }
  if (WIDE && !per_wave) {
    // tree merge, 8 -> 4 -> 2 -> 1 waves; each level has its own LDS slots
    // (4 + 2 + 1), so one barrier per level
    __shared__ __attribute__((aligned(16))) float red[(kWaves - 1) * 3 * 64 * CPT];
    int slot0 = 0;
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half >>= 1) {
      if (wave >= half && wave < 2 * half) put_state<CPT>(red, slot0 + wave - half, c0, mx, sm, acc);
      __syncthreads();
      if (wave < half) {
        float om[CPT], os[CPT], oa[CPT];
        get_state<CPT>(red, slot0 + wave, c0, om, os, oa);
        merge_state<CPT>(mx, sm, acc, om, os, oa);
      }
      slot0 += half;
    }
    if (wave > 0) return;
  }
  float x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = (c0 + k < d) ? acc[k] / sm[k] : 0.f;

  if (a.do_norm) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) ss += x[k] * x[k];
    ss = wave_sum_dpp(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + a.rms_eps);
#pragma unroll
    for (int k = 0; k < CPT; ++k) x[k] *= r;
  }

  const int d0 = d - a.d_rope;                          // first rotated channel
  if (a.d_rope > 0) {
    const double pos = (double)m * (double)i;
    if constexpr (CPT % 2 == 0) {
      const int n_pairs = a.d_rope >> 1;
      if (n_pairs <= 64) {
        // lane u forms the angle of pair u once; lanes holding rotated
        // channels fetch their pairs' cos / sin from those lanes
        float cs_l = 1.f, sn_l = 0.f;
        if (lane < n_pairs) rope_cos_sin(pos, lane, a.d_rope, a.log_theta, &cs_l, &sn_l);
#pragma unroll
        for (int k = 0; k < CPT; k += 2) {
          const int c = c0 + k;
          const int u = (c - d0) >> 1;
          const int src = (c >= d0 && c < d) ? u : 0;
          const float cs = __shfl(cs_l, src, 64), sn = __shfl(sn_l, src, 64);
          if (c >= d0 && c < d) {
            const float xe = x[k], xo = x[k + 1];
            x[k] = xe * cs - xo * sn;
            x[k + 1] = xe * sn + xo * cs;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < CPT; k += 2) {
          const int c = c0 + k;
          if (c >= d0 && c < d) {
            float cs, sn;
            rope_cos_sin(pos, (c - d0) >> 1, a.d_rope, a.log_theta, &cs, &sn);
            const float xe = x[k], xo = x[k + 1];
            x[k] = xe * cs - xo * sn;
            x[k + 1] = xe * sn + xo * cs;
          }
        }
      }
    } else {
      // one channel per lane: the pair partner sits in the neighbouring lane
      const float other = __shfl_xor(x[0], 1, 64);
      const int c = c0;
      if (c >= d0 && c < d) {
        float cs, sn;
        rope_cos_sin(pos, (c - d0) >> 1, a.d_rope, a.log_theta, &cs, &sn);
        x[0] = (c & 1) == 0 ? x[0] * cs - other * sn : other * sn + x[0] * cs;
      }
    }
  }

  const int64_t off0 = compress_out_off(a, b, i, a.out0_stride, a.out0_seq_stride);
  const int64_t off1 = compress_out_off(a, b, i, a.out1_stride, a.out1_seq_stride);
  if (off0 < 0) return;                                // unallocated block
  if (a.out_fmt == CSA_FMT_F32) {
    float* o = (float*)((char*)a.out0 + off0);
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (c0 + k < d) o[c0 + k] = x[k];
  } else if (a.out_fmt == CSA_FMT_FP8_BF16) {
    uint8_t* on = (uint8_t*)a.out0 + off0;
    uint16_t* orr = (uint16_t*)((char*)a.out1 + off1);
    if constexpr (CPT == 8) {
      // a lane's 8 channels are all FP8 or all BF16 when d - d_rope is a
      // multiple of 8: one 8-byte or 16-byte store where aligned
      if (c0 + CPT <= d0 && ((uintptr_t)(on + c0) & 7) == 0) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < CPT; ++k) w[k >> 2] |= f32_to_e4m3(x[k]) << (8 * (k & 3));
        *(u32x2*)(on + c0) = (u32x2){w[0], w[1]};
        return;
      }
      if (c0 >= d0 && c0 + CPT <= d && ((uintptr_t)(orr + (c0 - d0)) & 15) == 0) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (uint32_t)f32_to_bf16(x[2 * k]) | ((uint32_t)f32_to_bf16(x[2 * k + 1]) << 16);
        *(u32x4*)(orr + (c0 - d0)) = w;
        return;
      }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = c0 + k;
      if (c < d0) on[c] = (uint8_t)f32_to_e4m3(x[k]);
      else if (c < d) orr[c - d0] = f32_to_bf16(x[k]);
    }
  } else {  // MXFP4: CPT is even, 32 / CPT lanes share one block
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) amax = fmaxf(amax, fabsf(x[k]));
    for (int o = 1; o < 32 / CPT; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const int E = mx_block_exponent(amax);
    uint8_t* oc = (uint8_t*)a.out0 + off0;
    uint8_t* os = (uint8_t*)a.out1 + off1;
    if (c0 < d) {
#pragma unroll
      for (int k = 0; k < CPT; k += 2) {
        const uint32_t lo = e2m1_code(ldexpf(x[k], -E));
        const uint32_t hi = e2m1_code(ldexpf(x[k + 1], -E));
        oc[(c0 + k) >> 1] = (uint8_t)(lo | (hi << 4));
      }
      if ((c0 & 31) == 0) os[c0 >> 5] = (uint8_t)(E + 127);
    }
  }
}

// Long blocks (m >= 16) over many workgroups: workgroup (entry, group) folds
// the kPartCands candidates kPartCands*group .. of one entry over its four
// wavefronts, merges them through LDS and writes the group's per-channel
// (max, sum, weighted sum) to a.part; compress_kernel then merges the groups
// and finishes the entry.  Jobs without a.part are skipped.
template <typename T, int CPT, bool VEC>
__global__ void __launch_bounds__(256, 2) compress_part_kernel(CompressBatch batch) {
  const CompressLaunch& a = batch.job[blockIdx.z];
  if (!a.part) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.x / a.n_parts, g = blockIdx.x % a.n_parts;
  const int b = blockIdx.y;
  if (b >= a.B || e >= a.n_entries) return;
  const int64_t i = compress_entry(a, b, e);
  if (i < 0) return;
  const int n_cand = (a.kv_b && i >= 1) ? 2 * a.m : a.m;
  const int c_lo = g * kPartCands;
  const int c_end = c_lo + kPartCands < n_cand ? c_lo + kPartCands : n_cand;
  float mx[CPT], sm[CPT], acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { mx[k] = -INFINITY; sm[k] = 0.f; acc[k] = 0.f; }
  fold_candidates<T, CPT, VEC, kPartCands / 4>(a, b, i, lane, c_lo + wave, 4, c_end, mx, sm, acc);
  __shared__ __attribute__((aligned(16))) float red[3 * 3 * 64 * CPT];   // waves 1..3
  const int c0 = lane * CPT;
  if (wave > 0) put_state<CPT>(red, wave - 1, c0, mx, sm, acc);
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    float om[CPT], os[CPT], oa[CPT];
    get_state<CPT>(red, w, c0, om, os, oa);
    merge_state<CPT>(mx, sm, acc, om, os, oa);
  }
  const int d = a.d;
  float* q = a.part + (((int64_t)b * a.n_entries + e) * a.n_parts + g) * 3 * d;
  if (CPT % 4 == 0 && c0 + CPT <= d) {
#pragma unroll
    for (int k = 0; k < CPT; k += 4) {
      *(f32x4*)(q + c0 + k) = (f32x4){mx[k], mx[k + 1], mx[k + 2], mx[k + 3]};
      *(f32x4*)(q + d + c0 + k) = (f32x4){sm[k], sm[k + 1], sm[k + 2], sm[k + 3]};
      *(f32x4*)(q + 2 * d + c0 + k) = (f32x4){acc[k], acc[k + 1], acc[k + 2], acc[k + 3]};
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (c0 + k < d) {
        q[c0 + k] = mx[k];
        q[d + c0 + k] = sm[k];
        q[2 * d + c0 + k] = acc[k];
      }
    }
  }
}

template <typename T, int CPT, bool VEC>
static void launch_cpt(const CompressBatch& bt, int B, bool wide, hipStream_t s) {
  int n_part_wg = 0;
  for (int j = 0; j < bt.n_jobs; ++j)
    if (bt.job[j].part && bt.job[j].n_entries * bt.job[j].n_parts > n_part_wg)
      n_part_wg = bt.job[j].n_entries * bt.job[j].n_parts;
  if (n_part_wg > 0) compress_part_kernel<T, CPT, VEC><<<dim3(n_part_wg, B, bt.n_jobs), 256, 0, s>>>(bt);
  // workgroups per job: wide launches take a long-block entry per workgroup
  // and eight short-block entries (one per wave); narrow ones four entries
  int gx = 1;
  for (int j = 0; j < bt.n_jobs; ++j) {
    const CompressLaunch& a = bt.job[j];
    const int n = wide ? (a.m >= 16 ? a.n_entries : (a.n_entries + 7) / 8) : (a.n_entries + 3) / 4;
    gx = n > gx ? n : gx;
  }
  if (wide) {
    compress_kernel<T, CPT, true, VEC><<<dim3(gx, B, bt.n_jobs), 512, 0, s>>>(bt);
  } else {
    compress_kernel<T, CPT, false, VEC><<<dim3(gx, B, bt.n_jobs), 256, 0, s>>>(bt);
  }
}

// Every input slice a lane reads starts on a multiple of its size (capped at 16 B).
template <typename T, int CPT>
static bool vec_ok(const CompressLaunch& a) {
  const uint64_t al = CPT * sizeof(T) < 16 ? CPT * sizeof(T) : 16;
  const uint64_t alb = CPT * 4 < 16 ? CPT * 4 : 16;
  auto ok = [](const void* p, uint64_t n) { return p == nullptr || ((uint64_t)p % n) == 0; };
  return ok(a.kv_a, al) && ok(a.gate_a, al) && ok(a.kv_b, al) && ok(a.gate_b, al) &&
         (uint64_t)a.in_row_stride % al == 0 && (uint64_t)a.in_seq_stride % al == 0 &&
         ok(a.bias_a, alb) && ok(a.bias_b, alb) && ((uint64_t)a.d * 4) % alb == 0;
}

template <typename T, int CPT>
static void launch_cpt(const CompressBatch& bt, int B, bool wide, hipStream_t s) {
  bool vec = true;
  for (int j = 0; j < bt.n_jobs; ++j) vec = vec && vec_ok<T, CPT>(bt.job[j]);
  if (vec) launch_cpt<T, CPT, true>(bt, B, wide, s);
  else launch_cpt<T, CPT, false>(bt, B, wide, s);
}

template <typename T>
static hipError_t launch_t(const CompressBatch& bt, hipStream_t s) {
  int cpt = 1, B = 1;
  bool wide = false;
  for (int j = 0; j < bt.n_jobs; ++j) {
    const CompressLaunch& a = bt.job[j];
    int c = (a.d + 63) / 64;
    if (a.out_fmt == CSA_FMT_MXFP4 && c < 2) c = 2;  // a lane packs whole bytes
    cpt = c > cpt ? c : cpt;
    B = a.B > B ? a.B : B;
    wide = wide || a.m >= 16;
  }
  if (cpt <= 1) launch_cpt<T, 1>(bt, B, wide, s);
  else if (cpt <= 2) launch_cpt<T, 2>(bt, B, wide, s);
  else if (cpt <= 4) launch_cpt<T, 4>(bt, B, wide, s);
  else if (cpt <= 8) launch_cpt<T, 8>(bt, B, wide, s);
  else launch_cpt<T, 16>(bt, B, wide, s);
  return hipGetLastError();
}

// All jobs of a batch share the input dtype (the host splits batches that do not).
hipError_t launch_compress(const CompressBatch& bt, hipStream_t s) {
  return bt.job[0].in_dtype == CSA_DT_F32 ? launch_t<float>(bt, s) : launch_t<uint16_t>(bt, s);
}

}  // namespace csa
