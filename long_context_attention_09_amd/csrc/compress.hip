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

// WIDE: one 512-thread workgroup per entry, its eight wavefronts fold
// interleaved candidates and merge their running (max, sum, weighted sum)
// through LDS (the 128-token HCA blocks); otherwise one wavefront per entry.
// blockIdx.z selects one of up to kMaxJobs independent jobs of one launch.
template <typename T, int CPT, bool WIDE, bool VEC>
__global__ void __launch_bounds__(WIDE ? 512 : 256) compress_kernel(CompressBatch batch) {
  const CompressLaunch& a = batch.job[blockIdx.z];
  constexpr int kWaves = WIDE ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int entry_local = WIDE ? (int)blockIdx.x : (int)blockIdx.x * 4 + wave;
  const int b = blockIdx.y;
  if (b >= a.B || entry_local >= a.n_entries) return;
  const int64_t i = a.i_first + entry_local;           // absolute entry index
  const int c0 = lane * CPT;
  const int d = a.d;
  const int m = a.m;
  const char* base_ka = (const char*)a.kv_a + (int64_t)b * a.in_seq_stride;
  const char* base_ga = a.gate_a ? (const char*)a.gate_a + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_kb = a.kv_b ? (const char*)a.kv_b + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_gb = a.gate_b ? (const char*)a.gate_b + (int64_t)b * a.in_seq_stride : nullptr;
  // candidates: c < m is token m*i + c of the a-branch (bias row c); m <= c < 2m
  // is token m*(i-1) + c - m of the b-branch (bias row c - m); entry 0 has no b-branch
  const int n_cand = (base_kb && i >= 1) ? 2 * m : m;

  float mx[CPT], sm[CPT], acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { mx[k] = -INFINITY; sm[k] = 0.f; acc[k] = 0.f; }

  const int c_first = WIDE ? wave : 0;
  const int c_step = WIDE ? kWaves : 1;
  constexpr int kBatch = CPT >= 16 ? 4 : 8;   // candidates whose loads are in flight together
  // Branch-free batches: a dead slot re-reads candidate 0 and gets logit -inf.
  for (int cb = c_first; cb < n_cand; cb += kBatch * c_step) {
    float v[kBatch][CPT], z[kBatch][CPT], bias[kBatch][CPT];
    bool live[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int c = cb + u * c_step;
      live[u] = c < n_cand;
      c = live[u] ? c : 0;
      const bool a_side = c < m;
      const int64_t row = a_side ? m * i + c - a.pos0 : m * (i - 1) + (c - m) - a.pos0;
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
  if constexpr (WIDE) {
    __shared__ float red[kWaves - 1][3][64 * CPT];  // waves 1..: max, sum, weighted sum
    if (wave > 0) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        red[wave - 1][0][c0 + k] = mx[k];
        red[wave - 1][1][c0 + k] = sm[k];
        red[wave - 1][2][c0 + k] = acc[k];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const float om = red[w][0][c0 + k];
        const float nm = fmaxf(mx[k], om);
        if (nm == -INFINITY) continue;
        const float r0 = fast_exp2(mx[k] - nm), r1 = fast_exp2(om - nm);
        sm[k] = sm[k] * r0 + red[w][1][c0 + k] * r1;
        acc[k] = acc[k] * r0 + red[w][2][c0 + k] * r1;
        mx[k] = nm;
      }
  }
  float x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = (c0 + k < d) ? acc[k] / sm[k] : 0.f;

  if (a.do_norm) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) ss += x[k] * x[k];
    ss = wave_sum(ss);
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

  if (a.out_fmt == CSA_FMT_F32) {
    float* o = (float*)((char*)a.out0 + (int64_t)b * a.out0_seq_stride + (i - a.out_row0) * a.out0_stride);
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (c0 + k < d) o[c0 + k] = x[k];
  } else if (a.out_fmt == CSA_FMT_FP8_BF16) {
    uint8_t* on = (uint8_t*)a.out0 + (int64_t)b * a.out0_seq_stride + (i - a.out_row0) * a.out0_stride;
    uint16_t* orr = (uint16_t*)((char*)a.out1 + (int64_t)b * a.out1_seq_stride + (i - a.out_row0) * a.out1_stride);
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
    uint8_t* oc = (uint8_t*)a.out0 + (int64_t)b * a.out0_seq_stride + (i - a.out_row0) * a.out0_stride;
    uint8_t* os = (uint8_t*)a.out1 + (int64_t)b * a.out1_seq_stride + (i - a.out_row0) * a.out1_stride;
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

template <typename T, int CPT, bool VEC>
static void launch_cpt(const CompressBatch& bt, int B, int n_entries, bool wide, hipStream_t s) {
  if (wide) {
    compress_kernel<T, CPT, true, VEC><<<dim3(n_entries, B, bt.n_jobs), 512, 0, s>>>(bt);
  } else {
    compress_kernel<T, CPT, false, VEC><<<dim3((n_entries + 3) / 4, B, bt.n_jobs), 256, 0, s>>>(bt);
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
static void launch_cpt(const CompressBatch& bt, int B, int n_entries, bool wide, hipStream_t s) {
  bool vec = true;
  for (int j = 0; j < bt.n_jobs; ++j) vec = vec && vec_ok<T, CPT>(bt.job[j]);
  if (vec) launch_cpt<T, CPT, true>(bt, B, n_entries, wide, s);
  else launch_cpt<T, CPT, false>(bt, B, n_entries, wide, s);
}

template <typename T>
static hipError_t launch_t(const CompressBatch& bt, hipStream_t s) {
  int cpt = 1, B = 1, n_entries = 1;
  bool wide = false;
  for (int j = 0; j < bt.n_jobs; ++j) {
    const CompressLaunch& a = bt.job[j];
    int c = (a.d + 63) / 64;
    if (a.out_fmt == CSA_FMT_MXFP4 && c < 2) c = 2;  // a lane packs whole bytes
    cpt = c > cpt ? c : cpt;
    B = a.B > B ? a.B : B;
    n_entries = a.n_entries > n_entries ? a.n_entries : n_entries;
    wide = wide || a.m >= 16;
  }
  if (cpt <= 1) launch_cpt<T, 1>(bt, B, n_entries, wide, s);
  else if (cpt <= 2) launch_cpt<T, 2>(bt, B, n_entries, wide, s);
  else if (cpt <= 4) launch_cpt<T, 4>(bt, B, n_entries, wide, s);
  else if (cpt <= 8) launch_cpt<T, 8>(bt, B, n_entries, wide, s);
  else launch_cpt<T, 16>(bt, B, n_entries, wide, s);
  return hipGetLastError();
}

// All jobs of a batch share the input dtype (the host splits batches that do not).
hipError_t launch_compress(const CompressBatch& bt, hipStream_t s) {
  return bt.job[0].in_dtype == CSA_DT_F32 ? launch_t<float>(bt, s) : launch_t<uint16_t>(bt, s);
}

}  // namespace csa
