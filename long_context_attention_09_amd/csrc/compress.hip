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

template <typename T, int CPT>
__device__ __forceinline__ void load_row(const T* row, int c0, int d, float* v) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) v[k] = (c0 + k < d) ? load_elem<T>(row + c0 + k) : 0.0f;
}

template <typename T, int CPT>
__global__ void __launch_bounds__(256) compress_kernel(CompressLaunch a) {
  const int lane = threadIdx.x & 63;
  const int entry_local = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (entry_local >= a.n_entries) return;
  const int64_t i = a.i_first + entry_local;           // absolute entry index
  const int c0 = lane * CPT;
  const int d = a.d;
  const char* base_ka = (const char*)a.kv_a + (int64_t)b * a.in_seq_stride;
  const char* base_ga = a.gate_a ? (const char*)a.gate_a + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_kb = a.kv_b ? (const char*)a.kv_b + (int64_t)b * a.in_seq_stride : nullptr;
  const char* base_gb = a.gate_b ? (const char*)a.gate_b + (int64_t)b * a.in_seq_stride : nullptr;

  float mx[CPT], sm[CPT], acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { mx[k] = -INFINITY; sm[k] = 0.f; acc[k] = 0.f; }

  auto fold = [&](const char* kb, const char* gb, const float* bias, int64_t row) {
    float v[CPT], z[CPT];
    load_row<T, CPT>((const T*)(kb + row * a.in_row_stride), c0, d, v);
    if (gb) load_row<T, CPT>((const T*)(gb + row * a.in_row_stride), c0, d, z);
    else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) z[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float lg = z[k] + (bias && c0 + k < d ? bias[c0 + k] : 0.f);
      const float nm = fmaxf(mx[k], lg);
      const float r = expf(mx[k] - nm);       // 0 on the first candidate (mx = -inf)
      const float e = expf(lg - nm);
      sm[k] = sm[k] * r + e;
      acc[k] = acc[k] * r + e * v[k];
      mx[k] = nm;
    }
  };

  const int m = a.m;
  // a-branch: tokens m*i .. m*i+m-1, bias row = offset in the block
  for (int r = 0; r < m; ++r) {
    const int64_t row = m * i + r - a.pos0;
    fold(base_ka, base_ga, a.bias_a ? a.bias_a + (int64_t)r * d : nullptr, row);
  }
  // b-branch: tokens m*(i-1) .. m*i-1 (entry 0 has none)
  if (base_kb && i >= 1) {
    for (int r = 0; r < m; ++r) {
      const int64_t row = m * (i - 1) + r - a.pos0;
      fold(base_kb, base_gb, a.bias_b ? a.bias_b + (int64_t)r * d : nullptr, row);
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

template <typename T>
static hipError_t launch_t(const CompressLaunch& a, hipStream_t s) {
  int cpt = (a.d + 63) / 64;
  if (a.out_fmt == CSA_FMT_MXFP4 && cpt < 2) cpt = 2;  // a lane packs whole bytes
  dim3 grid((a.n_entries + 3) / 4, a.B);
  dim3 block(256);
  if (cpt <= 1) compress_kernel<T, 1><<<grid, block, 0, s>>>(a);
  else if (cpt <= 2) compress_kernel<T, 2><<<grid, block, 0, s>>>(a);
  else if (cpt <= 4) compress_kernel<T, 4><<<grid, block, 0, s>>>(a);
  else if (cpt <= 8) compress_kernel<T, 8><<<grid, block, 0, s>>>(a);
  else compress_kernel<T, 16><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressLaunch& a, hipStream_t s) {
  return a.in_dtype == CSA_DT_F32 ? launch_t<float>(a, s) : launch_t<uint16_t>(a, s);
}

}  // namespace csa
