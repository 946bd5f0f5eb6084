// Exact n-way merge of partial attention states over disjoint key sets:
// lse = ln sum_p exp(lse_p), o = sum_p exp(lse_p - lse) * o_p (TensorRT-LLM
// PR #21738, "Add opt-in cascade attention for wide beam search on KVCM V2",
// Description: Solution, merged exactly with the log-sum-exp).
//
// One thread produces 4 consecutive output elements of one (row, head); the
// lse values of the parts are read by every thread of the head (cached).
#include "bsp_internal.h"
#include "device_common.h"

namespace bsp {

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int chunks = p.d / 4;
  const int64_t total = (int64_t)p.rows * p.heads * chunks;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % chunks);
  const int64_t rh = idx / chunks;  // row * heads + head

  // Both passes are unrolled so that a group's loads are in flight together:
  // with many parts and few rows (a split one-row decode) each dependent load
  // would otherwise cost a full memory round trip.
  float m = -INFINITY;
#pragma unroll 8
  for (int part = 0; part < p.n_parts; ++part)
    m = fmaxf(m, p.lse_parts[part * p.lse_stride + rh]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float denom = 0.f;
#pragma unroll 8
    for (int part = 0; part < p.n_parts; ++part) {
      const float l = p.lse_parts[part * p.lse_stride + rh];
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride +
                                                       rh * p.d + c * 4);
      const float w = fast_exp2((l - m) * kLog2e);  // exp(-inf) -> 0
      // an empty part adds nothing, whatever its o holds (a select, not w * o)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? fmaf(w, o[e], acc[e]) : acc[e];
      denom += w;
    }
    acc *= 1.f / denom;
    lse = m + __logf(denom);
  }
  T* out = static_cast<T*>(p.o_out) + rh * p.d + c * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = Traits<T>::from_f(acc[e]);
  if (p.lse_out != nullptr && c == 0) p.lse_out[rh] = lse;
}

// Few (row, head) pairs and many parts (a one-row decode split into dozens of
// key chunks): one workgroup per (row, head). The parts are spread over the
// threads for the max and the denominator (block reductions), then over 8
// slices of 32 threads for the weighted sum, each slice covering head_dim in
// 4-element chunks and every eighth part; the slices are summed through LDS.
// Up to 64 parts, every global load (one lse per thread, the slice's o chunks)
// is issued before any is used: one memory round trip, the rest in registers
// and LDS. More parts take the looping form.
constexpr int kMergeSlices = 8;
constexpr int kMergeRegParts = 8;  // parts per slice held in registers
template <typename T>
__global__ __launch_bounds__(256) void merge_wide_kernel(MergeParams p) {
  __shared__ float red[4];
  __shared__ float w_s[kMergeSlices * kMergeRegParts];
  __shared__ float acc_s[kMergeSlices][256];  // head_dim <= 256
  const int64_t rh = blockIdx.x;  // row * heads + head
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const float* lse_p = p.lse_parts + rh;

  if (p.n_parts <= kMergeSlices * kMergeRegParts) {
    const int slice = tid / 32;
    const int cl = tid % 32;
    const int chunks = p.d / 4;  // <= 64: two per lane of a slice at most
    const float my_lse = tid < p.n_parts ? lse_p[tid * p.lse_stride] : -INFINITY;
    f32x4 o[2][kMergeRegParts];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = cl + 32 * cc;
#pragma unroll
      for (int k = 0; k < kMergeRegParts; ++k) {
        const int part = slice + kMergeSlices * k;
        o[cc][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c < chunks && part < p.n_parts)
          o[cc][k] = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride + rh * p.d + c * 4);
      }
    }
    float m = wave_max(my_lse);
    if ((tid & 63) == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    if (m == -INFINITY) {  // every part empty
      T* out = static_cast<T*>(p.o_out) + rh * p.d;
      for (int i = tid; i < p.d; i += 256) out[i] = Traits<T>::from_f(0.f);
      if (p.lse_out != nullptr && tid == 0) p.lse_out[rh] = -INFINITY;
      return;
    }
    const float wt = tid < p.n_parts ? fast_exp2((my_lse - m) * kLog2e) : 0.f;  // exp(-inf) -> 0
    if (tid < kMergeSlices * kMergeRegParts) w_s[tid] = wt;
    const float dsum = wave_sum(wt);
    if ((tid & 63) == 0) red[wave] = dsum;
    __syncthreads();
    const float den = (red[0] + red[1]) + (red[2] + red[3]);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = cl + 32 * cc;
      if (c >= chunks) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kMergeRegParts; ++k) {
        const int part = slice + kMergeSlices * k;
        const float w = part < p.n_parts ? w_s[part] : 0.f;
        // an empty part adds nothing, whatever its o holds (a select, not w * o)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? fmaf(w, o[cc][k][e], acc[e]) : acc[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc_s[slice][c * 4 + e] = acc[e];
    }
    __syncthreads();
    const float inv = 1.f / den;
    T* out = static_cast<T*>(p.o_out) + rh * p.d;
    for (int i = tid; i < p.d; i += 256) {
      float v = 0.f;
#pragma unroll
      for (int sl = 0; sl < kMergeSlices; ++sl) v += acc_s[sl][i];
      out[i] = Traits<T>::from_f(v * inv);
    }
    if (p.lse_out != nullptr && tid == 0) p.lse_out[rh] = m + __logf(den);
    return;
  }

  float m = -INFINITY;
  for (int part = tid; part < p.n_parts; part += 256) m = fmaxf(m, lse_p[part * p.lse_stride]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  if (m == -INFINITY) {  // every part empty
    T* out = static_cast<T*>(p.o_out) + rh * p.d;
    for (int i = tid; i < p.d; i += 256) out[i] = Traits<T>::from_f(0.f);
    if (p.lse_out != nullptr && tid == 0) p.lse_out[rh] = -INFINITY;
    return;
  }
  float den = 0.f;
  for (int part = tid; part < p.n_parts; part += 256)
    den += fast_exp2((lse_p[part * p.lse_stride] - m) * kLog2e);
  den = wave_sum(den);
  if ((tid & 63) == 0) red[wave] = den;
  __syncthreads();
  den = (red[0] + red[1]) + (red[2] + red[3]);

  const int slice = tid / 32;
  const int cl = tid % 32;
  const int chunks = p.d / 4;
  for (int c = cl; c < chunks; c += 32) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int part = slice; part < p.n_parts; part += kMergeSlices) {
      const float w = fast_exp2((lse_p[part * p.lse_stride] - m) * kLog2e);
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride + rh * p.d + c * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? fmaf(w, o[e], acc[e]) : acc[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc_s[slice][c * 4 + e] = acc[e];
  }
  __syncthreads();
  const float inv = 1.f / den;
  T* out = static_cast<T*>(p.o_out) + rh * p.d;
  for (int i = tid; i < p.d; i += 256) {
    float v = 0.f;
#pragma unroll
    for (int sl = 0; sl < kMergeSlices; ++sl) v += acc_s[sl][i];
    out[i] = Traits<T>::from_f(v * inv);
  }
  if (p.lse_out != nullptr && tid == 0) p.lse_out[rh] = m + __logf(den);
}

hipError_t launch_merge(const MergeParams& p, int out_dtype, hipStream_t s) {
  const int64_t pairs = (int64_t)p.rows * p.heads;
  if (pairs == 0) return hipSuccess;
  if (pairs <= 4096 && p.n_parts > kMergeSlices && p.d <= 256) {
    const unsigned blocks = (unsigned)pairs;
    if (out_dtype == BSP_F32)
      merge_wide_kernel<float><<<blocks, 256, 0, s>>>(p);
    else if (out_dtype == BSP_F16)
      merge_wide_kernel<_Float16><<<blocks, 256, 0, s>>>(p);
    else
      merge_wide_kernel<__bf16><<<blocks, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  const int64_t total = pairs * (p.d / 4);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (out_dtype == BSP_F32)
    merge_kernel<float><<<blocks, 256, 0, s>>>(p);
  else if (out_dtype == BSP_F16)
    merge_kernel<_Float16><<<blocks, 256, 0, s>>>(p);
  else
    merge_kernel<__bf16><<<blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsp
