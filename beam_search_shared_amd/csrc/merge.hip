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

  float m = -INFINITY;
  for (int part = 0; part < p.n_parts; ++part)
    m = fmaxf(m, p.lse_parts[part * p.lse_stride + rh]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float denom = 0.f;
    for (int part = 0; part < p.n_parts; ++part) {
      const float l = p.lse_parts[part * p.lse_stride + rh];
      const float w = fast_exp2((l - m) * kLog2e);  // exp(-inf) -> 0
      if (w == 0.f) continue;                          // an empty part adds nothing
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride +
                                                       rh * p.d + c * 4);
      acc += w * o;
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

hipError_t launch_merge(const MergeParams& p, int out_dtype, hipStream_t s) {
  const int64_t total = (int64_t)p.rows * p.heads * (p.d / 4);
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
