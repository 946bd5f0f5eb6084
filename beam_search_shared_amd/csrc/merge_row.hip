// One-row cached-prefix decode, second launch: the exact log-sum-exp merge of
// the cache chunks' partial states (PR #21738, "Add opt-in cascade attention
// for wide beam search on KVCM V2", Description: Solution, and the review
// thread on the FA4 split-generation kernels: split the keys, then merge the
// splits) folded with the call's own row (PR #2202, "perf(phi4_multimodal):
// prefill and decode over the cached prefix, not the whole KV allocation",
// Background: a decode step attends the valid cached rows plus its own row).
// The row is one more part: lse = scale * q . k_new, o = v_new. It is then
// written into its page, so the call needs no separate KV-write launch.
//
// One workgroup per (request, query head), as the many-part merge: the parts
// are spread over the threads for the max and the denominator, then over 8
// slices of 32 threads for the weighted sum (each slice covering head_dim in
// 4-element chunks and every eighth part), the slices summed through LDS. Up
// to 64 parts every global load is issued before any is used.
#include "device_common.h"
#include "merge_row.h"
#include "tile_index.h"

namespace bsp {

constexpr int kRowSlices = 8;
constexpr int kRowRegParts = 8;  // parts per slice held in registers (64 in all)

template <typename T>
__global__ __launch_bounds__(256) void merge_row_kernel(MergeRowParams p) {
  __shared__ float red_m[4], red_d[4];
  __shared__ float s_new_sh;
  __shared__ float w_s[kRowSlices * kRowRegParts];
  __shared__ float acc_s[kRowSlices][256];  // head_dim <= 256
  const int64_t rh = blockIdx.x;  // request * hq + head
  const int b = (int)(rh / p.hq);
  const int h = (int)(rh % p.hq);
  const int group = p.hq / p.hkv;
  const int g = h / group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slice = tid / 32;
  const int cl = tid % 32;
  const int chunks = p.d / 4;  // <= 64: two per lane of a slice at most
  const bool fast = p.n_parts <= kRowSlices * kRowRegParts;
  const float* lse_p = p.lse_parts + rh;
  const T* qrow = static_cast<const T*>(p.q) + rh * p.d;
  const int64_t nrow = (int64_t)b * p.new_stride + (int64_t)g * p.d;
  const T* krow = static_cast<const T*>(p.k_new) + nrow;
  const T* vrow = static_cast<const T*>(p.v_new) + nrow;

  // ---- loads: the parts' lse, the slice's output chunks, the row's q, k and v
  const float my_lse = fast && tid < p.n_parts ? lse_p[tid * p.lse_stride] : -INFINITY;
  f32x4 o[2][kRowRegParts];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = cl + 32 * cc;
#pragma unroll
    for (int k = 0; k < kRowRegParts; ++k) {
      const int part = slice + kRowSlices * k;
      o[cc][k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (fast && c < chunks && part < p.n_parts)
        o[cc][k] = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride + rh * p.d + c * 4);
    }
  }
  float dot = 0.f;
  if (wave == 0)
    for (int i = lane; i < p.d; i += 64)
      dot = fmaf(Traits<T>::to_f(qrow[i]), Traits<T>::to_f(krow[i]), dot);
  // the row's write into its page, once per (request, KV head) by the group's
  // first head: its slot and 16-byte chunks are loaded with everything else
  const bool writer = h % group == 0 && tid < p.d / 8;
  int32_t slot = -1;
  u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
  if (writer) {
    slot = p.slots[b];
    kw = *reinterpret_cast<const u32x4*>(krow + tid * 8);
    vw = *reinterpret_cast<const u32x4*>(vrow + tid * 8);
  }
  u32x2 vv[2] = {u32x2{0u, 0u}, u32x2{0u, 0u}};  // slice 0: the row's value, 4 columns a chunk
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = cl + 32 * cc;
    if (slice == 0 && c < chunks) vv[cc] = *reinterpret_cast<const u32x2*>(vrow + c * 4);
  }

  // ---- the maximum over the parts and the row's score
  float m = my_lse;
  if (!fast)
    for (int part = tid; part < p.n_parts; part += 256) m = fmaxf(m, lse_p[part * p.lse_stride]);
  m = wave_max(m);
  if (wave == 0) dot = wave_sum(dot);
  if (lane == 0) red_m[wave] = m;
  if (tid == 0) s_new_sh = dot * p.scale;
  __syncthreads();
  const float s_new = s_new_sh;
  const float M = fmaxf(fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3])), s_new);

  // ---- weights and the denominator (an empty part, lse -inf, weighs 0)
  float dl = 0.f;
  if (fast) {
    const float wt = tid < p.n_parts ? fast_exp2((my_lse - M) * kLog2e) : 0.f;
    if (tid < kRowSlices * kRowRegParts) w_s[tid] = wt;
    dl = wt;
  } else {
    for (int part = tid; part < p.n_parts; part += 256)
      dl += fast_exp2((lse_p[part * p.lse_stride] - M) * kLog2e);
  }
  dl = wave_sum(dl);
  if (lane == 0) red_d[wave] = dl;
  __syncthreads();
  const float w_new = fast_exp2((s_new - M) * kLog2e);
  const float den = ((red_d[0] + red_d[1]) + (red_d[2] + red_d[3])) + w_new;

  // ---- weighted sums per slice; slice 0 adds the row's value
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = cl + 32 * cc;
    if (c >= chunks) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (fast) {
#pragma unroll
      for (int k = 0; k < kRowRegParts; ++k) {
        const int part = slice + kRowSlices * k;
        const float w = part < p.n_parts ? w_s[part] : 0.f;
        // an empty part adds nothing, whatever its o holds (a select, not w * o)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? fmaf(w, o[cc][k][e], acc[e]) : acc[e];
      }
    } else {
#pragma unroll 4
      for (int part = slice; part < p.n_parts; part += kRowSlices) {
        const float w = fast_exp2((lse_p[part * p.lse_stride] - M) * kLog2e);
        const f32x4 op = *reinterpret_cast<const f32x4*>(p.o_parts + part * p.o_stride + rh * p.d + c * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w > 0.f ? fmaf(w, op[e], acc[e]) : acc[e];
      }
    }
    if (slice == 0) {
      const T* ve = reinterpret_cast<const T*>(&vv[cc]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w_new, Traits<T>::to_f(ve[e]), acc[e]);
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
    for (int sl = 0; sl < kRowSlices; ++sl) v += acc_s[sl][i];
    out[i] = Traits<T>::from_f(v * inv);
  }
  if (p.lse_out != nullptr && tid == 0) p.lse_out[rh] = M + __logf(den);

  // ---- the row into its page (a slot outside the pool is skipped and recorded)
  if (writer) {
    if (slot < 0 || (int64_t)slot >= ((int64_t)p.num_pages << p.page_shift)) {
      if (tid == 0)
        record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value, kErrWriteSlot, slot);
    } else {
      const int64_t dst = pool_row(slot >> p.page_shift, p.hkv, g, p.page_shift,
                                   slot & ((1 << p.page_shift) - 1), p.d) + tid * 8;
      *reinterpret_cast<u32x4*>(static_cast<T*>(p.k_pool) + dst) = kw;
      *reinterpret_cast<u32x4*>(static_cast<T*>(p.v_pool) + dst) = vw;
    }
  }
}

hipError_t launch_merge_row(const MergeRowParams& p, int dtype, hipStream_t s) {
  const int64_t pairs = (int64_t)p.rows * p.hq;
  if (pairs == 0) return hipSuccess;
  if (dtype == BSP_F16)
    merge_row_kernel<_Float16><<<(unsigned)pairs, 256, 0, s>>>(p);
  else
    merge_row_kernel<__bf16><<<(unsigned)pairs, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsp
