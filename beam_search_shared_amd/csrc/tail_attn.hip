// Per-beam tail attention through cache_indirection.
//
// Each beam's generated positions P_b <= j < S_b are read from the beam that
// cache_indirection names for that position (TensorRT-LLM PR #21738, "Add
// opt-in cascade attention for wide beam search on KVCM V2", Description:
// Solution, and the fused-tail commit message). The tail is short (a few
// positions), so this is a gather: one wave handles one (request, beam, KV
// head); its 64 lanes split head_dim, every tail row is one contiguous
// head_dim-long read of the page, and the dot products are summed with DPP
// row reductions plus four lane reads. The wave loops over the G query heads
// of its KV head; the rows it re-reads for the next head come from L1.
#include "bsp_internal.h"
#include "device_common.h"

namespace bsp {

template <typename T, int EPL>
struct alignas(sizeof(T) * EPL) VecT {
  T v[EPL];
};

template <typename T, int EPL>
__device__ __forceinline__ void load_row(const T* ptr, float (&out)[EPL]) {
  const VecT<T, EPL> x = *reinterpret_cast<const VecT<T, EPL>*>(ptr);
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = Traits<T>::to_f(x.v[e]);
}

// Resolve tail position t of beam bk (= b * W + k) to a flat slot, or -1 for a
// bad parent or page (recorded in the error word).
__device__ __forceinline__ int32_t resolve_tail_slot(const TailParams& p, int b, int bk,
                                                     int P, int t) {
  const int j = P + t;
  const int32_t src = p.ci[(int64_t)bk * p.max_seq_len + j];
  if (src < 0 || src >= p.W) {
    record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value, kErrTailParent,
                 src);
    return -1;
  }
  const int blk = j >> p.page_shift;
  const int32_t page = p.block_tables[((int64_t)b * p.W + src) * p.max_blocks + blk];
  if (page < 0 || page >= p.num_pages) {
    record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value, kErrTailPage,
                 page);
    return -1;
  }
  return (page << p.page_shift) + (j & ((1 << p.page_shift) - 1));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void tail_kernel(TailParams p) {
  constexpr int EPL = D / 64;
  constexpr int CHUNK = 8;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.B * p.W * p.hkv) return;  // the whole wave leaves together
  const int g = item % p.hkv;
  const int bk = item / p.hkv;
  const int b = bk / p.W;
  const ReqInfo ri = p.req[b];
  const int n_tail = ri.tail;
  const int P = ri.prefix;
  const int ps = 1 << p.page_shift;
  const T* kp = static_cast<const T*>(p.k_pool);
  const T* vp = static_cast<const T*>(p.v_pool);

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = g * p.group + hh;
    float q[EPL];
    load_row<T, EPL>(static_cast<const T*>(p.q) + ((int64_t)bk * p.hq + h) * D + lane * EPL, q);
    float m = -INFINITY, l = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    for (int t0 = 0; t0 < n_tail; t0 += CHUNK) {
      float kr[CHUNK][EPL], vr[CHUNK][EPL];
      int32_t slot[CHUNK];
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        slot[c] = (t0 + c < n_tail) ? resolve_tail_slot(p, b, bk, P, t0 + c) : -1;
        if (slot[c] >= 0) {
          const int page = slot[c] >> p.page_shift;
          const int row = slot[c] & (ps - 1);
          const int64_t off = (((int64_t)page * p.hkv + g) * ps + row) * D + lane * EPL;
          load_row<T, EPL>(kp + off, kr[c]);
          load_row<T, EPL>(vp + off, vr[c]);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) kr[c][e] = vr[c][e] = 0.f;
        }
      }
      float s[CHUNK];
      float cmax = -INFINITY;
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(q[e], kr[c][e], part);
        s[c] = slot[c] >= 0 ? wave_sum(part) * p.scale_log2e : -INFINITY;
        cmax = fmaxf(cmax, s[c]);
      }
      const float m_new = fmaxf(m, cmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int c = 0; c < CHUNK; ++c) {
        const float pc = fast_exp2(s[c] - m_use);
        l += pc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pc, vr[c][e], acc[e]);
      }
      m = m_new;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* o = p.o_tail + ((int64_t)bk * p.hq + h) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
    if (lane == 0)
      p.lse_tail[(int64_t)bk * p.hq + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// Debug: resolved slot of every (request, beam, tail position), -1 past the tail.
__global__ __launch_bounds__(256) void tail_slots_kernel(TailParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.W * p.tail_pad;
  if (idx >= total) return;
  const int t = (int)(idx % p.tail_pad);
  const int bk = (int)(idx / p.tail_pad);
  const int b = bk / p.W;
  const ReqInfo ri = p.req[b];
  p.slots_out[idx] = t < ri.tail ? resolve_tail_slot(p, b, bk, ri.prefix, t) : -1;
}

hipError_t launch_tail(const TailParams& p, int dtype, int head_dim, hipStream_t s) {
  const int items = p.B * p.W * p.hkv;
  const unsigned blocks = (unsigned)((items + 3) / 4);
#define BSP_TAIL(TT, DD) tail_kernel<TT, DD><<<blocks, 256, 0, s>>>(p)
#define BSP_TAIL_D(TT)             \
  if (head_dim == 64) BSP_TAIL(TT, 64);   \
  else if (head_dim == 128) BSP_TAIL(TT, 128); \
  else BSP_TAIL(TT, 256);
  if (dtype == BSP_F32) {
    BSP_TAIL_D(float)
  } else if (dtype == BSP_F16) {
    BSP_TAIL_D(_Float16)
  } else {
    BSP_TAIL_D(__bf16)
  }
#undef BSP_TAIL_D
#undef BSP_TAIL
  return hipGetLastError();
}

hipError_t launch_tail_slots(const TailParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.W * p.tail_pad;
  if (total == 0) return hipSuccess;
  tail_slots_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsp
