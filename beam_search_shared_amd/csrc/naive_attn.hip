// Comparator: per-beam decode attention over each beam's whole sequence.
//
// This is the shape of the decode kernel the cascade replaces: one workgroup
// per (request, beam, query head), reading every cached row of that beam, the
// shared prompt included, once per beam and head (TensorRT-LLM PR #21738, "Add
// opt-in cascade attention for wide beam search on KVCM V2", first commit
// message). Prompt positions are read through the beam's own block table,
// tail positions through cache_indirection.
//
// Inside the workgroup it is a reasonable split-K decode kernel: each group of
// LPK lanes reads one 16-byte slice per lane of one key row, the 4 waves and
// the key groups inside them walk interleaved key sets with their own online
// softmax, and the partial states are combined through LDS at the end.
#include "bsp_internal.h"
#include "device_common.h"

namespace bsp {

template <typename T, int D>
__global__ __launch_bounds__(256) void naive_kernel(TailParams p, void* o_out, float* lse_out) {
  constexpr int VEC = 16 / sizeof(T);            // elements per lane per key
  constexpr int LPK = D / VEC;                   // lanes per key row (8 .. 64)
  constexpr int KPW = 64 / LPK;                  // key rows per wave per step
  constexpr int GROUPS = 4 * KPW;                // independent key walkers per workgroup
  static_assert(LPK == 8 || LPK == 16 || LPK == 32 || LPK == 64, "lanes per key");
  __shared__ float st_o[GROUPS][D];
  __shared__ float st_m[GROUPS], st_l[GROUPS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / LPK;                    // key slot inside the wave
  const int li = lane % LPK;
  const int group = wave * KPW + sub;

  const int item = blockIdx.x;                   // ((b * W + k) * Hq + h)
  const int h = item % p.hq;
  const int bk = item / p.hq;
  const int b = bk / p.W;
  const int k = bk % p.W;
  const int g = h / p.group;
  const ReqInfo ri = p.req[b];
  const int P = ri.prefix, S = ri.seq;
  const int ps = 1 << p.page_shift;
  const T* kp = static_cast<const T*>(p.k_pool);
  const T* vp = static_cast<const T*>(p.v_pool);

  float q[VEC];
  {
    const T* qp = static_cast<const T*>(p.q) + ((int64_t)bk * p.hq + h) * D + li * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) q[e] = Traits<T>::to_f(qp[e]);
  }
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int j = group; j < S; j += GROUPS) {
    const int src = j < P ? k : p.ci[(int64_t)bk * p.max_seq_len + j];
    float s = -INFINITY;
    float vv[VEC];
    bool ok = src >= 0 && src < p.W;
    int32_t page = -1;
    if (ok) {
      page = p.block_tables[((int64_t)b * p.W + src) * p.max_blocks + (j >> p.page_shift)];
      ok = page >= 0 && page < p.num_pages;
    }
    float part = 0.f;
    if (ok) {
      const int64_t off =
          (((int64_t)page * p.hkv + g) * ps + (j & (ps - 1))) * D + li * VEC;
      const u32x4 kraw = *reinterpret_cast<const u32x4*>(kp + off);
      const u32x4 vraw = *reinterpret_cast<const u32x4*>(vp + off);
      const T* ke = reinterpret_cast<const T*>(&kraw);
      const T* ve = reinterpret_cast<const T*>(&vraw);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        part = fmaf(q[e], Traits<T>::to_f(ke[e]), part);
        vv[e] = Traits<T>::to_f(ve[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) vv[e] = 0.f;
    }
    // reduce the dot product over the LPK lanes of this key slot
    part += dpp_mov<kDppXor1>(part);
    part += dpp_mov<kDppXor2>(part);
    part += dpp_mov<kDppHalfMirror>(part);
    if (LPK >= 16) part += dpp_mov<kDppMirror>(part);
    if (LPK >= 32) part += __shfl_xor(part, 16, 64);
    if (LPK == 64) part += __shfl_xor(part, 32, 64);
    if (ok) s = part * p.scale_log2e;
    const float m_new = fmaxf(m, s);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    const float pj = fast_exp2(s - m_use);
    l = l * alpha + pj;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pj, vv[e], acc[e] * alpha);
    m = m_new;
  }

#pragma unroll
  for (int e = 0; e < VEC; ++e) st_o[group][li * VEC + e] = acc[e];
  if (li == 0) {
    st_m[group] = m;
    st_l[group] = l;
  }
  __syncthreads();
  if (tid < D) {
    float mm = -INFINITY;
    for (int gi = 0; gi < GROUPS; ++gi) mm = fmaxf(mm, st_m[gi]);
    const float mu = mm == -INFINITY ? 0.f : mm;
    float ll = 0.f, oo = 0.f;
    for (int gi = 0; gi < GROUPS; ++gi) {
      const float w = fast_exp2(st_m[gi] - mu);
      ll += st_l[gi] * w;
      oo += st_o[gi][tid] * w;
    }
    T* out = static_cast<T*>(o_out) + ((int64_t)bk * p.hq + h) * D;
    out[tid] = Traits<T>::from_f(ll > 0.f ? oo / ll : 0.f);
    if (tid == 0 && lse_out != nullptr)
      lse_out[(int64_t)bk * p.hq + h] = ll > 0.f ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_naive(const TailParams& p, void* o_out, float* lse_out, int dtype,
                        int head_dim, hipStream_t s) {
  const unsigned blocks = (unsigned)(p.B * p.W * p.hq);
#define BSP_NAIVE(TT, DD) naive_kernel<TT, DD><<<blocks, 256, 0, s>>>(p, o_out, lse_out)
#define BSP_NAIVE_D(TT)                             \
  if (head_dim == 64) BSP_NAIVE(TT, 64);            \
  else if (head_dim == 128) BSP_NAIVE(TT, 128);     \
  else BSP_NAIVE(TT, 256);
  if (dtype == BSP_F32) {
    BSP_NAIVE_D(float)
  } else if (dtype == BSP_F16) {
    BSP_NAIVE_D(_Float16)
  } else {
    BSP_NAIVE_D(__bf16)
  }
#undef BSP_NAIVE_D
#undef BSP_NAIVE
  return hipGetLastError();
}

}  // namespace bsp
