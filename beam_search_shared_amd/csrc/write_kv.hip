// Current-token KV write: one launch writes K and V of every new token into the
// paged pools, deriving (page, row) from the token's flat slot in registers
// (TensorRT-LLM PR #18614, "Fuse MiniMax-M3 MSA per-layer KV-cache writes into
// one kernel", Description: The fix).
//
// One thread moves 16 bytes of K and the same 16 bytes of V. Consecutive
// threads cover one (token, head) row, so both the read of k_new and the write
// into the page are contiguous per row.
#include "bsp_internal.h"
#include "device_common.h"

namespace bsp {

template <typename T>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteKvParams p) {
  constexpr int VEC = 16 / sizeof(T);
  const int chunks_per_row = p.d / VEC;
  const int64_t total = (int64_t)p.n * p.hkv * chunks_per_row;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % chunks_per_row);
  const int64_t th = idx / chunks_per_row;
  const int h = (int)(th % p.hkv);
  const int i = (int)(th / p.hkv);

  const int32_t slot = p.slots[i];
  if (slot < 0 || (int64_t)slot >= p.num_slots) {
    if (h == 0 && c == 0 && p.fault != nullptr)
      record_fault(p.fault, p.fault + 1, p.fault + 2, kErrWriteSlot, slot);
    return;
  }
  const int page = slot / p.page_size;
  const int row = slot - page * p.page_size;
  const int64_t src = (int64_t)i * p.src_stride + (int64_t)h * p.d + (int64_t)c * VEC;
  const int64_t dst = (((int64_t)page * p.hkv + h) * p.page_size + row) * p.d + (int64_t)c * VEC;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const T*>(p.k_new) + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const T*>(p.v_new) + src);
  *reinterpret_cast<u32x4*>(static_cast<T*>(p.k_pool) + dst) = kv;
  *reinterpret_cast<u32x4*>(static_cast<T*>(p.v_pool) + dst) = vv;
}

hipError_t launch_write_kv(const WriteKvParams& p, int dtype, hipStream_t s) {
  const int vec = dtype == BSP_F32 ? 4 : 8;
  const int64_t total = (int64_t)p.n * p.hkv * (p.d / vec);
  const int64_t blocks = (total + 255) / 256;
  if (dtype == BSP_F32)
    write_kv_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else if (dtype == BSP_F16)
    write_kv_kernel<_Float16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  else
    write_kv_kernel<__bf16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bsp
