// The second launch of a one-row cached-prefix decode (bsp_cached_decode_merge):
// the exact n-way merge of the cache chunks' partial states folded with the
// call's own row, and that row's write into its page.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsp_internal.h"

namespace bsp {

struct MergeRowParams {
  int32_t rows, hq, hkv, d, n_parts;  // rows: requests, one query row each
  const float* o_parts;               // [n_parts][rows][hq][d]
  const float* lse_parts;             // [n_parts][rows][hq]
  int64_t o_stride, lse_stride;       // floats between two parts
  const void* q;                      // [rows][hq][d]
  const void* k_new;                  // request b's row at element b * new_stride, [hkv][d]
  const void* v_new;
  int64_t new_stride;
  const int32_t* slots;  // [rows]: page * page_size + row of the call's row
  void* k_pool;
  void* v_pool;
  int32_t page_shift, num_pages;
  float scale;  // softmax scale of the scores
  void* o_out;  // [rows][hq][d]
  float* lse_out;  // [rows][hq] or null
  DevHeader* hdr;  // fault record (a slot outside the pool)
};

hipError_t launch_merge_row(const MergeRowParams& p, int dtype, hipStream_t s);

}  // namespace bsp
