// Index-set check: a debugging aid for callers that build the sparse layer's
// index rows themselves (the sparse layer requires distinct entries: a key
// listed twice would enter the global branch's softmax twice).  One
// workgroup per row: the row's entries mark a bitmap of the row's positions
// in LDS (an entry already marked is a duplicate), and each entry is compared
// with its predecessor for the canonical form that top-K writes (strictly
// ascending, -1 padding only at the end).  Nothing traps: the findings are
// status bits per row.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kNT = 256;

__global__ __launch_bounds__(kNT) void check_indices_kernel(const int32_t* idx, int k, int row_len, ValidLen vl,
                                                            int32_t* status) {
  extern __shared__ uint32_t bitmap[];
  __shared__ uint32_t wflags[kNT / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = valid_len_of(vl, row);
  const int words = (row_len + 31) / 32;
  for (int w = tid; w < words; w += kNT) bitmap[w] = 0u;
  __syncthreads();
  const int32_t* r = idx + row * (int64_t)k;
  uint32_t flags = 0;
  for (int e = tid; e < k; e += kNT) {
    const int32_t x = r[e];
    const int32_t p = e > 0 ? r[e - 1] : -2;
    if (x >= 0) {
      if (x >= n) flags |= kIdxOutOfRange;
      if (x < row_len) {
        const uint32_t bit = 1u << (x & 31);
        if (atomicOr(&bitmap[x >> 5], bit) & bit) flags |= kIdxDuplicate;
      }
      if (e > 0 && (p < 0 || p >= x)) flags |= kIdxOrder;  // after padding, or not ascending
    } else if (x < -1) {
      flags |= kIdxOutOfRange;
    }
  }
  // OR over the workgroup
  for (int off = 32; off > 0; off >>= 1) flags |= (uint32_t)__shfl_xor((int)flags, off);
  if ((tid & 63) == 0) wflags[tid >> 6] = flags;
  __syncthreads();
  if (tid == 0) status[row] = (int32_t)(wflags[0] | wflags[1] | wflags[2] | wflags[3]);
}

}  // namespace

int check_indices_max_row_len() { return 64 * 1024 * 8; }  // a 64 KiB bitmap

hipError_t launch_check_indices(const int32_t* idx, int64_t n_rows, int k, int row_len, const ValidLen& vl,
                                int32_t* status, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const uint32_t lds = (uint32_t)((row_len + 31) / 32) * 4u;
  return launch("check_indices", check_indices_kernel, dim3((unsigned)n_rows), dim3(kNT), lds, st, idx, k, row_len,
                vl, status);
}

}  // namespace hys
