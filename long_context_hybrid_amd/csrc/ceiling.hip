// Size-matched bandwidth ceilings for the decode-time sparse layer: how fast
// one launch of this size can move the bytes the layer moves, with nothing
// else to do.  The layer is memory-bound (Baidu article, "Key Engineering
// Considerations": decoding is limited by memory bandwidth, which is what to
// measure), and a launch of a few tens of MB cannot reach the HBM peak, so
// its achieved rate is also stated against these two kernels:
//   * a streaming read of N contiguous bytes;
//   * a gather of rows of the KV cache at given row indices (the layer's own
//     global and window rows), K and V rows both, indices loaded first.
// Neither computes anything: each thread folds what it loads into one word
// so that the loads are kept, and each workgroup writes one word.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kNT = 256;
constexpr int kStreamU = 4;  // 16-byte loads per thread in flight
constexpr int kGatherU = 4;  // rows per thread in flight (x2: K and V)

__global__ __launch_bounds__(kNT) void ceiling_stream_kernel(const unsigned char* p, int64_t n16, uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * kNT * kStreamU + threadIdx.x;
  uint32_t acc = 0;
  uint4 x[kStreamU];
#pragma unroll
  for (int u = 0; u < kStreamU; ++u) {
    const int64_t c = base + (int64_t)u * kNT;
    x[u] = c < n16 ? load16_stream<true>(p + c * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kStreamU; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  __shared__ uint32_t red[kNT / 64];
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// 16 threads per row (16 bytes each, rows of row_bytes <= 256), 16 rows per
// workgroup pass, kGatherU passes in flight.  Row indices outside
// [0, n_buf_rows) are skipped.
__global__ __launch_bounds__(kNT) void ceiling_gather_kernel(const unsigned char* k, const unsigned char* v,
                                                             int64_t row_stride, const int32_t* rows, int64_t n_rows,
                                                             int64_t n_buf_rows, int row_chunks, uint32_t* sink) {
  const int lane16 = threadIdx.x & 15, r16 = threadIdx.x >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 16 * kGatherU + r16;
  int32_t j[kGatherU];
#pragma unroll
  for (int u = 0; u < kGatherU; ++u) {
    const int64_t r = r0 + 16 * u;
    j[u] = r < n_rows ? rows[r] : -1;
  }
  uint4 x[2 * kGatherU];
#pragma unroll
  for (int u = 0; u < kGatherU; ++u) {
    const bool in = j[u] >= 0 && j[u] < n_buf_rows && lane16 < row_chunks;
    const int64_t off = (int64_t)(j[u] < 0 ? 0 : j[u]) * row_stride + 16 * lane16;
    x[2 * u] = in ? load16_stream<false>(k + off) : make_uint4(0, 0, 0, 0);
    x[2 * u + 1] = in ? load16_stream<false>(v + off) : make_uint4(0, 0, 0, 0);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 2 * kGatherU; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  __shared__ uint32_t red[kNT / 64];
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int64_t ceiling_stream_blocks(int64_t n_bytes) {
  const int64_t n16 = n_bytes / 16;
  return (n16 + (int64_t)kNT * kStreamU - 1) / ((int64_t)kNT * kStreamU);
}

int64_t ceiling_gather_blocks(int64_t n_rows) { return (n_rows + 16 * kGatherU - 1) / (16 * kGatherU); }

hipError_t launch_ceiling_stream(const void* p, int64_t n_bytes, uint32_t* sink, hipStream_t st) {
  const int64_t nb = ceiling_stream_blocks(n_bytes);
  if (nb == 0) return hipSuccess;
  return launch("ceiling_stream", ceiling_stream_kernel, dim3((unsigned)nb), dim3(kNT), 0, st,
                static_cast<const unsigned char*>(p), n_bytes / 16, sink);
}

hipError_t launch_ceiling_gather(const void* k, const void* v, int64_t row_stride_bytes, int64_t n_buf_rows,
                                 const int32_t* rows, int64_t n_rows, int row_bytes, uint32_t* sink, hipStream_t st) {
  const int64_t nb = ceiling_gather_blocks(n_rows);
  if (nb == 0) return hipSuccess;
  return launch("ceiling_gather", ceiling_gather_kernel, dim3((unsigned)nb), dim3(kNT), 0, st,
                static_cast<const unsigned char*>(k), static_cast<const unsigned char*>(v), row_stride_bytes, rows,
                n_rows, n_buf_rows, row_bytes / 16, sink);
}

}  // namespace hys
