// Top-K selection over float32 score rows, bit-exact and deterministic.
//
// Rule (Baidu article, "Fine-Grained Sparse Attention: Indexer + Top-K": keep
// the K highest-scoring positions; ties and output order are fixed here): the
// float bits are mapped to an order-preserving 32-bit key; the K largest keys
// win, lower index first among equal keys; the winners are written in
// ascending index order, padded with -1 when a row has fewer than K
// candidates.
//
// Method: radix select of the K-th largest key T in three digit passes
// (12 + 12 + 8 bits).  Each pass is one launch over (row, 4096-element chunk)
// workgroups: a chunk histogram in LDS is added to the row histogram with
// integer atomics (order-independent), and the row's last-arriving workgroup
// scans it, fixes the next digit of T and the number of keys equal to T that
// still have to be taken, then clears the histogram.  Afterwards a count pass
// and a write pass compact the selection in index order:
//   position(j) = #{j' < j : key > T} + min(#{j' < j : key == T}, k_rem)
// so the output is sorted without a sort and identical on every run.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kTkThreads = 256;
constexpr int kTkPer = 16;
constexpr int kTkChunk = kTkThreads * kTkPer;  // 4096 elements per workgroup
constexpr int kBins = 4096;

struct TopkArgs {
  const float* scores;
  int64_t n_rows;
  int32_t row_len;
  int64_t row_stride;
  ValidLen vl;
  int32_t k;
  int32_t* idx;
  uint32_t* hist;    // [n_rows][kBins]
  uint32_t* state;   // [n_rows][2]: key prefix, keys still to take at the prefix
  uint32_t* arrive;  // [n_rows]
  uint32_t* counts;  // [n_rows][nchunk][2]: (#greater, #equal) per chunk
  int nchunk;
};

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += sh[w];
  __syncthreads();
  return pre + x - v;
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x)
    p[x] = v;
}

template <int PASS>
__global__ __launch_bounds__(kTkThreads) void topk_hist_kernel(TopkArgs a) {
  constexpr int SHIFT = PASS == 0 ? 20 : (PASS == 1 ? 8 : 0);
  constexpr int NBITS = PASS == 2 ? 8 : 12;
  constexpr int NB = 1 << NBITS;
  constexpr uint32_t DMASK = (uint32_t)NB - 1u;
  constexpr uint32_t PMASK = PASS == 0 ? 0u : (PASS == 1 ? 0xFFF00000u : 0xFFFFFF00u);
  constexpr int PER = NB / kTkThreads;

  __shared__ uint32_t h[kBins];
  __shared__ uint32_t suf[kTkThreads];
  __shared__ int last_flag;

  const int64_t row = blockIdx.x / a.nchunk;
  const int c = blockIdx.x - (int)(row * a.nchunk);
  const int n = valid_len_of(a.vl, row);
  if (n <= a.k) return;
  const int nch = (n + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  const int t = threadIdx.x;
  uint32_t prefix = 0, krem = (uint32_t)a.k;
  if (PASS > 0) {
    prefix = a.state[row * 2];
    krem = a.state[row * 2 + 1];
  }
  for (int x = t; x < NB; x += kTkThreads) h[x] = 0;
  __syncthreads();
  const float* srow = a.scores + row * a.row_stride;
  const int j0 = c * kTkChunk;
#pragma unroll 4
  for (int r = 0; r < kTkPer; ++r) {
    const int j = j0 + r * kTkThreads + t;
    if (j < n) {
      const uint32_t u = order_key(srow[j]);
      if ((u & PMASK) == prefix) atomicAdd(&h[(u >> SHIFT) & DMASK], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + row * kBins;
  for (int x = t; x < NB; x += kTkThreads) {
    const uint32_t v = h[x];
    if (v) atomicAdd(&gh[x], v);
  }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t old = atomicAdd(&a.arrive[row], 1u);
    last_flag = (old == (uint32_t)nch - 1u);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  // last workgroup of the row: choose the digit holding the krem-th largest key
  for (int x = t; x < NB; x += kTkThreads) h[x] = __hip_atomic_load(&gh[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) tot += h[t * PER + e];
  suf[t] = tot;
  __syncthreads();
  for (int off = 1; off < kTkThreads; off <<= 1) {
    const uint32_t v = suf[t] + ((t + off < kTkThreads) ? suf[t + off] : 0u);
    __syncthreads();
    suf[t] = v;
    __syncthreads();
  }
  const uint32_t above = suf[t] - tot;  // keys with a higher digit than this thread's digits
  if (above < krem && krem <= above + tot) {
    uint32_t cum = above;
    for (int e = PER - 1; e >= 0; --e) {
      const int d = t * PER + e;
      if (cum + h[d] >= krem) {
        a.state[row * 2] = prefix | ((uint32_t)d << SHIFT);
        a.state[row * 2 + 1] = krem - cum;
        break;
      }
      cum += h[d];
    }
  }
  for (int x = t; x < NB; x += kTkThreads) gh[x] = 0;
  if (t == 0) a.arrive[row] = 0;
}

__global__ __launch_bounds__(kTkThreads) void topk_count_kernel(TopkArgs a) {
  __shared__ uint32_t sh[4];
  const int64_t row = blockIdx.x / a.nchunk;
  const int c = blockIdx.x - (int)(row * a.nchunk);
  const int n = valid_len_of(a.vl, row);
  if (n <= a.k) return;
  const int nch = (n + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  const uint32_t T = a.state[row * 2];
  const float* srow = a.scores + row * a.row_stride;
  const int j0 = c * kTkChunk;
  uint32_t gt = 0, eq = 0;
#pragma unroll 4
  for (int r = 0; r < kTkPer; ++r) {
    const int j = j0 + r * kTkThreads + threadIdx.x;
    if (j < n) {
      const uint32_t u = order_key(srow[j]);
      gt += (u > T);
      eq += (u == T);
    }
  }
  // packed (gt << 16 | eq): both <= 4096 per chunk
  const uint32_t packed = (gt << 16) | eq;
  const uint32_t ex = block_excl_scan(packed, sh);
  if (threadIdx.x == kTkThreads - 1) {
    const uint32_t tot = ex + packed;
    a.counts[(row * a.nchunk + c) * 2 + 0] = tot >> 16;
    a.counts[(row * a.nchunk + c) * 2 + 1] = tot & 0xFFFFu;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_write_kernel(TopkArgs a) {
  __shared__ uint32_t sh[4];
  __shared__ uint32_t base_s[2];
  const int64_t row = blockIdx.x / a.nchunk;
  const int c = blockIdx.x - (int)(row * a.nchunk);
  const int n = valid_len_of(a.vl, row);
  int32_t* out = a.idx + row * a.k;
  const int t = threadIdx.x;
  const int j0 = c * kTkChunk;
  if (n <= a.k) {  // every candidate is selected
    if (c == 0)
      for (int x = n + t; x < a.k; x += kTkThreads) out[x] = -1;
    for (int r = 0; r < kTkPer; ++r) {
      const int j = j0 + r * kTkThreads + t;
      if (j < n) out[j] = j;
    }
    return;
  }
  const int nch = (n + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  const uint32_t T = a.state[row * 2];
  const uint32_t krem = a.state[row * 2 + 1];
  if (t == 0) {
    uint32_t bg = 0, be = 0;
    for (int cc = 0; cc < c; ++cc) {
      bg += a.counts[(row * a.nchunk + cc) * 2 + 0];
      be += a.counts[(row * a.nchunk + cc) * 2 + 1];
    }
    base_s[0] = bg;
    base_s[1] = be;
  }
  // each thread owns 16 consecutive elements
  const float* srow = a.scores + row * a.row_stride;
  const int jt = j0 + t * kTkPer;
  uint32_t keys[kTkPer];
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) {
    const int j = jt + e;
    keys[e] = (j < n) ? order_key(srow[j]) : 0u;
    const bool in = j < n;
    gt += (in && keys[e] > T);
    eq += (in && keys[e] == T);
  }
  const uint32_t packed = (gt << 16) | eq;
  const uint32_t ex = block_excl_scan(packed, sh);
  uint32_t g_before = base_s[0] + (ex >> 16);
  uint32_t e_before = base_s[1] + (ex & 0xFFFFu);
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) {
    const int j = jt + e;
    if (j < n) {
      if (keys[e] > T) {
        const uint32_t p = g_before + min(e_before, krem);
        if (p < (uint32_t)a.k) out[p] = j;
        ++g_before;
      } else if (keys[e] == T) {
        const uint32_t p = g_before + e_before;
        if (e_before < krem && p < (uint32_t)a.k) out[p] = j;
        ++e_before;
      }
    }
  }
}

struct TopkWs {
  uint32_t *hist, *arrive, *state, *counts;
};

TopkWs carve_topk(void* ws, int64_t n_rows, int nchunk) {
  TopkWs w;
  unsigned char* c = static_cast<unsigned char*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(c);
  w.arrive = w.hist + (size_t)n_rows * kBins;  // contiguous with hist: cleared together
  c += align_up((size_t)n_rows * (kBins + 1) * sizeof(uint32_t));
  w.state = reinterpret_cast<uint32_t*>(c);
  c += align_up((size_t)n_rows * 2 * sizeof(uint32_t));
  w.counts = reinterpret_cast<uint32_t*>(c);
  return w;
}

}  // namespace

size_t topk_ws_bytes(int64_t n_rows, int32_t row_len, int32_t /*k*/) {
  const int nchunk = (row_len + kTkChunk - 1) / kTkChunk;
  return align_up((size_t)n_rows * (kBins + 1) * sizeof(uint32_t)) + align_up((size_t)n_rows * 2 * sizeof(uint32_t)) +
         align_up((size_t)n_rows * nchunk * 2 * sizeof(uint32_t));
}

hipError_t launch_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                       const ValidLen& vl, int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int nchunk = (row_len + kTkChunk - 1) / kTkChunk;
  const TopkWs w = carve_topk(ws, n_rows, nchunk);
  TopkArgs a{};
  a.scores = scores;
  a.n_rows = n_rows;
  a.row_len = row_len;
  a.row_stride = row_stride;
  a.vl = vl;
  a.k = k;
  a.idx = idx;
  a.hist = w.hist;
  a.state = w.state;
  a.arrive = w.arrive;
  a.counts = w.counts;
  a.nchunk = nchunk;
  const int64_t nclear = n_rows * (int64_t)(kBins + 1);
  int64_t fb = (nclear + 255) / 256;
  if (fb > 4096) fb = 4096;
  fill_u32_kernel<<<(unsigned)fb, 256, 0, st>>>(w.hist, 0u, nclear);
  const int64_t grid = n_rows * nchunk;
  topk_hist_kernel<0><<<(unsigned)grid, kTkThreads, 0, st>>>(a);
  topk_hist_kernel<1><<<(unsigned)grid, kTkThreads, 0, st>>>(a);
  topk_hist_kernel<2><<<(unsigned)grid, kTkThreads, 0, st>>>(a);
  topk_count_kernel<<<(unsigned)grid, kTkThreads, 0, st>>>(a);
  topk_write_kernel<<<(unsigned)grid, kTkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hys
