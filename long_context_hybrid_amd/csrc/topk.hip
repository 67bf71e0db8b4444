// Top-K selection over float32 score rows, bit-exact and deterministic.
//
// Rule (Baidu article, "Fine-Grained Sparse Attention: Indexer + Top-K": keep
// the K highest-scoring positions; ties and output order are fixed here): the
// float bits are mapped to an order-preserving 32-bit key; the K largest keys
// win, lower index first among equal keys; the winners are written in
// ascending index order, padded with -1 when a row has fewer than K
// candidates.
//
// One workgroup per row, no cross-workgroup communication.  The row's keys
// are held in registers when the row fits one segment of NT * EPT elements
// (thread t owns EPT consecutive elements of each segment); longer rows
// re-read their segments from global memory (L2) in every pass.  A radix select finds the K-th largest key T in three digit
// passes (12 + 12 + 8 bits) over LDS histograms; the histogram is replicated
// eight times (copy = lane % 8) so lanes of a wave that hit the same digit
// rarely collide on one LDS address.  The selection is then compacted in
// index order with one block-wide scan:
//   position(j) = #{j' < j : key > T} + min(#{j' < j : key == T}, k_rem)
// where k_rem is the number of keys equal to T that belong to the top K, so
// the output is sorted without a sort.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kBins = 4096;
constexpr int kRep = 8;

struct TopkArgs {
  const float* scores;
  int64_t n_rows;
  int32_t row_len;
  int64_t row_stride;
  ValidLen vl;
  int32_t k;
  int32_t* idx;
};

// Exclusive block scan of 64-bit values; sh must hold NT/64 entries.
template <int NT>
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint64_t* sh, uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint64_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) pre += sh[w];
    tot += sh[w];
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_row_kernel(TopkArgs a) {
  constexpr int SEG = NT * EPT;
  __shared__ uint32_t hist[kRep * kBins];
  __shared__ uint32_t suf[NT];
  __shared__ uint64_t scan_sh[NT / 64];
  __shared__ uint32_t sel_s[2];

  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const int kk = a.k;
  int32_t* out = a.idx + row * kk;
  if (n <= kk) {  // every candidate is selected
    for (int x = t; x < kk; x += NT) out[x] = x < n ? x : -1;
    return;
  }
  const float* srow = a.scores + row * a.row_stride;
  const int nseg = (n + SEG - 1) / SEG;

  uint32_t keys[EPT];
  // 16-byte loads when the row base is 16-byte aligned
  const bool vec = ((reinterpret_cast<uintptr_t>(srow) & 15) == 0);
  auto load_seg = [&](int sg) {
    const int j0 = sg * SEG + t * EPT;
    if (vec && j0 + EPT <= n) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(srow + j0 + e);
        keys[e] = order_key(x.x);
        keys[e + 1] = order_key(x.y);
        keys[e + 2] = order_key(x.z);
        keys[e + 3] = order_key(x.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int j = j0 + e;
        keys[e] = j < n ? order_key(srow[j]) : 0u;
      }
    }
  };

  uint32_t prefix = 0, krem = (uint32_t)kk;
  const int rep = (t & (kRep - 1)) * kBins;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nbins = pass == 2 ? 256 : 4096;
    const uint32_t dmask = (uint32_t)nbins - 1u;
    const uint32_t pmask = pass == 0 ? 0u : (pass == 1 ? 0xFFF00000u : 0xFFFFFF00u);
    for (int x = t; x < kRep * kBins; x += NT) hist[x] = 0u;
    __syncthreads();
#pragma unroll 1
    for (int sg = 0; sg < nseg; ++sg) {
      if (nseg > 1 || pass == 0) load_seg(sg);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int j = sg * SEG + t * EPT + e;
        const uint32_t u = keys[e];
        if (j < n && (u & pmask) == prefix) atomicAdd(&hist[rep + ((u >> shift) & dmask)], 1u);
      }
    }
    __syncthreads();
    // fold the copies, then find the digit holding the krem-th largest key
    constexpr int PBMAX = kBins / NT > 0 ? kBins / NT : 1;
    const int pb = nbins / NT > 0 ? nbins / NT : 1;  // bins per thread
    const int owner_threads = nbins / pb;
    uint32_t cnt[PBMAX];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < PBMAX; ++e) {
      cnt[e] = 0u;
      if (e < pb && t < owner_threads) {
        const int d = t * pb + e;
#pragma unroll
        for (int r = 0; r < kRep; ++r) cnt[e] += hist[r * kBins + d];
        tot += cnt[e];
      }
    }
    suf[t] = tot;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const uint32_t v = suf[t] + ((t + off < NT) ? suf[t + off] : 0u);
      __syncthreads();
      suf[t] = v;
      __syncthreads();
    }
    const uint32_t above = suf[t] - tot;
    if (t < owner_threads && above < krem && krem <= above + tot) {
      uint32_t cum = above;
      for (int e = pb - 1; e >= 0; --e) {
        if (cum + cnt[e] >= krem) {
          sel_s[0] = prefix | ((uint32_t)(t * pb + e) << shift);
          sel_s[1] = krem - cum;
          break;
        }
        cum += cnt[e];
      }
    }
    __syncthreads();
    prefix = sel_s[0];
    krem = sel_s[1];
    __syncthreads();
  }

  // compaction in index order
  const uint32_t T = prefix;
  uint64_t g_base = 0, e_base = 0;  // counts of earlier segments (block-uniform)
#pragma unroll 1
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t gt = 0, eq = 0;
    if (nseg > 1) load_seg(sg);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int j = sg * SEG + t * EPT + e;
      const bool in = j < n;
      gt += (in && keys[e] > T);
      eq += (in && keys[e] == T);
    }
    uint64_t total;
    const uint64_t ex = block_excl_scan64<NT>(((uint64_t)gt << 32) | eq, scan_sh, &total);
    // positions fit 32 bits: rows are shorter than 2^31
    uint32_t gb = (uint32_t)(g_base + (ex >> 32));
    uint32_t eb = (uint32_t)(e_base + (ex & 0xFFFFFFFFull));
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int j = sg * SEG + t * EPT + e;
      const bool in = j < n;
      const bool is_gt = in && keys[e] > T;
      const bool is_eq = in && keys[e] == T;
      const uint32_t p = gb + (is_gt ? min(eb, krem) : eb);
      if ((is_gt || (is_eq && eb < krem)) && p < (uint32_t)kk) out[p] = j;
      gb += is_gt;
      eb += is_eq;
    }
    g_base += total >> 32;
    e_base += total & 0xFFFFFFFFull;
  }
}

}  // namespace

size_t topk_ws_bytes(int64_t, int32_t, int32_t) { return 0; }

hipError_t launch_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                       const ValidLen& vl, int32_t k, int32_t* idx, void* /*ws*/, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  TopkArgs a{};
  a.scores = scores;
  a.n_rows = n_rows;
  a.row_len = row_len;
  a.row_stride = row_stride;
  a.vl = vl;
  a.k = k;
  a.idx = idx;
  TraceScope ts(st, "topk");
  if (row_len <= 256 * 4)
    topk_row_kernel<256, 4><<<(unsigned)n_rows, 256, 0, st>>>(a);
  else if (row_len <= 1024 * 8)
    topk_row_kernel<1024, 8><<<(unsigned)n_rows, 1024, 0, st>>>(a);
  else  // longer rows run in register-sized segments of 16384
    topk_row_kernel<512, 32><<<(unsigned)n_rows, 512, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hys
