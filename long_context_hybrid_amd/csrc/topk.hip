// Top-K selection over float32 score rows, bit-exact and deterministic.
//
// Rule (Baidu article, "Fine-Grained Sparse Attention: Indexer + Top-K": keep
// the K highest-scoring positions; ties and output order are fixed here): the
// float bits are mapped to an order-preserving 32-bit key; the K largest keys
// win, lower index first among equal keys; the winners are written in
// ascending index order, padded with -1 when a row has fewer than K
// candidates.
//
// One workgroup (1024 threads) per row, no cross-workgroup communication.
//
// 1. Candidate filter.  A row longer than the LDS candidate capacity is first
//    sampled (64 evenly spread runs of 64 keys); a two-pass radix select on the
//    sample gives a threshold t0 a little below the sample's expected K-th
//    largest key.  One pass over the row keeps every key >= t0, in index
//    order, in LDS.  If at least K keys survive, the exact top K are among
//    them (every key outside is below t0, hence below the K-th largest), so
//    the result is exact whatever the sample was; otherwise, or if too many
//    survive, the row falls back to a radix select over the whole row.
// 2. Exact select: radix select of the K-th largest key T in three digit
//    passes (12 + 12 + 8 bits) over an LDS histogram.
// 3. Index-order compaction with one block-wide scan:
//      position(j) = #{j' < j : key > T} + min(#{j' < j : key == T}, k_rem)
//    where k_rem is the number of keys equal to T that belong to the top K,
//    so the output is sorted without a sort.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kNT = 1024;          // threads per row
constexpr int kEPT = 16;           // row elements per thread per segment
constexpr int kSeg = kNT * kEPT;   // 16384
constexpr int kCap = 12288;        // candidate capacity (LDS)
constexpr int kRuns = 64;          // sample: kRuns runs of kRunLen keys
constexpr int kRunLen = 64;
constexpr int kNS = kRuns * kRunLen;
constexpr int kBins = 4096;

struct TopkArgs {
  const float* scores;
  int64_t n_rows;
  int32_t row_len;
  int64_t row_stride;
  ValidLen vl;
  int32_t k;
  int32_t* idx;
};

struct TopkSmem {
  uint32_t ckey[kCap];
  int32_t cidx[kCap];
  uint32_t hist[kBins];
  uint32_t wsum[kNT / 64];
  uint32_t sel[4];
};

// Exclusive block-wide scan of one value per thread; returns the exclusive
// prefix and the total.  Two barriers.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    const uint32_t s = wsum[w];
    pre += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

// Radix select: the k-th largest key T over the keys the visitor hands to its
// callback (this thread's keys), and the number k_rem of keys equal to T that
// belong to the top k.  Requires k <= number of keys.  With `levels` = 2 only
// the top 24 bits are resolved (T's low byte is 0): used for the sample.
template <class Visit>
__device__ __forceinline__ void radix_select(uint32_t k, int levels, Visit visit, TopkSmem& sm, uint32_t* T_out,
                                             uint32_t* krem_out) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, krem = k;
  for (int pass = 0; pass < levels; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const uint32_t dmask = pass == 2 ? 0xFFu : 0xFFFu;
    const uint32_t pmask = pass == 0 ? 0u : (pass == 1 ? 0xFFF00000u : 0xFFFFFF00u);
#pragma unroll
    for (int e = 0; e < kBins / kNT; ++e) sm.hist[t * (kBins / kNT) + e] = 0u;
    __syncthreads();
    visit([&](uint32_t u) {
      if ((u & pmask) == prefix) atomicAdd(&sm.hist[(u >> shift) & dmask], 1u);
    });
    __syncthreads();
    // thread t owns bins [4t, 4t + 4); count keys in higher bins
    uint32_t c[kBins / kNT];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < kBins / kNT; ++e) {
      c[e] = sm.hist[t * (kBins / kNT) + e];
      tot += c[e];
    }
    uint32_t all;
    const uint32_t below = block_scan(tot, sm.wsum, &all);
    const uint32_t above = all - below - tot;
    if (above < krem && krem <= above + tot) {
      uint32_t cum = above;
#pragma unroll
      for (int e = kBins / kNT - 1; e >= 0; --e) {
        if (cum < krem && krem <= cum + c[e]) {
          sm.sel[0] = prefix | ((uint32_t)(t * (kBins / kNT) + e) << shift);
          sm.sel[1] = krem - cum;
        }
        cum += c[e];
      }
    }
    __syncthreads();
    prefix = sm.sel[0];
    krem = sm.sel[1];
    __syncthreads();
  }
  *T_out = prefix;
  *krem_out = krem;
}

__global__ __launch_bounds__(kNT) void topk_row_kernel(TopkArgs a) {
  __shared__ TopkSmem sm;
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  int32_t* out = a.idx + row * a.k;
  if (n <= a.k) {  // every candidate is selected
    for (int x = t; x < a.k; x += kNT) out[x] = x < n ? x : -1;
    return;
  }
  const float* srow = a.scores + row * a.row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  const int nseg = (n + kSeg - 1) / kSeg;

  // this thread's kEPT consecutive keys of segment sg (0 past the row end)
  auto load_seg = [&](int sg, uint32_t (&keys)[kEPT]) {
    const int j0 = sg * kSeg + t * kEPT;
    if (vec && j0 + kEPT <= n) {
#pragma unroll
      for (int e = 0; e < kEPT; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(srow + j0 + e);
        keys[e] = order_key(x.x);
        keys[e + 1] = order_key(x.y);
        keys[e + 2] = order_key(x.z);
        keys[e + 3] = order_key(x.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kEPT; ++e) keys[e] = (j0 + e < n) ? order_key(srow[j0 + e]) : 0u;
    }
  };

  // ---- 1. threshold from a sample (rows longer than the capacity)
  uint32_t t0 = 0u;
  if (n > kCap) {
    // run r covers keys [base_r, base_r + kRunLen); runs are evenly spread
    for (int s = t; s < kNS; s += kNT) {
      const int r = s / kRunLen, o = s - r * kRunLen;
      const int64_t base = (int64_t)r * (n - kRunLen) / (kRuns - 1);
      sm.ckey[s] = order_key(srow[base + o]);
    }
    __syncthreads();
    // rank in the sample: twice the expected count of top-K keys, plus slack
    int64_t q = ((int64_t)kk * kNS + n - 1) / n * 2 + 32;
    if (q > kNS) q = kNS;
    uint32_t T0, r0;
    radix_select((uint32_t)q, 2, [&](auto f) {
      for (int s = t; s < kNS; s += kNT) f(sm.ckey[s]);
    }, sm, &T0, &r0);
    t0 = T0;  // low byte 0: keys >= t0 include the q-th sample key
  }

  // ---- filter: keys >= t0 into LDS, index order
  uint32_t C = 0;  // candidates kept (block-uniform)
  bool fits = true;
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[kEPT];
    load_seg(sg, keys);
    const int j0 = sg * kSeg + t * kEPT;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) cnt += (j0 + e < n && keys[e] >= t0);
    uint32_t tot;
    uint32_t off = C + block_scan(cnt, sm.wsum, &tot);
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      if (j0 + e < n && keys[e] >= t0) {
        if (off < (uint32_t)kCap) {
          sm.ckey[off] = keys[e];
          sm.cidx[off] = j0 + e;
        }
        ++off;
      }
    }
    C += tot;
    if (C > (uint32_t)kCap) {
      fits = false;
      break;
    }
  }
  __syncthreads();

  if (fits && C >= kk) {
    // ---- 2. exact select among the candidates (thread t owns a contiguous run)
    const uint32_t per = (C + kNT - 1) / kNT;
    const uint32_t c0 = min(C, t * per), c1 = min(C, c0 + per);
    uint32_t T, krem;
    radix_select(kk, 3, [&](auto f) {
      for (uint32_t c = c0; c < c1; ++c) f(sm.ckey[c]);
    }, sm, &T, &krem);
    // ---- 3. index-order compaction
    uint32_t gt = 0, eq = 0;
    for (uint32_t c = c0; c < c1; ++c) {
      gt += sm.ckey[c] > T;
      eq += sm.ckey[c] == T;
    }
    uint32_t tg, te;
    uint32_t gb = block_scan(gt, sm.wsum, &tg);
    uint32_t eb = block_scan(eq, sm.wsum, &te);
    for (uint32_t c = c0; c < c1; ++c) {
      const uint32_t u = sm.ckey[c];
      const bool is_gt = u > T, is_eq = u == T;
      const uint32_t p = gb + (is_gt ? min(eb, krem) : eb);
      if ((is_gt || (is_eq && eb < krem)) && p < kk) out[p] = sm.cidx[c];
      gb += is_gt;
      eb += is_eq;
    }
    return;
  }

  // ---- fallback: radix select and compaction over the whole row
  uint32_t T, krem;
  radix_select(kk, 3, [&](auto f) {
    for (int sg = 0; sg < nseg; ++sg) {
      uint32_t keys[kEPT];
      load_seg(sg, keys);
      const int j0 = sg * kSeg + t * kEPT;
#pragma unroll
      for (int e = 0; e < kEPT; ++e)
        if (j0 + e < n) f(keys[e]);
    }
  }, sm, &T, &krem);
  uint32_t g_base = 0, e_base = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[kEPT];
    load_seg(sg, keys);
    const int j0 = sg * kSeg + t * kEPT;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const bool in = j0 + e < n;
      gt += (in && keys[e] > T);
      eq += (in && keys[e] == T);
    }
    uint32_t tg, te;
    uint32_t gb = g_base + block_scan(gt, sm.wsum, &tg);
    uint32_t eb = e_base + block_scan(eq, sm.wsum, &te);
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const bool in = j0 + e < n;
      const bool is_gt = in && keys[e] > T;
      const bool is_eq = in && keys[e] == T;
      const uint32_t p = gb + (is_gt ? min(eb, krem) : eb);
      if ((is_gt || (is_eq && eb < krem)) && p < kk) out[p] = j0 + e;
      gb += is_gt;
      eb += is_eq;
    }
    g_base += tg;
    e_base += te;
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
  topk_row_kernel<<<(unsigned)n_rows, kNT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hys
