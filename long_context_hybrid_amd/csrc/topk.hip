// Top-K selection over float32 score rows, bit-exact and deterministic.
//
// Rule (Baidu article, "Fine-Grained Sparse Attention: Indexer + Top-K": keep
// the K highest-scoring positions; ties and output order are fixed here): the
// float bits are mapped to an order-preserving 32-bit key; the K largest keys
// win, lower index first among equal keys; the winners are written in
// ascending index order, padded with -1 when a row has fewer than K
// candidates.
//
// One workgroup (1024 threads) per row.  When there are few long rows (decode:
// a handful of rows of the whole context) the candidate filter of step 1 is
// spread over `nparts` workgroups per row, each writing the survivors of its
// part of the row, in index order, to its own workspace region; a second
// kernel concatenates the regions in part order and runs steps 2 and 3.
// Both forms select exactly the same indices.
//
// 1. Candidate filter.  A row longer than the LDS candidate capacity is first
//    sampled (64 evenly spread runs of 64 keys); a radix select on the
//    sample gives a threshold t0, the sample key of rank about twice the
//    expected rank of the K-th largest key.  One pass over the row keeps every key >= t0, in index
//    order, in LDS.  If at least K keys survive, the exact top K are among
//    them (every key outside is below t0, hence below the K-th largest), so
//    the result is exact whatever the sample was; otherwise, or if too many
//    survive, the row falls back to a radix select over the whole row.
// 2. Exact select: radix select of the K-th largest key T over an LDS
//    histogram, with 12-bit digits of (key - min) taken over the range the
//    keys actually span (at most three passes).
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
constexpr int kPartLen = 4096;     // parallel filter: keys per part pass (kNT x 4)
constexpr int kPartRows = 256;     // rows below which long rows are filtered in parts
constexpr int kMaxParts = 64;
constexpr int kPartWGs = 512;      // target workgroups of the parallel filter

struct TopkArgs {
  const float* scores;
  int64_t n_rows;
  int32_t row_len;
  int64_t row_stride;
  ValidLen vl;
  int32_t k;
  int32_t* idx;
  // parallel filter: part p of row r keeps its survivors in
  // pkey/pidx[(r * nparts + p) * kCap ...] and their number in pcnt[r * nparts + p]
  int nparts;
  int part_len;  // multiple of kPartLen
  uint32_t* pkey;
  int32_t* pidx;
  uint32_t* pcnt;
};

// LDS of a row workgroup: the candidate list and the radix histogram.
struct TopkSmem {
  uint32_t ckey[kCap];
  int32_t cidx[kCap];
  uint32_t hist[kBins];
  uint32_t wsum[kNT / 64];
  uint32_t wmin[kNT / 64];
  uint32_t wmax[kNT / 64];
  uint32_t sel[4];
};
// LDS of a part workgroup: the sample only (several fit on one CU).
struct SampleSmem {
  uint32_t ckey[kNS];
  uint32_t hist[kBins];
  uint32_t wsum[kNT / 64];
  uint32_t wmin[kNT / 64];
  uint32_t wmax[kNT / 64];
  uint32_t sel[4];
};

// Exclusive block-wide scan of one value per thread; returns the exclusive
// prefix and the total.  Two barriers.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
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

// Block-wide min and max of one pair per thread (two barriers).
template <class SM>
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SM& sm, uint32_t* mn_out,
                                             uint32_t* mx_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_min_max(mn, mx);
  if (lane == 0) {
    sm.wmin[wave] = mn;
    sm.wmax[wave] = mx;
  }
  __syncthreads();
  uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    a = min(a, sm.wmin[w]);
    b = max(b, sm.wmax[w]);
  }
  __syncthreads();
  *mn_out = a;
  *mx_out = b;
}

// Radix select: the k-th largest key T over the keys the visitor hands to its
// callback (this thread's keys), and the number k_rem of keys equal to T that
// belong to the top k.  Requires 1 <= k <= number of keys.  The digits are
// taken from r = key - min over the keys' own range (12 bits at a time from
// the top of max - min), so the histogram bins are spread over the values
// actually present.  After the first digit the keys of the selected bin are
// usually few: up to kRankList of them are ranked directly in LDS instead of
// running the remaining digit passes.
constexpr uint32_t kRankList = 512;

template <class Visit, class SM>
__device__ __forceinline__ void radix_select(uint32_t k, Visit visit, SM& sm, uint32_t* T_out,
                                             uint32_t* krem_out) {
  const int t = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  visit([&](uint32_t u) {
    lo = min(lo, u);
    hi = max(hi, u);
  });
  uint32_t base, top;
  block_minmax(lo, hi, sm, &base, &top);
  const uint32_t range = top - base;
  int s_hi = range == 0u ? 0 : 32 - __clz(range);  // every r = key - base is < 2^s_hi
  uint32_t P = 0, krem = k;                         // selected value of r >> s_hi
  while (s_hi > 0) {
    const int s_lo = s_hi > 12 ? s_hi - 12 : 0;
    const uint32_t dmask = (1u << (s_hi - s_lo)) - 1u;
#pragma unroll
    for (int e = 0; e < kBins / kNT; ++e) sm.hist[t * (kBins / kNT) + e] = 0u;
    if (t == 0) sm.sel[2] = 0u;
    __syncthreads();
    visit([&](uint32_t u) {
      const uint32_t r = u - base;
      if ((uint32_t)((uint64_t)r >> s_hi) == P) atomicAdd(&sm.hist[(r >> s_lo) & dmask], 1u);
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
          sm.sel[0] = (P << (s_hi - s_lo)) | (uint32_t)(t * (kBins / kNT) + e);
          sm.sel[1] = krem - cum;
          sm.sel[3] = c[e];  // keys in the selected bin
        }
        cum += c[e];
      }
    }
    __syncthreads();
    P = sm.sel[0];
    krem = sm.sel[1];
    const uint32_t nbin = sm.sel[3];
    __syncthreads();
    s_hi = s_lo;
    if (s_hi > 0 && nbin <= kRankList) {
      // the selected bin's keys into a list (hist reused), then rank them
      visit([&](uint32_t u) {
        const uint32_t r = u - base;
        if ((r >> s_hi) == P) sm.hist[atomicAdd(&sm.sel[2], 1u)] = u;
      });
      __syncthreads();
      if ((uint32_t)t < nbin) {
        const uint32_t x = sm.hist[t];
        uint32_t g = 0, e = 0;
        for (uint32_t i = 0; i < nbin; ++i) {
          const uint32_t y = sm.hist[i];
          g += y > x;
          e += y == x;
        }
        if (g < krem && krem <= g + e) {  // x is the krem-th largest of the bin
          sm.sel[0] = x;
          sm.sel[1] = krem - g;
        }
      }
      __syncthreads();
      *T_out = sm.sel[0];
      *krem_out = sm.sel[1];
      __syncthreads();
      return;
    }
  }
  *T_out = base + P;
  *krem_out = krem;
}

// Threshold t0 from a sample of the row (n > kCap): keys >= t0 include, in
// expectation, about twice the top K.  Every workgroup of a row computes the
// same value (same sample, same arithmetic).
template <class SM>
__device__ __forceinline__ uint32_t sample_threshold(const float* srow, int n, uint32_t kk, SM& sm) {
  const int t = threadIdx.x;
  // run r covers keys [base_r, base_r + kRunLen); runs are evenly spread.
  // Fixed trip count: all of a thread's loads are in flight together.
  float v[kNS / kNT];
#pragma unroll
  for (int e = 0; e < kNS / kNT; ++e) {
    const int s = t + e * kNT, r = s / kRunLen, o = s - r * kRunLen;
    const int base = (int)((int64_t)r * (n - kRunLen) / (kRuns - 1));
    v[e] = srow[base + o];
  }
#pragma unroll
  for (int e = 0; e < kNS / kNT; ++e) sm.ckey[t + e * kNT] = order_key(v[e]);
  __syncthreads();
  // rank in the sample: twice the expected count of top-K keys, plus slack
  int64_t q = ((int64_t)kk * kNS + n - 1) / n * 2 + 32;
  if (q > kNS) q = kNS;
  uint32_t T0, r0;
  radix_select((uint32_t)q, [&](auto f) {
#pragma unroll
    for (int e = 0; e < kNS / kNT; ++e) f(sm.ckey[t + e * kNT]);
  }, sm, &T0, &r0);
  return T0;  // the q-th largest sample key: keys >= t0 include the top q of the sample
}

// Steps 2 and 3 over the C candidates in sm.ckey / sm.cidx (index order).
__device__ __forceinline__ void select_candidates(uint32_t C, uint32_t kk, int32_t* out, TopkSmem& sm) {
  const int t = threadIdx.x;
  // thread t owns a contiguous run of candidates; an odd run length keeps the
  // lanes' strided LDS reads on distinct banks
  const uint32_t per = ((C + kNT - 1) / kNT) | 1u;
  const uint32_t c0 = min(C, t * per), c1 = min(C, c0 + per);
  uint32_t T, krem;
  radix_select(kk, [&](auto f) {
    for (uint32_t c = c0; c < c1; ++c) f(sm.ckey[c]);
  }, sm, &T, &krem);
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
}

// this thread's kEPT consecutive keys of segment sg (0 past the row end)
// A row of at most kCap keys is its own candidate list: coalesced loads
// (thread t takes keys t, t + kNT, ...; clamped indices, so all are in
// flight together) stored at their index in LDS (consecutive lanes,
// consecutive words: no bank conflicts), then select_candidates.
__device__ __forceinline__ void select_short_row(const float* srow, int n, uint32_t kk, int32_t* out,
                                                 TopkSmem& sm) {
  const int t = threadIdx.x;
  constexpr int kB = kCap / kNT;  // 12 loads per thread
  float v[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) v[e] = srow[min(t + e * kNT, n - 1)];
#pragma unroll
  for (int e = 0; e < kB; ++e)
    if (t + e * kNT < n) {
      sm.ckey[t + e * kNT] = order_key(v[e]);
      sm.cidx[t + e * kNT] = t + e * kNT;
    }
  __syncthreads();
  select_candidates((uint32_t)n, kk, out, sm);
}

__device__ __forceinline__ void load_seg(const float* srow, int n, bool vec, int sg, uint32_t (&keys)[kEPT]) {
  const int j0 = sg * kSeg + threadIdx.x * kEPT;
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
}

// Fallback: radix select and compaction over the whole row.
__device__ __forceinline__ void select_whole_row(const float* srow, int n, bool vec, uint32_t kk, int32_t* out,
                                                 TopkSmem& sm) {
  const int t = threadIdx.x;
  const int nseg = (n + kSeg - 1) / kSeg;
  uint32_t T, krem;
  radix_select(kk, [&](auto f) {
    for (int sg = 0; sg < nseg; ++sg) {
      uint32_t keys[kEPT];
      load_seg(srow, n, vec, sg, keys);
      const int j0 = sg * kSeg + t * kEPT;
#pragma unroll
      for (int e = 0; e < kEPT; ++e)
        if (j0 + e < n) f(keys[e]);
    }
  }, sm, &T, &krem);
  uint32_t g_base = 0, e_base = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[kEPT];
    load_seg(srow, n, vec, sg, keys);
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
  if (n <= kCap) {  // the whole row is the candidate list: no filter
    select_short_row(srow, n, kk, out, sm);
    return;
  }
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  const int nseg = (n + kSeg - 1) / kSeg;

  // ---- 1. threshold from a sample (rows longer than the capacity)
  const uint32_t t0 = n > kCap ? sample_threshold(srow, n, kk, sm) : 0u;

  // ---- filter: keys >= t0 into LDS, index order
  uint32_t C = 0;  // candidates kept (block-uniform)
  bool fits = true;
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[kEPT];
    load_seg(srow, n, vec, sg, keys);
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
  if (fits && C >= kk)
    select_candidates(C, kk, out, sm);
  else
    select_whole_row(srow, n, vec, kk, out, sm);
}

// Parallel filter, workgroup (row, part): the survivors (keys >= t0) of keys
// [p * part_len, (p + 1) * part_len) of a row longer than kCap, in index
// order, and their number (which may exceed kCap; then only kCap are kept).
__global__ __launch_bounds__(kNT) void topk_part_kernel(TopkArgs a) {
  __shared__ SampleSmem sm;
  const int64_t row = blockIdx.x / a.nparts;
  const int p = blockIdx.x - (int)(row * a.nparts);
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  if (n <= a.k || n <= kCap) return;  // the select kernel takes the row whole
  const float* srow = a.scores + row * a.row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  const uint32_t t0 = sample_threshold(srow, n, kk, sm);
  const int64_t slot = row * a.nparts + p;
  uint32_t* okey = a.pkey + slot * kCap;
  int32_t* oidx = a.pidx + slot * kCap;
  const int pend = min(n, (p + 1) * a.part_len);
  uint32_t C = 0;
  for (int j0 = p * a.part_len + 4 * t, jb = p * a.part_len; jb < pend; j0 += kPartLen, jb += kPartLen) {
    uint32_t keys[4];
    if (vec && j0 + 4 <= pend) {
      const float4 x = *reinterpret_cast<const float4*>(srow + j0);
      keys[0] = order_key(x.x);
      keys[1] = order_key(x.y);
      keys[2] = order_key(x.z);
      keys[3] = order_key(x.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = (j0 + e < pend) ? order_key(srow[j0 + e]) : 0u;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt += (j0 + e < pend && keys[e] >= t0);
    uint32_t tot;
    uint32_t off = C + block_scan(cnt, sm.wsum, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j0 + e < pend && keys[e] >= t0) {
        if (off < (uint32_t)kCap) {
          okey[off] = keys[e];
          oidx[off] = j0 + e;
        }
        ++off;
      }
    }
    C += tot;
    if (C > (uint32_t)kCap) break;  // the row will fall back to the whole-row select
  }
  if (t == 0) a.pcnt[slot] = C;
}

// Select after the parallel filter: one workgroup per row.
__global__ __launch_bounds__(kNT) void topk_select_kernel(TopkArgs a) {
  __shared__ TopkSmem sm;
  __shared__ uint32_t pstart[kMaxParts + 1];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  int32_t* out = a.idx + row * a.k;
  if (n <= a.k) {
    for (int x = t; x < a.k; x += kNT) out[x] = x < n ? x : -1;
    return;
  }
  const float* srow = a.scores + row * a.row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  if (n <= kCap) {  // the whole row is the candidate list
    select_short_row(srow, n, kk, out, sm);
    return;
  }
  if (t < 64) {  // one lane per part (nparts <= 64): counts, then an exclusive scan
    const uint32_t c = t < a.nparts ? a.pcnt[row * a.nparts + t] : 0u;
    const uint32_t x = wave_inclusive_scan(c);
    const bool ok = __builtin_amdgcn_ballot_w64(c > (uint32_t)kCap) == 0;
    if (t < a.nparts) pstart[t] = x - c;
    if (t == 63) pstart[a.nparts] = ok ? x : 0xFFFFFFFFu;
  }
  __syncthreads();
  const uint32_t C = pstart[a.nparts];
  if (C <= (uint32_t)kCap && C >= kk) {
    // part-major copy: tpp threads per part move its survivors to their
    // place in the concatenated list (part order); the first kU rounds are
    // unrolled with clamped indices, so those loads are all in flight
    // together, and a part with more survivors finishes in a loop
    const int tpp = kNT / a.nparts;
    const int pp = t / tpp, r = t - pp * tpp;
    if (pp < a.nparts) {
      const uint32_t c0 = pstart[pp], cnt = pstart[pp + 1] - c0;
      const int64_t base = (row * a.nparts + pp) * kCap;
      constexpr int kU = 8;
      uint32_t kv[kU];
      int32_t iv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = min((uint32_t)(r + u * tpp), cnt > 0u ? cnt - 1u : 0u);
        kv[u] = a.pkey[base + i];
        iv[u] = a.pidx[base + i];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = r + u * tpp;
        if (i < cnt) {
          sm.ckey[c0 + i] = kv[u];
          sm.cidx[c0 + i] = iv[u];
        }
      }
      for (uint32_t i = r + kU * tpp; i < cnt; i += tpp) {
        sm.ckey[c0 + i] = a.pkey[base + i];
        sm.cidx[c0 + i] = a.pidx[base + i];
      }
    }
    __syncthreads();
    select_candidates(C, kk, out, sm);
  } else {
    select_whole_row(srow, n, vec, kk, out, sm);
  }
}

int topk_parts(int64_t n_rows, int32_t row_len) {
  if (n_rows <= 0 || n_rows >= kPartRows || row_len <= kCap) return 1;
  int np = (int)((kPartWGs + n_rows - 1) / n_rows);
  const int by_len = (row_len + kPartLen - 1) / kPartLen;
  if (np > by_len) np = by_len;
  if (np > kMaxParts) np = kMaxParts;
  return np < 2 ? 1 : np;
}

int topk_part_len(int32_t row_len, int np) {
  const int per = (row_len + np - 1) / np;
  return (per + kPartLen - 1) / kPartLen * kPartLen;
}

}  // namespace

size_t topk_ws_bytes(int64_t n_rows, int32_t row_len, int32_t /*k*/) {
  const int np = topk_parts(n_rows, row_len);
  if (np == 1) return 0;
  const size_t slots = (size_t)n_rows * np;
  return align_up(slots * kCap * sizeof(uint32_t)) * 2 + align_up(slots * sizeof(uint32_t));
}

hipError_t launch_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                       const ValidLen& vl, int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  TopkArgs a{};
  a.scores = scores;
  a.n_rows = n_rows;
  a.row_len = row_len;
  a.row_stride = row_stride;
  a.vl = vl;
  a.k = k;
  a.idx = idx;
  a.nparts = topk_parts(n_rows, row_len);
  TraceScope ts(st, "topk");
  if (a.nparts == 1) {
    topk_row_kernel<<<(unsigned)n_rows, kNT, 0, st>>>(a);
    return hipGetLastError();
  }
  const size_t slots = (size_t)n_rows * a.nparts;
  unsigned char* c = static_cast<unsigned char*>(ws);
  a.pkey = reinterpret_cast<uint32_t*>(c);
  c += align_up(slots * kCap * sizeof(uint32_t));
  a.pidx = reinterpret_cast<int32_t*>(c);
  c += align_up(slots * kCap * sizeof(uint32_t));
  a.pcnt = reinterpret_cast<uint32_t*>(c);
  a.part_len = topk_part_len(row_len, a.nparts);
  topk_part_kernel<<<(unsigned)slots, kNT, 0, st>>>(a);
  topk_select_kernel<<<(unsigned)n_rows, kNT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hys
