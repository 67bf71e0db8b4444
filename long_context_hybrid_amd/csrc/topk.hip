// Top-K selection over float32 score rows, bit-exact and deterministic.
//
// Rule (Baidu article, "Fine-Grained Sparse Attention: Indexer + Top-K": keep
// the K highest-scoring positions; ties and output order are fixed here): the
// float bits are mapped to an order-preserving 32-bit key; the K largest keys
// win, lower index first among equal keys; the winners are written in
// ascending index order, padded with -1 when a row has fewer than K
// candidates.
//
// One workgroup per row, in one of two sizes (TopkCfg): many rows (prefill:
// one row per (KV group, 64-query block)) run in 256-thread workgroups, four
// per CU, so that the rows' barrier-separated phases overlap; few rows run in
// 1024-thread workgroups.  When there are few long rows (decode: a handful of
// rows of the whole context) the candidate filter of step 1 is spread over
// `nparts` workgroups per row, each writing the survivors of its part of the
// row, in index order, to its own workspace region; a second kernel
// concatenates the regions in part order and runs steps 2 and 3.  Every form
// selects exactly the same indices.
//
// 1. Candidate filter.  A row longer than the LDS candidate capacity is first
//    sampled (evenly spread runs of 64 keys); a radix select on the sample
//    gives a threshold t0, the sample key whose rank is a fixed multiple of
//    the expected rank of the K-th largest key.  One pass over the row keeps
//    every key >= t0, in index order, in LDS.  If at least K keys survive,
//    the exact top K are among them (every key outside is below t0, hence
//    below the K-th largest), so the result is exact whatever the sample
//    was; otherwise, or if too many survive, the row falls back to a radix
//    select over the whole row.
// 2. Exact select: radix select of the K-th largest key T over an LDS
//    histogram, with digits of (key - min) taken over the range the keys
//    actually span.
// 3. Index-order compaction with one block-wide scan:
//      position(j) = #{j' < j : key > T} + min(#{j' < j : key == T}, k_rem)
//    where k_rem is the number of keys equal to T that belong to the top K,
//    so the output is sorted without a sort.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kRunLen = 64;        // sample: runs of kRunLen consecutive keys
constexpr int kPartRows = 256;     // rows below which long rows are filtered in parts
constexpr int kMaxParts = 64;
constexpr int kPartWGs = 512;      // target workgroups of the parallel filter

// Sizes of one row workgroup.
template <int NT_, int CAP_, int DIGIT_, int NC_, int NS_LONG_, int QF4_, int QA_>
struct TopkCfg {
  static constexpr int NT = NT_;        // threads
  static constexpr int EPT = 16;        // row elements per thread per segment
  static constexpr int SEG = NT * EPT;
  static constexpr int CAP = CAP_;      // candidate capacity (LDS)
  static constexpr int DIGIT = DIGIT_;  // radix digit bits
  static constexpr int BINS = 1 << DIGIT;
  // histogram copies: thread t adds to copy t % NC (bin b, copy c at
  // b * NC + c), so the equal bins of one instruction's lanes fall on
  // different banks (a row's bulk often shares one bin)
  static constexpr int NC = NC_;
  // sample keys: NS, or NS_LONG for rows longer than LONG_ROW (a larger
  // sample keeps the survivor count's spread small when the expected sample
  // rank of the K-th key is small)
  static constexpr int NS = 4096;
  static constexpr int NS_LONG = NS_LONG_;
  static constexpr int LONG_ROW = 65536;
  // sample rank of the threshold: QF4 / 4 x the expected sample rank of the
  // K-th largest key, plus QA
  static constexpr int QF4 = QF4_, QA = QA_;
  // after the first digit, a selected bin of at most RANKLIST keys is ranked
  // directly (one key per thread)
  static constexpr uint32_t RANKLIST = NT < 512 ? NT : 512;
  static constexpr int PART_LEN = NT * 4;  // parallel filter: keys per part pass
  static_assert(NS <= NS_LONG && NS_LONG <= 2 * CAP && NS % NT == 0 && NS_LONG % NT == 0 && CAP % NT == 0 &&
                    BINS % NT == 0 && NS % kRunLen == 0 && NS_LONG % kRunLen == 0,
                "top-K sizes");
};
// few rows, and the decode-time parts: 12288 candidates, 12-bit digits,
// threshold at twice the expected rank of a 4096-key sample plus 32
using BigCfg = TopkCfg<1024, 12288, 12, 1, 4096, 8, 32>;
// many rows: 4096 candidates (37 KB of LDS: four workgroups per CU), 8-bit
// digits over four histogram copies, threshold at 1.5 times the expected
// sample rank, no slack: for K = 2048 the survivors (about 3072) stay between
// K and the capacity by more than four standard deviations of the sample's
// rank statistics (relative spread 1 / sqrt(rank)) up to 64K keys per row
// with 4096 sample keys and up to 128K with 8192
using SmallCfg = TopkCfg<256, 4096, 8, 4, 8192, 6, 0>;
constexpr int64_t kSmallRows = 384;  // rows from which SmallCfg is used (with K <= its capacity / 2)

struct TopkArgs {
  const float* scores;
  int64_t n_rows;
  int32_t row_len;
  int64_t row_stride;
  ValidLen vl;
  int32_t k;
  int32_t* idx;
  // parallel filter (BigCfg): part p of row r keeps its survivors in
  // pkey/pidx[(r * nparts + p) * slot_cap ...] and their number in
  // pcnt[r * nparts + p]
  int nparts;
  int part_len;  // multiple of PART_LEN
  int slot_cap;  // min(CAP, part_len): a part never has more survivors than keys
  uint32_t* pkey;
  int32_t* pidx;
  uint32_t* pcnt;
};

// LDS of a row workgroup: the candidate list (or, before the filter, the
// sample) and the radix histogram.
template <class C>
struct RowSmem {
  union {
    struct {
      uint32_t ckey[C::CAP];
      int32_t cidx[C::CAP];
    };
    uint32_t samp[2 * C::CAP];
  };
  uint32_t hist[C::BINS * C::NC];
  uint32_t wsum[2 * (C::NT / 64)];  // two scan buffers, used alternately by loops of scans
  uint32_t wmin[C::NT / 64];
  uint32_t wmax[C::NT / 64];
  uint32_t sel[4];
};
// LDS of a part workgroup: the sample only (several fit on one CU).
template <class C>
struct SampleSmem {
  uint32_t samp[C::NS_LONG];
  uint32_t hist[C::BINS * C::NC];
  uint32_t wsum[2 * (C::NT / 64)];
  uint32_t wmin[C::NT / 64];
  uint32_t wmax[C::NT / 64];
  uint32_t sel[4];
};

// Exclusive block-wide scan of one value per thread; returns the exclusive
// prefix and the total.  One barrier: the C::NT / 64 words at wsum may be
// written again only after another barrier (loops of scans alternate
// between two buffers, so the next scan's own barrier is that barrier).
template <class C>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < C::NT / 64; ++w) {
    const uint32_t s = wsum[w];
    pre += (w < wave) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return pre + x - v;
}

// Clears the radix histogram (and the rank-list counter) ahead of a radix
// select; the caller's next barrier publishes it.
template <class C, class SM>
__device__ __forceinline__ void hist_clear(SM& sm) {
  constexpr int E = C::BINS * C::NC / C::NT;
#pragma unroll
  for (int e = 0; e < E; ++e) sm.hist[threadIdx.x * E + e] = 0u;
  if (threadIdx.x == 0) sm.sel[2] = 0u;
}

// Block-wide min and max of one pair per thread (two barriers).
template <class C, class SM>
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
  for (int w = 0; w < C::NT / 64; ++w) {
    a = min(a, sm.wmin[w]);
    b = max(b, sm.wmax[w]);
  }
  __syncthreads();
  *mn_out = a;
  *mx_out = b;
}

// The bounds of a key set held in registers while the keys are being stored
// to LDS: each wave's minimum and maximum go to LDS with the keys, so the
// barrier that publishes the keys publishes the bounds too (range_read after
// it), instead of a separate min/max pass with two barriers of its own.
template <class SM>
__device__ __forceinline__ void range_publish(uint32_t mn, uint32_t mx, SM& sm) {
  wave_min_max(mn, mx);
  if ((threadIdx.x & 63) == 0) {
    sm.wmin[threadIdx.x >> 6] = mn;
    sm.wmax[threadIdx.x >> 6] = mx;
  }
}
template <class C, class SM>
__device__ __forceinline__ void range_read(SM& sm, uint32_t* base, uint32_t* top) {
  uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
  for (int w = 0; w < C::NT / 64; ++w) {
    a = min(a, sm.wmin[w]);
    b = max(b, sm.wmax[w]);
  }
  *base = a;
  *top = b;
}

// Radix select: the k-th largest key T over the keys the visitor hands to its
// callback (this thread's keys), and the number k_rem of keys equal to T that
// belong to the top k.  Requires 1 <= k <= number of keys and base <= every
// key <= top.  The digits are taken from r = key - base over the keys' own
// range (C::DIGIT bits at a time from the top of top - base), so the
// histogram bins are spread over the values actually present.  After the
// first digit the keys of the selected bin are usually few: up to
// C::RANKLIST of them are ranked directly in LDS instead of running the
// remaining digit passes.  With `cleared`, the caller has cleared the
// histogram (hist_clear) before the barrier that published the keys.
// Barriers: three per digit (histogram, scan, selected bin) plus one to
// clear the histogram for every digit after the first; two for the rank
// list.  No barrier follows the last LDS read, so the caller must pass one
// before writing sm.hist or sm.sel[0], sm.sel[1] again.
template <class C, class Visit, class SM>
__device__ __forceinline__ void radix_select_in(uint32_t k, uint32_t base, uint32_t top, Visit visit, SM& sm,
                                                uint32_t* T_out, uint32_t* krem_out, bool cleared) {
  const int t = threadIdx.x;
  const uint32_t range = top - base;
  int s_hi = range == 0u ? 0 : 32 - __clz(range);  // every r = key - base is < 2^s_hi
  uint32_t P = 0, krem = k;                         // selected value of r >> s_hi
  while (s_hi > 0) {
    const int s_lo = s_hi > C::DIGIT ? s_hi - C::DIGIT : 0;
    const uint32_t dmask = (1u << (s_hi - s_lo)) - 1u;
    constexpr int BPT = C::BINS / C::NT;  // bins per thread
    if (!cleared) {
      // the previous digit's histogram reads and rank-list counter use all
      // ended before its scan barrier
      hist_clear<C>(sm);
      __syncthreads();
    }
    cleared = false;
    visit([&](uint32_t u) {
      const uint32_t r = u - base;
      if ((uint32_t)((uint64_t)r >> s_hi) == P) atomicAdd(&sm.hist[((r >> s_lo) & dmask) * C::NC + (t % C::NC)], 1u);
    });
    __syncthreads();
    // thread t owns bins [BPT t, BPT (t + 1)); count keys in higher bins
    uint32_t c[BPT];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      c[e] = 0u;
#pragma unroll
      for (int x = 0; x < C::NC; ++x) c[e] += sm.hist[(t * BPT + e) * C::NC + x];
      tot += c[e];
    }
    uint32_t all;
    const uint32_t below = block_scan<C>(tot, sm.wsum, &all);
    const uint32_t above = all - below - tot;
    if (above < krem && krem <= above + tot) {
      uint32_t cum = above;
#pragma unroll
      for (int e = BPT - 1; e >= 0; --e) {
        if (cum < krem && krem <= cum + c[e]) {
          sm.sel[0] = (P << (s_hi - s_lo)) | (uint32_t)(t * BPT + e);
          sm.sel[1] = krem - cum;
          sm.sel[3] = c[e];  // keys in the selected bin
        }
        cum += c[e];
      }
    }
    __syncthreads();
    // no barrier after these reads: the next writes of sel[0], sel[1] and
    // sel[3] come after further barriers, and sel[2] and the histogram (read
    // before the scan's barrier) are other words
    P = sm.sel[0];
    krem = sm.sel[1];
    const uint32_t nbin = sm.sel[3];
    s_hi = s_lo;
    if (s_hi > 0 && nbin <= C::RANKLIST) {
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
      return;
    }
  }
  *T_out = base + P;
  *krem_out = krem;
}

// Radix select over keys whose bounds are not known yet: a min/max pass first.
template <class C, class Visit, class SM>
__device__ __forceinline__ void radix_select(uint32_t k, Visit visit, SM& sm, uint32_t* T_out,
                                             uint32_t* krem_out) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  visit([&](uint32_t u) {
    lo = min(lo, u);
    hi = max(hi, u);
  });
  uint32_t base, top;
  block_minmax<C>(lo, hi, sm, &base, &top);
  radix_select_in<C>(k, base, top, visit, sm, T_out, krem_out, false);
}

// Threshold t0 from an NS-key sample of the row (n > C::CAP): keys >= t0
// include, in expectation, C::QF4 / 4 times the top K (plus the slack C::QA).
// Every workgroup of a row computes the same value (same sample, same
// arithmetic).
template <class C, int NS, class SM>
__device__ __forceinline__ uint32_t sample_threshold(const float* srow, int n, uint32_t kk, SM& sm) {
  const int t = threadIdx.x;
  constexpr int RUNS = NS / kRunLen;
  // run r covers keys [base_r, base_r + kRunLen); runs are evenly spread.
  // Fixed trip count: all of a thread's loads are in flight together.
  constexpr int SPT = NS / C::NT;
  float v[SPT];
#pragma unroll
  for (int e = 0; e < SPT; ++e) {
    const int s = t + e * C::NT, r = s / kRunLen, o = s - r * kRunLen;
    const int base = (int)((int64_t)r * (n - kRunLen) / (RUNS - 1));
    v[e] = srow[base + o];
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int e = 0; e < SPT; ++e) {
    const uint32_t u = order_key(v[e]);
    sm.samp[t + e * C::NT] = u;
    mn = min(mn, u);
    mx = max(mx, u);
  }
  range_publish(mn, mx, sm);
  hist_clear<C>(sm);
  __syncthreads();
  uint32_t base, top;
  range_read<C>(sm, &base, &top);
  // rank in the sample: a multiple of the expected count of top-K keys, plus slack
  int64_t q = ((int64_t)kk * NS + n - 1) / n * C::QF4 / 4 + C::QA;
  if (q > NS) q = NS;
  uint32_t T0, r0;
  radix_select_in<C>((uint32_t)q, base, top, [&](auto f) {
#pragma unroll
    for (int e = 0; e < SPT; ++e) f(sm.samp[t + e * C::NT]);
  }, sm, &T0, &r0, true);
  return T0;  // the q-th largest sample key: keys >= t0 include the top q of the sample
}

// Steps 2 and 3 over the nc candidates in sm.ckey / sm.cidx (index order),
// whose keys lie in [base, top]; the histogram was cleared before the
// barrier that published the candidates.
template <class C>
__device__ __forceinline__ void select_candidates(uint32_t nc, uint32_t kk, uint32_t base, uint32_t top, int32_t* out,
                                                  RowSmem<C>& sm) {
  const int t = threadIdx.x;
  // thread t owns a contiguous run of candidates; an odd run length keeps the
  // lanes' strided LDS reads on distinct banks
  const uint32_t per = ((nc + C::NT - 1) / C::NT) | 1u;
  const uint32_t c0 = min(nc, t * per), c1 = min(nc, c0 + per);
  uint32_t T, krem;
  radix_select_in<C>(kk, base, top, [&](auto f) {
    for (uint32_t c = c0; c < c1; ++c) f(sm.ckey[c]);
  }, sm, &T, &krem, true);
  uint32_t gt = 0, eq = 0;
  for (uint32_t c = c0; c < c1; ++c) {
    gt += sm.ckey[c] > T;
    eq += sm.ckey[c] == T;
  }
  // both counts in one scan: (greater << 16) | equal (at most C::CAP < 2^16 each)
  uint32_t tot;
  // (the radix select's last scan used buffer 0, with barriers since)
  const uint32_t pre = block_scan<C>((gt << 16) | eq, sm.wsum + C::NT / 64, &tot);
  uint32_t gb = pre >> 16, eb = pre & 0xFFFFu;
  for (uint32_t c = c0; c < c1; ++c) {
    const uint32_t u = sm.ckey[c];
    const bool is_gt = u > T, is_eq = u == T;
    const uint32_t p = gb + (is_gt ? min(eb, krem) : eb);
    if ((is_gt || (is_eq && eb < krem)) && p < kk) out[p] = sm.cidx[c];
    gb += is_gt;
    eb += is_eq;
  }
}

// A row of at most C::CAP keys is its own candidate list: coalesced loads
// (thread t takes keys t, t + NT, ...; clamped indices, so all are in flight
// together) stored at their index in LDS (consecutive lanes, consecutive
// words: no bank conflicts), then select_candidates.
template <class C>
__device__ __forceinline__ void select_short_row(const float* srow, int n, uint32_t kk, int32_t* out,
                                                 RowSmem<C>& sm) {
  const int t = threadIdx.x;
  constexpr int kB = C::CAP / C::NT;  // loads per thread
  float v[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) v[e] = srow[min(t + e * C::NT, n - 1)];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int e = 0; e < kB; ++e)
    if (t + e * C::NT < n) {
      const uint32_t u = order_key(v[e]);
      sm.ckey[t + e * C::NT] = u;
      sm.cidx[t + e * C::NT] = t + e * C::NT;
      mn = min(mn, u);
      mx = max(mx, u);
    }
  range_publish(mn, mx, sm);
  hist_clear<C>(sm);
  __syncthreads();
  uint32_t base, top;
  range_read<C>(sm, &base, &top);
  select_candidates<C>((uint32_t)n, kk, base, top, out, sm);
}

// this thread's C::EPT consecutive keys of segment sg (0 past the row end)
template <class C>
__device__ __forceinline__ void load_seg(const float* srow, int n, bool vec, int sg, uint32_t (&keys)[C::EPT]) {
  const int j0 = sg * C::SEG + threadIdx.x * C::EPT;
  if (vec && j0 + C::EPT <= n) {
#pragma unroll
    for (int e = 0; e < C::EPT; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(srow + j0 + e);
      keys[e] = order_key(x.x);
      keys[e + 1] = order_key(x.y);
      keys[e + 2] = order_key(x.z);
      keys[e + 3] = order_key(x.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < C::EPT; ++e) keys[e] = (j0 + e < n) ? order_key(srow[j0 + e]) : 0u;
  }
}

// Fallback: radix select and compaction over the whole row.
template <class C>
__device__ __forceinline__ void select_whole_row(const float* srow, int n, bool vec, uint32_t kk, int32_t* out,
                                                 RowSmem<C>& sm) {
  const int t = threadIdx.x;
  const int nseg = (n + C::SEG - 1) / C::SEG;
  uint32_t T, krem;
  radix_select<C>(kk, [&](auto f) {
    for (int sg = 0; sg < nseg; ++sg) {
      uint32_t keys[C::EPT];
      load_seg<C>(srow, n, vec, sg, keys);
      const int j0 = sg * C::SEG + t * C::EPT;
#pragma unroll
      for (int e = 0; e < C::EPT; ++e)
        if (j0 + e < n) f(keys[e]);
    }
  }, sm, &T, &krem);
  uint32_t g_base = 0, e_base = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[C::EPT];
    load_seg<C>(srow, n, vec, sg, keys);
    const int j0 = sg * C::SEG + t * C::EPT;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < C::EPT; ++e) {
      const bool in = j0 + e < n;
      gt += (in && keys[e] > T);
      eq += (in && keys[e] == T);
    }
    // both counts in one scan (at most C::SEG < 2^16 each per segment)
    uint32_t tot;
    const uint32_t pre = block_scan<C>((gt << 16) | eq, sm.wsum + (sg & 1) * (C::NT / 64), &tot);
    uint32_t gb = g_base + (pre >> 16), eb = e_base + (pre & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < C::EPT; ++e) {
      const bool in = j0 + e < n;
      const bool is_gt = in && keys[e] > T;
      const bool is_eq = in && keys[e] == T;
      const uint32_t p = gb + (is_gt ? min(eb, krem) : eb);
      if ((is_gt || (is_eq && eb < krem)) && p < kk) out[p] = j0 + e;
      gb += is_gt;
      eb += is_eq;
    }
    g_base += tot >> 16;
    e_base += tot & 0xFFFFu;
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void topk_row_kernel(TopkArgs a) {
  __shared__ RowSmem<C> sm;
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  int32_t* out = a.idx + row * a.k;
  if (n <= a.k) {  // every candidate is selected
    for (int x = t; x < a.k; x += C::NT) out[x] = x < n ? x : -1;
    return;
  }
  const float* srow = a.scores + row * a.row_stride;
  if (n <= C::CAP) {  // the whole row is the candidate list: no filter
    select_short_row<C>(srow, n, kk, out, sm);
    return;
  }
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  const int nseg = (n + C::SEG - 1) / C::SEG;

  // ---- 1. threshold from a sample (rows longer than the capacity)
  const uint32_t t0 = (C::NS_LONG > C::NS && n > C::LONG_ROW) ? sample_threshold<C, C::NS_LONG>(srow, n, kk, sm)
                                                              : sample_threshold<C, C::NS>(srow, n, kk, sm);
  __syncthreads();  // the sample's LDS becomes the candidate list

  // ---- filter: keys >= t0 into LDS, index order
  uint32_t nc = 0;  // candidates kept (block-uniform)
  bool fits = true;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;  // bounds of this thread's kept keys
  for (int sg = 0; sg < nseg; ++sg) {
    uint32_t keys[C::EPT];
    load_seg<C>(srow, n, vec, sg, keys);
    const int j0 = sg * C::SEG + t * C::EPT;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < C::EPT; ++e) cnt += (j0 + e < n && keys[e] >= t0);
    uint32_t tot;
    uint32_t off = nc + block_scan<C>(cnt, sm.wsum + (sg & 1) * (C::NT / 64), &tot);
#pragma unroll
    for (int e = 0; e < C::EPT; ++e) {
      if (j0 + e < n && keys[e] >= t0) {
        if (off < (uint32_t)C::CAP) {
          sm.ckey[off] = keys[e];
          sm.cidx[off] = j0 + e;
        }
        ++off;
        mn = min(mn, keys[e]);
        mx = max(mx, keys[e]);
      }
    }
    nc += tot;
    if (nc > (uint32_t)C::CAP) {
      fits = false;
      break;
    }
  }
  range_publish(mn, mx, sm);
  hist_clear<C>(sm);  // the threshold's radix select ended before the barrier after it
  __syncthreads();
  if (fits && nc >= kk) {
    uint32_t base, top;
    range_read<C>(sm, &base, &top);
    select_candidates<C>(nc, kk, base, top, out, sm);
  } else
    select_whole_row<C>(srow, n, vec, kk, out, sm);
}

// Parallel filter (BigCfg), workgroup (row, part): the survivors (keys >= t0)
// of keys [p * part_len, (p + 1) * part_len) of a row longer than the
// capacity, in index order, and their number (which may exceed the capacity;
// then only CAP are kept).
__global__ __launch_bounds__(BigCfg::NT) void topk_part_kernel(TopkArgs a) {
  using C = BigCfg;
  __shared__ SampleSmem<C> sm;
  const int64_t row = blockIdx.x / a.nparts;
  const int p = blockIdx.x - (int)(row * a.nparts);
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  if (n <= a.k || n <= C::CAP) return;  // the select kernel takes the row whole
  const float* srow = a.scores + row * a.row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  const int pend = min(n, (p + 1) * a.part_len);
  // the part's first PART_LEN keys are loaded before the threshold is formed,
  // so their round trip overlaps the sample's
  const int jf = p * a.part_len + 4 * t;
  const bool first_vec = vec && jf + 4 <= pend;
  float4 first = make_float4(0.f, 0.f, 0.f, 0.f);
  if (first_vec) first = *reinterpret_cast<const float4*>(srow + jf);
  const uint32_t t0 = sample_threshold<C, C::NS>(srow, n, kk, sm);
  const int64_t slot = row * a.nparts + p;
  uint32_t* okey = a.pkey + slot * a.slot_cap;
  int32_t* oidx = a.pidx + slot * a.slot_cap;
  uint32_t nc = 0;
  for (int j0 = p * a.part_len + 4 * t, jb = p * a.part_len, ps = 0; jb < pend;
       j0 += C::PART_LEN, jb += C::PART_LEN, ++ps) {
    uint32_t keys[4];
    if (vec && j0 + 4 <= pend) {
      const float4 x = j0 == jf ? first : *reinterpret_cast<const float4*>(srow + j0);
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
    uint32_t off = nc + block_scan<C>(cnt, sm.wsum + (ps & 1) * (C::NT / 64), &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j0 + e < pend && keys[e] >= t0) {
        if (off < (uint32_t)a.slot_cap) {
          okey[off] = keys[e];
          oidx[off] = j0 + e;
        }
        ++off;
      }
    }
    nc += tot;
    if (nc > (uint32_t)a.slot_cap) break;  // the row will fall back to the whole-row select
  }
  if (t == 0) a.pcnt[slot] = nc;
}

// Select after the parallel filter (BigCfg): one workgroup per row.
__global__ __launch_bounds__(BigCfg::NT) void topk_select_kernel(TopkArgs a) {
  using C = BigCfg;
  __shared__ RowSmem<C> sm;
  __shared__ uint32_t pstart[kMaxParts + 1];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = valid_len_of(a.vl, row);
  const uint32_t kk = (uint32_t)a.k;
  int32_t* out = a.idx + row * a.k;
  if (n <= a.k) {
    for (int x = t; x < a.k; x += C::NT) out[x] = x < n ? x : -1;
    return;
  }
  const float* srow = a.scores + row * a.row_stride;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  if (n <= C::CAP) {  // the whole row is the candidate list
    select_short_row<C>(srow, n, kk, out, sm);
    return;
  }
  // part-major copy below: tpp threads per part; its first kU rounds of
  // survivor loads are issued before the counts are known (indices clamped
  // to the part's workspace slot), so both round trips overlap
  const int tpp = C::NT / a.nparts;
  const int pp = t / tpp, r = t - pp * tpp;
  const int64_t base = (row * a.nparts + (pp < a.nparts ? pp : 0)) * a.slot_cap;
  constexpr int kU = 8;
  uint32_t kv[kU];
  int32_t iv[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = min(r + u * tpp, a.slot_cap - 1);
    kv[u] = a.pkey[base + i];
    iv[u] = a.pidx[base + i];
  }
  if (t < 64) {  // one lane per part (nparts <= 64): counts, then an exclusive scan
    const uint32_t c = t < a.nparts ? a.pcnt[row * a.nparts + t] : 0u;
    const uint32_t x = wave_inclusive_scan(c);
    const bool ok = __builtin_amdgcn_ballot_w64(c > (uint32_t)a.slot_cap) == 0;
    if (t < a.nparts) pstart[t] = x - c;
    if (t == 63) pstart[a.nparts] = ok ? x : 0xFFFFFFFFu;
  }
  __syncthreads();
  const uint32_t nc = pstart[a.nparts];
  if (nc <= (uint32_t)C::CAP && nc >= kk) {
    // part-major copy: each part's survivors to their place in the
    // concatenated list (part order); a part with more survivors than the
    // first kU rounds finishes in a loop
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    if (pp < a.nparts) {
      const uint32_t c0 = pstart[pp], cnt = pstart[pp + 1] - c0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = r + u * tpp;
        if (i < cnt) {
          sm.ckey[c0 + i] = kv[u];
          sm.cidx[c0 + i] = iv[u];
          mn = min(mn, kv[u]);
          mx = max(mx, kv[u]);
        }
      }
      for (uint32_t i = r + kU * tpp; i < cnt; i += tpp) {
        const uint32_t u = a.pkey[base + i];
        sm.ckey[c0 + i] = u;
        sm.cidx[c0 + i] = a.pidx[base + i];
        mn = min(mn, u);
        mx = max(mx, u);
      }
    }
    range_publish(mn, mx, sm);
    hist_clear<C>(sm);
    __syncthreads();
    uint32_t lo, hi;
    range_read<C>(sm, &lo, &hi);
    select_candidates<C>(nc, kk, lo, hi, out, sm);
  } else {
    select_whole_row<C>(srow, n, vec, kk, out, sm);
  }
}

int topk_parts(int64_t n_rows, int32_t row_len) {
  if (n_rows <= 0 || n_rows >= kPartRows || row_len <= BigCfg::CAP) return 1;
  int np = (int)((kPartWGs + n_rows - 1) / n_rows);
  const int by_len = (row_len + BigCfg::PART_LEN - 1) / BigCfg::PART_LEN;
  if (np > by_len) np = by_len;
  if (np > kMaxParts) np = kMaxParts;
  return np < 2 ? 1 : np;
}

int topk_part_len(int32_t row_len, int np);
// survivors one part's workspace slot holds
int topk_slot_cap(int32_t row_len, int np) {
  const int pl = topk_part_len(row_len, np);
  return pl < BigCfg::CAP ? pl : BigCfg::CAP;
}

int topk_part_len(int32_t row_len, int np) {
  const int per = (row_len + np - 1) / np;
  return (per + BigCfg::PART_LEN - 1) / BigCfg::PART_LEN * BigCfg::PART_LEN;
}

// Many rows with K within half the small capacity: small workgroups.
bool topk_small(int64_t n_rows, int32_t k) { return n_rows >= kSmallRows && 2 * k <= SmallCfg::CAP; }

}  // namespace

size_t topk_ws_bytes(int64_t n_rows, int32_t row_len, int32_t /*k*/) {
  const int np = topk_parts(n_rows, row_len);
  if (np == 1) return 0;
  const size_t slots = (size_t)n_rows * np;
  const size_t cap = (size_t)topk_slot_cap(row_len, np);
  return align_up(slots * cap * sizeof(uint32_t)) * 2 + align_up(slots * sizeof(uint32_t));
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
  if (a.nparts == 1) {
    if (topk_small(n_rows, k))
      return launch("topk", topk_row_kernel<SmallCfg>, dim3((unsigned)n_rows), dim3(SmallCfg::NT), 0, st, a);
    return launch("topk", topk_row_kernel<BigCfg>, dim3((unsigned)n_rows), dim3(BigCfg::NT), 0, st, a);
  }
  const size_t slots = (size_t)n_rows * a.nparts;
  a.part_len = topk_part_len(row_len, a.nparts);
  a.slot_cap = topk_slot_cap(row_len, a.nparts);
  unsigned char* c = static_cast<unsigned char*>(ws);
  a.pkey = reinterpret_cast<uint32_t*>(c);
  c += align_up(slots * a.slot_cap * sizeof(uint32_t));
  a.pidx = reinterpret_cast<int32_t*>(c);
  c += align_up(slots * a.slot_cap * sizeof(uint32_t));
  a.pcnt = reinterpret_cast<uint32_t*>(c);
  hipError_t e = launch("topk_part", topk_part_kernel, dim3((unsigned)slots), dim3(BigCfg::NT), 0, st, a);
  if (e != hipSuccess) return e;
  return launch("topk_select", topk_select_kernel, dim3((unsigned)n_rows), dim3(BigCfg::NT), 0, st, a);
}

}  // namespace hys
