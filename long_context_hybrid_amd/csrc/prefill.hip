// Prefill path (q_len > 1) on gfx950 MFMA with LDS-staged 64-key tiles.
//
// Full layer, two sweeps (the importance score of a key needs each query's
// final log-sum-exp before any probability can be summed):
//   1. prefill_fwd:    causal flash attention per (KV group, query tile):
//                      O and the base-2 log-sum-exp of every (query, head) row;
//   2. prefill_scores: per (KV group, score block, key range): recompute the
//                      logits, P = 2^(logit2 - lse2) exactly, and sum P over
//                      the group's heads and the block's queries
//                      (score_block 64) or over the heads only (score_block 1).
// Sparse layer with 64-query score blocks (sparse_block): per (KV group,
// block, row chunk) the window keys of the block and then its selected keys
// are staged as 64-key tiles; each query row keeps a window state and a
// global state (online softmax) and the epilogue applies the sigmoid gate.
//
// Pages: the HySparse abstract (the full layer selects tokens for the sparse
// layers); the intelliparadigm article sections 2.2 and 3.1 (global branch on
// the shared KV at the TopK indices, 128-token window branch, gated sum,
// index sharing); the Baidu article's gather-then-attend pseudocode.
#include <type_traits>

#include "attn_tile.h"
#include "hys_internal.h"

namespace hys {

namespace {

// Launch shapes (waves per workgroup NW x row tiles per wave RTW; 16 rows per
// row tile), measured on MI355X at 32K: forward 8 x 2 (2 waves per SIMD) beats
// 4 x 4 by 1.3x, the second wave hiding the tile loads and the softmax; the
// score sweep (no O accumulators, one exp per product) prefers 4 x 4 (half
// the LDS reads per MFMA) by 1.2x; the sparse layer keeps two output states
// per row and fits only 8 x 1 without spills (4 x 2 is 1.25x slower).
#ifndef HYS_FWD_SHAPE
#define HYS_FWD_SHAPE 8, 2, 2
#endif
#ifndef HYS_SC_SHAPE
#define HYS_SC_SHAPE 4, 4
#endif
#ifndef HYS_SP_SHAPE
#define HYS_SP_SHAPE 8, 2
#endif
constexpr int kFwdShape[3] = {HYS_FWD_SHAPE};  // full layer, forward sweep (+ min waves per SIMD)
constexpr int kScShape[2] = {HYS_SC_SHAPE};    // full layer, score sweep
constexpr int kSpShape[2] = {HYS_SP_SHAPE};    // sparse layer (two output states per row)
constexpr int kFwdNW = kFwdShape[0], kFwdRTW = kFwdShape[1], kFwdWPE = kFwdShape[2];
constexpr int kScNW = kScShape[0], kScRTW = kScShape[1];
constexpr int kSpNW = kSpShape[0], kSpRTW = kSpShape[1];
constexpr int kIdxCh = 2048;                // sparse layer: selected indices staged in LDS per refill
// Both sweeps, bf16 with head_dim 128: tiles staged by LDS DMA into a ring
// of stages (the next tiles in flight while one is used).
#ifndef HYS_FWD_DMA
#define HYS_FWD_DMA 1
#endif
#ifndef HYS_SC_DMA
#define HYS_SC_DMA 1
#endif
// Ring stages: at step it, tiles it + 1 .. it + stages - 1 are in flight.
// Measured at 32K and 128K, two stages (one tile in flight, the DMA issued
// a whole tile step ahead) beat three by 1-1.5% in both sweeps; four were
// slower still.
#ifndef HYS_FWD_STAGES
#define HYS_FWD_STAGES 2
#endif
#ifndef HYS_SC_STAGES
#define HYS_SC_STAGES 2
#endif
constexpr int kFwdStages = HYS_FWD_STAGES;
constexpr int kScStages = HYS_SC_STAGES;
static_assert(kFwdStages >= 2 && kFwdStages <= 4 && kScStages >= 2 && kScStages <= 4, "ring stages");

// wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order) and its LDS reads are done
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// wait until the DMA of the ring's current tile has landed, while the PER
// instructions of each of the next min(N, rem) tiles may stay outstanding
template <int PER, int N>
__device__ __forceinline__ void wait_ring(int rem) {
  if constexpr (N == 0) {
    wait_vm_lgkm<0>();
  } else {
    if (rem >= N)
      wait_vm_lgkm<N * PER>();
    else
      wait_ring<PER, N - 1>(rem);
  }
}

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs_b, qs_t, qs_h, ks_b, ks_t, ks_h;
  int B, Tq, Tkv, Hq, Hkv, G;
  float sl2;
  int HW, QTW, NHC, nqt;  // heads and queries per workgroup, head chunks, query tiles
  void* out;
  float* lse;
  float* lse2;            // [B, Hq, Tq] base-2
  // scores
  float* scores;          // [B, Hkv, NB, Tkv]
  int SB, NB, nqb, nkr;   // score block, score blocks, query blocks of the kernel, key ranges
  // sparse
  const int32_t* idx;
  int k_top, window;
  GateRef gate;
  WinRef win;             // window branch keys/values (k == nullptr: the shared cache)
  int nrc;                // row chunks per score block
};

__device__ __forceinline__ int wave_min_int(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}

template <typename TR, int D>
__device__ __forceinline__ void load_q_frags(const PrefillArgs& a, int b, int i, int h, bool ok, int quad,
                                             typename TR::frag (&qf)[D / 32]) {
  const typename TR::storage* qrow =
      (const typename TR::storage*)a.q + (int64_t)b * a.qs_b + (int64_t)i * a.qs_t + (int64_t)h * a.qs_h;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = ok ? TR::load8(qrow + 32 * c + 8 * quad) : TR::zero8();
}

// ------------------------------------------------------------- sweep 1: fwd
// DMA: tiles come into a ring of LDS stages by global_load_lds (bf16,
// head_dim 128); otherwise through registers into one LDS tile.
template <typename TR, int D, int kNW, int kRTW, int kWPE, bool DMA>
__global__ __launch_bounds__(kNW * 64, kWPE) void prefill_fwd_kernel(PrefillArgs a) {
  constexpr int kNT = kNW * 64;
  using ST = typename TR::storage;
  using L = TileLayout<TR, D>;
  constexpr int KC = D / 32, DT = D / 16;
  static_assert(!DMA || (TR::kBytes == 2 && D == 128), "DMA staging is for bf16, head_dim 128");
  __shared__ __align__(16) unsigned char sm[DMA ? kFwdStages * DmaTile::kBytes : L::kBytes];
  __shared__ int kj[DMA ? 1 : kTK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, quad = lane >> 4;
  const int per_qt = a.B * a.Hkv * a.NHC;
  const int qt = a.nqt - 1 - (int)(blockIdx.x / per_qt);  // longest causal prefixes first
  const int rest = blockIdx.x - (blockIdx.x / per_qt) * per_qt;
  const int hc = rest % a.NHC, bg = rest / a.NHC;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int i0 = qt * a.QTW;

  typename TR::frag qf[kRTW][KC];
  int rpos[kRTW];
#pragma unroll
  for (int rt = 0; rt < kRTW; ++rt) {
    const int rho = (wave * kRTW + rt) * 16 + col;
    const int hl = rho / a.QTW, qi = rho - hl * a.QTW, i = i0 + qi;
    const bool ok = hl < a.HW && i < a.Tq;
    rpos[rt] = ok ? a.Tkv - a.Tq + i : -1;
    load_q_frags<TR, D>(a, b, i, g * a.G + hc * a.HW + hl, ok, quad, qf[rt]);
  }
  // smallest position among the wave's rows (rows past Tq are discarded): a
  // tile whose last key is not after it needs no causal mask
  int pmin = 0x7fffffff;
#pragma unroll
  for (int rt = 0; rt < kRTW; ++rt) pmin = rpos[rt] >= 0 ? min(pmin, rpos[rt]) : pmin;
  pmin = wave_min_int(pmin);
  const int last_i = min(i0 + a.QTW, a.Tq) - 1;
  const int pos_max = a.Tkv - a.Tq + last_i;
  const int nkt = pos_max / kTK + 1;
  const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const ST* vbase = (const ST*)a.v + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const int Tkv = a.Tkv;

  RowState<kRTW, D> st;
  st.reset();
  if constexpr (DMA) {
    // Ring of S = kFwdStages stages: at step it, tile it is used while
    // tiles it + 1 .. it + S - 1 are in flight.  Each wave waits for its own
    // DMA of tile it (the 2 * 16 / kNW instructions of each later tile may
    // remain outstanding); the barrier then makes every wave's part visible
    // and frees the stage of tile it - 1 for tile it + S - 1.  Keys past
    // kv_len are loaded from row kv_len - 1 and masked (they lie after every
    // position).
    constexpr int S = kFwdStages, P = S - 1;
    constexpr int kDmaPerTile = 2 * 16 / kNW;
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(kbase);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(vbase);
    const int last = Tkv - 1;
#pragma unroll
    for (int t = 0; t < P; ++t)
      if (t < nkt) dma_tile<kNW>(sm + t * DmaTile::kBytes, kb, vb, a.ks_t, t * kTK, last);
    // The Q fragments must be resident before the loop: the compiler cannot
    // count the ring's loads across steps and would otherwise wait for all
    // of them (vmcnt 0) at the first MFMA of every step.
#pragma unroll
    for (int rt = 0; rt < kRTW; ++rt)
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qf[rt][c]));
    int cur = 0;  // stage of tile it; tile it + P goes to the stage of tile it - 1
    for (int it = 0; it < nkt; ++it) {
      wait_ring<kDmaPerTile, P - 1>(nkt - 1 - it);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int nxt = cur == 0 ? S - 1 : cur - 1;
      if (it + P < nkt) dma_tile<kNW>(sm + nxt * DmaTile::kBytes, kb, vb, a.ks_t, (it + P) * kTK, last);
      const int j0 = it * kTK;
      attend_tile_dma<kRTW>(st, qf, sm + cur * DmaTile::kBytes, [j0](int e) { return j0 + e; }, a.sl2,
                            (it + 1) * kTK - 1 > pmin, [&](int rt, int j) { return j <= rpos[rt]; });
      cur = cur == S - 1 ? 0 : cur + 1;
    }
  } else {
    TileStage<TR, D, kNT, true> stg;
    stg.load(kbase, vbase, a.ks_t, [=](int t) { return t < Tkv ? t : -1; });
    for (int it = 0; it < nkt; ++it) {
      __syncthreads();
      stg.store(sm, kj);
      __syncthreads();
      if (it + 1 < nkt) {
        const int t0 = (it + 1) * kTK;
        stg.load(kbase, vbase, a.ks_t, [=](int t) { return t0 + t < Tkv ? t0 + t : -1; });
      }
      attend_tile<TR, D, kRTW>(st, qf, sm, kj, a.sl2, (it + 1) * kTK - 1 > pmin,
                               [&](int rt, int j) { return j <= rpos[rt]; });
    }
  }

#pragma unroll
  for (int rt = 0; rt < kRTW; ++rt) {
    const float lt = wave_sum16x4(st.l[rt]);
    {
      const int rho = (wave * kRTW + rt) * 16 + col;
      const int hl = rho / a.QTW, qi = rho - hl * a.QTW, i = i0 + qi;
      if (quad == 0 && hl < a.HW && i < a.Tq) {
        const int h = g * a.G + hc * a.HW + hl;
        const float l2 = st.m[rt] + log2f(lt);
        a.lse2[((int64_t)b * a.Hq + h) * a.Tq + i] = l2;
        if (a.lse) a.lse[((int64_t)b * a.Hq + h) * a.Tq + i] = l2 * kLn2;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = __shfl(lt, 4 * quad + r);
      const int rho = (wave * kRTW + rt) * 16 + 4 * quad + r;
      const int hl = rho / a.QTW, qi = rho - hl * a.QTW, i = i0 + qi;
      if (hl < a.HW && i < a.Tq) {
        const int h = g * a.G + hc * a.HW + hl;
        const float inv = 1.f / lr;
        ST* orow = (ST*)a.out + (((int64_t)b * a.Tq + i) * a.Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) orow[16 * dt + col] = TR::from_float(st.o[rt][dt][r] * inv);
      }
    }
  }
}

// ---------------------------------------------------------- sweep 2: scores
// One staged tile for the streaming score sweep: per key, the sum of P over
// the wave's RTW row tiles, written to wred[key].
// kfrag(ct, c): K fragment of key sub-tile ct, k-step c; keys(e): key index
// of tile entry e (-1: invalid).  Row tile x holds queries 16 (x % 4) .. of
// the block, so the position of the lane's row r is pos0 + 16 (x % 4) + r
// (padding rows have nl = -inf and add exactly 0 whatever the mask says).
template <typename TR, int D, int RTW, bool MASK, class KFrag, class Keys>
__device__ __forceinline__ void block_score_tile(const typename TR::frag (&qf)[RTW][D / 32],
                                                 const float (&nl)[RTW][4], int pos0, KFrag kfrag, Keys keys,
                                                 float sl2, float* wred) {
  constexpr int KC = D / 32;
  const int lane = threadIdx.x & 63, col = lane & 15;
  // logits of key sub-tile ct for the wave's row tiles
  auto qk = [&](int ct, f32x4_t (&s)[RTW]) {
    typename TR::frag kf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) kf[c] = kfrag(ct, c);
#pragma unroll
    for (int x = 0; x < RTW; ++x) {
      s[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) TR::mma(s[x], qf[x][c], kf[c]);
    }
  };
  // Software pipeline over the four sub-tiles: the MFMAs of sub-tile ct + 1
  // are issued beside the exponentials and sums of sub-tile ct (independent
  // work of one wave that the MFMA unit and the VALU can run at once).
  f32x4_t sc[2][RTW];
  qk(0, sc[0]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    if (ct + 1 < 4) qk(ct + 1, sc[(ct + 1) & 1]);
    const f32x4_t(&s)[RTW] = sc[ct & 1];
    const int j = MASK ? keys(16 * ct + col) : 0;
    float pr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < RTW; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(s[x][r], sl2, nl[x][r]));
        if constexpr (MASK)
          pr[r] += (j >= 0 && j <= pos0 + 16 * (x & 3) + r) ? p : 0.f;
        else
          pr[r] += p;
      }
    // the four lanes of a key hold the same sum (fixed order), so all of them
    // store it: no branch splits the scheduling region
    wred[16 * ct + col] = wave_sum16x4(pr[0] + pr[1] + pr[2] + pr[3]);
  }
}

// One staged 64-key tile of the score sweep for a wave's RTW row tiles:
// P = 2^(logit2 - lse2) per (row, key), summed into the wave's partials.
template <typename TR, int D, int SB, int RTW, int R, bool MASK>
__device__ __forceinline__ void score_tile(const typename TR::frag (&qf)[RTW][D / 32], const float (&nl)[RTW][4],
                                           const int (&rowpos)[RTW][4], const unsigned char* sm, const int* kj,
                                           float sl2, float* wred, int it) {
  constexpr int KC = D / 32;
  const int lane = threadIdx.x & 63, col = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    typename TR::frag kf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) kf[c] = lds_k_frag<TR, D>(sm, ct, c, col, quad);
    const int j = MASK ? kj[16 * ct + col] : 0;
    float pr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < RTW; ++x) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) TR::mma(s, qf[x][c], kf[c]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(s[r], sl2, nl[x][r]));
        if constexpr (MASK)
          pr[r] += (j >= 0 && j <= rowpos[x][r]) ? p : 0.f;
        else
          pr[r] += p;
      }
    }
    const int kc = it * kTK + 16 * ct + col;  // key within the range
    if constexpr (SB == 64) {
      const float v = wave_sum16x4(pr[0] + pr[1] + pr[2] + pr[3]);
      if (quad == 0) wred[kc] += v;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) wred[(4 * quad + r) * R + kc] += pr[r];
    }
  }
}

// SB = 64, streaming form: one workgroup per (b, g, score block n), longest
// prefixes first, so that the workgroups of one KV group run together (the
// groups of consecutive workgroups are dealt to different XCDs) and share its
// key tiles in that XCD's L2.  The block's 64 queries x G heads are covered in
// passes of NW * RTW row tiles (row tile rt: head rt / 4, queries
// 16 * (rt % 4) ..); every pass streams keys [0, last(n)] through LDS.  Per
// tile each wave sums P over its rows per key into red[wave][key]; the
// workgroup adds the wave sums in a fixed order and writes S (first pass) or
// adds to it (later passes; the same thread owns the same key in every pass,
// so the order of the additions is fixed).
// DMA (bf16, head_dim 128): K tiles come into a ring of LDS stages by
// global_load_lds, one barrier per tile, the wave sums double-buffered; the
// later passes add with a no-return atomic so that no load waits inside the
// ring.  Otherwise: global -> registers -> one LDS tile.
template <typename TR, int D, int kNW, int kRTW, bool DMA>
__global__ __launch_bounds__(kNW * 64, DMA ? 2 : 1) void prefill_block_scores_kernel(PrefillArgs a) {
  constexpr int kNT = kNW * 64;
  using ST = typename TR::storage;
  using L = TileLayout<TR, D>;
  constexpr int KC = D / 32;
  static_assert(!DMA || (TR::kBytes == 2 && D == 128), "DMA staging is for bf16, head_dim 128");
  static_assert(kRTW % 4 == 0, "a wave's row tiles cover whole groups of the block's 64 queries");
  __shared__ __align__(16) unsigned char sm[DMA ? kScStages * DmaTile::kHalf : L::kKBytes];
  __shared__ int kj[DMA ? 1 : kTK];
  __shared__ float red[DMA ? 2 : 1][kNW * kTK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, quad = lane >> 4;
  const int per_n = a.B * a.Hkv;
  const int n = a.NB - 1 - (int)(blockIdx.x / per_n);
  const int bg = blockIdx.x - (blockIdx.x / per_n) * per_n;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int i0 = n * 64, i1 = min(i0 + 64, a.Tq);
  const int pos_last = a.Tkv - a.Tq + i1 - 1;
  const int nkt = pos_last / kTK + 1;
  const int RT = 4 * a.G;
  const int npass = (RT + kNW * kRTW - 1) / (kNW * kRTW);
  const int Tkv = a.Tkv;
  float* srow = a.scores + ((int64_t)bg * a.NB + n) * Tkv;
  const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;

  // keys after the last tile are 0 for this block
  for (int j = nkt * kTK + tid; j < Tkv; j += kNT) srow[j] = 0.f;

  for (int ps = 0; ps < npass; ++ps) {
    typename TR::frag qf[kRTW][KC];
    float nl[kRTW][4];
    int pmin = 0x7fffffff;
#pragma unroll
    for (int x = 0; x < kRTW; ++x) {
      const int rt = ps * kNW * kRTW + wave * kRTW + x;
      const int hl = rt / 4, qoff = 16 * (rt % 4);
      {
        const int i = i0 + qoff + col;
        load_q_frags<TR, D>(a, b, i, g * a.G + hl, rt < RT && i < a.Tq, quad, qf[x]);
      }
      // the LSE of the lane's four rows, loaded unconditionally (clamped
      // index) so the loads are in flight together
      const float* l2row = a.lse2 + ((int64_t)b * a.Hq + g * a.G + min(hl, a.G - 1)) * a.Tq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + qoff + 4 * quad + r;
        const bool ok = rt < RT && i < a.Tq;
        const float l2 = l2row[min(i, a.Tq - 1)];
        nl[x][r] = ok ? -l2 : kNegInf;
        pmin = ok ? min(pmin, a.Tkv - a.Tq + i) : pmin;
      }
    }
    pmin = wave_min_int(pmin);
    const int pos0 = a.Tkv - a.Tq + i0 + 4 * quad;  // row r of row tile x: pos0 + 16 (x % 4) + r
    // tile t's key sums (red buffer rb) -> S (threads 0..63)
    auto flush = [&](int t, int rb) {
      const int j = t * kTK + tid;
      if (j < Tkv) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) v += red[rb][w * kTK + tid];
        if (ps == 0)
          srow[j] = v;
        else if (DMA)
          unsafeAtomicAdd(srow + j, v);  // no-return hardware fp32 add
        else
          srow[j] += v;
      }
    };
    if constexpr (DMA) {
      constexpr int S = kScStages, P = S - 1;
      constexpr int kDmaPerTile = 16 / kNW;
      const uint16_t* kb = reinterpret_cast<const uint16_t*>(kbase);
      const int last = Tkv - 1;
      // every wave is done with the previous pass's stages and sums
      __syncthreads();
#pragma unroll
      for (int t = 0; t < P; ++t)
        if (t < nkt) dma_tile_k<kNW>(sm + t * DmaTile::kHalf, kb, a.ks_t, t * kTK, last);
      // resident Q / LSE before the ring (see the forward sweep)
#pragma unroll
      for (int x = 0; x < kRTW; ++x) {
#pragma unroll
        for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qf[x][c]));
#pragma unroll
        for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(nl[x][r]));
      }
      int cur = 0;
      for (int it = 0; it < nkt; ++it) {
        wait_ring<kDmaPerTile, P - 1>(nkt - 1 - it);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (it > 0 && tid < kTK) flush(it - 1, (it - 1) & 1);
        const int nxt = cur == 0 ? S - 1 : cur - 1;
        if (it + P < nkt) dma_tile_k<kNW>(sm + nxt * DmaTile::kHalf, kb, a.ks_t, (it + P) * kTK, last);
        const unsigned char* stage = sm + cur * DmaTile::kHalf;
        const int j0 = it * kTK;
        auto kfrag = [&](int ct, int c) { return dma_k_frag(stage, ct, c, col, quad); };
        auto keys = [&](int e) { return j0 + e < Tkv ? j0 + e : -1; };
        float* wred = red[it & 1] + wave * kTK;
        if ((it + 1) * kTK - 1 > pmin)
          block_score_tile<TR, D, kRTW, true>(qf, nl, pos0, kfrag, keys, a.sl2, wred);
        else
          block_score_tile<TR, D, kRTW, false>(qf, nl, pos0, kfrag, keys, a.sl2, wred);
        cur = cur == S - 1 ? 0 : cur + 1;
      }
      __syncthreads();
      if (tid < kTK) flush(nkt - 1, (nkt - 1) & 1);
    } else {
      TileStage<TR, D, kNT, false> stg;
      stg.load(kbase, kbase, a.ks_t, [=](int t) { return t < Tkv ? t : -1; });
      auto kfrag = [&](int ct, int c) { return lds_k_frag<TR, D>(sm, ct, c, col, quad); };
      auto keys = [&](int e) { return kj[e]; };
      for (int it = 0; it < nkt; ++it) {
        __syncthreads();
        if (it > 0 && tid < kTK) flush(it - 1, 0);
        stg.store(sm, kj);
        __syncthreads();
        if (it + 1 < nkt) {
          const int t0 = (it + 1) * kTK;
          stg.load(kbase, kbase, a.ks_t, [=](int t) { return t0 + t < Tkv ? t0 + t : -1; });
        }
        if (tile_needs_mask(kj, pmin))
          block_score_tile<TR, D, kRTW, true>(qf, nl, pos0, kfrag, keys, a.sl2, red[0] + wave * kTK);
        else
          block_score_tile<TR, D, kRTW, false>(qf, nl, pos0, kfrag, keys, a.sl2, red[0] + wave * kTK);
      }
      __syncthreads();
      if (tid < kTK) flush(nkt - 1, 0);
    }
  }
}

// Score sweep by key ranges (used for score_block 1).
// SB = 64: rows of a workgroup = the block's 64 queries x G heads (row tile
//          rt = head rt / 4, queries 16 * (rt % 4) ..); output one score row.
// SB = 1 : rows = 16 queries x G heads (row tile rt = head rt); output 16 rows.
// Key range of R keys per workgroup; S = Q . K^T in the 16x16 accumulator
// layout gives each lane one key (l % 16) and four rows (4 * (l / 16) + r).
template <typename TR, int D, int SB, int kNW, int kRTW>
__global__ __launch_bounds__(kNW * 64) void prefill_scores_kernel(PrefillArgs a) {
  constexpr int kNT = kNW * 64;
  using ST = typename TR::storage;
  using L = TileLayout<TR, D>;
  constexpr int KC = D / 32;
  constexpr int QB = SB == 64 ? 64 : 16;
  constexpr int R = SB == 64 ? 512 : 128;  // keys per workgroup
  constexpr int NKT = R / kTK;
  // per-wave partial sums (fixed-order reduction over the waves at the end):
  //   SB = 64: [wave][R]      SB = 1: [wave][16 queries][R]
  constexpr int RED = SB == 64 ? kNW * R : kNW * 16 * R;
  __shared__ __align__(16) unsigned char sm[L::kKBytes];
  __shared__ int kj[kTK];
  __shared__ float red[RED];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, quad = lane >> 4;

  const int kr = blockIdx.x % a.nkr;
  const int rest = blockIdx.x / a.nkr;
  const int per_q = a.B * a.Hkv;
  const int qb = a.nqb - 1 - rest / per_q;
  const int bg = rest - (rest / per_q) * per_q;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int i0 = qb * QB, i1 = min(i0 + QB, a.Tq);
  const int pos_last = a.Tkv - a.Tq + i1 - 1;
  const int r0 = kr * R;
  const int RT = (QB / 16) * a.G;
  const int npass = (RT + kNW * kRTW - 1) / (kNW * kRTW);

  for (int x = tid; x < RED; x += kNT) red[x] = 0.f;

  if (r0 <= pos_last) {
    const int nkt = min(NKT, (pos_last - r0) / kTK + 1);
    const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
    const int Tkv = a.Tkv;
    float* wred = red + (SB == 64 ? wave * R : wave * 16 * R);
    for (int ps = 0; ps < npass; ++ps) {
      typename TR::frag qf[kRTW][KC];
      float nl[kRTW][4];  // -lse2 of the accumulator rows
      int rowpos[kRTW][4];
      int pmin = 0x7fffffff;
#pragma unroll
      for (int x = 0; x < kRTW; ++x) {
        const int rt = ps * kNW * kRTW + wave * kRTW + x;
        const int hl = SB == 64 ? rt / 4 : rt;
        const int qoff = SB == 64 ? 16 * (rt % 4) : 0;
        {  // A-operand row (l % 16)
          const int i = i0 + qoff + col;
          const bool ok = rt < RT && i < a.Tq;
          load_q_frags<TR, D>(a, b, i, g * a.G + hl, ok, quad, qf[x]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // accumulator rows 4 * quad + r
          const int i = i0 + qoff + 4 * quad + r;
          const bool ok = rt < RT && i < a.Tq;
          rowpos[x][r] = ok ? a.Tkv - a.Tq + i : -1;
          // padding rows get P = 2^-inf = 0, also on tiles taken unmasked
          nl[x][r] = ok ? -a.lse2[((int64_t)b * a.Hq + g * a.G + hl) * a.Tq + i] : kNegInf;
          pmin = ok ? min(pmin, rowpos[x][r]) : pmin;
        }
      }
      pmin = wave_min_int(pmin);
      TileStage<TR, D, kNT, false> stg;
      stg.load(kbase, kbase, a.ks_t, [=](int t) { return r0 + t < Tkv ? r0 + t : -1; });
      for (int it = 0; it < nkt; ++it) {
        __syncthreads();
        stg.store(sm, kj);
        __syncthreads();
        if (it + 1 < nkt) {
          const int t0 = r0 + (it + 1) * kTK;
          stg.load(kbase, kbase, a.ks_t, [=](int t) { return t0 + t < Tkv ? t0 + t : -1; });
        }
        if (tile_needs_mask(kj, pmin))
          score_tile<TR, D, SB, kRTW, R, true>(qf, nl, rowpos, sm, kj, a.sl2, wred, it);
        else
          score_tile<TR, D, SB, kRTW, R, false>(qf, nl, rowpos, sm, kj, a.sl2, wred, it);
      }
    }
  }
  __syncthreads();

  float* srow_base = a.scores + ((int64_t)(b * a.Hkv + g) * a.NB) * a.Tkv;
  if constexpr (SB == 64) {
    float* srow = srow_base + (int64_t)qb * a.Tkv;
    for (int x = tid; x < R; x += kNT) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) v += red[w * R + x];
      if (r0 + x < a.Tkv) srow[r0 + x] = v;
    }
  } else {
    for (int x = tid; x < 16 * R; x += kNT) {
      const int qi = x / R, jj = x - qi * R;
      const int i = i0 + qi;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) v += red[w * 16 * R + x];
      if (i < a.Tq && r0 + jj < a.Tkv) srow_base[(int64_t)i * a.Tkv + r0 + jj] = v;
    }
  }
}

// ------------------------------------------------------------ sparse block
// Indices staged kIdxCh at a time, tiles global -> registers -> one LDS tile,
// empty tiles skipped.  (The LDS-DMA ring of the full layer's sweeps made
// this kernel slower: it is not bound by the latency of its loads.)
template <typename TR, int D, int kNW, int kRTW>
__global__ __launch_bounds__(kNW * 64) void sparse_block_kernel(PrefillArgs a) {
  constexpr int kNT = kNW * 64;
  using ST = typename TR::storage;
  using L = TileLayout<TR, D>;
  constexpr int KC = D / 32, DT = D / 16;
  // bf16, head_dim 128: tiles in the swizzled DMA stage layout (conflict-free
  // fragment reads, V read transposed by ds_read_b64_tr_b16), still staged
  // through registers
  constexpr bool kSw = TR::kBytes == 2 && D == 128;
  constexpr size_t kTileBytes = kSw ? (size_t)DmaTile::kBytes : (size_t)L::kBytes;
  __shared__ __align__(16) unsigned char sm[kTileBytes];
  __shared__ int kj[kTK];
  __shared__ int idx_stage[kIdxCh];
  // the window branch's gated share of each output row, kept in LDS until
  // the global branch is done (when it fits beside the tile; otherwise in
  // the output itself); rows of SP elements (pitch D + 8: conflict-free)
  constexpr int SP = D + 8;
  constexpr size_t kStash = (size_t)kNW * kRTW * 16 * SP * sizeof(ST);
  constexpr bool kLdsStash = kTileBytes + kStash + (kTK + kIdxCh) * sizeof(int) <= 160 * 1024;
  __shared__ __align__(16) ST wstash[kLdsStash ? kNW * kRTW * 16 * SP : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 15, quad = lane >> 4;

  // the row chunks of one block share their gathered rows: keep them on one
  // XCD (blocks are dealt to the XCDs round-robin by workgroup id)
  const int per_b = a.B * a.Hkv * a.NB;
  int rc, unit;
  {
    const int w = blockIdx.x;
    const int grp = w / (8 * a.nrc), inner = w - grp * (8 * a.nrc);
    rc = inner / 8;
    unit = grp * 8 + (inner - rc * 8);
  }
  if (unit >= per_b) return;
  const int n = unit % a.NB, bg = unit / a.NB;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int i0 = n * 64, i1 = min(i0 + 64, a.Tq);
  const int pos_first = a.Tkv - a.Tq + i0, pos_last = a.Tkv - a.Tq + i1 - 1;

  typename TR::frag qf[kRTW][KC];
  int rpos[kRTW];
  bool tile_ok[kRTW];
#pragma unroll
  for (int x = 0; x < kRTW; ++x) {
    const int rt = rc * (kNW * kRTW) + wave * kRTW + x;
    const int hl = rt / 4, qoff = 16 * (rt % 4);
    tile_ok[x] = hl < a.G;
    const int i = i0 + qoff + col;
    const bool ok = tile_ok[x] && i < a.Tq;
    rpos[x] = ok ? a.Tkv - a.Tq + i : -1;
    load_q_frags<TR, D>(a, b, i, g * a.G + hl, ok, quad, qf[x]);
  }
  int pmin = 0x7fffffff;  // smallest position among the wave's rows
#pragma unroll
  for (int x = 0; x < kRTW; ++x) pmin = rpos[x] >= 0 ? min(pmin, rpos[x]) : pmin;
  pmin = wave_min_int(pmin);
  const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const ST* vbase = (const ST*)a.v + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const int W = a.window;
  const int wlo = max(0, pos_first - W + 1);
  const int nwt = (pos_last - wlo) / kTK + 1;
  const int32_t* idx_row = a.idx + ((int64_t)(b * a.Hkv + g) * a.NB + n) * a.k_top;
  const int ktop = a.k_top;
  // window tiles read the layer's own window keys/values when given
  const ST* wkbase = a.win.k ? (const ST*)a.win.k + (int64_t)b * a.win.sb + (int64_t)g * a.win.sh : kbase;
  const ST* wvbase = a.win.k ? (const ST*)a.win.v + (int64_t)b * a.win.sb + (int64_t)g * a.win.sh : vbase;
  const int64_t wst = a.win.k ? a.win.st : a.ks_t;
  const int ring = a.win.k ? a.win.ring : 0;

  RowState<kRTW, D> st;
  st.reset();
  // the sigmoid gate of each accumulator row 4 * quad + r of row tile x
  // (clamped indices, so all the loads are in flight together)
  auto load_gates = [&](float (&gsig)[kRTW][4]) {
    float w[kRTW][4];
#pragma unroll
    for (int x = 0; x < kRTW; ++x) {
      const int rt = rc * (kNW * kRTW) + wave * kRTW + x;
      const int hl = min(rt / 4, a.G - 1), qoff = 16 * (rt % 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = min(i0 + qoff + 4 * quad + r, a.Tq - 1);
        w[x][r] = a.gate.p[(int64_t)b * a.gate.sb + (int64_t)i * a.gate.st + g * a.G + hl];
      }
    }
#pragma unroll
    for (int x = 0; x < kRTW; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) gsig[x][r] = 1.f / (1.f + expf(-w[x][r]));
  };
  // output row (b, i, head) of accumulator row 4 * quad + r of row tile x, or
  // nullptr for padding rows
  auto orow_of = [&](int x, int r) -> ST* {
    const int rt = rc * (kNW * kRTW) + wave * kRTW + x;
    const int hl = rt / 4, qoff = 16 * (rt % 4);
    const int i = i0 + qoff + 4 * quad + r;
    if (!tile_ok[x] || i >= a.Tq) return nullptr;
    return (ST*)a.out + (((int64_t)b * a.Tq + i) * a.Hq + g * a.G + hl) * D;
  };
  // where the window share of that row lives (same lane writes and reads it)
  auto stash_of = [&](int x, int r, ST* orow) -> ST* {
    if constexpr (kLdsStash)
      return wstash + ((wave * kRTW + x) * 16 + 4 * quad + r) * SP;
    else
      return orow;
  };
  // window branch done: its share (1 - g) * o_window is stashed (rounded to
  // the output type, read back by the same lane in the epilogue); restart
  // for the global branch (two live output states would not fit the
  // registers)
  auto window_share = [&]() {
    float gsig[kRTW][4];
    load_gates(gsig);
#pragma unroll
    for (int x = 0; x < kRTW; ++x) {
      const float lt = wave_sum16x4(st.l[x]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lr = __shfl(lt, 4 * quad + r);
        const float sc = lr > 0.f ? (1.f - gsig[x][r]) / lr : 0.f;
        ST* orow = orow_of(x, r);
        if (orow) {
          ST* w = stash_of(x, r, orow);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) w[16 * dt + col] = TR::from_float(st.o[x][dt][r] * sc);
        }
      }
    }
    st.reset();
  };
  auto window_valid = [&](int rt, int j) { return j <= rpos[rt] && j > rpos[rt] - W; };
  auto causal_valid = [&](int rt, int j) { return j <= rpos[rt]; };

  {
    const int ngt = (ktop + kTK - 1) / kTK;
    // The selected indices are staged in LDS kIdxCh at a time (validated: -1
    // for padding and for keys after the block), so a gathered tile's row loads
    // do not wait on an index load from global memory.
    int* idx_s = idx_stage;
    auto refill = [&](int e0) {
      constexpr int kPer = (kIdxCh + kNT - 1) / kNT;  // fixed count: the loads are in flight together
      int jv[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int x = tid + r * kNT, e = e0 + x;
        jv[r] = (x < kIdxCh && e < ktop) ? idx_row[e] : -1;
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int x = tid + r * kNT;
        if (x < kIdxCh) idx_s[x] = (jv[r] >= 0 && jv[r] <= pos_last) ? jv[r] : -1;
      }
    };
    auto key_of = [=](int tile) {
      return [=](int t) -> int {
        if (tile < nwt) {
          const int j = wlo + tile * kTK + t;
          return j <= pos_last ? j : -1;
        }
        const int e = (tile - nwt) * kTK + t;
        return e < ktop ? idx_s[e & (kIdxCh - 1)] : -1;
      };
    };
    std::conditional_t<kSw, SwTileStage<kNT>, TileStage<TR, D, kNT, true>> stg;
    auto load_tile = [&](int tile) {
      if (tile < nwt)
        stg.load(wkbase, wvbase, wst, key_of(tile), [=](int j) { return ring > 0 ? j % ring : j; });
      else
        stg.load(kbase, vbase, a.ks_t, key_of(tile));
    };
    // tile 0 is a window tile (nwt >= 1) and needs no index: its loads fly
    // together with the first index chunk's
    load_tile(0);
    refill(0);
    __syncthreads();
    const int ntiles = nwt + ngt;
    // stage the current tile, prefetch the next one; returns whether any entry
    // of the staged tile is a key
    auto stage = [&](int it) -> int {
      __syncthreads();
      stg.store(sm, kj);
      __syncthreads();
      // whether any entry of the staged tile is a key (the same in every wave)
      const int any = __builtin_amdgcn_ballot_w64(kj[lane] >= 0) != 0;
      if (it + 1 < ntiles) {
        const int e1 = (it + 1 - nwt) * kTK;  // first list entry of the next tile
        if (e1 > 0 && (e1 & (kIdxCh - 1)) == 0) {
          refill(e1);  // the previous chunk's last reader was load(it), before the barrier above
          __syncthreads();
        }
        load_tile(it + 1);
      }
      return any;
    };
    // The two branches run as two loops (one live output state; separate loops
    // keep the register pressure of one attention step each).
    auto attend = [&](bool mask, auto valid) {
      if constexpr (kSw)
        attend_tile_dma<kRTW>(st, qf, sm, [&](int e) { return kj[e]; }, a.sl2, mask, valid);
      else
        attend_tile<TR, D, kRTW>(st, qf, sm, kj, a.sl2, mask, valid);
    };
    for (int it = 0; it < nwt; ++it) {
      if (stage(it)) attend(true, window_valid);
    }
    window_share();
    for (int it = nwt; it < ntiles; ++it) {
      if (stage(it)) attend(tile_needs_mask(kj, pmin), causal_valid);
    }
  }
  float gsig[kRTW][4];
  load_gates(gsig);
#pragma unroll
  for (int x = 0; x < kRTW; ++x) {
    const float lt = wave_sum16x4(st.l[x]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = __shfl(lt, 4 * quad + r);
      ST* orow = orow_of(x, r);
      if (orow) {
        const float sc = lr > 0.f ? gsig[x][r] / lr : 0.f;
        const ST* w = stash_of(x, r, orow);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          orow[16 * dt + col] = TR::from_float(st.o[x][dt][r] * sc + TR::to_float(w[16 * dt + col]));
      }
    }
  }
}

PrefillArgs base_args(const Geom& g, const void* q, const void* k, const void* v) {
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qs_b = g.qs_b;
  a.qs_t = g.qs_t;
  a.qs_h = g.qs_h;
  a.ks_b = g.ks_b;
  a.ks_t = g.ks_t;
  a.ks_h = g.ks_h;
  a.B = g.B;
  a.Tq = g.Tq;
  a.Tkv = g.Tkv;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.G = g.G;
  a.sl2 = g.scale * kLog2e;
  return a;
}

#define HYS_PF_DISPATCH(g, ...)  \
  do {                           \
    if ((g).dtype == 1 && (g).D == 128) {                       \
      using TR = BF16;                                          \
      constexpr int DD = 128;                                   \
      __VA_ARGS__;                                              \
    } else if ((g).dtype == 1 && (g).D == 64) {                 \
      using TR = BF16;                                          \
      constexpr int DD = 64;                                    \
      __VA_ARGS__;                                              \
    } else if ((g).dtype == 0 && (g).D == 128) {                \
      using TR = F32;                                           \
      constexpr int DD = 128;                                   \
      __VA_ARGS__;                                              \
    } else {                                                    \
      using TR = F32;                                           \
      constexpr int DD = 64;                                    \
      __VA_ARGS__;                                              \
    }                                                           \
  } while (0)

}  // namespace

size_t prefill_full_ws_bytes(const Geom& g, int /*score_block*/) {
  return align_up((size_t)g.B * g.Hq * g.Tq * sizeof(float));
}

hipError_t launch_full_prefill(const Geom& g, const void* q, const void* k, const void* v, int score_block, void* out,
                               float* lse, float* scores, void* ws, hipStream_t st) {
  PrefillArgs a = base_args(g, q, k, v);
  // heads per workgroup: the largest power of two dividing G (at most 16)
  constexpr int kRowsWG = kFwdNW * kFwdRTW * 16;
  int hw = 1;
  while (hw < 16 && g.G % (hw * 2) == 0 && kRowsWG / (hw * 2) >= 16) hw *= 2;
  a.HW = hw;
  a.QTW = kRowsWG / hw;
  a.NHC = g.G / hw;
  a.nqt = (g.Tq + a.QTW - 1) / a.QTW;
  a.out = out;
  a.lse = lse;
  a.lse2 = static_cast<float*>(ws);
  a.scores = scores;
  a.SB = score_block;
  a.NB = (g.Tq + score_block - 1) / score_block;
  hipError_t e = hipSuccess;
  HYS_PF_DISPATCH(g, {
    {
      constexpr bool kDma = HYS_FWD_DMA && TR::kBytes == 2 && DD == 128;
      e = launch("full_prefill_fwd", prefill_fwd_kernel<TR, DD, kFwdNW, kFwdRTW, kFwdWPE, kDma>,
                 dim3(a.nqt * g.B * g.Hkv * a.NHC), dim3(kFwdNW * 64), 0, st, a);
    }
    if (e != hipSuccess) {
    } else if (score_block == 64) {
      constexpr bool kDma = HYS_SC_DMA && TR::kBytes == 2 && DD == 128;
      e = launch("full_prefill_scores", prefill_block_scores_kernel<TR, DD, kScNW, kScRTW, kDma>,
                 dim3(a.NB * g.B * g.Hkv), dim3(kScNW * 64), 0, st, a);
    } else {
      a.nqb = (g.Tq + 15) / 16;
      a.nkr = (g.Tkv + 127) / 128;
      e = launch("full_prefill_scores", prefill_scores_kernel<TR, DD, 1, kScNW, kScRTW>,
                 dim3(a.nqb * g.B * g.Hkv * a.nkr), dim3(kScNW * 64), 0, st, a);
    }
  });
  return e;
}

size_t sparse_block_ws_bytes(const Geom&, int, int) { return 0; }

hipError_t launch_sparse_block(const Geom& g, const void* q, const void* k, const void* v, const int32_t* idx,
                               int k_top, int score_block, int window, const GateRef& gate, const WinRef& win,
                               void* out, void* /*ws*/,
                               hipStream_t st) {
  (void)score_block;  // 64 (rows of one block share its index set)
  PrefillArgs a = base_args(g, q, k, v);
  a.NB = (g.Tq + 63) / 64;
  a.idx = idx;
  a.k_top = k_top;
  a.window = window;
  a.gate = gate;
  a.win = win;
  a.out = out;
  a.nrc = (4 * g.G + kSpNW * kSpRTW - 1) / (kSpNW * kSpRTW);
  const int units = g.B * g.Hkv * a.NB;
  const int grid = ((units + 7) / 8) * 8 * a.nrc;
  hipError_t e = hipSuccess;
  HYS_PF_DISPATCH(g, {
    e = launch("sparse_prefill", sparse_block_kernel<TR, DD, kSpNW, kSpRTW>, dim3(grid), dim3(kSpNW * 64), 0, st, a);
  });
  return e;
}

}  // namespace hys
