// Hierarchical selection for decode (HISA abstract: a block-level coarse
// filter over pooled block representatives prunes regions, then the
// token-level selection runs only inside the surviving blocks).
//
//   1. pool_keys:     kbar[b, m, g, :] = mean of the keys of block m (the last
//                     block may be shorter), fp32;
//   2. block_scores:  per KV group, each query head's softmax over the pooled
//                     keys, summed over the group's heads;
//   3. top n_keep blocks by the top-K kernel (same order rule);
//   4. gather:        the full layer's scores S at the kept blocks' tokens, in
//                     ascending token order (only the last block can be short,
//                     and it sorts last);
//   5. top k_top candidates by the top-K kernel, mapped back to token indices.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kMaxBlocks = 1 << 20;  // pooled blocks per row

// Pooled keys of blocks [m_begin, m_begin + nm): one workgroup per (b, block
// m, g); 16-byte loads, a group of LPR lanes per key row, RG rows in flight
// per pass (four passes' loads at once), the RG partial sums added through
// LDS.  kbar[b * kbs + (m * Hkv + g) * D + d] (kbs: floats per batch entry).
template <typename TR, int D>
__global__ __launch_bounds__(256) void pool_keys_kernel(const void* k, int64_t ks_b, int64_t ks_t, int64_t ks_h, int Tkv,
                                                        int Hkv, int m_begin, int nm, int block, float* kbar,
                                                        int64_t kbs) {
  constexpr int EPC = 16 / TR::kBytes;  // elements per 16-byte load
  constexpr int LPR = D / EPC;          // lanes per key row
  constexpr int RG = 256 / LPR;         // key rows per pass
  __shared__ float part[RG][D];
  const int id = blockIdx.x;  // (b, m - m_begin, g)
  const int g = id % Hkv, m = m_begin + (id / Hkv) % nm, b = id / (Hkv * nm);
  const int t = threadIdx.x, rg = t / LPR, ln = t - (t / LPR) * LPR;
  const int j0 = m * block, j1 = min(j0 + block, Tkv);
  const typename TR::storage* base =
      (const typename TR::storage*)k + (int64_t)b * ks_b + (int64_t)g * ks_h + ln * EPC;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  for (int j = j0 + rg; j < j1; j += 4 * RG) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = j + u * RG;
      v[u] = jj < j1 ? *reinterpret_cast<const u32x4_t*>(base + (int64_t)jj * ks_t) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (TR::kBytes == 2)
          acc[e] += bf16_to_f32((uint16_t)((e & 1) ? (v[u][e >> 1] >> 16) : (v[u][e >> 1] & 0xFFFFu)));
        else
          acc[e] += __uint_as_float(v[u][e]);
      }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[rg][ln * EPC + e] = acc[e];
  __syncthreads();
  for (int d = t; d < D; d += 256) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += part[r][d];
    kbar[(int64_t)b * kbs + ((int64_t)m * Hkv + g) * D + d] = s / (float)(j1 - j0);
  }
}

// Block logits: one workgroup per (b, g, run of 64 pooled blocks); thread
// (block m, head h) computes logit2[b, g, h, m] = tau * log2(e) * q_h . kbar_m.
// The staging loads have fixed counts, so they are in flight together.
template <typename TR, int D>
__global__ __launch_bounds__(256) void block_logits_kernel(const void* q, int64_t qs_b, int64_t qs_h, const float* kbar,
                                                           int64_t kbs, int Hkv, int G, int M, float sl2,
                                                           float* logit2) {
  constexpr int QN = 16 * D / 256;  // G <= 16 query rows
  constexpr int KN = 64 * D / 256;  // 64 pooled rows
  constexpr int KP = D + 4;  // pooled-key row pitch: 16-byte reads, lanes 16 apart on the same banks only
  __shared__ __align__(16) float qs[16 * D];
  __shared__ __align__(16) float ks[64 * KP];
  const int nchunk = (M + 63) / 64;
  const int bg = blockIdx.x / nchunk, ch = blockIdx.x - (blockIdx.x / nchunk) * nchunk;
  const int b = bg / Hkv, g = bg - (bg / Hkv) * Hkv;
  const int t = threadIdx.x;
  const int m0 = ch * 64;
  float qv[QN], kv[KN];
#pragma unroll
  for (int r = 0; r < QN; ++r) {
    const int x = t + 256 * r, h = x / D, d = x - (x / D) * D;
    qv[r] = x < G * D ? TR::to_float(((const typename TR::storage*)q)[(int64_t)b * qs_b + (int64_t)(g * G + h) * qs_h + d])
                      : 0.f;
  }
#pragma unroll
  for (int r = 0; r < KN; ++r) {
    const int x = t + 256 * r, mm = x / D, d = x - (x / D) * D;
    kv[r] = (m0 + mm < M) ? kbar[(int64_t)b * kbs + ((int64_t)(m0 + mm) * Hkv + g) * D + d] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < QN; ++r) qs[t + 256 * r] = qv[r];
#pragma unroll
  for (int r = 0; r < KN; ++r) {
    const int x = t + 256 * r, mm = x / D, d = x - (x / D) * D;
    ks[mm * KP + d] = kv[r];
  }
  __syncthreads();
  // thread (block mm = t & 63, head group hq = t >> 6) computes heads hq,
  // hq + 4, hq + 8, hq + 12: one 16-byte pooled-key read feeds four heads
  // (the query reads are wave-uniform broadcasts)
  const int mm = t & 63, hq = t >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int d = 0; d < D; d += 4) {
    const float4 kk = *reinterpret_cast<const float4*>(ks + mm * KP + d);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 qq = *reinterpret_cast<const float4*>(qs + (hq + 4 * u) * D + d);
      acc[u] += qq.x * kk.x + qq.y * kk.y + qq.z * kk.z + qq.w * kk.w;
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int h = hq + 4 * u;
    if (h < G && m0 + mm < M) logit2[((int64_t)bg * G + h) * M + m0 + mm] = acc[u] * sl2;
  }
}

// Block scores: one workgroup per (b, g): per head the softmax over the
// pooled blocks (16 threads per head, an online (max, sum) over batches of
// 16 loads in flight, folded in a fixed order), summed over heads.
__global__ __launch_bounds__(256) void block_softmax_kernel(const float* logit2, int G, int M, float* bscore) {
  __shared__ float lse[16];
  const int bg = blockIdx.x, t = threadIdx.x;
  const int h = t >> 4, s = t & 15;
  const float* lg = logit2 + (int64_t)bg * G * M;
  float mx = kNegInf, sum = 0.f;
  for (int m0 = s; m0 < M; m0 += 16 * 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int m = m0 + 16 * u;
      v[u] = (h < G && m < M) ? lg[(int64_t)h * M + m] : kNegInf;
    }
    float bm = v[0];
#pragma unroll
    for (int u = 1; u < 16; ++u) bm = fmaxf(bm, v[u]);
    const float nm = fmaxf(mx, bm);
    if (nm != kNegInf) {
      float add = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) add += fast_exp2(v[u] - nm);
      sum = sum * fast_exp2(mx - nm) + add;
      mx = nm;
    }
  }
  // fold the 16 lanes of the head (one DPP row): quad butterflies, then the
  // row rotations by 4 and 8; lane s == 0 holds a fixed fold order
  auto fold = [&](float om, float os) {
    const float nm = fmaxf(mx, om);
    if (nm != kNegInf) {
      sum = sum * fast_exp2(mx - nm) + os * fast_exp2(om - nm);
      mx = nm;
    }
  };
  fold(dpp_self_f32<0xB1>(mx), dpp_self_f32<0xB1>(sum));
  fold(dpp_self_f32<0x4E>(mx), dpp_self_f32<0x4E>(sum));
  fold(dpp_self_f32<0x124>(mx), dpp_self_f32<0x124>(sum));
  fold(dpp_self_f32<0x128>(mx), dpp_self_f32<0x128>(sum));
  if (s == 0 && h < G) lse[h] = mx + log2f(sum);
  __syncthreads();
  for (int m = t; m < M; m += 256) {
    float e[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) e[hh] = hh < G ? lg[(int64_t)hh * M + m] : 0.f;
    float v = 0.f;
#pragma unroll
    for (int hh = 0; hh < 16; ++hh)
      if (hh < G) v += fast_exp2(e[hh] - lse[hh]);
    bscore[(int64_t)bg * M + m] = v;
  }
}

// cand[row][c] = S[row][token(c)], token(c) = blk[c / block] * block + c % block,
// for the kept blocks in ascending order; valid[row] = number of candidates
// (the kept list is ascending with -1 padding at its end).
__global__ __launch_bounds__(256) void gather_candidates_kernel(const float* S, int Tkv, const int32_t* blk, int n_keep,
                                                                int block, float* cand, int32_t* valid) {
  __shared__ int wsum[4];
  const int row = blockIdx.y;
  const int64_t ncand = (int64_t)n_keep * block;
  const int32_t* br = blk + (int64_t)row * n_keep;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < ncand; c += (int64_t)gridDim.x * 256) {
    const int bi = (int)(c / block), o = (int)(c - (int64_t)bi * block);
    const int m = br[bi];
    const int64_t j = (int64_t)m * block + o;
    cand[(int64_t)row * ncand + c] = (m >= 0 && j < Tkv) ? S[(int64_t)row * Tkv + j] : 0.f;
  }
  if (blockIdx.x == 0) {
    int nv = 0;
    for (int bi = threadIdx.x; bi < n_keep; bi += 256) {
      const int m = br[bi];
      nv += m < 0 ? 0 : min(block, Tkv - m * block);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nv += __shfl_xor(nv, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = nv;
    __syncthreads();
    if (threadIdx.x == 0) valid[row] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
}

__global__ __launch_bounds__(256) void map_positions_kernel(const int32_t* pos, const int32_t* blk, int n_keep,
                                                            int block, int k_top, int64_t n, int32_t* idx) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) {
    const int64_t row = x / k_top;
    const int p = pos[x];
    idx[x] = p < 0 ? -1 : blk[row * n_keep + p / block] * block + p % block;
  }
}

struct HierWs {
  float* kbar;
  float* logit2;
  float* bscore;
  int32_t* blk;
  float* cand;
  int32_t* valid;
  int32_t* pos;
  void* topk_ws;  // shared by the two top-K calls (they run in order)
};

size_t hier_topk_ws(const Geom& g, int block, int n_keep, int k_top) {
  const int M = (g.Tkv + block - 1) / block;
  const int64_t rows = (int64_t)g.B * g.Hkv;
  const size_t a = topk_ws_bytes(rows, M, n_keep);
  const size_t b = topk_ws_bytes(rows, (int32_t)((int64_t)n_keep * block), k_top);
  return a > b ? a : b;
}

HierWs carve(const Geom& g, int block, int n_keep, int k_top, void* ws) {
  const int M = (g.Tkv + block - 1) / block;
  const int64_t rows = (int64_t)g.B * g.Hkv;
  HierWs w{};
  unsigned char* c = static_cast<unsigned char*>(ws);
  w.kbar = reinterpret_cast<float*>(c);
  c += align_up((size_t)g.B * M * g.Hkv * g.D * sizeof(float));
  w.logit2 = reinterpret_cast<float*>(c);
  c += align_up((size_t)rows * g.G * M * sizeof(float));
  w.bscore = reinterpret_cast<float*>(c);
  c += align_up((size_t)rows * M * sizeof(float));
  w.blk = reinterpret_cast<int32_t*>(c);
  c += align_up((size_t)rows * n_keep * sizeof(int32_t));
  w.cand = reinterpret_cast<float*>(c);
  c += align_up((size_t)rows * n_keep * block * sizeof(float));
  w.valid = reinterpret_cast<int32_t*>(c);
  c += align_up((size_t)rows * sizeof(int32_t));
  w.pos = reinterpret_cast<int32_t*>(c);
  c += align_up((size_t)rows * k_top * sizeof(int32_t));
  w.topk_ws = c;
  return w;
}

}  // namespace

int hier_max_blocks() { return kMaxBlocks; }

size_t hier_ws_bytes(const Geom& g, int block, int n_keep, int k_top) {
  const int M = (g.Tkv + block - 1) / block;
  const int64_t rows = (int64_t)g.B * g.Hkv;
  return align_up((size_t)g.B * M * g.Hkv * g.D * sizeof(float)) + align_up((size_t)rows * g.G * M * sizeof(float)) +
         align_up((size_t)rows * M * sizeof(float)) +
         align_up((size_t)rows * n_keep * sizeof(int32_t)) + align_up((size_t)rows * n_keep * block * sizeof(float)) +
         align_up((size_t)rows * sizeof(int32_t)) + align_up((size_t)rows * k_top * sizeof(int32_t)) +
         hier_topk_ws(g, block, n_keep, k_top);
}

#define HIER_DT(...)                                                     \
  do {                                                                   \
    if (g.dtype == 1 && g.D == 128) { using TR = BF16; constexpr int DD = 128; __VA_ARGS__; } \
    else if (g.dtype == 1) { using TR = BF16; constexpr int DD = 64; __VA_ARGS__; }           \
    else if (g.D == 128) { using TR = F32; constexpr int DD = 128; __VA_ARGS__; }            \
    else { using TR = F32; constexpr int DD = 64; __VA_ARGS__; }                              \
  } while (0)

hipError_t launch_hier_pool(const Geom& g, const void* k, int block, int m_begin, int m_end, float* kbar,
                            int64_t kbar_blocks, hipStream_t st) {
  if (m_end <= m_begin) return hipSuccess;
  const int nm = m_end - m_begin;
  const int64_t kbs = kbar_blocks * g.Hkv * g.D;
  hipError_t e = hipSuccess;
  HIER_DT({
    e = launch("hier_pool_keys", pool_keys_kernel<TR, DD>, dim3(g.B * nm * g.Hkv), dim3(256), 0, st, k, g.ks_b,
               g.ks_t, g.ks_h, g.Tkv, g.Hkv, m_begin, nm, block, kbar, kbs);
  });
  return e;
}

hipError_t launch_hier_select(const Geom& g, const void* q, const void* k, const float* kbar_in, int64_t kbar_blocks,
                              const float* scores, int block, int n_keep, int k_top, float* bscore_out,
                              int32_t* blk_out, int32_t* idx, void* ws, hipStream_t st) {
  const int M = (g.Tkv + block - 1) / block;
  const int rows = g.B * g.Hkv;
  HierWs w = carve(g, block, n_keep, k_top, ws);
  float* bscore = bscore_out ? bscore_out : w.bscore;
  int32_t* blk = blk_out ? blk_out : w.blk;
  const float sl2 = g.scale * kLog2e;
  hipError_t e;
  // pooled keys: the caller's, or all blocks pooled into the workspace now
  const float* kbar = kbar_in;
  int64_t kbs = kbar_blocks * g.Hkv * g.D;
  if (!kbar) {
    if ((e = launch_hier_pool(g, k, block, 0, M, w.kbar, M, st)) != hipSuccess) return e;
    kbar = w.kbar;
    kbs = (int64_t)M * g.Hkv * g.D;
  }
  e = hipSuccess;
  HIER_DT({
    e = launch("hier_block_logits", block_logits_kernel<TR, DD>, dim3(rows * ((M + 63) / 64)), dim3(256), 0, st, q,
               g.qs_b, g.qs_h, kbar, kbs, g.Hkv, g.G, M, sl2, w.logit2);
  });
  if (e != hipSuccess) return e;
  if ((e = launch("hier_block_softmax", block_softmax_kernel, dim3(rows), dim3(256), 0, st, w.logit2, g.G, M,
                  bscore)) != hipSuccess)
    return e;
  ValidLen all{nullptr, M, 0, 1, 1, 1, 1};
  if ((e = launch_topk(bscore, rows, M, M, all, n_keep, blk, w.topk_ws, st)) != hipSuccess) return e;
  const int64_t ncand = (int64_t)n_keep * block;
  {
    int gx = (int)((ncand + 255) / 256);
    if (gx > 64) gx = 64;
    if ((e = launch("hier_gather", gather_candidates_kernel, dim3(gx, rows), dim3(256), 0, st, scores, g.Tkv, blk,
                    n_keep, block, w.cand, w.valid)) != hipSuccess)
      return e;
  }
  ValidLen vl{w.valid, (int32_t)ncand, 0, 1, 1, 1, 1};
  if ((e = launch_topk(w.cand, rows, (int32_t)ncand, ncand, vl, k_top, w.pos, w.topk_ws, st)) != hipSuccess) return e;
  const int64_t n = (int64_t)rows * k_top;
  int gb = (int)((n + 255) / 256);
  if (gb > 4096) gb = 4096;
  return launch("hier_map", map_positions_kernel, dim3(gb), dim3(256), 0, st, w.pos, blk, n_keep, block, k_top, n,
                idx);
}

#undef HIER_DT

}  // namespace hys
