// Split-K attention of single query rows against a key list, on gfx950 MFMA.
//
// One workgroup (4 waves) handles one split of one unit's key list.  A unit is
// one query row of one KV group with all of that group's query heads
// (G <= 16 heads padded to the 16 rows of a 16x16 MFMA tile):
//   * full layer (decode):  key list = the whole cache 0..Tkv-1; the scaled
//     logits are also written (base 2) so that the importance scores can be
//     formed once the log-sum-exp of every head is known;
//   * sparse layer (one query row per score row): key list = the row's top-K
//     indices (global branch) followed by the W window keys (local branch);
//     a split covers either global or window entries, never both.
//
// Per wave step of 32 keys (pages: the Baidu article's gather-then-attend
// pseudocode; Flash-style online softmax as in the Ultralytics glossary's
// "Attention Flash" entry):
//   S^T[32 keys x 16 heads] = K_sel . Q^T        (8 MFMA k-steps, K rows read
//                                                 straight into A fragments)
//   online softmax per head (base-2 logits)
//   O[16 heads x D] += P . V_sel                 (V rows staged transposed in a
//                                                 wave-private LDS tile)
// The four waves of the workgroup are merged through LDS and the workgroup
// writes one partial state (m, l, O) per head; small reduce kernels combine
// the splits (and for the sparse layer apply the sigmoid gate).
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 32;  // keys per wave step
constexpr int kVPad = 4;   // extra key slots per transposed-V row (bank spread)
constexpr int kScoreChunk = 1024;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs_b, qs_t, qs_h, ks_b, ks_t, ks_h;
  int B, Tq, Tkv, Hq, Hkv, G;
  float sl2;  // softmax scale * log2(e)
  const int32_t* idx;
  int k_top, score_block, NB, window;
  int chunk, nsplit, nsg;
  float* logits;
  float* part_o;
  float* part_ml;
};

template <typename TR, int D>
struct DecodeSmem {
  static constexpr int kVP = kStep + kVPad;
  static constexpr size_t kVt = (size_t)kWaves * D * kVP * TR::kBytes;
  static constexpr size_t kObuf = (size_t)kWaves * 16 * D * sizeof(float);
  static constexpr size_t kBytes = kVt > kObuf ? kVt : kObuf;
};

template <typename TR, int D, bool FULL>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  using ST = typename TR::storage;
  using frag = typename TR::frag;
  using quad_t = typename TR::quad_t;
  constexpr int KC = D / 32;            // MFMA k-steps over head_dim
  constexpr int EPC = 16 / TR::kBytes;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // 16-byte chunks per K/V row
  constexpr int NP = CPR / 8;           // (chunk, key-quad) pairs per lane and step
  constexpr int VP = kStep + kVPad;
  constexpr int DT = D / 16;            // 16-column output tiles

  __shared__ __align__(16) unsigned char smem[DecodeSmem<TR, D>::kBytes];
  __shared__ int kj_s[kWaves][kStep];
  __shared__ float ml_s[kWaves][16][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int split = blockIdx.x % a.nsplit;
  const int unit = blockIdx.x / a.nsplit;
  int b, g, i;
  if (FULL) {
    b = unit / a.Hkv;
    g = unit - b * a.Hkv;
    i = 0;
  } else {
    i = unit % a.Tq;
    const int bg = unit / a.Tq;
    b = bg / a.Hkv;
    g = bg - b * a.Hkv;
  }
  const int pos = a.Tkv - a.Tq + i;

  // this split's slice of the unit's key list
  int kind, t_begin, t_end, wbase = 0;
  const int32_t* idx_row = nullptr;
  if (FULL) {
    kind = 0;
    t_begin = split * a.chunk;
    t_end = min(t_begin + a.chunk, a.Tkv);
  } else if (split < a.nsg) {
    kind = 1;
    t_begin = split * a.chunk;
    t_end = min(t_begin + a.chunk, a.k_top);
    const int n = i / a.score_block;
    idx_row = a.idx + ((int64_t)(b * a.Hkv + g) * a.NB + n) * a.k_top;
  } else {
    kind = 2;
    t_begin = (split - a.nsg) * a.chunk;
    t_end = min(t_begin + a.chunk, a.window);
    wbase = pos - a.window + 1;
  }

  const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const ST* vbase = (const ST*)a.v + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;

  // B operand: Q^T, lane (head = col, group = quad) holds d = 32c + 8*quad + e
  frag qf[KC];
  {
    const ST* qrow = (const ST*)a.q + (int64_t)b * a.qs_b + (int64_t)i * a.qs_t +
                     (int64_t)(g * a.G + col) * a.qs_h;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = (col < a.G) ? TR::load8(qrow + 32 * c + 8 * quad) : TR::zero8();
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  ST* vt = reinterpret_cast<ST*>(smem) + (size_t)wave * D * VP;
  int* kj = kj_s[wave];
  float* lg_row = nullptr;
  if (FULL && col < a.G) lg_row = a.logits + ((int64_t)b * a.Hq + g * a.G + col) * a.Tkv;

  for (int t0 = t_begin + wave * kStep; t0 < t_end; t0 += kWaves * kStep) {
    wave_lds_sync();
    if (lane < kStep) {
      const int t = t0 + lane;
      int j = -1;
      if (t < t_end) j = (kind == 0) ? t : (kind == 1 ? idx_row[t] : wbase + t);
      kj[lane] = (j >= 0 && j <= pos) ? j : -1;
    }
    wave_lds_sync();

    // A operand: K rows of list entries t0 + 16*kt + col
    frag kf[2][KC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int j = kj[16 * kt + col];
      const ST* kr = kbase + (int64_t)(j >= 0 ? j : 0) * a.ks_t;
#pragma unroll
      for (int c = 0; c < KC; ++c) kf[kt][c] = TR::load8(kr + 32 * c + 8 * quad);
    }
    // V rows: lane owns (chunk tc, key quad kq) pairs, four rows each
    uint4 vr[NP][4];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int pidx = lane + 64 * pp;
      const int tc = pidx % CPR, kq = pidx / CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kj[4 * kq + r];
        vr[pp][r] = *reinterpret_cast<const uint4*>(vbase + (int64_t)(j >= 0 ? j : 0) * a.ks_t + tc * EPC);
      }
    }

    // S^T = K . Q^T ; sacc[kt][r] = logit of key 16*kt + 4*quad + r for head col
    f32x4_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) TR::mma(sacc[kt], kf[kt][c], qf[c]);
    }
    float s[2][4];
    float mt = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kj[16 * kt + 4 * quad + r];
        const float x = sacc[kt][r] * a.sl2;
        s[kt][r] = (j >= 0) ? x : kNegInf;
        if (FULL && lg_row != nullptr && j >= 0) lg_row[j] = x;
        mt = fmaxf(mt, s[kt][r]);
      }
    }
    mt = wave_max16x4(mt);
    const float m_new = fmaxf(m_run, mt);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - mu);
    float p[2][4];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = exp2f(s[kt][r] - mu);
        ls += p[kt][r];
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // rescale output rows (head 4*quad + r) by that head's alpha
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * quad + r);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][r] *= ar;
    }

    // stage V transposed: vt[d][key]
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int pidx = lane + 64 * pp;
      const int tc = pidx % CPR, kq = pidx / CPR;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        ST* dst = vt + (tc * EPC + e) * VP + 4 * kq;
        if constexpr (TR::kBytes == 2) {
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[pp][0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[pp][1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[pp][2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[pp][3]);
          const int sh = 16 * (e & 1);
          uint2 pk;
          pk.x = ((w0[e >> 1] >> sh) & 0xFFFFu) | (((w1[e >> 1] >> sh) & 0xFFFFu) << 16);
          pk.y = ((w2[e >> 1] >> sh) & 0xFFFFu) | (((w3[e >> 1] >> sh) & 0xFFFFu) << 16);
          *reinterpret_cast<uint2*>(dst) = pk;
        } else {
          const float* f0 = reinterpret_cast<const float*>(&vr[pp][0]);
          const float* f1 = reinterpret_cast<const float*>(&vr[pp][1]);
          const float* f2 = reinterpret_cast<const float*>(&vr[pp][2]);
          const float* f3 = reinterpret_cast<const float*>(&vr[pp][3]);
          *reinterpret_cast<float4*>(dst) = make_float4(f0[e], f1[e], f2[e], f3[e]);
        }
      }
    }
    wave_lds_sync();

    // O += P . V ; A = P (head = col, keys {4q..4q+3, 16+4q..16+4q+3})
    const frag pa = TR::pack(p[0], p[1]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const ST* row = vt + (16 * dt + col) * VP;
      const quad_t lo = *reinterpret_cast<const quad_t*>(row + 4 * quad);
      const quad_t hi = *reinterpret_cast<const quad_t*>(row + 16 + 4 * quad);
      TR::mma(o[dt], pa, TR::join(lo, hi));
    }
  }

  // merge the four waves of the workgroup
  l_run = wave_sum16x4(l_run);
  if (quad == 0) {
    ml_s[wave][col][0] = m_run;
    ml_s[wave][col][1] = l_run;
  }
  __syncthreads();
  float f[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * quad + r;
    float M = ml_s[0][h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, ml_s[w][h][0]);
    const float mu = (M == kNegInf) ? 0.f : M;
    f[r] = exp2f(ml_s[wave][h][0] - mu);
  }
  float* obuf = reinterpret_cast<float*>(smem);  // [kWaves][16][D]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) obuf[(wave * 16 + 4 * quad + r) * D + 16 * dt + col] = o[dt][r] * f[r];
  __syncthreads();

  const int64_t pbase = (int64_t)unit * a.nsplit + split;
  float* po = a.part_o + pbase * a.G * D;
  for (int x = tid; x < a.G * D; x += 256) {
    const int h = x / D, d = x - h * D;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += obuf[(w * 16 + h) * D + d];
    po[x] = acc;
  }
  if (tid < a.G) {
    const int h = tid;
    float M = ml_s[0][h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, ml_s[w][h][0]);
    const float mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += ml_s[w][h][1] * exp2f(ml_s[w][h][0] - mu);
    a.part_ml[(pbase * a.G + h) * 2 + 0] = M;
    a.part_ml[(pbase * a.G + h) * 2 + 1] = L;
  }
}

// Merge the partial states of splits [s0, s1) of one (unit, head): returns
// the normalised output element d (0 when no key was valid) and the base-2
// log-sum-exp.
__device__ __forceinline__ float merge_splits(const float* po, const float* pml, int s0, int s1, int G,
                                              int D, int h, int d, float* lse2_out) {
  float M = kNegInf;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, pml[(s * G + h) * 2]);
  const float mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f, acc = 0.f;
  for (int s = s0; s < s1; ++s) {
    const float w = exp2f(pml[(s * G + h) * 2] - mu);
    L += pml[(s * G + h) * 2 + 1] * w;
    acc += po[((int64_t)s * G + h) * D + d] * w;
  }
  if (lse2_out) *lse2_out = (L > 0.f) ? mu + log2f(L) : kNegInf;
  return (L > 0.f) ? acc / L : 0.f;
}

template <typename TR, int D>
__global__ __launch_bounds__(D) void decode_full_reduce_kernel(const float* part_o, const float* part_ml, int nsplit,
                                                               int G, int Hkv, void* out, float* lse,
                                                               float* lse2) {
  const int unit = blockIdx.x / G, h = blockIdx.x - (blockIdx.x / G) * G;
  const int b = unit / Hkv, g = unit - b * Hkv;
  const int Hq = Hkv * G, d = threadIdx.x;
  const float* po = part_o + (int64_t)unit * nsplit * G * D;
  const float* pml = part_ml + (int64_t)unit * nsplit * G * 2;
  float l2;
  const float o = merge_splits(po, pml, 0, nsplit, G, D, h, d, &l2);
  const int hq = g * G + h;
  reinterpret_cast<typename TR::storage*>(out)[((int64_t)b * Hq + hq) * D + d] = TR::from_float(o);
  if (d == 0) {
    lse2[(int64_t)b * Hq + hq] = l2;
    if (lse) lse[(int64_t)b * Hq + hq] = l2 * kLn2;
  }
}

// S[b, g, 0, j] = sum over the group's heads of 2^(logit2 - lse2)
__global__ __launch_bounds__(256) void decode_scores_kernel(const float* logits, const float* lse2, float* scores,
                                                            int Hkv, int G, int Tkv, int nchunk) {
  const int unit = blockIdx.x / nchunk, c = blockIdx.x - (blockIdx.x / nchunk) * nchunk;
  const int b = unit / Hkv, g = unit - b * Hkv, Hq = Hkv * G;
  const int j0 = c * kScoreChunk + 4 * threadIdx.x;
  if (j0 >= Tkv) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const bool vec = ((Tkv & 3) == 0) && (j0 + 3 < Tkv);
  for (int h = 0; h < G; ++h) {
    const int64_t hrow = (int64_t)b * Hq + g * G + h;
    const float L = lse2[hrow];
    const float* row = logits + hrow * Tkv;
    if (vec) {
      const float4 x = *reinterpret_cast<const float4*>(row + j0);
      acc[0] += exp2f(x.x - L);
      acc[1] += exp2f(x.y - L);
      acc[2] += exp2f(x.z - L);
      acc[3] += exp2f(x.w - L);
    } else {
      for (int e = 0; e < 4; ++e)
        if (j0 + e < Tkv) acc[e] += exp2f(row[j0 + e] - L);
    }
  }
  float* srow = scores + (int64_t)unit * Tkv;
  if (vec) {
    *reinterpret_cast<float4*>(srow + j0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    for (int e = 0; e < 4; ++e)
      if (j0 + e < Tkv) srow[j0 + e] = acc[e];
  }
}

template <typename TR, int D>
__global__ __launch_bounds__(D) void decode_sparse_reduce_kernel(const float* part_o, const float* part_ml,
                                                                 int nsplit, int nsg, int G, int Hkv, int Tq,
                                                                 const float* gate, void* out) {
  const int unit = blockIdx.x / G, h = blockIdx.x - (blockIdx.x / G) * G;
  const int i = unit % Tq, bg = unit / Tq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G, d = threadIdx.x;
  const float* po = part_o + (int64_t)unit * nsplit * G * D;
  const float* pml = part_ml + (int64_t)unit * nsplit * G * 2;
  const float og = merge_splits(po, pml, 0, nsg, G, D, h, d, nullptr);
  const float ol = merge_splits(po, pml, nsg, nsplit, G, D, h, d, nullptr);
  const float gt = 1.f / (1.f + expf(-gate[g * G + h]));
  const float y = gt * og + (1.f - gt) * ol;
  reinterpret_cast<typename TR::storage*>(out)[(((int64_t)b * Tq + i) * Hq + g * G + h) * D + d] = TR::from_float(y);
}

DecodeArgs make_args(const Geom& g, const DecodePlan& p, const void* q, const void* k, const void* v) {
  DecodeArgs a{};
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
  a.chunk = p.chunk;
  a.nsplit = p.nsplit;
  a.nsg = p.nsg;
  return a;
}

#define HYS_DISPATCH(g, ...)                                    \
  do {                                                          \
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

DecodePlan plan_full_decode(const Geom& g) {
  DecodePlan p{};
  p.units = g.B * g.Hkv;
  const int quantum = kWaves * kStep;  // one step per wave
  const int max_splits = (g.Tkv + quantum - 1) / quantum;
  int want = (2048 + p.units - 1) / p.units;
  if (want < 1) want = 1;
  int ns = want < max_splits ? want : max_splits;
  int chunk = (g.Tkv + ns - 1) / ns;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  p.chunk = chunk;
  p.nsplit = (g.Tkv + chunk - 1) / chunk;
  p.nsg = p.nsplit;
  return p;
}

DecodePlan plan_sparse_rows(const Geom& g, int k_top, int window) {
  DecodePlan p{};
  p.units = g.B * g.Hkv * g.Tq;
  p.chunk = kWaves * kStep;
  p.nsg = (k_top + p.chunk - 1) / p.chunk;
  p.nsplit = p.nsg + (window + p.chunk - 1) / p.chunk;
  return p;
}

static size_t decode_ws(const Geom& g, const DecodePlan& p, bool full) {
  size_t n = align_up((size_t)p.units * p.nsplit * g.G * g.D * sizeof(float));
  n += align_up((size_t)p.units * p.nsplit * g.G * 2 * sizeof(float));
  if (full) {
    n += align_up((size_t)g.B * g.Hq * g.Tkv * sizeof(float));
    n += align_up((size_t)g.B * g.Hq * sizeof(float));
  }
  return n;
}

size_t decode_full_ws_bytes(const Geom& g) { return decode_ws(g, plan_full_decode(g), true); }
size_t decode_sparse_ws_bytes(const Geom& g, int k_top, int window) {
  return decode_ws(g, plan_sparse_rows(g, k_top, window), false);
}

DecodeWs carve_decode_ws(const Geom& g, const DecodePlan& p, void* ws, bool full) {
  DecodeWs w{};
  unsigned char* c = static_cast<unsigned char*>(ws);
  w.part_o = reinterpret_cast<float*>(c);
  c += align_up((size_t)p.units * p.nsplit * g.G * g.D * sizeof(float));
  w.part_ml = reinterpret_cast<float*>(c);
  c += align_up((size_t)p.units * p.nsplit * g.G * 2 * sizeof(float));
  if (full) {
    w.logits = reinterpret_cast<float*>(c);
    c += align_up((size_t)g.B * g.Hq * g.Tkv * sizeof(float));
    w.lse2 = reinterpret_cast<float*>(c);
  }
  return w;
}

hipError_t launch_full_decode(const Geom& g, const void* q, const void* k, const void* v, void* out,
                              float* lse, float* scores, void* ws, hipStream_t st) {
  const DecodePlan p = plan_full_decode(g);
  const DecodeWs w = carve_decode_ws(g, p, ws, true);
  DecodeArgs a = make_args(g, p, q, k, v);
  a.logits = w.logits;
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  const int nchunk = (g.Tkv + kScoreChunk - 1) / kScoreChunk;
  HYS_DISPATCH(g, {
    decode_split_kernel<TR, DD, true><<<p.units * p.nsplit, 256, 0, st>>>(a);
    decode_full_reduce_kernel<TR, DD><<<p.units * g.G, DD, 0, st>>>(w.part_o, w.part_ml, p.nsplit, g.G, g.Hkv,
                                                                     out, lse, w.lse2);
  });
  decode_scores_kernel<<<p.units * nchunk, 256, 0, st>>>(w.logits, w.lse2, scores, g.Hkv, g.G, g.Tkv, nchunk);
  return hipGetLastError();
}

hipError_t launch_sparse_rows(const Geom& g, const void* q, const void* k, const void* v,
                              const int32_t* idx, int k_top, int score_block, int window,
                              const float* gate, void* out, void* ws, hipStream_t st) {
  const DecodePlan p = plan_sparse_rows(g, k_top, window);
  const DecodeWs w = carve_decode_ws(g, p, ws, false);
  DecodeArgs a = make_args(g, p, q, k, v);
  a.idx = idx;
  a.k_top = k_top;
  a.score_block = score_block;
  a.NB = (g.Tq + score_block - 1) / score_block;
  a.window = window;
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  HYS_DISPATCH(g, {
    decode_split_kernel<TR, DD, false><<<p.units * p.nsplit, 256, 0, st>>>(a);
    decode_sparse_reduce_kernel<TR, DD><<<p.units * g.G, DD, 0, st>>>(w.part_o, w.part_ml, p.nsplit, p.nsg, g.G,
                                                                       g.Hkv, g.Tq, gate, out);
  });
  return hipGetLastError();
}

}  // namespace hys
