// Split-K attention of single query rows against a key list, on gfx950 MFMA.
//
// One workgroup (4 waves) handles one split of one unit's key list.  A unit is
// one query row of one KV group with all of that group's query heads
// (G <= 16 heads padded to the 16 rows of a 16x16 MFMA tile):
//   * full layer (decode):  key list = the whole cache 0..Tkv-1; each key's
//     probability against the wave's running maximum (the P of the P.V
//     product, key-major: the group's heads of one key side by side) is also
//     written, with that maximum per 32-key step and head, so that the
//     importance scores can be formed once the log-sum-exp of every head is
//     known;
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
// writes one partial state (m, l, O) per head.  Sparse layer: a small merge
// kernel combines each unit's splits and applies the sigmoid gate.  Full
// layer: a second kernel forms each head's log-sum-exp from the partial
// states, then the output rows and the importance scores.  (Merging inside
// the split kernel by its last-arriving workgroup would need a device-scope
// fence per workgroup, which on this multi-die part writes back and
// invalidates the die's L2 and costs far more than a second launch.)
#include <type_traits>

#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 32;  // keys per wave step
constexpr int kVPad = 4;   // extra key slots per transposed-V row (bank spread)
constexpr int kScoreChunk = 1024;  // keys per score workgroup (multiple of 1024)


struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs_b, qs_t, qs_h, ks_b, ks_t, ks_h;
  int B, Tq, Tkv, Hq, Hkv, G;
  float sl2;  // softmax scale * log2(e)
  const int32_t* idx;
  int k_top, score_block, NB, window;
  int chunk, wchunk, nsplit, nsg;
  void* probs;          // full decode: step probabilities, key-major (see prob_slots)
  float* pmax;          // full decode: base-2 running maximum per (32-key step, head)
  int lgp;              // slots per key: G rounded up to 4, 8 or 16
  int64_t lus;          // elements per unit of probs
  int64_t mus;          // floats per unit of pmax
  float* part_o;
  float* part_ml;
  GateRef gate;         // sparse: gate logits
  WinRef win;           // sparse: window branch keys/values (k == nullptr: the shared cache)
  void* out;            // sparse: [B, Tq, Hq, D]
};

constexpr int kMaxSparseSplits = 64;

// Element format of the full layer's probability scratch.  The stored value
// is 2^(s - m) for a base-2 logit s and the running maximum m of its step, so
// it lies in [0, 1].  fp32 inputs keep it in fp32.  bf16 inputs keep it in
// three bytes: the fp32 value rounded (to nearest, ties to even) to its upper
// 24 bits, i.e. sign, exponent and 15 stored mantissa bits, a relative error
// of at most 2^-16 per value.  Four consecutive slots (four heads of one key)
// always travel together, in three dwords: the upper three bytes of each of
// the first three values, with the fourth value's three bytes in their low
// bytes.
template <typename TR>
struct ProbFmt;
template <>
struct ProbFmt<F32> {
  static constexpr int kSlotBytes = 4;
  __device__ static __forceinline__ void store4(unsigned char* p, const float (&w)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(w[0], w[1], w[2], w[3]);
  }
  __device__ static __forceinline__ f32x4_t load4(const unsigned char* p) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    return f32x4_t{x.x, x.y, x.z, x.w};
  }
};
template <>
struct ProbFmt<BF16> {
  static constexpr int kSlotBytes = 3;
  struct __attribute__((aligned(4))) pack_t {
    uint32_t x, y, z;
  };
  __device__ static __forceinline__ uint32_t round24(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;
  }
  __device__ static __forceinline__ void store4(unsigned char* p, const float (&w)[4]) {
    const uint32_t r3 = round24(w[3]);
    pack_t t;
    t.x = (round24(w[0]) << 8) | (r3 & 0xFFu);
    t.y = (round24(w[1]) << 8) | ((r3 >> 8) & 0xFFu);
    t.z = (round24(w[2]) << 8) | (r3 >> 16);
    *reinterpret_cast<pack_t*>(p) = t;
  }
  __device__ static __forceinline__ f32x4_t unpack(const pack_t& t) {
    const uint32_t v3 = ((t.x & 0xFFu) << 8) | ((t.y & 0xFFu) << 16) | (t.z << 24);
    return f32x4_t{__uint_as_float(t.x & ~0xFFu), __uint_as_float(t.y & ~0xFFu), __uint_as_float(t.z & ~0xFFu),
                   __uint_as_float(v3)};
  }
};

template <typename TR, int D>
struct DecodeSmem {
  static constexpr int kVP = kStep + kVPad;
  static constexpr size_t kVt = (size_t)kWaves * D * kVP * TR::kBytes;
  // wave-merge rows, pitch D + 4 floats: the four lane groups of a store
  // (rows 4 apart) fall on different banks
  static constexpr int kOP = D + 4;
  static constexpr size_t kObuf = (size_t)kWaves * 16 * kOP * sizeof(float);
  static constexpr size_t kMerge = 64 * 16 * 3 * sizeof(float);  // sparse merge: (m, l) + weights
  // bf16, head_dim 128: K is staged too (32 keys x 256 B per wave, after the
  // V tiles), so its loads are whole rows like V's
  static constexpr bool kLdsK = TR::kBytes == 2 && D == 128;
  static constexpr size_t kKt = kLdsK ? (size_t)kWaves * kStep * 256 : 0;
  static constexpr size_t kA = kVt + kKt > kObuf ? kVt + kKt : kObuf;
  static constexpr size_t kBytes = kA > kMerge ? kA : kMerge;
};

template <typename TR, int D, bool FULL>
__global__ __launch_bounds__(256, TR::kBytes == 4 ? 1 : 2) void decode_split_kernel(DecodeArgs a) {
  using ST = typename TR::storage;
  using frag = typename TR::frag;
  using quad_t = typename TR::quad_t;
  constexpr int KC = D / 32;            // MFMA k-steps over head_dim
  constexpr int EPC = 16 / TR::kBytes;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // 16-byte chunks per K/V row
  constexpr int NP = CPR / 8;           // (chunk, key-quad) pairs per lane and step
  constexpr int VP = kStep + kVPad;
  constexpr int DT = D / 16;            // 16-column output tiles
  // bf16, head_dim 128: each V load instruction reads four whole 256-byte
  // rows (16 lanes per row), the rows are staged unchanged (swizzled 16-byte
  // slots, conflict-free) and read back transposed by ds_read_b64_tr_b16
  constexpr bool kTrV = TR::kBytes == 2 && D == 128;
  static_assert(!kTrV || NP * 4 * 4 == kStep, "eight row loads of four keys cover a step");

  __shared__ __align__(16) unsigned char smem[DecodeSmem<TR, D>::kBytes];
  __shared__ int kj_s[kWaves][2 * kStep];
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
    t_begin = (split - a.nsg) * a.wchunk;
    t_end = min(t_begin + a.wchunk, a.window);
    wbase = pos - a.window + 1;
  }

  const ST* kbase = (const ST*)a.k + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  const ST* vbase = (const ST*)a.v + (int64_t)b * a.ks_b + (int64_t)g * a.ks_h;
  int64_t kst = a.ks_t;  // token stride of the rows this split reads
  int ring = 0;          // > 0: key j lives in row j % ring
  if (!FULL && kind == 2 && a.win.k) {  // the layer's own window keys/values
    kbase = (const ST*)a.win.k + (int64_t)b * a.win.sb + (int64_t)g * a.win.sh;
    vbase = (const ST*)a.win.v + (int64_t)b * a.win.sb + (int64_t)g * a.win.sh;
    kst = a.win.st;
    ring = a.win.ring;
  }
  auto row_of = [&](int j) -> int64_t { return j < 0 ? 0 : (ring > 0 ? j % ring : j); };

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
  // full layer: this unit's step probabilities, key-major [key][lgp] (heads
  // of a key contiguous, so a wave writes each step's values as whole runs),
  // and the running maximum of each (step, head)
  unsigned char* pr_unit =
      FULL ? static_cast<unsigned char*>(a.probs) + (int64_t)unit * a.lus * ProbFmt<TR>::kSlotBytes : nullptr;
  float* pm_unit = FULL ? a.pmax + (int64_t)unit * a.mus : nullptr;

  // key index of list entry t (-1: past the list, negative index or after pos)
  auto key_at = [&](int t) -> int {
    int j = -1;
    if (t < t_end) j = (kind == 0) ? t : (kind == 1 ? idx_row[t] : wbase + t);
    return (j >= 0 && j <= pos) ? j : -1;
  };
  // issue the K and V row loads of one step whose key indices are in kjb
  frag kf[2][KC];
  uint4 vr[NP][4];
  constexpr bool kLdsK = DecodeSmem<TR, D>::kLdsK;
  auto issue_loads = [&](const int* kjb) {
    if constexpr (kLdsK) {  // whole K rows, like V: chunk lane % 16 of key 4q + lane / 16
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = kjb[4 * q + (lane >> 4)];
        kf[q >> 2][q & 3] = __builtin_bit_cast(frag, load16_stream<FULL>(kbase + row_of(j) * kst + 8 * (lane & 15)));
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int j = kjb[16 * kt + col];
        const ST* kr = kbase + row_of(j) * kst;
#pragma unroll
        for (int c = 0; c < KC; ++c) kf[kt][c] = TR::template load8_stream<FULL>(kr + 32 * c + 8 * quad);
      }
    }
    if constexpr (kTrV) {
#pragma unroll
      for (int q = 0; q < NP * 4; ++q) {  // keys 4q .. 4q + 3, lane: chunk lane % 16 of key 4q + lane / 16
        const int j = kjb[4 * q + (lane >> 4)];
        vr[q >> 2][q & 3] = load16_stream<FULL>(vbase + row_of(j) * kst + 8 * (lane & 15));
      }
    } else {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int pidx = lane + 64 * pp;
        const int kq = pidx % (kStep / 4), tc = pidx / (kStep / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = kjb[4 * kq + r];
          vr[pp][r] = load16_stream<FULL>(vbase + row_of(j) * kst + tc * EPC);
        }
      }
    }
  };

  // software pipeline: the next step's loads are in flight while this step computes
  int buf = 0;
  if (t_begin + wave * kStep < t_end) {
    if (lane < kStep) kj[lane] = key_at(t_begin + wave * kStep + lane);
    wave_lds_sync();
    issue_loads(kj);
  }
  for (int t0 = t_begin + wave * kStep; t0 < t_end; t0 += kWaves * kStep) {
    wave_lds_sync();
    frag kfc[2][KC];
    uint4 vrc[NP][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < KC; ++c) kfc[kt][c] = kf[kt][c];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) vrc[pp][r] = vr[pp][r];
    const int* kjc = kj + buf * kStep;
    const int t1 = t0 + kWaves * kStep;
    if (t1 < t_end) {
      int* kjn = kj + (buf ^ 1) * kStep;
      if (lane < kStep) kjn[lane] = key_at(t1 + lane);
      wave_lds_sync();
      issue_loads(kjn);
    }
    buf ^= 1;
    if constexpr (kLdsK) {  // K rows into the wave's LDS tile (chunk c of key k in slot c ^ (k & 15)), then fragments
      unsigned char* ktb = smem + DecodeSmem<TR, D>::kVt + (size_t)wave * kStep * 256;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int key = 4 * q + (lane >> 4), c = lane & 15;
        *reinterpret_cast<frag*>(ktb + key * 256 + ((c ^ (key & 15)) << 4)) = kfc[q >> 2][q & 3];
      }
      wave_lds_sync();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kfc[kt][c] = *reinterpret_cast<const frag*>(ktb + (16 * kt + col) * 256 + (((4 * c + quad) ^ col) << 4));
    }
    // S^T = K . Q^T ; sacc[kt][r] = logit of key 16*kt + 4*quad + r for head col
    f32x4_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) TR::mma(sacc[kt], kfc[kt][c], qf[c]);
    }
    float s[2][4];
    float mt = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kjc[16 * kt + 4 * quad + r];
        s[kt][r] = (j >= 0) ? sacc[kt][r] * a.sl2 : kNegInf;
        mt = fmaxf(mt, s[kt][r]);
      }
    }
    mt = wave_max16x4(mt);
    const float m_new = fmaxf(m_run, mt);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mu);
    float p[2][4];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = fast_exp2(s[kt][r] - mu);
        ls += p[kt][r];
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    if constexpr (FULL) {
      // lane (head col, quad) holds keys 4*quad + r; after the transpose
      // inside each lane quad it holds heads (col & ~3) + e of key
      // 4*quad + (col & 3).  List entry t is key t in the full layer.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float w[4] = {p[kt][0], p[kt][1], p[kt][2], p[kt][3]};
        quad_transpose4(w);
        const int j = t0 + 16 * kt + 4 * quad + (col & 3);
        if (col < a.lgp && j < t_end)
          ProbFmt<TR>::store4(pr_unit + ((int64_t)j * a.lgp + (col & ~3)) * ProbFmt<TR>::kSlotBytes, w);
      }
      if (quad == 0 && col < a.lgp) pm_unit[(int64_t)(t0 / kStep) * a.lgp + col] = mu;
    }
    // rescale output rows (head 4*quad + r) by that head's alpha; nothing to
    // rescale on the wave's first step (o is zero; the sparse layer's waves
    // take one step each)
    if (t0 != t_begin + wave * kStep) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * quad + r);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][r] *= ar;
      }
    }

    unsigned char* vtb = reinterpret_cast<unsigned char*>(vt);
    if constexpr (kTrV) {  // V rows as loaded: key k's chunk c in slot c ^ 2 (k & 7)
#pragma unroll
      for (int q = 0; q < NP * 4; ++q) {
        const int key = 4 * q + (lane >> 4), c = lane & 15;
        *reinterpret_cast<uint4*>(vtb + key * 256 + ((c ^ (2 * (key & 7))) << 4)) = vrc[q >> 2][q & 3];
      }
    } else {
    // stage V transposed: vt[d][key]
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int pidx = lane + 64 * pp;
      const int kq = pidx % (kStep / 4), tc = pidx / (kStep / 4);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        ST* dst = vt + (tc * EPC + e) * VP + 4 * kq;
        if constexpr (TR::kBytes == 2) {
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vrc[pp][0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vrc[pp][1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vrc[pp][2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vrc[pp][3]);
          const int sh = 16 * (e & 1);
          uint2 pk;
          pk.x = ((w0[e >> 1] >> sh) & 0xFFFFu) | (((w1[e >> 1] >> sh) & 0xFFFFu) << 16);
          pk.y = ((w2[e >> 1] >> sh) & 0xFFFFu) | (((w3[e >> 1] >> sh) & 0xFFFFu) << 16);
          *reinterpret_cast<uint2*>(dst) = pk;
        } else {
          const float* f0 = reinterpret_cast<const float*>(&vrc[pp][0]);
          const float* f1 = reinterpret_cast<const float*>(&vrc[pp][1]);
          const float* f2 = reinterpret_cast<const float*>(&vrc[pp][2]);
          const float* f3 = reinterpret_cast<const float*>(&vrc[pp][3]);
          *reinterpret_cast<float4*>(dst) = make_float4(f0[e], f1[e], f2[e], f3[e]);
        }
      }
    }
    }
    wave_lds_sync();

    // O += P . V ; A = P (head = col, keys {4q..4q+3, 16+4q..16+4q+3})
    const frag pa = TR::pack(p[0], p[1]);
    if constexpr (kTrV) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) TR::mma(o[dt], pa, tr_v_frag(vtb, dt, 0, col, quad));
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const ST* row = vt + (16 * dt + col) * VP;
        const quad_t lo = *reinterpret_cast<const quad_t*>(row + 4 * quad);
        const quad_t hi = *reinterpret_cast<const quad_t*>(row + 16 + 4 * quad);
        TR::mma(o[dt], pa, TR::join(lo, hi));
      }
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
    f[r] = fast_exp2(ml_s[wave][h][0] - mu);
  }
  constexpr int OP = DecodeSmem<TR, D>::kOP;
  float* obuf = reinterpret_cast<float*>(smem);  // [kWaves][16][OP]
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) obuf[(wave * 16 + 4 * quad + r) * OP + 16 * dt + col] = o[dt][r] * f[r];
  __syncthreads();

  const int64_t pbase = (int64_t)unit * a.nsplit + split;
  float* po = a.part_o + pbase * a.G * D;
  for (int x = 4 * tid; x < a.G * D; x += 4 * 256) {  // four consecutive d per thread
    const int h = x / D, d = x - h * D;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float4 y = *reinterpret_cast<const float4*>(obuf + (w * 16 + h) * OP + d);
      acc.x += y.x;
      acc.y += y.y;
      acc.z += y.z;
      acc.w += y.w;
    }
    *reinterpret_cast<float4*>(po + x) = acc;
  }
  if (tid < a.G) {
    const int h = tid;
    float M = ml_s[0][h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, ml_s[w][h][0]);
    const float mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += ml_s[w][h][1] * fast_exp2(ml_s[w][h][0] - mu);
    a.part_ml[(pbase * a.G + h) * 2 + 0] = M;
    a.part_ml[(pbase * a.G + h) * 2 + 1] = L;
  }
}

// Sparse layer: merge the splits of one (unit, head) into its global and
// window outputs and apply the sigmoid gate,
//   out = g * o_global + (1 - g) * o_window,  g = 1 / (1 + exp(-w_h)).
// One workgroup of D threads per (unit, head), one output element per thread.
template <typename TR, int D>
__global__ __launch_bounds__(D) void sparse_merge_kernel(DecodeArgs a) {
  __shared__ float wts[kMaxSparseSplits];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.G, h = blockIdx.x - (blockIdx.x / a.G) * a.G;
  const int i = unit % a.Tq, bg = unit / a.Tq;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const float* pml = a.part_ml + (int64_t)unit * a.nsplit * a.G * 2;
  // the head's gate logit, first so that its load overlaps the others
  const float gw = a.gate.p[(int64_t)b * a.gate.sb + (int64_t)i * a.gate.st + g * a.G + h];
  // this thread's output element of every split, loaded before the weights
  // are known so that both reads are in flight together
  const float* po = a.part_o + (int64_t)unit * a.nsplit * a.G * D + (int64_t)h * D + tid;
  float pv[kMaxSparseSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSparseSplits; ++sp) pv[sp] = sp < a.nsplit ? po[(int64_t)sp * a.G * D] : 0.f;
  // weights: lanes 0..nsg-1 of wave 0 handle the global splits, the next
  // lanes the window splits (nsplit <= 64)
  if (tid < 64) {
    const int sp = tid;
    const bool in = sp < a.nsplit;
    const bool win = sp >= a.nsg;
    const float m = in ? pml[(sp * a.G + h) * 2] : kNegInf;
    const float l = in ? pml[(sp * a.G + h) * 2 + 1] : 0.f;
    // branch max and sum over the lanes of the same branch
    const float mg = wave_max_f32((in && !win) ? m : kNegInf), mw = wave_max_f32((in && win) ? m : kNegInf);
    const float mu = win ? (mw == kNegInf ? 0.f : mw) : (mg == kNegInf ? 0.f : mg);
    const float w = in ? exp2f(m - mu) : 0.f;
    const float lg = wave_sum_f32((in && !win) ? l * w : 0.f), lw = wave_sum_f32((in && win) ? l * w : 0.f);
    const float gt = 1.f / (1.f + expf(-gw));
    const float L = win ? lw : lg;
    const float scale = (L > 0.f) ? (win ? (1.f - gt) : gt) / L : 0.f;
    if (in) wts[sp] = w * scale;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxSparseSplits; ++sp)
    if (sp < a.nsplit) acc += wts[sp] * pv[sp];
  reinterpret_cast<typename TR::storage*>(a.out)[(((int64_t)b * a.Tq + i) * a.Hq + g * a.G + h) * D + tid] =
      TR::from_float(acc);
}

struct FinishArgs {
  const float* part_o;
  const float* part_ml;
  const void* probs;   // key-major [unit][key][lgp], see ProbFmt
  const float* pmax;   // [unit][key / 32][lgp]
  int lgp;             // slots per key (4, 8 or 16)
  int64_t lus;         // elements per unit of probs
  int64_t mus;         // floats per unit of pmax
  int nsplit, G, Hkv, Tkv, nchunk, units;
  void* out;
  float* lse;
  float* scores;
};

// Base-2 log-sum-exp of every head of a unit from its split states, into
// lse_s[0..G).  16 threads per head each fold a strided subset of the
// splits' (m, l) pairs in one pass (eight loads in flight), then a 16-lane
// butterfly folds the threads; the order is fixed, so every workgroup of the
// finish kernel computes bit-identical values.
__device__ __forceinline__ void fold_ml(float& M, float& L, float m, float l) {
  const float Mn = fmaxf(M, m);
  const float mu = (Mn == kNegInf) ? 0.f : Mn;
  L = L * exp2f(M - mu) + l * exp2f(m - mu);
  M = Mn;
}
__device__ __forceinline__ void unit_lse2(const float* pml, int nsplit, int G, float* lse_s) {
  const int tid = threadIdx.x, h = tid >> 4, t = tid & 15;
  float M = kNegInf, L = 0.f;
  if (h < G) {
    for (int base = t; base < nsplit; base += 16 * 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = base + 16 * u;
        v[u] = sp < nsplit ? *reinterpret_cast<const float2*>(pml + (sp * G + h) * 2) : make_float2(kNegInf, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) fold_ml(M, L, v[u].x, v[u].y);
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(M, off, 16), l2 = __shfl_xor(L, off, 16);
    fold_ml(M, L, m2, l2);
  }
  if (h < G && t == 0) lse_s[h] = (L > 0.f) ? M + log2f(L) : kNegInf;
  __syncthreads();
}

// Importance scores of a wave's 256 keys (4 groups of 64) from the
// key-major step probabilities, Q = lgp / 4 lanes per key.  The wave's keys
// span 8 steps, so the factor 2^(m - lse2 - shift) that turns a stored value
// into P takes 8 * lgp values: the wave forms them once into its LDS table
// ct (0 for padding heads).  The wave reads the probabilities as whole runs
// of 256 slots: in run xi of a group, lane l holds heads 4*(l % Q) .. +3 of
// key (64/Q)*xi + l/Q; a DPP sum over the key's Q lanes gives its S.  (The
// scratch holds nchunk * kScoreChunk keys per unit, so every run is in it;
// keys past kv_len are read but not stored.)  All loads are issued before
// the unit's LSE is formed (they do not depend on it).
template <typename TR, int Q>
__device__ __forceinline__ void score_runs(const FinishArgs& f, int unit, int key0, float* lse_s, float* ct) {
  using PF = ProbFmt<TR>;
  constexpr int SB = PF::kSlotBytes;
  using PV = std::conditional_t<SB == 3, typename ProbFmt<BF16>::pack_t, float4>;
  constexpr int LG = 4 * Q;   // slots per key
  constexpr int NR = 4 * Q;   // runs of 256 slots
  constexpr int KPR = 64 / Q; // keys per run
  constexpr int NCT = 8 * LG; // (step, head) factors of the wave, <= 128
  const int lane = threadIdx.x & 63, hg = lane % Q;
  const unsigned char* pr = static_cast<const unsigned char*>(f.probs) + ((int64_t)unit * f.lus + (int64_t)key0 * LG) * SB;
  const float* pm = f.pmax + (int64_t)unit * f.mus + (int64_t)(key0 / kStep) * LG;
  PV x[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) x[r] = *reinterpret_cast<const PV*>(pr + (r * 256 + 4 * lane) * SB);
  float mv[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) mv[e] = (lane + 64 * e < NCT) ? pm[lane + 64 * e] : 0.f;
  unit_lse2(f.part_ml + (int64_t)unit * f.nsplit * f.G * 2, f.nsplit, f.G, lse_s);
  // m <= lse2 for every stored key (the clamp only guards the steps whose
  // keys are all masked, where m was taken as 0)
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int t = lane + 64 * e, h = t % LG;
    if (t < NCT) ct[t] = (h < f.G) ? fast_exp2(fminf(mv[e] - lse_s[h], 0.f)) : 0.f;
  }
  wave_lds_sync();
  float* srow = f.scores + (int64_t)unit * f.Tkv;
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    float mine = 0.f;
#pragma unroll
    for (int xi = 0; xi < Q; ++xi) {
      const int r = grp * Q + xi;
      f32x4_t v;
      if constexpr (SB == 3)
        v = PF::unpack(x[r]);
      else
        v = f32x4_t{x[r].x, x[r].y, x[r].z, x[r].w};
      const float4 c = *reinterpret_cast<const float4*>(ct + ((r * KPR + lane / Q) / kStep) * LG + 4 * hg);
      float p = v[0] * c.x + v[1] * c.y + v[2] * c.z + v[3] * c.w;
      if constexpr (Q >= 2) p += dpp_quad<0xB1>(p);
      if constexpr (Q == 4) p += dpp_quad<0x4E>(p);
      mine = (xi == hg) ? p : mine;
    }
    const int j = key0 + 64 * grp + KPR * hg + lane / Q;
    if (j < f.Tkv) srow[j] = mine;
  }
}

// Blocks [0, units*G): output row of one (unit, head): O = sum_s 2^(m_s - lse2) O_s,
//   256 threads = D/4 float4 columns x NPH split phases, eight splits in flight.
// Blocks [units*G, ...): importance scores of one chunk of kScoreChunk keys of a unit:
//   S[b, g, 0, j] = sum over the group's heads of 2^(logit2[h, j] - lse2[h]),
//   formed as the stored 2^(logit2 - m) times 2^(m - lse2).
template <typename TR, int D>
__global__ __launch_bounds__(256) void decode_full_finish_kernel(FinishArgs f) {
  constexpr int DV = D / 4;      // float4 columns of a row
  constexpr int NPH = 256 / DV;  // split phases of the row merge
  __shared__ float lse_s[16];
  __shared__ __align__(16) float red[NPH][D];
  __shared__ __align__(16) float ct_s[4][128];
  const int tid = threadIdx.x;
  const int nrow = f.units * f.G;
  const int Hq = f.Hkv * f.G;
  if ((int)blockIdx.x < nrow) {
    const int unit = blockIdx.x / f.G, h = blockIdx.x - (blockIdx.x / f.G) * f.G;
    const int b = unit / f.Hkv, g = unit - b * f.Hkv;
    const float* pml = f.part_ml + (int64_t)unit * f.nsplit * f.G * 2;
    const float* po = f.part_o + (int64_t)unit * f.nsplit * f.G * D;
    const int d4 = tid % DV, ph = tid / DV;
    // batches of eight splits per thread (loading the first before the LSE
    // is formed needs 40 more VGPRs and costs the score blocks occupancy)
    float m[8];
    float4 o[8];
    auto load_batch = [&](int base) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = base + NPH * u;
        const bool in = sp < f.nsplit;
        m[u] = in ? pml[(sp * f.G + h) * 2] : kNegInf;
        o[u] = in ? *reinterpret_cast<const float4*>(po + ((int64_t)sp * f.G + h) * D + 4 * d4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    unit_lse2(pml, f.nsplit, f.G, lse_s);
    const float l2 = lse_s[h];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = ph; base < f.nsplit; base += NPH * 8) {
      load_batch(base);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = exp2f(m[u] - l2);
        acc.x += w * o[u].x;
        acc.y += w * o[u].y;
        acc.z += w * o[u].z;
        acc.w += w * o[u].w;
      }
    }
    *reinterpret_cast<float4*>(&red[ph][4 * d4]) = acc;
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
      for (int x = 0; x < NPH; ++x) sum += red[x][tid];
      const int hq = g * f.G + h;
      reinterpret_cast<typename TR::storage*>(f.out)[((int64_t)b * Hq + hq) * D + tid] = TR::from_float(sum);
      if (tid == 0 && f.lse) f.lse[(int64_t)b * Hq + hq] = l2 * kLn2;
    }
    return;
  }
  const int bid = blockIdx.x - nrow;
  const int unit = bid / f.nchunk, c = bid - (bid / f.nchunk) * f.nchunk;
  const int key0 = c * kScoreChunk + (tid >> 6) * (kScoreChunk / 4);  // the wave's 256 keys
  float* ct = ct_s[tid >> 6];
  if (f.lgp == 4)
    score_runs<TR, 1>(f, unit, key0, lse_s, ct);
  else if (f.lgp == 8)
    score_runs<TR, 2>(f, unit, key0, lse_s, ct);
  else
    score_runs<TR, 4>(f, unit, key0, lse_s, ct);
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
  a.wchunk = p.wchunk;
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
  p.wchunk = 0;
  p.nsplit = (g.Tkv + chunk - 1) / chunk;
  p.nsg = p.nsplit;
  return p;
}

#ifndef HYS_SPARSE_GSPLITS
#define HYS_SPARSE_GSPLITS 48
#endif

// Split-kernel workgroups resident at once: the instantiation's workgroups
// per CU at its register budget (__launch_bounds__: two for bf16, one for
// fp32) times the 256 CUs of gfx950.  A compile-time figure, not a device
// query, because the same plan sizes the workspace on hosts without a GPU.
// When the units would need a few rounds of split workgroups, fewer and
// longer global splits keep every workgroup in the first round, its waves
// pipelining their steps, instead of a second round of single-step waves
// (decode, batch 16, 8K context: 23.7 -> 21.8 us per sparse layer; batch 4
// at 128K keeps its 16 global splits).  The cap applies only while at least
// two global splits per unit fit: one long split per unit was measured
// slower (per-query prefill at 8K queries: 6.24 vs 5.12 ms with the default
// splits).
constexpr int kGfx950CUs = 256;
inline int sparse_resident_wgs(const Geom& g) { return kGfx950CUs * (g.dtype == 1 ? 2 : 1); }

DecodePlan plan_sparse_rows(const Geom& g, int k_top, int window) {
  // at most HYS_SPARSE_GSPLITS (<= 48) global and 16 window splits
  // (kMaxSparseSplits merge weights)
  static_assert(HYS_SPARSE_GSPLITS >= 1 && HYS_SPARSE_GSPLITS <= 48, "global split bound");
  DecodePlan p{};
  const int quantum = kWaves * kStep;
  p.units = g.B * g.Hkv * g.Tq;
  int cw = (window + 15) / 16;
  cw = (cw + quantum - 1) / quantum * quantum;
  p.wchunk = cw;
  const int nw = (window + cw - 1) / cw;
  int gs = HYS_SPARSE_GSPLITS;
  const int fit = sparse_resident_wgs(g) / p.units - nw;
  if (fit >= 2 && fit < gs) gs = fit;
  int cg = (k_top + gs - 1) / gs;
  cg = (cg + quantum - 1) / quantum * quantum;
  p.chunk = cg;
  p.nsg = (k_top + cg - 1) / cg;
  p.nsplit = p.nsg + nw;
  return p;
}

// Full-decode probability scratch: per unit (b, g), key-major rows of lgp
// slots (the group's G heads, padded to 4, 8 or 16) of 3 bytes (bf16 inputs,
// see ProbFmt) or 4, for kv_len rounded up to whole score chunks; and the
// running maxima, lgp floats per 32-key step.
static int prob_slots(const Geom& g) { return g.G <= 4 ? 4 : (g.G <= 8 ? 8 : 16); }
static int64_t score_keys(const Geom& g) { return (int64_t)(g.Tkv + kScoreChunk - 1) / kScoreChunk * kScoreChunk; }
static int64_t prob_unit_elems(const Geom& g) { return score_keys(g) * prob_slots(g); }
static int64_t pmax_unit_floats(const Geom& g) { return score_keys(g) / kStep * prob_slots(g); }
static size_t prob_elem_bytes(const Geom& g) { return g.dtype == 1 ? 3 : 4; }

static size_t decode_ws(const Geom& g, const DecodePlan& p, bool full) {
  size_t n = align_up((size_t)p.units * p.nsplit * g.G * g.D * sizeof(float));
  n += align_up((size_t)p.units * p.nsplit * g.G * 2 * sizeof(float));
  if (full) {
    n += align_up((size_t)p.units * prob_unit_elems(g) * prob_elem_bytes(g));
    n += align_up((size_t)p.units * pmax_unit_floats(g) * sizeof(float));
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
    w.probs = c;
    c += align_up((size_t)p.units * prob_unit_elems(g) * prob_elem_bytes(g));
    w.pmax = reinterpret_cast<float*>(c);
  }
  return w;
}

hipError_t launch_full_decode(const Geom& g, const void* q, const void* k, const void* v, void* out,
                              float* lse, float* scores, void* ws, hipStream_t st) {
  const DecodePlan p = plan_full_decode(g);
  const DecodeWs w = carve_decode_ws(g, p, ws, true);
  DecodeArgs a = make_args(g, p, q, k, v);
  a.probs = w.probs;
  a.pmax = w.pmax;
  a.lgp = prob_slots(g);
  a.lus = prob_unit_elems(g);
  a.mus = pmax_unit_floats(g);
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  FinishArgs f{};
  f.part_o = w.part_o;
  f.part_ml = w.part_ml;
  f.probs = w.probs;
  f.pmax = w.pmax;
  f.lgp = prob_slots(g);
  f.lus = prob_unit_elems(g);
  f.mus = pmax_unit_floats(g);
  f.nsplit = p.nsplit;
  f.G = g.G;
  f.Hkv = g.Hkv;
  f.Tkv = g.Tkv;
  f.nchunk = (g.Tkv + kScoreChunk - 1) / kScoreChunk;
  f.units = p.units;
  f.out = out;
  f.lse = lse;
  f.scores = scores;
  hipError_t e = hipSuccess;
  HYS_DISPATCH(g, {
    e = launch("full_decode_split", decode_split_kernel<TR, DD, true>, dim3(p.units * p.nsplit), dim3(256), 0, st,
               a);
    if (e == hipSuccess)
      e = launch("full_decode_finish", decode_full_finish_kernel<TR, DD>, dim3(p.units * (g.G + f.nchunk)),
                 dim3(256), 0, st, f);
  });
  return e;
}

hipError_t launch_sparse_rows(const Geom& g, const void* q, const void* k, const void* v,
                              const int32_t* idx, int k_top, int score_block, int window,
                              const GateRef& gate, const WinRef& win, void* out, void* ws, hipStream_t st) {
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
  a.gate = gate;
  a.win = win;
  a.out = out;
  hipError_t e = hipSuccess;
  HYS_DISPATCH(g, {
    e = launch("sparse_decode", decode_split_kernel<TR, DD, false>, dim3(p.units * p.nsplit), dim3(256), 0, st, a);
    if (e == hipSuccess)
      e = launch("sparse_merge", sparse_merge_kernel<TR, DD>, dim3(p.units * g.G), dim3(DD), 0, st, a);
  });
  return e;
}

}  // namespace hys
