// LDS-staged 64-key tiles and the per-wave MFMA attention step used by the
// prefill kernels (full layer and block-sparse layer).
//
// A workgroup stages one tile of 64 key rows at a time: K row-major (A/B
// fragments read 16 contiguous bytes per lane) and V transposed (Vt[d][key],
// so the PV product's B fragments are 8-byte reads of four consecutive keys).
// Key rows may come from any list (contiguous range, gathered indices,
// window); a row whose list entry is invalid is loaded from key 0 and masked
// with index -1, so every load stays in bounds.
//
// Rows: a "row tile" is 16 (query, head) rows of one KV group.  In the
// S^T = K . Q^T product a lane owns row (l % 16) of the tile; in the O = P.V
// accumulator it owns rows 4*(l/16) + r, r = 0..3 (16x16 MFMA layout).
#pragma once

#include "hys_common.h"

namespace hys {

constexpr int kTK = 64;  // keys per tile

template <typename TR, int D>
struct TileLayout {
  static constexpr int EPC = 16 / TR::kBytes;          // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per row
  static constexpr int KP = D * TR::kBytes + 16;       // K row pitch, bytes (68 dwords for D = 128 bf16)
  // Vt row pitch: 68 elements = 34 dwords (bf16) or 68 dwords (fp32), so the
  // fragment reads of 16 (bf16, 8-byte) or 8 (fp32, 16-byte) consecutive d
  // rows hit distinct banks.
  static constexpr int VPE = kTK + 4;
  static constexpr int kKBytes = kTK * KP;
  static constexpr int kVBytes = D * VPE * TR::kBytes;
  static constexpr int kBytes = kKBytes + kVBytes;
};

// Per-thread staging registers of one tile (global -> registers -> LDS), so
// the next tile's loads can be in flight while the current tile is used.
template <typename TR, int D, int NT, bool WITH_V>
struct TileStage {
  using ST = typename TR::storage;
  using L = TileLayout<TR, D>;
  static constexpr int NK = (kTK * L::CPR + NT - 1) / NT;
  // V is staged by key pairs: unit u = (pair u % 32, chunk u / 32), so the 32
  // lanes of one LDS store pass write 32 consecutive dwords of a Vt row
  // (bf16; fp32 stores 8 bytes per lane, 16 lanes per pass)
  static constexpr int NV = WITH_V ? (32 * L::CPR + NT - 1) / NT : 0;
  static constexpr bool kExactK = (kTK * L::CPR) % NT == 0;
  static constexpr bool kExactV = (32 * L::CPR) % NT == 0;
  // native vectors, not HIP's uint4 struct: struct copies become memcpys that
  // keep the staging array in scratch memory
  u32x4_t kr[NK];
  u32x4_t vr[NV > 0 ? NV : 1][2];
  int jk;

  // key(t) -> key index (position) of tile entry t, or -1 when the entry is
  // invalid; the row read for key j is row(j) of kbase / vbase (identity
  // unless the keys live in a ring of slots)
  template <class KeyFn>
  __device__ __forceinline__ void load(const ST* kbase, const ST* vbase, int64_t ks_t, KeyFn key) {
    load(kbase, vbase, ks_t, key, [](int j) { return j; });
  }
  template <class KeyFn, class RowFn>
  __device__ __forceinline__ void load(const ST* kbase, const ST* vbase, int64_t ks_t, KeyFn key, RowFn row) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int x = tid + s * NT;
      // the guard is static when NT divides the tile's chunk count: a
      // conditional write here would keep kr out of registers
      if (kExactK || x < kTK * L::CPR) {
        const int t = x / L::CPR, c = x - (x / L::CPR) * L::CPR;
        const int j = key(t);
        kr[s] = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)(j >= 0 ? row(j) : 0) * ks_t + c * L::EPC);
      }
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int s = 0; s < NV; ++s) {
        const int x = tid + s * NT;
        if (kExactV || x < 32 * L::CPR) {
          const int kp = x & 31, c = x >> 5;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int j = key(2 * kp + r);
            vr[s][r] = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)(j >= 0 ? row(j) : 0) * ks_t + c * L::EPC);
          }
        }
      }
    }
    jk = (tid < kTK) ? key(tid) : -1;
  }

  __device__ __forceinline__ void store(unsigned char* sm, int* kj) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int x = tid + s * NT;
      if (kExactK || x < kTK * L::CPR) {
        const int t = x / L::CPR, c = x - (x / L::CPR) * L::CPR;
        *reinterpret_cast<u32x4_t*>(sm + t * L::KP + c * 16) = kr[s];
      }
    }
    if constexpr (WITH_V) {
      ST* vt = reinterpret_cast<ST*>(sm + L::kKBytes);
#pragma unroll
      for (int s = 0; s < NV; ++s) {
        const int x = tid + s * NT;
        if (kExactV || x < 32 * L::CPR) {
          const int kp = x & 31, c = x >> 5;
#pragma unroll
          for (int e = 0; e < L::EPC; ++e) {
            ST* dst = vt + (c * L::EPC + e) * L::VPE + 2 * kp;
            if constexpr (TR::kBytes == 2) {
              const int w = e >> 1, sh = 16 * (e & 1);
              const uint32_t a0 = (vr[s][0][w] >> sh) & 0xFFFFu;
              const uint32_t a1 = (vr[s][1][w] >> sh) & 0xFFFFu;
              *reinterpret_cast<uint32_t*>(dst) = a0 | (a1 << 16);
            } else {
              typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
              *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{vr[s][0][e], vr[s][1][e]};
            }
          }
        }
      }
    }
    if (tid < kTK) kj[tid] = jk;
  }
};

// K fragment of key sub-tile kt (16 keys) for k-step c, from the staged tile:
// lane (key = l % 16, group = l / 16) gets K[16*kt + key][32c + 8*group + e].
template <typename TR, int D>
__device__ __forceinline__ typename TR::frag lds_k_frag(const unsigned char* sm, int kt, int c, int col, int quad) {
  using L = TileLayout<TR, D>;
  return TR::load8(reinterpret_cast<const typename TR::storage*>(sm + (16 * kt + col) * L::KP) + 32 * c + 8 * quad);
}

// Vt fragment for the P.V product: lane (d = 16*dt + l % 16, group q) gets
// keys {32kk + 4q + e} (e < 4) and {32kk + 16 + 4q + e - 4} (e >= 4).
template <typename TR, int D>
__device__ __forceinline__ typename TR::frag lds_v_frag(const unsigned char* sm, int dt, int kk, int col, int quad) {
  using L = TileLayout<TR, D>;
  using quad_t = typename TR::quad_t;
  const typename TR::storage* row =
      reinterpret_cast<const typename TR::storage*>(sm + L::kKBytes) + (16 * dt + col) * L::VPE + 32 * kk;
  const quad_t lo = *reinterpret_cast<const quad_t*>(row + 4 * quad);
  const quad_t hi = *reinterpret_cast<const quad_t*>(row + 16 + 4 * quad);
  return TR::join(lo, hi);
}

// Online-softmax state of RTW row tiles of one wave.
template <int RTW, int D>
struct RowState {
  f32x4_t o[RTW][D / 16];
  float m[RTW];  // running max (base 2) of the lane's row (l % 16)
  float l[RTW];  // lane-partial running sum of that row
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      m[rt] = kNegInf;
      l[rt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Lazy rescaling: a row's running max m is only raised when some logit of the
// tile exceeds it by more than this many powers of two, so unnormalised
// probabilities stay below 2^kRescaleSlack and the O rescale (and its
// cross-lane traffic) is skipped for most tiles.  O / l is unchanged: m
// cancels between numerator and denominator.
constexpr float kRescaleSlack = 8.f;

// The attention step of one wave on one staged tile, in three parts (QK^T,
// online softmax, PV) so that a caller can interleave the parts of
// different tiles.
//
// qk_tile: S^T[key][row] for the wave's RTW row tiles; sacc[rt][kt][r] is the
// logit of key 16*kt + 4*quad + r for the lane's row (l % 16).
template <typename TR, int D, int RTW>
__device__ __forceinline__ void qk_tile(f32x4_t (&sacc)[RTW][4], const typename TR::frag (&qf)[RTW][D / 32],
                                        const unsigned char* sm) {
  using frag = typename TR::frag;
  constexpr int KC = D / 32;
  const int lane = threadIdx.x & 63, col = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    frag kf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) kf[c] = lds_k_frag<TR, D>(sm, kt, c, col, quad);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      sacc[rt][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) TR::mma(sacc[rt][kt], kf[c], qf[rt][c]);
    }
  }
}

// mask_vote_tile: masks the logits when `mask` (wave-uniform) is set (valid(rt,
// j) says whether key j may be used by the lane's row of row tile rt; j < 0
// marks an invalid tile entry), then raises the running maxima that the tile
// exceeds by more than the slack, rescaling O and l (one wave vote).  After
// it, exp_pack_tile turns the logits into probabilities.
// NKT is the number of 16-key sub-tiles the logits cover (4: a whole tile).
template <typename TR, int D, int RTW, int NKT, class Keys, class Valid>
__device__ __forceinline__ void mask_vote_tile_k(RowState<RTW, D>& st, f32x4_t (&sacc)[RTW][NKT], Keys keys,
                                                 float sl2, bool mask, Valid valid) {
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63, quad = lane >> 4;
  if (mask) {  // masked logits in place
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = keys(16 * kt + 4 * quad + r);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          if (!(j >= 0 && valid(rt, j))) sacc[rt][kt][r] = kNegInf;
      }
  }
  // lane-local maxima, and one vote per tile on whether any row must raise
  // its running max
  float lm[RTW];
  bool over = false;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    lm[rt] = kNegInf;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) lm[rt] = fmaxf(lm[rt], sacc[rt][kt][r]);
    // scale > 0, so max(raw) * sl2 is the max of the scaled logits
    over = over || (lm[rt] * sl2 > st.m[rt] + kRescaleSlack);
  }
  if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float m_new = fmaxf(st.m[rt], wave_max16x4(lm[rt]) * sl2);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(st.m[rt] - m_new);
      st.l[rt] *= alpha;
      st.m[rt] = m_new;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * quad + r);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.o[rt][dt][r] *= ar;
      }
    }
  }
}

// The staged-tile form: tile entry e's key index is kj[e].
template <typename TR, int D, int RTW, class Valid>
__device__ __forceinline__ void mask_vote_tile(RowState<RTW, D>& st, f32x4_t (&sacc)[RTW][4], const int* kj,
                                               float sl2, bool mask, Valid valid) {
  mask_vote_tile_k<TR, D, RTW>(st, sacc, [kj](int e) { return kj[e]; }, sl2, mask, valid);
}

// exp_pack_tile: probabilities 2^(logit * sl2 - m) of a tile whose maxima
// mask_vote_tile has settled, added to the row sums and packed as PV's A
// operand.
template <typename TR, int D, int RTW, int NKT>
__device__ __forceinline__ void exp_pack_tile(RowState<RTW, D>& st, const f32x4_t (&sacc)[RTW][NKT], float sl2,
                                              typename TR::frag (&pa)[RTW][NKT / 2]) {
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float nmu = (st.m[rt] == kNegInf) ? 0.f : -st.m[rt];
    float p[NKT][4];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kt][r] = fast_exp2(fmaf(sacc[rt][kt][r], sl2, nmu));
        ls += p[kt][r];
      }
    st.l[rt] += ls;
#pragma unroll
    for (int kk = 0; kk < NKT / 2; ++kk) pa[rt][kk] = TR::pack(p[2 * kk], p[2 * kk + 1]);
  }
}

// softmax_tile: mask_vote_tile then exp_pack_tile.
template <typename TR, int D, int RTW, class Valid>
__device__ __forceinline__ void softmax_tile(RowState<RTW, D>& st, f32x4_t (&sacc)[RTW][4], const int* kj,
                                             float sl2, bool mask, Valid valid, typename TR::frag (&pa)[RTW][2]) {
  mask_vote_tile<TR, D, RTW>(st, sacc, kj, sl2, mask, valid);
  exp_pack_tile<TR, D, RTW>(st, sacc, sl2, pa);
}

// pv_tile: O += P . V for the wave's row tiles.
template <typename TR, int D, int RTW>
__device__ __forceinline__ void pv_tile(RowState<RTW, D>& st, const typename TR::frag (&pa)[RTW][2],
                                        const unsigned char* sm) {
  using frag = typename TR::frag;
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63, col = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const frag vb = lds_v_frag<TR, D>(sm, dt, kk, col, quad);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) TR::mma(st.o[rt][dt], pa[rt][kk], vb);
    }
}

// The whole step on one tile.  One code path for masked and unmasked tiles
// keeps a single copy of the step in the caller.
template <typename TR, int D, int RTW, class Valid>
__device__ __forceinline__ void attend_tile(RowState<RTW, D>& st, const typename TR::frag (&qf)[RTW][D / 32],
                                            const unsigned char* sm, const int* kj, float sl2, bool mask,
                                            Valid valid) {
  f32x4_t sacc[RTW][4];
  qk_tile<TR, D, RTW>(sacc, qf, sm);
  typename TR::frag pa[RTW][2];
  softmax_tile<TR, D, RTW>(st, sacc, kj, sl2, mask, valid, pa);
  pv_tile<TR, D, RTW>(st, pa, sm);
}

// ------------------------------------------------------ LDS-DMA staged tiles
// bf16, head_dim 128.  A stage holds one 64-key tile, K then V, each as 64
// unpadded 256-byte rows written by global_load_lds_dwordx4: one instruction
// fills 1 KB (four rows, lane l -> bytes 16 l .. 16 l + 15), and the lane ->
// global address mapping decides which 16-byte chunk lands in which slot.
// Chunk c (elements 8c .. 8c + 7) of key k sits in slot
//   K: c ^ (k & 15)      the 16 lanes of an A-fragment read (16 keys, one
//                        chunk) hit 16 different slots;
//   V: c ^ 2 (k & 7)     a transposed read (4 keys x 2 chunks per 16 lanes)
//                        hits 8 different slots, and lane groups 0 / 1 use
//                        the two halves of the banks.
// The DMA needs no staging registers and no LDS store instructions; the
// caller keeps several stages in flight and waits with vmcnt.

// One 16-byte-per-lane LDS DMA: lane l's 16 bytes at `gaddr` go to LDS
// address lds + 16 l (lds must be the same in every lane: it is M0).  Written
// as inline asm so that the compiler's own wait insertion, which cannot tell
// the ring's stages apart, does not drain the DMA before every LDS read; the
// callers wait with explicit vmcnt counts (these loads complete in issue
// order, so loads unknown to the compiler only make its waits stricter).
// M0 is saved and restored around the load (the compiler owns it), and one
// wait state separates the M0 write from the LDS DMA that reads it.
__device__ __forceinline__ void lds_dma16(const void* gaddr, HYS_LDS void* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(m0v)
      : "memory");
}

struct DmaTile {
  static constexpr int kRow = 256;           // bytes per key row (128 bf16)
  static constexpr int kHalf = kTK * kRow;   // 16 KB: K, then V
  static constexpr int kBytes = 2 * kHalf;
};

// Issue the DMA of tile keys t0 .. t0 + 63 into `stage`; keys past `last`
// (kv_len - 1) are loaded from row `last` and must be masked by the caller.
// The NW waves share the 32 one-kilobyte instructions (32 / NW each).
template <int NW>
__device__ __forceinline__ void dma_tile(unsigned char* stage, const uint16_t* kbase, const uint16_t* vbase,
                                         int64_t ks_t, int t0, int last) {
  static_assert(16 % NW == 0, "waves must divide the 16 instructions per tensor");
  constexpr int IPW = 16 / NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, slot = lane & 15;
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int m = wave * IPW + x;  // rows 4m .. 4m + 3
    const int row = 4 * m + (lane >> 4);
    const int64_t j = min(t0 + row, last);
    lds_dma16(kbase + j * ks_t + 8 * (slot ^ (row & 15)), (HYS_LDS void*)(stage + 1024 * m));
    lds_dma16(vbase + j * ks_t + 8 * (slot ^ (2 * (row & 7))), (HYS_LDS void*)(stage + DmaTile::kHalf + 1024 * m));
  }
}

// K only (16 KB stage): the NW waves share the 16 one-kilobyte instructions.
template <int NW>
__device__ __forceinline__ void dma_tile_k(unsigned char* stage, const uint16_t* kbase, int64_t ks_t, int t0,
                                           int last) {
  static_assert(16 % NW == 0, "waves must divide the 16 instructions per tensor");
  constexpr int IPW = 16 / NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, slot = lane & 15;
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int m = wave * IPW + x;
    const int row = 4 * m + (lane >> 4);
    const int64_t j = min(t0 + row, last);
    lds_dma16(kbase + j * ks_t + 8 * (slot ^ (row & 15)), (HYS_LDS void*)(stage + 1024 * m));
  }
}

// A tile staged through registers into the DMA stage layout (bf16, head_dim
// 128), for gathered rows: each thread loads whole 16-byte chunks of a key's
// K and V rows (chunk x & 15 of tile entry x >> 4) and stores them at their
// swizzled slots, so the tile is read with dma_k_frag / dma_v_frag and V
// needs no transposition on the way in.  Same interface as TileStage; a row
// whose entry is invalid is loaded from key 0 and masked with index -1.
template <int NT>
struct SwTileStage {
  static constexpr int kChunks = kTK * 16;  // 16-byte chunks per tensor
  static_assert(kChunks % NT == 0, "threads must divide the tile's chunks");
  static constexpr int NC = kChunks / NT;
  u32x4_t kr[NC];
  u32x4_t vr[NC];
  int jk;

  template <class KeyFn>
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase, int64_t ks_t, KeyFn key) {
    load(kbase, vbase, ks_t, key, [](int j) { return j; });
  }
  template <class KeyFn, class RowFn>
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase, int64_t ks_t, KeyFn key,
                                       RowFn row) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int s = 0; s < NC; ++s) {
      const int x = tid + s * NT, t = x >> 4, c = x & 15;
      const int j = key(t);
      const int64_t off = (int64_t)(j >= 0 ? row(j) : 0) * ks_t + 8 * c;
      kr[s] = *reinterpret_cast<const u32x4_t*>(kbase + off);
      vr[s] = *reinterpret_cast<const u32x4_t*>(vbase + off);
    }
    jk = (tid < kTK) ? key(tid) : -1;
  }
  __device__ __forceinline__ void store(unsigned char* stage, int* kj) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int s = 0; s < NC; ++s) {
      const int x = tid + s * NT, t = x >> 4, c = x & 15;
      *reinterpret_cast<u32x4_t*>(stage + t * DmaTile::kRow + ((c ^ (t & 15)) << 4)) = kr[s];
      *reinterpret_cast<u32x4_t*>(stage + DmaTile::kHalf + t * DmaTile::kRow + ((c ^ (2 * (t & 7))) << 4)) = vr[s];
    }
    if (tid < kTK) kj[tid] = jk;
  }
};

// K fragment (same lanes and k order as lds_k_frag) from a DMA stage.
__device__ __forceinline__ bf16x8_t dma_k_frag(const unsigned char* stage, int kt, int c, int col, int quad) {
  const int row = 16 * kt + col;  // row & 15 == col
  return __builtin_bit_cast(bf16x8_t,
                            *reinterpret_cast<const u32x4_t*>(stage + row * DmaTile::kRow + (((4 * c + quad) ^ col) << 4)));
}

// V fragment for P.V (same lanes and key order as lds_v_frag) from a DMA
// stage's V half (transposed LDS read, see tr_v_frag).
__device__ __forceinline__ bf16x8_t dma_v_frag(const unsigned char* stage, int dt, int kk, int col, int quad) {
  return tr_v_frag(stage + DmaTile::kHalf, dt, kk, col, quad);
}

// The attention step on a DMA stage; keys(e) is the key index of tile entry
// e (-1: invalid), evaluated only when the tile is masked.
template <int RTW, class Keys, class Valid>
__device__ __forceinline__ void attend_tile_dma(RowState<RTW, 128>& st, const bf16x8_t (&qf)[RTW][4],
                                                const unsigned char* stage, Keys keys, float sl2, bool mask,
                                                Valid valid) {
  const int lane = threadIdx.x & 63, col = lane & 15, quad = lane >> 4;
  // logits of the tile's four 16-key sub-tiles
  auto qk = [&](f32x4_t(&sacc)[RTW][4]) {
    // the next sub-tile's K fragments are read while this one's MFMAs run
    bf16x8_t kf[2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[0][c] = dma_k_frag(stage, 0, c, col, quad);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt + 1 < 4)
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[(kt + 1) & 1][c] = dma_k_frag(stage, kt + 1, c, col, quad);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        sacc[rt][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) BF16::mma(sacc[rt][kt], kf[kt & 1][c], qf[rt][c]);
      }
    }
  };
  f32x4_t sacc[RTW][4];
  qk(sacc);
  bf16x8_t pa[RTW][2];
  mask_vote_tile_k<BF16, 128, RTW>(st, sacc, keys, sl2, mask, valid);
  exp_pack_tile<BF16, 128, RTW>(st, sacc, sl2, pa);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8_t vb = dma_v_frag(stage, dt, kk, col, quad);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) BF16::mma(st.o[rt][dt], pa[rt][kk], vb);
    }
}

// Whether a wave must mask a staged tile: some entry is invalid (j < 0) or
// lies after `pos_min`, the smallest position among the wave's rows.  One
// LDS read per lane and a ballot; the result is wave-uniform.
__device__ __forceinline__ bool tile_needs_mask(const int* kj, int pos_min) {
  const int j = kj[threadIdx.x & 63];
  return __builtin_amdgcn_ballot_w64(j < 0 || j > pos_min) != 0;
}

}  // namespace hys
