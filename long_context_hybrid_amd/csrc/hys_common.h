// Device-side building blocks shared by the gfx950 kernels of libhysparse.
//
// Element traits pair a storage type with one 16x16 MFMA "k-step" of 32
// products per output element:
//   BF16: one v_mfma_f32_16x16x32_bf16 (8 bf16 per lane per operand)
//   F32 : eight v_mfma_f32_16x16x4_f32 (8 floats per lane per operand; the
//         lane's e-th element feeds the e-th instruction)
// In both, lane l holds operand row/column (l % 16) and eight k-values owned
// by lane group (l / 16).  Which k a (group, element) slot stands for is the
// caller's choice, as long as the A and B operands agree: the contraction sums
// over all 32 slots.  Accumulators follow the 16x16 layout: lane l holds
// rows 4*(l/16) + r (r = 0..3) of column l % 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hys {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 2^x with one v_exp_f32: results below 2^-126 flush to zero (a probability
// that small is below any tolerance of the sums it enters).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load; NT = true marks it non-temporal (streamed once, not worth
// keeping in the caches: the full layer's pass over the whole cache).
template <bool NT>
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  if constexpr (NT) {
    const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(u[0], u[1], u[2], u[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

struct BF16 {
  using storage = uint16_t;
  using frag = bf16x8_t;
  static constexpr int kBytes = 2;
  // 8 consecutive elements from 16-byte aligned memory
  __device__ static __forceinline__ frag load8(const storage* p) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(frag, u);
  }
  template <bool NT>
  __device__ static __forceinline__ frag load8_stream(const storage* p) {
    return __builtin_bit_cast(frag, load16_stream<NT>(p));
  }
  __device__ static __forceinline__ frag zero8() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ static __forceinline__ storage from_float(float x) { return f32_to_bf16_rne(x); }
  __device__ static __forceinline__ float to_float(storage x) { return bf16_to_f32(x); }
  // pack two groups of four floats (RNE) into one fragment
  __device__ static __forceinline__ frag pack(const float* lo4, const float* hi4) {
    const u32x4_t u = {pack_bf16x2(lo4[0], lo4[1]), pack_bf16x2(lo4[2], lo4[3]), pack_bf16x2(hi4[0], hi4[1]),
                       pack_bf16x2(hi4[2], hi4[3])};
    return __builtin_bit_cast(frag, u);
  }
  // four consecutive elements (8 bytes, 8-byte aligned) as a raw vector
  typedef uint2 quad_t;
  __device__ static __forceinline__ frag join(quad_t lo, quad_t hi) {
    return __builtin_bit_cast(frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

struct F32 {
  using storage = float;
  using frag = f32x8_t;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ frag load8(const storage* p) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return f;
  }
  template <bool NT>
  __device__ static __forceinline__ frag load8_stream(const storage* p) {
    const uint4 a = load16_stream<NT>(p), b = load16_stream<NT>(p + 4);
    frag f;
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
    return f;
  }
  __device__ static __forceinline__ frag zero8() {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.f;
    return f;
  }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }
  __device__ static __forceinline__ storage from_float(float x) { return x; }
  __device__ static __forceinline__ float to_float(storage x) { return x; }
  __device__ static __forceinline__ frag pack(const float* lo4, const float* hi4) {
    frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = lo4[e]; f[4 + e] = hi4[e]; }
    return f;
  }
  typedef float4 quad_t;
  __device__ static __forceinline__ frag join(quad_t lo, quad_t hi) {
    frag f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  }
};

// Order-preserving key of a float32 bit pattern (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}

// Compiler barrier plus wait for this wave's outstanding LDS operations, used
// between lanes of one wave exchanging data through a wave-private LDS region.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Cross-row exchange with the gfx950 permlane swaps.  With both operands the
// same register, permlane16_swap returns, in every lane l, the values of lanes
// (l & ~16) and (l | 16); permlane32_swap those of (l & ~32) and (l | 32).
__device__ __forceinline__ void pair16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// max / sum over the four lanes l, l^16, l^32, l^48 that share (l % 16); the
// sum is formed in the same order in all four lanes (bit-identical results)
__device__ __forceinline__ float wave_max16x4(float x) {
  float a, b;
  pair16(x, a, b);
  x = fmaxf(a, b);
  pair32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum16x4(float x) {
  float a, b;
  pair16(x, a, b);
  x = a + b;
  pair32(x, a, b);
  return a + b;
}

// DPP quad_perm move inside each group of four lanes: CTRL 0xB1 = lanes
// [1,0,3,2] (partner l ^ 1), 0x4E = [2,3,0,1] (partner l ^ 2).
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (row
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the row broadcasts of
// lanes 15 and 31 into the rows above); lanes without a source add 0.  Lane
// layout checked against a CPU prefix sum on the GPU.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWMASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Minimum and maximum over the 64 lanes of a wave (every lane gets both):
// DPP moves inside each row of 16 lanes, then the four row results.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_or_self(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp_or_self<0xB1>(mn));  // quad_perm [1,0,3,2]
  mx = max(mx, dpp_or_self<0xB1>(mx));
  mn = min(mn, dpp_or_self<0x4E>(mn));  // quad_perm [2,3,0,1]
  mx = max(mx, dpp_or_self<0x4E>(mx));
  mn = min(mn, dpp_or_self<0x124>(mn));  // row_ror:4
  mx = max(mx, dpp_or_self<0x124>(mx));
  mn = min(mn, dpp_or_self<0x128>(mn));  // row_ror:8
  mx = max(mx, dpp_or_self<0x128>(mx));
  // readlane returns int: compare the row results as unsigned
  auto lane_u = [](uint32_t x, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)x, l); };
  mn = min(min(lane_u(mn, 0), lane_u(mn, 16)), min(lane_u(mn, 32), lane_u(mn, 48)));
  mx = max(max(lane_u(mx, 0), lane_u(mx, 16)), max(lane_u(mx, 32), lane_u(mx, 48)));
}

// Float maximum / sum over the 64 lanes of a wave: DPP moves inside each row
// of 16 lanes, then the rows' lane-0 values combined in a fixed order, so the
// result is the same value in every lane and in every call.
template <int CTRL>
__device__ __forceinline__ float dpp_self_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_self_f32<0xB1>(x));
  x = fmaxf(x, dpp_self_f32<0x4E>(x));
  x = fmaxf(x, dpp_self_f32<0x124>(x));
  x = fmaxf(x, dpp_self_f32<0x128>(x));
  return fmaxf(fmaxf(lane_f32(x, 0), lane_f32(x, 16)), fmaxf(lane_f32(x, 32), lane_f32(x, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_self_f32<0xB1>(x);
  x += dpp_self_f32<0x4E>(x);
  x += dpp_self_f32<0x124>(x);
  x += dpp_self_f32<0x128>(x);
  return (lane_f32(x, 0) + lane_f32(x, 16)) + (lane_f32(x, 32) + lane_f32(x, 48));
}

#define HYS_LDS __attribute__((address_space(3)))
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// V fragment for P.V from a row-major bf16 V tile in LDS (head_dim 128, 256-byte
// key rows, 16-byte chunk c of key k in slot c ^ 2 (k & 7)), with the gfx950
// transposed LDS read: in each group of 16 lanes, lane L receives element
// L & 3 of the 8-byte read of lane 4e + (L >> 2) as its element e.  Lane s of
// the group reads key r0 + (s >> 2), columns d0 + 4 (s & 3) .. +3, so lane L
// receives keys r0 .. r0 + 3 of column d0 + L: keys 32 kk + 4 quad + e
// (e < 4) and 32 kk + 16 + 4 quad + e - 4 (e >= 4) of column 16 dt + col.
__device__ __forceinline__ bf16x8_t tr_v_frag(const unsigned char* vs, int dt, int kk, int col, int quad) {
  const int d = 16 * dt + 4 * (col & 3);
  const int r0 = 32 * kk + 4 * quad + (col >> 2);
  auto rd = [&](int row) {
    const int off = row * 256 + (((d >> 3) ^ (2 * (row & 7))) << 4) + 8 * (col & 1);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((HYS_LDS i16x4_t*)(vs + off));
  };
  const i16x4_t lo = rd(r0), hi = rd(r0 + 16);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, both);
}

// 4 x 4 transpose inside each group of four lanes: lane i (= l & 3) holds
// v[0..3] on entry and, on exit, v[k] = the entry v[i] of the group's lane k.
// Two exchange stages (lane bit 0 with value bit 0, then lane bit 1 with
// value bit 1), each two DPP moves.
__device__ __forceinline__ void quad_transpose4(float (&v)[4]) {
  const bool b0 = threadIdx.x & 1, b1 = threadIdx.x & 2;
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const float recv = dpp_quad<0xB1>(b0 ? v[2 * hi] : v[2 * hi + 1]);
    if (b0)
      v[2 * hi] = recv;
    else
      v[2 * hi + 1] = recv;
  }
#pragma unroll
  for (int lo = 0; lo < 2; ++lo) {
    const float recv = dpp_quad<0x4E>(b1 ? v[lo] : v[2 + lo]);
    if (b1)
      v[lo] = recv;
    else
      v[2 + lo] = recv;
  }
}

}  // namespace hys
