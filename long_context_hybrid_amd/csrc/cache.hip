// KV-cache append for the decode loop and for chunked prefill
// (intelliparadigm article section 3.1: only the full layers update the KV
// cache; the sparse layers read the full layer's cache).  The new rows of keys
// and values are copied into the cache at positions [pos, pos + n_new); the
// full layer then runs on the cache with kv_len = pos + n_new.
#include "hys_common.h"
#include "hys_internal.h"

namespace hys {

namespace {

// One thread per 16-byte chunk of a new row; rows (b, t, h) of the contiguous
// [B, n_new, Hkv, D] inputs, cache strides in elements.
__global__ __launch_bounds__(256) void append_kv_kernel(const u32x4_t* k_new, const u32x4_t* v_new, int64_t n_chunks,
                                                        int cpr, int Hkv, int n_new, int esz, int64_t ks_b,
                                                        int64_t ks_t, int64_t ks_h, int pos, unsigned char* k_cache,
                                                        unsigned char* v_cache) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n_chunks) return;
  const int64_t row = x / cpr;
  const int c = (int)(x - row * cpr);
  const int h = (int)(row % Hkv);
  const int64_t bt = row / Hkv;
  const int t = (int)(bt % n_new);
  const int64_t b = bt / n_new;
  const int64_t off = (b * ks_b + (int64_t)(pos + t) * ks_t + (int64_t)h * ks_h) * esz + (int64_t)c * 16;
  *reinterpret_cast<u32x4_t*>(k_cache + off) = k_new[x];
  *reinterpret_cast<u32x4_t*>(v_cache + off) = v_new[x];
}

}  // namespace

hipError_t launch_append_kv(const Geom& g, const void* k_new, const void* v_new, int n_new, int pos, void* k_cache,
                            void* v_cache, hipStream_t st) {
  const int esz = g.dtype == 1 ? 2 : 4;
  const int cpr = g.D * esz / 16;
  const int64_t n_chunks = (int64_t)g.B * n_new * g.Hkv * cpr;
  if (n_chunks == 0) return hipSuccess;
  return launch("append_kv", append_kv_kernel, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, st,
                static_cast<const u32x4_t*>(k_new), static_cast<const u32x4_t*>(v_new), n_chunks, cpr, g.Hkv, n_new,
                esz, g.ks_b, g.ks_t, g.ks_h, pos, static_cast<unsigned char*>(k_cache),
                static_cast<unsigned char*>(v_cache));
}

}  // namespace hys
