// Host-side interface between the C ABI (hysparse_api.cpp) and the kernel
// translation units.  Plain structs passed by value to the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

namespace hys {

// Problem geometry after validation (strides in elements).
struct Geom {
  int B, Tq, Tkv, Hq, Hkv, G, D;
  int dtype;  // 0 f32, 1 bf16
  float scale;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
};

// Row -> candidate count for top-K rows.  Either an explicit device array
// (clamped to row_len), or the causal rule of the hybrid block
// (row = ((b * Hkv + g) * NB + n): candidates = Tkv - Tq + min((n+1)*Sb, Tq)),
// or row_len everywhere.
struct ValidLen {
  const int32_t* ptr;
  int32_t row_len;
  int32_t causal;  // 1: use (nb, sb, tq, tkv)
  int32_t nb, sb, tq, tkv;
};

__host__ __device__ inline int32_t valid_len_of(const ValidLen& v, int64_t row) {
  int32_t n;
  if (v.ptr) {
    n = v.ptr[row];
    n = n < 0 ? 0 : (n > v.row_len ? v.row_len : n);
  } else if (v.causal) {
    int32_t blk = (int32_t)(row % v.nb);
    int32_t i1 = (blk + 1) * v.sb;
    if (i1 > v.tq) i1 = v.tq;
    n = v.tkv - v.tq + i1;
    if (n > v.row_len) n = v.row_len;
  } else {
    n = v.row_len;
  }
  return n;
}

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Kernel-level event tracing (see hysparse_trace_begin).  Every kernel goes
// through launch(): while a trace is active on the calling thread and has room,
// trace_slot hands out the next (start, stop) event pair and records the
// kernel's name, and the kernel is launched with hipExtLaunchKernelGGL, which
// stamps the two events with the dispatch's own begin and end times (no
// marker packets between kernels); otherwise it is an ordinary launch.
bool trace_slot(const char* name, hipEvent_t* start, hipEvent_t* stop);

template <typename... KArgs, typename... Args>
hipError_t launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t smem, hipStream_t st,
                  Args&&... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (trace_slot(name, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, smem, st, e0, e1, 0, std::forward<Args>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, st, std::forward<Args>(args)...);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode path
// Split-K attention of one query row per (batch, KV group) unit against a key
// list (the whole cache for the full layer; idx + window for a sparse layer).
struct DecodePlan {
  int units;     // full: B*Hkv ; sparse: B*Hkv*Tq
  int chunk;     // keys per split (full layer; sparse global branch)
  int wchunk;    // sparse: window keys per split
  int nsplit;    // splits per unit
  int nsg;       // sparse: global splits (the remaining ones cover the window)
};
DecodePlan plan_full_decode(const Geom& g);
DecodePlan plan_sparse_rows(const Geom& g, int k_top, int window);

struct DecodeWs {
  float* part_o;   // [units, nsplit, G, D]
  float* part_ml;  // [units, nsplit, G, 2]
  void* probs;     // full only: probabilities against each step's running maximum,
                   // [B, Hkv, keys, slots] (key-major), 3-byte rounded fp32 for bf16 inputs, fp32 otherwise
  float* pmax;     // full only: that maximum (base 2), [B, Hkv, keys / 32, slots]
};
size_t decode_full_ws_bytes(const Geom& g);
size_t decode_sparse_ws_bytes(const Geom& g, int k_top, int window);
DecodeWs carve_decode_ws(const Geom& g, const DecodePlan& p, void* ws, bool full);

hipError_t launch_full_decode(const Geom& g, const void* q, const void* k, const void* v, void* out,
                              float* lse, float* scores, void* ws, hipStream_t st);
// Gate logits of the sparse layer: the logit of (batch b, query i, query head
// h) is p[b * sb + i * st + h]; sb = st = 0 is one logit per head.
struct GateRef {
  const float* p;
  int64_t sb, st;
};

// Keys/values of the sparse layer's window branch: the shared cache (k ==
// nullptr) or the layer's own window K/V, position j in row (ring > 0 ? j %
// ring : j), strides in elements.
struct WinRef {
  const void* k;
  const void* v;
  int64_t sb, st, sh;
  int ring;
};

hipError_t launch_sparse_rows(const Geom& g, const void* q, const void* k, const void* v,
                              const int32_t* idx, int k_top, int score_block, int window,
                              const GateRef& gate, const WinRef& win, void* out, void* ws,
                              hipStream_t st);

// --------------------------------------------------------------- prefill path
size_t prefill_full_ws_bytes(const Geom& g, int score_block);
hipError_t launch_full_prefill(const Geom& g, const void* q, const void* k, const void* v,
                               int score_block, void* out, float* lse, float* scores, void* ws,
                               hipStream_t st);
size_t sparse_block_ws_bytes(const Geom& g, int k_top, int window);
hipError_t launch_sparse_block(const Geom& g, const void* q, const void* k, const void* v,
                               const int32_t* idx, int k_top, int score_block, int window,
                               const GateRef& gate, const WinRef& win, void* out, void* ws,
                              hipStream_t st);

// ---------------------------------------------------------------------- top-K
size_t topk_ws_bytes(int64_t n_rows, int32_t row_len, int32_t k);
hipError_t launch_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                       const ValidLen& vl, int32_t k, int32_t* idx, void* ws, hipStream_t st);

// ------------------------------------------------------ hierarchical select
int hier_max_blocks();
size_t hier_ws_bytes(const Geom& g, int block, int n_keep, int k_top);

// KV-cache append (cache.hip)
hipError_t launch_append_kv(const Geom& g, const void* k_new, const void* v_new, int n_new, int pos, void* k_cache,
                            void* v_cache, hipStream_t st);
// kbar_in: pooled keys [B, kbar_blocks, Hkv, D] fp32 from hysparse_hier_pool,
// or nullptr (all blocks pooled from k into the workspace first)
hipError_t launch_hier_select(const Geom& g, const void* q, const void* k, const float* kbar_in, int64_t kbar_blocks,
                              const float* scores, int block, int n_keep, int k_top, float* bscore_out,
                              int32_t* blk_out, int32_t* idx, void* ws, hipStream_t st);
// pooled keys of blocks [m_begin, m_end) of k into kbar [B, kbar_blocks, Hkv, D] fp32
hipError_t launch_hier_pool(const Geom& g, const void* k, int block, int m_begin, int m_end, float* kbar,
                            int64_t kbar_blocks, hipStream_t st);

// Index-set check (check.hip): status bits of one row.
constexpr uint32_t kIdxDuplicate = 1, kIdxOutOfRange = 2, kIdxOrder = 4;
int check_indices_max_row_len();
hipError_t launch_check_indices(const int32_t* idx, int64_t n_rows, int k, int row_len, const ValidLen& vl,
                                int32_t* status, hipStream_t st);

// Bandwidth ceilings of one launch (ceiling.hip): sink holds one word per
// workgroup.
int64_t ceiling_stream_blocks(int64_t n_bytes);
int64_t ceiling_gather_blocks(int64_t n_rows);
hipError_t launch_ceiling_stream(const void* p, int64_t n_bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_ceiling_gather(const void* k, const void* v, int64_t row_stride_bytes, int64_t n_buf_rows,
                                 const int32_t* rows, int64_t n_rows, int row_bytes, uint32_t* sink, hipStream_t st);

}  // namespace hys
