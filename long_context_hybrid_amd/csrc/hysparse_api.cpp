// C ABI of libhysparse: argument validation, workspace carving and launch
// sequencing.  No allocation, no global mutable state besides the calling
// thread's last-error text.
#include "hysparse.h"

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "hys_internal.h"

namespace {

thread_local std::string g_err;

// kernel-level event trace of the calling thread (profiling hook)
thread_local hipEvent_t* t_events = nullptr;
thread_local int32_t t_capacity = 0;
thread_local int32_t t_count = 0;
thread_local std::vector<const char*> t_names;

hys_status fail(hys_status s, const std::string& msg) {
  g_err = msg;
  return s;
}
hys_status ok() {
  g_err.clear();
  return HYS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hys_status check_desc(const hys_attn_desc* d, hys::Geom* g) {
  if (!d) return fail(HYS_ERR_NULL_PTR, "desc is NULL");
  if (d->batch < 1 || d->q_len < 1 || d->kv_len < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1)
    return fail(HYS_ERR_BAD_SHAPE, "batch, q_len, kv_len, head counts and head_dim must be >= 1");
  if (d->q_len > d->kv_len) return fail(HYS_ERR_BAD_SHAPE, "q_len must not exceed kv_len");
  if (d->n_q_heads % d->n_kv_heads != 0) return fail(HYS_ERR_BAD_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G > 16) return fail(HYS_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(HYS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->dtype != HYS_F32 && d->dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "dtype must be HYS_F32 or HYS_BF16");
  if (!(d->scale == d->scale) || std::isinf(d->scale)) return fail(HYS_ERR_BAD_SHAPE, "scale is not finite");
  const int64_t esz = d->dtype == HYS_BF16 ? 2 : 4;
  for (int x = 0; x < 3; ++x) {
    if (d->q_stride[x] < 0 || d->kv_stride[x] < 0) return fail(HYS_ERR_BAD_SHAPE, "negative stride");
    if ((d->q_stride[x] * esz) % 16 != 0 || (d->kv_stride[x] * esz) % 16 != 0)
      return fail(HYS_ERR_ALIGN, "batch/token/head strides must be multiples of 16 bytes");
  }
  if (d->q_stride[2] < d->head_dim && d->n_q_heads > 1) return fail(HYS_ERR_BAD_SHAPE, "q head stride < head_dim");
  if (d->kv_stride[2] < d->head_dim && d->n_kv_heads > 1) return fail(HYS_ERR_BAD_SHAPE, "kv head stride < head_dim");
  if (d->kv_stride[1] < 1 && d->kv_len > 1) return fail(HYS_ERR_BAD_SHAPE, "kv token stride must be >= 1");
  if (d->q_stride[1] < 1 && d->q_len > 1) return fail(HYS_ERR_BAD_SHAPE, "q token stride must be >= 1");
  g->B = d->batch;
  g->Tq = d->q_len;
  g->Tkv = d->kv_len;
  g->Hq = d->n_q_heads;
  g->Hkv = d->n_kv_heads;
  g->G = G;
  g->D = d->head_dim;
  g->dtype = d->dtype;
  g->scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  g->qs_b = d->q_stride[0];
  g->qs_t = d->q_stride[1];
  g->qs_h = d->q_stride[2];
  g->ks_b = d->kv_stride[0];
  g->ks_t = d->kv_stride[1];
  g->ks_h = d->kv_stride[2];
  return HYS_OK;
}

hys_status check_tensor(const void* p, const char* name, uintptr_t align) {
  if (!p) return fail(HYS_ERR_NULL_PTR, std::string(name) + " is NULL");
  if (!aligned(p, align)) return fail(HYS_ERR_ALIGN, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return HYS_OK;
}

int n_blocks(const hys::Geom& g, int sb) { return (g.Tq + sb - 1) / sb; }

hys_status check_sb(int sb) {
  if (sb != 1 && sb != 64) return fail(HYS_ERR_UNSUPPORTED, "score_block must be 1 or 64");
  return HYS_OK;
}

bool sparse_by_rows(const hys::Geom& g, int sb) { return sb == 1 || g.Tq == 1; }

size_t full_ws(const hys::Geom& g, int sb) {
  return g.Tq == 1 ? hys::decode_full_ws_bytes(g) : hys::prefill_full_ws_bytes(g, sb);
}
size_t topk_ws(const hys::Geom& g, int sb, int k) {
  return hys::topk_ws_bytes((int64_t)g.B * g.Hkv * n_blocks(g, sb), g.Tkv, k);
}
size_t sparse_ws(const hys::Geom& g, int sb, int k, int w) {
  return sparse_by_rows(g, sb) ? hys::decode_sparse_ws_bytes(g, k, w) : hys::sparse_block_ws_bytes(g, k, w);
}
size_t scores_bytes(const hys::Geom& g, int sb) {
  return hys::align_up((size_t)g.B * g.Hkv * n_blocks(g, sb) * g.Tkv * sizeof(float));
}
size_t idx_bytes(const hys::Geom& g, int sb, int k) {
  return hys::align_up((size_t)g.B * g.Hkv * n_blocks(g, sb) * (size_t)k * sizeof(int32_t));
}

hys_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return HYS_OK;
  if (!ws) return fail(HYS_ERR_WORKSPACE, "workspace is NULL; " + std::to_string(need) + " bytes needed");
  if (!aligned(ws, 16)) return fail(HYS_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(HYS_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes; " + std::to_string(need) + " needed");
  return HYS_OK;
}

hys_status from_hip(hipError_t e) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNotSupported) return fail(HYS_ERR_UNSUPPORTED, "this path is not compiled into the library");
  return fail(HYS_ERR_HIP, std::string("HIP error: ") + hipGetErrorString(e));
}

hipError_t run_full(const hys::Geom& g, const void* q, const void* k, const void* v, int sb, void* out, float* lse,
                    float* scores, void* ws, hipStream_t st) {
  if (g.Tq == 1) return hys::launch_full_decode(g, q, k, v, out, lse, scores, ws, st);
  return hys::launch_full_prefill(g, q, k, v, sb, out, lse, scores, ws, st);
}

hipError_t run_sparse(const hys::Geom& g, const void* q, const void* k, const void* v, const int32_t* idx, int kt,
                      int sb, int w, const hys::GateRef& gate, void* out, void* ws, hipStream_t st,
                      const hys::WinRef& win = hys::WinRef{nullptr, nullptr, 0, 0, 0, 0}) {
  if (sparse_by_rows(g, sb)) return hys::launch_sparse_rows(g, q, k, v, idx, kt, sb, w, gate, win, out, ws, st);
  return hys::launch_sparse_block(g, q, k, v, idx, kt, sb, w, gate, win, out, ws, st);
}

// Scratch of hysparse_sparse_attn_noalloc: a fixed device array of this
// library, one copy per GPU, held until the process ends.  Host code must
// never pass the array's name to a kernel or a copy (on the host it is only a
// stand-in): it uses the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hys_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HYS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HYS_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HYS_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return HYS_OK;
}

}  // namespace

namespace hys {
bool trace_slot(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!t_events || 2 * t_count + 1 >= t_capacity) return false;
  *start = t_events[2 * t_count];
  *stop = t_events[2 * t_count + 1];
  t_names.push_back(name);
  ++t_count;
  return true;
}
}  // namespace hys

extern "C" {

hys_status hysparse_full_attn_scores(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                     int32_t score_block, void* out, float* lse, float* scores, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(desc, &g))) return s;
  if ((s = check_sb(score_block))) return s;
  if ((s = check_tensor(q, "q", 16)) || (s = check_tensor(k, "k", 16)) || (s = check_tensor(v, "v", 16)) ||
      (s = check_tensor(out, "out", 16)) || (s = check_tensor(scores, "scores", 16)))
    return s;
  if (lse && !aligned(lse, 4)) return fail(HYS_ERR_ALIGN, "lse is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, full_ws(g, score_block)))) return s;
  return from_hip(run_full(g, q, k, v, score_block, out, lse, scores, ws, stream));
}

hys_status hysparse_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                         const int32_t* valid_len, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (n_rows < 0 || row_len < 1 || k < 1) return fail(HYS_ERR_BAD_SHAPE, "need n_rows >= 0, row_len >= 1, k >= 1");
  if (row_stride < row_len) return fail(HYS_ERR_BAD_SHAPE, "row_stride < row_len");
  if (row_stride % 4 != 0 && n_rows > 1) return fail(HYS_ERR_ALIGN, "row_stride must be a multiple of 4");
  if (n_rows == 0) return ok();
  hys_status s;
  if ((s = check_tensor(scores, "scores", 16)) || (s = check_tensor(idx, "idx", 4))) return s;
  if (valid_len && !aligned(valid_len, 4)) return fail(HYS_ERR_ALIGN, "valid_len is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, hys::topk_ws_bytes(n_rows, row_len, k)))) return s;
  hys::ValidLen vl{valid_len, row_len, 0, 1, 1, 1, 1};
  return from_hip(hys::launch_topk(scores, n_rows, row_len, row_stride, vl, k, idx, ws, stream));
}

hys_status hysparse_sparse_attn(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                const int32_t* idx, int32_t k_top, int32_t score_block, int32_t window,
                                const float* gate_logits, void* out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return hysparse_sparse_attn_token_gate(desc, q, k, v, idx, k_top, score_block, window, gate_logits, 0, 0, out,
                                         ws, ws_bytes, stream);
}

hys_status hysparse_sparse_attn_token_gate(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                           const int32_t* idx, int32_t k_top, int32_t score_block, int32_t window,
                                           const float* gate_logits, int64_t gate_stride_b, int64_t gate_stride_t,
                                           void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return hysparse_sparse_attn_ex(desc, q, k, v, idx, k_top, score_block, window, gate_logits, gate_stride_b,
                                 gate_stride_t, nullptr, out, ws, ws_bytes, stream);
}

hys_status hysparse_sparse_attn_ex(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const int32_t* idx, int32_t k_top, int32_t score_block, int32_t window,
                                   const float* gate_logits, int64_t gate_stride_b, int64_t gate_stride_t,
                                   const hys_window_kv* own_window, void* out, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(desc, &g))) return s;
  if (gate_stride_b < 0 || gate_stride_t < 0) return fail(HYS_ERR_BAD_SHAPE, "gate strides must be >= 0");
  hys::WinRef win{nullptr, nullptr, 0, 0, 0, 0};
  if (own_window) {
    const hys_window_kv& w = *own_window;
    if ((s = check_tensor(w.k, "own_window.k", 16)) || (s = check_tensor(w.v, "own_window.v", 16))) return s;
    const int64_t esz = g.dtype == HYS_BF16 ? 2 : 4;
    for (int x = 0; x < 3; ++x) {
      if (w.stride[x] < 0) return fail(HYS_ERR_BAD_SHAPE, "negative own-window stride");
      if ((w.stride[x] * esz) % 16 != 0) return fail(HYS_ERR_ALIGN, "own-window strides must be multiples of 16 bytes");
    }
    if (w.ring < 0) return fail(HYS_ERR_BAD_SHAPE, "own_window.ring must be >= 0");
    if (w.ring > 0 && (int64_t)w.ring < (int64_t)window + g.Tq - 1)
      return fail(HYS_ERR_BAD_SHAPE, "own_window.ring must be >= window + q_len - 1");
    win = hys::WinRef{w.k, w.v, w.stride[0], w.stride[1], w.stride[2], w.ring};
  }
  if ((s = check_sb(score_block))) return s;
  if (k_top < 1) return fail(HYS_ERR_BAD_SHAPE, "k_top must be >= 1");
  if (window < 1) return fail(HYS_ERR_BAD_SHAPE, "window must be >= 1");
  if ((s = check_tensor(q, "q", 16)) || (s = check_tensor(k, "k", 16)) || (s = check_tensor(v, "v", 16)) ||
      (s = check_tensor(out, "out", 16)) || (s = check_tensor(idx, "idx", 4)) ||
      (s = check_tensor(gate_logits, "gate_logits", 4)))
    return s;
  if ((s = check_ws(ws, ws_bytes, sparse_ws(g, score_block, k_top, window)))) return s;
  const hys::GateRef gate{gate_logits, gate_stride_b, gate_stride_t};
  return from_hip(run_sparse(g, q, k, v, idx, k_top, score_block, window, gate, out, ws, stream, win));
}

hys_status hysparse_sparse_attn_noalloc(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                        const int32_t* idx, int32_t k_top, int32_t score_block, int32_t window,
                                        const float* gate_logits, void* out, hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(desc, &g))) return s;
  if ((s = check_sb(score_block))) return s;
  if (k_top < 1) return fail(HYS_ERR_BAD_SHAPE, "k_top must be >= 1");
  if (window < 1) return fail(HYS_ERR_BAD_SHAPE, "window must be >= 1");
  if ((s = check_tensor(q, "q", 16)) || (s = check_tensor(k, "k", 16)) || (s = check_tensor(v, "v", 16)) ||
      (s = check_tensor(out, "out", 16)) || (s = check_tensor(idx, "idx", 4)) ||
      (s = check_tensor(gate_logits, "gate_logits", 4)))
    return s;
  const size_t need = sparse_ws(g, score_block, k_top, window);
  if (need > kScratchBytes)
    return fail(HYS_ERR_WORKSPACE, "this call needs " + std::to_string(need) + " bytes of scratch; the library's "
                "fixed scratch holds " + std::to_string(kScratchBytes) + " (use hysparse_sparse_attn with a workspace)");
  void* ws = nullptr;
  if (need > 0 && (s = scratch_on_current_device(&ws))) return s;
  const hys::GateRef gate{gate_logits, 0, 0};
  return from_hip(run_sparse(g, q, k, v, idx, k_top, score_block, window, gate, out, ws, stream));
}

size_t hysparse_noalloc_scratch_bytes(void) { return kScratchBytes; }

hys_status hysparse_hybrid_block(const hys_attn_desc* desc, const void* q_full, const void* k, const void* v,
                                 int32_t n_sparse, const void* const* q_sparse, const float* gate_logits,
                                 int32_t k_top, int32_t score_block, int32_t window, void* out_full,
                                 void* const* out_sparse, float* lse, float* scores, int32_t* idx, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(desc, &g))) return s;
  if ((s = check_sb(score_block))) return s;
  if (k_top < 1) return fail(HYS_ERR_BAD_SHAPE, "k_top must be >= 1");
  if (window < 1) return fail(HYS_ERR_BAD_SHAPE, "window must be >= 1");
  if (n_sparse < 0) return fail(HYS_ERR_BAD_SHAPE, "n_sparse must be >= 0");
  if ((s = check_tensor(q_full, "q_full", 16)) || (s = check_tensor(k, "k", 16)) || (s = check_tensor(v, "v", 16)) ||
      (s = check_tensor(out_full, "out_full", 16)))
    return s;
  if (n_sparse > 0) {
    if (!q_sparse || !out_sparse) return fail(HYS_ERR_NULL_PTR, "q_sparse / out_sparse array is NULL");
    if ((s = check_tensor(gate_logits, "gate_logits", 4))) return s;
    for (int l = 0; l < n_sparse; ++l) {
      if ((s = check_tensor(q_sparse[l], "q_sparse[l]", 16)) || (s = check_tensor(out_sparse[l], "out_sparse[l]", 16)))
        return s;
    }
  }
  if (lse && !aligned(lse, 4)) return fail(HYS_ERR_ALIGN, "lse is not 4-byte aligned");
  if (scores && !aligned(scores, 16)) return fail(HYS_ERR_ALIGN, "scores is not 16-byte aligned");
  if (idx && !aligned(idx, 4)) return fail(HYS_ERR_ALIGN, "idx is not 4-byte aligned");
  const size_t s_b = scores ? 0 : scores_bytes(g, score_block);
  const size_t i_b = idx ? 0 : idx_bytes(g, score_block, k_top);
  size_t inner = full_ws(g, score_block);
  const size_t tk = topk_ws(g, score_block, k_top);
  const size_t sp = n_sparse > 0 ? sparse_ws(g, score_block, k_top, window) : 0;
  if (tk > inner) inner = tk;
  if (sp > inner) inner = sp;
  if ((s = check_ws(ws, ws_bytes, s_b + i_b + inner))) return s;
  unsigned char* c = static_cast<unsigned char*>(ws);
  if (!scores) {
    scores = reinterpret_cast<float*>(c);
    c += s_b;
  }
  if (!idx) {
    idx = reinterpret_cast<int32_t*>(c);
    c += i_b;
  }
  void* inner_ws = c;
  hipError_t e = run_full(g, q_full, k, v, score_block, out_full, lse, scores, inner_ws, stream);
  if (e != hipSuccess) return from_hip(e);
  const int NB = n_blocks(g, score_block);
  hys::ValidLen vl{nullptr, g.Tkv, 1, NB, score_block, g.Tq, g.Tkv};
  e = hys::launch_topk(scores, (int64_t)g.B * g.Hkv * NB, g.Tkv, g.Tkv, vl, k_top, idx, inner_ws, stream);
  if (e != hipSuccess) return from_hip(e);
  for (int l = 0; l < n_sparse; ++l) {
    const hys::GateRef gate{gate_logits + (size_t)l * g.Hq, 0, 0};
    e = run_sparse(g, q_sparse[l], k, v, idx, k_top, score_block, window, gate, out_sparse[l], inner_ws, stream);
    if (e != hipSuccess) return from_hip(e);
  }
  return ok();
}

size_t hysparse_workspace_bytes(int32_t op, const hys_attn_desc* desc, int32_t score_block, int32_t k_top,
                                int32_t window) {
  hys::Geom g;
  if (check_desc(desc, &g) != HYS_OK) return 0;
  if (score_block != 1 && score_block != 64) return 0;
  if (k_top < 1) k_top = 1;
  if (window < 1) window = 1;
  switch (op) {
    case HYS_OP_FULL:
      return full_ws(g, score_block);
    case HYS_OP_TOPK:
      return topk_ws(g, score_block, k_top);
    case HYS_OP_SPARSE:
      return sparse_ws(g, score_block, k_top, window);
    case HYS_OP_HYBRID: {
      size_t inner = full_ws(g, score_block);
      const size_t tk = topk_ws(g, score_block, k_top);
      const size_t sp = sparse_ws(g, score_block, k_top, window);
      if (tk > inner) inner = tk;
      if (sp > inner) inner = sp;
      return scores_bytes(g, score_block) + idx_bytes(g, score_block, k_top) + inner;
    }
    default:
      return 0;
  }
}

static hys_status check_hier(const hys_attn_desc* desc, int32_t block, int32_t n_keep, int32_t k_top, hys::Geom* g) {
  hys_status s;
  if ((s = check_desc(desc, g))) return s;
  if (g->Tq != 1) return fail(HYS_ERR_UNSUPPORTED, "hierarchical selection is implemented for decode (q_len 1)");
  if (block < 1 || n_keep < 1 || k_top < 1) return fail(HYS_ERR_BAD_SHAPE, "block, n_keep and k_top must be >= 1");
  if ((int64_t)n_keep * block > (int64_t)1 << 30) return fail(HYS_ERR_BAD_SHAPE, "n_keep * block too large");
  if ((g->Tkv + block - 1) / block > hys::hier_max_blocks())
    return fail(HYS_ERR_UNSUPPORTED, "more than " + std::to_string(hys::hier_max_blocks()) + " pooled blocks per row");
  return HYS_OK;
}

hys_status hysparse_hier_select(const hys_attn_desc* desc, const void* q, const void* k, const float* scores,
                                int32_t block, int32_t n_keep, int32_t k_top, float* block_scores, int32_t* blocks,
                                int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_hier(desc, block, n_keep, k_top, &g))) return s;
  if ((s = check_tensor(q, "q", 16)) || (s = check_tensor(k, "k", 16)) || (s = check_tensor(scores, "scores", 16)) ||
      (s = check_tensor(idx, "idx", 4)))
    return s;
  if (block_scores && !aligned(block_scores, 4)) return fail(HYS_ERR_ALIGN, "block_scores is not 4-byte aligned");
  if (blocks && !aligned(blocks, 4)) return fail(HYS_ERR_ALIGN, "blocks is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, hys::hier_ws_bytes(g, block, n_keep, k_top)))) return s;
  return from_hip(hys::launch_hier_select(g, q, k, nullptr, 0, scores, block, n_keep, k_top, block_scores, blocks, idx,
                                          ws, stream));
}

hys_status hysparse_hier_pool(const hys_attn_desc* desc, const void* k, int32_t block, int32_t m_begin, int32_t m_end,
                              float* kbar, int32_t kbar_blocks, hipStream_t stream) {
  if (!desc) return fail(HYS_ERR_NULL_PTR, "desc is NULL");
  // only the cache (kv) fields are used: validate them with a stand-in query
  hys_attn_desc d = *desc;
  d.q_len = 1;
  d.n_q_heads = d.n_kv_heads;
  for (int x = 0; x < 3; ++x) d.q_stride[x] = d.kv_stride[x];
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(&d, &g))) return s;
  if (block < 1) return fail(HYS_ERR_BAD_SHAPE, "block must be >= 1");
  const int64_t M = ((int64_t)g.Tkv + block - 1) / block;
  if (M > hys::hier_max_blocks())
    return fail(HYS_ERR_UNSUPPORTED, "more than " + std::to_string(hys::hier_max_blocks()) + " pooled blocks per row");
  if (kbar_blocks < M || kbar_blocks > hys::hier_max_blocks())
    return fail(HYS_ERR_BAD_SHAPE, "kbar_blocks must cover ceil(kv_len / block) blocks");
  if (m_begin < 0 || m_end < m_begin || m_end > M)
    return fail(HYS_ERR_BAD_SHAPE, "need 0 <= m_begin <= m_end <= ceil(kv_len / block)");
  if ((s = check_tensor(k, "k", 16)) || (s = check_tensor(kbar, "kbar", 16))) return s;
  return from_hip(hys::launch_hier_pool(g, k, block, m_begin, m_end, kbar, kbar_blocks, stream));
}

hys_status hysparse_hier_select_pooled(const hys_attn_desc* desc, const void* q, const float* kbar, int32_t kbar_blocks,
                                       const float* scores, int32_t block, int32_t n_keep, int32_t k_top,
                                       float* block_scores, int32_t* blocks, int32_t* idx, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  hys::Geom g;
  hys_status s;
  if ((s = check_hier(desc, block, n_keep, k_top, &g))) return s;
  if (kbar_blocks < (g.Tkv + block - 1) / block || kbar_blocks > hys::hier_max_blocks())
    return fail(HYS_ERR_BAD_SHAPE, "kbar_blocks must cover ceil(kv_len / block) blocks");
  if ((s = check_tensor(q, "q", 16)) || (s = check_tensor(kbar, "kbar", 16)) ||
      (s = check_tensor(scores, "scores", 16)) || (s = check_tensor(idx, "idx", 4)))
    return s;
  if (block_scores && !aligned(block_scores, 4)) return fail(HYS_ERR_ALIGN, "block_scores is not 4-byte aligned");
  if (blocks && !aligned(blocks, 4)) return fail(HYS_ERR_ALIGN, "blocks is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, hys::hier_ws_bytes(g, block, n_keep, k_top)))) return s;
  return from_hip(hys::launch_hier_select(g, q, nullptr, kbar, kbar_blocks, scores, block, n_keep, k_top, block_scores,
                                          blocks, idx, ws, stream));
}

hys_status hysparse_append_kv(const hys_attn_desc* desc, const void* k_new, const void* v_new, int32_t n_new,
                              int32_t pos, void* k_cache, void* v_cache, hipStream_t stream) {
  if (!desc) return fail(HYS_ERR_NULL_PTR, "desc is NULL");
  // only the cache (kv) fields are used: validate them with a stand-in query
  hys_attn_desc d = *desc;
  d.q_len = 1;
  d.n_q_heads = d.n_kv_heads;
  for (int x = 0; x < 3; ++x) d.q_stride[x] = d.kv_stride[x];
  hys::Geom g;
  hys_status s;
  if ((s = check_desc(&d, &g))) return s;
  if (n_new < 1 || pos < 0 || (int64_t)pos + n_new > desc->kv_len)
    return fail(HYS_ERR_BAD_SHAPE, "need n_new >= 1, pos >= 0 and pos + n_new <= kv_len (the cache capacity)");
  if ((s = check_tensor(k_new, "k_new", 16)) || (s = check_tensor(v_new, "v_new", 16)) ||
      (s = check_tensor(k_cache, "k_cache", 16)) || (s = check_tensor(v_cache, "v_cache", 16)))
    return s;
  return from_hip(hys::launch_append_kv(g, k_new, v_new, n_new, pos, k_cache, v_cache, stream));
}

size_t hysparse_hier_workspace_bytes(const hys_attn_desc* desc, int32_t block, int32_t n_keep, int32_t k_top) {
  hys::Geom g;
  if (check_hier(desc, block, n_keep, k_top, &g) != HYS_OK) return 0;
  return hys::hier_ws_bytes(g, block, n_keep, k_top);
}

size_t hysparse_topk_workspace_bytes(int64_t n_rows, int32_t row_len, int32_t k) {
  if (n_rows < 0 || row_len < 1 || k < 1) return 0;
  return hys::topk_ws_bytes(n_rows, row_len, k);
}

hys_status hysparse_check_indices(const int32_t* idx, int64_t n_rows, int32_t k, int32_t row_len,
                                  const int32_t* valid_len, int32_t* status, hipStream_t stream) {
  static_assert(hys::kIdxDuplicate == HYS_IDX_DUPLICATE && hys::kIdxOutOfRange == HYS_IDX_OUT_OF_RANGE &&
                    hys::kIdxOrder == HYS_IDX_ORDER,
                "status bits");
  if (n_rows < 0 || n_rows > INT32_MAX || k < 1) return fail(HYS_ERR_BAD_SHAPE, "need 0 <= n_rows < 2^31 and k >= 1");
  if (row_len < 1 || row_len > hys::check_indices_max_row_len())
    return fail(HYS_ERR_UNSUPPORTED, "row_len must be in [1, " + std::to_string(hys::check_indices_max_row_len()) + "]");
  if (n_rows == 0) return ok();
  hys_status s;
  if ((s = check_tensor(idx, "idx", 4)) || (s = check_tensor(status, "status", 4))) return s;
  if (valid_len && !aligned(valid_len, 4)) return fail(HYS_ERR_ALIGN, "valid_len is not 4-byte aligned");
  hys::ValidLen vl{valid_len, row_len, 0, 1, 1, 1, 1};
  return from_hip(hys::launch_check_indices(idx, n_rows, k, row_len, vl, status, stream));
}

size_t hysparse_ceiling_workspace_bytes(int64_t n_bytes, int64_t n_rows) {
  if (n_bytes < 0 || n_rows < 0) return 0;
  const int64_t a = hys::ceiling_stream_blocks(n_bytes), b = hys::ceiling_gather_blocks(n_rows);
  return hys::align_up((size_t)(a > b ? a : b) * sizeof(uint32_t));
}

hys_status hysparse_ceiling_stream_read(const void* p, int64_t n_bytes, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (n_bytes < 0 || n_bytes % 16 != 0) return fail(HYS_ERR_BAD_SHAPE, "n_bytes must be a non-negative multiple of 16");
  if (n_bytes == 0) return ok();
  hys_status s;
  if ((s = check_tensor(p, "p", 16))) return s;
  if ((s = check_ws(ws, ws_bytes, hysparse_ceiling_workspace_bytes(n_bytes, 0)))) return s;
  return from_hip(hys::launch_ceiling_stream(p, n_bytes, static_cast<uint32_t*>(ws), stream));
}

hys_status hysparse_ceiling_gather(const void* k, const void* v, int64_t row_stride_bytes, int64_t n_buffer_rows,
                                   const int32_t* rows, int64_t n_rows, int32_t row_bytes, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (n_rows < 0 || n_buffer_rows < 0) return fail(HYS_ERR_BAD_SHAPE, "n_rows and n_buffer_rows must be >= 0");
  if (row_bytes < 16 || row_bytes > 256 || row_bytes % 16 != 0)
    return fail(HYS_ERR_UNSUPPORTED, "row_bytes must be a multiple of 16 in [16, 256]");
  if (row_stride_bytes < row_bytes || row_stride_bytes % 16 != 0)
    return fail(HYS_ERR_ALIGN, "row_stride_bytes must be >= row_bytes and a multiple of 16");
  if (n_rows == 0) return ok();
  hys_status s;
  if ((s = check_tensor(k, "k", 16)) || (s = check_tensor(v, "v", 16)) || (s = check_tensor(rows, "rows", 4))) return s;
  if ((s = check_ws(ws, ws_bytes, hysparse_ceiling_workspace_bytes(0, n_rows)))) return s;
  return from_hip(hys::launch_ceiling_gather(k, v, row_stride_bytes, n_buffer_rows, rows, n_rows, row_bytes,
                                             static_cast<uint32_t*>(ws), stream));
}

const char* hysparse_status_string(hys_status status) {
  switch (status) {
    case HYS_OK: return "ok";
    case HYS_ERR_NULL_PTR: return "null pointer";
    case HYS_ERR_BAD_SHAPE: return "bad shape";
    case HYS_ERR_UNSUPPORTED: return "unsupported";
    case HYS_ERR_ALIGN: return "misaligned pointer or stride";
    case HYS_ERR_WORKSPACE: return "workspace too small";
    case HYS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* hysparse_last_error(void) { return g_err.c_str(); }

int32_t hysparse_version(void) { return 100; }

void hysparse_trace_begin(hipEvent_t* events, int32_t capacity) {
  t_events = events;
  t_capacity = events ? capacity : 0;
  t_count = 0;
  t_names.clear();
}

int32_t hysparse_trace_end(void) {
  t_events = nullptr;
  t_capacity = 0;
  return t_count;
}

const char* hysparse_trace_name(int32_t i) {
  return (i >= 0 && i < (int32_t)t_names.size()) ? t_names[i] : "";
}

}  // extern "C"
