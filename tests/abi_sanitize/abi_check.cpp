// Host-side check of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_abi_sanitized.py with the
// library's host code compiled with both sanitizers and no device code).
// Every call here is rejected by the host-side validation before any HIP
// call, or is a pure size query; pointers are stand-ins that are never
// dereferenced.  Exits non-zero on the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "hysparse.h"

namespace {

int g_fail = 0;
void* const P = reinterpret_cast<void*>(0x10000);    // 16-byte aligned stand-in
void* const ODD = reinterpret_cast<void*>(0x10004);  // misaligned stand-in

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, hysparse_last_error());
    ++g_fail;
  }
}

hys_attn_desc desc(int B, int Tq, int Tkv, int Hq, int Hkv, int D, int dtype = HYS_BF16) {
  hys_attn_desc d{};
  d.batch = B;
  d.q_len = Tq;
  d.kv_len = Tkv;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.dtype = dtype;
  d.scale = 0.f;
  d.q_stride[0] = (int64_t)Tq * Hq * D;
  d.q_stride[1] = (int64_t)Hq * D;
  d.q_stride[2] = D;
  d.kv_stride[0] = (int64_t)Tkv * Hkv * D;
  d.kv_stride[1] = (int64_t)Hkv * D;
  d.kv_stride[2] = D;
  return d;
}

}  // namespace

int main() {
  // descriptor validation through every entry point that takes one
  hys_attn_desc d = desc(2, 1, 256, 8, 2, 128);
  expect(hysparse_full_attn_scores(nullptr, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 1, "desc null");
  hys_attn_desc bad = d;
  bad.q_len = 300;
  expect(hysparse_full_attn_scores(&bad, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 2, "q_len > kv_len");
  bad = d;
  bad.n_q_heads = 7;
  expect(hysparse_sparse_attn(&bad, P, P, P, (int32_t*)P, 8, 1, 4, (float*)P, P, P, 1 << 30, nullptr), 2, "Hq % Hkv");
  bad = d;
  bad.head_dim = 96;
  expect(hysparse_full_attn_scores(&bad, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 3, "head_dim 96");
  bad = d;
  bad.n_q_heads = 64;
  expect(hysparse_full_attn_scores(&bad, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 3, "G > 16");
  bad = d;
  bad.kv_stride[1] = 130;
  expect(hysparse_full_attn_scores(&bad, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 4, "stride align");
  bad = d;
  bad.scale = __builtin_nanf("");
  expect(hysparse_full_attn_scores(&bad, P, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 2, "NaN scale");
  expect(hysparse_full_attn_scores(&d, nullptr, P, P, 1, P, nullptr, (float*)P, P, 1 << 30, nullptr), 1, "q null");
  expect(hysparse_full_attn_scores(&d, P, P, P, 1, ODD, nullptr, (float*)P, P, 1 << 30, nullptr), 4, "out align");
  expect(hysparse_full_attn_scores(&d, P, P, P, 32, P, nullptr, (float*)P, P, 1 << 30, nullptr), 3, "score block 32");
  expect(hysparse_full_attn_scores(&d, P, P, P, 1, P, nullptr, (float*)P, nullptr, 0, nullptr), 5, "no workspace");
  // top-K
  expect(hysparse_topk((float*)P, 4, 100, 100, nullptr, 0, (int32_t*)P, P, 1 << 30, nullptr), 2, "topk k 0");
  expect(hysparse_topk((float*)P, 4, 100, 50, nullptr, 8, (int32_t*)P, P, 1 << 30, nullptr), 2, "topk stride");
  expect(hysparse_topk((float*)P, 4, 100, 102, nullptr, 8, (int32_t*)P, P, 1 << 30, nullptr), 4, "topk stride % 4");
  expect(hysparse_topk((float*)P, 0, 100, 100, nullptr, 8, (int32_t*)P, nullptr, 0, nullptr), 0, "topk empty");
  expect(hysparse_topk((float*)P, 16, 131072, 131072, nullptr, 2048, (int32_t*)P, nullptr, 0, nullptr), 5,
         "topk parts need workspace");
  // sparse layer variants
  expect(hysparse_sparse_attn(&d, P, P, P, (int32_t*)P, 0, 1, 4, (float*)P, P, P, 1 << 30, nullptr), 2, "k_top 0");
  expect(hysparse_sparse_attn(&d, P, P, P, (int32_t*)P, 8, 1, 0, (float*)P, P, P, 1 << 30, nullptr), 2, "window 0");
  expect(hysparse_sparse_attn_token_gate(&d, P, P, P, (int32_t*)P, 8, 1, 4, (float*)P, -1, 0, P, P, 1 << 30,
                                         nullptr), 2, "negative gate stride");
  hys_window_kv w{};
  w.k = P;
  w.v = ODD;
  w.stride[0] = w.stride[1] = w.stride[2] = 128;
  expect(hysparse_sparse_attn_ex(&d, P, P, P, (int32_t*)P, 8, 1, 4, (float*)P, 0, 0, &w, P, P, 1 << 30, nullptr), 4,
         "own window align");
  w.v = P;
  w.ring = 2;
  expect(hysparse_sparse_attn_ex(&d, P, P, P, (int32_t*)P, 8, 1, 4, (float*)P, 0, 0, &w, P, P, 1 << 30, nullptr), 2,
         "own window ring");
  expect(hysparse_sparse_attn_noalloc(&d, nullptr, P, P, (int32_t*)P, 8, 1, 4, (float*)P, P, nullptr), 1,
         "noalloc q null");
  hys_attn_desc big = desc(1, 8192, 8192, 32, 8, 128);
  expect(hysparse_sparse_attn_noalloc(&big, P, P, P, (int32_t*)P, 2048, 1, 128, (float*)P, P, nullptr), 5,
         "noalloc oversized");
  // hybrid block
  expect(hysparse_hybrid_block(&d, P, P, P, -1, nullptr, nullptr, 8, 1, 4, P, nullptr, nullptr, nullptr, nullptr, P,
                               1 << 30, nullptr), 2, "n_sparse < 0");
  expect(hysparse_hybrid_block(&d, P, P, P, 2, nullptr, (float*)P, 8, 1, 4, P, nullptr, nullptr, nullptr, nullptr, P,
                               1 << 30, nullptr), 1, "q_sparse null");
  // hierarchical selection, pooling, append
  expect(hysparse_hier_select(&big, P, P, (float*)P, 128, 64, 2048, nullptr, nullptr, (int32_t*)P, P, 1 << 30,
                              nullptr), 3, "hier prefill");
  expect(hysparse_hier_select(&d, P, P, (float*)P, 0, 64, 2048, nullptr, nullptr, (int32_t*)P, P, 1 << 30, nullptr),
         2, "hier block 0");
  expect(hysparse_hier_pool(&d, P, 128, 0, 5, (float*)P, 2, nullptr), 2, "pool range");
  expect(hysparse_hier_select_pooled(&d, P, (float*)P, 1, (float*)P, 128, 4, 16, nullptr, nullptr, (int32_t*)P, P,
                                     1 << 30, nullptr), 2, "pooled select, too few pooled blocks");
  expect(hysparse_append_kv(&d, P, P, 1, 256, P, P, nullptr), 2, "append past capacity");
  expect(hysparse_append_kv(&d, P, P, 0, 0, P, P, nullptr), 2, "append nothing");
  // index-set check
  expect(hysparse_check_indices((int32_t*)P, 4, 0, 100, nullptr, (int32_t*)P, nullptr), 2, "check k 0");
  expect(hysparse_check_indices((int32_t*)P, 4, 8, (1 << 19) + 1, nullptr, (int32_t*)P, nullptr), 3,
         "check row_len");
  expect(hysparse_check_indices(nullptr, 4, 8, 100, nullptr, (int32_t*)P, nullptr), 1, "check idx null");
  // measurement helpers
  expect(hysparse_ceiling_stream_read(P, 100, P, 1 << 20, nullptr), 2, "stream bytes % 16");
  expect(hysparse_ceiling_gather(P, P, 256, 100, (int32_t*)P, 10, 512, P, 1 << 20, nullptr), 3, "gather row bytes");
  // size queries over a spread of shapes (the planning arithmetic runs here)
  const int shapes[][6] = {{4, 1, 131072, 64, 4, 128},  {16, 1, 8192, 32, 8, 128}, {1, 32768, 32768, 32, 8, 128},
                           {1, 131072, 131072, 64, 4, 128}, {1, 256, 256, 4, 1, 64}, {64, 1, 1 << 20, 16, 1, 128},
                           {1, 1, 1, 1, 1, 64},          {3, 77, 1000, 12, 3, 64}};
  size_t acc = 0;
  for (const auto& s : shapes) {
    for (int dt = 0; dt < 2; ++dt) {
      hys_attn_desc e = desc(s[0], s[1], s[2], s[3], s[4], s[5], dt);
      for (int sb : {1, 64})
        for (int op = 0; op < 4; ++op) acc += hysparse_workspace_bytes(op, &e, sb, 2048, 128);
      if (s[1] == 1) acc += hysparse_hier_workspace_bytes(&e, 128, 64, 2048);
    }
    acc += hysparse_topk_workspace_bytes((int64_t)s[0] * s[4], s[2], 2048);
  }
  acc += hysparse_ceiling_workspace_bytes(18 << 20, 34816);
  if (acc == 0) {
    std::fprintf(stderr, "FAIL size queries all zero\n");
    ++g_fail;
  }
  for (int st = -1; st <= 7; ++st)
    if (!hysparse_status_string(st)) ++g_fail;
  std::printf("%s: %d unexpected results, size total %zu, version %d\n", g_fail ? "FAIL" : "OK", g_fail, acc,
              hysparse_version());
  return g_fail ? 1 : 0;
}
