// Host-only exercise of the C ABI's validation and planning code, built together with a
// copy of api.cpp compiled with AddressSanitizer and UndefinedBehaviorSanitizer for the host
// (tests/test_host_sanitizers.py). Every call here is refused on the host or is pure host
// arithmetic, so nothing reaches a GPU; the sanitizers watch the argument checks, the
// workspace and packed-size arithmetic, the k-split plan scan and the descriptor checks.
// Exit status 0 when every return code is the documented one.
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tel.h"

static int g_fail = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static tel_encoder_desc desc(int H, int heads, int F, int dtype, int int8 = 0, int sparse = 0,
                             int dyn = 0) {
  tel_encoder_desc d;
  std::memset(&d, 0, sizeof(d));
  d.hidden = H;
  d.heads = heads;
  d.ffn = F;
  d.dtype = dtype;
  d.int8_gemm = int8;
  d.ln_eps = 1e-5f;
  d.sparse_2of4 = sparse;
  d.dynamic_scales = dyn;
  return d;
}

int main() {
  // status strings for every code and one past the end
  for (int s = -1; s <= 6; ++s) EXPECT(tel_status_str(s) != nullptr);
  EXPECT(tel_version() != nullptr);

  // sizes: monotone in tokens, zero for unsupported descriptors
  const int dts[] = {TEL_F32, TEL_F16, TEL_BF16};
  for (int dt : dts) {
    for (int int8 = 0; int8 <= 2; ++int8) {
      if (int8 && dt != TEL_F16) continue;
      for (int H : {64, 96, 768, 1024}) {
        tel_encoder_desc d = desc(H, H / 32 ? H / 32 : 1, 4 * H, dt, int8);
        const size_t p = tel_encoder_packed_size(&d);
        EXPECT(p > 0);
        size_t prev = 0;
        for (int T : {0, 1, 31, 32, 33, 127, 128, 129, 640, 2557, 4096}) {
          const size_t w = tel_encoder_workspace_size(&d, T);
          EXPECT(w >= prev);
          prev = w;
        }
        EXPECT(tel_encoder_forward_workspace_size(&d, 32, 128) >= tel_encoder_workspace_size(&d, 32 * 128));
      }
    }
  }
  tel_encoder_desc bad = desc(100, 3, 400, TEL_F16);   // H % heads != 0
  EXPECT(tel_encoder_packed_size(&bad) == 0);
  EXPECT(tel_encoder_workspace_size(&bad, 128) == 0);
  EXPECT(tel_encoder_packed_size(nullptr) == 0);

  // the k-split plan over a grid of shapes and types
  for (int dt : {TEL_F32, TEL_F16, TEL_BF16, TEL_I8})
    for (int M : {1, 17, 64, 65, 127, 128, 129, 640, 2557, 14336})
      for (int N : {64, 768, 1024, 3072})
        for (int K : {64, 72, 768, 1024, 3072, 4096}) {
          int cfg = -9, sp = -9, pb = -9;
          EXPECT(tel_gemm_partial_plan(dt, M, N, K, &cfg, &sp, &pb) == TEL_OK);
          EXPECT(sp >= 1 && sp <= 8 && (pb == 2 || pb == 4));
        }
  int cfg, sp, pb;
  EXPECT(tel_gemm_partial_plan(TEL_F16, 128, 1024, 1024, nullptr, &sp, &pb) == TEL_EINVAL);
  EXPECT(tel_gemm_partial_plan(TEL_F16, -1, 1024, 1024, &cfg, &sp, &pb) == TEL_EINVAL);

  // entry points refuse bad arguments before any launch
  alignas(256) static char buf[4096], xb[4096], yb[4096];
  void* p = buf;
  void* odd = buf + 4;
  void* xp = xb;
  void* yp = yb;
  tel_encoder_desc d = desc(768, 12, 3072, TEL_F16);
  int32_t* ip = reinterpret_cast<int32_t*>(buf);
  EXPECT(tel_build_offsets(nullptr, 4, 8, ip, ip, nullptr) == TEL_EINVAL);
  EXPECT(tel_build_offsets(ip, -1, 8, ip, ip, nullptr) == TEL_EINVAL);
  EXPECT(tel_remove_padding(p, nullptr, ip, 4, 8, TEL_F16, nullptr) == TEL_EINVAL);
  EXPECT(tel_remove_padding(odd, p, ip, 4, 8, TEL_F16, nullptr) == TEL_EINVAL);
  EXPECT(tel_rebuild_padding(p, p, ip, 2, 0, 8, TEL_F16, nullptr) == TEL_EINVAL);
  EXPECT(tel_encoder_prepare(&bad, nullptr, p, 16, nullptr) != TEL_OK);
  EXPECT(tel_encoder_prepare(&d, nullptr, p, 16, nullptr) != TEL_OK);
  EXPECT(tel_encoder_layer_forward(&d, p, xp, yp, ip, 1, 10, 10, p, 16, nullptr) == TEL_EWORKSPACE);
  EXPECT(tel_encoder_layer_forward(&d, p, xp, xp, ip, 1, 10, 10, p, 1 << 30, nullptr) == TEL_EINVAL);
  EXPECT(tel_encoder_layer_forward(&d, nullptr, p, p, ip, 1, 10, 10, p, 1 << 30, nullptr) == TEL_EINVAL);
  EXPECT(tel_encoder_layer_forward(&d, p, odd, p, ip, 1, 10, 10, p, 1 << 30, nullptr) == TEL_EINVAL);
  EXPECT(tel_encoder_layer_forward(&bad, p, p, p, ip, 1, 10, 10, p, 1 << 30, nullptr) != TEL_OK);
  EXPECT(tel_gemm(TEL_EPI_BIAS, TEL_F16, p, p, nullptr, nullptr, p, 16, 16, 16, 1, nullptr) == TEL_EINVAL);
  EXPECT(tel_gemm(9, TEL_F16, p, p, (float*)p, nullptr, p, 16, 16, 16, 1, nullptr) == TEL_EINVAL);
  EXPECT(tel_gemm(TEL_EPI_BIAS, TEL_F16, p, p, (float*)p, nullptr, p, 16, 16, 12, 1, nullptr) == TEL_EUNSUPPORTED);
  EXPECT(tel_gemm(TEL_EPI_QKV_SPLIT, TEL_F16, p, p, (float*)p, nullptr, p, 16, 48, 16, 5, nullptr) == TEL_EUNSUPPORTED);
  EXPECT(tel_gemm_ex(TEL_EPI_BIAS, TEL_F16, 99, p, p, (float*)p, nullptr, p, 16, 16, 16, 1, nullptr) == TEL_EINVAL);
  EXPECT(tel_gemm_partial(TEL_F16, 0, 3, p, p, p, 4, 16, 16, 64, nullptr) == TEL_EUNSUPPORTED);
  EXPECT(tel_gemm_partial(TEL_BF16, 0, 1, p, p, p, 2, 16, 16, 64, nullptr) == TEL_EUNSUPPORTED);
  EXPECT(tel_attention_varlen(p, p, ip, 1, 8, 8, 2, 48, TEL_F16, nullptr) == TEL_EUNSUPPORTED);
  EXPECT(tel_attention_varlen(nullptr, p, ip, 1, 8, 8, 2, 64, TEL_F16, nullptr) == TEL_EINVAL);
  EXPECT(tel_layernorm(p, p, (float*)p, (float*)p, 4, 12, 1e-5f, TEL_F16, nullptr) != TEL_OK);
  EXPECT(tel_quantize_i8(odd, (int8_t*)p, 64, 1.f, TEL_F16, nullptr) == TEL_EINVAL);

  // the library's switches: query, set, restore (pure host state)
  const int pf = tel_weight_prefetch(-1);
  EXPECT(pf == 0 || pf == 1);
  EXPECT(tel_weight_prefetch(0) == pf && tel_weight_prefetch(-1) == 0);
  EXPECT(tel_weight_prefetch(1) == 0 && tel_weight_prefetch(-1) == 1);
  tel_weight_prefetch(pf);
  const int gr = tel_graph_cache(-1);
  EXPECT(gr == 0 || gr == 1);
  EXPECT(tel_graph_cache(gr) == gr);

  // the allocation-free entry point refuses what its scratch array cannot hold
  EXPECT(tel_encoder_layer_forward_noalloc(&d, p, xp, yp, ip, 1, 1 << 20, 128, nullptr) ==
         TEL_EWORKSPACE);

  // Swin descriptors
  tel_swin_desc s;
  std::memset(&s, 0, sizeof(s));
  s.batch = 1; s.height = 56; s.width = 56; s.channels = 96; s.heads = 3; s.window = 7;
  s.shift = 3; s.mlp_hidden = 384; s.dtype = TEL_F16; s.ln_eps = 1e-5f;
  EXPECT(tel_swin_packed_size(&s) > 0 && tel_swin_workspace_size(&s) > 0);
  s.height = 50;   // not a multiple of the window
  EXPECT(tel_swin_packed_size(&s) == 0);
  EXPECT(tel_window_attention_forward(&s, p, p, p, 0, p, 1 << 20, nullptr) == TEL_EINVAL);

  if (g_fail) std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
  else std::printf("host ABI checks passed\n");
  return g_fail ? 1 : 0;
}
