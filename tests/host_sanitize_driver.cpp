// Host-side checks of libdbd's argument validation, workspace sizing and carving, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (tests/test_host_sanitizers
// builds and runs it on the CPU).  Every call here returns before any HIP call: validation runs
// on the host before any launch, and the size queries never touch the device.
#include <cstdio>
#include <cstring>
#include <vector>

#include "dbd.h"

static int g_fails = 0;
#define EXPECT(cond)                                                                        \
  do {                                                                                      \
    if (!(cond)) {                                                                          \
      std::fprintf(stderr, "FAILED %s:%d %s (%s)\n", __FILE__, __LINE__, #cond,            \
                   dbd_last_error());                                                      \
      ++g_fails;                                                                            \
    }                                                                                       \
  } while (0)

static dbd_model_desc desc(int H, int qh, int kvh, int hd, int F, int L, int Lt, int V,
                           int dtype, int pairs) {
  dbd_model_desc d;
  std::memset(&d, 0, sizeof d);
  d.hidden = H; d.n_q_heads = qh; d.n_kv_heads = kvh; d.head_dim = hd; d.ffn = F;
  d.n_layers = L; d.n_target_layers = Lt; d.vocab = V; d.mask_token_id = V - 1;
  d.dtype = dtype; d.rms_eps = 1e-6f; d.act_pairs = pairs; d.rope_theta = 1e6;
  return d;
}

int main() {
  // the workload shapes and a few small ones, fp32 and bf16, with and without pairs
  std::vector<dbd_model_desc> ds = {
      desc(256, 4, 2, 64, 688, 2, 3, 1024, DBD_F32, 0),
      desc(2560, 32, 8, 128, 9728, 7, 9, 151936, DBD_BF16, 0),
      desc(4096, 32, 8, 128, 12288, 7, 9, 151936, DBD_BF16, 0),
      desc(2880, 64, 8, 64, 11520, 8, 7, 201088, DBD_BF16, 0),
      desc(3584, 28, 4, 128, 18944, 28, 0, 152064, DBD_BF16, 1),
      desc(512, 16, 2, 64, 1024, 2, 2, 2048, DBD_BF16, 1),
  };
  ds.push_back(ds[2]);
  ds.back().ctx_fusion = 1;
  ds.back().ctx_shared_kv = 1;
  const int batches[] = {1, 2, 3, 5, 8, 17, 32, 64};
  const int blocks[] = {2, 8, 16, 33, 64};
  const int ingests[] = {0, 1, 7, 100, 4097};
  const float temps[] = {0.f, 1.5f};
  int queries = 0;
  for (const dbd_model_desc& d : ds) {
    for (int N : batches)
      for (int B : blocks)
        for (int T : ingests)
          for (float t : temps) {
            const int na = d.n_target_layers ? 1 : 0;
            const int Tn = d.n_target_layers ? T : 0;
            const int K = t > 0.f ? 4 : 1;
            const int cap = ((3000 + B + 63) / 64) * 64;
            size_t bytes = 0, off = 0;
            int rc = dbd_draft_workspace_bytes(&d, N, B, na, Tn, K, t, cap, &bytes);
            EXPECT(rc == DBD_OK && bytes > 0 && bytes % 256 == 0);
            rc = dbd_draft_residual_offset(&d, N, B, na, Tn, K, t, cap, &off);
            EXPECT(rc == DBD_OK && off % 256 == 0 && off < bytes);
            ++queries;
          }
  }
  // validation: every one of these returns an error before any launch
  dbd_model_desc d = ds[2];
  dbd_weights w;
  std::memset(&w, 0, sizeof w);
  char* fake = reinterpret_cast<char*>(1 << 20);
  size_t b = 0;
  EXPECT(draft_block(&d, &w, 4, 16, 1, (int32_t*)fake, fake, 9 * 4096, 4096, 8, (int32_t*)fake,
                     (int32_t*)fake, fake, fake, 3136, 1, 0.f, 0, (int32_t*)fake, nullptr,
                     nullptr, fake, 1 << 30, nullptr) == DBD_ERR_ARG);        // NULL weights
  {
    // every weight present, one of them 8 bytes off a 16-byte boundary
    dbd_weights wa;
    const void** slots = reinterpret_cast<const void**>(&wa);
    for (size_t i = 0; i < sizeof wa / sizeof(void*); ++i) slots[i] = fake + 4096 * (i + 1);
    for (size_t bad = 0; bad < sizeof wa / sizeof(void*); ++bad) {
      slots[bad] = fake + 4096 * (bad + 1) + 8;
      EXPECT(draft_block(&d, &wa, 4, 16, 1, (int32_t*)fake, fake, 9 * 4096, 4096, 8,
                         (int32_t*)fake, (int32_t*)fake, fake, fake, 3136, 1, 0.f, 0,
                         (int32_t*)fake, nullptr, nullptr, fake, 1 << 30, nullptr) ==
             DBD_ERR_SHAPE);
      slots[bad] = fake + 4096 * (bad + 1);
    }
  }
  EXPECT(draft_block(&d, nullptr, 4, 16, 1, nullptr, nullptr, 0, 0, 0, nullptr, nullptr, nullptr,
                     nullptr, 3136, 1, 0.f, 0, nullptr, nullptr, nullptr, nullptr, 0,
                     nullptr) == DBD_ERR_ARG);
  EXPECT(dbd_draft_workspace_bytes(&d, 4, 65, 1, 0, 1, 0.f, 3136, &b) == DBD_ERR_SHAPE);
  EXPECT(dbd_draft_workspace_bytes(&d, 4, 16, 1, 0, 2, 0.f, 3136, &b) == DBD_ERR_ARG);
  EXPECT(dbd_draft_workspace_bytes(&d, 4, 16, 1, 0, 1, 0.f, 3100, &b) == DBD_ERR_CAPACITY);
  dbd_model_desc bad = d;
  bad.head_dim = 96;
  EXPECT(dbd_draft_workspace_bytes(&bad, 4, 16, 1, 0, 1, 0.f, 3136, &b) == DBD_ERR_SHAPE);
  bad = d;
  bad.vocab = 1 << 18;
  EXPECT(dbd_draft_workspace_bytes(&bad, 4, 16, 1, 0, 1, 0.f, 3136, &b) == DBD_ERR_SHAPE);
  bad = d;
  bad.n_q_heads = 30;
  EXPECT(dbd_draft_workspace_bytes(&bad, 4, 16, 1, 0, 1, 0.f, 3136, &b) == DBD_ERR_SHAPE);
  EXPECT(verify_greedy((float*)fake, (int32_t*)fake, 15, 32, 15, 17, 151936, (int32_t*)fake,
                       (int32_t*)fake, (int32_t*)fake, nullptr, fake, 1 << 30,
                       nullptr) == DBD_ERR_SHAPE);
  EXPECT(verify_greedy_noalloc((float*)fake, (int32_t*)fake, 64, 128, 64, 65, (1 << 18) - 1,
                               (int32_t*)fake, (int32_t*)fake, (int32_t*)fake, nullptr,
                               nullptr) == DBD_ERR_WORKSPACE);
  EXPECT(select_streak((float*)fake, (int32_t*)fake, 4, 8, 32, 34, 152064, (int32_t*)fake,
                       nullptr, (int32_t*)fake, (int32_t*)fake, (int32_t*)fake, nullptr, fake,
                       1 << 30, nullptr) == DBD_ERR_SHAPE);
  for (int cfg = -1; cfg <= 18; ++cfg)
    for (int split = 0; split <= 16; ++split) {
      size_t gb = 0;
      EXPECT(dbd_gemm_workspace_bytes(DBD_BF16, 512, 24576, 4096, cfg, split, &gb) == DBD_OK);
      EXPECT(dbd_gemm_workspace_bytes(DBD_BF16, 235, 1000, 2560, cfg, split, &gb) == DBD_OK);
    }
  EXPECT(dbd_gemm_override(DBD_STAGE_ATTN, 3, 0) == DBD_ERR_ARG);
  EXPECT(dbd_attn_override(8193, 0) == DBD_ERR_ARG);
  EXPECT(dbd_attn_override(-1, 0) == DBD_ERR_ARG);
  EXPECT(dbd_attn_override(0, 3) == DBD_ERR_ARG);
  EXPECT(dbd_attn_override(0, 0) == DBD_OK);
  std::printf("host checks: %d workspace queries, %d failures\n", queries, g_fails);
  return g_fails ? 1 : 0;
}
