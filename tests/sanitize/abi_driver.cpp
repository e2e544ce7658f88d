// Drives every entry point of the C ABI through its host-side checks (null pointers, bad and
// unsupported shapes, too-small workspaces, empty batches, the size queries and the status
// strings) so that a host address / undefined-behaviour sanitizer build of the library sees that
// code.  Nothing here reaches the GPU: every call returns before anything is enqueued.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "lsa.h"

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

static bool has_error() { return std::strlen(lsa_last_error()) > 0; }

int main() {
  void* p = reinterpret_cast<void*>(16);
  const int32_t* ip = static_cast<const int32_t*>(p);
  int32_t* op = static_cast<int32_t*>(p);
  float* fp = static_cast<float*>(p);
  for (int s = 0; s <= 6; ++s) CHECK(lsa_status_str(s) != nullptr);

  CHECK(lsa_index_scores(nullptr, nullptr, nullptr, nullptr, 2, 1, 32, 128, 100, nullptr, nullptr) == LSA_ERR_NULL_ARG && has_error());
  CHECK(lsa_index_scores(p, fp, p, ip, -1, 1, 32, 128, 100, fp, nullptr) == LSA_ERR_BAD_SHAPE && has_error());
  CHECK(lsa_index_scores(p, fp, p, ip, 1, 1, 33, 128, 100, fp, nullptr) == LSA_ERR_UNSUPPORTED && has_error());
  CHECK(lsa_index_scores(p, fp, p, ip, 1, 1, 32, 96, 100, fp, nullptr) == LSA_ERR_UNSUPPORTED && has_error());
  CHECK(lsa_index_scores(nullptr, nullptr, nullptr, nullptr, 0, 1, 32, 128, 100, nullptr, nullptr) == LSA_OK && !has_error());

  const size_t tneed = lsa_topk_workspace_bytes(32, 1, 131072, 2048, 16, 1024);
  CHECK(tneed > 0 && lsa_topk_workspace_bytes(1, 1, 4096, 8, 5, 4) == 0);
  CHECK(lsa_topk_select(fp, ip, 1, 1, 4096, 8, 5, 4, op, op, nullptr, 0, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_topk_select(fp, ip, 1, 1, (1 << 20) + 1, 2048, 16, 1024, op, op, nullptr, 0, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_topk_select(nullptr, ip, 1, 1, 4096, 256, 4, 64, op, op, nullptr, 0, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_topk_select(fp, ip, 32, 1, 131072, 2048, 16, 1024, op, op, p, tneed - 1, nullptr) == LSA_ERR_WORKSPACE && has_error());

  const size_t fneed = lsa_index_topk_workspace_bytes(32, 1, 131072, 2048, 16, 1024);
  CHECK(fneed > 0 && lsa_index_topk_workspace_bytes(1, 1, 4096, 8, 5, 4) == 0);
  CHECK(lsa_index_topk(p, fp, p, ip, 1, 1, 33, 128, 4096, 256, 4, 64, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_index_topk(p, fp, p, ip, 1, 1, 32, 128, 4096, 8, 5, 4, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_index_topk(p, nullptr, p, ip, 1, 1, 32, 128, 4096, 256, 4, 64, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_index_topk(p, fp, p, ip, 32, 1, 32, 128, 131072, 2048, 16, 1024, op, op, p, fneed - 1, nullptr) == LSA_ERR_WORKSPACE);
  CHECK(lsa_index_topk(nullptr, nullptr, nullptr, nullptr, 0, 1, 32, 128, 4096, 256, 4, 64, nullptr, nullptr, nullptr, 0, nullptr) == LSA_OK);

  const size_t mneed = lsa_mla_workspace_bytes(32, 1, 32, 512, 131072, 2048, 0);
  CHECK(mneed > 0 && lsa_mla_workspace_bytes(1, 4096, 32, 512, 131072, 2048, 0) == 0);
  CHECK(lsa_sparse_mla_decode(p, p, ip, ip, ip, 4, 32, 576, 640, 1000, 64, 0.1f, p, nullptr, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_sparse_mla_decode(p, p, ip, ip, ip, 4, 32, 512, 448, 1000, 64, 0.1f, p, nullptr, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_sparse_mla_decode(p, p, ip, nullptr, ip, 4, 32, 576, 512, 1000, 64, 0.1f, p, nullptr, p, size_t(1) << 30, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_sparse_mla_decode(p, p, ip, ip, ip, 4, 32, 576, 512, 1000, 64, std::nanf(""), p, nullptr, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_sparse_mla_decode(p, p, ip, ip, ip, 32, 32, 576, 512, 131072, 2048, 0.07f, p, nullptr, nullptr, 0, nullptr) == LSA_ERR_WORKSPACE && has_error());
  CHECK(lsa_sparse_mla_prefill(p, p, nullptr, nullptr, ip, 0, 10, 32, 576, 512, 100, 0, 0.1f, nullptr, nullptr, nullptr, 0, nullptr) == LSA_OK);
  // indexer front end: sizes, rotary and norm parameters, NULLs, workspace, empty batch
  const size_t feneed = lsa_index_frontend_workspace_bytes(32, 1, 1536, 3072, 32, 128);
  CHECK(feneed > 0 && lsa_index_frontend_workspace_bytes(32, 1, 1530, 3072, 32, 128) == 0);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1536, 3072, 32, 128, 63, 1e6f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE && has_error());
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1536, 3072, 32, 128, 130, 1e6f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1530, 3072, 32, 128, 64, 1e6f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1536, 3072, 32, 256, 64, 1e6f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1536, 3072, 32, 128, 64, 0.0f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 2, 1, 1536, 3072, 32, 128, 64, 1e6f, -1.0f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_index_frontend(p, p, p, p, nullptr, p, ip, 2, 1, 1536, 3072, 32, 128, 64, 1e6f, 1e-6f, 100, p, fp, p, p, size_t(1) << 30, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_index_frontend(p, p, p, p, fp, p, ip, 32, 1, 1536, 3072, 32, 128, 64, 1e6f, 1e-6f, 100, p, fp, p, p, feneed - 1, nullptr) == LSA_ERR_WORKSPACE && has_error());
  CHECK(lsa_index_frontend(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 1536, 3072, 32, 128, 64, 1e6f, 1e-6f, 100, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == LSA_OK && !has_error());

  // multi-token-prediction draft attention
  const size_t dneed = lsa_mtp_draft_workspace_bytes(32, 32, 512, 131072, 2048, 3);
  CHECK(dneed > 0 && lsa_mtp_draft_workspace_bytes(32, 32, 512, 131072, 2048, 65) == 0);
  CHECK(lsa_mtp_draft_attention(p, p, ip, ip, ip, ip, 4, 32, 576, 512, 131072, 2048, -1, 0.07f, p, fp, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE && has_error());
  CHECK(lsa_mtp_draft_attention(p, p, ip, ip, ip, ip, 4, 32, 576, 512, 131072, 65537, 3, 0.07f, p, fp, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_mtp_draft_attention(p, p, ip, ip, nullptr, ip, 4, 32, 576, 512, 131072, 2048, 3, 0.07f, p, fp, p, size_t(1) << 30, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_mtp_draft_attention(p, p, ip, ip, ip, ip, 32, 32, 576, 512, 131072, 2048, 3, 0.07f, p, fp, p, dneed - 1, nullptr) == LSA_ERR_WORKSPACE);
  CHECK(lsa_mtp_draft_attention(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 32, 576, 512, 100, 64, 3, 0.1f, nullptr, nullptr, nullptr, 0, nullptr) == LSA_OK && !has_error());
  // hierarchical indexing
  CHECK(lsa_block_keys(p, ip, 2, 4096, 128, 48, 0, p, nullptr) == LSA_ERR_UNSUPPORTED && has_error());
  CHECK(lsa_block_keys(p, ip, 2, 4096, 128, 64, -1, p, nullptr) == LSA_ERR_BAD_SHAPE);
  CHECK(lsa_block_keys(p, nullptr, 2, 4096, 128, 64, 0, p, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_block_keys(nullptr, nullptr, 0, 4096, 128, 64, 0, nullptr, nullptr) == LSA_OK && !has_error());
  const size_t hneed = lsa_hier_workspace_bytes(4, 131072, 64, 2048, 16, 1024, 32);
  CHECK(hneed > 0 && lsa_hier_workspace_bytes(4, 131072, 64, 2048, 16, 1024, 15) == 0);
  CHECK(lsa_hier_index_topk(p, fp, p, p, ip, 4, 32, 128, 131072, 2048, 16, 1024, 64, 15, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_BAD_SHAPE && has_error());
  CHECK(lsa_hier_index_topk(p, fp, p, p, ip, 4, 33, 128, 131072, 2048, 16, 1024, 64, 32, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_UNSUPPORTED);
  CHECK(lsa_hier_index_topk(p, fp, p, nullptr, ip, 4, 32, 128, 131072, 2048, 16, 1024, 64, 32, op, op, p, size_t(1) << 30, nullptr) == LSA_ERR_NULL_ARG);
  CHECK(lsa_hier_index_topk(p, fp, p, p, ip, 4, 32, 128, 131072, 2048, 16, 1024, 64, 32, op, op, p, hneed - 1, nullptr) == LSA_ERR_WORKSPACE);
  CHECK(lsa_hier_index_topk(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 32, 128, 131072, 2048, 16, 1024, 64, 32, nullptr, nullptr, nullptr, 0, nullptr) == LSA_OK && !has_error());
  std::puts("abi driver: ok");
  return 0;
}
