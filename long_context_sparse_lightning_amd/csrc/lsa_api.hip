// C ABI of the LSA hot path (declared in include/lsa.h): argument checks, workspace sizing and
// kernel launches.  Every check happens before anything is enqueued; on failure the status is
// returned and a thread-local message describes it.
#include <stdarg.h>
#include <stdio.h>

#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "lsa.h"
#include "lsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

lsa_status fail(lsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

lsa_status ok() {
  g_last_error[0] = '\0';
  return LSA_OK;
}

lsa_status launched(hipError_t err, const char* what) {
  if (err != hipSuccess)
    return fail(LSA_ERR_LAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(err));
  return ok();
}

// LSA_DEBUG_BOUNDS set (and not "0") in the environment: every entry point copies its sequence
// lengths to the host, waits for them and checks the device-side preconditions before
// launching (a debugging mode: it synchronises the stream on every call).
bool debug_bounds() {
  static const bool on = [] {
    const char* e = getenv("LSA_DEBUG_BOUNDS");
    return e != nullptr && *e != '\0' && strcmp(e, "0") != 0;
  }();
  return on;
}

lsa_status debug_check(const char* fn, const int32_t* seqlens, int B, int Lq, int S_max, void* stream,
                       const int32_t* index_seqlens = nullptr) {
  if (!debug_bounds() || B <= 0) return LSA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> h(static_cast<size_t>(B)), hi(index_seqlens ? static_cast<size_t>(B) : 0);
  hipError_t err = hipMemcpyAsync(h.data(), seqlens, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess && index_seqlens)
    err = hipMemcpyAsync(hi.data(), index_seqlens, hi.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess)
    return fail(LSA_ERR_LAUNCH, "%s: LSA_DEBUG_BOUNDS copy of seqlens failed: %s", fn, hipGetErrorString(err));
  const int bad = lsa_check_seqlens(h.data(), B, Lq, S_max);
  if (bad >= 0)
    return fail(LSA_ERR_BAD_SHAPE, "%s: seqlens[%d] = %d outside [Lq = %d, S_max = %d] (LSA_DEBUG_BOUNDS)", fn,
                bad, h[bad], Lq, S_max);
  for (int b = 0; b < static_cast<int>(hi.size()); ++b)
    if (hi[b] < 0 || hi[b] > h[b])
      return fail(LSA_ERR_BAD_SHAPE, "%s: index_seqlens[%d] = %d outside [0, seqlens[%d] = %d] (LSA_DEBUG_BOUNDS)",
                  fn, b, hi[b], b, h[b]);
  return LSA_OK;
}

}  // namespace

// ------------------------------------------------------------------ no-allocation variant
// The workspace of lsa_index_topk_noalloc: one static array per device the library runs on,
// resident until the process ends.  Host code never uses the array's name as an address (in
// host code it names a host-side stand-in): its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[LSA_INDEX_TOPK_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// Device address of `scratch` on the device that runs `stream` (the current device for the
// NULL stream), looked up on the first call for that device.
lsa_status scratch_for(hipStream_t stream, void** out, const char* fn) {
  int dev = 0;
  hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) return fail(LSA_ERR_LAUNCH, "%s: no device for the stream: %s", fn, hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LSA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the static workspace covers", fn, dev, kMaxDevices);
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      if ((err = hipGetDevice(&cur)) != hipSuccess)
        return fail(LSA_ERR_LAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(err));
      if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess)
        return fail(LSA_ERR_LAUNCH, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(err));
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (err != hipSuccess || !p)
        return fail(LSA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                    hipGetErrorString(err));
      if (back != hipSuccess)
        return fail(LSA_ERR_LAUNCH, "%s: hipSetDevice(%d): %s", fn, cur, hipGetErrorString(back));
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LSA_OK;
}
}  // namespace

extern "C" {

const char* lsa_status_str(lsa_status s) {
  switch (s) {
    case LSA_OK: return "LSA_OK";
    case LSA_ERR_NULL_ARG: return "LSA_ERR_NULL_ARG";
    case LSA_ERR_BAD_SHAPE: return "LSA_ERR_BAD_SHAPE";
    case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED";
    case LSA_ERR_WORKSPACE: return "LSA_ERR_WORKSPACE";
    case LSA_ERR_LAUNCH: return "LSA_ERR_LAUNCH";
    default: return "LSA_ERR_UNKNOWN";
  }
}

const char* lsa_last_error(void) { return g_last_error; }

int lsa_check_seqlens(const int32_t* seqlens_host, int B, int Lq, int S_max) {
  for (int b = 0; b < B; ++b)
    if (seqlens_host[b] < Lq || seqlens_host[b] > S_max) return b;
  return -1;
}

lsa_status lsa_index_scores(const void* q_idx, const float* w, const void* k_idx,
                            const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                            float* scores, void* stream) {
  if (B < 0 || Lq < 0) return fail(LSA_ERR_BAD_SHAPE, "lsa_index_scores: B=%d Lq=%d must be >= 0", B, Lq);
  if (Hi <= 0 || Di <= 0 || S_max <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "lsa_index_scores: Hi=%d Di=%d S_max=%d must be > 0", Hi, Di, S_max);
  if (Hi > 32) return fail(LSA_ERR_UNSUPPORTED, "lsa_index_scores: Hi=%d > 32", Hi);
  if (Di != 32 && Di != 64 && Di != 128)
    return fail(LSA_ERR_UNSUPPORTED, "lsa_index_scores: Di=%d not in {32, 64, 128}", Di);
  if (B == 0 || Lq == 0) return ok();
  if (!q_idx || !w || !k_idx || !seqlens || !scores)
    return fail(LSA_ERR_NULL_ARG, "lsa_index_scores: NULL q_idx/w/k_idx/seqlens/scores");
  if (lsa_status st = debug_check("lsa_index_scores", seqlens, B, Lq, S_max, stream)) return st;
  return launched(lsa::launch_index_scores(static_cast<const uint16_t*>(q_idx), w,
                                           static_cast<const uint16_t*>(k_idx), seqlens, B, Lq, Hi,
                                           Di, S_max, scores, static_cast<hipStream_t>(stream)),
                  "lsa_index_scores");
}

static lsa_status check_topk(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  if (B < 0 || Lq < 0) return fail(LSA_ERR_BAD_SHAPE, "lsa_topk_select: B=%d Lq=%d must be >= 0", B, Lq);
  if (S_max <= 0 || topk <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "lsa_topk_select: S_max=%d topk=%d must be > 0", S_max, topk);
  if (init_tokens < 0 || local_tokens < 0 ||
      static_cast<long>(init_tokens) + local_tokens > topk)
    return fail(LSA_ERR_BAD_SHAPE,
                "lsa_topk_select: need 0 <= init_tokens (%d), 0 <= local_tokens (%d), sum <= topk (%d)",
                init_tokens, local_tokens, topk);
  if (S_max > lsa::topk_max_positions())
    return fail(LSA_ERR_UNSUPPORTED, "lsa_topk_select: S_max=%d > %d", S_max, lsa::topk_max_positions());
  return LSA_OK;
}

size_t lsa_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens,
                                int local_tokens) {
  if (check_topk(B, Lq, S_max, topk, init_tokens, local_tokens) != LSA_OK) return 0;
  return lsa::topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens);
}

lsa_status lsa_topk_select(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max,
                           int topk, int init_tokens, int local_tokens, int32_t* indices,
                           int32_t* n_sel, void* workspace, size_t workspace_bytes, void* stream) {
  lsa_status st = check_topk(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (st != LSA_OK) return st;
  if (B == 0 || Lq == 0) return ok();
  if (!scores || !seqlens || !indices || !n_sel)
    return fail(LSA_ERR_NULL_ARG, "lsa_topk_select: NULL scores/seqlens/indices/n_sel");
  const size_t need = lsa::topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_WORKSPACE, "lsa_topk_select: workspace %zu bytes at %p, need %zu",
                workspace_bytes, workspace, need);
  if ((st = debug_check("lsa_topk_select", seqlens, B, Lq, S_max, stream))) return st;
  return launched(lsa::launch_topk(scores, seqlens, B, Lq, S_max, topk, init_tokens, local_tokens,
                                   indices, n_sel, workspace, static_cast<hipStream_t>(stream)),
                  "lsa_topk_select");
}

static lsa_status check_index(const char* fn, int B, int Lq, int Hi, int Di, int S_max) {
  if (B < 0 || Lq < 0) return fail(LSA_ERR_BAD_SHAPE, "%s: B=%d Lq=%d must be >= 0", fn, B, Lq);
  if (Hi <= 0 || Di <= 0 || S_max <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "%s: Hi=%d Di=%d S_max=%d must be > 0", fn, Hi, Di, S_max);
  if (Hi > 32) return fail(LSA_ERR_UNSUPPORTED, "%s: Hi=%d > 32", fn, Hi);
  if (Di != 32 && Di != 64 && Di != 128)
    return fail(LSA_ERR_UNSUPPORTED, "%s: Di=%d not in {32, 64, 128}", fn, Di);
  return LSA_OK;
}

size_t lsa_index_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens,
                                      int local_tokens) {
  if (check_topk(B, Lq, S_max, topk, init_tokens, local_tokens) != LSA_OK) return 0;
  if (B == 0 || Lq == 0) return 0;
  return lsa::index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens);
}

lsa_status lsa_index_topk(const void* q_idx, const float* w, const void* k_idx,
                          const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max, int topk,
                          int init_tokens, int local_tokens, int32_t* indices, int32_t* n_sel,
                          void* workspace, size_t workspace_bytes, void* stream) {
  lsa_status st = check_index("lsa_index_topk", B, Lq, Hi, Di, S_max);
  if (st != LSA_OK) return st;
  st = check_topk(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (st != LSA_OK) return st;
  if (B == 0 || Lq == 0) return ok();
  if (!q_idx || !w || !k_idx || !seqlens || !indices || !n_sel)
    return fail(LSA_ERR_NULL_ARG, "lsa_index_topk: NULL q_idx/w/k_idx/seqlens/indices/n_sel");
  const size_t need = lsa::index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_WORKSPACE, "lsa_index_topk: workspace %zu bytes at %p, need %zu",
                workspace_bytes, workspace, need);
  if ((st = debug_check("lsa_index_topk", seqlens, B, Lq, S_max, stream))) return st;
  return launched(lsa::launch_index_topk(static_cast<const uint16_t*>(q_idx), w,
                                         static_cast<const uint16_t*>(k_idx), seqlens, B, Lq, Hi, Di,
                                         S_max, topk, init_tokens, local_tokens, indices, n_sel,
                                         workspace, static_cast<hipStream_t>(stream)),
                  "lsa_index_topk");
}

// lsa_index_topk without a workspace argument: its workspace is the static `scratch` array.
lsa_status lsa_index_topk_noalloc(const void* q_idx, const float* w, const void* k_idx,
                                  const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                                  int topk, int init_tokens, int local_tokens, int32_t* indices,
                                  int32_t* n_sel, void* stream) {
  const char* fn = "lsa_index_topk_noalloc";
  lsa_status st = check_index(fn, B, Lq, Hi, Di, S_max);
  if (st != LSA_OK) return st;
  st = check_topk(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (st != LSA_OK) return st;
  if (B == 0 || Lq == 0) return ok();
  if (!q_idx || !w || !k_idx || !seqlens || !indices || !n_sel)
    return fail(LSA_ERR_NULL_ARG, "%s: NULL q_idx/w/k_idx/seqlens/indices/n_sel", fn);
  const size_t need = lsa::index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (need > LSA_INDEX_TOPK_SCRATCH_BYTES)
    return fail(LSA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of workspace, more than the %zu of the static one",
                fn, need, static_cast<size_t>(LSA_INDEX_TOPK_SCRATCH_BYTES));
  if ((st = debug_check(fn, seqlens, B, Lq, S_max, stream))) return st;
  void* ws = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = scratch_for(s, &ws, fn)) != LSA_OK) return st;
  return launched(lsa::launch_index_topk(static_cast<const uint16_t*>(q_idx), w,
                                         static_cast<const uint16_t*>(k_idx), seqlens, B, Lq, Hi, Di,
                                         S_max, topk, init_tokens, local_tokens, indices, n_sel, ws, s),
                  fn);
}

static bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

static lsa_status check_blocks(const char* fn, int B, int S_max, int Di, int Bk) {
  if (B < 0 || S_max <= 0 || Di <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "%s: B=%d S_max=%d Di=%d", fn, B, S_max, Di);
  if (!pow2_in(Bk, 8, 1024) || Bk > S_max)
    return fail(LSA_ERR_UNSUPPORTED, "%s: Bk=%d must be a power of two in [8, 1024], <= S_max=%d", fn,
                Bk, S_max);
  if (Di % 16 || Di > 128) return fail(LSA_ERR_UNSUPPORTED, "%s: Di=%d not a multiple of 16 <= 128", fn, Di);
  return LSA_OK;
}

lsa_status lsa_block_keys(const void* k_idx, const int32_t* seqlens, int B, int S_max, int Di,
                          int Bk, int first_block, void* block_keys, void* stream) {
  const char* fn = "lsa_block_keys";
  lsa_status st = check_blocks(fn, B, S_max, Di, Bk);
  if (st != LSA_OK) return st;
  if (first_block < 0) return fail(LSA_ERR_BAD_SHAPE, "%s: first_block=%d < 0", fn, first_block);
  if (B == 0) return ok();
  if (!k_idx || !seqlens || !block_keys) return fail(LSA_ERR_NULL_ARG, "%s: NULL k_idx/seqlens/block_keys", fn);
  if ((st = debug_check(fn, seqlens, B, 0, S_max, stream))) return st;
  return launched(lsa::launch_block_keys(static_cast<const uint16_t*>(k_idx), seqlens, B, S_max, Di, Bk,
                                         first_block, static_cast<uint16_t*>(block_keys),
                                         static_cast<hipStream_t>(stream)),
                  fn);
}

static lsa_status check_hier(int B, int S_max, int topk, int init_tokens, int local_tokens, int Bk,
                             int M) {
  const char* fn = "lsa_hier_index_topk";
  lsa_status st = check_topk(B, 1, S_max, topk, init_tokens, local_tokens);
  if (st != LSA_OK) return st;
  if (!pow2_in(Bk, 8, 1024) || Bk > S_max)
    return fail(LSA_ERR_UNSUPPORTED, "%s: Bk=%d must be a power of two in [8, 1024], <= S_max=%d", fn,
                Bk, S_max);
  if (M < 1 || M > S_max / Bk)
    return fail(LSA_ERR_BAD_SHAPE, "%s: M=%d outside [1, S_max / Bk = %d]", fn, M, S_max / Bk);
  if (static_cast<long>(M) * Bk < static_cast<long>(topk) - local_tokens)
    return fail(LSA_ERR_BAD_SHAPE, "%s: M*Bk=%ld below topk - local_tokens=%d (too few candidates)", fn,
                static_cast<long>(M) * Bk, topk - local_tokens);
  return LSA_OK;
}

size_t lsa_hier_workspace_bytes(int B, int S_max, int Bk, int topk, int init_tokens,
                                int local_tokens, int M) {
  if (B <= 0 || check_hier(B, S_max, topk, init_tokens, local_tokens, Bk, M) != LSA_OK) return 0;
  return lsa::hier_workspace_bytes(B, S_max, Bk, topk, init_tokens, local_tokens, M);
}

lsa_status lsa_hier_index_topk(const void* q_idx, const float* w, const void* k_idx,
                               const void* block_keys, const int32_t* seqlens, int B, int Hi,
                               int Di, int S_max, int topk, int init_tokens, int local_tokens,
                               int Bk, int M, int32_t* indices, int32_t* n_sel, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const char* fn = "lsa_hier_index_topk";
  lsa_status st = check_hier(B, S_max, topk, init_tokens, local_tokens, Bk, M);
  if (st != LSA_OK) return st;
  if (Hi <= 0 || Hi > lsa::hier_max_heads() || Di <= 0 || Di % 16 || Di > 128)
    return fail(LSA_ERR_UNSUPPORTED, "%s: Hi=%d (<= %d) Di=%d (multiple of 16, <= 128)", fn, Hi,
                lsa::hier_max_heads(), Di);
  if (B == 0) return ok();
  if (!q_idx || !w || !k_idx || !block_keys || !seqlens || !indices || !n_sel)
    return fail(LSA_ERR_NULL_ARG, "%s: NULL input or output", fn);
  const size_t need = lsa::hier_workspace_bytes(B, S_max, Bk, topk, init_tokens, local_tokens, M);
  if (!workspace || workspace_bytes < need)
    return fail(LSA_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", fn, workspace_bytes,
                workspace, need);
  if ((st = debug_check(fn, seqlens, B, 1, S_max, stream))) return st;
  return launched(lsa::launch_hier_index_topk(static_cast<const uint16_t*>(q_idx), w,
                                              static_cast<const uint16_t*>(k_idx),
                                              static_cast<const uint16_t*>(block_keys), seqlens, B,
                                              Hi, Di, S_max, topk, init_tokens, local_tokens, Bk, M,
                                              indices, n_sel, workspace, static_cast<hipStream_t>(stream)),
                  fn);
}

static lsa_status check_mla(const char* fn, int B, int Lq, int H, int Dqk, int Dv, int S_max, int topk,
                            bool dense, float softmax_scale) {
  if (B < 0 || Lq < 0) return fail(LSA_ERR_BAD_SHAPE, "%s: B=%d Lq=%d must be >= 0", fn, B, Lq);
  if (H <= 0 || Dqk <= 0 || Dv <= 0 || S_max <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "%s: H=%d Dqk=%d Dv=%d S_max=%d must be > 0", fn, H, Dqk, Dv, S_max);
  if (Dv > Dqk) return fail(LSA_ERR_BAD_SHAPE, "%s: Dv=%d > Dqk=%d", fn, Dv, Dqk);
  if (!dense && topk <= 0) return fail(LSA_ERR_BAD_SHAPE, "%s: topk=%d must be > 0", fn, topk);
  if (!dense && topk > LSA_MLA_MAX_TOPK)
    return fail(LSA_ERR_UNSUPPORTED, "%s: topk=%d > %d", fn, topk, LSA_MLA_MAX_TOPK);
  if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY || softmax_scale == -INFINITY)
    return fail(LSA_ERR_BAD_SHAPE, "%s: softmax_scale must be finite", fn);
  if (!((Dqk == 576 && Dv == 512) || (Dqk == 80 && Dv == 64)))
    return fail(LSA_ERR_UNSUPPORTED, "%s: (Dqk, Dv) = (%d, %d) not in {(576, 512), (80, 64)}", fn,
                Dqk, Dv);
  return LSA_OK;
}

size_t lsa_mla_workspace_bytes(int B, int Lq, int H, int Dv, int S_max, int topk, int dense) {
  if (B <= 0 || Lq <= 0 || H <= 0 || Dv <= 0 || S_max <= 0 ||
      (!dense && (topk <= 0 || topk > LSA_MLA_MAX_TOPK)))
    return 0;
  return lsa::mla_workspace_bytes(B, Lq, H, Dv, S_max, topk, dense);
}

static lsa_status run_mla(const char* fn, const void* q, const void* kv, const int32_t* indices,
                          const int32_t* n_sel, const int32_t* seqlens, int B, int Lq, int H,
                          int Dqk, int Dv, int S_max, int topk, float softmax_scale, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const bool dense = indices == nullptr;
  lsa_status st = check_mla(fn, B, Lq, H, Dqk, Dv, S_max, topk, dense, softmax_scale);
  if (st != LSA_OK) return st;
  if (B == 0 || Lq == 0) return ok();
  if (!q || !kv || !seqlens || !out) return fail(LSA_ERR_NULL_ARG, "%s: NULL q/kv/seqlens/out", fn);
  if (!dense && !n_sel) return fail(LSA_ERR_NULL_ARG, "%s: indices given without n_sel", fn);
  const size_t need = lsa::mla_workspace_bytes(B, Lq, H, Dv, S_max, topk, dense);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", fn, workspace_bytes,
                workspace, need);
  if ((st = debug_check(fn, seqlens, B, Lq, S_max, stream))) return st;
  return launched(lsa::launch_mla(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv),
                                  indices, n_sel, seqlens, B, Lq, H, Dqk, Dv, S_max, dense ? 0 : topk,
                                  softmax_scale, static_cast<uint16_t*>(out), lse, workspace,
                                  static_cast<hipStream_t>(stream)),
                  fn);
}

lsa_status lsa_sparse_mla_decode(const void* q, const void* kv, const int32_t* indices,
                                 const int32_t* n_sel, const int32_t* seqlens, int B, int H,
                                 int Dqk, int Dv, int S_max, int topk, float softmax_scale,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return run_mla("lsa_sparse_mla_decode", q, kv, indices, n_sel, seqlens, B, 1, H, Dqk, Dv, S_max,
                 topk, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

lsa_status lsa_sparse_mla_prefill(const void* q, const void* kv, const int32_t* indices,
                                  const int32_t* n_sel, const int32_t* seqlens, int B, int Lq,
                                  int H, int Dqk, int Dv, int S_max, int topk,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return run_mla("lsa_sparse_mla_prefill", q, kv, indices, n_sel, seqlens, B, Lq, H, Dqk, Dv,
                 S_max, topk, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

size_t lsa_mtp_draft_workspace_bytes(int B, int H, int Dv, int S_max, int topk, int max_appended) {
  if (B <= 0 || H <= 0 || Dv <= 0 || S_max <= 0 || topk <= 0 || topk > LSA_MTP_MAX_TOPK ||
      max_appended < 0 || max_appended > LSA_MTP_MAX_APPENDED)
    return 0;
  return lsa::mla_workspace_bytes(B, 1, H, Dv, S_max, topk, 0, max_appended);
}

lsa_status lsa_mtp_draft_attention(const void* q, const void* kv, const int32_t* indices,
                                   const int32_t* n_sel, const int32_t* index_seqlens,
                                   const int32_t* seqlens, int B, int H, int Dqk, int Dv,
                                   int S_max, int topk, int max_appended, float softmax_scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const char* fn = "lsa_mtp_draft_attention";
  lsa_status st = check_mla(fn, B, 1, H, Dqk, Dv, S_max, topk, false, softmax_scale);
  if (st != LSA_OK) return st;
  if (max_appended < 0 || max_appended > LSA_MTP_MAX_APPENDED)
    return fail(LSA_ERR_BAD_SHAPE, "%s: max_appended=%d outside [0, %d]", fn, max_appended,
                LSA_MTP_MAX_APPENDED);
  if (topk > LSA_MTP_MAX_TOPK)
    return fail(LSA_ERR_UNSUPPORTED, "%s: topk=%d > %d", fn, topk, LSA_MTP_MAX_TOPK);
  if (B == 0) return ok();
  if (!q || !kv || !seqlens || !out) return fail(LSA_ERR_NULL_ARG, "%s: NULL q/kv/seqlens/out", fn);
  if (!indices || !n_sel || !index_seqlens)
    return fail(LSA_ERR_NULL_ARG, "%s: NULL indices/n_sel/index_seqlens", fn);
  const size_t need = lsa::mla_workspace_bytes(B, 1, H, Dv, S_max, topk, 0, max_appended);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", fn, workspace_bytes,
                workspace, need);
  if ((st = debug_check(fn, seqlens, B, 1, S_max, stream, index_seqlens))) return st;
  return launched(lsa::launch_mla(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv),
                                  indices, n_sel, seqlens, B, 1, H, Dqk, Dv, S_max, topk, softmax_scale,
                                  static_cast<uint16_t*>(out), lse, workspace,
                                  static_cast<hipStream_t>(stream), index_seqlens, max_appended),
                  fn);
}

static lsa_status check_frontend(int B, int Lq, int q_lora, int hidden, int Hi, int Di,
                                 int rope_dim, int S_max) {
  const char* fn = "lsa_index_frontend";
  if (B < 0 || Lq < 0) return fail(LSA_ERR_BAD_SHAPE, "%s: B=%d Lq=%d must be >= 0", fn, B, Lq);
  if (q_lora <= 0 || hidden <= 0 || Hi <= 0 || Di <= 0 || S_max <= 0)
    return fail(LSA_ERR_BAD_SHAPE, "%s: q_lora=%d hidden=%d Hi=%d Di=%d S_max=%d must be > 0", fn,
                q_lora, hidden, Hi, Di, S_max);
  if (rope_dim < 0 || rope_dim > Di || (rope_dim & 1) || (Di & 1))
    return fail(LSA_ERR_BAD_SHAPE, "%s: rope_dim=%d must be even and in [0, Di=%d], Di even", fn,
                rope_dim, Di);
  if (q_lora % 16 || hidden % 16)
    return fail(LSA_ERR_UNSUPPORTED, "%s: q_lora=%d and hidden=%d must be multiples of 16", fn,
                q_lora, hidden);
  if (Di > 128 || Hi > 32) return fail(LSA_ERR_UNSUPPORTED, "%s: Di=%d > 128 or Hi=%d > 32", fn, Di, Hi);
  if (rope_dim > lsa::frontend_max_rot())
    return fail(LSA_ERR_UNSUPPORTED, "%s: rope_dim=%d > %d", fn, rope_dim, lsa::frontend_max_rot());
  return LSA_OK;
}

size_t lsa_index_frontend_workspace_bytes(int B, int Lq, int q_lora, int hidden, int Hi, int Di) {
  if (check_frontend(B, Lq, q_lora, hidden, Hi, Di, 0, 1) != LSA_OK) return 0;
  return lsa::frontend_workspace_bytes(B, Lq, q_lora, hidden, Hi, Di);
}

lsa_status lsa_index_frontend(const void* cq, const void* hid, const void* wq_b, const void* wk,
                              const float* k_norm_gain, const void* w_proj, const int32_t* seqlens,
                              int B, int Lq, int q_lora, int hidden, int Hi, int Di, int rope_dim,
                              float rope_theta, float norm_eps, int S_max, void* q_idx, float* w,
                              void* k_cache, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const char* fn = "lsa_index_frontend";
  lsa_status st = check_frontend(B, Lq, q_lora, hidden, Hi, Di, rope_dim, S_max);
  if (st != LSA_OK) return st;
  if (!(rope_theta > 0.0f) || rope_theta == INFINITY || !(norm_eps >= 0.0f) || norm_eps == INFINITY)
    return fail(LSA_ERR_BAD_SHAPE, "%s: rope_theta=%g must be finite > 0, norm_eps=%g finite >= 0",
                fn, rope_theta, norm_eps);
  if (B == 0 || Lq == 0) return ok();
  if (!cq || !hid || !wq_b || !wk || !k_norm_gain || !w_proj || !seqlens || !q_idx || !w || !k_cache)
    return fail(LSA_ERR_NULL_ARG, "%s: NULL input or output", fn);
  const size_t need = lsa::frontend_workspace_bytes(B, Lq, q_lora, hidden, Hi, Di);
  if (!workspace || workspace_bytes < need)
    return fail(LSA_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", fn, workspace_bytes,
                workspace, need);
  if ((st = debug_check(fn, seqlens, B, Lq, S_max, stream))) return st;
  return launched(lsa::launch_frontend(static_cast<const uint16_t*>(cq), static_cast<const uint16_t*>(hid),
                                       static_cast<const uint16_t*>(wq_b), static_cast<const uint16_t*>(wk),
                                       k_norm_gain, static_cast<const uint16_t*>(w_proj), seqlens, B, Lq,
                                       q_lora, hidden, Hi, Di, rope_dim, rope_theta, norm_eps, S_max,
                                       static_cast<uint16_t*>(q_idx), w, static_cast<uint16_t*>(k_cache),
                                       workspace, static_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"
