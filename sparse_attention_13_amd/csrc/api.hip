// api.hip -- the C ABI declared in include/dsa.h: argument validation, kernel selection, workspace
// layout.  Nothing here allocates, frees or synchronises; every failure is reported before any work
// is enqueued.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

// masked MHA mode: one workgroup's LDS holds a query row's mask words (2 per 64 keys, 64 KiB)
constexpr int kMhaMaxKeys = 1 << 19;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status_t ok() {
  g_last_error.clear();
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxTopK = 65536;

// ---------------------------------------------------------------------------------------- indexer
dsa_status_t check_indexer(const void* q, const float* q_scale, const void* k, const float* k_scale, const float* w,
                           int B, int n_q, int n_kv, int H_I, int d_I, dsa_dtype_t dtype, const float* scores,
                           int64_t ld, bool* fast) {
  if (!q || !k || !w || !scores) return fail(DSA_ERR_INVALID_ARG, "indexer: null q, k, w or scores");
  if (B < 1 || n_q < 1 || n_kv < 1 || H_I < 1 || d_I < 1)
    return fail(DSA_ERR_INVALID_ARG, "indexer: sizes must be positive (B=%d n_q=%d n_kv=%d H_I=%d d_I=%d)", B, n_q,
                n_kv, H_I, d_I);
  if (n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "indexer: n_q=%d exceeds n_kv=%d", n_q, n_kv);
  if (ld < n_kv) return fail(DSA_ERR_INVALID_ARG, "indexer: ld_scores=%lld < n_kv=%d", (long long)ld, n_kv);
  if (dtype == DSA_FP8_E4M3) {
    if (!q_scale || !k_scale) return fail(DSA_ERR_INVALID_ARG, "indexer: fp8 inputs need q_scale and k_scale");
  } else if (dtype == DSA_F32) {
    if (q_scale || k_scale) return fail(DSA_ERR_INVALID_ARG, "indexer: fp32 inputs take no scales (pass NULL)");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer: dtype %d not supported (fp8 e4m3 or fp32)", (int)dtype);
  }
  *fast = dtype == DSA_FP8_E4M3 && H_I == 64 && d_I == 128 && aligned(q, 16) && aligned(k, 16);
  if (!*fast && !(H_I <= 64 && d_I <= 256 && d_I % 4 == 0 && (size_t)(H_I * d_I + H_I) * 4 <= 65536))
    return fail(DSA_ERR_UNSUPPORTED, "indexer: H_I=%d d_I=%d not supported (fast path 64x128 fp8; generic H_I<=64, "
                "d_I<=256, d_I%%4==0)", H_I, d_I);
  return DSA_OK;
}

dsa_status_t run_indexer(const void* q, const float* q_scale, const void* k, const float* k_scale, const float* w,
                         int B, int n_q, int n_kv, int H_I, int d_I, dsa_dtype_t dtype, float* scores, int64_t ld,
                         bool fast, hipStream_t stream) {
  hipError_t e;
  if (fast)
    e = dsa::launch_indexer_fp8((const uint8_t*)q, q_scale, (const uint8_t*)k, k_scale, w, B, n_q, n_kv, scores, ld, 0,
                                stream);
  else
    e = dsa::launch_indexer_generic(q, q_scale, k, k_scale, w, B, n_q, n_kv, H_I, d_I, dtype == DSA_FP8_E4M3, scores,
                                    ld, stream);
  return hip_status(e, "dsa_indexer_scores");
}

// ------------------------------------------------------------------------------------------- top-k
dsa_status_t check_topk(const float* scores, int64_t ld, int B, int n_q, int n_kv, int k, const int32_t* idx) {
  if (!scores || !idx) return fail(DSA_ERR_INVALID_ARG, "topk: null scores or idx");
  if (B < 1 || n_q < 1 || n_kv < 1) return fail(DSA_ERR_INVALID_ARG, "topk: sizes must be positive");
  if (n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "topk: n_q=%d exceeds n_kv=%d", n_q, n_kv);
  if (ld < n_kv) return fail(DSA_ERR_INVALID_ARG, "topk: ld_scores=%lld < n_kv=%d", (long long)ld, n_kv);
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_INVALID_ARG, "topk: k=%d outside [1, %d]", k, kMaxTopK);
  if (n_q > 65535 * 1024 || B > 65535) return fail(DSA_ERR_UNSUPPORTED, "topk: grid too large");
  return DSA_OK;
}

dsa_status_t check_topk_ws(const dsa::TopkPlan& p, const void* workspace, size_t ws_bytes) {
  if (p.ws == 0) return DSA_OK;
  if (!workspace) return fail(DSA_ERR_WORKSPACE, "topk: workspace of %zu bytes required", p.ws);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_WORKSPACE, "topk: workspace must be 256-byte aligned");
  if (ws_bytes < p.ws) return fail(DSA_ERR_WORKSPACE, "topk: workspace %zu < %zu bytes", ws_bytes, p.ws);
  return DSA_OK;
}

// ------------------------------------------------------------------------------------------- attention
struct AttnPlan {
  bool fast = false;
  int n_split = 1;
  size_t ws = 0;
};

dsa_status_t plan_attn(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k, dsa_dtype_t dtype, AttnPlan* p) {
  if (B < 1 || n_q < 1 || n_kv < 1 || H < 1 || d_qk < 1 || d_v < 1 || k < 1)
    return fail(DSA_ERR_INVALID_ARG, "attn: sizes must be positive");
  if (d_v > d_qk) return fail(DSA_ERR_INVALID_ARG, "attn: d_v=%d exceeds d_qk=%d", d_v, d_qk);
  if (k > kMaxTopK) return fail(DSA_ERR_INVALID_ARG, "attn: k=%d exceeds %d", k, kMaxTopK);
  if (dtype == DSA_BF16) {
    if (!(H == 128 && d_qk == 576 && d_v == 512))
      return fail(DSA_ERR_UNSUPPORTED, "attn: bf16 supports H=128, d_qk=576, d_v=512 (got %d, %d, %d)", H, d_qk, d_v);
    // the kernel's row gathers address the rope part of a row with a 32-bit byte offset from the sequence's
    // base (row * 1152 + 1152 bytes at most), exact for every row below 2^21
    if (n_kv > (1 << 21)) return fail(DSA_ERR_UNSUPPORTED, "attn: bf16 supports n_kv <= 2^21 (got %d)", n_kv);
    p->fast = true;
    p->n_split = dsa::mla_bf16_pick_split(B, n_q, k);
    p->ws = dsa::mla_bf16_workspace_bytes(B, n_q, p->n_split);
  } else if (dtype == DSA_F32) {
    if (!(d_qk <= 256 && (size_t)(d_qk + k + 4) * 4 <= 65536 && H <= 65535))
      return fail(DSA_ERR_UNSUPPORTED, "attn: fp32 generic kernel needs d_qk<=256 and (d_qk+k)*4 <= 64 KiB");
    p->fast = false;
    p->n_split = 1;
    p->ws = 0;
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "attn: dtype %d not supported (bf16 or fp32)", (int)dtype);
  }
  if (n_q > 65535 * 64 || B > 65535) return fail(DSA_ERR_UNSUPPORTED, "attn: grid too large");
  return DSA_OK;
}

dsa_status_t check_attn_ptrs(const void* q, const void* kv, const int32_t* idx, const void* out, float sm_scale,
                             const AttnPlan& p, const void* ws, size_t ws_bytes) {
  if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "attn: null q, kv, idx or out");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "attn: sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (p.fast && !(aligned(q, 16) && aligned(kv, 16) && aligned(out, 16)))
    return fail(DSA_ERR_INVALID_ARG, "attn: bf16 path needs 16-byte aligned q, kv and out");
  if (p.ws > 0) {
    if (!ws) return fail(DSA_ERR_WORKSPACE, "attn: workspace of %zu bytes required", p.ws);
    if (!aligned(ws, 256)) return fail(DSA_ERR_WORKSPACE, "attn: workspace must be 256-byte aligned");
    if (ws_bytes < p.ws) return fail(DSA_ERR_WORKSPACE, "attn: workspace %zu < %zu bytes", ws_bytes, p.ws);
  }
  return DSA_OK;
}

dsa_status_t run_attn(const void* q, const void* kv, const int32_t* idx, int B, int n_q, int n_kv, int H, int d_qk,
                      int d_v, int k, float sm_scale, void* out, float* lse, const AttnPlan& p, void* ws,
                      hipStream_t stream) {
  hipError_t e;
  if (p.fast)
    e = dsa::launch_mla_bf16((const uint16_t*)q, (const uint16_t*)kv, idx, B, n_q, n_kv, k, sm_scale, (uint16_t*)out,
                             lse, p.n_split, ws, stream);
  else
    e = dsa::launch_attn_generic((const float*)q, (const float*)kv, idx, B, n_q, n_kv, H, d_qk, d_v, k, sm_scale,
                                 (float*)out, lse, stream);
  return hip_status(e, "dsa_sparse_mla_attn");
}

// ------------------------------------------------------------------------------------------- forward
struct FwdLayout {
  int64_t ld = 0;
  size_t off_scores = 0, off_idx = 0, off_topk = 0, off_attn = 0, total = 0;
  AttnPlan attn;
  dsa::TopkPlan topk;
};

dsa_status_t plan_forward(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k, dsa_dtype_t attn_dtype,
                          FwdLayout* L) {
  dsa_status_t st = plan_attn(B, n_q, n_kv, H, d_qk, d_v, k, attn_dtype, &L->attn);
  if (st != DSA_OK) return st;
  if (n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "forward: n_q=%d exceeds n_kv=%d", n_q, n_kv);
  L->ld = (int64_t)align_up((size_t)n_kv, 64);
  L->off_scores = 0;
  L->off_idx = align_up((size_t)B * n_q * L->ld * sizeof(float), 256);
  L->topk = dsa::plan_topk(B, n_q, n_kv, k);
  L->off_topk = align_up(L->off_idx + (size_t)B * n_q * k * sizeof(int32_t), 256);
  L->off_attn = L->off_topk + align_up(L->topk.ws, 256);
  L->total = L->off_attn + align_up(L->attn.ws, 256);
  return DSA_OK;
}

dsa_status_t forward(const void* q_i, const float* q_i_scale, const void* k_i, const float* k_i_scale, const float* w,
                     const void* q, const void* kv, int B, int n_q, int n_kv, int H_I, int d_I, int H, int d_qk,
                     int d_v, int k, float sm_scale, dsa_dtype_t idx_dtype, dsa_dtype_t attn_dtype, void* out,
                     float* lse, int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream_) {
  FwdLayout L;
  dsa_status_t st = plan_forward(B, n_q, n_kv, H, d_qk, d_v, k, attn_dtype, &L);
  if (st != DSA_OK) return st;
  if (!workspace) return fail(DSA_ERR_WORKSPACE, "forward: workspace of %zu bytes required", L.total);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_WORKSPACE, "forward: workspace must be 256-byte aligned");
  if (ws_bytes < L.total) return fail(DSA_ERR_WORKSPACE, "forward: workspace %zu < %zu bytes", ws_bytes, L.total);
  char* ws = (char*)workspace;
  float* scores = (float*)(ws + L.off_scores);
  int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + L.off_idx);
  bool fast_idx = false;
  st = check_indexer(q_i, q_i_scale, k_i, k_i_scale, w, B, n_q, n_kv, H_I, d_I, idx_dtype, scores, L.ld, &fast_idx);
  if (st != DSA_OK) return st;
  st = check_topk(scores, L.ld, B, n_q, n_kv, k, idx);
  if (st != DSA_OK) return st;
  st = check_attn_ptrs(q, kv, idx, out, sm_scale, L.attn, L.attn.ws ? ws + L.off_attn : nullptr, L.attn.ws);
  if (st != DSA_OK) return st;
  hipStream_t stream = (hipStream_t)stream_;
  st = run_indexer(q_i, q_i_scale, k_i, k_i_scale, w, B, n_q, n_kv, H_I, d_I, idx_dtype, scores, L.ld, fast_idx,
                   stream);
  if (st != DSA_OK) return st;
  st = hip_status(dsa::launch_topk(scores, L.ld, B, n_q, n_kv, k, idx, L.topk, ws + L.off_topk, stream), "dsa_topk");
  if (st != DSA_OK) return st;
  return run_attn(q, kv, idx, B, n_q, n_kv, H, d_qk, d_v, k, sm_scale, out, lse, L.attn,
                  L.attn.ws ? ws + L.off_attn : nullptr, stream);
}

// Workspace of the masked-MHA-mode forward: scores, selection, top-k candidates, selection bitmask.
struct MhaFwdLayout {
  int64_t ld = 0;
  size_t off_idx = 0, off_topk = 0, off_mask = 0, total = 0;
  dsa::TopkPlan topk;
};

dsa_status_t plan_forward_mha(int B, int n_q, int n_kv, int k_sel, MhaFwdLayout* L) {
  if (B < 1 || n_q < 1 || n_kv < 1 || k_sel < 1) return fail(DSA_ERR_INVALID_ARG, "forward_mha: sizes must be positive");
  if (n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "forward_mha: n_q=%d exceeds n_kv=%d", n_q, n_kv);
  if (k_sel > kMaxTopK) return fail(DSA_ERR_INVALID_ARG, "forward_mha: k=%d exceeds %d", k_sel, kMaxTopK);
  if (n_kv > kMhaMaxKeys) return fail(DSA_ERR_UNSUPPORTED, "forward_mha: n_kv=%d exceeds %d", n_kv, kMhaMaxKeys);
  L->ld = (int64_t)align_up((size_t)n_kv, 64);
  L->off_idx = align_up((size_t)B * n_q * L->ld * sizeof(float), 256);
  L->topk = dsa::plan_topk(B, n_q, n_kv, k_sel);
  L->off_topk = align_up(L->off_idx + (size_t)B * n_q * k_sel * sizeof(int32_t), 256);
  L->off_mask = L->off_topk + align_up(L->topk.ws, 256);
  L->total = L->off_mask + align_up((size_t)B * n_q * dsa::mha_mask_words(n_kv) * 4, 256);
  return DSA_OK;
}

// ------------------------------------------------------------------------------------------------
// Device scratch of the allocation-free decode entry point.  Each device holds its own copy of the
// array from module load until the process ends.  Host code never passes the array's name to a kernel
// (in host code it is only a stand-in): the per-device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
// ------------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// The calling thread's current device's scratch address (nullptr, with the error text set, on failure).
void* device_scratch(dsa_status_t* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = fail(DSA_ERR_HIP, "forward_decode_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    *st = fail(DSA_ERR_UNSUPPORTED, "forward_decode_noalloc: device %d beyond the %d devices served", dev,
               kMaxScratchDevices);
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    *st = fail(DSA_ERR_HIP, "forward_decode_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int dsa_version(void) { return 100; }

const char* dsa_status_string(dsa_status_t s) {
  // A C caller may pass any int: read the bits as an int (a C++ load of an enum outside its range is
  // undefined), then compare.
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: no kernel for this dtype/shape";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime error";
  }
  return "unknown dsa_status_t";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status_t dsa_indexer_scores(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                const float* w, int B, int n_q, int n_kv, int H_I, int d_I, dsa_dtype_t dtype,
                                float* scores, int64_t ld_scores, void* stream) {
  bool fast = false;
  dsa_status_t st = check_indexer(q, q_scale, k, k_scale, w, B, n_q, n_kv, H_I, d_I, dtype, scores, ld_scores, &fast);
  if (st != DSA_OK) return st;
  return run_indexer(q, q_scale, k, k_scale, w, B, n_q, n_kv, H_I, d_I, dtype, scores, ld_scores, fast,
                     (hipStream_t)stream);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int B, int n_q, int n_kv, int k, int32_t* idx,
                      void* workspace, size_t ws_bytes, void* stream) {
  dsa_status_t st = check_topk(scores, ld_scores, B, n_q, n_kv, k, idx);
  if (st != DSA_OK) return st;
  const dsa::TopkPlan p = dsa::plan_topk(B, n_q, n_kv, k);
  st = check_topk_ws(p, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  return hip_status(dsa::launch_topk(scores, ld_scores, B, n_q, n_kv, k, idx, p, workspace, (hipStream_t)stream),
                    "dsa_topk");
}

size_t dsa_topk_workspace_size(int B, int n_q, int n_kv, int k) {
  if (B < 1 || n_q < 1 || n_kv < 1 || k < 1 || k > kMaxTopK || n_q > n_kv) return 0;
  return dsa::plan_topk(B, n_q, n_kv, k).ws;
}

size_t dsa_sparse_mla_attn_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                          dsa_dtype_t dtype) {
  AttnPlan p;
  if (plan_attn(B, n_q, n_kv, H, d_qk, d_v, k, dtype, &p) != DSA_OK) return 0;
  return p.ws;
}

dsa_status_t dsa_sparse_mla_attn(const void* q, const void* kv, const int32_t* idx, int B, int n_q, int n_kv, int H,
                                 int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t dtype, void* out, float* lse,
                                 void* workspace, size_t ws_bytes, void* stream) {
  AttnPlan p;
  dsa_status_t st = plan_attn(B, n_q, n_kv, H, d_qk, d_v, k, dtype, &p);
  if (st != DSA_OK) return st;
  st = check_attn_ptrs(q, kv, idx, out, sm_scale, p, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  return run_attn(q, kv, idx, B, n_q, n_kv, H, d_qk, d_v, k, sm_scale, out, lse, p, workspace, (hipStream_t)stream);
}

size_t dsa_sparse_mla_backward_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                              dsa_dtype_t dtype) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv || k < 1 || k > 2048 || H != 128 || d_qk != 576 || d_v != 512 ||
      dtype != DSA_BF16 || (int64_t)B * n_q > 0x7FFFFFFF || (int64_t)B * n_kv > (1 << 26))
    return 0;
  return dsa::sbwd_workspace_bytes(B, n_q, n_kv, k);
}

dsa_status_t dsa_sparse_mla_backward(const void* q, const void* kv, const int32_t* idx, const void* out,
                                     const float* lse, const void* dout, int B, int n_q, int n_kv, int H, int d_qk,
                                     int d_v, int k, float sm_scale, dsa_dtype_t dtype, float* dq, float* dkv,
                                     float* pbar, void* workspace, size_t ws_bytes, void* stream) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv || k < 1) return fail(DSA_ERR_INVALID_ARG, "sparse_backward: bad sizes");
  if (dtype != DSA_BF16 || H != 128 || d_qk != 576 || d_v != 512)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_backward: supports bf16 with H=128, d_qk=576, d_v=512");
  if (k > 2048 || n_kv > (1 << 21) || (int64_t)B * n_q > 0x7FFFFFFF || (int64_t)B * n_kv > (1 << 26))
    return fail(DSA_ERR_UNSUPPORTED, "sparse_backward: k <= 2048, n_kv <= 2^21, B * n_kv <= 2^26");
  if (!q || !kv || !idx || !out || !lse || !dout || !dq || !dkv)
    return fail(DSA_ERR_INVALID_ARG, "sparse_backward: null pointer");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "sparse_backward: sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (!(aligned(q, 16) && aligned(kv, 16) && aligned(out, 16) && aligned(dout, 16)))
    return fail(DSA_ERR_INVALID_ARG, "sparse_backward: q, kv, out, dout must be 16-byte aligned");
  const size_t need = dsa::sbwd_workspace_bytes(B, n_q, n_kv, k);
  if (workspace == nullptr || ws_bytes < need || !aligned(workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "sparse_backward: workspace of %zu bytes (256-byte aligned) needed", need);
  return hip_status(dsa::launch_sparse_backward((const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)out, lse,
                                                (const uint16_t*)dout, B, n_q, n_kv, k, sm_scale, dq, dkv, pbar,
                                                workspace, (hipStream_t)stream),
                    "dsa_sparse_mla_backward");
}

dsa_status_t dsa_sparse_kl_loss(float* scores, int64_t ld_scores, const float* pbar, const int32_t* idx, int B,
                                int n_q, int n_kv, int k, float* loss, void* stream) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv || k < 1) return fail(DSA_ERR_INVALID_ARG, "sparse_kl_loss: bad sizes");
  if (B > 65535) return fail(DSA_ERR_UNSUPPORTED, "sparse_kl_loss: grid too large");
  if (!scores || !pbar || !idx || !loss) return fail(DSA_ERR_INVALID_ARG, "sparse_kl_loss: null pointer");
  if (ld_scores < n_kv) return fail(DSA_ERR_INVALID_ARG, "sparse_kl_loss: ld_scores below n_kv");
  return hip_status(dsa::launch_sparse_kl(scores, ld_scores, pbar, idx, B, n_q, n_kv, k, loss, (hipStream_t)stream),
                    "dsa_sparse_kl_loss");
}

dsa_status_t dsa_warmup_loss(const void* q, const void* kv, const float* lse, int B, int n_q, int n_kv, int H, int d_qk,
                             float sm_scale, dsa_dtype_t dtype, float* scores, int64_t ld_scores, float* target,
                             int64_t ld_target, float* loss, void* stream) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "warmup_loss: bad sizes");
  if (dtype != DSA_BF16 || H != 128 || d_qk != 576)
    return fail(DSA_ERR_UNSUPPORTED, "warmup_loss: supports bf16 with H=128, d_qk=576 (got %d, %d)", H, d_qk);
  if (B > 65535 || n_kv > (1 << 21)) return fail(DSA_ERR_UNSUPPORTED, "warmup_loss: B <= 65535, n_kv <= 2^21");
  if (!q || !kv || !lse || !scores || !target || !loss) return fail(DSA_ERR_INVALID_ARG, "warmup_loss: null pointer");
  if (ld_scores < n_kv || ld_target < n_kv) return fail(DSA_ERR_INVALID_ARG, "warmup_loss: ld below n_kv");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "warmup_loss: sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (!(aligned(q, 16) && aligned(kv, 16))) return fail(DSA_ERR_INVALID_ARG, "warmup_loss: q, kv must be 16-byte aligned");
  return hip_status(dsa::launch_warmup_forward((const uint16_t*)q, (const uint16_t*)kv, lse, B, n_q, n_kv, sm_scale,
                                               scores, ld_scores, target, ld_target, loss, (hipStream_t)stream),
                    "dsa_warmup_loss");
}

dsa_status_t dsa_warmup_indexer_backward(const void* q_i, const float* q_i_scale, const void* k_i,
                                         const float* k_i_scale, const float* w, const float* grad, int64_t ld_grad,
                                         int B, int n_q, int n_kv, int H_I, int d_I, dsa_dtype_t dtype, float* dq_i,
                                         float* dw, float* dk_i, void* stream) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "warmup_backward: bad sizes");
  if (dtype != DSA_FP8_E4M3 || H_I != 64 || d_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "warmup_backward: supports fp8 e4m3 with H_I=64, d_I=128");
  if (B > 65535 || n_kv > (1 << 21)) return fail(DSA_ERR_UNSUPPORTED, "warmup_backward: B <= 65535, n_kv <= 2^21");
  if (!q_i || !q_i_scale || !k_i || !k_i_scale || !w || !grad || !dq_i || !dw || !dk_i)
    return fail(DSA_ERR_INVALID_ARG, "warmup_backward: null pointer");
  if (ld_grad < n_kv) return fail(DSA_ERR_INVALID_ARG, "warmup_backward: ld_grad below n_kv");
  if (!(aligned(q_i, 16) && aligned(k_i, 16) && aligned(dq_i, 16)))
    return fail(DSA_ERR_INVALID_ARG, "warmup_backward: q_i, k_i and dq_i must be 16-byte aligned");
  return hip_status(dsa::launch_warmup_backward((const uint8_t*)q_i, q_i_scale, (const uint8_t*)k_i, k_i_scale, w,
                                                grad, ld_grad, B, n_q, n_kv, dq_i, dw, dk_i, (hipStream_t)stream),
                    "dsa_warmup_indexer_backward");
}

dsa_status_t dsa_mla_absorb_q(const void* q_mha, const void* w_ukt, void* q_mqa, int rows, int H, int d_nope,
                              int d_rope, int d_c, dsa_dtype_t dtype, void* stream) {
  if (rows < 1 || H < 1) return fail(DSA_ERR_INVALID_ARG, "absorb_q: rows and H must be positive");
  if (dtype != DSA_BF16 || d_nope != 128 || d_rope != 64 || d_c != 512)
    return fail(DSA_ERR_UNSUPPORTED, "absorb_q: supports bf16 with d_nope=128, d_rope=64, d_c=512");
  if (rows > (1 << 30) || (((long long)rows + 127) / 128 * H + 7) / 8 * 8 * 4 > 0x7FFFFFFFLL)
    return fail(DSA_ERR_UNSUPPORTED, "absorb_q: rows <= 2^30 and a grid below 2^31 workgroups");
  if (!q_mha || !w_ukt || !q_mqa) return fail(DSA_ERR_INVALID_ARG, "absorb_q: null pointer");
  if (!(aligned(q_mha, 16) && aligned(w_ukt, 16) && aligned(q_mqa, 16)))
    return fail(DSA_ERR_INVALID_ARG, "absorb_q: pointers must be 16-byte aligned");
  return hip_status(dsa::launch_mla_absorb_q((const uint16_t*)q_mha, (const uint16_t*)w_ukt, (uint16_t*)q_mqa, rows,
                                             H, (hipStream_t)stream),
                    "dsa_mla_absorb_q");
}

dsa_status_t dsa_mla_out_proj(const void* o_lat, const void* w_uv, void* o, int rows, int H, int d_c, int d_v,
                              dsa_dtype_t dtype, void* stream) {
  if (rows < 1 || H < 1) return fail(DSA_ERR_INVALID_ARG, "out_proj: rows and H must be positive");
  if (dtype != DSA_BF16 || d_c != 512 || d_v != 128)
    return fail(DSA_ERR_UNSUPPORTED, "out_proj: supports bf16 with d_c=512, d_v=128");
  if (rows > (1 << 30) || (((long long)rows + 127) / 128 * H + 7) / 8 * 8 > 0x7FFFFFFFLL)
    return fail(DSA_ERR_UNSUPPORTED, "out_proj: rows <= 2^30 and a grid below 2^31 workgroups");
  if (!o_lat || !w_uv || !o) return fail(DSA_ERR_INVALID_ARG, "out_proj: null pointer");
  if (!(aligned(o_lat, 16) && aligned(w_uv, 16) && aligned(o, 16)))
    return fail(DSA_ERR_INVALID_ARG, "out_proj: pointers must be 16-byte aligned");
  return hip_status(dsa::launch_mla_out_proj((const uint16_t*)o_lat, (const uint16_t*)w_uv, (uint16_t*)o, rows, H,
                                             (hipStream_t)stream),
                    "dsa_mla_out_proj");
}

size_t dsa_masked_mha_workspace_size(int B, int n_q, int n_kv) {
  if (B < 1 || n_q < 1 || n_kv < 1 || n_q > n_kv || n_kv > kMhaMaxKeys) return 0;
  return align_up((size_t)B * n_q * dsa::mha_mask_words(n_kv) * 4, 256);
}

dsa_status_t dsa_masked_mha_attn(const void* q, const void* k, const void* v, const int32_t* idx, int B, int n_q,
                                 int n_kv, int H, int d_qk, int d_v, int k_sel, float sm_scale, dsa_dtype_t dtype,
                                 void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (B < 1 || n_q < 1 || n_kv < 1 || H < 1 || k_sel < 1)
    return fail(DSA_ERR_INVALID_ARG, "masked_mha: sizes must be positive");
  if (n_q > n_kv) return fail(DSA_ERR_INVALID_ARG, "masked_mha: n_q=%d exceeds n_kv=%d", n_q, n_kv);
  if (dtype != DSA_BF16 || d_qk != 192 || d_v != 128)
    return fail(DSA_ERR_UNSUPPORTED, "masked_mha: supports bf16 with d_qk=192, d_v=128 (got dtype %d, %d, %d)",
                (int)dtype, d_qk, d_v);
  if (n_kv > kMhaMaxKeys) return fail(DSA_ERR_UNSUPPORTED, "masked_mha: n_kv=%d exceeds %d", n_kv, kMhaMaxKeys);
  if (B > 65535 || (long long)((n_q + 127) / 128) * H > 0x7FFFFFFFLL)
    return fail(DSA_ERR_UNSUPPORTED, "masked_mha: grid too large");
  if (!q || !k || !v || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "masked_mha: null q, k, v, idx or out");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "masked_mha: sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (!(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(out, 16)))
    return fail(DSA_ERR_INVALID_ARG, "masked_mha: q, k, v and out must be 16-byte aligned");
  const size_t need = dsa_masked_mha_workspace_size(B, n_q, n_kv);
  if (!workspace) return fail(DSA_ERR_WORKSPACE, "masked_mha: workspace of %zu bytes required", need);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_WORKSPACE, "masked_mha: workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "masked_mha: workspace %zu < %zu bytes", ws_bytes, need);
  const hipError_t e = dsa::launch_masked_mha((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, B, n_q,
                                              n_kv, H, k_sel, sm_scale, (uint16_t*)out, lse, (uint32_t*)workspace,
                                              (hipStream_t)stream);
  return hip_status(e, "dsa_masked_mha_attn");
}

size_t dsa_forward_workspace_size(int B, int n_q, int n_kv, int H, int d_qk, int d_v, int k,
                                  dsa_dtype_t attn_dtype) {
  FwdLayout L;
  if (plan_forward(B, n_q, n_kv, H, d_qk, d_v, k, attn_dtype, &L) != DSA_OK) return 0;
  return L.total;
}

dsa_status_t dsa_forward_prefill(const void* q_i, const float* q_i_scale, const void* k_i, const float* k_i_scale,
                                 const float* w, const void* q, const void* kv, int B, int n_q, int n_kv, int H_I,
                                 int d_I, int H, int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t idx_dtype,
                                 dsa_dtype_t attn_dtype, void* out, float* lse, int32_t* idx_out, void* workspace,
                                 size_t ws_bytes, void* stream) {
  return forward(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, B, n_q, n_kv, H_I, d_I, H, d_qk, d_v, k, sm_scale,
                 idx_dtype, attn_dtype, out, lse, idx_out, workspace, ws_bytes, stream);
}

dsa_status_t dsa_forward_decode(const void* q_i, const float* q_i_scale, const void* k_i, const float* k_i_scale,
                                const float* w, const void* q, const void* kv, int B, int n_kv, int H_I, int d_I,
                                int H, int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t idx_dtype,
                                dsa_dtype_t attn_dtype, void* out, float* lse, int32_t* idx_out, void* workspace,
                                size_t ws_bytes, void* stream) {
  return forward(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, B, 1, n_kv, H_I, d_I, H, d_qk, d_v, k, sm_scale, idx_dtype,
                 attn_dtype, out, lse, idx_out, workspace, ws_bytes, stream);
}


// ---------------------------------------------------------------------------------------- decode stages
dsa_status_t dsa_indexer_scores_decode(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                       const float* w, int B, int n_kv, int H_I, int d_I, dsa_dtype_t dtype,
                                       float* scores, int64_t ld_scores, void* stream) {
  return dsa_indexer_scores(q, q_scale, k, k_scale, w, B, 1, n_kv, H_I, d_I, dtype, scores, ld_scores, stream);
}

size_t dsa_topk_decode_workspace_size(int B, int n_kv, int k) { return dsa_topk_workspace_size(B, 1, n_kv, k); }

dsa_status_t dsa_topk_decode(const float* scores, int64_t ld_scores, int B, int n_kv, int k, int32_t* idx,
                             void* workspace, size_t ws_bytes, void* stream) {
  return dsa_topk(scores, ld_scores, B, 1, n_kv, k, idx, workspace, ws_bytes, stream);
}

size_t dsa_sparse_mla_attn_decode_workspace_size(int B, int n_kv, int H, int d_qk, int d_v, int k,
                                                 dsa_dtype_t dtype) {
  return dsa_sparse_mla_attn_workspace_size(B, 1, n_kv, H, d_qk, d_v, k, dtype);
}

dsa_status_t dsa_sparse_mla_attn_decode(const void* q, const void* kv, const int32_t* idx, int B, int n_kv, int H,
                                        int d_qk, int d_v, int k, float sm_scale, dsa_dtype_t dtype, void* out,
                                        float* lse, void* workspace, size_t ws_bytes, void* stream) {
  return dsa_sparse_mla_attn(q, kv, idx, B, 1, n_kv, H, d_qk, d_v, k, sm_scale, dtype, out, lse, workspace, ws_bytes,
                             stream);
}

// ---------------------------------------------------------------------------------------- masked MHA mode forward
size_t dsa_forward_prefill_masked_mha_workspace_size(int B, int n_q, int n_kv, int k_sel) {
  MhaFwdLayout L;
  if (plan_forward_mha(B, n_q, n_kv, k_sel, &L) != DSA_OK) return 0;
  return L.total;
}

dsa_status_t dsa_forward_prefill_masked_mha(const void* q_i, const float* q_i_scale, const void* k_i,
                                            const float* k_i_scale, const float* w, const void* q, const void* k,
                                            const void* v, int B, int n_q, int n_kv, int H_I, int d_I, int H,
                                            int d_qk, int d_v, int k_sel, float sm_scale, dsa_dtype_t idx_dtype,
                                            dsa_dtype_t attn_dtype, void* out, float* lse, int32_t* idx_out,
                                            void* workspace, size_t ws_bytes, void* stream_) {
  MhaFwdLayout L;
  dsa_status_t st = plan_forward_mha(B, n_q, n_kv, k_sel, &L);
  if (st != DSA_OK) return st;
  if (attn_dtype != DSA_BF16 || d_qk != 192 || d_v != 128)
    return fail(DSA_ERR_UNSUPPORTED, "forward_mha: attention supports bf16 with d_qk=192, d_v=128 (got dtype %d, %d, %d)",
                (int)attn_dtype, d_qk, d_v);
  if (H < 1) return fail(DSA_ERR_INVALID_ARG, "forward_mha: H must be positive");
  if (B > 65535 || (long long)((n_q + 127) / 128) * H > 0x7FFFFFFFLL)
    return fail(DSA_ERR_UNSUPPORTED, "forward_mha: grid too large");
  if (!q || !k || !v || !out) return fail(DSA_ERR_INVALID_ARG, "forward_mha: null q, k, v or out");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "forward_mha: sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (!(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(out, 16)))
    return fail(DSA_ERR_INVALID_ARG, "forward_mha: q, k, v and out must be 16-byte aligned");
  if (!workspace) return fail(DSA_ERR_WORKSPACE, "forward_mha: workspace of %zu bytes required", L.total);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_WORKSPACE, "forward_mha: workspace must be 256-byte aligned");
  if (ws_bytes < L.total) return fail(DSA_ERR_WORKSPACE, "forward_mha: workspace %zu < %zu bytes", ws_bytes, L.total);
  char* ws = (char*)workspace;
  float* scores = (float*)ws;
  int32_t* idx = idx_out ? idx_out : (int32_t*)(ws + L.off_idx);
  bool fast_idx = false;
  st = check_indexer(q_i, q_i_scale, k_i, k_i_scale, w, B, n_q, n_kv, H_I, d_I, idx_dtype, scores, L.ld, &fast_idx);
  if (st != DSA_OK) return st;
  st = check_topk(scores, L.ld, B, n_q, n_kv, k_sel, idx);
  if (st != DSA_OK) return st;
  hipStream_t stream = (hipStream_t)stream_;
  st = run_indexer(q_i, q_i_scale, k_i, k_i_scale, w, B, n_q, n_kv, H_I, d_I, idx_dtype, scores, L.ld, fast_idx, stream);
  if (st != DSA_OK) return st;
  st = hip_status(dsa::launch_topk(scores, L.ld, B, n_q, n_kv, k_sel, idx, L.topk, ws + L.off_topk, stream), "dsa_topk");
  if (st != DSA_OK) return st;
  return hip_status(dsa::launch_masked_mha((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, B, n_q, n_kv,
                                           H, k_sel, sm_scale, (uint16_t*)out, lse, (uint32_t*)(ws + L.off_mask), stream),
                    "dsa_forward_prefill_masked_mha");
}

// ---------------------------------------------------------------------------------------- allocation-free decode
size_t dsa_forward_decode_noalloc_max_bytes(void) { return kScratchBytes; }

dsa_status_t dsa_forward_decode_noalloc(const void* q_i, const float* q_i_scale, const void* k_i,
                                        const float* k_i_scale, const float* w, const void* q, const void* kv, int B,
                                        int n_kv, int H_I, int d_I, int H, int d_qk, int d_v, int k, float sm_scale,
                                        dsa_dtype_t idx_dtype, dsa_dtype_t attn_dtype, void* out, float* lse,
                                        int32_t* idx_out, void* stream) {
  FwdLayout L;
  dsa_status_t st = plan_forward(B, 1, n_kv, H, d_qk, d_v, k, attn_dtype, &L);
  if (st != DSA_OK) return st;
  if (L.total > kScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "forward_decode_noalloc: this call needs %zu bytes of scratch, beyond the fixed %zu bytes (fewer "
                "sequences or a shorter context, or dsa_forward_decode with a workspace)",
                L.total, kScratchBytes);
  // Argument errors come before the scratch lookup, so they read DSA_ERR_INVALID_ARG on any machine; the
  // full checks run again in forward().
  if (!q_i || !k_i || !w || !q || !kv || !out)
    return fail(DSA_ERR_INVALID_ARG, "forward_decode_noalloc: null q_i, k_i, w, q, kv or out");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "forward_decode_noalloc: sm_scale must be finite and > 0 (got %g)",
                (double)sm_scale);
  void* ws = device_scratch(&st);
  if (!ws) return st;
  return forward(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, B, 1, n_kv, H_I, d_I, H, d_qk, d_v, k, sm_scale, idx_dtype,
                 attn_dtype, out, lse, idx_out, ws, kScratchBytes, stream);
}

}  // extern "C"
