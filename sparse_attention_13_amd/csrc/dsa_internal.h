// dsa_internal.h -- shared definitions of the gfx950 kernels behind include/dsa.h.
// Internal to the library: kernels, launch helpers and the vector types used with the CDNA4
// matrix-core builtins.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// bf16 <-> fp32.  Widening is exact; narrowing is the hardware round-to-nearest-even conversion.
__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __uint_as_float(((unsigned int)b) << 16);
}
// Two fp32 -> packed bf16x2 (low half = a): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((v2f){a, b}, v2bf));
}
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  return (unsigned short)(pack_bf16x2(f, 0.f) & 0xFFFFu);
}

// OCP e4m3fn byte -> fp32 through the hardware converter.
__device__ __forceinline__ float e4m3_to_f32(unsigned int byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Sum of x over the lane pair (l, l ^ 32).
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum of x over the lane pair (l, l ^ 16).
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dsa

// ---------------------------------------------------------------------------------------------
// Launch helpers (host side), one per kernel family.  They assume arguments already validated by
// the C-ABI layer and return the HIP launch status.
// ---------------------------------------------------------------------------------------------
namespace dsa {

hipError_t launch_indexer_generic(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                  const float* w, int B, int n_q, int n_kv, int H_I, int d_I, bool fp8,
                                  float* scores, int64_t ld, hipStream_t stream);

// FP8 matrix-core indexer, H_I = 64, d_I = 128.  keys_per_wave <= 0 means "whole causal row".
hipError_t launch_indexer_fp8(const uint8_t* q, const float* q_scale, const uint8_t* k, const float* k_scale,
                              const float* w, int B, int n_q, int n_kv, float* scores, int64_t ld,
                              int keys_per_wave, hipStream_t stream);

// Top-k launch plan: one LDS-resident pass per row; for few long rows, threshold candidates per chunk
// and an exact merge per row; two stages (each chunk's top k in a workspace, then a merge) for rows too
// long or too few otherwise; or a kernel that re-reads long rows from memory.
struct TopkPlan {
  enum Mode { kSingle = 0, kTwoStage = 1, kUncached = 2, kCandidates = 3 };
  int mode;
  int chunk;     // keys per chunk (two stages, candidates)
  int n_chunks;
  int t_lo;      // candidates: keys a chunk keeps at least
  size_t ws;     // workspace bytes (two stages, candidates), else 0
};
TopkPlan plan_topk(int B, int n_q, int n_kv, int k);
hipError_t launch_topk(const float* scores, int64_t ld, int B, int n_q, int n_kv, int k, int32_t* idx,
                       const TopkPlan& plan, void* workspace, hipStream_t stream);

hipError_t launch_attn_generic(const float* q, const float* kv, const int32_t* idx, int B, int n_q, int n_kv,
                               int H, int d_qk, int d_v, int k, float sm_scale, float* out, float* lse,
                               hipStream_t stream);

// bf16 matrix-core sparse MLA, H = 128, d_qk = 576, d_v = 512.  n_split > 1 splits each query's
// selection into n_split contiguous parts whose partial results go to `partial` (normalised O in bf16,
// then the parts' log-sum-exp in fp32) and are merged by a second kernel.
// MQA-mode projections (bf16, H heads): q_mqa [rows][H][576] from q_mha [rows][H][192] and w_ukt [H][512][128];
// o [rows][H][128] from o_lat [rows][H][512] and w_uv [H][128][512].
hipError_t launch_mla_absorb_q(const uint16_t* q_mha, const uint16_t* w_ukt, uint16_t* q_mqa, int rows, int H,
                               hipStream_t stream);
hipError_t launch_mla_out_proj(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int rows, int H,
                               hipStream_t stream);
// Indexer warm-up loss: target p [B][n_q][ld_p] from the main attention (bf16, H = 128, d_qk = 576) and its
// log-sum-exp lse [B][n_q][128], then per row the loss and g = softmax(I) - p over the scores [B][n_q][ld_s].
hipError_t launch_warmup_forward(const uint16_t* q, const uint16_t* kv, const float* lse, int B, int n_q, int n_kv,
                                 float sm_scale, float* scores, int64_t ld_s, float* p, int64_t ld_p, float* loss,
                                 hipStream_t stream);
// Gradients of the warm-up loss through the fp8 indexer (H_I = 64, d_I = 128), given g [B][n_q][ld_g]:
// dq [B][n_q][64][128], dw [B][n_q][64], dk [B][n_kv][128] fp32 (dk is zeroed, then accumulated).
hipError_t launch_warmup_backward(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                                  const float* w, const float* g, int64_t ld_g, int B, int n_q, int n_kv, float* dq,
                                  float* dw, float* dk, hipStream_t stream);
// Sparse training backward (bf16, H = 128, d_qk = 576, d_v = 512, k <= 2048): dq [rows][128][576] and dkv
// [B][n_kv][576] fp32 (overwritten), pbar [rows][k] (optional); the workspace holds
// sbwd_workspace_bytes(...) bytes (P, dS, the dkv terms of one chunk of query rows, the per-key lists).
int sbwd_chunk_rows(int rows);
size_t sbwd_workspace_bytes(int B, int n_q, int n_kv, int k);
hipError_t launch_sparse_backward(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, int B, int n_q, int n_kv, int k,
                                  float sm_scale, float* dq, float* dkv, float* pbar, void* workspace,
                                  hipStream_t stream);
hipError_t launch_sparse_kl(float* scores, int64_t ld_s, const float* pbar, const int32_t* idx, int B, int n_q,
                            int n_kv, int k, float* loss, hipStream_t stream);
// Masked MHA mode (bf16, d_qk = 192, d_v = 128): mask words per query row, and the two launches
// (mask from the selection, then dense attention under it).  mask: [B][n_q][mha_mask_words(n_kv)] u32.
int mha_mask_words(int n_kv);
hipError_t launch_masked_mha(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx, int B,
                             int n_q, int n_kv, int H, int k_sel, float sm_scale, uint16_t* out, float* lse,
                             uint32_t* mask, hipStream_t stream);
size_t mla_bf16_workspace_bytes(int B, int n_q, int n_split);
int mla_bf16_pick_split(int B, int n_q, int k);
hipError_t launch_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int B, int n_q, int n_kv,
                           int k, float sm_scale, uint16_t* out, float* lse, int n_split, void* partial,
                           hipStream_t stream);

}  // namespace dsa
