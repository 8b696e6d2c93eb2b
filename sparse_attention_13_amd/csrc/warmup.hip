// warmup.hip -- the indexer's dense warm-up loss (velog summary "DeepSeek-V3.2: Pushing the Frontier of
// Open Large Language Models", Continued Pre-Training, Stage 1: the main model is frozen, the indexer
// learns to reproduce the main attention; its target is the main attention summed over heads and
// L1-normalised, its loss the KL divergence from that target to the softmax of the index scores).
//
//   warmup_target_kernel  p[t][s] = (1/H) sum_h exp(sm_scale q[t][h] . kv[s] - lse[t][h]) for s <= pos_t,
//                         the head mean of the main (dense, causal, MQA-mode) attention; lse is that
//                         attention's log-sum-exp per (query, head).  One workgroup of 4 waves per query;
//                         wave w owns heads 32w..32w+31 and computes S[heads][keys] = Q . K^T on the
//                         32x32x16 bf16 matrix core (Q in registers, 32 consecutive latent rows per step
//                         copied into LDS), so that each lane holds 16 heads of one key: the head sum is
//                         lane-local plus one swap, then one LDS exchange across the waves.
//   warmup_loss_kernel    per query row: lse_I of the index scores, loss_t = sum_s p (log p - log softmax(I)),
//                         g = softmax(I) - p written over the scores.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kWD = 576;                 // d_qk of the main attention
constexpr int kWH = 128;                 // heads of the main attention
constexpr int kWRow = kWD * 2;           // 1152-byte latent row
constexpr int kWChunks = kWRow / 16;     // 72 chunks of 16 bytes
constexpr int kWTile = 32 * kWRow;       // 36864 B: 32 rows, contiguous, chunks swizzled by (row >> 1) & 7
constexpr int kWCopies = 32 * kWChunks / 64 / 4;  // 9 copies of 1 KiB per wave
constexpr float kLog2eW = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void_w;

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rows s0 .. s0+31 of the latent cache into a tile: copy i of wave w fills slots (9w + i) * 64 + lane =
// (row, chunk'), fetching global chunk chunk' ^ ((row >> 1) & 7) (rows past the last key re-read it).
__device__ __forceinline__ void copy_rows(const char* __restrict__ kvb, int s0, int n_kv, char* tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kWCopies; i++) {
    const int slot = (kWCopies * wave + i) * 64 + lane;
    const int r = slot / kWChunks, cs = slot % kWChunks;
    const int c = cs ^ ((r >> 1) & 7);
    const int s = min(s0 + r, n_kv - 1);
    __builtin_amdgcn_global_load_lds((const void*)(kvb + (size_t)s * kWRow + 16 * c),
                                     (lds_void_w*)(tile + (kWCopies * wave + i) * 1024), 16, 0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void warmup_target_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const float* __restrict__ lse, int n_q, int n_kv,
                                                               float sm_scale, float* __restrict__ p, int64_t ld) {
  __shared__ __attribute__((aligned(1024))) char tile0[kWTile];
  __shared__ __attribute__((aligned(1024))) char tile1[kWTile];
  __shared__ float part[2][4][32];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = n_q - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const size_t row = (size_t)b * n_q + t;
  const int pos = n_kv - n_q + t;
  const int n_steps = (pos + 32) / 32;
  const char* kvb = (const char*)(kv + (size_t)b * n_kv * kWD);

  // Q fragments (A operand): lane holds head 32w + l%32, dims 16ks + 8(l/32) .. +8
  v8bf qf[kWD / 16];
  {
    const uint16_t* qh = q + (row * kWH + 32 * wave + (lane & 31)) * kWD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kWD / 16; ks++) qf[ks] = *(const v8bf*)(qh + 16 * ks);
  }
  // lse (log2 units) of the heads this lane's accumulator rows hold: 32w + 8(r/4) + 4(l/32) + r%4
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; r++)
    lse2[r] = lse[row * kWH + 32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] * kLog2eW;
  const float c_scale = sm_scale * kLog2eW;
  // K fragment (B operand) of k-step ks: row l%32, logical chunk 2ks + l/32, swizzled
  const int kr = lane & 31;
  auto kfrag = [&](const char* tile, int ks) -> v8bf {
    const int c = 2 * ks + (lane >> 5);
    return *(const v8bf*)(tile + kr * kWRow + 16 * (c ^ ((kr >> 1) & 7)));
  };

  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // query side complete before any tile copy
  copy_rows(kvb, 0, n_kv, tile0, wave, lane);
  wait_vm();
  bar();
  auto step = [&](int i, const char* tile, char* next) {
    copy_rows(kvb, 32 * (i + 1), n_kv, next, wave, lane);  // past the row: re-reads in-bounds rows, unused
    v16f sacc;
#pragma unroll
    for (int ks = 0; ks < kWD / 16; ks++) {
      const v8bf kf = kfrag(tile, ks);
      if (ks == 0)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0], kf, (v16f){}, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, sacc, 0, 0, 0);
    }
    // lane: key 32i + l%32, heads 8(r/4) + 4(l/32) + r%4 of the wave's 32
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) sum += __builtin_amdgcn_exp2f(fmaf(sacc[r], c_scale, -lse2[r]));
    sum = xor32_sum(sum);
    if (lane < 32) part[i & 1][wave][lane] = sum;
    wait_vm();
    bar();
    if (wave == 0 && lane < 32) {
      const int s = 32 * i + lane;
      const float v = (part[i & 1][0][lane] + part[i & 1][1][lane] + part[i & 1][2][lane] + part[i & 1][3][lane]) *
                      (1.0f / kWH);
      if (s <= pos) p[row * ld + s] = v;
    }
  };
  for (int i = 0; i < n_steps; i += 2) {
    step(i, tile0, tile1);
    if (i + 1 < n_steps) step(i + 1, tile1, tile0);
  }
}

// One workgroup per query row: the row's scores -> loss and g (over the scores, in place).
__global__ __launch_bounds__(256) void warmup_loss_kernel(float* __restrict__ scores, int64_t ld_s,
                                                          const float* __restrict__ p, int64_t ld_p, int n_q,
                                                          int n_kv, float* __restrict__ loss) {
  __shared__ float red[8];
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * n_q + t;
  const int n = n_kv - n_q + t + 1;
  float* ir = scores + row * ld_s;
  const float* pr = p + row * ld_p;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto block_reduce = [&](float v, bool is_max) {
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off, 64);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < 4; i++) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
  };
  float m = -INFINITY;
  for (int s = threadIdx.x; s < n; s += 256) m = fmaxf(m, ir[s]);
  m = block_reduce(m, true);
  float l = 0.f;
  for (int s = threadIdx.x; s < n; s += 256) l += __expf(ir[s] - m);
  l = block_reduce(l, false);
  const float lse_i = m + __logf(l);
  float kl = 0.f;
  for (int s = threadIdx.x; s < n; s += 256) {
    const float logq = ir[s] - lse_i;
    const float ps = pr[s];
    if (ps > 0.f) kl += ps * (__logf(ps) - logq);
    ir[s] = __expf(logq) - ps;
  }
  kl = block_reduce(kl, false);
  if (threadIdx.x == 0) loss[row] = kl;
}

}  // namespace

hipError_t launch_warmup_forward(const uint16_t* q, const uint16_t* kv, const float* lse, int B, int n_q, int n_kv,
                                 float sm_scale, float* scores, int64_t ld_s, float* p, int64_t ld_p, float* loss,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(warmup_target_kernel, dim3(n_q, B), dim3(256), 0, stream, q, kv, lse, n_q, n_kv, sm_scale, p,
                     ld_p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(warmup_loss_kernel, dim3(n_q, B), dim3(256), 0, stream, scores, ld_s, (const float*)p, ld_p, n_q,
                     n_kv, loss);
  return hipGetLastError();
}

}  // namespace dsa
