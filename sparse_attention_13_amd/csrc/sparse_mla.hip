// sparse_mla.hip -- attention over the selected latent rows only, MLA in MQA mode (velog summary
// "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models", section 1.2: u_t = Attn over
// the entries whose index score is in the top-k; section 1.3: every latent KV entry is shared by all
// query heads).  K = the whole 576-wide latent row, V = its first 512 columns, explicit softmax scale.
//
// bf16 fast path (H = 128, d_qk = 576, d_v = 512), one workgroup of 4 waves per query (or per part
// of a query's selection when split), 32 selected rows per step:
//   gather   32 rows x 1152 B are copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//            for step i+1 while step i computes (two LDS buffers; rows padded to 1168 B);
//   QK       wave w owns heads 32w..32w+31: S^T[32 keys][32 heads] = K . Q^T on the 32x32x16 bf16
//            matrix core; K fragments are plain 16-B LDS reads, Q^T fragments stay in registers;
//   softmax  each lane owns one head and 16 keys of the step: online max/sum with a lazy rescale
//            (the running max moves only when it grows by more than 2^8), exp2 domain;
//   PV       wave w owns output columns d = 128w..128w+127 for all 128 heads:
//            O^T[d][h] += V^T[d][keys] . P^T[keys][h].  V^T fragments come straight from the
//            row-major tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16); P^T
//            fragments are exchanged through LDS in operand order.  The key order inside one
//            instruction is permuted identically on both operands so the softmax registers are
//            already in operand layout.
// The accumulator O^T keeps the head in the lane's column, the same lane that owns that head's
// softmax statistics, so rescaling and normalisation are lane-local.
#include "dsa_internal.h"

namespace dsa {

// ------------------------------------------------------------------------------------------------
// Generic fp32 kernel (any H, d_qk <= 256, d_v <= d_qk, k <= 16384): one workgroup per (query, head).
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    float o = __shfl_xor(v, off, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; i++) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__global__ __launch_bounds__(256) void attn_generic_kernel(const float* __restrict__ q, const float* __restrict__ kv,
                                                           const int32_t* __restrict__ idx, int n_q, int n_kv, int H,
                                                           int d_qk, int d_v, int k, float sm_scale,
                                                           float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float sm[];
  float* qs = sm;             // [d_qk]
  float* z = sm + d_qk;       // [k]
  float* red = z + k;         // [4]
  const int t = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const size_t row = (size_t)b * n_q + t;
  const float* qp = q + (row * H + h) * d_qk;
  const int32_t* sel = idx + row * k;
  const float* kvb = kv + (size_t)b * n_kv * d_qk;
  for (int e = threadIdx.x; e < d_qk; e += blockDim.x) qs[e] = qp[e];
  __syncthreads();
  float m = -INFINITY;
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    int s = sel[i];
    float zi = -INFINITY;
    if (s >= 0 && s < n_kv) {
      const float* c = kvb + (size_t)s * d_qk;
      float dot = 0.f;
      for (int e = 0; e < d_qk; e++) dot = fmaf(qs[e], c[e], dot);
      zi = dot * sm_scale;
    }
    z[i] = zi;
    m = fmaxf(m, zi);
  }
  m = block_reduce(m, red, true);
  const float m_use = (m == -INFINITY) ? 0.f : m;
  float l = 0.f;
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    float p = __expf(z[i] - m_use);
    z[i] = p;
    l += p;
  }
  l = block_reduce(l, red, false);  // the barrier inside also publishes z
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = out + (row * H + h) * d_v;
  for (int e = threadIdx.x; e < d_v; e += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < k; i++) {
      int s = sel[i];
      if (s >= 0 && s < n_kv) acc = fmaf(z[i], kvb[(size_t)s * d_qk + e], acc);
    }
    op[e] = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[row * H + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

hipError_t launch_attn_generic(const float* q, const float* kv, const int32_t* idx, int B, int n_q, int n_kv,
                               int H, int d_qk, int d_v, int k, float sm_scale, float* out, float* lse,
                               hipStream_t stream) {
  dim3 grid(n_q, B, H);
  size_t lds = (size_t)(d_qk + k + 4) * sizeof(float);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(256), lds, stream, q, kv, idx, n_q, n_kv, H, d_qk, d_v, k,
                     sm_scale, out, lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// bf16 matrix-core kernel.
// ------------------------------------------------------------------------------------------------
constexpr int kH = 128;
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kNB = 32;                        // selected rows per step
constexpr int kRowChunks = kDQK * 2 / 16;      // 72 chunks of 16 B per latent row
constexpr int kTileChunks = kRowChunks + 1;    // padded row: 73 chunks = 1168 B
constexpr int kTileRowBytes = kTileChunks * 16;
constexpr int kGatherPerWave = 10;             // wave-wide 1 KiB copies per wave and step
constexpr int kGatherInstr = 4 * kGatherPerWave;   // 40 >= 32 rows * 73 chunks / 64
constexpr int kBufBytes = kGatherInstr * 1024;     // 40960 B (the tail absorbs the last copies)
constexpr int kNBuf = 3;                           // steps in flight: the current one and two ahead
constexpr int kMaxSel = 2048;                      // selection entries handled by one workgroup
constexpr int kOffBuf = 0;
constexpr int kOffP = kNBuf * kBufBytes;            // [4 head blocks][2 k-steps][64 lanes][16 B]
constexpr int kOffSel = kOffP + 4 * 2 * 64 * 16;    // [kMaxSel] i32, the workgroup's selection
constexpr int kOffAlpha = kOffSel + kMaxSel * 4;    // [128] f32
constexpr int kOffRFlag = kOffAlpha + kH * 4;       // [4] u32 per-wave "rescaled" bits
constexpr int kOffL = kOffRFlag + 64;               // [128] f32
constexpr int kOffM = kOffL + kH * 4;               // [128] f32
constexpr int kOffMisc = kOffM + kH * 4;            // [16] i32
constexpr int kLdsBytes = kOffMisc + 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
static_assert(kGatherInstr * 64 >= kNB * kTileChunks, "gather covers the tile");
static_assert(kLdsBytes <= 163840, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bool valid_entry(int s, int n_kv) { return s >= 0 && s < n_kv; }

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait for this wave's LDS operations, then meet the other waves.  No vector-memory wait: copies
// into other LDS buffers stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy the 32 rows of one step into an LDS buffer: wave-wide copy c (c = wave + 4j) covers tile
// chunks 64c .. 64c+63 (row = chunk / 73, column = chunk % 73; column 72 is padding, chunks past the
// tile land in the buffer's tail).  Row indices come from the LDS copy of the selection (-1 =
// invalid, which copies row 0: its scores are masked).  Exactly kGatherPerWave copies per wave.
__device__ __forceinline__ void gather_step(const char* __restrict__ kvb, const int* sel_l, int e0, int e_n,
                                            char* buf, int wave, int lane) {
  int srow[kGatherPerWave];
#pragma unroll
  for (int j = 0; j < kGatherPerWave; j++) {  // all selection reads first (no wait between them)
    const int p = (wave + 4 * j) * 64 + lane;
    const int r = p / kTileChunks;
    const int e = max(0, min(e0 + min(r, kNB - 1), e_n - 1));  // in bounds; replaced below if unused
    srow[j] = sel_l[e];
  }
#pragma unroll
  for (int j = 0; j < kGatherPerWave; j++) {
    const int c = wave + 4 * j;
    const int p = c * 64 + lane;
    const int r = p / kTileChunks;
    int col = p - r * kTileChunks;
    const int s = (r < kNB && e0 + r < e_n && srow[j] >= 0) ? srow[j] : 0;
    col = col >= kRowChunks ? 0 : col;
    const char* src = kvb + (size_t)s * (kDQK * 2) + col * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(buf + c * 1024), 16, 0, 0);
  }
}

// Bit i set <=> selection entry e0 + i (i < 32) is a valid row.
__device__ __forceinline__ unsigned int step_valid_mask(const int* sel_l, int e0, int e_n, int lane) {
  bool v = (lane < kNB && e0 + lane < e_n) ? (sel_l[e0 + lane] >= 0) : false;
  return (unsigned int)(__ballot(v) & 0xFFFFFFFFull);
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
mla_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
                int n_q, int n_kv, int k, float sm_scale, int n_split, int per_split, uint16_t* __restrict__ out,
                float* __restrict__ lse, float* __restrict__ part, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % n_split;
  const int t = blockIdx.x / n_split;
  const int b = blockIdx.y;
  const size_t row = (size_t)b * n_q + t;
  const int32_t* sel = idx + row * k;
  const char* kvb = (const char*)(kv + (size_t)b * n_kv * kDQK);
  const int e_begin = split * per_split;
  const int e_n = max(0, min(k, e_begin + per_split) - e_begin);  // <= kMaxSel entries

  int* misc = (int*)(smem + kOffMisc);
  int* sel_l = (int*)(smem + kOffSel);
  float* alpha_l = (float*)(smem + kOffAlpha);
  unsigned int* rflag = (unsigned int*)(smem + kOffRFlag);

  // this workgroup's part of the selection -> LDS (invalid entries as -1), and its extent
  if (tid == 0) misc[0] = -1;
  __syncthreads();
  {
    int last = -1;
    for (int e = tid; e < e_n; e += 256) {
      const int v = sel[e_begin + e];
      const bool ok = valid_entry(v, n_kv);
      sel_l[e] = ok ? v : -1;
      if (ok) last = e;
    }
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
    if (lane == 0) atomicMax(&misc[0], last);
  }
  __syncthreads();
  const int n_span = misc[0] + 1;
  const int n_steps = (n_span + kNB - 1) / kNB;

  // Q^T fragments of this wave's 32 heads: lane holds head 32w + l%32, dims 16ks + 8(l/32) .. +8
  v8bf qf[kDQK / 16];
  {
    const uint16_t* qh = q + (row * kH + 32 * wave + (lane & 31)) * kDQK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kDQK / 16; ks++) qf[ks] = *(const v8bf*)(qh + 16 * ks);
  }

  v16f o[4][4];  // O^T blocks [d block][head block]
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) o[i][j][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c_scale = sm_scale * kLog2e;

  // prologue: steps 0 and 1 in flight (unconditionally: entries past the selection copy row 0),
  // then wait for the query fragments (loaded before the copies, so the copies stay in flight;
  // otherwise every step would wait for all copies) and for step 0
  gather_step(kvb, sel_l, 0, e_n, smem + kOffBuf, wave, lane);
  gather_step(kvb, sel_l, kNB, e_n, smem + kOffBuf + kBufBytes, wave, lane);
#pragma unroll
  for (int ks = 0; ks < kDQK / 16; ks++) asm volatile("" ::"v"(qf[ks]));
  wait_vmcnt<kGatherPerWave>();
  lds_barrier();

  int cur = 0;
  for (int it = 0; it < n_steps; it++) {
    char* buf = smem + kOffBuf + cur * kBufBytes;
    const int e0 = it * kNB;
    const bool ahead2 = it + 2 < n_steps;
    if (ahead2) {
      int nb = cur + 2;
      nb = nb >= kNBuf ? nb - kNBuf : nb;
      gather_step(kvb, sel_l, e0 + 2 * kNB, e_n, smem + kOffBuf + nb * kBufBytes, wave, lane);
    }
    const unsigned int vmask = step_valid_mask(sel_l, e0, e_n, lane);

    // ---- S^T = K . Q^T for this wave's heads (S kept in VGPRs: the AGPR file holds O)
    v16f sacc;
    {
      const char* kp = buf + (lane & 31) * kTileRowBytes + (lane >> 5) * 16;
      {
        v8bf kf = *(const v8bf*)(kp);
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(kf), "v"(qf[0]));
      }
#pragma unroll
      for (int ks = 1; ks < kDQK / 16; ks++) {
        v8bf kf = *(const v8bf*)(kp + ks * 32);
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(kf), "v"(qf[ks]));
      }
      asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sacc));
    }

    // ---- online softmax: this lane = head 32w + l%32; its 16 values are keys 8(r/4) + 4(l/32) + r%4
    float x[16];
    float bm = -INFINITY;
    const unsigned int vm = vmask >> (4 * (lane >> 5));
#pragma unroll
    for (int r = 0; r < 16; r++) {
      x[r] = ((vm >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[r] * c_scale : -INFINITY;
      bm = fmaxf(bm, x[r]);
    }
    bm = xor32_max(bm);
    float alpha = 1.f;
    if (bm > m_run + kRescaleThreshold) {
      alpha = __builtin_amdgcn_exp2f(m_run - bm);  // 0 when m_run = -inf
      m_run = bm;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
    unsigned int pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = __builtin_amdgcn_exp2f(x[r] - m_use), p1 = __builtin_amdgcn_exp2f(x[r + 1] - m_use);
      psum += p0 + p1;
      pk[r >> 1] = pack_bf16x2(p0, p1);
    }
    l_run = l_run * alpha + xor32_sum(psum);
    {
      u32x4* pl = (u32x4*)(smem + kOffP);
      pl[(wave * 2 + 0) * 64 + lane] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      pl[(wave * 2 + 1) * 64 + lane] = u32x4{pk[4], pk[5], pk[6], pk[7]};
      if (lane < 32) alpha_l[32 * wave + lane] = alpha;
      unsigned long long any = __ballot(alpha != 1.f);
      if (lane == 0) rflag[wave] = any ? 1u : 0u;
    }
    lds_barrier();

    // ---- rescale O^T where some head's running max moved (rare after the first step)
    if (rflag[0] | rflag[1] | rflag[2] | rflag[3]) {
#pragma unroll
      for (int hb = 0; hb < 4; hb++) {
        const float a = alpha_l[32 * hb + (lane & 31)];
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            // scale the accumulator in place in the AGPR file
            float tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(o[db][hb][r]), "=&v"(tmp) : "v"(a));
          }
      }
      asm volatile("s_nop 4" ::: "memory");
    }

    // ---- O^T[d][h] += V^T[d][keys] . P^T[keys][h]
    {
      const int G = lane >> 4, j = lane & 15;
      const u32x4* pl = (const u32x4*)(smem + kOffP);
      // V^T fragments of both 16-key halves: 16 transposing LDS reads issued together and waited for
      // inside the same asm block (the values are complete when the block ends)
      const unsigned int vbase =
          (unsigned int)(uintptr_t)(lds_void*)(buf + (4 * (G >> 1) + (j >> 2)) * kTileRowBytes +
                                               (128 * wave + 16 * (G & 1) + 4 * (j & 3)) * 2);
      u32x2 vr[2][4][2];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
          "ds_read_b64_tr_b16 %1, %16 offset:9344\n\t"
          "ds_read_b64_tr_b16 %2, %16 offset:64\n\t"
          "ds_read_b64_tr_b16 %3, %16 offset:9408\n\t"
          "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
          "ds_read_b64_tr_b16 %5, %16 offset:9472\n\t"
          "ds_read_b64_tr_b16 %6, %16 offset:192\n\t"
          "ds_read_b64_tr_b16 %7, %16 offset:9536\n\t"
          "ds_read_b64_tr_b16 %8, %16 offset:18688\n\t"
          "ds_read_b64_tr_b16 %9, %16 offset:28032\n\t"
          "ds_read_b64_tr_b16 %10, %16 offset:18752\n\t"
          "ds_read_b64_tr_b16 %11, %16 offset:28096\n\t"
          "ds_read_b64_tr_b16 %12, %16 offset:18816\n\t"
          "ds_read_b64_tr_b16 %13, %16 offset:28160\n\t"
          "ds_read_b64_tr_b16 %14, %16 offset:18880\n\t"
          "ds_read_b64_tr_b16 %15, %16 offset:28224\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(vr[0][0][0]), "=&v"(vr[0][0][1]), "=&v"(vr[0][1][0]), "=&v"(vr[0][1][1]), "=&v"(vr[0][2][0]),
            "=&v"(vr[0][2][1]), "=&v"(vr[0][3][0]), "=&v"(vr[0][3][1]), "=&v"(vr[1][0][0]), "=&v"(vr[1][0][1]),
            "=&v"(vr[1][1][0]), "=&v"(vr[1][1][1]), "=&v"(vr[1][2][0]), "=&v"(vr[1][2][1]), "=&v"(vr[1][3][0]),
            "=&v"(vr[1][3][1])
          : "v"(vbase));
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ks2++) {
        v8bf pf[4];
#pragma unroll
        for (int hb = 0; hb < 4; hb++) pf[hb] = __builtin_bit_cast(v8bf, pl[(hb * 2 + ks2) * 64 + lane]);
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const u32x4 v4 = {vr[ks2][db][0][0], vr[ks2][db][0][1], vr[ks2][db][1][0], vr[ks2][db][1][1]};
          const v8bf vf = __builtin_bit_cast(v8bf, v4);
#pragma unroll
          for (int hb = 0; hb < 4; hb++)
            o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[hb], o[db][hb], 0, 0, 0);
        }
      }
    }
    // step it+1's rows must have landed (step it+2's copies may stay in flight)
    if (ahead2)
      wait_vmcnt<kGatherPerWave>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    cur = cur + 1 == kNBuf ? 0 : cur + 1;
  }

  // ---- epilogue: publish per-head (m, l), normalise, store
  float* l_l = (float*)(smem + kOffL);
  float* m_l = (float*)(smem + kOffM);
  if (lane < 32) {
    l_l[32 * wave + lane] = l_run;
    m_l[32 * wave + lane] = m_run;
  }
  __syncthreads();
  if (n_split == 1) {
#pragma unroll
    for (int hb = 0; hb < 4; hb++) {
      const int h = 32 * hb + (lane & 31);
      const float lh = l_l[h];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      uint16_t* op = out + (row * kH + h) * kDV + 128 * wave + 4 * (lane >> 5);
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          u32x2 v;
          v[0] = pack_bf16x2(o[db][hb][4 * qd + 0] * inv, o[db][hb][4 * qd + 1] * inv);
          v[1] = pack_bf16x2(o[db][hb][4 * qd + 2] * inv, o[db][hb][4 * qd + 3] * inv);
          *(u32x2*)(op + 32 * db + 8 * qd) = v;
        }
    }
    if (lse && lane < 32) {
      const float lh = l_run;
      lse[row * kH + 32 * wave + lane] = lh > 0.f ? (m_run + log2f(lh)) * kLn2 : -INFINITY;
    }
  } else {
    // partial result of this split: normalised O (fp32) and its log-sum-exp
    float* pbase = part + ((row * n_split + split) * kH) * kDV;
#pragma unroll
    for (int hb = 0; hb < 4; hb++) {
      const int h = 32 * hb + (lane & 31);
      const float lh = l_l[h];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      float* op = pbase + (size_t)h * kDV + 128 * wave + 4 * (lane >> 5);
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          v4f v = {o[db][hb][4 * qd] * inv, o[db][hb][4 * qd + 1] * inv, o[db][hb][4 * qd + 2] * inv,
                   o[db][hb][4 * qd + 3] * inv};
          *(v4f*)(op + 32 * db + 8 * qd) = v;
        }
    }
    if (lane < 32) {
      const float lh = l_run;
      part_lse[(row * n_split + split) * kH + 32 * wave + lane] = lh > 0.f ? (m_run + log2f(lh)) * kLn2 : -INFINITY;
    }
  }
}

// Merge the n_split partial results of each (query, head): lse = log sum exp(lse_j),
// out = sum_j exp(lse_j - lse) * O_j.  One workgroup per query, 256 threads.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ part_lse, int n_split,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse) {
  const size_t row = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int lane = threadIdx.x & 63;
  for (int h = threadIdx.x >> 6; h < kH; h += 4) {
    float mx = -INFINITY;
    for (int j = 0; j < n_split; j++) mx = fmaxf(mx, part_lse[(row * n_split + j) * kH + h]);
    float wsum = 0.f;
    float acc[kDV / 64];
#pragma unroll
    for (int i = 0; i < kDV / 64; i++) acc[i] = 0.f;
    for (int j = 0; j < n_split; j++) {
      const float lj = part_lse[(row * n_split + j) * kH + h];
      if (lj == -INFINITY) continue;
      const float wj = __expf(lj - mx);
      wsum += wj;
      const float* pj = part + ((row * n_split + j) * kH + h) * kDV;
#pragma unroll
      for (int i = 0; i < kDV / 64; i++) acc[i] = fmaf(wj, pj[i * 64 + lane], acc[i]);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t* op = out + (row * kH + h) * kDV;
#pragma unroll
    for (int i = 0; i < kDV / 64; i++) op[i * 64 + lane] = f32_to_bf16_bits(acc[i] * inv);
    if (lse && lane == 0) lse[row * kH + h] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
  }
}

size_t mla_bf16_workspace_bytes(int B, int n_q, int n_split) {
  if (n_split <= 1) return 0;
  return (size_t)B * n_q * n_split * kH * (kDV + 1) * sizeof(float);  // O parts, then lse parts
}

int mla_bf16_pick_split(int B, int n_q, int k) {
  const long long rows = (long long)B * n_q;
  const int min_split = (k + kMaxSel - 1) / kMaxSel;  // one workgroup holds at most kMaxSel entries
  int split = 1;
  if (rows < 512) {
    // aim for >= 256 workgroups, each with at least 4 steps of 32 rows
    split = (int)((256 + rows - 1) / rows);
    const int max_split = (k + 4 * kNB - 1) / (4 * kNB);
    if (split > max_split) split = max_split;
  }
  return split < min_split ? min_split : (split < 1 ? 1 : split);
}

hipError_t launch_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int B, int n_q, int n_kv,
                           int k, float sm_scale, uint16_t* out, float* lse, int n_split, void* partial,
                           hipStream_t stream) {
  if (n_split < 1) n_split = 1;
  int per_split = (k + n_split - 1) / n_split;
  per_split = ((per_split + kNB - 1) / kNB) * kNB;
  dim3 grid(n_q * n_split, B);
  float* part = (float*)partial;
  float* part_lse = part ? part + (size_t)B * n_q * n_split * kH * kDV : nullptr;
  hipLaunchKernelGGL(mla_bf16_kernel, grid, dim3(256), 0, stream, q, kv, idx, n_q, n_kv, k, sm_scale, n_split,
                     per_split, out, lse, part, part_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(n_q, B), dim3(256), 0, stream, (const float*)part,
                     (const float*)part_lse, n_split, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
