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
// Step tile in LDS.  Region A: the 512 latent columns (1 KiB) of each row at a 1072-byte stride (the
// padding makes both the 16-byte K-fragment reads and the transposing V reads bank-conflict free).
// Region B: the 64 rope columns (128 B) of each row, 16-byte chunks XOR-swizzled by (row>>1)&7.
// One wave-wide 1 KiB copy brings a row's region A (lane l copies chunk l), four copies bring region B
// for 8 rows each: 36 copies per step, 9 per wave.
constexpr int kRowA = 1072;
constexpr int kTileA = kNB * kRowA;                  // 34304 B
constexpr int kTileBytes = kTileA + kNB * 128;       // 38400 B
constexpr int kGatherPerWave = 9;
constexpr int kNBuf = 3;                           // tiles: step i-1 (PV), step i (QK), step i+1 (landing)
constexpr int kMaxSel = 2048;                      // selection entries handled by one workgroup
constexpr int kPBytes = 4 * 2 * 64 * 16;           // P^T fragments of one step: [4 head blocks][2][64][16 B]
constexpr int kOffBuf = 0;
constexpr int kOffP = kNBuf * kTileBytes;           // two P buffers (step parity)
constexpr int kOffSel = kOffP + 2 * kPBytes;        // [kMaxSel] i32, the workgroup's selection
constexpr int kOffAlpha = kOffSel + kMaxSel * 4;    // [2][128] f32 rescale factors (step parity)
constexpr int kOffRFlag = kOffAlpha + 2 * kH * 4;   // [2][4] u32 per-wave "rescaled" bits
constexpr int kOffL = kOffRFlag + 64;               // [128] f32
constexpr int kOffM = kOffL + kH * 4;               // [128] f32
constexpr int kOffMisc = kOffM + kH * 4;            // [16] i32
constexpr int kLdsBytes = kOffMisc + 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
static_assert(kLdsBytes <= 163840, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bool valid_entry(int s, int n_kv) { return s >= 0 && s < n_kv; }

// Wait until no vector-memory operation of this wave is outstanding (expcnt and lgkmcnt untouched).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
// Wait for this wave's LDS operations, then meet the other waves.  No vector-memory wait is implied.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rows of one step copied by this wave: region A of rows w, w+4, ..., w+28 and region B of rows
// 8w .. 8w+7 (lane l: row 8w + l/8).  Entries past the selection or invalid (-1) copy row 0, whose
// scores are masked.  Row indices come from the LDS copy of the selection; lane i < 8 holds the
// region-A row of copy i (read back with readlane), every lane holds its region-B row.
struct GatherRows {
  int a;  // lanes 0..7: latent row of copy i
  int b;  // rope row of this lane
};
__device__ __forceinline__ GatherRows gather_rows(const int* sel_l, int e0, int e_n, int wave, int lane) {
  GatherRows g;
  {
    const int e = e0 + wave + 4 * (lane & 7);
    const int v = sel_l[max(0, min(e, e_n - 1))];
    g.a = (e < e_n && v >= 0) ? v : 0;
  }
  const int e = e0 + 8 * wave + (lane >> 3);
  const int v = sel_l[max(0, min(e, e_n - 1))];
  g.b = (e < e_n && v >= 0) ? v : 0;
  return g;
}
// Copy number j (0..8) of this wave into `tile`: j < 8 -> region A of row w + 4j (lane l: chunk l);
// j == 8 -> region B of rows 8w .. 8w+7 (stored chunk l%8 holds rope chunk (l%8) ^ ((row>>1)&7)).
__device__ __forceinline__ void gather_copy(const char* __restrict__ kvb, const GatherRows& g, int j, char* tile,
                                            int wave, int lane) {
  if (j < 8) {
    const int s = __builtin_amdgcn_readlane(g.a, j);
    const char* src = kvb + (size_t)s * (kDQK * 2) + lane * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(tile + (wave + 4 * j) * kRowA), 16, 0, 0);
  } else {
    const int rb = 8 * wave + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rb >> 1) & 7);
    const char* src = kvb + (size_t)g.b * (kDQK * 2) + 1024 + chunk * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(tile + kTileA + wave * 1024), 16, 0, 0);
  }
}

// Bit i set <=> selection entry e0 + i (i < 32) is a valid row.
__device__ __forceinline__ unsigned int step_valid_mask(const int* sel_l, int e0, int e_n, int lane) {
  bool v = (lane < kNB && e0 + lane < e_n) ? (sel_l[e0 + lane] >= 0) : false;
  return (unsigned int)(__ballot(v) & 0xFFFFFFFFull);
}

// V^T fragments of one 16-key half (ks2) of a step for this wave's 128 output columns: 8 transposing
// LDS reads issued together and completed inside the same asm block.  vr[db][0/1]: keys
// 16ks2 + (0..7 | 8..15 in the permuted key order), columns 128w + 32db + l%32.
// Offsets: +64 B per 32-column block, +8 rows (8576 B) for the second read of a fragment.
template <int KS2>
__device__ __forceinline__ void load_vfrags(const char* tile, int wave, int lane, u32x2 (&vr)[4][2]) {
  const int G = lane >> 4, j = lane & 15;
  const unsigned int vbase =
      (unsigned int)(uintptr_t)(lds_void*)(tile + (16 * KS2 + 4 * (G >> 1) + (j >> 2)) * kRowA +
                                           (128 * wave + 16 * (G & 1) + 4 * (j & 3)) * 2);
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:8576\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:8640\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:8704\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:8768\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vr[0][0]), "=&v"(vr[0][1]), "=&v"(vr[1][0]), "=&v"(vr[1][1]), "=&v"(vr[2][0]), "=&v"(vr[2][1]),
        "=&v"(vr[3][0]), "=&v"(vr[3][1])
      : "v"(vbase));
}

__device__ __forceinline__ v8bf vfrag(const u32x2 (&vr)[4][2], int db) {
  const u32x4 v4 = {vr[db][0][0], vr[db][0][1], vr[db][1][0], vr[db][1][1]};
  return __builtin_bit_cast(v8bf, v4);
}

// O^T *= alpha (per head column) in place in the AGPR file, when some head of the step rescaled.
__device__ __forceinline__ void rescale_o(v16f (&o)[4][4], const float* alpha_l, int lane) {
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    const float a = alpha_l[32 * hb + (lane & 31)];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(o[db][hb][r]), "=&v"(tmp)
                     : "v"(a));
      }
  }
  asm volatile("s_nop 4" ::: "memory");
}

struct PipeState {
  float m;  // running max (log2 units, scaled), per head of this lane
  float l;  // running sum of exp2(. - m)
};

// ---- steady-state step helpers ----------------------------------------------------------------------
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef short v8s __attribute__((ext_vector_type(8)));

// base + OFF in a register the compiler cannot fold or hoist: the transposing-read builtin takes no
// immediate offset, and hoisted per-read addresses would cost a register each.
template <int OFF>
__device__ __forceinline__ unsigned int lds_add(unsigned int base) {
  unsigned int a;
  asm("v_add_u32 %0, %1, %2" : "=v"(a) : "i"(OFF), "v"(base));
  return a;
}
// V^T fragment of d block DB (the two transposing reads of load_vfrags, through the builtin so the
// compiler places the waits).  `base` is the LDS byte address of the half's first read.
template <int DB>
__device__ __forceinline__ v8bf vread(unsigned int base) {
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(size_t)lds_add<64 * DB>(base));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(size_t)lds_add<8576 + 64 * DB>(base));
  const v8s c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(v8bf, c);
}
__device__ __forceinline__ v8bf vread_db(unsigned int base, int db) {
  switch (db) {
    case 0: return vread<0>(base);
    case 1: return vread<1>(base);
    case 2: return vread<2>(base);
    default: return vread<3>(base);
  }
}

// gather_copy for the steady state, the LDS-DMA load written in asm with an SGPR base and a 32-bit
// lane offset.  Two reasons: the compiler treats a visible LDS-DMA load as leaving every later LDS
// read of unknown completion order, so each of its LDS waits becomes a full drain (lgkmcnt(0)) until
// the next vmcnt wait; and the SGPR base needs no per-copy 64-bit vector address arithmetic.  The
// copy writes no register.  Its data is consumed only after this wave's vmcnt(0) and the step's
// barrier; hiding it from the compiler's vmcnt bookkeeping is safe because vector-memory loads
// complete in issue order and the only vmcnt wait in the loop is that full one.
__device__ __forceinline__ void gather_copy_steady(const char* __restrict__ kvb, const GatherRows& g, int j,
                                                   char* tile, int wave, int lane) {
  if (j < 8) {
    const int s = __builtin_amdgcn_readlane(g.a, j);
    const char* rowp = kvb + (size_t)s * (kDQK * 2);
    const unsigned int dst = (unsigned int)(uintptr_t)(lds_void*)(tile + (wave + 4 * j) * kRowA);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane * 16), "s"(rowp),
                 "s"(dst)
                 : "m0");
  } else {
    const int rb = 8 * wave + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rb >> 1) & 7);
    const unsigned int off = (unsigned int)g.b * (kDQK * 2) + 1024 + chunk * 16;  // < 2^32: n_kv <= 2^21
    const unsigned int dst = (unsigned int)(uintptr_t)(lds_void*)(tile + kTileA + wave * 1024);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(kvb), "s"(dst)
                 : "m0");
  }
}

// One pipeline iteration (see the kernel): QK of step `it` (if DO_QK) with the copies of step it+1,
// then PV of step it-1 (if DO_PV) interleaved with the softmax of step it, then one barrier.
template <bool DO_QK, bool DO_PV>
__device__ __forceinline__ bool pipeline_step(int it, int n_steps, int e_n, const char* __restrict__ kvb, char* smem,
                                              const int* sel_l, const v8bf (&qf)[kDQK / 16], v16f (&o)[4][4],
                                              PipeState& st, float c_scale, int wave, int lane) {
  const int cur = it % kNBuf;
  const int prv = (it + kNBuf - 1) % kNBuf;
  const int nxt = (it + 1) % kNBuf;
  char* tile = smem + kOffBuf + cur * kTileBytes;
  char* ptile = smem + kOffBuf + prv * kTileBytes;
  char* ntile = smem + kOffBuf + nxt * kTileBytes;
  const int e0 = it * kNB;
  // The copies for step it+1 are issued unconditionally: after the last step they fill a free tile
  // with row 0 (never read), which keeps the instruction stream free of branches.
  constexpr bool has_next = DO_QK;

  v16f sacc;
  unsigned int vmask = 0;
  GatherRows g;
  if (DO_QK) {
    g = gather_rows(sel_l, e0 + kNB, e_n, wave, lane);
    vmask = step_valid_mask(sel_l, e0, e_n, lane);
    // K fragments: 36 16-byte reads (32 from region A, 4 from the swizzled region B), kept 8 ahead
    // of the dependent chain of matrix-core instructions
    const char* kp = tile + (lane & 31) * kRowA + (lane >> 5) * 16;
    const int rr = lane & 31;
    const char* kb = tile + kTileA + rr * 128;
    const int sw = (rr >> 1) & 7;
    constexpr int kDepth = 8;
    v8bf kf[kDepth];
#pragma unroll
    for (int ks = 0; ks < kDepth; ks++) kf[ks] = *(const v8bf*)(kp + ks * 32);
#pragma unroll
    for (int ks = 0; ks < kDQK / 16; ks++) {
      if (ks == 0)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(kf[0]), "v"(qf[0]));
      else
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(kf[ks % kDepth]), "v"(qf[ks]));
      const int nk = ks + kDepth;
      if (nk < 32)
        kf[ks % kDepth] = *(const v8bf*)(kp + nk * 32);
      else if (nk < kDQK / 16)
        kf[ks % kDepth] = *(const v8bf*)(kb + (((2 * (nk - 32) + (lane >> 5)) ^ sw) << 4));
    }
    asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sacc));
  }

  // PV of step it-1 (the caller has already rescaled O if that step moved some head's max)
  const int pp = (it + 1) & 1;  // parity of step it-1
  u32x2 vr[4][2];
  if (DO_PV) load_vfrags<0>(ptile, wave, lane, vr);
  const u32x4* pl = (const u32x4*)(smem + kOffP + pp * kPBytes);

  // online softmax of step it: this lane = head 32w + l%32, its 16 values are keys 8(r/4) + 4(l/32) + r%4
  float x[16];
  float alpha = 1.f, neg_m = 0.f;
  if (DO_QK) {
    if (vmask == 0xFFFFFFFFu) {
#pragma unroll
      for (int r = 0; r < 16; r++) x[r] = sacc[r];
    } else {
      const unsigned int vm = vmask >> (4 * (lane >> 5));
#pragma unroll
      for (int r = 0; r < 16; r++) x[r] = ((vm >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[r] : -INFINITY;
    }
    float bm = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) bm = fmaxf(fmaxf(bm, x[r]), x[r + 1]);
    bm = fmaxf(bm, x[15]);
    bm = xor32_max(bm) * c_scale;
    if (bm > st.m + kRescaleThreshold) {
      alpha = __builtin_amdgcn_exp2f(st.m - bm);  // 0 when m = -inf
      st.m = bm;
    }
    neg_m = (st.m == -INFINITY) ? 0.f : -st.m;
  }
  float psum = 0.f;
  unsigned int pk[8];
  // P^T fragments of one 16-key half, one per head block: read once per half (they serve all four
  // output blocks), before the copies below, which the compiler must assume may write any LDS byte
  v8bf pf[4];
#pragma unroll
  for (int g8 = 0; g8 < 8; g8++) {
    if (DO_PV && (g8 & 3) == 0) {
#pragma unroll
      for (int hb = 0; hb < 4; hb++) pf[hb] = __builtin_bit_cast(v8bf, pl[(hb * 2 + (g8 >> 2)) * 64 + lane]);
    }
    if (has_next) gather_copy(kvb, g, g8, ntile, wave, lane);
    if (DO_PV) {
      const int db = g8 & 3;
      if (g8 == 4) load_vfrags<1>(ptile, wave, lane, vr);
      const v8bf vf = vfrag(vr, db);
#pragma unroll
      for (int hb = 0; hb < 4; hb++) o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[hb], o[db][hb], 0, 0, 0);
    }
    if (DO_QK) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(x[2 * g8], c_scale, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(x[2 * g8 + 1], c_scale, neg_m));
      psum += p0 + p1;
      pk[g8] = pack_bf16x2(p0, p1);
    }
  }
  if (has_next) gather_copy(kvb, g, 8, ntile, wave, lane);
  if (DO_QK) {
    st.l = st.l * alpha + xor32_sum(psum);
    const int pc = it & 1;
    u32x4* plw = (u32x4*)(smem + kOffP + pc * kPBytes);
    plw[(wave * 2 + 0) * 64 + lane] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    plw[(wave * 2 + 1) * 64 + lane] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    if (lane < 32) ((float*)(smem + kOffAlpha))[kH * pc + 32 * wave + lane] = alpha;
    const unsigned long long any = __ballot(alpha != 1.f);
    if (lane == 0) ((unsigned int*)(smem + kOffRFlag))[4 * pc + wave] = any ? 1u : 0u;
  }
  // step it+1's rows have landed (this wave's copies), then meet: every wave's copies landed, step
  // it's P^T is published and step it-1's tile is free
  wait_vmcnt0();
  lds_barrier();
  // did step it move the running max of some head (anywhere in the workgroup)?
  if (!DO_QK) return false;
  const unsigned int* rf = (const unsigned int*)(smem + kOffRFlag) + 4 * (it & 1);
  return (rf[0] | rf[1] | rf[2] | rf[3]) != 0u;
}

// Bookkeeping carried from one steady step to the next: the rows whose copies the step issues and the
// valid entries of the step's own rows, both read from the LDS selection a step ahead.
struct StepCtx {
  GatherRows g;        // rows of step it+1
  unsigned int vmask;  // bit i: entry 32 it + i is valid
};

// The steady-state iteration (both QK of step `it` and PV of step it-1), scheduled by hand: the source
// order is the issue order, fixed by scheduling barriers between units of one matrix-core op each.
//   QK (36 ops): K fragments read five ops ahead; the nine copies of step it+1 one per fourth op; during
//                the last twelve ops the P^T and V^T fragments of the PV's first half.
//   PV (32 ops): first half d block by d block, second half head block by head block; the softmax of
//                step it is spread over the first nineteen ops (max, rescale decision, then one
//                exponential per op), the second half's fragments are read as the first half frees
//                their registers, the next step's bookkeeping is read late and used later.
// Numerically the same operations as the edge steps (pipeline_step), except that the row sum adds the
// sixteen exponentials one by one.
__device__ __forceinline__ bool pipeline_step_steady(int it, int e_n, const char* __restrict__ kvb, char* smem,
                                                     const int* sel_l, const v8bf (&qf)[kDQK / 16], v16f (&o)[4][4],
                                                     PipeState& st, StepCtx& cx, float c_scale, int wave, int lane) {
  const int cur = it % kNBuf, prv = (it + kNBuf - 1) % kNBuf, nxt = (it + 1) % kNBuf;
  const char* tile = smem + kOffBuf + cur * kTileBytes;
  const char* ptile = smem + kOffBuf + prv * kTileBytes;
  char* ntile = smem + kOffBuf + nxt * kTileBytes;
  const int pp = (it + 1) & 1, pc = it & 1;
  const u32x4* pl = (const u32x4*)(smem + kOffP + pp * kPBytes);
  const int G = lane >> 4, jj = lane & 15;
  const unsigned int vb0 = (unsigned int)(uintptr_t)(lds_void*)ptile + (4 * (G >> 1) + (jj >> 2)) * kRowA +
                           (128 * wave + 16 * (G & 1) + 4 * (jj & 3)) * 2;
  const unsigned int vb1 = vb0 + 16 * kRowA;
  const GatherRows g = cx.g;
  const unsigned int vmask = cx.vmask;

  // ---- QK^T of step it
  const char* kp = tile + (lane & 31) * kRowA + (lane >> 5) * 16;
  const int rr = lane & 31;
  const char* kb = tile + kTileA + rr * 128;
  const int sw = (rr >> 1) & 7;
  constexpr int kDepth = 5;
  constexpr int kLead = 12;  // PV operands are read during the last kLead ops
  v8bf kf[kDepth];
#pragma unroll
  for (int ks = 0; ks < kDepth; ks++) kf[ks] = *(const v8bf*)(kp + ks * 32);
  v16f sacc;
  v8bf pf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < kDQK / 16; ks++) {
    if (ks == 0)
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(kf[0]), "v"(qf[0]));
    else
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(kf[ks % kDepth]), "v"(qf[ks]));
    const int nk = ks + kDepth;
    if (nk < 32)
      kf[ks % kDepth] = *(const v8bf*)(kp + nk * 32);
    else if (nk < kDQK / 16)
      kf[ks % kDepth] = *(const v8bf*)(kb + (((2 * (nk - 32) + (lane >> 5)) ^ sw) << 4));
    if ((ks & 3) == 1) gather_copy_steady(kvb, g, ks >> 2, ntile, wave, lane);
    const int lp = ks - (kDQK / 16 - kLead);
    if (lp >= 0 && lp < 4) pf[lp] = __builtin_bit_cast(v8bf, pl[(lp * 2) * 64 + lane]);
    if (lp >= 4 && lp < 8) vf[lp - 4] = vread_db(vb0, lp - 4);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- PV of step it-1 with the softmax of step it
  float alpha = 1.f, neg_m = 0.f, psum = 0.f, bm = 0.f, b01 = 0.f, pe = 0.f;
  unsigned int pk[8];
  int raw_a = 0, raw_b = 0, raw_v = 0;
#pragma unroll
  for (int u = 0; u < 32; u++) {
    const int db = u < 16 ? (u >> 2) : (u & 3);
    const int hb = u < 16 ? (u & 3) : ((u - 16) >> 2);
    o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pf[hb], o[db][hb], 0, 0, 0);
    if (u == 0) {
      asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sacc));  // the QK result is readable
      if (vmask != 0xFFFFFFFFu) {  // some entries of the step are invalid (rare): their scores -> -inf
        const unsigned int vm = vmask >> (4 * (lane >> 5));
#pragma unroll
        for (int r = 0; r < 16; r++) sacc[r] = ((vm >> (8 * (r >> 2) + (r & 3))) & 1u) ? sacc[r] : -INFINITY;
      }
      b01 = fmaxf(fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]),
                  fmaxf(fmaxf(sacc[3], sacc[4]), fmaxf(sacc[5], fmaxf(sacc[6], sacc[7]))));
    } else if (u == 1) {
      const float b23 = fmaxf(fmaxf(fmaxf(sacc[8], sacc[9]), sacc[10]),
                              fmaxf(fmaxf(sacc[11], sacc[12]), fmaxf(sacc[13], fmaxf(sacc[14], sacc[15]))));
      bm = xor32_max(fmaxf(b01, b23)) * c_scale;
    } else if (u == 2) {
      if (bm > st.m + kRescaleThreshold) {
        alpha = __builtin_amdgcn_exp2f(st.m - bm);  // 0 when m = -inf
        st.m = bm;
      }
      neg_m = (st.m == -INFINITY) ? 0.f : -st.m;
    } else if (u >= 3 && u < 19) {
      const int r = u - 3;
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c_scale, neg_m));
      psum += p;
      if (r & 1)
        pk[r >> 1] = pack_bf16x2(pe, p);
      else
        pe = p;
    }
    if (u < 16) {
      if ((u & 3) == 3 && u < 15) vf[db] = vread_db(vb1, db);  // second half, d block db
      if (u >= 12) pf[hb] = __builtin_bit_cast(v8bf, pl[(hb * 2 + 1) * 64 + lane]);  // second half, head block hb
      if (u == 15) vf[3] = vread<3>(vb1);
    }
    if (u == 19) {  // publish step it's P^T
      u32x4* plw = (u32x4*)(smem + kOffP + pc * kPBytes);
      plw[(wave * 2 + 0) * 64 + lane] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      plw[(wave * 2 + 1) * 64 + lane] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
    if (u == 20) {
      st.l = st.l * alpha + xor32_sum(psum);
      // lanes l and l+32 hold the same head and store the same factor; every lane stores the same flag
      ((float*)(smem + kOffAlpha))[kH * pc + 32 * wave + (lane & 31)] = alpha;
      const unsigned long long any = __ballot(alpha != 1.f);
      ((unsigned int*)(smem + kOffRFlag))[4 * pc + wave] = any ? 1u : 0u;
    }
    if (u == 21) {  // next step's bookkeeping: raw entries now, decisions at u = 29
      const int e2 = (it + 2) * kNB, e1 = (it + 1) * kNB;
      raw_a = sel_l[max(0, min(e2 + wave + 4 * (lane & 7), e_n - 1))];
      raw_b = sel_l[max(0, min(e2 + 8 * wave + (lane >> 3), e_n - 1))];
      raw_v = sel_l[max(0, min(e1 + lane, e_n - 1))];
    }
    if (u == 29) {
      const int e2 = (it + 2) * kNB, e1 = (it + 1) * kNB;
      const int ea = e2 + wave + 4 * (lane & 7), eb = e2 + 8 * wave + (lane >> 3);
      cx.g.a = (ea < e_n && raw_a >= 0) ? raw_a : 0;
      cx.g.b = (eb < e_n && raw_b >= 0) ? raw_b : 0;
      cx.vmask = (unsigned int)(__ballot(lane < kNB && e1 + lane < e_n && raw_v >= 0) & 0xFFFFFFFFull);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // step it+1's rows have landed (this wave's copies), then meet: every wave's copies landed, step it's
  // P^T is published and step it-1's tile is free
  wait_vmcnt0();
  lds_barrier();
  const unsigned int* rf = (const unsigned int*)(smem + kOffRFlag) + 4 * pc;
  return (rf[0] | rf[1] | rf[2] | rf[3]) != 0u;
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
mla_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
                int n_q, int n_kv, int k, float sm_scale, int n_split, int per_split, uint16_t* __restrict__ out,
                float* __restrict__ lse, uint16_t* __restrict__ part, float* __restrict__ part_lse) {
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

  // this workgroup's part of the selection -> LDS (invalid entries as -1), and its extent.  The
  // selection's loads go first (all of a thread's at once, e_n <= kMaxSel = 8 x 256), then the Q
  // fragments': loads complete in issue order, so the selection, which the first copies wait for,
  // does not wait behind the 147 KB of Q.
  if (tid == 0) misc[0] = -1;
  int v[kMaxSel / 256];
#pragma unroll
  for (int u = 0; u < kMaxSel / 256; u++) {
    const int e = tid + 256 * u;
    v[u] = sel[min(e_begin + min(e, max(e_n - 1, 0)), k - 1)];  // clamped into the row; past e_n unused
  }
  // Q^T fragments of this wave's 32 heads: lane holds head 32w + l%32, dims 16ks + 8(l/32) .. +8.
  v8bf qf[kDQK / 16];
  {
    const uint16_t* qh = q + (row * kH + 32 * wave + (lane & 31)) * kDQK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kDQK / 16; ks++) qf[ks] = *(const v8bf*)(qh + 16 * ks);
  }
  __syncthreads();
  {
    int last = -1;
#pragma unroll
    for (int u = 0; u < kMaxSel / 256; u++) {
      const int e = tid + 256 * u;
      const bool ok = e < e_n && valid_entry(v[u], n_kv);
      if (e < e_n) sel_l[e] = ok ? v[u] : -1;
      if (ok) last = e;
    }
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
    if (lane == 0) atomicMax(&misc[0], last);
  }
  __syncthreads();
  const int n_span = misc[0] + 1;
  const int n_steps = (n_span + kNB - 1) / kNB;

  v16f o[4][4];  // O^T blocks [d block][head block]
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) o[i][j][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c_scale = sm_scale * kLog2e;

  // prologue: step 0's rows, then wait for them and for the query fragments
  {
    const GatherRows g0 = gather_rows(sel_l, 0, e_n, wave, lane);
#pragma unroll
    for (int j = 0; j < kGatherPerWave; j++) gather_copy(kvb, g0, j, smem + kOffBuf, wave, lane);
  }
  wait_vmcnt0();
  lds_barrier();

  // Software pipeline.  Iteration `it`: the copies of step it+1 are issued between the QK^T
  // instructions of step it; then PV of step it-1 (matrix cores) runs interleaved with the softmax of
  // step it (VALU); then step it's P^T is published and the waves meet once.
  // The rescale of O (rare once the running max has settled) happens outside the inner loop, so the
  // loop itself only ever touches O through the matrix cores.  Step 0 needs none: O is still zero.
  PipeState st{m_run, l_run};
  if (n_steps > 0) {
    pipeline_step<true, false>(0, n_steps, e_n, kvb, smem, sel_l, qf, o, st, c_scale, wave, lane);
    int it = 1;
    StepCtx cx;
    cx.g = gather_rows(sel_l, 2 * kNB, e_n, wave, lane);
    cx.vmask = step_valid_mask(sel_l, kNB, e_n, lane);
    while (it < n_steps) {
      bool moved = false;
      for (; it < n_steps && !moved; it++)
        moved = pipeline_step_steady(it, e_n, kvb, smem, sel_l, qf, o, st, cx, c_scale, wave, lane);
      if (moved) rescale_o(o, (const float*)(smem + kOffAlpha) + kH * ((it - 1) & 1), lane);
    }
    pipeline_step<false, true>(n_steps, n_steps, e_n, kvb, smem, sel_l, qf, o, st, c_scale, wave, lane);
  }
  m_run = st.m;
  l_run = st.l;

  // ---- epilogue: publish per-head (m, l), normalise, store
  // The lane index again, from a fresh computation: carrying the early one through the loop made the
  // compiler spill two lane-derived addresses to scratch.
  const int le = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  float* l_l = (float*)(smem + kOffL);
  float* m_l = (float*)(smem + kOffM);
  if (le < 32) {
    l_l[32 * wave + le] = l_run;
    m_l[32 * wave + le] = m_run;
  }
  __syncthreads();
  // O goes out through LDS (the tiles are free after the last step): 64 heads at a time are written as
  // bf16 rows of 1040 B, then every wave stores 16 whole 1 KiB head rows, 16 bytes per lane, instead of
  // 8-byte pieces spread over 32 rows per instruction.  A split part writes its normalised partial O (bf16)
  // and its log-sum-exp to the partial buffers, the merge kernel combines them.
  uint16_t* obase = n_split == 1 ? out + row * kH * kDV : part + ((row * n_split + split) * kH) * kDV;
  char* stg = smem + kOffBuf;
  constexpr int kStgRow = 1040;
  static_assert(64 * kStgRow <= kNBuf * kTileBytes, "staging fits in the tiles");
#pragma unroll
  for (int pass = 0; pass < 2; pass++) {
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      const int hb = 2 * pass + hh;
      const float lh = l_l[32 * hb + (le & 31)];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      char* rowp = stg + (32 * hh + (le & 31)) * kStgRow + (128 * wave + 4 * (le >> 5)) * 2;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          u32x2 v;
          v[0] = pack_bf16x2(o[db][hb][4 * qd + 0] * inv, o[db][hb][4 * qd + 1] * inv);
          v[1] = pack_bf16x2(o[db][hb][4 * qd + 2] * inv, o[db][hb][4 * qd + 3] * inv);
          *(u32x2*)(rowp + (32 * db + 8 * qd) * 2) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int hl = 16 * wave + r;
      const u32x4 v = *(const u32x4*)(stg + hl * kStgRow + le * 16);
      *(u32x4*)(obase + (64 * pass + hl) * kDV + 8 * le) = v;
    }
    __syncthreads();
  }
  if (le < 32) {
    const float lh = l_run;
    const float lv = lh > 0.f ? (m_run + log2f(lh)) * kLn2 : -INFINITY;
    if (n_split == 1) {
      if (lse) lse[row * kH + 32 * wave + le] = lv;
    } else {
      part_lse[(row * n_split + split) * kH + 32 * wave + le] = lv;
    }
  }
}

// Merge the n_split partial results of each (query, head): lse = log sum exp(lse_j),
// out = sum_j exp(lse_j - lse) * O_j.  One wave per (query, head), 4 heads per workgroup; lane l holds
// output columns 8l..8l+7 (one 16-byte load of bf16 partial per part), accumulated in fp32.  The parts
// go in groups of kCombineGroup whose loads are all issued before any is used (part indexes clamped
// into range, weights of the extra slots zero): one memory round trip per group instead of one per part.
constexpr int kCombineGroup = 8;
__global__ __launch_bounds__(256) void mla_combine_kernel(const uint16_t* __restrict__ part,
                                                          const float* __restrict__ part_lse, int n_split,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.y * (gridDim.x / (kH / 4)) + blockIdx.x / (kH / 4);
  const int h = (blockIdx.x % (kH / 4)) * 4 + wave;
  const float* pl = part_lse + row * n_split * kH + h;
  float wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float mx = -INFINITY;
  if (n_split <= kCombineGroup) {
    // the usual case (decode: 4 parts): every load of the row in one round trip
    float l[kCombineGroup];
    u32x4 x[kCombineGroup];
#pragma unroll
    for (int j = 0; j < kCombineGroup; j++) {
      const int jc = min(j, n_split - 1);
      l[j] = pl[(size_t)jc * kH];
      x[j] = *reinterpret_cast<const u32x4*>(part + ((row * n_split + jc) * kH + h) * kDV + 8 * lane);
    }
#pragma unroll
    for (int j = 0; j < kCombineGroup; j++) mx = fmaxf(mx, l[j]);
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kCombineGroup; j++) {
        const float wj = (j < n_split && l[j] != -INFINITY) ? __expf(l[j] - mx) : 0.f;
        wsum += wj;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          acc[2 * q] += wj * __uint_as_float(x[j][q] << 16);
          acc[2 * q + 1] += wj * __uint_as_float(x[j][q] & 0xFFFF0000u);
        }
      }
    }
  } else {
    // more parts: the maximum first, then the weighted sum, a group of loads at a time
    for (int j0 = 0; j0 < n_split; j0 += kCombineGroup) {
      float l[kCombineGroup];
#pragma unroll
      for (int j = 0; j < kCombineGroup; j++) l[j] = pl[(size_t)min(j0 + j, n_split - 1) * kH];
#pragma unroll
      for (int j = 0; j < kCombineGroup; j++) mx = fmaxf(mx, l[j]);  // clamped slots repeat a real part
    }
    if (mx != -INFINITY) {
      for (int j0 = 0; j0 < n_split; j0 += kCombineGroup) {
        float l[kCombineGroup];
        u32x4 x[kCombineGroup];
#pragma unroll
        for (int j = 0; j < kCombineGroup; j++) {
          const int jc = min(j0 + j, n_split - 1);
          l[j] = pl[(size_t)jc * kH];
          x[j] = *reinterpret_cast<const u32x4*>(part + ((row * n_split + jc) * kH + h) * kDV + 8 * lane);
        }
#pragma unroll
        for (int j = 0; j < kCombineGroup; j++) {
          // a part without valid entries (lse = -inf) and the clamped slots contribute nothing
          const float wj = (j0 + j < n_split && l[j] != -INFINITY) ? __expf(l[j] - mx) : 0.f;
          wsum += wj;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            acc[2 * q] += wj * __uint_as_float(x[j][q] << 16);
            acc[2 * q + 1] += wj * __uint_as_float(x[j][q] & 0xFFFF0000u);
          }
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const u32x4 o = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(out + (row * kH + h) * kDV + 8 * lane) = o;
  if (lse && lane == 0) lse[row * kH + h] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

// Split-k partials: normalised O of every part (bf16), then the parts' log-sum-exp (fp32), each region
// 256-byte aligned.
size_t mla_partial_o_bytes(int B, int n_q, int n_split) {
  return (((size_t)B * n_q * n_split * kH * kDV * sizeof(uint16_t)) + 255) / 256 * 256;
}

size_t mla_bf16_workspace_bytes(int B, int n_q, int n_split) {
  if (n_split <= 1) return 0;
  return mla_partial_o_bytes(B, n_q, n_split) + (((size_t)B * n_q * n_split * kH * sizeof(float)) + 255) / 256 * 256;
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
  uint16_t* part = (uint16_t*)partial;
  float* part_lse = part ? (float*)((char*)partial + mla_partial_o_bytes(B, n_q, n_split)) : nullptr;
  hipLaunchKernelGGL(mla_bf16_kernel, grid, dim3(256), 0, stream, q, kv, idx, n_q, n_kv, k, sm_scale, n_split,
                     per_split, out, lse, part, part_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(n_q * (kH / 4), B), dim3(256), 0, stream, (const uint16_t*)part,
                     (const float*)part_lse, n_split, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
