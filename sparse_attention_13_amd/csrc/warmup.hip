// warmup.hip -- the indexer's dense warm-up loss (velog summary "DeepSeek-V3.2: Pushing the Frontier of
// Open Large Language Models", Continued Pre-Training, Stage 1: the main model is frozen, the indexer
// learns to reproduce the main attention; its target is the main attention summed over heads and
// L1-normalised, its loss the KL divergence from that target to the softmax of the index scores).
//
//   warmup_target_kernel  p[t][s] = (1/H) sum_h exp(sm_scale q[t][h] . kv[s] - lse[t][h]) for s <= pos_t,
//                         the head mean of the main (dense, causal, MQA-mode) attention; lse is that
//                         attention's log-sum-exp per (query, head).  One workgroup of 8 waves per pair of
//                         queries; wave w owns heads 32(w%4).. of query w/4 and computes S[heads][keys] =
//                         Q . K^T on the 32x32x16 bf16 matrix core (Q in registers).  Steps of 64 latent rows
//                         (two 32-row tiles, 36 KiB each) are copied into LDS one step ahead (four buffers,
//                         one barrier per step), shared by both queries.  Each lane holds 16 heads of one
//                         key: the head sum is lane-local plus one swap, then one LDS exchange across the
//                         waves; the target row is written one step late, after the next copies are issued,
//                         so the wait for a tile never waits for a store.
//   warmup_loss_kernel    per query row: lse_I of the index scores, loss_t = sum_s p (log p - log softmax(I)),
//                         g = softmax(I) - p written over the scores.
//   warmup_dq_kernel      gradients of the loss through I = sum_j w_j ReLU(q^_j . k^_s) for 4 queries per
//                         workgroup (8 waves: one query and 32 heads each): dw[t][j] = sum_s g ReLU(d),
//                         dq^[t][j] = w_j sum_s g [d > 0] k^_s.  The key codes of a 64-key block are converted
//                         to bf16 (exact for e4m3) into LDS (two buffers, one barrier per block); D^T = K . Q^T
//                         on the bf16 matrix core gives each lane one head and 16 keys, the ReLU decision and
//                         g k_scale make M^T in registers, in the key order the second product takes (as P^T in
//                         attention), and dq^T += K^T . M^T reads K^T through the transposing LDS read.
//   warmup_dk_kernel      dk^[s] = sum_t sum_j g w_j [d > 0] q^_j: the same two products with the roles of
//                         queries and keys exchanged (256 keys per workgroup of 8 waves, the key codes in
//                         registers, one bf16 query tile per barrier).  The queries that see a key block are cut
//                         into parts of equal size, one workgroup each, so that the causal triangle spreads
//                         evenly; parts are summed with atomics into dk, which a fill kernel zeroes first.
// The ReLU decisions use d = q^ . k^ = q_scale k_scale (codes . codes), so the codes' dot product decides.
#include <algorithm>

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
// The lane's slot arithmetic is redone at every call (kept from being hoisted out of the key loop, where
// it would hold registers across the matrix products); n_kv * 1152 fits 32 bits.
__device__ __forceinline__ void copy_rows(const char* __restrict__ kvb, int s0, int n_kv, char* tile, int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int i = 0; i < kWCopies; i++) {
    const int slot = (kWCopies * wave + i) * 64 + l;
    const int r = slot / kWChunks, cs = slot - kWChunks * r;
    const int c = cs ^ ((r >> 1) & 7);
    const unsigned int off = (unsigned int)min(s0 + r, n_kv - 1) * kWRow + 16u * c;
    __builtin_amdgcn_global_load_lds((const void*)(kvb + off), (lds_void_w*)(tile + (kWCopies * wave + i) * 1024), 16,
                                     0, 0);
  }
}

// Wait until at most one vector memory operation of this wave is outstanding (n = 1) or none (n = 0); they
// complete in issue order.
__device__ __forceinline__ void wait_vm_n(int n) {
  if (n == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
  else __builtin_amdgcn_s_waitcnt(0x0F71);
}

__global__ __launch_bounds__(512, 1) void warmup_target_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const float* __restrict__ lse, int n_q, int n_kv,
                                                               float sm_scale, float* __restrict__ p, int64_t ld) {
  __shared__ __attribute__((aligned(1024))) char tile0[kWTile];
  __shared__ __attribute__((aligned(1024))) char tile1[kWTile];
  __shared__ __attribute__((aligned(1024))) char tile2[kWTile];
  __shared__ __attribute__((aligned(1024))) char tile3[kWTile];
  __shared__ float part[2][8][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qsel = wave >> 2, hw = wave & 3;  // query of the pair, block of 32 heads
  const int t_a = n_q - 1 - 2 * (int)blockIdx.x;  // longest rows first; the pair is (t_a, t_a - 1)
  const int t = t_a - qsel;
  const bool live = t >= 0;
  const int b = blockIdx.y;
  const size_t row = (size_t)b * n_q + max(t, 0);
  const int pos = n_kv - n_q + t;
  const int n_steps = (n_kv - n_q + t_a + 64) / 64;  // steps of 64 keys
  const char* kvb = (const char*)(kv + (size_t)b * n_kv * kWD);
  const bool copier = wave < 4;          // waves 0..3 copy the tiles
  const bool writer = hw == 0 && live;   // waves 0 and 4 write their query's target row
  // target row of this wave's query as a buffer: stores past the query's position are dropped
  const __amdgpu_buffer_rsrc_t prow =
      __builtin_amdgcn_make_buffer_rsrc(p + row * ld, 0, live ? (pos + 1) * 4 : 0, 0x00020000);

  // Q fragments (A operand): lane holds head 32hw + l%32, dims 16ks + 8(l/32) .. +8
  v8bf qf[kWD / 16];
  {
    const uint16_t* qh = q + (row * kWH + 32 * hw + (lane & 31)) * kWD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kWD / 16; ks++) qf[ks] = *(const v8bf*)(qh + 16 * ks);
  }
  // lse (log2 units) of the heads this lane's accumulator rows hold: 32hw + 8(r/4) + 4(l/32) + r%4
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; r++)
    lse2[r] = lse[row * kWH + 32 * hw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] * kLog2eW;
  const float c_scale = sm_scale * kLog2eW;
  // K fragment (B operand) of k-step ks = 4m + j: row l%32, logical chunk 2ks + l/32 = 8m + (2j + l/32),
  // stored at 8m + ((2j + l/32) ^ ((row >> 1) & 7)): four lane offsets, the rest immediate
  int kb[4];
  {
    const int kr = lane & 31;
#pragma unroll
    for (int j = 0; j < 4; j++) kb[j] = kr * kWRow + 16 * ((2 * j + (lane >> 5)) ^ ((kr >> 1) & 7));
  }
  auto kfrag = [&](const char* tile, int ks) -> v8bf {
    return *(const v8bf*)(tile + kb[ks & 3] + 128 * (ks >> 2));
  };
  // the target of the 32 keys of step i from the four waves' partial sums (writer waves, lanes < 32)
  auto store_target = [&](int i) {
    if (writer) {
      const float* pp = &part[i & 1][4 * qsel][lane];
      const float v = (pp[0] + pp[64] + pp[128] + pp[192]) * (1.0f / kWH);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), prow, (64 * i + lane) * 4, 0, 0);
    }
  };

  wait_vm();  // query side complete before any tile copy
  if (copier) {
    copy_rows(kvb, 0, n_kv, tile0, wave, lane);
    copy_rows(kvb, 32, n_kv, tile1, wave, lane);
  }
  wait_vm();
  bar();
  auto half = [&](int i, int u, const char* tile) {
    v16f sacc;
#pragma unroll
    for (int ks = 0; ks < kWD / 16; ks++) {
      const v8bf kf = kfrag(tile, ks);
      if (ks == 0)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0], kf, (v16f){}, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, sacc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < kWD / 16 - 4; ks++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) sum += __builtin_amdgcn_exp2f(fmaf(sacc[r], c_scale, -lse2[r]));
    sum = xor32_sum(sum);
    if (lane < 32) part[i & 1][wave][32 * u + lane] = sum;
  };
  auto step = [&](int i, const char* ta, const char* tb, char* na, char* nb) {
    if (copier) {
      copy_rows(kvb, 64 * (i + 1), n_kv, na, wave, lane);
      copy_rows(kvb, 64 * (i + 1) + 32, n_kv, nb, wave, lane);
    }
    if (i > 0) store_target(i - 1);
    half(i, 0, ta);
    half(i, 1, tb);
    wait_vm_n(writer && i > 0 ? 1 : 0);
    bar();
  };
  for (int i = 0; i < n_steps; i += 2) {
    step(i, tile0, tile1, tile2, tile3);
    if (i + 1 < n_steps) step(i + 1, tile2, tile3, tile0, tile1);
  }
  store_target(n_steps - 1);
  wait_vm();  // no copy into LDS outlives the workgroup
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


// ---------------------------------------------------------------------------------------------- backward
constexpr int kIH = 64;   // indexer heads
constexpr int kID = 128;  // indexer head dim
constexpr int kBKT = 32 * kID * 2;  // bf16 key tile of 32 rows: 8 KiB

// 16-byte chunk swizzle of a 256-byte bf16 row: the fragment reads (16 rows, one chunk) and the
// transposing reads (8 rows, four 8-byte units) both hit every bank once.
__device__ __forceinline__ int cswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// 16 e4m3 codes -> 16 bf16 values (exact), as 8 packed pairs
__device__ __forceinline__ void codes_to_bf16(const u32x4 c, unsigned int (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], true);
    o[2 * i] = pack_bf16x2(a[0], a[1]);
    o[2 * i + 1] = pack_bf16x2(b[0], b[1]);
  }
}

// Write one 16-code chunk (dims 16c .. 16c+15) of tile row r as bf16 chunks 2c, 2c+1 (swizzled).
__device__ __forceinline__ void store_row_chunk(char* tile, int r, int c, const u32x4 codes) {
  unsigned int o[8];
  codes_to_bf16(codes, o);
  char* rowp = tile + r * (kID * 2);
  *(u32x4*)(rowp + 16 * ((2 * c) ^ cswz(r))) = (u32x4){o[0], o[1], o[2], o[3]};
  *(u32x4*)(rowp + 16 * ((2 * c + 1) ^ cswz(r))) = (u32x4){o[4], o[5], o[6], o[7]};
}

// Transposing reads of a bf16 tile (256-byte rows): for the 16-row half at row r0, the A operand of
// four 32-column blocks (as V^T in attention): out[db][0] rows r0 + 0..7, out[db][1] rows r0 + 8..15.
// toff[db][rd]: the lane's byte offset for column block db and 8-row half rd (the swizzle differs).
typedef short v4s_w __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_w lds_v4s_w;
__device__ __forceinline__ void tr_frags(const char* tile, const int (&toff)[4][2], int r0, u32x2 (&vr)[4][2]) {
  const char* base = tile + r0 * (kID * 2);
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int rd = 0; rd < 2; rd++)
      vr[db][rd] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_w*)(lds_void_w*)(base + toff[db][rd])));
}

// Lane offsets for tr_frags: rows 8rd + 4(G>>1) + (j>>2), columns 32db + 16(G&1) + 4(j&3) (G = l/16, j = l%16).
__device__ __forceinline__ void tr_offsets(int lane, int (&toff)[4][2]) {
  const int G = lane >> 4, j = lane & 15;
#pragma unroll
  for (int rd = 0; rd < 2; rd++) {
    const int r = 8 * rd + 4 * (G >> 1) + (j >> 2);  // r0 (a multiple of 16) does not change cswz
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const int c = 4 * db + 2 * (G & 1) + ((j & 3) >> 1);
      toff[db][rd] = r * (kID * 2) + 16 * (c ^ cswz(r)) + 8 * (j & 1);
    }
  }
}

// A-operand fragment offset (row l%32 of a 32-row block, k-step ks of 16 dims) in a bf16 tile.
__device__ __forceinline__ int frag_offset(int lane, int ks) {
  const int r = lane & 31;
  return r * (kID * 2) + 16 * ((2 * ks + (lane >> 5)) ^ cswz(r));
}

__device__ __forceinline__ float relu_f(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Write 8 codes (dims 8c .. 8c+7) of tile row r as bf16 chunk c (swizzled).
__device__ __forceinline__ void store_row_half(char* tile, int r, int c, const u32x2 codes) {
  const v2f a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[0], false);
  const v2f a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[0], true);
  const v2f b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[1], false);
  const v2f b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[1], true);
  *(u32x4*)(tile + r * (kID * 2) + 16 * (c ^ cswz(r))) =
      (u32x4){pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a1[0], a1[1]), pack_bf16x2(b0[0], b0[1]),
              pack_bf16x2(b1[0], b1[1])};
}

constexpr int kDqKeys = 64;                    // keys per block (one barrier)
constexpr int kDqTile = kDqKeys * kID * 2;     // 16 KiB

template <int Q>  // queries per workgroup (two waves each)
__global__ __launch_bounds__(128 * Q, 2) void warmup_dq_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                                           const uint8_t* __restrict__ k8, const float* __restrict__ ks,
                                                           const float* __restrict__ w, const float* __restrict__ g,
                                                           int64_t ld_g, int n_q, int n_kv, int n_grp,
                                                           float* __restrict__ dq, float* __restrict__ dw) {
  __shared__ __attribute__((aligned(1024))) char kt0[kDqTile];
  __shared__ __attribute__((aligned(1024))) char kt1[kDqTile];
  __shared__ __attribute__((aligned(16))) float gk0[Q][kDqKeys];
  __shared__ __attribute__((aligned(16))) float gk1[Q][kDqKeys];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wave >> 1, hb = wave & 1;  // query of the workgroup's Q, block of 32 heads
  const int grp = n_grp - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int t0 = Q * grp;
  const int t = min(t0 + qw, n_q - 1);
  const int pos_last = n_kv - n_q + min(t0 + Q - 1, n_q - 1);
  const int n_blk = pos_last / kDqKeys + 1;
  const size_t row = (size_t)b * n_q + t;
  const uint8_t* kb = k8 + (size_t)b * n_kv * kID;
  const float* ksb = ks + (size_t)b * n_kv;

  // Q^T (B operand of D^T = K . Q^T): lane holds head 32hb + l%32, dims 16ks + 8(l/32) .. +8, as bf16
  v8bf qf[kID / 16];
  {
    const uint8_t* qp = q8 + (row * kIH + 32 * hb + (lane & 31)) * kID + 8 * (lane >> 5);
#pragma unroll
    for (int k2 = 0; k2 < kID / 32; k2++) {
      // dims 32 k2 + 8(l/32) .. +8 and 32 k2 + 16 + 8(l/32) .. +8: two k-steps from two 8-byte loads
      const u32x2 c0 = *(const u32x2*)(qp + 32 * k2);
      const u32x2 c1 = *(const u32x2*)(qp + 32 * k2 + 16);
      unsigned int o[8];
      codes_to_bf16((u32x4){c0[0], c0[1], c1[0], c1[1]}, o);
      qf[2 * k2] = __builtin_bit_cast(v8bf, (u32x4){o[0], o[1], o[2], o[3]});
      qf[2 * k2 + 1] = __builtin_bit_cast(v8bf, (u32x4){o[4], o[5], o[6], o[7]});
    }
  }
  int koff[kID / 16], toff[4][2];
#pragma unroll
  for (int k = 0; k < kID / 16; k++) koff[k] = frag_offset(lane, k);
  tr_offsets(lane, toff);

  v16f acc[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;
  float dwa = 0.f;

  // staging of block i: 64 key rows of 16 chunks of 8 codes, 8/Q per thread (rows tid/16 + 8Q j); threads
  // < 64Q also fetch g k_scale of (query tid/64, key tid%64), zero past the query's position
  constexpr int kRowsPer = 8 * Q;
  const int st_r = tid >> 4, st_c = tid & 15;
  // (the loads are issued by every thread, in bounds, and their values are only combined at the store, so
  // no wait for them falls before the block's products)
  u32x2 st_codes[kDqKeys / kRowsPer];
  float st_g = 0.f, st_k = 0.f;
  bool st_ok = false;
  auto stage_load = [&](int i) {
#pragma unroll
    for (int u = 0; u < kDqKeys / kRowsPer; u++) {
      const int s = min(kDqKeys * i + kRowsPer * u + st_r, n_kv - 1);
      st_codes[u] = *(const u32x2*)(kb + (size_t)s * kID + 8 * st_c);
    }
    const int qt = min(t0 + ((tid >> 6) & (Q - 1)), n_q - 1);
    const int key = kDqKeys * i + (tid & 63);
    const int kc = min(key, n_kv - 1);
    st_g = g[((size_t)b * n_q + qt) * ld_g + min(kc, n_kv - n_q + qt)];
    st_k = ksb[kc];
    st_ok = key <= n_kv - n_q + qt;
  };
  auto stage_store = [&](char* tile, float (*gk)[kDqKeys]) {
#pragma unroll
    for (int u = 0; u < kDqKeys / kRowsPer; u++) store_row_half(tile, kRowsPer * u + st_r, st_c, st_codes[u]);
    if (tid < 64 * Q) gk[tid >> 6][tid & 63] = st_ok ? st_g * st_k : 0.f;
  };

  auto sub = [&](const char* tile, const float* gkq) {
    // D^T[key][head] for the wave's query and heads: lane = head 32hb + l%32, value r = key 8(r/4) + 4(l/32) + r%4
    v16f d;
#pragma unroll
    for (int k = 0; k < kID / 16; k++) {
      const v8bf kf = *(const v8bf*)(tile + koff[k]);
      d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], k == 0 ? (v16f){} : d, 0, 0, 0);
    }
    float gkv[16];
#pragma unroll
    for (int qd = 0; qd < 4; qd++) {
      const v4f v = *(const v4f*)(gkq + 8 * qd + 4 * (lane >> 5));
#pragma unroll
      for (int e = 0; e < 4; e++) gkv[4 * qd + e] = v[e];
    }
    unsigned int pk[8];
    {
      float m[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        dwa = fmaf(gkv[r], relu_f(d[r]), dwa);
        m[r] = d[r] > 0.f ? gkv[r] : 0.f;
      }
#pragma unroll
      for (int g8 = 0; g8 < 8; g8++) pk[g8] = pack_bf16x2(m[2 * g8], m[2 * g8 + 1]);
    }
    // dq^T[dim][head] += K^T[dim][keys] . M^T[keys][head], two 16-key halves
#pragma unroll
    for (int kh = 0; kh < 2; kh++) {
      u32x2 vr[4][2];
      tr_frags(tile, toff, 16 * kh, vr);
      const v8bf mf = __builtin_bit_cast(v8bf, (u32x4){pk[4 * kh], pk[4 * kh + 1], pk[4 * kh + 2], pk[4 * kh + 3]});
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const v8bf kf = __builtin_bit_cast(v8bf, (u32x4){vr[db][0][0], vr[db][0][1], vr[db][1][0], vr[db][1][1]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, mf, acc[db], 0, 0, 0);
      }
    }
  };
  auto block = [&](const char* tile, float (*gk)[kDqKeys]) {
    sub(tile, &gk[qw][0]);
    __builtin_amdgcn_sched_barrier(0);
    sub(tile + 32 * (kID * 2), &gk[qw][32]);
  };

  stage_load(0);
  stage_store(kt0, gk0);
  stage_load(1);
  __syncthreads();
  for (int i = 0; i < n_blk; i += 2) {
    stage_store(kt1, gk1);  // block i+1 (its buffers were last read in block i-1)
    stage_load(i + 2);
    block(kt0, gk0);
    __syncthreads();
    stage_store(kt0, gk0);  // block i+2
    stage_load(i + 3);
    if (i + 1 < n_blk) block(kt1, gk1);
    __syncthreads();
  }

  if (t0 + qw < n_q) {
    const int h = 32 * hb + (lane & 31);
    const float wh = w[row * kIH + h];
    float* dqp = dq + (row * kIH + h) * kID + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int qd = 0; qd < 4; qd++)
        *(v4f*)(dqp + 32 * db + 8 * qd) = (v4f){acc[db][4 * qd] * wh, acc[db][4 * qd + 1] * wh,
                                                acc[db][4 * qd + 2] * wh, acc[db][4 * qd + 3] * wh};
    const float dsum = xor32_sum(dwa);
    if (lane < 32) dw[row * kIH + h] = dsum * qs[row * kIH + h];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0.f;
}

constexpr int kQT = kIH * kID * 2;  // bf16 query tile: 64 heads x 128 dims, 16 KiB

template <int KW>  // waves per workgroup, 32 keys each
__global__ __launch_bounds__(64 * KW, 2) void warmup_dk_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                                           const uint8_t* __restrict__ k8, const float* __restrict__ w,
                                                           const float* __restrict__ g, int64_t ld_g, int n_q,
                                                           int n_kv, int q_part, int kb_major, float* __restrict__ dk) {
  __shared__ __attribute__((aligned(1024))) char qt0[kQT];
  __shared__ __attribute__((aligned(1024))) char qt1[kQT];
  __shared__ __attribute__((aligned(16))) float cf0[kIH], cf1[kIH];  // w q_scale per head
  __shared__ float gq0[32 * KW], gq1[32 * KW];                          // g of the workgroup's keys
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // part `part` of the queries that see key block `kblk`: q_part queries from the first one.  The grid's
  // fastest dimension is the part (kb_major = 0) or the key block (kb_major = 1); along it, groups of eight
  // alternate direction, so that the round-robin placement of consecutive workgroups on the eight XCDs
  // gives each XCD early and late (fuller and emptier) indexes alike.
  int fast = (int)blockIdx.x;
  {
    const int grp = fast >> 3, r = fast & 7;
    if ((grp & 1) && 8 * grp + 7 < (int)gridDim.x) fast = 8 * grp + 7 - r;
  }
  const int kblk = kb_major ? fast : (int)blockIdx.y;
  const int part = kb_major ? (int)blockIdx.y : fast;
  const int s_base = 32 * KW * kblk, b = blockIdx.z;
  const int off = n_kv - n_q;  // pos_t = t + off
  const int t_lo = max(0, s_base - off) + q_part * part;
  const int t_hi = min(n_q, t_lo + q_part);
  if (t_lo >= t_hi) return;  // whole workgroup: past the last query
  const int s_lane = s_base + 32 * wave + (lane & 31);

  // K (B operand of D = Q . K^T): lane holds key s_lane, dims 16ks + 8(l/32) .. +8, as bf16
  v8bf kf[kID / 16];
  {
    const uint8_t* kp = k8 + ((size_t)b * n_kv + min(s_lane, n_kv - 1)) * kID + 8 * (lane >> 5);
#pragma unroll
    for (int k2 = 0; k2 < kID / 32; k2++) {
      const u32x2 c0 = *(const u32x2*)(kp + 32 * k2);
      const u32x2 c1 = *(const u32x2*)(kp + 32 * k2 + 16);
      unsigned int o[8];
      codes_to_bf16((u32x4){c0[0], c0[1], c1[0], c1[1]}, o);
      kf[2 * k2] = __builtin_bit_cast(v8bf, (u32x4){o[0], o[1], o[2], o[3]});
      kf[2 * k2 + 1] = __builtin_bit_cast(v8bf, (u32x4){o[4], o[5], o[6], o[7]});
    }
  }
  int qoff[kID / 16], toff[4][2];
#pragma unroll
  for (int k = 0; k < kID / 16; k++) qoff[k] = frag_offset(lane, k);
  tr_offsets(lane, toff);
  v16f acc[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;

  // staging of query t: the 64 x 8 chunks of 16 codes, 8/KW per thread (chunk j = (8/KW) tid + u: head j/8,
  // codes 16 (j%8) ..); threads < 64 the head's w q_scale; threads 64 .. 64 + 32KW g of key s_base + tid - 64
  // (zero past t's position)
  constexpr int kU = 8 / KW;
  // (every thread issues its loads, in bounds, and the values are only combined at the store, so no wait
  // for them falls before the query's products)
  u32x4 st_q[kU];
  float st_x = 0.f, st_y = 0.f;
  bool st_ok = false;
  auto stage_load = [&](int t) {
    const size_t row = (size_t)b * n_q + t;
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int j = kU * tid + u;
      st_q[u] = *(const u32x4*)(q8 + (row * kIH + (j >> 3)) * kID + 16 * (j & 7));
    }
    const int s = s_base + tid - kIH;
    const int pos = t + off;
    const float* px = tid < kIH ? w + row * kIH + tid : g + row * ld_g + max(0, min(s, pos));
    const float* py = tid < kIH ? qs + row * kIH + tid : px;
    st_x = *px;
    st_y = *py;
    st_ok = s <= pos;
  };
  auto stage_store = [&](char* tile, float* cf, float* gq) {
#pragma unroll
    for (int u = 0; u < kU; u++) {
      const int j = kU * tid + u;
      store_row_chunk(tile, j >> 3, j & 7, st_q[u]);
    }
    if (tid < kIH) cf[tid] = st_x * st_y;
    else if (tid < kIH + 32 * KW) gq[tid - kIH] = st_ok ? st_x : 0.f;
  };
  auto query = [&](const char* tile, const float* cf, const float* gq) {
    // D[head][key]: lane = key s_lane, value r of block hb = head 32hb + 8(r/4) + 4(l/32) + r%4
    v16f d[2];
#pragma unroll
    for (int k = 0; k < kID / 16; k++)
#pragma unroll
      for (int hb = 0; hb < 2; hb++) {
        const v8bf qf = *(const v8bf*)(tile + hb * 32 * (kID * 2) + qoff[k]);
        d[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[k], k == 0 ? (v16f){} : d[hb], 0, 0, 0);
      }
    const float gv = gq[32 * wave + (lane & 31)];
    unsigned int pk[2][8];
#pragma unroll
    for (int hb = 0; hb < 2; hb++) {
      float cv[16];
#pragma unroll
      for (int qd = 0; qd < 4; qd++) {
        const v4f v = *(const v4f*)(cf + 32 * hb + 8 * qd + 4 * (lane >> 5));
#pragma unroll
        for (int e = 0; e < 4; e++) cv[4 * qd + e] = v[e];
      }
      float m[16];
#pragma unroll
      for (int r = 0; r < 16; r++) m[r] = d[hb][r] > 0.f ? gv * cv[r] : 0.f;
#pragma unroll
      for (int g8 = 0; g8 < 8; g8++) pk[hb][g8] = pack_bf16x2(m[2 * g8], m[2 * g8 + 1]);
    }
    // dk^T[dim][key] += Q^T[dim][heads] . N[heads][key], four 16-head halves
#pragma unroll
    for (int hb = 0; hb < 2; hb++)
#pragma unroll
      for (int kh = 0; kh < 2; kh++) {
        u32x2 vr[4][2];
        tr_frags(tile, toff, 32 * hb + 16 * kh, vr);
        const v8bf nf = __builtin_bit_cast(v8bf, (u32x4){pk[hb][4 * kh], pk[hb][4 * kh + 1], pk[hb][4 * kh + 2],
                                                         pk[hb][4 * kh + 3]});
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const v8bf qf = __builtin_bit_cast(v8bf, (u32x4){vr[db][0][0], vr[db][0][1], vr[db][1][0], vr[db][1][1]});
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, nf, acc[db], 0, 0, 0);
        }
      }
  };

  stage_load(t_lo);
  stage_store(qt0, cf0, gq0);
  stage_load(min(t_lo + 1, t_hi - 1));
  __syncthreads();
  for (int t = t_lo; t < t_hi; t += 2) {
    stage_store(qt1, cf1, gq1);  // query t+1 (its buffers were last read for query t-1)
    stage_load(min(t + 2, t_hi - 1));
    query(qt0, cf0, gq0);
    __syncthreads();
    stage_store(qt0, cf0, gq0);  // query t+2
    stage_load(min(t + 3, t_hi - 1));
    if (t + 1 < t_hi) query(qt1, cf1, gq1);
    __syncthreads();
  }
  if (s_lane < n_kv) {
    float* dkp = dk + ((size_t)b * n_kv + s_lane) * kID + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int qd = 0; qd < 4; qd++)
#pragma unroll
        for (int e = 0; e < 4; e++) atomicAdd(dkp + 32 * db + 8 * qd + e, acc[db][4 * qd + e]);
  }
}


}  // namespace

hipError_t launch_warmup_forward(const uint16_t* q, const uint16_t* kv, const float* lse, int B, int n_q, int n_kv,
                                 float sm_scale, float* scores, int64_t ld_s, float* p, int64_t ld_p, float* loss,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(warmup_target_kernel, dim3((n_q + 1) / 2, B), dim3(512), 0, stream, q, kv, lse, n_q, n_kv,
                     sm_scale, p, ld_p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(warmup_loss_kernel, dim3(n_q, B), dim3(256), 0, stream, scores, ld_s, (const float*)p, ld_p, n_q,
                     n_kv, loss);
  return hipGetLastError();
}

hipError_t launch_warmup_backward(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                                  const float* w, const float* g, int64_t ld_g, int B, int n_q, int n_kv, float* dq,
                                  float* dw, float* dk, hipStream_t stream) {
  constexpr int kQ = 4;
  const int n_grp = (n_q + kQ - 1) / kQ;
  hipLaunchKernelGGL(warmup_dq_kernel<kQ>, dim3(n_grp, B), dim3(128 * kQ), 0, stream, q8, qs, k8, ks, w, g, ld_g, n_q,
                     n_kv, n_grp, dq, dw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n_dk = (size_t)B * n_kv * kID;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<size_t>((n_dk + 255) / 256, 4096)), dim3(256), 0, stream,
                     dk, n_dk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Every key block's queries in parts of q_part (a multiple of 32; workgroups past a block's last query
  // exit at once): about 4 parts per workgroup slot (one per CU) over the causal total, 32 .. 1024 queries.
  constexpr int kKW = 8, kKeys = 32 * kKW;
  const int n_kblk = (n_kv + kKeys - 1) / kKeys;
  const int off = n_kv - n_q;
  int64_t total = 0;
  for (int kb = 0; kb < n_kblk; kb++) total += n_q - std::max(0, std::min(n_q, kKeys * kb - off));
  total *= B;
  const int q_part = (int)std::min<int64_t>(1024, std::max<int64_t>(32, (total / 1024 + 31) / 32 * 32));
  const int n_parts = (n_q + q_part - 1) / q_part;
  // Order of the workgroups.  Each reads the codes of its queries (8 KiB each) one query ahead of their
  // use.  Part-major order runs the parts of one key block together: they read disjoint queries, which
  // the last-level cache serves while all queries' codes fit it (8K: 67 MB).  Beyond that (32K: 268 MB)
  // those reads wait on HBM, and key-block-major order, whose neighbouring key blocks read overlapping
  // query ranges, is faster (32K warm-up backward 42.1 -> 33.7 ms; 24K 20.2 -> 19.8; 16K 9.5 either way;
  // 8K 2.44 against 3.0 ms in part-major order).
  const int kb_major = (size_t)B * n_q * kIH * kID > ((size_t)192 << 20) ? 1 : 0;
  const dim3 grid = kb_major ? dim3(n_kblk, n_parts, B) : dim3(n_parts, n_kblk, B);
  hipLaunchKernelGGL(warmup_dk_kernel<kKW>, grid, dim3(64 * kKW), 0, stream, q8, qs, k8, w, g, ld_g, n_q, n_kv,
                     q_part, kb_major, dk);
  return hipGetLastError();
}

}  // namespace dsa

