// sparse_bwd.hip -- gradients of the sparse MQA-mode attention for the sparse training stage (velog
// summary "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models", Continued Pre-Training,
// Stage 2: the whole model trains through the top-k selection of section 1.2; section 1.3: one latent
// row serves as the key (576 columns) and the value (its first 512) of every head).  With P the
// attention probabilities over the selected entries and dP = dout . V:
//   dS = P (dP - D),  D = dout . out  (per head; equal to sum_j P_j dP_j)
//   dq = sm_scale dS K,   dkv[s] += sm_scale dS^T q + [P^T dout, 0]   (scatter over the selection)
// The same pass yields the head mean of P per selected entry, the indexer's target in that stage.
//
// Two kernels per chunk of query rows, sized to one CU's registers and LDS:
//   sbwd_probs_kernel  one workgroup of 8 waves per query.  The selected latent rows are copied into LDS
//                      32 per step (two buffers).  Waves 0..3 hold Q of 32 heads each in registers and
//                      compute S = Q K^T on the 32x32x16 bf16 matrix core, so each lane holds one key and
//                      16 heads, then P = exp(S sm_scale - lse); waves 4..7 hold dout of the same heads and
//                      compute dP = dout V^T in the same layout.  P crosses to the dP waves through LDS,
//                      which form sm_scale dS, and both go out as bf16, key-major ([entry][128 heads],
//                      256 B per entry) through an LDS staging tile.  The head mean of P is lane-local
//                      plus one swap and one exchange across the waves.
//   sbwd_grads_kernel  one workgroup of 8 waves per (query, 192 of the 576 latent columns); the three
//                      column blocks of a query run on one XCD so its P and dS tiles come through one L2.
//                      Per step of 32 entries the dS, P and latent-column tiles are copied into LDS
//                      (two buffers).  dq[128 x 192] += dS K on the 32x32x16 core, both operands by
//                      transposing LDS reads; dkv[32 x 192] = dS^T Q + P^T dout on the 16x16x32 core,
//                      with the Q and dout operands held in registers for the whole query (loaded once
//                      through LDS); the products are formed transposed so that each lane holds four
//                      consecutive columns of one entry.  Each entry's dkv terms go to HBM as bf16 rows,
//                      one step late and after the next copies are issued, so the wait for a tile never
//                      waits for a store.
//   dkv                without 576-wide atomics (fp32 atomics run at about 5e10 adds/s here, far below
//                      what the scatter needs): the chunk's (query, entry) pairs are listed per key by a
//                      counting sort, and one wave per key sums its pairs' rows into dkv.
#include <algorithm>

#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kBH = 128;                  // heads
constexpr int kBD = 576;                  // latent row (key) width
constexpr int kBV = 512;                  // value width
constexpr int kBRow = kBD * 2;            // 1152 B
constexpr int kBChunks = kBRow / 16;      // 72
constexpr int kBTile = 32 * kBRow;        // 36864 B: 32 rows, chunks swizzled by (row >> 1) & 7
constexpr float kBLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void_b;

__device__ __forceinline__ void vm_wait0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void lds_bar() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte chunk swizzle of a 256-byte bf16 row (entry-major P and dS tiles): fragment reads (16 rows,
// one chunk) and transposing reads (8 rows, four 8-byte units) both hit every bank once.
__device__ __forceinline__ int cswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// ------------------------------------------------------------------------------------------------ probs

// The 32 latent rows of one step into a tile (waves 0..3, 9 copies of 1 KiB each): copy i of wave w
// fills slots (9w + i) * 64 + lane = (row, chunk'), fetching global chunk chunk' ^ ((row >> 1) & 7) of
// latent row sel_l[e0 + row] (row 0 for an invalid entry).
__device__ __forceinline__ void gather_step(const char* __restrict__ kvb, const int* sel_l, int e0, char* tile,
                                            int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int i = 0; i < 9; i++) {
    const int slot = (9 * wave + i) * 64 + l;
    const int r = slot / kBChunks, cs = slot - kBChunks * r;
    const int c = cs ^ ((r >> 1) & 7);
    const int s = max(sel_l[e0 + r], 0);
    const unsigned int off = (unsigned int)s * kBRow + 16u * c;
    __builtin_amdgcn_global_load_lds((const void*)(kvb + off), (lds_void_b*)(tile + (9 * wave + i) * 1024), 16, 0,
                                     0);
  }
}

constexpr int kBMaxK = 2048;

// Four K/V fragments of k-steps 4M .. 4M+3 (lane addresses a[j] = tile + kb[j], offset 128M).  The two
// roles run separate loops, so the compiler sees no copy in flight into the tile being read.
template <int M>
__device__ __forceinline__ void rd4(const unsigned int (&a)[4], v8bf (&x)[4]) {
#pragma unroll
  for (int j = 0; j < 4; j++) x[j] = *(const v8bf*)((const char*)(lds_void_b*)(uintptr_t)a[j] + 128 * M);
}

template <int NM, int M = 0>
__device__ __forceinline__ void chain(const unsigned int (&a)[4], const v8bf (&f)[kBD / 16], v16f& acc) {
  v8bf x[4];
  rd4<M>(a, x);
#pragma unroll
  for (int j = 0; j < 4; j++)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[4 * M + j], x[j], M + j == 0 ? (v16f){} : acc, 0, 0, 0);
  if constexpr (M + 1 < NM) chain<NM, M + 1>(a, f, acc);
}

__global__ __launch_bounds__(512, 1) void sbwd_probs_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ kv,
                                                            const int32_t* __restrict__ idx,
                                                            const uint16_t* __restrict__ out,
                                                            const float* __restrict__ lse,
                                                            const uint16_t* __restrict__ dout, int r0, int n_q,
                                                            int n_kv, int k, float sm_scale,
                                                            uint16_t* __restrict__ ws_p, uint16_t* __restrict__ ws_s,
                                                            float* __restrict__ pbar) {
  __shared__ __attribute__((aligned(1024))) char tile0[kBTile];
  __shared__ __attribute__((aligned(1024))) char tile1[kBTile];
  __shared__ __attribute__((aligned(16))) v4f xp[4][4][64];  // P of the S waves: [wave][register quad][lane]
  __shared__ __attribute__((aligned(1024))) char stp[32 * 256];  // staging: [entry][128 heads] bf16, swizzled
  __shared__ __attribute__((aligned(1024))) char sts[32 * 256];
  __shared__ float part[4][32];
  __shared__ float dl[kBH];
  __shared__ int sel_l[kBMaxK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool sw = wave < 4;   // S waves (Q, P) or dP waves (dout, dS)
  const int hw = wave & 3;    // heads 32hw .. 32hw + 31
  const int row = r0 + (int)blockIdx.x;
  const int b = row / n_q;
  const int n_steps = (k + 31) / 32;
  const char* kvb = (const char*)(kv + (size_t)b * n_kv * kBD);

  // the row's selection: valid latent row or -1 (also past k, up to the last step's end); as in the
  // forward attention, an entry is valid when it names a key row, whatever the query's position
  {
    int sv[kBMaxK / 512];  // all of a thread's loads in flight at once (k <= kBMaxK)
#pragma unroll
    for (int u = 0; u < kBMaxK / 512; u++) {
      const int e = tid + 512 * u;
      sv[u] = e < k ? idx[(size_t)row * k + e] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBMaxK / 512; u++) {
      const int e = tid + 512 * u;
      if (e < 32 * n_steps) sel_l[e] = (sv[u] >= 0 && sv[u] < n_kv) ? sv[u] : -1;
    }
  }
  // S waves: Q (A operand of S = Q K^T): lane holds head 32hw + l%32, dims 16ks + 8(l/32) .. +8.
  // dP waves: dout of the same heads, first 32 k-steps.
  v8bf f[kBD / 16];
  float hv[16];  // per accumulator register (head 32hw + 8(r/4) + 4(l/32) + r%4): lse (log2) or D
  if (sw) {
    const uint16_t* qh = q + ((size_t)row * kBH + 32 * hw + (lane & 31)) * kBD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kBD / 16; ks++) f[ks] = *(const v8bf*)(qh + 16 * ks);
#pragma unroll
    for (int r = 0; r < 16; r++)
      hv[r] = lse[(size_t)row * kBH + 32 * hw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] * kBLog2e;
  } else {
    const size_t ho = ((size_t)row * kBH + 32 * hw + (lane & 31)) * kBV + 8 * (lane >> 5);
    float dd = 0.f;
#pragma unroll
    for (int ks = 0; ks < kBV / 16; ks++) {
      f[ks] = *(const v8bf*)(dout + ho + 16 * ks);
      const v8bf o = *(const v8bf*)(out + ho + 16 * ks);
#pragma unroll
      for (int e = 0; e < 8; e++) dd = fmaf((float)f[ks][e], (float)o[e], dd);
    }
    dd = xor32_sum(dd);  // lanes l and l ^ 32 hold the two halves of each 16-column step
    if (lane < 32) dl[32 * hw + lane] = dd;
  }
  lds_bar();
  if (!sw) {
#pragma unroll
    for (int r = 0; r < 16; r++) hv[r] = dl[32 * hw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
  }
  // K fragment (B operand) of k-step ks = 4m + j: row l%32, logical chunk 8m + (2j + l/32), stored at
  // 8m + ((2j + l/32) ^ ((row >> 1) & 7))
  int kb[4];
  {
    const int kr = lane & 31;
#pragma unroll
    for (int j = 0; j < 4; j++) kb[j] = kr * kBRow + 16 * ((2 * j + (lane >> 5)) ^ ((kr >> 1) & 7));
  }
  unsigned int ta0[4], ta1[4];  // fragment addresses in the two tiles
#pragma unroll
  for (int j = 0; j < 4; j++) {
    ta0[j] = (unsigned int)(uintptr_t)(lds_void_b*)(tile0 + kb[j]);
    ta1[j] = (unsigned int)(uintptr_t)(lds_void_b*)(tile1 + kb[j]);
  }
  const float c_scale = sm_scale * kBLog2e;
  if (sw) {
    gather_step(kvb, sel_l, 0, tile0, wave, lane);
    vm_wait0();
  }
  lds_bar();

  // The two roles run separate loops with the same barriers (two per step).
  if (sw) {
    // S waves: copies of step i+1, S = Q K^T, P, the head sums; wait for the copies
    auto step = [&](int i, const unsigned int (&ta)[4], char* next) {
      const int e0 = 32 * i;
      if (i + 1 < n_steps) gather_step(kvb, sel_l, e0 + 32, next, wave, lane);
      v16f acc;
      chain<kBD / 64>(ta, f, acc);
      // lane: entry e0 + l%32, heads 32hw + 8(r/4) + 4(l/32) + r%4
      const bool valid = sel_l[e0 + (lane & 31)] >= 0;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        acc[r] = valid ? __builtin_amdgcn_exp2f(fmaf(acc[r], c_scale, -hv[r])) : 0.f;
        psum += acc[r];
      }
#pragma unroll
      for (int qd = 0; qd < 4; qd++)
        xp[hw][qd][lane] = (v4f){acc[4 * qd], acc[4 * qd + 1], acc[4 * qd + 2], acc[4 * qd + 3]};
      psum = xor32_sum(psum);
      if (lane < 32) part[hw][lane] = psum;
      lds_bar();
      vm_wait0();  // this wave's copies of the next step have landed
      lds_bar();
    };
    for (int i = 0; i < n_steps; i += 2) {
      step(i, ta0, tile1);
      if (i + 1 < n_steps) step(i + 1, ta1, tile0);
    }
  } else {
    // dP waves: dP = dout V^T; after the exchange sm_scale dS = sm_scale P (dP - D), P and dS staged and
    // written out (256 B per entry), the head mean of P
    auto step = [&](int i, const unsigned int (&ta)[4]) {
      const int e0 = 32 * i;
      v16f acc;
      chain<kBV / 64>(ta, f, acc);
      lds_bar();
      const int key = lane & 31;
#pragma unroll
      for (int qd = 0; qd < 4; qd++) {
        const v4f p4 = xp[hw][qd][lane];
        float d4[4];
#pragma unroll
        for (int e = 0; e < 4; e++) d4[e] = p4[e] * (acc[4 * qd + e] - hv[4 * qd + e]) * sm_scale;
        const int h0 = 32 * hw + 8 * qd + 4 * (lane >> 5);
        const int off = key * 256 + 16 * ((h0 >> 3) ^ (key & 15)) + 2 * (h0 & 7);
        *(u32x2*)(stp + off) = (u32x2){pack_bf16x2(p4[0], p4[1]), pack_bf16x2(p4[2], p4[3])};
        *(u32x2*)(sts + off) = (u32x2){pack_bf16x2(d4[0], d4[1]), pack_bf16x2(d4[2], d4[3])};
      }
      if (wave == 4 && pbar != nullptr && lane < 32 && e0 + lane < k)
        pbar[(size_t)row * k + e0 + lane] = (part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane]) * (1.0f / kBH);
      lds_bar();
      // staging -> workspace rows (row - r0) * k_pad + e (entries past k hold zeros): 2 chunks of each
      // tile per thread
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int j = (tid - 256) + 256 * u;
        const int ky = j >> 4, c = j & 15;
        const int so = ky * 256 + 16 * (c ^ (ky & 15));
        const size_t go = ((size_t)(row - r0) * (32 * n_steps) + e0 + ky) * kBH + 8 * c;
        *(u32x4*)(ws_p + go) = *(const u32x4*)(stp + so);
        *(u32x4*)(ws_s + go) = *(const u32x4*)(sts + so);
      }
    };
    for (int i = 0; i < n_steps; i += 2) {
      step(i, ta0);
      if (i + 1 < n_steps) step(i + 1, ta1);
    }
  }
}

// ------------------------------------------------------------------------------------------------ grads

constexpr int kGD = 192;                 // latent columns per workgroup
constexpr int kGRow = kGD * 2;           // 384 B
constexpr int kGChunks = kGRow / 16;     // 24
constexpr int kGK = 32 * kGRow;          // 12288 B: latent-column tile of a step
constexpr int kGS = 32 * 256;            // 8192 B: P or dS tile of a step
constexpr int kGStage = kBH * kGRow;     // 49152 B: Q or dout columns of the query (prologue only)

// Chunk swizzles of 384-byte rows: latent-column tile (32x32 transposing reads: 4 rows x 64 B per half
// wave) and Q / dout staging (16x16 transposing reads: 8 rows x 32 B per half wave).
__device__ __forceinline__ int swz_k(int r) { return 4 * ((r >> 1) & 1); }
__device__ __forceinline__ int swz_q(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) and two 16-byte LDS reads.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ void tr2(const char* a0, const char* a1, u32x2& x0, u32x2& x1) {
  x0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_void_b*)a0));
  x1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_void_b*)a1));
}
__device__ __forceinline__ void rd2(const char* a0, const char* a1, v8bf& x0, v8bf& x1) {
  x0 = *(const v8bf*)a0;
  x1 = *(const v8bf*)a1;
}
__device__ __forceinline__ v8bf as_frag(const u32x2 x0, const u32x2 x1) {
  return __builtin_bit_cast(v8bf, (u32x4){x0[0], x0[1], x1[0], x1[1]});
}

__global__ __launch_bounds__(512, 1) void sbwd_grads_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ kv,
                                                            const int32_t* __restrict__ idx,
                                                            const uint16_t* __restrict__ dout,
                                                            const uint16_t* __restrict__ ws_p,
                                                            const uint16_t* __restrict__ ws_s, int r0, int n_rows,
                                                            int n_q, int n_kv, int k, float* __restrict__ dq,
                                                            uint16_t* __restrict__ contrib) {
  // step buffers as separate LDS objects: reads of one never wait for copies into another
  __shared__ __attribute__((aligned(1024))) char kt0[kGK];
  __shared__ __attribute__((aligned(1024))) char kt1[kGK];
  __shared__ __attribute__((aligned(1024))) char st0[kGS];
  __shared__ __attribute__((aligned(1024))) char st1[kGS];
  __shared__ __attribute__((aligned(1024))) char pt0[kGS];
  __shared__ __attribute__((aligned(1024))) char pt1[kGS];
  __shared__ __attribute__((aligned(1024))) char stage[kGStage];  // Q, then dout, in the prologue
  __shared__ int sel_l[kBMaxK];  // the row's selection: valid latent row or -1
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup b runs on XCD b % 8: the three column blocks of a row share b % 8
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int rr = (slot / 3) * 8 + xcd;
  if (rr >= n_rows) return;
  const int cb = slot % 3;
  const int d0 = kGD * cb;
  const int row = r0 + rr;
  const int b = row / n_q;
  const int n_steps = (k + 31) / 32;
  const int G = lane >> 4, jj = lane & 15;

  // ---- prologue: Q and dout columns d0 .. d0+191 of the 128 heads through LDS into B-operand registers
  // of the 16x16x32 products: wave w, column block n = 3(w%4) + j (16 wide), k-step kk (32 heads):
  // lane (G, jj) holds column 16n + jj, heads 32kk + 8G .. +8.
  {
    int sv[kBMaxK / 512];  // all of a thread's loads in flight at once (k <= kBMaxK)
#pragma unroll
    for (int u = 0; u < kBMaxK / 512; u++) {
      const int e = tid + 512 * u;
      sv[u] = e < k ? idx[(size_t)row * k + e] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBMaxK / 512; u++) {
      const int e = tid + 512 * u;
      if (e < 32 * n_steps) sel_l[e] = (sv[u] >= 0 && sv[u] < n_kv) ? sv[u] : -1;
    }
  }
  const int nq0 = 3 * (wave & 3);  // first 16-wide column block of the wave's dkv tiles
  v8bf bq[3][4], bo[3][4];
#pragma unroll
  for (int pass = 0; pass < 2; pass++) {
    // pass 0: Q columns d0.. of the 128 heads; pass 1: dout columns (zero from column 512 on)
#pragma unroll
    for (int u = 0; u < 6; u++) {
      const int j = tid + 512 * u;
      const int r = j / kGChunks, c = j - kGChunks * r;
      const size_t hrow = (size_t)row * kBH + r;
      u32x4 v;
      if (pass == 0) v = *(const u32x4*)(q + hrow * kBD + d0 + 8 * c);
      else v = (d0 + 8 * c < kBV) ? *(const u32x4*)(dout + hrow * kBV + d0 + 8 * c) : (u32x4){0, 0, 0, 0};
      *(u32x4*)(stage + r * kGRow + 16 * (c ^ swz_q(r))) = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 3; j++) {
      const int n = nq0 + j;
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const int ra = 32 * kk + 8 * G + (jj >> 2), rb = ra + 4;
        const int c = 2 * n + ((jj & 3) >> 1);
        u32x2 x0, x1;
        tr2(stage + ra * kGRow + 16 * (c ^ swz_q(ra)) + 8 * (jj & 1),
            stage + rb * kGRow + 16 * (c ^ swz_q(rb)) + 8 * (jj & 1), x0, x1);
        if (pass == 0) bq[j][kk] = as_frag(x0, x1);
        else bo[j][kk] = as_frag(x0, x1);
      }
    }
    __syncthreads();
  }


  const uint16_t* wsr_p = ws_p + (size_t)rr * (32 * n_steps) * kBH;  // rows of k_pad = 32 n_steps entries
  const uint16_t* wsr_s = ws_s + (size_t)rr * (32 * n_steps) * kBH;
  const char* kvb = (const char*)(kv + (size_t)b * n_kv * kBD + d0);
  // copies of step i: the dS and P tiles (one 1 KiB copy each per wave: slot = 64w + lane = (entry,
  // chunk'), global chunk chunk' ^ cswz(entry)), the latent-column tile (waves 0..3, three copies: slot
  // (3w + u) * 64 + lane = (entry, chunk'), global chunk chunk' ^ swz_k(entry))
  auto issue = [&](int i, int selv, char* ktb, char* stb, char* ptb) {
    {
      const int sl = wave * 64 + lane;
      const int r = sl >> 4, c = (sl & 15) ^ cswz(sl >> 4);
      const size_t go = (size_t)(32 * i + r) * kBH + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)(wsr_s + go), (lds_void_b*)(stb + wave * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(wsr_p + go), (lds_void_b*)(ptb + wave * 1024), 16, 0, 0);
    }
    if (wave < 4) {
#pragma unroll
      for (int u = 0; u < 3; u++) {
        const int sl = (3 * wave + u) * 64 + lane;
        const int r = sl / kGChunks, c = (sl - kGChunks * r) ^ swz_k(r);
        const int s = max(__shfl(selv, r), 0);
        const unsigned int off = (unsigned int)s * kBRow + 16u * c;
        __builtin_amdgcn_global_load_lds((const void*)(kvb + off), (lds_void_b*)(ktb + (3 * wave + u) * 1024), 16,
                                         0, 0);
      }
    }
  };

  // dq tiles: head block hb = w/2 (32 heads), column blocks 3(w%2) + j (32 wide); transposing-read offsets
  const int hb = wave >> 1, nd0 = 3 * (wave & 1);
  int toff_s[2], toff_k[3][2];
#pragma unroll
  for (int rd = 0; rd < 2; rd++) {
    const int r = 8 * rd + 4 * (G >> 1) + (jj >> 2);
    const int cs = 4 * hb + 2 * (G & 1) + ((jj & 3) >> 1);
    toff_s[rd] = r * 256 + 16 * (cs ^ cswz(r)) + 8 * (jj & 1);
#pragma unroll
    for (int j = 0; j < 3; j++) {
      const int ck = 4 * (nd0 + j) + 2 * (G & 1) + ((jj & 3) >> 1);
      toff_k[j][rd] = r * kGRow + 16 * (ck ^ swz_k(r)) + 8 * (jj & 1);
    }
  }
  // dkv tiles: entry block eb = w/4 (16 entries); the dS and P fragments (B operand): entry 16eb + l%16,
  // heads 32kk + 8G .. +8
  const int eb = wave >> 2;
  const int ar = 16 * eb + jj;
  int aoff[4];
#pragma unroll
  for (int kk = 0; kk < 4; kk++) aoff[kk] = ar * 256 + 16 * ((4 * kk + G) ^ cswz(ar));
  const bool has_v = d0 + 16 * nq0 < kBV;  // some of the wave's dkv columns are value columns

  v16f acc_q[3];
#pragma unroll
  for (int j = 0; j < 3; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc_q[j][r] = 0.f;
  v4f acc_k[3];

  // the previous step's dkv terms -> contrib[entry][576] (bf16).  The products are formed transposed
  // (Q^T and dout^T as the A operand, the dS and P tiles as B), so lane (G, jj) of tile j holds entry
  // 16eb + jj and the four consecutive columns 16n + 4G .. +4: one 8-byte store per tile, three per wave.
  uint16_t* cr = contrib + (size_t)rr * (32 * n_steps) * kBD + d0 + 4 * G;
  auto flush = [&](int step_i) {
    const int e = 32 * step_i + 16 * eb + jj;
#pragma unroll
    for (int j = 0; j < 3; j++)
      *(u32x2*)(cr + (size_t)e * kBD + 16 * (nq0 + j)) =
          (u32x2){pack_bf16x2(acc_k[j][0], acc_k[j][1]), pack_bf16x2(acc_k[j][2], acc_k[j][3])};
  };

  auto compute = [&](const char* ktb, const char* stb, const char* ptb) {
    // dq[heads][cols] += dS[heads][entries] K[entries][cols], two 16-entry halves
#pragma unroll
    for (int kh = 0; kh < 2; kh++) {
      u32x2 x0, x1;
      tr2(stb + 16 * kh * 256 + toff_s[0], stb + 16 * kh * 256 + toff_s[1], x0, x1);
      const v8bf a = as_frag(x0, x1);
#pragma unroll
      for (int j = 0; j < 3; j++) {
        tr2(ktb + 16 * kh * kGRow + toff_k[j][0], ktb + 16 * kh * kGRow + toff_k[j][1], x0, x1);
        acc_q[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_frag(x0, x1), acc_q[j], 0, 0, 0);
      }
    }
    // dkv[entries][cols] = dS^T Q + P^T dout over the 128 heads (no P^T dout past the value columns)
#pragma unroll
    for (int j = 0; j < 3; j++) acc_k[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (has_v) {
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        v8bf as, ap;
        rd2(stb + aoff[kk], ptb + aoff[kk], as, ap);
#pragma unroll
        for (int j = 0; j < 3; j++) {
          acc_k[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[j][kk], as, acc_k[j], 0, 0, 0);
          acc_k[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo[j][kk], ap, acc_k[j], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        v8bf as, ap;
        rd2(stb + aoff[kk], ptb + aoff[kk], as, ap);
#pragma unroll
        for (int j = 0; j < 3; j++) acc_k[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[j][kk], as, acc_k[j], 0, 0, 0);
      }
    }
  };

  // selection of step i in lanes l%32 (from LDS: no memory wait in the loop but the copies' own)
  auto sel_of = [&](int i) -> int { return sel_l[32 * i + (lane & 31)]; };
  issue(0, sel_of(0), kt0, st0, pt0);
  vm_wait0();
  lds_bar();
  // step i: copies of step i+1 (other buffers, last read in step i-1), the stores of step i-1, the
  // products of step i; then wait for the copies only (the 3 stores may still be in flight)
  auto step = [&](int i, const char* ktb, const char* stb, const char* ptb, char* ktn, char* stn, char* ptn) {
    if (i + 1 < n_steps) issue(i + 1, sel_of(i + 1), ktn, stn, ptn);
    if (i > 0) flush(i - 1);
    compute(ktb, stb, ptb);
    if (i > 0) __builtin_amdgcn_s_waitcnt(0x0F70 | 3);
    else vm_wait0();
    lds_bar();
  };
  for (int i = 0; i < n_steps; i += 2) {
    step(i, kt0, st0, pt0, kt1, st1, pt1);
    if (i + 1 < n_steps) step(i + 1, kt1, st1, pt1, kt0, st0, pt0);
  }
  flush(n_steps - 1);

  // dq: lane = column 32n + l%32, registers = heads 32hb + 8(r/4) + 4(l/32) + r%4
#pragma unroll
  for (int j = 0; j < 3; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int h = 32 * hb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      dq[((size_t)row * kBH + h) * kBD + d0 + 32 * (nd0 + j) + (lane & 31)] = acc_q[j][r];
    }
  vm_wait0();
}

// Stage-2 indexer loss per query row: lse of the index scores over s <= pos, loss = sum_j pbar_j (log pbar_j -
// (I[idx_j] - lse)), and g = softmax(I) - p written over the scores, p = pbar scattered to the selection.
__global__ __launch_bounds__(256) void sparse_kl_kernel(float* __restrict__ scores, int64_t ld_s,
                                                        const float* __restrict__ pbar, const int32_t* __restrict__ idx,
                                                        int n_q, int n_kv, int k, float* __restrict__ loss) {
  __shared__ float red[4];
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * n_q + t;
  const int pos = n_kv - n_q + t, n = pos + 1;
  float* ir = scores + row * ld_s;
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
  for (int j = threadIdx.x; j < k; j += 256) {
    const int s = idx[row * k + j];
    const float pj = pbar[row * k + j];
    if (s >= 0 && s <= pos && pj > 0.f) kl += pj * (__logf(pj) - (ir[s] - lse_i));
  }
  kl = block_reduce(kl, false);  // its barriers also order every read of I above before the writes below
  for (int s = threadIdx.x; s < n; s += 256) ir[s] = __expf(ir[s] - lse_i);
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += 256) {
    const int s = idx[row * k + j];
    if (s >= 0 && s <= pos) ir[s] -= pbar[row * k + j];
  }
  if (threadIdx.x == 0) loss[row] = kl;
}

// ------------------------------------------------------------------------------------------------ dkv
// dkv[key] = the sum of contrib over the (query, entry) pairs that select the key, without atomics on
// the 576-wide rows: the pairs of a chunk are listed per key (a counting sort: count, scan, fill) and one
// wave per key sums its list.  key = b * n_kv + s.

__global__ __launch_bounds__(256) void sbwd_count_kernel(const int32_t* __restrict__ idx, int r0, int n_rows, int n_q,
                                                         int n_kv, int k, int* __restrict__ count) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)n_rows * k) return;
  const int rr = (int)(i / k), e = (int)(i - (size_t)rr * k);
  const int row = r0 + rr, b = row / n_q;
  const int s = idx[(size_t)row * k + e];
  if (s >= 0 && s < n_kv) atomicAdd(&count[(size_t)b * n_kv + s], 1);
}

// offs = exclusive prefix sum of count (one workgroup), count reset to zero for the fill's cursors.
// Thread t owns the contiguous entries [t*per, t*per + per), per a multiple of 32, read 32 at a time
// with every load in flight (16-byte loads: the workspace arrays are 256-byte aligned); the thread
// totals are scanned with wave shuffles and one exchange across the 16 waves.
__device__ __forceinline__ void scan_load32(const int* __restrict__ p, int i, int e, int (&v)[32]) {
  if (i + 32 <= e) {
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int4 q = *(const int4*)(p + i + 4 * u);
      v[4 * u] = q.x; v[4 * u + 1] = q.y; v[4 * u + 2] = q.z; v[4 * u + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; j++) v[j] = i + j < e ? p[i + j] : 0;
  }
}
__global__ __launch_bounds__(1024) void sbwd_scan_kernel(int* __restrict__ count, int* __restrict__ offs, int n) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (((n + 1023) / 1024) + 31) & ~31;
  const int a = min(n, tid * per), e = min(n, a + per);
  int sum = 0;
  for (int i = a; i < e; i += 32) {
    int v[32];
    scan_load32(count, i, e, v);
#pragma unroll
    for (int j = 0; j < 32; j++) sum += v[j];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w2 = 0; w2 < wave; w2++) run += wsum[w2];
  for (int i = a; i < e; i += 32) {
    int v[32];
    scan_load32(count, i, e, v);
    int o[32];
#pragma unroll
    for (int j = 0; j < 32; j++) {
      o[j] = run;
      run += v[j];
    }
    if (i + 32 <= e) {
#pragma unroll
      for (int u = 0; u < 8; u++) {
        *(int4*)(offs + i + 4 * u) = make_int4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
        *(int4*)(count + i + 4 * u) = make_int4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; j++)
        if (i + j < e) {
          offs[i + j] = o[j];
          count[i + j] = 0;
        }
    }
  }
}

__global__ __launch_bounds__(256) void sbwd_fill_kernel(const int32_t* __restrict__ idx, int r0, int n_rows, int n_q,
                                                        int n_kv, int k, int k_pad, const int* __restrict__ offs,
                                                        int* __restrict__ count, int* __restrict__ list) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)n_rows * k) return;
  const int rr = (int)(i / k), e = (int)(i - (size_t)rr * k);
  const int row = r0 + rr, b = row / n_q;
  const int s = idx[(size_t)row * k + e];
  if (s >= 0 && s < n_kv) {
    const size_t key = (size_t)b * n_kv + s;
    list[offs[key] + atomicAdd(&count[key], 1)] = rr * k_pad + e;
  }
}

// one workgroup per key: its four waves take every fourth pair of the key's list (lane l: columns 8l ..
// 8l+7, lanes < 8 also 512 + 8l ..), the partial sums meet in LDS and dkv[key] += their sum; count[key]
// back to zero for the next chunk
__global__ __launch_bounds__(256) void sbwd_reduce_kernel(const uint16_t* __restrict__ contrib,
                                                          const int* __restrict__ offs, int* __restrict__ count,
                                                          const int* __restrict__ list, int n_keys,
                                                          float* __restrict__ dkv) {
  __shared__ __attribute__((aligned(16))) float red[4][kBD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the most-selected keys of a causal chunk are its most recent ones (the highest indices): they are
  // dispatched first, so that the long sums do not start last and trail the grid
  const int key = n_keys - 1 - (int)blockIdx.x;
  const int n = count[key];
  if (n == 0) return;  // whole workgroup
  const int* lp = list + offs[key];
  float a0[8], a1[8];
#pragma unroll
  for (int e = 0; e < 8; e++) a0[e] = a1[e] = 0.f;
  auto add = [&](const u32x4 v, float (&acc)[8]) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      acc[2 * e] += __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
    }
  };
  int p = wave;
  for (; p + 12 < n; p += 16) {
    u32x4 v[4], w[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const uint16_t* row = contrib + (size_t)lp[p + 4 * u] * kBD;
      v[u] = *(const u32x4*)(row + 8 * lane);
      if (lane < 8) w[u] = *(const u32x4*)(row + kBV + 8 * lane);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      add(v[u], a0);
      if (lane < 8) add(w[u], a1);
    }
  }
  for (; p < n; p += 4) {
    const uint16_t* row = contrib + (size_t)lp[p] * kBD;
    add(*(const u32x4*)(row + 8 * lane), a0);
    if (lane < 8) add(*(const u32x4*)(row + kBV + 8 * lane), a1);
  }
  *(v4f*)&red[wave][8 * lane] = (v4f){a0[0], a0[1], a0[2], a0[3]};
  *(v4f*)&red[wave][8 * lane + 4] = (v4f){a0[4], a0[5], a0[6], a0[7]};
  if (lane < 8) {
    *(v4f*)&red[wave][kBV + 8 * lane] = (v4f){a1[0], a1[1], a1[2], a1[3]};
    *(v4f*)&red[wave][kBV + 8 * lane + 4] = (v4f){a1[4], a1[5], a1[6], a1[7]};
  }
  __syncthreads();
  float* d = dkv + (size_t)key * kBD;
  for (int c = threadIdx.x; c < kBD; c += 256) d[c] += red[0][c] + red[1][c] + red[2][c] + red[3][c];
  if (threadIdx.x == 0) count[key] = 0;
}

__global__ __launch_bounds__(256) void sbwd_zero_kernel(float* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0.f;
}

}  // namespace

int sbwd_chunk_rows(int rows) { return rows < 512 ? rows : 512; }

size_t sbwd_workspace_bytes(int B, int n_q, int n_kv, int k) {
  const size_t chunk = (size_t)sbwd_chunk_rows(B * n_q), k_pad = (size_t)(k + 31) / 32 * 32;
  const size_t n_keys = (size_t)B * n_kv;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * up(chunk * k_pad * kBH * 2) + up(chunk * k_pad * kBD * 2) + up(chunk * k_pad * 4) + 2 * up(n_keys * 4);
}

hipError_t launch_sparse_backward(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, int B, int n_q, int n_kv, int k,
                                  float sm_scale, float* dq, float* dkv, float* pbar, void* workspace,
                                  hipStream_t stream) {
  const int rows = B * n_q;
  const int chunk = sbwd_chunk_rows(rows);
  const int k_pad = (k + 31) / 32 * 32;
  const size_t n_keys = (size_t)B * n_kv;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = (char*)workspace;
  uint16_t* ws_p = (uint16_t*)w;
  w += up((size_t)chunk * k_pad * kBH * 2);
  uint16_t* ws_s = (uint16_t*)w;
  w += up((size_t)chunk * k_pad * kBH * 2);
  uint16_t* contrib = (uint16_t*)w;
  w += up((size_t)chunk * k_pad * kBD * 2);
  int* list = (int*)w;
  w += up((size_t)chunk * k_pad * 4);
  int* count = (int*)w;
  w += up(n_keys * 4);
  int* offs = (int*)w;

  const size_t n_dkv = n_keys * kBD;
  hipLaunchKernelGGL(sbwd_zero_kernel, dim3((unsigned)std::min<size_t>((n_dkv + 255) / 256, 4096)), dim3(256), 0,
                     stream, dkv, n_dkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sbwd_zero_kernel, dim3((unsigned)std::min<size_t>((n_keys + 255) / 256, 4096)), dim3(256), 0,
                     stream, (float*)count, n_keys);  // int zero == float zero
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int r0 = 0; r0 < rows; r0 += chunk) {
    const int n = std::min(chunk, rows - r0);
    const unsigned n_ent = (unsigned)(((size_t)n * k + 255) / 256);
    hipLaunchKernelGGL(sbwd_count_kernel, dim3(n_ent), dim3(256), 0, stream, idx, r0, n, n_q, n_kv, k, count);
    hipLaunchKernelGGL(sbwd_probs_kernel, dim3(n), dim3(512), 0, stream, q, kv, idx, out, lse, dout, r0, n_q, n_kv,
                       k, sm_scale, ws_p, ws_s, pbar);
    hipLaunchKernelGGL(sbwd_grads_kernel, dim3((n + 7) / 8 * 8 * 3), dim3(512), 0, stream, q, kv, idx, dout,
                       (const uint16_t*)ws_p, (const uint16_t*)ws_s, r0, n, n_q, n_kv, k, dq, contrib);
    hipLaunchKernelGGL(sbwd_scan_kernel, dim3(1), dim3(1024), 0, stream, count, offs, (int)n_keys);
    hipLaunchKernelGGL(sbwd_fill_kernel, dim3(n_ent), dim3(256), 0, stream, idx, r0, n, n_q, n_kv, k, k_pad,
                       (const int*)offs, count, list);
    hipLaunchKernelGGL(sbwd_reduce_kernel, dim3((unsigned)n_keys), dim3(256), 0, stream,
                       (const uint16_t*)contrib, (const int*)offs, count, (const int*)list, (int)n_keys, dkv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sparse_kl(float* scores, int64_t ld_s, const float* pbar, const int32_t* idx, int B, int n_q,
                            int n_kv, int k, float* loss, hipStream_t stream) {
  hipLaunchKernelGGL(sparse_kl_kernel, dim3(n_q, B), dim3(256), 0, stream, scores, ld_s, pbar, idx, n_q, n_kv, k, loss);
  return hipGetLastError();
}

}  // namespace dsa
