// masked_mha.hip -- masked MHA mode for short prefills (velog summary "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models", section 3.3 Inference Cost; notes.yuuk.io page of the same
// title, section on inference cost): attention runs in MHA form, every head with its own key and value
// rows, densely over the causal keys, and the top-k selection enters as a mask.  Masked keys leave the
// softmax, so the result is exactly the attention over the selected entries, as in the sparse path.
//
//   mha_mask_kernel    idx [B][n_q][k_sel] -> one bit per (query, key): mask [B][n_q][W] u32,
//                      W = 2 * ceil(n_kv / 64) (whole 64-key tiles; bits past the keys are zero).
//                      Entries outside 0 <= s <= pos_t are ignored.
//   mha_masked_kernel  bf16, d_qk = 192, d_v = 128, any H.  One workgroup of 4 waves per (128 queries,
//                      head); wave w owns queries 32w..32w+31 of the tile and streams 64-key tiles:
//     tiles   K [64][192] and V [64][128] of the head are copied HBM/L2 -> LDS with
//             global_load_lds_dwordx4, tile j+1 while tile j computes (two buffers, separate LDS
//             objects so that reads of one never wait for copies into the other).  Rows are
//             contiguous; 16-byte chunks are XOR-swizzled inside each row (K: chunk ^ ((row>>1)&7),
//             V: chunk ^ ((row&3)<<2)) so that the fragment reads hit every bank once; the copy of
//             LDS slot (row, chunk') fetches global chunk chunk' ^ swizzle(row).
//     QK      S^T[32 keys][32 queries] = K . Q^T on the 32x32x16 bf16 matrix core, Q^T in registers;
//     mask    the lane's query word of the mask: bit (s & 31) of word s / 32;
//     softmax each lane owns one query and 16 keys of a 32-key block; online max/sum in the exp2
//             domain, rescale of O only when the running max grows by more than 2^8;
//     PV      O^T[128 d][32 queries] += V^T . P^T: V^T through the transposing LDS read, P^T straight
//             from the softmax registers (the key order inside one instruction is the same permutation
//             on both operands).
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kMD = 192;                    // d_qk of the fast path
constexpr int kMV = 128;                    // d_v of the fast path
constexpr int kMBK = 64;                    // keys per tile
constexpr int kMhaQB = 1;  // 32-query blocks per wave (128 QB queries per workgroup); two blocks
                           // would halve the LDS reads per flop but exceed the register file
constexpr int kKTile = kMBK * kMD * 2;      // 24576 B
constexpr int kVTile = kMBK * kMV * 2;      // 16384 B
constexpr int kKCopies = kKTile / 1024 / 4;  // 6 copies of 1 KiB per wave
constexpr int kVCopies = kVTile / 1024 / 4;  // 4
constexpr float kLog2eM = 1.4426950408889634f;
constexpr float kLn2M = 0.6931471805599453f;
constexpr float kRescaleM = 8.0f;

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane sources of this wave's tile copies: packed (row << 10) | byte offset inside the row.
struct TileSrc {
  int k[kKCopies];
  int v[kVCopies];
};

__device__ __forceinline__ TileSrc tile_sources(int wave, int lane) {
  TileSrc t;
#pragma unroll
  for (int i = 0; i < kKCopies; i++) {
    const int slot = (kKCopies * wave + i) * 64 + lane;  // 24 chunks of 16 B per K row
    const int r = slot / 24, cs = slot % 24;
    t.k[i] = (r << 10) | ((cs ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < kVCopies; i++) {
    const int slot = (kVCopies * wave + i) * 64 + lane;  // 16 chunks per V row
    const int r = slot >> 4, cs = slot & 15;
    t.v[i] = (r << 10) | ((cs ^ ((r & 3) << 2)) << 4);
  }
  return t;
}

// Copies of key tile j of head h into (kt, vt); rows past the last key re-read the last key.
__device__ __forceinline__ void issue_tile(const char* __restrict__ kh, const char* __restrict__ vh, size_t row_k,
                                           size_t row_v, int j, int n_kv, const TileSrc& src, char* kt, char* vt,
                                           int wave) {
  const int s0 = j * kMBK;
#pragma unroll
  for (int i = 0; i < kKCopies; i++) {
    const int s = min(s0 + (src.k[i] >> 10), n_kv - 1);
    __builtin_amdgcn_global_load_lds((const void*)(kh + (size_t)s * row_k + (src.k[i] & 1023)),
                                     (lds_void_t*)(kt + (kKCopies * wave + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kVCopies; i++) {
    const int s = min(s0 + (src.v[i] >> 10), n_kv - 1);
    __builtin_amdgcn_global_load_lds((const void*)(vh + (size_t)s * row_v + (src.v[i] & 1023)),
                                     (lds_void_t*)(vt + (kVCopies * wave + i) * 1024), 16, 0, 0);
  }
}

struct MhaState {
  float m;  // running max, log2 units (scaled)
  float l;  // running sum
};

// V^T fragments of one 16-key half (rows r0 .. r0+15 of the tile) for the four 32-column blocks:
// eight transposing reads completed inside the block.
typedef short v4s_m __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_m lds_v4s_m;
__device__ __forceinline__ void vt_frags(const char* vt, const int (&voff)[4], int r0, u32x2 (&vr)[4][2]) {
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int rd = 0; rd < 2; rd++)
      vr[db][rd] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_v4s_m*)(lds_void_t*)(vt + voff[db] + r0 * 256 + 2048 * rd)));
}

// One key tile for this wave's QB x 32 queries (query block qb: queries 32qb + l%32 of the wave's).
template <int QB>
__device__ __forceinline__ void compute_tile(const char* kt, const char* vt, const uint32_t (&mw)[QB][2],
                                             const v8bf (&qf)[QB][kMD / 16], const int (&koff)[4],
                                             const int (&voff)[4], v16f (&o)[QB][4], MhaState (&st)[QB],
                                             float c_scale, int lane) {
  // no selected key for any of this wave's queries in the tile: nothing to do
  uint32_t any_w = 0u;
#pragma unroll
  for (int qb = 0; qb < QB; qb++) any_w |= mw[qb][0] | mw[qb][1];
  if (__ballot(any_w != 0u) == 0ull) return;

  v16f sacc[QB][2];
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
#pragma unroll
    for (int ks = 0; ks < kMD / 16; ks++) {
      const v8bf kf = *(const v8bf*)(kt + koff[ks & 3] + 128 * (ks >> 2) + kb * 32 * (kMD * 2));
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        if (ks == 0)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][0], (v16f){}, 0, 0, 0);
        else
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], sacc[qb][kb], 0, 0, 0);
      }
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // at most 4 K fragments in flight
    }
  }
  // mask, then the online softmax of this lane's queries over the tile's 64 keys (32 here, 32 in lane
  // l ^ 32).  Value r of block kb is key 32kb + 8(r/4) + 4(l/32) + r%4.  Scores stay unscaled until
  // the exponent (c_scale > 0 keeps the maximum).
  const int kk0 = 4 * (lane >> 5);
  unsigned int pk[QB][2][8];
  float alpha[QB];
  bool rescale = false;
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    float bm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (__ballot(mw[qb][kb] != 0xFFFFFFFFu) != 0ull) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int kk = 8 * (r >> 2) + kk0 + (r & 3);
          sacc[qb][kb][r] = ((mw[qb][kb] >> kk) & 1u) ? sacc[qb][kb][r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r++) bm = fmaxf(bm, sacc[qb][kb][r]);
    }
    bm = xor32_max(bm) * c_scale;
    alpha[qb] = 1.f;
    if (bm > st[qb].m + kRescaleM) {
      alpha[qb] = __builtin_amdgcn_exp2f(st[qb].m - bm);  // 0 while m = -inf
      st[qb].m = bm;
    }
    rescale |= alpha[qb] != 1.f;
    const float neg_m = (st[qb].m == -INFINITY) ? 0.f : -st[qb].m;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int g = 0; g < 8; g++) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][2 * g], c_scale, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][2 * g + 1], c_scale, neg_m));
        psum += p0 + p1;
        pk[qb][kb][g] = pack_bf16x2(p0, p1);
      }
    st[qb].l = st[qb].l * alpha[qb] + xor32_sum(psum);
  }
  if (__ballot(rescale) != 0ull) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) o[qb][db][r] *= alpha[qb];
  }

  // PV: four 16-key halves, four 32-column blocks each; every V^T fragment serves all query blocks
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int kh = 0; kh < 2; kh++) {
      __builtin_amdgcn_sched_barrier(0);
      u32x2 vr[4][2];
      vt_frags(vt, voff, 32 * kb + 16 * kh, vr);
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        const v8bf pf = __builtin_bit_cast(v8bf, (u32x4){pk[qb][kb][4 * kh], pk[qb][kb][4 * kh + 1],
                                                         pk[qb][kb][4 * kh + 2], pk[qb][kb][4 * kh + 3]});
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const v8bf vf =
              __builtin_bit_cast(v8bf, (u32x4){vr[db][0][0], vr[db][0][1], vr[db][1][0], vr[db][1][1]});
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[qb][db], 0, 0, 0);
        }
      }
    }
}

template <int QB>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void mha_masked_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint32_t* __restrict__ mask, int n_q, int n_kv,
                                                            int H, int W, float sm_scale, int n_qt,
                                                            uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char kt0[kKTile];
  __shared__ __attribute__((aligned(1024))) char kt1[kKTile];
  __shared__ __attribute__((aligned(1024))) char vt0[kVTile];
  __shared__ __attribute__((aligned(1024))) char vt1[kVTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = n_qt - 1 - (int)blockIdx.x / H;  // longest query tiles first
  const int h = (int)blockIdx.x % H;
  const int b = blockIdx.y;
  constexpr int kQ = 128 * QB;  // queries per workgroup
  const int t0 = qt * kQ;
  const int t_last = min(t0 + kQ - 1, n_q - 1);
  const int pos_last = n_kv - n_q + t_last;
  const int n_tiles = pos_last / kMBK + 1;

  // Q^T fragments: query block qb of lane l is query t0 + 32(QB w + qb) + l%32, dims 16ks + 8(l/32) .. +8
  v8bf qf[QB][kMD / 16];
  const uint32_t* mrow[QB];
  int tq_[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int t = t0 + 32 * (QB * wave + qb) + (lane & 31);
    tq_[qb] = t;
    const size_t qrow = (size_t)b * n_q + min(t, n_q - 1);
    const uint16_t* qp = q + (qrow * H + h) * kMD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kMD / 16; ks++) qf[qb][ks] = *(const v8bf*)(qp + 16 * ks);
    mrow[qb] = mask + qrow * W;
  }

  // fragment offsets inside a tile (see the header: swizzled 16-byte chunks)
  int koff[4], voff[4];
  {
    const int r = lane & 31;
#pragma unroll
    for (int a = 0; a < 4; a++) koff[a] = r * (kMD * 2) + 16 * ((2 * a + (lane >> 5)) ^ ((r >> 1) & 7));
    const int G = lane >> 4, j = lane & 15;
    const int base = (4 * (G >> 1) + (j >> 2)) * (kMV * 2) + 32 * (G & 1) + 8 * (j & 3);
#pragma unroll
    for (int db = 0; db < 4; db++) voff[db] = base + 64 * (db ^ (j >> 2));
  }
  const TileSrc src = tile_sources(wave, lane);
  const size_t row_k = (size_t)H * kMD * 2, row_v = (size_t)H * kMV * 2;
  const char* kh = (const char*)k + ((size_t)b * n_kv * H + h) * (kMD * 2);
  const char* vh = (const char*)v + ((size_t)b * n_kv * H + h) * (kMV * 2);

  v16f o[QB][4];
  MhaState st[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int r = 0; r < 16; r++) o[qb][db][r] = 0.f;
    st[qb] = MhaState{-INFINITY, 0.f};
  }
  const float c_scale = sm_scale * kLog2eM;

  // The query side is complete before the first copy is issued, so the waits below only ever cover
  // tile copies and mask words.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  uint32_t mw0[QB][2], mw1[QB][2];
  auto load_mask = [&](uint32_t (&mw)[QB][2], int j) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      mw[qb][0] = mrow[qb][2 * j];
      mw[qb][1] = mrow[qb][2 * j + 1];
    }
  };
  issue_tile(kh, vh, row_k, row_v, 0, n_kv, src, kt0, vt0, wave);
  load_mask(mw0, 0);
  wait_vm0();
  barrier_lds();
  // Two tiles per round, buffer 0 then buffer 1.  Copies are unconditional (past the last tile they
  // re-read the last one into the free buffer) and so are the mask loads (clamped to the last tile).
  for (int j = 0; j < n_tiles; j += 2) {
    const int j1 = min(j + 1, n_tiles - 1);
    issue_tile(kh, vh, row_k, row_v, j1, n_kv, src, kt1, vt1, wave);
    load_mask(mw1, j1);
    compute_tile<QB>(kt0, vt0, mw0, qf, koff, voff, o, st, c_scale, lane);
    wait_vm0();
    barrier_lds();
    const int j2 = min(j + 2, n_tiles - 1);
    issue_tile(kh, vh, row_k, row_v, j2, n_kv, src, kt0, vt0, wave);
    load_mask(mw0, j2);
    if (j + 1 < n_tiles) compute_tile<QB>(kt1, vt1, mw1, qf, koff, voff, o, st, c_scale, lane);
    wait_vm0();
    barrier_lds();
  }

#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int t = tq_[qb];
    if (t < n_q) {
      const float inv = st[qb].l > 0.f ? 1.f / st[qb].l : 0.f;
      uint16_t* op = out + (((size_t)b * n_q + t) * H + h) * kMV + 4 * (lane >> 5);
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          u32x2 w2;
          w2[0] = pack_bf16x2(o[qb][db][4 * qd + 0] * inv, o[qb][db][4 * qd + 1] * inv);
          w2[1] = pack_bf16x2(o[qb][db][4 * qd + 2] * inv, o[qb][db][4 * qd + 3] * inv);
          *(u32x2*)(op + 32 * db + 8 * qd) = w2;
        }
      if (lse != nullptr && lane < 32)
        lse[((size_t)b * n_q + t) * H + h] = st[qb].l > 0.f ? (st[qb].m + log2f(st[qb].l)) * kLn2M : -INFINITY;
    }
  }
}

// One workgroup per (query row, sequence): the row's bits in LDS, then written out whole.
__global__ __launch_bounds__(256) void mha_mask_kernel(const int32_t* __restrict__ idx, int n_q, int n_kv, int k_sel,
                                                       int W, uint32_t* __restrict__ mask) {
  extern __shared__ uint32_t words[];
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * n_q + t;
  const int pos = n_kv - n_q + t;
  for (int i = threadIdx.x; i < W; i += 256) words[i] = 0u;
  __syncthreads();
  const int32_t* sel = idx + row * k_sel;
  // eight entries per thread and round, all loads in flight before the first is used
  for (int e0 = 0; e0 < k_sel; e0 += 8 * 256) {
    int sv[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int e = e0 + 256 * u + (int)threadIdx.x;
      sv[u] = e < k_sel ? sel[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (sv[u] >= 0 && sv[u] <= pos) atomicOr(&words[sv[u] >> 5], 1u << (sv[u] & 31));
  }
  __syncthreads();
  uint32_t* mrow = mask + row * W;
  for (int i = threadIdx.x; i < W; i += 256) mrow[i] = words[i];
}

}  // namespace

int mha_mask_words(int n_kv) { return 2 * ((n_kv + kMBK - 1) / kMBK); }

hipError_t launch_masked_mha(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx, int B,
                             int n_q, int n_kv, int H, int k_sel, float sm_scale, uint16_t* out, float* lse,
                             uint32_t* mask, hipStream_t stream) {
  const int W = mha_mask_words(n_kv);
  hipLaunchKernelGGL(mha_mask_kernel, dim3(n_q, B), dim3(256), (size_t)W * 4, stream, idx, n_q, n_kv, k_sel, W, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int QB = kMhaQB;
  const int n_qt = (n_q + 128 * QB - 1) / (128 * QB);
  hipLaunchKernelGGL(mha_masked_kernel<QB>, dim3(n_qt * H, B), dim3(256), 0, stream, q, k, v, (const uint32_t*)mask,
                     n_q, n_kv, H, W, sm_scale, n_qt, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
