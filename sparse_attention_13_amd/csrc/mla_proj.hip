// mla_proj.hip -- the dense products on either side of MQA-mode attention (velog summary "DeepSeek-V3.2:
// Pushing the Frontier of Open Large Language Models", section 1.3: MLA in MQA mode shares every latent
// entry across the query heads, which needs the key up-projection absorbed into the query and the value
// up-projection applied to the latent attention output):
//   absorb   q'[r][h] = [ W_UK,h^T q_nope[r][h] ; q_rope[r][h] ]   (d_nope = 128 -> d_c = 512, rope 64 copied)
//   out      o[r][h]  = W_UV,h o'[r][h]                            (d_c = 512 -> d_v = 128)
// Both are per-head products C = A . W^T with the weights stored row-major as [N][K] (so both matrix-core
// operands are contiguous along K), bf16 in, fp32 accumulation, bf16 out.
//
// Kernel: one workgroup of 4 waves per (128 rows, 128 output columns, head), the column tiles of one row
// tile on one XCD (shared A rows in one L2); K in steps of 32.  A and W
// tiles ([128][32] bf16 each, 8 KiB) are copied HBM/L2 -> LDS with global_load_lds_dwordx4 into two
// buffers (separate LDS objects: reads of one never wait for copies into the other), 16-byte chunks
// XOR-swizzled by (row >> 2) & 3 so that the fragment reads hit every bank once.  Wave w computes the
// 64x64 block (w & 1, w >> 1) as 2x2 32x32x16 bf16 instructions per 16 of K, accumulating C^T (so each
// lane holds four consecutive output columns of one row).  The result is staged through LDS and written
// as whole 256-byte row segments.  The four column-tile blocks of a row tile also copy the rope part of
// the query, 32 rows each.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kPB = 128;            // rows and columns per workgroup tile
constexpr int kPK = 32;             // K per step
constexpr int kPTile = kPB * kPK * 2;  // 8192 B; the four tile buffers (32 KiB) also stage the C tile

typedef __attribute__((address_space(3))) void lds_void_p;

__device__ __forceinline__ void wait_vmem0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copies of one K step: A rows m0.. (clamped to M-1), W rows n0..; copy i of wave w fills LDS slots
// (2w + i) * 64 + lane = (row, chunk'), fetching global chunk chunk' ^ ((row >> 2) & 3).
__device__ __forceinline__ void issue_step(const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ w,
                                           int K, int m0, int M, int n0, int k0, char* at, char* wt, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int slot = (2 * wave + i) * 64 + lane;
    const int r = slot >> 2, c = (slot & 3) ^ ((r >> 2) & 3);
    const int m = min(m0 + r, M - 1);
    __builtin_amdgcn_global_load_lds((const void*)(a + m * lda + k0 + 8 * c), (lds_void_p*)(at + (2 * wave + i) * 1024),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(w + (int64_t)(n0 + r) * K + k0 + 8 * c),
                                     (lds_void_p*)(wt + (2 * wave + i) * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void mma_step(const char* at, const char* wt, const int (&frag)[2], int wave,
                                         v16f (&acc)[2][2]) {
  const int am = 64 * (wave & 1), wn = 64 * (wave >> 1);
#pragma unroll
  for (int ks = 0; ks < 2; ks++) {
    v8bf af[2], wf[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      af[i] = *(const v8bf*)(at + (am + 32 * i) * 64 + frag[ks]);
      wf[i] = *(const v8bf*)(wt + (wn + 32 * i) * 64 + frag[ks]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], af[mb], acc[nb][mb], 0, 0, 0);
  }
}

// C[m][n] = sum_k A[m][k] W[n][k] for one head; A row m at a + m*lda, W [N][K], C row m at c + m*ldc.
// Optionally copies rope[m][0..64) to c + m*ldc + N (with rope: N = 4 kPB and n_rope = 64, the 128-byte
// rope row split over the four column-tile blocks as 32 rows each).
__global__ __launch_bounds__(256, 4) void proj_gemm_kernel(const uint16_t* __restrict__ a, int64_t lda, int64_t a_head,
                                                        const uint16_t* __restrict__ w, int64_t w_head,
                                                        uint16_t* __restrict__ c, int64_t ldc, int64_t c_head, int M,
                                                        int N, int K, const uint16_t* __restrict__ rope,
                                                        int n_rope, int n_mh) {
  __shared__ __attribute__((aligned(1024))) char tiles[4][kPTile];
  char* at0 = tiles[0];
  char* at1 = tiles[1];
  char* wt0 = tiles[2];
  char* wt1 = tiles[3];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Consecutive workgroups go to the 8 XCDs in turn, each with its own L2.  Workgroup b runs on XCD b % 8:
  // the column tiles of one (row tile, head) all get the same b % 8, so its A rows come through one L2.
  const int nt = N / kPB;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int mh = (slot / nt) * 8 + xcd;  // (row tile, head) index
  if (mh >= n_mh) return;
  const int m_tiles = (M + kPB - 1) / kPB;
  const int n0 = (slot % nt) * kPB, m0 = (mh % m_tiles) * kPB, h = mh / m_tiles;
  const uint16_t* ah = a + h * a_head;
  const uint16_t* wh = w + h * w_head;
  // The rope part (64 columns = 128 B per row) is copied by the four column-tile blocks of a row tile,
  // 32 rows each: one 16-byte chunk per thread, loaded here so that the load is in flight under the
  // product and stored after the C tile.
  const bool do_rope = rope != nullptr;
  const int rope_row = (slot % nt) * (kPB / 4) + (threadIdx.x >> 3), rope_ck = threadIdx.x & 7;
  u32x4 rp = {0u, 0u, 0u, 0u};
  if (do_rope && m0 + rope_row < M) rp = *(const u32x4*)(rope + h * a_head + (int64_t)(m0 + rope_row) * lda + 8 * rope_ck);

  // fragment offset inside a row of a tile for each 16-wide half of the K step: row l%32 of the block,
  // logical chunk 2ks + l/32, stored at chunk ^ ((row >> 2) & 3)
  int frag[2];
  {
    const int r = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) frag[ks] = r * 64 + 16 * ((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3));
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  const int n_steps = K / kPK;
  issue_step(ah, lda, wh, K, m0, M, n0, 0, at0, wt0, wave, lane);
  wait_vmem0();
  lds_sync();
  for (int s = 0; s < n_steps; s += 2) {
    issue_step(ah, lda, wh, K, m0, M, n0, min(s + 1, n_steps - 1) * kPK, at1, wt1, wave, lane);
    mma_step(at0, wt0, frag, wave, acc);
    wait_vmem0();
    lds_sync();
    issue_step(ah, lda, wh, K, m0, M, n0, min(s + 2, n_steps - 1) * kPK, at0, wt0, wave, lane);
    if (s + 1 < n_steps) mma_step(at1, wt1, frag, wave, acc);
    wait_vmem0();
    lds_sync();
  }

  // stage C (rows m, columns n) in the tile buffers, 256-byte rows with 16-byte chunk c of row r at
  // c ^ (r & 15): the accumulator block [nb][mb] is C^T, lane = row 32mb + l%32 of the wave's block,
  // registers 4q..4q+3 = columns 32nb + 8q + 4(l/32) + 0..3
  char* stage = tiles[0];
  {
    const int am = 64 * (wave & 1), wn = 64 * (wave >> 1);
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      const int row = am + 32 * mb + (lane & 31);
#pragma unroll
      for (int nb = 0; nb < 2; nb++)
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          const int col = wn + 32 * nb + 8 * qd + 4 * (lane >> 5);
          u32x2 v;
          v[0] = pack_bf16x2(acc[nb][mb][4 * qd], acc[nb][mb][4 * qd + 1]);
          v[1] = pack_bf16x2(acc[nb][mb][4 * qd + 2], acc[nb][mb][4 * qd + 3]);
          *(u32x2*)(stage + row * 256 + (((col >> 3) ^ (row & 15)) << 4) + ((col >> 2) & 1) * 8) = v;
        }
    }
  }
  __syncthreads();
  uint16_t* ch = c + h * c_head;
  // 128 rows x 256 B: 16 lanes per row, 16 rows per pass
  for (int i = threadIdx.x; i < kPB * 16; i += 256) {
    const int row = i >> 4, ch16 = i & 15;
    // nontemporal: nothing reads the output back soon (2-3% faster than plain stores)
    if (m0 + row < M)
      __builtin_nontemporal_store(*(const u32x4*)(stage + row * 256 + ((ch16 ^ (row & 15)) << 4)),
                                  (u32x4*)(ch + (int64_t)(m0 + row) * ldc + n0 + 8 * ch16));
  }
  if (do_rope && m0 + rope_row < M)
    __builtin_nontemporal_store(rp, (u32x4*)(ch + (int64_t)(m0 + rope_row) * ldc + N + 8 * rope_ck));
}

}  // namespace

hipError_t launch_mla_absorb_q(const uint16_t* q_mha, const uint16_t* w_ukt, uint16_t* q_mqa, int rows, int H,
                               hipStream_t stream) {
  // A = no-rope query (K = 128) of head h in row r: q_mha + (r*H + h)*192; W = w_ukt[h] [512][128];
  // C = q_mqa + (r*H + h)*576, N = 512; rope (64) from q_mha + 128.
  const int n_mh = (rows + kPB - 1) / kPB * H;
  const dim3 grid((n_mh + 7) / 8 * 8 * (512 / kPB));
  hipLaunchKernelGGL(proj_gemm_kernel, grid, dim3(256), 0, stream, q_mha, (int64_t)H * 192, (int64_t)192, w_ukt,
                     (int64_t)512 * 128, q_mqa, (int64_t)H * 576, (int64_t)576, rows, 512, 128, q_mha + 128, 64, n_mh);
  return hipGetLastError();
}

hipError_t launch_mla_out_proj(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int rows, int H,
                               hipStream_t stream) {
  // A = latent output (K = 512) of head h: o_lat + (r*H + h)*512; W = w_uv[h] [128][512]; C = o + (r*H + h)*128.
  const int n_mh = (rows + kPB - 1) / kPB * H;
  const dim3 grid((n_mh + 7) / 8 * 8 * (128 / kPB));
  hipLaunchKernelGGL(proj_gemm_kernel, grid, dim3(256), 0, stream, o_lat, (int64_t)H * 512, (int64_t)512, w_uv,
                     (int64_t)128 * 512, o, (int64_t)H * 128, (int64_t)128, rows, 128, 512, (const uint16_t*)nullptr,
                     0, n_mh);
  return hipGetLastError();
}

}  // namespace dsa
