// indexer.hip -- lightning-indexer scores on gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over s <= pos_t (velog summary "DeepSeek-V3.2:
// Pushing the Frontier of Open Large Language Models", section 1.1; few indexer heads in FP8).
//
// Fast path (H_I = 64, d_I = 128, e4m3 inputs): the 64 heads of one query form the M dimension of
// the 16x16x128 FP8 matrix-core instruction (4 row blocks of 16 heads), 16 keys form N, and the
// whole d_I = 128 is one instruction's K.  With scales positive, ReLU commutes with them, so the
// epilogue is  k_scale[s] * sum_h (w * q_scale)[h] * max(acc[h,s], 0).  Each lane owns 4 heads of
// every row block for one key column, so the head sum is 16 lane-local FMAs followed by two
// cross-lane adds (lane ^ 16, lane ^ 32).  The per-head [H_I, T, S] products are never stored.
//
// Work decomposition: one wave = QW consecutive queries x a range of keys, streamed in groups of
// 64 keys (4 MFMA column blocks) with the next group's keys loaded while the current one is
// computed.  Prefill: one range = the whole causal row, longest rows dispatched first.  Decode
// (one query per sequence): the row is split into chunks so that thousands of waves stream keys.
#include "dsa_internal.h"

#include <type_traits>

namespace dsa {

// ------------------------------------------------------------------------------------------------
// Generic kernel: any H_I <= 64, d_I <= 256; fp32 or e4m3 inputs.  One workgroup per query row; the
// query (dequantised exactly like the definition: fp32(e4m3 * scale)) and its weights sit in LDS.
// ------------------------------------------------------------------------------------------------
template <bool FP8>
__global__ __launch_bounds__(256) void indexer_generic_kernel(const void* __restrict__ q_,
                                                              const float* __restrict__ q_scale,
                                                              const void* __restrict__ k_,
                                                              const float* __restrict__ k_scale,
                                                              const float* __restrict__ w, int n_q, int n_kv,
                                                              int H_I, int d_I, float* __restrict__ scores,
                                                              int64_t ld) {
  extern __shared__ float smem[];
  float* qs = smem;              // [H_I][d_I]
  float* ws = smem + H_I * d_I;  // [H_I]
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t qrow = (size_t)b * n_q + t;
  for (int e = threadIdx.x; e < H_I * d_I; e += blockDim.x) {
    float v;
    if (FP8) {
      const uint8_t* q8 = (const uint8_t*)q_ + qrow * H_I * d_I;
      v = e4m3_to_f32(q8[e]) * q_scale[qrow * H_I + e / d_I];
    } else {
      v = ((const float*)q_)[qrow * H_I * d_I + e];
    }
    qs[e] = v;
  }
  for (int j = threadIdx.x; j < H_I; j += blockDim.x) ws[j] = w[qrow * H_I + j];
  __syncthreads();
  const int pos = n_kv - n_q + t;
  for (int s = threadIdx.x; s <= pos; s += blockDim.x) {
    const size_t krow = (size_t)b * n_kv + s;
    float kscale = FP8 ? k_scale[krow] : 1.0f;
    float acc = 0.0f;
    for (int j = 0; j < H_I; j++) {
      float dot = 0.0f;
      for (int i = 0; i < d_I; i++) {
        float kv;
        if (FP8)
          kv = e4m3_to_f32(((const uint8_t*)k_)[krow * d_I + i]) * kscale;
        else
          kv = ((const float*)k_)[krow * d_I + i];
        dot = fmaf(qs[j * d_I + i], kv, dot);
      }
      acc = fmaf(ws[j], fmaxf(dot, 0.0f), acc);
    }
    scores[qrow * ld + s] = acc + 0.0f;
  }
}

hipError_t launch_indexer_generic(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                  const float* w, int B, int n_q, int n_kv, int H_I, int d_I, bool fp8,
                                  float* scores, int64_t ld, hipStream_t stream) {
  dim3 grid(n_q, B);
  size_t lds = (size_t)(H_I * d_I + H_I) * sizeof(float);
  if (fp8)
    hipLaunchKernelGGL(indexer_generic_kernel<true>, grid, dim3(256), lds, stream, q, q_scale, k, k_scale, w,
                       n_q, n_kv, H_I, d_I, scores, ld);
  else
    hipLaunchKernelGGL(indexer_generic_kernel<false>, grid, dim3(256), lds, stream, q, q_scale, k, k_scale, w,
                       n_q, n_kv, H_I, d_I, scores, ld);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// FP8 matrix-core kernel, H_I = 64, d_I = 128.
// ------------------------------------------------------------------------------------------------
constexpr int kHI = 64;
constexpr int kDI = 128;

__device__ __forceinline__ v4f mfma_f8_16x16x128(v8i a, v8i b) {
  v4f c = {0.f, 0.f, 0.f, 0.f};
  // Scale operands 0 select the unscaled instruction (v_mfma_f32_16x16x128_f8f6f4, e4m3 x e4m3).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One group = 64 keys = 4 column blocks of 16.  Lane l loads key (16*j + l%16), bytes 32*(l/16)..+32
// of column block j: the matrix-core B-operand layout; with it, the scale of key g0 + l.  Keys past the
// end are clamped (their scores are never stored).
struct KeyGroup {
  v8i kf[4];
  float ksc;
};

// STREAM: the keys are read once (decode), so the loads are nontemporal; prefill keys are shared by
// every query row and stay cacheable.
template <bool STREAM>
__device__ __forceinline__ void load_key_group(const uint8_t* __restrict__ kb, const float* __restrict__ ksb, int g0,
                                               int n_kv, int lane, KeyGroup& g) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int s = min(g0 + 16 * j + (lane & 15), n_kv - 1);
    const v8i* p = (const v8i*)(kb + (size_t)s * kDI + (lane >> 4) * 32);
    g.kf[j] = STREAM ? __builtin_nontemporal_load(p) : *p;
  }
  const float* ps = ksb + min(g0 + lane, n_kv - 1);
  g.ksc = STREAM ? __builtin_nontemporal_load(ps) : *ps;
}

// max(x, 0) as one integer max on the bit pattern: every negative float (and -0) has the sign bit set
// and compares below 0, the rest are unchanged.  (fmaxf costs two instructions here: the IEEE mode
// canonicalises its input first.)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of one key group for the wave's QW queries: afterwards lane l holds in out[qi] the score of
// key g0 + l for query qi.
template <int QW>
__device__ __forceinline__ void key_group_scores(const KeyGroup& g, const v8i (&qa)[QW][4],
                                                 const float (&ww)[QW][4][4], float (&out)[QW]) {
  // part[qi][j]: this lane's share (its 16 heads) of the score of key 16j + l%16
  float part[QW][4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    v4f acc[QW][4];
#pragma unroll
    for (int qi = 0; qi < QW; qi++)
#pragma unroll
      for (int mb = 0; mb < 4; mb++) acc[qi][mb] = mfma_f8_16x16x128(qa[qi][mb], g.kf[j]);
#pragma unroll
    for (int qi = 0; qi < QW; qi++) {
      float v = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 4; mb++)
#pragma unroll
        for (int r = 0; r < 4; r++) v = fmaf(ww[qi][mb][r], relu_bits(acc[qi][mb][r]), v);
      part[qi][j] = v;
    }
  }
  // Reduce-scatter over the four 16-lane rows: afterwards lane l holds the full score of key 16(l/16)
  // + l%16 = l.  Step 1 (lanes l, l^32): the lower half keeps blocks 0 and 1, the upper half 2 and 3;
  // step 2 (lanes l, l^16): rows keep block row.  Each swap-and-add is one permlane swap and one add.
#pragma unroll
  for (int qi = 0; qi < QW; qi++) {
    // permlane32_swap(a, b) trades the upper 32 lanes of a with the lower 32 lanes of b, so the lower
    // half ends with (a, partner's a) and the upper half with (partner's b, b); permlane16_swap does
    // the same between the odd rows of a and the even rows of b.
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qi][0]), __float_as_uint(part[qi][2]),
                                                      false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qi][1]), __float_as_uint(part[qi][3]),
                                                      false, false);
    const float ra = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // block 0 (lower) / 2 (upper)
    const float rb = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // block 1 (lower) / 3 (upper)
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(ra), __float_as_uint(rb), false, false);
    out[qi] = (__uint_as_float(s[0]) + __uint_as_float(s[1])) * g.ksc + 0.0f;  // + 0 maps -0 to +0
  }
}

// Scores of one key group, stored straight to the score rows: lane l stores key g0 + l.
template <int QW>
__device__ __forceinline__ void score_key_group(const KeyGroup& g, const v8i (&qa)[QW][4],
                                                const float (&ww)[QW][4][4], int g0, int s_end, int pos0,
                                                int nq_here, int lane, float* __restrict__ srow, int64_t ld) {
  float out[QW];
  key_group_scores<QW>(g, qa, ww, out);
  const int s = g0 + lane;
  if (s < s_end) {
#pragma unroll
    for (int qi = 0; qi < QW; qi++)
      if (qi < nq_here && s <= pos0 + qi) srow[(size_t)qi * ld + s] = out[qi];
  }
}

// Decode key groups are read contiguously: load u of lane l brings bytes 16(l%8) .. +16 of key g0 + 8u + l/8,
// so every wave-wide load covers 1 KiB of whole 128-byte rows (the operand layout, 32 bytes of one key per
// lane, touches each row in half-line pieces and streams about 12 % slower).  Each 16-key block is then
// turned into the matrix-core layout through a per-wave LDS slot: 16-byte chunk c of row r at chunk
// c ^ ((r >> 1) & 7), so both the contiguous writes and the operand reads hit every bank once.
struct RawGroup {
  u32x4 r[8];
  float ksc;
};
__device__ __forceinline__ void load_raw_group(const uint8_t* __restrict__ kb, const float* __restrict__ ksb, int g0,
                                               int n_kv, int lane, RawGroup& g) {
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int s = min(g0 + 8 * u + (lane >> 3), n_kv - 1);
    g.r[u] = __builtin_nontemporal_load((const u32x4*)(kb + (size_t)s * kDI + (lane & 7) * 16));
  }
  g.ksc = __builtin_nontemporal_load(ksb + min(g0 + lane, n_kv - 1));
}
// Blocks 2h and 2h+1 of a raw group into kf[2h], kf[2h+1] through the wave's 4 KiB slot `tr`.
__device__ __forceinline__ void transpose_pair(const RawGroup& g, int h, char* tr, int lane, KeyGroup& kg) {
#pragma unroll
  for (int q = 0; q < 4; q++) {  // load 4h + q: rows 8q .. 8q+7 of the 32-row pair slot
    const int r = 8 * q + (lane >> 3), c = lane & 7;
    *(u32x4*)(tr + r * 128 + 16 * (c ^ ((r >> 1) & 7))) = g.r[4 * h + q];
  }
#pragma unroll
  for (int jj = 0; jj < 2; jj++) {
    const int r = 16 * jj + (lane & 15), c0 = 2 * (lane >> 4);
    const u32x4 lo = *(const u32x4*)(tr + r * 128 + 16 * (c0 ^ ((r >> 1) & 7)));
    const u32x4 hi = *(const u32x4*)(tr + r * 128 + 16 * ((c0 + 1) ^ ((r >> 1) & 7)));
    kg.kf[2 * h + jj] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

// One query per wave (decode) stages its scores in LDS and writes them out after its last key load.
// Stores count in the same counter as loads and their acknowledgements come back slowly under a full
// read stream, so a store issued per group holds every later wait for the next group's keys: the
// stream then loses its lead and the scoring work stops overlapping it.
constexpr int kStageKeys = 4096;  // keys per wave, at most, when scores are staged (16 KB of LDS)

template <int QW, int NB>
__global__ __launch_bounds__(256, 2) void indexer_fp8_kernel(const uint8_t* __restrict__ q8,
                                                             const float* __restrict__ q_scale,
                                                             const float* __restrict__ w,
                                                             const uint8_t* __restrict__ k8,
                                                             const float* __restrict__ k_scale,
                                                             float* __restrict__ scores, int64_t ld, int B,
                                                             int n_q, int n_kv, int n_qgroups, int n_chunks,
                                                             int chunk_keys, int n_items) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int kc = item % n_chunks;
  const int rest = item / n_chunks;
  const int b = rest % B;
  const int qg = n_qgroups - 1 - rest / B;  // longest rows first
  const int t0 = qg * QW;
  const int nq_here = min(QW, n_q - t0);
  const int pos0 = n_kv - n_q + t0;
  const int pos_last = pos0 + nq_here - 1;
  const int s_begin = kc * chunk_keys;
  if (s_begin > pos_last) return;
  const int s_end = min(pos_last + 1, s_begin + chunk_keys);
  constexpr bool kStaged = QW == 1;  // chunk_keys <= kStageKeys then (checked by the launch)
  __shared__ float stage_all[kStaged ? 4 * kStageKeys : 1];
  float* stage = stage_all + (kStaged ? (threadIdx.x >> 6) * kStageKeys : 0);
  __shared__ __attribute__((aligned(16))) char tr_all[kStaged ? 4 * 4096 : 16];  // decode: transpose slots
  char* tr = tr_all + (kStaged ? (threadIdx.x >> 6) * 4096 : 0);

  const uint8_t* kb = k8 + (size_t)b * n_kv * kDI;
  const float* ksb = k_scale + (size_t)b * n_kv;
  float* srow = scores + ((size_t)b * n_q + t0) * ld;

  // Key loads are unconditional (indexes are clamped into the row, so groups past the range re-read
  // in-bounds keys that are never scored): with no load skipped on any path, each wait below covers
  // exactly the group it needs.
  using Ring = typename std::conditional<kStaged, RawGroup, KeyGroup>::type;
  auto load_group = [&](int g0, Ring& g) {
    if constexpr (kStaged) load_raw_group(kb, ksb, g0, n_kv, lane, g);
    else load_key_group<false>(kb, ksb, g0, n_kv, lane, g);
  };
  Ring ring[NB];
#pragma unroll
  for (int p = 0; p < NB - 1; p++) {
    load_group(s_begin + 64 * p, ring[p]);
    // in issue order, each group's scale right after its keys: the wait for a group's scale then
    // never covers the keys of the group after it
    __builtin_amdgcn_sched_barrier(0);
  }

  // A operands: row block mb holds heads 16*mb .. 16*mb+15; lane l supplies head 16*mb + l%16,
  // bytes 32*(l/16) .. +32 of that head's 128-byte query.
  v8i qa[QW][4];
  float ww[QW][4][4];  // (w * q_scale) of head 16*mb + 4*(l/16) + r: the accumulator rows lane l owns
#pragma unroll
  for (int qi = 0; qi < QW; qi++) {
    const int t = t0 + min(qi, nq_here - 1);
    const size_t qrow = (size_t)b * n_q + t;
    const uint8_t* qp = q8 + qrow * kHI * kDI;
#pragma unroll
    for (int mb = 0; mb < 4; mb++) qa[qi][mb] = *(const v8i*)(qp + (16 * mb + (lane & 15)) * kDI + (lane >> 4) * 32);
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int h = 16 * mb + 4 * (lane >> 4) + r;
        ww[qi][mb][r] = w[qrow * kHI + h] * q_scale[qrow * kHI + h];
      }
  }
  // One wait for the query side and the first key groups together (the key loads were issued first, so
  // the two memory round trips overlap); the loop below then only ever waits for key groups.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // Ring of NB key groups: group i lives in slot i % NB.  The main loop runs whole rounds of NB groups
  // with no early exit (every slot index static, every wait exact); loads for group i + NB - 1 are
  // issued before group i is scored.  The last n_groups % NB groups are already in slots 0.. and are
  // scored after the loop.
  auto score = [&](const Ring& g, int g0) {
    if constexpr (kStaged) {
      KeyGroup kg;
      transpose_pair(g, 0, tr, lane, kg);
      transpose_pair(g, 1, tr, lane, kg);
      kg.ksc = g.ksc;
      float out[1];
      key_group_scores<1>(kg, qa, ww, out);
      stage[g0 - s_begin + lane] = out[0];  // < chunk_keys: groups start inside the chunk
    } else {
      score_key_group<QW>(g, qa, ww, g0, s_end, pos0, nq_here, lane, srow, ld);
    }
  };
  const int n_groups = (s_end - s_begin + 63) / 64;
  int gi = 0;
  for (; gi + NB <= n_groups; gi += NB) {
#pragma unroll
    for (int p = 0; p < NB; p++) {
      const int g0 = s_begin + 64 * (gi + p);
      load_group(g0 + 64 * (NB - 1), ring[(p + NB - 1) % NB]);
      score(ring[p], g0);
      __builtin_amdgcn_sched_barrier(0);  // one group at a time: no loads hoisted across groups
    }
  }
#pragma unroll
  for (int p = 0; p < NB - 1; p++)
    if (gi + p < n_groups) score(ring[p], s_begin + 64 * (gi + p));

  if constexpr (kStaged) {
    // each wave reads back only what it wrote; the fences keep the LDS reads after the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n = s_end - s_begin;
    float* dst = srow + s_begin;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      for (int i = 4 * lane; i < n; i += 256) {
        if (i + 4 <= n) {
          *(v4f*)(dst + i) = *(const v4f*)(stage + i);
        } else {
          for (int e = i; e < n; e++) dst[e] = stage[e];
        }
      }
    } else {
      for (int i = lane; i < n; i += 64) dst[i] = stage[i];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Prefill: one workgroup = 4 waves x 2 queries = 8 consecutive queries that share their keys.  Each
// 64-key group is read from memory once per workgroup (every wave loads a quarter of it into
// registers one group ahead, then writes it to LDS), and every wave takes its matrix-core operands
// from LDS: the cache traffic for keys drops four-fold against one load per wave.
// LDS group layout: 64 rows of 128 B, 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 7), so
// the operand reads (16 rows x one chunk per 16 lanes) hit every bank once; then the 64 scales.
// Two group slots: while group g is scored from one, group g+1 is written into the other; one barrier
// per group.
// ------------------------------------------------------------------------------------------------
constexpr int kGrpKeyBytes = 64 * kDI;
constexpr int kGrpBytes = kGrpKeyBytes + 64 * 4;

__device__ __forceinline__ int chunk_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(256, 2) void indexer_fp8_shared_kernel(const uint8_t* __restrict__ q8,
                                                                    const float* __restrict__ q_scale,
                                                                    const float* __restrict__ w,
                                                                    const uint8_t* __restrict__ k8,
                                                                    const float* __restrict__ k_scale,
                                                                    float* __restrict__ scores, int64_t ld,
                                                                    int n_q, int n_kv, int n_oct) {
  constexpr int QW = 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kGrpBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int o = n_oct - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int t_last = min(8 * o + 7, n_q - 1);
  const int pos_max = n_kv - n_q + t_last;
  const int n_groups = (pos_max + 64) / 64;  // keys 0 .. pos_max
  const int t0 = 8 * o + QW * wave;
  const int nq_here = max(0, min(QW, n_q - t0));  // 0 for the spare waves of the last octet
  const int pos0 = n_kv - n_q + t0;

  const uint8_t* kb = k8 + (size_t)b * n_kv * kDI;
  const float* ksb = k_scale + (size_t)b * n_kv;
  float* srow = scores + ((size_t)b * n_q + min(t0, n_q - 1)) * ld;

  // this wave's quarter of a group: row 16w + l/4, bytes 32 (l%4) .. +32; lane l also loads scale l
  const int st_row = 16 * wave + (lane >> 2);
  const int st_c = 2 * (lane & 3);
  auto stage_load = [&](int g, v8i& kv, float& sc) {
    const int r = min(64 * g + st_row, n_kv - 1);
    kv = *(const v8i*)(kb + (size_t)r * kDI + st_c * 16);
    sc = ksb[min(64 * g + lane, n_kv - 1)];
  };
  auto stage_store = [&](int slot, const v8i& kv, float sc) {
    unsigned char* base = lds[slot] + st_row * kDI;
    *(u32x4*)(base + (chunk_slot(st_row, st_c) << 4)) = (u32x4){(unsigned)kv[0], (unsigned)kv[1], (unsigned)kv[2],
                                                                (unsigned)kv[3]};
    *(u32x4*)(base + (chunk_slot(st_row, st_c + 1) << 4)) =
        (u32x4){(unsigned)kv[4], (unsigned)kv[5], (unsigned)kv[6], (unsigned)kv[7]};
    if (wave == 0) ((float*)(lds[slot] + kGrpKeyBytes))[lane] = sc;
  };

  // A operands and head weights of this wave's two queries (clamped to a valid row; spare waves
  // compute on it and store nothing)
  v8i qa[QW][4];
  float ww[QW][4][4];
#pragma unroll
  for (int qi = 0; qi < QW; qi++) {
    const int t = min(t0 + qi, n_q - 1);
    const size_t qrow = (size_t)b * n_q + t;
    const uint8_t* qp = q8 + qrow * kHI * kDI;
#pragma unroll
    for (int mb = 0; mb < 4; mb++) qa[qi][mb] = *(const v8i*)(qp + (16 * mb + (lane & 15)) * kDI + (lane >> 4) * 32);
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int h = 16 * mb + 4 * (lane >> 4) + r;
        ww[qi][mb][r] = w[qrow * kHI + h] * q_scale[qrow * kHI + h];
      }
  }

  v8i stg;
  float stg_sc;
  stage_load(0, stg, stg_sc);
  stage_store(0, stg, stg_sc);
  stage_load(1, stg, stg_sc);
  __syncthreads();

  // operand reads: block j, lane l: row 16j + l%16, chunks 2(l/16) and 2(l/16)+1
  const int fr_c = 2 * (lane >> 4);
  for (int g = 0; g < n_groups; g++) {
    const int cur = g & 1;
    stage_store(cur ^ 1, stg, stg_sc);  // group g+1 (its slot was last read in step g-1)
    stage_load(g + 2, stg, stg_sc);     // rows clamped: past the end it re-reads in-bounds keys
    KeyGroup kg;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int r = 16 * j + (lane & 15);
      const unsigned char* rowp = lds[cur] + r * kDI;
      const u32x4 lo = *(const u32x4*)(rowp + (chunk_slot(r, fr_c) << 4));
      const u32x4 hi = *(const u32x4*)(rowp + (chunk_slot(r, fr_c + 1) << 4));
      kg.kf[j] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    kg.ksc = ((const float*)(lds[cur] + kGrpKeyBytes))[lane];
    if (nq_here > 0)
      score_key_group<QW>(kg, qa, ww, 64 * g, pos0 + nq_here, pos0, nq_here, lane, srow, ld);
    __syncthreads();
  }
}

hipError_t launch_indexer_fp8(const uint8_t* q, const float* q_scale, const uint8_t* k, const float* k_scale,
                              const float* w, int B, int n_q, int n_kv, float* scores, int64_t ld,
                              int keys_per_wave, hipStream_t stream) {
  if (n_q >= 8 && keys_per_wave <= 0) {
    const int n_oct = (n_q + 7) / 8;
    hipLaunchKernelGGL(indexer_fp8_shared_kernel, dim3(n_oct, B), dim3(256), 0, stream, q, q_scale, w, k, k_scale,
                       scores, ld, n_q, n_kv, n_oct);
  } else if (n_q >= 2) {
    constexpr int QW = 2;
    const int n_qgroups = (n_q + QW - 1) / QW;
    const int chunk = keys_per_wave > 0 ? ((keys_per_wave + 63) / 64) * 64 : ((n_kv + 63) / 64) * 64;
    const int n_chunks = (n_kv + chunk - 1) / chunk;
    const long long items = (long long)B * n_qgroups * n_chunks;
    if (items > (1LL << 30)) return hipErrorInvalidValue;
    const int blocks = (int)((items + 3) / 4);
    hipLaunchKernelGGL((indexer_fp8_kernel<QW, 2>), dim3(blocks), dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, scores, ld, B, n_q, n_kv, n_qgroups, n_chunks, chunk, (int)items);
  } else {
    constexpr int QW = 1;
    const int n_qgroups = n_q;
    int chunk = keys_per_wave;
    if (chunk <= 0) {
      // one round of waves that streams from every CU: 2048 waves, 8 per CU (two workgroups at this
      // kernel's register count)
      long long waves_per_row = (2048 + (long long)B * n_q - 1) / ((long long)B * n_q);
      chunk = (int)((n_kv + waves_per_row - 1) / waves_per_row);
      chunk = chunk < 512 ? 512 : chunk;
    }
    chunk = ((chunk + 63) / 64) * 64;
    chunk = chunk < kStageKeys ? chunk : kStageKeys;  // the staged scores of one wave fit its LDS slice
    const int n_chunks = (n_kv + chunk - 1) / chunk;
    const long long items = (long long)B * n_qgroups * n_chunks;
    if (items > (1LL << 30)) return hipErrorInvalidValue;
    const int blocks = (int)((items + 3) / 4);
    hipLaunchKernelGGL((indexer_fp8_kernel<QW, 3>), dim3(blocks), dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, scores, ld, B, n_q, n_kv, n_qgroups, n_chunks, chunk, (int)items);
  }
  return hipGetLastError();
}

}  // namespace dsa
