// topk.hip -- fine-grained token selection: per query row, the k largest index scores among the
// causal candidates s <= pos_t (velog summary "DeepSeek-V3.2: Pushing the Frontier of Open Large
// Language Models", section 1.2; k = 2048 in the sparse-training stage).
//
// Exact radix select on order-preserving 32-bit keys (-0 folded onto +0), one workgroup per row:
//   * four 8-bit digit passes, most significant first, each building a 256-bin histogram of the
//     keys that share the digits fixed so far, then fixing the digit that holds the k-th largest
//     key; after the fourth pass tau (the k-th largest key) is known, together with how many keys
//     equal to tau must be taken (the lowest positions win ties);
//   * an ordered compaction: every wave owns a contiguous segment of the row, counts its "> tau"
//     and "== tau" keys, a scan over waves gives each its output offset, and the wave writes its
//     selected positions in ascending order (ballot + mbcnt), so the result is sorted by position.
// The histogram has 16 copies (a lane uses copy lane%16) padded to 257 words, which spreads the
// heavy same-bin traffic of the first pass (scores of similar magnitude share their top byte)
// over distinct addresses and banks.
// Rows that fit in LDS (n <= 36736) are read from HBM once and kept as keys in LDS; longer rows
// are re-read from memory in every pass.
#include "dsa_internal.h"

namespace dsa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;
constexpr int kHistWords = kHistCopies * kHistStride;
constexpr int kMiscWords = 64;
constexpr int kLdsBytesMax = 163840;
constexpr int kRowCapMax = ((kLdsBytesMax - (kHistWords + kMiscWords) * 4) / 4) / 64 * 64;  // 36736

__device__ __forceinline__ unsigned int score_key(float f) {
  unsigned int u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool CACHED>
__device__ __forceinline__ unsigned int row_key(const float* __restrict__ row, const unsigned int* rowk, int i) {
  if (CACHED) return rowk[i];
  return score_key(row[i]);
}

template <bool CACHED>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores, int64_t ld, int n_q,
                                                          int n_kv, int k, int32_t* __restrict__ idx) {
  extern __shared__ unsigned int lds[];
  unsigned int* hist = lds;                           // [16][257]
  unsigned int* misc = lds + kHistWords;              // [64]
  unsigned int* rowk = lds + kHistWords + kMiscWords;  // [n] (CACHED only)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = n_q - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int n = n_kv - n_q + t + 1;
  const size_t rowid = (size_t)b * n_q + t;
  const float* row = scores + rowid * ld;
  int32_t* out = idx + rowid * (size_t)k;

  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = (i < n) ? i : -1;
    return;
  }

  unsigned int prefix = 0u;
  int k_rem = k;
  unsigned int* h = hist + (lane & (kHistCopies - 1)) * kHistStride;

#pragma unroll 1
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
    __syncthreads();
    if (pass == 0) {
      for (int i = tid; i < n; i += kTkThreads) {
        unsigned int key = score_key(row[i]);
        if (CACHED) rowk[i] = key;
        atomicAdd(&h[key >> 24], 1u);
      }
    } else {
      for (int i = tid; i < n; i += kTkThreads) {
        unsigned int key = row_key<CACHED>(row, rowk, i);
        if ((key >> (shift + 8)) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4l .. 4l+3 (summed over the copies)
      unsigned int c[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        unsigned int s = 0;
        for (int cp = 0; cp < kHistCopies; cp++) s += hist[cp * kHistStride + 4 * lane + j];
        c[j] = s;
      }
      unsigned int mine = c[0] + c[1] + c[2] + c[3];
      // inclusive suffix sum over lanes: ge_lane = sum of bins >= 4*lane
      unsigned int suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        unsigned int o = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += o;
      }
      unsigned int above = suf - mine;  // keys in bins >= 4*lane + 4
      // ge(bin) for bins 4l+3 .. 4l; the digit is the highest bin with ge >= k_rem
#pragma unroll
      for (int j = 3; j >= 0; j--) {
        unsigned int ge = above + c[j];
        if (above < (unsigned int)k_rem && ge >= (unsigned int)k_rem) {
          misc[0] = 4u * lane + j;
          misc[1] = above;  // keys strictly above this digit (within the prefix)
        }
        above = ge;
      }
    }
    __syncthreads();
    const unsigned int d = misc[0];
    const unsigned int gt = misc[1];
    prefix = (prefix << 8) | d;
    k_rem -= (int)gt;
    __syncthreads();  // misc is rewritten by the next pass
  }
  const unsigned int tau = prefix;  // the k-th largest key; k_rem keys equal to tau are taken

  // ordered compaction over per-wave contiguous segments
  const int seg = ((n + kTkWaves * 64 - 1) / (kTkWaves * 64)) * 64;
  const int s0 = wave * seg;
  const int s1 = min(n, s0 + seg);
  unsigned int n_gt = 0, n_eq = 0;
  for (int i0 = s0; i0 < s1; i0 += 64) {
    const int i = i0 + lane;
    unsigned int key = (i < s1) ? row_key<CACHED>(row, rowk, i) : 0u;
    bool g = (i < s1) && key > tau;
    bool e = (i < s1) && key == tau;
    n_gt += __popcll(__ballot(g));
    n_eq += __popcll(__ballot(e));
  }
  if (lane == 0) {
    misc[2 + wave] = n_gt;
    misc[2 + kTkWaves + wave] = n_eq;
  }
  __syncthreads();
  unsigned int gt_before = 0, eq_before = 0;
  for (int w2 = 0; w2 < wave; w2++) {
    gt_before += misc[2 + w2];
    eq_before += misc[2 + kTkWaves + w2];
  }
  unsigned int e_run = eq_before;
  unsigned int p_run = gt_before + min(eq_before, (unsigned int)k_rem);
  for (int i0 = s0; i0 < s1; i0 += 64) {
    const int i = i0 + lane;
    unsigned int key = (i < s1) ? row_key<CACHED>(row, rowk, i) : 0u;
    bool g = (i < s1) && key > tau;
    bool e = (i < s1) && key == tau;
    unsigned long long be = __ballot(e);
    unsigned int erank = e_run + (unsigned int)__builtin_amdgcn_mbcnt_hi((unsigned int)(be >> 32),
                                                                          __builtin_amdgcn_mbcnt_lo((unsigned int)be, 0u));
    bool sel = g || (e && erank < (unsigned int)k_rem);
    unsigned long long bs = __ballot(sel);
    unsigned int opos = p_run + (unsigned int)__builtin_amdgcn_mbcnt_hi((unsigned int)(bs >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((unsigned int)bs, 0u));
    if (sel && opos < (unsigned int)k) out[opos] = i;
    e_run += __popcll(be);
    p_run += __popcll(bs);
  }
}

static bool g_topk_attr_set = false;

hipError_t launch_topk(const float* scores, int64_t ld, int B, int n_q, int n_kv, int k, int32_t* idx,
                       hipStream_t stream) {
  dim3 grid(n_q, B);
  if (n_kv <= kRowCapMax) {
    if (!g_topk_attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytesMax);
      if (e != hipSuccess) return e;
      g_topk_attr_set = true;
    }
    size_t lds = (size_t)(kHistWords + kMiscWords + ((n_kv + 3) / 4) * 4) * 4;
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTkThreads), lds, stream, scores, ld, n_q, n_kv, k, idx);
  } else {
    size_t lds = (size_t)(kHistWords + kMiscWords) * 4;
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTkThreads), lds, stream, scores, ld, n_q, n_kv, k, idx);
  }
  return hipGetLastError();
}

}  // namespace dsa
