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
// Memory access: every pass reads in chunks of kUnroll independent loads per thread (16-byte loads
// when rows are 16-byte aligned) before using any of them (the scores come from HBM once; a row that fits in LDS is kept there as keys).  The
// histogram has 16 copies (a lane uses copy lane%16) padded to 257 words, which spreads the heavy
// same-bin traffic of the first pass (scores of similar magnitude share their top byte); the copies
// are summed by 256 threads in parallel.
#include "dsa_internal.h"

namespace dsa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;
constexpr int kHistWords = kHistCopies * kHistStride;
constexpr int kMiscWords = 64 + 256;  // digit/count scratch + summed histogram
constexpr int kLdsBytesMax = 163840;
constexpr int kRowCapMax = ((kLdsBytesMax - (kHistWords + kMiscWords) * 4) / 4) / 64 * 64;
constexpr int kUnroll = 8;

__device__ __forceinline__ unsigned int score_key(float f) {
  unsigned int u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum the histogram copies (256 threads, one bin each), then wave 0 fixes the digit: the highest bin
// whose suffix count reaches k_rem.  Writes misc[0] = digit, misc[1] = keys above it.
__device__ __forceinline__ void select_digit(const unsigned int* hist, unsigned int* misc, unsigned int* tot,
                                             int k_rem, int tid, int wave, int lane) {
  if (tid < 256) {
    unsigned int s = 0;
#pragma unroll
    for (int cp = 0; cp < kHistCopies; cp++) s += hist[cp * kHistStride + tid];
    tot[tid] = s;
  }
  __syncthreads();
  if (wave == 0) {
    unsigned int c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] = tot[4 * lane + j];
    const unsigned int mine = c[0] + c[1] + c[2] + c[3];
    unsigned int suf = mine;  // inclusive suffix sum over lanes: keys in bins >= 4*lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int o = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += o;
    }
    unsigned int above = suf - mine;  // keys in bins >= 4*lane + 4
#pragma unroll
    for (int j = 3; j >= 0; j--) {
      const unsigned int ge = above + c[j];
      if (above < (unsigned int)k_rem && ge >= (unsigned int)k_rem) {
        misc[0] = 4u * lane + j;
        misc[1] = above;
      }
      above = ge;
    }
  }
  __syncthreads();
}

template <bool CACHED>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores, int64_t ld, int n_q,
                                                          int n_kv, int k, int32_t* __restrict__ idx, bool vec4) {
  extern __shared__ unsigned int lds[];
  unsigned int* hist = lds;                         // [16][257]
  unsigned int* misc = lds + kHistWords;            // [64] scratch
  unsigned int* tot = misc + 64;                    // [256] summed histogram
  unsigned int* rowk = lds + kHistWords + kMiscWords;  // [n] keys (CACHED only)

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
    if (pass == 0 || !CACHED) {
      if (vec4) {
        // 16-byte loads: kUnroll float4 per thread in flight, the tail (n % 4 keys) one by one
        const float4* row4 = reinterpret_cast<const float4*>(row);
        const int n4 = n >> 2;
        for (int base = 0; base < n4; base += kTkThreads * kUnroll) {
          float4 v[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; u++) {
            const int j = base + u * kTkThreads + tid;
            v[u] = j < n4 ? row4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int u = 0; u < kUnroll; u++) {
            const int j = base + u * kTkThreads + tid;
            if (j < n4) {
              const unsigned int key[4] = {score_key(v[u].x), score_key(v[u].y), score_key(v[u].z),
                                           score_key(v[u].w)};
              if (CACHED) reinterpret_cast<u32x4*>(rowk)[j] = (u32x4){key[0], key[1], key[2], key[3]};
#pragma unroll
              for (int e = 0; e < 4; e++)
                if (pass == 0 || (key[e] >> (shift + 8)) == prefix) atomicAdd(&h[(key[e] >> shift) & 255u], 1u);
            }
          }
        }
        const int i = 4 * n4 + tid;
        if (i < n) {
          const unsigned int key = score_key(row[i]);
          if (CACHED) rowk[i] = key;
          if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
        }
      } else {
        for (int base = 0; base < n; base += kTkThreads * kUnroll) {
          float v[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; u++) {
            const int i = base + u * kTkThreads + tid;
            v[u] = i < n ? row[i] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < kUnroll; u++) {
            const int i = base + u * kTkThreads + tid;
            if (i < n) {
              const unsigned int key = score_key(v[u]);
              if (CACHED) rowk[i] = key;
              if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
            }
          }
        }
      }
    } else {
      for (int i = tid; i < n; i += kTkThreads) {
        const unsigned int key = rowk[i];
        if ((key >> (shift + 8)) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    select_digit(hist, misc, tot, k_rem, tid, wave, lane);
    prefix = (prefix << 8) | misc[0];
    k_rem -= (int)misc[1];
    __syncthreads();  // misc is rewritten by the next pass
  }
  const unsigned int tau = prefix;  // the k-th largest key; k_rem keys equal to tau are taken

  // ordered compaction over per-wave contiguous segments (kUnroll 64-wide groups per load batch)
  const int seg = ((n + kTkWaves * 64 - 1) / (kTkWaves * 64)) * 64;
  const int s0 = wave * seg;
  const int s1 = min(n, s0 + seg);
  unsigned int n_gt = 0, n_eq = 0;
  for (int i0 = s0; i0 < s1; i0 += 64 * kUnroll) {
    unsigned int key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      key[u] = (i < s1) ? (CACHED ? rowk[i] : score_key(row[i])) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      n_gt += __popcll(__ballot(i < s1 && key[u] > tau));
      n_eq += __popcll(__ballot(i < s1 && key[u] == tau));
    }
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
  for (int i0 = s0; i0 < s1; i0 += 64 * kUnroll) {
    unsigned int key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      key[u] = (i < s1) ? (CACHED ? rowk[i] : score_key(row[i])) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      const bool g = (i < s1) && key[u] > tau;
      const bool e = (i < s1) && key[u] == tau;
      const unsigned long long be = __ballot(e);
      const unsigned int erank = e_run + (unsigned int)__builtin_amdgcn_mbcnt_hi(
                                             (unsigned int)(be >> 32), __builtin_amdgcn_mbcnt_lo((unsigned int)be, 0u));
      const bool sel = g || (e && erank < (unsigned int)k_rem);
      const unsigned long long bs = __ballot(sel);
      const unsigned int opos = p_run + (unsigned int)__builtin_amdgcn_mbcnt_hi(
                                            (unsigned int)(bs >> 32), __builtin_amdgcn_mbcnt_lo((unsigned int)bs, 0u));
      if (sel && opos < (unsigned int)k) out[opos] = i;
      e_run += __popcll(be);
      p_run += __popcll(bs);
    }
  }
}

hipError_t launch_topk(const float* scores, int64_t ld, int B, int n_q, int n_kv, int k, int32_t* idx,
                       hipStream_t stream) {
  dim3 grid(n_q, B);
  // rows start on 16-byte boundaries when the base is aligned and ld is a multiple of 4
  const bool vec4 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && (ld & 3) == 0;
  if (n_kv <= kRowCapMax) {
    // more than 64 KiB of dynamic LDS needs an explicit opt-in (done once; thread-safe static init)
    static const hipError_t attr = hipFuncSetAttribute((const void*)topk_kernel<true>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytesMax);
    if (attr != hipSuccess) return attr;
    size_t lds = (size_t)(kHistWords + kMiscWords + ((n_kv + 3) / 4) * 4) * 4;
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTkThreads), lds, stream, scores, ld, n_q, n_kv, k, idx, vec4);
  } else {
    size_t lds = (size_t)(kHistWords + kMiscWords) * 4;
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTkThreads), lds, stream, scores, ld, n_q, n_kv, k, idx, vec4);
  }
  return hipGetLastError();
}

}  // namespace dsa
