// topk.hip -- fine-grained token selection: per query row, the k largest index scores among the
// causal candidates s <= pos_t (velog summary "DeepSeek-V3.2: Pushing the Frontier of Open Large
// Language Models", section 1.2; k = 2048 in the sparse-training stage).
//
// Exact radix select on order-preserving 32-bit keys (-0 folded onto +0):
//   * four 8-bit digit passes, most significant first, each building a 256-bin histogram of the
//     keys that share the digits fixed so far, then fixing the digit that holds the k-th largest
//     key; afterwards tau (the k-th largest key) is known, and so is the number of keys equal to
//     tau that are taken (the lowest positions win ties);
//   * an ordered compaction: every wave owns a contiguous segment of the row, counts its keys above
//     and equal to tau, a scan over waves gives each its output offset, and the wave writes its
//     selected positions in ascending order (ballots over per-lane counts), so the result is sorted.
// One workgroup (8 waves) selects from up to kKeyCap keys held in LDS: the first pass reads them from
// memory (kLoadUnroll independent 16-byte loads per thread in flight), every later pass and the
// compaction read LDS in 16-byte pieces, kLdsUnroll per lane in flight.  Rows of at most 32768 keys
// keep their keys in registers instead (topk_reg_kernel): the workgroup then needs only about 34 KB of
// LDS and two of them share a compute unit.
//
// Rows that are longer than one workgroup holds, or too few to fill the GPU, run in two stages.  Stage
// one cuts each row into chunks (at most kRegKeys keys, selected by the register-resident kernel, when
// a chunk's top k fit its staging area; else at most kKeyCap, in LDS)
// and selects the top k of every chunk as (key, position) candidates; stage two selects the top k among
// a row's candidates.  Every member of the row's top k is in its own chunk's
// top k (fewer than k keys of the row, hence of the chunk, beat it), so the result is exact.  The
// candidates of a row are stored chunk after chunk, each chunk's in ascending position, so array
// order is position order and the stage-two compaction keeps both the tie rule and the sorted output.
// Rows the two stages cannot take (k too large for the LDS budget) use a kernel that re-reads the row
// from memory in every pass.
#include <atomic>

#include "dsa_internal.h"

#include <algorithm>
#include <type_traits>

namespace dsa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;
constexpr int kHistWords = kHistCopies * kHistStride;
constexpr int kMiscWords = 64 + 256;  // digit/count scratch + summed histogram
constexpr int kLdsBytesMax = 163840;
constexpr int kKeyCap = ((kLdsBytesMax / 4 - kHistWords - kMiscWords) / 256) * 256;  // 36352 keys
constexpr int kLoadUnroll = 16;
constexpr int kLdsUnroll = 4;
constexpr int kSeg = 256;  // keys per wave-wide 16-byte LDS read

enum { kSrcScores = 0, kSrcCand = 1 };
enum { kDstIdx = 0, kDstCand = 1 };

struct TopkArgs {
  const float* scores;    // kSrcScores: [B][n_q][ld]
  int64_t ld;
  const uint32_t* ckey;   // kSrcCand: [B][n_q][n_cand] keys and positions
  const int32_t* cpos;
  int n_cand;
  int n_q, n_kv, k;
  int chunk;              // kSrcScores: keys per chunk (a multiple of 256); blockIdx.z = chunk number
  int n_chunks;
  int32_t* idx;           // kDstIdx: [B][n_q][k]
  uint32_t* okey;         // kDstCand: [B][n_q][n_chunks * k]
  int32_t* opos;
  bool vec4;              // the first pass may use 16-byte loads
};

__device__ __forceinline__ unsigned int score_key(float f) {
  unsigned int u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned int lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((unsigned int)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned int)m, 0u));
}

// Exclusive prefix over lanes of c (0 <= c <= 7) and its wave total, from the ballots of c's bits.
__device__ __forceinline__ void lane_scan3(unsigned int c, unsigned int* before, unsigned int* total) {
  const unsigned long long b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
  *before = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
  *total = (unsigned int)__popcll(b0) + 2u * (unsigned int)__popcll(b1) + 4u * (unsigned int)__popcll(b2);
}

__device__ __forceinline__ unsigned int wave_sum(unsigned int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// kLdsUnroll 16-byte LDS reads of keys [base + 256u + 4*lane, +4), all issued before any is used: the
// address is clamped into [0, s1) so no read needs a branch; callers discard keys at or past s1.
__device__ __forceinline__ void load_keys(const unsigned int* rowk, int base, int s1, int lane,
                                          u32x4 (&kk)[kLdsUnroll]) {
  const int last = (s1 - 1) & ~3;
#pragma unroll
  for (int u = 0; u < kLdsUnroll; u++) {
    const int i = min(base + kSeg * u + 4 * lane, last);
    kk[u] = *reinterpret_cast<const u32x4*>(rowk + i);
  }
}

// Inclusive suffix sum over the 64 lanes (lane l: sum of v over lanes >= l).  Within each row of 16
// lanes, four DPP row shifts toward lower lanes (sources past the row's end read 0); then every row
// adds the totals of the rows above it, read from their first lanes.
__device__ __forceinline__ unsigned int suffix_sum(unsigned int v, int lane) {
  v += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xF, 0xF, true);  // row_shl:1
  v += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xF, 0xF, true);  // row_shl:2
  v += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, true);  // row_shl:4
  v += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, 0x108, 0xF, 0xF, true);  // row_shl:8
  const unsigned int r1 = (unsigned int)__builtin_amdgcn_readlane((int)v, 16);
  const unsigned int r2 = (unsigned int)__builtin_amdgcn_readlane((int)v, 32);
  const unsigned int r3 = (unsigned int)__builtin_amdgcn_readlane((int)v, 48);
  const int row = lane >> 4;
  return v + (row < 1 ? r1 : 0u) + (row < 2 ? r2 : 0u) + (row < 3 ? r3 : 0u);
}

__device__ __forceinline__ void scan_digit(const unsigned int* tot, unsigned int* misc, int k_rem, int wave, int lane);

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
  scan_digit(tot, misc, k_rem, wave, lane);
}

// Wave 0 fixes the digit from the summed histogram `tot`: the highest bin whose suffix count reaches
// k_rem.  Writes misc[0] = digit, misc[1] = keys above it; ends with a barrier.
__device__ __forceinline__ void scan_digit(const unsigned int* tot, unsigned int* misc, int k_rem, int wave, int lane) {
  if (wave == 0) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(tot + 4 * lane);
    const unsigned int mine = c[0] + c[1] + c[2] + c[3];
    const unsigned int suf = suffix_sum(mine, lane);  // keys in bins >= 4*lane
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

template <int SRC, int DST>
__global__ __launch_bounds__(kTkThreads) void topk_select_kernel(TopkArgs a) {
  extern __shared__ unsigned int lds[];
  unsigned int* hist = lds;                            // [16][257]
  unsigned int* misc = lds + kHistWords;               // [64] scratch
  unsigned int* tot = misc + 64;                       // [256] summed histogram
  unsigned int* rowk = lds + kHistWords + kMiscWords;  // [m] keys

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = a.n_q - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int k = a.k;
  const int n = a.n_kv - a.n_q + t + 1;  // causal row length
  const size_t rowid = (size_t)b * a.n_q + t;

  int lo = 0, m;
  if (SRC == kSrcScores) {
    lo = (int)blockIdx.z * a.chunk;
    m = min(n, lo + a.chunk) - lo;  // <= 0 when the chunk lies past pos_t
  } else {
    m = a.n_cand;
  }
  const float* srow = SRC == kSrcScores ? a.scores + rowid * a.ld + lo : nullptr;
  const uint32_t* crow = SRC == kSrcCand ? a.ckey + rowid * (size_t)a.n_cand : nullptr;
  const int32_t* cprow = SRC == kSrcCand ? a.cpos + rowid * (size_t)a.n_cand : nullptr;
  int32_t* out_idx = DST == kDstIdx ? a.idx + rowid * (size_t)k : nullptr;
  const size_t ostride = (size_t)a.n_chunks * k;
  uint32_t* out_key = DST == kDstCand ? a.okey + rowid * ostride + (size_t)blockIdx.z * k : nullptr;
  int32_t* out_pos = DST == kDstCand ? a.opos + rowid * ostride + (size_t)blockIdx.z * k : nullptr;

  if (n <= k) {  // the row keeps all of its keys; stage one leaves such rows to stage two
    if (DST == kDstIdx)
      for (int i = tid; i < k; i += kTkThreads) out_idx[i] = (i < n) ? i : -1;
    return;
  }
  if (DST == kDstCand && m <= k) {  // the whole chunk is candidates (none when m <= 0); pad with key 0
    for (int i = tid; i < k; i += kTkThreads) {
      const bool v = i < m;
      out_key[i] = v ? score_key(srow[i]) : 0u;
      out_pos[i] = v ? lo + i : -1;
    }
    return;
  }

  // ---- pass 0: keys from memory into LDS, histogram of the top byte
  unsigned int* h = hist + (lane & (kHistCopies - 1)) * kHistStride;
  for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
  __syncthreads();
  if (a.vec4) {
    const int n4 = m >> 2;
    for (int base = 0; base < n4; base += kTkThreads * kLoadUnroll) {
      // every load is issued unconditionally (index clamped into the row) so that all of them are in
      // flight before the first is used; out-of-range values are discarded below
      u32x4 v[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int j = min(base + u * kTkThreads + tid, n4 - 1);
        if (SRC == kSrcScores)
          v[u] = __builtin_bit_cast(u32x4, reinterpret_cast<const float4*>(srow)[j]);
        else
          v[u] = reinterpret_cast<const u32x4*>(crow)[j];
      }
      const bool full = base + kLoadUnroll * kTkThreads <= n4;  // no bounds test per element
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int j = base + u * kTkThreads + tid;
        if (SRC == kSrcScores)
          v[u] = (u32x4){score_key(__uint_as_float(v[u][0])), score_key(__uint_as_float(v[u][1])),
                         score_key(__uint_as_float(v[u][2])), score_key(__uint_as_float(v[u][3]))};
        if (full || j < n4) {
          reinterpret_cast<u32x4*>(rowk)[j] = v[u];
#pragma unroll
          for (int e = 0; e < 4; e++) atomicAdd(&h[v[u][e] >> 24], 1u);
        }
      }
    }
    const int i = 4 * n4 + tid;  // tail of fewer than 4 keys
    if (i < m) {
      const unsigned int key = SRC == kSrcScores ? score_key(srow[i]) : crow[i];
      rowk[i] = key;
      atomicAdd(&h[key >> 24], 1u);
    }
  } else {
    for (int base = 0; base < m; base += kTkThreads * kLoadUnroll) {
      unsigned int v[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int i = min(base + u * kTkThreads + tid, m - 1);
        v[u] = SRC == kSrcScores ? __float_as_uint(srow[i]) : crow[i];
      }
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int i = base + u * kTkThreads + tid;
        if (SRC == kSrcScores) v[u] = score_key(__uint_as_float(v[u]));
        if (i < m) {
          rowk[i] = v[u];
          atomicAdd(&h[v[u] >> 24], 1u);
        }
      }
    }
  }
  __syncthreads();
  select_digit(hist, misc, tot, k, tid, wave, lane);
  unsigned int prefix = misc[0];
  int k_rem = k - (int)misc[1];
  __syncthreads();

  // wave segments of the LDS keys: [s0, s1), s0 a multiple of 256
  const int segw = ((m + kTkWaves * kSeg - 1) / (kTkWaves * kSeg)) * kSeg;
  const int s0 = wave * segw;
  const int s1 = min(m, s0 + segw);

  // ---- passes over LDS: one histogram pass per digit over the whole row, digits first .. last-1
  auto lds_hist_passes = [&](int first, int last) {
#pragma unroll 1
    for (int pass = first; pass < last; pass++) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
      __syncthreads();
      for (int base = s0; base < s1; base += kSeg * kLdsUnroll) {
        u32x4 kk[kLdsUnroll];
        load_keys(rowk, base, s1, lane, kk);
        unsigned int hit = 0;  // bit 4u+e: key (u, e) is in range and carries the digits fixed so far
#pragma unroll
        for (int u = 0; u < kLdsUnroll; u++) {
          const int i = base + kSeg * u + 4 * lane;
#pragma unroll
          for (int e = 0; e < 4; e++)
            hit |= (i + e < s1 && (kk[u][e] >> (shift + 8)) == prefix) ? 1u << (4 * u + e) : 0u;
        }
        if (__ballot(hit != 0) == 0) continue;
        // no branch per key: keys off the prefix count into the pad word of the copy (bin 256)
#pragma unroll
        for (int u = 0; u < kLdsUnroll; u++)
#pragma unroll
          for (int e = 0; e < 4; e++)
            atomicAdd(&h[(hit & (1u << (4 * u + e))) ? (kk[u][e] >> shift) & 255u : 256u], 1u);
      }
      __syncthreads();
      select_digit(hist, misc, tot, k_rem, tid, wave, lane);
      prefix = (prefix << 8) | misc[0];
      k_rem -= (int)misc[1];
      __syncthreads();  // misc is rewritten next
    }
  };
  lds_hist_passes(1, 2);  // second byte: nearly every key still carries the first

  // ---- one sweep over the row: per wave, the keys above the 16-bit prefix are counted and the
  // positions of the keys on it (the candidates, a small set for real score rows) are listed in the
  // histogram area.  The last two digits and the per-wave counts above and at tau then come from the
  // list.  A list that does not fit (rows with very many keys on one 16-bit prefix) falls back to
  // two more histogram passes over the row and a counting sweep.
  unsigned int* clist = hist;
  unsigned int* ccount = misc + 20;
  if (tid == 0) *ccount = 0u;
  __syncthreads();
  unsigned int n_above = 0;
  for (int base = s0; base < s1; base += kSeg * kLdsUnroll) {
    u32x4 kk[kLdsUnroll];
    load_keys(rowk, base, s1, lane, kk);
    unsigned int cmask = 0;  // bit 4u+e: key (u, e) is a candidate
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) {
      const int i = base + kSeg * u + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const bool v = i + e < s1;
        const unsigned int top = kk[u][e] >> 16;
        n_above += (v && top > prefix) ? 1u : 0u;
        cmask |= (v && top == prefix) ? 1u << (4 * u + e) : 0u;
      }
    }
    if (__ballot(cmask != 0) != 0) {  // a few candidates per batch: append them, one slot range per lane
      unsigned int slot = cmask ? atomicAdd(ccount, (unsigned int)__popc(cmask)) : 0u;
      while (cmask) {
        const int b = __builtin_ctz(cmask);
        cmask &= cmask - 1u;
        if (slot < (unsigned int)kHistWords) clist[slot] = (unsigned int)(base + kSeg * (b >> 2) + 4 * lane + (b & 3));
        slot++;
      }
    }
  }
  n_above = wave_sum(n_above);
  __syncthreads();
  const unsigned int n_cand = *ccount;
  if (n_cand <= (unsigned int)kHistWords) {
#pragma unroll 1
    for (int pass = 2; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) tot[tid] = 0u;
      __syncthreads();
      for (unsigned int c = tid; c < n_cand; c += kTkThreads) {
        const unsigned int key = rowk[clist[c]];
        if ((key >> (shift + 8)) == prefix) atomicAdd(&tot[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      scan_digit(tot, misc, k_rem, wave, lane);
      prefix = (prefix << 8) | misc[0];
      k_rem -= (int)misc[1];
      __syncthreads();
    }
    if (lane == 0) {
      misc[2 + wave] = n_above;
      misc[2 + kTkWaves + wave] = 0u;
    }
    __syncthreads();
    for (unsigned int c = tid; c < n_cand; c += kTkThreads) {
      const unsigned int pos = clist[c];
      const unsigned int key = rowk[pos];
      const unsigned int w = pos / (unsigned int)segw;
      if (key > prefix) atomicAdd(&misc[2 + w], 1u);
      else if (key == prefix) atomicAdd(&misc[2 + kTkWaves + w], 1u);
    }
    __syncthreads();
  } else {
    lds_hist_passes(2, 4);
    const unsigned int t = prefix;
    unsigned int n_gt = 0, n_eq = 0;
    for (int base = s0; base < s1; base += kSeg * kLdsUnroll) {
      u32x4 kk[kLdsUnroll];
      load_keys(rowk, base, s1, lane, kk);
#pragma unroll
      for (int u = 0; u < kLdsUnroll; u++) {
        const int i = base + kSeg * u + 4 * lane;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool v = i + e < s1;
          n_gt += (v && kk[u][e] > t) ? 1u : 0u;
          n_eq += (v && kk[u][e] == t) ? 1u : 0u;
        }
      }
    }
    n_gt = wave_sum(n_gt);
    n_eq = wave_sum(n_eq);
    if (lane == 0) {
      misc[2 + wave] = n_gt;
      misc[2 + kTkWaves + wave] = n_eq;
    }
    __syncthreads();
  }
  const unsigned int tau = prefix;  // the k-th largest key; k_rem keys equal to tau are taken

  // ---- ordered compaction: every wave writes its selected positions from its output offset
  unsigned int gt_before = 0, eq_before = 0;
  for (int w2 = 0; w2 < wave; w2++) {
    gt_before += misc[2 + w2];
    eq_before += misc[2 + kTkWaves + w2];
  }
  unsigned int e_run = eq_before;  // keys equal to tau before this point, in row order
  unsigned int p_run = gt_before + min(eq_before, (unsigned int)k_rem);  // selected before this point
  // The selection is staged in the (now free) histogram area and copied out by the whole workgroup
  // afterwards: k contiguous, coalesced stores instead of scattered per-lane ones.
  unsigned int* stage = hist;  // [k] row offsets, then (candidate output) [k] keys
  const bool staged = (DST == kDstIdx ? k : 2 * k) < kHistWords;  // the last word is the dummy slot
  for (int base = s0; base < s1; base += kSeg * kLdsUnroll) {
    u32x4 kk[kLdsUnroll];
    load_keys(rowk, base, s1, lane, kk);
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) {
      const int i = base + kSeg * u + 4 * lane;
      unsigned int eq_mask = 0, gt_mask = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const bool v = i + e < s1;
        gt_mask |= (v && kk[u][e] > tau) ? (1u << e) : 0u;
        eq_mask |= (v && kk[u][e] == tau) ? (1u << e) : 0u;
      }
      unsigned int sel_mask = gt_mask;
      if (__ballot(eq_mask != 0) != 0) {  // keys equal to tau: the first k_rem of them in row order
        unsigned int e_before, e_total;
        lane_scan3((unsigned int)__popc(eq_mask), &e_before, &e_total);
        unsigned int er = e_run + e_before;  // tie rank of this lane's first key equal to tau
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if (eq_mask & (1u << e)) {
            if (er < (unsigned int)k_rem) sel_mask |= 1u << e;
            er++;
          }
        }
        e_run += e_total;
      }
      unsigned int s_before, s_total;
      lane_scan3((unsigned int)__popc(sel_mask), &s_before, &s_total);
      unsigned int op = p_run + s_before;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if (staged) {  // no branch: unselected lanes write the last word of the area
          const bool sel = (sel_mask & (1u << e)) && op < (unsigned int)k;
          stage[sel ? op : kHistWords - 1] = (unsigned int)(i + e);
          if (DST == kDstCand) stage[sel ? k + op : kHistWords - 1] = kk[u][e];
        } else if ((sel_mask & (1u << e)) && op < (unsigned int)k) {
          if (DST == kDstIdx) {
            out_idx[op] = SRC == kSrcScores ? lo + i + e : cprow[i + e];
          } else {
            out_key[op] = kk[u][e];
            out_pos[op] = SRC == kSrcScores ? lo + i + e : cprow[i + e];
          }
        }
        op += (sel_mask >> e) & 1u;
      }
      p_run += s_total;
    }
  }
  if (staged) {  // exactly k entries were staged (m > k)
    __syncthreads();
    for (int j = tid; j < k; j += kTkThreads) {
      const unsigned int r = stage[j];
      const int pos = SRC == kSrcScores ? lo + (int)r : cprow[r];
      if (DST == kDstIdx) {
        out_idx[j] = pos;
      } else {
        out_key[j] = stage[k + j];
        out_pos[j] = pos;
      }
    }
  }
}

// Rows of at most kRegKeys keys: the same select, with every key held in
// registers instead of LDS.  Wave w owns the segment [w*segw, w*segw + segw) (segw a multiple of 256,
// at most 16 blocks of 256); lane l holds keys 256u + 64e + l (e = 0..3) of its wave's block u, so row
// order is (u, e, lane) and one ballot per key vector ranks keys in the compaction.  LDS keeps only
// the histograms, the candidate list and the staged output (about 34 KB), so two workgroups share a
// compute unit and one's barriers and memory waits overlap the other's passes.  DST = kDstIdx selects
// whole rows; DST = kDstCand is stage one of the two-stage plan for longer rows: blockIdx.z is the chunk
// of `chunk` keys (a multiple of 256, at most kRegKeys), whose top k go out as keys and positions.
// SRC = kSrcCand is stage two: the row is the n_in (key, position) candidates of stage one.
constexpr int kRegBlocks = 16;
constexpr int kRegKeys = kTkWaves * kRegBlocks * kSeg;  // 32768

template <int SRC, int DST>
__global__ __launch_bounds__(kTkThreads, 2) void topk_reg_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 int n_q, int n_kv, int k, int chunk, int n_chunks,
                                                                 int32_t* __restrict__ idx, uint32_t* __restrict__ okey,
                                                                 int32_t* __restrict__ opos,
                                                                 const uint32_t* __restrict__ ckey_in,
                                                                 const int32_t* __restrict__ cpos_in, int n_in) {
  __shared__ unsigned int hist[kHistWords];   // histograms; then the candidates' positions; then the output
  __shared__ unsigned int misc[kMiscWords];   // [64] scratch + [256] summed histogram
  __shared__ unsigned int ckey[kHistWords];   // the candidates' keys
  unsigned int* tot = misc + 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int t = n_q - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int n = n_kv - n_q + t + 1;  // causal row length
  const size_t rowid = (size_t)b * n_q + t;
  int32_t* out_idx = DST == kDstIdx ? idx + rowid * (size_t)k : nullptr;
  if (n <= k) {  // the row keeps all of its keys; stage one leaves such rows to stage two
    if (DST == kDstIdx)
      for (int i = tid; i < k; i += kTkThreads) out_idx[i] = (i < n) ? i : -1;
    return;
  }
  const int lo = DST == kDstCand ? (int)blockIdx.z * chunk : 0;
  // keys of this row, chunk (<= 0: past pos_t) or candidate list
  const int m = SRC == kSrcCand ? n_in : DST == kDstCand ? min(n, lo + chunk) - lo : n;
  const uint32_t* crow = SRC == kSrcCand ? ckey_in + rowid * (size_t)n_in : nullptr;
  const int32_t* cprow = SRC == kSrcCand ? cpos_in + rowid * (size_t)n_in : nullptr;
  const size_t ostride = (size_t)n_chunks * k;
  uint32_t* out_key = DST == kDstCand ? okey + rowid * ostride + (size_t)blockIdx.z * k : nullptr;
  int32_t* out_pos = DST == kDstCand ? opos + rowid * ostride + (size_t)blockIdx.z * k : nullptr;
  const float* srow = SRC == kSrcScores ? scores + rowid * ld + lo : nullptr;
  if (DST == kDstCand && m <= k) {  // the whole chunk is candidates (none when m <= 0); pad with key 0
    for (int i = tid; i < k; i += kTkThreads) {
      const bool v = i < m;
      out_key[i] = v ? score_key(srow[i]) : 0u;
      out_pos[i] = v ? lo + i : -1;
    }
    return;
  }
  const int segw = ((m + kTkWaves * kSeg - 1) / (kTkWaves * kSeg)) * kSeg;  // <= kRegBlocks * kSeg
  const int s0 = wave * segw;
  const int s1 = min(m, s0 + segw);
  const int nb = segw / kSeg;  // blocks per wave (uniform)

  // ---- pass 0: the wave's keys into registers (every load in flight at once, clamped into the row),
  // histogram of the top byte
  unsigned int* h = hist + (lane & (kHistCopies - 1)) * kHistStride;
  for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
  u32x4 kr[kRegBlocks];
#pragma unroll
  for (int u = 0; u < kRegBlocks; u++) {
    if (u < nb) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = min(s0 + kSeg * u + 64 * e + lane, m - 1);
        kr[u][e] = SRC == kSrcCand ? crow[i] : __float_as_uint(srow[i]);
      }
    } else {
      kr[u] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();  // histogram cleared
#pragma unroll
  for (int u = 0; u < kRegBlocks; u++) {
    if (u < nb) {
      const int i = s0 + kSeg * u + lane;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // positions past the segment (values from a clamped load) hold key 0 and are never counted:
        // every later pass tests i + 64 * e < s1 again
        unsigned int key = 0u;
        if (i + 64 * e < s1) {
          key = SRC == kSrcCand ? kr[u][e] : score_key(__uint_as_float(kr[u][e]));
          atomicAdd(&h[key >> 24], 1u);
        }
        kr[u][e] = key;
      }
    }
  }
  __syncthreads();
  select_digit(hist, misc, tot, k, tid, wave, lane);
  unsigned int prefix = misc[0];
  int k_rem = k - (int)misc[1];
  __syncthreads();

  // one histogram pass over the registers for each digit in [first, last)
  auto reg_hist_passes = [&](int first, int last) {
#pragma unroll 1
    for (int pass = first; pass < last; pass++) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kRegBlocks; u++) {
        if (u < nb) {
          const int i = s0 + kSeg * u + lane;
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (i + 64 * e < s1 && (kr[u][e] >> (shift + 8)) == prefix) atomicAdd(&h[(kr[u][e] >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      select_digit(hist, misc, tot, k_rem, tid, wave, lane);
      prefix = (prefix << 8) | misc[0];
      k_rem -= (int)misc[1];
      __syncthreads();  // misc is rewritten next
    }
  };
  reg_hist_passes(1, 2);

  // ---- candidates: keys on the 16-bit prefix, listed with their positions; keys above it counted
  unsigned int* clist = hist;
  unsigned int* ccount = misc + 20;
  if (tid == 0) *ccount = 0u;
  __syncthreads();
  unsigned int n_above = 0;
#pragma unroll
  for (int u = 0; u < kRegBlocks; u++) {
    if (u < nb) {
      const int i = s0 + kSeg * u + lane;
      unsigned int cmask = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const bool v = i + 64 * e < s1;
        const unsigned int top = kr[u][e] >> 16;
        n_above += (v && top > prefix) ? 1u : 0u;
        cmask |= (v && top == prefix) ? 1u << e : 0u;
      }
      if (__ballot(cmask != 0) != 0) {
        unsigned int slot = cmask ? atomicAdd(ccount, (unsigned int)__popc(cmask)) : 0u;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          if (cmask & (1u << e)) {
            if (slot < (unsigned int)kHistWords) {
              clist[slot] = (unsigned int)(i + 64 * e);
              ckey[slot] = kr[u][e];
            }
            slot++;
          }
        }
      }
    }
  }
  n_above = wave_sum(n_above);
  __syncthreads();
  const unsigned int n_cand = *ccount;
  if (n_cand <= (unsigned int)kHistWords) {
#pragma unroll 1
    for (int pass = 2; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) tot[tid] = 0u;
      __syncthreads();
      for (unsigned int c = tid; c < n_cand; c += kTkThreads) {
        const unsigned int key = ckey[c];
        if ((key >> (shift + 8)) == prefix) atomicAdd(&tot[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      scan_digit(tot, misc, k_rem, wave, lane);
      prefix = (prefix << 8) | misc[0];
      k_rem -= (int)misc[1];
      __syncthreads();
    }
    if (lane == 0) {
      misc[2 + wave] = n_above;
      misc[2 + kTkWaves + wave] = 0u;
    }
    __syncthreads();
    for (unsigned int c = tid; c < n_cand; c += kTkThreads) {
      const unsigned int key = ckey[c];
      const unsigned int w = clist[c] / (unsigned int)segw;
      if (key > prefix) atomicAdd(&misc[2 + w], 1u);
      else if (key == prefix) atomicAdd(&misc[2 + kTkWaves + w], 1u);
    }
    __syncthreads();
  } else {
    reg_hist_passes(2, 4);
    unsigned int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int u = 0; u < kRegBlocks; u++) {
      if (u < nb) {
        const int i = s0 + kSeg * u + lane;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool v = i + 64 * e < s1;
          n_gt += (v && kr[u][e] > prefix) ? 1u : 0u;
          n_eq += (v && kr[u][e] == prefix) ? 1u : 0u;
        }
      }
    }
    n_gt = wave_sum(n_gt);
    n_eq = wave_sum(n_eq);
    if (lane == 0) {
      misc[2 + wave] = n_gt;
      misc[2 + kTkWaves + wave] = n_eq;
    }
    __syncthreads();
  }
  const unsigned int tau = prefix;  // the k-th largest key; k_rem keys equal to tau are taken

  // ---- ordered compaction into the (free) histogram area, then k contiguous stores
  unsigned int gt_before = 0, eq_before = 0;
  for (int w2 = 0; w2 < wave; w2++) {
    gt_before += misc[2 + w2];
    eq_before += misc[2 + kTkWaves + w2];
  }
  unsigned int e_run = eq_before;
  unsigned int p_run = gt_before + min(eq_before, (unsigned int)k_rem);
  // [k] positions, then (candidate output) [k] keys; 2k <= kHistWords - 1: the last word is the dummy slot
  unsigned int* stage = hist;
  // Does this wave take any key equal to tau?  Only when it holds some and the waves before it have not
  // used up the k_rem taken ones.  Usually not: then a key is selected exactly when it is above tau, and
  // the loop below runs without the per-vector branch of the tie rule, so the compiler can overlap the
  // ballot and store chains of neighbouring key vectors.
  const bool eq_taken = __builtin_amdgcn_readfirstlane(misc[2 + kTkWaves + wave]) != 0u &&
                        (unsigned int)__builtin_amdgcn_readfirstlane(eq_before) < (unsigned int)k_rem;
  if (!eq_taken) {
#pragma unroll
    for (int u = 0; u < kRegBlocks; u++) {
      if (u < nb) {
        const int i = s0 + kSeg * u + lane;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool sel = i + 64 * e < s1 && kr[u][e] > tau;
          const unsigned long long bs = __ballot(sel);
          const unsigned int op = p_run + lanes_below(bs);
          const bool st = sel && op < (unsigned int)k;
          stage[st ? op : kHistWords - 1] = (unsigned int)(i + 64 * e);
          if (DST == kDstCand) stage[st ? k + op : kHistWords - 1] = kr[u][e];
          p_run += (unsigned int)__popcll(bs);
        }
      }
    }
  } else {
    // positions 256u + 64e + lane: row order is (u, e, lane), so one ballot per key vector ranks the keys
  #pragma unroll
    for (int u = 0; u < kRegBlocks; u++) {
      if (u < nb) {
        const int i = s0 + kSeg * u + lane;
  #pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool v = i + 64 * e < s1;
          bool sel = v && kr[u][e] > tau;
          const bool eq = v && kr[u][e] == tau;
          const unsigned long long be = __ballot(eq);
          if (be != 0ull) {  // keys equal to tau: the first k_rem of them in row order
            sel = sel || (eq && e_run + lanes_below(be) < (unsigned int)k_rem);
            e_run += (unsigned int)__popcll(be);
          }
          const unsigned long long bs = __ballot(sel);
          const unsigned int op = p_run + lanes_below(bs);
          const bool st = sel && op < (unsigned int)k;
          stage[st ? op : kHistWords - 1] = (unsigned int)(i + 64 * e);
          if (DST == kDstCand) stage[st ? k + op : kHistWords - 1] = kr[u][e];
          p_run += (unsigned int)__popcll(bs);
        }
      }
  }
  }
  __syncthreads();
  for (int j = tid; j < k; j += kTkThreads) {
    if (DST == kDstIdx) {
      out_idx[j] = SRC == kSrcCand ? cprow[stage[j]] : (int)stage[j];
    } else {
      out_key[j] = stage[k + j];
      out_pos[j] = lo + (int)stage[j];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Selection that re-reads its keys in every pass (from memory or LDS), for rows no resident kernel
// holds.  key_at(i) returns the order-preserving key of entry i (0 <= i < n), pos_at(i) the position
// written for it.  Both steps are called by every thread of a 512-thread workgroup; hist, misc and tot
// are its LDS scratch (kHistWords, 64 and 256 words).
// ------------------------------------------------------------------------------------------------
struct TauK {
  unsigned int tau;  // the k-th largest key
  int k_rem;         // how many keys equal to tau are taken (the lowest entries win)
};

template <typename KeyAt>
__device__ __forceinline__ TauK select_tau(int n, int k, unsigned int* hist, unsigned int* misc, unsigned int* tot,
                                           KeyAt key_at) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned int prefix = 0u;
  int k_rem = k;
  unsigned int* h = hist + (lane & (kHistCopies - 1)) * kHistStride;
#pragma unroll 1
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kHistWords; i += kTkThreads) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += kTkThreads * kLoadUnroll) {
      unsigned int v[kLoadUnroll];
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) v[u] = key_at(min(base + u * kTkThreads + tid, n - 1));
#pragma unroll
      for (int u = 0; u < kLoadUnroll; u++) {
        const int i = base + u * kTkThreads + tid;
        if (i < n && (pass == 0 || (v[u] >> (shift + 8)) == prefix)) atomicAdd(&h[(v[u] >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    select_digit(hist, misc, tot, k_rem, tid, wave, lane);
    prefix = (prefix << 8) | misc[0];
    k_rem -= (int)misc[1];
    __syncthreads();
  }
  return TauK{prefix, k_rem};
}

// Ordered write of the selection fixed by (tau, k_rem): every wave owns a contiguous segment of the
// entries, a scan over the waves' counts gives each its output offset, and ballots order the lanes.
template <typename KeyAt, typename PosAt>
__device__ __forceinline__ void select_write(int n, int k, TauK tk, int32_t* __restrict__ out, unsigned int* misc,
                                             KeyAt key_at, PosAt pos_at) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned int tau = tk.tau;
  const int k_rem = tk.k_rem;
  const int seg = ((n + kTkWaves * 64 - 1) / (kTkWaves * 64)) * 64;
  const int s0 = wave * seg;
  const int s1 = min(n, s0 + seg);
  unsigned int n_gt = 0, n_eq = 0;
  for (int i0 = s0; i0 < s1; i0 += 64 * kLdsUnroll) {
    unsigned int key[kLdsUnroll];
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) key[u] = key_at(min(i0 + 64 * u + lane, s1 - 1));
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      n_gt += (i < s1 && key[u] > tau) ? 1u : 0u;
      n_eq += (i < s1 && key[u] == tau) ? 1u : 0u;
    }
  }
  n_gt = wave_sum(n_gt);
  n_eq = wave_sum(n_eq);
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
  for (int i0 = s0; i0 < s1; i0 += 64 * kLdsUnroll) {
    unsigned int key[kLdsUnroll];
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) key[u] = key_at(min(i0 + 64 * u + lane, s1 - 1));
#pragma unroll
    for (int u = 0; u < kLdsUnroll; u++) {
      const int i = i0 + 64 * u + lane;
      const bool g = (i < s1) && key[u] > tau;
      const bool e = (i < s1) && key[u] == tau;
      const unsigned long long be = __ballot(e);
      const unsigned int erank = e_run + lanes_below(be);
      const bool sel = g || (e && erank < (unsigned int)k_rem);
      const unsigned long long bs = __ballot(sel);
      const unsigned int opos = p_run + lanes_below(bs);
      if (sel && opos < (unsigned int)k) out[opos] = pos_at(i);
      e_run += __popcll(be);
      p_run += __popcll(bs);
    }
  }
}

// Fallback for rows the LDS-resident kernels cannot take: every pass re-reads the row from memory.
__global__ __launch_bounds__(kTkThreads) void topk_uncached_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   int n_q, int n_kv, int k,
                                                                   int32_t* __restrict__ idx) {
  extern __shared__ unsigned int lds[];
  unsigned int* hist = lds;
  unsigned int* misc = lds + kHistWords;
  unsigned int* tot = misc + 64;
  const int tid = threadIdx.x;
  const int t = n_q - 1 - (int)blockIdx.x;
  const int b = blockIdx.y;
  const int n = n_kv - n_q + t + 1;
  const size_t rowid = (size_t)b * n_q + t;
  const float* row = scores + rowid * ld;
  int32_t* out = idx + rowid * (size_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  auto key_at = [&](int i) { return score_key(row[i]); };
  auto pos_at = [](int i) { return i; };
  const TauK tk = select_tau(n, k, hist, misc, tot, key_at);
  select_write(n, k, tk, out, misc, key_at, pos_at);
}

// ------------------------------------------------------------------------------------------------
// Few long rows (decode): threshold candidates per chunk, then one exact merge per row.
//
// Stage one cuts each row into chunks of at most kCandChunk keys (one 256-thread workgroup each, the
// keys in registers) and keeps, per chunk, every key at or above a threshold theta_c: digits of 12, 12
// and 8 bits are fixed from the top, as in a select of the chunk's top t_lo keys, but only until the
// keys at or above the current prefix number at most 2 t_lo (usually after the first digit: sign,
// exponent and three mantissa bits).  So a chunk keeps between t_lo and kCandCap keys, in ascending
// position, and every key it drops is below theta_c.  t_lo is a chunk's expected share of the row's
// top k plus six standard deviations of it and a margin.
// Stage two (one workgroup per row) gathers the row's candidates into LDS (chunk after chunk, so in
// position order) and selects their top k exactly: tau and the number of keys equal to tau to take.
// That is the row's selection exactly when tau >= theta_c for every chunk: each dropped key is then
// below tau, and every key equal to tau is a candidate.  Otherwise (a chunk holding much of the row's
// top k, or more than kCandCap keys tied at one value) the workgroup selects from the row's scores in
// memory instead.
// ------------------------------------------------------------------------------------------------
constexpr int kCandThreads = 256;
constexpr int kCandChunk = 8192;    // keys per chunk at most: 32 per thread
constexpr int kCandPerThread = kCandChunk / kCandThreads;
constexpr int kCandCap = 1024;      // candidates a chunk keeps at most
constexpr int kMergeCand = 16384;   // candidates of a row at most (n_chunks * kCandCap)

struct CandArgs {
  const float* scores;
  int64_t ld;
  int n_q, n_kv, k;
  int chunk, n_chunks, t_lo;
  uint32_t* ckey;  // [rows][n_chunks][kCandCap]
  int32_t* cpos;   // [rows][n_chunks][kCandCap]
  int32_t* chdr;   // [rows][n_chunks][2]: candidate count (-1: more than kCandCap tied), theta_c
  int32_t* idx;    // [rows][k]
};

template <bool VEC4>
__global__ __launch_bounds__(kCandThreads) void topk_cand_kernel(CandArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned int hist[4096];
  __shared__ unsigned int wsum[8];
  __shared__ unsigned int res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  const int n = a.n_kv - a.n_q + t + 1;  // causal row length
  const size_t rowid = (size_t)b * a.n_q + t;
  const int lo = c * a.chunk;
  const int m = min(n, lo + a.chunk) - lo;  // keys of this chunk (<= 0 past the row's end)
  const size_t slot = rowid * a.n_chunks + c;
  uint32_t* okey = a.ckey + slot * kCandCap;
  int32_t* opos = a.cpos + slot * kCandCap;
  const float* srow = a.scores + rowid * a.ld + lo;
  if (n <= a.k) return;  // the merge keeps the whole row
  if (m <= a.t_lo) {  // the whole chunk is candidates (none past the row's end)
    for (int i = tid; i < max(m, 0); i += kCandThreads) {
      okey[i] = score_key(srow[i]);
      opos[i] = lo + i;
    }
    if (tid == 0) {
      a.chdr[2 * slot] = max(m, 0);
      a.chdr[2 * slot + 1] = 0;
    }
    return;
  }

  // keys in registers: wave w owns entries [w*seg, w*seg + seg), lane l holds 4 consecutive keys of
  // each 256-key block u at w*seg + 256u + 4l (every load issued before any is used, indexes clamped
  // into the chunk; keys at or past m are masked below)
  const int seg = ((m + 4 * 256 - 1) / (4 * 256)) * 256;  // multiple of 256, <= kCandChunk / 4
  const int w0 = wave * seg;
  u32x4 kk[kCandPerThread / 4];
  if (VEC4) {
    const int last4 = ((m + 3) >> 2) - 1;  // the row's allocation holds whole 16-byte groups (ld % 4 == 0)
#pragma unroll
    for (int u = 0; u < kCandPerThread / 4; u++) {
      const int j = min((w0 + 256 * u + 4 * lane) >> 2, last4);
      kk[u] = __builtin_bit_cast(u32x4, reinterpret_cast<const float4*>(srow)[j]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kCandPerThread / 4; u++)
#pragma unroll
      for (int e = 0; e < 4; e++) kk[u][e] = __float_as_uint(srow[min(w0 + 256 * u + 4 * lane + e, m - 1)]);
  }
  unsigned int valid = 0;  // bit 4u+e: entry (u, e) lies in the wave's segment and the chunk
#pragma unroll
  for (int u = 0; u < kCandPerThread / 4; u++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int i = w0 + 256 * u + 4 * lane + e;
      kk[u][e] = score_key(__uint_as_float(kk[u][e]));
      valid |= (256 * u < seg && i < m) ? 1u << (4 * u + e) : 0u;
    }

  // digits from the top (12, 12, 8 bits) until the keys at or above the prefix number at most
  // 2 t_lo (at most kCandCap after the last digit, else the chunk reports an overflow)
  const unsigned int t_stop = min(2u * (unsigned int)a.t_lo, (unsigned int)kCandCap);
  unsigned int prefix = 0u, above = 0u, n_ge = 0u;
  int shift = 20;
  bool overflow = true;
  // One digit: histogram of the keys on the prefix (key >> PSHIFT == prefix), then the bin where the count
  // from the top, plus `above`, reaches t_lo.  Thread t owns the NB/256 consecutive bins from NB/256 * t
  // and holds their counts in registers; a suffix scan over the threads gives the count above each range.
  auto digit = [&](auto nb_c, auto shift_c, auto pshift_c, bool first) {
    constexpr int NB = decltype(nb_c)::value, SH = decltype(shift_c)::value, PSH = decltype(pshift_c)::value;
    constexpr int PER = NB / kCandThreads;  // 16 or 1
#pragma unroll
    for (int i = 0; i < PER; i++) hist[PER * tid + i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kCandPerThread / 4; u++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const unsigned int key = kk[u][e];
        const bool on = ((valid >> (4 * u + e)) & 1u) && (first || (key >> PSH) == prefix);
        if (on) atomicAdd(&hist[(key >> SH) & (unsigned int)(NB - 1)], 1u);
      }
    __syncthreads();
    unsigned int cnt[PER];
    if constexpr (PER == 16) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(hist + PER * tid + 4 * q);
        cnt[4 * q] = v[0]; cnt[4 * q + 1] = v[1]; cnt[4 * q + 2] = v[2]; cnt[4 * q + 3] = v[3];
      }
    } else {
      cnt[0] = hist[tid];
    }
    unsigned int mine = 0;
#pragma unroll
    for (int j = 0; j < PER; j++) mine += cnt[j];
    const unsigned int wsuf = suffix_sum(mine, lane);  // within the wave: bins >= PER * tid
    if (lane == 0) wsum[wave] = wsuf;
    __syncthreads();
    unsigned int higher = 0;  // keys in the waves above this one
#pragma unroll
    for (int w2 = 1; w2 < kCandThreads / 64; w2++) higher += (w2 > wave) ? wsum[w2] : 0u;
    unsigned int run = above + higher + (wsuf - mine);  // keys in bins above this thread's range
    const unsigned int need = (unsigned int)a.t_lo;
    if (run < need && run + mine >= need) {
      bool found = false;
#pragma unroll
      for (int j = PER - 1; j >= 0; j--) {
        if (!found && run + cnt[j] >= need) {
          res[0] = (unsigned int)(PER * tid + j);
          res[1] = run;           // keys above the bin
          res[2] = run + cnt[j];  // keys at or above the bin
          found = true;
        }
        run += cnt[j];
      }
    }
    __syncthreads();
    const unsigned int dig = res[0];
    above = res[1];
    n_ge = res[2];
    prefix = first ? dig : ((prefix << (PSH - SH)) | dig);
    shift = SH;
    __syncthreads();  // hist and res are rewritten by the next digit
  };
  digit(std::integral_constant<int, 4096>(), std::integral_constant<int, 20>(), std::integral_constant<int, 32>(),
        true);
  if (n_ge <= t_stop) {
    overflow = false;
  } else {
    digit(std::integral_constant<int, 4096>(), std::integral_constant<int, 8>(), std::integral_constant<int, 20>(),
          false);
    if (n_ge <= t_stop) {
      overflow = false;
    } else {
      digit(std::integral_constant<int, 256>(), std::integral_constant<int, 0>(), std::integral_constant<int, 8>(),
            false);
      overflow = n_ge > (unsigned int)kCandCap;
    }
  }
  const unsigned int theta = overflow ? 0u : prefix << shift;  // candidates: keys >= theta
  if (overflow) {
    if (tid == 0) {
      a.chdr[2 * slot] = -1;
      a.chdr[2 * slot + 1] = 0;
    }
    return;
  }

  // ordered compaction of the keys >= theta: per-wave counts, a scan over the four waves, then
  // ballots in position order inside each wave
  unsigned int cnt_mine = 0;
#pragma unroll
  for (int u = 0; u < kCandPerThread / 4; u++)
#pragma unroll
    for (int e = 0; e < 4; e++) cnt_mine += (((valid >> (4 * u + e)) & 1u) && kk[u][e] >= theta) ? 1u : 0u;
  const unsigned int wtot = wave_sum(cnt_mine);
  if (lane == 0) wsum[4 + wave] = wtot;
  __syncthreads();
  unsigned int orun = 0;
  for (int w2 = 0; w2 < wave; w2++) orun += wsum[4 + w2];
#pragma unroll
  for (int u = 0; u < kCandPerThread / 4; u++) {
    unsigned int sm = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) sm |= (((valid >> (4 * u + e)) & 1u) && kk[u][e] >= theta) ? 1u << e : 0u;
    unsigned int before, total;
    lane_scan3((unsigned int)__popc(sm), &before, &total);
    unsigned int o = orun + before;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      if ((sm >> e) & 1u) {
        okey[o] = kk[u][e];
        opos[o] = lo + w0 + 256 * u + 4 * lane + e;
        o++;
      }
    }
    orun += total;
  }
  if (tid == 0) {
    a.chdr[2 * slot] = (int)n_ge;
    a.chdr[2 * slot + 1] = (int)theta;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(CandArgs a) {
  extern __shared__ unsigned int lds[];
  unsigned int* hist = lds;
  unsigned int* misc = lds + kHistWords;
  unsigned int* tot = misc + 64;
  unsigned int* ck = tot + 256;                       // [kMergeCand] candidate keys
  int* cp = reinterpret_cast<int*>(ck + kMergeCand);  // [kMergeCand] their positions
  __shared__ int off_l[64];            // per chunk: offset of its candidates (n_chunks <= 64)
  __shared__ int cnt_l[64];            // per chunk: its candidate count
  __shared__ unsigned int row_l[3];    // total candidates, fallback flag, the largest threshold
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int b = blockIdx.y;
  const int n = a.n_kv - a.n_q + t + 1;
  const size_t rowid = (size_t)b * a.n_q + t;
  int32_t* out = a.idx + rowid * (size_t)a.k;
  if (n <= a.k) {
    for (int i = tid; i < a.k; i += kTkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const int32_t* rh = a.chdr + rowid * a.n_chunks * 2;
  if (wave == 0) {  // one lane per chunk (n_chunks <= 64): offsets by a wave scan, the largest threshold
    const bool has = lane < a.n_chunks;
    const int cnt = has ? rh[2 * lane] : 0;
    const unsigned int th = (has && cnt > 0) ? (unsigned int)rh[2 * lane + 1] : 0u;
    const unsigned int c = cnt > 0 ? (unsigned int)cnt : 0u;
    unsigned int incl = c;  // inclusive prefix sum over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    unsigned int mx = th;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (unsigned int)__shfl_xor(mx, off, 64));
    const bool bad = __ballot(has && cnt < 0) != 0ull;
    if (has) {
      off_l[lane] = (int)(incl - c);
      cnt_l[lane] = (int)c;
    }
    if (lane == 63) {
      row_l[0] = incl;
      row_l[1] = (bad || incl < (unsigned int)a.k || incl > (unsigned int)kMergeCand) ? 1u : 0u;
      row_l[2] = mx;
    }
  }
  __syncthreads();
  const float* row = a.scores + rowid * a.ld;
  auto row_key = [&](int i) { return score_key(row[i]); };
  auto row_pos = [](int i) { return i; };
  const int m = (int)row_l[0];
  if (row_l[1]) {  // a chunk kept too many tied keys, or the candidates are fewer than k: the row itself
    const TauK tk = select_tau(n, a.k, hist, misc, tot, row_key);
    select_write(n, a.k, tk, out, misc, row_key, row_pos);
    return;
  }
  const unsigned int theta_max = row_l[2];
  // gather the candidates, chunk after chunk: wave w copies chunks w, w + 8, ..., each lane loading all of
  // its (at most kCandCap / 64) entries of a chunk before storing any
  for (int c = wave; c < a.n_chunks; c += kTkWaves) {
    const int cnt = cnt_l[c];
    const int off = off_l[c];
    const size_t slot = rowid * a.n_chunks + c;
    const uint32_t* sk = a.ckey + slot * kCandCap;
    const int32_t* sp = a.cpos + slot * kCandCap;
    constexpr int kPer = kCandCap / 64;
    uint32_t kv_[kPer];
    int32_t pv_[kPer];
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      const int i = min(lane + 64 * u, kCandCap - 1);  // in the slot's bounds; entries at or past cnt are dropped
      kv_[u] = sk[i];
      pv_[u] = sp[i];
    }
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      const int i = lane + 64 * u;
      if (i < cnt) {
        ck[off + i] = kv_[u];
        cp[off + i] = pv_[u];
      }
    }
  }
  __syncthreads();
  auto c_key = [&](int i) { return ck[i]; };
  auto c_pos = [&](int i) { return cp[i]; };
  const TauK tk = select_tau(m, a.k, hist, misc, tot, c_key);
  if (tk.tau >= theta_max) {
    select_write(m, a.k, tk, out, misc, c_key, c_pos);
  } else {  // some chunk may hold keys at or above tau that it dropped
    const TauK tr = select_tau(n, a.k, hist, misc, tot, row_key);
    select_write(n, a.k, tr, out, misc, row_key, row_pos);
  }
}

// ------------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------------
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// More than 64 KiB of dynamic LDS needs an explicit opt-in, per kernel and device.  The outcome is
// remembered per device (a race between two threads only repeats the idempotent call).
constexpr int kMaxDevices = 64;

template <int SRC, int DST>
hipError_t allow_full_lds() {
  static std::atomic<int> done[kMaxDevices];  // 0: not yet, 1: opted in on that device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)topk_select_kernel<SRC, DST>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytesMax);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done[dev].store(1, std::memory_order_release);
  return e;
}

size_t merge_lds_bytes() { return (size_t)(kHistWords + kMiscWords + 2 * kMergeCand) * 4; }

hipError_t allow_full_lds_merge() {
  static std::atomic<int> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)topk_merge_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)merge_lds_bytes());
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done[dev].store(1, std::memory_order_release);
  return e;
}

size_t lds_bytes(int keys) { return (size_t)(kHistWords + kMiscWords + ((keys + 3) / 4) * 4) * 4; }

}  // namespace

TopkPlan plan_topk(int B, int n_q, int n_kv, int k) {
  TopkPlan p;
  const long long rows = (long long)B * n_q;
  p.mode = TopkPlan::kSingle;
  p.chunk = n_kv;
  p.n_chunks = 1;
  p.t_lo = 0;
  p.ws = 0;
  if (k < 1 || n_kv <= k) return p;  // every row keeps all of its keys (k < 1 is rejected by the caller)
  if (rows < 256) {
    // few long rows: threshold candidates per chunk when a chunk's expected share of the row's top k is
    // small against the candidate capacity, with chunks as short as the merge's capacity allows
    for (int chunk = 2048; chunk <= kCandChunk; chunk *= 2) {
      const int n_chunks = (int)(((long long)n_kv + chunk - 1) / chunk);
      // t_lo: a chunk's expected share of the row's top k plus six standard deviations of it and a margin,
      // so that a chunk of independent scores holds more than t_lo of the row's top k essentially never
      const long long share = ((long long)k * chunk + n_kv - 1) / n_kv;
      long long sd = 1;
      while (sd * sd < share) sd++;
      const long long t_lo = share + 6 * sd + 32;
      if (n_chunks < 2 || n_chunks * kCandCap > kMergeCand || 2 * t_lo > kCandCap) continue;
      p.mode = TopkPlan::kCandidates;
      p.chunk = chunk;
      p.n_chunks = n_chunks;
      p.t_lo = (int)t_lo;
      const size_t slots = (size_t)rows * n_chunks;
      p.ws = 2 * align256(slots * kCandCap * 4) + align256(slots * 2 * 4);
      return p;
    }
  }
  // chunks of at most kRegKeys keys when the register-resident kernel can stage a chunk's top k (keys and
  // positions), else of at most the LDS row cache
  const int cap = 2 * k < kHistWords ? kRegKeys : kKeyCap;
  int want = 1;
  if (n_kv > cap) want = (int)(((long long)n_kv + cap - 1) / cap);
  if (rows < 256) {
    // too few rows to fill the GPU: split each into chunks of at least 4k keys, aiming at one
    // workgroup per CU (a large chunk's row cache leaves room for only one), so that all chunks run
    // in a single round
    const long long more = std::min<long long>((256 + rows - 1) / rows, n_kv / (4LL * k));
    if (more > want) want = (int)more;
  }
  if (want <= 1) return p;
  const int chunk = (int)((((long long)n_kv + want - 1) / want + kSeg - 1) / kSeg * kSeg);
  const int n_chunks = (int)(((long long)n_kv + chunk - 1) / chunk);
  if (n_chunks < 2 || chunk <= k || chunk > cap || (long long)n_chunks * k > kKeyCap) {
    if (n_kv > kKeyCap) p.mode = TopkPlan::kUncached;
    return p;
  }
  p.mode = TopkPlan::kTwoStage;
  p.chunk = chunk;
  p.n_chunks = n_chunks;
  const size_t n_cand = (size_t)rows * n_chunks * k;
  p.ws = align256(n_cand * sizeof(uint32_t)) + align256(n_cand * sizeof(int32_t));
  return p;
}

hipError_t launch_topk(const float* scores, int64_t ld, int B, int n_q, int n_kv, int k, int32_t* idx,
                       const TopkPlan& p, void* workspace, hipStream_t stream) {
  TopkArgs a = {};
  a.scores = scores;
  a.ld = ld;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.k = k;
  a.idx = idx;
  // rows start on 16-byte boundaries when the base is aligned and ld is a multiple of 4
  const bool rows16 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && (ld & 3) == 0;
  if (p.mode == TopkPlan::kCandidates) {
    hipError_t e = allow_full_lds_merge();
    if (e != hipSuccess) return e;
    const size_t slots = (size_t)B * n_q * p.n_chunks;
    CandArgs c;
    c.scores = scores;
    c.ld = ld;
    c.n_q = n_q;
    c.n_kv = n_kv;
    c.k = k;
    c.chunk = p.chunk;
    c.n_chunks = p.n_chunks;
    c.t_lo = p.t_lo;
    c.ckey = (uint32_t*)workspace;
    c.cpos = (int32_t*)((char*)workspace + align256(slots * kCandCap * 4));
    c.chdr = (int32_t*)((char*)workspace + 2 * align256(slots * kCandCap * 4));
    c.idx = idx;
    if (rows16)
      hipLaunchKernelGGL(topk_cand_kernel<true>, dim3(p.n_chunks, n_q, B), dim3(kCandThreads), 0, stream, c);
    else
      hipLaunchKernelGGL(topk_cand_kernel<false>, dim3(p.n_chunks, n_q, B), dim3(kCandThreads), 0, stream, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(n_q, B), dim3(kTkThreads), merge_lds_bytes(), stream, c);
    return hipGetLastError();
  }
  if (p.mode == TopkPlan::kUncached) {
    hipLaunchKernelGGL(topk_uncached_kernel, dim3(n_q, B), dim3(kTkThreads), lds_bytes(0), stream, scores, ld, n_q,
                       n_kv, k, idx);
    return hipGetLastError();
  }
  if (p.mode == TopkPlan::kSingle && n_kv <= kRegKeys && k < kHistWords) {
    hipLaunchKernelGGL((topk_reg_kernel<kSrcScores, kDstIdx>), dim3(n_q, B), dim3(kTkThreads), 0, stream, scores, ld,
                       n_q, n_kv, k, n_kv, 1, idx, nullptr, nullptr, nullptr, nullptr, 0);
    return hipGetLastError();
  }
  if (p.mode == TopkPlan::kSingle) {
    hipError_t e = allow_full_lds<kSrcScores, kDstIdx>();
    if (e != hipSuccess) return e;
    a.chunk = n_kv;
    a.n_chunks = 1;
    a.vec4 = rows16;
    hipLaunchKernelGGL((topk_select_kernel<kSrcScores, kDstIdx>), dim3(n_q, B, 1), dim3(kTkThreads),
                       lds_bytes(n_kv > k ? n_kv : 0), stream, a);
    return hipGetLastError();
  }
  // two stages: chunk candidates into the workspace, then the merge
  hipError_t e = allow_full_lds<kSrcScores, kDstCand>();
  if (e != hipSuccess) return e;
  e = allow_full_lds<kSrcCand, kDstIdx>();
  if (e != hipSuccess) return e;
  const size_t n_cand_all = (size_t)B * n_q * p.n_chunks * k;
  uint32_t* ckey = (uint32_t*)workspace;
  int32_t* cpos = (int32_t*)((char*)workspace + align256(n_cand_all * sizeof(uint32_t)));
  a.chunk = p.chunk;
  a.n_chunks = p.n_chunks;
  a.okey = ckey;
  a.opos = cpos;
  a.vec4 = rows16;  // chunk starts are multiples of 256 keys
  if (p.chunk <= kRegKeys && 2 * k < kHistWords)
    hipLaunchKernelGGL((topk_reg_kernel<kSrcScores, kDstCand>), dim3(n_q, B, p.n_chunks), dim3(kTkThreads), 0, stream,
                       scores, ld, n_q, n_kv, k, p.chunk, p.n_chunks, nullptr, ckey, cpos, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((topk_select_kernel<kSrcScores, kDstCand>), dim3(n_q, B, p.n_chunks), dim3(kTkThreads),
                       lds_bytes(p.chunk), stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TopkArgs c = a;
  c.ckey = ckey;
  c.cpos = cpos;
  c.n_cand = p.n_chunks * k;
  c.vec4 = (c.n_cand & 3) == 0;  // the workspace is 256-byte aligned
  c.okey = nullptr;
  c.opos = nullptr;
  if (c.n_cand <= kRegKeys && k < kHistWords)
    hipLaunchKernelGGL((topk_reg_kernel<kSrcCand, kDstIdx>), dim3(n_q, B), dim3(kTkThreads), 0, stream, nullptr, 0,
                       n_q, n_kv, k, 0, 1, idx, nullptr, nullptr, ckey, cpos, c.n_cand);
  else
    hipLaunchKernelGGL((topk_select_kernel<kSrcCand, kDstIdx>), dim3(n_q, B, 1), dim3(kTkThreads),
                       lds_bytes(c.n_cand), stream, c);
  return hipGetLastError();
}

}  // namespace dsa
