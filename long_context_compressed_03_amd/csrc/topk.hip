// Top-k selection of compressed entries: exact selection with the
// lower-index tie rule, output in ascending index order.
//
// The pages keep the k compressed entries the indexer finds most relevant
// (blog.nickys.cn DeepSeek-V4 post, 三大架构改动 §1 CSA).  Ties (equal scores,
// -0 == +0) go to the lower index and the result is written in ascending
// index order; this is this library's rule, not the pages'.
//
// One 1024-thread block per query row.  Scores become order-preserving
// uint32 keys (negative floats bit-inverted, non-negative ones with the sign
// bit set, -0 folded onto +0); key 0 (a NaN pattern) marks "not a candidate".
// A row is held in registers, 32768 keys at a time: each thread holds 32
// keys, and the element a lane loads is chosen so that every wave-wide load
// covers 64 consecutive indices (coalesced 256-byte reads) and every wave
// ballot of a per-key predicate IS two words of an index-ordered bitmap.
//
// On one CU the kernel is bound by per-key VALU work and LDS traffic, so the
// number of passes over the keys is kept to three:
//  1. load + key transform + an LDS histogram of the top 14 key bits (sign,
//     exponent, 5 mantissa bits: a fixed, range-free bucketing);
//     one wave then finds the bucket holding the k-th largest key;
//  2. the keys of that bucket (usually under a few hundred) are appended to
//     an LDS list with one atomic per wave; a list of at most 1024 keys is
//     ranked exactly, one key per thread (a longer one takes an exact radix
//     select), to find the k-th key
//     and how many keys equal to it are still needed (rows whose bucket is
//     too crowded for the list take radix passes over all keys);
//  3. emission: ballots of "greater" and "equal" give the bitmaps directly;
//     thread w then owns 32 consecutive indices, and one block scan of the
//     packed counts gives each selected index its slot: #greater before it +
//     min(#equal before it, equal keys still needed).
#include "select.hpp"

namespace {

using namespace csa_sel;

constexpr int kPer = 8;                        // rounds of 4 keys per thread
constexpr int kRound = kThreads * 4;           // 4096 consecutive keys per round
constexpr int kSuper = kRound * kPer;          // 32768 keys in registers
constexpr int kWords = kSuper / 32;            // bitmap words per super-tile
constexpr int kBucketShift = 18;               // 14-bit buckets
constexpr int kBuckets = 1 << (32 - kBucketShift);
constexpr int kCand = 4096;                    // capacity of the threshold-bucket list
constexpr int kRankMax = 1024;                 // lists up to this size are ranked one entry per lane

struct Shared {
  uint32_t hist[kBuckets];
  uint32_t bm_gt[kWords];
  uint32_t bm_eq[kWords];
  uint32_t cand[kCand];
  uint32_t smem[32];
  uint32_t n_cand;
  Sel sel;
};

// Index of key (j, c) of this thread within its super-tile.
CSA_DEV int key_index(int j, int c) { return j * kRound + c * kThreads + threadIdx.x; }

// Keys of super-tile `st`: wave w, lane l, key (j, c) is index j*4096 + c*1024 + 64w + l.
CSA_DEV void load_keys(const float* __restrict__ src, int nv, int st, uint32_t (&key)[kPer][4]) {
  const int base = st * kSuper;
  float v[kPer][4];
#pragma unroll
  for (int j = 0; j < kPer; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int x = base + key_index(j, c);
      v[j][c] = x < nv ? src[x] : 0.f;
    }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) key[j][c] = base + key_index(j, c) < nv ? ordered_key(v[j][c]) : 0u;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ q_pos0, int T_q, int cap, int m,
                                                        int k, int32_t* __restrict__ idx) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Shared& sh = *reinterpret_cast<Shared*>(smem_raw);

  const int row = blockIdx.x;
  const int b = row / T_q;
  const int i = row - b * T_q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = q_pos0[b] + i;
  int nv = (t + 1) / m;
  nv = max(0, min(nv, cap));
  int32_t* out = idx + size_t(row) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const float* src = scores + size_t(row) * cap;
  const int n_super = (nv + kSuper - 1) / kSuper;
  const uint64_t lanes_below = (uint64_t(1) << lane) - 1u;

  // ---- pass 1: keys, bucket histogram
  for (int j = tid; j < kBuckets; j += kThreads) sh.hist[j] = 0u;
  if (tid == 0) sh.n_cand = 0u;
  __syncthreads();
  uint32_t key[kPer][4];
#pragma unroll 1
  for (int st = 0; st < n_super; ++st) {
    load_keys(src, nv, st, key);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (key[j][c]) atomicAdd(&sh.hist[key[j][c] >> kBucketShift], 1u);
  }
  __syncthreads();
  find_bin(sh.hist, kBuckets, uint32_t(k), &sh.sel, sh.smem);
  const uint32_t B = sh.sel.bin;
  uint32_t remaining = sh.sel.remaining;
  const uint32_t cnt = sh.sel.bincount;
  uint32_t mask = ~((1u << kBucketShift) - 1u);
  uint32_t prefix = B << kBucketShift;
  __syncthreads();

  // visits every key of the row (reloading super-tiles when the row is long)
  auto each_key = [&](auto fn) {
#pragma unroll 1
    for (int st = 0; st < n_super; ++st) {
      if (n_super > 1) load_keys(src, nv, st, key);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) fn(key[j][c]);
    }
  };

  if (cnt != remaining) {
    if (cnt <= uint32_t(kCand)) {
      // ---- pass 2: list the threshold bucket, refine over the list
#pragma unroll 1
      for (int st = 0; st < n_super; ++st) {
        if (n_super > 1) load_keys(src, nv, st, key);
        uint32_t wave_total = 0u;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) wave_total += __popcll(__ballot(key[j][c] && (key[j][c] >> kBucketShift) == B));
        uint32_t base = 0u;
        if (lane == 0 && wave_total) base = atomicAdd(&sh.n_cand, wave_total);
        base = __shfl(base, 0);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool want = key[j][c] && (key[j][c] >> kBucketShift) == B;
            const uint64_t bal = __ballot(want);
            if (want) sh.cand[base + __popcll(bal & lanes_below)] = key[j][c];
            base += __popcll(bal);
          }
      }
      __syncthreads();
      const int nc = int(sh.n_cand);
      if (nc <= kRankMax) {
        // few candidates: each lane of the first waves ranks one of them
        // exactly against the whole list (read as broadcast 16-byte words,
        // zero-padded: key 0 is neither greater than nor equal to a
        // candidate); the k-th key x has #(greater) < remaining <=
        // #(greater) + #(equal)
        const int padded = (nc + 7) & ~7;
        if (tid >= nc && tid < padded) sh.cand[tid] = 0u;
        __syncthreads();
        if (tid < nc) {
          const uint32_t mine = sh.cand[tid];
          uint32_t n_gt = 0u, n_eq = 0u;
          const u32x4* c4 = reinterpret_cast<const u32x4*>(sh.cand);
          for (int x = 0; x < padded / 4; x += 2) {
            const u32x4 o0 = c4[x], o1 = c4[x + 1];
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              n_gt += (o0[y] > mine ? 1u : 0u) + (o1[y] > mine ? 1u : 0u);
              n_eq += (o0[y] == mine ? 1u : 0u) + (o1[y] == mine ? 1u : 0u);
            }
          }
          if (n_gt < remaining && remaining <= n_gt + n_eq) {
            sh.sel.bin = mine;
            sh.sel.remaining = remaining - n_gt;
          }
        }
        __syncthreads();
        prefix = sh.sel.bin;
        mask = 0xFFFFFFFFu;
        remaining = sh.sel.remaining;
      } else {
        auto each_cand = [&](auto fn) {
          for (int x = tid; x < nc; x += kThreads) fn(sh.cand[x]);
        };
        refine(each_cand, prefix, mask, remaining, sh);
      }
    } else {
      refine(each_key, prefix, mask, remaining, sh);
    }
  }

  // ---- pass 3: emission in index order
  uint32_t gt_off = 0u, eq_off = 0u;
  const int w = tid >> 6;
  // bitmap words of the wave's 64 keys (indices j*4096 + c*1024 + 64w + l):
  // a per-wave base plus (j*4096 + c*1024)/32
  uint32_t* const gt_w = sh.bm_gt + 2 * w;
  uint32_t* const eq_w = sh.bm_eq + 2 * w;
#pragma unroll 1
  for (int st = 0; st < n_super; ++st) {
    if (n_super > 1) load_keys(src, nv, st, key);
    __syncthreads();   // earlier readers of the bitmaps are done
#pragma unroll
    for (int j = 0; j < kPer; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t km = key[j][c] & mask;
        const uint64_t g = __ballot(key[j][c] && km > prefix);
        const uint64_t e = __ballot(key[j][c] && km == prefix);
        const int word = (j * kRound + c * kThreads) >> 5;
        if (lane == 0) {
          gt_w[word] = uint32_t(g);
          gt_w[word + 1] = uint32_t(g >> 32);
          eq_w[word] = uint32_t(e);
          eq_w[word + 1] = uint32_t(e >> 32);
        }
      }
    __syncthreads();
    const uint32_t wg = sh.bm_gt[tid];
    const uint32_t we = sh.bm_eq[tid];
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((uint32_t(__popc(we)) << 16) | uint32_t(__popc(wg)), sh.smem, &tot);
    uint32_t gt_before = gt_off + (ex & 0xFFFFu);
    uint32_t eq_before = eq_off + (ex >> 16);
    const int x0 = st * kSuper + tid * 32;
    uint32_t any = wg | we;
    while (any) {
      const int bit = __ffs(any) - 1;
      any &= any - 1u;
      if ((wg >> bit) & 1u) {
        out[gt_before + min(eq_before, remaining)] = x0 + bit;
        ++gt_before;
      } else {
        if (eq_before < remaining) out[gt_before + eq_before] = x0 + bit;
        ++eq_before;
      }
    }
    gt_off += tot & 0xFFFFu;
    eq_off += tot >> 16;
  }
}

hipError_t launch_topk(long rows, hipStream_t st, const float* scores, const int32_t* q_pos0, int T_q, int cap, int m,
                       int k, int32_t* idx) {
  static bool attr = false;   // more than 64 KB of LDS needs the opt-in
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(Shared)));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(unsigned(rows)), dim3(kThreads), sizeof(Shared), st, scores, q_pos0, T_q, cap,
                     m, k, idx);
  return hipGetLastError();
}

}  // namespace

extern "C" csa_status_t csa_topk(const float* scores, const int32_t* q_pos0, int32_t B, int32_t T_q, int32_t cap,
                                 int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!scores || !q_pos0 || !idx) return CSA_EINVAL;
  if (B < 0 || T_q < 0 || cap < 0 || m < 1 || k < 1) return CSA_EINVAL;
  const long rows = long(B) * T_q;
  if (rows == 0) return CSA_OK;
  if (rows > 0x7FFFFFFFL) return CSA_ENOTSUP;
  const hipError_t e = launch_topk(rows, static_cast<hipStream_t>(stream), scores, q_pos0, T_q, cap, m, k, idx);
  return e == hipSuccess ? CSA_OK : CSA_EHIP;
}
