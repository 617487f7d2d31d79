// Top-k selection of compressed entries: exact radix select with the
// lower-index tie rule, output in ascending index order.
//
// The pages keep the k compressed entries the indexer finds most relevant
// (blog.nickys.cn DeepSeek-V4 post, 三大架构改动 §1 CSA).  Ties (equal scores,
// -0 == +0) go to the lower index and the result is written in ascending
// index order; this is this library's rule, not the pages'.
//
// One 1024-thread block per query row.  Scores become order-preserving
// uint32 keys (negative floats bit-inverted, non-negative ones with the sign
// bit set, -0 folded onto +0).  Radix passes over the top 11, next 11 and last
// 10 bits narrow the k-th key: after each pass a histogram in LDS and one
// block scan find the bin holding the k-th largest key; the search stops as
// soon as that bin is taken whole.  Rows of up to 32768 entries are held in
// LDS after the first read (one pad word per 32 keeps the per-thread chunk
// reads of the emission pass free of bank conflicts); longer rows are
// re-read from L2 on every pass.  Emission: each thread owns a contiguous
// index range, so two block-wide exclusive scans (equal-key ranks, then output
// offsets) give every selected index its slot in ascending order.
#include "common.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kCacheMax = 32768;
constexpr int kCacheWords = kCacheMax + kCacheMax / 32;

CSA_DEV uint32_t ordered_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

CSA_DEV int lds_pos(int x) { return x + (x >> 5); }

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ q_pos0, int T_q, int cap, int m,
                                                        int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;                       // kCacheWords (only when cached)
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan_smem[17];
  __shared__ uint32_t sel_bin, sel_remaining, sel_bincount;

  const int row = blockIdx.x;
  const int b = row / T_q;
  const int i = row - b * T_q;
  const int tid = threadIdx.x;
  const int t = q_pos0[b] + i;
  int nv = (t + 1) / m;
  nv = max(0, min(nv, cap));
  int32_t* out = idx + size_t(row) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const float* src = scores + size_t(row) * cap;
  const bool cached = nv <= kCacheMax;

  uint32_t prefix = 0u, mask = 0u;
  uint32_t remaining = uint32_t(k);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbits = pass == 2 ? 10 : 11;
    const int nb = 1 << nbits;
    for (int j = tid; j < nb; j += kThreads) hist[j] = 0u;
    __syncthreads();
    for (int x = tid; x < nv; x += kThreads) {
      uint32_t key;
      if (pass == 0 || !cached) {
        key = ordered_key(src[x]);
        if (pass == 0 && cached) keys[lds_pos(x)] = key;
      } else {
        key = keys[lds_pos(x)];
      }
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & uint32_t(nb - 1)], 1u);
    }
    __syncthreads();
    // bins in descending order: thread tid owns bins hi = nb-1-2*tid and lo = hi-1
    const int hi = nb - 1 - 2 * tid;
    const uint32_t c_hi = hi >= 0 ? hist[hi] : 0u;
    const uint32_t c_lo = hi >= 1 ? hist[hi - 1] : 0u;
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(c_hi + c_lo, scan_smem, &tot);
    if (hi >= 0 && above < remaining && remaining <= above + c_hi) {
      sel_bin = uint32_t(hi); sel_remaining = remaining - above; sel_bincount = c_hi;
    }
    if (hi >= 1 && above + c_hi < remaining && remaining <= above + c_hi + c_lo) {
      sel_bin = uint32_t(hi - 1); sel_remaining = remaining - above - c_hi; sel_bincount = c_lo;
    }
    __syncthreads();
    prefix |= sel_bin << shift;
    mask |= uint32_t(nb - 1) << shift;
    remaining = sel_remaining;
    const bool whole = sel_bincount == remaining;
    __syncthreads();
    if (whole) break;
  }

  // emission: entries with (key & mask) > prefix are in; of those equal, the
  // first `remaining` by index
  const int chunk = (nv + kThreads - 1) / kThreads;
  const int x0 = min(tid * chunk, nv);
  const int x1 = min(x0 + chunk, nv);
  uint32_t n_gt = 0, n_eq = 0;
  for (int x = x0; x < x1; ++x) {
    const uint32_t key = (cached ? keys[lds_pos(x)] : ordered_key(src[x])) & mask;
    n_gt += key > prefix;
    n_eq += key == prefix;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, scan_smem, &tot);
  const uint32_t take_eq = remaining > eq_before ? min(remaining - eq_before, n_eq) : 0u;
  uint32_t pos = block_exclusive_scan(n_gt + take_eq, scan_smem, &tot);
  uint32_t eq_seen = 0;
  for (int x = x0; x < x1; ++x) {
    const uint32_t key = (cached ? keys[lds_pos(x)] : ordered_key(src[x])) & mask;
    bool take = key > prefix;
    if (key == prefix) {
      take = eq_seen < take_eq;
      ++eq_seen;
    }
    if (take) out[pos++] = x;
  }
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
  static bool attr_set = false;
  const size_t dyn = size_t(kCacheWords) * sizeof(uint32_t);
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(dyn)) != hipSuccess)
      return CSA_EHIP;
    attr_set = true;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(topk_kernel, dim3(unsigned(rows)), dim3(kThreads), dyn, st, scores, q_pos0, T_q, cap, m, k, idx);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}
