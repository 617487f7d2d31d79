// The split top-k path for few long rows, shared by csa_topk (scores given)
// and csa_indexer_topk (scores computed in the same kernel as the slice
// pass): per 2048-entry slice, a local bound and the compacted candidates;
// then one block per row selects among them (launched by
// launch_topk_split_rows, defined with that kernel).
//
// Slice pass (exact for any input): with the slice's share q_s =
// ceil(k n_s / nv) of the row's nv visible entries, v_s is the lower edge of
// the 14-bit key bucket that holds the slice's c_s-th largest key, c_s =
// min(n_s, q_s + 6 sqrt(q_s) + 6) (1 = every key when the window of kWindow
// buckets below the slice's top bucket holds fewer than c_s keys); the slice
// stores every key >= v_s with its index, in index order.  The shares sum to
// at least k, so the candidates hold at least k keys, and they hold every key
// of the row >= max v_s: when the selected keys are all >= max v_s the
// selection among the candidates is the row's (the row kernel checks it and
// otherwise falls back to the one-block algorithm over the row).  The margin
// over the share follows the spread of a Poisson count with mean q_s (about
// six standard deviations): with scores spread evenly over the slices the
// check almost never fails; inputs that crowd the top keys into a few slices
// take the fallback.
#pragma once
#include "select.hpp"
#include "compress_core.hpp"

namespace csa_split {

constexpr int kSlice = 2048;                   // keys per slice
constexpr int kSliceThreads = 256;             // slice pass over given scores
constexpr int kSlicePer = kSlice / kSliceThreads;
constexpr int kSliceCap = 512;                 // candidates kept per slice
constexpr int kWindow = 1024;                  // buckets below the slice's top bucket
constexpr int kBucketShift = 18;               // 14-bit buckets
constexpr int kSplitMaxRows = 128;
constexpr int kSplitMinCap = 8192;
constexpr int kMaxSlices = 1024;

inline int n_slices(int cap) { return (cap + kSlice - 1) / kSlice; }
inline bool use_split(long rows, int cap) {
  return rows <= kSplitMaxRows && cap >= kSplitMinCap && n_slices(cap) <= kMaxSlices;
}

// Workspace of the split path: bounds [rows][G], counts [rows][G], largest
// keys [rows][G], candidate keys and indices [rows][G][kSliceCap].
struct SplitWs {
  uint32_t* bound;
  uint32_t* count;
  uint32_t* top;
  uint32_t* key;
  int32_t* idx;
};
inline size_t split_ws_bytes(long rows, int cap) {
  return size_t(rows) * n_slices(cap) * (3 * sizeof(uint32_t) + kSliceCap * (sizeof(uint32_t) + sizeof(int32_t)));
}
inline SplitWs split_ws(void* ws, long rows, int cap) {
  const size_t n = size_t(rows) * n_slices(cap);
  SplitWs w;
  w.bound = static_cast<uint32_t*>(ws);
  w.count = w.bound + n;
  w.top = w.count + n;
  w.key = w.top + n;
  w.idx = reinterpret_cast<int32_t*>(w.key + n * kSliceCap);
  return w;
}

struct alignas(16) SliceShared {   // hist is read as 16-byte words
  uint32_t hist[kWindow];
  uint32_t smax[16];
  uint32_t wc[32];
  uint32_t v;
};

// Largest key over a wave (every lane receives it).
CSA_DEV uint32_t wave_umax(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), o)));
  return v;
}
CSA_DEV uint32_t wave_umin(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, uint32_t(__shfl_xor(int(v), o)));
  return v;
}

// What slice_finish expects before its call, behind a barrier: the window
// histogram cleared and sh.smax[w] = the largest key wave w holds (or wrote).
// clear_window: every thread of a block of kT threads calls it.
template <int kT>
CSA_DEV void clear_window(SliceShared& sh) {
#pragma unroll
  for (int i = 0; i < kWindow / kT; ++i) sh.hist[threadIdx.x * (kWindow / kT) + i] = 0u;
}

// The slice pass on keys already in registers, by a block of kT threads
// (256 or 1024): thread t holds the keys of indices base + j*kT + t (0 for
// entries past the visible count); n_s > 0 visible entries in the slice,
// nv > k in the row.  Writes count[slot], bound[slot], top[slot] (the
// slice's largest key, one of its candidates) and the slot's candidates.  Every thread of the block calls it, after a barrier that
// follows clear_window and the waves' sh.smax writes.
template <int kT>
CSA_DEV void slice_finish(const uint32_t (&key)[kSlice / kT], int base, int n_s, int nv, int k, size_t slot,
                          const SplitWs& ws, SliceShared& sh) {
  constexpr int kP = kSlice / kT;       // keys per thread
  constexpr int kW = kT / 64;           // waves
  static_assert(kP * kW == 32, "32 ballot groups per slice");
  static_assert(kWindow % 256 == 0, "rounds of 256 buckets");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t quota = uint32_t((uint64_t(k) * uint32_t(n_s) + uint32_t(nv) - 1u) / uint32_t(nv));
  const uint32_t want = min(uint32_t(n_s), quota + uint32_t(6.f * sqrtf(float(quota))) + 6u);
  uint32_t mx = sh.smax[0];
#pragma unroll
  for (int x = 1; x < kW; ++x) mx = max(mx, sh.smax[x]);
  const int top = int(mx >> kBucketShift);
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int rel = top - int(key[j] >> kBucketShift);
    if (key[j] && rel < kWindow) atomicAdd(&sh.hist[rel], 1u);
  }
  __syncthreads();
  // wave 0 finds the bound: four rounds over 256 buckets each, lane l taking
  // buckets [4l, 4l + 4) of the round (contiguous 16-byte reads, no bank
  // conflicts), a prefix sum over the wave plus the rounds before; the lane
  // where the count reaches `want` names the bucket
  if (w == 0) {
    uint32_t v = 1u;                    // fewer than `want` keys in the window: every key
    uint32_t carry = 0u;
#pragma unroll
    for (int q = 0; q < kWindow / 256; ++q) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(&sh.hist[256 * q + 4 * lane]);
      const uint32_t s4 = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = carry + wave_inclusive_scan(s4);
      const uint32_t excl = incl - s4;
      const uint64_t hit = __ballot(excl < want && want <= incl);
      if (hit) {
        const uint32_t c0 = excl + h[0], c1 = c0 + h[1], c2 = c1 + h[2];
        const int y = c0 >= want ? 0 : c1 >= want ? 1 : c2 >= want ? 2 : 3;
        const int r = __shfl(256 * q + 4 * lane + y, int(__ffsll(static_cast<long long>(hit))) - 1);
        v = uint32_t(top - r) << kBucketShift;
        break;
      }
      carry = uint32_t(__shfl(int(incl), 63));
    }
    if (lane == 0) sh.v = v;
  }
  __syncthreads();
  const uint32_t lo = sh.v;
  uint64_t bal[kP];
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    bal[j] = __ballot(key[j] != 0u && key[j] >= lo);
    if (lane == 0) sh.wc[j * kW + w] = uint32_t(__popcll(bal[j]));
  }
  __syncthreads();
  // exclusive offsets of the 32 (key j, wave) groups in index order
  const uint32_t cw = lane < 32 ? sh.wc[lane] : 0u;
  const uint32_t gincl = wave_inclusive_scan(cw);
  const uint32_t ex = gincl - cw;
  const uint64_t below = (uint64_t(1) << lane) - 1u;
  uint32_t* const ck = ws.key + slot * kSliceCap;
  int32_t* const ci = ws.idx + slot * kSliceCap;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const uint32_t pos = uint32_t(__shfl(int(ex), j * kW + w)) + uint32_t(__popcll(bal[j] & below));
    if (((bal[j] >> lane) & 1u) && pos < uint32_t(kSliceCap)) {
      ck[pos] = key[j];
      ci[pos] = base + j * kT + tid;
    }
  }
  const uint32_t total = uint32_t(__shfl(int(gincl), 31));   // all lanes take part
  if (tid == 0) {
    ws.count[slot] = total;
    ws.bound[slot] = lo;
    ws.top[slot] = mx;
  }
}

// Empty slice (no visible entry): no candidates, no bound.
CSA_DEV void slice_empty(size_t slot, const SplitWs& ws) {
  if (threadIdx.x == 0) {
    ws.count[slot] = 0u;
    ws.bound[slot] = 0u;
    ws.top[slot] = 0u;
  }
}

// The row pass of the split path (one 1024-thread block per row) over the
// slice results in `ws`; `scores` [rows][cap] serve its fallback.  `ride`, if
// not null, is a short-block compression (m < 32, arguments already checked)
// run by extra blocks of the same launch; it must touch nothing the row pass
// reads or writes.
hipError_t launch_topk_split_rows(long rows, hipStream_t st, const float* scores, const int32_t* q_pos0, int T_q,
                                  int cap, int m, int k, int32_t* idx, const SplitWs& ws,
                                  const csa_cmp::CompressArgs* ride = nullptr);

}  // namespace csa_split
