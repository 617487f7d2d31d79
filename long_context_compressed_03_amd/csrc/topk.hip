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
// A row is held in registers, 16384 keys at a time: each thread holds 16
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
//     thread w < 512 then owns 32 consecutive indices, and one block scan of the
//     packed counts gives each selected index its slot: #greater before it +
//     min(#equal before it, equal keys still needed).
//
// Few long rows (decode) would leave most of the chip idle with one block per
// row: one CU both reads the row slowly (a lone CU draws a small share of
// HBM bandwidth) and does every per-key step.  They take a split path of two
// launches, exact for any input:
//  a. per 2048-key slice s (n_s of the row's nv keys), one block finds a
//     local bound v_s: the lower edge of the 14-bit bucket that holds the
//     slice's c_s-th largest key, c_s = min(n_s, q_s + 6 sqrt(q_s) + 6), with the slice's
//     share q_s = ceil(k n_s / nv); it stores every key >= v_s, with its
//     index, in index order.  The shares sum to at least k, so the candidate
//     set C holds at least k keys;
//  b. per row, one block gathers C into an LDS list; one histogram pass finds
//     the bucket of the k-th largest, whose keys are ranked exactly; the list
//     is emitted in order.  C holds every key of the row >= max v_s, so when
//     the selected keys are all >= max v_s the result is the row's (which
//     fails only if one slice holds far more than its share of the top k,
//     or the ties crowd a slice buffer or the list); otherwise the row
//     continues with the one-block algorithm above.
//     The row pass's launch leaves most CUs idle, so a short-block
//     compression of the same step can ride in it as extra blocks
//     (csa_compress_indexer_topk).
// Each thread holds 16 keys per register tile (not 32), so that no kernel
// here needs scratch memory: a kernel with scratch waits several
// microseconds longer for its dispatch.
#include "split.hpp"
#include "compress_core.hpp"

namespace {

using namespace csa_sel;
using namespace csa_split;

constexpr int kPer = 4;                        // rounds of 4 keys per thread
constexpr int kRound = kThreads * 4;           // 4096 consecutive keys per round
constexpr int kSuper = kRound * kPer;          // 16384 keys in registers
constexpr int kWords = kSuper / 32;            // bitmap words per super-tile
constexpr int kBuckets = 1 << (32 - kBucketShift);   // 14-bit buckets
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

// split path: the row pass
constexpr int kList = 8192;                    // candidates per row held in LDS
constexpr int kListBits = 9;                   // list histogram: 512 buckets over [lo, top]
constexpr int kListBuckets = 1 << kListBits;
constexpr int kPreLoads = 8;                   // candidate entries per lane loaded with the counts

struct ListShared {
  uint32_t key[kList];
  int32_t idx[kList];
  uint32_t hist[2048];                         // the list histogram; the radix passes of refine (<= 11 bits)
  uint32_t off[kMaxSlices];
  uint32_t cnt[kMaxSlices];
  uint32_t wred[48];                           // per-wave min bound, max bound, max key
  uint32_t rank[kRankMax];
  uint32_t n_rank;
  uint32_t smem[32];
  Sel sel, sel2;
};

union RowShared {
  Shared full;
  ListShared list;
};

CSA_DEV int visible_entries(const int32_t* q_pos0, int T_q, int row, int cap, int m) {
  const int b = row / T_q;
  const int t = q_pos0[b] + (row - b * T_q);
  return max(0, min((t + 1) / m, cap));
}

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

// Scores of slice s: thread t holds indices base + j*256 + t (coalesced, and
// a wave ballot over key j covers 64 consecutive indices); n_load bounds the
// loads (the row's end), the visible count masks them afterwards.
CSA_DEV void load_slice(const float* __restrict__ src, int base, int n_load, float (&v)[kSlicePer]) {
#pragma unroll
  for (int j = 0; j < kSlicePer; ++j) {
    const int x = j * kSliceThreads + int(threadIdx.x);
    v[j] = x < n_load ? src[base + x] : 0.f;
  }
}

// Pass a, one block per slice: v_s = the lower edge of the 14-bit bucket
// that holds the slice's c_s-th largest key, c_s = min(n_s, q_s + 6 sqrt(q_s) + 6)
// with q_s = ceil(k n_s / nv) (1 = every key when the window below the top
// bucket holds fewer than c_s keys); then the slice's keys >= v_s and their
// indices, in index order, into its buffer (at most kSliceCap stored;
// count[row][s] is the full count, bound[row][s] = v_s; an empty slice
// stores count 0 and bound 0).
__global__ __launch_bounds__(kSliceThreads) void slice_select_kernel(const float* __restrict__ scores,
                                                                     const int32_t* __restrict__ q_pos0, int T_q,
                                                                     int cap, int m, int k, int G, SplitWs ws) {
  __shared__ SliceShared sh;
  const int row = blockIdx.y, sl = blockIdx.x, tid = threadIdx.x;
  const int base = sl * kSlice;
  // the scores load alongside the query position (they do not depend on it)
  float v[kSlicePer];
  load_slice(scores + size_t(row) * cap, base, min(kSlice, cap - base), v);
  const int nv = visible_entries(q_pos0, T_q, row, cap, m);
  asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
  if (nv <= k) return;
  const int n_s = min(kSlice, nv - base);
  const size_t slot = size_t(row) * G + sl;
  if (n_s <= 0) {
    slice_empty(slot, ws);
    return;
  }
  uint32_t key[kSlicePer];
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < kSlicePer; ++j) {
    key[j] = j * kSliceThreads + tid < n_s ? ordered_key(v[j]) : 0u;
    mx = max(mx, key[j]);
  }
  mx = wave_umax(mx);
  if ((tid & 63) == 0) sh.smax[tid >> 6] = mx;
  clear_window<kSliceThreads>(sh);
  __syncthreads();
  slice_finish<kSliceThreads>(key, base, n_s, nv, k, slot, ws, sh);
}

// Pass c, gathering: the row's candidates into the LDS list in index order.
// The counts, the bounds and the first entries of each wave's slices are
// loaded together: kPreLoads entries per lane spread over the wave's first
// spw slices (spw = slices per wave, up to 8; 512/spw entries of each),
// entries past a slice's count read but unused.
// Returns the list size, or -1 (block-uniform) when the candidates do not
// fit; lo / hi = min / max over the slices' bounds (empty slices ignored),
// top = max candidate key.
// The selection's histogram and rank counter start at zero: cleared by the
// gathers before their last barrier (the list does not overlap them).
CSA_DEV void clear_list_hist(ListShared& sh) {
  for (int j = threadIdx.x; j < kListBuckets; j += kThreads) sh.hist[j] = 0u;
  if (threadIdx.x == 0) sh.n_rank = 0u;
}

// Pass c, gathering, for rows of at most 64 slices: every wave reads the
// counts, bounds and largest keys of all the row's slices itself (lane x:
// slice x) and takes their prefix sums, the bounds and the largest key with
// wave operations, so the only barrier is the one that publishes the list.
// Same results and contract as gather_list.
CSA_DEV int gather_list_wave(const SplitWs& ws, int row, int G, int k, ListShared& sh, uint32_t& lo, uint32_t& hi,
                             uint32_t& top) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int kWaves = kThreads / 64;
  const size_t rbase = size_t(row) * G;
  const bool own = lane < G;
  const size_t at_s = rbase + (own ? lane : 0);   // address-selected: every lane loads
  const uint32_t c_raw = ws.count[at_s], b_raw = ws.bound[at_s], t_raw = ws.top[at_s];
  const int spw_need = (G + kWaves - 1) / kWaves;
  const int spw = spw_need <= 1 ? 1 : spw_need <= 2 ? 2 : spw_need <= 4 ? 4 : 8;
  const int per = kPreLoads / spw;
  uint32_t pk[kPreLoads];
  int32_t pi[kPreLoads];
#pragma unroll
  for (int i = 0; i < kPreLoads; ++i) {
    const int sl = w + kWaves * (i / per);
    const size_t at = (rbase + (sl < G ? sl : 0)) * kSliceCap + lane + 64 * (i % per);
    pk[i] = sl < G ? ws.key[at] : 0u;
    pi[i] = sl < G ? ws.idx[at] : 0;
  }
  const uint32_t cl = own ? c_raw : 0u;
  const uint32_t bl = own ? b_raw : 0u;
  const uint32_t incl = wave_inclusive_scan(cl);
  const uint32_t total = uint32_t(__shfl(int(incl), 63));
  const uint32_t excl = incl - cl;
  lo = wave_umin(bl != 0u ? bl : 0xFFFFFFFFu);
  hi = wave_umax(bl);
  top = wave_umax(own ? t_raw : 0u);
  const bool over = __ballot(cl > uint32_t(kSliceCap)) != 0ull;
  if (over || total > uint32_t(kList) || total < uint32_t(k)) return -1;   // every wave sees the same
#pragma unroll
  for (int i = 0; i < kPreLoads; ++i) {
    const int sl = w + kWaves * (i / per);
    if (sl < G) {
      const uint32_t o = uint32_t(__shfl(int(excl), sl)), n = uint32_t(__shfl(int(cl), sl));
      const uint32_t x = uint32_t(lane + 64 * (i % per));
      if (x < n) {
        sh.key[o + x] = pk[i];
        sh.idx[o + x] = pi[i];
      }
    }
  }
  clear_list_hist(sh);
  // the rest: entries past the early ones, and the slices beyond them
  for (int sl = w; sl < G; sl += kWaves) {
    const uint32_t o = uint32_t(__shfl(int(excl), sl)), n = uint32_t(__shfl(int(cl), sl));
    const uint32_t x0 = sl < w + kWaves * spw ? uint32_t(64 * per) : 0u;
    for (uint32_t x = x0 + lane; x < n; x += 64) {
      sh.key[o + x] = ws.key[(rbase + sl) * kSliceCap + x];
      sh.idx[o + x] = ws.idx[(rbase + sl) * kSliceCap + x];
    }
  }
  __syncthreads();
  return int(total);
}

CSA_DEV int gather_list(const SplitWs& ws, int row, int G, int k, ListShared& sh, uint32_t& lo, uint32_t& hi,
                        uint32_t& top) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int kWaves = kThreads / 64;
  const size_t rbase = size_t(row) * G;
  if (G <= 64) return gather_list_wave(ws, row, G, k, sh, lo, hi, top);
  const uint32_t c = tid < G ? ws.count[rbase + tid] : 0u;
  const uint32_t bnd = tid < G ? ws.bound[rbase + tid] : 0u;
  uint32_t b = bnd != 0u ? bnd : 0xFFFFFFFFu;
  uint32_t bh = bnd;
  // slices per wave (power of two, at most kPreLoads) and entries of each
  const int spw_need = (G + kWaves - 1) / kWaves;
  const int spw = spw_need <= 1 ? 1 : spw_need <= 2 ? 2 : spw_need <= 4 ? 4 : 8;
  const int per = kPreLoads / spw;
  uint32_t pk[kPreLoads];
  int32_t pi[kPreLoads];
#pragma unroll
  for (int i = 0; i < kPreLoads; ++i) {
    const int sl = w + kWaves * (i / per);
    const size_t at = (rbase + (sl < G ? sl : 0)) * kSliceCap + lane + 64 * (i % per);
    pk[i] = sl < G ? ws.key[at] : 0u;
    pi[i] = sl < G ? ws.idx[at] : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    b = min(b, uint32_t(__shfl_xor(int(b), o)));
    bh = max(bh, uint32_t(__shfl_xor(int(bh), o)));
  }
  if (lane == 0) {
    sh.wred[w] = b;
    sh.wred[16 + w] = bh;
  }
  if (tid < G) sh.cnt[tid] = c;
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(c, sh.smem, &total);   // its barriers publish wred, cnt
  if (tid < G) sh.off[tid] = excl;
  lo = sh.wred[0];
  hi = sh.wred[16];
#pragma unroll
  for (int x = 1; x < kWaves; ++x) {
    lo = min(lo, sh.wred[x]);
    hi = max(hi, sh.wred[16 + x]);
  }
  const bool over = __syncthreads_or(c > uint32_t(kSliceCap));
  if (over || total > uint32_t(kList) || total < uint32_t(k)) return -1;
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < kPreLoads; ++i) {
    const int sl = w + kWaves * (i / per);
    if (sl < G) {
      const uint32_t o = sh.off[sl], n = sh.cnt[sl];
      const uint32_t x = uint32_t(lane + 64 * (i % per));
      if (x < n) {
        sh.key[o + x] = pk[i];
        sh.idx[o + x] = pi[i];
        mx = max(mx, pk[i]);
      }
    }
  }
  // the rest: entries past the early ones, and the slices beyond them
  for (int sl = w; sl < G; sl += kWaves) {
    const uint32_t o = sh.off[sl], n = sh.cnt[sl];
    const uint32_t x0 = sl < w + kWaves * spw ? uint32_t(64 * per) : 0u;
    for (uint32_t x = x0 + lane; x < n; x += 64) {
      const uint32_t kk = ws.key[(rbase + sl) * kSliceCap + x];
      sh.key[o + x] = kk;
      sh.idx[o + x] = ws.idx[(rbase + sl) * kSliceCap + x];
      mx = max(mx, kk);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, uint32_t(__shfl_xor(int(mx), o)));
  if (lane == 0) sh.wred[32 + w] = mx;
  clear_list_hist(sh);
  __syncthreads();
  top = sh.wred[32];
#pragma unroll
  for (int x = 1; x < kWaves; ++x) top = max(top, sh.wred[32 + x]);
  return int(total);
}

// Pass c, selection: the k largest of the nc list keys (all >= lo, at most
// top; nc >= k), written to out in list order (= index order).  One
// histogram pass over [lo, top] in at most 512 buckets; one wave finds the
// bucket of the k-th largest; that bucket's keys are ranked exactly (a
// crowded bucket takes the exact radix refinement over the list instead).
// The list holds every row key >= hi (each slice kept all of its keys >= its
// bound, hi the largest bound), so when the selected keys are all >= hi the
// list's top k are the row's top k, ties included.  Otherwise nothing is
// written and false is returned (block-uniform).
CSA_DEV bool list_select_emit(int nc, uint32_t lo, uint32_t hi, uint32_t top, int k, int32_t* __restrict__ out,
                              ListShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // sh.hist and sh.n_rank were cleared by the gather, behind its last barrier
  const uint32_t range = top - lo;
  const int bits = range == 0u ? 0 : 32 - __clz(range);
  const int shift = bits > kListBits ? bits - kListBits : 0;
  for (int x = tid; x < nc; x += kThreads) atomicAdd(&sh.hist[(sh.key[x] - lo) >> shift], 1u);
  __syncthreads();
  if (w == 0) {
    // lane l holds the kBL buckets below hi = kListBuckets - 1 - kBL l, in registers
    constexpr int kBL = kListBuckets / 64;
    const int hi = kListBuckets - 1 - kBL * lane;
    const u32x4* h4 = reinterpret_cast<const u32x4*>(sh.hist + hi - (kBL - 1));
    u32x4 hv[kBL / 4];
    uint32_t sum = 0u;
#pragma unroll
    for (int q = 0; q < kBL / 4; ++q) {
      hv[q] = h4[q];
      sum += hv[q][0] + hv[q][1] + hv[q][2] + hv[q][3];
    }
    const uint32_t incl = wave_inclusive_scan(sum);
    const uint32_t excl = incl - sum;
    if (excl < uint32_t(k) && uint32_t(k) <= incl) {
      uint32_t run = excl;
      bool found = false;
#pragma unroll
      for (int y = kBL - 1; y >= 0; --y) {     // bucket hi - (kBL - 1) + y, from the top down
        const uint32_t cy = hv[y >> 2][y & 3];
        if (!found && run + cy >= uint32_t(k)) {
          sh.sel.bin = uint32_t(hi - (kBL - 1) + y);
          sh.sel.remaining = uint32_t(k) - run;
          sh.sel.bincount = cy;
          found = true;
        }
        run += cy;
      }
    }
  }
  __syncthreads();
  const uint32_t B = sh.sel.bin, r = sh.sel.remaining, cB = sh.sel.bincount;
  uint32_t prefix, mask = 0xFFFFFFFFu, remaining;
  if (cB <= uint32_t(kRankMax)) {
    for (int x = tid; x < nc; x += kThreads) {
      const uint32_t kk = sh.key[x];
      if (((kk - lo) >> shift) == B) sh.rank[atomicAdd(&sh.n_rank, 1u)] = kk;
    }
    __syncthreads();
    if (uint32_t(tid) < cB) {
      const uint32_t mine = sh.rank[tid];
      uint32_t n_gt = 0u, n_eq = 0u;
      for (uint32_t y = 0; y < cB; ++y) {
        const uint32_t o = sh.rank[y];
        n_gt += o > mine ? 1u : 0u;
        n_eq += o == mine ? 1u : 0u;
      }
      if (n_gt < r && r <= n_gt + n_eq) {   // equal keys write equal values
        sh.sel2.bin = mine;
        sh.sel2.remaining = r - n_gt;
      }
    }
    __syncthreads();
    prefix = sh.sel2.bin;
    remaining = sh.sel2.remaining;
  } else {
    prefix = 0u;
    mask = 0u;
    remaining = uint32_t(k);
    auto each_cand = [&](auto fn) {
      for (int x = tid; x < nc; x += kThreads) fn(sh.key[x]);
    };
    refine(each_cand, prefix, mask, remaining, sh);
  }
  // every selected key has (key & mask) >= prefix, so key >= prefix
  if (prefix < hi) return false;
  // emission: thread t walks list entries [t*per, t*per + per) in index order
  const int per = (nc + kThreads - 1) / kThreads;
  const int x0 = tid * per, x1 = min(nc, x0 + per);
  uint32_t n_gt = 0u, n_eq = 0u;
  for (int x = x0; x < x1; ++x) {
    const uint32_t km = sh.key[x] & mask;
    n_gt += km > prefix ? 1u : 0u;
    n_eq += km == prefix ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan((n_eq << 16) | n_gt, sh.smem, &tot, false);   // last use of smem
  uint32_t gt_before = ex & 0xFFFFu, eq_before = ex >> 16;
  for (int x = x0; x < x1; ++x) {
    const uint32_t km = sh.key[x] & mask;
    if (km > prefix) {
      out[gt_before + min(eq_before, remaining)] = sh.idx[x];
      ++gt_before;
    } else if (km == prefix) {
      if (eq_before < remaining) out[gt_before + eq_before] = sh.idx[x];
      ++eq_before;
    }
  }
  return true;
}

// Blocks past the rows of a split-path launch: a short-block compression
// (m < 32) that rides along on CUs the rows leave idle, 64 entries per block
// (one 16-lane group each).  The launch that adds these blocks guarantees that
// the compression touches nothing the selection reads or writes.
CSA_DEV void compress_part(const csa_cmp::CompressArgs& c, int blk) {
  using namespace csa_cmp;
  const int ne = c.L / c.m;
  const long gid = long(blk) * (kThreads / kGroup) + int(threadIdx.x) / kGroup;
  if (gid >= long(c.B) * ne) return;   // whole 16-lane groups leave together
  const int lane_c = threadIdx.x & (kGroup - 1);
#define CSA_RIDE(F, O) \
  compress_group<F, O>(c.k, c.v, c.logits, ne, c.ld_in, c.m, c.k_out, c.v_out, c.k_scale, c.v_scale, c.ld_out, gid, lane_c)
  if (c.in_dtype == CSA_F32) {
    if (c.out_dtype == CSA_F32) CSA_RIDE(1, CSA_F32);
    else if (c.out_dtype == CSA_BF16) CSA_RIDE(1, CSA_BF16);
    else CSA_RIDE(1, CSA_FP8_E4M3);
  } else {
    if (c.out_dtype == CSA_F32) CSA_RIDE(0, CSA_F32);
    else if (c.out_dtype == CSA_BF16) CSA_RIDE(0, CSA_BF16);
    else CSA_RIDE(0, CSA_FP8_E4M3);
  }
#undef CSA_RIDE
}

template <bool kSplit>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ q_pos0, int T_q, int cap, int m,
                                                        int k, int32_t* __restrict__ idx, SplitWs ws, int G, int rows,
                                                        csa_cmp::CompressArgs ride) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  RowShared& rs = *reinterpret_cast<RowShared*>(smem_raw);
  Shared& sh = rs.full;

  if constexpr (kSplit) {
    if (int(blockIdx.x) >= rows) {
      compress_part(ride, int(blockIdx.x) - rows);
      return;
    }
  }
  const int row = blockIdx.x;
  const int b = row / T_q;
  const int i = row - b * T_q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = q_pos0[b] + i;
  int32_t* out = idx + size_t(row) * k;
  // split path: the candidates are gathered before the visibility is known
  // (their loads overlap the query position's); a row that needs no
  // selection leaves them unused (its buffers then hold stale counts, which
  // the gather's size checks reject before any is used as a size)
  uint32_t lo = 0u, hi = 0u, top = 0u;
  int nc = -1;
  if constexpr (kSplit) nc = gather_list(ws, row, G, k, rs.list, lo, hi, top);
  int nv = (t + 1) / m;
  nv = max(0, min(nv, cap));
  if (nv <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const float* src = scores + size_t(row) * cap;
  if constexpr (kSplit) {
    if (nc >= 0 && list_select_emit(nc, lo, hi, top, k, out, rs.list)) return;
    __syncthreads();
  }
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
    const uint32_t wg = tid < kWords ? sh.bm_gt[tid] : 0u;   // thread t owns word t (32 indices)
    const uint32_t we = tid < kWords ? sh.bm_eq[tid] : 0u;
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

template <bool kSplit>
hipError_t set_lds_limit() {
  return csa_lds_opt_in(reinterpret_cast<const void*>(&topk_kernel<kSplit>), sizeof(RowShared));
}

hipError_t launch_topk(long rows, hipStream_t st, const float* scores, const int32_t* q_pos0, int T_q, int cap, int m,
                       int k, int32_t* idx, void* ws) {
  if (!use_split(rows, cap)) {
    hipError_t e = set_lds_limit<false>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel<false>, dim3(unsigned(rows)), dim3(kThreads), sizeof(RowShared), st, scores, q_pos0,
                       T_q, cap, m, k, idx, SplitWs{}, 0, int(rows), csa_cmp::CompressArgs{});
    return hipGetLastError();
  }
  const int G = n_slices(cap);
  const SplitWs w = split_ws(ws, rows, cap);
  const dim3 grid{unsigned(G), unsigned(rows), 1u};
  hipLaunchKernelGGL(slice_select_kernel, grid, dim3(kSliceThreads), 0, st, scores, q_pos0, T_q, cap, m, k, G, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_split_rows(rows, st, scores, q_pos0, T_q, cap, m, k, idx, w);
}

}  // namespace

hipError_t csa_split::launch_topk_split_rows(long rows, hipStream_t st, const float* scores, const int32_t* q_pos0,
                                             int T_q, int cap, int m, int k, int32_t* idx, const SplitWs& ws,
                                             const csa_cmp::CompressArgs* ride) {
  hipError_t e = set_lds_limit<true>();
  if (e != hipSuccess) return e;
  long extra = 0;
  csa_cmp::CompressArgs c{};
  if (ride) {
    c = *ride;
    const long entries = long(c.B) * (c.L / c.m);
    extra = (entries + kThreads / csa_cmp::kGroup - 1) / (kThreads / csa_cmp::kGroup);
  }
  hipLaunchKernelGGL(topk_kernel<true>, dim3(unsigned(rows + extra)), dim3(kThreads), sizeof(RowShared), st, scores,
                     q_pos0, T_q, cap, m, k, idx, ws, n_slices(cap), int(rows), c);
  return hipGetLastError();
}

extern "C" csa_status_t csa_topk(const float* scores, const int32_t* q_pos0, int32_t B, int32_t T_q, int32_t cap,
                                 int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !q_pos0 || !idx) return CSA_EINVAL;
  if (B < 0 || T_q < 0 || cap < 0 || m < 1 || k < 1) return CSA_EINVAL;
  const long rows = long(B) * T_q;
  if (rows == 0) return CSA_OK;
  if (rows > 0x7FFFFFFFL) return CSA_ENOTSUP;
  if (use_split(rows, cap) && (!ws || ws_bytes < split_ws_bytes(rows, cap))) return CSA_EWORKSPACE;
  const hipError_t e = launch_topk(rows, static_cast<hipStream_t>(stream), scores, q_pos0, T_q, cap, m, k, idx, ws);
  return e == hipSuccess ? CSA_OK : CSA_EHIP;
}

size_t csa_topk_workspace_size(long rows, int cap) { return use_split(rows, cap) ? split_ws_bytes(rows, cap) : 0; }
