// csa_indexer_topk: the lightning indexer and the top-k selection fused, so
// the fp32 scores of a prefill chunk (T_q x cap of them) never reach HBM.
//
// Passages: the indexer scores every query token against every compressed
// block in FP4 (sz-guanghua.com.cn ifanr repost, 百萬長上下文) and CSA keeps the
// k entries it finds most relevant (blog.nickys.cn DeepSeek-V4 post,
// 三大架构改动 §1 CSA).  The result is by construction identical, bit for bit,
// to csa_topk applied to csa_indexer_scores.
//
// Two kernels:
//  1. the indexer kernel of csa_indexer_scores, writing for each visible
//     (query, entry) the top 16 bits of the order-preserving uint32 key of its
//     score (half the bytes of the fp32 score) into the workspace;
//  2. per query row one 1024-thread block.  The row's first 65536 (or 32768)
//     16-bit keys are held in registers, two per register; keys past that are
//     streamed from the workspace 16384 at a time.
//     a. estimate: a histogram of 14-bit buckets over a fixed 1/8 sample of
//        the held keys gives, from the sample ranks k*(sample/row) -+ a
//        margin of 4 standard deviations (+16), a window of buckets that
//        should hold the k-th largest key;
//     b. one pass counts the keys above the window (one LDS atomic per wave)
//        and lists the keys inside it (index and 16-bit key);
//     c. if the window does hold the k-th key, an exact histogram of the
//        listed 16-bit keys gives the k-th 16-bit key T; otherwise (a miss,
//        or a window too full for the list) a histogram of 14-bit buckets over
//        every key does, and T is that bucket;
//     d. keys above T are selected outright, keys below are not; the entries
//        whose key equals T are RE-SCORED with the indexer's own instruction
//        sequence (same MFMA, same operand values, same head-sum order),
//        which gives back their exact fp32 scores, and an exact radix
//        refinement over their full 32-bit keys finds the k-th key and how
//        many keys equal to it are still needed (when T's class holds more
//        entries than the list, it is re-scored in rounds of 4096 keys);
//     e. emission as in csa_topk: bitmaps of "greater" and "equal" entries,
//        one block scan, ascending output with the lower-index tie rule.
#include <utility>

#include "indexer_core.hpp"
#include "split.hpp"

namespace {

using namespace csa_sel;
using namespace csa_ix;

constexpr int kRound = kThreads * 4;   // 4096 consecutive keys per round of loads
constexpr int kBatch = 4;              // rounds streamed per batch (16 loads in flight)
constexpr int kList = 4096;            // capacity of the LDS entry lists
constexpr int kWinPer = kList / (kThreads / 64);   // window-list slots of each wave
constexpr int kBuckets = 1 << 14;      // 14-bit buckets of the 16-bit keys
constexpr int kMaxJ = 20;              // rounds held in registers, largest variant
constexpr int kMaxWords = kMaxJ * kRound / 32;
static_assert(kMaxJ % kBatch == 0, "chunks are whole batches of rounds");

struct Shared {
  uint32_t hist[kBuckets];
  struct {
    uint32_t gt[kMaxWords];   // index-ordered bitmaps of one chunk: selected outright,
    uint32_t eq[kMaxWords];   // and equal to the k-th key (taken lowest index first)
  } bm;
  int32_t win_idx[kList];     // window entries (index): wave w fills [w*kWinPer, +win_cnt[w])
  uint16_t win_key[kList];    // their 16-bit keys
  uint32_t win_cnt[kThreads / 64];
  int32_t cand_idx[kList];    // entries to re-score
  uint32_t cand_key[kList];   // their exact 32-bit keys
  uint32_t smem[32];
  uint32_t n_win, n_gt, n_cand;
  Sel sel, sel2;
};

// 16-bit key (j, c) from the packed registers (c = 0..3 within round j).
template <int kJ>
CSA_DEV uint32_t kget(const uint32_t (&P)[kJ][2], int j, int c) {
  return (P[j][c >> 1] >> ((c & 1) * 16)) & 0xFFFFu;
}

// Tells the compiler the packed keys may have changed, so values unpacked
// from them in one phase are recomputed in the next instead of being held in
// registers across it (which would not fit beside the keys themselves).
template <int kJ>
CSA_DEV void opaque(uint32_t (&P)[kJ][2]) {
#pragma unroll
  for (int j = 0; j < kJ; ++j) asm volatile("" : "+v"(P[j][0]), "+v"(P[j][1]));
}

// Index of key (j, c) of thread (w, l) in a chunk: j*4096 + c*1024 + 64w + l,
// so a wave-wide load reads 64 consecutive keys and a wave ballot is two
// words of an index-ordered bitmap.
CSA_DEV int key_offset(int j, int c) { return j * kRound + c * kThreads + int(threadIdx.x); }

// Buffer resource over keys [0, nv) of a row: loads past nv return 0, which
// is the "absent" key, so no load needs a bounds test of its own.
CSA_DEV __amdgpu_buffer_rsrc_t row_rsrc(const uint16_t* src, int nv) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), (short)0, nv * 2, 0x00020000);
}

// Key at index x0 + c*1024 + threadIdx.x for c = 0..3 (x0 a multiple of
// 4096); the byte offset is all in the VGPR operand, so the range check of
// the resource covers it.
CSA_DEV void load4(__amdgpu_buffer_rsrc_t r, int x0, uint32_t (&v)[4]) {
  const int o0 = (x0 + int(threadIdx.x)) * 2;
  v[0] = __builtin_amdgcn_raw_buffer_load_b16(r, o0, 0, 0);
  v[1] = __builtin_amdgcn_raw_buffer_load_b16(r, o0 + 2048, 0, 0);
  v[2] = __builtin_amdgcn_raw_buffer_load_b16(r, o0 + 4096, 0, 0);
  v[3] = __builtin_amdgcn_raw_buffer_load_b16(r, o0 + 6144, 0, 0);
}

// The first chunk (kJ rounds) of a row into registers, every load in flight
// at once (nothing else is live yet).
template <int kJ>
CSA_DEV void load_chunk0(__amdgpu_buffer_rsrc_t r, uint32_t (&P)[kJ][2]) {
  uint32_t v[kJ][4];
#pragma unroll
  for (int j = 0; j < kJ; ++j) load4(r, j * kRound, v[j]);
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    P[j][0] = v[j][0] | (v[j][1] << 16);
    P[j][1] = v[j][2] | (v[j][3] << 16);
  }
}

// Streams keys [r_begin, r_end) (r_begin a multiple of 4096) in batches of
// kBatch rounds; fn(v, base) sees the batch's keys v[j][c] = key at base +
// key_offset(j, c) (0 past nv).  Every thread must call it.
template <typename Fn>
CSA_DEV void stream_batches(__amdgpu_buffer_rsrc_t r, int r_begin, int r_end, Fn fn) {
#pragma unroll 1
  for (int base = r_begin; base < r_end; base += kBatch * kRound) {
    uint32_t v[kBatch][4];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) load4(r, base + j * kRound, v[j]);
    fn(v, base);
  }
}

// Appends to an LDS list the keys of a batch of kR rounds (given by get(j, c))
// that satisfy in_window and, when n_above is given, counts the keys that
// satisfy above.  Each thread counts its own keys, one wave scan of the packed
// counts gives each thread its slots, and one LDS atomic per wave reserves
// the wave's range (list order is therefore not index order; nothing
// downstream depends on it).  Entries past the list capacity are counted but
// not stored.  between() runs between the counting and the storing pass (a
// register barrier for keys unpacked from packed registers).
template <int kR, typename Get, typename In, typename Above, typename Between>
CSA_DEV void list_batch(Get get, int base, In in_window, Above above, int32_t* idx_out, uint16_t* key_out,
                        uint32_t* n_list, uint32_t* n_above, Between between) {
  const int lane = threadIdx.x & 63;
  uint32_t cnt = 0u, n_gt = 0u;
#pragma unroll
  for (int j = 0; j < kR; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kk = get(j, c);
      cnt += in_window(kk) ? 1u : 0u;
      if (n_above) n_gt += above(kk) ? 1u : 0u;
    }
  // inclusive wave scan of (above << 16 | listed); both totals stay below 2^16
  const uint32_t packed = (n_gt << 16) | cnt;
  uint32_t incl = packed;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const uint32_t wave_tot = __shfl(incl, 63);
  uint32_t at = 0u;
  if (lane == 63) {
    if (wave_tot & 0xFFFFu) at = atomicAdd(n_list, wave_tot & 0xFFFFu);
    if (n_above && (wave_tot >> 16)) atomicAdd(n_above, wave_tot >> 16);
  }
  uint32_t slot = __shfl(at, 63) + ((incl - packed) & 0xFFFFu);
  between();
#pragma unroll
  for (int j = 0; j < kR; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kk = get(j, c);
      if (in_window(kk)) {
        if (slot < uint32_t(kList)) {
          idx_out[slot] = base + key_offset(j, c);
          if (key_out) key_out[slot] = uint16_t(kk);
        }
        ++slot;
      }
    }
}

// One pass of the window step over a batch of kR rounds (keys from get(j, c),
// chunk offsets base + key_offset(j, c)): keys above hi16 are counted (a
// per-wave scalar sum, one LDS atomic at the end) and, when bm_above is given
// (a batch that is a whole chunk), set in the chunk's index-ordered bitmap;
// keys in [lo16, hi16] are appended to the wave's own region of the window
// list at a wave-uniform running count (n_in; a count past the region's size
// marks an overflow).  lo16 > 0, so absent keys (0) are in neither set.
// `word` with lane L replaced by the wave-uniform `val` (V_WRITELANE_B32, no
// exec-mask change).  `val` is usually a ballot just written by a vector
// compare: reading such a scalar register in V_WRITELANE needs wait states,
// which the compiler inserts for its own instructions but not inside asm, so
// the asm carries them itself.
template <int L>
CSA_DEV uint32_t write_lane(uint32_t word, uint32_t val) {
  asm("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(word) : "s"(val), "n"(L));
  return word;
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
CSA_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
CSA_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int kR, typename Get>
CSA_DEV void window_pass(Get get, int base, uint32_t lo16, uint32_t hi16, uint32_t* bm_above, uint32_t& n_in,
                         Shared& sh) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint32_t span = hi16 - lo16;
  uint32_t n_above = 0u;                 // wave-uniform
  // bitmap words collected in VGPR lanes: group i = 4j + c puts its two ballot
  // words in lanes 2i and 2i + 1 (no exec-mask flips, no scalar registers
  // held across the pass); one store per lane at the end
  constexpr int kWords = (kR * 4 * 2 + 63) / 64;
  uint32_t words[kWords];
#pragma unroll
  for (int q = 0; q < kWords; ++q) words[q] = 0u;
  static_for<kR * 4>([&](auto I) {
    constexpr int gi = decltype(I)::value;
    const int j = gi / 4, c = gi % 4;
    const uint32_t kk = get(j, c);
    const uint64_t bab = __ballot(kk > hi16);
    n_above += uint32_t(__popcll(bab));
    if (bm_above) {
      constexpr int i2 = 2 * gi;
      words[i2 / 64] = write_lane<i2 % 64>(words[i2 / 64], uint32_t(bab));
      words[(i2 + 1) / 64] = write_lane<(i2 + 1) % 64>(words[(i2 + 1) / 64], uint32_t(bab >> 32));
    }
    const bool in = kk - lo16 <= span;
    const uint64_t bin = __ballot(in);
    const uint32_t slot =
        n_in + __builtin_amdgcn_mbcnt_hi(uint32_t(bin >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bin), 0u));
    if (in && slot < uint32_t(kWinPer)) {
      sh.win_idx[wv * kWinPer + slot] = base + key_offset(j, c);
      sh.win_key[wv * kWinPer + slot] = uint16_t(kk);
    }
    n_in += uint32_t(__popcll(bin));
  });
  if (bm_above) {
    // the wave's 64 keys of group (j, c) are indices j*4096 + c*1024 + 64w + l:
    // bitmap words (j*4096 + c*1024)/32 + 2w and the next
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const int g2 = 64 * q + lane;   // 2 * group + half
      const int gi = g2 >> 1;
      if (gi < kR * 4) bm_above[(gi >> 2) * (kRound / 32) + (gi & 3) * (kThreads / 32) + 2 * wv + (g2 & 1)] = words[q];
    }
  }
  if (lane == 0 && n_above) atomicAdd(&sh.n_gt, n_above);
}

// Visits fn(slot) for every filled slot of the window list (all threads).
template <typename Fn>
CSA_DEV void each_window(const Shared& sh, Fn fn) {
  for (int x = threadIdx.x; x < kList; x += kThreads)
    if (uint32_t(x % kWinPer) < sh.win_cnt[x / kWinPer]) fn(x);
}

// Row context for re-scoring: the row's query as the A operand, in the
// tile slot it occupies in the indexer kernel, and its head weights.
template <int kHI, int kKS>
struct Rescore {
  u32x4 a[kKS];
  int sa[kKS];
  float wv[4];
  bool mine;  // this lane's C rows belong to the row's query
};

template <int kHI, int kKS>
CSA_DEV void rescore_setup(Rescore<kHI, kKS>& R, const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                           size_t qrow, int i, int nblk, int row_bytes) {
  constexpr int kQPT = 16 / kHI;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int slot = i % kQPT;
  const bool a_mine = col / kHI == slot;
  load_a<kHI, kKS>(q_codes, q_e8m0, qrow * kHI + (col % kHI), a_mine, g, nblk, row_bytes, R.a, R.sa);
  const int rc = 4 * g;
  R.mine = rc / kHI == slot;
#pragma unroll
  for (int x = 0; x < 4; ++x) R.wv[x] = R.mine ? w[qrow * kHI + (rc + x) % kHI] : 0.f;
}

// Exact keys of the listed entries cand_idx[0..n) into cand_key[0..n); the
// 16 waves take 16-entry groups in turn.  Ends with a block barrier.
template <int kHI, int kKS>
CSA_DEV void rescore_list(const Rescore<kHI, kKS>& R, __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t re,
                          uint32_t c_bytes, uint32_t e_bytes, int n, int nblk, int row_bytes, Shared& sh) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int wid = threadIdx.x >> 6;
  for (int grp = wid; grp * 16 < n; grp += kThreads / 64) {
    const int j = grp * 16 + col;
    const int e = j < n ? sh.cand_idx[j] : 0;
    u32x4 bk[kKS];
    int sb[kKS];
    load_b<kKS, false>(rc, re, c_bytes, e_bytes, e, j < n, g, nblk, row_bytes, bk, sb);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) acc = mfma_fp4(R.a[ks], R.sa[ks], bk[ks], sb[ks], acc);
    bool writer;
    const float p = head_sum<kHI>(acc, R.wv, g, writer);
    if (writer && R.mine && j < n) sh.cand_key[j] = ordered_key(p);
  }
  __syncthreads();
}

CSA_DEV uint32_t pow2_ceil(uint32_t x) { return x <= 1u ? 1u : 1u << (32 - __clz(x - 1u)); }

template <int kHI, int kKS, int kJ>
__global__ __launch_bounds__(kThreads) void select_kernel(const uint16_t* __restrict__ key16,
                                                          const uint8_t* __restrict__ q_codes,
                                                          const uint8_t* __restrict__ q_e8m0,
                                                          const float* __restrict__ w,
                                                          const uint8_t* __restrict__ k_codes,
                                                          const uint8_t* __restrict__ k_e8m0,
                                                          const int32_t* __restrict__ q_pos0, int T_q, int d_I,
                                                          int cap, int m, int k, int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cu_rows, int n_seq,
                                                          const uint32_t* __restrict__ gate) {
  constexpr int kS = kJ * kRound;          // keys per chunk; chunk 0 stays in registers
  constexpr int kWPT = (kS / 32 + kThreads - 1) / kThreads;  // bitmap words per thread (the last ones may be past the chunk)
  static_assert(kS < (1 << 17), "a chunk's equal counts fit 17 bits");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Shared& sh = *reinterpret_cast<Shared*>(smem_raw);

  if (gate && *gate == 0u) return;   // the whole block: the fallback launch has nothing to do
  // row = packed row (sequence b, query i of it); cu_rows: packed batches
  const int row = blockIdx.x;
  const int b = cu_rows ? csa_packed_seq(cu_rows, n_seq, row) : row / T_q;
  const int i = cu_rows ? row - cu_rows[b] : row - b * T_q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = q_pos0[b] + i;
  const int nv = max(0, min((t + 1) / m, cap));
  int32_t* out = idx + size_t(row) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const uint16_t* src = key16 + size_t(row) * cap;
  const int n_chunks = (nv + kS - 1) / kS;
  const int nblk = d_I >> 5;
  const int row_bytes = d_I >> 1;
  const uint8_t* kc_seq = k_codes + size_t(b) * cap * row_bytes;
  const uint8_t* ke_seq = k_e8m0 + size_t(b) * cap * nblk;
  const uint32_t c_bytes = uint32_t(cap) * uint32_t(row_bytes);   // < 2^31 (argument check)
  const uint32_t e_bytes = uint32_t(cap) * uint32_t(nblk);
  const __amdgpu_buffer_rsrc_t rc = seq_rsrc(kc_seq, c_bytes);
  const __amdgpu_buffer_rsrc_t re = seq_rsrc(ke_seq, e_bytes);

  for (int j = tid; j < kBuckets; j += kThreads) sh.hist[j] = 0u;
  for (int j = tid; j < kS / 32; j += kThreads) sh.bm.eq[j] = 0u;
  if (tid == 0) {
    sh.n_win = 0u;
    sh.n_gt = 0u;
    sh.n_cand = 0u;
  }
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, nv);
  uint32_t P[kJ][2];
  load_chunk0<kJ>(rs, P);
  __syncthreads();

  // ---- a: sample histogram: keys (j, 0) of the even rounds j of chunk 0
  // (the first 1024 of every 8192 indices)
#pragma unroll
  for (int j = 0; j < kJ; j += 2) {
    const uint32_t kk = kget<kJ>(P, j, 0);
    if (kk) atomicAdd(&sh.hist[kk >> 2], 1u);
  }
  int n_sample = 0;
#pragma unroll
  for (int j = 0; j < kJ; j += 2) n_sample += max(0, min(nv - j * kRound, kThreads));
  __syncthreads();
  const int k_s = max(1, int((long(k) * n_sample) / nv));
  const int margin = 4 * int(sqrtf(float(k_s))) + 16;
  const uint32_t r_hi = uint32_t(max(1, k_s - margin));
  const uint32_t r_lo = uint32_t(min(n_sample, k_s + margin));
  find_bin(sh.hist, kBuckets, r_hi, &sh.sel, sh.smem);
  find_bin(sh.hist, kBuckets, r_lo, &sh.sel2, sh.smem);
  const uint32_t b_hi = sh.sel.bin, b_lo = sh.sel2.bin;   // b_lo <= b_hi

  // ---- b: keys above the window counted, keys inside listed
  {
    const uint32_t lo16 = b_lo << 2, hi16 = (b_hi << 2) | 3u;
    uint32_t n_in = 0u;
    opaque<kJ>(P);
    window_pass<kJ>([&](int j, int c) { return kget<kJ>(P, j, c); }, 0, lo16, hi16, sh.bm.gt, n_in, sh);
    stream_batches(rs, kS, nv, [&](uint32_t(&v)[kBatch][4], int base) {
      window_pass<kBatch>([&](int j, int c) { return v[j][c]; }, base, lo16, hi16, nullptr, n_in, sh);
    });
    if (lane == 0) {
      sh.win_cnt[tid >> 6] = min(n_in, uint32_t(kWinPer));
      atomicAdd(&sh.n_win, n_in);
      if (n_in > uint32_t(kWinPer)) atomicAdd(&sh.n_win, uint32_t(kList) + 1u);   // overflow: a miss
    }
  }
  __syncthreads();
  const uint32_t n_above = sh.n_gt, n_win = sh.n_win;
  const uint32_t win_bins = pow2_ceil((b_hi - b_lo + 1u) * 4u);
  const bool hit = n_above < uint32_t(k) && n_above + n_win >= uint32_t(k) && n_win <= uint32_t(kList) &&
                   win_bins <= uint32_t(kBuckets);

  // ---- c: the k-th 16-bit key T (shift 0) or, on a miss, its 14-bit bucket (shift 2)
  uint32_t thr, remaining, cnt;
  int shift;
  if (hit) {
    const uint32_t lo16 = b_lo << 2;
    for (int j = tid; j < int(win_bins); j += kThreads) sh.hist[j] = 0u;
    __syncthreads();
    each_window(sh, [&](int x) { atomicAdd(&sh.hist[uint32_t(sh.win_key[x]) - lo16], 1u); });
    __syncthreads();
    find_bin(sh.hist, int(win_bins), uint32_t(k) - n_above, &sh.sel, sh.smem);
    thr = lo16 + sh.sel.bin;
    remaining = sh.sel.remaining;
    cnt = sh.sel.bincount;
    shift = 0;
  } else {
    for (int j = tid; j < kBuckets; j += kThreads) sh.hist[j] = 0u;
    __syncthreads();
    opaque<kJ>(P);
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = kget<kJ>(P, j, c);
        if (kk) atomicAdd(&sh.hist[kk >> 2], 1u);
      }
    stream_batches(rs, kS, nv, [&](uint32_t(&v)[kBatch][4], int) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (v[j][c]) atomicAdd(&sh.hist[v[j][c] >> 2], 1u);
    });
    __syncthreads();
    find_bin(sh.hist, kBuckets, uint32_t(k), &sh.sel, sh.smem);
    thr = sh.sel.bin;
    remaining = sh.sel.remaining;
    cnt = sh.sel.bincount;
    shift = 2;
  }
  const bool whole = cnt == remaining;   // T's class is taken whole: no re-scoring
  const bool crowded = !whole && cnt > uint32_t(kList);
  const int low_bits = 16 + shift;       // exact keys of T's class share their top 32 - low_bits bits
  uint32_t prefix = thr << low_bits;
  uint32_t mask = ~((1u << low_bits) - 1u);
  auto in_class = [&](uint32_t kk) { return kk != 0u && (kk >> shift) == thr; };
  auto none = [](uint32_t) { return false; };

  // ---- d: exact keys of T's class, radix refinement
  Rescore<kHI, kKS> R;
  if (!whole) {
    rescore_setup<kHI, kKS>(R, q_codes, q_e8m0, w, size_t(row), i, nblk, row_bytes);
    if (!crowded) {
      if (hit) {
        // the class is a subset of the window list
        for (int x0 = 0; x0 < kList; x0 += kThreads) {
          const int x = x0 + tid;
          const bool want = uint32_t(x % kWinPer) < sh.win_cnt[x / kWinPer] && uint32_t(sh.win_key[x]) == thr;
          const uint64_t bal = __ballot(want);
          uint32_t at = 0u;
          if (lane == 0 && bal) at = atomicAdd(&sh.n_cand, uint32_t(__popcll(bal)));
          at = __shfl(at, 0);
          if (want) sh.cand_idx[at + __popcll(bal & ((uint64_t(1) << lane) - 1u))] = sh.win_idx[x];
        }
      } else {
        opaque<kJ>(P);
        list_batch<kJ>([&](int j, int c) { return kget<kJ>(P, j, c); }, 0, in_class, none, sh.cand_idx, nullptr,
                       &sh.n_cand, nullptr, [&] { opaque<kJ>(P); });
        stream_batches(rs, kS, nv, [&](uint32_t(&v)[kBatch][4], int base) {
          list_batch<kBatch>([&](int j, int c) { return v[j][c]; }, base, in_class, none, sh.cand_idx, nullptr,
                             &sh.n_cand, nullptr, [] {});
        });
      }
      __syncthreads();
      const int nc = int(sh.n_cand);
      rescore_list<kHI, kKS>(R, rc, re, c_bytes, e_bytes, nc, nblk, row_bytes, sh);
      auto each_listed = [&](auto fn) {
        for (int x = tid; x < nc; x += kThreads) fn(sh.cand_key[x]);
      };
      refine(each_listed, prefix, mask, remaining, sh);
    } else {
      // batches of 16384 keys read from the key row: list, re-score, visit
      auto each_batch = [&](auto fn) {
        stream_batches(rs, 0, nv, [&](uint32_t(&v)[kBatch][4], int base) {
          for (int r = 0; r < kBatch; ++r) {
            if (tid == 0) sh.n_cand = 0u;
            __syncthreads();
            list_batch<1>([&](int, int c) { return v[r][c]; }, base + r * kRound, in_class, none, sh.cand_idx,
                          nullptr, &sh.n_cand, nullptr, [] {});
            __syncthreads();
            const int nc = int(sh.n_cand);
            rescore_list<kHI, kKS>(R, rc, re, c_bytes, e_bytes, nc, nblk, row_bytes, sh);
            for (int x = tid; x < nc; x += kThreads) fn(sh.cand_key[x]);
            __syncthreads();
          }
        });
      };
      refine(each_batch, prefix, mask, remaining, sh);
    }
  }

  // ---- e: emission in index order, one chunk of kS keys at a time
  uint32_t gt_off = 0u, eq_off = 0u;
  const int wv = tid >> 6;
  auto gt_of = [&](uint32_t kk) {
    const uint32_t ck = kk >> shift;
    return kk != 0u && (whole ? ck >= thr : ck > thr);
  };
  // bitmap words of the wave's 64 keys at chunk offset off + 64w (off a
  // multiple of 1024): a per-wave base plus off/32
  uint32_t* const gt_w = sh.bm.gt + 2 * wv;
  uint32_t* const eq_w = sh.bm.eq + 2 * wv;
  auto put_words = [&](int off, uint64_t gbal) {
    if (lane == 0) {
      gt_w[off >> 5] = uint32_t(gbal);
      gt_w[(off >> 5) + 1] = uint32_t(gbal >> 32);
      eq_w[off >> 5] = 0u;
      eq_w[(off >> 5) + 1] = 0u;
    }
  };
#pragma unroll 1
  for (int ch = 0; ch < n_chunks; ++ch) {
    opaque<kJ>(P);
    __syncthreads();   // earlier readers of the bitmaps are done
    if (ch == 0 && hit) {
      // keys above the window are already marked; add the window keys above T
      // (and T's class itself when it is taken whole)
      each_window(sh, [&](int x) {
        const int e = sh.win_idx[x];
        const uint32_t kk = sh.win_key[x];
        if (e < kS && (kk > thr || (whole && kk == thr))) atomicOr(&sh.bm.gt[e >> 5], 1u << (e & 31));
      });
    } else if (ch == 0) {
#pragma unroll
      for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) put_words(j * kRound + c * kThreads, __ballot(gt_of(kget<kJ>(P, j, c))));
    } else {
      // words of rounds past nv are zero; batches holding keys are streamed
      const int r_end = min(nv, (ch + 1) * kS);
      const int w_from = ((r_end - ch * kS + kBatch * kRound - 1) / (kBatch * kRound)) * (kBatch * kRound) / 32;
      for (int x = w_from + tid; x < kS / 32; x += kThreads) {
        sh.bm.gt[x] = 0u;
        sh.bm.eq[x] = 0u;
      }
      stream_batches(rs, ch * kS, r_end, [&](uint32_t(&v)[kBatch][4], int base) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            put_words(base - ch * kS + j * kRound + c * kThreads, __ballot(gt_of(v[j][c])));
      });
    }
    __syncthreads();
    if (!whole) {
      // T's class in this chunk, by the exact keys
      auto mark = [&](int e, uint32_t kx) {
        const int x = e - ch * kS;
        if (x < 0 || x >= kS) return;
        const uint32_t km = kx & mask;
        if (km > prefix) atomicOr(&sh.bm.gt[x >> 5], 1u << (x & 31));
        else if (km == prefix) atomicOr(&sh.bm.eq[x >> 5], 1u << (x & 31));
      };
      if (!crowded) {
        const int nc = int(sh.n_cand);
        for (int x = tid; x < nc; x += kThreads) mark(sh.cand_idx[x], sh.cand_key[x]);
      } else {
        stream_batches(rs, ch * kS, min(nv, (ch + 1) * kS), [&](uint32_t(&v)[kBatch][4], int base) {
          for (int r = 0; r < kBatch; ++r) {
            if (tid == 0) sh.n_cand = 0u;
            __syncthreads();
            list_batch<1>([&](int, int c) { return v[r][c]; }, base + r * kRound, in_class, none, sh.cand_idx,
                          nullptr, &sh.n_cand, nullptr, [] {});
            __syncthreads();
            const int nc = int(sh.n_cand);
            rescore_list<kHI, kKS>(R, rc, re, c_bytes, e_bytes, nc, nblk, row_bytes, sh);
            for (int x = tid; x < nc; x += kThreads) mark(sh.cand_idx[x], sh.cand_key[x]);
            __syncthreads();
          }
        });
      }
      __syncthreads();
    }
    // thread t owns bitmap words [t*kWPT, (t+1)*kWPT) (words past the chunk's
    // kS/32 read as empty); greater counts fit 15 bits (at most k < 32768) and
    // equal counts 17 bits (<= keys per chunk)
    uint32_t wg[kWPT], we[kWPT];
    uint32_t n_g = 0u, n_e = 0u;
#pragma unroll
    for (int x = 0; x < kWPT; ++x) {
      const int wi = tid * kWPT + x;
      wg[x] = wi < kS / 32 ? sh.bm.gt[wi] : 0u;
      we[x] = wi < kS / 32 ? sh.bm.eq[wi] : 0u;
      n_g += __popc(wg[x]);
      n_e += __popc(we[x]);
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((n_g << 17) | n_e, sh.smem, &tot);
    uint32_t gt_before = gt_off + (ex >> 17);
    uint32_t eq_before = eq_off + (ex & 0x1FFFFu);
#pragma unroll
    for (int x = 0; x < kWPT; ++x) {
      const int x0 = ch * kS + (tid * kWPT + x) * 32;
      uint32_t any = wg[x] | we[x];
      while (any) {
        const int bit = __ffs(any) - 1;
        any &= any - 1u;
        if ((wg[x] >> bit) & 1u) {
          out[gt_before + min(eq_before, remaining)] = x0 + bit;
          ++gt_before;
        } else {
          if (eq_before < remaining) out[gt_before + eq_before] = x0 + bit;
          ++eq_before;
        }
      }
    }
    gt_off += tot >> 17;
    eq_off += tot & 0x1FFFFu;
  }
}

// Decoding (one query per sequence) with few rows: one block per (sequence,
// 2048-entry slice).  The block scores its slice exactly as the scoring kernel
// does (same instruction sequence, so the same bits), stores the fp32 scores
// for the row pass's fallback, keeps their order-preserving keys in LDS and
// runs the split path's slice pass on them: the scores are never read back
// for the common case.
constexpr int kFusedThreads = 1024;   // 16 waves x 128 entries: the whole slice's keys in flight at once

template <int kHI, int kKS>
__global__ __launch_bounds__(kFusedThreads) void indexer_slice_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_e8m0, const float* __restrict__ w,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_e8m0, const int32_t* __restrict__ q_pos0,
    int d_I, int cap, int m, int k, int G, float* __restrict__ scores, csa_split::SplitWs ws) {
  using namespace csa_split;
  constexpr int kFrag = 4;
  constexpr int kBatch16 = 16 * kFrag;                      // entries per batch of a wave
  constexpr int kPerWave = kSlice / (kFusedThreads / 64);   // 128 entries per wave
  constexpr int kNB = kPerWave / kBatch16;                  // batches per wave, all loaded up front
  __shared__ uint32_t skey[kSlice];
  __shared__ SliceShared sh;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int b = blockIdx.y, sl = blockIdx.x;
  const int nblk = d_I >> 5, row_bytes = d_I >> 1;
  const int nv = min((q_pos0[b] + 1) / m, cap);
  if (nv <= k) return;   // the row pass writes this row's output without selection
  const int base = sl * kSlice;
  const int n_s = min(kSlice, nv - base);
  const size_t slot = size_t(b) * G + sl;
  if (n_s <= 0) {
    slice_empty(slot, ws);
    return;
  }
  // A operand: tile rows r < kHI are (query, head r); the other rows are zero
  u32x4 a[kKS];
  int sa[kKS];
  csa_ix::load_a<kHI, kKS>(q_codes, q_e8m0, size_t(b) * kHI + col, col < kHI, g, nblk, row_bytes, a, sa);
  const int rc = 4 * g;            // first C row this lane holds
  const bool mine = rc < kHI;      // C rows of the query (not of the zero rows)
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = mine ? w[size_t(b) * kHI + (rc + i) % kHI] : 0.f;
  const uint8_t* kc_seq = k_codes + size_t(b) * cap * row_bytes;
  const uint8_t* ke_seq = k_e8m0 + size_t(b) * cap * nblk;
  const uint32_t c_bytes = uint32_t(cap) * uint32_t(row_bytes);   // < 2^31 (argument check)
  const uint32_t e_bytes = uint32_t(cap) * uint32_t(nblk);
  const __amdgpu_buffer_rsrc_t rc_k = csa_ix::seq_rsrc(kc_seq, c_bytes);
  const __amdgpu_buffer_rsrc_t re_k = csa_ix::seq_rsrc(ke_seq, e_bytes);
  float* srow = scores + size_t(b) * cap;
  clear_window<kFusedThreads>(sh);   // published by the barrier after the scores

  const int e_wave0 = base + wid * kPerWave;
  u32x4 bk[kNB][kFrag][kKS];
  int sb[kNB][kFrag][kKS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      const int e = e_wave0 + nb * kBatch16 + f * 16 + col;
      csa_ix::load_b<kKS, true>(rc_k, re_k, c_bytes, e_bytes, e, e < nv, g, nblk, row_bytes, bk[nb][f], sb[nb][f]);
    }
  uint32_t kmax = 0u;   // largest key this lane writes
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    v4f acc[kFrag];
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      acc[f] = csa_ix::mfma_fp4(a[0], sa[0], bk[nb][f][0], sb[nb][f][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < kKS; ++ks)
        acc[f] = csa_ix::mfma_fp4(a[ks], sa[ks], bk[nb][f][ks], sb[nb][f][ks], acc[f]);
    }
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      bool writer;
      const float p = csa_ix::head_sum<kHI>(acc[f], wv, g, writer);
      const int e = e_wave0 + nb * kBatch16 + f * 16 + col;
      if (writer && mine) {
        const bool vis = e < nv;
        const uint32_t kk = vis ? ordered_key(p) : 0u;
        skey[e - base] = kk;
        kmax = max(kmax, kk);
        if (vis) srow[e] = p;
      }
    }
  }
  kmax = wave_umax(kmax);
  if (lane == 0) sh.smax[wid] = kmax;
  __syncthreads();
  uint32_t key[kSlice / kFusedThreads];
#pragma unroll
  for (int j = 0; j < kSlice / kFusedThreads; ++j) key[j] = skey[j * kFusedThreads + threadIdx.x];
  slice_finish<kFusedThreads>(key, base, n_s, nv, k, slot, ws, sh);
}

template <int kHI>
hipError_t launch_indexer_slice_h(int ks, int B, hipStream_t st, const uint8_t* qc, const uint8_t* qe, const float* w,
                                  const uint8_t* kc, const uint8_t* ke, const int32_t* pos, int d_I, int cap, int m,
                                  int k, float* scores, const csa_split::SplitWs& sw) {
  const int G = csa_split::n_slices(cap);
  const dim3 grid{unsigned(G), unsigned(B), 1u};
  const dim3 block(kFusedThreads);
  if (ks == 1)
    hipLaunchKernelGGL((indexer_slice_kernel<kHI, 1>), grid, block, 0, st, qc, qe, w, kc, ke, pos, d_I, cap, m, k, G,
                       scores, sw);
  else
    hipLaunchKernelGGL((indexer_slice_kernel<kHI, 2>), grid, block, 0, st, qc, qe, w, kc, ke, pos, d_I, cap, m, k, G,
                       scores, sw);
  return hipGetLastError();
}

// Decoding with few long rows takes the split path (fp32 scores, then the
// slice results, in the workspace); d_I <= 256 keeps a slice's key operands
// in registers.
bool use_fused_split(long rows, int T_q, int d_I, int cap) {
  return T_q == 1 && d_I <= 256 && csa_split::use_split(rows, cap);
}
size_t split_scores_bytes(long rows, int cap) { return (size_t(rows) * size_t(cap) * 4u + 255u) / 256u * 256u; }

template <int kHI, int kKS, int kJ>
hipError_t launch_select_j(long rows, hipStream_t st, const uint16_t* key16, const uint8_t* qc, const uint8_t* qe,
                           const float* w, const uint8_t* kc, const uint8_t* ke, const int32_t* pos, int T_q,
                           int d_I, int cap, int m, int k, int32_t* idx, const int32_t* cu_rows, int n_seq,
                           const uint32_t* gate) {
  if (hipError_t e = csa_lds_opt_in(reinterpret_cast<const void*>(&select_kernel<kHI, kKS, kJ>), sizeof(Shared));
      e != hipSuccess)
    return e;
  hipLaunchKernelGGL((select_kernel<kHI, kKS, kJ>), dim3(unsigned(rows)), dim3(kThreads), sizeof(Shared), st, key16, qc, qe, w, kc, ke, pos, T_q,
                     d_I, cap, m, k, idx, cu_rows, n_seq, gate);
  return hipGetLastError();
}

template <int kHI, int kKS>
hipError_t launch_select_ks(long rows, hipStream_t st, const uint16_t* key16, const uint8_t* qc, const uint8_t* qe,
                            const float* w, const uint8_t* kc, const uint8_t* ke, const int32_t* pos, int T_q,
                            int d_I, int cap, int m, int k, int32_t* idx, const int32_t* cu_rows, int n_seq,
                            const uint32_t* gate) {
  // rows of up to 32768 keys are held whole in 8 rounds of registers; longer
  // rows keep their first 81920 keys in 20 rounds (65536 in 16 when d_I > 128
  // leaves fewer registers free) and read the rest
  if (cap <= 8 * kRound)
    return launch_select_j<kHI, kKS, 8>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
  if constexpr (kKS == 1)
    return launch_select_j<kHI, kKS, 20>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
  return launch_select_j<kHI, kKS, 16>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
}

template <int kHI>
hipError_t launch_select_h(int ks, long rows, hipStream_t st, const uint16_t* key16, const uint8_t* qc,
                           const uint8_t* qe, const float* w, const uint8_t* kc, const uint8_t* ke,
                           const int32_t* pos, int T_q, int d_I, int cap, int m, int k, int32_t* idx,
                           const int32_t* cu_rows, int n_seq, const uint32_t* gate = nullptr) {
  switch (ks) {
    case 1: return launch_select_ks<kHI, 1>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
    case 2: return launch_select_ks<kHI, 2>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
    case 3: return launch_select_ks<kHI, 3>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
    default: return launch_select_ks<kHI, 4>(rows, st, key16, qc, qe, w, kc, ke, pos, T_q, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
  }
}

// ---------------------------------------------------------------------------
// Threshold selection (rows of the row-tile path, k <= kCandMaxK).
//
// A sample pass scores the first 16 entries of every 1024
// (indexer_kernel<kSample>) and cand_threshold_kernel takes, per row, the
// 16-bit key of the r-th largest sampled score, r = k_s + 4 sqrt(k_s) + 16
// with k_s the sample's share of k: more than k entries of the row reach it
// unless the sample is far off.  The threshold pass (indexer_kernel<kCand>)
// keeps the (key, entry) pairs at or above it, and cand_select_kernel finds
// the k-th pair exactly (key descending, entry ascending) and writes the
// first k in entry order.  A row with fewer than k pairs, or more than
// kCandCap, sets the miss flag; the 16-bit-key pass and select_kernel then
// run in full (they are launched behind a gate on that flag and do nothing
// otherwise).  Every score is the indexer's own (same instruction sequence),
// so the result is exactly csa_topk's on csa_indexer_scores, whichever way a
// row goes.

constexpr int kCandMaxK = csa_ix::kCandCap * 2 / 5;   // k beyond this: the 16-bit-key path only
constexpr int kCandMaxCap = 1 << 19;                  // entries the output bitmap covers
constexpr int kCandMinCap = 8 * kRound;               // shorter rows: select_kernel holds them whole
constexpr int kTThreads = 256;                        // threshold and candidate selection kernels

// Row `row` of a call: its sequence and query index (packed rows or B x T_q).
CSA_DEV void row_of(int row, int T_q, const int32_t* __restrict__ cu_rows, int n_seq, int* b, int* i) {
  *b = cu_rows ? csa_packed_seq(cu_rows, n_seq, row) : row / T_q;
  *i = cu_rows ? row - cu_rows[*b] : row - *b * T_q;
}

// Radix selection over the block (kTThreads threads, values in registers):
// the r-th largest (kDesc) or r-th smallest value among the elements for
// which part(x) holds, one byte per pass from the top.  Each wave counts into
// its own histogram (same-bin updates then collide only within a wave), the
// waves' counts are added per bin, and wave 0 finds the byte.  Returns the
// value; *n_at gets how many participating elements equal it and *rank_in
// the rank it has among them (1-based, from the selection's side).
struct RadixLds {
  uint32_t hist[kTThreads / 64][256];
  uint32_t tot[256];
  uint32_t res[4];
};

template <bool kDesc>
CSA_DEV void pick_bin(const uint32_t* tot, uint32_t r, uint32_t* res) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4], sum = 0u;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int bin = kDesc ? 255 - (4 * lane + x) : 4 * lane + x;
    c[x] = tot[bin];
    sum += c[x];
  }
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const uint32_t excl = incl - sum;
  const bool here = excl < r && incl >= r;
  if (here) {
    uint32_t run = excl;
    int x = 0;
    for (; x < 3; ++x) {
      if (run + c[x] >= r) break;
      run += c[x];
    }
    res[0] = uint32_t(kDesc ? 255 - (4 * lane + x) : 4 * lane + x);   // the bin
    res[1] = run;                                                     // before it
    res[2] = c[x];                                                    // in it
  }
}

// One histogram update per element slot of the wave: the lanes whose bin is
// the first active lane's add together through that lane (values of a row
// mostly share their leading byte), the others each add their own.
CSA_DEV void wave_hist_add(uint32_t* hist, bool on, uint32_t bin) {
  const uint64_t act = __ballot(on);
  if (!act) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const uint32_t lb = uint32_t(__shfl(int(bin), leader));
  const uint64_t same = __ballot(on && bin == lb);
  if (lane == leader) atomicAdd(&hist[lb], uint32_t(__popcll(same)));
  else if (on && bin != lb) atomicAdd(&hist[bin], 1u);
}

template <bool kDesc, int kBits, int kPer, typename Part>
CSA_DEV uint32_t radix_select(const uint32_t (&v)[kPer], Part part, uint32_t r, RadixLds& sh, uint32_t* n_at,
                              uint32_t* rank_in) {
  const int wv = threadIdx.x >> 6;
  uint32_t prefix = 0u, mask = 0u;
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    for (int x = threadIdx.x; x < (kTThreads / 64) * 256; x += kTThreads) (&sh.hist[0][0])[x] = 0u;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kPer; ++x)
      wave_hist_add(sh.hist[wv], part(x) && (v[x] & mask) == prefix, (v[x] >> shift) & 255u);
    __syncthreads();
    {
      uint32_t t = 0u;
#pragma unroll
      for (int w = 0; w < kTThreads / 64; ++w) t += sh.hist[w][threadIdx.x];
      sh.tot[threadIdx.x] = t;
    }
    __syncthreads();
    if (threadIdx.x < 64) pick_bin<kDesc>(sh.tot, r, sh.res);
    __syncthreads();
    prefix |= sh.res[0] << shift;
    mask |= 255u << shift;
    r -= sh.res[1];
    *n_at = sh.res[2];
    __syncthreads();
  }
  *rank_in = r;
  return prefix;
}

// The score whose order-preserving key is `key` (keys below -inf's: -inf).
CSA_DEV float key_score(uint32_t key) {
  if (key <= csa_sel::ordered_key(-INFINITY)) return -INFINITY;
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

constexpr int kSampleMax = kCandMaxCap / csa_ix::kSampleGroup * 16 + 16;   // sampled entries per row, at most
constexpr int kSPer = (kSampleMax + kTThreads - 1) / kTThreads;

__global__ __launch_bounds__(kTThreads) void cand_threshold_kernel(const uint16_t* __restrict__ sample, int n_s,
                                                                   const int32_t* __restrict__ q_pos0, int T_q,
                                                                   const int32_t* __restrict__ cu_rows, int n_seq,
                                                                   int cap, int m, int k, uint32_t* __restrict__ thr,
                                                                   uint32_t* __restrict__ cnt,
                                                                   uint32_t* __restrict__ miss) {
  __shared__ RadixLds sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int b, i;
  row_of(row, T_q, cu_rows, n_seq, &b, &i);
  const int t = q_pos0[b] + i;
  const int nv = max(0, min((t + 1) / m, cap));
  if (tid == 0) {
    cnt[row] = 0u;
    if (row == 0) *miss = 0u;
  }
  const int nsv = csa_ix::sampled_count(nv);
  const int k_s = nv > 0 ? int((long(k) * nsv + nv - 1) / nv) : 0;
  const int r = k_s + 4 * int(sqrtf(float(k_s))) + 16;
  if (nv <= k || r > nsv) {   // every entry is a candidate (or the row needs no selection)
    if (tid == 0) thr[row] = __float_as_uint(-INFINITY);
    return;
  }
  const uint16_t* src = sample + size_t(row) * n_s;
  uint32_t v[kSPer];
#pragma unroll
  for (int x = 0; x < kSPer; ++x) {
    const int j = tid + x * kTThreads;
    v[x] = j < nsv ? uint32_t(src[j]) : 0u;
  }
  uint32_t n_at, rank_in;
  const uint32_t key16 = radix_select<true, 16>(v, [&](int x) { return tid + x * kTThreads < nsv; }, uint32_t(r),
                                                sh, &n_at, &rank_in);
  if (tid == 0) thr[row] = __float_as_uint(key_score(key16 << 16));
}

// LDS of cand_select_kernel: the radix histograms, then the bitmap of the
// selected entries (whole groups of 8 words, 16-byte aligned), then per
// group the selected entries before it (both sized for the call's capacity).
struct CandSelLds {
  RadixLds rx;
  uint32_t red[kTThreads / 64];
};
static_assert(sizeof(CandSelLds) % 16 == 0, "the bitmap after it is read as 16-byte words");
size_t cand_select_lds(int cap) {
  const size_t words = (size_t(cap) + 31) / 32, groups = (words + 7) / 8;
  return sizeof(CandSelLds) + groups * 8 * 4 + groups * 4;
}
constexpr int kGroupsPerThread = (kCandMaxCap / 32 / 8 + kTThreads - 1) / kTThreads;   // bitmap groups a thread scans

// Set bits of an 8-word bitmap group.
CSA_DEV uint32_t group_popc(const uint32_t* g8) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(g8);
  const u32x4 b = *reinterpret_cast<const u32x4*>(g8 + 4);
  return __popc(a[0]) + __popc(a[1]) + __popc(a[2]) + __popc(a[3]) + __popc(b[0]) + __popc(b[1]) + __popc(b[2]) +
         __popc(b[3]);
}

__global__ __launch_bounds__(kTThreads) void cand_select_kernel(const uint2* __restrict__ cand,
                                                                const uint32_t* __restrict__ cnt,
                                                                const int32_t* __restrict__ q_pos0, int T_q,
                                                                const int32_t* __restrict__ cu_rows, int n_seq,
                                                                int cap, int m, int k, int32_t* __restrict__ idx,
                                                                uint32_t* __restrict__ miss) {
  constexpr int kPer = csa_ix::kCandCap / kTThreads;
  extern __shared__ __attribute__((aligned(16))) unsigned char cs_smem[];
  CandSelLds& sh = *reinterpret_cast<CandSelLds*>(cs_smem);
  const int cap_groups = ((cap + 31) / 32 + 7) / 8;
  uint32_t* bits = reinterpret_cast<uint32_t*>(cs_smem + sizeof(CandSelLds));
  uint32_t* pre = bits + cap_groups * 8;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  int b, i;
  row_of(row, T_q, cu_rows, n_seq, &b, &i);
  const int t = q_pos0[b] + i;
  const int nv = max(0, min((t + 1) / m, cap));
  int32_t* out = idx + size_t(row) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kTThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const uint32_t n = cnt[row];
  if (n < uint32_t(k) || n > uint32_t(csa_ix::kCandCap)) {
    if (tid == 0) atomicOr(miss, 1u);
    return;
  }
  const uint2* src = cand + size_t(row) * csa_ix::kCandCap;
  uint32_t key[kPer], ent[kPer];
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    const int j = tid + x * kTThreads;
    const uint2 c = j < int(n) ? src[j] : make_uint2(0u, 0xFFFFFFFFu);
    key[x] = j < int(n) ? csa_sel::ordered_key(__uint_as_float(c.x)) : 0u;   // staged as score bits
    ent[x] = c.y;
  }
  auto valid = [&](int x) { return tid + x * kTThreads < int(n); };
  // K: the k-th largest key; need: how many of key K the selection takes
  uint32_t n_eq, need;
  const uint32_t K = radix_select<true, 32>(key, valid, uint32_t(k), sh.rx, &n_eq, &need);
  // among the entries of key K, the need-th lowest index I (all of them: no limit)
  uint32_t I = 0xFFFFFFFFu;
  if (need < n_eq) {
    uint32_t n_i, r_i;
    I = radix_select<false, 32>(ent, [&](int x) { return valid(x) && key[x] == K; }, need, sh.rx, &n_i, &r_i);
  }
  // the selected entries as a bitmap, then each one's rank among them
  auto chosen = [&](int x) { return valid(x) && (key[x] > K || (key[x] == K && ent[x] <= I)); };
  const int n_words = (nv + 31) / 32;
  const int n_groups = (n_words + 7) / 8;
  for (int w = tid; w < n_groups * 8; w += kTThreads) bits[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < kPer; ++x)
    if (chosen(x)) atomicOr(&bits[ent[x] >> 5], 1u << (ent[x] & 31u));
  __syncthreads();
  // groups of 8 words: thread tid counts groups [tid * per, (tid + 1) * per)
  // (per <= kGroupsPerThread), each group read as two 16-byte words
  const int per = (n_groups + kTThreads - 1) / kTThreads;
  uint32_t gc[kGroupsPerThread];
  uint32_t mine = 0u;
#pragma unroll
  for (int q = 0; q < kGroupsPerThread; ++q) {
    const int gi = tid * per + q;
    gc[q] = q < per && gi < n_groups ? group_popc(bits + gi * 8) : 0u;
    mine += gc[q];
  }
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += y;
  }
  if ((tid & 63) == 63) sh.red[tid >> 6] = incl;
  __syncthreads();
  uint32_t run = incl - mine;
  for (int w = 0; w < (tid >> 6); ++w) run += sh.red[w];
#pragma unroll
  for (int q = 0; q < kGroupsPerThread; ++q) {
    const int gi = tid * per + q;
    if (q < per && gi < n_groups) pre[gi] = run;
    run += gc[q];
  }
  __syncthreads();
  // each selected entry's rank: the selected entries of the groups before
  // its group, then of the words before its word, then of the bits below it
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    if (chosen(x)) {
      const uint32_t e = ent[x];
      const int w = int(e >> 5);
      const uint32_t* g8 = bits + (w & ~7);
      const u32x4 a = *reinterpret_cast<const u32x4*>(g8);
      const u32x4 c = *reinterpret_cast<const u32x4*>(g8 + 4);
      const uint32_t word[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
      const int wi = w & 7;
      uint32_t slot = pre[w >> 3];
#pragma unroll
      for (int y = 0; y < 8; ++y) slot += y < wi ? __popc(word[y]) : 0u;
      slot += __popc(bits[w] & ((1u << (e & 31u)) - 1u));
      out[slot] = int32_t(e);
    }
  }
}

// Workspace of the row-tile path: the 16-bit keys (fallback), the sampled
// keys, the candidates, and per row the threshold and count; the miss flag.
struct TileWs {
  uint16_t* key16;
  uint16_t* sample;
  uint2* cand;
  uint32_t* thr;
  uint32_t* cnt;
  uint32_t* miss;
};
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
size_t tile_ws_bytes(long rows, int cap) {
  const size_t n_s = size_t(csa_ix::sampled_count(cap));
  return align256(size_t(rows) * cap * 2) + align256(size_t(rows) * n_s * 2) +
         align256(size_t(rows) * csa_ix::kCandCap * 8) + 2 * align256(size_t(rows) * 4) + 256;
}
TileWs tile_ws(void* ws, long rows, int cap) {
  const size_t n_s = size_t(csa_ix::sampled_count(cap));
  char* p = static_cast<char*>(ws);
  TileWs w;
  w.key16 = reinterpret_cast<uint16_t*>(p);
  p += align256(size_t(rows) * cap * 2);
  w.sample = reinterpret_cast<uint16_t*>(p);
  p += align256(size_t(rows) * n_s * 2);
  w.cand = reinterpret_cast<uint2*>(p);
  p += align256(size_t(rows) * csa_ix::kCandCap * 8);
  w.thr = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(rows) * 4);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(rows) * 4);
  w.miss = reinterpret_cast<uint32_t*>(p);
  return w;
}

// Scoring and selection of `rows` rows (B sequences of T_q rows, or packed
// rows when cu_rows is set) by row tiles: the threshold path when k allows
// it, else (and as its fallback) the 16-bit keys and select_kernel.
hipError_t tile_path(int H_I, long rows, const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                     const uint8_t* k_codes, const uint8_t* k_e8m0, const int32_t* q_pos0, int B, int T_q,
                     const int32_t* cu_rows, int d_I, int cap, int m, int k, int32_t* idx, void* ws, hipStream_t st) {
  const int ks = (d_I + 127) / 128;
  const TileWs tw = tile_ws(ws, rows, cap);
  const int n_rows = cu_rows ? int(rows) : 0;
  const int n_seq = cu_rows ? B : 0;
  const int T_rows = cu_rows ? 1 : T_q;
  const uint32_t* gate = nullptr;
  hipError_t err = hipSuccess;
  if (k <= kCandMaxK && cap > kCandMinCap && cap <= kCandMaxCap) {
    const int n_s = csa_ix::sampled_count(cap);
    err = csa_ix::launch_indexer<csa_ix::kSample>(H_I, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap,
                                                  m, tw.sample, st, cu_rows, n_rows);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(cand_threshold_kernel, dim3(unsigned(rows)), dim3(kTThreads), 0, st, tw.sample, n_s, q_pos0,
                       T_rows, cu_rows, n_seq, cap, m, k, tw.thr, tw.cnt, tw.miss);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    csa_ix::IxExtra x{};
    x.thr = tw.thr;
    x.cnt = tw.cnt;
    x.cand = tw.cand;
    // a wave's walk sized so a (block, row) expects at most about 55 of its
    // row's ~1.75 k candidates (the staging holds kBlockCand = 256; a
    // (block, row) past it sends the row to the fallback).  Measured on the
    // 1M chunk (k = 1024 of 262656): walks of ~1000 entries 715 us, ~1700
    // entries 676 us, ~2700 entries 861 us.
    x.wave_entries = max(256, min(csa_ix::kWaveEntries, int(8L * cap / k) / 64 * 64));
    err = csa_ix::launch_indexer<csa_ix::kCand>(H_I, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap,
                                                m, nullptr, st, cu_rows, n_rows, x);
    if (err != hipSuccess) return err;
    const size_t lds = cand_select_lds(cap);
    if ((err = csa_lds_opt_in(reinterpret_cast<const void*>(&cand_select_kernel), cand_select_lds(kCandMaxCap))) !=
        hipSuccess)
      return err;
    hipLaunchKernelGGL(cand_select_kernel, dim3(unsigned(rows)), dim3(kTThreads), lds, st, tw.cand,
                       tw.cnt, q_pos0, T_rows, cu_rows, n_seq, cap, m, k, idx, tw.miss);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    gate = tw.miss;
  }
  if (cap > 0) {
    csa_ix::IxExtra x{};
    x.gate = gate;
    err = csa_ix::launch_indexer<csa_ix::kKey16>(H_I, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap,
                                                 m, tw.key16, st, cu_rows, n_rows, x);
    if (err != hipSuccess) return err;
  }
  switch (H_I) {
    case 4: return launch_select_h<4>(ks, rows, st, tw.key16, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, T_rows, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
    case 8: return launch_select_h<8>(ks, rows, st, tw.key16, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, T_rows, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
    default: return launch_select_h<16>(ks, rows, st, tw.key16, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, T_rows, d_I, cap, m, k, idx, cu_rows, n_seq, gate);
  }
}

}  // namespace

// Workspace of csa_indexer_topk: on the decode path the fp32 scores and the
// slice lists; otherwise the row-tile path's buffers.
size_t csa_indexer_topk_workspace_size(long rows, int T_q, int d_I, int cap) {
  if (use_fused_split(rows, T_q, d_I, cap)) return split_scores_bytes(rows, cap) + csa_split::split_ws_bytes(rows, cap);
  return tile_ws_bytes(rows, cap);
}
size_t csa_indexer_topk_varlen_workspace_size(long n_rows, int cap) { return n_rows > 0 ? tile_ws_bytes(n_rows, cap) : 0; }

namespace {

// csa_indexer_topk, with an optional short-block compression (arguments
// already checked) that runs before the selection's results are needed: on
// the decode path it rides in the row pass's launch, otherwise it is its own
// launch ahead of the indexer.
csa_status_t indexer_topk_impl(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w, const uint8_t* k_codes,
                               const uint8_t* k_e8m0, const int32_t* q_pos0, int32_t B, int32_t T_q, int32_t H_I,
                               int32_t d_I, int32_t cap, int32_t m, int32_t k, int32_t* idx, void* ws,
                               size_t ws_bytes, hipStream_t st, const csa_cmp::CompressArgs* ride) {
  if (!idx || k < 1) return CSA_EINVAL;
  const csa_status_t s = csa_ix::check_indexer_args(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, H_I, d_I,
                                                    cap, m);
  if (s != CSA_OK) return s;
  if (k > 32767) return CSA_ENOTSUP;
  const long rows = long(B) * T_q;
  if (rows > 0x7FFFFFFFL) return CSA_ENOTSUP;
  const size_t need = rows == 0 ? 0 : csa_indexer_topk_workspace_size(rows, T_q, d_I, cap);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_EWORKSPACE;
  const bool ride_along = ride && rows > 0 && ride->m < 32 && use_fused_split(rows, T_q, d_I, cap);
  if (ride && !ride_along) {
    const csa_status_t c = csa_compress_kv(ride->k, ride->v, ride->in_dtype, ride->logits, ride->B, ride->L,
                                           ride->ld_in, kHeadDim, ride->m, ride->k_out, ride->v_out, ride->k_scale,
                                           ride->v_scale, ride->ld_out, ride->out_dtype, st);
    if (c != CSA_OK) return c;
  }
  if (rows == 0) return CSA_OK;
  const int ks = (d_I + 127) / 128;
  if (use_fused_split(rows, T_q, d_I, cap)) {
    float* scores = static_cast<float*>(ws);
    const csa_split::SplitWs sw =
        csa_split::split_ws(static_cast<char*>(ws) + split_scores_bytes(rows, cap), rows, cap);
    hipError_t e;
    switch (H_I) {
      case 4: e = launch_indexer_slice_h<4>(ks, B, st, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, d_I, cap, m, k, scores, sw); break;
      case 8: e = launch_indexer_slice_h<8>(ks, B, st, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, d_I, cap, m, k, scores, sw); break;
      default: e = launch_indexer_slice_h<16>(ks, B, st, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, d_I, cap, m, k, scores, sw); break;
    }
    if (e != hipSuccess) return CSA_EHIP;
    e = csa_split::launch_topk_split_rows(rows, st, scores, q_pos0, 1, cap, m, k, idx, sw,
                                          ride_along ? ride : nullptr);
    return e == hipSuccess ? CSA_OK : CSA_EHIP;
  }
  const hipError_t err = tile_path(H_I, rows, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, nullptr, d_I, cap,
                                   m, k, idx, ws, st);
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}

}  // namespace

extern "C" csa_status_t csa_indexer_topk(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                                         const uint8_t* k_codes, const uint8_t* k_e8m0, const int32_t* q_pos0,
                                         int32_t B, int32_t T_q, int32_t H_I, int32_t d_I, int32_t cap, int32_t m,
                                         int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return indexer_topk_impl(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, H_I, d_I, cap, m, k, idx, ws,
                           ws_bytes, static_cast<hipStream_t>(stream), nullptr);
}

extern "C" csa_status_t csa_compress_indexer_topk(const void* k, const void* v, int32_t in_dtype, const float* logits,
                                                  int32_t L, int32_t ld_in, int32_t d, void* k_out, void* v_out,
                                                  float* k_scale_out, float* v_scale_out, int32_t ld_out,
                                                  int32_t out_dtype, const uint8_t* q_codes, const uint8_t* q_e8m0,
                                                  const float* w, const uint8_t* k_codes, const uint8_t* k_e8m0,
                                                  const int32_t* q_pos0, int32_t B, int32_t T_q, int32_t H_I,
                                                  int32_t d_I, int32_t cap, int32_t m, int32_t k_sel, int32_t* idx,
                                                  void* ws, size_t ws_bytes, void* stream) {
  const csa_cmp::CompressArgs ca{k, v, logits, in_dtype, B, L, ld_in, m, ld_out, out_dtype,
                                 k_out, v_out, k_scale_out, v_scale_out};
  const csa_status_t c = csa_cmp::check_compress_args(ca, d);
  if (c != CSA_OK) return c;
  return indexer_topk_impl(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, H_I, d_I, cap, m, k_sel, idx, ws,
                           ws_bytes, static_cast<hipStream_t>(stream), &ca);
}

// Packed rows of several sequences (decode rows and prefill chunks together):
// the indexer over row tiles of one sequence each, then the per-row select,
// exactly as csa_indexer_topk does for one sequence's chunk.
extern "C" csa_status_t csa_indexer_topk_varlen(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                                                const uint8_t* k_codes, const uint8_t* k_e8m0, const int32_t* cu_rows,
                                                const int32_t* q_pos0, int32_t B, int32_t n_rows, int32_t H_I,
                                                int32_t d_I, int32_t cap, int32_t m, int32_t k, int32_t* idx,
                                                void* ws, size_t ws_bytes, void* stream) {
  if (!idx || !cu_rows || k < 1 || n_rows < 0) return CSA_EINVAL;
  const csa_status_t s = csa_ix::check_indexer_args(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, 1, H_I, d_I,
                                                    cap, m);
  if (s != CSA_OK) return s;
  if (k > 32767) return CSA_ENOTSUP;
  if (n_rows == 0) return CSA_OK;
  if (B < 1) return CSA_EINVAL;
  const int per_tile = 64 / H_I;   // queries per row tile of the packed indexer launch
  if ((long(n_rows) + per_tile - 1) / per_tile + B > 65535) return CSA_ENOTSUP;
  const size_t need = csa_indexer_topk_varlen_workspace_size(n_rows, cap);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_EWORKSPACE;
  const hipError_t err = tile_path(H_I, n_rows, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, 1, cu_rows, d_I, cap,
                                   m, k, idx, ws, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}
