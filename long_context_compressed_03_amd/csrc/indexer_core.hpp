// Lightning-indexer scoring on the CDNA4 block-scaled MXFP4 matrix cores,
// shared by csa_indexer_scores (fp32 scores out) and csa_indexer_topk (16-bit
// order-preserving keys out, then exact re-scoring of the boundary entries).
//
// The pages say the indexer scores every query token against every compressed
// block in FP4 (sz-guanghua.com.cn ifanr repost, 百萬長上下文) and that the FP4
// form on the indexer's query-key path is MXFP4 ("DeepSeek V4技术揭秘", §一).
// Score (this library's reading):  s(t,e) = sum_h w[t,h] * ReLU(q[t,h] . k[e]).
//
// The contraction [query*head rows] x [d_I] x [entries] runs on
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both operands in E2M1 and one E8M0
// scale per 32 elements, which is exactly the MXFP4 block format: the
// instruction applies the block scales itself, so operands go from HBM to the
// matrix core untouched.  Lane layout (checked on gfx950): lane l supplies row
// (A) / column (B) l%16 and the 32 contraction elements [32*(l/16), +32) of a
// 128-wide step as 16 bytes, with its block's E8M0 in byte 0 of the scale
// operand; C lane l holds column l%16, rows 4*(l/16) .. +3.
//
// Rows of a 16-row tile are (query, head) pairs, head fastest, so one tile
// holds 16/H_I whole queries; query i always sits in slot i % (16/H_I) of its
// tile.  The head sum is 4 rows inside a lane plus, for H_I > 4, a cross-lane
// add (head_sum).  Every score of a (query, entry) pair is produced by the
// same instruction sequence on the same operand values wherever it is
// computed, so a re-scored entry reproduces the first score bit for bit.
#pragma once
#include "select.hpp"

namespace csa_ix {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxKSteps = 4;  // d_I <= 512

enum Out { kScoresF32 = 0, kKey16 = 1, kSample = 2, kCand = 3 };

// Entries of the sample pass: the first 16-entry fragment of every group of
// kSampleGroup entries (entries 0..15, 1024..1039, ...), so its loads stay
// whole fragments.  Sampled entry j is entry (j / 16) * kSampleGroup + j % 16.
constexpr int kSampleGroup = 1024;
CSA_DEV_HOST_INLINE int sampled_count(int n) {   // sampled entries below n
  return (n / kSampleGroup) * 16 + (n % kSampleGroup < 16 ? n % kSampleGroup : 16);
}
// Entries a wave walks in the batched (non-streaming) launches, about.
constexpr int kWaveEntries = 2048;
// Candidate slots per row of the threshold pass, and per (block, row) in LDS.
constexpr int kCandCap = 8192;
constexpr int kBlockCand = 256;

// Extra arguments of the selection passes of csa_indexer_topk.
//   gate   (any mode) null, or a flag: the launch does nothing while it is 0
//   thr    (kCand) per row: the 32-bit order-preserving key a candidate reaches
//   cnt    (kCand) per row: candidates found (atomic; past kCandCap: overflow)
//   cand   (kCand) per row: kCandCap (score bits, entry) pairs, in no particular order
//   wave_entries  (batched launches) about how many entries a wave walks; 0: kWaveEntries
struct IxExtra {
  const uint32_t* gate;
  const uint32_t* thr;
  uint32_t* cnt;
  uint2* cand;
  int wave_entries;
};

// A block's candidates of its rows, staged in LDS before one global
// reservation per (block, row).
struct CandLds {
  uint32_t n[64];               // [0, 16): staged count per row; [32, 48): its reserved base
  uint2 item[16][kBlockCand];   // at most 16 rows per block (4 tiles of 16 / H_I queries)
};

CSA_DEV v4f mfma_fp4(u32x4 a, int sa, u32x4 b, int sb, v4f c) {
  v8i av = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
  v8i bv = {int(b[0]), int(b[1]), int(b[2]), int(b[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// ReLU as one integer max on the bit pattern: every negative float (and -0)
// has a negative int pattern and becomes +0; non-negative floats are kept.
CSA_DEV float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum of p over the lane pairs (l, l ^ 16) (kX == 16) or (l, l ^ 32)
// (kX == 32), taken as (value of the lower lane) + (value of the upper lane)
// on both lanes, through the CDNA4 row-swap permutes (no LDS round trip).
template <int kX>
CSA_DEV float pair_sum(float p) {
  const uint32_t u = __float_as_uint(p);
  if constexpr (kX == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// Weighted ReLU sum over the heads of one query from a 16x16 score tile:
// lane l holds rows 4*(l/16) .. +3 (heads of one query) of column l%16 in
// acc, with their weights in wv.  The result is valid on the writer lanes:
// for H_I = 4 every lane, for 8 the lanes with (l/16) even, for 16 lanes 0..15.
template <int kHI>
CSA_DEV float head_sum(v4f acc, const float (&wv)[4], int g, bool& writer) {
  float p = wv[0] * relu(acc[0]);
  p = fmaf(wv[1], relu(acc[1]), p);
  p = fmaf(wv[2], relu(acc[2]), p);
  p = fmaf(wv[3], relu(acc[3]), p);
  writer = true;
  if constexpr (kHI == 8) {
    p = pair_sum<16>(p);
    writer = (g & 1) == 0;
  } else if constexpr (kHI == 16) {
    p = pair_sum<16>(p);
    p = pair_sum<32>(p);
    writer = g == 0;
  }
  return p;
}

// A operand of one row tile: lane row `col` is (query, head) = (q, h); rows
// of queries outside [0, T_q) or not selected by `use` are zero.
template <int kHI, int kKS>
CSA_DEV void load_a(const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_e8m0, size_t vec, bool use,
                    int g, int nblk, int row_bytes, u32x4 (&a)[kKS], int (&sa)[kKS]) {
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int c = ks * 4 + g;
    if (use && c < nblk) {
      a[ks] = *reinterpret_cast<const u32x4*>(q_codes + vec * row_bytes + c * 16);
      sa[ks] = q_e8m0[vec * nblk + c];
    } else {
      a[ks] = u32x4{0u, 0u, 0u, 0u};
      sa[ks] = 127;
    }
  }
}

// Buffer resource over one sequence's key codes or scales: a load at an
// offset past `bytes` returns zeros without touching memory.
CSA_DEV __amdgpu_buffer_rsrc_t seq_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, bytes, 0x00020000);
}

// B operand of one 16-entry fragment: lane column `col` is entry e (absent if
// !use).  An absent entry or contraction block reads past the resource and
// gets zero codes and a zero scale byte (2^-127): a zero contribution.  Every
// lane issues the same loads, with no branch: loads inside divergent branches
// make the compiler wait for every load in flight at the join (the two sides
// share registers), which would drain the next batch's loads early.
template <int kKS, bool kStream>
CSA_DEV void load_b(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t re, uint32_t c_bytes, uint32_t e_bytes, int e,
                    bool use, int g, int nblk, int row_bytes, u32x4 (&bk)[kKS], int (&sb)[kKS]) {
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int c = ks * 4 + g;
    const bool ok = use && c < nblk;
    const uint32_t oc = ok ? uint32_t(e) * uint32_t(row_bytes) + uint32_t(c) * 16u : c_bytes;
    const uint32_t oe = ok ? uint32_t(e) * uint32_t(nblk) + uint32_t(c) : e_bytes;
    bk[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, kStream ? 2 : 0));
    sb[ks] = __builtin_amdgcn_raw_buffer_load_b8(re, oe, 0, 0);
  }
}

// The kFrag fragments of one batch of a wave's walk over consecutive entries
// e .. e + 16 kFrag - 1 (lane column `col` adds to e; the caller passes
// e = cap when there is no batch to load).  Offsets past the resource read
// zeros, so no per-fragment selects: an entry at or past cap, and a lane
// whose contraction block is absent (its lane offset is the resource size),
// read zeros; entries between the block's visibility and cap are read and
// their scores discarded.  Offsets stay below 2^32: cap * row_bytes < 2^31.
template <int kKS, int kFrag>
CSA_DEV void load_b_run(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t re, uint32_t e, const uint32_t (&oc)[kKS],
                        const uint32_t (&oe)[kKS], int row_bytes, int nblk, u32x4 (&bk)[kFrag][kKS],
                        int (&sb)[kFrag][kKS]) {
  const uint32_t c0 = e * uint32_t(row_bytes), e0 = e * uint32_t(nblk);
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const uint32_t cb = c0 + oc[ks], eb = e0 + oe[ks];
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      // the fragment's distance goes into the range-checked vector offset
      // (a buffer load's scalar offset is not range-checked)
      bk[f][ks] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, cb + uint32_t(f * 16 * row_bytes), 0, 0));
      sb[f][ks] = __builtin_amdgcn_raw_buffer_load_b8(re, eb + uint32_t(f * 16 * nblk), 0, 0);
    }
  }
}

// Row tile `tile` of a packed batch: sequence b's rows are cut into tiles of
// `per` rows each, sequences in order; sets the tile's sequence and its first
// row within it.  False past the last tile (the grid is a bound: at most
// ceil(n_rows / per) + B tiles).
CSA_DEV bool tile_of_packed(const int32_t* __restrict__ cu_rows, int B, int per, int tile, int* b, int* q_first) {
  int t = 0;
  for (int s = 0; s < B; ++s) {
    const int n = cu_rows[s + 1] - cu_rows[s];
    const int tiles = (n + per - 1) / per;
    if (tile < t + tiles) {
      *b = s;
      *q_first = (tile - t) * per;
      return true;
    }
    t += tiles;
  }
  return false;
}

// kHI: indexer heads (4, 8 or 16); kRT: 16-row tiles per block; kKS: 128-wide
// contraction steps; kFrag: 16-entry fragments per wave per batch of loads;
// kStream: keys read once (decode) with non-temporal loads; kOut: fp32
// scores (-inf past nvis), the top 16 bits of the order-preserving key (0
// past nvis), the same 16-bit keys of the sampled entries only (kSample: row
// stride sampled_count(cap)), or the (key, entry) pairs whose score reaches
// the row's threshold (kCand).
//
// Work split: a block of 4 waves owns kRT row tiles of one sequence; each
// wave walks its own run of entries, 16 per MFMA, with the A fragments
// (queries) held in registers for the whole run.
template <int kHI, int kRT, int kKS, int kFrag, bool kStream, int kOut, bool kWalk>
__global__ __launch_bounds__(kBlock) void indexer_kernel(const uint8_t* __restrict__ q_codes,
                                                         const uint8_t* __restrict__ q_e8m0,
                                                         const float* __restrict__ w,
                                                         const uint8_t* __restrict__ k_codes,
                                                         const uint8_t* __restrict__ k_e8m0,
                                                         const int32_t* __restrict__ q_pos0, int T_q_all, int d_I,
                                                         int cap, int m, int entries_per_wave, void* __restrict__ out,
                                                         const int32_t* __restrict__ cu_rows, int n_seq, IxExtra x) {
  constexpr int kQPT = 16 / kHI;  // queries per row tile
  // Head-major tiles (every batched launch): the kHI / 4 tiles of a query
  // group hold heads 0-3, 4-7, ... of the same 4 queries, so each lane ends
  // with whole scores (no cross-lane head sum) and the group's partial sums
  // are added in the order head_sum uses (lower heads + upper heads, pairwise).
  // Streaming (decode) launches have a single tile: 16 / kHI queries per tile,
  // head fastest, summed with head_sum.
  // (16 heads keep the tile-per-query form: built head-major, the second
  // batch of each wave came out wrong on gfx950 -- cause not found, the
  // index mapping checks out on the host -- while 4 and 8 heads are exact.)
  constexpr int kGrp = kHI / 4;
  constexpr bool kHM = !kStream && kRT % kGrp == 0 && kHI <= 8;
  auto q_of = [](int rt, int r) { return kHM ? (rt / kGrp) * 4 + r / 4 : (rt * 16 + r) / kHI; };
  auto h_of = [](int rt, int r) { return kHM ? (rt % kGrp) * 4 + r % 4 : (rt * 16 + r) % kHI; };
  // entry space the waves walk: every entry, or the sampled ones
  auto real_entry = [](int e) { return kOut == kSample ? (e >> 4) * kSampleGroup + (e & 15) : e; };
  auto space = [](int n) { return kOut == kSample ? sampled_count(n) : n; };
  if (x.gate && *x.gate == 0u) return;   // the whole block
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  // this block's sequence b, its queries q_block .. (T_q of them), and the
  // packed row of its query 0 (row_base); packed batches (cu_rows) find the
  // sequence from the tile index
  // row tile blockIdx.y; kWalk (the gated fallback launch, whose few blocks
  // walk them all): blockIdx.y, + gridDim.y, ...
  for (int tile = blockIdx.y;; tile += gridDim.y) {
  int b, q_block, T_q;
  size_t row_base;
  if (cu_rows) {
    if (!tile_of_packed(cu_rows, n_seq, kRT * kQPT, tile, &b, &q_block)) break;
    row_base = size_t(cu_rows[b]);
    T_q = cu_rows[b + 1] - cu_rows[b];
  } else {
    b = blockIdx.z;
    q_block = tile * kRT * kQPT;
    if (q_block >= T_q_all) break;
    T_q = T_q_all;
    row_base = size_t(b) * T_q;
  }
  const int nblk = d_I >> 5;            // 32-element blocks per vector
  const int row_bytes = d_I >> 1;
  const int pos0 = q_pos0[b];

  // ---- A fragments (queries), weights and visibility for this lane's rows
  u32x4 a[kRT][kKS];
  int sa[kRT][kKS];
  float wv[kRT][4];
  int nv_lane[kRT];  // visible entries of the query whose rows this lane holds in C
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int q = q_block + q_of(rt, col);
    const int h = h_of(rt, col);
    load_a<kHI, kKS>(q_codes, q_e8m0, (row_base + q) * kHI + h, q < T_q, g, nblk, row_bytes, a[rt], sa[rt]);
    const int qc = q_block + q_of(rt, 4 * g);   // the query of the C rows this lane holds
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h_of(rt, 4 * g + i);
      wv[rt][i] = qc < T_q ? w[(row_base + qc) * kHI + hh] : 0.f;
    }
    int nv = 0;
    if (qc < T_q) nv = min((pos0 + qc + 1) / m, cap);
    nv_lane[rt] = space(nv);
  }
  // largest visibility among the block's queries (the last valid one)
  const int q_last = min(q_block + kRT * kQPT, T_q) - 1;
  const int nv_max = space(min((pos0 + q_last + 1) / m, cap));
  const int ecap = space(cap);   // entries (sampled ones: row stride)

  const int e_wave0 = (blockIdx.x * kWavesPerBlock + wid) * entries_per_wave;
  const int e_wave1 = min(e_wave0 + entries_per_wave, ecap);

  const uint8_t* kc_seq = k_codes + size_t(b) * cap * row_bytes;
  const uint8_t* ke_seq = k_e8m0 + size_t(b) * cap * nblk;
  const uint32_t c_bytes = uint32_t(cap) * uint32_t(row_bytes);   // < 2^31 (argument check)
  const uint32_t e_bytes = uint32_t(cap) * uint32_t(nblk);
  const __amdgpu_buffer_rsrc_t rc = seq_rsrc(kc_seq, c_bytes);
  const __amdgpu_buffer_rsrc_t re = seq_rsrc(ke_seq, e_bytes);

  // output row of each row tile's query (the query whose rows the lane holds)
  bool q_in[kRT];
  size_t orow[kRT];
  float thr[kRT];   // kCand: the threshold score of the lane's query
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int q = q_block + q_of(rt, 4 * g);
    q_in[rt] = q < T_q;
    orow[rt] = (row_base + (q < T_q ? q : 0)) * size_t(ecap);
    thr[rt] = 0.f;
    if constexpr (kOut == kCand) thr[rt] = __uint_as_float(x.thr[row_base + (q < T_q ? q : 0)]);
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char ix_smem[];
  CandLds& cl = *reinterpret_cast<CandLds*>(ix_smem);
  constexpr int kRowsPerBlock = kRT * kQPT;
  static_assert(kOut != kCand || kRowsPerBlock <= 16, "candidate staging holds 16 rows");
  if constexpr (kOut == kCand) {
    for (int i = threadIdx.x; i < kRowsPerBlock; i += kBlock) cl.n[i] = 0u;
    __syncthreads();
  }
  auto put = [&](int rt, int e, float p) {
    if constexpr (kOut == kCand) {
      // a float compare (the threshold is a score whose key is the row's
      // 32-bit threshold key: same order, -0 == +0 included).  Visibility
      // alone bounds the test: a lane of a query past T_q sees no entry, and
      // a batch (64 entries, walks of whole batches) never crosses into the
      // next wave's walk.  The score's bits are staged; the selection turns
      // them into order-preserving keys.
      if (e < nv_lane[rt] && p >= thr[rt]) {
        const int lr = q_of(rt, 4 * g);   // the query's slot among the block's rows
        const uint32_t slot = atomicAdd(&cl.n[lr], 1u);
        if (slot < uint32_t(kBlockCand)) cl.item[lr][slot] = make_uint2(__float_as_uint(p), uint32_t(e));
      }
    } else if (q_in[rt] && e < e_wave1) {
      const bool vis = e < nv_lane[rt];
      if constexpr (kOut == kScoresF32) {
        static_cast<float*>(out)[orow[rt] + e] = vis ? p : -INFINITY;
      } else {
        static_cast<uint16_t*>(out)[orow[rt] + e] = vis ? uint16_t(csa_sel::ordered_key(p) >> 16) : uint16_t(0);
      }
    }
  };

  // key fragments of the next batch load while the current one computes.
  // Walks over consecutive entries (not the sample pass, not streaming) load
  // a batch with load_b_run: per lane, the offsets of its contraction blocks
  // (the resource size for a block past d_I).
  constexpr bool kRun = !kStream && kOut != kSample;
  uint32_t oc_lane[kKS], oe_lane[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int c = ks * 4 + g;
    oc_lane[ks] = c < nblk ? uint32_t(c) * 16u : c_bytes;
    oe_lane[ks] = c < nblk ? uint32_t(c) : e_bytes;
  }
  auto run_entry = [&](int e0, bool any) {   // the lane's entry of a batch starting at e0, or cap
    return any ? uint32_t(min(e0 + col, cap)) : uint32_t(cap);
  };
  u32x4 bk[kFrag][kKS];
  int sb[kFrag][kKS];
  if constexpr (kRun) {
    load_b_run<kKS, kFrag>(rc, re, run_entry(e_wave0, e_wave0 < nv_max), oc_lane, oe_lane, row_bytes,
                           nblk, bk, sb);
  } else {
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      const int e = e_wave0 + f * 16 + col;
      load_b<kKS, kStream>(rc, re, c_bytes, e_bytes, real_entry(e), e < nv_max, g, nblk, row_bytes, bk[f], sb[f]);
    }
  }
  // One batch: the keys of the batch after it load into (nk, ns) while this
  // one computes from (ck, cs); two buffers swap roles from batch to batch (no
  // register copies).  A streaming wave owns a single batch: nothing to prefetch.
  auto batch = [&](auto& ck, auto& cs, auto& nk, auto& ns, int e_frag0, bool prefetch) {
    if (prefetch) {
      const bool more = e_frag0 + 16 * kFrag < e_wave1;
      if constexpr (kRun) {
        const int en = e_frag0 + 16 * kFrag;
        load_b_run<kKS, kFrag>(rc, re, run_entry(en, more && en < nv_max), oc_lane, oe_lane, row_bytes,
                               nblk, nk, ns);
      } else {
#pragma unroll
        for (int f = 0; f < kFrag; ++f) {
          const int e = e_frag0 + 16 * kFrag + f * 16 + col;
          load_b<kKS, kStream>(rc, re, c_bytes, e_bytes, real_entry(e), more && e < nv_max, g, nblk, row_bytes,
                               nk[f], ns[f]);
        }
      }
    }
    // every MFMA of the batch first, into its own accumulator; entries past
    // every query's visibility carry zero operands and their scores are
    // computed (and discarded) like any other
    v4f acc[kFrag][kRT];
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        acc[f][rt] = mfma_fp4(a[rt][0], sa[rt][0], ck[f][0], cs[f][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ks = 1; ks < kKS; ++ks) acc[f][rt] = mfma_fp4(a[rt][ks], sa[rt][ks], ck[f][ks], cs[f][ks], acc[f][rt]);
      }
    if constexpr (kHM) {
      // each lane: the whole score of query (rt / kGrp) * 4 + g at entry
      // e_frag0 + 16 f + col, one per (fragment, query group)
      constexpr int kQG = kRT / kGrp;
#pragma unroll
      for (int f = 0; f < kFrag; ++f)
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi) {
          float part[kGrp];
#pragma unroll
          for (int hq = 0; hq < kGrp; ++hq) {
            const v4f& c = acc[f][gi * kGrp + hq];
            const float(&wq)[4] = wv[gi * kGrp + hq];
            float p = wq[0] * relu(c[0]);
            p = fmaf(wq[1], relu(c[1]), p);
            p = fmaf(wq[2], relu(c[2]), p);
            p = fmaf(wq[3], relu(c[3]), p);
            part[hq] = p;
          }
          float p;
          if constexpr (kGrp == 1) p = part[0];
          else if constexpr (kGrp == 2) p = part[0] + part[1];
          else p = (part[0] + part[1]) + (part[2 % kGrp] + part[3 % kGrp]);
          const int rt = gi * kGrp;
          const int e = e_frag0 + f * 16 + col;
          if constexpr (kOut == kCand) {
            // the wave takes the append path only when one of its lanes has a
            // candidate here (rare); put re-checks everything.  (One test per
            // batch instead keeps every score of the batch live at once: 156
            // VGPRs, one wave fewer per SIMD, measured slower.)
            if (__ballot(p >= thr[rt])) put(rt, e, p);
          } else {
            put(rt, e, p);
          }
        }
    } else if constexpr (kHI == 8 && kFrag % 2 == 0) {
      // both lane halves of a query hold its sum after head_sum: the even one
      // stores fragment f, the odd one fragment f + 1
      const bool odd = (g & 1) != 0;
#pragma unroll
      for (int f = 0; f < kFrag; f += 2)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          bool writer;
          const float p0 = head_sum<kHI>(acc[f][rt], wv[rt], g, writer);
          const float p1 = head_sum<kHI>(acc[f + 1][rt], wv[rt], g, writer);
          put(rt, e_frag0 + (f + (odd ? 1 : 0)) * 16 + col, odd ? p1 : p0);
        }
    } else {
#pragma unroll
      for (int f = 0; f < kFrag; ++f)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          bool writer;
          const float p = head_sum<kHI>(acc[f][rt], wv[rt], g, writer);
          if (writer) put(rt, e_frag0 + f * 16 + col, p);
        }
    }
  };
  if constexpr (kStream) {
    batch(bk, sb, bk, sb, e_wave0, false);
  } else {
    u32x4 bn[kFrag][kKS];
    int sn[kFrag][kKS];
    for (int e_frag0 = e_wave0; e_frag0 < e_wave1; e_frag0 += 2 * 16 * kFrag) {
      batch(bk, sb, bn, sn, e_frag0, true);
      if (e_frag0 + 16 * kFrag >= e_wave1) break;
      batch(bn, sn, bk, sb, e_frag0 + 16 * kFrag, true);
    }
  }
  if constexpr (kOut == kCand) {
    // one reservation per (block, row), then the staged pairs copied out; a
    // (block, row) whose staging overflowed pushes the row's count past the
    // capacity, so the selection sees the overflow
    __syncthreads();
    if (int(threadIdx.x) < kRowsPerBlock) {
      const int q = q_block + int(threadIdx.x);
      const uint32_t n = cl.n[threadIdx.x];
      uint32_t base = 0u;
      if (q < T_q && n > 0u)
        base = atomicAdd(&x.cnt[row_base + q], n > uint32_t(kBlockCand) ? uint32_t(kCandCap) + 1u : n);
      cl.n[32 + threadIdx.x] = base;
    }
    __syncthreads();
    for (int lr = 0; lr < kRowsPerBlock; ++lr) {
      const int q = q_block + lr;
      const uint32_t n = min(cl.n[lr], uint32_t(kBlockCand));
      const uint32_t base = cl.n[32 + lr];
      if (q >= T_q) break;
      for (uint32_t i = threadIdx.x; i < n; i += kBlock)
        if (base + i < uint32_t(kCandCap)) x.cand[(row_base + q) * size_t(kCandCap) + base + i] = cl.item[lr][i];
    }
    __syncthreads();   // the staging is reused by the next tile
  }
  if constexpr (!kWalk) break;
  }   // tiles
}

template <int kHI, int kRT, int kKS, bool kStream, int kOut>
hipError_t launch_indexer_ks(const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             void* out, hipStream_t st, const int32_t* cu_rows, int n_rows, const IxExtra& x) {
  constexpr int kFrag = 4;
  constexpr int kQPT = 16 / kHI;
  const int ecap = kOut == kSample ? sampled_count(cap) : cap;
  // streaming: one batch per wave.  Otherwise a wave walks about
  // kWaveEntries entries (its block's set-up -- query fragments, weights,
  // thresholds, the candidate reservation -- is paid once per walk), the
  // walk length chosen so the entry blocks come to a whole number of rounds
  // over the 8 XCDs (a function of the shape only)
  int entries_per_wave = 16 * kFrag;
  if constexpr (!kStream) {
    const int target = x.wave_entries > 0 ? x.wave_entries : kWaveEntries;
    const int per_xcd_round = 8 * kWavesPerBlock;   // waves in one entry block per XCD
    const int rounds = max(1, (ecap + per_xcd_round * target - 1) / (per_xcd_round * target));
    const int step = 16 * kFrag;                     // one batch
    entries_per_wave = ((ecap + per_xcd_round * rounds - 1) / (per_xcd_round * rounds) + step - 1) / step * step;
  }
  const int per_block = entries_per_wave * kWavesPerBlock;
  const size_t lds = kOut == kCand ? sizeof(CandLds) : 0;
  if (lds) {
    if (hipError_t e = csa_lds_opt_in(
            reinterpret_cast<const void*>(&indexer_kernel<kHI, kRT, kKS, kFrag, kStream, kOut, false>), lds);
        e != hipSuccess)
      return e;
  }
  // Blocks are dealt to the 8 XCDs round-robin in linear order (x fastest);
  // with the entry dimension padded to a multiple of 8, entry block x always
  // runs on XCD x % 8, so each XCD's L2 holds a fixed eighth of the keys
  // while the query tiles stream past it.  Padding blocks exit at once.
  const int n_eb = ((ecap + per_block - 1) / per_block + 7) / 8 * 8;
  // packed batches (cu_rows): a bound on the tiles, sequences found in the kernel
  // the gated fallback launch: 2 tile blocks per (entry block, sequence),
  // walking the tiles (cheap to dispatch when the gate keeps it idle)
  const int tiles = cu_rows ? (n_rows + kRT * kQPT - 1) / (kRT * kQPT) + B : (T_q + kRT * kQPT - 1) / (kRT * kQPT);
  const int ty = x.gate ? min(tiles, 2) : tiles;
  const dim3 grid = cu_rows ? dim3(n_eb, ty, 1) : dim3(n_eb, ty, B);
  if (x.gate) {
    if constexpr (kOut == kKey16)
      hipLaunchKernelGGL((indexer_kernel<kHI, kRT, kKS, kFrag, kStream, kOut, true>), grid, dim3(kBlock), lds, st, qc,
                         qe, w, kc, ke, pos, T_q, d_I, cap, m, entries_per_wave, out, cu_rows, B, x);
    else
      return hipErrorInvalidValue;   // only the 16-bit-key pass serves as a gated fallback
  } else {
    hipLaunchKernelGGL((indexer_kernel<kHI, kRT, kKS, kFrag, kStream, kOut, false>), grid, dim3(kBlock), lds, st, qc,
                       qe, w, kc, ke, pos, T_q, d_I, cap, m, entries_per_wave, out, cu_rows, B, x);
  }
  return hipGetLastError();
}

template <int kHI, int kRT, bool kStream, int kOut>
hipError_t launch_indexer_rt(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             void* out, hipStream_t st, const int32_t* cu_rows, int n_rows, const IxExtra& x) {
  switch (ks) {
    case 1: return launch_indexer_ks<kHI, kRT, 1, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
    case 2: return launch_indexer_ks<kHI, kRT, 2, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
    case 3: return launch_indexer_ks<kHI, kRT, 3, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
    default: return launch_indexer_ks<kHI, kRT, 4, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
  }
}

template <int kHI, int kOut>
hipError_t launch_indexer_h(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                            const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                            void* out, hipStream_t st, const int32_t* cu_rows, int n_rows, const IxExtra& x) {
  // one row tile when the whole call has at most one tile of queries (decode);
  // several otherwise so every key fragment feeds several MFMAs (packed batches
  // always take the several-tile form)
  if (!cu_rows && T_q * kHI <= 16)
    return launch_indexer_rt<kHI, 1, true, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
  return launch_indexer_rt<kHI, 4, false, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
}

// Shared argument checks of the two indexer entry points.
inline csa_status_t check_indexer_args(const void* q_codes, const void* q_e8m0, const void* w, const void* k_codes,
                                       const void* k_e8m0, const void* q_pos0, int32_t B, int32_t T_q, int32_t H_I,
                                       int32_t d_I, int32_t cap, int32_t m) {
  if (!q_codes || !q_e8m0 || !w || !k_codes || !k_e8m0 || !q_pos0) return CSA_EINVAL;
  if (d_I < 32 || d_I > 128 * kMaxKSteps || d_I % 32 != 0) return CSA_EINVAL;
  if (B < 0 || T_q < 0 || cap < 0 || m < 1) return CSA_EINVAL;
  if (H_I != 4 && H_I != 8 && H_I != 16) return CSA_ENOTSUP;
  if (B > 65535 || T_q > (1 << 24)) return CSA_ENOTSUP;
  if (long(cap) * (d_I / 2) >= (1L << 31)) return CSA_ENOTSUP;   // one sequence's key codes under 2 GiB
  return CSA_OK;
}

// cu_rows (device, or null): packed rows of B sequences, n_rows in all (T_q
// unused); otherwise B sequences of T_q rows each.
template <int kOut>
hipError_t launch_indexer(int H_I, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                          const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m, void* out,
                          hipStream_t st, const int32_t* cu_rows = nullptr, int n_rows = 0,
                          const IxExtra& x = IxExtra{}) {
  const int ks = (d_I + 127) / 128;
  switch (H_I) {
    case 4: return launch_indexer_h<4, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
    case 8: return launch_indexer_h<8, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
    default: return launch_indexer_h<16, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows, x);
  }
}

}  // namespace csa_ix
