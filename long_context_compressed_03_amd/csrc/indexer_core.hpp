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

enum Out { kScoresF32 = 0, kKey16 = 1 };

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
// scores (-inf past nvis) or the top 16 bits of the order-preserving key
// (0 past nvis).
//
// Work split: a block of 4 waves owns kRT row tiles of one sequence; each
// wave walks its own run of entries, 16 per MFMA, with the A fragments
// (queries) held in registers for the whole run.
template <int kHI, int kRT, int kKS, int kFrag, bool kStream, int kOut>
__global__ __launch_bounds__(kBlock) void indexer_kernel(const uint8_t* __restrict__ q_codes,
                                                         const uint8_t* __restrict__ q_e8m0,
                                                         const float* __restrict__ w,
                                                         const uint8_t* __restrict__ k_codes,
                                                         const uint8_t* __restrict__ k_e8m0,
                                                         const int32_t* __restrict__ q_pos0, int T_q, int d_I,
                                                         int cap, int m, int entries_per_wave, void* __restrict__ out,
                                                         const int32_t* __restrict__ cu_rows, int n_seq) {
  constexpr int kQPT = 16 / kHI;  // queries per row tile
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  // this block's sequence b, its queries q_block .. (T_q of them), and the
  // packed row of its query 0 (row_base); packed batches (cu_rows) find the
  // sequence from the tile index
  int b, q_block;
  size_t row_base;
  if (cu_rows) {
    if (!tile_of_packed(cu_rows, n_seq, kRT * kQPT, blockIdx.y, &b, &q_block)) return;
    row_base = size_t(cu_rows[b]);
    T_q = cu_rows[b + 1] - cu_rows[b];
  } else {
    b = blockIdx.z;
    q_block = blockIdx.y * kRT * kQPT;
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
    const int r = rt * 16 + col;
    const int q = q_block + r / kHI;
    const int h = r % kHI;
    load_a<kHI, kKS>(q_codes, q_e8m0, (row_base + q) * kHI + h, q < T_q, g, nblk, row_bytes, a[rt], sa[rt]);
    const int rc = rt * 16 + 4 * g;  // first C row this lane holds
    const int qc = q_block + rc / kHI;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = (rc + i) % kHI;
      wv[rt][i] = qc < T_q ? w[(row_base + qc) * kHI + hh] : 0.f;
    }
    int nv = 0;
    if (qc < T_q) nv = min((pos0 + qc + 1) / m, cap);
    nv_lane[rt] = nv;
  }
  // largest visibility among the block's queries (the last valid one)
  const int q_last = min(q_block + kRT * kQPT, T_q) - 1;
  const int nv_max = min((pos0 + q_last + 1) / m, cap);

  const int e_wave0 = (blockIdx.x * kWavesPerBlock + wid) * entries_per_wave;
  const int e_wave1 = min(e_wave0 + entries_per_wave, cap);

  const uint8_t* kc_seq = k_codes + size_t(b) * cap * row_bytes;
  const uint8_t* ke_seq = k_e8m0 + size_t(b) * cap * nblk;
  const uint32_t c_bytes = uint32_t(cap) * uint32_t(row_bytes);   // < 2^31 (argument check)
  const uint32_t e_bytes = uint32_t(cap) * uint32_t(nblk);
  const __amdgpu_buffer_rsrc_t rc = seq_rsrc(kc_seq, c_bytes);
  const __amdgpu_buffer_rsrc_t re = seq_rsrc(ke_seq, e_bytes);

  // output row of each row tile's query (the query whose rows the lane holds)
  bool q_in[kRT];
  size_t orow[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int q = q_block + (rt * 16 + 4 * g) / kHI;
    q_in[rt] = q < T_q;
    orow[rt] = (row_base + (q < T_q ? q : 0)) * cap;
  }
  auto put = [&](int rt, int e, float p) {
    if (q_in[rt] && e < e_wave1) {
      const bool vis = e < nv_lane[rt];
      if constexpr (kOut == kScoresF32) {
        static_cast<float*>(out)[orow[rt] + e] = vis ? p : -INFINITY;
      } else {
        static_cast<uint16_t*>(out)[orow[rt] + e] = vis ? uint16_t(csa_sel::ordered_key(p) >> 16) : uint16_t(0);
      }
    }
  };

  // key fragments of the next batch load while the current one computes
  u32x4 bk[kFrag][kKS];
  int sb[kFrag][kKS];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) {
    const int e = e_wave0 + f * 16 + col;
    load_b<kKS, kStream>(rc, re, c_bytes, e_bytes, e, e < nv_max, g, nblk, row_bytes, bk[f], sb[f]);
  }
  // One batch: the keys of the batch after it load into (nk, ns) while this
  // one computes from (ck, cs); two buffers swap roles from batch to batch (no
  // register copies).  A streaming wave owns a single batch: nothing to prefetch.
  auto batch = [&](auto& ck, auto& cs, auto& nk, auto& ns, int e_frag0, bool prefetch) {
    if (prefetch) {
      const bool more = e_frag0 + 16 * kFrag < e_wave1;
#pragma unroll
      for (int f = 0; f < kFrag; ++f) {
        const int e = e_frag0 + 16 * kFrag + f * 16 + col;
        load_b<kKS, kStream>(rc, re, c_bytes, e_bytes, e, more && e < nv_max, g, nblk, row_bytes, nk[f], ns[f]);
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
    if constexpr (kHI == 8 && kFrag % 2 == 0) {
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
}

template <int kHI, int kRT, int kKS, bool kStream, int kOut>
hipError_t launch_indexer_ks(const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             void* out, hipStream_t st, const int32_t* cu_rows, int n_rows) {
  constexpr int kFrag = 4;
  constexpr int kQPT = 16 / kHI;
  const int entries_per_wave = kStream ? 16 * kFrag : 256;   // streaming: one batch per wave
  const int per_block = entries_per_wave * kWavesPerBlock;
  // Blocks are dealt to the 8 XCDs round-robin in linear order (x fastest);
  // with the entry dimension padded to a multiple of 8, entry block x always
  // runs on XCD x % 8, so each XCD's L2 holds a fixed eighth of the keys
  // while the query tiles stream past it.  Padding blocks exit at once.
  const int n_eb = ((cap + per_block - 1) / per_block + 7) / 8 * 8;
  // packed batches (cu_rows): a bound on the tiles, sequences found in the kernel
  const dim3 grid = cu_rows ? dim3(n_eb, (n_rows + kRT * kQPT - 1) / (kRT * kQPT) + B, 1)
                            : dim3(n_eb, (T_q + kRT * kQPT - 1) / (kRT * kQPT), B);
  hipLaunchKernelGGL((indexer_kernel<kHI, kRT, kKS, kFrag, kStream, kOut>), grid, dim3(kBlock), 0, st, qc, qe, w,
                     kc, ke, pos, T_q, d_I, cap, m, entries_per_wave, out, cu_rows, B);
  return hipGetLastError();
}

template <int kHI, int kRT, bool kStream, int kOut>
hipError_t launch_indexer_rt(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             void* out, hipStream_t st, const int32_t* cu_rows, int n_rows) {
  switch (ks) {
    case 1: return launch_indexer_ks<kHI, kRT, 1, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
    case 2: return launch_indexer_ks<kHI, kRT, 2, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
    case 3: return launch_indexer_ks<kHI, kRT, 3, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
    default: return launch_indexer_ks<kHI, kRT, 4, kStream, kOut>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
  }
}

template <int kHI, int kOut>
hipError_t launch_indexer_h(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                            const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                            void* out, hipStream_t st, const int32_t* cu_rows, int n_rows) {
  // one row tile when the whole call has at most one tile of queries (decode);
  // several otherwise so every key fragment feeds several MFMAs (packed batches
  // always take the several-tile form)
  if (!cu_rows && T_q * kHI <= 16)
    return launch_indexer_rt<kHI, 1, true, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
  return launch_indexer_rt<kHI, 4, false, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
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
                          hipStream_t st, const int32_t* cu_rows = nullptr, int n_rows = 0) {
  const int ks = (d_I + 127) / 128;
  switch (H_I) {
    case 4: return launch_indexer_h<4, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
    case 8: return launch_indexer_h<8, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
    default: return launch_indexer_h<16, kOut>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, out, st, cu_rows, n_rows);
  }
}

}  // namespace csa_ix
