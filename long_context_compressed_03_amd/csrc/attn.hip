// CSA sparse attention and HCA dense attention, each with the sliding window.
//
// Pages: CSA attends only over the k selected compressed entries and also
// keeps a few uncompressed window entries (blog.nickys.cn DeepSeek-V4 post,
// 三大架构改动 §1 CSA); HCA attends densely over all compressed entries
// (§2 HCA); both add the window branch so each token sees its nearest
// neighbours in full (sz-guanghua.com.cn ifanr repost, 百萬長上下文).  The
// selected/visible entries and the window keys form one key list under one
// softmax (this library's reading of "additionally keep").
//
// All query heads share the single KV head, so heads are the M dimension of
// the matrix-core tiles and a gathered key row serves every head.  Keys are
// gathered in chunks of 64 into LDS (K row-major; V transposed so a P*V
// operand reads 4 or 8 keys of one head dimension as 8-byte words); the next
// chunk's rows are already in flight in registers while the current one is
// computed.  Thread t gathers key pair t/16 and 16-byte segment t%16, so a
// wave's load covers whole rows and each row's cache lines are requested by
// one wave.  Per 16-head tile:
//   S^T[keys x 16 heads] = K * Q^T    (bf16 MFMA 16x16x32, Q held in VGPRs)
//   online softmax per head in fp32, exp2 domain
//   O^T[128 x 16 heads] += V^T * P^T  (P^T taken straight from S^T's C layout)
// fp8 (E4M3FN) entries are widened to bf16 exactly by the hardware
// conversion (fp32 variant: in software); the per-entry K scale
// multiplies the logits and the V scale is folded into P, which enters the
// P*V product as two bf16 operands, hi + lo (16 significant bits: one bf16
// rounding of P would cost 2^-9 of |V| per output).  The fp32 variant
// runs the same data flow on the fp32 MFMA 16x16x4 (V row-major there).
//
// A block owns one query and one split of its key list; its 8 waves take the
// head tiles (w % 4, and w % 4 + 4 when H > 64) over one key half each of
// every chunk, so each gathered row serves all heads from LDS, every SIMD has
// two waves to interleave, and each wave's dependent chain per chunk is half
// a chunk long; the two key halves merge through LDS at the end.  With few query rows (decoding) the key list
// is cut into short splits so that every CU gets work and each block's chain
// of dependent loads stays short; each split writes its unnormalised O,
// running max and sum, and a second small kernel merges the splits in split
// order (a kernel boundary instead of device-scope fences, which on this chip
// write back and invalidate the XCD's whole L2).  The split depends only on
// the shape and every reduction has a fixed order: results are bitwise
// reproducible run to run.
#pragma clang fp contract(off)
#include "common.hpp"

namespace {

constexpr int kNK = 64;                       // keys per chunk
constexpr int kThreads = 512;                 // 8 waves
constexpr int kKRow = kHeadDim + 16;          // bf16 per K row in LDS (288-byte rows: the
                                              // K fragment reads are free of bank conflicts,
                                              // measured; 272-byte rows cost 4 cycles a read)
constexpr int kVRow = kNK + 16;               // bf16 per V^T row in LDS
constexpr int kVGroup = 8 * kVRow + 8;         // bf16 per group of 8 V^T rows (rows, then a pad)
constexpr int kFRow = kHeadDim + 4;           // fp32 per K/V row in LDS (fp32 path)
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4s __attribute__((ext_vector_type(4)));

CSA_DEV v4f mfma_k32(const u32x4& a, const u32x4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}
CSA_DEV v4f mfma_k16(const u32x2& a, const u32x2& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), c, 0, 0,
                                                   0);
}
CSA_DEV v4f mfma_f32(float a, float b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
CSA_DEV v4f mfma_h32(const u32x4& a, const u32x4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}
// Two fp32 values rounded to the nearest fp16 (ties to even), packed low/high.
CSA_DEV uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{lo, hi}, v2h));
}

struct AttnArgs {
  const void* q;
  const void* ck;
  const void* cv;
  const float* ck_scale;
  const float* cv_scale;
  const int32_t* idx;      // sparse only
  const void* k_win;
  const void* v_win;
  const int32_t* raw_pos0;
  const int32_t* q_pos0;
  const int32_t* cu_rows;  // varlen: sequence b owns packed rows cu_rows[b] .. cu_rows[b+1]-1
                           // at q_pos0[b], q_pos0[b]+1, ... (else null: row / T_q)
  void* out;
  float* lse;
  float* part_ml;          // [rows, n_splits, H, 2]: running max (log2 domain), sum
  float* part_o;           // [rows, n_splits, H, 128]: unnormalised output
  int cap;
  int k;                   // sparse: list length; dense: m_prime
  int L_raw;
  int W;
  int T_q;
  int H;
  int n_list;              // key-list length (k + W or cap + W)
  int split_len;           // keys per split (multiple of kNK)
  int n_splits;
  int n_seq;               // varlen: sequences
  int piece_len;           // varlen many-query: keys per piece of a one-tile sequence
  int n_pieces;            // ... and pieces per such sequence
  float sm_log2;           // sm_scale * log2(e)
};

// Packed row r of a varlen call: its sequence and position.
CSA_DEV void packed_row(const AttnArgs& a, long r, int* b, int* t) {
  *b = csa_packed_seq(a.cu_rows, a.n_seq, int(r));
  *t = a.q_pos0[*b] + int(r - a.cu_rows[*b]);
}

// Source of key-list slot j for query (b, i) at position t.
// 0 = empty / invisible, 1 = compressed entry `row`, 2 = raw window `row`.
// `e` is idx[b, i, j] for sparse slots j < k (loaded by the caller so that
// the index loads of several slots are in flight together); `raw0` is
// raw_pos0[b].
template <bool kDense>
CSA_DEV int key_source(const AttnArgs& a, int b, int t, int raw0, int j, int e, long* row) {
  int head_len;
  if constexpr (kDense) {
    head_len = a.cap;
    if (j < a.cap) {
      const int nv = min((t + 1) / a.k, a.cap);
      *row = long(b) * a.cap + j;
      return j < nv ? 1 : 0;
    }
  } else {
    head_len = a.k;
    if (j < a.k) {
      *row = long(b) * a.cap + e;
      return (e >= 0 && e < a.cap) ? 1 : 0;
    }
  }
  const int w = j - head_len;
  if (w >= a.W) return 0;
  const int p = t - a.W + 1 + w;
  const int r = p - raw0;
  *row = long(b) * a.L_raw + r;
  return (p >= 0 && r >= 0 && r < a.L_raw) ? 2 : 0;
}

// Registers holding one gather item: two keys x 8 head dims of K and V.
template <int kIO>
struct Pre {
  static constexpr int R = kIO == CSA_F32 ? 2 : 1;  // 16-byte words per 8 dims of the widest source
  u32x4 k[2][R], v[2][R];
  float sk[2], sv[2];
  int src[2];
};

// Loads of one gather slot x: the K and V parts (8 head dims [8 dg, 8 dg + 8))
// of `row` in the compressed cache (src 1) or the raw window (src 2); an
// empty slot (src 0) reads the start of the query buffer instead (always
// valid; the value is never used).  Every lane issues the same loads with its
// own address, with no branch: loads issued inside divergent branches make
// the compiler wait for every load in flight (the two sides of the branch
// share registers), which would end each prefetch before the compute it is
// meant to overlap.  An fp8 part (8 bytes) is fetched as the aligned 16 bytes
// that hold it (inside its 128-byte row); part_bf16 / part_f32 pick the half.
// The fp8 scales are loaded raw and applied by store_chunk for src 1 only.
template <int kIO, int kCKV>
CSA_DEV void gather_slot(const AttnArgs& a, Pre<kIO>& pr, int x, int src, long row, int dg) {
  constexpr long kCB = kCKV == CSA_F32 ? 4 : kCKV == CSA_BF16 ? 2 : 1;   // bytes per compressed value
  constexpr long kWB = kIO == CSA_F32 ? 4 : 2;                           // bytes per window value
  const char* safe = static_cast<const char*>(a.q);
  const long coff = row * (kHeadDim * kCB) + (kCKV == CSA_FP8_E4M3 ? long(dg & ~1) * 8 : long(dg) * 8 * kCB);
  const long woff = row * (kHeadDim * kWB) + long(dg) * 8 * kWB;
  const char* pk = src == 1 ? static_cast<const char*>(a.ck) + coff
                 : src == 2 ? static_cast<const char*>(a.k_win) + woff : safe;
  const char* pv = src == 1 ? static_cast<const char*>(a.cv) + coff
                 : src == 2 ? static_cast<const char*>(a.v_win) + woff : safe;
  pr.k[x][0] = *reinterpret_cast<const u32x4*>(pk);
  pr.v[x][0] = *reinterpret_cast<const u32x4*>(pv);
  if constexpr (Pre<kIO>::R == 2) {
    // second 16 bytes of a 32-byte part (fp32); a 16-byte compressed part reads the safe address
    const bool wide = src == 2 || (src == 1 && kCKV == CSA_F32);
    pr.k[x][1] = *reinterpret_cast<const u32x4*>(wide ? pk + 16 : safe);
    pr.v[x][1] = *reinterpret_cast<const u32x4*>(wide ? pv + 16 : safe);
  }
  if constexpr (kCKV == CSA_FP8_E4M3) {
    pr.sk[x] = *(src == 1 ? a.ck_scale + row : reinterpret_cast<const float*>(safe));
    pr.sv[x] = *(src == 1 ? a.cv_scale + row : reinterpret_cast<const float*>(safe));
  } else {
    pr.sk[x] = 1.f;
    pr.sv[x] = 1.f;
  }
  pr.src[x] = src;
}

// Gather item of thread t: key pair kp = t / 16 (keys 2kp, 2kp+1 of the
// chunk), head dims [8*dg, 8*dg+8) with dg = t % 16.  A wave's load for one
// slot covers 4 whole rows, so each row's cache lines are requested by one
// wave (not by all eight).
CSA_DEV int item_kp() { return int(threadIdx.x) >> 4; }
CSA_DEV int item_dg() { return int(threadIdx.x) & 15; }
//
// Selected-entry indices of the item's two slots in chunk jc (sparse lists);
// they are loaded one chunk ahead of the rows they name, so a row load never
// waits on an index load issued in the same step.
// The load is unconditional (position clamped into the list; slots past the
// list or the split are never used), for the same reason as gather_slot.
template <bool kDense>
CSA_DEV void load_idx(const AttnArgs& a, int (&e)[2], long qrow, int jc, int j_end) {
  e[0] = e[1] = -1;
  if constexpr (!kDense) {
    const int kp = item_kp();
    const int32_t* ip = a.idx + qrow * a.k;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = jc + 2 * kp + x;
      e[x] = ip[min(j, a.k - 1)];
    }
  }
  (void)j_end;
}

// Rows of the item's two slots of chunk jc (e: their indices from load_idx).
template <int kIO, int kCKV, bool kDense>
CSA_DEV void prefetch(const AttnArgs& a, Pre<kIO>& pr, const int (&e)[2], int b, int t, int raw0, int jc, int j_end) {
  const int kp = item_kp();
  const int dg = item_dg();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int j = jc + 2 * kp + x;
    long row = 0;
    const int src = j < j_end ? key_source<kDense>(a, b, t, raw0, j, e[x], &row) : 0;
    gather_slot<kIO, kCKV>(a, pr, x, src, row, dg);
  }
}

// Rows of the item's two slots of a chunk made of selected-entry slots only
// (sparse lists, slots below k): the rows come straight from the indices,
// with no source selects; an empty slot (-1, or an index past cap) reads
// entry 0 of its sequence and is masked by its bias (src 0), so its finite
// values contribute exactly nothing.  Requires cap > 0.
template <int kCKV>
CSA_DEV void prefetch_sel(const AttnArgs& a, Pre<CSA_BF16>& pr, const int (&e)[2], int b) {
  constexpr long kCB = kCKV == CSA_BF16 ? 2 : 1;   // bytes per compressed value (bf16 or fp8)
  const int dg = item_dg();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const bool ok = unsigned(e[x]) < unsigned(a.cap);
    const long row = long(b) * a.cap + (ok ? e[x] : 0);
    const long off = row * (kHeadDim * kCB) + (kCKV == CSA_FP8_E4M3 ? long(dg & ~1) * 8 : long(dg) * 8 * kCB);
    pr.k[x][0] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.ck) + off);
    pr.v[x][0] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.cv) + off);
    if constexpr (kCKV == CSA_FP8_E4M3) {
      pr.sk[x] = a.ck_scale[row];
      pr.sv[x] = a.cv_scale[row];
    } else {
      pr.sk[x] = 1.f;
      pr.sv[x] = 1.f;
    }
    pr.src[x] = ok ? 1 : 0;
  }
}

// 8 values of a gathered part as fp32 (src 0 -> zeros)
template <int kIO, int kCKV>
CSA_DEV void part_f32(const u32x4* w, int src, int h, float* x) {
  if (src == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  } else if (kCKV == CSA_FP8_E4M3 && src == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = e4m3_to_f32((w[0][2 * h + (e >> 2)] >> (8 * (e & 3))) & 0xFFu);
  } else if constexpr (kIO == CSA_BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = w[0][e];
      x[2 * e] = __uint_as_float(u << 16);
      x[2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e >> 2][e & 3]);
  }
}

// Position of key `kk` of a chunk in a V^T row.  A P*V operand lane (column
// group g of 32-key step st) takes keys 32 st + 4 g .. +3 and 32 st + 16 + 4 g
// .. +3 (the key order of S^T's C layout); they are stored side by side at
// 32 st + 8 g .. +7, so the lane reads them as one 16-byte word.  Key pairs
// (2i, 2i + 1) stay adjacent.
CSA_DEV int vt_key_pos(int kk) {
  return (kk & ~31) + 8 * ((kk & 15) >> 2) + 4 * ((kk >> 4) & 1) + (kk & 3);
}

// LDS layout of one chunk
struct LdsBf16 {
  uint16_t K[kNK][kKRow];
  // V^T, head dim x key (keys at vt_key_pos): rows of 40 words, 4 words of
  // pad after every 8 rows.  Measured bank conflicts per wave instruction:
  // 2 cycles for the transposed key-pair writes, 4 for the 16-byte operand
  // reads (8 with the keys in order, read as two 8-byte halves).
  uint16_t Vt[kHeadDim / 8][kVGroup];
  // per key: K scale x logit scale, V scale, and 0 (present) or -inf (absent:
  // its K row is zeros, so logit = product * sk + bias needs no branch)
  float sk[kNK];
  float sv[kNK];
  float bias[kNK];
};
struct LdsF32 {
  float K[kNK][kFRow];
  float V[kNK][kFRow];
  float sk[kNK];
  float sv[kNK];
  float bias[kNK];
};
template <int kIO>
using LdsChunk = typename std::conditional<kIO == CSA_BF16, LdsBf16, LdsF32>::type;

// Hand-over of one key half's state to the other at the end of a block.
template <int kHTW>
struct LdsHalf {
  float o[4 * kHTW][16][kHeadDim + 4];
  float m[4 * kHTW][16];
  float l[4 * kHTW][16];
};

// Running state of the batch-invariant fold (kFold), per head tile.
template <int kHTW>
struct LdsFold {
  float o[4 * kHTW][16][kHeadDim + 4];
  float m[4 * kHTW][16];
  float l[4 * kHTW][16];
};

template <int kIO, int kHTW>
constexpr size_t lds_bytes() {
  return sizeof(LdsChunk<kIO>) > sizeof(LdsHalf<kHTW>) ? sizeof(LdsChunk<kIO>) : sizeof(LdsHalf<kHTW>);
}

// 8 head dims of a gathered part as four bf16 pairs (src 0 -> zeros).  E4M3
// codes go through the CDNA4 fp8 -> bf16 conversion, which is exact (every
// E4M3 value is a bf16 value); the per-entry scale is applied elsewhere.
// kAll: every slot holds a compressed entry (src 1), so no selects.
template <int kCKV, bool kAll = false>
CSA_DEV u32x4 part_bf16(const u32x4* w, int src, int h) {
  // selects, not branches (see gather_slot): the result depends on src only
  u32x4 r = w[0];
  if constexpr (kCKV == CSA_FP8_E4M3) {
    const uint32_t c0 = h ? w[0][2] : w[0][0], c1 = h ? w[0][3] : w[0][1];
    const u32x4 cv = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, 1.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, 1.0f, true))};
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = kAll || src == 1 ? cv[q] : r[q];
  }
  if constexpr (!kAll) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = src == 0 ? 0u : r[q];
  }
  return r;
}

// 8 head dims of a gathered fp8 entry part as four fp16 pairs: every E4M3
// value is an fp16 value (exponents -9 .. 8), so the conversion is exact.
CSA_DEV u32x4 part_f16_fp8(const u32x4* w, int h) {
  const uint32_t c0 = h ? w[0][2] : w[0][0], c1 = h ? w[0][3] : w[0][1];
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true))};
}

// sk_mul: factor folded into the stored K scale (the logit scale in the log2 domain).
// kAll (bf16 path): the item's slots are compressed entries (prefetch_entries);
// with fp8 entries V^T is then stored as fp16 (exact) for the one-product
// P*V of the many-query kernel.
// kVF16 (all-entries chunks of fp8 entries in the many-query kernel): V^T as
// fp16 instead of bf16.  kSrcBias: an empty slot (src 0) gets the -inf bias
// (an all-entries chunk of the many-query kernel has none).
template <int kIO, int kCKV, bool kAll = false, bool kVF16 = kAll && kCKV == CSA_FP8_E4M3, bool kSrcBias = !kAll>
CSA_DEV void store_chunk(LdsChunk<kIO>& s, const Pre<kIO>& pr, float sk_mul) {
  static_assert(!kVF16 || (kAll && kCKV == CSA_FP8_E4M3), "fp16 V^T holds fp8 entries only");
  const int kp = item_kp();
  const int dg = item_dg();
  if constexpr (kIO == CSA_BF16) {
    // values are exact in bf16 (bf16 inputs or E4M3 codes)
    u32x4 kw[2], vw[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kw[e] = part_bf16<kCKV, kAll>(pr.k[e], pr.src[e], dg & 1);
      if constexpr (kVF16)
        vw[e] = part_f16_fp8(pr.v[e], dg & 1);
      else
        vw[e] = part_bf16<kCKV, kAll>(pr.v[e], pr.src[e], dg & 1);
      *reinterpret_cast<u32x4*>(&s.K[2 * kp + e][dg * 8]) = kw[e];
    }
    // V^T: head dim x of keys 2kp and 2kp+1 as one bf16 pair
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      uint16_t* vt = &s.Vt[dg][2 * x * kVRow + vt_key_pos(2 * kp)];   // rows 8 dg + 2x and 8 dg + 2x + 1
      *reinterpret_cast<uint32_t*>(vt) = (vw[0][x] & 0xFFFFu) | (vw[1][x] << 16);
      *reinterpret_cast<uint32_t*>(vt + kVRow) = (vw[0][x] >> 16) | (vw[1][x] & 0xFFFF0000u);
    }
  } else {
    float xk[2][8], xv[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      part_f32<kIO, kCKV>(pr.k[e], pr.src[e], dg & 1, xk[e]);
      part_f32<kIO, kCKV>(pr.v[e], pr.src[e], dg & 1, xv[e]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int x = 0; x < 8; x += 4) {
        *reinterpret_cast<v4f*>(&s.K[2 * kp + e][dg * 8 + x]) = v4f{xk[e][x], xk[e][x + 1], xk[e][x + 2], xk[e][x + 3]};
        *reinterpret_cast<v4f*>(&s.V[2 * kp + e][dg * 8 + x]) = v4f{xv[e][x], xv[e][x + 1], xv[e][x + 2], xv[e][x + 3]};
      }
  }
  if (dg == 0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool scaled = kCKV == CSA_FP8_E4M3 && (kAll || pr.src[e] == 1);
      s.sk[2 * kp + e] = (scaled ? pr.sk[e] : 1.f) * sk_mul;
      s.sv[2 * kp + e] = scaled ? pr.sv[e] : 1.f;
      s.bias[2 * kp + e] = !kSrcBias || pr.src[e] != 0 ? 0.f : -INFINITY;
    }
  }
}

// S^T for one 16-key tile `kt` of the chunk, scaled to the log2 domain and masked.
template <int kIO>
CSA_DEV void logits_tile(const LdsChunk<kIO>& s, const u32x4* qb, const float* qf, int kt, int col, int g, float* x) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kIO == CSA_BF16) {
    u32x4 kf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[ks] = *reinterpret_cast<const u32x4*>(&s.K[kt * 16 + col][ks * 32 + g * 8]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma_k32(kf[ks], qb[ks], acc);
  } else {
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) acc = mfma_f32(s.K[kt * 16 + col][ks * 4 + g], qf[ks], acc);
  }
  // keys kt*16 + 4g .. +3: one 16-byte read each for the scales and biases,
  // no branch (an absent key's product is 0, and 0 * sk + -inf = -inf)
  const v4f skv = *reinterpret_cast<const v4f*>(&s.sk[kt * 16 + 4 * g]);
  const v4f bv = *reinterpret_cast<const v4f*>(&s.bias[kt * 16 + 4 * g]);
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = __builtin_fmaf(acc[r], skv[r], bv[r]);
}

template <int kIO>
CSA_DEV void store_out4(void* out, long orow, int d4, v4f v) {
  if constexpr (kIO == CSA_BF16) {
    const uint32_t w0 = pack_bf16x2(v[0], v[1]);
    const uint32_t w1 = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow * kHeadDim + d4 * 4) = u32x2{w0, w1};
  } else {
    *reinterpret_cast<v4f*>(static_cast<float*>(out) + orow * kHeadDim + d4 * 4) = v;
  }
}

// Sequential fold of a piece's state (m, l, o) into a running one (Mr, Lr,
// Or), used wherever the batch-invariant calls combine pieces: in a block
// that walks a row's pieces (attn_kernel<..., kFold>) and in attn_fold_kernel
// over the pieces' partials.  The same two functions in both places keep the
// operations, and so the bits, identical.
struct FoldW {
  float fa, fb;   // weights of the running state and of the piece
  float M, L;     // the new running max and sum
};
CSA_DEV FoldW fold_weights(float Mr, float Lr, float m, float l) {
  FoldW w;
  w.M = fmaxf(Mr, m);
  const float Mu = w.M == -INFINITY ? 0.f : w.M;
  w.fa = __builtin_amdgcn_exp2f(Mr - Mu);
  w.fb = __builtin_amdgcn_exp2f(m - Mu);
  w.L = __builtin_fmaf(Lr, w.fa, l * w.fb);
  return w;
}
CSA_DEV float fold_elem(float Or, float o, const FoldW& w) { return __builtin_fmaf(Or, w.fa, o * w.fb); }

// kFold (batch-invariant calls, one block per query row): the block walks
// every piece (split) of its row in order and folds each piece's state into a
// running one (fold_weights / fold_elem), as attn_fold_kernel folds the
// pieces' partials when the pieces run as blocks of their own.
template <int kIO, int kCKV, bool kDense, int kHTW, int kDepth, bool kVarlen, bool kFold>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kIO == CSA_BF16 && kHTW == 1
                                       ? (kDepth > 1 || (kFold && kCKV == CSA_FP8_E4M3) ? 2 : 4)
                                       : 1)))
void attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsChunk<kIO>& s = *reinterpret_cast<LdsChunk<kIO>*>(smem);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int kh = wid >> 2;
  const int wt = wid & 3;

  const long qrow = kFold ? long(blockIdx.x) : blockIdx.x / a.n_splits;
  const int split = kFold ? 0 : int(blockIdx.x - qrow * a.n_splits);
  int b, t;
  if constexpr (kVarlen) {
    packed_row(a, qrow, &b, &t);
  } else {
    b = int(qrow / a.T_q);
    t = a.q_pos0[b] + int(qrow - long(b) * a.T_q);
  }
  const int raw0 = a.W > 0 ? a.raw_pos0[b] : 0;
  const int n_tiles = a.H / 16;
  const int j_begin = split * a.split_len;
  const int j_end = kFold ? a.n_list : min(j_begin + a.split_len, a.n_list);

  bool act[kHTW];
  u32x4 qb[kHTW][4];
  float qf[kHTW][kIO == CSA_F32 ? 32 : 1];
#pragma unroll
  for (int ht = 0; ht < kHTW; ++ht) {
    const int tile = wt + 4 * ht;
    act[ht] = tile < n_tiles;
    if (!act[ht]) continue;
    const int head = tile * 16 + col;
    if constexpr (kIO == CSA_BF16) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[ht][ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
    } else {
      const float* qp = static_cast<const float*>(a.q) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) qf[ht][ks] = qp[ks * 4 + g];
    }
  }

  v4f o[kHTW][8];
  float m_run[kHTW], l_run[kHTW];
#pragma unroll
  for (int ht = 0; ht < kHTW; ++ht) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }

  // one chunk in LDS: logits, online softmax and P*V for this wave's tiles
  auto compute = [&]() {
#pragma unroll
    for (int ht = 0; ht < kHTW; ++ht) {
      if (!act[ht]) continue;
      float x[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) logits_tile<kIO>(s, qb[ht], qf[ht], 2 * kh + kk, col, g, x[kk]);
      float cmax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, x[kk][r]);
      cmax = column_max(cmax);
      // lazy running max: it moves only when a logit exceeds it by more than
      // 8 (log2 domain), so exponentials stay below 2^8 and waves whose lanes
      // all keep their max skip the rescale of o and l
      const bool grow = cmax > m_run[ht] + 8.f;
      const float m_new = grow ? cmax : m_run[ht];
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      if (__ballot(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[ht] - m_use) : 1.f;
        l_run[ht] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[ht][dt] *= alpha;
      }
      m_run[ht] = m_new;
      float p[2][4];
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kk][r] = __builtin_amdgcn_exp2f(x[kk][r] - m_use);
          psum += p[kk][r];
        }
      l_run[ht] += psum;

      // O^T += V^T P^T (P carries the per-entry V scale)
      if constexpr (kIO == CSA_BF16) {
        // one 32-key step: contraction slot 8g+j <-> key 4g+j (j<4) / 16+4g+(j-4) of the half
        // P as bf16 hi + lo (two passes): a single bf16 rounding of P would
        // cost 2^-9 of |V| per output, beyond the bf16 bound for large V
        uint32_t ph[4], pl[4];
        const v4f svv[2] = {*reinterpret_cast<const v4f*>(&s.sv[(2 * kh) * 16 + 4 * g]),
                            *reinterpret_cast<const v4f*>(&s.sv[(2 * kh + 1) * 16 + 4 * g])};
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          const int kk = h2 >> 1;
          const int r0 = (h2 & 1) * 2;
          split_bf16x2(p[kk][r0] * svv[kk][r0], p[kk][r0 + 1] * svv[kk][r0 + 1], &ph[h2], &pl[h2]);
        }
        const u32x4 pbh = {ph[0], ph[1], ph[2], ph[3]};
        const u32x4 pbl = {pl[0], pl[1], pl[2], pl[3]};
        const int k0 = kh * 32 + 4 * g;
        if constexpr (kHTW == 1 && kDepth == 1 && !(kFold && kCKV == CSA_FP8_E4M3)) {
          // 128-VGPR budget (two blocks per CU): one V^T fragment at a time
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            // row dt*16 + col, keys k0 .. k0+3 and k0+16 .. k0+19 (one 16-byte word)
            const u32x4 vf = *reinterpret_cast<const u32x4*>(&s.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0 + 4 * g]);
            o[ht][dt] = mfma_k32(vf, pbh, o[ht][dt]);
            o[ht][dt] = mfma_k32(vf, pbl, o[ht][dt]);
          }
        } else {
          // every V^T fragment requested first, then the hi products, then the lo ones
          u32x4 vf[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            // row dt*16 + col, keys k0 .. k0+3 and k0+16 .. k0+19 (one 16-byte word)
            vf[dt] = *reinterpret_cast<const u32x4*>(&s.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0 + 4 * g]);
          }
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[ht][dt] = mfma_k32(vf[dt], pbh, o[ht][dt]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[ht][dt] = mfma_k32(vf[dt], pbl, o[ht][dt]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = (2 * kh + kk) * 16 + 4 * g + r;
            const float pv = p[kk][r] * s.sv[key];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[ht][dt] = mfma_f32(s.V[key][dt * 16 + col], pv, o[ht][dt]);
          }
      }
    }
  };

  // kDepth chunks in flight: buffer d holds chunks d, d + kDepth, ...  Every
  // prefetch is issued, past the split too (empty slots read a dummy
  // address): the same loads on every path keep the compiler's waits exact.
  // Indices run one round of chunks ahead of the rows they name.
  Pre<kIO> pr[kDepth];
  int e_nx[kDepth][2];
  // kSel (sparse lists, bf16 queries, one chunk in flight, no fold): chunks
  // [j_begin, j_sel) hold selected-entry slots only and take prefetch_sel and
  // the select-free store_chunk; the rest (the window) the general path
  constexpr bool kSel = !kDense && kIO == CSA_BF16 && kDepth == 1 && !kFold;
  const int j_sel = kSel && a.cap > 0 ? j_begin + max(0, min(a.k, j_end) - j_begin) / kNK * kNK : j_begin;
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_idx<kDense>(a, e_nx[d], qrow, j_begin + d * kNK, j_end);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    if constexpr (kSel) {
      if (j_begin < j_sel)
        prefetch_sel<kCKV>(a, pr[d], e_nx[d], b);
      else
        prefetch<kIO, kCKV, kDense>(a, pr[d], e_nx[d], b, t, raw0, j_begin + d * kNK, j_end);
    } else {
      prefetch<kIO, kCKV, kDense>(a, pr[d], e_nx[d], b, t, raw0, j_begin + d * kNK, j_end);
    }
    load_idx<kDense>(a, e_nx[d], qrow, j_begin + (d + kDepth) * kNK, j_end);
  }
  // The state of the keys walked since the last piece start: the second key
  // half hands its (o, max, sum) to the first through LDS; the first-half
  // waves (kh == 0) then merge it with their own, 16 head dims at a time, and
  // hand each merged slice to `emit(ht, dt, oo)` after `head(ht, M, L)` gave
  // the merged max and sum (no array of the merged state is held).
  LdsHalf<kHTW>& hf = *reinterpret_cast<LdsHalf<kHTW>*>(smem);
  auto piece_state = [&](auto&& head, auto&& emit) {
    float l_tot[kHTW];
#pragma unroll
    for (int ht = 0; ht < kHTW; ++ht) l_tot[ht] = column_sum(l_run[ht]);
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int ht = 0; ht < kHTW; ++ht) {
        if (!act[ht]) continue;
        const int tile = wt + 4 * ht;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(&hf.o[tile][col][dt * 16 + 4 * g]) = o[ht][dt];
        if (g == 0) {
          hf.m[tile][col] = m_run[ht];
          hf.l[tile][col] = l_tot[ht];
        }
      }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int ht = 0; ht < kHTW; ++ht) {
        if (!act[ht]) continue;
        const int tile = wt + 4 * ht;
        const float m1 = hf.m[tile][col];
        const float M = fmaxf(m_run[ht], m1);
        const float Mu = M == -INFINITY ? 0.f : M;
        const float f0 = __builtin_amdgcn_exp2f(m_run[ht] - Mu);
        const float f1 = __builtin_amdgcn_exp2f(m1 - Mu);
        head(ht, M, __builtin_fmaf(l_tot[ht], f0, hf.l[tile][col] * f1));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v4f h1 = *reinterpret_cast<const v4f*>(&hf.o[tile][col][dt * 16 + 4 * g]);
          v4f oo;
#pragma unroll
          for (int c = 0; c < 4; ++c) oo[c] = __builtin_fmaf(o[ht][dt][c], f0, h1[c] * f1);
          emit(ht, dt, oo);
        }
      }
    }
  };

  // kFold: the running state of the pieces folded so far lives in LDS beside
  // the chunk and hand-over areas (held in registers it would not fit)
  LdsFold<kHTW>& fs = *reinterpret_cast<LdsFold<kHTW>*>(smem + lds_bytes<kIO, kHTW>());
  int piece_end = kFold ? min(a.split_len, j_end) : j_end;
  if constexpr (kFold) {
    // the fold starts from the empty state (max -inf, sum 0, output 0), as
    // attn_fold_kernel's does; each wave owns its own slots (no barrier needed)
    if (kh == 0) {
#pragma unroll
      for (int ht = 0; ht < kHTW; ++ht) {
        const int tile = wt + 4 * ht;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(&fs.o[tile][col][dt * 16 + 4 * g]) = v4f{0.f, 0.f, 0.f, 0.f};
        if (g == 0) {
          fs.m[tile][col] = -INFINITY;
          fs.l[tile][col] = 0.f;
        }
      }
    }
  }
  int j_gen = j_begin;   // first chunk of the general walk
  if constexpr (kSel) {
    // selected-entry chunks, each stored as it was fetched (the next one's
    // form follows its own position)
    for (; j_gen < j_sel; j_gen += kNK) {
      __syncthreads();
      store_chunk<kIO, kCKV, true, false, true>(s, pr[0], a.sm_log2);
      __syncthreads();
      if (j_gen + kNK < j_sel)
        prefetch_sel<kCKV>(a, pr[0], e_nx[0], b);
      else
        prefetch<kIO, kCKV, kDense>(a, pr[0], e_nx[0], b, t, raw0, j_gen + kNK, j_end);
      load_idx<kDense>(a, e_nx[0], qrow, j_gen + 2 * kNK, j_end);
      compute();
    }
  }
  for (int j0 = j_gen; j0 < j_end; j0 += kDepth * kNK) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (d > 0 && j0 + d * kNK >= j_end) break;
      __syncthreads();
      store_chunk<kIO, kCKV>(s, pr[d], a.sm_log2);
      __syncthreads();
      prefetch<kIO, kCKV, kDense>(a, pr[d], e_nx[d], b, t, raw0, j0 + (d + kDepth) * kNK, j_end);
      load_idx<kDense>(a, e_nx[d], qrow, j0 + (d + 2 * kDepth) * kNK, j_end);
      compute();
      if constexpr (kFold) {
        if (j0 + (d + 1) * kNK >= piece_end) {   // last chunk of a piece (uniform)
          // fold the piece into the running state, 16 head dims at a time
          FoldW fw[kHTW];
          piece_state(
              [&](int ht, float M, float L) {
                const int tile = wt + 4 * ht;
                fw[ht] = fold_weights(fs.m[tile][col], fs.l[tile][col], M, L);
                if (g == 0) {
                  fs.m[tile][col] = fw[ht].M;
                  fs.l[tile][col] = fw[ht].L;
                }
              },
              [&](int ht, int dt, const v4f& oo) {
                v4f* slot = reinterpret_cast<v4f*>(&fs.o[wt + 4 * ht][col][dt * 16 + 4 * g]);
                const v4f Or = *slot;
                v4f On;
#pragma unroll
                for (int c = 0; c < 4; ++c) On[c] = fold_elem(Or[c], oo[c], fw[ht]);
                *slot = On;
              });
          piece_end = min(piece_end + a.split_len, j_end);
#pragma unroll
          for (int ht = 0; ht < kHTW; ++ht) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
            m_run[ht] = -INFINITY;
            l_run[ht] = 0.f;
          }
        }
      }
    }
  }
  if constexpr (kFold) {
    // the row's output from the folded state (as attn_fold_kernel finishes it)
    if (kh == 1) return;
#pragma unroll
    for (int ht = 0; ht < kHTW; ++ht) {
      if (!act[ht]) continue;
      const int tile = wt + 4 * ht;
      const long orow = qrow * a.H + tile * 16 + col;
      const float M = fs.m[tile][col], L = fs.l[tile][col];
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        store_out4<kIO>(a.out, orow, dt * 4 + g, *reinterpret_cast<const v4f*>(&fs.o[tile][col][dt * 16 + 4 * g]) * inv);
      if (a.lse && g == 0) a.lse[orow] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
    }
  } else {
    float Ls[kHTW], invs[kHTW];
    piece_state(
        [&](int ht, float M, float L) {
          const int tile = wt + 4 * ht;
          const long orow = qrow * a.H + tile * 16 + col;
          Ls[ht] = L;
          invs[ht] = L > 0.f ? 1.f / L : 0.f;
          if (a.n_splits == 1) {
            if (a.lse && g == 0) a.lse[orow] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
          } else if (g == 0) {
            // this split's unnormalised state; the merge kernel combines the splits
            // (streaming stores: the partials are read once, by another kernel)
            const long slot = (qrow * a.n_splits + split) * a.H + tile * 16 + col;
            __builtin_nontemporal_store(M, &a.part_ml[slot * 2]);
            __builtin_nontemporal_store(L, &a.part_ml[slot * 2 + 1]);
          }
        },
        [&](int ht, int dt, const v4f& oo) {
          const int tile = wt + 4 * ht;
          if (a.n_splits == 1) {
            store_out4<kIO>(a.out, qrow * a.H + tile * 16 + col, dt * 4 + g, oo * invs[ht]);
          } else {
            const long slot = (qrow * a.n_splits + split) * a.H + tile * 16 + col;
            __builtin_nontemporal_store(oo, reinterpret_cast<v4f*>(a.part_o + slot * kHeadDim + dt * 16 + 4 * g));
          }
        });
    (void)Ls;
  }
}

// Merge of the key splits of one (query, head) by one wave: lane x reads
// split x's (max, sum) (at most 64 splits); the wave-wide max and the
// weighted sum go through permutes and DPP rotations (no LDS round trips),
// the per-split weights through a 64-entry LDS array.  Lane (h, d4)
// accumulates splits h, h+2, ... of float4 d4 (their loads issued before the
// reductions), and the two halves are added at the end.  Fixed order.
template <int kIO>
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                        const float* __restrict__ part_o, int n_splits, int H,
                                                        void* out, float* lse, const int32_t* __restrict__ cu_rows,
                                                        int kq) {
  __shared__ float wsh[64];
  const long hid = blockIdx.x;                  // partial row * H + head
  const int lane = threadIdx.x;
  const long qrow = hid / H;
  const int head = int(hid - qrow * H);
  const long base = qrow * n_splits * H + head; // slot of split 0; split x adds x*H
  // cu_rows: partial row qrow is query qrow % kq of sequence qrow / kq, a
  // sequence of at most kq rows (the pieces of the varlen many-query launch);
  // rows of other sequences have no partials (the whole wave leaves)
  long ohid = hid;
  if (cu_rows) {
    const int b = int(qrow / kq);
    const int qi = int(qrow - long(b) * kq);
    const int n = cu_rows[b + 1] - cu_rows[b];
    if (n > kq || qi >= n) return;
    ohid = (long(cu_rows[b]) + qi) * H + head;
  }
  const int half = lane >> 5;
  const int d4 = lane & 31;
  constexpr int kU = 16;   // 32 splits per batch of loads
  auto load_batch = [&](int x0, v4f (&pv)[kU]) {
#pragma unroll
    for (int y = 0; y < kU; ++y) {
      const int x = x0 + 2 * y + half;
      pv[y] = x < n_splits ? *reinterpret_cast<const v4f*>(part_o + (base + long(x) * H) * kHeadDim + d4 * 4)
                           : v4f{0.f, 0.f, 0.f, 0.f};
    }
  };
  v4f pv[kU];
  load_batch(0, pv);
  float mx = -INFINITY, lx = 0.f;
  if (lane < n_splits) {
    mx = part_ml[(base + long(lane) * H) * 2];
    lx = part_ml[(base + long(lane) * H) * 2 + 1];
  }
  const float M = wave_max_all(mx);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float fx = lane < n_splits ? exp2f(mx - Mu) : 0.f;
  const float L = wave_sum_all(lx * fx);
  wsh[lane] = fx;
  __syncthreads();
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int x0 = 0; x0 < n_splits; x0 += 2 * kU) {
    if (x0 > 0) load_batch(x0, pv);
#pragma unroll
    for (int y = 0; y < kU; ++y) {
      const int x = x0 + 2 * y + half;
      if (x < n_splits) acc += pv[y] * wsh[x];
    }
  }
  auto add = [](float u, float w) { return u + w; };
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = swap_combine<32>(acc[c], add);
  if (half == 0) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    store_out4<kIO>(out, ohid, d4, acc * inv);
    if (lse && d4 == 0) lse[ohid] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
  }
}

// Fold of the pieces of one (query, head) for the batch-invariant calls, by
// one wave: lane x holds piece x's (max, sum) (at most 64 pieces), lane l
// the head dims 2l, 2l+1; pieces 0, 1, ... fold in order into the empty state
// (max -inf, sum 0, output 0) with fold_weights / fold_elem -- as
// attn_kernel<..., kFold> does when one block walks the pieces -- and the row
// is normalised as there.
template <int kIO>
__global__ __launch_bounds__(64) void attn_fold_kernel(const float* __restrict__ part_ml,
                                                       const float* __restrict__ part_o, int n_splits, int H,
                                                       void* out, float* lse) {
  const long hid = blockIdx.x;                  // query row * H + head
  const int lane = threadIdx.x;
  const long qrow = hid / H;
  const int head = int(hid - qrow * H);
  const long base = qrow * n_splits * H + head; // slot of piece 0; piece x adds x*H
  float mx = -INFINITY, lx = 0.f;
  if (lane < n_splits) {
    mx = part_ml[(base + long(lane) * H) * 2];
    lx = part_ml[(base + long(lane) * H) * 2 + 1];
  }
  constexpr int kU = 16;
  v2f_t ov[kU];
  auto load_batch = [&](int x0) {
#pragma unroll
    for (int y = 0; y < kU; ++y) {
      const int x = min(x0 + y, n_splits - 1);
      ov[y] = *reinterpret_cast<const v2f_t*>(part_o + (base + long(x) * H) * kHeadDim + 2 * lane);
    }
  };
  load_batch(0);
  float M = -INFINITY, L = 0.f;
  v2f_t O = {0.f, 0.f};
  for (int x0 = 0; x0 < n_splits; x0 += kU) {
    if (x0 > 0) load_batch(x0);
#pragma unroll
    for (int y = 0; y < kU; ++y) {
      const int x = x0 + y;
      if (x >= n_splits) continue;
      const FoldW fw = fold_weights(M, L, __shfl(mx, x), __shfl(lx, x));
      O[0] = fold_elem(O[0], ov[y][0], fw);
      O[1] = fold_elem(O[1], ov[y][1], fw);
      M = fw.M;
      L = fw.L;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const v2f_t r = O * inv;
  if constexpr (kIO == CSA_BF16) {
    static_cast<uint32_t*>(out)[(hid * kHeadDim + 2 * lane) / 2] = pack_bf16x2(r[0], r[1]);
  } else {
    *reinterpret_cast<v2f_t*>(static_cast<float*>(out) + hid * kHeadDim + 2 * lane) = r;
  }
  if (lse && lane == 0) lse[hid] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
}

// ---------------------------------------------------------- decode rows --
// Few query rows over long key lists (decoding).  A block takes one split of
// a row's key list (at most kDecChunks chunks, 256 keys) and one group of
// kT 16-head tiles; all of the split's index and row loads are issued at
// once, the whole split is staged in LDS behind one barrier, and the chip is
// filled by splits and head groups rather than by a pipeline of chunks inside
// a block.  The G head groups of one split run on the same XCD (block b runs
// on XCD b % 8), so G-1 of the G gathers of each row are served by that
// XCD's L2: a split count G times smaller for the same number of blocks, and
// G times fewer partial outputs to write and merge.
// Waves: tile slot w % kT (heads (group * kT + w % kT) * 16 ..), key part
// p = w / kT of kP = 8 / kT parts: the 32-key steps s = p, p + kP, ... of the
// split.  The parts fold into part 0 through LDS in part order, then the
// block writes its row's output (one split) or its split's partial state.
constexpr int kDecChunks = 4;

struct DecFold {
  float o[7][16][kHeadDim + 4];   // parts 1 .. kP-1 of every tile slot (kT * (kP - 1) <= 7)
  float m[7][16];
  float l[7][16];
};

template <int kCKV, bool kDense, bool kVarlen>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void attn_decode_kernel(AttnArgs a, int kT, int n_groups, long n_units) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsBf16* ch = reinterpret_cast<LdsBf16*>(smem);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int kP = 8 / kT;
  const int ts = wid % kT;
  const int part = wid / kT;

  // block -> (unit = query row x split, head group); the groups of a unit share an XCD
  const long bid = blockIdx.x;
  const int xcd = int(bid & 7);
  const long slot = bid >> 3;
  const int grp = int(slot % n_groups);
  const long unit = (slot / n_groups) * 8 + xcd;
  if (unit >= n_units) return;
  const long qrow = unit / a.n_splits;
  const int split = int(unit - qrow * a.n_splits);
  int b, t;
  if constexpr (kVarlen) {
    packed_row(a, qrow, &b, &t);
  } else {
    b = int(qrow / a.T_q);
    t = a.q_pos0[b] + int(qrow - long(b) * a.T_q);
  }
  const int raw0 = a.W > 0 ? a.raw_pos0[b] : 0;
  const int j_begin = split * a.split_len;
  const int j_end = min(j_begin + a.split_len, a.n_list);
  const int n_keys = j_end - j_begin;

  // every index, then every row of the split in flight (empty slots read a
  // dummy address; see gather_slot).  Chunks past the split issue nothing: the
  // branch is uniform over the block, so no load sits under a divergent mask.
  const int n_ch = (n_keys + kNK - 1) / kNK;
  int e[kDecChunks][2];
#pragma unroll
  for (int c = 0; c < kDecChunks; ++c)
    if (c < n_ch) load_idx<kDense>(a, e[c], qrow, j_begin + c * kNK, j_end);
  Pre<CSA_BF16> pr[kDecChunks];
#pragma unroll
  for (int c = 0; c < kDecChunks; ++c)
    if (c < n_ch) prefetch<CSA_BF16, kCKV, kDense>(a, pr[c], e[c], b, t, raw0, j_begin + c * kNK, j_end);
  const int tile = grp * kT + ts;
  const int head = tile * 16 + col;
  u32x4 qb[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
  }
  // chunks past the split's keys are not staged (the LDS holds only the split)
#pragma unroll
  for (int c = 0; c < kDecChunks; ++c)
    if (c < n_ch) store_chunk<CSA_BF16, kCKV>(ch[c], pr[c], a.sm_log2);
  __syncthreads();

  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // 32-key steps of this wave's part; steps past the split's keys are skipped
  for (int st = part; st * 32 < n_keys; st += kP) {
    const LdsBf16& s = ch[st >> 1];
    const int kh = st & 1;
    float x[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) logits_tile<CSA_BF16>(s, qb, nullptr, 2 * kh + kk, col, g, x[kk]);
    float cmax = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, x[kk][r]);
    cmax = column_max(cmax);
    // lazy running max, as in attn_kernel
    const bool grow = cmax > m_run + 8.f;
    const float m_new = grow ? cmax : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    m_run = m_new;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kk][r] = __builtin_amdgcn_exp2f(x[kk][r] - m_use);
        psum += p[kk][r];
      }
    l_run += psum;
    uint32_t ph[4], pl[4];
    const v4f svv[2] = {*reinterpret_cast<const v4f*>(&s.sv[(2 * kh) * 16 + 4 * g]),
                        *reinterpret_cast<const v4f*>(&s.sv[(2 * kh + 1) * 16 + 4 * g])};
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2) {
      const int kk = h2 >> 1;
      const int r0 = (h2 & 1) * 2;
      split_bf16x2(p[kk][r0] * svv[kk][r0], p[kk][r0 + 1] * svv[kk][r0 + 1], &ph[h2], &pl[h2]);
    }
    const u32x4 pbh = {ph[0], ph[1], ph[2], ph[3]};
    const u32x4 pbl = {pl[0], pl[1], pl[2], pl[3]};
    const int k0 = kh * 32 + 4 * g;
    // every V^T fragment requested first, then the 8 hi products, then the 8
    // lo ones (no product waits on the one before it)
    u32x4 vf[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      // row dt*16 + col, keys k0 .. k0+3 and k0+16 .. k0+19 (one 16-byte word)
      vf[dt] = *reinterpret_cast<const u32x4*>(&s.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0 + 4 * g]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = mfma_k32(vf[dt], pbh, o[dt]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = mfma_k32(vf[dt], pbl, o[dt]);
  }
  float l_tot = column_sum(l_run);

  // fold parts 1 .. kP-1 into part 0, in part order: every part > 0 of every
  // tile slot parks its state at once (kT * (kP - 1) <= 7 slots), one barrier
  DecFold& fd = *reinterpret_cast<DecFold*>(smem);
  __syncthreads();
  if (part > 0) {
    const int f = ts * (kP - 1) + part - 1;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(&fd.o[f][col][dt * 16 + 4 * g]) = o[dt];
    if (g == 0) {
      fd.m[f][col] = m_run;
      fd.l[f][col] = l_tot;
    }
  }
  __syncthreads();
  if (part == 0) {
    for (int q = 1; q < kP; ++q) {
      const int f = ts * (kP - 1) + q - 1;
      const float m1 = fd.m[f][col];
      const float M = fmaxf(m_run, m1);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float f0 = __builtin_amdgcn_exp2f(m_run - Mu);
      const float f1 = __builtin_amdgcn_exp2f(m1 - Mu);
      l_tot = l_tot * f0 + fd.l[f][col] * f1;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = o[dt] * f0 + *reinterpret_cast<const v4f*>(&fd.o[f][col][dt * 16 + 4 * g]) * f1;
      m_run = M;
    }
  }
  if (part > 0) return;
  if (a.n_splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const long orow = qrow * a.H + head;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_out4<CSA_BF16>(a.out, orow, dt * 4 + g, o[dt] * inv);
    if (a.lse && g == 0) a.lse[orow] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  } else {
    const long pslot = (qrow * a.n_splits + split) * a.H + head;
    float* po = a.part_o + pslot * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) __builtin_nontemporal_store(o[dt], reinterpret_cast<v4f*>(po + dt * 16 + 4 * g));
    if (g == 0) {
      __builtin_nontemporal_store(m_run, &a.part_ml[pslot * 2]);
      __builtin_nontemporal_store(l_tot, &a.part_ml[pslot * 2 + 1]);
    }
  }
}

// ------------------------------------------------- dense, many queries --
// HCA prefill: consecutive queries of a sequence see nearly the same keys
// (entries e < floor((t+1)/m') and a window that moves by one position per
// query), so a block takes kQB = 256/H consecutive queries (H = 32, 64, 128) and streams the
// UNION of their key lists: entries [0, nvis(last query)) then raw positions
// [t_first - W + 1, t_last].  Every gathered chunk serves all kQB queries;
// each key carries a tag (entry index, or raw position) from which each
// query's wave applies its own visibility.  Wave w takes query w / (8/kQB)
// and two 16-head tiles; both tiles share every K and V^T fragment it reads
// from LDS.  Each key takes part exactly as in the one-query kernel, so the
// arithmetic per (query, head) is the same online softmax over 64-key chunks.
struct LdsMQ {
  LdsBf16 c[2];           // two chunk buffers: one computed while the next is stored
  uint32_t vis[2][kNK];   // bit q: the key is visible to the block's query q
  // each wave's query fragments (2 head tiles x 4 contraction steps, one
  // 16-byte word per lane), re-read for every chunk instead of held in
  // registers through the P*V products
  u32x4 q[8][2][4][64];
};

// Gather items of chunk jc of the union list, and for each key the mask of
// the block's queries (positions t0 + q, q < n_q) that see it: entry j is seen
// from t >= (j+1)*m' - 1 on, raw position p by t in [p, p + W - 1].
template <int kCKV>
CSA_DEV void prefetch_mq(const AttnArgs& a, Pre<CSA_BF16>& pr, uint32_t (&vis)[2], int b, int raw0, int nv_max,
                         int p_lo, int n_list, int jc, int t0, int n_q) {
  const int kp = item_kp();
  const int dg = item_dg();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int j = jc + 2 * kp + x;
    long row = 0;
    int src = 0, q_from = n_q, q_to = -1;
    if (j < nv_max) {
      row = long(b) * a.cap + j;
      src = 1;
      q_from = max(0, (j + 1) * a.k - 1 - t0);
      q_to = n_q - 1;
    } else if (j < n_list) {
      const int p = p_lo + (j - nv_max);
      const int r = p - raw0;
      if (p >= 0 && r >= 0 && r < a.L_raw) {
        row = long(b) * a.L_raw + r;
        src = 2;
        q_from = max(0, p - t0);
        q_to = min(n_q - 1, p + a.W - 1 - t0);
      }
    }
    vis[x] = q_from <= q_to ? ((2u << q_to) - 1u) & ~((1u << q_from) - 1u) : 0u;
    gather_slot<CSA_BF16, kCKV>(a, pr, x, src, row, dg);
  }
}

// Rows of a chunk whose 64 slots are the compressed entries row0 .. row0 + 63,
// every one seen by every query of the block (most chunks of a dense list):
// no window rows, no empty slots, so neither source selects nor visibility
// masks.  Same item mapping and loads as gather_slot with src 1.
template <int kCKV>
CSA_DEV void prefetch_entries(const AttnArgs& a, Pre<CSA_BF16>& pr, long row0) {
  constexpr long kCB = kCKV == CSA_BF16 ? 2 : 1;   // bytes per compressed value (bf16 or fp8)
  const int kp = item_kp();
  const int dg = item_dg();
  const long r = row0 + 2 * kp;
  const long off = r * (kHeadDim * kCB) + (kCKV == CSA_FP8_E4M3 ? long(dg & ~1) * 8 : long(dg) * 8 * kCB);
  const char* pk = static_cast<const char*>(a.ck) + off;
  const char* pv = static_cast<const char*>(a.cv) + off;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    pr.k[x][0] = *reinterpret_cast<const u32x4*>(pk + x * kHeadDim * kCB);
    pr.v[x][0] = *reinterpret_cast<const u32x4*>(pv + x * kHeadDim * kCB);
    if constexpr (kCKV == CSA_FP8_E4M3) {
      pr.sk[x] = a.ck_scale[r + x];
      pr.sv[x] = a.cv_scale[r + x];
    } else {
      pr.sk[x] = 1.f;
      pr.sv[x] = 1.f;
    }
    pr.src[x] = 1;
  }
}

// Tile `tile` of a varlen many-query launch: the rows of every sequence with
// more than kQB rows cut into tiles of kQB, sequences in order (sequences of
// at most kQB rows are served by pieces instead).  False past the last tile.
template <int kQB>
CSA_DEV bool mq_tile(const int32_t* __restrict__ cu_rows, int n_seq, long tile, int* b, int* i0) {
  long t = 0;
  for (int x = 0; x < n_seq; ++x) {
    const int n = cu_rows[x + 1] - cu_rows[x];
    const long tiles = n > kQB ? (n + kQB - 1) / kQB : 0;
    if (tile < t + tiles) {
      *b = x;
      *i0 = int(tile - t) * kQB;
      return true;
    }
    t += tiles;
  }
  return false;
}

// kPacked (varlen calls): blocks [0, n_seq * n_pieces) take piece x of
// sequence b's key list (b = block / n_pieces) when that sequence has at most
// kQB rows, and write the piece's partial state for attn_merge_kernel; the
// rest take the tiles of the longer sequences (mq_tile) whole.  A decode row
// then spreads over many CUs instead of holding one for a whole tile's time.
template <int kCKV, int kQB, bool kPacked>
__global__ __launch_bounds__(kThreads) void attn_mq_kernel(AttnArgs a) {
  static_assert(kQB == 2 || kQB == 4 || kQB == 8, "two 16-head tiles per wave");
  constexpr int kWPQ = 8 / kQB;   // waves per query; each takes two 16-head tiles
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsMQ& s = *reinterpret_cast<LdsMQ*>(smem);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  int b, i0, T_b, piece = -1;
  long row_base;   // packed row of the sequence's query 0
  if constexpr (kPacked) {
    const long n_piece_blocks = long(a.n_seq) * a.n_pieces;
    if (long(blockIdx.x) < n_piece_blocks) {
      b = int(blockIdx.x / a.n_pieces);
      piece = int(blockIdx.x - long(b) * a.n_pieces);
      T_b = a.cu_rows[b + 1] - a.cu_rows[b];
      if (T_b == 0 || T_b > kQB) return;   // the whole block, before any barrier
      i0 = 0;
    } else {
      if (!mq_tile<kQB>(a.cu_rows, a.n_seq, long(blockIdx.x) - n_piece_blocks, &b, &i0)) return;
      T_b = a.cu_rows[b + 1] - a.cu_rows[b];
    }
    row_base = a.cu_rows[b];
  } else {
    const int blocks_per_seq = (a.T_q + kQB - 1) / kQB;
    b = int(blockIdx.x / blocks_per_seq);
    i0 = int(blockIdx.x - long(b) * blocks_per_seq) * kQB;
    T_b = a.T_q;
    row_base = long(b) * a.T_q;
  }
  const int qi = wid / kWPQ;
  const int i = i0 + qi;
  const bool q_ok = i < T_b;
  const int pos0 = a.q_pos0[b];
  const int raw0 = a.W > 0 ? a.raw_pos0[b] : 0;
  const int i_last = min(i0 + kQB, T_b) - 1;
  const int nv_max = min((pos0 + i_last + 1) / a.k, a.cap);
  const int p_lo = pos0 + i0 - a.W + 1;
  const int n_win = a.W > 0 ? a.W + (i_last - i0) : 0;
  const int n_list = nv_max + n_win;
  const int t0 = pos0 + i0;
  const int n_q = i_last - i0 + 1;
  // the slots of the union list this block walks: all, or one piece
  const int j_lo = piece < 0 ? 0 : min(piece * a.piece_len, n_list);
  const int j_hi = piece < 0 ? n_list : min(j_lo + a.piece_len, n_list);

#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = ((wid % kWPQ) * 2 + ht) * 16 + col;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((row_base + (q_ok ? i : i0)) * a.H + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s.q[wid][ht][ks][lane] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
  }
  v4f o[2][8];
  float m_run[2], l_run[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }
  // fp8 entries: o is kept in units of vref, a power of two within 2^7 of
  // the current chunk's largest V scale (2^-126 .. 2^126), so that P x V
  // scale / vref stays below 2^15 and, for the chunk's larger scales, above
  // fp16's subnormal range in the one fp16 product of an all-entries chunk;
  // vref follows the scales lazily, o rescaled by an exact power of two (at
  // most 2^64 up per chunk)
  float vref = 0.f, vinv = 0.f;

  // Chunks [j_lo, j_full) hold only entries that every query of the block
  // sees (entry e is seen from position (e+1)*m' - 1 on; the block's first
  // query is the earliest): they are gathered without source selects and
  // scored without visibility masks.  The rest (the last entries, the
  // window) take the general path.
  const int nv_all = min((t0 + 1) / a.k, a.cap);
  const int j_full = j_lo + max(0, min(nv_all, j_hi) - j_lo) / kNK * kNK;
  const long row_b = long(b) * a.cap;
  auto fetch = [&](Pre<CSA_BF16>& prc, uint32_t (&tgc)[2], int jc) {
    if (jc < j_full)
      prefetch_entries<kCKV>(a, prc, row_b + jc);
    else
      prefetch_mq<kCKV>(a, prc, tgc, b, raw0, nv_max, p_lo, n_list, jc, t0, n_q);
  };
  // Pipeline: while chunk c is computed from LDS buffer c % 2, chunk c + 1
  // (loaded into registers during chunk c - 1) is stored into the other
  // buffer and chunk c + 2 loads into the registers; one barrier per chunk
  // separates the computing of chunk c from the overwriting of its buffer
  // and publishes chunk c + 1.
  Pre<CSA_BF16> pr;
  uint32_t tag[2];
  auto store = [&](auto all_t, int buf) {
    constexpr bool kAll = decltype(all_t)::value;
    store_chunk<CSA_BF16, kCKV, kAll>(s.c[buf], pr, a.sm_log2);
    if (!kAll && item_dg() == 0) {
      s.vis[buf][2 * item_kp()] = tag[0];
      s.vis[buf][2 * item_kp() + 1] = tag[1];
    }
  };
  auto compute = [&](auto all_t, int buf) {
    constexpr bool kAll = decltype(all_t)::value;
    const LdsBf16& c = s.c[buf];
    // S^T for the 4 key tiles x 2 head tiles; K fragments shared by both tiles,
    // contraction steps outermost so only one step's query fragments are live
    float x[2][4][4];
    // logits relative to the running max, x = S * scale - m (one fma; m = 0
    // before the first finite logit); a key the query does not see gets -inf
    float mu[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) mu[ht] = m_run[ht] == -INFINITY ? 0.f : m_run[ht];
    {
      v4f acc[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc[kt][0] = acc[kt][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // one contraction step's fragments requested together, then its 8 products
        const u32x4 q0 = s.q[wid][0][ks][lane];
        const u32x4 q1 = s.q[wid][1][ks][lane];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(&c.K[kt * 16 + col][ks * 32 + g * 8]);
          acc[kt][0] = mfma_k32(kf, q0, acc[kt][0]);
          acc[kt][1] = mfma_k32(kf, q1, acc[kt][1]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        // keys kt*16 + 4g .. +3 (16-byte reads)
        const v4f scl = *reinterpret_cast<const v4f*>(&c.sk[kt * 16 + 4 * g]);
        if constexpr (kAll) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) x[ht][kt][r] = __builtin_fmaf(acc[kt][ht][r], scl[r], -mu[ht]);
        } else {
          const u32x4 vb = *reinterpret_cast<const u32x4*>(&s.vis[buf][kt * 16 + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool seen = (vb[r] >> qi) & 1u;
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
              x[ht][kt][r] = __builtin_fmaf(acc[kt][ht][r], scl[r], seen ? -mu[ht] : -INFINITY);
          }
        }
      }
    }
    // all-entries chunks of fp8 entries: V^T is fp16 (exact) and P one fp16
    // operand (11 significant bits, about 2^-12 of |P V| per product); other
    // chunks: bf16 V^T and P as bf16 hi + lo
    constexpr bool kF16 = decltype(all_t)::value && kCKV == CSA_FP8_E4M3;
    // V scales of the chunk's keys (kt*16 + 4g .. +3), over vref
    v4f svk[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) svk[kt] = *reinterpret_cast<const v4f*>(&c.sv[kt * 16 + 4 * g]);
    if constexpr (kCKV == CSA_FP8_E4M3) {
      float smax = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) smax = fmaxf(smax, svk[kt][r]);
      smax = column_max(smax);   // every lane: the chunk's largest V scale
      const bool down = smax > 0.f && smax * 128.f < vref;
      if (smax > vref * 128.f || down) {
        // the power of two at or above smax (2^-126 .. 2^126), at most 2^64
        // below the old one; its inverse (exponent field 254 - E) and the
        // rescale of o are exact
        uint32_t eb = min((__float_as_uint(smax) + 0x007FFFFFu) & 0x7F800000u, 0x7E800000u);
        if (down) eb = max(eb, max(__float_as_uint(vref), 0x20800000u) - 0x20000000u);
        const float ninv = __uint_as_float(0x7F000000u - eb);
        const float f = vref * ninv;   // 0 before the first reference (o is 0 then)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[ht][dt] *= f;
        vref = __uint_as_float(eb);
        vinv = ninv;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) svk[kt] *= vinv;
    }
    uint32_t pw[2][2][4], pl[2][2][4];   // [ht][32-key step][pair]: P (fp16, or bf16 hi + lo)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float cmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, x[ht][kt][r]);
      cmax = column_max(cmax);
      // lazy running max, as in the one-query kernel: it moves only for a
      // first finite logit or one more than 2^8 above it (P stays <= 2^8)
      const bool grow = m_run[ht] == -INFINITY ? cmax > -INFINITY : cmax > 8.f;
      if (__ballot(grow)) {
        const float m_new = grow ? mu[ht] + cmax : m_run[ht];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[ht] - m_new) : 1.f;   // 0 from -inf
        const float sh = grow ? cmax : 0.f;
        l_run[ht] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[ht][dt] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[ht][kt][r] -= sh;
        m_run[ht] = m_new;
      }
      float psum = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kt][r] = __builtin_amdgcn_exp2f(x[ht][kt][r]);
          psum += p[kt][r];
        }
      l_run[ht] += psum;
      // 32-key step st covers key tiles 2st, 2st+1: contraction slot 8g+j <->
      // key (2st)*16 + 4g + j (j < 4) / (2st+1)*16 + 4g + j - 4
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int st = kt >> 1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int h2 = (kt & 1) * 2 + hh;
          const float a0 = p[kt][2 * hh] * svk[kt][2 * hh];
          const float a1 = p[kt][2 * hh + 1] * svk[kt][2 * hh + 1];
          if constexpr (kF16)
            pw[ht][st][h2] = pack_f16x2(a0, a1);
          else
            split_bf16x2(a0, a1, &pw[ht][st][h2], &pl[ht][st][h2]);
        }
      }
    }
    // O^T += V^T P^T; V^T fragments shared by both tiles
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int k0 = st * 32 + 4 * g;
      const u32x4 pb0 = {pw[0][st][0], pw[0][st][1], pw[0][st][2], pw[0][st][3]};
      const u32x4 pb1 = {pw[1][st][0], pw[1][st][1], pw[1][st][2], pw[1][st][3]};
      const u32x4 pl0 = {pl[0][st][0], pl[0][st][1], pl[0][st][2], pl[0][st][3]};
      const u32x4 pl1 = {pl[1][st][0], pl[1][st][1], pl[1][st][2], pl[1][st][3]};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        // row dt*16 + col, keys k0 .. k0+3 and k0+16 .. k0+19 (one 16-byte word)
        const u32x4 vf = *reinterpret_cast<const u32x4*>(&c.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0 + 4 * g]);
        if constexpr (kF16) {
          o[0][dt] = mfma_h32(vf, pb0, o[0][dt]);
          o[1][dt] = mfma_h32(vf, pb1, o[1][dt]);
        } else {
          o[0][dt] = mfma_k32(vf, pb0, o[0][dt]);
          o[1][dt] = mfma_k32(vf, pb1, o[1][dt]);
          o[0][dt] = mfma_k32(vf, pl0, o[0][dt]);
          o[1][dt] = mfma_k32(vf, pl1, o[1][dt]);
        }
      }
    }
  };
  const std::true_type all_entries;
  const std::false_type general;
  // A chunk is stored and computed in the same form (all-entries chunks hold
  // fp16 V^T for fp8 entries), and each form of a step sits in a loop of its
  // own: the walk over all-entries chunks, the one step where the next chunk
  // is general, then the general chunks.
  int buf = 0;
  if (j_lo < j_hi) {
    fetch(pr, tag, j_lo);
    if (j_lo < j_full) store(all_entries, 0); else store(general, 0);
    if (j_lo + kNK < j_hi) fetch(pr, tag, j_lo + kNK);
  }
  __syncthreads();
  int j0 = j_lo;
  for (; j0 + kNK < j_full; j0 += kNK) {
    store(all_entries, buf ^ 1);
    if (j0 + 2 * kNK < j_hi) fetch(pr, tag, j0 + 2 * kNK);
    compute(all_entries, buf);
    __syncthreads();
    buf ^= 1;
  }
  if (j0 < j_full) {
    if (j0 + kNK < j_hi) {
      store(general, buf ^ 1);
      if (j0 + 2 * kNK < j_hi) fetch(pr, tag, j0 + 2 * kNK);
    }
    compute(all_entries, buf);
    __syncthreads();
    buf ^= 1;
    j0 += kNK;
  }
  for (; j0 < j_hi; j0 += kNK) {
    if (j0 + kNK < j_hi) {
      store(general, buf ^ 1);
      if (j0 + 2 * kNK < j_hi) fetch(pr, tag, j0 + 2 * kNK);
    }
    compute(general, buf);
    __syncthreads();
    buf ^= 1;
  }
  if (!q_ok) return;
  if constexpr (kCKV == CSA_FP8_E4M3) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[ht][dt] *= vref;
  }
  if (kPacked && piece >= 0) {
    // the piece's partial state (max in the log2 domain, sum, unnormalised
    // output), in attn_merge_kernel's layout: partial row b * kQB + i, split
    // `piece` (an empty piece writes max -inf, sum 0, output 0)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float L = column_sum(l_run[ht]);
      const int head = ((wid % kWPQ) * 2 + ht) * 16 + col;
      const long slot = ((long(b) * kQB + i) * a.n_pieces + piece) * a.H + head;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<v4f*>(a.part_o + slot * kHeadDim + (dt * 4 + g) * 4) = o[ht][dt];
      if (g == 0) {
        a.part_ml[slot * 2] = m_run[ht];
        a.part_ml[slot * 2 + 1] = L;
      }
    }
    return;
  }
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const float L = column_sum(l_run[ht]);
    const int head = ((wid % kWPQ) * 2 + ht) * 16 + col;
    const long orow = (row_base + i) * a.H + head;
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_out4<CSA_BF16>(a.out, orow, dt * 4 + g, o[ht][dt] * inv);
    if (a.lse && g == 0) a.lse[orow] = L > 0.f ? m_run[ht] * kLn2 + logf(L) : -INFINITY;
  }
}

// ------------------------------------------------------------------ host --
struct Plan {
  int n_splits, split_len;
  long blocks;
  bool invariant;   // pieces folded in order (batch-invariant calls)
  bool fold;        // ... inside one block per row (no partials)
};

// Batch-invariant calls with at least this many rows walk each row's pieces
// inside one block; fewer rows run the pieces as blocks of their own and
// attn_fold_kernel folds their partials.  Both give the same bits.
constexpr long kFoldRows = 128;

// The default work split depends only on (rows, n_list): never on data or timing.
// At most about one block per CU: past 256 blocks some CUs run two, whose
// tail then sets the kernel time, and the partials to write back and merge
// grow with the split count.  A split is a whole number of 64-key chunks.
// invariant: the split length depends on the key-list length only (at least
// two chunks per split, at most kMaxSplits splits), so a row's splits, and
// with them its result bits, are the same whatever the batch around it.
Plan make_plan(long rows, int n_list, bool invariant) {
  Plan p{};
  const long chunks = (max(n_list, 1) + kNK - 1) / kNK;
  if (invariant) {
    // pieces of max(8, ceil(chunks / 64)) chunks: a function of the list
    // length alone
    const long per = max(8L, (chunks + kMaxSplits - 1) / kMaxSplits);
    p.split_len = int(per * kNK);
    p.n_splits = int((chunks + per - 1) / per);
    p.invariant = true;
    p.fold = p.n_splits > 1 && rows >= kFoldRows;
    p.blocks = p.fold ? rows : rows * p.n_splits;
    return p;
  }
  long want = (256 + rows - 1) / rows;
  if (want > chunks) want = chunks;
  if (want > kMaxSplits) want = kMaxSplits;
  if (want < 1) want = 1;
  const long per = (chunks + want - 1) / want;
  p.split_len = int(per * kNK);
  p.n_splits = int((chunks + per - 1) / per);
  p.blocks = rows * p.n_splits;
  return p;
}

// Decode plan (few rows, bf16 queries): (splits S, split length, head groups G)
// for attn_decode_kernel.  A split holds at most kDecChunks chunks; the chip
// holds 256 blocks per round (fewer LDS bytes per block: more).  Among G in
// {1, 2, 4} (16-head tiles per block <= 4) the plan with the least estimated
// time wins: the unique rows over HBM (~6.5 TB/s), a block's rows at a CU's
// rate when its head groups share them through L2 (~95 GB/s; measured), and
// the partial outputs written and read back by the merge (~5 TB/s each way).
// The estimate depends on the shape only (rows, keys, heads), never on data.
struct DecodePlan {
  int n_splits = 0, split_len = 0, groups = 0, kT = 0, chunks = 0;
  long units = 0, blocks = 0;
  size_t lds = 0;
};

constexpr long kDecodeMaxRows = 64;

size_t decode_lds_bytes(int chunks) {
  const size_t c = size_t(chunks) * sizeof(LdsBf16);
  return c > sizeof(DecFold) ? c : sizeof(DecFold);
}

DecodePlan make_decode_plan(long rows, int n_list, int H) {
  DecodePlan best{};
  double best_t = 1e30;
  const int tiles = H / 16;
  const long max_len = long(kDecChunks) * kNK;
  const double row_bytes = 512.0;   // bf16 K + V rows (fp8 entries move half: the choice is the same)
  for (int G = 4; G >= 1; G >>= 1) {
    if (tiles % G || tiles / G > 4) continue;
    long S = max((256 + rows * G - 1) / (rows * G), (long(n_list) + max_len - 1) / max_len);
    long len = (n_list + S - 1) / S;
    len = (len + 31) / 32 * 32;
    S = (n_list + len - 1) / len;
    const int chunks = int((len + kNK - 1) / kNK);
    const size_t lds = decode_lds_bytes(chunks);
    const long per_cu = max(1L, long((160 * 1024) / lds));
    const long units = rows * S;
    const long blocks = (units + 7) / 8 * 8 * G;
    const double rounds = double((blocks + 256 * per_cu - 1) / (256 * per_cu));
    const double t_read = max(double(rows) * n_list * row_bytes / 6.5e6, double(len) * row_bytes / 95e3);
    const double partial = S > 1 ? double(rows) * S * H * (kHeadDim + 2) * 4 : 0.0;
    const double t = rounds * t_read + 2.0 * partial / 5e6 + (S > 1 ? 1.65 : 0.0);
    if (t < best_t) {
      best_t = t;
      best.n_splits = int(S);
      best.split_len = int(len);
      best.groups = G;
      best.kT = tiles / G;
      best.chunks = chunks;
      best.units = units;
      best.blocks = blocks;
      best.lds = lds;
    }
  }
  return best;
}

bool use_decode(int io_dtype, long rows, bool invariant) {
  return !invariant && io_dtype == CSA_BF16 && rows <= kDecodeMaxRows;
}

size_t plan_ws_bytes(const Plan& p, long rows, int H) {
  if (p.n_splits <= 1 || p.fold) return 0;
  const size_t slots = size_t(rows) * p.n_splits * H;
  const size_t ml = ((slots * 2 * 4 + 255) / 256) * 256;
  return ml + slots * kHeadDim * 4;
}

template <int kIO, int kCKV, bool kDense, int kHTW, int kDepth, bool kVarlen, bool kFold>
hipError_t launch_attn(const AttnArgs& a, const Plan& p, hipStream_t st) {
  constexpr size_t bytes = lds_bytes<kIO, kHTW>() + (kFold ? sizeof(LdsFold<kHTW>) : 0);
  auto fn = attn_kernel<kIO, kCKV, kDense, kHTW, kDepth, kVarlen, kFold>;
  if (hipError_t e = csa_lds_opt_in(reinterpret_cast<const void*>(fn), bytes); e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(unsigned(p.blocks)), dim3(kThreads), bytes, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1 || kFold) return e;
  const long heads = p.blocks / a.n_splits * a.H;
  if (p.invariant)
    hipLaunchKernelGGL(attn_fold_kernel<kIO>, dim3(unsigned(heads)), dim3(64), 0, st, a.part_ml, a.part_o, a.n_splits,
                       a.H, a.out, a.lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<kIO>, dim3(unsigned(heads)), dim3(64), 0, st, a.part_ml, a.part_o,
                       a.n_splits, a.H, a.out, a.lse, nullptr, 0);
  return hipGetLastError();
}

// B sequences of T_q rows; or, for a packed varlen call (a.cu_rows), B =
// n_rows: a bound on the tiles plus the pieces, then the merge of the pieces.
template <int kCKV, int kQB>
hipError_t launch_mq_q(const AttnArgs& a, long B, hipStream_t st) {
  constexpr size_t bytes = sizeof(LdsMQ);
  if (!a.cu_rows) {
    if (hipError_t e = csa_lds_opt_in(reinterpret_cast<const void*>(&attn_mq_kernel<kCKV, kQB, false>), bytes);
        e != hipSuccess)
      return e;
    const long blocks = B * ((a.T_q + kQB - 1) / kQB);
    hipLaunchKernelGGL((attn_mq_kernel<kCKV, kQB, false>), dim3(unsigned(blocks)), dim3(kThreads), bytes, st, a);
    return hipGetLastError();
  }
  if (hipError_t e = csa_lds_opt_in(reinterpret_cast<const void*>(&attn_mq_kernel<kCKV, kQB, true>), bytes);
      e != hipSuccess)
    return e;
  const long blocks = long(a.n_seq) * a.n_pieces + (B + kQB - 1) / kQB + a.n_seq;
  hipLaunchKernelGGL((attn_mq_kernel<kCKV, kQB, true>), dim3(unsigned(blocks)), dim3(kThreads), bytes, st, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const long heads = long(a.n_seq) * kQB * a.H;
  hipLaunchKernelGGL(attn_merge_kernel<CSA_BF16>, dim3(unsigned(heads)), dim3(64), 0, st, a.part_ml, a.part_o,
                     a.n_pieces, a.H, a.out, a.lse, a.cu_rows, kQB);
  return hipGetLastError();
}

template <int kCKV>
hipError_t launch_mq(const AttnArgs& a, long B, hipStream_t st) {
  switch (a.H) {
    case 32: return launch_mq_q<kCKV, 8>(a, B, st);
    case 64: return launch_mq_q<kCKV, 4>(a, B, st);
    default: return launch_mq_q<kCKV, 2>(a, B, st);
  }
}

// Pieces of the varlen many-query launch: a sequence of at most kQB rows has
// its union list (at most n_list + kQB - 1 slots) cut into n_pieces pieces of
// piece_len slots (whole chunks, about kPieceChunks each, at most 64 pieces:
// the merge kernel's limit).
constexpr int kPieceChunks = 4;
struct MQPieces {
  int kqb, n_pieces, piece_len;
};
MQPieces mq_pieces(int H, int n_list) {
  MQPieces m{};
  m.kqb = H == 32 ? 8 : H == 64 ? 4 : 2;
  const long chunks = (long(n_list) + m.kqb - 1 + kNK - 1) / kNK;
  long S = (chunks + kPieceChunks - 1) / kPieceChunks;
  S = S < 1 ? 1 : S > 64 ? 64 : S;
  const long per = (chunks + S - 1) / S;
  m.n_pieces = int((chunks + per - 1) / per);
  m.piece_len = int(per * kNK);
  return m;
}
size_t mq_pieces_ws_bytes(int n_seq, int H, int n_list) {
  const MQPieces m = mq_pieces(H, n_list);
  const size_t slots = size_t(n_seq) * m.kqb * m.n_pieces * H;
  return ((slots * 2 * 4 + 255) / 256) * 256 + slots * kHeadDim * 4;
}

// The plain varlen dense call takes the many-query kernel (with pieces for
// short sequences) for bf16 queries over bf16 / fp8 entries once the call has
// enough rows to fill the chip.
bool use_mq_varlen(int io_dtype, int ckv_dtype, int H, long n_rows) {
  return io_dtype == CSA_BF16 && (ckv_dtype == CSA_BF16 || ckv_dtype == CSA_FP8_E4M3) &&
         (H == 32 || H == 64 || H == 128) && n_rows >= 256;
}

// The many-query dense kernel serves bf16 queries with H in {32, 64, 128}
// when a sequence has enough queries to fill its blocks and the key lists
// need no split.
bool use_mq(int io_dtype, int H, int T_q, const Plan& p) {
  return io_dtype == CSA_BF16 && (H == 32 || H == 64 || H == 128) && T_q >= 64 && p.n_splits == 1;
}

template <int kIO, int kCKV, bool kDense, bool kVarlen>
hipError_t launch_tiles(const AttnArgs& a, const Plan& p, hipStream_t st) {
  // one block per row walking every piece (batch-invariant, many rows)
  if (p.fold)
    return a.H <= 64 ? launch_attn<kIO, kCKV, kDense, 1, 1, kVarlen, true>(a, p, st)
                     : launch_attn<kIO, kCKV, kDense, 2, 1, kVarlen, true>(a, p, st);
  // split key lists of more than two chunks take the two-chunk pipeline
  // (fp32 queries over more than 64 heads would not fit its registers); with
  // two chunks the one-ahead prefetch already overlaps the second, and more
  // chunks in flight only delay the first (a CU's loads in flight are few)
  if (a.n_splits > 1 && a.split_len > 2 * kNK) {
    if (a.H <= 64) return launch_attn<kIO, kCKV, kDense, 1, 2, kVarlen, false>(a, p, st);
    if constexpr (kIO == CSA_BF16) return launch_attn<kIO, kCKV, kDense, 2, 2, kVarlen, false>(a, p, st);
  }
  return a.H <= 64 ? launch_attn<kIO, kCKV, kDense, 1, 1, kVarlen, false>(a, p, st)
                   : launch_attn<kIO, kCKV, kDense, 2, 1, kVarlen, false>(a, p, st);
}

template <bool kDense, bool kVarlen>
csa_status_t tiles_for(const AttnArgs& a, int io_dtype, int ckv_dtype, const Plan& p, hipStream_t st) {
  hipError_t err;
  if (io_dtype == CSA_BF16 && ckv_dtype == CSA_BF16) err = launch_tiles<CSA_BF16, CSA_BF16, kDense, kVarlen>(a, p, st);
  else if (io_dtype == CSA_BF16 && ckv_dtype == CSA_FP8_E4M3) err = launch_tiles<CSA_BF16, CSA_FP8_E4M3, kDense, kVarlen>(a, p, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_F32) err = launch_tiles<CSA_F32, CSA_F32, kDense, kVarlen>(a, p, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_FP8_E4M3) err = launch_tiles<CSA_F32, CSA_FP8_E4M3, kDense, kVarlen>(a, p, st);
  else return CSA_ENOTSUP;
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}

template <int kCKV, bool kDense, bool kVarlen>
hipError_t launch_decode(const AttnArgs& a, const DecodePlan& d, hipStream_t st) {
  auto fn = attn_decode_kernel<kCKV, kDense, kVarlen>;
  if (hipError_t e = csa_lds_opt_in(reinterpret_cast<const void*>(fn), d.lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(unsigned(d.blocks)), dim3(kThreads), d.lds, st, a, d.kT, d.groups, d.units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  const long heads = d.units / a.n_splits * a.H;
  hipLaunchKernelGGL(attn_merge_kernel<CSA_BF16>, dim3(unsigned(heads)), dim3(64), 0, st, a.part_ml, a.part_o,
                     a.n_splits, a.H, a.out, a.lse, nullptr, 0);
  return hipGetLastError();
}

// Decode rows: bf16 queries over bf16 or fp8 entries.
template <bool kDense>
csa_status_t run_decode(AttnArgs a, int ckv_dtype, long rows, void* ws, size_t ws_size, hipStream_t st) {
  const DecodePlan d = make_decode_plan(rows, a.n_list, a.H);
  a.n_splits = d.n_splits;
  a.split_len = d.split_len;
  Plan p{};
  p.n_splits = d.n_splits;
  const size_t need = plan_ws_bytes(p, rows, a.H);
  if (need > 0) {
    if (!ws || ws_size < need) return CSA_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    const size_t slots = size_t(rows) * d.n_splits * a.H;
    const size_t ml = ((slots * 2 * 4 + 255) / 256) * 256;
    a.part_ml = reinterpret_cast<float*>(w);
    a.part_o = reinterpret_cast<float*>(w + ml);
  }
  hipError_t err;
  if (ckv_dtype == CSA_FP8_E4M3)
    err = a.cu_rows ? launch_decode<CSA_FP8_E4M3, kDense, true>(a, d, st) : launch_decode<CSA_FP8_E4M3, kDense, false>(a, d, st);
  else if (ckv_dtype == CSA_BF16)
    err = a.cu_rows ? launch_decode<CSA_BF16, kDense, true>(a, d, st) : launch_decode<CSA_BF16, kDense, false>(a, d, st);
  else
    return CSA_ENOTSUP;
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}

template <bool kDense>
csa_status_t run_attn(AttnArgs a, int io_dtype, int ckv_dtype, int B, void* ws, size_t ws_size, hipStream_t st,
                      bool invariant) {
  const long rows = long(B) * a.T_q;
  if (rows == 0) return CSA_OK;
  if (use_decode(io_dtype, rows, invariant)) return run_decode<kDense>(a, ckv_dtype, rows, ws, ws_size, st);
  const Plan p = make_plan(rows, a.n_list, invariant);
  if (p.blocks > 0x7FFFFFFFL) return CSA_ENOTSUP;
  a.n_splits = p.n_splits;
  a.split_len = p.split_len;
  const size_t need = plan_ws_bytes(p, rows, a.H);
  if (need > 0) {
    if (!ws || ws_size < need) return CSA_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    const size_t slots = size_t(rows) * p.n_splits * a.H;
    const size_t ml = ((slots * 2 * 4 + 255) / 256) * 256;
    a.part_ml = reinterpret_cast<float*>(w);
    a.part_o = reinterpret_cast<float*>(w + ml);
  }
  hipError_t err;
  if (kDense && !invariant && use_mq(io_dtype, a.H, a.T_q, p) &&
      (ckv_dtype == CSA_BF16 || ckv_dtype == CSA_FP8_E4M3)) {
    err = ckv_dtype == CSA_BF16 ? launch_mq<CSA_BF16>(a, B, st) : launch_mq<CSA_FP8_E4M3>(a, B, st);
    return err == hipSuccess ? CSA_OK : CSA_EHIP;
  }
  return a.cu_rows ? tiles_for<kDense, true>(a, io_dtype, ckv_dtype, p, st)
                   : tiles_for<kDense, false>(a, io_dtype, ckv_dtype, p, st);
}

csa_status_t check_common(const void* q, int io_dtype, const void* ck, const void* cv, const float* ck_scale,
                          const float* cv_scale, int ckv_dtype, int cap, const void* k_win, const void* v_win,
                          const int32_t* raw_pos0, int L_raw, const int32_t* q_pos0, int W, int B, int T_q, int H,
                          int d, void* out) {
  if (!q || !ck || !cv || !q_pos0 || !out) return CSA_EINVAL;
  if (io_dtype != CSA_BF16 && io_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(ckv_dtype)) return CSA_EINVAL;
  if (ckv_dtype == CSA_FP8_E4M3 && (!ck_scale || !cv_scale)) return CSA_EINVAL;
  if (d != kHeadDim) return CSA_EINVAL;
  // supported pairs: bf16 queries over bf16 or fp8 entries; fp32 over fp32 or fp8
  if (ckv_dtype != CSA_FP8_E4M3 && ckv_dtype != io_dtype) return CSA_ENOTSUP;
  if (B < 0 || T_q < 0 || cap < 0 || W < 0 || L_raw < 0) return CSA_EINVAL;
  if (H < 16 || H > 128 || H % 16 != 0) return CSA_ENOTSUP;
  if (W > 0 && (!k_win || !v_win || !raw_pos0 || L_raw < 1)) return CSA_EINVAL;
  if (B > 0 && T_q > 0x7FFFFFFF / B) return CSA_ENOTSUP;
  return CSA_OK;
}

}  // namespace

// Workspace for either kernel family (the queries' type picks one; the size
// covers both).
size_t csa_attn_workspace_size(long rows, int H, int n_list, bool invariant) {
  size_t need = plan_ws_bytes(make_plan(rows, n_list, invariant), rows, H);
  if (use_decode(CSA_BF16, rows, invariant) && rows > 0) {
    Plan p{};
    p.n_splits = make_decode_plan(rows, n_list, H).n_splits;
    need = max(need, plan_ws_bytes(p, rows, H));
  }
  return need;
}

namespace {

csa_status_t sparse_attn_impl(const void* q, int32_t io_dtype, const void* ck, const void* cv, const float* ck_scale,
                              const float* cv_scale, int32_t ckv_dtype, int32_t cap, const int32_t* idx, int32_t k,
                              const void* k_win, const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                              const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q, int32_t H, int32_t d,
                              float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream,
                              bool invariant) {
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, B, T_q, H, d, out);
  if (c != CSA_OK) return c;
  if (!idx || k < 1) return CSA_EINVAL;
  if (long(k) + W > 0x7FFFFFFFL - kNK) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = idx; a.k = k; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.T_q = T_q; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = k + W;
  return run_attn<false>(a, io_dtype, ckv_dtype, B, ws, ws_bytes, static_cast<hipStream_t>(stream), invariant);
}

csa_status_t dense_attn_impl(const void* q, int32_t io_dtype, const void* ck, const void* cv, const float* ck_scale,
                             const float* cv_scale, int32_t ckv_dtype, int32_t cap, int32_t m_prime,
                             const void* k_win, const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                             const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q, int32_t H, int32_t d,
                             float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream,
                             bool invariant) {
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, B, T_q, H, d, out);
  if (c != CSA_OK) return c;
  if (m_prime < 1) return CSA_EINVAL;
  if (long(cap) + W > 0x7FFFFFFFL - kNK) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = nullptr; a.k = m_prime; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.T_q = T_q; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = cap + W;
  return run_attn<true>(a, io_dtype, ckv_dtype, B, ws, ws_bytes, static_cast<hipStream_t>(stream), invariant);
}

// Varlen: n_rows packed query rows of B sequences (decode rows and prefill
// chunks together).  invariant: the batch-invariant plan, so each row's bits
// equal those of the *_batch_invariant calls on its own sequence; otherwise
// the plain calls' kernels, chosen for the call as a whole.
csa_status_t varlen_attn(AttnArgs a, bool dense, int io_dtype, int ckv_dtype, const int32_t* cu_rows, int n_rows,
                         int B, bool invariant, void* ws, size_t ws_bytes, hipStream_t st) {
  if (n_rows == 0) return CSA_OK;
  if (!cu_rows || B < 1) return CSA_EINVAL;
  a.cu_rows = cu_rows;
  a.n_seq = B;
  a.T_q = 1;
  if (dense && !invariant && use_mq_varlen(io_dtype, ckv_dtype, a.H, n_rows)) {
    const MQPieces m = mq_pieces(a.H, a.n_list);
    const size_t need = mq_pieces_ws_bytes(B, a.H, a.n_list);
    if (!ws || ws_bytes < need) return CSA_EWORKSPACE;
    const size_t slots = size_t(B) * m.kqb * m.n_pieces * a.H;
    a.part_ml = static_cast<float*>(ws);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + ((slots * 2 * 4 + 255) / 256) * 256);
    a.n_pieces = m.n_pieces;
    a.piece_len = m.piece_len;
    const long blocks = long(B) * m.n_pieces + (n_rows + m.kqb - 1) / m.kqb + B;
    if (blocks > 0x7FFFFFFFL || long(B) * m.kqb * a.H > 0x7FFFFFFFL) return CSA_ENOTSUP;
    const hipError_t err = ckv_dtype == CSA_BF16 ? launch_mq<CSA_BF16>(a, n_rows, st)
                                                 : launch_mq<CSA_FP8_E4M3>(a, n_rows, st);
    return err == hipSuccess ? CSA_OK : CSA_EHIP;
  }
  return dense ? run_attn<true>(a, io_dtype, ckv_dtype, n_rows, ws, ws_bytes, st, invariant)
               : run_attn<false>(a, io_dtype, ckv_dtype, n_rows, ws, ws_bytes, st, invariant);
}

}  // namespace

// Workspace of a varlen call in either mode (n_list = k + W or cap + W).
size_t csa_attn_varlen_workspace_size(long n_rows, int n_seq, int H, int n_list, bool dense) {
  size_t need = max(csa_attn_workspace_size(n_rows, H, n_list, true), csa_attn_workspace_size(n_rows, H, n_list, false));
  if (dense && n_rows > 0) need = max(need, mq_pieces_ws_bytes(n_seq, H, n_list));
  return need;
}

extern "C" csa_status_t csa_sparse_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                               const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                               int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                                               const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                                               const int32_t* cu_rows, const int32_t* q_pos0, int32_t n_rows,
                                               int32_t W, int32_t B, int32_t H, int32_t d, float sm_scale,
                                               int32_t invariant, void* out, float* lse, void* ws, size_t ws_bytes,
                                               void* stream) {
  if (n_rows < 0 || B < 0) return CSA_EINVAL;
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, n_rows, 1, H, d, out);
  if (c != CSA_OK) return c;
  if (!idx || k < 1) return CSA_EINVAL;
  if (long(k) + W > 0x7FFFFFFFL - kNK) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = idx; a.k = k; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = k + W;
  return varlen_attn(a, false, io_dtype, ckv_dtype, cu_rows, n_rows, B, invariant != 0, ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

extern "C" csa_status_t hca_dense_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                              const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                              int32_t cap, int32_t m_prime, const void* k_win, const void* v_win,
                                              const int32_t* raw_pos0, int32_t L_raw, const int32_t* cu_rows,
                                              const int32_t* q_pos0, int32_t n_rows, int32_t W, int32_t B, int32_t H,
                                              int32_t d, float sm_scale, int32_t invariant, void* out, float* lse,
                                              void* ws, size_t ws_bytes, void* stream) {
  if (n_rows < 0 || B < 0) return CSA_EINVAL;
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, n_rows, 1, H, d, out);
  if (c != CSA_OK) return c;
  if (m_prime < 1) return CSA_EINVAL;
  if (long(cap) + W > 0x7FFFFFFFL - kNK) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = nullptr; a.k = m_prime; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = cap + W;
  return varlen_attn(a, true, io_dtype, ckv_dtype, cu_rows, n_rows, B, invariant != 0, ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

#define CSA_SPARSE_ARGS                                                                                          \
  const void *q, int32_t io_dtype, const void *ck, const void *cv, const float *ck_scale, const float *cv_scale, \
      int32_t ckv_dtype, int32_t cap, const int32_t *idx, int32_t k, const void *k_win, const void *v_win,      \
      const int32_t *raw_pos0, int32_t L_raw, const int32_t *q_pos0, int32_t W, int32_t B, int32_t T_q,         \
      int32_t H, int32_t d, float sm_scale, void *out, float *lse, void *ws, size_t ws_bytes, void *stream
#define CSA_SPARSE_PASS                                                                                     \
  q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, idx, k, k_win, v_win, raw_pos0, L_raw, q_pos0, W, \
      B, T_q, H, d, sm_scale, out, lse, ws, ws_bytes, stream
#define CSA_DENSE_ARGS                                                                                           \
  const void *q, int32_t io_dtype, const void *ck, const void *cv, const float *ck_scale, const float *cv_scale, \
      int32_t ckv_dtype, int32_t cap, int32_t m_prime, const void *k_win, const void *v_win,                    \
      const int32_t *raw_pos0, int32_t L_raw, const int32_t *q_pos0, int32_t W, int32_t B, int32_t T_q,         \
      int32_t H, int32_t d, float sm_scale, void *out, float *lse, void *ws, size_t ws_bytes, void *stream
#define CSA_DENSE_PASS                                                                                    \
  q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, m_prime, k_win, v_win, raw_pos0, L_raw, q_pos0, \
      W, B, T_q, H, d, sm_scale, out, lse, ws, ws_bytes, stream

extern "C" csa_status_t csa_sparse_attn(CSA_SPARSE_ARGS) { return sparse_attn_impl(CSA_SPARSE_PASS, false); }
extern "C" csa_status_t csa_sparse_attn_batch_invariant(CSA_SPARSE_ARGS) {
  return sparse_attn_impl(CSA_SPARSE_PASS, true);
}
extern "C" csa_status_t hca_dense_attn(CSA_DENSE_ARGS) { return dense_attn_impl(CSA_DENSE_PASS, false); }
extern "C" csa_status_t hca_dense_attn_batch_invariant(CSA_DENSE_ARGS) {
  return dense_attn_impl(CSA_DENSE_PASS, true);
}

// ------------------------------------------------ allocation-free entry --
// csa_sparse_attn_noalloc keeps the split partials in a fixed device array
// instead of a caller workspace, for callers that cannot allocate.  Each GPU
// holds its own copy of the array until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (set up on its first use).
csa_status_t scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CSA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return CSA_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" csa_status_t csa_sparse_attn_noalloc(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                                const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                                int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                                                const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                                                const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q, int32_t H,
                                                int32_t d, float sm_scale, void* out, float* lse, void* stream) {
  // the same argument checks as csa_sparse_attn come first, then the size check
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, B, T_q, H, d, out);
  if (c != CSA_OK) return c;
  if (!idx || k < 1) return CSA_EINVAL;
  if (long(k) + W > 0x7FFFFFFFL - kNK) return CSA_ENOTSUP;
  if (csa_attn_workspace_size(long(B) * T_q, H, k + W, false) > kScratchBytes) return CSA_ESCRATCH;
  void* ws = nullptr;
  c = scratch_of_current_device(&ws);
  if (c != CSA_OK) return c;
  return sparse_attn_impl(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, idx, k, k_win, v_win, raw_pos0,
                          L_raw, q_pos0, W, B, T_q, H, d, sm_scale, out, lse, ws, kScratchBytes, stream, false);
}
