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
// multiplies the logits and the V scale is folded into P.  The fp32 variant
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
#include "common.hpp"

namespace {

constexpr int kNK = 64;                       // keys per chunk
constexpr int kThreads = 512;                 // 8 waves
constexpr int kKRow = kHeadDim + 8;           // bf16 per K row in LDS
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
  const int32_t* row_seq;  // varlen: sequence of each query row (else null: row / T_q)
  const int32_t* row_pos;  // varlen: position of each query row
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
  float sm_log2;           // sm_scale * log2(e)
};

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

// LDS layout of one chunk
struct LdsBf16 {
  uint16_t K[kNK][kKRow];
  // V^T, head dim x key: rows of 40 words, 4 words of pad after every 8 rows.
  // A wave's writes (16 row groups x 4 key pairs) then fall in distinct
  // banks and the 8-byte reads of the P*V products take two passes.
  uint16_t Vt[kHeadDim / 8][kVGroup];
  float sk[kNK];
  float sv[kNK];
  int valid[kNK];
};
struct LdsF32 {
  float K[kNK][kFRow];
  float V[kNK][kFRow];
  float sk[kNK];
  float sv[kNK];
  int valid[kNK];
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

template <int kIO, int kHTW>
constexpr size_t lds_bytes() {
  return sizeof(LdsChunk<kIO>) > sizeof(LdsHalf<kHTW>) ? sizeof(LdsChunk<kIO>) : sizeof(LdsHalf<kHTW>);
}

// 8 head dims of a gathered part as four bf16 pairs (src 0 -> zeros).  E4M3
// codes go through the CDNA4 fp8 -> bf16 conversion, which is exact (every
// E4M3 value is a bf16 value); the per-entry scale is applied elsewhere.
template <int kCKV>
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
    for (int q = 0; q < 4; ++q) r[q] = src == 1 ? cv[q] : r[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = src == 0 ? 0u : r[q];
  return r;
}

// sk_mul: factor folded into the stored K scale (the logit scale in the log2 domain).
template <int kIO, int kCKV>
CSA_DEV void store_chunk(LdsChunk<kIO>& s, const Pre<kIO>& pr, float sk_mul) {
  const int kp = item_kp();
  const int dg = item_dg();
  if constexpr (kIO == CSA_BF16) {
    // values are exact in bf16 (bf16 inputs or E4M3 codes)
    u32x4 kw[2], vw[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kw[e] = part_bf16<kCKV>(pr.k[e], pr.src[e], dg & 1);
      vw[e] = part_bf16<kCKV>(pr.v[e], pr.src[e], dg & 1);
      *reinterpret_cast<u32x4*>(&s.K[2 * kp + e][dg * 8]) = kw[e];
    }
    // V^T: head dim x of keys 2kp and 2kp+1 as one bf16 pair
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      uint16_t* vt = &s.Vt[dg][2 * x * kVRow + 2 * kp];   // rows 8 dg + 2x and 8 dg + 2x + 1
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
      const bool scaled = kCKV == CSA_FP8_E4M3 && pr.src[e] == 1;
      s.sk[2 * kp + e] = (scaled ? pr.sk[e] : 1.f) * sk_mul;
      s.sv[2 * kp + e] = scaled ? pr.sv[e] : 1.f;
      s.valid[2 * kp + e] = pr.src[e] != 0;
    }
  }
}

// S^T for one 16-key tile `kt` of the chunk, scaled to the log2 domain and masked.
template <int kIO>
CSA_DEV void logits_tile(const LdsChunk<kIO>& s, const u32x4* qb, const float* qf, int kt, int col, int g, float* x) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kIO == CSA_BF16) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma_k32(*reinterpret_cast<const u32x4*>(&s.K[kt * 16 + col][ks * 32 + g * 8]), qb[ks], acc);
  } else {
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) acc = mfma_f32(s.K[kt * 16 + col][ks * 4 + g], qf[ks], acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kk = kt * 16 + 4 * g + r;
    x[r] = s.valid[kk] ? acc[r] * s.sk[kk] : -INFINITY;
  }
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

// 8 waves: wave w takes head tiles (w % 4) [+ 4 when kHTW == 2] and key half
// w / 4 (keys [32*(w/4), 32*(w/4)+32) of every chunk); the two halves merge at
// the end of the block through LDS.
// kDepth > 1 (split key lists, at most about one block per CU): that many
// chunks in flight instead of one, with the register budget of two waves per
// SIMD.
// kVarlen: query rows are mapped through row_seq / row_pos (the varlen calls).
template <int kIO, int kCKV, bool kDense, int kHTW, int kDepth, bool kVarlen>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kIO == CSA_BF16 && kHTW == 1 ? (kDepth > 1 ? 2 : 4) : 1)))
void attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsChunk<kIO>& s = *reinterpret_cast<LdsChunk<kIO>*>(smem);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int kh = wid >> 2;
  const int wt = wid & 3;

  const long qrow = blockIdx.x / a.n_splits;
  const int split = int(blockIdx.x - qrow * a.n_splits);
  int b, t;
  if constexpr (kVarlen) {
    b = a.row_seq[qrow];
    t = a.row_pos[qrow];
  } else {
    b = int(qrow / a.T_q);
    t = a.q_pos0[b] + int(qrow - long(b) * a.T_q);
  }
  const int raw0 = a.W > 0 ? a.raw_pos0[b] : 0;
  const int n_tiles = a.H / 16;
  const int j_begin = split * a.split_len;
  const int j_end = min(j_begin + a.split_len, a.n_list);

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
        uint32_t pw[4];
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          const int kk = h2 >> 1;
          const int r0 = (h2 & 1) * 2;
          const int key = (2 * kh + kk) * 16 + 4 * g + r0;
          pw[h2] = pack_bf16x2(p[kk][r0] * s.sv[key], p[kk][r0 + 1] * s.sv[key + 1]);
        }
        const u32x4 pb = {pw[0], pw[1], pw[2], pw[3]};
        const int k0 = kh * 32 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint16_t* vt = &s.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0];   // row dt*16 + col
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vt);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + 16);
          o[ht][dt] = mfma_k32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[ht][dt]);
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
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_idx<kDense>(a, e_nx[d], qrow, j_begin + d * kNK, j_end);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    prefetch<kIO, kCKV, kDense>(a, pr[d], e_nx[d], b, t, raw0, j_begin + d * kNK, j_end);
    load_idx<kDense>(a, e_nx[d], qrow, j_begin + (d + kDepth) * kNK, j_end);
  }
  for (int j0 = j_begin; j0 < j_end; j0 += kDepth * kNK) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (d > 0 && j0 + d * kNK >= j_end) break;
      __syncthreads();
      store_chunk<kIO, kCKV>(s, pr[d], a.sm_log2);
      __syncthreads();
      prefetch<kIO, kCKV, kDense>(a, pr[d], e_nx[d], b, t, raw0, j0 + (d + kDepth) * kNK, j_end);
      load_idx<kDense>(a, e_nx[d], qrow, j0 + (d + 2 * kDepth) * kNK, j_end);
      compute();
    }
  }

  float l_tot[kHTW];
#pragma unroll
  for (int ht = 0; ht < kHTW; ++ht) {
    l_tot[ht] = column_sum(l_run[ht]);
  }
  // hand the second key half to the first
  LdsHalf<kHTW>& hf = *reinterpret_cast<LdsHalf<kHTW>*>(smem);
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
  if (kh == 1) return;
#pragma unroll
  for (int ht = 0; ht < kHTW; ++ht) {
    if (!act[ht]) continue;
    const int tile = wt + 4 * ht;
    const int head = tile * 16 + col;
    const float m1 = hf.m[tile][col];
    const float M = fmaxf(m_run[ht], m1);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float f0 = __builtin_amdgcn_exp2f(m_run[ht] - Mu);
    const float f1 = __builtin_amdgcn_exp2f(m1 - Mu);
    const float L = l_tot[ht] * f0 + hf.l[tile][col] * f1;
    v4f oo[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      oo[dt] = o[ht][dt] * f0 + *reinterpret_cast<const v4f*>(&hf.o[tile][col][dt * 16 + 4 * g]) * f1;
    if (a.n_splits == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const long orow = qrow * a.H + head;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) store_out4<kIO>(a.out, orow, dt * 4 + g, oo[dt] * inv);
      if (a.lse && g == 0) a.lse[orow] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
    } else {
      // this split's unnormalised state; the merge kernel combines the splits
      // (streaming stores: the partials are read once, by another kernel)
      const long slot = (qrow * a.n_splits + split) * a.H + head;
      float* po = a.part_o + slot * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) __builtin_nontemporal_store(oo[dt], reinterpret_cast<v4f*>(po + dt * 16 + 4 * g));
      if (g == 0) {
        __builtin_nontemporal_store(M, &a.part_ml[slot * 2]);
        __builtin_nontemporal_store(L, &a.part_ml[slot * 2 + 1]);
      }
    }
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
                                                        void* out, float* lse) {
  __shared__ float wsh[64];
  const long hid = blockIdx.x;                  // query row * H + head
  const int lane = threadIdx.x;
  const long qrow = hid / H;
  const int head = int(hid - qrow * H);
  const long base = qrow * n_splits * H + head; // slot of split 0; split x adds x*H
  const int half = lane >> 5;
  const int d4 = lane & 31;
  constexpr int kU = 8;
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
    store_out4<kIO>(out, hid, d4, acc * inv);
    if (lse && d4 == 0) lse[hid] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
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
  LdsBf16 c;
  uint32_t vis[kNK];   // bit q: the key is visible to the block's query q
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

template <int kCKV, int kQB>
__global__ __launch_bounds__(kThreads) void attn_mq_kernel(AttnArgs a) {
  static_assert(kQB == 2 || kQB == 4 || kQB == 8, "two 16-head tiles per wave");
  constexpr int kWPQ = 8 / kQB;   // waves per query; each takes two 16-head tiles
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsMQ& s = *reinterpret_cast<LdsMQ*>(smem);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int blocks_per_seq = (a.T_q + kQB - 1) / kQB;
  const int b = int(blockIdx.x / blocks_per_seq);
  const int i0 = int(blockIdx.x - long(b) * blocks_per_seq) * kQB;
  const int qi = wid / kWPQ;
  const int i = i0 + qi;
  const bool q_ok = i < a.T_q;
  const int pos0 = a.q_pos0[b];
  const int raw0 = a.W > 0 ? a.raw_pos0[b] : 0;
  const int i_last = min(i0 + kQB, a.T_q) - 1;
  const int nv_max = min((pos0 + i_last + 1) / a.k, a.cap);
  const int p_lo = pos0 + i0 - a.W + 1;
  const int n_win = a.W > 0 ? a.W + (i_last - i0) : 0;
  const int n_list = nv_max + n_win;
  const int t0 = pos0 + i0;
  const int n_q = i_last - i0 + 1;

  u32x4 qb[2][4];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = ((wid % kWPQ) * 2 + ht) * 16 + col;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long(b) * a.T_q + (q_ok ? i : i0)) * a.H + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ht][ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
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

  // two chunks in flight: chunk c is stored from one register set while
  // chunk c + 1 is still loading into the other
  Pre<CSA_BF16> pr[2];
  uint32_t tag[2][2];
  if (n_list > 0) prefetch_mq<kCKV>(a, pr[0], tag[0], b, raw0, nv_max, p_lo, n_list, 0, t0, n_q);
  if (n_list > kNK) prefetch_mq<kCKV>(a, pr[1], tag[1], b, raw0, nv_max, p_lo, n_list, kNK, t0, n_q);
  auto step = [&](Pre<CSA_BF16>& prc, uint32_t (&tgc)[2], int j0) {
    __syncthreads();
    store_chunk<CSA_BF16, kCKV>(s.c, prc, a.sm_log2);
    if (item_dg() == 0) {
      s.vis[2 * item_kp()] = tgc[0];
      s.vis[2 * item_kp() + 1] = tgc[1];
    }
    __syncthreads();
    if (j0 + 2 * kNK < n_list)
      prefetch_mq<kCKV>(a, prc, tgc, b, raw0, nv_max, p_lo, n_list, j0 + 2 * kNK, t0, n_q);
    // S^T for the 4 key tiles x 2 head tiles; K fragments shared by both tiles
    float x[2][4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(&s.c.K[kt * 16 + col][ks * 32 + g * 8]);
        acc[0] = mfma_k32(kf, qb[0][ks], acc[0]);
        acc[1] = mfma_k32(kf, qb[1][ks], acc[1]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kt * 16 + 4 * g + r;
        const bool vis = (s.vis[kk] >> qi) & 1u;
        const float scl = s.c.sk[kk];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) x[ht][kt][r] = vis ? acc[ht][r] * scl : -INFINITY;
      }
    }
    uint32_t pw[2][2][4];   // [ht][32-key step][pair]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float cmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, x[ht][kt][r]);
      cmax = column_max(cmax);
      // lazy running max, as in the one-query kernel
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
      float psum = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kt][r] = __builtin_amdgcn_exp2f(x[ht][kt][r] - m_use);
          psum += p[kt][r];
        }
      l_run[ht] += psum;
      // 32-key step st covers key tiles 2st, 2st+1: contraction slot 8g+j <->
      // key (2st)*16 + 4g + j (j < 4) / (2st+1)*16 + 4g + j - 4
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          const int kt = 2 * st + (h2 >> 1);
          const int r0 = (h2 & 1) * 2;
          const int key = kt * 16 + 4 * g + r0;
          pw[ht][st][h2] = pack_bf16x2(p[kt][r0] * s.c.sv[key], p[kt][r0 + 1] * s.c.sv[key + 1]);
        }
    }
    // O^T += V^T P^T; V^T fragments shared by both tiles
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int k0 = st * 32 + 4 * g;
      const u32x4 pb0 = {pw[0][st][0], pw[0][st][1], pw[0][st][2], pw[0][st][3]};
      const u32x4 pb1 = {pw[1][st][0], pw[1][st][1], pw[1][st][2], pw[1][st][3]};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint16_t* vt = &s.c.Vt[2 * dt + (col >> 3)][(col & 7) * kVRow + k0];   // row dt*16 + col
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vt);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + 16);
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
        o[0][dt] = mfma_k32(vf, pb0, o[0][dt]);
        o[1][dt] = mfma_k32(vf, pb1, o[1][dt]);
      }
    }
  };
  for (int j0 = 0; j0 < n_list; j0 += 2 * kNK) {
    step(pr[0], tag[0], j0);
    if (j0 + kNK < n_list) step(pr[1], tag[1], j0 + kNK);
  }
  if (!q_ok) return;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const float L = column_sum(l_run[ht]);
    const int head = ((wid % kWPQ) * 2 + ht) * 16 + col;
    const long orow = (long(b) * a.T_q + i) * a.H + head;
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
};

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
    const long per = max(2L, (chunks + kMaxSplits - 1) / kMaxSplits);
    p.split_len = int(per * kNK);
    p.n_splits = int((chunks + per - 1) / per);
    p.blocks = rows * p.n_splits;
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

size_t plan_ws_bytes(const Plan& p, long rows, int H) {
  if (p.n_splits <= 1) return 0;
  const size_t slots = size_t(rows) * p.n_splits * H;
  const size_t ml = ((slots * 2 * 4 + 255) / 256) * 256;
  return ml + slots * kHeadDim * 4;
}

template <int kIO, int kCKV, bool kDense, int kHTW, int kDepth, bool kVarlen>
hipError_t launch_attn(const AttnArgs& a, long blocks, hipStream_t st) {
  static bool attr = false;   // per instantiation; dynamic LDS above 64 KB needs the opt-in
  constexpr size_t bytes = lds_bytes<kIO, kHTW>();
  auto fn = attn_kernel<kIO, kCKV, kDense, kHTW, kDepth, kVarlen>;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(bytes));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(fn, dim3(unsigned(blocks)), dim3(kThreads), bytes, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  const long heads = blocks / a.n_splits * a.H;
  hipLaunchKernelGGL(attn_merge_kernel<kIO>, dim3(unsigned(heads)), dim3(64), 0, st, a.part_ml, a.part_o, a.n_splits,
                     a.H, a.out, a.lse);
  return hipGetLastError();
}

template <int kCKV, int kQB>
hipError_t launch_mq_q(const AttnArgs& a, int B, hipStream_t st) {
  static bool attr = false;
  constexpr size_t bytes = sizeof(LdsMQ);
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_mq_kernel<kCKV, kQB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    attr = true;
  }
  const long blocks = long(B) * ((a.T_q + kQB - 1) / kQB);
  hipLaunchKernelGGL((attn_mq_kernel<kCKV, kQB>), dim3(unsigned(blocks)), dim3(kThreads), bytes, st, a);
  return hipGetLastError();
}

template <int kCKV>
hipError_t launch_mq(const AttnArgs& a, int B, hipStream_t st) {
  switch (a.H) {
    case 32: return launch_mq_q<kCKV, 8>(a, B, st);
    case 64: return launch_mq_q<kCKV, 4>(a, B, st);
    default: return launch_mq_q<kCKV, 2>(a, B, st);
  }
}

// The many-query dense kernel serves bf16 queries with H in {32, 64, 128}
// when a sequence has enough queries to fill its blocks and the key lists
// need no split.
bool use_mq(int io_dtype, int H, int T_q, const Plan& p) {
  return io_dtype == CSA_BF16 && (H == 32 || H == 64 || H == 128) && T_q >= 64 && p.n_splits == 1;
}

template <int kIO, int kCKV, bool kDense, bool kVarlen>
hipError_t launch_tiles(const AttnArgs& a, long blocks, hipStream_t st) {
  // split key lists of more than two chunks take the two-chunk pipeline
  // (fp32 queries over more than 64 heads would not fit its registers); with
  // two chunks the one-ahead prefetch already overlaps the second, and more
  // chunks in flight only delay the first (a CU's loads in flight are few)
  if (a.n_splits > 1 && a.split_len > 2 * kNK) {
    if (a.H <= 64) return launch_attn<kIO, kCKV, kDense, 1, 2, kVarlen>(a, blocks, st);
    if constexpr (kIO == CSA_BF16) return launch_attn<kIO, kCKV, kDense, 2, 2, kVarlen>(a, blocks, st);
  }
  return a.H <= 64 ? launch_attn<kIO, kCKV, kDense, 1, 1, kVarlen>(a, blocks, st)
                   : launch_attn<kIO, kCKV, kDense, 2, 1, kVarlen>(a, blocks, st);
}

template <bool kDense, bool kVarlen>
csa_status_t tiles_for(const AttnArgs& a, int io_dtype, int ckv_dtype, long blocks, hipStream_t st) {
  hipError_t err;
  if (io_dtype == CSA_BF16 && ckv_dtype == CSA_BF16) err = launch_tiles<CSA_BF16, CSA_BF16, kDense, kVarlen>(a, blocks, st);
  else if (io_dtype == CSA_BF16 && ckv_dtype == CSA_FP8_E4M3) err = launch_tiles<CSA_BF16, CSA_FP8_E4M3, kDense, kVarlen>(a, blocks, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_F32) err = launch_tiles<CSA_F32, CSA_F32, kDense, kVarlen>(a, blocks, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_FP8_E4M3) err = launch_tiles<CSA_F32, CSA_FP8_E4M3, kDense, kVarlen>(a, blocks, st);
  else return CSA_ENOTSUP;
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}

template <bool kDense>
csa_status_t run_attn(AttnArgs a, int io_dtype, int ckv_dtype, int B, void* ws, size_t ws_size, hipStream_t st,
                      bool invariant) {
  const long rows = long(B) * a.T_q;
  if (rows == 0) return CSA_OK;
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
  return a.row_seq ? tiles_for<kDense, true>(a, io_dtype, ckv_dtype, p.blocks, st)
                   : tiles_for<kDense, false>(a, io_dtype, ckv_dtype, p.blocks, st);
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

size_t csa_attn_workspace_size(long rows, int H, int n_list, bool invariant) {
  return plan_ws_bytes(make_plan(rows, n_list, invariant), rows, H);
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

// Varlen: n_rows query rows of any mix of sequences (decode rows and prefill
// chunks together), row r of sequence row_seq[r] at position row_pos[r];
// the batch-invariant plan, so each row's bits equal those of the
// *_batch_invariant calls on its own sequence.
csa_status_t varlen_attn(AttnArgs a, bool dense, int io_dtype, int ckv_dtype, const int32_t* row_seq,
                         const int32_t* row_pos, int n_rows, void* ws, size_t ws_bytes, hipStream_t st) {
  if (n_rows > 0 && (!row_seq || !row_pos)) return CSA_EINVAL;
  a.row_seq = row_seq;
  a.row_pos = row_pos;
  a.T_q = 1;
  return dense ? run_attn<true>(a, io_dtype, ckv_dtype, n_rows, ws, ws_bytes, st, true)
               : run_attn<false>(a, io_dtype, ckv_dtype, n_rows, ws, ws_bytes, st, true);
}

}  // namespace

extern "C" csa_status_t csa_sparse_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                               const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                               int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                                               const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                                               const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                                               int32_t W, int32_t B, int32_t H, int32_t d, float sm_scale, void* out,
                                               float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (n_rows < 0 || B < 0) return CSA_EINVAL;
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                row_pos ? row_pos : reinterpret_cast<const int32_t*>(q), W, n_rows, 1, H, d, out);
  if (c != CSA_OK) return c;
  if (!idx || k < 1) return CSA_EINVAL;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = idx; a.k = k; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.W = W; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = k + W;
  return varlen_attn(a, false, io_dtype, ckv_dtype, row_seq, row_pos, n_rows, ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

extern "C" csa_status_t hca_dense_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                              const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                              int32_t cap, int32_t m_prime, const void* k_win, const void* v_win,
                                              const int32_t* raw_pos0, int32_t L_raw, const int32_t* row_seq,
                                              const int32_t* row_pos, int32_t n_rows, int32_t W, int32_t B, int32_t H,
                                              int32_t d, float sm_scale, void* out, float* lse, void* ws,
                                              size_t ws_bytes, void* stream) {
  if (n_rows < 0 || B < 0) return CSA_EINVAL;
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                row_pos ? row_pos : reinterpret_cast<const int32_t*>(q), W, n_rows, 1, H, d, out);
  if (c != CSA_OK) return c;
  if (m_prime < 1) return CSA_EINVAL;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = nullptr; a.k = m_prime; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.W = W; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = cap + W;
  return varlen_attn(a, true, io_dtype, ckv_dtype, row_seq, row_pos, n_rows, ws, ws_bytes,
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
