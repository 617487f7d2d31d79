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
// All query heads share the single KV head, so the heads are the M dimension
// of the matrix-core tiles: a key row is fetched once and used by every head.
// One block owns one query (all H heads, one wave per 16 heads) and one
// contiguous split of its key list.  Keys are gathered in chunks of 32 into
// LDS (K row-major; V transposed so the P*V operand reads 8 keys of one head
// dimension as two 8-byte words), then per wave:
//   S^T[32 keys x 16 heads] = K * Q^T       (bf16 MFMA 16x16x32, Q in VGPRs)
//   online softmax per head (fp32, exp2 domain)
//   O^T[128 x 16 heads]    += V^T * P^T     (P^T straight from S^T's C layout;
//                                            the contraction order of the 32
//                                            keys is permuted to match it)
// fp8 (E4M3FN) entries are widened to bf16 exactly; the per-entry K scale is
// applied to the logits and the V scale folded into P before the P*V product.
// The fp32 variant uses the fp32 MFMA 16x16x4 with the same data flow (V stays
// row-major there: the 4-wide contraction lines up with S^T's rows).
//
// Split-K: with few queries (decode) each query's key list is cut into
// fixed-size splits (a function of the shape only); every split writes its
// unnormalised O, running max and sum to the workspace and the last block to
// finish (agent-scope atomic counter) merges the splits in split order, so the
// result is bitwise reproducible.  The last block also re-arms the counter.
#include "common.hpp"

namespace {

constexpr int kNK = 32;                 // keys per chunk
constexpr int kKPad = 8;                // bf16 pad per K row in LDS
constexpr int kVPad = 4;                // bf16 pad per V^T row in LDS
constexpr int kF32Pad = 4;              // fp32 pad per row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

CSA_DEV v4f mfma_bf16(const v8bf& a, const v8bf& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
CSA_DEV v4f mfma_f32(float a, float b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

CSA_DEV v8bf as_v8bf(u32x4 u) { return __builtin_bit_cast(v8bf, u); }

struct AttnArgs {
  const void* q;
  const void* ck;
  const void* cv;
  const float* ck_scale;
  const float* cv_scale;
  int cap;
  const int32_t* idx;   // sparse only
  int k;                // sparse: list length; dense: m_prime
  const void* k_win;
  const void* v_win;
  const int32_t* raw_pos0;
  int L_raw;
  const int32_t* q_pos0;
  int W;
  int T_q;
  int H;
  float sm_log2;        // sm_scale * log2(e)
  void* out;
  float* lse;
  int n_list;           // key-list length (k + W or cap + W)
  int split_len;        // keys per split (multiple of kNK)
  int n_splits;
  uint32_t* counters;   // [rows]
  float* part_ml;       // [rows, n_splits, H, 2]
  float* part_o;        // [rows, n_splits, H, 128]
};

// Where key-list slot j of query (b, t) comes from.  Returns false for an
// empty / invisible slot.  *from_ckv tells which buffer; *row is its row.
template <bool kDense>
CSA_DEV bool key_source(const AttnArgs& a, int b, int i, int t, int j, bool* from_ckv, long* row) {
  int head_len;
  if constexpr (kDense) {
    head_len = a.cap;
    if (j < a.cap) {
      const int nv = min((t + 1) / a.k, a.cap);
      *from_ckv = true;
      *row = long(b) * a.cap + j;
      return j < nv;
    }
  } else {
    head_len = a.k;
    if (j < a.k) {
      const int e = a.idx[(long(b) * a.T_q + i) * a.k + j];
      *from_ckv = true;
      *row = long(b) * a.cap + e;
      return e >= 0 && e < a.cap;
    }
  }
  const int w = j - head_len;
  if (w >= a.W) return false;
  const int p = t - a.W + 1 + w;
  const int r = p - a.raw_pos0[b];
  *from_ckv = false;
  *row = long(b) * a.L_raw + r;
  return p >= 0 && r >= 0 && r < a.L_raw;
}

// --------------------------------------------------------------------------
// Load 16 consecutive head-dim values [16*dc, 16*dc+16) of a K or V row as
// fp32 (valid) or zeros.
template <int kDT>
CSA_DEV void load16(const void* base, long row, int dc, float* x) {
  if constexpr (kDT == CSA_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + row * kHeadDim + dc * 16);
    u32x4 u0 = p[0], u1 = p[1];
    uint32_t w[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else if constexpr (kDT == CSA_F32) {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(base) + row * kHeadDim + dc * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4f v = p[i];
      x[4 * i] = v[0]; x[4 * i + 1] = v[1]; x[4 * i + 2] = v[2]; x[4 * i + 3] = v[3];
    }
  } else {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(base) + row * kHeadDim + dc * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = e4m3_to_f32((u[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  }
}

template <int kIO, int kCKV>
struct Smem;

// bf16 compute path
template <int kCKV>
struct Smem<CSA_BF16, kCKV> {
  uint16_t K[kNK][kHeadDim + kKPad];
  uint16_t Vt[kHeadDim][kNK + kVPad];
  float sk[kNK];
  float sv[kNK];
  int valid[kNK];
  uint32_t flag;
};
// fp32 compute path
template <int kCKV>
struct Smem<CSA_F32, kCKV> {
  float K[kNK][kHeadDim + kF32Pad];
  float V[kNK][kHeadDim + kF32Pad];
  float sk[kNK];
  float sv[kNK];
  int valid[kNK];
  uint32_t flag;
};

template <int kIO, int kCKV, bool kDense>
CSA_DEV void gather_chunk(const AttnArgs& a, Smem<kIO, kCKV>& s, int b, int i, int t, int j0, int j_end) {
  for (int u = threadIdx.x; u < kNK * 8; u += blockDim.x) {
    const int kk = u >> 3;
    const int dc = u & 7;
    const int j = j0 + kk;
    bool from_ckv = false;
    long row = 0;
    const bool ok = j < j_end && key_source<kDense>(a, b, i, t, j, &from_ckv, &row);
    float xk[16], xv[16];
    float sck = 1.f, scv = 1.f;
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { xk[e] = 0.f; xv[e] = 0.f; }
    } else if (from_ckv) {
      load16<kCKV>(a.ck, row, dc, xk);
      load16<kCKV>(a.cv, row, dc, xv);
      if constexpr (kCKV == CSA_FP8_E4M3) {
        sck = a.ck_scale[row];
        scv = a.cv_scale[row];
      }
    } else {
      load16<kIO>(a.k_win, row, dc, xk);
      load16<kIO>(a.v_win, row, dc, xv);
    }
    if constexpr (kIO == CSA_BF16) {
      // values are exact in bf16 (bf16 inputs, or E4M3 codes)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const uint32_t w = (__float_as_uint(xk[e]) >> 16) | (__float_as_uint(xk[e + 1]) & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&s.K[kk][dc * 16 + e]) = w;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s.Vt[dc * 16 + e][kk] = uint16_t(__float_as_uint(xv[e]) >> 16);
    } else {
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        *reinterpret_cast<v4f*>(&s.K[kk][dc * 16 + e]) = v4f{xk[e], xk[e + 1], xk[e + 2], xk[e + 3]};
        *reinterpret_cast<v4f*>(&s.V[kk][dc * 16 + e]) = v4f{xv[e], xv[e + 1], xv[e + 2], xv[e + 3]};
      }
    }
    if (dc == 0) {
      s.sk[kk] = sck;
      s.sv[kk] = scv;
      s.valid[kk] = ok ? 1 : 0;
    }
  }
}

template <int kIO, int kCKV, bool kDense>
__global__ __launch_bounds__(512) void attn_kernel(AttnArgs a) {
  __shared__ Smem<kIO, kCKV> s;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;   // head within the wave's 16 (S^T / O^T column)
  const int g = lane >> 4;
  const int split = blockIdx.x;
  const long qrow = blockIdx.y;            // b * T_q + i
  const int b = int(qrow / a.T_q);
  const int i = int(qrow - long(b) * a.T_q);
  const int t = a.q_pos0[b] + i;
  const int head = wid * 16 + col;
  const int j_begin = split * a.split_len;
  const int j_end = min(j_begin + a.split_len, a.n_list);

  // ---- Q fragment (B operand of S^T = K Q^T): head `head`, this lane's d-slice
  constexpr int kQRegs = kIO == CSA_BF16 ? 4 : 32;
  u32x4 qb[kIO == CSA_BF16 ? 4 : 1];
  float qf[kIO == CSA_BF16 ? 1 : 32];
  if constexpr (kIO == CSA_BF16) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32 + g * 8);
  } else {
    const float* qp = static_cast<const float*>(a.q) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = qp[ks * 4 + g];
  }
  (void)kQRegs;

  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max (log2 domain) of this lane's head
  float l_run = 0.f;         // this lane's partial sum (its 8 keys per chunk)

  for (int j0 = j_begin; j0 < j_end; j0 += kNK) {
    __syncthreads();
    gather_chunk<kIO, kCKV, kDense>(a, s, b, i, t, j0, j_end);
    __syncthreads();

    // ---- S^T for two 16-key tiles
    float x[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kIO == CSA_BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(&s.K[mt * 16 + col][ks * 32 + g * 8]);
          acc = mfma_bf16(as_v8bf(kv), as_v8bf(qb[ks]), acc);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) acc = mfma_f32(s.K[mt * 16 + col][ks * 4 + g], qf[ks], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = mt * 16 + 4 * g + r;
        x[mt][r] = s.valid[kk] ? acc[r] * s.sk[kk] * a.sm_log2 : -INFINITY;
      }
    }
    // ---- online softmax (per head = per column; 4 lane groups share a head)
    float cmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);   // m_run == -inf -> 0
    m_run = m_new;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mt][r] = exp2f(x[mt][r] - m_use);
        psum += p[mt][r];
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (kIO == CSA_BF16) {
      uint32_t pw[4];
#pragma unroll
      for (int h2 = 0; h2 < 4; ++h2) {
        const int mt = h2 >> 1;
        const int r0 = (h2 & 1) * 2;
        const float p0 = p[mt][r0] * s.sv[mt * 16 + 4 * g + r0];
        const float p1 = p[mt][r0 + 1] * s.sv[mt * 16 + 4 * g + r0 + 1];
        pw[h2] = uint32_t(f32_to_bf16(p0)) | (uint32_t(f32_to_bf16(p1)) << 16);
      }
      const v8bf pb = as_v8bf(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = dt * 16 + col;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&s.Vt[d][4 * g]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&s.Vt[d][16 + 4 * g]);
        o[dt] = mfma_bf16(as_v8bf(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, o[dt]);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = mt * 16 + 4 * g + r;
          const float pv = p[mt][r] * s.sv[kk];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[dt] = mfma_f32(s.V[kk][dt * 16 + col], pv, o[dt]);
        }
    }
  }

  // per-head sum over the 4 lane groups
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  if (a.n_splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if constexpr (kIO == CSA_BF16) {
      uint16_t* op = static_cast<uint16_t*>(a.out) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t w0 = uint32_t(f32_to_bf16(o[dt][0] * inv)) | (uint32_t(f32_to_bf16(o[dt][1] * inv)) << 16);
        const uint32_t w1 = uint32_t(f32_to_bf16(o[dt][2] * inv)) | (uint32_t(f32_to_bf16(o[dt][3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(op + dt * 16 + 4 * g) = u32x2{w0, w1};
      }
    } else {
      float* op = static_cast<float*>(a.out) + (qrow * a.H + head) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(op + dt * 16 + 4 * g) = o[dt] * inv;
    }
    if (a.lse && g == 0)
      a.lse[qrow * a.H + head] = l_tot > 0.f ? (m_run * kLn2 + logf(l_tot)) : -INFINITY;
    return;
  }

  // ---- split-K: publish this split's partial state
  {
    const long base = (qrow * a.n_splits + split) * a.H + head;
    float* po = a.part_o + base * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(po + dt * 16 + 4 * g) = o[dt];
    if (g == 0) {
      a.part_ml[base * 2] = m_run;
      a.part_ml[base * 2 + 1] = l_tot;
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.counters[qrow], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s.flag = prev == uint32_t(a.n_splits - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s.flag) return;
  __threadfence();
  // ---- last block: merge the splits in split order
  const int n_el = a.H * kHeadDim;
  for (int e = threadIdx.x; e < n_el; e += blockDim.x) {
    const int h = e / kHeadDim;
    const int d = e - h * kHeadDim;
    float M = -INFINITY;
    for (int sp = 0; sp < a.n_splits; ++sp)
      M = fmaxf(M, __builtin_nontemporal_load(&a.part_ml[((qrow * a.n_splits + sp) * a.H + h) * 2]));
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int sp = 0; sp < a.n_splits; ++sp) {
      const long base = (qrow * a.n_splits + sp) * a.H + h;
      const float ms = __builtin_nontemporal_load(&a.part_ml[base * 2]);
      const float ls = __builtin_nontemporal_load(&a.part_ml[base * 2 + 1]);
      const float f = exp2f(ms - Mu);
      L = fmaf(ls, f, L);
      acc = fmaf(__builtin_nontemporal_load(&a.part_o[base * kHeadDim + d]), f, acc);
    }
    const float v = L > 0.f ? acc / L : 0.f;
    if constexpr (kIO == CSA_BF16)
      static_cast<uint16_t*>(a.out)[(qrow * a.H + h) * kHeadDim + d] = f32_to_bf16(v);
    else
      static_cast<float*>(a.out)[(qrow * a.H + h) * kHeadDim + d] = v;
    if (a.lse && d == 0) a.lse[qrow * a.H + h] = L > 0.f ? (M * kLn2 + logf(L)) : -INFINITY;
  }
  if (threadIdx.x == 0) a.counters[qrow] = 0u;
}

// ------------------------------------------------------------------ host --
struct SplitPlan {
  int split_len, n_splits;
};

SplitPlan plan_splits(long rows, int n_list) {
  // Enough blocks to fill the 256 CUs about twice; a split is never shorter
  // than 64 keys and is a multiple of the 32-key chunk.  Depends only on the
  // shape, never on data or timing.
  constexpr long kTargetBlocks = 512;
  SplitPlan p;
  if (n_list <= 0) return SplitPlan{kNK, 1};
  long want = (kTargetBlocks + rows - 1) / rows;
  if (want < 1) want = 1;
  long len = (n_list + want - 1) / want;
  len = ((len + kNK - 1) / kNK) * kNK;
  if (len < 64) len = 64;
  if (len > n_list) len = ((n_list + kNK - 1) / kNK) * kNK;
  p.split_len = int(len);
  p.n_splits = int((n_list + len - 1) / len);
  return p;
}

size_t ws_bytes_for(long rows, int H, int n_splits) {
  if (n_splits <= 1) return 0;
  const size_t cnt = ((size_t(rows) * 4 + 255) / 256) * 256;
  const size_t ml = ((size_t(rows) * n_splits * H * 2 * 4 + 255) / 256) * 256;
  const size_t po = size_t(rows) * n_splits * H * kHeadDim * 4;
  return cnt + ml + po;
}

template <int kIO, int kCKV, bool kDense>
hipError_t launch_attn(const AttnArgs& a, long rows, hipStream_t st) {
  dim3 grid(a.n_splits, unsigned(rows));
  hipLaunchKernelGGL((attn_kernel<kIO, kCKV, kDense>), grid, dim3(64 * (a.H / 16)), 0, st, a);
  return hipGetLastError();
}

template <bool kDense>
csa_status_t run_attn(AttnArgs a, int io_dtype, int ckv_dtype, int B, int d, void* ws, size_t ws_size,
                      hipStream_t st) {
  const long rows = long(B) * a.T_q;
  if (rows == 0) return CSA_OK;
  if (rows > 0x7FFFFFFFL) return CSA_ENOTSUP;
  const SplitPlan p = plan_splits(rows, a.n_list);
  a.split_len = p.split_len;
  a.n_splits = p.n_splits;
  const size_t need = ws_bytes_for(rows, a.H, p.n_splits);
  if (need > 0) {
    if (!ws || ws_size < need) return CSA_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    const size_t cnt = ((size_t(rows) * 4 + 255) / 256) * 256;
    const size_t ml = ((size_t(rows) * p.n_splits * a.H * 2 * 4 + 255) / 256) * 256;
    a.counters = reinterpret_cast<uint32_t*>(w);
    a.part_ml = reinterpret_cast<float*>(w + cnt);
    a.part_o = reinterpret_cast<float*>(w + cnt + ml);
  }
  (void)d;
  hipError_t err;
  if (io_dtype == CSA_BF16 && ckv_dtype == CSA_BF16) err = launch_attn<CSA_BF16, CSA_BF16, kDense>(a, rows, st);
  else if (io_dtype == CSA_BF16 && ckv_dtype == CSA_FP8_E4M3) err = launch_attn<CSA_BF16, CSA_FP8_E4M3, kDense>(a, rows, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_F32) err = launch_attn<CSA_F32, CSA_F32, kDense>(a, rows, st);
  else if (io_dtype == CSA_F32 && ckv_dtype == CSA_FP8_E4M3) err = launch_attn<CSA_F32, CSA_FP8_E4M3, kDense>(a, rows, st);
  else return CSA_ENOTSUP;
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
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

size_t csa_attn_workspace_size(long rows, int H, int n_list) {
  return ws_bytes_for(rows, H, plan_splits(rows, n_list).n_splits);
}

extern "C" csa_status_t csa_sparse_attn(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                        const float* ck_scale, const float* cv_scale, int32_t ckv_dtype, int32_t cap,
                                        const int32_t* idx, int32_t k, const void* k_win, const void* v_win,
                                        const int32_t* raw_pos0, int32_t L_raw, const int32_t* q_pos0, int32_t W,
                                        int32_t B, int32_t T_q, int32_t H, int32_t d, float sm_scale, void* out,
                                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, B, T_q, H, d, out);
  if (c != CSA_OK) return c;
  if (!idx || k < 1) return CSA_EINVAL;
  if (long(k) + W > 0x7FFFFFFFL) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = idx; a.k = k; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.T_q = T_q; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = k + W;
  return run_attn<false>(a, io_dtype, ckv_dtype, B, d, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" csa_status_t hca_dense_attn(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                       const float* ck_scale, const float* cv_scale, int32_t ckv_dtype, int32_t cap,
                                       int32_t m_prime, const void* k_win, const void* v_win, const int32_t* raw_pos0,
                                       int32_t L_raw, const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q,
                                       int32_t H, int32_t d, float sm_scale, void* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  csa_status_t c = check_common(q, io_dtype, ck, cv, ck_scale, cv_scale, ckv_dtype, cap, k_win, v_win, raw_pos0, L_raw,
                                q_pos0, W, B, T_q, H, d, out);
  if (c != CSA_OK) return c;
  if (m_prime < 1) return CSA_EINVAL;
  if (long(cap) + W > 0x7FFFFFFFL) return CSA_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.ck = ck; a.cv = cv; a.ck_scale = ck_scale; a.cv_scale = cv_scale; a.cap = cap;
  a.idx = nullptr; a.k = m_prime; a.k_win = k_win; a.v_win = v_win; a.raw_pos0 = raw_pos0; a.L_raw = L_raw;
  a.q_pos0 = q_pos0; a.W = W; a.T_q = T_q; a.H = H; a.sm_log2 = sm_scale * kLog2e; a.out = out; a.lse = lse;
  a.n_list = cap + W;
  return run_attn<true>(a, io_dtype, ckv_dtype, B, d, ws, ws_bytes, static_cast<hipStream_t>(stream));
}
