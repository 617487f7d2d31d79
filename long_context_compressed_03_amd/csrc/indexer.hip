// Lightning-indexer scores on the CDNA4 block-scaled MXFP4 matrix cores.
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
// holds 16/H_I whole queries; the head sum is 4 rows inside a lane plus, for
// H_I > 4, a cross-lane add.  Products of E2M1 values times power-of-two
// scales are exact and the inputs keep every partial sum inside fp32's
// integer range, so the GPU scores equal the exact scores bit for bit.
//
// Work split: a block of 4 waves owns RT row tiles of one sequence; each wave
// walks its own run of entries, 16 per MFMA, with the A fragments (queries)
// held in registers for the whole run.  Decode (one query) is a pure stream of
// the keys: 68 B per entry for d_I = 128.
#include "common.hpp"

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxKSteps = 4;  // d_I <= 512

CSA_DEV v4f mfma_fp4(u32x4 a, int sa, u32x4 b, int sb, v4f c) {
  v8i av = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
  v8i bv = {int(b[0]), int(b[1]), int(b[2]), int(b[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// kHI: indexer heads (4, 8 or 16); kRT: 16-row tiles per block; kKS: 128-wide
// contraction steps; kFrag: 16-entry fragments per wave per batch of loads.
template <int kHI, int kRT, int kKS, int kFrag, bool kStream>
__global__ __launch_bounds__(kBlock) void indexer_kernel(const uint8_t* __restrict__ q_codes,
                                                         const uint8_t* __restrict__ q_e8m0,
                                                         const float* __restrict__ w,
                                                         const uint8_t* __restrict__ k_codes,
                                                         const uint8_t* __restrict__ k_e8m0,
                                                         const int32_t* __restrict__ q_pos0, int T_q, int d_I,
                                                         int cap, int m, int entries_per_wave,
                                                         float* __restrict__ scores) {
  constexpr int kQPT = 16 / kHI;  // queries per row tile
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.z;
  const int q_block = blockIdx.y * kRT * kQPT;
  const int nblk = d_I >> 5;            // 32-element blocks per vector
  const int row_bytes = d_I >> 1;
  const int pos0 = q_pos0[b];

  // ---- A fragments (queries), weights and visibility for this lane's rows
  u32x4 a[kRT][kKS];
  int sa[kRT][kKS];
  float wv[kRT][4];
  int nv_lane[kRT];  // visible entries of the query whose rows this lane holds in C
  int nv_max = 0;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = rt * 16 + col;
    const int q = q_block + r / kHI;
    const int h = r % kHI;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const int c = ks * 4 + g;
      if (q < T_q && c < nblk) {
        const size_t vec = (size_t(b) * T_q + q) * kHI + h;
        a[rt][ks] = *reinterpret_cast<const u32x4*>(q_codes + vec * row_bytes + c * 16);
        sa[rt][ks] = q_e8m0[vec * nblk + c];
      } else {
        a[rt][ks] = u32x4{0u, 0u, 0u, 0u};
        sa[rt][ks] = 127;
      }
    }
    const int rc = rt * 16 + 4 * g;  // first C row this lane holds
    const int qc = q_block + rc / kHI;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = (rc + i) % kHI;
      wv[rt][i] = qc < T_q ? w[(size_t(b) * T_q + qc) * kHI + hh] : 0.f;
    }
    int nv = 0;
    if (qc < T_q) nv = min((pos0 + qc + 1) / m, cap);
    nv_lane[rt] = nv;
  }
  {
    // largest visibility among the block's queries (the last valid one)
    const int q_last = min(q_block + kRT * kQPT, T_q) - 1;
    nv_max = min((pos0 + q_last + 1) / m, cap);
  }

  const int e_wave0 = (blockIdx.x * kWavesPerBlock + wid) * entries_per_wave;
  const int e_wave1 = min(e_wave0 + entries_per_wave, cap);

  const uint8_t* kc_seq = k_codes + size_t(b) * cap * row_bytes;
  const uint8_t* ke_seq = k_e8m0 + size_t(b) * cap * nblk;

  for (int e_frag0 = e_wave0; e_frag0 < e_wave1; e_frag0 += 16 * kFrag) {
    u32x4 bk[kFrag][kKS];
    int sb[kFrag][kKS];
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      const int e = e_frag0 + f * 16 + col;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const int c = ks * 4 + g;
        if (e < nv_max && c < nblk) {
          const u32x4* p = reinterpret_cast<const u32x4*>(kc_seq + size_t(e) * row_bytes + c * 16);
          bk[f][ks] = kStream ? __builtin_nontemporal_load(p) : *p;
          sb[f][ks] = ke_seq[size_t(e) * nblk + c];
        } else {
          bk[f][ks] = u32x4{0u, 0u, 0u, 0u};
          sb[f][ks] = 127;
        }
      }
    }
#pragma unroll
    for (int f = 0; f < kFrag; ++f) {
      const int e0 = e_frag0 + f * 16;
      if (e0 >= e_wave1) break;
      const int e = e0 + col;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        if (e0 < nv_max) {
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) acc = mfma_fp4(a[rt][ks], sa[rt][ks], bk[f][ks], sb[f][ks], acc);
        }
        float p = wv[rt][0] * fmaxf(acc[0], 0.f);
        p = fmaf(wv[rt][1], fmaxf(acc[1], 0.f), p);
        p = fmaf(wv[rt][2], fmaxf(acc[2], 0.f), p);
        p = fmaf(wv[rt][3], fmaxf(acc[3], 0.f), p);
        bool writer = true;
        if constexpr (kHI == 8) {
          p += __shfl_xor(p, 16);
          writer = (g & 1) == 0;
        } else if constexpr (kHI == 16) {
          p += __shfl_xor(p, 16);
          p += __shfl_xor(p, 32);
          writer = g == 0;
        }
        const int q = q_block + (rt * 16 + 4 * g) / kHI;
        if (writer && q < T_q && e < e_wave1) {
          scores[(size_t(b) * T_q + q) * cap + e] = e < nv_lane[rt] ? p : -INFINITY;
        }
      }
    }
  }
}

template <int kHI, int kRT, int kKS, bool kStream>
hipError_t launch_indexer_ks(const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             float* scores, hipStream_t st) {
  constexpr int kFrag = 4;
  constexpr int kQPT = 16 / kHI;
  const int entries_per_wave = kStream ? 64 : 256;
  const int per_block = entries_per_wave * kWavesPerBlock;
  dim3 grid((cap + per_block - 1) / per_block, (T_q + kRT * kQPT - 1) / (kRT * kQPT), B);
  hipLaunchKernelGGL((indexer_kernel<kHI, kRT, kKS, kFrag, kStream>), grid, dim3(kBlock), 0, st, qc, qe, w, kc, ke,
                     pos, T_q, d_I, cap, m, entries_per_wave, scores);
  return hipGetLastError();
}

template <int kHI, int kRT, bool kStream>
hipError_t launch_indexer_rt(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                             const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                             float* scores, hipStream_t st) {
  switch (ks) {
    case 1: return launch_indexer_ks<kHI, kRT, 1, kStream>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
    case 2: return launch_indexer_ks<kHI, kRT, 2, kStream>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
    case 3: return launch_indexer_ks<kHI, kRT, 3, kStream>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
    default: return launch_indexer_ks<kHI, kRT, 4, kStream>(qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
  }
}

template <int kHI>
hipError_t launch_indexer_h(int ks, const uint8_t* qc, const uint8_t* qe, const float* w, const uint8_t* kc,
                            const uint8_t* ke, const int32_t* pos, int B, int T_q, int d_I, int cap, int m,
                            float* scores, hipStream_t st) {
  // one row tile when the whole call has at most one tile of queries (decode);
  // several otherwise so every key fragment feeds several MFMAs
  if (T_q * kHI <= 16)
    return launch_indexer_rt<kHI, 1, true>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
  return launch_indexer_rt<kHI, 4, false>(ks, qc, qe, w, kc, ke, pos, B, T_q, d_I, cap, m, scores, st);
}

}  // namespace

extern "C" csa_status_t csa_indexer_scores(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                                           const uint8_t* k_codes, const uint8_t* k_e8m0, const int32_t* q_pos0,
                                           int32_t B, int32_t T_q, int32_t H_I, int32_t d_I, int32_t cap, int32_t m,
                                           float* scores, void* stream) {
  if (!q_codes || !q_e8m0 || !w || !k_codes || !k_e8m0 || !q_pos0 || !scores) return CSA_EINVAL;
  if (H_I != 4 && H_I != 8 && H_I != 16) return CSA_ENOTSUP;
  if (d_I < 32 || d_I > 128 * kMaxKSteps || d_I % 32 != 0) return CSA_EINVAL;
  if (B < 0 || T_q < 0 || cap < 0 || m < 1) return CSA_EINVAL;
  if (B > 65535 || T_q > (1 << 24)) return CSA_ENOTSUP;
  if (B == 0 || T_q == 0 || cap == 0) return CSA_OK;
  const int ks = (d_I + 127) / 128;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (H_I) {
    case 4: err = launch_indexer_h<4>(ks, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap, m, scores, st); break;
    case 8: err = launch_indexer_h<8>(ks, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap, m, scores, st); break;
    default: err = launch_indexer_h<16>(ks, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap, m, scores, st); break;
  }
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}
