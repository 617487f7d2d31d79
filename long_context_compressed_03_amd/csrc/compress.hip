// Softmax-pool KV compression: one entry per complete block of m tokens.
//
// The pages (blog.nickys.cn DeepSeek-V4 post, 三大架构改动 §1 CSA and §2 HCA)
// state that every m (resp. m') tokens' K/V become one entry; the pooling rule
// (softmax weights from one logit per token, shared by K and V) is this
// library's reading.  This is a pure HBM stream: every input byte is read
// once and every output byte written once, no reuse.
//
// Mapping: lane c of a 16-lane group owns head columns [8c, 8c+8) (16 B of
// bf16 per row), so a row is read by the group as one contiguous 256-B
// segment.  Short blocks (m < 32, the CSA case): one group owns one entry and
// a 256-thread block covers 16 entries, walking rows with 4 loads in flight
// per lane for each of K and V.  Long blocks (the HCA case, m' = 128): the 16
// groups of a block share one tensor (K or V) of one entry, group r taking
// rows r, r+16, ..., so all rows are in flight at once; the 16 partial sums
// meet in LDS and are added in group order.
#include "common.hpp"

namespace {

constexpr int kGroup = 16;            // lanes per entry
constexpr int kColsPerLane = 8;       // 16 lanes x 8 = 128 head columns
constexpr int kBlock = 256;
constexpr int kEntriesPerBlock = kBlock / kGroup;

template <int kInF32>
CSA_DEV void load_row8(const void* base, size_t row, int lane_c, float* out) {
  if constexpr (kInF32) {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(base) + row * kHeadDim + lane_c * 8);
    v4f a = __builtin_nontemporal_load(p);
    v4f b = __builtin_nontemporal_load(p + 1);
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + row * kHeadDim + lane_c * 8);
    u32x4 a = __builtin_nontemporal_load(p);
    uint32_t w[4] = {a[0], a[1], a[2], a[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <int kOut>
CSA_DEV void store_entry(void* out, float* scale_out, size_t entry, int lane_c, const float* x) {
  if constexpr (kOut == CSA_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + entry * kHeadDim + lane_c * 8);
    p[0] = make_float4(x[0], x[1], x[2], x[3]);
    p[1] = make_float4(x[4], x[5], x[6], x[7]);
  } else if constexpr (kOut == CSA_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(f32_to_bf16(x[2 * i])) | (uint32_t(f32_to_bf16(x[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + entry * kHeadDim + lane_c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = group_max<kGroup>(amax);
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_e4m3(x[i] / scale) << (8 * (i & 3));
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(out) + entry * kHeadDim + lane_c * 8) = make_uint2(w[0], w[1]);
    if (lane_c == 0) scale_out[entry] = scale;
  }
}

template <int kInF32, int kOut>
__global__ __launch_bounds__(kBlock) void compress_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                          const float* __restrict__ logits, int B, int n_entries,
                                                          int ld_in, int m, void* k_out, void* v_out,
                                                          float* k_scale, float* v_scale, int ld_out) {
  const int lane_c = threadIdx.x & (kGroup - 1);
  const long gid = long(blockIdx.x) * (blockDim.x / kGroup) + (threadIdx.x / kGroup);
  if (gid >= long(B) * n_entries) return;  // whole 16-lane groups exit together
  const int b = int(gid / n_entries);
  const int e = int(gid - long(b) * n_entries);
  const size_t row0 = size_t(b) * ld_in + size_t(e) * m;
  const float* z = logits + row0;

  // softmax statistics of the block's logits, spread over the 16 lanes;
  // computed after the first rows are requested, so the two memory round
  // trips overlap
  float zmax = 0.f, inv = 0.f;
  auto stats = [&]() {
    zmax = -INFINITY;
    for (int x = lane_c; x < m; x += kGroup) zmax = fmaxf(zmax, z[x]);
    zmax = group_max<kGroup>(zmax);
    float zsum = 0.f;
    for (int x = lane_c; x < m; x += kGroup) zsum += expf(z[x] - zmax);
    zsum = group_sum<kGroup>(zsum);
    inv = 1.f / zsum;
  };

  float ak[8], av[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { ak[i] = 0.f; av[i] = 0.f; }

  constexpr int kU = 4;
  int j = 0;
  for (; j + kU <= m; j += kU) {
    float kr[kU][8], vr[kU][8], a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      load_row8<kInF32>(k, row0 + j + u, lane_c, kr[u]);
      load_row8<kInF32>(v, row0 + j + u, lane_c, vr[u]);
    }
    if (j == 0) stats();
#pragma unroll
    for (int u = 0; u < kU; ++u) a[u] = expf(z[j + u] - zmax) * inv;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ak[i] = fmaf(a[u], kr[u][i], ak[i]);
        av[i] = fmaf(a[u], vr[u][i], av[i]);
      }
    }
  }
  if (m < kU) stats();
  for (; j < m; ++j) {
    float kr[8], vr[8];
    load_row8<kInF32>(k, row0 + j, lane_c, kr);
    load_row8<kInF32>(v, row0 + j, lane_c, vr);
    const float a = expf(z[j] - zmax) * inv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ak[i] = fmaf(a, kr[i], ak[i]);
      av[i] = fmaf(a, vr[i], av[i]);
    }
  }
  const size_t entry = size_t(b) * ld_out + e;
  store_entry<kOut>(k_out, k_scale, entry, lane_c, ak);
  store_entry<kOut>(v_out, v_scale, entry, lane_c, av);
}

// One tensor of one entry per block (blockIdx.y: 0 = K, 1 = V; each has its
// own fp8 scale, so the two never meet): 16 groups split the rows, partial
// sums meet in LDS.  The softmax statistics are reduced over the block.
template <int kInF32, int kOut>
__global__ __launch_bounds__(kBlock) void compress_long_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                               const float* __restrict__ logits, int n_entries,
                                                               int ld_in, int m, void* k_out, void* v_out,
                                                               float* k_scale, float* v_scale, int ld_out) {
  __shared__ float part[kEntriesPerBlock][kHeadDim + 4];
  __shared__ float wz[kBlock];              // exp(z_r - max) of the first 256 rows
  __shared__ float red[2][kBlock / 64];
  const int lane_c = threadIdx.x & (kGroup - 1);
  const int grp = threadIdx.x / kGroup;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.x / n_entries;
  const int e = blockIdx.x - b * n_entries;
  const int kv = blockIdx.y;
  const void* src = kv ? v : k;
  const size_t row0 = size_t(b) * ld_in + size_t(e) * m;
  const float* z = logits + row0;

  float ak[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ak[i] = 0.f;
  constexpr int kU = 8;
  constexpr int kStride = kU * kEntriesPerBlock;   // rows per batch of the block
  float kr[kU][8];
  // rows past the block are read as its last row and weighted 0 (no branches
  // around the loads, so the waits for them stay exact)
  auto load_batch = [&](int j) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = j + u * kEntriesPerBlock;
      load_row8<kInF32>(src, row0 + min(r, m - 1), lane_c, kr[u]);
    }
  };
  float zmax, inv;
  auto add_batch = [&](int j) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = j + u * kEntriesPerBlock;
      const float a = r >= m ? 0.f : (r < kBlock ? wz[r] : expf(z[r] - zmax)) * inv;
#pragma unroll
      for (int i = 0; i < 8; ++i) ak[i] = fmaf(a, kr[u][i], ak[i]);
    }
  };

  // softmax statistics over the block: thread t takes logits t, t + 256, ...;
  // its first logit is requested before the rows, so the statistics wait for
  // the logits only and are done while the rows arrive
  const float z0 = z[int(threadIdx.x) < m ? int(threadIdx.x) : 0];
  const float zt = int(threadIdx.x) < m ? z0 : -INFINITY;
  load_batch(grp);   // m >= 32: every group has rows in the first batch
  {
    float zm = zt;
    for (int x = threadIdx.x + kBlock; x < m; x += kBlock) zm = fmaxf(zm, z[x]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) zm = fmaxf(zm, __shfl_xor(zm, o));
    if (lane == 0) red[0][wv] = zm;
    __syncthreads();
    zmax = red[0][0];
#pragma unroll
    for (int x = 1; x < kBlock / 64; ++x) zmax = fmaxf(zmax, red[0][x]);
    const float et = int(threadIdx.x) < m ? expf(zt - zmax) : 0.f;
    wz[threadIdx.x] = et;
    float zs = et;
    for (int x = threadIdx.x + kBlock; x < m; x += kBlock) zs += expf(z[x] - zmax);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) zs += __shfl_xor(zs, o);
    if (lane == 0) red[1][wv] = zs;
    __syncthreads();
    float sum = red[1][0];
#pragma unroll
    for (int x = 1; x < kBlock / 64; ++x) sum += red[1][x];
    inv = 1.f / sum;
  }
  add_batch(grp);
  for (int j = grp + kStride; j < m; j += kStride) {
    load_batch(j);
    add_batch(j);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[grp][lane_c * 8 + i] = ak[i];
  __syncthreads();
  // thread t < 128 adds the 16 partials of head column t in group order and
  // stores it (the upper half of the block repeats the sums and stores nothing)
  const int col = threadIdx.x & (kHeadDim - 1);
  const bool own = threadIdx.x < kHeadDim;
  float x = 0.f;
#pragma unroll
  for (int r = 0; r < kEntriesPerBlock; ++r) x += part[r][col];
  const size_t entry = size_t(b) * ld_out + e;
  void* out = kv ? v_out : k_out;
  if constexpr (kOut == CSA_F32) {
    if (own) static_cast<float*>(out)[entry * kHeadDim + col] = x;
  } else if constexpr (kOut == CSA_BF16) {
    if (own) static_cast<uint16_t*>(out)[entry * kHeadDim + col] = f32_to_bf16(x);
  } else {
    // per-entry scale from the max magnitude over the entry's 128 values (waves 0 and 1)
    __shared__ float wmax[kBlock / 64];
    float amax = fabsf(x);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(wmax[0], wmax[1]);
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    if (own) static_cast<uint8_t*>(out)[entry * kHeadDim + col] = uint8_t(f32_to_e4m3(x / scale));
    if (col == 0 && own) (kv ? v_scale : k_scale)[entry] = scale;
  }
}

template <int kInF32, int kOut>
hipError_t launch_one(dim3 grid_short, long total, hipStream_t st, const void* k, const void* v, const float* lg, int B,
                      int ne, int ld_in, int m, void* ko, void* vo, float* ks, float* vs, int ld_out) {
  (void)grid_short;
  if (m >= 32) {
    hipLaunchKernelGGL((compress_long_kernel<kInF32, kOut>), dim3(unsigned(total), 2u), dim3(kBlock), 0, st, k, v, lg, ne,
                       ld_in, m, ko, vo, ks, vs, ld_out);
  } else {
    // few entries (decoding): 4 per 64-thread block, so their rows are
    // fetched by several CUs; otherwise 16 per 256-thread block
    const int threads = total <= 256 ? 64 : kBlock;
    const long per = threads / kGroup;
    hipLaunchKernelGGL((compress_kernel<kInF32, kOut>), dim3(unsigned((total + per - 1) / per)), dim3(threads), 0, st,
                       k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out);
  }
  return hipGetLastError();
}

template <int kInF32>
hipError_t launch_compress(int out_dt, dim3 grid, long total, hipStream_t st, const void* k, const void* v,
                           const float* lg, int B, int ne, int ld_in, int m, void* ko, void* vo, float* ks, float* vs,
                           int ld_out) {
  switch (out_dt) {
    case CSA_BF16:
      return launch_one<kInF32, CSA_BF16>(grid, total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out);
    case CSA_F32:
      return launch_one<kInF32, CSA_F32>(grid, total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out);
    default:
      return launch_one<kInF32, CSA_FP8_E4M3>(grid, total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out);
  }
}

}  // namespace

extern "C" csa_status_t csa_compress_kv(const void* k, const void* v, int32_t in_dtype, const float* logits,
                                        int32_t B, int32_t L, int32_t ld_in, int32_t d, int32_t m, void* k_out,
                                        void* v_out, float* k_scale_out, float* v_scale_out, int32_t ld_out,
                                        int32_t out_dtype, void* stream) {
  if (!k || !v || !logits || !k_out || !v_out) return CSA_EINVAL;
  if (in_dtype != CSA_BF16 && in_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(out_dtype)) return CSA_EINVAL;
  if (d != kHeadDim || m < 1 || B < 0 || L < 0 || L % m != 0 || ld_in < L) return CSA_EINVAL;
  const int ne = L / m;
  if (ld_out < ne) return CSA_EINVAL;
  if (out_dtype == CSA_FP8_E4M3 && (!k_scale_out || !v_scale_out)) return CSA_EINVAL;
  const long total = long(B) * ne;
  if (total == 0) return CSA_OK;
  const long blocks = (total + kEntriesPerBlock - 1) / kEntriesPerBlock;
  if (blocks > 0x7FFFFFFFL) return CSA_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (total > 0x7FFFFFFFL) return CSA_EINVAL;
  hipError_t err = in_dtype == CSA_F32
                       ? launch_compress<1>(out_dtype, dim3(unsigned(blocks)), total, st, k, v, logits, B, ne, ld_in, m,
                                            k_out, v_out, k_scale_out, v_scale_out, ld_out)
                       : launch_compress<0>(out_dtype, dim3(unsigned(blocks)), total, st, k, v, logits, B, ne, ld_in, m,
                                            k_out, v_out, k_scale_out, v_scale_out, ld_out);
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}
