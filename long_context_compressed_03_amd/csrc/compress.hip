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
#include "compress_core.hpp"

namespace {

using namespace csa_cmp;

constexpr int kBlock = 256;
constexpr int kEntriesPerBlock = kBlock / kGroup;

template <int kInF32, int kOut>
__global__ __launch_bounds__(kBlock) void compress_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                          const float* __restrict__ logits, int B, int n_entries,
                                                          int ld_in, int m, void* k_out, void* v_out,
                                                          float* k_scale, float* v_scale, int ld_out,
                                                          PackedEntries pk) {
  const int lane_c = threadIdx.x & (kGroup - 1);
  const long gid = long(blockIdx.x) * (blockDim.x / kGroup) + (threadIdx.x / kGroup);
  if (gid >= long(B) * n_entries) return;  // whole 16-lane groups exit together
  if (pk.cu) {   // packed: B = 1, n_entries = all sequences' entries
    size_t row, entry;
    packed_entry(pk, int(gid), ld_in, m, ld_out, &row, &entry);
    compress_group_at<kInF32, kOut>(k, v, logits, row, m, k_out, v_out, k_scale, v_scale, entry, lane_c);
    return;
  }
  compress_group<kInF32, kOut>(k, v, logits, n_entries, ld_in, m, k_out, v_out, k_scale, v_scale, ld_out, gid, lane_c);
}

// Cache append, short blocks (m < 32): cache_append_short_at, one 64-thread
// block per 4 sequences.
template <int kInF32, int kOut>
__global__ __launch_bounds__(64) void cache_append_short_kernel(AppendArgs a) {
  cache_append_short_at<kInF32, kOut>(a, int(blockIdx.x));
}

// One tensor of one entry per block (blockIdx.y: 0 = K, 1 = V; each has its
// own fp8 scale, so the two never meet): 16 groups split the rows, partial
// sums meet in LDS.  The softmax statistics are reduced over the block.
// kAppend (the cache append, m >= 32): block (x, t) writes tensor t's rows
// of sequence x's new token (both ring copies; the logit and window base with
// t = 0) and pools the block the token completes, its newest row read from
// the input, as the short kernel does.
template <int kInF32, int kOut, bool kAppend>
__global__ __launch_bounds__(kBlock) void compress_long_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                               const float* __restrict__ logits, int n_entries,
                                                               int ld_in, int m, void* k_out, void* v_out,
                                                               float* k_scale, float* v_scale, int ld_out,
                                                               AppendArgs app, PackedEntries pk) {
  __shared__ float part[kEntriesPerBlock][kHeadDim + 4];
  __shared__ float wz[kBlock];              // exp(z_r - max) of the first 256 rows
  __shared__ float red[2][kBlock / 64];
  const int lane_c = threadIdx.x & (kGroup - 1);
  const int grp = threadIdx.x / kGroup;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kv = blockIdx.y;
  int b, e;
  size_t row0;
  const void* newest = nullptr;           // kAppend: the token's row and logit
  const float* znew = nullptr;
  if constexpr (kAppend) {
    b = blockIdx.x;
    const int p = app.pos[b];
    const AppendPlan pl = append_plan(p, app.L, app.m, app.cap);
    constexpr int kEl = kInF32 ? 4 : 2;
    constexpr int kChunks = kHeadDim * kEl / 16;   // 16-B pieces per row
    const size_t ring0 = size_t(b) * 2 * app.L;
    const uint8_t* nrow = static_cast<const uint8_t*>(kv ? app.v_new : app.k_new) + size_t(b) * kHeadDim * kEl;
    if (p >= 0) {
      const int s = p % app.L;
      if (int(threadIdx.x) < 2 * kChunks) {
        const int c = threadIdx.x % kChunks;
        const int copy = threadIdx.x / kChunks;
        uint8_t* dst = static_cast<uint8_t*>(kv ? app.v_ring : app.k_ring) +
                       (ring0 + s + size_t(copy) * app.L) * kHeadDim * kEl + c * 16;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(nrow + c * 16);
      }
      if (kv == 0 && threadIdx.x < 2) app.z_ring[ring0 + s + size_t(threadIdx.x) * app.L] = app.z_new[b];
    }
    if (kv == 0 && threadIdx.x == 0) app.raw_pos0[b] = pl.base;
    if (!pl.done) return;                 // the whole block, before any barrier
    e = pl.entry;
    row0 = ring0 + pl.first_row;
    newest = nrow;
    znew = app.z_new + b;
  } else if (pk.cu) {   // packed: the entry's sequence b and slot e within it
    b = csa_packed_seq(pk.cu, pk.B, int(blockIdx.x));
    const int j = int(blockIdx.x) - pk.cu[b];
    e = pk.entry0[b] + j;
    row0 = size_t(b) * ld_in + size_t(pk.row0[b]) + size_t(j) * m;
  } else {
    b = blockIdx.x / n_entries;
    e = blockIdx.x - b * n_entries;
    row0 = size_t(b) * ld_in + size_t(e) * m;
  }
  const void* src = kv ? v : k;
  const float* z = logits + row0;
  auto zat = [&](int x) -> float {
    if constexpr (kAppend) return *(x == m - 1 ? znew : z + x);
    else return z[x];
  };

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
      const int rc = min(r, m - 1);
      if constexpr (kAppend) {
        const bool nw = rc == m - 1;
        load_row8<kInF32>(nw ? newest : src, nw ? size_t(0) : row0 + rc, lane_c, kr[u]);
      } else {
        load_row8<kInF32>(src, row0 + rc, lane_c, kr[u]);
      }
    }
  };
  float zmax, inv;
  auto add_batch = [&](int j) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = j + u * kEntriesPerBlock;
      const float a = r >= m ? 0.f : (r < kBlock ? wz[r] : expf(zat(r) - zmax)) * inv;
#pragma unroll
      for (int i = 0; i < 8; ++i) ak[i] = fmaf(a, kr[u][i], ak[i]);
    }
  };

  // softmax statistics over the block: thread t takes logits t, t + 256, ...;
  // its first logit is requested before the rows, so the statistics wait for
  // the logits only and are done while the rows arrive
  const float z0 = zat(int(threadIdx.x) < m ? int(threadIdx.x) : 0);
  const float zt = int(threadIdx.x) < m ? z0 : -INFINITY;
  load_batch(grp);   // m >= 32: every group has rows in the first batch
  {
    float zm = zt;
    for (int x = threadIdx.x + kBlock; x < m; x += kBlock) zm = fmaxf(zm, zat(x));
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
    for (int x = threadIdx.x + kBlock; x < m; x += kBlock) zs += expf(zat(x) - zmax);
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

// total = B * ne entries (packed: B = 1, ne = all entries, pk.cu set)
template <int kInF32, int kOut>
hipError_t launch_one(long total, hipStream_t st, const void* k, const void* v, const float* lg, int B, int ne,
                      int ld_in, int m, void* ko, void* vo, float* ks, float* vs, int ld_out, const PackedEntries& pk) {
  if (m >= 32) {
    hipLaunchKernelGGL((compress_long_kernel<kInF32, kOut, false>), dim3(unsigned(total), 2u), dim3(kBlock), 0, st, k, v,
                       lg, ne, ld_in, m, ko, vo, ks, vs, ld_out, AppendArgs{}, pk);
  } else {
    // few entries (decoding): 4 per 64-thread block, so their rows are
    // fetched by several CUs; otherwise 16 per 256-thread block
    const int threads = total <= 256 ? 64 : kBlock;
    const long per = threads / kGroup;
    hipLaunchKernelGGL((compress_kernel<kInF32, kOut>), dim3(unsigned((total + per - 1) / per)), dim3(threads), 0, st,
                       k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out, pk);
  }
  return hipGetLastError();
}

template <int kInF32>
hipError_t launch_compress(int out_dt, long total, hipStream_t st, const void* k, const void* v, const float* lg, int B,
                           int ne, int ld_in, int m, void* ko, void* vo, float* ks, float* vs, int ld_out,
                           const PackedEntries& pk = PackedEntries{}) {
  switch (out_dt) {
    case CSA_BF16:
      return launch_one<kInF32, CSA_BF16>(total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out, pk);
    case CSA_F32:
      return launch_one<kInF32, CSA_F32>(total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out, pk);
    default:
      return launch_one<kInF32, CSA_FP8_E4M3>(total, st, k, v, lg, B, ne, ld_in, m, ko, vo, ks, vs, ld_out, pk);
  }
}

template <int kInF32, int kOut>
hipError_t launch_cache_append_one(const AppendArgs& a, hipStream_t st) {
  if (a.m >= 32) {
    hipLaunchKernelGGL((compress_long_kernel<kInF32, kOut, true>), dim3(unsigned(a.B), 2u), dim3(kBlock), 0, st,
                       a.k_ring, a.v_ring, a.z_ring, a.B, 2 * a.L, a.m, a.ck, a.cv, a.ck_scale, a.cv_scale, a.cap, a,
                       PackedEntries{});
  } else {
    constexpr int kPer = 64 / kGroup;    // 4 sequences per 64-thread block
    hipLaunchKernelGGL((cache_append_short_kernel<kInF32, kOut>), dim3(unsigned((a.B + kPer - 1) / kPer)), dim3(64),
                       0, st, a);
  }
  return hipGetLastError();
}

template <int kInF32>
hipError_t launch_cache_append_in(int ckv_dtype, const AppendArgs& a, hipStream_t st) {
  switch (ckv_dtype) {
    case CSA_BF16: return launch_cache_append_one<kInF32, CSA_BF16>(a, st);
    case CSA_F32: return launch_cache_append_one<kInF32, CSA_F32>(a, st);
    default: return launch_cache_append_one<kInF32, CSA_FP8_E4M3>(a, st);
  }
}

}  // namespace

hipError_t csa_cmp::launch_cache_append(int io_dtype, int ckv_dtype, const AppendArgs& a, hipStream_t st) {
  return io_dtype == CSA_F32 ? launch_cache_append_in<1>(ckv_dtype, a, st) : launch_cache_append_in<0>(ckv_dtype, a, st);
}

extern "C" csa_status_t csa_compress_kv(const void* k, const void* v, int32_t in_dtype, const float* logits,
                                        int32_t B, int32_t L, int32_t ld_in, int32_t d, int32_t m, void* k_out,
                                        void* v_out, float* k_scale_out, float* v_scale_out, int32_t ld_out,
                                        int32_t out_dtype, void* stream) {
  const CompressArgs ca{k, v, logits, in_dtype, B, L, ld_in, m, ld_out, out_dtype, k_out, v_out, k_scale_out, v_scale_out};
  const csa_status_t chk = check_compress_args(ca, d);
  if (chk != CSA_OK) return chk;
  const int ne = L / m;
  const long total = long(B) * ne;
  if (total == 0) return CSA_OK;
  const long blocks = (total + kEntriesPerBlock - 1) / kEntriesPerBlock;
  if (blocks > 0x7FFFFFFFL) return CSA_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (total > 0x7FFFFFFFL) return CSA_EINVAL;
  hipError_t err = in_dtype == CSA_F32
                       ? launch_compress<1>(out_dtype, total, st, k, v, logits, B, ne, ld_in, m, k_out, v_out,
                                            k_scale_out, v_scale_out, ld_out)
                       : launch_compress<0>(out_dtype, total, st, k, v, logits, B, ne, ld_in, m, k_out, v_out,
                                            k_scale_out, v_scale_out, ld_out);
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}

// New entries of several sequences in one launch (a mixed decode/prefill
// step): entry j of sequence b pools its rows row0[b] + j*m .. into slot
// entry0[b] + j, exactly as csa_compress_kv pools a block.
extern "C" csa_status_t csa_compress_kv_varlen(const void* k, const void* v, int32_t in_dtype, const float* logits,
                                               int32_t B, int32_t ld_in, int32_t d, int32_t m,
                                               const int32_t* cu_entries, const int32_t* row0,
                                               const int32_t* entry0, int32_t n_entries, void* k_out, void* v_out,
                                               float* k_scale_out, float* v_scale_out, int32_t ld_out,
                                               int32_t out_dtype, void* stream) {
  const CompressArgs ca{k, v, logits, in_dtype, B, 0, ld_in, m, ld_out, out_dtype, k_out, v_out, k_scale_out, v_scale_out};
  const csa_status_t chk = check_compress_args(ca, d);
  if (chk != CSA_OK) return chk;
  if (n_entries < 0 || ld_in < m || ld_out < 1) return CSA_EINVAL;
  if (n_entries == 0) return CSA_OK;
  if (B < 1 || !cu_entries || !row0 || !entry0) return CSA_EINVAL;
  const PackedEntries pk{cu_entries, row0, entry0, B};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = in_dtype == CSA_F32
                       ? launch_compress<1>(out_dtype, n_entries, st, k, v, logits, 1, n_entries, ld_in, m, k_out,
                                            v_out, k_scale_out, v_scale_out, ld_out, pk)
                       : launch_compress<0>(out_dtype, n_entries, st, k, v, logits, 1, n_entries, ld_in, m, k_out,
                                            v_out, k_scale_out, v_scale_out, ld_out, pk);
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}
