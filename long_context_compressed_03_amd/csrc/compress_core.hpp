// Softmax-pool compression of short blocks (m < 32), one entry per 16-lane
// group: shared by the compression kernels and by the launch that runs the
// compression beside the decode indexer pass.
//
// The pages (blog.nickys.cn DeepSeek-V4 post, 三大架构改动 §1 CSA and §2 HCA)
// state that every m (resp. m') tokens' K/V become one entry; the pooling rule
// (softmax weights from one logit per token, shared by K and V) is this
// library's reading.
#pragma once
#include "common.hpp"

namespace csa_cmp {

constexpr int kGroup = 16;            // lanes per entry
constexpr int kColsPerLane = 8;       // 16 lanes x 8 = 128 head columns

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

// The entry pooled from rows [row0, row0 + m) (and their logits) into
// output slot `entry`, by the 16-lane group whose lane lane_c owns head
// columns [8 lane_c, 8 lane_c + 8); rows are walked with 4 loads in flight
// per lane for each of K and V.  kNewest: the block's last row and logit
// are read from k_new, v_new, z_new instead (the cache append pools a block
// whose newest token it is writing in the same launch).
template <int kInF32, int kOut, bool kNewest = false>
CSA_DEV void compress_group_at(const void* __restrict__ k, const void* __restrict__ v,
                               const float* __restrict__ logits, size_t row0, int m, void* k_out, void* v_out,
                               float* k_scale, float* v_scale, size_t entry, int lane_c,
                               const void* k_new = nullptr, const void* v_new = nullptr,
                               const float* z_new = nullptr) {
  const float* z = logits + row0;
  // row j of the block (address selected, no branch around the load)
  auto krow = [&](int jj, float* out) {
    if constexpr (kNewest) {
      const bool nw = jj == m - 1;
      load_row8<kInF32>(nw ? k_new : k, nw ? size_t(0) : row0 + jj, lane_c, out);
    } else {
      load_row8<kInF32>(k, row0 + jj, lane_c, out);
    }
  };
  auto vrow = [&](int jj, float* out) {
    if constexpr (kNewest) {
      const bool nw = jj == m - 1;
      load_row8<kInF32>(nw ? v_new : v, nw ? size_t(0) : row0 + jj, lane_c, out);
    } else {
      load_row8<kInF32>(v, row0 + jj, lane_c, out);
    }
  };
  auto zat = [&](int x) -> float {
    if constexpr (kNewest) return *(x == m - 1 ? z_new : z + x);
    else return z[x];
  };

  // softmax statistics of the block's logits, spread over the 16 lanes;
  // computed after the first rows are requested, so the two memory round
  // trips overlap
  float zmax = 0.f, inv = 0.f;
  auto stats = [&]() {
    zmax = -INFINITY;
    for (int x = lane_c; x < m; x += kGroup) zmax = fmaxf(zmax, zat(x));
    zmax = group_max<kGroup>(zmax);
    float zsum = 0.f;
    for (int x = lane_c; x < m; x += kGroup) zsum += expf(zat(x) - zmax);
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
      krow(j + u, kr[u]);
      vrow(j + u, vr[u]);
    }
    if (j == 0) stats();
#pragma unroll
    for (int u = 0; u < kU; ++u) a[u] = expf(zat(j + u) - zmax) * inv;
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
    krow(j, kr);
    vrow(j, vr);
    const float a = expf(zat(j) - zmax) * inv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ak[i] = fmaf(a, kr[i], ak[i]);
      av[i] = fmaf(a, vr[i], av[i]);
    }
  }
  store_entry<kOut>(k_out, k_scale, entry, lane_c, ak);
  store_entry<kOut>(v_out, v_scale, entry, lane_c, av);
}

// Entry gid (< B * n_entries): sequence b's block e, rows b * ld_in + e * m.
template <int kInF32, int kOut>
CSA_DEV void compress_group(const void* __restrict__ k, const void* __restrict__ v, const float* __restrict__ logits,
                            int n_entries, int ld_in, int m, void* k_out, void* v_out, float* k_scale, float* v_scale,
                            int ld_out, long gid, int lane_c) {
  const int b = int(gid / n_entries);
  const int e = int(gid - long(b) * n_entries);
  compress_group_at<kInF32, kOut>(k, v, logits, size_t(b) * ld_in + size_t(e) * m, m, k_out, v_out, k_scale, v_scale,
                                  size_t(b) * ld_out + e, lane_c);
}

// Packed new entries of several sequences (csa_compress_kv_varlen): sequence
// b's entries are items cu[b] .. cu[b + 1] - 1; its j-th pools raw rows
// row0[b] + j*m .. of that sequence into entry entry0[b] + j.  cu == nullptr:
// the plain layout (B sequences of n_entries entries from row 0 / entry 0).
struct PackedEntries {
  const int32_t* cu;
  const int32_t* row0;
  const int32_t* entry0;
  int B;
};

// Raw row of the block and output slot of packed entry gid.
CSA_DEV void packed_entry(const PackedEntries& p, int gid, int ld_in, int m, int ld_out, size_t* row,
                          size_t* entry) {
  const int b = csa_packed_seq(p.cu, p.B, gid);
  const int j = gid - p.cu[b];
  *row = size_t(b) * ld_in + size_t(p.row0[b]) + size_t(j) * m;
  *entry = size_t(b) * ld_out + size_t(p.entry0[b]) + j;
}

// One decode token per sequence into the mirrored window ring, and the pool
// of a block it completes (the cache append; see cache.hip for the layout).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const float* z_new;
  const int32_t* pos;
  void* k_ring;
  void* v_ring;
  float* z_ring;
  int32_t* raw_pos0;
  int B, L, m, cap;
  void* ck;
  void* cv;
  float* ck_scale;
  float* cv_scale;
};

// Where sequence b's token at p goes and what it completes.
struct AppendPlan {
  bool done;       // a block ends at p and its entry is below the capacity
  int entry;       // (p + 1) / m - 1
  int first_row;   // ring row of the block's first token: (p - m + 1) mod L
  int base;        // window base for a query at p
};

CSA_DEV AppendPlan append_plan(int p, int L, int m, int cap) {
  AppendPlan a;
  a.done = p >= 0 && (p + 1) % m == 0 && (p + 1) / m - 1 < cap;
  a.entry = (p + 1) / m - 1;
  a.first_row = a.done ? (p - m + 1) % L : 0;
  const int q0 = max(0, p - L + 1);
  a.base = p >= 0 ? q0 - q0 % L : 0;
  return a;
}

hipError_t launch_cache_append(int io_dtype, int ckv_dtype, const AppendArgs& a, hipStream_t st);

// Cache append, short blocks (m < 32), for block `blk` of 64 threads:
// 16-lane group g serves sequence 4 * blk + g.  It writes the token's K/V rows
// (both ring copies; lane c its 8 columns) and logit, the window base, and
// pools the block the token completes with its newest row read from the input
// (the ring rows it reads hold older tokens, never the two rows being written).
template <int kInF32, int kOut>
CSA_DEV void cache_append_short_at(const AppendArgs& a, int blk) {
  const int lane_c = threadIdx.x & (kGroup - 1);
  const int b = blk * 4 + int(threadIdx.x / kGroup);
  if (b >= a.B) return;                    // whole 16-lane groups leave together
  const int p = a.pos[b];
  const AppendPlan pl = append_plan(p, a.L, a.m, a.cap);
  constexpr int kEl = kInF32 ? 4 : 2;
  constexpr int kLaneBytes = kColsPerLane * kEl;
  const size_t ring0 = size_t(b) * 2 * a.L;
  const uint8_t* kn = static_cast<const uint8_t*>(a.k_new) + size_t(b) * kHeadDim * kEl;
  const uint8_t* vn = static_cast<const uint8_t*>(a.v_new) + size_t(b) * kHeadDim * kEl;
  if (p >= 0) {
    const int s = p % a.L;
#pragma unroll
    for (int h = 0; h < kLaneBytes / 16; ++h) {
      const uint4 xk = *reinterpret_cast<const uint4*>(kn + lane_c * kLaneBytes + h * 16);
      const uint4 xv = *reinterpret_cast<const uint4*>(vn + lane_c * kLaneBytes + h * 16);
#pragma unroll
      for (int copy = 0; copy < 2; ++copy) {
        const size_t off = (ring0 + s + size_t(copy) * a.L) * kHeadDim * kEl + lane_c * kLaneBytes + h * 16;
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.k_ring) + off) = xk;
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.v_ring) + off) = xv;
      }
    }
    if (lane_c < 2) a.z_ring[ring0 + s + size_t(lane_c) * a.L] = a.z_new[b];
  }
  if (lane_c == 0) a.raw_pos0[b] = pl.base;
  if (!pl.done) return;
  compress_group_at<kInF32, kOut, true>(a.k_ring, a.v_ring, a.z_ring, ring0 + pl.first_row, a.m, a.ck, a.cv,
                                        a.ck_scale, a.cv_scale, size_t(b) * a.cap + pl.entry, lane_c, kn, vn,
                                        a.z_new + b);
}

// The arguments of one compression call.
struct CompressArgs {
  const void* k;
  const void* v;
  const float* logits;
  int in_dtype, B, L, ld_in, m, ld_out, out_dtype;
  void* k_out;
  void* v_out;
  float* k_scale;
  float* v_scale;
};

inline csa_status_t check_compress_args(const CompressArgs& c, int d) {
  if (!c.k || !c.v || !c.logits || !c.k_out || !c.v_out) return CSA_EINVAL;
  if (c.in_dtype != CSA_BF16 && c.in_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(c.out_dtype)) return CSA_EINVAL;
  if (d != kHeadDim || c.m < 1 || c.B < 0 || c.L < 0 || c.L % c.m != 0 || c.ld_in < c.L) return CSA_EINVAL;
  if (c.ld_out < c.L / c.m) return CSA_EINVAL;
  if (c.out_dtype == CSA_FP8_E4M3 && (!c.k_scale || !c.v_scale)) return CSA_EINVAL;
  if (long(c.B) * (c.L / c.m) > 0x7FFFFFFFL) return CSA_EINVAL;
  return CSA_OK;
}

}  // namespace csa_cmp
