// Block-wide selection helpers shared by the top-k kernels (1024-thread
// blocks): bucket search over an LDS histogram, block AND/OR, and an exact
// radix refinement over any set of order-preserving uint32 keys.
#pragma once
#include "common.hpp"

namespace csa_sel {

constexpr int kThreads = 1024;

struct Sel {
  uint32_t bin, remaining, bincount;
};

// Order-preserving uint32 key of an fp32 score: negative values bit-inverted,
// non-negative ones with the sign bit set, -0 folded onto +0.  Larger score
// <=> larger key; no finite or infinite score maps to 0.
CSA_DEV uint32_t ordered_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The whole block finds, among nb bins counted from the top, the bin where
// the running count first reaches `remaining`: thread t sums the nb/1024 bins
// t*per .. from the top (a short stride, so its 16-byte LDS reads spread over
// the banks), one block scan places the crossing inside one thread's range.
// Every thread must call it; the result lands in *out.
CSA_DEV void find_bin(const uint32_t* hist, int nb, uint32_t remaining, Sel* out, uint32_t* smem) {
  const int tid = threadIdx.x;
  const int per = nb > kThreads ? nb / kThreads : 1;
  const int lo = tid * per;                    // bins nb-1-lo ... nb-per-lo (descending)
  uint32_t mine = 0u;
  if (lo < nb) {
    if (per >= 4) {
      const u32x4* h4 = reinterpret_cast<const u32x4*>(hist + (nb - lo - per));
      for (int x = 0; x < per / 4; ++x) {
        const u32x4 v = h4[x];
        mine += v[0] + v[1] + v[2] + v[3];
      }
    } else {
      for (int x = 0; x < per; ++x) mine += hist[nb - 1 - (lo + x)];
    }
  }
  uint32_t tot;
  const uint32_t excl = block_exclusive_scan(mine, smem, &tot);
  if (lo < nb && excl < remaining && remaining <= excl + mine) {
    uint32_t run = excl;
    for (int x = 0; x < per; ++x) {
      const int bin = nb - 1 - (lo + x);
      const uint32_t c = hist[bin];
      if (run < remaining && remaining <= run + c) {
        out->bin = uint32_t(bin);
        out->remaining = remaining - run;
        out->bincount = c;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

CSA_DEV void block_and_or(uint32_t& a, uint32_t& b, uint32_t* smem) {
  for (int o = 32; o > 0; o >>= 1) {
    a &= __shfl_xor(a, o);
    b |= __shfl_xor(b, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { smem[w] = a; smem[16 + w] = b; }
  __syncthreads();
  a = smem[0];
  b = smem[16];
  for (int x = 1; x < kThreads / 64; ++x) { a &= smem[x]; b |= smem[16 + x]; }
  __syncthreads();
}

// Exact radix refinement of (prefix, mask) over a set of keys visited by
// `each(fn)` (fn is called for every key of the set, in any order, on every
// thread; 0 = absent).  On entry the set's keys all match (key & mask) ==
// prefix and `remaining` of them are wanted from the top; on return (prefix,
// mask) select the k-th key and `remaining` counts the keys equal to it that
// are still needed.
template <typename Each, typename Sh>
CSA_DEV void refine(Each each, uint32_t& prefix, uint32_t& mask, uint32_t& remaining, Sh& sh) {
  const int tid = threadIdx.x;
  uint32_t k_and = 0xFFFFFFFFu, k_or = 0u;
  each([&](uint32_t kk) {
    if (kk != 0u && (kk & mask) == prefix) { k_and &= kk; k_or |= kk; }
  });
  block_and_or(k_and, k_or, sh.smem);
  if (k_or == 0u) return;
  const int common = (k_and ^ k_or) == 0u ? 32 : __clz(k_and ^ k_or);
  mask = common == 0 ? 0u : (common == 32 ? 0xFFFFFFFFu : ~(0xFFFFFFFFu >> common));
  prefix = k_and & mask;
  int bits_left = 32 - common;
  while (bits_left > 0) {
    const int width = bits_left < 11 ? bits_left : 11;
    const int shift = bits_left - width;
    const int nb = 1 << width;
    bits_left = shift;
    for (int j = tid; j < nb; j += kThreads) sh.hist[j] = 0u;
    __syncthreads();
    const uint32_t pm = prefix, mm = mask;
    each([&](uint32_t kk) {
      if (kk != 0u && (kk & mm) == pm) atomicAdd(&sh.hist[(kk >> shift) & uint32_t(nb - 1)], 1u);
    });
    __syncthreads();
    find_bin(sh.hist, nb, remaining, &sh.sel, sh.smem);
    prefix |= sh.sel.bin << shift;
    mask |= uint32_t(nb - 1) << shift;
    remaining = sh.sel.remaining;
    const bool done = sh.sel.bincount == remaining;   // the bin is taken whole
    __syncthreads();
    if (done) break;
  }
}

}  // namespace csa_sel
