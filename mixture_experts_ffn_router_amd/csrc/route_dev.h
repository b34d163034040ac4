// Per-token routing on one wavefront, shared by the routing kernel and the
// decode kernels (which recompute the routing of their few tokens in every
// block).  See route.hip for the method and its sources.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// One token's routing on one wavefront: lane k < K ends with slot k's weight
// and expert id.  z points at the token's E logits; load_logits / route_logits
// split the load from the arithmetic so a caller can issue several tokens'
// loads at once.
// The logits a lane holds: experts lane, lane + 64, ... (0 past E).
template <int VPL>
struct TokenLogits {
  float v[VPL];
};
template <int VPL>
__device__ __forceinline__ TokenLogits<VPL> load_logits(const float* __restrict__ z, int E, int lane) {
  TokenLogits<VPL> r;
#pragma unroll
  for (int j = 0; j < VPL; ++j) r.v[j] = lane + 64 * j < E ? z[lane + 64 * j] : 0.f;
  return r;
}

// Group-limited routing (llama.cpp MoE lesson: experts split into groups, groups
// picked first): the experts form G equal contiguous ranges; a range's score is
// its largest key (the same order as its largest logit or probability).  The KG
// best ranges are picked, ties to the lower range, and every other expert's key
// is cleared to 0, below every real key, so the top-k never takes it while K is
// at most the number of experts in the picked ranges.
template <int VPL>
__device__ __forceinline__ void mask_groups(uint32_t (&key)[VPL], int E, int G, int KG, int lane) {
  const int gsz = E / G;
  uint32_t gkey = 0u;  // lane g < G: the best key of range g
  for (int g = 0; g < G; ++g) {
    uint32_t b = 0u;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int idx = lane + 64 * j;
      if (idx < E && idx / gsz == g && key[j] > b) b = key[j];
    }
    b = wave_max_u32(b);
    if (lane == g) gkey = b;
  }
  uint64_t picked = 0;  // the same on every lane
  for (int r = 0; r < KG; ++r) {
    const bool open = lane < G && !((picked >> lane) & 1ull);
    const uint32_t c = open ? gkey : 0u;
    const uint32_t gk = wave_max_u32(c);
    const uint32_t gi = wave_min_u32(open && c == gk ? (uint32_t)lane : 0xFFFFFFFFu);
    picked |= 1ull << gi;
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int idx = lane + 64 * j;
    if (idx < E && !((picked >> (idx / gsz)) & 1ull)) key[j] = 0u;
  }
}

template <int VPL>
__device__ __forceinline__ void route_logits(const TokenLogits<VPL>& zl, int E, int K, const RouteOpts& o,
                                             const float* __restrict__ pes, int lane, float& w_slot,
                                             int& id_slot) {
  float v[VPL];
  uint32_t key[VPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    int idx = lane + 64 * j;
    v[j] = zl.v[j];
    if (idx < E) {
      key[j] = f32_order_key(v[j]);
      lmax = fmaxf(lmax, v[j]);
    } else {
      key[j] = 0u;  // below every finite key: never selected while K <= E
    }
  }
  if (o.groups > 1) mask_groups<VPL>(key, E, o.groups, o.topk_groups, lane);
  const bool sigmoid = o.scoring == SCORE_SIGMOID;
  const float m = sigmoid ? 0.f : wave_max_f32(lmax);

  double s_all = 1.0;  // softmax without renormalisation: the sum over all E
  if (!o.renorm && !sigmoid) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) s += (double)expf(v[j] - m);
    s_all = wave_sum_f64(s);
  }

  uint32_t taken = 0;  // bit j: this lane's value j already selected
  double my_e = 0.0;
  int my_id = 0;
  double denom = 0.0;
  for (int k = 0; k < K; ++k) {
    uint32_t bk = 0, bi = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (!((taken >> j) & 1u) && key[j] > bk) {  // j ascending: lowest index wins ties
        bk = key[j];
        bi = (uint32_t)(lane + 64 * j);
      }
    }
    const uint32_t gk = wave_max_u32(bk);
    const uint32_t gi = wave_min_u32(bk == gk ? bi : 0xFFFFFFFFu);
    if ((int)(gi & 63u) == lane) taken |= 1u << (gi >> 6);
    const float zk = f32_from_order_key(gk);
    // softmax: fp32 exp(z - max); sigmoid: 1 / (1 + exp(-z)) in fp64
    const double e = sigmoid ? 1.0 / (1.0 + exp(-(double)zk)) : (double)expf(zk - m);
    denom += e;  // slot order
    if (lane == k) {
      my_e = e;
      my_id = (int)gi;
    }
  }
  w_slot = 0.f;
  id_slot = 0;
  if (lane < K) {
    const double d = o.renorm ? (denom > 0.0 ? denom : 1.0) : s_all;
    double w = my_e / d;
    if (pes) w *= (double)pes[my_id];
    w_slot = (float)w;
    id_slot = my_id;
  }
}

}  // namespace moe
