// Per-token routing on one wavefront, shared by the routing kernel and the
// decode kernels (which recompute the routing of their few tokens in every
// block).  See route.hip for the method and its sources.
#pragma once

#include "common.h"

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

template <int VPL>
__device__ __forceinline__ void route_logits(const TokenLogits<VPL>& zl, int E, int K, int renorm,
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
  const float m = wave_max_f32(lmax);

  double s_all = 1.0;
  if (!renorm) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < E) s += (double)expf(v[j] - m);
    s_all = wave_sum_f64(s);
  }

  uint32_t taken = 0;  // bit j: this lane's value j already selected
  float my_e = 0.f;
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
    const float e = expf(f32_from_order_key(gk) - m);
    denom += (double)e;  // slot order
    if (lane == k) {
      my_e = e;
      my_id = (int)gi;
    }
  }
  w_slot = 0.f;
  id_slot = 0;
  if (lane < K) {
    const double d = renorm ? (denom > 0.0 ? denom : 1.0) : s_all;
    double w = (double)my_e / d;
    if (pes) w *= (double)pes[my_id];
    w_slot = (float)w;
    id_slot = my_id;
  }
}

template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ z, int E, int K, int renorm,
                                            const float* __restrict__ pes, int lane, float& w_slot,
                                            int& id_slot) {
  route_logits<VPL>(load_logits<VPL>(z, E, lane), E, K, renorm, pes, lane, w_slot, id_slot);
}

}  // namespace moe
