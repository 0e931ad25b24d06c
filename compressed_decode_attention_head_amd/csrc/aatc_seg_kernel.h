// Merge kernel of multi-segment decode attention (gfx950).
//
// Page "SPHERICAL KV ..." (RDKV abstract): after prefill each token is kept uncompressed,
// coded at some width, or evicted.  Here a KV head's tokens are split into segments by tier --
// coded segments (their own packed caches and bit allocations) and a raw bf16 segment in the
// original basis; evicted tokens are in none.  One softmax runs over the union: softmax is
// invariant to token order, so each segment (or split of one) yields a normalised output
// and its log-sum-exp, and the states merge exactly as split-softmax partials do.  Raw
// segments are handled by the dense kernel (aatc_dense_kernel.h).
//
// k_merge_states: grid (batch * n_q), MW waves; merges n_states states per q head.  Wave w takes
// states w, w + MW, ..., MU of them per round (one round up to MW * MU states), keeps its own
// running max, sum and output, and the waves combine at the end the same way.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_seg {

constexpr int D = AATC_D;
constexpr int MW = 16;                   // waves of the merge kernel
constexpr int MU = 8;                    // states in flight per wave and round

// out = sum_s w_s out_s, w_s = exp(lse_s - lse), lse = ln sum_s exp(lse_s).  A state with
// lse = -inf has no tokens; no state with tokens gives out = 0, lse = -inf; a NaN state
// poisons its q head.
__global__ __launch_bounds__(MW * 64) void k_merge_states(const float* __restrict__ out_states,
                                                         const float* __restrict__ lse_states, int n_states,
                                                         int64_t bq, float* out, float* lse) {
  __shared__ float sm[MW], sl[MW];
  __shared__ int sn[MW];
  __shared__ float2 so[MW][64];
  const int64_t qh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float mw = -INFINITY, lw = 0.f;
  float2 o = make_float2(0.f, 0.f);
  int nan = 0;
  // lane holds channels 2 lane, 2 lane + 1; every lane reads the same lse values
  for (int s0 = wave; s0 < n_states; s0 += MW * MU) {
    float l[MU];
    float2 x[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int s = s0 + u * MW;
      l[u] = s < n_states ? lse_states[s * bq + qh] : -INFINITY;
      x[u] = s < n_states ? reinterpret_cast<const float2*>(out_states + (s * bq + qh) * D)[lane]
                          : make_float2(0.f, 0.f);
    }
    float mr = mw;
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      nan |= l[u] != l[u];
      mr = fmaxf(mr, l[u]);
    }
    if (mr != -INFINITY) {
      const float f = mw == -INFINITY ? 0.f : expf(mw - mr);
      lw *= f;
      o.x *= f;
      o.y *= f;
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const float w = l[u] == -INFINITY ? 0.f : expf(l[u] - mr);
        lw += w;
        o.x = fmaf(w, x[u].x, o.x);
        o.y = fmaf(w, x[u].y, o.y);
      }
      mw = mr;
    }
  }
  so[wave][lane] = o;
  if (lane == 0) {
    sm[wave] = mw;
    sl[wave] = lw;
    sn[wave] = nan;
  }
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
    for (int w = 0; w < MW; ++w) {
      M = fmaxf(M, sm[w]);
      nan |= sn[w];
    }
    float L = 0.f;
    o = make_float2(0.f, 0.f);
    if (M != -INFINITY) {
      for (int w = 0; w < MW; ++w) {
        if (sm[w] == -INFINITY) continue;
        const float f = expf(sm[w] - M);
        L = fmaf(sl[w], f, L);
        o.x = fmaf(so[w][lane].x, f, o.x);
        o.y = fmaf(so[w][lane].y, f, o.y);
      }
    }
    const float2 r = nan ? make_float2(NAN, NAN) : (L > 0.f ? make_float2(o.x / L, o.y / L) : make_float2(0.f, 0.f));
    reinterpret_cast<float2*>(out + qh * D)[lane] = r;
    if (lse && lane == 0) lse[qh] = nan ? NAN : (L > 0.f ? M + logf(L) : -INFINITY);
  }
}

}  // namespace aatc_seg
