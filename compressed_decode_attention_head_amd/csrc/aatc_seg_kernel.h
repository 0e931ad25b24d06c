// Kernels of multi-segment decode attention (gfx950).
//
// Page "SPHERICAL KV ..." (RDKV abstract): after prefill every token gets a bit width from
// full precision down to zero.  Here a KV head's tokens are split into segments by tier --
// coded segments (their own packed caches and bit allocations) and a raw bf16 segment in the
// original basis; evicted tokens are in none.  One softmax runs over the union: softmax is
// invariant to token order, so each segment (or split of one) yields a normalised output
// and its log-sum-exp, and the states merge exactly as split-softmax partials do.
//
// k_raw_attn: grid (token chunks of RCH, KV heads, batch), RCH threads; one state per q head
//   and chunk: out_s = sum_t p_t v_t / sum_t p_t and lse_s = ln sum_t exp(s_t).
// k_merge_states: grid (batch * n_q), D threads; merges n_states states per q head.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_seg {

constexpr int D = AATC_D;
constexpr int RCH = 256;                 // tokens per workgroup of the raw kernel (one per thread)
constexpr int MAXG = AATC_MAX_GROUP;

struct RawArgs {
  const uint16_t* k;                     // bf16 [batch][n_kv][cap][128]
  const uint16_t* v;
  int64_t cap;
  const int32_t* seq_lens;               // [batch][n_kv], or null: max_seq
  int64_t max_seq;
  const float* q;                        // fp32 [batch][n_q][128]
  int n_kv, n_q, group;
  float scale2;                          // softmax scale * log2(e)
  float* out_states;                     // [n_states][batch * n_q][128]
  float* lse_states;                     // [n_states][batch * n_q]
  int state0;                            // state index of chunk 0
  int64_t bq;                            // batch * n_q
};

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline float wmax(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ inline float wsum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__global__ __launch_bounds__(RCH) void k_raw_attn(RawArgs a) {
  __shared__ float qs[MAXG][D];
  __shared__ float ps[MAXG][RCH];
  __shared__ float red[MAXG][RCH / 64];
  __shared__ float mh[MAXG], lh[MAXG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int64_t bh = static_cast<int64_t>(b) * a.n_kv + h;
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[bh]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);
  const int64_t t0 = static_cast<int64_t>(c) * RCH;
  const int nt = seq - t0 <= 0 ? 0 : (seq - t0 < RCH ? static_cast<int>(seq - t0) : RCH);
  const float* qg = a.q + (static_cast<int64_t>(b) * a.n_q + static_cast<int64_t>(h) * G) * D;
  for (int e = tid; e < MAXG * D; e += RCH) qs[e / D][e % D] = e < G * D ? qg[e] : 0.f;
  __syncthreads();

  // scores: thread tid = token t0 + tid
  float s[MAXG];
#pragma unroll
  for (int g = 0; g < MAXG; ++g) s[g] = 0.f;
  if (tid < nt) {
    const uint4* kr = reinterpret_cast<const uint4*>(a.k + (bh * a.cap + t0 + tid) * D);
#pragma unroll 4
    for (int u = 0; u < D / 8; ++u) {
      const uint4 w = kr[u];
      const float kv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int g = 0; g < MAXG; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) s[g] = fmaf(qs[g][8 * u + j], kv[j], s[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    const float sc = tid < nt ? s[g] * a.scale2 : -INFINITY;
    s[g] = sc;
    const float m = wmax(sc);
    if (lane == 0) red[g][wave] = m;
  }
  __syncthreads();
  if (tid < MAXG) {
    float m = -INFINITY;
    for (int w = 0; w < RCH / 64; ++w) m = fmaxf(m, red[tid][w]);
    mh[tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    const float p = (tid < nt) ? exp2f(s[g] - mh[g]) : 0.f;
    ps[g][tid] = p;
    const float l = wsum(p);
    if (lane == 0) red[g][wave] = l;
  }
  __syncthreads();
  if (tid < MAXG) {
    float l = 0.f;
    for (int w = 0; w < RCH / 64; ++w) l += red[tid][w];
    lh[tid] = l;
  }
  __syncthreads();

  // PV: thread = channel j (two threads per channel, each half of the heads)
  const int j = tid & (D - 1), hs = tid / D;
  float acc[MAXG / 2];
#pragma unroll
  for (int r = 0; r < MAXG / 2; ++r) acc[r] = 0.f;
  const uint16_t* vr = a.v + (bh * a.cap + t0) * D + j;
  for (int t = 0; t < nt; ++t) {
    const float vv = __uint_as_float(static_cast<uint32_t>(vr[static_cast<int64_t>(t) * D]) << 16);
#pragma unroll
    for (int r = 0; r < MAXG / 2; ++r) acc[r] = fmaf(ps[hs + 2 * r][t], vv, acc[r]);
  }
  const int st = a.state0 + c;
#pragma unroll
  for (int r = 0; r < MAXG / 2; ++r) {
    const int g = hs + 2 * r;
    if (g < G) {
      const int64_t qh = static_cast<int64_t>(b) * a.n_q + static_cast<int64_t>(h) * G + g;
      const float l = lh[g];
      a.out_states[(static_cast<int64_t>(st) * a.bq + qh) * D + j] = l > 0.f ? acc[r] / l : 0.f;
      if (j == 0)
        a.lse_states[static_cast<int64_t>(st) * a.bq + qh] =
            l > 0.f ? (mh[g] + log2f(l)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

// out = sum_s w_s out_s, w_s = exp(lse_s - lse), lse = ln sum_s exp(lse_s).  A state with
// lse = -inf has no tokens; no state with tokens gives out = 0, lse = -inf; a NaN state
// poisons its q head.
__global__ __launch_bounds__(D) void k_merge_states(const float* __restrict__ out_states,
                                                    const float* __restrict__ lse_states, int n_states, int64_t bq,
                                                    float* out, float* lse) {
  const int64_t qh = blockIdx.x;
  const int j = threadIdx.x;
  float M = -INFINITY;
  bool nan = false;
  for (int s = 0; s < n_states; ++s) {
    const float l = lse_states[s * bq + qh];
    nan |= l != l;
    M = fmaxf(M, l);
  }
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_states; ++s) {
      const float l = lse_states[s * bq + qh];
      if (l == -INFINITY) continue;
      const float w = expf(l - M);
      L += w;
      o = fmaf(w, out_states[(s * bq + qh) * D + j], o);
    }
  }
  out[qh * D + j] = nan ? NAN : (L > 0.f ? o / L : 0.f);
  if (lse && j == 0) lse[qh] = nan ? NAN : (L > 0.f ? M + logf(L) : -INFINITY);
}

}  // namespace aatc_seg
