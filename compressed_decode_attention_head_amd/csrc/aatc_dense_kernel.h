// Dense bf16 decode attention on the matrix cores (gfx950), the full-cache comparator of the
// compressed path and the kernel of raw bf16 token segments.
//
// Page "SPHERICAL KV ..." (RDKV abstract): the compressed cache is compared with the
// full-precision one, which every decode step reads from HBM again.  This is that step for a bf16
// cache [batch][n_kv][capacity][128]: each workgroup takes a chunk of consecutive tokens of one
// (batch, KV head) -- CHUNK, or a power-of-two fraction of it for short segments -- and all q heads of its GQA group, and writes one split-softmax state per q
// head (normalised output and log-sum-exp); k_merge_states merges the states.
//
// One wave handles 32 tokens per step on v_mfma_f32_16x16x32_bf16:
//  * scores: S^T[t][g] = sum_d K[t][d] q[g][d] with K as the A operand (row = token) and the
//    scaled query as B (column = q head, 16 columns of which the group uses up to 8).  The
//    contraction index d is paired arbitrarily between the operands, so each lane reads the
//    64 bytes of its token's row that suit it: d = 32 kk + 8 (lane / 16) + 0..7 in step kk.
//  * the query is fp32; it enters as a bf16 high part plus a bf16 low part (two MFMAs), so the
//    scores carry about 16 mantissa bits of q; K is exact in bf16.
//  * values: O^T[c][g] = sum_t V[t][c] P[g][t] with V^T as the A operand (row = channel) and
//    P^T as B.  The token order of the contraction is free, so it is the order in which the
//    score MFMAs left the probabilities in each lane: no cross-lane move.  The channel of row
//    m in value MFMA j is 8 m + j, so a lane reads 16 contiguous bytes (channels 8m..8m+7) of
//    each of its 8 tokens and regroups them in registers (one byte permute per dword).
//  * P also enters as bf16 high plus low parts; the running max and sum are fp32.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_dense {

constexpr int D = AATC_D;
constexpr int NW = 8;                      // waves per workgroup
constexpr int CHUNK = 2048;                // longest token chunk per workgroup (one state per q head)
constexpr int MIN_CHUNK = NW * 32;         // one 32-token block per wave
constexpr int MAXG = AATC_MAX_GROUP;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct DenseArgs {
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
  int chunk;                             // tokens per workgroup: MIN_CHUNK * 2^i <= CHUNK
  int64_t bq;                            // batch * n_q
};

// bf16 of x, round to nearest even (finite x)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// Splits 8 fp32 values into bf16 high and low parts packed two per dword.
__device__ inline void split8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = bf16_rne(x[i]);
    l[i] = bf16_rne(x[i] - bf16_val(h[i]));
  }
  hi = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
  lo = make_uint4(l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16);
}

__device__ inline f4 mfma(const uint4& a, const uint4& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Value of lane ^ 16 / lane ^ 32 (permlane swaps, no LDS).
__device__ inline float xor16(float x, int lane) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float((lane & 16) ? p[0] : p[1]);
}
__device__ inline float xor32(float x, int lane) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(lane < 32 ? p[1] : p[0]);
}

// dword of 16-bit element `j` (even: low halves, odd: high halves) of x and y, x low
__device__ inline uint32_t pick(uint32_t x, uint32_t y, int odd) {
  return __builtin_amdgcn_perm(y, x, odd ? 0x07060302u : 0x05040100u);
}

__device__ inline uint32_t word(const uint4& u, int i) { return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w; }

// Two waves per SIMD: the registers hold two 32-token blocks per wave (one computing, one in
// flight), 32 KB of loads per wave.
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_dense_attn(DenseArgs a) {
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float4 sm_acc[NW][MAXG][D / 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int g = lane & 15, qq = lane >> 4;
  const int64_t bh = static_cast<int64_t>(b) * a.n_kv + h;
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[bh]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);
  const int64_t t_begin = static_cast<int64_t>(c) * a.chunk;
  const int nt = seq - t_begin <= 0 ? 0 : (seq - t_begin < a.chunk ? static_cast<int>(seq - t_begin) : a.chunk);

  // query operand: column g, contraction d = 32 kk + 8 qq + 0..7, scaled, split hi + lo
  uint4 qh[4], ql[4];
  {
    const int gq = g < G ? g : 0;
    const float* qr = a.q + (static_cast<int64_t>(b) * a.n_q + static_cast<int64_t>(h) * G + gq) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float4 x0 = *reinterpret_cast<const float4*>(qr + 32 * kk + 8 * qq);
      const float4 x1 = *reinterpret_cast<const float4*>(qr + 32 * kk + 8 * qq + 4);
      const float s = g < G ? a.scale2 : 0.f;
      const float x[8] = {x0.x * s, x0.y * s, x0.z * s, x0.w * s, x1.x * s, x1.y * s, x1.z * s, x1.w * s};
      split8(x, qh[kk], ql[kk]);
    }
  }

  f4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int nb = (nt + 31) >> 5;
  const uint16_t* kb = a.k + bh * a.cap * D;
  const uint16_t* vb = a.v + bh * a.cap * D;
  const int64_t last = seq - 1;
  // K: token tb + 16 h2 + g, 64 bytes at d = 32 kk + 8 qq; V: token tb + 16 (e / 4) + 4 qq + e % 4,
  // channels 8 g .. 8 g + 7.  Tokens past the end read the last one (their weight is 0).
  auto load = [&](int blk, uint4 (&kv)[2][4], uint4 (&vv)[8]) {
    const int64_t tb = t_begin + 32 * blk;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      int64_t t = tb + 16 * h2 + g;
      t = t < last ? t : last;
      const uint4* row = reinterpret_cast<const uint4*>(kb + t * D);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kv[h2][kk] = row[4 * kk + qq];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t t = tb + 16 * (e >> 2) + 4 * qq + (e & 3);
      t = t < last ? t : last;
      vv[e] = reinterpret_cast<const uint4*>(vb + t * D)[g];
    }
  };
  auto step = [&](int blk, const uint4 (&kv)[2][4], const uint4 (&vv)[8]) {
    // scores in log2 units: lane holds tokens 16 h2 + 4 qq + i of q head g
    float s[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc = mfma(kv[h2][kk], qh[kk], sc);
        sc = mfma(kv[h2][kk], ql[kk], sc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rel = 32 * blk + 16 * h2 + 4 * qq + i;
        s[4 * h2 + i] = rel < nt ? sc[i] : -INFINITY;
      }
    }
    float bm = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, s[e]);
    bm = fmaxf(bm, xor16(bm, lane));
    bm = fmaxf(bm, xor32(bm, lane));
    const float m_new = fmaxf(m_run, bm);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
      const float al = exp2f(m_run - m_new);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= al;
      l_run *= al;
      m_run = m_new;
    }
    float p[8];
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(s[e] - m_run);
      ls += p[e];
    }
    l_run += ls;
    uint4 ph, pl;
    split8(p, ph, pl);
    // values: MFMA j takes channel 8 m + j of row m; element e of the lane is token e's value
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1, odd = j & 1;
      const uint4 va = make_uint4(pick(word(vv[0], w), word(vv[1], w), odd), pick(word(vv[2], w), word(vv[3], w), odd),
                                  pick(word(vv[4], w), word(vv[5], w), odd), pick(word(vv[6], w), word(vv[7], w), odd));
      acc[j] = mfma(va, ph, acc[j]);
      acc[j] = mfma(va, pl, acc[j]);
    }
  };
  // the next block's loads are in flight while this block computes; the two register sets
  // alternate, and the load past a wave's last block re-reads the chunk's last block (no branch)
  int blk = wave;
  if (blk < nb) {
    uint4 k0[2][4], v0[8], k1[2][4], v1[8];
    load(blk, k0, v0);
    for (;;) {
      int nx = blk + NW;
      load(nx < nb ? nx : nb - 1, k1, v1);
      step(blk, k0, v0);
      blk = nx;
      if (blk >= nb) break;
      nx = blk + NW;
      load(nx < nb ? nx : nb - 1, k0, v0);
      step(blk, k1, v1);
      blk = nx;
      if (blk >= nb) break;
    }
  }

  // the four lanes of a q head hold disjoint token sets under one running max
  l_run += xor16(l_run, lane);
  l_run += xor32(l_run, lane);
  if (g < G) {
    if (qq == 0) {
      sm_m[wave][g] = m_run;
      sm_l[wave][g] = l_run;
    }
    // lane holds channel 32 qq + 8 i + j of q head g in acc[j][i]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm_acc[wave][g][8 * qq + 2 * i] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      sm_acc[wave][g][8 * qq + 2 * i + 1] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
    }
  }
  __syncthreads();
  const int st = a.state0 + c;
  const float* accf = reinterpret_cast<const float*>(&sm_acc[0][0][0]);
  for (int e = tid; e < G * D; e += NW * 64) {
    const int gg = e / D, ch = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][gg]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (sm_m[w][gg] == -INFINITY) continue;
        const float f = exp2f(sm_m[w][gg] - M);
        L = fmaf(sm_l[w][gg], f, L);
        O = fmaf(accf[(w * MAXG + gg) * D + ch], f, O);
      }
    }
    const int64_t qh_ = static_cast<int64_t>(b) * a.n_q + static_cast<int64_t>(h) * G + gg;
    a.out_states[(static_cast<int64_t>(st) * a.bq + qh_) * D + ch] = L > 0.f ? O / L : 0.f;
    if (ch == 0)
      a.lse_states[static_cast<int64_t>(st) * a.bq + qh_] =
          L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
  }
}

}  // namespace aatc_dense
