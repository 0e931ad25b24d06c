// Decode attention over caches whose codes index a table of reconstruction levels (gfx950): the
// cache pass for Lloyd-Max caches, and for any cache that pairs one with a uniform one.
//
// Page "SPHERICAL KV ..." (NOVA-KV abstract: fixed-width uniform scalar quantizers lose at low
// rates) and page "Ablation ..." (OCTOPUS abstract: Lloyd-Max quantized coordinates, keys
// rebuilt on the fly inside attention).  A Lloyd-Max level is not affine in its code, so the
// summed-code formulation of k_attn_main does not apply; this pass works on levels:
//
//   score_t = sum_i w_i l_(b_i)[c_(t,i)] + const,   w_i = scale log2(e) (R_K q)_i s^K_i,
//   acc_i   = sum_t p_t l_(b_i)[c^V_(t,i)],        y_hat_i = o^V_i + s^V_i acc_i / sum_t p_t,
//
// with l_b the blob's standardized level table (uniform blobs: c - 2^(b-1) + 1/2, s = delta).
// k_attn_lm, grid (S splits, KV heads, batch), 256 threads; per 64-token tile of its range a
// workgroup copies the K and V words to LDS, decodes the K levels of the tile into an LDS matrix,
// scores every (token, q head), updates the online softmax in fp32, decodes the V levels into
// the same matrix and accumulates the probability-weighted levels per (channel, q head).  It
// writes the records k_attn_combine reads, with one column per channel.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_lm {

constexpr int THREADS = 256;
constexpr int T = AATC_TILE;
constexpr int D = AATC_D;
constexpr int LD = D + 1;                 // row stride of the level matrix (bank spread)
constexpr int MAXW = 2 * AATC_MAX_ATTN_BITS;   // words of one K or V tile at most
constexpr int PHDR = 4;                   // record header: max (log2 units), sum, sum, 0
constexpr float PSCALE = 16383.f;         // sums in the units k_attn_combine expects

struct LmArgs {
  const uint32_t* kcodes;
  const uint32_t* vcodes;
  int64_t tiles_per_seq;
  int n_kv, n_q, group;
  const int32_t* seq_lens;
  int seq_per_head;                       // seq_lens is [batch][n_kv] (else [batch])
  int64_t max_seq;
  const float* q;
  float scale2;                           // softmax scale * log2(e)
  float* part;                            // [batch*n_kv][S][group][prec]
  float* offs;                            // [batch*n_kv][8] lse offset per q head (log2 units)
  int S, tpw, prec;
  int kB, vB;
  int quant;                              // bit 0: K blobs Lloyd-Max, bit 1: V blobs
};

// Level of channel i of token t from a V tile (field-major words, see aatc.h): the channel's
// fields hold its code bits; bit b of a w-bit field value of token t = 16G + 4r + m sits at
//   w=1: 32(G/2) + 8m + 2r + G%2,  w=2: 32G + (8m + 2r + b + G%2) mod 32,  w=4: 64G + 32(r/2) + 8m + 4(r%2) + b
__device__ inline int v_field_value(const uint32_t* vw, int word0, int wd, int t) {
  const int G = t >> 4, r = (t >> 2) & 3, m = t & 3;
  if (wd == 1) return static_cast<int>((vw[word0 + (G >> 1)] >> (8 * m + 2 * r + (G & 1))) & 1u);
  if (wd == 2) {
    const uint32_t x = vw[word0 + G];
    const uint32_t rot = (G & 1) ? ((x >> 1) | (x << 31)) : x;     // undo the odd groups' rotation
    return static_cast<int>((rot >> (8 * m + 2 * r)) & 3u);
  }
  return static_cast<int>((vw[word0 + 2 * G + (r >> 1)] >> (8 * m + 4 * (r & 1))) & 15u);
}

__device__ inline float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(THREADS) void k_attn_lm(LmArgs a, const aatc_calib* __restrict__ kcal,
                                                     const aatc_calib* __restrict__ vcal) {
  __shared__ float lvl[T * LD];           // K levels of the tile, then its V levels, [t][i]
  __shared__ uint32_t kw[MAXW + 2], vw[MAXW + 2];
  __shared__ float wk[8 * D];             // score weight of (q head, channel)
  __shared__ float qs[8 * D];
  __shared__ float lk[AATC_LEVELS], lvt[AATC_LEVELS];
  __shared__ int kpb[D], kbit[D], vbit[D];
  __shared__ int vfw[3 * D], vfs[3 * D];  // V fields of each channel: first word, width | shift << 4
  __shared__ float ps[T * 8];             // scores, then probabilities, [t][g]
  __shared__ float mrun[8], lrun[8], fsc[8], beta[8];
  __shared__ int s_bad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.n_kv + h;
  const int G = a.group;
  const aatc_calib* kc = kcal + h;
  const aatc_calib* vc = vcal + h;
  const int Bk = a.kB, Bv = a.vB;

  // ---- tables and queries
  if (tid == 0) {
    const bool ok = kc->magic == AATC_MAGIC && vc->magic == AATC_MAGIC && kc->total_bits == Bk &&
                    vc->total_bits == Bv && kc->quantizer == (a.quant & 1) && vc->quantizer == ((a.quant >> 1) & 1);
    s_bad = ok ? 0 : 1;
  }
  for (int k = tid; k < AATC_LEVELS; k += THREADS) {
    lk[k] = kc->level32[k];
    lvt[k] = vc->level32[k];
  }
  if (tid < D) {
    kbit[tid] = kc->bits[tid];
    vbit[tid] = vc->bits[tid];
    for (int k = 0; k < 3; ++k) {
      const int f = vc->channel_field[3 * tid + k];
      vfw[3 * tid + k] = f >= 0 ? vc->field_word[f] : -1;
      vfs[3 * tid + k] = f >= 0 ? (vc->field_width[f] | (vc->field_shift[f] << 4)) : 0;
    }
  }
  for (int e = tid; e < G * D; e += THREADS) qs[e] = a.q[(static_cast<int64_t>(b) * a.n_q + h * G) * D + e];
  __syncthreads();
  if (tid == 0) {
    int p = 0;
    for (int i = 0; i < D; ++i) {
      kpb[i] = p;
      p += kbit[i];
    }
  }
  // q~ = R_K q (the blob's R: orthogonal rotations and the NOVA query transform alike), then
  // the weights and the constant of the score (the lse offset)
  {
    const int i = tid & (D - 1), gh = tid >> 7;
    float qt[4] = {0.f, 0.f, 0.f, 0.f};
    const float4* row = reinterpret_cast<const float4*>(kc->R32 + i * D);
    for (int j4 = 0; j4 < D / 4; ++j4) {
      const float4 r4 = row[j4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = gh + 2 * u;
        if (g < G) {
          const float* qg = qs + g * D + 4 * j4;
          qt[u] = fmaf(r4.x, qg[0], fmaf(r4.y, qg[1], fmaf(r4.z, qg[2], fmaf(r4.w, qg[3], qt[u]))));
        }
      }
    }
    __syncthreads();                      // every row product has read qs
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = gh + 2 * u;
      if (g < G) {
        wk[g * D + i] = kbit[i] ? a.scale2 * qt[u] * kc->scale32[i] : 0.f;
        qs[g * D + i] = a.scale2 * qt[u] * kc->o32[i];      // constant part of the score
      }
    }
  }
  __syncthreads();
  for (int g = wave; g < G; g += THREADS / 64) {
    const float c0 = wave_sum(qs[g * D + lane] + qs[g * D + 64 + lane]);
    if (lane == 0) {
      beta[g] = c0;
      mrun[g] = -INFINITY;
      lrun[g] = 0.f;
    }
  }
  __syncthreads();
  if (s == 0 && tid < G) a.offs[bh * 8 + tid] = beta[tid];

  int64_t seq64 = a.seq_lens ? static_cast<int64_t>(a.seq_lens[a.seq_per_head ? bh : b]) : a.max_seq;
  seq64 = seq64 < 0 ? 0 : (seq64 > a.max_seq ? a.max_seq : seq64);
  const int seq = static_cast<int>(seq64);
  const int ntiles = (seq + T - 1) / T;
  const int t0 = s * a.tpw;
  const int t1 = (t0 + a.tpw < ntiles) ? t0 + a.tpw : ntiles;
  const bool good = s_bad == 0;
  const int64_t kwords = 2 * static_cast<int64_t>(Bk), vwords = 2 * static_cast<int64_t>(Bv);
  const uint32_t* kseq = a.kcodes + static_cast<int64_t>(bh) * a.tiles_per_seq * kwords;
  const uint32_t* vseq = a.vcodes + static_cast<int64_t>(bh) * a.tiles_per_seq * vwords;

  // PV accumulators: channel i = tid & 127, q heads gh, gh + 2, gh + 4, gh + 6
  const int pi = tid & (D - 1), pgh = tid >> 7;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int dt = tid >> 2, dq = tid & 3;  // decode: token dt, channels dq + 4k

  for (int tile = good ? t0 : t1; tile < t1; ++tile) {
    const int nvalid = seq - tile * T < T ? seq - tile * T : T;
    for (int w = tid; w < kwords; w += THREADS) kw[w] = kseq[tile * kwords + w];
    for (int w = tid; w < vwords; w += THREADS) vw[w] = vseq[tile * vwords + w];
    if (tid < 2) {
      kw[kwords + tid] = 0u;
      vw[vwords + tid] = 0u;
    }
    __syncthreads();
    // K levels: channel i's code sits at bits [t Bk + kpb_i, + b_i) of the tile's string
    for (int k = 0; k < D / 4; ++k) {
      const int i = dq + 4 * k, bi = kbit[i];
      float l = 0.f;
      if (bi) {
        const int pos = dt * Bk + kpb[i];
        const uint32_t x = __builtin_amdgcn_alignbit(kw[(pos >> 5) + 1], kw[pos >> 5], static_cast<uint32_t>(pos & 31));
        l = lk[(1 << bi) - 2 + static_cast<int>(x & ((1u << bi) - 1u))];
      }
      lvl[dt * LD + i] = l;
    }
    __syncthreads();
    // scores of (token, q head) pairs
    for (int pr = tid; pr < T * G; pr += THREADS) {
      const int t = pr & (T - 1), g = pr >> 6;
      float sc = 0.f;
      const float* lr = lvl + t * LD;
      const float* wr = wk + g * D;
#pragma unroll 8
      for (int i = 0; i < D; ++i) sc = fmaf(lr[i], wr[i], sc);
      ps[t * 8 + g] = t < nvalid ? sc : -INFINITY;
    }
    __syncthreads();
    // online softmax per q head (log2 units): wave w takes heads w, w + 4
    for (int g = wave; g < G; g += THREADS / 64) {
      const float sc = ps[lane * 8 + g];
      const float mt = wave_max(sc);
      const float mo = mrun[g];
      const float mn = fmaxf(mo, mt);
      const float p = sc == -INFINITY ? 0.f : exp2f(sc - mn);
      const float ls = wave_sum(p);
      ps[lane * 8 + g] = p;
      if (lane == 0) {
        const float f = mo == -INFINITY ? 0.f : exp2f(mo - mn);
        fsc[g] = f;
        lrun[g] = lrun[g] * f + ls;
        mrun[g] = mn;
      }
    }
    __syncthreads();
    // V levels: channel i's code is the sum of its fields' values shifted into place
    for (int k = 0; k < D / 4; ++k) {
      const int i = dq + 4 * k, bi = vbit[i];
      float l = 0.f;
      if (bi) {
        int code = 0;
#pragma unroll
        for (int f = 0; f < 3; ++f) {
          const int w0 = vfw[3 * i + f];
          if (w0 >= 0) code |= v_field_value(vw, w0, vfs[3 * i + f] & 15, dt) << (vfs[3 * i + f] >> 4);
        }
        l = lvt[(1 << bi) - 2 + code];
      }
      lvl[dt * LD + i] = l;
    }
    __syncthreads();
    // probability-weighted levels of channel pi for its q heads
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = pgh + 2 * u;
      if (g < G) {
        float sum = 0.f;
#pragma unroll 8
        for (int t = 0; t < T; ++t) sum = fmaf(ps[t * 8 + g], lvl[t * LD + pi], sum);
        acc[u] = acc[u] * fsc[g] + sum;
      }
    }
    __syncthreads();                      // lvl, ps and the words are rewritten next tile
  }

  // ---- records: [max, sum, sum, 0, per-channel weighted level sums], sums in units of PSCALE
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = pgh + 2 * u;
    if (g < G) {
      float* rec = a.part + ((static_cast<int64_t>(bh) * a.S + s) * G + g) * a.prec;
      rec[PHDR + pi] = acc[u] * PSCALE;
      if (pi == 0) {
        rec[0] = good ? mrun[g] : NAN;
        rec[1] = lrun[g] * PSCALE;
        rec[2] = lrun[g] * PSCALE;
        rec[3] = 0.f;
      }
    }
  }
}

}  // namespace aatc_lm
