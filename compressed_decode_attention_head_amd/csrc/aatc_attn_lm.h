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
//
// k_attn_lm, grid (S splits, KV heads, batch), 8 waves.  A workgroup owns a contiguous range of
// 64-token tiles of one sequence; each wave takes every eighth tile and keeps its own online
// softmax, with no barrier until the final merge.  Per tile a wave:
//  1. copies the tile's K and V words into its own LDS slot with global_load_lds (no registers),
//     one tile ahead (two slots per wave; one slot, no overlap, when two would not fit LDS: more
//     than about 1100 bits per K + V vector pair);
//  2. scores on v_mfma_f32_16x16x32_bf16, as the dense kernel does: K levels as the A operand
//     (row = token, 8 consecutive channels per lane, decoded from the token-major bit string: one
//     64-bit window per 8 channels, then a mask and a table read per channel), the weights as B;
//     levels and weights each enter as bf16 high plus low parts (three MFMAs: the low x low
//     product, about 2^-16 of the whole, is dropped);
//  3. an fp32 online softmax per q head in log2 units;
//  4. PV on the same MFMA: V levels as the A operand (row = channel), decoded from the V field
//     layout in the token order the score MFMAs leave the probabilities in each lane (tokens
//     16 h + 4 (lane / 16) + i): every field word then yields four of the lane's tokens;
//     probabilities as B, high plus low parts.
// The waves' states merge through LDS into one record per q head: [max, sum, sum, 0, one
// column per channel], sums in units of 1/PSCALE, which k_attn_combine turns into the output.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_lm {

constexpr int NW = 8;                     // waves per workgroup
constexpr int THREADS = NW * 64;
constexpr int T = AATC_TILE;
constexpr int D = AATC_D;
constexpr int MAXG = AATC_MAX_GROUP;
constexpr int PHDR = 4;                   // record header: max (log2 units), sum, sum, 0
constexpr float PSCALE = 16383.f;         // sums in the units k_attn_combine expects
constexpr int NLVL = AATC_LEVELS + 1;     // entry 0: the level of a 0-bit channel

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

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
  int nslot;                              // LDS slots per wave: 2 (the next tile in flight) or 1
};

// Bytes of a wave's slot for one tile: the K words, then the V words, each from the 16-byte unit
// at or below its start, with 16 bytes of slack for the reads past the last word.
__host__ __device__ inline int slot_region(int B) { return B > 0 ? ((8 * B + 8 + 16 + 15) / 16) * 16 : 0; }
__host__ __device__ inline int slot_bytes(int kB, int vB) { return slot_region(kB) + slot_region(vB); }
// dynamic LDS: nslot slots per wave (the merge reuses them: NW x MAXG x 128 floats)
__host__ __device__ inline size_t dyn_lds(int kB, int vB, int nslot) {
  const size_t s = static_cast<size_t>(NW) * nslot * slot_bytes(kB, vB);
  const size_t m = static_cast<size_t>(NW) * MAXG * D * 4;
  return s > m ? s : m;
}

__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }
// bf16 high part in the low half, bf16 low part (x - high) in the high half
__device__ inline uint32_t split_pack(float x) {
  const uint32_t h = bf16_rne(x);
  return h | (bf16_rne(x - bf16_val(h)) << 16);
}
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
// high parts (low halves) and low parts (high halves) of two packed levels, element x first
__device__ inline uint32_t his(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ inline uint32_t los(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

__device__ inline f4 mfma(const uint4& a, const uint4& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
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
__device__ inline float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// s_waitcnt vmcnt(n) for a run-time n (0..23; larger waits for all)
__device__ inline void wait_vm(int n) {
#define AATC_LMW(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
  switch (n) {
    AATC_LMW(0) AATC_LMW(1) AATC_LMW(2) AATC_LMW(3) AATC_LMW(4) AATC_LMW(5) AATC_LMW(6) AATC_LMW(7)
    AATC_LMW(8) AATC_LMW(9) AATC_LMW(10) AATC_LMW(11) AATC_LMW(12) AATC_LMW(13) AATC_LMW(14) AATC_LMW(15)
    AATC_LMW(16) AATC_LMW(17) AATC_LMW(18) AATC_LMW(19) AATC_LMW(20) AATC_LMW(21) AATC_LMW(22) AATC_LMW(23)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
#undef AATC_LMW
}

// Copies the 16-byte units covering words [w, w + n) to LDS dst (from the unit at or below w);
// returns the copy instructions this wave issued.  The byte offset of word w in dst is
// 4 w mod 16.
__device__ inline int copy_words(const uint32_t* w, int n, unsigned char* dst, int lane) {
  if (n <= 0) return 0;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(w) & ~static_cast<uintptr_t>(15);
  const int units = static_cast<int>((reinterpret_cast<uintptr_t>(w + n) - a0 + 15) / 16);
  int ni = 0;
  for (int i = 0; i < units; i += 64, ++ni)
    if (i + lane < units)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a0 + 16 * (i + lane)), dst + 16 * i, 16, 0, 0);
  return ni;
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_attn_lm(
    LmArgs a, const aatc_calib* __restrict__ kcal, const aatc_calib* __restrict__ vcal) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ uint32_t lk[NLVL], lv[NLVL];  // packed bf16 levels (high | low << 16); entry 0 = 0
  __shared__ int kpb[D + 1];                // first plane of each channel in a token's string
  __shared__ uint8_t kbit[D];
  __shared__ uint2 vdesc[D];                // V fields of each channel (see below) and its bits
  __shared__ float qs[MAXG * D];            // q, then the score weights
  __shared__ float qt[MAXG * D];            // q~ = R_K q
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float beta[MAXG];
  __shared__ int s_bad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15, qq = lane >> 4;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.n_kv + h;
  const int G = a.group;
  const aatc_calib* kc = kcal + h;
  const aatc_calib* vc = vcal + h;
  const int Bk = a.kB, Bv = a.vB;

  // ---- tile range and the first copies (they depend on arguments only)
  int64_t seq64 = a.seq_lens ? static_cast<int64_t>(a.seq_lens[a.seq_per_head ? bh : b]) : a.max_seq;
  seq64 = seq64 < 0 ? 0 : (seq64 > a.max_seq ? a.max_seq : seq64);
  const int seq = static_cast<int>(seq64);
  const int ntiles = (seq + T - 1) / T;
  const int t0 = s * a.tpw;
  const int t1 = (t0 + a.tpw < ntiles) ? t0 + a.tpw : ntiles;
  const int64_t kwords = 2 * static_cast<int64_t>(Bk), vwords = 2 * static_cast<int64_t>(Bv);
  const uint32_t* kseq = a.kcodes + static_cast<int64_t>(bh) * a.tiles_per_seq * kwords;
  const uint32_t* vseq = a.vcodes + static_cast<int64_t>(bh) * a.tiles_per_seq * vwords;
  const int sb = slot_bytes(Bk, Bv), kreg = slot_region(Bk);
  unsigned char* slot0 = dyn + static_cast<size_t>(wave) * a.nslot * sb;
  auto issue = [&](int tile, int si) -> int {
    unsigned char* sl = slot0 + si * sb;
    return copy_words(kseq + tile * kwords, static_cast<int>(kwords), sl, lane) +
           copy_words(vseq + tile * vwords, static_cast<int>(vwords), sl + kreg, lane);
  };
  int tile = t0 + wave;
  int n_cur = tile < t1 ? issue(tile, 0) : 0;

  // ---- tables
  if (tid == 0) {
    const bool ok = kc->magic == AATC_MAGIC && vc->magic == AATC_MAGIC && kc->total_bits == Bk &&
                    vc->total_bits == Bv && kc->quantizer == (a.quant & 1) && vc->quantizer == ((a.quant >> 1) & 1);
    s_bad = ok ? 0 : 1;
  }
  for (int k = tid; k < NLVL; k += THREADS) {
    lk[k] = k ? split_pack(kc->level32[k - 1]) : 0u;
    lv[k] = k ? split_pack(vc->level32[k - 1]) : 0u;
  }
  if (tid < D) {
    kbit[tid] = static_cast<uint8_t>(kc->bits[tid]);
    // V fields: 16 bits each, word (< 2 x 1024) | log2(2 w) << 11 | shift << 13 (0: none)
    uint32_t f16[3] = {0u, 0u, 0u};
    for (int k = 0; k < 3; ++k) {
      const int f = vc->channel_field[3 * tid + k];
      if (f >= 0) {
        const int wd = vc->field_width[f];
        const uint32_t lw = wd == 4 ? 3u : (wd == 2 ? 2u : 1u);
        f16[k] = static_cast<uint32_t>(vc->field_word[f]) | (lw << 11) | (static_cast<uint32_t>(vc->field_shift[f]) << 13);
      }
    }
    vdesc[tid] = make_uint2(f16[0] | (f16[1] << 16), f16[2] | (static_cast<uint32_t>(vc->bits[tid]) << 16));
  }
  for (int e = tid; e < G * D; e += THREADS) qs[e] = a.q[(static_cast<int64_t>(b) * a.n_q + h * G) * D + e];
  __syncthreads();
  if (wave < 2) {
    // first plane of each channel: a scan of the bit counts over two waves
    const int i = 64 * wave + lane;
    int x = kbit[i];
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    kpb[i + 1] = x;                       // inclusive; wave 1 adds wave 0's total below
    if (i == 0) kpb[0] = 0;
  }
  {
    // q~ = R_K q: thread (channel i, quarter u) takes q heads u and u + 4
    const int i = tid & (D - 1), u = tid >> 7;
    float acc0 = 0.f, acc1 = 0.f;
    const float4* row = reinterpret_cast<const float4*>(kc->R32 + i * D);
    const bool h0 = u < G, h1 = u + 4 < G;
    for (int j4 = 0; j4 < D / 4; ++j4) {
      const float4 r4 = row[j4];
      if (h0) {
        const float* qg = qs + u * D + 4 * j4;
        acc0 = fmaf(r4.x, qg[0], fmaf(r4.y, qg[1], fmaf(r4.z, qg[2], fmaf(r4.w, qg[3], acc0))));
      }
      if (h1) {
        const float* qg = qs + (u + 4) * D + 4 * j4;
        acc1 = fmaf(r4.x, qg[0], fmaf(r4.y, qg[1], fmaf(r4.z, qg[2], fmaf(r4.w, qg[3], acc1))));
      }
    }
    if (h0) qt[u * D + i] = acc0;
    if (h1) qt[(u + 4) * D + i] = acc1;
  }
  __syncthreads();
  if (wave == 1) kpb[64 + lane + 1] += kpb[64];
  {
    // score weights (into qs) and the constant part of the score (the lse offset)
    const int i = tid & (D - 1), u = tid >> 7;
    const float sk = kc->scale32[i];
    const bool coded = kc->bits[i] != 0;
    for (int gg = u; gg < G; gg += 4) qs[gg * D + i] = coded ? a.scale2 * qt[gg * D + i] * sk : 0.f;
    for (int gg = wave; gg < G; gg += NW) {
      const float c0 = wave_sum(a.scale2 * (qt[gg * D + lane] * kc->o32[lane] + qt[gg * D + 64 + lane] * kc->o32[64 + lane]));
      if (lane == 0) beta[gg] = c0;
    }
  }
  __syncthreads();
  if (s == 0 && tid < G) a.offs[bh * 8 + tid] = beta[tid];
  const bool good = s_bad == 0;

  // ---- per-lane operands: weights of q head g (B operand, channels 32 kk + 8 qq + e), the K run
  // of channels 32 kk + 8 qq .. + 7 (first plane, packed widths)
  uint4 wh[4], wl[4];
  int kp[4];
  uint32_t kwid[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    float x[8];
    const int c0 = 32 * kk + 8 * qq;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = g < G ? qs[g * D + c0 + e] : 0.f;
    split8(x, wh[kk], wl[kk]);
    kp[kk] = kpb[c0];
    uint32_t wdp = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) wdp |= static_cast<uint32_t>(kbit[c0 + e]) << (4 * e);
    kwid[kk] = wdp;
  }

  f4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  int si = 0;
  for (; good && tile < t1; tile += NW) {
    const int nxt = tile + NW;
    const int n_nxt = (a.nslot == 2 && nxt < t1) ? issue(nxt, si ^ 1) : 0;
    wait_vm(n_nxt);                                        // this tile's copies have landed
    const unsigned char* sl = slot0 + si * sb;
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(sl + ((reinterpret_cast<uintptr_t>(kseq + tile * kwords)) & 15));
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(sl + kreg + ((reinterpret_cast<uintptr_t>(vseq + tile * vwords)) & 15));
    const int nvalid = seq - tile * T < T ? seq - tile * T : T;
#pragma unroll 1
    for (int blk = 0; blk < 2; ++blk) {
      // ---- scores: lane holds tokens 32 blk + 16 h2 + 4 qq + i of q head g
      float sc8[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int t = 32 * blk + 16 * h2 + g;              // the A row this lane feeds
        f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t lvl[8];
          if (Bk > 0) {
            const int pos = t * Bk + kp[kk];
            const int w0 = pos >> 5;
            const uint32_t x0 = kw[w0], x1 = kw[w0 + 1], x2 = kw[w0 + 2];
            const uint32_t lo = __builtin_amdgcn_alignbit(x1, x0, static_cast<uint32_t>(pos & 31));
            const uint32_t hi = __builtin_amdgcn_alignbit(x2, x1, static_cast<uint32_t>(pos & 31));
            uint64_t run = (static_cast<uint64_t>(hi) << 32) | lo;
            const uint32_t wd = kwid[kk];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t bw = (wd >> (4 * e)) & 15u;
              const uint32_t mask = (1u << bw) - 1u;
              lvl[e] = lk[(static_cast<uint32_t>(run) & mask) + mask];
              run >>= bw;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) lvl[e] = 0u;
          }
          const uint4 ah = make_uint4(his(lvl[0], lvl[1]), his(lvl[2], lvl[3]), his(lvl[4], lvl[5]), his(lvl[6], lvl[7]));
          const uint4 al = make_uint4(los(lvl[0], lvl[1]), los(lvl[2], lvl[3]), los(lvl[4], lvl[5]), los(lvl[6], lvl[7]));
          sc = mfma(ah, wh[kk], sc);
          sc = mfma(ah, wl[kk], sc);
          sc = mfma(al, wh[kk], sc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rel = 32 * blk + 16 * h2 + 4 * qq + i;
          sc8[4 * h2 + i] = rel < nvalid ? sc[i] : -INFINITY;
        }
      }
      // ---- online softmax (log2 units)
      float bm = sc8[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sc8[e]);
      bm = fmaxf(bm, xor16(bm, lane));
      bm = fmaxf(bm, xor32(bm, lane));
      const float m_new = fmaxf(m_run, bm);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
        const float al = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= al;
        l_run *= al;
        m_run = m_new;
      }
      float p[8];
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = m_run == -INFINITY ? 0.f : exp2f(sc8[e] - m_run);
        ls += p[e];
      }
      l_run += ls;
      uint4 ph, pl;
      split8(p, ph, pl);
      // ---- values: MFMA j, row g is channel 16 j + g; element e of the lane is token
      // 32 blk + 16 (e / 4) + 4 qq + e % 4, i.e. field group Gf = 2 blk + e / 4, r = qq, m = e % 4
      if (Bv > 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = 16 * j + g;
          const uint2 dsc = vdesc[c];
          const uint32_t bits = dsc.y >> 16;
          const uint32_t mask = (1u << bits) - 1u;
          uint32_t code[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
          for (int f = 0; f < 3; ++f) {
            const uint32_t fd = (f == 0 ? dsc.x : (f == 1 ? dsc.x >> 16 : dsc.y)) & 0xffffu;
            const uint32_t lw = (fd >> 11) & 3u;
            if (lw == 0) continue;
            const int fw = static_cast<int>(fd & 2047u);
            const uint32_t sh = fd >> 13, wbits = 1u << (lw - 1u);
            const bool w4 = lw == 3u, w2 = lw == 2u;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              // field group Gf = 2 blk + h2: w=4 word 2 Gf + qq/2, bits 4 (qq % 2) + 8 m; w=2 word
              // Gf (rotated left by one when Gf is odd), bits 2 qq + 8 m; w=1 word Gf/2, bits
              // 2 qq + Gf % 2 + 8 m (Gf % 2 = h2)
              const int Gf = 2 * blk + h2;
              const int wi = fw + (w4 ? 2 * Gf + (qq >> 1) : (w2 ? Gf : blk));
              const uint32_t b0 = w4 ? 4u * (qq & 1) : (w2 ? 2u * qq : 2u * qq + h2);
              uint32_t x = vw[wi];
              if (h2 == 1 && w2) x = __builtin_amdgcn_alignbit(x, x, 1u);   // undo the odd groups' rotation
#pragma unroll
              for (int i = 0; i < 4; ++i) code[4 * h2 + i] |= __builtin_amdgcn_ubfe(x, 8u * i + b0, wbits) << sh;
            }
          }
          uint32_t lvl[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) lvl[e] = lv[code[e] + mask];   // code < 2^bits
          const uint4 vh = make_uint4(his(lvl[0], lvl[1]), his(lvl[2], lvl[3]), his(lvl[4], lvl[5]), his(lvl[6], lvl[7]));
          const uint4 vl = make_uint4(los(lvl[0], lvl[1]), los(lvl[2], lvl[3]), los(lvl[4], lvl[5]), los(lvl[6], lvl[7]));
          acc[j] = mfma(vh, ph, acc[j]);
          acc[j] = mfma(vh, pl, acc[j]);
          acc[j] = mfma(vl, ph, acc[j]);
        }
      }
    }
    // one slot: the next tile's copies go out once this tile's reads have been consumed
    if (a.nslot == 2)
      si ^= 1;
    else if (nxt < t1)
      issue(nxt, 0);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));        // vmcnt(0): no copy in flight into the slots

  // ---- merge the waves: the four lanes of a q head hold disjoint token sets under one max
  l_run += xor16(l_run, lane);
  l_run += xor32(l_run, lane);
  __syncthreads();                                         // every wave is done with its slots
  float* sm_acc = reinterpret_cast<float*>(dyn);           // [NW][MAXG][128]
  if (g < G) {
    if (qq == 0) {
      sm_m[wave][g] = m_run;
      sm_l[wave][g] = l_run;
    }
    // acc[j][i]: channel 16 j + 4 qq + i of q head g
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_acc[(wave * MAXG + g) * D + 16 * j + 4 * qq + i] = acc[j][i];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += THREADS) {
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
        O = fmaf(sm_acc[(w * MAXG + gg) * D + ch], f, O);
      }
    }
    float* rec = a.part + ((static_cast<int64_t>(bh) * a.S + s) * G + gg) * a.prec;
    rec[PHDR + ch] = O * PSCALE;
    if (ch == 0) {
      rec[0] = good ? M : NAN;
      rec[1] = L * PSCALE;
      rec[2] = L * PSCALE;
      rec[3] = 0.f;
    }
  }
}

}  // namespace aatc_lm
