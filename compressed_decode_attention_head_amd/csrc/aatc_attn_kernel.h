// Decode attention that reads the packed cache directly (gfx950): two kernels per step.
//
// Page "SPECTRA ..." (Abstract) and page "SPHERICAL KV ..." (RDKV abstract): the cache is
// re-read in full at every generated token, so decode is bound by HBM reads of the cache;
// page "Ablation ..." (OCTOPUS abstract): keys are reconstructed on the fly, never
// materialised.  Here nothing is reconstructed per token at all:
//
//   score_t = scale q.k_hat_t = sum_p w_p bit_p(t) + const,  w_(i,k) = scale (R_K q)_i delta_i 2^k,
//
// a contraction of the token's K bit-planes (0/1) with per-plane weights; the constant (the
// dequantization offset) cancels in the softmax and is only added back for the lse.
// Values: sum_t p_t c_(t,i) is accumulated on the packed V codes; the affine dequantization
// and R_V^T are applied once per step to the softmax-weighted code sums.
//
// Both contractions run on the int8 matrix cores (v_mfma_i32_16x16x64_i8, exact int32
// accumulation).  Bits and codes are exact int8 operands; weights and probabilities are
// fixed point split into int8 limbs that occupy the 16 MFMA rows:
//   scores, LIMBS=2: 8 q-head slots x 2 limbs (15-bit weights), GQA <= 8;
//   scores, LIMBS=3: 4 q-head slots x 3 limbs (22-bit weights), GQA <= 4;
//   values: 8 q-head slots x 2 limbs of a 14-bit probability.
//
// k_attn_main, grid (S splits, KV heads, batch), WAVES waves per workgroup; a workgroup owns
// a contiguous range of 64-token tiles of one sequence, each wave `tpw` consecutive tiles:
//   1. the K tables and the queries, then the wave's tiles, are copied straight from HBM into
//      LDS with global_load_lds (no registers); the small tables land first,
//   2. while the tiles fly, the workgroup rotates the queries and builds the limb weights,
//   3. each wave streams its tiles out of LDS: scores -> online softmax -> PV, int32 sums,
//   4. the waves merge in LDS and the workgroup writes one partial record per q head:
//      (running max, sum of probabilities, softmax-weighted code sum per V field column).
// k_attn_combine, grid (q heads per KV head, KV heads, batch): merges the S records of a
// q head, folds field columns into channel code sums, dequantizes, applies R_V^T and writes
// out and lse.  The kernel boundary orders the records; no atomics, no workspace clearing.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_attn {

constexpr int D = AATC_D;
constexpr int PS = 16383;                 // probability scale: 14-bit fixed point, two 7-bit limbs
// log2(16383 / 65535) - 2^-20: pknorm(x) = rint(65535 x), so a token at the running max maps
// to 16383 and none exceeds it
constexpr float PKN_BIAS = -2.000067f;
constexpr int PHDR = 4;                   // record header floats: max (log2 units), sum, 0, 0
constexpr int UNION_BYTES = 3 * 8 * D * 4;    // prologue q / q~ / alpha
constexpr int TAB_BYTES = 2304;           // K delta32 | o32 | bits | plane_channel | plane_bit
constexpr int PL_WAVE = 16 * 64;          // one wave's probability limb rows (16 x 64 bytes)
constexpr int DMA_PAD = 1024;             // LDS slack after the tile areas (bounded over-reads)
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Waves per workgroup of the main kernel: 16 (four per SIMD) while the accumulators leave
// room for it, else 8.
constexpr int waves_for(int np, int nvb) { return (np + nvb) > 0 ? 8 : 8; }

struct AttnArgs {
  const aatc_calib* kcal;
  const aatc_calib* vcal;
  const uint32_t* kcodes;
  const uint32_t* vcodes;
  int64_t tiles_per_seq;
  int n_kv, n_q, group;
  const int32_t* seq_lens;
  int64_t max_seq;
  const float* q;
  float scale2;                       // softmax scale * log2(e)
  float* out;
  float* lse;
  float* part;                        // [batch*n_kv][S][group][prec] partial records
  float* offs;                        // [batch*n_kv][8] lse offset per q head (log2 units)
  int S, tpw, prec;                   // splits per sequence, tiles per wave, floats per record
  int kB, vB;
  int np_half;                        // 1 if the last K pair carries <= 64 planes
  int chunk;                          // tiles per LDS chunk
  int nbuf;                           // 1 or 2 chunk buffers per wave
  int ks_bytes, vs_bytes;             // K / V area of one chunk buffer (multiples of 1024)
};

__device__ inline int row_max16_i(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));
  return x;
}

__device__ inline unsigned row_sum16_u(unsigned x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x121, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x122, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x124, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xf, 0xf, false);
  return x;
}

__device__ inline float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Orders this wave's LDS accesses for the compiler.  A wavefront's LDS instructions execute
// in order, so no hardware wait is needed; a wavefront-scope fence does not wait on
// outstanding global loads.
__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Waits until at most n (0..63) vector-memory instructions of this wave are outstanding.
__device__ inline void wait_vmcnt(int n) {
#define AATC_VMW(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
  switch (n) {
    AATC_VMW(0) AATC_VMW(1) AATC_VMW(2) AATC_VMW(3) AATC_VMW(4) AATC_VMW(5) AATC_VMW(6) AATC_VMW(7)
    AATC_VMW(8) AATC_VMW(9) AATC_VMW(10) AATC_VMW(11) AATC_VMW(12) AATC_VMW(13) AATC_VMW(14) AATC_VMW(15)
    AATC_VMW(16) AATC_VMW(17) AATC_VMW(18) AATC_VMW(19) AATC_VMW(20) AATC_VMW(21) AATC_VMW(22) AATC_VMW(23)
    AATC_VMW(24) AATC_VMW(25) AATC_VMW(26) AATC_VMW(27) AATC_VMW(28) AATC_VMW(29) AATC_VMW(30) AATC_VMW(31)
    AATC_VMW(32) AATC_VMW(33) AATC_VMW(34) AATC_VMW(35) AATC_VMW(36) AATC_VMW(37) AATC_VMW(38) AATC_VMW(39)
    AATC_VMW(40) AATC_VMW(41) AATC_VMW(42) AATC_VMW(43) AATC_VMW(44) AATC_VMW(45) AATC_VMW(46) AATC_VMW(47)
    AATC_VMW(48) AATC_VMW(49) AATC_VMW(50) AATC_VMW(51) AATC_VMW(52) AATC_VMW(53) AATC_VMW(54) AATC_VMW(55)
    AATC_VMW(56) AATC_VMW(57) AATC_VMW(58) AATC_VMW(59) AATC_VMW(60) AATC_VMW(61) AATC_VMW(62) AATC_VMW(63)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
#undef AATC_VMW
}

// Plane base (within a token's B-bit string) of the K window that lane group `grp` reads for
// MFMA pair u; a half pair (last pair with <= 64 planes) interleaves 4-plane groups so that
// one MFMA covers 64 planes.
__device__ inline int plane_base(int u, int grp, bool half) {
  return half ? 128 * u + 32 * (grp >> 1) + 4 * (grp & 1) : 128 * u + 32 * grp;
}

template <int LIMBS>
struct Lim;
template <>
struct Lim<2> {
  static constexpr int WBITS = 14;       // |w_q| < 2^14
  static constexpr int PROW = 8;         // row stride between limbs
  __device__ static int limb(int l, int v) { return l == 0 ? (v >> 7) : (v & 127); }
};
template <>
struct Lim<3> {
  static constexpr int WBITS = 21;
  static constexpr int PROW = 4;
  __device__ static int limb(int l, int v) { return l == 0 ? (v >> 14) : (l == 1 ? ((v >> 7) & 127) : (v & 127)); }
};

// Copies bytes [start, start + n*1024) (start aligned down to 16) of one sequence's packed
// words into LDS, 16 bytes per lane per instruction; lanes past `end` re-read the last valid
// 16 bytes (their LDS slots are padding).
__device__ inline void dma_block(const char* start, const char* end, const char* base, uint8_t* dst, int n,
                                 int lane) {
  const char* last = reinterpret_cast<const char*>((reinterpret_cast<uintptr_t>(end) - 16) & ~static_cast<uintptr_t>(15));
  last = last < base ? base : last;            // allocations are >= 16 bytes and 16-byte aligned
  for (int ii = 0; ii < n; ++ii) {
    const char* p = start + (ii * 64 + lane) * 16;
    p = p > last ? last : p;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p), dst + ii * 1024, 16, 0, 0);
  }
}

// Copies nwords 32-bit words src[0..nwords) to LDS dst[0..nwords), 64 words per instruction,
// instruction k issued by wave k % WAVES.  Lanes past nwords re-read src[0]; their LDS words
// (up to the next multiple of 64) are padding.  Returns the running instruction index.
template <int WAVES>
__device__ inline int dma_words(const void* src, void* dst, int nwords, int k, int wave, int lane) {
  for (int i = 0; i < nwords; i += 64, ++k)
    if (k % WAVES == wave) {
      const uint32_t* p = static_cast<const uint32_t*>(src) + i + lane;
      if (i + lane >= nwords) p = static_cast<const uint32_t*>(src);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p), static_cast<uint32_t*>(dst) + i, 4, 0, 0);
    }
  return k;
}

template <int NP, int NVB, int LIMBS>
__global__ __launch_bounds__(waves_for(NP, NVB) * 64) void k_attn_main(AttnArgs a) {
  constexpr int WAVES = waves_for(NP, NVB);
  constexpr int NT = WAVES * 64;
  using LM = Lim<LIMBS>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);                       // [8][128]   q
  float* qt = qs + 8 * D;                                           // [8][128]   R_K q
  float* al = qt + 8 * D;                                           // [8][128]   alpha
  uint8_t* pl = smem + UNION_BYTES;                                 // [WAVES][16][64] P limbs
  int* wa_lds = reinterpret_cast<int*>(pl);                         // [NP*2*4*64] (prologue)
  uint8_t* tab = pl + WAVES * PL_WAVE;
  float* t_delta = reinterpret_cast<float*>(tab);                   // [128]
  float* t_o = t_delta + D;                                         // [128]
  const uint8_t* t_bits = tab + 1024;                               // [128]
  const uint8_t* t_pch = tab + 1280;                                // [<=512]
  const uint8_t* t_pbit = tab + 1792;                               // [<=512]
  uint8_t* chunks = tab + TAB_BYTES;                                // [WAVES][nbuf][ks+vs]
  float* mg = reinterpret_cast<float*>(chunks);                     // merge: [WAVES][NVB][32 lanes][4]
  __shared__ float s_m[WAVES][8], s_l[WAVES][8];
  __shared__ float s_M[8], s_L[8], esc[8];
  __shared__ int wexp[8];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.n_kv + h;
  const aatc_calib* kc = a.kcal + h;
  const aatc_calib* vc = a.vcal + h;
  const int G = a.group;
  const int Bk = a.kB, Bv = a.vB;
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[b]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);     // never read past the cache
  const int64_t ntiles = (seq + 63) / 64;
  const int64_t t0 = (static_cast<int64_t>(s) * WAVES + wave) * a.tpw;
  const int64_t t1 = t0 + a.tpw < ntiles ? t0 + a.tpw : ntiles;

  // ---- 1. K tables and queries to LDS (first, so they land before the tiles)
  {
    int k = 0;
    k = dma_words<WAVES>(a.q + (static_cast<int64_t>(b) * a.n_q + h * G) * D, qs, G * D, k, wave, lane);
    k = dma_words<WAVES>(kc->delta32, t_delta, D, k, wave, lane);
    k = dma_words<WAVES>(kc->o32, t_o, D, k, wave, lane);
    k = dma_words<WAVES>(kc->bits, tab + 1024, D / 4, k, wave, lane);
    k = dma_words<WAVES>(kc->plane_channel, tab + 1280, (Bk + 3) / 4, k, wave, lane);
    k = dma_words<WAVES>(kc->plane_bit, tab + 1792, (Bk + 3) / 4, k, wave, lane);
    for (int e = G * D + tid; e < 8 * D; e += NT) qs[e] = 0.f;
  }

  // ---- 2. this wave's tiles: chunk 0 (and chunk 1 when double-buffered)
  const bool half = a.np_half != 0;
  const int64_t kbytes = 8 * static_cast<int64_t>(Bk), vbytes = 8 * static_cast<int64_t>(Bv);
  const char* kseq = reinterpret_cast<const char*>(a.kcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * kbytes;
  const char* vseq = reinterpret_cast<const char*>(a.vcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * vbytes;
  const char* kend = kseq + a.tiles_per_seq * kbytes;
  const char* vend = vseq + a.tiles_per_seq * vbytes;
  const int CH = a.chunk, NBUF = a.nbuf;
  const int nki = Bk > 0 ? a.ks_bytes >> 10 : 0, nvi = Bv > 0 ? a.vs_bytes >> 10 : 0;
  uint8_t* wbuf = chunks + static_cast<size_t>(wave) * NBUF * (a.ks_bytes + a.vs_bytes);
  // the copies depend on arguments only; the blob headers are checked after they are issued
  const int64_t ntile_w = t1 > t0 ? t1 - t0 : 0;
  const int nchunks_dma = static_cast<int>((ntile_w + CH - 1) / CH);
  // K/V data of chunk c start this many bytes into their areas (16-byte alignment)
  auto kpad = [&](int c) { return static_cast<int>(reinterpret_cast<uintptr_t>(kseq + (t0 + c * CH) * kbytes) & 15); };
  auto vpad = [&](int c) { return static_cast<int>(reinterpret_cast<uintptr_t>(vseq + (t0 + c * CH) * vbytes) & 15); };
  auto issue = [&](int c, int buf) {
    uint8_t* kb = wbuf + buf * (a.ks_bytes + a.vs_bytes);
    const char* ks = kseq + (t0 + c * CH) * kbytes;
    const char* vs = vseq + (t0 + c * CH) * vbytes;
    dma_block(reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(ks) & ~static_cast<uintptr_t>(15)), kend,
              reinterpret_cast<const char*>(a.kcodes), kb, nki, lane);
    dma_block(reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(vs) & ~static_cast<uintptr_t>(15)), vend,
              reinterpret_cast<const char*>(a.vcodes), kb + a.ks_bytes, nvi, lane);
  };
  int inflight = 0;
  if (nchunks_dma > 0) { issue(0, 0); inflight += nki + nvi; }
  if (nchunks_dma > 1 && NBUF == 2) { issue(1, 1); inflight += nki + nvi; }
  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4, T1 = (n1 + 15) >> 4;
  const int NV = T4 + T2 + T1;
  const bool ok = kc->magic == AATC_MAGIC && vc->magic == AATC_MAGIC && kc->total_bits == Bk &&
                  vc->total_bits == Bv && NV <= NVB && PHDR + 16 * NV <= a.prec;
  // a bad blob streams nothing (issued copies are still waited for below) and yields NaN
  const int nchunks = ok ? nchunks_dma : 0;
  wait_vmcnt(inflight);                  // this wave's table copies have landed
  __syncthreads();

  // ---- 3. prologue: q~ = R_K q, alpha, exponents, lse offsets, limb weights
  const int rot = kc->rotation;
  if (rot == AATC_ROT_WHT) {
    // Sylvester-ordered fast Walsh-Hadamard transform, one wave per head slot, then 1/sqrt(128)
    if (wave < 8) {
      float x0 = qs[wave * D + lane], x1 = qs[wave * D + 64 + lane];
      const float y = x0;
      x0 = y + x1;
      x1 = y - x1;
#pragma unroll
      for (int len = 1; len < 64; len <<= 1) {
        const float o0 = __shfl_xor(x0, len), o1 = __shfl_xor(x1, len);
        const bool hi = (lane & len) != 0;
        x0 = hi ? o0 - x0 : x0 + o0;
        x1 = hi ? o1 - x1 : x1 + o1;
      }
      qt[wave * D + lane] = x0 * 0.08838834764831845f;
      qt[wave * D + 64 + lane] = x1 * 0.08838834764831845f;
    }
  } else if (rot == AATC_ROT_KLT) {
    // row i of R_K: NT/128 threads per row, eight q heads per thread
    constexpr int TPR = NT / D, CPT = D / TPR;
    const int i = tid / TPR, qq = tid % TPR;
    float part[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) part[g] = 0.f;
    const float2* row = reinterpret_cast<const float2*>(kc->R32 + i * D + CPT * qq);
#pragma unroll
    for (int c2 = 0; c2 < CPT / 2; ++c2) {
      const float2 r = row[c2];
      const int j = CPT * qq + 2 * c2;
#pragma unroll
      for (int g = 0; g < 8; ++g) part[g] += r.x * qs[g * D + j] + r.y * qs[g * D + j + 1];
    }
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) part[g] += __shfl_xor(part[g], o);
    if (qq == 0)
#pragma unroll
      for (int g = 0; g < 8; ++g) qt[g * D + i] = part[g];
  } else {
    for (int e = tid; e < 8 * D; e += NT) qt[e] = qs[e];
  }
  __syncthreads();
  if (wave < 8) {
    // one wave per head slot: alpha, the lse offset and the weight exponent
    const int g = wave;
    float m = 0.f, off = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      const int bi = t_bits[i];
      const float v = qt[g * D + i];
      const float alpha = bi ? v * t_delta[i] * a.scale2 : 0.f;
      al[g * D + i] = alpha;
      if (bi) m = fmaxf(m, fabsf(alpha) * static_cast<float>(1 << (bi - 1)));
      const float o = bi ? t_o[i] - t_delta[i] * (static_cast<float>(1 << (bi - 1)) - 0.5f) : t_o[i];
      off += v * o * a.scale2;
    }
    m = wave_max(m);
    off = wave_sum(off);
    int e = 0;
    if (m > 0.f) {
      frexpf(m, &e);
      e = LM::WBITS - e;                 // m * 2^e in [2^(WBITS-1), 2^WBITS)
    }
    if (lane == 0) {
      wexp[g] = e;
      esc[g] = (m > 0.f) ? ldexpf(1.f, -e) : 0.f;
      if (s == 0 && g < G) a.offs[bh * 8 + g] = off;
    }
  }
  __syncthreads();
  {
    const int nw = NP * 2 * 4 * 64;
    const int wmaxq = (1 << LM::WBITS) - 1;
    for (int e = tid; e < nw; e += NT) {
      const int ln = e & 63, jj = (e >> 6) & 3, hh = (e >> 8) & 1, u = e >> 9;
      const int row = ln & 15, lg = ln >> 4;
      const int l = row / LM::PROW;
      const int g = row % LM::PROW;
      const bool hp = half && u == NP - 1;
      uint32_t word = 0;
      for (int m = 0; m < 4; ++m) {
        const int p = plane_base(u, lg, hp) + 8 * m + (hp ? jj : 4 * hh + jj);
        int val = 0;
        if (p < Bk && g < G && l < LIMBS && !(hp && hh)) {
          const int ch = t_pch[p], kb = t_pbit[p];
          int wq = static_cast<int>(rintf(ldexpf(al[g * D + ch], kb + wexp[g])));
          wq = wq > wmaxq ? wmaxq : (wq < -wmaxq ? -wmaxq : wq);
          val = LM::limb(l, wq);
        }
        word |= (static_cast<uint32_t>(val) & 0xffu) << (8 * m);
      }
      wa_lds[e] = static_cast<int>(word);
    }
  }
  __syncthreads();
  v4i wa[NP][2];
#pragma unroll
  for (int u = 0; u < NP; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[u][hh][j] = wa_lds[((u * 2 + hh) * 4 + j) * 64 + lane];
  __syncthreads();                       // wa_lds aliases the probability rows
  for (int e = tid; e < WAVES * PL_WAVE / 4; e += NT) reinterpret_cast<uint32_t*>(pl)[e] = 0u;
  __syncthreads();

  // head slots this lane holds after the limb merge: LIMBS=2 pair a {0,4,1,5}[grp] and
  // pair b {2,6,3,7}[grp]; LIMBS=3 head grp
  const int ha = LIMBS == 2 ? (grp & 1) * 4 + (grp >> 1) : grp;
  const int hb = ha + 2;
  const float esa = esc[ha], esb = LIMBS == 2 ? esc[hb] : 0.f;
  // score lane n16 of token group tau holds token 16*(n16/4) + 4*(n16%4) + tau, so that the
  // probability bytes it packs are the PV operand's K order (token 16*grp + 4*i + byte)
  const int tok0 = 16 * (n16 >> 2) + 4 * (n16 & 3);
  int kofs[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) kofs[u] = tok0 * Bk + plane_base(u, grp, half && u == NP - 1);
  uint8_t* pw = pl + wave * PL_WAVE;
  // probability rows (limb l, head slot x) = row 8l + x; dword n16 of a row sits in 16-byte
  // quad (n16/4) ^ (row%4)
  auto prow_addr = [&](int row) { return row * 64 + 16 * ((n16 >> 2) ^ (row & 3)) + 4 * (n16 & 3); };
  const int wa0 = prow_addr(ha), wa1 = prow_addr(8 + ha);
  const int wb0 = prow_addr(hb), wb1 = prow_addr(8 + hb);
  const int prd = n16 * 64 + 16 * (grp ^ (n16 & 3));

  v4i acc[NVB];
#pragma unroll
  for (int v = 0; v < NVB; ++v) acc[v] = v4i{0, 0, 0, 0};
  int ima = INT_MIN, imb = INT_MIN;       // running integer score maxima (INT_MIN: none yet)
  unsigned la = 0, lb = 0;
  const v2u16 ones = {1, 1};

  // ---- 4. stream the chunks out of LDS
  if (!ok) wait_vmcnt(0);
  for (int c = 0; c < nchunks; ++c) {
    const int buf = NBUF == 2 ? (c & 1) : 0;
    if (NBUF == 2 && c + 1 < nchunks) wait_vmcnt(nki + nvi);
    else wait_vmcnt(0);
    wave_sync_lds();
    const uint8_t* kb = wbuf + buf * (a.ks_bytes + a.vs_bytes);
    const uint32_t* kchunk = reinterpret_cast<const uint32_t*>(kb + kpad(c));
    const uint32_t* vchunk = reinterpret_cast<const uint32_t*>(kb + a.ks_bytes + vpad(c));
    const int64_t ctile0 = t0 + static_cast<int64_t>(c) * CH;
    const int nt = static_cast<int>(t1 - ctile0 < CH ? t1 - ctile0 : CH);
    for (int it = 0; it < nt; ++it) {
      const int64_t tile = ctile0 + it;
      const uint32_t* kl = kchunk + it * 2 * Bk;
      const uint32_t* vl = vchunk + it * 2 * Bv;
      // scores: 4 token groups; integer scores of head pair a / b (LIMBS=3: one head)
      int sa[4], sb[4];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        v4i cc = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const bool hp = half && u == NP - 1;
          const int o = kofs[u] + tau * Bk;
          const uint32_t* w = kl + (o >> 5);
          const uint32_t dw = __builtin_amdgcn_alignbit(w[1], w[0], static_cast<uint32_t>(o));
          v4i b0;
#pragma unroll
          for (int j = 0; j < 4; ++j) b0[j] = static_cast<int>((dw >> j) & 0x01010101u);
          cc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][0], b0, cc, 0, 0, 0);
          if (!hp) {
            v4i b1;
#pragma unroll
            for (int j = 0; j < 4; ++j) b1[j] = static_cast<int>((dw >> (j + 4)) & 0x01010101u);
            cc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][1], b1, cc, 0, 0, 0);
          }
        }
        if (LIMBS == 2) {
          const auto p01 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[0]), static_cast<unsigned>(cc[1]),
                                                            false, false);
          const auto p23 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[2]), static_cast<unsigned>(cc[3]),
                                                            false, false);
          sa[tau] = (static_cast<int>(p01[0]) << 7) + static_cast<int>(p01[1]);
          sb[tau] = (static_cast<int>(p23[0]) << 7) + static_cast<int>(p23[1]);
        } else {
          // 4x4 transpose of 16-lane blocks: rows (limb l, head r) -> lane group = head
          const auto x02 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[0]), static_cast<unsigned>(cc[2]),
                                                            false, false);
          const auto x13 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[1]), static_cast<unsigned>(cc[3]),
                                                            false, false);
          const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);   // limb 0, limb 1
          const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);   // limb 2, unused
          sa[tau] = (static_cast<int>(y01[0]) << 14) + (static_cast<int>(y01[1]) << 7) + static_cast<int>(y23[0]);
          sb[tau] = 0;
        }
      }
      const int64_t nvalid = seq - tile * 64;
      const bool ragged = nvalid < 64;
      if (ragged) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
          if (tok0 + tau >= nvalid) { sa[tau] = INT_MIN; sb[tau] = INT_MIN; }
      }
      // a tile has at least one visible token, so its maxima are real scores
      const int ita = row_max16_i(max(max(sa[0], sa[1]), max(sa[2], sa[3])));
      const int itb = LIMBS == 2 ? row_max16_i(max(max(sb[0], sb[1]), max(sb[2], sb[3]))) : INT_MIN;
      // online softmax: rescale the integer accumulators when a running max grows
      if (__ballot(ita > ima || itb > imb)) {
        const int nma = max(ima, ita), nmb = max(imb, itb);
        const float fa = (ima == INT_MIN) ? 0.f : __builtin_amdgcn_exp2f(static_cast<float>(ima - nma) * esa);
        const float fb = (imb == INT_MIN) ? 0.f : __builtin_amdgcn_exp2f(static_cast<float>(imb - nmb) * esb);
        la = static_cast<unsigned>(rintf(static_cast<float>(la) * fa));
        lb = static_cast<unsigned>(rintf(static_cast<float>(lb) * fb));
        ima = nma;
        imb = nmb;
        float fr[4];
        if (LIMBS == 2) {
          // acc register r of lane group grp holds head 4*(grp&1)+r; the factor of head hd
          // lives in pair a (heads {0,4,1,5} in lane groups 0..3) or pair b ({2,6,3,7})
          const float f0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 0));
          const float f4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 16));
          const float f1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 32));
          const float f5 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 48));
          const float f2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fb), 0));
          const float f6 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fb), 16));
          const float f3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fb), 32));
          const float f7 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fb), 48));
          const bool odd = grp & 1;
          fr[0] = odd ? f4 : f0;
          fr[1] = odd ? f5 : f1;
          fr[2] = odd ? f6 : f2;
          fr[3] = odd ? f7 : f3;
        } else {
          // acc register r holds head r (rows 8l + r); head r's factor lives in lane group r
#pragma unroll
          for (int r = 0; r < 4; ++r) fr[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 16 * r));
        }
#pragma unroll
        for (int v = 0; v < NVB; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[v][r] = static_cast<int>(rintf(static_cast<float>(acc[v][r]) * fr[r]));
      }
      // probabilities in 14-bit fixed point (pknorm rounds 65535 * x), two 7-bit limbs per
      // byte row: the four tokens of this lane fill one dword per (head, limb)
      {
        float pa[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
          pa[tau] = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sa[tau] - ima), esa, PKN_BIAS));
        if (ragged) {
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) pa[tau] = (tok0 + tau >= nvalid) ? 0.f : pa[tau];
        }
        const v2u16 q01 = __builtin_amdgcn_cvt_pknorm_u16(pa[0], pa[1]);
        const v2u16 q23 = __builtin_amdgcn_cvt_pknorm_u16(pa[2], pa[3]);
        la = __builtin_amdgcn_udot2(q01, ones, la, false);
        la = __builtin_amdgcn_udot2(q23, ones, la, false);
        const uint32_t u01 = __builtin_bit_cast(uint32_t, q01), u23 = __builtin_bit_cast(uint32_t, q23);
        const uint32_t hi = __builtin_amdgcn_perm((u23 >> 7) & 0x007F007Fu, (u01 >> 7) & 0x007F007Fu, 0x06040200u);
        const uint32_t lo = __builtin_amdgcn_perm(u23 & 0x007F007Fu, u01 & 0x007F007Fu, 0x06040200u);
        *reinterpret_cast<uint32_t*>(pw + wa0) = hi;
        *reinterpret_cast<uint32_t*>(pw + wa1) = lo;
      }
      if (LIMBS == 2) {
        float pb[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
          pb[tau] = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sb[tau] - imb), esb, PKN_BIAS));
        if (ragged) {
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) pb[tau] = (tok0 + tau >= nvalid) ? 0.f : pb[tau];
        }
        const v2u16 q01 = __builtin_amdgcn_cvt_pknorm_u16(pb[0], pb[1]);
        const v2u16 q23 = __builtin_amdgcn_cvt_pknorm_u16(pb[2], pb[3]);
        lb = __builtin_amdgcn_udot2(q01, ones, lb, false);
        lb = __builtin_amdgcn_udot2(q23, ones, lb, false);
        const uint32_t u01 = __builtin_bit_cast(uint32_t, q01), u23 = __builtin_bit_cast(uint32_t, q23);
        const uint32_t hi = __builtin_amdgcn_perm((u23 >> 7) & 0x007F007Fu, (u01 >> 7) & 0x007F007Fu, 0x06040200u);
        const uint32_t lo = __builtin_amdgcn_perm(u23 & 0x007F007Fu, u01 & 0x007F007Fu, 0x06040200u);
        *reinterpret_cast<uint32_t*>(pw + wb0) = hi;
        *reinterpret_cast<uint32_t*>(pw + wb1) = lo;
      }
      wave_sync_lds();
      const uint4 pv = *reinterpret_cast<const uint4*>(pw + prd);
      const v4i pA = {static_cast<int>(pv.x), static_cast<int>(pv.y), static_cast<int>(pv.z), static_cast<int>(pv.w)};
      // PV on packed V fields (width-uniform column groups: w4 | w2 | w1); columns past a
      // class's field count read neighbouring words and are never used
#pragma unroll
      for (int v = 0; v < NVB; ++v) {
        if (v < NV) {
          v4i bv;
          if (v < T4) {
            const uint2 d2 = *reinterpret_cast<const uint2*>(vl + 8 * ((v << 4) + n16) + 2 * grp);
            const uint32_t m4 = 0x0F0F0F0Fu;
            bv[0] = static_cast<int>(d2.x & m4);
            bv[1] = static_cast<int>((d2.x >> 4) & m4);
            bv[2] = static_cast<int>(d2.y & m4);
            bv[3] = static_cast<int>((d2.y >> 4) & m4);
          } else if (v < T4 + T2) {
            const uint32_t d = vl[8 * n4 + 4 * (((v - T4) << 4) + n16) + grp];
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = static_cast<int>((d >> (2 * r)) & 0x03030303u);
          } else {
            const uint32_t d = vl[8 * n4 + 4 * n2 + 2 * (((v - T4 - T2) << 4) + n16) + (grp >> 1)] >> (4 * (grp & 1));
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = static_cast<int>((d >> r) & 0x01010101u);
          }
          acc[v] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pA, bv, acc[v], 0, 0, 0);
        }
      }
      wave_sync_lds();
    }
    if (NBUF == 2 && c + 2 < nchunks) issue(c + 2, buf);
    else if (NBUF == 1 && c + 1 < nchunks) issue(c + 1, 0);
  }

  // ---- 5. workgroup merge in LDS
  la = row_sum16_u(la);
  lb = row_sum16_u(lb);
  const float ma = ima == INT_MIN ? -INFINITY : static_cast<float>(ima) * esa;
  const float mb = imb == INT_MIN ? -INFINITY : static_cast<float>(imb) * esb;
  if (n16 == 0) {
    s_m[wave][ha] = ma;
    s_l[wave][ha] = static_cast<float>(la);
    if (LIMBS == 2) {
      s_m[wave][hb] = mb;
      s_l[wave][hb] = static_cast<float>(lb);
    }
  }
  if (LIMBS == 3 && lane >= 4 && lane < 8) {
    s_m[wave][lane] = -INFINITY;
    s_l[wave][lane] = 0.f;
  }
  __syncthreads();                       // every wave is done with its tile area
  if (tid < 8) {
    float m = -INFINITY;
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, s_m[w][tid]);
    float l = 0.f;
    for (int w = 0; w < WAVES; ++w)
      if (s_m[w][tid] != -INFINITY) l += s_l[w][tid] * __builtin_amdgcn_exp2f(s_m[w][tid] - m);
    s_M[tid] = m;
    s_L[tid] = l;
  }
  __syncthreads();
  {
    // limb merge: lanes 0..31 (limb 0 rows) take the limb-1 rows of lanes 32..63; lane
    // group grp<2 then holds head slots 4*grp + r, scaled to the workgroup max
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * (grp & 1) + r;
      const float mine = s_m[wave][hd];
      f[r] = (mine == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mine - s_M[hd]);
    }
#pragma unroll
    for (int v = 0; v < NVB; ++v) {
      if (v < NV) {
        float4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const auto sw = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(acc[v][r]),
                                                           static_cast<unsigned>(acc[v][r]), false, false);
          const float c = (128.f * static_cast<float>(acc[v][r]) + static_cast<float>(static_cast<int>(sw[1]))) * f[r];
          if (r == 0) o.x = c;
          if (r == 1) o.y = c;
          if (r == 2) o.z = c;
          if (r == 3) o.w = c;
        }
        if (lane < 32) reinterpret_cast<float4*>(mg)[(wave * NVB + v) * 32 + lane] = o;
      }
    }
  }
  __syncthreads();
  // ---- 6. partial records: [max, sum, 0, 0, column sums]
  {
    const int ncol = ok ? 16 * NV : 0;     // a bad blob's field count may not fit a record
    float* rec = a.part + (static_cast<int64_t>(bh) * a.S + s) * G * a.prec;
    for (int e = tid; e < G * ncol; e += NT) {
      const int hd = e / ncol, col = e - hd * ncol;
      const int v = col >> 4, ln = (col & 15) + 16 * (hd >> 2), r = hd & 3;
      float sum = 0.f;
#pragma unroll 4
      for (int w = 0; w < WAVES; ++w) sum += mg[((w * NVB + v) * 32 + ln) * 4 + r];
      rec[hd * a.prec + PHDR + col] = sum;
    }
    if (tid < G) {
      float* r0 = rec + tid * a.prec;
      r0[0] = ok ? s_M[tid] : NAN;
      r0[1] = s_L[tid];
      r0[2] = 0.f;
      r0[3] = 0.f;
    }
  }
}

// Merge of the S partial records of one (batch, KV head, q head); out and lse.
constexpr int CNT = 256;                 // combine threads (4 waves)
constexpr int CR_BYTES = D * D * 4;      // LDS for R_V (fp32) when the rotation is a KLT

struct CombArgs {
  const aatc_calib* vcal;
  const float* part;
  const float* offs;
  int n_kv, n_q, group, S, prec;
  int SC;                                // splits per LDS chunk of records
  int rec_bytes;                         // LDS bytes of one chunk (multiple of 1024)
  const int32_t* seq_lens;
  int64_t max_seq;
  float* out;
  float* lse;
};

#ifdef AATC_ATTN_COMBINE_TU   // defined by the one translation unit that launches it
// Copies n16 16-byte units, unit e = (record e / q4, quad e % q4) of records spaced `stride`
// floats apart, into consecutive LDS quads; lanes past n16 re-read unit 0 (padding).
__device__ inline int dma_records(const float* rec0, int64_t stride, int q4, int n16, uint8_t* dst, int k, int wave,
                                  int lane) {
  for (int i = 0; i < n16; i += 64, ++k)
    if (k % (CNT / 64) == wave) {
      const int e = i + lane < n16 ? i + lane : 0;
      const int sp = e / q4, qd = e - sp * q4;
      const float* p = rec0 + sp * stride + 4 * qd;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p), dst + i * 16, 16, 0, 0);
    }
  return k;
}

__global__ __launch_bounds__(CNT) void k_attn_combine(CombArgs a) {
  extern __shared__ __align__(16) unsigned char csm[];
  float* recs = reinterpret_cast<float*>(csm);                        // [SC][prec]
  float* rv = reinterpret_cast<float*>(csm + a.rec_bytes);            // [128][128] (KLT)
  __shared__ __align__(16) float t_o[D], t_delta[D];
  __shared__ __align__(16) uint8_t t_bits[256];
  __shared__ __align__(16) int16_t t_cf[3 * D];
  __shared__ __align__(16) uint8_t t_fs[512];
  __shared__ float wsl[1024];
  __shared__ float csum[3 * D];
  __shared__ float yt[D];
  __shared__ float red[CNT / 64][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group, S = a.S, prec = a.prec, SC = a.SC, q4 = prec / 4;
  const int bh = b * a.n_kv + h;
  const aatc_calib* vc = a.vcal + h;
  const float* rec0 = a.part + (static_cast<int64_t>(bh) * S * G + g) * prec;
  const int64_t stride = static_cast<int64_t>(G) * prec;

  // records of the first chunk, the V tables and (KLT) R_V, all in flight at once
  int k = 0;
  const int n0 = S < SC ? S : SC;
  k = dma_records(rec0, stride, q4, n0 * q4, csm, k, wave, lane);
  k = dma_words<CNT / 64>(vc->o32, t_o, D, k, wave, lane);
  k = dma_words<CNT / 64>(vc->delta32, t_delta, D, k, wave, lane);
  k = dma_words<CNT / 64>(vc->bits, t_bits, D / 4, k, wave, lane);
  k = dma_words<CNT / 64>(vc->channel_field, t_cf, 3 * D / 2, k, wave, lane);
  k = dma_words<CNT / 64>(vc->field_shift, t_fs, 3 * D / 4, k, wave, lane);
  const int rot = vc->rotation;
  if (rot == AATC_ROT_KLT) k = dma_words<CNT / 64>(vc->R32, rv, D * D, k, wave, lane);
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[b]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);
  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4;
  const int ncol_blob = 16 * (T4 + T2 + ((n1 + 15) >> 4));
  bool bad = PHDR + ncol_blob > prec;      // fields that do not fit a record: NaN result
  const int ncol = bad ? 0 : ncol_blob;
  for (int e = tid; e < 3 * D; e += CNT) csum[e] = 0.f;

  float M = -INFINITY, L = 0.f;
  for (int c0 = 0; c0 < S; c0 += SC) {
    const int n = S - c0 < SC ? S - c0 : SC;
    if (c0 > 0) dma_records(rec0 + c0 * stride, stride, q4, n * q4, csm, 0, wave, lane);
    wait_vmcnt(0);
    __syncthreads();
    // chunk max; rescale what is already summed
    float m = -INFINITY;
    bool nan = false;
    for (int sp = tid; sp < n; sp += CNT) {
      const float v = recs[sp * prec];
      nan |= v != v;
      m = fmaxf(m, v);
    }
    m = wave_max(m);
    nan = __ballot(nan) != 0;
    if (lane == 0) {
      red[wave][0] = m;
      red[wave][1] = nan ? 1.f : 0.f;
    }
    __syncthreads();
    float cm = -INFINITY;
    for (int w = 0; w < CNT / 64; ++w) {
      cm = fmaxf(cm, red[w][0]);
      bad |= red[w][1] != 0.f;
    }
    const float nM = fmaxf(M, cm);
    const float fold = (M == -INFINITY) ? 0.f : exp2f(M - nM);
    float l = 0.f;
    for (int sp = tid; sp < n; sp += CNT) {
      const float v = recs[sp * prec];
      const float w = (v == -INFINITY || nM == -INFINITY) ? 0.f : exp2f(v - nM);
      wsl[sp] = w;
      l += w * recs[sp * prec + 1];
    }
    l = wave_sum(l);
    __syncthreads();                      // red is reused; wsl is complete
    if (lane == 0) red[wave][0] = l;
    __syncthreads();
    float lc = 0.f;
    for (int w = 0; w < CNT / 64; ++w) lc += red[w][0];
    L = L * fold + lc;
    M = nM;
    for (int col = tid; col < ncol; col += CNT) {
      float sacc = csum[col] * fold;
      for (int sp = 0; sp < n; ++sp) sacc += wsl[sp] * recs[sp * prec + PHDR + col];
      csum[col] = sacc;
    }
    __syncthreads();                      // recs, wsl and red are reused by the next chunk
  }
  // fold field columns into channel code sums; y = o + delta (c_bar - 2^(b-1) + 1/2)
  for (int i = tid; i < D; i += CNT) {
    float cs = 0.f;
    for (int kk = 0; kk < 3; ++kk) {
      const int f = t_cf[3 * i + kk];
      if (f < 0 || f >= AATC_MAX_FIELDS) break;
      int col;
      if (f < n4) col = f;
      else if (f < n4 + n2) col = 16 * T4 + (f - n4);
      else col = 16 * (T4 + T2) + (f - n4 - n2);
      if (col < ncol) cs += ldexpf(csum[col], t_fs[f]);
    }
    const int bi = t_bits[i];
    float y = t_o[i];
    if (bi && L > 0.f) y = t_o[i] + t_delta[i] * (cs / L - (static_cast<float>(1 << (bi - 1)) - 0.5f));
    yt[i] = y;
  }
  __syncthreads();
  float o = 0.f;
  if (rot == AATC_ROT_WHT) {
    if (wave == 0) {
      float x0 = yt[lane], x1 = yt[64 + lane];
      const float y = x0;
      x0 = y + x1;
      x1 = y - x1;
#pragma unroll
      for (int len = 1; len < 64; len <<= 1) {
        const float o0 = __shfl_xor(x0, len), o1 = __shfl_xor(x1, len);
        const bool hi = (lane & len) != 0;
        x0 = hi ? o0 - x0 : x0 + o0;
        x1 = hi ? o1 - x1 : x1 + o1;
      }
      csum[lane] = x0 * 0.08838834764831845f;
      csum[64 + lane] = x1 * 0.08838834764831845f;
    }
  } else if (rot == AATC_ROT_KLT) {
    // out_j = sum_i R[i][j] y_i: two threads per output, 64 rows each
    const int j = tid & 127, hf = tid >> 7;
#pragma unroll 16
    for (int i = 64 * hf; i < 64 * hf + 64; ++i) o = fmaf(rv[i * D + j], yt[i], o);
  } else if (tid < D) {
    csum[tid] = yt[tid];
  }
  __syncthreads();
  if (rot == AATC_ROT_KLT) {
    if (tid >= 128) csum[tid - 128] = o;
    __syncthreads();
    if (tid < 128) csum[128 + tid] = o + csum[tid];
    __syncthreads();
  }
  const float* res = rot == AATC_ROT_KLT ? csum + 128 : csum;
  const int64_t qh = static_cast<int64_t>(b) * a.n_q + h * G + g;
  const bool empty = seq == 0;
  for (int j = tid; j < D; j += CNT)
    a.out[qh * D + j] = bad ? NAN : (L > 0.f ? res[j] : (empty ? 0.f : NAN));
  if (a.lse && tid == 0) {
    const float l2 = bad ? NAN : (L > 0.f ? M + log2f(L / static_cast<float>(PS)) + a.offs[bh * 8 + g]
                                          : (empty ? -INFINITY : NAN));
    a.lse[qh] = l2 * 0.69314718055994530942f;
  }
}
#endif

template <int NP, int NVB, int LIMBS>
hipError_t launch_one(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_attn_main<NP, NVB, LIMBS>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn_main<NP, NVB, LIMBS>), grid, dim3(waves_for(NP, NVB) * 64), lds, st, a);
  return hipGetLastError();
}

template <int NP, int NVB>
hipError_t launch_limbs(int limbs, const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  return limbs == 3 ? launch_one<NP, NVB, 3>(a, grid, lds, st) : launch_one<NP, NVB, 2>(a, grid, lds, st);
}

// One translation unit per NP instantiates this (all V buckets and limb modes).
template <int NP>
hipError_t launch_np(int nvb, int limbs, const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st, bool* found) {
  *found = true;
  switch (nvb) {
    case 8: return launch_limbs<NP, 8>(limbs, a, grid, lds, st);
    case 12: return launch_limbs<NP, 12>(limbs, a, grid, lds, st);
    case 16: return launch_limbs<NP, 16>(limbs, a, grid, lds, st);
    case 24: return launch_limbs<NP, 24>(limbs, a, grid, lds, st);
  }
  *found = false;
  return hipSuccess;
}

extern template hipError_t launch_np<1>(int, int, const AttnArgs&, dim3, size_t, hipStream_t, bool*);
extern template hipError_t launch_np<2>(int, int, const AttnArgs&, dim3, size_t, hipStream_t, bool*);
extern template hipError_t launch_np<3>(int, int, const AttnArgs&, dim3, size_t, hipStream_t, bool*);
extern template hipError_t launch_np<4>(int, int, const AttnArgs&, dim3, size_t, hipStream_t, bool*);

}  // namespace aatc_attn
