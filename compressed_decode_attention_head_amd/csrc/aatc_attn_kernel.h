// Decode attention that reads the packed cache directly (gfx950), one kernel per step.
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
//   LIMBS=2: 8 q-head slots x 2 limbs (15-bit weights, 14-bit probabilities), GQA <= 8;
//   LIMBS=3: 4 q-head slots x 3 limbs (22-bit weights, 21-bit probabilities), GQA <= 4.
//
// Work split: grid (S splits, KV heads, batch); a workgroup of 8 waves owns a contiguous
// range of 64-token tiles of one sequence, each wave `tpw` consecutive tiles.  Every wave
//   1. copies its tiles straight from HBM into its LDS area with global_load_lds (16 bytes
//      per lane, no registers), the whole range at once or in double-buffered chunks,
//   2. while those loads fly, the workgroup rotates the queries and builds limb weights,
//   3. streams its tiles out of LDS: scores -> online softmax -> PV, int32 accumulators,
// then the workgroup merges its waves in LDS, writes one partial (max, sum, 128 channel code
// sums per q head) to its slot, and the last workgroup of a (sequence, KV head) (atomic
// counter) merges the slots, dequantizes, applies R_V^T and writes out/lse.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace aatc_attn {

constexpr int D = AATC_D;
constexpr int WAVES = 8;
constexpr int NT = WAVES * 64;
constexpr int PROW_MAX = 130;         // partial row: max, sum, 128 channel sums
constexpr int UNION_BYTES = 3 * 8 * D * 4;   // prologue q/q~/alpha; later acc_s, finalize
constexpr int PL_BYTES = WAVES * 16 * 64;    // probability limb bytes, per wave 16 rows x 64
typedef int v4i __attribute__((ext_vector_type(4)));

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
  float* part;                        // [batch*n_kv][S][8][PROW_MAX]
  unsigned* counters;                 // [batch*n_kv]
  int S, tpw;
  int kB, vB;
  int np_half;                        // 1 if the last K pair carries <= 64 planes
  int chunk;                          // tiles per LDS chunk
  int nbuf;                           // 1 or 2 chunk buffers per wave
  int ks_bytes, vs_bytes;             // K / V area of one chunk buffer (multiples of 1024)
};

__device__ inline float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  return x;
}

__device__ inline int row_sum16(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);
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

__device__ inline long long wave_sum_ll(long long x) {
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

// Waits until at most n (0..31) vector-memory instructions of this wave are outstanding.
__device__ inline void wait_vmcnt(int n) {
#define AATC_VMW(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
  switch (n) {
    AATC_VMW(0) AATC_VMW(1) AATC_VMW(2) AATC_VMW(3) AATC_VMW(4) AATC_VMW(5) AATC_VMW(6) AATC_VMW(7)
    AATC_VMW(8) AATC_VMW(9) AATC_VMW(10) AATC_VMW(11) AATC_VMW(12) AATC_VMW(13) AATC_VMW(14) AATC_VMW(15)
    AATC_VMW(16) AATC_VMW(17) AATC_VMW(18) AATC_VMW(19) AATC_VMW(20) AATC_VMW(21) AATC_VMW(22) AATC_VMW(23)
    AATC_VMW(24) AATC_VMW(25) AATC_VMW(26) AATC_VMW(27) AATC_VMW(28) AATC_VMW(29) AATC_VMW(30) AATC_VMW(31)
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
  static constexpr int PS = 16383;       // probability scale
  static constexpr int PROW = 8;         // row stride between limbs
  __device__ static int limb(int l, int v) { return l == 0 ? (v >> 7) : (v & 127); }
};
template <>
struct Lim<3> {
  static constexpr int WBITS = 21;
  static constexpr int PS = (1 << 21) - 1;
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

template <int NP, int NVB, int LIMBS>
__global__ __launch_bounds__(NT) void k_attn(AttnArgs a) {
  using LM = Lim<LIMBS>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);                       // [8][128]   (prologue)
  float* qt = qs + 8 * D;                                           // [8][128]   (prologue)
  float* al = qt + 8 * D;                                           // [8][128]   (prologue)
  float* acc_s = qs;                                                // [8][16*NVB] (merge)
  uint8_t* pl = smem + UNION_BYTES;                                 // [WAVES][16][64]
  int* wa_lds = reinterpret_cast<int*>(pl);                         // [NP*2*4*64] (prologue)
  uint8_t* chunks = pl + PL_BYTES;                                  // [WAVES][nbuf][ks+vs]
  __shared__ float mws[WAVES][8];
  __shared__ int wexp[8];
  __shared__ float esc[8], mref[8], offs[8], l_s[8], mhead[8];
  __shared__ int last_flag;

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
  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4, T1 = (n1 + 15) >> 4;
  const int NV = T4 + T2 + T1;
  const bool ok = kc->magic == AATC_MAGIC && vc->magic == AATC_MAGIC && kc->total_bits == Bk &&
                  vc->total_bits == Bv && NV <= NVB;
  const bool half = a.np_half != 0;

  // ---- 1. start the tile DMA: chunk 0 (and chunk 1 when double-buffered)
  const int64_t kbytes = 8 * static_cast<int64_t>(Bk), vbytes = 8 * static_cast<int64_t>(Bv);
  const char* kseq = reinterpret_cast<const char*>(a.kcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * kbytes;
  const char* vseq = reinterpret_cast<const char*>(a.vcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * vbytes;
  const char* kend = kseq + a.tiles_per_seq * kbytes;
  const char* vend = vseq + a.tiles_per_seq * vbytes;
  const int CH = a.chunk, NBUF = a.nbuf;
  const int nki = Bk > 0 ? a.ks_bytes >> 10 : 0, nvi = Bv > 0 ? a.vs_bytes >> 10 : 0;
  uint8_t* wbuf = chunks + static_cast<size_t>(wave) * NBUF * (a.ks_bytes + a.vs_bytes);
  const int64_t ntile_w = (ok && t1 > t0) ? t1 - t0 : 0;
  const int nchunks = static_cast<int>((ntile_w + CH - 1) / CH);
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
  if (nchunks > 0) issue(0, 0);
  if (nchunks > 1 && NBUF == 2) issue(1, 1);

  // ---- 2. prologue: q~ = R_K q, alpha, exponents, score bound, limb weights
  for (int e = tid; e < 8 * D; e += NT) {
    const int g = e >> 7, j = e & 127;
    qs[e] = (g < G) ? a.q[(static_cast<int64_t>(b) * a.n_q + h * G + g) * D + j] : 0.f;
  }
  __syncthreads();
  if (kc->rotation == AATC_ROT_WHT) {
    // Sylvester-ordered fast Walsh-Hadamard transform of each query, then 1/sqrt(128)
    for (int e = tid; e < 8 * D; e += NT) qt[e] = qs[e];
    __syncthreads();
    for (int len = 1; len < D; len <<= 1) {
      const int g = tid >> 6, k = tid & 63;                 // 8 heads x 64 butterflies
      const int i0 = (k / len) * 2 * len + (k % len), i1 = i0 + len;
      const float x0 = qt[g * D + i0], x1 = qt[g * D + i1];
      __syncthreads();
      qt[g * D + i0] = x0 + x1;
      qt[g * D + i1] = x0 - x1;
      __syncthreads();
    }
    for (int e = tid; e < 8 * D; e += NT) qt[e] *= 0.08838834764831845f;
  } else {
    // row i of R_K: four threads per row, eight q heads per thread
    const int i = tid >> 2, qq = tid & 3;
    float part[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) part[g] = 0.f;
    const float2* row = reinterpret_cast<const float2*>(kc->R32 + i * D + 32 * qq);
#pragma unroll
    for (int c2 = 0; c2 < 16; ++c2) {
      const float2 r = row[c2];
      const int j = 32 * qq + 2 * c2;
#pragma unroll
      for (int g = 0; g < 8; ++g) part[g] += r.x * qs[g * D + j] + r.y * qs[g * D + j + 1];
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      part[g] += __shfl_xor(part[g], 1);
      part[g] += __shfl_xor(part[g], 2);
    }
    if (qq == 0)
#pragma unroll
      for (int g = 0; g < 8; ++g) qt[g * D + i] = part[g];
  }
  __syncthreads();
  {
    // one wave per head slot: alpha, the lse offset, the exponent and the score bound
    const int g = wave;
    float m = 0.f, off = 0.f;
    for (int i = lane; i < D; i += 64) {
      const int bi = kc->bits[i];
      const float v = qt[g * D + i];
      const float alpha = bi ? v * kc->delta32[i] * a.scale2 : 0.f;
      al[g * D + i] = alpha;
      if (bi) m = fmaxf(m, fabsf(alpha) * static_cast<float>(1 << (bi - 1)));
      const float o = bi ? kc->o32[i] - kc->delta32[i] * (static_cast<float>(1 << (bi - 1)) - 0.5f) : kc->o32[i];
      off += v * o * a.scale2;
    }
    m = wave_max(m);
    off = wave_sum(off);
    int e = 0;
    if (m > 0.f) {
      frexpf(m, &e);
      e = LM::WBITS - e;                 // m * 2^e in [2^(WBITS-1), 2^WBITS)
    }
    const int wmaxq = (1 << LM::WBITS) - 1;
    long long pos = 0;
    for (int p = lane; p < Bk; p += 64) {
      const int ch = kc->plane_channel[p], kb = kc->plane_bit[p];
      int wq = static_cast<int>(rintf(ldexpf(al[g * D + ch], kb + e)));
      wq = wq > wmaxq ? wmaxq : (wq < -wmaxq ? -wmaxq : wq);
      if (wq > 0) pos += wq;
    }
    pos = wave_sum_ll(pos);
    if (lane == 0) {
      wexp[g] = e;
      esc[g] = (m > 0.f) ? ldexpf(1.f, -e) : 0.f;
      mref[g] = (m > 0.f) ? ldexpf(static_cast<float>(pos), -e) : 0.f;
      offs[g] = off;
      l_s[g] = 0.f;
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
          const int ch = kc->plane_channel[p], kb = kc->plane_bit[p];
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
  for (int e = tid; e < PL_BYTES / 4; e += NT) reinterpret_cast<uint32_t*>(pl)[e] = 0u;
  __syncthreads();
  // head slots this lane holds after the limb merge: LIMBS=2 pair a {0,4,1,5}[grp] and
  // pair b {2,6,3,7}[grp]; LIMBS=3 head grp
  const int ha = LIMBS == 2 ? (grp & 1) * 4 + (grp >> 1) : grp;
  const int hb = ha + 2;
  const float esa = esc[ha], esb = LIMBS == 2 ? esc[hb] : 0.f;
  int pbase[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) pbase[u] = plane_base(u, grp, half && u == NP - 1);
  const int tokoff = n16 * Bk;
  uint8_t* pw = pl + wave * 16 * 64;

  v4i acc[NVB];
#pragma unroll
  for (int v = 0; v < NVB; ++v) acc[v] = v4i{0, 0, 0, 0};
  float ma = -INFINITY, mb = -INFINITY;
  int la = 0, lb = 0;

  // ---- 3. stream the chunks out of LDS
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
      // scores: 4 groups of 16 tokens (token 16*tau + n16)
      float sa[4], sb[4];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        v4i cc = {0, 0, 0, 0};
        const int tb = tokoff + tau * 16 * Bk;
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const bool hp = half && u == NP - 1;
          uint32_t dw = 0;
          if (pbase[u] < Bk) {
            const int o = tb + pbase[u];
            const int wi = o >> 5;
            dw = __builtin_amdgcn_alignbit(kl[wi + 1], kl[wi], static_cast<uint32_t>(o));
          }
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
          sa[tau] = static_cast<float>((static_cast<int>(p01[0]) << 7) + static_cast<int>(p01[1])) * esa;
          sb[tau] = static_cast<float>((static_cast<int>(p23[0]) << 7) + static_cast<int>(p23[1])) * esb;
        } else {
          // 4x4 transpose of 16-lane blocks: rows (limb l, head r) -> lane group = head
          const auto x02 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[0]), static_cast<unsigned>(cc[2]),
                                                            false, false);
          const auto x13 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[1]), static_cast<unsigned>(cc[3]),
                                                            false, false);
          const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);   // limb 0, limb 1
          const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);   // limb 2, unused
          const int si = (static_cast<int>(y01[0]) << 14) + (static_cast<int>(y01[1]) << 7) + static_cast<int>(y23[0]);
          sa[tau] = static_cast<float>(si) * esa;
          sb[tau] = -INFINITY;
        }
      }
      const int64_t nvalid = seq - tile * 64;
      if (nvalid < 64) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
          if (16 * tau + n16 >= nvalid) { sa[tau] = -INFINITY; sb[tau] = -INFINITY; }
      }
      const float mta = row_max16(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])));
      const float mtb = LIMBS == 2 ? row_max16(fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3]))) : -INFINITY;
      // online softmax: rescale the integer accumulators when a running max grows
      if (__ballot(mta > ma || mtb > mb)) {
        const float nma = fmaxf(ma, mta), nmb = fmaxf(mb, mtb);
        const float fa = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - nma);
        const float fb = (mb == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mb - nmb);
        la = static_cast<int>(rintf(static_cast<float>(la) * fa));
        lb = static_cast<int>(rintf(static_cast<float>(lb) * fb));
        ma = nma;
        mb = nmb;
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
          // acc register r holds head r; head r's factor lives in lane group r
#pragma unroll
          for (int r = 0; r < 4; ++r) fr[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fa), 16 * r));
        }
#pragma unroll
        for (int v = 0; v < NVB; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[v][r] = static_cast<int>(rintf(static_cast<float>(acc[v][r]) * fr[r]));
      }
      // probabilities as fixed point -> limb bytes in LDS, row = limb * PROW + head
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const int t = 16 * tau + n16;
        const int pa = static_cast<int>(fmaf(__builtin_amdgcn_exp2f(sa[tau] - ma), static_cast<float>(LM::PS), 0.5f));
        la += pa;
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) pw[(l * LM::PROW + ha) * 64 + t] = static_cast<uint8_t>(LM::limb(l, pa));
        if (LIMBS == 2) {
          const int pb = static_cast<int>(fmaf(__builtin_amdgcn_exp2f(sb[tau] - mb), static_cast<float>(LM::PS), 0.5f));
          lb += pb;
#pragma unroll
          for (int l = 0; l < LIMBS; ++l) pw[(l * LM::PROW + hb) * 64 + t] = static_cast<uint8_t>(LM::limb(l, pb));
        }
      }
      wave_sync_lds();
      const uint4 pv = *reinterpret_cast<const uint4*>(pw + n16 * 64 + 16 * grp);
      const v4i pA = {static_cast<int>(pv.x), static_cast<int>(pv.y), static_cast<int>(pv.z), static_cast<int>(pv.w)};
      // PV on packed V fields (width-uniform column groups: w4 | w2 | w1)
#pragma unroll
      for (int v = 0; v < NVB; ++v) {
        if (v < NV) {
          v4i bv = {0, 0, 0, 0};
          if (v < T4) {
            const int k = (v << 4) + n16;
            if (k < n4) {
              const uint2 d2 = *reinterpret_cast<const uint2*>(vl + 8 * k + 2 * grp);
              const uint32_t m4 = 0x0F0F0F0Fu;
              bv[0] = static_cast<int>(d2.x & m4);
              bv[1] = static_cast<int>((d2.x >> 4) & m4);
              bv[2] = static_cast<int>(d2.y & m4);
              bv[3] = static_cast<int>((d2.y >> 4) & m4);
            }
          } else if (v < T4 + T2) {
            const int k = ((v - T4) << 4) + n16;
            if (k < n2) {
              const uint32_t d = vl[8 * n4 + 4 * k + grp];
#pragma unroll
              for (int r = 0; r < 4; ++r) bv[r] = static_cast<int>((d >> (2 * r)) & 0x03030303u);
            }
          } else {
            const int k = ((v - T4 - T2) << 4) + n16;
            if (k < n1) {
              const uint32_t d = vl[8 * n4 + 4 * n2 + 2 * k + (grp >> 1)] >> (4 * (grp & 1));
#pragma unroll
              for (int r = 0; r < 4; ++r) bv[r] = static_cast<int>((d >> r) & 0x01010101u);
            }
          }
          acc[v] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pA, bv, acc[v], 0, 0, 0);
        }
      }
      wave_sync_lds();
    }
    if (NBUF == 2 && c + 2 < nchunks) issue(c + 2, buf);
    else if (NBUF == 1 && c + 1 < nchunks) issue(c + 1, 0);
  }

  // ---- 4. workgroup merge in LDS
  la = row_sum16(la);
  lb = row_sum16(lb);
  if (n16 == 0) {
    mws[wave][ha] = ma;
    if (LIMBS == 2) mws[wave][hb] = mb;
  }
  if (LIMBS == 3 && lane < 4) mws[wave][4 + lane] = -INFINITY;
  for (int e = tid; e < 8 * 16 * NVB; e += NT) acc_s[e] = 0.f;
  __syncthreads();
  if (tid < 8) {
    float m = -INFINITY;
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, mws[w][tid]);
    mhead[tid] = m;
  }
  __syncthreads();
  if (n16 == 0) {
    const float sca = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - mhead[ha]);
    if (ha < G && sca != 0.f) atomicAdd(&l_s[ha], static_cast<float>(la) * sca);
    if (LIMBS == 2) {
      const float scb = (mb == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mb - mhead[hb]);
      if (hb < G && scb != 0.f) atomicAdd(&l_s[hb], static_cast<float>(lb) * scb);
    }
  }
  {
    const int l = LIMBS == 2 ? (grp >> 1) : grp;
    const float lw = static_cast<float>(1 << (7 * (LIMBS - 1 - (l < LIMBS ? l : 0))));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = LIMBS == 2 ? 4 * (grp & 1) + r : r;
      const float mine = mws[wave][hd];
      const float scr = (mine == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mine - mhead[hd]) * lw;
      if (l < LIMBS && hd < G && scr != 0.f) {
#pragma unroll
        for (int v = 0; v < NVB; ++v)
          if (v < NV && acc[v][r] != 0)
            atomicAdd(&acc_s[hd * 16 * NVB + 16 * v + n16], static_cast<float>(acc[v][r]) * scr);
      }
    }
  }
  __syncthreads();
  // ---- 5. partial slot: max, sum and 128 channel code sums per q head (fields folded)
  float* slot = a.part + (static_cast<int64_t>(bh) * a.S + s) * 8 * PROW_MAX;
  for (int e = tid; e < G * D; e += NT) {
    const int hd = e >> 7, i = e & 127;
    float cs = 0.f;
    for (int k = 0; k < 3; ++k) {
      const int f = vc->channel_field[3 * i + k];
      if (f < 0) break;
      int col;
      if (f < n4) col = f;
      else if (f < n4 + n2) col = 16 * T4 + (f - n4);
      else col = 16 * (T4 + T2) + (f - n4 - n2);
      cs += ldexpf(acc_s[hd * 16 * NVB + col], vc->field_shift[f]);
    }
    slot[hd * PROW_MAX + 2 + i] = cs;
    if (i == 0) {
      slot[hd * PROW_MAX] = ok ? mhead[hd] : NAN;
      slot[hd * PROW_MAX + 1] = l_s[hd];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(a.counters + bh, 1u);
    last_flag = (prev == static_cast<unsigned>(a.S - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();

  // ---- 6. last workgroup: merge the S slots, out = R_V^T (o + delta (c_bar - 2^(b-1) + 1/2))
  float* yt = qs;                        // [8][128]
  float* ot = qt;                        // [8][128]
  float* wsl = reinterpret_cast<float*>(chunks);   // [8][S] slot weights (tile area is free now)
  const float* slots = a.part + static_cast<int64_t>(bh) * a.S * 8 * PROW_MAX;
  float* Lh = &mhead[0];                  // reuse: per-head total sum
  {
    const int hd = wave;                  // one wave per head slot
    float m = -INFINITY;
    bool bad = false;
    for (int sp = lane; sp < a.S; sp += 64) {
      const float v = __hip_atomic_load(slots + (static_cast<int64_t>(sp) * 8 + hd) * PROW_MAX, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      bad |= (v != v);
      m = fmaxf(m, v);
    }
    m = wave_max(m);
    bad = __ballot(bad) != 0;
    float lsum = 0.f;
    for (int sp = lane; sp < a.S; sp += 64) {
      const float* sl = slots + (static_cast<int64_t>(sp) * 8 + hd) * PROW_MAX;
      const float mv = __hip_atomic_load(sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float w = (mv == -INFINITY || m == -INFINITY) ? 0.f : exp2f(mv - m);
      wsl[hd * a.S + sp] = w;
      lsum += w * __hip_atomic_load(sl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lsum = wave_sum(lsum);
    if (lane == 0) {
      Lh[hd] = bad ? NAN : lsum;
      mws[0][hd] = m;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int hd = e >> 7, i = e & 127;
    float csum = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < a.S; ++sp)
      csum += wsl[hd * a.S + sp] *
              __hip_atomic_load(slots + (static_cast<int64_t>(sp) * 8 + hd) * PROW_MAX + 2 + i, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    const float L = Lh[hd];
    const int bi = vc->bits[i];
    float y = vc->o32[i];
    if (bi && L > 0.f) y = vc->o32[i] + vc->delta32[i] * (csum / L - (static_cast<float>(1 << (bi - 1)) - 0.5f));
    yt[e] = y;
  }
  __syncthreads();
  if (vc->rotation == AATC_ROT_WHT) {
    for (int len = 1; len < D; len <<= 1) {
      const int g = tid >> 6, k = tid & 63;
      const int i0 = (k / len) * 2 * len + (k % len), i1 = i0 + len;
      float x0 = 0.f, x1 = 0.f;
      if (g < G) { x0 = yt[g * D + i0]; x1 = yt[g * D + i1]; }
      __syncthreads();
      if (g < G) { yt[g * D + i0] = x0 + x1; yt[g * D + i1] = x0 - x1; }
      __syncthreads();
    }
    for (int e = tid; e < G * D; e += NT) ot[e] = yt[e] * 0.08838834764831845f;
  } else {
    for (int e = tid; e < G * D; e += NT) {
      const int hd = e >> 7, j = e & 127;
      float o = 0.f;
#pragma unroll 8
      for (int i = 0; i < D; ++i) o = fmaf(vc->R32[i * D + j], yt[hd * D + i], o);
      ot[e] = o;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int hd = e >> 7, j = e & 127;
    const float L = Lh[hd];
    const int64_t oi = (static_cast<int64_t>(b) * a.n_q + h * G + hd) * D + j;
    a.out[oi] = (L != L) ? NAN : (L > 0.f ? ot[e] : (ntiles > 0 ? NAN : 0.f));
  }
  if (a.lse && tid < G) {
    const float L = Lh[tid];
    const float l2 = (L != L) ? NAN
                              : (L > 0.f ? mws[0][tid] + log2f(L / static_cast<float>(LM::PS)) + offs[tid]
                                         : (ntiles > 0 ? NAN : -INFINITY));
    a.lse[static_cast<int64_t>(b) * a.n_q + h * G + tid] = l2 * 0.69314718055994530942f;
  }
  if (tid == 0) atomicExch(a.counters + bh, 0u);
}

template <int NP, int NVB, int LIMBS>
hipError_t launch_one(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_attn<NP, NVB, LIMBS>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn<NP, NVB, LIMBS>), grid, dim3(NT), lds, st, a);
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
