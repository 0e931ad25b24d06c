// Encode (rotate -> quantize -> pack) and decode (unpack -> dequantize -> rotate back)
// kernels for gfx950, plus their C-ABI launchers.
//
// Page "KV Cache Compression Through the Lens of Transform Coding" (Full text): transform
// coding of the cache; page "SPECTRA ..." (Abstract): the cache is re-encoded in the rotated
// coordinate system; page "Ablation, Statistical Inference, and Validation for KV-Cache
// Compression" (first abstract): a scalar MSE quantizer after the rotation.
//
// One workgroup owns one 64-token tile of one (batch, KV head) sequence, so every packed
// word has exactly one writer.  Rotation and quantization run in fp64 so that codes agree
// with an fp64 definition except for values within rounding distance of a bin edge.
// This file is compiled with -ffp-contract=off: the quantizer expression must be the
// separately rounded fp64 sequence of the format definition; the GEMM uses explicit fma().
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "aatc_internal.h"

namespace {

constexpr int D = AATC_D;
constexpr int T = AATC_TILE;
constexpr int KC = 32;          // rotation rows staged per LDS chunk
constexpr int THREADS = 256;
constexpr size_t kDecodeLds = T * D * 8 + KC * D * 8 + D * 4;   // y_hat (f64), R chunk, plane bases

__device__ inline double load_x(const void* x, int dt, int64_t i) {
  if (dt == AATC_F32) return static_cast<double>(static_cast<const float*>(x)[i]);
  const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(x)[i]) << 16;
  return static_cast<double>(__uint_as_float(u));
}

__device__ inline void store_out(void* out, int dt, int64_t i, double v) {
  if (dt == AATC_F32) {
    static_cast<float*>(out)[i] = static_cast<float>(v);
  } else {  // bf16, round to nearest even from fp32
    const float f = static_cast<float>(v);
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      u = 0x7fc00000u;
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
    }
    static_cast<uint16_t*>(out)[i] = static_cast<uint16_t>(u >> 16);
  }
}

// Y[t][i] = sum_k A[t][k] * M(i,k) for a 64x128 tile, fp64; A in LDS (row stride D),
// M(i,k) = R[i*D+k] when TRANS_R (encode: y = R x), R[k*D+i] otherwise (decode: R^T y).
// 256 threads, each owns 4 tokens x 8 channels.  Rows of R are staged through LDS.
template <bool TRANS_R, class AT>
__device__ void tile_gemm(const AT* A, const double* __restrict__ R, double* mchunk, double acc[4][8]) {
  const int tid = threadIdx.x;
  const int tb = tid >> 4, cb = tid & 15;
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  for (int k0 = 0; k0 < D; k0 += KC) {
    __syncthreads();
    for (int e = tid; e < KC * D; e += THREADS) {
      const int kk = e / D, i = e % D;   // mchunk[kk][i] = M(i, k0+kk)
      mchunk[kk * D + i] = TRANS_R ? R[i * D + k0 + kk] : R[(k0 + kk) * D + i];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      double av[4], mv[8];
      for (int a = 0; a < 4; ++a) av[a] = static_cast<double>(A[(tb * 4 + a) * D + k0 + kk]);
      for (int b = 0; b < 8; ++b) mv[b] = mchunk[kk * D + cb * 8 + b];
      for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 8; ++b) acc[a][b] = fma(av[a], mv[b], acc[a][b]);
    }
  }
}

// V field strings (2w words per field and tile).  Bit b of the w-bit value of token
// t = 16G + 4r + m sits at string bit
//   w=1: 32(G/2) + 8m + 2r + G%2,   w=2: 32G + (8m + 2r + b + G%2) mod 32,
//   w=4: 64G + 32(r/2) + 8m + 4(r%2) + b,
// so the attention kernel expands every w<=2 word with one per-lane rotation and shared shifts.
__device__ inline int v_bit(int t, int w, int b) {
  const int G = t >> 4, r = (t >> 2) & 3, m = t & 3;
  if (w == 1) return 32 * (G >> 1) + 8 * m + 2 * r + (G & 1);
  if (w == 2) return 32 * G + ((8 * m + 2 * r + b + (G & 1)) & 31);
  return 64 * G + 32 * (r >> 1) + 8 * m + 4 * (r & 1) + b;
}

// Token and value bit held by bit q of word j of a field string (the inverse of v_bit).
__device__ inline int v_token(int j, int q, int w, int* bit) {
  int G, r, m;
  if (w == 1) {
    G = 2 * j + (q & 1);
    m = q >> 3;
    r = (q & 7) >> 1;
    *bit = 0;
  } else if (w == 2) {
    const int u = (q - (j & 1)) & 31;
    G = j;
    m = u >> 3;
    r = (u & 7) >> 1;
    *bit = u & 1;
  } else {
    G = j >> 1;
    m = q >> 3;
    r = 2 * (j & 1) + ((q & 7) >> 2);
    *bit = q & 3;
  }
  return 16 * G + 4 * r + m;
}

struct CodecArgs {
  const aatc_calib* calib;     // n_kv_heads blobs
  uint32_t* codes;             // packed words
  int64_t tiles_per_seq;
  int n_kv_heads;
  int which;                   // 0 = K (token-major planes), 1 = V (field-major)
  int64_t tok_off, n_tok;      // token range written / read
  int64_t tile0;               // first tile touched
  const void* x;               // encode input / decode output
  int dtype;
  int vec16;                   // encode: x and every row start 16-byte aligned
  int64_t tile_end;            // one past the last tile touched
  int64_t s_b, s_h, s_t;
};

// ---------------------------------------------------------------------------------------
// Encode.  Grid (G, KV heads, batch); a workgroup loads its head's quantizer and packing tables
// into LDS once, then walks tiles tile0 + blockIdx.x, + G, ...  Per tile:
//  1. the x rows into LDS as fp32.  With 16-byte aligned rows the next tile's rows are loaded
//     into registers while this tile computes: the barriers here wait for LDS only, and LDS
//     atomics are written by hand, so nothing waits for those loads before their use;
//  2. y = E x in fp64.  A Walsh-Hadamard blob runs the fast transform: thread = (token,
//     quarter of the channels), five butterfly stages in registers and two across lanes,
//     then one multiply by the blob's 1/sqrt(d) (its R[0]); other blobs run the 64x128x128
//     GEMM with E staged through LDS;
//  3. codes stay in the thread's registers;
//  4. the tile's packed words are OR-ed together in LDS: for K each thread appends its
//     channels' codes as one contiguous bit run per token (planes are ordered by channel), for
//     V it ORs each field value at its bit position; then one writer per word.
// ---------------------------------------------------------------------------------------
constexpr int KCE = 16;                                 // rows of E per GEMM staging chunk
constexpr size_t kXs = T * D * 4;                       // x tile, fp32
constexpr size_t kMc = KCE * D * 8;                     // E chunk, fp64; the packed words overlay it
constexpr size_t kTabO = kXs + kMc;                     // fp64 o[128], 1/delta[128]
constexpr size_t kTabBits = kTabO + 2 * D * 8;          // u8 bits[128]
constexpr size_t kTabPb = kTabBits + D;                 // u16 first plane of each channel [128]
constexpr size_t kTabFw = kTabPb + 2 * D;               // u16 first word of each field
constexpr size_t kTabFs = kTabFw + 2 * AATC_MAX_FIELDS; // u8 width | shift << 4 of each field
constexpr size_t kTabFc = kTabFs + AATC_MAX_FIELDS;     // u8 channel of each field
constexpr size_t kTabWf = kTabFc + AATC_MAX_FIELDS;     // u16 field of each V word [2*1024]
constexpr size_t kTabTh = kTabWf + 2 * 2 * AATC_D * AATC_MAX_BITS;   // fp64 Lloyd-Max thresholds
constexpr size_t kEncodeLds = kTabTh + 8 * AATC_LEVELS;
static_assert(2 * AATC_D * AATC_MAX_BITS * 4 <= kMc, "packed words fit the staging area");

// u = (y - o) * (1/Delta) + 2^(b-1) as separately rounded fp64 operations; code =
// clamp(floor(u), 0, 2^b - 1), NaN -> 0.  On [0, 2^b - 1) truncation is the floor.
// Branch-free: the clamp runs in fp64 (NaN fails u >= 0), so the conversion is always in range.
__device__ inline int quantize(double y, double o, double inv, int bi) {
  double u = (y - o) * inv;
  u = u + static_cast<double>(1 << (bi > 0 ? bi - 1 : 0));
  const double top = static_cast<double>((1 << bi) - 1);
  const double uc = u >= 0.0 ? fmin(u, top) : 0.0;
  return bi > 0 ? static_cast<int>(uc) : 0;
}

// Lloyd-Max: z = (y - o) * (1/s) as separately rounded fp64 operations; the code is the number
// of the b-bit table's 2^b - 1 ascending thresholds at or below z, by a b-step binary search
// (NaN compares false: code 0; +-Inf: the ends).
__device__ inline int quantize_lm(double y, double o, double inv, int bi, const double* thr) {
  const double z = (y - o) * inv;
  const double* t = thr + (1 << bi) - 2;
  int c = 0;
  for (int st = (1 << bi) >> 1; st > 0; st >>= 1)
    if (z >= t[c + st - 1]) c += st;
  return bi > 0 ? c : 0;
}

// The fp64 value of another lane of the same quad, by a DPP quad permutation (CTRL 0xB1: lane ^ 1,
// 0x4E: lane ^ 2) of both halves: no LDS round trip.
template <int CTRL>
__device__ inline double quad_xor(double x) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffu), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                                     static_cast<unsigned>(lo)));
}

// Workgroup barrier that waits for this wave's LDS operations only (global loads stay in flight).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// LDS OR without a return value, not ordered by the compiler against global loads in flight.
__device__ inline void lds_or(uint32_t* p, uint32_t v) {
  asm volatile("ds_or_b32 %0, %1" : : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p))), "v"(v) : "memory");
}
// OR the low n (1..32) bits of v into the bit string S at bit position pos.
__device__ inline void or_bits(uint32_t* S, int pos, uint32_t v) {
  if (!v) return;
  const int w = pos >> 5, sh = pos & 31;
  lds_or(S + w, v << sh);
  if (sh && (v >> (32 - sh))) lds_or(S + w + 1, v >> (32 - sh));
}

// y = E x for the tile (A = x in LDS), fp64, as tile_gemm but with LDS-only barriers.
__device__ void tile_gemm_e(const float* A, const double* __restrict__ E, double* mchunk, double acc[4][8]) {
  const int tid = threadIdx.x;
  const int tb = tid >> 4, cb = tid & 15;
  for (int aa = 0; aa < 4; ++aa)
    for (int bb = 0; bb < 8; ++bb) acc[aa][bb] = 0.0;
  for (int k0 = 0; k0 < D; k0 += KCE) {
    lds_barrier();
    for (int e = tid; e < KCE * D; e += THREADS) {
      const int kk = e / D, i = e % D;   // mchunk[kk][i] = E(i, k0+kk)
      mchunk[kk * D + i] = E[i * D + k0 + kk];
    }
    lds_barrier();
#pragma unroll 2
    for (int kk = 0; kk < KCE; ++kk) {
      double av[4], mv[8];
      for (int aa = 0; aa < 4; ++aa) av[aa] = static_cast<double>(A[(tb * 4 + aa) * D + k0 + kk]);
      for (int bb = 0; bb < 8; ++bb) mv[bb] = mchunk[kk * D + cb * 8 + bb];
      for (int aa = 0; aa < 4; ++aa)
        for (int bb = 0; bb < 8; ++bb) acc[aa][bb] = fma(av[aa], mv[bb], acc[aa][bb]);
    }
  }
}

// The tiles of one workgroup; WHT selects the fast transform.  Not inlined, so that each form
// gets its own register allocation (both together would spill).
template <bool WHT>
__device__ __attribute__((noinline)) void encode_tiles(const CodecArgs& a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);
  double* mchunk = reinterpret_cast<double*>(smem + kXs);
  uint32_t* S = reinterpret_cast<uint32_t*>(smem + kXs);                  // overlays mchunk
  double* t_o = reinterpret_cast<double*>(smem + kTabO);
  double* t_inv = t_o + D;
  uint8_t* t_bits = smem + kTabBits;
  uint16_t* t_pb = reinterpret_cast<uint16_t*>(smem + kTabPb);
  uint16_t* t_fw = reinterpret_cast<uint16_t*>(smem + kTabFw);
  uint8_t* t_fs = smem + kTabFs;
  uint8_t* t_fc = smem + kTabFc;
  uint16_t* t_wf = reinterpret_cast<uint16_t*>(smem + kTabWf);
  double* t_th = reinterpret_cast<double*>(smem + kTabTh);
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const aatc_calib* c = a.calib + h;
  const int B = c->total_bits, nf = c->n_fields;
  constexpr bool wht = WHT;
  const double rs = c->R[0];                           // WHT: 1/sqrt(d) as the blob holds it
  const bool lm = c->quantizer == AATC_QUANT_LLOYD_MAX;

  // ---- tables, once per workgroup
  if (tid < D) {
    t_o[tid] = c->o[tid];
    t_inv[tid] = lm ? c->inv_scale[tid] : c->inv_delta[tid];
    t_bits[tid] = c->bits[tid];
  }
  if (lm)
    for (int k = tid; k < AATC_LEVELS; k += THREADS) t_th[k] = c->thresh[k];
  for (int f = tid; f < nf; f += THREADS) {
    const int fw = c->field_word[f], wd = c->field_width[f];
    t_fw[f] = static_cast<uint16_t>(fw);
    t_fs[f] = static_cast<uint8_t>(wd | (c->field_shift[f] << 4));
    t_fc[f] = static_cast<uint8_t>(c->field_channel[f]);
    if (a.which == 1)
      for (int j = 0; j < 2 * wd; ++j) t_wf[fw + j] = static_cast<uint16_t>(f);
  }
  lds_barrier();
  if (tid < D) {
    int s0 = 0;
    for (int i = 0; i < tid; ++i) s0 += t_bits[i];
    t_pb[tid] = static_cast<uint16_t>(s0);
  }

  const int64_t xrow = b * a.s_b + h * a.s_h - a.tok_off * a.s_t;    // + absolute token * s_t
  const int64_t step = gridDim.x;
  const bool bf16v = a.vec16 && a.dtype == AATC_BF16, f32v = a.vec16 && a.dtype == AATC_F32;
  // rows of a tile held in registers: bf16 4 x 16 B per thread (row u >> 4, 8 channels),
  // fp32 8 x 16 B (row u >> 5, 4 channels), u = tid + 256 r
  uint4 pf[8];
  auto tile_range = [&](int64_t tile, int& lo, int& hi) {
    const int64_t tok0 = tile * T;
    lo = a.tok_off > tok0 ? static_cast<int>(a.tok_off - tok0) : 0;
    const int64_t end = a.tok_off + a.n_tok - tok0;
    hi = end < T ? static_cast<int>(end) : T;
  };
  auto load_rows = [&](int64_t tile) {
    int lo, hi;
    tile_range(tile, lo, hi);
    const int64_t tok0 = tile * T;
    if (bf16v) {
      const uint16_t* xb = static_cast<const uint16_t*>(a.x);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = tid + THREADS * r, t = u >> 4;
        const int tc = t < lo ? lo : (t >= hi ? hi - 1 : t);         // always a written slot
        pf[r] = *reinterpret_cast<const uint4*>(xb + xrow + (tok0 + tc) * a.s_t + 8 * (u & 15));
      }
    } else if (f32v) {
      const float* xf = static_cast<const float*>(a.x);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int u = tid + THREADS * r, t = u >> 5;
        const int tc = t < lo ? lo : (t >= hi ? hi - 1 : t);
        pf[r] = *reinterpret_cast<const uint4*>(xf + xrow + (tok0 + tc) * a.s_t + 4 * (u & 31));
      }
    }
  };

  int64_t tile = a.tile0 + blockIdx.x;
  if (tile < a.tile_end) load_rows(tile);
  for (; tile < a.tile_end; tile += step) {
    int lo, hi;
    tile_range(tile, lo, hi);
    const int64_t tok0 = tile * T;
    lds_barrier();                                       // the previous tile is done with LDS
    // ---- 1. x rows into LDS (slots outside [lo, hi) read as 0)
    if (bf16v) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = tid + THREADS * r, t = u >> 4;
        const bool in = t >= lo && t < hi;
        const uint32_t w[4] = {pf[r].x, pf[r].y, pf[r].z, pf[r].w};
        float4* dst = reinterpret_cast<float4*>(xs + t * D + 8 * (u & 15));
        dst[0] = in ? make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                  __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u))
                    : make_float4(0.f, 0.f, 0.f, 0.f);
        dst[1] = in ? make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                  __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u))
                    : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else if (f32v) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int u = tid + THREADS * r, t = u >> 5;
        const bool in = t >= lo && t < hi;
        reinterpret_cast<uint4*>(xs + t * D)[u & 31] = in ? pf[r] : make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      for (int e = tid; e < T * D; e += THREADS) {
        const int t = e / D, j = e % D;
        xs[e] = (t >= lo && t < hi) ? static_cast<float>(load_x(a.x, a.dtype, xrow + (tok0 + t) * a.s_t + j)) : 0.f;
      }
    }
    if (tile + step < a.tile_end) load_rows(tile + step);   // next tile's rows, in flight from here
    lds_barrier();

    // ---- 2 + 3. rotate and quantize; codes packed four to a register
    uint32_t cp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cp[k] = 0u;
    const int q4 = tid & 3, tb = tid >> 4, cb = tid & 15;
    if constexpr (wht) {
      const int tq = tid >> 2, i0 = 32 * q4;
      double v[32];
#pragma unroll
      for (int k4 = 0; k4 < 8; ++k4) {
        const float4 f = reinterpret_cast<const float4*>(xs + tq * D + i0)[k4];
        v[4 * k4] = f.x;
        v[4 * k4 + 1] = f.y;
        v[4 * k4 + 2] = f.z;
        v[4 * k4 + 3] = f.w;
      }
      // Sylvester order: y_i = sum_j (-1)^popcount(i & j) x_j; butterflies on index bits 0..4 in
      // the thread, then bits 5 and 6 (lanes ^1 and ^2 hold the other channel quarters)
#pragma unroll
      for (int m = 1; m < 32; m <<= 1)
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if (!(k & m)) {
            const double x0 = v[k], x1 = v[k + m];
            v[k] = x0 + x1;
            v[k + m] = x0 - x1;
          }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const double pv = quad_xor<0xB1>(v[k]);      // lane ^ 1
        v[k] = (q4 & 1) ? pv - v[k] : v[k] + pv;
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const double pv = quad_xor<0x4E>(v[k]);      // lane ^ 2
        v[k] = (q4 & 2) ? pv - v[k] : v[k] + pv;
      }
#pragma unroll
      for (int k = 0; k < 32; ++k)
        cp[k >> 2] |= static_cast<uint32_t>(lm ? quantize_lm(v[k] * rs, t_o[i0 + k], t_inv[i0 + k], t_bits[i0 + k], t_th)
                                                : quantize(v[k] * rs, t_o[i0 + k], t_inv[i0 + k], t_bits[i0 + k]))
                      << (8 * (k & 3));
    } else {
      double acc[4][8];
      tile_gemm_e(xs, c->E, mchunk, acc);
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int i = 8 * cb + bb;
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          const int n = 8 * aa + bb;
          cp[n >> 2] |= static_cast<uint32_t>(lm ? quantize_lm(acc[aa][bb], t_o[i], t_inv[i], t_bits[i], t_th)
                                                  : quantize(acc[aa][bb], t_o[i], t_inv[i], t_bits[i]))
                        << (8 * (n & 3));
        }
      }
    }
    lds_barrier();                                       // x and the staging area are free
    // codes over the x tile: K token-major [64][128], V channel-major [128][64]; slots outside
    // [lo, hi) hold 0
    uint8_t* cs = reinterpret_cast<uint8_t*>(xs);
    if (wht) {
      const int t = tid >> 2;
      const bool in = t >= lo && t < hi;
      if (a.which == 0) {
        uint4* dst = reinterpret_cast<uint4*>(cs + t * D + 32 * q4);
        dst[0] = in ? make_uint4(cp[0], cp[1], cp[2], cp[3]) : make_uint4(0u, 0u, 0u, 0u);
        dst[1] = in ? make_uint4(cp[4], cp[5], cp[6], cp[7]) : make_uint4(0u, 0u, 0u, 0u);
      } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) cs[(32 * q4 + k) * T + t] = in ? static_cast<uint8_t>(cp[k >> 2] >> (8 * (k & 3))) : 0;
      }
    } else {
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int t = 4 * tb + aa;
        if (t < lo || t >= hi) {
          cp[2 * aa] = 0u;
          cp[2 * aa + 1] = 0u;
        }
      }
      if (a.which == 0) {
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
          *reinterpret_cast<uint2*>(cs + (4 * tb + aa) * D + 8 * cb) = make_uint2(cp[2 * aa], cp[2 * aa + 1]);
      } else {
        // channel 8 cb + bb, tokens 4 tb .. 4 tb + 3: one dword
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          uint32_t w4 = 0;
#pragma unroll
          for (int aa = 0; aa < 4; ++aa) w4 |= ((cp[2 * aa + (bb >> 2)] >> (8 * (bb & 3))) & 0xffu) << (8 * aa);
          *reinterpret_cast<uint32_t*>(cs + (8 * cb + bb) * T + 4 * tb) = w4;
        }
      }
    }
    if (a.which == 0)
      for (int w = tid; w < 2 * B; w += THREADS) S[w] = 0u;
    lds_barrier();

    // ---- 4. K: OR each (token, quarter of the channels) run into the words; planes are
    // ordered by channel, so a quarter's planes are one contiguous run of the token's bits
    if (a.which == 0) {
      const int t = tid >> 2, i0 = 32 * q4;
      if (t >= lo && t < hi) {
        const uint4* cr = reinterpret_cast<const uint4*>(cs + t * D + i0);
        const uint4* br = reinterpret_cast<const uint4*>(t_bits + i0);
        const uint4 c0 = cr[0], c1 = cr[1], b0 = br[0], b1 = br[1];
        const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        int pos = t * B + t_pb[i0];
        uint64_t acc = 0;
        int nb = 0;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          acc |= static_cast<uint64_t>((cw[k >> 2] >> (8 * (k & 3))) & 0xffu) << nb;
          nb += (bw[k >> 2] >> (8 * (k & 3))) & 0xffu;
          if (nb >= 32) {
            or_bits(S, pos, static_cast<uint32_t>(acc));
            pos += 32;
            acc >>= 32;
            nb -= 32;
          }
        }
        if (nb > 0) or_bits(S, pos, static_cast<uint32_t>(acc));
      }
      lds_barrier();
    }

    // ---- 5. one writer per word (V: gathered from the field's channel column); bits of tokens
    // before lo keep their old value
    uint32_t* out = a.codes + ((static_cast<int64_t>(b) * a.n_kv_heads + h) * a.tiles_per_seq + tile) * (2 * B);
    for (int w = tid; w < 2 * B; w += THREADS) {
      uint32_t word;
      int f = 0, wd = 0, j = 0;
      if (a.which == 0) {
        word = S[w];
      } else {
        f = t_wf[w];
        const int ws = t_fs[f], sh = ws >> 4;
        wd = ws & 15;
        j = w - t_fw[f];
        const uint8_t* col = cs + t_fc[f] * T;
        word = 0;
        if (wd == 4) {
          // tokens 16 G + 4 r + m, r = 2 (j & 1) + (n >> 2), m = n & 3: bits 8 m + 4 (r & 1)
          const uint2 u = *reinterpret_cast<const uint2*>(col + 8 * j);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const uint32_t code = ((n < 4 ? u.x : u.y) >> (8 * (n & 3))) & 0xffu;
            word |= ((code >> sh) & 15u) << (8 * (n & 3) + 4 * (n >> 2));
          }
        } else if (wd == 2) {
          // tokens 16 j + n: bits (8 m + 2 r + b + j % 2) mod 32
          const uint4 u = *reinterpret_cast<const uint4*>(col + 16 * j);
          const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int n = 0; n < 16; ++n) {
            const uint32_t v = ((uw[n >> 2] >> (8 * (n & 3))) >> sh) & 3u;
            const int base = (8 * (n & 3) + 2 * (n >> 2) + (j & 1)) & 31;
            word |= ((v & 1u) << base) | ((v >> 1) << ((base + 1) & 31));
          }
        } else {
          // tokens 32 j + n: bit 8 m + 2 r + n / 16
          const uint4* u2 = reinterpret_cast<const uint4*>(col + 32 * j);
          const uint4 ua = u2[0], ub = u2[1];
          const uint32_t uw[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            const uint32_t v = ((uw[n >> 2] >> (8 * (n & 3))) >> sh) & 1u;
            word |= v << (8 * (n & 3) + 2 * ((n >> 2) & 3) + (n >> 4));
          }
        }
      }
      if (lo > 0) {
        uint32_t keep = 0;
        if (a.which == 0) {
          const int64_t kb = static_cast<int64_t>(lo) * B - 32 * w;     // kept bits in this word
          keep = kb >= 32 ? 0xffffffffu : (kb <= 0 ? 0u : ((1u << kb) - 1u));
        } else {
          for (int q = 0; q < 32; ++q) {
            int bit;
            if (v_token(j, q, wd, &bit) < lo) keep |= 1u << q;
          }
        }
        if (keep) word |= out[w] & keep;
      }
      out[w] = word;
    }
  }
}

// Two waves per SIMD (two workgroups per CU): the fast transform keeps 32 fp64 values per thread.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_encode(CodecArgs a) {
  const aatc_calib* c = a.calib + blockIdx.y;
  if (c->magic != AATC_MAGIC) return;
  if (c->rotation == AATC_ROT_WHT)
    encode_tiles<true>(a);
  else
    encode_tiles<false>(a);
}

// ---------------------------------------------------------------------------------------
// Decode (reconstruct): one workgroup per (tile, head, batch).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(THREADS) void k_decode(CodecArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* ys = reinterpret_cast<double*>(smem);                             // 64*128 f64
  double* mchunk = reinterpret_cast<double*>(smem + T * D * 8);             // KC*128 f64
  int* pbase = reinterpret_cast<int*>(smem + T * D * 8 + KC * D * 8);       // 128
  const int tid = threadIdx.x;
  const int64_t tile = a.tile0 + blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const aatc_calib* c = a.calib + h;
  const int B = c->total_bits;
  if (c->magic != AATC_MAGIC) return;
  const int64_t tok0 = tile * T;
  const uint32_t* in = a.codes + ((static_cast<int64_t>(b) * a.n_kv_heads + h) * a.tiles_per_seq + tile) * (2 * B);
  if (tid == 0) {
    int s = 0;
    for (int i = 0; i < D; ++i) { pbase[i] = s; s += c->bits[i]; }
  }
  __syncthreads();
  for (int e = tid; e < T * D; e += THREADS) {
    const int t = e / D, i = e % D;
    const int bi = c->bits[i];
    double y = c->o[i];
    if (bi) {
      int code = 0;
      if (a.which == 0) {
        const int s = t * B + pbase[i];
        const int wi = s >> 5, sh = s & 31;
        uint64_t two = in[wi];
        if (wi + 1 < 2 * B) two |= static_cast<uint64_t>(in[wi + 1]) << 32;
        code = static_cast<int>((two >> sh) & ((1u << bi) - 1u));
      } else {
        for (int k = 0; k < 3; ++k) {
          const int f = c->channel_field[3 * i + k];
          if (f < 0) break;
          const int wd = c->field_width[f];
          int v = 0;
          for (int bb = 0; bb < wd; ++bb) {
            const int pos = 32 * c->field_word[f] + v_bit(t, wd, bb);
            v |= static_cast<int>((in[pos >> 5] >> (pos & 31)) & 1u) << bb;
          }
          code |= v << c->field_shift[f];
        }
      }
      // o + scale * level: the uniform quantizer's level is c - 2^(b-1) + 1/2, Lloyd-Max's the table's
      y = c->o[i] + c->scale[i] * c->level[(1 << bi) - 2 + code];
    }
    ys[e] = y;
  }
  double acc[4][8];
  tile_gemm<false>(ys, c->R, mchunk, acc);
  const int tb = tid >> 4, cb = tid & 15;
  for (int aa = 0; aa < 4; ++aa) {
    const int64_t at = tok0 + tb * 4 + aa;
    if (at < a.tok_off || at >= a.tok_off + a.n_tok) continue;
    const int64_t base = b * a.s_b + h * a.s_h + (at - a.tok_off) * a.s_t + cb * 8;
    for (int bb = 0; bb < 8; ++bb) store_out(const_cast<void*>(a.x), a.dtype, base + bb, acc[aa][bb]);
  }
}

aatc_status check_cache(const aatc_cache* c, int which) {
  if (!c) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null cache");
  if (c->d != AATC_D) return aatc::fail(AATC_ERR_UNSUPPORTED, "d=%d (only 128)", c->d);
  if (which != 0 && which != 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "which=%d", which);
  if (c->batch < 1 || c->n_kv_heads < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "batch/heads");
  if (c->capacity_tokens < 0 || c->capacity_tokens % AATC_TILE)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "capacity_tokens must be a multiple of 64");
  const int bits = which ? c->v_bits : c->k_bits;
  if (bits < 0 || bits > 8 * AATC_D) return aatc::fail(AATC_ERR_BUDGET, "bits=%d", bits);
  const void* cal = which ? c->v_calib : c->k_calib;
  const void* codes = which ? c->v_codes : c->k_codes;
  if (!cal || (!codes && bits > 0)) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null calib/codes");
  if ((reinterpret_cast<uintptr_t>(cal) & 15) || (reinterpret_cast<uintptr_t>(codes) & 15))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "calib/codes must be 16-byte aligned");
  return AATC_OK;
}

aatc_status launch_codec(bool encode, const aatc_cache* c, int which, const void* x, aatc_dtype dt,
                         const int64_t* strides, int64_t off, int64_t n, void* stream) {
  aatc::clear_error();
  aatc_status s = check_cache(c, which);
  if (s != AATC_OK) return s;
  if (!x || !strides) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null x/strides");
  if (dt != AATC_F32 && dt != AATC_BF16) return aatc::fail(AATC_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (off < 0 || n < 0 || off + n > c->capacity_tokens)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "token range [%lld, %lld) outside capacity %lld",
                      (long long)off, (long long)(off + n), (long long)c->capacity_tokens);
  if (n == 0) return AATC_OK;
  if (encode && (which ? c->v_bits : c->k_bits) == 0) return AATC_OK;   // 0 bits: no words to write
  CodecArgs a;
  a.calib = static_cast<const aatc_calib*>(which ? c->v_calib : c->k_calib);
  a.codes = static_cast<uint32_t*>(which ? c->v_codes : c->k_codes);
  a.tiles_per_seq = c->capacity_tokens / AATC_TILE;
  a.n_kv_heads = c->n_kv_heads;
  a.which = which;
  a.tok_off = off;
  a.n_tok = n;
  a.tile0 = off / AATC_TILE;
  a.x = x;
  a.dtype = dt;
  a.s_b = strides[0];
  a.s_h = strides[1];
  a.s_t = strides[2];
  {
    const int64_t el = dt == AATC_F32 ? 4 : 2, per16 = 16 / el;
    a.vec16 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && strides[0] % per16 == 0 && strides[1] % per16 == 0 &&
              strides[2] % per16 == 0;
  }
  const int64_t tile_end = (off + n + AATC_TILE - 1) / AATC_TILE;
  a.tile_end = tile_end;
  // encode: two workgroups per CU in all, each walking tiles of one (batch, head)
  int64_t gx = tile_end - a.tile0;
  if (encode) {
    const int64_t per = (512 + static_cast<int64_t>(c->n_kv_heads) * c->batch - 1) /
                        (static_cast<int64_t>(c->n_kv_heads) * c->batch);
    if (gx > per) gx = per;
  }
  dim3 grid(static_cast<unsigned>(gx), c->n_kv_heads, c->batch);
  auto st = static_cast<hipStream_t>(stream);
  const size_t lds = encode ? kEncodeLds : kDecodeLds;
  const void* fn = encode ? reinterpret_cast<const void*>(&k_encode) : reinterpret_cast<const void*>(&k_decode);
  const hipError_t ea = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (ea != hipSuccess) return aatc::fail(AATC_ERR_HIP, "LDS attribute: %s", hipGetErrorString(ea));
  if (encode) {
    hipLaunchKernelGGL(k_encode, grid, dim3(THREADS), lds, st, a);
  } else {
    hipLaunchKernelGGL(k_decode, grid, dim3(THREADS), lds, st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "%s launch: %s", encode ? "encode" : "decode",
                                         hipGetErrorString(e));
  return AATC_OK;
}

}  // namespace

extern "C" {

aatc_status aatc_encode(const aatc_cache* cache, int32_t which, const void* x_dev, aatc_dtype dtype,
                        const int64_t strides[3], int64_t token_offset, int64_t n_tokens, void* stream) {
  return launch_codec(true, cache, which, x_dev, dtype, strides, token_offset, n_tokens, stream);
}

aatc_status aatc_decode(const aatc_cache* cache, int32_t which, int64_t token_offset, int64_t n_tokens,
                        void* out_dev, aatc_dtype out_dtype, const int64_t strides[3], void* stream) {
  return launch_codec(false, cache, which, out_dev, out_dtype, strides, token_offset, n_tokens, stream);
}

}  // extern "C"
