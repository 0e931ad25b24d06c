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
constexpr size_t kEncodeLds = T * D * 4 + KC * D * 8 + T * D;   // x (f32), R chunk, codes
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
  int64_t s_b, s_h, s_t;
};

// ---------------------------------------------------------------------------------------
// Encode: one workgroup per (tile, head, batch).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(THREADS) void k_encode(CodecArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);                               // 64*128 f32
  double* mchunk = reinterpret_cast<double*>(smem + T * D * 4);             // KC*128 f64
  uint8_t* cs = smem + T * D * 4 + KC * D * 8;                              // 64*128 u8
  const int tid = threadIdx.x;
  const int64_t tile = a.tile0 + blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const aatc_calib* c = a.calib + h;
  const int B = c->total_bits;
  if (c->magic != AATC_MAGIC) return;
  const int64_t tok0 = tile * T;                       // absolute token of tile slot 0
  // stage x (tokens outside the written range read as 0)
  for (int e = tid; e < T * D; e += THREADS) {
    const int t = e / D, j = e % D;
    const int64_t at = tok0 + t;
    float v = 0.f;
    if (at >= a.tok_off && at < a.tok_off + a.n_tok)
      v = static_cast<float>(load_x(a.x, a.dtype, b * a.s_b + h * a.s_h + (at - a.tok_off) * a.s_t + j));
    xs[e] = v;
  }
  double acc[4][8];
  tile_gemm<true>(xs, c->E, mchunk, acc);       // y = E x
  // quantize: u = (y - o) * inv + 2^(b-1); c = clamp(floor(u), 0, 2^b - 1); NaN -> 0
  const int tb = tid >> 4, cb = tid & 15;
  for (int bb = 0; bb < 8; ++bb) {
    const int i = cb * 8 + bb;
    const int bi = c->bits[i];
    const double o = c->o[i], inv = c->inv_delta[i];
    const double half = bi ? ldexp(1.0, bi - 1) : 0.0;
    const double top = bi ? ldexp(1.0, bi) - 1.0 : 0.0;
    for (int aa = 0; aa < 4; ++aa) {
      int code = 0;
      if (bi) {
        double u = (acc[aa][bb] - o) * inv;
        u = u + half;
        double f = floor(u);
        if (f != f) f = 0.0;
        f = f < 0.0 ? 0.0 : (f > top ? top : f);
        code = static_cast<int>(f);
      }
      cs[(tb * 4 + aa) * D + i] = static_cast<uint8_t>(code);
    }
  }
  __syncthreads();
  uint32_t* out = a.codes + ((static_cast<int64_t>(b) * a.n_kv_heads + h) * a.tiles_per_seq + tile) * (2 * B);
  const bool keep_old = tok0 < a.tok_off;
  if (a.which == 0) {
    for (int w = tid; w < 2 * B; w += THREADS) {
      int t = (32 * w) / B, p = 32 * w - t * B;
      uint32_t word = 0, mask_new = 0, mask_keep = 0;
      for (int q = 0; q < 32; ++q) {
        const int64_t at = tok0 + t;
        if (at >= a.tok_off && at < a.tok_off + a.n_tok) {
          mask_new |= 1u << q;
          word |= static_cast<uint32_t>((cs[t * D + c->plane_channel[p]] >> c->plane_bit[p]) & 1) << q;
        } else if (at < a.tok_off) {
          mask_keep |= 1u << q;
        }
        if (++p == B) { p = 0; ++t; }
      }
      if (keep_old && mask_keep) word |= out[w] & mask_keep;
      out[w] = word;
    }
  } else {
    const int nf = c->n_fields;
    for (int w = tid; w < 2 * B; w += THREADS) {
      int lo = 0, hi = nf - 1;           // last field whose first word <= w
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (c->field_word[mid] <= w) lo = mid; else hi = mid - 1;
      }
      const int f = lo;
      const int wd = c->field_width[f], ch = c->field_channel[f], sh = c->field_shift[f];
      const int j = w - c->field_word[f];
      uint32_t word = 0, mask_keep = 0;
      for (int q = 0; q < 32; ++q) {
        int bit;
        const int t = v_token(j, q, wd, &bit);
        const int64_t at = tok0 + t;
        if (at >= a.tok_off && at < a.tok_off + a.n_tok) {
          word |= static_cast<uint32_t>((cs[t * D + ch] >> (sh + bit)) & 1) << q;
        } else if (at < a.tok_off) {
          mask_keep |= 1u << q;
        }
      }
      if (keep_old && mask_keep) word |= out[w] & mask_keep;
      out[w] = word;
    }
  }
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
      const double half = ldexp(1.0, bi - 1);
      y = c->o[i] + c->delta[i] * ((static_cast<double>(code) - half) + 0.5);
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
  const int64_t tile_end = (off + n + AATC_TILE - 1) / AATC_TILE;
  dim3 grid(static_cast<unsigned>(tile_end - a.tile0), c->n_kv_heads, c->batch);
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
