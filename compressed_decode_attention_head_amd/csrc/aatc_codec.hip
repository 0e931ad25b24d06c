// Encode (rotate -> quantize -> pack) and decode (unpack -> dequantize -> rotate back)
// kernels for gfx950, plus their C-ABI launchers.
//
// Page "KV Cache Compression Through the Lens of Transform Coding" (Full text): transform
// coding of the cache; page "SPECTRA ..." (Abstract): the cache is re-encoded in the rotated
// coordinate system; page "Ablation, Statistical Inference, and Validation for KV-Cache
// Compression" (first abstract): a scalar MSE quantizer after the rotation.
//
// Every packed word has exactly one writer: in the encoder one wave per 32-token half tile,
// in the decoder one workgroup per 64-token tile.  Rotation and quantization run in fp64 so
// that codes agree with an fp64 definition except for values within rounding distance of a
// bin edge.
// This file is compiled with -ffp-contract=off: the quantizer expression must be the
// separately rounded fp64 sequence of the format definition; the GEMM uses explicit fma().
#include <hip/hip_runtime.h>

#include <type_traits>

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
// Encode.  Grid (G, KV heads, batch) of 4-wave workgroups (K and V in one launch: batch
// doubled, K's workgroups first).  A workgroup loads its head's
// quantizer and packing tables into LDS once (its only barriers); after that every wave works
// alone on half tiles: 32 consecutive tokens of one sequence, whose packed words no other half
// tile touches (K: the 32 B bits of the half tile are B whole words; V: w words of every w-bit
// field).  Per half tile:
//  1. rows straight from memory into registers (16-byte aligned bf16 rows of a Walsh-Hadamard
//     blob: the next half tile's rows are in flight while this one computes);
//  2. y = E x in fp64:
//     - Walsh-Hadamard: lane = (token, quarter of the channels, on channel bits 3 and 4); five
//       butterfly stages in registers over the other channel bits and two across the quad (DPP
//       moves), all exact on bf16 rows, then one multiply by the blob's 1/sqrt(d) (its R[0]);
//     - other rotations: v_mfma_f64_16x16x4f64 with E as the A operand (16 output channels x 4
//       input channels) and the rows as B (4 input channels x 16 tokens), two token blocks x 8
//       channel blocks of accumulators per wave.  The contraction runs over the input channels
//       in the order 32 g + s (g = the lane's k slot, s = the step), so each lane reads one
//       contiguous 32-channel chunk of its rows and one of each E row it needs; E streams
//       through a ring of LDS chunks shared by the four waves;
//     - launches of at most 8 tokens per sequence (decode-step appends): the same product on
//       the vector ALU, E rows in registers, all of the workgroup's tokens at once;
//  3. the quantizer in fp64, separately rounded (this file is built without contraction);
//  4. packing in the wave's own LDS area: K runs of consecutive channels OR-ed into the half
//     tile's token-major bit string, V codes stored channel-major and gathered per word;
//  5. the words to memory, keeping the bits of tokens before the first one written.
// ---------------------------------------------------------------------------------------
constexpr int HT = 32;                                      // tokens of a half tile
constexpr int WAVES = THREADS / 64;
constexpr size_t kQ = 0;                                    // fp64 {o, 1/scale}, then 2^(b-1), per channel (padded rows)
constexpr size_t kTBits = kQ + 32 * D;                      // u8 bits[128]
constexpr size_t kTPb = kTBits + D;                         // u16 first plane of each channel
constexpr size_t kTFw = kTPb + 2 * D;                       // u16 first word of each field
constexpr size_t kTFs = kTFw + 2 * AATC_MAX_FIELDS;         // u8 width | shift << 4 of each field
constexpr size_t kTFc = kTFs + AATC_MAX_FIELDS;             // u8 channel of each field
constexpr size_t kTHf = kTFc + AATC_MAX_FIELDS;             // u16 field of each word of a half tile
constexpr size_t kTTh = kTHf + 2 * AATC_D * AATC_MAX_BITS;  // fp64 Lloyd-Max thresholds
constexpr size_t kWave = kTTh + 8 * AATC_LEVELS;            // per wave: a half tile's K words or V codes
constexpr int XS = D + 8;                                   // bf16 row stride of the GEMM's staged rows
constexpr size_t kWaveBytes = HT * XS * 2;                  // 32 bf16 rows; >= 32 x 128 code bytes, B <= 1024 words
constexpr int NECH = 4;                                     // GEMM: 8 KB chunks of E in LDS ...
constexpr int ECH_AHEAD = NECH - 1;                         // ... copied this many steps ahead
constexpr int SMALL_N = 8;                                  // GEMM form: launches of at most this many
                                                            // tokens per sequence transform on the VALU
constexpr size_t kEch = kWave + WAVES * kWaveBytes;
constexpr size_t kEncodeLds = kEch + NECH * 2 * AATC_D * 4 * 8;
// two workgroups per CU
static_assert(2 * kEncodeLds <= 160 * 1024, "two encode workgroups fit one CU's LDS");
static_assert(2 * SMALL_N * AATC_D * 8 <= NECH * 2 * AATC_D * 4 * 8, "small-launch products and inputs fit the E ring");
static_assert(kTTh % 16 == 0 && kWave % 16 == 0 && kEch % 16 == 0, "LDS tables aligned");
static_assert(AATC_D * AATC_MAX_BITS * 4 <= kWaveBytes, "a half tile's K words (B <= 1024) fit the wave area");
static_assert(AATC_D * HT + AATC_D * AATC_MAX_BITS * 4 <= kWaveBytes, "V codes and the kept V words fit the wave area");

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
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u & 0xffffffffu), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                                     static_cast<unsigned>(lo)));
}

// LDS OR without a return value, not ordered by the compiler against global loads in flight.
__device__ inline void lds_or(uint32_t* p, uint32_t v) {
  asm volatile("ds_or_b32 %0, %1" : : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p))), "v"(v) : "memory");
}

typedef double f64x4 __attribute__((ext_vector_type(4)));
// global-memory views of the encoder's pointers (a pointer reached through the argument struct
// is otherwise a flat pointer)
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef __attribute__((address_space(1))) float gf32;
typedef __attribute__((address_space(1))) double gf64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu4;

__device__ inline double bf16_lo(uint32_t w) { return static_cast<double>(__uint_as_float(w << 16)); }
__device__ inline double bf16_hi(uint32_t w) { return static_cast<double>(__uint_as_float(w & 0xffff0000u)); }

// v_cvt_i32_f64: truncation toward zero, NaN -> 0, values beyond the int32 range clamped to it
// (the instruction's own definition, which a C++ conversion does not promise).
__device__ inline int cvt_i32_trunc(double u) {
  int r;
  asm("v_cvt_i32_f64_e32 %0, %1" : "=v"(r) : "v"(u));
  return r;
}

// Quantizer table of a channel: {o, 1/scale} and 2^(b-1).  In the Walsh-Hadamard form it sits
// at a padded position: the four lanes of a token read channels 8 apart, which the padding puts
// in disjoint LDS banks (each 32 channels take 40 rows, each 8 of them 10).  The GEMM form's
// lanes read four channels 4 apart, already in disjoint banks, at the plain position.
constexpr int kQRows = 40 * (D / 32);
static_assert(24 * kQRows <= 32 * D, "padded quantizer table fits its LDS area");
template <bool PAD>
__device__ inline int qpos(int i) {
  return PAD ? 40 * (i >> 5) + 10 * ((i >> 3) & 3) + (i & 7) : i;
}

// Code of value y of a channel with table entries o, inv = 1/scale, half = 2^(b-1).  Uniform:
// clamp(floor((y - o) * (1/Delta) + 2^(b-1)), 0, 2^b - 1) with NaN -> 0.  Truncation toward zero
// equals the floor on [0, 2^b - 1], and every value outside (NaN included) lands on the clamp's
// side it belongs to, so the clamp runs on the truncated integer.
// Lloyd-Max: the b-bit table's threshold count (quantize_lm).
template <bool LM>
__device__ inline int code_with(double y, double2 oi, double half, int bi, const double* thr) {
  if (LM) return quantize_lm(y, oi.x, oi.y, bi, thr);
  double u = (y - oi.x) * oi.y;
  u = u + half;
  const int top = (1 << bi) - 1;
  const int ci = cvt_i32_trunc(u);
  return ci < 0 ? 0 : (ci > top ? top : ci);
}
template <bool PAD, bool LM>
__device__ inline int code_of(double y, const double2* qoi, const double* qh, int i, int bi, const double* thr) {
  const int p = qpos<PAD>(i);
  return code_with<LM>(y, qoi[p], qh[p], bi, thr);
}

// OR the run v (at most 64 bits, higher bits zero) into the bit string S at bit position pos;
// words the run does not reach are not touched.
__device__ inline void or_run(uint32_t* S, int pos, uint64_t v) {
  if (!v) return;
  const int w = pos >> 5, sh = pos & 31;
  const uint64_t lo = v << sh;
  const uint32_t top = sh ? static_cast<uint32_t>(v >> (64 - sh)) : 0u;
  if (static_cast<uint32_t>(lo)) lds_or(S + w, static_cast<uint32_t>(lo));
  if (static_cast<uint32_t>(lo >> 32)) lds_or(S + w + 1, static_cast<uint32_t>(lo >> 32));
  if (top) lds_or(S + w + 2, top);
}


// Element i of the encoder's input (fp32 or bf16) through a global-memory pointer, so that the
// load is not a flat access (which the LDS waits would also count).
__device__ inline double gload_x(const void* x, int dt, int64_t i) {
  if (dt == AATC_F32) return static_cast<double>(((const gf32*)(x))[i]);
  const uint32_t u = static_cast<uint32_t>(((const gu16*)(x))[i]) << 16;
  return static_cast<double>(__uint_as_float(u));
}

// A half tile's K words (the B words of its 32 tokens' bit string, built in S) to memory; bits
// of tokens before lo keep their value.
__device__ inline void write_k_words(const uint32_t* S, gu32* out, int B, int lo, int lane) {
  for (int u = lane; u < B; u += 64) {
    uint32_t word = S[u];
    if (lo > 0) {
      const int kb = lo * B - 32 * u;                            // kept bits in this word
      const uint32_t keep = kb >= 32 ? 0xffffffffu : (kb <= 0 ? 0u : ((1u << kb) - 1u));
      if (keep) word |= out[u] & keep;
    }
    out[u] = word;
  }
}

// A half tile's V words from its codes cs[channel][32 tokens]: word jj of field f is word
// fw + half w + jj of the tile, holding the tokens the tile layout (include/aatc.h) gives it,
// less 32 half; bits of tokens before lo keep their value.  The words that hold such tokens are
// all read first (one memory round trip, parked in the wave's free LDS at oldw), so a partial
// half tile costs one round trip, not one per word.
__device__ __attribute__((noinline)) void write_v_words(const uint8_t* cs, gu32* out, int B, int half, int lo, int lane,
                                     const uint16_t* t_hf, const uint16_t* t_fw, const uint8_t* t_fs,
                                     const uint8_t* t_fc, uint32_t* oldw) {
  auto word_of = [&](int u) {        // tile word of half-tile word u
    const int f = t_hf[u];
    const int fw = t_fw[f], wd = t_fs[f] & 15;
    return fw + half * wd + (u - fw / 2);
  };
  if (lo > 0) {
    constexpr int PER = AATC_D * AATC_MAX_BITS / 64;    // words per lane, at most
    uint32_t old[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int u = lane + 64 * k;
      old[k] = out[word_of(u < B ? u : 0)];   // clamped, unconditional: the loads fly together
    }
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (lane + 64 * k < B) oldw[lane + 64 * k] = old[k];
  }
  // Each of a column's 4-byte groups q (tokens 4 q .. 4 q + 3, one code byte each) lands in the
  // word by one shift and mask: a w-bit field's code bits of token 4 q + m sit at bit 8 m + (a
  // position set by q, jj and w) of its word.  The kept bits are the same positions of the
  // tokens before lo, taken from bytes that are all ones for those tokens (ow).
  auto ow = [&](int q) {
    const int cnt = lo - 4 * q;
    return cnt >= 4 ? 0xffffffffu : (cnt <= 0 ? 0u : (1u << (8 * cnt)) - 1u);
  };
  auto rotl = [](uint32_t x, int k) { return k ? (x << k) | (x >> (32 - k)) : x; };
  for (int u = lane; u < B; u += 64) {
    const int f = t_hf[u];
    const int fw = t_fw[f], ws = t_fs[f], sh = ws >> 4, wd = ws & 15;
    const int jj = u - fw / 2;
    const uint32_t* col = reinterpret_cast<const uint32_t*>(cs + t_fc[f] * HT);
    uint32_t word = 0, keep = 0;          // keep: the bits of tokens before lo
    if (wd == 4) {
      // tokens 8 jj .. 8 jj + 7; token 8 jj + 4 rl + m at bits 8 m + 4 rl
      word = ((col[2 * jj] >> sh) & 0x0f0f0f0fu) | (((col[2 * jj + 1] >> sh) & 0x0f0f0f0fu) << 4);
      keep = (ow(2 * jj) & 0x0f0f0f0fu) | ((ow(2 * jj + 1) & 0x0f0f0f0fu) << 4);
    } else if (wd == 2) {
      // tokens 16 jj + 4 r + m: bits (8 m + 2 r + b + jj % 2) mod 32
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        word |= rotl((col[4 * jj + r] >> sh) & 0x03030303u, 2 * r + (jj & 1));
        keep |= rotl(ow(4 * jj + r) & 0x03030303u, 2 * r + (jj & 1));
      }
    } else {
      // tokens 4 q + m = 0..31: bit 8 m + 2 (q % 4) + q / 4
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        word |= ((col[q] >> sh) & 0x01010101u) << (2 * (q & 3) + (q >> 2));
        keep |= (ow(q) & 0x01010101u) << (2 * (q & 3) + (q >> 2));
      }
    }
    if (lo > 0) word |= oldw[u] & keep;
    out[fw + half * wd + jj] = word;
  }
}

template <bool WHT, bool LM>
__device__ __attribute__((noinline)) void encode_waves(const CodecArgs& a, int b) {
  extern __shared__ __align__(16) unsigned char smem[];
  double2* qoi = reinterpret_cast<double2*>(smem + kQ);
  double* qh = reinterpret_cast<double*>(smem + kQ + 16 * kQRows);
  uint8_t* t_bits = smem + kTBits;
  uint16_t* t_pb = reinterpret_cast<uint16_t*>(smem + kTPb);
  uint16_t* t_fw = reinterpret_cast<uint16_t*>(smem + kTFw);
  uint8_t* t_fs = smem + kTFs;
  uint8_t* t_fc = smem + kTFc;
  uint16_t* t_hf = reinterpret_cast<uint16_t*>(smem + kTHf);
  double* t_th = reinterpret_cast<double*>(smem + kTTh);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const aatc_calib* c = a.calib + h;
  const int B = c->total_bits, nf = c->n_fields;
  constexpr bool lm = LM;
  const bool isv = a.which == 1;

  // ---- tables, once per workgroup
  if (tid < D) {
    const int bi = c->bits[tid];
    qoi[qpos<WHT>(tid)] = make_double2(c->o[tid], lm ? c->inv_scale[tid] : c->inv_delta[tid]);
    qh[qpos<WHT>(tid)] = static_cast<double>(bi ? 1 << (bi - 1) : 0);
    t_bits[tid] = static_cast<uint8_t>(bi);
  }
  if (lm)
    for (int k = tid; k < AATC_LEVELS; k += THREADS) t_th[k] = c->thresh[k];
  if (isv)
    for (int f = tid; f < nf; f += THREADS) {
      const int fw = c->field_word[f], wd = c->field_width[f];
      t_fw[f] = static_cast<uint16_t>(fw);
      t_fs[f] = static_cast<uint8_t>(wd | (c->field_shift[f] << 4));
      t_fc[f] = static_cast<uint8_t>(c->field_channel[f]);
      for (int j = 0; j < wd; ++j) t_hf[fw / 2 + j] = static_cast<uint16_t>(f);   // fields are contiguous
    }
  __syncthreads();
  if (wave == 0) {
    // first plane of each channel: prefix sums of the bit counts, one ballot per bit level
    // (channel lane and 64 + lane)
    const int b0 = t_bits[lane], b1 = t_bits[64 + lane];
    const uint64_t below = (1ull << lane) - 1ull;
    int p0 = 0, p1 = 0, tot0 = 0;
#pragma unroll
    for (int k = 1; k <= AATC_MAX_BITS; ++k) {
      const uint64_t m0 = __ballot(b0 >= k), m1 = __ballot(b1 >= k);
      p0 += __popcll(m0 & below);
      p1 += __popcll(m1 & below);
      tot0 += __popcll(m0);
    }
    t_pb[lane] = static_cast<uint16_t>(p0);
    t_pb[64 + lane] = static_cast<uint16_t>(tot0 + p1);
  }
  __syncthreads();

  unsigned char* warea = smem + kWave + wave * kWaveBytes;
  uint32_t* wb = reinterpret_cast<uint32_t*>(warea);           // K words of the half tile
  uint8_t* cs = warea;                                          // V codes, [channel][32 tokens]
  uint32_t* oldw = reinterpret_cast<uint32_t*>(warea + D * HT);   // V words kept in part, B <= 1024
  uint16_t* xsb = reinterpret_cast<uint16_t*>(warea);           // GEMM bf16 rows, [32][XS]
  const int64_t xrow = b * a.s_b + h * a.s_h - a.tok_off * a.s_t;    // + absolute token * s_t
  const int64_t s_t = a.s_t;
  const void* xp = a.x;
  const int dtype = a.dtype;
  const bool bf16v = a.vec16 && a.dtype == AATC_BF16;
  const int64_t ht_end = 2 * a.tile_end;                               // the last tile is completed
  const int64_t hstep = static_cast<int64_t>(gridDim.x) * WAVES;
  gu32* seq_out = ((gu32*)(a.codes)) + (static_cast<int64_t>(b) * a.n_kv_heads + h) * a.tiles_per_seq * (2 * B);
  const gu16* xb = ((const gu16*)(a.x));
  // tokens [lo, hi) of half tile hti are written (half-local indices; hi <= lo: none)
  auto half_range = [&](int64_t hti, int& lo, int& hi) {
    const int64_t tok0 = hti * HT;
    lo = a.tok_off > tok0 ? static_cast<int>(a.tok_off - tok0) : 0;
    const int64_t e = a.tok_off + a.n_tok - tok0;
    hi = e < 0 ? 0 : (e < HT ? static_cast<int>(e) : HT);
  };
  // 16-byte piece of bf16 row t (half-local, clamped into [lo, hi)) at column col
  auto piece = [&](int64_t hti, int lo, int hi, int t, int col) -> u32x4 {
    const int tc = t < lo ? lo : (t >= hi ? hi - 1 : t);
    return *reinterpret_cast<const gu4*>(xb + xrow + (hti * HT + tc) * a.s_t + col);
  };

  int64_t ht = a.tok_off / HT + static_cast<int64_t>(blockIdx.x) * WAVES + wave;
  if constexpr (WHT) {
    // lane (tq, q4) = (lane >> 2, lane & 3); pass p of a half tile covers its tokens 16 p + tq.
    // Slot k of the lane: channel (k & 7) | q4 << 3 | (k >> 3) << 5, read as 16-byte pieces
    // 4 j + q4 of the row (j = k >> 3), so the four lanes of a token read 64 contiguous bytes.
    const int tq = lane >> 2, q4 = lane & 3;
    auto load_pass = [&](int64_t hti, int p, u32x4 (&dst)[4]) {
      int lo, hi;
      half_range(hti, lo, hi);
      if (hi <= lo) return;
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = piece(hti, lo, hi, 16 * p + tq, 8 * (4 * j + q4));
    };
    u32x4 pf[4];
    if (bf16v && ht < ht_end) load_pass(ht, 0, pf);
    const double rs = c->R[0];
    for (; ht < ht_end; ht += hstep) {
      int lo, hi;
      half_range(ht, lo, hi);
      const int half = static_cast<int>(ht & 1);
      gu32* out = seq_out + (ht >> 1) * (2 * B);
      if (!isv)
        for (int u = lane; u < B; u += 64) wb[u] = 0u;
#pragma unroll 1
      for (int p = 0; p < 2; ++p) {
        const int t = 16 * p + tq;
        const bool in = t >= lo && t < hi;
        double v[32];
        if (bf16v) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w4[4] = {pf[j].x, pf[j].y, pf[j].z, pf[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[8 * j + 2 * e] = bf16_lo(w4[e]);
              v[8 * j + 2 * e + 1] = bf16_hi(w4[e]);
            }
          }
          if (p == 0) load_pass(ht, 1, pf);                     // in flight from here
          else if (ht + hstep < ht_end) load_pass(ht + hstep, 0, pf);
        } else {
#pragma unroll
          for (int k = 0; k < 32; ++k)
            v[k] = in ? gload_x(a.x, a.dtype, xrow + (ht * HT + t) * a.s_t + ((k & 7) | (q4 << 3) | ((k >> 3) << 5))) : 0.0;
        }
        // Sylvester order: y_i = sum_j (-1)^popcount(i & j) x_j, one butterfly per index bit; the
        // stages commute, and on bf16 rows every sum is exact in fp64.  Channel bits 0-2 and 5-6
        // in registers, bits 3 and 4 across the lanes of a quad (y0 = x0 + x1 on the lower lane,
        // y1 = x0 - x1 on the upper one).
#pragma unroll
        for (int m = 1; m < 32; m <<= 1)
#pragma unroll
          for (int k = 0; k < 32; ++k)
            if (!(k & m)) {
              const double x0 = v[k], x1 = v[k + m];
              v[k] = x0 + x1;
              v[k + m] = x0 - x1;
            }
        const double s1 = (q4 & 1) ? -1.0 : 1.0, s2 = (q4 & 2) ? -1.0 : 1.0;
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = fma(s1, v[k], quad_xor<0xB1>(v[k]));
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = fma(s2, v[k], quad_xor<0x4E>(v[k]));
        uint32_t cw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) cw[k] = 0u;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const int i = (k & 7) | (q4 << 3) | ((k >> 3) << 5);
          cw[k >> 2] |= static_cast<uint32_t>(code_of<true, LM>(v[k] * rs, qoi, qh, i, t_bits[i], t_th)) << (8 * (k & 3));
        }
        if (!in) {
#pragma unroll
          for (int k = 0; k < 8; ++k) cw[k] = 0u;
        }
        if (!isv) {
          // four runs of 8 consecutive channels, 8 (4 j + q4) ..
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i0 = 8 * (4 * j + q4);
            uint64_t run = 0;
            int nb = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              run |= static_cast<uint64_t>((cw[2 * j + (e >> 2)] >> (8 * (e & 3))) & 0xffu) << nb;
              nb += t_bits[i0 + e];
            }
            or_run(wb, t * B + t_pb[i0], run);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 32; ++k)
            cs[((k & 7) | (q4 << 3) | ((k >> 3) << 5)) * HT + t] = static_cast<uint8_t>(cw[k >> 2] >> (8 * (k & 3)));
        }
      }
      if (!isv) write_k_words(wb, out + half * B, B, lo, lane);
      else write_v_words(cs, out, B, half, lo, lane, t_hf, t_fw, t_fs, t_fc, oldw);
    }
  } else {
    // GEMM.  The four waves run in step, one half tile each per round, and share E through LDS:
    // chunk sp (step pair sp) is E[., 32 g + 2 sp .. + 1] of every row and g (8 KB).  Chunks go
    // round a ring of NECH buffers, copied ECH_AHEAD steps before they are used, so the copies'
    // L2 latency hides behind the MFMAs of the steps between; each step waits for its own chunk
    // only, then one barrier, then its 32 MFMAs (16 when one token block has no token).
    // Lane (tt, g) = (lane & 15, lane >> 4) feeds rows 16 tb + tt of its half tile, channels
    // 32 g + s; accumulator block (tb, cb), register r: token 16 tb + tt, channel 16 cb + 4 g + r.
    const int tt = lane & 15, g = lane >> 4;
    double2* ech = reinterpret_cast<double2*>(smem + kEch);    // [NECH][128 rows][4 g]
    // chunk piece pc = 256 m + 64 wave + lane: row pc >> 2, g' = pc & 3, copied by global_load_lds
    // (no registers) to ech[buffer][pc]
    const gf64* esrc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int pc = THREADS * m + tid;
      esrc[m] = ((const gf64*)(c->E)) + (pc >> 2) * D + 32 * (pc & 3);
    }
    auto copy_chunk = [&](int sp, int bi) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        __builtin_amdgcn_global_load_lds((const void*)(esrc[m] + 2 * sp),
                                         ech + bi * 512 + THREADS * m + 64 * wave, 16, 0, 0);
    };
    // v_mfma_f64_16x16x4f64 leaves D[i][j] in register i >> 2 of lane 16 (i & 3) + j, so the lane
    // that feeds row i of A feeds E row 16 cb + 4 (i & 3) + (i >> 2): the output of lane (tt, g),
    // register r is then channel 16 cb + 4 g + r, and a lane's four registers are adjacent channels
    const int arow = 4 * (tt & 3) + (tt >> 2);
    // the first ECH_AHEAD chunks; every later step copies the chunk ECH_AHEAD ahead (wrapping to
    // the next round's first ones), so ECH_AHEAD chunks' copies (2 instructions each) are always
    // in flight behind the one a step waits for
    static_assert(ECH_AHEAD == 3, "the step's wait counts 2 * (ECH_AHEAD - 1) copy instructions");
    // A launch of at most SMALL_N tokens per sequence (a decode step's append) takes the
    // transform on the vector ALU instead: one workgroup per (batch, head) holds all of them (at
    // most two half tiles), so its 256 threads share E = 128 rows x 2 halves, each thread one half
    // row in registers (one memory round trip), and the products land in the E ring's LDS.  The
    // MFMA form would stream all of E through 16 barrier steps for a 16-token block per token.
    const bool small = a.n_tok <= SMALL_N;
    double* ysm = reinterpret_cast<double*>(smem + kEch);      // [SMALL_N][128] products
    double* xsm = ysm + SMALL_N * D;                            // [SMALL_N][128] inputs
    if (!small)
#pragma unroll
      for (int k = 0; k < ECH_AHEAD; ++k) copy_chunk(k, k);
    const int64_t first = a.tok_off / HT + static_cast<int64_t>(blockIdx.x) * WAVES;
    for (int64_t base = first; base < ht_end; base += hstep) {
      const int64_t ht = base + wave;
      const bool act = ht < ht_end;
      int lo = 0, hi = 0;
      if (act) half_range(ht, lo, hi);
      // bf16 rows of the half tile into the wave's area, [32][XS] (coalesced: 16-byte piece
      // 64 j + lane is row (64 j + lane) >> 4, column 8 ((64 j + lane) & 15))
      if (!small && act && bf16v && hi > lo) {
        u32x4 pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pc = 64 * j + lane;
          pr[j] = piece(ht, lo, hi, pc >> 4, 8 * (pc & 15));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pc = 64 * j + lane;
          *reinterpret_cast<u32x4*>(xsb + (pc >> 4) * XS + 8 * (pc & 15)) = pr[j];
        }
      }
      if (small) {
        // all of the launch's tokens (one round: they span at most two half tiles), before any
        // accumulator is live
        const int nt = static_cast<int>(a.n_tok);
        for (int e = tid; e < nt * D; e += THREADS)
          xsm[e] = gload_x(xp, dtype, xrow + (a.tok_off + e / D) * s_t + (e % D));
        // wave w holds E rows 32 w .. 32 w + 31, lane l columns l and 64 + l of each (each read is
        // 512 contiguous bytes); a token's 32 row sums are then halved across the lanes five times (each lane
        // keeps the half of the rows its lane bit selects and adds its partner's) and finished
        // with lane l ^ 1: lane l ends with row 32 w + ((l >> 1) & 31)
        double ev[64];
        // the wave's first row in scalar registers, so each read is that base plus a scalar row
        // offset plus the lane's column (no 64-bit address per read)
        const uint64_t e0 = reinterpret_cast<uint64_t>(c->E) + static_cast<uint64_t>(32 * wave) * D * sizeof(double);
        // (readfirstlane returns int: each half goes back through uint32_t, or a low word with
        // bit 31 set would sign-extend over the high word)
        const uint32_t e_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(e0 >> 32)));
        const uint32_t e_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(e0)));
        const gf64* eb = reinterpret_cast<const gf64*>((static_cast<uint64_t>(e_hi) << 32) | e_lo);
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          ev[2 * r] = eb[r * D + lane];
          ev[2 * r + 1] = eb[r * D + 64 + lane];
        }
        __syncthreads();
        for (int k = 0; k < nt; ++k) {
          const double x0 = xsm[k * D + lane], x1 = xsm[k * D + 64 + lane];
          // the first halving takes the products as it goes: rows r and r + 16 of the wave's
          double v[16];
          {
            const bool up = (lane & 32) != 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const double lo_r = fma(ev[2 * r + 1], x1, ev[2 * r] * x0);
              const double hi_r = fma(ev[2 * r + 33], x1, ev[2 * r + 32] * x0);
              v[r] = (up ? hi_r : lo_r) + __shfl_xor(up ? lo_r : hi_r, 32);
            }
          }
          // one halving: the lanes with bit 2N set keep rows [N, 2N) of the current set
          auto halve = [&](auto n_tag) {
            constexpr int N = decltype(n_tag)::value;
            const bool up = (lane & (2 * N)) != 0;
#pragma unroll
            for (int r = 0; r < N; ++r) {
              const double send = up ? v[r] : v[r + N];
              const double keep = up ? v[r + N] : v[r];
              v[r] = keep + __shfl_xor(send, 2 * N);
            }
          };
          halve(std::integral_constant<int, 8>());
          halve(std::integral_constant<int, 4>());
          halve(std::integral_constant<int, 2>());
          halve(std::integral_constant<int, 1>());
          const double y = v[0] + __shfl_xor(v[0], 1);
          if ((lane & 1) == 0) ysm[k * D + 32 * wave + ((lane >> 1) & 31)] = y;
        }
        __syncthreads();
      }
      f64x4 acc[2][8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[tb][cb] = f64x4{0.0, 0.0, 0.0, 0.0};
      // token blocks with a token of the half tile in range (the others' MFMAs are skipped: their
      // accumulators stay zero and no code is taken from them)
      const bool blk0 = act && hi > lo && lo < 16, blk1 = act && hi > 16;
      // one step pair: this wave's copies of chunk sp have landed once at most the 4 copy
      // instructions of chunks sp + 1 and sp + 2 are outstanding (any vector-memory instruction
      // issued since only makes the wait longer); the barrier then publishes everyone's, and its
      // readers of the buffer chunk sp + 3 goes to (chunk sp - 1) have passed it.  The barrier is
      // written out: a workgroup fence would also wait for the chunks still in flight.
      auto step_pair = [&](int sp, auto get_x) {
        const double2* buf = ech + (sp & (NECH - 1)) * 512;
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        copy_chunk((sp + ECH_AHEAD) & 15, (sp + ECH_AHEAD) & (NECH - 1));
        const double* bd = reinterpret_cast<const double*>(buf);
        // the MFMAs of token blocks B0 and B1 (wave-uniform choice, one branch per step)
        auto mfmas = [&](auto b0_tag, auto b1_tag) {
          constexpr bool B0 = decltype(b0_tag)::value, B1 = decltype(b1_tag)::value;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            double x0, x1;
            get_x(2 * sp + u, x0, x1);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
              const double ev = bd[2 * ((16 * cb + arow) * 4 + g) + u];
              if (B0) acc[0][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(ev, x0, acc[0][cb], 0, 0, 0);
              if (B1) acc[1][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(ev, x1, acc[1][cb], 0, 0, 0);
            }
          }
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (blk0 && blk1) mfmas(T_(), T_());
        else if (blk0) mfmas(T_(), F_());
        else if (blk1) mfmas(F_(), T_());
      };
      if (small) {
        // (quantized straight from the products below)
      } else if (bf16v) {
#pragma unroll 1
        for (int sp = 0; sp < 16; ++sp)
          step_pair(sp, [&](int s, double& x0, double& x1) {
            const uint32_t w0 = *reinterpret_cast<const uint32_t*>(xsb + tt * XS + 32 * g + (s & ~1));
            const uint32_t w1 = *reinterpret_cast<const uint32_t*>(xsb + (16 + tt) * XS + 32 * g + (s & ~1));
            x0 = (s & 1) ? bf16_hi(w0) : bf16_lo(w0);
            x1 = (s & 1) ? bf16_hi(w1) : bf16_lo(w1);
          });
      } else {
        const int64_t r0 = xrow + ht * HT * s_t;
        const bool in0 = tt >= lo && tt < hi, in1 = 16 + tt >= lo && 16 + tt < hi;
#pragma unroll 1
        for (int sp = 0; sp < 16; ++sp)
          step_pair(sp, [&](int s, double& x0, double& x1) {
            x0 = in0 ? gload_x(xp, dtype, r0 + tt * s_t + 32 * g + s) : 0.0;
            x1 = in1 ? gload_x(xp, dtype, r0 + (16 + tt) * s_t + 32 * g + s) : 0.0;
          });
      }
      if (!act) continue;
      const int half = static_cast<int>(ht & 1);
      gu32* out = seq_out + (ht >> 1) * (2 * B);
      if (!isv)
        for (int u = lane; u < B; u += 64) wb[u] = 0u;
      if (small) {
        // this wave's tokens of the launch, channels lane and 64 + lane of each: codes straight
        // from the products (V: every other token of the half tile gets code 0, as below)
        if (isv)
          for (int u = lane; u < D * HT / 4; u += 64) reinterpret_cast<uint32_t*>(cs)[u] = 0u;
        for (int t = lo; t < hi; ++t) {
          const int k = static_cast<int>(ht * HT + t - a.tok_off);      // launch-local token
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int i = lane + 64 * hh;
            const double y = ysm[k * D + i];
            const uint32_t cd = static_cast<uint32_t>(code_of<false, LM>(y, qoi, qh, i, t_bits[i], t_th));
            if (!isv) or_run(wb, t * B + t_pb[i], cd);
            else cs[i * HT + t] = static_cast<uint8_t>(cd);
          }
        }
      }
      // per channel block, its four channels' tables once for both token blocks
#pragma unroll
      for (int cb = 0; cb < 8 && !small; ++cb) {
        const int i0 = 16 * cb + 4 * g;
        double2 oi[4];
        double hh[4];
        int bb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          oi[r] = qoi[qpos<false>(i0 + r)];
          hh[r] = qh[qpos<false>(i0 + r)];
          bb[r] = t_bits[i0 + r];
        }
        const int pb = t_pb[i0];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = 16 * tb + tt;
          const bool in = t >= lo && t < hi;
          uint32_t cd[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            cd[r] = in ? static_cast<uint32_t>(code_with<LM>(acc[tb][cb][r], oi[r], hh[r], bb[r], t_th)) : 0u;
          if (!isv) {
            uint64_t run = 0;
            int nb = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              run |= static_cast<uint64_t>(cd[r]) << nb;
              nb += bb[r];
            }
            or_run(wb, t * B + pb, run);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) cs[(i0 + r) * HT + t] = static_cast<uint8_t>(cd[r]);
          }
        }
      }
      if (!isv) write_k_words(wb, out + half * B, B, lo, lane);
      else write_v_words(cs, out, B, half, lo, lane, t_hf, t_fw, t_fs, t_fc, oldw);
    }
    // the last steps' copies of the next round's first chunks: landed before the wave ends (no
    // copy may write the LDS of a workgroup that follows on this CU)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Two waves per SIMD: the GEMM form keeps 16 accumulator blocks (128 registers) per lane.
__device__ inline void encode_tensor(const CodecArgs& a, int b) {
  const aatc_calib* c = a.calib + blockIdx.y;
  if (c->magic != AATC_MAGIC) return;
  const bool lm = c->quantizer == AATC_QUANT_LLOYD_MAX;
  if (c->rotation == AATC_ROT_WHT) {
    if (lm)
      encode_waves<true, true>(a, b);
    else
      encode_waves<true, false>(a, b);
  } else {
    if (lm)
      encode_waves<false, true>(a, b);
    else
      encode_waves<false, false>(a, b);
  }
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_encode(CodecArgs a) {
  encode_tensor(a, blockIdx.z);
}

// K and V of the same token range in one launch: grid z = 2 x batch, K's workgroups first.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_encode_kv(CodecArgs ak,
                                                                                                  CodecArgs av,
                                                                                                  int batch) {
  const int z = blockIdx.z;
  if (z < batch)
    encode_tensor(ak, z);
  else
    encode_tensor(av, z - batch);
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

// Validated arguments and grid width of one tensor's encode or decode; *none when there is
// nothing to do (no tokens, or an encode of a 0-bit tensor).
aatc_status codec_args(bool encode, const aatc_cache* c, int which, const void* x, aatc_dtype dt,
                       const int64_t* strides, int64_t off, int64_t n, CodecArgs* out, int64_t* gx_out, bool* none) {
  *none = false;
  aatc_status s = check_cache(c, which);
  if (s != AATC_OK) return s;
  if (!x || !strides) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null x/strides");
  if (dt != AATC_F32 && dt != AATC_BF16) return aatc::fail(AATC_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (off < 0 || n < 0 || off + n > c->capacity_tokens)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "token range [%lld, %lld) outside capacity %lld",
                      (long long)off, (long long)(off + n), (long long)c->capacity_tokens);
  if (n == 0 || (encode && (which ? c->v_bits : c->k_bits) == 0)) {   // 0 bits: no words to write
    *none = true;
    return AATC_OK;
  }
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
  // encode: two workgroups per CU in all, each walking half tiles of one (batch, head) with its
  // four waves
  int64_t gx = tile_end - a.tile0;
  if (encode) {
    const int64_t halves = 2 * tile_end - off / 32;
    const int64_t per = (512 + static_cast<int64_t>(c->n_kv_heads) * c->batch - 1) /
                        (static_cast<int64_t>(c->n_kv_heads) * c->batch);
    gx = (halves + 3) / 4;
    if (gx > per) gx = per;
  }
  *out = a;
  *gx_out = gx;
  return AATC_OK;
}

aatc_status launch_codec(bool encode, const aatc_cache* c, int which, const void* x, aatc_dtype dt,
                         const int64_t* strides, int64_t off, int64_t n, void* stream) {
  aatc::clear_error();
  CodecArgs a;
  int64_t gx = 0;
  bool none = false;
  const aatc_status s = codec_args(encode, c, which, x, dt, strides, off, n, &a, &gx, &none);
  if (s != AATC_OK || none) return s;
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

aatc_status aatc_encode_kv(const aatc_cache* cache, const void* k_dev, const void* v_dev, aatc_dtype dtype,
                           const int64_t k_strides[3], const int64_t v_strides[3], int64_t token_offset,
                           int64_t n_tokens, void* stream) {
  aatc::clear_error();
  CodecArgs ak, av;
  int64_t gk = 0, gv = 0;
  bool nk = false, nv = false;
  aatc_status s = codec_args(true, cache, 0, k_dev, dtype, k_strides, token_offset, n_tokens, &ak, &gk, &nk);
  if (s != AATC_OK) return s;
  s = codec_args(true, cache, 1, v_dev, dtype, v_strides, token_offset, n_tokens, &av, &gv, &nv);
  if (s != AATC_OK) return s;
  if (nk || nv) {                           // a 0-bit tensor (or no tokens): the other one alone
    if (!nk) return launch_codec(true, cache, 0, k_dev, dtype, k_strides, token_offset, n_tokens, stream);
    if (!nv) return launch_codec(true, cache, 1, v_dev, dtype, v_strides, token_offset, n_tokens, stream);
    return AATC_OK;
  }
  // the grid width depends on the token range and the cache shape only: the same for both
  const dim3 grid(static_cast<unsigned>(gk), cache->n_kv_heads, 2 * cache->batch);
  const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_encode_kv),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kEncodeLds));
  if (ea != hipSuccess) return aatc::fail(AATC_ERR_HIP, "LDS attribute: %s", hipGetErrorString(ea));
  hipLaunchKernelGGL(k_encode_kv, grid, dim3(THREADS), kEncodeLds, static_cast<hipStream_t>(stream), ak, av,
                     static_cast<int>(cache->batch));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "encode_kv launch: %s", hipGetErrorString(e));
  return AATC_OK;
}

aatc_status aatc_decode(const aatc_cache* cache, int32_t which, int64_t token_offset, int64_t n_tokens,
                        void* out_dev, aatc_dtype out_dtype, const int64_t strides[3], void* stream) {
  return launch_codec(false, cache, which, out_dev, out_dtype, strides, token_offset, n_tokens, stream);
}

}  // extern "C"
