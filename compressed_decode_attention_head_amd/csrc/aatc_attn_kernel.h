// Decode attention that reads the packed cache directly (gfx950): two kernels per step.
//
// Page "SPECTRA ..." (Abstract) and page "SPHERICAL KV ..." (RDKV abstract): the cache is
// read again in full for each new token, so decode is bound by HBM reads of the cache;
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
// k_attn_main, grid (S splits, KV heads, batch): a workgroup of CW compute waves owns a
// contiguous range of 64-token tiles of one sequence, each wave `tpw` consecutive tiles.
//   1. Tile copies go straight from HBM into per-wave rings of LDS slots with global_load_lds
//      (no registers), issued before any load from memory.  In the producer form four extra
//      copy waves copy the tables and all but each compute wave's first two tiles and publish
//      every tile through an LDS flag as it lands; otherwise each compute wave copies its own.
//   2. The compute waves rotate the queries and build the limb weights while tiles land.
//   3. Each wave streams its tiles out of LDS in groups: scores -> one running-max update per
//      group -> probability rows -> PV, all in int32.
//   4. The waves merge in LDS; the workgroup writes one partial record per q head: (running
//      max, sum of probabilities, softmax-weighted code sum per V field column).
// Waves synchronise through LDS flags written and polled with hand-written ds instructions (an
// atomic or volatile access, or a workgroup barrier, would first wait for every copy in
// flight); every such wait is bounded.
// k_attn_combine, grid (q heads per KV head, KV heads, batch): merges the S records of a
// q head, folds field columns into channel code sums, dequantizes, applies R_V^T and writes
// out and lse.  The kernel boundary orders the records; no atomics, no workspace clearing.
#pragma once
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "aatc_internal.h"

namespace aatc_attn {

constexpr int D = AATC_D;
constexpr int PS = 16383;                 // probability scale: 14-bit fixed point, two 7-bit limbs
// log2(16383 / 65535) - 2^-20: pknorm(x) = rint(65535 x), so a token at the running max maps
// to 16383 and none exceeds it
constexpr float PKN_BIAS = -2.000067f;
constexpr int PHDR = 4;                   // record header floats: max (log2 units), sum of the
                                          // rounded probabilities, sum of the unrounded ones, 0
constexpr int CW = 8;                     // waves per workgroup
constexpr int TG = 4;                     // at most this many tiles per score group
constexpr int UNION_BYTES = 2 * 8 * D * 4;    // q / q~
constexpr int TAB_BYTES = 1280;           // K delta32 | o32 | bits
constexpr int WA_BYTES = 4 * 2 * 4 * 64 * 4;  // limb weight operands, NP <= 4
constexpr int FIXED_LDS = UNION_BYTES + TAB_BYTES + WA_BYTES;   // then the ring
constexpr int PROW_BYTES = 16 * 64;       // probability rows of one tile (16 rows x 64 bytes)
constexpr int DMA_PAD = 1024;             // LDS slack after the ring (bounded over-reads)
constexpr int SPIN_LIMIT = 1 << 22;       // polls before a wait gives up (results become NaN)
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint32_t* kcodes;
  const uint32_t* vcodes;
  int64_t tiles_per_seq;
  int n_kv, n_q, group;
  const int32_t* seq_lens;
  int seq_per_head;                   // seq_lens is [batch][n_kv] (else [batch])
  int64_t max_seq;
  const float* q;
  float scale2;                       // softmax scale * log2(e)
  float* part;                        // [batch*n_kv][S][group][prec] partial records
  float* offs;                        // [batch*n_kv][8] lse offset per q head (log2 units)
  int S, tpw, prec;                   // splits per sequence, tiles per wave, floats per record
  int kB, vB;
  int nslot;                          // ring slots per compute wave (>= 1)
  int slot_bytes, ksz;                // bytes per slot (K area first, ksz bytes)
  int wave_bytes;                     // ring bytes per compute wave: its slots, then (at the
                                      // end) its [NVB][32][4] floats of the merge
  int gs;                             // tiles per score group, 1..TGM, <= nslot
  int prod;                           // copy waves (0 or NPROD_MAX) issue every tile copy
  int kswz;                           // K tiles of whole 16-byte units per token (B_K = 128 U,
                                      // U = 1..4): the unit swizzle mask (3, 7, 3, 15); else 0
};

// Merge area per column group and wave: up to 12 groups every lane's raw int32 sums (both
// probability limbs, combined when the records are written); more groups fold the limbs in
// registers first (32 lanes x float4), to fit the ring.
constexpr int merge_group_bytes(int nvb) { return nvb <= 12 ? 64 * 16 : 32 * 16; }

constexpr int NPROD_MAX = 4;              // copy waves of the producer form (one per SIMD)
constexpr int SELF = 2;                   // producer form: tiles a compute wave copies itself, first

// Wave handshakes, in static LDS.
struct Sync {
  int arrive[CW];                     // barriers passed, per wave
  int landed[CW];                     // producer form: tiles of compute wave w in LDS
  int tabs[NPROD_MAX];                // producer form: copy wave p's table copies in LDS
  int broken;                         // a bounded wait gave up
  int prog[CW];                       // stream steps done, per compute wave
};


__device__ inline int row_max16_i(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));
  return x;
}

__device__ inline float row_sum16_f(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  return x;
}

__device__ inline unsigned row_sum16_u(unsigned x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x121, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x122, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x124, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xf, 0xf, false);
  return x;
}

// Value of lane (lane ^ M) for M in {1, 2, 4, 8, 16, 32}, on the vector ALU alone (DPP and
// permlane forms): no LDS round trip, which costs most while tile copies stream into LDS.
template <int M>
__device__ inline float xor_lanes(float x, int lane) {
  const int xi = __float_as_int(x);
  if (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xf, 0xf, false));   // quad [1,0,3,2]
  if (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xf, 0xf, false));   // quad [2,3,0,1]
  if (M == 4) {
    // lanes 0-3 and 8-11 of each row take lane + 4 (row_shl:4, banks 0 and 2), the others
    // lane - 4 (row_shr:4, banks 1 and 3)
    const int t = __builtin_amdgcn_update_dpp(xi, xi, 0x104, 0xf, 0x5, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(t, xi, 0x114, 0xf, 0xA, false));
  }
  if (M == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x128, 0xf, 0xf, false));  // row_ror 8
  if (M == 16) {
    // odd rows of the first result hold the even rows' values, even rows of the second the
    // odd rows' values
    const auto p = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(xi), static_cast<unsigned>(xi), false, false);
    return __int_as_float(static_cast<int>((lane & 16) ? p[0] : p[1]));
  }
  const auto p = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(xi), static_cast<unsigned>(xi), false, false);
  return __int_as_float(static_cast<int>(lane < 32 ? p[1] : p[0]));
}

__device__ inline float wave_max_x(float x) {
  const int lane = threadIdx.x & 63;
  x = fmaxf(x, xor_lanes<1>(x, lane));
  x = fmaxf(x, xor_lanes<2>(x, lane));
  x = fmaxf(x, xor_lanes<4>(x, lane));
  x = fmaxf(x, xor_lanes<8>(x, lane));
  x = fmaxf(x, xor_lanes<16>(x, lane));
  return fmaxf(x, xor_lanes<32>(x, lane));
}

__device__ inline float wave_sum_x(float x) {
  const int lane = threadIdx.x & 63;
  x += xor_lanes<1>(x, lane);
  x += xor_lanes<2>(x, lane);
  x += xor_lanes<4>(x, lane);
  x += xor_lanes<8>(x, lane);
  x += xor_lanes<16>(x, lane);
  return x + xor_lanes<32>(x, lane);
}

// Wave max of m and wave sum of x together: each stage's two exchanges are in flight at once.
__device__ inline void wave_max_sum_x(float& m, float& x) {
  const int lane = threadIdx.x & 63;
  m = fmaxf(m, xor_lanes<1>(m, lane));
  x += xor_lanes<1>(x, lane);
  m = fmaxf(m, xor_lanes<2>(m, lane));
  x += xor_lanes<2>(x, lane);
  const float m4 = xor_lanes<4>(m, lane), x4 = xor_lanes<4>(x, lane);
  m = fmaxf(m, m4);
  x += x4;
  m = fmaxf(m, xor_lanes<8>(m, lane));
  x += xor_lanes<8>(x, lane);
  const float m16 = xor_lanes<16>(m, lane), x16 = xor_lanes<16>(x, lane);
  m = fmaxf(m, m16);
  x += x16;
  m = fmaxf(m, xor_lanes<32>(m, lane));
  x += xor_lanes<32>(x, lane);
}

// Unnormalised Walsh-Hadamard transform (Sylvester order) of the 128 values x0 = v[lane],
// x1 = v[64 + lane] held by one wave: butterflies on index bit 6 in registers, bits 0..5
// across lanes (their order does not matter).
template <int M>
__device__ inline void fwht_stage(float& x0, float& x1, int lane) {
  const float p0 = xor_lanes<M>(x0, lane), p1 = xor_lanes<M>(x1, lane);
  const float sg = (lane & M) ? -1.f : 1.f;
  x0 = fmaf(sg, x0, p0);
  x1 = fmaf(sg, x1, p1);
}

__device__ inline void fwht128(float& x0, float& x1, int lane) {
  const float t = x0;
  x0 = t + x1;
  x1 = t - x1;
  fwht_stage<1>(x0, x1, lane);
  fwht_stage<2>(x0, x1, lane);
  fwht_stage<4>(x0, x1, lane);
  fwht_stage<8>(x0, x1, lane);
  fwht_stage<16>(x0, x1, lane);
  fwht_stage<32>(x0, x1, lane);
}

// Orders this wave's LDS accesses for the compiler.  A wavefront's LDS instructions execute
// in order, so no hardware wait is needed; a wavefront-scope fence does not wait on
// outstanding global loads.
__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Waits until at most n (0..63) vector-memory instructions of this wave are outstanding
// (n outside 0..63: until none are).
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

// LDS accesses the compiler does not order against copies in flight.  Any atomic or
// volatile LDS access is preceded by a wait for every outstanding vector-memory instruction,
// copies into LDS included; these hand-written forms are not (the load waits for itself).
__device__ inline uint32_t lds_addr(const void* p) { return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)); }
__device__ inline int lds_load_now(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ inline void lds_store(int* p, int v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// Compute waves w and w ^ 4 share a SIMD, whose arbiter favours the older wave throughout: on
// the batch-16 layer the younger one finished its tiles 7 us later, and the merge waited for it.
// At each stream step a wave publishes its step count and runs at the higher priority while it
// is behind its partner.  (With copy waves on the same SIMDs, whose publishing the compute
// waves wait for, it cost the 128K 1.33-bit layer 0.5 us; that form alternates by tile instead.)
__device__ inline void balance_simd(Sync* sy, int wave, int step) {
  lds_store(&sy->prog[wave], step);
  const int other = __builtin_amdgcn_readfirstlane(lds_load_now(&sy->prog[wave ^ 4]));
  if (step < other)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Barrier of the CW waves on per-wave LDS flags (`phase` counts the barriers this wave has
// passed).  Unlike s_barrier with a workgroup fence it does not wait for this wave's copies in
// flight: a wave's LDS operations complete in issue order, so its writes before the flag are
// visible once the flag is.  Bounded: after SPIN_LIMIT polls the workgroup is marked broken.
__device__ inline void compute_barrier(Sync* sy, int& phase, int lane) {
  ++phase;
  if (lane == 0) lds_store(&sy->arrive[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)], phase);
  for (int it = 0; it < SPIN_LIMIT; ++it) {
    const int v = lane < CW ? lds_load_now(&sy->arrive[lane]) : phase;
    if (__builtin_amdgcn_ballot_w64(v < phase) == 0) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0) lds_store(&sy->broken, 1);
}

// Waits (bounded) until *p >= v; on giving up marks the workgroup broken.
__device__ inline void poll_ge(const int* p, int v, Sync* sy, int lane) {
#pragma unroll 1
  for (int it = 0; it < SPIN_LIMIT; ++it) {
    // every lane reads the same word: compare once, in a scalar register
    if (__builtin_amdgcn_readfirstlane(lds_load_now(p)) >= v) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0) lds_store(&sy->broken, 1);
}

// Whole-power-of-two step that keeps a group's maximum mx below a reference of im * es + sh
// (log2 units, im an integer score anchor): 0 when it already is, else the k with
// im * es + sh + k >= mx * es + 2^-16 (the margin absorbs the rounding of the product).
__device__ inline int ref_shift(int mx, int im, float es, int sh) {
  if (mx == INT_MIN || im == INT_MIN) return 0;
  const float x = static_cast<float>(mx - im) * es - static_cast<float>(sh) + 1.52587890625e-5f;
  return x > 0.f ? static_cast<int>(ceilf(x)) : 0;
}

// x / 2^k rounded to nearest (k >= 0; 0 for k >= 32).
__device__ inline unsigned shift_round(unsigned x, int k) {
  if (k <= 0) return x;
  if (k >= 32) return 0u;
  return static_cast<unsigned>((static_cast<uint64_t>(x) + (1ull << (k - 1))) >> k);
}

// Exact rescale by 2^-k of a probability-weighted code sum held as two limbs: lanes 0..31 hold
// the high limb (weight 128) and lane + 32 the low limb of the same (head, column).  A 32-lane
// swap of the register with itself hands every lane both limbs (high in the first result, low
// in the second); the value 128 * high + low (below 2^31 while a wave streams at most 64 tiles)
// is divided with one rounding, (v + rnd) >> k, and split again by a per-lane field extract:
// bits 7.. on high-limb lanes (off 7, width 25), bits 0..6 on low-limb lanes (off 0, width 7).
// The caller passes k <= 31 and rnd = 2^(k-1) (0 for k = 0); a shift of 32 or more, where the
// value rounds to 0, is k = 31 with rnd = 0.
__device__ inline int shift_limbs(int x, unsigned k, unsigned rnd, unsigned off, unsigned width) {
  const auto p = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
  const unsigned v = ((p[0] << 7) + p[1] + rnd) >> k;
  return static_cast<int>(__builtin_amdgcn_ubfe(v, off, width));
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

// Copies the 16-byte units covering bytes [p, p + n) (p rounded down to 16) to LDS dst, one
// instruction per 64 units (lanes past the last unit idle).  Returns the instructions issued.
// With swz != 0 (a K tile of B = 128 U bits, U = 1..4, so 16-byte aligned and 64 U units, a
// whole number of 16-unit blocks) LDS unit s holds source unit s ^ ((s >> 4) & swz): an
// involution within each 16-unit block that puts the units one score instruction reads (tokens
// 16a + 4b + tau of a fixed tau, one unit each) in 16 different bank groups instead of four or
// fewer (B = 512: the 64-byte token stride maps them all to the same banks).
__device__ inline int dma_bytes(const char* p, int n, uint8_t* dst, int lane, int swz = 0) {
  const char* a = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(p) & ~static_cast<uintptr_t>(15));
  const int units = static_cast<int>((p + n - a + 15) >> 4);
  int ni = 0;
  for (int i = 0; i < units; i += 64, ++ni)
    if (i + lane < units) {
      const int s = i + lane;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a + (s ^ ((s >> 4) & swz)) * 16), dst + i * 16, 16,
                                       0, 0);
    }
  return ni;
}

// Word of a K tile in LDS holding plane bits [o, o + 32) of the tile's string (o a multiple of
// 32 when swz != 0): the unit o / 128 moved by dma_bytes' swizzle.
__device__ inline int k_word(int o, int swz) {
  const int pu = o >> 7;
  return ((pu ^ ((pu >> 4) & swz)) << 2) | ((o >> 5) & 3);
}

template <int NP, bool HALF, int NVB, int LIMBS, int NPROD, int TGM>
__global__ __launch_bounds__((CW + NPROD) * 64) void k_attn_main(AttnArgs a, const aatc_calib* __restrict__ kcal,
                                                                 const aatc_calib* __restrict__ vcal) {
  using LM = Lim<LIMBS>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);                       // [8][128]   q
  float* qt = qs + 8 * D;                                           // [8][128]   R_K q (KLT)
  uint8_t* tab = smem + UNION_BYTES;
  float* t_delta = reinterpret_cast<float*>(tab);                   // [128]
  float* t_o = t_delta + D;                                         // [128]
  const uint8_t* t_bits = tab + 1024;                               // [128]
  int* wa_lds = reinterpret_cast<int*>(smem + UNION_BYTES + TAB_BYTES);        // [NP*2*4*64]
  uint8_t* ring = smem + FIXED_LDS;                                 // [CW][wave_bytes]
  // probability limb rows live in their own static array: no tile copy can write them, so
  // reading them needs no wait on the copies in flight
  __shared__ __align__(16) uint8_t pl[CW * TGM * PROW_BYTES];       // [CW][TGM][16][64]
  __shared__ float s_m[CW][8], s_l[CW][8], s_e[CW][8];
  __shared__ float esc[8];
  __shared__ Sync sy;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // wave-uniform, kept scalar
  // the flags start at zero: the only workgroup barrier, before any load or copy
  if (tid < CW) {
    sy.arrive[tid] = 0;
    sy.landed[tid] = 0;
    sy.prog[tid] = 0;
  }
  if (tid < NPROD_MAX) sy.tabs[tid] = 0;
  if (tid == 0) sy.broken = 0;
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  const int n16 = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.n_kv + h;
  const aatc_calib* kc = kcal + h;
  const aatc_calib* vc = vcal + h;
  const int G = a.group;
  const int Bk = a.kB, Bv = a.vB;
  const int NS = a.nslot;
  const int64_t kbytes = 8 * static_cast<int64_t>(Bk), vbytes = 8 * static_cast<int64_t>(Bv);
  const char* kseq = reinterpret_cast<const char*>(a.kcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * kbytes;
  const char* vseq = reinterpret_cast<const char*>(a.vcodes) + static_cast<int64_t>(bh) * a.tiles_per_seq * vbytes;
  auto first_tile = [&](int w) { return (s * CW + w) * a.tpw; };
  // the producer form is planned only when every tile of a wave has its own slot
  auto slot_of = [&](int w, int r) { return ring + w * a.wave_bytes + (NPROD > 0 ? r : r % NS) * a.slot_bytes; };

  const int tw0 = first_tile(wave);

  // ---- 1. copies, issued before any load from memory: this wave's share of the queries and
  // K tables, then as many of its tiles as its ring holds (usually all of them; they land
  // while the prologue runs).  Until the sequence length is known, tiles up to max_seq are
  // copied (they lie inside the cache); only tiles below the length are used.
  // table copies of the WAVES copying waves, instruction k by wave k % WAVES
  auto copy_tables = [&](auto waves_tag, int me) {
    constexpr int WAVES = decltype(waves_tag)::value;
    int k = 0;
    k = dma_words<WAVES>(a.q + (static_cast<int64_t>(b) * a.n_q + h * G) * D, qs, G * D, k, me, lane);
    k = dma_words<WAVES>(kc->delta32, t_delta, D, k, me, lane);
    k = dma_words<WAVES>(kc->o32, t_o, D, k, me, lane);
    k = dma_words<WAVES>(kc->bits, tab + 1024, D / 4, k, me, lane);
  };
  if (NPROD == 0) copy_tables(std::integral_constant<int, CW>(), wave);
  // tile r of this wave goes to ring slot r % NS; copies are issued in tile order, so tile r
  // has landed once at most (instructions issued after it) copies are outstanding
  // tile r of compute wave w: its K and V bytes, the copy instructions they take, its slot
  auto kaddr_w = [&](int w, int r) { return kseq + (first_tile(w) + r) * kbytes; };
  auto vaddr_w = [&](int w, int r) { return vseq + (first_tile(w) + r) * vbytes; };
  auto ninstr_w = [&](int w, int r) {
    const int uk = Bk > 0 ? static_cast<int>((((reinterpret_cast<uintptr_t>(kaddr_w(w, r)) & 15) + kbytes + 15) >> 4)) : 0;
    const int uv = Bv > 0 ? static_cast<int>((((reinterpret_cast<uintptr_t>(vaddr_w(w, r)) & 15) + vbytes + 15) >> 4)) : 0;
    return ((uk + 63) >> 6) + ((uv + 63) >> 6);
  };
  auto copy_tile = [&](int w, int r) {
    uint8_t* sl = slot_of(w, r);
    if (Bk > 0) dma_bytes(kaddr_w(w, r), static_cast<int>(kbytes), sl, lane, a.kswz);
    if (Bv > 0) dma_bytes(vaddr_w(w, r), static_cast<int>(vbytes), sl + a.ksz, lane);
  };
  auto ninstr = [&](int r) { return ninstr_w(wave, r); };
  int nxt = 0;                           // next tile of this wave to copy (self-issue form)
  auto issue_upto = [&](int limit, int nmax) {   // copy tiles [nxt, min(limit, nmax))
    const int lim = limit < nmax ? limit : nmax;
    for (; nxt < lim; ++nxt) copy_tile(wave, nxt);
  };
  auto wait_tile = [&](int r) {
    int after = 0;
    for (int t = r + 1; t < nxt; ++t) after += ninstr(t);
    wait_vmcnt(after);
  };
  // tiles of compute wave w below max_seq (copied before the sequence length is known)
  auto ncap_w = [&](int w) {
    const int n = static_cast<int>((a.max_seq + 63) / 64) - first_tile(w);
    return n < 0 ? 0 : (n < a.tpw ? n : a.tpw);
  };
  // Form without copy waves: the tables and, for KLT and NOVA caches, this thread's quarter
  // row of R_K (into registers) are loaded first and the prologue runs on them before any tile
  // copy is issued (the first stream group issues them).  Every wave issuing its first tiles at
  // once saturates HBM, and issuing then blocks until the queue drains (about 3 us at 4 bits),
  // so copies issued before the prologue would hold it back by that long.
  constexpr int TPR = CW * 64 / D, CPT = D / TPR;
  static_assert(TPR == 4, "threads per row");
  float2 rrow[CPT / 2];
  bool rpre = false;
  if constexpr (NPROD == 0) {
    const int rot0 = kc->rotation;
    rpre = rot0 == AATC_ROT_KLT || rot0 == AATC_ROT_NOVA;
    if (rpre) {
      const float2* row = reinterpret_cast<const float2*>(kc->R32 + (tid / TPR) * D + CPT * (tid % TPR));
#pragma unroll
      for (int c2 = 0; c2 < CPT / 2; ++c2) rrow[c2] = row[c2];
    }
  }
  // producer form: a copy wave sustains only a few GB/s, so the compute waves copy their own
  // first SELF tiles (all eight waves issuing at once) and the copy waves the rest
  if (NPROD > 0 && wave < CW) issue_upto(SELF, ncap_w(wave));
  if (NPROD > 0 && wave >= CW) {
    // ---- copy wave p: the tables' share k % NPROD == p, then every tile of compute waves
    // CPP*p .. CPP*p + CPP - 1 in the order they are consumed, publishing each as it lands.
    // The compute waves never block on an issue queue that HBM drains.
    constexpr int CPP = CW / (NPROD > 0 ? NPROD : 1);
    const int p = wave - CW;
    copy_tables(std::integral_constant<int, (NPROD > 0 ? NPROD : 1)>(), p);
    wait_vmcnt(0);                       // the compute waves start their prologue on the tables
    if (lane == 0) lds_store(&sy.tabs[p], 1);
    int total = 0;
    for (int r = SELF; r < a.tpw; ++r)
      for (int ci = 0; ci < CPP; ++ci) {
        const int w = CPP * p + ci;
        if (r < ncap_w(w)) {
          copy_tile(w, r);
          total += ninstr_w(w, r);
        }
      }
    for (int r = SELF; r < a.tpw; ++r)
      for (int ci = 0; ci < CPP; ++ci) {
        const int w = CPP * p + ci;
        if (r < ncap_w(w)) {
          total -= ninstr_w(w, r);
          wait_vmcnt(total);             // copies complete in issue order
          if (lane == 0) lds_store(&sy.landed[w], r + 1);
        }
      }
    return;
  }

  asm volatile("" ::: "memory");         // the loads below stay behind the copies

  int64_t seq64 = a.seq_lens ? static_cast<int64_t>(a.seq_lens[a.seq_per_head ? bh : b]) : a.max_seq;
  seq64 = seq64 < 0 ? 0 : (seq64 > a.max_seq ? a.max_seq : seq64);     // never read past the cache
  const int seq = static_cast<int>(seq64);                      // tokens per sequence < 2^31
  const int ntiles = (seq + 63) / 64;
  auto tiles_of = [&](int w) {
    const int t0 = first_tile(w);
    const int n = ntiles - t0 < a.tpw ? ntiles - t0 : a.tpw;
    return n > 0 ? n : 0;
  };

  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;   // scalar loads
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4, T1 = (n1 + 15) >> 4;
  const int NV = T4 + T2 + T1;
  // every header field is loaded at once: a short-circuit chain would wait for each in turn
  const uint32_t kmag = kc->magic, vmag = vc->magic;
  const int kbits = kc->total_bits, vbits = vc->total_bits;
  // (Lloyd-Max blobs take the level pass: their levels are not affine in the codes)
  const int kq = kc->quantizer, vq = vc->quantizer;
  const bool ok = (kmag == AATC_MAGIC) & (vmag == AATC_MAGIC) & (kbits == Bk) & (vbits == Bv) & (n4 >= 0) &
                  (n2 >= 0) & (n1 >= 0) & (NV <= NVB) & (PHDR + 16 * NV <= a.prec) & (kq == 0) & (vq == 0);
  // a NOVA blob holds its query transform E^-T where a KLT blob holds R: the same GEMV
  const int rot = kc->rotation == AATC_ROT_NOVA ? AATC_ROT_KLT : kc->rotation;
  const int nw = ok ? tiles_of(wave) : 0;   // a bad blob streams nothing

  // ---- stream set-up that needs no table: it runs while the tables are in flight
  // head slots this lane holds after the limb merge: LIMBS=2 pair a {0,4,1,5}[grp] and
  // pair b {2,6,3,7}[grp]; LIMBS=3 head grp
  const int ha = LIMBS == 2 ? (grp & 1) * 4 + (grp >> 1) : grp;
  const int hb = ha + 2;
  // score lane n16 of token group tau holds token 16*(n16/4) + 4*(n16%4) + tau, so that the
  // probability bytes it packs are the PV operand's K order (token 16*grp + 4*i + byte)
  const int tok0 = 16 * (n16 >> 2) + 4 * (n16 & 3);
  int kofs[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) kofs[u] = tok0 * Bk + plane_base(u, grp, HALF && u == NP - 1);
  uint8_t* pw = pl + wave * TGM * PROW_BYTES;
  // probability rows (limb l, head slot x) = row 8l + x; dword n16 of a row sits in 16-byte
  // quad (n16/4) ^ (row%4)
  auto prow_addr = [&](int row) { return row * 64 + 16 * ((n16 >> 2) ^ (row & 3)) + 4 * (n16 & 3); };
  const int wa0 = prow_addr(ha), wa1 = prow_addr(8 + ha);
  const int wb0 = prow_addr(hb), wb1 = prow_addr(8 + hb);
  const int prd = n16 * 64 + 16 * (grp ^ (n16 & 3));
  // LDS byte offset (within a tile's V area) of the V word(s) this lane reads for column group v:
  // a scalar part (the group's class and position) plus one of three lane parts
  const int L4 = 32 * n16 + 8 * grp, L2 = 16 * n16 + 4 * grp, L1 = 8 * n16 + 4 * (grp >> 1);
  int voff[NVB];
#pragma unroll
  for (int v = 0; v < NVB; ++v) {
    const int s4 = 512 * v, s2 = 32 * n4 + 256 * (v - T4), s1 = 32 * n4 + 16 * n2 + 128 * (v - T4 - T2);
    // unused group (v >= NV): a harmless read of the tile's first words
    voff[v] = v < T4 ? s4 + L4 : (v < T4 + T2 ? s2 + L2 : (v < NV ? s1 + L1 : 0));
  }
  const uint32_t rot1 = grp & 1;

  v4i acc[NVB];
#pragma unroll
  for (int v = 0; v < NVB; ++v) acc[v] = v4i{0, 0, 0, 0};
  int ima = INT_MIN, imb = INT_MIN;       // integer score anchors: the first group's maxima
  int sha = 0, shb = 0;                   // reference = anchor (log2 units) + this power of two
  float bia = PKN_BIAS, bib = PKN_BIAS;   // PKN_BIAS - sha, PKN_BIAS - shb
  unsigned la = 0, lb = 0;               // sums of the rounded probabilities (PV's weights)
  float ea = 0.f, eb = 0.f;               // sums of the unrounded ones (for the lse)
  const v2u16 ones = {1, 1};

  int phase = 0;
  if (NPROD == 0) {
    int after = 0;                       // this wave's table copies have landed ...
    for (int t = 0; t < nxt; ++t) after += ninstr(t);
    wait_vmcnt(after);
    compute_barrier(&sy, phase, lane);   // ... and so have everyone else's
  } else {
    for (int q = 0; q < NPROD; ++q) poll_ge(&sy.tabs[q], 1, &sy, lane);
  }

  // ---- 1. prologue: q~ = R_K q, alpha, exponents, lse offsets, limb weights
  // wave x (< 8) owns head slot x: q~ at channels lane and 64 + lane.  With three limbs (at most
  // four head slots) and the rotation's barrier to order them, waves x and x + 4 share head slot
  // x: both zero the limb rows beforehand, and each writes the planes of one half of the channels.
  const bool halves = LIMBS == 3 && rot == AATC_ROT_KLT;
  const int hslot = halves ? (wave & 3) : wave;
  float y0 = 0.f, y1 = 0.f;
  if (rot == AATC_ROT_KLT) {
    // row i of R_K: 4 threads per row, GH q heads per thread (the head slots a group can use:
    // 4 with three limbs, 8 with two)
    constexpr int GH = LIMBS == 3 ? 4 : 8;
    const int i = tid / TPR, qq = tid % TPR;
    float part[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) part[g] = 0.f;
    const float2* row = reinterpret_cast<const float2*>(kc->R32 + i * D + CPT * qq);
    if (NPROD == 0 && rpre) {
#pragma unroll
      for (int c2 = 0; c2 < CPT / 2; ++c2) {
        const float2 rr = rrow[c2];
        const int j = CPT * qq + 2 * c2;
#pragma unroll
        for (int g = 0; g < GH; ++g) part[g] += rr.x * qs[g * D + j] + rr.y * qs[g * D + j + 1];
      }
    } else {
#pragma unroll 4
      for (int c2 = 0; c2 < CPT / 2; ++c2) {
        const float2 rr = row[c2];
        const int j = CPT * qq + 2 * c2;
#pragma unroll
        for (int g = 0; g < GH; ++g) part[g] += rr.x * qs[g * D + j] + rr.y * qs[g * D + j + 1];
      }
    }
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      part[g] += xor_lanes<1>(part[g], lane);
      part[g] += xor_lanes<2>(part[g], lane);
    }
    if (qq == 0)
#pragma unroll
      for (int g = 0; g < GH; ++g) qt[g * D + i] = part[g];
    if (halves)
      for (int k = tid; k < NP * 2 * 4 * 64; k += CW * 64) wa_lds[k] = 0;
    compute_barrier(&sy, phase, lane);
    y0 = qt[hslot * D + lane];
    y1 = qt[hslot * D + 64 + lane];
  } else {
    y0 = qs[wave * D + lane];
    y1 = qs[wave * D + 64 + lane];
    if (rot == AATC_ROT_WHT) {
      // Sylvester-ordered fast Walsh-Hadamard transform across the wave, then 1/sqrt(128)
      fwht128(y0, y1, lane);
      y0 *= 0.08838834764831845f;
      y1 *= 0.08838834764831845f;
    }
  }
  {
    // alpha, the lse offset and the weight exponent of head slot hslot (zero past G)
    const int g = hslot;
    if (g >= G) {
      y0 = 0.f;
      y1 = 0.f;
    }
    float m = 0.f, off = 0.f;
    float alr[2], dl[2], ol[2];
    int bir[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {        // every table read issued before any is used
      const int i = lane + 64 * r;
      bir[r] = t_bits[i];
      dl[r] = t_delta[i];
      ol[r] = t_o[i];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int bi = bir[r];
      const float v = r ? y1 : y0;
      const float half = static_cast<float>((1 << bi) >> 1);   // 2^(b-1), 0 for b = 0
      const float alpha = bi ? v * dl[r] * a.scale2 : 0.f;
      alr[r] = alpha;
      m = fmaxf(m, fabsf(alpha) * half);
      const float o = bi ? ol[r] - dl[r] * (half - 0.5f) : ol[r];
      off += v * o * a.scale2;
    }
    wave_max_sum_x(m, off);
    int e = 0;
    if (m > 0.f) {
      frexpf(m, &e);
      e = LM::WBITS - e;                 // m * 2^e in [2^(WBITS-1), 2^WBITS)
    }
    if (lane == 0 && (!halves || wave < 4)) {
      esc[g] = (m > 0.f) ? ldexpf(1.f, -e) : 0.f;
      if (s == 0 && g < G) a.offs[bh * 8 + g] = off;
    }
    // limb operand rows of head slot g (the wave's own, or with halves its and its partner's,
    // which writes other bytes): LIMBS=2 rows g and 8+g; LIMBS=3 rows g, 4+g, 8+g for g < 4 and
    // the spare row 8+g else.  Operand dword (pair u, half hh, dword j, lane) holds bytes m of
    // row lane%16, lane group lane/16 (the plane_base windows).  First zero them (with halves,
    // every row before the rotation's barrier), then write each plane's limbs.
    const int nrows = (LIMBS == 3 && g >= 4) ? 1 : LIMBS;
    auto row_of = [&](int l) { return LIMBS == 2 ? 8 * l + g : (g < 4 ? 4 * l + g : 8 + g); };
    if (!halves)
      for (int k = lane; k < nrows * NP * 32; k += 64) {
        const int l = k / (NP * 32), c = (k >> 2) % (NP * 8), lg = k & 3;
        wa_lds[c * 64 + lg * 16 + row_of(l)] = 0;
      }
    // plane index of this lane's channels' bit 0: prefix sums of the bit counts, one ballot
    // per bit level
    const uint64_t below = (1ull << lane) - 1ull;
    int pb0 = 0, pb1 = 0, tot0 = 0;
    int kmax = 0;
    for (int k = 1; k <= AATC_MAX_BITS; ++k) {
      const uint64_t b0 = __ballot(bir[0] >= k), b1 = __ballot(bir[1] >= k);
      if ((b0 | b1) == 0) break;
      kmax = k;
      pb0 += __popcll(b0 & below);
      pb1 += __popcll(b1 & below);
      tot0 += __popcll(b0);
    }
    pb1 += tot0;
    uint8_t* wab = reinterpret_cast<uint8_t*>(wa_lds);
    const int wmaxq = (1 << LM::WBITS) - 1;
    if (g < G) {
      for (int kb = 0; kb < kmax; ++kb) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (kb < bir[r] && (!halves || r == (wave >> 2))) {
            const int p = (r ? pb1 : pb0) + kb;
            const int u = p >> 7, pp = p & 127, q = pp & 31;
            const bool hp = HALF && u == NP - 1;
            const int lg = hp ? 2 * (pp >> 5) + ((pp >> 2) & 1) : (pp >> 5);
            const int hh = hp ? 0 : ((q >> 2) & 1);
            const int dw = ((u * 2 + hh) * 4 + (q & 3)) * 64 + lg * 16;
            int wq = static_cast<int>(rintf(ldexpf(alr[r], kb + e)));
            wq = wq > wmaxq ? wmaxq : (wq < -wmaxq ? -wmaxq : wq);
#pragma unroll
            for (int l = 0; l < LIMBS; ++l) wab[4 * (dw + row_of(l)) + (q >> 3)] = static_cast<uint8_t>(LM::limb(l, wq));
          }
        }
      }
    }
  }
  // producer form: this wave's own tiles (issued first) have long landed; waiting for them here,
  // before the weights, keeps later register spill stores out of the wait
  if (NPROD > 0) wait_vmcnt(0);
  compute_barrier(&sy, phase, lane);
  v4i wa[NP][2];
#pragma unroll
  for (int u = 0; u < NP; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[u][hh][j] = wa_lds[((u * 2 + hh) * 4 + j) * 64 + lane];

  const float esa = esc[ha], esb = LIMBS == 2 ? esc[hb] : 0.f;

  // ---- 2. stream this wave's tiles, groups of gs
  bool started = false;
  int step = 0;                          // balance_simd steps (forms without copy waves): each tile's
                                         // scores, each group's PV
#pragma unroll 1
  for (int g0 = 0; g0 < nw; g0 += a.gs) {
    const int ng = nw - g0 < a.gs ? nw - g0 : a.gs;
    if (NPROD == 0) issue_upto(g0 + NS, nw);   // every free slot: tiles before g0 are done with

    // opaque copies of the V class bounds: keeps the compiler from hoisting one condition
    // register pair per column group out of the loop
    int cT4 = T4, cT42 = T4 + T2, cNV = NV;
    asm volatile("" : "+s"(cT4), "+s"(cT42), "+s"(cNV));
    int sa[TGM][4], sb[TGM][4];
    // scores, tile by tile as each lands: 4 token groups of 16 = 4 independent MFMA chains
#pragma unroll
    for (int g = 0; g < TGM; ++g) {
      if (g >= ng) {                                    // past the group's end: no tile, masked
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          sa[g][tau] = INT_MIN;
          sb[g][tau] = INT_MIN;
        }
        continue;
      }
      const int rr = g0 + g;
      if (NPROD > 0) {
        // its own copies (the first SELF tiles) were waited for before the weights
        if (g0 + g >= SELF) poll_ge(&sy.landed[wave], g0 + g + 1, &sy, lane);
      } else {
        wait_tile(g0 + g);
      }
      wave_sync_lds();
      if (NPROD == 0) balance_simd(&sy, wave, ++step);
      // producer form: the flag round trips of balance_simd cost more than they even out (the
      // copy waves share the SIMDs); the two compute waves of a SIMD take turns by tile instead
      if (NPROD > 0) {
        if ((g + (wave >> 2)) & 1)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
      const int64_t tile = tw0 + rr;
      // opaque slot offset: per-(tile, tau, pair) addresses are not worth registers
      int kt = static_cast<int>((slot_of(wave, rr) - ring) + ((reinterpret_cast<uintptr_t>(kseq) + tile * kbytes) & 15));
      asm volatile("" : "+v"(kt));
      const uint8_t* klt = ring + kt;
      v4i cc[4];
      // swizzled K tiles (whole units per token, so every window is one aligned word) read one
      // word at a moved address; the two forms are separate loops, so neither pays for the other
      auto scores = [&](auto swz_tag) {
        constexpr bool SWZ = decltype(swz_tag)::value;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          cc[tau] = v4i{0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < NP; ++u) {
            const bool hp = HALF && u == NP - 1;
            const int o = kofs[u] + tau * Bk;
            const uint32_t* kwp = reinterpret_cast<const uint32_t*>(klt);
            uint32_t dw;
            if constexpr (SWZ) {
              dw = kwp[k_word(o, a.kswz)];
            } else {
              const uint32_t* w = kwp + (o >> 5);
              dw = __builtin_amdgcn_alignbit(w[1], w[0], static_cast<uint32_t>(o));
            }
            v4i b0;
#pragma unroll
            for (int j = 0; j < 4; ++j) b0[j] = static_cast<int>((dw >> j) & 0x01010101u);
            cc[tau] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][0], b0, cc[tau], 0, 0, 0);
            if (!hp) {
              v4i b1;
#pragma unroll
              for (int j = 0; j < 4; ++j) b1[j] = static_cast<int>((dw >> (j + 4)) & 0x01010101u);
              cc[tau] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][1], b1, cc[tau], 0, 0, 0);
            }
          }
        }
      };
      if constexpr (!HALF) {
        if (a.kswz != 0)
          scores(std::true_type{});
        else
          scores(std::false_type{});
      } else {
        scores(std::false_type{});
      }
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        if (LIMBS == 2) {
          const auto p01 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[tau][0]),
                                                            static_cast<unsigned>(cc[tau][1]), false, false);
          const auto p23 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[tau][2]),
                                                            static_cast<unsigned>(cc[tau][3]), false, false);
          sa[g][tau] = (static_cast<int>(p01[0]) << 7) + static_cast<int>(p01[1]);
          sb[g][tau] = (static_cast<int>(p23[0]) << 7) + static_cast<int>(p23[1]);
        } else {
          // 4x4 transpose of 16-lane blocks: rows (limb l, head r) -> lane group = head
          const auto x02 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[tau][0]),
                                                            static_cast<unsigned>(cc[tau][2]), false, false);
          const auto x13 = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(cc[tau][1]),
                                                            static_cast<unsigned>(cc[tau][3]), false, false);
          const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);   // limb 0, 1
          const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);   // limb 2, -
          sa[g][tau] = (static_cast<int>(y01[0]) << 14) + (static_cast<int>(y01[1]) << 7) + static_cast<int>(y23[0]);
          sb[g][tau] = INT_MIN;
        }
      }
    }
    // tiles past the group's end and tokens past the sequence's end take no part
    const bool masked = ng < TGM || seq - (tw0 + g0 + ng - 1) * 64 < 64;
    if (masked) {
#pragma unroll
      for (int g = 0; g < TGM; ++g) {
        const int nvalid = g < ng ? seq - (tw0 + g0 + g) * 64 : 0;
        if (nvalid < 64) {
#pragma unroll
          for (int tau = 0; tau < 4; ++tau)
            if (tok0 + tau >= nvalid) { sa[g][tau] = INT_MIN; sb[g][tau] = INT_MIN; }
        }
      }
    }
    // group maxima (every tile has a visible token, so they are real scores)
    int mxa = INT_MIN, mxb = INT_MIN;
#pragma unroll
    for (int g = 0; g < TGM; ++g) {
      mxa = max(mxa, max(max(sa[g][0], sa[g][1]), max(sa[g][2], sa[g][3])));
      if (LIMBS == 2) mxb = max(mxb, max(max(sb[g][0], sb[g][1]), max(sb[g][2], sb[g][3])));
    }
    mxa = row_max16_i(mxa);
    if (LIMBS == 2) mxb = row_max16_i(mxb);
    // online softmax.  The first group anchors each head's reference at its integer maximum;
    // a later group whose maximum passes the reference raises it by a whole power of two, so
    // that the accumulators are rescaled exactly (no rounding of the high limb on its own)
    if (!started) {
      ima = mxa;
      imb = mxb;
      started = true;
    } else {
      const int ka = ref_shift(mxa, ima, esa, sha);
      const int kb = LIMBS == 2 ? ref_shift(mxb, imb, esb, shb) : 0;
      if (__ballot((ka | kb) != 0)) {
        la = shift_round(la, ka);
        lb = shift_round(lb, kb);
        ea = ldexpf(ea, -ka);
        eb = ldexpf(eb, -kb);
        // shift of each accumulator register, per lane, and whether any lane of it moves (a
        // wave-uniform test: registers whose heads keep their reference are left alone)
        int kr[4], kany[4];
        if (LIMBS == 2) {
          // acc register r of lane group grp holds head 4*(grp&1)+r; the shift of head hd
          // lives in pair a (heads {0,4,1,5} in lane groups 0..3) or pair b ({2,6,3,7})
          const bool odd = grp & 1;
          const int a0 = __builtin_amdgcn_readlane(ka, 0), a1 = __builtin_amdgcn_readlane(ka, 16);
          const int a2 = __builtin_amdgcn_readlane(ka, 32), a3 = __builtin_amdgcn_readlane(ka, 48);
          const int b0 = __builtin_amdgcn_readlane(kb, 0), b1 = __builtin_amdgcn_readlane(kb, 16);
          const int b2 = __builtin_amdgcn_readlane(kb, 32), b3 = __builtin_amdgcn_readlane(kb, 48);
          kr[0] = odd ? a1 : a0;
          kr[1] = odd ? a3 : a2;
          kr[2] = odd ? b1 : b0;
          kr[3] = odd ? b3 : b2;
          kany[0] = a0 | a1;
          kany[1] = a2 | a3;
          kany[2] = b0 | b1;
          kany[3] = b2 | b3;
        } else {
          // acc register r holds head r (rows 8l + r); head r's shift lives in lane group r
#pragma unroll
          for (int r = 0; r < 4; ++r) kany[r] = kr[r] = __builtin_amdgcn_readlane(ka, 16 * r);
        }
        const unsigned off = lane < 32 ? 7u : 0u, width = lane < 32 ? 25u : 7u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (kany[r] != 0) {
            const unsigned k = static_cast<unsigned>(kr[r]);
            const unsigned kk = k > 31u ? 31u : k;
            const unsigned rnd = (k == 0u || k > 31u) ? 0u : (1u << (k - 1u));
#pragma unroll
            for (int v = 0; v < NVB; ++v) acc[v][r] = shift_limbs(acc[v][r], kk, rnd, off, width);
          }
        }
        sha += ka;
        shb += kb;
        bia = PKN_BIAS - static_cast<float>(sha);
        bib = PKN_BIAS - static_cast<float>(shb);
      }
    }
    // probabilities in 14-bit fixed point (pknorm rounds 65535 * x), two 7-bit limbs; the
    // four tokens of this lane fill one dword per (head, limb); tile g uses rows at g*1024
#pragma unroll
    for (int g = 0; g < TGM; ++g) {
      if (g < ng) {
        uint8_t* pg = pw + g * PROW_BYTES;
        {
          float pa[4];
#pragma unroll
          for (int tau = 0; tau < 4; ++tau)
            pa[tau] = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sa[g][tau] - ima), esa, bia));
          if (masked) {
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) pa[tau] = sa[g][tau] == INT_MIN ? 0.f : pa[tau];
          }
          const v2u16 q01 = __builtin_amdgcn_cvt_pknorm_u16(pa[0], pa[1]);
          const v2u16 q23 = __builtin_amdgcn_cvt_pknorm_u16(pa[2], pa[3]);
          la = __builtin_amdgcn_udot2(q01, ones, la, false);
          la = __builtin_amdgcn_udot2(q23, ones, la, false);
          ea += (pa[0] + pa[1]) + (pa[2] + pa[3]);
          const uint32_t u01 = __builtin_bit_cast(uint32_t, q01), u23 = __builtin_bit_cast(uint32_t, q23);
          *reinterpret_cast<uint32_t*>(pg + wa0) =
              __builtin_amdgcn_perm((u23 >> 7) & 0x007F007Fu, (u01 >> 7) & 0x007F007Fu, 0x06040200u);
          *reinterpret_cast<uint32_t*>(pg + wa1) = __builtin_amdgcn_perm(u23 & 0x007F007Fu, u01 & 0x007F007Fu, 0x06040200u);
        }
        if (LIMBS == 2) {
          float pb[4];
#pragma unroll
          for (int tau = 0; tau < 4; ++tau)
            pb[tau] = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sb[g][tau] - imb), esb, bib));
          if (masked) {
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) pb[tau] = sb[g][tau] == INT_MIN ? 0.f : pb[tau];
          }
          const v2u16 q01 = __builtin_amdgcn_cvt_pknorm_u16(pb[0], pb[1]);
          const v2u16 q23 = __builtin_amdgcn_cvt_pknorm_u16(pb[2], pb[3]);
          lb = __builtin_amdgcn_udot2(q01, ones, lb, false);
          lb = __builtin_amdgcn_udot2(q23, ones, lb, false);
          eb += (pb[0] + pb[1]) + (pb[2] + pb[3]);
          const uint32_t u01 = __builtin_bit_cast(uint32_t, q01), u23 = __builtin_bit_cast(uint32_t, q23);
          *reinterpret_cast<uint32_t*>(pg + wb0) =
              __builtin_amdgcn_perm((u23 >> 7) & 0x007F007Fu, (u01 >> 7) & 0x007F007Fu, 0x06040200u);
          *reinterpret_cast<uint32_t*>(pg + wb1) = __builtin_amdgcn_perm(u23 & 0x007F007Fu, u01 & 0x007F007Fu, 0x06040200u);
        }
      }
    }
    wave_sync_lds();
    if (NPROD == 0) balance_simd(&sy, wave, ++step);
    if (NPROD > 0) {                     // and the younger wave leads the PV
      if (wave >> 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    // PV on packed V fields (width-uniform column groups: w4 | w2 | w1); columns past a
    // class's field count read neighbouring words and are never used
#pragma unroll
    for (int g = 0; g < TGM; ++g) {
      if (g < ng) {
        const uint4 pv = *reinterpret_cast<const uint4*>(pw + g * PROW_BYTES + prd);
        const v4i pA = {static_cast<int>(pv.x), static_cast<int>(pv.y), static_cast<int>(pv.z), static_cast<int>(pv.w)};
        const int64_t tile = tw0 + g0 + g;
        int vt = static_cast<int>((slot_of(wave, g0 + g) - ring) + a.ksz +
                                  ((reinterpret_cast<uintptr_t>(vseq) + tile * vbytes) & 15));
        asm volatile("" : "+v"(vt));
        const uint8_t* vl = ring + vt;
        uint32_t x0[NVB];
#pragma unroll
        for (int v = 0; v < NVB; ++v)           // unconditional: no per-read waits
          x0[v] = *reinterpret_cast<const uint32_t*>(vl + voff[v]);
#pragma unroll
        for (int v = 0; v < NVB; ++v) {
          if (v < cNV) {
            // 2- and 1-bit fields: one rotation by the lane group's parity, then the same
            // shifts for both widths; only the mask differs (a scalar select)
            v4i bv;
            const uint32_t msk = v < cT42 ? 0x03030303u : 0x01010101u;
            const uint32_t d = __builtin_amdgcn_alignbit(x0[v], x0[v], rot1);
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = static_cast<int>((d >> (2 * r)) & msk);
            if (__builtin_expect(v < cT4, 0)) {
              // nibble fields (first in the tile): the second word only here (registers are
              // the scarce resource)
              const uint32_t x1 = *reinterpret_cast<const uint32_t*>(vl + voff[v] + 4);
              bv[0] = static_cast<int>(x0[v] & 0x0F0F0F0Fu);
              bv[1] = static_cast<int>((x0[v] >> 4) & 0x0F0F0F0Fu);
              bv[2] = static_cast<int>(x1 & 0x0F0F0F0Fu);
              bv[3] = static_cast<int>((x1 >> 4) & 0x0F0F0F0Fu);
            }
            acc[v] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pA, bv, acc[v], 0, 0, 0);
          }
        }
      }
    }
    wave_sync_lds();                     // the group's slots and rows are reused next
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- 3. workgroup merge in LDS: each wave parks its limb-merged code sums (unscaled) in its
  // own ring area once every copy into it has landed; one barrier; then every thread scales
  // and sums the CW waves' values of its record entries
  la = row_sum16_u(la);
  lb = row_sum16_u(lb);
  ea = row_sum16_f(ea) * 65535.f;        // the units of la: pknorm rounds 65535 x
  eb = row_sum16_f(eb) * 65535.f;
  const float ma = ima == INT_MIN ? -INFINITY : static_cast<float>(ima) * esa + static_cast<float>(sha);
  const float mb = imb == INT_MIN ? -INFINITY : static_cast<float>(imb) * esb + static_cast<float>(shb);
  if (n16 == 0) {
    s_m[wave][ha] = ma;
    s_l[wave][ha] = static_cast<float>(la);
    s_e[wave][ha] = ea;
    if (LIMBS == 2) {
      s_m[wave][hb] = mb;
      s_l[wave][hb] = static_cast<float>(lb);
      s_e[wave][hb] = eb;
    }
  }
  if (LIMBS == 3 && lane >= 4 && lane < 8) {
    s_m[wave][lane] = -INFINITY;
    s_l[wave][lane] = 0.f;
    s_e[wave][lane] = 0.f;
  }
  wait_vmcnt(0);                         // this wave's own copies, past the sequence's end too
  if (NPROD > 0 && ncap_w(wave) > SELF)  // and the copy waves' ones into its slots
    poll_ge(&sy.landed[wave], ncap_w(wave), &sy, lane);
  constexpr bool RAW = merge_group_bytes(NVB) == 64 * 16;
  if (RAW) {
    // every lane's sums as they are: lane group grp, register r holds row 4*grp + r (limb
    // grp/2, head slot 4*(grp%2) + r)
    v4i* mgw = reinterpret_cast<v4i*>(ring + wave * a.wave_bytes);
#pragma unroll
    for (int v = 0; v < NVB; ++v)
      if (v < NV) mgw[v * 64 + lane] = acc[v];
  } else {
    // limb merge: lanes 0..31 (limb 0 rows) take the limb-1 rows of lanes 32..63; lane group
    // grp<2 then holds head slots 4*grp + r
    float4* mgw = reinterpret_cast<float4*>(ring + wave * a.wave_bytes);
#pragma unroll
    for (int v = 0; v < NVB; ++v) {
      if (v < NV) {
        float4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const auto sw = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(acc[v][r]),
                                                           static_cast<unsigned>(acc[v][r]), false, false);
          const float c = 128.f * static_cast<float>(acc[v][r]) + static_cast<float>(static_cast<int>(sw[1]));
          if (r == 0) o.x = c;
          if (r == 1) o.y = c;
          if (r == 2) o.z = c;
          if (r == 3) o.w = c;
        }
        if (lane < 32) mgw[v * 32 + lane] = o;
      }
    }
  }
  compute_barrier(&sy, phase, lane);
  // ---- 4. partial records: [max, sum, 0, 0, column sums], every wave's values scaled to the
  // workgroup max of their q head
  if (RAW) {
    // wave 2j + qd: head quad qd (heads 4qd..4qd+3), column 64j + lane; each of a column's
    // sums is one 16-byte read per wave and limb (consecutive lanes, consecutive words)
    const int qd = wave & 1, col = (wave >> 1) * 64 + lane;
    const bool good = ok && __hip_atomic_load(&sy.broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
    const int ncol = ok ? 16 * NV : 0;     // a bad blob's field count may not fit a record
    // factors 2^(m_w - M) of the quad's heads: lane k < 32 holds wave k/4, head 4qd + k%4
    const int kw = (lane >> 2) & 7, kh = 4 * qd + (lane & 3);
    float mk = -INFINITY;
#pragma unroll
    for (int w = 0; w < CW; ++w) mk = fmaxf(mk, s_m[w][kh]);
    const float own = s_m[kw][kh];
    const float fk = own == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(own - mk);
    auto fw = [&](int w, int r) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fk), 4 * w + r)); };
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    const int cc = col < ncol ? col : 0;
    const int o = (cc >> 4) * 64 + 16 * qd + (cc & 15);     // limb 0; limb 1 is 32 lanes on
    // (128 * limb 0 + limb 1 stays inside int32 while a wave streams at most 64 tiles)
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      const v4i* mw_ = reinterpret_cast<const v4i*>(ring + w * a.wave_bytes);
      const v4i x0 = mw_[o], x1 = mw_[o + 32];
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] = fmaf(static_cast<float>(x0[r] * 128 + x1[r]), fw(w, r), sum[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * qd + r;
      float* rec = a.part + ((static_cast<int64_t>(bh) * a.S + s) * G + (hd < G ? hd : 0)) * a.prec;
      if (hd < G && col < ncol) rec[PHDR + col] = sum[r];
      if (hd < G && wave < 2 && lane == 0) {
        float l = 0.f, le = 0.f;
#pragma unroll
        for (int w = 0; w < CW; ++w) {
          l += s_l[w][hd] * fw(w, r);
          le += s_e[w][hd] * fw(w, r);
        }
        const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), r));
        rec[0] = good ? m : NAN;
        rec[1] = l;
        rec[2] = le;
        rec[3] = 0.f;
      }
    }
  } else if (wave < G) {
    const int hd = wave;
    const bool good = ok && __hip_atomic_load(&sy.broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
    const int ncol = ok ? 16 * NV : 0;     // a bad blob's field count may not fit a record
    float* rec = a.part + ((static_cast<int64_t>(bh) * a.S + s) * G + hd) * a.prec;
    float mw[CW], f[CW];
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      mw[w] = s_m[w][hd];
      m = fmaxf(m, mw[w]);
    }
    float l = 0.f, le = 0.f;
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      f[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - m);
      l += s_l[w][hd] * f[w];
      le += s_e[w][hd] * f[w];
    }
    const int r = hd & 3;
    for (int col = lane; col < ncol; col += 64) {
      const int ln = (col & 15) + 16 * (hd >> 2);
      float sum = 0.f;
      if (RAW) {
        const int o = ((col >> 4) * 64 + ln) * 4 + r;     // limb 0; limb 1 is 32 lanes on
#pragma unroll
        for (int w = 0; w < CW; ++w) {
          const int* mw_ = reinterpret_cast<const int*>(ring + w * a.wave_bytes);
          sum += fmaf(128.f, static_cast<float>(mw_[o]), static_cast<float>(mw_[o + 128])) * f[w];
        }
      } else {
        const int o = ((col >> 4) * 32 + ln) * 4 + r;
#pragma unroll
        for (int w = 0; w < CW; ++w) sum += reinterpret_cast<const float*>(ring + w * a.wave_bytes)[o] * f[w];
      }
      rec[PHDR + col] = sum;
    }
    if (lane == 0) {
      rec[0] = good ? m : NAN;
      rec[1] = l;
      rec[2] = le;
      rec[3] = 0.f;
    }
  }
}

// Merge of the S partial records of one (batch, KV head, q head); out and lse.
constexpr int CNT = 1024;                // combine threads
constexpr int SPC = 64;                  // splits per pass (one header per lane)
constexpr int KPC = 4;                   // 16-byte pieces per loader and pass (a pass covers
                                         // min(SPC, KPC * CNT / P) splits of P-piece records)
constexpr int MAXCOL = 16 * 24;          // field columns of a record, at most

struct CombArgs {
  const float* part;
  const float* offs;
  int n_kv, n_q, group, S, prec;
  const int32_t* seq_lens;
  int seq_per_head;                      // seq_lens is [batch][n_kv] (else [batch])
  int64_t max_seq;
  float* out;
  float* lse;
  int lm;                                // records of the level pass: one column per channel
};

#ifdef AATC_ATTN_COMBINE_TU   // defined by the one translation unit that launches it
// Every input of the merge is read with ordinary loads issued at once at kernel entry (records,
// V tables, R_V), so the kernel pays about one memory round trip before its arithmetic.
__global__ __launch_bounds__(CNT) void k_attn_combine(CombArgs a, const aatc_calib* __restrict__ vcal) {
  __shared__ float4 part[CNT];            // [split group q][piece p] partial sums, q * P + p
  __shared__ float csum[MAXCOL];
  __shared__ float t_o[D], t_delta[D];
  __shared__ int t_bits[D];
  __shared__ int16_t t_cf[3 * D];
  __shared__ uint8_t t_fs[AATC_MAX_FIELDS];
  __shared__ float yt[D], res[D];
  __shared__ float part8[8][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group, S = a.S, prec = a.prec;
  const int bh = b * a.n_kv + h;
  const aatc_calib* vc = vcal + h;
  const float* rec0 = a.part + (static_cast<int64_t>(bh) * S * G + g) * prec;
  const int64_t stride = static_cast<int64_t>(G) * prec;
  // a record is P 16-byte pieces (its header first); thread t < Q P sums piece t % P of the
  // splits t / P + k Q of each pass, one 16-byte load per split
  const int P = prec >> 2, Q = CNT / P;
  const int pp = tid % P, qq = tid / P;
  const bool loader = qq < Q;
  const int SPP = Q * KPC < SPC ? Q * KPC : SPC;   // splits per pass

  // the first pass's records (every lane a header, every loader its pieces) before anything
  // that depends on a load: these are the long pole
  float4 hd = make_float4(-INFINITY, 0.f, 0.f, 0.f);
  float4 xv[KPC];
  auto load_pass = [&](int s0) {
    const int n = S - s0 < SPP ? S - s0 : SPP;
    // unconditional loads from clamped (always valid) addresses, masked afterwards: a load under
    // a branch makes the compiler wait for every load before it at the join
    const bool hv = lane < n;
    hd = *reinterpret_cast<const float4*>(rec0 + (s0 + (hv ? lane : 0)) * stride);
#pragma unroll
    for (int k = 0; k < KPC; ++k) {
      const int sp = qq + Q * k;
      const bool sv = loader && sp < n;
      xv[k] = *reinterpret_cast<const float4*>(rec0 + (s0 + (sv ? sp : 0)) * stride + 4 * (sv ? pp : 0));
    }
    if (!hv) hd = make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < KPC; ++k)
      if (!(loader && qq + Q * k < n)) xv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  };
  load_pass(0);
  // tables and R_V, consumed last
  const int ti = tid & (D - 1), tf = tid < 3 * D ? tid : 0;   // clamped table indexes
  const float r_o = vc->o32[ti], r_d = a.lm ? vc->scale32[ti] : vc->delta32[ti];
  const int r_b = vc->bits[ti], r_cf = vc->channel_field[tf], r_fs = vc->field_shift[tf];
  // NOVA: R_V^T is E^-1, applied by the same GEMV as a KLT blob's R^T
  const int rot = vc->rotation == AATC_ROT_NOVA ? AATC_ROT_KLT : vc->rotation;
  float rv[16];
  if (rot == AATC_ROT_KLT) {
    const int j = tid & (D - 1), e8 = tid >> 7;
#pragma unroll
    for (int k = 0; k < 16; ++k) rv[k] = vc->R32[(16 * e8 + k) * D + j];
  }
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[a.seq_per_head ? bh : b]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);
  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4;
  const int ncol_blob = a.lm ? D : 16 * (T4 + T2 + ((n1 + 15) >> 4));
  bool bad = PHDR + ncol_blob > prec || ncol_blob > MAXCOL || n4 < 0 || n2 < 0 || n1 < 0;
  const int ncol = bad ? 0 : ncol_blob;

  // L sums the rounded probabilities that weighted the code sums (it normalises the output);
  // LE the unrounded ones (the lse: rounding each token to 14 bits would bias it low).  Every
  // wave reduces the pass's headers itself (lane s holds split s0 + s), so the passes need no
  // barrier; a loader takes its splits' factors from the lanes that hold them.
  float M = -INFINITY, L = 0.f, LE = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += SPP) {
    if (s0 > 0) load_pass(s0);
    const float hm = hd.x;
    bad |= __ballot(hm != hm) != 0;
    const float m = wave_max_x(hm);
    const float nM = fmaxf(M, m);
    const float w = (hm == -INFINITY || nM == -INFINITY) ? 0.f : exp2f(hm - nM);
    const float l = wave_sum_x(w * hd.y), le = wave_sum_x(w * hd.z);
    const float fold = (M == -INFINITY) ? 0.f : exp2f(M - nM);
    L = L * fold + l;
    LE = LE * fold + le;
    M = nM;
    float4 pv = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < KPC; ++k) {
      const int src = (qq + Q * k) & (SPC - 1);
      const float wk = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(w)));
      pv.x = fmaf(wk, xv[k].x, pv.x);
      pv.y = fmaf(wk, xv[k].y, pv.y);
      pv.z = fmaf(wk, xv[k].z, pv.z);
      pv.w = fmaf(wk, xv[k].w, pv.w);
    }
    acc.x = fmaf(acc.x, fold, pv.x);
    acc.y = fmaf(acc.y, fold, pv.y);
    acc.z = fmaf(acc.z, fold, pv.z);
    acc.w = fmaf(acc.w, fold, pv.w);
  }
  // split groups -> column sums; tables -> LDS
  if (loader) part[qq * P + pp] = acc;
  if (tid < D) {
    t_o[tid] = r_o;
    t_delta[tid] = r_d;
    t_bits[tid] = r_b;
  }
  if (tid < 3 * D) t_cf[tid] = static_cast<int16_t>(r_cf);
  if (tid < AATC_MAX_FIELDS) t_fs[tid] = static_cast<uint8_t>(r_fs);
  __syncthreads();
  if (tid < ncol) {
    // column tid is component (tid + PHDR) % 4 of piece (tid + PHDR) / 4
    const float* pf = reinterpret_cast<const float*>(part) + 4 * ((tid + PHDR) >> 2) + ((tid + PHDR) & 3);
    float cs = 0.f;
    for (int q = 0; q < Q; ++q) cs += pf[4 * P * q];
    csum[tid] = cs;
  }
  __syncthreads();
  // fold field columns into channel code sums; y = o + delta (c_bar - 2^(b-1) + 1/2); records
  // of the level pass hold each channel's weighted level sum: y = o + scale l_bar
  if (tid < D && a.lm) {
    const int i = tid;
    yt[i] = (t_bits[i] && L > 0.f && i < ncol) ? t_o[i] + t_delta[i] * (csum[i] / L) : t_o[i];
  } else if (tid < D) {
    const int i = tid;
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
  if (rot == AATC_ROT_WHT) {
    if (wave == 0) {
      float x0 = yt[lane], x1 = yt[64 + lane];
      fwht128(x0, x1, lane);
      res[lane] = x0 * 0.08838834764831845f;
      res[64 + lane] = x1 * 0.08838834764831845f;
    }
  } else if (rot == AATC_ROT_KLT) {
    // out_j = sum_i R[i][j] y_i: eight threads per output, 16 rows each
    const int j = tid & (D - 1), e8 = tid >> 7;
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) o = fmaf(rv[k], yt[16 * e8 + k], o);
    part8[e8][j] = o;
    __syncthreads();
    if (tid < D)
      res[tid] = ((part8[0][tid] + part8[1][tid]) + (part8[2][tid] + part8[3][tid])) +
                 ((part8[4][tid] + part8[5][tid]) + (part8[6][tid] + part8[7][tid]));
  } else if (tid < D) {
    res[tid] = yt[tid];
  }
  __syncthreads();
  const int64_t qh = static_cast<int64_t>(b) * a.n_q + h * G + g;
  const bool empty = seq == 0;
  if (tid < D) a.out[qh * D + tid] = bad ? NAN : (L > 0.f ? res[tid] : (empty ? 0.f : NAN));
  if (a.lse && tid == 0) {
    const float l2 = bad ? NAN : (L > 0.f ? M + log2f(LE / static_cast<float>(PS)) + a.offs[bh * 8 + g]
                                          : (empty ? -INFINITY : NAN));
    a.lse[qh] = l2 * 0.69314718055994530942f;
  }
}
#endif

template <int NP, bool HALF, int NVB, int LIMBS, int NPROD, int TGM>
hipError_t launch_one(const AttnArgs& a, const aatc_calib* kcal, const aatc_calib* vcal, dim3 grid, size_t lds,
                      hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_attn_main<NP, HALF, NVB, LIMBS, NPROD, TGM>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn_main<NP, HALF, NVB, LIMBS, NPROD, TGM>), grid, dim3((CW + NPROD) * 64), lds, st, a,
                     kcal, vcal);
  return hipGetLastError();
}

// The producer form runs 12 waves, 3 per SIMD, so only the smallest V bucket with at most two
// bit-plane pairs fits its registers; it is planned only when every tile has a slot, so it
// always scores groups of up to TG tiles.  The ring form (tg = 1; not for the widest V bucket,
// whose registers it would spill) scores one tile per group and keeps one probability row block
// per wave, leaving the LDS to the ring.
template <int NP, bool HALF, int NVB>
hipError_t launch_limbs(int limbs, int tg, const AttnArgs& a, const aatc_calib* kcal, const aatc_calib* vcal,
                        dim3 grid, size_t lds, hipStream_t st) {
  if constexpr (NVB == 12 && NP <= 2) {
    if (a.prod)
      return limbs == 3 ? launch_one<NP, HALF, NVB, 3, NPROD_MAX, TG>(a, kcal, vcal, grid, lds, st)
                        : launch_one<NP, HALF, NVB, 2, NPROD_MAX, TG>(a, kcal, vcal, grid, lds, st);
  }
  if constexpr (NVB != 24) {
    if (tg == 1)
      return limbs == 3 ? launch_one<NP, HALF, NVB, 3, 0, 1>(a, kcal, vcal, grid, lds, st)
                        : launch_one<NP, HALF, NVB, 2, 0, 1>(a, kcal, vcal, grid, lds, st);
  }
  return limbs == 3 ? launch_one<NP, HALF, NVB, 3, 0, TG>(a, kcal, vcal, grid, lds, st)
                    : launch_one<NP, HALF, NVB, 2, 0, TG>(a, kcal, vcal, grid, lds, st);
}

template <int NP, bool HALF>
hipError_t launch_nvb(int nvb, int limbs, int tg, const AttnArgs& a, const aatc_calib* kcal, const aatc_calib* vcal,
                      dim3 grid, size_t lds, hipStream_t st, bool* found) {
  *found = true;
  switch (nvb) {
    case 12: return launch_limbs<NP, HALF, 12>(limbs, tg, a, kcal, vcal, grid, lds, st);
    case 16: return launch_limbs<NP, HALF, 16>(limbs, tg, a, kcal, vcal, grid, lds, st);
    case 24: return launch_limbs<NP, HALF, 24>(limbs, tg, a, kcal, vcal, grid, lds, st);
  }
  *found = false;
  return hipSuccess;
}

// One translation unit per NP instantiates this (both pair kinds, all V buckets, limb modes and
// group sizes).
template <int NP>
hipError_t launch_np(int half, int nvb, int limbs, int tg, const AttnArgs& a, const aatc_calib* kcal,
                     const aatc_calib* vcal, dim3 grid, size_t lds, hipStream_t st, bool* found) {
  return half ? launch_nvb<NP, true>(nvb, limbs, tg, a, kcal, vcal, grid, lds, st, found)
              : launch_nvb<NP, false>(nvb, limbs, tg, a, kcal, vcal, grid, lds, st, found);
}

#define AATC_LAUNCH_NP_SIG(N)                                                                     \
  hipError_t launch_np<N>(int, int, int, int, const AttnArgs&, const aatc_calib*, const aatc_calib*, dim3, \
                          size_t, hipStream_t, bool*)
extern template AATC_LAUNCH_NP_SIG(1);
extern template AATC_LAUNCH_NP_SIG(2);
extern template AATC_LAUNCH_NP_SIG(3);
extern template AATC_LAUNCH_NP_SIG(4);

}  // namespace aatc_attn
