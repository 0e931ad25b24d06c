// Decode attention on the packed cache: host-side plan, validation and launch.
// The kernel (and the method it implements) is described in aatc_attn_kernel.h.
#define AATC_ATTN_COMBINE_TU
#include "aatc_attn_kernel.h"
#include "aatc_attn_lm.h"
#include "aatc_dense_kernel.h"
#include "aatc_seg_kernel.h"

#include <cstdio>
#include <mutex>

// Workspace of aatc_decode_attn_noalloc: a fixed array in device memory, one copy per GPU the
// library runs on, kept until the process ends.  Host code never passes its name to a kernel
// (on the host it is only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns, once per device.
static __device__ __align__(256) unsigned char scratch[AATC_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace aatc_attn;

constexpr size_t kLdsLimit = 160 * 1024;
constexpr size_t kLmStaticLds = 16 * 1024;  // k_attn_lm's static LDS (tables, q, merge headers), rounded up
// __shared__ arrays of the kernel: the probability rows of tg tiles per wave plus scalars
// (rounded up)
constexpr size_t static_lds(int tg) { return static_cast<size_t>(CW) * tg * PROW_BYTES + 2048; }

int vtiles_bucket(int vt) {
  if (vt <= 12) return 12;
  if (vt <= 16) return 16;
  if (vt <= 24) return 24;
  return -1;
}

struct Plan {
  bool lm;                               // the level pass (k_attn_lm): a Lloyd-Max tensor
  int NP, NVB, LIMBS, S, tpw, half, prec, prod, tg;
  int nslot, slot_bytes, ksz, gs, wave_bytes;
  size_t lds;
  size_t part_bytes, offs_bytes;
  size_t q_bytes;                        // fp32 copy of a bf16 q (batch x n_q x 128 floats)
  bool fits;
};

int round16(int64_t x) { return static_cast<int>((x + 15) / 16 * 16); }

// Tiles per wave fill 256 CUs x CW waves once; each wave gets a ring of LDS slots (one tile
// each), as many as fit, at most its tile count.
Plan make_plan(const aatc_cache* c, int n_q, int64_t max_seq) {
  Plan p;
  p.q_bytes = 0;
  // the level pass: a Lloyd-Max tensor, or more bits per vector than k_attn_main reads
  p.lm = c->quantizer != 0 || c->k_bits > AATC_MAX_ATTN_BITS || c->v_bits > AATC_MAX_ATTN_BITS;
  if (p.lm) {
    // the level pass: about one workgroup (eight waves) per CU, each a contiguous range of
    // tiles of one sequence (tpw: tiles per workgroup)
    const int group = c->n_kv_heads > 0 ? n_q / c->n_kv_heads : 1;
    const int64_t ntiles = (max_seq + 63) / 64;
    const int64_t seqs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
    int64_t S = (256 + seqs - 1) / seqs;
    if (S > ntiles) S = ntiles;
    if (S < 1) S = 1;
    int64_t tpw = (ntiles + S - 1) / S;
    if (tpw < 1) tpw = 1;
    p.tpw = static_cast<int>(tpw);
    S = (ntiles + tpw - 1) / tpw;
    p.S = static_cast<int>(S < 1 ? 1 : S);
    p.prec = aatc_lm::PHDR + AATC_D;
    p.NP = p.NVB = p.LIMBS = p.half = p.prod = p.tg = 0;
    p.nslot = p.slot_bytes = p.ksz = p.gs = p.wave_bytes = 0;
    p.nslot = aatc_lm::dyn_lds(c->k_bits, c->v_bits, 2) + kLmStaticLds <= kLdsLimit ? 2 : 1;
    p.lds = aatc_lm::dyn_lds(c->k_bits, c->v_bits, p.nslot);
    p.fits = p.lds + kLmStaticLds <= kLdsLimit;
    p.part_bytes = static_cast<size_t>(seqs) * p.S * group * p.prec * 4;
    p.offs_bytes = static_cast<size_t>(seqs) * 8 * 4;
    return p;
  }
  const int kb = c->k_bits, vb = c->v_bits;
  p.NP = kb > 0 ? (kb + 127) / 128 : 1;
  p.half = (kb > 0 && kb - 128 * (p.NP - 1) <= 64) ? 1 : 0;
  p.NVB = vtiles_bucket(c->v_tiles);
  const int group = c->n_kv_heads > 0 ? n_q / c->n_kv_heads : 1;
  p.LIMBS = group <= 4 ? 3 : 2;
  p.prec = PHDR + 16 * (c->v_tiles > 0 ? c->v_tiles : 1);
  const int64_t ntiles = (max_seq + 63) / 64;
  const int64_t seqs = static_cast<int64_t>(c->batch) * c->n_kv_heads;
  const int64_t target_waves = 256 * static_cast<int64_t>(CW);
  int64_t tpw = (ntiles * seqs + target_waves - 1) / target_waves;
  if (tpw < 1) tpw = 1;
  // at most 64 tiles per wave (more workgroups instead): keeps a wave's integer code sums and
  // their limb combination (128 * high + low) inside int32
  if (tpw > 64) tpw = 64;
  p.tpw = static_cast<int>(tpw);
  int64_t S = (ntiles + CW * tpw - 1) / (CW * tpw);
  if (S < 1) S = 1;
  p.S = static_cast<int>(S);
  // slot: K bytes of a tile (plus up to 15 bytes of alignment), then V
  p.ksz = kb > 0 ? round16(8LL * kb + 16) : 0;
  const int vsz = vb > 0 ? round16(8LL * vb + 16) : 0;
  p.slot_bytes = p.ksz + vsz > 0 ? p.ksz + vsz : 16;
  // one score group per wave when its tiles all fit (no running-max rescale at all); otherwise
  // the ring form: one tile per group, with probability rows for one tile per wave, so that
  // the LDS they free holds more slots and the next tiles' copies fly meanwhile
  auto slots = [&](int tg) {
    const size_t avail = kLdsLimit - static_lds(tg) - FIXED_LDS - DMA_PAD;
    return static_cast<int>(avail / (static_cast<size_t>(CW) * p.slot_bytes));
  };
  int ns = slots(TG);
  if (ns >= p.tpw) {
    p.tg = TG;
    ns = p.tpw;
    p.gs = p.tpw < TG ? p.tpw : TG;
  } else if (p.NVB == 24) {
    // the widest V bucket keeps groups of half the slots (its one-tile form spills registers)
    p.tg = TG;
    p.gs = ns / 2 < TG ? ns / 2 : TG;
    if (p.gs < 1) p.gs = 1;
  } else {
    p.tg = 1;
    ns = slots(1);
    if (ns > p.tpw) ns = p.tpw;
    p.gs = 1;
  }
  p.nslot = ns;
  p.fits = ns >= 1;
  // a wave's ring area holds its slots, and at the end its merge values
  p.wave_bytes = (ns > 0 ? ns : 1) * p.slot_bytes;
  if (p.wave_bytes < p.NVB * merge_group_bytes(p.NVB)) p.wave_bytes = p.NVB * merge_group_bytes(p.NVB);
  const size_t ring = static_cast<size_t>(CW) * p.wave_bytes + DMA_PAD;
  p.lds = FIXED_LDS + ring;
  if (p.lds + static_lds(p.tg) > kLdsLimit) p.fits = false;
  // copy waves issue every tile when all of a wave's tiles have slots and the copy count of one
  // copy wave stays within what one wait can count
  {
    const int ik = kb > 0 ? (static_cast<int>((15 + 8LL * kb + 15) / 16) + 63) / 64 : 0;
    const int iv = vb > 0 ? (static_cast<int>((15 + 8LL * vb + 15) / 16) + 63) / 64 : 0;
    p.prod = (p.NVB == 12 && p.NP <= 2 && p.tg == TG && ns >= p.tpw && (CW / NPROD_MAX) * p.tpw * (ik + iv) <= 60) ? NPROD_MAX : 0;
  }
  p.part_bytes = static_cast<size_t>(seqs) * p.S * group * p.prec * 4;
  p.offs_bytes = static_cast<size_t>(seqs) * 8 * 4;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool dispatch(const Plan& p, const AttnArgs& a, const aatc_calib* kc, const aatc_calib* vc, dim3 grid, hipStream_t st,
              hipError_t* err) {
  bool found = false;
  switch (p.NP) {
    case 1: *err = launch_np<1>(p.half, p.NVB, p.LIMBS, p.tg, a, kc, vc, grid, p.lds, st, &found); break;
    case 2: *err = launch_np<2>(p.half, p.NVB, p.LIMBS, p.tg, a, kc, vc, grid, p.lds, st, &found); break;
    case 3: *err = launch_np<3>(p.half, p.NVB, p.LIMBS, p.tg, a, kc, vc, grid, p.lds, st, &found); break;
    case 4: *err = launch_np<4>(p.half, p.NVB, p.LIMBS, p.tg, a, kc, vc, grid, p.lds, st, &found); break;
  }
  return found;
}

}  // namespace

extern "C" {

size_t aatc_decode_attn_workspace_bytes(const aatc_cache* c, int32_t n_q_heads, int64_t max_seq_len) {
  if (!c || max_seq_len < 0 || n_q_heads < 1) return 0;
  const Plan p = make_plan(c, n_q_heads, max_seq_len);
  // partial records, lse offsets, and room for an fp32 copy of a bf16 q
  return align256(p.part_bytes) + align256(p.offs_bytes) +
         align256(static_cast<size_t>(c->batch > 0 ? c->batch : 0) * n_q_heads * AATC_D * 4);
}

}  // extern "C"

namespace {

// Shared argument checks and plan of the decode-attention entry points (all but the workspace).
aatc_status check_cache_and_plan(const aatc_cache* c, int32_t n_q, int64_t max_seq, Plan* p) {
  if (!c) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (c->d != AATC_D) return aatc::fail(AATC_ERR_UNSUPPORTED, "d=%d (only 128)", c->d);
  if (c->batch < 1 || c->n_kv_heads < 1 || n_q < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "shape");
  if (n_q % c->n_kv_heads) return aatc::fail(AATC_ERR_UNSUPPORTED, "n_q_heads %% n_kv_heads != 0");
  const int group = n_q / c->n_kv_heads;
  if (group > AATC_MAX_GROUP) return aatc::fail(AATC_ERR_UNSUPPORTED, "GQA group %d > 8", group);
  if (c->k_bits < 0 || c->k_bits > 8 * AATC_D || c->v_bits < 0 || c->v_bits > 8 * AATC_D)
    return aatc::fail(AATC_ERR_BUDGET, "k_bits %d / v_bits %d outside 0..%d", c->k_bits, c->v_bits, 8 * AATC_D);
  if (c->quantizer < 0 || c->quantizer > 3) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "quantizer %d", c->quantizer);
  const bool summed = c->quantizer == 0 && c->k_bits <= AATC_MAX_ATTN_BITS && c->v_bits <= AATC_MAX_ATTN_BITS;
  if (c->v_tiles < 0 || (summed && vtiles_bucket(c->v_tiles) < 0))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "v_tiles %d", c->v_tiles);
  if (!c->k_calib || !c->v_calib || (!c->k_codes && c->k_bits > 0) || (!c->v_codes && c->v_bits > 0))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null cache pointer");
  if ((reinterpret_cast<uintptr_t>(c->k_codes) & 15) || (reinterpret_cast<uintptr_t>(c->v_codes) & 15))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "codes must be 16-byte aligned");
  if (max_seq < 0 || max_seq > c->capacity_tokens)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "max_seq_len %lld > capacity", (long long)max_seq);
  *p = make_plan(c, n_q, max_seq);
  p->q_bytes = static_cast<size_t>(c->batch) * n_q * AATC_D * 4;
  if (!p->fits) return aatc::fail(AATC_ERR_UNSUPPORTED, "tiles of %d+%d bits do not fit LDS", c->k_bits, c->v_bits);
  return AATC_OK;
}

size_t plan_workspace(const Plan& p) { return align256(p.part_bytes) + align256(p.offs_bytes) + align256(p.q_bytes); }

// q as the kernels take it (fp32): the caller's buffer, or for bf16 an fp32 copy in the
// workspace's last area (one small conversion kernel on the stream).
__global__ void k_q_bf16_to_f32(const uint16_t* __restrict__ in, float* __restrict__ out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = __uint_as_float(static_cast<uint32_t>(in[i]) << 16);
}

aatc_status prepare_q(const void* q, aatc_dtype qdt, const Plan& p, void* ws, hipStream_t st, const float** q32) {
  if (qdt == AATC_F32) {
    *q32 = static_cast<const float*>(q);
    return AATC_OK;
  }
  if (qdt != AATC_BF16) return aatc::fail(AATC_ERR_UNSUPPORTED, "q dtype %d (fp32 or bf16)", static_cast<int>(qdt));
  float* dst = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(p.part_bytes) + align256(p.offs_bytes));
  const int64_t n = static_cast<int64_t>(p.q_bytes / 4);
  hipLaunchKernelGGL(k_q_bf16_to_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), dst, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "q conversion launch: %s", hipGetErrorString(e));
  *q32 = dst;
  return AATC_OK;
}

aatc_status check_and_plan(const aatc_cache* c, int32_t n_q, int64_t max_seq, void* ws, size_t ws_bytes, Plan* p) {
  if (!ws) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const aatc_status r = check_cache_and_plan(c, n_q, max_seq, p);
  if (r != AATC_OK) return r;
  const size_t need = plan_workspace(*p);
  if (ws_bytes < need) return aatc::fail(AATC_ERR_BUFFER_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
  return AATC_OK;
}

aatc_status launch_level_pass(const aatc_cache* c, const Plan& p, const float* q, int32_t n_q,
                              const int32_t* seq_lens, int seq_per_head, int64_t max_seq, float scale, void* ws,
                              hipStream_t st) {
  aatc_lm::LmArgs a;
  a.kcodes = static_cast<const uint32_t*>(c->k_codes);
  a.vcodes = static_cast<const uint32_t*>(c->v_codes);
  a.tiles_per_seq = c->capacity_tokens / 64;
  a.n_kv = c->n_kv_heads;
  a.n_q = n_q;
  a.group = n_q / c->n_kv_heads;
  a.seq_lens = seq_lens;
  a.seq_per_head = seq_per_head;
  a.max_seq = max_seq;
  a.q = q;
  a.scale2 = (scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(AATC_D))) * 1.4426950408889634f;
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<float*>(w);
  a.offs = reinterpret_cast<float*>(w + align256(p.part_bytes));
  a.S = p.S;
  a.tpw = p.tpw;
  a.prec = p.prec;
  a.kB = c->k_bits;
  a.vB = c->v_bits;
  a.quant = c->quantizer;
  a.nslot = p.nslot;
  const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&aatc_lm::k_attn_lm),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(p.lds));
  if (ea != hipSuccess) return aatc::fail(AATC_ERR_HIP, "level pass LDS attribute: %s", hipGetErrorString(ea));
  hipLaunchKernelGGL(aatc_lm::k_attn_lm, dim3(p.S, c->n_kv_heads, c->batch), dim3(aatc_lm::THREADS), p.lds, st, a,
                     static_cast<const aatc_calib*>(c->k_calib), static_cast<const aatc_calib*>(c->v_calib));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "decode_attn level pass launch: %s", hipGetErrorString(err));
  return AATC_OK;
}

aatc_status launch_partial(const aatc_cache* c, const Plan& p, const float* q, int32_t n_q, const int32_t* seq_lens,
                           int seq_per_head, int64_t max_seq, float scale, void* ws, hipStream_t st) {
  if (p.lm) return launch_level_pass(c, p, q, n_q, seq_lens, seq_per_head, max_seq, scale, ws, st);
  AttnArgs a;
  const aatc_calib* kcal = static_cast<const aatc_calib*>(c->k_calib);
  const aatc_calib* vcal = static_cast<const aatc_calib*>(c->v_calib);
  a.kcodes = static_cast<const uint32_t*>(c->k_codes);
  a.vcodes = static_cast<const uint32_t*>(c->v_codes);
  a.tiles_per_seq = c->capacity_tokens / 64;
  a.n_kv = c->n_kv_heads;
  a.n_q = n_q;
  a.group = n_q / c->n_kv_heads;
  a.seq_lens = seq_lens;
  a.seq_per_head = seq_per_head;
  a.max_seq = max_seq;
  a.q = q;
  a.scale2 = (scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(AATC_D))) * 1.4426950408889634f;
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<float*>(w);
  a.offs = reinterpret_cast<float*>(w + align256(p.part_bytes));
  a.S = p.S;
  a.tpw = p.tpw;
  a.prec = p.prec;
  a.kB = c->k_bits;
  a.vB = c->v_bits;
  a.nslot = p.nslot;
  a.slot_bytes = p.slot_bytes;
  a.wave_bytes = p.wave_bytes;
  a.ksz = p.ksz;
  a.gs = p.gs;
  a.prod = p.prod;
  // K tiles of whole 16-byte units per token (U = B_K / 128 of them): swizzled in LDS (see
  // dma_bytes) with the mask that spreads one score read over 16 bank groups for that U
  const int ku = (!p.half && c->k_bits % 128 == 0) ? c->k_bits / 128 : 0;
  a.kswz = ku == 1 || ku == 3 ? 3 : ku == 2 ? 7 : ku == 4 ? 15 : 0;
  const dim3 grid(p.S, c->n_kv_heads, c->batch);
  hipError_t err = hipSuccess;
  const bool ok = dispatch(p, a, kcal, vcal, grid, st, &err);
  if (!ok) return aatc::fail(AATC_ERR_UNSUPPORTED, "plan NP=%d NVB=%d", p.NP, p.NVB);
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "decode_attn launch: %s", hipGetErrorString(err));
  return AATC_OK;
}

// Merge for launches with few splits per sequence (batch decoding, where the grid has one
// workgroup per sequence and KV head or a few): one workgroup of 256 threads per (batch, KV head)
// merges the records of all its q heads, so the KLT or NOVA R_V is read once for all of them
// (the per-q-head merge reads it once per q head: 64 KB each) and the grid launches a sixteenth
// of the waves.  Inputs, outputs and arithmetic as k_attn_combine; wave w takes q heads w, w + 4.
constexpr int CH_THREADS = 256;
constexpr int CH_MAXS = 8;                 // splits per sequence this form takes
constexpr int CH_COLS = MAXCOL / 64;       // column sums per lane, at most

__global__ __launch_bounds__(CH_THREADS) void k_attn_combine_heads(CombArgs a, const aatc_calib* __restrict__ vcal) {
  __shared__ float csum[4][MAXCOL];        // per wave: column sums of its q head
  __shared__ float yt[8][D];               // per q head: the rotated-domain output
  __shared__ float part2[2][8][D];         // KLT: the two half sums of every output
  __shared__ float hml[8][4];              // per q head: M, L, LE, bad
  __shared__ float t_o[D], t_d[D];
  __shared__ int t_bits[D];
  __shared__ int16_t t_cf[3 * D];
  __shared__ uint8_t t_fs[AATC_MAX_FIELDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.group, S = a.S, prec = a.prec;
  const int bh = b * a.n_kv + h;
  const aatc_calib* vc = vcal + h;
  const int64_t stride = static_cast<int64_t>(G) * prec;      // split s of q head g at s * stride
  // ---- every load that does not depend on another, at once: one memory round trip
  // this wave's first q head's records (lane s < S a header, every lane its columns of every
  // split, from clamped addresses)
  float4 hd0;
  float x[CH_COLS][CH_MAXS];
  auto load_head = [&](int g) {
    const float* rec0 = a.part + (static_cast<int64_t>(bh) * S * G + g) * prec;
    hd0 = *reinterpret_cast<const float4*>(rec0 + (lane < S ? lane : 0) * stride);
#pragma unroll
    for (int k = 0; k < CH_COLS; ++k)
#pragma unroll
      for (int sp = 0; sp < CH_MAXS; ++sp) {
        const int col = lane + 64 * k;     // clamped to the record's end below
        x[k][sp] = rec0[(sp < S ? sp : 0) * stride + PHDR + (PHDR + col < prec ? col : 0)];
      }
  };
  if (wave < G) load_head(wave);
  // tables, and for a KLT or NOVA blob this thread's 64 rows of R_V column j
  const int ti = tid & (D - 1);
  const float r_o = vc->o32[ti], r_d = a.lm ? vc->scale32[ti] : vc->delta32[ti];
  const int r_b = vc->bits[ti];
  const int c0 = vc->channel_field[tid], c1 = vc->channel_field[tid < D ? 2 * D + tid : 0];
  const int f0 = vc->field_shift[tid], f1 = vc->field_shift[tid < D ? 2 * D + tid : 0];
  const int rot = vc->rotation == AATC_ROT_NOVA ? AATC_ROT_KLT : vc->rotation;
  const int j = tid & (D - 1), hf = tid >> 7;
  float rv[64];
  if (rot == AATC_ROT_KLT) {
    const float* rcol = vc->R32 + (64 * hf) * D + j;
#pragma unroll
    for (int i = 0; i < 64; ++i) rv[i] = rcol[i * D];
  }
  const int n4 = vc->n_fields4, n2 = vc->n_fields2, n1 = vc->n_fields1;
  const int T4 = (n4 + 15) >> 4, T2 = (n2 + 15) >> 4;
  const int ncol_blob = a.lm ? D : 16 * (T4 + T2 + ((n1 + 15) >> 4));
  const bool bad0 = PHDR + ncol_blob > prec || ncol_blob > MAXCOL || n4 < 0 || n2 < 0 || n1 < 0;
  const int ncol = bad0 ? 0 : ncol_blob;
  int64_t seq = a.seq_lens ? static_cast<int64_t>(a.seq_lens[a.seq_per_head ? bh : b]) : a.max_seq;
  seq = seq < 0 ? 0 : (seq > a.max_seq ? a.max_seq : seq);
  if (tid < D) {
    t_o[tid] = r_o;
    t_d[tid] = r_d;
    t_bits[tid] = r_b;
    t_cf[2 * D + tid] = static_cast<int16_t>(c1);
    t_fs[2 * D + tid] = static_cast<uint8_t>(f1);
  }
  t_cf[tid] = static_cast<int16_t>(c0);
  t_fs[tid] = static_cast<uint8_t>(f0);
  __syncthreads();

  for (int g = wave; g < G; g += 4) {
    if (g != wave) load_head(g);
    const float4 hd = lane < S ? hd0 : make_float4(-INFINITY, 0.f, 0.f, 0.f);
    const bool bad = bad0 || __ballot(hd.x != hd.x) != 0;
    const float M = wave_max_x(hd.x);
    const float w = (hd.x == -INFINITY || M == -INFINITY) ? 0.f : exp2f(hd.x - M);
    const float L = wave_sum_x(w * hd.y), LE = wave_sum_x(w * hd.z);
#pragma unroll
    for (int k = 0; k < CH_COLS; ++k) {
      const int col = lane + 64 * k;
      float cs = 0.f;
#pragma unroll
      for (int sp = 0; sp < CH_MAXS; ++sp) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp));   // 0 past S
        cs = fmaf(ws, x[k][sp], cs);
      }
      if (col < ncol) csum[wave][col] = cs;
    }
    wave_sync_lds();
    // fold field columns into channel code sums and dequantize (channels lane, 64 + lane)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      const int bi = t_bits[i];
      const float o = t_o[i];
      float y = o;
      if (a.lm) {
        if (bi && L > 0.f && i < ncol) y = o + t_d[i] * (csum[wave][i] / L);
      } else {
        float cs = 0.f;
        for (int kk = 0; kk < 3; ++kk) {
          const int f = t_cf[3 * i + kk];
          if (f < 0 || f >= AATC_MAX_FIELDS) break;
          int col;
          if (f < n4) col = f;
          else if (f < n4 + n2) col = 16 * T4 + (f - n4);
          else col = 16 * (T4 + T2) + (f - n4 - n2);
          if (col < ncol) cs += ldexpf(csum[wave][col], t_fs[f]);
        }
        if (bi && L > 0.f) y = o + t_d[i] * (cs / L - (static_cast<float>(1 << (bi - 1)) - 0.5f));
      }
      yt[g][i] = y;
    }
    if (lane == 0) {
      hml[g][0] = M;
      hml[g][1] = L;
      hml[g][2] = LE;
      hml[g][3] = bad ? 1.f : 0.f;
    }
    wave_sync_lds();                       // csum is this wave's again for its next q head
  }
  __syncthreads();
  // R_V^T for every q head: an FWHT per q head (wave w: q heads w, w + 4), or the GEMV with the
  // rows held in registers: thread (output j, half of the rows) sums every q head
  if (rot == AATC_ROT_WHT) {
    for (int g = wave; g < G; g += 4) {
      float x0 = yt[g][lane], x1 = yt[g][64 + lane];
      fwht128(x0, x1, lane);
      part2[0][g][lane] = x0 * 0.08838834764831845f;
      part2[0][g][64 + lane] = x1 * 0.08838834764831845f;
    }
  } else if (rot == AATC_ROT_KLT) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 64; ++i) acc = fmaf(rv[i], yt[g][64 * hf + i], acc);
        part2[hf][g][j] = acc;
      }
    }
  } else {
    for (int e = tid; e < G * D; e += CH_THREADS) part2[0][e / D][e % D] = yt[e / D][e % D];
  }
  __syncthreads();
  const bool empty = seq == 0;
  for (int e = tid; e < G * D; e += CH_THREADS) {
    const int g = e / D, jj = e % D;
    const float res = rot == AATC_ROT_KLT ? part2[0][g][jj] + part2[1][g][jj] : part2[0][g][jj];
    const float L = hml[g][1];
    const bool bad = hml[g][3] != 0.f;
    const int64_t qh = static_cast<int64_t>(b) * a.n_q + h * G + g;
    a.out[qh * D + jj] = bad ? NAN : (L > 0.f ? res : (empty ? 0.f : NAN));
  }
  if (a.lse && tid < G) {
    const int g = tid;
    const float M = hml[g][0], L = hml[g][1], LE = hml[g][2];
    const bool bad = hml[g][3] != 0.f;
    const float l2 = bad ? NAN : (L > 0.f ? M + log2f(LE / static_cast<float>(PS)) + a.offs[bh * 8 + g]
                                          : (empty ? -INFINITY : NAN));
    a.lse[static_cast<int64_t>(b) * a.n_q + h * G + g] = l2 * 0.69314718055994530942f;
  }
}

aatc_status launch_merge(const aatc_cache* c, const Plan& p, int32_t n_q, const int32_t* seq_lens, int seq_per_head,
                         int64_t max_seq, float* out, float* lse, void* ws, hipStream_t st) {
  const int group = n_q / c->n_kv_heads;
  char* w = static_cast<char*>(ws);
  CombArgs cb;
  cb.part = reinterpret_cast<const float*>(w);
  cb.offs = reinterpret_cast<const float*>(w + align256(p.part_bytes));
  cb.n_kv = c->n_kv_heads;
  cb.n_q = n_q;
  cb.group = group;
  cb.S = p.S;
  cb.prec = p.prec;
  cb.seq_lens = seq_lens;
  cb.seq_per_head = seq_per_head;
  cb.max_seq = max_seq;
  cb.out = out;
  cb.lse = lse;
  cb.lm = p.lm ? 1 : 0;
  if (p.S <= CH_MAXS && group <= 8)
    hipLaunchKernelGGL(k_attn_combine_heads, dim3(c->n_kv_heads, c->batch), dim3(CH_THREADS), 0, st, cb,
                       static_cast<const aatc_calib*>(c->v_calib));
  else
    hipLaunchKernelGGL(k_attn_combine, dim3(group, c->n_kv_heads, c->batch), dim3(CNT), 0, st, cb,
                       static_cast<const aatc_calib*>(c->v_calib));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "decode_attn combine launch: %s", hipGetErrorString(err));
  return AATC_OK;
}

}  // namespace

extern "C" {

aatc_status aatc_decode_attn(const aatc_cache* c, const void* q, aatc_dtype q_dtype, int32_t n_q,
                             const int32_t* seq_lens, int64_t max_seq, float scale, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  aatc::clear_error();
  if (!q || !out) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (q_dtype != AATC_F32 && q_dtype != AATC_BF16)
    return aatc::fail(AATC_ERR_UNSUPPORTED, "q dtype %d (fp32 or bf16)", static_cast<int>(q_dtype));
  Plan p;
  aatc_status r = check_and_plan(c, n_q, max_seq, ws, ws_bytes, &p);
  if (r != AATC_OK) return r;
  auto st = static_cast<hipStream_t>(stream);
  const float* q32 = nullptr;
  r = prepare_q(q, q_dtype, p, ws, st, &q32);
  if (r != AATC_OK) return r;
  r = launch_partial(c, p, q32, n_q, seq_lens, 0, max_seq, scale, ws, st);
  if (r != AATC_OK) return r;
  return launch_merge(c, p, n_q, seq_lens, 0, max_seq, out, lse, ws, st);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];            // device address of `scratch` on each device, once known

// The current device's copy of `scratch`, looked up on the first call on that device.
aatc_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return aatc::fail(AATC_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return aatc::fail(AATC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return AATC_OK;
}

}  // namespace

extern "C" {

aatc_status aatc_decode_attn_noalloc(const aatc_cache* c, const void* q, aatc_dtype q_dtype, int32_t n_q,
                                     const int32_t* seq_lens, int64_t max_seq, float scale, float* out, float* lse,
                                     void* stream) {
  aatc::clear_error();
  if (!q || !out) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (q_dtype != AATC_F32 && q_dtype != AATC_BF16)
    return aatc::fail(AATC_ERR_UNSUPPORTED, "q dtype %d (fp32 or bf16)", static_cast<int>(q_dtype));
  // every argument is checked before the scratch address is looked up
  Plan p;
  aatc_status r = check_cache_and_plan(c, n_q, max_seq, &p);
  if (r != AATC_OK) return r;
  const size_t need = plan_workspace(p);
  if (need > AATC_NOALLOC_SCRATCH_BYTES)
    return aatc::fail(AATC_ERR_BUFFER_TOO_SMALL,
                      "this step needs %zu bytes of partial records, more than the %u-byte static workspace of "
                      "aatc_decode_attn_noalloc (call aatc_decode_attn with a workspace instead)",
                      need, static_cast<unsigned>(AATC_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  r = scratch_address(&ws);
  if (r != AATC_OK) return r;
  auto st = static_cast<hipStream_t>(stream);
  const float* q32 = nullptr;
  r = prepare_q(q, q_dtype, p, ws, st, &q32);
  if (r != AATC_OK) return r;
  r = launch_partial(c, p, q32, n_q, seq_lens, 0, max_seq, scale, ws, st);
  if (r != AATC_OK) return r;
  return launch_merge(c, p, n_q, seq_lens, 0, max_seq, out, lse, ws, st);
}

aatc_status aatc_decode_attn_partial(const aatc_cache* c, const void* q, aatc_dtype q_dtype, int32_t n_q,
                                     const int32_t* seq_lens, int64_t max_seq, float scale, void* ws, size_t ws_bytes,
                                     void* stream) {
  aatc::clear_error();
  if (!q) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (q_dtype != AATC_F32 && q_dtype != AATC_BF16)
    return aatc::fail(AATC_ERR_UNSUPPORTED, "q dtype %d (fp32 or bf16)", static_cast<int>(q_dtype));
  Plan p;
  aatc_status r = check_and_plan(c, n_q, max_seq, ws, ws_bytes, &p);
  if (r != AATC_OK) return r;
  auto st = static_cast<hipStream_t>(stream);
  const float* q32 = nullptr;
  r = prepare_q(q, q_dtype, p, ws, st, &q32);
  if (r != AATC_OK) return r;
  return launch_partial(c, p, q32, n_q, seq_lens, 0, max_seq, scale, ws, st);
}

aatc_status aatc_decode_attn_merge(const aatc_cache* c, int32_t n_q, const int32_t* seq_lens, int64_t max_seq,
                                   float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  aatc::clear_error();
  if (!out) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  Plan p;
  const aatc_status r = check_and_plan(c, n_q, max_seq, ws, ws_bytes, &p);
  if (r != AATC_OK) return r;
  return launch_merge(c, p, n_q, seq_lens, 0, max_seq, out, lse, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- multi-segment decode attention -----------------------------------------------------------
namespace {

struct SegPlan {
  int n_states;
  size_t states_off, lse_off, attn_off, attn_bytes, total;
};

// Tokens per dense workgroup: the longest chunk, halved (down to one block per wave) while the
// launch would have fewer workgroups than the chip has compute units.
int raw_chunk(const aatc_segment& sg, int32_t batch, int32_t n_kv) {
  int chunk = aatc_dense::CHUNK;
  const int64_t seqs = static_cast<int64_t>(batch) * n_kv;
  while (chunk > aatc_dense::MIN_CHUNK && (sg.max_seq_len + chunk - 1) / chunk * seqs < 256) chunk >>= 1;
  return chunk;
}

int64_t raw_chunks(const aatc_segment& sg, int32_t batch, int32_t n_kv) {
  const int chunk = raw_chunk(sg, batch, n_kv);
  const int64_t nc = (sg.max_seq_len + chunk - 1) / chunk;
  return nc > 0 ? nc : 1;
}

aatc_status seg_plan(const aatc_segment* segs, int32_t n_segs, int32_t batch, int32_t n_kv, int32_t n_q,
                     SegPlan* sp) {
  if (!segs || n_segs < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "no segments");
  if (batch < 1 || n_kv < 1 || n_q < 1 || n_q % n_kv) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "shape");
  if (n_q / n_kv > AATC_MAX_GROUP) return aatc::fail(AATC_ERR_UNSUPPORTED, "GQA group %d > 8", n_q / n_kv);
  if (batch > 65535 || n_kv > 65535) return aatc::fail(AATC_ERR_UNSUPPORTED, "batch or n_kv_heads > 65535");
  int64_t states = 0;
  size_t attn = 0;
  for (int s = 0; s < n_segs; ++s) {
    const aatc_segment& sg = segs[s];
    if (sg.max_seq_len < 0) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "segment %d: max_seq_len < 0", s);
    if (sg.cache) {
      const aatc_cache* c = sg.cache;
      if (c->batch != batch || c->n_kv_heads != n_kv)
        return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "segment %d: cache shape differs from the call", s);
      const size_t w = aatc_decode_attn_workspace_bytes(c, n_q, sg.max_seq_len);
      if (w > attn) attn = w;
      states += 1;
    } else {
      if (!sg.k_raw || !sg.v_raw) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "segment %d: null raw pointer", s);
      if (sg.max_seq_len > sg.raw_capacity)
        return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "segment %d: max_seq_len > raw_capacity", s);
      if ((reinterpret_cast<uintptr_t>(sg.k_raw) & 15) || (reinterpret_cast<uintptr_t>(sg.v_raw) & 15))
        return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "segment %d: raw tensors must be 16-byte aligned", s);
      states += raw_chunks(sg, batch, n_kv);
    }
  }
  if (states > (1 << 20)) return aatc::fail(AATC_ERR_UNSUPPORTED, "too many segment states");
  const size_t bq = static_cast<size_t>(batch) * n_q;
  sp->n_states = static_cast<int>(states);
  sp->states_off = 0;
  sp->lse_off = align256(static_cast<size_t>(states) * bq * AATC_D * 4);
  sp->attn_off = sp->lse_off + align256(static_cast<size_t>(states) * bq * 4);
  sp->attn_bytes = attn;
  sp->total = sp->attn_off + align256(attn);
  return AATC_OK;
}

}  // namespace

extern "C" {

size_t aatc_decode_attn_segments_workspace_bytes(const aatc_segment* segs, int32_t n_segs, int32_t batch,
                                                 int32_t n_kv_heads, int32_t n_q_heads) {
  SegPlan sp;
  if (seg_plan(segs, n_segs, batch, n_kv_heads, n_q_heads, &sp) != AATC_OK) return 0;
  return sp.total;
}

aatc_status aatc_decode_attn_segments(const aatc_segment* segs, int32_t n_segs, int32_t batch, int32_t n_kv,
                                      const float* q, int32_t n_q, float scale, float* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  aatc::clear_error();
  if (!q || !out || !ws) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(q) & 15) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "q not 16-byte aligned");
  SegPlan sp;
  aatc_status r = seg_plan(segs, n_segs, batch, n_kv, n_q, &sp);
  if (r != AATC_OK) return r;
  if (ws_bytes < sp.total) return aatc::fail(AATC_ERR_BUFFER_TOO_SMALL, "workspace %zu < %zu", ws_bytes, sp.total);
  // validate every coded segment before launching anything
  for (int s = 0; s < n_segs; ++s) {
    if (!segs[s].cache) continue;
    Plan p;
    r = check_and_plan(segs[s].cache, n_q, segs[s].max_seq_len, static_cast<char*>(ws) + sp.attn_off, sp.attn_bytes,
                       &p);
    if (r != AATC_OK) {
      char msg[400];
      snprintf(msg, sizeof msg, "%s", aatc_last_error());
      return aatc::fail(r, "segment %d: %s", s, msg);
    }
  }
  auto st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* out_states = reinterpret_cast<float*>(w + sp.states_off);
  float* lse_states = reinterpret_cast<float*>(w + sp.lse_off);
  void* attn_ws = w + sp.attn_off;
  const int64_t bq = static_cast<int64_t>(batch) * n_q;
  const float scale_v = scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(AATC_D));
  int state = 0;
  for (int s = 0; s < n_segs; ++s) {
    const aatc_segment& sg = segs[s];
    if (sg.cache) {
      Plan p;
      r = check_and_plan(sg.cache, n_q, sg.max_seq_len, attn_ws, sp.attn_bytes, &p);
      if (r != AATC_OK) return r;
      r = launch_partial(sg.cache, p, q, n_q, sg.seq_lens_dev, 1, sg.max_seq_len, scale, attn_ws, st);
      if (r != AATC_OK) return r;
      r = launch_merge(sg.cache, p, n_q, sg.seq_lens_dev, 1, sg.max_seq_len, out_states + state * bq * AATC_D,
                       lse_states + state * bq, attn_ws, st);
      if (r != AATC_OK) return r;
      state += 1;
    } else {
      aatc_dense::DenseArgs ra;
      ra.k = static_cast<const uint16_t*>(sg.k_raw);
      ra.v = static_cast<const uint16_t*>(sg.v_raw);
      ra.cap = sg.raw_capacity;
      ra.seq_lens = sg.seq_lens_dev;
      ra.max_seq = sg.max_seq_len;
      ra.q = q;
      ra.n_kv = n_kv;
      ra.n_q = n_q;
      ra.group = n_q / n_kv;
      ra.scale2 = scale_v * 1.4426950408889634f;
      ra.out_states = out_states;
      ra.lse_states = lse_states;
      ra.state0 = state;
      ra.bq = bq;
      ra.chunk = raw_chunk(sg, batch, n_kv);
      const int64_t nc = raw_chunks(sg, batch, n_kv);
      hipLaunchKernelGGL(aatc_dense::k_dense_attn, dim3(static_cast<unsigned>(nc), n_kv, batch),
                         dim3(aatc_dense::NW * 64), 0, st, ra);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "raw segment launch: %s", hipGetErrorString(e));
      state += static_cast<int>(nc);
    }
  }
  hipLaunchKernelGGL(aatc_seg::k_merge_states, dim3(static_cast<unsigned>(bq)), dim3(aatc_seg::MW * 64), 0, st, out_states,
                     lse_states, sp.n_states, bq, out, lse);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return aatc::fail(AATC_ERR_HIP, "segment merge launch: %s", hipGetErrorString(e));
  return AATC_OK;
}

// ---- dense bf16 decode attention: one raw segment ------------------------------------------
static aatc_segment dense_segment(const void* k, const void* v, int64_t capacity, const int32_t* seq_lens,
                                  int64_t max_seq) {
  aatc_segment sg;
  sg.cache = nullptr;
  sg.k_raw = k;
  sg.v_raw = v;
  sg.raw_capacity = capacity;
  sg.seq_lens_dev = seq_lens;
  sg.max_seq_len = max_seq;
  return sg;
}

size_t aatc_decode_attn_dense_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                              int64_t max_seq_len) {
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  const aatc_segment sg = dense_segment(dummy, dummy, max_seq_len, nullptr, max_seq_len);
  return aatc_decode_attn_segments_workspace_bytes(&sg, 1, batch, n_kv_heads, n_q_heads);
}

aatc_status aatc_decode_attn_dense(const void* k_dev, const void* v_dev, int32_t batch, int32_t n_kv_heads,
                                   int64_t capacity_tokens, const int32_t* seq_lens_dev, int64_t max_seq_len,
                                   const float* q_dev, int32_t n_q_heads, float softmax_scale, float* out_dev,
                                   float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  aatc::clear_error();
  if (capacity_tokens < 0) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "capacity_tokens < 0");
  const aatc_segment sg = dense_segment(k_dev, v_dev, capacity_tokens, seq_lens_dev, max_seq_len);
  return aatc_decode_attn_segments(&sg, 1, batch, n_kv_heads, q_dev, n_q_heads, softmax_scale, out_dev, lse_dev,
                                   workspace_dev, workspace_bytes, stream);
}

}  // extern "C"
