// Decode attention on the packed cache: host-side plan, validation and launch.
// The kernel (and the method it implements) is described in aatc_attn_kernel.h.
#define AATC_ATTN_COMBINE_TU
#include "aatc_attn_kernel.h"
#include "aatc_dense_kernel.h"
#include "aatc_seg_kernel.h"

#include <cstdio>

namespace {

using namespace aatc_attn;

constexpr size_t kLdsLimit = 160 * 1024;
// __shared__ arrays of the kernel: the probability rows plus scalars (rounded up)
constexpr size_t kStaticLds = static_cast<size_t>(CW) * TG * PROW_BYTES + 2048;

int vtiles_bucket(int vt) {
  if (vt <= 12) return 12;
  if (vt <= 16) return 16;
  if (vt <= 24) return 24;
  return -1;
}

struct Plan {
  int NP, NVB, LIMBS, S, tpw, half, prec, prod;
  int nslot, slot_bytes, ksz, gs, wave_bytes;
  size_t lds;
  size_t part_bytes, offs_bytes;
  bool fits;
};

int round16(int64_t x) { return static_cast<int>((x + 15) / 16 * 16); }

// Tiles per wave fill 256 CUs x CW waves once; each wave gets a ring of LDS slots (one tile
// each), as many as fit, at most its tile count.
Plan make_plan(const aatc_cache* c, int n_q, int64_t max_seq) {
  Plan p;
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
  const size_t avail = kLdsLimit - kStaticLds - FIXED_LDS - DMA_PAD;
  int ns = static_cast<int>(avail / (static_cast<size_t>(CW) * p.slot_bytes));
  if (ns > p.tpw) ns = p.tpw;
  p.nslot = ns;
  p.fits = ns >= 1;
  // one score group per wave when its tiles all fit (no running-max rescale at all);
  // otherwise groups of half the slots, so that the next group's copies fly meanwhile
  if (ns >= p.tpw) {
    p.gs = p.tpw < TG ? p.tpw : TG;
  } else {
    p.gs = ns / 2 < TG ? ns / 2 : TG;
    if (p.gs < 1) p.gs = 1;
  }
  // a wave's ring area holds its slots, and at the end its merge values
  p.wave_bytes = (ns > 0 ? ns : 1) * p.slot_bytes;
  if (p.wave_bytes < p.NVB * merge_group_bytes(p.NVB)) p.wave_bytes = p.NVB * merge_group_bytes(p.NVB);
  const size_t ring = static_cast<size_t>(CW) * p.wave_bytes + DMA_PAD;
  p.lds = FIXED_LDS + ring;
  if (p.lds + kStaticLds > kLdsLimit) p.fits = false;
  // copy waves issue every tile when all of a wave's tiles have slots and the copy count of one
  // copy wave stays within what one wait can count
  {
    const int ik = kb > 0 ? (static_cast<int>((15 + 8LL * kb + 15) / 16) + 63) / 64 : 0;
    const int iv = vb > 0 ? (static_cast<int>((15 + 8LL * vb + 15) / 16) + 63) / 64 : 0;
    p.prod = (p.NVB == 12 && p.NP <= 2 && ns >= p.tpw && (CW / NPROD_MAX) * p.tpw * (ik + iv) <= 60) ? NPROD_MAX : 0;
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
    case 1: *err = launch_np<1>(p.half, p.NVB, p.LIMBS, a, kc, vc, grid, p.lds, st, &found); break;
    case 2: *err = launch_np<2>(p.half, p.NVB, p.LIMBS, a, kc, vc, grid, p.lds, st, &found); break;
    case 3: *err = launch_np<3>(p.half, p.NVB, p.LIMBS, a, kc, vc, grid, p.lds, st, &found); break;
    case 4: *err = launch_np<4>(p.half, p.NVB, p.LIMBS, a, kc, vc, grid, p.lds, st, &found); break;
  }
  return found;
}

}  // namespace

extern "C" {

size_t aatc_decode_attn_workspace_bytes(const aatc_cache* c, int32_t n_q_heads, int64_t max_seq_len) {
  if (!c || max_seq_len < 0 || n_q_heads < 1) return 0;
  const Plan p = make_plan(c, n_q_heads, max_seq_len);
  return align256(p.part_bytes) + align256(p.offs_bytes);
}

}  // extern "C"

namespace {

// Shared argument checks and plan of the three decode-attention entry points.
aatc_status check_and_plan(const aatc_cache* c, int32_t n_q, int64_t max_seq, void* ws, size_t ws_bytes, Plan* p) {
  if (!c || !ws) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (c->d != AATC_D) return aatc::fail(AATC_ERR_UNSUPPORTED, "d=%d (only 128)", c->d);
  if (c->batch < 1 || c->n_kv_heads < 1 || n_q < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "shape");
  if (n_q % c->n_kv_heads) return aatc::fail(AATC_ERR_UNSUPPORTED, "n_q_heads %% n_kv_heads != 0");
  const int group = n_q / c->n_kv_heads;
  if (group > AATC_MAX_GROUP) return aatc::fail(AATC_ERR_UNSUPPORTED, "GQA group %d > 8", group);
  if (c->k_bits < 0 || c->k_bits > 512 || c->v_bits < 0 || c->v_bits > 512)
    return aatc::fail(AATC_ERR_UNSUPPORTED, "k_bits %d / v_bits %d: decode attention handles 0..512 bits per vector",
                      c->k_bits, c->v_bits);
  if (vtiles_bucket(c->v_tiles) < 0 || c->v_tiles < 0)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "v_tiles %d", c->v_tiles);
  if (!c->k_calib || !c->v_calib || (!c->k_codes && c->k_bits > 0) || (!c->v_codes && c->v_bits > 0))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null cache pointer");
  if ((reinterpret_cast<uintptr_t>(c->k_codes) & 15) || (reinterpret_cast<uintptr_t>(c->v_codes) & 15) ||
      (reinterpret_cast<uintptr_t>(ws) & 255))
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "codes must be 16-byte and workspace 256-byte aligned");
  if (max_seq < 0 || max_seq > c->capacity_tokens)
    return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "max_seq_len %lld > capacity", (long long)max_seq);
  *p = make_plan(c, n_q, max_seq);
  const size_t need = align256(p->part_bytes) + align256(p->offs_bytes);
  if (ws_bytes < need) return aatc::fail(AATC_ERR_BUFFER_TOO_SMALL, "workspace %zu < %zu", ws_bytes, need);
  if (!p->fits) return aatc::fail(AATC_ERR_UNSUPPORTED, "tiles of %d+%d bits do not fit LDS", c->k_bits, c->v_bits);
  return AATC_OK;
}

aatc_status launch_partial(const aatc_cache* c, const Plan& p, const float* q, int32_t n_q, const int32_t* seq_lens,
                           int seq_per_head, int64_t max_seq, float scale, void* ws, hipStream_t st) {
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
  const dim3 grid(p.S, c->n_kv_heads, c->batch);
  hipError_t err = hipSuccess;
  const bool ok = dispatch(p, a, kcal, vcal, grid, st, &err);
  if (!ok) return aatc::fail(AATC_ERR_UNSUPPORTED, "plan NP=%d NVB=%d", p.NP, p.NVB);
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "decode_attn launch: %s", hipGetErrorString(err));
  return AATC_OK;
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
  hipLaunchKernelGGL(k_attn_combine, dim3(group, c->n_kv_heads, c->batch), dim3(CNT), 0, st, cb,
                     static_cast<const aatc_calib*>(c->v_calib));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return aatc::fail(AATC_ERR_HIP, "decode_attn combine launch: %s", hipGetErrorString(err));
  return AATC_OK;
}

}  // namespace

extern "C" {

aatc_status aatc_decode_attn(const aatc_cache* c, const float* q, int32_t n_q, const int32_t* seq_lens,
                             int64_t max_seq, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream) {
  aatc::clear_error();
  if (!q || !out) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  Plan p;
  aatc_status r = check_and_plan(c, n_q, max_seq, ws, ws_bytes, &p);
  if (r != AATC_OK) return r;
  auto st = static_cast<hipStream_t>(stream);
  r = launch_partial(c, p, q, n_q, seq_lens, 0, max_seq, scale, ws, st);
  if (r != AATC_OK) return r;
  return launch_merge(c, p, n_q, seq_lens, 0, max_seq, out, lse, ws, st);
}

aatc_status aatc_decode_attn_partial(const aatc_cache* c, const float* q, int32_t n_q, const int32_t* seq_lens,
                                     int64_t max_seq, float scale, void* ws, size_t ws_bytes, void* stream) {
  aatc::clear_error();
  if (!q) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  Plan p;
  const aatc_status r = check_and_plan(c, n_q, max_seq, ws, ws_bytes, &p);
  if (r != AATC_OK) return r;
  return launch_partial(c, p, q, n_q, seq_lens, 0, max_seq, scale, ws, static_cast<hipStream_t>(stream));
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
