/*
 * aatc.h -- C ABI of the MI355X (gfx950) transform-coded KV-cache library.
 *
 * The method (page "KV Cache Compression Through the Lens of Transform Coding", Key points
 * and Full text; page "SPECTRA: Pushing the KV Cache Beyond the 2-Bit Cliff via Spectral
 * Transform Coding", Abstract): per KV head, rotate the cached vectors into a decorrelating
 * basis computed from calibration statistics (KLT), or a Walsh-Hadamard basis (page
 * "Ablation, Statistical Inference, and Validation for KV-Cache Compression", first
 * abstract); give each rotated channel 0..8 bits by reverse water-filling under a
 * bits-per-element budget; quantize each channel with a uniform scalar quantizer and pack
 * the codes at a fixed number of bits per token (page "SPHERICAL KV ...", NOVA-KV abstract:
 * fixed per-token bit count).  Decode attention reads the packed codes directly: the query
 * is rotated once, scores are formed in the rotated domain and values are dequantized and
 * rotated back only after the softmax-weighted sum (page "Ablation ...", OCTOPUS abstract:
 * keys are never materialised).  Also here:
 *  - attention-aware key bits (query channel weights) and a joint K/V bit split (AATC
 *    abstract);
 *  - a non-orthogonal key transform from query statistics (NOVA-KV abstract);
 *  - token tiers with multi-segment attention (RDKV abstract);
 *  - a dense bf16 decode attention as the full-cache comparator.
 *
 * Conventions for every call:
 *  - Every call returns an aatc_status.  Arguments are validated on the host before any
 *    device work is queued; on an error nothing is written and aatc_last_error() (per
 *    thread) holds a message.  No C++ exception crosses this interface.
 *  - Device calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream).  Faults during execution surface at the caller's next synchronisation.
 *  - The caller owns and frees every buffer.  The library allocates no device memory and
 *    keeps no device state between calls.
 *  - Head dimension d is 128.  Channel stride is 1 in every tensor; other strides are in
 *    elements.
 *  - Concurrent calls that write the same cache tile are a caller race.
 */
#ifndef AATC_H
#define AATC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AATC_OK = 0,
  AATC_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad shape, range or stride */
  AATC_ERR_UNSUPPORTED = 2,      /* d != 128, GQA group > 8, dtype not handled */
  AATC_ERR_BUDGET = 3,           /* bits per vector outside [0, 8d] */
  AATC_ERR_NUMERICAL = 4,        /* non-finite calibration data, eigensolver did not converge */
  AATC_ERR_BAD_ARTEFACT = 5,     /* calibration blob magic/version/checksum/contents wrong */
  AATC_ERR_BUFFER_TOO_SMALL = 6, /* output blob or workspace smaller than required */
  AATC_ERR_HIP = 7               /* a HIP launch failed; message in aatc_last_error() */
} aatc_status;

typedef enum { AATC_F32 = 0, AATC_BF16 = 1, AATC_F64 = 2 } aatc_dtype;
typedef enum { AATC_ROT_KLT = 0, AATC_ROT_WHT = 1, AATC_ROT_IDENTITY = 2, AATC_ROT_NOVA = 3 } aatc_rotation;
typedef enum { AATC_QUANT_UNIFORM = 0, AATC_QUANT_LLOYD_MAX = 1 } aatc_quantizer;

#define AATC_D 128
#define AATC_TILE 64             /* tokens per packed tile */
#define AATC_MAX_BITS 8
#define AATC_MAX_FIELDS 384      /* 3 fields per channel at most (7 = 4+2+1) */
#define AATC_MAX_GROUP 8         /* q heads per KV head handled by decode attention */
#define AATC_MAX_ATTN_BITS 512   /* bits per K or V vector the summed-code cache pass reads (4 per
                                    element); decode attention over more takes the level pass */
#define AATC_MAGIC 0x43544141u   /* "AATC" */
#define AATC_VERSION 3u
#define AATC_LEVELS 510          /* level-table entries: 2^b for each b = 1..8, table b at 2^b - 2 */

/*
 * Calibration artefact of one (layer, KV head, tensor K|V): a plain-old-data blob that is
 * written by aatc_calibrate on the host, copied byte for byte to device memory by the
 * caller, and read there by the kernels.  A cache tensor uses n_kv_heads consecutive blobs.
 *
 * Packed formats (fixed per-token bit count B = total_bits; a 64-token tile is exactly
 * 64*B bits = 2B little-endian uint32 words; string bit s is bit s%32 of word s/32; tile j of
 * sequence (b,h) starts at word ((b*n_kv_heads + h)*tiles_per_seq + j)*2B):
 *
 *  K tiles, token-major bit-planes.  Token t (0..63) owns string bits [tB, tB+B).  Its plane
 *    p (plane_channel[p], plane_bit[p]) sits at bit tB+p; planes are ordered by channel
 *    ascending, then code bit ascending (plane (i,k) holds bit k of code c_i).
 *
 *  V tiles, field-major.  Channel i's code is split by the binary expansion of b_i into
 *    fields of width 4, 2, 1 (8 = 4+4), low code bits in the widest field.  Fields are
 *    ordered by width descending, channel ascending, shift ascending; field f of width w owns
 *    the 2w words starting at field_word[f].  Bit b (LSB first) of the w-bit value of token
 *    t = 16G + 4r + m (G,r,m in 0..3) sits at this bit offset of the field's 64w-bit string:
 *       w=1: 32*(G/2) + 8m + 2r + (G%2)
 *       w=2: 32G + ((8m + 2r + b + (G%2)) mod 32)      (odd G: the word rotated left by 1)
 *       w=4: 64G + 32*(r/2) + 8m + 4*(r%2) + b
 *    (so that four tokens' values land in the four bytes of one word after a shift).
 *
 * Quantizer, uniform (mid-rise, per channel): for b_i >= 1,
 *    c_i = clamp(floor((y_i - o_i) * inv_delta_i + 2^(b_i-1)), 0, 2^b_i - 1),  y = E x,
 *    evaluated in fp64 with separately rounded operations; NaN -> 0; +-Inf -> clamp ends.
 *    Reconstruction y_hat_i = o_i + delta_i (c_i - 2^(b_i-1) + 1/2); b_i = 0 gives o_i;
 *    x_hat = R^T y_hat.
 * Quantizer, Lloyd-Max (page "SPHERICAL KV ...", NOVA-KV abstract: fixed-width uniform scalar
 *    quantizers lose at low rates; page "Ablation ...", OCTOPUS abstract: coordinates quantized
 *    with the Lloyd-Max quantizer of their marginal): channel i uses the 2^b_i-level
 *    MSE-optimal quantizer of N(0,1), scaled by scale_i (the channel's standard deviation):
 *    z = (y_i - o_i) * inv_scale_i (fp64, separately rounded), c_i = the number of
 *    thresholds t_(b,k) <= z (NaN -> 0), y_hat_i = o_i + scale_i l_(b,c).  Codes keep b_i bits, so
 *    the packed formats are the same.
 * Either way y_hat_i = o_i + scale_i level[2^b - 2 + c] with scale_i = delta_i and level =
 * c - 2^(b-1) + 1/2 for the uniform quantizer.
 */
typedef struct aatc_calib {
  uint32_t magic;          /* AATC_MAGIC */
  uint32_t version;        /* AATC_VERSION */
  int32_t d;               /* 128 */
  int32_t rotation;        /* aatc_rotation */
  int32_t total_bits;      /* B = sum_i bits[i] */
  int32_t max_bits;        /* 8 */
  int32_t n_coded;         /* channels with bits > 0 */
  int32_t n_fields;        /* V fields = n_fields4 + n_fields2 + n_fields1 */
  int32_t n_fields4, n_fields2, n_fields1;
  int32_t n_calib;         /* calibration rows used */
  uint64_t checksum;       /* FNV-1a 64 of the whole blob with this field set to 0 */
  double R[AATC_D * AATC_D];         /* query transform q~ = R q and reconstruction x = R^T y;
                                        orthogonal, except NOVA: R = E^-T */
  double mu[AATC_D];                 /* calibration mean (original basis) */
  double o[AATC_D];                  /* per-channel offset E mu */
  double sigma2[AATC_D];             /* rotated-channel variance */
  double delta[AATC_D];              /* quantizer step (0 for b_i = 0) */
  double inv_delta[AATC_D];          /* 1/delta, correctly rounded (0 for b_i = 0) */
  float R32[AATC_D * AATC_D];        /* fp32 copy of R */
  float o32[AATC_D];
  float delta32[AATC_D];
  uint8_t bits[AATC_D];              /* b_i in 0..8 */
  uint8_t plane_channel[AATC_D * AATC_MAX_BITS];
  uint8_t plane_bit[AATC_D * AATC_MAX_BITS];
  uint16_t field_channel[AATC_MAX_FIELDS];
  uint8_t field_shift[AATC_MAX_FIELDS];
  uint8_t field_width[AATC_MAX_FIELDS];
  uint16_t field_word[AATC_MAX_FIELDS];
  int16_t channel_field[AATC_D * 3];  /* fields of channel i, -1 padded */
  double E[AATC_D * AATC_D];         /* encoder: coefficients y = E x (E = R except NOVA) */
  int32_t quantizer;                 /* aatc_quantizer */
  int32_t pad0;
  double scale[AATC_D];              /* reconstruction scale: delta (uniform), sigma (Lloyd-Max);
                                        0 for b_i = 0 */
  double inv_scale[AATC_D];          /* 1/scale, correctly rounded (0 for b_i = 0) */
  float scale32[AATC_D];
  double level[AATC_LEVELS];         /* standardized reconstruction levels of b = 1..8 bits */
  double thresh[AATC_LEVELS];        /* Lloyd-Max: the 2^b - 1 standardized thresholds of each b,
                                        ascending, at 2^b - 2 (uniform: 0) */
  float level32[AATC_LEVELS];
  uint8_t reserved[64];
} aatc_calib;

typedef struct {
  int32_t d;               /* 128 */
  int32_t rotation;        /* aatc_rotation */
  double bits_per_elem;    /* average budget b; B = floor(b*d + 1/2) */
  int32_t max_bits;        /* per-channel cap, 8 (1..8) */
  int32_t quantizer;       /* aatc_quantizer: 0 uniform (default), 1 Lloyd-Max */
  const double* channel_weight;  /* NULL: the cache-MSE allocation; else d weights w_i >= 0 of
                                    the rotated channels (attention-aware keys: see
                                    aatc_query_channel_weights) */
  const double* query_moment;    /* AATC_ROT_NOVA only: d x d row-major second moment
                                    E[q q^T] of calibration queries (aatc_query_moment);
                                    NULL otherwise */
} aatc_calib_params;

/* Readable bytes a codes buffer must have past its last sequence's words: decode attention
 * copies whole 16-byte units. */
#define AATC_CODES_SLACK 16

/* A compressed cache of one layer, one tensor pair: every pointer is device memory.
 * k_codes/v_codes hold batch*n_kv_heads*(capacity_tokens/64) tiles of 2*k_bits (2*v_bits)
 * words, followed by AATC_CODES_SLACK readable bytes (contents unused).  k_calib/v_calib
 * point at n_kv_heads consecutive aatc_calib blobs whose
 * total_bits equal k_bits / v_bits (checked by the kernels: a mismatching head is skipped
 * and its decode-attention outputs are NaN).  A tensor with 0 bits may pass NULL codes. */
typedef struct {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t d;                /* 128 */
  int32_t k_bits;           /* B of every K blob */
  int32_t v_bits;           /* B of every V blob */
  int32_t v_tiles;          /* max over the V blobs of aatc_calib_v_tiles() (<= 24) */
  int32_t quantizer;        /* bit 0: the K blobs are Lloyd-Max, bit 1: the V blobs (checked by the
                               kernels like k_bits / v_bits) */
  int32_t reserved;         /* 0 */
  int64_t capacity_tokens;  /* tokens per (b,h); multiple of 64 */
  const void* k_calib;
  const void* v_calib;
  void* k_codes;
  void* v_codes;
} aatc_cache;

/* Status text; thread-local message of the last failing call on this thread. */
const char* aatc_status_string(aatc_status s);
const char* aatc_last_error(void);

/* Sizes.  aatc_calib_bytes(d) = sizeof(aatc_calib) for d = 128, 0 otherwise.
 * aatc_bits_budget = floor(b*d + 1/2), or -1 when outside [0, 8d].
 * aatc_packed_bytes = ceil(n/64) * 8 * total_bits (one (b,h) sequence). */
size_t aatc_calib_bytes(int32_t d);
int32_t aatc_bits_budget(double bits_per_elem, int32_t d);
size_t aatc_packed_bytes(int32_t total_bits, int64_t n_tokens);

/*
 * aatc_calibrate -- host, synchronous, fp64.  [AATC Full text: "allocates bits over a
 * calibration set"; SPECTRA Abstract: a coordinate system computed from the cache's own
 * statistics; RDKV abstract: reverse water-filling applied once after prefill]
 *   mean and centred covariance (1/M) of the n_calib rows of x_host (row r at
 *   x_host + r*row_stride elements, dtype F32/BF16/F64); rotation R (KLT: eigenvectors of
 *   the covariance, descending eigenvalues, largest-magnitude entry of each row positive;
 *   WHT: Sylvester Hadamard / sqrt(d); IDENTITY); integer reverse water-filling of
 *   B = floor(b*d+1/2) bits over the rotated variances (the B largest candidates
 *   w_i sigma_i^2 4^-k, k < max_bits, ordered by value desc, channel asc, bit asc; w_i = 1
 *   unless params->channel_weight is given, which then makes the allocation minimise
 *   sum_i w_i sigma_i^2 4^-b_i, the weighted, attention-aware distortion); quantizer
 *   step delta_i = sigma_i g(b_i) where g(b) minimises the MSE of the 2^b-level mid-rise
 *   uniform quantizer on N(0,1); offset o = E mu; packing tables.  E = R for KLT, WHT and
 *   IDENTITY.
 *   NOVA [SPHERICAL KV page, NOVA-KV abstract: a closed-form key transform from calibration
 *   statistics that is not orthogonal and turns the attention-aware distortion into MSE of
 *   the transformed coefficients]: with S = params->query_moment (eigenvalues below 1e-6 of
 *   the largest raised to it), E = U S^(1/2) where the rows of U are the KLT (as above) of
 *   S^(1/2) C S^(1/2), sigma2 its eigenvalues, and R = E^-T = U S^(-1/2): decode attention
 *   scores q.x as (R q).(E x) and reconstructs x = R^T y, so the kernels run unchanged.
 *   Writes one aatc_calib into calib_host (calib_bytes >= aatc_calib_bytes(d)).
 *   Errors: d != 128 -> UNSUPPORTED; B outside [0, 8d] or max_bits outside 1..8 -> BUDGET;
 *   n_calib < 2, null pointers, row_stride < d, a negative channel weight, NOVA without a
 *   query moment or a moment that is not symmetric -> INVALID_ARGUMENT; a non-finite value,
 *   weight or moment, a moment with no positive eigenvalue -> NUMERICAL; small blob ->
 *   BUFFER_TOO_SMALL.  Zero-variance (or zero-weight) channels get 0 bits unless the budget
 *   exceeds 8 x (the other channels).
 */
aatc_status aatc_calibrate(const aatc_calib_params* params, const void* x_host, aatc_dtype dtype,
                           int64_t n_calib, int64_t row_stride, void* calib_host,
                           size_t calib_bytes);

/*
 * aatc_query_channel_weights -- host, synchronous, fp64.  [AATC abstract: when quantization
 * errors are modelled as white noise, the mean attention-aware error is a sum of a key part
 * and a value part, each separable over tokens and over channels]  For a key blob's rotation R and n calibration
 * queries q (row r at q_host + r*row_stride elements, dtype F32/BF16/F64: the query heads
 * that share the KV head), w_out[i] = (1/n) sum_r ((R q_r)_i)^2.  The expected squared score
 * error of a zero-mean white key error is sum_i w_i E[e_i^2], so passing w as channel_weight
 * to aatc_calibrate (on the same keys, which gives the same R) allocates the key bits to
 * minimise the score error instead of the cache MSE.
 *   Errors: the blob's aatc_calib_validate status; n < 1, null pointers, row_stride < d ->
 *   INVALID_ARGUMENT; a non-finite query -> NUMERICAL.
 */
aatc_status aatc_query_channel_weights(const void* calib_host, size_t calib_bytes, const void* q_host,
                                       aatc_dtype dtype, int64_t n, int64_t row_stride, double* w_out);

/*
 * aatc_query_moment -- host, synchronous, fp64.  [SPHERICAL KV page, NOVA-KV abstract: the key
 * transform comes from key and query calibration statistics]  moment_out[d*d] (row-major) =
 * (1/n) sum_r q_r q_r^T over n query rows (row r at q_host + r*row_stride elements, dtype
 * F32/BF16/F64), the second moment (not centred) that aatc_calibrate's NOVA transform takes.
 *   Errors: n < 1, null pointers, row_stride < d -> INVALID_ARGUMENT; a non-finite query ->
 *   NUMERICAL.
 */
aatc_status aatc_query_moment(const void* q_host, aatc_dtype dtype, int64_t n, int64_t row_stride,
                              double* moment_out);

/*
 * aatc_joint_kv_split -- host, synchronous, fp64.  [AATC abstract: the expected
 * attention-aware distortion splits into a key term and a value term]  How to share
 * total_bits bits per (key, value) vector pair between the K and V caches of one layer, whose
 * heads all use the same B_K (and B_V = total_bits - B_K):
 *   B_K = argmin sum_h lambda_h D_K,h(B_K) + D_V,h(total_bits - B_K),
 *   D(B) = sum_i w_i sigma2_i 4^-b_i(B) with b(B) the water-filling of aatc_calibrate at the
 *   blob's max_bits (keys: w = k_weight row of the head, or 1; values: w = 1), and
 *   lambda_h = scale^2 sum_i sigma2_V,h,i (scale = softmax_scale, or 1/sqrt(d) if <= 0): to
 *   first order a score error ds_t moves the output by sum_t p_t ds_t (v_t - out) and a value
 *   error e_t by sum_t p_t e_t, so with independent errors the two mean squares are
 *   sum_t p_t^2 |v_t - out|^2 scale^2 D_K and sum_t p_t^2 D_V, and |v_t - out|^2 averages
 *   tr(C_V) when the output sits near the values' mean.  Among values within 1e-12 (relative)
 *   of the minimum the smallest B_K is taken.  The blobs' allocations are ignored: only their
 *   sigma2 and max_bits are used, so any budget may have produced them; calibrate again with
 *   bits_per_elem = B_K/d and B_V/d.
 *   k_calib_host / v_calib_host: n_heads consecutive blobs each; k_weight: NULL or
 *   [n_heads][d] fp64 (aatc_query_channel_weights of each head; NULL for NOVA keys, whose
 *   coefficients already carry the query statistics).
 *   B_K and B_V are each limited to min(d max_bits, AATC_MAX_ATTN_BITS), so that the split
 *   keeps both tensors on decode attention's summed-code pass (past it a tensor takes the
 *   slower level pass).
 *   Errors: a blob's aatc_calib_validate status; n_heads < 1, null pointers, a negative weight
 *   -> INVALID_ARGUMENT; a non-finite weight -> NUMERICAL; total_bits outside
 *   [0, min(d max_bits_K, AATC_MAX_ATTN_BITS) + min(d max_bits_V, AATC_MAX_ATTN_BITS)] -> BUDGET.
 */
aatc_status aatc_joint_kv_split(const void* k_calib_host, const void* v_calib_host, int32_t n_heads,
                                const double* k_weight, float softmax_scale, int32_t total_bits,
                                int32_t* k_bits_out, int32_t* v_bits_out);

/* Checks magic, version, d, checksum and internal consistency of a host blob. */
aatc_status aatc_calib_validate(const void* calib_host, size_t calib_bytes);

/* Number of 16-field column groups decode attention uses for a V blob:
 * ceil(n_fields4/16) + ceil(n_fields2/16) + ceil(n_fields1/16) (0..24); -1 for a null blob or
 * a wrong magic or d (the checksum is aatc_calib_validate's job). */
int32_t aatc_calib_v_tiles(const void* calib_host);

/*
 * aatc_encode -- device, async.  [page "Ablation, Statistical Inference, and Validation for
 * KV-Cache Compression", first abstract: a Walsh-Hadamard transform followed by a scalar MSE
 * quantizer; page "SPHERICAL KV ...", NOVA-KV abstract: a fixed number of bits per token; page
 * "SPECTRA ...", Abstract: the cache is coded in the rotated coordinates]  Quantizes and packs
 * tokens [token_offset, token_offset + n_tokens) of every (b,h) of tensor `which` (0 = K, 1 = V)
 * into the cache.
 *   x_dev: element (b,h,t,j) at x_dev[b*strides[0] + h*strides[1] + t*strides[2] + j],
 *   t relative to token_offset; dtype F32 or BF16.  The blob's encoder y = E x (E = R except
 *   for NOVA keys) and the quantizer run in fp64.  Any 16-byte aligned rows are read with
 *   vector loads, others element by element; the result is the same.
 *   In every tile it touches, tokens before token_offset are preserved and tokens at or
 *   after token_offset + n_tokens are cleared to zero (append-only cache).
 *   Errors: bad which/dtype/pointers, token_offset < 0, n_tokens < 0, token_offset +
 *   n_tokens > capacity -> INVALID_ARGUMENT; d != 128 -> UNSUPPORTED; launch -> HIP.
 */
aatc_status aatc_encode(const aatc_cache* cache, int32_t which, const void* x_dev, aatc_dtype dtype,
                        const int64_t strides[3], int64_t token_offset, int64_t n_tokens,
                        void* stream);

/*
 * aatc_encode_kv -- device, async.  [page "SPHERICAL KV ...", RDKV abstract: the bit allocation
 * is fixed after prefill, and every decode step then appends a token's K and V]  aatc_encode of
 * K (k_dev, k_strides) and of V (v_dev, v_strides) over the same tokens [token_offset,
 * token_offset + n_tokens), in one launch: a decode step's append costs one launch, and the two
 * tensors' memory round trips overlap.  Results are those of the two aatc_encode calls, word for
 * word.  dtype applies to both; a 0-bit tensor is skipped as aatc_encode skips it.
 *   Errors: as aatc_encode, for either tensor (K checked first).
 */
aatc_status aatc_encode_kv(const aatc_cache* cache, const void* k_dev, const void* v_dev, aatc_dtype dtype,
                           const int64_t k_strides[3], const int64_t v_strides[3], int64_t token_offset,
                           int64_t n_tokens, void* stream);

/*
 * aatc_decode -- device, async.  Reconstructs x_hat = R^T y_hat (fp64, stored as F32 or BF16)
 * for tokens [token_offset, token_offset + n_tokens) of every (b,h) into out_dev with the
 * same stride convention as aatc_encode.  Used for checks and for promoting tokens back to
 * full precision (page "SPHERICAL KV ...", QEvict abstract: a quantized window is
 * dequantized and promoted), never on the per-token decode path.
 */
aatc_status aatc_decode(const aatc_cache* cache, int32_t which, int64_t token_offset,
                        int64_t n_tokens, void* out_dev, aatc_dtype out_dtype,
                        const int64_t strides[3], void* stream);

/* Workspace bytes aatc_decode_attn needs for this cache, q-head count and longest sequence. */
size_t aatc_decode_attn_workspace_bytes(const aatc_cache* cache, int32_t n_q_heads,
                                        int64_t max_seq_len);

/*
 * aatc_decode_attn -- device, async; one decode step over the compressed cache.
 * [SPECTRA Abstract and RDKV abstract: every decode step reads the whole cache again;
 *  NOVA-KV abstract: decode is bandwidth-bound]
 *   q_dev: [batch][n_q_heads][128] of q_dtype AATC_F32 or AATC_BF16 (a bf16 q is first widened
 *   to an fp32 copy in the workspace by one small kernel; other dtypes -> UNSUPPORTED); q head g
 *   reads KV head g / (n_q_heads/n_kv_heads)
 *   (contiguous groups, 1..8 q heads per KV head).  seq_lens_dev: int32 [batch] tokens
 *   visible per sequence (each <= max_seq_len <= capacity), or NULL for max_seq_len.
 *   softmax_scale <= 0 selects 1/sqrt(128).
 *   out_dev: fp32 [batch][n_q_heads][128] = sum_t softmax_t(scale q.k_hat_t) v_hat_t with
 *   k_hat, v_hat the reconstructions of aatc_decode, computed as: q~ = R_K q once; scores
 *   from the packed K bits weighted by q~ delta^K (the reconstruction offset cancels in the
 *   softmax); online softmax; softmax-weighted sums of the packed V codes; the affine V
 *   dequantization and R_V^T applied once to the sum.  When either tensor is Lloyd-Max
 *   (cache->quantizer != 0) the levels are not affine in the codes, and when either tensor has
 *   more than AATC_MAX_ATTN_BITS bits per vector the summed-code pass does not take it: the
 *   cache pass then decodes each tile's codes to levels through the blobs' level tables (the
 *   uniform quantizer's table is c - 2^(b-1) + 1/2) and sums probability-weighted V levels
 *   instead (a separate kernel, same arguments and results).  lse_dev (nullable): fp32
 *   [batch][n_q_heads] natural-log sum of exp of the scores.  A sequence with 0 visible
 *   tokens yields out = 0, lse = -inf.
 *   workspace_dev: >= aatc_decode_attn_workspace_bytes(...) bytes of device memory, 256-byte
 *   aligned, for the per-split partial records of the kernels the call launches on `stream`
 *   (and a bf16 q's fp32 copy); its contents need no initialisation.  Calls that share a workspace must be
 *   ordered (same stream) or not overlap in time.
 *   Limits: k_bits and v_bits <= 8d (1024), q-head group <= 8; the summed-code pass (uniform
 *   blobs, both tensors <= AATC_MAX_ATTN_BITS) needs v_tiles <= 24.
 *   Errors: group > 8 or not an integer -> UNSUPPORTED; bits outside 0..8d -> BUDGET; bad
 *   pointers, v_tiles, seq length > capacity -> INVALID_ARGUMENT; workspace too small ->
 *   BUFFER_TOO_SMALL; launch -> HIP.  The status is the launch's: errors inside the kernels
 *   reach the caller as values.  A blob that fails the kernels' header checks, and a workgroup
 *   whose bounded wait on another wave gives up (the bound only keeps a fault from hanging the
 *   GPU; a correct launch never reaches it), make the affected q heads' out and lse NaN.
 */
aatc_status aatc_decode_attn(const aatc_cache* cache, const void* q_dev, aatc_dtype q_dtype, int32_t n_q_heads,
                             const int32_t* seq_lens_dev, int64_t max_seq_len, float softmax_scale,
                             float* out_dev, float* lse_dev, void* workspace_dev,
                             size_t workspace_bytes, void* stream);

/*
 * aatc_decode_attn_noalloc -- device, async; aatc_decode_attn without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: the partial records go to a static
 * array of AATC_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held until the process
 * ends; its device address is looked up once per device on the first call there (the current
 * device, which must be the one `stream` belongs to).
 *   Arguments, results and errors as aatc_decode_attn, minus the workspace.  A step whose
 *   records need more than AATC_NOALLOC_SCRATCH_BYTES (aatc_decode_attn_workspace_bytes) ->
 *   BUFFER_TOO_SMALL before anything is queued.
 *   Every call on one GPU uses that GPU's single array, so calls that may overlap in time on one
 *   GPU (different streams, or other threads) race; order them on one stream.  The array keeps
 *   the last call's records; nothing in it needs clearing between calls.
 */
#define AATC_NOALLOC_SCRATCH_BYTES (8u << 20)
aatc_status aatc_decode_attn_noalloc(const aatc_cache* cache, const void* q_dev, aatc_dtype q_dtype,
                                     int32_t n_q_heads, const int32_t* seq_lens_dev, int64_t max_seq_len,
                                     float softmax_scale, float* out_dev, float* lse_dev, void* stream);

/*
 * aatc_decode_attn_partial and aatc_decode_attn_merge -- the two halves of aatc_decode_attn,
 * launched by it back to back; called separately they let a caller time or overlap the halves,
 * or merge the partial states of several sequence shards.  [SPECTRA Abstract: the cache pass
 * is the bandwidth-bound part; the merge of split softmax states is the usual log-sum-exp
 * combination]
 *   _partial reads the packed cache once and writes, into workspace_dev, one partial record
 *   per (sequence split, q head): running max, sum of probabilities and the softmax-weighted
 *   V code sums of its tokens.  The record layout is internal to the library.
 *   _merge reads those records (written by _partial with the same cache, n_q_heads,
 *   seq_lens_dev and max_seq_len, earlier on the same stream or otherwise ordered before it)
 *   and writes out_dev / lse_dev exactly as aatc_decode_attn does.
 *   Arguments, ownership and errors as for aatc_decode_attn; each call validates them itself.
 */
aatc_status aatc_decode_attn_partial(const aatc_cache* cache, const void* q_dev, aatc_dtype q_dtype,
                                     int32_t n_q_heads, const int32_t* seq_lens_dev, int64_t max_seq_len,
                                     float softmax_scale, void* workspace_dev, size_t workspace_bytes,
                                     void* stream);
aatc_status aatc_decode_attn_merge(const aatc_cache* cache, int32_t n_q_heads,
                                   const int32_t* seq_lens_dev, int64_t max_seq_len, float* out_dev,
                                   float* lse_dev, void* workspace_dev, size_t workspace_bytes,
                                   void* stream);

/*
 * Token tiers.  [SPHERICAL KV page, RDKV abstract: bit widths from full precision down to
 * zero per token, by reverse water-filling once after prefill; AATC Key points: the output
 * distortion factors over tokens and channels]  Tiers are 0 (evicted), 2 and 4 (coded with
 * that many bits per element, same rotation, own water-filling) and 16 (raw bf16).
 *
 * aatc_tier_distortions -- host.  dist_out[j] for tiers {0,2,4,16}: sum over the n_tensors
 *   rotated variance vectors sigma2[n_tensors][d] (e.g. K and V of one head) of
 *   sum_i sigma2_i 4^-b_i(tau), b(tau) the water-filling at tau*d bits (aatc_calibrate's);
 *   dist_out[0] = total variance, dist_out[3] = 0.
 *   Errors: d != 128 -> UNSUPPORTED; max_bits outside 4..8 -> BUDGET; negative or non-finite
 *   variance -> NUMERICAL; null pointers -> INVALID_ARGUMENT.
 *
 * aatc_token_tiers -- host.  For n tokens with attention mass attn_mass[n] >= 0, the tier of
 *   each token minimising sum_t a_t^2 dist[tier_t] subject to sum_t tier_t * d <=
 *   avg_bits * n * d: per token argmin of a_t^2 dist[j] + lambda d tier_j (ties to the lower
 *   tier) with lambda bisected (200 steps) to the smallest value that fits the budget.
 *   tiers_out[n] receives 0, 2, 4 or 16.
 *   Errors: avg_bits outside [0, 16] -> BUDGET; negative or non-finite inputs -> NUMERICAL.
 */
aatc_status aatc_tier_distortions(const double* sigma2, int32_t n_tensors, int32_t d, int32_t max_bits,
                                  double dist_out[4]);
aatc_status aatc_token_tiers(const double* attn_mass, int64_t n, const double dist[4], int32_t d,
                             double avg_bits, int8_t* tiers_out);

/*
 * One segment of a KV head's tokens for aatc_decode_attn_segments: either a coded cache
 * (cache != NULL; its k_codes/v_codes hold this segment's tokens, compacted, under the
 * segment's own artefacts) or raw bf16 tokens in the original basis (cache == NULL;
 * k_raw/v_raw bf16 [batch][n_kv_heads][raw_capacity][128], 16-byte aligned).
 * seq_lens_dev: int32 [batch][n_kv_heads] tokens of this segment per (b,h), each <=
 * max_seq_len (NULL: max_seq_len everywhere); max_seq_len <= the segment's capacity.
 */
typedef struct {
  const aatc_cache* cache;
  const void* k_raw;
  const void* v_raw;
  int64_t raw_capacity;
  const int32_t* seq_lens_dev;
  int64_t max_seq_len;
} aatc_segment;

/* Workspace bytes of aatc_decode_attn_segments (0 for invalid arguments). */
size_t aatc_decode_attn_segments_workspace_bytes(const aatc_segment* segs, int32_t n_segs,
                                                 int32_t batch, int32_t n_kv_heads,
                                                 int32_t n_q_heads);

/*
 * aatc_decode_attn_segments -- device, async.  One decode step whose softmax runs over the
 * union of the segments' tokens (tier-0 tokens are in no segment).  [SPHERICAL KV page,
 * RDKV abstract; softmax is order-invariant, so the union is the log-sum-exp merge of
 * per-segment states]  Coded segments run the cache pass and merge of aatc_decode_attn with
 * per-(b,h) lengths; raw segments run the dense bf16 pass of aatc_decode_attn_dense in
 * token chunks of 2048, halved (down to 256) while fewer than 256 workgroups would run; one
 * final kernel merges all states.  q (16-byte aligned), out, lse, scale
 * and GQA mapping as aatc_decode_attn.
 *   Errors: as aatc_decode_attn, per segment; caches whose batch or n_kv_heads differ from the
 *   call, misaligned q -> INVALID_ARGUMENT; batch or n_kv_heads > 65535 -> UNSUPPORTED;
 *   workspace too small -> BUFFER_TOO_SMALL.
 */
aatc_status aatc_decode_attn_segments(const aatc_segment* segs, int32_t n_segs, int32_t batch,
                                      int32_t n_kv_heads, const float* q_dev, int32_t n_q_heads,
                                      float softmax_scale, float* out_dev, float* lse_dev,
                                      void* workspace_dev, size_t workspace_bytes, void* stream);

/* Workspace bytes of aatc_decode_attn_dense (0 for invalid arguments). */
size_t aatc_decode_attn_dense_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                              int64_t max_seq_len);

/*
 * aatc_decode_attn_dense -- device, async; one decode step of plain softmax attention over an
 * uncompressed bf16 cache, the full-precision baseline that the compressed cache is compared
 * with.  [SPHERICAL KV page, RDKV abstract: speedup over the full cache, which every decode
 * step reads from HBM again]
 *   k_dev, v_dev: bf16 [batch][n_kv_heads][capacity_tokens][128], 16-byte aligned, read only.
 *   seq_lens_dev: int32 [batch][n_kv_heads] visible tokens per (b,h) (each <= max_seq_len), or
 *   NULL for max_seq_len; max_seq_len <= capacity_tokens.  q_dev: fp32 [batch][n_q_heads][128],
 *   16-byte aligned; q head g reads KV head g / (n_q_heads/n_kv_heads), group 1..8.
 *   out_dev = sum_t softmax_t(scale q.k_t) v_t, fp32 [batch][n_q_heads][128]; lse_dev
 *   (nullable) the natural-log sum of exp of the scores; 0 visible tokens -> out 0, lse -inf.
 *   Scores use q as a bf16 high part plus a bf16 low part and the probabilities likewise, with
 *   fp32 accumulation; K and V enter exactly.
 *   workspace_dev: >= aatc_decode_attn_dense_workspace_bytes(...) bytes, 256-byte aligned, no
 *   initialisation needed; one state per token chunk (2048 tokens, or down to 256 when fewer
 *   than 256 workgroups would run) and q head.
 *   Errors: as aatc_decode_attn_segments with one raw segment.
 */
aatc_status aatc_decode_attn_dense(const void* k_dev, const void* v_dev, int32_t batch,
                                   int32_t n_kv_heads, int64_t capacity_tokens,
                                   const int32_t* seq_lens_dev, int64_t max_seq_len,
                                   const float* q_dev, int32_t n_q_heads, float softmax_scale,
                                   float* out_dev, float* lse_dev, void* workspace_dev,
                                   size_t workspace_bytes, void* stream);

/*
 * Measurement helper (not a step of the method).  aatc_probe_read -- device, async: reads
 * `bytes` of device memory at src once with 16-byte loads and writes one XOR digest per
 * workgroup to sink (aatc_probe_read_sink_bytes() bytes), so that the read bandwidth a plain
 * streaming kernel reaches on this GPU can be timed beside the decode-attention pass.
 *   Errors: null pointers, src or sink not 16-byte aligned, bytes 0 or not a multiple of 16 ->
 *   INVALID_ARGUMENT; launch -> HIP.
 */
#define AATC_PROBE_WORKGROUPS 2048
size_t aatc_probe_read_sink_bytes(void);
aatc_status aatc_probe_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AATC_H */
