/*
 * kvtc.h -- C ABI of the transform-coded KV-cache library (libkvtc.so), gfx950.
 *
 * The method (KVTC cache module page, veloxquant_mlx.cache.kvtc_cache, module
 * docstring "Design"; PALU cache API page, veloxquant_mlx.cache.palu_cache,
 * "Design"): a basis, a mean and a per-component bit allocation are fitted
 * once on the prefill rows of every unit and frozen.  A unit is one
 * (batch, head) pair, or one (batch, contiguous head group) whose heads share
 * one projection.  Append projects new rows through the frozen basis,
 * quantises every kept latent component at its frozen width (0 bits drops a
 * component) and packs the codes.  Fetch unpacks, dequantises and
 * reconstructs the whole stored sequence to fp16 [B, H, S, D].
 *
 * Conventions for every entry point:
 *   - all pointers are plain addresses; "host" pointers are CPU memory,
 *     "dev" pointers are device (HBM) memory of the current HIP device;
 *   - the caller owns every buffer; the library allocates no device memory
 *     and is reentrant; host scratch lives only for the duration of a call;
 *     its only process-wide state is the record of which kernels it has
 *     already allowed to use a CU's whole LDS (set once per kernel and device)
 *     and, for kvtc_attend_noalloc, one fixed scratch array per device and the
 *     record of its address;
 *   - device work is enqueued on the given hipStream_t (NULL = the null
 *     stream) and the call returns after the enqueue;
 *   - every argument is validated before anything is launched or written; a
 *     failing call returns a negative status and writes nothing;
 *   - no C++ exception crosses this interface.
 */
#ifndef KVTC_H
#define KVTC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define KVTC_OK          0
#define KVTC_E_CONFIG   -1  /* invalid or infeasible configuration (budget < 0: the
                               KVTC page's QuantizerConfigError in KVTCKVCache.__init__) */
#define KVTC_E_SHAPE    -2  /* shape, stride or alignment does not match the state */
#define KVTC_E_DTYPE    -3  /* unsupported element type */
#define KVTC_E_CAPACITY -4  /* rows outside [0, capacity) */
#define KVTC_E_STATE    -5  /* state blob missing, unfitted or corrupt */
#define KVTC_E_BUFSIZE  -6  /* output buffer too small (the size needed is returned) */
#define KVTC_E_DEVICE   -7  /* HIP launch or runtime error */
#define KVTC_E_ARG      -8  /* NULL pointer or out-of-range scalar argument */

#define KVTC_F32 0
#define KVTC_F16 1

/* KVTC_MODE_DP: one unit per (batch, head); per-unit DP bit allocation under a
 *   bits-per-token budget, per-component frozen (min, scale) (KVTC page).
 * KVTC_MODE_MIXED: one unit per (batch, group of heads_per_unit contiguous
 *   heads) sharing one projection; the leading hi_fraction of components at
 *   hi_bits, the rest at lo_bits; per-token (min, scale) in fp16 for every
 *   group_size consecutive components (PALU page, palu_* parameters). */
#define KVTC_MODE_DP    0
#define KVTC_MODE_MIXED 1

#define KVTC_MAX_CHOICES 8

/* Configuration; kvtc_config_default() fills the documented defaults
 * (KVTC page, KVTCKVCache.__init__; PALU page, PALUKVCache parameters). */
typedef struct kvtc_config {
    int32_t mode;              /* KVTC_MODE_DP or KVTC_MODE_MIXED */
    int32_t head_dim;          /* D; the device path needs D % 64 == 0 */
    int32_t heads_per_unit;    /* 1 in DP mode; the head-group size in mixed mode */
    int32_t rank;              /* > 0: kept components per unit (<= heads_per_unit*D);
                                  0: smallest rank reaching energy_threshold */
    double  energy_threshold;  /* default 0.90 */
    int32_t bit_budget;        /* DP: code bits per token per unit, >= 0; default 4*D */
    int32_t n_choices;         /* DP: allowed widths, a subset of {0,1,2,3,4,8} */
    int32_t choices[KVTC_MAX_CHOICES];
    double  beta;              /* DP distortion-proxy constant, default 1.0 */
    int32_t hi_bits;           /* mixed: default 4 */
    int32_t lo_bits;           /* mixed: default 2 */
    int32_t group_size;        /* mixed: components per (min, scale) pair, default 32,
                                  must be a multiple of 16 */
    double  hi_fraction;       /* mixed: default 0.25 */
} kvtc_config;

/* ------------------------------------------------------------ state blob */
/* The frozen state of one tensor (K or V) is one position-independent blob:
 * this header followed by 256-byte aligned sections at the given offsets.
 * The host copy and the device copy hold the same bytes.  "slot" j of a unit
 * is its j-th stored component: in DP mode the j-th component with a
 * non-zero width (index order), in mixed mode component j. */
#define KVTC_MAGIC   0x4354564Bu  /* "KVTC" little-endian */
#define KVTC_VERSION 1u

typedef struct kvtc_unit_info {
    int32_t rank;        /* kept components (DP: before dropping 0-bit ones) */
    int32_t n_slots;     /* stored components */
    int32_t row_bits;    /* code bits per token */
    int32_t reserved;
} kvtc_unit_info;

typedef struct kvtc_state_header {
    uint32_t magic, version;
    int32_t  mode, head_dim, heads_per_unit, dg;   /* dg = heads_per_unit * head_dim */
    int64_t  batch, heads, units;                  /* units = batch*heads/heads_per_unit */
    int32_t  rmax;          /* widest kept rank over units */
    int32_t  kslots;        /* slot capacity per unit: max n_slots rounded up to 16 (>= 16) */
    int32_t  row_stride;    /* bytes per stored code row: 4 * ceil(max row_bits / 32) */
    int32_t  n_qgroups;     /* mixed: (min, scale) pairs per token; 0 in DP mode */
    int32_t  group_size, hi_bits, lo_bits, n_hi;
    int32_t  bit_budget, n_choices;
    int32_t  choices[KVTC_MAX_CHOICES];
    double   beta;
    double   energy_threshold;
    int32_t  rank_cfg;      /* configured rank (0 = energy threshold) */
    int32_t  kfetch;        /* fetch contraction length: runs of equal widths among the
                               stored slots, each padded to a multiple of 16 slots */
    int64_t  s_prefill;     /* rows the state was fitted on (0 if built from parts) */
    /* per-unit sections */
    uint64_t off_unit;      /* kvtc_unit_info [units] */
    uint64_t off_lambda;    /* double [units][dg]   eigenvalues, descending (0 if unknown) */
    uint64_t off_bits;      /* uint8  [units][rmax] width of component i (0 = dropped) */
    uint64_t off_qmin;      /* float  [units][rmax] DP frozen min of component i */
    uint64_t off_qscale;    /* float  [units][rmax] DP frozen scale of component i */
    uint64_t off_mu;        /* float  [units][dg]   mean */
    uint64_t off_slot_comp; /* int32  [units][kslots] component index of slot j (-1 = empty) */
    uint64_t off_slot_bits; /* uint32 [units][kslots] bit offset in the row | width << 24 */
    uint64_t off_basis;     /* float  [units][kslots][dg] basis vector of slot j (0 = empty) */
    uint64_t off_qlo;       /* double [units][kslots] DP: min of slot j, as stored (fp32 value) */
    uint64_t off_qinv;      /* double [units][kslots] DP: 1/scale of slot j (0 if scale is 0) */
    uint64_t off_w16;       /* half   [units][dg][kfetch] fetch operand in k-step order: DP
                               scale_j*basis_j, mixed basis_j, rounded to fp16, 0 for padding;
                               within each 8-slot half of a 4-bit k-step the slots are stored
                               in the order 0,2,4,6,1,3,5,7; a 2-bit k-step stores its slots in
                               the order 0,4,8,12,1,5,9,13,2,6,10,14,3,7,11,15 */
    uint64_t off_bias;      /* float  [units][dg] fetch bias: DP mu + sum_j min_j*basis_j,
                               mixed mu */
    uint64_t total_bytes;
    uint64_t off_kdesc;     /* uint32 [units][kfetch/16] fetch k-step t (k = 16t..16t+15): bit
                               offset of its first field (bits 0-15) | width of all its fields
                               (16-19, 0 = empty) | quantisation group (20-31, mixed mode) */
    uint64_t off_fslot;     /* int32  [units][kfetch] stored slot whose fetch operand is column k
                               of off_w16 (-1 = padding column) */
    uint64_t off_vdig;      /* int8   [units][5][kslots][dg] the basis in exact integer digits for
                               the int8 append: vq = rint(basis * 2^38) = sum_i d_i 256^i with
                               balanced digits d_i in [-128, 127]; 0 (absent) when some basis
                               entry exceeds 1 in magnitude */
    uint64_t off_mv;        /* double [units][kslots] the int8 append's slot offset: mean . basis_j
                               - 2^-62 * 0x808080 * sum_d vq_jd, in float64 (0 when off_vdig is) */
} kvtc_state_header;

/* ---------------------------------------------------------- entry points */

/* Fill *cfg with the defaults of the given mode and head dimension. */
void kvtc_config_default(kvtc_config *cfg, int32_t mode, int32_t head_dim);

/* Identity of this build: the first 16 hex digits of the SHA-256 over the
 * library's source files, fixed at compile time (static string).  A caller can
 * compare it with the hash of the sources it expects, to refuse a stale build. */
const char *kvtc_build_id(void);

/* Human-readable name of a status code (static string). */
const char *kvtc_status_string(int32_t status);

/* HIP's message for the error behind the calling thread's last KVTC_E_DEVICE
 * (a launch HIP refused, or a failed device call); "no error" if there was none.
 * Static string. */
const char *kvtc_device_error_string(void);

/* Fit the frozen state of one tensor on its prefill rows (host).
 * KVTC page, update_and_fetch and _TensorKVTC.fit_prefill_from_pca: local PCA
 * per unit on the prefill batch, then the DP bit allocation, then the
 * per-component ranges; PALU page "Design" steps 1-2 for mixed mode.
 *   rows_host   contiguous [B, H, S, D] host rows, dtype KVTC_F32 or KVTC_F16
 *   S           prefill rows, >= 2 (the KVTC page fits on the first call with S > 1)
 *   state_out   host buffer of *state_bytes bytes, or NULL to query the size
 *   state_bytes in: capacity of state_out; out: bytes needed / written
 * Returns KVTC_E_CONFIG for an invalid or infeasible configuration,
 * KVTC_E_BUFSIZE (with *state_bytes set) if state_out is too small. */
int32_t kvtc_fit_host(const kvtc_config *cfg, const void *rows_host, int32_t dtype,
                      int64_t B, int64_t H, int64_t S,
                      void *state_out, size_t *state_bytes);

/* Bytes that suffice for the state blob of any fit of this configuration and
 * shape (host, no fitting): a caller can allocate this much, fit once and keep
 * the first *state_bytes bytes the fit reports. */
int32_t kvtc_fit_bytes_bound(const kvtc_config *cfg, int64_t B, int64_t H, size_t *bytes);

/* Device workspace kvtc_fit_device needs for S prefill rows (per unit: the
 * mean, its partial sums and the covariance in float64; per unit and slot: the
 * basis and the range keys of the range pass). */
int32_t kvtc_fit_workspace(const kvtc_config *cfg, int64_t B, int64_t H, int64_t S, size_t *bytes);

/* The fit of kvtc_fit_host from rows already on the device (device + host).
 * KVTC page, update_and_fetch: the local PCA of every unit is fitted in one
 * batched call on the prefill (the page's batched SVD fit), then the DP
 * allocation and the per-component ranges.  The mean and the centred
 * covariance of every unit (float64 MFMA) and the min/max of every kept
 * component's latents over the prefill rows run on the device; the
 * eigen-decomposition, rank and DP allocation run on the host.  The call waits
 * for its stream and returns the host blob.
 *   rows_dev    [B, H, S, D] device rows of dtype, element strides (strides[3] == 1)
 *   work_dev    device workspace of kvtc_fit_workspace() bytes, 256-byte aligned
 *   state_out, state_bytes   as for kvtc_fit_host
 * The result equals kvtc_fit_host's up to the order of float64 summation (the
 * mean exactly for fp16 rows; eigenvalues, fp32 basis and ranges to their last
 * rounding).  D % 64 == 0, at most 65535 units, and in DP mode the configured
 * rank (or D) at most 256; KVTC_E_BUFSIZE for a missing or short workspace. */
int32_t kvtc_fit_device(const kvtc_config *cfg, const void *rows_dev, int32_t dtype, const int64_t strides[4],
                        int64_t B, int64_t H, int64_t S, void *work_dev, size_t work_bytes,
                        void *state_out, size_t *state_bytes, void *hip_stream);

/* Build a state blob from an already fitted frozen state (host), for example a
 * basis calibrated elsewhere.  Arrays are host memory, unit-major:
 *   ranks   int32 [U]           kept components per unit (1..rmax)
 *   mu      float [U][dg]
 *   basis   float [U][rmax][dg] component i's basis vector in row i
 *   lambda  double [U][dg] or NULL
 *   bits    uint8 [U][rmax]     widths in {0,1,2,3,4,8} (DP) -- ignored in mixed
 *                               mode, where the hi/lo rule of cfg decides them
 *   qmin, qscale float [U][rmax] DP frozen (min, scale) -- NULL in mixed mode
 * U = B*H/heads_per_unit, dg = heads_per_unit*head_dim. */
int32_t kvtc_state_build(const kvtc_config *cfg, int64_t B, int64_t H, int32_t rmax,
                         const int32_t *ranks, const float *mu, const float *basis,
                         const double *lambda, const uint8_t *bits,
                         const float *qmin, const float *qscale, int64_t s_prefill,
                         void *state_out, size_t *state_bytes);

/* DP bit allocation alone (host): minimise sum_i D_i(b_i) subject to
 * sum_i b_i <= budget, b_i in choices, with D_i(0) = lambda_i and
 * D_i(b) = beta * lambda_i * 4^-b (KVTC page: DP-optimal discrete allocation
 * over an analytic distortion proxy; a component may get 0 bits).  Narrower
 * widths and fewer total bits win ties.  bits_out: uint8 [r]. */
int32_t kvtc_allocate_bits(const double *lambda, int32_t r, int32_t budget,
                           const int32_t *choices, int32_t n_choices, double beta,
                           uint8_t *bits_out);

/* Bytes of the device code store and of the mixed-mode parameter store for a
 * given capacity (rows per unit).  Layouts:
 *   codes  uint8 [units][capacity][row_stride], little-endian bit stream per row,
 *          slot j's code at bit offset (slot_bits & 0xFFFFFF), LSB first
 *   params fp16  [units][capacity][n_qgroups][2] = (min, scale)   (mixed only) */
int32_t kvtc_store_bytes(const void *state_host, int64_t capacity,
                         size_t *codes_bytes, size_t *params_bytes);

/* Append rows [s0, s0 + n) of every unit (device).
 * KVTC page "Design", decode step 1: project through the frozen basis,
 * quantise at the frozen widths, grow the latent store.  PALU page "Design",
 * decode steps 1-2 for mixed mode.
 *   state_host/state_dev  the same blob in host and device memory
 *   x_dev      [B, H, n, D] rows of dtype KVTC_F16 or KVTC_F32; x_strides are in
 *              elements for (b, h, s, d) and x_strides[3] must be 1
 *   codes_dev  code store (layout above), params_dev the mixed-mode store (NULL in DP)
 * Codes are computed from float64 latents, so a row's codes depend only on
 * that row: appending one token at a time or all at once stores the same bytes.
 * Needs s0 >= 0, n >= 0, s0 + n <= capacity. */
int32_t kvtc_append(const void *state_host, const void *state_dev,
                    const void *x_dev, int32_t dtype, const int64_t x_strides[4],
                    int64_t B, int64_t H, int64_t n, int64_t s0,
                    void *codes_dev, void *params_dev, int64_t capacity, void *hip_stream);

/* Reconstruct rows [s_begin, s_end) of every unit to fp16 (device).
 * KVTC page "Design": every call returns reconstructed fp16 [B, H, S_total, D];
 * PALU page: latent -> dequant -> reconstruct on every fetch.
 *   out_dev    fp16 [B, H, s_end - s_begin, D] with element strides out_strides
 *              (out_strides[3] must be 1, rows 16-byte aligned); row s of the
 *              store goes to out index s - s_begin.
 * Needs 0 <= s_begin <= s_end <= capacity.  KVTC_E_SHAPE for head_dim not a
 * multiple of 64 or more than 256 fetch slots, and where a stored row and its
 * group-head parameters exceed 192 bytes (the 32-row tile the kernels stage in
 * registers; appending and entropy coding take rows up to 256 bytes). */
int32_t kvtc_fetch(const void *state_host, const void *state_dev,
                   const void *codes_dev, const void *params_dev, int64_t capacity,
                   int64_t s_begin, int64_t s_end,
                   void *out_dev, const int64_t out_strides[4], void *hip_stream);

/* One tensor's operands in a paired call (kvtc_append_kv, kvtc_fetch_kv).
 *   state_host/state_dev  the tensor's blob in host and device memory
 *   codes_dev, params_dev its stores (params_dev NULL in DP mode), of `capacity` rows
 *   rows_dev   append: the input rows x [B, H, n, D] (read only), of element type dtype;
 *              fetch: the fp16 output [B, H, s_end - s_begin, D] (dtype is ignored)
 *   strides    element strides of rows_dev for (b, h, s, d); strides[3] must be 1 */
typedef struct kvtc_tensor_ref {
    const void *state_host;
    const void *state_dev;
    void *codes_dev;
    void *params_dev;
    int64_t capacity;
    void *rows_dev;
    int32_t dtype;
    int32_t reserved;
    int64_t strides[4];
} kvtc_tensor_ref;

/* Append the same rows [s0, s0 + n) to the key and the value tensor of a layer
 * in one call (device).  The KVTC page's update_and_fetch takes the new keys
 * and values together and the KVTC cache holds one _TensorKVTC for each; this
 * entry point does what kvtc_append does for k and then for v, with the same
 * arguments, arithmetic, results and errors.  Decode appends (n <= 16) of two
 * DP tensors with the same element type and unit width run as one launch;
 * anything else as one launch per tensor.  Both tensors are validated before
 * anything is launched. */
int32_t kvtc_append_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v,
                       int64_t B, int64_t H, int64_t n, int64_t s0, void *hip_stream);

/* Reconstruct rows [s_begin, s_end) of the key and the value tensor of a layer
 * in one call (device): the KVTC page's update_and_fetch returns the whole
 * reconstructed keys and values of every call.  Same results and errors as
 * kvtc_fetch for k and then for v.  Two tensors of the same mode and head size
 * run as one launch whose blocks cover both; otherwise one launch each.  Both
 * tensors are validated before anything is launched. */
int32_t kvtc_fetch_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v,
                      int64_t s_begin, int64_t s_end, void *hip_stream);

/* Bytes of device workspace kvtc_attend needs for rows [0, s_end) of the given
 * key and value states: partial softmax statistics per unit and segment when
 * the rows take two or more segments (segments of at most 9216 rows, at least
 * 256 unless the cache is shorter, enough of them to give the device about 512
 * blocks); 0 when every unit's rows fit one segment.  kvtc_attend_gqa's general
 * path (grouped query heads, group-head caches) has its own figure. */
int32_t kvtc_attend_workspace(const void *k_state_host, const void *v_state_host, int64_t s_end,
                              size_t *bytes);

/* kvtc_attend with Hq = q_heads query heads, a multiple G of the stored heads H
 * (grouped-query attention: query head hq attends KV head hq / G, consecutive
 * query heads sharing one; the Llama-3-8B-like layer has 32 query heads over 8
 * KV heads).  q_dev [B, Hq, D], out_dev fp16 [B, Hq, D]; the other arguments,
 * the arithmetic and the errors as for kvtc_attend.  Both kvtc_attend and this
 * call serve per-head (DP) and group-head caches: for a group-head cache the
 * (min, scale) of each token and quantisation group enter the scores through
 * per-group code sums and the value sums through the dequantised latents.
 * The queries per unit (G times heads_per_unit) are at most 32. */
int32_t kvtc_attend_gqa_workspace(const void *k_state_host, const void *v_state_host, int64_t q_heads, int64_t s_end,
                                  size_t *bytes);
int32_t kvtc_attend_gqa(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t q_heads, const void *q_dev,
                        int32_t q_dtype, const int64_t q_strides[3], int64_t s_end, void *out_dev,
                        const int64_t out_strides[3], void *work_dev, size_t work_bytes, void *hip_stream);

/* Decode attention over the stored rows [0, s_end) of a key and a value tensor,
 * computed from their codes without reconstructing keys or values (device).
 * TurboQuant cache module page, attend: one query per head is scored against
 * every stored key, the scores are divided by sqrt(D), softmax-weighted over the
 * stored rows, and the decoded values are summed with those weights; an empty
 * cache gives zeros.  PALU cache API page, "Design": latents are reconstructed
 * only for attention.  Per (b, h): out = sum_s p_s xv_s with
 * p = softmax(q . xk_s / sqrt(D)), where xk_s, xv_s are the rows kvtc_fetch
 * would reconstruct (before their fp16 rounding); evaluated in fp32 through the
 * latent space: q is projected onto the key basis once, every stored key code
 * is weighted by it, and the softmax-weighted value codes are reconstructed
 * once per (b, h).
 *   k, v        tensors with the same B, H, D (D <= 256) and heads per unit,
 *               per-head (DP) or group-head; their rows_dev, dtype and strides
 *               are not used (params_dev is, for a group-head tensor)
 *   q_dev       queries [B, H, D] of dtype q_dtype (KVTC_F16 or KVTC_F32), element
 *               strides q_strides for (b, h, d), q_strides[2] == 1
 *   out_dev     fp16 [B, H, D] with element strides out_strides, out_strides[2] == 1
 *   work_dev    device workspace of at least kvtc_attend_workspace() bytes,
 *               256-byte aligned, owned by the caller (contents are scratch);
 *               may be NULL when that size is 0
 * Needs 0 <= s_end <= both capacities; KVTC_E_SHAPE for tensors of different
 * shapes, KVTC_E_BUFSIZE for a missing or short workspace. */
int32_t kvtc_attend(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v,
                    const void *q_dev, int32_t q_dtype, const int64_t q_strides[3], int64_t s_end,
                    void *out_dev, const int64_t out_strides[3],
                    void *work_dev, size_t work_bytes, void *hip_stream);

/* ----------------------------------------------------------- measurement
 * Traffic probe of kvtc_fetch_kv (device): not part of the method.  Same
 * arguments, validation and launch plan (blocks, waves, pairing) as
 * kvtc_fetch_kv, and the same memory traffic -- every block reads its W slice
 * and bias, every tile's code rows (and params) are read and its output rows
 * written with 16-byte non-temporal stores -- but nothing is decoded or
 * contracted and no store waits for a load.  Its rate is the practical
 * ceiling of the fetch's traffic, the reference the fetch kernel is measured
 * against.  The output rows receive placeholder values, not a reconstruction. */
int32_t kvtc_fetch_kv_probe(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t s_begin, int64_t s_end,
                            void *hip_stream);

/* ------------------------------------------------------------ refit mode
 * KVTC cache module page, _TensorKVTC.append and _requantize: every call joins
 * the new rows to all rows accumulated so far, re-projects them through the
 * frozen basis and mean, and quantises each kept component with a min/max
 * fitted over all of them; the basis, mean and widths never change, the
 * per-component (min, scale) and every stored code follow the accumulated
 * sequence.  (kvtc_append instead keeps the prefill ranges frozen and clamps.)
 * DP-mode tensors only (group-head rows carry per-token ranges already);
 * KVTC_E_STATE otherwise.
 *
 * Buffers, owned by the caller, all device memory:
 *   latents_dev  double [units][capacity][kslots]: the fp64 latents of every
 *                appended row (computed once per row; a row's latents never
 *                change under the frozen basis), 8-byte aligned
 *   refit_dev    256-byte aligned, of the size kvtc_refit_bytes returns; its
 *                sections, each 256-byte aligned, in this order:
 *                  qmin32, qscale32  float  [units][kslots] the refitted min and
 *                                    scale of slot j (fp32 of the float64 min and
 *                                    of (max - min) / (2^b - 1); scale 0 for a
 *                                    constant component)
 *                  qlo, qinv         double [units][kslots] the quantiser's min and 1/scale
 *                  w16               half   [units][dg][kfetch] fetch operand, laid
 *                                    out as the blob's off_w16 section
 *                  bias              float  [units][dg] fetch bias (as off_bias)
 *                  part              double [units][chunks][kslots][2] scratch, with
 *                                    chunks = clamp(ceil(capacity / 256), 1, 256)
 */
int32_t kvtc_refit_bytes(const void *state_host, int64_t capacity, size_t *latent_bytes, size_t *refit_bytes);

/* Refit-mode append (device): the latents of rows x [B, H, n, D] go to rows
 * [s0, s0 + n) of the latent store; then every kept component's range is
 * refitted over rows [0, s0 + n) of the store (the accumulated sequence; rows
 * past it are ignored, so lowering s0 + n is the page's trim), refit_dev's
 * quantiser and fetch operands are rewritten, and the codes of every row
 * [0, s0 + n) are re-quantised and re-packed into codes_dev (layout as for
 * kvtc_append).  n = 0 refits the first s0 rows.  Arguments and errors as for
 * kvtc_append; a row's latents and codes depend only on the rows accumulated,
 * not on how they arrived. */
int32_t kvtc_append_refit(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                          const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0,
                          void *latents_dev, void *codes_dev, void *refit_dev, int64_t capacity, void *hip_stream);

/* Refit-mode fetch (device): kvtc_fetch of rows [s_begin, s_end) dequantised
 * with the ranges of the last kvtc_append_refit (refit_dev's fetch operands).
 * Arguments and errors as for kvtc_fetch. */
int32_t kvtc_fetch_refit(const void *state_host, const void *state_dev, const void *codes_dev,
                         const void *refit_dev, int64_t capacity, int64_t s_begin, int64_t s_end,
                         void *out_dev, const int64_t out_strides[4], void *hip_stream);

/* kvtc_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same validation, kernels and results as kvtc_attend, with the workspace taken
 * from a fixed scratch array of KVTC_ATTEND_SCRATCH_BYTES that the library holds
 * on every device that loads it until the process ends (its address is looked
 * up once per device, on the first call).  Nothing is allocated.  Returns
 * KVTC_E_BUFSIZE, before anything is launched, when the call needs more than
 * KVTC_ATTEND_SCRATCH_BYTES (kvtc_attend_workspace tells the need).  Every call
 * on a device shares that device's scratch: calls that overlap on one device
 * race and must be ordered by the caller (for instance on one stream).  The
 * scratch needs no clearing: every word a call reads was written by that call. */
#define KVTC_ATTEND_SCRATCH_BYTES (16u << 20)
int32_t kvtc_attend_noalloc(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                            const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                            void *hip_stream);

/* ------------------------------------------------------- entropy-coded storage
 * KVTC page, "Byte accounting" (and _encode_survived_codes): the stored latents
 * are order-0 Huffman coded per kept component, and a fixed-width packing is
 * kept instead whenever coding does not pay.  kvtc_entropy_encode turns the
 * first S rows of a DP tensor's code store into that storage, an archive in
 * device memory; kvtc_entropy_decode restores the fixed-width rows from it,
 * bit for bit, for kvtc_fetch.  Per unit, in unit order, byte aligned, the
 * archive holds
 *   coded (when stream + table < fixed width): the table -- for each stored
 *     slot in order, 2^b bytes, byte k the code length of symbol k (0 if
 *     absent) -- then the stream: for each slot in order, the canonical prefix
 *     code of every row's code in row order, most significant code bit first,
 *     stream bit p being bit p % 8 of byte p / 8;
 *   fixed width: the rows' bits back to back (row s at bits [s*rb, (s+1)*rb)
 *     of the unit's part), ceil(S * rb / 8) bytes.
 * So the archive is exactly kvtc_bytes' stored_payload + entropy_table.  The
 * canonical code of given lengths orders the symbols by (length, value) and
 * gives them consecutive code values, doubling at every length step.  Code
 * lengths come from a Huffman tree on the slot's code counts (ties broken
 * towards lower weight, then lower node index), at most 32 bits.
 *
 * The index (host blob, and a device copy for decoding) records what a
 * parallel decoder needs besides the archive: per unit the part's offset, size
 * and form; per slot the canonical decode table; per slot and chunk of
 * chunk_rows rows the bit position of the chunk's first code.  It is not part
 * of the stored bytes the pages count (it is recomputable from the archive). */
#define KVTC_ENTROPY_MAGIC   0x4554564Bu  /* "KVTE" little-endian */
#define KVTC_ENTROPY_VERSION 1u
#define KVTC_ENTROPY_MAX_LEN 32

typedef struct kvtc_entropy_unit {
    uint64_t offset;         /* byte offset of the unit's part in the archive */
    uint64_t bytes;          /* size of the part */
    uint32_t coded;          /* 1: table + stream, 0: fixed width */
    uint32_t table_bytes;    /* sum of 2^b over the unit's slots (the table, when coded) */
} kvtc_entropy_unit;

typedef struct kvtc_entropy_dec {
    uint32_t first[KVTC_ENTROPY_MAX_LEN + 1];   /* first canonical code of each length */
    uint16_t count[KVTC_ENTROPY_MAX_LEN + 1];   /* symbols of each length */
    uint16_t base[KVTC_ENTROPY_MAX_LEN + 1];    /* index of the first symbol of each length */
    uint32_t sym_off;                           /* offset of the slot's sorted symbols in off_syms */
    uint32_t max_len;
} kvtc_entropy_dec;

typedef struct kvtc_entropy_header {
    uint32_t magic, version;
    int64_t  S;              /* rows covered */
    int64_t  units;
    int32_t  kslots;         /* as the state's */
    int32_t  chunk_rows;     /* rows per decode chunk */
    int32_t  nchunks;        /* ceil(S / chunk_rows) */
    int32_t  nsym;           /* symbol positions per unit: the largest sum of 2^b over a unit's slots */
    uint64_t archive_bytes;  /* stored_payload + entropy_table of kvtc_bytes */
    uint64_t payload_bytes;  /* coded streams and fixed-width parts */
    uint64_t table_bytes;    /* tables of the coded units */
    int64_t  units_coded;
    uint64_t off_unit;       /* kvtc_entropy_unit [units] */
    uint64_t off_dec;        /* kvtc_entropy_dec [units][kslots] */
    uint64_t off_syms;       /* uint8 [units][nsym]: each slot's symbols sorted by (length, value) */
    uint64_t off_chunk;      /* uint64 [units][kslots][nchunks]: archive bit position of each chunk's first code */
    uint64_t total_bytes;
} kvtc_entropy_header;

/* Sizes (host): the device workspace kvtc_entropy_encode needs, a bound on the
 * archive (the fixed-width total; an archive is never larger) and the index. */
int32_t kvtc_entropy_bytes(const void *state_host, int64_t S, size_t *work_bytes, size_t *archive_bytes,
                           size_t *index_bytes);

/* Encode rows [0, S) of a DP tensor's device code store (device + host; waits
 * for its stream): code counts per slot on the device, code lengths and
 * canonical tables on the host, the archive written on the device.
 *   codes_dev     the code store of `capacity` rows (layout of kvtc_append)
 *   work_dev      workspace of kvtc_entropy_bytes() bytes, 256-byte aligned
 *   archive_dev   archive_bytes >= the bound, 4-byte aligned; on return its
 *                 first header.archive_bytes bytes are the archive
 *   index_host    index_bytes >= kvtc_entropy_bytes()'s, receives the index
 * KVTC_E_STATE for a group-head tensor; KVTC_E_SHAPE if a code would be longer
 * than KVTC_ENTROPY_MAX_LEN bits (needs more than ~3.5 million rows). */
int32_t kvtc_entropy_encode(const void *state_host, const void *state_dev, const void *codes_dev, int64_t capacity,
                            int64_t S, void *work_dev, size_t work_bytes, void *archive_dev, size_t archive_bytes,
                            void *index_host, size_t index_bytes, void *hip_stream);

/* Decode an archive back into rows [0, S) of a code store (device, enqueued on
 * the stream): the rows come back bit-identical to the encoded ones.
 *   index_host/index_dev  the index kvtc_entropy_encode returned, on host and
 *                         device (same bytes; the device copy 16-byte aligned) */
int32_t kvtc_entropy_decode(const void *state_host, const void *state_dev, const void *index_host,
                            const void *index_dev, const void *archive_dev, void *codes_dev, int64_t capacity,
                            void *hip_stream);

/* Storage accounting of one tensor over its first S rows (host).
 * KVTC page "Byte accounting" and the kvtc_bytes / pre_entropy_bytes
 * properties: order-0 Huffman per kept DP component, kept only when payload +
 * table is below fixed-width packing; basis and quantiser parameters counted
 * at fp16.  PALU page "Byte accounting": mixed-bit latents + fp32 projection. */
typedef struct kvtc_bytes_report {
    uint64_t fixed_payload;       /* sum over units of ceil(S * row_bits / 8) */
    uint64_t entropy_payload;     /* Huffman payload of entropy-coded units */
    uint64_t entropy_table;       /* one byte per symbol of each coded component */
    uint64_t stored_payload;      /* payload counted in total (coded or fixed) */
    uint64_t basis;               /* DP: fp16 basis + mean; mixed: fp32 projection + mean */
    uint64_t quant_params;        /* DP: fp16 (min, scale) per component; mixed: per token-group */
    uint64_t total;               /* stored_payload + entropy_table + basis + quant_params */
    uint64_t pre_entropy;         /* fixed_payload + basis + quant_params */
    uint64_t fp16_equiv;          /* B * H * S * D * 2 */
    uint64_t device_store;        /* units * S * row_stride (+ params) actually held on device */
    int64_t  n_survived;          /* kept non-zero-width components over units */
    int64_t  units_entropy_coded;
} kvtc_bytes_report;

/*   codes_host   [units][capacity][row_stride] copy of the device store
 *   params_host  mixed-mode parameter store copy (NULL in DP mode) */
int32_t kvtc_bytes(const void *state_host, const void *codes_host, const void *params_host,
                   int64_t capacity, int64_t S, kvtc_bytes_report *out);

#ifdef __cplusplus
}
#endif
#endif /* KVTC_H */
