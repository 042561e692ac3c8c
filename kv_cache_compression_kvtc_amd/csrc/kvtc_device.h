// Shared declarations of the device half of libkvtc (gfx950): element types,
// kernel argument blocks, the field decoder shared by the fetch and attention
// kernels, and the launchers each translation unit provides.  Not part of the
// public interface.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kvtc.h"
#include "kvtc_internal.h"

namespace kvtc {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;        // 4 waves of 64
constexpr int kAppTok = 64;          // tokens per append block (16 per wave)
constexpr int kAppKC = 16;           // feature columns staged per append step
constexpr int kAppPad = kAppKC + 1;  // LDS row pitch (elements) of the staged chunks
constexpr int kFetTok = 32;          // tokens per fetch tile (one wave)
constexpr int kFetchRegWords = 24;   // per-lane register staging of one tile's rows+params
constexpr int kMaxSlots = 256;
constexpr int kMaxRowStride = 256;
constexpr int kFetchBlocks = 512;    // target block count of a fetch (one block per unit at the batched-decode shape)

// ------------------------------------------------------------ small helpers
// Nearest-even binary16 of a double from its value: the binade is read from
// the exponent bits, power-of-two scalings are exact and rint rounds half to even.
__device__ inline uint16_t half_bits_rne(double x) {
    const uint64_t bits = __double_as_longlong(x);
    const uint16_t sign = static_cast<uint16_t>((bits >> 48) & 0x8000u);
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
    if (mag > 0x7FF0000000000000ull) return sign | 0x7E00u;
    const double a = __longlong_as_double(mag);
    if (a >= 65520.0) return sign | 0x7C00u;
    if (a < 6.103515625e-05) return sign | static_cast<uint16_t>(__builtin_rint(a * 16777216.0));
    int ex = static_cast<int>(mag >> 52) - 1023;
    double q = __builtin_rint(__builtin_amdgcn_ldexp(a, 10 - ex));
    if (q == 2048.0) {
        q = 1024.0;
        ++ex;
    }
    if (ex + 15 >= 31) return sign | 0x7C00u;
    return sign | static_cast<uint16_t>(((ex + 15) << 10) | (static_cast<int>(q) - 1024));
}

__device__ inline double half_bits_to_double(uint16_t h) {
    return static_cast<double>(__builtin_bit_cast(_Float16, h));
}

// An unsigned integer whose order is the order of the double x (for atomic
// min/max of doubles): negative values bit-inverted, others with the sign bit set.
__device__ inline unsigned long long order_key(double x) {
    const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(x));
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// ORs a width-w code into an LSB-first bit row held as 32-bit words in LDS.
__device__ inline void or_field(uint32_t *row, uint32_t off, uint32_t w, uint32_t c) {
    const uint32_t wi = off >> 5, sh = off & 31u;
    atomicOr(&row[wi], c << sh);
    if (sh + w > 32u) atomicOr(&row[wi + 1], c >> (32u - sh));
}

__device__ inline double quantise(double l, double lo, double inv, double cmax) {
    double q = __builtin_rint((l - lo) * inv);
    if (q != q) q = 0.0;
    return fmin(fmax(q, 0.0), cmax);
}

template <typename XT>
__device__ inline double load_x(const XT *p) {
    return static_cast<double>(*p);
}


// ================================================================ append
struct AppendArgs {
    const void *x;
    int64_t xsb, xsh, xss;             // element strides of x (d stride is 1)
    int64_t n, s0, capacity;
    const kvtc_unit_info *ui;
    const float *mu;                   // [U][dg]
    const float *basis;                // [U][kslots][dg]
    const double *qlo, *qinv;          // [U][kslots]
    const uint32_t *sbits;             // [U][kslots]
    uint8_t *codes;                    // [U][capacity][row_stride]
    uint32_t *params;                  // [U][capacity][n_qg] packed (min16 | scale16 << 16)
    double *lat;                       // refit mode: latents [U][capacity][kslots] (else unused)
    unsigned long long *keys;          // device fit: per-slot (min, max) order keys [U][kslots][2]
    int dg, D, hpu, groups, kslots, row_stride, n_qg, gs;
    float inv_dg, inv_q4;              // 1/dg and 4/dg: exact quotients of small indices
    int x_vec;                         // rows and strides aligned to 4 elements (raw vector loads)
    const int8_t *vdig;                // int8 append: basis digits [U][5][kslots][dg] (null if absent)
    const double *mv;                  // int8 append: mean . basis_j [U][kslots]
};

// Four consecutive input elements as raw bits (one 8- or 16-byte load), and
// element i of them as a double.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename XT>
struct RawX4;
template <>
struct RawX4<_Float16> {
    typedef u32x2 v;
    static __device__ inline double get(v r, int i) {
        const uint32_t w = r[i >> 1];
        return static_cast<double>(
            __builtin_bit_cast(_Float16, static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xFFFFu))));
    }
};
template <>
struct RawX4<float> {
    typedef u32x4 v;
    static __device__ inline double get(v r, int i) {
        const uint32_t w = r[i];   // the element as a scalar first: bit_cast of r[i] itself reads element 0
        return static_cast<double>(__builtin_bit_cast(float, w));
    }
};

// One block: 64 tokens of one unit, all of its stored components.


// One decode launch covers one tensor or two (the K and V of a layer): units
// below `split` (blockIdx.y) belong to t[0], the rest to t[1].
struct AppendPair {
    AppendArgs t[2];
    int64_t split;
};

// ================================================================ fetch
struct FetchArgs {
    const uint8_t *codes;              // [U][capacity][row_stride]
    const uint32_t *params;            // [U][capacity][n_qg] (min16 | scale16 << 16)
    int64_t capacity, s_begin, s_end;
    const uint16_t *w16;               // [U][dg][kfetch]
    const float *bias;                 // [U][dg]
    const uint32_t *kdesc;             // [U][kfetch/8]
    _Float16 *out;
    int64_t osb, osh, oss;             // element strides of out (d stride is 1)
    int dg, D, hpu, groups, kfetch, row_stride, n_qg;
    float nqg_inv;                     // 1 / n_qg (group-head mode)
    int nslices, nchunks, tiles_per_block, ntiles;
    int nks;                           // k-steps of this tensor (kfetch / 16)
    int64_t nblocks;                   // blocks of this tensor
    // dynamic LDS carve-up (bytes)
    int lds_w, lds_desc, lds_bias, lds_wave, lds_rows, lds_par, lds_out, wpitch, opitch;
    int lds_b, lds_dummy;              // weight-stationary blocks: operand buffers, scratch words
};

// One fetch launch covers one tensor or two (the K and V of a layer): the
// first `split` logical blocks belong to t[0], the rest to t[1].
struct FetchPair {
    FetchArgs t[2];
    int64_t split, nblocks_real, nblocks_per_xcd;
    bool narrow;                       // (host) every width of both tensors is 0, 2, 4 or 8
};

// Code widths a kernel decodes (bit W set for width W): every width, or only 2,
// 4 and 8 bits (the common choice sets; a shorter dispatch per k-step).
constexpr int kWidthsAll = (1 << 1) | (1 << 2) | (1 << 3) | (1 << 4) | (1 << 8);
constexpr int kWidths248 = (1 << 2) | (1 << 4) | (1 << 8);

// Whether a tensor's width choices (which every stored width is one of) are
// all among 0, 2, 4 and 8.
inline bool widths_248(const kvtc_state_header *h) {
    for (int i = 0; i < std::min<int>(h->n_choices, KVTC_MAX_CHOICES); ++i)
        if (h->choices[i] != 0 && h->choices[i] != 2 && h->choices[i] != 4 && h->choices[i] != 8) return false;
    return true;
}

typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// 0x64 as the high byte of an fp16 makes the low byte an integer offset from
// 1024: the half 0x64XX is exactly 1024 + XX.
constexpr uint32_t kMagic = 0x64646464u;

// Eight W-bit fields (W <= 3, all inside the low word) as four half2 pairs of
// 1024 + code, in field order.
template <int W>
__device__ inline void small_fields(uint32_t lo, uint32_t (&pr)[4]) {
    constexpr uint32_t kMask = (1u << W) - 1u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t c0 = (lo >> (2 * e * W)) & kMask, c1 = (lo >> ((2 * e + 1) * W)) & kMask;
        pr[e] = (c0 | (c1 << 16)) | 0x64006400u;
    }
}

// One lane's eight B-operand values of one k-step (16 fetch slots of a single
// width w > 0): the fields starting at the k-step's first field plus 8w for
// the upper operand half (for w = 2: the k-step's whole 32-bit window, shifted
// by 4 bits for the upper half), read from the lane's token row as a 64-bit
// window and turned into exact fp16 integers.  In group-head mode each code is
// dequantised with the row's fp16 (min, scale) of the k-step's quantisation
// group in one fp16 fma; mypar points at the lane's token in the group-major
// parameter staging.  Widths 2, 4 and 8 share one branch-free form; with WS =
// kWidthsAll two uniform tests route 1 and 3 bits to their own extraction.
template <bool MIXED, int WS = kWidthsAll>
__device__ __forceinline__ half8 decode_kstep(uint32_t kd, const uint32_t *myrow, const uint32_t *mypar,
                                              uint32_t half_k) {
    const uint32_t w = (kd >> 16) & 0xFu;
    const uint32_t off = (kd & 0xFFFFu) + (w == 2u ? 0u : (half_k << 3) * w);
    const uint32_t wi = off >> 5, sh = off & 31u;
    const uint32_t r0 = myrow[wi], r1 = myrow[wi + 1];
    const uint32_t lo = __builtin_amdgcn_alignbit(r1, r0, sh);
    uint32_t pr[4];                                        // 4 packed half2 of 1024 + code
    if (WS != kWidths248 && w == 1u) {
        small_fields<1>(lo, pr);
    } else if (WS != kWidths248 && w == 3u) {
        small_fields<3>(lo, pr);
    } else {
        // widths 2, 4 and 8 in one branch-free form (uniform selects): 8 bits:
        // the window's eight bytes; 4 bits: nibbles stored 0,2,4,6,1,3,5,7 (even
        // then odd nibbles); 2 bits: slots 0,4,8,12 then 1,5,9,13 (2,6,10,14 then
        // 3,7,11,15 in the upper half)
        const uint32_t hi = __builtin_amdgcn_alignbit(myrow[wi + 2], r1, sh);
        const uint32_t t = w == 2u ? lo >> (half_k << 2) : lo;
        const uint32_t msk = w == 8u ? 0xFFFFFFFFu : (w == 4u ? 0x0F0F0F0Fu : 0x03030303u);
        const uint32_t x0 = t & msk;
        const uint32_t x1 = (w == 8u ? hi : t >> (w == 4u ? 4u : 2u)) & msk;
        pr[0] = __builtin_amdgcn_perm(kMagic, x0, 0x04010400u);
        pr[1] = __builtin_amdgcn_perm(kMagic, x0, 0x04030402u);
        pr[2] = __builtin_amdgcn_perm(kMagic, x1, 0x04010400u);
        pr[3] = __builtin_amdgcn_perm(kMagic, x1, 0x04030402u);
    }
    half8 bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // (1024 + c) - 1024 = c exactly
        const half2 cv = __builtin_bit_cast(half2, pr[e]) -
                         half2{static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
        if constexpr (MIXED) {
            const uint32_t p = mypar[(kd >> 20) * kFetTok];
            const half2 mn2 = __builtin_bit_cast(half2, (p & 0xFFFFu) | (p << 16));
            const half2 sc2 = __builtin_bit_cast(half2, (p >> 16) | (p & 0xFFFF0000u));
            const half2 r = __builtin_elementwise_fma(cv, sc2, mn2);
            bv[2 * e] = r[0];
            bv[2 * e + 1] = r[1];
        } else {
            bv[2 * e] = cv[0];
            bv[2 * e + 1] = cv[1];
        }
    }
    return bv;
}

// Accumulators seeded with the bias: C[d][token] starts at bias[d] for the

constexpr int kLdsMax = 160 * 1024;

// Whether a fetch block takes the branch-free tile path: rows of at most 16
// words per lane (four-wave group-head blocks with k >= 128 would spill on it).
constexpr bool fetch_flat_path(bool mixed, int ks, int rw, int nw) { return rw <= 16 && !(mixed && nw == 4 && ks >= 8); }

// Register words per lane the fetch kernel is instantiated with for tiles of
// rw words per lane (the narrowest of 8, 16 or 24 that holds them; 16 only for
// whole-head blocks).
constexpr int fetch_rw_inst(int ndb, int rw) { return rw <= 8 ? 8 : (ndb == 4 && rw <= 16 ? 16 : 24); }

// Dynamic LDS carve-up of a fetch block for one tensor: sets the offsets and
// pitches in a and returns the bytes the block needs.  The W slice
// [ds][kfetch + 8] fp16, room for the k-step descriptors, the bias [ds] fp32,
// then per wave: the tile's rows back to back (plus slack for the 3-word field
// window of a padded k-step's upper operand half; on the branch-free path at
// least rw words per lane, all of which are stashed), the group-head params
// (plus one dummy word per lane for the branch-free stash) and the output
// staging of nh 32-column blocks.
inline size_t fetch_lds_plan(FetchArgs &a, bool mixed, int ds, int nw, int nh, int rw, bool flat) {
    a.wpitch = a.kfetch + 8;
    a.opitch = 32 * nh + 8;
    a.lds_w = 0;
    a.lds_desc = static_cast<int>(align_up(static_cast<uint64_t>(ds) * a.wpitch * 2, 16));
    a.lds_bias = static_cast<int>(align_up(a.lds_desc + 16, 16));
    a.lds_wave = static_cast<int>(align_up(a.lds_bias + ds * 4, 16));
    int rows_b = static_cast<int>(align_up((kFetTok * (a.row_stride / 4) + 8) * 4, 16));
    if (flat) rows_b = std::max(rows_b, rw * 64 * 4);
    const int par_b = mixed ? static_cast<int>(align_up((kFetTok * a.n_qg + 64) * 4, 16)) : 0;
    const int out_b = static_cast<int>(align_up(kFetTok * a.opitch * 2, 16));
    a.lds_par = rows_b;
    a.lds_out = rows_b + par_b;
    a.lds_rows = rows_b + par_b + out_b;                 // per-wave bytes
    return a.lds_wave + nw * static_cast<size_t>(a.lds_rows);
}

constexpr int kWsWaves = 8;                   // waves per weight-stationary block

// Output columns of a weight-stationary block whose waves each hold ndbw
// 32-column blocks of W.
constexpr int fetch_ws_cols(int ndbw) { return 32 * ndbw * kWsWaves; }

// fp16 pitch of a wave's output staging rows (ndbw 32-column blocks).
constexpr int fetch_ws_pitch(int ndbw) { return 32 * ndbw + 8; }

// Dynamic LDS carve-up of a weight-stationary block for one tensor (ks = the
// launch's k-steps): the bias of the block's columns, two operand buffers of ks
// k-steps [ks][64 lanes] x 8 fp16, two staging buffers, each a tile's rows (plus
// the slack of a field window), its group-head parameters (group-major) and one
// scratch word per thread for the stash of words past the tile, then each
// wave's output staging [32][pitch] fp16.  lds_par and lds_dummy are offsets
// inside a staging buffer, lds_rows the buffer's size.
inline size_t fetch_ws_lds_plan(FetchArgs &a, bool mixed, int ks, int ndbw) {
    a.wpitch = 0;
    a.opitch = fetch_ws_pitch(ndbw);
    a.lds_w = 0;
    a.lds_desc = 0;
    a.lds_bias = 0;
    a.lds_b = fetch_ws_cols(ndbw) * 4;
    a.lds_wave = a.lds_b + 2 * ks * 64 * 16;
    const int rows_b = static_cast<int>(align_up((kFetTok * (a.row_stride / 4) + 8) * 4, 16));
    const int par_b = mixed ? static_cast<int>(align_up(kFetTok * a.n_qg * 4, 16)) : 0;
    a.lds_par = rows_b;
    a.lds_dummy = rows_b + par_b;
    a.lds_rows = rows_b + par_b + 64 * kWsWaves * 4;     // bytes per staging buffer
    a.lds_out = a.lds_wave + 2 * a.lds_rows;
    return static_cast<size_t>(a.lds_out) + kWsWaves * kFetTok * a.opitch * 2;
}

// LDS a weight-stationary block's prologue stages its W rows through: per
// wave 32 rows of 16 ks slots (pitch padded by 16 bytes).
constexpr size_t fetch_ws_w_staging(int ks) { return static_cast<size_t>(kWsWaves) * 32 * (ks * 32 + 16); }

// Row words each thread of a weight-stationary block loads per tile.
constexpr int fetch_ws_rwb(int tile_words) { return (tile_words + 64 * kWsWaves - 1) / (64 * kWsWaves); }

// Lets a kernel use up to the whole LDS of a CU as dynamic shared memory (set
// once per kernel and device).
bool allow_lds(const void *kern);

// ============================================================== call plans
// Everything a call needs to launch, after its arguments have been validated.
struct AppendPlan {
    AppendArgs a;
    int64_t units, ntiles;
    int nb;                            // 16-slot N-blocks of the bulk kernels
    int32_t dtype;
    bool mixed;
    int i8_ns, i8_nsg;                 // int8 append: 32-slot tiles per block, slot groups (0: not used)
};

struct FetchPlan {
    FetchArgs a;
    int ds, rw;                        // columns per block (128 or 64), row words per lane
    bool mixed;
    bool narrow;                       // DP with every width choice among 0, 2, 4, 8
};

// ------------------------------------------------------------ refit mode
// Device buffer of a refit-mode tensor (caller-owned), sections 256-byte aligned
// in this order: qmin32, qscale32 float [U][kslots] (the refitted ranges of
// slot j), qlo, qinv double [U][kslots] (the quantiser's min and 1/scale),
// w16 half [U][dg][kfetch] and bias float [U][dg] (fetch operands, laid out as
// the blob's), part double [U][chunks][kslots][2] (per-chunk min and max).
struct RefitLayout {
    uint64_t qmin32, qscale32, qlo, qinv, w16, bias, part, total;
    int chunks;
};

inline RefitLayout refit_layout(const kvtc_state_header *h, int64_t capacity) {
    RefitLayout L{};
    const uint64_t U = static_cast<uint64_t>(h->units), ks = h->kslots;
    int64_t c = (capacity + 255) / 256;
    L.chunks = static_cast<int>(c < 1 ? 1 : (c > 256 ? 256 : c));
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = o;
        o = align_up(o + (bytes ? bytes : 1), kSectionAlign);
        return at;
    };
    L.qmin32 = take(U * ks * 4);
    L.qscale32 = take(U * ks * 4);
    L.qlo = take(U * ks * 8);
    L.qinv = take(U * ks * 8);
    L.w16 = take(U * static_cast<uint64_t>(h->dg) * h->kfetch * 2);
    L.bias = take(U * static_cast<uint64_t>(h->dg) * 4);
    L.part = take(U * static_cast<uint64_t>(L.chunks) * ks * 16);
    L.total = o;
    return L;
}

struct RefitArgs {
    const double *lat;                 // [U][capacity][kslots] latents of the stored rows
    int64_t capacity, S;               // rows [0, S) are accumulated
    int64_t rows_per_chunk;
    const kvtc_unit_info *ui;
    const uint32_t *sbits;             // [U][kslots]
    const float *basis;                // [U][kslots][dg]
    const float *mu;                   // [U][dg]
    const int32_t *fslot;              // [U][kfetch]
    float *qmin32, *qscale32;          // [U][kslots]
    double *qlo, *qinv;                // [U][kslots]
    uint16_t *w16;                     // [U][dg][kfetch]
    float *bias;                       // [U][dg]
    double *part;                      // [U][chunks][kslots][2]
    uint8_t *codes;                    // [U][capacity][row_stride]
    int kslots, dg, kfetch, row_stride, chunks;
};

// Ranges over rows [0, S), the quantiser and fetch operands they imply, then
// the codes of every row [0, S) re-quantised and re-packed (kvtc_refit.hip).
int32_t launch_refit_requantise(const RefitArgs &a, int64_t units, hipStream_t stream);

// ------------------------------------------------------------ launchers
// append (kvtc_append.hip)
// KVTC_OK after a launch that HIP accepted, else KVTC_E_DEVICE with HIP's error
// kept for kvtc_device_error_string (per calling thread).
int32_t launch_status();
void note_device_error(hipError_t e);
hipError_t g_device_error_value();
int32_t launch_append_plan(const AppendPlan &p, hipStream_t stream);
// Bulk append of fp16 rows on int8 MFMA with certified decisions
// (kvtc_append_i8.hip); plans with i8_ns set only.
int32_t launch_append_i8(const AppendPlan &p, hipStream_t stream);
bool decode_path(const AppendPlan &p);
int32_t launch_decode(const AppendPlan &p0, const AppendPlan *p1, hipStream_t stream);
int append_nb(int kslots);
// device fit: per-slot min and max of the latents of rows [0, n) into a.keys,
// as order-preserving integer keys (kvtc_append.hip)
int32_t launch_fit_ranges(const AppendArgs &a, int64_t units, int nb, int32_t dtype, hipStream_t stream);
// refit mode: fp64 latents of rows [s0, s0 + n) into a.lat (kvtc_append.hip)
int32_t launch_refit_project(const AppendPlan &p, hipStream_t stream);

// traffic probe of the fetch with the fetch's launch plan (kvtc_probe.hip):
// ds columns per block, nw waves per block, the fetch's dynamic LDS bytes
int32_t launch_fetch_probe(const FetchPair &m, int ds, int nw, bool mixed, int rw, size_t lds, hipStream_t stream);
// the weight-stationary kernel's probe (group-head, ks k-steps, ndbw 32-column
// blocks per wave, tile_words row and parameter words per tile)
int32_t launch_fetch_ws_probe(FetchPair m, int nt, int ks, int ndbw, int tile_words, hipStream_t stream);

// fetch: one launcher per contraction length in 16-slot k-steps, each compiled
// in a translation unit of its own (kvtc_fetch_ks.hip)
#define KVTC_DECLARE_FETCH_KS(N) \
    int32_t launch_fetch_ks##N(bool mixed, int ndb, const FetchPair &m, int nt, int rw, hipStream_t stream);
KVTC_DECLARE_FETCH_KS(1)
KVTC_DECLARE_FETCH_KS(2)
KVTC_DECLARE_FETCH_KS(3)
KVTC_DECLARE_FETCH_KS(4)
KVTC_DECLARE_FETCH_KS(5)
KVTC_DECLARE_FETCH_KS(6)
KVTC_DECLARE_FETCH_KS(7)
KVTC_DECLARE_FETCH_KS(8)
KVTC_DECLARE_FETCH_KS(9)
KVTC_DECLARE_FETCH_KS(10)
KVTC_DECLARE_FETCH_KS(11)
KVTC_DECLARE_FETCH_KS(12)
KVTC_DECLARE_FETCH_KS(13)
KVTC_DECLARE_FETCH_KS(14)
KVTC_DECLARE_FETCH_KS(15)
KVTC_DECLARE_FETCH_KS(16)
#undef KVTC_DECLARE_FETCH_KS

}  // namespace kvtc
