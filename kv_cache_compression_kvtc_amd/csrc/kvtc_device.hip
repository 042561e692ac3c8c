// Device half of libkvtc for gfx950 (CDNA4): the fused append and fetch
// kernels and their C-ABI launchers.
//
// Append (KVTC cache module page, module docstring "Design", decode step 1;
// PALU cache API page, "Design", decode steps 1-2): every row is centred,
// projected through the frozen basis of its unit, each stored component is
// quantised at its frozen width and the codes are OR-ed into a little-endian
// bit row in LDS, which is then written to the store with coalesced stores.
// The projection runs on fp64 MFMA so that codes are decided from latents
// accurate to ~1e-16, i.e. identical to a float64 evaluation except when a
// value lies within rounding distance of a quantisation boundary.
//
// Fetch (same pages: every call returns the whole sequence reconstructed to
// fp16): code rows stream from HBM into LDS, each lane extracts its fields,
// forms the fp16 contraction operand and the [tokens x slots] x [slots x d]
// product runs on fp16 MFMA with fp32 accumulation; a bias is added, the
// result is rounded to fp16 and transposed through LDS into fully coalesced
// 16-byte non-temporal stores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "kvtc.h"
#include "kvtc_internal.h"

namespace kvtc {
namespace {

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
    int dg, D, hpu, groups, kslots, row_stride, n_qg, gs;
    float inv_dg, inv_q4;              // 1/dg and 4/dg: exact quotients of small indices
    int x_vec;                         // rows and strides aligned to 4 elements (raw vector loads)
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
// Wave w owns tokens 16w..16w+15; N-block nb covers slots 16nb..16nb+15.
template <bool MIXED, typename XT, int NB, bool XVEC>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    double *xs = reinterpret_cast<double *>(smem);                         // [2][64][kAppPad]
    float *vs = reinterpret_cast<float *>(xs + 2 * kAppTok * kAppPad);     // [2][NB*16][kAppPad]
    uint32_t *rows = reinterpret_cast<uint32_t *>(vs + 2 * NB * 16 * kAppPad);  // [64][row_words]

    const int u = blockIdx.y;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kAppTok;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = u / a.groups, g = u % a.groups;
    const int nvalid = static_cast<int>(min<int64_t>(kAppTok, a.n - t0));
    const int n_slots = a.ui[u].n_slots;
    const int row_words = a.row_stride >> 2;
    const XT *x = static_cast<const XT *>(a.x);

    for (int w = tid; w < kAppTok * row_words; w += kThreads) rows[w] = 0u;

    // staging map: thread -> (token, 4 consecutive columns) of a 64 x 16 chunk,
    // and (slot, 4 columns) of the NB*16 x 16 basis chunk
    const int st_tok = tid >> 2, st_col = (tid & 3) * 4;
    constexpr int kVReps = (NB * 16 + 63) / 64;
    // a chunk's loads only fill these registers (indices clamped, so no load
    // sits behind a branch); centring and the fp64 conversion happen when the
    // chunk is written to LDS, after the MFMAs of the previous chunk, so the
    // loads are in flight during those MFMAs
    typename RawX4<XT>::v xv;
    XT xraw[4];
    float muv[4];
    float vr[kVReps][4];
    const int tok_c = min(st_tok, nvalid - 1);

    auto load_chunk = [&](int kc) {
        const int gd = kc * kAppKC + st_col;          // column within the unit's row
        const int j = gd / a.D, dd = gd - j * a.D;
        const int h = g * a.hpu + j;
        const float *mu = a.mu + static_cast<int64_t>(u) * a.dg + gd;
        const XT *p = x + b * a.xsb + h * a.xsh + (t0 + tok_c) * a.xss + dd;
        if constexpr (XVEC) {
            xv = *reinterpret_cast<const typename RawX4<XT>::v *>(p);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) xraw[i] = p[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) muv[i] = mu[i];
#pragma unroll
        for (int rep = 0; rep < kVReps; ++rep) {
            const int slot = min(rep * 64 + st_tok, a.kslots - 1);
            const float *q = a.basis + (static_cast<int64_t>(u) * a.kslots + slot) * a.dg + gd;
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[rep][i] = q[i];
        }
    };
    auto store_chunk = [&](int buf) {
        double *xb = xs + buf * kAppTok * kAppPad + st_tok * kAppPad + st_col;
        const bool tok_ok = st_tok < nvalid;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double xi = XVEC ? RawX4<XT>::get(xv, i) : load_x(&xraw[i]);
            xb[i] = tok_ok ? xi - static_cast<double>(muv[i]) : 0.0;
        }
#pragma unroll
        for (int rep = 0; rep < kVReps; ++rep) {
            const int slot = rep * 64 + st_tok;
            if (slot < NB * 16) {
                const bool keep = slot < a.kslots;      // slots past kslots are zero
                float *vb = vs + (buf * NB * 16 + slot) * kAppPad + st_col;
#pragma unroll
                for (int i = 0; i < 4; ++i) vb[i] = keep ? vr[rep][i] : 0.0f;
            }
        }
    };

    doublex4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = doublex4{0.0, 0.0, 0.0, 0.0};

    const int nchunks = a.dg / kAppKC;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    const int mrow = wave * 16 + (lane & 15);   // A operand row (token) of this lane
    const int kcol = lane >> 4;                 // A/B operand k of this lane
    // k-step order: k-step 4c + e of the contraction takes, at operand k = q, the
    // feature 16c + 4q + e (c = 16-column chunk); every append kernel uses this
    // order, so that a lane of the decode kernel holds its operands as whole
    // 16-byte vectors of the basis
    for (int kc = 0; kc < nchunks; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nchunks) load_chunk(kc + 1);
        const double *xb = xs + buf * kAppTok * kAppPad;
        const float *vb = vs + buf * NB * 16 * kAppPad;
#pragma unroll
        for (int ks = 0; ks < kAppKC / 4; ++ks) {
            const double av = xb[mrow * kAppPad + kcol * 4 + ks];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const double bv = static_cast<double>(vb[(nb * 16 + (lane & 15)) * kAppPad + kcol * 4 + ks]);
                acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[nb], 0, 0, 0);
            }
        }
        if (kc + 1 < nchunks) store_chunk(buf ^ 1);
        __syncthreads();
    }

    // fp64 16x16x4 result layout: acc[nb][i] is row (lane>>4) + 4i, column lane&15, i.e.
    // the latent of token 16*wave + (lane>>4) + 4i and slot 16*nb + (lane&15)
    const int tbase = wave * 16 + (lane >> 4);
    const int64_t ub = static_cast<int64_t>(u) * a.kslots;
    if constexpr (!MIXED) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int j = nb * 16 + (lane & 15);
            if (j < n_slots) {
                const double lo = a.qlo[ub + j], inv = a.qinv[ub + j];
                const uint32_t sb = a.sbits[ub + j];
                const uint32_t off = sb & kOffsetMask, w = sb >> 24;
                const double cmax = static_cast<double>((1u << w) - 1u);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tbase + 4 * i;
                    if (t < nvalid) {
                        const uint32_t c = static_cast<uint32_t>(quantise(acc[nb][i], lo, inv, cmax));
                        or_field(rows + t * row_words, off, w, c);
                    }
                }
            }
        }
    } else {
        const int ngroups = (n_slots + a.gs - 1) / a.gs;
        for (int gi = 0; gi < ngroups; ++gi) {
            const int j0 = gi * a.gs, j1 = min(n_slots, j0 + a.gs);
            const uint32_t w = a.sbits[ub + j0] >> 24;
            const double cmax = static_cast<double>((1u << w) - 1u);
            double mn[4], mx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mn[i] = __builtin_huge_val();
                mx[i] = -__builtin_huge_val();
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int j = nb * 16 + (lane & 15);
                if (j >= j0 && j < j1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        mn[i] = fmin(mn[i], acc[nb][i]);
                        mx[i] = fmax(mx[i], acc[nb][i]);
                    }
                }
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mn[i] = fmin(mn[i], __shfl_xor(mn[i], m, 16));
                    mx[i] = fmax(mx[i], __shfl_xor(mx[i], m, 16));
                }
            }
            double lo16[4], inv16[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t hmin = half_bits_rne(mn[i]);
                const uint16_t hscale = half_bits_rne((mx[i] - mn[i]) / cmax);
                lo16[i] = half_bits_to_double(hmin);
                const double sc = half_bits_to_double(hscale);
                inv16[i] = sc > 0.0 ? 1.0 / sc : 0.0;
                const int t = tbase + 4 * i;
                if ((lane & 15) == 0 && t < nvalid)
                    a.params[(static_cast<int64_t>(u) * a.capacity + a.s0 + t0 + t) * a.n_qg + gi] =
                        static_cast<uint32_t>(hmin) | (static_cast<uint32_t>(hscale) << 16);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int j = nb * 16 + (lane & 15);
                if (j >= j0 && j < j1) {
                    const uint32_t off = a.sbits[ub + j] & kOffsetMask;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tbase + 4 * i;
                        if (t < nvalid) {
                            const uint32_t c = static_cast<uint32_t>(quantise(acc[nb][i], lo16[i], inv16[i], cmax));
                            or_field(rows + t * row_words, off, w, c);
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    if (row_words > 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            a.codes + (static_cast<int64_t>(u) * a.capacity + a.s0 + t0) * a.row_stride);
        for (int w = tid; w < nvalid * row_words; w += kThreads) dst[w] = rows[w];
    }
}

// Few-row append (decode): one block per unit and up to 16 rows.  The whole
// basis of the unit is staged in LDS with every load in flight at once, and the
// N-blocks are spread over the 4 waves.  Each row goes through exactly the same
// sequence of fp64 MFMAs (same operands, same k order) as in append_kernel, so
// a row's codes do not depend on which kernel appended it.
template <typename XT, int NB>
__global__ __launch_bounds__(kThreads) void append_small_kernel(AppendArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int xpitch = a.dg + 1, vpitch = a.dg + 1;
    double *xs = reinterpret_cast<double *>(smem);                       // [16][xpitch]
    float *vs = reinterpret_cast<float *>(xs + 16 * xpitch);             // [NB*16][vpitch]
    uint32_t *rows = reinterpret_cast<uint32_t *>(vs + NB * 16 * vpitch);  // [16][row_words]

    const int u = blockIdx.y;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = u / a.groups, g = u % a.groups;
    const int nvalid = static_cast<int>(min<int64_t>(16, a.n - t0));
    const int n_slots = a.ui[u].n_slots;
    const int row_words = a.row_stride >> 2;
    const XT *x = static_cast<const XT *>(a.x);

    constexpr int NBW = (NB + 3) / 4;       // N-blocks of this wave: wave, wave+4, ...
    // Every global load of the block is issued before the first LDS write, so
    // the kernel waits for memory once: this lane's slot constants (indices
    // clamped; unused past n_slots), the first batch of the basis, then the
    // valid input rows.  Quotients of indices by dg and dg/4 come from float
    // reciprocals, exact for indices below 2^16.
    const int64_t ub = static_cast<int64_t>(u) * a.kslots;
    double qlo_r[NBW], qinv_r[NBW];
    uint32_t sb_r[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int j = min((wave + 4 * q) * 16 + (lane & 15), a.kslots - 1);
        qlo_r[q] = a.qlo[ub + j];
        qinv_r[q] = a.qinv[ub + j];
        sb_r[q] = a.sbits[ub + j];
    }
    const int q4 = a.dg / 4;
    const float *basis = a.basis + static_cast<int64_t>(u) * a.kslots * a.dg;
    const int nv = NB * 16 * q4, nload = a.kslots * q4;
    constexpr int kBatchV = 16;
    float4 vb[kBatchV];
    auto load_basis = [&](int i0) {
#pragma unroll
        for (int q = 0; q < kBatchV; ++q) {
            const int i = min(i0 + q * kThreads + tid, nload - 1);
            vb[q] = *reinterpret_cast<const float4 *>(basis + static_cast<int64_t>(i) * 4);
        }
    };
    auto store_basis = [&](int i0) {
#pragma unroll
        for (int q = 0; q < kBatchV; ++q) {
            const int i = i0 + q * kThreads + tid;
            if (i < nv) {
                const int slot = static_cast<int>((static_cast<float>(i) + 0.5f) * a.inv_q4);
                const int c = (i - slot * q4) * 4;
                const bool keep = i < nload;           // slots past kslots are zero
                float *dst = vs + slot * vpitch + c;
                dst[0] = keep ? vb[q].x : 0.f;
                dst[1] = keep ? vb[q].y : 0.f;
                dst[2] = keep ? vb[q].z : 0.f;
                dst[3] = keep ? vb[q].w : 0.f;
            }
        }
    };
    load_basis(0);
    {
        const float *mu = a.mu + static_cast<int64_t>(u) * a.dg;
        const int nx = nvalid * a.dg;
        for (int i = tid; i < nx; i += kThreads) {
            const int t = static_cast<int>((static_cast<float>(i) + 0.5f) * a.inv_dg);
            const int d = i - t * a.dg;
            xs[t * xpitch + d] =
                load_x(x + b * a.xsb + g * a.xsh + (t0 + t) * a.xss + d) - static_cast<double>(mu[d]);
        }
        for (int i = nx + tid; i < 16 * a.dg; i += kThreads) {
            const int t = static_cast<int>((static_cast<float>(i) + 0.5f) * a.inv_dg);
            xs[t * xpitch + (i - t * a.dg)] = 0.0;
        }
    }
    for (int w = tid; w < 16 * row_words; w += kThreads) rows[w] = 0u;
    store_basis(0);
    for (int i0 = kBatchV * kThreads; i0 < nv; i0 += kBatchV * kThreads) {
        load_basis(i0);
        store_basis(i0);
    }
    __syncthreads();

    doublex4 acc[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) acc[q] = doublex4{0.0, 0.0, 0.0, 0.0};
    const int mrow = lane & 15, kcol = lane >> 4;
    for (int ks = 0; ks < a.dg / 4; ++ks) {
        const int col = (ks >> 2) * 16 + kcol * 4 + (ks & 3);   // k-step order of append_kernel
        const double av = xs[mrow * xpitch + col];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = wave + 4 * q;
            if (nb < NB) {
                const double bv = static_cast<double>(vs[(nb * 16 + (lane & 15)) * vpitch + col]);
                acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[q], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int nb = wave + 4 * q;
        const int j = nb * 16 + (lane & 15);
        if (nb < NB && j < n_slots) {
            const double lo = qlo_r[q], inv = qinv_r[q];
            const uint32_t sb = sb_r[q];
            const uint32_t off = sb & kOffsetMask, w = sb >> 24;
            const double cmax = static_cast<double>((1u << w) - 1u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = (lane >> 4) + 4 * i;
                if (t < nvalid) {
                    const uint32_t c = static_cast<uint32_t>(quantise(acc[q][i], lo, inv, cmax));
                    or_field(rows + t * row_words, off, w, c);
                }
            }
        }
    }
    __syncthreads();
    if (row_words > 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            a.codes + (static_cast<int64_t>(u) * a.capacity + a.s0 + t0) * a.row_stride);
        for (int w = tid; w < nvalid * row_words; w += kThreads) dst[w] = rows[w];
    }
}

// One decode launch covers one tensor or two (the K and V of a layer): units
// below `split` (blockIdx.y) belong to t[0], the rest to t[1].
struct AppendPair {
    AppendArgs t[2];
    int64_t split;
};

size_t decode_lds_bytes(int dg, int row_stride) {
    return 16 * static_cast<size_t>(dg + 1) * sizeof(double) + 16 * static_cast<size_t>(row_stride / 4) * sizeof(uint32_t);
}

// Decode append (up to 16 rows per unit, DP mode, unit width DG): one block per
// unit, one wave per 16-slot N-block.  In the k-step order of append_kernel a
// lane's basis operands (slot 16*wave + lane%16, features 16c + 4*(lane/16) +
// 0..3 for k-steps 4c..4c+3) are whole 16-byte vectors, loaded straight into
// registers: the basis never passes through LDS and every load of the block is
// in flight before its first wait; only the centred rows are staged in LDS.  The fp64 MFMA sequence per row (operands and k order) is
// the one of append_kernel, so a row's codes do not depend on the kernel that
// appended it.  Rows past the valid ones are left unset in LDS: a row of the
// MFMA result depends only on the same row of A, and those rows are not used.
template <typename XT, int DG>
__global__ __launch_bounds__(512) void append_decode_kernel(AppendPair m) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int XP = DG + 1;          // LDS pitch (doubles) of a centred row
    constexpr int NKS = DG / 4;         // MFMA k-steps
    double *xs = reinterpret_cast<double *>(smem);                    // [16][XP]
    uint32_t *rows = reinterpret_cast<uint32_t *>(xs + 16 * XP);      // [16][row_words]

    const bool second = blockIdx.y >= m.split;         // block-uniform
    const AppendArgs &a = second ? m.t[1] : m.t[0];
    const int u = static_cast<int>(blockIdx.y - (second ? m.split : 0));
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nthreads = blockDim.x;
    const int b = u / a.groups, g = u % a.groups;
    const int nvalid = static_cast<int>(min<int64_t>(16, a.n - t0));
    const int row_words = a.row_stride >> 2;
    const bool active = wave < (a.kslots >> 4);        // this tensor's N-blocks
    const int j = wave * 16 + (lane & 15), kq = lane >> 4;
    const int64_t ub = static_cast<int64_t>(u) * a.kslots;

    float4 vr[NKS / 4];
    double lo = 0.0, inv = 0.0;
    uint32_t sb = 0u;
    if (active) {
        const float4 *vp = reinterpret_cast<const float4 *>(a.basis + (ub + j) * DG + 4 * kq);
#pragma unroll
        for (int c = 0; c < NKS / 4; ++c) vr[c] = vp[4 * c];
        lo = a.qlo[ub + j];
        inv = a.qinv[ub + j];
        sb = a.sbits[ub + j];
    }
    const XT *x = static_cast<const XT *>(a.x) + b * a.xsb + g * a.xsh + t0 * a.xss;
    const float *mu = a.mu + static_cast<int64_t>(u) * DG;
    for (int i = tid; i < nvalid * DG; i += nthreads) {
        const int t = i / DG, d = i % DG;
        xs[t * XP + d] = load_x(x + t * a.xss + d) - static_cast<double>(mu[d]);
    }
    for (int w = tid; w < 16 * row_words; w += nthreads) rows[w] = 0u;
    __syncthreads();

    if (active) {
        doublex4 acc = doublex4{0.0, 0.0, 0.0, 0.0};
        const double *xr = xs + (lane & 15) * XP + 4 * kq;
#pragma unroll
        for (int c = 0; c < NKS / 4; ++c) {
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[16 * c + 0], static_cast<double>(vr[c].x), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[16 * c + 1], static_cast<double>(vr[c].y), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[16 * c + 2], static_cast<double>(vr[c].z), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[16 * c + 3], static_cast<double>(vr[c].w), acc, 0, 0, 0);
        }
        // result layout: acc[i] is token kq + 4i, slot j
        if (j < a.ui[u].n_slots) {
            const uint32_t off = sb & kOffsetMask, w = sb >> 24;
            const double cmax = static_cast<double>((1u << w) - 1u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = kq + 4 * i;
                if (t < nvalid) or_field(rows + t * row_words, off, w, static_cast<uint32_t>(quantise(acc[i], lo, inv, cmax)));
            }
        }
    }
    __syncthreads();
    if (row_words > 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            a.codes + (static_cast<int64_t>(u) * a.capacity + a.s0 + t0) * a.row_stride);
        for (int w = tid; w < nvalid * row_words; w += nthreads) dst[w] = rows[w];
    }
}

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
};

// One fetch launch covers one tensor or two (the K and V of a layer): the
// first `split` logical blocks belong to t[0], the rest to t[1].
struct FetchPair {
    FetchArgs t[2];
    int64_t split, nblocks_real, nblocks_per_xcd;
};

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
// parameter staging.
template <bool MIXED>
__device__ __forceinline__ half8 decode_kstep(uint32_t kd, const uint32_t *myrow, const uint32_t *mypar,
                                              uint32_t half_k) {
    const uint32_t w = (kd >> 16) & 0xFu;
    const uint32_t off = (kd & 0xFFFFu) + (w == 2u ? 0u : (half_k << 3) * w);
    const uint32_t wi = off >> 5, sh = off & 31u;
    const uint32_t r0 = myrow[wi], r1 = myrow[wi + 1];
    const uint32_t lo = __builtin_amdgcn_alignbit(r1, r0, sh);
    uint32_t pr[4];                                        // 4 packed half2 of 1024 + code
    if (w == 8u) {
        const uint32_t hi = __builtin_amdgcn_alignbit(myrow[wi + 2], r1, sh);
        pr[0] = __builtin_amdgcn_perm(kMagic, lo, 0x04010400u);
        pr[1] = __builtin_amdgcn_perm(kMagic, lo, 0x04030402u);
        pr[2] = __builtin_amdgcn_perm(kMagic, hi, 0x04010400u);
        pr[3] = __builtin_amdgcn_perm(kMagic, hi, 0x04030402u);
    } else if (w == 4u) {
        // nibbles of a 4-bit k-step are stored in the order 0,2,4,6,1,3,5,7
        const uint32_t ev = lo & 0x0F0F0F0Fu, od = (lo >> 4) & 0x0F0F0F0Fu;
        pr[0] = __builtin_amdgcn_perm(kMagic, ev, 0x04010400u);
        pr[1] = __builtin_amdgcn_perm(kMagic, ev, 0x04030402u);
        pr[2] = __builtin_amdgcn_perm(kMagic, od, 0x04010400u);
        pr[3] = __builtin_amdgcn_perm(kMagic, od, 0x04030402u);
    } else if (w == 2u) {
        // slots 0,4,8,12 then 1,5,9,13 (2,6,10,14 then 3,7,11,15 in the upper half)
        const uint32_t t = lo >> (half_k << 2);
        const uint32_t ev = t & 0x03030303u, od = (t >> 2) & 0x03030303u;
        pr[0] = __builtin_amdgcn_perm(kMagic, ev, 0x04010400u);
        pr[1] = __builtin_amdgcn_perm(kMagic, ev, 0x04030402u);
        pr[2] = __builtin_amdgcn_perm(kMagic, od, 0x04010400u);
        pr[3] = __builtin_amdgcn_perm(kMagic, od, 0x04030402u);
    } else if (w == 1u) {
        small_fields<1>(lo, pr);
    } else {
        small_fields<3>(lo, pr);
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
// rows d = 32db + 8q + 4half_k + e this lane holds.
template <int NDB>
__device__ __forceinline__ void seed_bias(floatx16 (&acc)[NDB], const float *biasl, int half_k) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 bq = *reinterpret_cast<const float4 *>(biasl + db * 32 + q * 8 + half_k * 4);
            acc[db][q * 4 + 0] = bq.x;
            acc[db][q * 4 + 1] = bq.y;
            acc[db][q * 4 + 2] = bq.z;
            acc[db][q * 4 + 3] = bq.w;
        }
}

// fp16 rounding of a 32-token x 32*NDB-column block of accumulators, transposed
// through this wave's LDS staging into rows of 16-byte chunks, written with
// non-temporal stores (the first `valid` tokens only).  orow points at the
// output row of the tile's first token, first column of the block.
template <int NDB, bool FULL = false>
__device__ __forceinline__ void store_tile(const floatx16 *acc, _Float16 *outl, int opitch, int lane,
                                           _Float16 *orow, int64_t oss, int valid) {
    constexpr int DS = 32 * NDB;
    const int tok = lane & 31, half_k = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int dl = db * 32 + q * 8 + half_k * 4;
            const float2v p0 = {acc[db][q * 4 + 0], acc[db][q * 4 + 1]};
            const float2v p1 = {acc[db][q * 4 + 2], acc[db][q * 4 + 3]};
            const half2 h0 = __builtin_convertvector(p0, half2), h1 = __builtin_convertvector(p1, half2);
            half4 hv;
            hv[0] = h0[0];
            hv[1] = h0[1];
            hv[2] = h1[0];
            hv[3] = h1[1];
            *reinterpret_cast<half4 *>(outl + tok * opitch + dl) = hv;
        }
    }
    __builtin_amdgcn_wave_barrier();
    constexpr int kChunksPerRow = DS / 8;
    if (FULL || valid == kFetTok) {              // whole tile: no per-row masks
#pragma unroll
        for (int it = 0; it < kFetTok * kChunksPerRow / 64; ++it) {
            const int idx = it * 64 + lane;
            const int t = idx / kChunksPerRow, c = idx - t * kChunksPerRow;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(outl + t * opitch + c * 8);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(orow + t * oss + c * 8));
        }
    } else {
#pragma unroll
        for (int it = 0; it < kFetTok * kChunksPerRow / 64; ++it) {
            const int idx = it * 64 + lane;
            const int t = idx / kChunksPerRow, c = idx - t * kChunksPerRow;
            if (t < valid) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(outl + t * opitch + c * 8);
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(orow + t * oss + c * 8));
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Waves per fetch block: four, or eight for a 128-column slice of a long
// contraction (10+ k-steps), whose W slice leaves LDS for one block per CU.
template <int NDB, int KS>
constexpr int fetch_waves() { return (NDB == 4 && KS >= 10) ? 8 : 4; }

// Accumulator blocks per epilogue pass: the whole slice, or half of it with
// eight waves (whose LDS staging must then be half as large).
template <int NDB, int NW>
constexpr int fetch_epilogue_blocks() { return NW == 8 ? NDB / 2 : NDB; }

// Tiles of stored rows each fetch wave keeps in flight: where a tile's rows
// fit in 8 words per lane three (DP) or two (group-head, whose decode needs
// more registers), in 16 words two (DP) or one, otherwise one.
// Whether a fetch kernel takes the branch-free tile path (rows of at most 16
// words per lane; four-wave group-head kernels with k >= 128 would spill on
// it and keep the conditional loads).
template <bool MIXED, int KS, int RW, int NW>
constexpr bool fetch_flat() { return RW <= 16 && !(MIXED && NW == 4 && KS >= 8); }

template <bool MIXED, int RW>
constexpr int fetch_prefetch() { return RW <= 8 ? (MIXED ? 2 : 3) : (RW <= 16 && !MIXED ? 2 : 1); }

// One block: one (unit, d-slice of 32*NDB columns), a run of 32-token tiles;
// each of its NW waves reconstructs whole tiles with the block's W slice in
// LDS, prefetching the next tile's rows (RW words per lane) into registers.
// Serves contractions of up to 256 slots.  MFMA operands: A = W rows (d),
// B = per-token code values (fetch slots), C[d][token] accumulates in fp32.
// With four waves two such blocks fit a CU (two waves per SIMD) and the
// epilogue writes whole rows of the slice, 16-byte chunks of up to four rows
// per store; with eight waves (long contractions) one block does, and the
// epilogue writes the slice in two halves.
template <bool MIXED, int NDB, int KS, int RW, int NW, int PF>
__global__ __launch_bounds__(64 * NW, 2) void fetch_kernel(FetchPair m) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int DS = 32 * NDB;
    constexpr int NT = 64 * NW;
    constexpr int NH = fetch_epilogue_blocks<NDB, NW>();
    // blocks are dealt to the 8 XCDs round-robin; regroup them so that the
    // blocks of one unit (and its d-slices) run on the same XCD
    const int64_t bid = blockIdx.x;
    int64_t logical = (bid & 7) * m.nblocks_per_xcd + (bid >> 3);
    if (logical >= m.nblocks_real) return;
    const bool second = logical >= m.split;           // block-uniform
    const FetchArgs &a = second ? m.t[1] : m.t[0];
    if (second) logical -= m.split;
    const int slice = static_cast<int>(logical % a.nslices);
    const int64_t rest = logical / a.nslices;
    const int chunk = static_cast<int>(rest % a.nchunks);
    const int u = static_cast<int>(rest / a.nchunks);
    const int b = u / a.groups, g = u % a.groups;
    const int d0 = slice * DS;
    const int head = g * a.hpu + d0 / a.D, dd0 = d0 % a.D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar tile loops
    const int row_words = a.row_stride >> 2;

    _Float16 *wl = reinterpret_cast<_Float16 *>(smem + a.lds_w);       // [DS][wpitch]
    float *biasl = reinterpret_cast<float *>(smem + a.lds_bias);        // [DS]
    unsigned char *wbase = smem + a.lds_wave + wave * a.lds_rows;
    uint32_t *rowsl = reinterpret_cast<uint32_t *>(wbase);              // [32*row_words + 8]
    uint32_t *parl = reinterpret_cast<uint32_t *>(wbase + a.lds_par);   // [n_qg][32]
    _Float16 *outl = reinterpret_cast<_Float16 *>(wbase + a.lds_out);   // [32][opitch]

    // stage this slice of W and the bias
    {
        const uint16_t *src = a.w16 + (static_cast<int64_t>(u) * a.dg + d0) * a.kfetch;
        const int vec_per_row = a.kfetch / 8;
#pragma unroll 4
        for (int i = tid; i < DS * vec_per_row; i += NT) {
            const int r = i / vec_per_row, c = i - r * vec_per_row;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src + r * a.kfetch + c * 8);
            *reinterpret_cast<u32x4 *>(wl + r * a.wpitch + c * 8) = v;
        }
        for (int i = tid; i < DS; i += NT) biasl[i] = a.bias[static_cast<int64_t>(u) * a.dg + d0 + i];
    }
    __syncthreads();

    const int tile_begin = chunk * a.tiles_per_block;
    const int tile_end = min(a.ntiles, tile_begin + a.tiles_per_block);
    const int row_tile_words = kFetTok * row_words;
    const int tile_words = row_tile_words + (MIXED ? kFetTok * a.n_qg : 0);
    const int64_t ubase = static_cast<int64_t>(u) * a.capacity;
    const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(a.codes);

    // rows (then params) of one tile into registers: word i of the tile's rows
    // is row word i of the store from the tile's first row; zero past the end
    // Tiles whose rows (and params) fit in 16 words per lane take a
    // branch-free path: every lane loads (address clamped to the tile's last
    // valid row or parameter word) and stashes all RW words into a rows area
    // sized for them.  Words past the valid rows repeat a valid word: they only
    // feed token columns that are not stored, or padding slots whose W is
    // exactly zero (codes and fp16 params of valid rows are finite), so they
    // need no masking, and the loaded values are not touched until the tile is
    // stashed.  Without per-lane branches or selects the wait counts stay exact
    // and the ring's other tiles stay in flight.
    constexpr bool kFlat = fetch_flat<MIXED, KS, RW, NW>();
    auto fetch_tile = [&](int tile, uint32_t (&r)[RW]) {
        const int64_t s = a.s_begin + static_cast<int64_t>(tile) * kFetTok;
        const int valid = static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
        const uint32_t *src = codes32 + (ubase + s) * row_words;
        const uint32_t *psrc = MIXED ? a.params + (ubase + s) * a.n_qg : nullptr;
        const int vrow = valid * row_words, vpar = MIXED ? valid * a.n_qg : 0;
        if constexpr (kFlat) {
            if constexpr (MIXED) {
                // group-head: word i is a row word below row_tile_words, else a
                // parameter word; both addresses clamped to the valid part
#pragma unroll
                for (int k = 0; k < RW; ++k) {
                    const int i = k * 64 + lane;
                    const uint32_t *ra = src + min(i, max(vrow - 1, 0));
                    const uint32_t *pa = psrc + min(max(i - row_tile_words, 0), vpar - 1);
                    r[k] = *(i < row_tile_words && vrow > 0 ? ra : pa);
                }
            } else if (vrow > 0) {
#pragma unroll
                for (int k = 0; k < RW; ++k) r[k] = src[min(k * 64 + lane, vrow - 1)];
            } else {
#pragma unroll
                for (int k = 0; k < RW; ++k) r[k] = 0u;
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            const int i = k * 64 + lane;
            uint32_t v = 0u;
            if (i < row_tile_words) {
                if (i < vrow) v = src[i];
            } else if (MIXED && i < tile_words) {
                if (i - row_tile_words < vpar) v = psrc[i - row_tile_words];
            }
            r[k] = v;
        }
    };
    auto stash_tile = [&](const uint32_t (&r)[RW]) {
        if constexpr (kFlat) {
#pragma unroll
            for (int k = 0; k < RW; ++k) {
                rowsl[k * 64 + lane] = r[k];
                if constexpr (MIXED) {
                    // parameter word j = i - row_tile_words is (token j / n_qg, group
                    // j % n_qg), staged group-major; other lanes write a dummy word
                    // of their own past the parameters
                    const int i = k * 64 + lane, j = i - row_tile_words;
                    const int t = static_cast<int>((static_cast<float>(j) + 0.5f) * a.nqg_inv);
                    const bool is_par = i >= row_tile_words && i < tile_words;
                    parl[is_par ? (j - t * a.n_qg) * kFetTok + t : a.n_qg * kFetTok + lane] = r[k];
                }
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            const int i = k * 64 + lane;
            if (i < row_tile_words) {
                rowsl[i] = r[k];
            } else if (MIXED && i < tile_words) {
                // parameter word j of the tile is (token j / n_qg, group j % n_qg);
                // staged group-major so that a k-step's reads hit 32 banks
                const int j = i - row_tile_words;
                const int t = static_cast<int>((static_cast<float>(j) + 0.5f) * a.nqg_inv);
                parl[(j - t * a.n_qg) * kFetTok + t] = r[k];
            }
        }
    };

    const int tok = lane & 31;            // B-operand column / C column of this lane
    const uint32_t half_k = lane >> 5;    // this lane feeds fetch slots 8..15 of a k-step if set

    // the unit's k-step descriptors (first field offset, width, quantisation
    // group), block-uniform, held in scalar registers for all tiles; k-steps
    // past this tensor's own count (a launch shared with a wider tensor) are empty
    uint32_t kd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kd[ks] = ks < a.nks ? __builtin_amdgcn_readfirstlane(a.kdesc[static_cast<int64_t>(u) * a.nks + ks]) : 0u;

    auto process = [&](int tile, auto full) {
        constexpr bool kFull = decltype(full)::value;
        const int64_t s = a.s_begin + static_cast<int64_t>(tile) * kFetTok;
        const int valid = kFull ? kFetTok : static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
        __builtin_amdgcn_wave_barrier();
        floatx16 acc[NDB];
        seed_bias<NDB>(acc, biasl, half_k);
        const uint32_t *myrow = rowsl + tok * row_words;
        const uint32_t *mypar = MIXED ? parl + tok : nullptr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (((kd[ks] >> 16) & 0xFu) == 0u) continue;          // empty k-step (wave-uniform)
            const half8 bv = decode_kstep<MIXED>(kd[ks], myrow, mypar, half_k);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const half8 av = *reinterpret_cast<const half8 *>(wl + (db * 32 + tok) * a.wpitch + ks * 16 + half_k * 8);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[db], 0, 0, 0);
            }
        }
        _Float16 *orow = a.out + b * a.osb + head * a.osh + (s - a.s_begin) * a.oss + dd0;
#pragma unroll
        for (int hb = 0; hb < NDB; hb += NH)
            store_tile<NH, kFull>(acc + hb, outl, a.opitch, lane, orow + hb * 32, a.oss, valid);
    };

    // wave w takes tiles w, w + NW, ...; the rows of the next PF of them are in
    // flight in a register ring.  A wave's loads and stores retire in order, so
    // waiting for a tile's rows also waits for every store issued before those
    // rows were requested: with PF tiles in flight that is the stores of PF
    // tiles back, which overlaps the store latency with PF tiles of work.
    // Branch-free path: the main loop covers whole tiles only and its body
    // has no conditions (prefetches past the run are clamped to its last tile
    // and never processed), so the compiler keeps exact wait counts across
    // it; the last partial round and a ragged final tile run after it.
    const int t0 = tile_begin + wave;
    const int last = tile_end - 1;
    uint32_t ring[PF][RW];
    if constexpr (!kFlat) {
        // rows with parameters or wider than 8 words per lane: one loop with
        // per-tile conditions (keeps the register footprint of one tile body)
#pragma unroll
        for (int p = 0; p < PF; ++p)
            if (t0 + p * NW < tile_end) fetch_tile(t0 + p * NW, ring[p]);
        for (int tile = t0; tile < tile_end; tile += PF * NW) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                const int tt = tile + p * NW;
                if (tt < tile_end) {
                    stash_tile(ring[p]);
                    if (tt + PF * NW < tile_end) fetch_tile(tt + PF * NW, ring[p]);
                    process(tt, std::false_type{});
                }
            }
        }
        return;
    }
    const bool ragged_end = a.s_begin + static_cast<int64_t>(tile_end) * kFetTok > a.s_end;
    const int full_end = ragged_end ? tile_end - 1 : tile_end;
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (t0 <= last) fetch_tile(min(t0 + p * NW, last), ring[p]);
    int tile = t0;
    for (; tile + (PF - 1) * NW < full_end; tile += PF * NW) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int tt = tile + p * NW;
            stash_tile(ring[p]);
            fetch_tile(min(tt + PF * NW, last), ring[p]);
            process(tt, std::true_type{});
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int tt = tile + p * NW;
        if (tt < tile_end) {
            stash_tile(ring[p]);
            process(tt, std::false_type{});
        }
    }
}

// ============================================================== decode attention
// Attention of one query per (b, h) over the stored keys and values, computed
// from the codes (TurboQuant cache module page, attend: scores of the query
// against every stored key divided by sqrt(d), softmax over the stored rows,
// weighted sum of the decoded values; PALU cache API page, "Design": latents
// are reconstructed only for attention).  With the DP dequantisation
// l_j = min_j + c_j*scale_j and x = sum_j l_j V_j + mu, the score of row s is
//   q.x_s / sqrt(D) = sum_j c_sj * qt_j + beta,
//   qt_j = scale_j (q.V_j) / sqrt(D),  beta = (q.mu + sum_j min_j (q.V_j)) / sqrt(D),
// and the output is sum_s p_s x_s = sum_j abar_j scale_j V_j + bias with
// abar_j = sum_s p_s c_sj (softmax weights p summing to one), so neither keys nor
// values are ever reconstructed per row.  The rows are split into chunks whose
// partial softmax statistics (max, sum, weighted code sums) are merged per unit.
constexpr int kAttChunk = 512;       // rows per partial block
constexpr int kAttKsK = 16;          // k-steps of the key contraction (kfetch <= 256)

struct AttendSide {
    const uint8_t *codes;
    int64_t capacity;
    const kvtc_unit_info *ui;
    const float *basis, *mu, *qmin, *qscale, *bias;
    const int32_t *comp;
    const uint32_t *sbits;
    const uint32_t *kdesc;             // fetch k-step descriptors [U][kfetch/16]
    const int32_t *fslot;              // stored slot of fetch column k [U][kfetch]
    int kslots, rmax, row_words, kfetch;
};

struct AttendArgs {
    AttendSide k, v;
    const void *q;
    int64_t qsb, qsh;
    int q_f16;
    _Float16 *out;
    int64_t osb, osh;
    int64_t s_end;
    int nchunks, H, D;
    float inv_sqrt_d;
    float *qt;          // [U][k.kslots + 1]: qt_j, then beta
    uint16_t *qf;       // [U][2][k.kfetch]: fp16 high and low parts of qt * 2^-e, fetch order
    float *qmul;        // [U]: 2^e
    float *part;        // [U][nchunks][v.kslots + 2]: abar partial sums, then max, sum
};

__device__ inline uint32_t row_field(const uint32_t *row, uint32_t sb) {
    const uint32_t off = sb & kOffsetMask, w = sb >> 24;
    const uint32_t wi = off >> 5, sh = off & 31u;
    return __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh) & ((1u << w) - 1u);
}

__device__ inline float block_reduce(float v, float *red, bool is_max) {
    for (int m = 32; m >= 1; m >>= 1) {
        const float o = __shfl_xor(v, m, 64);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// Per unit: the query's score coefficients qt_j and offset beta (fp32).
__global__ __launch_bounds__(256) void attend_prep_kernel(AttendArgs a) {
    __shared__ float ql[kMaxSlots];
    __shared__ float mpart[kMaxSlots];
    const int u = blockIdx.x, b = u / a.H, h = u % a.H, tid = threadIdx.x;
    for (int d = tid; d < a.D; d += blockDim.x)
        ql[d] = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[b * a.qsb + h * a.qsh + d])
                        : static_cast<const float *>(a.q)[b * a.qsb + h * a.qsh + d];
    __syncthreads();
    const AttendSide &k = a.k;
    const int ns = k.ui[u].n_slots;
    float qt = 0.f, mp = 0.f;
    if (tid < ns) {
        const float *vrow = k.basis + (static_cast<int64_t>(u) * k.kslots + tid) * a.D;
        float acc = 0.f;
        for (int d = 0; d < a.D; ++d) acc = fmaf(ql[d], vrow[d], acc);
        const int c = k.comp[static_cast<int64_t>(u) * k.kslots + tid];
        qt = k.qscale[static_cast<int64_t>(u) * k.rmax + c] * acc * a.inv_sqrt_d;
        mp = k.qmin[static_cast<int64_t>(u) * k.rmax + c] * acc;
    }
    __shared__ float qts[kMaxSlots];
    __shared__ float red[4];
    if (tid < k.kslots) {
        a.qt[static_cast<int64_t>(u) * (k.kslots + 1) + tid] = qt;
        mpart[tid] = mp;
        qts[tid] = qt;
    }
    // the scorer's operands in fetch order: qt * 2^-e as an fp16 high part and an
    // fp16 remainder, with 2^e > max |qt| so that neither overflows (padding
    // columns are zero)
    const float amax = block_reduce(fabsf(qt), red, true);
    int e = 0;
    if (amax > 0.f) frexpf(amax, &e);
    for (int kk = tid; kk < k.kfetch; kk += blockDim.x) {
        const int j = k.fslot[static_cast<int64_t>(u) * k.kfetch + kk];
        const float v = j >= 0 ? ldexpf(qts[j], -e) : 0.f;
        const _Float16 hi = static_cast<_Float16>(v);
        const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
        a.qf[(static_cast<int64_t>(u) * 2 + 0) * k.kfetch + kk] = __builtin_bit_cast(uint16_t, hi);
        a.qf[(static_cast<int64_t>(u) * 2 + 1) * k.kfetch + kk] = __builtin_bit_cast(uint16_t, lo);
    }
    if (tid == 0) {
        a.qmul[u] = ldexpf(1.0f, e);
        float beta = 0.f;
        for (int d = 0; d < a.D; ++d) beta = fmaf(ql[d], k.mu[static_cast<int64_t>(u) * a.D + d], beta);
        for (int j = 0; j < k.kslots; ++j) beta += mpart[j];
        a.qt[static_cast<int64_t>(u) * (k.kslots + 1) + k.kslots] = beta * a.inv_sqrt_d;
    }
}

// Per (chunk of kAttChunk rows, unit): scores from the key codes, the chunk's
// softmax max and sum, and the p-weighted sums of the value codes.  Rows are
// staged in LDS at an odd pitch of at least row_words + 1 words: a thread per
// row then reads without bank conflicts, and every row ends in a slack word for
// its last field window (fields end inside the row, so the slack word's bits
// are always masked off).
__global__ __launch_bounds__(256) void attend_partial_kernel(AttendArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AttendSide &K = a.k, &V = a.v;
    float *qt_l = reinterpret_cast<float *>(smem);                       // [K.kslots + 1]
    uint32_t *ksb = reinterpret_cast<uint32_t *>(qt_l + kMaxSlots + 4);  // [2][K.kfetch] fp16 (16-byte aligned)
    uint32_t *vsb = ksb + kMaxSlots;                                     // [V.kslots]
    float *pl = reinterpret_cast<float *>(vsb + kMaxSlots);              // [kAttChunk]
    float *red = pl + kAttChunk;                                         // [4][kMaxSlots]
    uint32_t *rows = reinterpret_cast<uint32_t *>(red + 4 * kMaxSlots);  // [kAttChunk][pitch]
    const int64_t s0 = static_cast<int64_t>(c) * kAttChunk;
    const int nrows = static_cast<int>(min<int64_t>(kAttChunk, a.s_end - s0));
    const int nv = V.ui[u].n_slots;
    // word i of a chunk's rows goes to (i / row_words, i % row_words); the
    // quotient from a float reciprocal is exact for i < 2^16
    auto stage = [&](const AttendSide &T, int pitch) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(T.codes) + (static_cast<int64_t>(u) * T.capacity + s0) * T.row_words;
        const float inv = 1.0f / static_cast<float>(max(T.row_words, 1));
        for (int i = tid; i < nrows * T.row_words; i += blockDim.x) {
            const int r = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
            rows[r * pitch + (i - r * T.row_words)] = src[i];
        }
    };
    const int kp = (K.row_words + 1) | 1, vp = (V.row_words + 1) | 1;   // odd, > row_words

    for (int i = tid; i <= K.kslots; i += blockDim.x) qt_l[i] = a.qt[static_cast<int64_t>(u) * (K.kslots + 1) + i];
    {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.qf + static_cast<int64_t>(u) * 2 * K.kfetch);
        for (int i = tid; i < K.kfetch; i += blockDim.x) ksb[i] = src[i];   // 2*kfetch halves
    }
    for (int i = tid; i < V.kslots; i += blockDim.x) vsb[i] = V.sbits[static_cast<int64_t>(u) * V.kslots + i];
    stage(K, kp);
    __syncthreads();

    // scores of this thread's two rows, k-step by k-step in the fetch order: the
    // fetch kernel's field decode gives a k-step's 16 codes as exact fp16 values,
    // which are dotted (fp32 accumulation) with the high and low fp16 parts of the
    // prescaled coefficients; rows past the chunk are decoded from stale words and
    // never stored, and padding columns have zero coefficients
    float mloc = -__builtin_huge_valf();
    {
        uint32_t kd[kAttKsK];
        const int nksK = K.kfetch / 16;
#pragma unroll
        for (int ks = 0; ks < kAttKsK; ++ks)
            kd[ks] = ks < nksK ? __builtin_amdgcn_readfirstlane(K.kdesc[static_cast<int64_t>(u) * nksK + ks]) : 0u;
        const _Float16 *qh = reinterpret_cast<const _Float16 *>(ksb), *ql = qh + K.kfetch;
        const int r0 = tid, r1 = tid + 256;
        const uint32_t *row0 = rows + r0 * kp, *row1 = rows + r1 * kp;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int ks = 0; ks < kAttKsK; ++ks) {
            if (((kd[ks] >> 16) & 0xFu) == 0u) continue;               // empty k-step (uniform)
#pragma unroll
            for (uint32_t hk = 0; hk < 2; ++hk) {
                const half8 h8 = *reinterpret_cast<const half8 *>(qh + ks * 16 + hk * 8);
                const half8 l8 = *reinterpret_cast<const half8 *>(ql + ks * 16 + hk * 8);
                const half8 c0 = decode_kstep<false>(kd[ks], row0, nullptr, hk);
                const half8 c1 = decode_kstep<false>(kd[ks], row1, nullptr, hk);
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const half2 hv = {h8[e], h8[e + 1]}, lv = {l8[e], l8[e + 1]};
                    const half2 v0 = {c0[e], c0[e + 1]}, v1 = {c1[e], c1[e + 1]};
                    acc0 = __builtin_amdgcn_fdot2(v0, hv, acc0, false);
                    acc0 = __builtin_amdgcn_fdot2(v0, lv, acc0, false);
                    acc1 = __builtin_amdgcn_fdot2(v1, hv, acc1, false);
                    acc1 = __builtin_amdgcn_fdot2(v1, lv, acc1, false);
                }
            }
        }
        const float beta = qt_l[K.kslots], mul = a.qmul[u];
        acc0 = fmaf(acc0, mul, beta);
        acc1 = fmaf(acc1, mul, beta);
        if (r0 < nrows) {
            pl[r0] = acc0;
            mloc = acc0;
        }
        if (r1 < nrows) {
            pl[r1] = acc1;
            mloc = fmaxf(mloc, acc1);
        }
    }
    const float M = block_reduce(mloc, red, true);     // (its barriers also end the score phase)
    float lsum = 0.f;
    for (int r = tid; r < nrows; r += blockDim.x) {
        const float p = expf(pl[r] - M);
        pl[r] = p;
        lsum += p;
    }
    stage(V, vp);
    const float L = block_reduce(lsum, red, false);
    __syncthreads();

    // p-weighted sums of the value codes: wave w takes rows w, w+4, ...; lane
    // takes slots lane + 64t
    float acc[kMaxSlots / 64];
    uint32_t mysb[kMaxSlots / 64];
#pragma unroll
    for (int t = 0; t < kMaxSlots / 64; ++t) {
        acc[t] = 0.f;
        mysb[t] = lane + 64 * t < nv ? vsb[lane + 64 * t] : 0u;
    }
    const int ngroups = (nv + 63) >> 6;                // wave-uniform
    for (int r = wave; r < nrows; r += 4) {
        const float p = pl[r];
        const uint32_t *row = rows + r * vp;
#pragma unroll
        for (int t = 0; t < kMaxSlots / 64; ++t)
            if (t < ngroups) acc[t] = fmaf(p, static_cast<float>(row_field(row, mysb[t])), acc[t]);
    }
    __syncthreads();                                   // the reductions' scratch is reused below
#pragma unroll
    for (int t = 0; t < kMaxSlots / 64; ++t) red[wave * kMaxSlots + lane + 64 * t] = acc[t];
    __syncthreads();
    float *dst = a.part + (static_cast<int64_t>(u) * a.nchunks + c) * (V.kslots + 2);
    for (int j = tid; j < V.kslots; j += blockDim.x)
        dst[j] = (red[j] + red[kMaxSlots + j]) + (red[2 * kMaxSlots + j] + red[3 * kMaxSlots + j]);
    if (tid == 0) {
        dst[V.kslots] = M;
        dst[V.kslots + 1] = L;
    }
}

// Per unit: merge the chunks' softmax statistics, then reconstruct the output
// once: out = bias + sum_j (abar_j scale_j) V_j, rounded to fp16.
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a) {
    __shared__ float coef[kMaxSlots];
    __shared__ float red[4];
    const int u = blockIdx.x, b = u / a.H, h = u % a.H, tid = threadIdx.x;
    const AttendSide &V = a.v;
    const int nv = V.ui[u].n_slots, stride = V.kslots + 2;
    const float *part = a.part + static_cast<int64_t>(u) * a.nchunks * stride;
    float m = -__builtin_huge_valf();
    for (int c = tid; c < a.nchunks; c += blockDim.x) m = fmaxf(m, part[c * stride + V.kslots]);
    const float M = block_reduce(m, red, true);
    float l = 0.f;
    for (int c = tid; c < a.nchunks; c += blockDim.x)
        l += expf(part[c * stride + V.kslots] - M) * part[c * stride + V.kslots + 1];
    const float L = block_reduce(l, red, false);
    if (tid < V.kslots) {
        float s = 0.f;
        if (tid < nv) {
            for (int c = 0; c < a.nchunks; ++c) s = fmaf(expf(part[c * stride + V.kslots] - M), part[c * stride + tid], s);
            const int ci = V.comp[static_cast<int64_t>(u) * V.kslots + tid];
            s = s / L * V.qscale[static_cast<int64_t>(u) * V.rmax + ci];
        }
        coef[tid] = s;
    }
    __syncthreads();
    for (int d = tid; d < a.D; d += blockDim.x) {
        float o = 0.f;
        if (a.nchunks > 0) {
            o = V.bias[static_cast<int64_t>(u) * a.D + d];
            const float *vb = V.basis + static_cast<int64_t>(u) * V.kslots * a.D + d;
            for (int j = 0; j < nv; ++j) o = fmaf(coef[j], vb[static_cast<int64_t>(j) * a.D], o);
        }
        a.out[b * a.osb + h * a.osh + d] = static_cast<_Float16>(o);
    }
}

// ============================================================== launchers
constexpr int kLdsMax = 160 * 1024;

// Lets a kernel use up to the whole LDS of a CU as dynamic shared memory.  The
// attribute belongs to the kernel, not to a call, so it is set once per kernel
// (and per device; the set is an idempotent per-process cache of that fact).
bool allow_lds(const void *kern) {
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kern, dev})) return true;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess) return false;
    done.insert({kern, dev});
    return true;
}

int append_nb(int kslots) {
    const int need = kslots / 16;
    const int opts[] = {1, 2, 4, 6, 8, 12, 16};
    for (int o : opts)
        if (o >= need) return o;
    return -1;
}

template <bool MIXED, typename XT, int NB>
int32_t launch_append_nb(const AppendArgs &a, int64_t ntiles, int64_t U, hipStream_t stream) {
    const size_t lds = 2 * kAppTok * kAppPad * sizeof(double) + 2 * NB * 16 * kAppPad * sizeof(float) +
                       static_cast<size_t>(kAppTok) * (a.row_stride / 4) * sizeof(uint32_t);
    auto kern = a.x_vec ? append_kernel<MIXED, XT, NB, true> : append_kernel<MIXED, XT, NB, false>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(ntiles), static_cast<unsigned>(U)), dim3(kThreads), lds,
                       stream, a);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

constexpr int kSmallRows = 16;
constexpr size_t kSmallLdsLimit = 96 * 1024;

size_t small_lds_bytes(int dg, int nb, int row_stride) {
    return 16 * static_cast<size_t>(dg + 1) * sizeof(double) + static_cast<size_t>(nb) * 16 * (dg + 1) * sizeof(float) +
           16 * static_cast<size_t>(row_stride / 4) * sizeof(uint32_t);
}

template <typename XT, int NB>
int32_t launch_small_nb(const AppendArgs &a, int64_t U, hipStream_t stream) {
    const size_t lds = small_lds_bytes(a.dg, NB, a.row_stride);
    auto kern = append_small_kernel<XT, NB>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    const int64_t blocks = (a.n + kSmallRows - 1) / kSmallRows;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(U)), dim3(kThreads), lds,
                       stream, a);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

template <typename XT>
int32_t launch_small(const AppendArgs &a, int64_t U, int nb, hipStream_t st) {
    switch (nb) {
        case 1: return launch_small_nb<XT, 1>(a, U, st);
        case 2: return launch_small_nb<XT, 2>(a, U, st);
        case 4: return launch_small_nb<XT, 4>(a, U, st);
        case 6: return launch_small_nb<XT, 6>(a, U, st);
        case 8: return launch_small_nb<XT, 8>(a, U, st);
        case 12: return launch_small_nb<XT, 12>(a, U, st);
        case 16: return launch_small_nb<XT, 16>(a, U, st);
        default: return KVTC_E_SHAPE;
    }
}

template <bool MIXED, typename XT>
int32_t launch_append(const AppendArgs &a, int64_t ntiles, int64_t U, int nb, hipStream_t st) {
    if (!MIXED && a.n <= kSmallRows && small_lds_bytes(a.dg, nb, a.row_stride) <= kSmallLdsLimit)
        return launch_small<XT>(a, U, nb, st);
    switch (nb) {
        case 1: return launch_append_nb<MIXED, XT, 1>(a, ntiles, U, st);
        case 2: return launch_append_nb<MIXED, XT, 2>(a, ntiles, U, st);
        case 4: return launch_append_nb<MIXED, XT, 4>(a, ntiles, U, st);
        case 6: return launch_append_nb<MIXED, XT, 6>(a, ntiles, U, st);
        case 8: return launch_append_nb<MIXED, XT, 8>(a, ntiles, U, st);
        case 12: return launch_append_nb<MIXED, XT, 12>(a, ntiles, U, st);
        case 16: return launch_append_nb<MIXED, XT, 16>(a, ntiles, U, st);
        default: return KVTC_E_SHAPE;
    }
}

template <bool MIXED, int NDB, int KS, int RW>
int32_t launch_fetch_rw(FetchPair m, int nt, hipStream_t stream) {
    constexpr int DS = 32 * NDB, NW = fetch_waves<NDB, KS>();
    constexpr int NH = fetch_epilogue_blocks<NDB, NW>();
    size_t lds = 0;
    for (int i = 0; i < nt; ++i) {
        FetchArgs &a = m.t[i];
        if (kFetTok * (a.row_stride / 4 + (MIXED ? a.n_qg : 0)) > 64 * RW) return KVTC_E_SHAPE;
        a.wpitch = a.kfetch + 8;
        a.opitch = 32 * NH + 8;
        a.lds_w = 0;
        a.lds_desc = static_cast<int>(align_up(static_cast<uint64_t>(DS) * a.wpitch * 2, 16));
        a.lds_bias = static_cast<int>(align_up(a.lds_desc + 16, 16));
        a.lds_wave = static_cast<int>(align_up(a.lds_bias + DS * 4, 16));
        // rows of a tile back to back, plus slack for the 3-word field window of the
        // upper operand half of a padded k-step (the branch-free path stashes all
        // RW words per lane, so its rows area holds at least that many)
        int rows_b = static_cast<int>(align_up((kFetTok * (a.row_stride / 4) + 8) * 4, 16));
        if (fetch_flat<MIXED, KS, RW, NW>()) rows_b = std::max(rows_b, RW * 64 * 4);
        // (plus one dummy word per lane for the branch-free stash)
        const int par_b = MIXED ? static_cast<int>(align_up((kFetTok * a.n_qg + 64) * 4, 16)) : 0;
        const int out_b = static_cast<int>(align_up(kFetTok * a.opitch * 2, 16));
        a.lds_par = rows_b;
        a.lds_out = rows_b + par_b;
        a.lds_rows = rows_b + par_b + out_b;                 // per-wave bytes
        lds = std::max(lds, a.lds_wave + NW * static_cast<size_t>(a.lds_rows));
    }
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    const int64_t grid = m.nblocks_per_xcd * 8;
    auto kern = fetch_kernel<MIXED, NDB, KS, RW, NW, fetch_prefetch<MIXED, RW>()>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * NW), lds, stream, m);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

// Register staging of a tile's rows: the narrowest instantiated width that
// holds them (whole-head tiles: 8, 16 or 24 words per lane; 64-column: 8 or 24).
template <bool MIXED, int NDB, int KS>
int32_t launch_fetch_ks(const FetchPair &m, int nt, int rw, hipStream_t stream) {
    if (rw <= 8) return launch_fetch_rw<MIXED, NDB, KS, 8>(m, nt, stream);
    if (NDB == 4 && rw <= 16) return launch_fetch_rw<MIXED, NDB, KS, (NDB == 4 ? 16 : 24)>(m, nt, stream);
    if (rw <= kFetchRegWords) return launch_fetch_rw<MIXED, NDB, KS, kFetchRegWords>(m, nt, stream);
    return KVTC_E_SHAPE;
}

template <bool MIXED, int NDB>
int32_t launch_fetch(const FetchPair &m, int nt, int ks, int rw, hipStream_t stream) {
    switch (ks) {
        case 1: return launch_fetch_ks<MIXED, NDB, 1>(m, nt, rw, stream);
        case 2: return launch_fetch_ks<MIXED, NDB, 2>(m, nt, rw, stream);
        case 3: return launch_fetch_ks<MIXED, NDB, 3>(m, nt, rw, stream);
        case 4: return launch_fetch_ks<MIXED, NDB, 4>(m, nt, rw, stream);
        case 5: return launch_fetch_ks<MIXED, NDB, 5>(m, nt, rw, stream);
        case 6: return launch_fetch_ks<MIXED, NDB, 6>(m, nt, rw, stream);
        case 7: return launch_fetch_ks<MIXED, NDB, 7>(m, nt, rw, stream);
        case 8: return launch_fetch_ks<MIXED, NDB, 8>(m, nt, rw, stream);
        case 9: return launch_fetch_ks<MIXED, NDB, 9>(m, nt, rw, stream);
        case 10: return launch_fetch_ks<MIXED, NDB, 10>(m, nt, rw, stream);
        case 11: return launch_fetch_ks<MIXED, NDB, 11>(m, nt, rw, stream);
        case 12: return launch_fetch_ks<MIXED, NDB, 12>(m, nt, rw, stream);
        case 13: return launch_fetch_ks<MIXED, NDB, 13>(m, nt, rw, stream);
        case 14: return launch_fetch_ks<MIXED, NDB, 14>(m, nt, rw, stream);
        case 15: return launch_fetch_ks<MIXED, NDB, 15>(m, nt, rw, stream);
        case 16: return launch_fetch_ks<MIXED, NDB, 16>(m, nt, rw, stream);
        default: return KVTC_E_SHAPE;
    }
}

// ============================================================== call plans
// Everything a call needs to launch, after its arguments have been validated.
struct AppendPlan {
    AppendArgs a;
    int64_t units, ntiles;
    int nb;                            // 16-slot N-blocks of the bulk kernels
    int32_t dtype;
    bool mixed;
};

struct FetchPlan {
    FetchArgs a;
    int ds, rw;                        // columns per block (128 or 64), row words per lane
    bool mixed;
};

int32_t plan_append(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                    const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0,
                    void *codes_dev, void *params_dev, int64_t capacity, AppendPlan *p) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (!state_dev || !x_strides) return KVTC_E_ARG;
    if (dtype != KVTC_F16 && dtype != KVTC_F32) return KVTC_E_DTYPE;
    if (B != h->batch || H != h->heads) return KVTC_E_SHAPE;
    if (x_strides[3] != 1 || x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0) return KVTC_E_SHAPE;
    if (n < 0 || s0 < 0 || capacity < 0) return KVTC_E_ARG;
    if (s0 + n > capacity) return KVTC_E_CAPACITY;
    if (h->kslots > kMaxSlots || h->row_stride > kMaxRowStride || h->dg % kAppKC != 0 ||
        h->head_dim % kAppKC != 0 || h->units > 65535)
        return KVTC_E_SHAPE;
    const bool mixed = h->mode == KVTC_MODE_MIXED;
    if (mixed && h->group_size % 16 != 0) return KVTC_E_STATE;
    *p = AppendPlan{};
    p->a.n = n;
    if (n == 0) return KVTC_OK;
    if (!x_dev) return KVTC_E_ARG;
    if (h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4 != 0)) return KVTC_E_ARG;
    if (mixed && (!params_dev || reinterpret_cast<uintptr_t>(params_dev) % 4 != 0)) return KVTC_E_ARG;
    const int nb = append_nb(h->kslots);
    if (nb < 0) return KVTC_E_SHAPE;
    const int64_t ntiles = (n + kAppTok - 1) / kAppTok;
    if (ntiles > 0x7FFFFFFF) return KVTC_E_SHAPE;

    const char *sd = static_cast<const char *>(state_dev);
    AppendArgs &a = p->a;
    a.x = x_dev;
    a.xsb = x_strides[0];
    a.xsh = x_strides[1];
    a.xss = x_strides[2];
    a.s0 = s0;
    a.capacity = capacity;
    a.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    a.mu = reinterpret_cast<const float *>(sd + h->off_mu);
    a.basis = reinterpret_cast<const float *>(sd + h->off_basis);
    a.qlo = reinterpret_cast<const double *>(sd + h->off_qlo);
    a.qinv = reinterpret_cast<const double *>(sd + h->off_qinv);
    a.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    a.codes = static_cast<uint8_t *>(codes_dev);
    a.params = static_cast<uint32_t *>(params_dev);
    a.dg = h->dg;
    a.D = h->head_dim;
    a.hpu = h->heads_per_unit;
    a.groups = static_cast<int>(h->heads / h->heads_per_unit);
    a.kslots = h->kslots;
    a.row_stride = h->row_stride;
    a.n_qg = h->n_qgroups;
    a.gs = h->group_size;
    {
        const int64_t esz = dtype == KVTC_F16 ? 2 : 4;
        a.x_vec = reinterpret_cast<uintptr_t>(x_dev) % (4 * esz) == 0 && x_strides[0] % 4 == 0 &&
                  x_strides[1] % 4 == 0 && x_strides[2] % 4 == 0;
    }
    a.inv_dg = 1.0f / static_cast<float>(h->dg);
    a.inv_q4 = 4.0f / static_cast<float>(h->dg);
    p->units = h->units;
    p->ntiles = ntiles;
    p->nb = nb;
    p->dtype = dtype;
    p->mixed = mixed;
    return KVTC_OK;
}

// Decode appends of DP tensors (one head per unit) whose unit width has a
// register-resident kernel; one wave per 16 slots, at most dg slots.
bool decode_path(const AppendPlan &p) {
    return !p.mixed && p.a.n <= kSmallRows && p.a.hpu == 1 && (p.a.dg == 64 || p.a.dg == 128) &&
           p.a.kslots <= p.a.dg;
}

template <typename XT, int DG>
int32_t launch_decode_dg(const AppendPair &m, int64_t nrows, int64_t units, int nblk, hipStream_t stream) {
    int row_stride = 0;
    for (int i = 0; i < (m.split < units ? 2 : 1); ++i) row_stride = std::max(row_stride, m.t[i].row_stride);
    const size_t lds = decode_lds_bytes(DG, row_stride);
    auto kern = append_decode_kernel<XT, DG>;
    const int64_t blocks = (nrows + kSmallRows - 1) / kSmallRows;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(units)), dim3(64 * nblk), lds,
                       stream, m);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

// One decode launch for one plan (p1 == NULL) or for two plans of the same
// element type and unit width (rows of every unit of p0, then of p1).
int32_t launch_decode(const AppendPlan &p0, const AppendPlan *p1, hipStream_t stream) {
    AppendPair m{};
    m.t[0] = p0.a;
    m.split = p0.units;
    int64_t units = p0.units;
    int nblk = p0.a.kslots / 16;
    if (p1) {
        m.t[1] = p1->a;
        units += p1->units;
        nblk = std::max(nblk, p1->a.kslots / 16);
    }
    if (units > 65535) return KVTC_E_SHAPE;
    const bool f16 = p0.dtype == KVTC_F16;
    if (p0.a.dg == 128)
        return f16 ? launch_decode_dg<_Float16, 128>(m, p0.a.n, units, nblk, stream)
                   : launch_decode_dg<float, 128>(m, p0.a.n, units, nblk, stream);
    return f16 ? launch_decode_dg<_Float16, 64>(m, p0.a.n, units, nblk, stream)
               : launch_decode_dg<float, 64>(m, p0.a.n, units, nblk, stream);
}

int32_t launch_append_plan(const AppendPlan &p, hipStream_t stream) {
    if (p.a.n == 0) return KVTC_OK;
    if (decode_path(p)) return launch_decode(p, nullptr, stream);
    if (p.dtype == KVTC_F16)
        return p.mixed ? launch_append<true, _Float16>(p.a, p.ntiles, p.units, p.nb, stream)
                       : launch_append<false, _Float16>(p.a, p.ntiles, p.units, p.nb, stream);
    return p.mixed ? launch_append<true, float>(p.a, p.ntiles, p.units, p.nb, stream)
                   : launch_append<false, float>(p.a, p.ntiles, p.units, p.nb, stream);
}

// share: how many tensors the launch is shared by (1 or 2); the block target
// of one launch is split between them
int32_t plan_fetch(const void *state_host, const void *state_dev, const void *codes_dev, const void *params_dev,
                   int64_t capacity, int64_t s_begin, int64_t s_end, void *out_dev, const int64_t out_strides[4],
                   FetchPlan *p, int share = 1) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (!state_dev || !out_strides) return KVTC_E_ARG;
    if (capacity < 0 || s_begin < 0 || s_end < s_begin) return KVTC_E_ARG;
    if (s_end > capacity) return KVTC_E_CAPACITY;
    if (out_strides[3] != 1 || out_strides[0] < 0 || out_strides[1] < 0 || out_strides[2] < 0)
        return KVTC_E_SHAPE;
    const bool mixed = h->mode == KVTC_MODE_MIXED;
    if (h->kfetch > kMaxSlots || h->head_dim % 64 != 0) return KVTC_E_SHAPE;
    const int tw = h->row_stride / 4 + (mixed ? h->n_qgroups : 0);
    if (kFetTok * tw > 64 * kFetchRegWords) return KVTC_E_SHAPE;
    *p = FetchPlan{};
    if (s_end == s_begin) return KVTC_OK;
    if (!out_dev || reinterpret_cast<uintptr_t>(out_dev) % 16 != 0) return KVTC_E_ARG;
    if ((out_strides[0] * 2) % 16 || (out_strides[1] * 2) % 16 || (out_strides[2] * 2) % 16) return KVTC_E_SHAPE;
    if (h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4 != 0)) return KVTC_E_ARG;
    if (mixed && (!params_dev || reinterpret_cast<uintptr_t>(params_dev) % 4 != 0)) return KVTC_E_ARG;

    const char *sd = static_cast<const char *>(state_dev);
    FetchArgs &a = p->a;
    a.codes = static_cast<const uint8_t *>(codes_dev);
    a.params = static_cast<const uint32_t *>(params_dev);
    a.capacity = capacity;
    a.s_begin = s_begin;
    a.s_end = s_end;
    a.w16 = reinterpret_cast<const uint16_t *>(sd + h->off_w16);
    a.bias = reinterpret_cast<const float *>(sd + h->off_bias);
    a.kdesc = reinterpret_cast<const uint32_t *>(sd + h->off_kdesc);
    a.out = static_cast<_Float16 *>(out_dev);
    a.osb = out_strides[0];
    a.osh = out_strides[1];
    a.oss = out_strides[2];
    a.dg = h->dg;
    a.D = h->head_dim;
    a.hpu = h->heads_per_unit;
    a.groups = static_cast<int>(h->heads / h->heads_per_unit);
    a.kfetch = h->kfetch;
    a.nks = h->kfetch / 16;
    a.row_stride = h->row_stride;
    a.n_qg = h->n_qgroups;
    a.nqg_inv = mixed ? 1.0f / static_cast<float>(h->n_qgroups) : 0.0f;
    // a block covers whole output rows of a head (128 columns) where the head
    // size allows, so every token's fields are decoded once per head
    const int DS = (h->head_dim % 128 == 0) ? 128 : 64;
    a.nslices = h->dg / DS;
    const int64_t ntiles = (s_end - s_begin + kFetTok - 1) / kFetTok;
    if (ntiles > 0x7FFFFFFF) return KVTC_E_SHAPE;
    a.ntiles = static_cast<int>(ntiles);
    const int64_t work = h->units * a.nslices * ntiles;
    const int nw = (DS == 128 && h->kfetch >= 160) ? 8 : 4;
    // about two four-wave blocks, or one eight-wave block, per CU in one round
    // (shared between the tensors of a paired launch)
    const int64_t target = kFetchBlocks * 4 / nw / share;
    const int64_t tpb = std::min<int64_t>(std::max<int64_t>(nw, (work + target - 1) / target), ntiles);
    a.tiles_per_block = static_cast<int>(tpb);
    a.nchunks = static_cast<int>((ntiles + tpb - 1) / tpb);
    a.nblocks = h->units * a.nslices * a.nchunks;
    if (a.nblocks > 0x7FFFFFFF) return KVTC_E_SHAPE;
    p->ds = DS;
    p->rw = (kFetTok * tw + 63) / 64;
    p->mixed = mixed;
    return KVTC_OK;
}

// One fetch launch for one plan (p1 == NULL) or for two plans of the same
// mode and block width; the kernel is instantiated for the wider contraction.
int32_t launch_fetch_plans(const FetchPlan &p0, const FetchPlan *p1, hipStream_t stream) {
    FetchPair m{};
    m.t[0] = p0.a;
    m.split = p0.a.nblocks;
    m.nblocks_real = p0.a.nblocks;
    int ks = p0.a.nks, rw = p0.rw, nt = 1;
    if (p1) {
        m.t[1] = p1->a;
        m.nblocks_real += p1->a.nblocks;
        ks = std::max(ks, p1->a.nks);
        rw = std::max(rw, p1->rw);
        nt = 2;
    }
    m.nblocks_per_xcd = (m.nblocks_real + 7) / 8;
    if (m.nblocks_per_xcd * 8 > 0x7FFFFFFF) return KVTC_E_SHAPE;
    if (p0.ds == 128)
        return p0.mixed ? launch_fetch<true, 4>(m, nt, ks, rw, stream) : launch_fetch<false, 4>(m, nt, ks, rw, stream);
    return p0.mixed ? launch_fetch<true, 2>(m, nt, ks, rw, stream) : launch_fetch<false, 2>(m, nt, ks, rw, stream);
}

// Validation shared by the attention entry points: a DP tensor with one head
// per unit, head size and slot count within the kernels' limits.
int32_t attend_side_ok(const kvtc_state_header *h) {
    if (h->mode != KVTC_MODE_DP || h->heads_per_unit != 1) return KVTC_E_STATE;
    if (h->head_dim > kMaxSlots || h->kslots > kMaxSlots || h->kfetch > kMaxSlots || h->row_stride > kMaxRowStride)
        return KVTC_E_SHAPE;
    return KVTC_OK;
}

AttendSide attend_side(const kvtc_state_header *h, const void *state_dev, const void *codes, int64_t capacity) {
    const char *sd = static_cast<const char *>(state_dev);
    AttendSide sd_{};
    sd_.codes = static_cast<const uint8_t *>(codes);
    sd_.capacity = capacity;
    sd_.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    sd_.basis = reinterpret_cast<const float *>(sd + h->off_basis);
    sd_.mu = reinterpret_cast<const float *>(sd + h->off_mu);
    sd_.qmin = reinterpret_cast<const float *>(sd + h->off_qmin);
    sd_.qscale = reinterpret_cast<const float *>(sd + h->off_qscale);
    sd_.bias = reinterpret_cast<const float *>(sd + h->off_bias);
    sd_.comp = reinterpret_cast<const int32_t *>(sd + h->off_slot_comp);
    sd_.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    sd_.kdesc = reinterpret_cast<const uint32_t *>(sd + h->off_kdesc);
    sd_.fslot = reinterpret_cast<const int32_t *>(sd + h->off_fslot);
    sd_.kslots = h->kslots;
    sd_.rmax = h->rmax;
    sd_.row_words = h->row_stride / 4;
    sd_.kfetch = h->kfetch;
    return sd_;
}

// Workspace regions, each 256-byte aligned: qt [U][kslots_k + 1] f32,
// qf [U][2][kfetch_k] f16, qmul [U] f32, partial sums [U][nchunks][kslots_v + 2] f32.
struct AttendWork {
    uint64_t qt, qf, qmul, part, total;
};

AttendWork attend_work(const kvtc_state_header *hk, const kvtc_state_header *hv, int64_t s_end) {
    AttendWork w{};
    const int64_t nchunks = (s_end + kAttChunk - 1) / kAttChunk;
    w.qt = 0;
    w.qf = align_up(static_cast<uint64_t>(hk->units) * (hk->kslots + 1) * sizeof(float), 256);
    w.qmul = w.qf + align_up(static_cast<uint64_t>(hk->units) * 2 * hk->kfetch * sizeof(uint16_t), 256);
    w.part = w.qmul + align_up(static_cast<uint64_t>(hk->units) * sizeof(float), 256);
    w.total = w.part + static_cast<uint64_t>(hv->units) * nchunks * (hv->kslots + 2) * sizeof(float);
    return w;
}

size_t attend_work_bytes(const kvtc_state_header *hk, const kvtc_state_header *hv, int64_t s_end) {
    return attend_work(hk, hv, s_end).total;
}

}  // namespace
}  // namespace kvtc

using namespace kvtc;

extern "C" {

int32_t kvtc_append(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                    const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0,
                    void *codes_dev, void *params_dev, int64_t capacity, void *hip_stream) {
    AppendPlan p;
    const int32_t st = plan_append(state_host, state_dev, x_dev, dtype, x_strides, B, H, n, s0, codes_dev,
                                   params_dev, capacity, &p);
    if (st != KVTC_OK) return st;
    return launch_append_plan(p, static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_fetch(const void *state_host, const void *state_dev, const void *codes_dev,
                   const void *params_dev, int64_t capacity, int64_t s_begin, int64_t s_end,
                   void *out_dev, const int64_t out_strides[4], void *hip_stream) {
    FetchPlan p;
    const int32_t st = plan_fetch(state_host, state_dev, codes_dev, params_dev, capacity, s_begin, s_end, out_dev,
                                  out_strides, &p);
    if (st != KVTC_OK || s_end == s_begin) return st;
    return launch_fetch_plans(p, nullptr, static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_append_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t B, int64_t H, int64_t n,
                       int64_t s0, void *hip_stream) {
    if (!k || !v) return KVTC_E_ARG;
    AppendPlan pk, pv;
    int32_t st = plan_append(k->state_host, k->state_dev, k->rows_dev, k->dtype, k->strides, B, H, n, s0,
                             k->codes_dev, k->params_dev, k->capacity, &pk);
    if (st != KVTC_OK) return st;
    st = plan_append(v->state_host, v->state_dev, v->rows_dev, v->dtype, v->strides, B, H, n, s0, v->codes_dev,
                     v->params_dev, v->capacity, &pv);
    if (st != KVTC_OK || n == 0) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (decode_path(pk) && decode_path(pv) && pk.dtype == pv.dtype && pk.a.dg == pv.a.dg)
        return launch_decode(pk, &pv, stream);
    st = launch_append_plan(pk, stream);
    if (st != KVTC_OK) return st;
    return launch_append_plan(pv, stream);
}

int32_t kvtc_fetch_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t s_begin, int64_t s_end,
                      void *hip_stream) {
    if (!k || !v) return KVTC_E_ARG;
    FetchPlan pk, pv;
    int32_t st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                            k->rows_dev, k->strides, &pk);
    if (st != KVTC_OK) return st;
    st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                    v->rows_dev, v->strides, &pv);
    if (st != KVTC_OK || s_end == s_begin) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (pk.mixed == pv.mixed && pk.ds == pv.ds) {
        // one launch: re-plan both with the block target split between them
        st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                        k->rows_dev, k->strides, &pk, 2);
        if (st != KVTC_OK) return st;
        st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                        v->rows_dev, v->strides, &pv, 2);
        if (st != KVTC_OK) return st;
        return launch_fetch_plans(pk, &pv, stream);
    }
    st = launch_fetch_plans(pk, nullptr, stream);
    if (st != KVTC_OK) return st;
    return launch_fetch_plans(pv, nullptr, stream);
}

int32_t kvtc_attend_workspace(const void *k_state_host, const void *v_state_host, int64_t s_end, size_t *bytes) {
    const kvtc_state_header *hk = nullptr, *hv = nullptr;
    int32_t st = check_state(k_state_host, &hk);
    if (st != KVTC_OK) return st;
    st = check_state(v_state_host, &hv);
    if (st != KVTC_OK) return st;
    if (!bytes || s_end < 0) return KVTC_E_ARG;
    *bytes = attend_work_bytes(hk, hv, s_end);
    return KVTC_OK;
}

int32_t kvtc_attend(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                    const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                    void *work_dev, size_t work_bytes, void *hip_stream) {
    if (!k || !v || !q_strides || !out_strides) return KVTC_E_ARG;
    const kvtc_state_header *hk = nullptr, *hv = nullptr;
    int32_t st = check_state(k->state_host, &hk);
    if (st != KVTC_OK) return st;
    st = check_state(v->state_host, &hv);
    if (st != KVTC_OK) return st;
    if ((st = attend_side_ok(hk)) != KVTC_OK || (st = attend_side_ok(hv)) != KVTC_OK) return st;
    if (hk->batch != hv->batch || hk->heads != hv->heads || hk->head_dim != hv->head_dim) return KVTC_E_SHAPE;
    if (q_dtype != KVTC_F16 && q_dtype != KVTC_F32) return KVTC_E_DTYPE;
    if (q_strides[2] != 1 || out_strides[2] != 1 || q_strides[0] < 0 || q_strides[1] < 0 || out_strides[0] < 0 ||
        out_strides[1] < 0)
        return KVTC_E_SHAPE;
    if (s_end < 0 || k->capacity < 0 || v->capacity < 0) return KVTC_E_ARG;
    if (s_end > k->capacity || s_end > v->capacity) return KVTC_E_CAPACITY;
    if (!k->state_dev || !v->state_dev || !q_dev || !out_dev) return KVTC_E_ARG;
    if (s_end > 0 && ((hk->row_stride > 0 && (!k->codes_dev || reinterpret_cast<uintptr_t>(k->codes_dev) % 4)) ||
                      (hv->row_stride > 0 && (!v->codes_dev || reinterpret_cast<uintptr_t>(v->codes_dev) % 4))))
        return KVTC_E_ARG;
    if (reinterpret_cast<uintptr_t>(out_dev) % 2 || reinterpret_cast<uintptr_t>(q_dev) % (q_dtype == KVTC_F16 ? 2 : 4))
        return KVTC_E_ARG;
    const size_t need = attend_work_bytes(hk, hv, s_end);
    if (!work_dev || work_bytes < need || reinterpret_cast<uintptr_t>(work_dev) % 256) return KVTC_E_BUFSIZE;
    const int64_t nchunks = (s_end + kAttChunk - 1) / kAttChunk;
    if (hk->units > 0x7FFFFFFF || nchunks > 0x7FFFFFFF || hk->units > 65535) return KVTC_E_SHAPE;

    AttendArgs a{};
    a.k = attend_side(hk, k->state_dev, k->codes_dev, k->capacity);
    a.v = attend_side(hv, v->state_dev, v->codes_dev, v->capacity);
    a.q = q_dev;
    a.qsb = q_strides[0];
    a.qsh = q_strides[1];
    a.q_f16 = q_dtype == KVTC_F16;
    a.out = static_cast<_Float16 *>(out_dev);
    a.osb = out_strides[0];
    a.osh = out_strides[1];
    a.s_end = s_end;
    a.nchunks = static_cast<int>(nchunks);
    a.H = static_cast<int>(hk->heads);
    a.D = hk->head_dim;
    a.inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(hk->head_dim));
    const AttendWork wl = attend_work(hk, hv, s_end);
    char *wb = static_cast<char *>(work_dev);
    a.qt = reinterpret_cast<float *>(wb + wl.qt);
    a.qf = reinterpret_cast<uint16_t *>(wb + wl.qf);
    a.qmul = reinterpret_cast<float *>(wb + wl.qmul);
    a.part = reinterpret_cast<float *>(wb + wl.part);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const unsigned U = static_cast<unsigned>(hk->units);
    hipLaunchKernelGGL(attend_prep_kernel, dim3(U), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return KVTC_E_DEVICE;
    if (nchunks > 0) {
        const int rw = std::max(a.k.row_words, a.v.row_words);
        const size_t lds = (kMaxSlots + 4 + 2 * kMaxSlots + kAttChunk + 4 * kMaxSlots) * sizeof(float) +
                           (static_cast<size_t>(kAttChunk) * ((rw + 1) | 1) + 8) * sizeof(uint32_t);
        if (lds > kLdsMax) return KVTC_E_SHAPE;
        if (!allow_lds(reinterpret_cast<const void *>(attend_partial_kernel))) return KVTC_E_DEVICE;
        hipLaunchKernelGGL(attend_partial_kernel, dim3(static_cast<unsigned>(nchunks), U), dim3(256), lds, stream, a);
        if (hipGetLastError() != hipSuccess) return KVTC_E_DEVICE;
    }
    hipLaunchKernelGGL(attend_merge_kernel, dim3(U), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

}  // extern "C"
