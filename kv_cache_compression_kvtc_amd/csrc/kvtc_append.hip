// Append kernels of libkvtc for gfx950 (CDNA4) and their launchers.
//
// Append (KVTC cache module page, module docstring "Design", decode step 1;
// PALU cache API page, "Design", decode steps 1-2): every row is centred,
// projected through the frozen basis of its unit, each stored component is
// quantised at its frozen width and the codes are OR-ed into a little-endian
// bit row in LDS, which is then written to the store with coalesced stores.
// The projection runs on fp64 MFMA so that codes are decided from latents
// accurate to ~1e-16, i.e. identical to a float64 evaluation except when a
// value lies within rounding distance of a quantisation boundary.
#include "kvtc_append_tile.h"

namespace kvtc {
namespace {

// Wave w owns tokens 16w..16w+15; N-block nb covers slots 16nb..16nb+15.
// With RANGES set (device fit) nothing is stored: the block's per-slot min and
// max over its valid tokens go to a.keys with atomic min / max.
template <bool MIXED, typename XT, int NB, bool XVEC, bool RANGES = false>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *rows = reinterpret_cast<uint32_t *>(smem + f64_stage_bytes(NB));  // [64][row_words]

    const int u = blockIdx.y;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kAppTok;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nvalid = static_cast<int>(min<int64_t>(kAppTok, a.n - t0));
    const int n_slots = a.ui[u].n_slots;
    const int row_words = a.row_stride >> 2;

    if constexpr (!RANGES)
        for (int w = tid; w < kAppTok * row_words; w += kThreads) rows[w] = 0u;

    doublex4 acc[NB];
    f64_project<XT, NB, XVEC>(a, u, t0, nvalid, 0, smem, acc);

    // fp64 16x16x4 result layout: acc[nb][i] is row (lane>>4) + 4i, column lane&15, i.e.
    // the latent of token 16*wave + (lane>>4) + 4i and slot 16*nb + (lane&15)
    const int tbase = wave * 16 + (lane >> 4);
    if constexpr (RANGES) {
        // min / max over this lane's tokens, its wave's four token groups (lanes
        // 16 apart) and the block's four waves (staged in the now idle row chunks)
        double *red = reinterpret_cast<double *>(smem);   // [4][NB*16][2]
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            double mn = __builtin_huge_val(), mx = -__builtin_huge_val();
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tbase + 4 * i < nvalid) {
                    mn = fmin(mn, acc[nb][i]);
                    mx = fmax(mx, acc[nb][i]);
                }
            mn = fmin(mn, __shfl_xor(mn, 16, 64));
            mx = fmax(mx, __shfl_xor(mx, 16, 64));
            mn = fmin(mn, __shfl_xor(mn, 32, 64));
            mx = fmax(mx, __shfl_xor(mx, 32, 64));
            if (lane < 16) {
                red[(wave * NB * 16 + nb * 16 + lane) * 2] = mn;
                red[(wave * NB * 16 + nb * 16 + lane) * 2 + 1] = mx;
            }
        }
        __syncthreads();
        for (int j = tid; j < min(NB * 16, n_slots); j += kThreads) {
            double mn = red[j * 2], mx = red[j * 2 + 1];
            for (int w = 1; w < 4; ++w) {
                mn = fmin(mn, red[(w * NB * 16 + j) * 2]);
                mx = fmax(mx, red[(w * NB * 16 + j) * 2 + 1]);
            }
            unsigned long long *k = a.keys + (static_cast<int64_t>(u) * a.kslots + j) * 2;
            atomicMin(k, order_key(mn));
            atomicMax(k + 1, order_key(mx));
        }
        return;
    }
    f64_quantise<MIXED, NB>(a, u, t0, nvalid, 0, acc, rows);
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
// With LAT set (refit mode) the latents themselves are the output: the fp64
// result of every slot below kslots goes to a.lat[u][s0 + t][j] and no codes are
// formed.
template <typename XT, int NB, bool LAT = false>
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
    if constexpr (LAT) {
        // result layout: acc[q][i] is token (lane >> 4) + 4i, slot 16 * (wave + 4q) + lane % 16
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = wave + 4 * q;
            const int j = nb * 16 + (lane & 15);
            if (nb < NB && j < a.kslots) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = (lane >> 4) + 4 * i;
                    if (t < nvalid)
                        a.lat[(static_cast<int64_t>(u) * a.capacity + a.s0 + t0 + t) * a.kslots + j] = acc[q][i];
                }
            }
        }
        return;
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


template <bool MIXED, typename XT, int NB>
int32_t launch_append_nb(const AppendArgs &a, int64_t ntiles, int64_t U, hipStream_t stream) {
    const size_t lds = f64_stage_bytes(NB) + static_cast<size_t>(kAppTok) * (a.row_stride / 4) * sizeof(uint32_t);
    auto kern = a.x_vec ? append_kernel<MIXED, XT, NB, true> : append_kernel<MIXED, XT, NB, false>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(ntiles), static_cast<unsigned>(U)), dim3(kThreads), lds,
                       stream, a);
    return launch_status();
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
    return launch_status();
}

template <typename XT, int NB>
int32_t launch_refit_nb(const AppendArgs &a, int64_t U, hipStream_t stream) {
    const size_t lds = small_lds_bytes(a.dg, NB, a.row_stride);
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    auto kern = append_small_kernel<XT, NB, true>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    const int64_t blocks = (a.n + kSmallRows - 1) / kSmallRows;
    if (blocks > 0x7FFFFFFF) return KVTC_E_SHAPE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(U)), dim3(kThreads), lds,
                       stream, a);
    return launch_status();
}

template <typename XT>
int32_t launch_refit(const AppendArgs &a, int64_t U, int nb, hipStream_t st) {
    switch (nb) {
        case 1: return launch_refit_nb<XT, 1>(a, U, st);
        case 2: return launch_refit_nb<XT, 2>(a, U, st);
        case 4: return launch_refit_nb<XT, 4>(a, U, st);
        case 6: return launch_refit_nb<XT, 6>(a, U, st);
        case 8: return launch_refit_nb<XT, 8>(a, U, st);
        case 12: return launch_refit_nb<XT, 12>(a, U, st);
        case 16: return launch_refit_nb<XT, 16>(a, U, st);
        default: return KVTC_E_SHAPE;
    }
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

template <typename XT, int DG>
int32_t launch_decode_dg(const AppendPair &m, int64_t nrows, int64_t units, int nblk, hipStream_t stream) {
    int row_stride = 0;
    for (int i = 0; i < (m.split < units ? 2 : 1); ++i) row_stride = std::max(row_stride, m.t[i].row_stride);
    const size_t lds = decode_lds_bytes(DG, row_stride);
    auto kern = append_decode_kernel<XT, DG>;
    const int64_t blocks = (nrows + kSmallRows - 1) / kSmallRows;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(units)), dim3(64 * nblk), lds,
                       stream, m);
    return launch_status();
}

// One decode launch for one plan (p1 == NULL) or for two plans of the same

}  // namespace

int append_nb(int kslots) {
    const int need = kslots / 16;
    const int opts[] = {1, 2, 4, 6, 8, 12, 16};
    for (int o : opts)
        if (o >= need) return o;
    return -1;
}

// Decode appends of DP tensors (one head per unit) whose unit width has a
// register-resident kernel; one wave per 16 slots, at most dg slots.
bool decode_path(const AppendPlan &p) {
    return !p.mixed && p.a.n <= kSmallRows && p.a.hpu == 1 && (p.a.dg == 64 || p.a.dg == 128) &&
           p.a.kslots <= p.a.dg;
}


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

template <typename XT, int NB>
int32_t launch_ranges_nb(const AppendArgs &a, int64_t U, hipStream_t stream) {
    // the block's row chunks double as the [4][NB*16][2] reduction area
    static_assert(2 * kAppTok * kAppPad >= 4 * NB * 16 * 2, "reduction area");
    const size_t lds = f64_stage_bytes(NB);
    auto kern = a.x_vec ? append_kernel<false, XT, NB, true, true> : append_kernel<false, XT, NB, false, true>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    const int64_t tiles = (a.n + kAppTok - 1) / kAppTok;
    if (tiles > 0x7FFFFFFF || U > 65535) return KVTC_E_SHAPE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(U)), dim3(kThreads), lds, stream,
                       a);
    return launch_status();
}

template <typename XT>
int32_t launch_ranges(const AppendArgs &a, int64_t U, int nb, hipStream_t st) {
    switch (nb) {
        case 1: return launch_ranges_nb<XT, 1>(a, U, st);
        case 2: return launch_ranges_nb<XT, 2>(a, U, st);
        case 4: return launch_ranges_nb<XT, 4>(a, U, st);
        case 6: return launch_ranges_nb<XT, 6>(a, U, st);
        case 8: return launch_ranges_nb<XT, 8>(a, U, st);
        case 12: return launch_ranges_nb<XT, 12>(a, U, st);
        case 16: return launch_ranges_nb<XT, 16>(a, U, st);
        default: return KVTC_E_SHAPE;
    }
}

// Device fit: the prefill rows go through the bulk append kernel's fp64 MFMA
// projection; its per-slot min and max replace the quantise-and-pack step.
int32_t launch_fit_ranges(const AppendArgs &a, int64_t units, int nb, int32_t dtype, hipStream_t stream) {
    if (a.n == 0) return KVTC_OK;
    return dtype == KVTC_F16 ? launch_ranges<_Float16>(a, units, nb, stream) : launch_ranges<float>(a, units, nb, stream);
}

// Refit mode: every row's latents come from append_small_kernel's fp64 MFMA
// sequence whatever n is, so a row's latents do not depend on the call.
int32_t launch_refit_project(const AppendPlan &p, hipStream_t stream) {
    if (p.a.n == 0) return KVTC_OK;
    if (p.mixed || !p.a.lat) return KVTC_E_STATE;
    return p.dtype == KVTC_F16 ? launch_refit<_Float16>(p.a, p.units, p.nb, stream)
                               : launch_refit<float>(p.a, p.units, p.nb, stream);
}

int32_t launch_append_plan(const AppendPlan &p, hipStream_t stream) {
    if (p.a.n == 0) return KVTC_OK;
    if (decode_path(p)) return launch_decode(p, nullptr, stream);
    if (p.i8_ns) return launch_append_i8(p, stream);
    if (p.dtype == KVTC_F16)
        return p.mixed ? launch_append<true, _Float16>(p.a, p.ntiles, p.units, p.nb, stream)
                       : launch_append<false, _Float16>(p.a, p.ntiles, p.units, p.nb, stream);
    return p.mixed ? launch_append<true, float>(p.a, p.ntiles, p.units, p.nb, stream)
                   : launch_append<false, float>(p.a, p.ntiles, p.units, p.nb, stream);
}

// share: how many tensors the launch is shared by (1 or 2); the block target

}  // namespace kvtc
