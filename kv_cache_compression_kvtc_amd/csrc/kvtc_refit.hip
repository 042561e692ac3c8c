// Refit mode (gfx950): the KVTC cache module page's own decode semantics.
// _TensorKVTC.append joins the new rows to every row accumulated so far and
// _requantize re-projects them all through the frozen basis and mean, then
// quantises each kept component with a min/max fitted over all of them: the
// basis, mean and widths stay frozen, the per-component (min, scale) and with
// them every stored code follow the accumulated sequence.
//
// A row's latents never change under the frozen basis, so they are computed
// once, on append, in fp64 and kept in a latent store; each call then
//   1. reduces every kept component's min and max over rows [0, S)
//      (per-chunk partials, then one block per unit),
//   2. forms the quantiser (fp32 min and scale, as the prefill ranges are
//      stored) and the fetch operands they imply (fp16 scale*basis and the
//      fp32 bias mean + sum_j min_j basis_j, evaluated as the host builds the
//      blob's),
//   3. re-quantises and re-packs the codes of every row [0, S).
#include "kvtc_device.h"

namespace kvtc {
namespace {

constexpr int kRefitThreads = 256;
constexpr int kRefitRows = 64;      // rows per re-quantisation block

// Phase p of a block's threads scans rows p, p + P, ... of slot j = tid % kslots
// (P = threads / kslots), so a wave's loads of one row are contiguous.
__global__ __launch_bounds__(kRefitThreads) void refit_range_kernel(RefitArgs a) {
    __shared__ double red[2][kRefitThreads];
    const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
    const int ks = a.kslots, P = kRefitThreads / ks;
    const int j = tid % ks, p = tid / ks;
    const int64_t s_lo = static_cast<int64_t>(c) * a.rows_per_chunk;
    const int64_t s_hi = min(a.S, s_lo + a.rows_per_chunk);
    double mn = __builtin_huge_val(), mx = -__builtin_huge_val();
    if (p < P) {
        const double *col = a.lat + static_cast<int64_t>(u) * a.capacity * ks + j;
        for (int64_t s = s_lo + p; s < s_hi; s += P) {
            const double v = col[s * ks];
            mn = fmin(mn, v);
            mx = fmax(mx, v);
        }
    }
    red[0][tid] = mn;
    red[1][tid] = mx;
    __syncthreads();
    if (tid < ks) {
        for (int q = 1; q < P; ++q) {
            mn = fmin(mn, red[0][q * ks + tid]);
            mx = fmax(mx, red[1][q * ks + tid]);
        }
        double *dst = a.part + ((static_cast<int64_t>(u) * a.chunks + c) * ks + tid) * 2;
        dst[0] = mn;
        dst[1] = mx;
    }
}

// One block per unit: the ranges of its kept slots, the quantiser and the fetch
// operands.  Slot order is component order, as in the blob.
__global__ __launch_bounds__(kRefitThreads) void refit_finalize_kernel(RefitArgs a) {
    __shared__ float qm[kMaxSlots], qs[kMaxSlots];
    const int u = blockIdx.x, tid = threadIdx.x;
    const int ks = a.kslots, ns = a.ui[u].n_slots;
    const int64_t ub = static_cast<int64_t>(u) * ks;
    for (int j = tid; j < ks; j += kRefitThreads) {
        float m32 = 0.f, s32 = 0.f;
        double lo = 0.0, inv = 0.0;
        if (j < ns) {
            double mn = __builtin_huge_val(), mx = -__builtin_huge_val();
            const double *pp = a.part + (static_cast<int64_t>(u) * a.chunks * ks + j) * 2;
            for (int c = 0; c < a.chunks; ++c) {
                mn = fmin(mn, pp[static_cast<int64_t>(c) * ks * 2]);
                mx = fmax(mx, pp[static_cast<int64_t>(c) * ks * 2 + 1]);
            }
            const uint32_t w = a.sbits[ub + j] >> 24;
            m32 = static_cast<float>(mn);
            s32 = mx > mn ? static_cast<float>((mx - mn) / static_cast<double>((1u << w) - 1u)) : 0.f;
            lo = static_cast<double>(m32);
            inv = s32 > 0.f ? 1.0 / static_cast<double>(s32) : 0.0;
        }
        a.qmin32[ub + j] = m32;
        a.qscale32[ub + j] = s32;
        a.qlo[ub + j] = lo;
        a.qinv[ub + j] = inv;
        qm[j] = m32;
        qs[j] = s32;
    }
    __syncthreads();
    const int dg = a.dg, kf = a.kfetch;
    const float *basis = a.basis + ub * dg;
    const int32_t *fs = a.fslot + static_cast<int64_t>(u) * kf;
    for (int i = tid; i < dg * kf; i += kRefitThreads) {
        const int d = i / kf, kk = i - d * kf;
        const int j = fs[kk];
        a.w16[(static_cast<int64_t>(u) * dg + d) * kf + kk] =
            j >= 0 ? half_bits_rne(static_cast<double>(qs[j]) * static_cast<double>(basis[static_cast<int64_t>(j) * dg + d]))
                   : uint16_t(0);
    }
    for (int d = tid; d < dg; d += kRefitThreads) {
        // separate multiply and add, in slot order, as the host accumulates the blob's bias
        double acc = static_cast<double>(a.mu[static_cast<int64_t>(u) * dg + d]);
        for (int j = 0; j < ns; ++j)
            acc = __dadd_rn(acc, __dmul_rn(static_cast<double>(qm[j]), static_cast<double>(basis[static_cast<int64_t>(j) * dg + d])));
        a.bias[static_cast<int64_t>(u) * dg + d] = static_cast<float>(acc);
    }
}

// Rows [64 blockIdx.x, +64) of one unit: every kept latent quantised with the
// refitted range and OR-ed into an LSB-first bit row in LDS, then the rows are
// written with coalesced 32-bit stores.
__global__ __launch_bounds__(kRefitThreads) void refit_requant_kernel(RefitArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *rows = reinterpret_cast<uint32_t *>(smem);          // [64][row_words]
    const int u = blockIdx.y, tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRefitRows;
    const int nvalid = static_cast<int>(min<int64_t>(kRefitRows, a.S - t0));
    const int row_words = a.row_stride >> 2;
    for (int w = tid; w < kRefitRows * row_words; w += kRefitThreads) rows[w] = 0u;
    __syncthreads();
    const int ks = a.kslots, P = kRefitThreads / ks, ns = a.ui[u].n_slots;
    const int j = tid % ks, p = tid / ks;
    const int64_t ub = static_cast<int64_t>(u) * ks;
    if (p < P && j < ns) {
        const double lo = a.qlo[ub + j], inv = a.qinv[ub + j];
        const uint32_t sb = a.sbits[ub + j];
        const uint32_t off = sb & kOffsetMask, w = sb >> 24;
        const double cmax = static_cast<double>((1u << w) - 1u);
        const double *col = a.lat + (static_cast<int64_t>(u) * a.capacity + t0) * ks + j;
        for (int t = p; t < nvalid; t += P)
            or_field(rows + t * row_words, off, w, static_cast<uint32_t>(quantise(col[static_cast<int64_t>(t) * ks], lo, inv, cmax)));
    }
    __syncthreads();
    if (row_words > 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + (static_cast<int64_t>(u) * a.capacity + t0) * a.row_stride);
        for (int w = tid; w < nvalid * row_words; w += kRefitThreads) dst[w] = rows[w];
    }
}

}  // namespace

int32_t launch_refit_requantise(const RefitArgs &a0, int64_t units, hipStream_t stream) {
    if (a0.S <= 0) return KVTC_OK;
    if (a0.kslots > kRefitThreads || units > 65535) return KVTC_E_SHAPE;
    RefitArgs a = a0;
    // as many chunks as the partial buffer holds, and no empty ones
    const int64_t want = (a.S + kRefitRows - 1) / kRefitRows;
    a.chunks = static_cast<int>(std::min<int64_t>(a.chunks, want));
    a.rows_per_chunk = (a.S + a.chunks - 1) / a.chunks;
    a.chunks = static_cast<int>((a.S + a.rows_per_chunk - 1) / a.rows_per_chunk);
    const unsigned U = static_cast<unsigned>(units);
    hipLaunchKernelGGL(refit_range_kernel, dim3(static_cast<unsigned>(a.chunks), U), dim3(kRefitThreads), 0, stream, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(refit_finalize_kernel, dim3(U), dim3(kRefitThreads), 0, stream, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    const int64_t tiles = (a.S + kRefitRows - 1) / kRefitRows;
    if (tiles > 0x7FFFFFFF) return KVTC_E_SHAPE;
    const size_t lds = static_cast<size_t>(kRefitRows) * (a.row_stride / 4) * sizeof(uint32_t);
    hipLaunchKernelGGL(refit_requant_kernel, dim3(static_cast<unsigned>(tiles), U), dim3(kRefitThreads), lds, stream, a);
    return launch_status();
}

}  // namespace kvtc
