// Device half of the prefill fit (gfx950): the per-unit moments and the range
// pass of kvtc_fit_device.
//
// KVTC cache module page, update_and_fetch: the local PCA of every (batch,
// head) is fitted for all units in one batched call on the prefill, then the
// DP allocation and the per-component ranges follow.  The data-heavy steps run
// here: the mean and the centred covariance C = (X - mu)^T (X - mu) / S of every
// unit on fp64 MFMA, and the min/max of every kept component's latents over
// the prefill rows (the bulk append kernel's projection).  The eigenpairs, the
// rank and the DP allocation stay on the host (a few ms per unit in all).
#include <cstring>
#include <vector>

#include "kvtc_device.h"

namespace kvtc {
namespace {

constexpr int kFitThreads = 256;
constexpr int kCovTile = 64;          // covariance tile (64 x 64 features per block)
constexpr int kCovRows = 16;          // rows staged per step (four fp64 MFMA k-steps)
constexpr int kCovPitch = kCovTile + 1;

struct FitKArgs {
    const void *x;
    int64_t sb, sh, ss;
    int64_t S;
    int D, hpu, dg, groups, mchunks;
    int64_t rows_per_chunk;
    double *mpart;                    // [U][mchunks][dg]
    double *mean;                     // [U][dg]
    double *cov;                      // [U][dg][dg]
};

template <typename XT>
__device__ inline const XT *unit_col(const FitKArgs &a, int u, int c) {
    const int b = u / a.groups, g = u % a.groups;
    const int j = c / a.D, dd = c - j * a.D;
    return static_cast<const XT *>(a.x) + b * a.sb + (g * a.hpu + j) * a.sh + dd;
}

// Partial column sums of one unit over one chunk of rows: 64 columns per block,
// four row phases per column, reduced in a fixed order.  For fp16 rows every
// partial and total sum is exact in float64 (the values are multiples of 2^-24
// far below 2^29 in magnitude), so the mean does not depend on the order.
template <typename XT>
__global__ __launch_bounds__(kFitThreads) void fit_mean_kernel(FitKArgs a) {
    __shared__ double red[4][64];
    const int c = blockIdx.x * 64 + (threadIdx.x & 63), p = threadIdx.x >> 6;
    const int u = blockIdx.y, mc = blockIdx.z;
    const int64_t s_lo = static_cast<int64_t>(mc) * a.rows_per_chunk;
    const int64_t s_hi = min(a.S, s_lo + a.rows_per_chunk);
    double acc = 0.0;
    if (c < a.dg) {
        const XT *col = unit_col<XT>(a, u, c);
        for (int64_t s = s_lo + p; s < s_hi; s += 4) acc += static_cast<double>(col[s * a.ss]);
    }
    red[p][threadIdx.x & 63] = acc;
    __syncthreads();
    if (p == 0 && c < a.dg)
        a.mpart[(static_cast<int64_t>(u) * a.mchunks + mc) * a.dg + c] =
            ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
}

__global__ __launch_bounds__(kFitThreads) void fit_mean_final_kernel(FitKArgs a) {
    const int u = blockIdx.x;
    for (int c = threadIdx.x; c < a.dg; c += kFitThreads) {
        double s = 0.0;
        for (int mc = 0; mc < a.mchunks; ++mc) s += a.mpart[(static_cast<int64_t>(u) * a.mchunks + mc) * a.dg + c];
        a.mean[static_cast<int64_t>(u) * a.dg + c] = s / static_cast<double>(a.S);
    }
}

// One block: a 64 x 64 tile (ti <= tj) of one unit's covariance.  Wave w owns
// the 32 x 32 sub-tile (w >> 1, w & 1) as 2 x 2 fp64 16x16x4 MFMA tiles; rows
// stream through LDS 16 at a time, centred in float64 as they are staged, with
// the next 16 rows' loads in flight during the current MFMAs.
template <typename XT>
__global__ __launch_bounds__(kFitThreads) void fit_cov_kernel(FitKArgs a) {
    __shared__ double ya[kCovRows][kCovPitch], yb[kCovRows][kCovPitch];
    // triangular tile index -> (ti, tj), ti <= tj
    int t = blockIdx.x, ti = 0;
    const int nt = a.dg / kCovTile;
    while (t >= nt - ti) {
        t -= nt - ti;
        ++ti;
    }
    const int tj = ti + t;
    const int u = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool diag = ti == tj;
    // staging map: thread -> row tid / 16, four columns 4 * (tid % 16)
    const int sr = tid >> 4, sc = (tid & 15) * 4;
    const int c_a = ti * kCovTile + sc, c_b = tj * kCovTile + sc;
    double mu_a[4], mu_b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mu_a[e] = a.mean[static_cast<int64_t>(u) * a.dg + c_a + e];
        mu_b[e] = a.mean[static_cast<int64_t>(u) * a.dg + c_b + e];
    }
    const XT *pa = unit_col<XT>(a, u, c_a), *pb = unit_col<XT>(a, u, c_b);
    XT ra[4], rb[4];
    auto load = [&](int64_t s0) {
        const int64_t s = min(s0 + sr, a.S - 1);          // clamped: rows past S are zeroed when staged
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ra[e] = pa[s * a.ss + e];
            rb[e] = pb[s * a.ss + e];
        }
    };
    auto stage = [&](int64_t s0) {
        const bool ok = s0 + sr < a.S;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ya[sr][sc + e] = ok ? static_cast<double>(ra[e]) - mu_a[e] : 0.0;
            yb[sr][sc + e] = ok ? static_cast<double>(rb[e]) - mu_b[e] : 0.0;
        }
    };
    doublex4 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = doublex4{0.0, 0.0, 0.0, 0.0};
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
    const int li = lane & 15, lk = lane >> 4;
    load(0);
    for (int64_t s0 = 0; s0 < a.S; s0 += kCovRows) {
        stage(s0);
        __syncthreads();
        if (s0 + kCovRows < a.S) load(s0 + kCovRows);
#pragma unroll
        for (int ks = 0; ks < kCovRows / 4; ++ks) {
            const int r = 4 * ks + lk;
            const double a0 = ya[r][wr + li], a1 = ya[r][wr + 16 + li];
            const double b0 = yb[r][wc + li], b1 = yb[r][wc + 16 + li];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();
    }
    // result layout: acc[mi][ni][i] is row 16 mi + (lane >> 4) + 4i, column 16 ni + lane % 16
    const double sd = static_cast<double>(a.S);
    double *cu = a.cov + static_cast<int64_t>(u) * a.dg * a.dg;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d1 = ti * kCovTile + wr + 16 * mi + lk + 4 * i;
                const int d2 = tj * kCovTile + wc + 16 * ni + li;
                const double v = acc[mi][ni][i] / sd;
                cu[static_cast<int64_t>(d1) * a.dg + d2] = v;
                if (!diag) cu[static_cast<int64_t>(d2) * a.dg + d1] = v;
            }
}

__global__ __launch_bounds__(kFitThreads) void fill_keys_kernel(unsigned long long *keys, int64_t n_pairs) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFitThreads + threadIdx.x; i < n_pairs;
         i += static_cast<int64_t>(gridDim.x) * kFitThreads) {
        keys[2 * i] = ~0ull;        // min: above every key
        keys[2 * i + 1] = 0ull;     // max: below every key
    }
}

double key_value(unsigned long long k) {
    const unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    double d;
    std::memcpy(&d, &b, sizeof d);
    return d;
}

FitKArgs kargs(const FitDeviceRows &r, const FitDeviceLayout &L) {
    char *w = static_cast<char *>(r.work);
    FitKArgs a{};
    a.x = r.rows;
    a.sb = r.sb;
    a.sh = r.sh;
    a.ss = r.ss;
    a.S = r.S;
    a.D = r.D;
    a.hpu = r.hpu;
    a.dg = r.dg;
    a.groups = static_cast<int>(r.H / r.hpu);
    a.mchunks = L.mchunks;
    a.rows_per_chunk = (r.S + L.mchunks - 1) / L.mchunks;
    a.mpart = reinterpret_cast<double *>(w + L.mpart);
    a.mean = reinterpret_cast<double *>(w + L.mean);
    a.cov = reinterpret_cast<double *>(w + L.cov);
    return a;
}

template <typename XT>
int32_t launch_moments(const FitKArgs &a, int64_t U, hipStream_t st) {
    const unsigned u = static_cast<unsigned>(U);
    hipLaunchKernelGGL(fit_mean_kernel<XT>, dim3((a.dg + 63) / 64, u, a.mchunks), dim3(kFitThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(fit_mean_final_kernel, dim3(u), dim3(kFitThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    const int nt = a.dg / kCovTile;
    hipLaunchKernelGGL(fit_cov_kernel<XT>, dim3(nt * (nt + 1) / 2, u), dim3(kFitThreads), 0, st, a);
    return launch_status();
}

}  // namespace

int32_t fit_device_moments(const FitDeviceRows &r, double *mean_host, double *cov_host) {
    if (r.units > 65535 || r.dg % kCovTile != 0 || r.S < 1) return KVTC_E_SHAPE;
    const FitDeviceLayout L = fit_device_layout(r.units, r.dg, r.S, r.kslots);
    const FitKArgs a = kargs(r, L);
    hipStream_t st = static_cast<hipStream_t>(r.stream);
    const int32_t s = r.dtype == KVTC_F16 ? launch_moments<_Float16>(a, r.units, st) : launch_moments<float>(a, r.units, st);
    if (s != KVTC_OK) return s;
    const uint64_t nd = static_cast<uint64_t>(r.units) * r.dg;
    if (hipMemcpyAsync(mean_host, a.mean, nd * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipMemcpyAsync(cov_host, a.cov, nd * r.dg * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return KVTC_E_DEVICE;
    return KVTC_OK;
}

int32_t fit_device_ranges(const FitDeviceRows &r, const float *mu32_host, const float *basis_slots_host,
                          const int32_t *n_slots_host, double *mn_host, double *mx_host) {
    if (r.kslots < 16 || r.kslots > kMaxSlots || r.kslots % 16 != 0 || r.units > 65535) return KVTC_E_SHAPE;
    const FitDeviceLayout L = fit_device_layout(r.units, r.dg, r.S, r.kslots);
    char *w = static_cast<char *>(r.work);
    hipStream_t st = static_cast<hipStream_t>(r.stream);
    const uint64_t U = static_cast<uint64_t>(r.units);
    std::vector<kvtc_unit_info> ui(U);
    for (uint64_t u = 0; u < U; ++u) ui[u] = kvtc_unit_info{0, n_slots_host[u], 0, 0};
    std::vector<unsigned long long> keys(U * r.kslots * 2);
    if (hipMemcpyAsync(w + L.basis, basis_slots_host, U * r.kslots * r.dg * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(w + L.mu32, mu32_host, U * r.dg * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(w + L.ui, ui.data(), U * sizeof(kvtc_unit_info), hipMemcpyHostToDevice, st) != hipSuccess)
        return KVTC_E_DEVICE;
    auto *kd = reinterpret_cast<unsigned long long *>(w + L.keys);
    hipLaunchKernelGGL(fill_keys_kernel, dim3(256), dim3(kFitThreads), 0, st, kd, static_cast<int64_t>(U * r.kslots));
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    AppendArgs a{};
    a.x = r.rows;
    a.xsb = r.sb;
    a.xsh = r.sh;
    a.xss = r.ss;
    a.n = r.S;
    a.capacity = r.S;
    a.ui = reinterpret_cast<const kvtc_unit_info *>(w + L.ui);
    a.mu = reinterpret_cast<const float *>(w + L.mu32);
    a.basis = reinterpret_cast<const float *>(w + L.basis);
    a.keys = kd;
    a.dg = r.dg;
    a.D = r.D;
    a.hpu = r.hpu;
    a.groups = static_cast<int>(r.H / r.hpu);
    a.kslots = r.kslots;
    a.row_stride = 0;
    const int64_t esz = r.dtype == KVTC_F16 ? 2 : 4;
    a.x_vec = reinterpret_cast<uintptr_t>(r.rows) % (4 * esz) == 0 && r.sb % 4 == 0 && r.sh % 4 == 0 && r.ss % 4 == 0;
    a.inv_dg = 1.0f / static_cast<float>(r.dg);
    a.inv_q4 = 4.0f / static_cast<float>(r.dg);
    const int32_t s = launch_fit_ranges(a, r.units, append_nb(r.kslots), r.dtype, st);
    if (s != KVTC_OK) return s;
    if (hipMemcpyAsync(keys.data(), kd, keys.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return KVTC_E_DEVICE;
    for (uint64_t i = 0; i < U * r.kslots; ++i) {
        mn_host[i] = key_value(keys[2 * i]);
        mx_host[i] = key_value(keys[2 * i + 1]);
    }
    return KVTC_OK;
}

}  // namespace kvtc
