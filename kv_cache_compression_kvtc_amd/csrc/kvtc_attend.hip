// Decode attention from the codes (gfx950): kvtc_attend and its kernels.
#include <mutex>

#include "kvtc_device.h"

namespace kvtc {
namespace {

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

// Scratch of the allocation-free entry point (kvtc_attend_noalloc): a fixed
// device array of the library, KVTC_ATTEND_SCRATCH_BYTES per device that loads
// it, held until the process ends.  Host code never uses this name as an
// address: each device's copy is found once with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KVTC_ATTEND_SCRATCH_BYTES];

namespace kvtc {
namespace {

constexpr size_t kAttendScratchBytes = KVTC_ATTEND_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// This device's copy of scratch, looked up once per device (with that device
// current) and kept.
int32_t scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVTC_E_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVTC_E_DEVICE;
        addr[dev] = p;
    }
    *out = addr[dev];
    return KVTC_OK;
}

int32_t attend_impl(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                    const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                    void *work_dev, size_t work_bytes, bool noalloc, hipStream_t stream);

}  // namespace
}  // namespace kvtc

using namespace kvtc;

extern "C" {

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
    return attend_impl(k, v, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, work_dev, work_bytes, false,
                       static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_attend_noalloc(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                            const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                            void *hip_stream) {
    return attend_impl(k, v, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, nullptr, 0, true,
                       static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

namespace kvtc {
namespace {

// Validates the call, then launches the three attention kernels on the given
// workspace; with noalloc the workspace is this device's scratch array (after
// its size has been checked against the call's need).
int32_t attend_impl(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                    const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                    void *work_dev, size_t work_bytes, bool noalloc, hipStream_t stream) {
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
    if (noalloc) {
        if (need > kAttendScratchBytes) return KVTC_E_BUFSIZE;
        const int32_t sa = scratch_address(&work_dev);
        if (sa != KVTC_OK) return sa;
        work_bytes = kAttendScratchBytes;
    }
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

}  // namespace
}  // namespace kvtc
