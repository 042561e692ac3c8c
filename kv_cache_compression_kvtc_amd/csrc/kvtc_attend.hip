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
constexpr int kAttPass = 4;          // value k-steps accumulated per pass over a chunk's rows

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
    int nchunks, chunk_rows, H, D;     // chunks of chunk_rows rows (the last one shorter), <= kAttChunk
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

// Sum of v over each half of the wave (lanes 0-31 and 32-63), left in lanes
// 16-31 and 48-63, with DPP moves only: neighbours in quads, then octets (half
// row mirror), rows (row mirror), and row 0 (2) into row 1 (3).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float half_wave_sum(float v) {
    v += dpp_f32<0xB1, 0xF>(v);      // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E, 0xF>(v);      // quad_perm [2,3,0,1]
    v += dpp_f32<0x141, 0xF>(v);     // row_half_mirror
    v += dpp_f32<0x140, 0xF>(v);     // row_mirror
    v += dpp_f32<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
    return v;
}

// Staging of a chunk's code rows (256-thread blocks): word i of the chunk goes
// to row i / row_words, word i % row_words, of an LDS array of odd pitch.  A
// thread holds SB words per batch (words base + k*256 + tid), all loaded before
// any is stored, so a chunk of up to 256*SB words costs one memory round trip
// (issued early, the loads overlap other work).  The quotient from a float
// reciprocal is exact for word indices below 2^16.
constexpr int kStageB = 24;

__device__ inline void stage_load(const uint32_t *src, int total, int base, uint32_t (&r)[kStageB]) {
#pragma unroll
    for (int k = 0; k < kStageB; ++k) {
        const int i = base + k * 256 + static_cast<int>(threadIdx.x);
        r[k] = i < total ? src[i] : 0u;
    }
}

__device__ inline void stage_store(int total, int base, int row_words, int pitch, uint32_t *rows,
                                   const uint32_t (&r)[kStageB]) {
    const float inv = 1.0f / static_cast<float>(max(row_words, 1));
#pragma unroll
    for (int k = 0; k < kStageB; ++k) {
        const int i = base + k * 256 + static_cast<int>(threadIdx.x);
        if (i < total) {
            const int q = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
            rows[q * pitch + (i - q * row_words)] = r[k];
        }
    }
}

// The whole chunk: batch 0 from registers already loaded, the rest (chunks of
// more than 256*kStageB words) loaded and stored batch by batch.
__device__ inline void stage_rows(const uint32_t *src, int total, int row_words, int pitch, uint32_t *rows,
                                  uint32_t (&r)[kStageB]) {
    stage_store(total, 0, row_words, pitch, rows, r);
    for (int base = 256 * kStageB; base < total; base += 256 * kStageB) {
        stage_load(src, total, base, r);
        stage_store(total, base, row_words, pitch, rows, r);
    }
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
    // beta = (q . mu + sum_j min_j q . V_j) / sqrt(D), summed over the block
    float bpart = 0.f;
    for (int d = tid; d < a.D; d += blockDim.x) bpart = fmaf(ql[d], k.mu[static_cast<int64_t>(u) * a.D + d], bpart);
    if (tid < k.kslots) bpart += mpart[tid];
    const float beta = block_reduce(bpart, red, false);
    if (tid == 0) {
        a.qmul[u] = ldexpf(1.0f, e);
        a.qt[static_cast<int64_t>(u) * (k.kslots + 1) + k.kslots] = beta * a.inv_sqrt_d;
    }
}

// Per (chunk of chunk_rows <= kAttChunk rows, unit): scores from the key codes, the chunk's
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
    const int64_t s0 = static_cast<int64_t>(c) * a.chunk_rows;
    const int nrows = static_cast<int>(min<int64_t>(a.chunk_rows, a.s_end - s0));
    const int kp = (K.row_words + 1) | 1, vp = (V.row_words + 1) | 1;   // odd, > row_words

    // the unit's coefficients (at most 257 and 256 words: two and one per
    // thread), then the chunk's key and value rows, all requested before any is
    // used
    uint32_t cq[2], cf;
    {
        const float *qsrc = a.qt + static_cast<int64_t>(u) * (K.kslots + 1);
        const uint32_t *fsrc = reinterpret_cast<const uint32_t *>(a.qf + static_cast<int64_t>(u) * 2 * K.kfetch);
        cq[0] = tid <= K.kslots ? __float_as_uint(qsrc[tid]) : 0u;
        cq[1] = tid + 256 <= K.kslots ? __float_as_uint(qsrc[tid + 256]) : 0u;
        cf = tid < K.kfetch ? fsrc[tid] : 0u;                           // 2*kfetch halves
    }
    const uint32_t *ksrc = reinterpret_cast<const uint32_t *>(K.codes) + (static_cast<int64_t>(u) * K.capacity + s0) * K.row_words;
    const uint32_t *vsrc = reinterpret_cast<const uint32_t *>(V.codes) + (static_cast<int64_t>(u) * V.capacity + s0) * V.row_words;
    const int ktot = nrows * K.row_words, vtot = nrows * V.row_words;
    uint32_t kr[kStageB], vr[kStageB];
    stage_load(ksrc, ktot, 0, kr);
    stage_load(vsrc, vtot, 0, vr);
    if (tid <= K.kslots) qt_l[tid] = __uint_as_float(cq[0]);
    if (tid + 256 <= K.kslots) qt_l[tid + 256] = __uint_as_float(cq[1]);
    if (tid < K.kfetch) ksb[tid] = cf;
    stage_rows(ksrc, ktot, K.row_words, kp, rows, kr);
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
    stage_rows(vsrc, vtot, V.row_words, vp, rows, vr);   // the key rows are no longer read
    const float L = block_reduce(lsum, red, false);
    __syncthreads();

    // p-weighted sums of the value codes in the fetch order: wave w takes the
    // 32-row tiles w, w + 4, ... of the chunk (lane: row lane & 31, half k-step
    // lane >> 5) and decodes each of its k-steps' 8 codes as exact fp16 values
    // (the fetch kernel's field decode); each code is accumulated as
    // c * (p_hi + p_lo) in fp32 with one v_dot2, p * 2^12 split into two fp16
    // parts (together within 2^-22 of p; the 2^12 keeps them normal).  The
    // rows' sums are then added across the 32 row lanes, and the fetch columns
    // mapped back to slots.  Up to kAttPass k-steps per pass over the rows.
    __syncthreads();                                   // the reductions' scratch is reused below
    {
        for (int j = lane; j < kMaxSlots; j += 64) red[wave * kMaxSlots + j] = 0.f;   // this wave's sums only
        const int nksV = V.kfetch / 16;
        const uint32_t half_k = lane >> 5;
        const int tok = lane & 31;
        const int ntiles = (nrows + 31) >> 5;
        const int32_t *fs = V.fslot + static_cast<int64_t>(u) * V.kfetch;
        for (int k0 = 0; k0 < nksV; k0 += kAttPass) {
            uint32_t kd[kAttPass];
#pragma unroll
            for (int q = 0; q < kAttPass; ++q)
                kd[q] = k0 + q < nksV ? __builtin_amdgcn_readfirstlane(V.kdesc[static_cast<int64_t>(u) * nksV + k0 + q])
                                      : 0u;
            float acc[kAttPass][8];
#pragma unroll
            for (int q = 0; q < kAttPass; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
            for (int t = wave; t < ntiles; t += 4) {
                const int r = t * 32 + tok;
                const float ps = r < nrows ? pl[r] * 4096.0f : 0.0f;
                const _Float16 ph = static_cast<_Float16>(ps);
                const half2 pw = {ph, static_cast<_Float16>(ps - static_cast<float>(ph))};
                const uint32_t *row = rows + r * vp;
#pragma unroll
                for (int q = 0; q < kAttPass; ++q) {
                    if (((kd[q] >> 16) & 0xFu) == 0u) continue;            // empty or past the end (uniform)
                    const half8 cv = decode_kstep<false>(kd[q], row, nullptr, half_k);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const half2 cc = {cv[i], cv[i]};
                        acc[q][i] = __builtin_amdgcn_fdot2(cc, pw, acc[q][i], false);
                    }
                }
            }
            // sums over the 32 row lanes of each half (in its lanes 16-31), then
            // into this wave's slot sums (each slot has one fetch column;
            // padding columns none)
#pragma unroll
            for (int q = 0; q < kAttPass; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[q][i] = half_wave_sum(acc[q][i]);
            if (tok == 16) {
#pragma unroll
                for (int q = 0; q < kAttPass; ++q) {
                    if (k0 + q >= nksV) break;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int j = fs[(k0 + q) * 16 + half_k * 8 + i];
                        if (j >= 0) red[wave * kMaxSlots + j] = acc[q][i] * 0x1p-12f;
                    }
                }
            }
        }
    }
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
    // the chunks' weights exp(m_c - M), 256 chunks at a time, shared by the slots
    __shared__ float wch[256];
    float s = 0.f;
    for (int c0 = 0; c0 < a.nchunks; c0 += 256) {
        __syncthreads();
        if (c0 + tid < a.nchunks) wch[tid] = expf(part[(c0 + tid) * stride + V.kslots] - M);
        __syncthreads();
        if (tid < nv) {
            const int cn = min(256, a.nchunks - c0);
            for (int c = 0; c < cn; ++c) s = fmaf(wch[c], part[(c0 + c) * stride + tid], s);
        }
    }
    if (tid < V.kslots) {
        if (tid < nv) {
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

// ============================================================ general path
// Any number G of query heads per KV head (grouped-query attention: query head
// hq attends KV head hq / G) and per-head or group-head caches on either side.
// A unit of hpu heads is attended by Q = hpu * G queries; query i of unit u is
// query head (group(u) * hpu + i / G) * G + i % G and sees the D features
// [(i / G) * D, (i / G + 1) * D) of the unit's rows.  With x_s = sum_j l_sj V_j + mu
// and q~_ij = (q_i . V_j[slice_i]) / sqrt(D):
//   per-head (DP) rows, l = min_j + c * scale_j:  score = sum_j c q~_ij scale_j + beta_i,
//     beta_i = (q_i . mu[slice] + sum_j min_j (q_i . V_j[slice])) / sqrt(D);
//   group-head rows, l = min16_g + c * scale16_g per token and quantisation group g:
//     score = sum_g (min16_g P_ig + scale16_g sum_{j in g} c q~_ij) + q_i . mu[slice] / sqrt(D),
//     P_ig = sum_{j in g} q~_ij;
// the output is sum_j abar_ij V_j[slice_i] + mu[slice_i] with abar_ij = sum_s p_is l_sj.
constexpr int kGenRows = 256;        // rows per partial block (one thread per row)
constexpr int kGenMaxQ = 32;         // queries per unit

struct GenSide {
    const uint8_t *codes;
    const uint32_t *params;            // group-head rows: [U][capacity][n_qg] (min16 | scale16 << 16)
    int64_t capacity;
    const kvtc_unit_info *ui;
    const float *basis, *mu, *qmin, *qscale, *bias;
    const int32_t *comp;
    const uint32_t *sbits;
    int kslots, rmax, row_words, n_qg, gs, mixed, dg;
};

struct GenArgs {
    GenSide k, v;
    const void *q;
    int64_t qsb, qsh;
    int q_f16;
    _Float16 *out;
    int64_t osb, osh;
    int64_t s_end;
    int nchunks, G, hpu, groups, D, Q;
    float inv_sqrt_d;
    float *qt;       // [U][Q][k.kslots]   q~ (times scale_j for per-head keys)
    float *qb;       // [U][Q]             beta
    float *qp;       // [U][Q][k.n_qg]     group sums of q~ (group-head keys)
    float *part;     // [U][nchunks][Q][v.kslots + 2]: abar partial sums, then max, sum
};

__device__ inline void gen_query(const GenArgs &a, int u, int i, int &b, int &hq, int &slice) {
    b = u / a.groups;
    const int jh = i / a.G;
    hq = ((u % a.groups) * a.hpu + jh) * a.G + i % a.G;
    slice = jh * a.D;
}

// Per (unit, query): the score coefficients, in fixed orders.
__global__ __launch_bounds__(256) void attend_gen_prep_kernel(GenArgs a) {
    __shared__ float ql[kMaxSlots];
    __shared__ float qts[kMaxSlots];
    __shared__ float mpart[kMaxSlots];
    const int u = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
    int b, hq, slice;
    gen_query(a, u, i, b, hq, slice);
    for (int d = tid; d < a.D; d += blockDim.x)
        ql[d] = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[b * a.qsb + hq * a.qsh + d])
                        : static_cast<const float *>(a.q)[b * a.qsb + hq * a.qsh + d];
    __syncthreads();
    const GenSide &K = a.k;
    const int ns = K.ui[u].n_slots;
    for (int j = tid; j < K.kslots; j += blockDim.x) {
        float qt = 0.f, mp = 0.f;
        if (j < ns) {
            const float *vrow = K.basis + (static_cast<int64_t>(u) * K.kslots + j) * K.dg + slice;
            float dot = 0.f;
            for (int d = 0; d < a.D; ++d) dot = fmaf(ql[d], vrow[d], dot);
            if (K.mixed) {
                qt = dot * a.inv_sqrt_d;
            } else {
                const int c = K.comp[static_cast<int64_t>(u) * K.kslots + j];
                qt = K.qscale[static_cast<int64_t>(u) * K.rmax + c] * dot * a.inv_sqrt_d;
                mp = K.qmin[static_cast<int64_t>(u) * K.rmax + c] * dot;
            }
        }
        a.qt[(static_cast<int64_t>(u) * a.Q + i) * K.kslots + j] = qt;
        qts[j] = qt;
        mpart[j] = mp;
    }
    __syncthreads();
    if (tid == 0) {
        float beta = 0.f;
        for (int d = 0; d < a.D; ++d) beta = fmaf(ql[d], K.mu[static_cast<int64_t>(u) * K.dg + slice + d], beta);
        for (int j = 0; j < K.kslots; ++j) beta += mpart[j];
        a.qb[static_cast<int64_t>(u) * a.Q + i] = beta * a.inv_sqrt_d;
    }
    if (K.mixed)
        for (int g = tid; g < K.n_qg; g += blockDim.x) {
            float p = 0.f;
            for (int j = g * K.gs; j < min(ns, (g + 1) * K.gs); ++j) p += qts[j];
            a.qp[(static_cast<int64_t>(u) * a.Q + i) * K.n_qg + g] = p;
        }
}

// n words from global memory into LDS, eight per thread in flight per batch.
__device__ inline void lds_copy(uint32_t *dst, const uint32_t *src, int n) {
    for (int base = 0; base < n; base += 256 * 8) {
        uint32_t r[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + k * 256 + static_cast<int>(threadIdx.x);
            r[k] = i < n ? src[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + k * 256 + static_cast<int>(threadIdx.x);
            if (i < n) dst[i] = r[k];
        }
    }
}

// The code rows of rows [s0, s0 + n) of unit u (batch 0 already in r) at an
// odd pitch and, for group-head rows, their (min, scale) words group-major.
__device__ inline void gen_stage(const GenSide &T, const uint32_t *src, int n, uint32_t *rows, int pitch,
                                 uint32_t *prm, const uint32_t *ps, uint32_t (&r)[kStageB]) {
    stage_rows(src, n * T.row_words, T.row_words, pitch, rows, r);
    if (T.mixed) {
        const int total = n * T.n_qg;
        for (int base = 0; base < total; base += 256 * 8) {
            uint32_t pv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + k * 256 + static_cast<int>(threadIdx.x);
                pv[k] = i < total ? ps[i] : 0u;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + k * 256 + static_cast<int>(threadIdx.x);
                if (i < total) {
                    const int q = i / T.n_qg;
                    prm[(i - q * T.n_qg) * kGenRows + q] = pv[k];
                }
            }
        }
    }
}

__device__ inline float half_lo(uint32_t p) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(p & 0xFFFFu))); }
__device__ inline float half_hi(uint32_t p) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(p >> 16))); }

// Per (chunk of 256 rows, unit): every query's scores of the chunk's rows (one
// thread per row), the chunk's softmax max and sum per query, and the
// p-weighted sums of every value slot (one thread per slot).
template <int QM>
__global__ __launch_bounds__(256) void attend_gen_partial_kernel(GenArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const GenSide &K = a.k, &V = a.v;
    const int c = blockIdx.x, u = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int Q = a.Q;
    float *qt = reinterpret_cast<float *>(smem);                     // [QM][K.kslots]
    float *qb = qt + QM * K.kslots;                                  // [QM]
    float *qp = qb + QM;                                             // [QM][K.n_qg]
    float *sc = qp + QM * max(K.n_qg, 1);                            // [QM][256] scores, then weights
    float *stat = sc + QM * kGenRows;                                // [QM][2]
    uint32_t *sb = reinterpret_cast<uint32_t *>(stat + 2 * QM);     // [kMaxSlots]
    uint32_t *rows = sb + kMaxSlots;                                 // [256][pitch]
    const int pitch = (max(K.row_words, V.row_words) + 1) | 1;
    uint32_t *prm = rows + kGenRows * pitch;                         // [n_qg][256]
    const int64_t s0 = static_cast<int64_t>(c) * kGenRows;
    const int nrows = static_cast<int>(min<int64_t>(kGenRows, a.s_end - s0));

    // the chunk's key and value rows are requested first; the unit's
    // coefficients and slot descriptors are copied while they are in flight
    const uint32_t *ksrc = reinterpret_cast<const uint32_t *>(K.codes) + (static_cast<int64_t>(u) * K.capacity + s0) * K.row_words;
    const uint32_t *vsrc = reinterpret_cast<const uint32_t *>(V.codes) + (static_cast<int64_t>(u) * V.capacity + s0) * V.row_words;
    uint32_t kr[kStageB], vr[kStageB];
    stage_load(ksrc, nrows * K.row_words, 0, kr);
    stage_load(vsrc, nrows * V.row_words, 0, vr);
    lds_copy(reinterpret_cast<uint32_t *>(qt), reinterpret_cast<const uint32_t *>(a.qt + static_cast<int64_t>(u) * Q * K.kslots),
             Q * K.kslots);
    lds_copy(reinterpret_cast<uint32_t *>(qb), reinterpret_cast<const uint32_t *>(a.qb + static_cast<int64_t>(u) * Q), Q);
    if (K.mixed)
        lds_copy(reinterpret_cast<uint32_t *>(qp), reinterpret_cast<const uint32_t *>(a.qp + static_cast<int64_t>(u) * Q * K.n_qg),
                 Q * K.n_qg);
    lds_copy(sb, K.sbits + static_cast<int64_t>(u) * K.kslots, K.kslots);
    gen_stage(K, ksrc, nrows, rows, pitch, prm,
              K.mixed ? K.params + (static_cast<int64_t>(u) * K.capacity + s0) * K.n_qg : nullptr, kr);
    __syncthreads();

    float acc[QM];
#pragma unroll
    for (int i = 0; i < QM; ++i) acc[i] = i < Q ? qb[i] : 0.f;
    if (t < nrows) {
        const uint32_t *row = rows + t * pitch;
        const int ns = K.ui[u].n_slots;
        if (!K.mixed) {
            for (int j = 0; j < ns; ++j) {
                const float cf = static_cast<float>(row_field(row, sb[j]));
#pragma unroll
                for (int i = 0; i < QM; ++i)
                    if (i < Q) acc[i] = fmaf(cf, qt[i * K.kslots + j], acc[i]);
            }
        } else {
            for (int g = 0; g < K.n_qg; ++g) {
                float gacc[QM];
#pragma unroll
                for (int i = 0; i < QM; ++i) gacc[i] = 0.f;
                for (int j = g * K.gs; j < min(ns, (g + 1) * K.gs); ++j) {
                    const float cf = static_cast<float>(row_field(row, sb[j]));
#pragma unroll
                    for (int i = 0; i < QM; ++i)
                        if (i < Q) gacc[i] = fmaf(cf, qt[i * K.kslots + j], gacc[i]);
                }
                const uint32_t p = prm[g * kGenRows + t];
                const float mn = half_lo(p), scl = half_hi(p);
#pragma unroll
                for (int i = 0; i < QM; ++i)
                    if (i < Q) acc[i] = fmaf(scl, gacc[i], fmaf(mn, qp[i * K.n_qg + g], acc[i]));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < QM; ++i)
        if (i < Q) sc[i * kGenRows + t] = t < nrows ? acc[i] : -__builtin_huge_valf();
    __syncthreads();
    // softmax statistics: wave w takes queries w, w + 4, ...
    for (int i = wave; i < Q; i += 4) {
        float m = -__builtin_huge_valf();
        for (int r = lane; r < kGenRows; r += 64) m = fmaxf(m, sc[i * kGenRows + r]);
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        float l = 0.f;
        for (int r = lane; r < kGenRows; r += 64) {
            const float p = r < nrows ? expf(sc[i * kGenRows + r] - m) : 0.f;
            sc[i * kGenRows + r] = p;
            l += p;
        }
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
        if (lane == 0) {
            stat[2 * i] = m;
            stat[2 * i + 1] = l;
        }
    }
    __syncthreads();
    // value rows
    lds_copy(sb, V.sbits + static_cast<int64_t>(u) * V.kslots, V.kslots);
    gen_stage(V, vsrc, nrows, rows, pitch, prm,
              V.mixed ? V.params + (static_cast<int64_t>(u) * V.capacity + s0) * V.n_qg : nullptr, vr);
    __syncthreads();
    float va[QM];
#pragma unroll
    for (int i = 0; i < QM; ++i) va[i] = 0.f;
    const int nv = V.ui[u].n_slots;
    if (t < nv) {
        const uint32_t sbj = sb[t];
        const int g = V.mixed ? t / V.gs : 0;
        for (int r = 0; r < nrows; ++r) {
            const float cf = static_cast<float>(row_field(rows + r * pitch, sbj));
            float l = cf;
            if (V.mixed) {
                const uint32_t p = prm[g * kGenRows + r];
                l = fmaf(cf, half_hi(p), half_lo(p));
            }
#pragma unroll
            for (int i = 0; i < QM; ++i)
                if (i < Q) va[i] = fmaf(sc[i * kGenRows + r], l, va[i]);
        }
    }
    float *dst = a.part + (static_cast<int64_t>(u) * a.nchunks + c) * Q * (V.kslots + 2);
    if (t < V.kslots) {
#pragma unroll
        for (int i = 0; i < QM; ++i)
            if (i < Q) dst[i * (V.kslots + 2) + t] = va[i];
    }
    for (int i = t; i < Q; i += blockDim.x) {
        dst[i * (V.kslots + 2) + V.kslots] = stat[2 * i];
        dst[i * (V.kslots + 2) + V.kslots + 1] = stat[2 * i + 1];
    }
}

// Per (unit, query): merge the chunks and reconstruct the output once.
__global__ __launch_bounds__(256) void attend_gen_merge_kernel(GenArgs a) {
    __shared__ float coef[kMaxSlots];
    __shared__ float red[4];
    const int u = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
    int b, hq, slice;
    gen_query(a, u, i, b, hq, slice);
    const GenSide &V = a.v;
    const int nv = V.ui[u].n_slots, stride = V.kslots + 2;
    const float *part = a.part + static_cast<int64_t>(u) * a.nchunks * a.Q * stride + static_cast<int64_t>(i) * stride;
    const int64_t cstride = static_cast<int64_t>(a.Q) * stride;
    float m = -__builtin_huge_valf();
    for (int c = tid; c < a.nchunks; c += blockDim.x) m = fmaxf(m, part[c * cstride + V.kslots]);
    const float M = block_reduce(m, red, true);
    float l = 0.f;
    for (int c = tid; c < a.nchunks; c += blockDim.x) l += expf(part[c * cstride + V.kslots] - M) * part[c * cstride + V.kslots + 1];
    const float L = block_reduce(l, red, false);
    for (int j = tid; j < V.kslots; j += blockDim.x) {
        float s = 0.f;
        if (j < nv) {
            for (int c = 0; c < a.nchunks; ++c) s = fmaf(expf(part[c * cstride + V.kslots] - M), part[c * cstride + j], s);
            s = s / L;
            if (!V.mixed) s *= V.qscale[static_cast<int64_t>(u) * V.rmax + V.comp[static_cast<int64_t>(u) * V.kslots + j]];
        }
        coef[j] = s;
    }
    __syncthreads();
    for (int d = tid; d < a.D; d += blockDim.x) {
        float o = 0.f;
        if (a.nchunks > 0) {
            o = (V.mixed ? V.mu : V.bias)[static_cast<int64_t>(u) * V.dg + slice + d];
            const float *vb = V.basis + static_cast<int64_t>(u) * V.kslots * V.dg + slice + d;
            for (int j = 0; j < nv; ++j) o = fmaf(coef[j], vb[static_cast<int64_t>(j) * V.dg], o);
        }
        a.out[b * a.osb + hq * a.osh + d] = static_cast<_Float16>(o);
    }
}

GenSide gen_side(const kvtc_state_header *h, const void *state_dev, const void *codes, const void *params,
                 int64_t capacity) {
    const char *sd = static_cast<const char *>(state_dev);
    GenSide g{};
    g.codes = static_cast<const uint8_t *>(codes);
    g.params = static_cast<const uint32_t *>(params);
    g.capacity = capacity;
    g.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    g.basis = reinterpret_cast<const float *>(sd + h->off_basis);
    g.mu = reinterpret_cast<const float *>(sd + h->off_mu);
    g.qmin = reinterpret_cast<const float *>(sd + h->off_qmin);
    g.qscale = reinterpret_cast<const float *>(sd + h->off_qscale);
    g.bias = reinterpret_cast<const float *>(sd + h->off_bias);
    g.comp = reinterpret_cast<const int32_t *>(sd + h->off_slot_comp);
    g.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    g.kslots = h->kslots;
    g.rmax = h->rmax;
    g.row_words = h->row_stride / 4;
    g.n_qg = h->mode == KVTC_MODE_MIXED ? h->n_qgroups : 0;
    g.gs = h->group_size;
    g.mixed = h->mode == KVTC_MODE_MIXED;
    g.dg = h->dg;
    return g;
}

// Workspace of the general path, regions 256-byte aligned: qt, qb, qp, part.
struct GenWork {
    uint64_t qt, qb, qp, part, total;
};

GenWork gen_work(const kvtc_state_header *hk, const kvtc_state_header *hv, int Q, int64_t s_end) {
    GenWork w{};
    const uint64_t U = static_cast<uint64_t>(hk->units);
    const int64_t nch = (s_end + kGenRows - 1) / kGenRows;
    const int ng = hk->mode == KVTC_MODE_MIXED ? hk->n_qgroups : 0;
    w.qt = 0;
    w.qb = align_up(U * Q * hk->kslots * 4, 256);
    w.qp = w.qb + align_up(U * Q * 4, 256);
    w.part = w.qp + align_up(U * Q * std::max(ng, 1) * 4, 256);
    w.total = w.part + U * static_cast<uint64_t>(nch) * Q * (hv->kslots + 2) * 4;
    return w;
}

size_t gen_lds_bytes(const kvtc_state_header *hk, const kvtc_state_header *hv, int QM) {
    const int ng = hk->mode == KVTC_MODE_MIXED ? hk->n_qgroups : 0;
    const int ngv = hv->mode == KVTC_MODE_MIXED ? hv->n_qgroups : 0;
    const int pitch = (std::max(hk->row_stride, hv->row_stride) / 4 + 1) | 1;
    return (static_cast<size_t>(QM) * hk->kslots + QM + static_cast<size_t>(QM) * std::max(ng, 1) +
            static_cast<size_t>(QM) * kGenRows + 2 * QM) * 4 +
           (kMaxSlots + static_cast<size_t>(kGenRows) * pitch + static_cast<size_t>(std::max(ng, ngv)) * kGenRows) * 4;
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

int32_t attend_impl(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t q_heads, const void *q_dev,
                    int32_t q_dtype, const int64_t q_strides[3], int64_t s_end, void *out_dev,
                    const int64_t out_strides[3], void *work_dev, size_t work_bytes, bool noalloc, hipStream_t stream);
int32_t attend_workspace_impl(const void *k_state_host, const void *v_state_host, int64_t q_heads, int64_t s_end,
                              size_t *bytes);

}  // namespace
}  // namespace kvtc

using namespace kvtc;

extern "C" {

int32_t kvtc_attend_workspace(const void *k_state_host, const void *v_state_host, int64_t s_end, size_t *bytes) {
    const kvtc_state_header *hk = nullptr;
    const int32_t st = check_state(k_state_host, &hk);
    if (st != KVTC_OK) return st;
    return attend_workspace_impl(k_state_host, v_state_host, hk->heads, s_end, bytes);
}

int32_t kvtc_attend_gqa_workspace(const void *k_state_host, const void *v_state_host, int64_t q_heads, int64_t s_end,
                                  size_t *bytes) {
    return attend_workspace_impl(k_state_host, v_state_host, q_heads, s_end, bytes);
}

int32_t kvtc_attend(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                    const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                    void *work_dev, size_t work_bytes, void *hip_stream) {
    return attend_impl(k, v, 0, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, work_dev, work_bytes, false,
                       static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_attend_gqa(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t q_heads, const void *q_dev,
                        int32_t q_dtype, const int64_t q_strides[3], int64_t s_end, void *out_dev,
                        const int64_t out_strides[3], void *work_dev, size_t work_bytes, void *hip_stream) {
    if (q_heads < 1) return KVTC_E_ARG;
    return attend_impl(k, v, q_heads, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, work_dev, work_bytes,
                       false, static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_attend_noalloc(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const void *q_dev, int32_t q_dtype,
                            const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                            void *hip_stream) {
    return attend_impl(k, v, 0, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, nullptr, 0, true,
                       static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

namespace kvtc {
namespace {

// The path a call takes: the per-head kernels (DP caches, one query per head)
// or the general ones; the workspace it needs; KVTC_OK or why it is refused.
struct AttendRoute {
    bool fast;
    int Q, G, QM;
    size_t work;
};

int32_t attend_route(const kvtc_state_header *hk, const kvtc_state_header *hv, int64_t q_heads, int64_t s_end,
                     AttendRoute *r) {
    if (hk->batch != hv->batch || hk->heads != hv->heads || hk->head_dim != hv->head_dim ||
        hk->heads_per_unit != hv->heads_per_unit)
        return KVTC_E_SHAPE;
    if (q_heads < 1 || q_heads % hk->heads != 0) return KVTC_E_SHAPE;
    const int64_t G = q_heads / hk->heads;
    r->G = static_cast<int>(std::min<int64_t>(G, 1 << 20));
    r->fast = G == 1 && attend_side_ok(hk) == KVTC_OK && attend_side_ok(hv) == KVTC_OK;
    if (r->fast) {
        r->Q = 1;
        r->QM = 1;
        r->work = attend_work_bytes(hk, hv, s_end);
        return KVTC_OK;
    }
    const int64_t Q = G * hk->heads_per_unit;
    if (Q > kGenMaxQ || hk->head_dim > kMaxSlots || hk->kslots > kMaxSlots || hv->kslots > kMaxSlots ||
        hk->row_stride > kMaxRowStride || hv->row_stride > kMaxRowStride)
        return KVTC_E_SHAPE;
    r->Q = static_cast<int>(Q);
    r->QM = Q <= 8 ? 8 : kGenMaxQ;
    if (gen_lds_bytes(hk, hv, r->QM) > kLdsMax) return KVTC_E_SHAPE;
    r->work = gen_work(hk, hv, r->Q, s_end).total;
    return KVTC_OK;
}

int32_t attend_workspace_impl(const void *k_state_host, const void *v_state_host, int64_t q_heads, int64_t s_end,
                              size_t *bytes) {
    const kvtc_state_header *hk = nullptr, *hv = nullptr;
    int32_t st = check_state(k_state_host, &hk);
    if (st != KVTC_OK) return st;
    st = check_state(v_state_host, &hv);
    if (st != KVTC_OK) return st;
    if (!bytes || s_end < 0) return KVTC_E_ARG;
    AttendRoute r{};
    st = attend_route(hk, hv, q_heads, s_end, &r);
    if (st != KVTC_OK) return st;
    *bytes = r.work;
    return KVTC_OK;
}

int32_t launch_gen(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, const kvtc_state_header *hk,
                   const kvtc_state_header *hv, const AttendRoute &r, const void *q_dev, int32_t q_dtype,
                   const int64_t q_strides[3], int64_t s_end, void *out_dev, const int64_t out_strides[3],
                   void *work_dev, hipStream_t stream) {
    GenArgs a{};
    a.k = gen_side(hk, k->state_dev, k->codes_dev, k->params_dev, k->capacity);
    a.v = gen_side(hv, v->state_dev, v->codes_dev, v->params_dev, v->capacity);
    a.q = q_dev;
    a.qsb = q_strides[0];
    a.qsh = q_strides[1];
    a.q_f16 = q_dtype == KVTC_F16;
    a.out = static_cast<_Float16 *>(out_dev);
    a.osb = out_strides[0];
    a.osh = out_strides[1];
    a.s_end = s_end;
    a.nchunks = static_cast<int>((s_end + kGenRows - 1) / kGenRows);
    a.G = r.G;
    a.hpu = hk->heads_per_unit;
    a.groups = static_cast<int>(hk->heads / hk->heads_per_unit);
    a.D = hk->head_dim;
    a.Q = r.Q;
    a.inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(hk->head_dim));
    const GenWork wl = gen_work(hk, hv, r.Q, s_end);
    char *wb = static_cast<char *>(work_dev);
    a.qt = reinterpret_cast<float *>(wb + wl.qt);
    a.qb = reinterpret_cast<float *>(wb + wl.qb);
    a.qp = reinterpret_cast<float *>(wb + wl.qp);
    a.part = reinterpret_cast<float *>(wb + wl.part);
    const unsigned U = static_cast<unsigned>(hk->units), Q = static_cast<unsigned>(r.Q);
    hipLaunchKernelGGL(attend_gen_prep_kernel, dim3(U, Q), dim3(256), 0, stream, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    if (a.nchunks > 0) {
        const size_t lds = gen_lds_bytes(hk, hv, r.QM);
        auto kern = r.QM == 8 ? attend_gen_partial_kernel<8> : attend_gen_partial_kernel<kGenMaxQ>;
        if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.nchunks), U), dim3(256), lds, stream, a);
        if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    }
    hipLaunchKernelGGL(attend_gen_merge_kernel, dim3(U, Q), dim3(256), 0, stream, a);
    return launch_status();
}

// Validates the call, then launches the attention kernels on the given
// workspace; with noalloc the workspace is this device's scratch array (after
// its size has been checked against the call's need).  q_heads == 0: one query
// per stored head.
int32_t attend_impl(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t q_heads, const void *q_dev,
                    int32_t q_dtype, const int64_t q_strides[3], int64_t s_end, void *out_dev,
                    const int64_t out_strides[3], void *work_dev, size_t work_bytes, bool noalloc, hipStream_t stream) {
    if (!k || !v || !q_strides || !out_strides) return KVTC_E_ARG;
    const kvtc_state_header *hk = nullptr, *hv = nullptr;
    int32_t st = check_state(k->state_host, &hk);
    if (st != KVTC_OK) return st;
    st = check_state(v->state_host, &hv);
    if (st != KVTC_OK) return st;
    if (q_heads == 0) q_heads = hk->heads;
    if (q_dtype != KVTC_F16 && q_dtype != KVTC_F32) return KVTC_E_DTYPE;
    if (q_strides[2] != 1 || out_strides[2] != 1 || q_strides[0] < 0 || q_strides[1] < 0 || out_strides[0] < 0 ||
        out_strides[1] < 0)
        return KVTC_E_SHAPE;
    if (s_end < 0 || k->capacity < 0 || v->capacity < 0) return KVTC_E_ARG;
    AttendRoute route{};
    if ((st = attend_route(hk, hv, q_heads, s_end, &route)) != KVTC_OK) return st;
    if (s_end > k->capacity || s_end > v->capacity) return KVTC_E_CAPACITY;
    if (!k->state_dev || !v->state_dev || !q_dev || !out_dev) return KVTC_E_ARG;
    if (s_end > 0 && ((hk->row_stride > 0 && (!k->codes_dev || reinterpret_cast<uintptr_t>(k->codes_dev) % 4)) ||
                      (hv->row_stride > 0 && (!v->codes_dev || reinterpret_cast<uintptr_t>(v->codes_dev) % 4))))
        return KVTC_E_ARG;
    if (s_end > 0 && ((hk->mode == KVTC_MODE_MIXED && (!k->params_dev || reinterpret_cast<uintptr_t>(k->params_dev) % 4)) ||
                      (hv->mode == KVTC_MODE_MIXED && (!v->params_dev || reinterpret_cast<uintptr_t>(v->params_dev) % 4))))
        return KVTC_E_ARG;
    if (reinterpret_cast<uintptr_t>(out_dev) % 2 || reinterpret_cast<uintptr_t>(q_dev) % (q_dtype == KVTC_F16 ? 2 : 4))
        return KVTC_E_ARG;
    const size_t need = route.work;
    if (noalloc) {
        if (need > kAttendScratchBytes) return KVTC_E_BUFSIZE;
        const int32_t sa = scratch_address(&work_dev);
        if (sa != KVTC_OK) return sa;
        work_bytes = kAttendScratchBytes;
    }
    if (!work_dev || work_bytes < need || reinterpret_cast<uintptr_t>(work_dev) % 256) return KVTC_E_BUFSIZE;
    const int64_t nchunks = (s_end + kAttChunk - 1) / kAttChunk;
    if (hk->units > 0x7FFFFFFF || nchunks > 0x7FFFFFFF || hk->units > 65535) return KVTC_E_SHAPE;
    if (!route.fast)
        return launch_gen(k, v, hk, hv, route, q_dev, q_dtype, q_strides, s_end, out_dev, out_strides, work_dev, stream);

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
    // rows shared evenly between the chunks (no nearly empty last chunk)
    a.chunk_rows = nchunks > 0 ? static_cast<int>((s_end + nchunks - 1) / nchunks) : 0;
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
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    if (nchunks > 0) {
        const int rw = std::max(a.k.row_words, a.v.row_words);
        const size_t lds = (kMaxSlots + 4 + 2 * kMaxSlots + kAttChunk + 4 * kMaxSlots) * sizeof(float) +
                           (static_cast<size_t>(kAttChunk) * ((rw + 1) | 1) + 8) * sizeof(uint32_t);
        if (lds > kLdsMax) return KVTC_E_SHAPE;
        if (!allow_lds(reinterpret_cast<const void *>(attend_partial_kernel))) return KVTC_E_DEVICE;
        hipLaunchKernelGGL(attend_partial_kernel, dim3(static_cast<unsigned>(nchunks), U), dim3(256), lds, stream, a);
        if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    }
    hipLaunchKernelGGL(attend_merge_kernel, dim3(U), dim3(256), 0, stream, a);
    return launch_status();
}

}  // namespace
}  // namespace kvtc
