// Bulk append on int8 MFMA (gfx950): the projection of fp16 rows as an exact
// integer product, every decision certified against an error bound, and the
// fp64 tile of append_kernel for any block with a decision it cannot certify.
//
// KVTC cache module page, _TensorKVTC.append / _requantize (centre, project,
// min/max affine codes); PALU cache API page, "Design" (per-token fp16 ranges of
// groups of latents).
//
// The latent of row x and slot j is l = (x - mu) . V_j.  Every fp16 value is an
// integer multiple of 2^-24, so X = x * 2^24 is an exact integer (below
// 127 * 2^24 in magnitude when |x| < 127) and splits exactly into four balanced
// base-256 digits; the blob holds vq = rint(V_j * 2^38) in five.  The digit
// products on v_mfma_i32_32x32x32_i8 accumulate exactly in int32, one
// accumulator per weight 256^w (w = sum of the two digit indices); the weights
// w >= 2 give
//   l~ = 2^-62 * sum_{w>=2} 256^w acc_w  -  mu . V_j       (mu . V_j from the blob)
// with |l~ - l| <= sum|x| 2^-39 (rounding of vq) + dg 2^-39 (1 + 2^-9) (weights
// 0 and 1 left out) + dg 2^-53 sum|mu| (mu . V_j in float64) + float64
// roundings below 2^-51 (sum|x| + sum|mu|).  The fp64 kernels' latent R (their
// MFMA sequence on fp64 x - mu) lies within (dg + 9) 2^-53 (sum|x| + sum|mu|) of
// l (|V| <= 1).  For dg <= 2048 the sum of these stays below
//   E = 2^-39 (1.5 sum|x| + 1.1 dg + 0.5 sum|mu|)
// (sum|x| and sum|mu| summed in fp32, short by far less than the margins), so R
// lies inside [l~ - E, l~ + E].  The quantiser and the
// fp16 rounding of a group's range are monotone in the latents, so a decision
// that comes out the same at both ends of that interval is the decision the
// fp64 kernels take on R.  A block with any decision that differs at the two
// ends (or a row value with |x| >= 127 or not finite) runs the fp64 tile of
// append_kernel on its tokens and slots instead, so every row gets exactly the
// codes and params the fp64 kernels give it.
#include "kvtc_append_tile.h"

namespace kvtc {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kI8Tok = 64;          // tokens per block: two 32-token tiles
constexpr int kI8K = 32;            // features per k-step (one MFMA K)
constexpr int kXd = 4, kVd = 5;     // digits of a row value and of a basis value
constexpr int kXChunks = kI8Tok * kI8K / 4;   // 4-element row chunks per k-step
constexpr int kI8Ring = 4;          // k-steps of loads in flight (the unit width is a multiple of 4 k-steps)

// LDS of the digit staging: [2][4][64][32] row digits and [2][5][32 NS][32]
// basis digits (bytes).
__host__ __device__ constexpr size_t i8_stage_bytes(int ns) {
    return static_cast<size_t>(2) * kXd * kI8Tok * kI8K + static_cast<size_t>(2) * kVd * 32 * ns * kI8K;
}

// The four balanced base-256 digits of X (|X| < 127 * 2^24), low digit first.
__device__ inline void digits4(int X, int (&d)[kXd]) {
    d[0] = (X << 24) >> 24;
    X = (X - d[0]) >> 8;
    d[1] = (X << 24) >> 24;
    X = (X - d[1]) >> 8;
    d[2] = (X << 24) >> 24;
    d[3] = (X - d[2]) >> 8;
}

// Block = 64 tokens x 32 NS slots [slot0, slot0 + 32 NS) of one unit; wave w
// computes the 32 x 32 tile of tokens 32 (w & 1).. and slots 32 (w >> 1)..
// (MFMA A = basis digits, rows = slots; B = row digits, columns = tokens).
// Blocks are numbered unit-major (unit, slot group, token tile) and spread so
// that each XCD runs a contiguous range: the units' basis digits stay in its L2.
template <bool MIXED, int NS, int PF>
__global__ __launch_bounds__(128 * NS, 2) void append_i8_kernel(AppendArgs a, int tiles, int nsg, int nlogical,
                                                             int per_xcd) {
    constexpr int NT = 128 * NS, SL = 32 * NS;
    constexpr int XI = (kXChunks + NT - 1) / NT;             // row chunks per thread and k-step
    constexpr int VI = (kVd * SL * 2 + NT - 1) / NT;         // 16-byte digit chunks per thread and k-step
    static_assert(f64_stage_bytes(2 * NS) <= i8_stage_bytes(NS), "fp64 tile staging fits the digit staging");
    extern __shared__ __align__(16) unsigned char smem[];
    uint8_t *xd = smem;                                              // [2][4][64][32]
    uint8_t *vd = smem + static_cast<size_t>(2) * kXd * kI8Tok * kI8K;   // [2][5][SL][32]
    const int row_words = a.row_stride >> 2;
    uint32_t *rows = reinterpret_cast<uint32_t *>(smem + i8_stage_bytes(NS));     // [64][row_words]
    float *tabs = reinterpret_cast<float *>(rows + kI8Tok * row_words);           // [64] sum |x| per token
    float *misc = tabs + kI8Tok;                                                  // sum |mu|, fallback flag
    uint8_t *trash = reinterpret_cast<uint8_t *>(misc + 4);   // 16 bytes nobody reads (stores of chunks past the end)

    const int logical = static_cast<int>((blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3));
    if (logical >= nlogical) return;
    const int tile = logical % tiles, rest = logical / tiles;
    const int sg = rest % nsg, u = rest / nsg;
    const int slot0 = sg * SL;
    const int64_t t0 = static_cast<int64_t>(tile) * kI8Tok;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = u / a.groups, g = u % a.groups;
    const int nvalid = static_cast<int>(min<int64_t>(kI8Tok, a.n - t0));
    const int n_slots = a.ui[u].n_slots;
    const int64_t ub = static_cast<int64_t>(u) * a.kslots;
    const _Float16 *x = static_cast<const _Float16 *>(a.x);

    for (int w = tid; w < kI8Tok * row_words; w += NT) rows[w] = 0u;
    if (tid < kI8Tok) tabs[tid] = 0.f;
    if (tid < 4) misc[tid] = 0.f;
    int *gmask = reinterpret_cast<int *>(misc + 2);   // 16-token groups with a decision left to the fp64 tile
    __syncthreads();
    {   // sum |mu| over the unit's row (a term of the error bound only)
        float s = 0.f;
        for (int d = tid; d < a.dg; d += NT) s += fabsf(a.mu[static_cast<int64_t>(u) * a.dg + d]);
        atomicAdd(&misc[0], s);
    }

    // k-step loads go to a register ring PF deep: the loads of k-step kk + PF
    // are issued while k-step kk is multiplied, and k-step kk + 1's registers
    // become digits in LDS after it.  Every load is issued unconditionally
    // (indices clamped; past the last k-step the last one is loaded again), so
    // no load sits behind a branch and each wait covers only the oldest k-step.
    // Per-thread addresses are fixed; a k-step adds a wave-uniform offset.
    const _Float16 *xp[XI];
    const int8_t *vp[VI];
    uint8_t *xdst[XI];
    uint8_t *vdst[VI];
    bool xreal[XI], vreal[VI], vkeep[VI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int c = tid + i * NT;
        const bool real = c < kXChunks;
        const int cc = real ? c : kXChunks - 1;
        const int tok = min(cc >> 3, nvalid - 1);          // rows past the valid ones repeat the last
        xp[i] = x + b * a.xsb + static_cast<int64_t>(g) * a.hpu * a.xsh + (t0 + tok) * a.xss + (cc & 7) * 4;
        xreal[i] = real;
        xdst[i] = xd + (cc >> 3) * kI8K + (cc & 7) * 4;
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
        const int c = tid + i * NT;
        const bool real = c < kVd * SL * 2;
        const int cc = real ? c : 0;
        const int sd = cc / (2 * SL), rem = cc - sd * 2 * SL;
        vkeep[i] = slot0 + (rem >> 1) < a.kslots;           // slots past kslots are zero
        const int slot = min(slot0 + (rem >> 1), a.kslots - 1);
        vp[i] = a.vdig + ((static_cast<int64_t>(u) * kVd + sd) * a.kslots + slot) * a.dg + (rem & 1) * 16;
        vreal[i] = real;
        vdst[i] = vd + (sd * SL + (rem >> 1)) * kI8K + (rem & 1) * 16;
    }
    constexpr int kXPlane = kI8Tok * kI8K, kVBuf = kVd * SL * kI8K;   // bytes of a row-digit plane, a basis buffer
    u32x2 xr[PF][XI];
    i32x4 vr[PF][VI];
    float sabs[XI], amax = 0.f;
#pragma unroll
    for (int i = 0; i < XI; ++i) sabs[i] = 0.f;
    auto load = [&](int kk, u32x2 (&xs)[XI], i32x4 (&vs)[VI]) __attribute__((always_inline)) {
        const int f = kk * kI8K, j = f / a.D;                        // wave-uniform: one head per k-step
        const int64_t xo = j * a.xsh + (f - j * a.D);
#pragma unroll
        for (int i = 0; i < XI; ++i) xs[i] = *reinterpret_cast<const u32x2 *>(xp[i] + xo);
#pragma unroll
        for (int i = 0; i < VI; ++i) vs[i] = *reinterpret_cast<const i32x4 *>(vp[i] + f);
    };
    // Digits of one k-step into LDS buffer buf.  With X = x * 2^24 (an integer,
    // |X| < 2^31), the bytes s_k of X ^ 0x808080 read as int8 satisfy
    //   X = sum_k 256^k s_k + 0x808080
    // (adding 2^31 and 128 per byte makes every byte unsigned, and each byte u
    // read as int8 is u - 128), so the row digits are plain byte planes and the
    // constant goes into the per-slot offset of the blob.  count: add |x| to the
    // per-token sums.
    auto store = [&](int buf, const u32x2 (&xs)[XI], const i32x4 (&vs)[VI], bool count) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t hb = static_cast<uint16_t>(xs[i][e >> 1] >> (16 * (e & 1)));
                const float xf = static_cast<float>(__builtin_bit_cast(_Float16, hb));
                amax = fmaxf(amax, fabsf(xf));
                sabs[i] += count ? fabsf(xf) : 0.f;
                w[e] = static_cast<uint32_t>(static_cast<int>(xf * 16777216.0f)) ^ 0x808080u;
            }
            // 4 x 4 byte transpose: plane k holds byte k of the four values
            const uint32_t t0 = __builtin_amdgcn_perm(w[1], w[0], 0x06020400u);
            const uint32_t t1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030501u);
            const uint32_t t2 = __builtin_amdgcn_perm(w[3], w[2], 0x06020400u);
            const uint32_t t3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030501u);
            const uint32_t pl[kXd] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x05040100u),
                                      __builtin_amdgcn_perm(t2, t0, 0x07060302u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
            for (int k = 0; k < kXd; ++k) {
                uint8_t *dst = xreal[i] ? xdst[i] + (buf * kXd + k) * kXPlane : trash;   // no store behind a branch
                *reinterpret_cast<uint32_t *>(dst) = pl[k];
            }
        }
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const i32x4 z = {0, 0, 0, 0};
            uint8_t *dst = vreal[i] ? vdst[i] + buf * kVBuf : trash;
            *reinterpret_cast<i32x4 *>(dst) = vkeep[i] ? vs[i] : z;
        }
    };

    const int tt = wave & 1, st = wave >> 1;
    i32x16 acc[6];          // weights 256^2 .. 256^7
#pragma unroll
    for (int w = 0; w < 6; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[w][i] = 0;
    auto product = [&](int buf) __attribute__((always_inline)) {
        i32x4 xb[kXd], va[kVd];
#pragma unroll
        for (int k = 0; k < kXd; ++k)
            xb[k] = *reinterpret_cast<const i32x4 *>(xd + ((buf * kXd + k) * kI8Tok + 32 * tt + (lane & 31)) * kI8K +
                                                     (lane >> 5) * 16);
#pragma unroll
        for (int s = 0; s < kVd; ++s)
            va[s] = *reinterpret_cast<const i32x4 *>(vd + ((buf * kVd + s) * SL + 32 * st + (lane & 31)) * kI8K +
                                                     (lane >> 5) * 16);
        // digit pairs (row digit i, basis digit k) into weight i + k; consecutive
        // products go to different accumulators
#define KVTC_I8(W, I, K) acc[(W) - 2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va[K], xb[I], acc[(W) - 2], 0, 0, 0)
        KVTC_I8(2, 0, 2); KVTC_I8(3, 0, 3); KVTC_I8(4, 0, 4); KVTC_I8(5, 1, 4); KVTC_I8(6, 2, 4); KVTC_I8(7, 3, 4);
        KVTC_I8(2, 1, 1); KVTC_I8(3, 1, 2); KVTC_I8(4, 1, 3); KVTC_I8(5, 2, 3); KVTC_I8(6, 3, 3);
        KVTC_I8(2, 2, 0); KVTC_I8(3, 2, 1); KVTC_I8(4, 2, 2); KVTC_I8(5, 3, 2);
        KVTC_I8(3, 3, 0); KVTC_I8(4, 3, 1);
#undef KVTC_I8
    };
    const int nk = a.dg / kI8K;          // a multiple of PF (checked when the launch is planned)
#pragma unroll
    for (int r = 0; r < PF; ++r) load(r, xr[r], vr[r]);
    store(0, xr[0], vr[0], true);
    __syncthreads();
    for (int kb = 0; kb < nk; kb += PF) {
#pragma unroll
        for (int r = 0; r < PF; ++r) {
            const int kk = kb + r;
            product(r & 1);
            // the phases stay in this order (the scheduler would otherwise convert
            // later ring slots early and wait for their loads): the VALU work of
            // the store runs while the MFMAs issued above execute
            __builtin_amdgcn_sched_barrier(0);
            // k-step kk + 1 into the other buffer (past the end: a repeat, not counted)
            store((r & 1) ^ 1, xr[(r + 1) % PF], vr[(r + 1) % PF], kk + 1 < nk);
            __builtin_amdgcn_sched_barrier(0);
            load(min(kk + PF, nk - 1), xr[r], vr[r]);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
    }

    // sum |x| per token: for each chunk index the eight threads of a token are
    // eight consecutive lanes
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        float s = sabs[i];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        const int c = tid + i * NT;
        if ((tid & 7) == 0 && c < kXChunks) tabs[c >> 3] = s;
    }
    // a row value with |x| >= 127, or not a number (the sums then are not finite),
    // leaves the int8 range: the block takes the fp64 tile
    bool xbad = !(amax < 127.0f);
#pragma unroll
    for (int i = 0; i < XI; ++i) xbad = xbad || !(sabs[i] < 3.0e38f);
    if (xbad) misc[1] = 1.f;
    __syncthreads();

    // 32x32 result layout: element 4q + e of a lane is slot 32 st + 8q + 4 (lane >> 5) + e
    // (of the block's range) and token 32 tt + (lane & 31)
    const int tok = 32 * tt + (lane & 31);
    const bool tok_ok = tok < nvalid;
    const double E = 0x1p-39 * (1.5 * static_cast<double>(tabs[tok]) + 1.1 * static_cast<double>(a.dg) +
                                0.5 * static_cast<double>(misc[0]));
    bool bad = false;        // a decision of this lane's token left to the fp64 tile
    double lt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int sl = slot0 + 32 * st + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        double h = static_cast<double>(acc[5][i]);
#pragma unroll
        for (int w = 4; w >= 0; --w) h = h * 256.0 + static_cast<double>(acc[w][i]);
        lt[i] = h * 0x1p-46 - (sl < a.kslots ? a.mv[ub + sl] : 0.0);
    }
    uint32_t *myrow = rows + tok * row_words;
    if constexpr (!MIXED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int sl = slot0 + 32 * st + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (tok_ok && sl < n_slots) {
                const double lo = a.qlo[ub + sl], inv = a.qinv[ub + sl];
                const uint32_t sb = a.sbits[ub + sl];
                const uint32_t w = sb >> 24;
                const double cmax = static_cast<double>((1u << w) - 1u);
                const double c1 = quantise(lt[i] - E, lo, inv, cmax), c2 = quantise(lt[i] + E, lo, inv, cmax);
                if (c1 != c2)
                    bad = true;
                else
                    or_field(myrow, sb & kOffsetMask, w, static_cast<uint32_t>(c1));
            }
        }
    } else {
        // one quantisation group (32 slots) per wave tile: a token's values are
        // in lanes l and l ^ 32
        const int j0 = slot0 + 32 * st;
        if (j0 < n_slots) {
            const uint32_t w = a.sbits[ub + j0] >> 24;
            const double cmax = static_cast<double>((1u << w) - 1u);
            double mn = __builtin_huge_val(), mx = -__builtin_huge_val();
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int sl = j0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (sl < n_slots) {
                    mn = fmin(mn, lt[i]);
                    mx = fmax(mx, lt[i]);
                }
            }
            mn = fmin(mn, __shfl_xor(mn, 32, 64));
            mx = fmax(mx, __shfl_xor(mx, 32, 64));
            const uint16_t hmin = half_bits_rne(mn - E), hmin2 = half_bits_rne(mn + E);
            const uint16_t hs = half_bits_rne(((mx - E) - (mn + E)) / cmax);
            const uint16_t hs2 = half_bits_rne(((mx + E) - (mn - E)) / cmax);
            if (tok_ok) {
                if (hmin != hmin2 || hs != hs2) {
                    bad = true;
                } else {
                    const double lo16 = half_bits_to_double(hmin), sc = half_bits_to_double(hs);
                    const double inv16 = sc > 0.0 ? 1.0 / sc : 0.0;
                    if (lane < 32)
                        a.params[(static_cast<int64_t>(u) * a.capacity + a.s0 + t0 + tok) * a.n_qg + j0 / a.gs] =
                            static_cast<uint32_t>(hmin) | (static_cast<uint32_t>(hs) << 16);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int sl = j0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                        if (sl < n_slots) {
                            const double c1 = quantise(lt[i] - E, lo16, inv16, cmax);
                            const double c2 = quantise(lt[i] + E, lo16, inv16, cmax);
                            if (c1 != c2)
                                bad = true;
                            else
                                or_field(myrow, a.sbits[ub + sl] & kOffsetMask, w, static_cast<uint32_t>(c1));
                        }
                    }
                }
            }
        }
    }

    // block-wide OR of the flags in the LDS word that already holds the row-range
    // flag (any writer stores 1; a thread that read it early saw 0 or 1, both
    // consistent with the outcome); no static LDS, so the kernel may use the
    // whole LDS dynamically
    // the 16-token groups (the fp64 tile's waves) with a decision left to it;
    // a row value outside the int8 range sends every group
    if (bad) atomicOr(gmask, 1 << (tok >> 4));
    __syncthreads();
    const int need = misc[1] != 0.f ? 0xF : *gmask;
    if (need) {
        // the fp64 tile of append_kernel on this block's slots, for the groups
        // that need it: their rows are cleared and rewritten, the others keep
        // their certified codes (every row's result is its own: the same bytes)
        for (int w = tid; w < kI8Tok * row_words; w += NT)
            if ((need >> ((w / row_words) >> 4)) & 1) rows[w] = 0u;
        doublex4 acc64[2 * NS];
        const bool active = wave < 4 && ((need >> wave) & 1);
        f64_project<_Float16, 2 * NS, true>(a, u, t0, nvalid, slot0, smem, acc64, active);
        if (active) f64_quantise<MIXED, 2 * NS>(a, u, t0, nvalid, slot0, acc64, rows);
        __syncthreads();
    }

    // this block's words of each row: slot group boundaries inside a unit's
    // slots are whole words (checked when the launch is planned)
    int w_lo = 0, w_hi = row_words;
    if (sg > 0) w_lo = slot0 < n_slots ? static_cast<int>((a.sbits[ub + slot0] & kOffsetMask) >> 5) : row_words;
    if (sg + 1 < nsg)
        w_hi = slot0 + SL < n_slots ? static_cast<int>((a.sbits[ub + slot0 + SL] & kOffsetMask) >> 5) : row_words;
    const int nw = w_hi - w_lo;
    if (nw > 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            a.codes + (static_cast<int64_t>(u) * a.capacity + a.s0 + t0) * a.row_stride);
        for (int i = tid; i < nvalid * nw; i += NT) {
            const int t = i / nw, w = w_lo + (i - t * nw);
            dst[t * row_words + w] = rows[t * row_words + w];
        }
    }
}

template <bool MIXED, int NS>
int32_t launch_i8_ns(const AppendPlan &p, hipStream_t stream) {
    const AppendArgs &a = p.a;
    const int64_t tiles = (a.n + kI8Tok - 1) / kI8Tok;
    const int64_t nlogical = tiles * p.units * p.i8_nsg;
    if (nlogical > 0x7FFFFFF0LL) return KVTC_E_SHAPE;
    const int64_t per_xcd = (nlogical + 7) / 8;
    const size_t lds = i8_stage_bytes(NS) + static_cast<size_t>(kI8Tok) * (a.row_stride / 4) * sizeof(uint32_t) +
                       (kI8Tok + 4) * sizeof(float) + 16;
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    auto kern = append_i8_kernel<MIXED, NS, kI8Ring>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(128 * NS), lds, stream, a,
                       static_cast<int>(tiles), p.i8_nsg, static_cast<int>(nlogical), static_cast<int>(per_xcd));
    return launch_status();
}

}  // namespace

int32_t launch_append_i8(const AppendPlan &p, hipStream_t stream) {
    if (p.a.n == 0) return KVTC_OK;
    switch (p.i8_ns) {
        case 2: return p.mixed ? launch_i8_ns<true, 2>(p, stream) : launch_i8_ns<false, 2>(p, stream);
        case 3: return p.mixed ? launch_i8_ns<true, 3>(p, stream) : launch_i8_ns<false, 3>(p, stream);
        case 4: return p.mixed ? launch_i8_ns<true, 4>(p, stream) : launch_i8_ns<false, 4>(p, stream);
        default: return KVTC_E_SHAPE;
    }
}

}  // namespace kvtc
