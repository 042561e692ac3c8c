// The fp64 tile of the bulk append (gfx950): projection of 64 tokens of one
// unit onto a range of 16-slot N-blocks on fp64 MFMA, then quantisation and
// packing into LDS bit rows.  append_kernel runs it over all slots; the int8
// append kernel runs it over its own slot range whenever it cannot certify a
// decision, so both give a row the same latents, bit for bit.
//
// KVTC cache module page, _TensorKVTC.append / _requantize (centre, project,
// min/max affine codes); PALU cache API page, "Design" (per-token group ranges).
#pragma once
#include "kvtc_device.h"

namespace kvtc {

// LDS of the projection's staging: [2][64][kAppPad] centred rows (fp64) and
// [2][NB*16][kAppPad] basis columns (fp32).
__host__ __device__ constexpr size_t f64_stage_bytes(int nb) {
    return 2 * kAppTok * kAppPad * sizeof(double) + 2 * static_cast<size_t>(nb) * 16 * kAppPad * sizeof(float);
}

// Latents of tokens [t0, t0 + nvalid) of unit u on slots [slot0, slot0 + 16 NB):
// the block's first four waves hold the result, acc[nb][i] being the latent of
// token 16*wave + (lane >> 4) + 4i and slot slot0 + 16nb + (lane & 15); a wave
// called with active false skips its products (its tokens are not needed).  The
// first 256 threads stage; every thread of the block must call this (barriers).
// K-step order: k-step 4c + e of the contraction takes, at operand k = q, the
// feature 16c + 4q + e (c = 16-column chunk); every append kernel uses this
// order, so that a lane of the decode kernel holds its operands as whole
// 16-byte vectors of the basis.
template <typename XT, int NB, bool XVEC>
__device__ __forceinline__ void f64_project(const AppendArgs &a, int u, int64_t t0, int nvalid, int slot0,
                                            unsigned char *smem, doublex4 (&acc)[NB], bool active = true) {
    double *xs = reinterpret_cast<double *>(smem);                         // [2][64][kAppPad]
    float *vs = reinterpret_cast<float *>(xs + 2 * kAppTok * kAppPad);     // [2][NB*16][kAppPad]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool stager = tid < kThreads;
    const int b = u / a.groups, g = u % a.groups;
    const XT *x = static_cast<const XT *>(a.x);

    // staging map: thread -> (token, 4 consecutive columns) of a 64 x 16 chunk,
    // and (slot, 4 columns) of the NB*16 x 16 basis chunk
    const int st_tok = (tid & 255) >> 2, st_col = (tid & 3) * 4;
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

    auto load_chunk = [&](int kc) __attribute__((always_inline)) {
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
            const int slot = min(slot0 + rep * 64 + st_tok, a.kslots - 1);
            const float *q = a.basis + (static_cast<int64_t>(u) * a.kslots + slot) * a.dg + gd;
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[rep][i] = q[i];
        }
    };
    auto store_chunk = [&](int buf) __attribute__((always_inline)) {
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
                const bool keep = slot0 + slot < a.kslots;      // slots past kslots are zero
                float *vb = vs + (buf * NB * 16 + slot) * kAppPad + st_col;
#pragma unroll
                for (int i = 0; i < 4; ++i) vb[i] = keep ? vr[rep][i] : 0.0f;
            }
        }
    };

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = doublex4{0.0, 0.0, 0.0, 0.0};

    const int nchunks = a.dg / kAppKC;
    if (stager) {
        load_chunk(0);
        store_chunk(0);
    }
    __syncthreads();
    const int mrow = wave * 16 + (lane & 15);   // A operand row (token) of this lane
    const int kcol = lane >> 4;                 // A/B operand k of this lane
    for (int kc = 0; kc < nchunks; ++kc) {
        const int buf = kc & 1;
        if (stager && kc + 1 < nchunks) load_chunk(kc + 1);
        if (wave < 4 && active) {
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
        }
        if (stager && kc + 1 < nchunks) store_chunk(buf ^ 1);
        __syncthreads();
    }
}

// Quantisation and packing of f64_project's latents (block waves 0-3): every
// valid token's codes of slots [slot0, slot0 + 16 NB) below n_slots are OR-ed
// into its LDS bit row (rows [64][row_words]); in group-head mode the groups of
// those slots (whole groups: slot0 and 16 NB multiples of the group size, or
// slot0 = 0 with every slot) get their fp16 (min, scale), written to the
// params store.
template <bool MIXED, int NB>
__device__ __forceinline__ void f64_quantise(const AppendArgs &a, int u, int64_t t0, int nvalid, int slot0,
                                             const doublex4 (&acc)[NB], uint32_t *rows) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave >= 4) return;
    const int n_slots = a.ui[u].n_slots;
    const int row_words = a.row_stride >> 2;
    const int tbase = wave * 16 + (lane >> 4);
    const int64_t ub = static_cast<int64_t>(u) * a.kslots;
    if constexpr (!MIXED) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int j = slot0 + nb * 16 + (lane & 15);
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
        const int g_lo = slot0 / a.gs;
        const int g_hi = (min(n_slots, slot0 + NB * 16) + a.gs - 1) / a.gs;
        for (int gi = g_lo; gi < g_hi; ++gi) {
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
                const int j = slot0 + nb * 16 + (lane & 15);
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
                const int j = slot0 + nb * 16 + (lane & 15);
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
}

}  // namespace kvtc
