// The weight-stationary fetch kernel (gfx950) for wide units: group-head
// caches whose units span several heads (PALU cache API page, "Design": one
// shared projection per group of heads, latent -> dequant -> reconstruct on
// every fetch), contractions of 128 to 256 slots over 512-column slices.
//
// The contraction [tokens x k] x [k x d] is the same as fetch_kernel's and is
// accumulated in the same order (bias first, then the k-steps in order), so
// both kernels give the same rows.  What differs is where the operands live.
// fetch_kernel keeps a 128-column W slice in LDS and has each wave decode
// every k-step of its own tiles: per 32 x 32 product one W read from LDS and,
// per 128 columns, a full decode of the tile.  Here each of the block's eight
// waves holds the W rows of its own 64 output columns in registers for the
// whole block (8 VGPRs per k-step), the block decodes each tile's fetch
// operand once per 512 columns (each wave decodes one k-step in eight) into a
// double-buffered LDS array, and every wave multiplies the whole operand
// against its resident W rows, one LDS read per two products.
#pragma once

#include "kvtc_fetch_kernel.h"

namespace kvtc {

// One block: one (unit, slice of 32 NDBW NW columns, run of 32-token tiles).
// The tiles run through a software pipeline with one block barrier per tile:
// in the iteration of tile i every wave decodes its k-steps of tile i + 1 into
// one operand buffer, multiplies tile i's operand (the other buffer) into NDBW
// 32 x 32 fp32 accumulators seeded with the bias, rounds them to fp16 and
// stores its 32 NDBW columns of the tile's rows, then stashes tile i + 2's rows (loaded PF tiles
// earlier into a register ring) into the staging buffer tile i's rows leave
// free and requests the rows of tile i + 2 + PF.  MFMA operands: A = the
// wave's W rows (d), B = per-token fetch operand, C[d][token] in fp32.
template <bool MIXED, int KS, int NDBW, int RWB, int PF, bool PROBE = false>
__global__ __launch_bounds__(64 * kWsWaves, 4 / NDBW) void fetch_ws_kernel(FetchPair m) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = kWsWaves, NT = 64 * NW, CW = 32 * NDBW, DS = CW * NW;
    constexpr int DJ = (KS + NW - 1) / NW;          // k-steps each wave decodes
    static_assert(PF % 2 == 0, "ring depth keeps the buffer parity static");
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
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tok = lane & 31;
    const uint32_t half_k = lane >> 5;
    const int row_words = a.row_stride >> 2;
    const int d0 = slice * DS, dw = d0 + wave * CW;            // this wave's first column
    const int head = g * a.hpu + dw / a.D, ddw = dw % a.D;

    float *biasl = reinterpret_cast<float *>(smem + a.lds_bias);            // [DS]
    half8 *bbuf = reinterpret_cast<half8 *>(smem + a.lds_b);                // [2][KS][64]
    unsigned char *rstage = smem + a.lds_wave;                              // [2] x lds_rows
    uint32_t *dummy = reinterpret_cast<uint32_t *>(smem + a.lds_dummy) + tid;
    _Float16 *outl = reinterpret_cast<_Float16 *>(smem + a.lds_out) + wave * kFetTok * a.opitch;

    // this wave's W rows: lane (tok, half_k) holds W[dw + 32 db + tok][16 ks + 8 half_k + 0..7]
    half8 wa[NDBW][KS];
#pragma unroll
    for (int db = 0; db < NDBW; ++db) {
        const uint16_t *wrow =
            a.w16 + (static_cast<int64_t>(u) * a.dg + dw + db * 32 + tok) * a.kfetch + half_k * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            wa[db][ks] = !PROBE && ks < a.nks ? *reinterpret_cast<const half8 *>(wrow + ks * 16) : half8{};
    }
    for (int i = tid; i < DS; i += NT) biasl[i] = a.bias[static_cast<int64_t>(u) * a.dg + d0 + i];
    // the descriptors of the k-steps this wave decodes (wave, wave + NW, ...)
    uint32_t kdw[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int ks = wave + j * NW;
        kdw[j] = ks < a.nks ? __builtin_amdgcn_readfirstlane(a.kdesc[static_cast<int64_t>(u) * a.nks + ks]) : 0u;
    }

    const int tile_begin = chunk * a.tiles_per_block;
    const int n = min(a.ntiles, tile_begin + a.tiles_per_block) - tile_begin;   // >= 1
    const int lastl = n - 1;
    const int row_tile_words = kFetTok * row_words;
    const int tile_words = row_tile_words + (MIXED ? kFetTok * a.n_qg : 0);
    const int64_t ubase = static_cast<int64_t>(u) * a.capacity;
    const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(a.codes);

    // the rows (then parameters) of local tile lt: word i = k NT + tid of the
    // tile, every address clamped to the tile's valid part (words past the
    // valid rows repeat a valid word; they feed only token columns that are
    // not stored, and the words past the tile go to the thread's scratch word)
    auto fetch_rows = [&](int lt, uint32_t (&r)[RWB]) {
        const int64_t s = a.s_begin + static_cast<int64_t>(tile_begin + lt) * kFetTok;
        const int valid = static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
        const uint32_t *src = codes32 + (ubase + s) * row_words;
        const int vrow = valid * row_words;
#pragma unroll
        for (int k = 0; k < RWB; ++k) {
            const int i = k * NT + tid;
            if constexpr (MIXED) {
                const uint32_t *psrc = a.params + (ubase + s) * a.n_qg;
                const uint32_t *ra = src + min(i, vrow - 1);
                const uint32_t *pa = psrc + min(max(i - row_tile_words, 0), valid * a.n_qg - 1);
                r[k] = *(i < row_tile_words ? ra : pa);
            } else {
                r[k] = src[min(i, vrow - 1)];
            }
        }
    };
    // parameter word j of a tile is (token j / n_qg, group j % n_qg), staged
    // group-major so that a k-step's reads hit 32 banks
    auto stash_rows = [&](const uint32_t (&r)[RWB], int buf) {
        uint32_t *rows = reinterpret_cast<uint32_t *>(rstage + buf * a.lds_rows);
        uint32_t *par = reinterpret_cast<uint32_t *>(rstage + buf * a.lds_rows + a.lds_par);
#pragma unroll
        for (int k = 0; k < RWB; ++k) {
            const int i = k * NT + tid, j = i - row_tile_words;
            uint32_t *dst = i < row_tile_words ? rows + i : dummy;
            if constexpr (MIXED) {
                const int t = static_cast<int>((static_cast<float>(j) + 0.5f) * a.nqg_inv);
                if (i >= row_tile_words && i < tile_words) dst = par + (j - t * a.n_qg) * kFetTok + t;
            }
            *dst = r[k];
        }
    };
    // this wave's k-steps of the tile in staging buffer buf, into operand buffer ob
    auto decode = [&](int buf, int ob) {
        if constexpr (PROBE) return;
        const uint32_t *rows = reinterpret_cast<const uint32_t *>(rstage + buf * a.lds_rows);
        const uint32_t *par = reinterpret_cast<const uint32_t *>(rstage + buf * a.lds_rows + a.lds_par);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            const int ks = wave + j * NW;
            if (ks >= KS) continue;                                       // wave-uniform
            // an empty k-step (past this tensor's own count in a shared launch)
            // contributes exact zeros
            bbuf[(ob * KS + ks) * 64 + lane] =
                ((kdw[j] >> 16) & 0xFu) == 0u
                    ? half8{}
                    : decode_kstep<MIXED>(kdw[j], rows + tok * row_words, MIXED ? par + tok : nullptr, half_k);
        }
    };
    // tile lt's product from operand buffer ob, rounded and stored
    auto product = [&](int lt, int ob, auto full) {
        constexpr bool kFull = decltype(full)::value;
        const int64_t s = a.s_begin + static_cast<int64_t>(tile_begin + lt) * kFetTok;
        const int valid = kFull ? kFetTok : static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
        floatx16 acc[NDBW];
        seed_bias<NDBW>(acc, biasl + wave * CW, half_k);
        const half8 *bb = bbuf + ob * KS * 64 + lane;
        if constexpr (!PROBE) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const half8 bv = bb[ks * 64];
#pragma unroll
                for (int db = 0; db < NDBW; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[db][ks], bv, acc[db], 0, 0, 0);
            }
        }
        _Float16 *orow = a.out + b * a.osb + head * a.osh + (s - a.s_begin) * a.oss + ddw;
        store_tile<NDBW, kFull>(acc, outl, a.opitch, lane, orow, a.oss, valid);
    };

    // prologue: tiles 0 and 1 staged, tile 0 decoded, the ring holding tiles
    // 2 .. PF + 1 (clamped to the last tile; clamped copies are never stored)
    uint32_t ring[PF][RWB];
    {
        uint32_t r0[RWB];
        fetch_rows(0, r0);
        stash_rows(r0, 0);
        fetch_rows(min(1, lastl), r0);
        stash_rows(r0, 1);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch_rows(min(2 + p, lastl), ring[p]);
    __syncthreads();
    decode(0, 0);
    __syncthreads();

    // iteration i: staging buffer (i + 1) & 1 holds tile i + 1, operand buffer
    // i & 1 tile i; ring slot i % PF holds tile i + 2
    auto iteration = [&](int i, auto full, auto slot) {
        constexpr int P = decltype(slot)::value, PAR = P & 1;   // i % PF == P, i & 1 == PAR
        decode(PAR ^ 1, PAR ^ 1);
        product(i, PAR, full);
        stash_rows(ring[P], PAR);
        fetch_rows(min(i + 2 + PF, lastl), ring[P]);
        __syncthreads();
    };
    const bool ragged = a.s_begin + static_cast<int64_t>(tile_begin + n) * kFetTok > a.s_end;
    const int nfull = ragged ? n - 1 : n;
    int base = 0;
    for (; base + PF <= nfull; base += PF) {
        iteration(base + 0, std::true_type{}, std::integral_constant<int, 0>{});
        iteration(base + 1, std::true_type{}, std::integral_constant<int, 1>{});
        if constexpr (PF == 4) {
            iteration(base + 2, std::true_type{}, std::integral_constant<int, 2>{});
            iteration(base + 3, std::true_type{}, std::integral_constant<int, 3>{});
        }
    }
    // the last partial round (block-uniform conditions)
    if (base + 0 < n) iteration(base + 0, std::false_type{}, std::integral_constant<int, 0>{});
    if (base + 1 < n) iteration(base + 1, std::false_type{}, std::integral_constant<int, 1>{});
    if constexpr (PF == 4) {
        if (base + 2 < n) iteration(base + 2, std::false_type{}, std::integral_constant<int, 2>{});
        if (base + 3 < n) iteration(base + 3, std::false_type{}, std::integral_constant<int, 3>{});
    }
}

template <bool MIXED, int KS, int NDBW, int RWB>
int32_t launch_fetch_ws_rwb(FetchPair m, int nt, hipStream_t stream) {
    constexpr int DS = fetch_ws_cols(NDBW);
    size_t lds = 0;
    for (int i = 0; i < nt; ++i) {
        FetchArgs &a = m.t[i];
        if (a.dg % DS != 0 || a.nslices * DS != a.dg || a.D % (32 * NDBW) != 0) return KVTC_E_SHAPE;
        if (fetch_ws_rwb(kFetTok * (a.row_stride / 4 + (MIXED ? a.n_qg : 0))) > RWB) return KVTC_E_SHAPE;
        lds = std::max(lds, fetch_ws_lds_plan(a, MIXED, KS, NDBW));
    }
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    const int64_t grid = m.nblocks_per_xcd * 8;
    auto kern = fetch_ws_kernel<MIXED, KS, NDBW, RWB, 2>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * kWsWaves), lds, stream, m);
    return hipGetLastError() == hipSuccess ? KVTC_OK : KVTC_E_DEVICE;
}

// Group-head contractions of 8 to 16 k-steps over 512-column blocks, tiles of
// at most 1536 row and parameter words (three per thread).
template <int KS>
int32_t launch_fetch_ws(const FetchPair &m, int nt, int tile_words, hipStream_t stream) {
    if constexpr (KS < 8) {
        return KVTC_E_SHAPE;
    } else {
        const int rwb = fetch_ws_rwb(tile_words);
        if (rwb <= 2) return launch_fetch_ws_rwb<true, KS, 2, 2>(m, nt, stream);
        if (rwb <= 3) return launch_fetch_ws_rwb<true, KS, 2, 3>(m, nt, stream);
        return KVTC_E_SHAPE;
    }
}

}  // namespace kvtc
