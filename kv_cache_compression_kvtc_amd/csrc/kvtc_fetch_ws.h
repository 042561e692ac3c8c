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

// One lane's eight B-operand values of one k-step (the same values as
// decode_kstep) from three row words already in registers: r0, r1 at the word
// of the lane's first field and r2 after them.  Fields of 2, 4 and 8 bits take
// one branch-free path (each of the eight codes lands in a byte of x0:x1 in
// slot order), 1 and 3 bits the bit-by-bit one.  In group-head mode p is the
// row's (min, scale) word of the k-step's quantisation group.
template <bool MIXED>
__device__ __forceinline__ half8 decode_window(uint32_t kd, uint32_t sh, uint32_t r0, uint32_t r1, uint32_t r2,
                                               uint32_t p, uint32_t half_k) {
    const uint32_t w = (kd >> 16) & 0xFu;
    const uint32_t lo = __builtin_amdgcn_alignbit(r1, r0, sh);
    uint32_t pr[4];
    if (w == 1u) {
        small_fields<1>(lo, pr);
    } else if (w == 3u) {
        small_fields<3>(lo, pr);
    } else {
        // 8 bits: the window's eight bytes; 4 bits: nibbles stored 0,2,4,6,1,3,5,7
        // (even then odd nibbles); 2 bits: slots 0,4,8,12 / 1,5,9,13 of the
        // k-step's 32-bit window (2,6,10,14 / 3,7,11,15 in the upper half)
        const uint32_t hi = __builtin_amdgcn_alignbit(r2, r1, sh);
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
        const half2 cv = __builtin_bit_cast(half2, pr[e]) -
                         half2{static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
        if constexpr (MIXED) {
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

// One block: one (unit, slice of 32 NDBW NW columns, run of 32-token tiles).
// The tiles run through a software pipeline with one block barrier per tile.
// In the iteration of tile i every wave
//   - stashes tile i + 2's rows (loaded two tiles earlier into a register ring)
//     into the staging buffer tile i's rows leave free and requests the rows of
//     tile i + 4,
//   - multiplies tile i's operand (one operand buffer) into NDBW 32 x 32 fp32
//     accumulators seeded with the bias, and in between the MFMAs decodes its
//     k-steps of tile i + 1 into the other operand buffer and sends the
//     previous tile's rounded rows (staged in its LDS) to memory in 16-byte
//     passes, so that decode and stores run under the MFMAs,
//   - rounds tile i to fp16 into its staging.
// MFMA operands: A = the wave's W rows (d), B = per-token fetch operand,
// C[d][token] in fp32.
template <bool MIXED, int KS, int NDBW, int RWB, bool PROBE = false>
__global__ __launch_bounds__(64 * kWsWaves, 4 / NDBW) void fetch_ws_kernel(FetchPair m) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = kWsWaves, NT = 64 * NW, CW = 32 * NDBW, DS = CW * NW, PF = 2;
    constexpr int DJ = (KS + NW - 1) / NW;          // k-steps each wave decodes
    constexpr int CPR = CW / 8, NPASS = kFetTok * CPR / 64;   // 16-byte chunks per staged row, passes
    constexpr int FS = KS / NPASS;                             // k-steps per store pass
    static_assert(FS >= 2, "at least two k-steps per store pass");
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
    _Float16 *outl = reinterpret_cast<_Float16 *>(smem + a.lds_out) + wave * kFetTok * a.opitch;
    half8 wa[NDBW][KS];                                 // this wave's W rows (filled in the prologue)


    // the k-steps this wave decodes (wave, wave + NW, ...): descriptor, and the
    // lane's row-word offset, bit shift and parameter index, the same for every tile
    uint32_t kdw[DJ], dec_off[DJ], dec_sh[DJ], dec_par[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int ks = wave + j * NW;
        const uint32_t kd =
            ks < a.nks ? __builtin_amdgcn_readfirstlane(a.kdesc[static_cast<int64_t>(u) * a.nks + ks]) : 0u;
        const uint32_t w = (kd >> 16) & 0xFu;
        const uint32_t off = (kd & 0xFFFFu) + (w == 2u ? 0u : (half_k << 3) * w);
        kdw[j] = kd;
        dec_off[j] = tok * row_words + (off >> 5);
        dec_sh[j] = off & 31u;
        dec_par[j] = (kd >> 20) * kFetTok + tok;
    }

    const int tile_begin = chunk * a.tiles_per_block;
    const int n = min(a.ntiles, tile_begin + a.tiles_per_block) - tile_begin;   // >= 1
    const int64_t s0 = a.s_begin + static_cast<int64_t>(tile_begin) * kFetTok;  // first row of the run
    const int valid_last = static_cast<int>(min<int64_t>(kFetTok, a.s_end - (s0 + (n - 1) * kFetTok)));
    const int row_tile_words = kFetTok * row_words;
    const int tile_words = row_tile_words + (MIXED ? kFetTok * a.n_qg : 0);
    const int64_t ubase = static_cast<int64_t>(u) * a.capacity;
    const uint32_t *rbase = reinterpret_cast<const uint32_t *>(a.codes) + (ubase + s0) * row_words;
    const uint32_t *pbase = MIXED ? a.params + (ubase + s0) * a.n_qg : nullptr;

    // word i = k NT + tid of a tile: a row word (i < row_tile_words), a
    // parameter word, or past the tile (re-reads the tile's last parameter or
    // row word and goes to the thread's scratch word).  Per word: its offset
    // within the tile's rows or parameters, the words per token of that array
    // (for the clamp of a ragged last tile), and its byte offset in a staging
    // buffer (parameters group-major, so that a k-step's reads hit 32 banks).
    int ld_off[RWB], ld_unit[RWB], st_off[RWB];
    bool ld_row[RWB];
#pragma unroll
    for (int k = 0; k < RWB; ++k) {
        const int i = k * NT + tid;
        if (MIXED && i >= row_tile_words) {
            const int j = min(i - row_tile_words, kFetTok * a.n_qg - 1);
            const int t = j / a.n_qg;
            ld_row[k] = false;
            ld_off[k] = j;
            ld_unit[k] = a.n_qg;
            st_off[k] = i < tile_words ? a.lds_par + ((j - t * a.n_qg) * kFetTok + t) * 4 : a.lds_dummy + tid * 4;
        } else {
            ld_row[k] = true;
            ld_off[k] = min(i, row_tile_words - 1);
            ld_unit[k] = row_words;
            st_off[k] = i < row_tile_words ? i * 4 : a.lds_dummy + tid * 4;
        }
    }
    // the words of local tile lt (words past the valid rows of a ragged last
    // tile repeat a valid word: they feed only token columns that are not stored)
    const bool ragged = valid_last < kFetTok;
    auto fetch_rows = [&](int lt, uint32_t (&r)[RWB]) {
        const int valid = ragged && lt == n - 1 ? valid_last : kFetTok;
        const uint32_t *rt = rbase + static_cast<int64_t>(lt) * row_tile_words;
        const uint32_t *pt = MIXED ? pbase + static_cast<int64_t>(lt) * kFetTok * a.n_qg : nullptr;
#pragma unroll
        for (int k = 0; k < RWB; ++k) {
            const int o = min(ld_off[k], valid * ld_unit[k] - 1);
            r[k] = (ld_row[k] ? rt : pt)[o];
        }
    };
    auto stash_rows = [&](const uint32_t (&r)[RWB], int buf) {
#pragma unroll
        for (int k = 0; k < RWB; ++k) *reinterpret_cast<uint32_t *>(rstage + buf * a.lds_rows + st_off[k]) = r[k];
    };
    // this wave's k-steps of the tile in staging buffer buf: its row and
    // parameter words (dec_load), then each k-step's operand into operand buffer
    // ob (dec_emit); an empty k-step (past this tensor's own count in a shared
    // launch) contributes exact zeros
    uint32_t dr0[DJ], dr1[DJ], dr2[DJ], dpw[DJ];
    auto dec_load = [&](int buf) {
        const uint32_t *rows = reinterpret_cast<const uint32_t *>(rstage + buf * a.lds_rows);
        const uint32_t *par = reinterpret_cast<const uint32_t *>(rstage + buf * a.lds_rows + a.lds_par);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            if (wave + j * NW >= KS) continue;                            // wave-uniform
            dr0[j] = rows[dec_off[j]];
            dr1[j] = rows[dec_off[j] + 1];
            dr2[j] = rows[dec_off[j] + 2];
            dpw[j] = MIXED ? par[dec_par[j]] : 0u;
        }
    };
    auto dec_emit = [&](int j, int ob) {
        const int ks = wave + j * NW;
        if (ks >= KS) return;
        bbuf[(ob * KS + ks) * 64 + lane] =
            ((kdw[j] >> 16) & 0xFu) == 0u ? half8{}
                                          : decode_window<MIXED>(kdw[j], dec_sh[j], dr0[j], dr1[j], dr2[j], dpw[j], half_k);
    };

    // output: the wave's 32 x CW block of a tile, rounded to fp16 into its
    // staging (token-major), then written in NPASS passes of 16 bytes per lane
    // (chunk c of the tile: token c / CPR, 8 columns c % CPR)
    auto stage = [&](const floatx16 (&acc)[NDBW]) {
#pragma unroll
        for (int db = 0; db < NDBW; ++db)
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
                *reinterpret_cast<half4 *>(outl + tok * a.opitch + dl) = hv;
            }
    };
    auto out_row = [&](int lt) {
        return a.out + b * a.osb + head * a.osh + static_cast<int64_t>(tile_begin + lt) * kFetTok * a.oss + ddw;
    };
    auto flush = [&](_Float16 *orow, int k) {                             // one pass, whole tile
        const int idx = k * 64 + lane, t = idx / CPR, c = idx - t * CPR;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(outl + t * a.opitch + c * 8);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(orow + t * a.oss + c * 8));
    };
    auto flush_last = [&]() {                                            // the staged last tile, valid rows only
        _Float16 *orow = out_row(n - 1);
        const int valid = ragged ? valid_last : kFetTok;
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
            const int idx = k * 64 + lane, t = idx / CPR, c = idx - t * CPR;
            if (t < valid) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(outl + t * a.opitch + c * 8);
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(orow + t * a.oss + c * 8));
            }
        }
    };
    // (product and iteration are inlined: the accumulators and W rows they
    // reach by reference must stay in registers)
    // the product of the tile in operand buffer ob into acc (seeded with the
    // bias beforehand); in between its MFMAs, pinned to fixed k-steps, the next
    // tile is decoded from staging buffer dbuf into operand buffer dob (reads
    // after the first k-step, one k-step's operand after k-steps 3 and 7) and
    // the staged tile prev (a whole tile) is flushed when FLUSH.  B operands are
    // read two k-steps ahead, so the pinned work never waits on them.  Then this
    // tile is staged in prev's place and acc seeded again for the next tile.
    floatx16 acc[NDBW];
    auto product = [&](int ob, int dbuf, int dob, int prev, auto flush_prev) __attribute__((always_inline)) {
        const half8 *bb = bbuf + ob * KS * 64 + lane;
        _Float16 *orow = decltype(flush_prev)::value ? out_row(prev) : nullptr;
        half8 bq[3];
        if constexpr (!PROBE) {
            bq[0] = bb[0];
            bq[1] = bb[64];
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (!PROBE) {
                if (ks + 2 < KS) bq[(ks + 2) % 3] = bb[(ks + 2) * 64];
#pragma unroll
                for (int db = 0; db < NDBW; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[db][ks], bq[ks % 3], acc[db], 0, 0, 0);
                if (ks == 0) {
                    dec_load(dbuf);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int j = 0; j < DJ; ++j)
                    if (ks == 3 + 4 * j) {
                        dec_emit(j, dob);
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
            if constexpr (decltype(flush_prev)::value) {
                if (ks % FS == 1 && ks / FS < NPASS) {
                    flush(orow, ks / FS);
                    __builtin_amdgcn_sched_barrier(0);       // keep the pass between these k-steps
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        stage(acc);
        __builtin_amdgcn_wave_barrier();
        seed_bias<NDBW>(acc, biasl + wave * CW, half_k);
    };

    // prologue: tiles 0 and 1 staged, tile 0 decoded, the ring holding tiles
    // 2 and 3 (clamped to the last tile; clamped copies are never stored)
    static_assert(3 + 4 * (DJ - 1) < KS, "decode slots inside the product");
    // (the rows are requested first and stashed once the W staging is done)
    const int lastl = n - 1;
    uint32_t ring[PF][RWB], pre[2][RWB];
    fetch_rows(0, pre[0]);
    fetch_rows(min(1, lastl), pre[1]);
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch_rows(min(2 + p, lastl), ring[p]);
    // this wave's W rows: lane (tok, half_k) holds W[dw + 32 db + tok][16 ks + 8 half_k + 0..7].
    // Each 32-row block is read whole rows at a time (16 bytes per lane, two rows
    // of 16 KS slots per instruction, every cache line once) into the wave's own
    // LDS region, then gathered into that layout; k-steps past this tensor's
    // own count are zero.
    if constexpr (!PROBE) {
        constexpr int CH = 2 * KS;                      // 16-byte chunks per row
        constexpr int WP = CH * 16 + 16;                // row pitch of the staging (bytes)
        unsigned char *wst = smem + wave * 32 * WP;
#pragma unroll
        for (int db = 0; db < NDBW; ++db) {
            const uint16_t *wblk = a.w16 + (static_cast<int64_t>(u) * a.dg + dw + db * 32) * a.kfetch;
            u32x4 tmp[KS];
#pragma unroll
            for (int it = 0; it < KS; ++it) {
                const int c = it * 64 + lane, r = c / CH, ch = c - r * CH;
                tmp[it] = ch < 2 * a.nks ? *reinterpret_cast<const u32x4 *>(wblk + r * a.kfetch + ch * 8) : u32x4{};
            }
#pragma unroll
            for (int it = 0; it < KS; ++it) {
                const int c = it * 64 + lane, r = c / CH, ch = c - r * CH;
                *reinterpret_cast<u32x4 *>(wst + r * WP + ch * 16) = tmp[it];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                wa[db][ks] = *reinterpret_cast<const half8 *>(wst + tok * WP + (2 * ks + half_k) * 16);
            __builtin_amdgcn_wave_barrier();
        }
    } else {
#pragma unroll
        for (int db = 0; db < NDBW; ++db)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) wa[db][ks] = half8{};
    }
    __syncthreads();                                    // the W staging is reused from here on
    for (int i = tid; i < DS; i += NT) biasl[i] = a.bias[static_cast<int64_t>(u) * a.dg + d0 + i];
    stash_rows(pre[0], 0);
    stash_rows(pre[1], 1);
    __syncthreads();
    if constexpr (!PROBE) {
        dec_load(0);
#pragma unroll
        for (int j = 0; j < DJ; ++j) dec_emit(j, 0);
    }
    seed_bias<NDBW>(acc, biasl + wave * CW, half_k);
    __syncthreads();

    // iteration i: staging buffer (i + 1) & 1 holds tile i + 1, operand buffer
    // i & 1 tile i, the wave's output staging tile i - 1, ring slot i & 1 tile
    // i + 2.  The ring slot goes to staging buffer i & 1 (free: tile i was
    // decoded in the previous iteration) and is refilled with tile i + 4 before
    // the product, which decodes tile i + 1.
    auto iteration = [&](int i, auto parity, auto first) __attribute__((always_inline)) {
        constexpr int PAR = decltype(parity)::value;           // i & 1
        stash_rows(ring[PAR], PAR);
        fetch_rows(min(i + 2 + PF, lastl), ring[PAR]);
        product(PAR, PAR ^ 1, PAR ^ 1, i - 1, std::integral_constant<bool, !decltype(first)::value>{});
        __syncthreads();
    };
    iteration(0, std::integral_constant<int, 0>{}, std::true_type{});
    if (n > 1) {                                          // block-uniform
        iteration(1, std::integral_constant<int, 1>{}, std::false_type{});
        // ring slot 0 (requested a tile ago) is complete from here on, so the
        // loop's wait counts are those of its own body: without this they would
        // be sized for the entry from the first tile, which stores nothing, and
        // every other iteration would also wait for the previous tile's stores
        constexpr int kAfter = RWB + NPASS;              // slot 1's loads and tile 1's stores
        __builtin_amdgcn_s_waitcnt((kAfter & 0xF) | (0x7 << 4) | (0xF << 8) | ((kAfter >> 4) << 14));
        int i = 2;
        for (; i + 2 <= n; i += 2) {
            iteration(i, std::integral_constant<int, 0>{}, std::false_type{});
            iteration(i + 1, std::integral_constant<int, 1>{}, std::false_type{});
        }
        if (i < n) iteration(i, std::integral_constant<int, 0>{}, std::false_type{});
    }
    flush_last();
}

template <bool MIXED, int KS, int NDBW, int RWB>
int32_t launch_fetch_ws_rwb(FetchPair m, int nt, hipStream_t stream) {
    constexpr int DS = fetch_ws_cols(NDBW);
    size_t lds = 0;
    for (int i = 0; i < nt; ++i) {
        FetchArgs &a = m.t[i];
        if (a.dg % DS != 0 || a.nslices * DS != a.dg || a.D % (32 * NDBW) != 0) return KVTC_E_SHAPE;
        if (fetch_ws_rwb(kFetTok * (a.row_stride / 4 + (MIXED ? a.n_qg : 0))) > RWB) return KVTC_E_SHAPE;
        if (a.row_stride < 4 || (MIXED && a.n_qg < 1)) return KVTC_E_SHAPE;
        lds = std::max(lds, fetch_ws_lds_plan(a, MIXED, KS, NDBW));
    }
    lds = std::max(lds, fetch_ws_w_staging(KS));       // the prologue's W staging
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    const int64_t grid = m.nblocks_per_xcd * 8;
    auto kern = fetch_ws_kernel<MIXED, KS, NDBW, RWB>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * kWsWaves), lds, stream, m);
    return launch_status();
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
