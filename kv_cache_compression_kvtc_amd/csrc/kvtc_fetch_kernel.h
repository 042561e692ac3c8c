// The fetch kernel (gfx950) and its launch templates, instantiated per
// contraction length by kvtc_fetch_ks.hip.
//
// Fetch (KVTC cache module page, module docstring "Design": every call returns
// the whole sequence reconstructed to fp16; PALU cache API page, "Design":
// latent -> dequant -> reconstruct on every fetch): code rows stream from HBM
// into LDS, each lane extracts its fields, forms the fp16 contraction operand
// and the [tokens x slots] x [slots x d] product runs on fp16 MFMA with fp32
// accumulation; a bias is added, the result is rounded to fp16 and transposed
// through LDS into fully coalesced 16-byte non-temporal stores.
#pragma once

#include <type_traits>

#include "kvtc_device.h"

namespace kvtc {

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
template <bool MIXED, int NDB, int KS, int RW, int NW, int PF, int WS>
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

    // this lane's W rows (A operand: row db * 32 + tok, its k-half), one address
    // per 32-column block for the whole block: the per-k-step offsets are
    // constants (no pitch multiply or argument reload in the tile loop)
    const _Float16 *wrow[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) wrow[db] = wl + (db * 32 + tok) * a.wpitch + half_k * 8;

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
            const half8 bv = decode_kstep<MIXED, WS>(kd[ks], myrow, mypar, half_k);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const half8 av = *reinterpret_cast<const half8 *>(wrow[db] + ks * 16);
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
    // one round: the PF tiles from tile on, each stashed, its ring slot refilled
    // PF tiles ahead, then processed
    auto round = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int tt = tile + p * NW;
            stash_tile(ring[p]);
            fetch_tile(min(tt + PF * NW, last), ring[p]);
            process(tt, std::true_type{});
        }
    };
    // The first round is peeled: the loop is then entered only after a round
    // like its own body, so its waits are those of the steady state (each slot
    // waits for its own rows, requested PF tiles back).  Entered straight from
    // the prologue, the loads would be the youngest memory operations and the
    // waits would drain everything, the previous tiles' stores included.
    int tile = t0;
    if (tile + (PF - 1) * NW < full_end) {
        round(tile);
        tile += PF * NW;
        for (; tile + (PF - 1) * NW < full_end; tile += PF * NW) round(tile);
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

template <bool MIXED, int NDB, int KS, int RW>
int32_t launch_fetch_rw(FetchPair m, int nt, hipStream_t stream) {
    constexpr int DS = 32 * NDB, NW = fetch_waves<NDB, KS>();
    constexpr int NH = fetch_epilogue_blocks<NDB, NW>();
    static_assert(fetch_flat<MIXED, KS, RW, NW>() == fetch_flat_path(MIXED, KS, RW, NW), "flat path rule");
    size_t lds = 0;
    for (int i = 0; i < nt; ++i) {
        FetchArgs &a = m.t[i];
        if (kFetTok * (a.row_stride / 4 + (MIXED ? a.n_qg : 0)) > 64 * RW) return KVTC_E_SHAPE;
        lds = std::max(lds, fetch_lds_plan(a, MIXED, DS, NW, NH, RW, fetch_flat<MIXED, KS, RW, NW>()));
    }
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    const int64_t grid = m.nblocks_per_xcd * 8;
    constexpr int PF = fetch_prefetch<MIXED, RW>();
    auto kern = fetch_kernel<MIXED, NDB, KS, RW, NW, PF, kWidthsAll>;
    if constexpr (!MIXED)
        if (m.narrow) kern = fetch_kernel<MIXED, NDB, KS, RW, NW, PF, kWidths248>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * NW), lds, stream, m);
    return launch_status();
}

// Register staging of a tile's rows: the narrowest instantiated width that
// holds them (whole-head tiles: 8, 16 or 24 words per lane; 64-column: 8 or 24).
template <bool MIXED, int NDB, int KS>
int32_t launch_fetch_ks(const FetchPair &m, int nt, int rw, hipStream_t stream) {
    static_assert(fetch_rw_inst(NDB, 8) == 8 && fetch_rw_inst(NDB, 9) == (NDB == 4 ? 16 : 24), "rw rule");
    if (rw <= 8) return launch_fetch_rw<MIXED, NDB, KS, 8>(m, nt, stream);
    if (NDB == 4 && rw <= 16) return launch_fetch_rw<MIXED, NDB, KS, (NDB == 4 ? 16 : 24)>(m, nt, stream);
    if (rw <= kFetchRegWords) return launch_fetch_rw<MIXED, NDB, KS, kFetchRegWords>(m, nt, stream);
    return KVTC_E_SHAPE;
}

}  // namespace kvtc
