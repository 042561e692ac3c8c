// Traffic probe of the fetch (gfx950): a measurement kernel, not part of the
// method.  It runs the fetch's blocks with the fetch's memory traffic -- the W
// slice and the bias read once per block, the code rows (and group-head
// params) of every tile read, every output row of every tile written with
// 16-byte non-temporal stores of whole rows -- with the fetch's register ring
// (the same number of tiles' rows in flight per wave), and nothing else: no
// decode, no contraction, no LDS staging (it requests the fetch's LDS only to
// share CUs as the fetch does).  Its rate is the
// practical ceiling of the fetch's traffic on this memory system, against
// which the fetch kernel is measured.  What it writes is not a reconstruction.
#include "kvtc_fetch_ws.h"

namespace kvtc {
namespace {

template <int DS, int NW, bool MIXED, int RW, int PF>
__global__ __launch_bounds__(64 * NW) void fetch_probe_kernel(FetchPair m) {
    constexpr int NT = 64 * NW;
    constexpr int kChunks = DS / 8;                   // 16-byte chunks per output row of the slice
    const int64_t bid = blockIdx.x;
    int64_t logical = (bid & 7) * m.nblocks_per_xcd + (bid >> 3);
    if (logical >= m.nblocks_real) return;
    const bool second = logical >= m.split;
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_words = a.row_stride >> 2;

    uint32_t acc = 0u;
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.w16 + (static_cast<int64_t>(u) * a.dg + d0) * a.kfetch);
        for (int i = tid; i < DS * a.kfetch / 8; i += NT) {
            const u32x4 v = src[i];
            acc ^= (v[0] ^ v[1]) ^ (v[2] ^ v[3]);
        }
        const uint32_t *bs = reinterpret_cast<const uint32_t *>(a.bias) + static_cast<int64_t>(u) * a.dg + d0;
        for (int i = tid; i < DS; i += NT) acc ^= bs[i];
    }
    const int tile_begin = chunk * a.tiles_per_block;
    const int tile_end = min(a.ntiles, tile_begin + a.tiles_per_block);
    const int64_t ubase = static_cast<int64_t>(u) * a.capacity;
    const uint32_t *codes32 = reinterpret_cast<const uint32_t *>(a.codes);
    const int row_tile_words = kFetTok * row_words;
    // a tile's rows (then params) into RW words per lane, addresses clamped to
    // the tile's valid words (no branch between a load and its use), as the
    // fetch kernel's ring loads them
    auto fetch_tile = [&](int tile, uint32_t (&r)[RW]) {
        const int64_t s = a.s_begin + static_cast<int64_t>(tile) * kFetTok;
        const int valid = static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
        const uint32_t *src = codes32 + (ubase + s) * row_words;
        const int vrow = max(valid * row_words, 1);
        if constexpr (MIXED) {
            const uint32_t *psrc = a.params + (ubase + s) * a.n_qg;
            const int vpar = max(valid * a.n_qg, 1);
#pragma unroll
            for (int k = 0; k < RW; ++k) {
                const int i = k * 64 + lane;
                r[k] = i < row_tile_words ? src[min(i, vrow - 1)] : psrc[min(i - row_tile_words, vpar - 1)];
            }
        } else {
#pragma unroll
            for (int k = 0; k < RW; ++k) r[k] = src[min(k * 64 + lane, vrow - 1)];
        }
    };
    // wave w takes tiles w, w + NW, ...; the rows of the next PF of them are in flight
    const int t0 = tile_begin + wave;
    uint32_t ring[PF][RW];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (t0 + p * NW < tile_end) fetch_tile(t0 + p * NW, ring[p]);
    _Float16 *last = nullptr;
    for (int tile = t0; tile < tile_end; tile += PF * NW) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int tt = tile + p * NW;
            if (tt >= tile_end) break;
#pragma unroll
            for (int k = 0; k < RW; ++k) acc ^= ring[p][k];
            if (tt + PF * NW < tile_end) fetch_tile(tt + PF * NW, ring[p]);
            const int64_t s = a.s_begin + static_cast<int64_t>(tt) * kFetTok;
            const int valid = static_cast<int>(min<int64_t>(kFetTok, a.s_end - s));
            _Float16 *orow = a.out + b * a.osb + head * a.osh + (s - a.s_begin) * a.oss + dd0;
            const u32x4 val = {static_cast<uint32_t>(tt), static_cast<uint32_t>(lane), 0u, 0u};
            for (int idx = lane; idx < valid * kChunks; idx += 64) {
                const int t = idx / kChunks, c = idx - t * kChunks;
                __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(orow + t * a.oss + c * 8));
            }
            last = orow;
        }
    }
    // the loaded words end up in one word of the wave's last tile, so no load is
    // dead (masked to two finite fp16 values)
    if (last && lane == 0) *reinterpret_cast<uint32_t *>(last) = acc & 0x03FF03FFu;
}

// lds: the fetch kernel's dynamic LDS for the same launch, requested (and left
// unused) so that as many probe blocks share a CU as fetch blocks would
template <int DS, int NW, int RW>
int32_t launch_probe_dn(const FetchPair &m, bool mixed, size_t lds, hipStream_t stream) {
    const int64_t grid = m.nblocks_per_xcd * 8;
    // the fetch kernel's ring depth for these rows
    auto kern = mixed ? fetch_probe_kernel<DS, NW, true, RW, (RW <= 8 ? 2 : 1)>
                      : fetch_probe_kernel<DS, NW, false, RW, (RW <= 8 ? 3 : (RW <= 16 ? 2 : 1))>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * NW), lds, stream, m);
    return launch_status();
}

template <int RW>
int32_t launch_probe_rw(const FetchPair &m, int ds, int nw, bool mixed, size_t lds, hipStream_t stream) {
    if (ds == 128)
        return nw == 8 ? launch_probe_dn<128, 8, RW>(m, mixed, lds, stream)
                       : launch_probe_dn<128, 4, RW>(m, mixed, lds, stream);
    if (ds == 64) return launch_probe_dn<64, 4, RW>(m, mixed, lds, stream);
    return KVTC_E_SHAPE;
}

}  // namespace

// The weight-stationary kernel's probe is that kernel with its arithmetic
// compiled out: the same blocks, staging, barriers and stores (of the bias).
int32_t launch_fetch_ws_probe(FetchPair m, int nt, int ks, int ndbw, int tile_words, hipStream_t stream) {
    if (ndbw != 2) return KVTC_E_SHAPE;
    size_t lds = 0;
    for (int i = 0; i < nt; ++i) lds = std::max(lds, fetch_ws_lds_plan(m.t[i], true, ks, ndbw));
    lds = std::max(lds, fetch_ws_w_staging(ks));        // as the kernel requests, for the same occupancy
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    const int rwb = fetch_ws_rwb(tile_words);
    if (rwb > 3) return KVTC_E_SHAPE;
    auto kern = rwb <= 2 ? fetch_ws_kernel<true, 16, 2, 2, true> : fetch_ws_kernel<true, 16, 2, 3, true>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(m.nblocks_per_xcd * 8)), dim3(64 * kWsWaves), lds, stream, m);
    return launch_status();
}

int32_t launch_fetch_probe(const FetchPair &m, int ds, int nw, bool mixed, int rw, size_t lds, hipStream_t stream) {
    switch (rw) {
        case 8: return launch_probe_rw<8>(m, ds, nw, mixed, lds, stream);
        case 16: return launch_probe_rw<16>(m, ds, nw, mixed, lds, stream);
        case 24: return launch_probe_rw<24>(m, ds, nw, mixed, lds, stream);
        default: return KVTC_E_SHAPE;
    }
}

}  // namespace kvtc
