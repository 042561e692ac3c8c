// Internal helpers shared by the host and device halves of libkvtc:
// state-blob access and validation.  Not part of the public interface.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

#include "kvtc.h"

namespace kvtc {

constexpr int kSlotAlign = 16;          // slots per unit are padded to a multiple of this
constexpr int kSectionAlign = 256;      // blob sections start on this boundary
constexpr uint32_t kOffsetMask = 0xFFFFFFu;
constexpr int kKStep = 16;              // slots per fetch k-step (one MFMA K); one width each

// Order in which the fetch kernel's 4-bit unpack delivers the 8 fields of one
// operand half (even nibbles first, then odd ones); W rows are stored to match.
constexpr int kNibbleOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};
// Fetch-operand column c of a 2-bit k-step holds the field of slot
// kTwoBitOrder[c]: masking the k-step's 32-bit window with 0x03030303 after
// shifts of 0, 2 (lanes of the lower operand half) and 4, 6 (upper half)
// yields the codes of these slots one per byte.  The map is its own inverse.
constexpr int kTwoBitOrder[16] = {0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15};

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

template <typename T>
inline const T *section(const void *blob, uint64_t off) {
    return reinterpret_cast<const T *>(static_cast<const char *>(blob) + off);
}
template <typename T>
inline T *section_mut(void *blob, uint64_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(blob) + off);
}

// Validates the header of a host copy of a state blob: magic, version, mode,
// shape fields, every section's extent inside total_bytes, and the per-unit
// counts.  The blob must hold at least total_bytes readable bytes (the caller
// passes no length; the Python binding checks it).  Returns KVTC_OK, KVTC_E_ARG
// for a NULL blob or KVTC_E_STATE; on success *out points at the header.
inline int32_t check_state(const void *blob, const kvtc_state_header **out) {
    if (blob == nullptr) return KVTC_E_ARG;
    const auto *h = static_cast<const kvtc_state_header *>(blob);
    if (h->magic != KVTC_MAGIC || h->version != KVTC_VERSION) return KVTC_E_STATE;
    if (h->mode != KVTC_MODE_DP && h->mode != KVTC_MODE_MIXED) return KVTC_E_STATE;
    if (h->head_dim <= 0 || h->heads_per_unit <= 0 || h->dg != h->head_dim * h->heads_per_unit)
        return KVTC_E_STATE;
    if (h->batch <= 0 || h->heads <= 0 || h->heads % h->heads_per_unit != 0 ||
        h->units != h->batch * (h->heads / h->heads_per_unit))
        return KVTC_E_STATE;
    if (h->rmax <= 0 || h->rmax > h->dg || h->kslots < kSlotAlign || h->kslots % kSlotAlign != 0 ||
        h->row_stride < 0 || h->row_stride % 4 != 0 || h->kfetch < kSlotAlign ||
        h->kfetch % kSlotAlign != 0)
        return KVTC_E_STATE;
    if (h->mode == KVTC_MODE_MIXED && (h->n_qgroups <= 0 || h->group_size <= 0)) return KVTC_E_STATE;
    if (h->dg > 65536 || h->kslots > 65536 || h->kfetch > 65536 || h->row_stride > 65536 ||
        h->units > (int64_t(1) << 31))
        return KVTC_E_STATE;
    // every section lies inside the blob: its start and its end, the size
    // recomputed from the header fields (no product below can overflow 64 bits
    // with the caps above)
    const uint64_t U = static_cast<uint64_t>(h->units), dg = h->dg, rmax = h->rmax, ks = h->kslots,
                   kf = h->kfetch;
    const struct {
        uint64_t off, bytes;
    } secs[] = {{h->off_unit, U * sizeof(kvtc_unit_info)},
                {h->off_lambda, U * dg * 8},
                {h->off_bits, U * rmax},
                {h->off_qmin, U * rmax * 4},
                {h->off_qscale, U * rmax * 4},
                {h->off_mu, U * dg * 4},
                {h->off_slot_comp, U * ks * 4},
                {h->off_slot_bits, U * ks * 4},
                {h->off_basis, U * ks * dg * 4},
                {h->off_qlo, U * ks * 8},
                {h->off_qinv, U * ks * 8},
                {h->off_w16, U * kf * dg * 2},
                {h->off_bias, U * dg * 4},
                {h->off_kdesc, U * (kf / kSlotAlign) * 4},
                {h->off_fslot, U * kf * 4}};
    for (const auto &s : secs)
        if (s.off < sizeof(kvtc_state_header) || s.off % kSectionAlign != 0 || s.off >= h->total_bytes ||
            s.bytes > h->total_bytes - s.off)
            return KVTC_E_STATE;
    // the int8 append's sections: both present or both absent
    if ((h->off_vdig == 0) != (h->off_mv == 0)) return KVTC_E_STATE;
    if (h->off_vdig) {
        const struct {
            uint64_t off, bytes;
        } opt[] = {{h->off_vdig, U * 5 * ks * dg}, {h->off_mv, U * ks * 8}};
        for (const auto &s : opt)
            if (s.off < sizeof(kvtc_state_header) || s.off % kSectionAlign != 0 || s.off >= h->total_bytes ||
                s.bytes > h->total_bytes - s.off)
                return KVTC_E_STATE;
    }
    // per-unit counts within the header's capacities (the kernels index the
    // slot arrays with them)
    const auto *ui = reinterpret_cast<const kvtc_unit_info *>(static_cast<const char *>(blob) + h->off_unit);
    for (uint64_t u = 0; u < U; ++u)
        if (ui[u].rank < 1 || ui[u].rank > h->rmax || ui[u].n_slots < 0 || ui[u].n_slots > h->kslots ||
            ui[u].n_slots > ui[u].rank || ui[u].row_bits < 0 || ui[u].row_bits > 8 * h->row_stride)
            return KVTC_E_STATE;
    if (out) *out = h;
    return KVTC_OK;
}

// ------------------------------------------------------------ device fit
// The device half of kvtc_fit_device (kvtc_fit.hip); the host half (eigen-
// decomposition, rank, allocation, blob) is kvtc_host.cpp's.  Plain types only:
// the host half is compiled without the HIP headers.
struct FitDeviceRows {
    const void *rows;          // device [B, H, S, D] of dtype, element strides sb, sh, ss (d stride 1)
    int32_t dtype;
    int64_t sb, sh, ss;
    int64_t B, H, S;
    int D, hpu, dg;
    int64_t units;
    int kslots;                // slot capacity of the range pass (multiple of 16, <= 256; 0: no ranges)
    void *work;                // device workspace, fit_device_layout(...).total bytes, 256-byte aligned
    void *stream;              // hipStream_t
};

struct FitDeviceLayout {
    uint64_t mpart, mean, cov, basis, mu32, ui, keys, total;
    int mchunks;               // row chunks of the mean's partial sums
};

inline FitDeviceLayout fit_device_layout(int64_t U, int dg, int64_t S, int kslots) {
    FitDeviceLayout L{};
    int64_t mc = (S + 1023) / 1024;
    L.mchunks = static_cast<int>(mc < 1 ? 1 : (mc > 64 ? 64 : mc));
    const uint64_t u = static_cast<uint64_t>(U), d = static_cast<uint64_t>(dg), k = static_cast<uint64_t>(kslots);
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = o;
        o = align_up(o + (bytes ? bytes : 1), kSectionAlign);
        return at;
    };
    L.mpart = take(u * L.mchunks * d * 8);
    L.mean = take(u * d * 8);
    L.cov = take(u * d * d * 8);
    L.basis = take(u * k * d * 4);
    L.mu32 = take(u * d * 4);
    L.ui = take(u * sizeof(kvtc_unit_info));
    L.keys = take(u * k * 16);
    L.total = o;
    return L;
}

// Mean [U][dg] and 1/S covariance [U][dg][dg] (float64, host memory) of every
// unit's rows; waits for the stream.  Returns a status.
int32_t fit_device_moments(const FitDeviceRows &r, double *mean_host, double *cov_host);
// Per-slot min and max [U][kslots] (host) of the latents (x - mu32) . basis_j of
// every row, in float64 (fp64 MFMA); basis_slots [U][kslots][dg] and mu32
// [U][dg] fp32 host arrays, n_slots [U]; waits for the stream.
int32_t fit_device_ranges(const FitDeviceRows &r, const float *mu32_host, const float *basis_slots_host,
                          const int32_t *n_slots_host, double *mn_host, double *mx_host);

// ------------------------------------------------------------ entropy-coded storage
// Layouts shared by the host half (kvtc_host.cpp: code lengths, canonical
// tables, index) and the device half (kvtc_entropy.hip: counts, archive).
constexpr int kEntropyChunk = 256;      // rows per decode chunk

struct EntropyIndexLayout {
    uint64_t off_unit, off_dec, off_syms, off_chunk, total;
};

inline EntropyIndexLayout entropy_index_layout(int64_t U, int kslots, int nsym, int nchunks) {
    EntropyIndexLayout L{};
    uint64_t o = align_up(sizeof(kvtc_entropy_header), kSectionAlign);
    auto take = [&](uint64_t bytes) {
        const uint64_t at = o;
        o = align_up(o + (bytes ? bytes : 1), kSectionAlign);
        return at;
    };
    const uint64_t u = static_cast<uint64_t>(U);
    L.off_unit = take(u * sizeof(kvtc_entropy_unit));
    L.off_dec = take(u * kslots * sizeof(kvtc_entropy_dec));
    L.off_syms = take(u * static_cast<uint64_t>(nsym));
    L.off_chunk = take(u * kslots * static_cast<uint64_t>(nchunks) * 8);
    L.total = o;
    return L;
}

// Device workspace of the encoder, sections 256-byte aligned.
struct EntropyWorkLayout {
    uint64_t sym_off, counts, enc_code, enc_len, units, slot_pos, chunk_bits, chunk_pos, total;
};

inline EntropyWorkLayout entropy_work_layout(int64_t U, int kslots, int nsym, int nchunks) {
    EntropyWorkLayout L{};
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = o;
        o = align_up(o + (bytes ? bytes : 1), kSectionAlign);
        return at;
    };
    const uint64_t u = static_cast<uint64_t>(U), k = static_cast<uint64_t>(kslots), n = static_cast<uint64_t>(nsym);
    L.sym_off = take(u * k * 4);
    L.counts = take(u * n * 4);
    L.enc_code = take(u * n * 4);
    L.enc_len = take(u * n);
    L.units = take(u * sizeof(kvtc_entropy_unit));
    L.slot_pos = take(u * k * 8);
    L.chunk_bits = take(u * k * static_cast<uint64_t>(nchunks) * 4);
    L.chunk_pos = take(u * k * static_cast<uint64_t>(nchunks) * 8);
    L.total = o;
    return L;
}

// What the device half of the encoder and decoder works on (device pointers).
struct EntropyDevArgs {
    const kvtc_unit_info *ui;          // state: per unit
    const uint32_t *sbits;             // state: [U][kslots] bit offset | width << 24
    uint8_t *codes;                    // code store [U][capacity][row_stride]
    int64_t capacity, S, units;
    int kslots, row_stride, nsym, nchunks;
    const uint32_t *sym_off;           // [U][kslots] first symbol position of each slot
    uint32_t *counts;                  // [U][nsym]
    const uint32_t *enc_code;          // [U][nsym] bit-reversed canonical codes
    const uint8_t *enc_len;            // [U][nsym] code lengths
    const kvtc_entropy_unit *unit;     // [U]
    const uint64_t *slot_pos;          // [U][kslots] archive bit position of each slot's stream
    uint32_t *chunk_bits;              // [U][kslots][nchunks]
    uint64_t *chunk_pos;               // [U][kslots][nchunks]
    const kvtc_entropy_dec *dec;       // [U][kslots]
    const uint8_t *syms;               // [U][nsym]
    uint32_t *archive;                 // 32-bit words
    uint64_t archive_words;
    void *stream;                      // hipStream_t
};

// Host -> device copy on the stream (enqueued).
int32_t fit_device_upload(void *dst_dev, const void *src_host, size_t bytes, void *stream);
// Code counts [U][nsym] of rows [0, S) into counts_host (waits for the stream).
int32_t entropy_device_counts(const EntropyDevArgs &a, uint32_t *counts_host);
// The archive from the uploaded tables; chunk positions into chunk_pos_host (waits).
int32_t entropy_device_encode(const EntropyDevArgs &a, const uint32_t *enc_code_host, const uint8_t *enc_len_host,
                              const kvtc_entropy_unit *units_host, const uint64_t *slot_pos_host,
                              uint64_t *chunk_pos_host);
// Rows [0, S) of the code store from the archive (enqueued only).
int32_t entropy_device_decode(const EntropyDevArgs &a);

}  // namespace kvtc
