// Entropy-coded storage on the device (gfx950): the counts, the encoder and
// the chunk-parallel decoder of kvtc_entropy_encode / kvtc_entropy_decode.
//
// KVTC cache module page, "Byte accounting": the stored latents are order-0
// Huffman coded per kept component, with a fixed-width fallback.  The code
// lengths and canonical tables are built on the host from the counts computed
// here; the archive layout is the one kvtc.h documents.  Codes are emitted
// most significant bit first into an LSB-first bit stream, so a code of length
// L is written as its bit reversal; every write is an atomic OR into a 32-bit
// word of the zeroed archive, since neighbouring codes share words.  The
// decoder works per (unit, chunk of rows) in LDS and writes whole row words.
#include <vector>

#include "kvtc_device.h"

namespace kvtc {
namespace {

constexpr int kEntThreads = 256;
constexpr int kHistRows = 1024;          // rows per histogram block
constexpr int kHistLds = 16384;          // symbol positions a block counts in LDS

// The field of slot descriptor sb in a row (the next word is read only when
// the field runs into it, so it lies inside the row).
__device__ inline uint32_t field_of(const uint32_t *row, uint32_t sb) {
    const uint32_t off = sb & kOffsetMask, w = sb >> 24;
    const uint32_t wi = off >> 5, sh = off & 31u;
    uint32_t v = row[wi] >> sh;
    if (sh + w > 32u) v |= row[wi + 1] << (32u - sh);
    return v & ((1u << w) - 1u);
}

// bits [pos, pos + n) of the archive (n <= 32) OR-ed with v
__device__ inline void or_bits(uint32_t *arc, uint64_t pos, uint32_t v, int n) {
    if (n <= 0) return;
    const uint64_t x = static_cast<uint64_t>(v) << (pos & 31u);
    const uint64_t w = pos >> 5;
    atomicOr(arc + w, static_cast<uint32_t>(x));
    if ((pos & 31u) + static_cast<uint64_t>(n) > 32u) atomicOr(arc + w + 1, static_cast<uint32_t>(x >> 32));
}

// bits [pos, pos + n) of the archive (n <= 32); words past the archive's end
// (a corrupt index) read as zero
__device__ inline uint32_t read_bits(const uint32_t *arc, uint64_t nwords, uint64_t pos, int n) {
    const uint64_t w = pos >> 5;
    const uint32_t sh = pos & 31u;
    uint64_t x = w < nwords ? arc[w] : 0u;
    if (sh + static_cast<uint32_t>(n) > 32u && w + 1 < nwords) x |= static_cast<uint64_t>(arc[w + 1]) << 32;
    return static_cast<uint32_t>(x >> sh) & (n == 32 ? 0xFFFFFFFFu : ((1u << n) - 1u));
}

__global__ __launch_bounds__(kEntThreads) void fill_u32_kernel(uint32_t *p, uint64_t n) {
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kEntThreads + threadIdx.x; i < n;
         i += static_cast<uint64_t>(gridDim.x) * kEntThreads)
        p[i] = 0u;
}

// Counts of every (slot, code) of rows [1024 blockIdx.x, +1024) of one unit,
// in LDS when the unit's symbol positions fit, else straight to global memory.
__global__ __launch_bounds__(kEntThreads) void entropy_hist_kernel(EntropyDevArgs a) {
    __shared__ uint32_t h[kHistLds];
    const int u = blockIdx.y, tid = threadIdx.x;
    const bool in_lds = a.nsym <= kHistLds;
    if (in_lds)
        for (int i = tid; i < a.nsym; i += kEntThreads) h[i] = 0u;
    __syncthreads();
    const int ns = a.ui[u].n_slots, rw = a.row_stride >> 2;
    const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kHistRows;
    const int n = static_cast<int>(min<int64_t>(kHistRows, a.S - s0));
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(a.codes) + (static_cast<int64_t>(u) * a.capacity + s0) * rw;
    const uint32_t *sb = a.sbits + static_cast<int64_t>(u) * a.kslots;
    const uint32_t *so = a.sym_off + static_cast<int64_t>(u) * a.kslots;
    uint32_t *g = a.counts + static_cast<int64_t>(u) * a.nsym;
    for (int i = tid; i < n * ns; i += kEntThreads) {
        const int s = i / ns, j = i - s * ns;
        const uint32_t c = field_of(rows + static_cast<int64_t>(s) * rw, sb[j]);
        if (in_lds) atomicAdd(&h[so[j] + c], 1u);
        else atomicAdd(&g[so[j] + c], 1u);
    }
    __syncthreads();
    if (in_lds)
        for (int i = tid; i < a.nsym; i += kEntThreads)
            if (h[i]) atomicAdd(&g[i], h[i]);
}

// Coded bits of every (unit, slot, chunk): one thread per chunk.
__global__ __launch_bounds__(kEntThreads) void entropy_chunk_bits_kernel(EntropyDevArgs a) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x;
    const int64_t per_unit = static_cast<int64_t>(a.kslots) * a.nchunks;
    if (t >= a.units * per_unit) return;
    const int u = static_cast<int>(t / per_unit);
    const int j = static_cast<int>((t % per_unit) / a.nchunks), c = static_cast<int>(t % a.nchunks);
    uint32_t bits = 0;
    if (a.unit[u].coded && j < a.ui[u].n_slots) {
        const int rw = a.row_stride >> 2;
        const uint32_t sb = a.sbits[static_cast<int64_t>(u) * a.kslots + j];
        const uint8_t *len = a.enc_len + static_cast<int64_t>(u) * a.nsym + a.sym_off[static_cast<int64_t>(u) * a.kslots + j];
        const int64_t s1 = min(a.S, static_cast<int64_t>(c + 1) * kEntropyChunk);
        const uint32_t *rows = reinterpret_cast<const uint32_t *>(a.codes) + static_cast<int64_t>(u) * a.capacity * rw;
        for (int64_t s = static_cast<int64_t>(c) * kEntropyChunk; s < s1; ++s) bits += len[field_of(rows + s * rw, sb)];
    }
    a.chunk_bits[t] = bits;
}

// Archive bit position of each chunk: the slot's stream position plus the bits
// of the slot's earlier chunks.  One thread per (unit, slot).
__global__ __launch_bounds__(kEntThreads) void entropy_chunk_pos_kernel(EntropyDevArgs a) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x;
    if (t >= a.units * a.kslots) return;
    uint64_t p = a.slot_pos[t];
    for (int c = 0; c < a.nchunks; ++c) {
        a.chunk_pos[t * a.nchunks + c] = p;
        p += a.chunk_bits[t * a.nchunks + c];
    }
}

// One thread per (unit, slot, chunk) of a coded unit: the chunk's codes.
__global__ __launch_bounds__(kEntThreads) void entropy_encode_kernel(EntropyDevArgs a) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x;
    const int64_t per_unit = static_cast<int64_t>(a.kslots) * a.nchunks;
    if (t >= a.units * per_unit) return;
    const int u = static_cast<int>(t / per_unit);
    const int j = static_cast<int>((t % per_unit) / a.nchunks), c = static_cast<int>(t % a.nchunks);
    if (!a.unit[u].coded || j >= a.ui[u].n_slots) return;
    const int rw = a.row_stride >> 2;
    const uint32_t sb = a.sbits[static_cast<int64_t>(u) * a.kslots + j];
    const int64_t so = static_cast<int64_t>(u) * a.nsym + a.sym_off[static_cast<int64_t>(u) * a.kslots + j];
    const int64_t s1 = min(a.S, static_cast<int64_t>(c + 1) * kEntropyChunk);
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(a.codes) + static_cast<int64_t>(u) * a.capacity * rw;
    uint64_t pos = a.chunk_pos[t];
    for (int64_t s = static_cast<int64_t>(c) * kEntropyChunk; s < s1; ++s) {
        const uint32_t sym = field_of(rows + s * rw, sb);
        const int n = a.enc_len[so + sym];
        or_bits(a.archive, pos, a.enc_code[so + sym], n);
        pos += n;
    }
}

// The tables of the coded units (their code lengths, slot after slot, which is
// the unit's first table_bytes symbol positions) and the fixed-width parts:
// one thread per (unit, row) for the rows, per (unit, 4 table bytes) for tables.
__global__ __launch_bounds__(kEntThreads) void entropy_plain_kernel(EntropyDevArgs a) {
    const int u = blockIdx.y;
    const kvtc_entropy_unit un = a.unit[u];
    const uint64_t base = un.offset * 8;
    if (un.coded) {
        const uint8_t *len = a.enc_len + static_cast<int64_t>(u) * a.nsym;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x; i < un.table_bytes;
             i += static_cast<int64_t>(gridDim.x) * kEntThreads)
            or_bits(a.archive, base + 8 * i, len[i], 8);
        return;
    }
    const int rb = a.ui[u].row_bits, rw = a.row_stride >> 2;
    const uint32_t *rows = reinterpret_cast<const uint32_t *>(a.codes) + static_cast<int64_t>(u) * a.capacity * rw;
    for (int64_t s = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x; s < a.S;
         s += static_cast<int64_t>(gridDim.x) * kEntThreads) {
        const uint64_t pos = base + static_cast<uint64_t>(s) * rb;
        for (int k = 0; 32 * k < rb; ++k) or_bits(a.archive, pos + 32 * k, rows[s * rw + k], min(32, rb - 32 * k));
    }
}

// word w of the archive, zero past its end (a corrupt index)
__device__ inline uint32_t arc_word(const uint32_t *arc, uint64_t nwords, uint64_t w) { return w < nwords ? arc[w] : 0u; }

// Decoding state of one slot's stream in one chunk: a 64-bit window of the
// archive refilled one aligned word at a time.
struct BitWindow {
    uint64_t win, next;
    uint32_t nb;                                                        // valid bits in win
};

__device__ inline BitWindow window_at(const EntropyDevArgs &a, uint64_t pos) {
    BitWindow w;
    w.next = (pos >> 5) + 2;
    w.win = ((static_cast<uint64_t>(arc_word(a.archive, a.archive_words, w.next - 1)) << 32) |
             arc_word(a.archive, a.archive_words, w.next - 2)) >> (pos & 31u);
    w.nb = 64u - static_cast<uint32_t>(pos & 31u);
    return w;
}

// The next code of the stream, matched length by length against the slot's
// canonical table (a code that matches no length decodes to 0)
__device__ inline uint32_t next_symbol(const EntropyDevArgs &a, BitWindow &w, const kvtc_entropy_dec &d,
                                       const uint8_t *syms) {
    if (w.nb <= 32u) {                                                 // at least 33 bits before a code
        w.win |= static_cast<uint64_t>(arc_word(a.archive, a.archive_words, w.next++)) << w.nb;
        w.nb += 32u;
    }
    uint32_t v = 0;
    for (uint32_t L = 1; L <= d.max_len; ++L) {
        v = (v << 1) | static_cast<uint32_t>(w.win & 1u);
        w.win >>= 1;
        --w.nb;
        const uint32_t k = v - d.first[L];
        if (v >= d.first[L] && k < d.count[L]) return syms[d.base[L] + k];
    }
    return 0u;
}

// One block per (chunk of kEntropyChunk rows, unit) of a coded unit.  Thread j
// decodes slot j's codes of the chunk against the slot's canonical table,
// staged in LDS, and its symbol list, in LDS (SLDS) or global memory.  Fields
// are OR-ed into the chunk's rows in LDS (slots share row words); the block then
// writes every word of those rows once.  The decode is a serial chain per
// slot and chunk (each code's position follows from the previous code's
// length); two chunks per block with the chains interleaved measured slower
// (larger blocks, fewer resident).
template <bool SLDS>
__global__ __launch_bounds__(kEntThreads) void entropy_decode_kernel(EntropyDevArgs a) {
    extern __shared__ __align__(16) uint32_t sm[];
    const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
    if (!a.unit[u].coded) return;                                      // block-uniform
    const int64_t s0 = static_cast<int64_t>(c) * kEntropyChunk;
    const int n = static_cast<int>(min<int64_t>(kEntropyChunk, a.S - s0));
    const int ns = a.ui[u].n_slots, rw = a.row_stride >> 2;
    uint32_t *rows = sm;                                                // [kEntropyChunk][rw]
    kvtc_entropy_dec *dec = reinterpret_cast<kvtc_entropy_dec *>(sm + kEntropyChunk * rw);   // [ns]
    uint8_t *lsyms = reinterpret_cast<uint8_t *>(dec + a.kslots);                            // [nsym]
    constexpr int kDecWords = sizeof(kvtc_entropy_dec) / 4;
    const uint8_t *gsyms = a.syms + static_cast<int64_t>(u) * a.nsym;
    for (int i = tid; i < n * rw; i += kEntThreads) rows[i] = 0u;
    {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.dec + static_cast<int64_t>(u) * a.kslots);
        uint32_t *dst = reinterpret_cast<uint32_t *>(dec);
        for (int i = tid; i < ns * kDecWords; i += kEntThreads) dst[i] = src[i];
        if constexpr (SLDS)
            for (int i = tid; i < a.nsym; i += kEntThreads) lsyms[i] = gsyms[i];
    }
    __syncthreads();
    if (tid < ns) {
        const kvtc_entropy_dec &d = dec[tid];
        const uint8_t *sy = (SLDS ? lsyms : gsyms) + d.sym_off;
        const uint32_t sb = a.sbits[static_cast<int64_t>(u) * a.kslots + tid];
        const uint32_t off = sb & kOffsetMask, wi = off >> 5, sh = off & 31u;
        BitWindow w = window_at(a, a.chunk_pos[(static_cast<int64_t>(u) * a.kslots + tid) * a.nchunks + c]);
        for (int s = 0; s < n; ++s) {
            const uint64_t x = static_cast<uint64_t>(next_symbol(a, w, d, sy)) << sh;   // the field in row s
            atomicOr(rows + s * rw + wi, static_cast<uint32_t>(x));
            if ((x >> 32) != 0u) atomicOr(rows + s * rw + wi + 1, static_cast<uint32_t>(x >> 32));
        }
    }
    __syncthreads();
    uint32_t *out = reinterpret_cast<uint32_t *>(a.codes) + (static_cast<int64_t>(u) * a.capacity + s0) * rw;
    for (int i = tid; i < n * rw; i += kEntThreads) out[i] = rows[i];
}

template <bool SLDS>
int32_t launch_entropy_decode(const EntropyDevArgs &a, size_t lds, hipStream_t st) {
    auto kern = entropy_decode_kernel<SLDS>;
    if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.nchunks), static_cast<unsigned>(a.units)), dim3(kEntThreads),
                       lds, st, a);
    return launch_status();
}

// Fixed-width units: one thread per (unit, row) copies the row's bits back.
__global__ __launch_bounds__(kEntThreads) void entropy_unplain_kernel(EntropyDevArgs a) {
    const int u = blockIdx.y;
    const kvtc_entropy_unit un = a.unit[u];
    if (un.coded) return;
    const int rb = a.ui[u].row_bits, rw = a.row_stride >> 2;
    uint32_t *rows = reinterpret_cast<uint32_t *>(a.codes) + static_cast<int64_t>(u) * a.capacity * rw;
    for (int64_t s = static_cast<int64_t>(blockIdx.x) * kEntThreads + threadIdx.x; s < a.S;
         s += static_cast<int64_t>(gridDim.x) * kEntThreads) {
        const uint64_t pos = un.offset * 8 + static_cast<uint64_t>(s) * rb;
        for (int k = 0; k < rw; ++k) {
            const int n = min(32, rb - 32 * k);
            rows[s * rw + k] = n > 0 ? read_bits(a.archive, a.archive_words, pos + 32 * k, n) : 0u;
        }
    }
}

unsigned grid_for(int64_t n) { return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n + kEntThreads - 1) / kEntThreads, 1 << 20))); }

}  // namespace

int32_t fit_device_upload(void *dst_dev, const void *src_host, size_t bytes, void *stream) {
    return hipMemcpyAsync(dst_dev, src_host, bytes, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? KVTC_OK
               : KVTC_E_DEVICE;
}

int32_t entropy_device_counts(const EntropyDevArgs &a, uint32_t *counts_host) {
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    const uint64_t n = static_cast<uint64_t>(a.units) * a.nsym;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(static_cast<int64_t>(n))), dim3(kEntThreads), 0, st, a.counts, n);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    const int64_t blocks = (a.S + kHistRows - 1) / kHistRows;
    if (blocks > 0) {
        hipLaunchKernelGGL(entropy_hist_kernel, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(a.units)),
                           dim3(kEntThreads), 0, st, a);
        if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    }
    if (hipMemcpyAsync(counts_host, a.counts, n * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return KVTC_E_DEVICE;
    return KVTC_OK;
}

int32_t entropy_device_encode(const EntropyDevArgs &a, const uint32_t *enc_code_host, const uint8_t *enc_len_host,
                              const kvtc_entropy_unit *units_host, const uint64_t *slot_pos_host,
                              uint64_t *chunk_pos_host) {
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    const uint64_t U = static_cast<uint64_t>(a.units), n = U * a.nsym, nk = U * a.kslots;
    const uint64_t nc = nk * static_cast<uint64_t>(a.nchunks);
    if (hipMemcpyAsync(const_cast<uint32_t *>(a.enc_code), enc_code_host, n * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(const_cast<uint8_t *>(a.enc_len), enc_len_host, n, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(const_cast<kvtc_entropy_unit *>(a.unit), units_host, U * sizeof(kvtc_entropy_unit),
                       hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(const_cast<uint64_t *>(a.slot_pos), slot_pos_host, nk * 8, hipMemcpyHostToDevice, st) != hipSuccess)
        return KVTC_E_DEVICE;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(static_cast<int64_t>(a.archive_words))), dim3(kEntThreads), 0, st,
                       a.archive, a.archive_words);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(entropy_chunk_bits_kernel, dim3(grid_for(static_cast<int64_t>(nc))), dim3(kEntThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(entropy_chunk_pos_kernel, dim3(grid_for(static_cast<int64_t>(nk))), dim3(kEntThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    hipLaunchKernelGGL(entropy_encode_kernel, dim3(grid_for(static_cast<int64_t>(nc))), dim3(kEntThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    const unsigned gx = static_cast<unsigned>(std::min<int64_t>((a.S + kEntThreads - 1) / kEntThreads + 1, 4096));
    hipLaunchKernelGGL(entropy_plain_kernel, dim3(gx, static_cast<unsigned>(U)), dim3(kEntThreads), 0, st, a);
    if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
    if (hipMemcpyAsync(chunk_pos_host, a.chunk_pos, nc * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return KVTC_E_DEVICE;
    return KVTC_OK;
}

int32_t entropy_device_decode(const EntropyDevArgs &a) {
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    if (a.S == 0) return KVTC_OK;
    const uint64_t U = static_cast<uint64_t>(a.units);
    if (a.kslots > kEntThreads) return KVTC_E_SHAPE;
    // coded units: every word of rows [0, S) written by the decoder; fixed-width
    // units: by the copy below
    // the symbol lists in LDS where they fit next to the rows and tables, else
    // read from global memory (at most 64 KB of rows and 68 KB of tables: fits)
    const size_t rows1 = static_cast<size_t>(kEntropyChunk) * (a.row_stride / 4) * 4;
    const size_t tabs = static_cast<size_t>(a.kslots) * sizeof(kvtc_entropy_dec), syml = static_cast<size_t>(a.nsym);
    const int32_t rc = rows1 + tabs + syml <= kLdsMax ? launch_entropy_decode<true>(a, rows1 + tabs + syml, st)
                                                      : launch_entropy_decode<false>(a, rows1 + tabs, st);
    if (rc != KVTC_OK) return rc;
    const unsigned gr = static_cast<unsigned>(std::min<int64_t>((a.S + kEntThreads - 1) / kEntThreads, 4096));
    hipLaunchKernelGGL(entropy_unplain_kernel, dim3(gr, static_cast<unsigned>(U)), dim3(kEntThreads), 0, st, a);
    return launch_status();
}

}  // namespace kvtc
