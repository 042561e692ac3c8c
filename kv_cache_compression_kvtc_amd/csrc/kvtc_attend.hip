// Decode attention from the codes (gfx950): kvtc_attend and its kernels.
#include <mutex>
#include <type_traits>

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
constexpr int kAttSegMax = 9216;     // rows per partial block at most (their scores stay in LDS)
constexpr int kAttSeg = 256;         // rows per segment at least (unless the cache is shorter)
constexpr int kAttBlocks = 512;      // partial blocks worth filling the GPU with (two per CU)
constexpr int kAttWaves = 8;         // waves per partial block
constexpr int kAttPairs = 8;         // scorer products whose operands a lane keeps in registers
constexpr int kAttThreads = 64 * kAttWaves;
constexpr int kAttStage = 3;         // staged 16-byte chunks per thread and sub-chunk at most (24 KiB per block)
constexpr int kAttKsK = 16;          // k-steps of the key contraction (kfetch <= 256)
constexpr int kAttBatch = 16;        // basis loads in flight per lane (prologue and output)

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
    int nchunks, chunk_rows, H, D;     // segments of chunk_rows rows (the last one shorter), <= kAttSegMax
    int sub;                           // rows per staged sub-chunk: 64, 128 or 256 (the window fits the staging)
    float inv_sqrt_d;
    float *part;        // [U][nchunks][v.kslots + 2]: abar partial sums, then max, sum (two or more segments)
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// The sixteen codes of one k-step (16 fetch columns of width W; off: the
// k-step's first bit in the lane's row) of a row as int8 bytes in four
// registers: byte b of R[r] is the code of fetch column t = 4r + b of the
// k-step, whose field starts at bit pos(W, t) of the k-step's window, with
//   W = 8: 8t,  W = 4: 32(r >> 1) + 4(r & 1) + 8b,  W = 2: 8b + 2r,  W = 3: 3t,
//   W = 1: 4r + b,
// the bit positions the fetch kernel's decode gives its columns (so byte order
// and fetch order agree).  8-bit codes become c - 128 (c ^ 0x80 read as int8),
// which the callers correct for; narrower codes are their own values.  The
// window reads up to five words from the k-step's first word; words past the
// row's fields only reach padding columns.
template <int W>
__device__ __forceinline__ void kstep_bytes_w(uint32_t off, const uint32_t *row, uint32_t (&R)[4]) {
    const uint32_t wi = off >> 5, sh = off & 31u;
    if constexpr (W == 2) {
        const uint32_t x = __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = (x >> (2 * r)) & 0x03030303u;
    } else if constexpr (W == 4) {
        const uint32_t x0 = __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh);
        const uint32_t x1 = __builtin_amdgcn_alignbit(row[wi + 2], row[wi + 1], sh);
        R[0] = x0 & 0x0F0F0F0Fu;
        R[1] = (x0 >> 4) & 0x0F0F0F0Fu;
        R[2] = x1 & 0x0F0F0F0Fu;
        R[3] = (x1 >> 4) & 0x0F0F0F0Fu;
    } else if constexpr (W == 8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = __builtin_amdgcn_alignbit(row[wi + r + 1], row[wi + r], sh) ^ 0x80808080u;
    } else if constexpr (W == 1) {
        // nibble r spread over the four bytes: the shifted copies 0, 7, 14, 21 of a
        // 4-bit value never overlap, so the product has no carries
        const uint32_t x = __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = (((x >> (4 * r)) & 0xFu) * 0x00204081u) & 0x01010101u;
    } else if constexpr (W == 3) {
        const uint32_t x0 = __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh);
        const uint32_t x1 = __builtin_amdgcn_alignbit(row[wi + 2], row[wi + 1], sh);
        const uint32_t y = __builtin_amdgcn_alignbit(x1, x0, 16);      // window bits 16..47
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int t = 4 * r + b;
                const uint32_t f = t < 6 ? (x0 >> (3 * t)) & 7u : (y >> (3 * t - 16)) & 7u;
                v |= f << (8 * b);
            }
            R[r] = v;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = 0u;
    }
}

// 4x4 byte transpose inside each quad of lanes (lanes 4q..4q+3): lane 4q+n
// returns, as byte s, byte n of lane 4q+s's v.  Two butterfly stages, each a
// DPP exchange with the partner lane and a byte select (s1, s2: the lane's
// selectors from quad_selectors).
__device__ __forceinline__ void quad_selectors(uint32_t lane, uint32_t &s1, uint32_t &s2) {
    s1 = (lane & 1u) ? 0x03070105u : 0x06020400u;   // swaps lane bit 0 with byte bit 0
    s2 = (lane & 2u) ? 0x03020706u : 0x05040100u;   // swaps lane bit 1 with byte bit 1
}
__device__ __forceinline__ uint32_t quad_transpose(uint32_t v, uint32_t s1, uint32_t s2) {
    uint32_t p = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    v = __builtin_amdgcn_perm(p, v, s1);
    p = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    return __builtin_amdgcn_perm(p, v, s2);
}

// The value side's operands of one k-step for the 4x4x4 products: lane n of a
// quad ends with B[r] holding, as byte s, the code of fetch column 4r + n in
// the quad's row s (kstep_bytes_w's bytes, transposed across the quad).  For
// widths 2, 4 and 8 the raw window words are transposed first, which yields
// the same bytes with fewer transposes.
template <int W>
__device__ __forceinline__ void kstep_bytes_quad_w(uint32_t off, const uint32_t *row, uint32_t s1, uint32_t s2,
                                                   uint32_t (&B)[4]) {
    const uint32_t wi = off >> 5, sh = off & 31u;
    if constexpr (W == 2) {
        const uint32_t u0 = quad_transpose(__builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh), s1, s2);
#pragma unroll
        for (int r = 0; r < 4; ++r) B[r] = (u0 >> (2 * r)) & 0x03030303u;
    } else if constexpr (W == 4) {
        const uint32_t u0 = quad_transpose(__builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh), s1, s2);
        const uint32_t u1 = quad_transpose(__builtin_amdgcn_alignbit(row[wi + 2], row[wi + 1], sh), s1, s2);
        B[0] = u0 & 0x0F0F0F0Fu;
        B[1] = (u0 >> 4) & 0x0F0F0F0Fu;
        B[2] = u1 & 0x0F0F0F0Fu;
        B[3] = (u1 >> 4) & 0x0F0F0F0Fu;
    } else if constexpr (W == 8) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            B[r] = quad_transpose(__builtin_amdgcn_alignbit(row[wi + r + 1], row[wi + r], sh), s1, s2) ^ 0x80808080u;
    } else {
        uint32_t R[4];
        kstep_bytes_w<W>(off, row, R);
#pragma unroll
        for (int r = 0; r < 4; ++r) B[r] = quad_transpose(R[r], s1, s2);
    }
}

// One k-step's p-weighted sums over the sub-chunk's G groups of 64 rows (group
// g's digits of P in Ag[g], zero for rows past the chunk; its rows at
// row0 + g * 64 * row_words).
template <int W, int G>
__device__ __forceinline__ void value_kstep(i32x4 (&acc)[4], uint32_t off, const uint32_t *row0, int row_words,
                                            const uint32_t (&Ag)[G], uint32_t s1, uint32_t s2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t B[4];
        kstep_bytes_quad_w<W>(off, row0 + g * 64 * row_words, s1, s2, B);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            acc[rr] = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(Ag[g]), static_cast<int>(B[rr]), acc[rr], 0, 0, 0);
    }
}

// A k-step's score operand bytes for a width known only at run time (uniform),
// among the widths WS allows.
template <int WS>
__device__ __forceinline__ void kstep_bytes_any(uint32_t wid, uint32_t off, const uint32_t *row0, uint32_t (&R)[4]) {
    if constexpr (WS == kWidths248) {
        if (wid == 4u)
            kstep_bytes_w<4>(off, row0, R);
        else if (wid == 2u)
            kstep_bytes_w<2>(off, row0, R);
        else
            kstep_bytes_w<8>(off, row0, R);
    } else {
        if (wid == 2u)
            kstep_bytes_w<2>(off, row0, R);
        else if (wid == 4u)
            kstep_bytes_w<4>(off, row0, R);
        else if (wid == 8u)
            kstep_bytes_w<8>(off, row0, R);
        else if (wid == 1u)
            kstep_bytes_w<1>(off, row0, R);
        else
            kstep_bytes_w<3>(off, row0, R);
    }
}

// value_kstep for a run-time width among those WS allows (0: no k-step).
template <int WS, int G>
__device__ __forceinline__ void value_kstep_any(uint32_t wid, i32x4 (&acc)[4], uint32_t off, const uint32_t *row0,
                                                int row_words, const uint32_t (&Ag)[G], uint32_t s1, uint32_t s2) {
    if constexpr (WS == kWidths248) {
        if (wid == 4u)
            value_kstep<4, G>(acc, off, row0, row_words, Ag, s1, s2);
        else if (wid == 2u)
            value_kstep<2, G>(acc, off, row0, row_words, Ag, s1, s2);
        else if (wid == 8u)
            value_kstep<8, G>(acc, off, row0, row_words, Ag, s1, s2);
    } else {
        switch (wid) {
            case 2: value_kstep<2, G>(acc, off, row0, row_words, Ag, s1, s2); break;
            case 4: value_kstep<4, G>(acc, off, row0, row_words, Ag, s1, s2); break;
            case 8: value_kstep<8, G>(acc, off, row0, row_words, Ag, s1, s2); break;
            case 1: value_kstep<1, G>(acc, off, row0, row_words, Ag, s1, s2); break;
            case 3: value_kstep<3, G>(acc, off, row0, row_words, Ag, s1, s2); break;
            default: break;                                    // no such k-step
        }
    }
}

__device__ inline uint32_t row_field(const uint32_t *row, uint32_t sb) {
    const uint32_t off = sb & kOffsetMask, w = sb >> 24;
    const uint32_t wi = off >> 5, sh = off & 31u;
    return __builtin_amdgcn_alignbit(row[wi + 1], row[wi], sh) & ((1u << w) - 1u);
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

// Staging of a sub-chunk's code rows: its bytes are copied as the 16-byte
// chunks of the aligned window [a0, a0 + 16 nch) that covers them, chunk
// k * kAttThreads + tid per thread (every load issued, past the end clamped to the last
// chunk, so all are in flight before any is stored), into a linear LDS buffer:
// the sub-chunk's row r then starts at word delta + r * row_words.  The window
// lies in the pages of the rows it covers.
typedef const u32x4 __attribute__((address_space(1))) *GlobalChunks;   // global memory (not flat)

struct SubSrc {
    GlobalChunks src;
    int nch, delta;
};

__device__ inline SubSrc sub_src(const uint8_t *codes, int64_t row0, int nrows, int row_stride) {
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(codes) + static_cast<uintptr_t>(row0) * row_stride;
    const uintptr_t a0 = b0 & ~static_cast<uintptr_t>(15);
    SubSrc g;
    g.src = reinterpret_cast<GlobalChunks>(a0);
    g.delta = static_cast<int>((b0 - a0) >> 2);
    g.nch = static_cast<int>((b0 - a0 + static_cast<uintptr_t>(nrows) * row_stride + 15) >> 4);
    return g;
}

template <int ST>
__device__ inline void sub_load(const SubSrc &g, u32x4 (&r)[ST]) {
#pragma unroll
    for (int k = 0; k < ST; ++k)
        r[k] = g.src[min(k * kAttThreads + static_cast<int>(threadIdx.x), max(g.nch, 1) - 1)];
}

template <int ST>
__device__ inline void sub_store(const SubSrc &g, uint32_t *buf, const u32x4 (&r)[ST]) {
#pragma unroll
    for (int k = 0; k < ST; ++k) {
        const int i = k * kAttThreads + static_cast<int>(threadIdx.x);
        if (i < g.nch) reinterpret_cast<u32x4 *>(buf)[i] = r[k];
    }
}

// The wave's max or sum of v in every lane: quads and rows of 16 with DPP
// moves (neighbours, pairs, half-row and row mirrors), then the row pairs and
// halves of the wave swapped in.
__device__ inline float wave_reduce(float v, bool is_max) {
    auto op = [is_max](float x, float y) { return is_max ? fmaxf(x, y) : x + y; };
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
    v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
    v = op(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
    v = op(v, dpp(v, std::integral_constant<int, 0x140>{}));   // row_mirror
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

__device__ inline float block_reduce(float v, float *red, bool is_max) {
    v = wave_reduce(v, is_max);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// Per (segment of chunk_rows <= kAttSegMax rows, unit): scores from the key codes,
// the segment's softmax max and sum, and the p-weighted sums of the value
// codes, both contractions on int8 MFMA with exact int32 accumulation.  The
// key rows, then the value rows, stream through two LDS buffers of `sub` rows
// (linear copies of the rows' 16-byte-aligned windows, with slack words after
// the last row for its k-step windows): while one buffer is decoded, the next
// sub-chunk's chunks are in flight in registers.  The
// segment's scores stay in LDS, turned into weights once the keys are done.
template <int KW, int G, int WS, int ST>
__global__ __launch_bounds__(kAttThreads) void attend_partial_kernel(AttendArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
    const uint32_t lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AttendSide &K = a.k, &V = a.v;
    u32x4 *qal = reinterpret_cast<u32x4 *>(smem);                        // [kAttKsK][4] + 1 scorer operands
    float *red = reinterpret_cast<float *>(qal + kAttKsK * 4 + 1);      // [kAttWaves] block reductions
    float *ql = red + kAttWaves;                                         // [kMaxSlots] the query
    float *qts = ql + kMaxSlots;                                         // [kMaxSlots] qt_j, then abar_j
    float *mpt = qts + kMaxSlots;                                        // [kMaxSlots] min_j q.V_j
    uint32_t *kds = reinterpret_cast<uint32_t *>(mpt + kMaxSlots);      // [kAttKsK] key k-step descriptors
    uint32_t *ptab = kds + kAttKsK;                                      // [1 + 2 kAttKsK] scorer products
    uint32_t *plt = ptab + 1 + 2 * kAttKsK + 3;                          // [kAttPairs][64] lanes' product operands
    int *vfs = reinterpret_cast<int *>(plt + kAttPairs * 64);            // [kMaxSlots] value slot of each fetch column
    float *vsc = reinterpret_cast<float *>(vfs + kMaxSlots);            // [kMaxSlots] value scale of each slot
    float *pl = vsc + kMaxSlots;                                         // [chunk_rows, rounded up to sub] scores, then weights
    uint32_t *pw = reinterpret_cast<uint32_t *>(pl);                     //   as int8 digit words
    const int sub = a.sub, bw = (sub * max(K.row_words, V.row_words) + 16 + 3) & ~3;   // buffer words
    uint32_t *buf0 = reinterpret_cast<uint32_t *>(pl + (a.chunk_rows + sub - 1) / sub * sub);
    uint32_t *buf1 = buf0 + bw;
    const int64_t s0 = static_cast<int64_t>(c) * a.chunk_rows;
    const int nrows = static_cast<int>(min<int64_t>(a.chunk_rows, a.s_end - s0));
    const int nsub = (nrows + sub - 1) / sub;
    // step j < nsub stages key sub-chunk j, step nsub + j value sub-chunk j
    const uint8_t *kfirst = K.codes + (static_cast<int64_t>(u) * K.capacity + s0) * K.row_words * 4;
    const uint8_t *vfirst = V.codes + (static_cast<int64_t>(u) * V.capacity + s0) * V.row_words * 4;
    auto step_src = [&](int st) __attribute__((always_inline)) {
        const bool key = st < nsub;
        const int j = key ? st : st - nsub;
        const int rs = (key ? K.row_words : V.row_words) * 4;
        return sub_src(key ? kfirst : vfirst, static_cast<int64_t>(j) * sub, min(sub, nrows - j * sub), rs);
    };
    // the next step's source, advanced by a running pointer (the key rows, then
    // the value rows from their own first row)
    const uint8_t *nxt_first = kfirst + static_cast<int64_t>(sub) * K.row_words * 4;
    int nxt_rs = K.row_words * 4, nxt_left = nrows - sub;
    SubSrc last_src{};
    auto next_src = [&](int st1) __attribute__((always_inline)) {
        if (st1 >= 2 * nsub) return last_src;         // past the last step: its chunks again
        if (st1 == nsub) {
            nxt_first = vfirst;
            nxt_rs = V.row_words * 4;
            nxt_left = nrows;
        }
        last_src = sub_src(nxt_first, 0, min(sub, nxt_left), nxt_rs);
        nxt_first += static_cast<int64_t>(sub) * nxt_rs;
        nxt_left -= sub;
        return last_src;
    };

    u32x4 stg[ST], stg2[ST];
    SubSrc g0 = step_src(0);
    sub_load(g0, stg);
    SubSrc g1 = next_src(1);
    sub_load(g1, stg2);
    // ---- the query's scorer operands (while the first sub-chunk is in flight)
    const int nksK = K.kfetch >> 4;
    float beta, mul, bias_t;
    {
        const int b = u / a.H, h = u % a.H;
        // every global operand of the prologue and of the output is requested
        // before the first use (one memory round trip, not one per step)
        const int ns = K.ui[u].n_slots, nv = V.ui[u].n_slots;
        const float qd = tid < a.D ? (a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[b * a.qsb + h * a.qsh + tid])
                                              : static_cast<const float *>(a.q)[b * a.qsb + h * a.qsh + tid])
                                   : 0.f;
        const uint32_t kdt = tid < nksK ? K.kdesc[static_cast<int64_t>(u) * nksK + tid] : 0u;
        const int fsl = tid < K.kfetch ? K.fslot[static_cast<int64_t>(u) * K.kfetch + tid] : -1;
        const float mu_t = tid < a.D ? K.mu[static_cast<int64_t>(u) * a.D + tid] : 0.f;
        bias_t = tid < a.D ? V.bias[static_cast<int64_t>(u) * a.D + tid] : 0.f;
        const int vfs_t = tid < V.kfetch ? V.fslot[static_cast<int64_t>(u) * V.kfetch + tid] : -1;
        const int vc_t = tid < nv ? V.comp[static_cast<int64_t>(u) * V.kslots + tid] : 0;
        const float vsc_t = tid < nv ? V.qscale[static_cast<int64_t>(u) * V.rmax + vc_t] : 0.f;
        // the key ranges of the slots this lane's quad forms (at most 2 x 128 slots)
        float ksc[2], kmn[2];
#pragma unroll
        for (int pj = 0; pj < 2; ++pj) {
            const int j = pj * (kAttThreads / 4) + (tid >> 2);
            const int cj = j < ns ? K.comp[static_cast<int64_t>(u) * K.kslots + j] : 0;
            ksc[pj] = j < ns ? K.qscale[static_cast<int64_t>(u) * K.rmax + cj] : 0.f;
            kmn[pj] = j < ns ? K.qmin[static_cast<int64_t>(u) * K.rmax + cj] : 0.f;
        }
        if (tid < a.D) ql[tid] = qd;
        if (tid < nksK) kds[tid] = kdt;
        if (tid < kMaxSlots) {
            vfs[tid] = vfs_t;
            vsc[tid] = vsc_t;
        }
        if (tid == 0) qal[kAttKsK * 4] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        // qt_j = scale_j (q . V_j) / sqrt(D), and min_j (q . V_j) for the offset:
        // four lanes per slot, lane p of a quad taking the features d = p (mod 4)
        // (or, rows of 16-byte multiples, the features 4f..4f+3 for f = p (mod 4))
        const bool vec4 = (a.D & 3) == 0 && (reinterpret_cast<uintptr_t>(K.basis) & 15u) == 0;
#pragma unroll
        for (int pj = 0; pj < 2; ++pj) {
            const int j = pj * (kAttThreads / 4) + (tid >> 2), part = tid & 3;
            if (pj * (kAttThreads / 4) >= K.kslots) break;                   // (uniform)
            float acc = 0.f;
            if (j < ns) {
                // the row's loads issued kAttBatch at a time (one memory round
                // trip per batch, not per feature)
                const float *vrow = K.basis + (static_cast<int64_t>(u) * K.kslots + j) * a.D;
                if (vec4) {                                                  // 16-byte rows: lane p takes quads p (mod 4)
                    const float4 *vr4 = reinterpret_cast<const float4 *>(vrow);
                    const float4 *q4 = reinterpret_cast<const float4 *>(ql);
                    for (int f0 = part; f0 < (a.D >> 2); f0 += 4 * (kAttBatch / 2)) {
                        float4 v[kAttBatch / 2];
#pragma unroll
                        for (int k = 0; k < kAttBatch / 2; ++k)
                            v[k] = f0 + 4 * k < (a.D >> 2) ? vr4[f0 + 4 * k] : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int k = 0; k < kAttBatch / 2; ++k)
                            if (f0 + 4 * k < (a.D >> 2)) {
                                const float4 qv = q4[f0 + 4 * k];
                                acc = fmaf(qv.x, v[k].x, fmaf(qv.y, v[k].y, fmaf(qv.z, v[k].z, fmaf(qv.w, v[k].w, acc))));
                            }
                    }
                } else {                                                     // (a device blob off 16 bytes)
                    for (int d0 = part; d0 < a.D; d0 += 4 * kAttBatch) {
                        float v[kAttBatch];
#pragma unroll
                        for (int k = 0; k < kAttBatch; ++k) v[k] = d0 + 4 * k < a.D ? vrow[d0 + 4 * k] : 0.f;
#pragma unroll
                        for (int k = 0; k < kAttBatch; ++k)
                            if (d0 + 4 * k < a.D) acc = fmaf(ql[d0 + 4 * k], v[k], acc);
                    }
                }
            }
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xF, 0xF, false));
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, false));
            if (part == 0 && j < K.kslots) {
                qts[j] = ksc[pj] * acc * a.inv_sqrt_d;
                mpt[j] = kmn[pj] * acc;
            }
        }
        __syncthreads();
        const float qt = tid < K.kslots ? qts[tid] : 0.f;
        // fetch column 16 ks + t: Q = rint(qt * 2^(30 - e)), 2^e > max |qt| so that
        // |Q| < 2^30, as four balanced int8 digits (Q = sum_d d_d 256^d; the bytes
        // of (Q + 0x808080) ^ 0x808080), digit d at byte (4 ks + d) * 16 + t;
        // padding columns are zero.  The scorer reads 8-bit codes as c - 128; the
        // missing 128 * sum Q over the 8-bit columns is added to the offset.
        const float amax = block_reduce(fabsf(qt), red, true);
        int e = 0;
        if (amax > 0.f) frexpf(amax, &e);
        float q8 = 0.f;
        if (tid < K.kfetch) {
            const int j = fsl;
            const int ks = tid >> 4, t = tid & 15;
            const int32_t Q = j >= 0 ? static_cast<int32_t>(rintf(ldexpf(qts[j], 30 - e))) : 0;
            const uint32_t W = (static_cast<uint32_t>(Q) + 0x808080u) ^ 0x808080u;
            uint8_t *qab = reinterpret_cast<uint8_t *>(qal);
#pragma unroll
            for (int d = 0; d < 4; ++d) qab[(ks * 4 + d) * 16 + t] = static_cast<uint8_t>(W >> (8 * d));
            if (j >= 0 && ((kds[ks] >> 16) & 0xFu) == 8u) q8 = static_cast<float>(Q);
        }
        const float c8 = block_reduce(q8, red, false);
        // (q . mu + sum_j min_j q . V_j) / sqrt(D)
        float bpart = tid < a.D ? qd * mu_t : 0.f;
        if (tid < K.kslots) bpart += mpt[tid];
        const float bsum = block_reduce(bpart, red, false);
        beta = bsum * a.inv_sqrt_d + ldexpf(128.0f * c8, e - 30);
        mul = ldexpf(1.0f, e - 30);
        // the products: consecutive k-steps of one width in pairs (lanes 0-31 take
        // the first, lanes 32-63 the second, so a product decodes one width).
        // Wave 0, lane l for k-step l: a run of equal widths starts where the
        // width changes; k-steps at even positions of a run of nonzero width head
        // a product, with the next one if it is in the run; products in k-step
        // order (heads counted below each lane).
        if (wave == 0) {
            const int l = static_cast<int>(lane);
            const uint32_t kdl = l < nksK ? kds[l] : 0u;
            const uint32_t w = (kdl >> 16) & 0xFu;
            const uint32_t wprev = __shfl_up(w, 1), wnext = __shfl_down(w, 1), kdn = __shfl_down(kdl, 1);
            const uint64_t starts = __ballot(l == 0 || w != wprev);
            const uint64_t upto = l == 63 ? ~0ull : (2ull << l) - 1ull;
            const int run0 = 63 - __clzll(starts & upto);
            const bool head = w != 0u && ((l - run0) & 1) == 0;
            const uint64_t heads = __ballot(head);
            if (head) {
                const int np = __popcll(heads & ((1ull << l) - 1ull));
                const bool two = l + 1 < nksK && wnext == w;
                const uint32_t kb = two ? static_cast<uint32_t>(l + 1) : 0xFFu;
                ptab[1 + 2 * np] = static_cast<uint32_t>(l) | (kb << 8) | (w << 16);
                ptab[2 + 2 * np] = (kdl & 0xFFFFu) | (two ? (kdn & 0xFFFFu) << 16 : 0u);
            }
            if (l == 0) ptab[0] = static_cast<uint32_t>(__popcll(heads));
        }
        __syncthreads();
    }
    // the scorer's products (uniform widths), and per lane its k-step's offset
    // and the LDS address of its A operand (digit row d < 4 of the lane's
    // k-step; a zero vector for lanes 4-31 of a half and for a product's
    // missing second k-step)
    const int npairs = __builtin_amdgcn_readfirstlane(static_cast<int>(ptab[0]));
    // (the first kAttPairs products from registers, any others decoded per use)
    auto pair_lane = [&](int m, uint32_t &wid, uint32_t &off, uint32_t &addr) __attribute__((always_inline)) {
        const uint32_t meta = __builtin_amdgcn_readfirstlane(ptab[1 + 2 * m]);
        const uint32_t offs = __builtin_amdgcn_readfirstlane(ptab[2 + 2 * m]);
        const bool hi = lane >= 32;
        const uint32_t ks = hi ? (meta >> 8) & 0xFFu : meta & 0xFFu;
        const bool ok = ks != 0xFFu;
        wid = (meta >> 16) & 0xFu;
        off = ok && hi ? offs >> 16 : offs & 0xFFFFu;
        addr = ok && (lane & 31u) < 4u ? ks * 4u + (lane & 31u) : static_cast<uint32_t>(kAttKsK * 4);
    };
    // widths uniform; each lane's offset and operand address in an LDS table
    // (offset | address << 16, one word per product and lane)
    uint32_t pwid[kAttPairs];
#pragma unroll
    for (int m = 0; m < kAttPairs; ++m) {
        pwid[m] = 0u;
        if (m < npairs) {
            uint32_t off, addr;
            pair_lane(m, pwid[m], off, addr);
            if (wave == 0) plt[m * 64 + lane] = off | (addr << 16);
        }
    }
    // this wave's value k-steps w + kAttWaves i: widths and offsets (uniform), and the
    // stored slots of the columns lane n of a quad sums (fetch columns 4r + n)
    const int nksV = V.kfetch >> 4;
    const uint32_t n = lane & 3u;
    uint32_t vw[KW], voff[KW];
#pragma unroll
    for (int i = 0; i < KW; ++i) {
        const int ks = wave + kAttWaves * i;
        const uint32_t kd = ks < nksV ? V.kdesc[static_cast<int64_t>(u) * nksV + ks] : 0u;
        vw[i] = (kd >> 16) & 0xFu;
        voff[i] = kd & 0xFFFFu;
    }
    uint32_t s1, s2;
    quad_selectors(lane, s1, s2);
    sub_store(g0, buf0, stg);
    __syncthreads();

    float mloc = -__builtin_huge_valf(), M = 0.f, L = 0.f;
    i32x4 acc[KW][4];
#pragma unroll
    for (int i = 0; i < KW; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[i][rr] = i32x4{0, 0, 0, 0};
    // Step st decodes buffer st & 1 and, at its start, loads the chunks of step
    // st + 2 into the free staging set (every load issued: past the last step
    // the last step's chunks again), so two sub-chunks are in flight while one
    // is decoded; at its end it stores step st + 1's set into the other buffer.
    uint32_t pe_r[kAttPairs];                         // the lane's product operands, held through the key steps
    auto step = [&](auto key_c, int st, u32x4 (&s_free)[ST], u32x4 (&s_next)[ST],
                    const SubSrc &g_next, SubSrc &g_load, int dcur) __attribute__((always_inline)) {
        const uint32_t *cur = ((st & 1) ? buf1 : buf0) + dcur;
        uint32_t *nxt = (st & 1) ? buf0 : buf1;
        g_load = next_src(st + 2);
        sub_load(g_load, s_free);
        if constexpr (decltype(key_c)::value) {
            // scores (32x32x32 products, D[d][row] = sum_k A[d][k] B[k][row]): A
            // holds the query's digits (row d = digit d, rows 4-31 zero), B a
            // tile's codes; lane l supplies row or column l & 31 over k-range
            // 16(l >> 5), lanes 0-31 the pair's first k-step, lanes 32-63 its
            // second.  Wave w takes tile w of the sub-chunk; lane l (< 32) ends
            // with the four digit sums of the tile's row l.
            const int j0 = st * sub, rows_j = min(sub, nrows - j0);
            if (wave * 32 < sub) {
                const uint32_t *row0 = cur + (wave * 32 + static_cast<int>(lane & 31)) * K.row_words;
                i32x16 a0;
#pragma unroll
                for (int i = 0; i < 16; ++i) a0[i] = 0;
                // a lane without a k-step decodes its product's other one: its
                // operand A is zero, so those products vanish
                auto product = [&](uint32_t wid, uint32_t off, uint32_t addr) __attribute__((always_inline)) {
                    const u32x4 qv = qal[addr];
                    uint32_t R[4];
                    kstep_bytes_any<WS>(wid, off, row0, R);
                    a0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, qv),
                                                               __builtin_bit_cast(i32x4, u32x4{R[0], R[1], R[2], R[3]}),
                                                               a0, 0, 0, 0);
                };
#pragma unroll
                for (int m = 0; m < kAttPairs; ++m) {
                    if (m < npairs) {
                        product(pwid[m], pe_r[m] & 0xFFFFu, pe_r[m] >> 16);
                    }
                }
                for (int m = kAttPairs; m < npairs; ++m) {
                    uint32_t wid, off, addr;
                    pair_lane(m, wid, off, addr);
                    product(wid, off, addr);
                }
                const int r0 = wave * 32 + static_cast<int>(lane);
                if (lane < 32 && r0 < rows_j) {
                    const float T = fmaf(static_cast<float>(a0[3]), 16777216.0f,
                                         fmaf(static_cast<float>(a0[2]), 65536.0f,
                                              fmaf(static_cast<float>(a0[1]), 256.0f, static_cast<float>(a0[0]))));
                    const float sc = fmaf(T, mul, beta);
                    pl[j0 + r0] = sc;
                    mloc = fmaxf(mloc, sc);
                }
            }
        } else {
            if (st == nsub) {
                // every score is in: the weights p = exp(s - M), their sum, and
                // their digit words (P = rint(p * 2^30) <= 2^30 as four balanced
                // int8 digits) in place of the scores.  A thread takes a quad of
                // rows and stores its words transposed: word 4q + n holds digit n
                // of rows 4q..4q+3 (byte s: row 4q + s), operand A as the value
                // products read it.
                M = block_reduce(mloc, red, true);
                float lsum = 0.f;
                uint64_t psum = 0;
                for (int q4 = tid; 4 * q4 < nsub * sub; q4 += blockDim.x) {     // (zero words up to the last sub-chunk's end)
                    const u32x4 sc4 = reinterpret_cast<const u32x4 *>(pl)[q4];
                    uint32_t W[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p = 4 * q4 + i < nrows ? expf(__uint_as_float(sc4[i]) - M) : 0.f;
                        lsum += p;
                        const uint32_t P = static_cast<uint32_t>(rintf(p * 1073741824.0f));
                        psum += P;
                        W[i] = (P + 0x808080u) ^ 0x808080u;
                    }
                    // 4x4 byte transpose: T[n] byte s = W[s] byte n
                    const uint32_t x01l = __builtin_amdgcn_perm(W[1], W[0], 0x05010400u);   // W0.0 W1.0 W0.1 W1.1
                    const uint32_t x01h = __builtin_amdgcn_perm(W[1], W[0], 0x07030602u);   // W0.2 W1.2 W0.3 W1.3
                    const uint32_t x23l = __builtin_amdgcn_perm(W[3], W[2], 0x05010400u);
                    const uint32_t x23h = __builtin_amdgcn_perm(W[3], W[2], 0x07030602u);
                    const u32x4 T = {__builtin_amdgcn_perm(x23l, x01l, 0x05040100u), __builtin_amdgcn_perm(x23l, x01l, 0x07060302u),
                                     __builtin_amdgcn_perm(x23h, x01h, 0x05040100u), __builtin_amdgcn_perm(x23h, x01h, 0x07060302u)};
                    reinterpret_cast<u32x4 *>(pw)[q4] = T;
                }
                // sum P exactly (below 2^44) for the 8-bit columns' correction: per
                // wave, into the scorer operands' space (free once the keys are done)
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) psum += __shfl_xor(psum, o);
                if (lane == 0) reinterpret_cast<uint64_t *>(qal)[wave] = psum;
                L = block_reduce(lsum, red, false);   // (its barriers publish the digit words and sums)
            }
            // p-weighted sums of the value codes on 4x4x4 products (16 blocks of
            // 4 lanes, D[d][col] = sum_k A[d][k] B[k][col]): lane l holds row l of
            // each 64-row group (quad q: rows 4q..4q+3); A is the quad's digits of
            // P (stored transposed), B its codes of fetch columns 4r + n (lane n,
            // register r), from the lanes' own rows by a byte transpose across
            // the quad.  Wave
            // w takes the k-steps w + kAttWaves i over every row.  Sums are exact in int32
            // (|digit|, |code| <= 128, at most 9216 rows).
            // the sub-chunk's G = sub / 64 groups, rows past the segment with zero
            // A (their codes are stale words inside the buffer)
            const int j0 = (st - nsub) * sub;
            uint32_t Ag[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                Ag[g] = pw[j0 + g * 64 + static_cast<int>(lane)];
            }
            const uint32_t *vrow0 = cur + static_cast<int>(lane) * V.row_words;
#pragma unroll
            for (int i = 0; i < KW; ++i) value_kstep_any<WS, G>(vw[i], acc[i], voff[i], vrow0, V.row_words, Ag, s1, s2);
        }
        if (st + 1 < 2 * nsub) sub_store(g_next, nxt, s_next);
        __syncthreads();
    };
    // the key steps, then the value steps, each loop taking two steps at a time
    // (the staging sets alternate); an odd number of sub-chunks puts the last
    // key step and the first value step in one pair
    const std::integral_constant<bool, true> key_step;
    const std::integral_constant<bool, false> value_step;
    SubSrc gA = g0, gB = g1;
#pragma unroll
    for (int m = 0; m < kAttPairs; ++m) pe_r[m] = plt[m * 64 + lane];   // (entries past npairs unused)
    int st = 0;
    for (; st + 1 < nsub; st += 2) {
        SubSrc ga, gb;
        step(key_step, st, stg, stg2, gB, ga, gA.delta);
        step(key_step, st + 1, stg2, stg, ga, gb, gB.delta);
        gA = ga;
        gB = gb;
    }
    if (st < nsub) {
        SubSrc ga, gb;
        step(key_step, st, stg, stg2, gB, ga, gA.delta);
        step(value_step, st + 1, stg2, stg, ga, gb, gB.delta);
        gA = ga;
        gB = gb;
        st += 2;
    }
    for (; st < 2 * nsub; st += 2) {
        SubSrc ga, gb;
        step(value_step, st, stg, stg2, gB, ga, gA.delta);
        step(value_step, st + 1, stg2, stg, ga, gb, gB.delta);
        gA = ga;
        gB = gb;
    }
    if (nsub == 0) {                                   // (an empty segment: never launched)
        M = -__builtin_huge_valf();
    }

    // totals over the 16 quads: rotations by 4 and 8 lanes inside each row of 16,
    // then the row pairs and halves swapped in (lane n of every quad ends with
    // its column's sums)
    auto quad_total = [](int v) __attribute__((always_inline)) {
        v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);   // row_ror:4
        v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);   // row_ror:8
        const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = static_cast<int>(p16[0]) + static_cast<int>(p16[1]);
        const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return static_cast<int>(p32[0]) + static_cast<int>(p32[1]);
    };
#pragma unroll
    for (int i = 0; i < KW; ++i) {
        if (vw[i] == 0u) continue;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) acc[i][rr][dd] = quad_total(acc[i][rr][dd]);
    }
    // sum P over the segment (the waves' exact sums from the softmax pass)
    double sp = 0.0;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) sp += static_cast<double>(reinterpret_cast<const uint64_t *>(qal)[w]);
    // abar of fetch column 16 ks + 4r + n = 2^-30 (sum_d 256^d acc_d), plus
    // 128 * sum P for 8-bit columns (read as c - 128); lanes 0-3 write, to the
    // partial sums of a segment or (a single segment) to LDS for the output
    const bool single = a.nchunks == 1;
    float *dst = single ? qts : a.part + (static_cast<int64_t>(u) * a.nchunks + c) * (V.kslots + 2);
    if (lane < 4) {
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            if (vw[i] == 0u) continue;
            const double corr = vw[i] == 8u ? 128.0 * sp : 0.0;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int j = vfs[(wave + kAttWaves * i) * 16 + 4 * rr + static_cast<int>(n)];
                if (j < 0) continue;
                const i32x4 v = acc[i][rr];
                const double T = ((static_cast<double>(v[3]) * 256.0 + v[2]) * 256.0 + v[1]) * 256.0 + v[0];
                dst[j] = static_cast<float>((T + corr) * 0x1p-30);
            }
        }
    }
    if (!single) {
        if (tid == 0) {
            dst[V.kslots] = M;
            dst[V.kslots + 1] = L;
        }
        return;
    }
    // a single segment: out = bias + sum_j (abar_j / L) scale_j V_j, rounded to fp16
    // (the merge of one chunk, whose weight is 1)
    __syncthreads();
    const int nv = V.ui[u].n_slots;
    if (tid < nv) mpt[tid] = qts[tid] / L * vsc[tid];
    __syncthreads();
    // np parts per feature (np * D <= 512 partial sums in ql and qts), part p
    // summing the slots j = p (mod np)
    const int b = u / a.H, h = u % a.H;
    const int np = a.D <= 128 ? 4 : 2;
    float *ob = ql;
    if (tid < np * a.D) {
        const int d = tid % a.D, part = tid / a.D;
        const float *vb = V.basis + static_cast<int64_t>(u) * V.kslots * a.D + d;
        float o = 0.f;
        for (int j0 = part; j0 < nv; j0 += np * 2 * kAttBatch) {
            float v[2 * kAttBatch];
#pragma unroll
            for (int k = 0; k < 2 * kAttBatch; ++k) {
                const int j = j0 + np * k;
                v[k] = j < nv ? vb[static_cast<int64_t>(j) * a.D] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 2 * kAttBatch; ++k)
                if (j0 + np * k < nv) o = fmaf(mpt[j0 + np * k], v[k], o);
        }
        ob[part * a.D + d] = o;
    }
    __syncthreads();
    if (tid < a.D) {
        float o = bias_t;
        for (int p2 = 0; p2 < np; ++p2) o += ob[p2 * a.D + tid];
        a.out[b * a.osb + h * a.osh + tid] = static_cast<_Float16>(o);
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
            for (int j0 = 0; j0 < nv; j0 += kAttBatch) {
                float v[kAttBatch];
#pragma unroll
                for (int k = 0; k < kAttBatch; ++k) v[k] = j0 + k < nv ? vb[static_cast<int64_t>(j0 + k) * a.D] : 0.f;
#pragma unroll
                for (int k = 0; k < kAttBatch; ++k)
                    if (j0 + k < nv) o = fmaf(coef[j0 + k], v[k], o);
            }
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

// Workspace: the partial sums [U][segments][kslots_v + 2] f32 when the rows
// take two or more segments (one segment is finished in its block: none).
struct AttendWork {
    uint64_t part, total;
};

// Segments of the rows [0, s_end) for the partial blocks: at most kAttSegMax
// rows each, and as many as fill kAttBlocks blocks over the units without
// going below kAttSeg rows (a short cache gets fewer).  Every segment holds at
// least one row.
struct AttendSegs {
    int64_t count;
    int rows, sub;
};

AttendSegs attend_segs(const kvtc_state_header *hk, const kvtc_state_header *hv, int64_t s_end) {
    AttendSegs g{};
    // sub-chunks of 256, 128 or 64 rows whose 16-byte window fits the staged
    // chunks (rows of up to 256 bytes fit at 64)
    const int rs = std::max(hk->row_stride, hv->row_stride);
    g.sub = 256;
    while (g.sub > 64 && g.sub * rs + 16 > 16 * kAttThreads * kAttStage) g.sub >>= 1;
    if (s_end <= 0) return g;
    const int64_t units = std::max<int64_t>(1, hk->units);
    const int64_t fill = std::min<int64_t>((kAttBlocks + units - 1) / units, (s_end + kAttSeg - 1) / kAttSeg);
    const int64_t n0 = std::max<int64_t>({1, (s_end + kAttSegMax - 1) / kAttSegMax, fill});
    g.rows = static_cast<int>((s_end + n0 - 1) / n0);
    g.count = (s_end + g.rows - 1) / g.rows;
    return g;
}

// LDS of a partial block: scorer operands, reductions, the query's working
// arrays and product table, the segment's scores (rounded up to whole
// sub-chunks, whose weight digits past the last row are zero), and two sub-chunk
// buffers (the longer row times the sub-chunk plus sixteen slack words each).
size_t attend_partial_lds(const AttendSegs &g, int k_row_words, int v_row_words) {
    const size_t bw = (static_cast<size_t>(g.sub) * std::max(k_row_words, v_row_words) + 16 + 3) & ~static_cast<size_t>(3);
    return (kAttKsK * 4 + 1) * sizeof(u32x4) + (kAttWaves + 3 * kMaxSlots) * sizeof(float) +
           (kAttKsK + 1 + 2 * kAttKsK + 3 + kAttPairs * 64 + 2 * kMaxSlots) * sizeof(uint32_t) +
           static_cast<size_t>((g.rows + g.sub - 1) / g.sub * g.sub) * sizeof(float) +
           2 * bw * sizeof(uint32_t);
}

AttendWork attend_work(const kvtc_state_header *hk, const kvtc_state_header *hv, int64_t s_end) {
    AttendWork w{};
    const int64_t nchunks = attend_segs(hk, hv, s_end).count;
    w.part = 0;
    w.total = nchunks >= 2 ? static_cast<uint64_t>(hv->units) * nchunks * (hv->kslots + 2) * sizeof(float) : 0;
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
    if (need > 0 && (!work_dev || work_bytes < need || reinterpret_cast<uintptr_t>(work_dev) % 256))
        return KVTC_E_BUFSIZE;
    const AttendSegs segs = attend_segs(hk, hv, s_end);
    const int64_t nchunks = segs.count;
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
    a.chunk_rows = segs.rows;
    a.sub = segs.sub;
    a.H = static_cast<int>(hk->heads);
    a.D = hk->head_dim;
    a.inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(hk->head_dim));
    const AttendWork wl = attend_work(hk, hv, s_end);
    a.part = wl.total > 0 ? reinterpret_cast<float *>(static_cast<char *>(work_dev) + wl.part) : nullptr;
    const unsigned U = static_cast<unsigned>(hk->units);
    if (nchunks > 0) {
        const size_t lds = attend_partial_lds(segs, a.k.row_words, a.v.row_words);
        if (lds > kLdsMax) return KVTC_E_SHAPE;
        // value k-steps per wave (at most 16 k-steps over kAttWaves waves): 16
        // accumulator registers each
        const int kw = (a.v.kfetch / 16 + kAttWaves - 1) / kAttWaves;
        // the short width dispatch when both tensors' widths are within {0, 2, 4, 8}
        const bool w248 = widths_248(hk) && widths_248(hv);
        // two staged chunks per thread where a 256-row sub-chunk fits them (fewer
        // loads per step), else three
        const int rs = std::max(hk->row_stride, hv->row_stride);
        const bool st2 = a.sub == 256 && a.sub * rs + 16 <= 16 * kAttThreads * 2;
        auto pick = [&](auto k1, auto k2, auto k1n, auto k2n) { return w248 ? (kw <= 1 ? k1n : k2n) : (kw <= 1 ? k1 : k2); };
        auto kern = a.sub == 256
                        ? (st2 ? pick(attend_partial_kernel<1, 4, kWidthsAll, 2>, attend_partial_kernel<2, 4, kWidthsAll, 2>,
                                      attend_partial_kernel<1, 4, kWidths248, 2>, attend_partial_kernel<2, 4, kWidths248, 2>)
                               : pick(attend_partial_kernel<1, 4, kWidthsAll, 3>, attend_partial_kernel<2, 4, kWidthsAll, 3>,
                                      attend_partial_kernel<1, 4, kWidths248, 3>, attend_partial_kernel<2, 4, kWidths248, 3>))
                    : a.sub == 128
                        ? pick(attend_partial_kernel<1, 2, kWidthsAll, 3>, attend_partial_kernel<2, 2, kWidthsAll, 3>,
                               attend_partial_kernel<1, 2, kWidths248, 3>, attend_partial_kernel<2, 2, kWidths248, 3>)
                        : pick(attend_partial_kernel<1, 1, kWidthsAll, 3>, attend_partial_kernel<2, 1, kWidthsAll, 3>,
                               attend_partial_kernel<1, 1, kWidths248, 3>, attend_partial_kernel<2, 1, kWidths248, 3>);
        if (!allow_lds(reinterpret_cast<const void *>(kern))) return KVTC_E_DEVICE;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nchunks), U), dim3(kAttThreads), lds, stream, a);
        if (launch_status() != KVTC_OK) return KVTC_E_DEVICE;
        if (nchunks == 1) return KVTC_OK;            // the partial blocks wrote the output
    }
    // two or more segments: merged per unit; no rows: zeros
    hipLaunchKernelGGL(attend_merge_kernel, dim3(U), dim3(256), 0, stream, a);
    return launch_status();
}

}  // namespace
}  // namespace kvtc
