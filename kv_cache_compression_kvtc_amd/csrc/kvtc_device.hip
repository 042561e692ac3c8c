// Device-call entry points of libkvtc (gfx950): argument validation, call
// plans and the launches of kvtc_append, kvtc_fetch and their paired forms.
// The kernels live in kvtc_append.hip, kvtc_fetch_kernel.h (instantiated by
// kvtc_fetch_ks.hip) and kvtc_attend.hip.
#include <mutex>
#include <set>
#include <utility>

#include "kvtc_device.h"

namespace kvtc {

// Lets a kernel use up to the whole LDS of a CU as dynamic shared memory.  The
// attribute belongs to the kernel, not to a call, so it is set once per kernel
// (and per device; the set is an idempotent per-process cache of that fact).
bool allow_lds(const void *kern) {
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        note_device_error(e);
        return false;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kern, dev})) return true;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) {
        note_device_error(e);
        return false;
    }
    done.insert({kern, dev});
    return true;
}

namespace {
thread_local hipError_t g_device_error = hipSuccess;
}

void note_device_error(hipError_t e) { g_device_error = e; }
hipError_t g_device_error_value() { return g_device_error; }

int32_t launch_status() {
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return KVTC_OK;
    g_device_error = e;
    return KVTC_E_DEVICE;
}

namespace {

typedef int32_t (*FetchKsLauncher)(bool, int, const FetchPair &, int, int, hipStream_t);
const FetchKsLauncher kFetchKs[16] = {launch_fetch_ks1,  launch_fetch_ks2,  launch_fetch_ks3,  launch_fetch_ks4,
                                      launch_fetch_ks5,  launch_fetch_ks6,  launch_fetch_ks7,  launch_fetch_ks8,
                                      launch_fetch_ks9,  launch_fetch_ks10, launch_fetch_ks11, launch_fetch_ks12,
                                      launch_fetch_ks13, launch_fetch_ks14, launch_fetch_ks15, launch_fetch_ks16};

int32_t launch_fetch(bool mixed, int ndb, const FetchPair &m, int nt, int ks, int rw, hipStream_t stream) {
    if (ks < 1 || ks > 16) return KVTC_E_SHAPE;
    return kFetchKs[ks - 1](mixed, ndb, m, nt, rw, stream);
}

int32_t plan_append(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                    const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0,
                    void *codes_dev, void *params_dev, int64_t capacity, AppendPlan *p) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (!state_dev || !x_strides) return KVTC_E_ARG;
    if (dtype != KVTC_F16 && dtype != KVTC_F32) return KVTC_E_DTYPE;
    if (B != h->batch || H != h->heads) return KVTC_E_SHAPE;
    if (x_strides[3] != 1 || x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0) return KVTC_E_SHAPE;
    if (n < 0 || s0 < 0 || capacity < 0) return KVTC_E_ARG;
    if (s0 + n > capacity) return KVTC_E_CAPACITY;
    if (h->kslots > kMaxSlots || h->row_stride > kMaxRowStride || h->dg % kAppKC != 0 ||
        h->head_dim % kAppKC != 0 || h->units > 65535)
        return KVTC_E_SHAPE;
    const bool mixed = h->mode == KVTC_MODE_MIXED;
    if (mixed && h->group_size % 16 != 0) return KVTC_E_STATE;
    *p = AppendPlan{};
    p->a.n = n;
    if (n == 0) return KVTC_OK;
    if (!x_dev) return KVTC_E_ARG;
    if (h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4 != 0)) return KVTC_E_ARG;
    if (mixed && (!params_dev || reinterpret_cast<uintptr_t>(params_dev) % 4 != 0)) return KVTC_E_ARG;
    const int nb = append_nb(h->kslots);
    if (nb < 0) return KVTC_E_SHAPE;
    const int64_t ntiles = (n + kAppTok - 1) / kAppTok;
    if (ntiles > 0x7FFFFFFF) return KVTC_E_SHAPE;

    const char *sd = static_cast<const char *>(state_dev);
    AppendArgs &a = p->a;
    a.x = x_dev;
    a.xsb = x_strides[0];
    a.xsh = x_strides[1];
    a.xss = x_strides[2];
    a.s0 = s0;
    a.capacity = capacity;
    a.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    a.mu = reinterpret_cast<const float *>(sd + h->off_mu);
    a.basis = reinterpret_cast<const float *>(sd + h->off_basis);
    a.qlo = reinterpret_cast<const double *>(sd + h->off_qlo);
    a.qinv = reinterpret_cast<const double *>(sd + h->off_qinv);
    a.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    a.codes = static_cast<uint8_t *>(codes_dev);
    a.params = static_cast<uint32_t *>(params_dev);
    a.dg = h->dg;
    a.D = h->head_dim;
    a.hpu = h->heads_per_unit;
    a.groups = static_cast<int>(h->heads / h->heads_per_unit);
    a.kslots = h->kslots;
    a.row_stride = h->row_stride;
    a.n_qg = h->n_qgroups;
    a.gs = h->group_size;
    {
        const int64_t esz = dtype == KVTC_F16 ? 2 : 4;
        a.x_vec = reinterpret_cast<uintptr_t>(x_dev) % (4 * esz) == 0 && x_strides[0] % 4 == 0 &&
                  x_strides[1] % 4 == 0 && x_strides[2] % 4 == 0;
    }
    a.inv_dg = 1.0f / static_cast<float>(h->dg);
    a.inv_q4 = 4.0f / static_cast<float>(h->dg);
    p->units = h->units;
    p->ntiles = ntiles;
    p->nb = nb;
    p->dtype = dtype;
    p->mixed = mixed;
    // bulk appends of fp16 rows run on int8 MFMA (kvtc_append_i8.hip) when the
    // blob carries the basis digits, the units are wide (512 features or more:
    // for narrower ones the fp64 kernel, whose per-code work is lighter, is
    // faster), the contraction is whole rounds of four 32-feature k-steps of
    // single heads, and each block's slot group owns whole row
    // words (a group boundary inside a unit's slots falls on a word boundary)
    p->i8_ns = p->i8_nsg = 0;
    if (h->off_vdig && h->off_mv && dtype == KVTC_F16 && a.x_vec && n > 16 && h->dg % 128 == 0 &&
        h->dg >= 512 && h->head_dim % 32 == 0 && h->dg <= 2048 && h->kslots > 32 &&
        (!mixed || h->group_size == 32)) {
        const int ns = h->kslots <= 128 ? (h->kslots + 31) / 32 : 2;
        const int nsg = (h->kslots + 32 * ns - 1) / (32 * ns);
        const char *sh = static_cast<const char *>(state_host);
        const auto *ui = reinterpret_cast<const kvtc_unit_info *>(sh + h->off_unit);
        const auto *sb = reinterpret_cast<const uint32_t *>(sh + h->off_slot_bits);
        bool aligned = true;
        for (int64_t u = 0; u < h->units && aligned; ++u)
            for (int gi = 1; gi < nsg; ++gi) {
                const int j = gi * 32 * ns;
                if (j < ui[u].n_slots && (sb[u * h->kslots + j] & kOffsetMask) % 32 != 0) aligned = false;
            }
        if (aligned) {
            a.vdig = reinterpret_cast<const int8_t *>(sd + h->off_vdig);
            a.mv = reinterpret_cast<const double *>(sd + h->off_mv);
            p->i8_ns = ns;
            p->i8_nsg = nsg;
        }
    }
    return KVTC_OK;
}

int32_t plan_fetch(const void *state_host, const void *state_dev, const void *codes_dev, const void *params_dev,
                   int64_t capacity, int64_t s_begin, int64_t s_end, void *out_dev, const int64_t out_strides[4],
                   FetchPlan *p, int share = 1) {
    const kvtc_state_header *h = nullptr;
    int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (!state_dev || !out_strides) return KVTC_E_ARG;
    if (capacity < 0 || s_begin < 0 || s_end < s_begin) return KVTC_E_ARG;
    if (s_end > capacity) return KVTC_E_CAPACITY;
    if (out_strides[3] != 1 || out_strides[0] < 0 || out_strides[1] < 0 || out_strides[2] < 0)
        return KVTC_E_SHAPE;
    const bool mixed = h->mode == KVTC_MODE_MIXED;
    if (h->kfetch > kMaxSlots || h->head_dim % 64 != 0) return KVTC_E_SHAPE;
    const int tw = h->row_stride / 4 + (mixed ? h->n_qgroups : 0);
    if (kFetTok * tw > 64 * kFetchRegWords) return KVTC_E_SHAPE;
    *p = FetchPlan{};
    if (s_end == s_begin) return KVTC_OK;
    if (!out_dev || reinterpret_cast<uintptr_t>(out_dev) % 16 != 0) return KVTC_E_ARG;
    if ((out_strides[0] * 2) % 16 || (out_strides[1] * 2) % 16 || (out_strides[2] * 2) % 16) return KVTC_E_SHAPE;
    if (h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4 != 0)) return KVTC_E_ARG;
    if (mixed && (!params_dev || reinterpret_cast<uintptr_t>(params_dev) % 4 != 0)) return KVTC_E_ARG;

    const char *sd = static_cast<const char *>(state_dev);
    FetchArgs &a = p->a;
    a.codes = static_cast<const uint8_t *>(codes_dev);
    a.params = static_cast<const uint32_t *>(params_dev);
    a.capacity = capacity;
    a.s_begin = s_begin;
    a.s_end = s_end;
    a.w16 = reinterpret_cast<const uint16_t *>(sd + h->off_w16);
    a.bias = reinterpret_cast<const float *>(sd + h->off_bias);
    a.kdesc = reinterpret_cast<const uint32_t *>(sd + h->off_kdesc);
    a.out = static_cast<_Float16 *>(out_dev);
    a.osb = out_strides[0];
    a.osh = out_strides[1];
    a.oss = out_strides[2];
    a.dg = h->dg;
    a.D = h->head_dim;
    a.hpu = h->heads_per_unit;
    a.groups = static_cast<int>(h->heads / h->heads_per_unit);
    a.kfetch = h->kfetch;
    a.nks = h->kfetch / 16;
    a.row_stride = h->row_stride;
    a.n_qg = h->n_qgroups;
    a.nqg_inv = mixed ? 1.0f / static_cast<float>(h->n_qgroups) : 0.0f;
    // a block covers whole output rows of a head (128 columns) where the head
    // size allows, so every token's fields are decoded once per head; wide
    // group-head units with long contractions take weight-stationary blocks of
    // 512 columns
    const bool ws = mixed && h->dg % fetch_ws_cols(2) == 0 && h->kfetch >= 128 &&
                    fetch_ws_rwb(kFetTok * tw) <= 3;
    const int DS = ws ? fetch_ws_cols(2) : (h->head_dim % 128 == 0) ? 128 : 64;
    a.nslices = h->dg / DS;
    const int64_t ntiles = (s_end - s_begin + kFetTok - 1) / kFetTok;
    if (ntiles > 0x7FFFFFFF) return KVTC_E_SHAPE;
    a.ntiles = static_cast<int>(ntiles);
    const int64_t work = h->units * a.nslices * ntiles;
    const int nw = ws ? kWsWaves : (DS == 128 && h->kfetch >= 160) ? 8 : 4;
    // about two four-wave blocks, or one eight-wave block (weight-stationary
    // included), per CU in one round (shared between the tensors of a paired
    // launch); a weight-stationary block runs at least two tiles
    const int64_t target = (ws ? kFetchBlocks / 2 : kFetchBlocks * 4 / nw) / share;
    const int64_t tmin = ws ? 2 : nw;
    const int64_t tpb = std::min<int64_t>(std::max<int64_t>(tmin, (work + target - 1) / target), ntiles);
    a.tiles_per_block = static_cast<int>(tpb);
    a.nchunks = static_cast<int>((ntiles + tpb - 1) / tpb);
    a.nblocks = h->units * a.nslices * a.nchunks;
    if (a.nblocks > 0x7FFFFFFF) return KVTC_E_SHAPE;
    p->ds = DS;
    p->rw = (kFetTok * tw + 63) / 64;
    p->mixed = mixed;
    p->narrow = !mixed && widths_248(h);
    return KVTC_OK;
}

// One fetch launch for one plan (p1 == NULL) or for two plans of the same
// mode and block width; the kernel is instantiated for the wider contraction.
// The probe of one launch of launch_fetch_plans: same pair, blocks and waves.
int32_t launch_probe_plans(const FetchPlan &p0, const FetchPlan *p1, hipStream_t stream) {
    FetchPair m{};
    m.t[0] = p0.a;
    m.split = p0.a.nblocks;
    m.nblocks_real = p0.a.nblocks;
    int ks = p0.a.nks;
    if (p1) {
        m.t[1] = p1->a;
        m.nblocks_real += p1->a.nblocks;
        ks = std::max(ks, p1->a.nks);
    }
    m.nblocks_per_xcd = (m.nblocks_real + 7) / 8;
    if (m.nblocks_per_xcd * 8 > 0x7FFFFFFF) return KVTC_E_SHAPE;
    if (p0.ds == fetch_ws_cols(2)) {
        if (!p0.mixed) return KVTC_E_SHAPE;
        return launch_fetch_ws_probe(m, p1 ? 2 : 1, ks, 2, 64 * std::max(p0.rw, p1 ? p1->rw : 0), stream);
    }
    // the fetch kernel's waves per block and its dynamic LDS, so that as many
    // probe blocks share a CU as fetch blocks would
    const int ndb = p0.ds / 32;
    const int nw = (p0.ds == 128 && ks >= 10) ? 8 : 4;
    const int nh = nw == 8 ? ndb / 2 : ndb;
    const int rw = fetch_rw_inst(ndb, std::max(p0.rw, p1 ? p1->rw : 0));
    const bool flat = fetch_flat_path(p0.mixed, ks, rw, nw);
    size_t lds = fetch_lds_plan(m.t[0], p0.mixed, p0.ds, nw, nh, rw, flat);
    if (p1) lds = std::max(lds, fetch_lds_plan(m.t[1], p0.mixed, p0.ds, nw, nh, rw, flat));
    if (lds > kLdsMax) return KVTC_E_SHAPE;
    return launch_fetch_probe(m, p0.ds, nw, p0.mixed, rw, lds, stream);
}

int32_t launch_fetch_plans(const FetchPlan &p0, const FetchPlan *p1, hipStream_t stream) {
    FetchPair m{};
    m.t[0] = p0.a;
    m.split = p0.a.nblocks;
    m.nblocks_real = p0.a.nblocks;
    int ks = p0.a.nks, rw = p0.rw, nt = 1;
    if (p1) {
        m.t[1] = p1->a;
        m.nblocks_real += p1->a.nblocks;
        ks = std::max(ks, p1->a.nks);
        rw = std::max(rw, p1->rw);
        nt = 2;
    }
    m.narrow = p0.narrow && (!p1 || p1->narrow);
    m.nblocks_per_xcd = (m.nblocks_real + 7) / 8;
    if (m.nblocks_per_xcd * 8 > 0x7FFFFFFF) return KVTC_E_SHAPE;
    return launch_fetch(p0.mixed, p0.ds / 32, m, nt, ks, rw, stream);
}

}  // namespace
}  // namespace kvtc

using namespace kvtc;

extern "C" {

int32_t kvtc_append(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                    const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0,
                    void *codes_dev, void *params_dev, int64_t capacity, void *hip_stream) {
    AppendPlan p;
    const int32_t st = plan_append(state_host, state_dev, x_dev, dtype, x_strides, B, H, n, s0, codes_dev,
                                   params_dev, capacity, &p);
    if (st != KVTC_OK) return st;
    return launch_append_plan(p, static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_fetch(const void *state_host, const void *state_dev, const void *codes_dev,
                   const void *params_dev, int64_t capacity, int64_t s_begin, int64_t s_end,
                   void *out_dev, const int64_t out_strides[4], void *hip_stream) {
    FetchPlan p;
    const int32_t st = plan_fetch(state_host, state_dev, codes_dev, params_dev, capacity, s_begin, s_end, out_dev,
                                  out_strides, &p);
    if (st != KVTC_OK || s_end == s_begin) return st;
    return launch_fetch_plans(p, nullptr, static_cast<hipStream_t>(hip_stream));
}

int32_t kvtc_append_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t B, int64_t H, int64_t n,
                       int64_t s0, void *hip_stream) {
    if (!k || !v) return KVTC_E_ARG;
    AppendPlan pk, pv;
    int32_t st = plan_append(k->state_host, k->state_dev, k->rows_dev, k->dtype, k->strides, B, H, n, s0,
                             k->codes_dev, k->params_dev, k->capacity, &pk);
    if (st != KVTC_OK) return st;
    st = plan_append(v->state_host, v->state_dev, v->rows_dev, v->dtype, v->strides, B, H, n, s0, v->codes_dev,
                     v->params_dev, v->capacity, &pv);
    if (st != KVTC_OK || n == 0) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (decode_path(pk) && decode_path(pv) && pk.dtype == pv.dtype && pk.a.dg == pv.a.dg)
        return launch_decode(pk, &pv, stream);
    st = launch_append_plan(pk, stream);
    if (st != KVTC_OK) return st;
    return launch_append_plan(pv, stream);
}

int32_t kvtc_fetch_kv(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t s_begin, int64_t s_end,
                      void *hip_stream) {
    if (!k || !v) return KVTC_E_ARG;
    FetchPlan pk, pv;
    int32_t st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                            k->rows_dev, k->strides, &pk);
    if (st != KVTC_OK) return st;
    st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                    v->rows_dev, v->strides, &pv);
    if (st != KVTC_OK || s_end == s_begin) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (pk.mixed == pv.mixed && pk.ds == pv.ds) {
        // one launch: re-plan both with the block target split between them
        st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                        k->rows_dev, k->strides, &pk, 2);
        if (st != KVTC_OK) return st;
        st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                        v->rows_dev, v->strides, &pv, 2);
        if (st != KVTC_OK) return st;
        return launch_fetch_plans(pk, &pv, stream);
    }
    st = launch_fetch_plans(pk, nullptr, stream);
    if (st != KVTC_OK) return st;
    return launch_fetch_plans(pv, nullptr, stream);
}

// ------------------------------------------------------------ measurement
int32_t kvtc_fetch_kv_probe(const kvtc_tensor_ref *k, const kvtc_tensor_ref *v, int64_t s_begin, int64_t s_end,
                            void *hip_stream) {
    if (!k || !v) return KVTC_E_ARG;
    FetchPlan pk, pv;
    int32_t st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                            k->rows_dev, k->strides, &pk);
    if (st != KVTC_OK) return st;
    st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                    v->rows_dev, v->strides, &pv);
    if (st != KVTC_OK || s_end == s_begin) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (pk.mixed == pv.mixed && pk.ds == pv.ds) {
        st = plan_fetch(k->state_host, k->state_dev, k->codes_dev, k->params_dev, k->capacity, s_begin, s_end,
                        k->rows_dev, k->strides, &pk, 2);
        if (st != KVTC_OK) return st;
        st = plan_fetch(v->state_host, v->state_dev, v->codes_dev, v->params_dev, v->capacity, s_begin, s_end,
                        v->rows_dev, v->strides, &pv, 2);
        if (st != KVTC_OK) return st;
        return launch_probe_plans(pk, &pv, stream);
    }
    st = launch_probe_plans(pk, nullptr, stream);
    if (st != KVTC_OK) return st;
    return launch_probe_plans(pv, nullptr, stream);
}

// ------------------------------------------------------------ refit mode
int32_t kvtc_refit_bytes(const void *state_host, int64_t capacity, size_t *latent_bytes, size_t *refit_bytes) {
    const kvtc_state_header *h = nullptr;
    const int32_t st = check_state(state_host, &h);
    if (st != KVTC_OK) return st;
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (capacity < 0) return KVTC_E_ARG;
    if (latent_bytes) *latent_bytes = static_cast<size_t>(h->units) * capacity * h->kslots * sizeof(double);
    if (refit_bytes) *refit_bytes = refit_layout(h, capacity).total;
    return KVTC_OK;
}

int32_t kvtc_append_refit(const void *state_host, const void *state_dev, const void *x_dev, int32_t dtype,
                          const int64_t x_strides[4], int64_t B, int64_t H, int64_t n, int64_t s0, void *latents_dev,
                          void *codes_dev, void *refit_dev, int64_t capacity, void *hip_stream) {
    AppendPlan p;
    int32_t st = plan_append(state_host, state_dev, x_dev, dtype, x_strides, B, H, n, s0, codes_dev, nullptr,
                             capacity, &p);
    if (st != KVTC_OK) return st;
    const kvtc_state_header *h = static_cast<const kvtc_state_header *>(state_host);
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (h->kslots > 256) return KVTC_E_SHAPE;
    if (!latents_dev || reinterpret_cast<uintptr_t>(latents_dev) % 8 || !refit_dev ||
        reinterpret_cast<uintptr_t>(refit_dev) % kSectionAlign)
        return KVTC_E_ARG;
    const int64_t S = s0 + n;
    if (S > 0 && h->row_stride > 0 && (!codes_dev || reinterpret_cast<uintptr_t>(codes_dev) % 4)) return KVTC_E_ARG;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    // latents of the new rows
    p.a.lat = static_cast<double *>(latents_dev);
    st = launch_refit_project(p, stream);
    if (st != KVTC_OK) return st;
    // ranges over every accumulated row, then all of their codes
    const char *sd = static_cast<const char *>(state_dev);
    char *rb = static_cast<char *>(refit_dev);
    const RefitLayout L = refit_layout(h, capacity);
    RefitArgs a{};
    a.lat = static_cast<const double *>(latents_dev);
    a.capacity = capacity;
    a.S = S;
    a.ui = reinterpret_cast<const kvtc_unit_info *>(sd + h->off_unit);
    a.sbits = reinterpret_cast<const uint32_t *>(sd + h->off_slot_bits);
    a.basis = reinterpret_cast<const float *>(sd + h->off_basis);
    a.mu = reinterpret_cast<const float *>(sd + h->off_mu);
    a.fslot = reinterpret_cast<const int32_t *>(sd + h->off_fslot);
    a.qmin32 = reinterpret_cast<float *>(rb + L.qmin32);
    a.qscale32 = reinterpret_cast<float *>(rb + L.qscale32);
    a.qlo = reinterpret_cast<double *>(rb + L.qlo);
    a.qinv = reinterpret_cast<double *>(rb + L.qinv);
    a.w16 = reinterpret_cast<uint16_t *>(rb + L.w16);
    a.bias = reinterpret_cast<float *>(rb + L.bias);
    a.part = reinterpret_cast<double *>(rb + L.part);
    a.codes = static_cast<uint8_t *>(codes_dev);
    a.kslots = h->kslots;
    a.dg = h->dg;
    a.kfetch = h->kfetch;
    a.row_stride = h->row_stride;
    a.chunks = L.chunks;
    return launch_refit_requantise(a, h->units, stream);
}

int32_t kvtc_fetch_refit(const void *state_host, const void *state_dev, const void *codes_dev, const void *refit_dev,
                         int64_t capacity, int64_t s_begin, int64_t s_end, void *out_dev, const int64_t out_strides[4],
                         void *hip_stream) {
    FetchPlan p;
    const int32_t st = plan_fetch(state_host, state_dev, codes_dev, nullptr, capacity, s_begin, s_end, out_dev,
                                  out_strides, &p);
    if (st != KVTC_OK) return st;
    const kvtc_state_header *h = static_cast<const kvtc_state_header *>(state_host);
    if (h->mode != KVTC_MODE_DP) return KVTC_E_STATE;
    if (!refit_dev || reinterpret_cast<uintptr_t>(refit_dev) % kSectionAlign) return KVTC_E_ARG;
    if (s_end == s_begin) return KVTC_OK;
    const RefitLayout L = refit_layout(h, capacity);
    const char *rb = static_cast<const char *>(refit_dev);
    p.a.w16 = reinterpret_cast<const uint16_t *>(rb + L.w16);
    p.a.bias = reinterpret_cast<const float *>(rb + L.bias);
    return launch_fetch_plans(p, nullptr, static_cast<hipStream_t>(hip_stream));
}

const char *kvtc_device_error_string(void) { return hipGetErrorString(kvtc::g_device_error_value()); }

}  // extern "C"
