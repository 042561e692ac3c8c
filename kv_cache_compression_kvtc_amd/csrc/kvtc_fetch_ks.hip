// One translation unit per fetch contraction length: compiled once for every
// KVTC_FETCH_KS in 1..16 (16-slot k-steps), so the instantiations of the fetch
// kernels build in parallel.  ndb is the block's 32-column blocks: 2 or 4 for
// fetch_kernel, 16 for the weight-stationary kernel.
#include "kvtc_fetch_ws.h"

#ifndef KVTC_FETCH_KS
#error "KVTC_FETCH_KS must be defined (1..16)"
#endif

#define KVTC_CAT2(a, b) a##b
#define KVTC_CAT(a, b) KVTC_CAT2(a, b)

namespace kvtc {

int32_t KVTC_CAT(launch_fetch_ks, KVTC_FETCH_KS)(bool mixed, int ndb, const FetchPair &m, int nt, int rw,
                                                  hipStream_t stream) {
    constexpr int KS = KVTC_FETCH_KS;
    if (ndb == 16) return mixed ? launch_fetch_ws<KS>(m, nt, rw * 64, stream) : KVTC_E_SHAPE;
    if (ndb == 4)
        return mixed ? launch_fetch_ks<true, 4, KS>(m, nt, rw, stream) : launch_fetch_ks<false, 4, KS>(m, nt, rw, stream);
    if (ndb == 2)
        return mixed ? launch_fetch_ks<true, 2, KS>(m, nt, rw, stream) : launch_fetch_ks<false, 2, KS>(m, nt, rw, stream);
    return KVTC_E_SHAPE;
}

}  // namespace kvtc
