// Q4_0 prefill GEMM (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "qgemv.h"

extern "C" qg_status qgemm_q4_0_prefill(const void *Wp, const uint16_t *X, float *Y, int64_t M, int64_t N,
                                        int64_t K, void *stream)
{
    (void)Wp; (void)X; (void)Y; (void)M; (void)N; (void)K; (void)stream;
    return QG_ERR_LAUNCH;
}
