// Library-wide C-ABI entry points: error text, version, workspace sizing and
// the profiling hook.  The five compute entry points live beside their kernels.
#include <stdarg.h>
#include <stdio.h>

#include "abi_common.h"

namespace csa2 {

static thread_local char t_last_error[512] = "";


int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_last_error, sizeof t_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return CSA2_OK;
    return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace csa2

using namespace csa2;

extern "C" const char* csa2_last_error(void) { return t_last_error; }

extern "C" const char* csa2_version(void) { return "csa2-gfx950 0.1"; }

extern "C" size_t csa2_workspace_bytes(int op, int B, long long max_len, long long total_len,
                                       int H, int P, int k, int Hq, int D, int window) {
    (void)max_len;
    (void)H;
    if (B < 0) {
        fail(CSA2_ERR_INVALID, "csa2_workspace_bytes: B < 0");
        return 0;
    }
    switch (op) {
        case CSA2_OP_INDEX_FULL:
            if (total_len < 0 || P < 1 || k < 0 || k > P) {
                fail(CSA2_ERR_INVALID,
                     "csa2_workspace_bytes: total_len < 0, P < 1 or k outside [0, P]");
                return 0;
            }
            return index_full_ws_bytes(B, total_len, P, k);
        case CSA2_OP_SELECT_TOPK:
            return 0;
        case CSA2_OP_SPARSE_ATTN:
            if (Hq < 1 || D < 1 || k < 0 || window < 0) {
                fail(CSA2_ERR_INVALID, "csa2_workspace_bytes: bad attention sizes");
                return 0;
            }
            return sparse_attn_ws_bytes(B, Hq, D, k, window);
        default:
            fail(CSA2_ERR_INVALID, "csa2_workspace_bytes: unknown op %d", op);
            return 0;
    }
}

extern "C" size_t csa2_block_workspace_bytes(int op, int B, int T, int shared, long long max_len,
                                             long long total_len, int H, int P, int k, int Hq,
                                             int D, int window) {
    if (B < 0 || T < 1 || shared < 0 || shared > 1) {
        fail(CSA2_ERR_INVALID, "csa2_block_workspace_bytes: B < 0, T < 1 or shared not 0/1");
        return 0;
    }
    switch (op) {
        case CSA2_OP_INDEX_FULL:
            if (total_len < 0 || P < 1 || k < 0 || k > P) {
                fail(CSA2_ERR_INVALID,
                     "csa2_block_workspace_bytes: total_len < 0, P < 1 or k outside [0, P]");
                return 0;
            }
            return index_full_block_ws_bytes(B, T, shared, total_len, k);
        case CSA2_OP_SELECT_TOPK:
        case CSA2_OP_SPARSE_ATTN:
            return csa2_workspace_bytes(op, (int)((long long)B * T > 0x7FFFFFFF ? 0x7FFFFFFF : (long long)B * T),
                                        max_len, total_len, H, P, k, Hq, D, window);
        default:
            fail(CSA2_ERR_INVALID, "csa2_block_workspace_bytes: unknown op %d", op);
            return 0;
    }
}
