// Status strings and interface version of the SFA library.
#include "hd_sfa.h"

extern "C" const char* hd_status_string(int status) {
    switch (status) {
        case HD_OK: return "ok";
        case HD_ERR_NULL: return "a required pointer is NULL";
        case HD_ERR_SHAPE: return "invalid size, head grouping or pointer alignment";
        case HD_ERR_UNSUPPORTED: return "unsupported head_dim or size beyond the supported index range";
        case HD_ERR_CAPACITY: return "KV cache capacity too small for the appended entries";
        case HD_ERR_LAUNCH: return "kernel launch failed";
        case HD_ERR_WORKSPACE: return "decode workspace missing, misaligned or too small";
        case HD_ERR_SCRATCH: return "call needs more than the library's 16 MiB static decode scratch; pass a workspace to sfa_decode_step";
        default: return "unknown status";
    }
}

extern "C" int hd_abi_version(void) { return 2; }
