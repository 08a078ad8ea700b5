// Status text and version of the C ABI declared in pml.h.
#include "pml.h"

extern "C" const char *pml_status_string(int status) {
    switch (status) {
    case PML_OK: return "ok";
    case PML_ERR_NULL: return "a required pointer is NULL";
    case PML_ERR_SHAPE: return "unsupported heads / head_dim, or a negative or inconsistent size";
    case PML_ERR_BLOCK_KV: return "block_kv must be 32 or 64";
    case PML_ERR_VARLEN_NEXT_N: return "indices (varlen rows) require next_n == 1";
    case PML_ERR_STRIDE: return "page stride, table or output leading dimension too small or misaligned";
    case PML_ERR_ALIGN: return "a pointer breaks the 16-byte alignment";
    case PML_ERR_K: return "top-k k must be in [1, 4096]";
    case PML_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case PML_ERR_FORMAT: return "kv_format must be PML_KV_FP8 or PML_KV_MXFP4";
    case PML_ERR_UNSUPPORTED: return "argument combination not supported";
    case PML_ERR_HIP: return "a kernel launch failed (see hipGetLastError)";
    case PML_ERR_SCRATCH: return "input larger than the static scratch of the allocation-free call";
    default: return "unknown status";
    }
}

extern "C" int pml_version(void) { return 2 * 10000 + 0 * 100 + 0; }
