// abi.hip -- status strings and version of the NVFP4 C ABI (declared in nvfp4.h).
#include "nvfp4.h"

extern "C" const char* nvfp4_status_string(int status) {
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (negative extent or block dimension not a multiple of 16)";
    case NVFP4_ERR_ALIGN: return "pointer or leading dimension misaligned";
    case NVFP4_ERR_DTYPE: return "unknown dtype";
    case NVFP4_ERR_MODE: return "unknown or unsupported option combination";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }
