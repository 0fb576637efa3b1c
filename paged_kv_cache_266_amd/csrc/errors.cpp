// Status codes and the per-thread error message of the C ABI (host only).
#include <string>

#include "host.h"

namespace pkv {

static thread_local std::string g_last_error;

void clear_error() { g_last_error.clear(); }

pkv_status fail(pkv_status code, const char *msg)
{
    g_last_error = msg;
    return code;
}

}  // namespace pkv

extern "C" int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

extern "C" const char *pkv_status_string(pkv_status s)
{
    switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OOM: return "out of KV pages";
    case PKV_ERR_NO_SEQ: return "unknown sequence";
    case PKV_ERR_SEQ_EXISTS: return "sequence already exists";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_DEVICE: return "device error";
    case PKV_ERR_SHARED_PAGE: return "append needs a copy of a shared page";
    }
    return "unknown status";
}

extern "C" const char *pkv_last_error(void) { return pkv::g_last_error.c_str(); }
