// Status strings and the per-thread last-error message.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace wspmm {

spmm_status_t fail(spmm_status_t s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

spmm_status_t ok()
{
    g_last_error[0] = '\0';
    return SPMM_OK;
}

bool test_fail_alloc()
{
    const char *v = std::getenv("SPMM_TEST_FAIL_ALLOC");
    return v && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

}  // namespace wspmm

extern "C" const char *spmm_status_string(spmm_status_t s)
{
    switch (s) {
    case SPMM_OK: return "SPMM_OK";
    case SPMM_ERR_INVALID_ARGUMENT: return "SPMM_ERR_INVALID_ARGUMENT";
    case SPMM_ERR_BAD_FORMAT: return "SPMM_ERR_BAD_FORMAT";
    case SPMM_ERR_UNSUPPORTED: return "SPMM_ERR_UNSUPPORTED";
    case SPMM_ERR_OUT_OF_MEMORY: return "SPMM_ERR_OUT_OF_MEMORY";
    case SPMM_ERR_HIP: return "SPMM_ERR_HIP";
    }
    return "SPMM_ERR_UNKNOWN";
}

extern "C" const char *spmm_last_error(void) { return g_last_error; }
