// Error state of the C ABI: per-thread text behind tk_last_error().
#include <cstdarg>
#include <cstdio>

#include "tk_internal.h"

namespace tk {

namespace {
thread_local char g_error[512] = "";
}

tk_status fail(tk_status status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return status;
}

tk_status ok()
{
    g_error[0] = '\0';
    return TK_OK;
}

tk_status launched(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(TK_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace tk

TK_EXPORT const char* tk_last_error(void) { return tk::g_error; }
