/* Status strings for a host-only, sanitizer-instrumented build of the block
 * manager (test infrastructure): the real ones live in the HIP part of the
 * library, which a host compiler cannot build. */
#include <stdint.h>

const char *pa_status_string(int32_t status)
{
    static const char *names[] = {"PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED",
                                  "PA_ERR_WORKSPACE", "PA_ERR_HIP", "PA_ERR_POOL_EXHAUSTED"};
    return status >= 0 && status < 6 ? names[status] : "PA_UNKNOWN_STATUS";
}

const char *pa_last_error(void) { return "(sanitizer build: no detail)"; }
