// Host-side plumbing of the C ABI: version, error strings, view validation.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace csa2 {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

csa2_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: launch failed: %s", what, hipGetErrorString(e));
        return CSA2_EHIP;
    }
    return CSA2_OK;
}

csa2_status make_rowmap(const int32_t* page_table, int32_t page_size, int32_t max_pages, int64_t seq_stride,
                        int64_t n_needed, RowMap* out, const char* what) {
    out->page_table = page_table;
    out->seq_stride = seq_stride;
    out->max_pages = max_pages;
    out->page_shift = 0;
    out->capacity = seq_stride;
    if (page_table == nullptr) {
        CSA2_ARG(seq_stride >= n_needed, "%s: seq_stride=%lld smaller than the %lld entries addressed", what,
                 (long long)seq_stride, (long long)n_needed);
        return CSA2_OK;
    }
    CSA2_ARG(page_size >= 8 && page_size % 8 == 0,
             "%s: page_size=%d must be a multiple of 8 (8-entry blocks may not straddle pages)", what, page_size);
    CSA2_REQUIRE(is_pow2(page_size), CSA2_EUNSUPPORTED, "%s: page_size=%d must be a power of two", what, page_size);
    CSA2_ARG(max_pages > 0 && (int64_t)max_pages * page_size >= n_needed,
             "%s: max_pages=%d x page_size=%d cannot hold %lld entries", what, max_pages, page_size,
             (long long)n_needed);
    out->page_shift = ilog2(page_size);
    out->capacity = (int64_t)max_pages * page_size;
    return CSA2_OK;
}

}  // namespace csa2

extern "C" int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

extern "C" const char* csa2_last_error(void) { return csa2::g_err; }

extern "C" const char* csa2_status_string(csa2_status st) {
    switch (st) {
        case CSA2_OK: return "CSA2_OK";
        case CSA2_EINVAL: return "CSA2_EINVAL";
        case CSA2_EUNSUPPORTED: return "CSA2_EUNSUPPORTED";
        case CSA2_EWORKSPACE: return "CSA2_EWORKSPACE";
        case CSA2_EMODE: return "CSA2_EMODE";
        case CSA2_EHIP: return "CSA2_EHIP";
    }
    return "CSA2_UNKNOWN";
}
