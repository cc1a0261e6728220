// Host-side helpers shared by the forward and backward entry points (argument
// checks, sizes, logging).  Internal to the library.
#pragma once
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

namespace ssd_host {

inline int64_t elem_size(int32_t dtype) { return dtype == SSD_DTYPE_BF16 ? 2 : 4; }

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Factor on x in the state write: 0 none, 1 the step size (Euler), 2 the exact
// zero-order hold (exp(Delta A) - 1) / A.
inline int x_scale_of(const ssd_problem_t* p) {
    if (p->flags & SSD_FLAG_ZOH) return 2;
    return (p->flags & SSD_FLAG_DT_SCALES_X) ? 1 : 0;
}

inline bool misaligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; }

inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

inline bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("SSD_LOG");
        return v && v[0] == '1';
    }();
    return on;
}

inline int check_device() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return SSD_ERR_NO_DEVICE;
    return SSD_OK;
}

// Byte sizes of the tensors of a problem.
struct Sizes {
    int64_t x, dt, bc, y, state, seq;
};
inline Sizes sizes(const ssd_problem_t* p) {
    Sizes s;
    const int64_t bt = p->batch * p->seqlen;
    s.x = bt * p->nheads * p->headdim * elem_size(p->dtype);
    s.dt = bt * p->nheads * 4;
    s.bc = bt * p->ngroups * p->dstate * elem_size(p->dtype);
    s.y = bt * p->nheads * p->headdim * 4;
    s.state = p->nseqs * p->nheads * p->headdim * p->dstate * 4;
    s.seq = bt * 4;
    return s;
}

}  // namespace ssd_host
