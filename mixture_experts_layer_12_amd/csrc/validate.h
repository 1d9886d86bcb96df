// Input-contract checks run when COLIBRI_MOE_VALIDATE=1: before anything is
// launched, the call waits for its stream and checks on the host that every
// tensor argument lies inside one device allocation large enough for its
// shape, that floating-point inputs are finite and that index inputs lie in
// their range.  A failed check returns COLIBRI_ERR_INVALID_ARG, so a wrong
// pointer or size fails loudly instead of giving a silently wrong output (the
// failure mode that [zskr] http://www.zskr.cn/news/2272131 section 5.2
// reports).  Without the variable none of this runs: the checks copy inputs
// to the host and cost milliseconds.
#pragma once

#include <cstddef>
#include <cstdint>

#include "colibri_moe.h"

namespace colibri {

// COLIBRI_MOE_VALIDATE is set to something other than "" or "0" (read at every call)
bool validate_enabled();

class Validator {
   public:
    explicit Validator(hipStream_t stream) : stream_(stream) {}
    // [p, p + bytes) inside one device allocation (p == NULL is skipped)
    Validator &range(const void *p, size_t bytes);
    // range, then every one of n values (dtype COLIBRI_F32 or COLIBRI_BF16) finite
    Validator &finite(const void *p, size_t n, int dtype);
    // range, then every one of n int32 values in [lo, hi]
    Validator &indices(const int32_t *p, size_t n, int32_t lo, int32_t hi);
    // range, then offsets[0] = 0 <= offsets[1] <= ... <= offsets[n - 1] <= hi
    Validator &offsets(const int32_t *p, size_t n, int32_t hi);
    int status() const { return status_; }

   private:
    bool drain();
    bool fetch(const void *p, size_t bytes, void *dst);
    hipStream_t stream_;
    bool drained_ = false;
    int status_ = COLIBRI_OK;
};

}  // namespace colibri
