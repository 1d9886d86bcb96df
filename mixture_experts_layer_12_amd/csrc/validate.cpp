// COLIBRI_MOE_VALIDATE=1 input-contract checks (host side; see validate.h).
#include "validate.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace colibri {

namespace {
constexpr size_t kChunk = size_t(16) << 20;  // bytes copied to the host per step
}

bool validate_enabled() {
    const char *v = std::getenv("COLIBRI_MOE_VALIDATE");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

// Waits once for the work already queued on the stream: the inputs may be
// produced by it.
bool Validator::drain() {
    if (!drained_) {
        if (hipStreamSynchronize(stream_) != hipSuccess) {
            status_ = COLIBRI_ERR_HIP;
            return false;
        }
        drained_ = true;
    }
    return true;
}

bool Validator::fetch(const void *p, size_t bytes, void *dst) {
    if (hipMemcpy(dst, p, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        status_ = COLIBRI_ERR_HIP;
        return false;
    }
    return true;
}

Validator &Validator::range(const void *p, size_t bytes) {
    if (status_ != COLIBRI_OK || p == nullptr) return *this;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    // fails for anything that is not device memory of this process
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess || base == nullptr) {
        (void)hipGetLastError();
        status_ = COLIBRI_ERR_INVALID_ARG;
        return *this;
    }
    const uintptr_t b = (uintptr_t)base, q = (uintptr_t)p;
    if (q < b || q - b > size || bytes > size - (q - b)) status_ = COLIBRI_ERR_INVALID_ARG;
    return *this;
}

Validator &Validator::finite(const void *p, size_t n, int dtype) {
    const size_t es = dtype == COLIBRI_F32 ? 4 : 2;
    range(p, n * es);
    if (status_ != COLIBRI_OK || p == nullptr || n == 0 || !drain()) return *this;
    std::vector<uint8_t> buf(std::min(kChunk, n * es));
    for (size_t at = 0; at < n * es; at += buf.size()) {
        const size_t len = std::min(buf.size(), n * es - at);
        if (!fetch(static_cast<const uint8_t *>(p) + at, len, buf.data())) return *this;
        if (es == 4) {
            for (size_t i = 0; i < len; i += 4) {
                uint32_t u;
                std::memcpy(&u, buf.data() + i, 4);
                if ((u & 0x7F800000u) == 0x7F800000u) {  // Inf or NaN
                    status_ = COLIBRI_ERR_INVALID_ARG;
                    return *this;
                }
            }
        } else {
            for (size_t i = 0; i < len; i += 2) {
                uint16_t u;
                std::memcpy(&u, buf.data() + i, 2);
                if ((u & 0x7F80u) == 0x7F80u) {
                    status_ = COLIBRI_ERR_INVALID_ARG;
                    return *this;
                }
            }
        }
    }
    return *this;
}

Validator &Validator::indices(const int32_t *p, size_t n, int32_t lo, int32_t hi) {
    range(p, n * 4);
    if (status_ != COLIBRI_OK || p == nullptr || n == 0 || !drain()) return *this;
    std::vector<int32_t> buf(std::min(kChunk / 4, n));
    for (size_t at = 0; at < n; at += buf.size()) {
        const size_t len = std::min(buf.size(), n - at);
        if (!fetch(p + at, len * 4, buf.data())) return *this;
        for (size_t i = 0; i < len; ++i)
            if (buf[i] < lo || buf[i] > hi) {
                status_ = COLIBRI_ERR_INVALID_ARG;
                return *this;
            }
    }
    return *this;
}

Validator &Validator::offsets(const int32_t *p, size_t n, int32_t hi) {
    range(p, n * 4);
    if (status_ != COLIBRI_OK || p == nullptr || n == 0 || !drain()) return *this;
    std::vector<int32_t> v(n);
    if (!fetch(p, n * 4, v.data())) return *this;
    if (v[0] != 0) status_ = COLIBRI_ERR_INVALID_ARG;
    for (size_t i = 1; i < n && status_ == COLIBRI_OK; ++i)
        if (v[i] < v[i - 1] || v[i] > hi) status_ = COLIBRI_ERR_INVALID_ARG;
    return *this;
}

}  // namespace colibri
