// Host-side helpers shared by the entry points of libqkv_prep.so: device
// scoping, the sync-mode flag and pointer alignment.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

namespace qkvp {

inline bool env_flag(const char *name)
{
    const char *v = std::getenv(name);
    return v && v[0] == '1';
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Makes `device` current for the guard's lifetime and restores the caller's
// current device afterwards.  ok() is false when either step failed.
class DeviceScope {
public:
    explicit DeviceScope(int device)
    {
        if (hipGetDevice(&prev_) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        if (prev_ != device && hipSetDevice(device) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        ok_ = true;
        switched_ = prev_ != device;
    }
    ~DeviceScope()
    {
        if (switched_)
            (void)hipSetDevice(prev_);
    }
    DeviceScope(const DeviceScope &) = delete;
    DeviceScope &operator=(const DeviceScope &) = delete;
    bool ok() const { return ok_; }

private:
    int prev_ = -1;
    bool ok_ = false;
    bool switched_ = false;
};

// True when `device` names an existing HIP device.
inline bool device_exists(int device)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return device >= 0 && device < count;
}

}  // namespace qkvp
