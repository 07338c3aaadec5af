// RAII bracket for one kernel launch: records HIP events on the launch stream
// while kernel timing is enabled (see moe_profile_enable), nothing otherwise.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

class ProfScope {
public:
    ProfScope(hipStream_t stream, const char* name);
    ~ProfScope();
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;

private:
    hipStream_t stream_;
    const char* name_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

}  // namespace moe
