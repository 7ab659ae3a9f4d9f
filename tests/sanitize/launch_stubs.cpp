// Host-only stand-ins for the kernel launchers of libleapq, for the
// sanitizer build of the C ABI (no GPU): each records that it was reached
// and with which head count and record count, and launches nothing.
#include <hip/hip_runtime.h>

#include "leapq_internal.h"

namespace leapq {

int stub_calls = 0, stub_heads = -1, stub_n = -1;

static hipError_t note(int heads, int n)
{
    ++stub_calls;
    stub_heads = heads;
    stub_n = n;
    return hipSuccess;
}

hipError_t launch_init(const StateView &, int heads, const float *, int, float, hipStream_t) { return note(heads, 0); }
hipError_t launch_fold(const StateView &, int heads, int n, int, float, hipStream_t) { return note(heads, n); }
hipError_t launch_dequant(const StateView &, int heads, int n, int, float *, hipStream_t) { return note(heads, n); }
hipError_t launch_append(const StateView &, int heads, int n, int, const void *, const void *, const void *,
                         const float *, const float *, float *, const GateArgs &, hipStream_t)
{
    return note(heads, n);
}
hipError_t launch_append_fold(const StateView &, int heads, int n, int, const void *, const void *, const void *,
                              const float *, const float *, float *, int, float, const GateArgs &, hipStream_t)
{
    return note(heads, n);
}
hipError_t launch_step(const StateView &, int heads, int, const int *, int *, int, const void *, const void *,
                       const void *, const float *, const float *, float *, int, float, const GateArgs &,
                       hipStream_t)
{
    return note(heads, -2);
}
hipError_t launch_gdn_decode(int heads, int, int, int, void *, const void *, const void *, const void *,
                             const float *, const float *, float *, hipStream_t)
{
    return note(heads, -3);
}

}  // namespace leapq
