// k_select.hip -- stage 3 as its own kernel: one workgroup runs the top-k
// routine of qsa_select.h and writes the chosen block ids, ascending.
#include "qsa_select.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(sel::kT) void k_select(SelectArgs a)
{
    extern __shared__ uint4 sel_lds[];
    int32_t *out = a.sel;
    sel::run(a, reinterpret_cast<char *>(sel_lds), [=](uint32_t slot, uint32_t id) {
        out[slot] = (int32_t)id;
    });
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t s)
{
    if (a.T != 8 && a.T != 16 && a.T != 32)
        return hipErrorInvalidValue;
    const size_t lds = sel::lds_bytes(a.nb);
    if (lds > sel::kMaxLds)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        static hipError_t attr = hipFuncSetAttribute((const void *)k_select,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sel::kMaxLds);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL(k_select, dim3(1), dim3(sel::kT), lds, s, a);
    return hipGetLastError();
}

}  // namespace qsa
