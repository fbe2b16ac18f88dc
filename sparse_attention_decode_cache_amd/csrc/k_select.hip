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

// One workgroup per sequence of a batch; a sequence with nb <= k keeps every
// block (its ids, if asked for, are 0..nb-1, then -1 up to pad_to).
__global__ __launch_bounds__(sel::kT) void k_select_batch(SelectBatchArgs b)
{
    extern __shared__ uint4 sel_lds[];
    const SelectArgs &a = b.seq[blockIdx.x];
    int32_t *out = a.sel;
    if (a.nb <= a.k) {
        if (out)
            for (int i = threadIdx.x; i < a.nb || i < a.pad_to; i += sel::kT)
                out[i] = i < a.nb ? i : -1;
        return;
    }
    sel::run(a, reinterpret_cast<char *>(sel_lds), [=](uint32_t slot, uint32_t id) {
        out[slot] = (int32_t)id;
    });
}

}  // namespace

hipError_t launch_select_batch(const SelectBatchArgs &bin, hipStream_t s)
{
    SelectBatchArgs b = bin;
    if (b.n < 1 || b.n > kMaxBatch)
        return hipErrorInvalidValue;
    int32_t nb_max = 0;
    for (int i = 0; i < b.n; ++i) {
        if (b.seq[i].nb > b.seq[i].k && b.seq[i].T != 8 && b.seq[i].T != 16 && b.seq[i].T != 32)
            return hipErrorInvalidValue;
        nb_max = b.seq[i].nb > nb_max ? b.seq[i].nb : nb_max;
    }
    // one layout for every sequence: Smem, the bitmap of the longest, and
    // (when it fits) a key cache as long as the longest
    size_t lds = 0;
    for (int i = 0; i < b.n; ++i)
        lds = sel::lds_with_cache(b.seq[i], nb_max, sel::kMaxLds);
    if (lds > sel::kMaxLds)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        static hipError_t attr = hipFuncSetAttribute((const void *)k_select_batch,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sel::kMaxLds);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL(k_select_batch, dim3(b.n), dim3(sel::kT), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &ain, hipStream_t s)
{
    SelectArgs a = ain;
    if (a.T != 8 && a.T != 16 && a.T != 32)
        return hipErrorInvalidValue;
    const size_t lds = sel::lds_with_cache(a, a.nb, sel::kMaxLds);
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
