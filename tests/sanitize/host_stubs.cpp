// Stand-ins for the device side of libua (kernel launchers and the
// no-allocation scratch lookup) so that the C-ABI host layer (ua_api.cpp:
// validation, planning, argument marshalling) can be built with the host
// compiler's address and undefined-behaviour sanitizers and driven by the
// CPU ABI tests.  Nothing here runs on a GPU; each launcher only checks the
// grid it is handed and reports success.
#include "ua_internal.h"

#include <cstdlib>

namespace ua {

hipError_t launch_attention(const AttnArgs &a, bool, bool, bool, bool split, bool wide, bool mix, dim3 grid,
                            hipStream_t) {
    if (grid.x == 0 || grid.y == 0 || (wide && a.num_splits < 2) || (wide && !split))
        std::abort();
    // a launch that splits only the decode rows: unsplit prefill workgroups,
    // a one-dimensional grid holding every decode block
    if (mix && (split || a.num_splits < 2 || grid.y != 1 || a.mix_region < a.mix_dblocks ||
                (int64_t)grid.x < 8LL * a.mix_dblocks))
        std::abort();
    // persistent form: at most one workgroup per item
    if (a.persist_items > 0 && (int64_t)grid.x * grid.y > a.persist_items)
        std::abort();
    return hipSuccess;
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int32_t num_splits, int64_t rows,
                          int32_t, void *out, bool, int64_t, int64_t, float *, const int32_t *,
                          hipStream_t) {
    if (!o_part || !lse_part || !out || num_splits < 1 || rows < 0)
        std::abort();
    return hipSuccess;
}

hipError_t launch_combine_decode(const float *o_part, const float *lse_part, int32_t num_splits, int64_t rows,
                                 int32_t, int32_t num_kv_heads, int32_t num_seqs, const int32_t *cu_seqlens_q,
                                 void *out, bool, int64_t, int64_t, float *, hipStream_t) {
    if (!o_part || !lse_part || !out || !cu_seqlens_q || num_splits < 2 || rows < 0 || num_kv_heads <= 0 ||
        num_seqs < 0)
        std::abort();
    return hipSuccess;
}

hipError_t launch_append(const AppendArgs &a, bool, bool, hipStream_t) {
    if (a.num_tokens <= 0 || a.num_kv_heads <= 0)
        std::abort();
    return hipSuccess;
}

hipError_t launch_backward(const BwdArgs &a, bool, bool, hipStream_t) {
    if (a.group <= 0 || a.block_q <= 0)
        std::abort();
    return hipSuccess;
}

hipError_t noalloc_scratch(void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t(1) << 20);   // an aligned stand-in address
    return hipSuccess;
}

}  // namespace ua
