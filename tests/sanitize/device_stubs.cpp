// Stand-ins for the library's device entry points, linked only into the
// sanitizer build of the host sources (pd_host.cpp, pd_cascade_host.cpp),
// which g++ compiles without the HIP kernels.  Each refuses with
// PD_E_UNSUPPORTED, so a host test that reached one would fail loudly; the
// sanitizer run selects tests that call host entry points only.
#include <cstdint>

#include "pd_internal.h"

namespace pd {
int mla_q_heads_per_wg(int32_t) { return fail(PD_E_UNSUPPORTED, "sanitizer build: no MLA kernel"); }
int mla_resident_wgs(int32_t, int32_t) { return fail(PD_E_UNSUPPORTED, "sanitizer build: no device"); }
}  // namespace pd

#define PD_STUB(name, ...) \
    extern "C" int name(__VA_ARGS__) { return pd::fail(PD_E_UNSUPPORTED, "sanitizer build: no " #name); }

PD_STUB(paged_decode_partial, const void *, const void *, const void *, int64_t, int64_t, int64_t,
        int32_t, const int32_t *, const int32_t *, const int32_t *, const int32_t *,
        const int32_t *, const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
        int32_t, float, float *, float *, void *)
PD_STUB(paged_decode_fused, const void *, const void *, const void *, int64_t, int64_t, int64_t,
        int32_t, const int32_t *, const int32_t *, const int32_t *, const int32_t *,
        const int32_t *, const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
        int32_t, float, float *, float *, int32_t *, float *, float *, void *)
PD_STUB(paged_decode_fused_noalloc, const void *, const void *, const void *, int64_t, int64_t,
        int64_t, int32_t, const int32_t *, const int32_t *, const int32_t *, const int32_t *,
        const int32_t *, const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
        int32_t, float, float *, float *, void *)
PD_STUB(paged_merge_states, const float *, const float *, const int32_t *, int32_t, int32_t,
        int32_t, float *, float *, void *)
PD_STUB(paged_mla_decode_partial, const void *, const void *, const void *, const void *, int64_t,
        int64_t, int64_t, int64_t, int32_t, int32_t, int32_t, const int32_t *, const int32_t *,
        const int32_t *, const int32_t *, const int32_t *, const int32_t *, int32_t, int32_t,
        int32_t, int32_t, int32_t, float, float *, float *, void *)
PD_STUB(paged_decode_kernel_kind, int32_t, int32_t, int32_t, int32_t, int64_t)
PD_STUB(paged_decode_set_kernel_choice, int32_t)
PD_STUB(paged_decode_default_target_wgs, int32_t, int32_t, int32_t, int32_t, int32_t)
PD_STUB(paged_cascade_stack_q, const void *, int32_t, const int32_t *, int32_t, int32_t, int32_t,
        int32_t, void *, void *)
PD_STUB(paged_cascade_gather_states, const float *, const float *, int32_t, int32_t,
        const int32_t *, const float *, const float *, int32_t, const int32_t *, int32_t, int32_t,
        int32_t, float *, float *, void *)
PD_STUB(paged_cascade_merge_states, const float *, const float *, int32_t, const int32_t *,
        const float *, const float *, const int32_t *, int32_t, int32_t, int32_t, int32_t,
        float *, float *, void *)
PD_STUB(paged_cascade_partial, const void *, int32_t, const int32_t *, int32_t, int32_t,
        const void *, const void *, int64_t, int64_t, int64_t, int32_t, int32_t, int32_t, int32_t,
        int32_t, float, const paged_cascade_level *, const paged_cascade_level *, int32_t, void *)
PD_STUB(paged_sparse_csr, int32_t, int32_t, int32_t, int32_t, const int32_t *, int32_t *,
        int32_t *, int32_t *)
PD_STUB(paged_sparse_expand_blocks, const int32_t *, int32_t, int32_t, const int32_t *, int32_t,
        const int32_t *, const int32_t *, int32_t, int32_t *, void *)
PD_STUB(paged_hbm_read_probe, const void *, int64_t, int32_t, int32_t, uint32_t *, void *)
