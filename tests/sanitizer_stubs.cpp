// Launcher stand-ins for the host-only sanitizer build of the C ABI
// (tests/test_abi_host_sanitized.py): the argument checks, planning and
// workspace arithmetic of sv_api.cpp run under AddressSanitizer and
// UndefinedBehaviorSanitizer with every kernel launch replaced by a call
// that only records that it happened.  Test infrastructure, not product code.
#include "../draft_token_verification_sv_amd/csrc/sv_internal.h"

namespace sv {

int g_stub_launches = 0;

hipError_t launch_attn_mfma(const AttnParams &, int, int, int, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_attn_dma(const AttnParams &, int, int, int, bool, int, hipStream_t) {
    return ++g_stub_launches, hipSuccess;
}
int attn_dma_max_split_pages() { return 512; }
hipError_t launch_attn_q4c(const AttnParams &, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
int attn_q4c_max_split_pages() { return 512; }
hipError_t launch_attn_q4w(const AttnParams &, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
bool attn_q4w_supports(bool paged, int nts) { return nts >= 1 && nts <= (paged ? 2 : 3); }
hipError_t launch_attn_valu(const AttnParams &, int, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_attn_merge(const AttnParams &, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_accept(const AcceptParams &, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_topk_accept(const AcceptParams &, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_compact(const CompactParams &, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_append(const AppendParams &, int, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_conv_tree(const ConvTreeParams &, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_delta_tree(const DeltaParams &, int, int, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_commit(const CommitParams &, int, int, hipStream_t) { return ++g_stub_launches, hipSuccess; }
hipError_t launch_tree_schedule(const int32_t *, int, int, int32_t *, hipStream_t) {
    return ++g_stub_launches, hipSuccess;
}
unsigned int *device_error_word() { return nullptr; }

}  // namespace sv

extern "C" int sv_check_device_errors(void *) { return 0; }
extern "C" int sv_stub_launches(void) { return sv::g_stub_launches; }
