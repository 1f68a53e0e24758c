// Stand-ins for the kernel launchers of libpdllm, for a host-only build of
// its C-ABI layer and planner (pdllm_abi.cpp, plan.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Each records that it was reached and
// reports success; none touches the pointers it is given.
#include "../../diffusion_long_context_amd/csrc/pdllm_internal.h"

namespace pdllm {
int g_launches = 0;
int launch_decode_bf16(const DecodeArgs&, int, int, void*) { return ++g_launches, 0; }
int launch_decode_f32(const DecodeArgs&, int, void*) { return ++g_launches, 0; }
int launch_decode_ws(const DecodeArgs&, int, void*) { return ++g_launches, 0; }
int launch_resolve_rows(const ResolveArgs&, void*) { return ++g_launches, 0; }
int launch_lse_merge(const DecodeArgs&, int, bool, bool, void*) { return ++g_launches, 0; }
int launch_prefill_bf16(const PrefillArgs&, int, void*) { return ++g_launches, 0; }
int launch_prefill_f32(const PrefillArgs&, int, void*) { return ++g_launches, 0; }
int launch_prefill_stream(const PrefillArgs&, int, void*) { return ++g_launches, 0; }
int launch_score_finalize(const PrefillArgs&, void*) { return ++g_launches, 0; }
int launch_select_topb(const float*, const int32_t*, int, int, int, int32_t*, void*) { return ++g_launches, 0; }
int launch_select_topk(const TopkArgs&, void*) { return ++g_launches, 0; }
int launch_finalize_select(const FinalizeSelectArgs&, void*) { return ++g_launches, 0; }
int launch_chunk_score(const ChunkScoreArgs&, void*) { return ++g_launches, 0; }
int launch_compact(const CompactArgs&, void*) { return ++g_launches, 0; }
int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return 100;                               // hipErrorNoDevice: no device in a host-only build
}
}  // namespace pdllm
