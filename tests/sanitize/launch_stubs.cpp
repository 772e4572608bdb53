// launch_stubs.cpp -- stand-ins for the kernel launchers of libfa_mi355x.so,
// linked into the sanitizer build of the C-ABI layer (fa_api.hip) in place
// of the kernel sources.  The driver's requests must all be refused or
// empty before any launch; each stand-in therefore reports the launch it
// was asked for and aborts, which fails the test.
#include <stdio.h>
#include <stdlib.h>

#include "fa_kernels.h"

namespace {
[[noreturn]] void reached(const char *what) {
    fprintf(stderr, "FAIL: the C-ABI layer reached %s\n", what);
    abort();
}
}  // namespace

namespace fa {
int launch_fwd_bf16(const FwdParams &, int, bool, hipStream_t) { reached("launch_fwd_bf16"); }
bool fwd_bf16_wide_applies(const FwdParams &, int) { reached("fwd_bf16_wide_applies"); }
int launch_fwd_bf16_wide(const FwdParams &, hipStream_t) { reached("launch_fwd_bf16_wide"); }
bool fwd_bf16_splitk_applies(const FwdParams &, int) { reached("fwd_bf16_splitk_applies"); }
int launch_fwd_bf16_splitk(const FwdParams &, int, hipStream_t) { reached("launch_fwd_bf16_splitk"); }
int launch_fwd_fp8(const FwdParams &, int, float, float, uint32_t, hipStream_t) { reached("launch_fwd_fp8"); }
int launch_fwd_f32(const FwdParams &, int, hipStream_t) { reached("launch_fwd_f32"); }
int launch_splitkv_decode(const FwdParams &, int, hipStream_t) { reached("launch_splitkv_decode"); }
int splitkv_decode_max_rows() { reached("splitkv_decode_max_rows"); }
int launch_kv_append(const void *, const void *, void *, void *, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                     hipStream_t) {
    reached("launch_kv_append");
}
int launch_softmax(const void *, void *, float *, int64_t, int64_t, int, hipStream_t) { reached("launch_softmax"); }
int launch_softmax_topk(const void *, float *, int32_t *, float *, int64_t, int64_t, int, int, hipStream_t) {
    reached("launch_softmax_topk");
}
int launch_combine(const float *, const float *, const float *, void *, float *, int64_t, int, int, int,
                   hipStream_t) {
    reached("launch_combine");
}
}  // namespace fa
