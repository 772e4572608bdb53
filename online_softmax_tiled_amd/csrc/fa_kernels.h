// fa_kernels.h -- host-side launchers of the HIP kernels (internal to
// libfa_mi355x.so).  Each returns an fa_status; arguments are validated by
// the C ABI layer before any launcher is called.
#pragma once

#include "fa_device.h"

namespace fa {

// bf16 tiled forward (MFMA).  split: write per-split partials instead of O.
int launch_fwd_bf16(const FwdParams &p, int d, bool split, hipStream_t stream);
// bf16 tiled forward with 64 query rows per wave (d = 128, unsplit), for
// grids of at least 512 blocks of 256 query rows.
bool fwd_bf16_wide_applies(const FwdParams &p, int d);
int launch_fwd_bf16_wide(const FwdParams &p, hipStream_t stream);
// bf16 tiled forward for small grids: 4 waves per 32 query rows, each on a
// quarter of the keys, merged in LDS (d in {32, 64, 128}, unsplit).
bool fwd_bf16_splitk_applies(const FwdParams &p, int d);
int launch_fwd_bf16_splitk(const FwdParams &p, int d, hipStream_t stream);
// fp8 (E4M3) tiled forward (MFMA), bf16 output.  c_log2 > 0 multiplies the
// integer-exact fp8 dot products into base-2 score units; out_scale
// multiplies O; qflip is xor-ed into every 4 bytes of Q (0x80808080 negates Q).
int launch_fwd_fp8(const FwdParams &p, int d, float c_log2, float out_scale, uint32_t qflip, hipStream_t stream);
// fp32 tiled forward (VALU, fp32 throughout).
int launch_fwd_f32(const FwdParams &p, int d, hipStream_t stream);
// bf16 split-KV partial pass for few query rows per K/V head (decode).
int launch_splitkv_decode(const FwdParams &p, int d, hipStream_t stream);
// Rows of query rows per K/V head up to which the decode kernel is used.
int splitkv_decode_max_rows();
// Write rows of T tokens starting at pos into a rolling cache (sink rows,
// then a ring of window slots); n_rows = B * Hkv * T.
int launch_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache, int64_t n_rows, int64_t T,
                     int64_t pos, int64_t window, int64_t sinks, int d, hipStream_t stream);
// Row softmax (online normaliser) and its fused top-k.
int launch_softmax(const void *x, void *y, float *lse, int64_t rows, int64_t n, int dtype, hipStream_t stream);
int launch_softmax_topk(const void *x, float *probs, int32_t *idx, float *lse, int64_t rows, int64_t n, int k,
                        int dtype, hipStream_t stream);
// Merge per-split partials into O (bf16 or fp32) and lse.
int launch_combine(const float *o_part, const float *m_part, const float *l_part, void *o, float *lse,
                   int64_t rows, int num_splits, int d, int out_dtype, hipStream_t stream);

}  // namespace fa
