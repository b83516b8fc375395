// Host launchers of the qkv kernels (defined in encode.hip, decode.hip,
// attend.hip and xlayer.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "device.h"

namespace qkv {

void launch_header(const EncodeArgs &a, int streams, hipStream_t st);
void launch_init(const EncodeArgs &a, int streams, hipStream_t st);
void launch_assign(const EncodeArgs &a, int streams, hipStream_t st);
void launch_update(const EncodeArgs &a, int streams, hipStream_t st);
void launch_chan_flags(const EncodeArgs &a, int streams, hipStream_t st);
void launch_quantize(const EncodeArgs &a, int streams, hipStream_t st);
void launch_reconstruct(const ReconArgs &a, int n_layers, int64_t out_tokens, int out_t_off,
                        hipStream_t st);
void launch_attend(const AttnArgs &a, hipStream_t st);
// device address of the fixed partials array of the current device (0 on success)
int noalloc_scratch_address(void **ptr);
void launch_attend_fresh(const AttnArgs &a, hipStream_t st);
void launch_attend_merge2(const MergeArgs &m, hipStream_t st);
void launch_xl_predict(const XlArgs &a, int kv0, int n_kv, hipStream_t st);
void launch_xl_refit(const RefitArgs &a, hipStream_t st);
void launch_set_header(uint8_t *arena, const DevLayout &L, int layer0, int n_layers, int n_chunks,
                       int n_tokens, hipStream_t st);

}  // namespace qkv
