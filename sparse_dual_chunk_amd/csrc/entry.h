// Entry points of one chunk shared by the public calls and the whole-prompt
// driver.  positions == nullptr means the positions are implied (p0 + i with
// p0 = n_k - n_q) and are not checked on the device.
#pragma once
#include "../../include/dcasparse.h"

namespace dca {

int index_impl(const dca_bf16* q, const dca_bf16* k, const int32_t* positions, const dca_cfg* cfg,
               int32_t* v_idx, int32_t* s_off);
// Keys come raw (k), from a contiguous rotated cache (cache, values in v) or
// from a paged pool (paged: keys and values, gathered into the workspace).
int prefill_impl(const dca_bf16* q, const dca_bf16* k, const dca_key_cache* cache, const dca_paged_kv* paged,
                 const dca_bf16* v, const int32_t* positions, const dca_cfg* cfg, dca_bf16* out);
// Workspace bytes of one chunk's prefill from a paged pool (the gathered values added).
int paged_prefill_bytes(const dca_cfg* cfg, size_t* bytes);
// The host checks of a paged pool (pointers, sizes, page length).
int paged_valid(const dca_paged_kv* cache, int h_kv, int head_dim);

}  // namespace dca
