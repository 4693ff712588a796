// Entry points of one chunk shared by the public calls and the whole-prompt
// driver.  positions == nullptr means the positions are implied (p0 + i with
// p0 = n_k - n_q) and are not checked on the device.
#pragma once
#include "../../include/dcasparse.h"

namespace dca {

int index_impl(const dca_bf16* q, const dca_bf16* k, const int32_t* positions, const dca_cfg* cfg,
               int32_t* v_idx, int32_t* s_off);
int prefill_impl(const dca_bf16* q, const dca_bf16* k, const dca_key_cache* cache, const dca_bf16* v,
                 const int32_t* positions, const dca_cfg* cfg, dca_bf16* out);

}  // namespace dca
