// IndexCache F/S layer schedule (host only).
//
// IndexCache blog post, skip_topk snippet: without a pattern a layer skips
// top-k iff max(layer_id - offset + 1, 0) % freq != 0; with a pattern it skips
// iff pattern[layer_id] == 'S'.  PR #37735 report: the schedule applies only
// under use_index_cache, and a pattern must have one F/S character per layer
// (its "Risks & impact" section notes the character check was missing).

#include <string.h>

#include "idx.h"

extern "C" idx_status_t idx_layer_schedule(int32_t use_index_cache, const char* pattern,
                                           int32_t freq, int32_t offset, int32_t num_layers,
                                           uint8_t* is_full) {
  if (num_layers < 1 || is_full == nullptr) return IDX_ERR_INVALID_ARG;
  if (!use_index_cache) {
    for (int l = 0; l < num_layers; ++l) is_full[l] = 1;
    return IDX_OK;
  }
  if (pattern != nullptr) {
    if ((int64_t)strlen(pattern) != num_layers) return IDX_ERR_INVALID_ARG;
    for (int l = 0; l < num_layers; ++l)
      if (pattern[l] != 'F' && pattern[l] != 'S') return IDX_ERR_INVALID_ARG;
    if (pattern[0] != 'F') return IDX_ERR_INVALID_ARG;
    for (int l = 0; l < num_layers; ++l) is_full[l] = pattern[l] == 'F';
    return IDX_OK;
  }
  if (freq < 1) return IDX_ERR_INVALID_ARG;
  for (int l = 0; l < num_layers; ++l) {
    int v = l - offset + 1;
    v = v < 0 ? 0 : v;
    is_full[l] = (v % freq) == 0;
  }
  if (!is_full[0]) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}
