// Internal: the plan object behind the opaque fa_plan handle.
#pragma once

#include <stdint.h>

#include "fa_params.h"

struct fa_plan {
  fa::Params p;        // kernel parameter block (tile_prefix filled in phase 2)
  int32_t kind;        // fa::KernelKind
  int32_t dtype;       // fa_dtype of q/k/v/o
  int32_t bm, bn;      // query rows and keys per tile step
  int32_t block;       // threads per workgroup
  uint64_t ws_bytes;   // device workspace phase 2 needs
  uint64_t ws_map_off; // byte offset of the TND tile map in the workspace
  uint64_t ws_pse_off; // byte offset of the TND pse block offsets in the workspace
  uint64_t ws_cls_off; // byte offset of the mask block classes in the workspace
  uint64_t ws_part_off; // byte offset of the key split's partial outputs (then their statistics)
};

// Record the message fa_last_error_message() returns on this thread.
void fa_set_error(const char* msg);
