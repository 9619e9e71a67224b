// Kernel parameter blocks shared by the host API and the kernels (passed by value).
#pragma once

#include <stdint.h>

#include "moc.h"

namespace moc {

struct RouteParams {
  int B, H, L, C, S, k_eff, causal, m_cap;
  int drop_off, drop_in;
  float p_max;
  uint64_t seed;
  uint64_t thr[MOC_MAX_DROP_IN];  // drop-in Poisson CDF thresholds (x 2^32)
  const uint32_t* cmask;          // optional candidate mask [B*H][C][cmask_w] (outer routing)
  int cmask_w;
  const uint32_t* chk;            // layout check word (moc_layout.check) or NULL
};

struct VarlenParams {
  int B, H, L, C, S, nqt, tile_rows, max_rtiles, max_atiles;
  int text_begin, text_end;
  int key_rows, max_ktiles, n_text_split;  // backward key tiles
  const uint32_t* chk;                     // layout check word (moc_layout.check) or NULL
};

}  // namespace moc
