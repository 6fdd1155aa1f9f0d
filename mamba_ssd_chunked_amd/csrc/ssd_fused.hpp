// Launch layout shared by the fused forward kernels: one workgroup per CU walks
// one head's chunks, whole heads first and p halves of heads for a last round
// that is at most half full.
#pragma once

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// Block -> head. Slots 0 .. B*H - 1 list every head once. With unit_map
// ((B*G) % 8 == 0) slot s serves unit (s % 8) + 8 ((s / 8) / hpg), head
// (s / 8) % hpg of that unit (unit = batch * G + group), so slots on one XCD
// (block i runs on XCD i % 8) cover whole units and the int8 B/C data of a
// unit stay in one XCD's L2; otherwise slot s is unit s / hpg. Whole-head
// blocks [0, nfull) take slot = block. The p-half blocks after them take slots
// nfull .. B*H - 1, two blocks per slot: with half_il (nfull and the half count
// both multiples of 8) block nfull + bx takes slot nfull + bx % 8 + 8 (j / 2)
// and half j % 2 (j = bx / 8), so it runs on its slot's XCD; otherwise slot
// nfull + bx / 2 and half bx % 2. One slot map serves both parts, so every
// head is computed exactly once.
// ---------------------------------------------------------------------------
struct BlockHead {
  int64_t unit, hl;
  int ph;
};
template <int PW>
__device__ __forceinline__ BlockHead block_head(const Dims& d, int64_t bx, int64_t nfull, int unit_map,
                                                int half_il) {
  BlockHead r;
  int64_t slot;
  r.ph = 0;
  if (PW == 4) {
    slot = bx;
  } else if (half_il) {
    const int64_t j = bx / 8;
    slot = nfull + (bx % 8) + 8 * (j >> 1);
    r.ph = (int)(j & 1);
  } else {
    slot = nfull + bx / 2;
    r.ph = (int)(bx & 1);
  }
  if (unit_map) {
    const int64_t j = slot / 8;
    r.unit = (slot % 8) + 8 * (j / d.hpg);
    r.hl = j % d.hpg;
  } else {
    r.unit = slot / d.hpg;
    r.hl = slot % d.hpg;
  }
  return r;
}

// One workgroup per CU at a time: B*H heads run in ceil(B*H / CUs) rounds. When
// the last round is at most half full, its heads are split in two p halves so
// the round spreads over all CUs.
struct SplitPlan {
  int64_t nfull, nhalf;
  int unit_map, half_il;
};
inline SplitPlan split_plan(const Dims& d) {
  const int64_t BH = d.B * d.H;
  const int64_t ncu = cu_count();
  int64_t nhalf = 0;
  if (ncu > 0) {
    const int64_t rem = BH % ncu;
    if (rem != 0 && 2 * rem <= ncu) nhalf = rem;
  }
  SplitPlan p;
  p.nfull = BH - nhalf;
  p.nhalf = nhalf;
  p.unit_map = (d.B * d.G) % 8 == 0;
  p.half_il = p.nfull % 8 == 0 && nhalf % 8 == 0;
  return p;
}

constexpr size_t kWsAlign = 256;
inline size_t ws_align(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

}  // namespace ssd
