// Internal helpers shared by the host-side code and the launchers of the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "lora_sgmv.h"

namespace lora {

// Records a formatted message for lora_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Host-side checks of a descriptor that read no device memory: layout, sizes,
// non-null and 16-byte-aligned device pointers, page geometry.
int check_weights_desc(const lora_weights *w);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rank-rows per workgroup of a VALU shrink launch over `work_tiles` (tile,
// projection) pairs: 1, 2 or 4, to keep the grid near kTargetGroups workgroups, unless
// lora_set_plan fixed it for the calling thread (t_plan_jw > 0).
int32_t plan_shrink_jw(int32_t work_tiles, int32_t r_max);

// Overrides set by lora_set_plan for the calling thread: rank-rows per VALU shrink
// workgroup and rows per pass of the segment-form VALU kernels (0 = planned).
extern thread_local int32_t t_plan_jw, t_plan_nr;

// Tile height for a segment batch known only by its size (the offsets form, whose
// segment lengths are on the device): 64 when the segments average at least
// kLongSegment rows (n_rows >= kLongSegment * n_seg), else 2.
int32_t lora_tile_rows_for(int32_t n_rows, int32_t n_seg);

constexpr int32_t kMfmaMinRows = 8;      // launches with a tile this tall run the MFMA kernels
constexpr int32_t kTargetGroups = 1024;  // shrink workgroups to aim for
constexpr int32_t kLongSegment = 128;    // segments this long get 64-row (MFMA) tiles

}  // namespace lora
