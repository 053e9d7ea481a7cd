// Range check of gathered row ids.  Plain C++ (constexpr functions are callable from host code and
// from the gfx950 kernels alike), so that the host tests compile this same file.  An id outside
// [0, rows) reads the nearest row of the table instead of memory past it; rows >= 1 is checked on
// the host before any launch.
#pragma once

#include <stdint.h>

namespace hstu {

constexpr bool row_id_in_range(int64_t id, int64_t rows) { return id >= 0 && id < rows; }

constexpr int64_t clamp_row_id(int64_t id, int64_t rows) { return id < 0 ? 0 : (id >= rows ? rows - 1 : id); }

}  // namespace hstu
