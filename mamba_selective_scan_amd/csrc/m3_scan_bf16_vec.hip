// m3_scan_bf16_vec.hip -- kernel instances for one (io type, load path) pair.
#include "m3_scan_impl.hpp"

namespace m3 {
M3_DEFINE_VARIANT(scan_bf16_vec, IoBF16, kModeVec)
}  // namespace m3
