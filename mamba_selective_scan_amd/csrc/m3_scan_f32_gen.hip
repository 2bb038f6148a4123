// m3_scan_f32_gen.hip -- kernel instances for one (io type, load path) pair.
#include "m3_scan_impl.hpp"

namespace m3 {
M3_DEFINE_VARIANT(scan_f32_gen, IoF32, kModeGen)
}  // namespace m3
