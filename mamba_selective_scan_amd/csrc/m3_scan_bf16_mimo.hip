// m3_scan_bf16_mimo.hip -- kernel instances for one (io type, load path) pair.
#include "m3_scan_impl.hpp"

namespace m3 {
M3_DEFINE_VARIANT(scan_bf16_mimo, IoBF16, kModeMimo)
}  // namespace m3
