// MFMA prefill path: not compiled in yet; every shape falls back to the portable path.
#include "prefill_mfma.hpp"

namespace taylor {

bool prefill_mfma_has(int, int, int, int) { return false; }
long long prefill_mfma_ws_bytes(const Shape&, int, int, int) { return 0; }
int prefill_mfma_launch(const PrefillArgs&) { return -2; }

}  // namespace taylor
