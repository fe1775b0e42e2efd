#include "device.hpp"
#include "launch.hpp"
namespace paq {
bool prefill_mfma_supports(int, int, int, int) { return false; }
int launch_prefill_mfma(const AttnArgs&, hipStream_t) { return -1; }
}  // namespace paq
