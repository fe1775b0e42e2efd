#include "device.hpp"
#include "launch.hpp"
namespace paq {
bool decode_mfma_supports(int, int, int, int) { return false; }
int launch_decode_mfma(const AttnArgs&, hipStream_t) { return -1; }
}  // namespace paq
