#include "prefill.h"

namespace qw3 {
int32_t prefill_layers(uint8_t *, const Layout &, const Dims &, int, int, int, hipStream_t) {
    return QW3_UNSUPPORTED_SHAPE;
}
}  // namespace qw3
