// fa_types.hpp -- plain parameter structs shared by the host side (fa_api.cpp)
// and the kernels.
#pragma once

#include <stdint.h>

namespace fa {

// Attention dropout: element (bh, i, j) is dropped when byte j % 4 of word
// i % 4 of Philox4x32-10(counter (j / 4, i / 4, bh, 0), key (k0, k1)) is
// below t; survivors are scaled by keep_scale = 256 / (256 - t).  t = 0 means
// no dropout.
struct Dropout {
    uint32_t k0, k1;     // seed, low and high words
    uint32_t t;          // drop threshold in 1/256 units, 0..255
    float keep_scale;    // 256 / (256 - t)
};

}  // namespace fa
